// attn_fwd_bf16.hip — bf16 tiled attention forward on gfx950 matrix cores.
//
// Algorithm: "Softmax numerical stability and IO-aware attention" (zhouzhq2021.github.io),
// section 7: per query tile, initialise m = -inf, l = 0, O = 0; for every key/value
// tile form S = Q K^T, m_new = max(m, rowmax S), P = exp(S - m_new),
// alpha = exp(m - m_new), l = alpha l + rowsum P, O = alpha O + P V; finally O / l.
// Section 8 (FlashAttention-2) adds the choices kept here: the query tile is the outer
// loop so O is written once, the division by l is deferred to the end, and key tiles
// wholly above the causal diagonal are skipped.  LSE = m + ln l is written per row.
//
// gfx950 mapping (a design of its own, not the pages' warp/shared-memory scheme):
//
//   * Block = 4 wavefronts = 128 query rows; each wavefront owns 32 query rows for
//     the whole key loop.  Key tiles are 64 keys, double-buffered in LDS.
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     A = a 32-key slice of K (from LDS), B = Q^T (held in registers for the whole
//     loop).  In the 32x32 accumulator, lane l holds one column, i.e. one query row
//     (l mod 32), and 16 of its keys; the other 16 keys of that row sit in lane l^32.
//     So the row max is 31 in-lane maxima plus one exchange, and the row sum needs no
//     exchange at all until the end (each half keeps a partial l under the same m).
//   * The output is accumulated transposed too, O^T += V^T P^T: the B operand
//     (P^T, 8 keys x 1 query per lane) is exactly what the lane already holds after
//     the exponentials, converted to bf16 with no data movement.  V is staged in LDS
//     row-major, exactly like K, and the A operand (V^T) is read with the gfx950
//     transposing LDS load ds_read_b64_tr_b16: two of them give a lane the 8 keys
//     (4h..4h+3 and 8+4h..8+4h+3 of a 16-key group) of its output column, the order
//     in which the S^T accumulator hands P to the lanes.  The O^T accumulator keeps
//     one query row per lane as well, so alpha rescales it with no exchange.
//   * LDS row strides: K rows are D*2+16 bytes and V rows D*2+64 bytes, the paddings
//     under which the 16-byte K reads and the transposing V reads are free of bank
//     conflicts on gfx950's LDS.
//   * The row's reference maximum m moves lazily: only when a tile's maximum exceeds
//     it by more than 2^8 (kLazy).  Until then alpha is exactly 1 and the rescale of O
//     is skipped (decided per wavefront); P stays at most 2^8.  The result O / l and
//     LSE = m + ln l do not depend on which reference m is used.
//   * Exponentials use the hardware exp2 on scores pre-multiplied by scale * log2 e.
//   * Block ids are remapped so each of the 8 XCDs (which receive block ids round
//     robin) walks a contiguous range of (head, query tile) pairs: the key/value
//     stream of a head is then shared through that XCD's L2.  In causal mode the
//     tiles of a head run longest-first.
#include "device_common.hpp"
#include "launchers.hpp"

namespace mi355 {
namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;  // query rows per block
constexpr int kBN = 64;           // keys per tile

template <int D>
struct Smem {
    static constexpr int kStride = D + 8;    // bf16 per K row
    static constexpr int vStride = D + 32;   // bf16 per V row
    uint16_t k[2][kBN * kStride];
    uint16_t v[2][kBN * vStride];
};

// Two floats to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// The reference maximum of a row moves only when a tile's maximum exceeds it by more
// than this many powers of two; until then the probabilities exp2(c s - m) stay at
// most 2^kLazy (far from overflow) and O and l keep their scale, so the rescale of O
// is skipped.  O / l and LSE = m + log l are the same for any reference m.
constexpr float kLazy = 8.0f;

struct Params {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int N;
    int n_qtiles;
    int n_blocks;
    float scale_log2;  // |scale| * log2(e)
    int negate_q;      // scale < 0
};

// Global -> register -> LDS staging of one 64-key tile of K or V (64 x D, row-major),
// 16 bytes per access: consecutive threads take consecutive 16-byte chunks of a row,
// so global reads are fully coalesced and LDS writes are free of bank conflicts.
template <int D>
struct Prefetch {
    static constexpr int kChunks = kBN * D / 8 / 256;  // 16-byte chunks per thread
    u32x4 r[kChunks];

    __device__ __forceinline__ void load(const uint16_t* base, int j0, int N, int tid) {
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int idx = tid + 256 * c;
            // Rows past the end re-read row N-1: their scores are masked to -inf and
            // their probabilities are 0, so any finite content will do.
            const int key = min(j0 + idx / (D / 8), N - 1);
            r[c] = *reinterpret_cast<const u32x4*>(base + (int64_t)key * D + (idx % (D / 8)) * 8);
        }
    }

    __device__ __forceinline__ void store(uint16_t* tile, int stride, int tid) const {
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int idx = tid + 256 * c;
            *reinterpret_cast<u32x4*>(&tile[(idx / (D / 8)) * stride + (idx % (D / 8)) * 8]) = r[c];
        }
    }
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing LDS load: within each group of 16 lanes, lane i receives element i % 4
// of the 8-byte blocks addressed by lanes i / 4 + 4 k, k = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
    typedef __attribute__((address_space(3))) uint16_t lds_u16;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_u16*)(p));
}

// Per-wavefront state of the key loop and the three phases of one key tile.
template <int D, bool CAUSAL>
struct Wave {
    static constexpr int KS = D / 16;  // k-steps of Q K^T
    static constexpr int DB = D / 32;  // 32-wide blocks of the output dimension

    bf16x8 qf[KS];   // Q^T fragments (B operand of S^T = K Q^T)
    f32x16 acc[DB];  // O^T accumulator: this lane's query row, 16 of each 32 outputs
    float m;         // reference max of |scale| log2(e) score, this lane's row (see kLazy)
    float l;         // running partial sum over this lane's half of every tile
    float c;         // |scale| log2(e)
    int half, l32, k_off, v_off, my_q, key_lim;

    // S^T = K Q^T for the two 32-key halves of a tile (A = K rows from LDS).
    __device__ __forceinline__ void qk(f32x16 (&st)[2], const uint16_t* ktile) const {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            f32x16 a = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
                    ktile + k_off + 32 * sb * Smem<D>::kStride + 16 * ks);
                a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], a, 0, 0, 0);
            }
            st[sb] = a;
        }
    }

    // Online-softmax update of one tile: hidden keys (diagonal / ragged tiles only)
    // take no part; on return st holds P = exp2(c s - m_new) and the running state is
    // updated.  Returns alpha = exp2(m_old - m_new), exactly 1 when the reference
    // maximum stays.
    template <bool MASK>
    __device__ __forceinline__ float softmax(f32x16 (&st)[2], int j0) {
        if (MASK) {
            const int key0 = j0 + 4 * half;  // key of st[0][0]
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = key0 + 32 * sb + 8 * (r >> 2) + (r & 3);
                    st[sb][r] = key <= key_lim ? st[sb][r] : kNegInf;
                }
        }
        float mt = kNegInf;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, st[sb][r]);
        mt = fmaxf(mt, swap_halves(mt)) * c;
        // m = -inf (nothing seen yet) always moves: -inf + kLazy is -inf
        const float m_new = mt > m + kLazy ? mt : m;
        const float base = safe_base(m_new);
        const float alpha = fast_exp2(m - base);  // 1 when m stays; 0 when m = -inf
        float ps = 0.0f;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float e = fast_exp2(fmaf(st[sb][r], c, -base));
                // exactly 0 for hidden keys (exp2 of c * -inf is NaN when c = 0)
                if (MASK) e = st[sb][r] == kNegInf ? 0.0f : e;
                st[sb][r] = e;
                ps += e;
            }
        l = alpha * l + ps;
        m = m_new;
        return alpha;
    }

    // O^T = alpha O^T + V^T P^T.  A operand for output rows 32 b .. 32 b + 31 and key
    // group g: lane l needs V[16 g + 4 half + t][32 b + l32] (t = 0..3) and
    // V[16 g + 8 + 4 half + t][32 b + l32], read transposed from row-major V.
    __device__ __forceinline__ void pv(const f32x16 (&pt)[2], float alpha, const uint16_t* vtile) {
        if (__ballot(alpha != 1.0f) != 0) {  // skipped when no running max moved
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[b][r] *= alpha;
        }
        bf16x8 pf[4];  // P^T fragments: this lane's values 8 hb .. 8 hb + 7 of each half
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                u32x4 w;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    w[t] = pack_bf16x2(pt[sb][8 * hb + 2 * t], pt[sb][8 * hb + 2 * t + 1]);
                pf[2 * sb + hb] = __builtin_bit_cast(bf16x8, w);
            }
        const uint16_t* vb = vtile + v_off;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint16_t* pa = vb + 16 * g * Smem<D>::vStride + 32 * b;
                const i16x4 lo = lds_read_tr16(pa);
                const i16x4 hi = lds_read_tr16(pa + 8 * Smem<D>::vStride);
                const bf16x8 a =
                    __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[g], acc[b], 0, 0, 0);
            }
    }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(Params p) {
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    __shared__ Smem<D> sm;

    // XCD-aware remap: block id b runs on XCD b % 8; give each XCD a contiguous
    // range of logical ids.
    const int nb = p.n_blocks;
    int lid = blockIdx.x;
    if ((nb & 7) == 0) lid = (lid & 7) * (nb >> 3) + (lid >> 3);
    const int bh = lid / p.n_qtiles;
    int qt = lid % p.n_qtiles;
    if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // longest tiles first

    const int N = p.N;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int64_t head = (int64_t)bh * N * D;
    const uint16_t* kh = p.k + head;
    const uint16_t* vh = p.v + head;

    const int q0 = qt * kBM;
    const int qw0 = q0 + 32 * wave;  // this wavefront's first query row
    const int qw_last = min(qw0 + 31, N - 1);
    const bool wave_live = qw0 < N;

    Wave<D, CAUSAL> w;
    w.l32 = lane & 31;
    w.half = lane >> 5;
    w.my_q = qw0 + w.l32;
    w.key_lim = CAUSAL ? min(N - 1, w.my_q) : N - 1;  // last visible key of the row
    w.c = p.scale_log2;
    w.m = kNegInf;
    w.l = 0.0f;
    // K fragment of lane l: row l32 (+32 sb) of the tile, columns 16 ks + 8 half.
    w.k_off = w.l32 * Smem<D>::kStride + 8 * w.half;
    // Lane's block for the transposing V reads: row 4 half + (lane % 16) / 4 of the
    // key group, columns 16 ((lane / 16) % 2) + 4 (lane % 4) of the output block.
    w.v_off = (4 * w.half + ((lane & 15) >> 2)) * Smem<D>::vStride + 16 * ((lane >> 4) & 1) +
              4 * (lane & 3);

    // Q^T fragments: lane supplies Q[my_q][16 s + 8 half + 0..7].  With a negative
    // scale the query is negated (exact in bf16) and |scale| used, so the row maximum
    // of the raw products is the maximum of the scaled scores.
    const uint32_t qsign = p.negate_q ? 0x80008000u : 0u;
    const int q_row = min(w.my_q, N - 1);  // rows past the end compute garbage, never stored
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const u32x4 v4 =
            *reinterpret_cast<const u32x4*>(p.q + head + (int64_t)q_row * D + 16 * s + 8 * w.half);
        w.qf[s] = __builtin_bit_cast(bf16x8, v4 ^ qsign);
    }
#pragma unroll
    for (int b = 0; b < DB; ++b) w.acc[b] = f32x16{};

    const int q_last = min(q0 + kBM - 1, N - 1);
    const int n_kv = CAUSAL ? (q_last / kBN + 1) : (N + kBN - 1) / kBN;

    // Software pipeline over key tiles.  Iteration j reads K_{j+1} (scores of the next
    // tile, on the matrix cores) and V_j (output of this tile), while the vector ALUs
    // run the softmax of tile j; meanwhile K_{j+2} and V_{j+1} travel from HBM to
    // registers and are written to the buffers that iteration j-1 finished reading.
    // K is therefore one tile ahead of V; one barrier per tile orders it all.
    Prefetch<D> kpf, vpf;
    kpf.load(kh, 0, N, tid);
    vpf.load(vh, 0, N, tid);
    kpf.store(sm.k[0], Smem<D>::kStride, tid);
    vpf.store(sm.v[0], Smem<D>::vStride, tid);
    if (n_kv > 1) {
        kpf.load(kh, kBN, N, tid);
        kpf.store(sm.k[1], Smem<D>::kStride, tid);
    }
    __syncthreads();
    f32x16 sa[2], sb[2];
    if (wave_live) w.qk(sa, sm.k[0]);
    __syncthreads();  // K buffer 0 may now be refilled

    auto step = [&](int j, f32x16(&sc)[2], f32x16(&sn)[2]) {
        const int j0 = j * kBN;
        const bool has_next = j + 1 < n_kv;
        const bool act_cur = wave_live && (!CAUSAL || j0 <= qw_last);
        const bool act_next = wave_live && has_next && (!CAUSAL || j0 + kBN <= qw_last);
        const bool pf_k = j + 2 < n_kv;
        if (pf_k) kpf.load(kh, j0 + 2 * kBN, N, tid);
        if (has_next) vpf.load(vh, j0 + kBN, N, tid);
        const bool mask_cur = (CAUSAL && j0 + kBN - 1 > qw0) || (j0 + kBN > N);
        const uint16_t* kn = sm.k[(j + 1) & 1];
        float alpha = 1.0f;
        if (act_cur && act_next && !mask_cur) {
            // steady state: next tile's scores and this tile's softmax in one block
            w.qk(sn, kn);
            alpha = w.template softmax<false>(sc, j0);
            // Interleave: each of the 16 matrix instructions (32 cycles on the matrix
            // core) is followed by a run of the softmax's vector instructions, which
            // do not depend on it, so both units stay busy.
            // K fragments are read two matrix instructions ahead of their use.
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS reads (K fragments)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                if (i < 14) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // vector ALU
            }
        } else {
            if (act_next) w.qk(sn, kn);
            if (act_cur) alpha = mask_cur ? w.template softmax<true>(sc, j0) : w.template softmax<false>(sc, j0);
        }
        if (act_cur) w.pv(sc, alpha, sm.v[j & 1]);
        if (pf_k) kpf.store(sm.k[j & 1], Smem<D>::kStride, tid);
        if (has_next) vpf.store(sm.v[(j + 1) & 1], Smem<D>::vStride, tid);
        __syncthreads();
    };

    int j = 0;
    for (; j + 1 < n_kv; j += 2) {
        step(j, sa, sb);
        step(j + 1, sb, sa);
    }
    if (j < n_kv) step(j, sa, sb);

    if (!wave_live) return;
    const float l_row = w.l + swap_halves(w.l);
    if (w.my_q < N) {
        const float inv = 1.0f / l_row;
        uint16_t* orow = p.o + head + (int64_t)w.my_q * D;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u32x2 o2;
                o2[0] = pack_bf16x2(w.acc[b][4 * i + 0] * inv, w.acc[b][4 * i + 1] * inv);
                o2[1] = pack_bf16x2(w.acc[b][4 * i + 2] * inv, w.acc[b][4 * i + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + 32 * b + 8 * i + 4 * w.half) = o2;
            }
        }
        if (w.half == 0) p.lse[(int64_t)bh * N + w.my_q] = (w.m + fast_log2(l_row)) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const Params& p, hipStream_t st) {
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)p.n_blocks), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                int H, int N, int d, float scale, bool causal, hipStream_t st) {
    Params p;
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.o = static_cast<uint16_t*>(o);
    p.lse = lse;
    p.N = N;
    p.n_qtiles = (N + kBM - 1) / kBM;
    const int64_t blocks = (int64_t)B * H * p.n_qtiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    p.n_blocks = (int)blocks;
    p.scale_log2 = fabsf(scale) * kLog2e;
    p.negate_q = scale < 0.0f;
    if (d == 64) return causal ? launch<64, true>(p, st) : launch<64, false>(p, st);
    if (d == 128) return causal ? launch<128, true>(p, st) : launch<128, false>(p, st);
    return hipErrorInvalidValue;
}

}  // namespace mi355
