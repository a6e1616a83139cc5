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
//   * The rescale of O is skipped when alpha is exactly 1 on every lane of the
//     wavefront (the running maxima did not move), which is exact.
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

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const __bf16 a = (__bf16)lo, b = (__bf16)hi;  // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

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

// Global -> register -> LDS staging of one key/value tile (64 keys x D), both
// row-major, 16 bytes per access: consecutive threads take consecutive 16-byte
// chunks of a row, so global reads are fully coalesced and LDS writes are free of
// bank conflicts.
template <int D>
struct Stage {
    static constexpr int kChunks = kBN * D / 8 / 256;  // 16-byte chunks per thread per tensor
    u32x4 kr[kChunks];
    u32x4 vr[kChunks];

    __device__ __forceinline__ void load(const uint16_t* kh, const uint16_t* vh, int j0, int N, int tid) {
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int idx = tid + 256 * c;
            // Rows past the end re-read row N-1: their scores are masked to -inf and
            // their probabilities are 0, so any finite content will do.
            const int key = min(j0 + idx / (D / 8), N - 1);
            const int64_t off = (int64_t)key * D + (idx % (D / 8)) * 8;
            kr[c] = *reinterpret_cast<const u32x4*>(kh + off);
            vr[c] = *reinterpret_cast<const u32x4*>(vh + off);
        }
    }

    __device__ __forceinline__ void store(Smem<D>& sm, int buf, int tid) const {
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int idx = tid + 256 * c;
            const int key = idx / (D / 8);
            const int col = (idx % (D / 8)) * 8;
            *reinterpret_cast<u32x4*>(&sm.k[buf][key * Smem<D>::kStride + col]) = kr[c];
            *reinterpret_cast<u32x4*>(&sm.v[buf][key * Smem<D>::vStride + col]) = vr[c];
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

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(Params p) {
    constexpr int KS = D / 16;  // k-steps of Q K^T
    constexpr int DB = D / 32;  // 32-wide blocks of the output dimension
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
    const int l32 = lane & 31;
    const int half = lane >> 5;
    // Lane's block for the transposing V reads: row 4 half + (lane % 16) / 4 of the
    // key group, columns 16 ((lane / 16) % 2) + 4 (lane % 4) of the output block.
    const int v_lane_off = (4 * half + ((lane & 15) >> 2)) * Smem<D>::vStride +
                           16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int64_t head = (int64_t)bh * N * D;
    const uint16_t* kh = p.k + head;
    const uint16_t* vh = p.v + head;

    const int q0 = qt * kBM;
    const int qw0 = q0 + 32 * wave;          // this wavefront's first query row
    const int my_q = qw0 + l32;              // the query row this lane owns
    const int qw_last = min(qw0 + 31, N - 1);
    const bool wave_live = qw0 < N;

    // Q^T fragments (B operand): lane supplies Q[my_q][16 s + 8 half + 0..7].
    // With a negative scale the query is negated (exact in bf16) and |scale| used, so
    // the row maximum of the raw products is the maximum of the scaled scores.
    bf16x8 qf[KS];
    const uint32_t qsign = p.negate_q ? 0x80008000u : 0u;
    const int q_row = min(my_q, N - 1);  // rows past the end compute garbage, never stored
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(p.q + head + (int64_t)q_row * D + 16 * s + 8 * half);
        qf[s] = __builtin_bit_cast(bf16x8, w ^ qsign);
    }

    f32x16 acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = f32x16{};
    float m = kNegInf;  // running max of scale * log2e * score, this lane's row
    float l = 0.0f;     // running partial sum over this lane's half of each tile

    const int q_last = min(q0 + kBM - 1, N - 1);
    const int n_kv = CAUSAL ? (q_last / kBN + 1) : (N + kBN - 1) / kBN;

    Stage<D> stage;
    stage.load(kh, vh, 0, N, tid);
    stage.store(sm, 0, tid);
    __syncthreads();

    for (int j = 0; j < n_kv; ++j) {
        const int buf = j & 1;
        const int j0 = j * kBN;
        if (j + 1 < n_kv) stage.load(kh, vh, j0 + kBN, N, tid);

        const bool active = wave_live && (!CAUSAL || j0 <= qw_last);
        if (active) {
            // ---- S^T = K Q^T for the two 32-key halves of the tile
            f32x16 s[2] = {f32x16{}, f32x16{}};
            const uint16_t* kb = &sm.k[buf][0];
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                        kb + (32 * sb + l32) * Smem<D>::kStride + 16 * ks + 8 * half);
                    s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[sb], 0, 0, 0);
                }
            }

            // ---- row max of the raw products (scale >= 0 after the sign flip of Q);
            // on diagonal / ragged tiles hidden keys take no part.
            const bool need_mask = (CAUSAL && j0 + kBN - 1 > qw0) || (j0 + kBN > N);
            int key_lim = N - 1;  // last visible key of this lane's row
            if (CAUSAL) key_lim = min(key_lim, my_q);
            const int key0 = j0 + 4 * half;  // key of s[0][0]
            float mt = kNegInf;
            if (need_mask) {
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = key0 + 32 * sb + 8 * (r >> 2) + (r & 3);
                        s[sb][r] = key <= key_lim ? s[sb][r] : kNegInf;
                    }
            }
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[sb][r]);
            mt = fmaxf(mt, swap_halves(mt));
            // m is kept in log2 units of the scaled score: c * max(raw), c = |scale| log2 e
            const float m_new = fmaxf(m, mt * p.scale_log2);
            const float base = safe_base(m_new);
            const float alpha = fast_exp2(m - base);  // m = -inf gives 0

            // ---- P = exp2(c s - m_new) with one FMA per score, partial row sums.
            // Hidden keys get exactly 0 (not exp2 of c * -inf, which is NaN at c = 0).
            float ps = 0.0f;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float e = fast_exp2(fmaf(s[sb][r], p.scale_log2, -base));
                    if (need_mask) e = s[sb][r] == kNegInf ? 0.0f : e;
                    s[sb][r] = e;
                    ps += e;
                }
            }
            l = alpha * l + ps;
            m = m_new;

            // ---- rescale O (skipped when no running max moved: alpha == 1 exactly)
            if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
                for (int b = 0; b < DB; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[b][r] *= alpha;
            }

            // ---- P^T fragments: lane's values 8 hb .. 8 hb + 7 of each half-tile
            bf16x8 pf[4];
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    u32x4 w;
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        w[t] = pack_bf16x2(s[sb][8 * hb + 2 * t], s[sb][8 * hb + 2 * t + 1]);
                    pf[2 * sb + hb] = __builtin_bit_cast(bf16x8, w);
                }
            }

            // ---- O^T += V^T P^T.  A operand for output rows 32 b .. 32 b + 31 and key
            // group g: lane l needs V[16 g + 4 half + t][32 b + l32] (t = 0..3) and
            // V[16 g + 8 + 4 half + t][32 b + l32]; each lane of a 16-lane group
            // points at one 4-element block of those rows (see v_lane_off).
            const uint16_t* vb = &sm.v[buf][v_lane_off];
#pragma unroll
            for (int b = 0; b < DB; ++b) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint16_t* pa = vb + 16 * g * Smem<D>::vStride + 32 * b;
                    const i16x4 lo = lds_read_tr16(pa);
                    const i16x4 hi = lds_read_tr16(pa + 8 * Smem<D>::vStride);
                    const bf16x8 a = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[g], acc[b], 0, 0, 0);
                }
            }
        }

        if (j + 1 < n_kv) stage.store(sm, buf ^ 1, tid);
        __syncthreads();
    }

    if (!wave_live) return;
    const float l_row = l + swap_halves(l);
    if (my_q < N) {
        const float inv = 1.0f / l_row;
        uint16_t* orow = p.o + head + (int64_t)my_q * D;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u32x2 w;
                w[0] = pack_bf16x2(acc[b][4 * i + 0] * inv, acc[b][4 * i + 1] * inv);
                w[1] = pack_bf16x2(acc[b][4 * i + 2] * inv, acc[b][4 * i + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + 32 * b + 8 * i + 4 * half) = w;
            }
        }
        if (half == 0) p.lse[(int64_t)bh * N + my_q] = (m + fast_log2(l_row)) * kLn2;
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
