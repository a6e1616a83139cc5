// attn_bwd_bf16.hip — gradients of bf16 attention (dQ, dK, dV) on gfx950 matrix cores,
// recomputing the probabilities from the row statistics saved by the forward.
//
// What is computed: for O = softmax(scale Q K^T) V (causal or not) and an upstream
// gradient dO, the derivative of that definition,
//     P = exp(scale Q K^T - LSE)        (recomputed; LSE = m + ln l from the forward)
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D_i = dO_i . O_i
//     dQ = scale dS K,   dK = scale dS^T Q.
// D_i equals sum_j P_ij dP_ij (the softmax Jacobian's row term) because O_i = sum_j
// P_ij V_j.  Keeping only LSE and recomputing P tile by tile instead of storing the
// N x N probabilities is the pages' account of the backward pass ("Softmax numerical
// stability and IO-aware attention", section 7.2 and question 4).
//
// Two kernels, enqueued in order on one stream:
//   1. dQ: one block per 128 query rows, 4 wavefronts of 32 rows, streaming 64-key
//      tiles of K and V through LDS.  The layout is the forward's: S^T = K Q^T and
//      dP^T = V dO^T put one query row in each lane (Q and dO fragments stay in
//      registers), dS^T is formed in place and packed to bf16, and
//      dQ^T += K^T dS^T reads K^T with the transposing LDS load.  Each lane first forms
//      D_i = dO_i . O_i for its row from the O and dO fragments (half the columns,
//      plus the other half from its partner lane) and LSE_i log2(e), and the block
//      writes both into the caller's workspace for the second kernel.
//   2. dK/dV: one block per 128 keys, 8 wavefronts (4 groups of 32 keys, two roles per
//      group), streaming 64-row tiles of Q, dO, LSE and D through LDS.  Here S = Q K^T
//      and dP = dO V^T put one key in each lane (K or V fragments stay in registers);
//      P and dS, packed to bf16 as they lie, are the B operands of dV^T += dO^T P and
//      dK^T += Q^T dS, whose A operands are transposing reads of the dO and Q tiles.
//      One role computes S, P and dV, the other dP, dS and dK, with P passed through
//      LDS.  At d = 128 the roles run a tile apart with one barrier per tile; at
//      d = 64 they meet twice per tile (see the two kernels).
// Computing dQ in its own pass (recomputing S and dP there) keeps every gradient
// element owned by one lane of one block: no atomics, and results are bitwise
// repeatable.
//
// LDS tiles are unpadded rows with 16-byte chunks XOR-permuted by swz(row), a
// permutation under which both access patterns used on the same tile are free of
// bank conflicts: 16-byte reads of one chunk of 16 consecutive rows, and transposing
// reads of 32 bytes from rows 4h..4h+3 of an 8-row group.
#include <type_traits>

#include "device_common.hpp"
#include "launchers.hpp"
#include "mfma_bf16.hpp"

namespace mi355 {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdRows = 32 * kBwdWaves;    // query rows (dQ) or keys (dK/dV) per block
constexpr int kT = 64;                      // rows per streamed tile
constexpr int kDkdvWaves = 8;               // dK/dV: two roles x four key groups
constexpr int kDkdvThreads = 64 * kDkdvWaves;

template <int D>
struct BLayout {
    static constexpr int RB = 2 * D;               // bytes per row
    static constexpr int NCH = RB / 16;            // 16-byte chunks per row
    static constexpr int TILE = kT * RB;           // bytes per tile
    // Chunk position of logical chunk c in row r is c ^ swz(r).  d = 128 (a row spans
    // all 64 banks): the low two bits of the row pick bits 2..3 of the permutation and
    // bits 2..3 of the row pick bits 0..1, so 16 consecutive rows see 16 different
    // positions and rows 4h..4h+3 see chunk pairs {c, c+1} at 4 different places.
    // d = 64 (two rows per bank line): the same with row bit 1 in place of bits 0..1.
    // Both depend only on row mod 16, which the per-round copy offsets rely on.
    __device__ static constexpr int swz(int r) {
        return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
    }
};

struct BwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* dout;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    const uint16_t* o;   // the forward's output
    const float* lse;    // the forward's LSE
    float* delta;        // [B*H*N]  D_i = dO_i . O_i       (written by dQ, read by dK/dV)
    float* lse2;         // [B*H*N]  LSE_i * log2(e)     (written by dQ, read by dK/dV)
    int N;
    int n_tiles;         // ceil(N / kBwdRows)
    int n_blocks;
    float c;             // scale * log2(e)
    float scale;
};

// One 64-row tile of a [N, D] bf16 slab (rows r0 .. r0 + 63 of `head`) from HBM
// straight to LDS, by all THREADS threads of the block; `src_off` is the thread's
// fixed source offset within a round (see the kernels).  Rows at or past N read as
// zeros; live = false fills the tile with zeros without reading memory.
template <int D, int THREADS = kBwdThreads>
__device__ __forceinline__ void tile_to_lds(char* lds, const uint16_t* head, int r0, int N, int wave,
                                            int src_off, bool live) {
    using L = BLayout<D>;
    constexpr int kRound = 16 * THREADS;  // bytes one block-wide 16-byte copy moves
    constexpr int kRounds = L::TILE / kRound;
    const int rows = live ? min(N - r0, kT) : 0;
    const char* base = reinterpret_cast<const char*>(head) + (live ? (int64_t)r0 * L::RB : 0);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, rows * L::RB, kBufferWord3);
    char* dst = lds + 1024 * wave;  // the wave's 1 KiB of each round; lane offset implicit
#pragma unroll
    for (int r = 0; r < kRounds; ++r)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + kRound * r), 16, src_off, kRound * r, 0,
                                                 0);
}

// 64 floats (rows r0 .. r0 + 63 of a per-row vector) to LDS by one wavefront; rows at
// or past N read as zeros.
__device__ __forceinline__ void rowvec_to_lds(float* lds, const float* vec, int r0, int N, int lane, bool live) {
    const int rows = live ? min(N - r0, kT) : 0;
    const float* base = vec + (live ? r0 : 0);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, rows * 4, kBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds, 4, 4 * lane, 0, 0, 0);
}

// Block barrier for LDS data written with ds_write: waits for this wavefront's LDS
// operations only, not for HBM -> LDS copies still in flight (a workgroup fence would
// wait for those too, since they write LDS).  The asm statement is also a compiler
// barrier for memory accesses.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

// Per-lane LDS offsets for the two access patterns on a BLayout<D> tile.  The swizzle
// permutes chunk bits that the k-step (bits 1.. of the chunk index) and the output
// block (bits 2.. of it) occupy, and never carries, so every offset is the k-step 0 or
// block 0 offset with those bits flipped: one register per pattern.
template <int D>
struct TileReads {
    using L = BLayout<D>;
    int row0;    // 16-byte read of row l32 (+32 sb), logical chunk h; chunk 2 ks + h at row0 ^ 32 ks
    int tr_lo0;  // transposing read for output columns 0 .. 31, rows 4h + (lane%16)/4;
                 // columns 32 b .. at tr_lo0 ^ 64 b
    int tr_hi0;  // the same 8 rows further down
    __device__ int row(int ks) const { return row0 ^ (32 * ks); }
    __device__ int tr_lo(int b) const { return tr_lo0 ^ (64 * b); }
    __device__ int tr_hi(int b) const { return tr_hi0 ^ (64 * b); }
    __device__ void init(int lane) {
        const int l32 = lane & 31, h = lane >> 5;
        row0 = l32 * L::RB + 16 * (h ^ L::swz(l32));
        const int vr = 4 * h + ((lane & 15) >> 2);
        const int col = 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
        tr_lo0 = vr * L::RB + 16 * ((col >> 4) ^ L::swz(vr)) + (col & 15);
        tr_hi0 = (vr + 8) * L::RB + 16 * ((col >> 4) ^ L::swz(vr + 8)) + (col & 15);
    }
};

// acc (32 rows of the tile from row 32 sb, x 32 columns) = A B: A = 16-byte row reads of
// `tile` (rows = the accumulator's rows, k = the D columns), B = frag (per lane: column
// l32, k-slots 8h..8h+7 of each 16-wide k-step).  AHEAD: all of the sub-block's A
// operands are read before the first product (kernels with registers to spare), so that
// the products do not wait on LDS latency one pair at a time.
template <int D, bool AHEAD = false>
__device__ __forceinline__ f32x16 rows_times_frag(const char* tile, int sb, const TileReads<D>& rd,
                                                  const bf16x8 (&frag)[D / 16]) {
    f32x16 a = f32x16{};
    if (AHEAD) {
        bf16x8 t[D / 16];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            t[ks] = *reinterpret_cast<const bf16x8*>(tile + 32 * sb * BLayout<D>::RB + rd.row(ks));
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t[ks], frag[ks], a, 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 0);  // every read, then
        __builtin_amdgcn_sched_group_barrier(0x008, D / 16, 0);  // every product
        return a;
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 t = *reinterpret_cast<const bf16x8*>(tile + 32 * sb * BLayout<D>::RB + rd.row(ks));
        a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t, frag[ks], a, 0, 0, 0);
    }
    return a;
}

// acc[b] (output columns 32 b.., x 32 lanes' columns) += T^T B over the 16 tile rows
// of group g: A = transposing reads of `tile`, B = the packed operand for group g.
template <int D, bool AHEAD = false>
__device__ __forceinline__ void trans_times_packed(f32x16 (&acc)[D / 32], const char* tile, int g,
                                                   const TileReads<D>& rd, const bf16x8& bop) {
    const char* base = tile + 16 * g * BLayout<D>::RB;
    if (AHEAD) {
        bf16x8 a[D / 32];
#pragma unroll
        for (int b = 0; b < D / 32; ++b) a[b] = lds_read_tr_pair(base + rd.tr_lo(b), base + rd.tr_hi(b));
#pragma unroll
        for (int b = 0; b < D / 32; ++b) acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[b], bop, acc[b], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, D / 32, 0);
        return;
    }
#pragma unroll
    for (int b = 0; b < D / 32; ++b) {
        const bf16x8 a = lds_read_tr_pair(base + rd.tr_lo(b), base + rd.tr_hi(b));
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc[b], 0, 0, 0);
    }
}

// Fragment of a row-major [*, D] bf16 slab for a B operand: lane supplies row `row`,
// columns 16 ks + 8 h .. + 7.
template <int D>
__device__ __forceinline__ void load_frag(bf16x8 (&f)[D / 16], const uint16_t* slab, int row, int h) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
        f[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(slab + (int64_t)row * D + 16 * ks + 8 * h));
}

// Packs 8 consecutive accumulator entries (v = 8 t .. 8 t + 7) into one bf16x8 B operand.
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int t) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[8 * t + 2 * i], x[8 * t + 2 * i + 1]);
    return __builtin_bit_cast(bf16x8, w);
}

// Stores an accumulator pair layout (lane: row `row` of the output, columns
// 32 b + 8 (v/4) + 4 h + v%4) as bf16, multiplied by `mul`.
template <int D>
__device__ __forceinline__ void store_rows(uint16_t* out, int row, int h, const f32x16 (&acc)[D / 32], float mul) {
    uint16_t* orow = out + (int64_t)row * D;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x2 o2;
            o2[0] = pack_bf16x2(acc[b][4 * i + 0] * mul, acc[b][4 * i + 1] * mul);
            o2[1] = pack_bf16x2(acc[b][4 * i + 2] * mul, acc[b][4 * i + 3] * mul);
            *reinterpret_cast<u32x2*>(orow + 32 * b + 8 * i + 4 * h) = o2;
        }
}

// Logical block id -> (head, tile) with the forward's XCD-aware remap; causal grids
// run their longest tiles first (`longest_last`: the tile index with the most work is
// the last one for dQ, the first one for dK/dV).  In causal grids an XCD takes its heads
// in groups of G and runs each group's tiles longest first across the group, so that
// the tail of each group's work is short tiles of all its heads: G = 4 when the XCD has a
// multiple of 8 heads, 2 for a multiple of 4, else 1.  Timed interleaved against one head
// at a time (bitwise identical gradients): +1-2% at B=2 H=32 N=8192 d=128, +7-8% at
// B=4 H=16 N=4096 d=128, +5% at B=2 H=32 N=8192 d=64; all of an XCD's heads at once
// (G = 8 there) lost 1% at the first shape, and at B=1 H=32 N=16384 (4 heads per XCD)
// pairs gained 0.7% where G = 4 lost 1%.  The price is HBM reads: four heads' streams
// outgrow the XCD's L2 and the two kernels fetch 2.1-2.8 times their operands (0.8 TB/s
// at the first shape), while both stay matrix-core bound.
__device__ __forceinline__ void block_coords(const BwdParams& p, bool causal, bool longest_last, int& bh, int& t) {
    const int nb = p.n_blocks;
    int lid = blockIdx.x;
    if ((nb & 7) == 0) lid = (lid & 7) * (nb >> 3) + (lid >> 3);
    const int nt = p.n_tiles;
    bh = lid / nt;
    t = lid % nt;
    if (!causal) return;
    const int per_xcd = nb >> 3;
    const int hx = ((nb & 7) == 0 && per_xcd % nt == 0) ? per_xcd / nt : 0;  // heads per XCD
    const int G = hx == 0 ? 1 : hx % 8 == 0 ? 4 : hx % 4 == 0 ? 2 : 1;
    if (G > 1) {
        const int x = lid / per_xcd, li = lid % per_xcd;
        const int g = li / (G * nt), r = li % (G * nt);
        bh = x * hx + G * g + r % G;
        t = r / G;
    }
    if (longest_last) t = nt - 1 - t;
}

// ---------------------------------------------------------------------------------
// 1. dQ.  Lane: query row q = q0 + 32 wave + l32; S^T / dP^T rows are keys.
// ---------------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 2) void attn_bwd_dq_kernel(BwdParams p) {
    using L = BLayout<D>;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    // Double buffers as separate objects, selected at compile time, so that the compiler
    // can tell the buffer being filled from the one being read (it would otherwise wait
    // for the copies in flight before every read).
    __shared__ __attribute__((aligned(1024))) char k_lds0[L::TILE];
    __shared__ __attribute__((aligned(1024))) char k_lds1[L::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds0[L::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds1[L::TILE];

    int bh, qt;
    block_coords(p, CAUSAL, true, bh, qt);
    const int N = p.N;
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t head = (int64_t)bh * N * D;
    const int q0 = qt * kBwdRows;
    const int qw0 = q0 + 32 * wave;
    const int my_q = qw0 + l32;
    const int q_row = min(my_q, N - 1);  // rows past the end compute garbage, never stored

    const int t_row = tid / L::NCH, t_pos = tid % L::NCH;
    const int src_off = t_row * L::RB + 16 * (t_pos ^ L::swz(t_row));
    TileReads<D> rd;
    rd.init(lane);

    bf16x8 qf[KS], dof[KS];
    load_frag<D>(qf, p.q + head, q_row, h);
    load_frag<D>(dof, p.dout + head, q_row, h);
    // D = dO . O of the lane's row (its half of the columns here, the other half in lane
    // l ^ 32) and LSE log2(e); the block's rows are written for the dK/dV pass.
    float dlt = 0.0f;
    {
        bf16x8 of[KS];
        load_frag<D>(of, p.o + head, q_row, h);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 a = __builtin_bit_cast(u32x4, of[ks]);
            const u32x4 b = __builtin_bit_cast(u32x4, dof[ks]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dlt = fmaf(__uint_as_float(a[i] << 16), __uint_as_float(b[i] << 16), dlt);
                dlt = fmaf(__uint_as_float(a[i] & 0xffff0000u), __uint_as_float(b[i] & 0xffff0000u), dlt);
            }
        }
        dlt += __shfl_xor(dlt, 32, 64);
    }
    const float lse2 = p.lse[(int64_t)bh * N + q_row] * kLog2e;
    if (h == 0 && my_q < N) {
        p.delta[(int64_t)bh * N + my_q] = dlt;
        p.lse2[(int64_t)bh * N + my_q] = lse2;
    }
    const int key_lim = CAUSAL ? min(N - 1, my_q) : N - 1;

    f32x16 acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = f32x16{};

    const int q_last = min(q0 + kBwdRows - 1, N - 1);
    const int n_kv = CAUSAL ? q_last / kT + 1 : (N + kT - 1) / kT;
    const bool wave_live = qw0 < N;
    const int n_w = !wave_live ? 0 : CAUSAL ? min(n_kv, min(qw0 + 31, N - 1) / kT + 1) : n_kv;

    tile_to_lds<D>(k_lds0, p.k + head, 0, N, wave, src_off, true);
    tile_to_lds<D>(v_lds0, p.v + head, 0, N, wave, src_off, true);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();

    // tile j; PAR = j % 2 at compile time
    auto tile = [&](auto par, int j) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par)::value;
        // prefetch the next tile into the other buffers (read two barriers ago)
        tile_to_lds<D>(PAR ? k_lds0 : k_lds1, p.k + head, (j + 1) * kT, N, wave, src_off, j + 1 < n_kv);
        tile_to_lds<D>(PAR ? v_lds0 : v_lds1, p.v + head, (j + 1) * kT, N, wave, src_off, j + 1 < n_kv);
        if (j < n_w) {
            const char* kt = PAR ? k_lds1 : k_lds0;
            const char* vt = PAR ? v_lds1 : v_lds0;
            const int j0 = j * kT;
            // the mask is a compile-time choice so that whole tiles (the common case) run
            // without per-element branches
            auto body = [&](auto masked_c) __attribute__((always_inline)) {
                constexpr bool MASKED = decltype(masked_c)::value;
                // key j0 + 32 sb + 8 (r / 4) + 4 h + r % 4 is visible when its offset from
                // j0 + 4 h is at most lim (a compile-time offset against one register)
                const int lim = key_lim - j0 - 4 * h;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    f32x16 s = rows_times_frag<D>(kt, sb, rd, qf);    // S^T rows = keys
                    f32x16 dp = rows_times_frag<D>(vt, sb, rd, dof);  // dP^T
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float pr = fast_exp2(fmaf(s[r], p.c, -lse2));
                        if (MASKED) pr = 32 * sb + 8 * (r >> 2) + (r & 3) <= lim ? pr : 0.0f;
                        s[r] = pr * (dp[r] - dlt);  // dS^T
                    }
                    trans_times_packed<D>(acc, kt, 2 * sb + 0, rd, pack8(s, 0));
                    trans_times_packed<D>(acc, kt, 2 * sb + 1, rd, pack8(s, 1));
                }
            };
            if ((CAUSAL && j0 + kT - 1 > qw0) || (j0 + kT > N)) body(std::true_type{});
            else body(std::false_type{});
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next tiles have landed
        __syncthreads();
    };
    int j = 0;
    for (; j + 1 < n_kv; j += 2) {
        tile(std::integral_constant<int, 0>{}, j);
        tile(std::integral_constant<int, 1>{}, j + 1);
    }
    if (j < n_kv) tile(std::integral_constant<int, 0>{}, j);
    if (wave_live && my_q < N) store_rows<D>(p.dq + head, my_q, h, acc, p.scale);
}

// ---------------------------------------------------------------------------------
// 2a. dK and dV at d = 128, the two roles pipelined.  8 wavefronts, 128 keys: key
//    group kg = wave % 4 owns keys k0 + 32 kg + l32 (one key per lane), in two roles
//    that share a SIMD (waves w and w + 4).  The roles run one query tile apart, with
//    one barrier per tile.  In step
//    s (query tile i = i_begin + s):
//      role A (w < 4):  S = Q_i K^T, P = exp2(c S - LSE) -> P_i to LDS (fp32), then
//                       P packed to bf16 and dV^T += dO_i^T P
//      role B (w >= 4): dS = P_{i-1} (dP - D)_{i-1} with P_{i-1} from LDS and
//                       (dP - D)_{i-1} kept in registers since the previous step,
//                       dK^T += Q_{i-1}^T dS;  then (dP - D)_i = dO_i V^T - D_i
//    Both roles issue 32 matrix instructions per step and neither waits for the other
//    inside it; the barrier at the end of the step makes P_i visible to role B and
//    frees the buffers that the next step's copies overwrite.  Role B reads Q_{i-1}
//    while tile i + 1 is being copied, so Q has three LDS buffers (dO, LSE, D and the
//    P exchange two each).  After the last step role B finishes its tile alone.  Every
//    sub-block is computed; P is zero wherever a score is hidden (the mask is applied
//    once, in role A), so dS, dK and dV need no mask.  Role A runs at raised issue
//    priority so that its products, whose results its exponentials wait for, go first.
//    Results are bitwise those of the two-phase kernel below, which is faster at
//    d = 64: there its 66 KiB of LDS let two blocks share a CU, where this kernel's
//    five tile buffers and two P buffers (105 KiB at d = 64) leave one.
// ---------------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kDkdvThreads, 1) void attn_bwd_dkdv_kernel(BwdParams p) {
    using L = BLayout<D>;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    // Buffers as separate objects, selected at compile time (see the dQ kernel).
    __shared__ __attribute__((aligned(1024))) char q_lds0[L::TILE];
    __shared__ __attribute__((aligned(1024))) char q_lds1[L::TILE];
    __shared__ __attribute__((aligned(1024))) char q_lds2[L::TILE];
    __shared__ __attribute__((aligned(1024))) char do_lds0[L::TILE];
    __shared__ __attribute__((aligned(1024))) char do_lds1[L::TILE];
    __shared__ __attribute__((aligned(16))) f32x4 p_xch0[4][2][4][64];  // [kg][sb][g][lane]
    __shared__ __attribute__((aligned(16))) f32x4 p_xch1[4][2][4][64];
    __shared__ __attribute__((aligned(16))) float lse_lds0[kT];
    __shared__ __attribute__((aligned(16))) float lse_lds1[kT];
    __shared__ __attribute__((aligned(16))) float dl_lds0[kT];
    __shared__ __attribute__((aligned(16))) float dl_lds1[kT];

    int bh, kt;
    block_coords(p, CAUSAL, false, bh, kt);
    const int N = p.N;
    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave & 3;
    const bool role_a = wave < 4;
    const int64_t head = (int64_t)bh * N * D;
    const int64_t rowbase = (int64_t)bh * N;
    const int k0 = kt * kBwdRows;
    const int kw0 = k0 + 32 * kg;
    const int my_k = kw0 + (lane & 31);
    const int k_row = min(my_k, N - 1);  // keys past the end compute garbage, never stored

    const int t_row = tid / L::NCH, t_pos = tid % L::NCH;
    const int src_off = t_row * L::RB + 16 * (t_pos ^ L::swz(t_row));
    TileReads<D> rd;
    rd.init(lane);

    // role A: K fragments (B operand of S = Q K^T); role B: V fragments (dP = dO V^T)
    bf16x8 frag[KS];
    load_frag<D>(frag, (role_a ? p.k : p.v) + head, k_row, h);

    f32x16 acc[DB];  // role A: dV^T, role B: dK^T (unscaled)
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = f32x16{};

    // query tiles: causal blocks start at the tile holding their first key
    const int i_begin = CAUSAL ? k0 / kT : 0;
    const int n_q = (N + kT - 1) / kT;
    const int n_steps = n_q - i_begin;

    // buffers of step s: Q at s mod 3; dO, LSE, D and P at s mod 2
    auto q_buf = [&](auto b) -> char* {
        constexpr int B = decltype(b)::value;
        return B == 0 ? q_lds0 : B == 1 ? q_lds1 : q_lds2;
    };
    auto copy_tile = [&](auto s6, int i, bool live) __attribute__((always_inline)) {
        constexpr int S6 = decltype(s6)::value;
        tile_to_lds<D, kDkdvThreads>(q_buf(std::integral_constant<int, S6 % 3>{}), p.q + head, i * kT, N, wave,
                                     src_off, live);
        tile_to_lds<D, kDkdvThreads>(S6 % 2 ? do_lds1 : do_lds0, p.dout + head, i * kT, N, wave, src_off, live);
        if (wave == 0) rowvec_to_lds(S6 % 2 ? lse_lds1 : lse_lds0, p.lse2 + rowbase, i * kT, N, lane, live);
        if (wave == 1) rowvec_to_lds(S6 % 2 ? dl_lds1 : dl_lds0, p.delta + rowbase, i * kT, N, lane, live);
    };
    copy_tile(std::integral_constant<int, 0>{}, i_begin, true);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    // End of a step: the next tile has landed (vmcnt(0)), and the barrier publishes P.
    auto end_step = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    };

    // Role A, step s (S6 = s mod 6) on query tile i.
    auto step_a = [&](auto s6, int i) __attribute__((always_inline)) {
        constexpr int S6 = decltype(s6)::value;
        copy_tile(std::integral_constant<int, (S6 + 1) % 6>{}, i + 1, i + 1 < n_q);
        const char* qt = q_buf(std::integral_constant<int, S6 % 3>{});
        const char* dt = S6 % 2 ? do_lds1 : do_lds0;
        const float* lse_t = S6 % 2 ? lse_lds1 : lse_lds0;
        f32x4(*xch)[4][64] = S6 % 2 ? p_xch1[kg] : p_xch0[kg];
        const int i0 = i * kT;
        f32x16 x[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) x[sb] = rows_times_frag<D, true>(qt, sb, rd, frag);
        // P of sub-block sb; the mask is a compile-time choice so that whole sub-blocks
        // (the common case) run without per-element branches
        auto probs = [&](auto masked_c, int sb) __attribute__((always_inline)) {
            constexpr bool MASKED = decltype(masked_c)::value;
            // query qs0 + 8 g + 4 h + u is visible when its offset o = 8 g + u from
            // qs0 + 4 h satisfies o < n_lim and (causal) o >= k_lim
            const int qb = i0 + 32 * sb + 4 * h;
            const int n_lim = N - qb, k_lim = my_k - qb;
            f32x4 l4[4];  // rows 32 sb + 8 g + 4 h + 0..3 of the tile's LSE vector
#pragma unroll
            for (int g = 0; g < 4; ++g) l4[g] = *reinterpret_cast<const f32x4*>(&lse_t[32 * sb + 8 * g + 4 * h]);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 pv;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int r = 4 * g + u;
                    float pr = fast_exp2(fmaf(x[sb][r], p.c, -l4[g][u]));
                    if (MASKED) {
                        const int o = 8 * g + u;
                        pr = (o < n_lim && (!CAUSAL || o >= k_lim)) ? pr : 0.0f;
                    }
                    x[sb][r] = pr;
                    pv[u] = pr;
                }
                xch[sb][g][lane] = pv;
            }
        };
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int qs0 = i0 + 32 * sb;
            if ((CAUSAL && qs0 < kw0 + 31) || qs0 + 32 > N) probs(std::true_type{}, sb);
            else probs(std::false_type{}, sb);
        }
        // dV^T += dO^T P
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            trans_times_packed<D, true>(acc, dt, 2 * sb + 0, rd, pack8(x[sb], 0));
            trans_times_packed<D, true>(acc, dt, 2 * sb + 1, rd, pack8(x[sb], 1));
        }
        end_step();
    };

    // Role B: (dP - D) of the previous tile, carried across the barrier.
    f32x16 xb[2];
    // dS = P (dP - D) and dK^T += Q^T dS for the tile of step s - 1 (S6 = s mod 6).
    auto finish_b = [&](auto s6) __attribute__((always_inline)) {
        constexpr int S6 = decltype(s6)::value;
        const char* qp = q_buf(std::integral_constant<int, (S6 + 2) % 3>{});
        f32x4(*xch)[4][64] = (S6 + 1) % 2 ? p_xch1[kg] : p_xch0[kg];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            f32x4 pv[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) pv[g] = xch[sb][g][lane];
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int u = 0; u < 4; ++u) xb[sb][4 * g + u] *= pv[g][u];
            trans_times_packed<D, true>(acc, qp, 2 * sb + 0, rd, pack8(xb[sb], 0));
            trans_times_packed<D, true>(acc, qp, 2 * sb + 1, rd, pack8(xb[sb], 1));
        }
    };
    auto step_b = [&](auto s6, auto prev, int i) __attribute__((always_inline)) {
        constexpr int S6 = decltype(s6)::value;
        copy_tile(std::integral_constant<int, (S6 + 1) % 6>{}, i + 1, i + 1 < n_q);
        if constexpr (decltype(prev)::value) finish_b(s6);
        __builtin_amdgcn_sched_barrier(0);
        const char* dt = S6 % 2 ? do_lds1 : do_lds0;
        const float* dl_t = S6 % 2 ? dl_lds1 : dl_lds0;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            xb[sb] = rows_times_frag<D, true>(dt, sb, rd, frag);
            f32x4 d4[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) d4[g] = *reinterpret_cast<const f32x4*>(&dl_t[32 * sb + 8 * g + 4 * h]);
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int u = 0; u < 4; ++u) xb[sb][4 * g + u] -= d4[g][u];
        }
        end_step();
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    using I5 = std::integral_constant<int, 5>;
    // Steps 1 .. n_steps - 1 in groups of six, so that every buffer index is a
    // compile-time constant, then the remaining zero to five steps.
    const int n6 = (n_steps - 1) / 6;
    const int r6 = (n_steps - 1) % 6;
    if (role_a) {
        __builtin_amdgcn_s_setprio(1);
        step_a(I0{}, i_begin);
        int i = i_begin + 1;
        for (int g = 0; g < n6; ++g, i += 6) {
            step_a(I1{}, i);
            step_a(I2{}, i + 1);
            step_a(I3{}, i + 2);
            step_a(I4{}, i + 3);
            step_a(I5{}, i + 4);
            step_a(I0{}, i + 5);
        }
        if (r6 > 0) step_a(I1{}, i);
        if (r6 > 1) step_a(I2{}, i + 1);
        if (r6 > 2) step_a(I3{}, i + 2);
        if (r6 > 3) step_a(I4{}, i + 3);
        if (r6 > 4) step_a(I5{}, i + 4);
        __builtin_amdgcn_s_setprio(0);
    } else {
        step_b(I0{}, std::false_type{}, i_begin);
        int i = i_begin + 1;
        for (int g = 0; g < n6; ++g, i += 6) {
            step_b(I1{}, std::true_type{}, i);
            step_b(I2{}, std::true_type{}, i + 1);
            step_b(I3{}, std::true_type{}, i + 2);
            step_b(I4{}, std::true_type{}, i + 3);
            step_b(I5{}, std::true_type{}, i + 4);
            step_b(I0{}, std::true_type{}, i + 5);
        }
        if (r6 > 0) step_b(I1{}, std::true_type{}, i);
        if (r6 > 1) step_b(I2{}, std::true_type{}, i + 1);
        if (r6 > 2) step_b(I3{}, std::true_type{}, i + 2);
        if (r6 > 3) step_b(I4{}, std::true_type{}, i + 3);
        if (r6 > 4) step_b(I5{}, std::true_type{}, i + 4);
        // the last tile (step n_steps - 1), as if in step n_steps
        switch (n_steps % 6) {
            case 0: finish_b(I0{}); break;
            case 1: finish_b(I1{}); break;
            case 2: finish_b(I2{}); break;
            case 3: finish_b(I3{}); break;
            case 4: finish_b(I4{}); break;
            default: finish_b(I5{}); break;
        }
    }
    if (my_k < N) {
        if (role_a) store_rows<D>(p.dv + head, my_k, h, acc, 1.0f);
        else store_rows<D>(p.dk + head, my_k, h, acc, p.scale);
    }
}

// ---------------------------------------------------------------------------------
// 2b. dK and dV at d = 64, two phases per tile.  8 wavefronts, 128 keys: key group
//    kg = wave % 4 owns keys k0 + 32 kg + l32 (one key per lane), in two roles that
//    share a SIMD (waves w and w + 4).  Per 64-row tile of Q, dO, LSE and D:
//      phase 1  role A (w < 4):  S = Q K^T, P = exp2(c S - LSE)  -> P to LDS (fp32)
//               role B (w >= 4): dP = dO V^T, then dP - D
//      phase 2  role A:  P packed to bf16, dV^T += dO^T P
//               role B:  dS = P (dP - D) with A's P from LDS;  dK^T += Q^T dS
//    Each role issues 32 matrix instructions per tile, and on each SIMD one wavefront's
//    vector work (mostly A's exponentials in phase 1, B's dS in phase 2) runs beside the
//    other wavefront's matrix products; the vector steps that need no exchange sit in the
//    phase where their role has time to spare.  Role A runs at raised issue priority so
//    that its products, whose results the phase's vector work waits for, go first.
// ---------------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kDkdvThreads, 1) void attn_bwd_dkdv_phased_kernel(BwdParams p) {
    using L = BLayout<D>;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    // Double buffers as separate objects, selected at compile time (see the dQ kernel).
    __shared__ __attribute__((aligned(1024))) char q_lds0[L::TILE];
    __shared__ __attribute__((aligned(1024))) char q_lds1[L::TILE];
    __shared__ __attribute__((aligned(1024))) char do_lds0[L::TILE];
    __shared__ __attribute__((aligned(1024))) char do_lds1[L::TILE];
    __shared__ __attribute__((aligned(16))) f32x4 p_xch[4][2][4][64];  // [kg][sb][g][lane]
    __shared__ __attribute__((aligned(16))) float lse_lds0[kT];
    __shared__ __attribute__((aligned(16))) float lse_lds1[kT];
    __shared__ __attribute__((aligned(16))) float dl_lds0[kT];
    __shared__ __attribute__((aligned(16))) float dl_lds1[kT];

    int bh, kt;
    block_coords(p, CAUSAL, false, bh, kt);
    const int N = p.N;
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave & 3;
    const bool role_a = wave < 4;
    const int64_t head = (int64_t)bh * N * D;
    const int64_t rowbase = (int64_t)bh * N;
    const int k0 = kt * kBwdRows;
    const int kw0 = k0 + 32 * kg;
    const int my_k = kw0 + l32;
    const int k_row = min(my_k, N - 1);

    const int t_row = tid / L::NCH, t_pos = tid % L::NCH;
    const int src_off = t_row * L::RB + 16 * (t_pos ^ L::swz(t_row));
    TileReads<D> rd;
    rd.init(lane);

    // role A: K fragments (B operand of S = Q K^T); role B: V fragments (dP = dO V^T)
    bf16x8 frag[KS];
    load_frag<D>(frag, (role_a ? p.k : p.v) + head, k_row, h);

    f32x16 acc[DB];  // role A: dV^T, role B: dK^T (unscaled)
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = f32x16{};

    // query tiles: causal blocks start at the tile holding their first key
    const int i_begin = CAUSAL ? k0 / kT : 0;
    const int n_q = (N + kT - 1) / kT;
    const bool wave_live = kw0 < N;

    auto copy_tile = [&](auto buf, int i, bool live) __attribute__((always_inline)) {
        constexpr int BUF = decltype(buf)::value;
        tile_to_lds<D, kDkdvThreads>(BUF ? q_lds1 : q_lds0, p.q + head, i * kT, N, wave, src_off, live);
        tile_to_lds<D, kDkdvThreads>(BUF ? do_lds1 : do_lds0, p.dout + head, i * kT, N, wave, src_off, live);
        if (wave == 0) rowvec_to_lds(BUF ? lse_lds1 : lse_lds0, p.lse2 + rowbase, i * kT, N, lane, live);
        if (wave == 1) rowvec_to_lds(BUF ? dl_lds1 : dl_lds0, p.delta + rowbase, i * kT, N, lane, live);
    };
    copy_tile(std::integral_constant<int, 0>{}, i_begin, i_begin < n_q);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    // The two roles run separate copies of the tile loop (same trip count, same two
    // barriers per tile), so that neither role's registers are live in the other's.  The
    // mid-tile barrier orders only the P exchange in LDS; the next tile's copies, issued at
    // the start of the tile, have until the end-of-tile barrier to land.
    // tile i, held in buffer PAR = (i - i_begin) % 2 (compile time)
    auto tile = [&](auto role, auto par, int i) __attribute__((always_inline)) {
        constexpr bool A = decltype(role)::value;
        constexpr int PAR = decltype(par)::value;
        {
            copy_tile(std::integral_constant<int, PAR ^ 1>{}, i + 1, i + 1 < n_q);
            const char* qt = PAR ? q_lds1 : q_lds0;
            const char* dt = PAR ? do_lds1 : do_lds0;
            const float* lse_t = PAR ? lse_lds1 : lse_lds0;
            const float* dl_t = PAR ? dl_lds1 : dl_lds0;
            const int i0 = i * kT;
            // sub-block sb = tile rows 32 sb .. 32 sb + 31: skipped when every query
            // precedes this key group (causal) or lies past N; masked when some entries
            // are hidden
            auto live_sb = [&](int sb) {
                const int qs0 = i0 + 32 * sb;
                return wave_live && !(CAUSAL && qs0 + 31 < kw0) && qs0 < N;
            };
            auto masked_sb = [&](int sb) {
                const int qs0 = i0 + 32 * sb;
                return (CAUSAL && qs0 < kw0 + 31) || (qs0 + 32 > N);
            };
            f32x16 x[2];  // role A: S then P; role B: dP then dS
            if (A) {
                // phase 1: S, P (to LDS for role B, packed for dV)
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
                    if (live_sb(sb)) x[sb] = rows_times_frag<D, true>(qt, sb, rd, frag);
                // P of sub-block sb; the mask is a compile-time choice so that whole
                // sub-blocks (the common case) run without per-element branches
                auto probs = [&](auto masked_c, int sb) __attribute__((always_inline)) {
                    constexpr bool MASKED = decltype(masked_c)::value;
                    // query qs0 + 8 g + 4 h + u is visible when its offset o = 8 g + u from
                    // qs0 + 4 h satisfies o < n_lim and (causal) o >= k_lim
                    const int qb = i0 + 32 * sb + 4 * h;
                    const int n_lim = N - qb, k_lim = my_k - qb;
                    f32x4 l4[4];  // rows 32 sb + 8 g + 4 h + 0..3 of the tile's LSE vector
#pragma unroll
                    for (int g = 0; g < 4; ++g) l4[g] = *reinterpret_cast<const f32x4*>(&lse_t[32 * sb + 8 * g + 4 * h]);
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        f32x4 pv;
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int r = 4 * g + u;
                            float pr = fast_exp2(fmaf(x[sb][r], p.c, -l4[g][u]));
                            if (MASKED) {
                                const int o = 8 * g + u;
                                pr = (o < n_lim && (!CAUSAL || o >= k_lim)) ? pr : 0.0f;
                            }
                            x[sb][r] = pr;
                            pv[u] = pr;
                        }
                        p_xch[kg][sb][g][lane] = pv;
                    }
                };
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    if (!live_sb(sb)) continue;
                    if (masked_sb(sb)) probs(std::true_type{}, sb);
                    else probs(std::false_type{}, sb);
                }
                lds_barrier();  // P is in LDS; the next tile's copies stay in flight
                // phase 2: dV^T += dO^T P (P packed here, where role A has time to spare)
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    if (!live_sb(sb)) continue;
                    trans_times_packed<D, true>(acc, dt, 2 * sb + 0, rd, pack8(x[sb], 0));
                    trans_times_packed<D, true>(acc, dt, 2 * sb + 1, rd, pack8(x[sb], 1));
                }
            } else {
                // phase 1: dP - D (role B has time to spare here)
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    if (!live_sb(sb)) continue;
                    x[sb] = rows_times_frag<D, true>(dt, sb, rd, frag);
                    f32x4 d4[4];
#pragma unroll
                    for (int g = 0; g < 4; ++g) d4[g] = *reinterpret_cast<const f32x4*>(&dl_t[32 * sb + 8 * g + 4 * h]);
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int u = 0; u < 4; ++u) x[sb][4 * g + u] -= d4[g][u];
                }
                lds_barrier();
                // phase 2: dS = P (dP - D), dK^T += Q^T dS
#pragma unroll
                for (int sb = 0; sb < 2; ++sb) {
                    if (!live_sb(sb)) continue;
                    f32x4 pv[4];
#pragma unroll
                    for (int g = 0; g < 4; ++g) pv[g] = p_xch[kg][sb][g][lane];
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int u = 0; u < 4; ++u) x[sb][4 * g + u] *= pv[g][u];  // dS = P (dP - D)
                    trans_times_packed<D, true>(acc, qt, 2 * sb + 0, rd, pack8(x[sb], 0));
                    trans_times_packed<D, true>(acc, qt, 2 * sb + 1, rd, pack8(x[sb], 1));
                }
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next tile has landed
            __syncthreads();
        }
    };
    auto tile_loop = [&](auto role) __attribute__((always_inline)) {
        int i = i_begin;
        for (; i + 1 < n_q; i += 2) {
            tile(role, std::integral_constant<int, 0>{}, i);
            tile(role, std::integral_constant<int, 1>{}, i + 1);
        }
        if (i < n_q) tile(role, std::integral_constant<int, 0>{}, i);
    };
    if (role_a) {
        __builtin_amdgcn_s_setprio(1);
        tile_loop(std::true_type{});
    } else {
        tile_loop(std::false_type{});
    }
    __builtin_amdgcn_s_setprio(0);
    if (wave_live && my_k < N) {
        if (role_a) store_rows<D>(p.dv + head, my_k, h, acc, 1.0f);
        else store_rows<D>(p.dk + head, my_k, h, acc, p.scale);
    }
}

template <int D, bool CAUSAL>
hipError_t launch_main(BwdParams p, hipStream_t st) {
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)p.n_blocks), dim3(kBwdThreads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (D == 128)
        hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)p.n_blocks), dim3(kDkdvThreads), 0, st, p);
    else
        hipLaunchKernelGGL((attn_bwd_dkdv_phased_kernel<D, CAUSAL>), dim3((unsigned)p.n_blocks), dim3(kDkdvThreads), 0,
                           st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv, float* workspace, int B, int H,
                                int N, int d, float scale, bool causal, hipStream_t st) {
    const int64_t rows = (int64_t)B * H * N;
    BwdParams p;
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.dout = static_cast<const uint16_t*>(dout);
    p.o = static_cast<const uint16_t*>(o);
    p.lse = lse;
    p.dq = static_cast<uint16_t*>(dq);
    p.dk = static_cast<uint16_t*>(dk);
    p.dv = static_cast<uint16_t*>(dv);
    p.delta = workspace;
    p.lse2 = workspace + rows;
    p.N = N;
    p.n_tiles = (N + kBwdRows - 1) / kBwdRows;
    const int64_t blocks = (int64_t)B * H * p.n_tiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    p.n_blocks = (int)blocks;
    p.c = scale * kLog2e;
    p.scale = scale;

    if (d != 64 && d != 128) return hipErrorInvalidValue;
    if (d == 64) return causal ? launch_main<64, true>(p, st) : launch_main<64, false>(p, st);
    return causal ? launch_main<128, true>(p, st) : launch_main<128, false>(p, st);
}

}  // namespace mi355
