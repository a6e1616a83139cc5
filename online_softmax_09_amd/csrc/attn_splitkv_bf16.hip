// attn_splitkv_bf16.hip — split-KV attention forward for few queries against many keys
// (decoding with a key/value cache), and the log-domain merge of partial results.
//
// The key sequence is cut into parts; each part yields a normalised partial output
// O_p and LSE_p = ln sum_{j in part} exp(s_j) per query row, and the parts are merged
// with the rescaling rule of the online softmax ("Softmax numerical stability and
// IO-aware attention", section 4.1: m = max(m_a, m_b), l = l_a e^{m_a - m} + l_b e^{m_b - m},
// applied to the weighted sums as in the agentalpha.top interview's follow-up 1):
//     LSE = ln sum_p e^{LSE_p},    O = sum_p e^{LSE_p - LSE} O_p .
// Causal masking is bottom-right aligned: the N_q queries are the last N_q positions of
// the N_k keys, so query i sees keys j <= N_k - N_q + i.
//
// Partial kernel (gfx950): one wavefront per block and per (head, 32-query tile, part).
// With one or a few queries the work is a stream over the key/value cache, bound by
// HBM; each wavefront keeps its own two 32-key K and V sub-tile buffers in LDS (32 KiB at
// d = 128), fed by buffer_load ... lds copies issued one sub-tile ahead, so a block needs
// no barrier and five blocks fit a CU, which keeps enough bytes in flight (measured
// better than deeper rings with fewer blocks).  The buffers are separate LDS objects
// picked at compile time, so that the wait before a sub-tile's reads is the one the
// kernel states: for grids of under two blocks per CU the next sub-tile's copies stay in
// flight during the reads; otherwise its K copy is waited for as well (measured faster
// there, see launch_partial).  The products are the
// forward's: S^T = K Q^T with the Q fragments in registers (one query per lane column;
// columns past N_q compute garbage and are not stored) and O^T += V^T P^T with V^T read
// by the transposing LDS load.  The running maximum follows the pages' rule exactly
// (moved at every sub-tile); O is rescaled only when some row's maximum moved.
//
// One-query kernel: with a single query the part is a matrix-vector product, so it
// reads K and V rows straight into registers and reduces the dot products with DPP
// (no matrix cores, no LDS staging; see attn_decode_partial_kernel).
//
// Merge kernel: one block of 256 threads per query row; threads own a 16-byte chunk of
// the output columns and a lane of the parts.  Each lane loads its parts' LSEs and
// output chunks in one round of independent loads and keeps a running (m, l, O) state;
// the lanes' states then merge through LDS with the same rescaling rule.
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "launchers.hpp"
#include "mfma_bf16.hpp"

// Device-resident scratch of the allocation-free split-KV entry point: the partial
// results that fa_fwd_splitkv otherwise keeps in the caller's workspace.  Each device
// the library runs on holds its own copy for the life of the process.  In host code the
// name is only a stand-in; kernels receive the address hipGetSymbolAddress returns.
static __device__ __align__(256) float scratch[mi355::kSplitkvScratchBytes / sizeof(float)];

namespace mi355 {
namespace {

constexpr int kSK = 32;       // keys per sub-tile (one MFMA row block)
constexpr int kQT = 32;       // queries per wavefront
constexpr int kPartTile = 64; // part boundaries are multiples of this many keys

template <int D>
struct SLayout {
    static constexpr int RB = 2 * D;
    static constexpr int NCH = RB / 16;
    static constexpr int TILE = kSK * RB;        // bytes per sub-tile
    static constexpr int ROUNDS = TILE / 1024;   // 1 KiB per wavefront-wide 16-byte copy
    static constexpr int RPR = 1024 / RB;        // rows per round
    // Same permutations as the forward kernel's tiles: K is read as 16-byte fragments of
    // 32 consecutive rows, V with the transposing load on rows 4h..4h+3 of 8-row groups.
    __device__ static constexpr int k_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    __device__ static constexpr int v_swz(int r) { return D == 128 ? 4 * (r & 3) : 2 * (r & 3); }
    static constexpr int K_PERIOD = 16;          // rows after which k_swz repeats
    static constexpr int V_PERIOD = 4;
    static constexpr int K_NP = K_PERIOD > RPR ? K_PERIOD / RPR : 1;  // distinct round offsets
    static constexpr int V_NP = V_PERIOD > RPR ? V_PERIOD / RPR : 1;
};

// s_waitcnt operand for "at most n vector-memory operations outstanding" (gfx9 layout:
// vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_enc(int n) { return ((n >> 4) & 3) << 14 | (n & 15) | 0x0F70; }

struct SplitParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    float* o_part;    // [n_parts, B*H*Nq, D]
    float* lse_part;  // [n_parts, B*H*Nq]
    int Nq, Nk;
    int n_qt;         // ceil(Nq / kQT)
    int n_parts;
    int chunk;        // keys per part (multiple of kPartTile)
    int64_t rows;     // B*H*Nq
    float c;          // |scale| log2(e)
    int negate_q;
};

// One 32-row sub-tile of K or V (rows r0.. of a [Nk, D] slab) into LDS by one wavefront.
// off[] are the lane's source offsets for the first rounds of one swizzle period.
template <int D, int NP>
__device__ __forceinline__ void subtile_to_lds(char* lds, const uint16_t* head, int r0, int Nk, const int* off,
                                               bool live) {
    using L = SLayout<D>;
    const int rows = live ? min(Nk - r0, kSK) : 0;
    const char* base = reinterpret_cast<const char*>(head) + (live ? (int64_t)r0 * L::RB : 0);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, rows * L::RB, kBufferWord3);
#pragma unroll
    for (int r = 0; r < L::ROUNDS; ++r) {
        const int soff = (r / NP) * NP * L::RPR * L::RB;  // whole swizzle periods of rows
        const int voff = off[r % NP];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(lds + 1024 * r), 16, voff, soff, 0, 0);
    }
}

template <int D, bool CAUSAL, bool DEEP>
__global__ __launch_bounds__(64, 2) void attn_splitkv_partial_kernel(SplitParams p) {
    using L = SLayout<D>;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    // Two K and two V buffers as separate objects, picked at compile time: with one
    // [2][TILE] array indexed at run time the compiler cannot tell the buffer being read
    // from the one the next copy is filling, and waits for that copy before every read.
    __shared__ __attribute__((aligned(1024))) char k_lds0[L::TILE];
    __shared__ __attribute__((aligned(1024))) char k_lds1[L::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds0[L::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds1[L::TILE];

    // block -> (head bh, query tile qt, part s); parts of one head are adjacent
    const int64_t bid = blockIdx.x;
    const int s = (int)(bid % p.n_parts);
    const int64_t hq = bid / p.n_parts;
    const int qt = (int)(hq % p.n_qt);
    const int64_t bh = hq / p.n_qt;
    const int Nq = p.Nq, Nk = p.Nk;
    const int lane = threadIdx.x, l32 = lane & 31, h = lane >> 5;
    const int q0 = qt * kQT;
    const int my_q = q0 + l32;
    const int q_row = min(my_q, Nq - 1);
    const int64_t qhead = bh * (int64_t)Nq * D;
    const int64_t khead = bh * (int64_t)Nk * D;

    // keys of this part, cut to what the tile's last query can see
    const int lo = (int)min((int64_t)Nk, (int64_t)s * p.chunk);
    int hi = (int)min((int64_t)Nk, (int64_t)lo + p.chunk);
    const int shift = Nk - Nq;  // query i sits at key position shift + i
    if (CAUSAL) hi = min(hi, shift + min(q0 + kQT - 1, Nq - 1) + 1);
    const int n_t = hi > lo ? (hi - lo + kSK - 1) / kSK : 0;
    const int key_lim = CAUSAL ? shift + q_row : Nk - 1;  // last key this lane's query sees

    float m = kNegInf, l = 0.0f;
    f32x16 acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = f32x16{};

    if (n_t > 0) {
        bf16x8 qf[KS];
        const uint32_t qsign = p.negate_q ? 0x80008000u : 0u;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 v4 = *reinterpret_cast<const u32x4*>(p.q + qhead + (int64_t)q_row * D + 16 * ks + 8 * h);
            qf[ks] = __builtin_bit_cast(bf16x8, v4 ^ qsign);
        }
        int k_off[KS], v_off[DB];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) k_off[ks] = l32 * L::RB + 16 * ((2 * ks + h) ^ L::k_swz(l32));
        {
            const int vr = 4 * h + ((lane & 15) >> 2);
#pragma unroll
            for (int b = 0; b < DB; ++b) {
                const int col = 64 * b + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
                v_off[b] = vr * L::RB + 16 * ((col >> 4) ^ L::v_swz(vr)) + (col & 15);
            }
        }
        // per-lane copy source offsets for the rounds of one swizzle period
        int ck[L::K_NP], cv[L::V_NP];
#pragma unroll
        for (int r = 0; r < L::K_NP; ++r) {
            const int row = r * L::RPR + lane / L::NCH, pos = lane % L::NCH;
            ck[r] = row * L::RB + 16 * (pos ^ L::k_swz(row));
        }
#pragma unroll
        for (int r = 0; r < L::V_NP; ++r) {
            const int row = r * L::RPR + lane / L::NCH, pos = lane % L::NCH;
            cv[r] = row * L::RB + 16 * (pos ^ L::v_swz(row));
        }
        const uint16_t* kh = p.k + khead;
        const uint16_t* vh = p.v + khead;
        subtile_to_lds<D, L::K_NP>(k_lds0, kh, lo, Nk, ck, true);
        subtile_to_lds<D, L::V_NP>(v_lds0, vh, lo, Nk, cv, true);

        // sub-tile t in buffer PAR = t % 2 (compile time)
        auto tile = [&](auto par, int t) __attribute__((always_inline)) {
            constexpr int PAR = decltype(par)::value;
            {
                const int tn = t + 1;  // copy the next sub-tile into the other buffer
                subtile_to_lds<D, L::K_NP>(PAR ? k_lds0 : k_lds1, kh, lo + tn * kSK, Nk, ck, tn < n_t);
                subtile_to_lds<D, L::V_NP>(PAR ? v_lds0 : v_lds1, vh, lo + tn * kSK, Nk, cv, tn < n_t);
            }
            // DEEP: every copy but the next sub-tile's has landed.  Otherwise the next
            // sub-tile's K copy (issued first) has landed too, and only its V is in flight.
            __builtin_amdgcn_s_waitcnt(vmcnt_enc((DEEP ? 2 : 1) * L::ROUNDS));
            const char* kt = PAR ? k_lds1 : k_lds0;
            const char* vt = PAR ? v_lds1 : v_lds0;
            const int j0 = lo + t * kSK;
            // S^T = K Q^T: lane holds query column l32, keys j0 + 8 (r/4) + 4 h + r%4
            f32x16 st = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt + k_off[ks]);
                st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], st, 0, 0, 0);
            }
            // the mask is a compile-time choice so that whole sub-tiles (the common case)
            // run without per-element branches
            auto softmax = [&](auto masked_c) __attribute__((always_inline)) {
                constexpr bool MASKED = decltype(masked_c)::value;
                auto visible = [&](int r) {
                    const int key = j0 + 8 * (r >> 2) + 4 * h + (r & 3);
                    return key < hi && key <= key_lim;
                };
                float mx = kNegInf;
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, (!MASKED || visible(r)) ? st[r] : kNegInf);
                const HalfPair pm = half_pair(mx);
                const float mt = fmaxf(pm.lo, pm.hi);
                const float m_new = mt == kNegInf ? m : fmaxf(m, mt * p.c);
                const float base = safe_base(m_new);
                const float alpha = fast_exp2(m - base);  // 0 while m = -inf
                float sum = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float e = fast_exp2(fmaf(st[r], p.c, -base));
                    if (MASKED) e = visible(r) ? e : 0.0f;  // hidden keys get exactly 0
                    st[r] = e;
                    sum += e;
                }
                l = alpha * l + sum;
                m = m_new;
                if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
                    for (int b = 0; b < DB; ++b)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[b][r] *= alpha;
                }
            };
            if (j0 + kSK > hi || (CAUSAL && j0 + kSK - 1 > shift + q0)) softmax(std::true_type{});
            else softmax(std::false_type{});
            // O^T += V^T P^T over the two 16-key groups
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                u32x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(st[8 * g + 2 * i], st[8 * g + 2 * i + 1]);
                const bf16x8 pf = __builtin_bit_cast(bf16x8, w);
#pragma unroll
                for (int b = 0; b < DB; ++b) {
                    const char* pa = vt + 16 * g * L::RB + v_off[b];
                    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_tr_pair(pa, pa + 8 * L::RB), pf,
                                                                     acc[b], 0, 0, 0);
                }
            }
        };
        int t = 0;
        for (; t + 1 < n_t; t += 2) {
            tile(std::integral_constant<int, 0>{}, t);
            tile(std::integral_constant<int, 1>{}, t + 1);
        }
        if (t < n_t) tile(std::integral_constant<int, 0>{}, t);
        __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));  // no copy outlives the block
    }

    const HalfPair pl = half_pair(l);
    const float l_row = pl.lo + pl.hi;
    if (my_q < Nq) {
        const int64_t row = bh * (int64_t)Nq + my_q;
        float* orow = p.o_part + ((int64_t)s * p.rows + row) * D;
        const bool empty = !(l_row > 0.0f);
        const float inv = empty ? 0.0f : 1.0f / l_row;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 o4;
#pragma unroll
                for (int u = 0; u < 4; ++u) o4[u] = acc[b][4 * i + u] * inv;
                *reinterpret_cast<f32x4*>(orow + 32 * b + 8 * i + 4 * h) = o4;
            }
        if (h == 0) p.lse_part[(int64_t)s * p.rows + row] = empty ? kNegInf : (m + fast_log2(l_row)) * kLn2;
    }
}

// ---------------------------------------------------------------------------------
// One query (decoding one token per head): the part is a matrix-vector product over
// the key/value cache with no matrix-core work, so it skips the 32-query MFMA tile and
// the LDS staging.  Lane l of a wavefront reads the 16-byte column chunk l % CH of key
// row l / CH (CH = D / 8 lanes per row), and each wavefront loads U such rows of K and
// of V per iteration straight into registers (U * 2 KiB in flight per wavefront; with a
// block on every CU that keeps HBM busy without any LDS).  A score is the lane's
// 8-term partial dot product summed over the row's CH lanes with DPP; the online-softmax
// state (m, l, O chunk) is per lane and exact (m moves whenever a score exceeds it), and
// the states of the block's key rows merge through LDS with the same rule at the end.
// ---------------------------------------------------------------------------------
constexpr int kGvThreads = 256;
// Key rows per lane and iteration.  Timed at 8 heads x 131072 keys (GB/s, one box): 4 rows
// with one block per CU (32 parts) 6856; 8 rows 6454 there and 6733 with 24 parts (192
// blocks); 2 and 6 rows lower; plain instead of non-temporal loads 5669.  Eight rows win
// only when the grid leaves CUs idle.
constexpr int kGvU = 4;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// x + (x of lane `ctrl` points to), with every lane taking part.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF,
                                                                     false));
}

// Sum over aligned groups of CH lanes (CH = 16: a DPP row; CH = 8: half a row), left
// in every lane of the group.
template <int CH>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (CH == 16) {
        x = dpp_add<0x128>(x);  // row_ror:8
        x = dpp_add<0x124>(x);  // row_ror:4
    } else {
        x = dpp_add<0x141>(x);  // row_half_mirror
    }
    x = dpp_add<0x4E>(x);  // quad_perm [2, 3, 0, 1]
    x = dpp_add<0xB1>(x);  // quad_perm [1, 0, 3, 2]
    return x;
}

template <int D>
__global__ __launch_bounds__(kGvThreads) void attn_decode_partial_kernel(SplitParams p) {
    constexpr int CH = D / 8;                    // lanes per key row
    constexpr int KPW = 64 / CH;                 // key rows per wavefront load
    constexpr int WAVES = kGvThreads / 64;
    constexpr int KPI = WAVES * kGvU * KPW;      // keys per block iteration
    constexpr int R = WAVES * KPW;               // states merged at the end, per chunk
    __shared__ float sm_m[R][CH];
    __shared__ float sm_l[R][CH];
    __shared__ f32x4 sm_acc[R][CH][2];

    const int64_t bid = blockIdx.x;
    const int s = (int)(bid % p.n_parts);
    const int64_t bh = bid / p.n_parts;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int c = lane % CH, kr = lane / CH;
    const int Nk = p.Nk;
    const int lo = (int)min((int64_t)Nk, (int64_t)s * p.chunk);
    const int hi = (int)min((int64_t)Nk, (int64_t)lo + p.chunk);

    // the query's chunk, with the sign of the scale folded in (exact)
    float qf[8];
    {
        const u32x4 qw = *reinterpret_cast<const u32x4*>(p.q + bh * D + 8 * c);
        const float sg = p.negate_q ? -1.0f : 1.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            qf[2 * j] = sg * bf16_lo(qw[j]);
            qf[2 * j + 1] = sg * bf16_hi(qw[j]);
        }
    }
    const uint16_t* kh = p.k + bh * (int64_t)Nk * D + 8 * c;
    const uint16_t* vh = p.v + bh * (int64_t)Nk * D + 8 * c;

    float m = kNegInf, l = 0.0f;
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int kb = lo; kb < hi; kb += KPI) {
        const int k0 = kb + wave * kGvU * KPW + kr;  // this lane's first key row
        u32x4 kv[kGvU], vv[kGvU];
#pragma unroll
        for (int u = 0; u < kGvU; ++u) {
            const int key = min(k0 + u * KPW, hi - 1);  // rows past the part load its last row, masked below
            kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kh + (int64_t)key * D));
        }
#pragma unroll
        for (int u = 0; u < kGvU; ++u) {
            const int key = min(k0 + u * KPW, hi - 1);
            vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vh + (int64_t)key * D));
        }
        float sc[kGvU];
        float mx = kNegInf;
#pragma unroll
        for (int u = 0; u < kGvU; ++u) {
            float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                d0 = fmaf(qf[2 * j], bf16_lo(kv[u][j]), d0);
                d1 = fmaf(qf[2 * j + 1], bf16_hi(kv[u][j]), d1);
            }
            const float dot = group_sum<CH>(d0 + d1);
            sc[u] = k0 + u * KPW < hi ? dot * p.c : kNegInf;
            mx = fmaxf(mx, sc[u]);
        }
        const float m_new = fmaxf(m, mx);
        const float base = safe_base(m_new);
        const float alpha = fast_exp2(m - base);  // 0 while m = -inf
        l *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] *= alpha;
#pragma unroll
        for (int u = 0; u < kGvU; ++u) {
            const float e = fast_exp2(sc[u] - base);  // 0 for a masked row
            l += e;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[2 * j] = fmaf(e, bf16_lo(vv[u][j]), acc[2 * j]);
                acc[2 * j + 1] = fmaf(e, bf16_hi(vv[u][j]), acc[2 * j + 1]);
            }
        }
        m = m_new;
    }

    const int r = wave * KPW + kr;
    sm_m[r][c] = m;
    sm_l[r][c] = l;
    sm_acc[r][c][0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    sm_acc[r][c][1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    __syncthreads();
    if (t < D) {
        const int cc = t / 8, i = t % 8;
        float M = kNegInf;
#pragma unroll
        for (int q = 0; q < R; ++q) M = fmaxf(M, sm_m[q][cc]);
        const float base = safe_base(M);
        float a = 0.0f, L = 0.0f;
#pragma unroll
        for (int q = 0; q < R; ++q) {
            const float w = fast_exp2(sm_m[q][cc] - base);
            a = fmaf(w, sm_acc[q][cc][i / 4][i % 4], a);
            L = fmaf(w, sm_l[q][cc], L);
        }
        const bool empty = !(L > 0.0f);
        p.o_part[((int64_t)s * p.rows + bh) * D + t] = empty ? 0.0f : a / L;
        if (t == 0) p.lse_part[(int64_t)s * p.rows + bh] = empty ? kNegInf : (M + fast_log2(L)) * kLn2;
    }
}

// ---------------------------------------------------------------------------------
// Merge: one block of 256 threads per row.  Thread t owns the 16-byte column chunk
// c = t % (D / 4) of part lane t / (D / 4) (parts lane, lane + lanes, ...).  A lane
// loads the LSEs and output chunks of up to BATCH parts at once (with BATCH = 16 one
// round of independent loads covers 128 parts at d = 128 and 256 at d = 64; few parts
// take BATCH = 4, whose smaller register count lets more rows run at once), folds them
// into its own state (m, l, O chunk) with the online rescaling rule, and the lanes'
// states merge through LDS with the same rule.
// ---------------------------------------------------------------------------------
constexpr int kMergeThreads = 256;

template <int D, int BATCH>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(const float* o_parts, const float* lse_parts,
                                                                   uint16_t* o, float* lse, int n_parts,
                                                                   int64_t rows) {
    constexpr int C = D / 4;                  // 16-byte chunks per row
    constexpr int LANES = kMergeThreads / C;  // part lanes
    __shared__ f32x4 sm_acc[LANES][C];
    __shared__ float sm_m[LANES];
    __shared__ float sm_l[LANES];
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x, c = t % C, lane = t / C;

    float m = kNegInf, l = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int p0 = lane; p0 < n_parts; p0 += BATCH * LANES) {
        float lp[BATCH];
        f32x4 x[BATCH];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const int pidx = p0 + b * LANES;
            lp[b] = kNegInf;
            x[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (pidx < n_parts) {
                lp[b] = lse_parts[(int64_t)pidx * rows + row] * kLog2e;
                x[b] = *reinterpret_cast<const f32x4*>(o_parts + ((int64_t)pidx * rows + row) * D + 4 * c);
            }
        }
        float mx = kNegInf;
#pragma unroll
        for (int b = 0; b < BATCH; ++b) mx = fmaxf(mx, lp[b]);
        const float m_new = fmaxf(m, mx);
        const float base = safe_base(m_new);
        const float alpha = fast_exp2(m - base);  // 0 while m = -inf
        acc *= alpha;
        l *= alpha;
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const float w = fast_exp2(lp[b] - base);  // 0 for an empty part (LSE = -inf)
            if (w > 0.0f) acc += w * x[b];            // an empty part's output is never read into the sum
            l += w;
        }
        m = m_new;
    }
    sm_acc[lane][c] = acc;
    if (c == 0) {
        sm_m[lane] = m;
        sm_l[lane] = l;
    }
    __syncthreads();
    if (t < C) {
        float M = kNegInf;
#pragma unroll
        for (int i = 0; i < LANES; ++i) M = fmaxf(M, sm_m[i]);
        const float base = safe_base(M);
        f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
        float L = 0.0f;
#pragma unroll
        for (int i = 0; i < LANES; ++i) {
            const float w = fast_exp2(sm_m[i] - base);
            a += w * sm_acc[i][t];
            L += w * sm_l[i];
        }
        const float inv = 1.0f / L;
        u32x2 o2;
        o2[0] = pack_bf16x2(a[0] * inv, a[1] * inv);  // nearest even
        o2[1] = pack_bf16x2(a[2] * inv, a[3] * inv);
        *reinterpret_cast<u32x2*>(o + row * D + 4 * t) = o2;
        if (t == 0) lse[row] = (M + fast_log2(L)) * kLn2;
    }
}

template <int D>
hipError_t launch_merge(const float* o_parts, const float* lse_parts, void* o, float* lse, int n_parts,
                        int64_t rows, hipStream_t st) {
    if (n_parts <= 4 * (kMergeThreads / (D / 4)))
        hipLaunchKernelGGL((attn_merge_kernel<D, 4>), dim3((unsigned)rows), dim3(kMergeThreads), 0, st, o_parts,
                           lse_parts, static_cast<uint16_t*>(o), lse, n_parts, rows);
    else
        hipLaunchKernelGGL((attn_merge_kernel<D, 16>), dim3((unsigned)rows), dim3(kMergeThreads), 0, st, o_parts,
                           lse_parts, static_cast<uint16_t*>(o), lse, n_parts, rows);
    return hipGetLastError();
}

}  // namespace

int64_t splitkv_chunk(int Nk, int n_parts) {
    const int64_t per = ((int64_t)Nk + n_parts - 1) / n_parts;
    return kPartTile * ((per + kPartTile - 1) / kPartTile);
}

hipError_t launch_attn_merge(const float* o_parts, const float* lse_parts, void* o, float* lse, int n_parts,
                             int64_t rows, int d, hipStream_t st) {
    if (rows > 0x7fffffff) return hipErrorInvalidValue;
    if (d == 64) return launch_merge<64>(o_parts, lse_parts, o, lse, n_parts, rows, st);
    if (d == 128) return launch_merge<128>(o_parts, lse_parts, o, lse, n_parts, rows, st);
    return hipErrorInvalidValue;
}

namespace {

// The partial kernel's copy depth by blocks per CU, from interleaved timings (GB/s,
// bf16, d = 128): with fewer than two one-wavefront blocks per CU the wavefront keeps
// its next K and V sub-tiles in flight while it computes (1x32x32x65536 in 8 parts:
// 5055 against 3379 waiting for the next K; 16 queries x 128 heads x 32768 keys in 3
// parts: 5782 against 4871); from two per CU on, waiting for the next K as well was as
// fast or faster (4 parts: 6043 against 5665; 1x32x32x65536 in 16 parts: 5863 against
// 5715), the other wavefronts covering the wait.
template <int D, bool CAUSAL>
hipError_t launch_partial(const SplitParams& p, int64_t blocks, bool deep, hipStream_t st) {
    if (deep)
        hipLaunchKernelGGL((attn_splitkv_partial_kernel<D, CAUSAL, true>), dim3((unsigned)blocks), dim3(64), 0, st, p);
    else
        hipLaunchKernelGGL((attn_splitkv_partial_kernel<D, CAUSAL, false>), dim3((unsigned)blocks), dim3(64), 0, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_splitkv_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                    float* workspace, int B, int H, int Nq, int Nk, int d, float scale, bool causal,
                                    int n_parts, hipStream_t st) {
    SplitParams p;
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.Nq = Nq;
    p.Nk = Nk;
    p.n_qt = (Nq + kQT - 1) / kQT;
    p.n_parts = n_parts;
    p.chunk = (int)splitkv_chunk(Nk, n_parts);
    p.rows = (int64_t)B * H * Nq;
    p.o_part = workspace;
    p.lse_part = workspace + (int64_t)n_parts * p.rows * d;
    p.c = fabsf(scale) * kLog2e;
    p.negate_q = scale < 0.0f;
    const int64_t blocks = (int64_t)B * H * p.n_qt * n_parts;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (Nq == 1) {  // one query sees every key, causal or not
        if (d == 64)
            hipLaunchKernelGGL((attn_decode_partial_kernel<64>), dim3((unsigned)blocks), dim3(kGvThreads), 0, st, p);
        else if (d == 128)
            hipLaunchKernelGGL((attn_decode_partial_kernel<128>), dim3((unsigned)blocks), dim3(kGvThreads), 0, st, p);
        else
            return hipErrorInvalidValue;
    } else {
        const bool deep = blocks < 2 * (int64_t)device_cu_count();
        hipError_t e = hipSuccess;
        if (d == 64)
            e = causal ? launch_partial<64, true>(p, blocks, deep, st)
                       : launch_partial<64, false>(p, blocks, deep, st);
        else if (d == 128)
            e = causal ? launch_partial<128, true>(p, blocks, deep, st)
                       : launch_partial<128, false>(p, blocks, deep, st);
        else
            return hipErrorInvalidValue;
        if (e != hipSuccess) return e;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_attn_merge(p.o_part, p.lse_part, o, lse, n_parts, p.rows, d, st);
}

namespace {

// Device address of `scratch` on the current device, looked up once per device (with
// that device current) and kept.
constexpr int kMaxDevices = 64;

hipError_t scratch_address(float** out) {
    static std::mutex mu;
    static float* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (ptr == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = static_cast<float*>(ptr);
    }
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace

hipError_t launch_attn_splitkv_bf16_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                            int B, int H, int Nq, int Nk, int d, float scale, bool causal,
                                            int n_parts, hipStream_t st) {
    const int64_t need = (int64_t)n_parts * B * H * Nq * (int64_t)(d + 1) * (int64_t)sizeof(float);
    if (need > kSplitkvScratchBytes) return hipErrorInvalidValue;  // the C ABI rejects this first
    float* ws = nullptr;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return e;
    // Every partial row of every part is written by the partial kernel before the merge
    // reads it (an empty part writes O = 0 and LSE = -inf), so nothing is cleared.
    return launch_attn_splitkv_bf16(q, k, v, o, lse, ws, B, H, Nq, Nk, d, scale, causal, n_parts, st);
}

}  // namespace mi355
