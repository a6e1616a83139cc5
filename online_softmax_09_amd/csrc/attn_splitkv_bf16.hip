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
// better than deeper rings with fewer blocks).  The products are the
// forward's: S^T = K Q^T with the Q fragments in registers (one query per lane column;
// columns past N_q compute garbage and are not stored) and O^T += V^T P^T with V^T read
// by the transposing LDS load.  The running maximum follows the pages' rule exactly
// (moved at every sub-tile); O is rescaled only when some row's maximum moved.
//
// Merge kernel: one block of 256 threads per query row; threads own a 16-byte chunk of
// the output columns and a lane of the parts.  The row's LSEs are read once (and staged
// in LDS) for the maximum, then every part's output chunk is summed with the weight
// e^{LSE_p - max} (independent loads, unrolled), and the lanes' sums add up through LDS.
#include <mutex>

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
constexpr int kStages = 2;    // LDS buffers per wavefront
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

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64, 2) void attn_splitkv_partial_kernel(SplitParams p) {
    using L = SLayout<D>;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    __shared__ __attribute__((aligned(1024))) char k_lds[kStages][L::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds[kStages][L::TILE];

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
#pragma unroll
        for (int t = 0; t < kStages - 1; ++t) {
            subtile_to_lds<D, L::K_NP>(k_lds[t], kh, lo + t * kSK, Nk, ck, t < n_t);
            subtile_to_lds<D, L::V_NP>(v_lds[t], vh, lo + t * kSK, Nk, cv, t < n_t);
        }

        for (int t = 0; t < n_t; ++t) {
            {
                const int tn = t + kStages - 1;  // copy the next sub-tile
                subtile_to_lds<D, L::K_NP>(k_lds[tn % kStages], kh, lo + tn * kSK, Nk, ck, tn < n_t);
                subtile_to_lds<D, L::V_NP>(v_lds[tn % kStages], vh, lo + tn * kSK, Nk, cv, tn < n_t);
            }
            // every copy but the newest sub-tile's has landed
            __builtin_amdgcn_s_waitcnt(vmcnt_enc((kStages - 1) * 2 * L::ROUNDS));
            const char* kt = k_lds[t % kStages];
            const char* vt = v_lds[t % kStages];
            const int j0 = lo + t * kSK;
            // S^T = K Q^T: lane holds query column l32, keys j0 + 8 (r/4) + 4 h + r%4
            f32x16 st = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt + k_off[ks]);
                st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], st, 0, 0, 0);
            }
            const bool masked = j0 + kSK > hi || (CAUSAL && j0 + kSK - 1 > shift + q0);
            auto visible = [&](int r) {
                const int key = j0 + 8 * (r >> 2) + 4 * h + (r & 3);
                return key < hi && key <= key_lim;
            };
            float mx = kNegInf;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, (!masked || visible(r)) ? st[r] : kNegInf);
            const HalfPair pm = half_pair(mx);
            const float mt = fmaxf(pm.lo, pm.hi);
            const float m_new = mt == kNegInf ? m : fmaxf(m, mt * p.c);
            const float base = safe_base(m_new);
            const float alpha = fast_exp2(m - base);  // 0 while m = -inf
            float sum = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float e = fast_exp2(fmaf(st[r], p.c, -base));
                if (masked) e = visible(r) ? e : 0.0f;  // hidden keys get exactly 0
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
        }
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
// Merge: one block of 256 threads per row.  Thread t owns the 16-byte column chunk
// c = t % (D / 4) of part lane t / (D / 4) (parts lane, lane + lanes, ...).  Two rounds of
// independent loads: every part's LSE (staged in LDS as LSE log2 e), the block maximum,
// then every part's output chunk weighted by e^{LSE_p - max}; the lanes' sums then add
// up through LDS.  All weights share the block maximum, so no lane rescales another.
// ---------------------------------------------------------------------------------
constexpr int kMergeThreads = 256;
constexpr int kMergeStaged = 2048;  // parts whose LSE stays in LDS between the passes

template <int D>
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(const float* o_parts, const float* lse_parts,
                                                                   uint16_t* o, float* lse, int n_parts,
                                                                   int64_t rows) {
    constexpr int C = D / 4;                  // 16-byte chunks per row
    constexpr int LANES = kMergeThreads / C;  // part lanes
    __shared__ float sm_lse[kMergeStaged];
    __shared__ float sm_max[kMergeThreads / 64];
    __shared__ f32x4 sm_acc[LANES][C];
    __shared__ float sm_w[LANES];
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x, c = t % C, lane = t / C;

    float m = kNegInf;
    for (int pidx = t; pidx < n_parts; pidx += kMergeThreads) {
        const float x = lse_parts[(int64_t)pidx * rows + row] * kLog2e;
        if (pidx < kMergeStaged) sm_lse[pidx] = x;
        m = fmaxf(m, x);
    }
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) m = fmaxf(m, __shfl_xor(m, mask, 64));
    if ((t & 63) == 0) sm_max[t >> 6] = m;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMergeThreads / 64; ++i) m = fmaxf(m, sm_max[i]);
    const float base = safe_base(m);

    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float wsum = 0.0f;
#pragma unroll 8
    for (int pidx = lane; pidx < n_parts; pidx += LANES) {
        const float lp = pidx < kMergeStaged ? sm_lse[pidx] : lse_parts[(int64_t)pidx * rows + row] * kLog2e;
        const float w = fast_exp2(lp - base);  // 0 for an empty part (LSE = -inf)
        const f32x4 x = *reinterpret_cast<const f32x4*>(o_parts + ((int64_t)pidx * rows + row) * D + 4 * c);
        if (w > 0.0f) acc += w * x;            // an empty part's output is never read into the sum
        wsum += w;
    }
    sm_acc[lane][c] = acc;
    if (c == 0) sm_w[lane] = wsum;
    __syncthreads();
    if (t < C) {
        f32x4 a = sm_acc[0][t];
        float l = sm_w[0];
#pragma unroll
        for (int i = 1; i < LANES; ++i) {
            a += sm_acc[i][t];
            l += sm_w[i];
        }
        const float inv = 1.0f / l;
        u32x2 o2;
        o2[0] = pack_bf16x2(a[0] * inv, a[1] * inv);  // nearest even
        o2[1] = pack_bf16x2(a[2] * inv, a[3] * inv);
        *reinterpret_cast<u32x2*>(o + row * D + 4 * t) = o2;
        if (t == 0) lse[row] = (m + fast_log2(l)) * kLn2;
    }
}

template <int D>
hipError_t launch_merge(const float* o_parts, const float* lse_parts, void* o, float* lse, int n_parts,
                        int64_t rows, hipStream_t st) {
    hipLaunchKernelGGL((attn_merge_kernel<D>), dim3((unsigned)rows), dim3(kMergeThreads), 0, st, o_parts, lse_parts,
                       static_cast<uint16_t*>(o), lse, n_parts, rows);
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
    if (d == 64) {
        if (causal)
            hipLaunchKernelGGL((attn_splitkv_partial_kernel<64, true>), dim3((unsigned)blocks), dim3(64), 0, st, p);
        else
            hipLaunchKernelGGL((attn_splitkv_partial_kernel<64, false>), dim3((unsigned)blocks), dim3(64), 0, st, p);
    } else if (d == 128) {
        if (causal)
            hipLaunchKernelGGL((attn_splitkv_partial_kernel<128, true>), dim3((unsigned)blocks), dim3(64), 0, st, p);
        else
            hipLaunchKernelGGL((attn_splitkv_partial_kernel<128, false>), dim3((unsigned)blocks), dim3(64), 0, st, p);
    } else {
        return hipErrorInvalidValue;
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
