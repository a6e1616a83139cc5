// attn_fwd_f32.hip — float32 tiled attention forward (plain fp32 FMA, no matrix cores).
//
// Same algorithm as the bf16 kernel: "Softmax numerical stability and IO-aware
// attention" (zhouzhq2021.github.io), section 7 — for each query tile, stream the
// key/value tiles through on-chip memory, keep the running row maximum m and sum l,
// rescale the output accumulator by alpha = exp(m - m_new) whenever m grows
// (section 7 stresses that both l and the accumulator take alpha), and divide by l
// once at the end.  The lihaoran.work FlashAttention note ("why per-block softmaxes
// cannot be averaged") gives the same (m, l, u) recurrence for one scalar value.
//
// Mapping: 16 lanes (one DPP row) per query row, each holding D / 16 of the row's
// dimensions of q and of the output accumulator; a 256-thread block takes 16 rows.  A
// score is the lanes' partial dot products summed across the row's lanes with DPP (two
// quad permutes, a half-row mirror, a rotate by 8), so every lane of the row holds the
// full score and the same running (m, l).  Spreading a row over 16 lanes gives short
// sequences many wavefronts and each lane a sixteenth of the multiply-adds: at
// 1 x 1 x 256 x 64 a call took 28 us, against 271 us with one lane per row (35 and 49 us
// with 8 and 4 lanes).
// The key and value tiles are staged in LDS, where the lanes of a row read the same key
// row (an LDS broadcast across rows).  Scores are kept in their natural units and
// exponentiated as exp2((s - m) * log2 e): the difference is formed first, so large
// shifted scores (e.g. every score + 1000) lose no accuracy to the log2 e factor.
#include "device_common.hpp"
#include "launchers.hpp"

namespace mi355 {
namespace {

template <int CTRL>
__device__ __forceinline__ float dpp_sum(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF,
                                                                      false));
}

// Sum over the LPQ lanes of a row (lanes LPQ r .. LPQ r + LPQ - 1, LPQ = 4, 8 or 16), in
// every one of them.
template <int LPQ>
__device__ __forceinline__ float row_sum(float x) {
    x = dpp_sum<0xB1>(x);                      // quad_perm [1, 0, 3, 2]
    x = dpp_sum<0x4E>(x);                      // quad_perm [2, 3, 0, 1]
    if constexpr (LPQ >= 8) x = dpp_sum<0x141>(x);  // row_half_mirror: the other quad of 8
    if constexpr (LPQ == 16) x = dpp_sum<0x128>(x);  // row_ror:8: the other half of 16
    return x;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(const float* __restrict__ q,
                                                           const float* __restrict__ k,
                                                           const float* __restrict__ v,
                                                           float* __restrict__ o,
                                                           float* __restrict__ lse, int N,
                                                           int n_qtiles, float scale) {
    constexpr int LPQ = 16;           // lanes per query row
    constexpr int QPB = 256 / LPQ;    // query rows per block
    constexpr int DV = D / 64;        // float4 units of the row per lane (D / 16 dimensions)
    constexpr int BN = 32;            // keys per tile
    static_assert(BN * (D / 4) % 256 == 0, "a tile is a whole number of float4 units per thread");
    __shared__ float4 ks[BN][D / 4];
    __shared__ float4 vs[BN][D / 4];

    const int64_t bh = blockIdx.x / n_qtiles;
    const int q0 = (blockIdx.x % n_qtiles) * QPB;
    const int part = threadIdx.x % LPQ;      // which D / 16 dimensions
    const int i = q0 + threadIdx.x / LPQ;    // this lane's query row
    const bool row_ok = i < N;
    const int64_t head = bh * (int64_t)N * D;

    float4 qr[DV];
#pragma unroll
    for (int c = 0; c < DV; ++c)
        qr[c] = row_ok ? reinterpret_cast<const float4*>(q + head + (int64_t)i * D)[DV * part + c]
                       : make_float4(0.f, 0.f, 0.f, 0.f);

    float4 acc[DV];
#pragma unroll
    for (int c = 0; c < DV; ++c) acc[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    float m = kNegInf, l = 0.0f;

    // Causal: keys beyond the block's last query are never visible.
    const int kv_end = CAUSAL ? min(N, q0 + QPB) : N;
    // The next tile's K and V are loaded into registers while the current one is used,
    // so that the loop does not wait for memory once per tile.
    constexpr int PER = BN * (D / 4) / 256;  // float4 units of a tile per thread
    float4 kr[PER], vr[PER];
    auto fetch = [&](int j0) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int idx = threadIdx.x + 256 * u;
            const int r = idx / (D / 4), c = idx % (D / 4);
            const int key = j0 + r;
            const bool ok = key < N;
            const int64_t off = head + (int64_t)key * D;
            kr[u] = ok ? reinterpret_cast<const float4*>(k + off)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
            vr[u] = ok ? reinterpret_cast<const float4*>(v + off)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    fetch(0);
    for (int j0 = 0; j0 < kv_end; j0 += BN) {
        __syncthreads();  // the previous tile's reads of ks / vs are done
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int idx = threadIdx.x + 256 * u;
            ks[idx / (D / 4)][idx % (D / 4)] = kr[u];
            vs[idx / (D / 4)][idx % (D / 4)] = vr[u];
        }
        if (j0 + BN < kv_end) fetch(j0 + BN);
        __syncthreads();

        float s[BN];
        float mt = kNegInf;
#pragma unroll
        for (int jj = 0; jj < BN; ++jj) {
            float dot = 0.0f;
#pragma unroll
            for (int c = 0; c < DV; ++c) {
                const float4 kk = ks[jj][DV * part + c];
                dot = fmaf(qr[c].x, kk.x, dot);
                dot = fmaf(qr[c].y, kk.y, dot);
                dot = fmaf(qr[c].z, kk.z, dot);
                dot = fmaf(qr[c].w, kk.w, dot);
            }
            dot = row_sum<LPQ>(dot);
            const int key = j0 + jj;
            const bool visible = key < N && (!CAUSAL || key <= i);
            s[jj] = visible ? dot * scale : kNegInf;
            mt = fmaxf(mt, s[jj]);
        }
        const float m_new = fmaxf(m, mt);
        const float base = safe_base(m_new);
        const float alpha = (m == kNegInf) ? 0.0f : fast_exp2((m - base) * kLog2e);
        float ps = 0.0f;
#pragma unroll
        for (int jj = 0; jj < BN; ++jj) {
            s[jj] = fast_exp2((s[jj] - base) * kLog2e);
            ps += s[jj];
        }
        l = alpha * l + ps;
#pragma unroll
        for (int c = 0; c < DV; ++c) {
            float4 a = acc[c];
            a.x *= alpha;
            a.y *= alpha;
            a.z *= alpha;
            a.w *= alpha;
#pragma unroll
            for (int jj = 0; jj < BN; ++jj) {
                const float4 vv = vs[jj][DV * part + c];
                a.x = fmaf(s[jj], vv.x, a.x);
                a.y = fmaf(s[jj], vv.y, a.y);
                a.z = fmaf(s[jj], vv.z, a.z);
                a.w = fmaf(s[jj], vv.w, a.w);
            }
            acc[c] = a;
        }
        m = m_new;
    }

    if (row_ok) {
        float4* orow = reinterpret_cast<float4*>(o + head + (int64_t)i * D);
#pragma unroll
        for (int c = 0; c < DV; ++c)
            orow[DV * part + c] = make_float4(acc[c].x / l, acc[c].y / l, acc[c].z / l, acc[c].w / l);
        if (part == 0) lse[bh * N + i] = m + fast_log2(l) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const float* q, const float* k, const float* v, float* o, float* lse, int BH, int N,
                  float scale, hipStream_t st) {
    constexpr int QPB = 16;
    const int n_qtiles = (N + QPB - 1) / QPB;
    const int64_t blocks = (int64_t)BH * n_qtiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0, st, q, k,
                       v, o, lse, N, n_qtiles, scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                               int B, int H, int N, int d, float scale, bool causal, hipStream_t st) {
    const int BH = B * H;
    if (d == 64) return causal ? launch<64, true>(q, k, v, o, lse, BH, N, scale, st)
                               : launch<64, false>(q, k, v, o, lse, BH, N, scale, st);
    if (d == 128) return causal ? launch<128, true>(q, k, v, o, lse, BH, N, scale, st)
                                : launch<128, false>(q, k, v, o, lse, BH, N, scale, st);
    return hipErrorInvalidValue;
}

}  // namespace mi355
