// norm_rows.hip — fused residual add + LayerNorm / RMSNorm of rows, bf16 in and out,
// float32 statistics.
//
// "Softmax numerical stability and IO-aware attention" (zhouzhq2021.github.io), section
// 5: LayerNorm y = (h - mu) / sqrt(var + eps) * gamma + beta, RMSNorm
// y = h / sqrt(mean(h^2) + eps) * gamma; keep 16-bit inputs and outputs but accumulate
// the statistics in float32, compute the variance with a stable algorithm, and fuse the
// residual add, the normalisation and the type conversion so each row makes one trip
// through HBM.  Here h = x + residual is formed in float32, written back as the updated
// residual stream (bf16), and normalised from the float32 values.
//
// gfx950 mapping: one block per row, of 128 threads for rows of up to 256 units and 512
// above (256 on the 2-byte path).  Each thread loads NV units of 8 bf16 (16 bytes) spaced
// one block-width apart, so every load instruction of the block covers a contiguous
// stretch of the row (2 KiB or 8 KiB), and keeps h in registers: the row is read once and
// written once.
// LayerNorm statistics are exact two-pass values per thread (the
// thread's own mean, then the sum of squared deviations from it, both from registers),
// merged across threads with Chan's pairwise rule
//     n = n_a + n_b,  mu = mu_a + (mu_b - mu_a) n_b / n,
//     M2 = M2_a + M2_b + (mu_b - mu_a)^2 n_a n_b / n,
// the parallel form of Welford's update (lane exchanges within a wavefront, LDS across
// the four wavefronts).  This is the same shape of reduction as the (m, l) merge of the
// online softmax: a small state with its own combining rule instead of a plain sum.
// RMSNorm needs only the sum of squares.  Rows whose length is not a multiple of 8 or
// whose pointers are not 16-byte aligned take the same kernel with 2-byte units.
#include "device_common.hpp"
#include "launchers.hpp"
#include "mfma_bf16.hpp"

namespace mi355 {
namespace {


struct NormParams {
    const uint16_t* x;
    const uint16_t* res;     // may be null (h = x)
    const uint16_t* gamma;
    const uint16_t* beta;    // LayerNorm only
    uint16_t* y;
    uint16_t* res_out;       // may be null (h not written)
    int64_t cols;
    float eps;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

struct Welford {
    float n, mean, m2;
};

__device__ __forceinline__ Welford chan_merge(Welford a, Welford b) {
    const float n = a.n + b.n;
    if (n == 0.0f) return a;
    const float d = b.mean - a.mean;
    const float fb = b.n / n;
    return Welford{n, fmaf(d, fb, a.mean), a.m2 + b.m2 + d * d * a.n * fb};
}

// U = elements per unit (8: 16-byte vectors, 1: scalars); NV = units per thread;
// THREADS = threads per row (one block).
template <bool LAYER, int U, int NV, int THREADS>
__global__ __launch_bounds__(THREADS) void norm_rows_kernel(NormParams p) {
    __shared__ float sh[3][THREADS / 64];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t cols = p.cols;
    const int64_t units = cols / U;  // U divides cols on the vector path
    const int64_t base = row * cols;

    float h[NV][U];
    int nvalid = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int64_t u = tid + (int64_t)THREADS * i;
        if (u < units) {
            ++nvalid;
            if constexpr (U == 8) {
                const u32x4 xv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.x + base + 8 * u));
                u32x4 rv = u32x4{0, 0, 0, 0};
                if (p.res) rv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.res + base + 8 * u));
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    h[i][2 * j] = bf16_lo(xv[j]) + bf16_lo(rv[j]);
                    h[i][2 * j + 1] = bf16_hi(xv[j]) + bf16_hi(rv[j]);
                }
                if (p.res_out) {
                    u32x4 o;
#pragma unroll
                    for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(h[i][2 * j], h[i][2 * j + 1]);
                    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(p.res_out + base + 8 * u));
                }
            } else {
                const float xr = __uint_as_float((uint32_t)p.x[base + u] << 16);
                const float rr = p.res ? __uint_as_float((uint32_t)p.res[base + u] << 16) : 0.0f;
                h[i][0] = xr + rr;
                if (p.res_out) p.res_out[base + u] = (uint16_t)(pack_bf16x2(h[i][0], 0.0f) & 0xffffu);
            }
        } else {
#pragma unroll
            for (int j = 0; j < U; ++j) h[i][j] = 0.0f;
        }
    }

    // ---- statistics
    float mean = 0.0f, rstd;
    if constexpr (LAYER) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int j = 0; j < U; ++j) s += h[i][j];
        const float n = (float)(nvalid * U);
        const float mu = n > 0.0f ? s / n : 0.0f;
        float m2 = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
            if (i < nvalid)
#pragma unroll
                for (int j = 0; j < U; ++j) {
                    const float dv = h[i][j] - mu;
                    m2 = fmaf(dv, dv, m2);
                }
        Welford w{n, mu, m2};
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const Welford o{__shfl_xor(w.n, off, 64), __shfl_xor(w.mean, off, 64), __shfl_xor(w.m2, off, 64)};
            w = chan_merge(w, o);
        }
        if (lane == 0) {
            sh[0][wave] = w.n;
            sh[1][wave] = w.mean;
            sh[2][wave] = w.m2;
        }
        __syncthreads();
        Welford t{sh[0][0], sh[1][0], sh[2][0]};
#pragma unroll
        for (int k = 1; k < THREADS / 64; ++k) t = chan_merge(t, Welford{sh[0][k], sh[1][k], sh[2][k]});
        mean = t.mean;
        rstd = rsqrtf(t.m2 / (float)cols + p.eps);
    } else {
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int j = 0; j < U; ++j) ss = fmaf(h[i][j], h[i][j], ss);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
        if (lane == 0) sh[0][wave] = ss;
        __syncthreads();
        float tot = 0.0f;
#pragma unroll
        for (int k = 0; k < THREADS / 64; ++k) tot += sh[0][k];
        rstd = rsqrtf(tot / (float)cols + p.eps);
    }

    // ---- normalise and store
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int64_t u = tid + (int64_t)THREADS * i;
        if (u >= units) continue;
        if constexpr (U == 8) {
            const u32x4 gv = *reinterpret_cast<const u32x4*>(p.gamma + 8 * u);
            u32x4 bv = u32x4{0, 0, 0, 0};
            if (LAYER) bv = *reinterpret_cast<const u32x4*>(p.beta + 8 * u);
            u32x4 o;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float y0 = fmaf((h[i][2 * j] - mean) * rstd, bf16_lo(gv[j]), bf16_lo(bv[j]));
                const float y1 = fmaf((h[i][2 * j + 1] - mean) * rstd, bf16_hi(gv[j]), bf16_hi(bv[j]));
                o[j] = pack_bf16x2(y0, y1);
            }
            __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(p.y + base + 8 * u));
        } else {
            const float g = __uint_as_float((uint32_t)p.gamma[u] << 16);
            const float b = LAYER ? __uint_as_float((uint32_t)p.beta[u] << 16) : 0.0f;
            p.y[base + u] = (uint16_t)(pack_bf16x2(fmaf((h[i][0] - mean) * rstd, g, b), 0.0f) & 0xffffu);
        }
    }
}

template <bool LAYER, int U, int THREADS>
hipError_t launch_u(const NormParams& p, int64_t rows, int nv, hipStream_t st) {
    const dim3 grid((unsigned)rows), block(THREADS);
    switch (nv) {
        case 1: hipLaunchKernelGGL((norm_rows_kernel<LAYER, U, 1, THREADS>), grid, block, 0, st, p); break;
        case 2: hipLaunchKernelGGL((norm_rows_kernel<LAYER, U, 2, THREADS>), grid, block, 0, st, p); break;
        case 4: hipLaunchKernelGGL((norm_rows_kernel<LAYER, U, 4, THREADS>), grid, block, 0, st, p); break;
        case 8: hipLaunchKernelGGL((norm_rows_kernel<LAYER, U, 8, THREADS>), grid, block, 0, st, p); break;
        case 16: hipLaunchKernelGGL((norm_rows_kernel<LAYER, U, 16, THREADS>), grid, block, 0, st, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool LAYER, int U>
hipError_t launch_threads(const NormParams& p, int64_t rows, int64_t units, hipStream_t st) {
    // Threads per row from interleaved timings (GB/s, RMSNorm / LayerNorm, two boxes),
    // 16-byte units: 128 threads for rows of at most 256 units, 512 above.  Against 256
    // threads for every row: 8192 columns 6188 / 6038 against 5906 / 5734; 4096 +2-3%;
    // 16384 +8% / +1.5%; 32768 +7% / +4%; 1024 +2% / +26%; 512 +22% / +61%; 2048 within
    // 1.3%.  LayerNorm fell to 40-70% with 1024 threads, and with 512 on rows of 256 units.
    // Rows of 2-byte units keep 256 threads (4095 columns: 5-10% slower with 512).
    const int threads = U == 1 ? 256 : units <= 256 ? 128 : 512;
    const int64_t per = (units + threads - 1) / threads;
    int nv = 1;
    while (nv < per) nv *= 2;
    if (nv > 16) return hipErrorInvalidValue;
    if constexpr (U == 1) return launch_u<LAYER, U, 256>(p, rows, nv, st);
    return threads == 128 ? launch_u<LAYER, U, 128>(p, rows, nv, st) : launch_u<LAYER, U, 512>(p, rows, nv, st);
}

}  // namespace

hipError_t launch_norm_rows(bool layer, const void* x, const void* res, const void* gamma, const void* beta, void* y,
                            void* res_out, int64_t rows, int64_t cols, float eps, hipStream_t st) {
    NormParams p;
    p.x = static_cast<const uint16_t*>(x);
    p.res = static_cast<const uint16_t*>(res);
    p.gamma = static_cast<const uint16_t*>(gamma);
    p.beta = static_cast<const uint16_t*>(beta);
    p.y = static_cast<uint16_t*>(y);
    p.res_out = static_cast<uint16_t*>(res_out);
    p.cols = cols;
    p.eps = eps;
    const bool vec = norm_vec_path(layer, x, res, gamma, beta, y, res_out, cols);
    const int64_t units = vec ? cols / 8 : cols;
    if (layer) return vec ? launch_threads<true, 8>(p, rows, units, st) : launch_threads<true, 1>(p, rows, units, st);
    return vec ? launch_threads<false, 8>(p, rows, units, st) : launch_threads<false, 1>(p, rows, units, st);
}

}  // namespace mi355
