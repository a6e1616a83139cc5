// softmax_rows.hip — row-wise online softmax, y = exp(x - m) / l per row, float32.
//
// Method: "Softmax numerical stability and IO-aware attention" (zhouzhq2021.github.io),
// section 3 (a safe softmax needs the row maximum m and l = sum exp(x - m) before any
// output), section 4 (the (m, l) state, updated element by element) and section 4.1
// (the merge of two partial states).  Section 4.2 sketches the reduction hierarchy;
// here it is laid out for gfx950:
//
//   1. each lane owns a strided slice of the row, loaded with 16-byte (dwordx4) or
//      4-byte accesses that are contiguous across the 64 lanes of a wavefront, and
//      reduces it to a lane state (m_lane, l_lane) while overwriting x with
//      e = exp(x - m_lane) in registers;
//   2. the 64 lane states are merged as a tree across the wavefront (6 levels);
//   3. for rows spread over 4 or 8 wavefronts, the wave states meet in LDS and every
//      thread merges them in the same fixed order;
//   4. y = e * exp(m_lane - m) / l is written from registers.
//
// So a row that fits in registers is read from HBM once and written once: 8 bytes of
// algorithmic traffic per element (section 3 notes that a softmax is bound by memory
// traffic and reductions, and that short rows can be kept on chip).  Rows too long
// for registers take the two-scan streaming form: scan 1 folds the online state over
// the row, scan 2 re-reads x and writes y.
#include "device_common.hpp"
#include "launchers.hpp"

namespace mi355 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool VEC4>
struct Unit;
template <>
struct Unit<true> {
    using T = f32x4;
};
template <>
struct Unit<false> {
    using T = float;
};

__device__ __forceinline__ float umax(float a) { return a; }
__device__ __forceinline__ float umax(f32x4 a) { return fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w)); }

__device__ __forceinline__ float unit_exp_sum(float& a, float base) {
    a = fast_exp2((a - base) * kLog2e);
    return a;
}
__device__ __forceinline__ float unit_exp_sum(f32x4& a, float base) {
    a.x = fast_exp2((a.x - base) * kLog2e);
    a.y = fast_exp2((a.y - base) * kLog2e);
    a.z = fast_exp2((a.z - base) * kLog2e);
    a.w = fast_exp2((a.w - base) * kLog2e);
    return (a.x + a.y) + (a.z + a.w);
}

__device__ __forceinline__ void fill_neg_inf(float& a) { a = kNegInf; }
__device__ __forceinline__ void fill_neg_inf(f32x4& a) { a = f32x4{kNegInf, kNegInf, kNegInf, kNegInf}; }

__device__ __forceinline__ float scale_unit(float a, float c) { return a * c; }
__device__ __forceinline__ f32x4 scale_unit(f32x4 a, float c) { return a * c; }

// ---------------------------------------------------------------------------
// Short rows (cols <= 32): a group of G lanes per row, one element per lane.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void softmax_rows_small(const float* x, float* y, int64_t rows,
                                                          int cols) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t row = gid / G;
    const int c = (int)(gid % G);
    const bool mine = row < rows && c < cols;
    const float xv = mine ? x[row * cols + c] : kNegInf;
    // The state of a single element a is (a, exp(a - a)) = (a, 1).
    MLState s{xv, mine ? 1.0f : 0.0f};
    s = merge_group<G>(s);
    if (mine) y[row * cols + c] = fast_exp2((xv - s.m) * kLog2e) / s.l;
}

// ---------------------------------------------------------------------------
// Register-resident rows: WAVES wavefronts per row, NV units (float4 or float) per
// lane.  Unit u of the row lives in lane (u mod 64*WAVES) of the row's threads.
// ---------------------------------------------------------------------------
// HEAD (16-byte units only): rows need not start on a 16-byte boundary.  A row's first
// boundary lies `head` = 0..3 elements in; the elements before it and the 0..3 after its
// last whole unit are loaded one each by threads 0 .. head + tail - 1 and go through the
// same arithmetic as the units.  x and y share their 16-byte phase (the host checks), so
// the units of y are aligned too.
template <int WAVES, int NV, bool VEC4, bool HEAD>
__global__ __launch_bounds__(WAVES > 4 ? 64 * WAVES : 256) void softmax_rows_reg(const float* x, float* y,
                                                                                int64_t rows, int64_t cols) {
    static_assert(VEC4 || !HEAD, "the head form reads the body in 16-byte units");
    using U = typename Unit<VEC4>::T;
    constexpr int T = 64 * WAVES;        // threads per row
    constexpr int ROWS_PER_BLOCK = (WAVES > 4 ? T : 256) / T;  // a block of 256 threads, or one row
    const int t = threadIdx.x % T;
    const int64_t row = (int64_t)blockIdx.x * ROWS_PER_BLOCK + threadIdx.x / T;
    if (row >= rows) return;  // uniform over the row's wavefronts (and the block if WAVES == 4)
    const float* xrow = x + row * cols;
    float* yrow = y + row * cols;
    int head = 0;
    int64_t units = VEC4 ? cols / 4 : cols;
    int64_t e_idx = -1;     // this thread's single element outside the units, if any
    float ev = kNegInf;
    if constexpr (HEAD) {
        head = (int)((0u - (uint32_t)((uintptr_t)xrow >> 2)) & 3u);
        units = (cols - head) >> 2;
        const int n_extra = head + (int)((cols - head) & 3);
        if (t < n_extra) {
            e_idx = t < head ? t : head + 4 * units + (t - head);
            ev = __builtin_nontemporal_load(xrow + e_idx);
        }
    }
    const U* xr = reinterpret_cast<const U*>(xrow + head);
    U* yr = reinterpret_cast<U*>(yrow + head);

    U v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int64_t u = (int64_t)i * T + t;
        if (u < units)
            v[i] = __builtin_nontemporal_load(xr + u);
        else
            fill_neg_inf(v[i]);
    }

    // Lane state over the lane's own elements: m first (all values are in
    // registers), then l = sum exp(x - m); x is replaced by exp(x - m).
    float m_lane = ev;  // -inf unless the thread holds an element outside the units
#pragma unroll
    for (int i = 0; i < NV; ++i) m_lane = fmaxf(m_lane, umax(v[i]));
    const float base = safe_base(m_lane);
    float l_lane = 0.0f;
    if constexpr (HEAD) l_lane = unit_exp_sum(ev, base);
#pragma unroll
    for (int i = 0; i < NV; ++i) l_lane += unit_exp_sum(v[i], base);

    MLState s = merge_group<64>(MLState{m_lane, l_lane});
    if constexpr (WAVES > 1) {
        __shared__ MLState part[WAVES];
        if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
        __syncthreads();
        s = part[0];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) s = merge_state(s, part[w]);
    }

    // y = exp(x - m_lane) * exp(m_lane - m) / l.  A lane without elements has
    // nothing to store, whatever its factor.
    const float c = fast_exp2((base - s.m) * kLog2e) / s.l;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int64_t u = (int64_t)i * T + t;
        if (u < units) __builtin_nontemporal_store(scale_unit(v[i], c), yr + u);
    }
    if constexpr (HEAD) {
        if (e_idx >= 0) __builtin_nontemporal_store(ev * c, yrow + e_idx);
    }
}

// ---------------------------------------------------------------------------
// Streaming rows (too long for registers): one 256-thread block per row.
// Scan 1 folds each thread's elements into its online state chunk by chunk
// (section 4's update, a chunk at a time); scan 2 re-reads and writes.
// ---------------------------------------------------------------------------
template <bool VEC4>
__global__ __launch_bounds__(256) void softmax_rows_stream(const float* x, float* y,
                                                           int64_t /* rows: one block each */, int64_t cols) {
    using U = typename Unit<VEC4>::T;
    constexpr int CH = 4;  // units per thread per step, loaded together
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t units = VEC4 ? cols / 4 : cols;
    const U* xr = reinterpret_cast<const U*>(x + row * cols);
    U* yr = reinterpret_cast<U*>(y + row * cols);

    float m = kNegInf, l = 0.0f;
    for (int64_t u0 = 0; u0 < units; u0 += 256 * CH) {
        U v[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int64_t u = u0 + (int64_t)i * 256 + t;
            if (u < units)
                v[i] = xr[u];
            else
                fill_neg_inf(v[i]);
        }
        float mc = kNegInf;
#pragma unroll
        for (int i = 0; i < CH; ++i) mc = fmaxf(mc, umax(v[i]));
        const float m_new = fmaxf(m, mc);
        const float base = safe_base(m_new);
        float lc = 0.0f;
#pragma unroll
        for (int i = 0; i < CH; ++i) lc += unit_exp_sum(v[i], base);
        // an empty running state (m = -inf) carries nothing over
        const float carry = (m == kNegInf) ? 0.0f : fast_exp2((m - base) * kLog2e);
        l = l * carry + lc;
        m = m_new;
    }
    MLState s = merge_group<64>(MLState{m, l});
    __shared__ MLState part[4];
    if ((t & 63) == 0) part[t >> 6] = s;
    __syncthreads();
    s = part[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) s = merge_state(s, part[w]);

    const float inv_l = 1.0f / s.l;
    for (int64_t u0 = 0; u0 < units; u0 += 256 * CH) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int64_t u = u0 + (int64_t)i * 256 + t;
            if (u < units) {
                U a = xr[u];
                unit_exp_sum(a, s.m);
                __builtin_nontemporal_store(scale_unit(a, inv_l), yr + u);
            }
        }
    }
}

template <int WAVES, bool VEC4, bool HEAD>
hipError_t launch_reg(int nv, const float* x, float* y, int64_t rows, int64_t cols, hipStream_t st) {
    constexpr int rows_per_block = WAVES > 4 ? 1 : 4 / WAVES;
    const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(WAVES > 4 ? 64 * WAVES : 256);
#define MI355_REG_CASE(NVV)                                                                   \
    case NVV:                                                                                 \
        hipLaunchKernelGGL((softmax_rows_reg<WAVES, NVV, VEC4, HEAD>), grid, block, 0, st, x, y,   \
                           rows, cols);                                                       \
        break;
    switch (nv) {
        MI355_REG_CASE(1)
        MI355_REG_CASE(2)
        MI355_REG_CASE(4)
        MI355_REG_CASE(8)
        MI355_REG_CASE(16)
        MI355_REG_CASE(32)
        MI355_REG_CASE(64)
        default:
            return hipErrorInvalidValue;
    }
#undef MI355_REG_CASE
    return hipGetLastError();
}

int next_pow2(int64_t n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

}  // namespace

// Picks the variant for a shape.  Rows of 16-byte units go to four wavefronts beyond 256
// units (1024 columns): at 1536 to 4096 columns that moved 1.4-6% more bytes per second
// than one wavefront holding 8 to 16 units per lane, and was even at 8192.  From 769 to
// 1024 units (3076 to 4096 columns) eight wavefronts of 2 units per lane, in a block of
// their own, were faster again: 3584 +2.5%, 3840 +10%, 4000 +15%, 4096 +3-4%, 4095 +11%;
// at 768 units and below, and at 1536 and 2048, they were slower (2052 columns -26%,
// 8192 -5%).  Rows of 4-byte units keep one wavefront up to 1024 units.  Rows off the
// 16-byte grid take the head form when x and y share a phase: +2.5% to +128% over 4-byte
// units across the shapes timed with four wavefronts (4095 columns +5-6%), except 4097
// columns (-3%).
SoftmaxPlan softmax_plan(const float* x, const float* y, int64_t cols) {
    SoftmaxPlan p{};
    if (cols <= 32) {
        p.kind = SoftmaxPlan::kSmall;
        p.group = next_pow2(cols);
        return p;
    }
    const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y;
    p.vec4 = (cols % 4 == 0) && xa % 16 == 0 && ya % 16 == 0;
    // Other rows are read in 16-byte units from their first 16-byte boundary on, with up
    // to three elements on either side taken one by one, when x and y are 4-byte aligned
    // at the same 16-byte phase (so that the boundaries of x and y rows coincide).
    p.head = !p.vec4 && xa % 4 == 0 && ya % 4 == 0 && xa % 16 == ya % 16;
    const bool wide = p.vec4 || p.head;
    const int64_t units = wide ? cols / 4 : cols;
    const int nv_max = wide ? 16 : 64;  // 64 registers of row data per lane
    const int one_wave_max = wide ? 4 : 16;  // units per lane on the one-wavefront form
    if (units <= 64 * one_wave_max) {
        p.kind = SoftmaxPlan::kReg;
        p.waves = 1;
        p.nv = next_pow2((units + 63) / 64);
    } else if (wide && units > 768 && units <= 1024) {
        p.kind = SoftmaxPlan::kReg;
        p.waves = 8;
        p.nv = 2;
    } else if (units <= 256 * (int64_t)nv_max) {
        p.kind = SoftmaxPlan::kReg;
        p.waves = 4;
        p.nv = next_pow2((units + 255) / 256);
    } else {
        p.kind = SoftmaxPlan::kStream;  // reads rows that are not whole units in 4-byte units
        p.head = false;
    }
    return p;
}

hipError_t launch_softmax_rows(const float* x, float* y, int64_t rows, int64_t cols, hipStream_t st) {
    const SoftmaxPlan p = softmax_plan(x, y, cols);
    switch (p.kind) {
        case SoftmaxPlan::kSmall: {
            const int64_t blocks = (rows * p.group + 255) / 256;
            if (blocks > 0x7fffffff) return hipErrorInvalidValue;
            const dim3 grid((unsigned)blocks), block(256);
            switch (p.group) {
                case 1: hipLaunchKernelGGL(softmax_rows_small<1>, grid, block, 0, st, x, y, rows, (int)cols); break;
                case 2: hipLaunchKernelGGL(softmax_rows_small<2>, grid, block, 0, st, x, y, rows, (int)cols); break;
                case 4: hipLaunchKernelGGL(softmax_rows_small<4>, grid, block, 0, st, x, y, rows, (int)cols); break;
                case 8: hipLaunchKernelGGL(softmax_rows_small<8>, grid, block, 0, st, x, y, rows, (int)cols); break;
                case 16: hipLaunchKernelGGL(softmax_rows_small<16>, grid, block, 0, st, x, y, rows, (int)cols); break;
                case 32: hipLaunchKernelGGL(softmax_rows_small<32>, grid, block, 0, st, x, y, rows, (int)cols); break;
                default: return hipErrorInvalidValue;
            }
            return hipGetLastError();
        }
        case SoftmaxPlan::kReg:
            if (p.waves == 1)
                return p.head   ? launch_reg<1, true, true>(p.nv, x, y, rows, cols, st)
                       : p.vec4 ? launch_reg<1, true, false>(p.nv, x, y, rows, cols, st)
                                : launch_reg<1, false, false>(p.nv, x, y, rows, cols, st);
            if (p.waves == 8)  // 16-byte units only
                return p.head ? launch_reg<8, true, true>(p.nv, x, y, rows, cols, st)
                              : launch_reg<8, true, false>(p.nv, x, y, rows, cols, st);
            return p.head   ? launch_reg<4, true, true>(p.nv, x, y, rows, cols, st)
                   : p.vec4 ? launch_reg<4, true, false>(p.nv, x, y, rows, cols, st)
                            : launch_reg<4, false, false>(p.nv, x, y, rows, cols, st);
        case SoftmaxPlan::kStream: {
            if (rows > 0x7fffffff) return hipErrorInvalidValue;
            const dim3 grid((unsigned)rows), block(256);
            if (p.vec4)
                hipLaunchKernelGGL(softmax_rows_stream<true>, grid, block, 0, st, x, y, rows, cols);
            else
                hipLaunchKernelGGL(softmax_rows_stream<false>, grid, block, 0, st, x, y, rows, cols);
            return hipGetLastError();
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace mi355
