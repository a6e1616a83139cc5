// device_common.hpp — gfx950 device helpers shared by the kernels of libmi355attn.
//
// Online-softmax state (m, l) and its merge rule follow "Softmax numerical stability
// and IO-aware attention" (zhouzhq2021.github.io), sections 4 and 4.1: merging two
// states takes m = max(m_a, m_b) and l = l_a exp(m_a - m) + l_b exp(m_b - m).  The
// rule is associative in exact arithmetic, so a row is reduced as a tree: inside a
// lane, across the 64 lanes of a wavefront, then across wavefronts through LDS
// (section 4.2 sketches the same hierarchy for 32-lane warps and shared memory).
//
// The empty state is (-inf, 0) and must merge as the identity: a side whose m is
// -inf contributes 0 instead of 0 * exp(-inf - (-inf)) = NaN.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355 {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// 2^x on the hardware transcendental unit (v_exp_f32).  exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// log2(x) on the hardware unit (v_log_f32), for x > 0.
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// A finite stand-in for a maximum that may still be -inf (the empty state), so that
// exp2(value - base) is exp2(-inf) = 0 for empty entries and never NaN.
__device__ __forceinline__ float safe_base(float m) { return m == kNegInf ? 0.0f : m; }

// (m, l) in the units of the input: l is the sum of exp(x - m).
struct MLState {
    float m;
    float l;
};

// Merge two states whose maxima are in the input's units (exp via exp2 of the
// difference times log2 e).  Empty sides contribute nothing.
__device__ __forceinline__ MLState merge_state(MLState a, MLState b) {
    const float m = fmaxf(a.m, b.m);
    const float base = safe_base(m);
    const float fa = fast_exp2((a.m - base) * kLog2e);
    const float fb = fast_exp2((b.m - base) * kLog2e);
    return MLState{m, a.l * fa + b.l * fb};
}

// Merge with the lane `lane ^ mask` (both lanes end with the merged state).
__device__ __forceinline__ MLState merge_xor(MLState s, int mask) {
    MLState o;
    o.m = __shfl_xor(s.m, mask, 64);
    o.l = __shfl_xor(s.l, mask, 64);
    return merge_state(s, o);
}

// Tree-merge across groups of G lanes (G a power of two, <= 64): afterwards every
// lane of a group holds the group's merged state.
template <int G>
__device__ __forceinline__ MLState merge_group(MLState s) {
#pragma unroll
    for (int mask = G / 2; mask >= 1; mask >>= 1) s = merge_xor(s, mask);
    return s;
}

// Exchange a value with the lane 32 positions away: lane l of the result holds
// `x` from lane l ^ 32.
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// The values of `x` in lanes l mod 32 and l mod 32 + 32, delivered to every lane l by
// one v_permlane32_swap (a vector-ALU exchange, no LDS round trip).  Reductions over
// the pair, such as lo + hi, come out bitwise identical in both lanes.
struct HalfPair {
    float lo, hi;
};
__device__ __forceinline__ HalfPair half_pair(float x) {
    const unsigned u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return HalfPair{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

}  // namespace mi355
