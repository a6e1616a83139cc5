// launchers.hpp — host-side entry points of the kernels, called by the C ABI layer
// (api.cpp) after it has validated every argument.  Each returns the hipError_t of
// its launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace mi355 {

// Which row-softmax variant a shape takes.
struct SoftmaxPlan {
    enum Kind { kSmall, kReg, kStream } kind;
    int group;  // kSmall: lanes per row
    int waves;  // kReg: wavefronts per row (1, 4 or 8)
    int nv;     // kReg: units per lane
    bool vec4;  // 16-byte units (cols % 4 == 0 and both pointers 16-byte aligned)
    bool head;  // kReg: 16-byte units from each row's first 16-byte boundary, the rest one by one
};

SoftmaxPlan softmax_plan(const float* x, const float* y, int64_t cols);

hipError_t launch_softmax_rows(const float* x, float* y, int64_t rows, int64_t cols, hipStream_t st);

hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                               int B, int H, int N, int d, float scale, bool causal, hipStream_t st);

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int N, int d, float scale, bool causal, hipStream_t st);

// The same kernel on fp16 inputs and output (fp16 matrix products, P rounded to fp16).
hipError_t launch_attn_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int N, int d, float scale, bool causal, hipStream_t st);

// Keys per part of a split-KV call with n_parts parts over Nk keys.
int64_t splitkv_chunk(int Nk, int n_parts);

// workspace: n_parts * B*H*Nq * (d + 1) floats (partial outputs, then partial LSE).
hipError_t launch_attn_splitkv_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                    float* workspace, int B, int H, int Nq, int Nk, int d, float scale, bool causal,
                                    int n_parts, hipStream_t st);

// The same with the partials in the library's own device-resident scratch of
// kSplitkvScratchBytes per device (no allocation; calls that overlap on one device race).
constexpr int64_t kSplitkvScratchBytes = int64_t(32) << 20;
hipError_t launch_attn_splitkv_bf16_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                            int B, int H, int Nq, int Nk, int d, float scale, bool causal,
                                            int n_parts, hipStream_t st);

hipError_t launch_attn_merge(const float* o_parts, const float* lse_parts, void* o, float* lse, int n_parts,
                             int64_t rows, int d, hipStream_t st);

// Residual add + LayerNorm (layer) or RMSNorm of bf16 rows.  res, beta (RMSNorm) and
// res_out may be null.  norm_rows_max_cols gives the longest row the launch accepts for
// these pointers (rows of a multiple of 8 with 16-byte aligned pointers use 16-byte units).
// Threads per row block of the norm kernel.  norm_vec_path: whether a call takes the
// 16-byte path (host logic in host_plan.cpp, shared by the argument checks and the launch).
// Compute units of the current device (256 if the runtime cannot say), cached per device.
int device_cu_count();

constexpr int kNormRowThreads = 256;
bool norm_vec_path(bool layer, const void* x, const void* res, const void* gamma, const void* beta, const void* y,
                   const void* res_out, int64_t cols);
int64_t norm_rows_max_cols(bool layer, const void* x, const void* res, const void* gamma, const void* beta,
                           const void* y, const void* res_out, int64_t cols);
hipError_t launch_norm_rows(bool layer, const void* x, const void* res, const void* gamma, const void* beta, void* y,
                            void* res_out, int64_t rows, int64_t cols, float eps, hipStream_t st);

// workspace: 2 * B * H * N floats (per-row D, then LSE * log2(e)).
hipError_t launch_attn_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv, float* workspace, int B, int H,
                                int N, int d, float scale, bool causal, hipStream_t st);

}  // namespace mi355
