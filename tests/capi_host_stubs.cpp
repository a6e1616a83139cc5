// Stand-ins for the kernel launchers, for a host-only build of the C ABI's argument checks
// (api.cpp, host_plan.cpp) under AddressSanitizer.  The host tests only make calls that the
// checks reject before any HIP call, so reaching a launcher is itself a failure: each stub
// aborts.
#include <cstdio>
#include <cstdlib>

#include "launchers.hpp"

namespace {

[[noreturn]] void reached(const char* name) {
    std::fprintf(stderr, "capi_host_stubs: %s reached; the argument checks let a call through\n", name);
    std::abort();
}

}  // namespace

namespace mi355 {

SoftmaxPlan softmax_plan(const float*, const float*, int64_t) { reached("softmax_plan"); }
hipError_t launch_softmax_rows(const float*, float*, int64_t, int64_t, hipStream_t) { reached("launch_softmax_rows"); }
hipError_t launch_attn_fwd_f32(const float*, const float*, const float*, float*, float*, int, int, int, int, float,
                               bool, hipStream_t) {
    reached("launch_attn_fwd_f32");
}
hipError_t launch_attn_fwd_bf16(const void*, const void*, const void*, void*, float*, int, int, int, int, float, bool,
                                hipStream_t) {
    reached("launch_attn_fwd_bf16");
}
hipError_t launch_attn_fwd_f16(const void*, const void*, const void*, void*, float*, int, int, int, int, float, bool,
                               hipStream_t) {
    reached("launch_attn_fwd_f16");
}
int64_t splitkv_chunk(int, int) { reached("splitkv_chunk"); }
hipError_t launch_attn_splitkv_bf16(const void*, const void*, const void*, void*, float*, float*, int, int, int, int,
                                    int, float, bool, int, hipStream_t) {
    reached("launch_attn_splitkv_bf16");
}
hipError_t launch_attn_splitkv_bf16_noalloc(const void*, const void*, const void*, void*, float*, int, int, int, int,
                                            int, float, bool, int, hipStream_t) {
    reached("launch_attn_splitkv_bf16_noalloc");
}
hipError_t launch_attn_merge(const float*, const float*, void*, float*, int, int64_t, int, hipStream_t) {
    reached("launch_attn_merge");
}
hipError_t launch_norm_rows(bool, const void*, const void*, const void*, const void*, void*, void*, int64_t, int64_t,
                            float, hipStream_t) {
    reached("launch_norm_rows");
}
hipError_t launch_attn_bwd_bf16(const void*, const void*, const void*, const void*, const void*, const float*, void*,
                                void*, void*, float*, int, int, int, int, float, bool, hipStream_t) {
    reached("launch_attn_bwd_bf16");
}

}  // namespace mi355
