// host_plan.cpp — host-side planning shared by the argument checks (api.cpp) and the
// launchers: which path a call takes, and the size limits that follow from it.  Plain
// host code, with no device code, so the checks can also be built on their own.
#include <cstdint>

#include "launchers.hpp"

namespace mi355 {

namespace {

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

}  // namespace

// The fused norms use 16-byte units (8 bf16) when the row length is a multiple of 8 and
// every pointer is 16-byte aligned, else 2-byte units.
bool norm_vec_path(bool layer, const void* x, const void* res, const void* gamma, const void* beta, const void* y,
                   const void* res_out, int64_t cols) {
    return cols % 8 == 0 && aligned16(x) && aligned16(y) && aligned16(gamma) && (!res || aligned16(res)) &&
           (!res_out || aligned16(res_out)) && (!layer || aligned16(beta));
}

// Rows of up to 16 x 256 units are accepted; the kernel holds them in registers (at most
// 8 units per thread with 512 threads per row, 16 with 256 on the 2-byte path).
int64_t norm_rows_max_cols(bool layer, const void* x, const void* res, const void* gamma, const void* beta,
                           const void* y, const void* res_out, int64_t cols) {
    return norm_vec_path(layer, x, res, gamma, beta, y, res_out, cols) ? 16 * kNormRowThreads * 8
                                                                       : 16 * kNormRowThreads;
}

}  // namespace mi355
