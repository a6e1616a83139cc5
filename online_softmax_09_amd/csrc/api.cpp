// api.cpp — the extern "C" boundary of libmi355attn.so (declared in include/mi355attn.h).
//
// Every argument is validated here, before any HIP call, so bad input comes back as a
// return code without touching the device.  The launchers enqueue on the caller's
// stream and never synchronise.
#include <hip/hip_runtime_api.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "../../include/mi355attn.h"
#include "launchers.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxSoftmaxCols = 1 << 20;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte ranges [a, a + na) and [b, b + nb) intersect.
bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

int finish(hipError_t e) {
    if (e == hipSuccess) return FA_OK;
    g_last_hip_error = static_cast<int>(e);
    return FA_ERR_HIP;
}

// Checks shared by both attention entry points.  elem = bytes per element of q/k/v/o.
int check_attention(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
                    int H, int N, int d, float scale, uint64_t elem) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    const uint64_t rows = (uint64_t)B * (uint64_t)H * (uint64_t)N;
    if ((uint64_t)B * (uint64_t)H > (uint64_t)INT_MAX) return FA_ERR_UNSUPPORTED;
    const uint64_t tbytes = rows * (uint64_t)d * elem;
    const uint64_t lbytes = rows * sizeof(float);
    if (overlaps(o, tbytes, q, tbytes) || overlaps(o, tbytes, k, tbytes) || overlaps(o, tbytes, v, tbytes) ||
        overlaps(o, tbytes, lse, lbytes) || overlaps(lse, lbytes, q, tbytes) ||
        overlaps(lse, lbytes, k, tbytes) || overlaps(lse, lbytes, v, tbytes))
        return FA_ERR_INVALID_ARG;
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, void* stream) {
    const int rc = check_attention(q, k, v, o, lse, B, H, N, d, scale, 2);
    if (rc != FA_OK) return rc;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    return finish(mi355::launch_attn_fwd_bf16(q, k, v, o, lse, B, H, N, d, scale, causal != 0,
                                              static_cast<hipStream_t>(stream)));
}

int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, void* stream) {
    const int rc = check_attention(q, k, v, o, lse, B, H, N, d, scale, 2);
    if (rc != FA_OK) return rc;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    return finish(mi355::launch_attn_fwd_f16(q, k, v, o, lse, B, H, N, d, scale, causal != 0,
                                             static_cast<hipStream_t>(stream)));
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N,
               int d, float scale, int causal, void* stream) {
    const int rc = check_attention(q, k, v, o, lse, B, H, N, d, scale, 4);
    if (rc != FA_OK) return rc;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    return finish(mi355::launch_attn_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal != 0,
                                             static_cast<hipStream_t>(stream)));
}

int64_t fa_bwd_workspace_bytes(int B, int H, int N) {
    if (B < 1 || H < 1 || N < 1) return -1;
    return (int64_t)B * H * N * 2 * (int64_t)sizeof(float);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, void* workspace, int B, int H, int N, int d, float scale, int causal,
           void* stream) {
    // q, k, v, o and lse as for the forward (o is only read here)
    const int rc = check_attention(q, k, v, o, lse, B, H, N, d, scale, 2);
    if (rc != FA_OK) return rc;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!dout || !dq || !dk || !dv || !workspace) return FA_ERR_INVALID_ARG;
    if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
        return FA_ERR_INVALID_ARG;
    const uint64_t rows = (uint64_t)B * (uint64_t)H * (uint64_t)N;
    const uint64_t tb = rows * (uint64_t)d * 2;
    const uint64_t lb = rows * sizeof(float);
    const uint64_t wb = 2 * lb;
    const void* outs[4] = {dq, dk, dv, workspace};
    const uint64_t out_bytes[4] = {tb, tb, tb, wb};
    const void* ins[6] = {q, k, v, o, dout, lse};
    const uint64_t in_bytes[6] = {tb, tb, tb, tb, tb, lb};
    for (int a = 0; a < 4; ++a) {
        for (int b = a + 1; b < 4; ++b)
            if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b])) return FA_ERR_INVALID_ARG;
        for (int b = 0; b < 6; ++b)
            if (overlaps(outs[a], out_bytes[a], ins[b], in_bytes[b])) return FA_ERR_INVALID_ARG;
    }
    return finish(mi355::launch_attn_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, static_cast<float*>(workspace), B,
                                              H, N, d, scale, causal != 0, static_cast<hipStream_t>(stream)));
}

int64_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int d, int n_splits) {
    if (B < 1 || H < 1 || Nq < 1 || d < 1 || n_splits < 1) return -1;
    return (int64_t)n_splits * B * H * Nq * (int64_t)(d + 1) * (int64_t)sizeof(float);
}

}  // extern "C"

namespace {

// Checks of the split-KV entry points other than the workspace: pointers, sizes, scale,
// alignment and the overlap of the outputs with each other and the inputs.
int check_splitkv(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H, int Nq,
                  int Nk, int d, float scale, int causal, int n_splits) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (causal && Nq > Nk) return FA_ERR_INVALID_ARG;
    if (Nk > INT_MAX - 64) return FA_ERR_UNSUPPORTED;
    if (n_splits < 1 || n_splits > 4096) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    const uint64_t bh = (uint64_t)B * (uint64_t)H;
    if (bh * (uint64_t)((Nq + 31) / 32) * (uint64_t)n_splits > (uint64_t)INT_MAX) return FA_ERR_UNSUPPORTED;
    if (bh * (uint64_t)Nq > (uint64_t)INT_MAX) return FA_ERR_UNSUPPORTED;
    const uint64_t qb = bh * Nq * d * 2, kb = bh * Nk * d * 2, lb = bh * Nq * 4;
    const void* ins[3] = {q, k, v};
    const uint64_t in_bytes[3] = {qb, kb, kb};
    if (overlaps(o, qb, lse, lb)) return FA_ERR_INVALID_ARG;
    for (int b = 0; b < 3; ++b)
        if (overlaps(o, qb, ins[b], in_bytes[b]) || overlaps(lse, lb, ins[b], in_bytes[b])) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace, int B, int H,
                   int Nq, int Nk, int d, float scale, int causal, int n_splits, void* stream) {
    const int rc = check_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, n_splits);
    if (rc != FA_OK) return rc;
    if (!workspace || !aligned16(workspace)) return FA_ERR_INVALID_ARG;
    const uint64_t bh = (uint64_t)B * (uint64_t)H;
    const uint64_t qb = bh * Nq * d * 2, kb = bh * Nk * d * 2, lb = bh * Nq * 4;
    const uint64_t wb = (uint64_t)fa_fwd_splitkv_workspace_bytes(B, H, Nq, d, n_splits);
    const void* others[5] = {q, k, v, o, lse};
    const uint64_t other_bytes[5] = {qb, kb, kb, qb, lb};
    for (int b = 0; b < 5; ++b)
        if (overlaps(workspace, wb, others[b], other_bytes[b])) return FA_ERR_INVALID_ARG;
    return finish(mi355::launch_attn_splitkv_bf16(q, k, v, o, lse, static_cast<float*>(workspace), B, H, Nq, Nk, d,
                                                  scale, causal != 0, n_splits, static_cast<hipStream_t>(stream)));
}

int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                           int Nk, int d, float scale, int causal, int n_splits, void* stream) {
    const int rc = check_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, n_splits);
    if (rc != FA_OK) return rc;
    if (fa_fwd_splitkv_workspace_bytes(B, H, Nq, d, n_splits) > mi355::kSplitkvScratchBytes)
        return FA_ERR_UNSUPPORTED;
    return finish(mi355::launch_attn_splitkv_bf16_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal != 0,
                                                          n_splits, static_cast<hipStream_t>(stream)));
}

int attn_merge_states(const float* o_parts, const float* lse_parts, void* o, float* lse, int n_parts, int64_t rows,
                      int d, void* stream) {
    if (rows < 0 || n_parts < 1 || n_parts > 65536 || d < 1) return FA_ERR_INVALID_ARG;
    if (rows == 0) return FA_OK;
    if (!o_parts || !lse_parts || !o || !lse) return FA_ERR_INVALID_ARG;
    if (!aligned16(o_parts) || !aligned16(o) || (reinterpret_cast<uintptr_t>(lse_parts) & 3u) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u))
        return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (rows > (int64_t)INT_MAX) return FA_ERR_UNSUPPORTED;
    const uint64_t pb = (uint64_t)n_parts * rows * d * 4, plb = (uint64_t)n_parts * rows * 4;
    const uint64_t ob = (uint64_t)rows * d * 2, lb = (uint64_t)rows * 4;
    if (overlaps(o, ob, lse, lb) || overlaps(o, ob, o_parts, pb) || overlaps(o, ob, lse_parts, plb) ||
        overlaps(lse, lb, o_parts, pb) || overlaps(lse, lb, lse_parts, plb))
        return FA_ERR_INVALID_ARG;
    return finish(mi355::launch_attn_merge(o_parts, lse_parts, o, lse, n_parts, rows, d,
                                           static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Shared checks of the two fused normalisations.  beta is checked only for LayerNorm.
int check_norm(bool layer, const void* x, const void* res, const void* gamma, const void* beta, const void* y,
               const void* res_out, int64_t rows, int64_t cols, float eps) {
    if (rows < 0 || cols < 1) return FA_ERR_INVALID_ARG;
    if (!x || !gamma || !y || (layer && !beta)) return FA_ERR_INVALID_ARG;
    if (!std::isfinite(eps) || eps < 0.0f) return FA_ERR_INVALID_ARG;
    const void* ptrs[6] = {x, res, gamma, layer ? beta : nullptr, y, res_out};
    for (const void* q : ptrs)
        if (q && (reinterpret_cast<uintptr_t>(q) & 1u)) return FA_ERR_INVALID_ARG;
    if (rows > (int64_t)INT_MAX) return FA_ERR_UNSUPPORTED;
    if (cols > mi355::norm_rows_max_cols(layer, x, res, gamma, beta, y, res_out, cols))
        return FA_ERR_UNSUPPORTED;
    const uint64_t tb = (uint64_t)rows * (uint64_t)cols * 2, vb = (uint64_t)cols * 2;
    // outputs: identical to an input row buffer is allowed (each element is read before it
    // is overwritten, by the thread that overwrites it); any other overlap is not
    auto bad = [&](const void* out, const void* in, uint64_t nin) {
        return in && out != in && overlaps(out, tb, in, nin);
    };
    for (const void* out : {y, res_out}) {
        if (!out) continue;
        if (bad(out, x, tb) || bad(out, res, tb) || overlaps(out, tb, gamma, vb) ||
            (layer && overlaps(out, tb, beta, vb)))
            return FA_ERR_INVALID_ARG;
    }
    if (res_out && overlaps(y, tb, res_out, tb)) return FA_ERR_INVALID_ARG;
    return FA_OK;
}

}  // namespace

extern "C" {

int fused_add_rmsnorm(const void* x, const void* residual, const void* gamma, void* y, void* residual_out,
                      int64_t rows, int64_t cols, float eps, void* stream) {
    const int rc = check_norm(false, x, residual, gamma, nullptr, y, residual_out, rows, cols, eps);
    if (rc != FA_OK || rows == 0) return rc;
    return finish(mi355::launch_norm_rows(false, x, residual, gamma, nullptr, y, residual_out, rows, cols, eps,
                                          static_cast<hipStream_t>(stream)));
}

int fused_add_layernorm(const void* x, const void* residual, const void* gamma, const void* beta, void* y,
                        void* residual_out, int64_t rows, int64_t cols, float eps, void* stream) {
    const int rc = check_norm(true, x, residual, gamma, beta, y, residual_out, rows, cols, eps);
    if (rc != FA_OK || rows == 0) return rc;
    return finish(mi355::launch_norm_rows(true, x, residual, gamma, beta, y, residual_out, rows, cols, eps,
                                          static_cast<hipStream_t>(stream)));
}

int online_softmax_rows(const float* x, float* y, int64_t rows, int64_t cols, void* stream) {
    if (rows < 0 || cols < 1) return FA_ERR_INVALID_ARG;
    if (rows == 0) return FA_OK;
    if (!x || !y) return FA_ERR_INVALID_ARG;
    if (cols > kMaxSoftmaxCols) return FA_ERR_UNSUPPORTED;
    if (rows > (int64_t)INT_MAX) return FA_ERR_UNSUPPORTED;
    // 4-byte alignment is enough; the 16-byte vector path is chosen only when both
    // pointers and the row length allow it.
    if ((reinterpret_cast<uintptr_t>(x) & 3u) || (reinterpret_cast<uintptr_t>(y) & 3u))
        return FA_ERR_INVALID_ARG;
    const uint64_t bytes = (uint64_t)rows * (uint64_t)cols * sizeof(float);
    if (x != y && overlaps(x, bytes, y, bytes)) return FA_ERR_INVALID_ARG;
    return finish(mi355::launch_softmax_rows(x, y, rows, cols, static_cast<hipStream_t>(stream)));
}

const char* fa_strerror(int code) {
    switch (code) {
        case FA_OK:
            return "success";
        case FA_ERR_INVALID_ARG:
            return "invalid argument (null pointer, bad size or scale, misaligned or overlapping buffers)";
        case FA_ERR_UNSUPPORTED:
            return "unsupported shape (head dimension must be 64 or 128; size limits exceeded)";
        case FA_ERR_HIP:
            return "HIP runtime error at launch (see mi355attn_last_hip_error)";
        default:
            return "unknown mi355attn return code";
    }
}

const char* mi355attn_strerror(int code) { return fa_strerror(code); }

int mi355attn_last_hip_error(void) { return g_last_hip_error; }

int mi355attn_version(void) { return 100; }

}  // extern "C"
