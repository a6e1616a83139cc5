/*
 * mi355attn.h — C ABI of libmi355attn.so: exact tiled attention forward and
 * row-wise online softmax for AMD Instinct MI355X (gfx950).
 *
 * Operations (pages cited by title and section):
 *
 *   Attention forward, "Softmax numerical stability and IO-aware attention:
 *   from online normalisation to FlashAttention" (zhouzhq2021.github.io), section 7:
 *   O = softmax(scale * Q K^T) V, computed one query tile at a time while the
 *   key/value tiles stream through on-chip memory, keeping a running row maximum m
 *   and row sum l and rescaling the output accumulator by alpha = exp(m - m_new);
 *   the N x N score matrix never reaches device memory.  The lihaoran.work
 *   FlashAttention note, section "the problem starts with the intermediate matrix",
 *   states the same operation with scale = 1/sqrt(d).
 *
 *   Row softmax, same page, sections 3, 4, 4.1 and 4.2: y = exp(x - m) / l per row,
 *   where the (m, l) state of a row is reduced as a tree with the merge rule
 *   m = max(m_a, m_b), l = l_a exp(m_a - m) + l_b exp(m_b - m).
 *
 *   Attention gradients (fa_bwd), same page, section 7.2: dQ, dK, dV of the forward,
 *   recomputing the probabilities tile by tile from the saved per-row LSE.
 *
 *   Split-KV forward and merge (fa_fwd_splitkv, attn_merge_states), same page, section
 *   4.1: partial results over parts of the keys combined with the online-softmax merge.
 *
 *   Fused residual add + RMSNorm / LayerNorm of rows (fused_add_rmsnorm,
 *   fused_add_layernorm), same page, section 5.
 *
 * Conventions shared by every entry point:
 *
 *   Memory     All pointers are device pointers to memory owned by the caller.  The
 *              library allocates, frees and copies nothing, keeps no global mutable
 *              state, and may be called from several host threads at once.  The one
 *              exception is fa_fwd_splitkv_noalloc, whose device-resident scratch is
 *              shared by its calls on a device (see there).
 *   Streams    `stream` is a hipStream_t passed as void*; NULL means the default
 *              stream.  Work is enqueued asynchronously on that stream; outputs are
 *              valid once the caller has synchronised with it.  Nothing here
 *              synchronises, allocates or sets memory, so calls may be captured in a
 *              HIP graph and replayed.
 *   Errors     Arguments are checked before any HIP call.  A bad argument returns
 *              FA_ERR_INVALID_ARG, an unsupported shape or head dimension
 *              returns FA_ERR_UNSUPPORTED, and a failed launch returns FA_ERR_HIP
 *              (mi355attn_last_hip_error() then gives the hipError_t of that
 *              failure on the calling thread).  On any error no output has been
 *              written.  fa_strerror() names a code.
 *   Layout     Dense, row-major, no strides.  Attention tensors are [B, H, N, d]:
 *              element (b, h, n, t) lives at index ((b * H + h) * N + n) * d + t.
 *              LSE is [B, H, N] float32.  Row-softmax tensors are [rows, cols].
 *   Alignment  Attention pointers must be 16-byte aligned; row-softmax pointers 4-byte
 *              aligned (16-byte aligned rows of a multiple of 4 columns take a faster path).
 */
#ifndef MI355ATTN_H
#define MI355ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes.  The FA_* names are the boundary's own; the MI355ATTN_* names are the same
 * values under the library's prefix (kept for callers written against either). */
enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = -1, /* NULL pointer, bad size, bad scale, misaligned or overlapping buffers */
    FA_ERR_UNSUPPORTED = -2, /* head dimension or size the library has no kernel for */
    FA_ERR_HIP = -3,         /* the HIP runtime reported an error at launch */
    MI355ATTN_OK = FA_OK,
    MI355ATTN_ERR_INVALID_ARG = FA_ERR_INVALID_ARG,
    MI355ATTN_ERR_UNSUPPORTED = FA_ERR_UNSUPPORTED,
    MI355ATTN_ERR_HIP = FA_ERR_HIP
};

/*
 * fa_fwd — bf16 attention forward (the hot path).
 *
 *   q, k, v  [B, H, N, d] bf16 (raw IEEE bfloat16 bits, 2 bytes each), read only.
 *   o        [B, H, N, d] bf16, written: O = P V / l rounded once to bf16 (nearest even).
 *   lse      [B, H, N] float32, written: ln(sum over visible keys j of exp(scale * q_i . k_j)),
 *            natural log of the scaled scores, = m_i + ln l_i.
 *   B, H, N  >= 1.  N up to 2^31 - 1 (offsets are computed in 64 bits).
 *   d        64 or 128; anything else returns FA_ERR_UNSUPPORTED.
 *   scale    finite float multiplying every score before the softmax (callers pass 1/sqrt(d)).
 *   causal   0: every query sees all N keys.  1: self-attention, query i sees keys j <= i
 *            (top-left aligned, so no row is empty); tiles wholly above the diagonal are skipped.
 *   stream   hipStream_t or NULL.
 *
 * Arithmetic: Q K^T and P V run on bf16 matrix cores with float32 accumulation; the running
 * maximum, running sum, rescale factors and the output accumulator stay in float32; P is
 * rounded to bf16 (nearest even) as the operand of P V.
 * o must not overlap q, k, v or lse; lse must not overlap any other buffer.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * fa_fwd_f16 — fp16 twin of fa_fwd: q, k, v, o are [B, H, N, d] IEEE binary16; the matrix
 * products run on fp16 matrix cores with float32 accumulation, P is rounded to fp16 (nearest
 * even) for P V, and o is rounded once to fp16.  Statistics and lse stay float32.  Arguments,
 * errors and layout as for fa_fwd.  (The pages contrast fp16 with bf16 and fp32: "Softmax
 * numerical stability and IO-aware attention", section 6 and question Q3; the agentalpha.top
 * interview, standard answer point 3, gives fp16 and fp32 error levels.)
 */
int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * fa_fwd_f32 — float32 attention forward with the same semantics as fa_fwd.
 *
 *   q, k, v, o  [B, H, N, d] float32;  lse [B, H, N] float32.
 *   d           64 or 128.
 * Every product and sum is an ordinary float32 operation (no reduced-precision operand).
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * online_softmax_rows — y[r, :] = softmax(x[r, :]) for every row r, in float32.
 *
 *   x     [rows, cols] float32, read only.
 *   y     [rows, cols] float32, written.  y == x (in place) is allowed; any other overlap is not.
 *   rows  >= 0; rows == 0 does nothing and returns FA_OK.
 *   cols  >= 1 and cols <= 1048576 (larger rows return FA_ERR_UNSUPPORTED).
 *
 * Each row is read once from device memory when it fits on chip (cols <= 16384) and twice
 * otherwise; it is written once.  Entries may be -inf (masked: probability exactly 0) as
 * long as the row holds a finite entry; a row of -inf only has normaliser 0 and gives NaN.
 * +inf and NaN entries are not supported.
 */
int online_softmax_rows(const float* x, float* y, int64_t rows, int64_t cols, void* stream);

/*
 * fa_bwd — gradients of the bf16 attention of fa_fwd, recomputing the probabilities.
 *
 * Operation: "Softmax numerical stability and IO-aware attention" (zhouzhq2021.github.io),
 * section 7.2 and question 4: the backward pass keeps only per-row statistics from the
 * forward and recomputes the local scores tile by tile instead of storing the N x N
 * probability matrix.  The gradients are the derivative of O = softmax(scale Q K^T) V:
 *   P = exp(scale Q K^T - LSE),  dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
 *   D_i = dO_i . O_i,  dQ = scale dS K,  dK = scale dS^T Q.
 *
 *   q, k, v    [B, H, N, d] bf16, the forward's inputs, read only.
 *   o, lse     the forward's outputs for the same q, k, v, scale and causal (fa_fwd), read only.
 *   dout       [B, H, N, d] bf16, the upstream gradient dL/dO, read only.
 *   dq, dk, dv [B, H, N, d] bf16, written (float32 accumulation, rounded once).
 *   workspace  device memory of fa_bwd_workspace_bytes(B, H, N) bytes, 16-byte aligned, owned by
 *              the caller; overwritten (per-row D and LSE log2(e), float32).  It may be reused
 *              as soon as the stream has run this call.
 *   B, H, N, d, scale, causal, stream  as for fa_fwd.
 *
 * dq, dk, dv and workspace must not overlap each other or any input.  Each gradient element
 * is produced by one thread (no atomics), so results are bitwise repeatable.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, void* workspace,
           int B, int H, int N, int d, float scale, int causal, void* stream);

/* Bytes of workspace fa_bwd needs for B x H heads of N rows (8 per row); -1 if B, H or N < 1. */
int64_t fa_bwd_workspace_bytes(int B, int H, int N);

/*
 * fa_fwd_splitkv — bf16 attention forward for Nq queries against Nk keys, with the keys cut
 * into n_splits parts whose partial results are merged in the log domain (the shape of
 * decoding with a key/value cache: Nq small, Nk large).
 *
 * Operation: the same attention as fa_fwd, O = softmax(scale * Q K^T) V and LSE, over
 * rectangular Q [Nq] x K [Nk].  Parts are merged by the rescaling rule of "Softmax numerical
 * stability and IO-aware attention" (zhouzhq2021.github.io), section 4.1, applied to the
 * normalised partial outputs: LSE = ln sum_p e^{LSE_p}, O = sum_p e^{LSE_p - LSE} O_p.
 *
 *   q          [B, H, Nq, d] bf16, read only.
 *   k, v       [B, H, Nk, d] bf16, read only.
 *   o          [B, H, Nq, d] bf16, written (rounded once, nearest even).
 *   lse        [B, H, Nq] float32, written (natural log of the scaled scores' exp-sum).
 *   workspace  fa_fwd_splitkv_workspace_bytes(B, H, Nq, d, n_splits) bytes of device memory,
 *              16-byte aligned, owned by the caller; overwritten with the partial results
 *              (float32 [n_splits, B*H*Nq, d], then float32 [n_splits, B*H*Nq]).
 *   Nq, Nk     >= 1.  causal = 1 needs Nq <= Nk: query i sees keys j <= Nk - Nq + i
 *              (bottom-right aligned: the queries are the last Nq positions).
 *   n_splits   1 .. 4096.  Part p covers keys [p*C, (p+1)*C) with C = 64*ceil(ceil(Nk/n_splits)/64);
 *              trailing parts may be empty.  The call runs B*H*n_splits blocks of four
 *              wavefronts when Nq = 1, else B*H*ceil(Nq/32)*n_splits one-wavefront blocks (up
 *              to five per CU); counts that give every CU an equal share in one round stream
 *              fastest (one block per CU at Nq = 1, two per CU at Nq = 16 on 256 CUs).
 *   d, scale, stream  as for fa_fwd.
 * o, lse and workspace must not overlap each other or any input.
 * Arithmetic: with Nq > 1 the products run on bf16 matrix cores with float32 accumulation
 * and P rounded to bf16, as in fa_fwd; with Nq = 1 (one query per head) the scores and the
 * P V sums are float32 multiply-adds of the bf16 inputs, P not rounded.  The partial results
 * are float32; o is rounded once at the end of the merge.
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal, int n_splits, void* stream);

/* Bytes of workspace fa_fwd_splitkv needs: n_splits * B*H*Nq * (d + 1) * 4; -1 on bad sizes. */
int64_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int d, int n_splits);

/*
 * fa_fwd_splitkv_noalloc — fa_fwd_splitkv for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that forbid hipMalloc.
 * It takes no workspace.  The partial results go to a scratch array that the library keeps
 * in device memory, 32 MiB (33554432 bytes) per device, held from the first call on that
 * device until the process ends.  Nothing in this call allocates or frees memory.
 *
 *   Arguments, layout, results and errors as for fa_fwd_splitkv, without workspace.
 *   A call whose partials would need more than the scratch holds,
 *   fa_fwd_splitkv_workspace_bytes(B, H, Nq, d, n_splits) > 33554432, returns
 *   FA_ERR_UNSUPPORTED before any HIP call (fewer splits or fewer queries per call fit).
 *
 * Every call on one device shares that device's scratch, and each call fully rewrites the
 * part it reads, so nothing carries over from an earlier call.  Calls that may run at the
 * same time on one device (on different streams, or from several host threads without
 * ordering) race on the scratch and are not allowed; calls on one stream are ordered.
 * The first call on a device looks up the scratch address with that device current.
 */
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Nq, int Nk, int d, float scale, int causal, int n_splits,
                           void* stream);

/*
 * attn_merge_states — merges partial attention results computed over disjoint key sets
 * (for example by other devices, each holding part of the keys), by the rule above.
 *
 *   o_parts    [n_parts, rows, d] float32, each part's normalised output, read only.
 *   lse_parts  [n_parts, rows] float32, each part's LSE (natural log); -inf marks a part with
 *              no keys for that row, which contributes nothing.  Read only.
 *   o          [rows, d] bf16, written.   lse  [rows] float32, written.
 *   n_parts    1 .. 65536.  rows >= 0 (0 does nothing).  d 64 or 128.
 * A row whose parts all have LSE = -inf has no defined result.  o_parts and o must be 16-byte
 * aligned, lse_parts and lse 4-byte aligned; outputs must not overlap inputs or each other.
 */
int attn_merge_states(const float* o_parts, const float* lse_parts, void* o, float* lse,
                      int n_parts, int64_t rows, int d, void* stream);

/*
 * fused_add_rmsnorm / fused_add_layernorm — residual add followed by RMSNorm or LayerNorm of
 * every row, bf16 in and out, float32 statistics, one pass over memory.
 *
 * Operation: "Softmax numerical stability and IO-aware attention" (zhouzhq2021.github.io),
 * section 5: with h = x + residual (formed in float32),
 *   RMSNorm    y = h / sqrt(mean(h^2) + eps) * gamma
 *   LayerNorm  y = (h - mean(h)) / sqrt(var(h) + eps) * gamma + beta,  var = mean((h - mean)^2)
 * over each row; the variance comes from a stable pairwise (Welford / Chan) combination.
 *
 *   x             [rows, cols] bf16, read only.
 *   residual      [rows, cols] bf16 or NULL (then h = x), read only.
 *   gamma, beta   [cols] bf16 (beta for LayerNorm only), read only.
 *   y             [rows, cols] bf16, written (rounded once, nearest even).
 *   residual_out  [rows, cols] bf16 or NULL: h rounded to bf16 (the updated residual stream).
 *   rows >= 0 (0 does nothing); cols >= 1 and at most 32768 when cols % 8 == 0 and every
 *   pointer is 16-byte aligned, else at most 4096 (longer rows: FA_ERR_UNSUPPORTED).
 *   eps finite and >= 0.
 * Pointers need 2-byte alignment.  y and residual_out may each be exactly x or residual (in
 * place); no other overlap is allowed.
 */
int fused_add_rmsnorm(const void* x, const void* residual, const void* gamma, void* y, void* residual_out,
                      int64_t rows, int64_t cols, float eps, void* stream);
int fused_add_layernorm(const void* x, const void* residual, const void* gamma, const void* beta, void* y,
                        void* residual_out, int64_t rows, int64_t cols, float eps, void* stream);

/* Human-readable name of a return code (static string, never NULL).  mi355attn_strerror is
 * the same function under the library's prefix. */
const char* fa_strerror(int code);
const char* mi355attn_strerror(int code);

/* hipError_t of the last FA_ERR_HIP returned on the calling thread (0 if none). */
int mi355attn_last_hip_error(void);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int mi355attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MI355ATTN_H */
