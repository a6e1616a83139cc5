// attn_fwd_bf16.hip — bf16 tiled attention forward on gfx950 matrix cores.
//
// Algorithm: "Softmax numerical stability and IO-aware attention" (zhouzhq2021.github.io),
// section 7: per query tile, initialise m = -inf, l = 0, O = 0; for every key/value
// tile form S = Q K^T, take the new row maximum, P = exp(S - m_new),
// alpha = exp(m - m_new), l = alpha l + rowsum P, O = alpha O + P V; finally O / l.
// Section 8 (FlashAttention-2) adds the choices kept here: the query tile is the outer
// loop so O is written once, the division by l is deferred to the end, and key tiles
// wholly above the causal diagonal are skipped.  LSE = m + ln l is written per row.
//
// gfx950 mapping (a design of its own, not the pages' warp/shared-memory scheme):
//
//   * Each wavefront owns 32 query rows for the whole key loop; key tiles are 64 keys.
//     Two block forms share the code.  The ping-pong form has 8 wavefronts (256
//     query rows; waves w and w + 4 share a SIMD) and one block per CU.  The plain
//     form has 4 wavefronts (128 rows) and two blocks per CU (three at d = 64 when the
//     kernel needs no key masks, unless the host holds it to two, see launch).  The
//     host picks one per shape (launch_form).
//   * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     A = a 32-key slice of K (from LDS), B = Q^T (held in registers for the whole
//     loop).  In the 32x32 accumulator, lane l holds one column, i.e. one query row
//     (l mod 32), and 16 of its keys; the other 16 keys of that row sit in lane l^32.
//     So the row max is in-lane maxima plus one exchange.
//   * The row sum l is formed on the matrix cores as well: a 16x16x32 product of a 0/1
//     selection matrix with the packed P^T fragments adds each query's probabilities
//     (the same bf16 values that P V uses) into an accumulator that holds l for the
//     lane's own query row, so l costs no vector instruction per score.
//   * The output is accumulated transposed too, O^T += V^T P^T: the B operand
//     (P^T, 8 keys x 1 query per lane) is exactly what the lane already holds after
//     the exponentials, converted to bf16 with no data movement.  V is kept in LDS
//     row-major and the A operand (V^T) is read with the gfx950 transposing LDS load
//     ds_read_b64_tr_b16: two of them give a lane the 8 keys (4h..4h+3 and
//     8+4h..8+4h+3 of a 16-key group) of its output column, the order in which the
//     S^T accumulator hands P to the lanes.  The O^T accumulator keeps one query row
//     per lane as well, so alpha rescales it with no exchange.
//   * K and V tiles go from HBM straight into LDS (buffer_load_dwordx4 ... lds: each
//     lane's 16 bytes land at base + 16 * lane), with no registers and no LDS write
//     instructions.  The rows are unpadded and each row's 16-byte chunks are stored
//     XOR-permuted, a permutation chosen so that the 16-byte K reads and the
//     transposing V reads are free of LDS bank conflicts; a lane fetches the chunk
//     that belongs at its LDS position.
//   * The work on a tile is split into a matrix part (P V of the previous tile, then
//     S of the next) and a vector part (this tile's softmax).  In the ping-pong form
//     the two groups of four wavefronts run opposite parts in each half-step,
//     separated by block barriers, so each SIMD has one wavefront on each.  In the
//     plain form each wavefront runs the two parts in turn, and the two blocks on a CU
//     share the SIMDs with no common barrier.
//   * The row's reference maximum m moves lazily: only when a tile's maximum exceeds
//     it by more than 2^8 (kLazy).  Until then alpha is exactly 1 and the rescale of O
//     is skipped (decided per wavefront); P stays at most 2^8.  The result O / l and
//     LSE = m + ln l do not depend on which reference m is used.
//   * Exponentials use the hardware exp2 on |scale| log2(e) s - m (one FMA per score);
//     a negative scale negates Q, which is exact.
//   * Block ids are remapped so each of the 8 XCDs (which receive block ids round
//     robin) walks a contiguous range of (head, query tile) pairs: the key/value
//     stream of a head is then shared through that XCD's L2.  In causal mode an XCD
//     takes its heads in pairs (groups of four for rows of up to 4096) and runs each
//     group's query tiles longest first across the group (at d = 64 the shortest
//     quarter of every head's tiles comes last).
#include <type_traits>

#include "device_common.hpp"
#include "launchers.hpp"
#include "mfma_bf16.hpp"

namespace mi355 {
namespace {

// Two block forms (PP): 8 wavefronts in two groups of four that ping-pong (one of each
// group per SIMD, one block per CU), or one group of 4 wavefronts (two blocks per CU).
template <bool PP>
constexpr int waves_of() { return PP ? 8 : 4; }
template <bool PP>
constexpr int threads_of() { return 64 * waves_of<PP>(); }
template <bool PP>
constexpr int rows_of() { return 32 * waves_of<PP>(); }  // query rows per block
constexpr int kGroupThreads = 256;                       // one group: four wavefronts
constexpr int kRoundBytes = 16 * kGroupThreads;  // bytes one group-wide 16-byte copy moves
constexpr int kBN = 64;           // keys per tile

// The reference maximum of a row moves only when a tile's maximum exceeds it by more
// than this many powers of two; until then the probabilities exp2(c s - m) stay at
// most 2^kLazy (far from overflow) and O and l keep their scale, so the rescale of O
// is skipped.  O / l and LSE = m + log l are the same for any reference m.
constexpr float kLazy = 8.0f;

// LDS layout of one 64 x D tile: rows of D bf16 (RB bytes), 16-byte chunk c of row r
// stored at chunk position c ^ swz(r).
template <int D>
struct Layout {
    static constexpr int RB = 2 * D;            // bytes per row
    static constexpr int NCH = RB / 16;         // 16-byte chunks per row
    static constexpr int TILE = kBN * RB;       // bytes per tile
    static constexpr int ROUNDS = TILE / kRoundBytes;  // 16-byte copies per thread per tile
    static constexpr int ROWS_PER_ROUND = kRoundBytes / RB;
    // K is read as 16-byte fragments by 32 lanes on 32 consecutive rows.
    __device__ static constexpr int k_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    // V is read with the transposing 8-byte load on 8 consecutive rows x 4 chunks.
    // Both stay below NCH, so a permuted chunk never leaves its row.
    __device__ static constexpr int v_swz(int r) { return D == 128 ? 4 * (r & 3) : 2 * (r & 3); }
};

// Causal diagonal tiles.  The last key tile a wavefront needs starts D0 = 0 or 32 rows
// before the wavefront's first query row (query rows come in 32s, key tiles in 64s), and
// no earlier tile holds a hidden key.  In the S^T accumulator lane l holds query row
// l mod 32 and, in element r of half sb, the key 4 (l / 32) + 32 sb + 8 (r / 4) + r mod 4
// of the tile, so which lanes see that key is a constant bit mask per (D0, sb, r).
struct DiagMasks {
    uint64_t m[2][2][16];  // [D0 / 32][sb][r]: bit l set when lane l sees the key
};
constexpr DiagMasks make_diag_masks() {
    DiagMasks t{};
    for (int d0 = 0; d0 < 2; ++d0)
        for (int sb = 0; sb < 2; ++sb)
            for (int r = 0; r < 16; ++r)
                for (int lane = 0; lane < 64; ++lane) {
                    const int key = 4 * (lane >> 5) + 32 * sb + 8 * (r >> 2) + (r & 3);
                    if ((lane & 31) + 32 * d0 >= key) t.m[d0][sb][r] |= uint64_t(1) << lane;
                }
    return t;
}
constexpr DiagMasks kDiag = make_diag_masks();

struct Params {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int N;
    int64_t n_bh;  // B * H
    int n_qtiles;
    int n_blocks;
    float scale_log2;  // |scale| * log2(e)
    int negate_q;      // scale < 0
};

// One tile of K or V from HBM straight to LDS, by one group of kGroupThreads threads.
// Thread t of the group writes LDS bytes
// kRoundBytes * round + 16 * t, i.e. row ROWS_PER_ROUND * round + t / NCH at chunk position
// t % NCH, so it fetches logical chunk (t % NCH) ^ swz(row) of that row; `src_off` is
// that per-thread byte offset within a round (the same for every round and tile,
// because the swizzles repeat every ROWS_PER_ROUND rows).  The copy goes through a
// buffer resource that spans exactly the tile's rows below N: the per-tile address
// arithmetic is scalar, and rows at or past N (last tile only) read as zeros, whose
// scores are masked and whose probabilities are 0.
template <int D>
__device__ __forceinline__ void tile_to_lds(char* lds_tile, const char* head, int j0, int N, int gwave,
                                            int src_off) {
    using L = Layout<D>;
    const int rows = min(N - j0, kBN);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(head + (int64_t)j0 * L::RB), (short)0, rows * L::RB, kBufferWord3);
    char* dst = lds_tile + 1024 * gwave;  // gwave: the wave's index in its group (uniform);
                                          // the lane offset is implicit
#pragma unroll
    for (int r = 0; r < L::ROUNDS; ++r)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + kRoundBytes * r), 16, src_off, kRoundBytes * r,
                                                 0, 0);
}

// Per-wavefront state of the key loop and the phases of one key tile.
template <int D, bool CAUSAL, typename E>
struct Wave {
    using L = Layout<D>;
    static constexpr int KS = D / 16;  // k-steps of Q K^T
    static constexpr int DB = D / 32;  // 32-wide blocks of the output dimension

    using v8 = typename E::v8;
    v8 qf[KS];       // Q^T fragments (B operand of S^T = K Q^T)
    f32x16 acc[DB];  // O^T accumulator: this lane's query row, 16 of each 32 outputs
    v8 pf[4];        // P^T fragments of the last finished tile (B operand of O^T += V^T P^T)
    v8 sel;          // A operand of the row sums (0/1 selection, see rowsum)
    f32x4 lacc;      // row-sum accumulator: element 0 = l of this lane's query row
    int k_off[KS];   // byte offset of this lane's K fragment for k-step ks (row l32)
    int v_off[DB];   // byte offset of this lane's transposing V block for output block b
    float m;         // reference max of |scale| log2(e) score, this lane's row (see kLazy)
    float c;         // |scale| log2(e)
    float base;      // finite stand-in for m while a tile is exponentiated
    float alpha;     // exp2(m_old - m_new) of the tile in flight
    int half, key_lim;

    // S^T = K Q^T for the two 32-key halves of a tile (A = K rows from LDS).
    __device__ __forceinline__ void qk(f32x16 (&st)[2], const char* ktile) const {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            f32x16 a = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const v8 kf = *reinterpret_cast<const v8*>(ktile + 32 * sb * L::RB + k_off[ks]);
                a = E::mfma(kf, qf[ks], a);
            }
            st[sb] = a;
        }
    }

    // Online-softmax update of one tile, in two parts.  prep (reads S only): the row
    // maximum over the visible keys is taken and moves the reference m if it exceeds it
    // by more than kLazy.  expsum: the 32 keys are exponentiated (hidden keys, on
    // diagonal or ragged tiles only, get exactly 0) and packed to bf16 P^T fragments,
    // which the matrix part then multiplies into O and sums into l.  The maximum runs
    // as four independent partial chains so that no instruction waits long on the one
    // before it.
    __device__ __forceinline__ bool visible(int j0, int sb, int r) const {
        return j0 + 4 * half + 32 * sb + 8 * (r >> 2) + (r & 3) <= key_lim;
    }

    // Scores of keys a row does not see on its causal diagonal tile become -inf, in
    // place (one select per score against a constant lane mask).  The unmasked softmax
    // then gives them probability exp2(-inf) = 0; c > 0 always (the host passes a tiny
    // positive c for scale 0), so c * -inf is never NaN.
    template <int D0>
    __device__ __forceinline__ void mask_diag(f32x16 (&st)[2]) const {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                st[sb][r] = __builtin_amdgcn_inverse_ballot_w64(kDiag.m[D0 / 32][sb][r]) ? st[sb][r] : kNegInf;
    }

    template <bool MASK>
    __device__ __forceinline__ void prep(const f32x16 (&st)[2], int j0) {
        float mx[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mx[r & 3] = fmaxf(mx[r & 3], (!MASK || visible(j0, sb, r)) ? st[sb][r] : kNegInf);
        const HalfPair pm = half_pair(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])));
        const float mt = fmaxf(pm.lo, pm.hi) * c;
        // m = -inf (nothing seen yet) always moves: -inf + kLazy is -inf
        const float m_new = mt > m + kLazy ? mt : m;
        base = safe_base(m_new);
        alpha = fast_exp2(m - base);  // 1 when m stays; 0 when m = -inf
        m = m_new;
    }

    template <bool MASK>
    __device__ __forceinline__ void expsum(f32x16 (&st)[2], int j0) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float e = fast_exp2(fmaf(st[sb][r], c, -base));
                if (MASK) e = visible(j0, sb, r) ? e : 0.0f;
                st[sb][r] = e;
            }
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                u32x4 w;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    w[t] = E::pack2(st[sb][8 * hb + 2 * t], st[sb][8 * hb + 2 * t + 1]);
                pf[2 * sb + hb] = __builtin_bit_cast(v8, w);
            }
    }

    // The same work split in two (see the kernel): the exponentials of one 32-key half,
    // packed straight into the P^T fragments (the previous tile's fragments must have
    // been consumed).  The arithmetic and its order are those of expsum.
    template <bool MASK, int SB>
    __device__ __forceinline__ void exp_half(f32x16 (&st)[2], int j0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float e = fast_exp2(fmaf(st[SB][r], c, -base));
            if (MASK) e = visible(j0, SB, r) ? e : 0.0f;
            st[SB][r] = e;
        }
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            u32x4 w;
#pragma unroll
            for (int t = 0; t < 4; ++t) w[t] = E::pack2(st[SB][8 * hb + 2 * t], st[SB][8 * hb + 2 * t + 1]);
            pf[2 * SB + hb] = __builtin_bit_cast(v8, w);
        }
    }
    // O^T *= alpha and l *= alpha, skipped (per wavefront) when no row moved its
    // reference maximum.
    __device__ __forceinline__ void rescale() {
        if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
            for (int b = 0; b < DB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[b][r] *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) lacc[i] *= alpha;
        }
    }

    // l += the row sums of the packed P^T fragments, on the matrix cores: in the
    // 16x16x32 product lane l supplies B[8 (l / 16) + i][l % 16], i.e. query l % 32 in
    // the lanes whose l / 16 is even for n = l % 16 and odd for n = l % 16 + 16.  The
    // selection rows 0 and 8 add the even groups, rows 4 and 12 the odd ones, so element
    // 0 of the output (row 4 (l / 16), column l % 16) is the sum for query l % 32 in
    // every lane.  l is then the sum of the same bf16 P that P V uses.
    __device__ __forceinline__ void rowsum() {
#pragma unroll
        for (int g = 0; g < 4; ++g) lacc = E::mfma16(sel, pf[g], lacc);
    }

    // O^T += V^T P^T with the packed P of the last finished tile.  A operand for
    // output rows 32 b .. 32 b + 31 and key group g: lane l needs
    // V[16 g + 4 half + t][32 b + l32] (t = 0..3) and V[16 g + 8 + 4 half + t][32 b + l32],
    // read transposed from row-major V.  Rows 16 g and 16 g + 8 are multiples of 8, so
    // the swizzle (a function of the row mod 4 or mod 8) is already in v_off.
    __device__ __forceinline__ void pv(const char* vtile) {
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const char* pa = vtile + 16 * g * L::RB + v_off[b];
                const i16x4 lo = lds_read_tr16(pa);
                const i16x4 hi = lds_read_tr16(pa + 8 * L::RB);
                const v8 a = __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                acc[b] = E::mfma(a, pf[g], acc[b]);
            }
    }
};

// TAIL: the last key tile may run past N.  Causal kernels always take the general
// form (their diagonal tile covers a ragged end anyway); non-causal ones are built
// twice, and the form without key masks needs fewer registers (164 instead of 186 at
// d = 64, so three blocks fit a CU instead of two).
template <int D, bool CAUSAL, typename E, bool PP, bool TAIL>
__global__ __launch_bounds__(threads_of<PP>(), 2) void attn_fwd_bf16_kernel(Params p) {
    constexpr int kBM = rows_of<PP>();
    using L = Layout<D>;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    // Two K and two V tile buffers, as separate objects so that the compiler can tell
    // the buffer being filled from the one being read.
    __shared__ __attribute__((aligned(1024))) char k_lds0[L::TILE];
    __shared__ __attribute__((aligned(1024))) char k_lds1[L::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds0[L::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds1[L::TILE];

    // XCD-aware remap: block id b runs on XCD b % 8; give each XCD a contiguous
    // range of logical ids.
    const int nb = p.n_blocks;
    int lid = blockIdx.x;
    if ((nb & 7) == 0) lid = (lid & 7) * (nb >> 3) + (lid >> 3);
    int bh = lid / p.n_qtiles;
    int qt = lid % p.n_qtiles;
    if (CAUSAL) {
        qt = p.n_qtiles - 1 - qt;  // longest tiles first
        // An XCD's heads are taken in pairs, longest tiles first across the pair, so the
        // tail of each pair's work is short tiles of both heads.  Larger groups finished
        // sooner at some shapes but read keys and values from memory many more times
        // (per call at B=2 H=32 N=8192 d=128: 440 MB fetched one head at a time, 561 MB
        // in pairs, 907 MB in fours, 2463 MB in eights), once a group's keys and values
        // outgrew the XCD's L2.  At d = 64 (three blocks per CU) the shortest quarter of
        // every head's tiles is held back and dispatched last, longest first across all of
        // the XCD's heads, so that the launch ends on short tiles of every head rather
        // than on the last pair's long ones: +3-12% at causal d = 64 (2048-8192 rows),
        // -0.5% at d = 128, where it is off.
        const int per_xcd = nb >> 3;
        if ((nb & 7) == 0 && per_xcd % p.n_qtiles == 0) {
            const int nq = p.n_qtiles;
            const int hx = per_xcd / nq;  // heads per XCD
            // groups of four heads for short rows (N <= 4096, with a multiple of eight heads
            // per XCD): +6-7% at causal 4x32x2048 (d = 64 and 128), +3-6% at 8x32x1024,
            // +0.1-0.6% at N = 4096; pairs above, where four measured +0.2-0.5% but read
            // keys and values from memory half as often again (907 against 561 MB per
            // call at B=2 H=32 N=8192 d=128)
            const int G = (hx % 8 == 0 && p.N <= 4096) ? 4 : (hx % 2 == 0) ? 2 : 1;
            const int tq = D == 64 ? nq / 4 : 0;  // tiles per head held back
            const int hl = G * (nq - tq);         // tiles of one group before that
            const int x = lid / per_xcd, li = lid % per_xcd;
            if (li < (hx / G) * hl) {
                const int g = li / hl, r = li % hl;
                bh = x * hx + g * G + r % G;
                qt = nq - 1 - r / G;
            } else {
                const int t = li - (hx / G) * hl;
                bh = x * hx + t % hx;
                qt = tq - 1 - t / hx;
            }
        }
    }

    const int N = p.N;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int group = PP ? wave >> 2 : 0;  // PP: waves w and w + 4 share a SIMD
    const int gtid = tid & (kGroupThreads - 1);
    // The wavefront's index in its group, read from lane 0 so the compiler knows it is
    // uniform: the LDS copy destinations are then scalar.
    const int gwave = __builtin_amdgcn_readfirstlane(wave & 3);
    const int64_t head = (int64_t)bh * N * D;
    const char* kh = reinterpret_cast<const char*>(p.k + head);
    const char* vh = reinterpret_cast<const char*>(p.v + head);

    const int q0 = qt * kBM;
    const int qw0 = q0 + 32 * wave;  // this wavefront's first query row
    const bool wave_live = qw0 < N;

    // Per-thread source offsets of the HBM -> LDS copies (see tile_to_lds).
    const int t_row = gtid / L::NCH, t_pos = gtid % L::NCH;
    const int k_src = t_row * L::RB + 16 * (t_pos ^ L::k_swz(t_row));
    const int v_src = t_row * L::RB + 16 * (t_pos ^ L::v_swz(t_row));

    Wave<D, CAUSAL, E> w;
    const int l32 = lane & 31;
    w.half = lane >> 5;
    const int my_q = qw0 + l32;
    w.key_lim = CAUSAL ? min(N - 1, my_q) : N - 1;  // last visible key of the row
    w.c = p.scale_log2;
    w.m = kNegInf;
    w.lacc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    {
        const int m16 = lane & 15, kb = lane >> 4;
        const bool one = ((m16 == 0 || m16 == 8) && (kb & 1) == 0) || ((m16 == 4 || m16 == 12) && (kb & 1) == 1);
        const uint32_t wv = one ? E::kOnes2 : 0u;
        w.sel = __builtin_bit_cast(typename E::v8, u32x4{wv, wv, wv, wv});
    }
    // K fragment of lane l: row l32 (+32 sb) of the tile, logical chunk 2 ks + half.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) w.k_off[ks] = l32 * L::RB + 16 * ((2 * ks + w.half) ^ L::k_swz(l32));
    // Transposing V block of lane l: row 4 half + (lane % 16) / 4 of the key group,
    // byte column 64 b + 32 ((lane / 16) % 2) + 8 (lane % 4) of the output block.
    {
        const int vr = 4 * w.half + ((lane & 15) >> 2);
#pragma unroll
        for (int b = 0; b < DB; ++b) {
            const int col = 64 * b + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
            w.v_off[b] = vr * L::RB + 16 * ((col >> 4) ^ L::v_swz(vr)) + (col & 15);
        }
    }

    // Q^T fragments: lane supplies Q[my_q][16 s + 8 half + 0..7].  With a negative
    // scale the query is negated (exact in bf16) and |scale| used, so the row maximum
    // of the raw products is the maximum of the scaled scores.
    const uint32_t qsign = p.negate_q ? 0x80008000u : 0u;
    const int q_row = min(my_q, N - 1);  // rows past the end compute garbage, never stored
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const u32x4 v4 =
            *reinterpret_cast<const u32x4*>(p.q + head + (int64_t)q_row * D + 16 * s + 8 * w.half);
        w.qf[s] = __builtin_bit_cast(typename E::v8, v4 ^ qsign);
    }
#pragma unroll
    for (int b = 0; b < DB; ++b) w.acc[b] = f32x16{};

    const int q_last = min(q0 + kBM - 1, N - 1);
    const int n_kv = CAUSAL ? (q_last / kBN + 1) : (N + kBN - 1) / kBN;  // tiles of the block
    // tiles this wavefront needs (a prefix of the block's tiles)
    const int n_w = !wave_live ? 0 : CAUSAL ? min(n_kv, min(qw0 + 31, N - 1) / kBN + 1) : n_kv;

    // Ping-pong over key tiles.  For wave group g, the work on tile j is split into
    //   GEMM_j    = O += P_{j-1} V_{j-1}, then S_{j+1} = K_{j+1} Q^T  (matrix cores)
    //   SOFTMAX_j = P_j and alpha_j from S_j, then O *= alpha_j       (vector ALUs)
    // and group g runs GEMM_j in half-step 2 j + g and SOFTMAX_j in half-step 2 j + 1 + g.
    // The two wavefronts that share a SIMD are in different groups, so one always has
    // matrix work while the other has vector work.  At half-step 2 j, K_{j+2} (copied
    // by group 0 during its GEMM) and V_j (copied by group 1 during its SOFTMAX; V_0
    // with K_0 and K_1 before the loop) go from HBM to the LDS buffers that GEMM_{j-1}
    // finished reading; each has until the barrier after half-step 2 j + 1 to land.
    // V_0 goes with K_0 and K_1, so that its latency overlaps theirs and that of Q.
    if constexpr (PP) {
        const int ug = __builtin_amdgcn_readfirstlane(group);  // uniform copy of the group
        if (ug == 0 || n_kv > 1) tile_to_lds<D>(ug ? k_lds1 : k_lds0, kh, ug ? kBN : 0, N, gwave, k_src);
        if (ug == 1) tile_to_lds<D>(v_lds0, vh, 0, N, gwave, v_src);
    } else {
        tile_to_lds<D>(k_lds0, kh, 0, N, gwave, k_src);
        if (n_kv > 1) tile_to_lds<D>(k_lds1, kh, kBN, N, gwave, k_src);
        tile_to_lds<D>(v_lds0, vh, 0, N, gwave, v_src);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's copies have landed
    __syncthreads();
    f32x16 sa[2], sb[2];
    if (n_w > 0) w.qk(sa, k_lds0);
    __syncthreads();  // K buffer 0 may now be refilled

    auto is_masked = [&](int j) { return (CAUSAL && j * kBN + kBN - 1 > qw0) || (TAIL && j * kBN + kBN > N); };
    // In causal mode the only masked tile of a wavefront is its last, the diagonal tile
    // j = qw0 / 64, which starts 0 or 32 rows before the wavefront's rows.  Keys at or
    // past N on it lie above every stored row's diagonal, so the causal mask covers a
    // ragged end too (rows at or past N compute values that are never stored).
    auto diag = [&](f32x16(&sc)[2], int j) {
        if (qw0 == j * kBN) w.template mask_diag<0>(sc);
        else w.template mask_diag<32>(sc);
    };
    // GEMM_j (plus the copy of K_{j+2} when copy_k: group 0 in the ping-pong form, the
    // one group in the plain form; and the copy of V_j when copy_v: the plain form, where
    // issuing it here rather than after the matrix part gives it a whole tile to land).
    // PAR = j % 2 at compile time, so every buffer access names one LDS object.
    // With SPLIT the matrix part also takes the row maximum of S_j and the exponentials
    // of its first 32 keys, between its own matrix instructions, and the softmax part
    // keeps the other 32 keys.  In the plain form a wavefront runs both parts itself,
    // so this overlaps its own vector work with its matrix work.  In the ping-pong form
    // it evens out the halves at d = 64, where a tile has half the matrix work of
    // d = 128 but the same vector work; at d = 128 the halves are already even and
    // moving work there measured slower.
    constexpr bool SPLIT = D == 64 || !PP;
    auto gemm = [&](auto par, int j, f32x16(&sc)[2], f32x16(&sn)[2], bool copy_k, bool copy_v) {
        constexpr int PAR = decltype(par)::value;
        const char* vprev = PAR ? v_lds0 : v_lds1;  // holds V_{j-1}
        const char* knext = PAR ? k_lds0 : k_lds1;  // holds K_{j+1}
        const bool do_pv = j >= 1 && j - 1 < n_w;
        const bool do_qk = j + 1 < n_w;
        const bool do_sm = SPLIT && j < n_w;
        const int j0 = j * kBN;
        __builtin_amdgcn_s_setprio(1);
        if (do_pv && do_qk && !(SPLIT && is_masked(j))) {
            if (copy_k) tile_to_lds<D>(PAR ? k_lds1 : k_lds0, kh, (j + 2) * kBN, N, gwave, k_src);
            if (copy_v) tile_to_lds<D>(PAR ? v_lds1 : v_lds0, vh, j * kBN, N, gwave, v_src);
            w.pv(vprev);
            w.rowsum();
            if constexpr (SPLIT) w.template prep<false>(sc, j0);
            w.qk(sn, knext);
            if constexpr (SPLIT) w.template exp_half<false, 0>(sc, j0);
            // Keep LDS operand reads a few matrix instructions ahead of their use and
            // spread the copies (and, with SPLIT, the vector work) between the matrix
            // instructions.
            __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
            for (int i = 0; i < 20; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                if (SPLIT) __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
                if (i % 4 == 3 && i < 16) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < 10) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                if (SPLIT) __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
                if (i % 4 == 3) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        } else {
            if (copy_k) tile_to_lds<D>(PAR ? k_lds1 : k_lds0, kh, (j + 2) * kBN, N, gwave, k_src);
            if (copy_v) tile_to_lds<D>(PAR ? v_lds1 : v_lds0, vh, j * kBN, N, gwave, v_src);
            if (do_pv) {
                w.pv(vprev);
                w.rowsum();
            }
            if (do_sm) {
                if (CAUSAL && is_masked(j)) {
                    diag(sc, j);
                    w.template prep<false>(sc, j0);
                    w.template exp_half<false, 0>(sc, j0);
                } else if (is_masked(j)) {
                    w.template prep<true>(sc, j0);
                    w.template exp_half<true, 0>(sc, j0);
                } else {
                    w.template prep<false>(sc, j0);
                    w.template exp_half<false, 0>(sc, j0);
                }
            }
            if (do_qk) w.qk(sn, knext);
        }
        __builtin_amdgcn_s_setprio(0);
    };
    auto softmax = [&](int j, f32x16(&sc)[2]) {
        if (j < 0 || j >= n_w) return;
        if constexpr (SPLIT) {
            // a causal diagonal tile was masked in place by the matrix half
            if (!CAUSAL && is_masked(j)) w.template exp_half<true, 1>(sc, j * kBN);
            else w.template exp_half<false, 1>(sc, j * kBN);
        } else {
            // Only the ping-pong form gets here.  It keeps the per-score mask: sharing the
            // unmasked code with the lane-mask path split that code into separate
            // scheduling regions, which cost 1-1.5% on long causal rows, where the
            // diagonal tile is rare.
            if (is_masked(j)) {
                w.template prep<true>(sc, j * kBN);
                w.template expsum<true>(sc, j * kBN);
            } else {
                w.template prep<false>(sc, j * kBN);
                w.template expsum<false>(sc, j * kBN);
            }
        }
        w.rescale();  // O (holding tiles up to j-1) *= alpha_j before P_j V_j
    };
    // One tile step: S_j is in s_cur, S_{j-1} (or nothing) in s_oth, which GEMM_j
    // refills with S_{j+1}.
    auto step = [&](auto par, int j, f32x16(&s_cur)[2], f32x16(&s_oth)[2]) {
        constexpr int PAR = decltype(par)::value;
        if constexpr (PP) {
            // half-step 2 j
            if (group == 0) {
                gemm(par, j, s_cur, s_oth, j + 2 < n_kv, false);
            } else {
                if (j > 0 && j < n_kv) tile_to_lds<D>(PAR ? v_lds1 : v_lds0, vh, j * kBN, N, gwave, v_src);
                softmax(j - 1, s_oth);
            }
            __syncthreads();
            // half-step 2 j + 1
            if (group == 0) {
                softmax(j, s_cur);
            } else {
                gemm(par, j, s_cur, s_oth, false, false);
            }
        } else {
            // one group: GEMM_j (with the copies of K_{j+2} and V_j), SOFTMAX_j
            gemm(par, j, s_cur, s_oth, j + 2 < n_kv, j > 0 && j < n_kv);
            softmax(j, s_cur);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K_{j+2} and V_j have landed
        __syncthreads();
    };

    int j = 0;
    for (; j + 1 <= n_kv; j += 2) {
        step(std::integral_constant<int, 0>{}, j, sa, sb);
        step(std::integral_constant<int, 1>{}, j + 1, sb, sa);
    }
    if (j <= n_kv) step(std::integral_constant<int, 0>{}, j, sa, sb);

    if (!wave_live) return;
    const float l_row = w.lacc[0];
    if (my_q < N) {
        const float inv = 1.0f / l_row;
        uint16_t* orow = p.o + head + (int64_t)my_q * D;
#pragma unroll
        for (int b = 0; b < DB; ++b) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u32x2 o2;
                o2[0] = E::pack2(w.acc[b][4 * i + 0] * inv, w.acc[b][4 * i + 1] * inv);
                o2[1] = E::pack2(w.acc[b][4 * i + 2] * inv, w.acc[b][4 * i + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + 32 * b + 8 * i + 4 * w.half) = o2;
            }
        }
        if (w.half == 0) p.lse[(int64_t)bh * N + my_q] = (w.m + fast_log2(l_row)) * kLn2;
    }
}

// Blocks of equal length (non-causal) run in rounds of `occ` per CU.  With three
// 4-wavefront blocks per CU a CU does about 5% more work per unit time than with two,
// and a lone block (one wavefront per SIMD) about 25% less; the last, partial round
// decides which occupancy finishes first.  Returns true when two per CU is expected to
// be faster for `per_cu` blocks on the busiest CU (for 4 blocks per CU: 4.0 against
// 4.19 units; 7% faster measured at B=4 H=16 N=2048 d=64).
bool two_per_cu_faster(int64_t per_cu) {
    auto cost = [](int64_t n, int occ) {
        constexpr double thr[4] = {0.0, 0.75, 1.0, 1.05};
        return double(n / occ) * occ / thr[occ] + ((n % occ) ? double(n % occ) / thr[n % occ] : 0.0);
    };
    return cost(per_cu, 2) < cost(per_cu, 3);
}

template <int D, bool CAUSAL, typename E, bool PP, bool TAIL>
hipError_t launch(Params p, hipStream_t st) {
    p.n_qtiles = (p.N + rows_of<PP>() - 1) / rows_of<PP>();
    const int64_t blocks = (int64_t)p.n_bh * p.n_qtiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    p.n_blocks = (int)blocks;
    // d = 64 without key masks fits three blocks per CU by registers; unused dynamic
    // LDS (4 K/V tiles of 8 KiB + 24 KiB = 56 KiB of the CU's 160 KiB) holds it to two
    // when that finishes sooner.
    unsigned lds_pad = 0;
    if constexpr (D == 64 && !CAUSAL && !TAIL) {
        const int cus = device_cu_count();
        if (two_per_cu_faster((blocks + cus - 1) / cus)) lds_pad = 24 << 10;
    }
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, E, PP, TAIL>), dim3((unsigned)p.n_blocks),
                       dim3(threads_of<PP>()), lds_pad, st, p);
    return hipGetLastError();
}

// The block form per shape, from interleaved timings on one MI355X (bitwise identical
// results either way).  Two 4-wavefront blocks per CU let one block's start, end and
// causal diagonal run beside the other block's steady state; the ping-pong is faster
// per key tile once blocks are long.  At d = 128 (with the causal head pairs of the
// kernel's dispatch) the two met near causal N = 10240 (N / 128 key tiles per 256-row
// block on average; the ping-pong led by 0.5% at 12288 and 1.7% at 16384) and, for the
// non-causal builds without key masks, at N = 2048 (ping-pong +2.5% at 4096, +3.7% at
// 8192); at d = 64 the 4-wavefront form was faster at every length timed (2048 to 32768).
template <int D, bool CAUSAL, typename E, bool TAIL>
hipError_t launch_form(const Params& p, hipStream_t st) {
    if constexpr (D == 64) {
        return launch<D, CAUSAL, E, false, TAIL>(p, st);
    } else {
        const bool pp = CAUSAL ? p.N > 10240 : p.N > 2048;
        return pp ? launch<D, CAUSAL, E, true, TAIL>(p, st) : launch<D, CAUSAL, E, false, TAIL>(p, st);
    }
}

template <int D, typename E>
hipError_t launch_mask(const Params& p, bool causal, hipStream_t st) {
    if (causal) return launch_form<D, true, E, true>(p, st);
    return p.N % kBN ? launch_form<D, false, E, true>(p, st) : launch_form<D, false, E, false>(p, st);
}

template <typename E>
hipError_t launch_fwd16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                        float scale, bool causal, hipStream_t st) {
    Params p;
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.o = static_cast<uint16_t*>(o);
    p.lse = lse;
    p.N = N;
    p.n_bh = (int64_t)B * H;
    // c = |scale| log2(e), kept at least 2^-100: at scale 0 every exponent c s - m is then
    // below 2^-24 in size for any score below 2^76, so exp2 returns exactly 1 and the
    // weights stay exactly uniform, while a masked score of -inf still gives probability
    // 0 rather than 0 * -inf = NaN.
    p.scale_log2 = fmaxf(fabsf(scale) * kLog2e, 0x1p-100f);
    p.negate_q = scale < 0.0f;  // flipping the sign bit negates exactly in bf16 and in fp16
    if (d == 64) return launch_mask<64, E>(p, causal, st);
    if (d == 128) return launch_mask<128, E>(p, causal, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                int H, int N, int d, float scale, bool causal, hipStream_t st) {
    return launch_fwd16<ElemBF16>(q, k, v, o, lse, B, H, N, d, scale, causal, st);
}

hipError_t launch_attn_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                               int H, int N, int d, float scale, bool causal, hipStream_t st) {
    return launch_fwd16<ElemF16>(q, k, v, o, lse, B, H, N, d, scale, causal, st);
}

}  // namespace mi355
