/*
 * fa.h -- C ABI of libfa, the MI355X (gfx950) FlashAttention library: the forward,
 * its split-KV form, the row softmax and the backward.
 *
 * The one operation is exact scaled-dot-product attention,
 *
 *     O = softmax(scale * Q K^T) V,      LSE = log of the softmax normaliser,
 *
 * computed tile by tile with the online-softmax recurrence: each query row
 * keeps a running maximum m, a running sum l of exponentials measured against
 * m, and an un-divided weighted sum u of value rows; when a new key tile raises
 * the maximum, l and u are multiplied by exp(m_old - m_new); after the last tile
 * O = u / l.  The N x N score matrix never reaches device memory.
 *
 * Sources (page, section):
 *  - the recurrence for (m, l) and its rescale factor: mbrenndoerfer.com
 *    "Online Softmax Computation", its update equations; spicyshark.co
 *    online-softmax lesson, "The idea".
 *  - carrying the weighted sum of values with the same factor, and dividing
 *    once at the end: kbwen.com FlashAttention feed, "Two blocks" and "More than
 *    two blocks"; spicyshark.co lesson, "From softmax to attention";
 *    paweldubiel.com FlashAttention note, "Averaging block results is not
 *    enough".
 *  - query blocks in the outer loop, key/value blocks in the inner loop, per-row
 *    state on chip: kbwen.com feed, "More than two blocks" (last paragraphs).
 *  - causal masking by -inf scores, and the guard for a block with no finite
 *    score: spicyshark.co lesson, "The implementation".
 *  - grouped-query attention (fewer K/V heads than query heads): paweldubiel.com
 *    note, "Averaging block results is not enough" (last paragraph).
 *  - the per-row logsumexp is not on the pages: LSE = m + ln(l), the natural
 *    log of the normaliser, in units of the scaled score.
 *
 * Layout (all contiguous, row-major, head dimension fastest):
 *     q, o   [B][Hq][N][d]        k, v   [B][Hkv][N][d]        lse  [B][Hq][N]
 * Query head h reads K/V head h / (Hq / Hkv).  With causal = 1, key j is
 * visible to query i iff j <= i (queries and keys share the index 0..N-1).
 * o has the input dtype; lse is always float32.
 *
 * Ownership: every buffer belongs to the caller and is device memory of the
 * device the stream belongs to.  The library never allocates, frees or keeps a
 * pointer past the call; the only workspace it takes is fa_bwd_split's dkv_part
 * (fa_bwd_split_noalloc uses a static array of the library in its place).
 * q, k and v are only read; o and lse must not overlap the inputs or each other.
 * Every pointer must be 16-byte aligned.
 *
 * Errors: FA_ERR_INVALID_ARG and FA_ERR_UNSUPPORTED mean nothing was enqueued:
 * arguments are checked on the host before any HIP call.  FA_ERR_HIP reports a
 * failed launch; fa_last_error() then holds the HIP message (thread-local).  A
 * call that launches several kernels (the backward; a row softmax of more than
 * 2^23 rows, launched in pieces) may have enqueued the ones before it.
 * The call is asynchronous: faults during execution show at the caller's next
 * synchronisation of the stream.  No global mutable state beyond the
 * thread-local message: calls are re-entrant and may run on several streams and
 * threads at once.  Results are bitwise reproducible run to run (no atomics).
 */
#ifndef FA_H
#define FA_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_dtype {
    FA_DTYPE_F32 = 0,   /* float32 inputs, float32 MFMA, float32 output      */
    FA_DTYPE_BF16 = 1,  /* bfloat16 inputs, fp32 accumulate, bfloat16 output  */
    FA_DTYPE_F16 = 2    /* float16 inputs, fp32 accumulate, float16 output    */
} fa_dtype;

enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,   /* bad pointer, size, flag, alignment or overlap */
    FA_ERR_UNSUPPORTED = 2,   /* valid request the library does not implement  */
    FA_ERR_HIP = 3            /* the HIP runtime refused the launch            */
};

/*
 * fa_fwd: O and LSE for every query row.
 *
 *   q, k, v   device pointers to the inputs (dtype as given), layouts above
 *   o         device pointer, [B][Hq][N][d] in the input dtype (written)
 *   lse       device pointer, [B][Hq][N] float32 (written)
 *   B, N      >= 0; when either is 0 there is nothing to do and FA_OK is
 *             returned without touching any pointer
 *   Hq, Hkv   >= 1 with Hq % Hkv == 0
 *   d         64 or 128 (other positive values: FA_ERR_UNSUPPORTED)
 *   causal    0 or 1
 *   scale     any finite float whose product with log2(e) is finite in float32;
 *             multiplies q.k before the softmax (1/sqrt(d) gives the usual
 *             attention).  The scaled scores scale * q.k of visible pairs must
 *             stay below 2^29 in magnitude: the kernels subtract the row maximum
 *             after scaling, in float32, and beyond that the maximum's own
 *             rounding can overflow the exponentials (a 0 scale gives uniform
 *             weights; a negative one reverses the order of the scores)
 *   v         values' magnitude: the 16-bit kernels let a row's maximum run up
 *             to 2^8 (bf16 at d = 128: 2^48) above the reference they subtract
 *             before moving it, so O's float32 sums reach N * 2^48 * max|v|;
 *             bf16 inputs at d = 128 need N * max|v| < 2^80, the others
 *             N * max|v| < 2^120
 *   dtype     FA_DTYPE_F32, FA_DTYPE_BF16 or FA_DTYPE_F16
 *   stream    hipStream_t to enqueue on; NULL means the default stream
 *
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
           int dtype, void* stream);

/*
 * fa_fwd_tiled: fa_fwd with an explicit tile shape (block_m query rows per
 * workgroup, block_n keys per K/V tile).  Used to show that the result does not
 * depend on the tiling (the pages' block-size invariance, kbwen.com feed "More
 * than two blocks").  Shapes the library does not hold return
 * FA_ERR_UNSUPPORTED; fa_tile_shapes lists the ones it does.
 */
int fa_fwd_tiled(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                 int dtype, void* stream, int block_m, int block_n);

/*
 * fa_fwd_stamped: fa_fwd (bf16 or fp16, default tile) that also records when each
 * wave of the launch ran, for measuring the shader clock the kernel actually ran
 * at and the spread of work over the grid.  Not part of the method: the pages
 * give no hardware figures; this is the measurement side of the forward.
 *
 *   stamps       device pointer, 32-byte aligned, at least stamp_slots * 4
 *                unsigned 64-bit words, written: for wave w of the launch,
 *                stamps[4w + 0], [4w + 1] = the constant-rate real-time counter
 *                (fa_wall_clock_khz kHz) when the wave started and ended;
 *                stamps[4w + 2], [4w + 3] = the shader-cycle counter at the same
 *                two points, so (cycles / real-time ticks) * wall clock rate is the
 *                wave's average shader clock.  Must not overlap any other argument.
 *   stamp_slots  the buffer's capacity in waves; fa_fwd_stamp_slots gives a
 *                number the launch cannot exceed (fewer than the launch has:
 *                FA_ERR_INVALID_ARG); slots past the launch's waves are not
 *                written.  A wave may cover several query tiles in turn: its
 *                stamps span all of them
 *   other arguments, ownership and errors: as for fa_fwd; FA_DTYPE_F32 returns
 *   FA_ERR_UNSUPPORTED.  o and lse are bitwise the same as fa_fwd's.
 */
int fa_fwd_stamped(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                   int dtype, void* stream, unsigned long long* stamps, long long stamp_slots);

/* Waves of an fa_fwd launch of this shape (16-bit dtypes), i.e. the slots
 * fa_fwd_stamped writes; -1 for a bad size or dtype. */
long long fa_fwd_stamp_slots(int B, int Hq, int N, int d, int dtype);

/* Rate of the real-time counter of device `device` in kHz (hipDeviceAttributeWallClockRate),
 * or -1 if the runtime does not report it. */
int fa_wall_clock_khz(int device);

/*
 * fa_tile_shapes: the (block_m, block_n) pairs compiled for (dtype, d).
 * Writes up to cap pairs into block_m[] and block_n[] (either may be NULL when
 * cap is 0) and returns how many exist, or -1 for an unknown dtype/d.  The
 * first pair is the one fa_fwd uses.
 */
int fa_tile_shapes(int dtype, int d, int* block_m, int* block_n, int cap);

/*
 * fa_fwd_splitkv: partial attention states over contiguous key ranges
 * (split-KV).  Each range yields the state (m, l, acc) the pages carry from
 * one block of keys, in normalised form; fa_merge then combines the ranges with
 * the pages' merge of states of disjoint key sets (kbwen.com feed, "Two
 * blocks": the first block alone is the answer for a query with only those keys;
 * spicyshark.co online-softmax lesson, "From softmax to attention", two workers
 * merging their halves, and its "Check yourself" answer).
 *
 *   q         [B][Hq][Nq][d]; k, v [B][Hkv][Nk][d]; bf16 or fp16.  The queries are
 *             the last Nq positions of the Nk keys: with causal = 1, key j is
 *             visible to query i iff j <= i + (Nk - Nq); causal needs Nq <= Nk.
 *             (Nq == Nk is the square problem of fa_fwd.)
 *   splits    num_splits in 1..1024; range s holds keys
 *             [s*c, min(Nk, (s+1)*c)) with c = fa_split_chunk(Nk, num_splits)
 *             (ranges past Nk are empty)
 *   o_part    [num_splits][B][Hq][Nq][d] float32 (written): the attention output
 *             of each row over the range's visible keys alone, acc / l
 *   lse_part  [num_splits][B][Hq][Nq] float32 (written): m + ln l of that state;
 *             a row with no visible key in the range gets lse = -inf and o = 0
 *             (the empty state, which carries no weight in the merge)
 *   B, Nq     >= 0 (0: FA_OK, nothing touched); Nk >= 1 when Nq >= 1;
 *             (Hq / Hkv) * Nq <= 2^31 - 129 and (Nk + 128) * d * 2 < 2^31
 *             (else FA_ERR_UNSUPPORTED)
 *   Hq, Hkv, d, scale, stream: as for fa_fwd; dtype FA_DTYPE_BF16 or
 *             FA_DTYPE_F16 (FA_DTYPE_F32 returns FA_ERR_UNSUPPORTED)
 * Ownership, alignment, overlap and error rules as for fa_fwd (o_part and lse_part
 * take the place of o and lse).
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                   int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                   int dtype, int num_splits, void* stream);

/*
 * fa_merge: combine num_splits partial states per row.
 *
 *   o_part    [num_splits][B][H][N][d] float32, lse_part [num_splits][B][H][N]
 *             float32: states in the form fa_fwd_splitkv writes (read only)
 *   o         [B][H][N][d] in dtype (FA_DTYPE_F32, FA_DTYPE_BF16 or FA_DTYPE_F16), written
 *   lse       [B][H][N] float32, written
 *   per row:  m = max_s lse_s,  w_s = exp(lse_s - m),  lse = m + ln sum_s w_s,
 *             o = sum_s w_s o_s / sum_s w_s; a row whose states are all empty
 *             gets o = 0 and lse = -inf
 *   d         64 or 128; B, N >= 0 (0: FA_OK, nothing touched); H >= 1;
 *             B * H * N <= 67108860 rows (one launch of four rows per workgroup
 *             within 2^32 work-items; FA_ERR_UNSUPPORTED beyond)
 * Any set of states of disjoint key sets in this form may be merged, e.g. the
 * outputs of fa_fwd_splitkv over different K/V shards.  Ownership, alignment,
 * overlap and error rules as for fa_fwd.
 */
int fa_merge(const float* o_part, const float* lse_part, void* o, float* lse, int num_splits,
             int B, int H, int N, int d, int dtype, void* stream);

/* Keys per range of fa_fwd_splitkv: ceil(Nk / num_splits) rounded up to a
 * multiple of 64; -1 for Nk < 0 or num_splits outside 1..1024. */
int fa_split_chunk(int Nk, int num_splits);

/* A split count that fills the GPU for this shape (about 1024 workgroups, at
 * least 256 keys per range; a workgroup serves 128 rows of the Hq/Hkv query
 * heads that share one K/V head), or -1 for a bad size. */
int fa_splitkv_num_splits(int B, int Hq, int Hkv, int Nq, int Nk);

/* Algorithms of fa_softmax. */
enum {
    FA_SOFTMAX_ONLINE = 0,   /* running max and sum in one read, then the output: 2 reads + 1 write */
    FA_SOFTMAX_SAFE = 1      /* max, then sum, then the output: 3 reads + 1 write                 */
};

/*
 * fa_softmax: the softmax of every row of a matrix,
 *     y[r][j] = exp(x[r][j] - m_r) / l_r,   m_r = max_j x[r][j],
 *     l_r = sum_j exp(x[r][j] - m_r),       lse[r] = m_r + ln l_r,
 * the safe softmax of the pages (spicyshark.co online-softmax lesson, "The fix:
 * subtract the maximum").  algo picks how often each row is read ("The cost: three
 * passes"; "Why reading once matters"; "The idea" for the running max and sum
 * that the online form keeps, the update of Milakov and Gimelshein the pages cite).
 *
 *   x, y      device pointers, [rows][cols] contiguous, dtype FA_DTYPE_F32,
 *             FA_DTYPE_BF16 or FA_DTYPE_F16 (both the same dtype; the arithmetic is
 *             fp32); y may be x itself (in place) but must not otherwise overlap it
 *   lse       device pointer, [rows] float32, written; may be NULL
 *   rows      0 .. 2^31 - 1 (0: FA_OK, nothing touched)
 *   cols      1 .. 2^31 - 4096 (longer rows: FA_ERR_UNSUPPORTED)
 *   algo      FA_SOFTMAX_ONLINE or FA_SOFTMAX_SAFE (same result up to rounding)
 * A row whose entries are all -inf has no softmax: its y is nan and its lse -inf.
 * Ownership, alignment (16 bytes for x, y and lse) and error rules as for fa_fwd.
 */
int fa_softmax(const void* x, void* y, float* lse, long long rows, int cols, int dtype, int algo,
               void* stream);

/*
 * fa_bwd: gradients of the square problem of fa_fwd with respect to q, k and v,
 * given the upstream gradient dout of o.  The forward's N x N weights are not
 * kept: the backward recomputes them from q, k and the forward's lse (the
 * paweldubiel.com FlashAttention note, "Mechanism and details", and the
 * spicyshark.co lesson, "Further reading": training recomputes in the backward
 * what the forward did not store).  With P = softmax(scale q K^T) (masked keys 0):
 *     D  = rowsum(dout * o),   dP = dout v^T,   dS = P * (dP - D)
 *     dq = scale dS k,         dk = scale dS^T q,   dv = P^T dout
 * dk and dv of a K/V head sum over the Hq/Hkv query heads that read it.
 *
 *   q, k, v, o, lse   the forward's inputs and outputs (o and lse as fa_fwd wrote
 *             them for the same q, k, v, causal and scale), read only
 *   dout      [B][Hq][N][d] in dtype, read only
 *   dq        [B][Hq][N][d] in dtype, written
 *   dk, dv    [B][Hkv][N][d] in dtype, written
 *   delta     [B][Hq][N] float32, written: D of every row (workspace of the call,
 *             returned because it is useful)
 *   dtype     FA_DTYPE_BF16 or FA_DTYPE_F16 (FA_DTYPE_F32: FA_ERR_UNSUPPORTED);
 *             products in the 16-bit type with fp32 accumulation, P and dS
 *             rounded to the 16-bit type as the MFMA operands they are
 *   B, N, Hq, Hkv, d, causal, scale, stream: as for fa_fwd
 * dq, dk, dv and delta must not overlap each other or any input.  Ownership,
 * alignment and error rules as for fa_fwd.  Every output element is accumulated
 * in a fixed order: results are bitwise reproducible (no atomics).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int Hq, int Hkv,
           int N, int d, int causal, float scale, int dtype, void* stream);

/*
 * fa_bwd_split: fa_bwd with the dK/dV work of each 128-key tile shared out over
 * num_splits workgroups, for problems whose grid of key tiles is too small to fill
 * the GPU evenly (e.g. one sequence of a GQA model with 8 K/V heads): split s takes
 * a contiguous share of the key tile's (query head, 32-query tile) pairs.  Each
 * split writes fp32 partial sums, which a last kernel adds in split order and rounds
 * into dk and dv, so results stay bitwise reproducible (and may differ from
 * fa_bwd's only by the rounding of that sum).
 *
 *   dkv_part    [2][num_splits][B][Hkv][N][d] float32 device workspace owned by the
 *               caller (partial dK planes, then dV planes); contents on entry are
 *               ignored; may be NULL when num_splits is 1; must not overlap any
 *               other argument
 *   num_splits  1..8; 1 is fa_bwd exactly; fa_bwd_num_splits suggests one
 *   other arguments, ownership, alignment and errors: as for fa_bwd
 */
int fa_bwd_split(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, float* delta, float* dkv_part,
                 int num_splits, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                 int dtype, void* stream);

/* A split count for fa_bwd_split that gives about 1024 dK/dV workgroups (1 when the
 * key tiles alone reach that, at most 8), or -1 for a bad size. */
int fa_bwd_num_splits(int B, int Hq, int Hkv, int N);

/*
 * fa_bwd_split_noalloc: fa_bwd_split without the caller's workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The fp32 dK/dV partials go to a static device
 * array of the library instead of dkv_part: fa_bwd_noalloc_max_bytes() bytes
 * (128 MiB), one copy per GPU, held from the library's first use on that GPU until
 * the process ends.  The call allocates nothing.
 *
 *   num_splits  1..8 as for fa_bwd_split; the partials take
 *               2 * num_splits * B * Hkv * N * d * 4 bytes (none when num_splits is 1);
 *               more than the array holds returns FA_ERR_UNSUPPORTED, nothing enqueued
 *   other arguments, ownership, alignment and errors: as for fa_bwd_split.  The results
 *   are bitwise fa_bwd_split's for the same arguments.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (other streams, other threads) race and must be serialised by the caller.  Nothing
 * in it needs clearing: each call overwrites the part it reads.
 */
int fa_bwd_split_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv, float* delta, int num_splits,
                         int B, int Hq, int Hkv, int N, int d, int causal, float scale, int dtype,
                         void* stream);

/* Bytes of the static workspace of fa_bwd_split_noalloc. */
long long fa_bwd_noalloc_max_bytes(void);

/* Static text for a return code. */
const char* fa_error_string(int code);

/* Detail of the last failure on the calling thread ("" if none). */
const char* fa_last_error(void);

/* ABI version of this header: 7. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
