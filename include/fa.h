/*
 * fa.h -- C ABI of libfa, the MI355X (gfx950) FlashAttention forward library.
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
 * pointer past the call and takes no workspace.  q, k and v are only read; o and
 * lse must not overlap the inputs or each other.  Every pointer must be 16-byte
 * aligned.
 *
 * Errors: a return value other than FA_OK means nothing was enqueued.  Argument
 * errors are found on the host before any HIP call.  FA_ERR_HIP reports a
 * failed launch; fa_last_error() then holds the HIP message (thread-local).
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
    FA_DTYPE_F16 = 2    /* reserved: returns FA_ERR_UNSUPPORTED               */
} fa_dtype;

enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,   /* bad pointer, size, flag, alignment or overlap */
    FA_ERR_UNSUPPORTED = 2,   /* valid request this build does not implement   */
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
 *   scale     any finite float; multiplies q.k before the softmax
 *             (1/sqrt(d) gives the usual attention)
 *   dtype     FA_DTYPE_F32 or FA_DTYPE_BF16
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
 * than two blocks").  Shapes this build does not hold return
 * FA_ERR_UNSUPPORTED; fa_tile_shapes lists the ones it does.
 */
int fa_fwd_tiled(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                 int dtype, void* stream, int block_m, int block_n);

/*
 * fa_tile_shapes: the (block_m, block_n) pairs compiled for (dtype, d).
 * Writes up to cap pairs into block_m[] and block_n[] (either may be NULL when
 * cap is 0) and returns how many exist, or -1 for an unknown dtype/d.  The
 * first pair is the one fa_fwd uses.
 */
int fa_tile_shapes(int dtype, int d, int* block_m, int* block_n, int cap);

/* Static text for a return code. */
const char* fa_error_string(int code);

/* Detail of the last failure on the calling thread ("" if none). */
const char* fa_last_error(void);

/* ABI version of this header: 1. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
