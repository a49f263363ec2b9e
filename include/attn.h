/*
 * attn.h -- C ABI of the MI355X (gfx950) tiled online-softmax attention
 * forward library (libattn.so).
 *
 * The operation is exact scaled-dot-product attention,
 *
 *     O_i   = sum_{j in Vis(i)} exp(s_ij - m_i) v_j / l_i,
 *     s_ij  = scale * q_i . k_j,   m_i = max_j s_ij,   l_i = sum_j exp(s_ij - m_i),
 *     LSE_i = m_i + ln l_i,
 *
 * as defined by the direct reference of "Verify tiled attention" (section
 * "Compare the attention outputs") and by "FlashAttention implemented,
 * verified and measured" (section "The reference implementation, in full").
 * The library computes it tile by tile with the online softmax of "Tiled
 * attention: preserving results without a full score matrix" (section
 * "Online normalization"): per query row a running maximum m, a normaliser l
 * and an unnormalised accumulator a, with l and a rescaled by exp(m_old -
 * m_new) whenever a key/value tile raises the maximum, and O = a / l at the
 * end.  The score matrix never leaves the chip.
 *
 * Visibility: key j is visible to query row i iff j < Skv and, for causal
 * attention (causal = 1), j <= i + (Skv - Sq): the "j <= i" causal rule of
 * the lab page, aligned to the end of the key sequence when Sq != Skv.
 * causal = 2 aligns the rule to the start instead (j <= i).  The two agree
 * when Sq == Skv.  A row with no visible key (Skv == 0, or end-aligned causal
 * with i < Sq - Skv) gets O = 0 and LSE = -inf; no NaN is produced.
 *
 * Layout (all tensors dense, row-major, the head dimension fastest):
 *     q, o : [B, H, Sq,  d]
 *     k, v : [B, H, Skv, d]       (value width equals d)
 *     lse  : [B, H, Sq]  float32  (natural log of the sum of exponentials
 *                                  of the scaled scores)
 *
 * Ownership and execution: every pointer is a device pointer on the current
 * HIP device, owned by the caller.  The library allocates no device memory,
 * never synchronises, and only enqueues work on `stream` (a hipStream_t; NULL
 * means the null stream).  Calls return as soon as the work is enqueued;
 * faults inside the kernels surface at the caller's next synchronisation.
 * Argument validation happens on the host before any HIP call.  All entry
 * points are thread-safe; the error message is kept per thread.  For a fixed
 * tile configuration results are bitwise deterministic (no atomics).
 */
#ifndef ATTN_H
#define ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  Accumulation is always at least fp32. */
typedef enum {
    ATTN_F32 = 0,          /* q, k, v, o float32.  Scores are accumulated in
                              float64 (fp32 x fp32 products are exact there) so
                              that scores of magnitude ~1e2-1e3 keep their
                              fp32-level relative accuracy after the max shift;
                              exponentials, l and P.V are fp32.              */
    ATTN_BF16 = 1,         /* q, k, v, o bfloat16; QK^T and P.V on bf16 MFMA
                              with fp32 accumulation, P rounded to bf16 (RNE). */
    ATTN_BF16_OUT_F32 = 2, /* q, k, v bfloat16, o float32 (same arithmetic as
                              ATTN_BF16, output not rounded to bf16).         */
    ATTN_F16 = 3,          /* q, k, v, o float16 (IEEE half); fp16 MFMA with
                              fp32 accumulation, P rounded to fp16 (RNE).     */
    ATTN_F16_OUT_F32 = 4   /* q, k, v float16, o float32.                     */
} attn_dtype;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1,  /* null pointer for a non-empty tensor, negative
                                  size, non-finite or non-positive scale,
                                  unknown dtype, causal not 0/1/2, size overflow,
                                  o aliasing an input                         */
    ATTN_ERR_UNSUPPORTED = 2,  /* head dim or forced tile shape not built      */
    ATTN_ERR_MISALIGNED = 3,   /* a pointer not 16-byte aligned                */
    ATTN_ERR_HIP = 4           /* the HIP runtime reported an error at launch  */
} attn_status;

/*
 * attn_fwd -- enqueue O (and LSE) = attention(q, k, v) on `stream`.
 *
 *   q, k, v  : inputs, layout above, element type per `dtype`.
 *   o        : output [B, H, Sq, d]; must not overlap q, k, v or lse.
 *   lse      : output [B, H, Sq] float32, or NULL to skip it.
 *   B, H     : batch and heads (>= 0).
 *   Sq, Skv  : query and key lengths (>= 0).  Sq == 0 is a no-op.
 *   d        : head dimension: 16, 32, 64 or 128 (fp32); 32, 64 or 128
 *              (bf16, fp16).
 *   scale    : score scale, finite and > 0 (usually 1/sqrt(d)).
 *   causal   : 0 (none), 1 (end-aligned mask above) or 2 (start-aligned).
 *   dtype    : an attn_dtype.
 *   stream   : hipStream_t or NULL.
 * Returns an attn_status; on failure attn_last_error() describes it and
 * nothing was enqueued (except for ATTN_ERR_HIP, reported after a launch).
 * Tiles come from attn_select_tiles().
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Sq, int Skv, int d, float scale, int causal,
             int dtype, void* stream);

/*
 * attn_fwd_tiles -- attn_fwd with a forced tile shape: `block_m` query rows
 * and `block_n` key rows per tile (the block_q / block_kv of the tiled lab
 * function on "Verify tiled attention").  block_m = block_n = 0 means "use
 * the selector".  Built shapes:
 *   ATTN_F32            block_m in {16, 32, 64},  block_n in {16, 32, 64}
 *                       (every d), and block_m = 16 with block_n = 128
 *   ATTN_BF16[_OUT_F32], ATTN_F16[_OUT_F32]
 *                       block_m in {64, 128},     block_n in {32, 64} (d = 64,
 *                       128) or block_n = 64 (d = 32), block_m = 128 with
 *                       block_n = 128 when d = 32, and block_m = 256 with
 *                       block_n = 32 when d = 128
 * Any other pair returns ATTN_ERR_UNSUPPORTED.
 */
int attn_fwd_tiles(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Sq, int Skv, int d, float scale, int causal,
                   int dtype, void* stream, int block_m, int block_n);

/*
 * attn_select_tiles -- the tile / occupancy selector (host only, no HIP
 * call).  "Verify tiled attention", section "Separate storage savings from
 * runtime": the tile size, register pressure, cache reuse and precision of
 * the chosen kernel decide its speed, so the choice is made here per head
 * dimension, dtype and grid size rather than fixed.  On the 16-bit path,
 * d = 32 takes 128-key tiles in 128-row workgroups and 64-key tiles in
 * 64-row ones (a 32-key tile would give each step only two score MFMAs, too
 * few to hide the softmax under), d = 64 takes 64-key tiles in 128-row
 * workgroups and 32-key tiles in 64-row ones, d = 128 takes 32-key tiles.
 * Writes the tile shape attn_fwd would use for this problem:
 * query rows per workgroup, key rows per tile, 64-wide waves per workgroup
 * and LDS bytes per workgroup.  fp32 waves own 16 query rows each; with
 * 16-row query tiles on a grid of fewer than 512 (1024) query tiles, four
 * (two) waves share each 16-row block, each taking its part of every key
 * tile, and merge their states at the end (at most block_n / 16 waves).
 * fp32 grids of fewer than 512 such tiles over more than 128 keys at
 * d <= 64 take 128-key tiles shared by eight waves (16 keys each); forced
 * 128-key tiles run eight waves, four at d = 128.
 * `BH` is B * H.  Any output pointer may be NULL.  Returns ATTN_OK,
 * ATTN_ERR_INVALID_ARG or ATTN_ERR_UNSUPPORTED.
 */
int attn_select_tiles(int d, int Sq, int Skv, int BH, int dtype, int causal,
                      int* block_m, int* block_n, int* waves, int* lds_bytes);

/*
 * attn_fwd_split -- attn_fwd with the key range cut into chunks that run in
 * separate workgroups, for problems whose query tiles alone leave compute
 * units idle (few heads, short query blocks against long key sequences, as
 * in decoding against a cached prefix).  Each chunk c produces the partial
 * state of the online normalisation of "Tiled attention: preserving results
 * without a full score matrix" (section "Online normalization") over its own
 * keys -- O_c = a_c / l_c and LSE_c = m_c + ln l_c -- and a second kernel
 * merges the states of each row with the same rescale rule applied to whole
 * states: M = max_c LSE_c, w_c = exp(LSE_c - M),
 *     O = sum_c w_c O_c / sum_c w_c,   LSE = M + ln sum_c w_c.
 * Results equal attn_fwd's up to rounding (not bitwise).
 *
 *   q ... stream  : as attn_fwd (tiles from attn_select_tiles).
 *   n_splits      : number of key chunks; 0 = choose (attn_select_splits).
 *                   Rounded to whole key tiles, so fewer chunks may run; 1
 *                   runs attn_fwd's path.  At most 4096.
 *   workspace     : caller-owned device buffer, 256-byte aligned, of at least
 *                   attn_split_workspace_bytes(B, H, Sq, d, n) bytes for the
 *                   number of chunks that runs (for n_splits = 0, ask
 *                   attn_select_splits).  It must not overlap q, k, v, o or
 *                   lse.  May be NULL when one chunk runs.  Its contents are
 *                   scratch: overwritten, never read before written.
 *   workspace_bytes : its size.
 * Returns as attn_fwd; ATTN_ERR_INVALID_ARG also for a missing or too small
 * workspace, ATTN_ERR_MISALIGNED for a workspace not 256-byte aligned.
 * Enqueues two kernels on `stream` when the key range is split.
 */
int attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Sq, int Skv, int d, float scale, int causal,
                   int dtype, void* stream, int n_splits, void* workspace,
                   long long workspace_bytes);

/*
 * attn_select_splits -- the key-chunk count attn_fwd_split uses for
 * n_splits = 0 (host only, no HIP call): 1 when the query tiles alone reach
 * the target, else enough chunks of whole key tiles to reach it (at most
 * 64).  Target: one workgroup per compute unit for 16-bit inputs, four
 * waves per compute unit (one per SIMD) for fp32; fp32 key ranges of fewer
 * than four key tiles stay in one chunk.  Writes the count and the
 * chunk length in keys; either pointer may be NULL.  Returns as
 * attn_select_tiles.
 */
int attn_select_splits(int d, int Sq, int Skv, int BH, int dtype, int causal,
                       int* n_splits, int* kv_chunk);

/*
 * attn_split_workspace_bytes -- bytes of workspace attn_fwd_split needs for
 * n_splits key chunks: partial O [n_splits, B, H, Sq, d] fp32, then at a
 * 256-byte boundary partial LSE [n_splits, B, H, Sq] fp64.  Returns -1 for
 * invalid sizes (negative, d <= 0, n_splits outside [1, 4096]).
 */
long long attn_split_workspace_bytes(int B, int H, int Sq, int d, int n_splits);

/*
 * attn_fwd_split_noalloc -- attn_fwd_split for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc.  It allocates nothing (no hipMalloc, hipFree or
 * allocating library call); the key chunks' partial states go to a static
 * device array of ATTN_NOALLOC_SCRATCH_BYTES bytes inside the library, one
 * copy per device, held from the library's first use on that device until
 * the process ends.  Its address is looked up once per device, on the
 * first call made with that device current.
 *
 *   q ... n_splits : as attn_fwd_split; the call runs on the current
 *                    device, and `stream` (if not NULL) must belong to it.
 * The chunk plan, kernels and results are those of attn_fwd_split with the
 * same arguments (bitwise).  The scratch needs no clearing: every byte a
 * call reads was written earlier in the same call.  All calls on one device
 * share its array: calls that overlap in time on one device (different
 * streams, host threads) race and give wrong results; calls in one stream
 * are ordered and safe.
 * Returns as attn_fwd_split; ATTN_ERR_INVALID_ARG (nothing enqueued) when
 * the chunks that would run need more than ATTN_NOALLOC_SCRATCH_BYTES
 * (attn_split_workspace_bytes of that chunk count) or `stream` belongs to
 * another device; ATTN_ERR_HIP if the array's address cannot be found.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (64ll << 20)
int attn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Sq, int Skv, int d, float scale, int causal,
                           int dtype, void* stream, int n_splits);

/* attn_last_error -- message for the last non-OK status on this thread
 * ("" if none).  The string stays valid until the next call on the thread. */
const char* attn_last_error(void);

/* attn_version -- library ABI version (major * 100 + minor). */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
