/*
 * fa.h -- C ABI of libfa.so, a FlashAttention forward pass for AMD MI355X (gfx950).
 *
 * Operation (fa_fwd):  O = softmax(scale * Q K^T + mask) V, per batch and query head, computed
 * tile by tile with a running (online) softmax so the S x S score matrix never reaches device
 * memory.  Pages this follows:
 *   - https://yetianai.com/news/16520, section "传统进化搜索的天花板": FlashAttention computes
 *     attention block-wise without storing the full attention matrix; FA4's correction step
 *     rescales the accumulator of the single-pass softmax.  Section "七天跑出的成绩单": forward
 *     prefill at head dim 128 in bf16, causal and non-causal, MHA and GQA (32 query heads over 4
 *     or 8 KV heads).
 *   - https://yunpan.plus/t/19526-1-1, section "AI生成的代码质量如何？", excerpt 2: the custom
 *     mask is one bit per (query row, key); key j is bit j % 32 of word j / 32 (least significant
 *     bit first); a set bit keeps the score; rows and keys at or beyond seq_len are never kept.
 *
 * Result definition, for batch b, query head h, query row i < S, with G = n_q_heads/n_kv_heads
 * and KV head g = h / G (each run of G consecutive query heads shares one KV head):
 *     s_j  = scale * <Q[b,i,h,:], K[b,j,g,:]>                 for keys j < S
 *     kept = none: every j;  causal: j <= i;  bitmask: bit (j % 32) of mask[b,h,i,j/32]
 *     O[b,i,h,:] = sum_j softmax over kept j (s_j) * V[b,j,g,:];   O = 0 when no key is kept.
 *
 * Layouts (row-major, contiguous, element strides implied by the shapes):
 *     q, o  [batch, seq_len, n_q_heads,  head_dim]   dtype elements (2 bytes)
 *     k, v  [batch, seq_len, n_kv_heads, head_dim]   dtype elements
 *     mask  [batch, n_q_heads, seq_len, W] uint32, W = ceil(seq_len / 32); bits for keys >= S
 *           are ignored.  Only read in FA_MASK_BITMASK mode.
 *
 * Numerics: Q K^T and P V run on bf16/fp16 matrix cores with fp32 accumulation; softmax runs in
 * fp32 (exp2 with log2(e) folded into the scale); P is rounded to the input dtype before P V;
 * O is rounded to the input dtype (round to nearest even).  The running max a row's weights are
 * taken against may trail its true max (it moves only when a lane's sum of a tile's weights
 * would pass 2^15), so weights up to 2^15 are rounded like all others instead of the largest
 * being exactly 1.  A negative scale is handled exactly
 * (the sign is moved onto Q).  Inputs must be finite and |scale * s_j| must stay below 1e30.
 * Results are bitwise deterministic for a given input and device.
 *
 * Ownership and threading: every pointer is a DEVICE pointer owned by the caller, 16-byte
 * aligned (mask: 4-byte aligned).  o must not alias q, k, v or mask.  The call never
 * synchronises; its work is enqueued on `stream` (a hipStream_t; NULL = default stream):
 *   - when a KV head's rows (seq_len x n_q_heads / n_kv_heads) make 32 or more row tiles of the
 *     call's workgroups, 64 for causal at head_dim 128 (fa_fwd_plan's packed_v: causal at
 *     head_dim 64 from 3969 rows, causal at head_dim 128 from 16129 rows, every other case from
 *     7937 rows), two kernels: a
 *     pre-pass that packs V into transposed tiles in a temporary device buffer (batch x
 *     n_kv_heads x ceil(seq_len / 64) x 64 x head_dim x 2 bytes, about the size of V), then the
 *     attention kernel.  The buffer is allocated and freed stream-ordered on `stream`
 *     (hipMallocFromPoolAsync / hipFreeAsync) from a memory pool the library creates on first
 *     use on each device and keeps until the process ends (memory freed to it is retained);
 *   - otherwise the attention kernel alone.
 * A caller that must not allocate passes its own buffer to fa_fwd_ex (`workspace`, sized by
 * fa_fwd_plan) and no pool is used.  The library keeps no other state (besides the per-thread
 * event pair of fa_set_kernel_events).  Calls are safe from several host threads.
 *
 * Errors: arguments are validated first, synchronously, with no HIP call; on error nothing is
 * enqueued and o is untouched.  A failed workspace allocation or a launch error reported by
 * HIP returns FA_ERR_HIP (after an allocation failure no kernel is enqueued; a buffer the call
 * had already taken is returned to the pool stream-ordered).  Faults during
 * execution surface at the caller's next synchronisation, as for any HIP kernel.  Nothing is
 * printed and no C++ exception crosses this interface.
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 9

typedef enum {
  FA_MASK_NONE = 0,     /* every key kept */
  FA_MASK_CAUSAL = 1,   /* key j kept for query i iff j <= i (diagonal kept) */
  FA_MASK_BITMASK = 2   /* packed per-(query, key) bits, 1 = keep */
} fa_mask_mode;

typedef enum { FA_DTYPE_F16 = 0, FA_DTYPE_BF16 = 1 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL_PTR = 1,      /* q, k, v or o (or fa_fwd_lse's lse) is NULL */
  FA_ERR_BAD_SHAPE = 2,     /* batch, seq_len or a head count <= 0, n_q_heads % n_kv_heads != 0,
                               or a tensor larger than 2^31 elements per batch */
  FA_ERR_UNSUPPORTED = 3,   /* head_dim not 64 or 128, unknown dtype, misaligned pointer */
  FA_ERR_BAD_MASK_MODE = 4, /* unknown mask_mode, or FA_MASK_BITMASK with mask == NULL */
  FA_ERR_HIP = 5,           /* the HIP runtime rejected a launch or the workspace allocation */
  /* codes past the five above: */
  FA_ERR_BAD_SCALE = 6,     /* scale is NaN or infinite */
  FA_ERR_WORKSPACE = 7,     /* a caller-supplied workspace is smaller than the call needs or not
                               256-byte aligned */
  FA_ERR_SCRATCH_LIMIT = 8  /* fa_fwd_noalloc: the call needs more than FA_NOALLOC_SCRATCH_BYTES */
} fa_status;

/* Forward attention (see the definition above).  Returns FA_OK once its work is enqueued. */
fa_status fa_fwd(fa_dtype dtype, fa_mask_mode mask_mode, int batch, int n_q_heads,
                 int n_kv_heads, int seq_len, int head_dim, float scale, const void* q,
                 const void* k, const void* v, const uint32_t* mask, void* o, void* stream);

/* Forward attention as fa_fwd, plus the log-sum-exp of each row's kept scaled scores:
 *     lse[b, h, i] = ln sum_{kept j} exp(s_j)      (s_j and "kept" as defined above),
 *     lse[b, h, i] = -inf when row i keeps no key.
 * This is the running softmax state (running max and running sum) that the online softmax
 * carries from tile to tile -- https://yetianai.com/news/16520, section "传统进化搜索的天花板"
 * (FA4's correction step rescales by it) -- returned so that a later pass can rebuild the
 * weights as exp(s_j - lse) without recomputing the row sums.
 *   lse  [batch, n_q_heads, seq_len] float32, DEVICE pointer owned by the caller, 4-byte
 *        aligned, not overlapping q, k, v, mask or o.  Every element is written.
 * Numerics: computed in fp32 from the same rounded weights that normalise O, so its error
 * against the exact value is at most about the relative rounding step of the input dtype
 * (2^-8 for bf16, 2^-11 for fp16).  o, the work enqueued, memory use and errors are as for
 * fa_fwd (o is bitwise the same); lse == NULL is FA_ERR_NULL_PTR, a misaligned lse
 * FA_ERR_UNSUPPORTED. */
fa_status fa_fwd_lse(fa_dtype dtype, fa_mask_mode mask_mode, int batch, int n_q_heads,
                     int n_kv_heads, int seq_len, int head_dim, float scale, const void* q,
                     const void* k, const void* v, const uint32_t* mask, void* o, float* lse,
                     void* stream);

/* The general form: fa_fwd plus four optional arguments.
 *   lse    NULL, or as for fa_fwd_lse.
 *   tiles  NULL, or (FA_MASK_BITMASK only) the per-block summary of `mask` made by
 *          fa_mask_tiles below ([batch, n_q_heads, R, TW] uint32, R = ceil(seq_len / 64),
 *          TW = ceil(R / 32), 4-byte aligned DEVICE pointer, R <= 2048).  Each workgroup
 *          then visits only the 64-key tiles in which some of its rows keep a key, loading no
 *          K or V for the others -- the tile skip of https://yunpan.plus/t/19526-1-1 section
 *          "AI生成的代码质量如何？" excerpt 1, taken before the loads.  The summary must cover
 *          every kept bit of `mask` (fa_mask_tiles' output, or any superset of its set bits):
 *          keys in tiles it marks empty are treated as masked.  With a valid summary the
 *          result equals fa_fwd's (bitwise).
 *   kv_splits  split-KV: 1 = off (fa_fwd's schedule); N in 2..16 = each row tile's key range
 *          is cut into N equal shares computed by separate workgroups, whose running states
 *          (max, row sum, unnormalised O) are combined by a second kernel exactly as the
 *          online softmax combines tiles; 0 = automatic: split (into up to 16 shares of at
 *          least 8 key tiles) only when the grid would fill at most half of the chip.  This
 *          keeps a small grid -- one long sequence with few heads -- from leaving CUs idle.
 *          Splitting changes the summation order, so O and lse then agree with fa_fwd's to the
 *          stated tolerances, not bitwise.  Not combined with tiles.  Workspace: n_splits x
 *          batch x seq_len x n_q_heads x (head_dim + 2) x 4 bytes, stream-ordered from the
 *          same pool as the packed-V buffer (see above); one more kernel is enqueued.
 *   workspace, workspace_bytes  NULL (workspace_bytes ignored): the call takes its device
 *          scratch (packed V, split-KV partials) from the library's pool as described above.
 *          Otherwise a DEVICE buffer owned by the caller, 256-byte aligned, of workspace_bytes
 *          bytes, at least fa_fwd_plan(...).workspace_bytes: the call then uses it and touches
 *          no pool, so it allocates nothing.  Its contents on entry do not matter; the enqueued
 *          work reads and writes it, so it must not be reused or freed before that work has run
 *          and must not be shared by calls that may run at the same time.  When the plan needs
 *          no workspace the buffer is not touched.
 * Errors as for fa_fwd, plus: tiles with another mask mode -> FA_ERR_BAD_MASK_MODE;
 * misaligned lse or tiles, R > 2048, kv_splits outside 0..16, or kv_splits > 1 with tiles
 * -> FA_ERR_UNSUPPORTED; a workspace that is too small or misaligned -> FA_ERR_WORKSPACE
 * (checked with the other arguments, before any HIP call). */
fa_status fa_fwd_ex(fa_dtype dtype, fa_mask_mode mask_mode, int batch, int n_q_heads,
                    int n_kv_heads, int seq_len, int head_dim, float scale, const void* q,
                    const void* k, const void* v, const uint32_t* mask, const uint32_t* tiles,
                    int kv_splits, void* o, float* lse, void* workspace,
                    uint64_t workspace_bytes, void* stream);

/* Device scratch of fa_fwd_noalloc, per GPU: 256 MiB. */
#define FA_NOALLOC_SCRATCH_BYTES (256u << 20)

/* fa_fwd_ex without any allocation, for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc.  Arguments, results and
 * errors are fa_fwd_ex's (no workspace argument); the device scratch the call needs (the
 * plan's workspace_bytes: packed V and split-KV partials) is a static array of
 * FA_NOALLOC_SCRATCH_BYTES in the library's device code, one per GPU it runs on, held until the
 * process ends.  The caller still allocates q, k, v, mask, tiles, o and lse.
 *   - A call whose plan needs more scratch than that returns FA_ERR_SCRATCH_LIMIT before any HIP
 *     call (fa_fwd_plan gives the figure): for example V of more than 256 MiB to pack, or large
 *     automatic split-KV partials.
 *   - The first call on a device resolves that device's array address (one HIP query, no
 *     allocation).  The call never calls hipMalloc, hipFree or an allocating routine.
 *   - Every call on one GPU shares its array, which keeps the previous call's contents (the
 *     kernels write every scratch byte they read, so nothing needs clearing).  Calls whose work
 *     may overlap on one GPU (other streams, other host threads) race on it: order them on one
 *     stream, or use fa_fwd_ex with a workspace per stream. */
fa_status fa_fwd_noalloc(fa_dtype dtype, fa_mask_mode mask_mode, int batch, int n_q_heads,
                         int n_kv_heads, int seq_len, int head_dim, float scale, const void* q,
                         const void* k, const void* v, const uint32_t* mask, const uint32_t* tiles,
                         int kv_splits, void* o, float* lse, void* stream);

/* The launch plan of a call, from its sizes alone (no pointer, no HIP call, no GPU needed): what
 * fa_fwd_ex with these arguments (with_tiles != 0: a tile summary is passed) would enqueue and
 * how much workspace it would take from the pool.  fa_fwd and fa_fwd_lse are kv_splits = 1,
 * with_tiles = 0.  The launches use the same planning code, so plan and call always agree. */
typedef struct {
  int rows_per_workgroup;    /* 128 (4 waves, two workgroups per CU) or 256 (8 waves, one) */
  int packed_v;              /* 1: a pre-pass packs V into transposed tiles first */
  int kv_splits;             /* key-range shares per row tile (1 = no split-KV) */
  int kernels;               /* kernels enqueued: attention, + V pre-pass, + split-KV merge */
  int64_t workgroups;        /* grid of the attention kernel */
  uint64_t workspace_bytes;  /* device scratch the call needs (from the pool, or the caller's
                                workspace in fa_fwd_ex), 0 if none */
} fa_plan;

/* Errors as for fa_fwd_ex's size, mode and kv_splits arguments; plan == NULL ->
 * FA_ERR_NULL_PTR. */
fa_status fa_fwd_plan(fa_dtype dtype, fa_mask_mode mask_mode, int batch, int n_q_heads,
                      int n_kv_heads, int seq_len, int head_dim, int with_tiles, int kv_splits,
                      fa_plan* plan);

/* Packs a byte mask into the layout fa_fwd reads in FA_MASK_BITMASK mode.
 *   mask_bytes [batch, n_heads, seq_len, seq_len] uint8, one byte per (query row, key):
 *              nonzero keeps the score.  Any alignment (16-byte aligned rows load faster).
 *   mask_words [batch, n_heads, seq_len, W] uint32, W = ceil(seq_len / 32), 4-byte aligned:
 *              bit j % 32 of word j / 32 of a row = (byte j != 0), least significant bit
 *              first; the padding bits of the last word (keys >= seq_len) are written as 0.
 * Layout from https://yunpan.plus/t/19526-1-1, section "AI生成的代码质量如何？", excerpt 2.
 * Both are DEVICE pointers owned by the caller and must not overlap.  One kernel is enqueued
 * on `stream`; nothing is allocated.  Errors: NULL pointer -> FA_ERR_NULL_PTR; a size <= 0
 * or a grid past 2^31 blocks -> FA_ERR_BAD_SHAPE; misaligned mask_words ->
 * FA_ERR_UNSUPPORTED; launch failure -> FA_ERR_HIP. */
fa_status fa_pack_mask(int batch, int n_heads, int seq_len, const uint8_t* mask_bytes,
                       uint32_t* mask_words, void* stream);

/* Per-tile summary of a packed mask: which 64 x 64 blocks of (query rows, keys) hold a kept
 * bit -- the tile a kernel may skip outright (same page, excerpt 1: a tile with no set mask
 * bit does no matrix work).
 *   mask_words [batch, n_heads, seq_len, W] uint32 as above (padding bits are ignored).
 *   tiles      [batch, n_heads, R, TW] uint32 with R = ceil(seq_len / 64) row blocks and
 *              TW = ceil(R / 32) words per block: bit t % 32 of word t / 32 of block r is set
 *              iff some kept bit lies in rows [64 r, 64 r + 64) x keys [64 t, 64 t + 64)
 *              (clipped to seq_len); bits for t >= R are 0.
 * DEVICE pointers owned by the caller, 4-byte aligned, not overlapping.  One kernel on
 * `stream`; nothing allocated.  Errors as for fa_pack_mask. */
fa_status fa_mask_tiles(int batch, int n_heads, int seq_len, const uint32_t* mask_words,
                        uint32_t* tiles, void* stream);

/* Static, NUL-terminated description of a status code (never NULL; an unknown code gives
 * "unknown status"). */
const char* fa_status_string(fa_status status);

/* FA_ABI_VERSION of the loaded library. */
int fa_abi_version(void);

/* Measurement hook, for timing the attention kernel apart from the V pre-pass and the split-KV
 * merge (a roofline divides a kernel's own work by its own duration).  `start` and `stop` are
 * hipEvent_t handles, created by the caller and owned by it.  The next fa_fwd, fa_fwd_lse,
 * fa_fwd_ex or fa_fwd_noalloc call made on the calling host thread records `start` on its stream
 * just before the attention kernel is enqueued and `stop` just after it (after the pre-pass,
 * before the merge); hipEventElapsedTime of the pair then gives that kernel's duration.  The
 * pair serves that one call, whatever its outcome: a call that fails validation or fails before
 * the attention kernel records neither, and a later call records nothing unless the hook is set
 * again.  (NULL, NULL) clears it.  Returns FA_ERR_NULL_PTR when exactly one of the two is NULL;
 * the recording's own HIP errors are the call's FA_ERR_HIP.  No HIP call is made here. */
fa_status fa_set_kernel_events(void* start, void* stop);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
