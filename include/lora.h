/*
 * lora.h -- C ABI of the MI355X (gfx950) multi-LoRA shrink/expand library.
 *
 * What the library computes.  A batch of T tokens carries one adapter slot per
 * token, idx[t] in {-1, 0 .. S-1}.  For every token whose slot s >= 0 and every
 * output slice i (fused projections such as q/k/v or gate/up):
 *
 *     v[i][t][k]            = scale[s] * sum_d A_i[s][k][d] * x[t][d]   (k < r_s)
 *     y[t][off_i + j]      += sum_k B_i[s][j][k] * v[i][t][k]
 *
 * Tokens with idx = -1 are base-model-only and are left untouched.
 *   - One batch mixes LoRA and base-only requests, and adapters of different
 *     ranks up to 64 ("Add multi-LoRA support", Features and Limitations).
 *   - The stacked adapter tensors keep the input dimension contiguous: A_i is
 *     [S][r_max][D] and B_i is [S][out_i][r_max] ("[Hardware][TPU][V1] Better
 *     tpu multilora compilation", the gather baseline in the review thread).
 *   - The intermediate v is fp32, because a half-precision intermediate loses
 *     accuracy ("Add multi-LoRA support", Limitations, on the SGMV kernel).
 *   - v is cleared inside lora_shrink, and only when some token is active
 *     ("[LoRA] LoRA cuda graph specialization", Implementation).
 *
 * Conventions for every entry point:
 *   - Pointers are device memory unless marked [host].  The caller owns every
 *     buffer; the library allocates nothing and keeps no per-call state.
 *   - Calls are asynchronous and stream-ordered on `stream` (a hipStream_t; NULL
 *     means the legacy default stream).  No call synchronises the device,
 *     except where an argument is documented to.
 *   - Arguments are checked on the host before anything is enqueued; on an
 *     error nothing is enqueued and no buffer is written.  lora_last_error()
 *     then returns a description (per thread).
 *   - The library is re-entrant; calls on distinct streams may overlap.
 *   - x, A, B and y of one call share one dtype (all adapters have one dtype,
 *     "Add multi-LoRA support", Limitations).  Arithmetic is fp32 accumulation
 *     of exact products; y is rounded once, to nearest even, into its dtype.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_ABI_VERSION 2

/* Largest supported rank ("Add multi-LoRA support", Limitations). */
#define LORA_MAX_RANK 64
/* Most output slices one call may cover (fused QKV uses 3, gate/up 2). */
#define LORA_MAX_SLICES 8
/* Most adapter slots one batch may index. */
#define LORA_MAX_SLOTS 1024

/* The enums below are 32-bit integers on the ABI.  A caller may pass any
 * int32 value in an enum argument (the library rejects those it does not
 * know); under C++ the enums get int32_t as their underlying type so that
 * such a value is well defined there too. */
#ifdef __cplusplus
#define LORA_ENUM enum : int32_t
#else
#define LORA_ENUM enum
#endif

typedef LORA_ENUM {
  LORA_OK = 0,
  LORA_ERR_INVALID_ARG = 1, /* a null pointer, a negative size, a bad stride */
  LORA_ERR_UNSUPPORTED = 2, /* a valid request outside the documented limits */
  LORA_ERR_INDEX = 3,       /* device-side: some idx outside [-1, S-1] */
  LORA_ERR_HIP = 4          /* the HIP runtime refused a launch or copy */
} lora_status;

typedef LORA_ENUM { LORA_F32 = 0, LORA_F16 = 1, LORA_BF16 = 2 } lora_dtype;

/* How lora_build_segments splits each slot's tokens into kernel work items.
 *   AUTO: slots with at least lora_sgmv_min_tokens() tokens go to the segmented
 *         MFMA path (SGMV) in tiles of 64 tokens; the rest go to the gather
 *         path (BGMV) in groups of at most 16 tokens.  The gather kernel
 *         suits decode-shaped batches and the segmented kernel prefill
 *         ("Add multi-LoRA support", Limitations: the gather kernel is not
 *         efficient for prefill).
 *   BGMV: every slot in groups of at most 16 tokens.
 *   SGMV: every slot in tiles of at most 64 tokens.
 * fp32 data always runs on the gather kernels, whatever the mode. */
typedef LORA_ENUM { LORA_MODE_AUTO = 0, LORA_MODE_BGMV = 1, LORA_MODE_SGMV = 2 } lora_mode;

/* How the rows of one slot's B are stored inside the slot's [out_i][r_max]
 * region of a stacked B_i [S][out_i][r_max] ("Add multi-LoRA support",
 * Features: adapters of different ranks, to be made more performant).
 *   PADDED:    row j of slot s at element j * r_max of the region, columns
 *              k >= r_s being padding.
 *   RANK_ROWS: the rows packed with stride roundup(r_s, 8) (fp16/bf16) or
 *              roundup(r_s, 4) (fp32) elements from the start of the region,
 *              so that a slot of low rank is read without its padding: row j at
 *              element j * roundup(r_s, ...) of the region; what lies past the
 *              packed rows is never read.  Entries between r_s and the rounded
 *              stride are ignored.  lora_copy_padded places an adapter this way
 *              when given that stride as dst_ld (see lora_copy_padded). */
typedef LORA_ENUM { LORA_B_PADDED = 0, LORA_B_RANK_ROWS = 1 } lora_b_layout;

/* ------------------------------------------------------------------------ */
/* Segment record                                                           */
/* ------------------------------------------------------------------------ */
/*
 * lora_build_segments groups the active tokens of a batch by slot, once per
 * batch; every LoRA layer of that batch then reuses the record.  The token
 * indices are built on the host and moved to the device once ("[Hardware]
 * [TPU][V1] Better tpu multilora compilation", review of the token index
 * buffer).
 *
 * The record is one caller-allocated device buffer of lora_segments_bytes(T, S)
 * bytes, 256-byte aligned, laid out as int32 words:
 *
 *   words [0, 16)             info
 *       info[0] num_active    tokens with a valid slot
 *       info[1] num_segments  slots with at least one token
 *       info[2] max_seg_len   largest token count of one slot (0 if none)
 *       info[3] status        LORA_OK, or LORA_ERR_INDEX if some idx was
 *                             outside [-1, S-1]; such tokens are treated as -1
 *       info[4] n_groups      gather work items (see mode)
 *       info[5] n_tiles       segmented work items
 *       info[6] T, info[7] S  the sizes the record was built for
 *       info[8..15]           zero
 *   perm       [T]      at lora_segments_offset(T, S, LORA_SEG_PERM); the first
 *                       num_active entries are the active tokens ordered by slot
 *                       ascending, then token index ascending (stable); the
 *                       remaining T - num_active entries are the other tokens
 *                       (idx -1 or out of range), ascending
 *   seg_slot   [S]      at ..._SEG_SLOT; first num_segments entries: the
 *                       non-empty slots, ascending
 *   seg_start  [S + 1]  at ..._SEG_START; segment g is
 *                       perm[seg_start[g] .. seg_start[g+1]); entry
 *                       num_segments equals num_active
 *   work items          internal to the library (unspecified contents)
 *
 * Entries past the counts are unspecified.  The record is bit-exact and
 * deterministic for a given (idx, S, mode).
 */
typedef LORA_ENUM {
  LORA_SEG_INFO = 0,
  LORA_SEG_PERM = 1,
  LORA_SEG_SLOT = 2,
  LORA_SEG_START = 3,
  LORA_SEG_GROUPS = 4,
  LORA_SEG_TILES = 5
} lora_seg_field;

/* Bytes of the segment record for T tokens and S slots (0 on bad sizes). */
size_t lora_segments_bytes(int32_t T, int32_t S);

/* Offset in int32 words of a field of the record (-1 on bad arguments). */
int64_t lora_segments_offset(int32_t T, int32_t S, lora_seg_field field);

/* Smallest slot token count that AUTO mode sends to the segmented kernels. */
int32_t lora_sgmv_min_tokens(void);

/*
 * Build the segment record of one batch.
 *   idx        [T] int32 device; slot per token, -1 for base-only
 *   T          0 <= T; T = 0 gives an empty record
 *   S          1 <= S <= LORA_MAX_SLOTS
 *   mode       a lora_mode
 *   seg        device record of lora_segments_bytes(T, S) bytes, 256-B aligned
 *   info_host  [host] nullable; pinned host memory of 16 int32.  When given, the
 *              16 info words are copied there asynchronously on `stream`; they
 *              are valid after the stream is synchronised.
 * One kernel; nothing else runs.  Below 512 tokens it is one workgroup;
 * from 512 tokens on (LORA_SEG_WIDE_MIN_T in the environment overrides the
 * threshold) one workgroup per 1024 tokens, which never wait for one another.
 * The record is the same either way.
 */
lora_status lora_build_segments(const int32_t *idx, int32_t T, int32_t S, int32_t mode,
                                void *seg, int32_t *info_host, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Shrink and expand                                                        */
/* ------------------------------------------------------------------------ */
/*
 * Common arguments:
 *   dt          dtype of x, A, B and y
 *   T           tokens in the batch (the same T the record was built for)
 *   n_slices    1 .. LORA_MAX_SLICES
 *   S, r_max    slots and padded rank of the stacked adapters; 1 <= r_max <=
 *               LORA_MAX_RANK and r_max a multiple of 8 (fp16/bf16) or 4 (fp32)
 *   ranks       [S] int32 device, nullable (= r_max for every slot); only rank
 *               rows/columns k < ranks[s] take part; values are clamped to
 *               [0, r_max]
 *   b_layout    (expand calls) a lora_b_layout: how each slot's B rows are
 *               stored in its region
 *   seg         the record lora_build_segments wrote for this batch's idx
 *   active_hint 0 when the caller knows that no token of the batch has a valid
 *               slot: the call then returns LORA_OK having enqueued nothing, so
 *               a base-only batch costs no kernel at all ("[LoRA] LoRA cuda
 *               graph specialization", Purpose and Implementation: the host
 *               picks the no-LoRA path).  Any other value: the kernels run and
 *               read the record's counts on the device, so the result is right
 *               whatever the batch holds.
 * Widths and strides (D, ldx, out_i, off_i, ldy) must be multiples of 8
 * elements for fp16/bf16 and of 4 for fp32, and every base pointer 16-byte
 * aligned; otherwise LORA_ERR_UNSUPPORTED.
 */

/*
 * Shrink: v[i][t][k] = scale[s] * sum_d A_i[s][k][d] * x[t][d].
 *   x        [T][ldx] device, row-major, D <= ldx
 *   A        [host] array of n_slices device pointers, each [S][r_max][D]
 *   scale    [S] fp32 device, nullable (= 1.0)
 *   v        [n_slices][T][r_max] fp32 device, written in full when the call
 *            runs: rows of inactive tokens and columns k >= r_s are 0
 * x ((T - 1) * ldx + D elements) and one slot's A rows (r_max * D elements)
 * must each span less than 4 GiB; otherwise LORA_ERR_UNSUPPORTED.
 */
lora_status lora_shrink(lora_dtype dt, const void *x, int64_t ldx, int32_t T, int32_t D,
                        int32_t n_slices, const void *const *A, int32_t S, int32_t r_max,
                        const int32_t *ranks, const float *scale, const void *seg,
                        int32_t active_hint, float *v, hipStream_t stream);

/*
 * Expand: y[t][off_i + j] += sum_{k < r_s} B_i[s][j][k] * v[i][t][k] for active t.
 *   v              fp32 device; slice i starts at v + i * v_slice_stride, rows of
 *                  r_max floats (v_slice_stride = 0 shares one v by all slices)
 *   B              [host] array of n_slices device pointers, each [S][out_i][r_max]
 *   out_sizes      [host] n_slices widths out_i >= 1
 *   out_offsets    [host] n_slices column offsets; off_i + out_i <= ldy
 *   y              [T][ldy] device, updated in place; rows of inactive tokens and
 *                  columns outside the slices are not read or written
 */
lora_status lora_expand(lora_dtype dt, const float *v, int64_t v_slice_stride, int32_t T,
                        int32_t n_slices, const void *const *B, const int64_t *out_sizes,
                        const int64_t *out_offsets, int32_t S, int32_t r_max,
                        const int32_t *ranks, int32_t b_layout, const void *seg, int32_t active_hint,
                        void *y, int64_t ldy, hipStream_t stream);

/*
 * Shrink then expand of one layer in a single call: the result of lora_shrink
 * followed by lora_expand (with the same b_layout) with v_slice_stride = T * r_max (the shrink and
 * expand of "Add multi-LoRA support", with the fp32 intermediate its
 * Limitations ask for), for decode-shaped batches whose layers are dominated
 * by launch and memory latency rather than by bytes.
 *   x, ldx, D, A, scale          as lora_shrink
 *   B, out_sizes, out_offsets    as lora_expand; y, ldy as lora_expand
 *   v          nullable; [n_slices][T][r_max] fp32 device.  When given it is
 *              written in full, exactly as lora_shrink writes it.
 *   idx        nullable; the batch's [T] int32 slots.  When given, the call
 *              builds the batch's segment record into seg itself, exactly as
 *              lora_build_segments(idx, T, S, LORA_MODE_AUTO, seg) would, and
 *              ignores what seg held: the first LoRA layer of a batch needs no
 *              separate build, and the later layers read the record.  When the
 *              call runs as one launch and S <= 256, every workgroup groups the
 *              tokens by slot itself, in LDS, and one workgroup builds the
 *              record beside the layer; otherwise the build kernel runs first.
 *              Without idx, seg must hold the batch's record.
 *   workspace  device memory of workspace_bytes >=
 *              lora_shrink_expand_workspace_bytes(T, S, n_slices, r_max)
 *              bytes, 256-byte aligned, owned by the caller; pass the same
 *              workspace_bytes with it every time (its layout depends only on
 *              that size).  Clear the whole workspace once after allocating it:
 *              its header and counters must be zero when a call starts, and
 *              every call leaves them zero again, so calls in stream order, of
 *              any shape that fits, can share one workspace.  Calls that may
 *              overlap (other streams) need distinct workspaces.  int32 word 0
 *              counts device-side waits that gave up (0 in every normal run;
 *              when a call raises it, that call's output is invalid; the
 *              counters are still left at zero, so later calls are valid
 *              again and leave the count unchanged).  Each wait gives up after a bounded
 *              number of polls, so a call always ends; the environment
 *              variable LORA_MI355X_FUSED_SPIN_LIMIT, when set, lowers that
 *              bound (for tests of the give-up path).
 * Batches of T <= lora_fused_max_tokens_for(dt) run as one launch (4096
 * tokens for fp16/bf16, 2048 for fp32): producer work units shrink 16-token
 * chunks over ranges of D into the workspace and consumer units expand each
 * chunk once every part of it is there (fp32 chunks on the vector ALUs).
 * Larger batches run as the shrink launch and the expand launch, with v in
 * the workspace when v is NULL.
 * Co-residency.  The one launch's consumers wait for its producers, so it
 * needs every one of its workgroups on the device at once: its grid is what
 * the current device holds at once (rounded down to a multiple of 8), and
 * where that is fewer than 16 workgroups (a partitioned or CU-masked device)
 * the call runs as the separate launches instead.  Kernels running on other
 * streams of the same device while the call runs take compute units the
 * launch counts on: the call then stays correct as long as its producers
 * still get to run within the wait bound, but it is slower, and if a wait
 * gives up the output is invalid (counted in the workspace's word 0, readable
 * with lora_workspace_errors).  Do not overlap a one-launch call with
 * long-running kernels on other streams of its device.
 * Errors and the no-op gate are those of lora_shrink and lora_expand, plus
 * LORA_ERR_INVALID_ARG for a null, misaligned or short workspace.
 */
size_t lora_shrink_expand_workspace_bytes(int32_t T, int32_t S, int32_t n_slices, int32_t r_max);

/* Largest T that lora_shrink_expand runs as one launch (16-bit data). */
int32_t lora_fused_max_tokens(void);

/* The same for data of type dt (0 for an unknown dt). */
int32_t lora_fused_max_tokens_for(lora_dtype dt);

lora_status lora_shrink_expand(lora_dtype dt, const void *x, int64_t ldx, int32_t T, int32_t D,
                               int32_t n_slices, const void *const *A, const void *const *B,
                               const int64_t *out_sizes, const int64_t *out_offsets, int32_t S,
                               int32_t r_max, const int32_t *ranks, int32_t b_layout,
                               const float *scale, const void *seg, const int32_t *idx,
                               int32_t active_hint, float *v, void *y, int64_t ldy, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * Shrink of a LoRA on an embedding table ("Add multi-LoRA support",
 * Features: adapters cover every linear layer and the embeddings, in PEFT
 * format).  For token id w the layer's input is the one-hot vector e_w, so
 * the shrink A_s e_w is column w of the adapter's r x V table A_s.  The
 * tables are stacked transposed, one contiguous rank vector per vocabulary
 * row:
 *     v[t][k] = scale[s] * A_emb[s][tok[t]][k]            (k < r_s)
 * for every token t with a valid slot s = idx[t] and 0 <= tok[t] < V; all
 * other entries of v (rows of base-only tokens, of ids outside the table --
 * such as tokens an adapter adds, which are looked up elsewhere -- and rank
 * columns k >= r_s) are written as 0.  The embedding's delta is then
 * lora_expand with one slice (B_emb [S][H][r_max], out_sizes = {H}) on v.
 *   tok        [T] int32 device token ids
 *   V          rows of the table (e.g. the vocabulary size)
 *   A_emb      [S][V][r_max] device, 16-byte aligned, dtype dt
 *   ranks, scale, active_hint   as lora_shrink
 *   idx        [T] int32 device slots (-1 for base-only); read directly, no
 *              segment record is needed
 *   v          [T][r_max] fp32 device, 16-byte aligned, written in full when
 *              the call runs
 * One launch of T x 16 threads.  Errors: LORA_ERR_INVALID_ARG for a bad size
 * or a null pointer, LORA_ERR_UNSUPPORTED for r_max outside the limits of
 * lora_shrink or misaligned pointers; nothing is enqueued on an error.
 */
lora_status lora_embedding_shrink(lora_dtype dt, const int32_t *tok, int32_t T, int64_t V,
                                  const void *A_emb, int32_t S, int32_t r_max, const int32_t *ranks,
                                  const float *scale, const int32_t *idx, int32_t active_hint, float *v,
                                  hipStream_t stream);

/*
 * Copy an adapter's matrix into its slot of a stacked tensor, zero-padded:
 * the GPU tier of the adapter cache is a fixed number of slots, and adapters
 * of different ranks share them ("Add multi-LoRA support", Features: tiered
 * Disk -> CPU (LRU) -> GPU (fixed number of slots) cache; LoRAs with
 * different ranks).  With M the source matrix (src, [m_rows][m_cols] with row
 * stride src_ld) or, when transpose is non-zero, its transpose (src is then
 * [m_cols][m_rows] with row stride src_ld):
 *     dst[i][j] = (i < m_rows && j < m_cols) ? M[i][j] : 0
 * for i < dst_rows and j < dst_cols, dst having row stride dst_ld.  For a
 * linear layer's slot s: A_i[s] gets the adapter's [r][D] matrix (dst_rows =
 * r_max, dst_cols = D), B_i[s] its [out][r] matrix (dst_cols = r_max); for an
 * embedding the PEFT [r][V] table is copied transposed into A_emb[s]
 * ([V][r_max]).  src and dst are device memory of dtype dt; the copy is
 * stream-ordered.  LORA_ERR_INVALID_ARG for negative sizes, a matrix larger
 * than the slot, a short stride or a null pointer.
 */
lora_status lora_copy_padded(lora_dtype dt, const void *src, int64_t m_rows, int64_t m_cols, int64_t src_ld,
                             int32_t transpose, void *dst, int64_t dst_rows, int64_t dst_cols,
                             int64_t dst_ld, hipStream_t stream);

/*
 * lora_shrink_expand without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments and result as lora_shrink_expand,
 * minus workspace and workspace_bytes; the call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine).
 *   errors_host  [host] nullable; pinned memory of one int32.  When given, the
 *                count of device-side waits that gave up in every call of this
 *                variant on the current device since the process started is
 *                copied there asynchronously after the call's kernels (0 in
 *                every normal run; see the co-residency note above).
 * Scratch.  In place of the workspace the kernels use a device array of
 * LORA_NOALLOC_SCRATCH_BYTES bytes that is part of the library's code object:
 * each device the library runs on holds its own copy until the process ends.
 * Its header and counters are cleared, in stream order, by the first call on
 * each device made outside stream capture (a call under capture records that
 * clearing in the graph); every call leaves its counters at zero again, so
 * later calls need no clearing.  Every call on one device shares that
 * device's scratch: calls that may overlap on one device (other streams, or
 * graphs replayed concurrently) race and must be serialised by the caller.
 * A call whose workspace would exceed LORA_NOALLOC_SCRATCH_BYTES
 * (lora_shrink_expand_workspace_bytes(T, S, n_slices, r_max) > the limit, e.g.
 * prefill batches of many tokens and slices) returns LORA_ERR_UNSUPPORTED
 * and enqueues nothing.  LORA_ERR_HIP if the scratch's device address cannot
 * be obtained.  Other errors and the no-op gate are those of
 * lora_shrink_expand.
 */
#define LORA_NOALLOC_SCRATCH_BYTES (32u << 20)

lora_status lora_shrink_expand_noalloc(lora_dtype dt, const void *x, int64_t ldx, int32_t T, int32_t D,
                                       int32_t n_slices, const void *const *A, const void *const *B,
                                       const int64_t *out_sizes, const int64_t *out_offsets, int32_t S,
                                       int32_t r_max, const int32_t *ranks, int32_t b_layout,
                                       const float *scale, const void *seg, const int32_t *idx,
                                       int32_t active_hint, float *v, void *y, int64_t ldy,
                                       int32_t *errors_host, hipStream_t stream);

/*
 * Mask ("laning") form of lora_shrink_expand, for batches whose adapters
 * stacked have few rank lanes: S * r_max <= 128.  "[Hardware][TPU][V1] Better
 * tpu multilora compilation" reports a masked formulation beating the
 * per-token gather on TPU, and LoRA laning (adapters packed side by side so
 * that one matrix product serves them all) cutting the number of products.
 * Here every 16-token tile of x is multiplied with all L = S * r_max stacked
 * rows of A_i (the tensor [S][r_max][D] read as one [L][D] matrix), each
 * token keeps the lanes of its own slot (times its scale, columns k < r_s),
 * and the expand multiplies all lanes of B with v masked to the token's own
 * lanes.  The result is that of lora_shrink_expand; no segment record is
 * needed (idx is read directly), and every row of x is read whatever its
 * slot (a dense product), while rows of y of tokens without a valid slot (or
 * whose slot has rank 0) are never written.
 *   arguments    as lora_shrink_expand, minus seg, with B in the padded layout
 *   idx          [T] int32 device slots (-1 base-only; out-of-range = base-only)
 *   v            nullable; when given, written in full as lora_shrink writes it
 *   workspace    device, 256-byte aligned, >= lora_mask_workspace_bytes(dt, T,
 *                D, S, n_slices, r_max) bytes: the shrink's fp32 partial sums
 *                (no clearing needed; contents are overwritten)
 * Two launches (the dense shrink in K parts, the masked expand summing the
 * parts in order).  LORA_ERR_UNSUPPORTED when S * r_max > 128; other errors
 * and the no-op gate as lora_shrink_expand.
 */
size_t lora_mask_workspace_bytes(lora_dtype dt, int32_t T, int32_t D, int32_t S, int32_t n_slices,
                                 int32_t r_max);

lora_status lora_shrink_expand_mask(lora_dtype dt, const void *x, int64_t ldx, int32_t T, int32_t D,
                                    int32_t n_slices, const void *const *A, const void *const *B,
                                    const int64_t *out_sizes, const int64_t *out_offsets, int32_t S,
                                    int32_t r_max, const int32_t *ranks, const float *scale,
                                    const int32_t *idx, int32_t active_hint, float *v, void *y,
                                    int64_t ldy, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * Copy the count of waits that gave up (int32 word 0 of a lora_shrink_expand
 * workspace) to host memory, asynchronously on `stream`, after the calls
 * enqueued before it on that stream.
 *   workspace  the device workspace, 256-byte aligned
 *   host_out   [host] pinned memory of one int32; valid once the stream is
 *              synchronised.  0 means every call on the workspace since it was
 *              cleared produced valid output.
 * LORA_ERR_INVALID_ARG for a null or misaligned pointer; LORA_ERR_HIP if the
 * copy cannot be enqueued.
 */
lora_status lora_workspace_errors(const void *workspace, int32_t *host_out, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Diagnostics                                                              */
/* ------------------------------------------------------------------------ */

/* Static name of a status code. */
const char *lora_status_string(lora_status s);

/* Description of the last error on the calling thread ("" if none). */
const char *lora_last_error(void);

/* LORA_ABI_VERSION of the built library. */
int32_t lora_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_H */
