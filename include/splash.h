/*
 * splash.h -- C ABI of the MI355X (gfx950) splash-attention forward library.
 *
 * The operations, as the splash-attention explainer page
 * (explainers.rudrite.com/splash-attention) describes them:
 *
 *  1. A mask compiler (FAQ "What is MaskInfo in splash attention?", "Does
 *     splash attention make every sparse mask faster?", "What does grid
 *     shrinking do in splash attention?"): cut a mask into grid-step blocks,
 *     label each 0 / 1 / 2 (empty / partial / full), build data_next,
 *     mask_next, the deduplicated partial_mask_blocks and q_sequence, shrink
 *     the grid to the longest non-empty block row and downcast the integer
 *     arrays.  A single computable mask (causal, local, chunked causal)
 *     stores no mask data; the kernel recomputes it.
 *
 *  2. The forward kernel (FAQ "What is splash attention and how is it
 *     different from flash attention?"): block-sparse online-softmax
 *     attention whose loop over key/value blocks is read from the MaskInfo.
 *     Label 0 runs nothing and fetches nothing, label 2 skips masking,
 *     label 1 computes and masks.  It also returns the per-row
 *     log-sum-exp residual (the running max and sum that the flash kernel
 *     keeps for its backward pass, pallas-flash-attention-tpu page, FAQ
 *     "What does the TPU flash attention kernel save for the backward
 *     pass?"), and takes the softmax scale and optional logits soft cap of
 *     the EasyDeL BlockSparseAttn.forward_native signature, optionally with
 *     the attention-sink logits (softmax_aux) of that signature.
 *
 *  3. The per-device part of ring attention (explainer FAQ "What does ring
 *     attention add on top of the splash kernel?"): MaskInfo slices along
 *     the key axis for key/value shards, and the log-sum-exp merge of the
 *     shards' results.
 *
 * Conventions
 *  - Every entry point returns a splash_status; on failure a message is
 *    available from splash_last_error() on the same thread.  No C++
 *    exception crosses this boundary.
 *  - Argument errors are reported before anything is launched or allocated.
 *  - Tensors are contiguous row-major, BHSD: q [B, Hq, Sq, D],
 *    k [B, Hkv, Skv, D], v [B, Hkv, Skv, Dv], out [B, Hq, Sq, Dv],
 *    lse [B, Hq, Sq] float32.
 *  - Query head h reads key/value head h / (Hq / Hkv)  (GQA / MQA).
 */
#ifndef SPLASH_H
#define SPLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPLASH_API __attribute__((visibility("default")))

typedef enum splash_status {
  SPLASH_OK = 0,
  SPLASH_EINVAL = 1,       /* bad argument: nothing was launched or allocated      */
  SPLASH_ENOMEM = 2,       /* host or device allocation failed                    */
  SPLASH_EHIP = 3,         /* a HIP runtime call or kernel launch failed          */
  SPLASH_EUNSUPPORTED = 4  /* valid request outside what the kernel is built for  */
} splash_status;

typedef enum splash_mask_kind {
  SPLASH_MASK_CAUSAL = 0,         /* key j allowed for query i iff j <= i                   */
  SPLASH_MASK_LOCAL = 1,          /* i - left <= j <= i + right; a side < 0 is unbounded     */
  SPLASH_MASK_CHUNKED_CAUSAL = 2, /* i / chunk == j / chunk and j <= i                       */
  SPLASH_MASK_DENSE = 3           /* explicit 0/1 bytes, [num_heads, q_len, kv_len]          */
} splash_mask_kind;

typedef enum splash_dtype {
  SPLASH_BF16 = 0, /* q, k, v, out are bfloat16; products in bf16 MFMA, fp32 accumulate  */
  SPLASH_F32 = 1   /* q, k, v, out are float32; fp32 MFMA, no rounding through bf16       */
} splash_dtype;

/* A mask, as the caller describes it.  Positions are plain indices
 * 0..q_len-1 and 0..kv_len-1 (top-left alignment). */
typedef struct splash_mask_desc {
  int32_t kind;          /* a splash_mask_kind                                              */
  int32_t num_heads;     /* DENSE: Hm, 1 (shared by every query head) or Hq; else must be 1 */
  int64_t q_len;         /* Sq >= 0                                                         */
  int64_t kv_len;        /* Skv >= 0                                                        */
  int64_t left;          /* LOCAL: left window, < 0 = unbounded                             */
  int64_t right;         /* LOCAL: right window, < 0 = unbounded                            */
  int64_t chunk;         /* CHUNKED_CAUSAL: chunk length > 0                                */
  const uint8_t *dense;  /* DENSE: HOST bytes [num_heads, q_len, kv_len], nonzero = allowed;
                            borrowed for the duration of the call only                      */
} splash_mask_desc;

/* The compiled mask.  Opaque; owned by the library. */
typedef struct splash_mask_info splash_mask_info;

/* Which array of a MaskInfo a view refers to. */
typedef enum splash_mi_array {
  SPLASH_MI_BLOCK_MASK = 0,     /* [Hm, nq, W] labels 0/1/2                               */
  SPLASH_MI_DATA_NEXT = 1,      /* [Hm, nq, W] key/value block column to fetch            */
  SPLASH_MI_MASK_NEXT = 2,      /* [Hm, nq, W] index into partial blocks (DENSE), or None */
  SPLASH_MI_PARTIAL_BLOCKS = 3, /* [P, bq, bk] uint8 deduplicated mixed blocks, or None   */
  SPLASH_MI_Q_SEQUENCE = 4      /* [Sq] int32 query positions (computable), or None       */
} splash_mi_array;

/* A read-only host view of one MaskInfo array. */
typedef struct splash_array_view {
  int32_t elem_bits;   /* 8, 16 or 32                                                  */
  int32_t is_signed;   /* 1 for the index arrays, 0 for the uint8 partial blocks        */
  int32_t ndim;        /* 1 or 3                                                       */
  int32_t _pad;
  int64_t shape[3];
  const void *data;    /* NULL <=> the array is None                                    */
} splash_array_view;

/* Flags of splash_make_mask_info. */
enum {
  SPLASH_FLAG_SHRINK = 1,   /* shrink the grid to the longest non-empty block row       */
  SPLASH_FLAG_DOWNCAST = 2, /* store each index array as int8/int16 when its max fits   */
  SPLASH_FLAG_DEFAULT = 3
};

/* Compile a mask into a MaskInfo (host work only; nothing touches the GPU).
 *
 * block_q, block_kv: grid-step block (>0, must divide q_len / kv_len).  The
 * forward kernel runs 128 x 128 blocks; other sizes are for inspection.
 * Labels follow any/all per block.  Mixed blocks of a DENSE mask are stored
 * once each, in first-appearance order over (head, row, column) of the
 * unshrunk grid.  Shrink keeps each block row's non-empty columns ascending
 * and pads with label-0 slots at the row end to W = max(1, longest row).
 * data_next at an empty slot holds the next non-empty slot's column in the
 * row, else the previous one's, else 0; mask_next at a non-partial slot holds
 * the next partial slot's index, else the previous one's, else 0.  With
 * SPLASH_FLAG_DOWNCAST each index array is int8 if its max <= 127, else int16
 * if <= 32767, else int32.  q_sequence is int32 arange(q_len) for computable
 * masks.
 *
 * On success *out owns a new MaskInfo; release it with
 * splash_mask_info_destroy().  Errors: SPLASH_EINVAL (NULL pointers, unknown
 * kind, non-dividing blocks, bad window / chunk / head count), SPLASH_ENOMEM. */
SPLASH_API splash_status splash_make_mask_info(const splash_mask_desc *mask, int32_t block_q,
                                               int32_t block_kv, uint32_t flags,
                                               splash_mask_info **out);

/* Host view of one array of a MaskInfo (valid until the MaskInfo is
 * destroyed).  A None array gives data == NULL and ndim == 0.
 * Errors: SPLASH_EINVAL for NULL arguments or an unknown array id. */
SPLASH_API splash_status splash_mask_info_view(const splash_mask_info *mi, int32_t which,
                                               splash_array_view *view);

/* Copy the MaskInfo to the current HIP device (once per device; later calls
 * return at once).  splash_fwd does this itself on first use; calling it
 * ahead keeps the copy out of the first forward call.  Allocates device
 * memory owned by the MaskInfo.  Errors: SPLASH_EINVAL, SPLASH_ENOMEM,
 * SPLASH_EHIP. */
SPLASH_API splash_status splash_mask_info_upload(splash_mask_info *mi);

/* Copy one array of the device copy on the current device back to host
 * memory `dst` of `nbytes` bytes (must equal the array's byte size), so the
 * device MaskInfo can be compared bit for bit with the host one.
 * Synchronous.  Errors: SPLASH_EINVAL (not uploaded to this device, None
 * array, size mismatch), SPLASH_EHIP. */
SPLASH_API splash_status splash_mask_info_read_device(const splash_mask_info *mi, int32_t which,
                                                      void *dst, size_t nbytes);

/* Free a MaskInfo and its device copies.  NULL-safe.  The caller must make
 * sure no kernel that reads it is still running. */
SPLASH_API void splash_mask_info_destroy(splash_mask_info *mi);

/* Splash-attention forward on the current HIP device, asynchronous on
 * hip_stream (a hipStream_t; NULL = the default stream).
 *
 * q, k, v, out: DEVICE pointers, contiguous BHSD in `dtype`.  lse: DEVICE
 * float32 [B, Hq, Sq], or NULL to skip it.  All are owned by the caller and
 * must stay valid until the stream reaches the kernel's end.
 *
 * For every (b, h, i): over the keys j the MaskInfo allows for query i
 * (mask head h if Hm == Hq, else 0),
 *   s_ij = softmax_scale * <q_i, k_j>, capped to c * tanh(s_ij / c) when a
 *   soft cap c is given; out_i = sum_j softmax(s_i)_j v_j and
 *   lse_i = log sum_j exp(s_ij) (natural log).
 * A row with no allowed key gets out_i = 0 and lse_i = -inf.
 * softmax_scale: NaN selects D ** -0.5; otherwise must be finite and > 0.
 * logits_soft_cap: a finite value > 0 turns the cap on; 0, a negative value,
 * NaN or +inf turn it off.
 *
 * Requirements: mi built with 128 x 128 blocks for q_len == Sq and
 * kv_len == Skv; Hm in {1, Hq}; Hq % Hkv == 0; head dims D == Dv in
 * {64, 128}, or any D and Dv that are multiples of 16 from 16 to 128 (the
 * EasyDeL BlockSparseAttn page types head_dim and vhead_dim apart
 * and, on GPU, sends only multiples of 16 to its block-sparse kernel, other
 * dims to plain attention).  Those run zero-padded inside the
 * 64-column kernel (both <= 64) or the 128-column one; rows stay packed at
 * D and Dv elements.
 * The default softmax_scale is D ** -0.5 of the true D.
 * B, Hq or Sq equal to 0 is a no-op.  Validation failures return
 * SPLASH_EINVAL (or SPLASH_EUNSUPPORTED for a head dim / block size the
 * kernel is not built for) before anything runs.  The first call on a device
 * uploads the MaskInfo (see splash_mask_info_upload); later calls allocate
 * nothing.  A launch failure returns SPLASH_EHIP. */
SPLASH_API splash_status splash_fwd(splash_mask_info *mi, const void *q, const void *k,
                                    const void *v, void *out, float *lse, int64_t B, int64_t Hq,
                                    int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D, int64_t Dv,
                                    int32_t dtype, float softmax_scale, float logits_soft_cap,
                                    void *hip_stream);

/* splash_fwd with attention sinks (the softmax_aux argument of the EasyDeL
 * BlockSparseAttn.forward_native signature, typed [num_kv_heads, num_sinks]
 * or [num_sinks]).  The pages name the argument but not its arithmetic; the
 * usual reading is taken: each sink logit a_k is one more softmax column with
 * no value, so for every row
 *   lse_i = log( sum_j exp(s_ij) + sum_k exp(a_k) ),
 *   out_i = sum_j exp(s_ij - lse_i) v_j,
 * with the a_k used as given (no softmax_scale, no soft cap).  A row with no
 * allowed key gets out_i = 0 and lse_i = log sum_k exp(a_k).
 *
 * softmax_aux: DEVICE float32 [aux_heads, num_sinks], row-major, owned by
 * the caller, valid until the kernel ends.  aux_heads == 1 shares one row
 * with every head, aux_heads == Hkv gives query head h the row h / (Hq/Hkv)
 * (the pages' [num_kv_heads, num_sinks]), aux_heads == Hq one row per query
 * head.  Logits must be finite or -inf (a -inf sink adds nothing).
 * num_sinks == 0 (softmax_aux may then be NULL) is exactly splash_fwd.
 * Other arguments, errors and ownership as for splash_fwd; a bad aux_heads,
 * a negative num_sinks or a NULL softmax_aux with num_sinks > 0 returns
 * SPLASH_EINVAL before anything runs. */
SPLASH_API splash_status splash_fwd_sinks(splash_mask_info *mi, const void *q, const void *k,
                                          const void *v, void *out, float *lse, int64_t B,
                                          int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv,
                                          int64_t D, int64_t Dv, int32_t dtype, float softmax_scale,
                                          float logits_soft_cap, const float *softmax_aux,
                                          int32_t aux_heads, int32_t num_sinks, void *hip_stream);

/* Split-key forward: splash_fwd_sinks with each block row's non-empty grid
 * positions divided into kv_splits ranges of about equal count, one
 * workgroup per range, and a second kernel that merges the ranges' results
 * by their log-sum-exp (the rescaling of partial results that ring
 * attention applies across devices, splash-attention explainer, FAQ "What
 * does ring attention add on top of the splash kernel?", applied here
 * across the workgroups of one device).  The result is the same attention;
 * it exists so that grids with fewer block rows than the GPU has workgroup
 * slots -- short sequences, few heads, a small batch -- still fill the
 * machine.
 *
 * kv_splits: 1..8 (1 is exactly splash_fwd_sinks; workspace may then be
 * NULL).  kv_splits > 1 runs bf16 only (float32 returns
 * SPLASH_EUNSUPPORTED).  workspace: DEVICE scratch of at least
 * splash_fwd_workspace_size bytes, 16-byte aligned, overwritten, owned by
 * the caller and valid until the kernels end.  The first call with a given
 * kv_splits on a device uploads that split's table of the MaskInfo (device
 * memory owned by the MaskInfo); later calls allocate nothing.  Other
 * arguments, requirements and errors as splash_fwd_sinks; a bad kv_splits
 * or a missing / small workspace returns SPLASH_EINVAL before anything
 * runs.  Asynchronous on hip_stream. */
SPLASH_API splash_status splash_fwd_split(splash_mask_info *mi, const void *q, const void *k, const void *v,
                                          void *out, float *lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                                          int64_t Skv, int64_t D, int64_t Dv, int32_t dtype, float softmax_scale,
                                          float logits_soft_cap, const float *softmax_aux, int32_t aux_heads,
                                          int32_t num_sinks, int32_t kv_splits, void *workspace,
                                          size_t workspace_bytes, void *hip_stream);

/* Workspace bytes of splash_fwd_split: the ranges' normalised outputs in
 * bf16 and their lses in float32, kv_splits * B * Hq * Sq * (2 * Dv + 4)
 * (0 for kv_splits == 1).
 * Errors: SPLASH_EINVAL for negative sizes, Dv <= 0, kv_splits outside
 * 1..8 or a NULL bytes. */
SPLASH_API splash_status splash_fwd_workspace_size(int64_t B, int64_t Hq, int64_t Sq, int64_t Dv, int32_t kv_splits,
                                                   size_t *bytes);

/* The key-split count the library recommends for this MaskInfo, batch and
 * head count on the current device: 1 when the grid of B * Hq * (block rows)
 * workgroups already fills the GPU's two workgroup slots per compute unit
 * (or for float32), else enough splits to fill them, at most 8 and keeping
 * at least two non-empty 128 x 128 blocks per split on average.  Host work
 * and a device-attribute query only.  Errors: SPLASH_EINVAL (NULL
 * arguments, negative sizes, unknown dtype), SPLASH_EHIP. */
SPLASH_API splash_status splash_fwd_plan(const splash_mask_info *mi, int64_t B, int64_t Hq, int32_t dtype,
                                         int32_t *kv_splits);

/* splash_fwd_split with the workgroup shape chosen by the caller (the block
 * shapes of the Pallas flash-attention page, FAQ "What does block_k_major
 * mean versus block_k in Pallas flash attention?": how much of the problem
 * one kernel instance holds and how each K/V transfer is shared).  A
 * workgroup holds one 128-row block row of heads_per_workgroup query heads:
 *   1  two waves, 128 query rows, two workgroups per compute unit;
 *   2  four waves, the same block row of two heads of one GQA group, which
 *      share their key/value head and their walk, so each K/V stage loaded
 *      into LDS serves 256 query rows; one workgroup per compute unit.
 *      Needs bf16, the 128-column kernel (D == Dv == 128, or padded dims
 *      with max(D, Dv) > 64), a computable mask (causal, local, chunked)
 *      with one mask head, and Hq / Hkv even; else SPLASH_EUNSUPPORTED.
 *   0  the library's choice (splash_fwd_heads_per_workgroup).
 * The result is the same either way, bit for bit (each row's arithmetic is
 * unchanged).  Other arguments, requirements and errors as
 * splash_fwd_split; heads_per_workgroup outside 0..2 returns SPLASH_EINVAL
 * before anything runs.  splash_fwd, splash_fwd_sinks and splash_fwd_split
 * use 0. */
SPLASH_API splash_status splash_fwd_tiled(splash_mask_info *mi, const void *q, const void *k, const void *v,
                                          void *out, float *lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                                          int64_t Skv, int64_t D, int64_t Dv, int32_t dtype, float softmax_scale,
                                          float logits_soft_cap, const float *softmax_aux, int32_t aux_heads,
                                          int32_t num_sinks, int32_t kv_splits, int32_t heads_per_workgroup,
                                          void *workspace, size_t workspace_bytes, void *hip_stream);

/* The heads per workgroup splash_fwd_tiled uses for heads_per_workgroup = 0
 * with Dv == D: 2 where two heads can share a workgroup (see
 * splash_fwd_tiled) and the
 * grid of B * Hq / 2 * (block rows) * kv_splits workgroups still gives 256
 * compute units one each, else 1.  Host work only.  Errors: SPLASH_EINVAL
 * (NULL arguments, negative sizes, Hkv <= 0, unknown dtype, kv_splits
 * outside 1..8). */
SPLASH_API splash_status splash_fwd_heads_per_workgroup(const splash_mask_info *mi, int64_t B, int64_t Hq,
                                                        int64_t Hkv, int64_t D, int32_t dtype, int32_t kv_splits,
                                                        int32_t *heads);

/* Key-axis slice of a mask (ring attention on the splash-attention explainer
 * page, FAQ "What does ring attention add on top of the splash kernel?": the
 * MaskInfo is cut along the key axis to match the key/value shard a device
 * holds).  Builds the MaskInfo of keys [kv_start, kv_start + kv_count) of the
 * mask `mask` describes over all mask->kv_len keys, exactly as
 * splash_make_mask_info would for the mask's columns in that range: its
 * kv_len is kv_count, its block columns are local to the slice, and a
 * computable mask keeps its kind, recomputed in the kernel at the slice's
 * key offset.  A dense mask is read from mask->dense over all kv_len keys.
 * Use it with splash_fwd on the shard's k and v ([B, Hkv, kv_count, D]) and
 * combine the shards' (out, lse) with splash_lse_merge.
 * kv_start and kv_count must be multiples of block_kv with
 * 0 <= kv_start <= kv_start + kv_count <= mask->kv_len (else SPLASH_EINVAL);
 * other arguments, errors and ownership as for splash_make_mask_info. */
SPLASH_API splash_status splash_make_mask_info_kv_slice(const splash_mask_desc *mask, int64_t kv_start,
                                                        int64_t kv_count, int32_t block_q,
                                                        int32_t block_kv, uint32_t flags,
                                                        splash_mask_info **out);

/* Merge two attention results over disjoint key sets into the result over
 * their union (same FAQ: each shard's result carries its own max and sum,
 * combined with flash attention's rescaling):
 *   lse = log(e^lse_a + e^lse_b),  out = e^(lse_a - lse) out_a + e^(lse_b - lse) out_b,
 * per row of `rows` rows of Dv elements.  A part whose lse is -inf adds
 * nothing, whatever its out holds; rows empty in both give out = 0 and
 * lse = -inf.
 *
 * out_a, out_b, out: DEVICE [rows, Dv] in dtype_a / dtype_b / dtype_out
 * (SPLASH_BF16 or SPLASH_F32; a float32 accumulator keeps a chain of merges
 * from rounding at every step), 16-byte aligned.  lse_a, lse_b, lse: DEVICE
 * float32 [rows].  out may be out_a (or out_b) and lse may be lse_a (or
 * lse_b) -- an in-place accumulation -- when the dtypes agree; any other
 * overlap is not allowed.  Dv a multiple of 8 up to 512 (else
 * SPLASH_EUNSUPPORTED).  Asynchronous on hip_stream; allocates
 * nothing.  Errors as for splash_fwd. */
SPLASH_API splash_status splash_lse_merge(const void *out_a, const float *lse_a, int32_t dtype_a,
                                          const void *out_b, const float *lse_b, int32_t dtype_b,
                                          void *out, float *lse, int32_t dtype_out, int64_t rows,
                                          int64_t Dv, void *hip_stream);

/* Backward of splash_fwd (no sinks): the gradients dq, dk, dv of the output
 * for the output gradient dout, as the pallas flash attention page describes
 * the flash backward (FAQ "What does the TPU flash attention kernel save for
 * the backward pass?", "Why does the TPU flash attention backward pass run
 * two kernels instead of one?"): the weights are rebuilt from q, k and the
 * forward's lse, di = <dout_i, out_i> is formed once into `delta`, then a
 * key-major kernel (one workgroup per key block, over the query blocks of
 * every query head of its GQA group that the MaskInfo's transposed block
 * lists give) writes dk and dv, and a query-major kernel (one workgroup per
 * query block, over the MaskInfo row) writes dq.  With s' the scaled (or
 * soft-capped) logit and p_ij = exp(s'_ij - lse_i) on allowed pairs:
 *   dv_j = sum_i p_ij dout_i,  ds_ij = p_ij (<dout_i, v_j> - di_i) g_ij
 *   (g = 1, or 1 - tanh^2 under the cap),  dq_i = scale sum_j ds_ij k_j,
 *   dk_j = scale sum_i ds_ij q_i  (summed over the group's query heads).
 *
 * q, k, v, out, lse: as passed to and returned by splash_fwd for the same
 * MaskInfo, scale and cap (lse is required).  dout: DEVICE [B, Hq, Sq, Dv].
 * dq, dk, dv: DEVICE outputs shaped like q, k, v, fully overwritten (key
 * blocks no query sees get zeros).  delta: DEVICE float32 workspace of
 * B * Hq * Sq elements, overwritten.  All caller-owned, 16-byte aligned
 * (lse and delta 4-byte), valid until the kernels end.  bf16 only (float32
 * returns SPLASH_EUNSUPPORTED); head dims as splash_fwd's bf16 forward (D
 * and Dv other than D == Dv in {64, 128} run zero-padded, dq and dk rows
 * packed at D elements and dv rows at Dv); other requirements as
 * splash_fwd.  The first
 * backward call on a device also uploads the transposed block lists of the
 * MaskInfo; later calls allocate nothing.  Asynchronous on hip_stream. */
SPLASH_API splash_status splash_bwd(splash_mask_info *mi, const void *q, const void *k, const void *v,
                                    const void *out, const float *lse, const void *dout, void *dq, void *dk,
                                    void *dv, float *delta, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                                    int64_t Skv, int64_t D, int64_t Dv, int32_t dtype, float softmax_scale,
                                    float logits_soft_cap, void *hip_stream);

/* Decode: one new query per (batch, query head) against every cached key
 * (q_len = 1).  The EasyDeL block-sparse module switches the causal mask off
 * in decode mode and sends a single query to plain attention on TPU
 * (EasyDeL BlockSparseAttn.forward_native); this entry point is that case on
 * MI355X: splash_fwd's attention with every key allowed,
 *   out_h = sum_j softmax_j(s_hj) v_j,  lse_h = log sum_j exp(s_hj),
 * s_hj = softmax_scale <q_h, k_j> (soft-capped if a cap is given), query head
 * h reading kv head h / (Hq / Hkv).  The keys are split into ranges, each
 * processed for a whole GQA group at once, and the ranges are merged by
 * log-sum-exp.  Range sizes depend on B * Hkv, the group, D and Skv;
 * splash_decode_workspace_size gives the matching scratch size.
 *
 * q: DEVICE bf16 [B, Hq, 1, D]; k, v: DEVICE bf16 [B, Hkv, Skv, D];
 * out: DEVICE bf16 [B, Hq, 1, D]; lse: DEVICE float32 [B, Hq] or NULL;
 * workspace: DEVICE scratch of at least splash_decode_workspace_size bytes,
 * overwritten.  All caller-owned, 16-byte aligned, valid until the kernels
 * end.  bf16 only; D == Dv, in {64, 128} or (run zero-padded inside the
 * 64- or 128-column kernel) another multiple of 16 up to 128, with rows
 * packed at D elements; Hq / Hkv in {1, 2, 4, 8, 16}; Skv >= 1
 * and Skv * D * 2 <= 2^31 - 1 bytes per head (else SPLASH_EUNSUPPORTED).
 * Asynchronous on hip_stream; allocates nothing. */
SPLASH_API splash_status splash_decode_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t Skv,
                                                      int64_t D, size_t *bytes);
SPLASH_API splash_status splash_decode(const void *q, const void *k, const void *v, void *out, float *lse,
                                       void *workspace, size_t workspace_bytes, int64_t B, int64_t Hq,
                                       int64_t Hkv, int64_t Skv, int64_t D, int64_t Dv, int32_t dtype,
                                       float softmax_scale, float logits_soft_cap, void *hip_stream);

/* splash_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels, results and errors as splash_decode, without the
 * workspace: the per-range partials live in a file-scope device array of the
 * library, 16 MiB (16777216 bytes) on each GPU it runs on, held until the
 * process ends; its device address is looked up on the first call on each
 * device.  A call whose partials need more than that (see
 * splash_decode_workspace_size) returns SPLASH_EUNSUPPORTED before anything
 * runs.  The call allocates nothing, on the device or the host.  Every call
 * on one GPU shares that GPU's array, which keeps the last call's partials
 * (no part of it needs to start at zero): calls that overlap on one GPU --
 * on different streams, or from several threads without ordering -- race
 * and give wrong results; calls ordered on one stream are safe. */
SPLASH_API splash_status splash_decode_static(const void *q, const void *k, const void *v, void *out, float *lse,
                                              int64_t B, int64_t Hq, int64_t Hkv, int64_t Skv, int64_t D, int64_t Dv,
                                              int32_t dtype, float softmax_scale, float logits_soft_cap,
                                              void *hip_stream);

/* Message of the last failed call on this thread ("" if none).  The string
 * stays valid until the next library call on this thread. */
SPLASH_API const char *splash_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPLASH_H */
