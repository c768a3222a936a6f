// Launch parameters shared by the C-ABI layer and the forward kernel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace splash {

struct FwdParams {
  const void *q, *k, *v;
  void *out;
  float *lse;             // may be null
  int64_t B, Hq, Hkv, Sq, Skv;
  int32_t D;              // the kernel's head dim (64 or 128); == Dv unless padded
  // Padded head dims (bf16 forward): q and k rows hold dk elements and v and
  // out rows dv, each a multiple of 16 up to D; the kernel runs them
  // zero-padded to D columns.  padded = 0: dk == dv == D.
  int32_t dk, dv, padded;
  int32_t group;          // Hq / Hkv
  int32_t nq, width, hm;  // MaskInfo grid: block rows, grid width W, mask heads
  const void *bm, *dn, *mn;           // device MaskInfo index arrays (downcast types)
  const uint8_t *pmb;                 // device partial blocks (dense masks), one byte per element
  const uint32_t *pmb_bits;           // the same packed to 32-key words (see DeviceCopy), or null
  int64_t pmb_bits_bytes;
  const int32_t *q_seq;               // device q_sequence (computable masks)
  const int32_t *row_order;           // device launch order of block rows
  int32_t bm_bytes, dn_bytes, mn_bytes;
  int32_t mask_kind;                  // 0 causal, 1 local, 2 chunked causal, 3 dense
  int64_t left, right, chunk;
  int64_t kv_offset;  // computable masks: global position of local key 0 (key-axis slices)
  float c2;       // no cap: softmax_scale * log2(e); cap: softmax_scale / cap
  float cap_out;  // cap * log2(e)
  int32_t cap;    // soft cap on
  int32_t dense;  // dense mask
  const float *aux;   // device sink logits [aux_heads, num_sinks], or null
  int32_t aux_heads;  // 1 (shared), Hkv (row h / group) or Hq (row h)
  int32_t num_sinks;
  // The bf16 kernels' walk (DeviceCopy::walk_kv / walk_mn / items): each
  // workgroup reads its item -- block row, first walk entry, entry count,
  // first data_next and mask_next -- and then its walk entries.  The
  // backward's dQ kernel walks the same lists (one split).
  const int32_t *walk_kv, *walk_mn, *items;
  // Split keys (bf16 kernel): the non-empty grid positions of each block row
  // are divided into kv_splits ranges of about equal count, one workgroup
  // each.  Each range writes its normalised output to part_o
  // [kv_splits, B, Hq, Sq, Dv] (bf16) and its lse (no sinks) to part_lse
  // [kv_splits, B, Hq, Sq] (float32); a second kernel merges them into out
  // and lse and adds the sinks.
  int32_t kv_splits;          // 1: no split, out and lse written directly
  void *part_o;
  float *part_lse;
  // Two query heads of a GQA group per workgroup (four waves sharing each
  // K/V stage).  Set only for D = 128, computable masks, one mask head and
  // an even group size.
  int32_t head_pairs;
};

// dtype: 0 = bf16, 1 = f32.  D in {64, 128}.  Returns hipGetLastError().
// With p.kv_splits > 1 (bf16 only) it launches the forward and the merge.
hipError_t launch_fwd(const FwdParams &p, int dtype, hipStream_t stream);

// Backward launch parameters (bf16 only).  The forward's walk lists (in `f`)
// drive the query-major dQ kernel; the key-major dK/dV kernel walks the
// transposed lists: for mask head hm and key block c, col_n[hm * nk + c]
// entries col_ent[(hm * nk + c) * col_w + e] = r | label << 30 (query block
// rows in ascending order) with, for dense masks, the partial block index
// col_mn[...] of each.
struct BwdParams {
  FwdParams f;            // q, k, v, out, lse (read), sizes, mask fields, c2 / cap_out / cap
  const void *dout;       // gradient of out, [B, Hq, Sq, Dv]
  float *delta;           // workspace [B, Hq, Sq]: <dout_i, out_i>
  void *dq, *dk, *dv;     // outputs, shaped like q, k, v
  float scale;            // softmax scale (applied to dq and dk)
  int32_t nk;             // key blocks
  const int32_t *col_n, *col_ent, *col_mn;
  const int32_t *col_order;   // key blocks by descending list length (summed over mask heads)
  int32_t col_w;
};

hipError_t launch_bwd(const BwdParams &p, hipStream_t stream);

// Decode (one query per (batch, query head), every key allowed), split into
// 256-key chunks whose partial max / sum / unnormalised output go to the
// workspace and are merged by a second kernel.
struct DecodeParams {
  const void *q, *k, *v;   // q [B, Hq, 1, D], k / v [B, Hkv, Skv, D] (bf16)
  void *out;               // [B, Hq, 1, D] bf16
  float *lse;              // [B, Hq] or null
  int32_t B, Hq, Hkv, group, D;   // D: the kernel's head dim (64 or 128)
  // Padded head dims: q, k, v and out rows hold `dim` elements (a multiple
  // of 16 up to D), run zero-padded to D columns.  padded = 0: dim == D.
  int32_t dim, padded;
  int64_t Skv;
  int32_t n_chunks;        // partial workgroups per (b, kv head)
  int64_t split_keys;      // keys per partial workgroup (the last one may hold fewer)
  float c2, cap_out;       // as FwdParams
  int32_t cap;
  float *ws_o, *ws_m, *ws_l;   // [B * Hkv * n_chunks * group] (x D for ws_o)
};

int64_t decode_split_keys(int64_t units, int64_t group, int64_t D, int64_t Skv);
int64_t decode_chunks(int64_t units, int64_t group, int64_t D, int64_t Skv);
hipError_t launch_decode(const DecodeParams &p, hipStream_t stream);

// The allocation-free decode's scratch: a file-scope device array of this
// many bytes, one per GPU.  decode_static_scratch returns its device address
// on the current device (looked up on the first call per device).
constexpr size_t kDecodeStaticScratchBytes = size_t(16) << 20;
hipError_t decode_static_scratch(void **ptr);

}  // namespace splash
