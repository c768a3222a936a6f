// Internal layout of a compiled MaskInfo (host side plus cached device
// copies).  Shared by the host mask compiler and the C-ABI / launch code.
#pragma once

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "splash.h"

namespace splash {

struct HostArray {
  bool present = false;     // false <=> None
  int32_t elem_bits = 32;   // 8 / 16 / 32
  bool is_signed = true;
  int32_t ndim = 0;
  int64_t shape[3] = {0, 0, 0};
  std::vector<uint8_t> bytes;
  int64_t numel() const {
    int64_t n = 1;
    for (int i = 0; i < ndim; ++i) n *= shape[i];
    return ndim ? n : 0;
  }
};

constexpr int kNumArrays = 5;
constexpr int kMaxDevices = 64;

struct DeviceCopy {
  int device = -1;
  void *ptr[kNumArrays] = {nullptr, nullptr, nullptr, nullptr, nullptr};
  int32_t *row_order = nullptr;
  // Partial mask blocks packed to bits for the bf16 kernel: for block p,
  // 32-key group j and block row i, word [(p * (bk / 32) + j) * bq + i] holds
  // in bit c whether key 32 j + c is allowed.  Null when there are none or
  // the block width is not a multiple of 32.
  uint32_t *mask_bits = nullptr;
  int64_t mask_bits_bytes = 0;
  // Transposed block lists for the key-major backward kernel, made on the
  // first backward call: for mask head hm and key block c, col_n[hm * nk + c]
  // entries col_ent[(hm * nk + c) * col_w + e] = r | label << 30, query block
  // rows in ascending order, and col_mn[...] their partial block (dense).
  // Kernel view of a MaskInfo whose blocks are larger than 128 x 128 (see
  // KernelView); null when the blocks are 128 x 128 and ptr[] serves.
  int32_t *kbm = nullptr, *kdn = nullptr, *kmn = nullptr, *krow_order = nullptr;
  uint8_t *kpmb = nullptr;
  uint32_t *kbits = nullptr;
  int64_t kbits_bytes = 0;
  bool has_cols = false;
  int32_t *col_n = nullptr, *col_ent = nullptr, *col_mn = nullptr;
  int32_t *col_order = nullptr;   // key blocks by descending list length (over mask heads)
  int32_t col_w = 0;
  // The bf16 forward's walk of the MaskInfo.  walk_kv / walk_mn: for every
  // block row of every mask head, in order, the row's non-empty grid
  // positions as data_next | label << 28 and mask_next (dense masks only),
  // int32.  items[S]: per mask head and launch rank (block rows longest
  // first, each followed by its S key splits) eight int32: block row, first
  // walk entry, entry count, and the data_next and mask_next of the first
  // entry (the split's non-empty positions divided into S ranges of about
  // equal count).  items[1] is made at upload, items[S > 1] on the first
  // call with S splits.
  static constexpr int kMaxSplits = 8;
  int32_t *walk_kv = nullptr, *walk_mn = nullptr;
  int32_t *items[kMaxSplits + 1] = {};
};

// A MaskInfo with mask blocks of bq x bk (multiples of 128) as the kernels
// walk it: 128 x 128 sub-blocks.  Every 128-row block row r of parent row
// r / (bq / 128) lists, for each non-empty parent slot in order, its bk / 128
// sub-columns with the parent's label; a partial parent block p gives its
// sub-blocks the indices (p * (bq/128) + i) * (bk/128) + j of the re-cut
// partial blocks.  int32 arrays [Hm, Sq / 128, W * bk / 128].
struct KernelView {
  int64_t nq = 0, nk = 0, width = 0;
  std::vector<int32_t> bm, dn, mn, row_order;
  std::vector<uint8_t> pmb;       // [P', 128, 128]
  std::vector<uint32_t> bits;     // pmb packed as the bf16 kernel reads it
};

}  // namespace splash

struct splash_mask_info {
  int32_t kind = 0;
  int32_t num_heads = 1;  // Hm
  int64_t q_len = 0, kv_len = 0;
  // Key-axis slice: this MaskInfo covers keys [kv_offset, kv_offset + kv_len)
  // of a mask over kv_total keys (0 and kv_len for a whole mask).
  int64_t kv_offset = 0, kv_total = 0;
  int64_t left = -1, right = -1, chunk = 0;
  int32_t block_q = 0, block_kv = 0;
  int64_t nq = 0, nk = 0, width = 0;
  uint32_t flags = 0;
  splash::HostArray arr[splash::kNumArrays];
  // Block rows ordered by descending non-empty block count (summed over mask
  // heads), ties by row index: the launch hands the longest rows out first.
  std::vector<int32_t> row_order;
  std::mutex mu;
  bool has_kview = false;         // built lazily for blocks larger than 128 x 128
  splash::KernelView kview;
  splash::DeviceCopy dev[splash::kMaxDevices];
};

namespace splash {
// Thread-local error message helpers (capi.cpp).
splash_status fail(splash_status st, const std::string &msg);
void clear_error();
}  // namespace splash
