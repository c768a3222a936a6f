// C-ABI layer: errors, device copies of a MaskInfo, validation and launch of
// the forward kernel.  Declarations and contracts are in include/splash.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <initializer_list>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "mask_info.h"
#include "splash_kernel.h"
#include "lse_merge.h"

namespace splash {

namespace {
thread_local std::string g_last_error;

size_t array_bytes(const HostArray &a) { return a.bytes.size(); }
}  // namespace

splash_status fail(splash_status st, const std::string &msg) {
  g_last_error = msg;
  return st;
}
void clear_error() { g_last_error.clear(); }

namespace {

splash_status hip_fail(hipError_t e, const char *what) {
  return fail(e == hipErrorOutOfMemory ? SPLASH_ENOMEM : SPLASH_EHIP,
              std::string(what) + ": " + hipGetErrorString(e));
}

void free_copy(DeviceCopy &dc) {
  if (dc.device < 0) return;
  int prev = -1;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(dc.device);
  for (void *&ptr : dc.ptr) {
    if (ptr) (void)hipFree(ptr);
    ptr = nullptr;
  }
  if (dc.row_order) (void)hipFree(dc.row_order);
  dc.row_order = nullptr;
  if (dc.mask_bits) (void)hipFree(dc.mask_bits);
  dc.mask_bits = nullptr;
  dc.mask_bits_bytes = 0;
  for (int32_t **c : {&dc.kbm, &dc.kdn, &dc.kmn, &dc.krow_order}) {
    if (*c) (void)hipFree(*c);
    *c = nullptr;
  }
  if (dc.kpmb) (void)hipFree(dc.kpmb);
  dc.kpmb = nullptr;
  if (dc.kbits) (void)hipFree(dc.kbits);
  dc.kbits = nullptr;
  dc.kbits_bytes = 0;
  for (int32_t **c : {&dc.col_n, &dc.col_ent, &dc.col_mn, &dc.col_order}) {
    if (*c) (void)hipFree(*c);
    *c = nullptr;
  }
  dc.has_cols = false;
  dc.col_w = 0;
  for (int32_t **t : {&dc.walk_kv, &dc.walk_mn}) {
    if (*t) (void)hipFree(*t);
    *t = nullptr;
  }
  for (int32_t *&t : dc.items) {
    if (t) (void)hipFree(t);
    t = nullptr;
  }
  dc.device = -1;
  if (prev >= 0) (void)hipSetDevice(prev);
}

// Partial blocks [P, bq, bk] (one byte per element) packed to 32-key words:
// word [(p * (bk / 32) + j) * bq + i], bit c <=> element (i, 32 j + c) != 0.
std::vector<uint32_t> pack_bits(const uint8_t *data, int64_t P, int64_t bq, int64_t bk) {
  const int64_t groups = bk / 32;
  std::vector<uint32_t> bits(static_cast<size_t>(P * groups * bq), 0u);
  for (int64_t b = 0; b < P; ++b)
    for (int64_t i = 0; i < bq; ++i) {
      const uint8_t *row = data + (b * bq + i) * bk;
      for (int64_t j = 0; j < groups; ++j) {
        uint32_t w = 0;
        for (int c = 0; c < 32; ++c) w |= (row[32 * j + c] != 0 ? 1u : 0u) << c;
        bits[static_cast<size_t>((b * groups + j) * bq + i)] = w;
      }
    }
  return bits;
}
std::vector<uint32_t> pack_mask_bits(const HostArray &pm) {
  return pack_bits(pm.bytes.data(), pm.shape[0], pm.shape[1], pm.shape[2]);
}

int64_t host_index(const HostArray &a, int64_t i);

// The 128 x 128 kernel view of a MaskInfo with larger blocks (KernelView).
void build_kview(splash_mask_info *mi) {
  KernelView &kv = mi->kview;
  const int64_t hm = mi->num_heads, W = mi->width;
  const int64_t fq = mi->block_q / 128, fk = mi->block_kv / 128;
  kv.nq = mi->q_len / 128;
  kv.nk = mi->kv_len / 128;
  kv.width = std::max<int64_t>(1, W * fk);
  const HostArray &bm = mi->arr[SPLASH_MI_BLOCK_MASK], &dn = mi->arr[SPLASH_MI_DATA_NEXT];
  const HostArray &mn = mi->arr[SPLASH_MI_MASK_NEXT], &pm = mi->arr[SPLASH_MI_PARTIAL_BLOCKS];
  const size_t n = static_cast<size_t>(hm * kv.nq * kv.width);
  kv.bm.assign(n, 0);
  kv.dn.assign(n, 0);
  kv.mn.assign(n, 0);
  std::vector<int64_t> work(static_cast<size_t>(std::max<int64_t>(kv.nq, 1)), 0);
  for (int64_t h = 0; h < hm; ++h)
    for (int64_t r = 0; r < kv.nq; ++r) {
      const int64_t R = r / fq, i = r % fq;
      int64_t out = 0;
      for (int64_t sl = 0; sl < W; ++sl) {
        const int64_t at = (h * mi->nq + R) * W + sl;
        const int64_t label = host_index(bm, at);
        if (label <= 0) continue;
        const int64_t c = host_index(dn, at);
        const int64_t p = (label == 1 && mn.present) ? host_index(mn, at) : 0;
        for (int64_t j = 0; j < fk; ++j, ++out) {
          const size_t o = static_cast<size_t>((h * kv.nq + r) * kv.width + out);
          kv.bm[o] = static_cast<int32_t>(label);
          kv.dn[o] = static_cast<int32_t>(c * fk + j);
          kv.mn[o] = static_cast<int32_t>(label == 1 ? (p * fq + i) * fk + j : 0);
        }
      }
      work[r] += out;
    }
  kv.row_order.resize(static_cast<size_t>(kv.nq));
  for (int64_t r = 0; r < kv.nq; ++r) kv.row_order[r] = static_cast<int32_t>(r);
  std::stable_sort(kv.row_order.begin(), kv.row_order.end(),
                   [&](int32_t a, int32_t b) { return work[a] > work[b]; });
  kv.pmb.clear();
  kv.bits.clear();
  if (pm.present && pm.ndim == 3 && pm.shape[0] > 0) {
    const int64_t P = pm.shape[0], bq = pm.shape[1], bk = pm.shape[2];
    const int64_t Psub = P * fq * fk;
    kv.pmb.assign(static_cast<size_t>(Psub * 128 * 128), 0);
    for (int64_t p = 0; p < P; ++p)
      for (int64_t i = 0; i < fq; ++i)
        for (int64_t j = 0; j < fk; ++j) {
          uint8_t *dst = kv.pmb.data() + ((p * fq + i) * fk + j) * 128 * 128;
          for (int64_t row = 0; row < 128; ++row)
            std::memcpy(dst + row * 128, pm.bytes.data() + (p * bq + i * 128 + row) * bk + j * 128, 128);
        }
    kv.bits = pack_bits(kv.pmb.data(), Psub, 128, 128);
  }
  mi->has_kview = true;
}

template <typename T>
hipError_t upload_vec(const std::vector<T> &v, T **dst) {
  const size_t nb = std::max<size_t>(v.size(), 1) * sizeof(T);
  hipError_t e = hipMalloc(reinterpret_cast<void **>(dst), nb);
  if (e == hipSuccess && !v.empty()) e = hipMemcpy(*dst, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice);
  return e;
}

// Grid geometry the forward kernels walk: the MaskInfo's own, or its kernel
// view for blocks larger than 128 x 128.
struct Walk {
  int64_t nq, width;
  bool view;
};
Walk walk_of(const splash_mask_info *mi) {
  if (mi->block_q != 128 || mi->block_kv != 128) return {mi->q_len / 128, std::max<int64_t>(1, mi->width * (mi->block_kv / 128)), true};
  return {mi->nq, mi->width, false};
}

// The non-empty grid positions of every block row of the walk geometry, in
// order: (data_next, label, mask_next) and each row's first entry.
struct WalkLists {
  std::vector<int32_t> kv, mn;      // kv: data_next | label << 28
  std::vector<int64_t> row_off;     // [Hm * nq + 1]
};
WalkLists build_walk(const splash_mask_info *mi) {
  const Walk wk = walk_of(mi);
  const int64_t hm = mi->num_heads;
  const HostArray &bm = mi->arr[SPLASH_MI_BLOCK_MASK], &dn = mi->arr[SPLASH_MI_DATA_NEXT];
  const HostArray &mn = mi->arr[SPLASH_MI_MASK_NEXT];
  WalkLists w;
  w.row_off.assign(static_cast<size_t>(hm * wk.nq + 1), 0);
  for (int64_t h = 0; h < hm; ++h)
    for (int64_t r = 0; r < wk.nq; ++r) {
      for (int64_t sl = 0; sl < wk.width; ++sl) {
        const int64_t at = (h * wk.nq + r) * wk.width + sl;
        const int64_t label = wk.view ? mi->kview.bm[at] : host_index(bm, at);
        if (label <= 0) continue;
        const int64_t c = wk.view ? mi->kview.dn[at] : host_index(dn, at);
        const int64_t m = wk.view ? mi->kview.mn[at] : (mn.present ? host_index(mn, at) : 0);
        w.kv.push_back(static_cast<int32_t>(c | (label << 28)));
        w.mn.push_back(static_cast<int32_t>(label == 1 ? m : 0));
      }
      w.row_off[h * wk.nq + r + 1] = static_cast<int64_t>(w.kv.size());
    }
  return w;
}

// The item table for S key splits (see DeviceCopy::items), uploaded to the
// device copy `dc`.  Called under the MaskInfo's lock, after the device copy
// (and the kernel view, if any) exists.
splash_status ensure_items(splash_mask_info *mi, DeviceCopy &dc, int S, const WalkLists *lists = nullptr) {
  if (dc.items[S]) return SPLASH_OK;
  WalkLists own;
  if (!lists) {
    own = build_walk(mi);
    lists = &own;
  }
  const Walk wk = walk_of(mi);
  const int64_t hm = mi->num_heads;
  const std::vector<int32_t> &order = wk.view ? mi->kview.row_order : mi->row_order;
  std::vector<int32_t> table(static_cast<size_t>(std::max<int64_t>(1, hm * wk.nq * S) * 8), 0);
  for (int64_t h = 0; h < hm; ++h)
    for (int64_t i = 0; i < wk.nq; ++i) {
      const int64_t r = order.empty() ? i : order[static_cast<size_t>(i)];
      const int64_t r0 = lists->row_off[h * wk.nq + r], n = lists->row_off[h * wk.nq + r + 1] - r0;
      for (int s = 0; s < S; ++s) {
        const int64_t a = n * s / S, e = n * (s + 1) / S;
        int32_t *it = table.data() + ((h * wk.nq + i) * S + s) * 8;
        it[0] = static_cast<int32_t>(r);
        it[1] = static_cast<int32_t>(r0 + a);
        it[2] = static_cast<int32_t>(e - a);
        // first block of the range, or of the row, or block 0: the prologue
        // starts its loads there, so it must name a real block
        const int64_t f = a < n ? r0 + a : (n > 0 ? r0 : -1);
        it[3] = f >= 0 ? (lists->kv[static_cast<size_t>(f)] & 0x0fffffff) : 0;
        it[4] = f >= 0 ? lists->mn[static_cast<size_t>(f)] : 0;
      }
    }
  int32_t *d = nullptr;
  hipError_t e = upload_vec(table, &d);
  if (e != hipSuccess) {
    if (d) (void)hipFree(d);
    return hip_fail(e, "uploading the forward's item table");
  }
  dc.items[S] = d;
  return SPLASH_OK;
}

// Device copy for the current device, uploading it if needed.
splash_status ensure_device_copy(splash_mask_info *mi, DeviceCopy **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SPLASH_EUNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(mi->mu);
  DeviceCopy &dc = mi->dev[dev];
  if (dc.device == dev) {
    *out = &dc;
    return SPLASH_OK;
  }
  DeviceCopy fresh;
  fresh.device = dev;
  for (int i = 0; i < kNumArrays; ++i) {
    const HostArray &a = mi->arr[i];
    if (!a.present || a.bytes.empty()) continue;
    e = hipMalloc(&fresh.ptr[i], array_bytes(a));
    if (e == hipSuccess) e = hipMemcpy(fresh.ptr[i], a.bytes.data(), array_bytes(a), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      free_copy(fresh);
      return hip_fail(e, "uploading MaskInfo");
    }
  }
  if (!mi->row_order.empty()) {
    const size_t nb = mi->row_order.size() * sizeof(int32_t);
    e = hipMalloc(reinterpret_cast<void **>(&fresh.row_order), nb);
    if (e == hipSuccess) e = hipMemcpy(fresh.row_order, mi->row_order.data(), nb, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      free_copy(fresh);
      return hip_fail(e, "uploading MaskInfo row order");
    }
  }
  const HostArray &pm = mi->arr[SPLASH_MI_PARTIAL_BLOCKS];
  if (pm.present && pm.ndim == 3 && pm.shape[0] > 0 && pm.shape[2] % 32 == 0) {
    const std::vector<uint32_t> bits = pack_mask_bits(pm);
    const size_t nb = bits.size() * sizeof(uint32_t);
    e = hipMalloc(reinterpret_cast<void **>(&fresh.mask_bits), nb);
    if (e == hipSuccess) e = hipMemcpy(fresh.mask_bits, bits.data(), nb, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      free_copy(fresh);
      return hip_fail(e, "uploading packed mask blocks");
    }
    fresh.mask_bits_bytes = static_cast<int64_t>(nb);
  }
  if (mi->block_q != 128 || mi->block_kv != 128) {
    try {
      if (!mi->has_kview) build_kview(mi);
    } catch (const std::bad_alloc &) {
      free_copy(fresh);
      return fail(SPLASH_ENOMEM, "out of host memory for the kernel view");
    }
    const KernelView &kv = mi->kview;
    e = upload_vec(kv.bm, &fresh.kbm);
    if (e == hipSuccess) e = upload_vec(kv.dn, &fresh.kdn);
    if (e == hipSuccess) e = upload_vec(kv.mn, &fresh.kmn);
    if (e == hipSuccess) e = upload_vec(kv.row_order, &fresh.krow_order);
    if (e == hipSuccess && !kv.pmb.empty()) e = upload_vec(kv.pmb, &fresh.kpmb);
    if (e == hipSuccess && !kv.bits.empty()) e = upload_vec(kv.bits, &fresh.kbits);
    if (e != hipSuccess) {
      free_copy(fresh);
      return hip_fail(e, "uploading the kernel view");
    }
    fresh.kbits_bytes = static_cast<int64_t>(kv.bits.size() * sizeof(uint32_t));
  }
  {
    WalkLists lists;
    try {
      lists = build_walk(mi);
    } catch (const std::bad_alloc &) {
      free_copy(fresh);
      return fail(SPLASH_ENOMEM, "out of host memory for the forward's walk lists");
    }
    e = upload_vec(lists.kv, &fresh.walk_kv);
    if (e == hipSuccess && mi->kind == SPLASH_MASK_DENSE) e = upload_vec(lists.mn, &fresh.walk_mn);
    if (e != hipSuccess) {
      free_copy(fresh);
      return hip_fail(e, "uploading the forward's walk lists");
    }
    const splash_status st = ensure_items(mi, fresh, 1, &lists);
    if (st != SPLASH_OK) {
      free_copy(fresh);
      return st;
    }
  }
  dc = fresh;
  *out = &dc;
  return SPLASH_OK;
}

int64_t host_index(const HostArray &a, int64_t i) {
  const uint8_t *p = a.bytes.data();
  if (a.elem_bits == 8) return static_cast<int8_t>(p[i]);
  if (a.elem_bits == 16) {
    int16_t x;
    std::memcpy(&x, p + 2 * i, 2);
    return x;
  }
  int32_t x;
  std::memcpy(&x, p + 4 * i, 4);
  return x;
}

// The transposed block lists of the backward's key-major kernel, on the
// device copy `dc` (already uploaded).  Called under the MaskInfo's lock.
splash_status ensure_cols(splash_mask_info *mi, DeviceCopy &dc) {
  if (dc.has_cols) return SPLASH_OK;
  const bool view = mi->has_kview;   // blocks larger than 128 x 128: walk the kernel view
  const int64_t hm = mi->num_heads;
  const int64_t nq = view ? mi->kview.nq : mi->nq, nk = view ? mi->kview.nk : mi->nk;
  const int64_t W = view ? mi->kview.width : mi->width;
  const HostArray &bm = mi->arr[SPLASH_MI_BLOCK_MASK], &dn = mi->arr[SPLASH_MI_DATA_NEXT];
  const HostArray &mn = mi->arr[SPLASH_MI_MASK_NEXT];
  std::vector<std::vector<int32_t>> ent(static_cast<size_t>(hm * nk)), pm(static_cast<size_t>(hm * nk));
  for (int64_t h = 0; h < hm; ++h)
    for (int64_t r = 0; r < nq; ++r)
      for (int64_t s = 0; s < W; ++s) {
        const int64_t at = (h * nq + r) * W + s;
        const int64_t label = view ? mi->kview.bm[at] : host_index(bm, at);
        if (label <= 0) continue;
        const int64_t c = view ? mi->kview.dn[at] : host_index(dn, at);
        ent[h * nk + c].push_back(static_cast<int32_t>(r | (label << 30)));
        pm[h * nk + c].push_back(view ? mi->kview.mn[at]
                                      : (mn.present ? static_cast<int32_t>(host_index(mn, at)) : 0));
      }
  int64_t w = 1;
  for (const auto &e : ent) w = std::max<int64_t>(w, static_cast<int64_t>(e.size()));
  std::vector<int32_t> n(static_cast<size_t>(std::max<int64_t>(hm * nk, 1)), 0);
  std::vector<int32_t> flat(static_cast<size_t>(std::max<int64_t>(hm * nk, 1) * w), 0), flat_mn(flat.size(), 0);
  for (int64_t i = 0; i < hm * nk; ++i) {
    n[i] = static_cast<int32_t>(ent[i].size());
    for (size_t e = 0; e < ent[i].size(); ++e) {
      flat[i * w + e] = ent[i][e];
      flat_mn[i * w + e] = pm[i][e];
    }
  }
  // Launch order of the key-major kernel: longest lists first.
  std::vector<int64_t> work(static_cast<size_t>(std::max<int64_t>(nk, 1)), 0);
  for (int64_t h = 0; h < hm; ++h)
    for (int64_t c = 0; c < nk; ++c) work[c] += static_cast<int64_t>(ent[h * nk + c].size());
  std::vector<int32_t> order(static_cast<size_t>(std::max<int64_t>(nk, 1)), 0);
  for (int64_t c = 0; c < nk; ++c) order[c] = static_cast<int32_t>(c);
  std::stable_sort(order.begin(), order.begin() + nk, [&](int32_t a, int32_t b2) { return work[a] > work[b2]; });
  hipError_t e = hipSuccess;
  int32_t **dst[4] = {&dc.col_n, &dc.col_ent, &dc.col_mn, &dc.col_order};
  const std::vector<int32_t> *src[4] = {&n, &flat, &flat_mn, &order};
  for (int i = 0; i < 4 && e == hipSuccess; ++i) {
    const size_t nb = src[i]->size() * sizeof(int32_t);
    e = hipMalloc(reinterpret_cast<void **>(dst[i]), nb);
    if (e == hipSuccess) e = hipMemcpy(*dst[i], src[i]->data(), nb, hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) {
    for (int i = 0; i < 4; ++i) {
      if (*dst[i]) (void)hipFree(*dst[i]);
      *dst[i] = nullptr;
    }
    return hip_fail(e, "uploading the transposed block lists");
  }
  dc.col_w = static_cast<int32_t>(w);
  dc.has_cols = true;
  return SPLASH_OK;
}


}  // namespace
}  // namespace splash

using namespace splash;

extern "C" SPLASH_API const char *splash_last_error(void) { return g_last_error.c_str(); }

extern "C" SPLASH_API void splash_mask_info_destroy(splash_mask_info *mi) {
  if (!mi) return;
  for (DeviceCopy &dc : mi->dev) free_copy(dc);
  delete mi;
}

extern "C" SPLASH_API splash_status splash_mask_info_upload(splash_mask_info *mi) {
  clear_error();
  if (!mi) return fail(SPLASH_EINVAL, "MaskInfo is NULL");
  DeviceCopy *dc = nullptr;
  return ensure_device_copy(mi, &dc);
}

extern "C" SPLASH_API splash_status splash_mask_info_read_device(const splash_mask_info *mi,
                                                                 int32_t which, void *dst,
                                                                 size_t nbytes) {
  clear_error();
  if (!mi || !dst) return fail(SPLASH_EINVAL, "NULL argument");
  if (which < 0 || which >= kNumArrays) return fail(SPLASH_EINVAL, "unknown MaskInfo array id");
  const HostArray &a = mi->arr[which];
  if (!a.present) return fail(SPLASH_EINVAL, "array is None");
  if (nbytes != a.bytes.size()) return fail(SPLASH_EINVAL, "nbytes does not match the array size");
  if (nbytes == 0) return SPLASH_OK;
  bool any_copy = false;
  for (const DeviceCopy &dc : mi->dev) any_copy = any_copy || dc.device >= 0;
  if (!any_copy) return fail(SPLASH_EINVAL, "MaskInfo has not been uploaded to any device");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices || mi->dev[dev].device != dev || !mi->dev[dev].ptr[which])
    return fail(SPLASH_EINVAL, "MaskInfo is not uploaded to the current device");
  e = hipMemcpy(dst, mi->dev[dev].ptr[which], nbytes, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "reading the device MaskInfo");
  return SPLASH_OK;
}

namespace {

// Largest byte count one buffer resource (32-bit size field) covers.
constexpr int64_t kMaxHeadBytes = 0x7fffffffLL;

// Head dims the bf16 forward runs zero-padded inside its 64- or 128-column
// kernel: D and Dv multiples of 16 up to 128.  (The EasyDeL BlockSparseAttn
// page types the key and value head dims apart, and on GPU sends only dims
// that are multiples of 16 to its block-sparse kernel.)
bool padded_dims_ok(int64_t D, int64_t Dv) {
  return D % 16 == 0 && Dv % 16 == 0 && D >= 16 && Dv >= 16 && D <= 128 && Dv <= 128;
}
bool native_dims(int64_t D, int64_t Dv) { return D == Dv && (D == 64 || D == 128); }
int64_t padded_kernel_dim(int64_t D, int64_t Dv) { return std::max(D, Dv) <= 64 ? 64 : 128; }

// Checks shared by the forward and the backward entry points.

splash_status validate_call(const splash_mask_info *mi, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                            int64_t Skv, int64_t D, int64_t Dv, int32_t dtype, float softmax_scale,
                            bool padded_ok = false) {
  if (!mi) return fail(SPLASH_EINVAL, "MaskInfo is NULL");
  if (B < 0 || Hq < 0 || Hkv < 0 || Sq < 0 || Skv < 0 || D <= 0 || Dv <= 0)
    return fail(SPLASH_EINVAL, "negative size or non-positive head dim");
  if (dtype != SPLASH_BF16 && dtype != SPLASH_F32) return fail(SPLASH_EINVAL, "unknown dtype");
  if (Sq != mi->q_len || Skv != mi->kv_len)
    return fail(SPLASH_EINVAL, "Sq / Skv do not match the MaskInfo's q_len / kv_len");
  if (Hkv == 0 && Hq > 0) return fail(SPLASH_EINVAL, "Hkv must be positive");
  if (Hkv > 0 && Hq % Hkv != 0) return fail(SPLASH_EINVAL, "Hq must be a multiple of Hkv");
  if (mi->num_heads != 1 && mi->num_heads != Hq)
    return fail(SPLASH_EINVAL, "MaskInfo head count must be 1 or Hq");
  if (!(std::isnan(softmax_scale) || (std::isfinite(softmax_scale) && softmax_scale > 0.f)))
    return fail(SPLASH_EINVAL, "softmax_scale must be NaN (default) or finite and > 0");
  if (mi->block_q % 128 || mi->block_kv % 128)
    return fail(SPLASH_EUNSUPPORTED, "the kernels run MaskInfo blocks that are multiples of 128 x 128");
  if (!native_dims(D, Dv)) {
    if (!padded_ok) return fail(SPLASH_EUNSUPPORTED, "head dims must satisfy D == Dv in {64, 128}");
    if (!padded_dims_ok(D, Dv))
      return fail(SPLASH_EUNSUPPORTED, "head dims must be D == Dv in {64, 128} or multiples of 16 up to 128");
  }
  const int64_t n_wg = B * Hq * (Sq / 128);
  if (n_wg > 0x7fffffffLL || B * Hq > 0x7fffffffLL || B * Hkv * (Skv / 128) > 0x7fffffffLL)
    return fail(SPLASH_EUNSUPPORTED, "grid too large");
  // The kernels address one head's q, k, v, out (and dout) through buffer
  // resources whose size field and stage offsets are 32-bit: a head larger
  // than 2^31 - 1 bytes would read zeros past that point instead of its data.
  const int64_t esize = dtype == SPLASH_BF16 ? 2 : 4;
  if (Skv * D * esize > kMaxHeadBytes || Skv * Dv * esize > kMaxHeadBytes || Sq * D * esize > kMaxHeadBytes ||
      Sq * Dv * esize > kMaxHeadBytes)
    return fail(SPLASH_EUNSUPPORTED, "one head of q, k, v or out exceeds 2^31 - 1 bytes");
  // Dense masks: the partial blocks, packed to one bit per element, are read
  // through one buffer resource as well.
  const HostArray &pm = mi->arr[SPLASH_MI_PARTIAL_BLOCKS];
  if (pm.present && pm.ndim == 3 && pm.shape[0] * pm.shape[1] * pm.shape[2] / 8 > kMaxHeadBytes)
    return fail(SPLASH_EUNSUPPORTED, "the packed partial mask blocks exceed 2^31 - 1 bytes");
  return SPLASH_OK;
}

bool aligned16(std::initializer_list<const void *> ptrs) {
  uintptr_t acc = 0;
  for (const void *p : ptrs) acc |= reinterpret_cast<uintptr_t>(p);
  return acc % 16 == 0;
}

FwdParams make_params(const splash_mask_info *mi, const DeviceCopy *dc, const void *q, const void *k,
                      const void *v, void *out, float *lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq,
                      int64_t Skv, int64_t D, float scale, float logits_soft_cap) {
  FwdParams p{};
  p.kv_splits = 1;
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Skv = Skv;
  p.D = static_cast<int32_t>(D);
  p.dk = p.dv = static_cast<int32_t>(D);
  p.padded = 0;
  p.group = static_cast<int32_t>(Hq / Hkv);
  p.nq = static_cast<int32_t>(mi->nq);
  p.width = static_cast<int32_t>(mi->width);
  p.hm = mi->num_heads;
  p.bm = dc->ptr[SPLASH_MI_BLOCK_MASK];
  p.dn = dc->ptr[SPLASH_MI_DATA_NEXT];
  p.mn = dc->ptr[SPLASH_MI_MASK_NEXT];
  p.pmb = static_cast<const uint8_t *>(dc->ptr[SPLASH_MI_PARTIAL_BLOCKS]);
  p.pmb_bits = dc->mask_bits;
  p.pmb_bits_bytes = dc->mask_bits_bytes;
  p.q_seq = static_cast<const int32_t *>(dc->ptr[SPLASH_MI_Q_SEQUENCE]);
  p.row_order = dc->row_order;
  p.walk_kv = dc->walk_kv;
  p.walk_mn = dc->walk_mn;
  p.items = dc->items[1];
  p.bm_bytes = mi->arr[SPLASH_MI_BLOCK_MASK].elem_bits / 8;
  p.dn_bytes = mi->arr[SPLASH_MI_DATA_NEXT].elem_bits / 8;
  p.mn_bytes = mi->arr[SPLASH_MI_MASK_NEXT].present ? mi->arr[SPLASH_MI_MASK_NEXT].elem_bits / 8 : 4;
  if (dc->kbm) {   // blocks larger than 128 x 128: the kernel view
    p.nq = static_cast<int32_t>(mi->kview.nq);
    p.width = static_cast<int32_t>(mi->kview.width);
    p.bm = dc->kbm;
    p.dn = dc->kdn;
    p.mn = dc->kmn;
    p.pmb = dc->kpmb;
    p.pmb_bits = dc->kbits;
    p.pmb_bits_bytes = dc->kbits_bytes;
    p.row_order = dc->krow_order;
    p.bm_bytes = p.dn_bytes = p.mn_bytes = 4;
  }
  p.mask_kind = mi->kind;
  p.left = mi->left;
  p.right = mi->right;
  p.chunk = mi->chunk;
  p.kv_offset = mi->kv_offset;
  p.dense = mi->kind == SPLASH_MASK_DENSE;
  const bool cap = std::isfinite(logits_soft_cap) && logits_soft_cap > 0.f;
  p.cap = cap;
  const double log2e = 1.4426950408889634;
  p.c2 = cap ? static_cast<float>(static_cast<double>(scale) / logits_soft_cap)
             : static_cast<float>(scale * log2e);
  p.cap_out = cap ? static_cast<float>(logits_soft_cap * log2e) : 0.f;
  return p;
}

float resolve_scale(float softmax_scale, int64_t D) {
  return std::isnan(softmax_scale) ? static_cast<float>(1.0 / std::sqrt(static_cast<double>(D))) : softmax_scale;
}

// Bytes of the split-key workspace: normalised partial outputs, bf16
// [S, B, Hq, Sq, Dv], then their lses, float32 [S, B, Hq, Sq].
int64_t split_workspace_bytes(int64_t B, int64_t Hq, int64_t Sq, int64_t Dv, int64_t S) {
  return S > 1 ? S * B * Hq * Sq * (2 * Dv + 4) : 0;
}

// Whether two query heads of a GQA group can share a workgroup (and its K/V
// stages): the bf16 kernel at D = 128 with a computable mask and one mask
// head (so both heads walk the same blocks) and an even group size (so the
// pair shares its K/V head).
bool head_pairs_possible(const splash_mask_info *mi, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                         int32_t dtype) {
  const int64_t kernel_dim = native_dims(D, Dv) ? D : padded_kernel_dim(D, Dv);
  return dtype == SPLASH_BF16 && kernel_dim == 128 && mi->kind != SPLASH_MASK_DENSE && mi->num_heads == 1 &&
         Hkv > 0 && (Hq / Hkv) % 2 == 0;
}

// The library's choice of heads per workgroup: pairs where possible, as long
// as the pairs still give each CU a workgroup (a pair fills a CU alone).
int32_t auto_heads_per_wg(const splash_mask_info *mi, int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                          int32_t dtype, int32_t kv_splits) {
  if (!head_pairs_possible(mi, Hq, Hkv, D, Dv, dtype)) return 1;
  return B * (Hq / 2) * walk_of(mi).nq * kv_splits >= 256 ? 2 : 1;
}

splash_status fwd_impl(splash_mask_info *mi, const void *q, const void *k, const void *v, void *out,
                       float *lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv,
                       int64_t D, int64_t Dv, int32_t dtype, float softmax_scale,
                       float logits_soft_cap, const float *aux, int32_t aux_heads,
                       int32_t num_sinks, int32_t kv_splits, int32_t heads_per_wg, void *workspace,
                       size_t workspace_bytes, void *hip_stream) {
  // ---- validation: nothing below launches or allocates until all passes ----
  splash_status st = validate_call(mi, B, Hq, Hkv, Sq, Skv, D, Dv, dtype, softmax_scale, true);
  if (st != SPLASH_OK) return st;
  const bool padded = !native_dims(D, Dv);
  if (heads_per_wg < 0 || heads_per_wg > 2) return fail(SPLASH_EINVAL, "heads_per_workgroup must be 0, 1 or 2");
  if (heads_per_wg == 2 && !head_pairs_possible(mi, Hq, Hkv, D, Dv, dtype))
    return fail(SPLASH_EUNSUPPORTED, "two heads per workgroup need bf16, the 128-column kernel, a computable mask "
                                     "with one mask head and an even GQA group");
  if (kv_splits < 1 || kv_splits > DeviceCopy::kMaxSplits)
    return fail(SPLASH_EINVAL, "kv_splits must be in 1..8");
  if (kv_splits > 1 && dtype != SPLASH_BF16)
    return fail(SPLASH_EUNSUPPORTED, "key splits run on the bf16 kernel only");
  if (B * Hq * (Sq / 128) * kv_splits > 0x7fffffffLL) return fail(SPLASH_EUNSUPPORTED, "grid too large");
  if (kv_splits > 1 && B > 0 && Hq > 0 && Sq > 0) {
    const int64_t need = split_workspace_bytes(B, Hq, Sq, Dv, kv_splits);
    if (!workspace || workspace_bytes < static_cast<size_t>(need))
      return fail(SPLASH_EINVAL, "workspace missing or smaller than splash_fwd_workspace_size");
    if (reinterpret_cast<uintptr_t>(workspace) % 16) return fail(SPLASH_EINVAL, "workspace must be 16-byte aligned");
  }
  if (num_sinks < 0) return fail(SPLASH_EINVAL, "num_sinks must be >= 0");
  if (num_sinks > 0) {
    if (!aux) return fail(SPLASH_EINVAL, "softmax_aux is NULL with num_sinks > 0");
    if (aux_heads != 1 && aux_heads != Hkv && aux_heads != Hq)
      return fail(SPLASH_EINVAL, "softmax_aux must have 1, Hkv or Hq rows");
    if (reinterpret_cast<uintptr_t>(aux) % 4 != 0) return fail(SPLASH_EINVAL, "softmax_aux must be 4-byte aligned");
  }
  if (B == 0 || Hq == 0 || Sq == 0) return SPLASH_OK;
  if (!q || !out || (Skv > 0 && (!k || !v)))
    return fail(SPLASH_EINVAL, "NULL tensor pointer");
  if (!aligned16({q, k, v, out})) return fail(SPLASH_EINVAL, "q, k, v and out must be 16-byte aligned");

  DeviceCopy *dc = nullptr;
  st = ensure_device_copy(mi, &dc);
  if (st != SPLASH_OK) return st;
  if (kv_splits > 1) {
    std::lock_guard<std::mutex> lock(mi->mu);
    st = ensure_items(mi, *dc, kv_splits);
    if (st != SPLASH_OK) return st;
  }

  FwdParams p = make_params(mi, dc, q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, resolve_scale(softmax_scale, D),
                            logits_soft_cap);
  p.aux = num_sinks > 0 ? aux : nullptr;
  p.aux_heads = num_sinks > 0 ? aux_heads : 0;
  p.num_sinks = num_sinks;
  p.kv_splits = kv_splits;
  p.items = dc->items[kv_splits];
  const int32_t hpw =
      heads_per_wg != 0 ? heads_per_wg : auto_heads_per_wg(mi, B, Hq, Hkv, D, Dv, dtype, kv_splits);
  p.head_pairs = hpw == 2 ? 1 : 0;
  if (padded) {
    p.D = static_cast<int32_t>(padded_kernel_dim(D, Dv));
    p.dk = static_cast<int32_t>(D);
    p.dv = static_cast<int32_t>(Dv);
    p.padded = 1;
  }
  if (kv_splits > 1) {
    p.part_o = workspace;
    p.part_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) + kv_splits * B * Hq * Sq * Dv * 2);
  }

  hipError_t e = launch_fwd(p, dtype, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(SPLASH_EHIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return SPLASH_OK;
}

}  // namespace

extern "C" SPLASH_API splash_status splash_fwd(splash_mask_info *mi, const void *q, const void *k,
                                               const void *v, void *out, float *lse, int64_t B,
                                               int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv,
                                               int64_t D, int64_t Dv, int32_t dtype,
                                               float softmax_scale, float logits_soft_cap,
                                               void *hip_stream) {
  clear_error();
  return fwd_impl(mi, q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, Dv, dtype, softmax_scale,
                  logits_soft_cap, nullptr, 0, 0, 1, 0, nullptr, 0, hip_stream);
}

extern "C" SPLASH_API splash_status splash_fwd_sinks(splash_mask_info *mi, const void *q, const void *k,
                                                     const void *v, void *out, float *lse, int64_t B,
                                                     int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Skv,
                                                     int64_t D, int64_t Dv, int32_t dtype,
                                                     float softmax_scale, float logits_soft_cap,
                                                     const float *softmax_aux, int32_t aux_heads,
                                                     int32_t num_sinks, void *hip_stream) {
  clear_error();
  return fwd_impl(mi, q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, Dv, dtype, softmax_scale,
                  logits_soft_cap, softmax_aux, aux_heads, num_sinks, 1, 0, nullptr, 0, hip_stream);
}

extern "C" SPLASH_API splash_status splash_fwd_workspace_size(int64_t B, int64_t Hq, int64_t Sq, int64_t Dv,
                                                              int32_t kv_splits, size_t *bytes) {
  clear_error();
  if (!bytes) return fail(SPLASH_EINVAL, "bytes is NULL");
  if (B < 0 || Hq < 0 || Sq < 0 || Dv <= 0) return fail(SPLASH_EINVAL, "negative size or non-positive head dim");
  if (kv_splits < 1 || kv_splits > DeviceCopy::kMaxSplits) return fail(SPLASH_EINVAL, "kv_splits must be in 1..8");
  *bytes = static_cast<size_t>(split_workspace_bytes(B, Hq, Sq, Dv, kv_splits));
  return SPLASH_OK;
}

extern "C" SPLASH_API splash_status splash_fwd_plan(const splash_mask_info *mi, int64_t B, int64_t Hq, int32_t dtype,
                                                    int32_t *kv_splits) {
  clear_error();
  if (!mi || !kv_splits) return fail(SPLASH_EINVAL, "NULL argument");
  if (B < 0 || Hq < 0) return fail(SPLASH_EINVAL, "negative size");
  if (dtype != SPLASH_BF16 && dtype != SPLASH_F32) return fail(SPLASH_EINVAL, "unknown dtype");
  *kv_splits = 1;
  if (dtype != SPLASH_BF16 || B == 0 || Hq == 0) return SPLASH_OK;
  int dev = -1, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "querying the device's compute units");
  const Walk wk = walk_of(mi);
  const int64_t n_wg = B * Hq * wk.nq;
  const int64_t slots = 2 * static_cast<int64_t>(cus);   // the bf16 kernel runs two workgroups per CU
  if (n_wg == 0 || n_wg >= slots) return SPLASH_OK;
  // non-empty 128 x 128 blocks per block row, on average
  const HostArray &bm = mi->arr[SPLASH_MI_BLOCK_MASK];
  int64_t nonempty = 0;
  for (int64_t i = 0; i < bm.numel(); ++i) nonempty += host_index(bm, i) > 0 ? 1 : 0;
  nonempty *= (mi->block_q / 128) * (mi->block_kv / 128);
  const int64_t rows = std::max<int64_t>(1, mi->num_heads * wk.nq);
  const int64_t per_row = nonempty / rows;
  int64_t S = (slots + n_wg - 1) / n_wg;
  S = std::min<int64_t>(S, std::max<int64_t>(1, per_row / 2));   // at least two blocks per split
  *kv_splits = static_cast<int32_t>(std::min<int64_t>(S, DeviceCopy::kMaxSplits));
  return SPLASH_OK;
}

extern "C" SPLASH_API splash_status splash_fwd_split(splash_mask_info *mi, const void *q, const void *k,
                                                     const void *v, void *out, float *lse, int64_t B, int64_t Hq,
                                                     int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D, int64_t Dv,
                                                     int32_t dtype, float softmax_scale, float logits_soft_cap,
                                                     const float *softmax_aux, int32_t aux_heads, int32_t num_sinks,
                                                     int32_t kv_splits, void *workspace, size_t workspace_bytes,
                                                     void *hip_stream) {
  clear_error();
  return fwd_impl(mi, q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, Dv, dtype, softmax_scale, logits_soft_cap,
                  softmax_aux, aux_heads, num_sinks, kv_splits, 0, workspace, workspace_bytes, hip_stream);
}

extern "C" SPLASH_API splash_status splash_fwd_tiled(splash_mask_info *mi, const void *q, const void *k,
                                                     const void *v, void *out, float *lse, int64_t B, int64_t Hq,
                                                     int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D, int64_t Dv,
                                                     int32_t dtype, float softmax_scale, float logits_soft_cap,
                                                     const float *softmax_aux, int32_t aux_heads, int32_t num_sinks,
                                                     int32_t kv_splits, int32_t heads_per_workgroup, void *workspace,
                                                     size_t workspace_bytes, void *hip_stream) {
  clear_error();
  return fwd_impl(mi, q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, Dv, dtype, softmax_scale, logits_soft_cap,
                  softmax_aux, aux_heads, num_sinks, kv_splits, heads_per_workgroup, workspace, workspace_bytes,
                  hip_stream);
}

extern "C" SPLASH_API splash_status splash_fwd_heads_per_workgroup(const splash_mask_info *mi, int64_t B,
                                                                   int64_t Hq, int64_t Hkv, int64_t D, int32_t dtype,
                                                                   int32_t kv_splits, int32_t *heads) {
  clear_error();
  if (!mi || !heads) return fail(SPLASH_EINVAL, "NULL argument");
  if (B < 0 || Hq < 0 || Hkv <= 0) return fail(SPLASH_EINVAL, "bad head counts");
  if (dtype != SPLASH_BF16 && dtype != SPLASH_F32) return fail(SPLASH_EINVAL, "unknown dtype");
  if (kv_splits < 1 || kv_splits > DeviceCopy::kMaxSplits) return fail(SPLASH_EINVAL, "kv_splits must be in 1..8");
  *heads = auto_heads_per_wg(mi, B, Hq, Hkv, D, D, dtype, kv_splits);
  return SPLASH_OK;
}

extern "C" SPLASH_API splash_status splash_lse_merge(const void *out_a, const float *lse_a, int32_t dtype_a,
                                                     const void *out_b, const float *lse_b, int32_t dtype_b,
                                                     void *out, float *lse, int32_t dtype_out, int64_t rows,
                                                     int64_t Dv, void *hip_stream) {
  clear_error();
  auto ok_dt = [](int32_t d) { return d == SPLASH_BF16 || d == SPLASH_F32; };
  if (!ok_dt(dtype_a) || !ok_dt(dtype_b) || !ok_dt(dtype_out)) return fail(SPLASH_EINVAL, "unknown dtype");
  if (rows < 0) return fail(SPLASH_EINVAL, "rows must be >= 0");
  if (Dv <= 0 || Dv % 8 != 0 || Dv > 512) return fail(SPLASH_EUNSUPPORTED, "Dv must be a multiple of 8 up to 512");
  if (rows == 0) return SPLASH_OK;
  if (!out_a || !lse_a || !out_b || !lse_b || !out || !lse) return fail(SPLASH_EINVAL, "NULL pointer");
  if ((reinterpret_cast<uintptr_t>(out_a) | reinterpret_cast<uintptr_t>(out_b) | reinterpret_cast<uintptr_t>(out)) % 16)
    return fail(SPLASH_EINVAL, "outputs must be 16-byte aligned");
  if ((out == out_a && dtype_out != dtype_a) || (out == out_b && dtype_out != dtype_b))
    return fail(SPLASH_EINVAL, "an output written in place must keep its dtype");
  if (rows > (int64_t(1) << 40) / Dv) return fail(SPLASH_EUNSUPPORTED, "too many elements");
  hipError_t e = launch_lse_merge(out_a, lse_a, dtype_a == SPLASH_BF16 ? 0 : 1, out_b, lse_b,
                                  dtype_b == SPLASH_BF16 ? 0 : 1, out, lse, dtype_out == SPLASH_BF16 ? 0 : 1,
                                  rows, static_cast<int>(Dv), static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(SPLASH_EHIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return SPLASH_OK;
}

extern "C" SPLASH_API splash_status splash_bwd(splash_mask_info *mi, const void *q, const void *k, const void *v,
                                               const void *out, const float *lse, const void *dout, void *dq,
                                               void *dk, void *dv, float *delta, int64_t B, int64_t Hq,
                                               int64_t Hkv, int64_t Sq, int64_t Skv, int64_t D, int64_t Dv,
                                               int32_t dtype, float softmax_scale, float logits_soft_cap,
                                               void *hip_stream) {
  clear_error();
  // ---- validation: nothing below launches or allocates until all passes ----
  splash_status st = validate_call(mi, B, Hq, Hkv, Sq, Skv, D, Dv, dtype, softmax_scale, true);
  if (st != SPLASH_OK) return st;
  if (dtype != SPLASH_BF16) return fail(SPLASH_EUNSUPPORTED, "the backward kernels run bf16 only");
  if (B == 0 || Hq == 0 || (Sq == 0 && Skv == 0)) return SPLASH_OK;
  if (Sq > 0 && (!q || !out || !lse || !dout || !dq || !delta)) return fail(SPLASH_EINVAL, "NULL tensor pointer");
  if (Skv > 0 && (!k || !v || !dk || !dv)) return fail(SPLASH_EINVAL, "NULL tensor pointer");
  if (!aligned16({q, k, v, out, dout, dq, dk, dv}))
    return fail(SPLASH_EINVAL, "q, k, v, out, dout, dq, dk and dv must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(lse) % 4 || reinterpret_cast<uintptr_t>(delta) % 4)
    return fail(SPLASH_EINVAL, "lse and delta must be 4-byte aligned");

  DeviceCopy *dc = nullptr;
  st = ensure_device_copy(mi, &dc);
  if (st != SPLASH_OK) return st;
  {
    std::lock_guard<std::mutex> lock(mi->mu);
    st = ensure_cols(mi, *dc);
  }
  if (st != SPLASH_OK) return st;

  BwdParams p{};
  p.f = make_params(mi, dc, q, k, v, const_cast<void *>(out), const_cast<float *>(lse), B, Hq, Hkv, Sq, Skv, D,
                    resolve_scale(softmax_scale, D), logits_soft_cap);
  if (!native_dims(D, Dv)) {   // run zero-padded, as the forward does
    p.f.D = static_cast<int32_t>(padded_kernel_dim(D, Dv));
    p.f.dk = static_cast<int32_t>(D);
    p.f.dv = static_cast<int32_t>(Dv);
    p.f.padded = 1;
  }
  p.dout = dout;
  p.delta = delta;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.scale = resolve_scale(softmax_scale, D);
  p.nk = static_cast<int32_t>(Skv / 128);
  p.col_n = dc->col_n;
  p.col_ent = dc->col_ent;
  p.col_mn = dc->col_mn;
  p.col_order = dc->col_order;
  p.col_w = dc->col_w;
  hipError_t e = launch_bwd(p, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(SPLASH_EHIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return SPLASH_OK;
}

namespace {
// The decode kernel's head dim: D itself (64 or 128), or the 64- or
// 128-column kernel that runs D zero-padded.
int64_t decode_kernel_dim(int64_t D) { return D == 64 || D == 128 ? D : padded_kernel_dim(D, D); }

int64_t decode_ws_floats(int64_t B, int64_t Hq, int64_t Hkv, int64_t Skv, int64_t D) {
  const int64_t group = Hkv > 0 ? Hq / Hkv : 0;
  return B * Hkv * decode_chunks(B * Hkv, group, D, Skv) * group * (decode_kernel_dim(D) + 2);
}
}  // namespace

extern "C" SPLASH_API splash_status splash_decode_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t Skv,
                                                                 int64_t D, size_t *bytes) {
  clear_error();
  if (!bytes) return fail(SPLASH_EINVAL, "bytes is NULL");
  if (B < 0 || Hq < 0 || Hkv <= 0 || Skv < 0 || D <= 0 || Hq % Hkv)
    return fail(SPLASH_EINVAL, "bad sizes (Hkv > 0 and Hq % Hkv == 0 required)");
  *bytes = static_cast<size_t>(decode_ws_floats(B, Hq, Hkv, Skv, D)) * sizeof(float);
  return SPLASH_OK;
}

namespace {

// Size and argument checks of both decode entry points (pointers and the
// workspace aside).  Returns SPLASH_OK with *noop set when there is nothing
// to compute.
splash_status decode_validate(int64_t B, int64_t Hq, int64_t Hkv, int64_t Skv, int64_t D, int64_t Dv, int32_t dtype,
                              float softmax_scale, bool *noop) {
  *noop = false;
  if (B < 0 || Hq < 0 || Hkv < 0 || Skv < 0 || D <= 0 || Dv <= 0)
    return fail(SPLASH_EINVAL, "negative size or non-positive head dim");
  if (dtype != SPLASH_BF16 && dtype != SPLASH_F32) return fail(SPLASH_EINVAL, "unknown dtype");
  if (dtype != SPLASH_BF16) return fail(SPLASH_EUNSUPPORTED, "decode runs bf16 only");
  if (Hkv == 0 && Hq > 0) return fail(SPLASH_EINVAL, "Hkv must be positive");
  if (Hkv > 0 && Hq % Hkv) return fail(SPLASH_EINVAL, "Hq must be a multiple of Hkv");
  if (D != Dv || !padded_dims_ok(D, Dv))
    return fail(SPLASH_EUNSUPPORTED, "decode head dims must satisfy D == Dv, a multiple of 16 up to 128");
  if (!(std::isnan(softmax_scale) || (std::isfinite(softmax_scale) && softmax_scale > 0.f)))
    return fail(SPLASH_EINVAL, "softmax_scale must be NaN (default) or finite and > 0");
  if (B == 0 || Hq == 0) {
    *noop = true;
    return SPLASH_OK;
  }
  const int64_t group = Hq / Hkv;
  if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16)
    return fail(SPLASH_EUNSUPPORTED, "decode runs GQA groups of 1, 2, 4, 8 or 16 query heads");
  if (Skv == 0) return fail(SPLASH_EUNSUPPORTED, "decode needs at least one key");
  if (B * Hkv > 0x7fffffffLL || decode_chunks(B * Hkv, group, D, Skv) > 65535 || B * Hq > 0x7fffffffLL)
    return fail(SPLASH_EUNSUPPORTED, "grid too large");
  if (Skv * D * 2 > kMaxHeadBytes)
    return fail(SPLASH_EUNSUPPORTED, "the K (or V) cache of one head exceeds 2 GiB");
  return SPLASH_OK;
}

// Launch of both decode entry points: the partial and merge kernels with
// their scratch at `workspace` (already checked to be large enough).
splash_status decode_launch(const void *q, const void *k, const void *v, void *out, float *lse, void *workspace,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t Skv, int64_t D, float softmax_scale,
                            float logits_soft_cap, void *hip_stream) {
  const int64_t group = Hq / Hkv;
  DecodeParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.B = static_cast<int32_t>(B);
  p.Hq = static_cast<int32_t>(Hq);
  p.Hkv = static_cast<int32_t>(Hkv);
  p.group = static_cast<int32_t>(group);
  const int64_t kd = decode_kernel_dim(D);
  p.D = static_cast<int32_t>(kd);
  p.dim = static_cast<int32_t>(D);
  p.padded = kd != D ? 1 : 0;
  p.Skv = Skv;
  p.n_chunks = static_cast<int32_t>(decode_chunks(B * Hkv, group, D, Skv));
  p.split_keys = decode_split_keys(B * Hkv, group, D, Skv);
  const float scale = resolve_scale(softmax_scale, D);
  const bool cap = std::isfinite(logits_soft_cap) && logits_soft_cap > 0.f;
  const double log2e = 1.4426950408889634;
  p.cap = cap;
  p.c2 = cap ? static_cast<float>(static_cast<double>(scale) / logits_soft_cap) : static_cast<float>(scale * log2e);
  p.cap_out = cap ? static_cast<float>(logits_soft_cap * log2e) : 0.f;
  const int64_t n_slot = B * Hkv * p.n_chunks * group;
  p.ws_o = static_cast<float *>(workspace);
  p.ws_m = p.ws_o + n_slot * kd;
  p.ws_l = p.ws_m + n_slot;
  hipError_t e = launch_decode(p, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(SPLASH_EHIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return SPLASH_OK;
}

}  // namespace

extern "C" SPLASH_API splash_status splash_decode(const void *q, const void *k, const void *v, void *out, float *lse,
                                                  void *workspace, size_t workspace_bytes, int64_t B, int64_t Hq,
                                                  int64_t Hkv, int64_t Skv, int64_t D, int64_t Dv, int32_t dtype,
                                                  float softmax_scale, float logits_soft_cap, void *hip_stream) {
  clear_error();
  bool noop = false;
  splash_status st = decode_validate(B, Hq, Hkv, Skv, D, Dv, dtype, softmax_scale, &noop);
  if (st != SPLASH_OK || noop) return st;
  if (!q || !k || !v || !out || !workspace) return fail(SPLASH_EINVAL, "NULL pointer");
  if (!aligned16({q, k, v, out, workspace})) return fail(SPLASH_EINVAL, "q, k, v, out and workspace must be 16-byte aligned");
  const int64_t floats = decode_ws_floats(B, Hq, Hkv, Skv, D);
  if (workspace_bytes < static_cast<size_t>(floats) * sizeof(float))
    return fail(SPLASH_EINVAL, "workspace smaller than splash_decode_workspace_size");
  return decode_launch(q, k, v, out, lse, workspace, B, Hq, Hkv, Skv, D, softmax_scale, logits_soft_cap, hip_stream);
}

extern "C" SPLASH_API splash_status splash_decode_static(const void *q, const void *k, const void *v, void *out,
                                                         float *lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Skv,
                                                         int64_t D, int64_t Dv, int32_t dtype, float softmax_scale,
                                                         float logits_soft_cap, void *hip_stream) {
  clear_error();
  bool noop = false;
  splash_status st = decode_validate(B, Hq, Hkv, Skv, D, Dv, dtype, softmax_scale, &noop);
  if (st != SPLASH_OK || noop) return st;
  if (!q || !k || !v || !out) return fail(SPLASH_EINVAL, "NULL pointer");
  if (!aligned16({q, k, v, out})) return fail(SPLASH_EINVAL, "q, k, v and out must be 16-byte aligned");
  const size_t need = static_cast<size_t>(decode_ws_floats(B, Hq, Hkv, Skv, D)) * sizeof(float);
  if (need > kDecodeStaticScratchBytes)
    return fail(SPLASH_EUNSUPPORTED, "this decode needs " + std::to_string(need) +
                                         " bytes of scratch; the library's static scratch holds " +
                                         std::to_string(kDecodeStaticScratchBytes) +
                                         " (use splash_decode with a workspace)");
  void *scratch = nullptr;
  const hipError_t e = decode_static_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "looking up the static decode scratch");
  return decode_launch(q, k, v, out, lse, scratch, B, Hq, Hkv, Skv, D, softmax_scale, logits_soft_cap, hip_stream);
}
