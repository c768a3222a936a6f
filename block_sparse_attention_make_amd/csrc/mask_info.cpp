// Host mask compiler: mask description -> MaskInfo.
//
// Implements the compile-time pass of the splash-attention explainer
// (explainers.rudrite.com/splash-attention), FAQ "What is MaskInfo in splash
// attention?", "Does splash attention make every sparse mask faster?" and
// "What does grid shrinking do in splash attention?":
//   * labels per grid-step block by the any / all questions (0 empty,
//     1 mixed, 2 full).  Computable masks are labelled in closed form from
//     the interval of keys each query row admits -- no mask is materialised;
//     dense masks are scanned byte by byte;
//   * the mixed blocks of a dense mask are deduplicated (hash + byte compare)
//     into partial_mask_blocks, one byte per element;
//   * grid shrink: each block row keeps its non-empty columns, padded to the
//     longest row;
//   * data_next / mask_next: what to fetch at each grid position without
//     fetching again across a skipped block;
//   * int8 / int16 downcast of the three index arrays when their max fits;
//   * q_sequence for computable masks (mask_next / partial blocks are None).
#include <algorithm>
#include <cstring>
#include <limits>
#include <new>
#include <numeric>
#include <unordered_map>

#include "mask_info.h"

namespace splash {
namespace {

constexpr int64_t kInf = std::numeric_limits<int64_t>::max() / 4;

int64_t sat_add(int64_t a, int64_t b) {
  if (b > 0 && a > kInf - b) return kInf;
  if (b < 0 && a < -kInf - b) return -kInf;
  return a + b;
}

int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  return (a % b != 0 && ((a < 0) != (b < 0))) ? q - 1 : q;
}

// Label of the block of query rows [i0, i1] x key columns [j0, j1] for a
// computable mask.  Each query row i admits one key interval [lo(i), hi(i)].
int label_computable(const splash_mask_info &m, int64_t i0, int64_t i1, int64_t j0, int64_t j1) {
  bool any = false, all = false;
  switch (m.kind) {
    case SPLASH_MASK_CAUSAL:  // lo = -inf, hi = i
      any = j0 <= i1;
      all = j1 <= i0;
      break;
    case SPLASH_MASK_LOCAL: {  // lo = i - left, hi = i + right
      const int64_t L = m.left < 0 ? kInf : m.left;
      const int64_t R = m.right < 0 ? kInf : m.right;
      // some row i in [i0, i1] with i - L <= j1 and i + R >= j0
      any = std::max(i0, sat_add(j0, -R)) <= std::min(i1, sat_add(j1, L));
      // every row admits [j0, j1]: the tightest rows are i1 (left) and i0 (right)
      all = sat_add(i1, -L) <= j0 && j1 <= sat_add(i0, R);
      break;
    }
    case SPLASH_MASK_CHUNKED_CAUSAL: {  // lo = chunk start of i, hi = i
      const int64_t C = m.chunk;
      const int64_t g0 = std::max(floor_div(i0, C), floor_div(j0, C));
      const int64_t g1 = std::min(floor_div(i1, C), floor_div(j1, C));
      for (int64_t g = g0; g <= g1 && !any; ++g) {
        const int64_t top_i = std::min(i1, g * C + C - 1);  // latest row in chunk g
        const int64_t first_j = std::max(j0, g * C);        // earliest key in chunk g
        any = first_j <= top_i && top_i >= std::max(i0, g * C) && first_j <= std::min(j1, g * C + C - 1);
      }
      all = floor_div(i0, C) == floor_div(i1, C) && floor_div(j0, C) == floor_div(j1, C) &&
            floor_div(i0, C) == floor_div(j0, C) && j1 <= i0;
      break;
    }
    default:
      break;
  }
  return all ? 2 : (any ? 1 : 0);
}

uint64_t fnv1a(const uint8_t *p, size_t n) {
  uint64_t h = 1469598103934665603ull;
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 1099511628211ull;
  }
  return h;
}

template <typename T>
void store_as(HostArray &a, const std::vector<int64_t> &v) {
  a.bytes.resize(v.size() * sizeof(T));
  T *dst = reinterpret_cast<T *>(a.bytes.data());
  for (size_t i = 0; i < v.size(); ++i) dst[i] = static_cast<T>(v[i]);
}

void fill_index_array(HostArray &a, const std::vector<int64_t> &v, int64_t d0, int64_t d1,
                      int64_t d2, bool downcast) {
  int64_t mx = 0;
  for (int64_t x : v) mx = std::max(mx, x);
  a.present = true;
  a.is_signed = true;
  a.ndim = 3;
  a.shape[0] = d0;
  a.shape[1] = d1;
  a.shape[2] = d2;
  if (downcast && mx <= 127) {
    a.elem_bits = 8;
    store_as<int8_t>(a, v);
  } else if (downcast && mx <= 32767) {
    a.elem_bits = 16;
    store_as<int16_t>(a, v);
  } else {
    a.elem_bits = 32;
    store_as<int32_t>(a, v);
  }
}

splash_status validate(const splash_mask_desc *d, int32_t bq, int32_t bk) {
  if (!d) return fail(SPLASH_EINVAL, "mask descriptor is NULL");
  if (bq <= 0 || bk <= 0) return fail(SPLASH_EINVAL, "block sizes must be positive");
  if (d->q_len < 0 || d->kv_len < 0) return fail(SPLASH_EINVAL, "sequence lengths must be >= 0");
  if (d->q_len % bq) return fail(SPLASH_EINVAL, "block_q must divide q_len");
  if (d->kv_len % bk) return fail(SPLASH_EINVAL, "block_kv must divide kv_len");
  if (d->q_len / bq > std::numeric_limits<int32_t>::max() ||
      d->kv_len / bk > std::numeric_limits<int32_t>::max())
    return fail(SPLASH_EINVAL, "too many blocks");
  switch (d->kind) {
    case SPLASH_MASK_CAUSAL:
    case SPLASH_MASK_LOCAL:
      if (d->num_heads != 1) return fail(SPLASH_EINVAL, "computable masks have num_heads == 1");
      break;
    case SPLASH_MASK_CHUNKED_CAUSAL:
      if (d->num_heads != 1) return fail(SPLASH_EINVAL, "computable masks have num_heads == 1");
      if (d->chunk <= 0) return fail(SPLASH_EINVAL, "chunked causal mask needs chunk > 0");
      break;
    case SPLASH_MASK_DENSE:
      if (d->num_heads <= 0) return fail(SPLASH_EINVAL, "dense mask needs num_heads >= 1");
      if (!d->dense && d->q_len > 0 && d->kv_len > 0)
        return fail(SPLASH_EINVAL, "dense mask bytes are NULL");
      break;
    default:
      return fail(SPLASH_EINVAL, "unknown mask kind");
  }
  return SPLASH_OK;
}

void compile(splash_mask_info &m, const splash_mask_desc &d) {
  const int64_t hm = m.num_heads, nq = m.nq, nk = m.nk, bq = m.block_q, bk = m.block_kv;
  const bool dense = m.kind == SPLASH_MASK_DENSE;
  const bool shrink = m.flags & SPLASH_FLAG_SHRINK;
  const bool downcast = m.flags & SPLASH_FLAG_DOWNCAST;

  // 1. Labels on the unshrunk grid.
  std::vector<uint8_t> label(static_cast<size_t>(hm * nq * nk), 0);
  if (!dense) {
    for (int64_t r = 0; r < nq; ++r)
      for (int64_t c = 0; c < nk; ++c)
        label[r * nk + c] = static_cast<uint8_t>(label_computable(
            m, r * bq, r * bq + bq - 1, m.kv_offset + c * bk, m.kv_offset + c * bk + bk - 1));
  } else {
    std::vector<uint8_t> seen_one(static_cast<size_t>(nk)), seen_zero(static_cast<size_t>(nk));
    for (int64_t h = 0; h < hm; ++h)
      for (int64_t r = 0; r < nq; ++r) {
        std::fill(seen_one.begin(), seen_one.end(), 0);
        std::fill(seen_zero.begin(), seen_zero.end(), 0);
        for (int64_t i = r * bq; i < r * bq + bq; ++i) {
          const uint8_t *row = d.dense + (h * m.q_len + i) * m.kv_total + m.kv_offset;
          for (int64_t c = 0; c < nk; ++c) {
            const uint8_t *seg = row + c * bk;
            for (int64_t j = 0; j < bk; ++j) {
              if (seg[j]) seen_one[c] = 1; else seen_zero[c] = 1;
            }
          }
        }
        for (int64_t c = 0; c < nk; ++c)
          label[(h * nq + r) * nk + c] = seen_one[c] ? (seen_zero[c] ? 1 : 2) : 0;
      }
  }

  // 2. Deduplicated stack of mixed blocks (dense masks only).
  std::vector<int64_t> pidx(static_cast<size_t>(hm * nq * nk), 0);
  std::vector<uint8_t> stack;
  int64_t n_partial = 0;
  if (dense) {
    const size_t blk = static_cast<size_t>(bq * bk);
    std::unordered_map<uint64_t, std::vector<int64_t>> by_hash;
    std::vector<uint8_t> cur(blk);
    for (int64_t h = 0; h < hm; ++h)
      for (int64_t r = 0; r < nq; ++r)
        for (int64_t c = 0; c < nk; ++c) {
          const size_t at = static_cast<size_t>((h * nq + r) * nk + c);
          if (label[at] != 1) continue;
          for (int64_t i = 0; i < bq; ++i) {
            const uint8_t *src = d.dense + (h * m.q_len + r * bq + i) * m.kv_total + m.kv_offset + c * bk;
            for (int64_t j = 0; j < bk; ++j) cur[i * bk + j] = src[j] ? 1 : 0;
          }
          const uint64_t key = fnv1a(cur.data(), blk);
          auto &cands = by_hash[key];
          int64_t found = -1;
          for (int64_t p : cands)
            if (std::memcmp(stack.data() + p * blk, cur.data(), blk) == 0) { found = p; break; }
          if (found < 0) {
            found = n_partial++;
            cands.push_back(found);
            stack.insert(stack.end(), cur.begin(), cur.end());
          }
          pidx[at] = found;
        }
  }

  // 3. Shrink: the columns each (head, block row) keeps.
  std::vector<int64_t> count(static_cast<size_t>(hm * nq), 0);
  int64_t width = shrink ? 1 : std::max<int64_t>(nk, 1);
  if (shrink) {
    for (int64_t hr = 0; hr < hm * nq; ++hr) {
      for (int64_t c = 0; c < nk; ++c) count[hr] += label[hr * nk + c] > 0;
      width = std::max(width, count[hr]);
    }
  }
  m.width = width;

  // 4./5. block_mask, data_next, mask_next on the (shrunk) grid.
  const size_t n_slots = static_cast<size_t>(hm * nq * width);
  std::vector<int64_t> bm(n_slots, 0), dn(n_slots, 0), mn(n_slots, 0);
  std::vector<int64_t> col(static_cast<size_t>(width));
  for (int64_t hr = 0; hr < hm * nq; ++hr) {
    const uint8_t *lab = &label[hr * nk];
    int64_t n = 0;
    if (shrink) {
      for (int64_t c = 0; c < nk; ++c)
        if (lab[c]) col[n++] = c;
    } else {
      for (int64_t c = 0; c < nk; ++c) col[n++] = c;
    }
    int64_t *rbm = &bm[hr * width], *rdn = &dn[hr * width], *rmn = &mn[hr * width];
    for (int64_t s = 0; s < n; ++s) rbm[s] = lab[col[s]];
    // Backward sweep: nearest non-empty / partial slot at or after s.
    int64_t next_data = -1, next_mask = -1;
    for (int64_t s = width - 1; s >= 0; --s) {
      if (rbm[s] > 0) next_data = col[s];
      if (rbm[s] == 1) next_mask = pidx[hr * nk + col[s]];
      rdn[s] = next_data;
      rmn[s] = next_mask;
    }
    // Forward sweep: slots with nothing after them take the last one before.
    int64_t prev_data = 0, prev_mask = 0;
    for (int64_t s = 0; s < width; ++s) {
      if (rbm[s] > 0) prev_data = col[s];
      if (rbm[s] == 1) prev_mask = pidx[hr * nk + col[s]];
      if (rdn[s] < 0) rdn[s] = prev_data;
      if (rmn[s] < 0) rmn[s] = prev_mask;
    }
  }

  // 6. Downcast.
  fill_index_array(m.arr[SPLASH_MI_BLOCK_MASK], bm, hm, nq, width, downcast);
  fill_index_array(m.arr[SPLASH_MI_DATA_NEXT], dn, hm, nq, width, downcast);
  if (dense) {
    fill_index_array(m.arr[SPLASH_MI_MASK_NEXT], mn, hm, nq, width, downcast);
    HostArray &p = m.arr[SPLASH_MI_PARTIAL_BLOCKS];
    p.present = true;
    p.elem_bits = 8;
    p.is_signed = false;
    p.ndim = 3;
    p.shape[0] = n_partial;
    p.shape[1] = bq;
    p.shape[2] = bk;
    p.bytes = std::move(stack);
  } else {
    // 7. q_sequence: the query positions the kernel recomputes the mask from.
    HostArray &qs = m.arr[SPLASH_MI_Q_SEQUENCE];
    qs.present = true;
    qs.elem_bits = 32;
    qs.is_signed = true;
    qs.ndim = 1;
    qs.shape[0] = m.q_len;
    std::vector<int64_t> seq(static_cast<size_t>(m.q_len));
    std::iota(seq.begin(), seq.end(), 0);
    store_as<int32_t>(qs, seq);
  }

  // Launch order: longest block rows first.
  std::vector<int64_t> row_work(static_cast<size_t>(nq), 0);
  for (int64_t h = 0; h < hm; ++h)
    for (int64_t r = 0; r < nq; ++r)
      for (int64_t c = 0; c < nk; ++c) row_work[r] += label[(h * nq + r) * nk + c] > 0;
  m.row_order.resize(static_cast<size_t>(nq));
  std::iota(m.row_order.begin(), m.row_order.end(), 0);
  std::stable_sort(m.row_order.begin(), m.row_order.end(),
                   [&](int32_t a, int32_t b) { return row_work[a] > row_work[b]; });
}

}  // namespace
}  // namespace splash

namespace splash {
namespace {

splash_status make_impl(const splash_mask_desc *mask, int64_t kv_start, int64_t kv_count,
                        int32_t block_q, int32_t block_kv, uint32_t flags, splash_mask_info **out) {
  if (!out) return fail(SPLASH_EINVAL, "out is NULL");
  *out = nullptr;
  splash_status st = validate(mask, block_q, block_kv);
  if (st != SPLASH_OK) return st;
  if (kv_start < 0 || kv_count < 0 || kv_start > mask->kv_len || kv_count > mask->kv_len - kv_start)
    return fail(SPLASH_EINVAL, "key slice lies outside [0, kv_len)");
  if (kv_start % block_kv || kv_count % block_kv)
    return fail(SPLASH_EINVAL, "block_kv must divide the key slice's start and length");
  if (flags & ~static_cast<uint32_t>(SPLASH_FLAG_SHRINK | SPLASH_FLAG_DOWNCAST))
    return fail(SPLASH_EINVAL, "unknown flag bits");
  splash_mask_info *m = new (std::nothrow) splash_mask_info();
  if (!m) return fail(SPLASH_ENOMEM, "out of host memory");
  m->kind = mask->kind;
  m->num_heads = mask->num_heads;
  m->q_len = mask->q_len;
  m->kv_len = kv_count;
  m->kv_offset = kv_start;
  m->kv_total = mask->kv_len;
  m->left = mask->kind == SPLASH_MASK_LOCAL ? mask->left : -1;
  m->right = mask->kind == SPLASH_MASK_LOCAL ? mask->right : -1;
  m->chunk = mask->kind == SPLASH_MASK_CHUNKED_CAUSAL ? mask->chunk : 0;
  m->block_q = block_q;
  m->block_kv = block_kv;
  m->nq = mask->q_len / block_q;
  m->nk = kv_count / block_kv;
  m->flags = flags;
  try {
    compile(*m, *mask);
  } catch (const std::bad_alloc &) {
    delete m;
    return fail(SPLASH_ENOMEM, "out of host memory while compiling the mask");
  } catch (...) {
    delete m;
    return fail(SPLASH_EINVAL, "mask compilation failed");
  }
  *out = m;
  return SPLASH_OK;
}

}  // namespace
}  // namespace splash

extern "C" SPLASH_API splash_status splash_make_mask_info(const splash_mask_desc *mask,
                                                          int32_t block_q, int32_t block_kv,
                                                          uint32_t flags, splash_mask_info **out) {
  splash::clear_error();
  return splash::make_impl(mask, 0, mask ? mask->kv_len : 0, block_q, block_kv, flags, out);
}

extern "C" SPLASH_API splash_status splash_make_mask_info_kv_slice(const splash_mask_desc *mask,
                                                                   int64_t kv_start, int64_t kv_count,
                                                                   int32_t block_q, int32_t block_kv,
                                                                   uint32_t flags,
                                                                   splash_mask_info **out) {
  splash::clear_error();
  if (!mask) {
    if (out) *out = nullptr;
    return splash::fail(SPLASH_EINVAL, "mask descriptor is NULL");
  }
  return splash::make_impl(mask, kv_start, kv_count, block_q, block_kv, flags, out);
}

extern "C" SPLASH_API splash_status splash_mask_info_view(const splash_mask_info *mi, int32_t which,
                                                          splash_array_view *view) {
  using namespace splash;
  clear_error();
  if (!mi || !view) return fail(SPLASH_EINVAL, "NULL argument");
  if (which < 0 || which >= kNumArrays) return fail(SPLASH_EINVAL, "unknown MaskInfo array id");
  const HostArray &a = mi->arr[which];
  std::memset(view, 0, sizeof(*view));
  if (!a.present) return SPLASH_OK;
  view->elem_bits = a.elem_bits;
  view->is_signed = a.is_signed ? 1 : 0;
  view->ndim = a.ndim;
  for (int i = 0; i < 3; ++i) view->shape[i] = a.shape[i];
  static const uint8_t kEmpty = 0;
  view->data = a.bytes.empty() ? static_cast<const void *>(&kEmpty) : a.bytes.data();
  return SPLASH_OK;
}
