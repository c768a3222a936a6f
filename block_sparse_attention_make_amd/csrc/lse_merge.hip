// Merge of two attention results over disjoint key sets (ring attention on
// the splash-attention explainer page, FAQ "What does ring attention add on
// top of the splash kernel?"): each part carries its own log-sum-exp, and
// the union's result is
//   lse = log(e^lse_a + e^lse_b),  o = e^(lse_a - lse) o_a + e^(lse_b - lse) o_b.
// A part whose lse is -inf (no allowed key in that shard) contributes
// nothing whatever its output holds (selected out, not multiplied by 0), as
// the tokamax variant zeroes inactive shards.  Rows with both parts empty
// give o = 0, lse = -inf.
//
// HBM-bound elementwise work: each thread moves 8 consecutive elements of
// one row with 16- or 32-byte accesses; the Dv / 8 threads of a row sit in
// one wavefront, so the row's lse is read by all of them before any store
// and the output may overwrite part a (or b) in place.  Every element is
// read and written once, with non-temporal loads and stores.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "lse_merge.h"

namespace splash {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct Eight { float x[8]; };

__device__ __forceinline__ Eight load8(const float *p) {
  const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
  const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + 4));
  return Eight{{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}};
}
__device__ __forceinline__ Eight load8(const __bf16 *p) {
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  Eight r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.x[2 * i] = __uint_as_float(w[i] << 16);
    r.x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
  return r;
}
__device__ __forceinline__ void store8(float *p, const Eight &v) {
  __builtin_nontemporal_store(f32x4{v.x[0], v.x[1], v.x[2], v.x[3]}, reinterpret_cast<f32x4 *>(p));
  __builtin_nontemporal_store(f32x4{v.x[4], v.x[5], v.x[6], v.x[7]}, reinterpret_cast<f32x4 *>(p + 4));
}
__device__ __forceinline__ void store8(__bf16 *p, const Eight &v) {
  union { __bf16 h[8]; u32x4 u; } pk;
#pragma unroll
  for (int i = 0; i < 8; ++i) pk.h[i] = static_cast<__bf16>(v.x[i]);
  __builtin_nontemporal_store(pk.u, reinterpret_cast<u32x4 *>(p));
}

// A row's dv / 8 chunks go to tpr threads (dv / 8 rounded up to a power of
// two, at most 64), so a row never straddles two wavefronts: in an in-place
// merge every thread of a row reads its lse before any of them writes it.
template <typename TA, typename TB, typename TO>
__global__ void __launch_bounds__(256) lse_merge_kernel(const TA *oa, const float *la, const TB *ob,
                                                        const float *lb, TO *oo, float *lo, int64_t rows,
                                                        int dv, int tpr) {
  const int64_t n_threads = rows * tpr;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < n_threads;
       t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = t / tpr;
    const int c = static_cast<int>(t % tpr);
    if (c * 8 >= dv) continue;   // a padding thread of the row
    const int64_t e0 = row * dv + c * 8;
    const float a = la[row], b = lb[row];
    const bool ha = a > -INFINITY, hb = b > -INFINITY;
    float l;
    if (ha && hb) {
      const float m = fmaxf(a, b);
      l = m + log1pf(expf(-fabsf(a - b)));
    } else {
      l = ha ? a : (hb ? b : -INFINITY);
    }
    const float wa = ha ? expf(a - l) : 0.f;
    const float wb = hb ? expf(b - l) : 0.f;
    Eight r;
    const Eight va = ha ? load8(oa + e0) : Eight{};
    const Eight vb = hb ? load8(ob + e0) : Eight{};
#pragma unroll
    for (int i = 0; i < 8; ++i) r.x[i] = (ha ? wa * va.x[i] : 0.f) + (hb ? wb * vb.x[i] : 0.f);
    store8(oo + e0, r);
    if (c == 0) lo[row] = l;
  }
}

template <typename TA, typename TB, typename TO>
hipError_t go(const void *oa, const float *la, const void *ob, const float *lb, void *oo, float *lo,
              int64_t rows, int dv, hipStream_t stream) {
  int tpr = 1;
  while (tpr * 8 < dv) tpr *= 2;   // threads per row, a power of two (dv <= 512: at most 64)
  const int64_t n_threads = rows * tpr;
  const int64_t want = (n_threads + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < 65536 ? want : 65536);
  hipLaunchKernelGGL((lse_merge_kernel<TA, TB, TO>), dim3(grid), dim3(256), 0, stream,
                     static_cast<const TA *>(oa), la, static_cast<const TB *>(ob), lb, static_cast<TO *>(oo), lo,
                     rows, dv, tpr);
  return hipGetLastError();
}

template <typename TA, typename TB>
hipError_t go_out(int dto, const void *oa, const float *la, const void *ob, const float *lb, void *oo, float *lo,
                  int64_t rows, int dv, hipStream_t s) {
  return dto == 0 ? go<TA, TB, __bf16>(oa, la, ob, lb, oo, lo, rows, dv, s)
                  : go<TA, TB, float>(oa, la, ob, lb, oo, lo, rows, dv, s);
}

template <typename TA>
hipError_t go_b(int dtb, int dto, const void *oa, const float *la, const void *ob, const float *lb, void *oo,
                float *lo, int64_t rows, int dv, hipStream_t s) {
  return dtb == 0 ? go_out<TA, __bf16>(dto, oa, la, ob, lb, oo, lo, rows, dv, s)
                  : go_out<TA, float>(dto, oa, la, ob, lb, oo, lo, rows, dv, s);
}

}  // namespace

hipError_t launch_lse_merge(const void *oa, const float *la, int dta, const void *ob, const float *lb, int dtb,
                            void *oo, float *lo, int dto, int64_t rows, int dv, hipStream_t stream) {
  return dta == 0 ? go_b<__bf16>(dtb, dto, oa, la, ob, lb, oo, lo, rows, dv, stream)
                  : go_b<float>(dtb, dto, oa, la, ob, lb, oo, lo, rows, dv, stream);
}

}  // namespace splash
