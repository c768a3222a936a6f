// Splash-attention backward for gfx950 (CDNA4), bf16.
//
// The backward the pages give for flash attention (pallas flash attention on
// TPU page, FAQ "What does the TPU flash attention kernel save for the
// backward pass?" and "Why does the TPU flash attention backward pass run two
// kernels instead of one?"), walked block-sparsely like the forward:
//   * the attention weights are not saved: each kernel recomputes the scores
//     from q and k and rebuilds p = exp(s' - lse) from the forward's per-row
//     log-sum-exp;
//   * di = <dout_i, out_i> is formed once, before both kernels (delta);
//   * the key/value gradients are sums over query blocks and the query
//     gradient a sum over key blocks, so there are two launches with opposite
//     loop orders: a key-major one (a workgroup per key block, looping over
//     the query blocks -- of every query head of the GQA group -- that the
//     mask lets see it, from the transposed block lists) and a query-major
//     one (a workgroup per query block, looping over the MaskInfo row);
//   * label 0 blocks are never visited, label 2 blocks are never masked.
// With s = q.k, s' = scale s (or c tanh(scale s / c) under a soft cap):
//   dv_j = sum_i p_ij do_i,  dp_ij = <do_i, v_j>,  ds_ij = p_ij (dp_ij - di_i) g_ij
//   (g = 1, or 1 - tanh^2 under the cap),  dq_i = scale sum_j ds_ij k_j,
//   dk_j = scale sum_i ds_ij q_i.
//
// MI355X mapping.  Four waves per workgroup, 32 rows (keys or queries) per
// wave, the 32x32x16 bf16 MFMA.  The wave's fixed operands (its keys' K and V
// in the key-major kernel, its queries' Q and dO in the query-major one) sit
// in registers as B operands; the streamed 128-row tiles are staged in LDS
// (XOR-swizzled 16-byte chunks) and read both as row A operands
// (ds_read_b128) and transposed (ds_read_b64_tr_b16) for the products that
// contract over their rows.  Gradients accumulate transposed (dK^T, dV^T,
// dQ^T) in fp32 registers, with p and ds fed from the score registers as B
// operands, as the forward does with P.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "splash_kernel.h"

namespace splash {
namespace {

constexpr int kBlk = 128;        // rows of a mask block (queries and keys)
constexpr int kThreads = 256;    // 4 waves x 32 rows
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int load_index(const void *p, int bytes, int64_t i) {
  if (bytes == 1) return static_cast<const int8_t *>(p)[i];
  if (bytes == 2) return static_cast<const int16_t *>(p)[i];
  return static_cast<const int32_t *>(p)[i];
}

// A 128 x D bf16 tile in LDS; 16-byte chunk c of row r sits at chunk
// c ^ swz(r), which spreads the row reads of 16 consecutive rows over all
// banks and keeps the transposing reads (4 rows x 4 chunks) apart too.
template <int D>
struct BTile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kBytes = kBlk * kRowBytes;
  __device__ static int swz(int row) {
    if constexpr (kChunks >= 16) return row & 15;
    else return (row >> 1) & 7;
  }
};

// Stage rows [0, 128) of a row-major [*, D] bf16 array into a tile.
template <int D>
__device__ __forceinline__ void stage(char *lds, const __bf16 *g, int tid) {
  using T = BTile<D>;
  constexpr int kPer = kBlk * T::kChunks / kThreads;
  u32x4 buf[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx / T::kChunks, c = idx % T::kChunks;
    buf[i] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(g) +
                                              static_cast<size_t>(row) * T::kRowBytes + c * 16);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx / T::kChunks, c = idx % T::kChunks;
    *reinterpret_cast<u32x4 *>(lds + row * T::kRowBytes + ((c ^ T::swz(row)) * 16)) = buf[i];
  }
}

// Row A operand of a 32x32x16 MFMA: row `row` of the tile, k-step ks.
template <int D>
__device__ __forceinline__ bf16x8 read_row(const char *lds, int row, int ks, int half) {
  using T = BTile<D>;
  return *reinterpret_cast<const bf16x8 *>(lds + row * T::kRowBytes + (((2 * ks + half) ^ T::swz(row)) * 16));
}

// Transposed A operand: the tile's columns 32 dt .. 32 dt + 31 as rows,
// contracted over tile rows r0 + 16 h + {4 half + 0..3, 8 + 4 half + 0..3} --
// the order in which a 32x32 score tile holds its rows in one lane's
// elements 8 h .. 8 h + 7, so these pair with B operands built from them.
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const char *lds, int r0, int h, int dt, int lane, int half) {
  using T = BTile<D>;
  const int trow = 4 * half + ((lane & 15) >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int row0 = r0 + 16 * h + trow;
  const int col = 32 * dt + tcol;
  const int c = col >> 3, within = (col & 7) * 2;
  const char *a0 = lds + row0 * T::kRowBytes + ((c ^ T::swz(row0)) * 16) + within;
  const char *a1 = lds + (row0 + 8) * T::kRowBytes + ((c ^ T::swz(row0 + 8)) * 16) + within;
  const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3))) *)(a0));
  const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3))) *)(a1));
  const s16x4 both[2] = {lo4, hi4};
  bf16x8 r;
  __builtin_memcpy(&r, both, 16);
  return r;
}

// B operands of a row block kept in registers: lane (j, half) holds row
// row0 + j, elements 16 ks + 8 half .. + 7.
template <int D>
__device__ __forceinline__ void load_rows_b(bf16x8 (&dst)[D / 16], const __bf16 *g, int lane, int half) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    dst[ks] = *reinterpret_cast<const bf16x8 *>(g + static_cast<int64_t>(lane & 31) * D + 16 * ks + 8 * half);
}

// Soft-cap pieces of one score: base-2 capped logit and the derivative
// factor 1 - tanh^2.
__device__ __forceinline__ void capped(float x, float c2, float cap_out, float &s2, float &g) {
  const float xs = x * c2;
  const float e = __builtin_amdgcn_exp2f(-2.f * kLog2e * fabsf(xs));
  const float th = (1.f - e) * __builtin_amdgcn_rcpf(1.f + e);
  const float t = copysignf(th, xs);
  s2 = t * cap_out;
  g = 1.f - t * t;
}

// Store a transposed fp32 accumulator (rows d, columns = the wave's 32 rows)
// as rows of a [*, D] bf16 array, times `mul`.
template <int D>
__device__ __forceinline__ void store_t(__bf16 *g, const f32x16 (&acc)[D / 32], float mul, int lane, int half) {
  __bf16 *row = g + static_cast<int64_t>(lane & 31) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      union { __bf16 h[4]; u32x2 u; } pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk.h[e] = static_cast<__bf16>(acc[dt][4 * q4 + e] * mul);
      *reinterpret_cast<u32x2 *>(row + 32 * dt + 8 * q4 + 4 * half) = pk.u;
    }
}

// ---- delta: di = <dout_i, out_i> ------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_delta(const __bf16 *o, const __bf16 *dout, float *delta, int64_t rows) {
  constexpr int kPerRow = D / 8;   // threads per row, 8 elements each
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = t / kPerRow;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(o + t * 8);
    const u32x4 b = *reinterpret_cast<const u32x4 *>(dout + t * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += __uint_as_float(a[i] << 16) * __uint_as_float(b[i] << 16);
      acc += __uint_as_float(a[i] & 0xffff0000u) * __uint_as_float(b[i] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int m = kPerRow / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && (t % kPerRow) == 0) delta[row] = acc;
}

// ---- key-major kernel: dK, dV ---------------------------------------------
// Workgroup (b, hkv, key block c); wave w owns keys 32 w .. 32 w + 31.
template <int D, bool CAP, bool DENSE>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv(const BwdParams p) {
  using T = BTile<D>;
  constexpr int kKS = D / 16, kDT = D / 32;
  __shared__ __attribute__((aligned(16))) char q_t[T::kBytes];
  __shared__ __attribute__((aligned(16))) char do_t[T::kBytes];
  __shared__ __attribute__((aligned(16))) float lse_s[kBlk], di_s[kBlk];
  __shared__ __attribute__((aligned(16))) int lo_s[kBlk], hi_s[kBlk];
  __shared__ __attribute__((aligned(16))) unsigned mw_s[4 * kBlk];

  const FwdParams &f = p.f;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pid = blockIdx.x;
  const int c = pid % p.nk;
  const int bh = pid / p.nk;
  const int b = bh / static_cast<int>(f.Hkv), hkv = bh % static_cast<int>(f.Hkv);
  const int64_t key0 = static_cast<int64_t>(c) * kBlk + 32 * wave;   // the wave's first key
  const int64_t kv_off = ((static_cast<int64_t>(b) * f.Hkv + hkv) * f.Skv + key0) * D;

  bf16x8 kb[kKS], vb[kKS];
  load_rows_b<D>(kb, static_cast<const __bf16 *>(f.k) + kv_off, lane, half);
  load_rows_b<D>(vb, static_cast<const __bf16 *>(f.v) + kv_off, lane, half);
  f32x16 dk[kDT], dv[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) dk[dt][v] = dv[dt][v] = 0.f;

  const int key_local = 32 * wave + (lane & 31);   // key of this lane's S column, within the block
  for (int g = 0; g < f.group; ++g) {
    const int hq = hkv * f.group + g;
    const int hm = f.hm == 1 ? 0 : hq;
    const int64_t lst = static_cast<int64_t>(hm) * p.nk + c;
    const int n = p.col_n[lst];
    for (int e = 0; e < n; ++e) {
      const int ent = p.col_ent[lst * p.col_w + e];
      const int r = ent & 0x3fffffff, label = static_cast<int>(static_cast<unsigned>(ent) >> 30);
      const int64_t row_base = (static_cast<int64_t>(b) * f.Hq + hq) * f.Sq + static_cast<int64_t>(r) * kBlk;
      __syncthreads();   // the previous block's tiles are no longer read
      stage<D>(q_t, static_cast<const __bf16 *>(f.q) + row_base * D, tid);
      stage<D>(do_t, static_cast<const __bf16 *>(p.dout) + row_base * D, tid);
      if (tid < kBlk) {
        const float l = f.lse[row_base + tid];
        lse_s[tid] = l * kLog2e;
        di_s[tid] = p.delta[row_base + tid];
        if constexpr (!DENSE) {
          const int64_t qpos = f.q_seq[static_cast<int64_t>(r) * kBlk + tid];
          const int64_t big = int64_t(1) << 40;
          int64_t lo, hi;
          if (f.mask_kind == 0) { lo = -big; hi = qpos; }
          else if (f.mask_kind == 1) { lo = f.left < 0 ? -big : qpos - f.left; hi = f.right < 0 ? big : qpos + f.right; }
          else { lo = (qpos / f.chunk) * f.chunk; hi = qpos; }
          // relative to this key block's first key (in the MaskInfo's key coordinates)
          const int64_t kb0 = f.kv_offset + static_cast<int64_t>(c) * kBlk;
          lo -= kb0;
          hi -= kb0;
          lo_s[tid] = static_cast<int>(lo < -1 ? -1 : (lo > kBlk ? kBlk : lo));
          hi_s[tid] = static_cast<int>(hi < -1 ? -1 : (hi > kBlk ? kBlk : hi));
        }
      }
      if constexpr (DENSE) {
        if (label == 1) {
          const int mn = p.col_mn[lst * p.col_w + e];
          for (int i = tid; i < 4 * kBlk; i += kThreads) mw_s[i] = f.pmb_bits[static_cast<int64_t>(mn) * 4 * kBlk + i];
        }
      }
      __syncthreads();

#pragma unroll 1
      for (int qb = 0; qb < 4; ++qb) {
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
          const bf16x8 aq = read_row<D>(q_t, 32 * qb + (lane & 31), ks, half);
          const bf16x8 ad = read_row<D>(do_t, 32 * qb + (lane & 31), ks, half);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kb[ks], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, vb[ks], dp, 0, 0, 0);
        }
        bf16x8 pb[2], sb[2];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int qi0 = 32 * qb + 8 * g4 + 4 * half;   // rows of elements 4 g4 .. 4 g4 + 3
          const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&lse_s[qi0]);
          const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&di_s[qi0]);
          unsigned mword[4] = {0u, 0u, 0u, 0u};
          int lo4[4] = {0, 0, 0, 0}, hi4[4] = {0, 0, 0, 0};
          if (label == 1) {
            if constexpr (DENSE) {
#pragma unroll
              for (int k = 0; k < 4; ++k) mword[k] = mw_s[wave * kBlk + qi0 + k];
            } else {
#pragma unroll
              for (int k = 0; k < 4; ++k) { lo4[k] = lo_s[qi0 + k]; hi4[k] = hi_s[qi0 + k]; }
            }
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int v = 4 * g4 + k;
            float s2, gf = 1.f;
            if constexpr (CAP) capped(s[v], f.c2, f.cap_out, s2, gf);
            else s2 = s[v] * f.c2;
            bool ok = l4[k] != -INFINITY;
            if (label == 1) {
              if constexpr (DENSE) ok = ok && ((mword[k] >> (lane & 31)) & 1u);
              else ok = ok && key_local >= lo4[k] && key_local <= hi4[k];
            }
            const float pv = ok ? __builtin_amdgcn_exp2f(s2 - l4[k]) : 0.f;
            const float dsv = pv * (dp[v] - d4[k]) * gf;
            pb[v / 8][v % 8] = static_cast<__bf16>(pv);
            sb[v / 8][v % 8] = static_cast<__bf16>(dsv);
          }
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int dt = 0; dt < kDT; ++dt) {
            const bf16x8 ado = read_tr<D>(do_t, 32 * qb, h2, dt, lane, half);
            const bf16x8 aq = read_tr<D>(q_t, 32 * qb, h2, dt, lane, half);
            dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ado, pb[h2], dv[dt], 0, 0, 0);
            dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, sb[h2], dk[dt], 0, 0, 0);
          }
      }
    }
  }
  store_t<D>(static_cast<__bf16 *>(p.dk) + kv_off, dk, p.scale, lane, half);
  store_t<D>(static_cast<__bf16 *>(p.dv) + kv_off, dv, 1.f, lane, half);
}

// ---- query-major kernel: dQ -----------------------------------------------
// Workgroup (b, hq, query block r); wave w owns queries 32 w .. 32 w + 31.
template <int D, bool CAP, bool DENSE>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq(const BwdParams p) {
  using T = BTile<D>;
  constexpr int kKS = D / 16, kDT = D / 32;
  __shared__ __attribute__((aligned(16))) char k_t[T::kBytes];
  __shared__ __attribute__((aligned(16))) char v_t[T::kBytes];
  __shared__ __attribute__((aligned(16))) unsigned mw_s[4 * kBlk];

  const FwdParams &f = p.f;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pid = blockIdx.x;
  const int r = pid % f.nq;
  const int bh = pid / f.nq;
  const int b = bh / static_cast<int>(f.Hq), hq = bh % static_cast<int>(f.Hq);
  const int hkv = hq / f.group;
  const int hm = f.hm == 1 ? 0 : hq;
  const int64_t q_row = static_cast<int64_t>(r) * kBlk + 32 * wave + (lane & 31);   // this lane's query
  const int64_t row_base = (static_cast<int64_t>(b) * f.Hq + hq) * f.Sq;
  const int64_t q0 = (row_base + static_cast<int64_t>(r) * kBlk + 32 * wave) * D;

  bf16x8 qb[kKS], dob[kKS];
  load_rows_b<D>(qb, static_cast<const __bf16 *>(f.q) + q0, lane, half);
  load_rows_b<D>(dob, static_cast<const __bf16 *>(p.dout) + q0, lane, half);
  const float l_raw = f.lse[row_base + q_row];
  const float lse2 = l_raw * kLog2e;
  const float di = p.delta[row_base + q_row];
  int64_t lo = 0, hi = 0;
  if constexpr (!DENSE) {
    const int64_t qpos = f.q_seq[q_row];
    const int64_t big = int64_t(1) << 40;
    if (f.mask_kind == 0) { lo = -big; hi = qpos; }
    else if (f.mask_kind == 1) { lo = f.left < 0 ? -big : qpos - f.left; hi = f.right < 0 ? big : qpos + f.right; }
    else { lo = (qpos / f.chunk) * f.chunk; hi = qpos; }
    lo -= f.kv_offset;
    hi -= f.kv_offset;
  }
  f32x16 dq[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) dq[dt][v] = 0.f;

  const int64_t kv_base = (static_cast<int64_t>(b) * f.Hkv + hkv) * f.Skv;
  const int64_t meta = (static_cast<int64_t>(hm) * f.nq + r) * f.width;
  for (int sl = 0; sl < f.width; ++sl) {
    const int label = load_index(f.bm, f.bm_bytes, meta + sl);
    if (label == 0) continue;
    const int c = load_index(f.dn, f.dn_bytes, meta + sl);
    __syncthreads();
    stage<D>(k_t, static_cast<const __bf16 *>(f.k) + (kv_base + static_cast<int64_t>(c) * kBlk) * D, tid);
    stage<D>(v_t, static_cast<const __bf16 *>(f.v) + (kv_base + static_cast<int64_t>(c) * kBlk) * D, tid);
    if constexpr (DENSE) {
      if (label == 1) {
        const int mn = load_index(f.mn, f.mn_bytes, meta + sl);
        for (int i = tid; i < 4 * kBlk; i += kThreads) mw_s[i] = f.pmb_bits[static_cast<int64_t>(mn) * 4 * kBlk + i];
      }
    }
    __syncthreads();
    const int64_t kbase = static_cast<int64_t>(c) * kBlk;
#pragma unroll 1
    for (int kb4 = 0; kb4 < 4; ++kb4) {
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const bf16x8 ak = read_row<D>(k_t, 32 * kb4 + (lane & 31), ks, half);
        const bf16x8 av = read_row<D>(v_t, 32 * kb4 + (lane & 31), ks, half);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qb[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, dob[ks], dp, 0, 0, 0);
      }
      unsigned mword = 0u;
      if constexpr (DENSE) {
        if (label == 1) mword = mw_s[kb4 * kBlk + 32 * wave + (lane & 31)];
      }
      bf16x8 sb[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kl = 32 * kb4 + 8 * (v / 4) + 4 * half + (v % 4);   // key within the block
        float s2, gf = 1.f;
        if constexpr (CAP) capped(s[v], f.c2, f.cap_out, s2, gf);
        else s2 = s[v] * f.c2;
        bool ok = lse2 != -INFINITY;
        if (label == 1) {
          if constexpr (DENSE) ok = ok && ((mword >> (kl & 31)) & 1u);
          else ok = ok && kbase + kl >= lo && kbase + kl <= hi;
        }
        const float pv = ok ? __builtin_amdgcn_exp2f(s2 - lse2) : 0.f;
        sb[v / 8][v % 8] = static_cast<__bf16>(pv * (dp[v] - di) * gf);
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          const bf16x8 ak = read_tr<D>(k_t, 32 * kb4, h2, dt, lane, half);
          dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, sb[h2], dq[dt], 0, 0, 0);
        }
    }
  }
  store_t<D>(static_cast<__bf16 *>(p.dq) + q0, dq, p.scale, lane, half);
}

template <int D, bool CAP, bool DENSE>
hipError_t go(const BwdParams &p, hipStream_t stream) {
  const FwdParams &f = p.f;
  const int64_t nkv = f.B * f.Hkv * p.nk;
  if (nkv > 0)
    hipLaunchKernelGGL((bwd_dkdv<D, CAP, DENSE>), dim3(static_cast<unsigned>(nkv)), dim3(kThreads), 0, stream, p);
  const int64_t nq = f.B * f.Hq * f.nq;
  if (nq > 0)
    hipLaunchKernelGGL((bwd_dq<D, CAP, DENSE>), dim3(static_cast<unsigned>(nq)), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t go_d(const BwdParams &p, hipStream_t stream) {
  const FwdParams &f = p.f;
  const int64_t rows = f.B * f.Hq * f.Sq;
  if (rows > 0) {
    const int64_t threads = rows * (D / 8);
    hipLaunchKernelGGL((bwd_delta<D>), dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const __bf16 *>(f.out), static_cast<const __bf16 *>(p.dout), p.delta, rows);
  }
  if (f.cap) return f.dense ? go<D, true, true>(p, stream) : go<D, true, false>(p, stream);
  return f.dense ? go<D, false, true>(p, stream) : go<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdParams &p, hipStream_t stream) {
  return p.f.D == 64 ? go_d<64>(p, stream) : go_d<128>(p, stream);
}

}  // namespace splash
