// Splash-attention forward kernel for gfx950 (CDNA4).
//
// What it computes is masked softmax attention (splash-attention explainer,
// FAQ "What is splash attention and how is it different from flash
// attention?"); how it walks the work comes from the compiled MaskInfo
// (FAQ "What is MaskInfo in splash attention?", "What does grid shrinking do
// in splash attention?"):
//   * one workgroup per (batch, query head, 128-row query block); its loop
//     runs over the W grid positions of that block row;
//   * label 0: nothing runs and no key/value bytes are fetched;
//   * label 2: the block is computed with no mask at all;
//   * label 1: the block is computed and masked -- computable masks are
//     recomputed from q_sequence and the key position, dense masks read the
//     partial block mask_next points at;
//   * data_next names the key/value block to fetch at each position.
// The softmax is the flash online softmax: a running max and running sum per
// query row, the accumulator rescaled whenever the max moves, one division by
// the final sum at the end, and the log-sum-exp kept as the per-row residual.
//
// MI355X mapping.  Four 64-lane waves per workgroup, each owning 32 query
// rows.  Scores are formed transposed, S^T = K Q^T, with the 32x32x16 bf16
// MFMA (32x32x2 f32 for float inputs): Q stays in registers as the B operand
// and K streams from LDS as the A operand.  In that output layout every lane
// holds one query row (lane % 32) and 16 of its keys per 32-key tile, so a
// row max or row sum is a per-lane reduction plus one v_permlane32_swap with
// the partner lane (lane ^ 32).  The output is accumulated transposed too,
// O^T = V^T P^T: P goes straight from the score registers into the B
// operand, and V^T comes out of the row-major V tile with the gfx950
// transposing LDS read ds_read_b64_tr_b16, so neither P nor V is shuffled.
// K and V tiles (128 x D) are staged through LDS with XOR-swizzled 16-byte
// chunks so that the staging writes, the K operand reads and the transposing
// V reads are bank-conflict free.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "splash_kernel.h"

namespace splash {
namespace {

constexpr int kBQ = 128;        // query rows per workgroup (= mask block rows)
constexpr int kBK = 128;        // keys per grid step (= mask block columns)
constexpr int kThreads = 256;   // 4 waves
constexpr int kMetaChunk = 256; // grid positions of metadata staged in LDS at a time
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int64_t clamp64(int64_t x, int64_t a, int64_t b) {
  return x < a ? a : (x > b ? b : x);
}

__device__ __forceinline__ int load_index(const void *p, int bytes, int64_t i) {
  if (bytes == 1) return static_cast<const int8_t *>(p)[i];
  if (bytes == 2) return static_cast<const int16_t *>(p)[i];
  return static_cast<const int32_t *>(p)[i];
}

// Tile geometry and swizzles.  A tile is 128 rows of D elements; a row is
// split into 16-byte chunks whose index is XORed with swz(row).
template <typename T, int D>
struct Tile {
  static constexpr int kRowBytes = D * static_cast<int>(sizeof(T));
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kBytes = kBK * kRowBytes;
  // K tile: the A-operand read has 16 consecutive lanes on 16 consecutive
  // rows at one chunk.
  __device__ static int swz_k(int row) {
    if constexpr (kChunks >= 16) return row & 15;
    else return (row >> 1) & 7;
  }
  // V tile: the transposing read has 32 lanes on 4 consecutive rows x 4
  // chunks (bf16); the f32 read has 32 lanes on one row.
  __device__ static int swz_v(int row) {
    if constexpr (sizeof(T) == 2) {
      if constexpr (kChunks >= 16) return (row & 3) << 2;
      else return ((row >> 1) & 1) << 2;
    } else {
      return row & 15;
    }
  }
};

// Copy one 128 x D tile from global memory (rows contiguous, D elements each)
// into a swizzled LDS tile.  Each lane moves 16-byte chunks; 16 lanes cover
// one 256-byte span of a row, so the global reads are fully coalesced.
template <typename T, int D, bool IS_V>
__device__ __forceinline__ void stage_tile(char *lds, const T *g, int tid) {
  using TL = Tile<T, D>;
  constexpr int kPerThread = kBK * TL::kChunks / kThreads;
  u32x4 buf[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx / TL::kChunks, c = idx % TL::kChunks;
    buf[i] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(g) +
                                              static_cast<size_t>(row) * TL::kRowBytes + c * 16);
  }
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx / TL::kChunks, c = idx % TL::kChunks;
    const int pc = c ^ (IS_V ? TL::swz_v(row) : TL::swz_k(row));
    *reinterpret_cast<u32x4 *>(lds + row * TL::kRowBytes + pc * 16) = buf[i];
  }
}

template <typename T, int D, bool CAP, bool DENSE>
__global__ __launch_bounds__(kThreads, (sizeof(T) == 2 || D == 64) ? 2 : 1)
void splash_fwd_kernel(const FwdParams p) {
  using TL = Tile<T, D>;
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int kDT = D / 32;  // 32-wide output tiles along Dv

  __shared__ __attribute__((aligned(16))) char smem[2 * TL::kBytes];
  __shared__ int meta_bm[kMetaChunk], meta_dn[kMetaChunk], meta_mn[kMetaChunk];
  char *lds_k = smem;
  char *lds_v = smem + TL::kBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;         // which half of the wave: keys +0 or +4 in a group of 8
  const int lrow = 32 * wave + (lane & 31);  // query row inside the 128-row block

  // ---- which (batch, head, block row) this workgroup owns ----------------
  // Consecutive workgroup ids go round-robin over the 8 XCDs; give each XCD a
  // contiguous range of (batch, head) pairs so the K/V of those heads (and of
  // a whole GQA group) stay in that XCD's L2, and hand rows out longest-first.
  const int nbh = static_cast<int>(p.B * p.Hq);
  const int pid = blockIdx.x;
  int bh, rank;
  if ((nbh & 7) == 0) {
    const int per = nbh >> 3, x = pid & 7, j = pid >> 3;
    bh = x * per + j % per;
    rank = j / per;
  } else {
    bh = pid % nbh;
    rank = pid / nbh;
  }
  const int r = p.row_order[rank];
  const int b = bh / static_cast<int>(p.Hq);
  const int hq = bh % static_cast<int>(p.Hq);
  const int hkv = hq / p.group;
  const int hm = p.hm == 1 ? 0 : hq;

  const int64_t q_row = static_cast<int64_t>(r) * kBQ + lrow;
  const T *qg = static_cast<const T *>(p.q) + ((static_cast<int64_t>(b) * p.Hq + hq) * p.Sq + q_row) * D;
  const T *kg = static_cast<const T *>(p.k) + (static_cast<int64_t>(b) * p.Hkv + hkv) * p.Skv * D;
  const T *vg = static_cast<const T *>(p.v) + (static_cast<int64_t>(b) * p.Hkv + hkv) * p.Skv * D;

  // ---- Q fragment (B operand of S^T = K Q^T), resident for the whole row ----
  // bf16: k-step ks covers d = 16 ks + 8 half + 0..7.  f32: the lane's half
  // owns d in [half D/2, (half+1) D/2) and k-step ks takes one of them.
  constexpr int kQRegs = kBf16 ? D / 16 : D / 2;
  using QFrag = typename std::conditional<kBf16, bf16x8, float>::type;
  QFrag qf[kQRegs];
  if constexpr (kBf16) {
#pragma unroll
    for (int ks = 0; ks < kQRegs; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8 *>(qg + 16 * ks + 8 * half);
  } else {
#pragma unroll
    for (int i = 0; i < kQRegs / 4; ++i) {
      const float4 x = *reinterpret_cast<const float4 *>(qg + half * (D / 2) + 4 * i);
      qf[4 * i + 0] = x.x; qf[4 * i + 1] = x.y; qf[4 * i + 2] = x.z; qf[4 * i + 3] = x.w;
    }
  }

  // ---- per-row mask interval for computable masks --------------------------
  // Every computable mask admits, for query position i, one interval of keys
  // [lo(i), hi(i)]: causal (-inf, i]; local [i - left, i + right]; chunked
  // causal [chunk start of i, i].
  int64_t lo = 0, hi = 0;
  if constexpr (!DENSE) {
    const int64_t qpos = p.q_seq[q_row];
    const int64_t big = int64_t(1) << 40;
    if (p.mask_kind == 0) { lo = -big; hi = qpos; }
    else if (p.mask_kind == 1) { lo = p.left < 0 ? -big : qpos - p.left; hi = p.right < 0 ? big : qpos + p.right; }
    else { lo = (qpos / p.chunk) * p.chunk; hi = qpos; }
  }

  // ---- running softmax state ----------------------------------------------
  const float c2 = p.c2;                   // score multiplier into base-2 units
  float m_run = -INFINITY;                 // running max (raw score units, or capped base-2 units)
  float l_run = 0.f;                       // this lane's share of the running sum
  f32x16 o[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[dt][v] = 0.f;

  const int64_t meta_base = (static_cast<int64_t>(hm) * p.nq + r) * p.width;

  for (int s0 = 0; s0 < p.width; s0 += kMetaChunk) {
    // Stage this chunk of the block row's MaskInfo entries in LDS.
    const int n_meta = min(kMetaChunk, p.width - s0);
    __syncthreads();
    if (tid < n_meta) {
      meta_bm[tid] = load_index(p.bm, p.bm_bytes, meta_base + s0 + tid);
      meta_dn[tid] = load_index(p.dn, p.dn_bytes, meta_base + s0 + tid);
      if constexpr (DENSE) meta_mn[tid] = load_index(p.mn, p.mn_bytes, meta_base + s0 + tid);
    }
    __syncthreads();

    for (int si = 0; si < n_meta; ++si) {
      const int label = __builtin_amdgcn_readfirstlane(meta_bm[si]);
      if (label == 0) continue;  // empty block: no fetch, no compute
      const int kvb = __builtin_amdgcn_readfirstlane(meta_dn[si]);

      // Dense partial block: this lane's 64 mask bytes, fetched early.
      unsigned mwords[16];
      if constexpr (DENSE) {
        if (label == 1) {
          const int pb = __builtin_amdgcn_readfirstlane(meta_mn[si]);
          const unsigned *mrow = reinterpret_cast<const unsigned *>(
              p.pmb + (static_cast<int64_t>(pb) * kBQ + lrow) * kBK);
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) mwords[4 * t + g] = mrow[8 * t + 2 * g + half];
        }
      }

      // ---- stage K and V of block kvb ----
      __syncthreads();
      stage_tile<T, D, false>(lds_k, kg + static_cast<int64_t>(kvb) * kBK * D, tid);
      stage_tile<T, D, true>(lds_v, vg + static_cast<int64_t>(kvb) * kBK * D, tid);
      __syncthreads();

      // ---- S^T = K Q^T: four 32-key tiles ----
      f32x16 sc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[t][v] = 0.f;
      if constexpr (kBf16) {
#pragma unroll
        for (int ks = 0; ks < kQRegs; ++ks)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int row = 32 * t + (lane & 31);
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                lds_k + row * TL::kRowBytes + (((2 * ks + half) ^ TL::swz_k(row)) * 16));
            sc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sc[t], 0, 0, 0);
          }
      } else {
#pragma unroll
        for (int i = 0; i < kQRegs / 4; ++i)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int row = 32 * t + (lane & 31);
            const int c = (half * (D / 2) + 4 * i) / 4;
            const float4 a = *reinterpret_cast<const float4 *>(
                lds_k + row * TL::kRowBytes + ((c ^ TL::swz_k(row)) * 16));
            sc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, qf[4 * i + 0], sc[t], 0, 0, 0);
            sc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, qf[4 * i + 1], sc[t], 0, 0, 0);
            sc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, qf[4 * i + 2], sc[t], 0, 0, 0);
            sc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, qf[4 * i + 3], sc[t], 0, 0, 0);
          }
      }

      // Lane holds, for query lrow, keys kvb*128 + 32t + 8(v/4) + 4*half + v%4.
      float c2e = c2;
      if constexpr (CAP) {
        // capped logit in base-2 units: cap*log2e * tanh(score * scale / cap)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float x = sc[t][v] * c2;                 // c2 = scale / cap here
            const float e = __builtin_amdgcn_exp2f(-2.f * kLog2e * fabsf(x));
            const float th = (1.f - e) * __builtin_amdgcn_rcpf(1.f + e);
            sc[t][v] = copysignf(th, x) * p.cap_out;
          }
        c2e = 1.f;
      }

      if (label == 1) {
        if constexpr (DENSE) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const unsigned byte = (mwords[4 * t + v / 4] >> (8 * (v % 4))) & 0xffu;
              sc[t][v] = byte ? sc[t][v] : -INFINITY;
            }
        } else {
          const int64_t kbase = static_cast<int64_t>(kvb) * kBK + 4 * half;
          const int rlo = static_cast<int>(clamp64(lo - kbase, -1, 128));
          const int rhi = static_cast<int>(clamp64(hi - kbase, -1, 128));
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int c = 32 * t + 8 * (v / 4) + (v % 4);
              sc[t][v] = (c >= rlo && c <= rhi) ? sc[t][v] : -INFINITY;
            }
        }
      }

      // ---- online softmax ----
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[t][v]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float mb = m_use * c2e;
      const float alpha = __builtin_amdgcn_exp2f(m_run * c2e - mb);
      float rs = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][v], c2e, -mb));
          sc[t][v] = e;
          rs += e;
        }
      l_run = l_run * alpha + rs;
      m_run = m_new;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[dt][v] *= alpha;
      }

      // ---- O^T += V^T P^T ----
      if constexpr (kBf16) {
        bf16x8 pf[4][2];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[t][h][e] = static_cast<__bf16>(sc[t][8 * h + e]);
        // Lane supplies V[key][dv] for dv = 32 dt + lane%32 and the 8 keys
        // 32t + 16h + 4 half + {0..3, 8..11}: two transposing reads, each lane
        // addressing row 32t + 16h + 4 half + (lane%16)/4 (+8) at column
        // 32 dt + 16 ((lane/16)%2) + 4 (lane%4).
        const int trow = 4 * half + ((lane & 15) >> 2);
        const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) {
              const int row0 = 32 * t + 16 * h + trow;
              const int col = 32 * dt + tcol;
              const int c = col >> 3, within = (col & 7) * 2;
              const char *a0 = lds_v + row0 * TL::kRowBytes + ((c ^ TL::swz_v(row0)) * 16) + within;
              const char *a1 = lds_v + (row0 + 8) * TL::kRowBytes + ((c ^ TL::swz_v(row0 + 8)) * 16) + within;
              const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (s16x4 __attribute__((address_space(3))) *)(a0));
              const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (s16x4 __attribute__((address_space(3))) *)(a1));
              const s16x4 both[2] = {lo4, hi4};
              bf16x8 a;
              __builtin_memcpy(&a, both, 16);
              o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[t][h], o[dt], 0, 0, 0);
            }
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = 32 * t + 8 * (v / 4) + 4 * half + (v % 4);
#pragma unroll
            for (int dt = 0; dt < kDT; ++dt) {
              const int col = 32 * dt + (lane & 31);
              const int c = col >> 2;
              const float a = *reinterpret_cast<const float *>(
                  lds_v + key * TL::kRowBytes + ((c ^ TL::swz_v(key)) * 16) + (col & 3) * 4);
              o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sc[t][v], o[dt], 0, 0, 0);
            }
          }
      }
    }
  }

  // ---- epilogue: O / l, lse ----
  const float l_tot = pair_sum(l_run);
  const bool has = l_tot > 0.f;
  const float inv = has ? 1.f / l_tot : 0.f;
  T *og = static_cast<T *>(p.out) + ((static_cast<int64_t>(b) * p.Hq + hq) * p.Sq + q_row) * D;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = 32 * dt + 8 * g + 4 * half;
      if constexpr (kBf16) {
        union { __bf16 h[4]; u32x2 u; } pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk.h[e] = static_cast<__bf16>(o[dt][4 * g + e] * inv);
        *reinterpret_cast<u32x2 *>(og + col) = pk.u;
      } else {
        float4 x;
        x.x = o[dt][4 * g + 0] * inv; x.y = o[dt][4 * g + 1] * inv;
        x.z = o[dt][4 * g + 2] * inv; x.w = o[dt][4 * g + 3] * inv;
        *reinterpret_cast<float4 *>(og + col) = x;
      }
    }
  if (p.lse && half == 0) {
    const float m_fin = m_run == -INFINITY ? 0.f : m_run;
    const float cfin = CAP ? 1.f : c2;
    p.lse[(static_cast<int64_t>(b) * p.Hq + hq) * p.Sq + q_row] =
        has ? (m_fin * cfin + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D, bool CAP, bool DENSE>
hipError_t launch_one(const FwdParams &p, hipStream_t stream) {
  const int64_t blocks = p.B * p.Hq * p.nq;
  hipLaunchKernelGGL((splash_fwd_kernel<T, D, CAP, DENSE>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const FwdParams &p, hipStream_t stream) {
  if (p.cap) return p.dense ? launch_one<T, D, true, true>(p, stream) : launch_one<T, D, true, false>(p, stream);
  return p.dense ? launch_one<T, D, false, true>(p, stream) : launch_one<T, D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdParams &p, int dtype, hipStream_t stream) {
  if (dtype == 0) return p.D == 64 ? launch_d<__bf16, 64>(p, stream) : launch_d<__bf16, 128>(p, stream);
  return p.D == 64 ? launch_d<float, 64>(p, stream) : launch_d<float, 128>(p, stream);
}

}  // namespace splash
