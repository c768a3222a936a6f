// Splash-attention forward kernel for gfx950 (CDNA4).
//
// What it computes is masked softmax attention (splash-attention explainer,
// FAQ "What is splash attention and how is it different from flash
// attention?"); how it walks the work comes from the compiled MaskInfo
// (FAQ "What is MaskInfo in splash attention?", "What does grid shrinking do
// in splash attention?"):
//   * one workgroup per (batch, query head, 128-row query block) -- or per
//     key split of it, or per block row of two heads of a GQA group; its
//     loop runs over the W grid positions of that block row (the bfloat16
//     kernel walks a flattened list of the non-empty ones);
//   * label 0: nothing runs and no key/value bytes are fetched;
//   * label 2: the block is computed with no mask at all;
//   * label 1: the block is computed and masked -- computable masks are
//     recomputed from q_sequence and the key position, dense masks read the
//     partial block mask_next points at;
//   * data_next names the key/value block to fetch at each position.
// The softmax is the flash online softmax: a per-row running max and running
// sum, one division by the final sum at the end, and the log-sum-exp kept as
// the per-row residual.
//
// Two kernels, one per input type:
//   * splash_fwd_wide (bfloat16): two 64-lane waves per 128-row block, 64
//     query rows per wave, K/V streamed through LDS by direct-to-LDS loads in
//     32-key stages, software-pipelined QK / softmax / PV over 32x32x16 bf16
//     MFMAs;
//   * splash_fwd_f32 (float32): four waves of 32 rows over 128-key tiles with
//     the 32x32x2 f32 MFMA.
// Both form the scores transposed, S^T = K Q^T, so that a lane holds one
// query row and row reductions stay inside a lane pair, and accumulate
// O^T = V^T P^T with P taken straight from the score registers.
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

// Attention sinks (softmax_aux of the EasyDeL BlockSparseAttn.forward_native
// signature): logits that join the softmax denominator of every row of a
// head and carry no value.  Returns log2 of the sum of e^(a_k) over the sink
// logits of query head hq, or -inf without sinks.  Uniform per workgroup.
__device__ __forceinline__ float sink_lse2(const FwdParams &p, int hq) {
  if (p.aux == nullptr || p.num_sinks <= 0) return -INFINITY;
  const int row = p.aux_heads == 1 ? 0 : (p.aux_heads == static_cast<int>(p.Hq) ? hq : hq / p.group);
  const float *a = p.aux + static_cast<int64_t>(row) * p.num_sinks;
  float mx = -INFINITY;
  for (int k = 0; k < p.num_sinks; ++k) mx = fmaxf(mx, a[k]);
  if (mx == -INFINITY) return -INFINITY;
  float sum = 0.f;
  for (int k = 0; k < p.num_sinks; ++k) sum += __builtin_amdgcn_exp2f((a[k] - mx) * kLog2e);
  return mx * kLog2e + __builtin_amdgcn_logf(sum);
}

// Final normalisation of one row from its sum l_tot of exponentials taken
// against base2 (log2 units) and the sinks' log2-sum sl2: the factor that
// turns the accumulated numerator into the output, and the natural-log lse.
// Without sinks: 1 / l_tot and (base2 + log2 l_tot) ln 2.  With sinks the
// row's own log-sum L and the sinks' S combine as T = log2(2^L + 2^S), and
// the output is scaled by 2^(L - T) / l_tot.  A row with no allowed key has
// output 0 and lse = S (-inf without sinks).
__device__ __forceinline__ void row_finish(float l_tot, float base2, float sl2, float &inv, float &lse) {
  const bool has = l_tot > 0.f;
  const float l2 = has ? base2 + __builtin_amdgcn_logf(l_tot) : -INFINITY;
  if (sl2 == -INFINITY) {
    inv = has ? 1.f / l_tot : 0.f;
    lse = has ? l2 * kLn2 : -INFINITY;
    return;
  }
  const float mx = fmaxf(l2, sl2);
  const float t2 = mx + __builtin_amdgcn_logf(__builtin_amdgcn_exp2f(l2 - mx) + __builtin_amdgcn_exp2f(sl2 - mx));
  inv = has ? __builtin_amdgcn_exp2f(l2 - t2) / l_tot : 0.f;
  lse = t2 * kLn2;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// The two 4-element halves of a transposing LDS read joined into one MFMA
// operand, in registers.  (Copying them through a local array made the
// compiler place that array in LDS, one slot per thread, which needs the
// workgroup size from the dispatch packet in host memory: microseconds of
// latency at the start of every workgroup.)
__device__ __forceinline__ bf16x8 join_tr_halves(s16x4 lo4, s16x4 hi4) {
  const s16x8 c = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}
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

// Tile geometry and swizzles of the float32 kernel.  A tile is 128 rows of
// D floats; a row is split into 16-byte chunks whose index is XORed with
// swz(row).
template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 4;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kBytes = kBK * kRowBytes;
  // K tile: the A-operand read has 32 lanes on 32 consecutive rows at one
  // chunk.
  __device__ static int swz_k(int row) {
    if constexpr (kChunks >= 16) return row & 15;
    else return (row >> 1) & 7;
  }
  // V tile: the operand read has 32 lanes on one row.
  __device__ static int swz_v(int row) { return row & 15; }
};

// Copy one 128 x D tile from global memory (rows contiguous, D elements each)
// into a swizzled LDS tile.  Each lane moves 16-byte chunks; 16 lanes cover
// one 256-byte span of a row, so the global reads are fully coalesced.
template <int D, bool IS_V>
__device__ __forceinline__ void stage_tile(char *lds, const float *g, int tid, int mrow) {
  using TL = Tile<D>;
  constexpr int kPerThread = kBK * TL::kChunks / kThreads;
  u32x4 buf[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx / TL::kChunks, c = idx % TL::kChunks;
    // padded head dims: rows of mrow bytes in memory, zeros past them
    buf[i] = c * 16 < mrow ? *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(g) +
                                                              static_cast<size_t>(row) * mrow + c * 16)
                           : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx / TL::kChunks, c = idx % TL::kChunks;
    const int pc = c ^ (IS_V ? TL::swz_v(row) : TL::swz_k(row));
    *reinterpret_cast<u32x4 *>(lds + row * TL::kRowBytes + pc * 16) = buf[i];
  }
}

// ===========================================================================
// float32 kernel.  Four 64-lane waves per workgroup, each owning 32 query
// rows.  Scores are formed transposed, S^T = K Q^T, with the 32x32x2 f32
// MFMA: Q stays in registers as the B operand and K streams from LDS as the A
// operand.  In that output layout every lane holds one query row (lane % 32)
// and 16 of its keys per 32-key tile, so a row max or row sum is a per-lane
// reduction plus one v_permlane32_swap with the partner lane (lane ^ 32).
// The output is accumulated transposed too, O^T = V^T P^T, with P taken
// straight from the score registers.  K and V tiles (128 x D) are staged
// through VGPRs into LDS with XOR-swizzled 16-byte chunks, so the staging
// writes and both operand reads are bank-conflict free.  The softmax keeps
// the exact running max: the accumulator is rescaled whenever a row's max
// moves.
template <int D, bool CAP, bool DENSE>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1)
void splash_fwd_f32(const FwdParams p) {
  using TL = Tile<D>;
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

  // Head dims in memory: D, or (padded) the caller's D and Dv, run
  // zero-padded to D columns (zeros in Q and the tiles past them; the
  // output's padding columns are not stored).
  const int mk = p.padded ? p.dk : D, mv = p.padded ? p.dv : D;
  const int64_t q_row = static_cast<int64_t>(r) * kBQ + lrow;
  const float *qg = static_cast<const float *>(p.q) + ((static_cast<int64_t>(b) * p.Hq + hq) * p.Sq + q_row) * mk;
  const float *kg = static_cast<const float *>(p.k) + (static_cast<int64_t>(b) * p.Hkv + hkv) * p.Skv * mk;
  const float *vg = static_cast<const float *>(p.v) + (static_cast<int64_t>(b) * p.Hkv + hkv) * p.Skv * mv;

  // ---- Q fragment (B operand of S^T = K Q^T), resident for the whole row ----
  // The lane's half owns d in [half D/2, (half+1) D/2) and k-step ks takes one of them.
  constexpr int kQRegs = D / 2;
  float qf[kQRegs];
#pragma unroll
  for (int i = 0; i < kQRegs / 4; ++i) {
    const int d0 = half * (D / 2) + 4 * i;
    const float4 x = d0 < mk ? *reinterpret_cast<const float4 *>(qg + d0) : make_float4(0.f, 0.f, 0.f, 0.f);
    qf[4 * i + 0] = x.x; qf[4 * i + 1] = x.y; qf[4 * i + 2] = x.z; qf[4 * i + 3] = x.w;
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
    lo -= p.kv_offset;   // into this (possibly key-sliced) MaskInfo's key coordinates
    hi -= p.kv_offset;
  }

  // ---- running softmax state ----------------------------------------------
  const float c2 = p.c2;                   // score multiplier into base-2 units
  float m_run = -INFINITY;                 // running max (raw score units, or capped base-2 units)
  float mb_run = -INFINITY;                // the same in base-2 units, as the exponentials used it
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
      stage_tile<D, false>(lds_k, kg + static_cast<int64_t>(kvb) * kBK * mk, tid, mk * 4);
      stage_tile<D, true>(lds_v, vg + static_cast<int64_t>(kvb) * kBK * mv, tid, mv * 4);
      __syncthreads();

      // ---- S^T = K Q^T: four 32-key tiles ----
      f32x16 sc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[t][v] = 0.f;
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
      float mb = m_use * c2e;
      // The base must be the same rounded float everywhere it is used: the
      // exponentials, alpha and the lse.  HIP contracts a*b+c into an FMA
      // across statements, which would fuse this product into
      // mb_run - mb and leave its rounding error in alpha: alpha one ulp off
      // 1 at every step of an unmoved max, a drift of the running sum and
      // the accumulator of about 1e-7 per block (2e-5 in lse after 258
      // blocks).  The empty asm makes mb an opaque, already rounded value.
      asm volatile("" : "+v"(mb));
      const float alpha = __builtin_amdgcn_exp2f(mb_run - mb);
      mb_run = mb;
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

  // ---- epilogue: O / l, lse ----
  const float l_tot = pair_sum(l_run);
  float inv, lse_row;
  row_finish(l_tot, mb_run == -INFINITY ? 0.f : mb_run, sink_lse2(p, hq), inv, lse_row);
  float *og = static_cast<float *>(p.out) + ((static_cast<int64_t>(b) * p.Hq + hq) * p.Sq + q_row) * mv;
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = 32 * dt + 8 * g + 4 * half;
      float4 x;
      x.x = o[dt][4 * g + 0] * inv; x.y = o[dt][4 * g + 1] * inv;
      x.z = o[dt][4 * g + 2] * inv; x.w = o[dt][4 * g + 3] * inv;
      if (col < mv) *reinterpret_cast<float4 *>(og + col) = x;
    }
  if (p.lse && half == 0) p.lse[(static_cast<int64_t>(b) * p.Hq + hq) * p.Sq + q_row] = lse_row;
}

// ===========================================================================
// bf16 kernel with 64 query rows per wave ("wide" rows).
//
// Why: with 32 rows per wave every wave reads the whole K and V tile from LDS
// for only 32 rows of work, which puts LDS read time at or above the MFMA
// time.  Here each wave owns 64 query rows -- two 32-row halves (qs = 0, 1)
// that share every K and V operand read -- so LDS reads per flop halve.  The
// price is registers (Q and O for 64 rows), so one wave runs per SIMD and the
// overlap of softmax (VALU) with matrix work (MFMA) comes from software
// pipelining inside the wave instead of from a second wave: pipeline step u
// (32 keys, a quarter of a 128-key block) runs
//     QK(u+1)  ||  softmax(u)  ||  PV(u-1)
// with independent register sets, so the exponentials of one step issue
// between the matrix instructions of its neighbours.
//
// Workgroup: two waves = 128 query rows = one mask block row; two workgroups
// share a CU.  K and V arrive in LDS through direct-to-LDS loads (no VGPRs),
// 32 keys per stage, four stages each.  The loads of K(u+4) and V(u+2) are
// issued during the first slices of iteration u into the stages iteration
// u-1 finished reading; step u+1's K and step u-1's V must have landed by the
// top of iteration u, so each load has about three iterations to arrive.
constexpr int kWWaves = 2;
constexpr int kWThreads = 64 * kWWaves;
constexpr int kSK = 32;            // keys per pipeline step
constexpr int kSteps = kBK / kSK;  // steps per mask block
constexpr int kStages = 4;         // LDS stages for K and for V

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Buffer resource over `bytes` bytes at `base` (gfx9 data-format word 3).
// Uniform by construction; readfirstlane keeps it in SGPRs.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, int64_t bytes) {
  const int n = bytes > 0x7fffffffLL ? 0x7fffffff : static_cast<int>(bytes);
  // The four descriptor words, built directly: base address (48 bits, stride
  // 0), the byte count, and the data-format word.  (Going through the
  // opaque resource type and a memcpy left a private copy that the compiler
  // placed in LDS per thread, which reads the workgroup size from the
  // dispatch packet in host memory at every workgroup's start.)
  const uint64_t a = reinterpret_cast<uintptr_t>(base);
  i32x4 v;
  v[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a)));
  v[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffffu));
  v[2] = __builtin_amdgcn_readfirstlane(n);
  v[3] = 0x00020000;
  return v;
}

// Barrier that waits only for this wave's LDS operations; global->LDS loads
// are awaited explicitly with wait_vmcnt, so a prefetch may stay in flight
// across it.  The asm is also a compiler memory barrier for LDS accesses.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One 32-key stage of K or V: 32 rows of D bf16, 16-byte chunks XOR-swizzled
// per row (the swizzles of the 128-row tiles above).
template <int D, int W = kWWaves>
struct Stage {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kBytes = kSK * kRowBytes;
  static constexpr int kInsts = kBytes / 1024 / W;  // 1 KiB loads per wave per stage (W waves share it)
  __device__ static int swz_k(int row) {
    if constexpr (kChunks >= 16) return row & 15;
    else return (row >> 1) & 7;
  }
  __device__ static int swz_v(int row) {
    if constexpr (kChunks >= 16) return (row & 3) << 2;
    else return ((row >> 1) & 1) << 2;
  }
};

// Issue the direct-to-LDS loads (buffer_load_dwordx4 ... lds) of one stage:
// rows [row0, row0 + 32) of a (batch, kv-head) K or V array described by
// `res`.  Wave w moves the stage's 1 KiB segments w*kInsts .. w*kInsts+kInsts-1.
// Each instruction writes 64 lanes x 16 bytes to consecutive LDS bytes
// (M0 + instruction offset + 16 lane); the instruction offset is added to
// the global address too, so one M0 value serves all of a wave's segments.
// The swizzle is applied on the global side: the lane that lands on chunk pc
// of a row fetches logical chunk pc ^ swz(row).  Reads past the resource's
// end return zeros instead of faulting.
//
// Issued from inline assembly so the compiler does not track them: it cannot
// tell that a load into one stage does not alias LDS reads of another and
// would otherwise drain every prefetch before each LDS read.  Completion is
// awaited with wait_vmcnt before the barrier that publishes a stage; waits the
// compiler computes for its own loads stay correct (loads retire in order, so
// extra loads in flight only make them more conservative).  M0 is written in
// the same statement as the loads that read it.
template <int D, bool IS_V, int W = kWWaves>
__device__ __forceinline__ uint32_t stage_voff(int wave, int lane, int i) {
  using SG = Stage<D, W>;
  constexpr int kRowsPerSeg = 1024 / SG::kRowBytes;
  constexpr int kLanesPerRow = SG::kChunks;
  const int seg = wave * SG::kInsts + i;
  const int row = seg * kRowsPerSeg + lane / kLanesPerRow;
  const int pc = lane % kLanesPerRow;
  const int c = pc ^ (IS_V ? SG::swz_v(row) : SG::swz_k(row));
  return static_cast<uint32_t>((lane / kLanesPerRow) * SG::kRowBytes + c * 16);
}

// Padded head dims (PAD): the stage keeps its D-column layout, but the array
// in memory has rows of `mrow` bytes of which the first `mvalid` hold data.
// Each segment then gets its own M0 and per-lane offsets (the instruction
// offset can no longer step the LDS and the global address together); a
// lane whose chunk lies in the padding gets an offset past the resource's
// end, which reads zeros.
template <int D, bool IS_V, int W>
__device__ __forceinline__ void issue_seg_padded(char *lds, i32x4 res, int64_t row0, int wave, int lane, int i,
                                                 uint32_t mrow, uint32_t mvalid) {
  using SG = Stage<D, W>;
  constexpr int kRowsPerSeg = 1024 / SG::kRowBytes;
  constexpr int kLanesPerRow = SG::kChunks;
  const int seg = wave * SG::kInsts + i;
  const int row = seg * kRowsPerSeg + lane / kLanesPerRow;
  const int c = (lane % kLanesPerRow) ^ (IS_V ? SG::swz_v(row) : SG::swz_k(row));
  const uint32_t voff = static_cast<uint32_t>(c * 16) < mvalid
      ? static_cast<uint32_t>((row0 + row) * mrow) + static_cast<uint32_t>(c * 16)
      : 0x80000000u;
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) char *)(lds + seg * 1024)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m0), "v"(voff), "s"(res) : "memory", "m0");
#pragma clang diagnostic pop
}

template <int D, bool IS_V, int W = kWWaves, bool PAD = false>
__device__ __forceinline__ void issue_stage(char *lds, i32x4 res, int64_t row0, int wave, int lane,
                                            uint32_t mrow = 0, uint32_t mvalid = 0) {
  using SG = Stage<D, W>;
  if constexpr (PAD) {
#pragma unroll
    for (int i = 0; i < SG::kInsts; ++i) issue_seg_padded<D, IS_V, W>(lds, res, row0, wave, lane, i, mrow, mvalid);
    return;
  }
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) char *)(lds + wave * SG::kInsts * 1024)));
  const uint32_t soff = static_cast<uint32_t>(row0 * SG::kRowBytes) + wave * SG::kInsts * 1024;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  if constexpr (SG::kInsts == 4) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %5, %6 offen lds\n\t"
        "buffer_load_dwordx4 %2, %5, %6 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %3, %5, %6 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %4, %5, %6 offen offset:3072 lds"
        :: "s"(m0), "v"(stage_voff<D, IS_V, W>(wave, lane, 0)), "v"(stage_voff<D, IS_V, W>(wave, lane, 1)),
           "v"(stage_voff<D, IS_V, W>(wave, lane, 2)), "v"(stage_voff<D, IS_V, W>(wave, lane, 3)), "s"(res), "s"(soff)
        : "memory", "m0");
  } else {
    static_assert(SG::kInsts == 2, "stage loads per wave");
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %3, %4 offen lds\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen offset:1024 lds"
        :: "s"(m0), "v"(stage_voff<D, IS_V, W>(wave, lane, 0)), "v"(stage_voff<D, IS_V, W>(wave, lane, 1)), "s"(res),
           "s"(soff)
        : "memory", "m0");
  }
#pragma clang diagnostic pop
}

// One segment (1 KiB, segment I of this wave's share) of a stage, for
// spreading a stage's loads over several slices of a step.
template <int D, bool IS_V, int I, int W = kWWaves, bool PAD = false>
__device__ __forceinline__ void issue_seg(char *lds, i32x4 res, int64_t row0, int wave, int lane,
                                          uint32_t mrow = 0, uint32_t mvalid = 0) {
  using SG = Stage<D, W>;
  static_assert(I < SG::kInsts, "segment index");
  if constexpr (PAD) {
    issue_seg_padded<D, IS_V, W>(lds, res, row0, wave, lane, I, mrow, mvalid);
    return;
  }
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) char *)(lds + wave * SG::kInsts * 1024)));
  const uint32_t soff = static_cast<uint32_t>(row0 * SG::kRowBytes) + wave * SG::kInsts * 1024;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen offset:%4 lds"
      :: "s"(m0), "v"(stage_voff<D, IS_V, W>(wave, lane, I)), "s"(res), "s"(soff), "n"(I * 1024)
      : "memory", "m0");
#pragma clang diagnostic pop
}

// One QK matrix instruction of the pipelined body, issued from inline
// assembly so its accumulator lives in VGPRs (where the softmax reads it) and
// its Q operand in AGPRs: left to itself the compiler keeps every MFMA
// accumulator in AGPRs and moves each score to VGPRs before the softmax.
// The compiler does not see this instruction's latency, so a VALU read of
// the accumulator must come at least kQkMfmaDrain cycles later (see
// qk_drain); the pipeline only reads it a whole step later, or after
// qk_drain.  A k-step that starts a tile writes the accumulator without
// reading it (C = 0) and must not share registers with its inputs.
__device__ __forceinline__ void qk_mfma(f32x16 &acc, const bf16x8 &a, const bf16x8 &q, bool first) {
  if (first)
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(q));
  else
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(q));
}

// Wait states covering the result latency of the last qk_mfma before its
// accumulator is read by VALU instructions: 24, above the 19 a 16-pass XDL
// result needs (the 32x32x16 bf16 instruction takes 8 passes).
__device__ __forceinline__ void qk_drain() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
}

// S^T for one 32-key step: sc[qs] holds, for this lane's row of half qs, keys
// 8(v/4) + 4 half + v%4 of the step.
template <int D>
__device__ __forceinline__ void wide_qk(const char *ks_lds, const bf16x8 (*qf)[D / 16], int lane, int half,
                                        f32x16 *sc) {
  using SG = Stage<D>;
  const int row = lane & 31;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
        ks_lds + row * SG::kRowBytes + (((2 * ks + half) ^ SG::swz_k(row)) * 16));
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) qk_mfma(sc[qs], a, qf[qs][ks], ks == 0);
  }
  qk_drain();   // callers read the scores right away
}

// Per-row softmax state of the wide kernel: the online softmax with a lazy
// running max.  A row's exponent base is set by its first step with an
// allowed key and moves only when, at the end of a 128-key block, the row's
// sum has grown past 2^40 (scores about 27 nats or more above the base):
// then the base becomes the block's last step's max and the accumulator and
// the sum are rescaled by 2^(old - new) -- the flash rescaling, taken rarely
// instead of at every step, so a normal step needs no row max.  Between moves, exponentials of
// larger scores simply exceed 1, which is exact far from the float range.
// Two rare cases remain for a final exact pass: a row whose sum ends above
// 2^64 (not expected after the moves; kept as a safety net) and a row whose
// sum ends below 2^-64 with allowed keys (its first allowed step was fully
// masked, so its base stayed 0, and all its logits lie far below 0).  Such a
// workgroup computes every row's exact max (a QK-only pass) and runs again
// with it as the base, where every exponential is at most 1.
constexpr float kOverflowSum = 18446744073709551616.f;   // 2^64
constexpr float kUnderflowSum = 5.421010862427522e-20f;   // 2^-64
constexpr float kRescaleSum = 1099511627776.f;            // 2^40: a step's sum that moves the base

struct RowState {
  float base[2];   // exponent base, base-2 units (-inf until the first allowed key)
  float l[2];      // this lane's share of the running sum
  bool over;       // the row needs the exact-max recompute
};

// The allowed keys of this lane's row of half qs in a 32-key step, as the
// bits 8 (v / 4) + v % 4 of score element v: dense masks take the row's
// staged word shifted to this lane's keys; computable masks turn the row's
// key interval [lo, hi] into the same bits (bit c <=> key kb + c).
template <bool DENSE>
__device__ __forceinline__ unsigned lane_key_word(int key0, int half, const int *lo, const int *hi,
                                                  const unsigned *mword, int qs) {
  if constexpr (DENSE) {
    return mword[qs] >> (4 * half);
  } else {
    const int kb = key0 + 4 * half;
    const int b0 = min(max(lo[qs] - kb, 0), kSK);       // first allowed bit
    const int b1 = min(max(hi[qs] - kb + 1, 0), kSK);   // one past the last
    const uint64_t span = b1 > b0 ? (uint64_t(1) << b1) - (uint64_t(1) << b0) : 0;
    return static_cast<uint32_t>(span);
  }
}

// Score element v of a lane with key bit word w: the score, or -inf where
// the key is masked -- bit c sign-extended (0 or all ones) selects, bit by
// bit: a bitfield extract and a bitfield select.
__device__ __forceinline__ float mask_select(float x, unsigned w, int v) {
  const int c = 8 * (v / 4) + (v % 4);
  const int m = __builtin_amdgcn_sbfe(static_cast<int>(w), c, 1);
  return __int_as_float((m & __float_as_int(x)) | (~m & static_cast<int>(0xff800000u)));
}

// Scores of one step -> capped (base-2 units), masked.  MASK: label-1 step.
// Computable masks use the row's key interval; dense masks the packed word
// of the row (bit c <=> key c of the step).
template <bool CAP, bool DENSE, bool MASK>
__device__ __forceinline__ void wide_cap_mask(const FwdParams &p, f32x16 *sc, int key0, int half, const int *lo,
                                              const int *hi, const unsigned *mword, unsigned *seen) {
  if constexpr (CAP) {
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        // a key masked before the cap stays at -inf (tanh alone would map it to -cap)
        const float x = sc[qs][v] * p.c2;  // c2 = scale / cap here
        const float e = __builtin_amdgcn_exp2f(-2.f * kLog2e * fabsf(x));
        const float th = (1.f - e) * __builtin_amdgcn_rcpf(1.f + e);
        sc[qs][v] = x == -INFINITY ? -INFINITY : copysignf(th, x) * p.cap_out;
      }
  }
  if constexpr (MASK) {
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const unsigned w = lane_key_word<DENSE>(key0, half, lo, hi, mword, qs);
      seen[qs] |= w & 0x0f0f0f0fu;   // this lane's keys: bits 8 (v / 4) + v % 4
#pragma unroll
      for (int v = 0; v < 16; ++v) sc[qs][v] = mask_select(sc[qs][v], w, v);
    }
  }
}

// O^T += V^T P^T for one step.  The lane supplies V[key][dv] for
// dv = 32 dt + lane%32 and the keys 16h + 4 half + {0..3, 8..11} -- the order
// in which pf holds them -- with two transposing reads.
template <int D>
__device__ __forceinline__ void wide_pv(const char *vs_lds, const bf16x8 (*pf)[2], int lane, int half,
                                        f32x16 (*o)[2]) {
  using SG = Stage<D>;
  const int trow = 4 * half + ((lane & 15) >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int row0 = 16 * h + trow;
      const int col = 32 * dt + tcol;
      const int c = col >> 3, within = (col & 7) * 2;
      const char *a0 = vs_lds + row0 * SG::kRowBytes + ((c ^ SG::swz_v(row0)) * 16) + within;
      const char *a1 = vs_lds + (row0 + 8) * SG::kRowBytes + ((c ^ SG::swz_v(row0 + 8)) * 16) + within;
      const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3))) *)(a0));
      const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3))) *)(a1));
      const bf16x8 a = join_tr_halves(lo4, hi4);
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
        o[dt][qs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qs][h], o[dt][qs], 0, 0, 0);
    }
}

// Wait until at most n vector-memory loads of this wave are in flight
// (n <= N; s_waitcnt takes an immediate, so walk down from N).
template <int N>
__device__ __forceinline__ void wait_at_most(int n) {
  if constexpr (N == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= N) wait_vmcnt<N>();
    else wait_at_most<N - 1>(n);
  }
}

// RU: query heads per workgroup.  RU = 2 runs two heads of one GQA group
// (which share their key/value head and, with one mask head, their walk)
// in four waves over one set of K/V stages: each stage's loads serve 256
// query rows instead of 128.
template <int D, bool CAP, bool DENSE, int RU = 1, bool PAD = false>
__global__ __launch_bounds__(64 * kWWaves * RU, 1)
void splash_fwd_wide(const FwdParams p) {
  static_assert(RU == 1 || (RU == 2 && D == 128 && !DENSE), "head pairs: D = 128, computable masks");
  constexpr int kW = kWWaves * RU;          // waves
  constexpr int kThr = 64 * kW;
  using SG = Stage<D, kW>;
  constexpr int kDT = D / 32;
  constexpr int kKS = D / 16;
  constexpr int kMaskBytes = kBQ * 4;            // one packed word per block row per step
  constexpr int kMaxInFlight = 5 * SG::kInsts + 3;

  __shared__ __attribute__((aligned(1024))) char k_st[kStages][SG::kBytes];
  __shared__ __attribute__((aligned(1024))) char v_st[kStages][SG::kBytes];
  __shared__ __attribute__((aligned(16))) char m_st[DENSE ? kStages : 1][kMaskBytes];
  __shared__ int wg_any[kW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int wr = wave % kWWaves;            // the wave's 64 rows of the block row
  const int hsub = wave / kWWaves;          // which of the workgroup's RU heads

  // Same (batch, head, row) mapping as the 32-row kernel: XCD x gets a
  // contiguous range of (batch, head) pairs, rows go out longest first.
  // With RU heads per workgroup the pairs are (batch, group of RU heads).
  const int heads_u = static_cast<int>(p.Hq) / RU;
  const int nbh = static_cast<int>(p.B) * heads_u;
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
  // With split keys, rank counts (row, split) pairs: the splits of a row
  // follow one another in launch order.
  const int n_split = p.kv_splits;
  const int split = rank % n_split;
  const int b = bh / heads_u;
  const int hq = (bh % heads_u) * RU + hsub;
  const int hkv = hq / p.group;
  const int hm = p.hm == 1 ? 0 : hq;
  // The workgroup's item and walk: one scalar load names the block row, the
  // range of its walk entries (the row's non-empty grid positions in order,
  // or this split's share of them) and the first entry's block, so the
  // first key/value loads can go out at once.  The tables are read-only for
  // the kernel's lifetime, so they are read through the constant address
  // space (scalar loads, counted with the LDS operations, not with the
  // key/value loads whose counts the pipeline waits on).
  typedef const __attribute__((address_space(4))) int32_t *cptr;
  const cptr items = (cptr)(p.items);
  const cptr walk_kv = (cptr)(p.walk_kv);
  const cptr walk_mn = (cptr)(DENSE ? p.walk_mn : p.walk_kv);
  const int64_t item_at = ((static_cast<int64_t>(hm) * p.nq) * n_split + rank) * 8;
  const int r = items[item_at + 0];
  const int w_off = items[item_at + 1];
  const int w_len = items[item_at + 2];
  const int row_in_block0 = 64 * wr + (lane & 31);      // qs = 0; qs = 1 adds 32
  const int64_t q_row0 = static_cast<int64_t>(r) * kBQ + row_in_block0;

  // Head dims in memory: D itself, or (PAD) the caller's D and Dv, which the
  // kernel runs zero-padded to D columns -- Q and the stages hold zeros in
  // the padding, so QK sums only real columns, and the padded output columns
  // are not stored.
  const int mk = PAD ? p.dk : D;
  const int mv = PAD ? p.dv : D;
  const __bf16 *kg = static_cast<const __bf16 *>(p.k) + (static_cast<int64_t>(b) * p.Hkv + hkv) * p.Skv * mk;
  const __bf16 *vg = static_cast<const __bf16 *>(p.v) + (static_cast<int64_t>(b) * p.Hkv + hkv) * p.Skv * mv;
  const i32x4 k_res = make_rsrc(kg, p.Skv * mk * 2);
  const i32x4 v_res = make_rsrc(vg, p.Skv * mv * 2);
  const uint32_t krow = static_cast<uint32_t>(mk * 2), vrow = static_cast<uint32_t>(mv * 2);
  const bool has_bits = DENSE && p.pmb_bits != nullptr;
  const i32x4 m_res = make_rsrc(has_bits ? static_cast<const void *>(p.pmb_bits) : p.k,
                                has_bits ? p.pmb_bits_bytes : 0);

  // Packed mask words of step t of partial block pb (dense masks): this
  // wave's 64 block rows, into mask stage `stage`.
  auto issue_mask = [&](int pb, int t, int stage) {
    const uint32_t soff = static_cast<uint32_t>(((pb * kSteps + t) * kBQ + 64 * wave) * 4);
    const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) char *)(m_st[stage] + 256 * wave)));
    const uint32_t voff = static_cast<uint32_t>(4 * lane);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(m0), "v"(voff), "s"(m_res), "s"(soff) : "memory", "m0");
#pragma clang diagnostic pop
  };

  // The prologue loads of the first block (K of its four steps, their mask
  // words, V of the first two) go out before the Q loads, so the two
  // latencies overlap.  (A split with no block loads a block it never uses.)
  const int dn_first = items[item_at + 3];
  const int mn_first = has_bits ? items[item_at + 4] : 0;
  if constexpr (PAD) {
    // the padding columns of every stage start (and stay) zero; written and
    // published before any load into the stages
#pragma unroll
    for (int i = 0; i < kStages * SG::kBytes / (16 * kThr); ++i) {
      reinterpret_cast<u32x4 *>(&k_st[0][0])[tid + kThr * i] = u32x4{0u, 0u, 0u, 0u};
      reinterpret_cast<u32x4 *>(&v_st[0][0])[tid + kThr * i] = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < kSteps; ++t) {
    issue_stage<D, false, kW, PAD>(k_st[t], k_res, static_cast<int64_t>(dn_first) * kBK + kSK * t, wave, lane, krow,
                                   krow);
    if (has_bits) issue_mask(mn_first, t, t);
  }
  issue_stage<D, true, kW, PAD>(v_st[0], v_res, static_cast<int64_t>(dn_first) * kBK, wave, lane, vrow, vrow);
  issue_stage<D, true, kW, PAD>(v_st[1], v_res, static_cast<int64_t>(dn_first) * kBK + kSK, wave, lane, vrow, vrow);
  static_assert(kSteps == kStages, "the prologue fills every K stage");

  // The other V stages start as zeros: the first step's PV(-1) reads the
  // last stage with zero P, and 0 * (uninitialised LDS) could be NaN.
#pragma unroll
  for (int i = 0; i < 2 * SG::kBytes / (16 * kThr); ++i)
    reinterpret_cast<u32x4 *>(&v_st[2][0])[tid + kThr * i] = u32x4{0u, 0u, 0u, 0u};

  bf16x8 qf[2][kKS];       // Q (B operand of S^T = K Q^T), rows of both halves
  int lo[2], hi[2];        // computable masks: allowed key interval, clamped to [-1, Skv]
  int64_t qpos_ld[2] = {0, 0};
  {
    // All Q loads (and the rows' positions) go out before anything waits
    // for them: a register move placed after each load would make every
    // load wait for the one before it.
    const __bf16 *qg = static_cast<const __bf16 *>(p.q) + ((static_cast<int64_t>(b) * p.Hq + hq) * p.Sq + q_row0) * mk;
    bf16x8 x[2][kKS];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        if (!PAD || 16 * ks + 8 * half < mk)
          x[qs][ks] = *reinterpret_cast<const bf16x8 *>(qg + static_cast<int64_t>(32 * qs) * mk + 16 * ks + 8 * half);
        else
          x[qs][ks] = bf16x8{};   // padding columns: zero
      }
    if constexpr (!DENSE) {
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) qpos_ld[qs] = p.q_seq[q_row0 + 32 * qs];
    }
    // Q lives in AGPRs for the whole kernel: the QK instructions read it
    // from there, which leaves the VGPRs to the scores and P.
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) asm volatile("" : "=a"(qf[qs][ks]) : "0"(x[qs][ks]));
  }
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    lo[qs] = hi[qs] = 0;
    if constexpr (!DENSE) {
      // Every computable mask admits, for query position i, one key interval:
      // causal (-inf, i]; local [i - left, i + right]; chunked [chunk start, i].
      const int64_t qpos = qpos_ld[qs];
      const int64_t big = int64_t(1) << 40;   // an unbounded side
      int64_t l64, h64;
      if (p.mask_kind == 0) { l64 = -big; h64 = qpos; }
      else if (p.mask_kind == 1) { l64 = p.left < 0 ? -big : qpos - p.left; h64 = p.right < 0 ? big : qpos + p.right; }
      else { l64 = (qpos / p.chunk) * p.chunk; h64 = qpos; }
      // into this (possibly key-sliced) MaskInfo's key coordinates
      lo[qs] = static_cast<int>(clamp64(l64 - p.kv_offset, -1, p.Skv));
      hi[qs] = static_cast<int>(clamp64(h64 - p.kv_offset, -1, p.Skv));
    }
  }
  // Scores leave the QK instructions as raw dot products.  Without a cap,
  // c2e = softmax_scale * log2(e) turns them into base-2 logits; with a cap
  // the cap takes p.c2 and the capped logits are already base-2.  (Q is not
  // pre-scaled: a bf16 rounding of Q * scale errs by up to 2^-8 of a logit,
  // which large logits along one dominant direction do not average away.)
  const float c2e = CAP ? 1.f : p.c2;

  // Walk entry j of this workgroup: key/value block, label, partial block.
  auto ent_kv = [&](int j) -> int { return walk_kv[w_off + j] & 0x0fffffff; };
  auto ent_lab = [&](int j) -> int { return static_cast<int>(static_cast<uint32_t>(walk_kv[w_off + j]) >> 28); };
  auto ent_mn = [&](int j) -> int { return DENSE ? walk_mn[w_off + j] : 0; };
  auto mask_words = [&](int stage, unsigned *mw) {
    if constexpr (DENSE) {
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
        mw[qs] = *reinterpret_cast<const unsigned *>(m_st[stage] + 4 * (row_in_block0 + 32 * qs));
    }
  };

  f32x16 o[kDT][2];        // O^T accumulators
  RowState rs;
  float base_init[2] = {-INFINITY, -INFINITY};
  // Whether each row met an allowed key: any full block, or a set bit in a
  // partial block's mask words (this lane's keys).  A row that met none has
  // a zero sum and needs no recompute.
  bool any_full = false;
  unsigned key_bits[2] = {0u, 0u};

  // Exponent base of rows that have none yet: the max of the chunk's first
  // step (after cap and mask; the cap is monotonic, so capping the max gives
  // the max of the capped scores), or 0 for a row whose keys in that step
  // are all masked.  A base far from the row's true max only matters at the
  // float range's ends, which the overflow and underflow tests catch.
  auto set_base = [&](const f32x16 *sc) {
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[qs][v]);
      mx = pair_max(mx);
      float mx2 = mx * c2e;
      if constexpr (CAP) {
        const float x = mx * p.c2;
        const float e = __builtin_amdgcn_exp2f(-2.f * kLog2e * fabsf(x));
        const float th = (1.f - e) * __builtin_amdgcn_rcpf(1.f + e);
        mx2 = x == -INFINITY ? -INFINITY : copysignf(th, x) * p.cap_out;
      }
      rs.base[qs] = rs.base[qs] == -INFINITY ? (mx2 == -INFINITY ? 0.f : mx2) : rs.base[qs];
    }
  };

  // One step: QK(u+1) || softmax(u) || PV(u-1) as straight-line code cut
  // into nine slices by scheduling barriers.  Slice i holds the QK MFMAs of
  // k-step i-1, the PV MFMAs of operand i-1, the LDS reads two slices ahead
  // of their MFMAs and an eighth of the softmax (four exponentials per row
  // half), so every matrix instruction has a little VALU work to hide under
  // and no operand lives longer than a few slices.  The softmax runs against
  // the row's fixed base; the step's row sums come from dot products of the
  // bf16 exponentials with ones (the same rounded values PV multiplies).
  // MC: std::true_type for a label-1 block, whose scores S(u) are masked
  // here, element by element beside the matrix instructions, with the key
  // words kw (computed at the end of the previous step).  Masked scores are
  // written back, so the block-end base move sees them.
  auto body = [&](int u, f32x16 *sc_cur, f32x16 *sc_nxt, bf16x8 (*pf_cur)[2], bf16x8 (*pf_prv)[2],
                  auto &&issue_loads, float *step_sum, auto mc, const unsigned *kw) {
    constexpr bool kMasked = decltype(mc)::value;
    constexpr int kPVOps = 2 * kDT;       // PV A operands per step: (h, dt)
    const char *kst = k_st[(u + 1) % kStages];
    const char *vst = v_st[(u + kStages - 1) % kStages];
    const int krow = lane & 31;
    const int trow = 4 * half + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto read_k = [&](int ks) -> bf16x8 {
      return *reinterpret_cast<const bf16x8 *>(kst + krow * SG::kRowBytes +
                                               (((2 * ks + half) ^ SG::swz_k(krow)) * 16));
    };
    auto read_v = [&](int i) -> bf16x8 {
      const int h = i / kDT, dt = i % kDT;
      const int row0 = 16 * h + trow;
      const int col = 32 * dt + tcol;
      const int c = col >> 3, within = (col & 7) * 2;
      const char *a0 = vst + row0 * SG::kRowBytes + ((c ^ SG::swz_v(row0)) * 16) + within;
      const char *a1 = vst + (row0 + 8) * SG::kRowBytes + ((c ^ SG::swz_v(row0 + 8)) * 16) + within;
      const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3))) *)(a0));
      const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3))) *)(a1));
      const bf16x8 r = join_tr_halves(lo4, hi4);
      return r;
    };
    bf16x8 ka[kKS], va[kPVOps];
    // Matrix instruction sub of slice i: QK k-step i for row half sub/2
    // (even sub), PV operand i for row half sub/2 (odd sub).
    auto mfma_one = [&](int i, int sub) {
      const int qs = sub >> 1;
      if ((sub & 1) == 0) {
        if (i < kKS) qk_mfma(sc_nxt[qs], ka[i], qf[qs][i], i == 0);
      } else if (i < kPVOps) {
        const int h = i / kDT, dt = i % kDT;
        o[dt][qs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i], pf_prv[qs][h], o[dt][qs], 0, 0, 0);
      }
    };
    auto reads_slice = [&](int i) {
      if (i < kKS) ka[i] = read_k(i);
      if (i < kPVOps) va[i] = read_v(i);
    };
    float b2[2], kr[2], sum[2] = {0.f, 0.f};   // kr (cap): cap log2(e) - base, per row
    const float kc2 = 2.f * kLog2e * p.c2;   // cap: raw score -> 2 y log2(e), y = logit / cap
    const float m2cap = -2.f * p.cap_out;
    float eg[2][4];   // exponentials of slices i (even / odd), until packed
    auto exp_one = [&](int i, int k) {   // element 4(i%4) + k of row half i/4
      const int qs = i / 4;
      float x = sc_cur[qs][4 * (i % 4) + k];
      if constexpr (kMasked) {
        x = mask_select(x, kw[qs], 4 * (i % 4) + k);
        sc_cur[qs][4 * (i % 4) + k] = x;
      }
      if constexpr (CAP) {
        // Capped logit in base-2 units, cap log2(e) tanh y with y = logit / cap:
        // with r = 1 / (1 + e^{2y}), tanh y = 1 - 2r, which reaches +-1
        // exactly at the float range's ends, so the exponent is one FMA,
        // r (-2 cap log2 e) + (cap log2 e - base).  x 2^-100 lies far below
        // the rounding of any finite logit but keeps a masked key (-inf) at
        // -inf, without a select (which the compiler turns into a branch
        // around the cap).
        const float r = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * kc2));
        eg[i & 1][k] = __builtin_amdgcn_exp2f(__builtin_fmaf(r, m2cap, __builtin_fmaf(x, 0x1p-100f, kr[qs])));
      } else {
        eg[i & 1][k] = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c2e, -b2[qs]));
      }
    };
    // With the cap each element's exponent is a chain of three dependent
    // transcendentals (e^{2y}, the reciprocal, the exponential).  Run as one
    // chain per sub-slice, the in-order wave waits out each link's latency
    // and the matrix unit idles; so the chain is cut into three stages and
    // sub-slice e issues stage A of element e + 2, B of e + 1 and C of e,
    // each reading what the previous sub-slice produced.  Elements are
    // numbered e = 4 i + k (slice i, sub-slice k), as exp_one numbers them.
    float cap_e[4], cap_r[4];   // stage outputs, ring indexed by e % 4
    auto cap_a = [&](int e) {   // masked score (written back), e^{2y}
      const int i = e >> 2, k = e & 3, qs = i / 4, v = 4 * (i % 4) + k;
      float x = sc_cur[qs][v];
      if constexpr (kMasked) {
        x = mask_select(x, kw[qs], v);
        sc_cur[qs][v] = x;
      }
      cap_e[e & 3] = __builtin_amdgcn_exp2f(x * kc2);
    };
    auto cap_b = [&](int e) { cap_r[e & 3] = __builtin_amdgcn_rcpf(1.f + cap_e[e & 3]); };
    auto cap_c = [&](int e) {   // the capped logit's exponential, as in exp_one
      const int i = e >> 2, k = e & 3, qs = i / 4;
      const float x = sc_cur[qs][4 * (i % 4) + k];
      eg[i & 1][k] = __builtin_amdgcn_exp2f(__builtin_fmaf(cap_r[e & 3], m2cap, __builtin_fmaf(x, 0x1p-100f, kr[qs])));
    };
    auto pack = [&](int i, int pr) {   // elements 2pr, 2pr+1 of slice i -> P, row sum
      const int qs = i / 4, v0 = 4 * (i % 4) + 2 * pr;
      const float e0 = eg[i & 1][2 * pr], e1 = eg[i & 1][2 * pr + 1];
      const bf16x2 pp = {static_cast<__bf16>(e0), static_cast<__bf16>(e1)};
      pf_cur[qs][v0 / 8][v0 % 8] = pp[0];
      pf_cur[qs][v0 / 8][v0 % 8 + 1] = pp[1];
      // Row sums of the float exponentials (round to nearest even makes the
      // bf16 P that PV multiplies unbiased against them).  Plain adds: the
      // bf16 dot product with ones stalled beside the matrix unit.
      sum[qs] += e0 + e1;
      asm volatile("" : "+v"(sum[qs]));   // keep the sums in this slice
    };

    // slice 0: operands of MFMA slices 0 and 1
    reads_slice(0);
    reads_slice(1);
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      b2[qs] = rs.base[qs] == -INFINITY ? 0.f : rs.base[qs];
      kr[qs] = p.cap_out - b2[qs];
    }
    if constexpr (CAP) {   // the cap pipeline's first stages
      cap_a(0);
      cap_a(1);
      cap_b(0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // Each slice is four sub-slices of one matrix instruction each, with
    // about one matrix instruction's worth of other work beneath it (an
    // exponential, its FMA, half a pack): the wave issues in order, so
    // back-to-back matrix instructions would leave the VALU idle while the
    // matrix unit is busy, and the VALU work after them would run alone.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        mfma_one(i, sub);
        __builtin_amdgcn_sched_barrier(0);   // the matrix instruction leads its sub-slice
        if (sub == 0 && i + 2 < 8) reads_slice(i + 2);
        if (sub == 1) issue_loads(i);
        if (sub == 0 && i > 0) pack(i - 1, 1);
        if constexpr (CAP) {
          const int e = 4 * i + sub;
          if (e + 2 < 32) cap_a(e + 2);
          if (e + 1 < 32) cap_b(e + 1);
          cap_c(e);
        } else {
          exp_one(i, sub);
        }
        if (sub == 2) pack(i, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    pack(7, 1);
    static_assert(kKS <= 8 && kPVOps <= 8, "slice plan assumes at most 8 operands");
    // Keep this step's softmax results here: without a use in this block
    // the compiler sinks the exponentials into the next step, after its
    // branches, where they no longer overlap these MFMAs.
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      rs.l[qs] += sum[qs];
      step_sum[qs] = sum[qs];
    }
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
#pragma unroll
      for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(pf_cur[qs][h]));
      asm volatile("" : "+v"(rs.l[qs]));
    }
  };

  // Rare: some row's sum, step u's exponentials included (scores sc, weights
  // in pf, this lane's part of the step's sum in step_sum), has outgrown 2^40 --
  // its scores have grown far past the base fixed at its first step.  Such a
  // row moves its base up to the step's max (if that is higher): the output
  // accumulator and the sum of the earlier steps are rescaled by
  // 2^(old - new), and the step's weights and sum are formed again against
  // the new base (with the body's own formulas, so the step's values stay
  // consistent with the earlier ones).  Other rows keep their base (factor 1,
  // same weights).  Whole-wave code on a uniform branch.
  auto rebase = [&](f32x16 *sc, bf16x8 (*pf)[2], const float *step_sum) {
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const bool need = pair_max(rs.l[qs] > kRescaleSum ? 1.f : 0.f) > 0.f;
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[qs][v]);
      mx = pair_max(mx);
      float m2 = mx * c2e;
      if constexpr (CAP) {
        const float x = mx * p.c2;
        const float e = __builtin_amdgcn_exp2f(-2.f * kLog2e * fabsf(x));
        const float th = (1.f - e) * __builtin_amdgcn_rcpf(1.f + e);
        m2 = copysignf(th, x) * p.cap_out;
      }
      const float old_b = rs.base[qs];
      const float new_b = need ? fmaxf(m2, old_b) : old_b;
      const float alpha = __builtin_amdgcn_exp2f(old_b - new_b);
      rs.base[qs] = new_b;
      // the earlier steps' sum (rs.l includes this step's): the subtraction
      // errs by an ulp of the old sum, which alpha then makes negligible
      rs.l[qs] = (rs.l[qs] - step_sum[qs]) * alpha;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[dt][qs][v] *= alpha;
      const float kc2 = 2.f * kLog2e * p.c2, m2cap = -2.f * p.cap_out, kr = p.cap_out - new_b;
      float sum = 0.f;
#pragma unroll
      for (int v0 = 0; v0 < 16; v0 += 2) {
        float e[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float x = sc[qs][v0 + k];
          if constexpr (CAP) {
            const float rr = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * kc2));
            e[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(rr, m2cap, __builtin_fmaf(x, 0x1p-100f, kr)));
          } else {
            e[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c2e, -new_b));
          }
        }
        pf[qs][v0 / 8][v0 % 8] = static_cast<__bf16>(e[0]);
        pf[qs][v0 / 8][v0 % 8 + 1] = static_cast<__bf16>(e[1]);
        sum += e[0] + e[1];
      }
      rs.l[qs] += sum;
    }
  };

  for (int attempt = 0; attempt < 2; ++attempt) {
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      rs.base[qs] = base_init[qs];
      rs.l[qs] = 0.f;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[dt][qs][v] = 0.f;
    }
    rs.over = false;
    any_full = false;
    key_bits[0] = key_bits[1] = 0u;

    do {
      const int nb = w_len;
      if (nb == 0) break;
      const int N = kSteps * nb;   // pipeline steps

      // Loads of (virtual) iteration w, counted per wave: K(w+4) with, for
      // dense masks, the mask words of step w+4, and V(w+2).  Iterations
      // -4 and -3 of the prologue issue K only; from -2 on every iteration
      // issues both (in the last block, whose successors do not exist, they
      // load the block's own K and V again into stages it has finished with).
      auto count = [&](int w) -> int {
        return SG::kInsts + (has_bits ? 1 : 0) + (w >= -2 ? SG::kInsts : 0);
      };
      auto load_k = [&](int stage, int kv, int t) {
        issue_stage<D, false, kW, PAD>(k_st[stage], k_res, static_cast<int64_t>(kv) * kBK + kSK * t, wave, lane, krow, krow);
      };
      auto load_v = [&](int stage, int kv, int t) {
        issue_stage<D, true, kW, PAD>(v_st[stage], v_res, static_cast<int64_t>(kv) * kBK + kSK * t, wave, lane, vrow, vrow);
      };
      auto load_m = [&](int stage, int mn, int t) {
        if (has_bits) issue_mask(mn, t, stage);
      };
      // Half h of this wave's segments of a K or V stage.
      auto load_k_half = [&](int h, int stage, int kv, int t) {
        const int64_t r0 = static_cast<int64_t>(kv) * kBK + kSK * t;
        if constexpr (SG::kInsts == 4) {
          if (h == 0) {
            issue_seg<D, false, 0, kW, PAD>(k_st[stage], k_res, r0, wave, lane, krow, krow);
            issue_seg<D, false, 1, kW, PAD>(k_st[stage], k_res, r0, wave, lane, krow, krow);
          } else {
            issue_seg<D, false, 2, kW, PAD>(k_st[stage], k_res, r0, wave, lane, krow, krow);
            issue_seg<D, false, 3, kW, PAD>(k_st[stage], k_res, r0, wave, lane, krow, krow);
          }
        } else {
          if (h == 0) issue_seg<D, false, 0, kW, PAD>(k_st[stage], k_res, r0, wave, lane, krow, krow);
          else issue_seg<D, false, 1, kW, PAD>(k_st[stage], k_res, r0, wave, lane, krow, krow);
        }
      };
      auto load_v_half = [&](int h, int stage, int kv, int t) {
        const int64_t r0 = static_cast<int64_t>(kv) * kBK + kSK * t;
        if constexpr (SG::kInsts == 4) {
          if (h == 0) {
            issue_seg<D, true, 0, kW, PAD>(v_st[stage], v_res, r0, wave, lane, vrow, vrow);
            issue_seg<D, true, 1, kW, PAD>(v_st[stage], v_res, r0, wave, lane, vrow, vrow);
          } else {
            issue_seg<D, true, 2, kW, PAD>(v_st[stage], v_res, r0, wave, lane, vrow, vrow);
            issue_seg<D, true, 3, kW, PAD>(v_st[stage], v_res, r0, wave, lane, vrow, vrow);
          }
        } else {
          if (h == 0) issue_seg<D, true, 0, kW, PAD>(v_st[stage], v_res, r0, wave, lane, vrow, vrow);
          else issue_seg<D, true, 1, kW, PAD>(v_st[stage], v_res, r0, wave, lane, vrow, vrow);
        }
      };

      f32x16 sc_a[2], sc_b[2];         // scores: step being exponentiated / step being formed
      bf16x8 pf_a[2][2], pf_b[2][2];   // P of the step being exponentiated / being multiplied
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int h = 0; h < 2; ++h) pf_b[qs][h] = bf16x8{};   // PV(-1) adds exact zeros

      // Masking of freshly formed scores S(u) of a label-1 step.  Computable
      // masks (mostly label-2 blocks) mask right after the QK that formed
      // them.  Dense masks (mostly label-1 blocks) only fetch the key words
      // kw here; the next step's body masks S(u) element by element beside
      // its matrix instructions (kw is all ones for a label-2 block).  S(0) of
      // a row is always masked right away (first), since the row's exponent
      // base is set from it.  (One body for both kinds of block: a second,
      // unmasked copy of the step in the same loop pushed the kernel past
      // its registers.)
      unsigned kw[2] = {~0u, ~0u};
      auto finish = [&](f32x16 *sc, int lab, int stage, int key0, bool first) {
        if (lab == 1) {
          unsigned mw[2] = {0u, 0u};
          mask_words(stage, mw);
          if (!DENSE || first) {
            qk_drain();   // the scores were formed by the step that just ended
            wide_cap_mask<false, DENSE, true>(p, sc, key0, half, lo, hi, mw, key_bits);
          }
          if constexpr (DENSE) {
#pragma unroll
            for (int qs = 0; qs < 2; ++qs) {
              kw[qs] = lane_key_word<DENSE>(key0, half, lo, hi, mw, qs);
              key_bits[qs] |= kw[qs] & 0x0f0f0f0fu;
            }
          }
        } else {
          any_full = true;
          kw[0] = kw[1] = ~0u;
        }
      };

      // prologue: loads of virtual iterations -4..-1 (K(0..3), mask words of
      // steps 0..3, V(0..1), all in block 0), then S(0)
      int kv0 = ent_kv(0), mn0 = ent_mn(0), lab0 = ent_lab(0);
      int kv1 = ent_kv(min(1, nb - 1)), mn1 = ent_mn(min(1, nb - 1)), lab1 = ent_lab(min(1, nb - 1));
      const bool early = attempt == 0 && kv0 == dn_first && (!has_bits || mn0 == mn_first);
      if (!early) {
        load_k(0, kv0, 0); load_m(0, mn0, 0);
        load_k(1, kv0, 1); load_m(1, mn0, 1);
        load_k(2, kv0, 2); load_m(2, mn0, 2); load_v(0, kv0, 0);
        load_k(3, kv0, 3); load_m(3, mn0, 3); load_v(1, kv0, 1);
      }
      wait_at_most<kMaxInFlight>(count(-3) + count(-2) + count(-1));
      lds_barrier();
      wide_qk<D>(k_st[0], qf, lane, half, sc_a);
      finish(sc_a, lab0, 0, kv0 * kBK, true);
      if (__builtin_amdgcn_ballot_w64(rs.base[0] == -INFINITY || rs.base[1] == -INFINITY) != 0) set_base(sc_a);

      // Trip j runs the four steps u = 4j + t of block j.  Step u:
      //   top     wait for step u+1's K and mask words and step u-1's V
      //           (issued three iterations ago), barrier;
      //   body    QK(u+1) || softmax(u) || PV(u-1), straight-line, with the
      //           refills of the stages iteration u-1 finished with --
      //           K(u+4), mask(u+4), V(u+2) -- in its first four slices;
      //   finish  mask of S(u+1).
      // Step 0's PV(-1) multiplies zero P, and step N-1's QK(N) reads a stale
      // stage whose result is dropped, so all steps share one body.
      for (int j = 0; j < nb; ++j) {
        const bool more = j + 1 < nb;
        // walk entry j+2, for the next trip (a scalar load, one trip ahead)
        const int kv2_v = ent_kv(min(j + 2, nb - 1));
        const int mn2_v = ent_mn(min(j + 2, nb - 1));
        const int lab2_v = ent_lab(min(j + 2, nb - 1));
        // the block's four steps, masked or not (label 1 / 2)
        auto trip = [&](auto mc) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < kSteps; ++t) {
          const int u = kSteps * j + t;
          f32x16 *sc_cur = (t & 1) ? sc_b : sc_a;
          f32x16 *sc_nxt = (t & 1) ? sc_a : sc_b;
          bf16x8 (*pf_cur)[2] = (t & 1) ? pf_b : pf_a;
          bf16x8 (*pf_prv)[2] = (t & 1) ? pf_a : pf_b;
          // top
          wait_at_most<kMaxInFlight>(count(u - 2) + count(u - 1));
          lds_barrier();
          // refills of the stages step u-1 finished with, spread over the
          // first four slices: K(u+4) and its mask words, then V(u+2)
          auto refill = [&](int i) {
            if (i < 2) {
              load_k_half(i, t, kv1, t);
              if (i == 0) load_m(t, mn1, t);
            } else if (i < 4) {
              if (t < 2) load_v_half(i - 2, t + 2, kv0, t + 2);
              else load_v_half(i - 2, t - 2, kv1, t - 2);
            }
          };
          // body (with the refills), then the finish of S(u+1)
          float step_sum[2];
          body(u, sc_cur, sc_nxt, pf_cur, pf_prv, refill, step_sum, mc, kw);
          // once per block: a row whose sum has outgrown its base moves it
          if (t == kSteps - 1 && __builtin_amdgcn_ballot_w64(fmaxf(rs.l[0], rs.l[1]) > kRescaleSum) != 0)
            rebase(sc_cur, pf_cur, step_sum);
          if (t < kSteps - 1) finish(sc_nxt, lab0, t + 1, kv0 * kBK + kSK * (t + 1), false);
          else if (more) finish(sc_nxt, lab1, 0, kv1 * kBK, false);
        }
        };
        trip(std::integral_constant<bool, DENSE>{});
        kv0 = kv1;
        mn0 = mn1;
        lab0 = lab1;
        kv1 = kv2_v;
        mn1 = mn2_v;
        lab1 = lab2_v;
      }
      // drain: PV(N-1); step N-1 = 4(nb-1) + 3 exponentiated into pf_b
      wait_vmcnt<0>();
      lds_barrier();
      wide_pv<D>(v_st[(N - 1) % kStages], pf_b, lane, half, o);
    } while (false);

    // Rows whose sum outgrew kOverflowSum had a base far below their max;
    // rows whose sum is tiny had a base far above it.  Both run again with
    // the exact max as base.  A row with no allowed key (zero sum) is
    // already final: out 0, lse -inf.  Workgroup-uniform decision: both
    // waves run the same barriers.
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const float l_tot = pair_sum(rs.l[qs]);
      const bool has_key = any_full || pair_max(key_bits[qs] != 0u ? 1.f : 0.f) > 0.f;
      rs.over |= attempt == 0 && has_key && (l_tot < kUnderflowSum || !(l_tot <= kOverflowSum));
    }
    // Workgroup OR of the flag through LDS: __syncthreads_or would read the
    // workgroup size from the dispatch packet, which sits in host memory --
    // a load that costs microseconds at every workgroup's start.
    if (lane == 0) wg_any[wave] = __builtin_amdgcn_ballot_w64(rs.over) != 0 ? 1 : 0;
    __syncthreads();
    int any_over = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) any_over |= wg_any[w];
    if (attempt == 1 || any_over == 0) break;

    // Rare: some row's scores outgrew its base.  Find every row's exact max
    // (QK only, one stage at a time) and run the row again with it as base.
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) base_init[qs] = -INFINITY;
    {
      const int nb = w_len;
      for (int u = 0; u < kSteps * nb; ++u) {
        const int key0u = ent_kv(u / kSteps) * kBK + kSK * (u % kSteps);
        wait_vmcnt<0>();
        lds_barrier();
        issue_stage<D, false, kW, PAD>(k_st[0], k_res, key0u, wave, lane, krow, krow);
        if (has_bits) issue_mask(ent_mn(u / kSteps), u % kSteps, 0);
        wait_vmcnt<0>();
        lds_barrier();
        f32x16 sc[2];
        wide_qk<D>(k_st[0], qf, lane, half, sc);
        unsigned mw[2] = {0u, 0u}, unused[2] = {0u, 0u};
        if (ent_lab(u / kSteps) == 1) {
          if (has_bits) mask_words(0, mw);
          wide_cap_mask<CAP, DENSE, true>(p, sc, key0u, half, lo, hi, mw, unused);
        } else {
          wide_cap_mask<CAP, DENSE, false>(p, sc, key0u, half, lo, hi, mw, unused);
        }
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
          float mx = -INFINITY;
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[qs][v]);
          base_init[qs] = fmaxf(base_init[qs], pair_max(mx) * c2e);
        }
      }
    }
    wait_vmcnt<0>();
    lds_barrier();
  }

  // ---- epilogue: O / l, lse
  // The O^T registers hold a lane's row in 4-element pieces 8 columns apart,
  // so a direct store would scatter 64 rows' pieces over one instruction
  // (64 partial-line writes).  Each wave instead writes its 64 normalised
  // bf16 rows into its half of the K stages (16-byte chunks swizzled by row)
  // and stores them back 16 bytes per lane, whole rows per instruction.  Both
  // waves are past their last K-stage read (the barrier that ends the
  // attempt loop); a workgroup with no block still has its prologue loads in
  // flight into those stages, hence the wait.
  // The global stores are non-temporal: nothing in this kernel reads the
  // output again, and marking it so leaves L2 to the K/V lines that other
  // workgroups re-read (the soft-capped 16k GQA forward, whose K/V exceeds
  // L2 most, runs about 2% faster; outputs are unchanged).
  wait_vmcnt<0>();
  float inv[2], lse_row[2];
  const float sl2 = n_split > 1 ? -INFINITY : sink_lse2(p, hq);   // the merge adds a split's sinks
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
    row_finish(pair_sum(rs.l[qs]), rs.base[qs] == -INFINITY ? 0.f : rs.base[qs], sl2, inv[qs], lse_row[qs]);
  {
    constexpr int kRB = SG::kRowBytes;
    constexpr int kChunks = kRB / 16;
    auto swz_o = [](int rr) { return rr & (kChunks - 1); };
    // wave w's rows: the K stages hold waves 0 and 1, the V stages 2 and 3
    char *st = (wave < kWWaves ? &k_st[0][0] : &v_st[0][0]) + wr * 64 * kRB;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int rr = (lane & 31) + 32 * qs;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          union { __bf16 h[4]; u32x2 u; } pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) pk.h[e] = static_cast<__bf16>(o[dt][qs][4 * g + e] * inv[qs]);
          *reinterpret_cast<u32x2 *>(st + rr * kRB + (((4 * dt + g) ^ swz_o(rr)) * 16) + 8 * half) = pk.u;
        }
    }
    // this wave's rows only: its LDS writes and reads complete in order
    const int64_t row_w = static_cast<int64_t>(r) * kBQ + 64 * wr;   // the wave's first row
    const int64_t ostride = PAD ? mv : D;   // output row in elements (PAD: the caller's Dv)
    char *dst = n_split > 1
        ? reinterpret_cast<char *>(static_cast<__bf16 *>(p.part_o) +
                                   (((static_cast<int64_t>(split) * p.B + b) * p.Hq + hq) * p.Sq + row_w) * ostride)
        : reinterpret_cast<char *>(static_cast<__bf16 *>(p.out) +
                                   ((static_cast<int64_t>(b) * p.Hq + hq) * p.Sq + row_w) * ostride);
    constexpr int kRowsPer = 1024 / kRB;   // rows per instruction
#pragma unroll
    for (int i = 0; i < 64 / kRowsPer; ++i) {
      const int rr = kRowsPer * i + lane / kChunks, c = lane % kChunks;
      const u32x4 v = *reinterpret_cast<const u32x4 *>(st + rr * kRB + ((c ^ swz_o(rr)) * 16));
      if (!PAD || c * 8 < mv)   // PAD: the padding columns stay unstored
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(dst + rr * ostride * 2 + c * 16));
    }
  }
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int64_t q_row = q_row0 + 32 * qs;
    if (half == 0) {
      if (n_split > 1)
        __builtin_nontemporal_store(lse_row[qs],
                                    &p.part_lse[((static_cast<int64_t>(split) * p.B + b) * p.Hq + hq) * p.Sq + q_row]);
      else if (p.lse)
        __builtin_nontemporal_store(lse_row[qs], &p.lse[(static_cast<int64_t>(b) * p.Hq + hq) * p.Sq + q_row]);
    }
  }
}

// Merge of the key splits' partial results into out and lse.  With
// lse_s the partial lse of split s over its keys and o_s its normalised
// output: lse = log sum_s e^(lse_s), out = sum_s e^(lse_s - lse) o_s -- the
// flash rescaling of partial results (splash explainer, FAQ "What does ring
// attention add on top of the splash kernel?").  Sinks join the sum once,
// here.  A split with no allowed key has lse_s = -inf and adds nothing
// (whatever its o_s holds).  Each thread moves 8 consecutive output
// elements of one row; the D/8 threads of a row sit in one wavefront.  The
// split count is a template parameter, so every load of a thread -- the S
// lses and the S partial rows -- goes out before the first one is used.  The
// partials are read once, with non-temporal loads (about 2% off a random
// dense 2k step), and the results stored non-temporal.
template <int D, int S>
__global__ __launch_bounds__(256)
void merge_splits(const FwdParams p) {
  constexpr int kTPR = D / 8;                 // threads per row
  const int64_t rows = p.B * p.Hq * p.Sq;
  const int64_t row = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) / kTPR;
  const int c0 = (threadIdx.x % kTPR) * 8;
  const int dv = p.padded ? p.dv : D;         // row length of the partials and the output
  if (row >= rows || c0 >= dv) return;
  const int64_t plane = rows;                 // rows per split
  float ls[S];
  union { u32x4 u; __bf16 h[8]; } x[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    ls[s] = __builtin_nontemporal_load(&p.part_lse[s * plane + row]);
    x[s].u = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4 *>(static_cast<const __bf16 *>(p.part_o) + (s * plane + row) * dv + c0));
  }
  float m = -INFINITY;
#pragma unroll
  for (int s = 0; s < S; ++s) m = fmaxf(m, ls[s]);
  const int hq = static_cast<int>((row / p.Sq) % p.Hq);
  const float sl2 = sink_lse2(p, hq);        // log2 of the sinks' sum, or -inf
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float l_sum = 0.f, lse2 = -INFINITY;
  if (m != -INFINITY) {
    const float m2 = m * kLog2e;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      // e^(-inf) = 0 weighs an empty split out; its o_s may hold anything
      // finite or not, so it is skipped rather than multiplied by zero
      if (ls[s] == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f(ls[s] * kLog2e - m2);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += w * static_cast<float>(x[s].h[e]);
      l_sum += w;
    }
    lse2 = m2 + __builtin_amdgcn_logf(l_sum);  // log2 of the keys' sum
  }
  float scale = m != -INFINITY ? 1.f / l_sum : 0.f;
  float lse2_tot = lse2;
  if (sl2 != -INFINITY) {
    const float mx = fmaxf(lse2, sl2);
    lse2_tot = mx + __builtin_amdgcn_logf(__builtin_amdgcn_exp2f(lse2 - mx) + __builtin_amdgcn_exp2f(sl2 - mx));
    if (m != -INFINITY) scale *= __builtin_amdgcn_exp2f(lse2 - lse2_tot);
  }
  union { __bf16 h[8]; u32x4 u; } pk;
#pragma unroll
  for (int e = 0; e < 8; ++e) pk.h[e] = static_cast<__bf16>(acc[e] * scale);
  __builtin_nontemporal_store(pk.u, reinterpret_cast<u32x4 *>(static_cast<__bf16 *>(p.out) + row * dv + c0));
  if (p.lse && c0 == 0) __builtin_nontemporal_store(lse2_tot * kLn2, &p.lse[row]);
}

template <int D, int S>
void launch_merge(const FwdParams &p, hipStream_t stream) {
  const int64_t threads = p.B * p.Hq * p.Sq * (D / 8);
  hipLaunchKernelGGL((merge_splits<D, S>), dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, stream,
                     p);
}

template <int D, bool CAP, bool DENSE, bool PAD>
hipError_t launch_wide_pad(const FwdParams &p, hipStream_t stream) {
  if constexpr (D == 128 && !DENSE) {
    if (p.head_pairs) {
      const int64_t blocks = p.B * (p.Hq / 2) * p.nq * p.kv_splits;
      hipLaunchKernelGGL((splash_fwd_wide<D, CAP, DENSE, 2, PAD>), dim3(static_cast<unsigned>(blocks)),
                         dim3(2 * kWThreads), 0, stream, p);
    }
  }
  if (!p.head_pairs || D != 128 || DENSE) {
    const int64_t blocks = p.B * p.Hq * p.nq * p.kv_splits;
    hipLaunchKernelGGL((splash_fwd_wide<D, CAP, DENSE, 1, PAD>), dim3(static_cast<unsigned>(blocks)), dim3(kWThreads),
                       0, stream, p);
  }
  switch (p.kv_splits) {   // 1..8, checked by the caller
    case 1: break;
    case 2: launch_merge<D, 2>(p, stream); break;
    case 3: launch_merge<D, 3>(p, stream); break;
    case 4: launch_merge<D, 4>(p, stream); break;
    case 5: launch_merge<D, 5>(p, stream); break;
    case 6: launch_merge<D, 6>(p, stream); break;
    case 7: launch_merge<D, 7>(p, stream); break;
    default: launch_merge<D, 8>(p, stream); break;
  }
  return hipGetLastError();
}

template <int D, bool CAP, bool DENSE>
hipError_t launch_wide(const FwdParams &p, hipStream_t stream) {
  return p.padded ? launch_wide_pad<D, CAP, DENSE, true>(p, stream) : launch_wide_pad<D, CAP, DENSE, false>(p, stream);
}

template <int D, bool CAP, bool DENSE>
hipError_t launch_f32(const FwdParams &p, hipStream_t stream) {
  const int64_t blocks = p.B * p.Hq * p.nq;
  hipLaunchKernelGGL((splash_fwd_f32<D, CAP, DENSE>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bf16(const FwdParams &p, hipStream_t stream) {
  if (p.cap) return p.dense ? launch_wide<D, true, true>(p, stream) : launch_wide<D, true, false>(p, stream);
  return p.dense ? launch_wide<D, false, true>(p, stream) : launch_wide<D, false, false>(p, stream);
}

template <int D>
hipError_t launch_float(const FwdParams &p, hipStream_t stream) {
  if (p.cap) return p.dense ? launch_f32<D, true, true>(p, stream) : launch_f32<D, true, false>(p, stream);
  return p.dense ? launch_f32<D, false, true>(p, stream) : launch_f32<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdParams &p, int dtype, hipStream_t stream) {
  if (dtype == 0) return p.D == 64 ? launch_bf16<64>(p, stream) : launch_bf16<128>(p, stream);
  return p.D == 64 ? launch_float<64>(p, stream) : launch_float<128>(p, stream);
}

}  // namespace splash
