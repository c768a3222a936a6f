// Decode: one new query per (batch, query head) against the whole key/value
// cache (q_len = 1).  The EasyDeL block-sparse module turns the causal mask
// off in decode mode and falls back to plain attention for a single query on
// TPU (EasyDeL BlockSparseAttn.forward_native); this is the MI355X-native
// path for that case.  It is the forward's masked softmax attention with
// every key allowed, split along the keys (flash decoding):
//   1. partials (decode_mfma): a workgroup per (batch, kv head, key range
//      of a few thousand keys) computes, for the G query heads of the kv
//      head's GQA group at once, the range's max m_c, sum l_c and
//      unnormalised output o_c.  It streams the range through a ring of five
//      32-key K/V stages in LDS, filled by direct-to-LDS loads four stages
//      ahead, so the cache is read without pauses; each of its two waves
//      keeps its own online softmax over half of every stage's keys, and the
//      waves merge once at the end;
//   2. merge: a wave per (batch, query head) combines the ranges,
//      m = max m_c, l = sum l_c e^(m_c - m), out = sum o_c e^(m_c - m) / l,
//      lse = m + log l (natural log).
// HBM-bound: every K and V row of the cache is read once per kv head and
// serves the whole GQA group.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "splash_kernel.h"

namespace splash {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Streaming partial kernel.
constexpr int kSKeys = 32;               // keys per stage
constexpr int kSStages = 5;              // ring of stages; loads run four ahead
constexpr int kSWaves = 2;               // 16 keys of every stage per wave
constexpr int kSThreads = 64 * kSWaves;
constexpr float kBaseSlack = 32.f;       // headroom of the exponent base (base 2)

// Buffer resource over `bytes` bytes at `base`; reads past the end return 0.
__device__ __forceinline__ i32x4 stream_rsrc(const void *base, int64_t bytes) {
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

// Stage geometry: 32 key rows of D bf16, rows of 16-byte chunks, chunk c of
// row r stored at chunk c ^ swz(r), so the 16 rows one K operand read spans
// (one chunk each) and the rows of a transposing V read spread over
// several bank groups instead of one.
template <int D>
struct SStage {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = kRowBytes / 16;            // 16 (D = 128) or 8 (D = 64)
  static constexpr int kBytes = kSKeys * kRowBytes;         // 8 KiB or 4 KiB
  static constexpr int kSegsPerWave = kBytes / 1024 / kSWaves;   // 1 KiB loads per wave: 4 or 2
  static constexpr int kRowsPerSeg = 1024 / kRowBytes;
  __device__ static int swz(int row) {
    if constexpr (D == 128) return row & 3;
    else return (row >> 1) & 1;
  }
};

// Direct-to-LDS loads of this wave's share of one stage: rows
// [row0, row0 + 32) of a (batch, kv head) K or V array.  Lane l lands on
// bytes 16 l of each 1 KiB segment; the swizzle is applied on the global side.
// With the row counts above, the row a lane lands on has the same swizzle in
// every segment, so one offset register and M0 value serve all segments (the
// instruction offset moves both the LDS and the global address).  Issued from
// inline assembly so the compiler does not order LDS reads of other stages
// behind them; completion is awaited with s_waitcnt vmcnt before a barrier.
// The loads are non-temporal: each cache row is read once per call, and
// streaming it past L2's retained lines reads the cache about 10% faster
// (a plain read with and without the hint differs as much).
template <int D>
__device__ __forceinline__ void stream_stage(char *lds, i32x4 res, int64_t row0, int wave, int lane) {
  using SG = SStage<D>;
  const int row = lane / SG::kChunks;   // + 1 KiB segment * kRowsPerSeg, same swizzle
  const uint32_t voff = static_cast<uint32_t>(row * SG::kRowBytes + ((lane % SG::kChunks) ^ SG::swz(row)) * 16);
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) char *)(lds + wave * SG::kSegsPerWave * 1024)));
  const uint32_t soff = static_cast<uint32_t>(row0 * SG::kRowBytes) + wave * SG::kSegsPerWave * 1024;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  if constexpr (SG::kSegsPerWave == 4) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen nt lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:1024 nt lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:2048 nt lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:3072 nt lds"
        :: "s"(m0), "v"(voff), "s"(res), "s"(soff) : "memory", "m0");
  } else {
    static_assert(SG::kSegsPerWave == 2, "stage loads per wave");
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen nt lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:1024 nt lds"
        :: "s"(m0), "v"(voff), "s"(res), "s"(soff) : "memory", "m0");
  }
#pragma clang diagnostic pop
}

// stream_stage for padded head dims: the arrays' rows hold `mrow` bytes (a
// multiple of 32, at most the stage's row), so each 1 KiB segment takes its
// own M0 and per-lane offsets, and a lane whose chunk lies in the padding
// gets an offset past the resource's end, which reads zeros (the stages'
// padding columns are zeroed before their first load and stay zero).
template <int D>
__device__ __forceinline__ void stream_stage_padded(char *lds, i32x4 res, int64_t row0, int wave, int lane,
                                                    uint32_t mrow) {
  using SG = SStage<D>;
#pragma unroll
  for (int i = 0; i < SG::kSegsPerWave; ++i) {
    const int seg = wave * SG::kSegsPerWave + i;
    const int row = seg * SG::kRowsPerSeg + lane / SG::kChunks;
    const int c = (lane % SG::kChunks) ^ SG::swz(row);
    const uint32_t voff = static_cast<uint32_t>(c * 16) < mrow
        ? static_cast<uint32_t>(row0 + row) * mrow + static_cast<uint32_t>(c * 16)
        : 0x80000000u;
    const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) char *)(lds + seg * 1024)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :: "s"(m0), "v"(voff), "s"(res) : "memory", "m0");
#pragma clang diagnostic pop
  }
}

// Wait until at most n of this wave's vector-memory loads are in flight.
template <int N>
__device__ __forceinline__ void stream_wait(int n) {
  if constexpr (N == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (n >= N) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
    else stream_wait<N - 1>(n);
  }
}

// Partial kernel: a workgroup of two waves per (b, kv head, key range), for
// every group size up to 16.  A wave takes 16 keys of every stage; the dot
// products and the output accumulation run on 16x16 MFMAs.
//  - Scores, transposed: S^T (16 keys x 16 heads) = K Q^T with D / 32
//    16x16x32 bf16 products.  K rows come from LDS (one 16-byte read per
//    product); Q^T stays in registers, its rows past G zero.  Lane l then
//    holds head l % 16 and keys 4 (l / 16) + 0..3.
//  - Output, transposed: O^T (D x 16 heads) += V^T P^T with D / 16 16x16x16
//    products.  P^T is the lane's four weights rounded to bf16, already in
//    the operand layout; V^T comes from the row-major V stage through the
//    transposing LDS read ds_read_b64_tr_b16 (lane l gets column l % 16 of
//    a 4 x 16 block of rows 4 (l / 16) + 0..3).
// Every register of a lane belongs to one head, so a rescale is lane-local.
// PAD: head dims other than D (rows of p.dim elements), zero-padded: Q^T and
// the stages are zero past p.dim, so the scores sum only real columns and
// the output's padding columns (zero) are dropped by the merge.
template <int D, int G, bool CAP, bool PAD>
__global__ __launch_bounds__(kSThreads, 1) void decode_mfma(const DecodeParams p) {
  using SG = SStage<D>;
  constexpr int kKC = D / 32;                  // QK products per stage and wave
  constexpr int kDT = D / 16;                  // PV products (output tiles)
  constexpr int kLoadsPerStage = 2 * SG::kSegsPerWave;
  constexpr int kStBytes = 2 * kSStages * SG::kBytes;
  constexpr int kOutBytes = kSWaves * G * D * 4;
  constexpr int kMrgBytes = 2 * kSWaves * G * 4;
  constexpr int kArena = kStBytes > kOutBytes + kMrgBytes ? kStBytes : kOutBytes + kMrgBytes;
  __shared__ __attribute__((aligned(1024))) char smem[kArena];
  char (*k_st)[SG::kBytes] = reinterpret_cast<char (*)[SG::kBytes]>(smem);
  char (*v_st)[SG::kBytes] = reinterpret_cast<char (*)[SG::kBytes]>(smem + kSStages * SG::kBytes);
  float (*mrg_m)[G] = reinterpret_cast<float (*)[G]>(smem + kOutBytes);
  float (*mrg_l)[G] = reinterpret_cast<float (*)[G]>(smem + kOutBytes + kSWaves * G * 4);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane & 15, grp = lane >> 4;    // head; group of four keys
  const bool hv = h < G;
  const int unit = blockIdx.x;                 // (b, hkv)
  const int split = blockIdx.y;
  const int b = unit / p.Hkv, hkv = unit % p.Hkv;
  const int64_t kb = static_cast<int64_t>(split) * p.split_keys;
  const int64_t ke = min(kb + p.split_keys, p.Skv);
  const int nst = static_cast<int>((ke - kb + kSKeys - 1) / kSKeys);   // >= 1

  const int md = PAD ? p.dim : D;                // row length in memory
  const int64_t kv_head = (static_cast<int64_t>(b) * p.Hkv + hkv) * p.Skv;
  const i32x4 k_res = stream_rsrc(static_cast<const __bf16 *>(p.k) + kv_head * md, p.Skv * md * 2);
  const i32x4 v_res = stream_rsrc(static_cast<const __bf16 *>(p.v) + kv_head * md, p.Skv * md * 2);
  auto issue = [&](int st) {
    const int64_t row0 = kb + static_cast<int64_t>(st) * kSKeys;
    if constexpr (PAD) {
      stream_stage_padded<D>(k_st[st % kSStages], k_res, row0, wave, lane, static_cast<uint32_t>(md * 2));
      stream_stage_padded<D>(v_st[st % kSStages], v_res, row0, wave, lane, static_cast<uint32_t>(md * 2));
    } else {
      stream_stage<D>(k_st[st % kSStages], k_res, row0, wave, lane);
      stream_stage<D>(v_st[st % kSStages], v_res, row0, wave, lane);
    }
  };
  if constexpr (PAD) {
    // the stages' padding columns start (and stay) zero; written and
    // published before any load into the stages
    constexpr int kVec = kStBytes / 16;
    static_assert(kVec % kSThreads == 0, "whole zeroing rounds");
#pragma unroll
    for (int i = 0; i < kVec / kSThreads; ++i)
      reinterpret_cast<u32x4 *>(smem)[tid + kSThreads * i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  }
#pragma unroll
  for (int st = 0; st < kSStages - 1; ++st)
    if (st < nst) issue(st);

  // Q^T operand: head h, dims 32 kk + 8 grp + 0..7
  bf16x8 qb[kKC];
  {
    const __bf16 *qr = static_cast<const __bf16 *>(p.q) + (static_cast<int64_t>(b) * p.Hq + hkv * G + (hv ? h : 0)) * md;
#pragma unroll
    for (int kk = 0; kk < kKC; ++kk) {
      u32x4 w = u32x4{0u, 0u, 0u, 0u};
      if (!PAD || 32 * kk + 8 * grp < md) w = *reinterpret_cast<const u32x4 *>(qr + 32 * kk + 8 * grp);
      if (!hv) w = u32x4{0u, 0u, 0u, 0u};
      __builtin_memcpy(&qb[kk], &w, sizeof(w));
    }
  }
  // byte offsets in a stage: the K operand row 16 wave + h, chunk 4 kk + grp;
  // the transposing V read of rows 16 wave + 4 grp + h / 4, columns
  // 16 dt + 4 (h % 4) + 0..3
  int koff[kKC], voff[kDT];
  {
    const int kr = 16 * wave + h;
#pragma unroll
    for (int kk = 0; kk < kKC; ++kk) koff[kk] = kr * SG::kRowBytes + (((4 * kk + grp) ^ SG::swz(kr)) * 16);
    const int vr = 16 * wave + 4 * grp + (h >> 2);
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
      const int col = 16 * dt + 4 * (h & 3);
      voff[dt] = vr * SG::kRowBytes + (((col >> 3) ^ SG::swz(vr)) * 16) + (col & 7) * 2;
    }
  }

  float m = -INFINITY, lsum = 0.f;   // head h's base (base 2) and this lane's share of its sum
  f32x4 o[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int u = 0; u < nst; ++u) {
    const int ahead = min(nst - 1 - u, kSStages - 2);
    stream_wait<(kSStages - 2) * kLoadsPerStage>(ahead * kLoadsPerStage);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (u + kSStages - 1 < nst) issue(u + kSStages - 1);
    const char *ks = k_st[u % kSStages];
    const char *vs = v_st[u % kSStages];

    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kKC; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(ks + koff[kk]);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[kk], sacc, 0, 0, 0);
    }
    const int64_t key0 = kb + static_cast<int64_t>(u) * kSKeys + 16 * wave + 4 * grp;
    float s2[4];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x;
      if constexpr (CAP) {
        const float xs = sacc[j] * p.c2;
        const float e = __builtin_amdgcn_exp2f(-2.f * kLog2e * fabsf(xs));
        const float th = (1.f - e) * __builtin_amdgcn_rcpf(1.f + e);
        x = copysignf(th, xs) * p.cap_out;
      } else {
        x = sacc[j] * p.c2;
      }
      s2[j] = hv && key0 + j < ke ? x : -INFINITY;
      mx = fmaxf(mx, s2[j]);
    }
    // Head h's exponent base is set by its first valid scores and moves,
    // with a rescale, only when a score exceeds it by more than 32 (base-2
    // units): weights stay below 2^32 and a step normally needs no
    // cross-lane max.  The test is a wave-wide ballot; the four lanes of a
    // head agree on the base.
    if (__builtin_amdgcn_ballot_w64(mx > m + kBaseSlack) != 0) {
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m, mx);
      const float a = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
      lsum *= a;
#pragma unroll
      for (int dt = 0; dt < kDT; ++dt) o[dt] *= a;
      m = mn;
    }
    float pe[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) pe[j] = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s2[j] - m);
    lsum += (pe[0] + pe[1]) + (pe[2] + pe[3]);
    const bf16x2 p01 = {static_cast<__bf16>(pe[0]), static_cast<__bf16>(pe[1])};
    const bf16x2 p23 = {static_cast<__bf16>(pe[2]), static_cast<__bf16>(pe[3])};
    const bf16x2 pp[2] = {p01, p23};
    s16x4 pb;
    __builtin_memcpy(&pb, pp, sizeof(pb));
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt) {
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (s16x4 __attribute__((address_space(3))) *)(vs + voff[dt]));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[dt], 0, 0, 0);
    }
  }

  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // stages free
  float *o_lds = reinterpret_cast<float *>(smem);   // [kSWaves][G][D]
  if (hv) {
#pragma unroll
    for (int dt = 0; dt < kDT; ++dt)
      *reinterpret_cast<float4 *>(&o_lds[(wave * G + h) * D + 16 * dt + 4 * grp]) =
          make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (grp == 0) {
      mrg_m[wave][h] = m;
      mrg_l[wave][h] = lsum;
    }
  }
  __syncthreads();
  const int64_t slot = static_cast<int64_t>(unit) * p.n_chunks + split;
  for (int idx = tid; idx < G * D; idx += kSThreads) {
    const int g = idx / D, d = idx % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSWaves; ++w) mm = fmaxf(mm, mrg_m[w][g]);
    float x = 0.f, lt = 0.f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kSWaves; ++w) {
        const float a = mrg_m[w][g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrg_m[w][g] - mm);
        x += a * o_lds[(w * G + g) * D + d];
        lt += a * mrg_l[w][g];
      }
    }
    p.ws_o[(slot * G + g) * D + d] = x;
    if (d == 0) {
      p.ws_m[slot * G + g] = mm;
      p.ws_l[slot * G + g] = lt;
    }
  }
}

// Merge of the chunks: one wave per (b, hq); lane i holds columns 2i, 2i+1
// (D = 128) or column i (D = 64).
template <int D, int G>
__global__ __launch_bounds__(64) void decode_merge(const DecodeParams p) {
  constexpr int kCols = D / 64;
  const int lane = threadIdx.x;
  const int bhq = blockIdx.x;
  const int b = bhq / p.Hq, hq = bhq % p.Hq;
  const int hkv = hq / G, g = hq % G;
  const int64_t unit = static_cast<int64_t>(b) * p.Hkv + hkv;
  float m = -INFINITY;
  for (int c = 0; c < p.n_chunks; ++c) m = fmaxf(m, p.ws_m[(unit * p.n_chunks + c) * G + g]);
  float l = 0.f, o[kCols];
#pragma unroll
  for (int j = 0; j < kCols; ++j) o[j] = 0.f;
  if (m != -INFINITY) {
    // An empty range has m = -inf (weight e^-inf = 0) and a written zero sum
    // and output, so no range is skipped: the loop body has no branch, and
    // the unrolled iterations' loads go out together.
#pragma unroll 8
    for (int c = 0; c < p.n_chunks; ++c) {
      const int64_t slot = (unit * p.n_chunks + c) * G + g;
      const float w = __builtin_amdgcn_exp2f(p.ws_m[slot] - m);
      l += w * p.ws_l[slot];
#pragma unroll
      for (int j = 0; j < kCols; ++j) o[j] += w * p.ws_o[slot * D + kCols * lane + j];
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const int md = p.padded ? p.dim : D;   // output row length (padded dims: the caller's)
  __bf16 *orow = static_cast<__bf16 *>(p.out) + static_cast<int64_t>(bhq) * md;
#pragma unroll
  for (int j = 0; j < kCols; ++j)
    if (kCols * lane + j < md) orow[kCols * lane + j] = static_cast<__bf16>(o[j] * inv);
  if (p.lse && lane == 0) p.lse[bhq] = l > 0.f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
}

template <int D, int G>
hipError_t go(const DecodeParams &p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p.B * p.Hkv), static_cast<unsigned>(p.n_chunks));
  if (p.padded) {
    if (p.cap) hipLaunchKernelGGL((decode_mfma<D, G, true, true>), grid, dim3(kSThreads), 0, s, p);
    else hipLaunchKernelGGL((decode_mfma<D, G, false, true>), grid, dim3(kSThreads), 0, s, p);
  } else {
    if (p.cap) hipLaunchKernelGGL((decode_mfma<D, G, true, false>), grid, dim3(kSThreads), 0, s, p);
    else hipLaunchKernelGGL((decode_mfma<D, G, false, false>), grid, dim3(kSThreads), 0, s, p);
  }
  hipLaunchKernelGGL((decode_merge<D, G>), dim3(static_cast<unsigned>(p.B * p.Hq)), dim3(64), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t go_g(const DecodeParams &p, hipStream_t s) {
  switch (p.group) {
    case 1: return go<D, 1>(p, s);
    case 2: return go<D, 2>(p, s);
    case 4: return go<D, 4>(p, s);
    case 8: return go<D, 8>(p, s);
    default: return go<D, 16>(p, s);
  }
}

}  // namespace

// Keys per partial workgroup: whole 32-key stages, about 512 workgroups over
// the launch (two per CU) when the cache is long enough, and at least four
// stages per workgroup.  (1024 shorter ranges measured 9% slower: each range
// ends with a merge of its waves.)  The same for every group size and D.
int64_t decode_split_keys(int64_t units, int64_t group, int64_t D, int64_t Skv) {
  (void)group;
  (void)D;
  if (Skv <= 0 || units <= 0) return kSKeys;
  const int64_t stages = (Skv + kSKeys - 1) / kSKeys;
  int64_t splits = (512 + units - 1) / units;
  splits = std::max<int64_t>(1, std::min(splits, (stages + 3) / 4));
  return (stages + splits - 1) / splits * kSKeys;
}

int64_t decode_chunks(int64_t units, int64_t group, int64_t D, int64_t Skv) {
  const int64_t k = decode_split_keys(units, group, D, Skv);
  return (Skv + k - 1) / k;
}

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream) {
  return p.D == 64 ? go_g<64>(p, stream) : go_g<128>(p, stream);
}

// Scratch of the allocation-free decode entry point: the per-range partial
// max, sum and output that splash_decode keeps in its caller's workspace.
// Each GPU the library runs on holds its own copy for the life of the
// process.  In host code `scratch` names a host-side stand-in, not device
// memory, so its device address is looked up once per device and only that
// address is handed to kernels.
static __device__ __align__(256) float scratch[kDecodeStaticScratchBytes / sizeof(float)];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices] = {};
}  // namespace

hipError_t decode_static_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace splash
