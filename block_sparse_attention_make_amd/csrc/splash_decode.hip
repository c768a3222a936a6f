// Decode: one new query per (batch, query head) against the whole key/value
// cache (q_len = 1).  The EasyDeL block-sparse module turns the causal mask
// off in decode mode and falls back to plain attention for a single query on
// TPU (EasyDeL BlockSparseAttn.forward_native); this is the MI355X-native
// path for that case.  It is the forward's masked softmax attention with
// every key allowed, split along the keys (flash decoding):
//   1. partials (decode_stream): a workgroup per (batch, kv head, key range
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

#include "splash_kernel.h"

namespace splash {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Streaming partial kernel.
constexpr int kSKeys = 32;               // keys per stage
constexpr int kSStages = 5;              // ring of stages; loads run four ahead
constexpr int kSWaves = 2;               // 16 keys of every stage per wave
constexpr int kSThreads = 64 * kSWaves;
constexpr float kBaseSlack = 32.f;       // see the exponent base in decode_stream

// Buffer resource over `bytes` bytes at `base`; reads past the end return 0.
__device__ __forceinline__ i32x4 stream_rsrc(const void *base, int64_t bytes) {
  const int n = bytes > 0x7fffffffLL ? 0x7fffffff : static_cast<int>(bytes);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
  i32x4 v;
  __builtin_memcpy(&v, &r, sizeof(v));
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __builtin_amdgcn_readfirstlane(v[i]);
  return v;
}

// Stage geometry: 32 key rows of D bf16, rows of 16-byte chunks, chunk c of
// row r stored at chunk c ^ swz(r).  Lane (key kw, part pt) of a wave reads
// the chunks of its quarter of a row; with the swizzle the 16 lanes of each
// quarter-wave of a 16-byte LDS read hit 16 different bank groups.
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
        "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:3072 lds"
        :: "s"(m0), "v"(voff), "s"(res), "s"(soff) : "memory", "m0");
  } else {
    static_assert(SG::kSegsPerWave == 2, "stage loads per wave");
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen offset:1024 lds"
        :: "s"(m0), "v"(voff), "s"(res), "s"(soff) : "memory", "m0");
  }
#pragma clang diagnostic pop
}

// Two bf16 from one 32-bit word (element 0 in the low half).  Through a copy:
// hipcc lowered __builtin_bit_cast of an ext-vector element as element 0 of
// the vector whatever the index.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) {
  bf16x2 r;
  __builtin_memcpy(&r, &w, sizeof(r));
  return r;
}

// Sum over the L lanes that hold the parts of one key's row (L = 4: a quad;
// 8: two quads; 16: a DPP row) with DPP lane moves: VALU only, no LDS round
// trip.
template <int L>
__device__ __forceinline__ float parts_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xb1, 0xf, 0xf, false));   // lanes ^ 1
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4e, 0xf, 0xf, false));   // lanes ^ 2
  if constexpr (L >= 8)   // row_half_mirror: lane i <-> 7 - i of each 8, the other quad
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false));
  if constexpr (L == 16)  // row_mirror: lane i <-> 15 - i of each 16, the other half-row
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xf, 0xf, false));
  return x;
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

template <int D, int G, bool CAP>
__global__ __launch_bounds__(kSThreads, 1) void decode_stream(const DecodeParams p) {
  using SG = SStage<D>;
  // L lanes share a key row: 4 while G * D <= 512, 8 up to 1024, else 16,
  // so a lane holds at most 128 outputs and 64 Q words; a wave covers 64 / L
  // keys per pass and 16 keys of every stage in 16 L / 64 passes.
  constexpr int L = G * D <= 512 ? 4 : G * D <= 1024 ? 8 : 16;
  constexpr int kKw = 64 / L;                  // keys per pass of a wave
  constexpr int kPasses = kSKeys / kSWaves / kKw;
  constexpr int kPart = D / L;                 // elements of a row per lane
  constexpr int kPC = kPart / 8;               // 16-byte chunks per lane
  static_assert(kPC >= 1 && kPasses >= 1, "lane split");
  constexpr int kLoadsPerStage = 2 * SG::kSegsPerWave;   // K and V, per wave
  // One arena: the stages during the loop; the waves' partial outputs and
  // the merge scalars after it.  80 KiB at D = 128, so two workgroups share
  // a CU's 160 KiB.
  constexpr int kStBytes = 2 * kSStages * SG::kBytes;
  constexpr int kOutBytes = kSWaves * kKw * G * D * 4;   // partial outputs at the end
  constexpr int kMrgBytes = 2 * kSWaves * G * 4;
  constexpr int kArena = kStBytes > kOutBytes + kMrgBytes ? kStBytes : kOutBytes + kMrgBytes;
  __shared__ __attribute__((aligned(1024))) char smem[kArena];
  char (*k_st)[SG::kBytes] = reinterpret_cast<char (*)[SG::kBytes]>(smem);
  char (*v_st)[SG::kBytes] = reinterpret_cast<char (*)[SG::kBytes]>(smem + kSStages * SG::kBytes);
  // (written after the loop, when the stages are free)
  float (*mrg_m)[G] = reinterpret_cast<float (*)[G]>(smem + kOutBytes);
  float (*mrg_l)[G] = reinterpret_cast<float (*)[G]>(smem + kOutBytes + kSWaves * G * 4);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = lane / L, pt = lane % L;      // key of the pass, part of the row
  const int unit = blockIdx.x;                 // (b, hkv)
  const int split = blockIdx.y;
  const int b = unit / p.Hkv, hkv = unit % p.Hkv;
  const int64_t kb = static_cast<int64_t>(split) * p.split_keys;
  const int64_t ke = min(kb + p.split_keys, p.Skv);
  const int nst = static_cast<int>((ke - kb + kSKeys - 1) / kSKeys);   // >= 1

  const int64_t kv_head = (static_cast<int64_t>(b) * p.Hkv + hkv) * p.Skv;
  const i32x4 k_res = stream_rsrc(static_cast<const __bf16 *>(p.k) + kv_head * D, p.Skv * SG::kRowBytes);
  const i32x4 v_res = stream_rsrc(static_cast<const __bf16 *>(p.v) + kv_head * D, p.Skv * SG::kRowBytes);
  auto issue = [&](int st) {   // stage st of this range into ring slot st % kSStages
    stream_stage<D>(k_st[st % kSStages], k_res, kb + static_cast<int64_t>(st) * kSKeys, wave, lane);
    stream_stage<D>(v_st[st % kSStages], v_res, kb + static_cast<int64_t>(st) * kSKeys, wave, lane);
  };
#pragma unroll
  for (int st = 0; st < kSStages - 1; ++st)
    if (st < nst) issue(st);

  // this lane's part of the G query rows, as bf16 pairs
  uint32_t qp[G][kPart / 2];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const __bf16 *qr = static_cast<const __bf16 *>(p.q) + (static_cast<int64_t>(b) * p.Hq + hkv * G + g) * D + kPart * pt;
#pragma unroll
    for (int c = 0; c < kPC; ++c) {
      const u32x4 w = *reinterpret_cast<const u32x4 *>(qr + 8 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) qp[g][4 * c + i] = w[i];
    }
  }

  float m[G], l[G], o[G][kPart];   // per wave: running max (base 2, uniform), this lane's sums
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < kPart; ++e) o[g][e] = 0.f;
  }

  for (int u = 0; u < nst; ++u) {
    // stage u has landed in every wave; the slot stage u+3 refills was read
    // in step u-1 by every wave
    const int ahead = min(nst - 1 - u, kSStages - 2);   // stages issued after u
    stream_wait<(kSStages - 2) * kLoadsPerStage>(ahead * kLoadsPerStage);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (u + kSStages - 1 < nst) issue(u + kSStages - 1);

#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
    const int row = kSKeys / kSWaves * wave + kKw * pass + kw;   // this lane's key row of the stage
    const int sw = SG::swz(row);
    const char *kst = k_st[u % kSStages] + row * SG::kRowBytes;
    const char *vst = v_st[u % kSStages] + row * SG::kRowBytes;
    u32x4 kc[kPC], vc[kPC];
#pragma unroll
    for (int c = 0; c < kPC; ++c) {
      kc[c] = *reinterpret_cast<const u32x4 *>(kst + ((kPC * pt + c) ^ sw) * 16);
      vc[c] = *reinterpret_cast<const u32x4 *>(vst + ((kPC * pt + c) ^ sw) * 16);
    }
    const bool valid = kb + static_cast<int64_t>(u) * kSKeys + row < ke;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float acc0 = 0.f, acc1 = 0.f;   // two chains of dot products
#pragma unroll
      for (int c = 0; c < kPC; ++c)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          acc0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kc[c][i]), as_bf16x2(qp[g][4 * c + i]), acc0, false);
          acc1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kc[c][i + 1]), as_bf16x2(qp[g][4 * c + i + 1]), acc1,
                                                 false);
        }
      const float acc = parts_sum<L>(acc0 + acc1);
      float s2;
      if constexpr (CAP) {
        const float xs = acc * p.c2;
        const float e = __builtin_amdgcn_exp2f(-2.f * kLog2e * fabsf(xs));
        const float th = (1.f - e) * __builtin_amdgcn_rcpf(1.f + e);
        s2 = copysignf(th, xs) * p.cap_out;
      } else {
        s2 = acc * p.c2;
      }
      s2 = valid ? s2 : -INFINITY;
      // The wave's exponent base m[g] is set by its first step with a valid
      // key and moves only when a score exceeds it by more than 32 (base-2
      // units), so exponentials stay below 2^32 and a step normally needs no
      // cross-lane reduction.  Both tests are wave-uniform (ballots).
      if (__builtin_amdgcn_ballot_w64(s2 > m[g] + kBaseSlack) != 0) {
        float mx = s2;
#pragma unroll
        for (int x = L; x < 64; x <<= 1) mx = fmaxf(mx, __shfl_xor(mx, x, 64));
        mx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mx)));
        const float a = __builtin_amdgcn_exp2f(m[g] - mx);   // 0 while m is -inf
        l[g] *= a;
#pragma unroll
        for (int e = 0; e < kPart; ++e) o[g][e] *= a;
        m[g] = mx;
      }
      const float pe = m[g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s2 - m[g]);
      l[g] += pe;
#pragma unroll
      for (int c = 0; c < kPC; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[g][8 * c + 2 * i] += pe * __uint_as_float(vc[c][i] << 16);
          o[g][8 * c + 2 * i + 1] += pe * __uint_as_float(vc[c][i] & 0xffff0000u);
        }
    }
    }   // pass
  }

  // wave totals through LDS (the stages are free now): lane (kw, pt) stores
  // its partial outputs at [wave][kw][g][part pt], then each output sums
  // the kKw lanes' partials of both waves.
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int x = L; x < 64; x <<= 1) l[g] += __shfl_xor(l[g], x, 64);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // stages free
  static_assert(kSWaves * kKw * G * D * 4 <= kArena, "partial outputs fit the arena");
  float *o_lds = reinterpret_cast<float *>(smem);   // [kSWaves][kKw][G][D]
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < kPart; e += 4)
      *reinterpret_cast<float4 *>(&o_lds[((wave * kKw + kw) * G + g) * D + kPart * pt + e]) =
          make_float4(o[g][e], o[g][e + 1], o[g][e + 2], o[g][e + 3]);
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      mrg_m[wave][g] = m[g];
      mrg_l[wave][g] = l[g];
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
        float ow = 0.f;
#pragma unroll
        for (int j = 0; j < kKw; ++j) ow += o_lds[((w * kKw + j) * G + g) * D + d];
        x += a * ow;
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
    for (int c = 0; c < p.n_chunks; ++c) {
      const int64_t slot = (unit * p.n_chunks + c) * G + g;
      const float mc = p.ws_m[slot];
      if (mc == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f(mc - m);
      l += w * p.ws_l[slot];
#pragma unroll
      for (int j = 0; j < kCols; ++j) o[j] += w * p.ws_o[slot * D + kCols * lane + j];
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  __bf16 *orow = static_cast<__bf16 *>(p.out) + static_cast<int64_t>(bhq) * D;
#pragma unroll
  for (int j = 0; j < kCols; ++j) orow[kCols * lane + j] = static_cast<__bf16>(o[j] * inv);
  if (p.lse && lane == 0) p.lse[bhq] = l > 0.f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
}

template <int D, int G>
hipError_t go(const DecodeParams &p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p.B * p.Hkv), static_cast<unsigned>(p.n_chunks));
  if (p.cap) hipLaunchKernelGGL((decode_stream<D, G, true>), grid, dim3(kSThreads), 0, s, p);
  else hipLaunchKernelGGL((decode_stream<D, G, false>), grid, dim3(kSThreads), 0, s, p);
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

}  // namespace splash
