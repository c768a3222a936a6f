// Decode: one new query per (batch, query head) against the whole key/value
// cache (q_len = 1).  The EasyDeL block-sparse module turns the causal mask
// off in decode mode and falls back to plain attention for a single query on
// TPU (EasyDeL BlockSparseAttn.forward_native); this is the MI355X-native
// path for that case.  It is the forward's masked softmax attention with
// every key allowed, split along the keys (flash decoding):
//   1. partials: a workgroup per (batch, kv head, 512-key chunk) computes, for
//      the G query heads of the kv head's GQA group at once, the chunk's
//      scores, its max m_c, sum l_c and unnormalised output o_c;
//   2. merge: a wave per (batch, query head) combines the chunks,
//      m = max m_c, l = sum l_c e^(m_c - m), out = sum o_c e^(m_c - m) / l,
//      lse = m + log l (natural log).
// HBM-bound: every K and V row of the cache is read once per kv head and
// serves the whole GQA group, with 16-byte lane loads, 16 lanes per row.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "splash_kernel.h"

namespace splash {
namespace {

constexpr int kChunk = 512;      // keys per partial workgroup
constexpr int kDThreads = 512;   // 8 waves; 512-key chunks measured 17 % faster than 256-key ones
static_assert(kChunk == kDThreads, "the softmax phase gives each thread one key");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void unpack8(const u32x4 w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Partials.  Threads: kPerRow = D / 8 lanes per key row (8 elements each), so
// a wave covers kRowsPerWave = 64 / kPerRow keys per pass.
template <int D, int G, bool CAP>
__global__ __launch_bounds__(kDThreads) void decode_partial(const DecodeParams p) {
  constexpr int kPerRow = D / 8;
  constexpr int kRowsPerWave = 64 / kPerRow;
  constexpr int kWaves = kDThreads / 64;
  __shared__ float s_lds[G][kChunk];        // scores (base-2 units), then exponentials
  __shared__ float red[kWaves][G];
  __shared__ float o_lds[kWaves][G][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / kPerRow;           // key row within the wave's pass
  const int part = lane % kPerRow;          // 8-element slice of the row
  const int unit = blockIdx.x;              // (b, hkv)
  const int chunk = blockIdx.y;
  const int b = unit / p.Hkv, hkv = unit % p.Hkv;
  const int64_t key_begin = static_cast<int64_t>(chunk) * kChunk;
  const int n_keys = static_cast<int>(min(static_cast<int64_t>(kChunk), p.Skv - key_begin));

  // this lane's slice of the G query rows
  float qv[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int hq = hkv * G + g;
    const __bf16 *qr = static_cast<const __bf16 *>(p.q) + (static_cast<int64_t>(b) * p.Hq + hq) * D + 8 * part;
    unpack8(*reinterpret_cast<const u32x4 *>(qr), qv[g]);
  }
  const int64_t kv_head = (static_cast<int64_t>(b) * p.Hkv + hkv) * p.Skv;
  const __bf16 *kbase = static_cast<const __bf16 *>(p.k) + (kv_head + key_begin) * D + 8 * part;
  const __bf16 *vbase = static_cast<const __bf16 *>(p.v) + (kv_head + key_begin) * D + 8 * part;

  // All of this lane's K rows are requested up front; its V rows once the
  // scores are formed, so their latency overlaps the softmax phase (loading
  // both at once costs occupancy and measured slower).
  constexpr int kIters = kChunk / (kWaves * kRowsPerWave);
  u32x4 kr[kIters], vr[kIters];
  auto load_v = [&]() {
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int key = wave * kRowsPerWave + it * kWaves * kRowsPerWave + sub;
      vr[it] = key < n_keys ? *reinterpret_cast<const u32x4 *>(vbase + static_cast<int64_t>(key) * D) : u32x4{0u, 0u, 0u, 0u};
    }
  };
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int key = wave * kRowsPerWave + it * kWaves * kRowsPerWave + sub;
    kr[it] = key < n_keys ? *reinterpret_cast<const u32x4 *>(kbase + static_cast<int64_t>(key) * D) : u32x4{0u, 0u, 0u, 0u};
  }

  // 1. scores
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int key = wave * kRowsPerWave + it * kWaves * kRowsPerWave + sub;
    float kx[8];
    unpack8(kr[it], kx);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += qv[g][i] * kx[i];
#pragma unroll
      for (int m = kPerRow / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
      if (part == 0) {
        float s2;
        if constexpr (CAP) {
          const float xs = acc * p.c2;
          const float e = __builtin_amdgcn_exp2f(-2.f * kLog2e * fabsf(xs));
          const float th = (1.f - e) * __builtin_amdgcn_rcpf(1.f + e);
          s2 = copysignf(th, xs) * p.cap_out;
        } else {
          s2 = acc * p.c2;
        }
        s_lds[g][key] = key < n_keys ? s2 : -INFINITY;
      }
    }
  }
  load_v();
  __syncthreads();

  // 2. per head: chunk max, exponentials, sum (thread t owns key t)
  float mx[G], sm[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float x = s_lds[g][tid];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
    if (lane == 0) red[wave][g] = x;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = red[0][g];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red[w][g]);
    mx[g] = m;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float e = mx[g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_lds[g][tid] - mx[g]);
    s_lds[g][tid] = e;
    float x = e;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    if (lane == 0) red[wave][g] = x;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) l += red[w][g];
    sm[g] = l;
  }

  // 3. unnormalised output: this lane's 8 columns, summed over its keys
  float acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int key = wave * kRowsPerWave + it * kWaves * kRowsPerWave + sub;
    float vx[8];
    unpack8(vr[it], vx);   // zeros past the chunk's end, whose exponentials are 0 too
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pe = s_lds[g][key];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[g][i] += pe * vx[i];
    }
  }
  // sum over the wave's key rows (lanes with the same slice), then over waves
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = acc[g][i];
#pragma unroll
      for (int m = kPerRow; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
      acc[g][i] = x;
    }
  if (sub == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) o_lds[wave][g][8 * part + i] = acc[g][i];
  }
  __syncthreads();
  const int64_t slot = static_cast<int64_t>(unit) * p.n_chunks + chunk;
  for (int idx = tid; idx < G * D; idx += kDThreads) {
    const int g = idx / D, d = idx % D;
    float x = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) x += o_lds[w][g][d];
    p.ws_o[(slot * G + g) * D + d] = x;
  }
  if (tid < G) {
    p.ws_m[slot * G + tid] = mx[tid];
    p.ws_l[slot * G + tid] = sm[tid];
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
  if (p.cap) hipLaunchKernelGGL((decode_partial<D, G, true>), grid, dim3(kDThreads), 0, s, p);
  else hipLaunchKernelGGL((decode_partial<D, G, false>), grid, dim3(kDThreads), 0, s, p);
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

int64_t decode_chunks(int64_t Skv) { return (Skv + kChunk - 1) / kChunk; }

hipError_t launch_decode(const DecodeParams &p, hipStream_t stream) {
  return p.D == 64 ? go_g<64>(p, stream) : go_g<128>(p, stream);
}

}  // namespace splash
