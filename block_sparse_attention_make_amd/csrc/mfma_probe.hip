// Measurement helpers, not part of the attention path.  First, the bf16 MFMA
// throughput this GPU sustains, to put the kernels' MFMA rates against the
// chip's own ceiling (clock under load included) beside the nominal peak.
// Every wave keeps four independent 32x32x16 bf16 accumulator chains busy
// back to back, from register operands only.
#include <hip/hip_runtime.h>

#include <cstdint>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float *sink) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(0.001f * static_cast<float>((threadIdx.x + i) & 7));
    b[i] = static_cast<__bf16>(0.002f * static_cast<float>((threadIdx.x * 3 + i) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The same throughput with operands like an attention step's: eight sets of
// pseudo-random bf16 values in [-2, 2) per lane, cycled so consecutive
// matrix instructions see different data.  The matrix cores draw more power
// on changing data than on the constant operands above, and under the GPU's
// power limit the clock, and so the rate, drops.
__device__ __forceinline__ float probe_value(unsigned x) {   // integer hash -> [-2, 2)
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return (static_cast<float>(x & 0xffffu) / 32768.f - 1.f) * 2.f;
}

__global__ __launch_bounds__(256) void mfma_probe_random_kernel(int iters, float *sink) {
  bf16x8 a[8], b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned s = (blockIdx.x * 256u + threadIdx.x) * 128u + k * 16u + i;
      a[k][i] = static_cast<__bf16>(probe_value(s));
      b[k][i] = static_cast<__bf16>(probe_value(s + 8u));
    }
  f32x16 c[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[k], c[k & 3], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[j][i];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Launches `blocks` workgroups of 4 waves, each wave running `iters` x 4
// MFMAs (32768 flops each) into sink[blocks * 256].
extern "C" __attribute__((visibility("default"))) int splash_probe_mfma(int blocks, int iters, float *sink,
                                                                       void *stream) {
  if (blocks <= 0 || iters <= 0 || !sink) return 1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// Launches `blocks` workgroups of 4 waves, each wave running `iters` x 8
// MFMAs (32768 flops each) on changing random operands into sink[blocks * 256].
extern "C" __attribute__((visibility("default"))) int splash_probe_mfma_random(int blocks, int iters, float *sink,
                                                                              void *stream) {
  if (blocks <= 0 || iters <= 0 || !sink) return 1;
  hipLaunchKernelGGL(mfma_probe_random_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters,
                     sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// The HBM read rate this GPU sustains, for the memory-bound kernels: each
// workgroup streams one contiguous share of n 16-byte words, four
// non-temporal 4 KiB loads (256 lanes x 16 bytes) in flight, XOR-folded into
// sink[blocks * 256] so the loads are not dropped.  (Of the patterns tried --
// grid-stride or per-workgroup chunks, 2 to 8 loads in flight, 8 to 64
// workgroups per CU, with and without the non-temporal hint -- this one at
// 8 workgroups per CU read fastest: about 6.7 TB/s against 5.8 for a
// grid-stride read.)
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4 *__restrict__ src, int64_t n, unsigned *sink) {
  const int64_t per = (n + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t b1 = b0 + per < n ? b0 + per : n;
  int64_t i = b0 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * 256 < b1; i += 4 * 256) {
    const u32x4 x0 = __builtin_nontemporal_load(src + i);
    const u32x4 x1 = __builtin_nontemporal_load(src + i + 256);
    const u32x4 x2 = __builtin_nontemporal_load(src + i + 512);
    const u32x4 x3 = __builtin_nontemporal_load(src + i + 768);
    acc ^= (x0 ^ x1) ^ (x2 ^ x3);
  }
  for (; i < b1; i += 256) acc ^= __builtin_nontemporal_load(src + i);
  sink[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// Reads `bytes` (a multiple of 16) at the 16-byte aligned `src` with `blocks`
// workgroups of 256 lanes into sink[blocks * 256].
extern "C" __attribute__((visibility("default"))) int splash_probe_read(const void *src, int64_t bytes, int blocks,
                                                                       unsigned *sink, void *stream) {
  if (!src || !sink || blocks <= 0 || bytes <= 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15)) return 1;
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4 *>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
