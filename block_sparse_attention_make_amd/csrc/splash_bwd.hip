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

// A 128 x D bf16 tile in LDS; 16-byte chunk c of row r sits at chunk
// c ^ swz(r).  Each tile is read both ways, so the swizzle serves both:
//  * row reads (ds_read_b128, 16 lanes on 16 consecutive rows, one logical
//    chunk): swz is a bijection on the row bits that share a bank line
//    (r mod 16 for D = 128, r / 2 mod 8 for D = 64), so the 16 lanes land
//    on 16 different chunk slots;
//  * transposing reads (ds_read_b64_tr_b16, 32 lanes on 4 consecutive rows
//    x 4 consecutive chunks): rows 4k .. 4k + 3 get different high chunk
//    bits (the bits above the 4 chunks' span), so the 16 chunks the 32
//    lanes touch are all different as well.
// The plain row & 15 kept the 4 rows' chunks inside one 4-chunk span: 4-way
// conflicts on every transposing read.
template <int D>
struct BTile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kBytes = kBlk * kRowBytes;
  __device__ static int swz(int row) {
    if constexpr (kChunks >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
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
  const bf16x8 r = join_tr_halves(lo4, hi4);
  return r;
}

// read_tr with the lane's addresses precomputed: for tile rows r0 + 16 h + t
// (r0 a multiple of 16) the swizzle depends only on t, so each lane's byte
// offsets for its two rows t and t + 8 and each column group dt are fixed,
// and only the uniform row base changes from read to read.
template <int D>
struct TrRead {
  using T = BTile<D>;
  int off_lo[D / 32], off_hi[D / 32];
  __device__ TrRead(int lane, int half) {
    const int trow = 4 * half + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int col = 32 * dt + tcol;
      const int c = col >> 3, within = (col & 7) * 2;
      off_lo[dt] = trow * T::kRowBytes + ((c ^ T::swz(trow)) * 16) + within;
      off_hi[dt] = (trow + 8) * T::kRowBytes + ((c ^ T::swz(trow + 8)) * 16) + within;
    }
  }
  __device__ __forceinline__ bf16x8 operator()(const char *lds, int r0, int h, int dt) const {
    const char *base = lds + (r0 + 16 * h) * T::kRowBytes;
    const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3))) *)(base + off_lo[dt]));
    const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3))) *)(base + off_hi[dt]));
    const bf16x8 r = join_tr_halves(lo4, hi4);
    return r;
  }
};

// A 32x32x16 bf16 MFMA from inline assembly, so its accumulator lives in
// VGPRs where the VALU reads it (left to itself the compiler keeps the
// score accumulators in AGPRs and copies every element out).  The compiler
// does not see this instruction's latency: a VALU read of the accumulator
// must wait for mfma_drain.  A first k-step (C = 0) must not share registers
// with its inputs.
__device__ __forceinline__ void mfma_v(f32x16 &acc, const bf16x8 &a, const bf16x8 &b, bool first) {
  if (first)
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  else
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// Wait states covering the result latency of the last mfma_v writing acc
// before a VALU instruction reads it (16 passes, generously).  Tied to the
// accumulators so it stays between their last MFMA and their first read.
__device__ __forceinline__ void mfma_drain(f32x16 &a, f32x16 &b) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(a), "+v"(b));
}

// B operands of a row block kept in registers: lane (j, half) holds row
// row0 + j, elements 16 ks + 8 half .. + 7.  PAD: the rows hold `mdim`
// elements in memory (a multiple of 16, at most D); the rest read as zeros.
template <int D, bool PAD = false>
__device__ __forceinline__ void load_rows_b(bf16x8 (&dst)[D / 16], const __bf16 *g, int lane, int half,
                                            int mdim = D) {
  const int stride = PAD ? mdim : D;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    if (!PAD || 16 * ks + 8 * half < mdim)
      dst[ks] = *reinterpret_cast<const bf16x8 *>(g + static_cast<int64_t>(lane & 31) * stride + 16 * ks + 8 * half);
    else
      dst[ks] = bf16x8{};
  }
}

// Soft-cap pieces of one score: base-2 capped logit and the derivative
// factor 1 - tanh^2.
// With y = x c2 and kc2 = 2 c2 log2 e: tanh y = 1 - 2 / (1 + e^{2y}), which
// reaches +-1 exactly at the float range's ends.
__device__ __forceinline__ void capped(float x, float kc2, float cap_out, float &s2, float &g) {
  const float t = __builtin_amdgcn_exp2f(x * kc2);
  const float th = __builtin_fmaf(-2.f, __builtin_amdgcn_rcpf(1.f + t), 1.f);
  s2 = th * cap_out;
  g = __builtin_fmaf(-th, th, 1.f);
}

// Store a transposed fp32 accumulator (rows d, columns = the wave's 32 rows)
// as rows of a [*, D] bf16 array, times `mul`, through LDS: the accumulator
// layout gives a lane 4-element pieces
// of its row 8 columns apart, so direct stores scatter 32 rows over one
// instruction.  The wave writes its 32 rows (bf16) into `lds` (32 x D, its
// own region; 16-byte chunks swizzled by row) and stores them back 16 bytes
// per lane, whole rows per instruction (non-temporal: the kernel does not
// read them again).  The wave's LDS writes and reads complete in order.
// PAD: the array's rows hold `mdim` elements (a multiple of 16, at most D);
// the padding columns are not stored.
template <int D, bool PAD = false>
__device__ __forceinline__ void store_t_rows(char *lds, __bf16 *g, const f32x16 (&acc)[D / 32], float mul, int lane,
                                             int half, int mdim = D) {
  constexpr int kRB = D * 2, kChunks = kRB / 16;
  const int rr = lane & 31;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      union { __bf16 h[4]; u32x2 u; } pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk.h[e] = static_cast<__bf16>(acc[dt][4 * q4 + e] * mul);
      *reinterpret_cast<u32x2 *>(lds + rr * kRB + (((4 * dt + q4) ^ (rr & (kChunks - 1))) * 16) + 8 * half) = pk.u;
    }
  constexpr int kRowsPer = 1024 / kRB;
#pragma unroll
  for (int i = 0; i < 32 / kRowsPer; ++i) {
    const int r2 = kRowsPer * i + lane / kChunks, c = lane % kChunks;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(lds + r2 * kRB + ((c ^ (r2 & (kChunks - 1))) * 16));
    if (!PAD || c * 8 < mdim)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(g) +
                                                                r2 * (PAD ? mdim * 2 : kRB) + c * 16));
  }
}

// ---- delta: di = <dout_i, out_i> ------------------------------------------
// Rows of dv elements (a multiple of 8, at most D); D / 8 threads per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta(const __bf16 *o, const __bf16 *dout, float *delta, int64_t rows,
                                                 int dv) {
  constexpr int kPerRow = D / 8;   // threads per row, 8 elements each
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = t / kPerRow;
  const int c = static_cast<int>(t % kPerRow);
  float acc = 0.f;
  if (row < rows && c * 8 < dv) {
    const int64_t at = row * dv + c * 8;
    const u32x4 a = *reinterpret_cast<const u32x4 *>(o + at);
    const u32x4 b = *reinterpret_cast<const u32x4 *>(dout + at);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += __uint_as_float(a[i] << 16) * __uint_as_float(b[i] << 16);
      acc += __uint_as_float(a[i] & 0xffff0000u) * __uint_as_float(b[i] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int m = kPerRow / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && c == 0) delta[row] = acc;
}

// ---- staging ----------------------------------------------------------------
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes at `base`; uniform, kept in SGPRs.
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

// Offset within its 1 KiB segment of the 16 bytes lane `lane` moves for
// segment `seg` of a tile: the lane that lands on chunk pc of a row fetches
// the row's logical chunk pc ^ swz(row), so the tile comes out swizzled.
template <int D>
__device__ __forceinline__ uint32_t seg_voff(int seg, int lane) {
  using T = BTile<D>;
  constexpr int kRowsPerSeg = 1024 / T::kRowBytes;
  const int rin = lane / T::kChunks;
  const int row = seg * kRowsPerSeg + rin;
  const int c = (lane % T::kChunks) ^ T::swz(row);
  return static_cast<uint32_t>(rin * T::kRowBytes + c * 16);
}

// Direct-to-LDS loads (buffer_load_dwordx4 ... lds) of this wave's quarter of
// a 128-row tile starting at byte `goff` of the resource: segments
// 4 g + 0..3 of the wave's share, one M0 per group of four (the instruction
// offset advances both the LDS and the global address).  Issued from inline
// assembly, awaited with an explicit vmcnt wait before the barrier that
// publishes the buffer.
//
// PAD: the array's rows hold `mrow` bytes in memory (a multiple of 32, at
// most the tile's row), and the tile starts at array row `row0` (goff is
// unused).  Each segment then takes its own M0 and per-lane offsets (the
// packed row stride no longer matches the tile's, so one instruction offset
// cannot step both addresses), and a lane whose chunk lies in the padding
// gets an offset past the resource's end, which reads zeros; the tiles'
// padding columns are zeroed before their first load and stay zero.
template <int D, int ROWS = kBlk, bool PAD = false>
__device__ __forceinline__ void issue_tile(char *lds, i32x4 res, uint32_t goff, int wave, int lane,
                                           uint32_t row0 = 0, uint32_t mrow = 0) {
  using T = BTile<D>;
  constexpr int kSegs = ROWS * T::kRowBytes / 1024 / 4;   // per wave
  static_assert(kSegs % 4 == 0, "whole groups of four segments per wave");
  if constexpr (PAD) {
    constexpr int kRowsPerSeg = 1024 / T::kRowBytes;
#pragma unroll
    for (int i = 0; i < kSegs; ++i) {
      const int seg = wave * kSegs + i;
      const int row = seg * kRowsPerSeg + lane / T::kChunks;
      const int c = (lane % T::kChunks) ^ T::swz(row);
      const uint32_t voff = static_cast<uint32_t>(c * 16) < mrow
          ? (row0 + static_cast<uint32_t>(row)) * mrow + static_cast<uint32_t>(c * 16)
          : 0x80000000u;
      const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
          (__attribute__((address_space(3))) char *)(lds + seg * 1024)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   :: "s"(m0), "v"(voff), "s"(res) : "memory", "m0");
#pragma clang diagnostic pop
    }
    return;
  }
#pragma unroll
  for (int g = 0; g < kSegs / 4; ++g) {
    const int seg0 = wave * kSegs + 4 * g;
    const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) char *)(lds + seg0 * 1024)));
    const uint32_t soff = goff + static_cast<uint32_t>(seg0 * 1024);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %5, %6 offen lds\n\t"
        "buffer_load_dwordx4 %2, %5, %6 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %3, %5, %6 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %4, %5, %6 offen offset:3072 lds"
        :: "s"(m0), "v"(seg_voff<D>(seg0, lane)), "v"(seg_voff<D>(seg0 + 1, lane)),
           "v"(seg_voff<D>(seg0 + 2, lane)), "v"(seg_voff<D>(seg0 + 3, lane)), "s"(res), "s"(soff)
        : "memory", "m0");
#pragma clang diagnostic pop
  }
}

__device__ __forceinline__ void wait_all_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Computable masks: the key interval [lo, hi] of query position qpos in the
// MaskInfo's key coordinates.
__device__ __forceinline__ void key_interval(const FwdParams &f, int64_t qpos, int64_t &lo, int64_t &hi) {
  const int64_t big = int64_t(1) << 40;
  if (f.mask_kind == 0) { lo = -big; hi = qpos; }
  else if (f.mask_kind == 1) { lo = f.left < 0 ? -big : qpos - f.left; hi = f.right < 0 ? big : qpos + f.right; }
  else { lo = (qpos / f.chunk) * f.chunk; hi = qpos; }
  lo -= f.kv_offset;
  hi -= f.kv_offset;
}

// Workgroup id -> (batch-head unit, rank): consecutive ids go round-robin
// over the 8 XCDs, and XCD x gets a contiguous range of units so a unit's
// shared operands stay in one L2; ranks (longest work first) vary fastest.
__device__ __forceinline__ void xcd_map(int pid, int units, int &unit, int &rank) {
  if ((units & 7) == 0) {
    const int per = units >> 3, x = pid & 7, j = pid >> 3;
    unit = x * per + j % per;
    rank = j / per;
  } else {
    unit = pid % units;
    rank = pid / units;
  }
}

// ---- key-major kernel: dK, dV ---------------------------------------------
// Workgroup (b, hkv, key block c); wave w owns keys 32 w .. 32 w + 31.  The
// query blocks to visit -- every (query head g of the group, entry e of the
// transposed list of mask head hm(g)) -- stream through two LDS buffers: the
// next block's Q and dO tiles load while the current one is computed.
// PAD: head dims other than the kernel's D (q, k, dq, dk rows of f.dk
// elements, v, dout, dv rows of f.dv), run zero-padded to D columns: the
// padding of every operand is zero, so every product sums only real
// columns, and the padding columns of dK and dV are not stored.
template <int D, bool CAP, bool DENSE, bool PAD>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv(const BwdParams p) {
  using T = BTile<D>;
  constexpr int kKS = D / 16, kDT = D / 32;
  // [buffer][Q, dO]: a buffer's two tiles sit within one LDS instruction
  // offset of each other, so their reads share address registers
  __shared__ __attribute__((aligned(1024))) char qdo_t[2][2][T::kBytes];
  __shared__ __attribute__((aligned(16))) float lse_s[2][kBlk], di_s[2][kBlk];
  // computable masks: each row's allowed keys in this key block as a first key
  // and a count (0 for none); dense masks: the packed words (all ones for
  // full blocks)
  __shared__ __attribute__((aligned(16))) int lo_s[2][kBlk], hi_s[2][kBlk];
  __shared__ __attribute__((aligned(16))) unsigned mw_s[2][4 * kBlk];

  const FwdParams &f = p.f;
  const float kc2 = 2.f * kLog2e * f.c2;   // soft cap: x -> 2 y log2 e
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bh, rank;
  xcd_map(blockIdx.x, static_cast<int>(f.B * f.Hkv), bh, rank);
  const int c = p.col_order[rank];
  const int b = bh / static_cast<int>(f.Hkv), hkv = bh % static_cast<int>(f.Hkv);
  const int64_t key0 = static_cast<int64_t>(c) * kBlk + 32 * wave;   // the wave's first key
  const int mk = PAD ? f.dk : D, mv = PAD ? f.dv : D;   // row lengths in memory
  const int64_t kv_row = (static_cast<int64_t>(b) * f.Hkv + hkv) * f.Skv + key0;

  bf16x8 kb[kKS], vb[kKS];
  load_rows_b<D, PAD>(kb, static_cast<const __bf16 *>(f.k) + kv_row * mk, lane, half, mk);
  load_rows_b<D, PAD>(vb, static_cast<const __bf16 *>(f.v) + kv_row * mv, lane, half, mv);
  if constexpr (PAD) {
    // the tiles' padding columns start (and stay) zero; written and
    // published before any load into the tiles
    constexpr int kVec = 2 * 2 * T::kBytes / 16;
#pragma unroll
    for (int i = 0; i < kVec / kThreads; ++i)
      reinterpret_cast<u32x4 *>(&qdo_t[0][0][0])[tid + kThreads * i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  }
  f32x16 dk[kDT], dv[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) dk[dt][v] = dv[dt][v] = 0.f;

  // Walk of the (g, e) pairs.
  auto list_of = [&](int g) -> int64_t {
    const int hq = hkv * f.group + g;
    return static_cast<int64_t>(f.hm == 1 ? 0 : hq) * p.nk + c;
  };
  auto count_of = [&](int g) -> int { return __builtin_amdgcn_readfirstlane(p.col_n[list_of(g)]); };
  auto advance = [&](int &g, int &e, int &n) {
    ++e;
    while (e >= n && g < f.group) {
      ++g;
      e = 0;
      n = g < f.group ? count_of(g) : 0;
    }
  };
  int g = 0, e = -1, n = count_of(0);
  advance(g, e, n);   // first pair (g == group when there is none)

  const int key_local = 32 * wave + (lane & 31);
  const TrRead<D> tr(lane, half);
  // Small per-block operands of pair (g, e), loaded to registers by the
  // first 128 threads: lse (base 2), di, and the key interval or mask words.
  struct Small { float l, d; int lo, hi; unsigned m0, m1; };
  auto load_small = [&](int gg, int ee, int label, Small &sm) {
    const int hq = hkv * f.group + gg;
    const int ent = p.col_ent[list_of(gg) * p.col_w + ee];
    const int r = ent & 0x3fffffff;
    const int64_t row_base = (static_cast<int64_t>(b) * f.Hq + hq) * f.Sq + static_cast<int64_t>(r) * kBlk;
    if (tid < kBlk) {
      sm.l = f.lse[row_base + tid] * kLog2e;
      sm.d = p.delta[row_base + tid];
      if constexpr (!DENSE) {
        int64_t lo, hi;
        key_interval(f, f.q_seq[static_cast<int64_t>(r) * kBlk + tid], lo, hi);
        const int64_t kb0 = static_cast<int64_t>(c) * kBlk;   // relative to this key block
        lo -= kb0;
        hi -= kb0;
        sm.lo = static_cast<int>(lo < -1 ? -1 : (lo > kBlk ? kBlk : lo));
        const int hc = static_cast<int>(hi < -1 ? -1 : (hi > kBlk ? kBlk : hi));
        sm.hi = hc >= sm.lo ? hc - sm.lo + 1 : 0;   // count of allowed keys from lo
      }
    }
    if constexpr (DENSE) {
      if (label == 1) {
        const int mn = p.col_mn[list_of(gg) * p.col_w + ee];
        const unsigned *src = f.pmb_bits + static_cast<int64_t>(mn) * 4 * kBlk;
        sm.m0 = src[tid];
        sm.m1 = src[tid + kThreads];
      }
    }
  };
  auto store_small = [&](int buf, int label, const Small &sm) {
    if (tid < kBlk) {
      lse_s[buf][tid] = sm.l;
      di_s[buf][tid] = sm.d;
      if constexpr (!DENSE) {
        lo_s[buf][tid] = sm.lo;
        hi_s[buf][tid] = sm.hi;
      }
    }
    if constexpr (DENSE) {
      mw_s[buf][tid] = label == 1 ? sm.m0 : ~0u;   // full blocks: every key allowed
      mw_s[buf][tid + kThreads] = label == 1 ? sm.m1 : ~0u;
    }
  };
  auto entry = [&](int gg, int ee, int &r, int &label) {
    const int ent = __builtin_amdgcn_readfirstlane(p.col_ent[list_of(gg) * p.col_w + ee]);
    r = ent & 0x3fffffff;
    label = static_cast<int>(static_cast<unsigned>(ent) >> 30);
  };
  auto issue = [&](int buf, int gg, int r) {
    const int hq = hkv * f.group + gg;
    const int64_t head = (static_cast<int64_t>(b) * f.Hq + hq) * f.Sq;   // the head's first row
    const i32x4 qr = make_rsrc(static_cast<const __bf16 *>(f.q) + head * mk, f.Sq * mk * 2);
    const i32x4 dr = make_rsrc(static_cast<const __bf16 *>(p.dout) + head * mv, f.Sq * mv * 2);
    if constexpr (PAD) {
      const uint32_t row0 = static_cast<uint32_t>(r) * kBlk;
      issue_tile<D, kBlk, true>(qdo_t[buf][0], qr, 0, wave, lane, row0, static_cast<uint32_t>(mk * 2));
      issue_tile<D, kBlk, true>(qdo_t[buf][1], dr, 0, wave, lane, row0, static_cast<uint32_t>(mv * 2));
    } else {
      const uint32_t goff = static_cast<uint32_t>(static_cast<int64_t>(r) * T::kBytes);
      issue_tile<D>(qdo_t[buf][0], qr, goff, wave, lane);
      issue_tile<D>(qdo_t[buf][1], dr, goff, wave, lane);
    }
  };

  // The walk runs one pair ahead of the tiles: the list entry of the pair
  // after the next is loaded while the current tile is computed (and
  // awaited with the tile loads), so naming the next tile's query block
  // never waits on a dependent load.  The raw entry travels in a VGPR until
  // then.
  int buf = 0;
  int g2 = g, e2 = e, n2 = n;   // the pair after the current one
  if (g < f.group) advance(g2, e2, n2);
  int ent_next = 0;             // its list entry, once loaded
  if (g < f.group) {
    int r, label;
    entry(g, e, r, label);
    Small sm{};
    load_small(g, e, label, sm);
    store_small(0, label, sm);   // waits for the small loads, issued before any tile load
    issue(0, g, r);
    if (g2 < f.group) ent_next = p.col_ent[list_of(g2) * p.col_w + e2];
  }
  wait_all_loads();
  __syncthreads();

  while (g < f.group) {
    const bool more = g2 < f.group;
    int r2 = 0, label2 = 0;
    if (more) {
      const int ent = __builtin_amdgcn_readfirstlane(ent_next);
      r2 = ent & 0x3fffffff;
      label2 = static_cast<int>(static_cast<unsigned>(ent) >> 30);
    }
    // the pair after that; its count is loaded only where the walk changes
    // query head, before any load of this iteration is in flight
    int g3 = g2, e3 = e2, n3 = n2;
    if (more) advance(g3, e3, n3);
    Small sm{};
    if (more) {
      load_small(g2, e2, label2, sm);   // before the tile loads: their wait does not wait on those
      issue(buf ^ 1, g2, r2);
    }
    if (g3 < f.group) ent_next = p.col_ent[list_of(g3) * p.col_w + e3];

    // The tile's four 32-row query blocks run as a software pipeline: step
    // qb forms S and dP of block qb + 1 (A), the softmax gradient of block qb
    // (B) and the dV / dK products of block qb - 1 (C).  A and C are
    // independent matrix work and B is VALU work on results of the step
    // before, so each step interleaves them one matrix instruction at a time
    // (sub-slices separated by scheduling barriers): the wave issues in
    // order, and phases run one after another would leave the matrix unit
    // idle during the softmax gradient.
    {
      constexpr int kA = 2 * kKS;      // A instructions of a block: (k-step, S | dP)
      constexpr int kC = 4 * kDT;      // C instructions: (h2, dt, dV | dK)
      constexpr int kSub = kA > kC ? 2 * kA : 2 * kC;
      const char *tq = qdo_t[buf][0];
      const char *td = qdo_t[buf][1];
      f32x16 sA[2], dpA[2];            // [block & 1]
      bf16x8 pbB[2][2], sbB[2][2];     // [block & 1][h2]
      auto a_read = [&](int qb, int a) -> bf16x8 {
        return read_row<D>((a & 1) ? td : tq, 32 * qb + (lane & 31), a >> 1, half);
      };
      auto a_mfma = [&](int qb, int a, const bf16x8 &op) {
        const int ks = a >> 1;
        if ((a & 1) == 0) mfma_v(sA[qb & 1], op, kb[ks], ks == 0);
        else mfma_v(dpA[qb & 1], op, vb[ks], ks == 0);
      };
      auto c_read = [&](int qb, int c) -> bf16x8 {
        const int h2 = c / (2 * kDT), dt = (c >> 1) % kDT;
        return tr((c & 1) ? tq : td, 32 * qb, h2, dt);   // dV contracts dO, dK contracts Q
      };
      auto c_mfma = [&](int qb, int c, const bf16x8 &op) {
        const int h2 = c / (2 * kDT), dt = (c >> 1) % kDT;
        if ((c & 1) == 0) dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, pbB[qb & 1][h2], dv[dt], 0, 0, 0);
        else dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, sbB[qb & 1][h2], dk[dt], 0, 0, 0);
      };
      // Per-row operands of elements 4 g4 .. 4 g4 + 3 (rows qi0 .. qi0 + 3).
      // The mask data is read unconditionally (stale unless label == 1) so
      // the step stays one basic block.
      struct Grp { f32x4 l4, d4; i32x4 lo4, hi4; unsigned mw[4]; };
      auto g_load = [&](int qb, int g4, Grp &G) {
        const int qi0 = 32 * qb + 8 * g4 + 4 * half;
        G.l4 = *reinterpret_cast<const f32x4 *>(&lse_s[buf][qi0]);
        G.d4 = *reinterpret_cast<const f32x4 *>(&di_s[buf][qi0]);
        if constexpr (DENSE) {
#pragma unroll
          for (int k = 0; k < 4; ++k) G.mw[k] = mw_s[buf][wave * kBlk + qi0 + k];
        } else {
          G.lo4 = *reinterpret_cast<const i32x4 *>(&lo_s[buf][qi0]);
          G.hi4 = *reinterpret_cast<const i32x4 *>(&hi_s[buf][qi0]);
        }
      };
      auto elem = [&](int qb, int v, const Grp &G) {
        const int k = v & 3;
        const float sv = sA[qb & 1][v], dpv = dpA[qb & 1][v];
        float s2, gf = 1.f;
        if constexpr (CAP) capped(sv, kc2, f.cap_out, s2, gf);
        else s2 = sv * f.c2;
        // The staged interval or words hold every key of a full block, and a
        // row with no allowed key (lse -inf) has none in any block, so this
        // one test covers labels 1 and 2 and empty rows.
        // select the exponent, not the exponential: a select between an
        // exponential and 0 becomes a branch around every exponential
        float x;
        if constexpr (DENSE) {   // the key's bit sign-extended selects, bit by bit
          const int m = __builtin_amdgcn_sbfe(static_cast<int>(G.mw[k]), lane & 31, 1);
          x = __int_as_float((m & __float_as_int(s2 - G.l4[k])) | (~m & static_cast<int>(0xff800000u)));
        } else {
          const bool in = static_cast<unsigned>(key_local - G.lo4[k]) < static_cast<unsigned>(G.hi4[k]);
          x = in ? s2 - G.l4[k] : -INFINITY;
        }
        const float pv = __builtin_amdgcn_exp2f(x);
        const float dsv = pv * (dpv - G.d4[k]) * gf;
        pbB[qb & 1][v / 8][v % 8] = static_cast<__bf16>(pv);
        sbB[qb & 1][v / 8][v % 8] = static_cast<__bf16>(dsv);
      };

      // One pipeline step: A(qa) (qa < 0: none), B(qbv) (qbv < 0: none),
      // C(qc) (qc < 0: none).  Sub-slice j holds A instruction j / 2 (even
      // j) or C instruction j / 2 (odd j), the operand reads of sub-slice
      // j + 2, and one element of B every kSub / 16 sub-slices.
      auto step = [&](int qa, int qbv, int qc) {
        bf16x8 opA[kA], opC[kC];
        auto reads = [&](int j) {
          if (j >= kSub) return;
          if ((j & 1) == 0) { if (qa >= 0 && (j >> 1) < kA) opA[j >> 1] = a_read(qa, j >> 1); }
          else { if (qc >= 0 && (j >> 1) < kC) opC[j >> 1] = c_read(qc, j >> 1); }
        };
        Grp G[2];
        if (qbv >= 0) g_load(qbv, 0, G[0]);
        reads(0);
        reads(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kSub; ++j) {
          if ((j & 1) == 0) { if (qa >= 0 && (j >> 1) < kA) a_mfma(qa, j >> 1, opA[j >> 1]); }
          else { if (qc >= 0 && (j >> 1) < kC) c_mfma(qc, j >> 1, opC[j >> 1]); }
          __builtin_amdgcn_sched_barrier(0);
          reads(j + 2);
          if (qbv >= 0 && j % (kSub / 16) == 0) {
            const int v = j / (kSub / 16);
            if ((v & 3) == 0 && v + 4 < 16) g_load(qbv, (v >> 2) + 1, G[((v >> 2) + 1) & 1]);
            elem(qbv, v, G[(v >> 2) & 1]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };

      // prologue: A(0), then the result latency of its last instruction
#pragma unroll
      for (int a = 0; a < kA; ++a) a_mfma(0, a, a_read(0, a));
      mfma_drain(sA[0], dpA[0]);
      step(1, 0, -1);
      step(2, 1, 0);
      step(3, 2, 1);
      step(-1, 3, 2);
      step(-1, -1, 3);
    }

    if (more) store_small(buf ^ 1, label2, sm);
    wait_all_loads();
    __syncthreads();   // the next buffer is complete; this one is free for the pair after
    buf ^= 1;
    g = g2;
    e = e2;
    n = n2;
    g2 = g3;
    e2 = e3;
    n2 = n3;
  }
  // Every wave is past the loop's last barrier and no load is in flight, so
  // the tiles are free: each wave stages its dk rows and then its dv rows in
  // its own 2 x 32 rows.
  char *st = &qdo_t[0][0][0] + wave * 64 * D * 2;
  wait_all_loads();
  store_t_rows<D, PAD>(st, static_cast<__bf16 *>(p.dk) + kv_row * mk, dk, p.scale, lane, half, mk);
  store_t_rows<D, PAD>(st + 32 * D * 2, static_cast<__bf16 *>(p.dv) + kv_row * mv, dv, 1.f, lane, half, mv);
}

// ---- query-major kernel: dQ -----------------------------------------------
// Workgroup (b, hq, query block r); wave w owns queries 32 w .. 32 w + 31.
// The row's non-empty key blocks stream through two LDS buffers.
// HALF (D = 128): the K and V tiles stream in 64-key halves (two buffers of
// two half tiles, 64 KiB of LDS), so two workgroups share a CU and two
// waves a SIMD: one wave's softmax gradient (VALU) runs beside the other's
// matrix instructions.  With whole 128-key tiles the buffers take 128 KiB,
// one workgroup per CU, and each wave's MFMAs stand still during its own
// VALU work; that shape stays for grids of at most one workgroup per CU,
// where half tiles only add barriers.  D = 64 takes whole tiles (64 KiB).
// PAD: padded head dims, as in bwd_dkdv.
template <int D, bool CAP, bool DENSE, bool HALF, bool PAD>
__global__ __launch_bounds__(kThreads, HALF ? 2 : 1) void bwd_dq(const BwdParams p) {
  static_assert(!HALF || D == 128, "half tiles at D = 128");
  using T = BTile<D>;
  constexpr int kKS = D / 16, kDT = D / 32;
  constexpr int kTileRows = HALF ? 64 : kBlk;   // keys per buffered tile
  constexpr int kSub = kTileRows / 32;              // 32-key groups per tile
  constexpr int kUnits = kBlk / kTileRows;          // tiles per 128-key block
  constexpr int kTileBytes = kTileRows * T::kRowBytes;
  // [buffer][K, V]
  __shared__ __attribute__((aligned(1024))) char kv_t[2][2][kTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned mw_s[2][4 * kBlk];

  const FwdParams &f = p.f;
  const float kc2 = 2.f * kLog2e * f.c2;   // soft cap: x -> 2 y log2 e
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bh, rank;
  xcd_map(blockIdx.x, static_cast<int>(f.B * f.Hq), bh, rank);
  const int r = f.row_order[rank];
  const int b = bh / static_cast<int>(f.Hq), hq = bh % static_cast<int>(f.Hq);
  const int hkv = hq / f.group;
  const int hm = f.hm == 1 ? 0 : hq;
  const int64_t q_row = static_cast<int64_t>(r) * kBlk + 32 * wave + (lane & 31);   // this lane's query
  const int64_t row_base = (static_cast<int64_t>(b) * f.Hq + hq) * f.Sq;
  const int mk = PAD ? f.dk : D, mv = PAD ? f.dv : D;   // row lengths in memory
  const int64_t q0 = row_base + static_cast<int64_t>(r) * kBlk + 32 * wave;   // the wave's first row

  bf16x8 qb[kKS], dob[kKS];
  load_rows_b<D, PAD>(qb, static_cast<const __bf16 *>(f.q) + q0 * mk, lane, half, mk);
  load_rows_b<D, PAD>(dob, static_cast<const __bf16 *>(p.dout) + q0 * mv, lane, half, mv);
  if constexpr (PAD) {
    // the tiles' padding columns start (and stay) zero; written and
    // published before any load into the tiles
    constexpr int kVec = 2 * 2 * kTileBytes / 16;
#pragma unroll
    for (int i = 0; i < kVec / kThreads; ++i)
      reinterpret_cast<u32x4 *>(&kv_t[0][0][0])[tid + kThreads * i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  }
  const float lse2 = f.lse[row_base + q_row] * kLog2e;
  const float di = p.delta[row_base + q_row];
  int64_t lo = 0, hi = 0;
  if constexpr (!DENSE) key_interval(f, f.q_seq[q_row], lo, hi);
  const TrRead<D> tr(lane, half);
  f32x16 dq[kDT];
#pragma unroll
  for (int dt = 0; dt < kDT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) dq[dt][v] = 0.f;

  const int64_t kv_head = (static_cast<int64_t>(b) * f.Hkv + hkv) * f.Skv;   // the head's first row
  const i32x4 kr = make_rsrc(static_cast<const __bf16 *>(f.k) + kv_head * mk, f.Skv * mk * 2);
  const i32x4 vr = make_rsrc(static_cast<const __bf16 *>(f.v) + kv_head * mv, f.Skv * mv * 2);
  // The row's walk: its non-empty blocks in order, one entry each (key
  // block | label << 28, and the dense mask's partial block), the same
  // lists the forward walks.  They are read-only for the kernel's lifetime,
  // so they go through the constant address space (scalar loads, counted
  // with the LDS operations rather than with the tile loads), and each
  // entry is read one block ahead of its tiles' loads.
  typedef const __attribute__((address_space(4))) int32_t *cptr;
  const cptr items = (cptr)(f.items);
  const cptr walk_kv = (cptr)(f.walk_kv);
  const cptr walk_mn = (cptr)(DENSE ? f.walk_mn : f.walk_kv);
  const int64_t item_at = (static_cast<int64_t>(hm) * f.nq + rank) * 8;
  const int w_off = items[item_at + 1];
  const int w_len = items[item_at + 2];
  auto ent_kv = [](int ent) -> int { return ent & 0x0fffffff; };
  auto ent_lab = [](int ent) -> int { return static_cast<int>(static_cast<uint32_t>(ent) >> 28); };
  // tile `hf` (kTileRows keys) of key block c into buffer buf
  auto issue = [&](int buf, int c, int hf) {
    if constexpr (PAD) {
      const uint32_t row0 = static_cast<uint32_t>(c) * kBlk + static_cast<uint32_t>(hf * kTileRows);
      issue_tile<D, kTileRows, true>(kv_t[buf][0], kr, 0, wave, lane, row0, static_cast<uint32_t>(mk * 2));
      issue_tile<D, kTileRows, true>(kv_t[buf][1], vr, 0, wave, lane, row0, static_cast<uint32_t>(mv * 2));
    } else {
      const uint32_t goff = static_cast<uint32_t>(static_cast<int64_t>(c) * T::kBytes + hf * kTileBytes);
      issue_tile<D, kTileRows>(kv_t[buf][0], kr, goff, wave, lane);
      issue_tile<D, kTileRows>(kv_t[buf][1], vr, goff, wave, lane);
    }
  };
  auto load_words = [&](int mn, unsigned &m0, unsigned &m1) {
    const unsigned *src = f.pmb_bits + static_cast<int64_t>(mn) * 4 * kBlk;
    m0 = src[tid];
    m1 = src[tid + kThreads];
  };

  // The walk: tiles (j, hf) of the row's entries in order; the mask words of
  // a block live in mw_s[mb] for all of its tiles.  ent / mn: entry j;
  // ent_n / mn_n: entry j + 1 (loaded a block ahead).
  int j = 0, hf = 0;
  int buf = 0, mb = 0;
  int ent = 0, mn = 0, ent_n = 0, mn_n = 0;
  if (w_len > 0) {
    ent = walk_kv[w_off];
    if constexpr (DENSE) mn = walk_mn[w_off];
    if (w_len > 1) {
      ent_n = walk_kv[w_off + 1];
      if constexpr (DENSE) mn_n = walk_mn[w_off + 1];
    }
    if constexpr (DENSE) {
      if (ent_lab(ent) == 1) {
        unsigned m0, m1;
        load_words(mn, m0, m1);
        mw_s[0][tid] = m0;
        mw_s[0][tid + kThreads] = m1;
      }
    }
    issue(0, ent_kv(ent), 0);
  }
  wait_all_loads();
  __syncthreads();

  while (j < w_len) {
    const int label = ent_lab(ent);
    const int64_t kbase = static_cast<int64_t>(ent_kv(ent)) * kBlk;
    // this lane's key interval relative to the block, clamped to [-1, kBlk]
    const int rlo = static_cast<int>(lo - kbase < -1 ? -1 : (lo - kbase > kBlk ? kBlk : lo - kbase));
    const int rhi = static_cast<int>(hi - kbase < -1 ? -1 : (hi - kbase > kBlk ? kBlk : hi - kbase));
    // the next tile: the block's next half, or the first tile of the next block
    const bool next_block = hf + 1 == kUnits;
    const int j2 = next_block ? j + 1 : j;
    const int hf2 = next_block ? 0 : hf + 1;
    const bool more = j2 < w_len;
    const int ent2 = next_block ? ent_n : ent;
    const int mn2 = next_block ? mn_n : mn;
    const int label2 = more && next_block ? ent_lab(ent2) : 0;
    unsigned m0 = 0u, m1 = 0u;
    if (more) {
      if constexpr (DENSE) {
        if (next_block && label2 == 1) load_words(mn2, m0, m1);   // before the tile loads
      }
      issue(buf ^ 1, ent_kv(ent2), hf2);
    }
    // entering a new block next: read the entry after it now
    int ent_n2 = ent_n, mn_n2 = mn_n;
    if (next_block && j2 + 1 < w_len) {
      ent_n2 = walk_kv[w_off + j2 + 1];
      if constexpr (DENSE) mn_n2 = walk_mn[w_off + j2 + 1];
    }

#pragma unroll 1
    for (int kb = 0; kb < kSub; ++kb) {
      const int kg = hf * kSub + kb;   // the 32-key group of the block
      f32x16 s, dp;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        const bf16x8 ak = read_row<D>(kv_t[buf][0], 32 * kb + (lane & 31), ks, half);
        const bf16x8 av = read_row<D>(kv_t[buf][1], 32 * kb + (lane & 31), ks, half);
        mfma_v(s, ak, qb[ks], ks == 0);
        mfma_v(dp, av, dob[ks], ks == 0);
      }
      mfma_drain(s, dp);
      // This lane's row's allowed keys among the 32 keys of group kg as a
      // word (bit c <=> key 32 kg + 4 half + c of the layout below), all ones
      // in a full block.  A row with no allowed key has an empty word in
      // every block it meets (label 2 blocks have none), so no lse test is
      // needed.
      unsigned word = ~0u;
      if (label == 1) {
        if constexpr (DENSE) {
          word = mw_s[mb][kg * kBlk + 32 * wave + (lane & 31)] >> (4 * half);
        } else {
          const int k0 = 32 * kg + 4 * half;
          const int b0 = min(max(rlo - k0, 0), 32);
          const int b1 = min(max(rhi - k0 + 1, 0), 32);
          word = b1 > b0 ? static_cast<unsigned>((uint64_t(1) << b1) - (uint64_t(1) << b0)) : 0u;
        }
      }
      bf16x8 sb[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int c = 8 * (v / 4) + (v % 4);   // key 32 kg + 4 half + c of the block
        float s2, gf = 1.f;
        if constexpr (CAP) capped(s[v], kc2, f.cap_out, s2, gf);
        else s2 = s[v] * f.c2;
        // bit c sign-extended selects the exponent or -inf, bit by bit
        const int m = __builtin_amdgcn_sbfe(static_cast<int>(word), c, 1);
        const float x = __int_as_float((m & __float_as_int(s2 - lse2)) | (~m & static_cast<int>(0xff800000u)));
        const float pv = __builtin_amdgcn_exp2f(x);
        sb[v / 8][v % 8] = static_cast<__bf16>(pv * (dp[v] - di) * gf);
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int dt = 0; dt < kDT; ++dt) {
          const bf16x8 ak = tr(kv_t[buf][0], 32 * kb, h2, dt);
          dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, sb[h2], dq[dt], 0, 0, 0);
        }
    }

    if constexpr (DENSE) {
      if (more && next_block && label2 == 1) {
        mw_s[mb ^ 1][tid] = m0;
        mw_s[mb ^ 1][tid + kThreads] = m1;
      }
    }
    wait_all_loads();
    __syncthreads();
    buf ^= 1;
    if (next_block) mb ^= 1;
    ent = ent2;
    mn = mn2;
    ent_n = ent_n2;
    mn_n = mn_n2;
    j = j2;
    hf = hf2;
  }
  // every wave is past the loop's last barrier
  wait_all_loads();
  store_t_rows<D, PAD>(&kv_t[0][0][0] + wave * 32 * D * 2, static_cast<__bf16 *>(p.dq) + q0 * mk, dq, p.scale, lane,
                       half, mk);
}

// Compute units of the current device (looked up once per device; 256 if
// the query fails).
int compute_units() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 256;
    __atomic_store_n(&cached[dev], v, __ATOMIC_RELAXED);
  }
  return v;
}

template <int D, bool CAP, bool DENSE, bool PAD>
hipError_t go(const BwdParams &p, hipStream_t stream) {
  const FwdParams &f = p.f;
  const int64_t nkv = f.B * f.Hkv * p.nk;
  if (nkv > 0)
    hipLaunchKernelGGL((bwd_dkdv<D, CAP, DENSE, PAD>), dim3(static_cast<unsigned>(nkv)), dim3(kThreads), 0, stream,
                       p);
  const int64_t nq = f.B * f.Hq * f.nq;
  if (nq > 0) {
    if (D == 128 && nq > compute_units())
      hipLaunchKernelGGL((bwd_dq<D, CAP, DENSE, D == 128, PAD>), dim3(static_cast<unsigned>(nq)), dim3(kThreads), 0,
                         stream, p);
    else
      hipLaunchKernelGGL((bwd_dq<D, CAP, DENSE, false, PAD>), dim3(static_cast<unsigned>(nq)), dim3(kThreads), 0,
                         stream, p);
  }
  return hipGetLastError();
}

template <int D, bool PAD>
hipError_t go_p(const BwdParams &p, hipStream_t stream) {
  if (p.f.cap) return p.f.dense ? go<D, true, true, PAD>(p, stream) : go<D, true, false, PAD>(p, stream);
  return p.f.dense ? go<D, false, true, PAD>(p, stream) : go<D, false, false, PAD>(p, stream);
}

template <int D>
hipError_t go_d(const BwdParams &p, hipStream_t stream) {
  const FwdParams &f = p.f;
  const int64_t rows = f.B * f.Hq * f.Sq;
  if (rows > 0) {
    const int64_t threads = rows * (D / 8);
    hipLaunchKernelGGL((bwd_delta<D>), dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const __bf16 *>(f.out), static_cast<const __bf16 *>(p.dout), p.delta, rows,
                       f.padded ? f.dv : D);
  }
  return f.padded ? go_p<D, true>(p, stream) : go_p<D, false>(p, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdParams &p, hipStream_t stream) {
  return p.f.D == 64 ? go_d<64>(p, stream) : go_d<128>(p, stream);
}

}  // namespace splash
