// Device helpers shared by the decode, prefill and quantiser kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16;
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));

#define RIVER_DEV __device__ __forceinline__

static constexpr int kWave = 64;
static constexpr int kBlock = 256;  // every kernel uses 4 waves per workgroup

// ---------------------------------------------------------------------------------------
// Weight-stream geometry. One "chunk" is what a wave reads of one matrix row with one
// 16-byte load per lane: 512 fp16 elements, or 2048 int4 elements (1 KiB either way).
// ---------------------------------------------------------------------------------------
static constexpr int kChunkF16 = 512;
static constexpr int kChunkW4 = 2048;

// Row stride (bytes) of the device int4 layout: ceil(K / 2048) chunks of 1 KiB.
__host__ __device__ inline int64_t w4_row_bytes(int K) {
  return (int64_t)((K + kChunkW4 - 1) / kChunkW4) * 1024;
}
// Scales per row of the device int4 layout (groups covering the padded row).
__host__ __device__ inline int64_t w4_row_scales(int K, int group) {
  return (int64_t)((K + kChunkW4 - 1) / kChunkW4) * (kChunkW4 / group);
}

// ---------------------------------------------------------------------------------------
// Bit casts, fp16 conversions
// ---------------------------------------------------------------------------------------
RIVER_DEV h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
RIVER_DEV uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }
RIVER_DEV float h2f(f16 x) { return (float)x; }
RIVER_DEV f16 f2h(float x) { return (f16)x; }  // round to nearest even

// fp32 dot of two fp16 pairs accumulated into c (v_dot2_f32_f16)
RIVER_DEV float dot2(h2 a, h2 b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }

// ---------------------------------------------------------------------------------------
// int4 unpack. A dword holds 8 offset-binary nibbles u_m (element m in bits 4m..4m+3).
// OR-ing a nibble into the mantissa of fp16 1024.0 (0x6400) gives 1024 + u exactly; a
// nibble in bits 4..7 of a half gives 1024 + 16u. Subtracting the bias leaves q = u - 8
// exactly in fp16. Output pairs: (q0,q4), (q1,q5), (q2,q6), (q3,q7).
// ---------------------------------------------------------------------------------------
RIVER_DEV void unpack8(uint32_t w, h2& p0, h2& p1, h2& p2, h2& p3) {
  const uint32_t lo = 0x000F000Fu, hi = 0x00F000F0u, magic = 0x64006400u;
  const uint32_t w8 = w >> 8;
  const h2 b0 = as_h2((w & lo) | magic);
  const h2 b1 = as_h2((w & hi) | magic);
  const h2 b2 = as_h2((w8 & lo) | magic);
  const h2 b3 = as_h2((w8 & hi) | magic);
  const h2 off = {(f16)1032.0f, (f16)1032.0f};
  const h2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
  const h2 off16 = {(f16)72.0f, (f16)72.0f};
  p0 = b0 - off;
  p1 = b1 * sixteenth - off16;
  p2 = b2 - off;
  p3 = b3 * sixteenth - off16;
}

// Reorders 8 consecutive fp16 values (x0..x7 as pairs (x0,x1),(x2,x3),(x4,x5),(x6,x7)) into
// the pairing unpack8 produces: (x0,x4),(x1,x5),(x2,x6),(x3,x7).
RIVER_DEV void pair_for_unpack(const uint32_t in[4], h2 out[4]) {
  // __builtin_amdgcn_perm(a, b, sel): byte k of result = byte sel_k of {a:b} (b = bytes 0-3)
  out[0] = as_h2(__builtin_amdgcn_perm(in[2], in[0], 0x05040100u));  // x0 | x4<<16
  out[1] = as_h2(__builtin_amdgcn_perm(in[2], in[0], 0x07060302u));  // x1 | x5<<16
  out[2] = as_h2(__builtin_amdgcn_perm(in[3], in[1], 0x05040100u));  // x2 | x6<<16
  out[3] = as_h2(__builtin_amdgcn_perm(in[3], in[1], 0x07060302u));  // x3 | x7<<16
}

// ---------------------------------------------------------------------------------------
// Wave / block reductions (fixed order: deterministic for identical inputs)
// ---------------------------------------------------------------------------------------
RIVER_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
// DPP lane permutation of a float (full row and bank masks: every lane is written).
template <int CTRL>
RIVER_DEV float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of N (8 or 16) lanes; every lane of the group gets the sum.
// quad_perm [1,0,3,2] and [2,3,0,1] make quad sums; the half-row mirror (lane i <-> 7-i) adds
// the other quad of the 8; the row mirror (i <-> 15-i) adds the other half of the 16.
template <int N>
RIVER_DEV float row_sum(float x) {
  static_assert(N == 8 || N == 16, "row group width");
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  if (N == 16) x += dpp_f<0x140>(x);
  return x;
}

// Sum over the wave without LDS traffic: row sums by DPP, then the four row results read as
// scalars. Every lane gets the result.
RIVER_DEV float wave_sum_fast(float v) {
  v = row_sum<16>(v);
  const int u = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 48));
  return (r0 + r1) + (r2 + r3);
}

// Max over the wave, same scheme as wave_sum_fast.
RIVER_DEV float wave_max_fast(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  const int u = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

RIVER_DEV double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
RIVER_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Sum over the 256 threads of a block; every thread gets the result. `red` is >= 4 slots.
RIVER_DEV float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}
RIVER_DEV double block_sum_d(double v, double* red) {
  v = wave_sum_d(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// ---------------------------------------------------------------------------------------
// Cross-workgroup "last arriver" merge without L2 write-backs. Partial results are written
// with agent-scope atomic stores (write-through to the device-coherent level, `sc1`) and read
// back with agent-scope atomic loads (which do not hit a stale line in this XCD's L2). Each
// wave waits for its own stores to complete (s_waitcnt vmcnt(0)), the workgroup meets at a
// barrier, and one thread bumps the counter; the workgroup that sees count-1 merges and resets
// the counter for the next launch. Nothing waits on another workgroup.
// ---------------------------------------------------------------------------------------
RIVER_DEV void wt_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
RIVER_DEV float wt_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
RIVER_DEV bool arrive_counter(int* counter, int count, int* lds_flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = (old == count - 1);
  }
  __syncthreads();
  return *lds_flag != 0;
}
RIVER_DEV void reset_counter(int* counter) {
  __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key).
RIVER_DEV uint32_t float_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
RIVER_DEV float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __builtin_bit_cast(float, u);
}
