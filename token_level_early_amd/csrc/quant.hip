// River construction: the W4A16 copy of every block (aitrends.kr article, construction
// paragraph: the exit layer copies the block's weights and applies 4-bit weight quantisation;
// paperlayer.ai summary of arXiv 2604.18396v3, section 4 "KV-Shared Exit Layer").
//
// Quantiser (the pages give no formula; this is the project's convention): symmetric
// round-to-nearest int4 per group of `group` consecutive input columns. For each group:
//   amax = max |w| (exact), s = fp16(fp32(amax / 7)), q = clamp(rint(fp32(w / s)), -8, 7)
//   (round half to even), s == 0 -> q = 0; stored nibble u = q + 8.
// The fp32 quotients are formed in fp64 and rounded once to fp32, which equals the correctly
// rounded fp32 quotient (53 >= 2*24 + 2), so codes and scales are bit-exact with any IEEE
// implementation of the same formula.
#include "params.hpp"

// Zero-point format (the scale-and-zero storage of the pages' other backends, HQQ and AWQ:
// paperlayer.ai summary, appendix A.1; without their calibration): asymmetric round-to-nearest
// int4 per group, the range widened to hold 0:
//   lo = min(min w, 0), hi = max(max w, 0), s = fp16(fp32((hi - lo) / 15)) (hi - lo exact in
//   fp64, fp64 quotient rounded to fp32, then to fp16), s == 0 -> q = 0 and z = 0, else
//   z = clamp(rint(fp32(-lo / s)), 0, 15), q = clamp(rint(fp32(w / s)) + z, 0, 15); nibble u = q.

// One thread per (row, group) of the padded device layout; `zeros` selects the format.
__global__ __launch_bounds__(kBlock) void k_quantize(const f16* __restrict__ W, int N, int K,
                                                     int group, uint8_t* __restrict__ out,
                                                     f16* __restrict__ scales,
                                                     uint8_t* __restrict__ zeros) {
  const int64_t rs = w4_row_scales(K, group);
  const int64_t rb = w4_row_bytes(K);
  const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (idx >= (int64_t)N * rs) return;
  const int n = (int)(idx / rs);
  const int j = (int)(idx % rs);
  const int lo = j * group;
  const int hi = min(lo + group, K);
  const f16* row = W + (size_t)n * K;
  if (zeros) {
    float wmin = 0.f, wmax = 0.f;  // the range always holds 0
    for (int k = lo; k < hi; ++k) {
      const float v = h2f(row[k]);
      wmin = fminf(wmin, v);
      wmax = fmaxf(wmax, v);
    }
    const f16 s16 = f2h((float)(((double)wmax - (double)wmin) / 15.0));
    const float s = h2f(s16);
    int z = 0;
    if (s != 0.f) z = (int)fminf(fmaxf(rintf((float)((double)(-wmin) / (double)s)), 0.f), 15.f);
    uint8_t* orow = out + (size_t)n * rb;
    for (int k = lo; k < lo + group; k += 2) {
      int u[2];
      for (int h = 0; h < 2; ++h) {
        const int kk = k + h;
        int q = 0;
        if (kk < hi && s != 0.f) {
          const float r = rintf((float)((double)h2f(row[kk]) / (double)s)) + (float)z;
          q = (int)fminf(fmaxf(r, 0.f), 15.f);
        }
        u[h] = q;
      }
      orow[k / 2] = (uint8_t)(u[0] | (u[1] << 4));
    }
    scales[(size_t)n * rs + j] = (lo < K) ? s16 : (f16)0.0f;
    zeros[(size_t)n * rs + j] = (uint8_t)((lo < K) ? z : 0);
    return;
  }
  float amax = 0.f;
  for (int k = lo; k < hi; ++k) amax = fmaxf(amax, fabsf(h2f(row[k])));
  const float s32 = (float)((double)amax / 7.0);
  const f16 s16 = f2h(s32);
  const float s = h2f(s16);
  uint8_t* orow = out + (size_t)n * rb;
  for (int k = lo; k < lo + group; k += 2) {
    int u[2];
    for (int h = 0; h < 2; ++h) {
      const int kk = k + h;
      int q = 0;
      if (kk < hi && s != 0.f) {
        const float r = rintf((float)((double)h2f(row[kk]) / (double)s));
        q = (int)fminf(fmaxf(r, -8.f), 7.f);
      }
      u[h] = q + 8;
    }
    orow[k / 2] = (uint8_t)(u[0] | (u[1] << 4));
  }
  scales[(size_t)n * rs + j] = (lo < K) ? s16 : (f16)0.0f;
}

// Canonical export: packed [N][ceil(K/2)], scales [N][ceil(K/group)] and, for the zero-point
// format, zero points [N][ceil(K/group)] (drops the padding).
__global__ __launch_bounds__(kBlock) void k_export(const uint8_t* __restrict__ in,
                                                   const f16* __restrict__ sin_,
                                                   const uint8_t* __restrict__ zin, int N, int K,
                                                   int group, uint8_t* __restrict__ packed,
                                                   uint16_t* __restrict__ scales,
                                                   uint8_t* __restrict__ zeros) {
  const int64_t rb = w4_row_bytes(K), rs = w4_row_scales(K, group);
  const int kb = (K + 1) / 2, ng = (K + group - 1) / group;
  const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int64_t nb = (int64_t)N * kb;
  if (idx < nb) {
    const int n = (int)(idx / kb), i = (int)(idx % kb);
    uint8_t v = in[(size_t)n * rb + i];
    if ((K & 1) && i == kb - 1) v = (uint8_t)((v & 0x0F) | (zin ? 0x00 : 0x80));  // pad nibble of odd K
    packed[idx] = v;
  }
  if (idx < (int64_t)N * ng) {
    const int n = (int)(idx / ng), j = (int)(idx % ng);
    scales[idx] = __builtin_bit_cast(uint16_t, sin_[(size_t)n * rs + j]);
    if (zin) zeros[idx] = zin[(size_t)n * rs + j];
  }
}

// RoPE table: (cos, sin) of pos * theta^(-2i/D) in fp64, rounded to fp32.
__global__ __launch_bounds__(kBlock) void k_rope_table(float2* tab, int Tmax, int D, double theta) {
  const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const int half = D / 2;
  if (idx >= (int64_t)Tmax * half) return;
  const int pos = (int)(idx / half), i = (int)(idx % half);
  const double inv = pow(theta, -2.0 * i / D);
  const double ang = (double)pos * inv;
  tab[idx] = make_float2((float)cos(ang), (float)sin(ang));
}

__global__ __launch_bounds__(kBlock) void k_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t river_launch_quantize(const f16* W, int N, int K, int group, uint8_t* out, f16* scales,
                                 uint8_t* zeros, hipStream_t st) {
  const int64_t n = (int64_t)N * w4_row_scales(K, group);
  const int64_t g = (n + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)g), dim3(kBlock), 0, st, W, N, K, group, out, scales,
                     zeros);
  return hipGetLastError();
}

hipError_t river_launch_export(const uint8_t* in, const f16* sin_, const uint8_t* zin, int N, int K,
                               int group, uint8_t* packed, uint16_t* scales, uint8_t* zeros,
                               hipStream_t st) {
  const int64_t n1 = (int64_t)N * ((K + 1) / 2), n2 = (int64_t)N * ((K + group - 1) / group);
  const int64_t n = n1 > n2 ? n1 : n2;
  hipLaunchKernelGGL(k_export, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, st, in,
                     sin_, zin, N, K, group, packed, scales, zeros);
  return hipGetLastError();
}

hipError_t river_launch_rope_table(float2* tab, int Tmax, int D, double theta, hipStream_t st) {
  const int64_t n = (int64_t)Tmax * (D / 2);
  hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, st,
                     tab, Tmax, D, theta);
  return hipGetLastError();
}

// Zero/fill with a kernel (no memset nodes: safe inside captured graphs too).
hipError_t river_launch_fill(void* p, int64_t bytes, uint32_t v, hipStream_t st) {
  const int64_t n = bytes / 4;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, st,
                     (uint32_t*)p, n, v);
  return hipGetLastError();
}

// Writes per KV slot from the debug build's per-element counters (same index as the cache
// [L][2][B][Hkv][Tmax][D]): out[l][b][t] = the common count of the slot's 2*Hkv*D elements, or
// 255 when they differ (part of the slot written more often than the rest). Counts cap at 254.
__global__ __launch_bounds__(kBlock) void k_kv_slot_counts(const uint32_t* __restrict__ cnt, int L, int B,
                                                           int Hkv, int Tmax, int D, uint8_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (idx >= (int64_t)L * B * Tmax) return;
  const int t = (int)(idx % Tmax);
  const int b = (int)((idx / Tmax) % B);
  const int l = (int)(idx / ((int64_t)Tmax * B));
  uint32_t first = 0;
  bool same = true;
  for (int kv = 0; kv < 2; ++kv)
    for (int h = 0; h < Hkv; ++h) {
      const uint32_t* p = cnt + (((((int64_t)l * 2 + kv) * B + b) * Hkv + h) * Tmax + t) * D;
      for (int i = 0; i < D; ++i) {
        if (kv == 0 && h == 0 && i == 0) first = p[0];
        same &= (p[i] == first);
      }
    }
  out[idx] = same ? (uint8_t)(first < 254u ? first : 254u) : (uint8_t)255;
}

hipError_t river_launch_kv_slot_counts(const uint32_t* cnt, int L, int B, int Hkv, int Tmax, int D,
                                       uint8_t* out, hipStream_t st) {
  const int64_t n = (int64_t)L * B * Tmax;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_kv_slot_counts, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock), 0, st,
                     cnt, L, B, Hkv, Tmax, D, out);
  return hipGetLastError();
}
