// Persistent early-exit decode for one row: one cooperative launch runs S decode steps.
//
// Every workgroup walks the same phase sequence -- per layer QKV, attention, O, gate|up, down,
// then the LM head -- and all workgroups meet at a grid barrier between phases. The method is
// the one the per-op kernels implement (River-LLM, Shen & Zou: the W4A16 exit layer of each
// block shares the block's KV slot, aitrends.kr construction and KV-share paragraphs,
// paperlayer.ai summary of arXiv 2604.18396v3 section 4; a token leaves the backbone after
// block l when cos(h(l-1), h(l)) > tau, aitrends exit-criterion paragraph).
//
// GEMV phases stream rows: the phase's N rows are split evenly over all waves of the grid;
// each wave walks its rows in weight segments (up to 8 KB per wave), double-buffered so the
// next segment's loads are in flight while the current one is reduced against the input
// vector, which every workgroup stages once per phase in LDS (normalised on the fly). No
// workgroup-level synchronisation happens per row; each row's dot product ends in a wave
// reduction and lane 0 stores the result. RoPE and the KV append move to the attention phase
// (the split that owns the new position rotates k, writes K/V[pos], then attends), SwiGLU to
// the staging of the down projection's input.
//
// Routes, the position and the token stay in registers (every workgroup derives identical
// values); activations cross XCDs through write-through stores and coherent loads. The grid
// barrier spins with a bound: a workgroup that waits too long raises an abort flag, after
// which every barrier returns at once, so every wave reaches the end of the kernel.
#include <type_traits>

#include "gemv.hpp"

static constexpr unsigned kSpinLimit = 1u << 22;
static constexpr int kMaxK = 16384;  // longest GEMV input the LDS staging buffer holds
static constexpr int kPB = 512;      // threads per persistent workgroup (one per CU)
static constexpr int kPW = kPB / kWave;

// Sum over the kPB threads of the workgroup, fixed order; every thread gets the result.
RIVER_DEV double pblock_sum_d(double v, double* red) {
  v = wave_sum_d(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < kPW; ++j) s += red[j];
  return s;
}

RIVER_DEV void grid_sync(unsigned* bar, unsigned& target, unsigned nwg, int* abort) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores have landed
  __syncthreads();
  target += nwg;
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned spins = 0;
    while (__hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(1);
      if ((++spins & 255u) == 0) {
        if (__hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
        if (spins > kSpinLimit) {
          __hip_atomic_store(abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------------------
// LDS
// ---------------------------------------------------------------------------------------
// Attention lane mapping: a position is handled by G*LPT lanes, LPT = D/8 lanes per query head
// (8 dims each); TPW positions per wave pass, NGRP position groups per workgroup.
template <int D, int G>
struct AttnBufs {
  static constexpr int LPT = D / 8;
  static constexpr int LPP = G * LPT;      // lanes per position
  static constexpr int TPW = kWave / LPP;  // positions per wave pass
  static constexpr int NGRP = kPW * TPW;
  float m[NGRP][G];
  float l[NGRP][G];
  float acc[NGRP][G][D];
  float w[G][64];
  float L[G];
};

template <int D, int G>
struct PSmem {
  union {
    h2 x[kMaxK / 2];  // staged GEMV input
    AttnBufs<D, G> at;
  };
  double red[kPW];
  double c3[3];
  int flag;
};

// ---------------------------------------------------------------------------------------
// Staging the input vector into LDS
// ---------------------------------------------------------------------------------------
// Layout: fp16 stream -> natural order; int4 stream -> for chunk c (2048 elements), sub-group
// m (8 elements) and lane j the 4 pairs unpack8 expects, at h2 index ((c*4 + m)*64 + j)*4.
// Groups past K are zero up to the last chunk.
template <bool IS4>
RIVER_DEV int lds_group_index(int g) {  // g: group of 8 elements -> h2 index
  if (!IS4) return g * 4;
  const int e = g * 8;
  const int c = e / kChunkW4, j = (e % kChunkW4) / 32, m = (e % 32) / 8;
  return ((c * 4 + m) * kWave + j) * 4;
}

RIVER_DEV uint4 silu_mul8(uint4 g, uint4 u) {
  uint32_t* pg = (uint32_t*)&g;
  const uint32_t* pu = (const uint32_t*)&u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const h2 gv = as_h2(pg[j]), uv = as_h2(pu[j]);
    h2 r;
    const float g0 = h2f(gv.x), g1 = h2f(gv.y);
    r.x = f2h(g0 / (1.f + __expf(-g0)) * h2f(uv.x));
    r.y = f2h(g1 / (1.f + __expf(-g1)) * h2f(uv.y));
    pg[j] = as_u32(r);
  }
  return g;
}

// Writes one group of 8 staged values into LDS in the stream's layout.
template <bool IS4>
RIVER_DEV void put_group(h2* xl, int g, uint4 u) {
  h2* dst = xl + lds_group_index<IS4>(g);
  if (IS4) {
    const uint32_t in[4] = {u.x, u.y, u.z, u.w};
    h2 o[4];
    pair_for_unpack(in, o);
    dst[0] = o[0];
    dst[1] = o[1];
    dst[2] = o[2];
    dst[3] = o[3];
  } else {
    dst[0] = as_h2(u.x);
    dst[1] = as_h2(u.y);
    dst[2] = as_h2(u.z);
    dst[3] = as_h2(u.w);
  }
}

// x = fp16(src * inv * gain) (HAS_GAIN), silu(g)*u of a gate|up vector (SWIGLU), or src, staged
// into LDS. NORM: inv = 1/rms(src) computed here in a fixed order (identical in every
// workgroup); then each thread holds its NG groups of 8 values across the reduction.
// Without NORM the groups stream through registers.
template <bool IS4, bool HAS_GAIN, bool NORM, bool SWIGLU, int NG>
RIVER_DEV void stage_x(const f16* src, const f16* gain, int K, int F, float inv, float eps,
                       h2* xl, double* red) {
  const int t = threadIdx.x;
  const int nch = IS4 ? (K + kChunkW4 - 1) / kChunkW4 : (K + kChunkF16 - 1) / kChunkF16;
  const int ngp = nch * (IS4 ? kChunkW4 : kChunkF16) / 8;
  if (NORM) {
    uint4 v[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int g = t + i * kPB;
      v[i] = (g * 8 < K) ? ldx16<true>(src + g * 8) : make_uint4(0, 0, 0, 0);
    }
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < NG; ++i) ss += sq8(v[i]);
    inv = inv_rms(pblock_sum_d(ss, red), K, eps);
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int g = t + i * kPB;
      if (g >= ngp) continue;
      uint4 u = v[i];
      if (HAS_GAIN && g * 8 < K) u = norm8(u, ldg16(gain + g * 8), inv, true);
      put_group<IS4>(xl, g, u);
    }
    for (int g = t + NG * kPB; g < ngp; g += kPB) put_group<IS4>(xl, g, make_uint4(0, 0, 0, 0));
  } else {
    for (int g = t; g < ngp; g += kPB) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (g * 8 < K) {
        u = ldx16<true>(src + g * 8);
        if (SWIGLU) u = silu_mul8(u, ldx16<true>(src + F + g * 8));
        if (HAS_GAIN) u = norm8(u, ldg16(gain + g * 8), inv, true);
      }
      put_group<IS4>(xl, g, u);
    }
  }
  __syncthreads();
}

// Exit-test reduction of cos(h(l-1), h(l)) over the whole block in a fixed order.
RIVER_DEV void block_cos(const f16* u, const f16* v, int d, double* red, double& dot, double& nu,
                         double& nv) {
  double s0 = 0, s1 = 0, s2 = 0;
  for (int g = threadIdx.x; g * 8 < d; g += kPB) {
    const uint4 a = ldx16<true>(u + g * 8), b = ldx16<true>(v + g * 8);
    const f16* ha = (const f16*)&a;
    const f16* hb = (const f16*)&b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double x = (double)h2f(ha[i]), y = (double)h2f(hb[i]);
      s0 += x * y;
      s1 += x * x;
      s2 += y * y;
    }
  }
  dot = pblock_sum_d(s0, red);
  nu = pblock_sum_d(s1, red);
  nv = pblock_sum_d(s2, red);
}

// ---------------------------------------------------------------------------------------
// Row streaming
// ---------------------------------------------------------------------------------------
template <int OP>
RIVER_DEV const f16* row16(const DecodeArgs& a, const LayerDev* lw, int n) {
  const Dims& dm = a.dm;
  if (OP == OP_QKV) {
    if (n < dm.hd) return lw->wq + (size_t)n * dm.d;
    if (n < dm.hd + dm.Hkv * dm.D) return lw->wk + (size_t)(n - dm.hd) * dm.d;
    return lw->wv + (size_t)(n - dm.hd - dm.Hkv * dm.D) * dm.d;
  }
  if (OP == OP_O) return lw->wo + (size_t)n * dm.hd;
  if (OP == OP_GU) return n < dm.F ? lw->wg + (size_t)n * dm.d : lw->wu + (size_t)(n - dm.F) * dm.d;
  if (OP == OP_DOWN) return lw->wd + (size_t)n * dm.F;
  return a.lm_head + (size_t)n * dm.d;
}

// One streamed item: SEG chunks of one row (fp16: 512 elements per chunk, int4: 2048).
template <bool IS4, int SEG>
struct Seg {
  uint4 w[SEG];
  f16 s[SEG];
};

template <int OP, bool IS4, int SEG>
RIVER_DEV void load_seg(const DecodeArgs& a, const LayerDev* lw, int K, int nch, int row, int seg,
                        Seg<IS4, SEG>& sg) {
  const int lane = threadIdx.x & (kWave - 1);
  if (!IS4) {
    const f16* rp = row16<OP>(a, lw, row);
#pragma unroll
    for (int c = 0; c < SEG; ++c) {
      const int ch = seg * SEG + c;
      if (ch >= nch) break;  // uniform; dot_seg stops at the same chunk
      const int e = ch * kChunkF16 + lane * 8;
      sg.w[c] = ldg16(rp + (e < K ? e : 0));  // past K (ragged row end) meets x = 0
    }
  } else {
    const uint8_t* rp;
    const f16* sp;
    w4_row(OP, row, *lw, a.dm, rp, sp);
#pragma unroll
    for (int c = 0; c < SEG; ++c) {
      const int ch = seg * SEG + c;
      if (ch >= nch) break;
      sg.w[c] = ldg16(rp + (size_t)ch * 1024 + lane * 16);
      sg.s[c] = ldg2(sp + (ch * kChunkW4 + lane * 32) / a.dm.group);
    }
  }
}

template <bool IS4, int SEG>
RIVER_DEV float dot_seg(const Seg<IS4, SEG>& sg, const h2* xl, int nch, int seg) {
  const int lane = threadIdx.x & (kWave - 1);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < SEG; ++c) {
    const int ch = seg * SEG + c;
    if (ch >= nch) break;
    if (!IS4) {
      const h2* x = xl + (ch * kWave + lane) * 4;
      acc = dot2(x[0], as_h2(sg.w[c].x), acc);
      acc = dot2(x[1], as_h2(sg.w[c].y), acc);
      acc = dot2(x[2], as_h2(sg.w[c].z), acc);
      acc = dot2(x[3], as_h2(sg.w[c].w), acc);
    } else {
      const uint32_t ww[4] = {sg.w[c].x, sg.w[c].y, sg.w[c].z, sg.w[c].w};
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const h2* x = xl + ((ch * 4 + m) * kWave + lane) * 4;
        h2 p0, p1, p2, p3;
        unpack8(ww[m], p0, p1, p2, p3);
        s = dot2(p0, x[0], s);
        s = dot2(p1, x[1], s);
        s = dot2(p2, x[2], s);
        s = dot2(p3, x[3], s);
      }
      acc = fmaf(h2f(sg.s[c]), s, acc);
    }
  }
  return acc;
}

// Epilogue inputs of a streamed phase.
struct StreamOut {
  f16* out;           // QKV -> qkvr, GU -> gu, O -> hmid, DOWN -> hs[l]
  const f16* resid;   // O, DOWN: residual input
  float* logits;      // LM (optional)
  unsigned long long* key;  // LM argmax key
};

// Streams this wave's rows [r0, r1) of an N-row phase; the input vector is staged in xl.
template <int OP, bool IS4, int SEG>
RIVER_DEV void stream_rows(const DecodeArgs& a, const LayerDev* lw, int N, int K, const h2* xl,
                           const StreamOut& so, Seg<IS4, SEG>& b0) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kPW + threadIdx.x / kWave, GW = gridDim.x * kPW;
  const int r0 = (int)((long long)gw * N / GW), r1 = (int)((long long)(gw + 1) * N / GW);
  const int nch = IS4 ? (K + kChunkW4 - 1) / kChunkW4 : (K + kChunkF16 - 1) / kChunkF16;
  const int nseg = (nch + SEG - 1) / SEG;
  const int nitems = (r1 - r0) * nseg;
  // residuals of this wave's rows, one per lane (O and DOWN)
  f16 res = (f16)0.0f;
  if ((OP == OP_O || OP == OP_DOWN) && r0 + lane < r1) res = ldh<true>(so.resid + r0 + lane);
  float best = -__builtin_inff();
  int bi = 0x7FFFFFFF;
  Seg<IS4, SEG> b1;  // b0 holds the first segment, issued by prefetch_first
  float acc = 0.f;
  auto finish = [&](int it, float part) {
    acc += part;
    const int seg = it % nseg;
    if (seg != nseg - 1) return;
    const int row = r0 + it / nseg;
    const float v = wave_sum(acc);
    acc = 0.f;
    if (OP == OP_LM) {
      if (v > best) {
        best = v;
        bi = row;
      }
    }
    const int rr = row - r0;
    f16 rv = (f16)0.0f;
    if (OP == OP_O || OP == OP_DOWN) {
      const int src = rr < kWave ? rr : 0;
      rv = __builtin_bit_cast(f16, (unsigned short)__shfl(__builtin_bit_cast(unsigned short, res), src, kWave));
      if (rr >= kWave) rv = ldh<true>(so.resid + row);
    }
    if (lane == 0) {
      if (OP == OP_QKV || OP == OP_GU) sth<true>(so.out + row, f2h(v));
      if (OP == OP_O || OP == OP_DOWN) sth<true>(so.out + row, f2h(h2f(rv) + h2f(f2h(v))));
      if (OP == OP_LM && so.logits) so.logits[row] = v;
    }
  };
  int it = 0;
  for (; it + 1 < nitems; it += 2) {
    load_seg<OP, IS4, SEG>(a, lw, K, nch, r0 + (it + 1) / nseg, (it + 1) % nseg, b1);
    finish(it, dot_seg<IS4, SEG>(b0, xl, nch, it % nseg));
    if (it + 2 < nitems) load_seg<OP, IS4, SEG>(a, lw, K, nch, r0 + (it + 2) / nseg, (it + 2) % nseg, b0);
    finish(it + 1, dot_seg<IS4, SEG>(b1, xl, nch, (it + 1) % nseg));
  }
  if (it < nitems) finish(it, dot_seg<IS4, SEG>(b0, xl, nch, it % nseg));
  if (OP == OP_LM && lane == 0 && bi != 0x7FFFFFFF) {
    const unsigned long long key = ((unsigned long long)float_key(best) << 32) |
                                   (unsigned long long)(0xFFFFFFFFu - (uint32_t)bi);
    __hip_atomic_fetch_max(so.key, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Issues the first segment of this wave's rows (weights only: allowed before the inputs of the
// phase exist, e.g. before the grid barrier or while the input vector is staged).
template <int OP, bool IS4, int SEG>
RIVER_DEV bool prefetch_first(const DecodeArgs& a, const LayerDev* lw, int N, int K,
                              Seg<IS4, SEG>& pre) {
  const int gw = blockIdx.x * kPW + threadIdx.x / kWave, GW = gridDim.x * kPW;
  const int r0 = (int)((long long)gw * N / GW), r1 = (int)((long long)(gw + 1) * N / GW);
  if (r0 >= r1) return false;
  const int nch = IS4 ? (K + kChunkW4 - 1) / kChunkW4 : (K + kChunkF16 - 1) / kChunkF16;
  load_seg<OP, IS4, SEG>(a, lw, K, nch, r0, 0, pre);
  return true;
}

// One GEMV phase: prefetch the first weight segment, stage the input, stream the rows.
template <int OP, bool IS4, int SEG, bool HAS_GAIN, bool NORM, bool SWIGLU, int NG>
RIVER_DEV void gemv_phase(const DecodeArgs& a, const LayerDev* lw, int N, int K, const f16* src,
                          const f16* gain, float inv, const StreamOut& so, h2* xl, double* red) {
  Seg<IS4, SEG> b0;
  prefetch_first<OP, IS4, SEG>(a, lw, N, K, b0);
  stage_x<IS4, HAS_GAIN, NORM, SWIGLU, NG>(src, gain, K, a.dm.F, inv, a.dm.eps, xl, red);
  stream_rows<OP, IS4, SEG>(a, lw, N, K, xl, so, b0);
  __syncthreads();  // LDS reuse by the next phase
}

// ---------------------------------------------------------------------------------------
// Attention (one split of one KV head), reading un-rotated q/k/v of the new position
// ---------------------------------------------------------------------------------------
static constexpr int kMinChunkP = 64;

template <int D, int G>
RIVER_DEV void attn_split(const DecodeArgs& a, int layer, int s, int kvh, int b, int pos,
                          int smax, AttnBufs<D, G>& sm, int* flag) {
  constexpr int LPT = AttnBufs<D, G>::LPT;
  constexpr int LPP = AttnBufs<D, G>::LPP;
  constexpr int TPW = AttnBufs<D, G>::TPW;
  constexpr int NGRP = AttnBufs<D, G>::NGRP;
  constexpr int U = 4;  // positions per group per iteration (loads in flight)
  static_assert(LPP <= kWave, "one position must fit in a wave");
  const Dims& dm = a.dm;
  const int T = pos + 1;
  const int chunk = max(kMinChunkP, (T + smax - 1) / smax);
  const int seff = (T + chunk - 1) / chunk;
  const size_t hstride = (size_t)dm.Tmax * D;
  f16* Kb = a.kv + ((((size_t)(layer - 1) * 2 + 0) * dm.B + b) * dm.Hkv + kvh) * hstride;
  f16* Vb = a.kv + ((((size_t)(layer - 1) * 2 + 1) * dm.B + b) * dm.Hkv + kvh) * hstride;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int grp = w * TPW + lane / LPP;     // position group
  const int g = (lane % LPP) / LPT;         // query head within the KV group
  const int sub = lane % LPT, d0 = sub * 8;  // dims [d0, d0+8)
  const size_t pbase = ((size_t)b * dm.H + (size_t)kvh * G) * smax;
  const f16* qkv = a.qkvr + (size_t)b * dm.nqkv;
  const float2* rope = a.rope + (size_t)pos * (D / 2);

  // rotate-half RoPE of dims [d0, d0+8): the partner dims (d +- D/2) sit in lane ^ LPT/2
  auto rope8 = [&](uint4 raw, float (&out)[8]) {
    const uint4 pr = make_uint4(__shfl_xor(raw.x, LPT / 2, kWave), __shfl_xor(raw.y, LPT / 2, kWave),
                                __shfl_xor(raw.z, LPT / 2, kWave), __shfl_xor(raw.w, LPT / 2, kWave));
    const f16* x = (const f16*)&raw;
    const f16* y = (const f16*)&pr;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int dim = d0 + i;
      const float xv = h2f(x[i]), yv = h2f(y[i]);
      if (dim < D / 2) {
        const float2 cs = rope[dim];
        out[i] = h2f(f2h(xv * cs.x - yv * cs.y));
      } else {
        const float2 cs = rope[dim - D / 2];
        out[i] = h2f(f2h(xv * cs.x + yv * cs.y));
      }
    }
  };

  if (s < seff) {
    const int t0 = s * chunk, t1 = min(T, t0 + chunk);
    if (t1 == T) {
      // this split owns the new position: rotate k, append K/V[pos] to the shared cache
      if (w == 0 && lane < LPT) {
        const uint4 kr = ldx16<true>(qkv + dm.hd + (size_t)kvh * D + d0);
        float kf[8];
        rope8(kr, kf);
        uint4 ko;
        f16* kh = (f16*)&ko;
#pragma unroll
        for (int i = 0; i < 8; ++i) kh[i] = f2h(kf[i]);
        const uint4 vr = ldx16<true>(qkv + dm.hd + (size_t)(dm.Hkv + kvh) * D + d0);
        const uint32_t* kw = (const uint32_t*)&ko;
        const uint32_t* vw = (const uint32_t*)&vr;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          __hip_atomic_store((__attribute__((address_space(1))) uint32_t*)(Kb + (size_t)pos * D + d0) + j,
                             kw[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store((__attribute__((address_space(1))) uint32_t*)(Vb + (size_t)pos * D + d0) + j,
                             vw[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    const float qs = 1.4426950408889634f / sqrtf((float)D);
    float qf[8];
    {
      const uint4 qr = ldx16<true>(qkv + (size_t)(kvh * G + g) * D + d0);
      float r[8];
      rope8(qr, r);
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[i] = r[i] * qs;
    }
    float m = -__builtin_inff(), l = 0.f, acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int tb = t0 + grp; tb < t1; tb += NGRP * U) {
      uint4 kk[U], vv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = tb + u * NGRP;
        const size_t tt = (size_t)(t < t1 ? t : t0);
        if (tt == (size_t)pos) {  // written above by this workgroup: read through
          kk[u] = ldx16<true>(Kb + tt * D + d0);
          vv[u] = ldx16<true>(Vb + tt * D + d0);
        } else {
          kk[u] = ldg16(Kb + tt * D + d0);
          vv[u] = ldg16(Vb + tt * D + d0);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = tb + u * NGRP;
        if (t >= t1) break;  // uniform within the position's lanes
        const f16* kh = (const f16*)&kk[u];
        const f16* vh = (const f16*)&vv[u];
        float sc = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) sc = fmaf(qf[i], h2f(kh[i]), sc);
#pragma unroll
        for (int o = 1; o < LPT; o <<= 1) sc += __shfl_xor(sc, o, kWave);
        const float mn = fmaxf(m, sc);
        const float c = exp2f(m - mn);
        const float p = exp2f(sc - mn);
        l = l * c + p;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(acc[i], c, p * h2f(vh[i]));
        m = mn;
      }
    }
    if (sub == 0) {
      sm.m[grp][g] = m;
      sm.l[grp][g] = l;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) sm.acc[grp][g][d0 + i] = acc[i];
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += kPB) {
      const int gg = idx / D, dd = idx % D;
      float M = -__builtin_inff();
      for (int j = 0; j < NGRP; ++j) M = fmaxf(M, sm.m[j][gg]);
      float Ls = 0.f, A = 0.f;
      for (int j = 0; j < NGRP; ++j) {
        const float sc = (sm.l[j][gg] > 0.f) ? exp2f(sm.m[j][gg] - M) : 0.f;
        Ls += sm.l[j][gg] * sc;
        A += sm.acc[j][gg][dd] * sc;
      }
      const size_t pi = pbase + (size_t)gg * smax + s;
      wt_store(&a.pacc[pi * D + dd], A);
      if (dd == 0) {
        wt_store(&a.pml[pi * 2 + 0], M);
        wt_store(&a.pml[pi * 2 + 1], Ls);
      }
    }
  }
  int* counter = a.cnt + CNT_ATTN + b * dm.Hkv + kvh;
  if (arrive_counter(counter, smax, flag)) {
    if (threadIdx.x < G) {
      const int g = threadIdx.x;
      float M = -__builtin_inff();
      for (int j = 0; j < seff; ++j) {
        sm.w[g][j] = wt_load(&a.pml[(pbase + (size_t)g * smax + j) * 2]);
        M = fmaxf(M, sm.w[g][j]);
      }
      float Ls = 0.f;
      for (int j = 0; j < seff; ++j) {
        const float e = exp2f(sm.w[g][j] - M);
        sm.w[g][j] = e;
        Ls += wt_load(&a.pml[(pbase + (size_t)g * smax + j) * 2 + 1]) * e;
      }
      sm.L[g] = Ls;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += kPB) {
      const int g = idx / D, dd = idx % D;
      float A = 0.f;
      for (int j = 0; j < seff; ++j) A += sm.w[g][j] * wt_load(&a.pacc[(pbase + (size_t)g * smax + j) * D + dd]);
      sth<true>(a.o + (size_t)b * dm.hd + (size_t)(kvh * G + g) * D + dd, f2h(A / sm.L[g]));
    }
    if (threadIdx.x == 0) reset_counter(counter);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------------------
template <int D, int G, int MODE, int SEG16, int SEG4, int NG>
__global__ __launch_bounds__(kPB) void k_persist(DecodeArgs a, int S, int splits, unsigned* bar,
                                                    int* abort) {
  __shared__ PSmem<D, G> sm;
  const Dims& dm = a.dm;
  const int b = 0;
  const unsigned nwg = gridDim.x;
  const int wg = blockIdx.x, t = threadIdx.x;
  unsigned target = 0;
  int pos = a.pos[b];
  int tok = a.tok_in[b];
  h2* xl = sm.x;

  for (int step = 0; step < S; ++step, ++pos) {
    if (tok < 0 || tok >= dm.V) {
      if (wg == 0 && t == 0) atomicOr(a.err, ERR_TOKEN);
      tok = 0;
    }
    int e_forced = dm.L;
    if (MODE == 0 && a.sched) {
      e_forced = a.sched[step * dm.B + b];
      if (e_forced < dm.entry || e_forced > dm.L) {
        if (wg == 0 && t == 0) atomicOr(a.err, ERR_FORCED);
        e_forced = dm.L;
      }
    }
    int route = ROUTE_BACKBONE;
    for (int l = 1; l <= dm.L; ++l) {
      const LayerDev* lw = &a.layers[l - 1];
      // ---------------- QKV (exit test after block l-1 first)
      const f16* hin = (l == 1) ? a.embed + (size_t)tok * dm.d : a.hs + ((size_t)(l - 1) * dm.B + b) * dm.d;
      bool norm_known = false;
      float inv = 1.f;
      if (l == 1) {
        if (wg == 0) {
          f16* h0 = a.hs + (size_t)b * dm.d;
          for (int i = t; i < dm.d; i += kPB) sth<true>(h0 + i, hin[i]);
          if (t == 0 && a.exit_out) a.exit_out[step * dm.B + b] = dm.L;
          if (a.sim_out)
            for (int i = t; i < dm.L; i += kPB)
              a.sim_out[((size_t)step * dm.B + b) * dm.L + i] = __builtin_nanf("");
        }
      } else if (MODE == 0 && route == ROUTE_BACKBONE && l - 1 >= dm.entry) {
        const int lp = l - 1;
        if (a.sched) {
          if (lp == e_forced) route = ROUTE_RIVER;
        } else {
          double dot, n1, n2;
          block_cos(a.hs + ((size_t)(lp - 1) * dm.B + b) * dm.d, hin, dm.d, sm.red, dot, n1, n2);
          const double sim = (n1 > 0.0 && n2 > 0.0) ? dot / sqrt(n1 * n2) : 0.0;
          if (wg == 0 && t == 0 && a.sim_out) a.sim_out[((size_t)step * dm.B + b) * dm.L + lp - 1] = (float)sim;
          if (sim > (double)a.tau) route = ROUTE_RIVER;
          inv = inv_rms(n2, dm.d, dm.eps);
          norm_known = true;
        }
        if (route == ROUTE_RIVER && wg == 0 && t == 0 && a.exit_out) a.exit_out[step * dm.B + b] = lp;
      }
      const bool r4 = route == ROUTE_RIVER;
      StreamOut so{};
      so.out = a.qkvr + (size_t)b * dm.nqkv;
      if (r4) {
        if (norm_known) gemv_phase<OP_QKV, true, SEG4, true, false, false, NG>(a, lw, dm.nqkv, dm.d, hin, lw->attn_norm, inv, so, xl, sm.red);
        else gemv_phase<OP_QKV, true, SEG4, true, true, false, NG>(a, lw, dm.nqkv, dm.d, hin, lw->attn_norm, inv, so, xl, sm.red);
      } else {
        if (norm_known) gemv_phase<OP_QKV, false, SEG16, true, false, false, NG>(a, lw, dm.nqkv, dm.d, hin, lw->attn_norm, inv, so, xl, sm.red);
        else gemv_phase<OP_QKV, false, SEG16, true, true, false, NG>(a, lw, dm.nqkv, dm.d, hin, lw->attn_norm, inv, so, xl, sm.red);
      }
      grid_sync(bar, target, nwg, abort);
      if (l == 1 && wg == 0 && t == 0)  // key of the next step: last read before this barrier
        __hip_atomic_store(a.amax + ((step + 1) & 1) * dm.B + b, 0ull, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      // ---------------- attention (+ RoPE and the KV append of position pos)
      for (int it = wg; it < dm.Hkv * splits; it += nwg)
        attn_split<D, G>(a, l, it % splits, it / splits, b, pos, splits, sm.at, &sm.flag);
      grid_sync(bar, target, nwg, abort);
      // ---------------- O + residual
      so.out = a.hmid + ((size_t)(l - 1) * dm.B + b) * dm.d;
      so.resid = a.hs + ((size_t)(l - 1) * dm.B + b) * dm.d;
      if (r4) gemv_phase<OP_O, true, SEG4, false, false, false, NG>(a, lw, dm.d, dm.hd, a.o + (size_t)b * dm.hd, nullptr, 1.f, so, xl, sm.red);
      else gemv_phase<OP_O, false, SEG16, false, false, false, NG>(a, lw, dm.d, dm.hd, a.o + (size_t)b * dm.hd, nullptr, 1.f, so, xl, sm.red);
      grid_sync(bar, target, nwg, abort);
      // ---------------- gate|up
      so.out = a.gu + (size_t)b * 2 * dm.F;
      so.resid = nullptr;
      {
        const f16* src = a.hmid + ((size_t)(l - 1) * dm.B + b) * dm.d;
        if (r4) gemv_phase<OP_GU, true, SEG4, true, true, false, NG>(a, lw, 2 * dm.F, dm.d, src, lw->mlp_norm, 1.f, so, xl, sm.red);
        else gemv_phase<OP_GU, false, SEG16, true, true, false, NG>(a, lw, 2 * dm.F, dm.d, src, lw->mlp_norm, 1.f, so, xl, sm.red);
      }
      grid_sync(bar, target, nwg, abort);
      // ---------------- down (SwiGLU while staging) + residual
      so.out = a.hs + ((size_t)l * dm.B + b) * dm.d;
      so.resid = a.hmid + ((size_t)(l - 1) * dm.B + b) * dm.d;
      if (r4) gemv_phase<OP_DOWN, true, SEG4, false, false, true, NG>(a, lw, dm.d, dm.F, a.gu + (size_t)b * 2 * dm.F, nullptr, 1.f, so, xl, sm.red);
      else gemv_phase<OP_DOWN, false, SEG16, false, false, true, NG>(a, lw, dm.d, dm.F, a.gu + (size_t)b * 2 * dm.F, nullptr, 1.f, so, xl, sm.red);
      grid_sync(bar, target, nwg, abort);
    }
    // ---------------- LM head (final RMSNorm while staging) + argmax
    {
      StreamOut so{};
      so.logits = a.logits ? a.logits + (size_t)b * dm.V : nullptr;
      so.key = a.amax + (step & 1) * dm.B + b;
      gemv_phase<OP_LM, false, SEG16, true, true, false, NG>(a, nullptr, dm.V, dm.d, a.hs + ((size_t)dm.L * dm.B + b) * dm.d,
                                                         a.final_norm, 1.f, so, xl, sm.red);
      grid_sync(bar, target, nwg, abort);
      const unsigned long long k = __hip_atomic_load(so.key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      tok = (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
      if (wg == 0 && t == 0) a.tok_out[step * dm.B + b] = tok;
    }
  }
  if (wg == 0 && t == 0) {
    a.pos[b] = pos;
    *a.step = S;
    if (__hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicOr(a.err, ERR_SYNC);
  }
}

// ---------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------
// The kernel function for this model and mode (batch 1, GEMV inputs up to 16384), or null.
const void* river_persist_fn(const Dims& dm, int mode) {
  if (dm.B != 1 || dm.d > kMaxK || dm.hd > kMaxK || dm.F > kMaxK) return nullptr;
  const int G = dm.H / dm.Hkv;
  const int ng = (dm.d + 8 * kPB - 1) / (8 * kPB);  // groups of 8 per thread for K = d
#define RIVER_PF(D_, G_, NG_)                                                                    \
  if (dm.D == D_ && G == G_ && ng == NG_)                                                        \
    return mode ? (const void*)k_persist<D_, G_, 1, 8, 4, NG_> : (const void*)k_persist<D_, G_, 0, 8, 4, NG_>;
  RIVER_PF(128, 4, 1)
  RIVER_PF(64, 4, 1)
  RIVER_PF(64, 2, 1)
#undef RIVER_PF
  return nullptr;
}

// Workgroups of the persistent grid: one per CU, all co-resident (cooperative launch).
int river_persist_grid(const void* fn) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kPB, 0) != hipSuccess) return 0;
  return per_cu >= 1 ? cus : 0;
}

hipError_t river_launch_persist(const void* fn, const DecodeArgs& a, int S, int nwg, int splits,
                                unsigned* bar, int* abort, hipStream_t st) {
  DecodeArgs aa = a;
  int SS = S, sp = splits;
  unsigned* br = bar;
  int* ab = abort;
  void* args[] = {&aa, &SS, &sp, &br, &ab};
  return hipLaunchCooperativeKernel(fn, dim3(nwg), dim3(kPB), args, 0, st);
}
