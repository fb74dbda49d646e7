// GEMV building blocks shared by the per-op decode kernels and the persistent decode kernel.
//
// A tile is TR consecutive rows of one weight stream (fp16 backbone or int4 river) handled by
// one workgroup of 4 waves; waves split the rows into row groups and, for long rows, the chunks
// of a row (WPR waves per row). COH selects coherent activation loads: inside one persistent
// launch, activations written by other workgroups (other XCDs) must be read past this XCD's
// L2 (agent-scope atomic loads, `sc1`); across kernel launches plain loads are coherent.
#pragma once

#include "params.hpp"

static constexpr int kRB16 = 2;  // rows per wave batch, fp16 stream
static constexpr int kRB4 = 4;   // rows per wave batch, int4 stream

template <int WPR>
struct TileF16 {
  static constexpr int NRG = 4 / WPR;
  static constexpr int TR = NRG * kRB16;
};
template <int WPR>
struct TileW4 {
  static constexpr int NRG = 4 / WPR;
  static constexpr int TR = NRG * kRB4;
};

// Logical output row of tile row r. QKV tiles of q/k heads pair row i with row i + D/2 of the
// same head (rotate-half RoPE needs both); gate|up tiles pair gate row f with up row f.
RIVER_DEV int logical_row(int op, int tile, int r, int TR, const Dims& dm) {
  if (op == OP_QKV) {
    const int qk_tiles = (dm.H + dm.Hkv) * dm.D / TR;
    if (tile < qk_tiles) {
      const int tph = dm.D / TR;
      const int head = tile / tph;
      const int half = TR / 2;
      const int i0 = (tile % tph) * half;
      return head * dm.D + (r < half ? i0 + r : dm.D / 2 + i0 + (r - half));
    }
    return tile * TR + r;
  }
  if (op == OP_GU) {
    const int half = TR / 2;
    return r < half ? tile * half + r : dm.F + tile * half + (r - half);
  }
  return tile * TR + r;
}

RIVER_DEV int op_rows(int op, const Dims& dm) {
  switch (op) {
    case OP_QKV: return dm.nqkv;
    case OP_GU: return 2 * dm.F;
    case OP_LM: return dm.V;
    default: return dm.d;
  }
}
RIVER_DEV int op_k(int op, const Dims& dm) {
  switch (op) {
    case OP_O: return dm.hd;
    case OP_DOWN: return dm.F;
    default: return dm.d;
  }
}

RIVER_DEV const f16* f16_row(int op, int n, const LayerDev& lw, const DecodeArgs& a) {
  const Dims& dm = a.dm;
  switch (op) {
    case OP_QKV:
      if (n < dm.hd) return lw.wq + (size_t)n * dm.d;
      if (n < dm.hd + dm.Hkv * dm.D) return lw.wk + (size_t)(n - dm.hd) * dm.d;
      return lw.wv + (size_t)(n - dm.hd - dm.Hkv * dm.D) * dm.d;
    case OP_O: return lw.wo + (size_t)n * dm.hd;
    case OP_GU: return n < dm.F ? lw.wg + (size_t)n * dm.d : lw.wu + (size_t)(n - dm.F) * dm.d;
    case OP_DOWN: return lw.wd + (size_t)n * dm.F;
    default: return a.lm_head + (size_t)n * dm.d;
  }
}

// Row n of the river copy of op: nibbles, scales and (zero-point format, else null) zero points.
RIVER_DEV void w4_row(int op, int n, const LayerDev& lw, const Dims& dm, const uint8_t*& rp,
                      const f16*& sp, const uint8_t*& zp) {
  const int K = op_k(op, dm);
  const int64_t rb = w4_row_bytes(K), rs = w4_row_scales(K, dm.group);
  const uint8_t* base;
  const f16* sbase;
  const uint8_t* zbase;
  switch (op) {
    case OP_QKV: base = lw.r_qkv; sbase = lw.s_qkv; zbase = lw.z_qkv; break;
    case OP_O: base = lw.r_o; sbase = lw.s_o; zbase = lw.z_o; break;
    case OP_GU: base = lw.r_gu; sbase = lw.s_gu; zbase = lw.z_gu; break;
    default: base = lw.r_d; sbase = lw.s_d; zbase = lw.z_d; break;
  }
  rp = base + (size_t)n * rb;
  sp = sbase + (size_t)n * rs;
  zp = zbase ? zbase + (size_t)n * rs : nullptr;
}

// ---------------------------------------------------------------------------------------
// Loads. Pointers reach the kernels through structs in memory, which hides their address
// space from the compiler; the casts make every weight/activation access a global_load
// (vmcnt only), never a flat_load (which LDS waits would also drain).
// ---------------------------------------------------------------------------------------
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) v4u g_v4u;
typedef const __attribute__((address_space(1))) f16 g_f16;
RIVER_DEV uint4 ldg16(const void* p) {
  const v4u v = *(g_v4u*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
RIVER_DEV f16 ldg2(const f16* p) { return *(g_f16*)p; }

typedef __attribute__((address_space(1))) unsigned long long g_u64;
typedef __attribute__((address_space(1))) unsigned short g_u16;
typedef __attribute__((address_space(1))) float g_f32;

// Activation access. COH = true: agent-scope atomic loads/stores (sc1: past this XCD's L2 /
// written through), for data produced by other workgroups inside one persistent launch.
template <bool COH>
RIVER_DEV uint4 ldx16(const void* p) {
  if (!COH) return ldg16(p);
  const unsigned long long lo = __hip_atomic_load((g_u64*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long hi = __hip_atomic_load((g_u64*)p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
}
template <bool COH>
RIVER_DEV f16 ldh(const f16* p) {
  if (!COH) return *(g_f16*)p;
  const unsigned short u = __hip_atomic_load((g_u16*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_bit_cast(f16, u);
}
template <bool COH>
RIVER_DEV void sth(f16* p, f16 v) {
  if (!COH) {
    *p = v;
    return;
  }
  __hip_atomic_store((g_u16*)p, __builtin_bit_cast(unsigned short, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------------------
// Tagged activations (persistent kernel). A value that crosses workgroups inside one launch is
// stored as a 32-bit word: the fp16 value in the low half and a 16-bit use tag in the high
// half. A consumer polls the words it reads until each carries the tag of the use it waits
// for, instead of meeting every other workgroup at a grid barrier. One word is written by
// one 32-bit store, so a word with the expected tag holds that use's value; every use rewrites
// every word of its buffer and consecutive uses of a buffer carry different tags, so a stale
// word never matches. The spin is bounded: a consumer that waits too long raises the abort
// word, after which every wait returns at once (the host reports a device error).
// ---------------------------------------------------------------------------------------
typedef __attribute__((address_space(1))) uint32_t g_u32;
static constexpr unsigned kTagSpinLimit = 1u << 20;

RIVER_DEV void st_tag(uint32_t* p, f16 v, uint32_t tag) {
  __hip_atomic_store((g_u32*)p, (tag << 16) | (uint32_t)__builtin_bit_cast(unsigned short, v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Bounded spin step: true when the wait must end (abort raised here or elsewhere).
RIVER_DEV bool tag_spin(unsigned& spins, int* abort) {
  ++spins;
  if ((spins & 255u) == 0) {
    if (__hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return true;
    if (spins > kTagSpinLimit) {
      __hip_atomic_store(abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return true;
    }
  }
  __builtin_amdgcn_s_sleep(1);
  return false;
}

// N groups of 8 tagged words at once (use[i] false: group i is not read and reads as 0): every
// group's loads are issued before any is checked, and only the groups not yet ready are
// reloaded, so a wait costs one round trip however many groups a thread reads.
RIVER_DEV bool tag8_ok(uint4 lo, uint4 hi, uint32_t t2) {
  return (((lo.x >> 16) | (lo.y & 0xFFFF0000u)) == t2) & (((lo.z >> 16) | (lo.w & 0xFFFF0000u)) == t2) &
         (((hi.x >> 16) | (hi.y & 0xFFFF0000u)) == t2) & (((hi.z >> 16) | (hi.w & 0xFFFF0000u)) == t2);
}
template <int N>
RIVER_DEV void ld_tag8n(const uint32_t* const (&p)[N], const bool (&use)[N], const uint32_t (&tag)[N],
                        int* abort, uint4 (&out)[N]) {
  uint4 lo[N], hi[N];
  bool ok[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    lo[i] = hi[i] = make_uint4(0, 0, 0, 0);
    if (use[i]) {
      lo[i] = ldx16<true>(p[i]);
      hi[i] = ldx16<true>(p[i] + 4);
    }
  }
  unsigned spins = 0;
  while (true) {
    bool all = true;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      ok[i] = !use[i] || tag8_ok(lo[i], hi[i], tag[i] | (tag[i] << 16));
      all &= ok[i];
    }
    if (all || tag_spin(spins, abort)) break;
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (!ok[i]) {
        lo[i] = ldx16<true>(p[i]);
        hi[i] = ldx16<true>(p[i] + 4);
      }
  }
#pragma unroll
  for (int i = 0; i < N; ++i)
    out[i] = use[i] ? make_uint4((lo[i].x & 0xFFFFu) | (lo[i].y << 16), (lo[i].z & 0xFFFFu) | (lo[i].w << 16),
                                 (hi[i].x & 0xFFFFu) | (hi[i].y << 16), (hi[i].z & 0xFFFFu) | (hi[i].w << 16))
                    : make_uint4(0, 0, 0, 0);
}
// Same, one tag for all groups.
template <int N>
RIVER_DEV void ld_tag8n(const uint32_t* const (&p)[N], const bool (&use)[N], uint32_t tag, int* abort,
                        uint4 (&out)[N]) {
  uint32_t tg[N];
#pragma unroll
  for (int i = 0; i < N; ++i) tg[i] = tag;
  ld_tag8n<N>(p, use, tg, abort, out);
}
RIVER_DEV f16 ld_tag1(const uint32_t* p, uint32_t tag, int* abort) {
  uint32_t w;
  unsigned spins = 0;
  while (true) {
    w = __hip_atomic_load((g_u32*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((w >> 16) == tag || tag_spin(spins, abort)) break;
  }
  return __builtin_bit_cast(f16, (unsigned short)(w & 0xFFFFu));
}

RIVER_DEV double sq8(uint4 u) {
  const f16* h = (const f16*)&u;
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double x = (double)h2f(h[i]);
    s += x * x;
  }
  return s;
}

// fp16(v * inv * gain) on 8 values (fp32 products), or v unchanged without a gain
RIVER_DEV uint4 norm8(uint4 u, uint4 g, float inv, bool has_gain) {
  if (!has_gain) return u;
  uint32_t* pu = (uint32_t*)&u;
  const uint32_t* pg = (const uint32_t*)&g;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const h2 v = as_h2(pu[j]), gg = as_h2(pg[j]);
    h2 r;
    r.x = f2h(h2f(v.x) * inv * h2f(gg.x));
    r.y = f2h(h2f(v.y) * inv * h2f(gg.y));
    pu[j] = as_u32(r);
  }
  return u;
}

// Exit-test reduction: dot(u, v), |u|^2, |v|^2 of two d-vectors in fp64, lane j taking 16-byte
// chunks j, j+64, ... and a fixed xor tree, so every wave that runs it gets identical bits.
template <bool COH>
RIVER_DEV void wave_cos3(const f16* u, const f16* v, int d, double& dot, double& nu, double& nv) {
  const int lane = threadIdx.x & (kWave - 1);
  double s0 = 0.0, s1 = 0.0, s2 = 0.0;
  for (int base = 0; base < d; base += 4 * kChunkF16) {
    uint4 ua[4], va[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = base + k * kChunkF16 + lane * 8;
      const int ee = e < d ? e : 0;
      ua[k] = ldx16<COH>(u + ee);
      va[k] = ldx16<COH>(v + ee);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (base + k * kChunkF16 + lane * 8 >= d) continue;
      const f16* hu = (const f16*)&ua[k];
      const f16* hv = (const f16*)&va[k];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double x = (double)h2f(hu[i]), y = (double)h2f(hv[i]);
        s0 += x * y;
        s1 += x * x;
        s2 += y * y;
      }
    }
  }
  dot = wave_sum_d(s0);
  nu = wave_sum_d(s1);
  nv = wave_sum_d(s2);
}

template <int NCH, int RB>
RIVER_DEV void dot_rows_f16(const uint4 (&w)[RB][NCH], const h2 (&x)[NCH][4], float (&acc)[RB]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      s = dot2(x[c][0], as_h2(w[rb][c].x), s);
      s = dot2(x[c][1], as_h2(w[rb][c].y), s);
      s = dot2(x[c][2], as_h2(w[rb][c].z), s);
      s = dot2(x[c][3], as_h2(w[rb][c].w), s);
    }
    acc[rb] = s;
  }
}

// int4 rows: per chunk sum_k q_k x_k over the lane's 32 elements (one group), times its scale.
// unpack8 gives q = u - 8; the zero-point format needs u - z = (u - 8) + (8 - z), so with `zp` the
// lane's input sum X is added (8 - z) times per chunk.
template <int NCH, int RB>
RIVER_DEV void dot_rows_w4(const uint4 (&w)[RB][NCH], const f16 (&sc)[RB][NCH],
                           const uint8_t (&zz)[RB][NCH], bool zp, const h2 (&x)[NCH][16],
                           float (&acc)[RB]) {
  float xsum[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    xsum[c] = 0.f;
    if (zp)
#pragma unroll
      for (int j = 0; j < 16; ++j) xsum[c] += h2f(x[c][j].x) + h2f(x[c][j].y);
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float tot = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint32_t ww[4] = {w[rb][c].x, w[rb][c].y, w[rb][c].z, w[rb][c].w};
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        h2 p0, p1, p2, p3;
        unpack8(ww[m], p0, p1, p2, p3);
        s = dot2(p0, x[c][m * 4 + 0], s);
        s = dot2(p1, x[c][m * 4 + 1], s);
        s = dot2(p2, x[c][m * 4 + 2], s);
        s = dot2(p3, x[c][m * 4 + 3], s);
      }
      if (zp) s = fmaf(8.f - (float)zz[rb][c], xsum[c], s);
      tot = fmaf(h2f(sc[rb][c]), s, tot);
    }
    acc[rb] = tot;
  }
}

// Block-wide fp64 sum of squares in one fixed order (thread t takes elements t, t+256, ...).
RIVER_DEV double block_sumsq(const f16* v, int n, double* red) {
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += kBlock) {
    const double x = (double)h2f(v[i]);
    s += x * x;
  }
  return block_sum_d(s, red);
}

RIVER_DEV float inv_rms(double ss, int n, float eps) {
  return (float)(1.0 / sqrt(ss / n + (double)eps));
}

// Sum of per-wave values over the WPR waves of this wave's row group (fixed order). WPR = 1
// needs no exchange.
template <int WPR>
RIVER_DEV double rowgroup_sum(double v, double* red) {
  if (WPR == 1) return v;
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  const int g0 = (w / WPR) * WPR;
  double s = 0.0;
  for (int j = 0; j < WPR; ++j) s += red[g0 + j];
  return s;
}

// One wave's share of a tile on the fp16 stream: RB rows x NCH chunks of 512 elements
// (chunk ids ws, ws+WPR, ...). Loads weights, the raw input and its gains, normalises the
// input (computing its rms from the loaded values when `want_norm`), returns the RB dots.
template <int NCH, int RB, int WPR, bool HAS_GAIN, bool COH>
RIVER_DEV void wave_gemv_f16(const f16* const (&rowp)[RB], const f16* xv, const f16* gain, int K,
                             int ws, bool want_norm, float inv, int dnorm, float eps, double* red,
                             float (&acc)[RB]) {
  const int lane = threadIdx.x & (kWave - 1);
  uint4 wv[RB][NCH];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e = (ws + c * WPR) * kChunkF16 + lane * 8;
      const bool ok = rowp[rb] != nullptr && e < K;
      // out-of-range chunks read a valid vector instead and meet x = 0; rows past N are
      // never stored
      wv[rb][c] = ldg16(ok ? (const void*)(rowp[rb] + e) : (const void*)xv);
    }
  uint4 xr[NCH], gr[NCH] = {};
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int e = (ws + c * WPR) * kChunkF16 + lane * 8;
    const int ee = e < K ? e : 0;
    xr[c] = ldx16<COH>(xv + ee);
    if (HAS_GAIN) gr[c] = ldg16(gain + ee);
  }
  if (want_norm) {
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if ((ws + c * WPR) * kChunkF16 + lane * 8 < K) ss += sq8(xr[c]);
    ss = rowgroup_sum<WPR>(wave_sum_d(ss), red);
    inv = inv_rms(ss, dnorm, eps);
  }
  h2 x[NCH][4];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const bool okx = (ws + c * WPR) * kChunkF16 + lane * 8 < K;
    const uint4 u = okx ? norm8(xr[c], gr[c], inv, HAS_GAIN) : make_uint4(0, 0, 0, 0);
    x[c][0] = as_h2(u.x);
    x[c][1] = as_h2(u.y);
    x[c][2] = as_h2(u.z);
    x[c][3] = as_h2(u.w);
  }
  dot_rows_f16<NCH, RB>(wv, x, acc);
}

// One wave's share of a tile on the int4 stream: RB rows x NCH chunks of 2048 elements.
template <int NCH, int RB, int WPR, bool HAS_GAIN, bool COH>
RIVER_DEV void wave_gemv_w4(const uint8_t* const (&rowp)[RB], const f16* const (&sclp)[RB],
                            const uint8_t* const (&zrp)[RB], bool zp, const f16* xv,
                            const f16* gain, int K, int group, int ws, bool want_norm, float inv,
                            int dnorm, float eps, double* red, float (&acc)[RB]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nch = (K + kChunkW4 - 1) / kChunkW4;
  uint4 wv[RB][NCH];
  f16 sc[RB][NCH];
  uint8_t zz[RB][NCH];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int cid = ws + c * WPR;
      const bool ok = rowp[rb] != nullptr && cid < nch;
      wv[rb][c] = ldg16(ok ? (const void*)(rowp[rb] + (size_t)cid * 1024 + lane * 16) : (const void*)xv);
      sc[rb][c] = ldg2(ok ? sclp[rb] + (cid * kChunkW4 + lane * 32) / group : xv);
      zz[rb][c] = (zp && ok) ? zrp[rb][(cid * kChunkW4 + lane * 32) / group] : (uint8_t)8;
    }
  uint4 xr[NCH][4], gr[NCH][4] = {};
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = (ws + c * WPR) * kChunkW4 + lane * 32 + m * 8;
      const int ee = e < K ? e : 0;
      xr[c][m] = ldx16<COH>(xv + ee);
      if (HAS_GAIN) gr[c][m] = ldg16(gain + ee);
    }
  if (want_norm) {
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if ((ws + c * WPR) * kChunkW4 + lane * 32 + m * 8 < K) ss += sq8(xr[c][m]);
    ss = rowgroup_sum<WPR>(wave_sum_d(ss), red);
    inv = inv_rms(ss, dnorm, eps);
  }
  h2 x[NCH][16];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const bool okx = (ws + c * WPR) * kChunkW4 + lane * 32 + m * 8 < K;
      const uint4 u = okx ? norm8(xr[c][m], gr[c][m], inv, HAS_GAIN) : make_uint4(0, 0, 0, 0);
      const uint32_t in[4] = {u.x, u.y, u.z, u.w};
      h2 o[4];
      pair_for_unpack(in, o);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[c][m * 4 + j] = o[j];
    }
  dot_rows_w4<NCH, RB>(wv, sc, zz, zp, x, acc);
}


// ---------------------------------------------------------------------------------------
// One GEMV tile plus the op's epilogue
// ---------------------------------------------------------------------------------------

// Per-tile inputs that do not depend on the tile.
struct TileIn {
  int layer, step, pos, b;
  const f16* xv;     // input vector (normalised on the fly when the op has a gain)
  const f16* gain;
  bool want_norm;    // compute 1/rms of xv from the loaded values
  float inv;         // 1/rms when !want_norm
  unsigned long long* key;  // LM head argmax key of this row
};

struct GemvSmem {
  float ypart[16][4];
  float y[16];
  double dred[4];
};

// GEMV of TR rows on the fp16 (is4 = false) or int4 stream, then the op's epilogue:
//   QKV: RoPE on q/k pairs, q -> a.q, k/v -> shared cache slot at in.pos
//   O: h_mid = h(l-1) + fp16(y);  GU: a2 = fp16(silu(fp16 g) * fp16 u);  DOWN: h(l) = h_mid + fp16(y)
//   LM: logits (optional) and a 64-bit atomic max of (value, lowest index) into *in.key.
template <int OP, bool COH, int NCH16, int WPR16, int NCH4, int WPR4>
RIVER_DEV void gemv_tile(const DecodeArgs& a, const LayerDev* lwp, const TileIn& in, int tile,
                         bool is4, GemvSmem& sm) {
  using T16 = TileF16<WPR16>;
  using T4 = TileW4<WPR4>;
  constexpr bool kHasGain = (OP == OP_QKV || OP == OP_GU || OP == OP_LM);
  const Dims& dm = a.dm;
  const int b = in.b, layer = in.layer;
  const int t = threadIdx.x;
  const int TR = is4 ? T4::TR : T16::TR;
  const int N = op_rows(OP, dm);
  const int K = op_k(OP, dm);
  const int w = t / kWave, lane = t % kWave;

  if (!is4) {
    constexpr int RB = kRB16;
    const int rg = w / WPR16, ws = w % WPR16;
    const f16* rowp[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int n = logical_row(OP, tile, rg * RB + rb, T16::TR, dm);
      rowp[rb] = (n < N) ? (OP == OP_LM ? a.lm_head + (size_t)n * dm.d : f16_row(OP, n, *lwp, a))
                         : nullptr;
    }
    float acc[RB];
    wave_gemv_f16<NCH16, RB, WPR16, kHasGain, COH>(rowp, in.xv, in.gain, K, ws, in.want_norm,
                                                   in.inv, dm.d, dm.eps, sm.dred, acc);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float v = wave_sum(acc[rb]);
      if (lane == 0) sm.ypart[rg * RB + rb][ws] = v;
    }
    __syncthreads();
    if (t < T16::TR) {
      float s = 0.f;
      for (int j = 0; j < WPR16; ++j) s += sm.ypart[t][j];
      sm.y[t] = s;
    }
  } else {
    constexpr int RB = kRB4;
    const int rg = w / WPR4, ws = w % WPR4;
    const uint8_t* rowp[RB];
    const f16* sclp[RB];
    const uint8_t* zrp[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int n = logical_row(OP, tile, rg * RB + rb, T4::TR, dm);
      if (n < N) {
        w4_row(OP, n, *lwp, dm, rowp[rb], sclp[rb], zrp[rb]);
      } else {
        rowp[rb] = nullptr;
        sclp[rb] = nullptr;
        zrp[rb] = nullptr;
      }
    }
    float acc[RB];
    wave_gemv_w4<NCH4, RB, WPR4, kHasGain, COH>(rowp, sclp, zrp, dm.zp != 0, in.xv, in.gain, K, dm.group,
                                                ws, in.want_norm, in.inv, dm.d, dm.eps, sm.dred, acc);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float v = wave_sum(acc[rb]);
      if (lane == 0) sm.ypart[rg * RB + rb][ws] = v;
    }
    __syncthreads();
    if (t < T4::TR) {
      float s = 0.f;
      for (int j = 0; j < WPR4; ++j) s += sm.ypart[t][j];
      sm.y[t] = s;
    }
  }
  __syncthreads();
  const float* y = sm.y;

  if (OP == OP_QKV) {
    const int pos = in.pos;
    const int qk_rows = (dm.H + dm.Hkv) * dm.D;
    const int n0 = logical_row(OP, tile, 0, TR, dm);
    if (n0 < qk_rows) {
      const int half = TR / 2;
      if (t < half) {
        const int n = logical_row(OP, tile, t, TR, dm);
        const int head = n / dm.D, i = n % dm.D;  // i < D/2
        const float x0 = h2f(f2h(y[t])), x1 = h2f(f2h(y[t + half]));
        const float2 cs = a.rope[(size_t)pos * (dm.D / 2) + i];
        const f16 r0 = f2h(x0 * cs.x - x1 * cs.y);
        const f16 r1 = f2h(x1 * cs.x + x0 * cs.y);
        f16* dst;
        if (head < dm.H) {
          dst = a.q + (size_t)b * dm.hd + head * dm.D;
        } else {
          const int kvh = head - dm.H;
          dst = a.kv + ((((size_t)(layer - 1) * 2 + 0) * dm.B + b) * dm.Hkv + kvh) *
                           (size_t)dm.Tmax * dm.D + (size_t)pos * dm.D;
        }
        sth<COH>(dst + i, r0);
        sth<COH>(dst + i + dm.D / 2, r1);
        if (head >= dm.H) {
          kv_count(a.kvcnt, a.kv, dst + i, 1);
          kv_count(a.kvcnt, a.kv, dst + i + dm.D / 2, 1);
        }
      }
    } else if (t < TR) {
      const int n = logical_row(OP, tile, t, TR, dm);
      if (n < N) {
        const int vi = n - qk_rows;
        const int kvh = vi / dm.D, i = vi % dm.D;
        f16* vd = a.kv + ((((size_t)(layer - 1) * 2 + 1) * dm.B + b) * dm.Hkv + kvh) *
                             (size_t)dm.Tmax * dm.D + (size_t)pos * dm.D;
        sth<COH>(vd + i, f2h(y[t]));
        kv_count(a.kvcnt, a.kv, vd + i, 1);
      }
    }
  } else if (OP == OP_GU) {
    const int half = TR / 2;
    if (t < half) {
      const int f = logical_row(OP, tile, t, TR, dm);
      if (f < dm.F) {
        const float g = h2f(f2h(y[t])), u = h2f(f2h(y[t + half]));
        const float sg = g / (1.f + __expf(-g));
        sth<COH>(a.a2 + (size_t)b * dm.F + f, f2h(sg * u));
      }
    }
  } else if (OP == OP_O) {
    if (t < TR) {
      const int n = tile * TR + t;
      if (n < N) {
        const size_t i = ((size_t)(layer - 1) * dm.B + b) * dm.d + n;
        sth<COH>(a.hmid + i, f2h(h2f(ldh<COH>(a.hs + i)) + h2f(f2h(y[t]))));
      }
    }
  } else if (OP == OP_DOWN) {
    if (t < TR) {
      const int n = tile * TR + t;
      if (n < N) {
        const size_t i = ((size_t)(layer - 1) * dm.B + b) * dm.d + n;
        sth<COH>(a.hs + (size_t)dm.B * dm.d + i, f2h(h2f(ldh<COH>(a.hmid + i)) + h2f(f2h(y[t]))));
      }
    }
  } else {  // OP_LM
    if (t == 0) {
      float best = -__builtin_inff();
      int bi = 0x7FFFFFFF;
      for (int r = 0; r < TR; ++r) {
        const int n = tile * TR + r;
        if (n >= N) break;
        const float v = y[r];
        if (a.logits) a.logits[(size_t)b * dm.V + n] = v;
        if (v > best) {
          best = v;
          bi = n;
        }
      }
      const unsigned long long key = ((unsigned long long)float_key(best) << 32) |
                                     (unsigned long long)(0xFFFFFFFFu - (uint32_t)bi);
      __hip_atomic_fetch_max(in.key, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();  // LDS reuse by the next tile
}
