// Decode-step kernels for one early-exit token per row (batch 1 on the VALU path).
//
// Per layer l the step runs five kernels:
//   QKV   RMSNorm(h(l-1)) -> QKV GEMV (backbone fp16 or river int4) -> RoPE -> KV append
//   ATTN  GQA flash-decode over the shared cache, split over positions, last-arriver merge
//   O     O GEMV + residual -> h_mid; last arriver: 1/rms(h_mid)
//   GU    RMSNorm(h_mid) -> gate|up GEMV -> SwiGLU
//   DOWN  down GEMV + residual -> h(l); last arriver: cos(h(l-1), h(l)), exit test, route of
//         layer l+1, 1/rms(h(l))
// and after layer L one LM-head kernel (final RMSNorm, fp16 LM head, greedy argmax).
//
// Method (River-LLM, Shen & Zou): the exit layer of block l is its W4A16 copy (aitrends.kr
// article, construction paragraph); both copies write the same KV slot (paperlayer.ai
// summary of arXiv 2604.18396v3, section 4 "KV-Shared Exit Layer"); the exit test compares
// the cosine of a block's input and output with tau (aitrends, exit-criterion paragraph;
// paperlayer section 4 "Error-Aware Exit Decisions"); after an exit the remaining blocks run
// on the river and the original LM head gives the token (paperlayer section 4 "Inference with
// Seamless Exit").
//
// GEMV launch layout: one grid holds both weight streams of a matrix. Workgroups
// [0, nwg16) are backbone tiles (fp16 rows), [nwg16, nwg16 + nwg4) river tiles (int4 rows).
// Each workgroup reads the row's route from device memory and returns at once if its stream
// is not the one this layer runs, so the path is chosen on the device with no host round trip
// and the launch sequence of a step never changes (graph-capturable).
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

RIVER_DEV void w4_row(int op, int n, const LayerDev& lw, const Dims& dm, const uint8_t*& rp,
                      const f16*& sp) {
  const int K = op_k(op, dm);
  const int64_t rb = w4_row_bytes(K), rs = w4_row_scales(K, dm.group);
  const uint8_t* base;
  const f16* sbase;
  switch (op) {
    case OP_QKV: base = lw.r_qkv; sbase = lw.s_qkv; break;
    case OP_O: base = lw.r_o; sbase = lw.s_o; break;
    case OP_GU: base = lw.r_gu; sbase = lw.s_gu; break;
    default: base = lw.r_d; sbase = lw.s_d; break;
  }
  rp = base + (size_t)n * rb;
  sp = sbase + (size_t)n * rs;
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
RIVER_DEV void wave_cos3(const f16* u, const f16* v, int d, double& dot, double& nu, double& nv) {
  const int lane = threadIdx.x & (kWave - 1);
  double s0 = 0.0, s1 = 0.0, s2 = 0.0;
  for (int base = 0; base < d; base += 4 * kChunkF16) {
    uint4 ua[4], va[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = base + k * kChunkF16 + lane * 8;
      const int ee = e < d ? e : 0;
      ua[k] = ldg16(u + ee);
      va[k] = ldg16(v + ee);
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

// int4 rows: per chunk sum_k q_k x_k over the lane's 32 elements (one group), times its scale
template <int NCH, int RB>
RIVER_DEV void dot_rows_w4(const uint4 (&w)[RB][NCH], const f16 (&sc)[RB][NCH],
                           const h2 (&x)[NCH][16], float (&acc)[RB]) {
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
template <int NCH, int RB, int WPR, bool HAS_GAIN>
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
    xr[c] = ldg16(xv + ee);
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
template <int NCH, int RB, int WPR, bool HAS_GAIN>
RIVER_DEV void wave_gemv_w4(const uint8_t* const (&rowp)[RB], const f16* const (&sclp)[RB],
                            const f16* xv, const f16* gain, int K, int group, int ws,
                            bool want_norm, float inv, int dnorm, float eps, double* red,
                            float (&acc)[RB]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nch = (K + kChunkW4 - 1) / kChunkW4;
  uint4 wv[RB][NCH];
  f16 sc[RB][NCH];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int cid = ws + c * WPR;
      const bool ok = rowp[rb] != nullptr && cid < nch;
      wv[rb][c] = ldg16(ok ? (const void*)(rowp[rb] + (size_t)cid * 1024 + lane * 16) : (const void*)xv);
      sc[rb][c] = ldg2(ok ? sclp[rb] + (cid * kChunkW4 + lane * 32) / group : xv);
    }
  uint4 xr[NCH][4], gr[NCH][4] = {};
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = (ws + c * WPR) * kChunkW4 + lane * 32 + m * 8;
      const int ee = e < K ? e : 0;
      xr[c][m] = ldg16(xv + ee);
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
  dot_rows_w4<NCH, RB>(wv, sc, x, acc);
}

// MODE 0: early-exit decode (both weight streams in the grid; the route of the layer is decided
//         by every QKV workgroup identically and read from device state by the later kernels).
// MODE 1: backbone-only decode (the full-depth fp16 model: no river tiles, no exit test).
template <int OP, int MODE, int NCH16, int WPR16, int NCH4, int WPR4>
__global__ __launch_bounds__(kBlock) void k_dec_gemv(DecodeArgs a, int layer, int nwg16, int nwg4) {
  using T16 = TileF16<WPR16>;
  using T4 = TileW4<WPR4>;
  constexpr int TRMAX = (T16::TR > T4::TR ? T16::TR : T4::TR);
  constexpr bool kHasGain = (OP == OP_QKV || OP == OP_GU || OP == OP_LM);
  __shared__ float ypart[TRMAX][4];
  __shared__ float y[TRMAX];
  __shared__ double dred[4];
  __shared__ double cos3[3];

  const Dims& dm = a.dm;
  const int b = 0;  // batch row (the VALU path decodes one row)
  const bool is4 = blockIdx.x >= (unsigned)nwg16;
  const int step = *a.step;
  const LayerDev* lwp = (OP == OP_LM) ? nullptr : &a.layers[layer - 1];
  const int t = threadIdx.x;

  // ---- route of this layer ------------------------------------------------------------
  int route = ROUTE_BACKBONE;
  bool have_inv = false;
  float inv = 1.f;
  const f16* vin = nullptr;
  if (OP == OP_QKV) {
    if (layer == 1) {
      int tok = (step == 0) ? a.tok_in[b] : a.tok_out[(step - 1) * dm.B + b];
      if (tok < 0 || tok >= dm.V) {
        if (blockIdx.x == 0 && t == 0) atomicOr(a.err, ERR_TOKEN);
        tok = 0;
      }
      vin = a.embed + (size_t)tok * dm.d;
      if (blockIdx.x == 0) {
        f16* h0 = a.hs + (size_t)b * dm.d;
        for (int i = t; i < dm.d; i += kBlock) h0[i] = vin[i];
        if (t == 0 && a.exit_out) a.exit_out[step * dm.B + b] = dm.L;
        if (a.sim_out)
          for (int i = t; i < dm.L; i += kBlock)
            a.sim_out[((size_t)step * dm.B + b) * dm.L + i] = __builtin_nanf("");
      }
    } else {
      vin = a.hs + ((size_t)(layer - 1) * dm.B + b) * dm.d;
      if (MODE == 0) {
        // exit test after backbone layer lp = layer-1: cos(h(lp-1), h(lp)) > tau (or forced)
        const int lp = layer - 1;
        const int prev = a.route[lp * dm.B + b];
        if (prev == ROUTE_RIVER) {
          route = ROUTE_RIVER;
        } else if (lp >= dm.entry) {
          if (a.sched) {
            int e = a.sched[step * dm.B + b];
            if (e < dm.entry || e > dm.L) {
              if (blockIdx.x == 0 && t == 0) atomicOr(a.err, ERR_FORCED);
              e = dm.L;
            }
            if (lp == e) route = ROUTE_RIVER;
          } else {
            if (t < kWave) {
              double dot, n1, n2;
              wave_cos3(a.hs + ((size_t)(lp - 1) * dm.B + b) * dm.d, vin, dm.d, dot, n1, n2);
              if (t == 0) {
                cos3[0] = dot;
                cos3[1] = n1;
                cos3[2] = n2;
              }
            }
            __syncthreads();
            const double dot = cos3[0], n1 = cos3[1], n2 = cos3[2];
            const double sim = (n1 > 0.0 && n2 > 0.0) ? dot / sqrt(n1 * n2) : 0.0;
            if (blockIdx.x == 0 && t == 0 && a.sim_out)
              a.sim_out[((size_t)step * dm.B + b) * dm.L + lp - 1] = (float)sim;
            if (sim > (double)a.tau) route = ROUTE_RIVER;
            inv = inv_rms(n2, dm.d, dm.eps);
            have_inv = true;
          }
        }
        if (blockIdx.x == 0 && t == 0) {
          a.route[layer * dm.B + b] = route;
          if (route == ROUTE_RIVER && prev == ROUTE_BACKBONE && a.exit_out)
            a.exit_out[step * dm.B + b] = lp;
        }
      }
    }
  } else if (OP != OP_LM && MODE == 0) {
    route = a.route[layer * dm.B + b];
  }
  if (is4 != (route == ROUTE_RIVER)) return;

  const int tile = is4 ? (int)blockIdx.x - nwg16 : (int)blockIdx.x;
  const int TR = is4 ? T4::TR : T16::TR;
  const int N = op_rows(OP, dm);
  const int K = op_k(OP, dm);
  const int w = t / kWave, lane = t % kWave;

  // input vector: x = fp16(v * inv * gain), or v itself
  const f16* xv;
  const f16* gain = nullptr;
  bool want_norm = false;
  if (OP == OP_QKV) {
    xv = vin;
    gain = lwp->attn_norm;
    want_norm = !have_inv;
  } else if (OP == OP_O) {
    xv = a.o + (size_t)b * dm.hd;
  } else if (OP == OP_GU) {
    xv = a.hmid + ((size_t)(layer - 1) * dm.B + b) * dm.d;
    gain = lwp->mlp_norm;
    want_norm = true;
  } else if (OP == OP_DOWN) {
    xv = a.a2 + (size_t)b * dm.F;
  } else {
    xv = a.hs + ((size_t)dm.L * dm.B + b) * dm.d;
    gain = a.final_norm;
    inv = a.inv_attn[dm.L * dm.B + b];
  }

  // ---- GEMV ---------------------------------------------------------------------------
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
    wave_gemv_f16<NCH16, RB, WPR16, kHasGain>(rowp, xv, gain, K, ws, want_norm, inv, dm.d, dm.eps, dred, acc);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float v = wave_sum(acc[rb]);
      if (lane == 0) ypart[rg * RB + rb][ws] = v;
    }
    __syncthreads();
    if (t < T16::TR) {
      float s = 0.f;
      for (int j = 0; j < WPR16; ++j) s += ypart[t][j];
      y[t] = s;
    }
  } else {
    constexpr int RB = kRB4;
    const int rg = w / WPR4, ws = w % WPR4;
    const uint8_t* rowp[RB];
    const f16* sclp[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int n = logical_row(OP, tile, rg * RB + rb, T4::TR, dm);
      if (n < N) {
        w4_row(OP, n, *lwp, dm, rowp[rb], sclp[rb]);
      } else {
        rowp[rb] = nullptr;
        sclp[rb] = nullptr;
      }
    }
    float acc[RB];
    wave_gemv_w4<NCH4, RB, WPR4, kHasGain>(rowp, sclp, xv, gain, K, dm.group, ws, want_norm, inv, dm.d,
                                 dm.eps, dred, acc);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float v = wave_sum(acc[rb]);
      if (lane == 0) ypart[rg * RB + rb][ws] = v;
    }
    __syncthreads();
    if (t < T4::TR) {
      float s = 0.f;
      for (int j = 0; j < WPR4; ++j) s += ypart[t][j];
      y[t] = s;
    }
  }
  __syncthreads();

  // ---- epilogues ----------------------------------------------------------------------
  if (OP == OP_QKV) {
    const int pos = a.pos[b];
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
        if (head < dm.H) {
          f16* qd = a.q + (size_t)b * dm.hd + head * dm.D;
          qd[i] = r0;
          qd[i + dm.D / 2] = r1;
        } else {
          const int kvh = head - dm.H;
          f16* kd = a.kv + ((((size_t)(layer - 1) * 2 + 0) * dm.B + b) * dm.Hkv + kvh) *
                               (size_t)dm.Tmax * dm.D + (size_t)pos * dm.D;
          kd[i] = r0;
          kd[i + dm.D / 2] = r1;
        }
      }
    } else if (t < TR) {
      const int n = logical_row(OP, tile, t, TR, dm);
      if (n < N) {
        const int vi = n - qk_rows;
        const int kvh = vi / dm.D, i = vi % dm.D;
        f16* vd = a.kv + ((((size_t)(layer - 1) * 2 + 1) * dm.B + b) * dm.Hkv + kvh) *
                             (size_t)dm.Tmax * dm.D + (size_t)pos * dm.D;
        vd[i] = f2h(y[t]);
      }
    }
  } else if (OP == OP_GU) {
    const int half = TR / 2;
    if (t < half) {
      const int f = logical_row(OP, tile, t, TR, dm);
      if (f < dm.F) {
        const float g = h2f(f2h(y[t])), u = h2f(f2h(y[t + half]));
        const float sg = g / (1.f + __expf(-g));
        a.a2[(size_t)b * dm.F + f] = f2h(sg * u);
      }
    }
  } else if (OP == OP_O) {
    if (t < TR) {
      const int n = tile * TR + t;
      if (n < N) {
        const size_t i = ((size_t)(layer - 1) * dm.B + b) * dm.d + n;
        a.hmid[i] = f2h(h2f(a.hs[i]) + h2f(f2h(y[t])));
      }
    }
  } else if (OP == OP_DOWN) {
    if (t < TR) {
      const int n = tile * TR + t;
      if (n < N) {
        const size_t i = ((size_t)(layer - 1) * dm.B + b) * dm.d + n;
        a.hs[(size_t)dm.B * dm.d + i] = f2h(h2f(a.hmid[i]) + h2f(f2h(y[t])));
      }
    }
  } else {  // OP_LM: logits, workgroup argmax (lowest index on ties), one 64-bit atomic max
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
      __hip_atomic_fetch_max(a.amax + b, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// 1/rms of the final residual stream (input of the LM head), one workgroup per row.
__global__ __launch_bounds__(kBlock) void k_final_norm(DecodeArgs a) {
  __shared__ double red[4];
  const int b = blockIdx.x;
  const double ss = block_sumsq(a.hs + ((size_t)a.dm.L * a.dm.B + b) * a.dm.d, a.dm.d, red);
  if (threadIdx.x == 0) a.inv_attn[a.dm.L * a.dm.B + b] = inv_rms(ss, a.dm.d, a.dm.eps);
}

// End of a step: greedy token from the argmax key, position and step counters advance.
__global__ void k_step_end(DecodeArgs a) {
  const int b = threadIdx.x;
  const int step = *a.step;
  if (b < a.dm.B) {
    const unsigned long long key =
        __hip_atomic_load(a.amax + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.tok_out[step * a.dm.B + b] = (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull));
    __hip_atomic_store(a.amax + b, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.pos[b] += 1;
  }
  __syncthreads();
  if (b == 0) *a.step = step + 1;
}

// ---------------------------------------------------------------------------------------
// GQA flash-decode attention over the shared cache. Grid (smax, Hkv, B). Workgroup s covers
// positions [s*chunk, min(T, (s+1)*chunk)) of one KV head for its G = H/Hkv query heads.
// Each group of D/8 lanes owns one position at a time (16-byte K and V loads per lane) and
// keeps an online-softmax state; groups merge in LDS, splits merge in the last arriver.
// ---------------------------------------------------------------------------------------
static constexpr int kMinChunk = 64;

template <int D, int G>
__global__ __launch_bounds__(kBlock) void k_dec_attn(DecodeArgs a, int layer) {
  constexpr int LPT = D / 8;       // lanes per position
  constexpr int TPW = kWave / LPT;  // positions per wave pass
  constexpr int NGRP = 4 * TPW;     // position groups per workgroup
  constexpr int U = 2;              // positions per group per iteration (loads in flight)
  __shared__ float sm_m[NGRP][G];
  __shared__ float sm_l[NGRP][G];
  __shared__ float sm_acc[NGRP][G][D];
  __shared__ float sm_w[G][64];
  __shared__ float sm_L[G];
  __shared__ int lflag;

  const Dims& dm = a.dm;
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int smax = a.attn_smax;
  const int T = a.pos[b] + 1;
  const int chunk = max(kMinChunk, (T + smax - 1) / smax);
  const int seff = (T + chunk - 1) / chunk;
  const size_t head_stride = (size_t)dm.Tmax * D;
  const f16* Kb = a.kv + ((((size_t)(layer - 1) * 2 + 0) * dm.B + b) * dm.Hkv + kvh) * head_stride;
  const f16* Vb = a.kv + ((((size_t)(layer - 1) * 2 + 1) * dm.B + b) * dm.Hkv + kvh) * head_stride;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int grp = w * TPW + lane / LPT, sub = lane % LPT, d0 = sub * 8;
  const size_t pbase = ((size_t)b * dm.H + (size_t)kvh * G) * smax;  // + g*smax + s

  if (s < seff) {
    const int t0 = s * chunk, t1 = min(T, t0 + chunk);
    const float qs = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(D)
    float qf[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 u = ldg16(a.q + (size_t)b * dm.hd + (size_t)(kvh * G + g) * D + d0);
      const f16* hp = (const f16*)&u;
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[g][i] = h2f(hp[i]) * qs;
    }
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -__builtin_inff();
      l[g] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
    }
    for (int tb = t0 + grp; tb < t1; tb += NGRP * U) {
      uint4 kk[U], vv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = tb + u * NGRP;
        const size_t tt = (size_t)(t < t1 ? t : t0);
        kk[u] = ldg16(Kb + tt * D + d0);
        vv[u] = ldg16(Vb + tt * D + d0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = tb + u * NGRP;
        if (t >= t1) break;  // uniform within the lane group
        const f16* kh = (const f16*)&kk[u];
        const f16* vh = (const f16*)&vv[u];
        float kf[8], vf[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          kf[i] = h2f(kh[i]);
          vf[i] = h2f(vh[i]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float sc = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) sc = fmaf(qf[g][i], kf[i], sc);
#pragma unroll
          for (int o = 1; o < LPT; o <<= 1) sc += __shfl_xor(sc, o, kWave);
          const float mn = fmaxf(m[g], sc);
          const float c = exp2f(m[g] - mn);
          const float p = exp2f(sc - mn);
          l[g] = l[g] * c + p;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[g][i] = fmaf(acc[g][i], c, p * vf[i]);
          m[g] = mn;
        }
      }
    }
    // merge the NGRP groups of this workgroup
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (sub == 0) {
        sm_m[grp][g] = m[g];
        sm_l[grp][g] = l[g];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) sm_acc[grp][g][d0 + i] = acc[g][i];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += kBlock) {
      const int g = idx / D, dd = idx % D;
      float M = -__builtin_inff();
      for (int j = 0; j < NGRP; ++j) M = fmaxf(M, sm_m[j][g]);
      float Lsum = 0.f, A = 0.f;
      for (int j = 0; j < NGRP; ++j) {
        const float sc = (sm_l[j][g] > 0.f) ? exp2f(sm_m[j][g] - M) : 0.f;
        Lsum += sm_l[j][g] * sc;
        A += sm_acc[j][g][dd] * sc;
      }
      const size_t pi = pbase + (size_t)g * smax + s;
      wt_store(&a.pacc[pi * D + dd], A);
      if (dd == 0) {
        wt_store(&a.pml[pi * 2 + 0], M);
        wt_store(&a.pml[pi * 2 + 1], Lsum);
      }
    }
  }

  int* counter = a.cnt + CNT_ATTN + b * dm.Hkv + kvh;
  if (arrive_counter(counter, smax, &lflag)) {
    // split weights exp2(m_s - M) / L per query head
    if (threadIdx.x < G) {
      const int g = threadIdx.x;
      float M = -__builtin_inff();
      for (int j = 0; j < seff; ++j) {
        sm_w[g][j] = wt_load(&a.pml[(pbase + (size_t)g * smax + j) * 2]);
        M = fmaxf(M, sm_w[g][j]);
      }
      float Lsum = 0.f;
      for (int j = 0; j < seff; ++j) {
        const float e = exp2f(sm_w[g][j] - M);
        sm_w[g][j] = e;
        Lsum += wt_load(&a.pml[(pbase + (size_t)g * smax + j) * 2 + 1]) * e;
      }
      sm_L[g] = Lsum;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += kBlock) {
      const int g = idx / D, dd = idx % D;
      float A = 0.f;
      for (int j = 0; j < seff; ++j) A += sm_w[g][j] * wt_load(&a.pacc[(pbase + (size_t)g * smax + j) * D + dd]);
      a.o[(size_t)b * dm.hd + (size_t)(kvh * G + g) * D + dd] = f2h(A / sm_L[g]);
    }
    if (threadIdx.x == 0) reset_counter(counter);
  }
}

// ---------------------------------------------------------------------------------------
// Host-side launchers (called from api.cpp)
// ---------------------------------------------------------------------------------------
template <int OP, int MODE, int NCH16, int WPR16, int NCH4, int WPR4>
static hipError_t launch_gemv_t(const DecodeArgs& a, int layer, int N, hipStream_t st) {
  const int tr16 = TileF16<WPR16>::TR, tr4 = TileW4<WPR4>::TR;
  int nwg16, nwg4;
  if (OP == OP_GU) {
    nwg16 = (N / 2) / (tr16 / 2);
    nwg4 = (N / 2) / (tr4 / 2);
  } else if (OP == OP_QKV) {
    nwg16 = N / tr16;
    nwg4 = N / tr4;
  } else {
    nwg16 = (N + tr16 - 1) / tr16;
    nwg4 = (N + tr4 - 1) / tr4;
  }
  if (OP == OP_LM || MODE == 1) nwg4 = 0;
  hipLaunchKernelGGL((k_dec_gemv<OP, MODE, NCH16, WPR16, NCH4, WPR4>), dim3(nwg16 + nwg4),
                     dim3(kBlock), 0, st, a, layer, nwg16, nwg4);
  return hipGetLastError();
}

// Picks the stream geometry from K: chunks per row (fp16: 512 elements, int4: 2048), waves per
// row WPR and chunks per wave NCH (fp16 <= 8, int4 <= 4).
template <int OP, int MODE>
static hipError_t launch_op(const DecodeArgs& a, int layer, hipStream_t st) {
  const Dims& dm = a.dm;
  const int N = (OP == OP_QKV) ? dm.nqkv : (OP == OP_GU) ? 2 * dm.F : (OP == OP_LM) ? dm.V : dm.d;
  const int K = (OP == OP_O) ? dm.hd : (OP == OP_DOWN) ? dm.F : dm.d;
  const int n16 = (K + kChunkF16 - 1) / kChunkF16;
  const int n4 = (K + kChunkW4 - 1) / kChunkW4;
  if (n16 <= 1 && n4 <= 1) return launch_gemv_t<OP, MODE, 1, 1, 1, 1>(a, layer, N, st);
  if (n16 <= 2 && n4 <= 1) return launch_gemv_t<OP, MODE, 2, 1, 1, 1>(a, layer, N, st);
  if (n16 <= 4 && n4 <= 1) return launch_gemv_t<OP, MODE, 4, 1, 1, 1>(a, layer, N, st);
  if (n16 <= 8 && n4 <= 2) return launch_gemv_t<OP, MODE, 8, 1, 2, 1>(a, layer, N, st);
  if (n16 <= 16 && n4 <= 4) return launch_gemv_t<OP, MODE, 4, 4, 4, 1>(a, layer, N, st);
  if (n16 <= 32 && n4 <= 8) return launch_gemv_t<OP, MODE, 8, 4, 4, 2>(a, layer, N, st);
  return hipErrorInvalidValue;
}

hipError_t river_launch_gemv(const DecodeArgs& a, int op, int layer, int mode, hipStream_t st) {
  switch (op * 2 + (mode ? 1 : 0)) {
    case OP_QKV * 2: return launch_op<OP_QKV, 0>(a, layer, st);
    case OP_QKV * 2 + 1: return launch_op<OP_QKV, 1>(a, layer, st);
    case OP_O * 2: return launch_op<OP_O, 0>(a, layer, st);
    case OP_O * 2 + 1: return launch_op<OP_O, 1>(a, layer, st);
    case OP_GU * 2: return launch_op<OP_GU, 0>(a, layer, st);
    case OP_GU * 2 + 1: return launch_op<OP_GU, 1>(a, layer, st);
    case OP_DOWN * 2: return launch_op<OP_DOWN, 0>(a, layer, st);
    case OP_DOWN * 2 + 1: return launch_op<OP_DOWN, 1>(a, layer, st);
    case OP_LM * 2:
    case OP_LM * 2 + 1: return launch_op<OP_LM, 0>(a, layer, st);
  }
  return hipErrorInvalidValue;
}

// Number of workgroups of each stream (for sizing partial-sum buffers).
int river_gemv_max_wg(const Dims& dm) {
  int m = 0;
  const int Ns[4] = {dm.nqkv, dm.d, 2 * dm.F, dm.d};
  for (int i = 0; i < 4; ++i) m = m > Ns[i] / 2 ? m : Ns[i] / 2;  // smallest tile is 2 rows
  return m;
}

hipError_t river_launch_attn(const DecodeArgs& a, int layer, hipStream_t st) {
  const Dims& dm = a.dm;
  const int G = dm.H / dm.Hkv;
  dim3 grid(a.attn_smax, dm.Hkv, dm.B);
  if (dm.D == 128 && G == 4) hipLaunchKernelGGL((k_dec_attn<128, 4>), grid, dim3(kBlock), 0, st, a, layer);
  else if (dm.D == 64 && G == 4) hipLaunchKernelGGL((k_dec_attn<64, 4>), grid, dim3(kBlock), 0, st, a, layer);
  else if (dm.D == 64 && G == 2) hipLaunchKernelGGL((k_dec_attn<64, 2>), grid, dim3(kBlock), 0, st, a, layer);
  else if (dm.D == 128 && G == 2) hipLaunchKernelGGL((k_dec_attn<128, 2>), grid, dim3(kBlock), 0, st, a, layer);
  else if (dm.D == 128 && G == 1) hipLaunchKernelGGL((k_dec_attn<128, 1>), grid, dim3(kBlock), 0, st, a, layer);
  else if (dm.D == 64 && G == 1) hipLaunchKernelGGL((k_dec_attn<64, 1>), grid, dim3(kBlock), 0, st, a, layer);
  else if (dm.D == 128 && G == 8) hipLaunchKernelGGL((k_dec_attn<128, 8>), grid, dim3(kBlock), 0, st, a, layer);
  else if (dm.D == 64 && G == 8) hipLaunchKernelGGL((k_dec_attn<64, 8>), grid, dim3(kBlock), 0, st, a, layer);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// Final norm, LM head + argmax, step bookkeeping (also ends a prefill).
hipError_t river_launch_head(const DecodeArgs& a, hipStream_t st, void (*timer)(void*, int, int),
                             void* tctx, int top) {
  hipLaunchKernelGGL(k_final_norm, dim3(a.dm.B), dim3(kBlock), 0, st, a);
  if (timer && top == TOP_LM) timer(tctx, TOP_LM, 0);
  hipError_t e = river_launch_gemv(a, OP_LM, a.dm.L + 1, 0, st);
  if (timer && top == TOP_LM) timer(tctx, TOP_LM, 1);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_step_end, dim3(1), dim3(64), 0, st, a);
  return hipGetLastError();
}

// Enqueues one decode step. `timer` (optional) is called before and after every launch of the
// timed op (TOP_* codes) so the host can bracket it with events.
hipError_t river_decode_layers(const DecodeArgs& a, int mode, hipStream_t st,
                               void (*timer)(void*, int, int), void* tctx, int top) {
  hipError_t e;
  auto T = [&](int o, int phase) {
    if (timer && o == top) timer(tctx, o, phase);
  };
  for (int l = 1; l <= a.dm.L; ++l) {
    T(TOP_QKV, 0);
    if ((e = river_launch_gemv(a, OP_QKV, l, mode, st)) != hipSuccess) return e;
    T(TOP_QKV, 1);
    T(TOP_ATTN, 0);
    if ((e = river_launch_attn(a, l, st)) != hipSuccess) return e;
    T(TOP_ATTN, 1);
    T(TOP_O, 0);
    if ((e = river_launch_gemv(a, OP_O, l, mode, st)) != hipSuccess) return e;
    T(TOP_O, 1);
    T(TOP_GU, 0);
    if ((e = river_launch_gemv(a, OP_GU, l, mode, st)) != hipSuccess) return e;
    T(TOP_GU, 1);
    T(TOP_DOWN, 0);
    if ((e = river_launch_gemv(a, OP_DOWN, l, mode, st)) != hipSuccess) return e;
    T(TOP_DOWN, 1);
  }
  return river_launch_head(a, st, timer, tctx, top);
}

__global__ void k_begin_steps(int* step) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *step = 0;
}

hipError_t river_launch_begin(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_begin_steps, dim3(1), dim3(64), 0, st, a.step);
  return hipGetLastError();
}
