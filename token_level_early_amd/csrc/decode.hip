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

// Input vector of the GEMV: x = fp16(v * inv * gain) (RMSNorm applied on the fly) or x = v.
struct XSrc {
  const f16* v;
  const f16* gain;
  float inv;
  int K;
};

RIVER_DEV void scale8(uint4& u, const XSrc& s, int e) {
  if (!s.gain) return;
  const uint4 g = *(const uint4*)(s.gain + e);
  uint32_t* pu = (uint32_t*)&u;
  const uint32_t* pg = (const uint32_t*)&g;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h2 v = as_h2(pu[j]), gg = as_h2(pg[j]);
    h2 r;
    r.x = f2h(h2f(v.x) * s.inv * h2f(gg.x));
    r.y = f2h(h2f(v.y) * s.inv * h2f(gg.y));
    pu[j] = as_u32(r);
  }
}

// fp16 stream: the wave's chunks are cid = ws + c*wpr; lane owns elements cid*512 + lane*8 + [0,8)
template <int NCH>
RIVER_DEV void load_x16(const XSrc& s, int ws, int wpr, h2 (&x)[NCH][4]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int e = (ws + c * wpr) * kChunkF16 + lane * 8;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (e < s.K) {
      u = *(const uint4*)(s.v + e);
      scale8(u, s, e);
    }
    x[c][0] = as_h2(u.x);
    x[c][1] = as_h2(u.y);
    x[c][2] = as_h2(u.z);
    x[c][3] = as_h2(u.w);
  }
}

// int4 stream: lane owns elements cid*2048 + lane*32 + [0,32), paired as unpack8 yields
template <int NCH>
RIVER_DEV void load_x4(const XSrc& s, int ws, int wpr, h2 (&x)[NCH][16]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = (ws + c * wpr) * kChunkW4 + lane * 32 + m * 8;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (e < s.K) {
        u = *(const uint4*)(s.v + e);
        scale8(u, s, e);
      }
      const uint32_t in[4] = {u.x, u.y, u.z, u.w};
      h2 o[4];
      pair_for_unpack(in, o);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[c][m * 4 + j] = o[j];
    }
  }
}

template <int NCH, int RB>
RIVER_DEV void rows_f16(const f16* const (&rowp)[RB], int K, int ws, int wpr,
                        const h2 (&x)[NCH][4], float (&acc)[RB]) {
  const int lane = threadIdx.x & (kWave - 1);
  uint4 w[RB][NCH];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e = (ws + c * wpr) * kChunkF16 + lane * 8;
      w[rb][c] = (rowp[rb] != nullptr && e < K) ? *(const uint4*)(rowp[rb] + e)
                                                 : make_uint4(0, 0, 0, 0);
    }
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

template <int NCH, int RB>
RIVER_DEV void rows_w4(const uint8_t* const (&rowp)[RB], const f16* const (&sclp)[RB], int nch,
                       int group, int ws, int wpr, const h2 (&x)[NCH][16], float (&acc)[RB]) {
  const int lane = threadIdx.x & (kWave - 1);
  uint4 w[RB][NCH];
  float sc[RB][NCH];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int cid = ws + c * wpr;
      if (rowp[rb] != nullptr && cid < nch) {
        w[rb][c] = *(const uint4*)(rowp[rb] + (size_t)cid * 1024 + lane * 16);
        sc[rb][c] = h2f(sclp[rb][(cid * kChunkW4 + lane * 32) / group]);
      } else {
        w[rb][c] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
        sc[rb][c] = 0.f;
      }
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
      tot = fmaf(sc[rb][c], s, tot);
    }
    acc[rb] = tot;
  }
}

// Sum of squares of a fp16 vector over the whole block, fixed order (fp64).
RIVER_DEV double block_sumsq(const f16* v, int n, double* red) {
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += kBlock) {
    const double x = (double)h2f(v[i]);
    s += x * x;
  }
  return block_sum_d(s, red);
}

// Sum of red[0..n)[j] for j < 3 over the block in a fixed order; results in out[0..3).
RIVER_DEV void block_sum_red(const double* red, int n, double* out, double* scratch) {
  double s0 = 0, s1 = 0, s2 = 0;
  for (int i = threadIdx.x; i < n; i += kBlock) {
    s0 += red[i * 4 + 0];
    s1 += red[i * 4 + 1];
    s2 += red[i * 4 + 2];
  }
  out[0] = block_sum_d(s0, scratch);
  out[1] = block_sum_d(s1, scratch);
  out[2] = block_sum_d(s2, scratch);
}

template <int NCH16, int WPR16, int NCH4, int WPR4>
__global__ __launch_bounds__(kBlock) void k_dec_gemv(DecodeArgs a, int op, int layer,
                                                     int nwg16, int nwg4) {
  using T16 = TileF16<WPR16>;
  using T4 = TileW4<WPR4>;
  constexpr int TRMAX = (T16::TR > T4::TR ? T16::TR : T4::TR);
  __shared__ float ypart[TRMAX][4];
  __shared__ float y[TRMAX];
  __shared__ double dred[4];
  __shared__ double dsum[4];
  __shared__ int lflag;

  const Dims& dm = a.dm;
  const int b = 0;  // batch row (VALU path decodes one row)
  const int route = (op == OP_LM) ? ROUTE_BACKBONE : a.route[layer * dm.B + b];
  const bool is4 = blockIdx.x >= (unsigned)nwg16;
  if (is4 != (route == ROUTE_RIVER)) return;
  const int tile = is4 ? (int)blockIdx.x - nwg16 : (int)blockIdx.x;
  const int TR = is4 ? T4::TR : T16::TR;
  const int nwg = is4 ? nwg4 : nwg16;
  const LayerDev* lwp = (op == OP_LM) ? nullptr : &a.layers[layer - 1];
  const int N = op_rows(op, dm);
  const int K = op_k(op, dm);
  const int step = *a.step;

  // ---- input vector -------------------------------------------------------------------
  XSrc xs;
  xs.K = K;
  xs.gain = nullptr;
  xs.inv = 1.f;
  if (op == OP_QKV) {
    xs.gain = lwp->attn_norm;
    if (layer == 1) {
      int tok = (step == 0) ? a.tok_in[b] : a.tok_out[(step - 1) * dm.B + b];
      if (tok < 0 || tok >= dm.V) {
        if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(a.err, ERR_TOKEN);
        tok = 0;
      }
      xs.v = a.embed + (size_t)tok * dm.d;
      const double ss = block_sumsq(xs.v, dm.d, dred);
      xs.inv = (float)(1.0 / sqrt(ss / dm.d + (double)dm.eps));
      if (blockIdx.x == (unsigned)(is4 ? nwg16 : 0)) {  // first active workgroup
        f16* h0 = a.hs + (size_t)b * dm.d;
        for (int i = threadIdx.x; i < dm.d; i += kBlock) h0[i] = xs.v[i];
        if (threadIdx.x == 0) {
          if (a.exit_out) a.exit_out[step * dm.B + b] = dm.L;
          a.inv_attn[b] = xs.inv;
        }
        if (a.sim_out)
          for (int i = threadIdx.x; i < dm.L; i += kBlock)
            a.sim_out[((size_t)step * dm.B + b) * dm.L + i] = __builtin_nanf("");
      }
    } else {
      xs.v = a.hs + ((size_t)(layer - 1) * dm.B + b) * dm.d;
      xs.inv = a.inv_attn[(layer - 1) * dm.B + b];
    }
  } else if (op == OP_O) {
    xs.v = a.o + (size_t)b * dm.hd;
  } else if (op == OP_GU) {
    xs.v = a.hmid + ((size_t)(layer - 1) * dm.B + b) * dm.d;
    xs.gain = lwp->mlp_norm;
    xs.inv = a.inv_mlp[(layer - 1) * dm.B + b];
  } else if (op == OP_DOWN) {
    xs.v = a.a2 + (size_t)b * dm.F;
  } else {
    xs.v = a.hs + ((size_t)dm.L * dm.B + b) * dm.d;
    xs.gain = a.final_norm;
    xs.inv = a.inv_attn[dm.L * dm.B + b];
  }

  // ---- GEMV ---------------------------------------------------------------------------
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (!is4) {
    constexpr int RB = kRB16;
    const int rg = w / WPR16, ws = w % WPR16;
    h2 x[NCH16][4];
    load_x16<NCH16>(xs, ws, WPR16, x);
    const f16* rowp[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = rg * RB + rb;
      const int n = logical_row(op, tile, r, T16::TR, dm);
      rowp[rb] = (n < N) ? (op == OP_LM ? a.lm_head + (size_t)n * dm.d : f16_row(op, n, *lwp, a))
                         : nullptr;
    }
    float acc[RB];
    rows_f16<NCH16, RB>(rowp, K, ws, WPR16, x, acc);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float v = wave_sum(acc[rb]);
      if (lane == 0) ypart[rg * RB + rb][ws] = v;
    }
    __syncthreads();
    if (threadIdx.x < T16::TR) {
      float s = 0.f;
      for (int j = 0; j < WPR16; ++j) s += ypart[threadIdx.x][j];
      y[threadIdx.x] = s;
    }
  } else {
    constexpr int RB = kRB4;
    const int rg = w / WPR4, ws = w % WPR4;
    h2 x[NCH4][16];
    load_x4<NCH4>(xs, ws, WPR4, x);
    const uint8_t* rowp[RB];
    const f16* sclp[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = rg * RB + rb;
      const int n = logical_row(op, tile, r, T4::TR, dm);
      if (n < N) {
        w4_row(op, n, *lwp, dm, rowp[rb], sclp[rb]);
      } else {
        rowp[rb] = nullptr;
        sclp[rb] = nullptr;
      }
    }
    const int nch = (K + kChunkW4 - 1) / kChunkW4;
    float acc[RB];
    rows_w4<NCH4, RB>(rowp, sclp, nch, dm.group, ws, WPR4, x, acc);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float v = wave_sum(acc[rb]);
      if (lane == 0) ypart[rg * RB + rb][ws] = v;
    }
    __syncthreads();
    if (threadIdx.x < T4::TR) {
      float s = 0.f;
      for (int j = 0; j < WPR4; ++j) s += ypart[threadIdx.x][j];
      y[threadIdx.x] = s;
    }
  }
  __syncthreads();

  // ---- epilogues ----------------------------------------------------------------------
  const int t = threadIdx.x;
  if (op == OP_QKV) {
    const int pos = a.pos[b];
    const int qk_rows = (dm.H + dm.Hkv) * dm.D;
    const int n0 = logical_row(op, tile, 0, TR, dm);
    if (n0 < qk_rows) {
      const int half = TR / 2;
      if (t < half) {
        const int n = logical_row(op, tile, t, TR, dm);
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
      const int n = logical_row(op, tile, t, TR, dm);
      if (n < N) {
        const int vi = n - qk_rows;
        const int kvh = vi / dm.D, i = vi % dm.D;
        f16* vd = a.kv + ((((size_t)(layer - 1) * 2 + 1) * dm.B + b) * dm.Hkv + kvh) *
                             (size_t)dm.Tmax * dm.D + (size_t)pos * dm.D;
        vd[i] = f2h(y[t]);
      }
    }
  } else if (op == OP_GU) {
    const int half = TR / 2;
    if (t < half) {
      const int f = logical_row(op, tile, t, TR, dm);
      if (f < dm.F) {
        const float g = h2f(f2h(y[t])), u = h2f(f2h(y[t + half]));
        const float sg = g / (1.f + __expf(-g));
        a.a2[(size_t)b * dm.F + f] = f2h(sg * u);
      }
    }
  } else if (op == OP_O || op == OP_DOWN) {
    double p0 = 0, p1 = 0, p2 = 0;
    if (t < TR) {
      const int n = logical_row(op, tile, t, TR, dm);
      if (n < N) {
        if (op == OP_O) {
          const f16 hin = a.hs[((size_t)(layer - 1) * dm.B + b) * dm.d + n];
          const f16 hm = f2h(h2f(hin) + h2f(f2h(y[t])));
          a.hmid[((size_t)(layer - 1) * dm.B + b) * dm.d + n] = hm;
          p2 = (double)h2f(hm) * (double)h2f(hm);
        } else {
          const f16 hm = a.hmid[((size_t)(layer - 1) * dm.B + b) * dm.d + n];
          const f16 ho = f2h(h2f(hm) + h2f(f2h(y[t])));
          a.hs[((size_t)layer * dm.B + b) * dm.d + n] = ho;
          const double hp = (double)h2f(a.hs[((size_t)(layer - 1) * dm.B + b) * dm.d + n]);
          const double hv = (double)h2f(ho);
          p0 = hp * hv;
          p1 = hp * hp;
          p2 = hv * hv;
        }
      }
    }
    // per-workgroup partials -> red[tile]; the last workgroup finishes the reduction
    const double s0 = block_sum_d(p0, dred);
    const double s1 = block_sum_d(p1, dred);
    const double s2 = block_sum_d(p2, dred);
    if (t == 0) {
      a.red[tile * 4 + 0] = s0;
      a.red[tile * 4 + 1] = s1;
      a.red[tile * 4 + 2] = s2;
    }
    int* counter = a.cnt + (op == OP_O ? CNT_O : CNT_DOWN);
    if (arrive_last(counter, nwg, &lflag)) {
      block_sum_red(a.red, nwg, dsum, dred);
      if (t == 0) {
        const double dot = dsum[0], n1 = dsum[1], n2 = dsum[2];
        if (op == OP_O) {
          a.inv_mlp[(layer - 1) * dm.B + b] = (float)(1.0 / sqrt(n2 / dm.d + (double)dm.eps));
        } else {
          a.inv_attn[layer * dm.B + b] = (float)(1.0 / sqrt(n2 / dm.d + (double)dm.eps));
          if (layer < dm.L) {
            int nr = route;
            if (route == ROUTE_BACKBONE) {
              bool ex = false;
              if (a.sched) {
                int e = a.sched[step * dm.B + b];
                if (e < dm.entry || e > dm.L) {
                  atomicOr(a.err, ERR_FORCED);
                  e = dm.L;
                }
                ex = (layer == e);
              } else if (layer >= dm.entry) {
                const double sim = (n1 > 0.0 && n2 > 0.0) ? dot / sqrt(n1 * n2) : 0.0;
                if (a.sim_out) a.sim_out[((size_t)step * dm.B + b) * dm.L + layer - 1] = (float)sim;
                ex = sim > (double)a.tau;
              }
              if (ex) {
                nr = ROUTE_RIVER;
                if (a.exit_out) a.exit_out[step * dm.B + b] = layer;
              }
            }
            a.route[(layer + 1) * dm.B + b] = nr;
          }
        }
        reset_counter(counter);
      }
    }
  } else {  // OP_LM: logits + argmax (lowest index on ties)
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
      const unsigned long long key =
          ((unsigned long long)float_key(best) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)bi);
      __hip_atomic_fetch_max(a.amax + b, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    int* counter = a.cnt + CNT_LM;
    if (arrive_last(counter, nwg, &lflag)) {
      if (t == 0) {
        const unsigned long long key =
            __hip_atomic_load(a.amax + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int tok = (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull));
        a.tok_out[step * dm.B + b] = tok;
        a.pos[b] += 1;
        *a.step = step + 1;
        __hip_atomic_store(a.amax + b, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        reset_counter(counter);
      }
    }
  }
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
      const uint4 u = *(const uint4*)(a.q + (size_t)b * dm.hd + (size_t)(kvh * G + g) * D + d0);
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
        if (t < t1) {
          kk[u] = *(const uint4*)(Kb + (size_t)t * D + d0);
          vv[u] = *(const uint4*)(Vb + (size_t)t * D + d0);
        }
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
      a.pacc[pi * D + dd] = A;
      if (dd == 0) {
        a.pml[pi * 2 + 0] = M;
        a.pml[pi * 2 + 1] = Lsum;
      }
    }
  }

  int* counter = a.cnt + CNT_ATTN + b * dm.Hkv + kvh;
  if (arrive_last(counter, smax, &lflag)) {
    // split weights exp2(m_s - M) / L per query head
    if (threadIdx.x < G) {
      const int g = threadIdx.x;
      float M = -__builtin_inff();
      for (int j = 0; j < seff; ++j) M = fmaxf(M, a.pml[(pbase + (size_t)g * smax + j) * 2]);
      float Lsum = 0.f;
      for (int j = 0; j < seff; ++j) {
        const float e = exp2f(a.pml[(pbase + (size_t)g * smax + j) * 2] - M);
        sm_w[g][j] = e;
        Lsum += a.pml[(pbase + (size_t)g * smax + j) * 2 + 1] * e;
      }
      sm_L[g] = Lsum;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += kBlock) {
      const int g = idx / D, dd = idx % D;
      float A = 0.f;
      for (int j = 0; j < seff; ++j) A += sm_w[g][j] * a.pacc[(pbase + (size_t)g * smax + j) * D + dd];
      a.o[(size_t)b * dm.hd + (size_t)(kvh * G + g) * D + dd] = f2h(A / sm_L[g]);
    }
    if (threadIdx.x == 0) reset_counter(counter);
  }
}

// ---------------------------------------------------------------------------------------
// Host-side launchers (called from api.cpp)
// ---------------------------------------------------------------------------------------
struct GemvShape {
  int nwg16, nwg4;
};

template <int NCH16, int WPR16, int NCH4, int WPR4>
static hipError_t launch_gemv_t(const DecodeArgs& a, int op, int layer, int N, hipStream_t st,
                                GemvShape* shape) {
  const int tr16 = TileF16<WPR16>::TR, tr4 = TileW4<WPR4>::TR;
  int nwg16 = 0, nwg4 = 0;
  if (op == OP_QKV || op == OP_GU) {
    nwg16 = (op == OP_GU) ? (N / 2) / (tr16 / 2) : N / tr16;
    nwg4 = (op == OP_LM) ? 0 : ((op == OP_GU) ? (N / 2) / (tr4 / 2) : N / tr4);
  } else {
    nwg16 = (N + tr16 - 1) / tr16;
    nwg4 = (op == OP_LM) ? 0 : (N + tr4 - 1) / tr4;
  }
  if (shape) {
    shape->nwg16 = nwg16;
    shape->nwg4 = nwg4;
  }
  hipLaunchKernelGGL((k_dec_gemv<NCH16, WPR16, NCH4, WPR4>), dim3(nwg16 + nwg4), dim3(kBlock), 0,
                     st, a, op, layer, nwg16, nwg4);
  return hipGetLastError();
}

// Picks the stream geometry from K: chunks per row nch, waves per row wpr, chunks per wave NCH.
hipError_t river_launch_gemv(const DecodeArgs& a, int op, int layer, hipStream_t st) {
  const Dims& dm = a.dm;
  const int N = (op == OP_QKV) ? dm.nqkv : (op == OP_GU) ? 2 * dm.F : (op == OP_LM) ? dm.V : dm.d;
  const int K = (op == OP_O) ? dm.hd : (op == OP_DOWN) ? dm.F : dm.d;
  const int n16 = (K + kChunkF16 - 1) / kChunkF16;
  const int n4 = (K + kChunkW4 - 1) / kChunkW4;
  // fp16: up to 8 chunks per wave; int4: up to 4
  if (n16 <= 1 && n4 <= 1) return launch_gemv_t<1, 1, 1, 1>(a, op, layer, N, st, nullptr);
  if (n16 <= 2 && n4 <= 1) return launch_gemv_t<2, 1, 1, 1>(a, op, layer, N, st, nullptr);
  if (n16 <= 4 && n4 <= 1) return launch_gemv_t<4, 1, 1, 1>(a, op, layer, N, st, nullptr);
  if (n16 <= 8 && n4 <= 2) return launch_gemv_t<8, 1, 2, 1>(a, op, layer, N, st, nullptr);
  if (n16 <= 16 && n4 <= 4) return launch_gemv_t<4, 4, 4, 1>(a, op, layer, N, st, nullptr);
  if (n16 <= 32 && n4 <= 8) return launch_gemv_t<8, 4, 4, 2>(a, op, layer, N, st, nullptr);
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

hipError_t river_decode_layers(const DecodeArgs& a, hipStream_t st) {
  hipError_t e;
  for (int l = 1; l <= a.dm.L; ++l) {
    if ((e = river_launch_gemv(a, OP_QKV, l, st)) != hipSuccess) return e;
    if ((e = river_launch_attn(a, l, st)) != hipSuccess) return e;
    if ((e = river_launch_gemv(a, OP_O, l, st)) != hipSuccess) return e;
    if ((e = river_launch_gemv(a, OP_GU, l, st)) != hipSuccess) return e;
    if ((e = river_launch_gemv(a, OP_DOWN, l, st)) != hipSuccess) return e;
  }
  return river_launch_gemv(a, OP_LM, a.dm.L + 1, st);
}

__global__ void k_begin_steps(int* step) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *step = 0;
}

hipError_t river_launch_begin(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_begin_steps, dim3(1), dim3(64), 0, st, a.step);
  return hipGetLastError();
}
