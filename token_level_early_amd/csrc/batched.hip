// Batched early-exit decode (2..16 rows) with matrix cores.
//
// Each row keeps its own route: at layer l, rows that are still on the backbone use block l's
// fp16 weights and rows that have exited use its W4A16 river copy (River-LLM paper, Method:
// token-level exit with one shared KV cache). A projection launch therefore has two weight
// streams; each workgroup serves one 16-column tile of one stream for all rows at once and
// skips its stream entirely when no row needs it, so a layer reads both copies only when its
// rows disagree.
//
// GEMM core: Y[16 rows][16 cols] = X[16][K] W[cols][K]^T on CDNA4's v_mfma_f32_16x16x32_f16 with
// fp32 accumulation; the batch is padded to 16 rows. Every lane loads 8 consecutive K elements
// of one input row (A operand) and of one weight row (B operand) per 32-wide K window: one MFMA
// per window; a dot product does not depend on which lane slot carries which K index as long as
// both operands agree. The int4
// stream turns 8 nibbles into exact fp16 integers (the 0x6400 exponent trick, pairs (0,4),
// (1,5), (2,6), (3,7)), permutes the input the same way, sums one quantisation group on the
// MFMA and applies the fp32 group scale per output column. The four waves of a workgroup split
// K and meet in LDS.
//
// Per layer: k_b_prep (exit test per row, then the attention RMSNorm) -> QKV (RoPE, q and the
// KV append at each row's position) -> attention (the split-K kernel shared with batch 1, one
// grid slice per row) -> O + residual -> k_b_prep (MLP RMSNorm) -> gate|up + SwiGLU -> down +
// residual. Head: final RMSNorm, fp16 LM head with a per-row 64-bit atomic-max argmax, step end.
#include "gemv.hpp"

static constexpr int kBR = 16;  // rows of an MFMA tile (the batch, padded)

typedef _Float16 bh4 __attribute__((ext_vector_type(4)));
typedef float bf4 __attribute__((ext_vector_type(4)));

typedef _Float16 bh8 __attribute__((ext_vector_type(8)));
typedef uint32_t bu4 __attribute__((ext_vector_type(4)));

// 8 fp16 values of a 16-byte load as one 16x16x32 MFMA operand
RIVER_DEV bh8 as8(uint4 u) { return __builtin_bit_cast(bh8, (bu4){u.x, u.y, u.z, u.w}); }

// ---------------------------------------------------------------------------------------
// Per-row preparation: KIND 0 = exit test + attention RMSNorm of layer `layer`'s input,
// KIND 1 = MLP RMSNorm of h_mid, KIND 2 = final RMSNorm of h(L). Writes xn[b][d].
// ---------------------------------------------------------------------------------------
template <int KIND>
__global__ __launch_bounds__(kBlock) void k_b_prep(DecodeArgs a, int layer, int mode, f16* xn) {
  __shared__ double red[4];
  const Dims& dm = a.dm;
  const int b = blockIdx.x, t = threadIdx.x;
  const int step = *a.step;
  const f16* hin;
  const f16* gain;
  if (KIND == 0) {
    const LayerDev& lw = a.layers[layer - 1];
    gain = lw.attn_norm;
    int route = ROUTE_BACKBONE;
    if (layer == 1) {
      int tok = (step == 0) ? a.tok_in[b] : a.tok_out[(step - 1) * dm.B + b];
      if (tok < 0 || tok >= dm.V) {
        if (t == 0) atomicOr(a.err, ERR_TOKEN);
        tok = 0;
      }
      hin = a.embed + (size_t)tok * dm.d;
      f16* h0 = a.hs + (size_t)b * dm.d;
      for (int i = t; i < dm.d; i += kBlock) h0[i] = hin[i];
      if (t == 0 && a.exit_out) a.exit_out[step * dm.B + b] = dm.L;
      if (a.sim_out)
        for (int i = t; i < dm.L; i += kBlock) a.sim_out[((size_t)step * dm.B + b) * dm.L + i] = __builtin_nanf("");
      if (mode == 0 && a.sched && a.sched[step * dm.B + b] == 0) {  // no backbone block at all
        route = ROUTE_RIVER;
        if (t == 0 && a.exit_out) a.exit_out[step * dm.B + b] = 0;
      }
    } else {
      hin = a.hs + ((size_t)(layer - 1) * dm.B + b) * dm.d;
      if (mode == 0) {
        const int lp = layer - 1;
        const int prev = a.route[lp * dm.B + b];
        if (prev == ROUTE_RIVER) {
          route = ROUTE_RIVER;
        } else if (lp >= dm.entry) {
          if (a.sched) {
            int e = a.sched[step * dm.B + b];
            if ((e < dm.entry && e != 0) || e > dm.L) {
              if (t == 0) atomicOr(a.err, ERR_FORCED);
              e = dm.L;
            }
            if (lp == e) route = ROUTE_RIVER;
          } else {
            const f16* hprev = a.hs + ((size_t)(lp - 1) * dm.B + b) * dm.d;
            double s0 = 0.0, s1 = 0.0, s2 = 0.0;
            for (int i = t; i < dm.d; i += kBlock) {
              const double x = (double)h2f(hprev[i]), y = (double)h2f(hin[i]);
              s0 += x * y;
              s1 += x * x;
              s2 += y * y;
            }
            const double dot = block_sum_d(s0, red), n1 = block_sum_d(s1, red), n2 = block_sum_d(s2, red);
            const double sim = (n1 > 0.0 && n2 > 0.0) ? dot / sqrt(n1 * n2) : 0.0;
            if (t == 0 && a.sim_out) a.sim_out[((size_t)step * dm.B + b) * dm.L + lp - 1] = (float)sim;
            if (sim > (double)a.tau) route = ROUTE_RIVER;
          }
          if (route == ROUTE_RIVER && t == 0 && a.exit_out) a.exit_out[step * dm.B + b] = lp;
        }
      }
    }
    if (t == 0) a.route[layer * dm.B + b] = route;
  } else if (KIND == 1) {
    hin = a.hmid + ((size_t)(layer - 1) * dm.B + b) * dm.d;
    gain = a.layers[layer - 1].mlp_norm;
  } else {
    hin = a.hs + ((size_t)dm.L * dm.B + b) * dm.d;
    gain = a.final_norm;
  }
  // RMSNorm (fp64 sum of squares), rounded to fp16 like every other path's staging
  double ss = 0.0;
  for (int i = t; i < dm.d; i += kBlock) {
    const double x = (double)h2f(hin[i]);
    ss += x * x;
  }
  const float inv = inv_rms(block_sum_d(ss, red), dm.d, dm.eps);
  f16* out = xn + (size_t)b * dm.d;
  for (int g = t; g * 8 < dm.d; g += kBlock)
    *(uint4*)(out + g * 8) = norm8(*(const uint4*)(hin + g * 8), *(const uint4*)(gain + g * 8), inv, true);
}

// ---------------------------------------------------------------------------------------
// Batched projection: grid (tiles of 16 logical columns, stream), 4 waves splitting K.
// ---------------------------------------------------------------------------------------
// 16-column tiles per workgroup: four for gate|up (two weight streams, the int4 one reading
// four times its own bytes of input per tile); one elsewhere, where fewer workgroups measured
// slower
static constexpr int kTW = 4;
__host__ __device__ constexpr int b_tw(int op) { return op == OP_GU ? 4 : 1; }
struct BSmem {
  float part[4][kTW][kBR][kBR];  // per wave (K slice)
  float y[kTW][kBR][kBR];
  int need;
};

template <int OP>
__global__ __launch_bounds__(kBlock) void k_b_gemm(DecodeArgs a, int layer, const f16* xin) {
  __shared__ BSmem sm;
  const Dims& dm = a.dm;
  const int stream = blockIdx.y;  // stream 0 backbone fp16, 1 river int4
  const int t = threadIdx.x, w = t / kWave, lane = t % kWave;
  const int N = op_rows(OP, dm), K = op_k(OP, dm);
  const LayerDev* lw = (OP == OP_LM) ? nullptr : &a.layers[layer - 1];
  // does any row run this stream at this layer?
  if (t == 0) sm.need = 0;
  __syncthreads();
  if (t < dm.B) {
    const int r = (OP == OP_LM) ? ROUTE_BACKBONE : a.route[layer * dm.B + t];
    if (r == stream) atomicOr(&sm.need, 1);
  }
  __syncthreads();
  if (!sm.need) return;

  // TW 16-column tiles per workgroup: every wave reads each input window once for all of
  // them (the inputs come from L2 for every tile, as many bytes as the fp16 weights)
  constexpr int TW = b_tw(OP);
  const int tile0 = blockIdx.x * TW;
  const int col = lane % 16, kq = lane / 16;
  int n[TW];
  bool nok[TW];
#pragma unroll
  for (int s = 0; s < TW; ++s) {  // this lane's weight column in tile s
    n[s] = logical_row(OP, tile0 + s, col, kBR, dm);
    nok[s] = n[s] < N;
  }
  const int xrow = lane % 16;  // batch row fed by this lane (A operand)
  const bool xok = xrow < dm.B;
  const f16* xp = xin + (size_t)(xok ? xrow : 0) * K;

  bf4 acc[TW];
#pragma unroll
  for (int s = 0; s < TW; ++s) acc[s] = bf4{0.f, 0.f, 0.f, 0.f};
  if (stream == 0) {
    const f16* wrow[TW];
#pragma unroll
    for (int s = 0; s < TW; ++s)
      wrow[s] = (OP == OP_LM) ? a.lm_head + (size_t)(nok[s] ? n[s] : 0) * dm.d : f16_row(OP, nok[s] ? n[s] : 0, *lw, a);
    const int nwin = (K + 31) / 32;
    const int w0 = w * nwin / 4, w1 = (w + 1) * nwin / 4;
    // batches of two 32-wide windows, double-buffered: the next batch's loads are in flight
    // while the current one runs on the MFMA
    constexpr int WB = 2;
    auto loadb = [&](int win, uint4 (&xa)[WB], uint4 (&wb)[WB][TW]) {
#pragma unroll
      for (int u = 0; u < WB; ++u) {
        const int k = (win + u) * 32 + kq * 8;
        const bool ok = win + u < w1 && k < K;
        xa[u] = (ok && xok) ? ldg16(xp + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int s = 0; s < TW; ++s) wb[u][s] = (ok && nok[s]) ? ldg16(wrow[s] + k) : make_uint4(0, 0, 0, 0);
      }
    };
    auto mmab = [&](const uint4 (&xa)[WB], const uint4 (&wb)[WB][TW]) {
#pragma unroll
      for (int u = 0; u < WB; ++u)
#pragma unroll
        for (int s = 0; s < TW; ++s) {
          acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as8(xa[u]), as8(wb[u][s]), acc[s], 0, 0, 0);
        }
    };
    uint4 xa0[WB], wb0[WB][TW], xa1[WB], wb1[WB][TW];
    int win = w0;
    if (win < w1) loadb(win, xa0, wb0);
    for (; win < w1; win += 2 * WB) {
      if (win + WB < w1) loadb(win + WB, xa1, wb1);
      mmab(xa0, wb0);  // windows past w1 are zero: they add nothing
      if (win + 2 * WB < w1) loadb(win + 2 * WB, xa0, wb0);
      if (win + WB < w1) mmab(xa1, wb1);
    }
  } else {
    const uint8_t* rp[TW];
    const f16* sp[TW];
    const uint8_t* zp[TW];  // zero-point format only (else null)
#pragma unroll
    for (int s = 0; s < TW; ++s) w4_row(OP, nok[s] ? n[s] : 0, *lw, dm, rp[s], sp[s], zp[s]);
    const bool zpf = dm.zp != 0;
    const int g = dm.group, wpg = g / 32;  // 32-wide windows per group (1, 2 or 4)
    const int ng = (K + g - 1) / g;
    const int g0 = w * ng / 4, g1 = (w + 1) * ng / 4;
    // one group's windows and scales per batch, double-buffered across groups
    auto loadg = [&](int grp, uint4 (&xr)[4], uint32_t (&wq)[4][TW], float (&sc)[TW], float (&zc)[TW]) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        xr[u] = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int s = 0; s < TW; ++s) wq[u][s] = 0x88888888u;
        if (u < wpg) {
          const int k = grp * g + u * 32 + kq * 8;
          const bool ok = k < K;
          xr[u] = (ok && xok) ? ldg16(xp + k) : make_uint4(0, 0, 0, 0);
          // 8 nibbles of this lane's weight row: bytes k/2 .. k/2+3 (padding nibbles are q = 0)
#pragma unroll
          for (int s = 0; s < TW; ++s)
            if (nok[s]) wq[u][s] = *(const __attribute__((address_space(1))) uint32_t*)(rp[s] + k / 2);
        }
      }
#pragma unroll
      for (int s = 0; s < TW; ++s) {
        sc[s] = nok[s] ? h2f(sp[s][grp]) : 0.f;  // scale of (column, group)
        zc[s] = (zpf && nok[s]) ? 8.f - (float)zp[s][grp] : 0.f;  // zero-point format: 8 - z
      }
    };
    // unpack8 gives q = u - 8; the zero-point format needs u - z = (u - 8) + (8 - z): the group's
    // input sums per batch row come from one more MFMA against a ones operand (they land in the
    // accumulator layout, every column holding its row's sum)
    auto mmag = [&](const uint4 (&xr)[4], const uint32_t (&wq)[4][TW], const float (&sc)[TW],
                    const float (&zc)[TW]) {
      bf4 tmp[TW];
      bf4 xs = bf4{0.f, 0.f, 0.f, 0.f};
      const bh8 ones = bh8{(f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f};
#pragma unroll
      for (int s = 0; s < TW; ++s) tmp[s] = bf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (u < wpg) {
          const uint32_t in[4] = {xr[u].x, xr[u].y, xr[u].z, xr[u].w};
          h2 xo[4];
          pair_for_unpack(in, xo);  // (x0,x4) (x1,x5) (x2,x6) (x3,x7)
          const bh8 a8 = __builtin_bit_cast(bh8, (bu4){as_u32(xo[0]), as_u32(xo[1]), as_u32(xo[2]), as_u32(xo[3])});
          if (zpf) xs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a8, ones, xs, 0, 0, 0);
#pragma unroll
          for (int s = 0; s < TW; ++s) {
            h2 p0, p1, p2, p3;
            unpack8(wq[u][s], p0, p1, p2, p3);  // (q0,q4) (q1,q5) (q2,q6) (q3,q7)
            const bh8 b8 = __builtin_bit_cast(bh8, (bu4){as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3)});
            tmp[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a8, b8, tmp[s], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int s = 0; s < TW; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[s][r] = fmaf(sc[s], zpf ? fmaf(zc[s], xs[r], tmp[s][r]) : tmp[s][r], acc[s][r]);
    };
    uint4 xr0[4], xr1[4];
    uint32_t wq0[4][TW], wq1[4][TW];
    float sc0[TW], sc1[TW], zc0[TW], zc1[TW];
    int grp = g0;
    if (grp < g1) loadg(grp, xr0, wq0, sc0, zc0);
    for (; grp < g1; grp += 2) {
      if (grp + 1 < g1) loadg(grp + 1, xr1, wq1, sc1, zc1);
      mmag(xr0, wq0, sc0, zc0);
      if (grp + 2 < g1) loadg(grp + 2, xr0, wq0, sc0, zc0);
      if (grp + 1 < g1) mmag(xr1, wq1, sc1, zc1);
    }
  }
  // lane holds Y[row 4*kq + r][col] of each tile; sum the four waves' K slices
#pragma unroll
  for (int s = 0; s < TW; ++s)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.part[w][s][4 * kq + r][col] = acc[s][r];
  __syncthreads();
  for (int i = t; i < TW * kBR * kBR; i += kBlock) {
    const int s = i / (kBR * kBR), row = (i / kBR) % kBR, c = i % kBR;
    sm.y[s][row][c] = (sm.part[0][s][row][c] + sm.part[1][s][row][c]) + (sm.part[2][s][row][c] + sm.part[3][s][row][c]);
  }
  __syncthreads();

  // epilogue per 16-column tile: thread -> (row b, tile column c), rows on this stream only
  auto epilogue = [&](int tile, const float (&y)[kBR][kBR]) {
  const int b = t / kBR, c = t % kBR;
  if (b >= dm.B) return;
  if (OP != OP_LM && a.route[layer * dm.B + b] != stream) return;
  const float yv = y[b][c];
  if (OP == OP_QKV) {
    const int pos = a.pos[b];
    const int qk_rows = (dm.H + dm.Hkv) * dm.D;
    const int n0 = logical_row(OP, tile, 0, kBR, dm);
    if (n0 < qk_rows) {
      if (c < kBR / 2) {
        const int nn = logical_row(OP, tile, c, kBR, dm);
        const int head = nn / dm.D, i = nn % dm.D;  // i < D/2
        const float x0 = h2f(f2h(yv)), x1 = h2f(f2h(y[b][c + kBR / 2]));
        const float2 cs = a.rope[(size_t)pos * (dm.D / 2) + i];
        const f16 r0 = f2h(x0 * cs.x - x1 * cs.y);
        const f16 r1 = f2h(x1 * cs.x + x0 * cs.y);
        f16* dst;
        if (head < dm.H) {
          dst = a.q + (size_t)b * dm.hd + head * dm.D;
        } else {
          const int kvh = head - dm.H;
          dst = a.kv + ((((size_t)(layer - 1) * 2 + 0) * dm.B + b) * dm.Hkv + kvh) * (size_t)dm.Tmax * dm.D +
                (size_t)pos * dm.D;
        }
        dst[i] = r0;
        dst[i + dm.D / 2] = r1;
        if (head >= dm.H) {
          kv_count(a.kvcnt, a.kv, dst + i, 1);
          kv_count(a.kvcnt, a.kv, dst + i + dm.D / 2, 1);
        }
      }
    } else {
      const int nn = logical_row(OP, tile, c, kBR, dm);
      if (nn < N) {
        const int vi = nn - qk_rows;
        const int kvh = vi / dm.D, i = vi % dm.D;
        f16* vd = a.kv + ((((size_t)(layer - 1) * 2 + 1) * dm.B + b) * dm.Hkv + kvh) * (size_t)dm.Tmax * dm.D +
                  (size_t)pos * dm.D + i;
        *vd = f2h(yv);
        kv_count(a.kvcnt, a.kv, vd, 1);
      }
    }
  } else if (OP == OP_GU) {
    if (c < kBR / 2) {
      const int f = logical_row(OP, tile, c, kBR, dm);
      if (f < dm.F) {
        const float gg = h2f(f2h(yv)), uu = h2f(f2h(y[b][c + kBR / 2]));
        const float sg = gg / (1.f + __expf(-gg));
        a.a2[(size_t)b * dm.F + f] = f2h(sg * uu);
      }
    }
  } else if (OP == OP_O) {
    const int nn = tile * kBR + c;
    if (nn < N) {
      const size_t i = ((size_t)(layer - 1) * dm.B + b) * dm.d + nn;
      a.hmid[i] = f2h(h2f(a.hs[i]) + h2f(f2h(yv)));
    }
  } else if (OP == OP_DOWN) {
    const int nn = tile * kBR + c;
    if (nn < N) {
      const size_t i = ((size_t)(layer - 1) * dm.B + b) * dm.d + nn;
      a.hs[(size_t)dm.B * dm.d + i] = f2h(h2f(a.hmid[i]) + h2f(f2h(yv)));
    }
  } else {  // OP_LM: the row's best column of this tile (lowest index on ties)
    const int nn = tile * kBR + c;
    float v = (nn < N) ? yv : -__builtin_inff();
    if (a.logits && nn < N) a.logits[(size_t)b * dm.V + nn] = yv;
    if (c == 0) {
      float best = -__builtin_inff();
      int bi = 0x7FFFFFFF;
      for (int j = 0; j < kBR; ++j) {
        const int nj = tile * kBR + j;
        if (nj >= N) break;
        const float vj = y[b][j];
        if (vj > best) {
          best = vj;
          bi = nj;
        }
      }
      if (bi != 0x7FFFFFFF) {
        const unsigned long long key = ((unsigned long long)float_key(best) << 32) |
                                       (unsigned long long)(0xFFFFFFFFu - (uint32_t)bi);
        __hip_atomic_fetch_max(a.amax + b, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    (void)v;
  }
  };
#pragma unroll
  for (int s = 0; s < TW; ++s) epilogue(tile0 + s, sm.y[s]);
}

// ---------------------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------------------
hipError_t river_launch_attn(const DecodeArgs& a, int layer, hipStream_t st);
hipError_t river_launch_step_end(const DecodeArgs& a, hipStream_t st);

template <int OP>
static hipError_t launch_b_gemm(const DecodeArgs& a, int layer, int mode, const f16* xin, hipStream_t st) {
  const Dims& dm = a.dm;
  const int N = (OP == OP_QKV) ? dm.nqkv : (OP == OP_GU) ? 2 * dm.F : (OP == OP_LM) ? dm.V : dm.d;
  const int tiles = ((N + kBR - 1) / kBR + b_tw(OP) - 1) / b_tw(OP);  // workgroups of 16-column tiles
  const int streams = (OP == OP_LM || mode == 1) ? 1 : 2;
  hipLaunchKernelGGL((k_b_gemm<OP>), dim3(tiles, streams), dim3(kBlock), 0, st, a, layer, xin);
  return hipGetLastError();
}

hipError_t river_launch_head_batched(const DecodeArgs& a, f16* xn, hipStream_t st,
                                     void (*timer)(void*, int, int), void* tctx, int top) {
  hipLaunchKernelGGL((k_b_prep<2>), dim3(a.dm.B), dim3(kBlock), 0, st, a, a.dm.L, 0, xn);
  if (timer && top == TOP_LM) timer(tctx, TOP_LM, 0);
  hipError_t e = launch_b_gemm<OP_LM>(a, a.dm.L + 1, 0, xn, st);
  if (timer && top == TOP_LM) timer(tctx, TOP_LM, 1);
  if (e != hipSuccess) return e;
  return river_launch_step_end(a, st);
}

// One batched decode step (mode 0 early exit, 1 backbone only). `xn` is scratch [B][d].
hipError_t river_decode_layers_batched(const DecodeArgs& a, f16* xn, int mode, hipStream_t st,
                                       void (*timer)(void*, int, int), void* tctx, int top) {
  hipError_t e;
  auto T = [&](int o, int phase) {
    if (timer && o == top) timer(tctx, o, phase);
  };
  const Dims& dm = a.dm;
  for (int l = 1; l <= dm.L; ++l) {
    hipLaunchKernelGGL((k_b_prep<0>), dim3(dm.B), dim3(kBlock), 0, st, a, l, mode, xn);
    T(TOP_QKV, 0);
    if ((e = launch_b_gemm<OP_QKV>(a, l, mode, xn, st)) != hipSuccess) return e;
    T(TOP_QKV, 1);
    T(TOP_ATTN, 0);
    if ((e = river_launch_attn(a, l, st)) != hipSuccess) return e;
    T(TOP_ATTN, 1);
    T(TOP_O, 0);
    if ((e = launch_b_gemm<OP_O>(a, l, mode, a.o, st)) != hipSuccess) return e;
    T(TOP_O, 1);
    hipLaunchKernelGGL((k_b_prep<1>), dim3(dm.B), dim3(kBlock), 0, st, a, l, mode, xn);
    T(TOP_GU, 0);
    if ((e = launch_b_gemm<OP_GU>(a, l, mode, xn, st)) != hipSuccess) return e;
    T(TOP_GU, 1);
    T(TOP_DOWN, 0);
    if ((e = launch_b_gemm<OP_DOWN>(a, l, mode, a.a2, st)) != hipSuccess) return e;
    T(TOP_DOWN, 1);
  }
  return river_launch_head_batched(a, xn, st, timer, tctx, top);
}
