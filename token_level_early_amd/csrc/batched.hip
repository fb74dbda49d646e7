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
// fp32 accumulation; the batch is padded to 16 rows. Every lane feeds 8 K elements of one input
// row (A operand) and of one weight row (B operand) to each MFMA (32 K per instruction). The
// int4 stream turns 8 nibbles into exact fp16 integers (the 0x6400 exponent trick, pairs (0,4),
// (1,5), (2,6), (3,7)), permutes the input the same way, sums one quantisation group on the
// MFMA and applies the fp32 group scale per output column (gate|up and down, symmetric
// group-128: biased codes against an input reordered once per workgroup, see k_b_gemm). The
// waves of a workgroup split K and meet in LDS.
//
// Per layer: k_b_prep (exit test per row, then the attention RMSNorm) -> QKV (RoPE, q and the
// KV append at each row's position) -> attention (the split-K kernel shared with batch 1, one
// grid slice per row) -> O + residual -> gate|up (the MLP RMSNorm in its input staging; a
// k_b_prep kernel where its K is split) + SwiGLU -> down + residual. Head: final RMSNorm, fp16
// LM head with a per-row 64-bit atomic-max argmax, step end.
#include "gemv.hpp"

static constexpr int kBR = 16;  // rows of an MFMA tile (the batch, padded)

typedef _Float16 bh4 __attribute__((ext_vector_type(4)));
typedef float bf4 __attribute__((ext_vector_type(4)));

typedef _Float16 bh8 __attribute__((ext_vector_type(8)));
typedef uint32_t bu4 __attribute__((ext_vector_type(4)));

// 8 fp16 values of a 16-byte load as one 16x16x32 MFMA operand
RIVER_DEV bh8 as8(uint4 u) { return __builtin_bit_cast(bh8, (bu4){u.x, u.y, u.z, u.w}); }

// (w & m) | c in one instruction (v_and_or_b32)
RIVER_DEV uint32_t b_and_or(uint32_t w, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(m), "v"(c));
  return r;
}

// ---------------------------------------------------------------------------------------
// Per-row preparation: KIND 0 = exit test + attention RMSNorm of layer `layer`'s input,
// KIND 1 = MLP RMSNorm of h_mid, KIND 2 = final RMSNorm of h(L). Writes xn[b][d].
// Every load of a row (input, gain, and h(l-2) for the exit test) is issued at once, 16 bytes
// per load, kPP pieces of 8 values per thread held in registers for the norm (rows longer than
// kPP * 8 * kBlock values stream the rest). The fp64 sums run per thread over its pieces in
// order, then over the block in a fixed order.
// ---------------------------------------------------------------------------------------
template <int KIND>
__global__ __launch_bounds__(kBlock) void k_b_prep(DecodeArgs a, int layer, int mode, f16* xn) {
  constexpr int kPP = 4;
  constexpr int kW = kBlock / kWave;
  __shared__ double red[3][kW];
  const Dims& dm = a.dm;
  const int b = blockIdx.x, t = threadIdx.x;
  const int np = dm.d / 8;
  const int step = *a.step;
  const f16* hin;
  const f16* gain;
  const f16* hprev = nullptr;  // KIND 0: h(l-2) when the exit test may run
  int route = ROUTE_BACKBONE, prev = ROUTE_BACKBONE;
  if (KIND == 0) {
    gain = a.layers[layer - 1].attn_norm;
    if (layer == 1) {
      int tok = (step == 0) ? a.tok_in[b] : a.tok_out[(step - 1) * dm.B + b];
      if (tok < 0 || tok >= dm.V) {
        if (t == 0) atomicOr(a.err, ERR_TOKEN);
        tok = 0;
      }
      hin = a.embed + (size_t)tok * dm.d;
      if (t == 0 && a.exit_out) a.exit_out[step * dm.B + b] = dm.L;
      if (a.sim_out)
        for (int i = t; i < dm.L; i += kBlock) a.sim_out[((size_t)step * dm.B + b) * dm.L + i] = __builtin_nanf("");
      if (mode == 0 && a.sched && a.sched[step * dm.B + b] == 0) {  // no backbone block at all
        route = ROUTE_RIVER;
        if (t == 0 && a.exit_out) a.exit_out[step * dm.B + b] = 0;
      }
    } else {
      const int lp = layer - 1;
      hin = a.hs + ((size_t)lp * dm.B + b) * dm.d;
      if (mode == 0) {
        prev = a.route[lp * dm.B + b];
        if (lp >= dm.entry && !a.sched) hprev = a.hs + ((size_t)(lp - 1) * dm.B + b) * dm.d;
      }
    }
  } else if (KIND == 1) {
    hin = a.hmid + ((size_t)(layer - 1) * dm.B + b) * dm.d;
    gain = a.layers[layer - 1].mlp_norm;
  } else {
    hin = a.hs + ((size_t)dm.L * dm.B + b) * dm.d;
    gain = a.final_norm;
  }
  // s2 = |h|^2 (the norm), s0 = h(l-2).h, s1 = |h(l-2)|^2 (the exit test)
  uint4 hv[kPP], gv[kPP], pv[kPP];
#pragma unroll
  for (int m = 0; m < kPP; ++m) {
    const int i = t + m * kBlock, ic = (i < np ? i : 0) * 8;
    hv[m] = ldg16(hin + ic);
    gv[m] = ldg16(gain + ic);
    if (KIND == 0 && hprev) pv[m] = ldg16(hprev + ic);
  }
  double s0 = 0.0, s1 = 0.0, s2 = 0.0;
  auto add = [&](uint4 y, uint4 x, bool both) {
    const f16* hy = (const f16*)&y;
    const f16* hx = (const f16*)&x;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double yv = (double)h2f(hy[e]);
      s2 += yv * yv;
      if (both) {
        const double xv = (double)h2f(hx[e]);
        s0 += xv * yv;
        s1 += xv * xv;
      }
    }
  };
  const bool both = KIND == 0 && hprev != nullptr;
#pragma unroll
  for (int m = 0; m < kPP; ++m)
    if (t + m * kBlock < np) add(hv[m], both ? pv[m] : hv[m], both);
  for (int i = t + kPP * kBlock; i < np; i += kBlock)
    add(ldg16(hin + i * 8), both ? ldg16(hprev + i * 8) : make_uint4(0, 0, 0, 0), both);
  // the three sums over the block at once: waves, then the kW wave totals in order
  s0 = wave_sum_d(s0);
  s1 = wave_sum_d(s1);
  s2 = wave_sum_d(s2);
  if (t % kWave == 0) {
    red[0][t / kWave] = s2;
    red[1][t / kWave] = s0;
    red[2][t / kWave] = s1;
  }
  __syncthreads();
  double n2 = 0.0, dot = 0.0, n1 = 0.0;
#pragma unroll
  for (int j = 0; j < kW; ++j) {
    n2 += red[0][j];
    dot += red[1][j];
    n1 += red[2][j];
  }
  if (KIND == 0) {
    if (layer > 1 && mode == 0) {
      const int lp = layer - 1;
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
        } else {  // cos(h(l-2), h(l-1)) > tau: exit after block l - 1
          const double sim = (n1 > 0.0 && n2 > 0.0) ? dot / sqrt(n1 * n2) : 0.0;
          if (t == 0 && a.sim_out) a.sim_out[((size_t)step * dm.B + b) * dm.L + lp - 1] = (float)sim;
          if (sim > (double)a.tau) route = ROUTE_RIVER;
        }
        if (route == ROUTE_RIVER && t == 0 && a.exit_out) a.exit_out[step * dm.B + b] = lp;
      }
    }
    if (t == 0) a.route[layer * dm.B + b] = route;
  }
  // RMSNorm (1/rms from the fp64 sum of squares), rounded to fp16 like every other path's staging
  const float inv = inv_rms(n2, dm.d, dm.eps);
  f16* out = xn + (size_t)b * dm.d;
  f16* h0 = a.hs + (size_t)b * dm.d;  // KIND 0, first layer: h(0) is the embedding row
  const bool first = KIND == 0 && layer == 1;
#pragma unroll
  for (int m = 0; m < kPP; ++m) {
    const int i = t + m * kBlock;
    if (i < np) {
      *(uint4*)(out + i * 8) = norm8(hv[m], gv[m], inv, true);
      if (first) *(uint4*)(h0 + i * 8) = hv[m];
    }
  }
  for (int i = t + kPP * kBlock; i < np; i += kBlock) {
    const uint4 x = ldg16(hin + i * 8);
    *(uint4*)(out + i * 8) = norm8(x, ldg16(gain + i * 8), inv, true);
    if (first) *(uint4*)(h0 + i * 8) = x;
  }
}

// ---------------------------------------------------------------------------------------
// Batched projection. Workgroup (g, s) of the grid (g < groups, s < S = b_split) stages slice s
// of the input's K range, X[rows][k0 .. k0 + Ks), in LDS once, then computes that slice's part
// of the 16-column tiles g, g + groups, ... of every stream a row runs at this layer. Its 8
// waves split the slice and run one double-buffered weight-load pipeline across all of its
// tiles (the next tile's weights are in flight while a tile's wave partials are summed in LDS
// and its epilogue runs), reading the A operand from LDS: an input read through the caches by
// every wave for every tile holds the weight stream to about half the bandwidth it reaches
// alone. With S > 1, each workgroup stores its partial tile (written through to memory) and
// counts it on the tile's counter; the one that completes the count sums the S partials in
// slice order, so results do not depend on which finishes last, and resets the counter.
// K slots inside one MFMA may be assigned freely as long as both operands agree: the fp16
// stream gives lane (column c, quarter kq) K = base + 32 j + 8 kq + i for MFMA j (each load
// instruction reads 64 contiguous bytes of every weight row), the int4 stream K = base +
// kq * (group / 4) + 8 j + i (each lane reads its nibbles as one contiguous 16-, 8- or 4-byte
// piece). LDS keeps piece p (8 values) of row r at p * 16 + r, so the 64 lanes of one A-operand
// read take 4 consecutive pieces of 16 rows: 1 KB contiguous.
#ifndef RIVER_BG_NB
#define RIVER_BG_NB 1
#endif
#ifndef RIVER_BG_NG
#define RIVER_BG_NG 2
#endif
static constexpr int kGB = 512;  // threads per projection workgroup
static constexpr int kBMaxTiles = 64;  // tiles per workgroup when K is split (b_split keeps to it)
static constexpr int kBMaxSplit = 8;   // K slices of one projection at most
static constexpr int kGW = kGB / kWave;

// WPG: 32-wide K windows per int4 quantisation group (group / 32). ZP: the river copy is in the
// zero-point format (else symmetric: no zero-point loads or input sums). EPI, where a tile's epilogue
// runs: EPI_LOOP as the tile completes (the LM head, whose epilogue loads nothing), EPI_LDS after
// the stream, from tile results kept in LDS (an epilogue's dependent loads inside the loop would
// wait for every weight load in flight), EPI_SPLIT after the stream, by the workgroup that
// completes the tile's slices (b_split > 1).
enum { EPI_LOOP = 0, EPI_LDS = 1, EPI_SPLIT = 2 };
static constexpr int kBDefer = 16;  // tile results a workgroup can keep for EPI_LDS (both streams)
// normin: the input is the raw residual stream after attention (h_mid of this layer) and is
// staged RMS-normalised with the layer's MLP gain, each row's 1/rms computed by every workgroup
// from the whole row in one fixed order (needs an unsplit K: the whole row in LDS).
template <int OP, int WPG, int EPI, bool ZP>
__global__ __launch_bounds__(kGB) void k_b_gemm(DecodeArgs a, int layer, const f16* xin, int streams,
                                                int normin) {
  constexpr bool SPLIT = EPI == EPI_SPLIT;
  __shared__ uint4 xs[kBXs / 8 * kBR];  // the input slice, piece-interleaved
  __shared__ float part[kGW][kBR][kBR];
  __shared__ float ysm[kBR][kBR];
  __shared__ float ytl[EPI == EPI_LDS ? kBDefer : 1][kBR][kBR];
  __shared__ int need[2], nlast, lastf[2 * kBMaxTiles], sroute[kBR];
  // symmetric group-128 river copy, gate|up and down: the int4 stream multiplies biased codes
  // (see below) and starts each group's accumulator from minus its input correction,
  // [group][row / 4][row % 4]. The input is transformed once per workgroup, which pays off only
  // with several tiles per workgroup (QKV and O have one or two).
  constexpr bool BIAS = WPG == 4 && !ZP && (OP == OP_GU || OP == OP_DOWN);
  __shared__ float4 corr[BIAS ? kBXs / 128 : 1][kBR / 4];
  const Dims& dm = a.dm;
  const int t = threadIdx.x, w = t / kWave, lane = t % kWave;
  const int N = b_rows(OP, dm), K = b_k(OP, dm);
  const int tiles = b_tiles(OP, dm), S = SPLIT ? b_split(OP, dm) : 1, Ks = b_slice(OP, dm);
  const int groups = gridDim.x / S, g = blockIdx.x / S, sl = blockIdx.x % S;
  const int k0 = sl * Ks;
  // the layer's weight pointers, read once (left in the table, they would be reloaded inside
  // the streaming loop behind the partial-tile stores, and each reload waits for every load)
  LayerDev lwc{};
  if (OP != OP_LM) lwc = a.layers[layer - 1];
  const LayerDev* lw = &lwc;
  // which streams does any row run at this layer? The routes' load is issued before the
  // staging loads and consumed after them, so that it adds no round trip of its own. need[] is
  // cleared and set by wave 0 alone (in program order), before the barrier that ends staging.
  if (t < 2) need[t] = 0;
  const int rt = (OP == OP_LM) ? ROUTE_BACKBONE : a.route[layer * dm.B + (t < dm.B ? t : 0)];
  // stage the slice (rows past the batch and values past K are zero): every load is issued
  // before the first LDS store (one round trip); workgroups start at different pieces so that
  // they do not all read the same lines at once
  {
    constexpr int kPer = kBXs / 8 * kBR / kGB;
    const int np = Ks / 8 * kBR;
    const int rot = (int)((blockIdx.x * 613u * kBR) % (unsigned)np);
    uint4 v[kPer];
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      int i = t + m * kGB + rot;
      i = i < np ? i : i - np;
      const int pc = i / kBR, r = i % kBR, k = k0 + pc * 8;
      const bool ok = t + m * kGB < np && r < dm.B && k < K;
      const uint4 x = ldg16(xin + (ok ? (size_t)r * K + k : 0));
      v[m] = ok ? x : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      int i = t + m * kGB + rot;
      i = i < np ? i : i - np;
      if (t + m * kGB < np) xs[i] = v[m];
    }
  }
  if (t < dm.B) {
    sroute[t] = rt;  // the epilogues read the routes here
    if (rt >= 0 && rt < streams) atomicOr(&need[rt], 1);
  }
  __syncthreads();
  if (normin) {  // RMSNorm in LDS: fp64 sum of squares per row, thread t of row t % 16 summing
               // pieces t / 16, t / 16 + 32, ... in that order, then the 32 partials in order
    __shared__ double rs[kBR][kGB / kBR];
    __shared__ float rinv[kBR];
    const int r = t % kBR, j0 = t / kBR, np = Ks / 8;
    // this thread's gain pieces, all in flight while the sums are formed
    constexpr int kPer = kBXs / 8 * kBR / kGB;
    uint4 gv[kPer];
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int pc = (t + m * kGB) / kBR;
      gv[m] = ldg16(lwc.mlp_norm + (pc * 8 < K ? pc * 8 : 0));
    }
    double ss = 0.0;
    for (int pc = j0; pc < np; pc += kGB / kBR) ss += sq8(xs[pc * kBR + r]);
    rs[r][j0] = ss;
    __syncthreads();
    if (t < kBR) {
      double tot = 0.0;
      for (int j = 0; j < kGB / kBR; ++j) tot += rs[t][j];
      rinv[t] = inv_rms(tot, K, dm.eps);
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int i = t + m * kGB, pc = i / kBR, row = i % kBR;
      if (i < np * kBR && row < dm.B && pc * 8 < K) xs[i] = norm8(xs[i], gv[m], rinv[row], true);
    }
    __syncthreads();
  }
  const bool need0 = need[0] != 0, need1 = need[1] != 0;

  const int col = lane % 16, kq = lane / 16;
  // tiles of this workgroup: g + i * groups, i < my
  const int my = g < tiles ? (tiles - 1 - g) / groups + 1 : 0;
  bf4 acc = bf4{0.f, 0.f, 0.f, 0.f};

  // epilogue per 16-column tile: thread -> (row b, tile column c), rows on this stream only
  auto epilogue = [&](int stream, int tile, const float (&y)[kBR][kBR], int tt) {
  const int b = tt / kBR, c = tt % kBR;
  if (b >= dm.B) return;
  if (OP != OP_LM && sroute[b] != stream) return;
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

  // sum the waves' parts of the tile in a fixed order; with one slice run the epilogue, else
  // store the slice's partial tile (written through to memory; counted at the end)
  auto finish = [&](int stream, int tile) {
#pragma unroll
    for (int r = 0; r < 4; ++r) part[w][4 * kq + r][col] = acc[r];
    acc = bf4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    if (t < kBR * kBR) {
      const int row = t / kBR, c = t % kBR;
      float y = part[0][row][c];
#pragma unroll
      for (int j = 1; j < kGW; ++j) y += part[j][row][c];
      if constexpr (EPI == EPI_LOOP) {
        ysm[row][c] = y;
      } else if constexpr (EPI == EPI_LDS) {
        ytl[stream * my + (tile - g) / groups][row][c] = y;
      } else {
        float* P = a.bpart + (((size_t)stream * tiles + tile) * S + sl) * (kBR * kBR);
        __hip_atomic_store((g_f32*)P + t, y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    if constexpr (EPI == EPI_LOOP) epilogue(stream, tile, ysm, t);
  };

  if (need0 && my > 0) {  // ---- fp16 backbone stream
    // blocks of 128 K (four 32-wide windows); wave w takes blocks [b0, b1) of the slice in
    // every tile. Its work is a sequence of upt units per tile (a unit is one block; waves
    // with fewer blocks have empty units), loaded NB units per batch, batches double-buffered.
    const int nb = Ks / 128;
    const int b0 = w * nb / kGW, b1 = (w + 1) * nb / kGW;
    constexpr int NB = RIVER_BG_NB;
    const int upt = (nb + kGW - 1) / kGW;  // the same in every wave
    const int U = my * upt, Qb = (U + NB - 1) / NB;
    // loads are unconditional (an in-range address, the value zeroed afterwards): a load behind
    // a branch leaves the compiler unable to count the loads in flight, and it then waits for
    // all of them, the next batch's included
    auto load = [&](int q, uint4 (&wb)[NB][4]) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int unit = q * NB + u;
        const int tile = g + (unit / upt) * groups;
        const int kb = b0 + unit % upt;
        const int n = logical_row(OP, tile, col, kBR, dm);
        const bool nok = unit < U && kb < b1 && n < N;
        const f16* wrow = (OP == OP_LM) ? a.lm_head + (size_t)(nok ? n : 0) * dm.d : f16_row(OP, nok ? n : 0, *lw, a);
        // the raw values stay in the buffer: a unit that is not this wave's reads an in-range
        // address and is cancelled at use through a zero A operand (finite weights times zero)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = k0 + kb * 128 + j * 32 + kq * 8;
          wb[u][j] = ldg16(wrow + ((nok && k < K) ? k : 0));
        }
      }
    };
    auto mma = [&](int q, const uint4 (&wb)[NB][4]) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int unit = q * NB + u;
        if (unit >= U) break;  // the same in every wave
        const int kb = b0 + unit % upt;
        const bool kok = kb < b1;  // values past K are zero in the staged slice
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int pc = (kok ? kb : 0) * 16 + 4 * j + kq;
          const uint4 xv = xs[pc * kBR + col];
          const uint4 xa = kok ? xv : make_uint4(0, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as8(xa), as8(wb[u][j]), acc, 0, 0, 0);
        }
        if (unit % upt == upt - 1) finish(0, g + (unit / upt) * groups);
      }
    };
    // Two register buffers in a ring: one batch's loads are in flight while the other is
    // multiplied. No load sits behind a branch (batches past the end read an in-range address
    // and are discarded), and the stages are fenced from the scheduler: hoisted above the
    // MFMAs that read the buffer it refills, a load would overlap the buffer's old and new
    // values and the loop would copy registers, waiting for every load in flight.
    uint4 wb0[NB][4], wb1[NB][4];
    load(0, wb0);
    for (int q = 0; q < Qb; q += 2) {
      load(q + 1, wb1);
      __builtin_amdgcn_sched_barrier(0);
      mma(q, wb0);
      __builtin_amdgcn_sched_barrier(0);
      load(q + 2, wb0);
      __builtin_amdgcn_sched_barrier(0);
      mma(q + 1, wb1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (need1 && my > 0) {  // ---- int4 river stream
    // one quantisation group per unit: lane reads 8 * WPG contiguous K values, i.e. 4 * WPG
    // bytes of nibbles (rows are padded to whole groups)
    constexpr int G = 32 * WPG;
    const int ng = Ks / G;  // groups of the slice (slices are whole 128-value blocks)
    const int g0 = w * ng / kGW, g1 = (w + 1) * ng / kGW;
    constexpr int NG = RIVER_BG_NG;  // units per batch
    const int upt = (ng + kGW - 1) / kGW;
    const int U = my * upt, Qb = (U + NG - 1) / NG;
    const int grp0 = k0 / G;  // first group of the slice
    // The loader and the multiplier each walk the units in order (every batch is loaded once
    // and multiplied once, both in increasing order): unit (tile index t, unit u of the tile),
    // advanced by counting instead of dividing. The lane's row pointers change once per tile.
    int lt = 0, lu = 0;  // next unit to load
    const uint8_t* rp;
    const f16* sp;
    const uint8_t* zp;  // zero-point format only (else null)
    bool nok;
    auto tile_rows = [&](int ti) {
      const int n = logical_row(OP, g + ti * groups, col, kBR, dm);
      nok = ti < my && n < N;
      w4_row(OP, nok ? n : 0, *lw, dm, rp, sp, zp);
    };
    tile_rows(0);
    auto load = [&](int q, uint32_t (&wq)[NG][WPG], f16 (&sc)[NG], uint8_t (&zc)[NG]) {
      (void)q;
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        const int gs = g0 + lu;  // group within the slice
        const int grp = grp0 + gs;
        const bool gok = nok && gs < g1 && grp * G < K;
        // raw values from in-range addresses (see the fp16 stream); a unit that is not this
        // wave's is cancelled at use through a zero scale
        const int gl = gok ? grp : 0;
        const uint8_t* wp = rp + (gl * G + kq * 8 * WPG) / 2;
        if (WPG == 4) {
          const uint4 v = ldg16(wp);
          wq[u][0] = v.x;
          wq[u][WPG > 1 ? 1 : 0] = v.y;
          wq[u][WPG > 2 ? 2 : 0] = v.z;
          wq[u][WPG > 3 ? 3 : 0] = v.w;
        } else if (WPG == 2) {
          const unsigned long long v = *(const __attribute__((address_space(1))) unsigned long long*)wp;
          wq[u][0] = (uint32_t)v;
          wq[u][WPG > 1 ? 1 : 0] = (uint32_t)(v >> 32);
        } else {
          wq[u][0] = *(const __attribute__((address_space(1))) uint32_t*)wp;
        }
        sc[u] = ldg2(sp + gl);  // scale of (column, group), converted at use
        if constexpr (ZP) zc[u] = *(const __attribute__((address_space(1))) uint8_t*)(zp + gl);
        else zc[u] = 8;
        if (++lu == upt) {
          lu = 0;
          tile_rows(++lt);
        }
      }
    };
    // unpack8 gives q = u - 8; the zero-point format needs u - z = (u - 8) + (8 - z): the group's
    // input sums per batch row come from one more MFMA against a ones operand (they land in the
    // accumulator layout, every column holding its row's sum)
    // A batch in two passes: first the products of all its units, on accumulators of their own
    // with no branch in between (the LDS reads, unpacking and matrix work of different units can
    // then overlap; a unit past the end reads in-range LDS and is dropped), then the scaled
    // accumulation and the tile ends in unit order.
    // BIAS: a nibble u OR-ed into fp16 1024.0 is 1024 + u (low nibble of a byte) or 1024 + 16 u
    // (high nibble) exactly; the staged input was reordered to the same pairs once, its
    // high-nibble elements divided by 16, so a group's product is sum x (u - 8) + C with the
    // per-row constant C = 1032 sum(even x) + 1152 sum(odd x / 16), taken off at the start.
    // Otherwise the codes are unpacked to u - 8 (u - z) and the input reordered per window.
    int mt = 0, mu = 0;  // next unit to multiply
    auto mma = [&](int q, const uint32_t (&wq)[NG][WPG], const f16 (&sc)[NG], const uint8_t (&zc)[NG]) {
      (void)q;
      const bh8 ones = bh8{(f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f, (f16)1.0f};
      bf4 tmp[NG], xsum[NG];
      uint4 xv[NG][WPG];
      float4 cv[NG];
      int pu = mu;  // the batch's units, without advancing the walk yet
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        const int gs0 = g0 + pu;
        pu = pu + 1 == upt ? 0 : pu + 1;
        const int gs = gs0 < g1 ? gs0 : 0;
#pragma unroll
        for (int j = 0; j < WPG; ++j) xv[u][j] = xs[(gs * 4 * WPG + kq * WPG + j) * kBR + col];
        if constexpr (BIAS) cv[u] = corr[gs][kq];
      }
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        if constexpr (BIAS) {
          tmp[u] = bf4{-cv[u].x, -cv[u].y, -cv[u].z, -cv[u].w};
        } else {
          tmp[u] = bf4{0.f, 0.f, 0.f, 0.f};
          xsum[u] = bf4{0.f, 0.f, 0.f, 0.f};
        }
      }
      // windows outer, units inner: consecutive matrix instructions are independent
#pragma unroll
      for (int j = 0; j < WPG; ++j) {
#pragma unroll
        for (int u = 0; u < NG; ++u) {
          if constexpr (BIAS) {
            const uint32_t w = wq[u][j], w8 = w >> 8, mg = 0x64006400u;
            const uint4 b = make_uint4(b_and_or(w, 0x000F000Fu, mg), b_and_or(w, 0x00F000F0u, mg),
                                       b_and_or(w8, 0x000F000Fu, mg), b_and_or(w8, 0x00F000F0u, mg));
            tmp[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as8(xv[u][j]), as8(b), tmp[u], 0, 0, 0);
          } else {
            const uint32_t in[4] = {xv[u][j].x, xv[u][j].y, xv[u][j].z, xv[u][j].w};
            h2 xo[4];
            pair_for_unpack(in, xo);  // (x0,x4) (x1,x5) (x2,x6) (x3,x7)
            const bh8 a8 = __builtin_bit_cast(bh8, (bu4){as_u32(xo[0]), as_u32(xo[1]), as_u32(xo[2]), as_u32(xo[3])});
            if constexpr (ZP) xsum[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a8, ones, xsum[u], 0, 0, 0);
            h2 p0, p1, p2, p3;
            unpack8(wq[u][j], p0, p1, p2, p3);  // (q0,q4) (q1,q5) (q2,q6) (q3,q7)
            const bh8 b8 = __builtin_bit_cast(bh8, (bu4){as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3)});
            tmp[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a8, b8, tmp[u], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        if (mt >= my) break;  // past the last unit (the same in every wave)
        const int gs0 = g0 + mu;
        const bool gv = gs0 < g1 && (grp0 + gs0) * G < K;  // else not this wave's: cancelled
        const float su = gv ? h2f(sc[u]) : 0.f;
        const float zu = 8.f - (float)zc[u];  // zero-point format: 8 - z
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = fmaf(su, ZP ? fmaf(zu, xsum[u][r], tmp[u][r]) : tmp[u][r], acc[r]);
        if (mu == upt - 1) finish(1, g + mt * groups);
        if (++mu == upt) {
          mu = 0;
          ++mt;
        }
      }
    };
    uint32_t wq0[NG][WPG], wq1[NG][WPG];
    f16 sc0[NG], sc1[NG];
    uint8_t zc0[NG], zc1[NG];
    load(0, wq0, sc0, zc0);
    if constexpr (BIAS) {
      // the staged slice, in place (the fp16 stream, if any, is done with it: its last tile
      // ended at a barrier): thread (row r, group gg) reorders the group's 16 pieces of row r to
      // the code pairs, divides its high-nibble elements by 16 and sums both kinds
      for (int pg = t; pg < ng * kBR; pg += kGB) {
        const int r = pg % kBR, gg = pg / kBR;
        float se = 0.f, so = 0.f;
        const h2 s16 = {(f16)0.0625f, (f16)0.0625f};
#pragma unroll 4
        for (int i = 0; i < G / 8; ++i) {
          uint4& x = xs[(gg * (G / 8) + i) * kBR + r];
          const uint4 v = x;
          const h2 e0 = as_h2(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u));  // x0 | x4<<16
          const h2 o0 = as_h2(__builtin_amdgcn_perm(v.z, v.x, 0x07060302u)) * s16;  // x1, x5
          const h2 e1 = as_h2(__builtin_amdgcn_perm(v.w, v.y, 0x05040100u));  // x2, x6
          const h2 o1 = as_h2(__builtin_amdgcn_perm(v.w, v.y, 0x07060302u)) * s16;  // x3, x7
          se += (h2f(e0.x) + h2f(e0.y)) + (h2f(e1.x) + h2f(e1.y));
          so += (h2f(o0.x) + h2f(o0.y)) + (h2f(o1.x) + h2f(o1.y));
          x = make_uint4(as_u32(e0), as_u32(o0), as_u32(e1), as_u32(o1));
        }
        ((float*)&corr[gg][0])[r] = 1032.f * se + 1152.f * so;
      }
      __syncthreads();
    }
    for (int q = 0; q < Qb; q += 2) {  // the ring, as in the fp16 stream
      load(q + 1, wq1, sc1, zc1);
      __builtin_amdgcn_sched_barrier(0);
      mma(q, wq0, sc0, zc0);
      __builtin_amdgcn_sched_barrier(0);
      load(q + 2, wq0, sc0, zc0);
      __builtin_amdgcn_sched_barrier(0);
      mma(q + 1, wq1, sc1, zc1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (EPI == EPI_LOOP || my == 0) return;
  if constexpr (EPI == EPI_LDS) {  // wave w runs the epilogues of kept tiles w, w + 8, ...
    for (int i = w; i < 2 * my; i += kGW) {
      const int stream = i / my;
      if (stream == 0 ? need0 : need1) {
#pragma unroll
        for (int m = 0; m < 4; ++m) epilogue(stream, g + (i % my) * groups, ytl[i], lane + m * kWave);
      }
    }
    return;
  }
  // ---- slices: every partial of this workgroup has been written through once its stores are
  // acknowledged; then count them, and finish the tiles whose count this workgroup completed
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t < 2 * my) {
    const int stream = t / my, tile = g + (t % my) * groups;
    int mine = 0;
    if (stream == 0 ? need0 : need1) {
      uint32_t* cn = a.bcnt + (size_t)stream * tiles + tile;
      const uint32_t done = __hip_atomic_fetch_add(cn, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      mine = done == (uint32_t)(S - 1);
      if (mine) __hip_atomic_store(cn, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    lastf[t] = mine;
  }
  __syncthreads();
  if (t == 0) {  // compact the list of tiles to finish
    int n = 0;
    for (int i = 0; i < 2 * my; ++i)
      if (lastf[i]) lastf[n++] = i;
    nlast = n;
  }
  __syncthreads();
  // wave w sums the slices of tiles w, w + 8, ... of the list into its own LDS tile (the input
  // slice is no longer needed), then all waves run the epilogues
  float(*yt)[kBR][kBR] = (float(*)[kBR][kBR])xs;
  for (int r0 = 0; r0 < nlast; r0 += kGW) {
    const int i = r0 + w;
    if (i < nlast) {
      const int stream = lastf[i] / my, tile = g + (lastf[i] % my) * groups;
      const float* P = a.bpart + ((size_t)stream * tiles + tile) * S * (kBR * kBR);
      // all S x 4 loads in flight at once, summed in slice order
      float pv[kBMaxSplit][4];
#pragma unroll
      for (int j = 0; j < kBMaxSplit; ++j)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          pv[j][m] = __hip_atomic_load((g_f32*)P + (j < S ? j : 0) * (kBR * kBR) + lane + m * kWave,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int e = lane + m * kWave;
        float v = pv[0][m];
#pragma unroll
        for (int j = 1; j < kBMaxSplit; ++j)
          if (j < S) v += pv[j][m];
        yt[w][e / kBR][e % kBR] = v;
      }
    }
    __syncthreads();
    if (i < nlast) {
      const int stream = lastf[i] / my, tile = g + (lastf[i] % my) * groups;
#pragma unroll
      for (int m = 0; m < 4; ++m) epilogue(stream, tile, yt[w], lane + m * kWave);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------------------
hipError_t river_launch_attn(const DecodeArgs& a, int layer, hipStream_t st);
hipError_t river_launch_step_end(const DecodeArgs& a, hipStream_t st);

template <int OP>
static hipError_t launch_b_gemm(const DecodeArgs& a, int layer, int mode, const f16* xin, hipStream_t st,
                                int normin = 0) {
  const Dims& dm = a.dm;
  const int streams = (OP == OP_LM || mode == 1) ? 1 : 2;
  const int S = b_split(OP, dm), groups = b_groups(OP, dm);
  if (S > kBMaxSplit || (S > 1 && (b_tiles(OP, dm) + groups - 1) / groups > kBMaxTiles)) return hipErrorInvalidValue;
  if (normin && S > 1) return hipErrorInvalidValue;  // normalising while staging needs whole rows
  const dim3 grid(groups * S), block(kGB);
  const int wpg = dm.group / 32;
  const int my = (b_tiles(OP, dm) + groups - 1) / groups;  // tiles per workgroup at most
  const int epi = S > 1 ? EPI_SPLIT : (OP == OP_LM || 2 * my > kBDefer) ? EPI_LOOP : EPI_LDS;
#define RIVER_B_LAUNCH2(E, Z)                                                                          \
  do {                                                                                               \
    if (wpg == 1) hipLaunchKernelGGL((k_b_gemm<OP, 1, E, Z>), grid, block, 0, st, a, layer, xin, streams, normin); \
    else if (wpg == 2) hipLaunchKernelGGL((k_b_gemm<OP, 2, E, Z>), grid, block, 0, st, a, layer, xin, streams, normin); \
    else hipLaunchKernelGGL((k_b_gemm<OP, 4, E, Z>), grid, block, 0, st, a, layer, xin, streams, normin);       \
  } while (0)
#define RIVER_B_LAUNCH(E)                  \
  do {                                     \
    if (dm.zp) RIVER_B_LAUNCH2(E, true);   \
    else RIVER_B_LAUNCH2(E, false);        \
  } while (0)
  if (epi == EPI_SPLIT) RIVER_B_LAUNCH(EPI_SPLIT);
  else if (epi == EPI_LDS) RIVER_B_LAUNCH(EPI_LDS);
  else RIVER_B_LAUNCH(EPI_LOOP);
#undef RIVER_B_LAUNCH
#undef RIVER_B_LAUNCH2
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
    // the MLP RMSNorm runs in gate|up's staging when its K is not split, else as its own kernel
    const bool fuse = b_split(OP_GU, dm) == 1;
    if (!fuse) hipLaunchKernelGGL((k_b_prep<1>), dim3(dm.B), dim3(kBlock), 0, st, a, l, mode, xn);
    T(TOP_GU, 0);
    if (fuse) e = launch_b_gemm<OP_GU>(a, l, mode, a.hmid + (size_t)(l - 1) * dm.B * dm.d, st, 1);
    else e = launch_b_gemm<OP_GU>(a, l, mode, xn, st);
    if (e != hipSuccess) return e;
    T(TOP_GU, 1);
    T(TOP_DOWN, 0);
    if ((e = launch_b_gemm<OP_DOWN>(a, l, mode, a.a2, st)) != hipSuccess) return e;
    T(TOP_DOWN, 1);
  }
  return river_launch_head_batched(a, xn, st, timer, tctx, top);
}
