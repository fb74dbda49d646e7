// Prompt prefill with a sequence-level exit (paperlayer.ai summary of arXiv 2604.18396v3,
// section 4 "Inference with Seamless Exit": prefill exits per sequence, generation per token;
// section 3 "Sequence-level Exit": the latest-exiting token sets the sequence's depth).
//
// Layer by layer over all B*P prompt rows:
//   RMSNorm -> QKV GEMM -> RoPE + KV write (positions 0..P-1 of the shared cache) -> causal
//   attention -> O GEMM + residual -> RMSNorm -> gate|up GEMM -> SwiGLU -> down GEMM + residual
//   -> per-token cos(h_t(l-1), h_t(l)) -> per-sequence exit decision (min over tokens > tau).
// A sequence on the river runs the int4 copy of the remaining blocks; both write the same KV.
//
// GEMMs use MFMA (v_mfma_f32_16x16x16_f16): 128x128 output tiles, 4 waves of 64x64. The int4
// copy is unpacked to exact fp16 codes q in LDS and each k-tile's product is scaled by the
// fp32 group scale of its column, so river rows compute sum_g s_g * sum_{k in g} q_k x_k.
#include "params.hpp"

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

enum { EPI_STORE = 0, EPI_RESID = 1 };

struct PfGemmArgs {
  const f16* A;  // [M][K] activations
  int M, N, K;
  // fp16 weights: up to three row segments [seg_start[i], seg_start[i+1]) -> seg_ptr[i]
  const f16* seg_ptr[3];
  int seg_start[4];
  // int4 weights (device layout)
  const uint8_t* w4;
  const f16* s4;
  const uint8_t* z4;  // zero-point format: zero points (else null)
  int group;
  // per-row route filter: row m belongs to sequence m / P; computed only if route matches
  const int* seq_route;  // [B]
  int P;
  int want_route;
  // epilogue
  f16* C;  // [M][N]
  const f16* R;  // residual [M][N] (EPI_RESID)
  int epi;
  // C_GLOBAL / R_GLOBAL: C or R is the whole residual stream, whose row for chunk-local row m
  // is (m / P) * Ptot + t0 + m % P
  int c_global, r_global, Ptot, t0;
};

// Residual-stream row of chunk-local row m (chunks of Ce positions from t0, prompts of P).
RIVER_DEV int64_t pf_row(int m, int Ce, int t0, int P) { return (int64_t)(m / Ce) * P + t0 + m % Ce; }

// ---------------------------------------------------------------------------------------
// Prompt GEMM on CDNA4's 16x16x32 fp16 MFMA: 128 x 128 output tiles, K in steps of 64 staged
// through a double-buffered LDS tile pair (the next step's global loads are in flight while the
// current one runs on the matrix cores; one barrier per step; the global loads run two steps
// ahead through two register sets). 4 waves of 64 x 64. The int4
// river tile is unpacked into LDS as the exact fp16 integers u - z (z = 8 for the symmetric
// format), and each step's product is scaled by the fp32 group scale of its column: a step of
// SG = 64 positions (32 when group = 32) lies inside one quantisation group.
// ---------------------------------------------------------------------------------------
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
static constexpr int QBM = 128, QBN = 128, QBK = 64, QLD = QBK;
// LDS tiles are 128-byte rows with no padding; 16-byte chunk c of row r sits at chunk
// c ^ ((r >> 1) & 7). A fragment read (16 rows, the same chunk, then the next chunk for the next
// 16 lanes) and a tile store (8 chunks of consecutive rows) then touch every bank once per
// 16 lanes on 64 banks and per 32 lanes on 128 banks (with the plain padded row, the stores and
// the wider read groups collided).
RIVER_DEV int qsw(int r, int k) { return ((((k >> 3) ^ (r >> 1)) & 7) << 3) | (k & 7); }

template <int MODE, int SG, bool IN = false>
__global__ __launch_bounds__(kBlock, MODE == 0 ? 2 : 1) void k_pf_gemm2(PfGemmArgs g) {
  __shared__ __attribute__((aligned(16))) f16 As[2][QBM][QLD];
  __shared__ __attribute__((aligned(16))) f16 Bs[2][QBN][QLD];
  const int m0 = blockIdx.y * QBM, n0 = blockIdx.x * QBN;
  {  // skip tiles whose rows all belong to sequences on the other route
    const int mlast = min(g.M, m0 + QBM) - 1;
    bool any = false;
    for (int sq = m0 / g.P; sq <= mlast / g.P; ++sq) any |= (g.seq_route[sq] == g.want_route);
    if (!any) return;
  }
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int wm = (w / 2) * 64, wn = (w % 2) * 64;
  const int64_t rb4 = w4_row_bytes(g.K), rs4 = w4_row_scales(g.K, g.group);
  f4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f4){0.f, 0.f, 0.f, 0.f};

  // loaders: A (and fp16 B) tiles are 128 rows x 64 halves = 1024 chunks of 16 B, thread t
  // takes chunks t + 256 i (row c / 8, halves (c % 8) * 8); an int4 B tile is 128 rows x 32 B,
  // thread t takes row t / 2, bytes (t % 2) * 16 (32 consecutive k)
  const f16* brow[4];
  if (MODE == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + (tid + 256 * i) / 8;
      int si = 0;
      while (si < 2 && n >= g.seg_start[si + 1]) ++si;
      brow[i] = (n < g.N) ? g.seg_ptr[si] + (size_t)(n - g.seg_start[si]) * g.K : nullptr;
    }
  }
  // one K step's global data of this thread, held in registers until it is stored to LDS
  struct Regs {
    uint4 a[4], b[4];
    uint4 q;
    f16 dz;
  };
  auto gload = [&](Regs& R, int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c / 8, k = k0 + (c % 8) * 8;
      const int m = m0 + r;
      R.a[i] = (m < g.M && k < g.K) ? *(const uint4*)(g.A + (size_t)m * g.K + k) : make_uint4(0, 0, 0, 0);
      if (MODE == 0) R.b[i] = (brow[i] && k < g.K) ? *(const uint4*)(brow[i] + k) : make_uint4(0, 0, 0, 0);
    }
    if (MODE == 1) {
      const int n = n0 + tid / 2, k = k0 + (tid % 2) * 32;
      R.q = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
      R.dz = (f16)0.0f;
      if (n < g.N && k < g.K) {
        R.q = *(const uint4*)(g.w4 + (size_t)n * rb4 + k / 2);
        if (g.z4) R.dz = (f16)(8.0f - (float)g.z4[(size_t)n * rs4 + k / g.group]);
      }
    }
  };
  // IN (fp16 weights; M, N and K multiples of the tile and step, so every tile is in range):
  // no bounds tests, hence no branches around the loads, and the wait before a step's LDS
  // stores then covers only that step's loads (the next step's stay in flight)
  static_assert(!IN || MODE == 0, "in-range variant: fp16 weights only");
  // Operands as scalar tile bases plus one 32-bit lane offset shared by A and B (a tile never
  // straddles two weight segments: their starts are multiples of the tile), so the addresses
  // hold one vector register; native vectors (arrays of HIP's uint4 wrapper were left in
  // private memory here).
  int si0 = 0;
  while (si0 < 2 && n0 >= g.seg_start[si0 + 1]) ++si0;
  const char* const At = (const char*)(g.A + (size_t)m0 * g.K);
  const char* const Bt = (const char*)(g.seg_ptr[si0] + (size_t)(n0 - g.seg_start[si0]) * g.K);
  const uint32_t loff = (uint32_t)((tid / 8) * g.K + (tid % 8) * 8) * 2u;
  auto gload_in = [&](h8 (&a)[4], h8 (&b)[4], int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t u = ((size_t)32 * i * g.K + k0) * 2;  // rows 32 i.., columns k0..
      a[i] = *(const h8*)(At + u + loff);
      b[i] = *(const h8*)(Bt + u + loff);
    }
  };
  auto lstore_in = [&](const h8 (&a)[4], const h8 (&b)[4], int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c / 8, kc = (c % 8) * 8;
      *(h8*)&As[buf][r][qsw(r, kc)] = a[i];
      *(h8*)&Bs[buf][r][qsw(r, kc)] = b[i];
    }
  };
  auto lstore = [&](const Regs& R, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c / 8, kc = (c % 8) * 8;
      *(uint4*)&As[buf][r][qsw(r, kc)] = R.a[i];
      if (MODE == 0) *(uint4*)&Bs[buf][r][qsw(r, kc)] = R.b[i];
    }
    if (MODE == 1) {
      const uint32_t wd[4] = {R.q.x, R.q.y, R.q.z, R.q.w};
      const h2 d2 = {R.dz, R.dz};  // zero-point format: u - 8 + (8 - z), exact small integers
      const int br = tid / 2;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        h2 p0, p1, p2, p3;
        unpack8(wd[h], p0, p1, p2, p3);  // pairs (q0,q4),(q1,q5),(q2,q6),(q3,q7)
        p0 += d2; p1 += d2; p2 += d2; p3 += d2;
        h8 v;
        v[0] = p0.x; v[1] = p1.x; v[2] = p2.x; v[3] = p3.x;
        v[4] = p0.y; v[5] = p1.y; v[6] = p2.y; v[7] = p3.y;
        *(h8*)&Bs[buf][br][qsw(br, (tid % 2) * 32 + h * 8)] = v;
      }
    }
  };
  // column scales of this lane's 4 tiles for the step starting at k0 (MODE 1)
  auto scales = [&](int k0, float (&sc)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn + j * 16 + lane % 16;
      sc[j] = (n < g.N) ? h2f(g.s4[(size_t)n * rs4 + k0 / g.group]) : 0.f;
    }
  };
  auto compute = [&](int cur, int kt) {
    float sc[2][4];
    if (MODE == 1) {
      scales(kt * QBK, sc[0]);
      if (SG == 32) scales(kt * QBK + 32, sc[1]);
    }
    f4 tmp[4][4];
    // both 32-wide halves' fragments are read first: the second half's LDS reads overlap the
    // first half's matrix work
    h8 afs[2][4], bfs[2][4];
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm + i * 16 + lane % 16;
        afs[hk][i] = *(const h8*)&As[cur][r][qsw(r, hk * 32 + 8 * (lane / 16))];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn + j * 16 + lane % 16;
        bfs[hk][j] = *(const h8*)&Bs[cur][r][qsw(r, hk * 32 + 8 * (lane / 16))];
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads together, ahead of the products
#pragma unroll
    for (int kk = 0; kk < QBK; kk += 32) {
      const h8(&af)[4] = afs[kk / 32];
      const h8(&bf)[4] = bfs[kk / 32];
      if (MODE == 1 && (SG == 32 || kk == 0)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) tmp[i][j] = (f4){0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (MODE == 0)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
          else
            tmp[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], tmp[i][j], 0, 0, 0);
        }
      if (MODE == 1 && (SG == 32 || kk == 32)) {
        const float* s = sc[(SG == 32 && kk == 32) ? 1 : 0];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] += s[j] * tmp[i][j];
      }
    }
  };
  // Two register sets alternate: step kt+1's data waits in one while step kt+2's loads land in
  // the other, so every load has two steps of matrix work to arrive behind.
  const int nk = (g.K + QBK - 1) / QBK;
  Regs r0, r1;
  if constexpr (IN) {
    // the last two steps reload the final K step instead of skipping their loads (the values
    // are never stored), so every iteration issues the same loads
    h8 a0[4], b0[4], a1[4], b1[4];
    gload_in(a0, b0, 0);
    lstore_in(a0, b0, 0);
    gload_in(a1, b1, min(1, nk - 1) * QBK);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      gload_in(a0, b0, min(kt + 2, nk - 1) * QBK);
      compute(0, kt);
      if (kt + 1 < nk) lstore_in(a1, b1, 1);
      __syncthreads();
      if (kt + 1 >= nk) break;
      gload_in(a1, b1, min(kt + 3, nk - 1) * QBK);
      compute(1, kt + 1);
      if (kt + 2 < nk) lstore_in(a0, b0, 0);
      __syncthreads();
    }
  } else {
    gload(r0, 0);
    lstore(r0, 0);
    if (nk > 1) gload(r1, QBK);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      if (kt + 2 < nk) gload(r0, (kt + 2) * QBK);
      compute(0, kt);
      if (kt + 1 < nk) lstore(r1, 1);
      __syncthreads();
      if (kt + 1 >= nk) break;
      if (kt + 3 < nk) gload(r1, (kt + 3) * QBK);
      compute(1, kt + 1);
      if (kt + 2 < nk) lstore(r0, 0);
      __syncthreads();
    }
  }
  // epilogue: D[i][j] at row 4*(lane/16)+r, column lane%16 of each 16x16 block
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn + j * 16 + lane % 16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm + i * 16 + 4 * (lane / 16) + r;
        if (m < g.M && n < g.N && g.seq_route[m / g.P] == g.want_route) {
          const f16 v = f2h(acc[i][j][r]);
          const int64_t cm = g.c_global ? pf_row(m, g.P, g.t0, g.Ptot) : m;
          if (g.epi == EPI_STORE) {
            g.C[cm * g.N + n] = v;
          } else {
            const int64_t rm = g.r_global ? pf_row(m, g.P, g.t0, g.Ptot) : m;
            g.C[cm * g.N + n] = f2h(h2f(g.R[rm * g.N + n]) + h2f(v));
          }
        }
      }
    }
}

// ---------------------------------------------------------------------------------------
// Elementwise prefill kernels (one workgroup per row unless stated)
// ---------------------------------------------------------------------------------------

__global__ __launch_bounds__(kBlock) void k_pf_embed(PfArgs p) {
  const int m = blockIdx.x;
  int tok = p.tokens[m];
  if (tok < 0 || tok >= p.dm.V) {
    if (threadIdx.x == 0) atomicOr(p.err, ERR_TOKEN);
    tok = 0;
  }
  const f16* src = p.embed + (size_t)tok * p.dm.d;
  for (int i = threadIdx.x; i < p.dm.d; i += kBlock) p.hin[(size_t)m * p.dm.d + i] = src[i];
}

// out[m] = fp16(x[m] / sqrt(mean(x[m]^2) + eps) * w); with gP > 0 x is the residual stream and
// its row is the global row of chunk-local row m (chunks of gCe positions from gt0)
__global__ __launch_bounds__(kBlock) void k_pf_rmsnorm(const f16* x, const f16* w, f16* out, int n,
                                                       float eps, int gP, int gCe, int gt0) {
  __shared__ double red[4];
  const int m = blockIdx.x;
  const f16* xr = x + (gP > 0 ? pf_row(m, gCe, gt0, gP) : (int64_t)m) * n;
  f16* orow = out + (size_t)m * n;
  if ((n & 7) == 0) {  // 16-byte pieces (rows start 16-byte aligned)
    double s = 0.0;
    for (int i = threadIdx.x * 8; i < n; i += kBlock * 8) {
      const uint4 v = *(const uint4*)(xr + i);
      const f16* v8 = (const f16*)&v;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double d = (double)h2f(v8[j]);
        s += d * d;
      }
    }
    s = block_sum_d(s, red);
    const float inv = (float)(1.0 / sqrt(s / n + (double)eps));
    for (int i = threadIdx.x * 8; i < n; i += kBlock * 8) {
      const uint4 v = *(const uint4*)(xr + i), g = *(const uint4*)(w + i);
      const f16* v8 = (const f16*)&v;
      const f16* g8 = (const f16*)&g;
      uint4 o;
      f16* o8 = (f16*)&o;
#pragma unroll
      for (int j = 0; j < 8; ++j) o8[j] = f2h(h2f(v8[j]) * inv * h2f(g8[j]));
      *(uint4*)(orow + i) = o;
    }
    return;
  }
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += kBlock) {
    const double v = (double)h2f(xr[i]);
    s += v * v;
  }
  s = block_sum_d(s, red);
  const float inv = (float)(1.0 / sqrt(s / n + (double)eps));
  for (int i = threadIdx.x; i < n; i += kBlock) orow[i] = f2h(h2f(xr[i]) * inv * h2f(w[i]));
}

// RoPE on q and k rows of qkv; q -> act [M][H*D]; k, v -> shared cache at (layer, b, kvh, t).
__global__ __launch_bounds__(kBlock) void k_pf_rope_kv(PfArgs p, int layer) {
  const Dims& dm = p.dm;
  const int m = blockIdx.x;  // chunk-local row
  const int b = m / p.Ce, t = p.t0 + m % p.Ce;
  const f16* row = p.qkv + (size_t)m * dm.nqkv;
  const int half = dm.D / 2;
  const size_t cache_row = (size_t)dm.Tmax * dm.D;
  if ((half & 7) == 0 && (dm.nqkv & 7) == 0) {
    // 8 consecutive pairs (i, i + half) per thread, 16-byte pieces (the same arithmetic)
    const int pw = half / 8;
    for (int idx = threadIdx.x; idx < (dm.H + dm.Hkv) * pw; idx += kBlock) {
      const int head = idx / pw, i0 = (idx % pw) * 8;
      const uint4 av = *(const uint4*)(row + head * dm.D + i0);
      const uint4 bv = *(const uint4*)(row + head * dm.D + i0 + half);
      const f16* a8 = (const f16*)&av;
      const f16* b8 = (const f16*)&bv;
      const float2* cs = p.rope + (size_t)t * half + i0;
      uint4 o0, o1;
      f16* r0 = (f16*)&o0;
      f16* r1 = (f16*)&o1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x0 = h2f(a8[j]), x1 = h2f(b8[j]);
        const float2 c = cs[j];
        r0[j] = f2h(x0 * c.x - x1 * c.y);
        r1[j] = f2h(x1 * c.x + x0 * c.y);
      }
      f16* dst;
      if (head < dm.H) {
        dst = p.act + (size_t)m * dm.hd + head * dm.D;
      } else {
        dst = p.kv + ((((size_t)(layer - 1) * 2 + 0) * dm.B + b) * dm.Hkv + (head - dm.H)) * cache_row +
              (size_t)t * dm.D;
        kv_count(p.kvcnt, p.kv, dst + i0, 8);
        kv_count(p.kvcnt, p.kv, dst + i0 + half, 8);
      }
      *(uint4*)(dst + i0) = o0;
      *(uint4*)(dst + i0 + half) = o1;
    }
    for (int idx = threadIdx.x; idx < dm.Hkv * dm.D / 8; idx += kBlock) {
      const int kvh = idx / (dm.D / 8), i0 = (idx % (dm.D / 8)) * 8;
      f16* vd = p.kv + ((((size_t)(layer - 1) * 2 + 1) * dm.B + b) * dm.Hkv + kvh) * cache_row + (size_t)t * dm.D;
      *(uint4*)(vd + i0) = *(const uint4*)(row + (dm.H + dm.Hkv) * dm.D + kvh * dm.D + i0);
      kv_count(p.kvcnt, p.kv, vd + i0, 8);
    }
    return;
  }
  const int npairs = (dm.H + dm.Hkv) * half;
  for (int idx = threadIdx.x; idx < npairs; idx += kBlock) {
    const int head = idx / half, i = idx % half;
    const float x0 = h2f(row[head * dm.D + i]), x1 = h2f(row[head * dm.D + i + half]);
    const float2 cs = p.rope[(size_t)t * half + i];
    const f16 r0 = f2h(x0 * cs.x - x1 * cs.y), r1 = f2h(x1 * cs.x + x0 * cs.y);
    if (head < dm.H) {
      f16* qd = p.act + (size_t)m * dm.hd + head * dm.D;
      qd[i] = r0;
      qd[i + half] = r1;
    } else {
      const int kvh = head - dm.H;
      f16* kd = p.kv + ((((size_t)(layer - 1) * 2 + 0) * dm.B + b) * dm.Hkv + kvh) *
                           (size_t)dm.Tmax * dm.D + (size_t)t * dm.D;
      kd[i] = r0;
      kd[i + half] = r1;
      kv_count(p.kvcnt, p.kv, kd + i, 1);
      kv_count(p.kvcnt, p.kv, kd + i + half, 1);
    }
  }
  const int nv = dm.Hkv * dm.D;
  for (int idx = threadIdx.x; idx < nv; idx += kBlock) {
    const int kvh = idx / dm.D, i = idx % dm.D;
    f16* vd = p.kv + ((((size_t)(layer - 1) * 2 + 1) * dm.B + b) * dm.Hkv + kvh) *
                         (size_t)dm.Tmax * dm.D + (size_t)t * dm.D;
    vd[i] = row[(dm.H + dm.Hkv) * dm.D + idx];
    kv_count(p.kvcnt, p.kv, vd + i, 1);
  }
}

// Causal attention. Workgroup = (query block, kv head, sequence). 16 lanes per (query, head);
// QB = 16/G queries x G heads per workgroup; K/V tiles of 64 positions staged in LDS.
// Causal GQA prompt attention on MFMA (flash-attention style). Workgroup = one KV head and
// 32 query positions; wave g handles query head kvh*G + g, so a staged K/V tile serves all G
// heads of the group. Per 64-key tile: S^T = K Q^T (v_mfma_f32_16x16x16_f16, fp32), causal mask,
// online softmax in the exp2 domain, then O^T += V^T P^T with P rounded to fp16. Computing the
// transposes puts each lane on one query column, so the softmax state and the rescale of the
// output accumulators are per-lane scalars and the probabilities come out of the score
// accumulators already in the operand layout of the second product. The exact result is
// softmax(q K^T / sqrt(D)) V over positions 0..t (the prompt attention every block runs).
template <int D, int G>
__global__ __launch_bounds__(G * kWave) void k_pf_fattn(PfArgs p, int layer) {
  constexpr int KT = 64, QW = 32;
  constexpr int NK = D / 16;  // 16-wide steps over the head dimension
  __shared__ f16 Ks[KT][D + 8];   // [key][dim]
  __shared__ f16 Vt[D][KT + 8];   // [dim][key]
  const Dims& dm = p.dm;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int q0 = p.t0 + blockIdx.x * QW;  // queries: positions of the current chunk
  const int tend = p.t0 + p.Ce;
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int lr = lane % 16, lq = lane / 16;
  const int h = kvh * G + w;
  const size_t hs = (size_t)dm.Tmax * D;
  const f16* Kb = p.kv + ((((size_t)(layer - 1) * 2 + 0) * dm.B + b) * dm.Hkv + kvh) * hs;
  const f16* Vb = p.kv + ((((size_t)(layer - 1) * 2 + 1) * dm.B + b) * dm.Hkv + kvh) * hs;
  const float qs = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(D)

  // Q^T operand: lane supplies Q[q = q0 + qb*16 + lr][dims ks*16 + 4*lq .. +3]
  h4 qf[2][NK];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int t = q0 + qb * 16 + lr;
    const f16* qrow = p.act + ((size_t)b * p.Ce + (t < tend ? t - p.t0 : 0)) * dm.hd + (size_t)h * D;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      h4 v = *(const h4*)(qrow + ks * 16 + 4 * lq);
      if (t >= tend) v = (h4){0, 0, 0, 0};
      qf[qb][ks] = v;
    }
  }
  f4 o[NK][2];  // O^T: lane holds dims db*16 + 4*lq + r of query qb*16 + lr
#pragma unroll
  for (int db = 0; db < NK; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) o[db][qb] = (f4){0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-__builtin_inff(), -__builtin_inff()};
  float lsum[2] = {0.f, 0.f};  // this lane's share of the softmax denominator

  const int kend = min(tend, q0 + QW);  // keys [0, kend) can be visible to this block
  for (int k0 = 0; k0 < kend; k0 += KT) {
    __syncthreads();
    for (int idx = tid; idx < KT * D / 8; idx += G * kWave) {
      const int r = idx / (D / 8), c = (idx % (D / 8)) * 8;
      uint4 kv4 = make_uint4(0, 0, 0, 0), vv4 = make_uint4(0, 0, 0, 0);
      if (k0 + r < kend) {
        kv4 = *(const uint4*)(Kb + (size_t)(k0 + r) * D + c);
        vv4 = *(const uint4*)(Vb + (size_t)(k0 + r) * D + c);
      }
      *(uint4*)&Ks[r][c] = kv4;
      const f16* vh = (const f16*)&vv4;
#pragma unroll
      for (int i = 0; i < 8; ++i) Vt[c + i][r] = vh[i];
    }
    __syncthreads();
    // S^T[key][q] for 4 key blocks x 2 query blocks
    f4 sc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) sc[kb][qb] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const h4 kf = *(const h4*)&Ks[kb * 16 + lr][ks * 16 + 4 * lq];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          sc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x16f16(kf, qf[qb][ks], sc[kb][qb], 0, 0, 0);
      }
    }
    // mask, tile max per query column, online rescale
    h4 pf[4][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int t = q0 + qb * 16 + lr;
      float mt = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + kb * 16 + 4 * lq + r;
          const float v = (key <= t && key < kend) ? sc[kb][qb][r] * qs : -__builtin_inff();
          sc[kb][qb][r] = v;
          mt = fmaxf(mt, v);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 16, kWave));
      mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
      const float mn = fmaxf(mrow[qb], mt);
      const bool live = mn > -__builtin_inff();  // some visible key so far
      const float c = live ? exp2f(mrow[qb] - mn) : 1.f;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        h4 pv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = live ? exp2f(sc[kb][qb][r] - mn) : 0.f;
          pv[r] = (f16)e;
          ps += e;
        }
        pf[kb][qb] = pv;
      }
      lsum[qb] = lsum[qb] * c + ps;
      mrow[qb] = mn;
#pragma unroll
      for (int db = 0; db < NK; ++db) o[db][qb] *= c;
    }
    // O^T[dim][q] += V^T P^T
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int db = 0; db < NK; ++db) {
        const h4 vf = *(const h4*)&Vt[db * 16 + lr][kb * 16 + 4 * lq];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x16f16(vf, pf[kb][qb], o[db][qb], 0, 0, 0);
      }
    }
  }
  // denominators (the four lanes of a query column hold disjoint keys), normalise, store
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = lsum[qb];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    const int t = q0 + qb * 16 + lr;
    if (t < tend) {
      f16* orow = p.attn + ((size_t)b * p.Ce + (t - p.t0)) * dm.hd + (size_t)h * D;
#pragma unroll
      for (int db = 0; db < NK; ++db) {
        h4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (f16)(o[db][qb][r] / l);
        *(h4*)(orow + db * 16 + 4 * lq) = v;
      }
    }
  }
}

// The same prompt attention on CDNA4's 16x16x32 MFMA. K/V tiles of 64 keys flow through two LDS
// stages filled by LDS DMA (global_load_lds_dwordx4: no registers held in flight), one tile
// ahead of the one being multiplied (one barrier per tile). Without registers for staging, the
// kernel fits two waves per SIMD (two workgroups per CU: 64 KB of LDS each at D = 128), and
// the other workgroup's products cover a tile's load. S^T = K Q^T takes 32 head dimensions per
// instruction; O^T += V^T P^T takes 32 keys per instruction, the probabilities coming straight
// from the score accumulators: lane group j holds keys 4j..4j+3 of two consecutive 16-key
// blocks, and V^T is read from the transposed tile with the same key order (a dot product only
// needs both operands to agree on it); V stays key-major in LDS and is read transposed.
// Both tiles are 16-byte chunks with no padding, chunk c of key row k stored at c ^ fK(k)
// (K) or c ^ fV(k) (V): a K fragment read (16 keys, one chunk) and a half-wave's transposing V
// reads (8 keys, one chunk pair) then touch every bank once. A DMA instruction writes 64
// consecutive chunks (lane i at M0 + 16 i), so each lane loads the global chunk that belongs
// at its slot. Keys past the causal end load the last visible key (finite, masked).
// A workgroup takes 16*NQB queries (32): every K/V tile it stages serves them all, so the
// causal prefix is re-read once per 32 queries of a KV head.
// V^T fragments from the key-major V tile with CDNA4's transposing LDS read (ds_read_b64_tr_b16):
// in each group of 16 lanes, lane i receives element i % 4 of the 8-byte pieces that lanes
// 4j + i / 4 address (j = 0..3). Lane r pointing at V[k0 + r / 4][d0 + 4 (r % 4)] therefore
// receives V[k0 + j][d0 + r] for j = 0..3: four consecutive keys of dimension d0 + r, the A
// operand layout of the V^T P^T product.
typedef short vt_s4 __attribute__((ext_vector_type(4)));
// s_waitcnt for vector memory only (at most N outstanding; expcnt and lgkmcnt left free)
template <int N>
RIVER_DEV void pf_vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}
RIVER_DEV h4 vt_read(const f16* p) {
  const vt_s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) vt_s4*)p);
  return __builtin_bit_cast(h4, v);
}

template <int D, int G, int NQB>
__global__ __launch_bounds__(G * kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_pf_fattn2(PfArgs p, int layer) {
  // (two waves per SIMD: at D = 128 the register allocator spills 20 bytes per lane, which
  // costs far less than the latency a second wave hides)
  constexpr int KT = 64, QW = 16 * NQB, NT = G * kWave;
  constexpr int NKS = D / 32;  // 32-wide steps over the head dimension
  constexpr int NDB = D / 16;  // 16-row blocks of O^T
  constexpr int CPR = D / 8;   // 16-byte chunks per key row
  constexpr int NI = KT * CPR / kWave / G;  // DMA instructions per wave per tile and matrix
  static_assert(NI >= 1 && NI * kWave * G == KT * CPR, "tile loads");
  static_assert(D == 128 || D == 64, "swizzles");
  // [key][chunk ^ fK(key)][8] and [key][chunk ^ fV(key)][8], one array per stage: the compiler
  // then sees that the stage being read is not the one the DMA in flight writes (with one array
  // it waits for every DMA before any LDS read)
  __shared__ __attribute__((aligned(16))) f16 Ks0[KT * D];
  __shared__ __attribute__((aligned(16))) f16 Ks1[KT * D];
  __shared__ __attribute__((aligned(16))) f16 Vs0[KT * D];
  __shared__ __attribute__((aligned(16))) f16 Vs1[KT * D];
  auto kst = [&](auto S) -> f16* { return decltype(S)::value == 0 ? Ks0 : Ks1; };
  auto vst = [&](auto S) -> f16* { return decltype(S)::value == 0 ? Vs0 : Vs1; };
  const Dims& dm = p.dm;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int q0 = p.t0 + blockIdx.x * QW;  // queries: positions of the current chunk
  const int tend = p.t0 + p.Ce;
  // the wave index as a scalar: the DMA's LDS addresses (M0) and the head are then scalar
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int lr = lane % 16, lq = lane / 16;
  const int h = kvh * G + w;
  const size_t hs = (size_t)dm.Tmax * D;
  const f16* Kb = p.kv + ((((size_t)(layer - 1) * 2 + 0) * dm.B + b) * dm.Hkv + kvh) * hs;
  const f16* Vb = p.kv + ((((size_t)(layer - 1) * 2 + 1) * dm.B + b) * dm.Hkv + kvh) * hs;
  const float qs = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(D)

  // Q^T operand: lane supplies Q[q = q0 + qb*16 + lr][dims ks*32 + 8*lq .. +8]
  h8 qf[NQB][NKS];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int t = q0 + qb * 16 + lr;
    const f16* qrow = p.act + ((size_t)b * p.Ce + (t < tend ? t - p.t0 : 0)) * dm.hd + (size_t)h * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      h8 v = *(const h8*)(qrow + ks * 32 + 8 * lq);
      if (t >= tend) v = (h8){0, 0, 0, 0, 0, 0, 0, 0};
      qf[qb][ks] = v;
    }
  }
  f4 o[NDB][NQB];  // O^T: lane holds dims db*16 + 4*lq + r of query qb*16 + lr
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) o[db][qb] = (f4){0.f, 0.f, 0.f, 0.f};
  float mrow[NQB], lsum[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    mrow[qb] = -__builtin_inff();
    lsum[qb] = 0.f;  // this lane's share of the softmax denominator
  }  // this lane's share of the softmax denominator

  const int kend = min(tend, q0 + QW);  // keys [0, kend) can be visible to this block
  auto fK = [](int key) { return D == 128 ? (key & 15) : ((key >> 1) & 7); };
  auto fV = [](int key) { return D == 128 ? ((key & 7) << 1) : (((key >> 1) & 3) << 1); };
  // tile at keys k0.. into stage st: instruction j of wave w fills chunks (w NI + j) 64 + lane
  // (scalar tile base + a 32-bit per-lane byte offset: rows past kend - 1 read row kend - 1)
  auto issue = [&](auto S, int k0) {
    f16* const Kd = kst(S);
    f16* const Vd = vst(S);
    const char* const Kt = (const char*)(Kb + (size_t)k0 * D);
    const char* const Vt = (const char*)(Vb + (size_t)k0 * D);
    const int lim = kend - 1 - k0;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int slot = (w * NI + j) * kWave;  // first chunk of this instruction
      const int P = slot + lane, key = P / CPR, pc = P % CPR;
      const uint32_t kr = (uint32_t)min(key, lim);
      const uint32_t ok = (kr * D + (pc ^ fK(key)) * 8) * 2, ov = (kr * D + (pc ^ fV(key)) * 8) * 2;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(Kt + ok),
                                       (__attribute__((address_space(3))) void*)(Kd + slot * 8), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(Vt + ov),
                                       (__attribute__((address_space(3))) void*)(Vd + slot * 8), 16, 0, 0);
    }
  };
  auto compute = [&](auto S, int k0) {
    const f16* const Kc = kst(S);
    const f16* const Vc = vst(S);
    f4 sc[4][NQB];  // S^T[key][q] for 4 key blocks x NQB query blocks
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) sc[kb][qb] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int key = kb * 16 + lr;
        const h8 kf = *(const h8*)&Kc[key * D + ((ks * 4 + lq) ^ fK(key)) * 8];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          sc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[qb][ks], sc[kb][qb], 0, 0, 0);
      }
    }
    // mask, tile max per query column, online rescale. A tile wholly at or below the first
    // query of the block (k0 + KT - 1 <= q0 < kend) is visible to every query of it: it takes
    // no mask, and every column then has a visible key.
    h4 pf[4][NQB];
    auto softmax = [&](auto EDGE) {
      constexpr bool E = decltype(EDGE)::value;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int t = q0 + qb * 16 + lr;
        float mt = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v = sc[kb][qb][r];  // unscaled: the scale is applied with the max below
            if (E) {
              const int key = k0 + kb * 16 + 4 * lq + r;
              v = (key <= t && key < kend) ? v : -__builtin_inff();
            }
            sc[kb][qb][r] = v;
            mt = fmaxf(mt, v);
          }
        mt = fmaxf(mt, __shfl_xor(mt, 16, kWave));
        mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
        // qs > 0 and rounding is monotonic, so mt * qs is the largest of the rounded scaled
        // scores; each exponent is then one fused s * qs - mn
        const float mn = fmaxf(mrow[qb], mt * qs);
        const bool live = !E || mn > -__builtin_inff();  // some visible key so far
        // v_exp_f32 itself: arguments below -126 give 0 instead of a subnormal, which the fp16
        // probabilities and the sums (at least 1 once a key is visible) cannot hold anyway
        const float cf = live ? __builtin_amdgcn_exp2f(mrow[qb] - mn) : 1.f;
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          h4 pv;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = live ? __builtin_amdgcn_exp2f(fmaf(sc[kb][qb][r], qs, -mn)) : 0.f;
            pv[r] = (f16)e;
            ps += e;
          }
          pf[kb][qb] = pv;
        }
        lsum[qb] = lsum[qb] * cf + ps;
        mrow[qb] = mn;
        // cf is exactly 1 in a column whose running max did not grow: the rescale is skipped
        // when that holds in every column of the wave
        if (__ballot(cf != 1.f)) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[db][qb] *= cf;
        }
      }
    };
    if (k0 + KT - 1 > q0) softmax(std::true_type{});
    else softmax(std::false_type{});
    // O^T[dim][q] += V^T P^T, 32 keys (blocks 2s and 2s+1) per instruction
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      h8 pb[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const h4 a0 = pf[2 * s2][qb], a1 = pf[2 * s2 + 1][qb];
        pb[qb] = (h8){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        // lane r: key kb0 + r / 4, dims 16 db + 4 (r % 4): chunk 2 db + (r % 4) / 2, half (r % 2)
        const int c = 2 * db + (lr % 4) / 2, hoff = 4 * (lr % 2);
        const int key0 = (2 * s2) * 16 + 4 * lq + lr / 4, key1 = key0 + 16;
        const h4 v0 = vt_read(&Vc[key0 * D + (c ^ fV(key0)) * 8 + hoff]);
        const h4 v1 = vt_read(&Vc[key1 * D + (c ^ fV(key1)) * 8 + hoff]);
        const h8 vf = (h8){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pb[qb], o[db][qb], 0, 0, 0);
      }
    }
  };
  const int nt = (kend + KT - 1) / KT;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // tile kt sits in stage kt % 2; the loop runs two tiles per iteration so that every stage is
  // known at compile time
  auto step = [&](auto S, auto SN, int kt) {
    pf_vm_wait<0>();  // this wave's DMA of tile kt (the only one in flight) is complete
    // every wave's part of tile kt landed; every wave is done with tile kt - 1 (its LDS reads
    // returned before the products that used them). A plain barrier: the workgroup fence of
    // __syncthreads would wait for the DMA issued after it as well. The empty asm statements
    // keep the compiler from moving memory accesses across it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + 1 < nt) issue(SN, (kt + 1) * KT);
    compute(S, kt * KT);
  };
  if (nt > 0) issue(S0{}, 0);
  for (int kt = 0; kt < nt; kt += 2) {
    step(S0{}, S1{}, kt);
    if (kt + 1 >= nt) break;
    step(S1{}, S0{}, kt + 1);
  }
  // denominators (the four lanes of a query column hold disjoint keys), normalise, store
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    float l = lsum[qb];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    const int t = q0 + qb * 16 + lr;
    if (t < tend) {
      f16* orow = p.attn + ((size_t)b * p.Ce + (t - p.t0)) * dm.hd + (size_t)h * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        h4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (f16)(o[db][qb][r] / l);
        *(h4*)(orow + db * 16 + 4 * lq) = v;
      }
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_pf_swiglu(PfArgs p) {
  const int m = blockIdx.x;
  const int F = p.dm.F;
  const f16* row = p.gu + (size_t)m * 2 * F;
  f16* out = p.a2 + (size_t)m * F;
  auto act = [](f16 gh, f16 uh) {
    const float g = h2f(gh), u = h2f(uh);
    return f2h(g / (1.f + __expf(-g)) * u);
  };
  if ((F & 7) == 0) {  // 16-byte pieces: the rows of both buffers then start 16-byte aligned
    for (int f = threadIdx.x * 8; f < F; f += kBlock * 8) {
      const uint4 gv = *(const uint4*)(row + f), uv = *(const uint4*)(row + F + f);
      const f16* g8 = (const f16*)&gv;
      const f16* u8 = (const f16*)&uv;
      uint4 o;
      f16* o8 = (f16*)&o;
#pragma unroll
      for (int i = 0; i < 8; ++i) o8[i] = act(g8[i], u8[i]);
      *(uint4*)(out + f) = o;
    }
  } else {
    for (int f = threadIdx.x; f < F; f += kBlock) out[f] = act(row[f], row[F + f]);
  }
}

// s_m = cos(hin[m], hout[m]) in fp64, m the global row of chunk-local row blockIdx.x
__global__ __launch_bounds__(kBlock) void k_pf_cos(PfArgs p) {
  __shared__ double red[4];
  const int64_t m = pf_row(blockIdx.x, p.Ce, p.t0, p.P);
  const int d = p.dm.d;
  double s0 = 0, s1 = 0, s2 = 0;
  for (int i = threadIdx.x; i < d; i += kBlock) {
    const double a = h2f(p.hin[(size_t)m * d + i]), c = h2f(p.hout[(size_t)m * d + i]);
    s0 += a * c;
    s1 += a * a;
    s2 += c * c;
  }
  s0 = block_sum_d(s0, red);
  s1 = block_sum_d(s1, red);
  s2 = block_sum_d(s2, red);
  if (threadIdx.x == 0) p.cosv[m] = (s1 > 0 && s2 > 0) ? s0 / sqrt(s1 * s2) : 0.0;
}

// Sequence-level exit after backbone layer `layer`. One workgroup per sequence.
__global__ __launch_bounds__(kBlock) void k_pf_decide(PfArgs p, int layer, int forced, float tau) {
  __shared__ double red[kBlock];
  const int b = blockIdx.x;
  const Dims& dm = p.dm;
  double mn = 1e300;
  for (int t = threadIdx.x; t < p.P; t += kBlock) mn = fmin(mn, p.cosv[(size_t)b * p.P + t]);
  red[threadIdx.x] = mn;
  __syncthreads();
  for (int s = kBlock / 2; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] = fmin(red[threadIdx.x], red[threadIdx.x + s]);
    __syncthreads();
  }
  // (with a forced exit layer, or before the entry layer, cosv is not written and not used)
  if (threadIdx.x == 0 && layer < dm.L && p.seq_route[b] == ROUTE_BACKBONE) {
    bool ex;
    if (forced > 0) {
      ex = (layer == forced);
    } else if (layer >= dm.entry) {
      const double s = red[0];
      if (p.min_sim) p.min_sim[(size_t)b * dm.L + layer - 1] = (float)s;
      ex = s > (double)tau;
    } else {
      ex = false;
    }
    if (ex) {
      p.seq_route[b] = ROUTE_RIVER;
      p.seq_exit[b] = layer;
    }
  }
}

// Hand the last prompt position of each row to the decode LM head: hs[L][b] = hout[b*P+P-1],
// pos[b] = P-1 and step = 0 (the step bookkeeping after the LM head advances them to P and 1).
__global__ __launch_bounds__(kBlock) void k_pf_finish(PfArgs p, DecodeArgs a) {
  const int b = blockIdx.x;
  const Dims& dm = p.dm;
  const f16* src = p.hin + ((size_t)b * p.P + p.P - 1) * dm.d;  // after the final swap
  f16* dst = a.hs + ((size_t)dm.L * dm.B + b) * dm.d;
  for (int i = threadIdx.x; i < dm.d; i += kBlock) dst[i] = src[i];
  if (threadIdx.x == 0) {
    a.pos[b] = p.P - 1;
    if (b == 0) *a.step = 0;
  }
}

__global__ void k_pf_init_routes(PfArgs p) {
  const int b = threadIdx.x;
  if (b < p.dm.B) {
    p.seq_route[b] = ROUTE_BACKBONE;
    p.seq_exit[b] = p.dm.L;
    if (p.min_sim)
      for (int l = 0; l < p.dm.L; ++l) p.min_sim[(size_t)b * p.dm.L + l] = __builtin_nanf("");
  }
}

// ---------------------------------------------------------------------------------------
static hipError_t gemm(const PfGemmArgs& g0, const LayerDev& lw, int which, int routes, hipStream_t st) {
  // which: 0 qkv, 1 o, 2 gu, 3 down. Launch the fp16 and the int4 variant; each skips the
  // tiles whose sequences are on the other route. routes: bit 0 / bit 1 = some sequence may be
  // on the backbone / on the river at this layer (a variant no sequence can use is not launched)
  dim3 grid((g0.N + QBN - 1) / QBN, (g0.M + QBM - 1) / QBM);
  PfGemmArgs g = g0;
  g.want_route = ROUTE_BACKBONE;
  if (routes & 1) {
    if (g.M % QBM == 0 && g.N % QBN == 0 && g.K % QBK == 0 && g.seg_start[1] % QBN == 0 &&
        g.seg_start[2] % QBN == 0)
      hipLaunchKernelGGL((k_pf_gemm2<0, 64, true>), grid, dim3(kBlock), 0, st, g);
    else
      hipLaunchKernelGGL((k_pf_gemm2<0, 64>), grid, dim3(kBlock), 0, st, g);
  }
  g.want_route = ROUTE_RIVER;
  if (routes & 2) {
    if (g.group >= 64) hipLaunchKernelGGL((k_pf_gemm2<1, 64>), grid, dim3(kBlock), 0, st, g);
    else hipLaunchKernelGGL((k_pf_gemm2<1, 32>), grid, dim3(kBlock), 0, st, g);
  }
  (void)lw;
  (void)which;
  return hipGetLastError();
}

hipError_t river_launch_prefill(const PfArgs& p, const DecodeArgs& a, const LayerDev* host_layers,
                                int forced, float tau, hipStream_t st) {
  const Dims& dm = p.dm;
  const int M = p.M;
  hipError_t e;
  hipLaunchKernelGGL(k_pf_init_routes, dim3(1), dim3(64), 0, st, p);
  hipLaunchKernelGGL(k_pf_embed, dim3(M), dim3(kBlock), 0, st, p);
  PfArgs q = p;  // hin/hout swap per layer
  for (int l = 1; l <= dm.L; ++l) {
    const LayerDev& lw = host_layers[l - 1];
    // a forced exit layer fixes every sequence's route: the backbone up to it, the river after
    const int routes = forced > 0 ? (l <= forced ? 1 : 2) : 3;
    for (int t0 = 0; t0 < q.P; t0 += q.Ct) {
      q.t0 = t0;
      q.Ce = min(q.Ct, q.P - t0);
      const int Mc = dm.B * q.Ce;  // rows of this chunk
      // attention half
      hipLaunchKernelGGL(k_pf_rmsnorm, dim3(Mc), dim3(kBlock), 0, st, (const f16*)q.hin, lw.attn_norm,
                         q.act, dm.d, dm.eps, q.P, q.Ce, q.t0);
      PfGemmArgs g{};
      g.M = Mc;
      g.group = dm.group;
      g.seq_route = q.seq_route;
      g.P = q.Ce;
      g.Ptot = q.P;
      g.t0 = q.t0;
      g.A = q.act;
      g.N = dm.nqkv;
      g.K = dm.d;
      g.seg_ptr[0] = lw.wq;
      g.seg_ptr[1] = lw.wk;
      g.seg_ptr[2] = lw.wv;
      g.seg_start[0] = 0;
      g.seg_start[1] = dm.hd;
      g.seg_start[2] = dm.hd + dm.Hkv * dm.D;
      g.seg_start[3] = dm.nqkv;
      g.w4 = lw.r_qkv;
      g.s4 = lw.s_qkv;
      g.z4 = lw.z_qkv;
      g.C = q.qkv;
      g.epi = EPI_STORE;
      if ((e = gemm(g, lw, 0, routes, st)) != hipSuccess) return e;
      hipLaunchKernelGGL(k_pf_rope_kv, dim3(Mc), dim3(kBlock), 0, st, q, l);
      {
        const int G = dm.H / dm.Hkv;
        dim3 grid((q.Ce + 31) / 32, dm.Hkv, dm.B);
        if (dm.D == 128 && G == 4) hipLaunchKernelGGL((k_pf_fattn2<128, 4, 2>), grid, dim3(4 * kWave), 0, st, q, l);
        else if (dm.D == 64 && G == 4) hipLaunchKernelGGL((k_pf_fattn2<64, 4, 2>), grid, dim3(4 * kWave), 0, st, q, l);
        else if (dm.D == 64 && G == 2) hipLaunchKernelGGL((k_pf_fattn2<64, 2, 2>), grid, dim3(2 * kWave), 0, st, q, l);
        else if (dm.D == 128 && G == 2) hipLaunchKernelGGL((k_pf_fattn2<128, 2, 2>), grid, dim3(2 * kWave), 0, st, q, l);
        else if (dm.D == 128 && G == 1) hipLaunchKernelGGL((k_pf_fattn<128, 1>), grid, dim3(kWave), 0, st, q, l);
        else if (dm.D == 64 && G == 1) hipLaunchKernelGGL((k_pf_fattn<64, 1>), grid, dim3(kWave), 0, st, q, l);
        else if (dm.D == 128 && G == 8) hipLaunchKernelGGL((k_pf_fattn2<128, 8, 2>), grid, dim3(8 * kWave), 0, st, q, l);
        else if (dm.D == 64 && G == 8) hipLaunchKernelGGL((k_pf_fattn2<64, 8, 2>), grid, dim3(8 * kWave), 0, st, q, l);
        else return hipErrorInvalidValue;
      }
      // O projection + residual (the residual stream rows of this chunk)
      g.A = q.attn;
      g.N = dm.d;
      g.K = dm.hd;
      g.seg_ptr[0] = lw.wo;
      g.seg_start[0] = 0;
      g.seg_start[1] = dm.d;
      g.seg_start[2] = dm.d;
      g.seg_start[3] = dm.d;
      g.w4 = lw.r_o;
      g.s4 = lw.s_o;
      g.z4 = lw.z_o;
      g.C = q.hmid;
      g.R = q.hin;
      g.r_global = 1;
      g.epi = EPI_RESID;
      if ((e = gemm(g, lw, 1, routes, st)) != hipSuccess) return e;
      g.r_global = 0;
      // MLP half
      hipLaunchKernelGGL(k_pf_rmsnorm, dim3(Mc), dim3(kBlock), 0, st, (const f16*)q.hmid, lw.mlp_norm,
                         q.act, dm.d, dm.eps, 0, 0, 0);
      g.A = q.act;
      g.N = 2 * dm.F;
      g.K = dm.d;
      g.seg_ptr[0] = lw.wg;
      g.seg_ptr[1] = lw.wu;
      g.seg_start[0] = 0;
      g.seg_start[1] = dm.F;
      g.seg_start[2] = 2 * dm.F;
      g.seg_start[3] = 2 * dm.F;
      g.w4 = lw.r_gu;
      g.s4 = lw.s_gu;
      g.z4 = lw.z_gu;
      g.C = q.gu;
      g.R = nullptr;
      g.epi = EPI_STORE;
      if ((e = gemm(g, lw, 2, routes, st)) != hipSuccess) return e;
      hipLaunchKernelGGL(k_pf_swiglu, dim3(Mc), dim3(kBlock), 0, st, q);
      g.A = q.a2;
      g.N = dm.d;
      g.K = dm.F;
      g.seg_ptr[0] = lw.wd;
      g.seg_start[0] = 0;
      g.seg_start[1] = dm.d;
      g.seg_start[2] = dm.d;
      g.seg_start[3] = dm.d;
      g.w4 = lw.r_d;
      g.s4 = lw.s_d;
      g.z4 = lw.z_d;
      g.C = q.hout;
      g.c_global = 1;
      g.R = q.hmid;
      g.epi = EPI_RESID;
      if ((e = gemm(g, lw, 3, routes, st)) != hipSuccess) return e;
      // per-token similarity of this chunk's rows (the exit test needs all of them; a forced
      // exit layer, or a layer before the entry layer, decides without them)
      if (l < dm.L && forced <= 0 && l >= dm.entry) hipLaunchKernelGGL(k_pf_cos, dim3(Mc), dim3(kBlock), 0, st, q);
    }
    // sequence-level exit decision after this layer (every chunk has run it)
    if (l < dm.L) hipLaunchKernelGGL(k_pf_decide, dim3(dm.B), dim3(kBlock), 0, st, q, l, forced, tau);
    f16* t = q.hin;
    q.hin = q.hout;
    q.hout = t;
  }
  hipLaunchKernelGGL(k_pf_finish, dim3(dm.B), dim3(kBlock), 0, st, q, a);
  return hipGetLastError();
}
