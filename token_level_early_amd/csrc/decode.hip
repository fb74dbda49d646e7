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

#include <type_traits>

#include "gemv.hpp"
#include "attn.hpp"

// MODE 0: early-exit decode (both weight streams in the grid; the route of the layer is decided
//         by every QKV workgroup identically and read from device state by the later kernels).
// MODE 1: backbone-only decode (the full-depth fp16 model: no river tiles, no exit test).
template <int OP, int MODE, int NCH16, int WPR16, int NCH4, int WPR4>
__global__ __launch_bounds__(kBlock) void k_dec_gemv(DecodeArgs a, int layer, int nwg16, int nwg4) {
  using T16 = TileF16<WPR16>;
  using T4 = TileW4<WPR4>;
  __shared__ GemvSmem gsm;
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
      if (MODE == 0) {  // forced exit 0: no backbone block at all
        if (a.sched && a.sched[step * dm.B + b] == 0) route = ROUTE_RIVER;
        if (blockIdx.x == 0 && t == 0) {
          a.route[dm.B + b] = route;  // layer 1's route, read by its later ops and the next exit test
          if (route == ROUTE_RIVER && a.exit_out) a.exit_out[step * dm.B + b] = 0;
        }
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
            if ((e < dm.entry && e != 0) || e > dm.L) {
              if (blockIdx.x == 0 && t == 0) atomicOr(a.err, ERR_FORCED);
              e = dm.L;
            }
            if (lp == e) route = ROUTE_RIVER;
          } else {
            if (t < kWave) {
              double dot, n1, n2;
              wave_cos3<false>(a.hs + ((size_t)(lp - 1) * dm.B + b) * dm.d, vin, dm.d, dot, n1, n2);
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

  TileIn in;
  in.layer = layer;
  in.step = step;
  in.pos = (OP == OP_QKV) ? a.pos[b] : 0;
  in.b = b;
  in.want_norm = false;
  in.inv = 1.f;
  in.gain = nullptr;
  if (OP == OP_QKV) {
    in.xv = vin;
    in.gain = lwp->attn_norm;
    in.want_norm = !have_inv;
    in.inv = inv;
  } else if (OP == OP_O) {
    in.xv = a.o + (size_t)b * dm.hd;
  } else if (OP == OP_GU) {
    in.xv = a.hmid + ((size_t)(layer - 1) * dm.B + b) * dm.d;
    in.gain = lwp->mlp_norm;
    in.want_norm = true;
  } else if (OP == OP_DOWN) {
    in.xv = a.a2 + (size_t)b * dm.F;
  } else {
    in.xv = a.hs + ((size_t)dm.L * dm.B + b) * dm.d;
    in.gain = a.final_norm;
    in.inv = a.inv_attn[dm.L * dm.B + b];
  }
  in.key = a.amax + b;
  const int tile = is4 ? (int)blockIdx.x - nwg16 : (int)blockIdx.x;
  gemv_tile<OP, false, NCH16, WPR16, NCH4, WPR4>(a, lwp, in, tile, is4, gsm);
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

// GQA split-K decode attention over the shared cache (attn.hpp). Grid (smax, Hkv, B).
template <int D, int G>
#ifndef RIVER_DATTN_UP
#define RIVER_DATTN_UP 4  // positions per lane per block
#endif
#ifndef RIVER_DATTN_GL
#define RIVER_DATTN_GL 2  // query heads per lane (at least what fits a wave)
#endif
#ifndef RIVER_DATTN_NT
#define RIVER_DATTN_NT kBlock  // threads per workgroup
#endif
__global__ __launch_bounds__(RIVER_DATTN_NT) void k_dec_attn(DecodeArgs a, int layer) {
  // query heads per lane: as requested, but enough that one slot's lanes fit a wave
  constexpr int GLmin = (G * (D / 8) + kWave - 1) / kWave;
  constexpr int GLr = RIVER_DATTN_GL < G ? RIVER_DATTN_GL : G;
  constexpr int GLP = GLr > GLmin ? GLr : GLmin;
  __shared__ AttnLds<D, G, RIVER_DATTN_NT, GLP> sm;
  const int b = blockIdx.z;
  attn_split<D, G, RIVER_DATTN_NT, false, RIVER_DATTN_UP, GLP>(a, layer, blockIdx.x, blockIdx.y, b, a.pos[b], a.attn_smax, sm);
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
  if (dm.D == 128 && G == 4) hipLaunchKernelGGL((k_dec_attn<128, 4>), grid, dim3(RIVER_DATTN_NT), 0, st, a, layer);
  else if (dm.D == 64 && G == 4) hipLaunchKernelGGL((k_dec_attn<64, 4>), grid, dim3(RIVER_DATTN_NT), 0, st, a, layer);
  else if (dm.D == 64 && G == 2) hipLaunchKernelGGL((k_dec_attn<64, 2>), grid, dim3(RIVER_DATTN_NT), 0, st, a, layer);
  else if (dm.D == 128 && G == 2) hipLaunchKernelGGL((k_dec_attn<128, 2>), grid, dim3(RIVER_DATTN_NT), 0, st, a, layer);
  else if (dm.D == 128 && G == 1) hipLaunchKernelGGL((k_dec_attn<128, 1>), grid, dim3(RIVER_DATTN_NT), 0, st, a, layer);
  else if (dm.D == 64 && G == 1) hipLaunchKernelGGL((k_dec_attn<64, 1>), grid, dim3(RIVER_DATTN_NT), 0, st, a, layer);
  else if (dm.D == 128 && G == 8) hipLaunchKernelGGL((k_dec_attn<128, 8>), grid, dim3(RIVER_DATTN_NT), 0, st, a, layer);
  else if (dm.D == 64 && G == 8) hipLaunchKernelGGL((k_dec_attn<64, 8>), grid, dim3(RIVER_DATTN_NT), 0, st, a, layer);
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

hipError_t river_launch_step_end(const DecodeArgs& a, hipStream_t st) {
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

// Start of a decode call on the per-op path: step counter and both argmax keys cleared.
__global__ void k_begin_steps(DecodeArgs a) {
  if (threadIdx.x == 0) *a.step = 0;
  if ((int)threadIdx.x < 2 * a.dm.B)
    __hip_atomic_store(a.amax + threadIdx.x, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t river_launch_begin(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_begin_steps, dim3(1), dim3(64), 0, st, a);
  return hipGetLastError();
}

