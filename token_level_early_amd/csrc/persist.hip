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
// (the split that owns the new position rotates k, writes K/V[pos], then attends); SwiGLU to
// the gate|up epilogue (each wave owns whole gate/up row pairs, so it is computed once per
// pair instead of once per workgroup while staging the down projection's input).
//
// Routes, the position and the token stay in registers (every workgroup derives identical
// values); activations cross XCDs through write-through stores and coherent loads. The grid
// barrier spins with a bound: a workgroup that waits too long raises an abort flag, after
// which every barrier returns at once, so every wave reaches the end of the kernel.
#include <mutex>
#include <type_traits>

#include "gemv.hpp"
#include "attn.hpp"

static constexpr unsigned kSpinLimit = 1u << 22;
static constexpr int kMaxK = 16384;  // longest GEMV input the LDS staging buffer holds
static constexpr int kPB = 512;      // threads per persistent workgroup (one per CU)
static constexpr int kPW = kPB / kWave;
// attention lane layout of the persistent kernel: query heads per lane (see attn_split); the
// positions per thread per block are the kernel's AU parameter (2, or 4 from kPersistLongCtx)
#ifndef RIVER_PATTN_GL
#define RIVER_PATTN_GL 1
#endif

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

// Two-level grid barrier. Workgroups arrive on the counter of their group of kBarGroup; the
// last arrival of a group bumps the completed-group counter; the arrival that completes the
// last group writes the epoch into every group's release flag, and each workgroup polls its own
// group's flag. Counters and flags only grow during a launch (epoch e is complete when the
// group counter reaches e * group size and the top counter e * groups), so no reset is needed
// between barriers. Same-address atomics per barrier: kBarGroup + groups instead of one per
// workgroup; pollers per line: kBarGroup instead of the whole grid.
// `pre` (weight loads of the next phase, which do not depend on the data the barrier
// protects) is issued while the barrier is pending: by every wave but the polling one before
// the wait, by the polling wave after it (its poll loads must not queue behind them).
static constexpr int kPoller = kPB - kWave;  // first lane of the last wave
template <typename Pre>
RIVER_DEV void grid_sync(unsigned* bar, unsigned& epoch, unsigned nwg, Pre&& pre) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores have landed
  __syncthreads();
  ++epoch;
  const unsigned ng = (nwg + kBarGroup - 1) / kBarGroup;
  const unsigned g = blockIdx.x / kBarGroup;
  unsigned* flags = bar + (kBarMaxGroups + 1) * kBarStride;
  if (threadIdx.x == kPoller) {  // arrive first, so the prefetch below does not queue ahead of it
    const unsigned gs = min((unsigned)kBarGroup, nwg - g * kBarGroup);
    const unsigned old = __hip_atomic_fetch_add(bar + (1 + g) * kBarStride, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    if (old == epoch * gs - 1) {
      const unsigned top = __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (top == epoch * ng - 1)
        for (unsigned j = 0; j < ng; ++j)
          __hip_atomic_store(flags + j * kBarStride, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  const bool poll_wave = threadIdx.x >= kPoller;
  if (!poll_wave) pre();
  if (threadIdx.x == kPoller) {
    int* abort = (int*)(bar + kBarAbort);
    unsigned spins = 0;
    while (__hip_atomic_load(flags + g * kBarStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < epoch) {
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
  if (poll_wave) pre();
}
RIVER_DEV void grid_sync(unsigned* bar, unsigned& epoch, unsigned nwg) {
  grid_sync(bar, epoch, nwg, [] {});
}

// ---------------------------------------------------------------------------------------
// LDS
// ---------------------------------------------------------------------------------------
template <int D, int G>
struct PSmem {
  union __attribute__((aligned(16))) {
    h2 x[kMaxK / 2];  // staged GEMV input
    AttnLds<D, G, kPB, (RIVER_PATTN_GL < G ? RIVER_PATTN_GL : G)> at;
  };
  float xc[kMaxK / 32];  // int4 stream: per (chunk, lane) bias correction of the staged input
  float xs[kMaxK / 32];  // zero-point format: per (chunk, lane) sum of the staged input
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

// Writes one group of 8 staged values into LDS in the stream's layout. For the int4 stream the
// odd elements of each pair set are stored divided by 16 (exact) and the bias correction of
// the (chunk, lane) the group belongs to is summed over its 4 groups (threads t..t+3 stage
// them; the quad is always complete) -- see dot_seg4 for how both are used. Zero-point format
// (ZP): the correction leaves the zero point out (it is per group of weights), and xs gets the
// plain sum of the lane's 32 inputs, which dot_seg4 scales by the group's zero point.
template <bool IS4, bool ZP = false>
RIVER_DEV void put_group(h2* xl, float* xc, float* xs, int g, uint4 u) {
  h2* dst = xl + lds_group_index<IS4>(g);
  if (IS4) {
    const uint32_t in[4] = {u.x, u.y, u.z, u.w};
    h2 o[4];
    pair_for_unpack(in, o);  // (x0,x4) (x1,x5) (x2,x6) (x3,x7)
    const float xlo = (h2f(o[0].x) + h2f(o[0].y)) + (h2f(o[2].x) + h2f(o[2].y));
    const float xhi = (h2f(o[1].x) + h2f(o[1].y)) + (h2f(o[3].x) + h2f(o[3].y));
    const h2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
    dst[0] = o[0];
    dst[1] = o[1] * sixteenth;
    dst[2] = o[2];
    dst[3] = o[3] * sixteenth;
    float c = ZP ? -1024.f * xlo - 64.f * xhi : -1032.f * xlo - 72.f * xhi;
    c += dpp_f<0xB1>(c);
    c += dpp_f<0x4E>(c);
    if ((g & 3) == 0) xc[g >> 2] = c;
    if (ZP) {
      float xsum = xlo + xhi;
      xsum += dpp_f<0xB1>(xsum);
      xsum += dpp_f<0x4E>(xsum);
      if ((g & 3) == 0) xs[g >> 2] = xsum;
    }
  } else {
    dst[0] = as_h2(u.x);
    dst[1] = as_h2(u.y);
    dst[2] = as_h2(u.z);
    dst[3] = as_h2(u.w);
  }
}

// x = fp16(src * inv * gain) (HAS_GAIN) or src, staged into LDS. TAG: src is a tagged vector
// (see ld_tag8n) whose words must carry `tag`; else a plain fp16 vector that does not change
// during the launch (the embedding row). NORM: inv = 1/rms(src) computed here in a fixed
// order (identical in every workgroup). Each thread reads its groups of 8 values two at a
// time (both waits in one round trip), together with their gains.
template <bool IS4, bool HAS_GAIN, bool NORM, bool TAG, int NG, bool ZP = false>
RIVER_DEV void stage_x(const void* src, uint32_t tag, int* abort, const f16* gain, int K, float inv,
                       float eps, h2* xl, float* xc, float* xs, double* red) {
  const int t = threadIdx.x;
  const int nch = IS4 ? (K + kChunkW4 - 1) / kChunkW4 : (K + kChunkF16 - 1) / kChunkF16;
  const int ngp = nch * (IS4 ? kChunkW4 : kChunkF16) / 8;
  // groups g0 and g0 + kPB of the source (zero past K)
  auto load2 = [&](int g0, uint4 (&v)[2]) {
    const int g1 = g0 + kPB;
    if (TAG) {
      const uint32_t* ts = (const uint32_t*)src;
      const uint32_t* pp[2] = {ts + (size_t)g0 * 8, ts + (size_t)(g1 * 8 < K ? g1 : g0) * 8};
      const bool use[2] = {g0 * 8 < K, g1 * 8 < K};
      ld_tag8n<2>(pp, use, tag, abort, v);
    } else {
      const f16* ps = (const f16*)src;
      v[0] = (g0 * 8 < K) ? ldg16(ps + (size_t)g0 * 8) : make_uint4(0, 0, 0, 0);
      v[1] = (g1 * 8 < K) ? ldg16(ps + (size_t)g1 * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  if (NORM) {
    static_assert(NG <= 2, "normalised inputs: at most two groups per thread");
    uint4 v[2], gv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int g = t + i * kPB;
      gv[i] = (HAS_GAIN && i < NG && g * 8 < K) ? ldg16(gain + g * 8) : make_uint4(0, 0, 0, 0);
    }
    load2(t, v);
    if (NG < 2) v[1] = make_uint4(0, 0, 0, 0);
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < NG; ++i) ss += sq8(v[i]);
    inv = inv_rms(pblock_sum_d(ss, red), K, eps);
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int g = t + i * kPB;
      if (g >= ngp) continue;
      uint4 u = v[i];
      if (HAS_GAIN && g * 8 < K) u = norm8(u, gv[i], inv, true);
      put_group<IS4, ZP>(xl, xc, xs, g, u);
    }
    for (int g = t + NG * kPB; g < ngp; g += kPB) put_group<IS4, ZP>(xl, xc, xs, g, make_uint4(0, 0, 0, 0));
  } else {
    for (int g0 = t; g0 < ngp; g0 += 2 * kPB) {
      uint4 v[2];
      load2(g0, v);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int g = g0 + i * kPB;
        if (g >= ngp) break;  // ngp is a multiple of 4: whole quads stay together
        uint4 u = v[i];
        if (HAS_GAIN && g * 8 < K) u = norm8(u, ldg16(gain + g * 8), inv, true);
        put_group<IS4, ZP>(xl, xc, xs, g, u);
      }
    }
  }
  __syncthreads();
}

// Exit-test reduction of cos(h(l-1), h(l)) over the whole block in a fixed order. h(l-1) is the
// embedding row (up, plain) or a tagged residual-stream vector (ut); h(l) is tagged.
RIVER_DEV void block_cos(const f16* up, const uint32_t* ut, uint32_t utag, const uint32_t* vt,
                         uint32_t vtag, int* abort, int d, double* red, double& dot, double& nu,
                         double& nv) {
  double s0 = 0, s1 = 0, s2 = 0;
  for (int g = threadIdx.x; g * 8 < d; g += kPB) {
    uint4 ab[2];
    const uint32_t* pp[2] = {ut ? ut + g * 8 : vt + g * 8, vt + g * 8};
    const bool use[2] = {ut != nullptr, true};
    const uint32_t tg[2] = {utag, vtag};
    ld_tag8n<2>(pp, use, tg, abort, ab);
    const uint4 a = up ? ldg16(up + g * 8) : ab[0], b = ab[1];
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
// The fp16 matrices a phase reads (up to three: q, k, v), read from the layer table once per
// phase and held wave-uniform; read per item, the table load (behind the phase's tagged
// stores, so never hoisted by the compiler) stalls the row stream.
template <typename T>
RIVER_DEV const T* uniform_ptr(const T* p) {
  const unsigned long long v = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return (const T*)(((unsigned long long)hi << 32) | lo);
}
struct W16 {
  const f16* p0;
  const f16* p1;
  const f16* p2;
};
template <int OP>
RIVER_DEV W16 w16_ptrs(const DecodeArgs& a, const LayerDev* lw) {
  W16 w{nullptr, nullptr, nullptr};
  if (OP == OP_QKV) w = W16{lw->wq, lw->wk, lw->wv};
  else if (OP == OP_O) w.p0 = lw->wo;
  else if (OP == OP_GU) w = W16{lw->wg, lw->wu, nullptr};
  else if (OP == OP_DOWN) w.p0 = lw->wd;
  else w.p0 = a.lm_head;
  return W16{uniform_ptr(w.p0), uniform_ptr(w.p1), uniform_ptr(w.p2)};
}
template <int OP>
RIVER_DEV const f16* row16(const W16& w, const Dims& dm, int n) {
  if (OP == OP_QKV) {
    if (n < dm.hd) return w.p0 + (size_t)n * dm.d;
    if (n < dm.hd + dm.Hkv * dm.D) return w.p1 + (size_t)(n - dm.hd) * dm.d;
    return w.p2 + (size_t)(n - dm.hd - dm.Hkv * dm.D) * dm.d;
  }
  if (OP == OP_O) return w.p0 + (size_t)n * dm.hd;
  if (OP == OP_GU) return n < dm.F ? w.p0 + (size_t)n * dm.d : w.p1 + (size_t)(n - dm.F) * dm.d;
  if (OP == OP_DOWN) return w.p0 + (size_t)n * dm.F;
  return w.p0 + (size_t)n * dm.d;
}

static constexpr uint32_t kMagic = 0x64006400u;  // fp16 1024.0 in both halves

// (w & m) | c in one instruction (v_and_or_b32; the mask rides in a scalar register).
RIVER_DEV uint32_t and_or(uint32_t w, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(m), "v"(c));
  return r;
}

// This wave's rows [r0, r1) of an N-row phase (rows split evenly over all waves of the grid).
RIVER_DEV void wave_rows(int N, int& r0, int& r1) {
  const int gw = blockIdx.x * kPW + threadIdx.x / kWave, GW = gridDim.x * kPW;
  // wave-uniform: keep the row walk (and the row pointers) in scalar registers
  r0 = __builtin_amdgcn_readfirstlane((int)((long long)gw * N / GW));
  r1 = __builtin_amdgcn_readfirstlane((int)((long long)(gw + 1) * N / GW));
}

// The rows a wave streams, as a virtual range [0, nv): virtual row v is physical row
// r0 + v below `split` and r0 + jump + v from there on. Every phase but gate|up takes a
// contiguous slice; gate|up takes whole (gate j, up j) pairs -- its gate rows [j0, j1), then
// the matching up rows [F + j0, F + j1) -- so the wave that finishes up row j also holds
// gate row j and applies SwiGLU itself.
struct RowRange {
  int r0, nv, split, jump;
  RIVER_DEV int row(int v) const { return v < split ? r0 + v : r0 + jump + v; }
  // physical chunk of virtual chunk q (nch chunks per row)
  RIVER_DEV int chunk(int q, int nch) const { return q < split * nch ? r0 * nch + q : (r0 + jump) * nch + q; }
};
template <int OP>
RIVER_DEV RowRange wave_range(int N) {
  int r0, r1;
  if (OP == OP_GU) {
    const int F = N / 2;
    wave_rows(F, r0, r1);
    const int n = r1 - r0;
    return RowRange{r0, 2 * n, n, F - n};
  }
  wave_rows(N, r0, r1);
  return RowRange{r0, r1 - r0, r1 - r0, 0};
}

// Streamed items. fp16 stream: an item is SEG chunks (512 elements each) of one row, a row
// being nseg items. int4 stream: the padded river layout makes the rows of one matrix a
// single run of 1 KiB chunks (2048 elements each; the group scales likewise), so a wave's rows
// [r0, r1) are the flat chunk range [r0*nch, r1*nch) and an item is the next SEG chunks of
// that range, crossing row ends: every item keeps SEG loads per lane in flight whatever K is.
template <int SEG>
struct Seg {
  uint4 w[SEG];
  uint4 sr;  // int4: this lane's share of the item's group scales (fetched per chunk by shuffle)
  uint2 zr;  // zero-point format: this lane's share of the item's zero points (bytes), likewise
};

// fp16: chunks [seg*SEG, seg*SEG+SEG) of `row`.
// Every load is issued (a chunk past the row re-reads the row's last chunk: dot_seg16 stops at
// nch), so that no load sits behind a branch: one there leaves the compiler unable to count the
// loads in flight, and every later wait then drains them all, the next item's included.
template <int OP, int SEG>
RIVER_DEV void load_seg16(const W16& w, const Dims& dm, int K, int nch, int row, int seg, Seg<SEG>& sg) {
  const int lane = threadIdx.x & (kWave - 1);
  const f16* rp = row16<OP>(w, dm, row);
#pragma unroll
  for (int c = 0; c < SEG; ++c) {
    const int ch = seg * SEG + c;
    const int e = (ch < nch ? ch : nch - 1) * kChunkF16 + lane * 8;
    sg.w[c] = ldg16(rp + (e < K ? e : 0));  // past K meets x = 0
  }
  sg.sr = make_uint4(0, 0, 0, 0);
}

template <int SEG>
RIVER_DEV float dot_seg16(const Seg<SEG>& sg, const h2* xl, int nch, int seg, float acc) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int c = 0; c < SEG; ++c) {
    const int ch = seg * SEG + c;
    if (ch >= nch) break;
    const uint4 x = ((const uint4*)xl)[ch * kWave + lane];  // one ds_read_b128
    acc = dot2(as_h2(x.x), as_h2(sg.w[c].x), acc);
    acc = dot2(as_h2(x.y), as_h2(sg.w[c].y), acc);
    acc = dot2(as_h2(x.z), as_h2(sg.w[c].z), acc);
    acc = dot2(as_h2(x.w), as_h2(sg.w[c].w), acc);
  }
  return acc;
}

// int4: flat chunks [q0, min(q0 + SEG, qend)) of the matrix starting at (base, sbase). The
// item's group scales are contiguous too (spc = 2048/group per chunk); one load per lane
// brings npl = SEG*spc/64 of them (lane L: scales [L*npl, L*npl + npl) of the item) instead of
// one small load per chunk.
template <int SEG, int GRP, bool ZP = false>
RIVER_DEV void load_seg4(const uint8_t* base, const f16* sbase, const uint8_t* zbase, const RowRange& rr,
                         int nch, int q0, int qend, Seg<SEG>& sg) {
  const int lane = threadIdx.x & (kWave - 1);
  // every load is issued, from an in-range address (see load_seg16): chunks past the end
  // re-read the last chunk and scales past the end the last scales; dot_seg4 uses neither
#pragma unroll
  for (int c = 0; c < SEG; ++c)
    sg.w[c] = ldg16(base + (size_t)rr.chunk(q0 + c < qend ? q0 + c : qend - 1, nch) * 1024 + lane * 16);
  constexpr int spc = kChunkW4 / GRP;
  constexpr int npl = SEG * spc / kWave;
  static_assert(npl == 1 || npl == 2 || npl == 4 || npl == 8, "scales per lane");
  const int s00 = q0 * spc + lane * npl;  // virtual scale index; npl divides spc
  const int s0 = s00 < qend * spc ? s00 : qend * spc - npl;  // npl divides both
  sg.sr = make_uint4(0, 0, 0, 0);
  if (ZP) sg.zr = make_uint2(0, 0);
  {
    const f16* sp = sbase + (size_t)rr.chunk(s0 / spc, nch) * spc + s0 % spc;
    if (npl == 1) {
      sg.sr.x = __builtin_bit_cast(unsigned short, ldg2(sp));
    } else if (npl == 2) {
      sg.sr.x = *(const __attribute__((address_space(1))) uint32_t*)sp;
    } else if (npl == 4) {
      const unsigned long long v = *(const __attribute__((address_space(1))) unsigned long long*)sp;
      sg.sr.x = (uint32_t)v;
      sg.sr.y = (uint32_t)(v >> 32);
    } else {
      sg.sr = ldg16(sp);
    }
    if (ZP) {  // the same scale indices' zero points, one byte each
      const uint8_t* zp = zbase + (size_t)rr.chunk(s0 / spc, nch) * spc + s0 % spc;
      if (npl == 1) sg.zr.x = *(const __attribute__((address_space(1))) uint8_t*)zp;
      else if (npl == 2) sg.zr.x = *(const __attribute__((address_space(1))) unsigned short*)zp;
      else if (npl == 4) sg.zr.x = *(const __attribute__((address_space(1))) uint32_t*)zp;
      else {
        typedef uint32_t v2u __attribute__((ext_vector_type(2)));
        const v2u v = *(const __attribute__((address_space(1))) v2u*)zp;
        sg.zr = make_uint2(v.x, v.y);
      }
    }
  }
}

// Scale of chunk c of an item for this lane's 32 elements: scale index c*spc + lane*spc/64 of
// the item, held by lane index/npl.
template <int SEG, int spc, int npl>
RIVER_DEV float item_scale(const Seg<SEG>& sg, int c) {
  const int lane = threadIdx.x & (kWave - 1);
  const int i = c * spc + (lane * spc) / kWave;
  const int src = i / npl, e = i % npl;
  uint32_t wv;
  if (npl <= 2) {
    wv = (uint32_t)__shfl((int)sg.sr.x, src, kWave);
  } else if (npl == 4) {
    const uint32_t w0 = (uint32_t)__shfl((int)sg.sr.x, src, kWave);
    const uint32_t w1 = (uint32_t)__shfl((int)sg.sr.y, src, kWave);
    wv = (e >> 1) ? w1 : w0;
  } else {
    const uint32_t w0 = (uint32_t)__shfl((int)sg.sr.x, src, kWave);
    const uint32_t w1 = (uint32_t)__shfl((int)sg.sr.y, src, kWave);
    const uint32_t w2 = (uint32_t)__shfl((int)sg.sr.z, src, kWave);
    const uint32_t w3 = (uint32_t)__shfl((int)sg.sr.w, src, kWave);
    const int k = e >> 1;
    wv = k == 0 ? w0 : k == 1 ? w1 : k == 2 ? w2 : w3;
  }
  const unsigned short hv = (unsigned short)((e & 1) ? (wv >> 16) : wv);
  return h2f(__builtin_bit_cast(f16, hv));
}

// Zero point of chunk c of an item for this lane's 32 elements (same index as item_scale).
template <int SEG, int spc, int npl>
RIVER_DEV float item_zero(const Seg<SEG>& sg, int c) {
  const int lane = threadIdx.x & (kWave - 1);
  const int i = c * spc + (lane * spc) / kWave;
  const int src = i / npl, e = i % npl;
  const uint32_t wx = (uint32_t)__shfl((int)sg.zr.x, src, kWave);
  uint32_t wv = wx;
  if (npl == 8) {
    const uint32_t wy = (uint32_t)__shfl((int)sg.zr.y, src, kWave);
    wv = (e >> 2) ? wy : wx;
  }
  return (float)((wv >> (8 * (e & 3))) & 0xFFu);
}

// Reduces the int4 item starting at flat chunk q0 (chunk ch of row `row`); calls fin(row, lane
// partial) at every row end and advances (row, ch).
template <int SEG, int GRP, bool ZP, typename Fin>
RIVER_DEV void dot_seg4(const Seg<SEG>& sg, const h2* xl, const float* xc, const float* xs, int nch,
                        int q0, int qend, int& row, int& ch, float& acc, Fin&& fin) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int spc = kChunkW4 / GRP, npl = SEG * spc / kWave;
#pragma unroll
  for (int c = 0; c < SEG; ++c) {
    if (q0 + c >= qend) break;
    // nibbles OR-ed into fp16 1024.0 give 1024 + u (low nibble of each half) or 1024 + 16u
    // (high nibble); against x (resp. x/16) the dot is sum (u - 8) x + 1032 X_lo + 72 X_hi,
    // and the staged correction -1032 X_lo - 72 X_hi starts the sum
    // zero-point format: sum (u - z) x = sum u x - z X, X the lane's input sum
    float sd = xc[ch * kWave + lane];
    if (ZP) sd = fmaf(-item_zero<SEG, spc, npl>(sg, c), xs[ch * kWave + lane], sd);
    uint4 xv[4];  // all four 16-byte reads of this chunk's inputs first
#pragma unroll
    for (int m = 0; m < 4; ++m) xv[m] = ((const uint4*)xl)[(ch * 4 + m) * kWave + lane];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t wm = (&sg.w[c].x)[m], w8 = wm >> 8;
      sd = dot2(as_h2(and_or(wm, 0x000F000Fu, kMagic)), as_h2(xv[m].x), sd);
      sd = dot2(as_h2(and_or(wm, 0x00F000F0u, kMagic)), as_h2(xv[m].y), sd);
      sd = dot2(as_h2(and_or(w8, 0x000F000Fu, kMagic)), as_h2(xv[m].z), sd);
      sd = dot2(as_h2(and_or(w8, 0x00F000F0u, kMagic)), as_h2(xv[m].w), sd);
    }
    acc = fmaf(item_scale<SEG, spc, npl>(sg, c), sd, acc);
    if (++ch == nch) {
      fin(row, acc);
      acc = 0.f;
      ch = 0;
      ++row;
    }
  }
}

// Base of the packed river matrix of OP and of its scales.
template <int OP>
RIVER_DEV void w4_base(const LayerDev* lw, const uint8_t*& base, const f16*& sbase, const uint8_t*& zbase) {
  if (OP == OP_QKV) { base = lw->r_qkv; sbase = lw->s_qkv; zbase = lw->z_qkv; }
  else if (OP == OP_O) { base = lw->r_o; sbase = lw->s_o; zbase = lw->z_o; }
  else if (OP == OP_GU) { base = lw->r_gu; sbase = lw->s_gu; zbase = lw->z_gu; }
  else { base = lw->r_d; sbase = lw->s_d; zbase = lw->z_d; }
}

// Epilogue inputs of a streamed phase.
// Phase timestamps (debug build with RIVER_PHASE_TRACE, libriver_phasetrace.so): thread 0 of
// every workgroup records the 100 MHz realtime counter at the boundaries of each phase, at
// [step][slot][event][workgroup] (slot l-1 for block l, slot L for the LM head; the events are
// the RIVER_EV_* below). The release build records nothing.
enum {
  RIVER_EV_START = 0,      // block: before the exit test; head: before its staging
  RIVER_EV_QKV_STAGED = 1, // head: LM input staged
  RIVER_EV_QKV_END = 2,    // head: LM rows done
  RIVER_EV_ATT_END = 3,    // head: past the step's grid barrier
  RIVER_EV_O_STAGED = 4,
  RIVER_EV_O_END = 5,
  RIVER_EV_GU_STAGED = 6,
  RIVER_EV_GU_END = 7,
  RIVER_EV_DN_STAGED = 8,
  RIVER_EV_DN_END = 9,
  RIVER_EV_COUNT = 10
};
static constexpr int kTrSteps = 8, kTrSlots = 65, kTrWgs = 256;
#ifdef RIVER_PHASE_TRACE
static __device__ unsigned long long g_phase_ts[kTrSteps * kTrSlots * RIVER_EV_COUNT * kTrWgs];
#define RIVER_TS(step, slot, ev)                                                                   \
  do {                                                                                             \
    if (threadIdx.x == 0 && (step) < kTrSteps && (slot) < kTrSlots && blockIdx.x < kTrWgs)        \
      g_phase_ts[(((size_t)(step) * kTrSlots + (slot)) * RIVER_EV_COUNT + (ev)) * kTrWgs + blockIdx.x] = \
          __builtin_amdgcn_s_memrealtime();                                                        \
  } while (0)
#else
#define RIVER_TS(step, slot, ev) \
  do {                           \
  } while (0)
#endif

struct StreamOut {
  uint32_t* out;      // tagged output: QKV -> q|k|v, O -> h_mid, GU -> SwiGLU vector, DOWN -> h(l)
  uint32_t tag;       // its tag
  f16* copy;          // DOWN: plain copy of h(l) (the residual stream kept for inspection)
  const f16* pres;    // O, DOWN: residual input, plain (the embedding row) ...
  const uint32_t* tres;  // ... or tagged
  uint32_t rtag;
  int* abort;
  float* logits;      // LM (optional)
  unsigned long long* key;  // LM argmax key
  int tr_step, tr_slot, tr_ev;  // phase trace: where the staged-input timestamp goes
};

template <bool IS4>
RIVER_DEV int n_chunks(int K) {
  return IS4 ? (K + kChunkW4 - 1) / kChunkW4 : (K + kChunkF16 - 1) / kChunkF16;
}

// Streams this wave's rows of an N-row phase; the input vector is staged in xl and the first
// item is already in b0 (prefetch_first).
template <int OP, bool IS4, int SEG, int GRP, bool ZP = false>
RIVER_DEV void stream_rows(const DecodeArgs& a, const LayerDev* lw, int N, int K, const h2* xl,
                           const float* xc, const float* xs, const StreamOut& so, Seg<SEG>& b0) {
  const int lane = threadIdx.x & (kWave - 1);
  const RowRange rr = wave_range<OP>(N);
  if (rr.nv <= 0) return;
  const int r0 = rr.r0, r1 = rr.r0 + rr.nv;  // contiguous for every phase but gate|up
  const int nch = n_chunks<IS4>(K);
  // residuals of this wave's rows, one per lane (O and DOWN)
  auto resid = [&](int row) {
    return so.pres ? ldg2(so.pres + row) : ld_tag1(so.tres + row, so.rtag, so.abort);
  };
  f16 res = (f16)0.0f;
  if ((OP == OP_O || OP == OP_DOWN) && r0 + lane < r1) res = resid(r0 + lane);
  float best = -__builtin_inff();
  int bi = 0x7FFFFFFF;
  float gk = 0.f;  // gate|up: gate row r0 + lane of this wave (its value before rounding)
  auto fin = [&](int vrow, float part) {
    const float v = wave_sum_fast(part);
    if (OP == OP_GU) {
      // a2[j] = fp16(silu(fp16(gate_j)) * fp16(up_j)), stored by the wave holding both
      if (vrow < rr.split) {
        if (lane == vrow) gk = v;
      } else {
        const int j = vrow - rr.split;
        const float g0 = h2f(f2h(__shfl(gk, j, kWave)));
        if (lane == 0) st_tag(so.out + r0 + j, f2h(g0 / (1.f + __expf(-g0)) * h2f(f2h(v))), so.tag);
      }
      return;
    }
    const int row = r0 + vrow;
    if (OP == OP_LM) {
      if (v > best) {
        best = v;
        bi = row;
      }
    }
    f16 rv = (f16)0.0f;
    if (OP == OP_O || OP == OP_DOWN) {
      const int src = vrow < kWave ? vrow : 0;
      rv = __builtin_bit_cast(f16, (unsigned short)__shfl(__builtin_bit_cast(unsigned short, res), src, kWave));
      if (vrow >= kWave) rv = resid(row);
    }
    if (lane == 0) {
      if (OP == OP_QKV) st_tag(so.out + row, f2h(v), so.tag);
      if (OP == OP_O || OP == OP_DOWN) {
        const f16 h = f2h(h2f(rv) + h2f(f2h(v)));
        st_tag(so.out + row, h, so.tag);
        if (OP == OP_DOWN) so.copy[row] = h;
      }
      if (OP == OP_LM && so.logits) so.logits[row] = v;
    }
  };
  Seg<SEG> b1;
  float acc = 0.f;
  if constexpr (!IS4) {
    const W16 w = w16_ptrs<OP>(a, lw);
    const int nseg = (nch + SEG - 1) / SEG;
    const int nitems = rr.nv * nseg;
    auto step = [&](int it, const Seg<SEG>& sg) {
      const int seg = it % nseg;
      acc = dot_seg16<SEG>(sg, xl, nch, seg, acc);
      if (seg == nseg - 1) {
        fin(it / nseg, acc);
        acc = 0.f;
      }
    };
    auto load = [&](int it, Seg<SEG>& sg) { load_seg16<OP, SEG>(w, a.dm, K, nch, rr.row(it / nseg), it % nseg, sg); };
    // Two buffers in a ring (b0 holds item 0). In the steady state no load is conditional, so
    // each wait covers only the item it reduces; the last one or two items follow. (Fencing
    // the stages from the scheduler as well measured slower here: more registers spilled.)
    int it = 0;
    for (; it + 2 < nitems; it += 2) {
      load(it + 1, b1);
      step(it, b0);
      load(it + 2, b0);
      step(it + 1, b1);
    }
    if (it + 1 < nitems) load(it + 1, b1);
    step(it, b0);
    if (it + 1 < nitems) step(it + 1, b1);
  } else {
    const uint8_t* base;
    const f16* sbase;
    const uint8_t* zbase;
    w4_base<OP>(lw, base, sbase, zbase);
    const int qend = rr.nv * nch;  // virtual chunks
    int row = 0, ch = 0;
    base = uniform_ptr(base);
    sbase = uniform_ptr(sbase);
    zbase = uniform_ptr(zbase);
    int q = 0;
    for (; q + 2 * SEG < qend; q += 2 * SEG) {  // the ring of the fp16 stream
      load_seg4<SEG, GRP, ZP>(base, sbase, zbase, rr, nch, q + SEG, qend, b1);
      dot_seg4<SEG, GRP, ZP>(b0, xl, xc, xs, nch, q, qend, row, ch, acc, fin);
      load_seg4<SEG, GRP, ZP>(base, sbase, zbase, rr, nch, q + 2 * SEG, qend, b0);
      dot_seg4<SEG, GRP, ZP>(b1, xl, xc, xs, nch, q + SEG, qend, row, ch, acc, fin);
    }
    if (q + SEG < qend) load_seg4<SEG, GRP, ZP>(base, sbase, zbase, rr, nch, q + SEG, qend, b1);
    dot_seg4<SEG, GRP, ZP>(b0, xl, xc, xs, nch, q, qend, row, ch, acc, fin);
    if (q + SEG < qend) dot_seg4<SEG, GRP, ZP>(b1, xl, xc, xs, nch, q + SEG, qend, row, ch, acc, fin);
  }
  if (OP == OP_LM && lane == 0 && bi != 0x7FFFFFFF) {
    const unsigned long long key = ((unsigned long long)float_key(best) << 32) |
                                   (unsigned long long)(0xFFFFFFFFu - (uint32_t)bi);
    __hip_atomic_fetch_max(so.key, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Issues the first item of this wave's rows (weights only: allowed before the inputs of the
// phase exist, e.g. before the grid barrier or while the input vector is staged).
template <int OP, bool IS4, int SEG, int GRP, bool ZP = false>
RIVER_DEV void prefetch_first(const DecodeArgs& a, const LayerDev* lw, int N, int K, Seg<SEG>& pre) {
  const RowRange rr = wave_range<OP>(N);
  if (rr.nv <= 0) {  // no rows: still define the whole buffer
#pragma unroll
    for (int c = 0; c < SEG; ++c) pre.w[c] = make_uint4(0, 0, 0, 0);
    pre.sr = make_uint4(0, 0, 0, 0);
    return;
  }
  const int nch = n_chunks<IS4>(K);
  if constexpr (!IS4) {
    load_seg16<OP, SEG>(w16_ptrs<OP>(a, lw), a.dm, K, nch, rr.row(0), 0, pre);
  } else {
    const uint8_t* base;
    const f16* sbase;
    const uint8_t* zbase;
    w4_base<OP>(lw, base, sbase, zbase);
    load_seg4<SEG, GRP, ZP>(base, sbase, zbase, rr, nch, 0, rr.nv * nch, pre);
  }
}

// One GEMV phase: stage the input (waiting for its tagged words), stream the rows. b0 holds the
// phase's first item when `have` (issued at the end of the previous phase), else it is issued
// here first.
template <int OP, bool IS4, int SEG, bool HAS_GAIN, bool NORM, bool TAG, int NG, int GRP, bool ZP = false>
RIVER_DEV void gemv_phase(const DecodeArgs& a, const LayerDev* lw, int N, int K, const void* src,
                          uint32_t stag, const f16* gain, float inv, const StreamOut& so, h2* xl,
                          float* xc, float* xs, double* red, Seg<SEG>& b0, bool have) {
  if (!have) prefetch_first<OP, IS4, SEG, GRP, ZP>(a, lw, N, K, b0);
  stage_x<IS4, HAS_GAIN, NORM, TAG, NG, ZP>(src, stag, so.abort, gain, K, inv, a.dm.eps, xl, xc, xs, red);
  RIVER_TS(so.tr_step, so.tr_slot, so.tr_ev);
  stream_rows<OP, IS4, SEG, GRP, ZP>(a, lw, N, K, xl, xc, xs, so, b0);
  __syncthreads();  // LDS reuse by the next phase
}

// First item of the next phase on the route's weight stream; returns what `pre` now holds
// (1: fp16 item, 2: int4 item).
template <int OP, int SEG, int GRP, bool ZP = false>
RIVER_DEV int prefetch_route(const DecodeArgs& a, const LayerDev* lw, int N, int K, bool r4, Seg<SEG>& pre) {
  if (r4) {
    prefetch_first<OP, true, SEG, GRP, ZP>(a, lw, N, K, pre);
    return 2;
  }
  prefetch_first<OP, false, SEG, GRP>(a, lw, N, K, pre);
  return 1;
}

// ---------------------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------------------
template <int D, int G, int MODE, int SEG16, int SEG4, int NG, int GRP, int AU, bool ZP = false>
__global__ __launch_bounds__(kPB) void k_persist(DecodeArgs a, int S, int splits, unsigned* bar) {
  static_assert(SEG16 == SEG4, "one prefetch buffer serves both weight streams");
  constexpr int SEG = SEG16;
  constexpr int AGL = RIVER_PATTN_GL < G ? RIVER_PATTN_GL : G;
  __shared__ PSmem<D, G> sm;
  const Dims& dm = a.dm;
  const int b = 0;
  const unsigned nwg = gridDim.x;
  const int wg = blockIdx.x, t = threadIdx.x;
  unsigned epoch = 0;
  int pos = a.pos[b];
  int tok = a.tok_in[b];
  h2* xl = sm.x;
  Seg<SEG> pre;  // first weight item of the next GEMV phase, issued at the end of the previous one
  int pf = 0;    // what `pre` holds: 0 nothing, 1 fp16 item, 2 int4 item
  int* abort = (int*)(bar + kBarAbort);
  // Use tags: (step, layer) of this launch. The counter advances by S*(L+1) per launch (at the
  // end), so tags continue across launches and graph replays; 0 is never a tag.
  const uint32_t tbase = __hip_atomic_load(a.tagc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t tbase32 = __hip_atomic_load(a.tagc + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  auto tag_of = [&](int st, int l) { return 1u + (tbase + (uint32_t)(st * (dm.L + 1) + l)) % 65535u; };
  // attention partials: a slot may go unwritten for many uses (a split past the context), so
  // their tag is 32 bits wide

  for (int step = 0; step < S; ++step, ++pos) {
    if (tok < 0 || tok >= dm.V) {
      if (wg == 0 && t == 0) atomicOr(a.err, ERR_TOKEN);
      tok = 0;
    }
    const f16* emb = a.embed + (size_t)tok * dm.d;  // h(0)
    int e_forced = dm.L;
    if (MODE == 0 && a.sched) {
      e_forced = a.sched[step * dm.B + b];
      if ((e_forced < dm.entry && e_forced != 0) || e_forced > dm.L) {  // 0: every block on the river
        if (wg == 0 && t == 0) atomicOr(a.err, ERR_FORCED);
        e_forced = dm.L;
      }
    }
    int route = ROUTE_BACKBONE;
    for (int l = 1; l <= dm.L; ++l) {
      const LayerDev* lw = &a.layers[l - 1];
      const uint32_t tg = tag_of(step, l), tgp = tag_of(step, l - 1);
      const uint32_t* hin_t = a.t_hs + (size_t)(l - 1) * dm.d;  // h(l-1), l > 1
      uint32_t* hmid_t = a.t_hmid + (size_t)(l - 1) * dm.d;
      uint32_t* o_t = a.t_o + (size_t)(l & 1) * dm.hd;  // two buffers by layer parity
      // ---------------- QKV (exit test after block l-1 first)
      RIVER_TS(step, l - 1, RIVER_EV_START);
      bool norm_known = false;
      float inv = 1.f;
      if (l == 1) {
        if (wg == 0) {
          f16* h0 = a.hs + (size_t)b * dm.d;
          for (int i = t; i < dm.d; i += kPB) h0[i] = emb[i];
          if (t == 0 && a.exit_out) a.exit_out[step * dm.B + b] = dm.L;
          if (a.sim_out)
            for (int i = t; i < dm.L; i += kPB)
              a.sim_out[((size_t)step * dm.B + b) * dm.L + i] = __builtin_nanf("");
        }
        if (MODE == 0 && a.sched && e_forced == 0) {  // no backbone block at all
          route = ROUTE_RIVER;
          if (wg == 0 && t == 0 && a.exit_out) a.exit_out[step * dm.B + b] = 0;
        }
      } else if (MODE == 0 && route == ROUTE_BACKBONE && l - 1 >= dm.entry) {
        const int lp = l - 1;
        if (a.sched) {
          if (lp == e_forced) route = ROUTE_RIVER;
        } else {
          double dot, n1, n2;
          block_cos(lp == 1 ? emb : nullptr, lp == 1 ? nullptr : a.t_hs + (size_t)(lp - 1) * dm.d,
                    tag_of(step, lp - 1), hin_t, tgp, abort, dm.d, sm.red, dot, n1, n2);
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
      so.abort = abort;
      so.out = a.t_qkv;
      so.tag = tg;
      so.tr_step = step;
      so.tr_slot = l - 1;
      so.tr_ev = RIVER_EV_QKV_STAGED;
      if (l == 1) {
        if (r4) gemv_phase<OP_QKV, true, SEG, true, true, false, NG, GRP, ZP>(a, lw, dm.nqkv, dm.d, emb, 0, lw->attn_norm, inv, so, xl, sm.xc, sm.xs, sm.red, pre, pf == 2);
        else gemv_phase<OP_QKV, false, SEG, true, true, false, NG, GRP, ZP>(a, lw, dm.nqkv, dm.d, emb, 0, lw->attn_norm, inv, so, xl, sm.xc, sm.xs, sm.red, pre, pf == 1);
      } else if (r4) {
        if (norm_known) gemv_phase<OP_QKV, true, SEG, true, false, true, NG, GRP, ZP>(a, lw, dm.nqkv, dm.d, hin_t, tgp, lw->attn_norm, inv, so, xl, sm.xc, sm.xs, sm.red, pre, pf == 2);
        else gemv_phase<OP_QKV, true, SEG, true, true, true, NG, GRP, ZP>(a, lw, dm.nqkv, dm.d, hin_t, tgp, lw->attn_norm, inv, so, xl, sm.xc, sm.xs, sm.red, pre, pf == 2);
      } else {
        if (norm_known) gemv_phase<OP_QKV, false, SEG, true, false, true, NG, GRP, ZP>(a, lw, dm.nqkv, dm.d, hin_t, tgp, lw->attn_norm, inv, so, xl, sm.xc, sm.xs, sm.red, pre, pf == 1);
        else gemv_phase<OP_QKV, false, SEG, true, true, true, NG, GRP, ZP>(a, lw, dm.nqkv, dm.d, hin_t, tgp, lw->attn_norm, inv, so, xl, sm.xc, sm.xs, sm.red, pre, pf == 1);
      }
      RIVER_TS(step, l - 1, RIVER_EV_QKV_END);
      // ---------------- attention (+ RoPE and the KV append of position pos); waits for q|k|v
      {
        const AttnTag at{a.t_qkv, o_t, tg, a.t_part, tbase32 + (uint32_t)(step * (dm.L + 1) + l), abort};
        for (int it = wg; it < dm.Hkv * splits; it += nwg)
          attn_split<D, G, kPB, true, AU, AGL, true>(a, l, it % splits, it / splits, b, pos, splits, sm.at, at);
      }
      RIVER_TS(step, l - 1, RIVER_EV_ATT_END);
      pf = prefetch_route<OP_O, SEG, GRP, ZP>(a, lw, dm.d, dm.hd, r4, pre);
      // ---------------- O + residual
      so = StreamOut{};
      so.abort = abort;
      so.out = hmid_t;
      so.tag = tg;
      so.tr_step = step;
      so.tr_slot = l - 1;
      so.tr_ev = RIVER_EV_O_STAGED;
      if (l == 1) {
        so.pres = emb;
      } else {
        so.tres = hin_t;
        so.rtag = tgp;
      }
      if (r4) gemv_phase<OP_O, true, SEG, false, false, true, NG, GRP, ZP>(a, lw, dm.d, dm.hd, o_t, tg, nullptr, 1.f, so, xl, sm.xc, sm.xs, sm.red, pre, pf == 2);
      else gemv_phase<OP_O, false, SEG, false, false, true, NG, GRP, ZP>(a, lw, dm.d, dm.hd, o_t, tg, nullptr, 1.f, so, xl, sm.xc, sm.xs, sm.red, pre, pf == 1);
      // The argmax key of the next step is the one every workgroup read after the previous
      // step's barrier; having staged all of o, this workgroup knows every split (hence every
      // workgroup) has passed this step's layer-1 attention, so none still reads that key.
      if (l == 1 && wg == 0 && t == 0)
        __hip_atomic_store(a.amax + ((step + 1) & 1) * dm.B + b, 0ull, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      RIVER_TS(step, l - 1, RIVER_EV_O_END);
      pf = prefetch_route<OP_GU, SEG, GRP, ZP>(a, lw, 2 * dm.F, dm.d, r4, pre);
      // ---------------- gate|up (+ SwiGLU in the epilogue)
      so = StreamOut{};
      so.abort = abort;
      so.out = a.t_a2;
      so.tag = tg;
      so.tr_step = step;
      so.tr_slot = l - 1;
      so.tr_ev = RIVER_EV_GU_STAGED;
      if (r4) gemv_phase<OP_GU, true, SEG, true, true, true, NG, GRP, ZP>(a, lw, 2 * dm.F, dm.d, hmid_t, tg, lw->mlp_norm, 1.f, so, xl, sm.xc, sm.xs, sm.red, pre, pf == 2);
      else gemv_phase<OP_GU, false, SEG, true, true, true, NG, GRP, ZP>(a, lw, 2 * dm.F, dm.d, hmid_t, tg, lw->mlp_norm, 1.f, so, xl, sm.xc, sm.xs, sm.red, pre, pf == 1);
      RIVER_TS(step, l - 1, RIVER_EV_GU_END);
      pf = prefetch_route<OP_DOWN, SEG, GRP, ZP>(a, lw, dm.d, dm.F, r4, pre);
      // ---------------- down (input: the SwiGLU vector) + residual -> h(l)
      so = StreamOut{};
      so.abort = abort;
      so.out = a.t_hs + (size_t)l * dm.d;
      so.tag = tg;
      so.tr_step = step;
      so.tr_slot = l - 1;
      so.tr_ev = RIVER_EV_DN_STAGED;
      so.copy = a.hs + ((size_t)l * dm.B + b) * dm.d;
      so.tres = hmid_t;
      so.rtag = tg;
      if (r4) gemv_phase<OP_DOWN, true, SEG, false, false, true, NG, GRP, ZP>(a, lw, dm.d, dm.F, a.t_a2, tg, nullptr, 1.f, so, xl, sm.xc, sm.xs, sm.red, pre, pf == 2);
      else gemv_phase<OP_DOWN, false, SEG, false, false, true, NG, GRP, ZP>(a, lw, dm.d, dm.F, a.t_a2, tg, nullptr, 1.f, so, xl, sm.xc, sm.xs, sm.red, pre, pf == 1);
      RIVER_TS(step, l - 1, RIVER_EV_DN_END);
      // next phase: QKV of layer l+1 on its route (the exit test may still switch a backbone
      // guess to the river, which then loads its own first item) or the LM head
      const bool next_r4 = r4 || (MODE == 0 && a.sched && l == e_forced && l >= dm.entry);
      if (l < dm.L) {
        pf = prefetch_route<OP_QKV, SEG, GRP, ZP>(a, &a.layers[l], dm.nqkv, dm.d, next_r4, pre);
      } else {
        prefetch_first<OP_LM, false, SEG, GRP>(a, nullptr, dm.V, dm.d, pre);
        pf = 1;
      }
    }
    // ---------------- LM head (final RMSNorm while staging) + argmax; the one grid barrier of
    // a step (every workgroup needs the whole argmax)
    {
      RIVER_TS(step, dm.L, RIVER_EV_START);
      StreamOut so{};
      so.abort = abort;
      so.logits = a.logits ? a.logits + (size_t)b * dm.V : nullptr;
      so.key = a.amax + (step & 1) * dm.B + b;
      so.tr_step = step;
      so.tr_slot = dm.L;
      so.tr_ev = RIVER_EV_QKV_STAGED;
      gemv_phase<OP_LM, false, SEG, true, true, true, NG, GRP, ZP>(a, nullptr, dm.V, dm.d, a.t_hs + (size_t)dm.L * dm.d,
                                                               tag_of(step, dm.L), a.final_norm, 1.f, so, xl, sm.xc, sm.xs, sm.red, pre, pf == 1);
      RIVER_TS(step, dm.L, RIVER_EV_QKV_END);
      grid_sync(bar, epoch, nwg, [&] { pf = prefetch_route<OP_QKV, SEG, GRP, ZP>(a, &a.layers[0], dm.nqkv, dm.d, false, pre); });
      RIVER_TS(step, dm.L, RIVER_EV_ATT_END);
      const unsigned long long k = __hip_atomic_load(so.key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      tok = (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
      if (wg == 0 && t == 0) a.tok_out[step * dm.B + b] = tok;
    }
  }
  if (wg == 0 && t == 0) {  // every workgroup read the tag counter before the last barrier
    a.pos[b] = pos;
    *a.step = S;
    __hip_atomic_store(a.tagc, (tbase + (uint32_t)(S * (dm.L + 1))) % 65535u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.tagc + 1, tbase32 + (uint32_t)(S * (dm.L + 1)), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (__hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicOr(a.err, ERR_SYNC);
  }
}

// ---------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------
// The kernel function for this model and mode (batch 1, GEMV inputs up to 16384), or null.
// `long_ctx`: the variant for launches that reach position kPersistLongCtx, whose attention
// keeps twice the K/V in flight per lane (a separate kernel: carrying both loop shapes in one
// costs the short-context case registers).
const void* river_persist_fn(const Dims& dm, int mode, int long_ctx) {
  if (dm.B != 1 || dm.d > kMaxK || dm.hd > kMaxK || dm.F > kMaxK) return nullptr;
  // tagged vectors are read in groups of 8 words; the split merge needs G*D a power of two
  if (dm.d % 8 || dm.hd % 8 || dm.F % 8) return nullptr;
  const int G = dm.H / dm.Hkv;
  if ((G & (G - 1)) || (dm.D & (dm.D - 1))) return nullptr;
  const int ng = (dm.d + 8 * kPB - 1) / (8 * kPB);  // groups of 8 per thread for K = d
  // the zero-point format has its own early-exit kernels (the backbone-only decode reads no river)
#define RIVER_PF(D_, G_, NG_, GRP_)                                                              \
  if (dm.D == D_ && G == G_ && ng == NG_ && dm.group == GRP_) {                                  \
    if (long_ctx)                                                                                \
      return mode ? (const void*)k_persist<D_, G_, 1, 8, 8, NG_, GRP_, 4>                       \
             : dm.zp ? (const void*)k_persist<D_, G_, 0, 8, 8, NG_, GRP_, 4, true>              \
                     : (const void*)k_persist<D_, G_, 0, 8, 8, NG_, GRP_, 4>;                   \
    return mode ? (const void*)k_persist<D_, G_, 1, 8, 8, NG_, GRP_, 2>                         \
           : dm.zp ? (const void*)k_persist<D_, G_, 0, 8, 8, NG_, GRP_, 2, true>                \
                   : (const void*)k_persist<D_, G_, 0, 8, 8, NG_, GRP_, 2>;                     \
  }
  RIVER_PF(128, 4, 1, 128)
  RIVER_PF(64, 4, 1, 128)
  RIVER_PF(64, 2, 1, 64)
#undef RIVER_PF
  return nullptr;
}

// Workgroups of the persistent grid: one per CU, all co-resident (cooperative launch).
int river_persist_grid(const void* fn) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kPB, 0) != hipSuccess) return 0;
  return (per_cu >= 1 && cus <= kBarGroup * kBarMaxGroups) ? cus : 0;
}

hipError_t river_launch_persist(const void* fn, const DecodeArgs& a, int S, int nwg, int splits,
                                unsigned* bar, hipStream_t st) {
  DecodeArgs aa = a;
  int SS = S, sp = splits;
  unsigned* br = bar;
  void* args[] = {&aa, &SS, &sp, &br};
  return hipLaunchCooperativeKernel(fn, dim3(nwg), dim3(kPB), args, 0, st);
}

// ---------------------------------------------------------------------------------------
// Fixed device scratch of river_decode_steps_static, for callers that cannot allocate device
// memory (code under graph capture, serving loops, harnesses that forbid it): the persistent
// kernel's cross-workgroup exchange buffers (tagged activations, split partials, tag counters,
// grid-barrier words, argmax keys) live in this file-scope array instead of the context's
// scratch. Every GPU the library runs on holds its own copy until the process ends. In host
// code the array's name is only a stand-in for the symbol: kernels get the device address
// that river_static_scratch looks up.
// ---------------------------------------------------------------------------------------
static constexpr size_t kStaticScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Device address and size of the current GPU's copy of `scratch`; looked up once per device
// (with that device current) and remembered.
// Phase trace (debug build): copies the timestamp array to host memory; its shape goes to
// dims[4] = {steps, slots, events, workgroups}. The release build reports hipErrorNotSupported.
hipError_t river_phase_trace_copy(unsigned long long* dst, size_t n, int* dims) {
  dims[0] = kTrSteps;
  dims[1] = kTrSlots;
  dims[2] = RIVER_EV_COUNT;
  dims[3] = kTrWgs;
#ifdef RIVER_PHASE_TRACE
  const size_t total = (size_t)kTrSteps * kTrSlots * RIVER_EV_COUNT * kTrWgs;
  if (!dst) return hipSuccess;
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_phase_ts), (n < total ? n : total) * 8, 0, hipMemcpyDeviceToHost);
#else
  (void)dst;
  (void)n;
  return hipErrorNotSupported;
#endif
}

hipError_t river_static_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}
