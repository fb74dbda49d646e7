// Split-K GQA decode attention over the shared KV cache (one query position per row).
//
// Both River-LLM routes of a layer (the fp16 backbone block and its W4A16 exit-river copy)
// read and write the same cache, so attention is route-independent: softmax(q K^T / sqrt(D)) V
// over positions 0..pos of the query's KV head (River-LLM paper, Method: KV sharing between
// backbone and exit river).
//
// Work split: workgroup `s` of KV head `kvh` owns positions [s*chunk, min(T, (s+1)*chunk)).
// Lane layout: a "slot" of LPP = (G/GL)*D/8 lanes owns one position at a time; inside it,
// D/8 lanes (8 dims each, one 16-byte K and V load per lane) serve GL query heads of the KV
// group. Every thread takes U positions per block; the first block's K/V loads, the q loads
// and (persistent path) the new position's k/v are all issued before any of them is used, and
// each later block is loaded while the previous one is reduced. Scores are summed across the
// D/8 lanes with DPP row permutations; softmax is exact per block and merged online (exp2
// domain). The slots merge in LDS, and the last-arriving split of a head merges all splits of
// it (one wave per query head for the weights, one batch of partial loads per thread for the
// output).
#pragma once

#include "common.hpp"
#include "gemv.hpp"
#include "params.hpp"

static constexpr int kMaxSplit = 64;  // partial-result slots per (row, query head)
static constexpr int kAttnMinChunk = 64;

// LDS of one attention split: per-slot softmax state (slots = position lanes of the workgroup;
// GL query heads per lane, see attn_split), the split weights of the final merge, a flag.
template <int D, int G, int NT, int GL = G>
struct AttnLds {
  static constexpr int NS = (NT / kWave) * (kWave / ((G / GL) * (D / 8)));
  float acc[NS][G][D];
  float m[NS][G];
  float l[NS][G];
  float w[G][kMaxSplit];
  int flag;
};

// Tagged mode of the persistent kernel: q/k/v are read from tagged words (the QKV phase's
// output, polled: no grid barrier before attention). Each split publishes its partial result
// as 64-bit words (fp32 value | 32-bit use tag << 32) -- a split with no positions publishes an
// empty one -- and every split workgroup of the KV head then merges its own slice of the head
// group's G*D outputs from all splits' partials (polled; one cross-lane reduction over the
// splits, no counter, no last arriver), writing them as tagged words. Every workgroup thus
// publishes something each layer that the next phase's inputs depend on.
struct AttnTag {
  const uint32_t* qkv;       // [nqkv] tagged q|k|v of this layer
  uint32_t* o;               // [H*D] tagged merged output
  uint32_t tag;              // 16-bit tag of this layer's use of both
  unsigned long long* part;  // [H][nsplit][D+2] split partials: acc[D], then max, sum
  uint32_t tag32;            // tag of this layer's partials
  int* abort;
};

RIVER_DEV void st_part(unsigned long long* p, float v, uint32_t tag32) {
  __hip_atomic_store((g_u64*)p, ((unsigned long long)tag32 << 32) | __builtin_bit_cast(uint32_t, v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// (max, sum) and, when `acc` is set, one accumulator of a split's partial, once all three
// carry tag32 (one round trip; see ld_tag8n for the bounded wait).
RIVER_DEV void ld_part3(const unsigned long long* pm, const unsigned long long* pa, bool acc,
                        uint32_t tag32, int* abort, float& m, float& l, float& av) {
  unsigned long long w0, w1, w2 = (unsigned long long)tag32 << 32;
  w0 = __hip_atomic_load((g_u64*)pm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  w1 = __hip_atomic_load((g_u64*)pm + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (acc) w2 = __hip_atomic_load((g_u64*)pa, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  unsigned spins = 0;
  while (true) {
    const bool o0 = (uint32_t)(w0 >> 32) == tag32, o1 = (uint32_t)(w1 >> 32) == tag32,
               o2 = (uint32_t)(w2 >> 32) == tag32;
    if ((o0 & o1 & o2) || tag_spin(spins, abort)) break;
    if (!o0) w0 = __hip_atomic_load((g_u64*)pm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!o1) w1 = __hip_atomic_load((g_u64*)pm + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!o2) w2 = __hip_atomic_load((g_u64*)pa, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  m = __builtin_bit_cast(float, (uint32_t)w0);
  l = __builtin_bit_cast(float, (uint32_t)w1);
  av = acc ? __builtin_bit_cast(float, (uint32_t)w2) : 0.f;
}

RIVER_DEV float4 ld4_coh(const float* p) {
  const uint4 u = ldx16<true>(p);
  return make_float4(__builtin_bit_cast(float, u.x), __builtin_bit_cast(float, u.y),
                     __builtin_bit_cast(float, u.z), __builtin_bit_cast(float, u.w));
}

// One split of one KV head for row b at position pos (T = pos + 1 positions).
//   ROPE = false: rotated q is in a.q and K/V[pos] is already in the cache (per-op path).
//   ROPE = true : un-rotated q/k/v are in a.qkvr (persistent path): q is rotated here; the
//                 split that owns position pos rotates k, uses k/v of pos from registers and
//                 appends them to the cache; activations move through agent-coherent accesses.
template <int D, int G, int NT, bool ROPE, int UP = 4, int GLP = G, bool TG = false>
RIVER_DEV void attn_split(const DecodeArgs& a, int layer, int s, int kvh, int b, int pos, int nsplit,
                          AttnLds<D, G, NT, GLP>& sm, const AttnTag& tg = AttnTag{}) {
  static_assert(!TG || ROPE, "tagged mode is the persistent kernel's");
  constexpr bool COH = ROPE;
  constexpr int LPT = D / 8;                       // lanes per head (8 dims each)
  constexpr int GL = GLP;                          // query heads per lane
  constexpr int HG = G / GL;                       // head groups per slot
  constexpr int LPP = HG * LPT;                    // lanes per slot
  constexpr int SPW = kWave / LPP;                 // slots per wave
  constexpr int NW = NT / kWave;
  constexpr int NS = NW * SPW;                     // slots per workgroup
  constexpr int U = UP;                            // positions per thread per block
  constexpr int BLK = NS * U;
  constexpr int NCOL = G * D / 4;                  // float4 columns of the merged output
  constexpr int TPC = NT / NCOL;                   // threads per column in the split merge
  constexpr int MB = (kMaxSplit / TPC < 8) ? kMaxSplit / TPC : 8;  // partial loads per batch
  static_assert(LPP <= kWave && HG * GL == G && (LPP & (LPP - 1)) == 0, "lane layout");
  static_assert(NCOL <= NT && (TPC & (TPC - 1)) == 0 && TPC <= kWave, "merge layout");
  const Dims& dm = a.dm;
  const int T = pos + 1;
  const int chunk = max(kAttnMinChunk, (T + nsplit - 1) / nsplit);
  const int seff = (T + chunk - 1) / chunk;
  const size_t hstride = (size_t)dm.Tmax * D;
  f16* Kb = a.kv + ((((size_t)(layer - 1) * 2 + 0) * dm.B + b) * dm.Hkv + kvh) * hstride;
  f16* Vb = a.kv + ((((size_t)(layer - 1) * 2 + 1) * dm.B + b) * dm.Hkv + kvh) * hstride;
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const int slot = w * SPW + lane / LPP;
  const int hg = (lane % LPP) / LPT;
  const int sub = lane % LPT, d0 = sub * 8;
  const size_t pbase = ((size_t)b * dm.H + (size_t)kvh * G) * nsplit;  // + g*nsplit + split

  if (s < seff) {
    const int t0 = s * chunk, t1 = min(T, t0 + chunk);
    const bool owner = ROPE && t1 == T;  // this split holds the new position

    auto load_block = [&](int tb, uint4 (&kk)[U], uint4 (&vv)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = tb + slot + u * NS;
        // past the split (masked later) or the new position of the persistent path (taken
        // from registers below): read a harmless in-range row instead
        const size_t tt = (size_t)((t < t1 && !(ROPE && t == pos)) ? t : t0);
        kk[u] = ldg16(Kb + tt * D + d0);
        vv[u] = ldg16(Vb + tt * D + d0);
      }
    };
    uint4 kc[U], vc[U];
    load_block(t0, kc, vc);

    float2 cs[8];
    if (ROPE) {
      const float2* rope = a.rope + (size_t)pos * (D / 2);
#pragma unroll
      for (int i = 0; i < 8; ++i) cs[i] = rope[(d0 + i) % (D / 2)];
    }
    // q of this lane's GL heads, dims [d0, d0+8)
    const f16* qkv = a.qkvr + (size_t)b * dm.nqkv;
    uint4 qraw[GL];
    uint4 kraw = make_uint4(0, 0, 0, 0), vpos = make_uint4(0, 0, 0, 0);
    const size_t ki = dm.hd + (size_t)kvh * D + d0, vi = dm.hd + (size_t)(dm.Hkv + kvh) * D + d0;
    if constexpr (TG) {  // q of the lane's heads (and k, v of pos for the owner) in one wait
      const uint32_t* pp[GL + 2];
      bool use[GL + 2];
      uint4 got[GL + 2];
#pragma unroll
      for (int gl = 0; gl < GL; ++gl) {
        pp[gl] = tg.qkv + (size_t)(kvh * G + hg * GL + gl) * D + d0;
        use[gl] = true;
      }
      pp[GL] = tg.qkv + ki;
      pp[GL + 1] = tg.qkv + vi;
      use[GL] = use[GL + 1] = owner;
      ld_tag8n<GL + 2>(pp, use, tg.tag, tg.abort, got);
#pragma unroll
      for (int gl = 0; gl < GL; ++gl) qraw[gl] = got[gl];
      kraw = got[GL];
      vpos = got[GL + 1];
    } else {
#pragma unroll
      for (int gl = 0; gl < GL; ++gl) {
        const int g = hg * GL + gl;
        const size_t qi = (size_t)(kvh * G + g) * D + d0;
        qraw[gl] = ROPE ? ldx16<true>(qkv + qi) : ldg16(a.q + (size_t)b * dm.hd + qi);
      }
      if (owner) {
        kraw = ldx16<true>(qkv + ki);
        vpos = ldx16<true>(qkv + vi);
      }
    }
    // rotate-half RoPE of dims [d0, d0+8), rounded to fp16; the partner dims (d +- D/2) are
    // held by lane ^ LPT/2 of the same head
    auto rope8 = [&](uint4 raw) {
      const uint4 pr = make_uint4(__shfl_xor(raw.x, LPT / 2, kWave), __shfl_xor(raw.y, LPT / 2, kWave),
                                  __shfl_xor(raw.z, LPT / 2, kWave), __shfl_xor(raw.w, LPT / 2, kWave));
      const f16* x = (const f16*)&raw;
      const f16* y = (const f16*)&pr;
      uint4 out;
      f16* o = (f16*)&out;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xv = h2f(x[i]), yv = h2f(y[i]);
        o[i] = (d0 < D / 2) ? f2h(xv * cs[i].x - yv * cs[i].y) : f2h(xv * cs[i].x + yv * cs[i].y);
      }
      return out;
    };
    h2 qh[GL][4];
#pragma unroll
    for (int gl = 0; gl < GL; ++gl) {
      const uint4 u = ROPE ? rope8(qraw[gl]) : qraw[gl];
      qh[gl][0] = as_h2(u.x);
      qh[gl][1] = as_h2(u.y);
      qh[gl][2] = as_h2(u.z);
      qh[gl][3] = as_h2(u.w);
    }
    uint4 kpos = make_uint4(0, 0, 0, 0);
    if (owner) {
      kpos = rope8(kraw);
      if (w == 0 && lane < LPT) {  // append K/V[pos] to the shared cache
        const unsigned long long k2[2] = {kpos.x | ((unsigned long long)kpos.y << 32), kpos.z | ((unsigned long long)kpos.w << 32)};
        const unsigned long long v2[2] = {vpos.x | ((unsigned long long)vpos.y << 32), vpos.z | ((unsigned long long)vpos.w << 32)};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          __hip_atomic_store((g_u64*)(Kb + (size_t)pos * D + d0) + j, k2[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store((g_u64*)(Vb + (size_t)pos * D + d0) + j, v2[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        kv_count(a.kvcnt, a.kv, Kb + (size_t)pos * D + d0, 8);
        kv_count(a.kvcnt, a.kv, Vb + (size_t)pos * D + d0, 8);
      }
    }
    // scores are scaled by log2(e)/sqrt(D) after the fp32 dot (exact fp16 products)
    const float qs = 1.4426950408889634f / sqrtf((float)D);

    float m[GL], l[GL], acc[GL][8];
#pragma unroll
    for (int gl = 0; gl < GL; ++gl) {
      m[gl] = -__builtin_inff();
      l[gl] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[gl][i] = 0.f;
    }
    // one block of positions [tb, tb + BLK) from the registers kk/vv
    // (the new position's k/v come from registers: selected where used, the ring itself is
    // never written outside its loads)
    auto process = [&](int tb, const uint4 (&kr)[U], const uint4 (&vr)[U]) {
      if (tb + slot < t1) {  // the slot has a position in this block (uniform per slot)
        uint4 kk[U], vv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const bool np = owner && tb + slot + u * NS == pos;
          kk[u] = np ? kpos : kr[u];
          vv[u] = np ? vpos : vr[u];
        }
        float sc[U][GL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const h2 k0 = as_h2(kk[u].x), k1 = as_h2(kk[u].y), k2 = as_h2(kk[u].z), k3 = as_h2(kk[u].w);
#pragma unroll
          for (int gl = 0; gl < GL; ++gl)
            sc[u][gl] = dot2(qh[gl][3], k3, dot2(qh[gl][2], k2, dot2(qh[gl][1], k1, dot2(qh[gl][0], k0, 0.f))));
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int gl = 0; gl < GL; ++gl) {
            const float v = row_sum<LPT>(sc[u][gl]) * qs;
            sc[u][gl] = (tb + slot + u * NS < t1) ? v : -__builtin_inff();
          }
#pragma unroll
        for (int gl = 0; gl < GL; ++gl) {
          float mb = m[gl];
#pragma unroll
          for (int u = 0; u < U; ++u) mb = fmaxf(mb, sc[u][gl]);
          const float c = exp2f(m[gl] - mb);  // 0 while m is still -inf (mb is finite here)
          float p[U], ps = 0.f;
#pragma unroll
          for (int u = 0; u < U; ++u) {
            p[u] = exp2f(sc[u][gl] - mb);
            ps += p[u];
          }
          l[gl] = l[gl] * c + ps;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            float x = acc[gl][i] * c;
#pragma unroll
            for (int u = 0; u < U; ++u) x = fmaf(p[u], h2f(((const f16*)&vv[u])[i]), x);
            acc[gl][i] = x;
          }
          m[gl] = mb;
        }
      }
    };
    // Two register buffers in a ring: a block's loads are in flight while the previous one is
    // reduced. The loads are unconditional (positions past the split read a harmless in-range
    // row and are masked; a block past the end is a no-op) and the stages are fenced from the
    // scheduler, which would otherwise pull uses of a just-issued load ahead of the other
    // block's arithmetic and wait on it at once.
    uint4 kn[U], vn[U];
    for (int tb = t0; tb < t1; tb += 2 * BLK) {
      load_block(tb + BLK, kn, vn);
      __builtin_amdgcn_sched_barrier(0);
      process(tb, kc, vc);
      __builtin_amdgcn_sched_barrier(0);
      load_block(tb + 2 * BLK, kc, vc);
      __builtin_amdgcn_sched_barrier(0);
      process(tb + BLK, kn, vn);
      __builtin_amdgcn_sched_barrier(0);
    }
    // every slot's softmax state to LDS, then merge the NS slots per (query head, dim)
#pragma unroll
    for (int gl = 0; gl < GL; ++gl) {
      const int g = hg * GL + gl;
#pragma unroll
      for (int i = 0; i < 8; ++i) sm.acc[slot][g][d0 + i] = acc[gl][i];
      if (sub == 0) {
        sm.m[slot][g] = m[gl];
        sm.l[slot][g] = l[gl];
      }
    }
    __syncthreads();
    // write this split's partial (scaled to its own max) and (max, sum)
    for (int idx = tid; idx < G * D; idx += NT) {
      const int g = idx / D, dd = idx % D;
      float M = -__builtin_inff();
      for (int j = 0; j < NS; ++j)
        if (sm.l[j][g] > 0.f) M = fmaxf(M, sm.m[j][g]);
      float Ls = 0.f, A = 0.f;
      for (int j = 0; j < NS; ++j) {
        const float sc = (sm.l[j][g] > 0.f) ? exp2f(sm.m[j][g] - M) : 0.f;
        Ls += sm.l[j][g] * sc;
        A += sm.acc[j][g][dd] * sc;
      }
      if constexpr (TG) {
        unsigned long long* r = tg.part + ((size_t)(kvh * G + g) * nsplit + s) * (D + 2);
        st_part(r + dd, A, tg.tag32);
        if (dd == 0) {
          st_part(r + D, M, tg.tag32);
          st_part(r + D + 1, Ls, tg.tag32);
        }
      } else {
        const size_t pi = pbase + (size_t)g * nsplit + s;
        wt_store(&a.pacc[pi * D + dd], A);
        if (dd == 0) {
          wt_store(&a.pml[pi * 2 + 0], M);
          wt_store(&a.pml[pi * 2 + 1], Ls);
        }
      }
    }
  } else if constexpr (TG) {  // no positions in this split: an empty partial (max -inf, sum 0)
    for (int g = tid; g < G; g += NT) {
      unsigned long long* r = tg.part + ((size_t)(kvh * G + g) * nsplit + s) * (D + 2);
      st_part(r + D, -__builtin_inff(), tg.tag32);
      st_part(r + D + 1, 0.f, tg.tag32);
    }
  }

  if constexpr (TG) {
    // this workgroup's slice: VPW consecutive outputs of one query head (nsplit and G*D are
    // powers of two and nsplit >= G, so VPW divides D). Lanes [k*P, k*P + P) of a wave hold
    // splits 0..P-1 of one output; max, sum and the weighted sum reduce across them.
    const int P = nsplit;
    const int VPW = (G * D >= P) ? G * D / P : 1;
    const int v0 = s * VPW;
    if (v0 < G * D) {
      const int g = v0 / D, dbase = v0 % D;
      for (int idx = tid; idx < VPW * P; idx += NT) {
        const int j = idx % P, v = idx / P;
        const unsigned long long* r = tg.part + ((size_t)(kvh * G + g) * P + j) * (D + 2);
        float mj, lj, aj;
        ld_part3(r + D, r + dbase + v, j < seff, tg.tag32, tg.abort, mj, lj, aj);
        float M = mj;
        for (int o = 1; o < P; o <<= 1) M = fmaxf(M, __shfl_xor(M, o, kWave));
        const float e = (j < seff) ? exp2f(mj - M) : 0.f;
        float Lsum = lj * e, A = aj * e;
        for (int o = 1; o < P; o <<= 1) {
          Lsum += __shfl_xor(Lsum, o, kWave);
          A += __shfl_xor(A, o, kWave);
        }
        if (j == 0) st_tag(tg.o + (size_t)(kvh * G + g) * D + dbase + v, f2h(A / Lsum), tg.tag);
      }
    }
    __syncthreads();  // LDS reuse by the next item
    return;
  }

  int* counter = a.cnt + CNT_ATTN + b * dm.Hkv + kvh;
  if (arrive_counter(counter, nsplit, &sm.flag)) {
    // last arriver. Split weights exp2(m_j - M) / sum_j l_j exp2(m_j - M): one wave per
    // query head, lane j holds split j. The (m, l) loads and the first batch of partial-sum
    // loads are issued together, so the merge waits on memory once.
    constexpr int GW = (G + NW - 1) / NW;  // query heads per wave
    float mj[GW], lj[GW];
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int g = w + i * NW;
      mj[i] = -__builtin_inff();
      lj[i] = 0.f;
      if (g < G && lane < seff) {
        const size_t pi = pbase + (size_t)g * nsplit + lane;
        mj[i] = wt_load(&a.pml[pi * 2 + 0]);
        lj[i] = wt_load(&a.pml[pi * 2 + 1]);
      }
    }
    const int col = tid / TPC, r = tid % TPC;
    const int g = col / (D / 4), d4 = (col % (D / 4)) * 4;
    float4 v[MB];
    auto load_batch = [&](int j0) {
#pragma unroll
      for (int k = 0; k < MB; ++k) {
        const int j = j0 + k * TPC;
        v[k] = (j < seff) ? ld4_coh(&a.pacc[(pbase + (size_t)g * nsplit + j) * D + d4])
                          : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    };
    load_batch(r);
#pragma unroll
    for (int i = 0; i < GW; ++i) {
      const int gw = w + i * NW;
      if (gw < G) {
        const float M = wave_max_fast(mj[i]);
        const float e = (lane < seff) ? exp2f(mj[i] - M) : 0.f;
        const float Ls = wave_sum_fast(lj[i] * e);
        sm.w[gw][lane] = e / Ls;
      }
    }
    __syncthreads();
    {
      float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int j0 = r; j0 < seff; j0 += MB * TPC) {
        if (j0 != r) load_batch(j0);
#pragma unroll
        for (int k = 0; k < MB; ++k) {
          const int j = j0 + k * TPC;
          const float wt = (j < seff) ? sm.w[g][j] : 0.f;
          A.x = fmaf(wt, v[k].x, A.x);
          A.y = fmaf(wt, v[k].y, A.y);
          A.z = fmaf(wt, v[k].z, A.z);
          A.w = fmaf(wt, v[k].w, A.w);
        }
      }
      // sum over the TPC lanes of the column (quad steps by DPP, wider ones by shuffle)
      if (TPC >= 2) {
        A.x += dpp_f<0xB1>(A.x);
        A.y += dpp_f<0xB1>(A.y);
        A.z += dpp_f<0xB1>(A.z);
        A.w += dpp_f<0xB1>(A.w);
      }
      if (TPC >= 4) {
        A.x += dpp_f<0x4E>(A.x);
        A.y += dpp_f<0x4E>(A.y);
        A.z += dpp_f<0x4E>(A.z);
        A.w += dpp_f<0x4E>(A.w);
      }
#pragma unroll
      for (int o = 4; o < TPC; o <<= 1) {
        A.x += __shfl_xor(A.x, o, kWave);
        A.y += __shfl_xor(A.y, o, kWave);
        A.z += __shfl_xor(A.z, o, kWave);
        A.w += __shfl_xor(A.w, o, kWave);
      }
      if (r == 0) {
        f16 hv[4] = {f2h(A.x), f2h(A.y), f2h(A.z), f2h(A.w)};
        f16* dst = a.o + (size_t)b * dm.hd + (size_t)(kvh * G + g) * D + d4;
        if (COH) {
          __hip_atomic_store((g_u64*)dst, __builtin_bit_cast(unsigned long long, hv), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        } else {
          *(uint2*)dst = __builtin_bit_cast(uint2, hv);
        }
      }
    }
    if (tid == 0) reset_counter(counter);
  }
  __syncthreads();  // LDS reuse by the next item
}
