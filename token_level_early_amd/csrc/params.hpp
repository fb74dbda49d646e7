// Argument blocks shared by the host driver (api.cpp) and the kernels.
#pragma once

#include <stdint.h>

#include "common.hpp"

// Per-layer device pointers: borrowed fp16 backbone weights and the river copy built at init.
// River matrices use the device int4 layout: rows in logical order, row stride
// w4_row_bytes(K), element 2i in the low nibble of byte i, padding nibbles 8 (q = 0); fp16
// scales [N][w4_row_scales(K, group)], padding groups 0.
//   r_qkv: rows [0,H*D) = wq, [H*D, H*D+Hkv*D) = wk, then wv      (K = d)
//   r_o:   wo                                                    (K = H*D)
//   r_gu:  rows [0,F) = w_gate, [F,2F) = w_up                     (K = d)
//   r_d:   w_down                                                (K = F)
struct LayerDev {
  const f16* attn_norm;
  const f16* wq;
  const f16* wk;
  const f16* wv;
  const f16* wo;
  const f16* mlp_norm;
  const f16* wg;
  const f16* wu;
  const f16* wd;
  const uint8_t* r_qkv;
  const uint8_t* r_o;
  const uint8_t* r_gu;
  const uint8_t* r_d;
  const f16* s_qkv;
  const f16* s_o;
  const f16* s_gu;
  const f16* s_d;
  // zero-point format only (else null): one zero point (uint8) per group, laid out like the scales
  const uint8_t* z_qkv;
  const uint8_t* z_o;
  const uint8_t* z_gu;
  const uint8_t* z_d;
};

struct Dims {
  int L, d, H, Hkv, D, F, V, group, B, Tmax, entry, tied, max_prefill;
  int zp;    // river format: 0 symmetric int4, 1 zero-point int4
  int pf_chunk;  // prefill positions per chunk
  float eps, theta;
  int hd;    // H*D
  int nqkv;  // H*D + 2*Hkv*D
};

// Route codes: which copy of block l a row runs.
enum { ROUTE_BACKBONE = 0, ROUTE_RIVER = 1 };

// Device error word bits.
enum { ERR_TOKEN = 1, ERR_FORCED = 2, ERR_POS = 4, ERR_SYNC = 8 };

// Everything a decode kernel needs. Passed by value.
struct DecodeArgs {
  Dims dm;
  const LayerDev* layers;  // device array [L]
  const f16* embed;        // [V][d]
  const f16* lm_head;      // [V][d] (the embedding when tied)
  const f16* final_norm;   // [d]
  f16* kv;                 // [L][2][B][Hkv][Tmax][D]
  const float2* rope;      // [Tmax][D/2] (cos, sin)
  // residual stream and activations (scratch)
  f16* hs;      // [L+1][B][d]
  f16* hmid;    // [L][B][d]   (index l-1 for layer l)
  f16* q;       // [B][H*D]
  f16* o;       // [B][H*D]
  f16* a2;      // [B][F]
  f16* qkvr;    // [B][nqkv] un-rotated q|k|v (persistent kernel)
  f16* gu;      // [B][2F]   gate|up outputs before SwiGLU (persistent kernel)
  float* inv_attn;  // [L+1][B]  1/rms of hs[l]
  float* inv_mlp;   // [L][B]    1/rms of hmid[l-1]
  int* route;       // [L+2][B]  route of layer l
  int* pos;         // [B]
  int* step;        // [1]
  int* err;         // [1]
  double* red;      // [kMaxRed][4] per-workgroup partial sums
  int* cnt;         // counters, see CNT_*
  float* pml;       // attention split partials (m, l): [B][H][smax][2]
  float* pacc;      // attention split partials acc: [B][H][smax][D]
  unsigned long long* amax;  // [2][B] LM-head argmax keys (by step parity in the persistent kernel)
  // persistent kernel (batch 1): tagged activations (fp16 value | 16-bit use tag << 16)
  uint32_t* t_qkv;   // [nqkv]
  uint32_t* t_o;     // [2][H*D]  by layer parity
  uint32_t* t_a2;    // [F]
  uint32_t* t_hmid;  // [L][d]
  uint32_t* t_hs;    // [L+1][d]  (row 0 unused: h(0) is the embedding row)
  unsigned long long* t_part;  // [H][splits][D+2] attention split partials (fp32 | tag32 << 32)
  uint32_t* tagc;    // [2] tag counters (16-bit activations, 32-bit partials), advanced per launch
  int attn_smax;    // split count of the attention grid
  // per-call I/O (device pointers)
  const int* tok_in;     // [B]
  const int* sched;      // [S][B] forced exit layers or null (tau mode)
  int* tok_out;          // [S][B]
  int* exit_out;         // [S][B] or null
  float* sim_out;        // [S][B][L] or null
  float* logits;         // [B][V] or null (single step only)
  float tau;
  uint32_t* kvcnt;       // debug build only: per-element KV write counters (KV layout), else null
  float* bpart;          // batched projections: partial tiles [stream][tile][slice][16][16]
  uint32_t* bcnt;        // batched projections: slices finished per [stream][tile] (back to 0 after each launch)
};

static constexpr int kMaxRed = 8192;
// Grid barrier of the persistent kernel, in u32 words: the completed-group counter at 0, the
// abort flag at kBarAbort, the arrival counter of workgroup group g at (g + 1) * kBarStride and
// its release flag at (kBarMaxGroups + 1 + g) * kBarStride (groups of kBarGroup workgroups;
// every word on its own 256-byte line).
static constexpr int kBarGroup = 16, kBarStride = 64, kBarMaxGroups = 64, kBarAbort = 32;
static constexpr int kBarWords = (2 * kBarMaxGroups + 1) * kBarStride;
// Persistent decode: launches that reach this position run the long-context kernel variant.
static constexpr int kPersistLongCtx = 8192;
// counter slots (each one int)
static constexpr int CNT_O = 0, CNT_DOWN = 1, CNT_LM = 2, CNT_ATTN = 8;  // attn: [B][Hkv]

// Decode GEMV operations (one launch each).
enum { OP_QKV = 0, OP_O = 1, OP_GU = 2, OP_DOWN = 3, OP_LM = 4 };

// Batched projections (2..16 rows). A launch is a grid of at most kBGrid workgroups; workgroup
// (g, s) holds slice s of the input's K range in LDS (at most kBXs values per row) and computes
// that slice's contribution to the 16-column tiles g, g + groups, ...; the b_split(op) partial
// tiles of a tile are summed, in slice order, by the workgroup that finishes it last.
static constexpr int kBGrid = 256;
#ifndef RIVER_BS_QKV  // preferred K slices per projection
#define RIVER_BS_QKV 1
#endif
#ifndef RIVER_BS_O
#define RIVER_BS_O 1
#endif
#ifndef RIVER_BS_GU
#define RIVER_BS_GU 1
#endif
#ifndef RIVER_BS_DOWN
#define RIVER_BS_DOWN 4
#endif
static constexpr int kBXs = 4096;
__host__ __device__ inline int b_rows(int op, const Dims& d) {
  return op == OP_QKV ? d.nqkv : op == OP_GU ? 2 * d.F : op == OP_LM ? d.V : d.d;
}
__host__ __device__ inline int b_k(int op, const Dims& d) {
  return op == OP_O ? d.hd : op == OP_DOWN ? d.F : d.d;
}
__host__ __device__ inline int b_tiles(int op, const Dims& d) { return (b_rows(op, d) + 15) / 16; }
__host__ __device__ inline int b_split(int op, const Dims& d) {
  const int K = b_k(op, d);
  // more slices give each workgroup more tiles to share its staged input with; slices of at
  // least 1024 values keep all 8 waves busy on every tile
  int s = op == OP_LM ? 1 : op == OP_GU ? RIVER_BS_GU : op == OP_DOWN ? RIVER_BS_DOWN : op == OP_O ? RIVER_BS_O : RIVER_BS_QKV;
  while (s > 1 && K / s < 1024) s /= 2;
  const int lds = (K + kBXs - 1) / kBXs;
  return s > lds ? s : lds;
}
// K values per slice: a whole number of 128-value blocks
__host__ __device__ inline int b_slice(int op, const Dims& d) {
  const int S = b_split(op, d), K = b_k(op, d);
  return ((K + S - 1) / S + 127) / 128 * 128;
}
__host__ __device__ inline int b_groups(int op, const Dims& d) {
  const int S = b_split(op, d), T = b_tiles(op, d);
  const int g = kBGrid / S;
  return T < g ? T : g;
}
// Timer op codes (public, see river_timer_arm): the launches of one decode step in order.
enum { TOP_QKV = 0, TOP_ATTN = 1, TOP_O = 2, TOP_GU = 3, TOP_DOWN = 4, TOP_LM = 5, TOP_PERSIST = 6 };

// Prefill activations and state (scratch), passed by value to the prefill kernels.
// The prompt runs layer by layer (the sequence-level exit after layer l needs every token's
// s_t(l)), each layer in chunks of Ct positions of every row: the residual stream hin/hout
// holds all B*P rows, the other activations only the B*Ce rows of the current chunk
// (chunk-local row mc <-> row b = mc / Ce, position t = t0 + mc % Ce, global row b*P + t).
struct PfArgs {
  Dims dm;
  int M, P;            // M = B*P rows
  int Ct;              // positions per chunk
  int t0, Ce;          // current chunk: positions [t0, t0 + Ce)
  const int* tokens;   // [B][P]
  const f16* embed;
  f16* hin;    // [M][d] block input (residual stream)
  f16* hout;   // [M][d] block output
  f16* hmid;   // [B*Ct][d]
  f16* act;    // [B*Ct][max(d, H*D)] normed input / rotated q
  f16* attn;   // [B*Ct][H*D] attention output
  f16* qkv;    // [B*Ct][nqkv]
  f16* gu;     // [B*Ct][2F]
  f16* a2;     // [B*Ct][F]
  double* cosv;    // [M]
  int* seq_route;  // [B]
  int* seq_exit;   // [B]
  float* min_sim;  // [B][L] or null
  int* err;
  f16* kv;
  const float2* rope;
  uint32_t* kvcnt;  // debug build only (see DecodeArgs::kvcnt)
};

// Debug build (RIVER_DEBUG_KV_COUNT): one 32-bit counter per element of the shared KV cache,
// at the element's own index, incremented by every store of that element; river_kv_write_counts
// reduces them to writes per (layer, row, position) slot. Release builds compile this away.
#ifdef RIVER_DEBUG_KV_COUNT
RIVER_DEV void kv_count(uint32_t* cnt, const f16* kv, const f16* dst, int n) {
  for (int i = 0; i < n; ++i)
    __hip_atomic_fetch_add(cnt + (dst - kv) + i, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
#else
RIVER_DEV void kv_count(uint32_t*, const f16*, const f16*, int) {}
#endif
