// C ABI of the early-exit decode library: argument checks, buffer layouts, river build,
// prefill and decode drivers (HIP-graph replay of the static per-step launch sequence).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/river.h"
#include "params.hpp"

// kernels (decode.hip, quant.hip, prefill.hip)
hipError_t river_decode_layers(const DecodeArgs& a, int mode, hipStream_t st,
                               void (*timer)(void*, int, int), void* tctx, int top);
hipError_t river_launch_gemv(const DecodeArgs& a, int op, int layer, int mode, hipStream_t st);
hipError_t river_launch_begin(const DecodeArgs& a, hipStream_t st);
hipError_t river_launch_head(const DecodeArgs& a, hipStream_t st, void (*timer)(void*, int, int),
                             void* tctx, int top);
int river_gemv_max_wg(const Dims& dm);
hipError_t river_launch_quantize(const f16* W, int N, int K, int group, uint8_t* out, f16* scales,
                                 uint8_t* zeros, hipStream_t st);
hipError_t river_launch_export(const uint8_t* in, const f16* sin_, const uint8_t* zin, int N, int K,
                               int group, uint8_t* packed, uint16_t* scales, uint8_t* zeros,
                               hipStream_t st);
hipError_t river_launch_rope_table(float2* tab, int Tmax, int D, double theta, hipStream_t st);
hipError_t river_launch_fill(void* p, int64_t bytes, uint32_t v, hipStream_t st);
hipError_t river_launch_kv_slot_counts(const uint32_t* cnt, int L, int B, int Hkv, int Tmax, int D,
                                       uint8_t* out, hipStream_t st);
const void* river_persist_fn(const Dims& dm, int mode, int long_ctx);
int river_persist_grid(const void* fn);
hipError_t river_launch_persist(const void* fn, const DecodeArgs& a, int S, int nwg, int splits,
                                unsigned* bar, hipStream_t st);
hipError_t river_static_scratch(void** ptr, size_t* bytes);
hipError_t river_phase_trace_copy(unsigned long long* dst, size_t n, int* dims);
hipError_t river_decode_layers_batched(const DecodeArgs& a, f16* xn, int mode, hipStream_t st,
                                       void (*timer)(void*, int, int), void* tctx, int top);
hipError_t river_launch_head_batched(const DecodeArgs& a, f16* xn, hipStream_t st,
                                     void (*timer)(void*, int, int), void* tctx, int top);

hipError_t river_launch_prefill(const PfArgs& p, const DecodeArgs& a, const LayerDev* host_layers,
                                int forced, float tau, hipStream_t st);



namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return RIVER_EHIP;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

int check_cfg(const river_config* c) {
  if (!c) return fail(RIVER_EINVAL, "cfg is NULL");
  if (c->n_layers < 1) return fail(RIVER_EINVAL, "n_layers must be >= 1");
  if (c->d_model < 8 || c->d_model % 8) return fail(RIVER_EINVAL, "d_model must be a positive multiple of 8");
  if (c->n_heads < 1 || c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads)
    return fail(RIVER_EINVAL, "n_heads must be a positive multiple of n_kv_heads");
  const int G = c->n_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(RIVER_EINVAL, "n_heads/n_kv_heads must be 1, 2, 4 or 8");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(RIVER_EINVAL, "head_dim must be 64 or 128");
  if (c->d_ffn < 8 || c->d_ffn % 8) return fail(RIVER_EINVAL, "d_ffn must be a positive multiple of 8");
  if (c->vocab < 1) return fail(RIVER_EINVAL, "vocab must be >= 1");
  if (c->group != 32 && c->group != 64 && c->group != 128) return fail(RIVER_EINVAL, "group must be 32, 64 or 128");
  const int hd = c->n_heads * c->head_dim;
  if (c->d_model > 16384 || hd > 16384 || c->d_ffn > 16384)
    return fail(RIVER_EINVAL, "d_model, n_heads*head_dim and d_ffn must be <= 16384");
  if (c->max_batch < 1 || c->max_batch > 16) return fail(RIVER_EINVAL, "max_batch must be in [1, 16]");
  if (c->max_seq < 1) return fail(RIVER_EINVAL, "max_seq must be >= 1");
  if (c->max_prefill < 1 || c->max_prefill > c->max_seq)
    return fail(RIVER_EINVAL, "max_prefill must be in [1, max_seq]");
  if (c->entry_layer < 1 || c->entry_layer > c->n_layers)
    return fail(RIVER_EINVAL, "entry_layer must be in [1, n_layers]");
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 0.f)) return fail(RIVER_EINVAL, "rms_eps and rope_theta must be > 0");
  if (c->tied_embeddings != 0 && c->tied_embeddings != 1) return fail(RIVER_EINVAL, "tied_embeddings must be 0 or 1");
  if (c->zero_point != 0 && c->zero_point != 1) return fail(RIVER_EINVAL, "zero_point must be 0 or 1");
  if (c->prefill_chunk < 0) return fail(RIVER_EINVAL, "prefill_chunk must be >= 0");
  return RIVER_OK;
}

Dims make_dims(const river_config* c) {
  Dims d{};
  d.L = c->n_layers;
  d.d = c->d_model;
  d.H = c->n_heads;
  d.Hkv = c->n_kv_heads;
  d.D = c->head_dim;
  d.F = c->d_ffn;
  d.V = c->vocab;
  d.group = c->group;
  d.B = c->max_batch;
  d.Tmax = c->max_seq;
  d.entry = c->entry_layer;
  d.tied = c->tied_embeddings;
  d.max_prefill = c->max_prefill;
  d.zp = c->zero_point;
  {
    const int def = 4096 / c->max_batch > 0 ? 4096 / c->max_batch : 1;
    const int want = c->prefill_chunk > 0 ? c->prefill_chunk : def;
    d.pf_chunk = want < c->max_prefill ? want : c->max_prefill;
  }
  d.eps = c->rms_eps;
  d.theta = c->rope_theta;
  d.hd = c->n_heads * c->head_dim;
  d.nqkv = d.hd + 2 * c->n_kv_heads * c->head_dim;
  return d;
}

int attn_smax(const Dims& d) {
  int s = 512 / (d.B * d.Hkv);
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return s;
}

// ---- river buffer layout: per layer qkv, o, gu, down (packed), then their scales
struct RiverLayout {
  uint64_t off_p[4], off_s[4], off_z[4];  // off_z: zero-point format only
  uint64_t layer_bytes;
  int N[4], K[4];
};

RiverLayout river_layout(const Dims& d) {
  RiverLayout r{};
  const int N[4] = {d.nqkv, d.d, 2 * d.F, d.d};
  const int K[4] = {d.d, d.hd, d.d, d.F};
  uint64_t off = 0;
  for (int i = 0; i < 4; ++i) {
    r.N[i] = N[i];
    r.K[i] = K[i];
    r.off_p[i] = off;
    off = align256(off + (uint64_t)N[i] * w4_row_bytes(K[i]));
  }
  for (int i = 0; i < 4; ++i) {
    r.off_s[i] = off;
    off = align256(off + (uint64_t)N[i] * w4_row_scales(K[i], d.group) * 2);
  }
  for (int i = 0; i < 4; ++i) {
    r.off_z[i] = off;
    if (d.zp) off = align256(off + (uint64_t)N[i] * w4_row_scales(K[i], d.group));
  }
  r.layer_bytes = off;
  return r;
}

// ---- scratch layout
struct ScratchLayout {
  uint64_t hs, hmid, q, o, a2, qkvr, gu, inv_attn, inv_mlp, route, pos, step, err, red, cnt, pml, pacc, amax,
      layers, rope, bar, xn;
  uint64_t t_qkv, t_o, t_a2, t_hmid, t_hs, t_part, tagc, t_end;  // tagged activations [t_qkv, t_end)
  uint64_t pf_hin, pf_hout, pf_hmid, pf_act, pf_attn, pf_qkv, pf_gu, pf_a2, pf_cos, pf_route, pf_exit,
      pf_minsim;
  uint64_t kvcnt;  // debug build: per-element KV write counters (0 bytes otherwise)
  uint64_t bpart, bcnt, bcnt_bytes;  // batched projections: partial tiles, per-tile slice counters
  uint64_t total;
  int smax;
  int ncnt;
};

ScratchLayout scratch_layout(const Dims& d) {
  ScratchLayout s{};
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const uint64_t B = d.B;
  s.smax = attn_smax(d);
  s.ncnt = CNT_ATTN + d.B * d.Hkv;
  s.hs = take((d.L + 1) * B * d.d * 2);
  s.hmid = take(d.L * B * d.d * 2);
  s.q = take(B * d.hd * 2);
  s.o = take(B * d.hd * 2);
  s.a2 = take(B * d.F * 2);
  s.qkvr = take(B * d.nqkv * 2);
  s.gu = take(B * 2 * d.F * 2);
  s.inv_attn = take((d.L + 1) * B * 4);
  s.inv_mlp = take(d.L * B * 4);
  s.route = take((d.L + 2) * B * 4);
  s.pos = take(B * 4);
  s.step = take(4);
  s.err = take(4);
  s.red = take((uint64_t)kMaxRed * 4 * 8);
  s.cnt = take((uint64_t)s.ncnt * 4);
  s.pml = take(B * d.H * s.smax * 2 * 4);
  s.pacc = take(B * d.H * s.smax * d.D * 4);
  s.amax = take(2 * B * 8);
  s.bar = take((uint64_t)kBarWords * 4);  // grid barrier of the persistent kernel
  s.t_qkv = take((uint64_t)d.nqkv * 4);
  s.t_o = take((uint64_t)2 * d.hd * 4);
  s.t_a2 = take((uint64_t)d.F * 4);
  s.t_hmid = take((uint64_t)d.L * d.d * 4);
  s.t_hs = take((uint64_t)(d.L + 1) * d.d * 4);
  s.t_part = take((uint64_t)d.H * s.smax * (d.D + 2) * 8);
  s.tagc = take(8);
  s.t_end = off;
  s.xn = take(B * d.d * 2);                // batched decode: normalised block inputs
  {  // batched projections split over K: partial tiles of both streams, slice counters
    uint64_t parts = 0, tiles = 0;
    for (int op = OP_QKV; op <= OP_LM; ++op) {
      const int S = b_split(op, d), T = b_tiles(op, d);
      if (S > 1 && (uint64_t)S * T > parts) parts = (uint64_t)S * T;
      if (S > 1 && (uint64_t)T > tiles) tiles = T;
    }
    if (B < 2) parts = tiles = 0;
    s.bpart = take(2 * parts * 256 * 4);
    s.bcnt_bytes = align256(2 * tiles * 4);
    s.bcnt = take(s.bcnt_bytes);
  }
  s.layers = take((uint64_t)d.L * sizeof(LayerDev));
  s.rope = take((uint64_t)d.Tmax * (d.D / 2) * 8);
  // prefill: the residual stream of every prompt row, the rest per chunk of positions
  const uint64_t M = B * d.max_prefill;
  const uint64_t Mc = B * d.pf_chunk;
  const uint64_t wide = (uint64_t)(d.d > d.hd ? d.d : d.hd);
  s.pf_hin = take(M * d.d * 2);
  s.pf_hout = take(M * d.d * 2);
  s.pf_cos = take(M * 8);
  s.pf_hmid = take(Mc * d.d * 2);
  s.pf_act = take(Mc * wide * 2);
  s.pf_attn = take(Mc * d.hd * 2);
  s.pf_qkv = take(Mc * d.nqkv * 2);
  s.pf_gu = take(Mc * 2 * d.F * 2);
  s.pf_a2 = take(Mc * d.F * 2);
  s.pf_route = take(B * 4);
  s.pf_exit = take(B * 4);
  s.pf_minsim = take(B * d.L * 4);
#ifdef RIVER_DEBUG_KV_COUNT
  s.kvcnt = take((uint64_t)d.L * 2 * B * d.Hkv * d.Tmax * d.D * 4);
#else
  s.kvcnt = off;
#endif
  s.total = off;
  return s;
}

// The persistent kernel's cross-workgroup exchange buffers, laid out from offset 0 (the
// static-scratch decode puts them in the library's fixed device array).
struct ExchangeLayout {
  uint64_t amax, bar, t_qkv, t_o, t_a2, t_hmid, t_hs, t_part, tagc, total;
};

ExchangeLayout exchange_layout(const Dims& d, int smax) {
  ExchangeLayout x{};
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t o = off;
    off = align256(off + bytes);
    return o;
  };
  x.amax = take((uint64_t)2 * d.B * 8);
  x.bar = take((uint64_t)kBarWords * 4);
  x.t_qkv = take((uint64_t)d.nqkv * 4);
  x.t_o = take((uint64_t)2 * d.hd * 4);
  x.t_a2 = take((uint64_t)d.F * 4);
  x.t_hmid = take((uint64_t)d.L * d.d * 4);
  x.t_hs = take((uint64_t)(d.L + 1) * d.d * 4);
  x.t_part = take((uint64_t)d.H * smax * (d.D + 2) * 8);
  x.tagc = take(8);
  x.total = off;
  return x;
}

// Device-visible address of a borrowed weight. The backbone may be partly offloaded (paperlayer
// summary, section 4 "Deployment Efficiency" and appendix A.3: under-used backbone blocks leave
// device memory while the river stays): device memory is used as is, page-locked host memory
// (hipHostMalloc, or a pinned torch tensor) through its mapped device address, so a kernel reads
// such a block over the host link only when some row runs it; any other pointer is rejected
// here, before a kernel could fault on it.
int weight_view(const void* p, const std::string& what, const void** out, bool* on_host) {
  hipPointerAttribute_t at{};
  hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // the query's error must not surface at the next launch check
    return fail(RIVER_EINVAL, what + ": neither device memory nor page-locked host memory");
  }
  if (at.type == hipMemoryTypeDevice && !at.isManaged) {
    *out = p;
    *on_host = false;
    return RIVER_OK;
  }
  if (at.type == hipMemoryTypeHost) {
    void* dp = nullptr;
    e = hipHostGetDevicePointer(&dp, const_cast<void*>(p), 0);
    if (e != hipSuccess || !dp) {
      (void)hipGetLastError();
      return fail(RIVER_EINVAL, what + ": host memory without a device mapping");
    }
    *out = dp;
    *on_host = true;
    return RIVER_OK;
  }
  return fail(RIVER_EINVAL, what + ": neither device memory nor page-locked host memory");
}

}  // namespace

struct river_ctx {
  river_config cfg;
  Dims dm;
  RiverLayout rl;
  ScratchLayout sl;
  char* kv;
  char* river;
  char* scratch;
  std::vector<LayerDev> layers;  // host copy of the device table
  const f16* embed;
  const f16* lm_head;
  const f16* final_norm;
  std::vector<int32_t> pos_host;
  hipStream_t cap_stream;
  struct Cached {
    bool valid = false;
    DecodeArgs key{};
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
  } graphs[2];  // [mode]: 0 early exit, 1 backbone only
  bool use_graph;
  // per-launch timing of one op (river_timer_arm)
  int timer_op = -1;
  int timer_cap = 0;
  int timer_n = 0;
  hipStream_t timer_stream = nullptr;
  std::vector<hipEvent_t> timer_ev;
  // persistent decode kernel ([mode]: 0 early exit, 1 backbone only); null = per-op kernels
  const void* persist_fn[2] = {nullptr, nullptr};
  const void* persist_fn_long[2] = {nullptr, nullptr};  // launches reaching kPersistLongCtx
  int persist_nwg[2] = {0, 0};
  int persist_chunk = 8;
  // this GPU's fixed device scratch (river_decode_steps_static); null if the lookup failed
  void* static_scratch = nullptr;
  size_t static_bytes = 0;
  std::string static_err;
  // parameter bytes of the borrowed weights by placement (backbone offloading), and the river
  uint64_t w_device_bytes = 0, w_host_bytes = 0, river_bytes = 0;
};

static DecodeArgs base_args(const river_ctx* c) {
  DecodeArgs a{};
  const ScratchLayout& s = c->sl;
  char* sc = c->scratch;
  a.dm = c->dm;
  a.layers = (const LayerDev*)(sc + s.layers);
  a.embed = c->embed;
  a.lm_head = c->lm_head;
  a.final_norm = c->final_norm;
  a.kv = (f16*)c->kv;
  a.rope = (const float2*)(sc + s.rope);
  a.hs = (f16*)(sc + s.hs);
  a.hmid = (f16*)(sc + s.hmid);
  a.q = (f16*)(sc + s.q);
  a.o = (f16*)(sc + s.o);
  a.a2 = (f16*)(sc + s.a2);
  a.qkvr = (f16*)(sc + s.qkvr);
  a.gu = (f16*)(sc + s.gu);
  a.inv_attn = (float*)(sc + s.inv_attn);
  a.inv_mlp = (float*)(sc + s.inv_mlp);
  a.route = (int*)(sc + s.route);
  a.pos = (int*)(sc + s.pos);
  a.step = (int*)(sc + s.step);
  a.err = (int*)(sc + s.err);
  a.red = (double*)(sc + s.red);
  a.cnt = (int*)(sc + s.cnt);
  a.pml = (float*)(sc + s.pml);
  a.pacc = (float*)(sc + s.pacc);
  a.amax = (unsigned long long*)(sc + s.amax);
  a.t_qkv = (uint32_t*)(sc + s.t_qkv);
  a.t_o = (uint32_t*)(sc + s.t_o);
  a.t_a2 = (uint32_t*)(sc + s.t_a2);
  a.t_hmid = (uint32_t*)(sc + s.t_hmid);
  a.t_hs = (uint32_t*)(sc + s.t_hs);
  a.t_part = (unsigned long long*)(sc + s.t_part);
  a.tagc = (uint32_t*)(sc + s.tagc);
  a.attn_smax = s.smax;
  a.bpart = (float*)(sc + s.bpart);
  a.bcnt = (uint32_t*)(sc + s.bcnt);
#ifdef RIVER_DEBUG_KV_COUNT
  a.kvcnt = (uint32_t*)(sc + s.kvcnt);
#endif
  return a;
}

extern "C" {

const char* river_last_error(void) { return g_err.c_str(); }

int river_kv_layout(const river_config* cfg, river_kv_desc* out) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!out) return fail(RIVER_EINVAL, "out is NULL");
  const int64_t dims[6] = {cfg->n_layers, 2, cfg->max_batch, cfg->n_kv_heads, cfg->max_seq, cfg->head_dim};
  int64_t stride = 1;
  for (int i = 5; i >= 0; --i) {
    out->dims[i] = dims[i];
    out->strides[i] = stride;
    stride *= dims[i];
  }
  out->elem_bytes = 2;
  out->total_bytes = (uint64_t)stride * 2;
  return RIVER_OK;
}

int river_workspace_bytes(const river_config* cfg, uint64_t* river_bytes, uint64_t* scratch_bytes) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!river_bytes || !scratch_bytes) return fail(RIVER_EINVAL, "output pointer is NULL");
  const Dims d = make_dims(cfg);
  *river_bytes = river_layout(d).layer_bytes * (uint64_t)d.L;
  *scratch_bytes = scratch_layout(d).total;
  return RIVER_OK;
}

int river_init(const river_config* cfg, const river_weights* w, void* kv, void* river_buf,
               void* scratch, void* stream, river_ctx** out) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (!w || !kv || !river_buf || !scratch || !out) return fail(RIVER_EINVAL, "NULL argument");
  if (!w->embed || !w->final_norm || !w->layers) return fail(RIVER_EINVAL, "NULL weight pointer");
  if (!cfg->tied_embeddings && !w->lm_head) return fail(RIVER_EINVAL, "lm_head is NULL but embeddings are not tied");
  for (int l = 0; l < cfg->n_layers; ++l) {
    const river_layer_weights& lw = w->layers[l];
    if (!lw.attn_norm || !lw.wq || !lw.wk || !lw.wv || !lw.wo || !lw.mlp_norm || !lw.w_gate ||
        !lw.w_up || !lw.w_down)
      return fail(RIVER_EINVAL, "NULL weight pointer in layer " + std::to_string(l));
  }
  hipStream_t st = (hipStream_t)stream;
  river_ctx* c = new (std::nothrow) river_ctx();
  if (!c) return fail(RIVER_ENOMEM, "host allocation failed");
  c->cfg = *cfg;
  c->dm = make_dims(cfg);
  c->rl = river_layout(c->dm);
  c->sl = scratch_layout(c->dm);
  c->kv = (char*)kv;
  c->river = (char*)river_buf;
  c->scratch = (char*)scratch;
  c->pos_host.assign(cfg->max_batch, 0);
  c->river_bytes = c->rl.layer_bytes * (uint64_t)cfg->n_layers;
  {  // device-visible weight addresses (device memory, or page-locked host memory)
    const uint64_t d = cfg->d_model, hd = (uint64_t)cfg->n_heads * cfg->head_dim,
                   kvd = (uint64_t)cfg->n_kv_heads * cfg->head_dim, F = cfg->d_ffn, V = cfg->vocab;
    auto view = [&](const void* p, const std::string& what, uint64_t elems, const void** out) {
      bool host = false;
      const int r = weight_view(p, what, out, &host);
      if (r == RIVER_OK) (host ? c->w_host_bytes : c->w_device_bytes) += 2 * elems;
      return r;
    };
    const void *emb = nullptr, *head = nullptr, *fin = nullptr;
    int r = view(w->embed, "embed", V * d, &emb);
    if (!r && !cfg->tied_embeddings) r = view(w->lm_head, "lm_head", V * d, &head);
    if (!r) r = view(w->final_norm, "final_norm", d, &fin);
    if (r) {
      delete c;
      return r;
    }
    c->embed = (const f16*)emb;
    c->lm_head = (const f16*)(cfg->tied_embeddings ? emb : head);
    c->final_norm = (const f16*)fin;
    c->layers.resize(cfg->n_layers);
    for (int l = 0; l < cfg->n_layers && !r; ++l) {
      const river_layer_weights& lw = w->layers[l];
      LayerDev& ld = c->layers[l];
      const std::string L = "layer " + std::to_string(l) + " ";
      const void* v[9] = {};
      if (!r) r = view(lw.attn_norm, L + "attn_norm", d, &v[0]);
      if (!r) r = view(lw.wq, L + "wq", hd * d, &v[1]);
      if (!r) r = view(lw.wk, L + "wk", kvd * d, &v[2]);
      if (!r) r = view(lw.wv, L + "wv", kvd * d, &v[3]);
      if (!r) r = view(lw.wo, L + "wo", d * hd, &v[4]);
      if (!r) r = view(lw.mlp_norm, L + "mlp_norm", d, &v[5]);
      if (!r) r = view(lw.w_gate, L + "w_gate", F * d, &v[6]);
      if (!r) r = view(lw.w_up, L + "w_up", F * d, &v[7]);
      if (!r) r = view(lw.w_down, L + "w_down", d * F, &v[8]);
      ld.attn_norm = (const f16*)v[0];
      ld.wq = (const f16*)v[1];
      ld.wk = (const f16*)v[2];
      ld.wv = (const f16*)v[3];
      ld.wo = (const f16*)v[4];
      ld.mlp_norm = (const f16*)v[5];
      ld.wg = (const f16*)v[6];
      ld.wu = (const f16*)v[7];
      ld.wd = (const f16*)v[8];
    }
    if (r) {
      delete c;
      return r;
    }
  }
  const char* ng = getenv("RIVER_NO_GRAPH");
  c->use_graph = !(ng && ng[0] == '1');
  hipError_t e = hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking);
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "hipStreamCreateWithFlags");
  }
  const Dims& d = c->dm;
  for (int l = 0; l < d.L; ++l) {
    LayerDev& ld = c->layers[l];
    char* base = c->river + (uint64_t)l * c->rl.layer_bytes;
    ld.r_qkv = (const uint8_t*)(base + c->rl.off_p[0]);
    ld.r_o = (const uint8_t*)(base + c->rl.off_p[1]);
    ld.r_gu = (const uint8_t*)(base + c->rl.off_p[2]);
    ld.r_d = (const uint8_t*)(base + c->rl.off_p[3]);
    ld.s_qkv = (const f16*)(base + c->rl.off_s[0]);
    ld.s_o = (const f16*)(base + c->rl.off_s[1]);
    ld.s_gu = (const f16*)(base + c->rl.off_s[2]);
    ld.s_d = (const f16*)(base + c->rl.off_s[3]);
    if (d.zp) {
      ld.z_qkv = (const uint8_t*)(base + c->rl.off_z[0]);
      ld.z_o = (const uint8_t*)(base + c->rl.off_z[1]);
      ld.z_gu = (const uint8_t*)(base + c->rl.off_z[2]);
      ld.z_d = (const uint8_t*)(base + c->rl.off_z[3]);
    }
    // quantise the seven matrices into the river copy
    struct Job {
      const void* W;
      int N, K, m, row0;
    } jobs[7] = {{ld.wq, d.hd, d.d, 0, 0},
                 {ld.wk, d.Hkv * d.D, d.d, 0, d.hd},
                 {ld.wv, d.Hkv * d.D, d.d, 0, d.hd + d.Hkv * d.D},
                 {ld.wo, d.d, d.hd, 1, 0},
                 {ld.wg, d.F, d.d, 2, 0},
                 {ld.wu, d.F, d.d, 2, d.F},
                 {ld.wd, d.d, d.F, 3, 0}};
    for (const Job& j : jobs) {
      uint8_t* p = (uint8_t*)(base + c->rl.off_p[j.m]) + (uint64_t)j.row0 * w4_row_bytes(j.K);
      f16* s = (f16*)(base + c->rl.off_s[j.m]) + (uint64_t)j.row0 * w4_row_scales(j.K, d.group);
      uint8_t* z = d.zp ? (uint8_t*)(base + c->rl.off_z[j.m]) + (uint64_t)j.row0 * w4_row_scales(j.K, d.group)
                        : nullptr;
      e = river_launch_quantize((const f16*)j.W, j.N, j.K, d.group, p, s, z, st);
      if (e != hipSuccess) {
        river_destroy(c);
        return hip_fail(e, "quantize launch");
      }
    }
  }
  DecodeArgs a = base_args(c);
  // device state: clear everything that must start at zero, the layer table, the RoPE table
  if ((e = river_launch_fill(c->scratch + c->sl.route, (uint64_t)(d.L + 2) * d.B * 4, 0, st)) ||
      (e = river_launch_fill(c->scratch + c->sl.pos, 256 * 3, 0, st)) ||
      (e = river_launch_fill(c->scratch + c->sl.cnt, align256((uint64_t)c->sl.ncnt * 4), 0, st)) ||
      (c->sl.bcnt_bytes && (e = river_launch_fill(c->scratch + c->sl.bcnt, c->sl.bcnt_bytes, 0, st))) ||
      (e = river_launch_fill(c->scratch + c->sl.amax, align256((uint64_t)2 * d.B * 8), 0, st)) ||
      (e = river_launch_fill(c->scratch + c->sl.t_qkv, c->sl.t_end - c->sl.t_qkv, 0, st)) ||
      (e = river_launch_fill(c->scratch + c->sl.kvcnt, c->sl.total - c->sl.kvcnt, 0, st)) ||
      (e = river_launch_rope_table((float2*)a.rope, d.Tmax, d.D, (double)d.theta, st))) {
    river_destroy(c);
    return hip_fail(e, "init kernels");
  }
  e = hipMemcpyAsync(c->scratch + c->sl.layers, c->layers.data(), sizeof(LayerDev) * d.L,
                     hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);  // the host table must outlive the copy
  if (e != hipSuccess) {
    river_destroy(c);
    return hip_fail(e, "layer table upload");
  }
  // the persistent decode kernel is the default path; RIVER_PERSIST=0 selects the per-op
  // kernels (graph-captured), which also serve shapes the persistent kernel does not cover
  const char* pe = getenv("RIVER_PERSIST");
  if (!(pe && pe[0] == '0')) {
    for (int m = 0; m < 2; ++m) {
      const void* fn = river_persist_fn(d, m, 0);
      const void* fn_long = river_persist_fn(d, m, 1);
      if (fn_long && river_persist_grid(fn_long) < (fn ? river_persist_grid(fn) : 0)) fn_long = fn;
      // every workgroup takes one attention split of one KV head (the splits of all heads
      // order the reuse of the kernel's activation buffers): the grid is Hkv times a power
      // of two, at least the query heads per KV head (each split merges a slice of one head)
      int nwg = fn ? river_persist_grid(fn) : 0;
      int sp = 1;
      while (2 * sp * d.Hkv <= nwg) sp *= 2;
      nwg = (sp >= d.H / d.Hkv) ? sp * d.Hkv : 0;
      // the attention phase needs one work item per (KV head, split); keep splits <= 64
      if (fn && nwg >= d.Hkv && nwg / d.Hkv <= c->sl.smax) {
        c->persist_fn[m] = fn;
        c->persist_fn_long[m] = fn_long;
        c->persist_nwg[m] = nwg;
      } else if (fn && nwg >= d.Hkv) {
        c->persist_fn[m] = fn;
        c->persist_fn_long[m] = fn_long;
        c->persist_nwg[m] = c->sl.smax * d.Hkv;
      }
    }
  }
  const char* pc = getenv("RIVER_PERSIST_CHUNK");
  if (pc && atoi(pc) > 0) c->persist_chunk = atoi(pc);
  // device address of the fixed scratch of river_decode_steps_static (once per device)
  e = river_static_scratch(&c->static_scratch, &c->static_bytes);
  if (e != hipSuccess) {
    c->static_scratch = nullptr;
    c->static_err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
  }
  *out = c;
  return RIVER_OK;
}

int river_destroy(river_ctx* c) {
  if (!c) return RIVER_OK;
  (void)hipDeviceSynchronize();
  for (auto& g : c->graphs) {
    if (g.exec) (void)hipGraphExecDestroy(g.exec);
    if (g.graph) (void)hipGraphDestroy(g.graph);
  }
  for (hipEvent_t ev : c->timer_ev) (void)hipEventDestroy(ev);
  if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
  delete c;
  return RIVER_OK;
}

int river_weight_placement(const void* p, int32_t* placement) {
  if (!p || !placement) return fail(RIVER_EINVAL, "NULL argument");
  const void* dv = nullptr;
  bool host = false;
  const int r = weight_view(p, "pointer", &dv, &host);
  if (r) return r;
  *placement = host ? 1 : 0;
  return RIVER_OK;
}

int river_weight_residency(const river_ctx* c, uint64_t* device_bytes, uint64_t* host_bytes,
                           uint64_t* river_bytes) {
  if (!c || !device_bytes || !host_bytes || !river_bytes) return fail(RIVER_EINVAL, "NULL argument");
  *device_bytes = c->w_device_bytes;
  *host_bytes = c->w_host_bytes;
  *river_bytes = c->river_bytes;
  return RIVER_OK;
}

int river_decode_path(const river_ctx* c, int32_t* persistent) {
  if (!c || !persistent) return fail(RIVER_EINVAL, "null argument");
  *persistent = (c->persist_fn[0] != nullptr) ? 1 : 0;
  return RIVER_OK;
}

int river_positions(const river_ctx* c, int32_t* pos) {
  if (!c || !pos) return fail(RIVER_EINVAL, "NULL argument");
  for (size_t i = 0; i < c->pos_host.size(); ++i) pos[i] = c->pos_host[i];
  return RIVER_OK;
}

int river_device_status(river_ctx* c, void* stream) {
  if (!c) return fail(RIVER_EINVAL, "ctx is NULL");
  hipStream_t st = (hipStream_t)stream;
  int v = 0;
  hipError_t e = hipMemcpyAsync(&v, c->scratch + c->sl.err, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "device status read");
  if (v) {
    (void)river_launch_fill(c->scratch + c->sl.err, 4, 0, st);
    (void)hipStreamSynchronize(st);
    return fail(RIVER_EDEVICE, "device error word " + std::to_string(v) +
                                   " (1: token id out of range, 2: forced exit out of range)");
  }
  return RIVER_OK;
}

int river_prefill(river_ctx* c, const int32_t* tokens, int32_t P, int32_t prefill_exit, float tau,
                  int32_t* next_tok, float* logits, int32_t* seq_exit, float* min_sim, void* stream) {
  if (!c || !tokens || !next_tok) return fail(RIVER_EINVAL, "NULL argument");
  const Dims& d = c->dm;
  if (P < 1 || P > d.max_prefill || P > d.Tmax) return fail(RIVER_ERANGE, "P out of range");
  if (prefill_exit != 0 && (prefill_exit < d.entry || prefill_exit > d.L))
    return fail(RIVER_ERANGE, "prefill_exit must be 0 or in [entry_layer, n_layers]");
  if (prefill_exit == 0 && std::isnan(tau)) return fail(RIVER_EINVAL, "tau is NaN");
  hipStream_t st = (hipStream_t)stream;
  char* sc = c->scratch;
  const ScratchLayout& s = c->sl;
  PfArgs p{};
  p.dm = d;
  p.M = d.B * P;
  p.P = P;
  p.Ct = d.pf_chunk < P ? d.pf_chunk : P;
  p.tokens = tokens;
  p.embed = c->embed;
  p.hin = (f16*)(sc + s.pf_hin);
  p.hout = (f16*)(sc + s.pf_hout);
  p.hmid = (f16*)(sc + s.pf_hmid);
  p.act = (f16*)(sc + s.pf_act);
  p.attn = (f16*)(sc + s.pf_attn);
  p.qkv = (f16*)(sc + s.pf_qkv);
  p.gu = (f16*)(sc + s.pf_gu);
  p.a2 = (f16*)(sc + s.pf_a2);
  p.cosv = (double*)(sc + s.pf_cos);
  p.seq_route = (int*)(sc + s.pf_route);
  p.seq_exit = (int*)(sc + s.pf_exit);
  p.min_sim = min_sim;
  p.err = (int*)(sc + s.err);
  p.kv = (f16*)c->kv;
  p.rope = (const float2*)(sc + s.rope);
  DecodeArgs a = base_args(c);
  p.kvcnt = a.kvcnt;
  a.tok_out = next_tok;
  a.logits = logits;
  // The LM head below takes an atomic max into argmax slot 0; a persistent decode launch leaves
  // the key of its last step in slot (S-1)&1, so both slots start from zero here.
  hipError_t e = river_launch_fill(sc + s.amax, (int64_t)2 * d.B * 8, 0, st);
  if (e != hipSuccess) return hip_fail(e, "argmax reset");
  e = river_launch_prefill(p, a, c->layers.data(), prefill_exit, tau, st);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  e = (d.B > 1) ? river_launch_head_batched(a, (f16*)(sc + s.xn), st, nullptr, nullptr, -1)
               : river_launch_head(a, st, nullptr, nullptr, -1);
  if (e != hipSuccess) return hip_fail(e, "prefill LM head launch");
  if (seq_exit) {
    e = hipMemcpyAsync(seq_exit, p.seq_exit, (size_t)d.B * 4, hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "seq_exit copy");
  }
  for (auto& v : c->pos_host) v = P;
  return RIVER_OK;
}

static bool same_key(const DecodeArgs& x, const DecodeArgs& y) {
  return x.tok_in == y.tok_in && x.sched == y.sched && x.tok_out == y.tok_out &&
         x.exit_out == y.exit_out && x.sim_out == y.sim_out && x.logits == y.logits &&
         std::memcmp(&x.tau, &y.tau, sizeof(float)) == 0;
}


static void timer_hook(void* p, int op, int phase) {
  river_ctx* c = (river_ctx*)p;
  (void)op;
  if (c->timer_n >= c->timer_cap) return;
  (void)hipEventRecord(c->timer_ev[2 * c->timer_n + phase], c->timer_stream);
  if (phase == 1) ++c->timer_n;
}

static int run_persist(river_ctx* c, const DecodeArgs& a, int S, int mode, hipStream_t st,
                       unsigned* bar) {
  const int B = c->dm.B, L = c->dm.L;
  const int nwg = c->persist_nwg[mode];
  const int splits = nwg / c->dm.Hkv;
  const bool timed = (c->timer_op == TOP_PERSIST);
  if (timed) c->timer_stream = st;
  for (int s0 = 0; s0 < S; s0 += c->persist_chunk) {
    const int n = (S - s0 < c->persist_chunk) ? S - s0 : c->persist_chunk;
    DecodeArgs b = a;
    b.tok_in = s0 ? a.tok_out + (size_t)(s0 - 1) * B : a.tok_in;
    b.sched = a.sched ? a.sched + (size_t)s0 * B : nullptr;
    b.tok_out = a.tok_out + (size_t)s0 * B;
    b.exit_out = a.exit_out ? a.exit_out + (size_t)s0 * B : nullptr;
    b.sim_out = a.sim_out ? a.sim_out + (size_t)s0 * B * L : nullptr;
    hipError_t e = river_launch_fill(bar, (int64_t)kBarWords * 4, 0, st);
    if (e == hipSuccess) e = river_launch_fill(a.amax, (int64_t)2 * B * 8, 0, st);
    if (e != hipSuccess) return hip_fail(e, "barrier/argmax reset");
    if (timed) timer_hook(c, TOP_PERSIST, 0);
    const bool long_ctx = (int64_t)c->pos_host[0] + s0 + n - 1 >= kPersistLongCtx;
    e = river_launch_persist(long_ctx ? c->persist_fn_long[mode] : c->persist_fn[mode], b, n, nwg,
                             splits, bar, st);
    if (timed) timer_hook(c, TOP_PERSIST, 1);
    if (e != hipSuccess) return hip_fail(e, "persistent decode launch");
  }
  return RIVER_OK;
}

// One decode step on the per-op kernels: batch 1 or the batched (MFMA) kernels.
static hipError_t step_layers(river_ctx* c, const DecodeArgs& a, int mode, hipStream_t st,
                              void (*timer)(void*, int, int), void* tctx, int top) {
  if (c->dm.B > 1) return river_decode_layers_batched(a, (f16*)(c->scratch + c->sl.xn), mode, st, timer, tctx, top);
  return river_decode_layers(a, mode, st, timer, tctx, top);
}

static int run_steps(river_ctx* c, const DecodeArgs& a, int S, int mode, hipStream_t st) {
  if (c->persist_fn[mode] && (c->timer_op < 0 || c->timer_op == TOP_PERSIST))
    return run_persist(c, a, S, mode, st, (unsigned*)(c->scratch + c->sl.bar));
  hipError_t e = river_launch_begin(a, st);
  if (e != hipSuccess) return hip_fail(e, "begin launch");
  if (c->timer_op >= 0) {  // timed: direct launches with events around the chosen op
    c->timer_stream = st;
    for (int i = 0; i < S; ++i)
      if ((e = step_layers(c, a, mode, st, timer_hook, c, c->timer_op)) != hipSuccess)
        return hip_fail(e, "decode launch");
    return RIVER_OK;
  }
  if (!c->use_graph) {
    for (int i = 0; i < S; ++i)
      if ((e = step_layers(c, a, mode, st, nullptr, nullptr, -1)) != hipSuccess)
        return hip_fail(e, "decode launch");
    return RIVER_OK;
  }
  river_ctx::Cached& g = c->graphs[mode];
  if (!g.valid || !same_key(a, g.key)) {
    if (g.exec) (void)hipGraphExecDestroy(g.exec);
    if (g.graph) (void)hipGraphDestroy(g.graph);
    g.exec = nullptr;
    g.graph = nullptr;
    g.valid = false;
    e = hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return hip_fail(e, "hipStreamBeginCapture");
    hipError_t le = step_layers(c, a, mode, c->cap_stream, nullptr, nullptr, -1);
    e = hipStreamEndCapture(c->cap_stream, &g.graph);
    if (le != hipSuccess) return hip_fail(le, "decode capture");
    if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
    e = hipGraphInstantiate(&g.exec, g.graph, nullptr, nullptr, 0);
    if (e != hipSuccess) return hip_fail(e, "hipGraphInstantiate");
    g.key = a;
    g.valid = true;
  }
  for (int i = 0; i < S; ++i)
    if ((e = hipGraphLaunch(g.exec, st)) != hipSuccess) return hip_fail(e, "hipGraphLaunch");
  return RIVER_OK;
}

int river_decode_steps(river_ctx* c, const int32_t* tok_in, const int32_t* sched, int32_t S,
                       float tau, int32_t* tok_out, int32_t* exit_layer, float* sim, void* stream) {
  if (!c || !tok_in || !tok_out) return fail(RIVER_EINVAL, "NULL argument");
  if (S < 1) return fail(RIVER_EINVAL, "S must be >= 1");
  if (!sched && std::isnan(tau)) return fail(RIVER_EINVAL, "tau is NaN");
  for (int32_t p : c->pos_host)
    if ((int64_t)p + S > c->dm.Tmax) return fail(RIVER_ERANGE, "position would pass max_seq");
  DecodeArgs a = base_args(c);
  a.tok_in = tok_in;
  a.sched = sched;
  a.tok_out = tok_out;
  a.exit_out = exit_layer;
  a.sim_out = sim;
  a.logits = nullptr;
  a.tau = sched ? 0.f : tau;
  int rc = run_steps(c, a, S, 0, (hipStream_t)stream);
  if (rc) return rc;
  for (auto& v : c->pos_host) v += S;
  return RIVER_OK;
}

int river_decode_steps_static(river_ctx* c, const int32_t* tok_in, const int32_t* sched, int32_t S,
                              float tau, int32_t* tok_out, int32_t* exit_layer, float* sim, void* stream) {
  if (!c || !tok_in || !tok_out) return fail(RIVER_EINVAL, "NULL argument");
  if (S < 1) return fail(RIVER_EINVAL, "S must be >= 1");
  if (!sched && std::isnan(tau)) return fail(RIVER_EINVAL, "tau is NaN");
  if (!c->persist_fn[0])
    return fail(RIVER_EINVAL, "the static-scratch decode runs on the persistent kernel only (batch 1, "
                              "supported shapes, RIVER_PERSIST not 0)");
  if (c->timer_op >= 0) return fail(RIVER_EINVAL, "timer armed: use river_decode_steps");
  if (!c->static_scratch) return fail(RIVER_EHIP, c->static_err);
  for (int32_t p : c->pos_host)
    if ((int64_t)p + S > c->dm.Tmax) return fail(RIVER_ERANGE, "position would pass max_seq");
  const ExchangeLayout x = exchange_layout(c->dm, c->sl.smax);
  if (x.total > c->static_bytes)
    return fail(RIVER_ENOMEM, "this model's exchange buffers need " + std::to_string(x.total) +
                                  " bytes; the static scratch holds " + std::to_string(c->static_bytes));
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)c->static_scratch;
  // the array keeps the last call's contents (possibly another context's): every tag, tag
  // counter and barrier word starts from zero (tags are never 0, so no stale word matches)
  hipError_t e = river_launch_fill(base, (int64_t)x.total, 0, st);
  if (e != hipSuccess) return hip_fail(e, "static scratch reset");
  DecodeArgs a = base_args(c);
  a.amax = (unsigned long long*)(base + x.amax);
  a.t_qkv = (uint32_t*)(base + x.t_qkv);
  a.t_o = (uint32_t*)(base + x.t_o);
  a.t_a2 = (uint32_t*)(base + x.t_a2);
  a.t_hmid = (uint32_t*)(base + x.t_hmid);
  a.t_hs = (uint32_t*)(base + x.t_hs);
  a.t_part = (unsigned long long*)(base + x.t_part);
  a.tagc = (uint32_t*)(base + x.tagc);
  a.tok_in = tok_in;
  a.sched = sched;
  a.tok_out = tok_out;
  a.exit_out = exit_layer;
  a.sim_out = sim;
  a.logits = nullptr;
  a.tau = sched ? 0.f : tau;
  int rc = run_persist(c, a, S, 0, st, (unsigned*)(base + x.bar));
  if (rc) return rc;
  for (auto& v : c->pos_host) v += S;
  return RIVER_OK;
}

int river_decode_backbone_steps(river_ctx* c, const int32_t* tok_in, int32_t S, int32_t* tok_out,
                                void* stream) {
  if (!c || !tok_in || !tok_out) return fail(RIVER_EINVAL, "NULL argument");
  if (S < 1) return fail(RIVER_EINVAL, "S must be >= 1");
  for (int32_t p : c->pos_host)
    if ((int64_t)p + S > c->dm.Tmax) return fail(RIVER_ERANGE, "position would pass max_seq");
  DecodeArgs a = base_args(c);
  a.tok_in = tok_in;
  a.tok_out = tok_out;
  int rc = run_steps(c, a, S, 1, (hipStream_t)stream);
  if (rc) return rc;
  for (auto& v : c->pos_host) v += S;
  return RIVER_OK;
}

int river_timer_arm(river_ctx* c, int32_t op, int32_t max_launches) {
  if (!c) return fail(RIVER_EINVAL, "ctx is NULL");
  if (op < TOP_QKV || op > TOP_PERSIST) return fail(RIVER_EINVAL, "op must be in [0, 6]");
  if (max_launches < 1) return fail(RIVER_EINVAL, "max_launches must be >= 1");
  while ((int)c->timer_ev.size() < 2 * max_launches) {
    hipEvent_t ev;
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    c->timer_ev.push_back(ev);
  }
  c->timer_op = op;
  c->timer_cap = max_launches;
  c->timer_n = 0;
  return RIVER_OK;
}

int river_timer_read(river_ctx* c, float* ms, int32_t* n) {
  if (!c || !ms || !n) return fail(RIVER_EINVAL, "NULL argument");
  if (c->timer_op < 0) return fail(RIVER_EINVAL, "timer not armed");
  const int cnt = c->timer_n < *n ? c->timer_n : *n;
  if (cnt > 0) {
    hipError_t e = hipEventSynchronize(c->timer_ev[2 * (c->timer_n - 1) + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
  }
  for (int i = 0; i < cnt; ++i) {
    hipError_t e = hipEventElapsedTime(&ms[i], c->timer_ev[2 * i], c->timer_ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
  }
  *n = cnt;
  c->timer_op = -1;
  c->timer_n = 0;
  return RIVER_OK;
}

int river_decode_step(river_ctx* c, const int32_t* tok_in, const int32_t* forced_exit, float tau,
                      int32_t* tok_out, float* logits, int32_t* exit_layer, float* sim, void* stream) {
  if (!c || !tok_in || !tok_out) return fail(RIVER_EINVAL, "NULL argument");
  if (!forced_exit && std::isnan(tau)) return fail(RIVER_EINVAL, "tau is NaN");
  for (int32_t p : c->pos_host)
    if ((int64_t)p + 1 > c->dm.Tmax) return fail(RIVER_ERANGE, "position would pass max_seq");
  DecodeArgs a = base_args(c);
  a.tok_in = tok_in;
  a.sched = forced_exit;
  a.tok_out = tok_out;
  a.exit_out = exit_layer;
  a.sim_out = sim;
  a.logits = logits;
  a.tau = forced_exit ? 0.f : tau;
  int rc = run_steps(c, a, 1, 0, (hipStream_t)stream);
  if (rc) return rc;
  for (auto& v : c->pos_host) v += 1;
  return RIVER_OK;
}

int river_export_river(river_ctx* c, int32_t layer, int32_t which, uint8_t* packed, uint16_t* scales,
                       uint8_t* zeros, void* stream) {
  if (!c || !packed || !scales) return fail(RIVER_EINVAL, "NULL argument");
  if ((zeros != nullptr) != (c->dm.zp != 0))
    return fail(RIVER_EINVAL, "zeros must be non-NULL exactly for the zero-point format");
  const Dims& d = c->dm;
  if (layer < 0 || layer >= d.L) return fail(RIVER_ERANGE, "layer out of range");
  if (which < 0 || which > 6) return fail(RIVER_EINVAL, "which must be in [0, 6]");
  const int mat[7] = {0, 0, 0, 1, 2, 2, 3};
  const int row0[7] = {0, d.hd, d.hd + d.Hkv * d.D, 0, 0, d.F, 0};
  const int Ns[7] = {d.hd, d.Hkv * d.D, d.Hkv * d.D, d.d, d.F, d.F, d.d};
  const int m = mat[which];
  const int K = c->rl.K[m];
  const char* base = c->river + (uint64_t)layer * c->rl.layer_bytes;
  const uint8_t* p = (const uint8_t*)(base + c->rl.off_p[m]) + (uint64_t)row0[which] * w4_row_bytes(K);
  const f16* s = (const f16*)(base + c->rl.off_s[m]) + (uint64_t)row0[which] * w4_row_scales(K, d.group);
  const uint8_t* z = d.zp ? (const uint8_t*)(base + c->rl.off_z[m]) + (uint64_t)row0[which] * w4_row_scales(K, d.group)
                          : nullptr;
  hipError_t e = river_launch_export(p, s, z, Ns[which], K, d.group, packed, scales, zeros, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "export launch");
  return RIVER_OK;
}

int river_kv_write_counts(river_ctx* c, uint8_t* cnt, void* stream) {
  if (!c || !cnt) return fail(RIVER_EINVAL, "NULL argument");
#ifdef RIVER_DEBUG_KV_COUNT
  const Dims& d = c->dm;
  hipError_t e = river_launch_kv_slot_counts((const uint32_t*)(c->scratch + c->sl.kvcnt), d.L, d.B, d.Hkv,
                                             d.Tmax, d.D, cnt, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv count launch");
  return RIVER_OK;
#else
  (void)stream;
  return fail(RIVER_EINVAL, "KV write counting needs the library built with RIVER_DEBUG_KV_COUNT");
#endif
}

int river_kv_counting(int32_t* enabled) {
  if (!enabled) return fail(RIVER_EINVAL, "NULL argument");
#ifdef RIVER_DEBUG_KV_COUNT
  *enabled = 1;
#else
  *enabled = 0;
#endif
  return RIVER_OK;
}

int river_phase_trace(uint64_t* dst, uint64_t n, int32_t* dims) {
  if (!dims) return fail(RIVER_EINVAL, "NULL argument");
  int d4[4];
  const hipError_t e = river_phase_trace_copy((unsigned long long*)dst, (size_t)n, d4);
  for (int i = 0; i < 4; ++i) dims[i] = d4[i];
  if (e == hipErrorNotSupported)
    return fail(RIVER_EINVAL, "phase timestamps need the library built with RIVER_PHASE_TRACE");
  if (e != hipSuccess) return hip_fail(e, "phase trace copy");
  return RIVER_OK;
}

int river_debug_hidden(river_ctx* c, void* dst, void* stream) {
  if (!c || !dst) return fail(RIVER_EINVAL, "NULL argument");
  const Dims& d = c->dm;
  hipError_t e = hipMemcpyAsync(dst, c->scratch + c->sl.hs, (size_t)(d.L + 1) * d.B * d.d * 2,
                                hipMemcpyDeviceToDevice, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hidden copy");
  return RIVER_OK;
}

}  // extern "C"
