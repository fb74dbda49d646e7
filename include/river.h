/*
 * river.h -- C ABI of the River-LLM token-level early-exit decode library (MI355X, gfx950).
 *
 * The method ("River-LLM: Large Language Model Seamless Exit Based on KV Share", Shen & Zou):
 *   - every backbone decoder block gets an exit layer that is a W4A16 copy of the block
 *     (int4 weights, fp16 activations): aitrends.kr article, exit-layer construction
 *     paragraph; paperlayer.ai summary of arXiv 2604.18396v3, section 4 "KV-Shared Exit Layer";
 *   - backbone and exit layers use the same KV addressing and one fp16 KV cache, so a token
 *     that leaves the backbone still fills every later layer's KV slot (KV Cache Absence is
 *     avoided without recomputation): paperlayer section 4, appendix A.3; aitrends KV-share
 *     paragraph; chatpaper.ai abstract;
 *   - a token leaves the backbone after layer l when the cosine similarity of that block's
 *     input h(l-1) and output h(l) exceeds tau, and then runs the remaining layers on the
 *     exit layers before the original LM head: aitrends exit-criterion paragraph; paperlayer
 *     section 4 "Error-Aware Exit Decisions" and "Inference with Seamless Exit";
 *   - prefill uses one exit depth for the whole sequence, generation decides per token:
 *     paperlayer section 4 "Inference with Seamless Exit", section 3 "Sequence-level Exit".
 *
 * Conventions
 *   - Layers are 1-based in the text (l = 1..L). The exit layer e of a token is the number of
 *     backbone layers it ran: layers 1..e on the backbone, e+1..L on the river. e = L means
 *     no exit; a forced e = 0 runs every layer on the river (the all-int4 "Full Quantization"
 *     comparator of the paperlayer.ai summary, section 5). Exit tests run after backbone
 *     layers l in [entry_layer, L-1].
 *   - Pointers are DEVICE pointers unless marked "host". fp16 tensors are IEEE binary16,
 *     row-major. `stream` is a hipStream_t passed as void* (NULL = the null stream); all
 *     device work of a call is enqueued on it and the call returns without synchronising,
 *     except where a function says it synchronises.
 *   - Every call returns an int status (RIVER_OK or a negative code). river_last_error()
 *     returns a message for the calling thread's last failure. No C++ exception crosses
 *     the ABI.
 *   - The library allocates only host-side objects: its opaque handle, a capture stream, HIP
 *     graphs of the decode step and (when armed) timing events. Every device buffer (KV
 *     cache, river weights, scratch) is allocated by the caller with the sizes these
 *     functions report.
 *   - Calls on one context must not overlap (they share its scratch buffer).
 */
#ifndef RIVER_H
#define RIVER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  RIVER_OK = 0,
  RIVER_EINVAL = -1,  /* bad argument or configuration */
  RIVER_ENOMEM = -2,  /* a caller buffer is too small or a host allocation failed */
  RIVER_ERANGE = -3,  /* position, length or exit layer out of range */
  RIVER_EHIP = -4,    /* a HIP runtime call failed */
  RIVER_EDEVICE = -5  /* a kernel reported bad device-side input (see river_device_status) */
};

/* Model and capacity. All fields are required (no defaults). */
typedef struct river_config {
  int32_t n_layers;        /* L >= 1 */
  int32_t d_model;         /* d, multiple of 8 */
  int32_t n_heads;         /* H */
  int32_t n_kv_heads;      /* Hkv, divides H */
  int32_t head_dim;        /* D in {64, 128} */
  int32_t d_ffn;           /* F, multiple of 8 */
  int32_t vocab;           /* V */
  int32_t tied_embeddings; /* 1: LM head is the embedding matrix */
  float rms_eps;           /* RMSNorm epsilon */
  float rope_theta;        /* RoPE base (rotate-half pairing (i, i + D/2)) */
  int32_t group;           /* int4 group size along the input dimension, in {32, 64, 128} */
  int32_t max_batch;       /* B: rows decoded together (every call uses exactly B rows) */
  int32_t max_seq;         /* Tmax: KV positions per row */
  int32_t max_prefill;     /* longest prompt river_prefill accepts (<= max_seq) */
  int32_t entry_layer;     /* E_min in [1, L]: first layer after which an exit is tested */
  int32_t prefill_chunk;   /* positions per prefill chunk, >= 0 (0: 4096 / max_batch): the prompt
                              runs layer by layer, each layer in chunks of this many positions of
                              every row; scratch grows with max_batch * chunk, not max_prefill */
  int32_t zero_point;      /* river format. 0: symmetric int4, one fp16 scale per group;
                              1: asymmetric int4, one fp16 scale and one integer zero point per
                              group (the scale-and-zero storage of the pages' other backends,
                              HQQ and AWQ: paperlayer appendix A.1; without their calibration) */
} river_config;

/* Borrowed fp16 backbone weights of one block (device pointers, row-major [out][in]). */
typedef struct river_layer_weights {
  const void* attn_norm; /* [d] */
  const void* wq;        /* [H*D][d] */
  const void* wk;        /* [Hkv*D][d] */
  const void* wv;        /* [Hkv*D][d] */
  const void* wo;        /* [d][H*D] */
  const void* mlp_norm;  /* [d] */
  const void* w_gate;    /* [F][d] */
  const void* w_up;      /* [F][d] */
  const void* w_down;    /* [d][F] */
} river_layer_weights;

typedef struct river_weights {
  const void* embed;                 /* [V][d] */
  const void* lm_head;               /* [V][d], or NULL when tied_embeddings */
  const void* final_norm;            /* [d] */
  const river_layer_weights* layers; /* host array of n_layers entries */
} river_weights;

/* Shape of the one shared KV cache: dims {L, 2 (K then V), B, Hkv, Tmax, D}. */
typedef struct river_kv_desc {
  int64_t dims[6];
  int64_t strides[6]; /* in elements */
  int32_t elem_bytes; /* 2 (fp16) */
  uint64_t total_bytes;
} river_kv_desc;

typedef struct river_ctx river_ctx;

/* Layout of the single shared KV cache (paperlayer section 4 "KV-Shared Exit Layer": the exit
 * layers use the backbone's KV addressing and an fp16 cache; appendix A.3: one KV set).
 * Host-only, allocates nothing. The caller allocates exactly one buffer of total_bytes; the
 * backbone and the river both write it. Returns RIVER_EINVAL for a bad cfg or NULL out. */
int river_kv_layout(const river_config* cfg, river_kv_desc* out /* host */);

/* Sizes of the two other caller-owned device buffers: `river_bytes` holds the int4 river
 * copy of every block (packed nibbles + fp16 group scales, built by river_init), `scratch_bytes`
 * the decode/prefill activations, split-attention partials and device state. Host-only. */
int river_workspace_bytes(const river_config* cfg, uint64_t* river_bytes /* host */,
                          uint64_t* scratch_bytes /* host */);

/* Builds the river (the W4A16 copy of every block: aitrends construction paragraph) into
 * `river_buf` by quantising the borrowed backbone weights on the device, clears the device
 * state in `scratch`, and returns a context in *out. `kv` (river_kv_layout().total_bytes),
 * `river_buf` and `scratch` (river_workspace_bytes) are caller-owned device buffers that must
 * outlive the context, as must the backbone weights. Enqueued on `stream`; the weights must
 * be ready on it. Errors: RIVER_EINVAL (cfg, NULL pointer), RIVER_EHIP. */
int river_init(const river_config* cfg, const river_weights* w /* host struct */, void* kv,
               void* river_buf, void* scratch, void* stream, river_ctx** out /* host */);

/* Frees the host handle, its stream, graphs and events. Device buffers are the
 * caller's. Synchronises the device. NULL is accepted. */
int river_destroy(river_ctx* ctx);

/* Prompt prefill with a sequence-level exit (paperlayer section 4 "Inference with Seamless
 * Exit"; section 3: the latest-exiting token sets a sequence's depth).
 *   tokens     [B][P] int32 token ids (device), P in [1, max_prefill], P <= max_seq
 *   prefill_exit  0: tau mode -- row b leaves the backbone after layer l (entry <= l < L) when
 *                 the minimum over its P tokens of cos(h_t(l-1), h_t(l)) exceeds tau;
 *                 in [entry, L]: every row exits after that layer (L = full depth)
 *   next_tok   [B] int32 out: greedy token after position P-1
 *   logits     [B][V] fp32 out at position P-1, or NULL
 *   seq_exit   [B] int32 out: each row's exit layer, or NULL
 *   min_sim    [B][L] fp32 out, or NULL: index l-1 holds the minimum similarity after
 *              backbone layer l where it was tested, NaN elsewhere
 * Writes KV slots [0, P) of every layer of every row and sets every row's position to P.
 * Errors: RIVER_EINVAL, RIVER_ERANGE (P or prefill_exit out of range), RIVER_EHIP. */
int river_prefill(river_ctx* ctx, const int32_t* tokens, int32_t P, int32_t prefill_exit,
                  float tau, int32_t* next_tok, float* logits, int32_t* seq_exit, float* min_sim,
                  void* stream);

/* One token-level early-exit decode step for all B rows (aitrends exit-criterion paragraph;
 * paperlayer section 4). Row b reads token tok_in[b], runs at its position pos[b], writes
 * exactly one KV slot per layer at pos[b] -- from the backbone block or its river copy,
 * whichever ran -- and then pos[b] += 1.
 *   tok_in       [B] int32 (may alias tok_out)
 *   forced_exit  [B] int32 exit layer in {0} or [entry, L], or NULL for tau mode (exit after backbone
 *                layer l in [entry, L-1] iff cos(h(l-1), h(l)) > tau). An out-of-range forced
 *                value is treated as L and flags RIVER_EDEVICE (river_device_status).
 *   tok_out      [B] int32 greedy next token (lowest index on ties)
 *   logits       [B][V] fp32, or NULL
 *   exit_layer   [B] int32, or NULL
 *   sim          [B][L] fp32, or NULL: index l-1 holds s(l) where it was computed (tau mode,
 *                backbone layers l >= entry, l < L), NaN elsewhere
 * Errors: RIVER_EINVAL, RIVER_ERANGE (a row's position would pass max_seq; checked on the
 * host against its mirror of the positions), RIVER_EHIP. */
int river_decode_step(river_ctx* ctx, const int32_t* tok_in, const int32_t* forced_exit, float tau,
                      int32_t* tok_out, float* logits, int32_t* exit_layer, float* sim,
                      void* stream);

/* S decode steps in one call, feeding each step's tokens to the next on the device.
 *   tok_in     [B] first input tokens
 *   sched      [S][B] forced exit layers, or NULL for tau mode
 *   tok_out    [S][B]; exit_layer [S][B] or NULL; sim [S][B][L] or NULL
 * Same semantics and errors as S calls of river_decode_step.
 * Execution: a batch-1 context whose shapes the persistent decode kernel covers runs up to 8
 * steps per cooperative launch (one workgroup per compute unit; inside a step each phase waits
 * only for the activations it reads, one grid barrier per step after the LM head); otherwise --
 * or when the environment variable RIVER_PERSIST is "0" at river_init -- the per-op kernels
 * run, replayed from a captured graph. Both give the same results up to floating-point
 * summation order. A wait inside the persistent kernel that exceeds its bound ends the launch
 * early and is reported as RIVER_EDEVICE. */
int river_decode_steps(river_ctx* ctx, const int32_t* tok_in, const int32_t* sched, int32_t S,
                       float tau, int32_t* tok_out, int32_t* exit_layer, float* sim,
                       void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): river_decode_steps with the persistent kernel's
 * cross-workgroup exchange buffers (tagged activations, attention split partials, tag counters,
 * grid-barrier words, argmax keys) in a fixed device array of the library (4 MiB, one per GPU,
 * held until the process ends) instead of the context's scratch. It calls no allocating
 * routine. Same arguments, semantics and results (bit for bit) as river_decode_steps. Every
 * call on a GPU shares that GPU's array and clears the part it uses before its launches, so
 * calls that overlap on one GPU (any contexts, any streams) race and must be serialised by
 * the caller. Errors: as river_decode_steps; RIVER_EINVAL when the context does not decode on
 * the persistent kernel (batch 1, a supported shape, RIVER_PERSIST not "0") or a timer is
 * armed; RIVER_ENOMEM when the model's exchange buffers exceed the array (the message gives
 * both sizes; the 8B shape needs about 3.3 MB); RIVER_EHIP when the array's device address
 * could not be looked up at river_init. */
int river_decode_steps_static(river_ctx* ctx, const int32_t* tok_in, const int32_t* sched, int32_t S,
                              float tau, int32_t* tok_out, int32_t* exit_layer, float* sim,
                              void* stream);

/* Full-depth fp16 decode of S steps: every layer on the backbone block, no exit test, no river
 * (the plain decoder the early exit is measured against). Same token I/O as river_decode_steps
 * with every forced exit = L; writes the same KV slots. Errors as river_decode_steps. */
int river_decode_backbone_steps(river_ctx* ctx, const int32_t* tok_in, int32_t S, int32_t* tok_out,
                                void* stream);

/* Benchmark support: per-launch timing of one kernel of the decode step with HIP events on the
 * call's stream. op: 0 QKV, 1 attention, 2 O projection, 3 gate|up, 4 down, 5 LM head, 6 persistent step kernel. While
 * armed, decode calls enqueue their kernels directly (no graph replay) and record an event pair
 * around each launch of `op`, up to max_launches pairs. op 6 times the launches of the
 * persistent decode kernel (several decode steps per launch) instead. river_timer_read waits for the last
 * event, writes the durations (ms) of up to *n launches in launch order, sets *n to the count
 * and disarms. */
int river_timer_arm(river_ctx* ctx, int32_t op, int32_t max_launches);
int river_timer_read(river_ctx* ctx, float* ms /* host */, int32_t* n /* host, in/out */);

/* Backbone offloading (paperlayer summary, section 4 "Deployment Efficiency" and appendix A.3:
 * under-used backbone blocks are moved out of device memory while the exit river stays, which
 * cuts parameter memory toward that of a static 4-bit model; aitrends offloading paragraph).
 * river_init accepts every borrowed weight pointer either in device memory or in page-locked
 * host memory (hipHostMalloc, or a pinned torch tensor) and uses host memory through its
 * mapped device address: a kernel then reads such a block over the host link, and only when a
 * row runs that backbone block (the batched kernels skip a weight stream no row needs; the
 * river, the embedding and the LM head stay wherever the caller put them). Any other pointer
 * makes river_init fail with RIVER_EINVAL. river_weight_residency (host-only) reports the bytes
 * of the borrowed weights in device memory and in host memory, and of the river buffer. */
int river_weight_residency(const river_ctx* ctx, uint64_t* device_bytes /* host */,
                           uint64_t* host_bytes /* host */, uint64_t* river_bytes /* host */);
/* How river_init would take the weight pointer p: *placement = 0 device memory, 1 page-locked
 * host memory; RIVER_EINVAL when river_init would reject it. Host-only (queries the runtime). */
int river_weight_placement(const void* p, int32_t* placement /* host */);

/* Which kernels serve the decode calls of this context: 1 the persistent decode kernel, 0 the
 * per-op kernels (see river_decode_steps). Host-only. Returns RIVER_EINVAL for NULL. */
int river_decode_path(const river_ctx* ctx, int32_t* persistent /* host */);

/* Host mirror of the rows' positions (number of filled KV slots per row). */
int river_positions(const river_ctx* ctx, int32_t* pos /* host [B] */);

/* Checks the device error word kernels set on bad device-side input (out-of-range token id
 * or forced exit layer). Synchronises `stream`. Returns RIVER_OK or RIVER_EDEVICE (and clears
 * the word). */
int river_device_status(river_ctx* ctx, void* stream);

/* Test support: the river copy of one matrix of one layer (0-based `layer`) in the canonical
 * layout -- packed [N][ceil(K/2)] bytes with element 2i in the low nibble of byte i, and fp16
 * scales [N][ceil(K/group)]. Symmetric format: nibble = q + 8 (q in [-8, 7]), an odd K pads
 * with 8. Zero-point format: nibble = q (q in [0, 15]), an odd K pads with 0, and `zeros`
 * receives the zero points [N][ceil(K/group)] (one byte each; it must be NULL for the
 * symmetric format and non-NULL for the zero-point format). which: 0 wq, 1 wk, 2 wv, 3 wo,
 * 4 w_gate, 5 w_up, 6 w_down. `packed`, `scales` and `zeros` are device buffers. */
int river_export_river(river_ctx* ctx, int32_t layer, int32_t which, uint8_t* packed,
                       uint16_t* scales, uint8_t* zeros, void* stream);

/* Test support: copies the residual stream of the last decode step, fp16 [L+1][B][d]
 * (index 0 = embedding row, index l = output of block l), into the device buffer `dst`. */
int river_debug_hidden(river_ctx* ctx, void* dst, void* stream);

/* Debug support: KV-slot write counts, the check that the shared cache never has an absent
 * or doubly written slot whatever the exit schedule (chatpaper.ai abstract: the KV Cache
 * Absence problem; paperlayer section 4 "KV-Shared Exit Layer": exit layers write the slot the
 * backbone would have written; appendix A.3: one KV set). Only a library built with
 * RIVER_DEBUG_KV_COUNT (libriver_kvcount.so) counts: it keeps one 32-bit counter per element of
 * the cache, incremented by every store of that element (in prefill and in every decode path),
 * cleared by river_init. river_kv_write_counts writes cnt[l][b][t] (uint8, device buffer of
 * L*B*max_seq bytes) = how many times slot (layer l, row b, position t) was written: the common
 * count of its 2*Hkv*D elements, capped at 254, or 255 when its elements were written unequal
 * numbers of times. Enqueued on `stream`. A release library returns RIVER_EINVAL.
 * river_kv_counting sets *enabled to 1 in the debug library, 0 otherwise (host-only). */
int river_kv_write_counts(river_ctx* ctx, uint8_t* cnt, void* stream);
int river_kv_counting(int32_t* enabled /* host */);

/* Debug support: phase timestamps of the persistent batch-1 decode kernel, the measurement
 * behind its per-phase timing (QKV, attention, O, gate|up and down of every block, the LM head
 * and the step's grid barrier). Only a library built with RIVER_PHASE_TRACE
 * (libriver_phasetrace.so) records them: thread 0 of every workgroup stores the 100 MHz
 * realtime counter at each phase boundary of the last persistent launch, at
 * [step][slot][event][workgroup] (slot l-1 for block l, slot L for the head; events: 0 start,
 * 1 input staged, 2 rows done, 3 attention done / past the barrier, 4-5 O staged/done, 6-7
 * gate|up staged/done, 8-9 down staged/done; 0 where nothing was recorded). river_phase_trace
 * writes the array's shape {steps, slots, events, workgroups} to dims[4] (host) and copies its
 * first min(n, size) words to the host buffer dst when dst is not NULL (synchronous; call after
 * the launch has finished). A release library fills dims and returns RIVER_EINVAL. */
int river_phase_trace(uint64_t* dst /* host */, uint64_t n, int32_t* dims /* host, 4 */);

/* Message for the calling thread's last failed call ("" if none). */
const char* river_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RIVER_H */
