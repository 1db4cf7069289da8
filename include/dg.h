/*
 * dg.h — C ABI of libdg: the denoise step of a block-autoregressive, uniform-state
 * discrete-diffusion language model on AMD MI355X (gfx950).
 *
 * The method (sources cited by tag; the pages are):
 *   [GUIDE] "DiffusionGemma Guia do Desenvolvedor para Decodificação Paralela a 1000+ Tokens/s"
 *           (dev.infolabhq.com), sections "Arquitetura em Detalhes" and the Sudoku demo;
 *   [NEWS]  "Google's DiffusionGemma Atinge 1.000 Tokens por Segundo" (aiexpert.news), 2nd ¶;
 *   [RANK]  "DiffusionGemma: geração de texto até 4x mais rápida…" (pulsar-ranking.com),
 *           "Pontos-chave";
 *   [DOCS]  Google's DiffusionGemma documentation (ai.google.dev/gemma/docs/diffusiongemma),
 *           feature list and table "Configuração de exibição recomendada".
 *
 * A prompt is prefilled causally into a KV cache ([GUIDE] "Arquitetura em Detalhes"; [NEWS]).
 * A canvas of 256 random tokens is then refined in parallel: each denoise step is one forward
 * pass in which every canvas position attends, unmasked, to the cached prefix and to the whole
 * canvas ([GUIDE] Sudoku demo; [RANK]; [DOCS] feature list), followed by a sampler that draws a
 * candidate per position at a falling temperature, commits the most confident positions and
 * puts random tokens back where confidence is low ([NEWS]; [DOCS] table).  A finished canvas is
 * appended to the KV cache and the next one starts ([GUIDE]; [NEWS]; [DOCS] feature list).
 *
 * Conventions for every function below:
 *  - Pointers are DEVICE memory unless marked (host).  bf16 tensors are passed as uint16_t
 *    (the upper half of an IEEE float32); all matrices are row-major, [out][in].
 *  - The caller owns every buffer it passes; libdg never frees caller memory.  libdg owns the
 *    context and a workspace it allocates in dg_create (activations, per-layer canvas K/V,
 *    split-attention partials, MoE routing tables) and frees in dg_destroy.
 *  - Calls are asynchronous on `stream` (hipStream_t).  No call synchronizes the stream.
 *  - Every argument and shape is validated BEFORE anything is enqueued: a non-zero return
 *    leaves the device untouched.  dg_last_error() returns the message of the last failure.
 *  - Device-side conditions (non-finite logits) are reported in dg_step_status, not as errors.
 *  - A context is not thread-safe; use one context per stream.  Kernels are deterministic:
 *    the same inputs give bit-identical outputs (no floating-point atomics).
 */
#ifndef DG_H_
#define DG_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dg_ctx dg_ctx;

enum {
  DG_OK = 0,
  DG_ERR_ARG = -1,         /* null pointer / bad value */
  DG_ERR_SHAPE = -2,       /* shape not supported by the kernels (see dg_create) */
  DG_ERR_CAPACITY = -3,    /* KV cache or workspace too small for the request */
  DG_ERR_HIP = -4,         /* HIP runtime error (message in dg_last_error) */
  DG_ERR_UNSUPPORTED = -5  /* flag combination not supported */
};

/* Model shape.  Supported: head_dim 64 or 128; d_model a multiple of 128 (<= 8192);
 * d_ff_expert a multiple of 128 (<= 1024); n_q_heads*head_dim and d_ff_shared multiples of 64; n_q_heads a multiple of n_kv_heads; 1 <= top_k <= n_experts
 * <= 64; vocab a multiple of 128, <= 131072; canvas == 256 ([GUIDE] "Arquitetura em Detalhes": fixed
 * 256-token blocks).  rope_theta 0 disables RoPE (rotate-half, absolute positions). */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim;
  int32_t n_experts, top_k, d_ff_expert, d_ff_shared /* 0 = no shared FFN */, vocab, canvas;
  float rms_eps, rope_theta;
  int32_t expert_fp8; /* 0: routed experts stream as bf16.  1: dg_create quantizes every routed
                         expert matrix to OCP E4M3 with one float32 scale per output channel
                         (dg_quantize_e4m3_rows) and the expert GEMMs stream those bytes
                         ([NEWS] third and fourth paragraphs: FP8 checkpoints, FP8 serving);
                         attention, router, shared FFN and head stay bf16. */
} dg_model_desc;

/* One decoder layer (pre-norm attention block, then routed MoE FFN + optional shared FFN).
 * Norm gains are float32 [d_model]; every matrix is bf16 row-major [out][in]. */
typedef struct {
  const float* attn_norm;
  const uint16_t* wq;       /* [n_q_heads*head_dim][d_model] */
  const uint16_t* wk;       /* [n_kv_heads*head_dim][d_model] */
  const uint16_t* wv;       /* [n_kv_heads*head_dim][d_model] */
  const uint16_t* wo;       /* [d_model][n_q_heads*head_dim] */
  const float* ffn_norm;
  const uint16_t* w_router; /* [n_experts][d_model] */
  const uint16_t* w_gate;   /* [n_experts][d_ff_expert][d_model] */
  const uint16_t* w_up;     /* [n_experts][d_ff_expert][d_model] */
  const uint16_t* w_down;   /* [n_experts][d_model][d_ff_expert] */
  const uint16_t* ws_gate;  /* [d_ff_shared][d_model], NULL when d_ff_shared == 0 */
  const uint16_t* ws_up;    /* [d_ff_shared][d_model] */
  const uint16_t* ws_down;  /* [d_model][d_ff_shared] */
} dg_layer_weights;

typedef struct {
  const uint16_t* embed;          /* [vocab][d_model] */
  const float* final_norm;        /* [d_model] */
  const uint16_t* lm_head;        /* [vocab][d_model] (untied) */
  const dg_layer_weights* layers; /* (host) [n_layers]; copied by dg_create */
} dg_weights;

/* KV cache: bf16 K (after RoPE) and V, layout [n_layers][n_slots][n_kv_heads][cap][head_dim].
 * A call works on `batch` requests; request b lives in slot slot[b] (slot NULL: slot b) of the
 * cache and of every per-request array passed with it (canvas tokens, canvas state, row
 * statistics, step status: all [n_slots][...]), and its random streams carry the slot, so a
 * request draws the same numbers whichever other requests share the call.  This lets a
 * scheduler run only the live requests of a larger pool (continuous batching).  len (host)
 * holds the committed length of each request of the call; dg_prefill_causal and
 * dg_commit_block advance it when they enqueue their work. */
typedef struct {
  uint16_t* k;
  uint16_t* v;
  int32_t cap;
  int32_t batch;          /* requests of this call, 1 <= batch <= max_batch */
  int32_t* len;           /* (host) [batch] */
  const int32_t* slot;    /* (host) [batch] distinct slots in [0, n_slots), or NULL */
  int32_t n_slots;        /* slots in k/v and in the per-request arrays; 0 means batch */
} dg_kv_cache;

/* Sampler state of `batch` canvases ([NEWS] 2nd ¶: committed anchors; re-noising). */
typedef struct {
  int32_t* tokens;     /* [batch][canvas] current token per slot */
  uint8_t* committed;  /* [batch][canvas] 1 = committed */
  int32_t* stable_run; /* [batch] consecutive steps that changed no token */
  int32_t* stopped;    /* [batch] 1 once the request's sampler has stopped; its canvas is then
                          left untouched by further sampler steps */
} dg_canvas_state;

/* Per-position statistics written by dg_denoise_step, consumed by dg_sample_commit.
 * With t = logits / T: cand = argmax(t + Gumbel), t_cand = t[cand], t_cur = t[current token],
 * lse = log-sum-exp(t), entropy of softmax(t).  Each [batch][canvas]. */
typedef struct {
  int32_t* cand;
  float* t_cand;
  float* t_cur;
  float* lse;
  float* entropy;
} dg_row_stats;

/* Sampler parameters ([DOCS] table "Configuração de exibição recomendada": 48 steps,
 * temperature linear 0.8 -> 0.4; commit/re-noise/stop readings documented in the oracle). */
typedef struct {
  int32_t max_steps;         /* 48 */
  float temp_start;          /* 0.8 */
  float temp_end;            /* 0.4 */
  int32_t commit_per_step;   /* 16 */
  float renoise_conf;        /* 0.1: re-noise when the tempered probability is below this */
  int32_t stable_steps;      /* 2: stop after this many consecutive unchanged steps */
  float entropy_stop;        /* < 0 off; else also stop when mean entropy < it and unchanged */
  int32_t renoise_committed; /* 1: committed positions whose confidence drops are re-noised */
  uint64_t seed;
  int32_t select_mode;       /* which uncommitted positions are committed each step:
                                0: the commit_per_step most confident ones;
                                1: entropy-bounded ([DOCS] table, token-selection row): in
                                   ascending order of entropy while the running float32 sum of
                                   their entropies stays <= entropy_budget, at least one */
  float entropy_budget;      /* 0.1 (select_mode 1) */
} dg_sampler_cfg;

/* Per-request result of dg_sample_commit (device [batch]). */
typedef struct {
  int32_t changed, n_committed, n_new, n_renoised, stable_run, stop, nonfinite;
  float mean_entropy;
} dg_step_status;

/* Optional per-step dumps (device buffers; any may be NULL).  Row index r = b*canvas + i. */
typedef struct {
  float* hidden_out;       /* [rows][d_model] residual stream after the last layer */
  uint16_t* attn_out;      /* [n_layers][rows][n_q_heads*head_dim] attention output (bf16) */
  float* h_mid;            /* [n_layers][rows][d_model] residual after the attention block */
  int32_t* expert_idx;     /* [n_layers][rows][top_k] */
  float* gates;            /* [n_layers][rows][top_k] */
  float* logits;           /* [rows][vocab] raw logits (test sizes only) */
  uint16_t* canvas_k;      /* [n_layers][batch][n_kv_heads][canvas][head_dim] */
  uint16_t* canvas_v;      /* same */
  float* layer_out;        /* [n_layers][rows][d_model] residual after each layer (the next
                              layer's input; the last one equals hidden_out) */
  /* The token permutation of every layer's routed experts.  Route r = row * top_k + j is the
   * j-th expert pick of row `row`; routes are ordered by (expert, r), a stable sort by expert. */
  int32_t* route_offs;     /* [n_layers][n_experts + 1] first sorted position of each expert */
  int32_t* route_perm;     /* [n_layers][rows * top_k] route at each sorted position */
  int32_t* route_inv;      /* [n_layers][rows * top_k] sorted position of each route */
} dg_debug;

enum {
  DG_STEP_HIDDEN_IN = 1u << 0, /* hidden_in = float32 [rows][d_model] replaces the embedding */
  DG_STEP_NO_HEAD = 1u << 1,   /* run the layers only (no vocab projection, no row stats) */
  DG_STEP_HEAD_ONLY = 1u << 2  /* hidden_in = bf16 [rows][d_model] already-normed final state;
                                  only the vocab projection + row statistics run */
};

typedef struct {
  int32_t step;          /* denoise step s (selects the temperature and the RNG counter) */
  uint32_t flags;        /* DG_STEP_* */
  const void* hidden_in; /* see flags */
  const dg_debug* debug; /* (host) optional, may be NULL */
  const int32_t* steps;  /* (host) [batch] the step of each request (requests at different
                            points of their canvases, continuous batching), or NULL: `step`
                            for every request */
} dg_step_params;

/* Create a context for `desc` over caller-owned device weights.  The expert banks (w_gate,
 * w_up, w_down) are copied once into the context's own memory in the layout the expert GEMMs
 * stream (MFMA operand fragments, contiguous per group of 16-row tiles; as E4M3 bytes plus
 * per-channel scales when desc->expert_fp8 is set); they are read only during
 * dg_create.  Every other weight pointer must stay valid for the context's lifetime.  max_batch: largest batch
 * (<= 64) of later calls; max_prefill_rows: largest prefill chunk processed at once (rows are
 * split into chunks of this size).  Returns DG_OK and *out, or an error code. */
int dg_create(const dg_model_desc* desc, const dg_weights* weights, int32_t max_batch,
              int32_t max_prefill_rows, dg_ctx** out);
void dg_destroy(dg_ctx* ctx);
/* Message of the last failure on ctx (or, when ctx is NULL, of the last failed dg_create or
 * dg_quantize_e4m3_rows). */
const char* dg_last_error(const dg_ctx* ctx);
/* The temperature of step `step`: T0 + (T1 - T0) * step / (max_steps - 1), rounded to float32
 * once ([DOCS] table, temperature row). */
float dg_temperature(const dg_sampler_cfg* cfg, int32_t step);

/* Per-row OCP E4M3 quantization, the rule dg_create applies to the experts when
 * desc->expert_fp8 is set ([NEWS] third paragraph: FP8 checkpoints).  w: device bf16
 * [rows][cols]; q: device uint8 [rows][cols]; scale: device float32 [rows].  Per row:
 * scale = amax / 448 in float32 (amax the largest |w|; 1 for an all-zero row), and
 * q = E4M3(float32(w) / scale) with the division in float32, rounding to nearest with ties to
 * even and saturating at +-448.  rows >= 0, 1 <= cols <= 65536.  Asynchronous on `stream`;
 * DG_ERR_ARG for null pointers or bad sizes (nothing enqueued). */
int dg_quantize_e4m3_rows(const uint16_t* w, int64_t rows, int32_t cols, uint8_t* q,
                          float* scale, hipStream_t stream);

/* Causal prefill ([GUIDE] "Arquitetura em Detalhes"; [NEWS] 2nd ¶; [DOCS] autoregressive
 * encoder): request b's n_new[b] tokens (packed back to back in `tokens`, device int32, each in
 * [0, vocab); an id outside is clamped and reported by dg_device_errors) are
 * placed at positions len[b] .. len[b]+n_new[b]-1; each attends to its cached history and to
 * itself and earlier new tokens.  Every layer's K (after RoPE) and V are written into the cache
 * and len[b] advances by n_new[b].  Needs len[b] + n_new[b] <= cap.  n_new: (host) [batch]. */
int dg_prefill_causal(dg_ctx* ctx, const int32_t* tokens, const int32_t* n_new, int32_t batch,
                      dg_kv_cache* kv, hipStream_t stream);

/* Uniform-state canvas start ([GUIDE] "Arquitetura em Detalhes"): slot i of request b gets the
 * uniform token Philox(seed; 0, len[b]+i, 0, (b<<8)|2) -> (w*V)>>32; committed = 0;
 * stable_run = 0; stopped = 0. */
int dg_canvas_init(dg_ctx* ctx, dg_canvas_state* state, const dg_kv_cache* kv,
                   const dg_sampler_cfg* cfg, hipStream_t stream);

/* One denoise forward pass over the canvases `canvas` ([batch][canvas] device int32, ids in
 * [0, vocab); an id outside is clamped and reported by dg_device_errors) of the
 * kv->batch requests: canvas slot i sits at position len[b]+i and attends, with no mask, to
 * cache[0:len[b]] and to all canvas slots; top-k MoE FFN; final norm; vocab projection fused
 * with temperature, log-sum-exp, entropy and the Gumbel-max draw (logits never reach HBM).
 * Writes `out` (unless DG_STEP_NO_HEAD) and keeps every layer's canvas K/V in the workspace
 * for dg_commit_block.  cfg supplies the temperature schedule and the seed. */
int dg_denoise_step(dg_ctx* ctx, const int32_t* canvas, const dg_kv_cache* kv,
                    const dg_sampler_cfg* cfg, const dg_step_params* params,
                    dg_row_stats* out, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): dg_denoise_step restricted to params->flags ==
 * DG_STEP_HEAD_ONLY (params->hidden_in = bf16 [batch*canvas][d_model] normed final states), with
 * the same arguments, checks and results, bit for bit.  Its scratch (the per-(row, 64-entry vocab
 * slice) partial statistics, and the gathered canvas tokens of a slot-mapped call) lives in a
 * fixed 16 MiB device array inside the library instead of the context's workspace, and the call
 * allocates nothing: rows * (vocab / 64) * 32 + rows * 4 bytes must fit in 16 MiB (at vocab 65536:
 * up to 512 rows, two canvases), else DG_ERR_CAPACITY with nothing enqueued.  The array is one
 * per device and keeps the last call's contents (every entry a call reads is written by that call
 * first); calls that overlap on one device, from any context or stream, race on it. */
int dg_denoise_head_static(dg_ctx* ctx, const int32_t* canvas, const dg_kv_cache* kv,
                           const dg_sampler_cfg* cfg, const dg_step_params* params,
                           dg_row_stats* out, hipStream_t stream);

/* Sampler step `step` on every canvas ([NEWS] 2nd ¶; [GUIDE] Sudoku demo; [DOCS] table):
 * commit the min(commit_per_step, #uncommitted) uncommitted slots with the highest candidate
 * log-confidence t_cand - lse (lowest slot on ties); re-noise committed slots whose current
 * log-confidence fell below log(renoise_conf) (if renoise_committed); other uncommitted slots
 * take their candidate if its log-confidence >= log(renoise_conf), else a fresh uniform token
 * Philox(seed; 0, pos, step, (b<<8)|1).  Updates state and writes status[batch].  A request
 * whose `stopped` flag is already set is left unchanged (status: stop 1, changed 0).  steps:
 * (host) [batch] per-request steps, or NULL for `step` everywhere. */
int dg_sample_commit(dg_ctx* ctx, dg_canvas_state* state, const dg_row_stats* stats,
                     const dg_sampler_cfg* cfg, int32_t step, const int32_t* steps,
                     const dg_kv_cache* kv, dg_step_status* status, hipStream_t stream);

/* Append each finished canvas's K/V to the cache at [len[b], len[b]+canvas) and advance len
 * ([GUIDE] "Arquitetura em Detalhes"; [NEWS] 2nd ¶).  refresh selects where the K/V come from:
 *   DG_COMMIT_LAST (0): the ones the last forward pass computed (bidirectional canvas),
 *     found by slot: every slot of `kv` must have been a request of that pass, in any order,
 *     else DG_ERR_ARG and nothing is written;
 *   DG_COMMIT_REFRESH (1): first re-run the layers (no head) on `canvas` ([batch][canvas]
 *     device int32), needed when the last sampler step changed the canvas;
 *   DG_COMMIT_CAUSAL (2): re-encode `canvas` causally, as a continuation of the prompt (each
 *     slot attends to the cache and to earlier slots; [DOCS] feature list, autoregressive
 *     encoder): exactly dg_prefill_causal of the canvas tokens.
 * The copy is bit-exact; nothing outside the appended slices is written. */
enum { DG_COMMIT_LAST = 0, DG_COMMIT_REFRESH = 1, DG_COMMIT_CAUSAL = 2 };
int dg_commit_block(dg_ctx* ctx, const int32_t* canvas, dg_kv_cache* kv, int32_t refresh,
                    hipStream_t stream);

/* Per-kernel device timing for measurement runs: while enabled, every kernel launch is
 * bracketed by HIP events recorded on its launch stream.  dg_timing_read waits for the recorded
 * events, writes up to `max` per-kernel-family totals (name is a static string) and clears the
 * record.  Returns the number of entries written, or a negative dg_status. */
typedef struct {
  const char* name;
  int32_t launches;
  float total_ms;
} dg_kernel_time;
int dg_timing_enable(dg_ctx* ctx, int32_t enable);
int dg_timing_read(dg_ctx* ctx, dg_kernel_time* out, int32_t max);

/* Sticky device-side error bits, set by kernels instead of reading out of bounds:
 *   DG_DEVERR_TOKEN_RANGE: a token id passed to dg_prefill_causal or dg_denoise_step (or a
 *     canvas token read by the head) lay outside [0, vocab); it was clamped into range, so the
 *     results of that call are not meaningful.
 * Waits for `stream`, writes the bits accumulated since the last read to *flags (host) and
 * clears them.  Token ids must lie in [0, vocab): this is the callers' precondition, the flag
 * only reports its violation. */
enum { DG_DEVERR_TOKEN_RANGE = 1 };
int dg_device_errors(dg_ctx* ctx, uint32_t* flags, hipStream_t stream);

/* Test hook: load canvas K/V ([n_layers][batch][n_kv_heads][canvas][head_dim] bf16) into the
 * workspace, as if a denoise step had produced them. */
int dg_debug_set_canvas_kv(dg_ctx* ctx, const uint16_t* k, const uint16_t* v, int32_t batch,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DG_H_ */
