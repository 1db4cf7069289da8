// Host-side launch interface of the libdg kernels (one family per source file).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

constexpr int kMaxBatch = 64;
constexpr int kMaxPairs = 128;  // (request, split) pairs of one balanced attention launch

// Per-request row bookkeeping passed by value to kernels: request b owns rows
// [b*rows_per_req, (b+1)*rows_per_req) and row i of it sits at position pos0[b] + i.
// Rows of a call: n_req requests of rows_per_req rows; request b starts at position pos0[b]
// and owns slot slot[b] of the KV cache and of every per-request array (and of the random
// streams, whose counters carry the slot).
struct RowMap {
  int32_t rows_per_req;
  int32_t n_req;
  int32_t pos0[kMaxBatch];
  int32_t slot[kMaxBatch];
};

// Bits of the sticky device-side error word (the workspace's err, read by dg_device_errors).
constexpr uint32_t kDevErrTokenRange = 1u;  // a token id outside [0, vocab) was clamped

// ---- k_norm.hip
// h = E[tok] as float32; with a gain also out = bf16(rmsnorm(h) * gain) (the first layer's
// input).  Ids outside [0, vocab) are clamped and set kDevErrTokenRange in *err.
void launch_embed(const int32_t* tok, const uint16_t* embed, float* h, int rows, int d, int vocab,
                  uint32_t* err, const float* gain, float eps, uint16_t* out, hipStream_t s);
void launch_rmsnorm(const float* h, const float* gain, float eps, uint16_t* out, int rows, int d,
                    hipStream_t s);
void launch_f32_to_bf16(const float* in, uint16_t* out, long n, hipStream_t s);
// Residual update + FFN norm + router: h += sum_z part_z (n_part split-K slices, z order;
// written back); x = h * rsqrt(mean h^2 + eps) * gain in float32 and its bf16 copy b (the
// experts' input); router logits W_router x from the float32 x; top-k (value desc, index asc);
// softmax gates over the k picks.  With w_router_packed (the launch_router_pack copy, when
// router_mfma_path holds) the logits run on MFMA as W (hi + lo), hi = bf16(x), lo = bf16(x - hi),
// float32 accumulation; otherwise on the vector ALUs in float32.
bool router_mfma_path(int d, int n_exp);
void launch_router_pack(const uint16_t* w_router, int n_exp, int d, uint16_t* out, hipStream_t s);
void launch_norm_router(float* h, const float* part, int n_part, long part_stride,
                        const float* gain, float eps, const uint16_t* w_router,
                        const uint16_t* w_router_packed, int rows, int d, int n_exp, int top_k,
                        uint16_t* b_out, int32_t* idx, float* gates, hipStream_t s);

// Destination of the fused QKV projection (EPI_ROPE_QKV): q heads and k heads rotated with
// the table (rotate-half; null table = no rotation), q -> q [rows][Hq*D] bf16, k / v ->
// k_dst / v_dst + ((b*Hkv + g)*kv_cap + slot0[b] + i)*D bf16 for row i of request b.
struct RopeArgs {
  int Hq; int Hkv; int D;
  const float* table;
  uint16_t* q; uint16_t* k_dst; uint16_t* v_dst; int kv_cap;  // per-layer base
  RowMap map; int32_t slot0[kMaxBatch];
};

// ---- k_gemm.hip : C[t][f] = sum_k X[t][k] * W[f][k]
// EPI_ROPE_QKV: W is the QKV weight with the rows of every q and k head in the order
// {j, j + D/2, j + 1, j + 1 + D/2} for j = 0, 2, 4, ... (launch_pack_qkv), so the four
// consecutive outputs a lane holds are two rotation pairs; the products go through RopeArgs.
enum GemmEpi { EPI_STORE_F32 = 0, EPI_ADD_F32 = 1, EPI_SWIGLU_BF16 = 2, EPI_STORE_BF16 = 3, EPI_ROPE_QKV = 4 };
struct GemmArgs {
  const uint16_t* x; int ldx; int n_tok;
  const uint16_t* w0; const uint16_t* w1;  // w1: up matrix for SwiGLU
  // optional segmented W (QKV): rows [seg_start[s], seg_start[s+1]) come from seg_w[s]
  const uint16_t* seg_w[3]; int seg_start[4]; int n_seg;
  int K; int N;
  float* out_f32; uint16_t* out_bf16; int ldo;
  // split-K: with split > 1 the k range is cut into `split` slices and slice z stores its raw
  // fp32 product to part + z * part_stride (+ part_stride / 2 for the up matrix of the SwiGLU
  // pair), row-major [n_tok][N]; the consumer sums the slices in z order.
  int split; float* part; long part_stride;
  RopeArgs rope;  // EPI_ROPE_QKV only (split 1)
};
// QKV weight for EPI_ROPE_QKV: rows of wq (Hq heads) then wk (Hkv heads) in the rotation-pair
// order above, then wv unchanged; out [(Hq+2Hkv)*D][d] bf16.
void launch_pack_qkv(const uint16_t* wq, const uint16_t* wk, const uint16_t* wv, uint16_t* out,
                     int Hq, int Hkv, int D, int d, hipStream_t s);
// Largest split (1, 2 or 4) that keeps >= 16 k-tiles of 64 per slice and stays within `cap`
// partial floats while the grid stays within ~512 work-groups.
int gemm_split(const GemmArgs& a, int epi, long cap);
void launch_gemm(const GemmArgs& a, int epi, hipStream_t s);
// act[t][f] = bf16(silu(sum_z gate_z) * sum_z up_z) over `split` partial slices
void launch_swiglu_reduce(const float* part, long part_stride, int split, uint16_t* act, int rows,
                          int n, hipStream_t s);

// Fused vocab head: logits never leave registers.  Writes per (row, 64-wide vocab slice)
// partial statistics; launch_head_merge reduces them into row statistics.
struct HeadArgs {
  const uint16_t* f; int n_rows;      // bf16 [rows][d] final normed state
  const uint16_t* w; int K; int V;    // lm_head [V][d]
  uint32_t k0, k1;                    // Philox key (seed)
  float temp[kMaxBatch];              // temperature T of each request (t = z / T)
  int32_t step[kMaxBatch];            // denoise step of each request (Philox counter)
  const int32_t* cur_tok;             // [rows] current canvas token
  RowMap map;
  float* part;                        // [rows][n_slices][8]
  float* dbg_logits;                  // optional [rows][V]
};
void launch_head(const HeadArgs& a, hipStream_t s);
// cur_tok ids outside [0, n_slices * slice_w) are clamped and set kDevErrTokenRange in *err
void launch_head_merge(const float* part, int n_rows, int n_slices, int slice_w,
                       const int32_t* cur_tok, uint32_t* err, int32_t* cand, float* t_cand,
                       float* t_cur, float* lse, float* ent, const RowMap& map, hipStream_t s);
// dst[b][i] = src[map.slot[b]][i] for the map's requests (rows_per_req ints each)
void launch_gather_rows(const int32_t* src, int32_t* dst, const RowMap& map, hipStream_t s);

// ---- k_attn.hip
constexpr int kMaxParts = 4;  // largest split-K slice count a consumer sums

// cos / sin of the RoPE angle pos * theta^(-2j/D) for every row and j < D/2, formed in float64
// and rounded to float32: table[r][j] = {cos, sin}.  Built once per step (all layers share it).
void launch_rope_table(const RowMap& map, int rows, int D, float theta, float* table, hipStream_t s);



struct AttnArgs {
  const uint16_t* q;       // [rows][Hq*D]
  uint16_t* out;           // [rows][Hq*D]
  const uint16_t* kc; const uint16_t* vc; int cap;   // cache base of the layer [slots][Hkv][cap][D]
  const uint16_t* kx; const uint16_t* vx; int xcap;  // extra keys (canvas) [B][Hkv][xcap][D]
  int Hq, Hkv, D;
  int rows_per_req; int n_req;
  int32_t n_cache[kMaxBatch];   // keys read from the cache per request
  int32_t n_extra;              // canvas keys (0 in prefill)
  int32_t q_pos0[kMaxBatch];    // position of the first query row of each request
  int32_t slot[kMaxBatch];      // cache slot of each request (kc/vc hold [n_slots][Hkv][cap][D])
  int causal;                   // key position <= query position
  float scale;                  // 1/sqrt(D)
  int n_split; int split_keys;  // split-KV: each split covers split_keys keys
  float* part_o; float* part_ml;  // partials when n_split > 1
  int n_waves;                    // query tasks per work-group: 4 or 8 (attention_waves)
  int q_tiles;                    // 16-row query tiles per wave task: 1 or 2 (0 means 2)
  // Per-request splits (the pipelined canvas kernel, attention_pipe_path): request b's keys
  // are cut into req_split[b] ranges of req_split_keys[b] keys (n_split is then the largest
  // count, the stride of the partial slots), and work-groups take the (request, split) pairs
  // pair[0 .. n_pairs) = request << 8 | split in that order, longest range first.
  int balanced;
  int32_t req_split[kMaxBatch];
  int32_t req_split_keys[kMaxBatch];
  int32_t n_pairs;
  uint16_t pair[kMaxPairs];
};
// True when launch_attention runs the pipelined kernel for these arguments (head dim 128, 8
// waves, 32-row query tasks, with or without the causal mask); it takes per-request splits.
bool attention_pipe_path(const AttnArgs& a);
// Work-group shape for a key range of max_keys.  Waves: 8 from 2048 keys on the canvas path
// and from 8192 in the causal prefill (each staged block serves more queries), else 4.  Query tiles per wave: 2 (32 rows) for long ranges and the
// causal prefill, where each K fragment read from LDS then feeds two MFMAs; 1 (16 rows) for a
// canvas over a prefix under 8192 keys, where the doubled task count lets a shorter split fill
// the chip (fewer split partials to write and merge) at fewer registers per wave.
int attention_waves(int max_keys, bool causal);
int attention_q_tiles(int max_keys, bool causal);
// The attention kernel (with n_split > 1 it writes split partials), then the fixed-order merge
// of the partials into `out` (nothing to do for one split).
void launch_attention(const AttnArgs& a, hipStream_t s);
void launch_attention_combine(const AttnArgs& a, hipStream_t s);

// ---- k_moe.hip
void launch_moe_permute(const int32_t* idx, int n_routes, int n_exp, int32_t* offs,
                        int32_t* perm, int32_t* inv, hipStream_t s);
struct MoeArgs {
  const uint16_t* x; int ldx;       // GEMM1: normed rows b [rows][d]; GEMM2: act [routes][F]
  const int32_t* perm; int top_k;   // GEMM1 gathers row perm[p]/top_k; GEMM2 reads row p
  const int32_t* offs;              // [E+1]
  const uint16_t* wp;               // expert weights in the packed fragment layout (below)
  int K; int N;                     // reduction length and output features per expert
  uint16_t* out_bf16; int ldo;      // GEMM1: bf16 SwiGLU; GEMM2: the bf16 products
  int n_exp;
  // E4M3 experts (instead of wp): packed bytes and per-channel scales [E][N] of matrix q
  const uint8_t* wp8; const float* wscale0; const float* wscale1;
  // GEMM1 only, optional: rank the routes itself from the router's choices idx [n_routes]
  // (n_routes <= kFusedRoutes) instead of reading offs / perm; the work-groups with
  // blockIdx.x = blockIdx.z = 0 then write offs_w [E+1], perm_w and inv_w [n_routes] for the
  // down projection and the combine.
  const int32_t* idx; int n_routes;
  int32_t* offs_w; int32_t* perm_w; int32_t* inv_w;
};
constexpr int kFusedRoutes = 2048;
// Packed expert weights: for expert e, 16-row tile ft and 32-wide k-step s, the MFMA A-operand
// fragment of every matrix q (GEMM1: q = gate, up; GEMM2: q = down) is 64 lanes x 16 B, lane l
// holding W_q[e][16 ft + l % 16][32 s + 8 (l / 16) .. + 8].  Order:
// [e][ft / G][s][ft % G][q][lane] with G = group_tiles, the tiles one work-group streams, so a
// work-group reads one contiguous run.  N must be a multiple of 16 G.
constexpr int kGroupTiles1 = 4;  // gate/up: 64 features per work-group
constexpr int kGroupTiles2 = 8;  // down: 128 features per work-group
void launch_moe_pack(const uint16_t* w0, const uint16_t* w1, uint16_t* out, int n_exp, int N,
                     int K, int group_tiles, hipStream_t s);
// E4M3 experts: per-row quantization (bf16 [rows][cols] -> bytes + float32 scale per row), and
// the byte layout [e][ft / G][s2][ft % G][q][lane][16 B] whose 16 bytes per lane are the A
// fragments of k-steps 2 s2 and 2 s2 + 1 (8 bytes each; K a multiple of 64)
void launch_quantize_e4m3(const uint16_t* w, long rows, int cols, uint8_t* q, float* scale,
                          hipStream_t s);
void launch_moe_pack_fp8(const uint8_t* q0, const uint8_t* q1, uint8_t* out, int n_exp, int N,
                         int K, int group_tiles, hipStream_t s);
// mean_rows: routed rows per expert on average (selects the token-tile depth per pass)
void launch_moe_gemm1(const MoeArgs& a, int mean_rows, hipStream_t s);
void launch_moe_gemm2(const MoeArgs& a, int mean_rows, hipStream_t s);
// h[t] += sum_z part_z[t] (n_part residual slices, z order) + sum_j gate[t][j] * y[inv[t][j]]
// (y: the down projection's bf16 outputs, widened exactly); with a gain also
// out[t] = bf16(rmsnorm(h[t]) * gain) (the next block's input)
void launch_moe_combine(float* h, const float* part, int n_part, long part_stride, const uint16_t* y,
                        const int32_t* inv, const float* gates, int rows, int d, int top_k,
                        const float* gain, float eps, uint16_t* out, hipStream_t s);

// ---- k_sampler.hip
struct SamplerArgs {
  int32_t* tokens; uint8_t* committed; int32_t* stable_run; int32_t* stopped;
  const int32_t* cand; const float* t_cand; const float* t_cur; const float* lse;
  const float* ent;
  void* status;  // dg_step_status[B]
  int C; int V; int max_steps; int commit_m; float log_tau; int stable_steps;
  float entropy_stop; int renoise_committed; uint32_t k0, k1;
  int select_mode;       // 0: top commit_m by confidence; 1: entropy-bounded
  float entropy_budget;  // select_mode 1: bound on the running entropy sum of the selection
  int32_t pos0[kMaxBatch];
  int32_t slot[kMaxBatch];  // per-request arrays (state, stats, status) are indexed by slot
  int32_t step[kMaxBatch];  // sampler step of each request
};
void launch_sample_commit(const SamplerArgs& a, int n_req, hipStream_t s);
void launch_canvas_init(int32_t* tokens, uint8_t* committed, int32_t* stable_run,
                        int32_t* stopped, int C, int V,
                        uint32_t k0, uint32_t k1, const RowMap& map, hipStream_t s);
// Copy canvas K/V [B][Hkv][C][D] of one layer into the cache at [len[b], len[b]+C).
// Request b of the map takes the canvas K/V of request src.idx[b] of the call that produced
// them (src [requests][Hkv][C][D]).
struct ReqIndex {
  int32_t idx[kMaxBatch];
};
void launch_kv_append(const uint16_t* src_k, const uint16_t* src_v, uint16_t* dst_k,
                      uint16_t* dst_v, int B, int Hkv, int C, int D, int cap,
                      const RowMap& map, const ReqIndex& src, hipStream_t s);

}  // namespace dg
