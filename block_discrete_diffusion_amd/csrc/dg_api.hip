// libdg C ABI: argument validation, workspace, and the launch sequence of each entry point.
// See include/dg.h for the contract of every function.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <mutex>
#include <vector>

#include "../../include/dg.h"
#include "dg_kernels.h"

using namespace dg;

// Fixed device scratch of the allocation-free head entry point (dg_denoise_head_static): the
// per-(row, slice) partial statistics of the vocab head, then the call's gathered canvas tokens.
// Each device the library runs on holds its own copy of this array until the process ends; host
// code never uses the array's name as an address (it is a host-side stand-in), only the device
// address hipGetSymbolAddress returns for the current device (scratch_address below).
constexpr long kStaticScratchBytes = 16L << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

thread_local std::string g_create_error;

// Device address of `scratch` on each device, looked up once per device with it current.
std::mutex g_scratch_mu;
void* g_scratch_ptr[256] = {};

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 256) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

struct Buf {
  void* p = nullptr;
  size_t bytes = 0;
};

}  // namespace

struct dg_ctx {
  dg_model_desc m{};
  dg_weights w{};
  std::vector<dg_layer_weights> layers;
  int max_batch = 0, max_prefill = 0;
  int r_canvas = 0;  // max_batch * canvas
  int r_max = 0;     // max(r_canvas, max_prefill)
  int part_cap = 0;  // (row, head, split) slots of the attention partial buffers
  std::string err;
  std::vector<void*> allocs;

  // measurement: HIP events around launches (dg_timing_enable)
  struct Rec {
    const char* name;
    hipEvent_t a, b;
  };
  bool timing = false;
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t event() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    (void)hipEventCreate(&e);
    return e;
  }

  // workspace
  float* h = nullptr;          // [r_max][d]
  uint16_t* a = nullptr;       // [r_max][d]
  uint16_t* q = nullptr;       // [r_max][Hq D]
  uint16_t* attn = nullptr;    // [r_max][Hq D]
  float* part_o = nullptr;     // [part_cap][D]
  float* part_ml = nullptr;    // [part_cap][2]
  int32_t* eidx = nullptr;     // [r_max][k]
  float* gates = nullptr;      // [r_max][k]
  int32_t* offs = nullptr;     // [E+1]
  int32_t* perm = nullptr;     // [r_max*k]
  int32_t* inv = nullptr;      // [r_max*k]
  uint16_t* act = nullptr;     // [r_max*k][F]
  uint16_t* y = nullptr;       // [r_max*k][d] bf16 expert outputs
  uint16_t* sact = nullptr;    // [r_max][Fs]
  uint16_t* f = nullptr;       // [r_canvas][d]
  float* head_part = nullptr;  // [r_canvas][V/64][8]
  float* gpart = nullptr;      // split-K partial slices of the dense GEMMs
  float* rope = nullptr;       // [r_max][D/2][2] cos/sin of the rows of the current step
  int32_t* tok = nullptr;      // [r_canvas] canvas tokens of a slot-mapped call, in call order
  uint32_t* dev_err = nullptr; // sticky device-side error bits (kDevErr*), read by dg_device_errors
  void* static_scratch = nullptr;  // this device's `scratch` (dg_denoise_head_static)
  std::vector<int32_t> last_slots;  // slots of the requests whose canvas K/V the workspace holds
  uint16_t* ck = nullptr;      // [L][max_batch][Hkv][C][D]
  uint16_t* cv = nullptr;
  std::vector<uint16_t*> wqkv;  // per layer: QKV weight in rotation-pair row order
  std::vector<uint16_t*> pk1;  // per layer: packed gate/up expert weights
  std::vector<uint16_t*> pk2;  // per layer: packed down expert weights
  std::vector<uint16_t*> wr_pk;  // per layer: router weights in MFMA fragment order (or empty)
  // E4M3 experts (desc.expert_fp8): packed bytes and per-channel scales [E][N] per matrix
  std::vector<uint8_t*> pk1_8, pk2_8;
  std::vector<float*> sc_gate, sc_up, sc_down;

  int fail(int code, const std::string& msg) {
    err = msg;
    return code;
  }
  template <typename T>
  bool alloc(T** out, size_t count) {
    void* p = nullptr;
    if (count == 0) count = 1;
    if (hipMalloc(&p, count * sizeof(T)) != hipSuccess) return false;
    allocs.push_back(p);
    *out = static_cast<T*>(p);
    return true;
  }
  ~dg_ctx() {
    for (auto& r : recs) {
      (void)hipEventDestroy(r.a);
      (void)hipEventDestroy(r.b);
    }
    for (hipEvent_t e : pool) (void)hipEventDestroy(e);
    for (void* p : allocs) (void)hipFree(p);
  }
};

namespace {

constexpr int kMaxSplit = 16;
constexpr long kGemmPartFloats = 8L << 20;  // 32 MB of split-K partial slices
constexpr int kHeadSlice = 64;  // vocab entries per head partial (half the 128-wide tile)

// Run `launch` (one or more kernel launches on stream s); with timing on, bracket it by events.
template <typename F>
void timed(dg_ctx* c, const char* name, hipStream_t s, F&& launch) {
  if (!c->timing) {
    launch();
    return;
  }
  hipEvent_t a = c->event(), b = c->event();
  (void)hipEventRecord(a, s);
  launch();
  (void)hipEventRecord(b, s);
  c->recs.push_back({name, a, b});
}

long kv_layer_stride(const dg_model_desc& m, int n_slots, int cap) {
  return static_cast<long>(n_slots) * m.n_kv_heads * cap * m.head_dim;
}
int kv_slots(const dg_kv_cache* kv) { return kv->n_slots > 0 ? kv->n_slots : kv->batch; }
int kv_slot(const dg_kv_cache* kv, int b) { return kv->slot ? kv->slot[b] : b; }
bool kv_identity(const dg_kv_cache* kv) {
  if (!kv->slot) return true;
  for (int b = 0; b < kv->batch; ++b)
    if (kv->slot[b] != b) return false;
  return true;
}

int check_hip(dg_ctx* c, const char* where) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    return c->fail(DG_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
  }
  return DG_OK;
}

std::string validate_desc(const dg_model_desc& m) {
  char buf[256];
  auto bad = [&](const char* what) {
    snprintf(buf, sizeof buf, "unsupported model shape: %s", what);
    return std::string(buf);
  };
  if (m.n_layers < 1) return bad("n_layers < 1");
  if (m.head_dim != 64 && m.head_dim != 128) return bad("head_dim must be 64 or 128");
  if (m.n_q_heads < 1 || m.n_kv_heads < 1 || m.n_q_heads % m.n_kv_heads) return bad("n_q_heads % n_kv_heads");
  if (m.d_model < 128 || m.d_model % 128 || m.d_model > 8192) return bad("d_model: multiple of 128, <= 8192");
  if ((m.n_q_heads * m.head_dim) % 64) return bad("n_q_heads*head_dim % 64");
  if (m.n_experts < 1 || m.n_experts > 64) return bad("n_experts in [1, 64]");
  if (m.top_k < 1 || m.top_k > m.n_experts) return bad("top_k in [1, n_experts]");
  if (m.d_ff_expert < 128 || m.d_ff_expert % 128 || m.d_ff_expert > 1024)
    return bad("d_ff_expert: multiple of 128, <= 1024");
  if (m.d_ff_shared < 0 || m.d_ff_shared % 64) return bad("d_ff_shared % 64");
  if (m.vocab < 128 || m.vocab % 128 || m.vocab > 131072) return bad("vocab: multiple of 128, <= 131072");
  if (m.canvas != 256) return bad("canvas must be 256");
  if (!(m.rms_eps > 0.f) || !(m.rope_theta >= 0.f)) return bad("rms_eps > 0, rope_theta >= 0");
  if (m.expert_fp8 != 0 && m.expert_fp8 != 1) return bad("expert_fp8 must be 0 or 1");
  return "";
}

RowMap make_map(int rows_per_req, int n_req, const int32_t* pos0, const dg_kv_cache* kv = nullptr) {
  RowMap r{};
  r.rows_per_req = rows_per_req;
  r.n_req = n_req;
  for (int b = 0; b < n_req; ++b) {
    r.pos0[b] = pos0 ? pos0[b] : 0;
    r.slot[b] = kv ? kv_slot(kv, b) : b;
  }
  return r;
}

int choose_split(const dg_ctx* c, int base_wgs, int n_keys, int rows, int waves) {
  // two waves per SIMD (two 4-wave or one 8-wave work-group per CU), each split keeping at
  // least four 64-key blocks
  const int target = 256 * (8 / waves);
  int ns = std::max(1, std::min(kMaxSplit, (target + base_wgs - 1) / base_wgs));
  ns = std::min(ns, std::max(1, n_keys / 256));
  ns = std::min(ns, std::max(1, c->part_cap / std::max(1, rows * c->m.n_q_heads)));
  return ns;
}

// Per-request splits for the pipelined canvas attention: about two work-groups per CU in all,
// the splits handed out one at a time to the request whose splits are then longest (each split
// keeps at least 256 keys), split lengths rounded up to 64-key blocks.  The (request, split)
// pairs are listed longest first: the dispatcher gives each CU its next work-group as the CU
// frees up, so the CUs that ran the longest ranges first take the shortest ones last.
void plan_pipe_splits(const dg_ctx* c, AttnArgs& at, int rows) {
  constexpr int kCUs = 256;
  const int n_req = at.n_req, Hkv = at.Hkv;
  const int group = at.Hq / Hkv, n_rb = (at.rows_per_req + 31) / 32;
  const int per_pair = (group * n_rb + 7) / 8 * Hkv;  // work-groups of one (request, split)
  const int cap = std::max(1, std::min(kMaxSplit, c->part_cap / std::max(1, rows * at.Hq)));
  int keys[kMaxBatch], ns[kMaxBatch];
  for (int b = 0; b < n_req; ++b) {
    keys[b] = at.n_cache[b] + at.n_extra;
    ns[b] = 1;
  }
  const int want = std::min(kMaxPairs, std::max(n_req, (2 * kCUs + per_pair - 1) / per_pair));
  for (int p = n_req; p < want; ++p) {
    int best = -1;
    long best_num = 0, best_den = 1;  // longest keys[b] / ns[b], compared exactly
    for (int b = 0; b < n_req; ++b) {
      if (ns[b] >= cap || keys[b] / (ns[b] + 1) < 256) continue;
      if (best < 0 || static_cast<long>(keys[b]) * best_den > best_num * ns[b]) {
        best = b;
        best_num = keys[b];
        best_den = ns[b];
      }
    }
    if (best < 0) break;
    ++ns[best];
  }
  struct Pair { int len, b, s; };
  Pair pairs[kMaxPairs];
  int n_pairs = 0, stride = 1;
  for (int b = 0; b < n_req; ++b) {
    const int sk = ((keys[b] + ns[b] - 1) / ns[b] + 63) / 64 * 64;
    ns[b] = (keys[b] + sk - 1) / sk;
    at.req_split[b] = ns[b];
    at.req_split_keys[b] = sk;
    stride = std::max(stride, ns[b]);
    for (int sp = 0; sp < ns[b]; ++sp) pairs[n_pairs++] = Pair{std::min(sk, keys[b] - sp * sk), b, sp};
  }
  std::stable_sort(pairs, pairs + n_pairs, [](const Pair& x, const Pair& y) { return x.len > y.len; });
  at.n_pairs = n_pairs;
  for (int i = 0; i < n_pairs; ++i) at.pair[i] = static_cast<uint16_t>((pairs[i].b << 8) | pairs[i].s);
  at.n_split = stride;
  at.split_keys = 0;
  at.balanced = 1;
}

// One decoder layer over `rows` rows (n_req requests of rows_per_req rows each).
// Denoise mode: K/V of the rows go to the canvas scratch; keys = cache[0:len) + canvas.
// Prefill mode (one request): K/V go to the cache at len..; keys = cache[0:len+rows), causal.
void run_layer(dg_ctx* c, int l, int n_req, int rows_per_req, const int32_t* len, bool prefill,
               uint16_t* kc_l, uint16_t* vc_l, int cap, const dg_debug* dbg, const float* next_gain,
               uint16_t* next_out, hipStream_t s, const dg_kv_cache* kv_slots_of = nullptr) {
  const dg_model_desc& m = c->m;
  const dg_layer_weights& lw = c->layers[l];
  const int rows = n_req * rows_per_req;
  const int d = m.d_model, Hq = m.n_q_heads, Hkv = m.n_kv_heads, D = m.head_dim;
  const int nqkv = (Hq + 2 * Hkv) * D;
  const RowMap map = make_map(rows_per_req, n_req, len);

  // c->a holds this layer's normed input (written by the embedding or the previous combine).
  // QKV projection with RoPE and the scatter of Q, K, V fused into its epilogue.
  GemmArgs g{};
  g.x = c->a; g.ldx = d; g.n_tok = rows;
  g.w0 = c->wqkv[l]; g.K = d; g.N = nqkv; g.split = 1;
  RopeArgs& ra = g.rope;
  ra.Hq = Hq; ra.Hkv = Hkv; ra.D = D;
  ra.table = m.rope_theta != 0.f ? c->rope : nullptr;  // filled by the caller for these rows
  ra.q = c->q; ra.map = map;
  const long ck_layer = static_cast<long>(l) * c->max_batch * Hkv * m.canvas * D;
  if (prefill) {
    ra.k_dst = kc_l; ra.v_dst = vc_l; ra.kv_cap = cap;
    for (int b = 0; b < n_req; ++b) ra.slot0[b] = len[b];
  } else {
    ra.k_dst = c->ck + ck_layer; ra.v_dst = c->cv + ck_layer; ra.kv_cap = m.canvas;
    for (int b = 0; b < n_req; ++b) ra.slot0[b] = 0;
  }
  timed(c, "gemm_qkv_rope", s, [&] { launch_gemm(g, EPI_ROPE_QKV, s); });

  AttnArgs at{};
  at.q = c->q; at.out = c->attn; at.kc = kc_l; at.vc = vc_l; at.cap = cap;
  at.kx = c->ck + ck_layer; at.vx = c->cv + ck_layer; at.xcap = m.canvas;
  at.Hq = Hq; at.Hkv = Hkv; at.D = D; at.rows_per_req = rows_per_req; at.n_req = n_req;
  int max_keys = 0;
  for (int b = 0; b < n_req; ++b) {
    at.n_cache[b] = prefill ? len[b] + rows_per_req : len[b];
    at.q_pos0[b] = len[b];
    at.slot[b] = kv_slots_of ? kv_slot(kv_slots_of, b) : b;
    max_keys = std::max(max_keys, at.n_cache[b] + (prefill ? 0 : m.canvas));
  }
  at.n_extra = prefill ? 0 : m.canvas;
  at.causal = prefill ? 1 : 0;
  at.scale = 1.0f / std::sqrt(static_cast<float>(D));
  at.q_tiles = attention_q_tiles(max_keys, prefill);
  const int tasks = (Hq / Hkv) * ((rows_per_req + 16 * at.q_tiles - 1) / (16 * at.q_tiles));
  at.n_waves = attention_waves(max_keys, prefill);
  if (attention_pipe_path(at)) {
    plan_pipe_splits(c, at, rows);
  } else {
    const int base = ((tasks + at.n_waves - 1) / at.n_waves) * n_req * Hkv;
    at.n_split = choose_split(c, base, max_keys, rows, at.n_waves);
    at.split_keys = (((max_keys + at.n_split - 1) / at.n_split + 63) / 64) * 64;
    at.n_split = (max_keys + at.split_keys - 1) / at.split_keys;
  }
  at.part_o = c->part_o; at.part_ml = c->part_ml;
  timed(c, "attention", s, [&] { launch_attention(at, s); });
  if (at.n_split > 1) timed(c, "attn_split_combine", s, [&] { launch_attention_combine(at, s); });
  if (dbg && dbg->attn_out)
    (void)hipMemcpyAsync(dbg->attn_out + static_cast<long>(l) * rows * Hq * D, c->attn,
                         sizeof(uint16_t) * rows * Hq * D, hipMemcpyDeviceToDevice, s);

  GemmArgs go{};
  go.part = c->gpart;
  go.x = c->attn; go.ldx = Hq * D; go.n_tok = rows; go.w0 = lw.wo; go.K = Hq * D; go.N = d;
  go.out_f32 = c->h; go.ldo = d;
  go.split = gemm_split(go, EPI_ADD_F32, kGemmPartFloats);
  go.part_stride = static_cast<long>(rows) * d;
  timed(c, "gemm_o_residual", s, [&] { launch_gemm(go, EPI_ADD_F32, s); });

  // (the attention-output residual lands here when the O-projection was split: h += slices)
  timed(c, "norm_router_topk", s, [&] {
    launch_norm_router(c->h, c->gpart, go.split > 1 ? go.split : 0, go.part_stride, lw.ffn_norm,
                       m.rms_eps, lw.w_router, c->wr_pk.empty() ? nullptr : c->wr_pk[l], rows, d,
                       m.n_experts, m.top_k, c->a, c->eidx, c->gates, s);
  });
  if (dbg && dbg->h_mid)
    (void)hipMemcpyAsync(dbg->h_mid + static_cast<long>(l) * rows * d, c->h,
                         sizeof(float) * rows * d, hipMemcpyDeviceToDevice, s);
  if (dbg && dbg->expert_idx)
    (void)hipMemcpyAsync(dbg->expert_idx + static_cast<long>(l) * rows * m.top_k, c->eidx,
                         sizeof(int32_t) * rows * m.top_k, hipMemcpyDeviceToDevice, s);
  if (dbg && dbg->gates)
    (void)hipMemcpyAsync(dbg->gates + static_cast<long>(l) * rows * m.top_k, c->gates,
                         sizeof(float) * rows * m.top_k, hipMemcpyDeviceToDevice, s);

  const int routes = rows * m.top_k;
  // up to kFusedRoutes routes the gate/up GEMM ranks its own expert's routes (one launch less);
  // beyond that a separate permutation pass does
  const bool fused_rank = routes <= kFusedRoutes;
  if (!fused_rank)
    timed(c, "moe_permute", s, [&] { launch_moe_permute(c->eidx, routes, m.n_experts, c->offs, c->perm, c->inv, s); });
  MoeArgs g1{};
  g1.x = c->a; g1.ldx = d; g1.perm = c->perm; g1.top_k = m.top_k; g1.offs = c->offs;
  if (fused_rank) {
    g1.idx = c->eidx; g1.n_routes = routes;
    g1.offs_w = c->offs; g1.perm_w = c->perm; g1.inv_w = c->inv;
  }
  g1.wp = c->pk1[l]; g1.K = d; g1.N = m.d_ff_expert;
  if (m.expert_fp8) { g1.wp8 = c->pk1_8[l]; g1.wscale0 = c->sc_gate[l]; g1.wscale1 = c->sc_up[l]; }
  g1.out_bf16 = c->act; g1.ldo = m.d_ff_expert; g1.n_exp = m.n_experts;
  timed(c, "moe_gemm1_swiglu", s, [&] { launch_moe_gemm1(g1, routes / m.n_experts, s); });
  // the route tables are complete once the gate/up GEMM has run (it writes them when it ranks)
  if (dbg && dbg->route_offs)
    (void)hipMemcpyAsync(dbg->route_offs + static_cast<long>(l) * (m.n_experts + 1), c->offs,
                         sizeof(int32_t) * (m.n_experts + 1), hipMemcpyDeviceToDevice, s);
  if (dbg && dbg->route_perm)
    (void)hipMemcpyAsync(dbg->route_perm + static_cast<long>(l) * routes, c->perm, sizeof(int32_t) * routes,
                         hipMemcpyDeviceToDevice, s);
  if (dbg && dbg->route_inv)
    (void)hipMemcpyAsync(dbg->route_inv + static_cast<long>(l) * routes, c->inv, sizeof(int32_t) * routes,
                         hipMemcpyDeviceToDevice, s);
  MoeArgs g2{};
  g2.x = c->act; g2.ldx = m.d_ff_expert; g2.perm = c->perm; g2.top_k = m.top_k; g2.offs = c->offs;
  g2.wp = c->pk2[l]; g2.K = m.d_ff_expert; g2.N = d; g2.out_bf16 = c->y; g2.ldo = d;
  if (m.expert_fp8) { g2.wp8 = c->pk2_8[l]; g2.wscale0 = c->sc_down[l]; }
  g2.n_exp = m.n_experts;
  timed(c, "moe_gemm2", s, [&] { launch_moe_gemm2(g2, routes / m.n_experts, s); });

  int n_res = 0;  // split-K slices of the shared down projection, added by the combine
  if (m.d_ff_shared > 0) {
    GemmArgs gs{};
    gs.part = c->gpart;
    gs.x = c->a; gs.ldx = d; gs.n_tok = rows; gs.w0 = lw.ws_gate; gs.w1 = lw.ws_up; gs.K = d;
    gs.N = m.d_ff_shared; gs.out_bf16 = c->sact; gs.ldo = m.d_ff_shared;
    gs.split = gemm_split(gs, EPI_SWIGLU_BF16, kGemmPartFloats);
    gs.part_stride = 2L * rows * m.d_ff_shared;
    timed(c, "shared_gate_up_swiglu", s, [&] {
      launch_gemm(gs, EPI_SWIGLU_BF16, s);
      if (gs.split > 1) launch_swiglu_reduce(c->gpart, gs.part_stride, gs.split, c->sact, rows, m.d_ff_shared, s);
    });
    GemmArgs gd{};
    gd.part = c->gpart;
    gd.x = c->sact; gd.ldx = m.d_ff_shared; gd.n_tok = rows; gd.w0 = lw.ws_down;
    gd.K = m.d_ff_shared; gd.N = d; gd.out_f32 = c->h; gd.ldo = d;
    gd.split = gemm_split(gd, EPI_ADD_F32, kGemmPartFloats);
    gd.part_stride = static_cast<long>(rows) * d;
    n_res = gd.split > 1 ? gd.split : 0;
    timed(c, "shared_down_residual", s, [&] { launch_gemm(gd, EPI_ADD_F32, s); });
  }
  timed(c, "moe_combine", s, [&] {
    launch_moe_combine(c->h, c->gpart, n_res, static_cast<long>(rows) * d, c->y, c->inv, c->gates, rows,
                       d, m.top_k, next_gain, m.rms_eps, next_out, s);
  });
  if (dbg && dbg->layer_out)
    (void)hipMemcpyAsync(dbg->layer_out + static_cast<long>(l) * rows * d, c->h,
                         sizeof(float) * rows * d, hipMemcpyDeviceToDevice, s);
}

int check_kv(dg_ctx* c, const dg_kv_cache* kv) {
  if (!kv || !kv->k || !kv->v || !kv->len) return c->fail(DG_ERR_ARG, "kv cache: null pointer");
  if (kv->batch < 1 || kv->batch > c->max_batch)
    return c->fail(DG_ERR_CAPACITY, "kv->batch must be in [1, max_batch]");
  if (kv->cap < 1) return c->fail(DG_ERR_ARG, "kv->cap < 1");
  if (kv->n_slots < 0 || (kv->n_slots > 0 && kv->n_slots < kv->batch))
    return c->fail(DG_ERR_ARG, "kv->n_slots must be 0 or >= batch");
  if (kv->slot) {
    const int ns = kv_slots(kv);
    for (int b = 0; b < kv->batch; ++b) {
      if (kv->slot[b] < 0 || kv->slot[b] >= ns) return c->fail(DG_ERR_ARG, "kv->slot out of [0, n_slots)");
      for (int e = 0; e < b; ++e)
        if (kv->slot[e] == kv->slot[b]) return c->fail(DG_ERR_ARG, "kv->slot entries must be distinct");
    }
  }
  for (int b = 0; b < kv->batch; ++b)
    if (kv->len[b] < 0 || kv->len[b] > kv->cap) return c->fail(DG_ERR_ARG, "kv->len out of [0, cap]");
  return DG_OK;
}

}  // namespace

extern "C" {

int dg_create(const dg_model_desc* desc, const dg_weights* weights, int32_t max_batch,
              int32_t max_prefill_rows, dg_ctx** out) {
  g_create_error.clear();
  if (!desc || !weights || !out) { g_create_error = "dg_create: null argument"; return DG_ERR_ARG; }
  *out = nullptr;
  const std::string bad = validate_desc(*desc);
  if (!bad.empty()) { g_create_error = bad; return DG_ERR_SHAPE; }
  if (max_batch < 1 || max_batch > kMaxBatch) {
    g_create_error = "max_batch must be in [1, 64]";
    return DG_ERR_ARG;
  }
  if (max_prefill_rows < 1 || max_prefill_rows > (1 << 16)) {
    g_create_error = "max_prefill_rows must be in [1, 65536]";
    return DG_ERR_ARG;
  }
  if (!weights->embed || !weights->final_norm || !weights->lm_head || !weights->layers) {
    g_create_error = "dg_create: null weight pointer";
    return DG_ERR_ARG;
  }
  for (int l = 0; l < desc->n_layers; ++l) {
    const dg_layer_weights& lw = weights->layers[l];
    if (!lw.attn_norm || !lw.wq || !lw.wk || !lw.wv || !lw.wo || !lw.ffn_norm || !lw.w_router ||
        !lw.w_gate || !lw.w_up || !lw.w_down ||
        (desc->d_ff_shared > 0 && (!lw.ws_gate || !lw.ws_up || !lw.ws_down))) {
      g_create_error = "dg_create: null weight pointer in layer " + std::to_string(l);
      return DG_ERR_ARG;
    }
  }
  dg_ctx* c = new (std::nothrow) dg_ctx();
  if (!c) { g_create_error = "out of host memory"; return DG_ERR_ARG; }
  c->m = *desc;
  c->w = *weights;
  c->layers.assign(weights->layers, weights->layers + desc->n_layers);
  c->w.layers = nullptr;
  c->max_batch = max_batch;
  c->max_prefill = max_prefill_rows;
  c->r_canvas = max_batch * desc->canvas;
  c->r_max = std::max(c->r_canvas, max_prefill_rows);
  // split partials for every row a call can hold (canvas rows or a prefill chunk), up to 4
  // splits per row at the largest count (the per-request plan asks for about two work-groups
  // per CU), 16 below
  c->part_cap = std::max(c->r_canvas * kMaxSplit, c->r_max * 4) * desc->n_q_heads;
  const dg_model_desc& m = c->m;
  const long R = c->r_max, d = m.d_model, HD = m.n_q_heads * m.head_dim;
  const long nqkv = (m.n_q_heads + 2L * m.n_kv_heads) * m.head_dim;
  const long ckv = static_cast<long>(m.n_layers) * max_batch * m.n_kv_heads * m.canvas * m.head_dim;
  bool ok = c->alloc(&c->h, R * d) && c->alloc(&c->a, R * d) && 
            c->alloc(&c->q, R * HD) && c->alloc(&c->attn, R * HD) &&
            c->alloc(&c->part_o, static_cast<long>(c->part_cap) * m.head_dim) &&
            c->alloc(&c->part_ml, static_cast<long>(c->part_cap) * 2) &&
            c->alloc(&c->eidx, R * m.top_k) && c->alloc(&c->gates, R * m.top_k) &&
            c->alloc(&c->offs, m.n_experts + 1) && c->alloc(&c->perm, R * m.top_k) &&
            c->alloc(&c->inv, R * m.top_k) && c->alloc(&c->act, R * m.top_k * m.d_ff_expert) &&
            c->alloc(&c->y, R * m.top_k * d) &&
            c->alloc(&c->sact, R * std::max(1, m.d_ff_shared)) &&
            c->alloc(&c->f, static_cast<long>(c->r_canvas) * d) &&
            c->alloc(&c->head_part, static_cast<long>(c->r_canvas) * (m.vocab / kHeadSlice) * 8) &&
            c->alloc(&c->ck, ckv) && c->alloc(&c->cv, ckv) &&
            c->alloc(&c->gpart, kGemmPartFloats) &&
            c->alloc(&c->rope, R * m.head_dim) && c->alloc(&c->tok, c->r_canvas) &&
            c->alloc(&c->dev_err, 1) && hipMemset(c->dev_err, 0, sizeof(uint32_t)) == hipSuccess;
  // expert banks, repacked once into the MFMA fragment order the expert GEMMs stream
  const long ew = static_cast<long>(m.n_experts) * m.d_ff_expert * m.d_model;
  const int E = m.n_experts, F = m.d_ff_expert;
  c->pk1.assign(m.n_layers, nullptr);
  c->pk2.assign(m.n_layers, nullptr);
  if (m.expert_fp8) {
    // quantize each matrix row-wise into scratch bytes, then lay the bytes out for streaming
    c->pk1_8.assign(m.n_layers, nullptr);
    c->pk2_8.assign(m.n_layers, nullptr);
    c->sc_gate.assign(m.n_layers, nullptr);
    c->sc_up.assign(m.n_layers, nullptr);
    c->sc_down.assign(m.n_layers, nullptr);
    uint8_t *qg = nullptr, *qu = nullptr, *qd = nullptr;
    ok = ok && hipMalloc(&qg, ew) == hipSuccess && hipMalloc(&qu, ew) == hipSuccess &&
         hipMalloc(&qd, ew) == hipSuccess;
    for (int l = 0; ok && l < m.n_layers; ++l) {
      ok = c->alloc(&c->pk1_8[l], 2 * ew) && c->alloc(&c->pk2_8[l], ew) &&
           c->alloc(&c->sc_gate[l], static_cast<long>(E) * F) && c->alloc(&c->sc_up[l], static_cast<long>(E) * F) &&
           c->alloc(&c->sc_down[l], static_cast<long>(E) * d);
      if (!ok) break;
      const dg_layer_weights& lw = c->layers[l];
      launch_quantize_e4m3(lw.w_gate, static_cast<long>(E) * F, static_cast<int>(d), qg, c->sc_gate[l], nullptr);
      launch_quantize_e4m3(lw.w_up, static_cast<long>(E) * F, static_cast<int>(d), qu, c->sc_up[l], nullptr);
      launch_quantize_e4m3(lw.w_down, static_cast<long>(E) * d, F, qd, c->sc_down[l], nullptr);
      launch_moe_pack_fp8(qg, qu, c->pk1_8[l], E, F, static_cast<int>(d), kGroupTiles1, nullptr);
      launch_moe_pack_fp8(qd, nullptr, c->pk2_8[l], E, static_cast<int>(d), F, kGroupTiles2, nullptr);
      ok = hipDeviceSynchronize() == hipSuccess;  // the scratch bytes are reused by the next layer
    }
    if (qg) (void)hipFree(qg);
    if (qu) (void)hipFree(qu);
    if (qd) (void)hipFree(qd);
  } else {
    for (int l = 0; ok && l < m.n_layers; ++l) {
      ok = c->alloc(&c->pk1[l], 2 * ew) && c->alloc(&c->pk2[l], ew);
      if (!ok) break;
      const dg_layer_weights& lw = c->layers[l];
      launch_moe_pack(lw.w_gate, lw.w_up, c->pk1[l], E, F, m.d_model, kGroupTiles1, nullptr);
      launch_moe_pack(lw.w_down, nullptr, c->pk2[l], E, m.d_model, F, kGroupTiles2, nullptr);
    }
  }
  // router weights, repacked once into the fragment order of the MFMA router
  if (router_mfma_path(m.d_model, m.n_experts)) {
    c->wr_pk.assign(m.n_layers, nullptr);
    for (int l = 0; ok && l < m.n_layers; ++l) {
      ok = c->alloc(&c->wr_pk[l], 64L * m.d_model);
      if (ok) launch_router_pack(c->layers[l].w_router, m.n_experts, m.d_model, c->wr_pk[l], nullptr);
    }
  }
  c->wqkv.assign(m.n_layers, nullptr);
  for (int l = 0; ok && l < m.n_layers; ++l) {
    ok = c->alloc(&c->wqkv[l], static_cast<long>(nqkv) * m.d_model);
    if (ok) {
      const dg_layer_weights& lw = c->layers[l];
      launch_pack_qkv(lw.wq, lw.wk, lw.wv, c->wqkv[l], m.n_q_heads, m.n_kv_heads, m.head_dim, m.d_model, nullptr);
    }
  }
  if (ok) ok = hipDeviceSynchronize() == hipSuccess && hipGetLastError() == hipSuccess;
  // the static scratch of the allocation-free head call, looked up on this (current) device
  if (ok && scratch_address(&c->static_scratch) != hipSuccess) {
    g_create_error = "dg_create: hipGetSymbolAddress of the static scratch failed";
    delete c;
    return DG_ERR_HIP;
  }
  if (!ok) {
    g_create_error = "workspace allocation or weight packing failed";
    delete c;
    return DG_ERR_HIP;
  }
  *out = c;
  return DG_OK;
}

void dg_destroy(dg_ctx* ctx) { delete ctx; }

const char* dg_last_error(const dg_ctx* ctx) {
  return ctx ? ctx->err.c_str() : g_create_error.c_str();
}

float dg_temperature(const dg_sampler_cfg* cfg, int32_t step) {
  if (!cfg) return 0.f;
  if (cfg->max_steps <= 1) return cfg->temp_start;
  const double t = static_cast<double>(cfg->temp_start) +
                   (static_cast<double>(cfg->temp_end) - static_cast<double>(cfg->temp_start)) *
                       step / (cfg->max_steps - 1);
  return static_cast<float>(t);
}

int dg_quantize_e4m3_rows(const uint16_t* w, int64_t rows, int32_t cols, uint8_t* q, float* scale,
                          hipStream_t s) {
  if (!w || !q || !scale) { g_create_error = "dg_quantize_e4m3_rows: null pointer"; return DG_ERR_ARG; }
  if (rows < 0 || rows > (int64_t(1) << 31) - 1 || cols < 1 || cols > 65536) {
    g_create_error = "dg_quantize_e4m3_rows: rows in [0, 2^31), cols in [1, 65536]";
    return DG_ERR_ARG;
  }
  launch_quantize_e4m3(w, static_cast<long>(rows), cols, q, scale, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) { g_create_error = hipGetErrorString(e); return DG_ERR_HIP; }
  return DG_OK;
}

int dg_prefill_causal(dg_ctx* c, const int32_t* tokens, const int32_t* n_new, int32_t batch,
                      dg_kv_cache* kv, hipStream_t s) {
  if (!c) return DG_ERR_ARG;
  if (!tokens || !n_new) return c->fail(DG_ERR_ARG, "prefill: null pointer");
  int rc = check_kv(c, kv);
  if (rc) return rc;
  if (batch != kv->batch) return c->fail(DG_ERR_ARG, "prefill: batch != kv->batch");
  for (int b = 0; b < batch; ++b) {
    if (n_new[b] < 0) return c->fail(DG_ERR_ARG, "prefill: n_new < 0");
    if (static_cast<long>(kv->len[b]) + n_new[b] > kv->cap)
      return c->fail(DG_ERR_CAPACITY, "prefill: len + n_new > cap");
  }
  const dg_model_desc& m = c->m;
  long tok_ofs = 0;
  for (int b = 0; b < batch; ++b) {
    for (int done = 0; done < n_new[b];) {
      const int n = std::min(c->max_prefill, n_new[b] - done);
      launch_embed(tokens + tok_ofs + done, c->w.embed, c->h, n, m.d_model, m.vocab, c->dev_err,
                   c->layers[0].attn_norm, m.rms_eps, c->a, s);
      const int32_t len_b = kv->len[b] + done;
      if (m.rope_theta != 0.f) launch_rope_table(make_map(n, 1, &len_b), n, m.head_dim, m.rope_theta, c->rope, s);
      for (int l = 0; l < m.n_layers; ++l) {
        const long base = l * kv_layer_stride(m, kv_slots(kv), kv->cap) +
                          static_cast<long>(kv_slot(kv, b)) * m.n_kv_heads * kv->cap * m.head_dim;
        const float* ng = (l + 1 < m.n_layers) ? c->layers[l + 1].attn_norm : nullptr;
        run_layer(c, l, 1, n, &len_b, true, kv->k + base, kv->v + base, kv->cap, nullptr, ng, c->a, s);
      }
      done += n;
    }
    tok_ofs += n_new[b];
  }
  rc = check_hip(c, "prefill");
  if (rc) return rc;
  for (int b = 0; b < batch; ++b) kv->len[b] += n_new[b];
  return DG_OK;
}

int dg_canvas_init(dg_ctx* c, dg_canvas_state* st, const dg_kv_cache* kv,
                   const dg_sampler_cfg* cfg, hipStream_t s) {
  if (!c) return DG_ERR_ARG;
  if (!st || !st->tokens || !st->committed || !st->stable_run || !st->stopped || !cfg)
    return c->fail(DG_ERR_ARG, "canvas_init: null pointer");
  int rc = check_kv(c, kv);
  if (rc) return rc;
  const RowMap map = make_map(c->m.canvas, kv->batch, kv->len, kv);
  launch_canvas_init(st->tokens, st->committed, st->stable_run, st->stopped, c->m.canvas, c->m.vocab,
                     static_cast<uint32_t>(cfg->seed), static_cast<uint32_t>(cfg->seed >> 32), map, s);
  return check_hip(c, "canvas_init");
}

// Vocab projection + row statistics of `rows` normed final states f, with the per-(row, 64-entry
// slice) partial statistics in `part` ([rows][vocab / 64][8] floats, every entry written by the
// head kernel before the merge reads it, so nothing needs clearing).
static void run_head(dg_ctx* c, const uint16_t* f, const int32_t* canvas, const dg_kv_cache* kv,
                     const dg_sampler_cfg* cfg, const dg_step_params* p, dg_row_stats* out, float* part,
                     bool time_it, hipStream_t s) {
  const dg_model_desc& m = c->m;
  const int B = kv->batch, C = m.canvas, rows = B * C;
  const dg_debug* dbg = p ? p->debug : nullptr;
  HeadArgs ha{};
  ha.f = f; ha.n_rows = rows; ha.w = c->w.lm_head; ha.K = m.d_model; ha.V = m.vocab;
  ha.k0 = static_cast<uint32_t>(cfg->seed); ha.k1 = static_cast<uint32_t>(cfg->seed >> 32);
  for (int b = 0; b < B; ++b) {
    ha.step[b] = (p && p->steps) ? p->steps[b] : (p ? p->step : 0);
    ha.temp[b] = dg_temperature(cfg, ha.step[b]);
  }
  ha.cur_tok = canvas;
  ha.map = make_map(C, B, kv->len, kv);
  ha.part = part;
  ha.dbg_logits = dbg ? dbg->logits : nullptr;
  auto merge = [&] {
    launch_head_merge(part, rows, m.vocab / kHeadSlice, kHeadSlice, canvas, c->dev_err, out->cand, out->t_cand,
                      out->t_cur, out->lse, out->entropy, ha.map, s);
  };
  if (time_it) {
    timed(c, "head_lse_gumbel", s, [&] { launch_head(ha, s); });
    timed(c, "head_merge", s, merge);
  } else {
    launch_head(ha, s);
    merge();
  }
}

static int denoise_impl(dg_ctx* c, const int32_t* canvas, const dg_kv_cache* kv,
                        const dg_sampler_cfg* cfg, const dg_step_params* p, dg_row_stats* out,
                        hipStream_t s) {
  const dg_model_desc& m = c->m;
  const int B = kv->batch, C = m.canvas, rows = B * C, d = m.d_model;
  const uint32_t flags = p ? p->flags : 0u;
  const dg_debug* dbg = p ? p->debug : nullptr;
  const bool head_only = flags & DG_STEP_HEAD_ONLY;
  const bool no_head = flags & DG_STEP_NO_HEAD;
  if (canvas && !kv_identity(kv)) {  // the rows of this call, in call order
    launch_gather_rows(canvas, c->tok, make_map(C, B, kv->len, kv), s);
    canvas = c->tok;
  }

  if (!head_only) {
    if (flags & DG_STEP_HIDDEN_IN) {
      (void)hipMemcpyAsync(c->h, p->hidden_in, sizeof(float) * rows * d, hipMemcpyDeviceToDevice, s);
      launch_rmsnorm(c->h, c->layers[0].attn_norm, m.rms_eps, c->a, rows, d, s);
    } else {
      timed(c, "embed_norm", s, [&] {
        launch_embed(canvas, c->w.embed, c->h, rows, d, m.vocab, c->dev_err, c->layers[0].attn_norm,
                     m.rms_eps, c->a, s);
      });
    }
    if (m.rope_theta != 0.f)
      timed(c, "rope_table", s, [&] {
        launch_rope_table(make_map(C, B, kv->len), rows, m.head_dim, m.rope_theta, c->rope, s);
      });
    // each layer's combine also norms the next layer's input; the last one the head's input
    for (int l = 0; l < m.n_layers; ++l) {
      const bool last = l + 1 == m.n_layers;
      const float* ng = !last ? c->layers[l + 1].attn_norm : (no_head ? nullptr : c->w.final_norm);
      run_layer(c, l, B, C, kv->len, false, kv->k + l * kv_layer_stride(m, kv_slots(kv), kv->cap),
                kv->v + l * kv_layer_stride(m, kv_slots(kv), kv->cap), kv->cap, dbg, ng,
                last ? c->f : c->a, s, kv);
    }
    c->last_slots.resize(B);
    for (int b = 0; b < B; ++b) c->last_slots[b] = kv_slot(kv, b);
    if (dbg && dbg->hidden_out)
      (void)hipMemcpyAsync(dbg->hidden_out, c->h, sizeof(float) * rows * d, hipMemcpyDeviceToDevice, s);
    if (dbg && (dbg->canvas_k || dbg->canvas_v)) {
      // workspace canvas K/V is [L][max_batch][Hkv][C][D]; dump [L][B][Hkv][C][D]
      const long per_b = static_cast<long>(m.n_kv_heads) * C * m.head_dim;
      for (int l = 0; l < m.n_layers; ++l) {
        const long src = static_cast<long>(l) * c->max_batch * per_b, dst = static_cast<long>(l) * B * per_b;
        if (dbg->canvas_k)
          (void)hipMemcpyAsync(dbg->canvas_k + dst, c->ck + src, 2 * B * per_b, hipMemcpyDeviceToDevice, s);
        if (dbg->canvas_v)
          (void)hipMemcpyAsync(dbg->canvas_v + dst, c->cv + src, 2 * B * per_b, hipMemcpyDeviceToDevice, s);
      }
    }
  }
  if (no_head) return DG_OK;
  // the final norm was fused into the last layer's combine
  const uint16_t* f = head_only ? static_cast<const uint16_t*>(p->hidden_in) : c->f;
  run_head(c, f, canvas, kv, cfg, p, out, c->head_part, true, s);
  return DG_OK;
}

// Argument checks shared by dg_denoise_step and its allocation-free head variant.
static int check_step_args(dg_ctx* c, const int32_t* canvas, const dg_kv_cache* kv,
                           const dg_sampler_cfg* cfg, const dg_step_params* p,
                           const dg_row_stats* out) {
  int rc = check_kv(c, kv);
  if (rc) return rc;
  const uint32_t flags = p ? p->flags : 0u;
  if (flags & ~(DG_STEP_HIDDEN_IN | DG_STEP_NO_HEAD | DG_STEP_HEAD_ONLY))
    return c->fail(DG_ERR_UNSUPPORTED, "denoise: unknown flag");
  if ((flags & DG_STEP_HEAD_ONLY) && (flags & (DG_STEP_NO_HEAD | DG_STEP_HIDDEN_IN)))
    return c->fail(DG_ERR_UNSUPPORTED, "denoise: HEAD_ONLY excludes NO_HEAD and HIDDEN_IN");
  if ((flags & (DG_STEP_HIDDEN_IN | DG_STEP_HEAD_ONLY)) && !p->hidden_in)
    return c->fail(DG_ERR_ARG, "denoise: hidden_in is null");
  const bool head = !(flags & DG_STEP_NO_HEAD);
  if (!canvas && (head || !(flags & DG_STEP_HIDDEN_IN)))
    return c->fail(DG_ERR_ARG, "denoise: canvas is null");
  if (head) {
    if (!cfg) return c->fail(DG_ERR_ARG, "denoise: sampler cfg is null");
    if (!out || !out->cand || !out->t_cand || !out->t_cur || !out->lse || !out->entropy)
      return c->fail(DG_ERR_ARG, "denoise: row stats pointer is null");
    if (cfg->max_steps < 1) return c->fail(DG_ERR_ARG, "denoise: max_steps < 1");
    for (int b = 0; b < kv->batch; ++b) {
      const int step = (p && p->steps) ? p->steps[b] : (p ? p->step : 0);
      if (step < 0 || step >= cfg->max_steps) return c->fail(DG_ERR_ARG, "denoise: step out of [0, max_steps)");
    }
    if (!(cfg->temp_start > 0.f) || !(cfg->temp_end > 0.f))
      return c->fail(DG_ERR_ARG, "denoise: temperatures must be > 0");
  }
  return DG_OK;
}

int dg_denoise_step(dg_ctx* c, const int32_t* canvas, const dg_kv_cache* kv,
                    const dg_sampler_cfg* cfg, const dg_step_params* p, dg_row_stats* out,
                    hipStream_t s) {
  if (!c) return DG_ERR_ARG;
  int rc = check_step_args(c, canvas, kv, cfg, p, out);
  if (rc) return rc;
  rc = denoise_impl(c, canvas, kv, cfg, p, out, s);
  if (rc) return rc;
  return check_hip(c, "denoise_step");
}

int dg_denoise_head_static(dg_ctx* c, const int32_t* canvas, const dg_kv_cache* kv,
                           const dg_sampler_cfg* cfg, const dg_step_params* p, dg_row_stats* out,
                           hipStream_t s) {
  if (!c) return DG_ERR_ARG;
  if (!p || p->flags != DG_STEP_HEAD_ONLY)
    return c->fail(DG_ERR_UNSUPPORTED, "denoise_head_static: params with flags == DG_STEP_HEAD_ONLY required");
  int rc = check_step_args(c, canvas, kv, cfg, p, out);
  if (rc) return rc;
  if (!c->static_scratch) return c->fail(DG_ERR_HIP, "denoise_head_static: no static scratch on this device");
  const int B = kv->batch, C = c->m.canvas, rows = B * C;
  const long part_bytes = static_cast<long>(rows) * (c->m.vocab / kHeadSlice) * 8 * sizeof(float);
  const long need = part_bytes + static_cast<long>(rows) * sizeof(int32_t);
  if (need > kStaticScratchBytes) {
    char msg[192];
    snprintf(msg, sizeof msg,
             "denoise_head_static: %d rows at vocab %d need %ld bytes of scratch, above the static %ld "
             "(at most %ld rows at this vocab)", rows, c->m.vocab, need, kStaticScratchBytes,
             kStaticScratchBytes / (need / rows));
    return c->fail(DG_ERR_CAPACITY, msg);
  }
  float* part = static_cast<float*>(c->static_scratch);
  if (canvas && !kv_identity(kv)) {  // the rows of this call, in call order, after the partials
    int32_t* tok = reinterpret_cast<int32_t*>(static_cast<char*>(c->static_scratch) + part_bytes);
    launch_gather_rows(canvas, tok, make_map(C, B, kv->len, kv), s);
    canvas = tok;
  }
  run_head(c, static_cast<const uint16_t*>(p->hidden_in), canvas, kv, cfg, p, out, part, false, s);
  return check_hip(c, "denoise_head_static");
}

int dg_sample_commit(dg_ctx* c, dg_canvas_state* st, const dg_row_stats* rs,
                     const dg_sampler_cfg* cfg, int32_t step, const int32_t* steps,
                     const dg_kv_cache* kv, dg_step_status* status, hipStream_t s) {
  if (!c) return DG_ERR_ARG;
  if (!st || !st->tokens || !st->committed || !st->stable_run || !st->stopped || !rs || !rs->cand ||
      !rs->t_cand ||
      !rs->t_cur || !rs->lse || !rs->entropy || !cfg || !status)
    return c->fail(DG_ERR_ARG, "sample_commit: null pointer");
  int rc = check_kv(c, kv);
  if (rc) return rc;
  for (int b = 0; b < kv->batch; ++b) {
    const int sb = steps ? steps[b] : step;
    if (cfg->max_steps < 1 || sb < 0 || sb >= cfg->max_steps)
      return c->fail(DG_ERR_ARG, "sample_commit: step out of [0, max_steps)");
  }
  if (cfg->commit_per_step < 0 || cfg->stable_steps < 1 || !(cfg->renoise_conf >= 0.f))
    return c->fail(DG_ERR_ARG, "sample_commit: bad sampler config");
  if (cfg->select_mode != 0 && cfg->select_mode != 1)
    return c->fail(DG_ERR_ARG, "sample_commit: select_mode must be 0 or 1");
  if (cfg->select_mode == 1 && !(cfg->entropy_budget >= 0.f && cfg->entropy_budget < INFINITY))
    return c->fail(DG_ERR_ARG, "sample_commit: entropy_budget must be finite and >= 0");
  SamplerArgs a{};
  a.tokens = st->tokens; a.committed = st->committed; a.stable_run = st->stable_run;
  a.stopped = st->stopped;
  a.cand = rs->cand; a.t_cand = rs->t_cand; a.t_cur = rs->t_cur; a.lse = rs->lse; a.ent = rs->entropy;
  a.status = status;
  a.C = c->m.canvas; a.V = c->m.vocab; a.max_steps = cfg->max_steps;
  a.commit_m = cfg->commit_per_step;
  a.log_tau = cfg->renoise_conf > 0.f ? static_cast<float>(std::log(static_cast<double>(cfg->renoise_conf)))
                                      : -INFINITY;
  a.stable_steps = cfg->stable_steps; a.entropy_stop = cfg->entropy_stop;
  a.renoise_committed = cfg->renoise_committed;
  a.select_mode = cfg->select_mode; a.entropy_budget = cfg->entropy_budget;
  a.k0 = static_cast<uint32_t>(cfg->seed); a.k1 = static_cast<uint32_t>(cfg->seed >> 32);
  for (int b = 0; b < kv->batch; ++b) {
    a.pos0[b] = kv->len[b];
    a.slot[b] = kv_slot(kv, b);
    a.step[b] = steps ? steps[b] : step;
  }
  timed(c, "sample_commit", s, [&] { launch_sample_commit(a, kv->batch, s); });
  return check_hip(c, "sample_commit");
}

int dg_commit_block(dg_ctx* c, const int32_t* canvas, dg_kv_cache* kv, int32_t refresh,
                    hipStream_t s) {
  if (!c) return DG_ERR_ARG;
  int rc = check_kv(c, kv);
  if (rc) return rc;
  if (refresh < DG_COMMIT_LAST || refresh > DG_COMMIT_CAUSAL)
    return c->fail(DG_ERR_ARG, "commit_block: refresh must be 0, 1 or 2");
  if (refresh && !canvas) return c->fail(DG_ERR_ARG, "commit_block: refresh needs the canvas");
  const dg_model_desc& m = c->m;
  for (int b = 0; b < kv->batch; ++b)
    if (static_cast<long>(kv->len[b]) + m.canvas > kv->cap)
      return c->fail(DG_ERR_CAPACITY, "commit_block: len + canvas > cap");
  if (refresh == DG_COMMIT_CAUSAL) {  // prefill takes the canvases back to back, in call order
    const int32_t* toks = canvas;
    if (!kv_identity(kv)) {
      launch_gather_rows(canvas, c->tok, make_map(m.canvas, kv->batch, kv->len, kv), s);
      toks = c->tok;
    }
    std::vector<int32_t> n_new(kv->batch, m.canvas);
    return dg_prefill_causal(c, toks, n_new.data(), kv->batch, kv, s);
  }
  if (refresh) {
    dg_step_params p{};
    p.flags = DG_STEP_NO_HEAD;
    rc = denoise_impl(c, canvas, kv, nullptr, &p, nullptr, s);
    if (rc) return rc;
  }
  const RowMap map = make_map(m.canvas, kv->batch, kv->len, kv);
  ReqIndex src{};  // where each request's canvas K/V sit in the workspace (the last forward)
  for (int b = 0; b < kv->batch; ++b) {
    src.idx[b] = -1;
    for (size_t j = 0; j < c->last_slots.size(); ++j)
      if (c->last_slots[j] == kv_slot(kv, b)) src.idx[b] = static_cast<int32_t>(j);
    if (src.idx[b] < 0)
      return c->fail(DG_ERR_ARG, "commit_block: the last forward pass did not cover this request's slot");
  }
  const long per_layer_ws = static_cast<long>(c->max_batch) * m.n_kv_heads * m.canvas * m.head_dim;
  for (int l = 0; l < m.n_layers; ++l) {
    const long dst = l * kv_layer_stride(m, kv_slots(kv), kv->cap);
    timed(c, "kv_append", s, [&] {
      launch_kv_append(c->ck + l * per_layer_ws, c->cv + l * per_layer_ws, kv->k + dst, kv->v + dst,
                       kv->batch, m.n_kv_heads, m.canvas, m.head_dim, kv->cap, map, src, s);
    });
  }
  rc = check_hip(c, "commit_block");
  if (rc) return rc;
  for (int b = 0; b < kv->batch; ++b) kv->len[b] += m.canvas;
  return DG_OK;
}

int dg_timing_enable(dg_ctx* c, int32_t enable) {
  if (!c) return DG_ERR_ARG;
  c->timing = enable != 0;
  return DG_OK;
}

int dg_timing_read(dg_ctx* c, dg_kernel_time* out, int32_t max) {
  if (!c) return DG_ERR_ARG;
  if (!out || max < 0) return c->fail(DG_ERR_ARG, "timing_read: bad output buffer");
  std::vector<dg_kernel_time> acc;
  for (auto& r : c->recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      return c->fail(DG_ERR_HIP, "timing_read: event query failed");
    auto it = std::find_if(acc.begin(), acc.end(),
                           [&](const dg_kernel_time& k) { return std::strcmp(k.name, r.name) == 0; });
    if (it == acc.end()) acc.push_back({r.name, 1, ms});
    else { it->launches += 1; it->total_ms += ms; }
    c->pool.push_back(r.a);
    c->pool.push_back(r.b);
  }
  c->recs.clear();
  const int n = std::min<int>(max, static_cast<int>(acc.size()));
  for (int i = 0; i < n; ++i) out[i] = acc[i];
  return n;
}

int dg_device_errors(dg_ctx* c, uint32_t* flags, hipStream_t s) {
  if (!c) return DG_ERR_ARG;
  if (!flags) return c->fail(DG_ERR_ARG, "device_errors: null pointer");
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, c->dev_err, sizeof v, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return c->fail(DG_ERR_HIP, "device_errors: read failed");
  if (v != 0 && hipMemsetAsync(c->dev_err, 0, sizeof v, s) != hipSuccess)
    return c->fail(DG_ERR_HIP, "device_errors: clear failed");
  *flags = v;
  return check_hip(c, "device_errors");
}

int dg_debug_set_canvas_kv(dg_ctx* c, const uint16_t* k, const uint16_t* v, int32_t batch,
                           hipStream_t s) {
  if (!c) return DG_ERR_ARG;
  if (!k || !v) return c->fail(DG_ERR_ARG, "set_canvas_kv: null pointer");
  if (batch < 1 || batch > c->max_batch) return c->fail(DG_ERR_ARG, "set_canvas_kv: bad batch");
  const dg_model_desc& m = c->m;
  const long per_b = static_cast<long>(m.n_kv_heads) * m.canvas * m.head_dim;
  for (int l = 0; l < m.n_layers; ++l) {
    const long dst = static_cast<long>(l) * c->max_batch * per_b, src = static_cast<long>(l) * batch * per_b;
    (void)hipMemcpyAsync(c->ck + dst, k + src, 2 * batch * per_b, hipMemcpyDeviceToDevice, s);
    (void)hipMemcpyAsync(c->cv + dst, v + src, 2 * batch * per_b, hipMemcpyDeviceToDevice, s);
  }
  c->last_slots.resize(batch);  // the rows now stand for slots 0..batch-1
  for (int b = 0; b < batch; ++b) c->last_slots[b] = b;
  return check_hip(c, "set_canvas_kv");
}

}  // extern "C"
