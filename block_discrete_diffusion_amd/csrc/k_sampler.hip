// Confidence sampler step, uniform-state canvas start, and the block commit (KV append).
//
// One work-group per canvas, one thread per slot.  Every uncommitted slot gets its rank under
// (key desc, slot asc) by counting the slots that beat it (256 compares from LDS), so ties are
// resolved exactly like a stable sort.  The key is the log-confidence t - lse for the top-m
// rule, and minus the entropy for the entropy-bounded rule ([DOCS] table, token-selection row),
// whose cut is found by one thread adding the entropies in rank order in float32, exactly the
// order the definition gives.  Decisions are taken in float32.  Re-noise tokens come from the
// Philox stream RENOISE keyed by (seed; 0, position, step, request).
#include "dg_common.h"
#include "dg_kernels.h"

namespace dg {
namespace {

struct StatusDev {
  int32_t changed, n_committed, n_new, n_renoised, stable_run, stop, nonfinite;
  float mean_entropy;
};

template <typename T>
DG_DEVICE T block_sum(T v, T* red) {
  // 256 threads: wave sums, then wave 0 sums the 4 partials in fixed order
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) red[w] = v;
  __syncthreads();
  const T tot = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return tot;
}

__global__ __launch_bounds__(256) void sample_commit_kernel(SamplerArgs a) {
  __shared__ __align__(16) float cc_s[256];
  __shared__ __align__(16) int u_s[256];
  __shared__ float h_sorted[256];
  __shared__ int m_s;
  __shared__ int ired[4];
  __shared__ float fred[4];
  const int b = blockIdx.x, i = threadIdx.x;
  const int sb = a.slot[b];  // the request's slot in every per-request array
  const int C = a.C;
  if (a.stopped[sb]) {  // finished canvas: frozen
    if (i == 0) {
      StatusDev st = reinterpret_cast<StatusDev*>(a.status)[sb];
      st.changed = 0;
      st.n_new = 0;
      st.n_renoised = 0;
      st.stop = 1;
      reinterpret_cast<StatusDev*>(a.status)[sb] = st;
    }
    return;
  }
  const bool slot = i < C;
  const long r = static_cast<long>(sb) * C + i;
  const int x_prev = slot ? a.tokens[r] : 0;
  const bool com_prev = slot ? a.committed[r] != 0 : true;
  const float lse = slot ? a.lse[r] : 0.f;
  const float cc = slot ? a.t_cand[r] - lse : 0.f;
  const float cu = slot ? a.t_cur[r] - lse : 0.f;
  const int cand = slot ? a.cand[r] : 0;
  const float ent = slot ? a.ent[r] : 0.f;
  const int stable_prev = a.stable_run[sb];
  const bool U = slot && !com_prev;
  const bool by_entropy = a.select_mode == 1;
  const float key = by_entropy ? -ent : cc;
  cc_s[i] = key;
  u_s[i] = U ? 1 : 0;
  const int n_u = block_sum<int>(U ? 1 : 0, ired);  // contains the barrier publishing cc_s/u_s
  // 16-byte LDS reads, eight in flight: the scan is latency-bound, not compare-bound
  int rank = 0;
  if (U) {
    const floatx4_t* cc4 = reinterpret_cast<const floatx4_t*>(cc_s);
    const u32x4_t* u4 = reinterpret_cast<const u32x4_t*>(u_s);
#pragma unroll 8
    for (int j4 = 0; j4 < C / 4; ++j4) {
      const floatx4_t cv = cc4[j4];
      const u32x4_t uv = u4[j4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = 4 * j4 + q;
        rank += (uv[q] && (cv[q] > key || (cv[q] == key && j < i))) ? 1 : 0;
      }
    }
  }
  int m = min(a.commit_m, n_u);
  if (by_entropy) {  // uniform branch
    if (U) h_sorted[rank] = ent;
    __syncthreads();
    if (i == 0) {
      // the longest prefix whose running float32 sum stays within the budget, at least one
      float run = 0.f;
      int k = 0;
      for (int j = 0; j < n_u; ++j) {
        run += h_sorted[j];
        if (j > 0 && run > a.entropy_budget) break;
        k = j + 1;
      }
      m_s = k;
    }
    __syncthreads();
    m = m_s;
  }
  const bool sel = U && rank < m;
  const int pos = a.pos0[b] + i;
  const philox_out rnd = philox4x32_10(0u, static_cast<uint32_t>(pos), static_cast<uint32_t>(a.step[b]),
                                       (static_cast<uint32_t>(sb) << 8) | kStreamRenoise, a.k0, a.k1);
  const int fresh = token_from_word(rnd.x[0], static_cast<uint32_t>(a.V));
  int x = x_prev;
  bool com = com_prev;
  int renoised = 0;
  if (slot) {
    if (sel) {
      x = cand;
      com = true;
    } else if (com_prev) {
      if (a.renoise_committed && cu < a.log_tau) { x = fresh; com = false; renoised = 1; }
    } else {
      if (by_entropy || cc < a.log_tau) { x = fresh; renoised = 1; }
      else x = cand;
    }
    a.tokens[r] = x;
    a.committed[r] = com ? 1 : 0;
  }
  const int changed = block_sum<int>((slot && x != x_prev) ? 1 : 0, ired);
  const int n_com = block_sum<int>((slot && com) ? 1 : 0, ired);
  const int n_ren = block_sum<int>(renoised, ired);
  const int nonfin = block_sum<int>((slot && !isfinite(lse)) ? 1 : 0, ired);
  const float ent_sum = block_sum<float>(ent, fred);
  if (i == 0) {
    const float mean_ent = ent_sum / static_cast<float>(C);
    const int sr = changed ? 0 : stable_prev + 1;
    int stop = (sr >= a.stable_steps) || (a.step[b] >= a.max_steps - 1);
    if (a.entropy_stop >= 0.f && !changed && mean_ent < a.entropy_stop) stop = 1;
    a.stable_run[sb] = sr;
    a.stopped[sb] = stop;
    StatusDev st;
    st.changed = changed ? 1 : 0;
    st.n_committed = n_com;
    st.n_new = m;
    st.n_renoised = n_ren;
    st.stable_run = sr;
    st.stop = stop;
    st.nonfinite = nonfin ? 1 : 0;
    st.mean_entropy = mean_ent;
    reinterpret_cast<StatusDev*>(a.status)[sb] = st;
  }
}

__global__ __launch_bounds__(256) void canvas_init_kernel(int32_t* tokens, uint8_t* committed,
                                                          int32_t* stable_run, int32_t* stopped,
                                                          int C, int V,
                                                          uint32_t k0, uint32_t k1, RowMap map) {
  const int b = blockIdx.x, sb = map.slot[b];
  for (int i = threadIdx.x; i < C; i += 256) {
    const philox_out rnd = philox4x32_10(0u, static_cast<uint32_t>(map.pos0[b] + i), 0u,
                                         (static_cast<uint32_t>(sb) << 8) | kStreamInit, k0, k1);
    tokens[static_cast<long>(sb) * C + i] = token_from_word(rnd.x[0], static_cast<uint32_t>(V));
    committed[static_cast<long>(sb) * C + i] = 0;
  }
  if (threadIdx.x == 0) {
    stable_run[sb] = 0;
    stopped[sb] = 0;
  }
}

// 16-byte chunks: src [requests][Hkv][C][D] (the producing call's requests) -> dst
// [slots][Hkv][cap][D]: request b takes source request src.idx[b] and writes cache slot
// slot[b] at positions pos0[b] + i.
__global__ __launch_bounds__(256) void kv_append_kernel(const uint16_t* __restrict__ sk,
                                                        const uint16_t* __restrict__ sv,
                                                        uint16_t* __restrict__ dk,
                                                        uint16_t* __restrict__ dv, int B, int Hkv,
                                                        int C, int D, int cap, RowMap map,
                                                        ReqIndex src) {
  const int cpr = D / 8;  // chunks per row
  const long n = static_cast<long>(B) * Hkv * C * cpr;
  const long t = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= n) return;
  const int ch = static_cast<int>(t % cpr);
  const long row = t / cpr;  // (b*Hkv + g)*C + i
  const int i = static_cast<int>(row % C);
  const long bg = row / C;
  const int b = static_cast<int>(bg / Hkv);
  const long g = bg - static_cast<long>(b) * Hkv;
  const long drow = (static_cast<long>(map.slot[b]) * Hkv + g) * cap + map.pos0[b] + i;
  const long srow = (static_cast<long>(src.idx[b]) * Hkv + g) * C + i;
  st16(dk + drow * D + ch * 8, ld16(sk + srow * D + ch * 8));
  st16(dv + drow * D + ch * 8, ld16(sv + srow * D + ch * 8));
}

}  // namespace

void launch_sample_commit(const SamplerArgs& a, int n_req, hipStream_t s) {
  hipLaunchKernelGGL(sample_commit_kernel, dim3(n_req), dim3(256), 0, s, a);
}

void launch_canvas_init(int32_t* tokens, uint8_t* committed, int32_t* stable_run,
                        int32_t* stopped, int C, int V, uint32_t k0, uint32_t k1, const RowMap& map,
                        hipStream_t s) {
  hipLaunchKernelGGL(canvas_init_kernel, dim3(map.n_req), dim3(256), 0, s, tokens, committed,
                     stable_run, stopped, C, V, k0, k1, map);
}

void launch_kv_append(const uint16_t* src_k, const uint16_t* src_v, uint16_t* dst_k,
                      uint16_t* dst_v, int B, int Hkv, int C, int D, int cap, const RowMap& map,
                      const ReqIndex& src, hipStream_t s) {
  const long n = static_cast<long>(B) * Hkv * C * (D / 8);
  hipLaunchKernelGGL(kv_append_kernel, dim3((n + 255) / 256), dim3(256), 0, s, src_k, src_v,
                     dst_k, dst_v, B, Hkv, C, D, cap, map, src);
}

}  // namespace dg
