// Top-k routed MoE: stable token permutation, expert grouped GEMMs (MFMA, weight-streaming),
// and the gate-weighted un-permute combine.
//
// At 256-2048 canvas rows each expert sees only ~16-130 routed rows, so the expert GEMMs are
// bound by streaming the expert weights from HBM, each byte used by a handful of tokens.  The
// kernels therefore make the weights the MFMA A operand, read every weight element exactly
// once (per pass of up to TMAX*16 tokens) straight from HBM into registers, and gather the
// few token rows (L2-resident) as the B operand.  No permuted copy of the activations is
// materialised: GEMM1 gathers row perm[p] / top_k of the normed activations directly.
#include "dg_common.h"
#include "dg_kernels.h"

namespace dg {
namespace {

// ------------------------------------------------------------------------------ permute
// One 1024-thread work-group.  Routes r = t*top_k + j are ranked by (expert, r): counts per
// expert (LDS integer atomics; the totals are order-independent), exclusive scan, then per
// 1024-route chunk each wave finds equal-expert lanes with 7 ballots, ranks within the wave
// by popcount, and offsets by the earlier waves' counts and the earlier chunks' totals.
__global__ __launch_bounds__(1024) void moe_permute_kernel(const int32_t* __restrict__ idx,
                                                           int n, int n_exp,
                                                           int32_t* __restrict__ offs,
                                                           int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ inv) {
  __shared__ int cnt[64];
  __shared__ int base[64];
  __shared__ int wcnt[16][64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid < 64) cnt[tid] = 0;
  __syncthreads();
  for (int r = tid; r < n; r += 1024) atomicAdd(&cnt[idx[r]], 1);
  __syncthreads();
  if (tid < 64) {
    // exclusive scan over 64 experts in one wave
    int c = (tid < n_exp) ? cnt[tid] : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    const int excl = incl - c;
    base[tid] = excl;
    if (tid < n_exp) offs[tid] = excl;
    if (tid == 0) offs[n_exp] = n;
  }
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < n; c0 += 1024) {
    wcnt[w][lane] = 0;
    __syncthreads();
    const int r = c0 + tid;
    const int e = (r < n) ? idx[r] : 127;
    unsigned long long match = ~0ull;
#pragma unroll
    for (int bit = 0; bit < 7; ++bit) {
      const bool set = (e >> bit) & 1;
      const unsigned long long bal = __ballot(set);
      match &= set ? bal : ~bal;
    }
    const int rank = __popcll(match & below);
    if (r < n && rank == 0) wcnt[w][e] = __popcll(match);
    __syncthreads();
    if (r < n) {
      int pre = 0;
      for (int v = 0; v < w; ++v) pre += wcnt[v][e];
      const int p = base[e] + pre + rank;
      perm[p] = r;
      inv[r] = p;
    }
    __syncthreads();
    if (tid < 64) {
      int tot = 0;
      for (int v = 0; v < 16; ++v) tot += wcnt[v][tid];
      base[tid] += tot;
    }
    __syncthreads();
  }
}

// --------------------------------------------------------------------------- expert GEMMs
// Work-group = 4 waves; wave w owns 16 output features of one expert.  K is walked in 32-wide
// MFMA steps, unrolled so several weight loads are in flight per lane.
constexpr int TMAX = 4;  // token tiles of 16 per pass

template <bool GATED>
__global__ __launch_bounds__(256) void moe_gemm_kernel(MoeArgs a) {
  const int e = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j4 = lane >> 4, l16 = lane & 15;
  const int p0 = a.offs[e], n_e = a.offs[e + 1] - p0;
  if (n_e == 0) return;
  const int f0 = blockIdx.x * 64 + w * 16;
  const long wrow = (static_cast<long>(e) * a.N + f0 + l16) * a.K + 8 * j4;
  const uint16_t* wg = a.w0 + wrow;
  const uint16_t* wu = GATED ? a.w1 + wrow : nullptr;

  for (int ps = 0; ps < n_e; ps += TMAX * 16) {
    const int nt = min(TMAX, (n_e - ps + 15) / 16);
    const uint16_t* xr[TMAX];
    bool xv[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      const int r = ps + t * 16 + l16;
      xv[t] = (t < nt) && (r < n_e);
      long row = 0;
      if (xv[t]) row = GATED ? (a.perm[p0 + r] / a.top_k) : (p0 + r);
      xr[t] = a.x + row * a.ldx + 8 * j4;
    }
    floatx4_t ag[TMAX], au[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      ag[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      au[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll 8
    for (int k = 0; k < a.K; k += 32) {
      const u32x4_t fg = ld16_nt(wg + k);
      u32x4_t fu;
      if constexpr (GATED) fu = ld16_nt(wu + k);
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        if (t < nt) {
          const u32x4_t xb = xv[t] ? ld16(xr[t] + k) : u32x4_t{0u, 0u, 0u, 0u};
          ag[t] = mfma16(fg, xb, ag[t]);
          if constexpr (GATED) au[t] = mfma16(fu, xb, au[t]);
        }
      }
    }
    // lane holds out[f0 + 4*j4 + i][token col l16] of each tile
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      const int r = ps + t * 16 + l16;
      if (t >= nt || r >= n_e) continue;
      const long orow = static_cast<long>(p0 + r) * a.ldo + f0 + 4 * j4;
      if constexpr (GATED) {
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = ag[t][i] / (1.0f + expf(-ag[t][i])) * au[t][i];
        *reinterpret_cast<u32x2_t*>(a.out_bf16 + orow) =
            u32x2_t{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])};
      } else {
        *reinterpret_cast<floatx4_t*>(a.out_f32 + orow) = ag[t];
      }
    }
  }
}

// h[t] += sum_j gate[t][j] * y[inv[t*k+j]]  (j in order; one thread per 4 columns)
__global__ __launch_bounds__(256) void moe_combine_kernel(float* __restrict__ h,
                                                          const float* __restrict__ y,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ gates,
                                                          int rows, int d, int top_k) {
  const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  const int per_row = d / 4;
  if (i >= static_cast<long>(rows) * per_row) return;
  const int t = static_cast<int>(i / per_row), c = static_cast<int>(i % per_row) * 4;
  floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < top_k; ++j) {
    const float g = gates[static_cast<long>(t) * top_k + j];
    const int p = inv[static_cast<long>(t) * top_k + j];
    acc += g * *reinterpret_cast<const floatx4_t*>(y + static_cast<long>(p) * d + c);
  }
  floatx4_t* hp = reinterpret_cast<floatx4_t*>(h + static_cast<long>(t) * d + c);
  floatx4_t o = *hp;
  o += acc;
  *hp = o;
}

}  // namespace

void launch_moe_permute(const int32_t* idx, int n_routes, int n_exp, int32_t* offs, int32_t* perm,
                        int32_t* inv, hipStream_t s) {
  hipLaunchKernelGGL(moe_permute_kernel, dim3(1), dim3(1024), 0, s, idx, n_routes, n_exp, offs,
                     perm, inv);
}

void launch_moe_gemm1(const MoeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(moe_gemm_kernel<true>, dim3(a.N / 64, a.n_exp), dim3(256), 0, s, a);
}

void launch_moe_gemm2(const MoeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(moe_gemm_kernel<false>, dim3(a.N / 64, a.n_exp), dim3(256), 0, s, a);
}

void launch_moe_combine(float* h, const float* y, const int32_t* inv, const float* gates, int rows,
                        int d, int top_k, hipStream_t s) {
  const long n = static_cast<long>(rows) * (d / 4);
  hipLaunchKernelGGL(moe_combine_kernel, dim3((n + 255) / 256), dim3(256), 0, s, h, y, inv, gates,
                     rows, d, top_k);
}

}  // namespace dg
