// Top-k routed MoE: stable token permutation, expert grouped GEMMs (MFMA, weight-streaming),
// and the gate-weighted un-permute combine.
//
// At 256-2048 canvas rows each expert sees only ~16-130 routed rows, so the expert GEMMs are
// bound by streaming the expert weights from HBM, each byte used by a handful of tokens.  The
// kernels therefore make the weights the MFMA A operand, read every weight element exactly
// once (per pass of up to TT*16 tokens) straight from HBM into registers, and gather the
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
// Work-group = 4 waves on one 16-row tile of one expert's weights; wave w takes the w-th
// quarter of the reduction dimension, so every wave streams a short contiguous run of the
// packed weights (many waves in flight, small tail), and the four partial tiles are added in
// LDS in wave order (deterministic).  The expert's routed rows are covered in passes of TT
// 16-row tiles.  The k loop runs over chunks of KS k-steps through a two-stage register
// pipeline: the weight fragments (non-temporal 16-byte loads; each wave-wide load is one
// contiguous 1 KB fragment) and the gathered activation fragments of chunk c+1 are issued
// before the MFMAs of chunk c.  Every load in the loop is unconditional (clamped row / chunk
// indices) and a scheduling fence keeps each prefetch ahead of the MFMAs, so the compiler
// waits only for the older chunk.
template <bool GATED, int TT, int KS>
__global__ __launch_bounds__(256) void moe_gemm_kernel(MoeArgs a) {
  constexpr int NA = GATED ? 2 : 1;
  __shared__ floatx4_t red[3][NA][TT][64];
  const int e = blockIdx.y, ft = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j4 = lane >> 4, l16 = lane & 15;
  const int p0 = a.offs[e], n_e = a.offs[e + 1] - p0;
  if (n_e == 0) return;  // uniform over the work-group
  const int S = a.K / 32, sq = S / 4, s0 = w * sq;  // this wave's k-steps [s0, s0 + sq)
  const uint16_t* wp =
      a.wp + ((static_cast<long>(e) * (a.N / 16) + ft) * S + s0) * NA * 512 + lane * 8;
  const int nch = sq / KS;

  for (int ps = 0; ps < n_e; ps += TT * 16) {
    // rows past the expert's count re-read its last row; those columns are never stored
    const uint16_t* xr[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const int r = min(ps + t * 16 + l16, n_e - 1);
      const long row = GATED ? (a.perm[p0 + r] / a.top_k) : (p0 + r);
      xr[t] = a.x + row * a.ldx + s0 * 32 + 8 * j4;
    }
    floatx4_t acc[NA][TT];
#pragma unroll
    for (int q = 0; q < NA; ++q)
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[q][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t fw[2][KS][NA], fx[2][KS][TT];
    auto load = [&](int b, int c) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int st = c * KS + ks;
#pragma unroll
        for (int q = 0; q < NA; ++q) fw[b][ks][q] = ld16_nt(wp + (st * NA + q) * 512);
#pragma unroll
        for (int t = 0; t < TT; ++t) fx[b][ks][t] = ld16(xr[t] + st * 32);
      }
    };
    auto compute = [&](int b) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int q = 0; q < NA; ++q) acc[q][t] = mfma16(fw[b][ks][q], fx[b][ks][t], acc[q][t]);
    };
    load(0, 0);
    for (int c = 0; c < nch; c += 2) {
      load(1, min(c + 1, nch - 1));
      sched_fence();
      compute(0);
      sched_fence();
      load(0, min(c + 2, nch - 1));
      sched_fence();
      if (c + 1 < nch) compute(1);
      sched_fence();
    }
    if (w > 0) {
#pragma unroll
      for (int q = 0; q < NA; ++q)
#pragma unroll
        for (int t = 0; t < TT; ++t) red[w - 1][q][t][lane] = acc[q][t];
    }
    __syncthreads();
    if (w == 0) {
      // lane holds out[16 ft + 4 j4 + i][token col l16] of each tile
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        floatx4_t v[NA];
#pragma unroll
        for (int q = 0; q < NA; ++q)
          v[q] = ((acc[q][t] + red[0][q][t][lane]) + red[1][q][t][lane]) + red[2][q][t][lane];
        const int r = ps + t * 16 + l16;
        if (r >= n_e) continue;
        const long orow = static_cast<long>(p0 + r) * a.ldo + ft * 16 + 4 * j4;
        if constexpr (GATED) {
          float y[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] = v[0][i] / (1.0f + expf(-v[0][i])) * v[NA - 1][i];
          *reinterpret_cast<u32x2_t*>(a.out_bf16 + orow) =
              u32x2_t{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])};
        } else {
          *reinterpret_cast<floatx4_t*>(a.out_f32 + orow) = v[0];
        }
      }
    }
    __syncthreads();  // red is reused by the next pass
  }
}

// Down projection (no gate): the expert's routed rows of the SwiGLU output are small (K = d_ff),
// so a work-group stages TT*16 of them in LDS once and its 4 waves each stream the full K of
// their own 16-row weight tile (64 output features per work-group) with the activation
// fragments read from LDS; only weights come from HBM in the k loop.
template <int TT, int KS>
__global__ __launch_bounds__(256) void moe_down_kernel(MoeArgs a) {
  extern __shared__ uint16_t xs[];  // [TT*16][K + 8]
  const int e = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j4 = lane >> 4, l16 = lane & 15;
  const int p0 = a.offs[e], n_e = a.offs[e + 1] - p0;
  if (n_e == 0) return;  // uniform over the work-group
  const int ft = blockIdx.x * 4 + w;
  const int S = a.K / 32, ldx = a.K + 8;
  const uint16_t* wp = a.wp + (static_cast<long>(e) * (a.N / 16) + ft) * S * 512 + lane * 8;
  const int nch = S / KS;
  const int cpr = a.K / 8;  // 16-byte chunks per activation row
  for (int ps = 0; ps < n_e; ps += TT * 16) {
    // stage rows [ps, ps + TT*16) (rows past the count repeat the last one; never stored)
    for (int c = threadIdx.x; c < TT * 16 * cpr; c += 256) {
      const int r = c / cpr, col = (c - r * cpr) * 8;
      const long row = p0 + min(ps + r, n_e - 1);
      st16(xs + r * ldx + col, ld16(a.x + row * a.ldx + col));
    }
    __syncthreads();
    floatx4_t acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t fw[2][KS];
    auto load = [&](int b, int c) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) fw[b][ks] = ld16_nt(wp + (c * KS + ks) * 512);
    };
    auto compute = [&](int b, int c) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int kk = (c * KS + ks) * 32 + 8 * j4;
#pragma unroll
        for (int t = 0; t < TT; ++t)
          acc[t] = mfma16(fw[b][ks], ld16(xs + (t * 16 + l16) * ldx + kk), acc[t]);
      }
    };
    load(0, 0);
    for (int c = 0; c < nch; c += 2) {
      load(1, min(c + 1, nch - 1));
      sched_fence();
      compute(0, c);
      sched_fence();
      load(0, min(c + 2, nch - 1));
      sched_fence();
      if (c + 1 < nch) compute(1, c + 1);
      sched_fence();
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const int r = ps + t * 16 + l16;
      if (r >= n_e) continue;
      *reinterpret_cast<floatx4_t*>(a.out_f32 + static_cast<long>(p0 + r) * a.ldo + ft * 16 + 4 * j4) = acc[t];
    }
    __syncthreads();  // xs is restaged by the next pass
  }
}

// One thread per 16-byte fragment piece of the packed layout.
__global__ __launch_bounds__(256) void moe_pack_kernel(const uint16_t* __restrict__ w0,
                                                       const uint16_t* __restrict__ w1,
                                                       uint16_t* __restrict__ out, int n_exp,
                                                       int N, int K, int na) {
  const int S = K / 32, T = N / 16;
  const long total = static_cast<long>(n_exp) * T * S * na * 64;
  const long c = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= total) return;
  const int lane = static_cast<int>(c % 64);
  long r = c / 64;
  const int q = static_cast<int>(r % na);
  r /= na;
  const int st = static_cast<int>(r % S);
  r /= S;
  const int ft = static_cast<int>(r % T);
  const long e = r / T;
  const uint16_t* src = (q == 0 ? w0 : w1) + ((e * N + ft * 16 + (lane & 15)) * static_cast<long>(K)) +
                        st * 32 + 8 * (lane >> 4);
  st16(out + c * 8, ld16(src));
}

// h[t] += sum_z part_z[t] + sum_j gate[t][j] * y[inv[t*k+j]]  (z then j in order; one thread
// per 4 columns)
__global__ __launch_bounds__(256) void moe_combine_kernel(float* __restrict__ h,
                                                          const float* __restrict__ part,
                                                          int n_part, long part_stride,
                                                          const float* __restrict__ y,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ gates,
                                                          int rows, int d, int top_k) {
  const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  const int per_row = d / 4;
  if (i >= static_cast<long>(rows) * per_row) return;
  const int t = static_cast<int>(i / per_row), c = static_cast<int>(i % per_row) * 4;
  floatx4_t pz[kMaxParts], yj[8];
  float gj[8];
#pragma unroll
  for (int z = 0; z < kMaxParts; ++z)
    if (z < n_part) pz[z] = *reinterpret_cast<const floatx4_t*>(part + z * part_stride + static_cast<long>(t) * d + c);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < top_k) {
      gj[j] = gates[static_cast<long>(t) * top_k + j];
      yj[j] = *reinterpret_cast<const floatx4_t*>(y + static_cast<long>(inv[static_cast<long>(t) * top_k + j]) * d + c);
    }
  floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int z = 0; z < kMaxParts; ++z)
    if (z < n_part) acc += pz[z];
  for (int j = 0; j < top_k; ++j) {
    if (j < 8) {
      acc += gj[j] * yj[j];
    } else {
      const float g = gates[static_cast<long>(t) * top_k + j];
      const int p = inv[static_cast<long>(t) * top_k + j];
      acc += g * *reinterpret_cast<const floatx4_t*>(y + static_cast<long>(p) * d + c);
    }
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

// Gate/up: token tiles per pass from the mean routed rows per expert; one k-step per chunk
// (measured fastest: lowest register count, most waves in flight).
void launch_moe_gemm1(const MoeArgs& a, int mean_rows, hipStream_t s) {
  const dim3 grid(a.N / 16, a.n_exp);
  if (mean_rows <= 24) hipLaunchKernelGGL((moe_gemm_kernel<true, 2, 1>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((moe_gemm_kernel<true, 4, 1>), grid, dim3(256), 0, s, a);
}

// Down: activation rows staged in LDS ((TT*16) x (K+8) bf16), 64 output features per group.
void launch_moe_gemm2(const MoeArgs& a, int mean_rows, hipStream_t s) {
  const dim3 grid(a.N / 64, a.n_exp);
  const int S = a.K / 32;
  if (mean_rows <= 24) {
    const size_t lds = 2 * 16 * static_cast<size_t>(a.K + 8) * 2;
    if (S % 4 == 0) hipLaunchKernelGGL((moe_down_kernel<2, 4>), grid, dim3(256), lds, s, a);
    else if (S % 2 == 0) hipLaunchKernelGGL((moe_down_kernel<2, 2>), grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL((moe_down_kernel<2, 1>), grid, dim3(256), lds, s, a);
  } else {
    const size_t lds = 4 * 16 * static_cast<size_t>(a.K + 8) * 2;
    if (S % 2 == 0) hipLaunchKernelGGL((moe_down_kernel<4, 2>), grid, dim3(256), lds, s, a);
    else hipLaunchKernelGGL((moe_down_kernel<4, 1>), grid, dim3(256), lds, s, a);
  }
}

void launch_moe_pack(const uint16_t* w0, const uint16_t* w1, uint16_t* out, int n_exp, int N, int K,
                     hipStream_t s) {
  const int na = w1 ? 2 : 1;
  const long total = static_cast<long>(n_exp) * (N / 16) * (K / 32) * na * 64;
  hipLaunchKernelGGL(moe_pack_kernel, dim3((total + 255) / 256), dim3(256), 0, s, w0, w1, out, n_exp,
                     N, K, na);
}

void launch_moe_combine(float* h, const float* part, int n_part, long part_stride, const float* y,
                        const int32_t* inv, const float* gates, int rows, int d, int top_k,
                        hipStream_t s) {
  const long n = static_cast<long>(rows) * (d / 4);
  hipLaunchKernelGGL(moe_combine_kernel, dim3((n + 255) / 256), dim3(256), 0, s, h, part, n_part,
                     part_stride, y, inv, gates, rows, d, top_k);
}

}  // namespace dg
