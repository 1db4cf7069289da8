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
// Expert GEMM with the activation operand shared through LDS: a work-group of 4 waves owns
// 64 * FPW output features of one expert (wave w: the FPW 16-row weight tiles 4 FPW blockIdx.x +
// FPW w + f) and covers the expert's routed rows in passes of TT 16-row tiles.  Per chunk of
// KC = 32 * KS columns the group stages the pass's rows (gathered through perm for the gate/up
// projection) into LDS once and all four waves read their B fragments from there, so each
// activation row is fetched once per 64 * FPW features.  The weights stream straight into
// registers from the packed fragment layout, whose tile groups match the work-groups: the
// group reads one contiguous run (non-temporal 16-byte loads), two chunks ahead.
//
// Pipeline per chunk c: MFMAs of chunk c (weights in register set c & 1, activations in LDS
// buffer c & 1); store chunk c+1's activations (loaded one chunk earlier) to the other buffer;
// issue the loads of chunk c+2; barrier.  Loads are unconditional (clamped chunk and row
// indices) and the loop body is the same on every trip, so the compiler's wait counts leave
// the younger chunks in flight.
template <bool GATED, int TT, int KS, int FPW>
__global__ __launch_bounds__(256) void expert_stream_kernel(MoeArgs a) {
  constexpr int NA = GATED ? 2 : 1;
  constexpr int GT = 4 * FPW;  // tiles per work-group = tiles per packed group
  constexpr int KC = 32 * KS, ROWS = TT * 16, LDX = KC + 8, CPR = KC / 8;
  constexpr int PIECES = ROWS * CPR, PPT = (PIECES + 255) / 256;
  __shared__ uint16_t xs[2][ROWS * LDX];
  const int e = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int j4 = lane >> 4, l16 = lane & 15;
  const int p0 = a.offs[e], n_e = a.offs[e + 1] - p0;
  if (n_e == 0) return;  // uniform over the work-group
  const int ft0 = blockIdx.x * GT + w * FPW;
  const int S = a.K / 32, nch = S / KS;
  const uint16_t* wp =
      a.wp + ((static_cast<long>(e) * (a.N / (16 * GT)) + blockIdx.x) * S * GT + w * FPW) * NA * 512 + lane * 8;

  // passes of ROWS rows: work-group z takes passes z, z + Z, ... (Z = gridDim.z), so an expert
  // with more rows than one pass holds is covered by parallel work-groups, not a serial pass
  for (int ps = blockIdx.z * ROWS; ps < n_e; ps += ROWS * static_cast<int>(gridDim.z)) {
    // this thread's staging pieces; rows past the expert's count repeat its last row and
    // pieces past the tile are loaded (clamped) but not stored
    const uint16_t* src[PPT];
    int dst[PPT];
    bool keep[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int piece = tid + 256 * j, pc = min(piece, PIECES - 1);
      const int r = pc / CPR, col = (pc % CPR) * 8;
      const int rr = min(ps + r, n_e - 1);
      const long row = GATED ? (a.perm[p0 + rr] / a.top_k) : static_cast<long>(p0 + rr);
      src[j] = a.x + row * a.ldx + col;
      dst[j] = r * LDX + col;
      keep[j] = piece < PIECES;
    }
    floatx4_t acc[FPW][NA][TT];
#pragma unroll
    for (int f = 0; f < FPW; ++f)
#pragma unroll
      for (int q = 0; q < NA; ++q)
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[f][q][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t fw[2][KS][FPW][NA], xr[PPT];
    auto load_w = [&](int b, int c) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int f = 0; f < FPW; ++f)
#pragma unroll
          for (int q = 0; q < NA; ++q)
            fw[b][ks][f][q] = ld16_nt(wp + (((c * KS + ks) * GT + f) * NA + q) * 512);
    };
    auto load_x = [&](int c) {
#pragma unroll
      for (int j = 0; j < PPT; ++j) xr[j] = ld16(src[j] + c * KC);
    };
    auto store_x = [&](int buf) {
#pragma unroll
      for (int j = 0; j < PPT; ++j)
        if (keep[j]) st16(&xs[buf][dst[j]], xr[j]);
    };
    auto compute = [&](int buf, int b) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const u32x4_t xf = ld16(&xs[buf][(t * 16 + l16) * LDX + ks * 32 + 8 * j4]);
#pragma unroll
          for (int f = 0; f < FPW; ++f)
#pragma unroll
            for (int q = 0; q < NA; ++q) acc[f][q][t] = mfma16(fw[b][ks][f][q], xf, acc[f][q][t]);
        }
    };
    load_x(0);
    load_w(0, 0);
    store_x(0);
    load_x(min(1, nch - 1));
    load_w(1, min(1, nch - 1));
    __syncthreads();
    int c = 0;
    for (; c + 1 < nch; c += 2) {
      compute(0, 0);
      sched_fence();
      store_x(1);
      load_x(min(c + 2, nch - 1));
      load_w(0, min(c + 2, nch - 1));
      sched_fence();
      __syncthreads();
      compute(1, 1);
      sched_fence();
      store_x(0);
      load_x(min(c + 3, nch - 1));
      load_w(1, min(c + 3, nch - 1));
      sched_fence();
      __syncthreads();
    }
    if (c < nch) compute(0, 0);  // odd chunk count: the last chunk sits in buffer / set 0
    // lane holds out[16 ft + 4 j4 + i][row col l16] of each tile
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const int r = ps + t * 16 + l16;
      if (r >= n_e) continue;
#pragma unroll
      for (int f = 0; f < FPW; ++f) {
        const long orow = static_cast<long>(p0 + r) * a.ldo + (ft0 + f) * 16 + 4 * j4;
        if constexpr (GATED) {
          float y[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            y[i] = acc[f][0][t][i] / (1.0f + expf(-acc[f][0][t][i])) * acc[f][NA - 1][t][i];
          *reinterpret_cast<u32x2_t*>(a.out_bf16 + orow) = u32x2_t{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])};
        } else {
          *reinterpret_cast<floatx4_t*>(a.out_f32 + orow) = acc[f][0][t];
        }
      }
    }
    if (ps + ROWS * static_cast<int>(gridDim.z) < n_e) __syncthreads();  // the next pass restages xs (uniform)
  }
}

// One thread per 16-byte fragment piece of the packed layout
// [e][tile group fg][k-step s][tile w in group][matrix q][lane], tile ft = gt fg + w.
__global__ __launch_bounds__(256) void moe_pack_kernel(const uint16_t* __restrict__ w0,
                                                       const uint16_t* __restrict__ w1,
                                                       uint16_t* __restrict__ out, int n_exp,
                                                       int N, int K, int na, int gt) {
  const int S = K / 32, G = N / (16 * gt);
  const long total = static_cast<long>(n_exp) * G * S * gt * na * 64;
  const long c = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= total) return;
  const int lane = static_cast<int>(c % 64);
  long r = c / 64;
  const int q = static_cast<int>(r % na);
  r /= na;
  const int w = static_cast<int>(r % gt);
  r /= gt;
  const int st = static_cast<int>(r % S);
  r /= S;
  const int fg = static_cast<int>(r % G);
  const long e = r / G;
  const int ft = gt * fg + w;
  const uint16_t* src = (q == 0 ? w0 : w1) + ((e * N + ft * 16 + (lane & 15)) * static_cast<long>(K)) +
                        st * 32 + 8 * (lane >> 4);
  st16(out + c * 8, ld16(src));
}

// Un-permute + residual, one work-group (8 waves) per row t:
// h[t] += sum_z part_z[t] + sum_j gate[t][j] * y[inv[t*k+j]]   (z then j in order);
// with a gain it also writes the next block's normed input out = bf16(rmsnorm(h[t]) * gain),
// which saves a pass over h.  All of a thread's loads are issued before any arithmetic.
template <int NCH>  // 4-element chunks per thread: ceil(d / 2048)
__global__ __launch_bounds__(512) void moe_combine_kernel(float* __restrict__ h,
                                                          const float* __restrict__ part,
                                                          int n_part, long part_stride,
                                                          const float* __restrict__ y,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ gates, int d,
                                                          int top_k, const float* __restrict__ gain,
                                                          float eps, uint16_t* __restrict__ out) {
  __shared__ float red[8];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float* hr = h + static_cast<long>(t) * d;
  constexpr int KJ = 8;  // routed slots held in registers; more are read in the second loop
  int pj[KJ];
  float gj[KJ];
#pragma unroll
  for (int j = 0; j < KJ; ++j)
    if (j < top_k) {
      pj[j] = inv[static_cast<long>(t) * top_k + j];
      gj[j] = gates[static_cast<long>(t) * top_k + j];
    }
  floatx4_t v[NCH], pz[kMaxParts][NCH], yj[KJ][NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = min((tid + 512 * i) * 4, d - 4);  // clamped; chunks past d are not stored
    v[i] = *reinterpret_cast<const floatx4_t*>(hr + c);
#pragma unroll
    for (int z = 0; z < kMaxParts; ++z)
      if (z < n_part) pz[z][i] = *reinterpret_cast<const floatx4_t*>(part + z * part_stride + static_cast<long>(t) * d + c);
#pragma unroll
    for (int j = 0; j < KJ; ++j)
      if (j < top_k) yj[j][i] = *reinterpret_cast<const floatx4_t*>(y + static_cast<long>(pj[j]) * d + c);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = (tid + 512 * i) * 4;
    floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int z = 0; z < kMaxParts; ++z)
      if (z < n_part) acc += pz[z][i];
#pragma unroll
    for (int j = 0; j < KJ; ++j)
      if (j < top_k) acc += gj[j] * yj[j][i];
    for (int j = KJ; j < top_k; ++j) {
      const float g = gates[static_cast<long>(t) * top_k + j];
      const int p = inv[static_cast<long>(t) * top_k + j];
      acc += g * *reinterpret_cast<const floatx4_t*>(y + static_cast<long>(p) * d + min(c, d - 4));
    }
    v[i] += acc;
    if (c < d) {
      *reinterpret_cast<floatx4_t*>(hr + c) = v[i];
      ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
    }
  }
  if (!gain) return;  // uniform
  ss = wave_sum(ss);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  ss = ((red[0] + red[1]) + (red[2] + red[3])) + ((red[4] + red[5]) + (red[6] + red[7]));
  const float rinv = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = (tid + 512 * i) * 4;
    if (c >= d) continue;
    const floatx4_t g = *reinterpret_cast<const floatx4_t*>(gain + c);
    *reinterpret_cast<u32x2_t*>(out + static_cast<long>(t) * d + c) =
        u32x2_t{pack_bf2(v[i][0] * rinv * g[0], v[i][1] * rinv * g[1]), pack_bf2(v[i][2] * rinv * g[2], v[i][3] * rinv * g[3])};
  }
}

}  // namespace

void launch_moe_permute(const int32_t* idx, int n_routes, int n_exp, int32_t* offs, int32_t* perm,
                        int32_t* inv, hipStream_t s) {
  hipLaunchKernelGGL(moe_permute_kernel, dim3(1), dim3(1024), 0, s, idx, n_routes, n_exp, offs,
                     perm, inv);
}

// Row tiles per pass from the mean routed rows per expert, sized so that the busiest expert
// (about four standard deviations above a uniform mean) still fits one pass; a second
// work-group per expert picks up any pass beyond the first (it exits at once when there is
// none), so a skewed routing costs a parallel work-group instead of a serial pass.
template <bool GATED, int FPW>
void launch_stream(const MoeArgs& a, int mean_rows, hipStream_t s) {
  const dim3 grid(a.N / (64 * FPW), a.n_exp, 2);
  if (mean_rows <= 24) hipLaunchKernelGGL((expert_stream_kernel<GATED, 3, 1, FPW>), grid, dim3(256), 0, s, a);
  else if (mean_rows <= 36) hipLaunchKernelGGL((expert_stream_kernel<GATED, 4, 2, FPW>), grid, dim3(256), 0, s, a);
  else if (mean_rows <= 84) hipLaunchKernelGGL((expert_stream_kernel<GATED, 8, 2, FPW>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((expert_stream_kernel<GATED, 10, 2, FPW>), grid, dim3(256), 0, s, a);
}

void launch_moe_gemm1(const MoeArgs& a, int mean_rows, hipStream_t s) { launch_stream<true, kGroupTiles1 / 4>(a, mean_rows, s); }
void launch_moe_gemm2(const MoeArgs& a, int mean_rows, hipStream_t s) { launch_stream<false, kGroupTiles2 / 4>(a, mean_rows, s); }

void launch_moe_pack(const uint16_t* w0, const uint16_t* w1, uint16_t* out, int n_exp, int N, int K,
                     int group_tiles, hipStream_t s) {
  const int na = w1 ? 2 : 1;
  const long total = static_cast<long>(n_exp) * (N / 16) * (K / 32) * na * 64;
  hipLaunchKernelGGL(moe_pack_kernel, dim3((total + 255) / 256), dim3(256), 0, s, w0, w1, out, n_exp,
                     N, K, na, group_tiles);
}

void launch_moe_combine(float* h, const float* part, int n_part, long part_stride, const float* y,
                        const int32_t* inv, const float* gates, int rows, int d, int top_k,
                        const float* gain, float eps, uint16_t* out, hipStream_t s) {
  const int nch = (d + 2047) / 2048;
#define DG_MC(N)                                                                              \
  hipLaunchKernelGGL(moe_combine_kernel<N>, dim3(rows), dim3(512), 0, s, h, part, n_part,         \
                     part_stride, y, inv, gates, d, top_k, gain, eps, out)
  if (nch <= 1) DG_MC(1);
  else if (nch <= 2) DG_MC(2);
  else DG_MC(4);
#undef DG_MC
}

}  // namespace dg
