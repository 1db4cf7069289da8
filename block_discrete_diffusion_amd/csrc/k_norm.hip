// Token embedding, RMSNorm, and the fused FFN-norm + router + top-k + gate softmax.
//
// The router works on the float32 normed row (not the bf16 copy fed to the experts) so that
// expert choices only differ from an exact computation at genuine near-ties of the logits.
// One wavefront = 64 lanes = one lane per expert (up to 64 experts): top-k is k rounds of a
// wave-wide arg-max by butterfly shuffles, ties going to the lower expert index.
#include "dg_common.h"
#include "dg_kernels.h"

namespace dg {
namespace {

// Embedding gather h = E[tok] (bf16 rows widened to float32), one work-group per row; with a
// gain it also writes the first layer's normed input out = bf16(h * rsqrt(mean h^2 + eps) * gain).
// A token id outside [0, vocab) is clamped into range (the table is never read out of bounds)
// and raises bit kDevErrTokenRange of the sticky error word.
template <int NCH>  // 8-element chunks per thread: ceil(d / 2048)
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tok,
                                                    const uint16_t* __restrict__ embed,
                                                    float* __restrict__ h, int d, int vocab,
                                                    uint32_t* __restrict__ err,
                                                    const float* __restrict__ gain, float eps,
                                                    uint16_t* __restrict__ out) {
  __shared__ float red[4];
  const int r = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int t = tok[r];
  if (static_cast<unsigned>(t) >= static_cast<unsigned>(vocab)) {
    if (threadIdx.x == 0) *err = kDevErrTokenRange;
    t = t < 0 ? 0 : vocab - 1;
  }
  const long src = static_cast<long>(t) * d;
  u32x4_t raw[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = (threadIdx.x + 256 * i) * 8;
    raw[i] = (c < d) ? ld16(embed + src + c) : u32x4_t{0u, 0u, 0u, 0u};
  }
  float o[NCH][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[i][2 * q] = __uint_as_float(raw[i][q] << 16);
      o[i][2 * q + 1] = __uint_as_float(raw[i][q] & 0xffff0000u);
    }
    const int c = (threadIdx.x + 256 * i) * 8;
    if (c >= d) continue;
    float* dst = h + static_cast<long>(r) * d + c;
    *reinterpret_cast<floatx4_t*>(dst) = floatx4_t{o[i][0], o[i][1], o[i][2], o[i][3]};
    *reinterpret_cast<floatx4_t*>(dst + 4) = floatx4_t{o[i][4], o[i][5], o[i][6], o[i][7]};
#pragma unroll
    for (int q = 0; q < 8; ++q) ss += o[i][q] * o[i][q];
  }
  if (!gain) return;  // uniform
  ss = wave_sum(ss);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  ss = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = (threadIdx.x + 256 * i) * 8;
    if (c >= d) continue;
    const floatx4_t g0 = *reinterpret_cast<const floatx4_t*>(gain + c);
    const floatx4_t g1 = *reinterpret_cast<const floatx4_t*>(gain + c + 4);
    *reinterpret_cast<u32x4_t*>(out + static_cast<long>(r) * d + c) =
        u32x4_t{pack_bf2(o[i][0] * inv * g0[0], o[i][1] * inv * g0[1]), pack_bf2(o[i][2] * inv * g0[2], o[i][3] * inv * g0[3]),
                pack_bf2(o[i][4] * inv * g1[0], o[i][5] * inv * g1[1]), pack_bf2(o[i][6] * inv * g1[2], o[i][7] * inv * g1[3])};
  }
}

// One work-group (4 waves) per row; thread t normalises the float4 chunks t, t+256, ...; all of
// a thread's loads are issued before the reduction.
template <int NCH>  // ceil(d / 1024)
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h,
                                                      const float* __restrict__ gain, float eps,
                                                      uint16_t* __restrict__ out, int rows, int d) {
  __shared__ float red[4];
  const int r = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float* x = h + static_cast<long>(r) * d;
  floatx4_t v[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = (threadIdx.x + 256 * i) * 4;
    v[i] = (c < d) ? *reinterpret_cast<const floatx4_t*>(x + c) : floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
  ss = wave_sum(ss);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  ss = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = (threadIdx.x + 256 * i) * 4;
    if (c >= d) continue;
    const floatx4_t g = *reinterpret_cast<const floatx4_t*>(gain + c);
    *reinterpret_cast<u32x2_t*>(out + static_cast<long>(r) * d + c) =
        u32x2_t{pack_bf2(v[i][0] * inv * g[0], v[i][1] * inv * g[1]),
                pack_bf2(v[i][2] * inv * g[2], v[i][3] * inv * g[3])};
  }
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ in,
                                                          uint16_t* __restrict__ out, long n) {
  const long i = (static_cast<long>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i + 3 < n) {
    const floatx4_t v = *reinterpret_cast<const floatx4_t*>(in + i);
    *reinterpret_cast<u32x2_t*>(out + i) = u32x2_t{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
  } else {
    for (long j = i; j < n; ++j) out[j] = f2bf(in[j]);
  }
}

// Residual update + FFN norm + router + top-k, one work-group (8 waves) per R rows.
//  - the router weights of the wave's experts (first round of columns) are requested before
//    the norm, so their latency hides behind it; with one row per group the row's residual and
//    slices are requested first (the wait for them then leaves the weights in flight), and no
//    global store precedes a barrier (a barrier after a store waits for every memory
//    operation of the wave, the weight loads included): h and the bf16 x are written after
//    the last one;
//  - per row, every load (residual, its split-K slices) is issued before the reduction;
//    h += slices (z order, written back); x = h * rsqrt(mean h^2 + eps) * gain in float32;
//    the bf16 copy of x feeds the experts and the float32 x is kept in LDS;
//  - router logits in float32: wave w owns experts 8w .. 8w+7; lane l owns the row elements
//    [8 (l + 64 j), +8) (coalesced 16-byte reads: a wave covers 1 KB of one expert row per
//    request), and every weight chunk is used for all R rows; the eight partials of a row are
//    summed over the wave by a transpose-reduce (three exchange steps halving the expert
//    window, then three plain steps), after which lane l holds expert 8w + (l >> 3);
//  - wave rr picks row rr's experts: lane e = expert e, k rounds of wave arg-max (ties to the
//    lower expert index), softmax gates over the k picks.
constexpr int kRouterWaves = 8;
template <int NCH, int R>  // NCH: 4-element chunks per thread, ceil(d / 2048); R rows (<= 8)
__global__ __launch_bounds__(512) void norm_router_kernel(
    float* __restrict__ h, const float* __restrict__ part, int n_part, long part_stride,
    const float* __restrict__ gain, float eps, const uint16_t* __restrict__ wr, int d, int n_exp,
    int top_k, int rows, uint16_t* __restrict__ bout, int32_t* __restrict__ idx,
    float* __restrict__ gates) {
  __shared__ float red[R][kRouterWaves];
  __shared__ float lg[R][64];
  __shared__ float xs[R][NCH * 2048];
  const int r0 = blockIdx.x * R, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nr = min(R, rows - r0);  // rows of this group (uniform)
  const int nj = (d + 511) / 512;

  // chunks of 512 columns per round of weight loads (fewer when many rows hold accumulators)
  constexpr int JR = (R >= 4 || R * NCH >= 8) ? 2 : 4;
  u32x4_t wv[JR][8];
  auto load_w = [&](int j0) {
#pragma unroll
    for (int jj = 0; jj < JR; ++jj)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = min((lane + 64 * (j0 + jj)) * 8, d - 8);  // clamped: always in bounds
        const int ee = min(8 * w + e, n_exp - 1);
        wv[jj][e] = ld16(wr + static_cast<long>(ee) * d + c);
      }
  };
  // residual and slices of row rr, chunk i (uniform row guard; lanes past d load nothing)
  floatx4_t v[R][NCH];
  constexpr int EP = (R == 1) ? kMaxParts : 1;  // one row: its slices are loaded up front
  floatx4_t pe[EP][NCH];
  auto load_row = [&](int rr, floatx4_t (&pz)[EP][NCH]) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = (tid + 512 * i) * 4;
      const bool ok = c < d;
      v[rr][i] = ok ? *reinterpret_cast<const floatx4_t*>(h + static_cast<long>(r0 + rr) * d + c)
                    : floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int z = 0; z < EP; ++z)
        if (z < n_part && ok)
          pz[z][i] = *reinterpret_cast<const floatx4_t*>(part + z * part_stride + static_cast<long>(r0 + rr) * d + c);
    }
  };
  // the norm gain, also ahead of the weights (a wait for a load waits for every older one)
  floatx4_t gv[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = (tid + 512 * i) * 4;
    gv[i] = c < d ? *reinterpret_cast<const floatx4_t*>(gain + c) : floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (R == 1) load_row(0, pe);
  load_w(0);

#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    if (rr >= nr) break;
    floatx4_t pz[kMaxParts][NCH];
    if constexpr (R == 1) {
#pragma unroll
      for (int z = 0; z < kMaxParts; ++z)
#pragma unroll
        for (int i = 0; i < NCH; ++i) pz[z][i] = pe[z][i];
    } else {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = (tid + 512 * i) * 4;
        const bool ok = c < d;
        v[rr][i] = ok ? *reinterpret_cast<const floatx4_t*>(h + static_cast<long>(r0 + rr) * d + c)
                      : floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int z = 0; z < kMaxParts; ++z)
          if (z < n_part && ok)
            pz[z][i] = *reinterpret_cast<const floatx4_t*>(part + z * part_stride + static_cast<long>(r0 + rr) * d + c);
      }
    }
    if (n_part > 0) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = (tid + 512 * i) * 4;
        if (c >= d) continue;  // no slices were loaded there: v stays zero
#pragma unroll
        for (int z = 0; z < kMaxParts; ++z)
          if (z < n_part) v[rr][i] += pz[z][i];
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) ss += v[rr][i][q] * v[rr][i][q];
    ss = wave_sum(ss);
    if (lane == 0) red[rr][w] = ss;
  }
  __syncthreads();
  u32x2_t xb[R][NCH];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    if (rr >= nr) break;
    const float ss = ((red[rr][0] + red[rr][1]) + (red[rr][2] + red[rr][3])) +
                     ((red[rr][4] + red[rr][5]) + (red[rr][6] + red[rr][7]));
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = (tid + 512 * i) * 4;
      if (c >= d) continue;
      floatx4_t x;
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = v[rr][i][q] * inv * gv[i][q];
      xb[rr][i] = u32x2_t{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3])};
      *reinterpret_cast<floatx4_t*>(&xs[rr][c]) = x;
    }
  }
  __syncthreads();
  // global stores only now: the updated residual (when slices were added) and the bf16 x
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    if (rr >= nr) break;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = (tid + 512 * i) * 4;
      if (c >= d) continue;
      if (n_part > 0) *reinterpret_cast<floatx4_t*>(h + static_cast<long>(r0 + rr) * d + c) = v[rr][i];
      *reinterpret_cast<u32x2_t*>(bout + static_cast<long>(r0 + rr) * d + c) = xb[rr][i];
    }
  }

  // router: 8 experts per wave, JR row chunks of 512 elements per round of loads
  float p[R][8];
#pragma unroll
  for (int rr = 0; rr < R; ++rr)
#pragma unroll
    for (int e = 0; e < 8; ++e) p[rr][e] = 0.f;
  for (int j0 = 0; j0 < nj; j0 += JR) {
    if (j0 > 0) load_w(j0);
#pragma unroll
    for (int jj = 0; jj < JR; ++jj) {
      const int c = (lane + 64 * (j0 + jj)) * 8;
      if (c >= d) continue;
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const floatx4_t x0 = *reinterpret_cast<const floatx4_t*>(&xs[rr][c]);
        const floatx4_t x1 = *reinterpret_cast<const floatx4_t*>(&xs[rr][c + 4]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float acc = p[rr][e];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            acc += __uint_as_float(wv[jj][e][q] << 16) * x0[2 * q];
            acc += __uint_as_float(wv[jj][e][q] & 0xffff0000u) * x0[2 * q + 1];
            acc += __uint_as_float(wv[jj][e][2 + q] << 16) * x1[2 * q];
            acc += __uint_as_float(wv[jj][e][2 + q] & 0xffff0000u) * x1[2 * q + 1];
          }
          p[rr][e] = acc;
        }
      }
    }
  }
  // transpose-reduce: halve the expert window over lane bits 5, 4, 3, then sum over bits 2..0
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
#pragma unroll
    for (int sft = 32, win = 4; sft >= 8; sft >>= 1, win >>= 1) {
      const bool up = (lane & sft) != 0;
#pragma unroll
      for (int j = 0; j < win; ++j) {
        const float keep = up ? p[rr][win + j] : p[rr][j];
        const float give = up ? p[rr][j] : p[rr][win + j];
        p[rr][j] = keep + __shfl_xor(give, sft, 64);
      }
    }
    p[rr][0] += __shfl_xor(p[rr][0], 4, 64);
    p[rr][0] += __shfl_xor(p[rr][0], 2, 64);
    p[rr][0] += __shfl_xor(p[rr][0], 1, 64);
    if ((lane & 7) == 0 && 8 * w + (lane >> 3) < 64) lg[rr][8 * w + (lane >> 3)] = p[rr][0];
  }
  __syncthreads();
  if (w >= nr) return;
  const long r = r0 + w;
  const float logit = (lane < n_exp) ? lg[w][lane] : -INFINITY;
  float vv = logit, my_val = -INFINITY, first = -INFINITY;
  int my_idx = 0;
  for (int j = 0; j < top_k; ++j) {
    float bv = vv;
    int bi = lane;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (j == 0) first = bv;
    if (lane == j) { my_val = bv; my_idx = bi; }
    if (lane == bi) vv = -INFINITY;
  }
  const float e = (lane < top_k) ? expf(my_val - first) : 0.f;
  const float zsum = wave_sum(e);
  if (lane < top_k) {
    idx[r * top_k + lane] = my_idx;
    gates[r * top_k + lane] = e / zsum;
  }
}

}  // namespace

void launch_embed(const int32_t* tok, const uint16_t* embed, float* h, int rows, int d, int vocab,
                  uint32_t* err, const float* gain, float eps, uint16_t* out, hipStream_t s) {
  const int nch = (d + 2047) / 2048;
  if (nch <= 1) hipLaunchKernelGGL(embed_kernel<1>, dim3(rows), dim3(256), 0, s, tok, embed, h, d, vocab, err, gain, eps, out);
  else if (nch <= 2) hipLaunchKernelGGL(embed_kernel<2>, dim3(rows), dim3(256), 0, s, tok, embed, h, d, vocab, err, gain, eps, out);
  else hipLaunchKernelGGL(embed_kernel<4>, dim3(rows), dim3(256), 0, s, tok, embed, h, d, vocab, err, gain, eps, out);
}

void launch_rmsnorm(const float* h, const float* gain, float eps, uint16_t* out, int rows, int d,
                    hipStream_t s) {
  const int nch = (d + 1023) / 1024;
  if (nch <= 2) hipLaunchKernelGGL(rmsnorm_kernel<2>, dim3(rows), dim3(256), 0, s, h, gain, eps, out, rows, d);
  else if (nch <= 4) hipLaunchKernelGGL(rmsnorm_kernel<4>, dim3(rows), dim3(256), 0, s, h, gain, eps, out, rows, d);
  else hipLaunchKernelGGL(rmsnorm_kernel<8>, dim3(rows), dim3(256), 0, s, h, gain, eps, out, rows, d);
}

void launch_f32_to_bf16(const float* in, uint16_t* out, long n, hipStream_t s) {
  const long blocks = (n + 1023) / 1024;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(blocks), dim3(256), 0, s, in, out, n);
}

void launch_norm_router(float* h, const float* part, int n_part, long part_stride,
                        const float* gain, float eps, const uint16_t* w_router, int rows, int d,
                        int n_exp, int top_k, uint16_t* b_out, int32_t* idx, float* gates,
                        hipStream_t s) {
  const int nch = (d + 2047) / 2048;
  // several rows per work-group once there are enough rows to fill the chip: the router
  // weights are then read once per group instead of once per row
  const int R = rows >= 2048 ? 8 : rows >= 1024 ? 4 : rows >= 512 ? 2 : 1;
#define DG_NR(N, RR)                                                                           \
  hipLaunchKernelGGL((norm_router_kernel<N, RR>), dim3((rows + RR - 1) / RR), dim3(512), 0, s, h, \
                     part, n_part, part_stride, gain, eps, w_router, d, n_exp, top_k, rows, b_out, \
                     idx, gates)
#define DG_NR_R(N)                \
  if (R == 8) DG_NR(N, 8);        \
  else if (R == 4) DG_NR(N, 4);   \
  else if (R == 2) DG_NR(N, 2);   \
  else DG_NR(N, 1)
  // LDS holds R float32 rows: R * nch <= 8 (64 KB)
  if (nch <= 1) { DG_NR_R(1); }
  else if (nch <= 2) { if (R >= 4) DG_NR(2, 4); else if (R == 2) DG_NR(2, 2); else DG_NR(2, 1); }
  else { if (R >= 2) DG_NR(4, 2); else DG_NR(4, 1); }
#undef DG_NR_R
#undef DG_NR
}

}  // namespace dg
