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

__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tok,
                                                    const uint16_t* __restrict__ embed,
                                                    float* __restrict__ h, int d) {
  const int r = blockIdx.x;
  const long src = static_cast<long>(tok[r]) * d;
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    const u32x4_t v = ld16(embed + src + c);
    float o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(v[i] << 16);
      o[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
    float* dst = h + static_cast<long>(r) * d + c;
    *reinterpret_cast<floatx4_t*>(dst) = floatx4_t{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<floatx4_t*>(dst + 4) = floatx4_t{o[4], o[5], o[6], o[7]};
  }
}

// One work-group (4 waves) per row; each thread normalises 4-element chunks.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h,
                                                      const float* __restrict__ gain, float eps,
                                                      uint16_t* __restrict__ out, int rows, int d) {
  __shared__ float red[4];
  const int r = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float* x = h + static_cast<long>(r) * d;
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    const floatx4_t v = *reinterpret_cast<const floatx4_t*>(x + c);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = wave_sum(ss);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  ss = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    const floatx4_t v = *reinterpret_cast<const floatx4_t*>(x + c);
    const floatx4_t g = *reinterpret_cast<const floatx4_t*>(gain + c);
    *reinterpret_cast<u32x2_t*>(out + static_cast<long>(r) * d + c) =
        u32x2_t{pack_bf2(v[0] * inv * g[0], v[1] * inv * g[1]),
                pack_bf2(v[2] * inv * g[2], v[3] * inv * g[3])};
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

constexpr int kRouterRows = 16;  // rows per work-group (one MFMA column tile)

// FFN norm + router + top-k.  Work-group: 16 rows, 4 waves.
//  1. wave w normalises rows w, w+4, .. (float32), writes their bf16 copy (the experts' input)
//     and keeps 1/rms in LDS;
//  2. router logits on MFMA: the float32 normed row x is split into bf16 parts x = hi + lo
//     (lo = bf16(x - hi), so the split is exact to ~2^-18 relative) and W x = W hi + W lo with
//     fp32 accumulation: bf16 x bf16 products are exact, so the logits carry float32-level error,
//     not bf16-level.  Wave w covers a quarter of d for all experts; the four partial logit
//     tiles are summed in LDS in wave order;
//  3. wave w takes rows w, w+4, ..: lane e = expert e, k rounds of wave arg-max (ties to the
//     lower expert index), softmax gates over the k picks.
__global__ __launch_bounds__(256) void norm_router_kernel(
    const float* __restrict__ h, const float* __restrict__ gain, float eps,
    const uint16_t* __restrict__ wr, int rows, int d, int n_exp, int top_k,
    uint16_t* __restrict__ b_out, int32_t* __restrict__ idx, float* __restrict__ gates) {
  __shared__ float inv_s[kRouterRows];
  __shared__ float lg[4][kRouterRows][65];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j4 = lane >> 4, l16 = lane & 15;
  const int r0 = blockIdx.x * kRouterRows;
  // 1. norms
  for (int rr = w; rr < kRouterRows; rr += 4) {
    const int r = r0 + rr;
    if (r >= rows) break;
    const float* x = h + static_cast<long>(r) * d;
    float ss = 0.f;
    for (int c = lane * 4; c < d; c += 256) {
      const floatx4_t v = *reinterpret_cast<const floatx4_t*>(x + c);
      ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
    if (lane == 0) inv_s[rr] = inv;
    for (int c = lane * 4; c < d; c += 256) {
      const floatx4_t v = *reinterpret_cast<const floatx4_t*>(x + c);
      const floatx4_t g = *reinterpret_cast<const floatx4_t*>(gain + c);
      *reinterpret_cast<u32x2_t*>(b_out + static_cast<long>(r) * d + c) =
          u32x2_t{pack_bf2(v[0] * inv * g[0], v[1] * inv * g[1]),
                  pack_bf2(v[2] * inv * g[2], v[3] * inv * g[3])};
    }
  }
  __syncthreads();
  // 2. logits: A = W_router rows (experts), B = normed rows split hi/lo
  const int row = r0 + l16;
  const bool row_ok = row < rows;
  const float inv = row_ok ? inv_s[l16] : 0.f;
  const float* xr = h + static_cast<long>(row_ok ? row : 0) * d;
  floatx4_t acc[4];
#pragma unroll
  for (int et = 0; et < 4; ++et) acc[et] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  const int kq = d / 4;  // this wave's quarter of the model dimension (a multiple of 16)
  // two-stage register pipeline over 32-wide k steps: step n+1's loads are issued before step
  // n's conversions and MFMAs
  floatx4_t xa[2][2], ga[2][2];
  u32x4_t wa[2][4];
  auto load = [&](int b, int k) {
    const int kk = k + 8 * j4;
    xa[b][0] = row_ok ? *reinterpret_cast<const floatx4_t*>(xr + kk) : floatx4_t{0.f, 0.f, 0.f, 0.f};
    xa[b][1] = row_ok ? *reinterpret_cast<const floatx4_t*>(xr + kk + 4) : floatx4_t{0.f, 0.f, 0.f, 0.f};
    ga[b][0] = *reinterpret_cast<const floatx4_t*>(gain + kk);
    ga[b][1] = *reinterpret_cast<const floatx4_t*>(gain + kk + 4);
#pragma unroll
    for (int et = 0; et < 4; ++et) {
      const int e = et * 16 + l16;
      wa[b][et] = (e < n_exp) ? ld16(wr + static_cast<long>(e) * d + kk) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto compute = [&](int b) {
    u32x4_t hi, lo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int hh = q >> 1, sub = (q & 1) * 2;
      const float v0 = xa[b][hh][sub] * inv * ga[b][hh][sub];
      const float v1 = xa[b][hh][sub + 1] * inv * ga[b][hh][sub + 1];
      const uint32_t hp = pack_bf2(v0, v1);
      hi[q] = hp;
      lo[q] = pack_bf2(v0 - __uint_as_float(hp << 16), v1 - __uint_as_float(hp & 0xffff0000u));
    }
#pragma unroll
    for (int et = 0; et < 4; ++et) {
      acc[et] = mfma16(wa[b][et], hi, acc[et]);
      acc[et] = mfma16(wa[b][et], lo, acc[et]);
    }
  };
  const int kb = w * kq, ke = kb + kq;
  if (kq > 0) load(0, kb);
  for (int k = kb; k < ke; k += 64) {
    if (k + 32 < ke) load(1, k + 32);
    compute(0);
    if (k + 64 < ke) load(0, k + 64);
    if (k + 32 < ke) compute(1);
  }
  // lane holds logit[expert et*16 + 4*j4 + i][row l16] (partial over this wave's quarter)
#pragma unroll
  for (int et = 0; et < 4; ++et)
#pragma unroll
    for (int i = 0; i < 4; ++i) lg[w][l16][et * 16 + 4 * j4 + i] = acc[et][i];
  __syncthreads();
  // 3. top-k per row
  for (int rr = w; rr < kRouterRows; rr += 4) {
    const int r = r0 + rr;
    if (r >= rows) break;
    const float logit = (lane < n_exp)
        ? ((lg[0][rr][lane] + lg[1][rr][lane]) + lg[2][rr][lane]) + lg[3][rr][lane] : -INFINITY;
    float v = logit, my_val = -INFINITY, first = -INFINITY;
    int my_idx = 0;
    for (int j = 0; j < top_k; ++j) {
      float bv = v;
      int bi = lane;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if (j == 0) first = bv;
      if (lane == j) { my_val = bv; my_idx = bi; }
      if (lane == bi) v = -INFINITY;
    }
    const float e = (lane < top_k) ? expf(my_val - first) : 0.f;
    const float z = wave_sum(e);
    if (lane < top_k) {
      idx[static_cast<long>(r) * top_k + lane] = my_idx;
      gates[static_cast<long>(r) * top_k + lane] = e / z;
    }
  }
}

}  // namespace

void launch_embed(const int32_t* tok, const uint16_t* embed, float* h, int rows, int d,
                  hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3(rows), dim3(256), 0, s, tok, embed, h, d);
}

void launch_rmsnorm(const float* h, const float* gain, float eps, uint16_t* out, int rows, int d,
                    hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, s, h, gain, eps, out, rows, d);
}

void launch_f32_to_bf16(const float* in, uint16_t* out, long n, hipStream_t s) {
  const long blocks = (n + 1023) / 1024;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(blocks), dim3(256), 0, s, in, out, n);
}

void launch_norm_router(const float* h, const float* gain, float eps, const uint16_t* w_router,
                        int rows, int d, int n_exp, int top_k, uint16_t* b_out, int32_t* idx,
                        float* gates, hipStream_t s) {
  hipLaunchKernelGGL(norm_router_kernel, dim3((rows + kRouterRows - 1) / kRouterRows), dim3(256), 0,
                     s, h, gain, eps, w_router, rows, d, n_exp, top_k, b_out, idx, gates);
}

}  // namespace dg
