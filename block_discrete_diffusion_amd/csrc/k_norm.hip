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

// One wave per row; 4 rows per work-group.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h,
                                                      const float* __restrict__ gain, float eps,
                                                      uint16_t* __restrict__ out, int rows, int d) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const float* x = h + static_cast<long>(r) * d;
  float ss = 0.f;
  for (int c = lane * 4; c < d; c += 256) {
    const floatx4_t v = *reinterpret_cast<const floatx4_t*>(x + c);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
  for (int c = lane * 4; c < d; c += 256) {
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

constexpr int kRouterRows = 4;  // rows per work-group (one wave each)

// Work-group: 4 waves, 4 rows.  Phase 1: wave w normalises row w into LDS (fp32) and writes
// the bf16 copy.  Phase 2: wave w computes the logits of row w, lane e = expert e, streaming
// W_router row e (L2-resident) against the LDS row.  Phase 3: k rounds of wave arg-max.
__global__ __launch_bounds__(256) void norm_router_kernel(
    const float* __restrict__ h, const float* __restrict__ gain, float eps,
    const uint16_t* __restrict__ wr, int rows, int d, int n_exp, int top_k,
    uint16_t* __restrict__ b_out, int32_t* __restrict__ idx, float* __restrict__ gates) {
  extern __shared__ float xs[];  // [kRouterRows][d]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = blockIdx.x * kRouterRows + w;
  const bool live = r < rows;
  float* xr = xs + w * d;
  if (live) {
    const float* x = h + static_cast<long>(r) * d;
    float ss = 0.f;
    for (int c = lane * 4; c < d; c += 256) {
      const floatx4_t v = *reinterpret_cast<const floatx4_t*>(x + c);
      ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(d) + eps);
    for (int c = lane * 4; c < d; c += 256) {
      const floatx4_t v = *reinterpret_cast<const floatx4_t*>(x + c);
      const floatx4_t g = *reinterpret_cast<const floatx4_t*>(gain + c);
      const floatx4_t y = floatx4_t{v[0] * inv * g[0], v[1] * inv * g[1], v[2] * inv * g[2],
                                    v[3] * inv * g[3]};
      *reinterpret_cast<floatx4_t*>(xr + c) = y;
      *reinterpret_cast<u32x2_t*>(b_out + static_cast<long>(r) * d + c) =
          u32x2_t{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])};
    }
  }
  __syncthreads();
  if (!live) return;
  float logit = -INFINITY;
  if (lane < n_exp) {
    const uint16_t* we = wr + static_cast<long>(lane) * d;
    float acc = 0.f;
    for (int c = 0; c < d; c += 8) {
      const u32x4_t v = ld16(we + c);
      const floatx4_t x0 = *reinterpret_cast<const floatx4_t*>(xr + c);
      const floatx4_t x1 = *reinterpret_cast<const floatx4_t*>(xr + c + 4);
      acc += __uint_as_float(v[0] << 16) * x0[0];
      acc += __uint_as_float(v[0] & 0xffff0000u) * x0[1];
      acc += __uint_as_float(v[1] << 16) * x0[2];
      acc += __uint_as_float(v[1] & 0xffff0000u) * x0[3];
      acc += __uint_as_float(v[2] << 16) * x1[0];
      acc += __uint_as_float(v[2] & 0xffff0000u) * x1[1];
      acc += __uint_as_float(v[3] << 16) * x1[2];
      acc += __uint_as_float(v[3] & 0xffff0000u) * x1[3];
    }
    logit = acc;
  }
  // k rounds of wave arg-max; round j's winner is parked in lane j.
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

}  // namespace

void launch_embed(const int32_t* tok, const uint16_t* embed, float* h, int rows, int d,
                  hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3(rows), dim3(256), 0, s, tok, embed, h, d);
}

void launch_rmsnorm(const float* h, const float* gain, float eps, uint16_t* out, int rows, int d,
                    hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, h, gain, eps, out,
                     rows, d);
}

void launch_f32_to_bf16(const float* in, uint16_t* out, long n, hipStream_t s) {
  const long blocks = (n + 1023) / 1024;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(blocks), dim3(256), 0, s, in, out, n);
}

void launch_norm_router(const float* h, const float* gain, float eps, const uint16_t* w_router,
                        int rows, int d, int n_exp, int top_k, uint16_t* b_out, int32_t* idx,
                        float* gates, hipStream_t s) {
  const size_t lds = sizeof(float) * kRouterRows * d;
  hipLaunchKernelGGL(norm_router_kernel, dim3((rows + kRouterRows - 1) / kRouterRows), dim3(256),
                     lds, s, h, gain, eps, w_router, rows, d, n_exp, top_k, b_out, idx, gates);
}

}  // namespace dg
