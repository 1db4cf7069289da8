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
//  - every load of the norm phase is issued at once (rows past the end of the matrix re-read
//    the last row; nothing of theirs is stored), the split-K slices with them for one row and
//    one slice at a time for several, and then the router weights of the first NB 512-column
//    chunks, whose latency hides behind the norm;
//  - h += slices (z order, written back); x = h * rsqrt(mean h^2 + eps) * gain in float32;
//    the bf16 copy of x feeds the experts and the float32 x is kept in LDS; h and the bf16 x
//    are stored after the norm's last barrier;
//  - router logits in float32: wave w owns experts 8w .. 8w+7; lane l owns the row elements
//    [8 (l + 64 j), +8) of 512-column chunk j (coalesced 16-byte reads: a wave covers 1 KB of
//    one expert row per request).  Each chunk's weights are widened to float32 once and used
//    for all R rows; chunk j + NB is requested as soon as chunk j is widened (NB register
//    sets).  The eight partials of a row are summed over the wave by a transpose-reduce
//    (three exchange steps halving the expert window, then three plain steps), after which
//    lane l holds expert 8w + (l >> 3);
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

  // norm inputs: gain, rows, then the slices (lanes past d load nothing and hold zeros)
  floatx4_t gv[NCH], v[R][NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = (tid + 512 * i) * 4;
    gv[i] = c < d ? *reinterpret_cast<const floatx4_t*>(gain + c) : floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    const long row = min(r0 + rr, rows - 1);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = (tid + 512 * i) * 4;
      v[rr][i] = c < d ? *reinterpret_cast<const floatx4_t*>(h + row * d + c) : floatx4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
  if constexpr (R == 1) {
    // one row: every slice is requested at once (slices past n_part re-read the last one and
    // are not added; with no slices, the row itself)
    floatx4_t pz[kMaxParts][NCH];
#pragma unroll
    for (int z = 0; z < kMaxParts; ++z)
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = (tid + 512 * i) * 4;
        const float* src = n_part > 0 ? part + min(z, n_part - 1) * part_stride + static_cast<long>(r0) * d
                                      : h + static_cast<long>(r0) * d;
        pz[z][i] = c < d ? *reinterpret_cast<const floatx4_t*>(src + c) : floatx4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int z = 0; z < kMaxParts; ++z)
#pragma unroll
      for (int i = 0; i < NCH; ++i)
        if (z < n_part) v[0][i] += pz[z][i];
  } else {
    for (int z = 0; z < n_part; ++z) {
      floatx4_t pz[R][NCH];
#pragma unroll
      for (int rr = 0; rr < R; ++rr) {
        const long row = min(r0 + rr, rows - 1);
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const int c = (tid + 512 * i) * 4;
          pz[rr][i] = c < d ? *reinterpret_cast<const floatx4_t*>(part + z * part_stride + row * d + c)
                            : floatx4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int i = 0; i < NCH; ++i) v[rr][i] += pz[rr][i];
    }
  }
  // router weights of chunk j (8 experts of this wave); NB register sets: with one row all
  // four chunks of a 2048-wide row are requested before the norm
  constexpr int NB = (R == 1) ? 4 : 2;
  u32x4_t wv[NB][8];
  auto load_w = [&](u32x4_t (&dst)[8], int j) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = min((lane + 64 * j) * 8, d - 8);  // clamped: always in bounds
      const int ee = min(8 * w + e, n_exp - 1);
      dst[e] = ld16(wr + static_cast<long>(ee) * d + c);
    }
  };
#pragma unroll
  for (int b = 0; b < NB; ++b) load_w(wv[b], min(b, nj - 1));

#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
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

  // router: 8 experts per wave, one 512-column chunk at a time
  float p[R][8];
#pragma unroll
  for (int rr = 0; rr < R; ++rr)
#pragma unroll
    for (int e = 0; e < 8; ++e) p[rr][e] = 0.f;
  float wf[8][8];
  auto widen = [&](const u32x4_t (&src)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wf[e][2 * q] = __uint_as_float(src[e][q] << 16);
        wf[e][2 * q + 1] = __uint_as_float(src[e][q] & 0xffff0000u);
      }
  };
  auto dot = [&](int j) {
    const int c = (lane + 64 * j) * 8;
    if (c >= d) return;  // lanes past d add nothing
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      const floatx4_t x0 = *reinterpret_cast<const floatx4_t*>(&xs[rr][c]);
      const floatx4_t x1 = *reinterpret_cast<const floatx4_t*>(&xs[rr][c + 4]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float acc = p[rr][e];
#pragma unroll
        for (int k = 0; k < 4; ++k) acc += wf[e][k] * x0[k];
#pragma unroll
        for (int k = 0; k < 4; ++k) acc += wf[e][4 + k] * x1[k];
        p[rr][e] = acc;
      }
    }
  };
  for (int j = 0; j < nj; j += NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (j + b >= nj) break;  // uniform
      widen(wv[b]);
      if (j + b + NB < nj) load_w(wv[b], j + b + NB);  // uniform
      dot(j + b);
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

// Router weights in MFMA A-fragment order for norm_router_mfma_kernel: fragment (k-step S,
// 16-expert tile t) holds for lane (l16, j4) the 8 weights W[min(16 t + l16, n_exp - 1)][32 S +
// 8 j4 .. + 8], stored [S][t][lane] so that a wave reads each fragment as one 1 KB run.  One
// thread per 16-byte piece.
__global__ __launch_bounds__(256) void router_pack_kernel(const uint16_t* __restrict__ w, int n_exp,
                                                          int d, uint16_t* __restrict__ out) {
  const long c = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= static_cast<long>(d / 32) * 4 * 64) return;
  const int lane = static_cast<int>(c % 64), t = static_cast<int>((c / 64) % 4);
  const long S = c / 256;
  const long e = min(16 * t + (lane & 15), n_exp - 1);
  st16(out + c * 8, ld16(w + e * d + 32 * S + 8 * (lane >> 4)));
}

// The same step (residual update, FFN norm, router, top-k, gates) with the router logits on
// MFMA, for d = 32 NW SPW, one work-group of NW waves per RW = 16 or 8 rows (8 where 16-row groups
// would leave CUs idle: every group reads the whole router matrix, so the CUs' load rate, not
// HBM, sets the pace).  The MFMA tiles stay 16 rows wide; with RW = 8, lanes l16 >= 8 repeat
// the rows of lanes l16 - 8 (the same addresses: no extra traffic) and store nothing.  Lane
// (l16, j4) of wave w takes row l16 % RW of the group and, in each of its SPW 32-column k-steps s, the columns
// 32 (w SPW + s) + 8 j4 .. + 8: exactly the MFMA B-operand fragment of those rows, so the normed
// row never goes through LDS.  The normed float32 x is split into bf16 hi = bf16(x) (the copy
// the experts read) and lo = bf16(x - hi), and each 16 x 16 logit tile is W hi + W lo with
// float32 accumulation: hi + lo carries x to about 2^-17 relative, so the logits stay within
// float32 rounding of W x.  The router weights are the A operand, read from the fragment-
// ordered copy (one 1 KB run per wave and fragment).
//  - loads: the wave's router weights (cold in HBM) first, then the rows (slices added in z
//    order, one slice at a time), with WH = 2 the second half of the weights only then (the
//    registers hold one half next to a row slice), and the gain (through LDS: lanes of equal
//    j4 share it);
//  - row sums of squares: per lane, over the four j4 lanes of a row, then over the waves in
//    LDS in a fixed order; with slices, h += slices is written back;
//  - the per-wave partial logit tiles go to LDS and are summed over the waves in a fixed order;
//    expert e's rank in its row = #experts with a larger logit or an equal one at a lower index
//    (the order of repeated arg-max with ties to the lower index); ranks < k are the picks, in
//    order, and the gates a softmax over them (exponents relative to the largest logit).
template <int NW>
DG_DEVICE float wave_tree_sum(const float* v, int stride) {  // v[i * stride], i < NW, fixed order
  if constexpr (NW == 1) return v[0];
  else return wave_tree_sum<NW / 2>(v, stride) + wave_tree_sum<NW / 2>(v + (NW / 2) * stride, stride);
}

template <int NW, int SPW, int WH, int RW>  // WH: the weights come in WH parts (2: the second after the rows)
__global__ __launch_bounds__(64 * NW) void norm_router_mfma_kernel(
    float* __restrict__ h, const float* __restrict__ part, int n_part, long part_stride,
    const float* __restrict__ gain, float eps, const uint16_t* __restrict__ wp, int d, int n_exp,
    int top_k, int rows, uint16_t* __restrict__ bout, int32_t* __restrict__ idx,
    float* __restrict__ gates) {
  constexpr int R = 16, NT = 4;  // rows of an MFMA tile, 16-expert tiles
  static_assert(R % NW == 0 || NW % R == 0, "rows split over the waves");
  static_assert(RW == 16 || RW == 8, "rows per work-group");
  __shared__ float red[NW][R];
  __shared__ float plg[NW][NT * 16][R + 1];
  __shared__ __align__(16) float lg[R][64];
  __shared__ __align__(16) float gs[NW * SPW * 32];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, j4 = lane >> 4;
  const int r0 = blockIdx.x * RW;
  const bool own = l16 < RW && r0 + l16 < rows;
  const long row = min(r0 + l16 % RW, rows - 1);  // rows past the end re-read the last one
  const int kc0 = w * SPW * 32 + 8 * j4;     // this lane's first column; k-step s adds 32 s

  constexpr int SH = SPW / WH;  // k-steps per part of the weights
  floatx4_t hv[SPW][2];
  u32x4_t wa[WH][NT][SH];
  auto load_w = [&](int part_w) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int s = 0; s < SH; ++s)
        wa[part_w][t][s] = ld16(wp + ((static_cast<long>(w * SPW + part_w * SH + s) * NT + t) * 64 + lane) * 8);
  };
  // the router weights first (cold in HBM): the wait for the rows then covers them too
  load_w(0);
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int q = 0; q < 2; ++q) hv[s][q] = *reinterpret_cast<const floatx4_t*>(h + row * d + kc0 + 32 * s + 4 * q);
  for (int z = 0; z < n_part; ++z) {
    floatx4_t pz[SPW][2];
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        pz[s][q] = *reinterpret_cast<const floatx4_t*>(part + z * part_stride + row * d + kc0 + 32 * s + 4 * q);
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
      for (int q = 0; q < 2; ++q) hv[s][q] += pz[s][q];
  }
  if constexpr (WH == 2) load_w(1);
  // the gain goes to LDS (each thread a slice), to be read per k-step: lanes of equal j4 share it
  constexpr int GPT = (32 * SPW + 63) / 64;  // gain floats per thread (some idle when SPW = 1)
  constexpr int DW = NW * SPW * 32;          // = d
  float gt[GPT];
#pragma unroll
  for (int i = 0; i < GPT; ++i) gt[i] = tid * GPT + i < DW ? gain[tid * GPT + i] : 0.f;
#pragma unroll
  for (int i = 0; i < GPT; ++i)
    if (tid * GPT + i < DW) gs[tid * GPT + i] = gt[i];

  float ss = 0.f;
#pragma unroll
  for (int s = 0; s < SPW; ++s)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) ss += hv[s][q][i] * hv[s][q][i];
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  if (j4 == 0) red[w][l16] = ss;
  if (n_part > 0 && own) {
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
      for (int q = 0; q < 2; ++q) *reinterpret_cast<floatx4_t*>(h + row * d + kc0 + 32 * s + 4 * q) = hv[s][q];
  }
  __syncthreads();
  const float inv = 1.0f / sqrtf(wave_tree_sum<NW>(&red[0][l16], R) / static_cast<float>(d) + eps);

  floatx4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    float x[8];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const floatx4_t g = *reinterpret_cast<const floatx4_t*>(&gs[kc0 + 32 * s + 4 * q]);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * q + i] = hv[s][q][i] * inv * g[i];
    }
    u32x4_t bhi, blo;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      bhi[p] = pack_bf2(x[2 * p], x[2 * p + 1]);
      const float h0 = __uint_as_float(bhi[p] << 16), h1 = __uint_as_float(bhi[p] & 0xffff0000u);
      blo[p] = pack_bf2(x[2 * p] - h0, x[2 * p + 1] - h1);
    }
    if (own) *reinterpret_cast<u32x4_t*>(bout + row * d + kc0 + 32 * s) = bhi;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      acc[t] = mfma16(wa[s / SH][t][s % SH], bhi, acc[t]);
      acc[t] = mfma16(wa[s / SH][t][s % SH], blo, acc[t]);
    }
  }
  // partial logits: lane holds experts 16 t + 4 j4 + i of row l16
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) plg[w][16 * t + 4 * j4 + i][l16] = acc[t][i];
  __syncthreads();
  // logits (lane = expert); experts past n_exp and NaN logits count as -inf
  constexpr int RPW = R / NW > 0 ? R / NW : 1;  // rows per wave
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int rr = w + NW * k;
    if (rr >= R) break;
    float lv = -INFINITY;
    if (lane < n_exp) {
      lv = wave_tree_sum<NW>(&plg[0][lane][rr], NT * 16 * (R + 1));
      if ((__float_as_uint(lv) & 0x7fffffffu) > 0x7f800000u) lv = -INFINITY;
    }
    lg[rr][lane] = lv;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int rr = w + NW * k;
    if (rr >= RW || r0 + rr >= rows) break;  // uniform
    const float mine = lg[rr][lane];
    float top = -INFINITY;
    int rank = 0;
#pragma unroll
    for (int jb = 0; jb < 16; ++jb) {
      const floatx4_t v = *reinterpret_cast<const floatx4_t*>(&lg[rr][4 * jb]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * jb + i;
        rank += (v[i] > mine || (v[i] == mine && j < lane)) ? 1 : 0;
        top = fmaxf(top, v[i]);
      }
    }
    const bool pick = rank < top_k;
    const float e = pick ? expf(mine - top) : 0.f;
    const float zsum = wave_sum(e);
    if (pick) {
      const long r = r0 + rr;
      idx[r * top_k + rank] = lane;
      gates[r * top_k + rank] = e / zsum;
    }
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

bool router_mfma_path(int d, int n_exp) {
  return d % 256 == 0 && d <= 2048 && n_exp <= 64;
}

void launch_router_pack(const uint16_t* w_router, int n_exp, int d, uint16_t* out, hipStream_t s) {
  const long n = static_cast<long>(d / 32) * 4 * 64;
  hipLaunchKernelGGL(router_pack_kernel, dim3((n + 255) / 256), dim3(256), 0, s, w_router, n_exp, d, out);
}

void launch_norm_router(float* h, const float* part, int n_part, long part_stride,
                        const float* gain, float eps, const uint16_t* w_router,
                        const uint16_t* w_router_packed, int rows, int d, int n_exp, int top_k,
                        uint16_t* b_out, int32_t* idx, float* gates, hipStream_t s) {
#define DG_NRM_R(NW, SPW, WH, RW)                                                                   \
  hipLaunchKernelGGL((norm_router_mfma_kernel<NW, SPW, WH, RW>), dim3((rows + RW - 1) / RW), dim3(64 * NW), 0, \
                     s, h, part, n_part, part_stride, gain, eps, w_router_packed, d, n_exp, top_k, rows,    \
                     b_out, idx, gates)
  // 8 rows per work-group while 16-row groups would not give every CU one
#define DG_NRM(NW, SPW, WH)                                  \
  if ((rows + 15) / 16 < 256) DG_NRM_R(NW, SPW, WH, 8);      \
  else DG_NRM_R(NW, SPW, WH, 16)
  // the MFMA router from 1024 rows (64 work-groups and more); below that a work-group per row
  if (w_router_packed && rows >= 1024 && router_mfma_path(d, n_exp)) {
    switch (d / 256) {  // 16 waves at 512 and 1024 columns, else 8 (registers)
      case 1: DG_NRM(8, 1, 1); return;
      case 2: DG_NRM(16, 1, 1); return;
      case 4: DG_NRM(16, 2, 1); return;
      case 8: DG_NRM(8, 8, 2); return;
      default: break;
    }
  }
#undef DG_NRM
#undef DG_NRM_R
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
