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
// Stable sort of the routes r = t*top_k + j by (expert, r), one work-group of 8 waves per expert
// e.  Wave w owns the contiguous routes [w S, (w + 1) S) (S a multiple of 64): in a first
// sweep it counts, with two ballots per 64 routes, the routes of expert e and of lower experts;
// one barrier shares the eight counts, which give offs[e] (all routes of lower experts) and
// the routes of e in earlier waves; a second sweep places the wave's routes of e in route
// order.  Each sweep requests up to kPermBatch groups of 64 routes at once.
constexpr int kPermWaves = 8, kPermBatch = 16;
__global__ __launch_bounds__(64 * kPermWaves) void moe_permute_kernel(const int32_t* __restrict__ idx,
                                                                     int n, int n_exp,
                                                                     int32_t* __restrict__ offs,
                                                                     int32_t* __restrict__ perm,
                                                                     int32_t* __restrict__ inv) {
  __shared__ int wc[2][kPermWaves];
  const int e = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int per = (n + 64 * kPermWaves - 1) / (64 * kPermWaves);  // groups of 64 per wave
  const int g0 = w * per;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int c_eq = 0, c_lt = 0;
  for (int gb = 0; gb < per; gb += kPermBatch) {
    int ex[kPermBatch];
#pragma unroll
    for (int i = 0; i < kPermBatch; ++i) {
      const int r = (g0 + gb + i) * 64 + lane;
      ex[i] = (gb + i < per && r < n) ? idx[r] : 0x7fffffff;
    }
#pragma unroll
    for (int i = 0; i < kPermBatch; ++i) {
      c_eq += __popcll(__ballot(ex[i] == e));
      c_lt += __popcll(__ballot(ex[i] < e));
    }
  }
  if (lane == 0) {
    wc[0][w] = c_eq;
    wc[1][w] = c_lt;
  }
  __syncthreads();
  int run = 0, p0 = 0;
  for (int v = 0; v < kPermWaves; ++v) {
    if (v < w) run += wc[0][v];
    p0 += wc[1][v];
  }
  if (threadIdx.x == 0) {
    offs[e] = p0;
    if (e == n_exp - 1) offs[n_exp] = n;
  }
  for (int gb = 0; gb < per; gb += kPermBatch) {
    int ex[kPermBatch];
#pragma unroll
    for (int i = 0; i < kPermBatch; ++i) {
      const int r = (g0 + gb + i) * 64 + lane;
      ex[i] = (gb + i < per && r < n) ? idx[r] : 0x7fffffff;
    }
#pragma unroll
    for (int i = 0; i < kPermBatch; ++i) {
      const unsigned long long eq = __ballot(ex[i] == e);
      if (ex[i] == e) {
        const int r = (g0 + gb + i) * 64 + lane;
        const int p = p0 + run + __popcll(eq & below);
        perm[p] = r;
        inv[r] = p;
      }
      run += __popcll(eq);
    }
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
template <bool GATED, int TT, int KS, int FPW, bool F8, bool FUSED, int SG>
__global__ __launch_bounds__(256 * SG) void expert_stream_kernel(MoeArgs a) {
  static_assert(!FUSED || GATED, "only the gate/up projection ranks the routes itself");
  static_assert(!FUSED || SG == 1, "the route ranking assumes four waves");
  constexpr int NA = GATED ? 2 : 1;
  constexpr int GT = 4 * FPW;  // tiles per packed group = tiles of one four-wave subgroup
  static_assert(!F8 || KS == 2, "E4M3 fragments come in pairs of k-steps");
  constexpr int NTH = 256 * SG;
  constexpr int KC = 32 * KS, ROWS = TT * 16, LDX = KC + 8, CPR = KC / 8;
  constexpr int PIECES = ROWS * CPR, PPT = (PIECES + NTH - 1) / NTH;
  __shared__ uint16_t xs[2][ROWS * LDX];
  // this expert's routes, in route order (only when the kernel ranks them itself: the array
  // would otherwise cost a work-group slot per CU at the largest row tiles)
  __shared__ int rl[FUSED ? kFusedRoutes : 1];
  __shared__ int wc[2][4];
  const int e = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wq = w & 3, sg = w >> 2;  // wave of subgroup sg, which streams packed group G SG + sg
  const int j4 = lane >> 4, l16 = lane & 15;
  const int grp = blockIdx.x * SG + sg;
  const int ft0 = grp * GT + wq * FPW;
  const int S = a.K / 32, nch = S / KS;
  const long wgrp = static_cast<long>(e) * (a.N / (16 * GT)) + grp;  // packed tile group
  const uint16_t* wp = F8 ? nullptr : a.wp + (wgrp * S * GT + wq * FPW) * NA * 512 + lane * 8;
  const uint8_t* wp8 = F8 ? a.wp8 + ((wgrp * (S / 2) * GT + wq * FPW) * NA * 64 + lane) * 16 : nullptr;
  // bf16: one 16-byte fragment per (k-step, tile, matrix); E4M3: one 16-byte load holds the
  // fragments of both k-steps of the chunk, widened to bf16 (exactly) right before the MFMA
  constexpr int WS = F8 ? 1 : KS;
  u32x4_t fw[2][WS][FPW][NA];
  auto load_w = [&](int b, int c) {
#pragma unroll
    for (int ks = 0; ks < WS; ++ks)
#pragma unroll
      for (int f = 0; f < FPW; ++f)
#pragma unroll
        for (int q = 0; q < NA; ++q) {
          if constexpr (F8) fw[b][ks][f][q] = ld16_nt(wp8 + ((c * GT + f) * NA + q) * 1024);
          else fw[b][ks][f][q] = ld16_nt(wp + (((c * KS + ks) * GT + f) * NA + q) * 512);
        }
  };
  int p0, n_e;
  constexpr bool fused = FUSED;  // the launch picks it when a.idx is set
  if (fused) {
    // rank this expert's routes from the router's choices: p0 = routes of lower experts, and
    // the routes of expert e in route order, i.e. the order of a stable sort by (expert,
    // route).  Wave w owns routes [64 PER w, 64 PER (w+1)); all its loads are issued at once,
    // then ballots count and place them (two barriers in all)
    constexpr int PER = kFusedRoutes / 256;
    const unsigned long long below_lane = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int ex[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int r = (w * PER + i) * 64 + lane;
      ex[i] = (r < a.n_routes) ? a.idx[r] : 0x7fffffff;
    }
    int c_eq = 0, c_lt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      c_eq += __popcll(__ballot(ex[i] == e));
      c_lt += __popcll(__ballot(ex[i] < e));
    }
    if (lane == 0) {
      wc[0][w] = c_eq;
      wc[1][w] = c_lt;
    }
    __syncthreads();
    int run = 0;
    for (int v = 0; v < w; ++v) run += wc[0][v];
    n_e = (wc[0][0] + wc[0][1]) + (wc[0][2] + wc[0][3]);
    p0 = (wc[1][0] + wc[1][1]) + (wc[1][2] + wc[1][3]);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const unsigned long long eq = __ballot(ex[i] == e);
      if (ex[i] == e) rl[run + __popcll(eq & below_lane)] = (w * PER + i) * 64 + lane;
      run += __popcll(eq);
    }
    __syncthreads();
    if (blockIdx.x == 0 && blockIdx.z == 0) {
      if (tid == 0) {
        a.offs_w[e] = p0;
        if (e == a.n_exp - 1) a.offs_w[a.n_exp] = a.n_routes;
      }
      for (int j = tid; j < n_e; j += 256) {
        a.perm_w[p0 + j] = rl[j];
        a.inv_w[rl[j]] = p0 + j;
      }
    }
  } else {
    p0 = a.offs[e];
    n_e = a.offs[e + 1] - p0;
  }
  if (n_e == 0) return;  // uniform over the work-group

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
      const int piece = tid + NTH * j, pc = min(piece, PIECES - 1);
      const int r = pc / CPR, col = (pc % CPR) * 8;
      const int rr = min(ps + r, n_e - 1);
      const long row = GATED ? ((fused ? rl[rr] : a.perm[p0 + rr]) / a.top_k) : static_cast<long>(p0 + rr);
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
    u32x4_t xr[PPT];
    auto frag = [&](int b, int ks, int f, int q) -> u32x4_t {
      if constexpr (F8) {
        const u32x4_t v = fw[b][0][f][q];
        const uint32_t lo = v[2 * ks], hi = v[2 * ks + 1];
        return u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
                       __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
                       __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
                       __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
      } else {
        return fw[b][ks][f][q];
      }
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
            for (int q = 0; q < NA; ++q) acc[f][q][t] = mfma16(frag(b, ks, f, q), xf, acc[f][q][t]);
          // with several subgroups (fewer registers per wave) the fragment reads go in pairs
          // of tiles instead of all ahead of the products
          if constexpr (SG > 1) {
            if (t % 2 == 1) sched_fence();
          }
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
    // E4M3: the per-channel scale multiplies the finished sums (scale * sum q x)
    if constexpr (F8) {
#pragma unroll
      for (int f = 0; f < FPW; ++f)
#pragma unroll
        for (int q = 0; q < NA; ++q) {
          const float* sp = (q == 0 ? a.wscale0 : a.wscale1) + static_cast<long>(e) * a.N + (ft0 + f) * 16 + 4 * j4;
          const floatx4_t sc = *reinterpret_cast<const floatx4_t*>(sp);
#pragma unroll
          for (int t = 0; t < TT; ++t) acc[f][q][t] *= sc;
        }
    }
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
          const floatx4_t v = acc[f][0][t];
          *reinterpret_cast<u32x2_t*>(a.out_bf16 + orow) = u32x2_t{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
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

// E4M3 byte layout: one thread per 16-byte piece [e][fg][k-step pair s2][tile w][matrix q][lane],
// bytes 0-7 = W_q[e][16 ft + l % 16][64 s2 + 8 (l / 16) .. + 8], bytes 8-15 the same 32 columns
// further (k-step 2 s2 + 1); tile ft = gt fg + w.
__global__ __launch_bounds__(256) void moe_pack_fp8_kernel(const uint8_t* __restrict__ q0,
                                                           const uint8_t* __restrict__ q1,
                                                           uint8_t* __restrict__ out, int n_exp,
                                                           int N, int K, int na, int gt) {
  const int S2 = K / 64, G = N / (16 * gt);
  const long total = static_cast<long>(n_exp) * G * S2 * gt * na * 64;
  const long c = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (c >= total) return;
  const int lane = static_cast<int>(c % 64);
  long r = c / 64;
  const int q = static_cast<int>(r % na);
  r /= na;
  const int w = static_cast<int>(r % gt);
  r /= gt;
  const int s2 = static_cast<int>(r % S2);
  r /= S2;
  const int fg = static_cast<int>(r % G);
  const long e = r / G;
  const int ft = gt * fg + w;
  const uint8_t* src = (q == 0 ? q0 : q1) + (e * N + ft * 16 + (lane & 15)) * static_cast<long>(K) +
                       s2 * 64 + 8 * (lane >> 4);
  const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(src);
  const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(src + 32);
  *reinterpret_cast<u32x4_t*>(out + c * 16) = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}

// OCP E4M3 encoding of a finite float32: 1 sign, 4 exponent (bias 7) and 3 mantissa bits, no
// infinities, largest finite 448; rounds to nearest with ties to even and saturates at 448.
DG_DEVICE uint32_t e4m3_encode(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float ax = fabsf(x);
  if (ax >= 448.0f) return sign | 0x7Eu;
  if (ax < 0x1p-6f)  // subnormal grid 2^-9; 8 steps round up to the smallest normal, code 0x08
    return sign | static_cast<uint32_t>(__builtin_rintf(ax * 512.0f));
  const uint32_t ab = bits & 0x7FFFFFFFu;
  int ex = static_cast<int>(ab >> 23) - 127;  // -6 .. 8
  uint32_t m = (ab >> 20) & 7u;
  const uint32_t rest = ab & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (m & 1u))) ++m;
  if (m == 8u) {
    m = 0;
    ++ex;
  }
  return sign | (static_cast<uint32_t>(ex + 7) << 3) | m;
}

// One work-group per row: scale = amax / 448 (1 for an all-zero row), q = E4M3(w / scale).
__global__ __launch_bounds__(256) void quantize_e4m3_kernel(const uint16_t* __restrict__ w, int cols,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  __shared__ float red[4];
  const long r = blockIdx.x;
  const int tid = threadIdx.x;
  const uint16_t* wr = w + r * cols;
  float amax = 0.f;
  for (int c = tid; c < cols; c += 256) amax = fmaxf(amax, fabsf(bf2f(wr[c])));
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
  if (tid == 0) scale[r] = sc;
  for (int c = tid; c < cols; c += 256) q[r * cols + c] = static_cast<uint8_t>(e4m3_encode(bf2f(wr[c]) / sc));
}

// Four bf16 values (two packed pairs) widened to float32, exactly.
DG_DEVICE floatx4_t bf4(const u32x2_t& p) {
  return floatx4_t{__uint_as_float(p[0] << 16), __uint_as_float(p[0] & 0xffff0000u),
                   __uint_as_float(p[1] << 16), __uint_as_float(p[1] & 0xffff0000u)};
}

// Un-permute + residual, one work-group (8 waves) per row t:
// h[t] += sum_z part_z[t] + sum_j gate[t][j] * y[inv[t*k+j]]   (z then j in order);
// with a gain it also writes the next block's normed input out = bf16(rmsnorm(h[t]) * gain),
// which saves a pass over h.  All of a thread's loads (the gain too) are issued before any
// arithmetic, and with a gain h is stored after the norm's barrier: a barrier after a global
// store waits for that store.  KJ routed slots (>= top_k up to 8) and NP slices (>= n_part) are
// loaded; the launch picks the smallest that hold the call's, so no load is made only to be
// dropped.
template <int NCH, int KJ, int NP>  // NCH: 4-element chunks per thread, ceil(d / 2048)
__global__ __launch_bounds__(512) void moe_combine_kernel(float* __restrict__ h,
                                                          const float* __restrict__ part,
                                                          int n_part, long part_stride,
                                                          const uint16_t* __restrict__ y,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ gates, int d,
                                                          int top_k, const float* __restrict__ gain,
                                                          float eps, uint16_t* __restrict__ out) {
  __shared__ float red[8];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float* hr = h + static_cast<long>(t) * d;
  static_assert(KJ == 4 || KJ == 8, "routed slots held in registers; more are read in the second loop");
  static_assert(NP >= 0 && NP <= kMaxParts, "split slices");
  // every load is unconditional (slots past top_k and slices past n_part re-read the last
  // valid one and are not added): loads under a condition would each get a wait of their own
  const int kl = min(top_k, KJ) - 1;
  int pj[KJ];
  float gj[KJ];
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    pj[j] = inv[static_cast<long>(t) * top_k + min(j, kl)];
    gj[j] = gates[static_cast<long>(t) * top_k + min(j, kl)];
  }
  constexpr int NPA = NP > 0 ? NP : 1;
  const float* zp[NPA];
#pragma unroll
  for (int z = 0; z < NPA; ++z)
    zp[z] = n_part > 0 ? part + min(z, n_part - 1) * part_stride + static_cast<long>(t) * d : hr;
  const float* gsrc = gain ? gain : hr;
  floatx4_t v[NCH], pz[NPA][NCH], gv[NCH];
  u32x2_t yj[KJ][NCH];  // four bf16 expert outputs each
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = min((tid + 512 * i) * 4, d - 4);  // clamped; chunks past d are not stored
    v[i] = *reinterpret_cast<const floatx4_t*>(hr + c);
    gv[i] = *reinterpret_cast<const floatx4_t*>(gsrc + c);
#pragma unroll
    for (int z = 0; z < NP; ++z) pz[z][i] = *reinterpret_cast<const floatx4_t*>(zp[z] + c);
#pragma unroll
    for (int j = 0; j < KJ; ++j) yj[j][i] = *reinterpret_cast<const u32x2_t*>(y + static_cast<long>(pj[j]) * d + c);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = (tid + 512 * i) * 4;
    floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int z = 0; z < NP; ++z)
      if (z < n_part) acc += pz[z][i];
#pragma unroll
    for (int j = 0; j < KJ; ++j)
      if (j < top_k) acc += gj[j] * bf4(yj[j][i]);
    for (int j = KJ; j < top_k; ++j) {
      const float g = gates[static_cast<long>(t) * top_k + j];
      const int p = inv[static_cast<long>(t) * top_k + j];
      acc += g * bf4(*reinterpret_cast<const u32x2_t*>(y + static_cast<long>(p) * d + min(c, d - 4)));
    }
    v[i] += acc;
    if (c < d) {
      if (!gain) *reinterpret_cast<floatx4_t*>(hr + c) = v[i];
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
    *reinterpret_cast<floatx4_t*>(hr + c) = v[i];
    const floatx4_t g = gv[i];
    *reinterpret_cast<u32x2_t*>(out + static_cast<long>(t) * d + c) =
        u32x2_t{pack_bf2(v[i][0] * rinv * g[0], v[i][1] * rinv * g[1]), pack_bf2(v[i][2] * rinv * g[2], v[i][3] * rinv * g[3])};
  }
}

}  // namespace

void launch_moe_permute(const int32_t* idx, int n_routes, int n_exp, int32_t* offs, int32_t* perm,
                        int32_t* inv, hipStream_t s) {
  hipLaunchKernelGGL(moe_permute_kernel, dim3(n_exp), dim3(64 * kPermWaves), 0, s, idx, n_routes,
                     n_exp, offs, perm, inv);
}

// Row tiles per pass from the mean routed rows per expert, sized so that the busiest expert
// (about four standard deviations above a uniform mean) still fits one pass; a second
// work-group per expert picks up any pass beyond the first (it exits at once when there is
// none), so a skewed routing costs a parallel work-group instead of a serial pass.
template <bool GATED, int FPW, bool F8>
void launch_stream_t(const MoeArgs& a, int mean_rows, hipStream_t s) {
  const dim3 grid(a.N / (64 * FPW), a.n_exp, 2);
  constexpr int KS1 = F8 ? 2 : 1;  // E4M3 fragments come in pairs of k-steps
  if (GATED && a.idx) {
    constexpr bool FU = GATED;  // (the branch is only taken for the gate/up projection)
    if (mean_rows <= 24) hipLaunchKernelGGL((expert_stream_kernel<GATED, 3, KS1, FPW, F8, FU, 1>), grid, dim3(256), 0, s, a);
    else if (mean_rows <= 36) hipLaunchKernelGGL((expert_stream_kernel<GATED, 4, 2, FPW, F8, FU, 1>), grid, dim3(256), 0, s, a);
    else if (mean_rows <= 84) hipLaunchKernelGGL((expert_stream_kernel<GATED, 8, 2, FPW, F8, FU, 1>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((expert_stream_kernel<GATED, 10, 2, FPW, F8, FU, 1>), grid, dim3(256), 0, s, a);
    return;
  }
  if (mean_rows <= 24) hipLaunchKernelGGL((expert_stream_kernel<GATED, 3, KS1, FPW, F8, false, 1>), grid, dim3(256), 0, s, a);
  else if (mean_rows <= 36) hipLaunchKernelGGL((expert_stream_kernel<GATED, 4, 2, FPW, F8, false, 1>), grid, dim3(256), 0, s, a);
  else if (mean_rows <= 84) hipLaunchKernelGGL((expert_stream_kernel<GATED, 8, 2, FPW, F8, false, 1>), grid, dim3(256), 0, s, a);
  else {
    // many rows per expert: every feature group re-reads the expert's staged rows, so the
    // groups of one expert share a work-group (SG subgroups of four waves, one staging of the
    // rows) while the grid still holds a work-group per CU.  With one work-group per CU an
    // expert whose rows need a second pass would add a second round of work-groups, so a pass
    // holds 192 rows here (a uniform router's 128 per expert plus five standard deviations;
    // 32-column chunks for the gate/up pair, whose registers then fit 12 waves per CU)
    constexpr int SG = GATED ? 3 : 2;
    constexpr int KSG = (GATED && !F8) ? 1 : 2;  // registers: 12 waves per CU hold 170 each
    if (!(GATED && F8) && (a.N / (64 * FPW)) % SG == 0 && (a.N / (64 * FPW * SG)) * a.n_exp >= 256) {
      const dim3 g(a.N / (64 * FPW * SG), a.n_exp, 2);
      hipLaunchKernelGGL((expert_stream_kernel<GATED, 12, KSG, FPW, F8, false, SG>), g, dim3(256 * SG), 0, s, a);
    } else {
      hipLaunchKernelGGL((expert_stream_kernel<GATED, 10, 2, FPW, F8, false, 1>), grid, dim3(256), 0, s, a);
    }
  }
}

template <bool GATED, int FPW>
void launch_stream(const MoeArgs& a, int mean_rows, hipStream_t s) {
  if (a.wp8) launch_stream_t<GATED, FPW, true>(a, mean_rows, s);
  else launch_stream_t<GATED, FPW, false>(a, mean_rows, s);
}

void launch_moe_gemm1(const MoeArgs& a, int mean_rows, hipStream_t s) { launch_stream<true, kGroupTiles1 / 4>(a, mean_rows, s); }
void launch_moe_gemm2(const MoeArgs& a, int mean_rows, hipStream_t s) { launch_stream<false, kGroupTiles2 / 4>(a, mean_rows, s); }

void launch_quantize_e4m3(const uint16_t* w, long rows, int cols, uint8_t* q, float* scale,
                          hipStream_t s) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(quantize_e4m3_kernel, dim3(rows), dim3(256), 0, s, w, cols, q, scale);
}

void launch_moe_pack_fp8(const uint8_t* q0, const uint8_t* q1, uint8_t* out, int n_exp, int N,
                         int K, int group_tiles, hipStream_t s) {
  const int na = q1 ? 2 : 1;
  const long total = static_cast<long>(n_exp) * (N / 16) * (K / 64) * na * 64;
  hipLaunchKernelGGL(moe_pack_fp8_kernel, dim3((total + 255) / 256), dim3(256), 0, s, q0, q1, out,
                     n_exp, N, K, na, group_tiles);
}

void launch_moe_pack(const uint16_t* w0, const uint16_t* w1, uint16_t* out, int n_exp, int N, int K,
                     int group_tiles, hipStream_t s) {
  const int na = w1 ? 2 : 1;
  const long total = static_cast<long>(n_exp) * (N / 16) * (K / 32) * na * 64;
  hipLaunchKernelGGL(moe_pack_kernel, dim3((total + 255) / 256), dim3(256), 0, s, w0, w1, out, n_exp,
                     N, K, na, group_tiles);
}

void launch_moe_combine(float* h, const float* part, int n_part, long part_stride, const uint16_t* y,
                        const int32_t* inv, const float* gates, int rows, int d, int top_k,
                        const float* gain, float eps, uint16_t* out, hipStream_t s) {
  const int nch = (d + 2047) / 2048;
#define DG_MC(N, KJ, NP)                                                                          \
  hipLaunchKernelGGL((moe_combine_kernel<N, KJ, NP>), dim3(rows), dim3(512), 0, s, h, part, n_part,  \
                     part_stride, y, inv, gates, d, top_k, gain, eps, out)
#define DG_MC_P(N, KJ)                    \
  if (n_part <= 0) DG_MC(N, KJ, 0);       \
  else if (n_part <= 2) DG_MC(N, KJ, 2);  \
  else DG_MC(N, KJ, 4)
#define DG_MC_K(N)                  \
  if (top_k <= 4) { DG_MC_P(N, 4); } \
  else { DG_MC_P(N, 8); }
  if (nch <= 1) { DG_MC_K(1); }
  else if (nch <= 2) { DG_MC_K(2); }
  else { DG_MC_K(4); }
#undef DG_MC_K
#undef DG_MC_P
#undef DG_MC
}

}  // namespace dg
