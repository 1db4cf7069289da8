// Canvas attention (bidirectional, no mask) and causal prefill attention on MFMA, plus the
// RoPE angle table (the rotation itself is applied in the QKV projection's epilogue).
//
// Each work-group serves one (request, KV head) and four or eight (query head, 16- or 32-row)
// tasks of that head's query group, one per wave, so every K/V tile staged in LDS is reused by
// all of them (GQA).
// Keys are the request's cached prefix followed by the canvas keys; the key range can be split
// across work-groups (split-KV) so that a 256-row canvas still fills the chip; the splits are
// merged in a fixed order afterwards (deterministic).
//
// Lane layout: per 64-key block a wave computes S^T = K Q^T with 16x16x32 MFMAs (A = K rows
// from LDS, B = its 32 queries from registers).  The accumulator gives each lane one query
// (lane % 16) and four keys, which is exactly the B-operand layout of the next MFMA,
// O^T += V^T P^T, if the 32 keys of one MFMA are taken as {4j..4j+3} of two 16-key sub-blocks
// (the k order inside an MFMA only has to agree between A and B).  V stays [key][d] in LDS and
// the A operand V^T[d][keys] is two transposing 8-byte LDS reads.  The online-softmax state
// (max, sum) is per query = per lane, so rescaling O^T needs no cross-lane traffic; the block
// maximum is reduced across the four lanes of a query with permlane swaps, and the sum of P
// comes from one more MFMA against an all-ones A operand.
#include "dg_common.h"
#include "dg_kernels.h"

namespace dg {
namespace {

// ---------------------------------------------------------------------------------- RoPE
// Angles reach ~10^5 radians at long prefixes, where a float32 angle is already off by ~1e-2,
// so the table is built in float64 (once per step: every layer uses the same positions).
__global__ __launch_bounds__(256) void rope_table_kernel(RowMap map, int rows, int D, float theta,
                                                         float* __restrict__ table) {
  const int half = D / 2;
  const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<long>(rows) * half) return;
  const int r = static_cast<int>(i / half), j = static_cast<int>(i % half);
  const int b = r / map.rows_per_req;
  const double pos = static_cast<double>(map.pos0[b] + (r - b * map.rows_per_req));
  double sn, cs;
  sincos(pos * pow(static_cast<double>(theta), -2.0 * j / D), &sn, &cs);
  table[2 * i] = static_cast<float>(cs);
  table[2 * i + 1] = static_cast<float>(sn);
}

// ---------------------------------------------------------------------------- attention
constexpr int KB = 64;       // keys per block

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each 16-lane group, lane s points
// at 4 consecutive 16-bit values of row s / 4, columns 4 (s % 4) .. +4 of a 4 x 16 block; lane
// 4a + c receives column 4a + c of the four rows.  Used so that V can stay [key][d] in LDS and
// still feed the A operand V^T of O^T += V^T P^T.
typedef short v4i16_t __attribute__((ext_vector_type(4)));
DG_DEVICE u32x2_t read_tr16(const uint16_t* p) {
  const v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

// 2^x with the hardware instruction alone: results below 2^-126 flush to zero instead of going
// through the denormal range fix-up (a probability that small is invisible next to the row sum,
// which is at least 1).
DG_DEVICE float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions across the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48 hold the same
// query).  The gfx950 permlane swaps exchange lane l with l^16 (rows of 16) or l^32 (halves):
// called with the same value in both operands they return {v[l], v[l^16]} (resp. l^32) to
// every lane, with no trip through the LDS crossbar.
DG_DEVICE float group_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// K and V blocks as they are in memory ([key][d]); rows padded by 32 bytes (measured on gfx950:
// the 16-byte K-fragment reads, 16 rows per 16 lanes, run about a third faster at a 288-byte
// pitch than at 272, and the transposing 8-byte V reads are at their best there too).
template <int D>
struct AttnSmem {
  uint16_t k[KB][D + 16];
  uint16_t v[KB][D + 16];
};

// NW waves (query tasks) share each staged K/V block; at most 256 registers per lane, so two
// waves per SIMD: with 4 waves two work-groups share a CU (one group's MFMAs overlap the other's
// softmax and staging), with 8 waves each block is staged once for twice the queries (less
// staging per MFMA, used for long key ranges).
template <int D, int NW, int QT>  // QT: 16-row query tiles per wave (1 or 2)
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attention_kernel(AttnArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int NKS = D / 32;   // MFMA k-steps over the head dimension
  constexpr int NDT = D / 16;   // 16-row tiles of O^T
  constexpr int KCH = KB * D / 8 / NT;      // 16-byte K/V chunks per thread
  __shared__ AttnSmem<D> sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j4 = lane >> 4, l16 = lane & 15;
  const int bg = blockIdx.z;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int group = a.Hq / a.Hkv;
  const int rows = a.rows_per_req;
  constexpr int RW = 16 * QT;  // query rows per wave task
  const int n_rb = (rows + RW - 1) / RW;
  const int task = blockIdx.x * NW + wave;
  const bool active = task < group * n_rb;
  const int hq = g * group + (active ? task % group : 0);
  const int rb = active ? task / group : 0;
  const int row0 = rb * RW;  // first query row (within the request) of this wave

  const int n_cache = a.n_cache[b];
  const int n_keys = n_cache + a.n_extra;
  // key range of this split; with a causal mask it ends after the last query of the group
  const int k_lo = blockIdx.y * a.split_keys;
  int k_hi = min(n_keys, k_lo + a.split_keys);
  if (a.causal) {
    const int last_task = min(blockIdx.x * NW + NW - 1, group * n_rb - 1);
    const int last_row = min(rows - 1, (last_task / group) * RW + RW - 1);
    k_hi = min(k_hi, a.q_pos0[b] + last_row + 1);
  }
  const long qrow_base = static_cast<long>(b) * rows;

  // queries (B operand): lane holds Q[qt*16 + l16][ks*32 + 8*j4 .. +8]
  u32x4_t qf[QT][NKS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qr = row0 + qt * 16 + l16;
    const bool ok = active && qr < rows;
    const uint16_t* qp = a.q + (qrow_base + qr) * a.Hq * D + hq * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[qt][ks] = ok ? ld16(qp + ks * 32 + 8 * j4) : u32x4_t{0u, 0u, 0u, 0u};
  }
  int qpos[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) qpos[qt] = a.q_pos0[b] + row0 + qt * 16 + l16;
  const int qmin = a.q_pos0[b] + row0;  // smallest query position of this wave

  floatx4_t o[NDT][QT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) o[dt][qt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  // running max (in log2 units, scale folded in) per query; the running sum of P is one more
  // MFMA per step with an all-ones A operand (every row of that tile is the column sum of P^T,
  // i.e. this lane's query sum over the step's keys, of the same bf16 P that multiplies V)
  float m_run[QT];
  floatx4_t l_acc[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -INFINITY;
    l_acc[qt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
  const u32x4_t ones = u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const float sl2 = a.scale * 1.4426950408889634f;

  const long kv_head = static_cast<long>(a.slot[b]) * a.Hkv + g;  // cache slot of the request
  const long kx_head = static_cast<long>(b) * a.Hkv + g;          // this call's canvas rows
  u32x4_t rk[KCH], rv[KCH];

  // S^T of one 64-key block for both query tiles (raw dot products)
  auto qk = [&](floatx4_t (&sc)[4][QT]) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) sc[kt][qt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const u32x4_t kf = ld16(&sm.k[kt * 16 + l16][ks * 32 + 8 * j4]);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) sc[kt][qt] = mfma16(kf, qf[qt][ks], sc[kt][qt]);
      }
    }
  };
  // online softmax per lane (= per query), in place: p = 2^(s*sl2 - m), one FMA + one exp each;
  // returns whether some lane's running max moved (O^T and the sum then need rescaling)
  auto softmax = [&](floatx4_t (&sc)[4][QT], int kb0, int kb_hi, float (&alpha)[QT]) {
    // mask only blocks that cross the range end or the causal diagonal (uniform branch)
    if ((kb0 + KB > kb_hi) || (a.causal && kb0 + KB - 1 > qmin)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kk = kb0 + kt * 16 + 4 * j4 + i;
            if (kk >= kb_hi || (a.causal && kk > qpos[qt])) sc[kt][qt][i] = -INFINITY;
          }
    }
    bool rescale = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        mx = fmaxf(fmaxf(mx, fmaxf(sc[kt][qt][0], sc[kt][qt][1])), fmaxf(sc[kt][qt][2], sc[kt][qt][3]));
      mx = group_max(mx);
      const float m_new = fmaxf(m_run[qt], mx * sl2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // all keys masked so far
      alpha[qt] = fast_exp2(m_run[qt] - m_use);                // 0 when m_run is -inf
      rescale |= (alpha[qt] != 1.f);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[kt][qt][i] = fast_exp2(fmaf(sc[kt][qt][i], sl2, -m_use));
      m_run[qt] = m_new;
    }
    return rescale;
  };
  // P as the bf16 B operand of the two 32-key MFMA steps: lane holds the 8 keys
  // {4 j4 .. 4 j4 + 3} of two 16-key sub-blocks for its query
  auto pack_p = [&](const floatx4_t (&sc)[4][QT], u32x4_t (&pf)[2][QT]) {
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const floatx4_t p0 = sc[2 * kk2][qt], p1 = sc[2 * kk2 + 1][qt];
        pf[kk2][qt] = u32x4_t{pack_bf2(p0[0], p0[1]), pack_bf2(p0[2], p0[3]), pack_bf2(p1[0], p1[1]),
                              pack_bf2(p1[2], p1[3])};
      }
  };
  // O^T = alpha O^T + V^T P^T over two 32-key steps (and the sum of P alongside)
  auto pv = [&](const u32x4_t (&pf)[2][QT], bool rescale, const float (&alpha)[QT]) {
    // rescaling by alpha == 1 is exact, so it is skipped when no lane of the wave needs it
    if (__any(rescale)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt][qt] *= alpha[qt];
        l_acc[qt] *= alpha[qt];
      }
    }
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        // A = V^T[d = 16 dt + l16][the 8 keys of P's lane group]: two transposing reads, each
        // giving this lane 4 consecutive keys of its d column
        const int kr = kk2 * 32 + 4 * j4 + (l16 >> 2), dc = dt * 16 + 4 * (l16 & 3);
        const u32x2_t lo = read_tr16(&sm.v[kr][dc]);
        const u32x2_t hi = read_tr16(&sm.v[kr + 16][dc]);
        const u32x4_t vf = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) o[dt][qt] = mfma16(vf, pf[kk2][qt], o[dt][qt]);
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) l_acc[qt] = mfma16(ones, pf[kk2][qt], l_acc[qt]);
    }
  };

  // Keys come in two ranges with one base pointer each (uniform, so addresses are a scalar
  // base plus a lane offset): the cached prefix [0, n_cache) and the canvas [n_cache, n_keys).
  // Keys past a range end re-read its last key (every load is unconditional, so wait counts
  // stay exact) and are masked to -inf.  The next block's global loads are in flight while
  // the current one is computed from LDS.
  auto run_range = [&](const uint16_t* kbase, const uint16_t* vbase, int key0, int kb_lo, int kb_hi) {
    auto gload = [&](int kb0) {
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int c = tid + NT * i, key = c / (D / 8), col = (c % (D / 8)) * 8;
        const long kk = min(kb0 + key, kb_hi - 1) - key0;
        rk[i] = ld16(kbase + kk * D + col);
        rv[i] = ld16(vbase + kk * D + col);
      }
    };
    auto sstore = [&]() {
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const int c = tid + NT * i, key = c / (D / 8), col = (c % (D / 8)) * 8;
        st16(&sm.k[key][col], rk[i]);
        st16(&sm.v[key][col], rv[i]);
      }
    };

    const int n_blk = (kb_hi > kb_lo) ? (kb_hi - kb_lo + KB - 1) / KB : 0;
    if (n_blk > 0) gload(kb_lo);
    for (int blk = 0; blk < n_blk; ++blk) {
      const int kb0 = kb_lo + blk * KB;
      __syncthreads();  // previous block's LDS reads are done
      sstore();
      __syncthreads();
      gload(blk + 1 < n_blk ? kb0 + KB : kb0);  // unconditional: exact wait counts
      sched_fence();
      if (!active) continue;
      floatx4_t sc[4][QT];
      u32x4_t pf[2][QT];
      float alpha[QT];
      qk(sc);
      const bool rescale = softmax(sc, kb0, kb_hi, alpha);
      pack_p(sc, pf);
      pv(pf, rescale, alpha);
    }
  };

  run_range(a.kc + kv_head * a.cap * D, a.vc + kv_head * a.cap * D, 0, k_lo, min(k_hi, n_cache));
  if (a.n_extra > 0)
    run_range(a.kx + kx_head * a.xcap * D, a.vx + kx_head * a.xcap * D, n_cache, max(k_lo, n_cache), k_hi);

  if (!active) return;
  float l_run[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) l_run[qt] = l_acc[qt][0];
  // write: lane owns query qt*16+l16, dims dt*16 + 4*j4 + i; partial maxima are in log2 units
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qr = row0 + qt * 16 + l16;
    if (qr >= rows) continue;
    const long orow = qrow_base + qr;
    if (a.n_split == 1) {
      const float inv = (l_run[qt] > 0.f) ? 1.0f / l_run[qt] : 0.f;
      uint16_t* op = a.out + orow * a.Hq * D + hq * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const floatx4_t v = o[dt][qt];
        *reinterpret_cast<u32x2_t*>(op + dt * 16 + 4 * j4) =
            u32x2_t{pack_bf2(v[0] * inv, v[1] * inv), pack_bf2(v[2] * inv, v[3] * inv)};
      }
    } else {
      const long slot = (orow * a.Hq + hq) * a.n_split + blockIdx.y;
      float* po = a.part_o + slot * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<floatx4_t*>(po + dt * 16 + 4 * j4) = o[dt][qt];
      if (j4 == 0) {
        a.part_ml[slot * 2] = m_run[qt];
        a.part_ml[slot * 2 + 1] = l_run[qt];
      }
    }
  }
}

// Merge split partials in split order: O = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s.
// Every (max, sum) pair and every partial row of a thread is requested before any arithmetic.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           uint16_t* __restrict__ out, int n_rh,
                                                           int n_split) {
  constexpr int TPR = D / 4;  // threads per (row, head): 4 dims each
  constexpr int MS = 16;      // most splits a launch uses
  const int rh = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  if (rh >= n_rh) return;
  const int d0 = (threadIdx.x % TPR) * 4;
  const long base = static_cast<long>(rh) * n_split;
  float2 ml[MS];
  floatx4_t po[MS];
#pragma unroll
  for (int s = 0; s < MS; ++s)
    if (s < n_split) {
      ml[s] = *reinterpret_cast<const float2*>(part_ml + (base + s) * 2);
      po[s] = *reinterpret_cast<const floatx4_t*>(part_o + (base + s) * D + d0);
    }
  float m = -INFINITY;
#pragma unroll
  for (int s = 0; s < MS; ++s)
    if (s < n_split) m = fmaxf(m, ml[s].x);
  floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    if (s >= n_split || ml[s].x == -INFINITY) continue;
    const float w = exp2f(ml[s].x - m);
    l += w * ml[s].y;
    acc += w * po[s];
  }
  const float inv = (l > 0.f) ? 1.0f / l : 0.f;
  *reinterpret_cast<u32x2_t*>(out + static_cast<long>(rh) * D + d0) =
      u32x2_t{pack_bf2(acc[0] * inv, acc[1] * inv), pack_bf2(acc[2] * inv, acc[3] * inv)};
}

template <int D, int NW>
void launch_attn_w(const AttnArgs& a, hipStream_t s) {
  const int group = a.Hq / a.Hkv;
  const int qt = a.q_tiles == 1 ? 1 : 2;
  const int tasks = group * ((a.rows_per_req + 16 * qt - 1) / (16 * qt));
  dim3 grid((tasks + NW - 1) / NW, a.n_split, a.n_req * a.Hkv);
  if (qt == 1) hipLaunchKernelGGL((attention_kernel<D, NW, 1>), grid, dim3(64 * NW), 0, s, a);
  else hipLaunchKernelGGL((attention_kernel<D, NW, 2>), grid, dim3(64 * NW), 0, s, a);
}

template <int D>
void launch_attn_d(const AttnArgs& a, hipStream_t s) {
  if (a.n_waves == 8) launch_attn_w<D, 8>(a, s);
  else launch_attn_w<D, 4>(a, s);
}

template <int D>
void launch_combine_d(const AttnArgs& a, hipStream_t s) {
  const int n_rh = a.n_req * a.rows_per_req * a.Hq;
  const int per = 256 / (D / 4);
  hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((n_rh + per - 1) / per), dim3(256), 0, s,
                     a.part_o, a.part_ml, a.out, n_rh, a.n_split);
}

}  // namespace

int attention_waves(int max_keys, bool causal) { return max_keys >= (causal ? 8192 : 2048) ? 8 : 4; }
int attention_q_tiles(int max_keys, bool causal) { return (!causal && max_keys < 8192) ? 1 : 2; }

void launch_rope_table(const RowMap& map, int rows, int D, float theta, float* table, hipStream_t s) {
  const long n = static_cast<long>(rows) * (D / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, map, rows, D, theta, table);
}

void launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.D == 128) launch_attn_d<128>(a, s);
  else launch_attn_d<64>(a, s);
}

void launch_attention_combine(const AttnArgs& a, hipStream_t s) {
  if (a.n_split <= 1) return;
  if (a.D == 128) launch_combine_d<128>(a, s);
  else launch_combine_d<64>(a, s);
}

}  // namespace dg
