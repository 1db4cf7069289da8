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

// ------------------------------------------------------------------ pipelined canvas kernel
// Attention over long key ranges at head_dim 128 (the canvas, unmasked, and the causal
// prefill, whose mask only touches the half blocks that cross a wave's diagonal), 8 waves of one
// 32-row query tile each, on the 32 x 32 x 16 matrix instruction:
//  * one 32 x 32 MFMA does the work of two 16 x 16 x 32 ones but holds the SIMD's issue for
//    about as long as one of them (measured on gfx950: each MFMA blocks vector issue for ~11
//    cycles, whatever its size), which leaves more issue cycles to the softmax's vector work
//    (an exponential and half a pack per score): 17 MFMAs per 32-key half (one of them the
//    offset below), where the 16 x 16 x 32 kernel issues 34;
//  * the scores leave the MFMAs ready for the exponential: the queries are multiplied by
//    scale * log2 e once (and rounded to bf16 again), and each QK^T chain starts with one more
//    MFMA that adds the query's exponent offset -m_ref (a ones column of K times an offset row of
//    Q^T), which replaces an FMA per score with one MFMA per 1024 scores;
//  * software pipeline: while the softmax of half block n runs (exp, pack to bf16, row sum),
//    the QK^T products of the next half are already issued; while P V of half n runs, the
//    maximum of the next half is taken.  Two score tiles alternate;
//  * a wave raises its issue priority for its P V groups: of the two waves of a SIMD, the one
//    with only matrix work queued then keeps the MFMA unit fed, while the other's softmax takes
//    the vector issue slots in between (measured 2.9 % faster than equal priorities, 1.7 % faster
//    than raising it for the softmax groups instead);
//  * K and V blocks go from global memory straight into LDS (global_load_lds_dwordx4) through
//    a ring of PS stages, three blocks ahead, one barrier per block; no staging registers.  A
//    1 KB load is four whole 256-byte key rows, so every instruction reads 1 KB of contiguous
//    memory; inside a row the 16-byte chunk c is stored at chunk c ^ swz_k(row) (K) or
//    c ^ swz_v(row) (V), below, which keeps the 16-byte K fragment reads and the transposing
//    8-byte V reads free of bank conflicts;
//  * lazy rescaling: the exponent reference of a query only moves when the block maximum
//    exceeds it by more than kLazy (log2 units), so P stays below about 2^kLazy and O and its row
//    sum are rescaled a handful of times per range instead of whenever the maximum grows; the
//    result is unchanged (O and the row sum share the reference, which cancels);
//  * the work-groups that share one (request, KV head, split) range are numbered so that they
//    land on the same XCD, whose L2 then serves the second reader.
//
// Lane layouts of the 32 x 32 x 16 bf16 MFMA (D = A B): lane l holds A[l % 32][8 (l / 32) ..
// + 8], B[8 (l / 32) .. + 8][l % 32] and D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32], i = 0..15.
// Scores are S^T = K Q^T (keys x queries): lane l holds 16 keys of query l % 32.  P^T feeds
// O^T += V^T P^T as the B operand in the same registers, so the keys of a 16-key chunk are taken
// in the order that layout gives: slot s of lane half hh = l / 32 is key 8 (s / 4) + 4 hh + s % 4;
// V^T (the A operand) is read in the same key order.
constexpr int PS = 4;          // LDS ring stages (3 blocks in flight)
constexpr float kLazy = 8.f;   // lazy-rescale margin, log2 units

template <int S>
using Stage = std::integral_constant<int, S % PS>;

typedef float floatx16_t __attribute__((ext_vector_type(16)));
DG_DEVICE floatx16_t mfma32(const u32x4_t& a, const u32x4_t& b, const floatx16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// acc + the two bf16 values of pk (v_dot2 with (1, 1)): the row sum of the rounded P
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
DG_DEVICE float add_bf2(uint32_t pk, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk),
                                         __builtin_bit_cast(bf16x2_t, 0x3F803F80u), acc, false);
}
// Sum and maximum of lanes l and l ^ 32 (gfx950 permlane32 swap, no trip through LDS): called
// with the same value in both operands the swap returns v[l] and v[l ^ 32] to every lane, as
// (low lane, high lane) in both, so both lanes add the same two numbers in the same order.
DG_DEVICE float pair_sum(float v) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
DG_DEVICE float pair_max(float v) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Chunk swizzles of the LDS key rows (16 chunks of 16 bytes): chunk c of K row r is stored at
// c ^ swz_k(r), of V row r at c ^ swz_v(r).
//  * A K fragment read takes one 16-byte chunk (2 k + hh) of 32 consecutive rows per lane half:
//    swz_k(r) = r % 16 puts the rows on all sixteen chunk positions, two rows each (512 bytes
//    over the 256 bytes of banks: the fewest passes there can be).  An even swizzle leaves only
//    eight positions, four rows each (counters: a third of the LDS cycles went to conflicts).
//  * A transposing V read takes the 32-byte pairs 2 dt and 2 dt + 1 of the four rows 4 hh .. + 3
//    per lane half.  swz_v(r) is even, so a pair stays together and pair p goes to
//    p ^ (swz_v(r) / 2); with swz_v(r) / 2 = 2 (r % 4) + (r / 4) % 2 the four rows' swizzles
//    differ above the lowest pair bit, and rows r and r + 4 take opposite parities, so the
//    eight pairs a lane half reads are distinct.
DG_DEVICE int swz_k(int r) { return r & 15; }
DG_DEVICE int swz_v(int r) { return ((r & 3) << 2) | ((r >> 1) & 2); }

// One global_load_lds_dwordx4: lane l's 16 bytes at g land at LDS address lds + 16 l.  Issued
// from inline assembly so that the compiler does not track it: its own tracking of such loads
// loses the stage of each one at the loop's back edge and then drains every load in flight
// before the first LDS read of the loop body.  The kernel waits for these loads itself
// (s_waitcnt vmcnt + barrier before a stage is read; vmcnt(0) before exit).  The instruction
// has no destination register, and its address registers are read when it issues.
// The address is a wave-uniform base (scalar registers) plus a 32-bit per-lane byte offset.
DG_DEVICE void dma16(const uint16_t* base, uint32_t lane_ofs, const uint16_t* lds) {
  const uint32_t l = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)lds));
  // the base is wave-uniform; reading it from the first lane puts it in scalar registers (the
  // builtin works on int: each half goes back to uint32_t before widening, no sign extension)
  const uint64_t b64 = reinterpret_cast<uint64_t>(base);
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b64 >> 32)));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b64 & 0xffffffffu)));
  const uint64_t sb = (static_cast<uint64_t>(hi) << 32) | lo;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(l), "v"(lane_ofs), "s"(sb)
               : "memory", "m0");
}

template <int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attention_pipe_kernel(AttnArgs a) {
  constexpr int D = 128, NKC = D / 16, NDT = D / 32;  // 16-dim k-chunks of QK^T; 32-dim O tiles
  constexpr int SEG = 2 * KB * D * 2 / 1024;  // 1 KB segments per stage (K then V)
  constexpr int LPW = SEG / NW;               // segments each wave loads per stage
  static_assert(SEG % NW == 0 && LPW * NW == SEG, "segments split evenly over the waves");
  // one LDS array per stage, [K, V][key][d] with 256-byte rows and XOR-swizzled chunks; stage
  // indices are compile-time (the loop is unrolled over the ring), so the compiler sees that
  // reads of one stage never alias the direct-to-LDS writes in flight to the others and does
  // not drain those loads before each read
  __shared__ uint16_t st0[2 * KB * D], st1[2 * KB * D], st2[2 * KB * D], st3[2 * KB * D];
  auto stage = [&](auto S) -> uint16_t* {
    constexpr int s = decltype(S)::value;
    if constexpr (s == 0) return st0;
    else if constexpr (s == 1) return st1;
    else if constexpr (s == 2) return st2;
    else return st3;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar registers
  const int l32 = lane & 31, hh = lane >> 5;  // query column of the tile; lane half
  const int l16 = lane & 15, g4 = lane >> 4;  // lane in, and index of, its 16-lane group
  // work-group -> (task group bx, unit u); unit u = (pair p, KV head g) and pair p = (request
  // b, split by), pairs longest first.  The dispatcher places work-group lin on XCD lin % 8 and
  // hands each XCD its work-groups in order, so unit u goes to XCD u % 8 with its task groups
  // next to each other there (the second reader of a key range hits that XCD's L2), and every
  // XCD starts on the longest ranges.
  const int group = a.Hq / a.Hkv;
  const int rows = a.rows_per_req;
  constexpr int RW = 32;
  const int n_rb = (rows + RW - 1) / RW;
  const int nx = (group * n_rb + NW - 1) / NW;
  const int lin = blockIdx.x;
  const int bx = (lin / 8) % nx;
  const int u = (lin / 8 / nx) * 8 + lin % 8;
  if (u >= a.n_pairs * a.Hkv) return;  // padding of the last row of eight units (uniform)
  const int pr = a.pair[u / a.Hkv];
  const int b = pr >> 8, by = pr & 255, g = u % a.Hkv;
  const int task = bx * NW + wave;
  const bool active = task < group * n_rb;
  const int hq = g * group + (active ? task % group : 0);
  const int row0 = (active ? task / group : 0) * RW;
  const long qrow_base = static_cast<long>(b) * rows;
  const int n_split_b = a.req_split[b];

  // key blocks: the cached prefix [k_lo, hi0) then the canvas [lo1, k_hi), KB keys each
  const int n_cache = a.n_cache[b];
  const int n_keys = n_cache + a.n_extra;
  const int k_lo = by * a.req_split_keys[b];
  int k_hi = min(n_keys, k_lo + a.req_split_keys[b]);
  // causal: the work-group's range ends after its last query (a split past it is empty)
  const int qpos0 = a.q_pos0[b] + row0;  // position of the wave's first query row
  if (a.causal) {
    const int last_task = min(bx * NW + NW - 1, group * n_rb - 1);
    const int last_row = min(rows - 1, (last_task / group) * RW + RW - 1);
    k_hi = min(k_hi, a.q_pos0[b] + last_row + 1);
  }
  const int hi0 = min(k_hi, n_cache), lo1 = max(k_lo, n_cache);
  const int nb0 = hi0 > k_lo ? (hi0 - k_lo + KB - 1) / KB : 0;
  const int nb = nb0 + (k_hi > lo1 ? (k_hi - lo1 + KB - 1) / KB : 0);
  const long kv_head = static_cast<long>(a.slot[b]) * a.Hkv + g;
  const long kx_head = static_cast<long>(b) * a.Hkv + g;
  const uint16_t* kc = a.kc + kv_head * a.cap * D;
  const uint16_t* vc = a.vc + kv_head * a.cap * D;
  const uint16_t* kx = a.kx + kx_head * a.xcap * D;
  const uint16_t* vx = a.vx + kx_head * a.xcap * D;
  auto first_key = [&](int bi) { return bi < nb0 ? k_lo + bi * KB : lo1 + (bi - nb0) * KB; };
  auto end_key = [&](int bi) { return bi < nb0 ? hi0 : k_hi; };

  // this lane's part of the wave's LPW segments: segment s of a stage holds key rows
  // 4 (s % 16) .. + 3 of K (s < 16) or V; lane i fills LDS chunk i % 16 of row i / 16 with the
  // global chunk (i % 16) ^ swz_k(row) (K) or ^ swz_v(row) (V)
  // (segment bases are wave-uniform: the cache and canvas arrays of K or V, the canvas one
  // offset so that both are indexed by the key's position in the request)
  int seg_row[LPW], seg_chunk[LPW];
  const uint16_t* seg_cb[LPW];
  const uint16_t* seg_xb[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int s = wave * LPW + i, r = 4 * (s & 15) + (lane >> 4);
    seg_row[i] = r;
    seg_chunk[i] = ((lane & 15) ^ (s < 16 ? swz_k(r) : swz_v(r))) * 8;
    seg_cb[i] = s < 16 ? kc : vc;
    seg_xb[i] = (s < 16 ? kx : vx) - static_cast<long>(n_cache) * D;
  }
  // block bi into stage S (= bi % PS); past the last block, a copy of it into a stage that is
  // not read again (or only by the unused scores of the step after the last)
  auto issue = [&](auto S, int bi) {
    uint16_t* sp = stage(S);
    bi = min(bi, nb - 1);
    const int kb0 = first_key(bi), lim = end_key(bi) - 1 - kb0;  // rows past lim re-read row lim
    const bool canvas = bi >= nb0;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int s = wave * LPW + i;
      const uint16_t* base = (canvas ? seg_xb[i] : seg_cb[i]) + static_cast<long>(kb0) * D;
      const uint32_t ofs = static_cast<uint32_t>(min(seg_row[i], lim) * (D * 2) + seg_chunk[i] * 2);
      dma16(base, ofs, sp + s * 512);
    }
  };

  // queries (B operand of S^T = K Q^T): lane holds Q[row0 + l32][16 c + 8 hh .. + 8]
  u32x4_t qf[NKC];
  {
    const int qr = row0 + l32;
    const bool ok = active && qr < rows;
    const uint16_t* qp = a.q + (qrow_base + qr) * a.Hq * D + hq * D;
#pragma unroll
    for (int c = 0; c < NKC; ++c) qf[c] = ok ? ld16(qp + 16 * c + 8 * hh) : u32x4_t{0u, 0u, 0u, 0u};
  }
  // scores in log2 units: Q <- bf16(Q * scale * log2 e)
  const float sl2 = a.scale * 1.4426950408889634f;
#pragma unroll
  for (int c = 0; c < NKC; ++c)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = qf[c][w];
      qf[c][w] = pack_bf2(__uint_as_float(x << 16) * sl2, __uint_as_float(x & 0xffff0000u) * sl2);
    }
  // the queries have landed before the first stage load is issued: the compiler does not see
  // those loads, so a wait it placed for a query register inside the loop would also wait for
  // the stage loads issued after it
  wait_vm_lgkm0<0>();
  floatx16_t o[NDT];  // O^T tile dt: lane holds d = 32 dt + 8 (i / 4) + 4 hh + i % 4 of its query
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  // per query (each lane pair l, l ^ 32 holds the same values): exponent reference m_ref (log2
  // units, a bf16 value) of O and the row sum; the offset -m_ref (0 while no key has been seen)
  // that the scores come out with; the offset score above which the reference has to move
  // (kLazy, or -inf while no key has been seen).  All three change only where the reference
  // does.  The row sum is this lane's keys only; the two halves are added at the end.
  float m_ref = -INFINITY, neg_mu = 0.f, thr = -INFINITY, l_acc = 0.f;
  // the offset MFMA's operands: A = a ones column (dim 0 of every key), B = the offset row
  // (dim 0 of every query: bf16(-m_ref), exact since m_ref is a bf16 value); lanes of half 1
  // hold dims 8..15, all zero
  const u32x4_t ones = {hh == 0 ? 0x3F80u : 0u, 0u, 0u, 0u};
  u32x4_t qb = {0u, 0u, 0u, 0u};

  // K fragment c of a half (A operand: key row l32, dims 16 c + 8 hh .. + 8, i.e. 16-byte chunk
  // 2 c + hh): element offsets inside the half, one register each (the swizzle is per row; the
  // second half's rows, 32 further, have the same swizzles)
  int kofs[NKC];
#pragma unroll
  for (int c = 0; c < NKC; ++c) kofs[c] = l32 * D + 8 * ((2 * c + hh) ^ swz_k(l32));
  // V^T fragment (16-key chunk c, 32-dim tile dt): A operand, lane holds d = 32 dt + l32 and the
  // keys of P's slots, 4 hh + 0..3 (lo) and 8 + 4 hh + 0..3 (hi) of the chunk.  In a transposing
  // read, lane s of 16-lane group g4 points at row 4 hh + s / 4 (+ 8 for hi) and columns
  // 32 dt + 16 (g4 % 2) + 4 (s % 4) .. + 4, and receives column 32 dt + l32 of those four rows.
  // Rows 16 c + vr and 16 c + 8 + vr (and the second half's, 32 further) share vr's swizzle.
  const int vr = 4 * hh + (l16 >> 2);
  int vofs[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const int col = 32 * dt + 16 * (g4 & 1) + 4 * (l16 & 3);
    vofs[dt] = vr * D + (((col >> 3) ^ swz_v(vr)) << 3) + (col & 7);
  }
  auto kread = [&](const uint16_t* kb, int c) { return ld16(kb + kofs[c]); };
  auto vread = [&](const uint16_t* vb, int c, int dt) {
    const u32x2_t lo = read_tr16(vb + 16 * c * D + vofs[dt]);
    const u32x2_t hi = read_tr16(vb + (16 * c + 8) * D + vofs[dt]);
    return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  };

  // scores of keys past the range end, and with a causal mask of keys after the lane's query,
  // go to -inf (uniform test: only half blocks that cross the end or the wave's diagonal)
  auto mask = [&](floatx16_t& sc, int bi, int h) {
    const int k0 = first_key(bi) + 32 * h, hi = end_key(bi);
    const bool diag = a.causal && k0 + 31 > qpos0;
    if (k0 + 32 <= hi && !diag) return;
    const int qp = qpos0 + l32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = k0 + 8 * (i >> 2) + 4 * hh + (i & 3);
      if (kk >= hi || (a.causal && kk > qp)) sc[i] = -INFINITY;
    }
  };
  // A half's maximum per query moves the reference (and rescales O and its sum) only when it
  // exceeds the reference by more than kLazy.  The check takes each lane's own maximum of the
  // offset scores (no query's maximum can pass the threshold unless one of its lanes' does);
  // only then are the two lanes of each query combined and the references that must move
  // moved: to the half's maximum rounded to bf16 (P then stays below about 2^kLazy), with the
  // already computed scores of that half shifted to the new offset.
  auto lane_max = [&](const floatx16_t& sc) {
    float m = sc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) m = fmaxf(m, sc[i]);
    return m;
  };
  auto rebase = [&](float mx, floatx16_t& sc) {
    if (__any(mx > thr)) {  // uniform: every lane takes part in the cross-lane maximum
      const float ms = pair_max(mx) - neg_mu;
      const bool up = ms > m_ref + kLazy;
      const uint32_t mb = pack_bf2(ms, 0.f) & 0xffffu;
      const float m_new = up ? __uint_as_float(mb << 16) : m_ref;
      const float alpha = up ? fast_exp2(m_ref - m_new) : 1.f;  // 0 from -inf
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
      l_acc *= alpha;
      m_ref = m_new;
      const float nm = (m_new == -INFINITY) ? 0.f : -m_new;
      const float shift = nm - neg_mu;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] += shift;
      neg_mu = nm;
      qb[0] = hh == 0 ? (pack_bf2(nm, 0.f) & 0xffffu) : 0u;
      thr = (m_new == -INFINITY) ? -INFINITY : kLazy;
    }
  };
  // One pipeline step on half H of block n (n % PS == R): its scores are in cur; the next half
  // ((n, 1), or (n + 1, 0) in the next stage) is multiplied into nxt meanwhile.  The step is
  // written as groups with scheduling fences between them, so that every LDS fragment is
  // requested three groups before the MFMA that uses it and the current half's softmax sits
  // between the next half's QK^T products:
  //   QK group c (8):  the MFMA of K chunk c (after the offset MFMA in group 0); exp, pack and
  //                    row sum of two P values;
  //                    request of K chunk c + 3
  //   PV group q (8):  the MFMA of key chunk q / 4 and O tile q % 4; request of V^T fragment
  //                    q + 3; a piece of the next half's per-lane maximum (the vector unit is
  //                    otherwise idle there)
  auto step = [&](auto R, auto H, floatx16_t& cur, floatx16_t& nxt, int n) {
    constexpr int r = decltype(R)::value, h = decltype(H)::value;
    if constexpr (h == 0) {
      wait_vm_lgkm0<LPW>();  // this wave's loads of block n + 1 have landed
      __builtin_amdgcn_s_barrier();
      issue(Stage<r + 3>{}, n + 3);
    }
    if (active) {
      // past the last block the next half's K is a copy whose scores are never used
      const uint16_t* kb = h == 0 ? stage(Stage<r>{}) + 32 * D : stage(Stage<r + 1>{});
      const uint16_t* vb = stage(Stage<r>{}) + KB * D + h * 32 * D;
      u32x4_t pf[2];
      u32x4_t kf[3] = {kread(kb, 0), kread(kb, 1), kread(kb, 2)};
      sched_fence();
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        if (c == 0) nxt = mfma32(ones, qb, floatx16_t{});
        nxt = mfma32(kf[c % 3], qf[c], nxt);
        // P slots 2 c, 2 c + 1 (of the 16 = P chunk c / 4, slots 2 (c % 4) .. + 1)
        const float p0 = fast_exp2(cur[2 * c]);
        const float p1 = fast_exp2(cur[2 * c + 1]);
        uint32_t pk = pack_bf2(p0, p1);
        asm volatile("" : "+v"(pk));  // computed here, in this group (not sunk to its first use)
        pf[c >> 2][c & 3] = pk;
        l_acc = add_bf2(pk, l_acc);
        if (c + 3 < NKC) kf[c % 3] = kread(kb, c + 3);
        sched_fence();
      }
      const bool has_next = (h == 0) || (n + 1 < nb);
      if (has_next) mask(nxt, h == 0 ? n : n + 1, 1 - h);
      u32x4_t vf[3] = {vread(vb, 0, 0), vread(vb, 0, 1), vread(vb, 0, 2)};
      float ma, mb;
      sched_fence();
      __builtin_amdgcn_s_setprio(1);  // P V groups: matrix work first (see above)
      sched_fence();
#pragma unroll
      for (int q = 0; q < 2 * NDT; ++q) {
        o[q % NDT] = mfma32(vf[q % 3], pf[q / NDT], o[q % NDT]);
        if (q + 3 < 2 * NDT) vf[q % 3] = vread(vb, (q + 3) / NDT, (q + 3) % NDT);
        // the next half's per-lane maximum, a piece per group (pinned there: not sunk to the use)
        // (scores 0-2, 3-5, then two more per group up to 14, 15 in group 6)
        if (q == 0) ma = fmaxf(fmaxf(nxt[0], nxt[1]), nxt[2]);
        if (q == 1) mb = fmaxf(fmaxf(nxt[3], nxt[4]), nxt[5]);
        if (q >= 2 && q <= 6 && q % 2 == 0) ma = fmaxf(fmaxf(ma, nxt[2 * q + 2]), nxt[2 * q + 3]);
        if (q >= 2 && q <= 6 && q % 2 == 1) mb = fmaxf(fmaxf(mb, nxt[2 * q + 2]), nxt[2 * q + 3]);
        if (q <= 6 && q % 2 == 0) asm volatile("" : "+v"(ma));
        if (q <= 6 && q % 2 == 1) asm volatile("" : "+v"(mb));
        sched_fence();
      }
      sched_fence();
      __builtin_amdgcn_s_setprio(0);
      sched_fence();
      if (has_next) rebase(fmaxf(ma, mb), nxt);
    }
  };

  if (nb > 0) {
    // a first (unused) load into stage 3 makes the loads in flight on entry to the loop the
    // same stages as on its back edge
    issue(Stage<3>{}, 0);
    issue(Stage<0>{}, 0);
    issue(Stage<1>{}, 1);
    issue(Stage<2>{}, 2);
    wait_vm_lgkm0<2 * LPW>();
    __builtin_amdgcn_s_barrier();
    floatx16_t sa, sb;
    if (active) {
      const uint16_t* kb = stage(Stage<0>{});
      sa = floatx16_t{};
#pragma unroll
      for (int c = 0; c < NKC; ++c) sa = mfma32(kread(kb, c), qf[c], sa);
      mask(sa, 0, 0);
      rebase(lane_max(sa), sa);
    }
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    static_assert(PS == 4, "the loop below is unrolled over a ring of four stages");
    for (int n = 0; n < nb; n += 4) {
      step(Stage<0>{}, H0{}, sa, sb, n);
      step(Stage<0>{}, H1{}, sb, sa, n);
      if (n + 1 >= nb) break;
      step(Stage<1>{}, H0{}, sa, sb, n + 1);
      step(Stage<1>{}, H1{}, sb, sa, n + 1);
      if (n + 2 >= nb) break;
      step(Stage<2>{}, H0{}, sa, sb, n + 2);
      step(Stage<2>{}, H1{}, sb, sa, n + 2);
      if (n + 3 >= nb) break;
      step(Stage<3>{}, H0{}, sa, sb, n + 3);
      step(Stage<3>{}, H1{}, sb, sa, n + 3);
    }
    wait_vm_lgkm0<0>();  // no load may still be writing this work-group's LDS at exit
  }

  // Output through LDS (the ring is free once every wave has read its last stage): each wave
  // writes its 32 rows of O / l as bf16 into [row][D + 8] rows of the ring, then stores whole
  // 256-byte rows as 16-byte pieces (16 lanes per row), to the output when the request has one
  // split, else to the split's partial slot; the split's exponent reference and row sum go
  // next to it.
  const float l_run = pair_sum(l_acc);  // every lane: the whole row sum of its query
  __syncthreads();
  if (!active) return;
  constexpr int OP = D + 8;  // staged row pitch (elements): 272 bytes
  uint16_t* ob = (wave < 3 ? st0 : wave < 6 ? st1 : st2) + (wave % 3) * 32 * OP;
  {
    const float inv = (l_run > 0.f) ? 1.0f / l_run : 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const floatx16_t& v = o[dt];
        *reinterpret_cast<u32x2_t*>(ob + l32 * OP + 32 * dt + 8 * i4 + 4 * hh) =
            u32x2_t{pack_bf2(v[4 * i4] * inv, v[4 * i4 + 1] * inv), pack_bf2(v[4 * i4 + 2] * inv, v[4 * i4 + 3] * inv)};
      }
    const int qr = row0 + l32;
    if (n_split_b > 1 && hh == 0 && qr < rows) {
      const long slot = ((qrow_base + qr) * a.Hq + hq) * a.n_split + by;
      a.part_ml[slot * 2] = m_ref;
      a.part_ml[slot * 2 + 1] = l_run;
    }
  }
  // the wave reads back only its own rows (LDS operations of a wave complete in order)
  uint16_t* part16 = reinterpret_cast<uint16_t*>(a.part_o);
#pragma unroll
  for (int k = 0; k < 32 / 4; ++k) {
    const int r = k * 4 + (lane >> 4), c = lane & 15;
    const int qr = row0 + r;
    if (qr >= rows) continue;
    const long orow = qrow_base + qr;
    uint16_t* dst = (n_split_b == 1) ? a.out + orow * a.Hq * D + hq * D
                                     : part16 + (((orow * a.Hq + hq) * a.n_split + by) * D);
    st16(dst + c * 8, ld16(ob + r * OP + c * 8));
  }
}

struct SplitCounts {
  int balanced, Hq, rows_per_req;
  int32_t n[kMaxBatch];
};

// Merge split partials in split order: O = sum_s 2^(m_s - m) O_s / sum_s 2^(m_s - m) l_s, with O_s
// the split's unnormalised fp32 output, or, from the pipelined kernel (NORM16), its normalised
// bf16 output O_s / l_s, weighted by 2^(m_s - m) l_s.  Every (max, sum) pair and every partial
// row of a thread is requested before any arithmetic.  With per-request splits a row of
// request b merges its own req_split[b] partials; a request with one split was written by the
// attention kernel itself.
template <int D, bool NORM16>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           uint16_t* __restrict__ out, int n_rh,
                                                           int stride, SplitCounts sc) {
  constexpr int DPT = NORM16 ? 8 : 4;  // dims per thread: one 16-byte load per split
  constexpr int TPR = D / DPT;         // threads per (row, head)
  constexpr int MS = 16;               // most splits a launch uses
  const int rh = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  if (rh >= n_rh) return;
  const int n_split = sc.balanced ? sc.n[rh / sc.Hq / sc.rows_per_req] : stride;
  if (n_split <= 1) return;
  const int d0 = (threadIdx.x % TPR) * DPT;
  const long base = static_cast<long>(rh) * stride;
  const uint16_t* part16 = reinterpret_cast<const uint16_t*>(part_o);
  float2 ml[MS];
  floatx4_t po[MS];
  u32x4_t ph[MS];
#pragma unroll
  for (int s = 0; s < MS; ++s)
    if (s < n_split) {
      ml[s] = *reinterpret_cast<const float2*>(part_ml + (base + s) * 2);
      if constexpr (NORM16) ph[s] = ld16(part16 + (base + s) * D + d0);
      else po[s] = *reinterpret_cast<const floatx4_t*>(part_o + (base + s) * D + d0);
    }
  float m = -INFINITY;
#pragma unroll
  for (int s = 0; s < MS; ++s)
    if (s < n_split) m = fmaxf(m, ml[s].x);
  floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f}, acc1 = acc;  // dims d0 .. + 3, d0 + 4 .. + 7
  float l = 0.f;
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    if (s >= n_split || ml[s].x == -INFINITY) continue;
    const float w = exp2f(ml[s].x - m);
    if constexpr (NORM16) {
      const float wl = w * ml[s].y;
      l += wl;
      const u32x4_t p = ph[s];
      acc += wl * floatx4_t{__uint_as_float(p[0] << 16), __uint_as_float(p[0] & 0xffff0000u),
                            __uint_as_float(p[1] << 16), __uint_as_float(p[1] & 0xffff0000u)};
      acc1 += wl * floatx4_t{__uint_as_float(p[2] << 16), __uint_as_float(p[2] & 0xffff0000u),
                             __uint_as_float(p[3] << 16), __uint_as_float(p[3] & 0xffff0000u)};
    } else {
      l += w * ml[s].y;
      acc += w * po[s];
    }
  }
  const float inv = (l > 0.f) ? 1.0f / l : 0.f;
  if constexpr (NORM16)
    st16(out + static_cast<long>(rh) * D + d0,
         u32x4_t{pack_bf2(acc[0] * inv, acc[1] * inv), pack_bf2(acc[2] * inv, acc[3] * inv),
                 pack_bf2(acc1[0] * inv, acc1[1] * inv), pack_bf2(acc1[2] * inv, acc1[3] * inv)});
  else
    *reinterpret_cast<u32x2_t*>(out + static_cast<long>(rh) * D + d0) =
        u32x2_t{pack_bf2(acc[0] * inv, acc[1] * inv), pack_bf2(acc[2] * inv, acc[3] * inv)};
}

template <int D, int NW>
void launch_attn_w(const AttnArgs& a, hipStream_t s) {
  const int group = a.Hq / a.Hkv;
  const int qt = a.q_tiles == 1 ? 1 : 2;
  const int tasks = group * ((a.rows_per_req + 16 * qt - 1) / (16 * qt));
  const int nx = (tasks + NW - 1) / NW;
  if (attention_pipe_path(a)) {
    // rows of eight units, each unit's nx task groups
    const int units = a.n_pairs * a.Hkv;
    hipLaunchKernelGGL((attention_pipe_kernel<8>), dim3((units + 7) / 8 * 8 * nx), dim3(64 * NW), 0, s, a);
    return;
  }
  dim3 grid(nx, a.n_split, a.n_req * a.Hkv);
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
  const int per = 256 / (D / (a.balanced ? 8 : 4));  // (row, head) pairs per work-group
  SplitCounts sc{};
  sc.balanced = a.balanced;
  sc.Hq = a.Hq;
  sc.rows_per_req = a.rows_per_req;
  for (int b = 0; b < a.n_req; ++b) sc.n[b] = a.req_split[b];
  if (a.balanced)
    hipLaunchKernelGGL((attn_combine_kernel<D, true>), dim3((n_rh + per - 1) / per), dim3(256), 0, s,
                       a.part_o, a.part_ml, a.out, n_rh, a.n_split, sc);
  else
    hipLaunchKernelGGL((attn_combine_kernel<D, false>), dim3((n_rh + per - 1) / per), dim3(256), 0, s,
                       a.part_o, a.part_ml, a.out, n_rh, a.n_split, sc);
}

}  // namespace

bool attention_pipe_path(const AttnArgs& a) {
  return a.D == 128 && a.n_waves == 8 && a.q_tiles != 1;
}

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
