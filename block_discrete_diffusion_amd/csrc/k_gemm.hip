// Dense projections on MFMA (QKV with RoPE and the K/V scatter fused into its epilogue, O-proj
// + residual, shared SwiGLU FFN) and the fused vocab head (projection + temperature +
// log-sum-exp + entropy + Gumbel-max; logits stay on chip).
//
// C[t][f] = sum_k X[t][k] * W[f][k]: both operands are k-contiguous ("NT"), which is the
// natural MFMA operand layout.  The weight tile is the A operand (rows = output features) and
// the activation tile the B operand (columns = tokens), so a lane's accumulator holds four
// consecutive output features of one token: one Philox call covers exactly the four vocab
// entries a lane owns, and stores are 16-byte (fp32) or 8-byte (bf16) per lane.
//
// Work-group tile BF features x BT tokens, 4 waves in a 2x2 grid, k-tile 64 double-buffered in
// LDS with rows padded to 144 B (16-lane ds_read_b128 phases hit distinct banks).  The tile ->
// work-group mapping keeps all token tiles of one weight tile on the same XCD so the weight
// tile is fetched from HBM once and re-read from that XCD's L2.
#include "dg_common.h"
#include "dg_kernels.h"

namespace dg {
namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;

template <int BF, int BT, bool DUAL>
struct Smem {
  uint16_t w[2][DUAL ? 2 : 1][BF][LDK];
  uint16_t x[2][BT][LDK];
};

// XCD-aware tile index: hardware hands consecutive work-group ids to the 8 XCDs round-robin;
// this makes consecutive logical tiles land on one XCD.
DG_DEVICE int xcd_remap(int bid, int G) {
  return (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
}

template <int BF, int BT, bool DUAL>
struct Mainloop {
  static constexpr int WF = BF / 2, WT = BT / 2, FM = WF / 16, TN = WT / 16;
  static constexpr int CW = BF * (BK / 8) / 256;  // 16-byte chunks per thread (weights)
  static constexpr int CX = BT * (BK / 8) / 256;  // 16-byte chunks per thread (activations)
  static_assert(CW >= 1 && CX >= 1, "tile too small for 256 threads");

  floatx4_t acc[FM][TN];
  floatx4_t acc1[DUAL ? FM : 1][DUAL ? TN : 1];

  // K: reduction length of this work-group; ldw: row stride of W (elements)
  DG_DEVICE void run(Smem<BF, BT, DUAL>& sm, const uint16_t* w0, const uint16_t* w1,
                     const uint16_t* x, int ldx, int n_tok, int t0, int K, int ldw) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wf = wave & 1, wt = wave >> 1;
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        acc[a][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (DUAL) acc1[a][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      }
    // two register sets of prefetched global tiles: two k-tiles are in flight while one is
    // multiplied out of LDS
    u32x4_t rw[2][CW], rw1[2][DUAL ? CW : 1], rx[2][CX];
    const int nk = K / BK;

    auto gload = [&](int set, int kt) {
      const int kof = kt * BK;
#pragma unroll
      for (int i = 0; i < CW; ++i) {
        const int c = tid + 256 * i, r = c >> 3, col = (c & 7) * 8;
        rw[set][i] = ld16(w0 + static_cast<long>(r) * ldw + kof + col);
        if constexpr (DUAL) rw1[set][i] = ld16(w1 + static_cast<long>(r) * ldw + kof + col);
      }
#pragma unroll
      for (int i = 0; i < CX; ++i) {
        const int c = tid + 256 * i, r = c >> 3, col = (c & 7) * 8;
        // rows past n_tok re-read the last row (unconditional loads keep the wait counts
        // exact); their outputs are never stored
        const int t = min(t0 + r, n_tok - 1);
        rx[set][i] = ld16(x + static_cast<long>(t) * ldx + kof + col);
      }
    };
    auto sstore = [&](int buf, int set) {
#pragma unroll
      for (int i = 0; i < CW; ++i) {
        const int c = tid + 256 * i, r = c >> 3, col = (c & 7) * 8;
        st16(&sm.w[buf][0][r][col], rw[set][i]);
        if constexpr (DUAL) st16(&sm.w[buf][DUAL ? 1 : 0][r][col], rw1[set][i]);
      }
#pragma unroll
      for (int i = 0; i < CX; ++i) {
        const int c = tid + 256 * i, r = c >> 3, col = (c & 7) * 8;
        st16(&sm.x[buf][r][col], rx[set][i]);
      }
    };
    auto compute = [&](int buf) {
#pragma unroll
      for (int ks = 0; ks < BK / 32; ++ks) {
        const int kk = ks * 32 + 8 * (lane >> 4);
        u32x4_t af[FM], af1[DUAL ? FM : 1], bx[TN];
#pragma unroll
        for (int a = 0; a < FM; ++a) {
          af[a] = ld16(&sm.w[buf][0][wf * WF + a * 16 + (lane & 15)][kk]);
          if constexpr (DUAL) af1[a] = ld16(&sm.w[buf][DUAL ? 1 : 0][wf * WF + a * 16 + (lane & 15)][kk]);
        }
#pragma unroll
        for (int b = 0; b < TN; ++b) bx[b] = ld16(&sm.x[buf][wt * WT + b * 16 + (lane & 15)][kk]);
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
          for (int b = 0; b < TN; ++b) {
            acc[a][b] = mfma16(af[a], bx[b], acc[a][b]);
            if constexpr (DUAL) acc1[a][b] = mfma16(af1[a], bx[b], acc1[a][b]);
          }
      }
    };

    // k-tile t lives in LDS buffer t & 1 and arrives through register set t & 1 (tile 0 is
    // stored at once); a register set is refilled with tile t + 2 right after its tile t went
    // to LDS, so tiles t + 1 and t + 2 are in flight while tile t is multiplied.
    // Loads are unconditional (tile index clamped to the last tile, which is then re-read) so
    // no branch surrounds a load and the compiler's wait counts stay exact.
    // The loop body always runs both halves and an odd last tile is handled after it: an exit
    // between the halves would give the loop header a second predecessor in which the other
    // register set was loaded last, and the compiler's wait counts would then drain every load.
    gload(0, 0);
    sstore(0, 0);
    gload(1, min(1, nk - 1));
    gload(0, min(2, nk - 1));
    __syncthreads();
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      compute(0);
      sched_fence();
      sstore(1, 1);
      gload(1, min(kt + 3, nk - 1));
      sched_fence();
      __syncthreads();
      compute(1);
      sched_fence();
      sstore(0, 0);
      gload(0, min(kt + 4, nk - 1));
      sched_fence();
      __syncthreads();
    }
    if (kt < nk) compute(0);  // odd tile count: the last tile sits in buffer 0
  }
};

// Fused QKV epilogue: the lane's four consecutive outputs f..f+3 of token t.  For q and k heads
// they are the rotation pairs (j, j + D/2) and (j + 1, j + 1 + D/2) of one head (packed weight
// row order), rotated with the table entries of (t, j) and (t, j + 1) (one 16-byte load) and
// stored as two bf16 pairs; for v heads they are four consecutive elements of one row.
DG_DEVICE void rope_store(const RopeArgs& r, int t, int f, const floatx4_t& v) {
  const int D = r.D, qk = (r.Hq + r.Hkv) * D;
  const int b = t / r.map.rows_per_req, i = t - b * r.map.rows_per_req;
  if (f < qk) {
    const int h = f / D, j = ((f - h * D) >> 2) * 2;
    float y0 = v[0], y1 = v[1], y2 = v[2], y3 = v[3];
    if (r.table) {
      const floatx4_t cs = *reinterpret_cast<const floatx4_t*>(r.table + (static_cast<long>(t) * (D / 2) + j) * 2);
      y0 = v[0] * cs[0] - v[1] * cs[1];
      y1 = v[1] * cs[0] + v[0] * cs[1];
      y2 = v[2] * cs[2] - v[3] * cs[3];
      y3 = v[3] * cs[2] + v[2] * cs[3];
    }
    uint16_t* dst = (h < r.Hq)
        ? r.q + static_cast<long>(t) * r.Hq * D + h * D
        : r.k_dst + ((static_cast<long>(b) * r.Hkv + (h - r.Hq)) * r.kv_cap + r.slot0[b] + i) * D;
    *reinterpret_cast<uint32_t*>(dst + j) = pack_bf2(y0, y2);
    *reinterpret_cast<uint32_t*>(dst + j + D / 2) = pack_bf2(y1, y3);
  } else {
    const int p = f - qk, g = p / D, dd = p - g * D;
    *reinterpret_cast<u32x2_t*>(r.v_dst + ((static_cast<long>(b) * r.Hkv + g) * r.kv_cap + r.slot0[b] + i) * D + dd) =
        u32x2_t{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
  }
}

// One lane's four consecutive outputs f..f+3 of token t (u: the up-projection sums of the
// SwiGLU pair).  With S > 1 the raw fp32 sums go to slice z of the partial buffer.
template <int EPI>
DG_DEVICE void store_out(const GemmArgs& a, int S, int z, int t, int f, const floatx4_t& v,
                         const floatx4_t& u) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU_BF16);
  if (S > 1) {
    float* p = a.part + z * a.part_stride + static_cast<long>(t) * a.N + f;
    *reinterpret_cast<floatx4_t*>(p) = v;
    if constexpr (DUAL) *reinterpret_cast<floatx4_t*>(p + a.part_stride / 2) = u;
  } else if constexpr (EPI == EPI_STORE_F32) {
    *reinterpret_cast<floatx4_t*>(a.out_f32 + static_cast<long>(t) * a.ldo + f) = v;
  } else if constexpr (EPI == EPI_ADD_F32) {
    floatx4_t* p = reinterpret_cast<floatx4_t*>(a.out_f32 + static_cast<long>(t) * a.ldo + f);
    floatx4_t o = *p;
    o += v;
    *p = o;
  } else if constexpr (EPI == EPI_ROPE_QKV) {
    rope_store(a.rope, t, f, v);
  } else if constexpr (EPI == EPI_SWIGLU_BF16) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = v[i] / (1.0f + expf(-v[i])) * u[i];
    *reinterpret_cast<u32x2_t*>(a.out_bf16 + static_cast<long>(t) * a.ldo + f) =
        u32x2_t{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])};
  } else {
    *reinterpret_cast<u32x2_t*>(a.out_bf16 + static_cast<long>(t) * a.ldo + f) =
        u32x2_t{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
  }
}

// Split-K: grid = tiles x S.  With S > 1 work-group (tile, z) multiplies the z-th K / S slice
// and stores the raw fp32 product to its own slice of the partial buffer; the consuming kernel
// adds the S slices in z order (a kernel boundary is the only synchronisation).
template <int BF, int BT, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a, int S) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU_BF16);
  using ML = Mainloop<BF, BT, DUAL>;
  __shared__ Smem<BF, BT, DUAL> sm;
  const int n_tt = (a.n_tok + BT - 1) / BT, n_ft = a.N / BF;
  const int L = xcd_remap(blockIdx.x, n_tt * n_ft * S);
  const int tile = L / S, z = L % S;
  const int ft = tile / n_tt, tt = tile % n_tt;
  const int f0 = ft * BF, t0 = tt * BT;
  const int kz = a.K / S, k0 = z * kz;
  const uint16_t* w0;
  const uint16_t* w1 = nullptr;
  if (a.n_seg > 0) {
    int sg = 0;
    while (sg + 1 < a.n_seg && f0 >= a.seg_start[sg + 1]) ++sg;
    w0 = a.seg_w[sg] + static_cast<long>(f0 - a.seg_start[sg]) * a.K + k0;
  } else {
    w0 = a.w0 + static_cast<long>(f0) * a.K + k0;
    if (DUAL) w1 = a.w1 + static_cast<long>(f0) * a.K + k0;
  }
  ML ml;
  ml.run(sm, w0, w1, a.x + k0, a.ldx, a.n_tok, t0, kz, a.K);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wf = wave & 1, wt = wave >> 1;
#pragma unroll
  for (int fm = 0; fm < ML::FM; ++fm)
#pragma unroll
    for (int tn = 0; tn < ML::TN; ++tn) {
      const int t = t0 + wt * ML::WT + tn * 16 + (lane & 15);
      const int f = f0 + wf * ML::WF + fm * 16 + 4 * (lane >> 4);
      if (t >= a.n_tok) continue;
      store_out<EPI>(a, S, z, t, f, ml.acc[fm][tn], ml.acc1[DUAL ? fm : 0][DUAL ? tn : 0]);
    }
}

// ------------------------------------------------------------------------------------------
// Large-tile path (from 1024 tokens).  A work-group of 8 waves owns 256 weight rows (for the
// SwiGLU pair: 128 gate rows + the same 128 up rows) x 128 tokens; wave (wa, wt) = (w & 3,
// w >> 2) multiplies 64 weight rows (32 gate + 32 up) by 64 tokens.
//
// Both operands go from global memory straight into LDS with gfx950's global_load_lds_dwordx4:
// lane l's 16 bytes land at the instruction's LDS base + 16 l, so one instruction fills a 1 KB
// block of 8 rows x 128 bytes (64 k).  Whole 128-byte row segments per instruction matter: on
// this part, instructions that touch 16 rows x 64 bytes at a 4 KB pitch read L2 about 4x slower
// than 8 rows x 128 bytes.  Inside a block, row r's 16-byte chunk c sits at slot c ^ ((r16 >> 1)
// & 7), r16 being the row's index within its 16-row MFMA fragment (the lane loading slot s of
// row r fetches chunk s ^ ((r16 >> 1) & 7)): the 16 lanes of each ds_read_b128 phase then hit
// 16 distinct 4-bank groups, so fragment reads are conflict-free.  No VGPRs or LDS write
// instructions stage the tiles.
//
// A stage is one k-step of 64 (32 weight blocks + 16 token blocks = 48 KB); a ring of NS = 3
// stages keeps the next k-step in flight while one is multiplied, with one barrier per k-step.
// The wait before the barrier names the number of this wave's loads allowed to stay in flight
// (6 per later stage); every stage is issued unconditionally (the tile index is clamped, so the
// last stages re-load the final k-step into buffers nobody reads again), which keeps that
// count exact.
// ------------------------------------------------------------------------------------------
constexpr int DL_BK = 64;  // k per stage

// Tile of RA weight rows (DUAL: RA / 2 gate + RA / 2 up rows) x BT tokens; NWA x NWT waves, each
// multiplying RA / NWA weight rows by BT / NWT tokens; a ring of NS stages of (RA + BT) / 8 1 KB
// blocks each (at most the 160 KB of LDS).
template <int RA_, int BT_, int NWA_, int NWT_, int NS_>
struct DlCfg {
  static constexpr int RA = RA_, BT = BT_, NWA = NWA_, NWT = NWT_, NW = NWA_ * NWT_, NS = NS_;
  static constexpr int BLK = (RA + BT) / 8;  // 1 KB blocks (8 rows x 128 B) per stage
  static_assert(BLK % NW == 0, "blocks per stage must split evenly over the waves");
  static_assert(NS >= 2 && NS * BLK <= 160, "the ring must fit the LDS");
  static constexpr int PW = BLK / NW;        // blocks each wave loads per stage
  static constexpr int FM = RA / NWA / 16;   // 16-row weight fragments per wave
  static constexpr int WT = BT / NWT;        // tokens per wave
  static constexpr int TN = WT / 16;         // 16-token fragments per wave
};
// many rows: one work-group per CU, 256 x 128 (3 stages) or 256 x 256 (2 stages)
using DlBig128 = DlCfg<256, 128, 4, 4, 3>;
using DlBig256 = DlCfg<256, 256, 4, 4, 2>;

template <class C>
struct DlSmem {
  uint16_t b[C::NS][C::BLK][512];
};


template <class C, bool DUAL>
struct DlMainloop {
  static constexpr int NS = C::NS, PW = C::PW, FM = C::FM, TN = C::TN;
  static_assert(!DUAL || FM % 2 == 0, "gate and up fragments in pairs");
  // acc[i][j]: weight fragment i (DUAL: the first FM / 2 gate, the rest up) x token fragment j
  floatx4_t acc[FM][TN];

  DG_DEVICE void run(DlSmem<C>& sm, const uint16_t* w0, const uint16_t* w1, const uint16_t* x,
                     int ldx, int n_tok, int t0, int K, int ldw) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wa = wave % C::NWA, wt = wave / C::NWA;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    // source of this lane in each block its wave loads: blocks below RA / 8 hold weight rows
    // 8 j .. 8 j + 7 (DUAL: the first half gate, the second up), the others tokens
    const uint16_t* src[PW];
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int j = wave * PW + i;
      const int r16 = (j & 1) * 8 + (lane >> 3);
      const int kof = 8 * ((lane & 7) ^ ((r16 >> 1) & 7));
      if (j < C::RA / 8) {
        const int r = j * 8 + (lane >> 3);
        src[i] = (DUAL && r >= C::RA / 2) ? w1 + static_cast<long>(r - C::RA / 2) * ldw + kof
                                          : w0 + static_cast<long>(r) * ldw + kof;
      } else {
        // rows past n_tok re-read the last row; their outputs are never stored
        const int t = min(t0 + (j - C::RA / 8) * 8 + (lane >> 3), n_tok - 1);
        src[i] = x + static_cast<long>(t) * ldx + kof;
      }
    }
    // fragment read offset (elements) of this lane inside a 16-row pair of blocks, per k half
    const int r16 = lane & 15;
    int fofs[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      fofs[h] = (r16 >> 3) * 512 + (r16 & 7) * 64 + 8 * ((4 * h + (lane >> 4)) ^ ((r16 >> 1) & 7));
    const int nk = K / DL_BK;
    auto issue = [&](int st, int kt) {
#pragma unroll
      for (int i = 0; i < PW; ++i)
        __builtin_amdgcn_global_load_lds(
            static_cast<const void*>(src[i] + kt * DL_BK),
            (__attribute__((address_space(3))) void*)(&sm.b[st][wave * PW + i][0]), 16, 0, 0);
    };
    auto compute = [&](int st) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4_t af[FM], bx[TN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          // 16-row weight fragment index (pairs of blocks)
          constexpr int HF = FM / 2;
          const int g = DUAL ? (i < HF ? wa * HF + i : C::RA / 32 + wa * HF + (i - HF)) : wa * FM + i;
          af[i] = ld16(&sm.b[st][2 * g][fofs[h]]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) bx[j] = ld16(&sm.b[st][C::RA / 8 + 2 * (wt * TN + j)][fofs[h]]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(af[i], bx[j], acc[i][j]);
      }
    };
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) issue(st, min(st, nk - 1));
    for (int kt = 0; kt < nk; ++kt) {
      // this wave's loads of stage kt have landed (NS - 2 later stages may still be in
      // flight) and its fragment reads of stage kt - 1 are done; after the barrier the same
      // holds for every wave, so stage kt is complete and buffer (kt - 1) % NS is free
      wait_vm_lgkm0<PW * (NS - 2)>();
      __builtin_amdgcn_s_barrier();
      issue((kt + NS - 1) % NS, min(kt + NS - 1, nk - 1));
      compute(kt % NS);
    }
    // no load may still be writing this work-group's LDS when it exits
    wait_vm_lgkm0<0>();
  }
};

// Fused QKV epilogue through LDS (the large tiles): after the last k-step the ring is free; each
// lane rotates its rotation pairs as rope_store does and writes the bf16 results into a
// [token][feature] tile at their place in the head (d = j, j + 1 and j + D/2, j + D/2 + 1), then
// every thread writes 16-byte pieces of whole head rows (16 consecutive threads cover one
// 256-byte row of D = 128).  The per-lane stores of rope_store cover 32 bytes per token row
// each; here each request stores whole rows.  Needs work-group tiles that hold whole heads of q,
// k or v (RA a multiple of D at the q/k and k/v boundaries).  Row pitch 528 bytes: the 4-byte
// writes of 16 tokens x 4 lanes and the 16-byte reads hit distinct banks.
constexpr int kQkvPitch = 264;  // bf16 elements per staged token row (256 features + 8)
template <class C, class Acc>
DG_DEVICE void qkv_staged_store(const RopeArgs& r, uint16_t* tile, const Acc& acc, int n_tok, int t0,
                                int f0, int wa, int wt) {
  constexpr int FM = C::RA / C::NWA / 16, TN = C::WT / 16, WF = C::RA / C::NWA;
  static_assert(C::RA == 256, "one staged row per token holds 256 features");
  const int lane = threadIdx.x & 63, l16 = lane & 15, j4 = lane >> 4;
  const int D = r.D, qk = (r.Hq + r.Hkv) * D;
  __syncthreads();  // every wave has read its last fragments from the ring
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int tl = wt * C::WT + tn * 16 + l16, fl = wa * WF + fm * 16 + 4 * j4;
      const int t = min(t0 + tl, n_tok - 1);  // rows past n_tok are staged but never stored
      const int f = f0 + fl;
      const floatx4_t v = acc[fm][tn];
      uint16_t* row = tile + tl * kQkvPitch;
      if (f < qk) {
        const int hb = ((f - f0) / D) * D, j = ((f - f0 - hb) >> 2) * 2;
        float y0 = v[0], y1 = v[1], y2 = v[2], y3 = v[3];
        if (r.table) {
          const floatx4_t cs = *reinterpret_cast<const floatx4_t*>(r.table + (static_cast<long>(t) * (D / 2) + j) * 2);
          y0 = v[0] * cs[0] - v[1] * cs[1];
          y1 = v[1] * cs[0] + v[0] * cs[1];
          y2 = v[2] * cs[2] - v[3] * cs[3];
          y3 = v[3] * cs[2] + v[2] * cs[3];
        }
        *reinterpret_cast<uint32_t*>(row + hb + j) = pack_bf2(y0, y2);
        *reinterpret_cast<uint32_t*>(row + hb + j + D / 2) = pack_bf2(y1, y3);
      } else {
        *reinterpret_cast<u32x2_t*>(row + fl) = u32x2_t{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
      }
    }
  __syncthreads();
  constexpr int PIECES = C::BT * 32;  // 16-byte pieces of the staged tile
#pragma unroll
  for (int i = 0; i < (PIECES + 64 * C::NW - 1) / (64 * C::NW); ++i) {
    const int c = threadIdx.x + 64 * C::NW * i;
    if (c >= PIECES) break;
    const int tl = c >> 5, pc = c & 31, t = t0 + tl;
    if (t >= n_tok) continue;
    const int f = f0 + pc * 8;                 // first feature of the piece
    const int h = f / D, dd = f - h * D;       // head (q heads, then k, then v) and dim
    const int b = t / r.map.rows_per_req, i_r = t - b * r.map.rows_per_req;
    uint16_t* dst;
    if (f < r.Hq * D) dst = r.q + static_cast<long>(t) * r.Hq * D + f;
    else if (f < qk) dst = r.k_dst + ((static_cast<long>(b) * r.Hkv + (h - r.Hq)) * r.kv_cap + r.slot0[b] + i_r) * D + dd;
    else dst = r.v_dst + ((static_cast<long>(b) * r.Hkv + (h - r.Hq - r.Hkv)) * r.kv_cap + r.slot0[b] + i_r) * D + dd;
    st16(dst, ld16(tile + tl * kQkvPitch + pc * 8));
  }
}

// Residual-adding epilogue through LDS (unsplit large tiles): the fp32 products go into a
// [token][feature] tile in the freed ring (row pitch RA + 4 floats), then every thread adds
// 16-byte pieces of whole output rows to h (one read and one write of 16 bytes each, 32
// consecutive threads covering a 512-byte row at RA = 128) instead of each lane updating 16
// bytes of 16 rows.
template <class C, class Acc>
DG_DEVICE void add_staged_store(const GemmArgs& a, float* tile, const Acc& acc, int t0, int f0, int wa,
                                int wt) {
  constexpr int FM = C::RA / C::NWA / 16, TN = C::WT / 16, WF = C::RA / C::NWA, P = C::RA + 4;
  const int lane = threadIdx.x & 63, l16 = lane & 15, j4 = lane >> 4;
  __syncthreads();  // every wave has read its last fragments from the ring
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      *reinterpret_cast<floatx4_t*>(tile + (wt * C::WT + tn * 16 + l16) * P + wa * WF + fm * 16 + 4 * j4) = acc[fm][tn];
  __syncthreads();
  constexpr int PR = C::RA / 4, PIECES = C::BT * PR;  // 16-byte pieces per row, per tile
#pragma unroll
  for (int i = 0; i < (PIECES + 64 * C::NW - 1) / (64 * C::NW); ++i) {
    const int c = threadIdx.x + 64 * C::NW * i;
    if (c >= PIECES) break;
    const int tl = c / PR, pc = c % PR, t = t0 + tl;
    if (t >= a.n_tok) continue;
    floatx4_t* o = reinterpret_cast<floatx4_t*>(a.out_f32 + static_cast<long>(t) * a.ldo + f0 + pc * 4);
    floatx4_t v = *o;
    v += *reinterpret_cast<const floatx4_t*>(tile + tl * P + pc * 4);
    *o = v;
  }
}

template <class C, int EPI>
__global__ __launch_bounds__(64 * C::NW) void gemm_dl_kernel(GemmArgs a, int S) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU_BF16);
  constexpr int BF = DUAL ? C::RA / 2 : C::RA;  // output features per tile
  constexpr int WF = BF / C::NWA;               // per wave
  using ML = DlMainloop<C, DUAL>;
  __shared__ DlSmem<C> sm;
  const int n_tt = (a.n_tok + C::BT - 1) / C::BT, n_ft = a.N / BF;
  const int L = xcd_remap(blockIdx.x, n_tt * n_ft * S);
  const int tile = L / S, z = L % S;
  const int ft = tile / n_tt, tt = tile % n_tt;
  const int f0 = ft * BF, t0 = tt * C::BT;
  const int kz = a.K / S, k0 = z * kz;
  const uint16_t* w0 = a.w0 + static_cast<long>(f0) * a.K + k0;
  const uint16_t* w1 = DUAL ? a.w1 + static_cast<long>(f0) * a.K + k0 : nullptr;
  ML ml;
  ml.run(sm, w0, w1, a.x + k0, a.ldx, a.n_tok, t0, kz, a.K);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wa = wave % C::NWA, wt = wave / C::NWA;
  constexpr int NF = DUAL ? ML::FM / 2 : ML::FM;
  if constexpr (EPI == EPI_ADD_F32 && sizeof(DlSmem<C>) >= C::BT * (C::RA + 4) * 4) {
    if (S == 1) {
      add_staged_store<C>(a, reinterpret_cast<float*>(&sm), ml.acc, t0, f0, wa, wt);
      return;
    }
  }
  if constexpr (EPI == EPI_ROPE_QKV && C::RA == 256 && sizeof(DlSmem<C>) >= C::BT * kQkvPitch * 2) {
    const RopeArgs& r = a.rope;
    if ((r.D == 64 || r.D == 128) && ((r.Hq + r.Hkv) * r.D) % BF == 0 && (r.Hkv * r.D) % BF == 0) {
      qkv_staged_store<C>(r, reinterpret_cast<uint16_t*>(&sm), ml.acc, a.n_tok, t0, f0, wa, wt);
      return;
    }
  }
#pragma unroll
  for (int fm = 0; fm < NF; ++fm)
#pragma unroll
    for (int tn = 0; tn < ML::TN; ++tn) {
      const int t = t0 + wt * C::WT + tn * 16 + (lane & 15);
      const int f = f0 + wa * WF + fm * 16 + 4 * (lane >> 4);
      if (t >= a.n_tok) continue;
      store_out<EPI>(a, S, z, t, f, ml.acc[fm][tn], ml.acc[DUAL ? fm + NF : fm][tn]);
    }
}

__global__ __launch_bounds__(256) void swiglu_reduce_kernel(const float* __restrict__ part,
                                                            long part_stride, int split,
                                                            uint16_t* __restrict__ act, long n4) {
  const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n4) return;
  floatx4_t gz[kMaxParts], uz[kMaxParts];
#pragma unroll
  for (int z = 0; z < kMaxParts; ++z)
    if (z < split) {
      gz[z] = *reinterpret_cast<const floatx4_t*>(part + z * part_stride + i * 4);
      uz[z] = *reinterpret_cast<const floatx4_t*>(part + z * part_stride + part_stride / 2 + i * 4);
    }
  floatx4_t g = floatx4_t{0.f, 0.f, 0.f, 0.f}, u = g;
#pragma unroll
  for (int z = 0; z < kMaxParts; ++z)
    if (z < split) { g += gz[z]; u += uz[z]; }
  float y[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) y[q] = g[q] / (1.0f + expf(-g[q])) * u[q];
  *reinterpret_cast<u32x2_t*>(act + i * 4) = u32x2_t{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3])};
}

// ------------------------------------------------------------------------------------------
// Fused vocab head.  Per lane and token: the four logits z of vocab entries v0..v0+3 (v0 a
// multiple of 4) give t = z * (1 / T), Gumbel noise from one Philox call (counter v0>>2,
// position, step, request), and running max / sum(exp) / sum(exp*t) / best (score, index, t).
// Lanes of the same token merge with two butterfly steps; one record per (token, wave slice of
// BF/2 vocab entries) goes to `part`.  The exponentials and the noise's logarithms use the
// hardware base-2 instructions (about one ulp each): the statistics are float32 sums either
// way, and the Gumbel-max pick only depends on them at ties closer than that.
// ------------------------------------------------------------------------------------------
struct Stat {
  float m, s, st, bs, bt, tc;
  int bi;
};

DG_DEVICE Stat merge_stat(const Stat& a, const Stat& b) {
  Stat r;
  if (a.m == -INFINITY) {
    r = b;
  } else if (b.m == -INFINITY) {
    r = a;
  } else {
    r.m = fmaxf(a.m, b.m);
    const float ea = __expf(a.m - r.m), eb = __expf(b.m - r.m);
    r.s = a.s * ea + b.s * eb;
    r.st = a.st * ea + b.st * eb;
  }
  const bool take_b = (b.bs > a.bs) || (b.bs == a.bs && b.bi < a.bi);
  r.bs = take_b ? b.bs : a.bs;
  r.bi = take_b ? b.bi : a.bi;
  r.bt = take_b ? b.bt : a.bt;
  r.tc = (a.tc == a.tc) ? a.tc : b.tc;  // NaN = current token not in this range
  return r;
}

DG_DEVICE Stat shfl_stat(const Stat& a, int o) {
  Stat r;
  r.m = __shfl_xor(a.m, o, 64);
  r.s = __shfl_xor(a.s, o, 64);
  r.st = __shfl_xor(a.st, o, 64);
  r.bs = __shfl_xor(a.bs, o, 64);
  r.bt = __shfl_xor(a.bt, o, 64);
  r.tc = __shfl_xor(a.tc, o, 64);
  r.bi = __shfl_xor(a.bi, o, 64);
  return r;
}

// Statistics of one wave's logits: FM 16-entry vocab fragments from v_base (64 entries, one
// slice) x TN 16-row token fragments from t_base.
template <int FM, int TN>
DG_DEVICE void head_stats(const HeadArgs& a, const floatx4_t (&acc)[FM][TN], int v_base, int t_base,
                          int slice, int n_slices) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int t = t_base + tn * 16 + (lane & 15);
    const bool ok = t < a.n_rows;
    const int tc = ok ? t : 0;
    const int b = tc / a.map.rows_per_req;
    const int pos = a.map.pos0[b] + (tc - b * a.map.rows_per_req);
    const int cur = ok ? a.cur_tok[tc] : -1;
    const float inv_temp = 1.0f / a.temp[b];
    float tv[FM][4];
    Stat st;
    st.m = -INFINITY; st.s = 0.f; st.st = 0.f; st.bs = -INFINITY; st.bt = 0.f; st.tc = NAN;
    st.bi = 0x7fffffff;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int v0 = v_base + fm * 16 + 4 * (lane >> 4);
      const philox_out rnd = philox4x32_10(static_cast<uint32_t>(v0 >> 2), static_cast<uint32_t>(pos),
                                           static_cast<uint32_t>(a.step[b]),
                                           (static_cast<uint32_t>(a.map.slot[b]) << 8) | kStreamGumbel, a.k0, a.k1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float z = acc[fm][tn][i];
        const float t_ = z * inv_temp;
        tv[fm][i] = t_;
        const float sc = t_ + gumbel(rnd.x[i]);
        if (sc > st.bs) { st.bs = sc; st.bi = v0 + i; st.bt = t_; }
        st.m = fmaxf(st.m, t_);
        if (v0 + i == cur) st.tc = t_;
        if (a.dbg_logits && ok) a.dbg_logits[static_cast<long>(t) * a.V + v0 + i] = z;
      }
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __expf(tv[fm][i] - st.m);
        st.s += e;
        st.st += e * tv[fm][i];
      }
    st = merge_stat(st, shfl_stat(st, 16));
    st = merge_stat(st, shfl_stat(st, 32));
    if (ok && (lane >> 4) == 0) {
      float* p = a.part + (static_cast<long>(t) * n_slices + slice) * 8;
      *reinterpret_cast<floatx4_t*>(p) = floatx4_t{st.m, st.s, st.st, st.bs};
      *reinterpret_cast<floatx4_t*>(p + 4) = floatx4_t{__int_as_float(st.bi), st.bt, st.tc, 0.f};
    }
  }
}

template <int BF, int BT>
__global__ __launch_bounds__(256) void head_kernel(HeadArgs a) {
  using ML = Mainloop<BF, BT, false>;
  __shared__ Smem<BF, BT, false> sm;
  const int n_tt = (a.n_rows + BT - 1) / BT, n_ft = a.V / BF;
  const int L = xcd_remap(blockIdx.x, n_tt * n_ft);
  const int ft = L / n_tt, tt = L % n_tt;
  const int f0 = ft * BF, t0 = tt * BT;
  ML ml;
  ml.run(sm, a.w + static_cast<long>(f0) * a.K, nullptr, a.f, a.K, a.n_rows, t0, a.K, a.K);
  const int wave = threadIdx.x >> 6, wf = wave & 1, wt = wave >> 1;
  static_assert(ML::WF == 64, "one statistics slice per wave");
  head_stats(a, ml.acc, f0 + wf * ML::WF, t0 + wt * ML::WT, (f0 + wf * ML::WF) / ML::WF, a.V / ML::WF);
}

// The same head on the direct-to-LDS mainloop: 256 vocab entries x BT rows per work-group, 64
// vocab entries (one statistics slice) x BT / NWT rows per wave.  Same k order and slices, so
// the statistics are bit-identical to the kernel above.
template <class C>
__global__ __launch_bounds__(64 * C::NW) void head_dl_kernel(HeadArgs a) {
  static_assert(C::RA / C::NWA == 64, "one statistics slice per wave");
  using ML = DlMainloop<C, false>;
  __shared__ DlSmem<C> sm;
  const int n_tt = (a.n_rows + C::BT - 1) / C::BT, n_ft = a.V / C::RA;
  const int L = xcd_remap(blockIdx.x, n_tt * n_ft);
  const int ft = L / n_tt, tt = L % n_tt;
  const int f0 = ft * C::RA, t0 = tt * C::BT;
  ML ml;
  ml.run(sm, a.w + static_cast<long>(f0) * a.K, nullptr, a.f, a.K, a.n_rows, t0, a.K, a.K);
  const int wave = threadIdx.x >> 6, wa = wave % C::NWA, wt = wave / C::NWA;
  head_stats(a, ml.acc, f0 + wa * 64, t0 + wt * C::WT, (f0 + wa * 64) / 64, a.V / 64);
}

// One work-group (4 waves) per row: thread t merges slices t, t + 256, ... (two 16-byte loads
// each, all issued first), then the wave and the 4 wave results merge in a fixed order.
// Row r of the call (request r / rows_per_req) writes its statistics at the request's slot.
__global__ __launch_bounds__(256) void head_merge_kernel(const float* __restrict__ part, int n_rows,
                                                         int n_slices, int slice_w,
                                                         const int32_t* __restrict__ cur_tok,
                                                         uint32_t* __restrict__ err,
                                                         int32_t* cand, float* t_cand, float* t_cur,
                                                         float* lse, float* ent, RowMap map) {
  constexpr int PER = 8;  // slices per thread held in registers (n_slices <= 2048)
  __shared__ float wm[4][8];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  floatx4_t p0[PER], p1[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int j = min(tid + 256 * k, n_slices - 1);  // clamped; merged only when in range
    const float* p = part + (static_cast<long>(row) * n_slices + j) * 8;
    p0[k] = *reinterpret_cast<const floatx4_t*>(p);
    p1[k] = *reinterpret_cast<const floatx4_t*>(p + 4);
  }
  Stat st;
  st.m = -INFINITY; st.s = 0.f; st.st = 0.f; st.bs = -INFINITY; st.bt = 0.f; st.tc = NAN;
  st.bi = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (tid + 256 * k >= n_slices) continue;
    Stat o;
    o.m = p0[k][0]; o.s = p0[k][1]; o.st = p0[k][2]; o.bs = p0[k][3];
    o.bi = __float_as_int(p1[k][0]); o.bt = p1[k][1]; o.tc = NAN;
    st = merge_stat(st, o);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) st = merge_stat(st, shfl_stat(st, o));
  if (lane == 0) {
    wm[w][0] = st.m; wm[w][1] = st.s; wm[w][2] = st.st; wm[w][3] = st.bs;
    wm[w][4] = __int_as_float(st.bi); wm[w][5] = st.bt;
  }
  __syncthreads();
  if (tid != 0) return;
  Stat r = st;
#pragma unroll
  for (int v = 1; v < 4; ++v) {
    Stat o;
    o.m = wm[v][0]; o.s = wm[v][1]; o.st = wm[v][2]; o.bs = wm[v][3];
    o.bi = __float_as_int(wm[v][4]); o.bt = wm[v][5]; o.tc = NAN;
    r = merge_stat(r, o);
  }
  const float l = r.m + logf(r.s);
  const int rb = row / map.rows_per_req;
  const long orow = static_cast<long>(map.slot[rb]) * map.rows_per_req + (row - rb * map.rows_per_req);
  lse[orow] = l;
  ent[orow] = l - r.st / r.s;
  cand[orow] = r.bi;
  t_cand[orow] = r.bt;
  int x = cur_tok[row];
  if (static_cast<unsigned>(x) >= static_cast<unsigned>(n_slices * slice_w)) {  // never read past the row
    *err = kDevErrTokenRange;
    x = x < 0 ? 0 : n_slices * slice_w - 1;
  }
  t_cur[orow] = part[(static_cast<long>(row) * n_slices + x / slice_w) * 8 + 6];
}

template <int BF, int BT, int EPI>
void launch_cfg(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.n_tok + BT - 1) / BT) * (a.N / BF);
  const int S = a.split > 1 ? a.split : 1;
  hipLaunchKernelGGL((gemm_kernel<BF, BT, EPI>), dim3(tiles * S), dim3(256), 0, s, a, S);
}

// Tile shape.  Up to 256 tokens (one canvas) 64 x 64 tiles: measured at these shapes they beat
// both wider token tiles (fewer, longer work-groups) and narrower feature tiles.  From 1024
// tokens 128 x 128 tiles (64 x 64 per wave: half the LDS fragment traffic per MFMA) where every
// weight segment is a whole number of tiles; otherwise 64 x 128 tiles when there are plenty of
// them, else 64 x 64 / 32 x 64.
bool segments_fit(const GemmArgs& a, int bf) {
  if (a.N % bf) return false;
  for (int sg = 0; sg < a.n_seg; ++sg)
    if ((a.seg_start[sg + 1] - a.seg_start[sg]) % bf) return false;
  return true;
}

template <int EPI>
void pick_tile(const GemmArgs& a, int* bf, int* bt) {
  const int tt64 = (a.n_tok + 63) / 64, tt128 = (a.n_tok + 127) / 128;
  if (EPI != EPI_SWIGLU_BF16 && a.n_tok >= 1024 && segments_fit(a, 128)) { *bf = 128; *bt = 128; }
  else if (a.n_tok >= 128 && (a.N / 64) * tt128 >= 512) { *bf = 64; *bt = 128; }
  else if (a.n_tok <= 256 || (a.N / 64) * tt64 >= 256 || EPI == EPI_SWIGLU_BF16) { *bf = 64; *bt = 64; }
  else { *bf = 32; *bt = 64; }
}

// Which direct-to-LDS configuration runs a GEMM (or none: the LDS-tiled kernel).
//  * From 1024 tokens the large tiles, where the weights come in whole tiles (256 rows; 128 for
//    the SwiGLU pair) and the grid fills the chip: one work-group per CU (its LDS ring takes
//    most of the CU), so below 256 work-groups the LDS-tiled kernel, which runs two per CU, is
//    faster.  256-token tiles (1.5x the MFMAs per staged byte) where there are 256 of them,
//    else 128-token tiles.  Measured at 2048 tokens: QKV 54.6 -> 42.4 us (128-token tiles),
//    shared gate/up 100 -> 72 us (256-token tiles).
//  * Up to 256 tokens (one canvas) 64 x 64 tiles with 8 waves and 8 stages for the QKV
//    projection (in the step: 15.7 -> 14.2 us) and, split in two K slices, for the fp32
//    projections (O-projection 11.1 -> 10.6 us, shared down at split 2 instead of 4
//    15.7 -> 15.1 us, and the combine, which then adds two slices fewer, 9.2 -> 8.3 us).  The
//    SwiGLU pair on 64 + 64 gate/up rows x 64 tokens with 8 waves (4 x 2) and 6 stages:
//    22.5 -> 20.2 us in the step; 64 x 64 tiles were faster only with the weights warm in the
//    last-level cache.
using DlSmallW8 = DlCfg<64, 64, 2, 4, 8>;
using DlSmallPair = DlCfg<128, 64, 4, 2, 6>;
//  * The residual-adding projections (O-projection, shared down) from 1024 rows on 128 x 128
//    tiles with 16 waves and 4 stages, unsplit, where that gives a chip's worth of tiles:
//    measured at 2048 rows the O-projection takes 25.4 us against 24.2 us in two K slices,
//    but then writes no partial slices for the router kernel to add (27.4 -> 15.7 us there).
using DlMid128 = DlCfg<128, 128, 4, 4, 4>;
enum DlKind { DL_NONE = 0, DL_BIG128, DL_BIG256, DL_SMALL_W8, DL_SMALL_PAIR, DL_MID128 };

template <int EPI, class C>
int dl_tiles(const GemmArgs& a) {
  constexpr int BF = (EPI == EPI_SWIGLU_BF16) ? C::RA / 2 : C::RA;
  return ((a.n_tok + C::BT - 1) / C::BT) * (a.N / BF);
}

template <int EPI>
int dl_kind(const GemmArgs& a, int S) {
  constexpr bool DUAL = (EPI == EPI_SWIGLU_BF16);
  if (a.n_seg != 0 || a.K % (DL_BK * S) != 0) return DL_NONE;
  if (a.n_tok <= 256) return (a.N % 64 != 0) ? DL_NONE : DUAL ? DL_SMALL_PAIR : DL_SMALL_W8;
  if (EPI == EPI_ADD_F32 && S == 1 && a.n_tok >= 1024 && a.N % 128 == 0 && dl_tiles<EPI, DlMid128>(a) >= 256)
    return DL_MID128;
  if (a.n_tok < 1024 || a.N % (DUAL ? 128 : 256) != 0) return DL_NONE;
  if (S == 1 && dl_tiles<EPI, DlBig256>(a) >= 256) return DL_BIG256;
  if (dl_tiles<EPI, DlBig128>(a) * S >= 256) return DL_BIG128;
  return DL_NONE;
}

template <int EPI, class C>
void launch_dl(const GemmArgs& a, int S, hipStream_t s) {
  hipLaunchKernelGGL((gemm_dl_kernel<C, EPI>), dim3(dl_tiles<EPI, C>(a) * S), dim3(64 * C::NW), 0, s, a, S);
}

template <int EPI>
void launch_epi(const GemmArgs& a, hipStream_t s) {
  const int S = a.split > 1 ? a.split : 1;
  switch (dl_kind<EPI>(a, S)) {
    case DL_BIG256: launch_dl<EPI, DlBig256>(a, S, s); return;
    case DL_BIG128: launch_dl<EPI, DlBig128>(a, S, s); return;
    case DL_MID128:
      if constexpr (EPI == EPI_ADD_F32) { launch_dl<EPI, DlMid128>(a, S, s); return; }
      break;
    case DL_SMALL_W8:
      if constexpr (EPI != EPI_SWIGLU_BF16) { launch_dl<EPI, DlSmallW8>(a, S, s); return; }
      break;
    case DL_SMALL_PAIR:
      if constexpr (EPI == EPI_SWIGLU_BF16) { launch_dl<EPI, DlSmallPair>(a, S, s); return; }
      break;
    default: break;
  }
  int bf, bt;
  pick_tile<EPI>(a, &bf, &bt);
  if constexpr (EPI != EPI_SWIGLU_BF16) {
    if (bf == 128) { launch_cfg<128, 128, EPI>(a, s); return; }
  }
  if (bf == 64 && bt == 128) launch_cfg<64, 128, EPI>(a, s);
  else if (bf == 64) launch_cfg<64, 64, EPI>(a, s);
  else launch_cfg<32, 64, EPI>(a, s);
}

template <int EPI>
int split_for(const GemmArgs& a, long cap) {
  constexpr int NA = (EPI == EPI_SWIGLU_BF16) ? 2 : 1;
  // one canvas: the split fp32 projections on the small tiles, in two K slices
  if (a.n_tok <= 256 && dl_kind<EPI>(a, 2) == DL_SMALL_W8 && 2L * NA * a.n_tok * a.N <= cap) return 2;
  // the large-tile kernel: unsplit when it has a chip's worth of tiles, else split K until
  // its 128-token tiles do (one work-group per CU)
  if (dl_kind<EPI>(a, 1) == DL_BIG256 || dl_kind<EPI>(a, 1) == DL_MID128) return 1;
  if (a.n_tok >= 1024) {
    const int t128 = dl_tiles<EPI, DlBig128>(a);
    int S = 1;
    while (S < kMaxParts && t128 * S < 256 && (a.K / BK) % (S * 2) == 0 && a.K / (S * 2) >= 16 * BK &&
           static_cast<long>(S) * 2 * NA * a.n_tok * a.N <= cap)
      S *= 2;
    if (dl_kind<EPI>(a, S) != DL_NONE) return S;
  }
  int bf, bt;
  pick_tile<EPI>(a, &bf, &bt);
  const int tiles = ((a.n_tok + bt - 1) / bt) * (a.N / bf);
  // split K while the grid stays within ~2 work-groups per CU and each slice keeps >= 16 k-tiles
  const int max_wg = 512;
  int S = 1;
  while (S < kMaxParts && tiles * S * 2 <= max_wg && (a.K / BK) % (S * 2) == 0 && a.K / (S * 2) >= 16 * BK &&
         static_cast<long>(S) * 2 * NA * a.n_tok * a.N <= cap)
    S *= 2;
  return S;
}

}  // namespace

int gemm_split(const GemmArgs& a, int epi, long cap) {
  switch (epi) {
    case EPI_ROPE_QKV: return 1;  // the epilogue needs the finished sums
    case EPI_STORE_F32: return split_for<EPI_STORE_F32>(a, cap);
    case EPI_ADD_F32: return split_for<EPI_ADD_F32>(a, cap);
    case EPI_SWIGLU_BF16: return 1;  // measured: the extra reduce pass costs more than it saves
    default: return 1;  // bf16 output: no split
  }
}

void launch_gemm(const GemmArgs& a, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_STORE_F32: launch_epi<EPI_STORE_F32>(a, s); break;
    case EPI_ADD_F32: launch_epi<EPI_ADD_F32>(a, s); break;
    case EPI_SWIGLU_BF16: launch_epi<EPI_SWIGLU_BF16>(a, s); break;
    case EPI_ROPE_QKV: launch_epi<EPI_ROPE_QKV>(a, s); break;
    default: launch_epi<EPI_STORE_BF16>(a, s); break;
  }
}

void launch_swiglu_reduce(const float* part, long part_stride, int split, uint16_t* act, int rows,
                          int n, hipStream_t s) {
  const long n4 = static_cast<long>(rows) * n / 4;
  hipLaunchKernelGGL(swiglu_reduce_kernel, dim3((n4 + 255) / 256), dim3(256), 0, s, part, part_stride,
                     split, act, n4);
}

// The head runs on the large-tile mainloop (256 vocab entries x 256 rows per work-group; with
// V 65536 there are at least 256 tiles at any row count).  Measured at 256 rows against the
// LDS-tiled 128 x 128 kernel: 87.5 against about 120 us; at 2048 rows 521 against about 900 us.
// Shapes the large tile does not divide use the LDS-tiled kernel (128 x 128: each vocab tile is
// streamed by half as many work-groups as with 64-row tiles).  The statistics do not depend on
// the tiling (same k order, same 64-entry slices).
void launch_head(const HeadArgs& a, hipStream_t s) {
  if (a.V % DlBig256::RA == 0 && a.K % DL_BK == 0) {
    const int G = ((a.n_rows + 255) / 256) * (a.V / DlBig256::RA);
    hipLaunchKernelGGL((head_dl_kernel<DlBig256>), dim3(G), dim3(64 * DlBig256::NW), 0, s, a);
    return;
  }
  const int G = ((a.n_rows + 127) / 128) * (a.V / 128);
  hipLaunchKernelGGL((head_kernel<128, 128>), dim3(G), dim3(256), 0, s, a);
}

void launch_head_merge(const float* part, int n_rows, int n_slices, int slice_w,
                       const int32_t* cur_tok, uint32_t* err, int32_t* cand, float* t_cand,
                       float* t_cur, float* lse, float* ent, const RowMap& map, hipStream_t s) {
  hipLaunchKernelGGL(head_merge_kernel, dim3(n_rows), dim3(256), 0, s, part, n_rows, n_slices,
                     slice_w, cur_tok, err, cand, t_cand, t_cur, lse, ent, map);
}

// One work-group per output row: row r of head h (q heads, then k heads) takes source row
// h*D + (e odd ? D/2 : 0) + 2*(w/4) + e/2 with w = r - h*D, e = w % 4; v rows are copied as is.
__global__ __launch_bounds__(256) void pack_qkv_kernel(const uint16_t* __restrict__ wq,
                                                       const uint16_t* __restrict__ wk,
                                                       const uint16_t* __restrict__ wv,
                                                       uint16_t* __restrict__ out, int Hq, int Hkv,
                                                       int D, int d) {
  const int r = blockIdx.x;
  const int qk = (Hq + Hkv) * D;
  const uint16_t* src;
  if (r < qk) {
    const int h = r / D, w = r - h * D, e = w & 3;
    const int sr = ((e & 1) ? D / 2 : 0) + 2 * (w >> 2) + (e >> 1);
    src = (h < Hq) ? wq + (static_cast<long>(h) * D + sr) * d : wk + (static_cast<long>(h - Hq) * D + sr) * d;
  } else {
    src = wv + static_cast<long>(r - qk) * d;
  }
  for (int c = threadIdx.x; c < d; c += 256) out[static_cast<long>(r) * d + c] = src[c];
}

void launch_pack_qkv(const uint16_t* wq, const uint16_t* wk, const uint16_t* wv, uint16_t* out,
                     int Hq, int Hkv, int D, int d, hipStream_t s) {
  hipLaunchKernelGGL(pack_qkv_kernel, dim3((Hq + 2 * Hkv) * D), dim3(256), 0, s, wq, wk, wv, out, Hq,
                     Hkv, D, d);
}

// Canvas tokens of this call's requests, compacted: dst[b][i] = src[slot[b]][i].
__global__ __launch_bounds__(256) void gather_rows_kernel(const int32_t* __restrict__ src,
                                                          int32_t* __restrict__ dst, RowMap map) {
  const int b = blockIdx.x;
  for (int i = threadIdx.x; i < map.rows_per_req; i += 256)
    dst[static_cast<long>(b) * map.rows_per_req + i] =
        src[static_cast<long>(map.slot[b]) * map.rows_per_req + i];
}

void launch_gather_rows(const int32_t* src, int32_t* dst, const RowMap& map, hipStream_t s) {
  hipLaunchKernelGGL(gather_rows_kernel, dim3(map.n_req), dim3(256), 0, s, src, dst, map);
}

}  // namespace dg
