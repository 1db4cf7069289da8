// Device-side common definitions for the gfx950 (CDNA4) kernels of libdg.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define DG_DEVICE __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace dg {

constexpr int kWave = 64;

// bfloat16 <-> float32.  float -> bf16 uses the gfx950 hardware conversion
// (v_cvt_pk_bf16_f32, round to nearest even).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
DG_DEVICE float bf2f(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }
DG_DEVICE uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }
DG_DEVICE uint32_t pack_bf2(float a, float b) {
  const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// One 16x16x32 bf16 MFMA step: D(16x16, fp32) += A(16x32) * B(32x16).
// Lane l supplies A[row l%16][8 k-values of group l/16] and B[same 8 k-values][col l%16];
// the k order inside a group only has to agree between A and B.
// Accumulator: lane l holds D[row 4*(l/16)+i][col l%16], i = 0..3.
DG_DEVICE floatx4_t mfma16(const u32x4_t& a, const u32x4_t& b, const floatx4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Keeps the machine scheduler from moving instructions across this point: used right after a
// prefetch is issued so the loads stay ahead of the MFMAs that do not need them.
DG_DEVICE void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// s_waitcnt with vmcnt = n (< 64) and lgkmcnt = 0 (expcnt not waited on).
template <int n>
DG_DEVICE void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | ((n >> 4) << 14));
}

DG_DEVICE u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
DG_DEVICE u32x4_t ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
DG_DEVICE void st16(void* p, const u32x4_t& v) { *reinterpret_cast<u32x4_t*>(p) = v; }

// Wave-wide reductions (64 lanes).
DG_DEVICE float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DG_DEVICE float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32->64 multiplies
// whose halves are swapped and xored with the key, the key advancing by two Weyl constants.
// ---------------------------------------------------------------------------------------------
struct philox_out { uint32_t x[4]; };

DG_DEVICE philox_out philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                   uint32_t k0, uint32_t k1) {
  // each 32x32->64 product as one 64-bit multiply: one v_mad_u64_u32 instead of a low and a
  // high multiply
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = static_cast<uint64_t>(c0) * 0xD2511F53u;
    const uint64_t p1 = static_cast<uint64_t>(c2) * 0xCD9E8D57u;
    const uint32_t lo0 = static_cast<uint32_t>(p0), hi0 = static_cast<uint32_t>(p0 >> 32);
    const uint32_t lo1 = static_cast<uint32_t>(p1), hi1 = static_cast<uint32_t>(p1 >> 32);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
  }
  philox_out o; o.x[0] = c0; o.x[1] = c1; o.x[2] = c2; o.x[3] = c3;
  return o;
}

enum : uint32_t { kStreamGumbel = 0, kStreamRenoise = 1, kStreamInit = 2 };

// Uniform in (0,1): ((w >> 9) + 0.5) * 2^-23, exact in fp32.
DG_DEVICE float u01(uint32_t w) { return (static_cast<float>(w >> 9) + 0.5f) * 0x1p-23f; }
// Gumbel(0,1) = -ln(-ln u) with the hardware base-2 logarithm (about one ulp; u >= 2^-24 and
// -ln u >= 2^-24 keep both arguments normal): -ln2 log2(-ln2 log2 u).
DG_DEVICE float gumbel(uint32_t w) {
  constexpr float kLn2 = 0.69314718055994531f;
  return -kLn2 * __log2f(-kLn2 * __log2f(u01(w)));
}
// Uniform token in [0, V): multiply-shift.
DG_DEVICE int32_t token_from_word(uint32_t w, uint32_t vocab) {
  return static_cast<int32_t>((static_cast<uint64_t>(w) * vocab) >> 32);
}

}  // namespace dg
