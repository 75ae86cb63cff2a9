// Device helpers shared by the gfx950 kernels of the token codec.
//
// Everything here is written for CDNA4 (gfx950, wave64).  The hardware
// conversion instructions used below were characterised on gfx950:
//   * v_cvt_scalef32_pk_fp4_f32 rounds to nearest-even onto the E2M1 grid,
//     saturates at 6, keeps the sign of zero, and divides by 2^k where k is
//     only the EXPONENT of its f32 scale operand (the significand is ignored);
//   * v_cvt_scalef32_pk_f32_fp4 multiplies by that same 2^k;
//   * v_cvt_pk_fp8_f32 is OCP E4M3FN round-to-nearest-even below 464;
//   * v_cvt_scalef32_pk_fp8_bf16 is E4M3 RNE of x / 2^k (exponent only).
// So any division by a block scale with a non-power-of-two significand is
// done in software (see quot_split below) and only the power of two is handed
// to the conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mtb {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (data read once: do not keep it in the caches).
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1, each
// body its own straight-line copy.  For loops whose bodies are too large for
// the compiler to unroll by itself: a loop left rolled indexes its register
// arrays with a variable, and such arrays are moved to scratch memory.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

constexpr int kWave = 64;
constexpr float kTokenBound = 2688.0f;  // 6 * 448

// ----------------------------------------------------------------- bit casts
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Power of two 2^k as a float, k in [-126, 127] (normal range only).
__device__ __forceinline__ float pow2f(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// Exponent of a float that is a power of two (normal or subnormal).
// Branch-free (a select), so that a load of p need not be waited for before
// the loads that follow it in program order are issued.  p = 0 gives -149.
__device__ __forceinline__ int pow2_exponent(float p) {
  uint32_t b = __float_as_uint(p);
  uint32_t ef = (b >> 23) & 0xFFu;
  const int sub = -149 + (31 - __builtin_clz((b & 0x7FFFFFu) | 1u));  // subnormal: position of the single set bit
  return ef ? (int)ef - 127 : sub;
}

// ----------------------------------------------------------------- E4M3
// E4M3FN code of y in [0, 448] (RNE; the caller guarantees the range).
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  // the converter keeps the upper half of its `old` operand: y's own bits, masked off
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, __float_as_int(y), false) & 0xFFu;
}
// Value of an E4M3FN code held in the low byte of w.
__device__ __forceinline__ float e4m3_decode(uint32_t w) { return __builtin_amdgcn_cvt_f32_fp8((int)w, 0); }

// ----------------------------------------------------------------- exact quotients
// A divisor s with a short significand (E4M3 scales: 4 bits) split as
// s = m * 2^k with m in [1, 2).  r_hi + r_lo approximates 1/m to about 2^-46:
// r_hi is rcp(m) moved down by one ulp if needed so that r_hi <= 1/m, and the
// residual 1 - m*r_hi (exact for a 4-bit m, and >= 0) gives r_lo >= 0.  Then
// fma(x, r_hi, x*r_lo) is the correctly rounded fl32(x / m) for any x whose
// exact quotient is at least 2^-28 (relative) away from a float32 rounding
// midpoint -- true for every x of at most 24 bits divided by a 4-bit m -- and
// it keeps the sign of x also for x = -0 (both terms carry x's sign).
struct QuotSplit {
  float r_hi, r_lo;
  int k;  // exponent of the divisor
};

// r ~ 1/m (positive) lowered to r <= 1/m; returns the non-negative residual in e.
__device__ __forceinline__ float rcp_below(float m, float& e) {
  float r = __builtin_amdgcn_rcpf(m);
  e = __builtin_fmaf(-m, r, 1.0f);
  if (e < 0.0f) {
    r = __uint_as_float(__float_as_uint(r) - 1u);
    e = __builtin_fmaf(-m, r, 1.0f);
  }
  return r;
}

__device__ __forceinline__ QuotSplit quot_split(float s) {
  QuotSplit q;
  q.k = __builtin_amdgcn_frexp_expf(s) - 1;   // s = m * 2^k, m in [1, 2)
  float m = __builtin_amdgcn_frexp_mantf(s) * 2.0f;
  float e;
  q.r_hi = rcp_below(m, e);
  q.r_lo = e * q.r_hi;
  return q;
}

__device__ __forceinline__ float quot_apply(float x, float r_hi, float r_lo) {
  return __builtin_fmaf(x, r_hi, x * r_lo);
}

// fl32(a / 6) for a >= 0 in float32's normal range: a / 1.5 with the split
// reciprocal of 1.5 (2/3 = R_HI + R_LO to ~2^-48), then an exact * 0.25.
__device__ __forceinline__ float div1_5(float a) {
  const float R_HI = 0.666666686534881591796875f;        // RN(2/3)
  const float R_LO = -1.98682149251302083333e-08f;       // RN(2/3 - R_HI)
  return __builtin_fmaf(a, R_HI, a * R_LO);
}
__device__ __forceinline__ float div6(float a) { return div1_5(a) * 0.25f; }

// ----------------------------------------------------------------- E2M1
// Four E2M1 codes of u0..u3 / 2^k packed as the two bytes of a 16-bit result
// written into byte pair `sel`; `scale` is 2^k as a float (exponent only).
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pack2(uint32_t old, float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}

// E2M1 value (times 2^k) of the two nibbles of byte SEL of w.
template <int SEL>
__device__ __forceinline__ f32x2 fp4_unpack2(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, SEL);
}

// ----------------------------------------------------------------- RHT
// The 16-bit sign mask of the 16-point RHT: d_i = -1 iff bit i is set.  It is
// the low half of word 0 of Philox4x32-10 at key (0,0), counter (0,0,0,0).
constexpr uint32_t kRhtSignMask = 0xE8D5u;

__host__ __device__ constexpr float rht_in_scale(int i) {
  return ((kRhtSignMask >> i) & 1u) ? -0.25f : 0.25f;
}

// In-place butterfly on z[0..15]: strides 1, 2, 4, 8; pair (i, i+h) with
// (i & h) == 0 becomes (z_i + z_{i+h}, z_i - z_{i+h}).  The inputs already
// carry the d_i / 4 factor.  No contraction can apply: adds only.
__device__ __forceinline__ void rht16_butterfly(float* z) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      float a = z[i], b = z[i + h];
      z[i] = a + b;
      z[i + h] = a - b;
    }
  }
}

// ----------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror, Shaw (SC'11): ten rounds of two 32x32->64 products,
// Weyl key schedule between rounds.  The three-way XORs of a round are one
// v_bitop3_b32 each (truth table 0x96 = a ^ b ^ c).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

struct U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                            uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
    uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  return U4{c0, c1, c2, c3};
}

// ----------------------------------------------------------------- stochastic E2M1
// E2M1 code nibble of one element by the hardware stochastic conversion:
// code of u / 2^k (k = the exponent of `scale`), rounding up iff
// floor(frac * 2^32) + w >= 2^32 -- the decision v_cvt_scalef32_sr_pk_fp4_f32
// makes for its first operand with random word w (its second operand gets the
// word rotated left by one bit; the other operand here is +0, which never
// moves).  Only the low byte of the result is defined.
__device__ __forceinline__ uint32_t sr_code_lo(float u, uint32_t w, float scale) {
  f32x2 p = {u, 0.0f};
  return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, p, w, scale, 0) & 0xFu;
}
__device__ __forceinline__ uint32_t sr_code_hi(float u, uint32_t w, float scale) {
  f32x2 p = {0.0f, u};
  return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, p, __builtin_amdgcn_alignbit(w, w, 1), scale, 0) & 0xF0u;
}

// Carry-form stochastic codes of eight quotients u[0..7] / scale, one word per
// element: element k takes word 0 of Philox4x32-10 at counter n0 + k (key =
// the seed), so each code's stream position is n0 + its index.  Value 2j goes
// to the low nibble of byte j.
__device__ __forceinline__ uint32_t sr_codes8(const float* u, uint64_t n0, uint32_t klo, uint32_t khi, float scale) {
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t na = n0 + 2 * j, nb = na + 1;
    const uint32_t wa = philox4x32_10((uint32_t)na, (uint32_t)(na >> 32), 0u, 0u, klo, khi).x;
    const uint32_t wb = philox4x32_10((uint32_t)nb, (uint32_t)(nb >> 32), 0u, 0u, klo, khi).x;
    w |= (sr_code_lo(u[2 * j], wa, scale) | sr_code_hi(u[2 * j + 1], wb, scale)) << (8 * j);
  }
  return w;
}

// sr_codes8 with the word-stream mapping: the word of position n is word
// (n & 3) of Philox block n >> 2, so 8 positions take two blocks (three when
// n0 is not a multiple of 4; callers' n0 mod 4 is the counter base's in every
// lane, so the block changes are uniform across the wave).
__device__ __forceinline__ uint32_t sr_codes8_stream(const float* u, uint64_t n0, uint32_t klo, uint32_t khi,
                                                     float scale) {
  uint64_t cur = n0 >> 2;
  U4 blk = philox4x32_10((uint32_t)cur, (uint32_t)(cur >> 32), 0u, 0u, klo, khi);
  auto word = [&](uint64_t n) -> uint32_t {
    if ((n >> 2) != cur) {
      cur = n >> 2;
      blk = philox4x32_10((uint32_t)cur, (uint32_t)(cur >> 32), 0u, 0u, klo, khi);
    }
    const uint32_t sel = (uint32_t)n & 3u;
    return sel == 0 ? blk.x : (sel == 1 ? blk.y : (sel == 2 ? blk.z : blk.w));
  };
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // each pair's codes as soon as its two words exist
    const uint32_t wa = word(n0 + 2 * j), wb = word(n0 + 2 * j + 1);
    w |= (sr_code_lo(u[2 * j], wa, scale) | sr_code_hi(u[2 * j + 1], wb, scale)) << (8 * j);
  }
  return w;
}

// The stochastic codes of 8 positions with the element (SRM 1) or stream (SRM 2) words.
template <int SRM>
__device__ __forceinline__ uint32_t sr_codes8_m(const float* u, uint64_t n0, uint32_t klo, uint32_t khi, float scale) {
  return SRM == 2 ? sr_codes8_stream(u, n0, klo, khi, scale) : sr_codes8(u, n0, klo, khi, scale);
}

// ----------------------------------------------------------------- reductions
// The value of the neighbouring lane (lane ^ 1), by a DPP quad permutation
// [1, 0, 3, 2] inside the VALU instead of an LDS permute.
__device__ __forceinline__ uint32_t lane_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t other = (uint32_t)__shfl_xor((int)v, o, kWave);
    v = v > other ? v : other;
  }
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// max of |bf16| over the two halves of 4 packed words, as a 16-bit magnitude pattern.
__device__ __forceinline__ uint32_t absmax_bf16x8(uint4 v) {
  u16x2 a = __builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu);
  u16x2 b = __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu);
  u16x2 c = __builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu);
  u16x2 d = __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu);
  u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  uint32_t lo = m[0], hi = m[1];
  return lo > hi ? lo : hi;
}

}  // namespace mtb
