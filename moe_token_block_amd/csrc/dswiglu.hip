// Grouped dSwiGLU epilogue with per-expert amax, then FC1-gradient NVFP4
// quantization that takes its global scales from that amax (P4, description:
// the epilogue already sees every dX value, so its max -- rounded to BF16 --
// is the rowwise amax, and four times it bounds the columnwise amax after the
// RHT; the quantizer then needs no max pass of its own).
//
// Launch 1 (epilogue): one wave per token row; per pair (a_j, b_j, dy_j):
//   s = sigmoid(a), da = dy*b*s*(1 + a*(1-s)), db = dy*a*s in FP32 -> BF16;
//   the row's max |dX| (over the BF16 values) goes to the workspace (one word
//   per row: no atomics, no contention).
// Launch 2 (reduce): one workgroup per expert: the expert row offsets (plain
//   and 16-padded) from the device counts, amax_e = max over its rows, and
//   D_row = fl32(amax/2688), D_col = fl32(4*amax/2688) (= 4*D_row unless D_row is subnormal).
// Launch 3 (quant): one workgroup per 256 padded rows x 128 columns, as the
//   direct receive: thread (cg, m) owns 8 columns x one 16-row block; the
//   rowwise operand (per-expert scale D_row = amax/2688) and the RHT
//   columnwise operand (D_col) come out of the same load of dX.
#include <atomic>
#include <mutex>

#include "common.h"
#include "launch.h"

namespace mtb {

constexpr int kQTileRows = 256;
constexpr int kQTileCols = 128;
constexpr int kQBlocks = kQTileRows / 16;
constexpr int kQThreads = 16 * kQBlocks;  // 16 threads (8 columns each) per 16-row block
constexpr unsigned kXcdsQ = 8;  // CDNA4: 8 XCDs, workgroups dealt round-robin

// Inclusive scan of one int per lane with the running total cut at cap
// (a saturating add of non-negative values is associative).
__device__ __forceinline__ int wave_scan_sat(int x, int cap) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x = min(x + y, cap);
  }
  return x;
}

// Block scan (1024 threads, one value each, non-negative): inclusive, cut at cap.
__device__ __forceinline__ int block_scan_sat(int x, int cap, int32_t* wsum /* 32 */) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  x = wave_scan_sat(x, cap);
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    int t = wave_scan_sat(lane < 16 ? wsum[lane] : 0, cap);
    if (lane < 16) wsum[16 + lane] = t;
  }
  __syncthreads();
  return w ? min(wsum[16 + w - 1] + x, cap) : x;
}

// Expert row offsets from the device counts: a[e] = first row of expert e,
// b[e] = its first 16-padded row, a[E], b[E] the totals (E <= 1024 entries,
// 1024 threads).  Counts are device data: negative counts count as 0 and the
// running total is cut at T, so the experts never cover more rows than exist.
__device__ __forceinline__ void expert_prefix(const int32_t* counts, int E, int T, int32_t* a, int32_t* b,
                                              int32_t* wsum) {
  const int tid = threadIdx.x;
  const int c = tid < E ? min(max(counts[tid], 0), T) : 0;
  const int incl = block_scan_sat(c, T, wsum);
  a[tid + 1] = incl;
  if (tid == 0) a[0] = b[0] = 0;
  __syncthreads();
  const int pc = (incl - a[tid] + 15) & ~15;  // padded size (0 past E); totals stay below 2^31
  b[tid + 1] = block_scan_sat(pc, INT32_MAX, wsum);
  __syncthreads();
}

// One workgroup per expert.  Workgroup 0 also publishes the offsets.  The
// row maxima are read 4 rows per load (the workspace pads them to a multiple
// of 4 rows; rows outside the expert are masked).
__global__ __launch_bounds__(1024) void k_dswiglu_reduce(const int32_t* __restrict__ counts, int E, int T,
                                                         const uint32_t* __restrict__ rowmax,
                                                         int32_t* __restrict__ offs, int32_t* __restrict__ poffs,
                                                         float* __restrict__ amax, float* __restrict__ row_scale,
                                                         float* __restrict__ col_scale) {
  __shared__ int32_t a[1025], b[1025], wsum[32];
  __shared__ uint32_t red[16];
  const int tid = threadIdx.x, e = blockIdx.x;
  expert_prefix(counts, E, T, a, b, wsum);
  if (e == 0 && tid < E) {  // entries 1..E (E may be 1024 = the block size), then entry 0
    offs[tid + 1] = a[tid + 1];
    poffs[tid + 1] = b[tid + 1];
    if (tid == 0) offs[0] = poffs[0] = 0;
  }
  const int r0 = a[e], r1 = a[e + 1];
  const uint4* rm4 = reinterpret_cast<const uint4*>(rowmax);
  uint32_t m = 0;
  for (int g = (r0 >> 2) + tid; 4 * g < r1; g += 1024) {
    const uint4 q = rm4[g];
    const int r = 4 * g;
    if (r >= r0) m = max(m, q.x);
    if (r + 1 >= r0 && r + 1 < r1) m = max(m, q.y);
    if (r + 2 >= r0 && r + 2 < r1) m = max(m, q.z);
    if (r + 3 < r1) m = max(m, q.w);
  }
  m = wave_max_u32(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    uint32_t r = 0;
    for (int i = 0; i < 16; ++i) r = max(r, red[i]);
    float am = __uint_as_float(r);  // a BF16 value (max |dX|), 0 for an empty expert
    float D = am / kTokenBound;     // fl32(amax / 2688)
    amax[e] = am;
    row_scale[e] = D;
    col_scale[e] = (4.0f * am) / kTokenBound;  // fl32(4 * amax / 2688): 4 * D only while D is a normal float
  }
}

__device__ __forceinline__ int expert_of(const int32_t* offs, int E, int r) {
  int lo = 0, hi = E - 1;  // last e with offs[e] <= r
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ void dswiglu_pair(float a, float b, float dy, float& da, float& db) {
  float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-a));
  float silu = a * sg;
  da = dy * b * sg * (1.0f + a * (1.0f - sg));
  db = dy * silu;
}

__device__ __forceinline__ uint32_t bf16pair(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// One wave per row; lane l owns 8-column chunks j = l + 64k of a, b and dy,
// NB of them per group.  A group's 3 * NB loads are issued before any of its
// arithmetic (chunks past the row's end load its last chunk and are not
// stored), so a 2048-column row costs one memory round trip, not one per chunk
// with the previous chunk's stores waited for too.
template <bool STORE, int NB>
__global__ __launch_bounds__(256) void k_dswiglu_epilogue(const uint16_t* __restrict__ preact,
                                                          const uint16_t* __restrict__ dy, int T, int F,
                                                          uint16_t* __restrict__ dx, uint32_t* __restrict__ rowmax) {
  const int lane = threadIdx.x & 63;
  const int r = (int)(blockIdx.x * 4u + (threadIdx.x >> 6));
  if (r >= T) return;
  const int nch = F >> 3;
  const uint4* pa = reinterpret_cast<const uint4*>(preact + (size_t)r * 2 * F);
  const uint4* pb = reinterpret_cast<const uint4*>(preact + (size_t)r * 2 * F + F);
  const uint4* pd = reinterpret_cast<const uint4*>(dy + (size_t)r * F);
  uint4* oa = reinterpret_cast<uint4*>(dx + (size_t)r * 2 * F);
  uint4* ob = reinterpret_cast<uint4*>(dx + (size_t)r * 2 * F + F);
  uint32_t m = 0;
  for (int c0 = 0; c0 < nch; c0 += 64 * NB) {
    uint4 va[NB], vb[NB], vd[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int j = min(c0 + lane + 64 * k, nch - 1);
      va[k] = ld_stream16(pa + j);
      vb[k] = ld_stream16(pb + j);
      vd[k] = ld_stream16(pd + j);
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int j = c0 + lane + 64 * k;
      const uint32_t wa[4] = {va[k].x, va[k].y, va[k].z, va[k].w}, wb[4] = {vb[k].x, vb[k].y, vb[k].z, vb[k].w};
      const uint32_t wd[4] = {vd[k].x, vd[k].y, vd[k].z, vd[k].w};
      uint32_t ra[4], rb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float da0, db0, da1, db1;
        dswiglu_pair(bf16lo(wa[i]), bf16lo(wb[i]), bf16lo(wd[i]), da0, db0);
        dswiglu_pair(bf16hi(wa[i]), bf16hi(wb[i]), bf16hi(wd[i]), da1, db1);
        ra[i] = bf16pair(da0, da1);
        rb[i] = bf16pair(db0, db1);
      }
      const uint4 oA = make_uint4(ra[0], ra[1], ra[2], ra[3]), oB = make_uint4(rb[0], rb[1], rb[2], rb[3]);
      if (STORE && j < nch) {
        oa[j] = oA;
        ob[j] = oB;
      }
      uint32_t x = absmax_bf16x8(oA), y = absmax_bf16x8(oB);
      x = x > y ? x : y;
      m = m > x ? m : x;  // a clamped chunk repeats one of the row: no effect on the max
    }
  }
  m = wave_max_u32(m);
  // non-negative floats order like their bit patterns: the integer max is exact
  if (lane == 0) rowmax[r] = m << 16;
}

// ------------------------------------------------------------------ grouped quant
// The FC1-gradient quantizer divides by a general FP32 decode scale D (and by
// c = fl32(s*D) per block).  Each divisor is split as m * 2^k with m in
// [1, 2); x/m is fma(x, r_hi, x*r_lo) with the split reciprocal of m, and 2^k
// goes to the converter (or to an exact ldexp).  With a 24-bit m the split
// reciprocal is within ~2^-45 of 1/m, so a quotient can differ from the
// correctly rounded one only within that distance of a float32 midpoint.

// x = m * 2^k, m in [1, 2), for any x > 0 (normal or subnormal).
__device__ __forceinline__ float split_pow2(float x, int& k) {
  int sub = 0;
  if (x < 0x1p-126f) { x *= 0x1p64f; sub = 64; }
  k = __builtin_amdgcn_frexp_expf(x) - 1 - sub;
  return __builtin_amdgcn_frexp_mantf(x) * 2.0f;
}

// Per-expert constants: D = m_D * 2^kD and the split reciprocal of m_D.
struct DScale {
  float D, r_hi, r_lo;
  int kD;
};
__device__ __forceinline__ DScale dscale(float D) {
  DScale d;
  d.D = D;
  d.kD = 0;
  d.r_hi = d.r_lo = 0.0f;
  if (D > 0.0f) {
    float e;
    float m = split_pow2(D, d.kD);
    d.r_hi = rcp_below(m, e);
    d.r_lo = e * d.r_hi;
  }
  return d;
}

// Block parameters for codes of x / c, c = fl32(s * D): split reciprocal of
// c's significand (times 2^P) and the converter scale 2^(kc + P).
struct GenBlock {
  float r_hi, r_lo, scale;
};
__device__ __forceinline__ GenBlock gen_block(uint32_t sc, float D) {
  GenBlock g;
  float c = e4m3_decode(sc) * D;   // fl32(s * D), rounded as written
  if (!(c > 0.0f)) {
    g.r_hi = g.r_lo = 0.0f;        // every code becomes a signed zero
    g.scale = 1.0f;
    return g;
  }
  int kc;
  float m = split_pow2(c, kc);
  float e;
  float r = rcp_below(m, e);
  int P = kc < -104 ? -104 - kc : 0;  // keep x * r_lo and the converter scale in range
  g.r_hi = __builtin_ldexpf(r, P);
  g.r_lo = __builtin_ldexpf(e * r, P);
  g.scale = pow2f(kc + P);
  return g;
}

template <int SEL>
__device__ __forceinline__ uint32_t enc_pair(uint32_t old, float a, float b, const GenBlock& g) {
  return fp4_pack2<SEL>(old, quot_apply(a, g.r_hi, g.r_lo), quot_apply(b, g.r_hi, g.r_lo), g.scale);
}

// The first byte pair of a word whose four byte pairs all get written: the
// converter's merge operand is the first quotient's own register (its other
// bytes are overwritten later), so no zeroed word is needed.
__device__ __forceinline__ uint32_t enc_first(float a, float b, const GenBlock& g) {
  const float qa = quot_apply(a, g.r_hi, g.r_lo);
  return fp4_pack2<0>(__float_as_uint(qa), qa, quot_apply(b, g.r_hi, g.r_lo), g.scale);
}

// Per 16-row block of a tile: the split reciprocals of c = fl32(s * D) for
// the 8 significands of s.  s * D = (m_s * m_D) * 2^(k_s + k_D), and while c
// is a normal float fl32(s * D) = fl32(m_s * m_D) * 2^(k_s + k_D); the table
// holds m_c = fl32(m_s * m_D) normalised to [1, 2) (kadj = 1 if it was >= 2).
struct MantEntry {
  float r_hi, r_lo;
  int kadj, pad;
};

__device__ __forceinline__ MantEntry mant_entry(int j, float mD) {
  float mc = (1.0f + 0.125f * (float)j) * mD;  // exact product rounded once
  MantEntry t;
  t.kadj = mc >= 2.0f ? 1 : 0;
  float m = t.kadj ? mc * 0.5f : mc;
  float e;
  t.r_hi = rcp_below(m, e);
  t.r_lo = e * t.r_hi;
  t.pad = 0;
  return t;
}

// Block parameters for E4M3 code sc with decode scale D = mD * 2^kD, from the
// block's significand table; falls back to gen_block when c is tiny (P > 0)
// or subnormal.  FAST (D >= 2^-85): the power of c is at least
// 2^(-9 - 85) > 2^-104, so the fallback is never taken and is left out.
template <bool FAST = false>
__device__ __forceinline__ GenBlock gen_block_tab(uint32_t sc, float D, int kD, const MantEntry* tab) {
  float s = e4m3_decode(sc);
  GenBlock g;
  if (FAST) {
    // branch-free: code 0 reads entry 0 and then zeros its reciprocal, so
    // every quotient is a signed zero; its power 2^(kD - 1 + kadj) is a
    // normal float for D >= 2^-85 (any normal power encodes a zero alike)
    const MantEntry t = tab[(__float_as_uint(s) >> 20) & 7u];
    const bool z = !(s > 0.0f);  // (D = 0 only gives the code 0)
    g.r_hi = z ? 0.0f : t.r_hi;
    g.r_lo = z ? 0.0f : t.r_lo;
    g.scale = pow2f(__builtin_amdgcn_frexp_expf(s) - 1 + kD + t.kadj);
    return g;
  }
  if (!(s > 0.0f)) {  // (D = 0 only gives the code 0)
    g.r_hi = g.r_lo = 0.0f;
    g.scale = 1.0f;
    return g;
  }
  int ks = __builtin_amdgcn_frexp_expf(s) - 1;
  const MantEntry t = tab[(__float_as_uint(s) >> 20) & 7u];
  int kc = ks + kD + t.kadj;
  if (kc < -104) return gen_block(sc, D);
  g.r_hi = t.r_hi;
  g.r_lo = t.r_lo;
  g.scale = pow2f(kc);
  return g;
}

// E4M3 code of fl32(fl32(a' / 6) / D) for a block max a = 2^x2 * a' (x2 = 2:
// the unscaled RHT below), each fl32 an IEEE binary32 rounding.  For a block
// max below 2^-100, a' / 6 may fall below FP32's normal range, where the first
// rounding is on the subnormal grid: it is taken by the correctly rounded
// division, and its result (at most 24 bits) scaled by 2^64 before the
// quotient by D, which is then exact to the last bit as in the normal range.
// Elsewhere div6 gives the same fl32(a / 6), and 2^x2 * fl32(a' / 6) =
// fl32(a / 6) exactly.
// FAST (D >= 2^-85): a block max below 2^-100 gives a quotient below 2^-17,
// code 0 whichever way a / 6 is rounded, so the tiny path is left out.
template <bool FAST = false>
__device__ __forceinline__ uint32_t gen_scale_code_x(float a, const DScale& d, int x2) {
  // D = 0 (an all-zero expert: a = 0) needs no test: its split reciprocal is 0, so the code is 0
  const bool tiny = !FAST && a < 0x1p-100f;
  float pre;
  if (tiny) {
    pre = (__builtin_ldexpf(a, -x2) / 6.0f) * 0x1p64f;   // fl32(a' / 6), subnormal or not, times 2^64
  } else {
    pre = div6(a);
  }
  float q = quot_apply(pre, d.r_hi, d.r_lo);
  float y = __builtin_ldexpf(q, -d.kD - (tiny ? 64 : x2));
  return e4m3_encode(fminf(y, 448.0f));
}

// dX column of the tile's column c (0..127): the tile's 128 contiguous
// columns, or with RECOMPUTE 64 da columns then the matching 64 db columns.
template <bool RECOMPUTE>
__device__ __forceinline__ int qtile_col(int col0, int c, int W) {
  if (!RECOMPUTE) return col0 + c;
  const int j0 = col0 >> 1;
  return c < 64 ? j0 + c : (W >> 1) + j0 + (c - 64);
}

// LDS staging of the transposed tile, as in the direct receive: entry
// (column c, block b) at c*kQBlocks + (b ^ ((c >> 3) % kQBlocks)).
__device__ __forceinline__ int qstage_at(int c, int b) { return c * kQBlocks + (b ^ ((c >> 3) & (kQBlocks - 1))); }

// Rowwise operand of one thread's 16 rows x 8 columns (half of each 16-column
// block; lane cg ^ 1 holds the other half): the pair's block max by a lane
// swap, the E4M3 scale from D_row, the codes of the 8 values.  Rows at or
// past nreal are not stored (every lane still takes part in the swap).
// SR: stochastic codes, element (row0 + i, xcol + k) at stream position
// n0 + i * W + k (n0 = the counter base + row0 * W + xcol: its index in the
// [T, W] code array).
template <int SR = 0, bool FAST = false>
__device__ __forceinline__ void fc1_rowwise(const uint4 (&v)[16], int nreal, float Drow, const MantEntry* tab,
                                            uint8_t* cbase, uint32_t coff, uint8_t* sbase, uint32_t soff, uint32_t W,
                                            bool even, uint64_t n0 = 0, uint32_t klo = 0, uint32_t khi = 0) {
  const DScale dsr = dscale(Drow);
  static_for<0, 16>([&](auto I) {
    constexpr int i = I;
    uint32_t am = absmax_bf16x8(v[i]);
    uint32_t o = lane_xor1(am);
    am = am > o ? am : o;
    if (i >= nreal) return;
    uint32_t sc = gen_scale_code_x<FAST>(__uint_as_float(am << 16), dsr, 0);
    GenBlock gb = gen_block_tab<FAST>(sc, Drow, dsr.kD, tab);
    uint32_t w;
    if (!SR) {
      w = enc_first(bf16lo(v[i].x), bf16hi(v[i].x), gb);
      w = enc_pair<1>(w, bf16lo(v[i].y), bf16hi(v[i].y), gb);
      w = enc_pair<2>(w, bf16lo(v[i].z), bf16hi(v[i].z), gb);
      w = enc_pair<3>(w, bf16lo(v[i].w), bf16hi(v[i].w), gb);
    } else {
      const uint32_t wv[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      float u[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        u[2 * k] = quot_apply(bf16lo(wv[k]), gb.r_hi, gb.r_lo);
        u[2 * k + 1] = quot_apply(bf16hi(wv[k]), gb.r_hi, gb.r_lo);
      }
      w = sr_codes8_m<SR>(u, n0 + (uint64_t)i * W, klo, khi, gb.scale);
    }
    *reinterpret_cast<uint32_t*>(cbase + (coff + (uint32_t)i * (W >> 1))) = w;
    if (even) sbase[soff + (uint32_t)i * (W >> 4)] = (uint8_t)sc;
  });
}

// Columnwise operand of column pairs [P0, P1) of one thread's 8 columns x 16
// rows (one block per column): 4x the RHT down each column (signs folded into the butterfly's
// adds), the E4M3 scale from D_col, the 16 codes; codes and scales go to the
// LDS stage at (column cg*8 + k, block m).
// SR: stochastic codes, the block's row 0 in the thread's column k at stream
// position n0 + k * n_step (its index in the columnwise code array plus the
// counter base).
template <int P0, int P1, int SR = 0, bool FAST = false, typename ScT>
__device__ __forceinline__ void fc1_columnwise(const uint4 (&v)[16], float Dcol, const MantEntry* tab, int cg, int m,
                                               uint2* stage_codes, ScT* stage_sc, uint64_t n0 = 0,
                                               uint64_t n_step = 0, uint32_t klo = 0, uint32_t khi = 0) {
  const DScale dsc = dscale(Dcol);
  static_for<P0, P1>([&](auto PI) {
    constexpr int p = PI;
    float z0[16], z1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t wv = p == 0 ? v[i].x : (p == 1 ? v[i].y : (p == 2 ? v[i].z : v[i].w));
      const bool neg = (kRhtSignMask >> i) & 1u;
      z0[i] = neg ? -bf16lo(wv) : bf16lo(wv);
      z1[i] = neg ? -bf16hi(wv) : bf16hi(wv);
    }
    rht16_butterfly(z0);
    rht16_butterfly(z1);
    float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      a0 = fmaxf(a0, fabsf(z0[i]));
      a1 = fmaxf(a1, fabsf(z1[i]));
    }
    uint32_t sc0 = gen_scale_code_x<FAST>(a0, dsc, 2);
    uint32_t sc1 = gen_scale_code_x<FAST>(a1, dsc, 2);
    GenBlock g0 = gen_block_tab<FAST>(sc0, Dcol, dsc.kD, tab);
    GenBlock g1 = gen_block_tab<FAST>(sc1, Dcol, dsc.kD, tab);
    // the values are 4x the transform: divide by 4 more
    g0.scale *= 4.0f;
    g1.scale *= 4.0f;
    uint32_t c00, c01, c10, c11;
    if (!SR) {
      c00 = enc_first(z0[0], z0[1], g0);
      c00 = enc_pair<1>(c00, z0[2], z0[3], g0);
      c00 = enc_pair<2>(c00, z0[4], z0[5], g0);
      c00 = enc_pair<3>(c00, z0[6], z0[7], g0);
      c01 = enc_first(z0[8], z0[9], g0);
      c01 = enc_pair<1>(c01, z0[10], z0[11], g0);
      c01 = enc_pair<2>(c01, z0[12], z0[13], g0);
      c01 = enc_pair<3>(c01, z0[14], z0[15], g0);
      c10 = enc_first(z1[0], z1[1], g1);
      c10 = enc_pair<1>(c10, z1[2], z1[3], g1);
      c10 = enc_pair<2>(c10, z1[4], z1[5], g1);
      c10 = enc_pair<3>(c10, z1[6], z1[7], g1);
      c11 = enc_first(z1[8], z1[9], g1);
      c11 = enc_pair<1>(c11, z1[10], z1[11], g1);
      c11 = enc_pair<2>(c11, z1[12], z1[13], g1);
      c11 = enc_pair<3>(c11, z1[14], z1[15], g1);
    } else {
      float u0[16], u1[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        u0[i] = quot_apply(z0[i], g0.r_hi, g0.r_lo);
        u1[i] = quot_apply(z1[i], g1.r_hi, g1.r_lo);
      }
      const uint64_t na = n0 + (uint64_t)(2 * p) * n_step, nb = na + n_step;
      c00 = sr_codes8_m<SR>(u0, na, klo, khi, g0.scale);
      c01 = sr_codes8_m<SR>(u0 + 8, na + 8, klo, khi, g0.scale);
      c10 = sr_codes8_m<SR>(u1, nb, klo, khi, g1.scale);
      c11 = sr_codes8_m<SR>(u1 + 8, nb + 8, klo, khi, g1.scale);
    }
    const int c0 = cg * 8 + 2 * p;
    stage_codes[qstage_at(c0, m)] = make_uint2(c00, c01);
    stage_codes[qstage_at(c0 + 1, m)] = make_uint2(c10, c11);
    stage_sc[qstage_at(c0, m)] = (ScT)sc0;
    stage_sc[qstage_at(c0 + 1, m)] = (ScT)sc1;
  });
}

// One workgroup per 256 padded rows x 128 columns of dX, 1-D grid with the
// tiles dealt to the 8 XCDs in contiguous ranges, column tile fastest (as in
// the direct receive).  Thread (cg, m) loads 8 columns x the 16 rows of block
// m once; the rowwise operand (16-element blocks split over lanes cg, cg^1)
// and the RHT columnwise operand come out of that one load.  The columnwise
// butterfly runs on the unscaled values with the signs d_i folded into its
// adds: the result is 4x the RHT exactly, and the 4 goes into the powers of
// two of the quantizer.
// RECOMPUTE: dX is not materialized; tile ct covers the da columns
// [64ct, 64ct + 64) and the db columns F + [64ct, 64ct + 64), and each thread
// recomputes its 8 columns of dX from preact and dy with the epilogue's own
// arithmetic (so the values, and the amax already taken from them, agree bit
// for bit).
// SR: stochastic codes (rowwise at counter base + row * W + col, columnwise at
// counter base + T * W + the code's index in the columnwise code array), each
// position's word its own Philox block's (SR = 1) or from the four-word stream
// (SR = 2).
// At most 168 VGPRs (three waves per SIMD): the other forms stay below that,
// the stream-word form would take 170 and two waves (slower by 20%); capped, it
// keeps three waves with a few bytes of spill.
template <bool RECOMPUTE, int SR = 0>
__global__ __launch_bounds__(kQThreads, 3) void k_fc1_quant(const uint16_t* __restrict__ dx, const uint16_t* __restrict__ preact,
                                                   const uint16_t* __restrict__ dy, int T, int W /* 2F */, int E,
                                                   int n_ct, const int32_t* __restrict__ offs,
                                                   const int32_t* __restrict__ poffs,
                                                   const float* __restrict__ row_scale,
                                                   const float* __restrict__ col_scale,
                                                   uint8_t* __restrict__ row_codes, uint8_t* __restrict__ row_scales,
                                                   uint8_t* __restrict__ col_codes, uint8_t* __restrict__ col_scales,
                                                   const uint64_t* __restrict__ sr_state) {
  __shared__ uint2 stage_codes[kQTileCols * kQBlocks > 1025 ? kQTileCols * kQBlocks : 1025];  // offsets, padded offsets first
  __shared__ uint32_t stage_sc[kQTileCols * kQBlocks];
  __shared__ MantEntry s_tab[kQBlocks][2][8];            // [block][row / col][significand of s]
  __shared__ int s_live[kQBlocks], s_row0[kQBlocks], s_nreal[kQBlocks];
  __shared__ float s_drow[kQBlocks], s_dcol[kQBlocks];
  __shared__ uint64_t s_cbase[kQBlocks], s_sbase[kQBlocks];
  __shared__ uint32_t s_cstr[kQBlocks], s_sstr[kQBlocks];
  int* s_offs = reinterpret_cast<int*>(stage_codes);
  int* s_poffs = s_offs + 1025;

  const int tid = threadIdx.x;
  const unsigned nb = gridDim.x, bx = blockIdx.x;
  const unsigned xq = nb / kXcdsQ, xr = nb % kXcdsQ, x = bx % kXcdsQ;
  const unsigned lt = x * xq + min(x, xr) + bx / kXcdsQ;
  const int rt = (int)(lt / (unsigned)n_ct), ct = (int)(lt % (unsigned)n_ct);
  const int gp_base = rt * kQTileRows;  // first padded row of the tile
  const int col0 = ct * kQTileCols;
  const int ncols = min(kQTileCols, W - col0);

  // Offsets and the experts' decode scales (in the column staging area until
  // the column phase): the four loads go out together at clamped indices.
  float* s_erow = reinterpret_cast<float*>(stage_sc);  // D_row of each expert (E <= 1024)
  float* s_ecol = s_erow + 1024;                       // D_col of each expert
  {
    const int io = min(tid, E), ie = min(tid, E - 1);
    const int o = offs[io], po = poffs[io];
    const float dr = row_scale[ie], dc = col_scale[ie];
    s_offs[io] = o;  // threads past E rewrite the last entries with their own values
    s_poffs[io] = po;
    s_erow[ie] = dr;
    s_ecol[ie] = dc;
    for (int i = tid + kQThreads; i <= E; i += kQThreads) {
      s_offs[i] = offs[i];
      s_poffs[i] = poffs[i];
      if (i < E) {
        s_erow[i] = row_scale[i];
        s_ecol[i] = col_scale[i];
      }
    }
  }
  __syncthreads();
  const int ptotal = s_poffs[E];
  if (gp_base >= ptotal) return;  // whole tile beyond the padded rows (uniform)

  if (tid < kQBlocks) {
    const int gp = gp_base + 16 * tid;
    const int live = gp < ptotal;
    s_live[tid] = live;
    if (live) {
      int lo = 0, hi = E - 1;  // last e with poffs[e] <= gp
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (s_poffs[mid] <= gp) lo = mid; else hi = mid - 1;
      }
      const int e = lo;
      const int poff = s_poffs[e], plen = s_poffs[e + 1] - poff;
      const int row0 = s_offs[e] + (gp - poff);                   // real row of the block's first row
      s_row0[tid] = row0;
      s_nreal[tid] = min(16, max(0, s_offs[e + 1] - row0));       // real rows of the block
      s_drow[tid] = s_erow[e];
      s_dcol[tid] = s_ecol[e];
      s_cbase[tid] = (uint64_t)W * (uint32_t)(poff >> 1) + (uint32_t)((gp - poff) >> 1);
      s_cstr[tid] = (uint32_t)(plen >> 1);
      s_sbase[tid] = (uint64_t)W * (uint32_t)(poff >> 4) + (uint32_t)((gp - poff) >> 4);
      s_sstr[tid] = (uint32_t)(plen >> 4);
    }
  }
  __syncthreads();
  {
    // significand tables: thread = (block, row/col, j)
    const int b = tid >> 4, rc = (tid >> 3) & 1, j = tid & 7;
    if (s_live[b]) {
      const float D = rc ? s_dcol[b] : s_drow[b];
      int kD = 0;
      const float mD = D > 0.0f ? split_pow2(D, kD) : 1.0f;
      s_tab[b][rc][j] = mant_entry(j, mD);
    }
  }

  const int cg = tid & 15, m = tid >> 4;
  const bool live = s_live[m] && cg * 8 < ncols;
  // Addresses: a workgroup-uniform base at the tile's first real row (block 0
  // of a live tile is live) plus 32-bit per-lane offsets, so each access costs
  // one 24-bit multiply-add instead of 64-bit address arithmetic.  The tile's
  // rows lie within 256 + 15 rows of that base: offsets stay below 2^32.
  const uint32_t rbase = (uint32_t)__builtin_amdgcn_readfirstlane(s_row0[0]);
  uint4 v[16];
  if (live) {
    const int row0 = s_row0[m], nreal = s_nreal[m];
    const uint32_t rrel = (uint32_t)row0 - rbase;
    if (nreal > 0) {
      // branch-free: rows past the expert's end re-read its last row and are zeroed
      if (!RECOMPUTE) {
        const char* base = reinterpret_cast<const char*>(dx + (size_t)rbase * (uint32_t)W + col0);
        const uint32_t w2 = 2u * (uint32_t)W, o0 = rrel * w2 + 16u * (uint32_t)cg;
        // plain loads, not streaming ones: dX was just written by the epilogue
        // and much of it still sits in the last-level cache
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          uint4 t = *reinterpret_cast<const uint4*>(base + (o0 + __umul24((uint32_t)min(i, nreal - 1), w2)));
          v[i] = i < nreal ? t : make_uint4(0, 0, 0, 0);
        }
      } else {
        const int F = W >> 1;
        const bool want_b = cg >= 8;                             // this thread keeps db (else da)
        const char* pbase = reinterpret_cast<const char*>(preact + (size_t)rbase * (uint32_t)W + (col0 >> 1));
        const char* dbase = reinterpret_cast<const char*>(dy + (size_t)rbase * (uint32_t)F + (col0 >> 1));
        const uint32_t w2 = 2u * (uint32_t)W, f2 = 2u * (uint32_t)F, jl = 16u * (uint32_t)(cg & 7);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t r = rrel + (uint32_t)min(i, nreal - 1);
          const uint32_t op = __umul24(r, w2) + jl, od = __umul24(r, f2) + jl;
          uint4 va = ld_stream16(pbase + op), vb = ld_stream16(pbase + (op + f2));
          uint4 vd = ld_stream16(dbase + od);
          uint32_t wa[4] = {va.x, va.y, va.z, va.w}, wb[4] = {vb.x, vb.y, vb.z, vb.w}, wd[4] = {vd.x, vd.y, vd.z, vd.w};
          uint32_t o[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float da0, db0, da1, db1;
            dswiglu_pair(bf16lo(wa[q]), bf16lo(wb[q]), bf16lo(wd[q]), da0, db0);
            dswiglu_pair(bf16hi(wa[q]), bf16hi(wb[q]), bf16hi(wd[q]), da1, db1);
            o[q] = want_b ? bf16pair(db0, db1) : bf16pair(da0, da1);
          }
          v[i] = i < nreal ? make_uint4(o[0], o[1], o[2], o[3]) : make_uint4(0, 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __syncthreads();  // tables ready

  // columnwise first: its transposed copy-out stores then drain while the
  // rowwise operand is computed (rowwise first leaves them as a final burst)
  uint32_t klo = 0, khi = 0;
  uint64_t n_base = 0;
  if (SR) {
    const uint64_t seed = sr_state[0];
    klo = (uint32_t)seed;
    khi = (uint32_t)(seed >> 32);
    n_base = sr_state[1];
  }
  if (live) {
    if (!SR) {
      // the block's expert has D_row >= 2^-85 (D_col = 4 D_row): the fast
      // block quantizers give the same codes without two dormant checks
      if (s_drow[m] >= 0x1p-85f) fc1_columnwise<0, 4, false, true>(v, s_dcol[m], s_tab[m][1], cg, m, stage_codes, stage_sc);
      else fc1_columnwise<0, 4>(v, s_dcol[m], s_tab[m][1], cg, m, stage_codes, stage_sc);
    } else {
      // the thread's 8 columns are contiguous in dX (also in the recompute mapping)
      const uint64_t h0 = (uint64_t)qtile_col<RECOMPUTE>(col0, 8 * cg, W);
      const uint64_t n0 = n_base + (uint64_t)(uint32_t)T * (uint32_t)W + 2 * (s_cbase[m] + h0 * s_cstr[m]);
      fc1_columnwise<0, 4, SR>(v, s_dcol[m], s_tab[m][1], cg, m, stage_codes, stage_sc, n0,
                                 2 * (uint64_t)s_cstr[m], klo, khi);
    }
  }
  __syncthreads();
  // transposed copy-out: thread (b, j) writes block b of columns j, j+16, ...
  const int b = tid % kQBlocks;
  if (s_live[b]) {
    const uint64_t cstr = s_cstr[b], sstr = s_sstr[b];
    // running pointers: column c advances by kQThreads / kQBlocks per step
    // (the recompute mapping's db half starts at column 64: its own base)
    const int c0 = tid / kQBlocks;
    const uint64_t h0 = (uint64_t)qtile_col<RECOMPUTE>(col0, c0, W);
    uint8_t* pc = col_codes + s_cbase[b] + h0 * cstr;
    uint8_t* ps = col_scales + s_sbase[b] + h0 * sstr;
    const uint64_t cstep = (uint64_t)(kQThreads / kQBlocks) * cstr, sstep = (uint64_t)(kQThreads / kQBlocks) * sstr;
#pragma unroll
    for (int r = 0; r < (kQTileCols * kQBlocks) / kQThreads; ++r) {
      const int c = r * (kQThreads / kQBlocks) + c0;
      if (c >= ncols) break;
      if (RECOMPUTE && c == 64 + c0) {  // da columns end, db columns begin
        const uint64_t h = (uint64_t)qtile_col<RECOMPUTE>(col0, c, W);
        pc = col_codes + s_cbase[b] + h * cstr;
        ps = col_scales + s_sbase[b] + h * sstr;
      }
      *reinterpret_cast<uint2*>(pc) = stage_codes[qstage_at(c, b)];
      *ps = (uint8_t)stage_sc[qstage_at(c, b)];
      pc += cstep;
      ps += sstep;
    }
  }
  if (live) {
    const uint32_t rrel = (uint32_t)s_row0[m] - rbase;
    const int xcol = qtile_col<RECOMPUTE>(col0, 8 * cg, W);  // this thread's first dX column
    uint8_t* const rcb = row_codes + (size_t)rbase * (uint32_t)(W >> 1);
    uint8_t* const rsb = row_scales + (size_t)rbase * (uint32_t)(W >> 4);
    const uint32_t rco = rrel * (uint32_t)(W >> 1) + (uint32_t)(xcol >> 1);
    const uint32_t rso = rrel * (uint32_t)(W >> 4) + (uint32_t)(xcol >> 4);
    const uint64_t rn0 = n_base + (uint64_t)(uint32_t)s_row0[m] * (uint32_t)W + (uint32_t)xcol;
    if (!SR && s_drow[m] >= 0x1p-85f)
      fc1_rowwise<0, true>(v, s_nreal[m], s_drow[m], s_tab[m][0], rcb, rco, rsb, rso, (uint32_t)W, (cg & 1) == 0);
    else
      fc1_rowwise<SR>(v, s_nreal[m], s_drow[m], s_tab[m][0], rcb, rco, rsb, rso, (uint32_t)W, (cg & 1) == 0, rn0, klo,
                      khi);
  }
}


}  // namespace mtb

using namespace mtb;

// Workspace: the row maxima (one word per row, padded to a multiple of 4
// rows, 16-byte aligned at the start), then the offsets and padded offsets.
static size_t rowmax_bytes(int64_t tokens) { return (size_t)((tokens + 3) / 4) * 16; }

MTB_EXPORT size_t dswiglu_workspace_bytes(int64_t tokens, int64_t num_experts) {
  if (num_experts < 1 || tokens < 0 || tokens >= kSizeLimit || num_experts >= kSizeLimit) return 0;
  return rowmax_bytes(tokens) + (size_t)(2 * (num_experts + 1) * sizeof(int32_t));
}

static int32_t dswiglu_quant_impl(const uint16_t* preact, const uint16_t* dy, int64_t tokens, int64_t ffn,
                                       const int32_t* counts, int64_t num_experts, uint16_t* dx, float* amax,
                                       uint8_t* row_codes, uint8_t* row_scales, float* row_scale,
                                       uint8_t* col_codes, uint8_t* col_scales, float* col_scale,
                                       void* workspace, size_t workspace_bytes,
                                       const uint64_t* sr_state, int sr_words, void* stream) {
  if (tokens < 0 || ffn <= 0 || ffn % 64 != 0 || num_experts < 1 || num_experts > 1024) return EP_ERR_SHAPE;
  if (tokens >= INT32_MAX / 8 || tokens + 16 * num_experts >= INT32_MAX / 8 || ffn > (1 << 20)) return EP_ERR_RANGE;
  if (!counts || !amax || !row_scale || !col_scale) return EP_ERR_NULL;
  if (tokens > 0 && (!preact || !dy || !row_codes || !row_scales || !col_codes || !col_scales)) return EP_ERR_NULL;
  if (!workspace || workspace_bytes < dswiglu_workspace_bytes(tokens, num_experts) || ((uintptr_t)workspace & 15))
    return EP_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int T = (int)tokens, F = (int)ffn, E = (int)num_experts;
  uint32_t* rowmax = (uint32_t*)workspace;
  int32_t* offs = (int32_t*)((char*)workspace + rowmax_bytes(tokens));
  int32_t* poffs = offs + (E + 1);
  if (T > 0) {
    // dX not wanted: the epilogue keeps only each row's max |dX|
    const int nb = (F / 8 + 63) / 64;
    const dim3 eg((unsigned)((T + 3) / 4)), eb(256);
#define MTB_EPI(ST, NBV) hipLaunchKernelGGL((k_dswiglu_epilogue<ST, NBV>), eg, eb, 0, s, preact, dy, T, F, dx, rowmax)
#define MTB_EPI_NB(ST)                  \
  do {                                  \
    if (nb <= 1) MTB_EPI(ST, 1);        \
    else if (nb <= 2) MTB_EPI(ST, 2);   \
    else MTB_EPI(ST, 4);                \
  } while (0)
    if (dx) MTB_EPI_NB(true);
    else MTB_EPI_NB(false);
#undef MTB_EPI_NB
#undef MTB_EPI
  }
  hipLaunchKernelGGL(k_dswiglu_reduce, dim3((unsigned)E), dim3(1024), 0, s, counts, E, T, rowmax, offs, poffs, amax,
                     row_scale, col_scale);
  // padded rows never exceed T + 15 E; tiles beyond poffs[E] exit at once
  const int64_t prow_bound = tokens + 15 * num_experts;
  const int64_t n_rt = (prow_bound + kQTileRows - 1) / kQTileRows, n_ct = (2 * F + kQTileCols - 1) / kQTileCols;
  if (n_rt * n_ct * kQThreads >= ((int64_t)1 << 32)) return EP_ERR_RANGE;  // one 1-D grid
  const dim3 grid((unsigned)(n_rt * n_ct)), block(kQThreads);
#define MTB_FC1(RC, SRM)                                                                                        \
  hipLaunchKernelGGL((k_fc1_quant<RC, SRM>), grid, block, 0, s, dx, preact, dy, T, 2 * F, E, (int)n_ct, offs, poffs, \
                     row_scale, col_scale, row_codes, row_scales, col_codes, col_scales, sr_state)
  const int srm = sr_state ? (sr_words == 2 ? 2 : 1) : 0;
  if (srm == 0) {
    if (dx) MTB_FC1(false, 0);
    else MTB_FC1(true, 0);
  } else if (srm == 1) {
    if (dx) MTB_FC1(false, 1);
    else MTB_FC1(true, 1);
  } else {
    if (dx) MTB_FC1(false, 2);
    else MTB_FC1(true, 2);
  }
#undef MTB_FC1
  return launch_status();
}

MTB_EXPORT int32_t dswiglu_nvfp4_quant(const uint16_t* preact, const uint16_t* dy, int64_t tokens, int64_t ffn,
                                       const int32_t* counts, int64_t num_experts, uint16_t* dx, float* amax,
                                       uint8_t* row_codes, uint8_t* row_scales, float* row_scale,
                                       uint8_t* col_codes, uint8_t* col_scales, float* col_scale,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  return dswiglu_quant_impl(preact, dy, tokens, ffn, counts, num_experts, dx, amax, row_codes, row_scales, row_scale,
                            col_codes, col_scales, col_scale, workspace, workspace_bytes, nullptr, 0, stream);
}

MTB_EXPORT int32_t dswiglu_nvfp4_quant_sr(const uint16_t* preact, const uint16_t* dy, int64_t tokens, int64_t ffn,
                                          const int32_t* counts, int64_t num_experts, uint16_t* dx, float* amax,
                                          uint8_t* row_codes, uint8_t* row_scales, float* row_scale,
                                          uint8_t* col_codes, uint8_t* col_scales, float* col_scale,
                                          void* workspace, size_t workspace_bytes, const uint64_t* sr_state,
                                          void* stream) {
  if (!sr_state) return EP_ERR_NULL;
  return dswiglu_quant_impl(preact, dy, tokens, ffn, counts, num_experts, dx, amax, row_codes, row_scales, row_scale,
                            col_codes, col_scales, col_scale, workspace, workspace_bytes, sr_state, 1, stream);
}

MTB_EXPORT int32_t dswiglu_nvfp4_quant_sr_stream(const uint16_t* preact, const uint16_t* dy, int64_t tokens,
                                                 int64_t ffn, const int32_t* counts, int64_t num_experts, uint16_t* dx,
                                                 float* amax, uint8_t* row_codes, uint8_t* row_scales,
                                                 float* row_scale, uint8_t* col_codes, uint8_t* col_scales,
                                                 float* col_scale, void* workspace, size_t workspace_bytes,
                                                 const uint64_t* sr_state, void* stream) {
  if (!sr_state) return EP_ERR_NULL;
  return dswiglu_quant_impl(preact, dy, tokens, ffn, counts, num_experts, dx, amax, row_codes, row_scales, row_scale,
                            col_codes, col_scales, col_scale, workspace, workspace_bytes, sr_state, 2, stream);
}

// ------------------------------------------------------------------ allocation-free variant
// dswiglu_nvfp4_quant for callers that cannot allocate (code under HIP graph
// capture, serving loops that forbid hipMalloc): its workspace -- one max
// |dX| word per row and the expert offsets, each fully written by the call
// before it is read, so nothing needs clearing -- lives in a file-scope
// device array instead of a caller buffer.  Each GPU holds its own copy for
// the life of the process; every call on one GPU shares it, so calls that
// overlap in time on one GPU race.
namespace {
constexpr size_t kScratchBytes = EP_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device, looked up once per
// device (the host-side name is only a stand-in for the symbol).
int32_t scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return EP_ERR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return EP_ERR_HIP;
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return EP_OK;
}
}  // namespace

MTB_EXPORT int32_t dswiglu_nvfp4_quant_noalloc(const uint16_t* preact, const uint16_t* dy, int64_t tokens,
                                               int64_t ffn, const int32_t* counts, int64_t num_experts, uint16_t* dx,
                                               float* amax, uint8_t* row_codes, uint8_t* row_scales, float* row_scale,
                                               uint8_t* col_codes, uint8_t* col_scales, float* col_scale,
                                               void* stream) {
  if (tokens < 0 || num_experts < 1) return EP_ERR_SHAPE;
  const size_t need = dswiglu_workspace_bytes(tokens, num_experts);   // 0: sizes past any byte count
  if (need == 0 || need > kScratchBytes) return EP_ERR_SCRATCH;
  void* ws = nullptr;
  const int32_t st = scratch_ptr(&ws);
  if (st != EP_OK) return st;
  return dswiglu_quant_impl(preact, dy, tokens, ffn, counts, num_experts, dx, amax, row_codes, row_scales, row_scale,
                            col_codes, col_scales, col_scale, ws, kScratchBytes, nullptr, 0, stream);
}
