// NVFP4 row pack (round-to-nearest and stochastic) and MXFP8 pack for gfx950.
//
// NVFP4 (P1, PR description): one BF16 token row -> E2M1 codes, one E4M3
// scale per 16 elements and a power-of-two FP32 token scale t.  MXFP8 (P2,
// description): E4M3 data with one E8M0 scale per 32 elements.
//
// Mapping (H < 4096): one wave64 per row; lane l owns 16-element blocks l,
// l+64, ..., loaded as two 16-byte vectors, so a block's max needs no
// cross-lane work and one wave-wide reduction gives the row max.  The whole
// row stays in VGPRs between the max and the encode.  From H = 4096 on, one
// 256-thread workgroup per row (k_nvfp4_pack_wg: thread j owns blocks j,
// j + 256, ...; the row max crosses its four waves through LDS).
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace mtb {

struct BlockQuant {
  float r_hi, r_lo;  // split reciprocal of the scale significand, times 2^P
  float scale;       // 2^(k + e + P): handed to the converter (exponent only)
  int kexp;          // k + e + P
};

// Block scale code and the quotient parameters for one 16-element block of a
// row with token exponent e.  ab = block max |x|.
__device__ __forceinline__ BlockQuant nvfp4_block(float ab, int e, uint32_t& sc_out) {
  // s_b = E4M3(ab / (6 * 2^e)): fl32(ab/6) never sits on an E4M3 tie unless it
  // is exact, so one float32 rounding before the E4M3 rounding changes nothing.
  bool tiny = ab < 0x1p-100f;
  float abs_ = tiny ? ab * 0x1p64f : ab;
  float y = __builtin_ldexpf(div6(abs_), -e - (tiny ? 64 : 0));
  uint32_t sc = e4m3_encode(fminf(y, 448.0f));
  float s = e4m3_decode(sc);
  sc_out = sc;
  BlockQuant q;
  if (s > 0.0f) {
    QuotSplit qs = quot_split(s);
    int K = qs.k + e;
    int P = K < -104 ? -104 - K : 0;  // keep x * r_lo and the converter's scale in normal range
    q.r_hi = __builtin_ldexpf(qs.r_hi, P);
    q.r_lo = __builtin_ldexpf(qs.r_lo, P);
    q.kexp = K + P;
  } else {
    q.r_hi = 0.0f;  // every element becomes a signed zero
    q.r_lo = 0.0f;
    q.kexp = 0;
  }
  q.scale = pow2f(q.kexp);
  return q;
}

__device__ __forceinline__ int token_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int E, sub = 0;
  if (amax < 0x1p-126f) { amax *= 0x1p64f; sub = 64; }  // BF16 subnormal: normalise first
  E = __builtin_amdgcn_frexp_expf(amax) - 1 - sub;
  float m = __builtin_amdgcn_frexp_mantf(amax) * 2.0f;
  return E - 11 + (m > 1.3125f ? 1 : 0);  // least e with amax <= 2688 * 2^e
}

// Stochastic rounding of one element: u = x / (m 2^-P) (signed), magnitude
// v = |u| * 2^-kexp = fl32(|x| / (s t)); r = 24 random bits.  Returns the
// rounded grid value with x's sign (then encoded exactly by the converter).
__device__ __forceinline__ float sr_round(float u, int kexp, uint32_t r) {
  float v = __builtin_ldexpf(fabsf(u), -kexp);
  float rf = (float)r * 0x1p-24f;
  float res;
  if (v >= 6.0f) {
    res = 6.0f;
  } else {
    // grid spacing 2^q: 0.5 on [0, 2), 1 on [2, 4), 2 on [4, 6)
    int q = v < 2.0f ? -1 : (v < 4.0f ? 0 : 1);
    float w = __builtin_ldexpf(v, -q);
    float fl = __builtin_floorf(w);
    float frac = w - fl;
    res = __builtin_ldexpf(fl + (rf < frac ? 1.0f : 0.0f), q);
  }
  return __builtin_copysignf(res, u);
}

// Where a packed row goes: the packed-row buffer (codes, scales and t of row r
// at r * row_bytes) or the grouped rowwise operand (codes, scales and t in
// three arrays, grouped row g at g * H/2, g * H/16 and g).
constexpr int kMaxScatter = 32;  // top-k limit of the fused pack + scatter

struct RowOut {
  uint8_t* codes;
  uint8_t* scales;
  uint8_t* t;
  uint32_t cstride, sstride, tstride;  // bytes between consecutive rows
};

__device__ __forceinline__ void store_block(const RowOut& o, uint32_t g, int j, uint32_t o0, uint32_t o1, uint32_t sc) {
  uint32_t* cw = reinterpret_cast<uint32_t*>(o.codes + (size_t)g * o.cstride + 8 * j);
  cw[0] = o0;
  cw[1] = o1;
  o.scales[(size_t)g * o.sstride + j] = (uint8_t)sc;
}

__device__ __forceinline__ void store_t(const RowOut& o, uint32_t g, float t) {
  *reinterpret_cast<float*>(o.t + (size_t)g * o.tstride) = t;
}

// The destinations of token row `row`: itself (packed rows), or its top-k
// grouped rows dst_row[row*k + j] (SCATTER; entries outside [0, r_cap) skipped).
template <bool SCATTER>
__device__ __forceinline__ int row_dests(int row, const int32_t* dst_row, int k, int r_cap, uint32_t* g) {
  if (!SCATTER) {
    g[0] = (uint32_t)row;
    return 1;
  }
  int n = 0;
  for (int j = 0; j < k; ++j) {
    int d = dst_row[(size_t)row * k + j];
    if (d >= 0 && d < r_cap) g[n++] = (uint32_t)d;
  }
  return n;
}

__device__ __forceinline__ void encode_rne(const uint4& v0, const uint4& v1, const BlockQuant& q,
                                           uint32_t& o0, uint32_t& o1) {
  uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  float u[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u[2 * i] = quot_apply(bf16lo(w[i]), q.r_hi, q.r_lo);
    u[2 * i + 1] = quot_apply(bf16hi(w[i]), q.r_hi, q.r_lo);
  }
  o0 = fp4_pack2<0>(__float_as_uint(u[0]), u[0], u[1], q.scale);  // the other bytes: overwritten next
  o0 = fp4_pack2<1>(o0, u[2], u[3], q.scale);
  o0 = fp4_pack2<2>(o0, u[4], u[5], q.scale);
  o0 = fp4_pack2<3>(o0, u[6], u[7], q.scale);
  o1 = fp4_pack2<0>(__float_as_uint(u[8]), u[8], u[9], q.scale);
  o1 = fp4_pack2<1>(o1, u[10], u[11], q.scale);
  o1 = fp4_pack2<2>(o1, u[12], u[13], q.scale);
  o1 = fp4_pack2<3>(o1, u[14], u[15], q.scale);
}


// Stochastic encode of one 16-element block at stream positions n0 .. n0+15.
template <int MODE>
__device__ __forceinline__ void encode_sr(const uint4& v0, const uint4& v1, const BlockQuant& q, uint64_t n0,
                                          uint32_t seed_lo, uint32_t seed_hi, uint32_t& o0, uint32_t& o1) {
  constexpr bool kElement = MODE == EP_ROUND_SR_ELEMENT || MODE == EP_ROUND_SR_ELEMENT_CARRY;
  constexpr bool kCarry = MODE == EP_ROUND_SR_ELEMENT_CARRY || MODE == EP_ROUND_SR_STREAM_CARRY;
  uint32_t rnd[16];
  if (kElement) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint64_t n = n0 + i;
      rnd[i] = philox4x32_10((uint32_t)n, (uint32_t)(n >> 32), 0u, 0u, seed_lo, seed_hi).x;
    }
  } else {
    // word n of the stream is word (n & 3) of block n >> 2
    uint64_t cur = n0 >> 2;
    U4 blk = philox4x32_10((uint32_t)cur, (uint32_t)(cur >> 32), 0u, 0u, seed_lo, seed_hi);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint64_t n = n0 + i;
      if ((n >> 2) != cur) {
        cur = n >> 2;
        blk = philox4x32_10((uint32_t)cur, (uint32_t)(cur >> 32), 0u, 0u, seed_lo, seed_hi);
      }
      uint32_t sel = (uint32_t)n & 3u;
      rnd[i] = sel == 0 ? blk.x : (sel == 1 ? blk.y : (sel == 2 ? blk.z : blk.w));
    }
  }
  uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  if (kCarry) {
    // the quotient fl32(x / m) * 2^P and the converter's power of two, as for
    // round-to-nearest; the converter decides each element with its own word
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      b[i] = sr_code_lo(quot_apply(bf16lo(w[i]), q.r_hi, q.r_lo), rnd[2 * i], q.scale) |
             sr_code_hi(quot_apply(bf16hi(w[i]), q.r_hi, q.r_lo), rnd[2 * i + 1], q.scale);
    o0 = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    o1 = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    return;
  }
  float g[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    g[2 * i] = sr_round(quot_apply(bf16lo(w[i]), q.r_hi, q.r_lo), q.kexp, rnd[2 * i] >> 8);
    g[2 * i + 1] = sr_round(quot_apply(bf16hi(w[i]), q.r_hi, q.r_lo), q.kexp, rnd[2 * i + 1] >> 8);
  }
  // g holds exact grid values with x's sign: encode with scale 1
  o0 = fp4_pack2<0>(__float_as_uint(g[0]), g[0], g[1], 1.0f);  // the other bytes: overwritten next
  o0 = fp4_pack2<1>(o0, g[2], g[3], 1.0f);
  o0 = fp4_pack2<2>(o0, g[4], g[5], 1.0f);
  o0 = fp4_pack2<3>(o0, g[6], g[7], 1.0f);
  o1 = fp4_pack2<0>(__float_as_uint(g[8]), g[8], g[9], 1.0f);
  o1 = fp4_pack2<1>(o1, g[10], g[11], 1.0f);
  o1 = fp4_pack2<2>(o1, g[12], g[13], 1.0f);
  o1 = fp4_pack2<3>(o1, g[14], g[15], 1.0f);
}

// Round-to-nearest: the row stays in VGPRs between the max and the encode.
template <int NB, bool SCATTER>
__global__ __launch_bounds__(256) void k_nvfp4_pack(const uint16_t* __restrict__ x, int rows, int H, const RowOut o,
                                                   const int32_t* __restrict__ dst_row, int k, int r_cap) {
  const int lane = threadIdx.x & 63;
  const int row = (int)(blockIdx.x * 4u + (threadIdx.x >> 6));
  if (row >= rows) return;
  const int nblk = H >> 4;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)row * H);

  uint4 v[NB][2];
  uint32_t bmax[NB];
  uint32_t rmax = 0;
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    int j = c * 64 + lane;
    if (j < nblk) {
      v[c][0] = ld_stream16(xr + 2 * j);
      v[c][1] = ld_stream16(xr + 2 * j + 1);
      uint32_t a = absmax_bf16x8(v[c][0]), b = absmax_bf16x8(v[c][1]);
      bmax[c] = a > b ? a : b;
    } else {
      v[c][0] = v[c][1] = make_uint4(0, 0, 0, 0);
      bmax[c] = 0;
    }
    rmax = rmax > bmax[c] ? rmax : bmax[c];
  }
  rmax = wave_max_u32(rmax);
  const int e = token_exponent(__uint_as_float(rmax << 16));
  uint32_t g[SCATTER ? kMaxScatter : 1];
  const int nd = row_dests<SCATTER>(row, dst_row, k, r_cap, g);
  if (lane == 0)
    for (int d = 0; d < nd; ++d) store_t(o, g[d], __builtin_ldexpf(1.0f, e));
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    int j = c * 64 + lane;
    if (j >= nblk) continue;
    uint32_t sc, o0, o1;
    BlockQuant q = nvfp4_block(__uint_as_float(bmax[c] << 16), e, sc);
    encode_rne(v[c][0], v[c][1], q, o0, o1);
    for (int d = 0; d < nd; ++d) store_block(o, g[d], j, o0, o1, sc);
  }
}

// Rows of >= 256 blocks (H >= 4096): one workgroup of 256 threads per row,
// thread j owns blocks j, j+256, ... (NBW of them), so a 4096-wide row is one
// block per thread; the row max goes through LDS.
template <int NBW, bool SCATTER>
__global__ __launch_bounds__(256) void k_nvfp4_pack_wg(const uint16_t* __restrict__ x, int /* rows: the grid */, int H,
                                                      const RowOut o,
                                                      const int32_t* __restrict__ dst_row, int k, int r_cap) {
  __shared__ uint32_t red[4];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int nblk = H >> 4;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)row * H);
  uint4 v[NBW][2];
  uint32_t bmax[NBW];
  uint32_t rmax = 0;
#pragma unroll
  for (int c = 0; c < NBW; ++c) {
    int j = c * 256 + tid;
    if (j < nblk) {
      v[c][0] = ld_stream16(xr + 2 * j);
      v[c][1] = ld_stream16(xr + 2 * j + 1);
      uint32_t a = absmax_bf16x8(v[c][0]), b = absmax_bf16x8(v[c][1]);
      bmax[c] = a > b ? a : b;
    } else {
      v[c][0] = v[c][1] = make_uint4(0, 0, 0, 0);
      bmax[c] = 0;
    }
    rmax = rmax > bmax[c] ? rmax : bmax[c];
  }
  rmax = wave_max_u32(rmax);
  if ((tid & 63) == 0) red[tid >> 6] = rmax;
  __syncthreads();
  rmax = max(max(red[0], red[1]), max(red[2], red[3]));
  const int e = token_exponent(__uint_as_float(rmax << 16));
  uint32_t g[SCATTER ? kMaxScatter : 1];
  const int nd = row_dests<SCATTER>(row, dst_row, k, r_cap, g);
  if (tid == 0)
    for (int d = 0; d < nd; ++d) store_t(o, g[d], __builtin_ldexpf(1.0f, e));
#pragma unroll
  for (int c = 0; c < NBW; ++c) {
    int j = c * 256 + tid;
    if (j >= nblk) continue;
    uint32_t sc, o0, o1;
    BlockQuant q = nvfp4_block(__uint_as_float(bmax[c] << 16), e, sc);
    encode_rne(v[c][0], v[c][1], q, o0, o1);
    for (int d = 0; d < nd; ++d) store_block(o, g[d], j, o0, o1, sc);
  }
}

// Stochastic rounding: ALU-bound on the Philox blocks, so the second pass
// re-reads each block (from cache) instead of holding the row in VGPRs.
template <int MODE>
__global__ __launch_bounds__(256) void k_nvfp4_pack_sr(const uint16_t* __restrict__ x, int rows, int H, const RowOut o,
                                                      const uint64_t* __restrict__ sr_state) {
  const int lane = threadIdx.x & 63;
  const int row = (int)(blockIdx.x * 4u + (threadIdx.x >> 6));
  if (row >= rows) return;
  const int nblk = H >> 4;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)row * H);
  uint32_t rmax = 0;
  for (int j = lane; j < nblk; j += 64) {
    uint32_t a = absmax_bf16x8(xr[2 * j]), b = absmax_bf16x8(xr[2 * j + 1]);
    a = a > b ? a : b;
    rmax = rmax > a ? rmax : a;
  }
  rmax = wave_max_u32(rmax);
  const int e = token_exponent(__uint_as_float(rmax << 16));
  if (lane == 0) store_t(o, (uint32_t)row, __builtin_ldexpf(1.0f, e));
  const uint64_t seed = sr_state[0];
  const uint32_t seed_lo = (uint32_t)seed, seed_hi = (uint32_t)(seed >> 32);
  const uint64_t n_row = sr_state[1] + (uint64_t)row * (uint64_t)H;
#pragma unroll 1
  for (int j = lane; j < nblk; j += 64) {
    uint4 v0 = xr[2 * j], v1 = xr[2 * j + 1];
    uint32_t a = absmax_bf16x8(v0), b = absmax_bf16x8(v1);
    uint32_t sc, o0, o1;
    BlockQuant q = nvfp4_block(__uint_as_float((a > b ? a : b) << 16), e, sc);
    encode_sr<MODE>(v0, v1, q, n_row + (uint64_t)(16 * j), seed_lo, seed_hi, o0, o1);
    store_block(o, (uint32_t)row, j, o0, o1, sc);
  }
}

// The same for H <= 4096 (at most four 16-element blocks per lane), rows held
// in registers and software-pipelined: a wave quantizes rows wave, wave + nw,
// ... and issues the loads of its next row before the Philox work of the
// current one, so the loads of one row overlap the arithmetic of the previous
// (a grid of one row per wave runs every load before any arithmetic).
template <int MODE>
__device__ __forceinline__ void sr_block(const uint4& v0, const uint4& v1, int j, int e, uint64_t n_row,
                                         uint32_t seed_lo, uint32_t seed_hi, const RowOut& o, int row) {
  uint32_t a = absmax_bf16x8(v0), b = absmax_bf16x8(v1);
  uint32_t sc, o0, o1;
  BlockQuant q = nvfp4_block(__uint_as_float((a > b ? a : b) << 16), e, sc);
  encode_sr<MODE>(v0, v1, q, n_row + (uint64_t)(16 * j), seed_lo, seed_hi, o0, o1);
  store_block(o, (uint32_t)row, j, o0, o1, sc);
}

// One row's NB blocks per lane held in registers (blocks j = lane + 64k; a
// lane past the row's end takes the last block: it computes and stores that
// block's bytes again, the same values).  Everything is unconditional, so the
// number of stores between two rows' loads is fixed and the wait for a row's
// data does not wait for the previous row's stores.
template <int NB>
struct SrRow {
  uint4 a[NB], b[NB];
};

template <int MODE, int NB>
__global__ __launch_bounds__(256) void k_nvfp4_pack_sr_rows(const uint16_t* __restrict__ x, int rows, int H,
                                                           const RowOut o, const uint64_t* __restrict__ sr_state) {
  const int lane = threadIdx.x & 63;
  const int nw = (int)gridDim.x * 4;
  int row = (int)(blockIdx.x * 4u + (threadIdx.x >> 6));
  if (row >= rows) return;
  const int nblk = H >> 4;  // 64 * (NB / 2) < nblk <= 64 * NB
  const uint64_t seed = sr_state[0];
  const uint32_t seed_lo = (uint32_t)seed, seed_hi = (uint32_t)(seed >> 32);
  const uint64_t n_base = sr_state[1];
  int jb[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) jb[k] = min(lane + 64 * k, nblk - 1);
  auto load = [&](int r, SrRow<NB>& d) {
    const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)min(r, rows - 1) * H);
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      d.a[k] = xr[2 * jb[k]];
      d.b[k] = xr[2 * jb[k] + 1];
    }
  };
  auto quantize = [&](int r, const SrRow<NB>& d) {
    uint32_t rmax = 0;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const uint32_t m0 = absmax_bf16x8(d.a[k]), m1 = absmax_bf16x8(d.b[k]);
      const uint32_t m = m0 > m1 ? m0 : m1;  // a clamped block repeats a block of the row: no effect
      rmax = rmax > m ? rmax : m;
    }
    rmax = wave_max_u32(rmax);
    const int e = token_exponent(__uint_as_float(rmax << 16));
    store_t(o, (uint32_t)r, __builtin_ldexpf(1.0f, e));  // every lane, the same 4 bytes
    const uint64_t n_row = n_base + (uint64_t)r * (uint64_t)H;
    // written out, not a loop: the compiler does not unroll a loop of four
    // Philox-heavy bodies, and the row's registers would then go to scratch
    sr_block<MODE>(d.a[0], d.b[0], jb[0], e, n_row, seed_lo, seed_hi, o, r);
    if constexpr (NB > 1) sr_block<MODE>(d.a[1], d.b[1], jb[1], e, n_row, seed_lo, seed_hi, o, r);
    if constexpr (NB > 2) sr_block<MODE>(d.a[2], d.b[2], jb[2], e, n_row, seed_lo, seed_hi, o, r);
    if constexpr (NB > 3) sr_block<MODE>(d.a[3], d.b[3], jb[3], e, n_row, seed_lo, seed_hi, o, r);
  };
  // Two register sets used in turn: while one row is quantized the next row's
  // loads (row index clamped: always issued) are in flight.  The first row is
  // peeled so that every quantize, also the first in the loop, has the same
  // instructions between its loads and itself (its set's loads, one row's
  // stores, the other set's loads): the wait for its data then never includes
  // the stores before it.  The scheduling barriers keep the arithmetic of a
  // row from being hoisted above the next row's loads.
  SrRow<NB> s0, s1;
  load(row, s0);
  load(row + nw, s1);
  __builtin_amdgcn_sched_barrier(0);
  quantize(row, s0);
  for (;;) {
    if (row + nw >= rows) break;  // wave-uniform
    load(row + 2 * nw, s0);
    __builtin_amdgcn_sched_barrier(0);
    quantize(row + nw, s1);
    if (row + 2 * nw >= rows) break;
    load(row + 3 * nw, s1);
    __builtin_amdgcn_sched_barrier(0);
    quantize(row + 2 * nw, s0);
    row += 2 * nw;
  }
}

// ----------------------------------------------------------------- MXFP8
// Two lanes per 32-element block (16 elements each): one xor-1 exchange gives
// the block max.  Data goes out as one 16-byte store per lane.
__device__ __forceinline__ int mx_exponent(float a) {
  if (!(a > 0.0f)) return 0;
  int sub = 0;
  if (a < 0x1p-126f) { a *= 0x1p64f; sub = 64; }
  int E = __builtin_amdgcn_frexp_expf(a) - 1 - sub;
  float m = __builtin_amdgcn_frexp_mantf(a) * 2.0f;
  int e = E - 8 + (m > 1.75f ? 1 : 0);  // least e with a <= 448 * 2^e
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__device__ __forceinline__ uint32_t fp8x4_from_bf16(uint32_t w0, uint32_t w1, float scale) {
  i16x2 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, w0), scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, w1), scale, true);
  return __builtin_bit_cast(uint32_t, r);
}

// Tiny blocks (e < -126): scale the inputs by 2^64 first so that the
// converter's power of two stays a normal float.
__device__ __forceinline__ uint32_t fp8x4_from_bf16_tiny(uint32_t w0, uint32_t w1, float scale) {
  i16x2 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, bf16lo(w0) * 0x1p64f, bf16hi(w0) * 0x1p64f, scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, bf16lo(w1) * 0x1p64f, bf16hi(w1) * 0x1p64f, scale, true);
  return __builtin_bit_cast(uint32_t, r);
}

__global__ __launch_bounds__(256) void k_mxfp8_pack(const uint16_t* __restrict__ x, int64_t total_chunks,
                                                    int /* H: chunks run over the whole tensor */,
                                                    uint8_t* __restrict__ data,
                                                    uint8_t* __restrict__ scales) {
  // one lane per 16-element chunk; chunk index runs over the whole tensor
  int64_t ch = (int64_t)blockIdx.x * 256 + threadIdx.x;
  bool valid = ch < total_chunks;
  int64_t chc = valid ? ch : 0;
  const uint4* xp = reinterpret_cast<const uint4*>(x) + 2 * chc;
  uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
  if (valid) {
    a = ld_stream16(xp);
    b = ld_stream16(xp + 1);
  }
  uint32_t m0 = absmax_bf16x8(a), m1 = absmax_bf16x8(b);
  uint32_t m = m0 > m1 ? m0 : m1;
  uint32_t o = lane_xor1(m);  // partner chunk of the same block
  m = m > o ? m : o;
  if (!valid) return;
  int e = mx_exponent(__uint_as_float(m << 16));
  uint4 d;
  if (e >= -126) {
    float sc = pow2f(e);
    d.x = fp8x4_from_bf16(a.x, a.y, sc);
    d.y = fp8x4_from_bf16(a.z, a.w, sc);
    d.z = fp8x4_from_bf16(b.x, b.y, sc);
    d.w = fp8x4_from_bf16(b.z, b.w, sc);
  } else {
    float sc = pow2f(e + 64);
    d.x = fp8x4_from_bf16_tiny(a.x, a.y, sc);
    d.y = fp8x4_from_bf16_tiny(a.z, a.w, sc);
    d.z = fp8x4_from_bf16_tiny(b.x, b.y, sc);
    d.w = fp8x4_from_bf16_tiny(b.z, b.w, sc);
  }
  reinterpret_cast<uint4*>(data)[ch] = d;
  // scales [rows, H/32] row-major: block (row, col/32) is global block ch/2
  if ((ch & 1) == 0) scales[ch >> 1] = (uint8_t)(e + 127);
}

}  // namespace mtb

using namespace mtb;

// Round-to-nearest pack launch: workgroup per row for H >= 4096, else wave per row.
template <bool SCATTER>
static void launch_rne_pack(const uint16_t* x, int rows, int H, const RowOut& o, const int32_t* dst_row, int k,
                            int r_cap, hipStream_t s) {
  const int nb = (H / 16 + 63) / 64;
  dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (H >= 4096) {
    const int nbw = (H / 16 + 255) / 256;
    dim3 g1((unsigned)rows);
    if (nbw <= 1)
      hipLaunchKernelGGL((k_nvfp4_pack_wg<1, SCATTER>), g1, block, 0, s, x, rows, H, o, dst_row, k, r_cap);
    else if (nbw <= 2)
      hipLaunchKernelGGL((k_nvfp4_pack_wg<2, SCATTER>), g1, block, 0, s, x, rows, H, o, dst_row, k, r_cap);
    else
      hipLaunchKernelGGL((k_nvfp4_pack_wg<4, SCATTER>), g1, block, 0, s, x, rows, H, o, dst_row, k, r_cap);
  } else if (nb <= 1) {
    hipLaunchKernelGGL((k_nvfp4_pack<1, SCATTER>), grid, block, 0, s, x, rows, H, o, dst_row, k, r_cap);
  } else if (nb <= 2) {
    hipLaunchKernelGGL((k_nvfp4_pack<2, SCATTER>), grid, block, 0, s, x, rows, H, o, dst_row, k, r_cap);
  } else if (nb <= 4) {
    hipLaunchKernelGGL((k_nvfp4_pack<4, SCATTER>), grid, block, 0, s, x, rows, H, o, dst_row, k, r_cap);
  } else if (nb <= 8) {
    hipLaunchKernelGGL((k_nvfp4_pack<8, SCATTER>), grid, block, 0, s, x, rows, H, o, dst_row, k, r_cap);
  } else {
    hipLaunchKernelGGL((k_nvfp4_pack<16, SCATTER>), grid, block, 0, s, x, rows, H, o, dst_row, k, r_cap);
  }
}

MTB_EXPORT int32_t ep_nvfp4_pack(const uint16_t* x, int64_t rows, int64_t hidden, uint8_t* packed,
                                 int32_t round_mode, const uint64_t* sr_state, void* stream) {
  if (rows < 0 || hidden <= 0 || hidden % 64 != 0 || hidden > 16384) return EP_ERR_SHAPE;
  if (rows > (int64_t)INT32_MAX / 4 || rows * hidden >= ((int64_t)1 << 40)) return EP_ERR_RANGE;
  if (round_mode < EP_ROUND_NEAREST || round_mode > EP_ROUND_SR_STREAM_CARRY) return EP_ERR_DTYPE;
  if (rows == 0) return EP_OK;
  if (!x || !packed) return EP_ERR_NULL;
  if (round_mode != EP_ROUND_NEAREST && !sr_state) return EP_ERR_NULL;
  const int H = (int)hidden;
  const uint32_t rb = (uint32_t)(9 * H / 16 + 4);
  const RowOut o{packed, packed + (H >> 1), packed + (H >> 1) + (H >> 4), rb, rb, rb};
  dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  hipStream_t s = (hipStream_t)stream;
  if (round_mode != EP_ROUND_NEAREST && H <= 4096) {
    // two or more rows per wave, at most 12 waves per CU (the 4-block kernel's
    // registers allow 3 per SIMD: more would need a second round)
    const int64_t waves = std::min<int64_t>((rows + 1) / 2, 256 * 12);
    const dim3 g((unsigned)((waves + 3) / 4));
    const int nb = (H / 16 + 63) / 64;
#define MTB_SR_ROWS(M)                                                                                   \
  do {                                                                                                   \
    if (nb <= 1) hipLaunchKernelGGL((k_nvfp4_pack_sr_rows<M, 1>), g, block, 0, s, x, (int)rows, H, o, sr_state); \
    else if (nb <= 2) hipLaunchKernelGGL((k_nvfp4_pack_sr_rows<M, 2>), g, block, 0, s, x, (int)rows, H, o, sr_state); \
    else hipLaunchKernelGGL((k_nvfp4_pack_sr_rows<M, 4>), g, block, 0, s, x, (int)rows, H, o, sr_state); \
  } while (0)
    if (round_mode == EP_ROUND_SR_ELEMENT) MTB_SR_ROWS(EP_ROUND_SR_ELEMENT);
    else if (round_mode == EP_ROUND_SR_STREAM) MTB_SR_ROWS(EP_ROUND_SR_STREAM);
    else if (round_mode == EP_ROUND_SR_ELEMENT_CARRY) MTB_SR_ROWS(EP_ROUND_SR_ELEMENT_CARRY);
    else MTB_SR_ROWS(EP_ROUND_SR_STREAM_CARRY);
#undef MTB_SR_ROWS
    return launch_status();
  }
  if (round_mode == EP_ROUND_SR_ELEMENT) {
    hipLaunchKernelGGL(k_nvfp4_pack_sr<EP_ROUND_SR_ELEMENT>, grid, block, 0, s, x, (int)rows, H, o, sr_state);
  } else if (round_mode == EP_ROUND_SR_STREAM) {
    hipLaunchKernelGGL(k_nvfp4_pack_sr<EP_ROUND_SR_STREAM>, grid, block, 0, s, x, (int)rows, H, o, sr_state);
  } else if (round_mode == EP_ROUND_SR_ELEMENT_CARRY) {
    hipLaunchKernelGGL(k_nvfp4_pack_sr<EP_ROUND_SR_ELEMENT_CARRY>, grid, block, 0, s, x, (int)rows, H, o, sr_state);
  } else if (round_mode == EP_ROUND_SR_STREAM_CARRY) {
    hipLaunchKernelGGL(k_nvfp4_pack_sr<EP_ROUND_SR_STREAM_CARRY>, grid, block, 0, s, x, (int)rows, H, o, sr_state);
  } else {
    launch_rne_pack<false>(x, (int)rows, H, o, nullptr, 1, 0, s);
  }
  return launch_status();
}

// Padding rows of the grouped rowwise operand (from off_e + count_e to
// off_{e+1}) are zero bytes, as the direct receive leaves them: one
// workgroup per expert.
__global__ __launch_bounds__(256) void k_zero_padding(const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ offsets, int r_cap, int H,
                                                      uint8_t* __restrict__ row_codes, uint8_t* __restrict__ row_scales,
                                                      float* __restrict__ row_t) {
  const int e = blockIdx.x;
  const int o0 = min(max(offsets[e], 0), r_cap), o1 = min(max(offsets[e + 1], o0), r_cap);
  const int g0 = min(o0 + max(counts[e], 0), o1);
  const int cw = H >> 3, sw = H >> 6;  // dwords of codes and of scales per row
  for (int g = g0; g < o1; ++g) {
    uint32_t* c = reinterpret_cast<uint32_t*>(row_codes + (size_t)g * (H >> 1));
    uint32_t* sc = reinterpret_cast<uint32_t*>(row_scales + (size_t)g * (H >> 4));
    for (int i = threadIdx.x; i < cw; i += 256) c[i] = 0u;
    for (int i = threadIdx.x; i < sw; i += 256) sc[i] = 0u;
    if (threadIdx.x == 0) row_t[g] = 0.0f;
  }
}

MTB_EXPORT int32_t ep_nvfp4_pack_scatter(const uint16_t* x, int64_t tokens, int64_t hidden, int64_t top_k,
                                         const int32_t* dst_row, int64_t num_experts, int64_t r_cap,
                                         const int32_t* counts, const int32_t* offsets, uint8_t* row_codes,
                                         uint8_t* row_scales, float* row_t, void* stream) {
  if (tokens < 0 || hidden <= 0 || hidden % 64 != 0 || hidden > 16384 || top_k < 1 || num_experts < 1 ||
      num_experts > 1024 || r_cap < 0)
    return EP_ERR_SHAPE;
  if (top_k > kMaxScatter) return EP_ERR_RANGE;
  if (tokens > (int64_t)INT32_MAX / 4 || tokens * hidden >= ((int64_t)1 << 40) || r_cap >= INT32_MAX / 4)
    return EP_ERR_RANGE;
  if (!counts || !offsets) return EP_ERR_NULL;
  if (r_cap > 0 && (!row_codes || !row_scales || !row_t)) return EP_ERR_NULL;
  if (tokens > 0 && (!x || !dst_row)) return EP_ERR_NULL;
  const int H = (int)hidden;
  hipStream_t s = (hipStream_t)stream;
  const RowOut o{row_codes, row_scales, reinterpret_cast<uint8_t*>(row_t), (uint32_t)(H / 2), (uint32_t)(H / 16), 4u};
  if (tokens > 0 && r_cap > 0) launch_rne_pack<true>(x, (int)tokens, H, o, dst_row, (int)top_k, (int)r_cap, s);
  if (r_cap > 0)
    hipLaunchKernelGGL(k_zero_padding, dim3((unsigned)num_experts), dim3(256), 0, s, counts, offsets, (int)r_cap, H,
                       row_codes, row_scales, row_t);
  return launch_status();
}

MTB_EXPORT int32_t ep_mxfp8_pack(const uint16_t* x, int64_t rows, int64_t hidden, uint8_t* data,
                                 uint8_t* scales, void* stream) {
  if (rows < 0 || hidden <= 0 || hidden % 32 != 0) return EP_ERR_SHAPE;
  if (rows > (((int64_t)1 << 40) - 1) / hidden) return EP_ERR_RANGE;   // rows * hidden >= 2^40
  if (rows == 0) return EP_OK;
  if (!x || !data || !scales) return EP_ERR_NULL;
  int64_t chunks = rows * hidden / 16;
  dim3 grid((unsigned)((chunks + 255) / 256)), block(256);
  hipLaunchKernelGGL(k_mxfp8_pack, grid, block, 0, (hipStream_t)stream, x, chunks, (int)hidden, data, scales);
  return launch_status();
}
