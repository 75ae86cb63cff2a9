// NVFP4 direct receive for gfx950 (P1, PR description: the receiving side
// produces both grouped operands of the expert GEMM from the packed rows it is
// handed -- the rowwise one by copying the sender's bytes into expert order,
// the columnwise one by decoding, applying the RHT and re-quantizing against a
// per-expert scale computed from the token scales alone, so neither a BF16
// copy of the rows nor a max pass over them is needed; P4, description: four
// times the rowwise amax bounds the RHT output).
//
// Launch 1 (k_expert_scale): D_e = 4 * max t over expert e's rows.  It reads
// only the 4-byte token scales, not the codes: no amax pass.
// Launch 2 (k_nvfp4_receive): one workgroup per 256 grouped rows x 256
// columns.  The rowwise operand is the gathered rows' bytes, stored unchanged
// in expert order; the columnwise operand is built per 16 x 16 block in one
// lane's registers (exact decode fused with the first butterfly stage, the
// other three stages, quantization against the expert's power-of-two D_e)
// and stored from there.  The kernel's own comment gives the lane mapping and
// the two load rounds.  Layouts: compact (each expert's columnwise operand one
// [H, P_e/2] code matrix) or K-blocked (the same in 256-row K-blocks).
// The MXFP4 receive (k_mxfp4_receive) has the same tiles and loads and
// re-quantizes both operands to E2M1 with power-of-two scales per 32.
// Without the columnwise operand the receive is a plain row gather
// (k_nvfp4_gather).
#include "common.h"
#include "launch.h"

namespace mtb {

constexpr int kXcds = 8;                 // CDNA4: 8 XCDs, workgroups dealt round-robin

__global__ __launch_bounds__(1024) void k_expert_scale(const uint8_t* __restrict__ packed, int T, int H, int row_bytes,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ src_row,
                                                       float* __restrict__ col_scale) {
  __shared__ uint32_t red[16];
  const int e = blockIdx.x;
  const int g0 = offsets[e], g1 = offsets[e + 1];
  const int toff = (H >> 1) + (H >> 4);
  uint32_t m = 0;  // t > 0 is a power of two: compare bit patterns
  // four rows per thread per round: the four source-row loads go out together,
  // then the four t loads (two dependent round trips per 4096 rows, not per
  // 1024).  The loads are unconditional, at indices clamped into range, so that
  // none waits behind a branch; out-of-range rows are dropped after.
  for (int g = g0 + (int)threadIdx.x; g < g1 && T > 0; g += 4 * 1024) {
    int src[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) src[q] = src_row[min(g + q * 1024, g1 - 1)];
    uint32_t tb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      tb[q] = *reinterpret_cast<const uint32_t*>(packed + (size_t)min(max(src[q], 0), T - 1) * row_bytes + toff);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (g + q * 1024 < g1 && src[q] >= 0 && src[q] < T) m = m > tb[q] ? m : tb[q];
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int i = 0; i < 16; ++i) r = r > red[i] ? r : red[i];
    col_scale[e] = 4.0f * __uint_as_float(r);  // 0 for an empty expert
  }
}

// D_e from the grouped rowwise operand: the expert's rows are contiguous, so
// this is a max over row_t[off_e .. off_{e+1}) (padding rows hold t = 0).
__global__ __launch_bounds__(1024) void k_expert_scale_grouped(const float* __restrict__ row_t, int r_cap,
                                                               const int32_t* __restrict__ offsets,
                                                               float* __restrict__ col_scale) {
  __shared__ uint32_t red[16];
  const int e = blockIdx.x;
  const int g0 = max(0, offsets[e]), g1 = min(r_cap, offsets[e + 1]);
  uint32_t m = 0;  // t >= 0: compare bit patterns
  for (int g = g0 + (int)threadIdx.x; g < g1; g += 4 * 1024) {
    uint32_t tb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) tb[q] = g + q * 1024 < g1 ? __float_as_uint(row_t[g + q * 1024]) : 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) m = m > tb[q] ? m : tb[q];
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int i = 0; i < 16; ++i) r = r > red[i] ? r : red[i];
    col_scale[e] = 4.0f * __uint_as_float(r);
  }
}

// Reciprocal split of every E4M3 block-scale code (see quot_split): entry c
// holds r_hi, r_lo of the significand of s = E4M3(c) and 2^k, s's power of
// two; code 0 (and the NaN code) hold zeros and 2^0, which quantize every
// value to a signed zero.
struct RcpEntry {
  float r_hi, r_lo, p2k;
};

__device__ __forceinline__ RcpEntry rcp_entry(int c) {
  RcpEntry r{0.0f, 0.0f, 1.0f};
  float s = e4m3_decode((uint32_t)c);
  if (c != 0 && c < 0x7F) {
    QuotSplit q = quot_split(s);
    r.r_hi = q.r_hi;
    r.r_lo = q.r_lo;
    r.p2k = pow2f(q.k);
  }
  return r;
}

// Quantizer parameters of one post-RHT column block with decode scale 2^dexp.
struct ColQuant {
  float r_hi, r_lo, scale;
  uint32_t sc;
};

__device__ __forceinline__ ColQuant col_block_quant(float amax, int dexp, const RcpEntry* tab) {
  // s = E4M3(fl32(amax / 6) / D): fl32(amax/6) is exact by div6 for normal
  // amax; tiny amax are scaled by 2^64 first (their E4M3 code is 0 unless D
  // is tiny too, and then the scaled path is the exact one).
  bool tiny = amax < 0x1p-100f;
  float a = tiny ? amax * 0x1p64f : amax;
  float y = __builtin_ldexpf(div6(a), -dexp - (tiny ? 64 : 0));
  ColQuant q;
  q.sc = e4m3_encode(fminf(y, 448.0f));
  RcpEntry r = tab[q.sc];  // a value in [0, 448]: code <= 0x7E
  // quotient by s * D = m * 2^K; for K < -104 the quotient is first scaled
  // up by 2^P (exact) so that the power handed to the converter stays normal
  int K = (int)(__float_as_uint(r.p2k) >> 23) - 127 + dexp;
  int P = max(-104 - K, 0);
  q.r_hi = __builtin_ldexpf(r.r_hi, P);
  q.r_lo = __builtin_ldexpf(r.r_lo, P);
  q.scale = q.sc ? pow2f(K + P) : 1.0f;
  return q;
}

// col_block_quant where the block's rows all have t >= 2^-88 (or t = 0) and
// 2^-95 <= D_e <= 2^119 -- the decode's fast path: a nonzero post-RHT value is
// then at least 2^-88 * 2^-9 * 2^-1 * 2^-2 = 2^-100 (decoded values are
// multiples of that, and a rounded sum is far above it), so div6 needs no
// prescale, and the power s * D_e = m * 2^K has -104 <= K <= 127, so the
// quotient needs none either and the converter's power is a normal float.
// With p2 = 2^(-2 - dexp) and pd = 2^dexp (normal floats in that range),
// fl32(amax / 1.5) * p2 is fl32(amax / 6) * 2^-dexp (the same exact scalings
// by powers of two), and the converter's power is 2^k * pd; code 0 keeps any
// normal power (its quotients are signed zeros).  The same codes as
// col_block_quant, fewer instructions.
__device__ __forceinline__ ColQuant col_block_quant_fast(float amax, float p2, float pd, const RcpEntry* tab) {
  const float y = div1_5(amax) * p2;
  ColQuant q;
  q.sc = e4m3_encode(fminf(y, 448.0f));
  const RcpEntry r = tab[q.sc];  // a value in [0, 448]: code <= 0x7E
  q.r_hi = r.r_hi;
  q.r_lo = r.r_lo;
  q.scale = r.p2k * pd;
  return q;
}

// 16 post-RHT values -> two code words (rows 0..7, rows 8..15; row 2j low nibble).
__device__ __forceinline__ void col_encode(const float* y, const ColQuant& q, uint32_t& w0, uint32_t& w1) {
  float u[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) u[i] = quot_apply(y[i], q.r_hi, q.r_lo);
  // (each word's first conversion keeps three bytes of its `old` operand that
  // the next three overwrite: any register will do)
  w0 = fp4_pack2<0>(__float_as_uint(u[0]), u[0], u[1], q.scale);
  w0 = fp4_pack2<1>(w0, u[2], u[3], q.scale);
  w0 = fp4_pack2<2>(w0, u[4], u[5], q.scale);
  w0 = fp4_pack2<3>(w0, u[6], u[7], q.scale);
  w1 = fp4_pack2<0>(__float_as_uint(u[8]), u[8], u[9], q.scale);
  w1 = fp4_pack2<1>(w1, u[10], u[11], q.scale);
  w1 = fp4_pack2<2>(w1, u[12], u[13], q.scale);
  w1 = fp4_pack2<3>(w1, u[14], u[15], q.scale);
}

__device__ __forceinline__ float absmax16(const float* y) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(y[i]));
  return m;
}

// Butterfly stages 2, 4, 8 (stage 1 is fused into the decode).
__device__ __forceinline__ void rht16_upper(float* z) {
#pragma unroll
  for (int h = 2; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      float a = z[i], b = z[i + h];
      z[i] = a + b;
      z[i + h] = a - b;
    }
  }
}

// Decode byte SEL (two columns) of the 16 code words and apply the first
// butterfly stage.  Fast blocks: the decoded value is e2m1 * c with c =
// s*t*d/4, each product exact, so stage 1's pair (i, i+1) becomes
// fma(g_i, c_i, +-g_{i+1} c_{i+1}) -- the same two roundings as adding the
// decoded values.  Slow blocks (a row with t < 2^-88, or D_e < 2^-95):
// z = ldexp(e2m1 * s*d/4, e) rounded once per row, then the plain stage.
template <int SEL, bool SLOW>
__device__ __forceinline__ void decode_stage1(const uint32_t* cw, const float* cm, const int* ce, float* z0,
                                              float* z1) {
  if (!SLOW) {
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      f32x2 g = fp4_unpack2<SEL>(cw[i], 1.0f), h = fp4_unpack2<SEL>(cw[i + 1], 1.0f);
      float b0 = h[0] * cm[i + 1], b1 = h[1] * cm[i + 1];
      z0[i] = __builtin_fmaf(g[0], cm[i], b0);
      z0[i + 1] = __builtin_fmaf(g[0], cm[i], -b0);
      z1[i] = __builtin_fmaf(g[1], cm[i], b1);
      z1[i + 1] = __builtin_fmaf(g[1], cm[i], -b1);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      f32x2 g = fp4_unpack2<SEL>(cw[i], 1.0f), h = fp4_unpack2<SEL>(cw[i + 1], 1.0f);
      float a0 = __builtin_ldexpf(g[0] * cm[i], ce[i]), a1 = __builtin_ldexpf(g[1] * cm[i], ce[i]);
      float b0 = __builtin_ldexpf(h[0] * cm[i + 1], ce[i + 1]), b1 = __builtin_ldexpf(h[1] * cm[i + 1], ce[i + 1]);
      z0[i] = a0 + b0;
      z0[i + 1] = a0 - b0;
      z1[i] = a1 + b1;
      z1[i + 1] = a1 - b1;
    }
  }
}

// Stochastic variant of col_encode: the same quotients, each code drawn by the
// carry-form converter with the Philox word of its stream position n0 + i.
// STREAM: word n of the stream is word (n & 3) of Philox block n >> 2, so the
// 16 positions take four blocks (five when n0 is not a multiple of 4; n0 mod
// 4 is the counter base's for every lane, so the block changes are uniform).
template <bool STREAM>
__device__ __forceinline__ void col_encode_sr(const float* y, const ColQuant& q, uint64_t n0, uint32_t klo,
                                              uint32_t khi, uint32_t& w0, uint32_t& w1) {
  float u[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) u[i] = quot_apply(y[i], q.r_hi, q.r_lo);
  if (!STREAM) {
    w0 = sr_codes8(u, n0, klo, khi, q.scale);
    w1 = sr_codes8(u + 8, n0 + 8, klo, khi, q.scale);
    return;
  }
  uint32_t rnd[16];
  uint64_t cur = n0 >> 2;
  U4 blk = philox4x32_10((uint32_t)cur, (uint32_t)(cur >> 32), 0u, 0u, klo, khi);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint64_t n = n0 + i;
    if ((n >> 2) != cur) {
      cur = n >> 2;
      blk = philox4x32_10((uint32_t)cur, (uint32_t)(cur >> 32), 0u, 0u, klo, khi);
    }
    const uint32_t sel = (uint32_t)n & 3u;
    rnd[i] = sel == 0 ? blk.x : (sel == 1 ? blk.y : (sel == 2 ? blk.z : blk.w));
  }
  uint32_t b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = sr_code_lo(u[2 * j], rnd[2 * j], q.scale) | sr_code_hi(u[2 * j + 1], rnd[2 * j + 1], q.scale);
  w0 = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
  w1 = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
}

// Where the kernel reads a row's codes, scales and t: the packed rows
// gathered through src_row (the direct receive), or the grouped rowwise
// operand itself (GROUPED: grouped row g is its own source).
struct RowSrc {
  const uint8_t* codes;
  const uint8_t* scales;
  const uint8_t* t;
  uint32_t cstride, sstride, tstride;  // bytes between consecutive rows
};

// ------------------------------------------------------------------ one-pass receive, 256 x 256 tiles
// One workgroup per 256 grouped rows x 256 columns (four waves):
//   * the tile's 32 KB of code bytes: thread t loads 16-byte pieces of rows
//     (t >> 3) + 32 i (eight threads per row's 128 bytes), keeps them for the
//     rowwise copy and writes them to LDS for the columnwise blocks;
//   * the rowwise operand: those pieces stored unchanged -- whole lines when H
//     is a multiple of 256, streamed past the caches (nothing in the path
//     reads them again) -- and row t's scale bytes (one 16-byte store) and t;
//   * the columnwise operand: wave w owns the 16-column groups cg = 4w .. 4w+3
//     of all sixteen 16-row blocks; lane (m, j) = (lane >> 2, lane & 3) reads
//     the 8 code bytes of column group 4w + j of the 16 rows of block m from
//     LDS, decodes them, runs the RHT and quantizes its 16 columns in
//     registers, and stores each column's 8 code bytes and scale byte
//     straight to the operand: the sixteen blocks of a column sit in one wave,
//     so every store instruction writes four columns' 128 contiguous code
//     bytes each.  In the K-blocked layout a K-block's columnwise output is
//     one contiguous, line-aligned region, and its code bytes are streamed too.
// Every byte of the tile is fetched once, by a 16-byte load: reading the
// columnwise blocks' bytes from global memory instead (sixteen 8-byte loads
// per lane, each instruction touching sixteen rows' lines) costs the memory
// pipeline about as many cycles as all the rest of the tile's loads together.
// Loads come in two rounds: each thread's source-row index (shared through
// LDS), then every byte load at once -- the row pieces, t and the scale bytes
// -- as range-checked buffer loads that read zeros for rows without a source.
// The copy is stored before the tile's second barrier, which hands the code
// bytes, row t's token scale and the tile's 16 scale bytes to the decode
// through LDS.
// 1-D grid of row_tiles * col_tiles workgroups.  Workgroup i runs on XCD
// i % 8, so the logical tile is taken from a contiguous range per XCD, column
// tile fastest: the column tiles of a row tile run on one XCD at about the
// same time and share the scale lines and token scales in its L2.
// KBLOCK: the columnwise operand in K-blocks -- each expert's grouped rows in
// blocks of 256 (the last one shorter, a multiple of 16), block kb of expert e
// an [H, len/2] code matrix at byte H*off_e/2 + 128*H*kb (scales [H, len/16]
// at H*off_e/16 + 16*H*kb).  Tiles then follow the K-blocks (never straddling
// experts), so a tile's columnwise output is one contiguous region.
// SR (the compact layout only): stochastic columnwise codes, the code of
// column h and grouped row g of expert e at stream position counter_base +
// H*off_e + h*P_e + (g - off_e) -- its index in col_codes, two per byte;
// SR = 1 takes each position's word from its own Philox block (element
// mapping), SR = 2 from the word stream (four words per block).
constexpr int kT2Rows = 256, kT2Cols = 256, kT2Threads = 256;
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
// Buffer resources: word 3 of a raw (unstrided, untyped) buffer on gfx9-family
// parts; a load at an offset beyond the resource's size returns zeros.
constexpr int kBufDword3 = 0x00020000;
constexpr uint32_t kNoRow = 0x80000000u;  // beyond every resource (sizes < 2^31)

// Tile row rt of the K-blocked layout: K-block rt of the concatenated
// per-expert K-block lists (each expert's grouped rows in blocks of kT2Rows,
// the last one shorter).  Gives its expert, K-block index within the expert,
// first grouped row and row count; false when rt is beyond the last K-block.
// s_offs holds offsets[0..E] (visible to every thread).  Each wave computes
// the same answer on its own -- an inclusive scan of the experts' K-block
// counts, 64 experts at a time, and the first expert whose running count
// passes rt -- so no barrier and no LDS scratch are needed.
__device__ __forceinline__ bool kblock_of_tile(int rt, int E, const int* s_offs, int& expert, int& kb, int& g_base,
                                               int& rows) {
  const int lane = threadIdx.x & 63;
  int before = 0;  // K-blocks of the experts of earlier chunks
  for (int c0 = 0; c0 < E; c0 += 64) {
    const int e = c0 + lane;
    const int n = e < E ? (max(s_offs[e + 1] - s_offs[e], 0) + kT2Rows - 1) / kT2Rows : 0;
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    const int total = __shfl(incl, 63, kWave);
    if (rt < before + total) {  // uniform: K-block rt belongs to an expert of this chunk
      // the first lane whose running count passes rt (empty experts never do)
      const int l = (int)__builtin_ctzll(__ballot(before + incl > rt));
      expert = c0 + l;
      kb = rt - before - __shfl(incl - n, l, kWave);
      g_base = s_offs[expert] + kb * kT2Rows;
      rows = min(kT2Rows, s_offs[expert + 1] - g_base);
      return true;
    }
    before += total;
  }
  return false;
}

template <int SEL, bool SLOW, int SR>
__device__ __forceinline__ void column_pair_out(const uint32_t* cw, const float* cm, const int* ce, int dexp,
                                                float p2, float pd, const RcpEntry* tab, uint64_t n0,
                                                uint64_t n_step, uint32_t klo, uint32_t khi, uint2& c0, uint2& c1,
                                                uint32_t& s0, uint32_t& s1) {
  float z0[16], z1[16];
  decode_stage1<SEL, SLOW>(cw, cm, ce, z0, z1);
  rht16_upper(z0);
  rht16_upper(z1);
  const ColQuant q0 = SLOW ? col_block_quant(absmax16(z0), dexp, tab) : col_block_quant_fast(absmax16(z0), p2, pd, tab);
  const ColQuant q1 = SLOW ? col_block_quant(absmax16(z1), dexp, tab) : col_block_quant_fast(absmax16(z1), p2, pd, tab);
  if (SR == 0) {
    col_encode(z0, q0, c0.x, c0.y);
    col_encode(z1, q1, c1.x, c1.y);
  } else {
    col_encode_sr<SR == 2>(z0, q0, n0, klo, khi, c0.x, c0.y);
    col_encode_sr<SR == 2>(z1, q1, n0 + n_step, klo, khi, c1.x, c1.y);
  }
  s0 = q0.sc;
  s1 = q1.sc;
}

template <bool GROUPED, bool KBLOCK, int SR = 0>
__global__ __launch_bounds__(kT2Threads) void k_nvfp4_receive(const RowSrc rs, int T, int H,
                                                              const int32_t* __restrict__ offsets, int E,
                                                              const int32_t* __restrict__ src_row, int r_cap, int n_ct,
                                                              uint8_t* __restrict__ row_codes,
                                                              uint8_t* __restrict__ row_scales,
                                                              float* __restrict__ row_t, uint8_t* __restrict__ col_codes,
                                                              uint8_t* __restrict__ col_scales,
                                                              const float* __restrict__ col_scale,
                                                              const uint64_t* __restrict__ sr_state) {
  // The tile's code bytes (256 rows x 128 bytes; row r's 16-byte piece q at
  // position q ^ ((r >> 4) & 7), so that the column phase's 8-byte reads of
  // sixteen rows 16 apart fall on different banks).  Until the tile's loads
  // return, the same bytes hold the expert offsets.
  // 40 KB in all, so that four workgroups share a CU's 160 KB.
  __shared__ __align__(16) uint8_t s_code[kT2Rows * 128];
  __shared__ RcpEntry s_tab[128];
  __shared__ float s_t[kT2Rows];
  __shared__ uint4 s_sw[kT2Rows];      // the tile's 16 scale bytes of each row
  __shared__ int s_tiny[kT2Rows / 16];  // a row of the 16-row block has 0 < t < 2^-88
  __shared__ __align__(16) int s_src[kT2Rows];  // source row of each grouped row (-1: none)
  int* const s_offs = reinterpret_cast<int*>(s_code);  // offsets[0..E]

  const int tid = threadIdx.x;
  const unsigned nb = gridDim.x, bx = blockIdx.x;
  const unsigned xq = nb / kXcds, xr = nb % kXcds, x = bx % kXcds;
  const unsigned lt = x * xq + min(x, xr) + bx / kXcds;
  const int rt = (int)(lt / (unsigned)n_ct), ct = (int)(lt % (unsigned)n_ct);
  const int col0 = ct * kT2Cols;
  const int ncols = min(kT2Cols, H - col0);  // 64, 128, 192 or 256
  int g_base = rt * kT2Rows;
  int kb = 0, tile_rows = kT2Rows, e = 0;
  for (int i = tid; i <= E; i += kT2Threads) s_offs[i] = offsets[i];
  __syncthreads();
  if (KBLOCK && !kblock_of_tile(rt, E, s_offs, e, kb, g_base, tile_rows)) return;

  const int lane = tid & 63, w = tid >> 6;
  const int m = lane >> 2;                    // 16-row block of the column phase
  const int cg = 4 * w + (lane & 3);          // 16-column group of the column phase
  const int gb = g_base + 16 * m;
  const bool col_live = 16 * cg < ncols;

  // this thread's own source-row index (issued first); the column block's
  // expert (the tile's in the K-blocked layout, else the last expert whose
  // offset is <= gb: empty experts share offsets), its offset, length and
  // decode scale; the reciprocal table into LDS.  Every read of s_offs comes
  // before the barrier that precedes the first write of the tile's code bytes.
  const int g = g_base + tid;
  int srcv = g;
  if (!GROUPED) srcv = src_row[(uint32_t)min(g, r_cap - 1)];
  if (!KBLOCK) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_offs[mid] <= gb) lo = mid; else hi = mid - 1;
    }
    e = lo;
  }
  const float d_e = col_scale[e];
  const int off = s_offs[e], len = s_offs[e + 1] - off;
  const int off_end_g = s_offs[E];
  if (tid < 128) s_tab[tid] = rcp_entry(tid);

  // The loads, in two rounds: each thread's own source-row index (into LDS, so
  // that the row pieces read theirs from there), then every byte load -- the
  // row pieces (16 bytes of rows (tid >> 3) + 32 i: the tile's whole 32 KB of
  // codes, which both the rowwise copy and the columnwise blocks use), its
  // row's t and the tile's scale bytes.  The byte loads are buffer loads over
  // the source rows: a row that is padding, an unused slot, past r_cap or out
  // of range gets an offset beyond the resource, and the hardware's range
  // check returns zeros for it -- no selects, and no access at all when T = 0.
  const int cq = tid & 7, nq = ncols >> 5;  // 16-byte pieces per row: 2, 4, 6 or 8
  s_src[tid] = g < r_cap ? srcv : -1;
  __syncthreads();
  int rsrc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) rsrc[i] = s_src[(tid >> 3) + 32 * i];
  const int src = s_src[tid];
  // resources of the T source rows (sizes < 2^31: checked at launch)
  const uint32_t nT = (uint32_t)max(T, 0);
  const __amdgpu_buffer_rsrc_t r_codes = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(rs.codes), (short)0, (int)(nT ? (nT - 1) * rs.cstride + (uint32_t)(H >> 1) : 0u), kBufDword3);
  const __amdgpu_buffer_rsrc_t r_scales = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(rs.scales), (short)0, (int)(nT ? (nT - 1) * rs.sstride + (uint32_t)(H >> 4) : 0u), kBufDword3);
  const __amdgpu_buffer_rsrc_t r_t = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(rs.t), (short)0, (int)(nT ? (nT - 1) * rs.tstride + 4u : 0u), kBufDword3);
  // byte offset of source row s (plus add), or kNoRow
  auto row_at = [&](int s, uint32_t stride, uint32_t add) -> uint32_t {
    return (uint32_t)s < nT ? __umul24((uint32_t)s, stride) + add : kNoRow;
  };
  u32x4v cv[8];
  {
    // dead pieces of a narrow tile re-read piece 0 (their bytes are never used)
    const uint32_t qa = (uint32_t)(col0 >> 1) + 16u * (uint32_t)(cq < nq ? cq : 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) cv[i] = __builtin_amdgcn_raw_buffer_load_b128(r_codes, row_at(rsrc[i], rs.cstride, qa), 0, 0);
  }
  const float t = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_t, row_at(src, rs.tstride, 0u), 0, 0));
  uint4 sw;
  {
    const uint32_t so = row_at(src, rs.sstride, (uint32_t)(col0 >> 4));
    if (ncols == kT2Cols) {
      const u32x4v q = __builtin_amdgcn_raw_buffer_load_b128(r_scales, so, 0, 0);
      sw = make_uint4(q.x, q.y, q.z, q.w);
    } else {
      const int nw = ncols >> 6;  // 1..3 dwords of scale bytes
      sw = make_uint4(__builtin_amdgcn_raw_buffer_load_b32(r_scales, so, 0, 0),
                      nw > 1 ? __builtin_amdgcn_raw_buffer_load_b32(r_scales, so + 4u, 0, 0) : 0u,
                      nw > 2 ? __builtin_amdgcn_raw_buffer_load_b32(r_scales, so + 8u, 0, 0) : 0u, 0u);
    }
  }
  const int off_end = min(off_end_g, r_cap & ~15);                       // whole 16-row blocks only
  const int tile_end = KBLOCK ? min(g_base + tile_rows, off_end) : off_end;  // rows this tile writes
  s_t[tid] = t;
  s_sw[tid] = sw;
  {
    // rows tid.. of this wave are blocks 4w .. 4w+3: one ballot gives their flags
    const uint64_t tiny = __ballot(t < 0x1p-88f && t > 0.0f);
    if ((tid & 63) < 4) s_tiny[4 * (tid >> 6) + (tid & 3)] = ((tiny >> (16 * (tid & 3))) & 0xFFFFu) != 0;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 3) + 32 * i;
    *reinterpret_cast<u32x4v*>(s_code + 128 * r + ((cq ^ ((r >> 4) & 7)) << 4)) = cv[i];
  }
  if (!GROUPED) {
    // rowwise operand: 16-byte pieces, eight threads per row's 128 code bytes
    // (whole lines when H is a multiple of 256), streamed past the caches --
    // nothing in the path reads them again; the row's scale bytes (one 16-byte
    // piece when H is a multiple of 256) and t
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int gr = g_base + (tid >> 3) + 32 * i;
      if (gr >= tile_end || cq >= nq) continue;
      __builtin_nontemporal_store(
          cv[i], reinterpret_cast<u32x4v*>(row_codes + (size_t)(uint32_t)gr * (uint32_t)(H >> 1) + (col0 >> 1) + 16 * cq));
    }
    if (g < tile_end) {
      uint32_t* rsc = reinterpret_cast<uint32_t*>(row_scales + (size_t)(uint32_t)g * (uint32_t)(H >> 4) + (col0 >> 4));
      if ((H & 255) == 0) {
        *reinterpret_cast<uint4*>(rsc) = sw;
      } else {
        rsc[0] = sw.x;
        if (ncols > 64) rsc[1] = sw.y;
        if (ncols > 128) rsc[2] = sw.z;
        if (ncols > 192) rsc[3] = sw.w;
      }
      if (ct == 0) row_t[g] = t;
    }
  }
  __syncthreads();
  if (!col_live || gb >= tile_end) return;

  // the block's decode exponent and output bases
  const int dexp = pow2_exponent(d_e);
  uint64_t cbase, sbase;
  uint32_t cstr, sstr;
  if (KBLOCK) {
    cbase = (uint64_t)H * (uint32_t)(off >> 1) + (uint64_t)H * 128u * (uint32_t)kb + 8u * (uint32_t)m;
    cstr = (uint32_t)(tile_rows >> 1);
    sbase = (uint64_t)H * (uint32_t)(off >> 4) + (uint64_t)H * 16u * (uint32_t)kb + (uint32_t)m;
    sstr = (uint32_t)(tile_rows >> 4);
  } else {
    cbase = (uint64_t)H * (uint32_t)(off >> 1) + (uint32_t)((gb - off) >> 1);
    cstr = (uint32_t)(len >> 1);
    sbase = (uint64_t)H * (uint32_t)(off >> 4) + (uint32_t)((gb - off) >> 4);
    sstr = (uint32_t)(len >> 4);
  }
  uint64_t n_col = 0, n_step = 0;
  uint32_t klo = 0, khi = 0;
  if (SR) {
    const uint64_t seed = sr_state[0];
    klo = (uint32_t)seed;
    khi = (uint32_t)(seed >> 32);
    n_col = sr_state[1] + 2 * cbase;   // the nibble index of (column 0, row gb), plus the counter base
    n_step = 2 * (uint64_t)cstr;
  }
  // decode factors of the 16 rows: c_i = s_i * t_i * d_i / 4 (exact products)
  const int h0 = col0 + 16 * cg;            // the thread's first column
  const int sh = 8 * (cg & 3);
  float cm[16], tv[16];
  uint32_t sb[16];
  const bool slow = dexp < -95 || dexp > 119 || s_tiny[m];
  const float p2 = slow ? 1.0f : pow2f(-2 - dexp), pd = slow ? 1.0f : pow2f(dexp);  // the fast quantizer's powers
  const uint32_t* swd = reinterpret_cast<const uint32_t*>(s_sw) + 4 * (16 * m) + (cg >> 2);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    tv[i] = s_t[16 * m + i];
    sb[i] = swd[4 * i] >> sh;
  }
  // the block's code bytes: 8 bytes (16 columns) of each of its 16 rows
  uint32_t wx[16], wy[16];
  {
    const uint8_t* cb = s_code + 128 * (16 * m) + ((((cg >> 1) ^ (m & 7)) << 4) + 8 * (cg & 1));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint2 v = *reinterpret_cast<const uint2*>(cb + 128 * i);
      wx[i] = v.x;
      wy[i] = v.y;
    }
  }
  uint8_t* cc = col_codes + cbase;
  uint8_t* cs = col_scales + sbase;
  uint8_t* kb_codes = col_codes;
  uint32_t kb_co = 0;
  if (KBLOCK) {
    const int off_u = __builtin_amdgcn_readfirstlane(off), kb_u = __builtin_amdgcn_readfirstlane(kb);
    kb_codes = col_codes + (uint64_t)H * (uint32_t)(off_u >> 1) + (uint64_t)H * 128u * (uint32_t)kb_u;
    kb_co = 8u * (uint32_t)m + (uint32_t)h0 * cstr;
  }
  // the K-blocked layout: a K-block's code bytes fill one contiguous region, streamed
  // A whole K-block's scale bytes: column h's sixteen at 16 h, so the wave's 64
  // columns fill one contiguous KB.  They are transposed through the wave's own
  // dword of each row of s_sw (wave w reads only dword w, and has read it) and
  // leave as one 16-byte store per lane instead of sixteen byte stores.
  const bool stage_sc = KBLOCK && tile_rows == kT2Rows && g_base + kT2Rows <= tile_end;  // uniform
  uint8_t* const s_scw = reinterpret_cast<uint8_t*>(s_sw) + 4 * w;  // byte b < 4 of row r: s_scw[16 r + b]
  auto store = [&](int c, uint2 a, uint2 b, uint32_t sa, uint32_t sb2) {
    const uint32_t h = (uint32_t)(h0 + c);
    // a K-block's region is H * 128 bytes: 32-bit offsets from its (uniform) base
    u32x2v* pa = reinterpret_cast<u32x2v*>(KBLOCK ? kb_codes + (kb_co + (uint32_t)c * cstr) : cc + (uint64_t)h * cstr);
    u32x2v* pb = reinterpret_cast<u32x2v*>(KBLOCK ? kb_codes + (kb_co + (uint32_t)(c + 1) * cstr)
                                                  : cc + (uint64_t)(h + 1) * cstr);
    if (KBLOCK) {
      __builtin_nontemporal_store(u32x2v{a.x, a.y}, pa);
      __builtin_nontemporal_store(u32x2v{b.x, b.y}, pb);
    } else {
      *pa = u32x2v{a.x, a.y};
      *pb = u32x2v{b.x, b.y};
    }
    if (stage_sc) {
      // the wave's column l = 16 j + c, block m: row 4 l + m / 4, byte m % 4
      const int l = 16 * (lane & 3) + c;
      s_scw[16 * (4 * l + (m >> 2)) + (m & 3)] = (uint8_t)sa;
      s_scw[16 * (4 * (l + 1) + (m >> 2)) + (m & 3)] = (uint8_t)sb2;
    } else {
      cs[(uint64_t)h * sstr] = (uint8_t)sa;
      cs[(uint64_t)(h + 1) * sstr] = (uint8_t)sb2;
    }
  };
  auto store_scales = [&]() {
    if (!stage_sc) return;
    const uint32_t* rd = reinterpret_cast<const uint32_t*>(s_scw + 64 * lane);  // rows 4 lane .. 4 lane + 3
    const uint4 v = make_uint4(rd[0], rd[4], rd[8], rd[12]);
    *reinterpret_cast<uint4*>(cs - m + 16u * (uint32_t)(col0 + 64 * w + lane)) = v;
  };
  if (!slow) {
#pragma unroll
    for (int i = 0; i < 16; ++i) cm[i] = e4m3_decode(sb[i]) * (tv[i] * rht_in_scale(i));  // exact
    static_for<0, 8>([&](auto P) {
      constexpr int p = P;
      uint2 a, b;
      uint32_t sa, sbb;
      const uint64_t n0 = n_col + (uint64_t)(h0 + 2 * p) * n_step;
      column_pair_out<p & 3, false, SR>((p < 4) ? wx : wy, cm, nullptr, dexp, p2, pd, s_tab, n0, n_step, klo, khi,
                                        a, b, sa, sbb);
      store(2 * p, a, b, sa, sbb);
    });
  } else {
    int ce[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ce[i] = tv[i] > 0.0f ? pow2_exponent(tv[i]) : 0;
      // t = 0 (padding): t * d_i / 4, the signed zero the fast path's factor has
      cm[i] = tv[i] == 0.0f ? tv[i] * rht_in_scale(i) : e4m3_decode(sb[i]) * rht_in_scale(i);
    }
    static_for<0, 8>([&](auto P) {
      constexpr int p = P;
      uint2 a, b;
      uint32_t sa, sbb;
      const uint64_t n0 = n_col + (uint64_t)(h0 + 2 * p) * n_step;
      column_pair_out<p & 3, true, SR>((p < 4) ? wx : wy, cm, ce, dexp, p2, pd, s_tab, n0, n_step, klo, khi, a, b,
                                       sa, sbb);
      store(2 * p, a, b, sa, sbb);
    });
  }
  store_scales();
}

// ------------------------------------------------------------------ MXFP4 receive
// The same routed rows re-quantized to MXFP4 -- E2M1 codes with one E8M0 scale
// (a power of two) per 32 elements, the operand format of gfx950's
// block-scaled matrix instructions -- rowwise along H and columnwise after the
// 16-point RHT, 32 grouped rows per columnwise block (two RHT blocks).  The
// NVFP4 decode and the RHT are exactly the NVFP4 receive's; only the final
// quantizer differs, and it needs no per-expert scale: no amax pass at all.

// Exponent of an MXFP4 block with max a >= 0: the least e with a <= 6 * 2^e
// (no element clipped), clamped to [-127, 127]; a = 0 gives 0.  For
// a = m * 2^E, m in [1, 2): e = E - 2 + [m > 1.5].
__device__ __forceinline__ int mx4_exponent(float a) {
  if (!(a > 0.0f)) return 0;
  int sub = 0;
  if (a < 0x1p-126f) { a *= 0x1p64f; sub = 64; }
  const int E = __builtin_amdgcn_frexp_expf(a) - 1 - sub;
  const float m = __builtin_amdgcn_frexp_mantf(a) * 2.0f;
  const int e = E - 2 + (m > 1.5f ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Eight values / 2^e -> one word of E2M1 codes (value 2j in the low nibble of
// byte j): the converter's rounding is an exact round-to-nearest-even of the
// quotient by its power of two.  Below 2^-126 that power is not a normal
// float, so the values are scaled by 2^64 first (exact).
__device__ __forceinline__ uint32_t mx4_word(const float* v, int e) {
  float k = 1.0f, sc;
  if (e >= -126) {
    sc = pow2f(e);
  } else {
    k = 0x1p64f;
    sc = pow2f(e + 64);
  }
  uint32_t w = fp4_pack2<0>(__float_as_uint(v[0]), v[0] * k, v[1] * k, sc);
  w = fp4_pack2<1>(w, v[2] * k, v[3] * k, sc);
  w = fp4_pack2<2>(w, v[4] * k, v[5] * k, sc);
  return fp4_pack2<3>(w, v[6] * k, v[7] * k, sc);
}

// mx4_word for e >= -126 (the power is a normal float; no prescale).
__device__ __forceinline__ uint32_t mx4_word_normal(const float* v, int e) {
  const float sc = pow2f(e);
  uint32_t w = fp4_pack2<0>(__float_as_uint(v[0]), v[0], v[1], sc);
  w = fp4_pack2<1>(w, v[2], v[3], sc);
  w = fp4_pack2<2>(w, v[4], v[5], sc);
  return fp4_pack2<3>(w, v[6], v[7], sc);
}

// One workgroup per 256 grouped rows x 256 columns, with the NVFP4 receive's
// tiles, lane mapping and two load rounds (the 16-byte row pieces, the column
// blocks' 8-byte gathers, t and the scale bytes, as range-checked buffer loads).
//   * rowwise: thread t re-quantizes the 16-byte pieces it loaded -- piece
//     t & 7 of rows (t >> 3) + 32 i, i.e. 32 codes, one MXFP4 block -- with
//     the row's t and two NVFP4 scale bytes from LDS, and stores its 16 code
//     bytes and scale byte (streamed: whole lines when H is a multiple of 256);
//   * columnwise: lane (m, j) decodes and transforms its 16 x 16 block as the
//     NVFP4 receive does; the 32-row block max joins blocks m and m ^ 1
//     (lanes 4 apart), and each column's 8 code bytes leave from registers --
//     the sixteen blocks of a column sit in one wave, so a store instruction
//     writes four columns' 128 contiguous bytes -- and each 32-row block's
//     scale byte from the even block's lane.
// Every expert's padded rows are a multiple of 32 (the host checks the
// alignment), so a 32-row block never straddles two experts; blocks m and
// m ^ 1 are both live or both dead.
// KBLOCK: the columnwise operand in 256-row K-blocks, as the NVFP4 receive's
// (block kb of expert e: an [H, len/2] code matrix at byte H*off_e/2 +
// 128*H*kb and an [H, len/32] scale matrix at byte H*off_e/32 + 8*H*kb), the
// tiles following the K-blocks; its code bytes are streamed.
template <bool KBLOCK>
__global__ __launch_bounds__(kT2Threads) void k_mxfp4_receive(const RowSrc rs, int T, int H,
                                                              const int32_t* __restrict__ offsets, int E,
                                                              const int32_t* __restrict__ src_row, int r_cap, int n_ct,
                                                              uint8_t* __restrict__ row_codes,
                                                              uint8_t* __restrict__ row_scales,
                                                              uint8_t* __restrict__ col_codes,
                                                              uint8_t* __restrict__ col_scales) {
  // the tile's code bytes (the NVFP4 receive's swizzled layout); the expert
  // offsets until the loads return
  __shared__ __align__(16) uint8_t s_code[kT2Rows * 128];
  __shared__ float s_t[kT2Rows];
  __shared__ uint4 s_sw[kT2Rows];      // the tile's 16 NVFP4 scale bytes of each row
  __shared__ int s_tiny[kT2Rows / 16];  // a row of the 16-row block has 0 < t < 2^-100
  __shared__ __align__(16) int s_src[kT2Rows];
  int* const s_offs = reinterpret_cast<int*>(s_code);

  const int tid = threadIdx.x;
  const unsigned nb = gridDim.x, bx = blockIdx.x;
  const unsigned xq = nb / kXcds, xr = nb % kXcds, x = bx % kXcds;
  const unsigned lt = x * xq + min(x, xr) + bx / kXcds;
  const int rt = (int)(lt / (unsigned)n_ct), ct = (int)(lt % (unsigned)n_ct);
  const int col0 = ct * kT2Cols;
  const int ncols = min(kT2Cols, H - col0);  // 64, 128, 192 or 256
  int g_base = rt * kT2Rows, kb = 0, tile_rows = kT2Rows, kex = 0;
  for (int i = threadIdx.x; i <= E; i += kT2Threads) s_offs[i] = offsets[i];
  __syncthreads();
  if (KBLOCK && !kblock_of_tile(rt, E, s_offs, kex, kb, g_base, tile_rows)) return;

  const int lane = tid & 63, w = tid >> 6;
  const int m = lane >> 2;                    // 16-row block of the column phase
  const int cg = 4 * w + (lane & 3);          // 16-column group of the column phase
  const int gb = g_base + 16 * m;
  const bool col_live = 16 * cg < ncols;

  const int g = g_base + tid;
  const int srcv = src_row[(uint32_t)min(g, r_cap - 1)];
  // the column block's expert offset and length (the tile's expert in the
  // K-blocked layout), read before the barrier that precedes the code bytes'
  // writes into the same LDS
  int off, len;
  if (KBLOCK) {
    off = s_offs[kex];
    len = s_offs[kex + 1] - off;
  } else {
    int lo = 0, hi = E - 1;  // last expert with offsets[e] <= gb (empty experts share offsets)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_offs[mid] <= gb) lo = mid; else hi = mid - 1;
    }
    off = s_offs[lo];
    len = s_offs[lo + 1] - off;
  }
  const int off_end = min(s_offs[E], r_cap & ~31);  // whole 32-row blocks inside the outputs
  const int cq = tid & 7, nq = ncols >> 5;  // 16-byte pieces (32 columns) per row: 2, 4, 6 or 8
  s_src[tid] = g < r_cap ? srcv : -1;
  __syncthreads();
  const int tile_end = KBLOCK ? min(g_base + tile_rows, off_end) : off_end;  // rows this tile writes
  int rsrc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) rsrc[i] = s_src[(tid >> 3) + 32 * i];
  const int src = s_src[tid];
  const uint32_t nT = (uint32_t)max(T, 0);
  const __amdgpu_buffer_rsrc_t r_codes = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(rs.codes), (short)0, (int)(nT ? (nT - 1) * rs.cstride + (uint32_t)(H >> 1) : 0u), kBufDword3);
  const __amdgpu_buffer_rsrc_t r_scales = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(rs.scales), (short)0, (int)(nT ? (nT - 1) * rs.sstride + (uint32_t)(H >> 4) : 0u), kBufDword3);
  const __amdgpu_buffer_rsrc_t r_t = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(rs.t), (short)0, (int)(nT ? (nT - 1) * rs.tstride + 4u : 0u), kBufDword3);
  auto row_at = [&](int s, uint32_t stride, uint32_t add) -> uint32_t {
    return (uint32_t)s < nT ? __umul24((uint32_t)s, stride) + add : kNoRow;
  };
  u32x4v cv[8];
  {
    const uint32_t qa = (uint32_t)(col0 >> 1) + 16u * (uint32_t)(cq < nq ? cq : 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) cv[i] = __builtin_amdgcn_raw_buffer_load_b128(r_codes, row_at(rsrc[i], rs.cstride, qa), 0, 0);
  }
  const float t = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_t, row_at(src, rs.tstride, 0u), 0, 0));
  uint4 sw;
  {
    // a 16-byte load past the resource's end reads zeros for the dwords beyond it
    const u32x4v q = __builtin_amdgcn_raw_buffer_load_b128(r_scales, row_at(src, rs.sstride, (uint32_t)(col0 >> 4)), 0, 0);
    sw = make_uint4(q.x, q.y, q.z, q.w);
  }
  s_t[tid] = t;
  s_sw[tid] = sw;
  {
    const uint64_t tiny = __ballot(t < 0x1p-100f && t > 0.0f);  // a block with a tiny t: two-step decode
    if (lane < 4) s_tiny[4 * w + lane] = ((tiny >> (16 * lane)) & 0xFFFFu) != 0;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 3) + 32 * i;
    *reinterpret_cast<u32x4v*>(s_code + 128 * r + ((cq ^ ((r >> 4) & 7)) << 4)) = cv[i];
  }
  __syncthreads();

  // rowwise: each of the thread's eight pieces is one 32-column block of a row
#pragma unroll 1
  for (int i = 0; i < 8; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const int gr = g_base + r;
    const float tr = s_t[r];
    const uint32_t sb2 = reinterpret_cast<const uint16_t*>(&s_sw[r])[cq];  // scale bytes 2cq, 2cq+1
    const float st0 = e4m3_decode(sb2) * tr, st1 = e4m3_decode(sb2 >> 8) * tr;
    const uint32_t cw4[4] = {cv[i].x, cv[i].y, cv[i].z, cv[i].w};
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float st = q < 2 ? st0 : st1;
      f32x2 u;
      u = fp4_unpack2<0>(cw4[q], 1.0f); v[8 * q + 0] = u[0] * st; v[8 * q + 1] = u[1] * st;
      u = fp4_unpack2<1>(cw4[q], 1.0f); v[8 * q + 2] = u[0] * st; v[8 * q + 3] = u[1] * st;
      u = fp4_unpack2<2>(cw4[q], 1.0f); v[8 * q + 4] = u[0] * st; v[8 * q + 5] = u[1] * st;
      u = fp4_unpack2<3>(cw4[q], 1.0f); v[8 * q + 6] = u[0] * st; v[8 * q + 7] = u[1] * st;
    }
    float a = 0.0f;
#pragma unroll
    for (int q = 0; q < 32; ++q) a = fmaxf(a, fabsf(v[q]));
    const int e = mx4_exponent(a);
    u32x4v out;
    if (__ballot(e < -126) == 0) {  // every lane's power is a normal float (uniform branch)
      out = u32x4v{mx4_word_normal(v, e), mx4_word_normal(v + 8, e), mx4_word_normal(v + 16, e),
                   mx4_word_normal(v + 24, e)};
    } else {
      out = u32x4v{mx4_word(v, e), mx4_word(v + 8, e), mx4_word(v + 16, e), mx4_word(v + 24, e)};
    }
    if (gr >= tile_end || cq >= nq) continue;
    __builtin_nontemporal_store(
        out, reinterpret_cast<u32x4v*>(row_codes + (size_t)(uint32_t)gr * (uint32_t)(H >> 1) + (col0 >> 1) + 16 * cq));
    row_scales[(size_t)(uint32_t)gr * (uint32_t)(H >> 5) + (uint32_t)((col0 >> 5) + cq)] = (uint8_t)(e + 127);
  }

  if (!col_live || gb >= tile_end) return;  // the partner block m ^ 1 returns with it
  uint8_t* cc;
  uint8_t* cs;
  uint32_t cstr, sstr;
  if (KBLOCK) {
    cc = col_codes + (uint64_t)H * (uint32_t)(off >> 1) + (uint64_t)H * 128u * (uint32_t)kb + 8u * (uint32_t)m;
    cs = col_scales + (uint64_t)H * (uint32_t)(off >> 5) + (uint64_t)H * 8u * (uint32_t)kb + (uint32_t)(m >> 1);
    cstr = (uint32_t)(tile_rows >> 1);
    sstr = (uint32_t)(tile_rows >> 5);
  } else {
    cc = col_codes + (uint64_t)H * (uint32_t)(off >> 1) + (uint32_t)((gb - off) >> 1);
    cs = col_scales + (uint64_t)H * (uint32_t)(off >> 5) + (uint32_t)((gb - off) >> 5);
    cstr = (uint32_t)(len >> 1);
    sstr = (uint32_t)(len >> 5);
  }
  const int h0 = col0 + 16 * cg;
  const int sh = 8 * (cg & 3);
  // the decode path is chosen per 32-row block, so that blocks m and m ^ 1 take
  // the same branch and the lane exchange of their maxima sees both lanes
  // (the two-step decode is exact for any t)
  const bool slow = (s_tiny[m] | s_tiny[m ^ 1]) != 0;
  float tv[16];
  uint32_t sb[16];
  const uint32_t* swd = reinterpret_cast<const uint32_t*>(s_sw) + 4 * (16 * m) + (cg >> 2);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    tv[i] = s_t[16 * m + i];
    sb[i] = swd[4 * i] >> sh;
  }
  uint32_t wx[16], wy[16];  // 8 code bytes (16 columns) of each of the block's 16 rows
  {
    const uint8_t* cb = s_code + 128 * (16 * m) + ((((cg >> 1) ^ (m & 7)) << 4) + 8 * (cg & 1));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint2 v = *reinterpret_cast<const uint2*>(cb + 128 * i);
      wx[i] = v.x;
      wy[i] = v.y;
    }
  }
  // one column pair: decode + RHT, the 32-row block max with block m ^ 1 (lane
  // ^ 4), codes and scale bytes
  auto pair_out = [&](auto P, const float* cm, const int* ce) {
    constexpr int p = decltype(P)::value;
    float z0[16], z1[16];
    if (ce == nullptr) decode_stage1<p & 3, false>((p < 4) ? wx : wy, cm, nullptr, z0, z1);
    else decode_stage1<p & 3, true>((p < 4) ? wx : wy, cm, ce, z0, z1);
    rht16_upper(z0);
    rht16_upper(z1);
    float a0 = absmax16(z0), a1 = absmax16(z1);
    a0 = fmaxf(a0, __shfl_xor(a0, 4, kWave));
    a1 = fmaxf(a1, __shfl_xor(a1, 4, kWave));
    const int e0 = mx4_exponent(a0), e1 = mx4_exponent(a1);
    const uint32_t h = (uint32_t)(h0 + 2 * p);
    u32x2v q0, q1;
    if (__ballot(min(e0, e1) < -126) == 0) {  // uniform branch, as in the rowwise phase
      q0 = u32x2v{mx4_word_normal(z0, e0), mx4_word_normal(z0 + 8, e0)};
      q1 = u32x2v{mx4_word_normal(z1, e1), mx4_word_normal(z1 + 8, e1)};
    } else {
      q0 = u32x2v{mx4_word(z0, e0), mx4_word(z0 + 8, e0)};
      q1 = u32x2v{mx4_word(z1, e1), mx4_word(z1 + 8, e1)};
    }
    u32x2v* const pa = reinterpret_cast<u32x2v*>(cc + (uint64_t)h * cstr);
    u32x2v* const pb = reinterpret_cast<u32x2v*>(cc + (uint64_t)(h + 1) * cstr);
    if (KBLOCK) {  // a K-block's code bytes fill one contiguous region: streamed
      __builtin_nontemporal_store(q0, pa);
      __builtin_nontemporal_store(q1, pb);
    } else {
      *pa = q0;
      *pb = q1;
    }
    if ((m & 1) == 0) {
      cs[(uint64_t)h * sstr] = (uint8_t)(e0 + 127);
      cs[(uint64_t)(h + 1) * sstr] = (uint8_t)(e1 + 127);
    }
  };
  float cm[16];
  if (!slow) {
    // s * t * d_i / 4: exact (s has 4 significant bits, t/4 is a power of two)
#pragma unroll
    for (int i = 0; i < 16; ++i) cm[i] = e4m3_decode(sb[i]) * (tv[i] * rht_in_scale(i));
    static_for<0, 8>([&](auto P) { pair_out(P, cm, nullptr); });
  } else {
    // a row with t < 2^-100: s * d_i / 4, and t applied per row
    int ce[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ce[i] = tv[i] > 0.0f ? pow2_exponent(tv[i]) : 0;
      // t = 0 (padding): t * d_i / 4, the signed zero the fast path's factor has
      cm[i] = tv[i] == 0.0f ? tv[i] * rht_in_scale(i) : e4m3_decode(sb[i]) * rht_in_scale(i);
    }
    static_for<0, 8>([&](auto P) { pair_out(P, cm, ce); });
  }
}

// Rowwise-only receive: a plain gather of whole packed rows (codes, scales
// and t), one wave per grouped row; rows below off_E with no source are zero.
__global__ __launch_bounds__(256) void k_nvfp4_gather(const uint8_t* __restrict__ packed, int T, int H, int row_bytes,
                                                      const int32_t* __restrict__ offsets, int E,
                                                      const int32_t* __restrict__ src_row, int r_cap,
                                                      uint8_t* __restrict__ row_codes, uint8_t* __restrict__ row_scales,
                                                      float* __restrict__ row_t) {
  const int lane = threadIdx.x & 63;
  const int g = (int)(blockIdx.x * 4u + (threadIdx.x >> 6));
  if (g >= r_cap || g >= offsets[E]) return;
  int src = src_row[g];
  if (src >= T) src = -1;
  const int cb = H >> 1, sb = H >> 4;  // code and scale bytes of a row (multiples of 32 and 4)
  uint8_t* rc = row_codes + (size_t)g * cb;
  uint8_t* rs = row_scales + (size_t)g * sb;
  if (src < 0) {
    for (int i = lane; i < cb / 16; i += 64) reinterpret_cast<uint4*>(rc)[i] = make_uint4(0, 0, 0, 0);
    for (int i = lane; i < sb / 4; i += 64) reinterpret_cast<uint32_t*>(rs)[i] = 0u;
    if (lane == 0) row_t[g] = 0.0f;
    return;
  }
  const uint8_t* prow = packed + (size_t)src * row_bytes;
  // codes start 4-byte aligned only (row_bytes = 9H/16 + 4): dword loads, 16-byte stores
  for (int i = lane; i < cb / 16; i += 64) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(prow + 16 * i);
    reinterpret_cast<uint4*>(rc)[i] = make_uint4(p[0], p[1], p[2], p[3]);
  }
  for (int i = lane; i < sb / 4; i += 64)
    reinterpret_cast<uint32_t*>(rs)[i] = reinterpret_cast<const uint32_t*>(prow + cb)[i];
  if (lane == 0) row_t[g] = *reinterpret_cast<const float*>(prow + cb + sb);
}

}  // namespace mtb

using namespace mtb;

// The receive kernels address source rows through buffer resources, by a 24-bit
// row index times the row stride, with 2^31 as the "no row" offset: fewer than
// 2^24 rows of fewer than 2^31 bytes in all.
static bool rows_addressable(int64_t rows, int64_t row_bytes) {
  return rows < ((int64_t)1 << 24) && rows * row_bytes < ((int64_t)1 << 31);
}

static int32_t receive_check(const uint8_t* packed, int64_t tokens, int64_t hidden, int64_t num_experts,
                             int64_t r_cap, const int32_t* offsets, const int32_t* src_row) {
  if (tokens < 0 || r_cap < 0 || num_experts < 1 || num_experts > 1024 || hidden <= 0 || hidden % 64 != 0)
    return EP_ERR_SHAPE;
  if (tokens >= INT32_MAX / 4 || r_cap >= INT32_MAX / 4 || hidden > (1 << 20)) return EP_ERR_RANGE;
  if (!rows_addressable(tokens, 9 * hidden / 16 + 4)) return EP_ERR_RANGE;
  if (!offsets || !src_row) return EP_ERR_NULL;
  if (tokens > 0 && !packed) return EP_ERR_NULL;
  return EP_OK;
}

MTB_EXPORT int32_t ep_nvfp4_expert_scale(const uint8_t* packed, int64_t tokens, int64_t hidden, int64_t num_experts,
                                         int64_t r_cap, const int32_t* offsets, const int32_t* src_row,
                                         float* col_scale, void* stream) {
  int32_t st = receive_check(packed, tokens, hidden, num_experts, r_cap, offsets, src_row);
  if (st != EP_OK) return st;
  if (!col_scale) return EP_ERR_NULL;
  const int H = (int)hidden;
  hipLaunchKernelGGL(k_expert_scale, dim3((unsigned)num_experts), dim3(1024), 0, (hipStream_t)stream, packed,
                     (int)tokens, H, 9 * H / 16 + 4, offsets, src_row, col_scale);
  return launch_status();
}

MTB_EXPORT int32_t ep_nvfp4_direct_receive_scaled(const uint8_t* packed, int64_t tokens, int64_t hidden,
                                                  int64_t num_experts, int64_t r_cap, const int32_t* offsets,
                                                  const int32_t* src_row, uint8_t* row_codes, uint8_t* row_scales,
                                                  float* row_t, uint8_t* col_codes, uint8_t* col_scales,
                                                  const float* col_scale, void* stream) {
  int32_t st = receive_check(packed, tokens, hidden, num_experts, r_cap, offsets, src_row);
  if (st != EP_OK) return st;
  if (!row_codes || !row_scales || !row_t || !col_codes || !col_scales || !col_scale) return EP_ERR_NULL;
  if (r_cap == 0) return EP_OK;
  const int H = (int)hidden;
  const int64_t n_rt = (r_cap + kT2Rows - 1) / kT2Rows, n_ct = (H + kT2Cols - 1) / kT2Cols;
  if (n_rt * n_ct * kT2Threads >= ((int64_t)1 << 32)) return EP_ERR_RANGE;  // one 1-D grid
  const uint32_t rb = (uint32_t)(9 * H / 16 + 4);
  const RowSrc src{packed, packed + (H >> 1), packed + (H >> 1) + (H >> 4), rb, rb, rb};
  hipLaunchKernelGGL((k_nvfp4_receive<false, false>), dim3((unsigned)(n_rt * n_ct)), dim3(kT2Threads), 0, (hipStream_t)stream, src,
                     (int)tokens, H, offsets, (int)num_experts, src_row, (int)r_cap, (int)n_ct, row_codes, row_scales,
                     row_t, col_codes, col_scales, col_scale, nullptr);
  return launch_status();
}

MTB_EXPORT int32_t ep_nvfp4_direct_receive_sr(const uint8_t* packed, int64_t tokens, int64_t hidden,
                                              int64_t num_experts, int64_t r_cap, const int32_t* offsets,
                                              const int32_t* src_row, uint8_t* row_codes, uint8_t* row_scales,
                                              float* row_t, uint8_t* col_codes, uint8_t* col_scales,
                                              const float* col_scale, const uint64_t* sr_state, void* stream) {
  int32_t st = receive_check(packed, tokens, hidden, num_experts, r_cap, offsets, src_row);
  if (st != EP_OK) return st;
  if (!row_codes || !row_scales || !row_t || !col_codes || !col_scales || !col_scale || !sr_state)
    return EP_ERR_NULL;
  if (r_cap == 0) return EP_OK;
  const int H = (int)hidden;
  const int64_t n_rt = (r_cap + kT2Rows - 1) / kT2Rows, n_ct = (H + kT2Cols - 1) / kT2Cols;
  if (n_rt * n_ct * kT2Threads >= ((int64_t)1 << 32)) return EP_ERR_RANGE;  // one 1-D grid
  const uint32_t rb = (uint32_t)(9 * H / 16 + 4);
  const RowSrc src{packed, packed + (H >> 1), packed + (H >> 1) + (H >> 4), rb, rb, rb};
  hipLaunchKernelGGL((k_nvfp4_receive<false, false, 1>), dim3((unsigned)(n_rt * n_ct)), dim3(kT2Threads), 0,
                     (hipStream_t)stream, src, (int)tokens, H, offsets, (int)num_experts, src_row, (int)r_cap, (int)n_ct,
                     row_codes, row_scales, row_t, col_codes, col_scales, col_scale, sr_state);
  return launch_status();
}

MTB_EXPORT int32_t ep_nvfp4_direct_receive_sr_stream(const uint8_t* packed, int64_t tokens, int64_t hidden,
                                                     int64_t num_experts, int64_t r_cap, const int32_t* offsets,
                                                     const int32_t* src_row, uint8_t* row_codes, uint8_t* row_scales,
                                                     float* row_t, uint8_t* col_codes, uint8_t* col_scales,
                                                     const float* col_scale, const uint64_t* sr_state, void* stream) {
  int32_t st = receive_check(packed, tokens, hidden, num_experts, r_cap, offsets, src_row);
  if (st != EP_OK) return st;
  if (!row_codes || !row_scales || !row_t || !col_codes || !col_scales || !col_scale || !sr_state)
    return EP_ERR_NULL;
  if (r_cap == 0) return EP_OK;
  const int H = (int)hidden;
  const int64_t n_rt = (r_cap + kT2Rows - 1) / kT2Rows, n_ct = (H + kT2Cols - 1) / kT2Cols;
  if (n_rt * n_ct * kT2Threads >= ((int64_t)1 << 32)) return EP_ERR_RANGE;  // one 1-D grid
  const uint32_t rb = (uint32_t)(9 * H / 16 + 4);
  const RowSrc src{packed, packed + (H >> 1), packed + (H >> 1) + (H >> 4), rb, rb, rb};
  hipLaunchKernelGGL((k_nvfp4_receive<false, false, 2>), dim3((unsigned)(n_rt * n_ct)), dim3(kT2Threads), 0,
                     (hipStream_t)stream, src, (int)tokens, H, offsets, (int)num_experts, src_row, (int)r_cap, (int)n_ct,
                     row_codes, row_scales, row_t, col_codes, col_scales, col_scale, sr_state);
  return launch_status();
}

MTB_EXPORT int32_t ep_nvfp4_direct_receive(const uint8_t* packed, int64_t tokens, int64_t hidden, int64_t num_experts,
                                           int64_t r_cap, const int32_t* offsets, const int32_t* src_row,
                                           uint8_t* row_codes, uint8_t* row_scales, float* row_t,
                                           uint8_t* col_codes, uint8_t* col_scales, float* col_scale, void* stream) {
  int32_t st = receive_check(packed, tokens, hidden, num_experts, r_cap, offsets, src_row);
  if (st != EP_OK) return st;
  if (!row_codes || !row_scales || !row_t) return EP_ERR_NULL;
  const bool col = col_codes != nullptr;
  if (col && (!col_scales || !col_scale)) return EP_ERR_NULL;
  if (r_cap == 0) return col ? ep_nvfp4_expert_scale(packed, tokens, hidden, num_experts, r_cap, offsets, src_row,
                                                       col_scale, stream) : EP_OK;
  if (col) {
    st = ep_nvfp4_expert_scale(packed, tokens, hidden, num_experts, r_cap, offsets, src_row, col_scale, stream);
    if (st != EP_OK) return st;
    return ep_nvfp4_direct_receive_scaled(packed, tokens, hidden, num_experts, r_cap, offsets, src_row, row_codes,
                                          row_scales, row_t, col_codes, col_scales, col_scale, stream);
  }
  const int H = (int)hidden;
  hipLaunchKernelGGL(k_nvfp4_gather, dim3((unsigned)((r_cap + 3) / 4)), dim3(256), 0, (hipStream_t)stream, packed,
                     (int)tokens, H, 9 * H / 16 + 4, offsets, (int)num_experts, src_row, (int)r_cap, row_codes,
                     row_scales, row_t);
  return launch_status();
}

MTB_EXPORT int32_t ep_nvfp4_columnwise_grouped(const uint8_t* row_codes, const uint8_t* row_scales, const float* row_t,
                                               int64_t hidden, int64_t num_experts, int64_t r_cap,
                                               const int32_t* offsets, uint8_t* col_codes, uint8_t* col_scales,
                                               float* col_scale, void* stream) {
  if (r_cap < 0 || num_experts < 1 || num_experts > 1024 || hidden <= 0 || hidden % 64 != 0) return EP_ERR_SHAPE;
  if (r_cap >= INT32_MAX / 4 || hidden > (1 << 20) || !rows_addressable(r_cap, hidden / 2)) return EP_ERR_RANGE;
  if (!offsets || !col_scale) return EP_ERR_NULL;
  if (r_cap > 0 && (!row_codes || !row_scales || !row_t || !col_codes || !col_scales)) return EP_ERR_NULL;
  const int H = (int)hidden;
  hipLaunchKernelGGL(k_expert_scale_grouped, dim3((unsigned)num_experts), dim3(1024), 0, (hipStream_t)stream, row_t,
                     (int)r_cap, offsets, col_scale);
  if (r_cap == 0) return launch_status();
  const int64_t n_rt = (r_cap + kT2Rows - 1) / kT2Rows, n_ct = (H + kT2Cols - 1) / kT2Cols;
  if (n_rt * n_ct * kT2Threads >= ((int64_t)1 << 32)) return EP_ERR_RANGE;  // one 1-D grid
  const RowSrc src{row_codes, row_scales, reinterpret_cast<const uint8_t*>(row_t), (uint32_t)(H / 2),
                   (uint32_t)(H / 16), 4u};
  hipLaunchKernelGGL((k_nvfp4_receive<true, false>), dim3((unsigned)(n_rt * n_ct)), dim3(kT2Threads), 0, (hipStream_t)stream, src,
                     (int)r_cap, H, offsets, (int)num_experts, nullptr, (int)r_cap, (int)n_ct, nullptr, nullptr, nullptr,
                     col_codes, col_scales, col_scale, nullptr);
  return launch_status();
}

MTB_EXPORT int32_t ep_nvfp4_direct_receive_kblock(const uint8_t* packed, int64_t tokens, int64_t hidden,
                                                  int64_t num_experts, int64_t r_cap, const int32_t* offsets,
                                                  const int32_t* src_row, uint8_t* row_codes, uint8_t* row_scales,
                                                  float* row_t, uint8_t* col_codes, uint8_t* col_scales,
                                                  const float* col_scale, void* stream) {
  int32_t st = receive_check(packed, tokens, hidden, num_experts, r_cap, offsets, src_row);
  if (st != EP_OK) return st;
  if (!row_codes || !row_scales || !row_t || !col_codes || !col_scales || !col_scale) return EP_ERR_NULL;
  if (r_cap == 0) return EP_OK;
  const int H = (int)hidden;
  // K-blocks over all experts: at most r_cap/256 + E of them
  const int64_t n_kb = (r_cap + kT2Rows - 1) / kT2Rows + num_experts, n_ct = (H + kT2Cols - 1) / kT2Cols;
  if (n_kb * n_ct * kT2Threads >= ((int64_t)1 << 32)) return EP_ERR_RANGE;  // one 1-D grid
  const uint32_t rb = (uint32_t)(9 * H / 16 + 4);
  const RowSrc src{packed, packed + (H >> 1), packed + (H >> 1) + (H >> 4), rb, rb, rb};
  hipLaunchKernelGGL((k_nvfp4_receive<false, true>), dim3((unsigned)(n_kb * n_ct)), dim3(kT2Threads), 0,
                     (hipStream_t)stream, src, (int)tokens, H, offsets, (int)num_experts, src_row, (int)r_cap, (int)n_ct,
                     row_codes, row_scales, row_t, col_codes, col_scales, col_scale, nullptr);
  return launch_status();
}

MTB_EXPORT int32_t ep_mxfp4_direct_receive(const uint8_t* packed, int64_t tokens, int64_t hidden, int64_t num_experts,
                                           int64_t alignment, int64_t r_cap, const int32_t* offsets,
                                           const int32_t* src_row, uint8_t* row_codes, uint8_t* row_scales,
                                           uint8_t* col_codes, uint8_t* col_scales, void* stream) {
  int32_t st = receive_check(packed, tokens, hidden, num_experts, r_cap, offsets, src_row);
  if (st != EP_OK) return st;
  if (alignment < 32 || alignment % 32 != 0) return EP_ERR_ALIGN;
  if (!row_codes || !row_scales || !col_codes || !col_scales) return EP_ERR_NULL;
  if (r_cap == 0) return EP_OK;
  const int H = (int)hidden;
  const int64_t n_rt = (r_cap + kT2Rows - 1) / kT2Rows, n_ct = (H + kT2Cols - 1) / kT2Cols;
  if (n_rt * n_ct * kT2Threads >= ((int64_t)1 << 32)) return EP_ERR_RANGE;  // one 1-D grid
  const uint32_t rb = (uint32_t)(9 * H / 16 + 4);
  const RowSrc src{packed, packed + (H >> 1), packed + (H >> 1) + (H >> 4), rb, rb, rb};
  hipLaunchKernelGGL(k_mxfp4_receive<false>, dim3((unsigned)(n_rt * n_ct)), dim3(kT2Threads), 0, (hipStream_t)stream, src,
                     (int)tokens, H, offsets, (int)num_experts, src_row, (int)r_cap, (int)n_ct, row_codes, row_scales,
                     col_codes, col_scales);
  return launch_status();
}

MTB_EXPORT int32_t ep_mxfp4_direct_receive_kblock(const uint8_t* packed, int64_t tokens, int64_t hidden,
                                                  int64_t num_experts, int64_t alignment, int64_t r_cap,
                                                  const int32_t* offsets, const int32_t* src_row, uint8_t* row_codes,
                                                  uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales,
                                                  void* stream) {
  int32_t st = receive_check(packed, tokens, hidden, num_experts, r_cap, offsets, src_row);
  if (st != EP_OK) return st;
  if (alignment < 32 || alignment % 32 != 0) return EP_ERR_ALIGN;
  if (!row_codes || !row_scales || !col_codes || !col_scales) return EP_ERR_NULL;
  if (r_cap == 0) return EP_OK;
  const int H = (int)hidden;
  // K-blocks over all experts: at most r_cap/256 + E of them
  const int64_t n_kb = (r_cap + kT2Rows - 1) / kT2Rows + num_experts, n_ct = (H + kT2Cols - 1) / kT2Cols;
  if (n_kb * n_ct * kT2Threads >= ((int64_t)1 << 32)) return EP_ERR_RANGE;  // one 1-D grid
  const uint32_t rb = (uint32_t)(9 * H / 16 + 4);
  const RowSrc src{packed, packed + (H >> 1), packed + (H >> 1) + (H >> 4), rb, rb, rb};
  hipLaunchKernelGGL(k_mxfp4_receive<true>, dim3((unsigned)(n_kb * n_ct)), dim3(kT2Threads), 0, (hipStream_t)stream,
                     src, (int)tokens, H, offsets, (int)num_experts, src_row, (int)r_cap, (int)n_ct, row_codes,
                     row_scales, col_codes, col_scales);
  return launch_status();
}

MTB_EXPORT size_t ep_receive_workspace_bytes(int64_t tokens, int64_t top_k, int64_t num_experts) {
  return ep_route_workspace_bytes(tokens, top_k, num_experts);
}

// The receive from the top-k indices in one call: the routing plan, then D_e
// and the grouped operands.  Every argument of both halves is checked before
// the first launch.
MTB_EXPORT int32_t ep_nvfp4_direct_receive_topk(const uint8_t* packed, int64_t tokens, int64_t hidden,
                                                const void* topk_idx, int32_t idx_dtype, int64_t top_k,
                                                int64_t num_experts, int64_t alignment, int64_t r_cap, int32_t* counts,
                                                int32_t* offsets, int32_t* dst_row, int32_t* src_row,
                                                uint8_t* row_codes, uint8_t* row_scales, float* row_t,
                                                uint8_t* col_codes, uint8_t* col_scales, float* col_scale,
                                                void* workspace, size_t workspace_bytes, int32_t* d_error,
                                                void* stream) {
  int32_t st = receive_check(packed, tokens, hidden, num_experts, r_cap, offsets, src_row);
  if (st != EP_OK) return st;
  if (!row_codes || !row_scales || !row_t) return EP_ERR_NULL;
  if (col_codes && (!col_scales || !col_scale)) return EP_ERR_NULL;
  st = ep_route_plan(topk_idx, idx_dtype, tokens, top_k, num_experts, alignment, r_cap, counts, offsets, dst_row,
                     src_row, workspace, workspace_bytes, d_error, stream);
  if (st != EP_OK) return st;
  return ep_nvfp4_direct_receive(packed, tokens, hidden, num_experts, r_cap, offsets, src_row, row_codes, row_scales,
                                 row_t, col_codes, col_scales, col_scale, stream);
}
