// NVFP4 direct receive for gfx950 (P1, PR description: the receiver builds the
// expert GEMM's grouped NVFP4 operands straight from the packed rows in one
// pass -- the rowwise operand reuses the sender's codes, the columnwise RHT
// operand is quantized with a bound-derived per-expert scale, so there is no
// BF16 round trip and no amax pass; P4, description: the post-RHT amax is
// bounded by 4x the rowwise amax).
//
// Launch 1 (k_expert_scale): D_e = 4 * max t over expert e's rows.  It reads
// only the 4-byte token scales, not the codes: no amax pass.
// Launch 2 (k_nvfp4_receive): one workgroup per 256 grouped rows x 128
// columns.  Thread (cg, m) owns columns [8cg, 8cg+8) of the tile and the
// 16-row block m:
//   * loads the 16 code dwords of its rows (gathered through src_row; a wave
//     reads 4 rows x 64 contiguous bytes per instruction) and stores them
//     unchanged to the rowwise operand;
//   * decodes them exactly (E2M1 via the converter, times s*t/4*d_i);
//   * runs the 16-point butterfly down each of its 8 columns in registers;
//   * quantizes each 16-value column block with the expert's power-of-two D_e
//     and stages 8 code bytes + 1 scale byte per column in LDS;
// then the workgroup writes the staged transposed tile with stores where 16
// consecutive threads cover one column's 128 contiguous bytes.
// Tiles are aligned to 256 global grouped rows; a tile may straddle experts
// (slots are 16-aligned), so every 16-row block looks up its own expert.
#include "common.h"
#include "launch.h"

namespace mtb {

constexpr int kTileRows = 256;
constexpr int kTileCols = 128;
constexpr int kBlocks = kTileRows / 16;  // 16-row blocks per tile

__global__ __launch_bounds__(1024) void k_expert_scale(const uint8_t* __restrict__ packed, int T, int H, int row_bytes,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ src_row,
                                                       float* __restrict__ col_scale) {
  __shared__ uint32_t red[16];
  const int e = blockIdx.x;
  const int g0 = offsets[e], g1 = offsets[e + 1];
  const int toff = (H >> 1) + (H >> 4);
  uint32_t m = 0;  // t > 0 is a power of two: compare bit patterns
  for (int g = g0 + (int)threadIdx.x; g < g1; g += 1024) {
    int src = src_row[g];
    if (src >= 0 && src < T) {
      uint32_t tb = *reinterpret_cast<const uint32_t*>(packed + (size_t)src * row_bytes + toff);
      m = m > tb ? m : tb;
    }
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

// Quantizer parameters of one post-RHT column block with decode scale 2^dexp.
struct ColQuant {
  float r_hi, r_lo, scale;
  uint32_t sc;
};

__device__ __forceinline__ ColQuant col_block_quant(float amax, int dexp) {
  // s = E4M3(fl32(amax / 6) / D): fl32(amax/6) is exact by div6 for normal
  // amax; tiny amax are scaled by 2^64 first (their E4M3 code is 0 unless D
  // is tiny too, and then the scaled path is the exact one).
  bool tiny = amax < 0x1p-100f;
  float a = tiny ? amax * 0x1p64f : amax;
  float y = __builtin_ldexpf(div6(a), -dexp - (tiny ? 64 : 0));
  ColQuant q;
  q.sc = e4m3_encode(fminf(y, 448.0f));
  float s = e4m3_decode(q.sc);
  if (s > 0.0f) {
    QuotSplit qs = quot_split(s);
    int K = qs.k + dexp;
    int P = K < -104 ? -104 - K : 0;
    q.r_hi = __builtin_ldexpf(qs.r_hi, P);
    q.r_lo = __builtin_ldexpf(qs.r_lo, P);
    q.scale = pow2f(K + P);
  } else {
    q.r_hi = 0.0f;
    q.r_lo = 0.0f;
    q.scale = 1.0f;
  }
  return q;
}

// 16 post-RHT values -> two code words (rows 0..7, rows 8..15; row 2j low nibble).
__device__ __forceinline__ void col_encode(const float* y, const ColQuant& q, uint32_t& w0, uint32_t& w1) {
  float u[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) u[i] = quot_apply(y[i], q.r_hi, q.r_lo);
  w0 = fp4_pack2<0>(0u, u[0], u[1], q.scale);
  w0 = fp4_pack2<1>(w0, u[2], u[3], q.scale);
  w0 = fp4_pack2<2>(w0, u[4], u[5], q.scale);
  w0 = fp4_pack2<3>(w0, u[6], u[7], q.scale);
  w1 = fp4_pack2<0>(0u, u[8], u[9], q.scale);
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

// Decode byte SEL (two columns) of the 16 code words into z0 (even column),
// z1 (odd column).  Fast rows: z = e2m1 * c with c = s*t*d/4 exact.  Slow
// rows (t tiny): z = ldexp(e2m1 * s*d/4, e), rounded once.
template <int SEL>
__device__ __forceinline__ void decode_pair(const uint32_t* cw, const float* cm, const int* ce, bool slow,
                                            float* z0, float* z1) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    f32x2 g = fp4_unpack2<SEL>(cw[i], 1.0f);
    if (!slow) {
      z0[i] = g[0] * cm[i];
      z1[i] = g[1] * cm[i];
    } else {
      z0[i] = __builtin_ldexpf(g[0] * cm[i], ce[i]);
      z1[i] = __builtin_ldexpf(g[1] * cm[i], ce[i]);
    }
  }
}

template <int SEL, bool COL>
__device__ __forceinline__ void column_pair(const uint32_t* cw, const float* cm, const int* ce, bool slow, int dexp,
                                            uint2* stage_codes, uint8_t* stage_sc, int col0, int m) {
  float z0[16], z1[16];
  decode_pair<SEL>(cw, cm, ce, slow, z0, z1);
  rht16_butterfly(z0);
  rht16_butterfly(z1);
  ColQuant q0 = col_block_quant(absmax16(z0), dexp);
  ColQuant q1 = col_block_quant(absmax16(z1), dexp);
  uint32_t a0, a1, b0, b1;
  col_encode(z0, q0, a0, a1);
  col_encode(z1, q1, b0, b1);
  const int c0 = col0 + 2 * SEL, c1 = c0 + 1;
  stage_codes[c0 * kBlocks + m] = make_uint2(a0, a1);
  stage_codes[c1 * kBlocks + m] = make_uint2(b0, b1);
  stage_sc[c0 * kBlocks + m] = (uint8_t)q0.sc;
  stage_sc[c1 * kBlocks + m] = (uint8_t)q1.sc;
}

template <bool COL>
__global__ __launch_bounds__(256) void k_nvfp4_receive(const uint8_t* __restrict__ packed, int T, int H, int row_bytes,
                                                       const int32_t* __restrict__ offsets, int E,
                                                       const int32_t* __restrict__ src_row, int r_cap,
                                                       uint8_t* __restrict__ row_codes, uint8_t* __restrict__ row_scales,
                                                       float* __restrict__ row_t, uint8_t* __restrict__ col_codes,
                                                       uint8_t* __restrict__ col_scales,
                                                       const float* __restrict__ col_scale) {
  __shared__ uint2 stage_codes[kTileCols * kBlocks];   // [column][block] 8 bytes
  __shared__ uint8_t stage_sc[kTileCols * kBlocks];    // [column][block]
  __shared__ int s_src[kTileRows];
  __shared__ float s_t[kTileRows];
  __shared__ uint32_t s_sw[kTileRows][2];              // the tile's 8 scale bytes of each row
  __shared__ int s_bexp[kBlocks];                      // expert of each 16-row block (-1: beyond off_E)
  __shared__ int s_off[kBlocks], s_len[kBlocks], s_dexp[kBlocks];

  const int tid = threadIdx.x;
  const int ct = blockIdx.x;                 // column tile
  const int g_base = blockIdx.y * kTileRows;  // first grouped row of the tile
  const int col0 = ct * kTileCols;
  const int ncols = min(kTileCols, H - col0);
  const int off_end = offsets[E];
  const int toff = (H >> 1) + (H >> 4);

  if (tid < kBlocks) {
    int g = g_base + 16 * tid;
    int e = -1;
    if (g < off_end && g < r_cap) {
      int lo = 0, hi = E - 1;  // last expert with offsets[e] <= g
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (offsets[mid] <= g) lo = mid; else hi = mid - 1;
      }
      e = lo;
      s_off[tid] = offsets[e];
      s_len[tid] = offsets[e + 1] - offsets[e];
      s_dexp[tid] = COL ? pow2_exponent(col_scale[e]) : 0;
    }
    s_bexp[tid] = e;
  }
  {
    // prologue: one thread per tile row -- source row, t, the tile's scale
    // bytes; rowwise scale bytes and t go out here.
    int g = g_base + tid;
    bool live = g < off_end && g < r_cap;
    int src = live ? src_row[g] : -1;
    if (src >= T) src = -1;
    float t = 0.0f;
    uint32_t sw0 = 0, sw1 = 0;
    if (src >= 0) {
      const uint8_t* prow = packed + (size_t)src * row_bytes;
      t = *reinterpret_cast<const float*>(prow + toff);
      const uint32_t* sp = reinterpret_cast<const uint32_t*>(prow + (H >> 1) + (col0 >> 4));
      sw0 = sp[0];
      if (ncols > 64) sw1 = sp[1];
    }
    s_src[tid] = src;
    s_t[tid] = t;
    s_sw[tid][0] = sw0;
    s_sw[tid][1] = sw1;
    if (live) {
      uint32_t* rs = reinterpret_cast<uint32_t*>(row_scales + (size_t)g * (H >> 4) + (col0 >> 4));
      rs[0] = sw0;
      if (ncols > 64) rs[1] = sw1;
      if (ct == 0) row_t[g] = t;
    }
  }
  __syncthreads();

  const int cg = tid & 15, m = tid >> 4;
  const bool live = s_bexp[m] >= 0 && cg * 8 < ncols;
  if (live) {
    uint32_t cw[16];
    float cm[16];
    int ce[16];
    bool slow = false;
    const int r0 = 16 * m;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int src = s_src[r0 + i];
      cw[i] = src >= 0 ? *reinterpret_cast<const uint32_t*>(packed + (size_t)src * row_bytes + (col0 >> 1) + 4 * cg) : 0u;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int g = g_base + r0 + i;
      *reinterpret_cast<uint32_t*>(row_codes + (size_t)g * (H >> 1) + (col0 >> 1) + 4 * cg) = cw[i];
    }
    if (COL) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint32_t sw = s_sw[r0 + i][cg >> 3];
        float s = e4m3_decode(sw >> (8 * ((cg >> 1) & 3)));
        float t = s_t[r0 + i];
        float sd = s * rht_in_scale(i);  // exact: s has 4 significant bits
        // t >= 2^-100 keeps s*t/4 and every product e2m1*s*t/4 exact or one rounding
        bool tiny = t < 0x1p-100f && t > 0.0f;
        slow |= tiny;
        cm[i] = sd;
        ce[i] = t > 0.0f ? pow2_exponent(t) : 0;
        if (!tiny) cm[i] = sd * t;
      }
      if (slow) {
        // one row of the block is tiny: use the per-element two-step decode for all 16
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          uint32_t sw = s_sw[r0 + i][cg >> 3];
          cm[i] = e4m3_decode(sw >> (8 * ((cg >> 1) & 3))) * rht_in_scale(i);
          if (s_t[r0 + i] == 0.0f) cm[i] = 0.0f;
        }
      }
      const int dexp = s_dexp[m];
      column_pair<0, COL>(cw, cm, ce, slow, dexp, stage_codes, stage_sc, cg * 8, m);
      column_pair<1, COL>(cw, cm, ce, slow, dexp, stage_codes, stage_sc, cg * 8, m);
      column_pair<2, COL>(cw, cm, ce, slow, dexp, stage_codes, stage_sc, cg * 8, m);
      column_pair<3, COL>(cw, cm, ce, slow, dexp, stage_codes, stage_sc, cg * 8, m);
    }
  }
  if (!COL) return;
  __syncthreads();
  // transposed copy-out: item = (column, block); 16 consecutive threads cover
  // one column's blocks, i.e. up to 128 contiguous code bytes.
#pragma unroll
  for (int r = 0; r < (kTileCols * kBlocks) / 256; ++r) {
    int it = r * 256 + tid;
    int c = it >> 4, b = it & 15;
    int e = s_bexp[b];
    if (e < 0 || c >= ncols) continue;
    int off = s_off[b], len = s_len[b];
    int g = g_base + 16 * b;
    size_t h = (size_t)(col0 + c);
    uint2* dst = reinterpret_cast<uint2*>(col_codes + (size_t)H * (off >> 1) + h * (size_t)(len >> 1) + ((g - off) >> 1));
    *dst = stage_codes[c * kBlocks + b];
    col_scales[(size_t)H * (off >> 4) + h * (size_t)(len >> 4) + ((g - off) >> 4)] = stage_sc[c * kBlocks + b];
  }
}

}  // namespace mtb

using namespace mtb;

static int32_t receive_check(const uint8_t* packed, int64_t tokens, int64_t hidden, int64_t num_experts,
                             int64_t r_cap, const int32_t* offsets, const int32_t* src_row) {
  if (tokens < 0 || r_cap < 0 || num_experts < 1 || hidden <= 0 || hidden % 64 != 0) return EP_ERR_SHAPE;
  if (tokens >= INT32_MAX / 4 || r_cap >= INT32_MAX / 4 || hidden > (1 << 20)) return EP_ERR_RANGE;
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
  dim3 grid((unsigned)((H + kTileCols - 1) / kTileCols), (unsigned)((r_cap + kTileRows - 1) / kTileRows));
  hipLaunchKernelGGL(k_nvfp4_receive<true>, grid, dim3(256), 0, (hipStream_t)stream, packed, (int)tokens, H,
                     9 * H / 16 + 4, offsets, (int)num_experts, src_row, (int)r_cap, row_codes, row_scales, row_t,
                     col_codes, col_scales, col_scale);
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
  dim3 grid((unsigned)((H + kTileCols - 1) / kTileCols), (unsigned)((r_cap + kTileRows - 1) / kTileRows));
  hipLaunchKernelGGL(k_nvfp4_receive<false>, grid, dim3(256), 0, (hipStream_t)stream, packed, (int)tokens, H,
                     9 * H / 16 + 4, offsets, (int)num_experts, src_row, (int)r_cap, row_codes, row_scales, row_t,
                     col_codes, col_scales, col_scale);
  return launch_status();
}
