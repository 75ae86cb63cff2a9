// NVFP4 rows -> BF16 (P1, PR description: rows not consumed directly are
// decoded to BF16), with an optional gather by a source-row map; and the
// MXFP8 grouped receive (a plain row gather).
//
// Unpack mapping: one wave64 per output row, lane l owns 8-element chunks
// l, l+64, ...: a 4-byte code load, the block's scale byte, one 16-byte store.
// Decode: the converter gives e2m1 * 2^(k+e) exactly (k = the scale's
// exponent, e = the row's), one multiply by the scale's significand makes the
// exact product e2m1 * s * t, and v_cvt_pk_bf16_f32 rounds it to BF16.
#include "common.h"
#include "launch.h"

namespace mtb {

__device__ __forceinline__ uint32_t bf16pair(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// 8 E2M1 codes of word w (4 bytes) times the block multiplier -> 4 packed BF16 pairs.
__device__ __forceinline__ void decode8(uint32_t w, float scale, float mant, uint32_t* o) {
  f32x2 p0 = fp4_unpack2<0>(w, scale), p1 = fp4_unpack2<1>(w, scale);
  f32x2 p2 = fp4_unpack2<2>(w, scale), p3 = fp4_unpack2<3>(w, scale);
  o[0] = bf16pair(p0[0] * mant, p0[1] * mant);
  o[1] = bf16pair(p1[0] * mant, p1[1] * mant);
  o[2] = bf16pair(p2[0] * mant, p2[1] * mant);
  o[3] = bf16pair(p3[0] * mant, p3[1] * mant);
}

// Rows whose k + e falls below -126 (t < 2^-117): exact e2m1 * s first, then
// one rounding by the power of two.
__device__ __forceinline__ void decode8_tiny(uint32_t w, float s, int e, uint32_t* o) {
  f32x2 p[4] = {fp4_unpack2<0>(w, 1.0f), fp4_unpack2<1>(w, 1.0f), fp4_unpack2<2>(w, 1.0f), fp4_unpack2<3>(w, 1.0f)};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = bf16pair(__builtin_ldexpf(p[i][0] * s, e), __builtin_ldexpf(p[i][1] * s, e));
}

// One wave per output row; lane l decodes 8-element chunks l, l+64, ... (a
// dword of codes -> 16 bytes of BF16), so every load instruction reads 256
// contiguous code bytes and every store writes 1 KiB contiguously.
// The BF16 rows go out with streaming (nontemporal) stores: whole lines, read by
// no later kernel of this library (their reader is a GEMM), so they are kept out
// of the 256 MB MALL, which is left to data that is read again soon (the packed
// rows the receive reads once per routed copy, the dX the FC1-grad quantizer
// re-reads).  Measured: the same call time alone (17.6 us on 67 MB; 548 -> 374 us
// on a 1.9 GB output), and the dispatch step with the MXFP8 receive done the same
// way 203 -> 185 us.
__global__ __launch_bounds__(256) void k_nvfp4_unpack(const uint8_t* __restrict__ packed, int rows_in, int H,
                                                      int row_bytes, const int32_t* __restrict__ src_row,
                                                      int rows_out, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int g = (int)(blockIdx.x * 4u + (threadIdx.x >> 6));
  if (g >= rows_out) return;
  int src = src_row ? src_row[g] : g;
  if (src >= rows_in) src = -1;  // out-of-range map entries decode as zero rows
  const int nch = H >> 3;
  u32x4* orow = reinterpret_cast<u32x4*>(out + (size_t)g * H);
  if (src < 0) {
    for (int c = lane; c < nch; c += 64) __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, orow + c);
    return;
  }
  const uint8_t* prow = packed + (size_t)src * row_bytes;
  const uint32_t* cw = reinterpret_cast<const uint32_t*>(prow);
  // eight chunks per lane at a time: their code and scale loads go out together
  // (indices clamped into the row), then the decodes and stores.  The row's t is
  // loaded with the first group, so that it costs no round trip of its own.
  uint32_t wv[8], sv[8];
  auto load_group = [&](int cb) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = min(cb + u * 64 + lane, nch - 1);
      wv[u] = cw[c];
      sv[u] = prow[(H >> 1) + (c >> 1)];
    }
  };
  auto decode_group = [&](int cb, int e) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = cb + u * 64 + lane;  // lanes past the row decode a clamped chunk and skip the store
      const float s = e4m3_decode(sv[u]);
      uint32_t o[4];
      if (s == 0.0f) {
        decode8(wv[u], 1.0f, 0.0f, o);  // zero scale: signed zeros
      } else {
        int k = __builtin_amdgcn_frexp_expf(s) - 1;
        float mant = __builtin_amdgcn_frexp_mantf(s) * 2.0f;
        int K = k + e;
        if (K >= -126) decode8(wv[u], pow2f(K), mant, o);
        else decode8_tiny(wv[u], s, e, o);
      }
      if (c < nch) __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]}, orow + c);
    }
  };
  load_group(0);
  const int e = pow2_exponent(*reinterpret_cast<const float*>(prow + (H >> 1) + (H >> 4)));
  decode_group(0, e);
  for (int cb = 8 * 64; cb < nch; cb += 8 * 64) {
    load_group(cb);
    decode_group(cb, e);
  }
}

// MXFP8 grouped receive: grouped row g copies token src_row[g] (data + scales);
// -1 rows are zero.  One wave per grouped row, 16-byte copies; streaming stores,
// as in the unpack (the grouped operand is a GEMM's, not read again here).
__global__ __launch_bounds__(256) void k_mxfp8_receive(const uint8_t* __restrict__ data,
                                                       const uint8_t* __restrict__ scales, int tokens, int H,
                                                       const int32_t* __restrict__ src_row, int r_cap,
                                                       uint8_t* __restrict__ g_data, uint8_t* __restrict__ g_scales) {
  const int lane = threadIdx.x & 63;
  const int g = (int)(blockIdx.x * 4u + (threadIdx.x >> 6));
  if (g >= r_cap) return;
  const int src = src_row[g];
  const int n16 = H >> 4, ns = H >> 5;
  u32x4* dst = reinterpret_cast<u32x4*>(g_data + (size_t)g * H);
  uint8_t* ds = g_scales + (size_t)g * ns;
  if (src < 0 || src >= tokens) {  // padding (or an out-of-range entry): zero bytes
    for (int i = lane; i < n16; i += 64) __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, dst + i);
    for (int i = lane; i < ns; i += 64) __builtin_nontemporal_store((uint8_t)0, ds + i);
    return;
  }
  // loads first, four per lane at a time at indices clamped into the row, so
  // that a row needs one memory round trip per 4 KiB, not one per 1 KiB
  const u32x4* sp = reinterpret_cast<const u32x4*>(data + (size_t)src * H);
  const uint8_t* ss = scales + (size_t)src * ns;
  for (int i0 = 0; i0 < n16 || i0 < ns; i0 += 4 * 64) {
    u32x4 v[4];
    uint32_t b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = sp[min(i0 + u * 64 + lane, n16 - 1)];
      b[u] = ss[min(i0 + u * 64 + lane, ns - 1)];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * 64 + lane;
      if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
      if (i < ns) __builtin_nontemporal_store((uint8_t)b[u], ds + i);
    }
  }
}

}  // namespace mtb

using namespace mtb;

MTB_EXPORT int32_t ep_nvfp4_unpack(const uint8_t* packed, int64_t rows_in, int64_t hidden, const int32_t* src_row,
                                   int64_t rows_out, uint16_t* out, void* stream) {
  if (rows_in < 0 || rows_out < 0 || hidden <= 0 || hidden % 64 != 0) return EP_ERR_SHAPE;
  if (!src_row && rows_out != rows_in) return EP_ERR_SHAPE;
  if (rows_in > INT32_MAX / 4 || rows_out > INT32_MAX / 4 || hidden > (1 << 20)) return EP_ERR_RANGE;
  if (rows_out == 0) return EP_OK;
  if (!out || (rows_in > 0 && !packed)) return EP_ERR_NULL;
  if (!src_row && rows_in == 0) return EP_OK;
  const int H = (int)hidden;
  dim3 grid((unsigned)((rows_out + 3) / 4)), block(256);
  hipLaunchKernelGGL(k_nvfp4_unpack, grid, block, 0, (hipStream_t)stream, packed, (int)rows_in, H, 9 * H / 16 + 4,
                     src_row, (int)rows_out, out);
  return launch_status();
}

MTB_EXPORT int32_t ep_mxfp8_direct_receive(const uint8_t* data, const uint8_t* scales, int64_t tokens,
                                           int64_t hidden, int64_t r_cap, const int32_t* src_row,
                                           uint8_t* g_data, uint8_t* g_scales, void* stream) {
  if (tokens < 0 || r_cap < 0 || hidden <= 0 || hidden % 32 != 0) return EP_ERR_SHAPE;
  if (tokens > INT32_MAX / 4 || r_cap > INT32_MAX / 4 || hidden > (1 << 24)) return EP_ERR_RANGE;
  if (r_cap == 0) return EP_OK;
  if (!src_row || !g_data || !g_scales || (tokens > 0 && (!data || !scales))) return EP_ERR_NULL;
  dim3 grid((unsigned)((r_cap + 3) / 4)), block(256);
  hipLaunchKernelGGL(k_mxfp8_receive, grid, block, 0, (hipStream_t)stream, data, scales, (int)tokens, (int)hidden, src_row,
                     (int)r_cap, g_data, g_scales);
  return launch_status();
}
