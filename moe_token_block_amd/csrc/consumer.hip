// A consumer of the K-blocked MXFP4 operand: gfx950's block-scaled matrix
// instruction (v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 operands) reading
// the bytes exactly as ep_mxfp4_direct_receive_kblock stores them.  It exists
// to check that the stored layout is the instruction's operand layout: lane
// l = 16 q + i takes row i's 32 consecutive K values [32 q, 32 q + 32) of a
// 128-value K step -- 16 contiguous code bytes, element 2j in the low nibble
// of byte j -- and that K group's scale byte, both at the places the layout
// gives them, with no reshuffle.  One 16 x 16 tile per call, not a GEMM.
#include "common.h"
#include "launch.h"

namespace mtb {

typedef int v8i32 __attribute__((ext_vector_type(8)));
typedef float v4f32 __attribute__((ext_vector_type(4)));
constexpr int kFmtE2M1 = 4;  // the instruction's operand format code for E2M1

// One wave: D[i][j] = sum over the K-block's len rows k of A[ha + i][k] * A[hb + j][k],
// A the K-block's [H, len] operand (codes [H, len/2] bytes, scales [H, len/32]).
// K values past len (the last K step of a block that is not a multiple of 128)
// enter as zero codes with scale 2^0.
__global__ __launch_bounds__(64) void k_mxfp4_kblock_tile(const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ scales, int len, int ha, int hb,
                                                          float* __restrict__ out) {
  const int l = threadIdx.x, i = l & 15, q = l >> 4;
  const uint32_t cstr = (uint32_t)len >> 1, sstr = (uint32_t)len >> 5;
  v4f32 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = 0; k0 < len; k0 += 128) {
    const int kk = k0 + 32 * q;  // this lane's first K value in the step
    v8i32 a = {0, 0, 0, 0, 0, 0, 0, 0}, b = {0, 0, 0, 0, 0, 0, 0, 0};
    int sa = 127, sb = 127;
    if (kk < len) {
      const uint4 va = *reinterpret_cast<const uint4*>(codes + (size_t)(uint32_t)(ha + i) * cstr + (kk >> 1));
      const uint4 vb = *reinterpret_cast<const uint4*>(codes + (size_t)(uint32_t)(hb + i) * cstr + (kk >> 1));
      a[0] = (int)va.x; a[1] = (int)va.y; a[2] = (int)va.z; a[3] = (int)va.w;
      b[0] = (int)vb.x; b[1] = (int)vb.y; b[2] = (int)vb.z; b[3] = (int)vb.w;
      sa = scales[(size_t)(uint32_t)(ha + i) * sstr + (kk >> 5)];
      sb = scales[(size_t)(uint32_t)(hb + i) * sstr + (kk >> 5)];
    }
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, kFmtE2M1, kFmtE2M1, 0, sa, 0, sb);
  }
  // the result: lane l holds rows 4q .. 4q+3 of column i
#pragma unroll
  for (int r = 0; r < 4; ++r) out[(4 * q + r) * 16 + i] = acc[r];
}

}  // namespace mtb

using namespace mtb;

MTB_EXPORT int32_t ep_mxfp4_kblock_tile(const uint8_t* col_codes, const uint8_t* col_scales, int64_t hidden,
                                        int64_t block_row, int64_t len, int64_t ha, int64_t hb, float* out,
                                        void* stream) {
  if (!col_codes || !col_scales || !out) return EP_ERR_NULL;
  if (hidden <= 0 || hidden % 64 != 0 || hidden > (1 << 20)) return EP_ERR_SHAPE;
  if (len <= 0 || len > 256 || len % 32 != 0 || block_row < 0 || block_row % 32 != 0) return EP_ERR_SHAPE;
  if (ha < 0 || hb < 0 || ha > hidden - 16 || hb > hidden - 16) return EP_ERR_SHAPE;
  if (block_row >= kSizeLimit || (block_row + len) * hidden / 2 >= ((int64_t)1 << 40)) return EP_ERR_RANGE;
  const uint8_t* codes = col_codes + hidden * block_row / 2;
  const uint8_t* scales = col_scales + hidden * block_row / 32;
  hipLaunchKernelGGL(k_mxfp4_kblock_tile, dim3(1), dim3(64), 0, (hipStream_t)stream, codes, scales, (int)len, (int)ha,
                     (int)hb, out);
  return launch_status();
}
