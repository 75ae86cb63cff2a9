/* Host-side argument validation of the C ABI, run against a library whose
 * host code is built with AddressSanitizer and UndefinedBehaviorSanitizer
 * (test_abi_sanitize.py builds and runs it on the CPU).  Every call below
 * must be refused, or be a no-op, before anything reaches the HIP runtime, so
 * no GPU is needed: the pointers are never dereferenced.  Sizes at the ends of
 * int64_t check that the validation's own products and sums do not overflow
 * (signed overflow aborts under -fno-sanitize-recover). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../include/moe_token_block.h"

static int failures = 0;

#define CHECK(expr, want)                                                                          \
  do {                                                                                             \
    long long got_ = (long long)(expr);                                                            \
    if (got_ != (long long)(want)) {                                                               \
      fprintf(stderr, "line %d: %s = %lld, want %lld\n", __LINE__, #expr, got_, (long long)(want)); \
      ++failures;                                                                                  \
    }                                                                                              \
  } while (0)

#define P ((void*)0x1000)
#define N ((void*)0)

static const int64_t MAX = INT64_MAX;
static const int64_t MAX64 = INT64_MAX & ~(int64_t)63;  /* the largest multiple of 64 */
static const int64_t MAX32 = INT64_MAX & ~(int64_t)31;
static const int64_t MAX16 = INT64_MAX & ~(int64_t)15;
static const int64_t I31 = ((int64_t)1 << 31) - 1;

static void helpers(void) {
  CHECK(ep_abi_version(), EP_ABI_VERSION);
  CHECK(ep_rht_sign_mask(), 0xE8D5);
  CHECK(ep_nvfp4_packed_row_bytes(7168), 4036);
  CHECK(ep_nvfp4_packed_row_bytes(100), EP_ERR_SHAPE);
  CHECK(ep_nvfp4_packed_row_bytes(-64), EP_ERR_SHAPE);
  CHECK(ep_nvfp4_packed_row_bytes(MAX64), EP_ERR_RANGE);
  CHECK(ep_route_capacity(4096, 2, 8, 16), 8312);
  CHECK(ep_route_capacity(1, 1, 1, 24), EP_ERR_ALIGN);
  CHECK(ep_route_capacity(MAX, 8, 32, 16), EP_ERR_RANGE);
  CHECK(ep_route_capacity(1, MAX, 1, 16), EP_ERR_RANGE);
  CHECK(ep_route_capacity(1, 1, MAX, 16), EP_ERR_RANGE);
  CHECK(ep_route_capacity(1, 1, 1, MAX16), EP_ERR_RANGE);
  CHECK(ep_route_capacity(I31, I31, I31, ((int64_t)1 << 31) - 16), I31 * I31 + I31 * (((int64_t)1 << 31) - 17));
  CHECK(ep_route_workspace_bytes(MAX, 1, 1), 0);
  CHECK(ep_route_workspace_bytes(1, 1, MAX), 0);
  CHECK(ep_route_workspace_bytes(I31, I31, I31), 0);   /* the byte count itself would overflow */
  CHECK(ep_route_workspace_bytes(512, 1, 8), 2 * 8 * 4);
  CHECK(ep_receive_workspace_bytes(I31, I31, I31), 0);
  CHECK(dswiglu_workspace_bytes(10, 8), 72 + 48);
  CHECK(dswiglu_workspace_bytes(MAX, 1), 0);
  CHECK(dswiglu_workspace_bytes(1, MAX), 0);
  CHECK(dswiglu_workspace_bytes(-1, 1), 0);
  const int32_t codes[] = {EP_OK, EP_ERR_NULL, EP_ERR_SHAPE, EP_ERR_ALIGN, EP_ERR_CAPACITY, EP_ERR_DTYPE,
                           EP_ERR_HIP, EP_ERR_WORKSPACE, EP_ERR_RANGE, EP_ERR_SCRATCH};
  for (size_t i = 0; i < sizeof(codes) / sizeof(codes[0]); ++i) {
    const char* s = ep_status_string(codes[i]);
    CHECK(s != NULL && strlen(s) > 0 && strcmp(s, "unknown status") != 0, 1);
  }
  CHECK(strcmp(ep_status_string(-100), "unknown status"), 0);
  CHECK(strcmp(ep_status_string(INT32_MIN), "unknown status"), 0);
  CHECK(strcmp(ep_status_string(INT32_MAX), "unknown status"), 0);
}

static void packs(void) {
  CHECK(ep_nvfp4_pack(P, 4, 100, P, 0, N, N), EP_ERR_SHAPE);
  CHECK(ep_nvfp4_pack(N, 4, 128, P, 0, N, N), EP_ERR_NULL);
  CHECK(ep_nvfp4_pack(P, 4, 128, P, 1, N, N), EP_ERR_NULL);
  CHECK(ep_nvfp4_pack(P, 4, 128, P, 7, N, N), EP_ERR_DTYPE);
  CHECK(ep_nvfp4_pack(P, 0, 128, N, 0, N, N), EP_OK);
  CHECK(ep_nvfp4_pack(P, MAX, 128, P, 0, N, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_pack(P, 4, MAX64, P, 0, N, N), EP_ERR_SHAPE);
  CHECK(ep_nvfp4_pack(P, -MAX, 128, P, 0, N, N), EP_ERR_SHAPE);
  CHECK(ep_mxfp8_pack(P, 4, 48, P, P, N), EP_ERR_SHAPE);
  CHECK(ep_mxfp8_pack(P, MAX, 32, P, P, N), EP_ERR_RANGE);
  CHECK(ep_mxfp8_pack(P, 2, MAX32, P, P, N), EP_ERR_RANGE);
  CHECK(ep_mxfp8_pack(P, ((int64_t)1 << 35), 32, P, P, N), EP_ERR_RANGE);  /* exactly 2^40 elements */
  CHECK(ep_nvfp4_pack_scatter(P, 4, 128, 33, P, 4, 64, P, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_pack_scatter(P, MAX, 128, 2, P, 4, 64, P, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_pack_scatter(P, 4, 128, MAX, P, 4, 64, P, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_pack_scatter(P, 4, 128, 2, P, 4, MAX, P, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_pack_scatter(P, 4, MAX64, 2, P, 4, 64, P, P, P, P, P, N), EP_ERR_SHAPE);
}

static void unpacks(void) {
  CHECK(ep_nvfp4_unpack(P, 4, 128, N, 5, P, N), EP_ERR_SHAPE);
  CHECK(ep_nvfp4_unpack(P, MAX, 128, N, MAX, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_unpack(P, 4, 128, P, MAX, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_unpack(P, 4, MAX64, N, 4, P, N), EP_ERR_RANGE);
  CHECK(ep_mxfp8_direct_receive(P, P, MAX, 32, 64, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_mxfp8_direct_receive(P, P, 4, MAX32, 64, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_mxfp8_direct_receive(P, P, 4, 32, MAX, P, P, P, N), EP_ERR_RANGE);
}

static void routing(void) {
  CHECK(ep_route_plan(P, 0, 10, 2, 4, 24, 100, P, P, P, P, P, 1 << 20, P, N), EP_ERR_ALIGN);
  CHECK(ep_route_plan(P, 0, 10, 2, 4, 16, 59, P, P, P, P, P, 1 << 20, P, N), EP_ERR_CAPACITY);
  CHECK(ep_route_plan(P, 3, 10, 2, 4, 16, 80, P, P, P, P, P, 1 << 20, P, N), EP_ERR_DTYPE);
  CHECK(ep_route_plan(P, 0, 10, 2, 4, 16, 80, P, P, P, P, P, 4, P, N), EP_ERR_WORKSPACE);
  CHECK(ep_route_plan(P, 0, MAX, 2, 4, 16, 100, P, P, P, P, P, 1 << 20, P, N), EP_ERR_RANGE);
  CHECK(ep_route_plan(P, 0, 10, MAX, 4, 16, 100, P, P, P, P, P, 1 << 20, P, N), EP_ERR_RANGE);
  CHECK(ep_route_plan(P, 0, 10, 2, 4, MAX16, 100, P, P, P, P, P, 1 << 20, P, N), EP_ERR_RANGE);
  CHECK(ep_route_plan(P, 0, 10, 2, 4, 16, MAX, P, P, P, P, P, 1 << 20, P, N), EP_ERR_RANGE);
  CHECK(ep_route_plan(P, 0, 10, 2, MAX, 16, 100, P, P, P, P, P, 1 << 20, P, N), EP_ERR_SHAPE);
  CHECK(ep_route_plan(P, 0, 10, 2, 4, 16, 100, P, P, P, P, P, (size_t)-1, P, N) == EP_ERR_WORKSPACE, 0);
}

static void receives(void) {
  CHECK(ep_nvfp4_direct_receive(P, 4, 128, 2, 64, N, P, P, P, P, N, N, N, N), EP_ERR_NULL);
  CHECK(ep_nvfp4_direct_receive(P, 4, 128, 1025, 64, P, P, P, P, P, N, N, N, N), EP_ERR_SHAPE);
  CHECK(ep_nvfp4_direct_receive(P, MAX, 128, 2, 64, P, P, P, P, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_direct_receive(P, 4, MAX64, 2, 64, P, P, P, P, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_direct_receive(P, 4, 128, 2, MAX, P, P, P, P, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_direct_receive(P, 4, 128, MAX, 64, P, P, P, P, P, P, P, P, N), EP_ERR_SHAPE);
  CHECK(ep_nvfp4_direct_receive(P, 1 << 24, 64, 2, 64, P, P, P, P, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_direct_receive_kblock(P, 532083, 7168, 2, 64, P, P, P, P, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_direct_receive_kblock(P, MAX, 7168, 2, 64, P, P, P, P, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_direct_receive_scaled(P, 4, 128, 2, MAX, P, P, P, P, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_direct_receive_sr(P, 4, 128, 2, 64, P, P, P, P, P, P, P, P, N, N), EP_ERR_NULL);
  CHECK(ep_nvfp4_direct_receive_sr_stream(P, MAX, 128, 2, 64, P, P, P, P, P, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_expert_scale(P, MAX, 128, 2, 64, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_columnwise_grouped(P, P, P, 7168, 2, 599187, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_columnwise_grouped(P, P, P, 128, 4, MAX, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_columnwise_grouped(P, P, P, MAX64, 4, 64, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_mxfp4_direct_receive(P, 4, 128, 2, 48, 64, P, P, P, P, P, P, N), EP_ERR_ALIGN);
  CHECK(ep_mxfp4_direct_receive(P, MAX, 128, 2, 32, 64, P, P, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_mxfp4_direct_receive(P, 4, 128, 2, MAX32, 0, P, P, P, P, P, P, N), EP_OK);  /* nothing to receive */
  CHECK(ep_mxfp4_direct_receive_kblock(P, 1 << 24, 64, 2, 32, 64, P, P, P, P, P, P, N), EP_ERR_RANGE);
  CHECK(ep_mxfp4_kblock_tile(P, P, 128, 0, 288, 0, 16, P, N), EP_ERR_SHAPE);
  CHECK(ep_mxfp4_kblock_tile(P, P, 128, MAX32, 256, 0, 16, P, N), EP_ERR_RANGE);
  CHECK(ep_mxfp4_kblock_tile(P, P, 128, 0, 256, MAX, 16, P, N), EP_ERR_SHAPE);
  CHECK(ep_mxfp4_kblock_tile(P, P, 128, 0, 256, 0, MAX, P, N), EP_ERR_SHAPE);
  CHECK(ep_mxfp4_kblock_tile(P, P, 128, 0, MAX32, 0, 16, P, N), EP_ERR_SHAPE);
  CHECK(ep_mxfp4_kblock_tile(P, P, MAX64, 0, 256, 0, 16, P, N), EP_ERR_SHAPE);
#define R10 P, P, P, P, P, P, P, P, P, P
  CHECK(ep_nvfp4_direct_receive_topk(P, 10, 128, P, 0, 2, 4, 16, 59, R10, P, 1 << 20, P, N), EP_ERR_CAPACITY);
  CHECK(ep_nvfp4_direct_receive_topk(P, 10, 128, P, 0, MAX, 4, 16, 80, R10, P, 1 << 20, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_direct_receive_topk(P, 10, 128, P, 0, 2, 4, MAX16, 80, R10, P, 1 << 20, P, N), EP_ERR_RANGE);
  CHECK(ep_nvfp4_direct_receive_topk(P, MAX, 128, P, 0, 2, 4, 16, 80, R10, P, 1 << 20, P, N), EP_ERR_RANGE);
#undef R10
}

static void dswiglu(void) {
  CHECK(dswiglu_nvfp4_quant(P, P, 10, 100, P, 2, P, P, P, P, P, P, P, P, P, 16, N), EP_ERR_SHAPE);
  CHECK(dswiglu_nvfp4_quant(P, P, 10, 128, P, 2, P, P, P, P, P, P, P, P, P, 4, N), EP_ERR_WORKSPACE);
  CHECK(dswiglu_nvfp4_quant(P, P, MAX, 128, P, 2, P, P, P, P, P, P, P, P, P, 4096, N), EP_ERR_RANGE);
  CHECK(dswiglu_nvfp4_quant(P, P, 10, MAX64, P, 2, P, P, P, P, P, P, P, P, P, 4096, N), EP_ERR_RANGE);
  CHECK(dswiglu_nvfp4_quant(P, P, 10, 128, P, MAX, P, P, P, P, P, P, P, P, P, 4096, N), EP_ERR_SHAPE);
  CHECK(dswiglu_nvfp4_quant_sr(P, P, 10, 128, P, 2, P, P, P, P, P, P, P, P, P, 4096, N, N), EP_ERR_NULL);
  CHECK(dswiglu_nvfp4_quant_sr_stream(P, P, MAX, 128, P, 2, P, P, P, P, P, P, P, P, P, 4096, P, N), EP_ERR_RANGE);
  CHECK(dswiglu_nvfp4_quant_noalloc(P, P, 1100000, 64, P, 8, P, P, P, P, P, P, P, P, N), EP_ERR_SCRATCH);
  CHECK(dswiglu_nvfp4_quant_noalloc(P, P, MAX, 64, P, 8, P, P, P, P, P, P, P, P, N), EP_ERR_SCRATCH);
  CHECK(dswiglu_nvfp4_quant_noalloc(P, P, 10, 64, P, MAX, P, P, P, P, P, P, P, P, N), EP_ERR_SCRATCH);
  CHECK(dswiglu_nvfp4_quant_noalloc(P, P, -1, 64, P, 8, P, P, P, P, P, P, P, P, N), EP_ERR_SHAPE);
}

int main(void) {
  helpers();
  packs();
  unpacks();
  routing();
  receives();
  dswiglu();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi validation: all checks passed\n");
  return 0;
}
