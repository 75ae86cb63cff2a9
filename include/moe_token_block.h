/*
 * moe_token_block -- block-scaled low-precision quantization of MoE token rows
 * on AMD Instinct MI355X (gfx950).  Plain C ABI.
 *
 * Sources (cited by page title and section):
 *   P1 "[Common][PyTorch] Add NVFP4 EP dispatch and combine backward"
 *      (TransformerEngine PR #3753) -- PR description, commit messages.
 *   P2 "[Common][PyTorch] EP dispatch with unfused MXFP8 quantization"
 *      (TransformerEngine PR #3270) -- description, "Changes", review comments.
 *   P3 "[PyTorch] Enable NVFP4 row-scaled (per-token) backward for
 *      GroupedLinear" (TransformerEngine PR #3324) -- description.
 *   P4 "[PyTorch] Optionally derive FC1 dy NVFP4 amaxes from the dGLU
 *      epilogue" (TransformerEngine PR #3755) -- description, test commit.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates nothing, never synchronizes the host, never changes the current
 *     device and launches only on `stream` (a hipStream_t; NULL = the null
 *     stream).  Every call is therefore capturable in a HIP graph.  The device
 *     that owns the buffers must be current.
 *   - BF16 tensors are passed as uint16_t bit patterns, row-major, contiguous.
 *   - Return value: EP_OK (0) or a negative EP_ERR_* code.  Arguments are
 *     validated on the host before anything is launched; on an error nothing
 *     is launched and no output is touched.  EP_ERR_HIP reports a failed launch
 *     (the HIP error is cleared).  Nothing is printed, nothing aborts, no C++
 *     exception crosses this boundary.
 *   - Errors that only the data can reveal (an expert id out of range) are
 *     reported by setting a caller-provided device word `d_error` to a
 *     non-zero EP_DEVERR_* bit; the offending entry is dropped.
 *   - Calls that share output buffers must not overlap in time.
 *
 * Formats (fixed by this library's readings of the pages; see each function):
 *   E2M1  4-bit code: bit 3 sign, bits 0..2 index into {0,.5,1,1.5,2,3,4,6};
 *         element 2j in the low nibble of byte j.
 *   E4M3  OCP FP8 E4M3FN (max 448, subnormals, never NaN here).
 *   E8M0  power-of-two scale 2^(code-127).
 *   NVFP4 packed row: [H/2 code bytes | H/16 E4M3 scale bytes | FP32 t, LE];
 *         stride 9H/16 + 4 bytes; value = e2m1 * s_b * t.
 */
#ifndef MOE_TOKEN_BLOCK_H
#define MOE_TOKEN_BLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EP_ABI_VERSION 1

enum ep_status {
  EP_OK = 0,
  EP_ERR_NULL = -1,      /* a required pointer is NULL                        */
  EP_ERR_SHAPE = -2,     /* a size is negative, zero where it must not be, or
                            not a multiple the format needs                  */
  EP_ERR_ALIGN = -3,     /* alignment is not a positive multiple of 16       */
  EP_ERR_CAPACITY = -4,  /* r_cap is below ep_route_capacity(...)             */
  EP_ERR_DTYPE = -5,     /* unknown index dtype or rounding mode             */
  EP_ERR_HIP = -6,       /* a kernel launch failed                            */
  EP_ERR_WORKSPACE = -7, /* workspace NULL or smaller than required          */
  EP_ERR_RANGE = -8,     /* a size exceeds what the kernels index (2^31)     */
  EP_ERR_SCRATCH = -9    /* sizes need more than the static scratch of an
                            allocation-free entry point                       */
};

/* Bytes of device scratch each GPU holds for the allocation-free entry point
 * dswiglu_nvfp4_quant_noalloc (4 MiB: the workspace of up to 1,046,524 token
 * rows with 1024 experts). */
#define EP_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)

/* device-side error bits written to *d_error (OR-ed) */
#define EP_DEVERR_EXPERT_ID 1 /* a top-k entry outside [-1, num_experts)     */

/* stochastic-rounding modes for ep_nvfp4_pack */
#define EP_ROUND_NEAREST 0   /* round-to-nearest-even                          */
#define EP_ROUND_SR_ELEMENT 1 /* Philox4x32-10 word 0 at counter n             */
#define EP_ROUND_SR_STREAM 2  /* 32-bit word n of the Philox4x32-10 stream     */
#define EP_ROUND_SR_ELEMENT_CARRY 3 /* as SR_ELEMENT, carry-form decision      */
#define EP_ROUND_SR_STREAM_CARRY 4  /* as SR_STREAM, carry-form decision       */

/* top-k index dtypes for ep_route_plan */
#define EP_IDX_INT32 0
#define EP_IDX_INT64 1

/* ---------------------------------------------------------------- helpers */

/* ABI version of the loaded library (EP_ABI_VERSION it was built with). */
int32_t ep_abi_version(void);

/* Static English text for a status code (never NULL). */
const char* ep_status_string(int32_t status);

/* Bytes of one packed NVFP4 row, 9*hidden/16 + 4; negative (EP_ERR_SHAPE) if
 * hidden is not a positive multiple of 64, EP_ERR_RANGE if hidden >= 2^31. */
int64_t ep_nvfp4_packed_row_bytes(int64_t hidden);

/* Grouped-row capacity the routing plan needs: tokens*top_k +
 * num_experts*(alignment-1); negative status on invalid arguments
 * (EP_ERR_RANGE if any argument is >= 2^31). */
int64_t ep_route_capacity(int64_t tokens, int64_t top_k, int64_t num_experts, int64_t alignment);

/* Workspace bytes ep_route_plan needs for these sizes; 0 if a size is
 * negative or zero where it must not be, or >= 2^31. */
size_t ep_route_workspace_bytes(int64_t tokens, int64_t top_k, int64_t num_experts);

/* The 16-bit RHT sign mask M: d_i = -1 iff bit i of M is set.  Exported so a
 * caller can apply the same transform to the other wgrad operand. */
uint32_t ep_rht_sign_mask(void);

/* Workspace bytes dswiglu_nvfp4_quant needs (offsets + one word per token
 * row); 0 if tokens < 0, num_experts < 1 or either is >= 2^31. */
size_t dswiglu_workspace_bytes(int64_t tokens, int64_t num_experts);

/* ---------------------------------------------------------------- pack */

/* NVFP4 row pack (P1, PR description: each BF16 token becomes one NVFP4 row
 * with E2M1 codes, E4M3 block scales and a power-of-two FP32 token scale; the
 * combine backward rounds stochastically).
 *
 *   x       [rows, hidden] BF16.        packed  [rows, 9*hidden/16 + 4] bytes.
 *   t = 2^e, e the least integer with max|x_row| <= 2688 * 2^e (t = 1 for a
 *   zero row); block scale s_b = E4M3(a_b / (6t)) of the block max a_b;
 *   code = sign(x) | E2M1 index of |x| / (s_b t) (0 if s_b = 0).
 *   round_mode EP_ROUND_NEAREST: round-to-nearest-even, sr_state ignored.
 *   round_mode EP_ROUND_SR_*: stochastic rounding of v = fl32(|x|/(s_b t))
 *     between its grid neighbours g_lo <= v < g_hi with the Philox4x32-10
 *     word w (key = seed) of stream position n = counter_base + row*hidden
 *     + col (SR_ELEMENT*: counter n, word 0; SR_STREAM*: counter n>>2, word
 *     n&3); frac = (v - g_lo)/(g_hi - g_lo).  SR_ELEMENT, SR_STREAM: up iff
 *     (w >> 8) * 2^-24 < frac.  SR_*_CARRY: up iff floor(frac*2^32) + w >=
 *     2^32 (the 32 random bits added below the kept precision, then
 *     truncated -- the decision gfx950's stochastic FP4 conversion makes,
 *     which these modes use).  sr_state is a DEVICE pointer to
 *     two uint64 {seed, counter_base} (read by the kernel, so a captured
 *     graph can be re-seeded between replays); required for SR modes.
 *   Requires hidden a positive multiple of 64, hidden <= 16384, rows >= 0. */
int32_t ep_nvfp4_pack(const uint16_t* x, int64_t rows, int64_t hidden, uint8_t* packed,
                      int32_t round_mode, const uint64_t* sr_state, void* stream);

/* MXFP8 pack (P2, description: BF16 -> E4M3 data with E8M0 scales per 32
 * elements; data-then-scales layout in one caller buffer).
 *   data [rows, hidden] bytes, scales [rows, hidden/32] bytes (scales may be
 *   data + rows*hidden to form the single data-then-scale buffer).
 *   e = least integer with amax_32 <= 448*2^e, clamped to [-127,127] (0 for a
 *   zero block); scale byte e+127; data = sign | E4M3(|x|/2^e), RNE.
 *   Requires hidden a positive multiple of 32. */
int32_t ep_mxfp8_pack(const uint16_t* x, int64_t rows, int64_t hidden, uint8_t* data,
                      uint8_t* scales, void* stream);

/* ---------------------------------------------------------------- unpack */

/* NVFP4 rows -> BF16 (P1, PR description: rows not consumed directly are
 * decoded to BF16).  out[g] = RNE_bf16(e2m1 * s_b * t) of packed row src_row[g]
 * (or row g when src_row is NULL); src_row[g] = -1 gives a zero row; any other
 * src_row value must lie in [0, rows_in).
 *   packed [rows_in, 9*hidden/16+4], src_row [rows_out] int32 or NULL,
 *   out [rows_out, hidden] BF16.  With src_row NULL, rows_out must equal rows_in. */
int32_t ep_nvfp4_unpack(const uint8_t* packed, int64_t rows_in, int64_t hidden,
                        const int32_t* src_row, int64_t rows_out, uint16_t* out, void* stream);

/* ---------------------------------------------------------------- routing */

/* Local routing permutation (P2, review comments: routing prepared once and
 * cached for dispatch and combine; expert slots padded to an alignment.
 * P1, commit messages: top_k, alignment and the index dtype are arguments).
 *   topk_idx [tokens, top_k] int32 or int64 (idx_dtype EP_IDX_*); -1 = unused.
 *   counts [E] int32; offsets [E+1] int32 with off_0 = 0 and
 *   off_{e+1} = off_e + roundup(count_e, alignment);
 *   dst_row [tokens, top_k] int32: grouped row of entry (t, j), -1 if unused;
 *   src_row [r_cap] int32: token of grouped row g, -1 for padding and for
 *   every row from off_E to r_cap.  Rows of an expert keep token order (then
 *   slot order) -- a stable counting sort.
 *   alignment: positive multiple of 16.  r_cap >= ep_route_capacity(...).
 *   workspace: device memory of ep_route_workspace_bytes(...) bytes.
 *   d_error: device int32, OR-ed with EP_DEVERR_EXPERT_ID on a bad id (such
 *   entries are dropped: dst_row -1, not counted).  num_experts <= 1024. */
int32_t ep_route_plan(const void* topk_idx, int32_t idx_dtype, int64_t tokens, int64_t top_k,
                      int64_t num_experts, int64_t alignment, int64_t r_cap,
                      int32_t* counts, int32_t* offsets, int32_t* dst_row, int32_t* src_row,
                      void* workspace, size_t workspace_bytes, int32_t* d_error, void* stream);

/* ---------------------------------------------------------------- receive */

/* NVFP4 direct receive, from a routing plan (P1, PR description: the
 * received rows are turned into the expert GEMM's grouped operands in a single
 * pass -- the rowwise operand is the sender's bytes regrouped, and the
 * columnwise operand gets an RHT and a per-expert scale derived from the token
 * scales, so neither a BF16 copy nor a max pass over the codes is made; P4,
 * description: the RHT output is bounded by four times the rowwise amax).
 *   packed [tokens, 9*hidden/16+4]; offsets [E+1], src_row [r_cap] from
 *   ep_route_plan (src_row values in [-1, tokens)).  The plan is an input so
 *   that one routing (the pages' cached routing, P2 review comments) serves
 *   every receive of a step; ep_nvfp4_direct_receive_topk routes and receives
 *   in one call.
 *   Rowwise (always): row_codes [r_cap, hidden/2], row_scales [r_cap, hidden/16],
 *   row_t [r_cap] FP32: grouped row g (< off_E) holds the code bytes, scale bytes
 *   and t of token src_row[g], zeros for padding.  Rows >= off_E untouched.
 *   Columnwise (when col_codes != NULL; col_scales and col_scale then required):
 *   D_e = 4 * max t over expert e's rows (0 if empty) -> col_scale [E];
 *   for each column h and 16-row block of expert e: y = (1/4) H16 diag(d) z
 *   (a fixed butterfly order, FP32), s = E4M3 of the exact max|y| / (6 D_e),
 *   code = E2M1 of fl32(|y| / (s D_e)).  Expert e's codes are an
 *   [hidden, P_e/2] byte matrix at byte hidden*off_e/2 of col_codes and its
 *   scales an [hidden, P_e/16] matrix at byte hidden*off_e/16 of col_scales
 *   (P_e = off_{e+1} - off_e); col_codes/col_scales need hidden*r_cap/2 and
 *   hidden*r_cap/16 bytes.
 *   Requires hidden a positive multiple of 64 and 1 <= num_experts <= 1024;
 *   tokens < 2^24 and tokens * (9*hidden/16+4) < 2^31 (the kernels address
 *   packed rows through buffer resources with 31-bit offsets; EP_ERR_RANGE
 *   otherwise -- this and every other receive entry point). */
int32_t ep_nvfp4_direct_receive(const uint8_t* packed, int64_t tokens, int64_t hidden,
                                int64_t num_experts, int64_t r_cap,
                                const int32_t* offsets, const int32_t* src_row,
                                uint8_t* row_codes, uint8_t* row_scales, float* row_t,
                                uint8_t* col_codes, uint8_t* col_scales, float* col_scale,
                                void* stream);

/* Workspace bytes ep_nvfp4_direct_receive_topk needs (its routing plan's). */
size_t ep_receive_workspace_bytes(int64_t tokens, int64_t top_k, int64_t num_experts);

/* The direct receive in one call from the top-k indices (P1, PR description:
 * dispatch then the one-pass receive; P1 commit messages: top_k, alignment and
 * the index dtype are arguments): ep_route_plan into counts / offsets /
 * dst_row / src_row (caller-owned, as for ep_route_plan), then
 * ep_nvfp4_direct_receive on that plan.  Arguments, layouts and error words
 * as for those two calls; workspace holds ep_receive_workspace_bytes(...)
 * bytes.  Every argument is checked before the first launch. */
int32_t ep_nvfp4_direct_receive_topk(const uint8_t* packed, int64_t tokens, int64_t hidden,
                                     const void* topk_idx, int32_t idx_dtype, int64_t top_k,
                                     int64_t num_experts, int64_t alignment, int64_t r_cap,
                                     int32_t* counts, int32_t* offsets, int32_t* dst_row, int32_t* src_row,
                                     uint8_t* row_codes, uint8_t* row_scales, float* row_t,
                                     uint8_t* col_codes, uint8_t* col_scales, float* col_scale,
                                     void* workspace, size_t workspace_bytes, int32_t* d_error, void* stream);

/* The two halves of ep_nvfp4_direct_receive, for callers that schedule them
 * separately (e.g. to reuse D_e, or to time the one-pass kernel alone):
 *   ep_nvfp4_expert_scale: col_scale[e] = D_e = 4 * max t over expert e's rows
 *     (0 if empty), reading only the 4-byte token scales (no amax pass);
 *   ep_nvfp4_direct_receive_scaled: the one-pass rowwise + columnwise kernel
 *     with D_e taken from col_scale (each a power of two, or 0 for an empty
 *     expert).  Arguments and layouts as in ep_nvfp4_direct_receive; col_codes,
 *     col_scales and col_scale are required here. */
int32_t ep_nvfp4_expert_scale(const uint8_t* packed, int64_t tokens, int64_t hidden, int64_t num_experts,
                              int64_t r_cap, const int32_t* offsets, const int32_t* src_row, float* col_scale,
                              void* stream);
int32_t ep_nvfp4_direct_receive_scaled(const uint8_t* packed, int64_t tokens, int64_t hidden,
                                       int64_t num_experts, int64_t r_cap,
                                       const int32_t* offsets, const int32_t* src_row,
                                       uint8_t* row_codes, uint8_t* row_scales, float* row_t,
                                       uint8_t* col_codes, uint8_t* col_scales, const float* col_scale,
                                       void* stream);

/* ep_nvfp4_direct_receive_scaled with stochastic columnwise codes (for a
 * gradient operand; TE's NVFP4 recipe, which P1's PR description follows,
 * rounds gradients stochastically).  Same scales; each columnwise code is the
 * carry-form stochastic rounding (see ep_nvfp4_pack, SR_ELEMENT_CARRY) of the
 * same quotient, with word 0 of Philox4x32-10 (key = seed) at counter n =
 * counter_base + the code's index in col_codes (two codes per byte, low nibble
 * first), i.e. counter_base + hidden*off_e + h*P_e + (g - off_e) for column h
 * and grouped row g of expert e.  The rowwise operand is the sender's bytes,
 * as in the deterministic receive.  sr_state: DEVICE pointer to {seed,
 * counter_base} (two uint64). */
int32_t ep_nvfp4_direct_receive_sr(const uint8_t* packed, int64_t tokens, int64_t hidden,
                                   int64_t num_experts, int64_t r_cap,
                                   const int32_t* offsets, const int32_t* src_row,
                                   uint8_t* row_codes, uint8_t* row_scales, float* row_t,
                                   uint8_t* col_codes, uint8_t* col_scales, const float* col_scale,
                                   const uint64_t* sr_state, void* stream);

/* ep_nvfp4_direct_receive_sr with the word-stream mapping of the pack's
 * EP_ROUND_SR_STREAM modes: the code at stream position n takes word (n & 3)
 * of Philox4x32-10 block n >> 2 (same key and positions), four words per
 * block instead of one.  Arguments, layouts and errors as there. */
int32_t ep_nvfp4_direct_receive_sr_stream(const uint8_t* packed, int64_t tokens, int64_t hidden,
                                          int64_t num_experts, int64_t r_cap,
                                          const int32_t* offsets, const int32_t* src_row,
                                          uint8_t* row_codes, uint8_t* row_scales, float* row_t,
                                          uint8_t* col_codes, uint8_t* col_scales, const float* col_scale,
                                          const uint64_t* sr_state, void* stream);

/* The direct receive with the columnwise operand in K-blocks, a layout a
 * grouped GEMM can stream (P1, PR description: the receiver builds the expert
 * GEMM's grouped operand): per expert, the grouped rows are cut into blocks
 * of 256 (the last one shorter, a multiple of 16); block kb of expert e
 * holds an [H, len/2] code matrix at byte H*off_e/2 + 128*H*kb of col_codes
 * and an [H, len/16] scale matrix at byte H*off_e/16 + 16*H*kb of
 * col_scales.  Same values as ep_nvfp4_direct_receive_scaled's compact
 * layout (the same bytes, re-placed); the rowwise operand is identical.
 * col_scale holds D_e (from ep_nvfp4_expert_scale).  A full K-block's
 * columnwise output for 256 columns is one contiguous 32 KB code region
 * (128-byte aligned: hidden*off_e/2 is a multiple of 512) and one 4 KB scale
 * region. */
int32_t ep_nvfp4_direct_receive_kblock(const uint8_t* packed, int64_t tokens, int64_t hidden,
                                       int64_t num_experts, int64_t r_cap,
                                       const int32_t* offsets, const int32_t* src_row,
                                       uint8_t* row_codes, uint8_t* row_scales, float* row_t,
                                       uint8_t* col_codes, uint8_t* col_scales, const float* col_scale,
                                       void* stream);

/* MXFP4 variant of the direct receive.  No page describes it: gfx950's
 * block-scaled matrix instructions take E2M1 elements with one E8M0 scale (a
 * power of two) per 32 elements along K, not NVFP4's E4M3 scale per 16, so
 * this receive re-quantizes the same routed rows to that format in one pass.
 * Decode (exact) and the columnwise RHT are those of ep_nvfp4_direct_receive;
 * the quantizer, per block of 32 values x: e = the least integer with
 * max|x| <= 6 * 2^e, clamped to [-127, 127] (0 for an all-zero block); scale
 * byte e + 127; code = sign(x) | E2M1 round-to-nearest-even of |x| / 2^e
 * (exact, nothing clips).  No per-expert scale and no amax pass.
 *   Rowwise: row_codes [r_cap, hidden/2] (element 2j in the low nibble of byte
 *   j), row_scales [r_cap, hidden/32], for grouped rows g < off_E; padding rows
 *   are zero values (codes 0, scale byte 127); rows >= off_E untouched.
 *   Columnwise: blocks of 32 consecutive grouped rows of one column (two RHT
 *   blocks).  Expert e's codes are an [hidden, P_e/2] byte matrix at byte
 *   hidden*off_e/2 of col_codes, its scales an [hidden, P_e/32] matrix at byte
 *   hidden*off_e/32 of col_scales (hidden*r_cap/2 and hidden*r_cap/32 bytes).
 *   alignment: the one the route plan was made with; a multiple of 32
 *   (EP_ERR_ALIGN otherwise), so no 32-row block straddles two experts.
 *   Requires hidden a positive multiple of 64 and 1 <= num_experts <= 1024. */
int32_t ep_mxfp4_direct_receive(const uint8_t* packed, int64_t tokens, int64_t hidden, int64_t num_experts,
                                int64_t alignment, int64_t r_cap, const int32_t* offsets, const int32_t* src_row,
                                uint8_t* row_codes, uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales,
                                void* stream);

/* The MXFP4 receive with its columnwise operand in K-blocks, as
 * ep_nvfp4_direct_receive_kblock lays out NVFP4's: each expert's grouped rows
 * in blocks of 256 (the last one shorter, a multiple of 32); block kb of
 * expert e holds an [hidden, len/2] code matrix at byte hidden*off_e/2 +
 * 128*hidden*kb of col_codes and an [hidden, len/32] scale matrix at byte
 * hidden*off_e/32 + 8*hidden*kb of col_scales.  The same bytes as
 * ep_mxfp4_direct_receive's, only placed per K-block; rowwise operand,
 * arguments, sizes and errors as there. */
int32_t ep_mxfp4_direct_receive_kblock(const uint8_t* packed, int64_t tokens, int64_t hidden, int64_t num_experts,
                                       int64_t alignment, int64_t r_cap, const int32_t* offsets,
                                       const int32_t* src_row, uint8_t* row_codes, uint8_t* row_scales,
                                       uint8_t* col_codes, uint8_t* col_scales, void* stream);

/* A consumer of that K-blocked operand, for checking that its bytes are the
 * operand layout of gfx950's block-scaled matrix instruction
 * (v_mfma_scale_f32_16x16x128_f8f6f4, E2M1 with one E8M0 scale per 32 K
 * values): no page describes it; it is not a GEMM.  For the K-block whose first
 * grouped row is block_row (off_e + 256*kb) and whose length is len (a
 * multiple of 32, at most 256), out[i*16 + j] = sum over its rows k of
 * A[ha+i][k] * A[hb+j][k], A the block's [hidden, len] operand, computed by
 * that instruction on the stored bytes (each lane reads 16 contiguous code
 * bytes and one scale byte).  out: 256 FP32, device.  col_codes and
 * col_scales must hold the block (hidden*(block_row+len)/2 and /32 bytes).
 * EP_ERR_SHAPE for hidden not a positive multiple of 64, len or block_row off
 * the 32-row grid, len > 256, or a 16-column range outside [0, hidden). */
int32_t ep_mxfp4_kblock_tile(const uint8_t* col_codes, const uint8_t* col_scales, int64_t hidden,
                             int64_t block_row, int64_t len, int64_t ha, int64_t hb, float* out, void* stream);

/* MXFP8 receive (P2, description and review comments: received data and block
 * scales are returned per expert, grouped, with 128-aligned slots there --
 * here any multiple of 16): grouped row g copies token src_row[g]'s data row
 * and scale row; padding rows (src -1, g < r_cap) are zero bytes.
 *   data [tokens, hidden], scales [tokens, hidden/32], src_row [r_cap],
 *   g_data [r_cap, hidden], g_scales [r_cap, hidden/32].  hidden % 32 == 0. */
int32_t ep_mxfp8_direct_receive(const uint8_t* data, const uint8_t* scales, int64_t tokens,
                                int64_t hidden, int64_t r_cap, const int32_t* src_row,
                                uint8_t* g_data, uint8_t* g_scales, void* stream);

/* ---------------------------------------------------------------- fused dispatch */

/* Sender-side pack + scatter (P1, PR description: token rows are quantized
 * once into the format the expert GEMM reads, with no BF16 round trip; here
 * the pack writes each packed row directly into its grouped slots, so the
 * intermediate [tokens, 9H/16+4] buffer and its k-fold re-read disappear).
 *   x [tokens, hidden] BF16; dst_row [tokens, top_k] int32 from
 *   ep_route_plan (entries outside [0, r_cap) are skipped); counts [E] and
 *   offsets [E+1] from the same plan.  Writes row_codes [r_cap, hidden/2],
 *   row_scales [r_cap, hidden/16], row_t [r_cap]: byte-identical to
 *   ep_nvfp4_pack (round to nearest) followed by the rowwise operand of
 *   ep_nvfp4_direct_receive (padding rows below offsets[E] zero, rows from
 *   offsets[E] to r_cap untouched).  top_k <= 32 (EP_ERR_RANGE), hidden as
 *   for ep_nvfp4_pack, 1 <= num_experts <= 1024. */
int32_t ep_nvfp4_pack_scatter(const uint16_t* x, int64_t tokens, int64_t hidden, int64_t top_k,
                              const int32_t* dst_row, int64_t num_experts, int64_t r_cap,
                              const int32_t* counts, const int32_t* offsets, uint8_t* row_codes,
                              uint8_t* row_scales, float* row_t, void* stream);

/* The columnwise half of the direct receive from a grouped rowwise operand
 * (as written by ep_nvfp4_pack_scatter or ep_nvfp4_direct_receive): the rows
 * are contiguous, so there is no gather.  D_e = 4 * max row_t over expert e's
 * rows -> col_scale [E]; col_codes / col_scales as in ep_nvfp4_direct_receive,
 * byte-identical.  hidden % 64 == 0, 1 <= num_experts <= 1024. */
int32_t ep_nvfp4_columnwise_grouped(const uint8_t* row_codes, const uint8_t* row_scales, const float* row_t,
                                    int64_t hidden, int64_t num_experts, int64_t r_cap,
                                    const int32_t* offsets, uint8_t* col_codes, uint8_t* col_scales,
                                    float* col_scale, void* stream);

/* ---------------------------------------------------------------- dSwiGLU */

/* Fused grouped dSwiGLU epilogue with per-expert amax, then FC1-gradient NVFP4
 * quantization with global scales taken from that amax (P4, description: the
 * epilogue's max of dX, rounded to BF16, serves as the rowwise amax and four
 * times it bounds the columnwise amax after the RHT, so the quantizer makes
 * no max pass of its own).
 *   preact [tokens, 2*ffn] BF16 = [a | b] (a = gate, first ffn columns);
 *   dy [tokens, ffn] BF16; rows are expert-major: expert e owns counts[e]
 *   consecutive rows (counts: DEVICE int32 [E], sum == tokens).
 *   dx [tokens, 2*ffn] BF16: da = dy*b*s*(1 + a*(1-s)), db = dy*a*s, s = sigmoid(a),
 *   computed in FP32 and rounded to BF16.
 *   amax [E] FP32 (BF16-representable): max |dx| over the expert's rows.
 *   Rowwise: D_row,e = fl32(amax_e/2688) -> row_scale [E]; per 16-element block:
 *   s = E4M3(fl32(fl32(a_b/6)/D)), code = E2M1 of fl32(|x| / fl32(s D));
 *   row_codes [tokens, ffn] bytes, row_scales [tokens, 2*ffn/16].
 *   Columnwise: D_col,e = fl32(4*amax_e/2688) -> col_scale [E]; rows zero-padded
 *   to P_e = roundup(count_e, 16); the same RHT and quantizer as the direct
 *   receive with D_col; expert e's codes are a [2*ffn, P_e/2] matrix at byte
 *   2*ffn*poff_e/2 (poff = padded offsets) and its scales [2*ffn, P_e/16] at
 *   byte 2*ffn*poff_e/16; col_codes and col_scales need
 *   2*ffn*(tokens + 15*E)/2 and 2*ffn*(tokens + 15*E)/16 bytes.
 *   workspace: device memory of dswiglu_workspace_bytes(tokens, E) bytes,
 *   16-byte aligned (EP_ERR_WORKSPACE otherwise).
 *   Requires ffn a positive multiple of 64.
 *   dx may be NULL: then no BF16 dX is written; the epilogue keeps only each
 *   row's max |dX| and the quantizer recomputes dX from preact and dy with
 *   the same arithmetic (so every output equals the dx != NULL call's).
 */
int32_t dswiglu_nvfp4_quant(const uint16_t* preact, const uint16_t* dy, int64_t tokens, int64_t ffn,
                            const int32_t* counts, int64_t num_experts,
                            uint16_t* dx, float* amax,
                            uint8_t* row_codes, uint8_t* row_scales, float* row_scale,
                            uint8_t* col_codes, uint8_t* col_scales, float* col_scale,
                            void* workspace, size_t workspace_bytes, void* stream);

/* dswiglu_nvfp4_quant with stochastic FC1-gradient codes: the same scales, each
 * rowwise and columnwise code the carry-form stochastic rounding of the same
 * quotient with word 0 of Philox4x32-10 (key = seed) at counter n: rowwise
 * element (row, col) n = counter_base + row*2*ffn + col; columnwise code n =
 * counter_base + tokens*2*ffn + its index in col_codes (two per byte, low
 * nibble first), i.e. + 2*ffn*poff_e + h*P_e + (g - poff_e).  sr_state:
 * DEVICE pointer to {seed, counter_base} (two uint64); other arguments as in
 * dswiglu_nvfp4_quant (dx may be NULL). */
int32_t dswiglu_nvfp4_quant_sr(const uint16_t* preact, const uint16_t* dy, int64_t tokens, int64_t ffn,
                               const int32_t* counts, int64_t num_experts,
                               uint16_t* dx, float* amax,
                               uint8_t* row_codes, uint8_t* row_scales, float* row_scale,
                               uint8_t* col_codes, uint8_t* col_scales, float* col_scale,
                               void* workspace, size_t workspace_bytes, const uint64_t* sr_state, void* stream);

/* dswiglu_nvfp4_quant_sr with the word-stream mapping of the pack's
 * EP_ROUND_SR_STREAM modes: the code at stream position n takes word (n & 3)
 * of Philox4x32-10 block n >> 2 (same key and positions).  Arguments, layouts
 * and errors as there. */
int32_t dswiglu_nvfp4_quant_sr_stream(const uint16_t* preact, const uint16_t* dy, int64_t tokens, int64_t ffn,
                                      const int32_t* counts, int64_t num_experts,
                                      uint16_t* dx, float* amax,
                                      uint8_t* row_codes, uint8_t* row_scales, float* row_scale,
                                      uint8_t* col_codes, uint8_t* col_scales, float* col_scale,
                                      void* workspace, size_t workspace_bytes, const uint64_t* sr_state,
                                      void* stream);

/* dswiglu_nvfp4_quant without the workspace argument, for callers that cannot
 * allocate (code under HIP graph capture, serving loops that forbid
 * hipMalloc).  The workspace lives in a static device array of
 * EP_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends; the library
 * allocates nothing on this path.  Sizes whose workspace
 * (dswiglu_workspace_bytes) exceeds it are refused with EP_ERR_SCRATCH before
 * anything is launched.  Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (other streams, other threads) race and
 * must be serialized by the caller.  Other arguments, layouts and results as
 * for dswiglu_nvfp4_quant. */
int32_t dswiglu_nvfp4_quant_noalloc(const uint16_t* preact, const uint16_t* dy, int64_t tokens, int64_t ffn,
                                    const int32_t* counts, int64_t num_experts, uint16_t* dx, float* amax,
                                    uint8_t* row_codes, uint8_t* row_scales, float* row_scale,
                                    uint8_t* col_codes, uint8_t* col_scales, float* col_scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_TOKEN_BLOCK_H */
