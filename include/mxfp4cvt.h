/*
 * mxfp4cvt.h -- C ABI of libmxfp4cvt: BF16 -> MXFP4 quantization and direct MXFP4 ->
 * block-scaled FP8 (E4M3) conversion, row and transposed-column layouts, over ragged
 * per-expert token segments, on AMD Instinct MI355X (gfx950).
 *
 * Method: "Practical FP4 Training for Large-Scale MoE Models on Hopper GPUs"
 * (technical summary, section 2 "Methodology"):
 *   item 1  MXFP4 = E2M1 elements (1 sign, 2 exponent, 1 mantissa bit) sharing one
 *           UE8M0 power-of-two scale per 32 elements; the FP8 target is E4M3 with
 *           128-element blocks, reached by a direct bitwise FP4 -> FP8 conversion
 *           (no BF16 intermediate) with hierarchical scale alignment to the
 *           largest of the four MX scales of a 128-block;
 *   item 2  activations are quantized right before the expert all-to-all and packed
 *           two codes per uint8;
 *   item 3  layout-aware kernels: row quantizer, row conversion (FPROP), column
 *           conversion with the transpose fused (Wgrad), ragged tensors without
 *           padding.
 * Conventions the page leaves open follow OCP MX v1.0: shared exponent
 * floor(log2 amax) - 2 (clamped to the UE8M0 range, 0 for an all-zero block), E2M1
 * round-to-nearest-even saturating at 6, E4M3FN (OCP, bias 7, no Inf) round-to-
 * nearest-even where a shift underflows, sign of zero kept, element 2i in the low
 * nibble of byte i.
 *
 * Common conventions of every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller.  The library
 *     allocates and frees nothing and keeps no state; calls are thread-safe.
 *   - Work is enqueued on `stream` and the call returns at once (no host sync, the
 *     offsets are never read on the host).
 *   - group_offsets: int32 [G+1] on the device, offs[0] = 0, non-decreasing,
 *     offs[G] = M_tot <= M_cap.  Expert g owns rows [offs[g], offs[g+1]).  These
 *     are preconditions (not checked; mxfp4_validate_offsets checks them with a
 *     host sync).  Rows [M_tot, M_cap) of every output are left untouched, so a
 *     capacity-sized launch needs no host knowledge of M_tot.
 *   - Arguments are validated before anything is enqueued; on any error nothing is
 *     enqueued:  NULL array pointer -> MXFP4_ERR_NULL;  G < 1, M_cap < 0, K <= 0,
 *     K not a multiple of 32 (quantize) or 128 (conversions), or sizes whose byte
 *     counts overflow int64 -> MXFP4_ERR_SHAPE;  an array pointer not 16-byte aligned
 *     (group_offsets: 4-byte) -> MXFP4_ERR_ALIGN.  A failed kernel launch ->
 *     MXFP4_ERR_HIP.
 *   - Outputs must not alias inputs.
 *   - UE8M0 scale bytes decode as 2^(b - 127); b = 0 is 2^-127 (an fp32 subnormal).
 */
#ifndef MXFP4CVT_H
#define MXFP4CVT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MXFP4_OK = 0,
    MXFP4_ERR_NULL = 1,
    MXFP4_ERR_SHAPE = 2,
    MXFP4_ERR_ALIGN = 3,
    MXFP4_ERR_HIP = 4
} mxfp4_status;

/* BF16 -> MXFP4 (the page's BF16ToFP4Row; technical summary section 2, items 1-2).
 *   x_bf16  [M_cap, K] row-major BF16 bits (finite values).
 *   codes   [M_cap, K/2]  E2M1 codes, element 2i in the low nibble of byte i.
 *   scales  [M_cap, K/32] UE8M0 bytes: floor(log2 amax) - 2 + 127 clamped to [0, 254].
 *   Rows [0, offs[G]) are written.  K must be a multiple of 32. */
mxfp4_status mxfp4_quantize_rows(const uint16_t* x_bf16, uint8_t* codes, uint8_t* scales,
                                 const int32_t* group_offsets, int32_t G, int64_t M_cap,
                                 int64_t K, hipStream_t stream);

/* BF16 -> NVFP4, the variant format of the NVFP4 recipe page ("Train models faster with
 * JAX and MaxText using NVFP4 on NVIDIA Blackwell": 16-element microblocks, E4M3 block
 * scales under one FP32 scale per tensor, nearest-even rounding for activations).
 *   x_bf16       [M_cap, K] row-major BF16 bits (finite values).
 *   codes        [M_cap, K/2]  E2M1 codes, element 2i in the low nibble of byte i.
 *   scales_e4m3  [M_cap, K/16] E4M3FN block scale bytes.
 *   tensor_amax  one float (device): max |x| over rows [0, offs[G]), 0 if there are none.
 *   With t = FP32(2688 / amax) (1 for amax 0, FLT_MAX if the quotient overflows), each
 *   16-element block with largest magnitude amax_b has scale S = E4M3(FP32(FP32(amax_b/6)
 *   * t)) (nearest even, subnormals, saturating at 448), and each element the code
 *   E2M1(FP32(x * FP32(t / S))) (nearest even, saturating at 6, sign kept; 0 codes where
 *   S is 0); it decodes as E2M1(code) * E4M3(S) / t.
 *   Rows [0, offs[G]) are written; tensor_amax is written even when there are none.
 *   K must be a multiple of 16.  Three launches on the stream (amax reset, tensor amax,
 *   quantize); calls that share tensor_amax must not overlap. */
mxfp4_status mxfp4_nvfp4_quantize_rows(const uint16_t* x_bf16, uint8_t* codes, uint8_t* scales_e4m3,
                                       float* tensor_amax, const int32_t* group_offsets, int32_t G,
                                       int64_t M_cap, int64_t K, hipStream_t stream);

/* BF16 -> NVFP4 with stochastic rounding of the element codes: the NVFP4 recipe page
 * rounds its gradient quantizers stochastically to keep small updates unbiased.  The
 * arguments, block scales, tensor amax, errors and launches are mxfp4_nvfp4_quantize_rows';
 * only the element codes differ.  With y = FP32(x * FP32(t / S)) as there: |y| >= 6 gives
 * the code of 6; otherwise, between the E2M1 values lo <= |y| < hi, the code of hi when
 * r < 65536 (|y| - lo) / (hi - lo) and of lo else (sign of x kept).  r is 16 random bits
 * from Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
 * 1, 2, 3", SC'11) under key (seed & 0xFFFFFFFF, seed >> 32): element (m, k), numbered
 * n = m K + k from row 0 of x, takes half n % 2 (0: the low 16 bits) of output word
 * (n % 8) / 2 of the call on counter (n / 8 low word, high word, 0, 0).  The same seed
 * gives the same codes; callers pass a new seed per step. */
mxfp4_status mxfp4_nvfp4_quantize_rows_sr(const uint16_t* x_bf16, uint8_t* codes, uint8_t* scales_e4m3,
                                          float* tensor_amax, const int32_t* group_offsets, int32_t G,
                                          int64_t M_cap, int64_t K, uint64_t seed, hipStream_t stream);

/* MXFP4 -> FP8 E4M3FN, row layout for FPROP (the page's FP4RowToFP8Row; technical
 * summary section 2, item 1, hierarchical scale alignment).
 *   codes, scales  as produced by mxfp4_quantize_rows.
 *   y_e4m3    [M_cap, K]     E4M3FN bytes: e2m1(c) * 2^(s - S) rounded to nearest even.
 *   y_scales  [M_cap, K/128] UE8M0 bytes S = max of the four MX scales of the block.
 *   Rows [0, offs[G]) are written.  K must be a multiple of 128. */
mxfp4_status mxfp4_to_fp8_rows(const uint8_t* codes, const uint8_t* scales, uint8_t* y_e4m3,
                               uint8_t* y_scales, const int32_t* group_offsets, int32_t G,
                               int64_t M_cap, int64_t K, hipStream_t stream);

/* MXFP4 -> FP8 E4M3FN, transposed column layout per expert for Wgrad (the page's
 * FP4RowToFP8Col; technical summary section 2, item 3: transpose fused, ragged, no
 * padding).  With M_g = offs[g+1] - offs[g], nb_g = ceil(M_g / 128) and
 * B_g = nb_0 + ... + nb_{g-1}:
 *   yT_e4m3    expert g: [K, M_g] at byte K*offs[g], element (k, m') at k*M_g + m'
 *              (m' = row - offs[g]); capacity K*M_cap bytes.
 *   yT_scales  expert g: [nb_g, K] at byte K*B_g; entry (b, k) = max of the MX
 *              scales of group k/32 over the rows of block b that exist (a partial
 *              last block uses only its rows); capacity
 *              mxfp4_cols_scale_capacity(M_cap, K, G) bytes.
 *   Element (k, m') = e2m1(c) * 2^(s - S) rounded to nearest even, s the row's own
 *   MX scale.  Bytes past each expert's M_g (and past offs[G]) are not written.
 *   K must be a multiple of 128 and at most 2^24 (larger K -> MXFP4_ERR_SHAPE). */
mxfp4_status mxfp4_to_fp8_cols_ragged(const uint8_t* codes, const uint8_t* scales,
                                      uint8_t* yT_e4m3, uint8_t* yT_scales,
                                      const int32_t* group_offsets, int32_t G, int64_t M_cap,
                                      int64_t K, hipStream_t stream);

/* BF16 -> FP8 E4M3FN with one UE8M0 scale per 1x128 block along the row: the
 * backward quantizer for gradients (DGRAD operand; technical summary section 2,
 * item 2: the backward pass stays on the standard FP8 path, E4M3 with 128-element
 * blocks as in item 1).
 *   x_bf16    [M_cap, K] row-major BF16 bits (finite values).
 *   y_e4m3    [M_cap, K]     E4M3FN bytes: x / 2^(S-127) rounded to nearest even,
 *             subnormals included, magnitudes above 448 saturated to 448, sign kept.
 *   y_scales  [M_cap, K/128] UE8M0 bytes S = floor(log2 amax) - 8 + 127 clamped to
 *             [0, 254] (8 = E4M3's largest exponent), 0 for an all-zero block.
 *   Rows [0, offs[G]) are written.  K must be a multiple of 128. */
mxfp4_status mxfp4_bf16_to_fp8_rows(const uint16_t* x_bf16, uint8_t* y_e4m3, uint8_t* y_scales,
                                    const int32_t* group_offsets, int32_t G, int64_t M_cap,
                                    int64_t K, hipStream_t stream);

/* BF16 -> FP8 E4M3FN in the transposed column layout per expert, one UE8M0 scale per
 * 1x128 block along the tokens: the backward quantizer for the Wgrad gradient operand
 * (technical summary section 2, item 2: backward pass on the FP8 path, E4M3 with
 * 128-element blocks as in item 1; item 3: per-expert transpose over ragged segments
 * without padding).  With M_g = offs[g+1] - offs[g], nb_g = ceil(M_g / 128) and
 * B_g = nb_0 + ... + nb_{g-1}:
 *   x_bf16     [M_cap, K] row-major BF16 bits (finite values).
 *   yT_e4m3    expert g: [K, M_g] at byte K*offs[g], element (k, m') at k*M_g + m';
 *              capacity K*M_cap bytes.  Element = x / 2^(S-127) rounded to nearest
 *              even (subnormals included), magnitudes above 448 saturated, sign kept.
 *   yT_scales  expert g: [nb_g, K] at byte K*B_g; entry (b, k) = S = floor(log2 amax)
 *              - 8 + 127 clamped to [0, 254] (0 for an all-zero block), amax over the
 *              rows of block b that exist (a partial last block uses only its rows);
 *              capacity mxfp4_cols_scale_capacity(M_cap, K, G) bytes.
 *   Bytes past each expert's M_g (and past offs[G]) are not written.
 *   K must be a multiple of 128 and at most 2^24 (larger K -> MXFP4_ERR_SHAPE). */
mxfp4_status mxfp4_bf16_to_fp8_cols_ragged(const uint16_t* x_bf16, uint8_t* yT_e4m3,
                                           uint8_t* yT_scales, const int32_t* group_offsets,
                                           int32_t G, int64_t M_cap, int64_t K,
                                           hipStream_t stream);

/* The backward FP8 quantizer in both layouts from one read of the gradient (technical
 * summary section 2, item 2: the backward pass runs in FP8; DGRAD takes the row layout and
 * WGRAD the transposed column layout of the same gradient).  Writes exactly what
 * mxfp4_bf16_to_fp8_rows writes to y_e4m3 / y_scales and what
 * mxfp4_bf16_to_fp8_cols_ragged writes to yT_e4m3 / yT_scales, with the same layouts,
 * capacities and untouched bytes, reading x once.
 *   K must be a multiple of 128 and at most 2^24 (else MXFP4_ERR_SHAPE). */
mxfp4_status mxfp4_bf16_to_fp8_rows_cols_ragged(const uint16_t* x_bf16, uint8_t* y_e4m3, uint8_t* y_scales,
                                                uint8_t* yT_e4m3, uint8_t* yT_scales,
                                                const int32_t* group_offsets, int32_t G, int64_t M_cap,
                                                int64_t K, hipStream_t stream);

/* Expert-grouped FP8 GEMM, forward (technical summary section 2: compute stays FP8 on
 * the block-scaled pipeline, E4M3 with 128-element blocks, item 1; it consumes the row
 * layout FP8 activations).  For the expert g owning row m (offs[g] <= m < offs[g+1]):
 *   y[m, n] = bf16( sum_k A[m,k] 2^(sA[m,k/128]-127) * W[g,n,k] 2^(sW[g,n,k/128]-127) )
 *   a_e4m3    [M_cap, K]     E4M3FN activations (e.g. mxfp4_to_fp8_rows output).
 *   a_scales  [M_cap, K/128] UE8M0.
 *   w_e4m3    [G, N, K]      E4M3FN weights, one [N, K] matrix per expert.
 *   w_scales  [G, N, K/128]  UE8M0 (a 128x128-block weight scale is this format with
 *             the scale repeated over its 128 rows).
 *   y_bf16    [M_cap, N]     BF16 bits; rows [offs[G], M_cap) are not written.
 *   The sum is accumulated in fp32 by the matrix cores (the precision of each 64-term
 *   dot product inside them is the hardware's) and rounded once to BF16 (nearest even).
 *   K must be a multiple of 128 and at most 2^20, N a multiple of 256 and at most 2^20
 *   (else MXFP4_ERR_SHAPE).  No NaN bytes (0x7F / 0xFF) in the operands. */
mxfp4_status mxfp4_fp8_grouped_gemm(const uint8_t* a_e4m3, const uint8_t* a_scales,
                                    const uint8_t* w_e4m3, const uint8_t* w_scales,
                                    uint16_t* y_bf16, const int32_t* group_offsets, int32_t G,
                                    int64_t M_cap, int64_t N, int64_t K, hipStream_t stream);

/* Expert-grouped FP8 GEMM, weight gradient (technical summary section 2: compute stays
 * FP8 on the block-scaled pipeline, item 1; the column conversion fuses the transpose
 * into the Wgrad operands over ragged experts with no padding, item 3).  For expert g
 * with M_g = offs[g+1] - offs[g] tokens, B_g = the 128-token blocks of the experts
 * before it, and b = m / 128:
 *   dW[g, n, k] = bf16( sum_{m < M_g} dY_g[m, n] 2^(sdy_g[b, n]-127) * X_g[m, k] 2^(sx_g[b, k]-127) )
 *   dyT_e4m3    column layout for width N, as mxfp4_bf16_to_fp8_cols_ragged writes it
 *               for a gradient [M_cap, N]: expert g [N, M_g] at byte N*offs[g];
 *               capacity N*M_cap bytes.
 *   dyT_scales  [nb_g, N] at byte N*B_g; capacity mxfp4_cols_scale_capacity(M_cap, N, G).
 *   xT_e4m3     the same layout for width K, as mxfp4_to_fp8_cols_ragged writes it for
 *               the activations [M_cap, K]; capacity K*M_cap bytes.
 *   xT_scales   [nb_g, K] at byte K*B_g; capacity mxfp4_cols_scale_capacity(M_cap, K, G).
 *   dw_bf16     [G, N, K] BF16 bits; every element is written (0 for an expert with no
 *               tokens, also when M_cap == 0).
 *   Accumulation and rounding as in mxfp4_fp8_grouped_gemm.  Reads stay within the
 *   stated capacities.  N and K must be multiples of 256 and at most 2^20, and N*M_cap
 *   and K*M_cap at most 2^30 (else MXFP4_ERR_SHAPE).  No NaN bytes in the operands. */
mxfp4_status mxfp4_fp8_grouped_gemm_wgrad(const uint8_t* dyT_e4m3, const uint8_t* dyT_scales,
                                          const uint8_t* xT_e4m3, const uint8_t* xT_scales,
                                          uint16_t* dw_bf16, const int32_t* group_offsets, int32_t G,
                                          int64_t M_cap, int64_t N, int64_t K, hipStream_t stream);

/* Bytes the column-layout scale buffer needs for any offsets with offs[G] <= M_cap:
 * K * (ceil(M_cap / 128) + G).  Returns -1 for invalid sizes. */
int64_t mxfp4_cols_scale_capacity(int64_t M_cap, int64_t K, int32_t G);

/* Debug helper: copies the G+1 offsets to the host (synchronizing `stream`) and
 * checks offs[0] == 0, non-decreasing, offs[G] <= M_cap.  MXFP4_OK if they hold,
 * MXFP4_ERR_SHAPE if not, MXFP4_ERR_NULL / MXFP4_ERR_HIP as usual.  With valid
 * offsets it also returns MXFP4_ERR_HIP while the current device's wait status (see
 * mxfp4_wait_status) is set; it does not clear it. */
mxfp4_status mxfp4_validate_offsets(const int32_t* group_offsets, int32_t G, int64_t M_cap,
                                    hipStream_t stream);

/* Not an operation of the method: the failure report of the column conversions
 * (mxfp4_to_fp8_cols_ragged, mxfp4_bf16_to_fp8_cols_ragged,
 * mxfp4_bf16_to_fp8_rows_cols_ragged).  Their waves hand strips to one another through
 * counters, and every wait for a counter is bounded: a wave that polls a counter the
 * wait limit's number of times without seeing it advance gives up, sets the current
 * device's wait status (one word per device, shared by every stream and call on it)
 * and leaves the kernel, so the call ends with part of its output unwritten instead of
 * hanging the GPU.  Only a protocol fault (or a limit set far too low) makes a wave give
 * up; the default limit is 2^24 polls, about a second.
 * mxfp4_wait_status synchronizes `stream`, then reports MXFP4_ERR_HIP if the status is
 * set (and clears it) or MXFP4_OK if not; a HIP failure also gives MXFP4_ERR_HIP.  It
 * sees every give-up of work finished before it; a kernel still running on another
 * stream may set the status after the check. */
mxfp4_status mxfp4_wait_status(hipStream_t stream);

/* Test hook for the give-up path: the polls each bounded wait of a column conversion
 * makes before it gives up, for launches made after this call by any thread of the
 * process; 0 restores the default (2^24).  A tiny limit makes waves give up early (each
 * still leaves the kernel normally) and the call's output incomplete. */
void mxfp4_set_wait_limit(uint32_t polls);

/* Measurement hook: binds two caller-created HIP events (hipEventCreate, owned by the
 * caller) to the kernel launches of the calling thread's next entry-point call: `start`
 * to its first kernel and `stop` to its last (hipExtLaunchKernel), so that
 * hipEventElapsedTime(start, stop) is the kernels' own execution time, with no marker
 * commands of their own on the stream.  The events are used once and then dropped; a
 * call that launches nothing (an argument error, M_cap = 0) leaves them armed, and
 * NULL, NULL disarms.  Either may be NULL.  Calls on other threads are not affected.
 * Returns MXFP4_OK. */
mxfp4_status mxfp4_time_next_launch(hipEvent_t start, hipEvent_t stop);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char* mxfp4_status_string(mxfp4_status status);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4CVT_H */
