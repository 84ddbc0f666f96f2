/*
 * nvfp4moe.h - C ABI of the MI355X (gfx950) NVFP4 W4A4 MoE hot-path library.
 *
 * The operations are the kernels the miniTE pages describe for native NVFP4
 * (W4A4) training of Qwen3-30B-A3B:
 *   - "miniTE NVFP4" blog (yuxiaoba.github.io), section "Two complementary
 *     interventions": contiguous buffers with device-side metadata instead of
 *     per-expert splitting and repacking; amax computed during permutation or
 *     during the weighted SwiGLU so no extra scan is needed; scale-layout
 *     conversion fused with quantisation; forward and backward precision are
 *     independent choices.  Same page, "Follow the numerical execution path":
 *     per-token scaling, and identities of tokens and experts kept so results
 *     can be compared after alignment.
 *   - "miniTE accélère le RL en NVFP4 sur B300" (news.hamidun.com), section
 *     "Diagnostic, alignement et noyaux rapides": optimised NVFP4 kernels,
 *     scaling scheme and grouped GEMMs for MoE.
 *
 * NVFP4 storage used throughout (row-major, one row = one token or one
 * weight output row, K = row length, K % 16 == 0):
 *   codes   uint8 [rows][K/2]   E2M1 codes, element 2i in the low nibble of byte i
 *   bscales uint8 [rows][K/16]  E4M3fn scale of each block of 16 elements
 *   rscales float [rows]        FP32 second-level scale of the row
 *   value(r, i) = e2m1(code) * e4m3(bscale[r][i/16]) * rscale[r]
 * Quantisation of a row:  s = amax / 2688 (FP32 division; 2688 = 6 * 448);
 * b_j = E4M3(blockamax_j / (6 * s)) (nearest-even, saturating at 448; 0 if
 * s == 0); d_j = b_j * s; code_i = E2M1(x_i / d_j) (nearest, ties to the even
 * grid index, saturating at 6, sign kept; a signed zero if d_j == 0).  All
 * steps are IEEE FP32 operations without fused multiply-add, so results are
 * bit-reproducible.
 *
 * Conventions for every entry point:
 *   - All pointers are DEVICE pointers owned by the caller (the library never
 *     allocates or frees), except where a parameter says otherwise.  Tensors
 *     must be contiguous in the stated layout.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued; nothing waits on the device and nothing reads device memory
 *     on the host.
 *   - Arguments are checked on the host before anything is enqueued; a check
 *     failure returns a non-zero nvfp4_status and enqueues nothing.
 *   - Routed rows: a routing of T tokens to k of E experts gives R = T*k
 *     routed rows, grouped by expert; expert_offsets[E+1] (device, int32)
 *     holds the first row of each expert and the total number of routed rows
 *     in expert_offsets[E].  Buffers sized for R_cap = T*k rows are always
 *     enough; rows at or beyond expert_offsets[E] are neither read nor written.
 *   - dev_err (optional device int32, may be NULL): bit 0 is OR-ed in on the
 *     device when a routing entry names an expert outside [0, E).  Such an
 *     entry takes no row (tk_to_row = -1) and is skipped by every later step.
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4MOE_API __attribute__((visibility("default")))
#define NVFP4MOE_ABI_VERSION 2
#define NVFP4MOE_MAX_K 8192      /* longest quantised row */
#define NVFP4MOE_MAX_EXPERTS 1024
#define NVFP4MOE_MAX_TOPK 32
#define NVFP4MOE_NOALLOC_MAX_ENTRIES (1 << 20)   /* T * k limit of nvfp4_quantize_permute_noalloc */

typedef enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,      /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,     /* a size is out of range (K % 16 != 0, k > E, <= 0, too large) */
  NVFP4_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
  NVFP4_ERR_WORKSPACE = 4, /* workspace smaller than required */
  NVFP4_ERR_LAUNCH = 5,    /* the HIP runtime reported an error when enqueuing */
  NVFP4_ERR_ARG = 6,       /* an enumerated argument has an unknown value, or an output aliases an input */
  NVFP4_ERR_SCRATCH = 7    /* the problem exceeds the fixed device scratch of an allocation-free entry point */
} nvfp4_status;

#define NVFP4_DEVERR_BAD_EXPERT 1   /* an expert id outside [0, E): that entry takes no row */

/* Text for a status code (static storage, never NULL). */
NVFP4MOE_API const char* nvfp4moe_status_string(int status);

/* NVFP4MOE_ABI_VERSION of the built library. */
NVFP4MOE_API int nvfp4moe_abi_version(void);

/* Bytes of device workspace nvfp4_quantize_permute needs for T tokens, top-k, E experts
 * (0 for invalid sizes). */
NVFP4MOE_API size_t nvfp4moe_permute_workspace_size(int64_t T, int32_t k, int32_t E);

/*
 * nvfp4moe_workspace_size - device workspace bytes an operation needs, keyed by
 * the operation.  Only the route + permute + quantise pass uses a workspace
 * (its per-(chunk, expert) count table and one rank per routing entry); every
 * other operation enqueues kernels on caller buffers alone and returns 0.
 *   op     NVFP4MOE_OP_* below
 *   T, E, k: tokens, experts, top-k of the routing (NVFP4MOE_OP_QUANTIZE_PERMUTE)
 *   R_max, N: routed-row capacity and output width (GEMMs; unused, 0 is returned)
 * Returns (size_t)-1 for an unknown op, 0 where no workspace is needed or the
 * sizes are invalid.
 */
#define NVFP4MOE_OP_QUANTIZE_PERMUTE 0
#define NVFP4MOE_OP_QUANTIZE_ROWS 1
#define NVFP4MOE_OP_GROUPED_GEMM 2
#define NVFP4MOE_OP_SWIGLU_QUANTIZE 3
#define NVFP4MOE_OP_UNPERMUTE_COMBINE 4
#define NVFP4MOE_OP_BF16_GROUPED_GEMM 5
#define NVFP4MOE_OP_SWIGLU_BACKWARD 6
#define NVFP4MOE_OP_GROUPED_GEMM_SWIGLU 7   /* R_max * 4 bytes (router weight per row) */
NVFP4MOE_API size_t nvfp4moe_workspace_size(int32_t op, int64_t T, int32_t E, int32_t k,
                                            int64_t R_max, int64_t N);

/*
 * Byte offsets of a row's NVFP4 block scale and element code in the two
 * storage layouts (host functions, no device access).  The "scale-layout
 * conversion fused into quantisation" of the blog "miniTE NVFP4" (section "Two
 * complementary interventions") is the quantiser writing the layout the GEMM
 * reads; these functions name where each byte of that layout lives.
 *   group_rows = 0: row-major, bscales [rows][K/16], codes [rows][K/2];
 *   group_rows = G > 0: K-tiled groups of G rows (nvfp4_quantize_rows_tiled),
 *     bscales [rows/G][K/64][G][4], codes [rows/G][K/64][G][32].
 * nvfp4moe_bscale_index: the byte of block kb (elements 16 kb .. 16 kb + 15) of
 * row r.  nvfp4moe_code_index: the byte holding element i of row r (low nibble
 * for even i, high nibble for odd i).  Requires K % 16 == 0 (row-major) or
 * K % 64 == 0 (K-tiled), 0 <= kb < K/16, 0 <= i < K, r >= 0; returns -1 otherwise.
 */
NVFP4MOE_API int64_t nvfp4moe_bscale_index(int64_t r, int64_t kb, int64_t K, int64_t group_rows);
NVFP4MOE_API int64_t nvfp4moe_code_index(int64_t r, int64_t i, int64_t K, int64_t group_rows);

/*
 * nvfp4_quantize_rows - NVFP4-quantise `rows` bf16 rows of length K, each with
 * its own FP32 scale (per-token scaling; per output row for weights).
 *   x        bf16 bits [rows][K]
 *   codes    out [rows][K/2]; bscales out [rows][K/16]; rscales out [rows]
 * Requires 1 <= K <= NVFP4MOE_MAX_K, K % 16 == 0, rows >= 0, x 16-byte aligned.
 */
NVFP4MOE_API int nvfp4_quantize_rows(const uint16_t* x, int64_t rows, int64_t K,
                                     uint8_t* codes, uint8_t* bscales, float* rscales,
                                     void* stream);

/*
 * nvfp4_quantize_rows_tiled - the same quantisation as nvfp4_quantize_rows,
 * written in the K-tiled layout that the grouped GEMM reads one contiguous
 * block per K-step from (the scale layout conversion done by the quantiser
 * itself; miniTE blog, "Two complementary interventions"):
 *   codes   [rows/G][K/64][G][32]: byte b of slab kc of row r holds elements
 *           64 kc + 2b (low nibble) and 64 kc + 2b + 1 of the row;
 *   bscales [rows/G][K/64][G][4]:  the 4 block scales of slab kc;
 *   rscales [rows] as in nvfp4_quantize_rows;
 * with G = group_rows (for expert weights [E][N][K]: G = N).  Exactly the bytes
 * of nvfp4_quantize_rows, moved.
 * Requires K % 64 == 0, K <= NVFP4MOE_MAX_K, group_rows > 0, rows % group_rows == 0.
 */
NVFP4MOE_API int nvfp4_quantize_rows_tiled(const uint16_t* x, int64_t rows, int64_t K,
                                           int64_t group_rows, uint8_t* codes,
                                           uint8_t* bscales, float* rscales, void* stream);

/*
 * nvfp4_quantize_permute - route, permute and quantise MoE activations in one
 * pass over x (the token amax is taken while the token is read for the
 * permutation).
 *   x          bf16 bits [T][H]
 *   topk_ids   int32 [T][k], expert of each (token, slot)
 * Outputs (all device, caller-allocated):
 *   expert_offsets int32 [E+1]: first row of each expert, [E] = routed rows
 *   tk_to_row      int32 [T*k]: row of (t, slot) at index t*k+slot, or -1
 *   row_to_tk      int32 [T*k]: t*k+slot of each routed row (rows < offsets[E])
 *   codes [T*k][H/2], bscales [T*k][H/16], rscales [T*k]: the NVFP4 rows of the
 *     expert-grouped buffer; row(t, slot) holds token t's quantisation (the
 *     same bytes for all k slots of a token).
 * Row order: rows are grouped by expert id; inside an expert they follow
 * (token, slot) order (a stable counting sort of the routing list).
 * Workspace: `workspace` must hold nvfp4moe_permute_workspace_size(T, k, E)
 * bytes (device memory; contents need not be initialised).  Calls that share
 * one workspace must be ordered (same stream, or synchronised): overlapping
 * calls on one workspace race.
 * Requires 1 <= k <= min(E, NVFP4MOE_MAX_TOPK), 1 <= E <= NVFP4MOE_MAX_EXPERTS,
 * H % 16 == 0, H <= NVFP4MOE_MAX_K, T * k <= INT32_MAX / 2.  k = 1, E = 1 with ids all 0 is a plain
 * per-token quantisation (dense projections).
 */
NVFP4MOE_API int nvfp4_quantize_permute(const uint16_t* x, int64_t T, int64_t H,
                                        const int32_t* topk_ids, int32_t k, int32_t E,
                                        uint8_t* codes, uint8_t* bscales, float* rscales,
                                        int32_t* expert_offsets, int32_t* row_to_tk,
                                        int32_t* tk_to_row, void* workspace,
                                        size_t workspace_bytes, int32_t* dev_err,
                                        void* stream);

/*
 * nvfp4_quantize_permute_noalloc - nvfp4_quantize_permute without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * workspace is a device array inside the library sized for
 * T * k <= NVFP4MOE_NOALLOC_MAX_ENTRIES routing entries and up to
 * NVFP4MOE_MAX_EXPERTS experts (5.2 MB, held by every device the library runs
 * on until the process ends); its device address is looked up on the first
 * call on each device.  This entry point allocates nothing and calls no
 * allocating routine.  Arguments, outputs, row order and errors are those of
 * nvfp4_quantize_permute; T * k above NVFP4MOE_NOALLOC_MAX_ENTRIES returns
 * NVFP4_ERR_SCRATCH and enqueues nothing.  Every call on one device shares
 * that device's scratch (each call writes what it reads, so nothing carries
 * over between calls): calls that overlap in time on one device (different
 * streams, no ordering between them) race and give wrong results.
 */
NVFP4MOE_API int nvfp4_quantize_permute_noalloc(const uint16_t* x, int64_t T, int64_t H,
                                                const int32_t* topk_ids, int32_t k, int32_t E,
                                                uint8_t* codes, uint8_t* bscales, float* rscales,
                                                int32_t* expert_offsets, int32_t* row_to_tk,
                                                int32_t* tk_to_row, int32_t* dev_err,
                                                void* stream);

/*
 * nvfp4_grouped_gemm - grouped W4A4 expert GEMM on the expert-grouped buffer:
 * for every expert e and row r in [offsets[e], offsets[e+1]):
 *     c[r][n] = sum_k value_A(r, k) * value_W(e, n, k)        (C = A W_e^T)
 * Elements are decoded exactly (e2m1 * e4m3 fits FP16) and multiplied on the
 * matrix cores with FP32 accumulation; the two FP32 row scales are applied in
 * the epilogue.  Error per element is within 2e-5 * sum_k |a_k w_k|.
 *   A (activations): a_codes [R_cap][K/2], a_bscales [R_cap][K/16], a_rscales [R_cap]
 *   W (weights), w_layout NVFP4_W_ROWMAJOR: w_codes [E][N][K/2], w_bscales [E][N][K/16];
 *                w_layout NVFP4_W_KTILED:   w_codes [E][K/64][N][32], w_bscales [E][K/64][N][4]
 *                (nvfp4_quantize_rows_tiled with group_rows = N); w_rscales [E][N]
 *   c                [R_cap][N] of c_dtype: NVFP4_OUT_F32 (float) or NVFP4_OUT_BF16
 *                    (bf16 bits, each FP32 result rounded to nearest even; halves the
 *                    output bytes, at 2^-9 relative error on top of the bound above);
 *                    only rows < expert_offsets[E] are written
 * E = 1 with expert_offsets = {0, M} is a dense GEMM of M rows.  The list of
 * (expert, row block, column block) tiles is derived on the device from
 * expert_offsets by every workgroup (no tile list argument).
 * expert_offsets are read as nvfp4_quantize_permute writes them (non-decreasing,
 * expert_offsets[E] <= R_cap); the kernel clamps each into [0, R_cap], so other
 * values give wrong rows but no access outside the buffers.
 * Requires K % 64 == 0, N % 16 == 0, 16 <= N <= 2^20, K <= 65536, all pointers
 * 16-byte aligned.  Unknown w_layout or c_dtype: NVFP4_ERR_ARG.
 */
#define NVFP4_W_ROWMAJOR 0
#define NVFP4_W_KTILED 1
#define NVFP4_OUT_F32 0
#define NVFP4_OUT_BF16 1
NVFP4MOE_API int nvfp4_grouped_gemm(const uint8_t* a_codes, const uint8_t* a_bscales,
                                    const float* a_rscales, const int32_t* expert_offsets,
                                    int32_t E, int64_t R_cap, const uint8_t* w_codes,
                                    const uint8_t* w_bscales, const float* w_rscales,
                                    int64_t N, int64_t K, int32_t w_layout, void* c,
                                    int32_t c_dtype, void* stream);

/*
 * nvfp4_grouped_gemm_swiglu - the gate_up grouped GEMM with the weighted SwiGLU
 * in its epilogue (the blog "miniTE NVFP4", section "Two complementary
 * interventions", takes the amax during the weighted SwiGLU; here the SwiGLU
 * itself moves into the GEMM that produces its input, so the gate_up output
 * need not make a round trip through memory).  For every routed row r of
 * expert e and h column j in [0, I):
 *     g = C[r][j], u = C[r][I + j]  (C = A W_e^T as nvfp4_grouped_gemm computes it, FP32)
 *     h[r][j] = (silu(g) * u) * w_r,  silu(g) = g / (1 + exp(-g)),  in FP32
 * with w_r = topk_w[row_to_tk[r]] (1 when topk_w is NULL).  exp and the
 * division are the hardware exp2 of -g log2(e) and reciprocal: h lies within
 * 2^-20 |h64| + 2^-24 max_row |h64| of the float64 value h64 of the same g and u.  Quantise h with nvfp4_quantize_rows_f32
 * (its amax is taken while it reads h).
 *   A, expert_offsets, E, R_cap, K: as nvfp4_grouped_gemm
 *   W: K-tiled only, w_codes [E][K/64][2I][32], w_bscales [E][K/64][2I][4],
 *      w_rscales [E][2I]: gate rows [0, I), up rows [I, 2I)
 *   h    float [R_cap][I]
 *   gu   float [R_cap][2I] or NULL: the plain GEMM's output (bit-identical to
 *        nvfp4_grouped_gemm's), for a backward pass that needs g and u
 *   workspace: nvfp4moe_workspace_size(NVFP4MOE_OP_GROUPED_GEMM_SWIGLU, ..., R_max = R_cap, ...)
 *        bytes when topk_w is given (may be NULL otherwise)
 * Requires I % 256 == 0, 256 <= I <= 2^19, K % 64 == 0, K <= 65536.
 */
NVFP4MOE_API int nvfp4_grouped_gemm_swiglu(const uint8_t* a_codes, const uint8_t* a_bscales,
                                           const float* a_rscales, const int32_t* expert_offsets,
                                           int32_t E, int64_t R_cap, const uint8_t* w_codes,
                                           const uint8_t* w_bscales, const float* w_rscales,
                                           int64_t I, int64_t K, const float* topk_w,
                                           const int32_t* row_to_tk, float* h, float* gu,
                                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_quantize_rows_f32 - the NVFP4 row quantisation of FP32 rows (the
 * definition at the top of this header, on FP32 inputs): rows
 * [0, min(expert_offsets[E], rows)) when expert_offsets is given, else all rows.
 *   x float [rows][K]; codes [rows][K/2]; bscales [rows][K/16]; rscales [rows]
 * Requires K % 16 == 0, K <= NVFP4MOE_MAX_K.
 */
NVFP4MOE_API int nvfp4_quantize_rows_f32(const float* x, int64_t rows, int64_t K,
                                         const int32_t* expert_offsets, int32_t E, uint8_t* codes,
                                         uint8_t* bscales, float* rscales, void* stream);

/*
 * The expert weight gradient in NVFP4, quantised along tokens (the blog "miniTE
 * NVFP4", section "Two complementary interventions": the backward's precision
 * is chosen independently of the forward's; a lower-bit backward is not
 * automatically faster).  For expert e with rows [offsets[e], offsets[e+1]):
 *     dW_e[m][n] = sum over its rows r of  G[r][m] * X[r][n]
 * (G the output gradient of the expert GEMM, X its input).  Both operands are
 * quantised along the contraction, i.e. along the expert's tokens: the slab
 * X_e^T [C][K_e] (K_e = the expert's rows rounded up to a multiple of 64, at
 * least 64, extra tokens zero) is quantised row by row with the definition at
 * the top of this header (one FP32 scale per (expert, channel), one E4M3 scale
 * per 16 tokens).  The slabs of all experts sit side by side along K: expert
 * e's tokens are K positions [64 kofs[e], 64 kofs[e+1]).
 *
 * nvfp4moe_token_blocks - kofs[E+1] (device int32) from expert_offsets: each
 * expert takes max(1, ceil(rows / 64)) steps of 64 tokens; kofs[E] <= R/64 + E.
 *
 * nvfp4_quantize_tokens - the slabs of all experts.
 *   x        [x_rows][C] of x_dtype (NVFP4_IN_BF16 bits or NVFP4_IN_F32)
 *   row_to_tk, k: if given, row r of the expert-grouped order is x row
 *            row_to_tk[r] / k (token order input, e.g. the output gradient);
 *            NULL: x is already in the expert-grouped order
 *   expert_offsets [E+1], kofs [E+1] (nvfp4moe_token_blocks)
 *   Kp       K capacity (positions) of the outputs, a multiple of 64 and at
 *            least 64 kofs[E]; 64 (ceil(R / 64) + E) always suffices
 *   layout   NVFP4_W_ROWMAJOR: codes [C][Kp/2], bscales [C][Kp/16] (the
 *            activation side of nvfp4_grouped_gemm_wgrad);
 *            NVFP4_W_KTILED:   codes [Kp/64][C][32], bscales [Kp/64][C][4] (its
 *            weight side)
 *   rscales  float [E][C]
 * Positions at or past 64 kofs[E] are not written.  Requires C % 256 == 0,
 * 256 <= C <= 2^20.
 *
 * nvfp4_grouped_gemm_wgrad - dW_e = dequant(G_e^T) dequant(X_e^T)^T for every
 * expert, exact products of the decoded values with FP32 accumulation (error
 * within 2e-5 * sum |a w| per element), for all experts in one launch:
 *   A (G side): row-major codes [M][Kp/2], bscales [M][Kp/16], rscales [E][M]
 *   W (X side): K-tiled codes [Kp/64][N][32], bscales [Kp/64][N][4], rscales [E][N]
 *   c          [E][M][N] of c_dtype: NVFP4_OUT_F32 (float) or NVFP4_OUT_BF16 (bf16 bits,
 *              each FP32 result rounded to nearest even)
 * Requires N % 16 == 0, 16 <= N <= 2^20, Kp % 64 == 0, M * Kp / 2 and
 * N * Kp / 2 below 2^32.  kofs as nvfp4moe_token_blocks writes it (kofs[E] <=
 * Kp / 64); each expert's range is clamped into [0, Kp / 64) with at least one
 * K-step, so other values give wrong results but no access outside the buffers.
 */
#define NVFP4_IN_BF16 0
#define NVFP4_IN_F32 1
NVFP4MOE_API int nvfp4moe_token_blocks(const int32_t* expert_offsets, int32_t E, int32_t* kofs,
                                       void* stream);
NVFP4MOE_API int nvfp4_quantize_tokens(const void* x, int32_t x_dtype, int64_t x_rows, int64_t C,
                                       const int32_t* row_to_tk, int32_t k,
                                       const int32_t* expert_offsets, const int32_t* kofs, int32_t E,
                                       int64_t Kp, int32_t layout, uint8_t* codes, uint8_t* bscales,
                                       float* rscales, void* stream);
NVFP4MOE_API int nvfp4_grouped_gemm_wgrad(const uint8_t* a_codes, const uint8_t* a_bscales,
                                          const float* a_rscales, const uint8_t* w_codes,
                                          const uint8_t* w_bscales, const float* w_rscales,
                                          const int32_t* kofs, int32_t E, int64_t M, int64_t N,
                                          int64_t Kp, void* c, int32_t c_dtype, void* stream);

/*
 * swiglu_quantize - weighted SwiGLU of the gate_up output with the amax taken
 * on the fly, then NVFP4 quantisation of each routed row (for the down GEMM).
 *   gu        float [R_cap][2I]: gate = columns [0, I), up = columns [I, 2I)
 *   topk_w    float [T*k] router weight of (t, slot) (NULL: weight 1)
 *   row_to_tk int32 [R_cap] from nvfp4_quantize_permute (needed if topk_w; an entry
 *             outside [0, R_cap) gives that row the router weight 0)
 *   h = float32( ((g / (1 + exp(-g))) * u) * w ), evaluated in FP64 (g times the
 *             sigmoid from the library's own exp and a Newton-refined reciprocal: within
 *             2^-50 relative of the exact value, so h can differ from the correctly
 *             rounded float32 only where that value lies next to a rounding midpoint)
 *   codes [R_cap][I/2], bscales [R_cap][I/16], rscales [R_cap]: NVFP4 of h
 *   h_out     float [R_cap][I] (NULL: not written)
 * Requires I % 16 == 0, 16 <= I <= NVFP4MOE_MAX_K.
 */
NVFP4MOE_API int swiglu_quantize(const float* gu, int64_t R_cap, int64_t I,
                                 const int32_t* expert_offsets, int32_t E,
                                 const float* topk_w, const int32_t* row_to_tk,
                                 uint8_t* codes, uint8_t* bscales, float* rscales,
                                 float* h_out, void* stream);

/*
 * unpermute_combine - sum each token's k routed rows back into token order:
 *   acc = w_0 * d[row(t,0)];  acc = acc + w_s * d[row(t,s)]  (s = 1..k-1)
 * in FP32, slot order, no fused multiply-add; y[t] = bf16(acc) (nearest even).
 * w_s = 1 when topk_w is NULL (the router weight already applied in
 * swiglu_quantize).  Pairs with tk_to_row = -1 are skipped, and so are entries at
 * or beyond T*k (d holds R_cap = T*k rows).
 *   d float [T*k][H]; tk_to_row int32 [T*k]; y bf16 bits [T][H]
 * Requires H % 8 == 0, 1 <= k <= NVFP4MOE_MAX_TOPK.
 */
NVFP4MOE_API int unpermute_combine(const float* d, int64_t T, int32_t k, int64_t H,
                                   const int32_t* tk_to_row, const float* topk_w,
                                   uint16_t* y, void* stream);

/*
 * permute_gather_bf16 - copy token rows to their routed rows (backward input):
 *   out[r] = x[row_to_tk[r] / k]  for r < expert_offsets[E] (and r < T*k)
 *   x bf16 bits [T][H]; out bf16 bits [T*k][H]; a token index outside [0, T) is
 *   clamped into it.  Requires H % 8 == 0.
 */
NVFP4MOE_API int permute_gather_bf16(const uint16_t* x, int64_t T, int64_t H, int32_t k,
                                     const int32_t* expert_offsets, int32_t E,
                                     const int32_t* row_to_tk, uint16_t* out, void* stream);

/*
 * bf16_grouped_gemm - BF16 grouped GEMM for the backward (dgrad):
 *   c[r][n] = sum_k a[r][k] * W_e[k][n]   for r in expert e's rows
 * with BF16 operands, FP32 accumulation, FP32 output.
 *   a  bf16 bits [R_cap][K]
 *   w  bf16 bits, layout by w_layout:
 *        NVFP4MOE_W_KN (0): [E][K][N]  (e.g. the forward weight [E][out][in]
 *                           used for the input gradient, contracting over out)
 *        NVFP4MOE_W_NK (1): [E][N][K]
 *   c  float [R_cap][N]
 * Requires K % 32 == 0, N % 16 == 0, and each operand under 4 GiB (R_cap * K * 2 and
 * E * N * K * 2 bytes).
 */
#define NVFP4MOE_W_KN 0
#define NVFP4MOE_W_NK 1
NVFP4MOE_API int bf16_grouped_gemm(const uint16_t* a, const int32_t* expert_offsets,
                                   int32_t E, int64_t R_cap, const uint16_t* w,
                                   int32_t w_layout, int64_t N, int64_t K, float* c,
                                   void* stream);

/*
 * bf16_grouped_gemm_gather - bf16_grouped_gemm whose left operand is gathered
 * from token order (permute_gather_bf16 fused into the GEMM's loads):
 *   c[r][n] = sum_k a[row_to_tk[r] / k][k'] * W_e[k'][n]   for r in expert e's rows
 *   a bf16 bits [T][K] (e.g. the output gradient of the tokens);
 *   row_to_tk int32 [R_cap] from nvfp4_quantize_permute; 1 <= k <= NVFP4MOE_MAX_TOPK.
 * Other arguments, layouts and requirements as bf16_grouped_gemm, with the
 * 4 GiB limit on T * K * 2.  A row_to_tk entry outside [0, T * k) reads a row
 * of a clamped into [0, T) (a wrong result, never an access outside a).
 */
NVFP4MOE_API int bf16_grouped_gemm_gather(const uint16_t* a, int64_t T, const int32_t* row_to_tk,
                                          int32_t k, const int32_t* expert_offsets, int32_t E,
                                          int64_t R_cap, const uint16_t* w, int32_t w_layout,
                                          int64_t N, int64_t K, float* c, void* stream);

/*
 * swiglu_backward - gradient of h = w * silu(g) * u with respect to g and u:
 *   t = dh * w;  du = t * silu(g);  dg = (t * u) * (sig * (1 + g * (1 - sig)))
 * with sig = 1 / (1 + exp(-g)), silu(g) = g / (1 + exp(-g)), in FP64 (sig as in
 * swiglu_quantize, silu = g * sig: within 2^-50 relative of the quotients); each
 * result rounded once to bf16 (nearest even).
 *   gu float [R_cap][2I] (forward gate_up output); dh float [R_cap][I]
 *   topk_w / row_to_tk as in swiglu_quantize (NULL topk_w: w = 1)
 *   dgu bf16 bits [R_cap][2I]: [0, I) = dg, [I, 2I) = du
 * A row_to_tk entry outside [0, R_cap) gives that row the router weight 0.
 * Requires I % 8 == 0.
 */
NVFP4MOE_API int swiglu_backward(const float* gu, const float* dh, int64_t R_cap, int64_t I,
                                 const int32_t* expert_offsets, int32_t E,
                                 const float* topk_w, const int32_t* row_to_tk,
                                 uint16_t* dgu, void* stream);

/*
 * bf16_transpose - out[b][j][i] = in[b][i][j] for `batches` bf16 matrices.
 * Weight preparation for a lower-precision backward: the blog "miniTE NVFP4"
 * (yuxiaoba.github.io, section "Two complementary interventions") keeps the
 * backward's precision independent of the forward's and notes that a
 * lower-bit backward is not automatically faster.  Its NVFP4 input-gradient
 * GEMM contracts a forward weight [E][out][in] over `out`, so it quantises
 * the transposed weight [E][in][out] along `out` (nvfp4_quantize_rows_tiled).
 *   in  bf16 bits [batches][rows][cols]; out bf16 bits [batches][cols][rows]
 * Requires rows % 8 == 0, cols % 8 == 0, rows * cols <= INT32_MAX,
 * 0 <= batches <= 65535; out must not overlap in (out == in: NVFP4_ERR_ARG).
 */
NVFP4MOE_API int bf16_transpose(const uint16_t* in, int64_t batches, int64_t rows, int64_t cols,
                                uint16_t* out, void* stream);

/* Measurement aid (no part of the MoE computation): the device's practical
 * FP16 MFMA rate.  256 workgroups of 8 wavefronts (two per SIMD on a 256-CU
 * MI355X) each issue `iters` rounds of 8 independent v_mfma_f32_32x32x16_f16 on
 * register operands, then write one float per thread to sink.
 *   iters in [1, 1e7]; sink: device, 16-byte aligned, 256 * 512 floats
 *   FLOPs issued = 256 * 8 * iters * 8 * 32768; the caller times the stream.
 */
NVFP4MOE_API int nvfp4moe_mfma_ceiling(int64_t iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4MOE_H */
