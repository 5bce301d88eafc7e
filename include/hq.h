/*
 * hq.h -- C ABI of the MI355X (gfx950) quantized GEMM library.
 *
 * The library multiplies activations by packed 4-bit weights that are
 * dequantised inside the kernel, in a dense form and in a grouped
 * mixture-of-experts (MoE) form.  Every entry point returns an hq_status;
 * nothing throws across this boundary, and a thread-local message
 * (hq_last_error) explains the last failure.
 *
 * What is computed (the Humming pages describe it in prose only):
 *   - "Humming: open-source kernel library for quantized inference"
 *     (news.ditty.ir), summary: every supported weight format is converted
 *     into one standard description in which the weight codes, the scales
 *     and the zero points are separate parameters; a layer is described by
 *     a layer config (shapes, data types), a compute config (which GEMM) and
 *     a tuning config (tile size, pipeline stages, matrix instruction),
 *     chosen by a heuristic; W4A16, W4A8 (including MXFP4 weights with FP8
 *     activations) and a grouped MoE path are supported.
 *   - cocoloop.cn (vi / fr), format section and speed-up table: WnA16,
 *     W4A8 and MXFP4 formats; dense single-layer GEMMs and MoE layers.
 *   - aube.news (pt): INT4 stores one weight in 4 bits; dense and MoE layers.
 *
 * Number formats follow the OCP Microscaling (MX) v1.0 specification (E2M1
 * elements, E8M0 shared scales, 32-element blocks) and the OCP 8-bit
 * floating-point specification (E4M3, "fn" variant: no infinities).
 *
 * Conventions that hold for every function below
 * -----------------------------------------------
 *   * Pointers named "device" point to memory the caller allocated on the
 *     GPU (hipMalloc, or a torch tensor's data_ptr()); "host" pointers point
 *     to CPU memory.  The library never allocates, frees or synchronises on
 *     the hq_gemm / hq_moe_* paths; work is queued on `stream` (a
 *     hipStream_t, passed as void* so this header needs no HIP headers;
 *     NULL is the default stream) and returns before it finishes.
 *   * Argument validation happens before any launch; a rejected call
 *     touches no memory.  A launch failure reported by the runtime returns
 *     HQ_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *     synchronisation, as for any asynchronous GPU work.
 *   * Device buffers must be 16-byte aligned.
 *   * Canonical (user-facing) weight layout, row-major, n-major:
 *       codes   int32 [N, K/8]: eight 4-bit codes per word along K; code
 *               k = 8j+i sits in bits [4i, 4i+4) of word j (low nibble
 *               first); the word is a bit container, its sign is irrelevant.
 *               INT8 weights (W8A16): uint8 [N, K], one byte per weight.
 *               INT2 weights (W2A16): int32 [N, K/16], code k = 16j + i in
 *               bits [2i, 2i+2) of word j.
 *               INT3 weights (W3A16): int32 [N, 3K/32], the dense 3-bit
 *               packing along K of GPTQ INT3: a row's words form one
 *               little-endian bit stream and code k takes its bits
 *               [3k, 3k+3) (codes may straddle two words).
 *       scales  fp16 or bf16 [N, K/G] (INT4 / INT8, G = 128): group g covers
 *               k in [G*g, G*g+G).
 *       zeros   uint8 [N, K/G] holding 0..15 (only with HQ_ZP_PER_GROUP_U4).
 *       e8m0    uint8 [N, K/32] (MXFP4, MXINT4): scale 2^(X-127) per 32 k.
 *       NVFP4   codes as MXFP4 (E2M1); block scales uint8 E4M3 [N, K/16],
 *               one per 16 k, passed where the zero points go; the fp32
 *               tensor scale (one float per expert) passed as `scales`.
 *     INT2 / INT3 / INT4 / INT8 dequantisation is w = (q - z) * s; MXFP4 is
 *     w = e2m1(q) * 2^(X-127); MXINT4 is w = int4(q) * 2^-2 * 2^(X-127) with
 *     int4 the two's-complement reading of the code (codes packed as INT4);
 *     NVFP4 is w = e2m1(q) * e4m3(S[n, k/16]) * s_tensor.
 *   * Activations: row-major [M, K] fp16 / bf16, or 8-bit codes (fp8 e4m3
 *     or int8) with one fp32 scale per row (value = code * scale[m]).
 *   * Output: row-major [M, N] fp16 / bf16, rounded to nearest even from
 *     the fp32 accumulator.  Outputs are fully overwritten (no beta).
 */
#ifndef HQ_H
#define HQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 3: hq_tuning gained tile_group; run-time specialisation (hq_plan_set_jit,
 * hq_jit_*) and hq_moe_gemm_by_slot added; the combine's workspace rows are
 * bf16 */
#define HQ_ABI_VERSION 3

typedef enum hq_status {
  HQ_OK = 0,
  HQ_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, ...     */
  HQ_ERR_UNSUPPORTED = 2, /* valid request this library does not implement */
  HQ_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required    */
  HQ_ERR_HIP = 4,         /* the HIP runtime reported an error             */
  HQ_ERR_INTERNAL = 5     /* unexpected failure inside the library         */
} hq_status;

typedef enum hq_dtype {
  HQ_F16 = 0,
  HQ_BF16 = 1,
  HQ_F32 = 2,
  HQ_FP8_E4M3 = 3, /* OCP e4m3fn */
  HQ_INT8 = 4,
  HQ_U4 = 5,       /* unsigned 4-bit integer code 0..15 */
  HQ_FP4_E2M1 = 6, /* OCP MX FP4 element */
  HQ_E8M0 = 7,     /* OCP MX shared scale */
  HQ_I32 = 8,
  HQ_U8 = 9,       /* unsigned 8-bit integer code 0..255 */
  HQ_U2 = 10,      /* unsigned 2-bit integer code 0..3 */
  HQ_U3 = 11,      /* unsigned 3-bit integer code 0..7 */
  HQ_I4 = 12       /* MXINT4 element: two's-complement 4-bit code, value (-8..7) * 2^-2 */
} hq_dtype;

typedef enum hq_zp_mode {
  HQ_ZP_NONE = 0,        /* no zero point (MXFP4)                        */
  HQ_ZP_FIXED = 1,       /* one integer zero point for every group       */
  HQ_ZP_PER_GROUP_U4 = 2 /* uint4 zero point per (n, group)              */
} hq_zp_mode;

typedef enum hq_ascale_mode {
  HQ_ASCALE_NONE = 0,         /* 16-bit activations, no scale        */
  HQ_ASCALE_PER_TOKEN_F32 = 1, /* 8-bit codes with one fp32 per row  */
  HQ_ASCALE_MX_E8M0 = 2        /* MXFP4 codes with an E8M0 scale per row and 32-element block */
} hq_ascale_mode;

/* The unified quantisation description: weight codes, scales, zero points
 * and activation type as separate parameters (Humming page on
 * news.ditty.ir, summary).  Supported combinations:
 *   W4A16      w_elem U4, group 128, scale F16|BF16, zp FIXED|PER_GROUP_U4,
 *              act F16|BF16, act_scale NONE, out F16|BF16
 *   W8A16      w_elem U8 (w_bits 8), group 128, scale F16|BF16, zp FIXED
 *              (0..255, 128 for the symmetric case), act F16|BF16,
 *              act_scale NONE, out F16|BF16 (dense only; one of the WnA16
 *              widths INT1..INT8 of cocoloop.cn, format section)
 *   W2A16      w_elem U2 (w_bits 2), group 128, scale F16|BF16, zp FIXED
 *              (0..3, 2 for the symmetric case), act F16|BF16, act_scale
 *              NONE, out F16|BF16 (dense only)
 *   W3A16      w_elem U3 (w_bits 3), group 128, scale F16|BF16, zp FIXED
 *              (0..7, 4 for the symmetric case), act F16|BF16, act_scale
 *              NONE, out F16|BF16 (dense only; GPTQ INT3, the format
 *              cocoloop.cn names for the compatibility route)
 *   W4A16-MXINT4 w_elem I4 (w_bits 4), group 32, scale E8M0, zp NONE,
 *              act F16|BF16, act_scale NONE, out F16|BF16 (dense only;
 *              MXINT4 is in the format list of cocoloop.cn, format section)
 *   W4A16-NVFP4 w_elem FP4_E2M1 (w_bits 4), group 16, scale FP8_E4M3,
 *              zp NONE, act F16|BF16, act_scale NONE, out F16|BF16 (dense
 *              only; NVFP4 as NVIDIA publishes it, named by the same page)
 *   W4A8-INT   w_elem U4, group 128, scale F16|BF16, zp FIXED (8),
 *              act INT8, act_scale PER_TOKEN_F32, out F16|BF16
 *   W4A8-FP8   w_elem U4, group 128, scale F16|BF16, zp FIXED|PER_GROUP_U4,
 *              act FP8_E4M3, act_scale PER_TOKEN_F32, out F16|BF16
 *   W4A8-MXFP4 w_elem FP4_E2M1, group 32, scale E8M0, zp NONE,
 *              act FP8_E4M3, act_scale PER_TOKEN_F32, out F16|BF16
 *   W4A4-MXFP4 w_elem FP4_E2M1, group 32, scale E8M0, zp NONE,
 *              act FP4_E2M1, act_scale MX_E8M0, out F16|BF16 (dense only;
 *              W4A4 and MXFP4 are among the supported combinations and
 *              formats of cocoloop.cn, format section)
 * Anything else returns HQ_ERR_UNSUPPORTED from hq_plan_create. */
typedef struct hq_quant_desc {
  hq_dtype w_elem;
  int w_bits;     /* 4 */
  int group_size; /* 128 (INT4) or 32 (MXFP4) */
  hq_dtype scale;
  hq_zp_mode zp;
  int zp_value;   /* HQ_ZP_FIXED: the zero point, 0..15 */
  hq_dtype act;
  hq_ascale_mode act_scale;
  hq_dtype out;
} hq_quant_desc;

/* Layer config: the weight's shape; num_experts > 1 for the grouped form. */
typedef struct hq_layer_desc {
  int64_t n, k;
  int num_experts;
  hq_quant_desc q;
} hq_layer_desc;

typedef enum hq_gemm_kind { HQ_GEMM_DENSE = 0, HQ_GEMM_GROUPED = 1 } hq_gemm_kind;

typedef enum hq_epilogue {
  HQ_EPI_NONE = 0,          /* plain output                                */
  HQ_EPI_SILU_MUL = 1,      /* grouped gate_up: SiLU(h[:, :N/2]) * h[:, N/2:] */
  HQ_EPI_SILU_MUL_QFP8 = 2, /* as above, then per-row fp8 e4m3 requant    */
  HQ_EPI_TOPK_COMBINE = 3,  /* grouped down: * topk weight, sum per token  */
  HQ_EPI_I32_ACC = 4        /* W4A8-INT debug: per-group int32 accumulators */
} hq_epilogue;

/* Operand type of the matrix instruction a plan runs on.  The quantisation
 * description fixes it (16-bit activations: HQ_MFMA_F16 / HQ_MFMA_BF16;
 * INT4 x int8: HQ_MFMA_INT8; INT4 x fp8: HQ_MFMA_FP8; MXFP4 x fp8:
 * HQ_MFMA_FP8_FP4; MXFP4 x MXFP4: HQ_MFMA_FP4); HQ_MFMA_AUTO takes that
 * type, any other value must name it. */
typedef enum hq_mfma_in {
  HQ_MFMA_AUTO = 0,
  HQ_MFMA_F16 = 1,
  HQ_MFMA_BF16 = 2,
  HQ_MFMA_FP8 = 3,
  HQ_MFMA_INT8 = 4,
  HQ_MFMA_FP8_FP4 = 5,
  HQ_MFMA_FP4 = 6
} hq_mfma_in;

/* Compute config: which GEMM, which epilogue, and the matrix-instruction
 * operand type (the pages' compute config: the GEMM type a layer runs as,
 * Humming page on news.ditty.ir, summary).  A request this library cannot
 * run (an operand type other than the description's, a combination without
 * a kernel) is HQ_ERR_UNSUPPORTED from hq_plan_create; the pages' answer to
 * a compute type the GPU lacks is to run the layer at a higher precision
 * (same page, summary), which the Python binding does by building the plan
 * again with 16-bit activations. */
typedef struct hq_compute {
  hq_gemm_kind kind;
  hq_epilogue epi;
  hq_mfma_in mfma_in;
} hq_compute;

/* Tuning config (execution choice, kept apart from the description).
 * Zero in any field means "let the heuristic choose". */
typedef struct hq_tuning {
  int kernel;  /* 0 auto, 1 skinny (small M, split-K), 2 tiled (large M)  */
  int tile_m;  /* skinny: rows per workgroup (16, 32, 64); tiled: 64 or 128     */
  int tile_n;  /* skinny: columns per workgroup (16, 32, 64); tiled: 128, 256 */
  int waves;   /* wavefronts per workgroup                                 */
  int split_k; /* workgroups sharing one output tile along K (dense)     */
  int stages;  /* skinny: 128-k groups in flight per wave (2, 4, 8);
                  tiled: groups in the LDS / register ring (2..5)          */
  int mfma;    /* 16 (16x16 MFMA); reserved for 32                         */
  int tile_group; /* tiled kernel launch order: row tiles per group (1 = row
                    by row); each group is walked column by column, so an XCD
                    works on a block of tiles that shares activations and
                    weights in its L2 (0 = the library's choice)          */
} hq_tuning;

typedef struct hq_plan hq_plan;

int hq_abi_version(void);
const char* hq_status_str(hq_status s);
/* Message of the last failed call on this thread ("" if none). */
const char* hq_last_error(void);

/* Validate a layer + compute description and pick an execution choice --
 * the pages' layer config (shapes, data types), compute config (GEMM type)
 * and tuning config (tile, pipeline, matrix instruction), the last chosen by
 * a rule-based heuristic (Humming page on news.ditty.ir, summary; cocoloop.cn,
 * limits section: tuning is heuristic).
 * max_m bounds the rows (tokens) a later call may pass.  `tuning` may be
 * NULL (heuristic, the rule-based selection the pages describe); non-zero
 * fields override it.  On success *out owns a host object released with
 * hq_plan_destroy.  A plan is immutable and may be used from several
 * streams and threads at once (each call with its own workspace). */
hq_status hq_plan_create(const hq_layer_desc* layer, const hq_compute* compute, int64_t max_m,
                         const hq_tuning* tuning, hq_plan** out);
hq_status hq_plan_destroy(hq_plan* plan);
/* Human-readable description of the plan's execution choice for m rows; for
 * a grouped plan, m is the number of routed slots (t * topk) of a call. */
hq_status hq_plan_describe(const hq_plan* plan, int64_t m, char* buf, size_t len);

/* Workspace a call with m rows needs, in bytes (0 if none) -- memory the
 * execution choice adds to the layer description, kept apart from it as the
 * pages keep the tuning config apart from the layer config (Humming page on
 * news.ditty.ir, summary): the fp32 partial
 * tiles [split][m][n] when K is split over workgroups (a second kernel of the
 * same call sums them in split order, so results are deterministic).  Its
 * contents need no initialisation.  Two calls that overlap in time must not
 * share one workspace. */
hq_status hq_plan_workspace_bytes(const hq_plan* plan, int64_t m, size_t* bytes);

/* Sizes of the repacked (device-layout) weight: w_bytes for the codes,
 * meta_bytes for scales + zero points (or E8M0 scales) -- the weight, scale
 * and zero point held as separate parameters of the one standard format
 * (Humming page on news.ditty.ir, summary; aube.news: INT4 stores one weight
 * in 4 bits).  For a grouped
 * plan both cover all experts. */
hq_status hq_repacked_bytes(const hq_plan* plan, size_t* w_bytes, size_t* meta_bytes);

/* Offline repack (the format conversion into the library's standard
 * layout that the pages describe for every supported format: Humming page on
 * news.ditty.ir, summary): canonical codes / scales / zeros-or-e8m0 (see above; for a
 * grouped plan each is stacked [E, ...]) -> the device layout, which places
 * the 4-bit codes in gfx950 MFMA operand order.  All pointers are device
 * pointers; the work is a kernel on `stream`.  `zeros_or_e8m0` is NULL for
 * HQ_ZP_FIXED.  The output is a private layout: only hq_gemm / hq_moe_gemm
 * of a plan with the same layer description and activation type read it. */
hq_status hq_repack(const hq_plan* plan, const void* codes, const void* scales,
                    const void* zeros_or_e8m0, void* w_out, void* meta_out, void* stream);
/* The same permutation on host memory (for preparing weights offline on a
 * machine without a GPU).  Produces bytes identical to hq_repack. */
hq_status hq_repack_host(const hq_plan* plan, const void* codes, const void* scales,
                         const void* zeros_or_e8m0, void* w_out, void* meta_out);

/* Dense GEMM: out[M, N] = A[M, K] . W_deq^T, the weights dequantised inside
 * the kernel from their packed codes (the mixed-precision GEMM of the pages:
 * Humming page on news.ditty.ir, summary -- WnA16, W4A8 including MXFP4 x
 * FP8, W4A4; cocoloop.cn, format section and speed-up table, dense rows).
 *   a        device [m, K] activations (act dtype of the plan)
 *   a_scale  device: fp32 [m] per-row scales for 8-bit activations; for
 *            MXFP4 activations (W4A4; the codes in `a` packed like the
 *            weights, two per byte along K, low nibble first: [m, K/2]
 *            bytes) the E8M0 block scales as group-major words uint8
 *            [K/128][m][4], byte j of word (g, r) scaling k-block 4g + j of
 *            row r (so that the 16 rows of one MFMA operand are 64
 *            contiguous bytes); else NULL
 *   w, meta  device, produced by hq_repack
 *   out      device [m, N] in the plan's out dtype; with HQ_EPI_I32_ACC
 *            (W4A8-INT only) int32 [m, N, K/128] holding
 *            P[m,n,g] = sum_{k in group g} a_q[m,k] * (q[n,k] - 8), exactly
 *   ws       device workspace of hq_plan_workspace_bytes(plan, m) bytes
 *            (may be NULL when that is 0)
 * m = 0 is a no-op; m > max_m is HQ_ERR_INVALID_ARG.  The kernels address
 * `a` and `w` through 32-bit buffer ranges: an `a` of 2 GiB or more, or a `w`
 * of 2 GiB or more, is HQ_ERR_UNSUPPORTED. */
hq_status hq_gemm(const hq_plan* plan, int64_t m, const void* a, const void* a_scale,
                  const void* w, const void* meta, void* out, void* ws, size_t ws_bytes,
                  void* stream);

/* hq_gemm for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It runs the same kernels as hq_gemm with the same plan
 * and execution choice; the split-K partials (the only scratch a dense call
 * needs) live in a 16 MiB device array owned by the library, one per GPU,
 * held until the process ends.  A call whose partials exceed 16 MiB (see
 * hq_plan_workspace_bytes) returns HQ_ERR_WORKSPACE before any launch.  The
 * call allocates nothing (no hipMalloc / hipFree); the first call on a device
 * looks the array's address up once (thread-safe).  Every call on one GPU
 * shares that GPU's array and overwrites what it reads, so nothing needs
 * clearing, but calls that overlap in time on one GPU (several streams or
 * threads) race on it: serialise them, or use hq_gemm with workspaces of
 * their own.  Arguments and results as hq_gemm. */
hq_status hq_gemm_noalloc(const hq_plan* plan, int64_t m, const void* a, const void* a_scale, const void* w,
                          const void* meta, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * Grouped (mixture-of-experts) path.  The pages describe a separate MoE
 * backend with its own "Grouped" GEMM path run with W4A16 or W4A8 weights
 * (Humming page on news.ditty.ir, summary; cocoloop.cn speed-up table).  A
 * layer is: routing ids -> hq_moe_align -> gate_up GEMM (+ SiLU * mul, or +
 * per-row fp8 requant) -> down GEMM (+ top-k weighted combine into tokens).
 * ------------------------------------------------------------------------- */

/* Rows per expert block that a grouped plan's kernels use for `t` tokens
 * routed to `topk` experts each: 16 when few slots land on each expert (the
 * weight-streaming kernel), 64 or 128 when many do (the MFMA-tiled kernel), or
 * what the plan's tuning fixes.  hq_moe_align must be called with this
 * block_m, and hq_moe_gemm with the same t and topk: the GEMM reads
 * sorted_ids and block_expert as laid out for this block size (a different
 * block size reads past their end).  The gate_up and down plans of one layer
 * share one alignment, so they must give the same block_m (true for
 * equal tuning). */
hq_status hq_moe_block_m(const hq_plan* plan, int64_t t, int topk, int* block_m);

/* Size of the aligned slot array for `t` tokens: the largest possible sum
 * over the num_experts + 1 segments (the experts, then out-of-range ids) of
 * count rounded up to block_m, i.e. t*topk + (num_experts + 1)*(block_m - 1)
 * rounded up to block_m. */
hq_status hq_moe_max_padded(int64_t t, int topk, int num_experts, int block_m, int64_t* max_padded);

/* Token sort / align by expert.  topk_ids: device int32 [t, topk].  Outputs
 * (device, int32): sorted_ids[max_padded]: flat slot indices t*topk + j
 * grouped by expert in increasing expert order, each expert's segment padded
 * to a multiple of block_m with the sentinel t*topk (order inside a segment
 * is unspecified); slots whose id is outside [0, num_experts) (for example
 * experts masked with -1) form one last segment; block_expert[max_padded /
 * block_m]: the expert of each block, -1 for the out-of-range segment;
 * num_padded[1]: the used length.  One workgroup; t * topk <= 2^20. */
hq_status hq_moe_align(int64_t t, int topk, int num_experts, int block_m, const int32_t* topk_ids,
                       int32_t* sorted_ids, int32_t* block_expert, int32_t* num_padded, void* stream);

/* Grouped GEMM over the aligned blocks (plan kind HQ_GEMM_GROUPED, layer n x k
 * per expert, num_experts experts, weights repacked by hq_repack).
 *   epi HQ_EPI_SILU_MUL       gate_up: row r of the aligned array takes token
 *                             sorted_ids[r] / topk of `a` [t, k];
 *                             out[max_padded, n/2] (plan out dtype) =
 *                             SiLU(h[:, :n/2]) * h[:, n/2:].
 *   epi HQ_EPI_SILU_MUL_QFP8  as above, then per-row fp8 e4m3 requant by the
 *                             rule of hq_quantize_per_token: out = uint8
 *                             codes [max_padded, n/2], out_scale = fp32
 *                             [max_padded], s = max|act| / 448 (1 for an
 *                             all-zero row), codes = RNE(act / s) with a
 *                             correctly rounded fp32 quotient, saturated to
 *                             +-448.  act is the fp32 value the epilogue
 *                             forms; after the call the first
 *                             max_padded * n/2 * 4 bytes of ws hold those
 *                             fp32 rows (rows of padding slots unspecified).
 *   epi HQ_EPI_TOPK_COMBINE   down: row r of `a` [max_padded, k] is the
 *                             intermediate of slot sorted_ids[r];
 *                             out = y [t, n] (plan out dtype),
 *                             y[tok] = sum_j topk_w[tok, j] * (a_row . W_e^T):
 *                             each slot's weighted row, rounded to bf16, goes
 *                             to the workspace, then a second kernel sums a
 *                             token's topk rows in fp32 in slot order and
 *                             rounds once, so the result is deterministic.
 *                             Slots with an out-of-range expert id
 *                             contribute zero.
 *   epi HQ_EPI_NONE           gate_up rows without the activation: out
 *                             [max_padded, n] (plan out dtype).
 * a_scale: per-row fp32 scales of 8-bit activations (per token for gate_up,
 * per aligned row for down), else NULL.  topk_w: device fp32 [t, topk]
 * (TOPK_COMBINE only).  Rows of padding slots (and, for gate_up, of slots
 * with an out-of-range expert id) are left unwritten.  ws: the workspace of
 * hq_moe_workspace_bytes (the fp8 requant's fp32 rows, or the combine's
 * t*topk weighted bf16 slot rows); every call writes what it reads, so its
 * contents need no initialisation and no state carries over between calls
 * (two calls that overlap in time must not share one workspace).  As for
 * hq_gemm, activations or one expert's weights of 2 GiB or more are
 * HQ_ERR_UNSUPPORTED. */
hq_status hq_moe_workspace_bytes(const hq_plan* plan, int64_t t, int topk, size_t* bytes);
hq_status hq_moe_gemm(const hq_plan* plan, int64_t t, int topk, const void* a, const float* a_scale,
                      const int32_t* sorted_ids, const int32_t* block_expert, const int32_t* num_padded,
                      const float* topk_w, const void* w, const void* meta, void* out, float* out_scale,
                      void* ws, size_t ws_bytes, void* stream);

/* The same grouped GEMMs without the alignment, for decode-sized t: the rows
 * are the routed slots themselves (slot s = t*topk index tok*topk + j, expert
 * topk_ids[s]), so no hq_moe_align call precedes them and a layer is two
 * launches (three with the fp8 requant).  Same plan, weights, metadata and
 * epilogue semantics as hq_moe_gemm (MoE path of the pages as cited above):
 *   topk_ids  device int32 [t, topk]; ids outside [0, num_experts) are
 *             allowed and contribute zero
 *   gate_up   (HQ_EPI_SILU_MUL / _QFP8 / NONE): `a` [t, k] (token rows),
 *             out [t*topk, n/2] (or [t*topk, n] for NONE) indexed by slot;
 *             a slot with an out-of-range id gets a zero row (fp8: zero
 *             codes, scale 1).  _QFP8: out_scale fp32 [t*topk]; ws holds
 *             the fp32 rows, align256(t*topk * n/2 * 4) bytes, after the
 *             call (hq_moe_workspace_bytes is always enough).
 *   down      (HQ_EPI_TOPK_COMBINE): `a` [t*topk, k] slot rows (the gate_up
 *             output), a_scale fp32 [t*topk] for fp8 rows; out = y [t, n],
 *             y[tok] = sum_j topk_w[tok, j] * (a[tok*topk + j] . W_e^T),
 *             summed in one fp32 accumulator per output (each slot's top-k
 *             weight folded into its group scales) and rounded once; no
 *             workspace.  Deterministic run to run; the sum order differs
 *             from hq_moe_gemm's, so the two agree to fp32 rounding.
 * Every block reads its slot's (token's) expert weights directly, so an
 * expert picked by several slots is read once per slot: the aligned path is
 * the one for large t.  t * topk <= 65535; in down mode all experts' weights
 * (and their scales) must stay below 2 GiB, in gate_up mode one expert's.
 * The plan's tuning tile_n (16, 32 or 64 columns per workgroup; at least 32
 * for gate_up) and waves (1..16) override the defaults where set.  Honours
 * hq_time_next_launch (first launch to last). */
hq_status hq_moe_gemm_by_slot(const hq_plan* plan, int64_t t, int topk, const void* a, const float* a_scale,
                              const int32_t* topk_ids, const float* topk_w, const void* w, const void* meta,
                              void* out, float* out_scale, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Per-token activation quantiser: the step before a W4A8 GEMM, which takes
 * 8-bit activations with one fp32 scale per row (W4A8: INT8 or FP8
 * activations, FP8 for MXFP4 weights -- Humming page on news.ditty.ir,
 * summary; cocoloop.cn, format section).  The pages do not say how the
 * activations are quantised; this is the plain symmetric per-row rule:
 *   scales[r]  = max_j |x[r, j]| / Q, computed in fp32 (1 for an all-zero row)
 *   codes[r,j] = x[r, j] / scales[r], the correctly rounded fp32 quotient,
 *                rounded to nearest even and saturated to +-Q
 * with Q = 448 and OCP e4m3fn codes (out = HQ_FP8_E4M3; -0 gives code 0) or
 * Q = 127 and two's-complement int8 codes (out = HQ_INT8; -128 is never
 * produced).  The (codes, scales) pair is what hq_gemm takes as (a, a_scale).
 *   x       device [m, k] fp16 / bf16 (in = HQ_F16 / HQ_BF16), finite values
 *           (non-finite inputs give unspecified codes, no fault)
 *   codes   device [m, k] bytes, fully overwritten
 *   scales  device fp32 [m], fully overwritten
 * k must be a positive multiple of 8 (at most 2^24), m at most 2^24; m = 0
 * is a no-op.  x, codes and scales must not overlap.  Honours
 * hq_time_next_launch (one kernel).  The MoE gate_up GEMM has the same
 * quantisation fused into its epilogue (HQ_EPI_SILU_MUL_QFP8). */
hq_status hq_quantize_per_token(int64_t m, int64_t k, hq_dtype in, hq_dtype out, const void* x, void* codes,
                                float* scales, void* stream);

/* MXFP4 block quantiser for W4A4 activations (W4A4 and MXFP4: cocoloop.cn,
 * format section), following the OCP Microscaling v1.0 conversion of a block
 * of 32 values: X = floor(log2(max |v|)) - 2 (2 = the largest E2M1 exponent),
 * clamped to [-127, 127], with X = 0 for an all-zero block; each element is
 * v / 2^X (exact) rounded to E2M1, nearest with ties to even, saturated to
 * +-6; a value that rounds to zero gives code 0.
 *   x      device [m, k] fp16 / bf16 (in = HQ_F16 / HQ_BF16), finite values
 *   codes  device [m, k/2] bytes: E2M1 codes two per byte along k, low
 *          nibble first (the `a` of a W4A4 hq_gemm), fully overwritten
 *   e8m0   device bytes, X + 127 per block, in the group-major word layout
 *          [k/128][m][4] that hq_gemm takes as the `a_scale` of W4A4
 * k must be a multiple of 128 (at most 2^24), m at most 2^24 and m * k at
 * most 2^36; m = 0 is a no-op.  Honours hq_time_next_launch (one kernel). */
hq_status hq_quantize_mxfp4(int64_t m, int64_t k, hq_dtype in, const void* x, void* codes, uint8_t* e8m0,
                            void* stream);

/* ---- Autotuning (dense plans) ----------------------------------------
 * The heuristic maps (format, n, k, m) to an execution choice by rules taken
 * from sweeps; the pages list that rule-based selection among the
 * limitations, with autotuning not yet finished (cocoloop.cn, limitations
 * section).  These calls replace the heuristic per row count m with a
 * measured choice.
 *
 * A plan keeps a table m -> hq_tuning (empty at creation).  For an m in the
 * table, every later call on the plan (hq_gemm, hq_plan_describe,
 * hq_plan_workspace_bytes) uses that entry in place of the plan's tuning;
 * other m keep the heuristic.  The table is changed only by the two calls
 * below, which must not overlap any other call that uses the plan. */

typedef struct hq_autotune_result {
  hq_tuning best;     /* the installed choice, every field resolved        */
  float best_us;      /* its mean device time per call, microseconds       */
  float current_us;   /* the same for the choice in force before the call  */
  int candidates;     /* execution choices timed (the current one included) */
} hq_autotune_result;

/* Time the current choice for m rows and every other candidate that fits
 * (skinny kernel up to 64 rows over row / column blocks, waves, groups in
 * flight and K split; tiled kernel from 17 rows over tile shape, ring depth
 * and K split) on the caller's buffers, exactly as hq_gemm takes them, then
 * install the fastest for m.  Each candidate runs once untimed and `reps`
 * times between two events on `stream` (mean taken); with flush_bytes > 0
 * a buffer of that size is read before each timed run so that the weights
 * come from HBM rather than the caches (use at least 2x the 256 MiB
 * last-level cache for an HBM-bound choice).  Candidates needing more than
 * ws_bytes of workspace are skipped (ws may be NULL: only choices without a
 * workspace).  `out` holds the product on return.  Synchronises `stream`;
 * allocates the flush buffer, events and a 16-byte sink with hipMalloc and
 * frees them before returning.  `result` may be NULL. */
hq_status hq_plan_autotune(hq_plan* plan, int64_t m, const void* a, const void* a_scale, const void* w,
                           const void* meta, void* out, void* ws, size_t ws_bytes, int reps, size_t flush_bytes,
                           void* stream, hq_autotune_result* result);

/* Install `tuning` for exactly m rows (validated like a plan's tuning and
 * stored resolved), or remove m's entry with tuning == NULL.  For a tuning
 * cache kept across processes: store hq_plan_get_tuning's result, install it
 * here in a later process. */
hq_status hq_plan_set_tuning(hq_plan* plan, int64_t m, const hq_tuning* tuning);

/* The resolved execution choice for m rows; *is_tuned (if not NULL) says
 * whether it comes from the table. */
hq_status hq_plan_get_tuning(const hq_plan* plan, int64_t m, hq_tuning* tuning, int* is_tuned);

/* Run-time specialisation (the pages compile each layer's kernel at run time
 * for its shape and keep the compiled kernels in a cache: "Humming:
 * open-source kernel library for quantized inference", news.ditty.ir,
 * summary; news.cocoloop.cn, limitations section, compile-speed paragraph).
 * With enable = 1, every hq_gemm on this dense plan runs its kernel compiled
 * by hipRTC with the call's M, N and K, the format and the resolved execution
 * choice (heuristic or tuning table) as compile-time constants.  The first
 * call of a shape on a device compiles it (about a second, host time, on the
 * calling thread) or loads it from the code-object cache: `cache_dir` (NULL or
 * "": $HQ_JIT_CACHE_DIR, else $XDG_CACHE_HOME/hq_jit, else
 * $HOME/.cache/hq_jit), one file per hq_jit_cache_key, written atomically;
 * an unwritable directory only means the next process compiles again.  The
 * kernel sources are read from the csrc directory next to the library.
 * Later calls of the shape launch the loaded kernel (modules stay loaded until
 * the process ends).  A compile failure makes hq_gemm return
 * HQ_ERR_UNSUPPORTED with the compiler's log in hq_last_error.  enable = 0
 * goes back to the precompiled kernels.  Dense plans only; not thread-safe
 * against concurrent calls on the same plan (like every setter). */
hq_status hq_plan_set_jit(hq_plan* plan, int enable, const char* cache_dir);

/* The cache key of the kernel hq_gemm runs for m rows under run-time
 * specialisation on architecture `arch` (e.g. "gfx950"): a NUL-terminated
 * string of at most 63 characters ("hq-<kernel>-<arch>-<64-bit hex hash>")
 * that changes with the kernel sources, the compile options, the format, the
 * shape and the execution choice.  Host only (no device call). */
hq_status hq_jit_cache_key(const hq_plan* plan, int64_t m, const char* arch, char* key, size_t key_bytes);

/* Compile the kernel hq_gemm would run for m rows under run-time
 * specialisation, for architecture `arch`, into the plan's code-object cache
 * directory (hq_plan_set_jit's cache_dir; the plan need not have run-time
 * specialisation enabled), unless a valid code object is there already.
 * Needs no device: a cache can be filled ahead of time on another machine.
 * HQ_ERR_UNSUPPORTED with the compiler's log if the compile fails,
 * HQ_ERR_INTERNAL if the cache file cannot be written. */
hq_status hq_jit_prepare(const hq_plan* plan, int64_t m, const char* arch);

/* Counters of the run-time specialisation since the library was loaded:
 * hipRTC compiles, code objects loaded from the disk cache, launches that found
 * the kernel already loaded, kernel launches, and the host seconds spent
 * compiling and loading. */
typedef struct hq_jit_stats {
  int64_t compiles;
  int64_t disk_hits;
  int64_t memory_hits;
  int64_t launches;
  double compile_seconds;
  double load_seconds;
} hq_jit_stats;
hq_status hq_jit_get_stats(hq_jit_stats* stats);

/* Kernel timing: the next hq_gemm, hq_moe_align, hq_moe_gemm,
 * hq_quantize_per_token, hq_quantize_mxfp4, hq_stream_read or hq_mfma_peak call on this
 * thread records `start` (hipEvent_t, created by the caller with timing
 * enabled) when its first kernel starts and `stop` when its last kernel ends
 * (the split-K reduce, the fp8 requant or the combine's final pass included;
 * dispatch times, so no host launch overhead), and hipEventElapsedTime gives
 * the call's device duration.  The request is consumed by that call (also when
 * it fails); passing NULL, NULL cancels a pending request. */
hq_status hq_time_next_launch(void* start_event, void* stop_event);

/* Bandwidth probe (measurement helper, not part of the GEMM): read `bytes`
 * (a multiple of 16) of the device buffer `buf` once with 16-byte loads on
 * `workgroups` workgroups of 256 threads; `sink` is a device uint32 that is
 * practically never written.  Honours hq_time_next_launch. */
hq_status hq_stream_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups, void* stream);

/* Matrix-core throughput probe (measurement helper, not part of the GEMM):
 * `workgroups` workgroups of 4 waves each run `iters` rounds of 4 independent
 * 16 x 16 matrix instructions of one operand type on register values, with
 * no memory traffic.  The types are those the GEMMs use: fp16 and bf16
 * (16x16x32), fp8 e4m3 x fp8, fp8 x fp4 e2m1 and fp4 x fp4 (the scaled
 * 16x16x128 form, unit scales) and int8 (16x16x64, int32 results).
 * *flops (if not NULL) receives the operations of the launch (2 * 16 * 16 * K
 * per instruction); with the duration from hq_time_next_launch it gives the
 * rate the chip sustains for that type.  `sink` is a device uint32 that is
 * practically never written.  workgroups in [1, 2^20], iters in [1, 2^24]. */
typedef enum { HQ_PEAK_F16 = 0, HQ_PEAK_BF16 = 1, HQ_PEAK_FP8 = 2, HQ_PEAK_FP8_FP4 = 3, HQ_PEAK_FP4 = 4,
               HQ_PEAK_INT8 = 5 } hq_peak_type;
hq_status hq_mfma_peak(int type, int workgroups, int iters, uint32_t* sink, double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HQ_H */
