/*
 * moe_mx.h - C ABI of the MI355X (gfx950) MoE-layer hot path:
 *   routing (stable counting sort of expert ids, inverse index, per-expert
 *   histogram) -> gather of token rows with MX quantization (FP8 E4M3FN/E5M2
 *   elements, E8M0 scale per 32) -> grouped GEMM1 + SwiGLU + MX requantization
 *   -> grouped GEMM2 -> topK-weighted combine into bf16 Y.
 *
 * Operator pages this follows:
 *   [V3]  "MoeInitRoutingV3" README (cann/ops-transformer moe/moe_init_routing_v3):
 *         计算公式 steps 1-6, 参数说明 (activeExpertRange, rowIdxType,
 *         expertTokensNumType, quantMode), 约束说明.
 *   [TP]  "moe_token_permute" article (CANN ops-transformer, torch_npu API):
 *         功能说明, 参数说明, 返回值说明, 约束说明.
 *   [MM]  "MegaMoE" README (ops-transformer mc2/mega_moe): "A8W8-FP quantization
 *         scenario", "Activation function formulas", "Parameter Description",
 *         "MXFP quantization scenario constraints".
 *
 * Conventions for every entry point
 *   - Pointers named as device buffers are device memory owned by the caller;
 *     the library never frees or keeps them. Host pointers are marked "host".
 *   - Calls are asynchronous: they validate on the host, enqueue kernels on
 *     `stream` (a hipStream_t; NULL = the null stream) and return. There is no
 *     host<->device synchronisation inside a call.
 *   - All validation happens before any launch. On an error status nothing has
 *     been enqueued and no output has been written; moe_last_error() returns a
 *     message for the calling thread (for MOE_ERR_WORKSPACE it names the byte
 *     count required). There is no silent truncation or fallback.
 *   - Scratch memory is the caller's: each call takes a device `workspace` of at
 *     least the size its *_workspace_size query reports (256-byte aligned).
 *   - Preconditions the host cannot check without reading device memory (expert
 *     ids in [0, expert_num), distinct ids per token for mega_moe, finite
 *     activations) are the caller's; violating them gives undefined results.
 *   - Results are deterministic (bit-identical on repeated calls), except the
 *     y_accum of moe_gmm2_combine, which adds each row's weighted O into it with
 *     fp32 atomics in no fixed order. mega_moe's y is deterministic: its combine
 *     gathers each token's expert rows and sums them in a fixed order.
 */
#ifndef MOE_MX_H
#define MOE_MX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, bad enum value, negative size */
  MOE_ERR_SHAPE = 2,        /* sizes inconsistent or outside the supported range */
  MOE_ERR_DTYPE = 3,        /* dtype not supported for this mode */
  MOE_ERR_UNSUPPORTED = 4,  /* a mode the pages define that this library does not implement */
  MOE_ERR_WORKSPACE = 5,    /* workspace too small (message gives the required bytes) */
  MOE_ERR_HIP = 6           /* a HIP runtime call or kernel launch failed */
} moe_status;

/* Element dtypes of activation buffers. */
enum { MOE_DTYPE_FP32 = 0, MOE_DTYPE_FP16 = 1, MOE_DTYPE_BF16 = 2,
       MOE_DTYPE_INT32 = 3, MOE_DTYPE_INT64 = 4,
       /* MX codes (moe_init_routing x only): one byte per FP8 element, two FP4    */
       /* elements per byte (element 2j in the low nibble)                          */
       MOE_DTYPE_FP8_E5M2 = 5, MOE_DTYPE_FP8_E4M3 = 6, MOE_DTYPE_FP4_E2M1 = 7 };

/* quantMode values of [V3] / quant_mode of [TP]: -1 none, 2 MXFP8 E5M2, 3 MXFP8 E4M3FN, */
/* 9 MXFP4 E2M1. MXFP4 codes are stored two per byte: element 2j in the low nibble,   */
/* 2j + 1 in the high nibble, so a row of `hidden` elements takes hidden / 2 bytes; E2M1 */
/* has magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (sign bit 0x8, no inf or NaN), emax 2.       */
enum { MOE_QUANT_NONE = -1, MOE_QUANT_MXFP8_E5M2 = 2, MOE_QUANT_MXFP8_E4M3 = 3, MOE_QUANT_MXFP4_E2M1 = 9 };

/* dispatchQuantOutDtype values of [MM]: 23 FLOAT8_E5M2, 24 FLOAT8_E4M3FN; weight type */
/* 296 FLOAT4_E2M1 (MXFP4 weights of the A8W4-FP scenario).                         */
enum { MOE_FP8_E5M2 = 23, MOE_FP8_E4M3 = 24, MOE_FP4_E2M1 = 296 };

/* rowIdxType of [V3]: 0 gather-type index, 1 scatter-type index. */
enum { MOE_ROW_IDX_GATHER = 0, MOE_ROW_IDX_SCATTER = 1 };

/* expertTokensNumType of [V3]: 0 cumsum, 1 count, 2 key_value. */
enum { MOE_TOKENS_CUMSUM = 0, MOE_TOKENS_COUNT = 1, MOE_TOKENS_KEY_VALUE = 2 };

/* Largest expert count accepted ([V3] expertNum range, non key_value modes). */
#define MOE_MAX_EXPERTS 10240
/* Flat index limit of [TP] 约束说明: numel(indices) < 16777215. */
#define MOE_MAX_FLAT_ROWS 16777215

/* Message describing the last error of the calling thread ("" if none). */
const char* moe_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int moe_version(void);

/* MX scale columns for `cols` elements per row: AlignUp(CeilDiv(cols, 32), 2)
 * ([TP] 返回值说明; [MM] weightScales (.., CeilDiv(K, 64), 2) is the same bytes). */
int64_t moe_mx_scale_cols(int64_t cols);

/* ------------------------------------------------------------------------ */
/* MX quantization of rows (weight preparation; the same Q_MX as stage 1 of   */
/* [MM] "A8W8-FP quantization scenario").                                    */
/*   x        device, [rows, cols] of `dtype` (BF16, FP16 or FP32), row-major */
/*   quant_mode  MOE_QUANT_MXFP8_E5M2, MOE_QUANT_MXFP8_E4M3 or MOE_QUANT_MXFP4_E2M1 */
/*   codes    device out, uint8 [rows, cols] FP8 codes ([rows, cols / 2] MXFP4) */
/*   scales   device out, uint8 [rows, moe_mx_scale_cols(cols)] E8M0 bytes;   */
/*            a padding column (odd group count) is written as 0x00           */
/* Scale rule: E8M0 = clamp(floor(log2(amax of the 32-group)) - emax + 127,   */
/* 0, 254), emax 8 (E4M3) / 15 (E5M2) / 2 (E2M1), 0 for an all-zero group;    */
/* elements are x / 2^(E8M0-127) rounded to nearest-even and clamped to the     */
/* largest finite value of the format, sign kept. Requires cols % 8 == 0. No    */
/* workspace.                                                                   */
/* ------------------------------------------------------------------------ */
moe_status moe_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int quant_mode,
                           uint8_t* codes, uint8_t* scales, void* stream);

/* ------------------------------------------------------------------------ */
/* Weight formats. MOE_WEIGHTS_ND is the pages' layout ([MM] "MXFP quantization */
/* scenario constraints": codes [G, N, K], scales [G, N, K/32]). MOE_WEIGHTS_PACKED */
/* is this library's MFMA-native layout (the analog of the pages' fractal weight  */
/* formats): codes in 16-channel x 128-K tiles of 2048 bytes in MFMA lane order   */
/* (tile (g, n/16, k/128), then half h, lane l: row 16*(n/16) + l%16, K bytes       */
/* [128*(k/128) + 64*h + 16*(l/16), +16)), same total size; scales as one dword per */
/* lane per 4 K steps: [G][N/16][CeilDiv(K, 512)][64][4] bytes.                     */
/* moe_mx_pack_weights converts ND codes/scales to the packed layout on `stream`;   */
/* moe_mx_packed_scale_bytes gives the packed scale size. N % 16 == 0 and           */
/* K % 128 == 0 are required.                                                        */
/* ------------------------------------------------------------------------ */
enum { MOE_WEIGHTS_ND = 0, MOE_WEIGHTS_PACKED = 1 };
/* MXFP4 weights (A8W4-FP): codes [groups, n, k/2] (two a byte) -> packed codes        */
/* [groups, n/16, k/128, 64, 16 B] (the same byte count) and packed scales as above.   */
moe_status moe_mx_pack_weights_fp4(const uint8_t* codes, const uint8_t* scales, int64_t groups, int64_t n,
                                   int64_t k, uint8_t* packed_codes, uint8_t* packed_scales, void* stream);
int64_t moe_mx_packed_scale_bytes(int64_t groups, int64_t n, int64_t k);
moe_status moe_mx_pack_weights(const uint8_t* codes, const uint8_t* scales, int64_t groups, int64_t n,
                               int64_t k, uint8_t* packed_codes, uint8_t* packed_scales, void* stream);

/* ------------------------------------------------------------------------ */
/* moe_init_routing  ([V3] 计算公式 1-6, dropless mode).                      */
/*   x            device, [num_rows, hidden] of x_dtype (BF16, FP16; FP32 too  */
/*                when quant_mode = -1), or MX codes (MOE_DTYPE_FP8_E5M2,       */
/*                _FP8_E4M3: [num_rows, hidden] bytes; _FP4_E2M1: [num_rows,    */
/*                hidden/2] bytes, hidden even) with quant_mode = -1: the rows  */
/*                are gathered as they are ([V3] quantMode -1 with an FP8/FP4 x) */
/*   scale        device or NULL ([V3] scaleOptional): only with x of MX codes,  */
/*                their E8M0 scales [num_rows, moe_mx_scale_cols(hidden)]       */
/*                (hidden % 32 == 0); expanded_scale then receives the gathered */
/*                scale rows (expandedScaleOut). Any other use: an error.       */
/*   expert_idx   device, int32 [num_rows, k]; flat row r = t*k + j            */
/*   expert_num   number of experts E, 1..MOE_MAX_EXPERTS                      */
/*   active_start, active_end  activeExpertRange [s, e), 0 <= s <= e <= E     */
/*   quant_mode   -1, 2, 3 or 9 (MX modes need hidden % 32 == 0)               */
/*   row_idx_type 0 gather / 1 scatter; expert_tokens_num_type 0 cumsum /      */
/*                1 count / 2 key_value (then expert_num <= 5120)               */
/* Outputs (device):                                                            */
/*   expanded_x        [num_rows*k, hidden]: row i (< availableIdxNum) holds     */
/*                     Q(x[src(i) / k]) where src(i) is the flat row at position */
/*                     i of the stable expert-major order restricted to [s, e);  */
/*                     FP8 codes in MX modes (packed MXFP4, hidden / 2 bytes a  */
/*                     row, in mode 9), x_dtype values otherwise (x's code rows */
/*                     when x holds MX codes). Rows >= availableIdxNum are not  */
/*                     written.                                                 */
/*   expanded_row_idx  int32 [num_rows*k]. Scatter type: entry r = position of   */
/*                     flat row r in expanded_x, or -1 if its expert is outside  */
/*                     [s, e). Gather type: entry i < availableIdxNum = src(i),  */
/*                     the rest -1.                                             */
/*   expert_tokens     int64 [e - s]: per-expert counts (count) or their          */
/*                     inclusive prefix sum (cumsum); key_value: int64           */
/*                     [expert_num, 2], one row (expert id, count) per expert of */
/*                     [s, e) with a non-zero count, ascending, then zero rows   */
/*                     (the pages leave those rows open)                        */
/*   expanded_scale    uint8 [num_rows*k, moe_mx_scale_cols(hidden)] in MX modes  */
/*                     and with a scale input (NULL allowed otherwise)          */
/*   available_idx_num int64 [1]: #{r : s <= expert_idx[r] < e}                 */
/* Ties between equal experts keep ascending flat row (stable sort).            */
/* ------------------------------------------------------------------------ */
moe_status moe_init_routing_workspace_size(int64_t num_rows, int64_t k, int64_t expert_num,
                                           size_t* bytes /* host out */);
moe_status moe_init_routing(const void* x, int x_dtype, const uint8_t* scale, int64_t num_rows, int64_t hidden,
                            const int32_t* expert_idx, int64_t k, int64_t expert_num,
                            int64_t active_start, int64_t active_end, int quant_mode,
                            int row_idx_type, int expert_tokens_num_type, void* expanded_x,
                            int32_t* expanded_row_idx, int64_t* expert_tokens,
                            uint8_t* expanded_scale, int64_t* available_idx_num,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* moe_init_routing_noalloc: moe_init_routing without a workspace, for callers */
/* that cannot allocate device memory (code under HIP graph capture, tight     */
/* serving loops, harnesses that forbid hipMalloc). Same arguments, outputs,    */
/* kernels and results as moe_init_routing; its scratch is a static array of    */
/* 8 MiB (8388608 bytes) that each GPU holds from the library's load until the  */
/* process ends. The call allocates nothing (no hipMalloc / hipFree). A call     */
/* whose scratch would exceed 8 MiB returns MOE_ERR_SHAPE before any launch (the */
/* message gives the bytes it needs); any call whose moe_init_routing_workspace_ */
/* size is at most 8388608 fits (e.g. num_rows*k up to 1397696 with 256 experts). */
/* Every call on one GPU shares that GPU's array and leaves its contents behind  */
/* (nothing in it needs to start at zero): calls that overlap on one GPU (other  */
/* streams, other threads) race and must be ordered by the caller.             */
/* ------------------------------------------------------------------------ */
moe_status moe_init_routing_noalloc(const void* x, int x_dtype, const uint8_t* scale, int64_t num_rows,
                                    int64_t hidden, const int32_t* expert_idx, int64_t k, int64_t expert_num,
                                    int64_t active_start, int64_t active_end, int quant_mode, int row_idx_type,
                                    int expert_tokens_num_type, void* expanded_x, int32_t* expanded_row_idx,
                                    int64_t* expert_tokens, uint8_t* expanded_scale, int64_t* available_idx_num,
                                    void* stream);

/* ------------------------------------------------------------------------ */
/* moe_token_permute  ([TP] 功能说明 / 返回值说明, padded_mode = False).        */
/*   tokens        device, [n, hidden] of dtype (BF16, FP16; FP32 too for -1)  */
/*   indices       device, int32 or int64 (indices_dtype) [n] (topk = 1) or     */
/*                 [n, topk]; F = n*topk must be < MOE_MAX_FLAT_ROWS            */
/*   num_experts   exclusive bound on index values (the counting sort's bucket */
/*                 count; the torch API infers it, this boundary takes it)     */
/*   num_out_tokens  0 = None; > 0 keeps min(n_out, F) rows; < 0 drops |n_out| */
/*                 rows from the end (M = max(F + n_out, 0))                   */
/*   padded_mode   must be 0 (MOE_ERR_UNSUPPORTED otherwise)                   */
/*   quant_mode    -1, 2, 3 or 9 (permuted_tokens rows of hidden / 2 bytes)      */
/* Outputs (device):                                                            */
/*   permuted_tokens  [M, hidden]: row i = Q(tokens[first(i) / topk]) where      */
/*                    first = stable argsort of the flattened indices           */
/*   sorted_indices   int32 [F] (never truncated): the inverse of first          */
/*   expanded_scale   uint8 [M, moe_mx_scale_cols(hidden)] in MX modes, else NULL */
/* ------------------------------------------------------------------------ */
int64_t moe_token_permute_out_rows(int64_t flat_rows, int64_t num_out_tokens);
moe_status moe_token_permute_workspace_size(int64_t flat_rows, int64_t num_experts,
                                            size_t* bytes /* host out */);
moe_status moe_token_permute(const void* tokens, int dtype, int64_t n, int64_t hidden,
                             const void* indices, int indices_dtype, int64_t topk,
                             int64_t num_experts, int64_t num_out_tokens, int padded_mode,
                             int quant_mode, void* permuted_tokens, int32_t* sorted_indices,
                             uint8_t* expanded_scale, void* workspace, size_t workspace_bytes,
                             void* stream);

/* ------------------------------------------------------------------------ */
/* mega_moe  ([MM] "A8W8-FP quantization scenario", all experts local: the    */
/* cross-rank Dispatch/Combine becomes an on-device permute/unpermute).       */
/*   stage 1  X^, S_X = Q_MX(x rows gathered expert-contiguously)              */
/*   stage 2  G = DQ(X^).DQ(W1[:, :I]),  U = DQ(X^).DQ(W1[:, I:]),             */
/*            A = SiLU(G) * U (fp32),  A^, S_A = Q_MX(A) with the same FP8 type */
/*   stage 3  O = DQ(A^).DQ(W2)                                                 */
/*   stage 4  y[t] = bf16( sum_k w[t,k] O[row(t,k)] + sum_s O_shared_s[t] )    */
/*            with every O row first rounded to bf16 (combine_comm_mode 0) or    */
/*            kept fp32 (combine_comm_mode 1), the sum in fp32                  */
/* Shapes ([MM] "MXFP quantization scenario constraints"):                     */
/*   x            bf16 [num_tokens, hidden]                                      */
/*   topk_ids     int32 [num_tokens, topk], values in [0, num_experts), distinct */
/*   topk_weights fp32 or bf16 (topk_weights_dtype) [num_tokens, topk]            */
/*   w1           fp8 [num_experts, 2*inter, hidden]; w1_scales uint8            */
/*                [num_experts, 2*inter, hidden/32] (= (.., CeilDiv(hidden,64), 2)) */
/*   w2           fp8 [num_experts, hidden, inter];  w2_scales uint8              */
/*                [num_experts, hidden, inter/32]                                 */
/*                (or both in MOE_WEIGHTS_PACKED layout, see weight_format)       */
/*   shared_*     the same for num_shared (0..4) shared experts, or NULL          */
/*   y            out, bf16 [num_tokens, hidden]                                  */
/*   expert_token_nums  out, int32 [num_experts] (nullable)                       */
/* Limits: hidden % 128 == 0, inter % 128 == 0, topk in [1, 32], num_experts in   */
/* [1, 1024].                                                                    */
/* activation ([MM] "Activation function formulas"; G = first inter channels of   */
/* the GMM1 output, U = the last inter, c the clamp, Gc = min(G, c),              */
/* Uc = clip(U, -c, c), sigma the logistic function):                             */
/*   MOE_ACT_SWIGLU      A = SiLU(Gc) * Uc;             params [] or [clamp]       */
/*   MOE_ACT_SWIGLUSTEP  A = min(SiLU(G), c) * Uc;      params [] or [clamp]       */
/*   MOE_ACT_SWIGLUOAI   A = Gc sigma(alpha Gc)(Uc + beta); params [] or          */
/*                       [clamp, alpha, beta] (defaults: no clamp, 1.702, 1.0)     */
/*   MOE_ACT_SITUGLU     A = beta tanh(G/beta) sigma(G) L(U), L(U) = U, or         */
/*                       lb tanh(U/lb) when linear_beta lb is given; params [],    */
/*                       [beta] or [beta, linear_beta] (default beta 1.0)          */
/*   MOE_ACT_GELU        A = Z sigma(sqrt(8/pi)(Z + 0.044715 Z^3)) on all 2*inter */
/*                       channels Z of the GMM1 output (no split, no clamp):      */
/*                       A and w2's input width are then 2*inter (w2 [num_experts,*/
/*                       hidden, 2*inter], aq/sa [F, 2*inter] / [F, 2*inter/32]);  */
/*                       params [] or the placeholder [FLT_MAX].                    */
/* A clamp of 0 (or none) means no clamp; clamp >= 0, alpha and beta finite,      */
/* situglu's betas finite and > 0; anything else is MOE_ERR_INVALID_ARG.           */
/* Optional device outputs for parity checks (NULL to skip): xq/sx the stage-1    */
/* operands [F, hidden] / [F, hidden/32] in expert-contiguous order; h1 fp32      */
/* [F, 2*inter] (G then U); aq/sa the stage-2 requantized activations            */
/* [F, inter] / [F, inter/32]; o fp32 [F, hidden] (unweighted); sorted_row_idx    */
/* int32 [F] (flat row at each position). F = num_tokens*topk.                    */
/* stage_events (nullable): MOE_MEGA_STAGE_EVENTS hipEvent_t handles (host array, */
/* NULL entries skipped; a timed record costs a few microseconds of GPU time)     */
/* recorded on `stream` at the stage boundaries: [0] start, [1] routing + tile list */
/* done, [2] gather/quantization done, [3] GMM1 done, [4] GMM2 done (O rows        */
/* written), [5] shared experts done, [6] weighted combine into bf16 y done.        */
/* The result is deterministic (no atomics on the mega_moe path).                  */
/* ------------------------------------------------------------------------ */
enum { MOE_ACT_SWIGLU = 0, MOE_ACT_SWIGLUSTEP = 1, MOE_ACT_SWIGLUOAI = 2, MOE_ACT_SITUGLU = 3,
       MOE_ACT_GELU = 4 };
#define MOE_MEGA_STAGE_EVENTS 7

typedef struct {
  const void* x;
  int64_t num_tokens;
  int64_t hidden;
  const int32_t* topk_ids;
  int64_t topk;
  const void* topk_weights;
  int topk_weights_dtype;         /* MOE_DTYPE_FP32 or MOE_DTYPE_BF16 */
  int64_t num_experts;
  int64_t inter;                  /* intermediateHidden I */
  const uint8_t* w1;
  const uint8_t* w1_scales;
  const uint8_t* w2;
  const uint8_t* w2_scales;
  int64_t num_shared;
  const uint8_t* shared_w1;
  const uint8_t* shared_w1_scales;
  const uint8_t* shared_w2;
  const uint8_t* shared_w2_scales;
  int quant_out_dtype;            /* MOE_FP8_E5M2 or MOE_FP8_E4M3 (= the weights' FP8 type) */
  int activation;                 /* MOE_ACT_*, see above */
  int weight_format;              /* MOE_WEIGHTS_ND or MOE_WEIGHTS_PACKED (routed and shared) */
  void* y;
  int32_t* expert_token_nums;
  /* optional parity outputs */
  uint8_t* xq;
  uint8_t* sx;
  float* h1;
  uint8_t* aq;
  uint8_t* sa;
  float* o;
  int32_t* sorted_row_idx;
  void** stage_events;            /* nullable, see above */
  int num_activation_params;      /* 0..3, see the activations above */
  float activation_params[3];
  int weight_dtype;               /* routed w1/w2: 0 or quant_out_dtype = FP8 (A8W8-FP),      */
                                  /* MOE_FP4_E2M1 = MXFP4 (A8W4-FP; needs FLOAT8_E4M3FN x)  */
  int shared_weight_dtype;        /* shared experts: 0 = as weight_dtype, or as above        */
  int x_is_quantized;             /* 0: x is bf16, quantized inside ([MM] dispatchQuantMode 4); */
                                  /* 1: pre-quantized pass-through (dispatchQuantMode 0): x   */
                                  /* holds FP8 codes of quant_out_dtype [num_tokens, hidden]  */
                                  /* and x_scales their E8M0 scales [num_tokens, hidden/32];  */
                                  /* stage 1 only gathers them                                */
  const uint8_t* x_scales;        /* device, with x_is_quantized; else NULL                 */
  int combine_comm_mode;          /* [MM] combineCommMode with every expert on this card:   */
                                  /* 0 (the pages' default, no deduplication): each expert's */
                                  /* output row, routed or shared, reaches the combine as   */
                                  /* BF16 and the weighted sum of those rows (fp32) is      */
                                  /* rounded to bf16 y; 1 (intra-card deduplication): a     */
                                  /* token's expert outputs are summed in fp32 and rounded  */
                                  /* once. The o parity output stays fp32 either way. Other */
                                  /* values: MOE_ERR_UNSUPPORTED (2 is a multi-server mode) */
} moe_mega_args;

/* A8W4-FP ([MM] "A8W4-FP quantization scenario"): with weight_dtype MOE_FP4_E2M1 the  */
/* routed w1 / w2 hold MXFP4 codes two a byte (element 2j in the low nibble): w1      */
/* uint8 [num_experts, 2*inter, hidden/2], w2 [num_experts, hidden, A/2] (A = inter,   */
/* or 2*inter for gelu), scales as for FP8 (E8M0, one per 32 along K); in the packed  */
/* weight format they come from moe_mx_pack_weights_fp4. X^ and A^ stay MXFP8 E4M3,   */
/* so both GEMMs multiply FP8 activations by FP4 weights on the matrix cores.          */
/* The shared experts may use the other weight type (shared_weight_dtype).             */
moe_status mega_moe_workspace_size(const moe_mega_args* args /* host */, size_t* bytes /* host out */);
moe_status mega_moe(const moe_mega_args* args /* host */, void* workspace, size_t workspace_bytes,
                    void* stream);

/* ------------------------------------------------------------------------ */
/* Stage entry points (the kernels mega_moe runs, on caller-given operands).  */
/*                                                                            */
/* moe_gmm1_swiglu_quant: [MM] stage 2 for a grouped batch.                   */
/*   xq, sx        device, fp8 [rows, hidden], uint8 [rows, hidden/32]         */
/*   group_offsets device, int32 [num_groups + 1], ascending, [0] = 0,         */
/*                 [num_groups] = rows: rows of group g are [off[g], off[g+1]) */
/*   w1, w1_scales as in mega_moe with num_groups experts                      */
/*   aq, sa        device out, fp8 [rows, inter], uint8 [rows, inter/32]       */
/*   h1            device out, fp32 [rows, 2*inter] or NULL                    */
/* moe_gmm2_combine: [MM] stages 3-4 for a grouped batch (O computed, then     */
/*   scattered into y_accum).                                                    */
/*   aq, sa        device, fp8 [rows, inter], uint8 [rows, inter/32]           */
/*   row_token     device, int32 [rows]: token receiving each row             */
/*   row_weight    device, fp32 [rows]: its combine weight                     */
/*   y_accum       device in/out, fp32 [num_tokens, hidden]: y_accum[token] +=  */
/*                 weight * O[row] (accumulated atomically)                    */
/*   o             device out, fp32 [rows, hidden] unweighted O, or NULL        */
/* moe_combine_finalize: y (bf16 [num_tokens, hidden]) = RNE(y_accum).         */
/* Limits as in mega_moe; fp8 = quant_out_dtype (23/24); weights in           */
/* weight_format. Workspace: moe_gmm_workspace_size (the same for both, given  */
/* rows, num_groups, hidden and inter; it holds the chunk list, the token      */
/* operands restaged into the kernels' tiled layout, each group padded to 16  */
/* rows: (rows + 15 * min(rows, num_groups)) * (max(hidden, inter) + inter)   */
/* bytes of codes plus 1/32 of that for scales, roughly, and an fp32 [rows,    */
/* hidden] O buffer).                                                          */
/* ------------------------------------------------------------------------ */
moe_status moe_gmm_workspace_size(int64_t rows, int64_t num_groups, int64_t hidden, int64_t inter,
                                  size_t* bytes /* host out */);
moe_status moe_gmm1_swiglu_quant(const uint8_t* xq, const uint8_t* sx, int64_t rows, int64_t hidden,
                                 int64_t inter, const int32_t* group_offsets, int64_t num_groups,
                                 const uint8_t* w1, const uint8_t* w1_scales, int weight_format, int quant_out_dtype,
                                 uint8_t* aq, uint8_t* sa, float* h1, void* workspace,
                                 size_t workspace_bytes, void* stream);
moe_status moe_gmm2_combine(const uint8_t* aq, const uint8_t* sa, int64_t rows, int64_t inter,
                            int64_t hidden, const int32_t* group_offsets, int64_t num_groups,
                            const uint8_t* w2, const uint8_t* w2_scales, int weight_format, int quant_out_dtype,
                            const int32_t* row_token, const float* row_weight, int64_t num_tokens,
                            float* y_accum, float* o, void* workspace, size_t workspace_bytes,
                            void* stream);
moe_status moe_combine_finalize(const float* y_accum, int64_t num_tokens, int64_t hidden, void* y,
                                void* stream);

/* ------------------------------------------------------------------------ */
/* Measured peaks for the roofline report (one launch each; the caller times   */
/* it with events on `stream`).                                                */
/* moe_probe_stream: mode 0 reads `bytes` from src (dst receives nothing      */
/*   unless an impossible value turns up; give a 16-byte buffer), mode 1     */
/*   copies them to dst, both with non-temporal accesses (the GPU's best      */
/*   streaming rates); mode 2 reads like mode 0 with plain, cache-filling      */
/*   loads (evicts other data from the caches, e.g. before a cold-cache       */
/*   timing). bytes: a positive multiple of 16; both device. Any other mode:   */
/*   MOE_ERR_INVALID_ARG.                                                     */
/* moe_probe_mfma: `iters` rounds of 16 independent V_MFMA_SCALE 16x16x128    */
/*   FP8 products per wave, two 256-thread blocks per compute unit; out:     */
/*   device fp32, at least *out_floats (host out, may be queried with        */
/*   out = NULL) elements; *flops (host out) = MFMA flops of the launch.     */
/* ------------------------------------------------------------------------ */
moe_status moe_probe_stream(int mode, const void* src, void* dst, int64_t bytes, void* stream);
moe_status moe_probe_mfma(int iters, float* out, int64_t* out_floats, double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MX_H */
