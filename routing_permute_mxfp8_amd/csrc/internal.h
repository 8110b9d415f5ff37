// Launchers shared between the C-ABI layer (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- routing (routing.hip) ----------------------------------------------------
// Stable counting sort of F flat keys (expert ids) restricted to [s, e), split in
// `nch` chunks of `chunk` keys (chunk % 64 == 0). Positions are relative to the
// start of the active segment.
struct RouteParams {
  const void* keys = nullptr;   // int32 or int64 [flat]
  int key_is64 = 0;
  int64_t flat = 0;
  int topk = 1;
  int s = 0, e = 0;             // active experts [s, e); A = e - s buckets
  int nch = 1, chunk = 64;
  // workspace
  int* hist = nullptr;          // [A * nch], expert-major: rows of (expert, chunk)
  int* base = nullptr;          // [A * nch], expert-major: rows of the expert in earlier chunks
  int* totals = nullptr;        // [A] rows per active expert
  int* offsets = nullptr;       // [A + 1] exclusive prefix of the active counts
  // outputs (nullable unless stated)
  int64_t* avail64 = nullptr;   // availableIdxNum
  int64_t* expert_tokens = nullptr;
  int tokens_type = 1;          // 1 count, 0 inclusive cumsum
  int32_t* token_nums32 = nullptr;
  int32_t* scat = nullptr;      // [flat] position of each flat row, -1 outside [s, e) (required)
  int32_t* gath = nullptr;      // [avail] flat row at each position
  int32_t* gath_fill = nullptr; // if set (== gath), positions [avail, flat) are written -1
  int32_t* row_token = nullptr; // [avail] flat row / topk at each position
  float* row_weight = nullptr;  // [avail] gate weight at each position
  const void* topk_w = nullptr; // fp32 or bf16 [flat]
  int topk_w_bf16 = 0;
};
hipError_t launch_routing(const RouteParams& p, hipStream_t stream);
// key_value counts from the active offsets [active + 1] of a routing pass: int64
// out[rows][2] = (s + a, count) for the experts with count > 0, ascending, then zeros.
hipError_t launch_key_value(const int* offsets, int active, int s, int rows, int64_t* out, hipStream_t stream);

// Chunks of up to `tm` rows (tm a multiple of 16) over groups given by int32 offsets
// [groups + 1] (clamped into [0, rows], non-decreasing):
//   tiles[j] = {group, padded row0, nrows, sorted row0},
// where the padded row space gives every group a whole number of 16-row tiles (see
// t16_padded_rows). *count = number of chunks (at most max_tiles are written).
hipError_t launch_build_tiles(const int* offsets, int groups, int rows, int tm, int max_tiles, int4* tiles,
                              int* count, hipStream_t stream);

// ---- tiled token layout (tiles.hip; layout in device_common.h) --------------------
// Upper bound of the padded row count of `rows` rows split into `groups` groups.
inline int64_t t16_padded_rows(int64_t rows, int64_t groups) {
  const int64_t p = rows + 15 * (rows < groups ? rows : groups);
  return (p + 15) / 16 * 16;
}
inline int64_t t16_code_bytes(int64_t padded_rows, int64_t k) { return padded_rows * k; }
inline int64_t t16_scale_bytes(int64_t padded_rows, int64_t k) { return padded_rows / 16 * ((k / 128 + 3) / 4) * 256; }

// Gather of the rows of each chunk (source token = row_token[sorted row], or the sorted
// row itself when row_token is null) with MX quantization, into the tiled layout.
struct PermuteTilesParams {
  const void* x = nullptr;       // [tokens, hidden] of in_dtype
  int in_dtype = 2;              // MOE_DTYPE_* (0 fp32, 1 fp16, 2 bf16)
  int hidden = 0;                // multiple of 128
  const int32_t* row_token = nullptr;
  const int4* chunks = nullptr;
  const int* chunk_count = nullptr;
  int max_chunks = 0, tt = 1;    // tt = 16-row tiles per chunk
  int fmt = 0;                   // 0 E4M3FN, 1 E5M2
  uint8_t* out = nullptr;        // tiled codes
  uint8_t* out_scales = nullptr; // tiled scales
};
hipError_t launch_permute_tiles(const PermuteTilesParams& p, hipStream_t stream);
// Row-major codes [rows, K] / scales [rows, K/32] (sorted rows) <-> tiled layout; the pack
// may gather (sorted row i <- source row row_token[i]).
hipError_t launch_pack_tokens(const uint8_t* codes, const uint8_t* scales, int K, const int4* chunks,
                              const int* chunk_count, int max_chunks, int tt, uint8_t* out, uint8_t* out_scales,
                              hipStream_t stream, const int32_t* row_token = nullptr);
hipError_t launch_unpack_tokens(const uint8_t* in, const uint8_t* in_scales, int K, const int4* chunks,
                                const int* chunk_count, int max_chunks, int tt, uint8_t* codes, uint8_t* scales,
                                hipStream_t stream);

// ---- permute + MX quantization (permute_quant.hip) ------------------------------
struct PermuteParams {
  const void* x = nullptr;      // [n, hidden] of in_dtype
  int in_dtype = 2;             // MOE_DTYPE_* (0 fp32, 1 fp16, 2 bf16)
  int64_t n = 0, hidden = 0;
  int topk = 1;
  const int32_t* scat = nullptr;  // [n * topk] destination rows (-1 = none); nullptr = identity
  int64_t m_limit = 0;          // only destinations < m_limit are written
  int quant = -1;               // -1 copy, 0 E4M3FN, 1 E5M2
  void* out = nullptr;          // [m_limit, hidden] codes or values
  uint8_t* out_scales = nullptr;  // [m_limit, scale_cols]
  int64_t scale_cols = 0;
  uint8_t* tok_out = nullptr;   // optional token-order copy [n, hidden] (MX modes only)
  uint8_t* tok_scales = nullptr;
};
hipError_t launch_permute(const PermuteParams& p, hipStream_t stream);
// Byte rows: out[dest] = x[t] for each destination of token t (scat as above, identity
// when null), row_bytes bytes a row.
hipError_t launch_permute_rows(const uint8_t* x, int64_t n, int64_t row_bytes, int topk, const int32_t* scat,
                               int64_t m_limit, uint8_t* out, hipStream_t stream);

// ---- grouped GEMMs (gmm.hip) -------------------------------------------------------
// GMM1's activation (MOE_ACT_* kinds; validated and defaulted by the API layer).
struct ActParams {
  int kind = 0;                  // 0 swiglu, 1 swiglustep, 2 swigluoai, 3 situglu, 4 gelu
  float clamp = __builtin_huge_valf();   // c; +inf = no clamp
  float alpha = 1.702f;          // swigluoai
  float beta = 1.0f;             // swigluoai beta / situglu beta
  float lin_beta = 0.0f;         // situglu linear beta; 0 = L(U) = U
};
constexpr int kActGelu = 4;
constexpr int kActSwigluNoClamp = 5;   // kind 0 with c = +inf (an instance of the streaming GMM1)

// Token operands and GMM1's requantized output are in the tiled layout, indexed by the
// chunks' padded rows; h1, o, row_token and row_weight are indexed by sorted rows.
// A shared expert folded into the routed experts' launch of an LDS-streaming GEMM: the
// chunks of group `group` take their weights from w / ws (one expert, the routed
// experts' format); their rows are in the launch's token and output buffers like the
// routed ones. w = nullptr: none.
struct SharedGroups {
  int group = 0;
  const uint8_t* w = nullptr;
  const uint8_t* ws = nullptr;
};

// The chunk list of an LDS-streaming GEMM split by chunk size: class c (list tiles +
// c stride, count[c]) holds the chunks of more than 4 kStreamClassRT[c - 1] and at most
// 4 kStreamClassRT[c] token tiles, run by the instance with kStreamClassRT[c] token tiles
// a wave (a 5-tile wave's MFMAs for a 40-row chunk would be mostly idle tiles); the
// classes run as phases of one launch. tiles = nullptr: one list, the 5-tile instance.
constexpr int kStreamClasses = 3;
constexpr int kStreamClassRT[kStreamClasses] = {2, 4, 5};
struct StreamClasses {
  const int4* tiles = nullptr;
  const int* count = nullptr;
  int stride = 0;
};

// Every chunk list of one layer call in one launch (one workgroup, routing.hip):
// * tiles[0, *count): the routed experts' chunks, as launch_build_tiles (offsets, groups,
//   rows, tm, max_tiles);
// * count_all != nullptr: one shared expert folded in, its chunks (group sh_group over
//   sh_rows token rows in chunks of sh_tm rows, padded rows sh_prow0 + r, sorted rows
//   sh_srow0 + r) right after the routed ones; *count_all = all chunks;
// * sh_tiles != nullptr: the shared expert's own list, {0, i sh_tm, rows, i sh_tm};
// * cls_tiles != nullptr: all chunks split into the classes above (stable order), class c
//   at cls_tiles + c cls_stride, cls_count[c].
struct ChunkListParams {
  const int* offsets = nullptr;
  int groups = 0, rows = 0, tm = 0, max_tiles = 0;
  int4* tiles = nullptr;
  int* count = nullptr;
  int sh_rows = 0, sh_tm = 16, sh_group = 0, sh_prow0 = 0, sh_srow0 = 0;
  int* count_all = nullptr;
  int4* sh_tiles = nullptr;
  int* sh_count = nullptr;
  int4* cls_tiles = nullptr;
  int* cls_count = nullptr;
  int cls_stride = 0;
};
hipError_t launch_chunk_lists(const ChunkListParams& p, hipStream_t stream);

struct Gmm1Params {
  const uint8_t* xq; const uint8_t* sx;        // tiled [padded rows, H]
  const uint8_t* w; const uint8_t* ws;         // [G, 2I, H], [G, 2I, H/32]
  const int4* tiles; const int* tile_count; int max_tiles;
  int hidden, inter, fmt, tt;                  // tt = 16-row token tiles per chunk (1, 2, 4, 8, kStreamTiles)
  uint8_t* aq; uint8_t* sa;                    // tiled [padded rows, I] (2I for gelu)
  float* h1;                                   // nullable [rows, 2I]
  int packed;                                  // weights in the MFMA-native packed layout
  ActParams act;                               // A = act(G, U) [rows, I], or gelu(Z) [rows, 2I]
  int wfp4 = 0;                                // weights MXFP4 E2M1 (codes [G, 2I, H/2]; fmt must be E4M3)
  SharedGroups shared;                         // LDS-streaming kernels only
  StreamClasses classes;                       // LDS-streaming kernels only
};
hipError_t launch_gmm1(const Gmm1Params& p, hipStream_t stream);

struct Gmm2Params {
  const uint8_t* aq; const uint8_t* sa;        // tiled [padded rows, I]
  const uint8_t* w; const uint8_t* ws;         // [G, H, I], [G, H, I/32]
  const int4* tiles; const int* tile_count; int max_tiles;
  int hidden, inter, fmt, tt;
  float* o;                                    // [rows, H] fp32, sorted rows
  int packed;
  int wfp4 = 0;                                // weights MXFP4 E2M1 (codes [G, H, I/2]; fmt must be E4M3)
  uint16_t* o16 = nullptr;                     // if set, O rows go here as bf16 (RNE) instead of o
  SharedGroups shared;                         // LDS-streaming kernels only
  StreamClasses classes;                       // LDS-streaming kernels only
};
hipError_t launch_gmm2(const Gmm2Params& p, hipStream_t stream);

// Token tiles (16 rows each) per chunk for `rows` rows over `groups` groups of an FFN of
// width hidden x inter (A of width aw): 1, 2, 4 or 8 (the register-streaming kernels of
// gmm.hip), or kStreamTiles (the LDS-streaming kernels of gmm_stream.hip) for layers whose
// experts hold more than 128 rows on average, when both GEMMs have a multiple of 4
// 128-wide K steps and one expert's weights stay below 2 GiB.
int gmm_token_tiles(int64_t rows, int64_t groups, int64_t hidden, int64_t inter, int64_t aw);
constexpr int kStreamTiles = 20;
hipError_t launch_gmm1_stream(const Gmm1Params& p, hipStream_t stream);
hipError_t launch_gmm2_stream(const Gmm2Params& p, hipStream_t stream);

// codes [G, N, K] + scales [G, N, K/32] -> MFMA-native packed codes (same size) and
// packed scales [G, N/16, ceil(K/512), 64, 4].
hipError_t launch_pack_weights(const uint8_t* codes, const uint8_t* scales, int64_t groups, int64_t n, int64_t k,
                               uint8_t* packed, uint8_t* packed_scales, hipStream_t stream);

// MXFP4 codes [G, N, K/2] + scales [G, N, K/32] -> packed codes [G, N/16, K/128, 64, 16 B]
// (1 KB tiles) and the same packed scales.
hipError_t launch_pack_weights_fp4(const uint8_t* codes, const uint8_t* scales, int64_t groups, int64_t n, int64_t k,
                                   uint8_t* packed, uint8_t* packed_scales, hipStream_t stream);


// ---- weighted combine (combine.hip) -------------------------------------------------
// Y[t] = bf16(sum_k w[t, k] * O[pos[t*K + k]] + sum_s O_shared[s][t]) for every token t:
// O [rows, H] fp32 in sorted-row order, pos the scatter index (flat row -> sorted row,
// -1 = none), w fp32 or bf16 [tokens * K], O_shared [num_shared][tokens, H] or null.
struct CombineParams {
  const void* o = nullptr;         // expert output rows: fp32, or bf16 when o_fmt == 2
  int o_fmt = 0;                   // 0 fp32, 1 fp32 rounded to bf16 as read, 2 bf16
  int sh_bf16 = 0;                 // shared rows stored bf16 (else fp32)
  const int32_t* pos = nullptr;
  const void* w = nullptr;
  int w_bf16 = 0;
  int topk = 1;
  const void* o_shared = nullptr;
  int num_shared = 0;
  int64_t tokens = 0;
  int hidden = 0;                  // multiple of 4
  uint16_t* y = nullptr;           // bf16 [tokens, H]
};
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);
// y_accum[row_token[r]] += row_weight[r] * O[r] (fp32 atomics), rows [0, rows).
hipError_t launch_scatter_add(const float* o, int64_t rows, int hidden, const int32_t* row_token,
                              const float* row_weight, float* y_accum, hipStream_t stream);
hipError_t launch_finalize(const float* acc, int64_t count, uint16_t* y, hipStream_t stream);


// ---- static scratch of the allocation-free entry point (noalloc.hip) ---------------------
// Bytes of the per-device scratch array moe_init_routing_noalloc uses instead of a
// caller workspace.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
// Device address of this device's scratch array (looked up once per device and kept).
hipError_t noalloc_scratch(void** out);

// ---- measured peaks (peaks.hip) ------------------------------------------------------
// mode 0: non-temporal read, 1: non-temporal copy, 2: plain (cache-filling) read
hipError_t launch_probe_stream(int mode, const void* src, void* dst, int64_t bytes, hipStream_t stream);
int probe_mfma_blocks();   // blocks of 256 threads the MFMA probe launches (one per CU)
hipError_t launch_probe_mfma(int iters, float* out, hipStream_t stream);
double probe_mfma_flops(int iters);

}  // namespace moe
