// C ABI of the MoE-layer hot path (include/moe_mx.h): host-side validation,
// workspace carving and the launch sequence of each entry point. Every check
// runs before the first launch; on an error nothing is enqueued. Error policy
// follows the MegaMoE README (Constraints: errors are raised before the kernel
// runs and report the bytes needed, without silent truncation or fallback).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "moe_mx.h"
#include "internal.h"

namespace {

thread_local std::string g_error;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

moe_status ok() {
  g_error.clear();
  return MOE_OK;
}

moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Bump allocator over the caller's workspace; with base == nullptr it only measures.
struct Carver {
  uint8_t* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<uint8_t*>(b)) {}
  template <class T>
  T* take(size_t count) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += std::max<size_t>(count, 1) * sizeof(T);
    return p;
  }
};

int64_t scale_cols(int64_t cols) {
  const int64_t g = (cols + 31) / 32;
  return g + (g & 1);
}

// Chunking of the routing passes: chunk of 256 rows (<= 4Ki rows) or 1024, grown
// until the per-chunk histogram table stays within 2Mi entries. 1024-row chunks keep the
// chunk count of mid-size layers (24Ki-64Ki rows) at or below 64, where the scatter pass
// scans the histogram itself (two launches instead of three or four).
void route_chunks(int64_t flat, int active, int* nch, int* chunk) {
  int64_t c = flat <= 4096 ? 256 : 1024;
  int64_t n = std::max<int64_t>(1, (flat + c - 1) / c);
  while (n * std::max(active, 1) > (int64_t(1) << 21)) {
    c *= 2;
    n = std::max<int64_t>(1, (flat + c - 1) / c);
  }
  *nch = (int)n;
  *chunk = (int)c;
}

struct RouteWs {
  int* hist;
  int* base;
  int* totals;
  int* offsets;
};

RouteWs carve_route(Carver& cv, int64_t flat, int active, int* nch, int* chunk) {
  route_chunks(flat, active, nch, chunk);
  RouteWs w;
  w.hist = cv.take<int>((size_t)*nch * std::max(active, 1));
  w.base = cv.take<int>((size_t)*nch * std::max(active, 1));
  w.totals = cv.take<int>((size_t)std::max(active, 1));
  w.offsets = cv.take<int>((size_t)active + 1);
  return w;
}

// quantMode -> element format of the permute kernels: 0 E4M3FN, 1 E5M2, 2 E2M1 (MXFP4).
int quant_fmt(int quant_mode) {
  return quant_mode == MOE_QUANT_MXFP8_E4M3 ? 0 : quant_mode == MOE_QUANT_MXFP4_E2M1 ? 2 : 1;
}

bool valid_quant_mode(int q) {
  return q == MOE_QUANT_NONE || q == MOE_QUANT_MXFP8_E5M2 || q == MOE_QUANT_MXFP8_E4M3 || q == MOE_QUANT_MXFP4_E2M1;
}

bool valid_x_dtype(int d) { return d == MOE_DTYPE_FP32 || d == MOE_DTYPE_FP16 || d == MOE_DTYPE_BF16; }

int token_tile_tt(int64_t rows, int64_t groups, int64_t hidden, int64_t inter, int64_t aw) {
  return moe::gmm_token_tiles(rows, groups, hidden, inter, aw);
}

// Scale bytes of one weight group (N output channels, K inputs) in a weight format.
int64_t group_scale_bytes(int64_t n, int64_t k, int format) {
  if (format == MOE_WEIGHTS_PACKED) return (n / 16) * (((k / 128) + 3) / 4) * 256;
  return n * (k / 32);
}

// ---- moe_init_routing ------------------------------------------------------------
struct InitRoutingWs {
  RouteWs r;
  int32_t* scat;  // scatter index when the user asked for the gather type
  int nch, chunk;
};

InitRoutingWs carve_init_routing(Carver& cv, int64_t flat, int active, bool need_scat) {
  InitRoutingWs w;
  w.r = carve_route(cv, flat, active, &w.nch, &w.chunk);
  w.scat = need_scat ? cv.take<int32_t>((size_t)flat) : nullptr;
  return w;
}

// ---- mega_moe --------------------------------------------------------------------
struct MegaWs {
  RouteWs r;
  int nch, chunk;
  int32_t* scat;
  int32_t* gath;
  int32_t* row_token;
  float* row_weight;
  int4* tiles;
  int* tile_count;
  int max_tiles, tt;
  int4* sh_tiles;
  int* sh_count;
  int sh_max_tiles, sh_tt;
  // one shared expert folded into the routed experts' GEMM launches (LDS-streaming
  // kernels for both, same weight type): its chunks follow the routed ones in `tiles`
  // (all_count counts both) and its rows follow theirs in xq / sx / aq / sa (from padded
  // row routed_padded) and in the O rows (from row flat); the *_sh buffers point there
  bool fold;
  int* all_count;
  int64_t routed_padded;
  // LDS-streaming GEMMs: the chunk list split by chunk size (one phase per class)
  int4* cls_tiles;
  int* cls_count;
  // x quantized once in token order (row-major codes [tokens, hidden] and scales
  // [tokens, hidden/32]) when the gather re-reads many x rows; else null
  uint8_t* xrow;
  uint8_t* xrow_s;
  // token operands in the tiled layout: routed rows (padded per expert) and the
  // token-order rows of the shared experts
  uint8_t* xq;
  uint8_t* sx;
  uint8_t* aq;
  uint8_t* sa;
  uint8_t* xq_sh;
  uint8_t* sx_sh;
  uint8_t* aq_sh;
  uint8_t* sa_sh;
  // expert outputs: fp32 (combine_comm_mode 1) or bf16 (mode 0) [F, hidden] in sorted
  // rows unless the caller's o (fp32) is given, and [num_shared, tokens, hidden]
  float* o;
  uint16_t* o16;
  float* o_sh;
  uint16_t* o16_sh;
};

// Width of GMM1's activation output A (= GMM2's K): inter for the gated activations,
// 2 * inter for gelu ([MM] "Activation function formulas", gelu).
int64_t act_width(const moe_mega_args* a) { return a->activation == MOE_ACT_GELU ? 2 * a->inter : a->inter; }

// Stage 1 in two passes (MX-quantize every token once, then gather its codes into the
// tiled layout) when topk >= 3 rows per token and x is large: the gather then reads one
// byte per element of each destination row instead of the two of bf16 x, and the shared
// experts' token-order operand is the same codes. Small layers keep the one-pass gather
// (one launch fewer). Q_MX is row-local, so both give the same bytes.
bool quantize_first(const moe_mega_args* a) {
  return !a->x_is_quantized && a->topk >= 3 && a->num_tokens * a->hidden >= (int64_t)1 << 22;
}

MegaWs carve_mega(Carver& cv, const moe_mega_args* a) {
  MegaWs w{};
  const int64_t n = a->num_tokens, h = a->hidden, i = act_width(a), e = a->num_experts;
  const int64_t flat = n * a->topk;
  w.r = carve_route(cv, flat, (int)e, &w.nch, &w.chunk);
  w.scat = cv.take<int32_t>(flat);
  w.gath = a->sorted_row_idx ? nullptr : cv.take<int32_t>(flat);
  w.row_token = cv.take<int32_t>(flat);
  w.row_weight = cv.take<float>(flat);
  w.tt = token_tile_tt(flat, e, h, a->inter, i);
  w.max_tiles = (int)(flat / (16 * w.tt) + e + 1);
  const int64_t S = a->num_shared;
  if (S > 0) {
    w.sh_tt = token_tile_tt(n, 1, h, a->inter, i);
    w.sh_max_tiles = (int)((n + 16 * w.sh_tt - 1) / (16 * w.sh_tt));
    const int sw = a->shared_weight_dtype ? a->shared_weight_dtype : a->weight_dtype;
    // (not with the caller's o: it has room for the routed rows only)
    w.fold = S == 1 && !a->o && w.tt == moe::kStreamTiles && w.sh_tt == moe::kStreamTiles &&
             (sw == MOE_FP4_E2M1) == (a->weight_dtype == MOE_FP4_E2M1);
  }
  const int all_max = w.max_tiles + (w.fold ? w.sh_max_tiles : 0);
  w.tiles = cv.take<int4>(all_max);
  w.tile_count = cv.take<int>(1);
  w.all_count = w.fold ? cv.take<int>(1) : nullptr;
  if (w.tt == moe::kStreamTiles) {
    w.cls_tiles = cv.take<int4>((size_t)moe::kStreamClasses * all_max);
    w.cls_count = cv.take<int>(moe::kStreamClasses);
  }
  if (quantize_first(a)) {
    w.xrow = cv.take<uint8_t>((size_t)(n * h));
    w.xrow_s = cv.take<uint8_t>((size_t)(n * (h / 32)));
  }
  const int64_t padded = moe::t16_padded_rows(flat, e);
  const int64_t padded_sh = S > 0 ? moe::t16_padded_rows(n, 1) : 0;
  const int64_t all_padded = padded + (w.fold ? padded_sh : 0);
  w.routed_padded = padded;
  w.xq = cv.take<uint8_t>((size_t)moe::t16_code_bytes(all_padded, h));
  w.sx = cv.take<uint8_t>((size_t)moe::t16_scale_bytes(all_padded, h));
  w.aq = cv.take<uint8_t>((size_t)moe::t16_code_bytes(all_padded, i));
  w.sa = cv.take<uint8_t>((size_t)moe::t16_scale_bytes(all_padded, i));
  if (S > 0) {
    w.sh_tiles = cv.take<int4>(w.sh_max_tiles);
    w.sh_count = cv.take<int>(1);
    if (w.fold) {
      w.xq_sh = w.xq + moe::t16_code_bytes(padded, h);
      w.sx_sh = w.sx + moe::t16_scale_bytes(padded, h);
      w.aq_sh = w.aq + moe::t16_code_bytes(padded, i);
      w.sa_sh = w.sa + moe::t16_scale_bytes(padded, i);
    } else {
      w.xq_sh = cv.take<uint8_t>((size_t)moe::t16_code_bytes(padded_sh, h));
      w.sx_sh = cv.take<uint8_t>((size_t)moe::t16_scale_bytes(padded_sh, h));
      w.aq_sh = cv.take<uint8_t>((size_t)moe::t16_code_bytes(padded_sh, i));
      w.sa_sh = cv.take<uint8_t>((size_t)moe::t16_scale_bytes(padded_sh, i));
    }
  }
  const bool rows16 = a->combine_comm_mode == 0;
  const size_t nsh = (size_t)S * n * h;
  // folded: the shared expert's O rows follow the routed rows
  const size_t orows = (size_t)flat * h + (w.fold ? nsh : 0);
  w.o = (a->o || rows16) ? nullptr : cv.take<float>(orows);
  w.o16 = (a->o || !rows16) ? nullptr : cv.take<uint16_t>(orows);
  if (w.fold) {
    w.o_sh = w.o ? w.o + (size_t)flat * h : nullptr;
    w.o16_sh = w.o16 ? w.o16 + (size_t)flat * h : nullptr;
  } else {
    w.o_sh = S > 0 && !rows16 ? cv.take<float>(nsh) : nullptr;
    w.o16_sh = S > 0 && rows16 ? cv.take<uint16_t>(nsh) : nullptr;
  }
  return w;
}

// activation + activation_params -> kernel parameters, with the pages' defaults
// ([MM] parameter description of activation_params): clamp none (0 = none), alpha
// 1.702, swigluoai beta 1.0, situglu beta 1.0 and no linear_beta.
moe_status act_params(const moe_mega_args* a, moe::ActParams* out) {
  const int np = a->num_activation_params;
  const float* v = a->activation_params;
  moe::ActParams p;
  p.kind = a->activation;
  auto bad = [&](const char* what) {
    return fail(MOE_ERR_INVALID_ARG, "mega_moe: activation %d: %s", a->activation, what);
  };
  auto clamp_of = [&](float c, moe::ActParams* q) -> bool {
    if (std::isnan(c) || c < 0.0f) return false;
    if (c > 0.0f) q->clamp = c;
    return true;
  };
  switch (a->activation) {
    case MOE_ACT_SWIGLU:
    case MOE_ACT_SWIGLUSTEP:
      if (np != 0 && np != 1) return bad("takes [] or [clamp]");
      if (np == 1 && !clamp_of(v[0], &p)) return bad("clamp must be >= 0 and not NaN");
      break;
    case MOE_ACT_SWIGLUOAI:
      if (np != 0 && np != 3) return bad("takes [] or [clamp, alpha, beta]");
      if (np == 3) {
        if (!clamp_of(v[0], &p)) return bad("clamp must be >= 0 and not NaN");
        if (!std::isfinite(v[1]) || !std::isfinite(v[2])) return bad("alpha and beta must be finite");
        p.alpha = v[1];
        p.beta = v[2];
      }
      break;
    case MOE_ACT_SITUGLU:
      if (np < 0 || np > 2) return bad("takes [], [beta] or [beta, linear_beta]");
      for (int j = 0; j < np; ++j)
        if (!std::isfinite(v[j]) || !(v[j] > 0.0f)) return bad("beta and linear_beta must be finite and > 0");
      if (np >= 1) p.beta = v[0];
      if (np == 2) p.lin_beta = v[1];
      break;
    case MOE_ACT_GELU:
      if (np != 0 && !(np == 1 && v[0] == FLT_MAX)) return bad("takes no clamp ([] or the placeholder [FLT_MAX])");
      break;
    default:
      return fail(MOE_ERR_INVALID_ARG, "mega_moe: activation %d not one of MOE_ACT_*", a->activation);
  }
  if (out) *out = p;
  return MOE_OK;
}

moe_status check_mega(const moe_mega_args* a) {
  if (!a) return fail(MOE_ERR_INVALID_ARG, "mega_moe: args is NULL");
  if (a->num_tokens < 0) return fail(MOE_ERR_SHAPE, "mega_moe: num_tokens %lld < 0", (long long)a->num_tokens);
  if (a->hidden < 128 || a->hidden % 128 != 0 || a->hidden > 65536)
    return fail(MOE_ERR_SHAPE, "mega_moe: hidden %lld must be a positive multiple of 128 (<= 65536)",
                (long long)a->hidden);
  if (a->inter < 128 || a->inter % 128 != 0 || a->inter > 65536)
    return fail(MOE_ERR_SHAPE, "mega_moe: inter %lld must be a positive multiple of 128 (<= 65536)",
                (long long)a->inter);
  if (a->topk < 1 || a->topk > 32) return fail(MOE_ERR_SHAPE, "mega_moe: topk %lld outside [1, 32]", (long long)a->topk);
  if (a->num_experts < 1 || a->num_experts > 1024)
    return fail(MOE_ERR_SHAPE, "mega_moe: num_experts %lld outside [1, 1024]", (long long)a->num_experts);
  if (a->topk > a->num_experts)
    return fail(MOE_ERR_SHAPE, "mega_moe: topk %lld > num_experts %lld (ids per token must be distinct)",
                (long long)a->topk, (long long)a->num_experts);
  if (a->num_tokens * a->topk >= MOE_MAX_FLAT_ROWS)
    return fail(MOE_ERR_SHAPE, "mega_moe: num_tokens*topk must be < %d", MOE_MAX_FLAT_ROWS);
  if (a->num_shared < 0 || a->num_shared > 4)
    return fail(MOE_ERR_SHAPE, "mega_moe: num_shared %lld outside [0, 4]", (long long)a->num_shared);
  if (a->quant_out_dtype != MOE_FP8_E5M2 && a->quant_out_dtype != MOE_FP8_E4M3)
    return fail(MOE_ERR_DTYPE, "mega_moe: quant_out_dtype %d must be 23 (FLOAT8_E5M2) or 24 (FLOAT8_E4M3FN)",
                a->quant_out_dtype);
  if (moe_status st = act_params(a, nullptr)) return st;
  for (int wd : {a->weight_dtype, a->shared_weight_dtype}) {
    if (wd != 0 && wd != MOE_FP8_E5M2 && wd != MOE_FP8_E4M3 && wd != MOE_FP4_E2M1)
      return fail(MOE_ERR_DTYPE, "mega_moe: weight dtype %d not 0, 23, 24 or 296", wd);
    if ((wd == MOE_FP8_E5M2 || wd == MOE_FP8_E4M3) && wd != a->quant_out_dtype)
      return fail(MOE_ERR_UNSUPPORTED, "mega_moe: FP8 weights must have the activations' FP8 type %d",
                  a->quant_out_dtype);
    if (wd == MOE_FP4_E2M1 && a->quant_out_dtype != MOE_FP8_E4M3)
      return fail(MOE_ERR_UNSUPPORTED, "mega_moe: MXFP4 weights (A8W4-FP) take FLOAT8_E4M3FN activations");
  }
  if (a->topk_weights_dtype != MOE_DTYPE_FP32 && a->topk_weights_dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_DTYPE, "mega_moe: topk_weights_dtype must be FP32 or BF16");
  if (a->weight_format != MOE_WEIGHTS_ND && a->weight_format != MOE_WEIGHTS_PACKED)
    return fail(MOE_ERR_INVALID_ARG, "mega_moe: weight_format %d not 0 (ND) or 1 (packed)", a->weight_format);
  if (a->num_tokens > 0 && (!a->x || !a->topk_ids || !a->topk_weights || !a->y))
    return fail(MOE_ERR_INVALID_ARG, "mega_moe: x, topk_ids, topk_weights and y must be non-NULL");
  if (a->x_is_quantized != 0 && a->x_is_quantized != 1)
    return fail(MOE_ERR_INVALID_ARG, "mega_moe: x_is_quantized must be 0 or 1");
  if (a->combine_comm_mode != 0 && a->combine_comm_mode != 1)
    return fail(MOE_ERR_UNSUPPORTED, "mega_moe: combine_comm_mode %d not 0 or 1 (one card)", a->combine_comm_mode);
  if (a->x_is_quantized && a->num_tokens > 0 && !a->x_scales)
    return fail(MOE_ERR_INVALID_ARG, "mega_moe: pre-quantized x needs x_scales");
  if (!a->x_is_quantized && a->x_scales)
    return fail(MOE_ERR_INVALID_ARG, "mega_moe: x_scales is only taken with pre-quantized x");
  if (!a->w1 || !a->w1_scales || !a->w2 || !a->w2_scales)
    return fail(MOE_ERR_INVALID_ARG, "mega_moe: w1, w1_scales, w2, w2_scales must be non-NULL");
  if (a->num_shared > 0 && (!a->shared_w1 || !a->shared_w1_scales || !a->shared_w2 || !a->shared_w2_scales))
    return fail(MOE_ERR_INVALID_ARG, "mega_moe: num_shared > 0 needs all four shared weight pointers");
  return MOE_OK;
}

moe_status check_gmm_common(const char* who, int64_t rows, int64_t hidden, int64_t inter, int64_t groups,
                            int quant_out_dtype) {
  if (rows < 0) return fail(MOE_ERR_SHAPE, "%s: rows < 0", who);
  if (hidden < 128 || hidden % 128 != 0 || hidden > 65536)
    return fail(MOE_ERR_SHAPE, "%s: hidden %lld must be a positive multiple of 128", who, (long long)hidden);
  if (inter < 128 || inter % 128 != 0 || inter > 65536)
    return fail(MOE_ERR_SHAPE, "%s: inter %lld must be a positive multiple of 128", who, (long long)inter);
  if (groups < 1 || groups > MOE_MAX_EXPERTS) return fail(MOE_ERR_SHAPE, "%s: num_groups outside [1, %d]", who, MOE_MAX_EXPERTS);
  if (rows >= MOE_MAX_FLAT_ROWS) return fail(MOE_ERR_SHAPE, "%s: rows must be < %d", who, MOE_MAX_FLAT_ROWS);
  if (quant_out_dtype != MOE_FP8_E5M2 && quant_out_dtype != MOE_FP8_E4M3)
    return fail(MOE_ERR_DTYPE, "%s: quant_out_dtype must be 23 or 24", who);
  return MOE_OK;
}

// The stage entry points take row-major token operands (the pages' layout) and stage
// them through the tiled layout of the kernels: in_* holds the packed input (K up to
// max(hidden, inter)), out_* GMM1's requantized output before it is unpacked.
struct GmmWs {
  int4* tiles;
  int* count;
  int max_tiles, tt;
  uint8_t* in_codes;
  uint8_t* in_scales;
  uint8_t* out_codes;
  uint8_t* out_scales;
  float* o;   // fp32 [rows, hidden] GMM2 output when the caller passes no o
};

GmmWs carve_gmm(Carver& cv, int64_t rows, int64_t groups, int64_t hidden, int64_t inter) {
  GmmWs w;
  w.tt = token_tile_tt(rows, groups, hidden, inter, inter);
  w.max_tiles = (int)(rows / (16 * w.tt) + groups + 1);
  w.tiles = cv.take<int4>(w.max_tiles);
  w.count = cv.take<int>(1);
  const int64_t padded = moe::t16_padded_rows(rows, groups), kin = std::max(hidden, inter);
  w.in_codes = cv.take<uint8_t>((size_t)moe::t16_code_bytes(padded, kin));
  w.in_scales = cv.take<uint8_t>((size_t)moe::t16_scale_bytes(padded, kin));
  w.out_codes = cv.take<uint8_t>((size_t)moe::t16_code_bytes(padded, inter));
  w.out_scales = cv.take<uint8_t>((size_t)moe::t16_scale_bytes(padded, inter));
  w.o = cv.take<float>((size_t)rows * hidden);
  return w;
}

moe_status check_ws(const char* who, size_t need, void* ws, size_t have) {
  if (have < need || (need > 0 && ws == nullptr))
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes required, %zu given", who, need, ws ? have : 0);
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", who);
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_error.c_str(); }

int moe_version(void) { return 100; }

int64_t moe_mx_scale_cols(int64_t cols) { return cols <= 0 ? 0 : scale_cols(cols); }

int64_t moe_token_permute_out_rows(int64_t flat_rows, int64_t num_out_tokens) {
  if (num_out_tokens == 0) return flat_rows;
  if (num_out_tokens > 0) return std::min(num_out_tokens, flat_rows);
  return std::max<int64_t>(flat_rows + num_out_tokens, 0);
}

moe_status moe_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int quant_mode, uint8_t* codes,
                           uint8_t* scales, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 8 != 0)
    return fail(MOE_ERR_SHAPE, "moe_mx_quantize: rows %lld >= 0 and cols %lld > 0 with cols %% 8 == 0 required",
                (long long)rows, (long long)cols);
  if (!valid_x_dtype(dtype)) return fail(MOE_ERR_DTYPE, "moe_mx_quantize: dtype %d not BF16/FP16/FP32", dtype);
  if (quant_mode != MOE_QUANT_MXFP8_E4M3 && quant_mode != MOE_QUANT_MXFP8_E5M2 && quant_mode != MOE_QUANT_MXFP4_E2M1)
    return fail(MOE_ERR_UNSUPPORTED, "moe_mx_quantize: quant_mode %d not 2, 3 or 9", quant_mode);
  if (rows == 0) return ok();
  if (!x || !codes || !scales) return fail(MOE_ERR_INVALID_ARG, "moe_mx_quantize: NULL buffer");
  moe::PermuteParams p;
  p.x = x; p.in_dtype = dtype; p.n = rows; p.hidden = cols; p.topk = 1; p.scat = nullptr; p.m_limit = rows;
  p.quant = quant_fmt(quant_mode); p.out = codes; p.out_scales = scales; p.scale_cols = scale_cols(cols);
  hipError_t e = moe::launch_permute(p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_mx_quantize launch");
  return ok();
}

int64_t moe_mx_packed_scale_bytes(int64_t groups, int64_t n, int64_t k) {
  if (groups < 0 || n <= 0 || k <= 0) return 0;
  return groups * group_scale_bytes(n, k, MOE_WEIGHTS_PACKED);
}

moe_status moe_mx_pack_weights(const uint8_t* codes, const uint8_t* scales, int64_t groups, int64_t n, int64_t k,
                               uint8_t* packed_codes, uint8_t* packed_scales, void* stream) {
  if (groups < 0 || n <= 0 || k <= 0 || n % 16 != 0 || k % 128 != 0)
    return fail(MOE_ERR_SHAPE, "moe_mx_pack_weights: groups >= 0, n %% 16 == 0 and k %% 128 == 0 required");
  if (groups == 0) return ok();
  if (!codes || !scales || !packed_codes || !packed_scales)
    return fail(MOE_ERR_INVALID_ARG, "moe_mx_pack_weights: NULL buffer");
  hipError_t e = moe::launch_pack_weights(codes, scales, groups, n, k, packed_codes, packed_scales, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_mx_pack_weights launch");
  return ok();
}

moe_status moe_mx_pack_weights_fp4(const uint8_t* codes, const uint8_t* scales, int64_t groups, int64_t n, int64_t k,
                                   uint8_t* packed_codes, uint8_t* packed_scales, void* stream) {
  if (groups < 0 || n <= 0 || k <= 0 || n % 16 != 0 || k % 128 != 0)
    return fail(MOE_ERR_SHAPE, "moe_mx_pack_weights_fp4: groups >= 0, n %% 16 == 0 and k %% 128 == 0 required");
  if (groups == 0) return ok();
  if (!codes || !scales || !packed_codes || !packed_scales)
    return fail(MOE_ERR_INVALID_ARG, "moe_mx_pack_weights_fp4: NULL buffer");
  hipError_t e =
      moe::launch_pack_weights_fp4(codes, scales, groups, n, k, packed_codes, packed_scales, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_mx_pack_weights_fp4 launch");
  return ok();
}

moe_status moe_init_routing_workspace_size(int64_t num_rows, int64_t k, int64_t expert_num, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "moe_init_routing_workspace_size: bytes is NULL");
  if (num_rows < 0 || k < 1 || expert_num < 1 || expert_num > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_SHAPE, "moe_init_routing_workspace_size: bad sizes");
  Carver cv(nullptr);
  carve_init_routing(cv, num_rows * k, (int)expert_num, true);
  *bytes = cv.off;
  return ok();
}

}  // extern "C"

namespace {

// moe_init_routing and moe_init_routing_noalloc: with noalloc the scratch is the
// library's static per-device array (its size checked here) instead of `workspace`.
moe_status init_routing_impl(const char* who, bool noalloc, const void* x, int x_dtype, const uint8_t* scale,
                             int64_t num_rows, int64_t hidden, const int32_t* expert_idx, int64_t k,
                             int64_t expert_num, int64_t active_start, int64_t active_end, int quant_mode,
                             int row_idx_type, int expert_tokens_num_type, void* expanded_x,
                             int32_t* expanded_row_idx, int64_t* expert_tokens, uint8_t* expanded_scale,
                             int64_t* available_idx_num, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_rows < 0 || hidden < 1) return fail(MOE_ERR_SHAPE, "%s: num_rows >= 0 and hidden >= 1 required", who);
  if (k < 1 || k > 64) return fail(MOE_ERR_SHAPE, "%s: k %lld outside [1, 64]", who, (long long)k);
  if (expert_num < 1 || expert_num > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_SHAPE, "%s: expert_num %lld outside [1, %d]", who, (long long)expert_num, MOE_MAX_EXPERTS);
  if (active_start < 0 || active_start > active_end || active_end > expert_num)
    return fail(MOE_ERR_SHAPE, "%s: active range [%lld, %lld) must satisfy 0 <= start <= end <= expert_num %lld", who,
                (long long)active_start, (long long)active_end, (long long)expert_num);
  const int64_t flat = num_rows * k;
  if (flat >= MOE_MAX_FLAT_ROWS) return fail(MOE_ERR_SHAPE, "%s: num_rows*k must be < %d", who, MOE_MAX_FLAT_ROWS);
  // x of MX codes ([V3] quantMode -1 with an FP8 / FP4 x): rows gathered as they are
  const bool codes = x_dtype == MOE_DTYPE_FP8_E5M2 || x_dtype == MOE_DTYPE_FP8_E4M3 || x_dtype == MOE_DTYPE_FP4_E2M1;
  if (!valid_x_dtype(x_dtype) && !codes)
    return fail(MOE_ERR_DTYPE, "%s: x_dtype %d not FP32/FP16/BF16 or FP8/FP4 codes", who, x_dtype);
  if (!valid_quant_mode(quant_mode))
    return fail(MOE_ERR_UNSUPPORTED, "%s: quant_mode %d not supported (-1, 2, 3, 9)", who, quant_mode);
  const bool mx = quant_mode != MOE_QUANT_NONE;
  if (codes && mx) return fail(MOE_ERR_UNSUPPORTED, "%s: x of FP8/FP4 codes takes quant_mode -1 (pass-through)", who);
  if (x_dtype == MOE_DTYPE_FP4_E2M1 && hidden % 2 != 0)
    return fail(MOE_ERR_SHAPE, "%s: FP4 codes need an even hidden", who);
  if (scale && !codes) return fail(MOE_ERR_INVALID_ARG, "%s: a scale input goes only with x of FP8/FP4 codes", who);
  if (scale && hidden % 32 != 0) return fail(MOE_ERR_SHAPE, "%s: scales need hidden %% 32 == 0", who);
  if (mx && hidden % 32 != 0) return fail(MOE_ERR_SHAPE, "%s: MX quantization needs hidden %% 32 == 0", who);
  if (row_idx_type != MOE_ROW_IDX_GATHER && row_idx_type != MOE_ROW_IDX_SCATTER)
    return fail(MOE_ERR_INVALID_ARG, "%s: row_idx_type %d not 0 or 1", who, row_idx_type);
  if (expert_tokens_num_type != MOE_TOKENS_CUMSUM && expert_tokens_num_type != MOE_TOKENS_COUNT &&
      expert_tokens_num_type != MOE_TOKENS_KEY_VALUE)
    return fail(MOE_ERR_INVALID_ARG, "%s: expert_tokens_num_type %d not 0, 1 or 2", who, expert_tokens_num_type);
  if (expert_tokens_num_type == MOE_TOKENS_KEY_VALUE && expert_num > 5120)
    return fail(MOE_ERR_SHAPE, "%s: key_value counts take expert_num <= 5120 (got %lld)", who, (long long)expert_num);
  if (flat > 0 && (!x || !expert_idx || !expanded_x || !expanded_row_idx))
    return fail(MOE_ERR_INVALID_ARG, "%s: x, expert_idx, expanded_x, expanded_row_idx must be non-NULL", who);
  if (!available_idx_num) return fail(MOE_ERR_INVALID_ARG, "%s: available_idx_num must be non-NULL", who);
  const bool key_value = expert_tokens_num_type == MOE_TOKENS_KEY_VALUE;
  if ((active_end > active_start || key_value) && !expert_tokens)
    return fail(MOE_ERR_INVALID_ARG, "%s: expert_tokens must be non-NULL", who);
  if ((mx || scale) && flat > 0 && !expanded_scale)
    return fail(MOE_ERR_INVALID_ARG, "%s: expanded_scale must be non-NULL in MX modes and with a scale input", who);
  const int active = (int)(active_end - active_start);
  const bool want_gather = row_idx_type == MOE_ROW_IDX_GATHER;
  Carver cv(nullptr);
  carve_init_routing(cv, flat, active, want_gather);
  if (noalloc) {
    if (cv.off > moe::kNoAllocScratchBytes)
      return fail(MOE_ERR_SHAPE, "%s: needs %zu bytes of scratch, more than the %zu bytes of its static scratch",
                  who, cv.off, moe::kNoAllocScratchBytes);
    hipError_t e = moe::noalloc_scratch(&workspace);
    if (e != hipSuccess) return hip_fail(e, "moe_init_routing_noalloc scratch lookup");
    workspace_bytes = moe::kNoAllocScratchBytes;
  } else if (moe_status st = check_ws(who, cv.off, workspace, workspace_bytes)) {
    return st;
  }
  Carver w(workspace);
  InitRoutingWs ws = carve_init_routing(w, flat, active, want_gather);
  hipStream_t st = (hipStream_t)stream;

  moe::RouteParams rp;
  rp.keys = expert_idx; rp.key_is64 = 0; rp.flat = flat; rp.topk = (int)k;
  rp.s = (int)active_start; rp.e = (int)active_end; rp.nch = ws.nch; rp.chunk = ws.chunk;
  rp.hist = ws.r.hist; rp.base = ws.r.base; rp.totals = ws.r.totals; rp.offsets = ws.r.offsets;
  rp.avail64 = available_idx_num; rp.expert_tokens = key_value ? nullptr : expert_tokens;
  rp.tokens_type = expert_tokens_num_type;
  if (want_gather) {
    rp.scat = ws.scat; rp.gath = expanded_row_idx; rp.gath_fill = expanded_row_idx;
  } else {
    rp.scat = expanded_row_idx;
  }
  hipError_t e = moe::launch_routing(rp, st);
  if (e != hipSuccess) return hip_fail(e, "moe_init_routing routing launch");
  if (key_value) {
    e = moe::launch_key_value(ws.r.offsets, active, (int)active_start, (int)expert_num, expert_tokens, st);
    if (e != hipSuccess) return hip_fail(e, "moe_init_routing key_value launch");
  }
  if (codes) {
    const int64_t row_bytes = x_dtype == MOE_DTYPE_FP4_E2M1 ? hidden / 2 : hidden;
    e = moe::launch_permute_rows(static_cast<const uint8_t*>(x), num_rows, row_bytes, (int)k, rp.scat, flat,
                                 static_cast<uint8_t*>(expanded_x), st);
    if (e == hipSuccess && scale)
      e = moe::launch_permute_rows(scale, num_rows, scale_cols(hidden), (int)k, rp.scat, flat, expanded_scale, st);
    if (e != hipSuccess) return hip_fail(e, "moe_init_routing gather launch");
    return ok();
  }
  moe::PermuteParams pp;
  pp.x = x; pp.in_dtype = x_dtype; pp.n = num_rows; pp.hidden = hidden; pp.topk = (int)k; pp.scat = rp.scat;
  pp.m_limit = flat; pp.quant = mx ? quant_fmt(quant_mode) : -1; pp.out = expanded_x;
  pp.out_scales = expanded_scale; pp.scale_cols = scale_cols(hidden);
  e = moe::launch_permute(pp, st);
  if (e != hipSuccess) return hip_fail(e, "moe_init_routing permute launch");
  return ok();
}

}  // namespace

extern "C" {

moe_status moe_init_routing(const void* x, int x_dtype, const uint8_t* scale, int64_t num_rows, int64_t hidden,
                            const int32_t* expert_idx, int64_t k, int64_t expert_num, int64_t active_start,
                            int64_t active_end, int quant_mode, int row_idx_type, int expert_tokens_num_type,
                            void* expanded_x, int32_t* expanded_row_idx, int64_t* expert_tokens,
                            uint8_t* expanded_scale, int64_t* available_idx_num, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return init_routing_impl("moe_init_routing", false, x, x_dtype, scale, num_rows, hidden, expert_idx, k, expert_num,
                           active_start, active_end, quant_mode, row_idx_type, expert_tokens_num_type, expanded_x,
                           expanded_row_idx, expert_tokens, expanded_scale, available_idx_num, workspace,
                           workspace_bytes, stream);
}

moe_status moe_init_routing_noalloc(const void* x, int x_dtype, const uint8_t* scale, int64_t num_rows,
                                    int64_t hidden, const int32_t* expert_idx, int64_t k, int64_t expert_num,
                                    int64_t active_start, int64_t active_end, int quant_mode, int row_idx_type,
                                    int expert_tokens_num_type, void* expanded_x, int32_t* expanded_row_idx,
                                    int64_t* expert_tokens, uint8_t* expanded_scale, int64_t* available_idx_num,
                                    void* stream) {
  return init_routing_impl("moe_init_routing_noalloc", true, x, x_dtype, scale, num_rows, hidden, expert_idx, k,
                           expert_num, active_start, active_end, quant_mode, row_idx_type, expert_tokens_num_type,
                           expanded_x, expanded_row_idx, expert_tokens, expanded_scale, available_idx_num, nullptr, 0,
                           stream);
}

moe_status moe_token_permute_workspace_size(int64_t flat_rows, int64_t num_experts, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "moe_token_permute_workspace_size: bytes is NULL");
  if (flat_rows < 0 || num_experts < 1 || num_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_SHAPE, "moe_token_permute_workspace_size: bad sizes");
  Carver cv(nullptr);
  int nch, chunk;
  carve_route(cv, flat_rows, (int)num_experts, &nch, &chunk);
  *bytes = cv.off;
  return ok();
}

moe_status moe_token_permute(const void* tokens, int dtype, int64_t n, int64_t hidden, const void* indices,
                             int indices_dtype, int64_t topk, int64_t num_experts, int64_t num_out_tokens,
                             int padded_mode, int quant_mode, void* permuted_tokens, int32_t* sorted_indices,
                             uint8_t* expanded_scale, void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "moe_token_permute";
  if (padded_mode != 0) return fail(MOE_ERR_UNSUPPORTED, "%s: padded_mode must be False", who);
  if (n < 0 || hidden < 1) return fail(MOE_ERR_SHAPE, "%s: n >= 0 and hidden >= 1 required", who);
  if (topk < 1 || topk > 64) return fail(MOE_ERR_SHAPE, "%s: topk %lld outside [1, 64]", who, (long long)topk);
  if (num_experts < 1 || num_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_SHAPE, "%s: num_experts %lld outside [1, %d]", who, (long long)num_experts, MOE_MAX_EXPERTS);
  const int64_t flat = n * topk;
  if (flat >= MOE_MAX_FLAT_ROWS) return fail(MOE_ERR_SHAPE, "%s: indices numel must be < %d", who, MOE_MAX_FLAT_ROWS);
  if (indices_dtype != MOE_DTYPE_INT32 && indices_dtype != MOE_DTYPE_INT64)
    return fail(MOE_ERR_DTYPE, "%s: indices dtype must be INT32 or INT64", who);
  if (!valid_x_dtype(dtype)) return fail(MOE_ERR_DTYPE, "%s: tokens dtype %d not FP32/FP16/BF16", who, dtype);
  if (!valid_quant_mode(quant_mode))
    return fail(MOE_ERR_UNSUPPORTED, "%s: quant_mode %d not supported (-1, 2, 3, 9)", who, quant_mode);
  const bool mx = quant_mode != MOE_QUANT_NONE;
  if (mx && dtype == MOE_DTYPE_FP32) return fail(MOE_ERR_DTYPE, "%s: MX quant modes take FP16/BF16 tokens", who);
  if (mx && hidden % 32 != 0) return fail(MOE_ERR_SHAPE, "%s: MX quantization needs hidden %% 32 == 0", who);
  const int64_t m = moe_token_permute_out_rows(flat, num_out_tokens);
  if (flat > 0 && (!tokens || !indices || !sorted_indices))
    return fail(MOE_ERR_INVALID_ARG, "%s: tokens, indices, sorted_indices must be non-NULL", who);
  if (m > 0 && (!permuted_tokens || (mx && !expanded_scale)))
    return fail(MOE_ERR_INVALID_ARG, "%s: permuted_tokens (and expanded_scale in MX modes) must be non-NULL", who);
  Carver cv(nullptr);
  int nch, chunk;
  carve_route(cv, flat, (int)num_experts, &nch, &chunk);
  if (moe_status st = check_ws(who, cv.off, workspace, workspace_bytes)) return st;
  Carver w(workspace);
  RouteWs rw = carve_route(w, flat, (int)num_experts, &nch, &chunk);
  hipStream_t st = (hipStream_t)stream;
  moe::RouteParams rp;
  rp.keys = indices; rp.key_is64 = indices_dtype == MOE_DTYPE_INT64; rp.flat = flat; rp.topk = (int)topk;
  rp.s = 0; rp.e = (int)num_experts; rp.nch = nch; rp.chunk = chunk;
  rp.hist = rw.hist; rp.base = rw.base; rp.totals = rw.totals; rp.offsets = rw.offsets; rp.scat = sorted_indices;
  hipError_t e = moe::launch_routing(rp, st);
  if (e != hipSuccess) return hip_fail(e, "moe_token_permute routing launch");
  moe::PermuteParams pp;
  pp.x = tokens; pp.in_dtype = dtype; pp.n = n; pp.hidden = hidden; pp.topk = (int)topk; pp.scat = sorted_indices;
  pp.m_limit = m; pp.quant = mx ? quant_fmt(quant_mode) : -1; pp.out = permuted_tokens;
  pp.out_scales = expanded_scale; pp.scale_cols = scale_cols(hidden);
  e = moe::launch_permute(pp, st);
  if (e != hipSuccess) return hip_fail(e, "moe_token_permute permute launch");
  return ok();
}

moe_status mega_moe_workspace_size(const moe_mega_args* args, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "mega_moe_workspace_size: bytes is NULL");
  if (moe_status s = check_mega(args)) return s;
  Carver cv(nullptr);
  carve_mega(cv, args);
  *bytes = cv.off;
  return ok();
}

moe_status mega_moe(const moe_mega_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  if (moe_status s = check_mega(a)) return s;
  Carver cv(nullptr);
  carve_mega(cv, a);
  if (moe_status s = check_ws("mega_moe", cv.off, workspace, workspace_bytes)) return s;
  Carver wc(workspace);
  MegaWs w = carve_mega(wc, a);
  hipStream_t st = (hipStream_t)stream;
  auto mark = [&](int k) -> hipError_t {
    return a->stage_events && a->stage_events[k] ? hipEventRecord((hipEvent_t)a->stage_events[k], st) : hipSuccess;
  };
  const int64_t n = a->num_tokens, h = a->hidden, inter = a->inter, ne = a->num_experts;
  const int64_t aw = act_width(a);   // width of A = K of GMM2
  const int64_t flat = n * a->topk;
  const int fmt = a->quant_out_dtype == MOE_FP8_E4M3 ? 0 : 1;
  moe::ActParams act;
  act_params(a, &act);
  int32_t* gath = a->sorted_row_idx ? a->sorted_row_idx : w.gath;

  // stage 1a: routing (full expert range, scatter + gather forms, combine row maps)
  moe::RouteParams rp;
  rp.keys = a->topk_ids; rp.flat = flat; rp.topk = (int)a->topk; rp.s = 0; rp.e = (int)ne;
  rp.nch = w.nch; rp.chunk = w.chunk; rp.hist = w.r.hist; rp.base = w.r.base; rp.totals = w.r.totals; rp.offsets = w.r.offsets;
  rp.token_nums32 = a->expert_token_nums; rp.scat = w.scat; rp.gath = gath;
  rp.row_token = w.row_token; rp.row_weight = w.row_weight; rp.topk_w = a->topk_weights;
  rp.topk_w_bf16 = a->topk_weights_dtype == MOE_DTYPE_BF16;
  hipError_t e = mark(0);
  if (e != hipSuccess) return hip_fail(e, "mega_moe event record");
  e = moe::launch_routing(rp, st);
  if (e != hipSuccess) return hip_fail(e, "mega_moe routing launch");
  if (n == 0) return ok();
  // the chunk lists: routed experts, the folded shared expert after them, the shared
  // expert's own list (its token-order rows), and the chunk classes
  moe::ChunkListParams cl;
  cl.offsets = w.r.offsets; cl.groups = (int)ne; cl.rows = (int)flat; cl.tm = 16 * w.tt; cl.max_tiles = w.max_tiles;
  cl.tiles = w.tiles; cl.count = w.tile_count;
  if (a->num_shared > 0) {
    cl.sh_rows = (int)n; cl.sh_tm = 16 * w.sh_tt;
    cl.sh_tiles = w.sh_tiles; cl.sh_count = w.sh_count;
    if (w.fold) {
      cl.sh_group = (int)ne; cl.sh_prow0 = (int)w.routed_padded; cl.sh_srow0 = (int)flat;
      cl.count_all = w.all_count;
    }
  }
  moe::StreamClasses classes;
  if (w.cls_tiles) {
    const int all_max = w.max_tiles + (w.fold ? w.sh_max_tiles : 0);
    cl.cls_tiles = w.cls_tiles; cl.cls_count = w.cls_count; cl.cls_stride = all_max;
    classes.tiles = w.cls_tiles; classes.count = w.cls_count; classes.stride = all_max;
  }
  e = moe::launch_chunk_lists(cl, st);
  if (e != hipSuccess) return hip_fail(e, "mega_moe chunk list launch");
  if ((e = mark(1)) != hipSuccess) return hip_fail(e, "mega_moe event record");
  // stage 1b: gather + MX quantization into the tiled layout (and the token-order rows
  // of the shared experts)
  // (pre-quantized x: the codes and scales are gathered as they are, [MM] dispatchQuantMode 0)
  const uint8_t* xcodes = static_cast<const uint8_t*>(a->x);
  const uint8_t* xscales = a->x_scales;
  bool codes_in = a->x_is_quantized != 0;
  if (w.xrow) {
    moe::PermuteParams q;
    q.x = a->x; q.in_dtype = MOE_DTYPE_BF16; q.n = n; q.hidden = h; q.topk = 1; q.scat = nullptr; q.m_limit = n;
    q.quant = fmt; q.out = w.xrow; q.out_scales = w.xrow_s; q.scale_cols = h / 32;
    e = moe::launch_permute(q, st);
    if (e != hipSuccess) return hip_fail(e, "mega_moe token quantization launch");
    xcodes = w.xrow;
    xscales = w.xrow_s;
    codes_in = true;
  }
  if (codes_in) {
    e = moe::launch_pack_tokens(xcodes, xscales, (int)h, w.tiles, w.tile_count, w.max_tiles, w.tt, w.xq, w.sx,
                                st, w.row_token);
  } else {
    moe::PermuteTilesParams pt;
    pt.x = a->x; pt.in_dtype = MOE_DTYPE_BF16; pt.hidden = (int)h; pt.row_token = w.row_token;
    pt.chunks = w.tiles; pt.chunk_count = w.tile_count; pt.max_chunks = w.max_tiles; pt.tt = w.tt; pt.fmt = fmt;
    pt.out = w.xq; pt.out_scales = w.sx;
    e = moe::launch_permute_tiles(pt, st);
  }
  if (e != hipSuccess) return hip_fail(e, "mega_moe permute launch");
  if (a->num_shared > 0) {
    if (codes_in) {
      e = moe::launch_pack_tokens(xcodes, xscales, (int)h, w.sh_tiles, w.sh_count, w.sh_max_tiles, w.sh_tt,
                                  w.xq_sh, w.sx_sh, st);
    } else {
      moe::PermuteTilesParams ps;
      ps.x = a->x; ps.in_dtype = MOE_DTYPE_BF16; ps.hidden = (int)h; ps.row_token = nullptr;
      ps.chunks = w.sh_tiles; ps.chunk_count = w.sh_count; ps.max_chunks = w.sh_max_tiles; ps.tt = w.sh_tt;
      ps.fmt = fmt; ps.out = w.xq_sh; ps.out_scales = w.sx_sh;
      e = moe::launch_permute_tiles(ps, st);
    }
    if (e != hipSuccess) return hip_fail(e, "mega_moe shared permute launch");
  }
  if (a->xq || a->sx) {
    e = moe::launch_unpack_tokens(w.xq, w.sx, (int)h, w.tiles, w.tile_count, w.max_tiles, w.tt, a->xq, a->sx, st);
    if (e != hipSuccess) return hip_fail(e, "mega_moe unpack launch");
  }
  if ((e = mark(2)) != hipSuccess) return hip_fail(e, "mega_moe event record");
  // stage 2: GMM1 + SwiGLU + MX requantization
  const int packed = a->weight_format == MOE_WEIGHTS_PACKED;
  const int wfp4 = a->weight_dtype == MOE_FP4_E2M1;
  const int swfp4 = (a->shared_weight_dtype ? a->shared_weight_dtype : a->weight_dtype) == MOE_FP4_E2M1;
  moe::Gmm1Params g1{w.xq, w.sx, a->w1, a->w1_scales, w.tiles, w.tile_count, w.max_tiles,
                     (int)h, (int)inter, fmt, w.tt, w.aq, w.sa, a->h1, packed, act, wfp4};
  if (w.fold) {   // the shared expert's chunks run in the same launch
    g1.tile_count = w.all_count;
    g1.max_tiles = w.max_tiles + w.sh_max_tiles;
    g1.shared.group = (int)ne; g1.shared.w = a->shared_w1; g1.shared.ws = a->shared_w1_scales;
  }
  g1.classes = classes;
  e = moe::launch_gmm1(g1, st);
  if (e != hipSuccess) return hip_fail(e, "mega_moe gmm1 launch");
  if (a->aq || a->sa) {
    e = moe::launch_unpack_tokens(w.aq, w.sa, (int)aw, w.tiles, w.tile_count, w.max_tiles, w.tt, a->aq, a->sa, st);
    if (e != hipSuccess) return hip_fail(e, "mega_moe unpack launch");
  }
  if ((e = mark(3)) != hipSuccess) return hip_fail(e, "mega_moe event record");
  // stage 3: GMM2, O rows in fp32
  float* o = a->o ? a->o : w.o;
  moe::Gmm2Params g2{w.aq, w.sa, a->w2, a->w2_scales, w.tiles, w.tile_count, w.max_tiles,
                     (int)h, (int)aw, fmt, w.tt, o, packed, wfp4};
  g2.o16 = o ? nullptr : w.o16;
  if (w.fold) {
    g2.tile_count = w.all_count;
    g2.max_tiles = g1.max_tiles;
    g2.shared.group = (int)ne; g2.shared.w = a->shared_w2; g2.shared.ws = a->shared_w2_scales;
  }
  g2.classes = classes;
  e = moe::launch_gmm2(g2, st);
  if (e != hipSuccess) return hip_fail(e, "mega_moe gmm2 launch");
  if ((e = mark(4)) != hipSuccess) return hip_fail(e, "mega_moe event record");
  // shared experts (when not folded into the launches above): the same FFN over all
  // tokens in token order
  for (int64_t s = 0; s < (w.fold ? 0 : a->num_shared); ++s) {
    // bytes of one shared expert's codes: halved for MXFP4 (two codes a byte)
    moe::Gmm1Params s1{w.xq_sh, w.sx_sh, a->shared_w1 + (s * 2 * inter * h >> swfp4),
                       a->shared_w1_scales + s * group_scale_bytes(2 * inter, h, a->weight_format), w.sh_tiles,
                       w.sh_count, w.sh_max_tiles, (int)h, (int)inter, fmt, w.sh_tt, w.aq_sh, w.sa_sh, nullptr,
                       packed, act, swfp4};
    e = moe::launch_gmm1(s1, st);
    if (e != hipSuccess) return hip_fail(e, "mega_moe shared gmm1 launch");
    moe::Gmm2Params s2{w.aq_sh, w.sa_sh, a->shared_w2 + (s * h * aw >> swfp4),
                       a->shared_w2_scales + s * group_scale_bytes(h, aw, a->weight_format), w.sh_tiles,
                       w.sh_count, w.sh_max_tiles, (int)h, (int)aw, fmt, w.sh_tt,
                       w.o_sh ? w.o_sh + s * n * h : nullptr, packed, swfp4};
    s2.o16 = w.o16_sh ? w.o16_sh + s * n * h : nullptr;
    e = moe::launch_gmm2(s2, st);
    if (e != hipSuccess) return hip_fail(e, "mega_moe shared gmm2 launch");
  }
  if ((e = mark(5)) != hipSuccess) return hip_fail(e, "mega_moe event record");
  // stage 4: weighted combine into bf16 y (one rounding, after the sum)
  moe::CombineParams cp;
  // combine_comm_mode 0: bf16 rows (rounded as read from the caller's fp32 o)
  cp.o = o ? (const void*)o : (const void*)w.o16;
  cp.o_fmt = a->combine_comm_mode == 0 ? (o ? 1 : 2) : 0;
  cp.sh_bf16 = a->combine_comm_mode == 0;
  cp.pos = w.scat; cp.w = a->topk_weights; cp.w_bf16 = a->topk_weights_dtype == MOE_DTYPE_BF16;
  cp.topk = (int)a->topk; cp.o_shared = w.o_sh ? (const void*)w.o_sh : (const void*)w.o16_sh; cp.num_shared = (int)a->num_shared; cp.tokens = n;
  cp.hidden = (int)h; cp.y = reinterpret_cast<uint16_t*>(a->y);
  e = moe::launch_combine(cp, st);
  if (e != hipSuccess) return hip_fail(e, "mega_moe combine launch");
  if ((e = mark(6)) != hipSuccess) return hip_fail(e, "mega_moe event record");
  return ok();
}

moe_status moe_gmm_workspace_size(int64_t rows, int64_t num_groups, int64_t hidden, int64_t inter, size_t* bytes) {
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "moe_gmm_workspace_size: bytes is NULL");
  if (moe_status s = check_gmm_common("moe_gmm_workspace_size", rows, hidden, inter, num_groups, MOE_FP8_E4M3))
    return s;
  Carver cv(nullptr);
  carve_gmm(cv, rows, num_groups, hidden, inter);
  *bytes = cv.off;
  return ok();
}

moe_status moe_gmm1_swiglu_quant(const uint8_t* xq, const uint8_t* sx, int64_t rows, int64_t hidden, int64_t inter,
                                 const int32_t* group_offsets, int64_t num_groups, const uint8_t* w1,
                                 const uint8_t* w1_scales, int weight_format, int quant_out_dtype, uint8_t* aq,
                                 uint8_t* sa, float* h1, void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "moe_gmm1_swiglu_quant";
  if (moe_status s = check_gmm_common(who, rows, hidden, inter, num_groups, quant_out_dtype)) return s;
  if (weight_format != MOE_WEIGHTS_ND && weight_format != MOE_WEIGHTS_PACKED)
    return fail(MOE_ERR_INVALID_ARG, "%s: weight_format %d not 0 or 1", who, weight_format);
  if (!group_offsets || !w1 || !w1_scales || (rows > 0 && (!xq || !sx || !aq || !sa)))
    return fail(MOE_ERR_INVALID_ARG, "%s: NULL buffer", who);
  Carver cv(nullptr);
  carve_gmm(cv, rows, num_groups, hidden, inter);
  if (moe_status s = check_ws(who, cv.off, workspace, workspace_bytes)) return s;
  if (rows == 0) return ok();
  Carver wc(workspace);
  GmmWs w = carve_gmm(wc, rows, num_groups, hidden, inter);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = moe::launch_build_tiles(group_offsets, (int)num_groups, (int)rows, 16 * w.tt, w.max_tiles, w.tiles, w.count, st);
  if (e != hipSuccess) return hip_fail(e, "tile list launch");
  e = moe::launch_pack_tokens(xq, sx, (int)hidden, w.tiles, w.count, w.max_tiles, w.tt, w.in_codes, w.in_scales, st);
  if (e != hipSuccess) return hip_fail(e, "token pack launch");
  moe::Gmm1Params g{w.in_codes, w.in_scales, w1, w1_scales, w.tiles, w.count, w.max_tiles, (int)hidden, (int)inter,
                    quant_out_dtype == MOE_FP8_E4M3 ? 0 : 1, w.tt, w.out_codes, w.out_scales, h1, weight_format};
  e = moe::launch_gmm1(g, st);
  if (e != hipSuccess) return hip_fail(e, "gmm1 launch");
  e = moe::launch_unpack_tokens(w.out_codes, w.out_scales, (int)inter, w.tiles, w.count, w.max_tiles, w.tt, aq, sa, st);
  if (e != hipSuccess) return hip_fail(e, "token unpack launch");
  return ok();
}

moe_status moe_gmm2_combine(const uint8_t* aq, const uint8_t* sa, int64_t rows, int64_t inter, int64_t hidden,
                            const int32_t* group_offsets, int64_t num_groups, const uint8_t* w2,
                            const uint8_t* w2_scales, int weight_format, int quant_out_dtype,
                            const int32_t* row_token, const float* row_weight, int64_t num_tokens, float* y_accum,
                            float* o, void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "moe_gmm2_combine";
  if (moe_status s = check_gmm_common(who, rows, hidden, inter, num_groups, quant_out_dtype)) return s;
  if (weight_format != MOE_WEIGHTS_ND && weight_format != MOE_WEIGHTS_PACKED)
    return fail(MOE_ERR_INVALID_ARG, "%s: weight_format %d not 0 or 1", who, weight_format);
  if (num_tokens < 1) return fail(MOE_ERR_SHAPE, "%s: num_tokens must be >= 1", who);
  if (!group_offsets || !w2 || !w2_scales || (rows > 0 && (!aq || !sa || !row_token || !row_weight || !y_accum)))
    return fail(MOE_ERR_INVALID_ARG, "%s: NULL buffer", who);
  Carver cv(nullptr);
  carve_gmm(cv, rows, num_groups, hidden, inter);
  if (moe_status s = check_ws(who, cv.off, workspace, workspace_bytes)) return s;
  if (rows == 0) return ok();
  Carver wc(workspace);
  GmmWs w = carve_gmm(wc, rows, num_groups, hidden, inter);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = moe::launch_build_tiles(group_offsets, (int)num_groups, (int)rows, 16 * w.tt, w.max_tiles, w.tiles, w.count, st);
  if (e != hipSuccess) return hip_fail(e, "tile list launch");
  e = moe::launch_pack_tokens(aq, sa, (int)inter, w.tiles, w.count, w.max_tiles, w.tt, w.in_codes, w.in_scales, st);
  if (e != hipSuccess) return hip_fail(e, "token pack launch");
  moe::Gmm2Params g{w.in_codes, w.in_scales, w2, w2_scales, w.tiles, w.count, w.max_tiles, (int)hidden, (int)inter,
                    quant_out_dtype == MOE_FP8_E4M3 ? 0 : 1, w.tt, o ? o : w.o, weight_format};
  e = moe::launch_gmm2(g, st);
  if (e != hipSuccess) return hip_fail(e, "gmm2 launch");
  e = moe::launch_scatter_add(o ? o : w.o, rows, (int)hidden, row_token, row_weight, y_accum, st);
  if (e != hipSuccess) return hip_fail(e, "scatter-add launch");
  return ok();
}

moe_status moe_combine_finalize(const float* y_accum, int64_t num_tokens, int64_t hidden, void* y, void* stream) {
  if (num_tokens < 0 || hidden < 1) return fail(MOE_ERR_SHAPE, "moe_combine_finalize: bad sizes");
  if (num_tokens == 0) return ok();
  if (!y_accum || !y) return fail(MOE_ERR_INVALID_ARG, "moe_combine_finalize: NULL buffer");
  hipError_t e = moe::launch_finalize(y_accum, num_tokens * hidden, reinterpret_cast<uint16_t*>(y), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "finalize launch");
  return ok();
}

moe_status moe_probe_stream(int mode, const void* src, void* dst, int64_t bytes, void* stream) {
  if (mode < 0 || mode > 2) return fail(MOE_ERR_INVALID_ARG, "moe_probe_stream: mode %d not 0, 1 or 2", mode);
  if (bytes <= 0 || bytes % 16 != 0) return fail(MOE_ERR_SHAPE, "moe_probe_stream: bytes must be a positive multiple of 16");
  if (!src || !dst) return fail(MOE_ERR_INVALID_ARG, "moe_probe_stream: NULL buffer");
  hipError_t e = moe::launch_probe_stream(mode, src, dst, bytes, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "stream probe launch");
  return ok();
}

moe_status moe_probe_mfma(int iters, float* out, int64_t* out_floats, double* flops, void* stream) {
  if (iters < 1) return fail(MOE_ERR_SHAPE, "moe_probe_mfma: iters must be >= 1");
  const int64_t need = (int64_t)moe::probe_mfma_blocks() * 256;
  if (out_floats) *out_floats = need;
  if (flops) *flops = moe::probe_mfma_flops(iters);
  if (!out) return ok();
  hipError_t e = moe::launch_probe_mfma(iters, out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mfma probe launch");
  return ok();
}

}  // extern "C"
