// Weighted combine of the expert outputs back into token order.
//
// MegaMoE README, "A8W8-FP quantization scenario", stage 4: Y[i] = sum_k W[i, k] *
// O[pi(i, k)], with pi the permutation of the routing (token i's k-th expert row), plus
// the outputs of the shared experts, which see every token, unweighted; the
// moe_token_permute article's unpermute direction is the same gather. The sum is fp32
// and Y is rounded to bf16 once, after it. MegaMoE's combineCommMode decides what the
// combine receives: with mode 0 (no deduplication, the default) every expert's output
// row arrives as BF16, so each O row is rounded to bf16 first (stored so by GMM2, or
// rounded here as it is read); with mode 1 (a token's experts merged in FP32 on the
// card) the rows stay fp32.
//
// Each thread owns 4 consecutive channels of one token (16- or 8-byte loads of the K
// expert rows and the shared rows, summed in the order k = 0..K-1, then the shared
// experts in order) and writes 8 bytes of bf16.

#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

__device__ __forceinline__ void fma4(float4& acc, float w, const float4& v) {
  acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
}

__device__ __forceinline__ float round_bf16(float v) { return bf16_to_f(f_to_bf16(v)); }

// 4 consecutive channels (index c of 4) of a row: OF 0 fp32, 1 fp32 rounded to bf16,
// 2 bf16.
template <int OF>
__device__ __forceinline__ float4 load4(const void* base, int64_t row, int hidden, int c) {
  // (each expert row is read once: non-temporal loads)
  if constexpr (OF == 2) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 u =
        __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(base) + row * hidden) + c);
    return make_float4(bf16_to_f((uint16_t)u[0]), bf16_to_f((uint16_t)(u[0] >> 16)), bf16_to_f((uint16_t)u[1]),
                       bf16_to_f((uint16_t)(u[1] >> 16)));
  } else {
    const v4f u =
        __builtin_nontemporal_load(reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(base) + row * hidden) + c);
    float4 v = make_float4(u[0], u[1], u[2], u[3]);
    if constexpr (OF == 1) v = make_float4(round_bf16(v.x), round_bf16(v.y), round_bf16(v.z), round_bf16(v.w));
    return v;
  }
}

// Block b covers token b / slices and 1024 channels (256 threads x 4) of it, so that few
// tokens still fill the chip. The K rows are loaded four at a time, all four loads in
// flight before their products are added (in order k = 0..K-1).
// OF: format of the routed rows (see load4); SF: of the shared rows (0 fp32, 2 bf16).
template <int OF, int SF>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ o, const int32_t* __restrict__ pos,
                                                      const void* __restrict__ wts, int w_bf16, int topk,
                                                      const void* __restrict__ o_shared, int num_shared,
                                                      int64_t tokens, int hidden, uint16_t* __restrict__ y) {
  const int h4 = hidden >> 2;
  const int slices = (h4 + 255) >> 8;
  const int64_t nblk = tokens * slices;
  for (int64_t b = blockIdx.x; b < nblk; b += gridDim.x) {
    const int64_t t = b / slices;
    const int c = (int)(b - t * slices) * 256 + (int)threadIdx.x;
    if (c >= h4) continue;
    auto weight = [&](int64_t f) {
      return w_bf16 ? bf16_to_f(reinterpret_cast<const uint16_t*>(wts)[f]) : reinterpret_cast<const float*>(wts)[f];
    };
    auto row = [&](int p) { return load4<OF>(o, p, hidden, c); };
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int k = 0;
    for (; k + 4 <= topk; k += 4) {
      const int64_t f = t * topk + k;
      int p[4];
      float4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = pos[f + j];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = row(p[j] < 0 ? 0 : p[j]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (p[j] >= 0) fma4(acc, weight(f + j), v[j]);
    }
    for (; k < topk; ++k) {
      const int64_t f = t * topk + k;
      const int p = pos[f];
      if (p >= 0) fma4(acc, weight(f), row(p));
    }
    for (int s = 0; s < num_shared; ++s) {
      const float4 v = load4<SF>(o_shared, (int64_t)s * tokens + t, hidden, c);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    u32x2 out;
    out[0] = (uint32_t)f_to_bf16(acc.x) | ((uint32_t)f_to_bf16(acc.y) << 16);
    out[1] = (uint32_t)f_to_bf16(acc.z) | ((uint32_t)f_to_bf16(acc.w) << 16);
    __builtin_nontemporal_store(out, reinterpret_cast<u32x2*>(y + t * hidden) + c);   // Y is not read back here
  }
}

__global__ __launch_bounds__(256) void scatter_add_kernel(const float* __restrict__ o, int64_t rows, int hidden,
                                                          const int32_t* __restrict__ row_token,
                                                          const float* __restrict__ row_weight,
                                                          float* __restrict__ y_accum) {
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const int64_t tok = row_token[r];
    const float w = row_weight[r];
    for (int c = threadIdx.x; c < hidden; c += blockDim.x)
      unsafeAtomicAdd(y_accum + tok * hidden + c, w * o[r * hidden + c]);
  }
}

__global__ void finalize_kernel(const float* __restrict__ acc, int64_t n, uint16_t* __restrict__ y) {
  const int64_t n4 = n >> 2;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    const float4 v = reinterpret_cast<const float4*>(acc)[i];
    uint2 out;
    out.x = (uint32_t)f_to_bf16(v.x) | ((uint32_t)f_to_bf16(v.y) << 16);
    out.y = (uint32_t)f_to_bf16(v.z) | ((uint32_t)f_to_bf16(v.w) << 16);
    reinterpret_cast<uint2*>(y)[i] = out;
  }
  for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    y[i] = f_to_bf16(acc[i]);
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t st) {
  if (p.tokens <= 0) return hipSuccess;
  const int64_t slices = ((p.hidden >> 2) + 255) >> 8;
  const unsigned grid = (unsigned)std::min<int64_t>(p.tokens * slices, 1 << 20);
  // routed rows fp32 (mode 1), fp32 rounded as read or bf16 (mode 0, shared rows bf16)
  auto kern = p.o_fmt == 2 ? combine_kernel<2, 2> : p.o_fmt == 1 ? combine_kernel<1, 2> : combine_kernel<0, 0>;
  if ((p.o_fmt != 0) != (p.sh_bf16 != 0)) return hipErrorInvalidValue;
  kern<<<grid, 256, 0, st>>>(p.o, p.pos, p.w, p.w_bf16, p.topk, p.o_shared, p.num_shared, p.tokens, p.hidden, p.y);
  return hipGetLastError();
}

hipError_t launch_scatter_add(const float* o, int64_t rows, int hidden, const int32_t* row_token,
                              const float* row_weight, float* y_accum, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>(rows, 65536);
  scatter_add_kernel<<<grid, 256, 0, st>>>(o, rows, hidden, row_token, row_weight, y_accum);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* acc, int64_t count, uint16_t* y, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((count / 4 + 255) / 256 + 1, 65536);
  finalize_kernel<<<(unsigned)blocks, 256, 0, st>>>(acc, count, y);
  return hipGetLastError();
}

}  // namespace moe
