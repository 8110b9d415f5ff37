// Gather of token rows into expert-contiguous order, fused with MX quantization.
//
// MegaMoE README, "A8W8-FP quantization scenario", stage 1: X^_e, S_X,e = Q_MX(X[T_e]),
// groups of 32 elements, FP8 E4M3FN/E5M2 codes with one E8M0 scale per group.
// MoeInitRoutingV3 README, 计算公式 5 (quantized gather) and moe_token_permute
// article, 功能说明 (row i of the output is token first(i) / topK); scale layout
// [rows, AlignUp(CeilDiv(H, 32), 2)] from the article's 返回值说明.
//
// The kernel is written in scatter form: one wave per *token*. The wave reads the
// token's K destination rows (the scatter-type index), skips the token if none is
// in range, otherwise reads the bf16 row once, quantizes it once and stores the
// same codes to every destination. Each lane owns 8 consecutive elements (one
// 16-byte load), so a 32-element group is a DPP quad and its amax takes two
// quad_perm max steps; a wave covers 512 elements per step and the loads of
// kUnroll steps are issued before any store.

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

// Vectors (8 elements) per lane in flight per step: 4 measured fastest on the
// 32768 x 7168 bf16 routing workload (8 and 16 cut occupancy).
constexpr int kUnroll = 4;

template <typename InT> struct Load8;
template <> struct Load8<uint16_t> {  // bf16
  static __device__ __forceinline__ void run(const uint16_t* p, float* f) {
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));   // each row is read once
    const uint32_t w[4] = {u[0], u[1], u[2], u[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Load8<_Float16> {
  static __device__ __forceinline__ void run(const _Float16* p, float* f) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 h = *reinterpret_cast<const h8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
  }
};
template <> struct Load8<float> {
  static __device__ __forceinline__ void run(const float* p, float* f) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

// Destination row of token t (-1 = none) held by lane j < topk.
__device__ __forceinline__ int token_dest(const int32_t* scat, int64_t t, int topk, int64_t m_limit, int lane) {
  int dest = -1;
  if (scat) {
    if (lane < topk) {
      const int d = scat[t * topk + lane];
      dest = (d >= 0 && d < m_limit) ? d : -1;
    }
  } else if (lane == 0) {
    dest = t < m_limit ? (int)t : -1;
  }
  return dest;
}

template <typename InT, int FMT>
__global__ __launch_bounds__(256) void permute_mx_kernel(
    const InT* __restrict__ x, int64_t n, int hidden, int topk, const int32_t* __restrict__ scat,
    int64_t m_limit, uint8_t* __restrict__ out, uint8_t* __restrict__ out_scales, int scale_cols,
    uint8_t* __restrict__ tok_out, uint8_t* __restrict__ tok_scales) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= n) return;  // uniform per wave
  const int dest = token_dest(scat, t, topk, m_limit, lane);
  const uint64_t dmask = __ballot(dest >= 0);
  if (dmask == 0 && tok_out == nullptr) return;
  const int nvec = hidden >> 3;
  const int groups = hidden >> 5;
  const InT* row = x + t * (int64_t)hidden;
  for (int v0 = 0; v0 < nvec; v0 += 64 * kUnroll) {
    float f[kUnroll][8];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * 64 + lane;
      if (v < nvec) {
        Load8<InT>::run(row + (int64_t)v * 8, f[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[u][i] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * 64 + lane;
      int m = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = max(m, __float_as_int(fabsf(f[u][i])));
      m = quad_max_bits(m);  // all lanes take part; a quad is all-valid or all-invalid
      const int b = mx_scale_byte<FMT>(__int_as_float(m));
      const float inv = mx_inv_scale(b);
      uint2 q;
      if constexpr (FMT == 2) {   // MXFP4: 8 nibbles, element 2j in the low nibble of byte j
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) w |= fp4_code(f[u][i] * inv) << (4 * i);
        q.x = w;
        q.y = 0;
      } else {
        q.x = pack4<FMT>(f[u][0] * inv, f[u][1] * inv, f[u][2] * inv, f[u][3] * inv);
        q.y = pack4<FMT>(f[u][4] * inv, f[u][5] * inv, f[u][6] * inv, f[u][7] * inv);
      }
      if (v < nvec) {
        const bool scale_lane = (lane & 3) == 0;
        for (uint64_t dm = dmask; dm; dm &= dm - 1) {
          const int k = __builtin_ctzll(dm);
          const int64_t d = __builtin_amdgcn_readlane(dest, k);
          // the permuted rows are written once and not read back here: non-temporal
          if constexpr (FMT == 2)
            __builtin_nontemporal_store(q.x, reinterpret_cast<uint32_t*>(out + d * (hidden >> 1) + (int64_t)v * 4));
          else
            __builtin_nontemporal_store(((uint64_t)q.y << 32) | q.x,
                                        reinterpret_cast<uint64_t*>(out + d * hidden + (int64_t)v * 8));
          if (scale_lane) out_scales[d * scale_cols + (v >> 2)] = (uint8_t)b;
        }
        if (tok_out) {
          *reinterpret_cast<uint2*>(tok_out + t * hidden + (int64_t)v * 8) = q;
          if (scale_lane) tok_scales[t * scale_cols + (v >> 2)] = (uint8_t)b;
        }
      }
    }
  }
  if (scale_cols > groups && lane == 0) {  // padding scale of an odd group count
    for (uint64_t dm = dmask; dm; dm &= dm - 1) {
      const int64_t d = __builtin_amdgcn_readlane(dest, __builtin_ctzll(dm));
      out_scales[d * scale_cols + groups] = 0;
    }
    if (tok_out) tok_scales[t * scale_cols + groups] = 0;
  }
}

// quant_mode -1: plain row copy (any element size; 16-byte vectors when possible).
__global__ __launch_bounds__(256) void permute_copy_kernel(const uint8_t* __restrict__ x, int64_t n,
                                                           int64_t row_bytes, int topk,
                                                           const int32_t* __restrict__ scat, int64_t m_limit,
                                                           uint8_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= n) return;
  const int dest = token_dest(scat, t, topk, m_limit, lane);
  const uint64_t dmask = __ballot(dest >= 0);
  if (dmask == 0) return;
  const uint8_t* row = x + t * row_bytes;
  if ((row_bytes & 15) == 0) {
    const int64_t nv = row_bytes >> 4;
    for (int64_t v = lane; v < nv; v += 64) {
      const uint4 val = reinterpret_cast<const uint4*>(row)[v];
      for (uint64_t dm = dmask; dm; dm &= dm - 1) {
        const int64_t d = __builtin_amdgcn_readlane(dest, __builtin_ctzll(dm));
        reinterpret_cast<uint4*>(out + d * row_bytes)[v] = val;
      }
    }
  } else {
    for (int64_t v = lane; v < row_bytes; v += 64) {
      const uint8_t val = row[v];
      for (uint64_t dm = dmask; dm; dm &= dm - 1) {
        const int64_t d = __builtin_amdgcn_readlane(dest, __builtin_ctzll(dm));
        out[d * row_bytes + v] = val;
      }
    }
  }
}

template <typename InT>
hipError_t launch_mx_typed(const PermuteParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((p.n + 3) / 4)), block(256);
  const InT* x = reinterpret_cast<const InT*>(p.x);
  uint8_t* out = reinterpret_cast<uint8_t*>(p.out);
  if (p.quant == 0)
    permute_mx_kernel<InT, 0><<<grid, block, 0, stream>>>(x, p.n, (int)p.hidden, p.topk, p.scat, p.m_limit, out,
                                                          p.out_scales, (int)p.scale_cols, p.tok_out, p.tok_scales);
  else if (p.quant == 1)
    permute_mx_kernel<InT, 1><<<grid, block, 0, stream>>>(x, p.n, (int)p.hidden, p.topk, p.scat, p.m_limit, out,
                                                          p.out_scales, (int)p.scale_cols, p.tok_out, p.tok_scales);
  else   // MXFP4 rows of hidden / 2 bytes (no token-order copy)
    permute_mx_kernel<InT, 2><<<grid, block, 0, stream>>>(x, p.n, (int)p.hidden, p.topk, p.scat, p.m_limit, out,
                                                          p.out_scales, (int)p.scale_cols, nullptr, nullptr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_permute_rows(const uint8_t* x, int64_t n, int64_t row_bytes, int topk, const int32_t* scat,
                               int64_t m_limit, uint8_t* out, hipStream_t stream) {
  if (n <= 0 || row_bytes <= 0) return hipSuccess;
  permute_copy_kernel<<<(unsigned)((n + 3) / 4), 256, 0, stream>>>(x, n, row_bytes, topk, scat, m_limit, out);
  return hipGetLastError();
}

hipError_t launch_permute(const PermuteParams& p, hipStream_t stream) {
  if (p.n <= 0) return hipSuccess;
  if (p.quant < 0) {
    const int64_t esz = p.in_dtype == 0 ? 4 : 2;
    permute_copy_kernel<<<(unsigned)((p.n + 3) / 4), 256, 0, stream>>>(
        reinterpret_cast<const uint8_t*>(p.x), p.n, p.hidden * esz, p.topk, p.scat, p.m_limit,
        reinterpret_cast<uint8_t*>(p.out));
    return hipGetLastError();
  }
  switch (p.in_dtype) {
    case 0: return launch_mx_typed<float>(p, stream);
    case 1: return launch_mx_typed<_Float16>(p, stream);
    default: return launch_mx_typed<uint16_t>(p, stream);
  }
}

}  // namespace moe
