// Token rows in the tiled operand layout of the grouped GEMMs.
//
// MegaMoE README, "A8W8-FP quantization scenario", stage 1: X^_e, S_X,e = Q_MX(X[T_e]):
// the rows of each expert, gathered from the token matrix and MX-quantized (groups of
// 32, FP8 E4M3FN/E5M2 codes, one E8M0 scale per group). Here the gathered rows are
// written straight into the tiled layout of device_common.h, in which one 16-row x
// 128-K tile is 2 KB of contiguous memory in MFMA lane order, so that a GEMM wave
// stages a tile with two 1 KB loads instead of sixteen 64-byte row pieces.
//
// All kernels walk the chunk list of the GEMMs (int4 {group, padded row0, rows, sorted
// row0}, chunks of up to 16*tt rows, padded row0 a multiple of 16) and give one wave
// to each (chunk, 16-row tile, quad of 128-K steps). Lane (g, r) handles row r of the
// tile and K bytes [16g, +16) and [64 + 16g, +16) of each step: the same bytes it
// holds as an MFMA operand, so every store is 1 KB contiguous per wave. Rows of a tile
// past the chunk's end are written as zeros (code 0, scale 0).

#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

template <typename InT> struct Load16;
template <> struct Load16<uint16_t> {  // bf16
  static __device__ __forceinline__ void run(const uint16_t* p, float* f) {
    const u32x4 a = reinterpret_cast<const u32x4*>(p)[0];
    const u32x4 b = reinterpret_cast<const u32x4*>(p)[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(a[i] << 16);
      f[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
      f[8 + 2 * i] = __uint_as_float(b[i] << 16);
      f[8 + 2 * i + 1] = __uint_as_float(b[i] & 0xffff0000u);
    }
  }
};
template <> struct Load16<_Float16> {
  static __device__ __forceinline__ void run(const _Float16* p, float* f) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 a = reinterpret_cast<const h8*>(p)[0];
    const h8 b = reinterpret_cast<const h8*>(p)[1];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f[i] = (float)a[i];
      f[8 + i] = (float)b[i];
    }
  }
};
template <> struct Load16<float> {
  static __device__ __forceinline__ void run(const float* p, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = reinterpret_cast<const float4*>(p)[i];
      f[4 * i] = v.x; f[4 * i + 1] = v.y; f[4 * i + 2] = v.z; f[4 * i + 3] = v.w;
    }
  }
};

// Item it -> (chunk, tile of the chunk, quad); false if the tile is past the chunk.
struct TileItem {
  int64_t tile;   // tile index in the padded row space
  int64_t srow;   // sorted (unpadded) row of the tile's first row
  int nvalid;     // rows of the tile inside the chunk (1..16)
  int quad;
};

__device__ __forceinline__ bool tile_item(int64_t it, int tt, int kq, const int4* __restrict__ chunks, TileItem* ti) {
  const int per_chunk = tt * kq;
  const int j = (int)(it / per_chunk);
  const int rem = (int)(it - (int64_t)j * per_chunk);
  const int u = rem / kq;
  const int4 c = chunks[j];
  if (16 * u >= c.z) return false;
  ti->tile = (int64_t)(c.y >> 4) + u;
  ti->srow = (int64_t)c.w + 16 * u;
  ti->nvalid = min(16, c.z - 16 * u);
  ti->quad = rem - u * kq;
  return true;
}

__device__ __forceinline__ int64_t tile_items(const int* chunk_count, int max_chunks, int tt, int kq) {
  return (int64_t)min(*chunk_count, max_chunks) * tt * kq;
}

// Gather + MX quantization into the tiled layout. row_token[sorted row] is the source
// token row (nullptr: the sorted row itself).
template <typename InT, int FMT>
__global__ __launch_bounds__(256) void permute_tiles_kernel(const InT* __restrict__ x, int hidden,
                                                            const int32_t* __restrict__ row_token,
                                                            const int4* __restrict__ chunks,
                                                            const int* __restrict__ chunk_count, int max_chunks,
                                                            int tt, uint8_t* __restrict__ out,
                                                            uint8_t* __restrict__ out_scales) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
  const int ks = hidden >> 7, kq = (ks + 3) >> 2;
  const int64_t items = tile_items(chunk_count, max_chunks, tt, kq);
  for (int64_t it = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); it < items; it += (int64_t)gridDim.x * 4) {
    TileItem ti;
    if (!tile_item(it, tt, kq, chunks, &ti)) continue;   // uniform per wave
    const bool valid = r < ti.nvalid;
    const int64_t src = valid ? (row_token ? (int64_t)row_token[ti.srow + r] : ti.srow + r) : 0;
    const InT* row = x + src * hidden;
    // The loads of all four steps first (steps past the end re-read the last one).
    float lo[4][16], hi[4][16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = min(4 * ti.quad + i, ks - 1);
      if (valid) {
        Load16<InT>::run(row + 128 * s + 16 * g, lo[i]);
        Load16<InT>::run(row + 128 * s + 64 + 16 * g, hi[i]);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) lo[i][e] = hi[i][e] = 0.0f;
      }
    }
    uint32_t sword = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 4 * ti.quad + i;
      if (s >= ks) break;   // uniform
      // K bytes [16g, +16) lie in MX group g/2 of the step, [64 + 16g, +16) in group
      // 2 + g/2; the two lanes g and g^1 (lane ^ 16) share each group.
      int mlo = 0, mhi = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        mlo = max(mlo, __float_as_int(fabsf(lo[i][e])));
        mhi = max(mhi, __float_as_int(fabsf(hi[i][e])));
      }
      mlo = max(mlo, __shfl_xor(mlo, 16));
      mhi = max(mhi, __shfl_xor(mhi, 16));
      const int blo = mx_scale_byte<FMT>(__int_as_float(mlo));
      const int bhi = mx_scale_byte<FMT>(__int_as_float(mhi));
      const float ilo = mx_inv_scale(blo), ihi = mx_inv_scale(bhi);
      u32x4 clo, chi;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        clo[w] = pack4<FMT>(lo[i][4 * w] * ilo, lo[i][4 * w + 1] * ilo, lo[i][4 * w + 2] * ilo, lo[i][4 * w + 3] * ilo);
        chi[w] = pack4<FMT>(hi[i][4 * w] * ihi, hi[i][4 * w + 1] * ihi, hi[i][4 * w + 2] * ihi, hi[i][4 * w + 3] * ihi);
      }
      uint8_t* tb = out + t16_codes(ti.tile, ks, s);
      reinterpret_cast<u32x4*>(tb)[lane] = clo;
      reinterpret_cast<u32x4*>(tb + 1024)[lane] = chi;
      // The scale lane (g, r) carries is that of MX group g: group g < 2 is the low
      // group of lanes 2g, 2g+1, group g >= 2 the high group of lanes 2g-4, 2g-3.
      const int both = blo | (bhi << 8);
      const int from = __shfl(both, ((2 * g) & 3) * 16 + r);
      sword |= (uint32_t)(g < 2 ? (from & 0xff) : (from >> 8)) << (8 * i);
    }
    reinterpret_cast<uint32_t*>(out_scales + t16_scales(ti.tile, kq, ti.quad))[lane] = sword;
  }
}

// Row-major FP8 codes [rows, K] and scales [rows, K/32] -> tiled layout. Sorted row i
// takes source row row_token[i] (a gather of already quantized tokens), or row i itself
// when row_token is null.
__global__ __launch_bounds__(256) void pack_tokens_kernel(const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ scales, int K,
                                                          const int32_t* __restrict__ row_token,
                                                          const int4* __restrict__ chunks,
                                                          const int* __restrict__ chunk_count, int max_chunks, int tt,
                                                          uint8_t* __restrict__ out, uint8_t* __restrict__ out_scales) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
  const int ks = K >> 7, kq = (ks + 3) >> 2, kb = K >> 5;
  const int64_t items = tile_items(chunk_count, max_chunks, tt, kq);
  for (int64_t it = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); it < items; it += (int64_t)gridDim.x * 4) {
    TileItem ti;
    if (!tile_item(it, tt, kq, chunks, &ti)) continue;
    const bool valid = r < ti.nvalid;
    const int64_t row = valid && row_token ? (int64_t)row_token[ti.srow + r] : ti.srow + r;
    // The loads of all four steps first (steps past the end re-read the last one and are
    // not stored), then the stores: a wave keeps 128 bytes a lane in flight.
    const uint8_t* src = codes + row * K + 16 * g;
    u32x4 lo[4], hi[4];
    uint32_t sb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = min(4 * ti.quad + i, ks - 1);
      lo[i] = hi[i] = u32x4{0u, 0u, 0u, 0u};
      sb[i] = 0;
      if (valid) {
        lo[i] = *reinterpret_cast<const u32x4*>(src + 128 * s);
        hi[i] = *reinterpret_cast<const u32x4*>(src + 128 * s + 64);
        sb[i] = scales[row * kb + 4 * s + g];
      }
    }
    uint32_t sword = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * ti.quad + i < ks) sword |= sb[i] << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 4 * ti.quad + i;
      if (s >= ks) break;
      // non-temporal: the tiles are read back by the GEMM's own loads (measured: GMM1 of
      // the prefill-shaped layer 2% faster than after plain stores)
      uint8_t* tb = out + t16_codes(ti.tile, ks, s);
      __builtin_nontemporal_store(lo[i], reinterpret_cast<u32x4*>(tb) + lane);
      __builtin_nontemporal_store(hi[i], reinterpret_cast<u32x4*>(tb + 1024) + lane);
    }
    reinterpret_cast<uint32_t*>(out_scales + t16_scales(ti.tile, kq, ti.quad))[lane] = sword;
  }
}

// Tiled layout -> row-major FP8 codes [rows, K] and scales [rows, K/32] (valid rows only;
// either output may be null).
__global__ __launch_bounds__(256) void unpack_tokens_kernel(const uint8_t* __restrict__ in,
                                                            const uint8_t* __restrict__ in_scales, int K,
                                                            const int4* __restrict__ chunks,
                                                            const int* __restrict__ chunk_count, int max_chunks,
                                                            int tt, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
  const int ks = K >> 7, kq = (ks + 3) >> 2, kb = K >> 5;
  const int64_t items = tile_items(chunk_count, max_chunks, tt, kq);
  for (int64_t it = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); it < items; it += (int64_t)gridDim.x * 4) {
    TileItem ti;
    if (!tile_item(it, tt, kq, chunks, &ti)) continue;
    if (r >= ti.nvalid) continue;   // per lane; no cross-lane work below
    const int64_t row = ti.srow + r;
    const uint32_t sword = reinterpret_cast<const uint32_t*>(in_scales + t16_scales(ti.tile, kq, ti.quad))[lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = 4 * ti.quad + i;
      if (s >= ks) break;
      if (codes) {
        const uint8_t* tb = in + t16_codes(ti.tile, ks, s);
        *reinterpret_cast<u32x4*>(codes + row * K + 128 * s + 16 * g) = reinterpret_cast<const u32x4*>(tb)[lane];
        *reinterpret_cast<u32x4*>(codes + row * K + 128 * s + 64 + 16 * g) =
            reinterpret_cast<const u32x4*>(tb + 1024)[lane];
      }
      if (scales) scales[row * kb + 4 * s + g] = (uint8_t)(sword >> (8 * i));
    }
  }
}

unsigned tile_grid(int max_chunks, int tt, int K) {
  const int64_t kq = ((K >> 7) + 3) >> 2;
  const int64_t waves = (int64_t)max_chunks * tt * kq;
  const int64_t blocks = (waves + 3) / 4;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(blocks, 4096));
}

template <typename InT>
hipError_t permute_tiles_typed(const PermuteTilesParams& p, hipStream_t st) {
  const unsigned grid = tile_grid(p.max_chunks, p.tt, p.hidden);
  const InT* x = reinterpret_cast<const InT*>(p.x);
  if (p.fmt == 0)
    permute_tiles_kernel<InT, 0><<<grid, 256, 0, st>>>(x, p.hidden, p.row_token, p.chunks, p.chunk_count,
                                                       p.max_chunks, p.tt, p.out, p.out_scales);
  else
    permute_tiles_kernel<InT, 1><<<grid, 256, 0, st>>>(x, p.hidden, p.row_token, p.chunks, p.chunk_count,
                                                       p.max_chunks, p.tt, p.out, p.out_scales);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_permute_tiles(const PermuteTilesParams& p, hipStream_t stream) {
  if (p.max_chunks <= 0) return hipSuccess;
  switch (p.in_dtype) {
    case 0: return permute_tiles_typed<float>(p, stream);
    case 1: return permute_tiles_typed<_Float16>(p, stream);
    default: return permute_tiles_typed<uint16_t>(p, stream);
  }
}

hipError_t launch_pack_tokens(const uint8_t* codes, const uint8_t* scales, int K, const int4* chunks,
                              const int* chunk_count, int max_chunks, int tt, uint8_t* out, uint8_t* out_scales,
                              hipStream_t stream, const int32_t* row_token) {
  if (max_chunks <= 0) return hipSuccess;
  pack_tokens_kernel<<<tile_grid(max_chunks, tt, K), 256, 0, stream>>>(codes, scales, K, row_token, chunks,
                                                                        chunk_count, max_chunks, tt, out, out_scales);
  return hipGetLastError();
}

hipError_t launch_unpack_tokens(const uint8_t* in, const uint8_t* in_scales, int K, const int4* chunks,
                                const int* chunk_count, int max_chunks, int tt, uint8_t* codes, uint8_t* scales,
                                hipStream_t stream) {
  if (max_chunks <= 0) return hipSuccess;
  unpack_tokens_kernel<<<tile_grid(max_chunks, tt, K), 256, 0, stream>>>(in, in_scales, K, chunks, chunk_count,
                                                                          max_chunks, tt, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
