// Grouped GEMMs of the MX expert FFN on gfx950 block-scaled MFMA.
//
// MegaMoE README, "A8W8-FP quantization scenario":
//   stage 2  G_e = DQ(X^_e).DQ(W1_e^(G)), U_e = DQ(X^_e).DQ(W1_e^(U)), A_e = SiLU(G_e)*U_e
//            ("Activation function formulas", swiglu without clamp), then
//            A^_e, S_A,e = Q_MX(A_e) in the same FP8 type as stage 1;
//   stage 3  O_e = DQ(A^_e).DQ(W2_e);
//   stage 4  Y[i] = sum_k W[i,k] O[pi(i,k)] (+ shared expert outputs).
// Weight layout ("MXFP quantization scenario constraints"): weight1 (E, 2I, H),
// weight2 (E, H, I), every output channel a K-contiguous row; W1's first I
// channels are the gate branch, the last I the up branch; E8M0 scales per 32 along K.
//
// Both GEMMs are computed transposed, C[channel][token] = sum_k W[channel][k] X[token][k],
// with V_MFMA_SCALE_F32_16X16X128_F8F6F4: the weight rows are the MFMA A operand
// (16 channels) and the token rows the B operand (16 tokens). A small expert (decode:
// ~4 rows) then pads only to 16 tokens while the weights stream through the matrix
// core once, straight from HBM into VGPRs; each K step (128) issues the next step's
// 16-byte loads before the current MFMAs (register double buffering).
//
// Work items are (token tile, channel block) pairs over a device-built tile list
// (tiles of 16*TT rows of one group), so no host readback of the expert counts.
// GMM1 wave: 32 gate + 32 up channels x 16*TT tokens. The matching gate and up
// accumulators sit in the same lane, so SwiGLU is lane-local; the 32-channel MX
// group of the requantization is the lane's 8 values plus the 3 other lanes with
// the same token (xor 16 / xor 32), and each lane stores 4 consecutive FP8 codes.
// GMM2 wave: 64 channels x 16*TT tokens; the epilogue scales by the row's gate
// weight and accumulates into the fp32 token rows with hardware float atomics.

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

__device__ __forceinline__ int scale_arg(const uint8_t* srow, int step, int g) {
  return (int)(*reinterpret_cast<const uint32_t*>(srow + 4 * step) >> (8 * g));
}

template <int FMT, int TT>
__global__ __launch_bounds__(256) void gmm1_swiglu_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ sx, const uint8_t* __restrict__ w,
    const uint8_t* __restrict__ ws, const int4* __restrict__ tiles, const int* __restrict__ tile_count,
    int hidden, int inter, uint8_t* __restrict__ aq, uint8_t* __restrict__ sa, float* __restrict__ h1) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int ncb = inter >> 7;
  const int j = blockIdx.x / ncb, cb = blockIdx.x - j * ncb;
  if (j >= *tile_count) return;
  const int4 tile = tiles[j];
  const int e = tile.x, row0 = tile.y, nrows = tile.z;
  const int n0 = cb * 128 + wave * 32;
  const int ks = hidden >> 7, hs = hidden >> 5;

  const uint8_t* wrow[4];
  const uint8_t* wsrow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ch = (q < 2 ? n0 + 16 * q : inter + n0 + 16 * (q - 2)) + r;
    const int64_t wr = (int64_t)e * 2 * inter + ch;
    wrow[q] = w + wr * hidden;
    wsrow[q] = ws + wr * hs;
  }
  const uint8_t* xrow[TT];
  const uint8_t* xsrow[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int rr = 16 * t + r;
    const int64_t row = row0 + (rr < nrows ? rr : 0);  // padding lanes re-read a valid row
    xrow[t] = xq + row * hidden;
    xsrow[t] = sx + row * hs;
  }

  v4f acc[4][TT];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[q][t] = v4f{0.f, 0.f, 0.f, 0.f};

  v8i a_cur[4], b_cur[TT];
  int sa_cur[4], sb_cur[TT];
#pragma unroll
  for (int q = 0; q < 4; ++q) { a_cur[q] = load_mx_operand(wrow[q], g); sa_cur[q] = scale_arg(wsrow[q], 0, g); }
#pragma unroll
  for (int t = 0; t < TT; ++t) { b_cur[t] = load_mx_operand(xrow[t], g); sb_cur[t] = scale_arg(xsrow[t], 0, g); }

  for (int s = 0; s < ks; ++s) {
    v8i a_nxt[4], b_nxt[TT];
    int sa_nxt[4], sb_nxt[TT];
    const int sn = s + 1 < ks ? s + 1 : s;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a_nxt[q] = load_mx_operand(wrow[q] + 128 * sn, g);
      sa_nxt[q] = scale_arg(wsrow[q], sn, g);
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      b_nxt[t] = load_mx_operand(xrow[t] + 128 * sn, g);
      sb_nxt[t] = scale_arg(xsrow[t], sn, g);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[q][t] = mfma_mx16<FMT>(a_cur[q], b_cur[t], acc[q][t], sa_cur[q], sb_cur[t]);
#pragma unroll
    for (int q = 0; q < 4; ++q) { a_cur[q] = a_nxt[q]; sa_cur[q] = sa_nxt[q]; }
#pragma unroll
    for (int t = 0; t < TT; ++t) { b_cur[t] = b_nxt[t]; sb_cur[t] = sb_nxt[t]; }
  }

  const int is = inter >> 5;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int rr = 16 * t + r;
    const bool valid = rr < nrows;
    const int64_t row = row0 + rr;
    float act[2][4];
    int m = 0;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gv = acc[jj][t][i], uv = acc[2 + jj][t][i];
        const float a = gv / (1.0f + expf(-gv)) * uv;
        act[jj][i] = a;
        m = max(m, __float_as_int(fabsf(a)));
      }
    m = max(m, __shfl_xor(m, 16));
    m = max(m, __shfl_xor(m, 32));
    const int b = mx_scale_byte<FMT>(__int_as_float(m));
    const float inv = mx_inv_scale(b);
    if (valid) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const uint32_t codes = pack4<FMT>(act[jj][0] * inv, act[jj][1] * inv, act[jj][2] * inv, act[jj][3] * inv);
        *reinterpret_cast<uint32_t*>(aq + row * inter + n0 + 16 * jj + 4 * g) = codes;
      }
      if (g == 0) sa[row * is + (n0 >> 5)] = (uint8_t)b;
      if (h1) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ch = n0 + 16 * jj + 4 * g + i;
            h1[row * 2 * inter + ch] = acc[jj][t][i];
            h1[row * 2 * inter + inter + ch] = acc[2 + jj][t][i];
          }
      }
    }
  }
}

template <int FMT, int TT>
__global__ __launch_bounds__(256) void gmm2_combine_kernel(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ sa, const uint8_t* __restrict__ w,
    const uint8_t* __restrict__ ws, const int4* __restrict__ tiles, const int* __restrict__ tile_count,
    int hidden, int inter, const int32_t* __restrict__ row_token, const float* __restrict__ row_weight,
    float* __restrict__ y_accum, float* __restrict__ o) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int ncb = hidden / (64 * nwaves);
  const int j = blockIdx.x / ncb, cb = blockIdx.x - j * ncb;
  if (j >= *tile_count) return;
  const int4 tile = tiles[j];
  const int e = tile.x, row0 = tile.y, nrows = tile.z;
  const int c0 = (cb * nwaves + wave) * 64;
  const int ks = inter >> 7, is = inter >> 5;

  const uint8_t* wrow[4];
  const uint8_t* wsrow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t wr = (int64_t)e * hidden + c0 + 16 * q + r;
    wrow[q] = w + wr * inter;
    wsrow[q] = ws + wr * is;
  }
  const uint8_t* arow[TT];
  const uint8_t* asrow[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int rr = 16 * t + r;
    const int64_t row = row0 + (rr < nrows ? rr : 0);
    arow[t] = aq + row * inter;
    asrow[t] = sa + row * is;
  }

  v4f acc[4][TT];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[q][t] = v4f{0.f, 0.f, 0.f, 0.f};

  v8i a_cur[4], b_cur[TT];
  int sa_cur[4], sb_cur[TT];
#pragma unroll
  for (int q = 0; q < 4; ++q) { a_cur[q] = load_mx_operand(wrow[q], g); sa_cur[q] = scale_arg(wsrow[q], 0, g); }
#pragma unroll
  for (int t = 0; t < TT; ++t) { b_cur[t] = load_mx_operand(arow[t], g); sb_cur[t] = scale_arg(asrow[t], 0, g); }

  for (int s = 0; s < ks; ++s) {
    v8i a_nxt[4], b_nxt[TT];
    int sa_nxt[4], sb_nxt[TT];
    const int sn = s + 1 < ks ? s + 1 : s;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a_nxt[q] = load_mx_operand(wrow[q] + 128 * sn, g);
      sa_nxt[q] = scale_arg(wsrow[q], sn, g);
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      b_nxt[t] = load_mx_operand(arow[t] + 128 * sn, g);
      sb_nxt[t] = scale_arg(asrow[t], sn, g);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[q][t] = mfma_mx16<FMT>(a_cur[q], b_cur[t], acc[q][t], sa_cur[q], sb_cur[t]);
#pragma unroll
    for (int q = 0; q < 4; ++q) { a_cur[q] = a_nxt[q]; sa_cur[q] = sa_nxt[q]; }
#pragma unroll
    for (int t = 0; t < TT; ++t) { b_cur[t] = b_nxt[t]; sb_cur[t] = sb_nxt[t]; }
  }

#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int rr = 16 * t + r;
    if (rr >= nrows) continue;
    const int64_t row = row0 + rr;
    const int64_t tok = row_token ? (int64_t)row_token[row] : row;
    const float wgt = row_token ? row_weight[row] : 1.0f;
    float* yrow = y_accum + tok * hidden;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = c0 + 16 * q + 4 * g + i;
        unsafeAtomicAdd(yrow + ch, wgt * acc[q][t][i]);
        if (o) o[row * hidden + ch] = acc[q][t][i];
      }
  }
}

__global__ void single_group_tiles_kernel(int rows, int tm, int4* __restrict__ tiles, int* __restrict__ count) {
  const int nt = (rows + tm - 1) / tm;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nt; i += gridDim.x * blockDim.x)
    tiles[i] = make_int4(0, i * tm, min(tm, rows - i * tm), 0);
  if (blockIdx.x == 0 && threadIdx.x == 0) *count = nt;
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t n4 = n >> 2;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x)
    reinterpret_cast<float4*>(p)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
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

template <int FMT, int TT>
void gmm1_go(const Gmm1Params& p, hipStream_t st) {
  const unsigned grid = (unsigned)p.max_tiles * (unsigned)(p.inter >> 7);
  gmm1_swiglu_kernel<FMT, TT><<<grid, 256, 0, st>>>(p.xq, p.sx, p.w, p.ws, p.tiles, p.tile_count, p.hidden,
                                                    p.inter, p.aq, p.sa, p.h1);
}

template <int FMT, int TT>
void gmm2_go(const Gmm2Params& p, hipStream_t st) {
  const int nwaves = (p.hidden % 256 == 0) ? 4 : 2;
  const unsigned grid = (unsigned)p.max_tiles * (unsigned)(p.hidden / (64 * nwaves));
  gmm2_combine_kernel<FMT, TT><<<grid, 64 * nwaves, 0, st>>>(p.aq, p.sa, p.w, p.ws, p.tiles, p.tile_count,
                                                             p.hidden, p.inter, p.row_token, p.row_weight,
                                                             p.y_accum, p.o);
}

}  // namespace

hipError_t launch_gmm1(const Gmm1Params& p, hipStream_t st) {
  if (p.max_tiles <= 0) return hipSuccess;
  if (p.fmt == 0) {
    if (p.tt == 1) gmm1_go<0, 1>(p, st); else if (p.tt == 2) gmm1_go<0, 2>(p, st); else gmm1_go<0, 4>(p, st);
  } else {
    if (p.tt == 1) gmm1_go<1, 1>(p, st); else if (p.tt == 2) gmm1_go<1, 2>(p, st); else gmm1_go<1, 4>(p, st);
  }
  return hipGetLastError();
}

hipError_t launch_gmm2(const Gmm2Params& p, hipStream_t st) {
  if (p.max_tiles <= 0) return hipSuccess;
  if (p.fmt == 0) {
    if (p.tt == 1) gmm2_go<0, 1>(p, st); else if (p.tt == 2) gmm2_go<0, 2>(p, st); else gmm2_go<0, 4>(p, st);
  } else {
    if (p.tt == 1) gmm2_go<1, 1>(p, st); else if (p.tt == 2) gmm2_go<1, 2>(p, st); else gmm2_go<1, 4>(p, st);
  }
  return hipGetLastError();
}

hipError_t launch_single_group_tiles(int rows, int tm, int4* tiles, int* count, hipStream_t st) {
  single_group_tiles_kernel<<<64, 256, 0, st>>>(rows, tm, tiles, count);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t count, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count / 4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  fill_zero_kernel<<<(unsigned)blocks, 256, 0, st>>>(p, count);
  return hipGetLastError();
}

hipError_t launch_finalize(const float* acc, int64_t count, uint16_t* y, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count / 4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  finalize_kernel<<<(unsigned)blocks, 256, 0, st>>>(acc, count, y);
  return hipGetLastError();
}

}  // namespace moe
