// Device helpers of the grouped GEMMs (gmm.hip, gmm_stream.hip): weight operand
// addressing, direct-to-LDS loads, waits and barriers, the persistent XCD-aware item
// split, the activations of MegaMoE's "Activation function formulas" and the MX
// requantization store of GMM1's epilogue, and the persistent launch shape.
#pragma once

#include <map>
#include <mutex>

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kXcds = 8;
constexpr int kTileBytes = 2048;   // one 16-row x 128-K MX operand tile
constexpr int kTileScaleBytes = 256;

// ---- weight operand loads --------------------------------------------------------
// WF: the weights' MFMA operand format, the tokens' FP8 format or kFmtFp4 (MXFP4 E2M1,
// two codes a byte: a 16-channel x 128-K tile is 1 KB, one 16-byte load per lane).
template <int WF>
struct WeightFmt {
  static constexpr bool kFp4 = WF == kFmtFp4;
  static constexpr int kStepBytes = kFp4 ? 1024 : 2048;   // one 16-channel x 128-K tile
  static constexpr int kParts = kFp4 ? 2 : 3;             // loads per tile and K step (data..., scale)
};

// ND: row pointer of channel (tile*16 + r) and its scale row.
// PACKED: tile base (group, 16-channel tile, K step 0) and its scale base + lane*4.
template <bool PACKED>
struct WPtr {
  const uint8_t* d;
  const uint8_t* s;
};

template <bool PACKED, int WF>
__device__ __forceinline__ WPtr<PACKED> weight_tile(const uint8_t* w, const uint8_t* ws, int64_t tile_index, int K,
                                                    int lane) {
  // tile_index = group * (N / 16) + channel_tile
  WPtr<PACKED> p;
  const int ks = K >> 7;
  if constexpr (PACKED) {
    const int kq = (ks + 3) >> 2;
    p.d = w + tile_index * ks * WeightFmt<WF>::kStepBytes;
    p.s = ws + tile_index * kq * kTileScaleBytes + lane * 4;
  } else {
    const int64_t row = tile_index * 16 + (lane & 15);
    p.d = w + row * (WeightFmt<WF>::kFp4 ? K >> 1 : K);
    p.s = ws + row * (K >> 5);
  }
  return p;
}

// The byte of a raw weight scale dword that the MFMA uses in K step `step` (the shift
// is done where the MFMA needs it, so no ALU work waits on a load before its data is
// due).
template <bool PACKED>
__device__ __forceinline__ int weight_scale(int sc_raw, int step, int lane) {
  if constexpr (PACKED)
    return (int)((uint32_t)sc_raw >> (8 * (step & 3)));
  else
    return (int)((uint32_t)sc_raw >> (8 * (lane >> 4)));
}

// ---- token staging ------------------------------------------------------------------
// The token rows of a chunk go straight from HBM/L2 to LDS (global_load_lds: lane l of
// a wave writes LDS base + 16 l, so a 1 KB half tile of the tiled layout lands as is)
// into a ring of 3 slots, two K steps ahead of their use. A slot holds NT tiles x
// {2 KB operand bytes, 256 B scale dwords (the raw dwords of the tiled layout: byte
// step % 4 of lane l is the lane's E8M0 scale of that step)}.
template <int NT>
struct StageLayout {
  static constexpr int kBufBytes = NT * (kTileBytes + kTileScaleBytes);
  static constexpr int kPerWave = (NT + 3) / 4;   // tiles loaded by each of 4 waves
};
constexpr int kRing = 3;

typedef __attribute__((address_space(3))) void* lds_void_ptr;

__device__ __forceinline__ void lds_dma16(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)dst, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)dst, 4, 0, 0);
}

// Operand and scale byte of token tile t of a slot for K step `step`.
template <int NT>
__device__ __forceinline__ void stage_read(const uint8_t* buf, int t, int step, int lane, v8i& v, int& sc) {
  const uint8_t* tile = buf + t * kTileBytes;
  v = join_operand(reinterpret_cast<const u32x4*>(tile)[lane], reinterpret_cast<const u32x4*>(tile + 1024)[lane]);
  sc = buf[NT * kTileBytes + t * kTileScaleBytes + 4 * lane + (step & 3)];
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Persistent, XCD-aware item range of this block: [*lo, *hi) stepping by *stride.
__device__ __forceinline__ void block_items(int total, int* first, int* stride, int* last) {
  const int nb = gridDim.x;
  const int xcd = blockIdx.x % kXcds;
  const int per = nb / kXcds;
  const int lo = (int)(((int64_t)total * xcd) / kXcds);
  const int hi = (int)(((int64_t)total * (xcd + 1)) / kXcds);
  *first = lo + blockIdx.x / kXcds;
  *stride = per;
  *last = hi;
}

// Workgroup barrier at the top of a K step. __syncthreads fences global memory, which
// waits for every outstanding load, the prefetches of later steps included; the waits
// this barrier must cover (every wave's DMA writes of the step's token tiles) are the
// explicit vmcnt wait before it, so chunks of 4 or more tiles use the bare s_barrier
// (scheduling fences keep the LDS accesses on their side of it). For 1- and 2-tile
// chunks the fenced barrier measured faster.
template <int NT>
__device__ __forceinline__ void block_barrier() {
  if constexpr (NT >= 4) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  } else {
    __syncthreads();
  }
}

// ---- activations (MegaMoE README, "Activation function formulas") ------------------
// sigma(z) = 1 / (1 + e^-z); SiLU(z) = z sigma(z); with the clamp c (+inf when none),
// Gc = min(G, c), Uc = clip(U, -c, c).
//
// e^x and 1/x by the hardware's V_EXP_F32 (2^(x log2 e)) and V_RCP_F32: a few ulp where
// the library's expf and an IEEE division take ten or more instructions each. A is
// requantized to FP8 right after (a step of 2^-4 of its group's scale), and its
// products carry the GEMM's own error (up to 2^-12 of their magnitudes), so the
// difference does not show. e^x overflows to +inf and underflows to 0 as expf does;
// 1/inf = 0.
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float sigmoid(float z) { return rcp_hw(1.0f + exp_hw(-z)); }

// swiglu: SiLU(Gc) Uc.
__device__ __forceinline__ float swiglu_act(float g, float u, float c) {
  const float gc = fminf(g, c), uc = fminf(fmaxf(u, -c), c);
  return gc * sigmoid(gc) * uc;
}

// tanh without branches: 1 - 2 / (e^(2|x|) + 1) with the sign of x (e^(2|x|) = inf gives
// 1 exactly; e^x and 1/x as above), and for |x| < 0.05, where that difference cancels, the series
// x (1 - x^2/3 + 2 x^4/15) (next term below 1e-10 relative there). The library tanhf
// branches, and a branch in the epilogue of the 240-accumulator GEMM costs it its
// register allocation.
__device__ __forceinline__ float tanh_nb(float x) {
  const float a = fabsf(x);
  const float big = 1.0f - 2.0f * rcp_hw(exp_hw(2.0f * a) + 1.0f);
  const float x2 = x * x;
  const float small = a * (1.0f - x2 * (1.0f / 3.0f) + x2 * x2 * (2.0f / 15.0f));
  return copysignf(a < 0.05f ? small : big, x);
}

// The gated activations of one (gate, up) pair; KIND = ActParams::kind (0-3).
// GMM1's epilogue is a template parameter (EPI = the activation kind), so that each
// kernel holds only its own activation code: with several behind a run-time switch
// the 256-row kernel runs out of registers and spills accumulators in its K loop.
template <int KIND>
__device__ __forceinline__ float gated_act(float g, float u, const ActParams& p) {
  if constexpr (KIND == 1) {  // swiglustep: min(SiLU(G), c) Uc
    const float uc = fminf(fmaxf(u, -p.clamp), p.clamp);
    return fminf(g * sigmoid(g), p.clamp) * uc;
  } else if constexpr (KIND == 2) {  // swigluoai: Gc sigma(alpha Gc) (Uc + beta)
    const float gc = fminf(g, p.clamp), uc = fminf(fmaxf(u, -p.clamp), p.clamp);
    return gc * sigmoid(p.alpha * gc) * (uc + p.beta);
  } else if constexpr (KIND == 3) {  // situglu: beta tanh(G / beta) sigma(G) L(U) (no clamp)
    // both forms of L computed and selected (no branch on linear_beta: a branch in the
    // epilogue of the 240-accumulator GEMM costs it its register allocation)
    const bool lin = p.lin_beta > 0.0f;
    const float lb = lin ? p.lin_beta : 1.0f;
    const float l = lin ? lb * tanh_nb(u / lb) : u;
    return p.beta * tanh_nb(g / p.beta) * sigmoid(g) * l;
  } else if constexpr (KIND == kActSwigluNoClamp) {   // swiglu with c = +inf: SiLU(G) U
    return g * sigmoid(g) * u;
  } else {
    return swiglu_act(g, u, p.clamp);
  }
}

// gelu (tanh form), element-wise on every GMM1 output channel: Z sigma(sqrt(8/pi)(Z + 0.044715 Z^3)).
__device__ __forceinline__ float gelu_act(float z) {
  constexpr float kSqrt8OverPi = 1.5957691216057308f;
  return z * sigmoid(kSqrt8OverPi * (z + 0.044715f * z * z * z));
}

// Maximum of m over the lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four 16-lane rows of the
// wave), for non-negative m. The gfx950 row-swap moves do it in the vector ALU: no LDS
// round trip and no lane-index address register (a register the epilogues cannot spare).
__device__ __forceinline__ int max_over_rows(int m) {
  // swap odd rows of one copy with even rows of the other: the pair holds rows (0,1) and (2,3)
  const auto a = __builtin_amdgcn_permlane16_swap((unsigned)m, (unsigned)m, false, false);
  m = max((int)a[0], (int)a[1]);
  // swap the upper half of one copy with the lower half of the other: halves (0,1)
  const auto b = __builtin_amdgcn_permlane32_swap((unsigned)m, (unsigned)m, false, false);
  return max((int)b[0], (int)b[1]);
}

// MX-quantize one 32-channel group held as 8 values per lane by the lanes of one 16-lane
// row (lane groups g = 0..3, xor 16 / 32), and store it into the tiled A layout at K step
// `step`, half `half` of the step, lane groups 2 * sub + jj: act[jj][i] is channel
// 16 jj + 4 g + i of the group.
template <int FMT>
__device__ __forceinline__ void store_group(const float (&act)[2][4], uint8_t* __restrict__ aq,
                                            uint8_t* __restrict__ sa, int64_t tl, int ks2, int kq2, int step,
                                            int cw, int g, int r) {
  int m = 0;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, __float_as_int(fabsf(act[jj][i])));
  m = max_over_rows(m);
  const int b = mx_scale_byte<FMT>(__int_as_float(m));
  const float inv = mx_inv_scale(b);
  uint8_t* ob = aq + t16_codes(tl, ks2, step) + (cw >> 1) * 1024;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const uint32_t codes = pack4<FMT>(act[jj][0] * inv, act[jj][1] * inv, act[jj][2] * inv, act[jj][3] * inv);
    *reinterpret_cast<uint32_t*>(ob + ((2 * (cw & 1) + jj) * 16 + r) * 16 + 4 * g) = codes;
  }
  if (g == 0) sa[t16_scales(tl, kq2, step >> 2) + (cw * 16 + r) * 4 + (step & 3)] = (uint8_t)b;
}

// ---- launch helpers: persistent grid = CUs x resident blocks per CU (multiple of 8) --
struct LaunchShape {
  int grid = 0;
  size_t lds = 0;
};

template <typename K>
hipError_t persistent_shape(K kernel, size_t lds, LaunchShape* out) {
  static std::mutex mu;
  static std::map<const void*, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  const void* key = reinterpret_cast<const void*>(kernel);
  auto itc = cache.find(key);
  int grid;
  if (itc == cache.end()) {
    hipError_t e = hipFuncSetAttribute(key, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    int dev = 0, cus = 0, per_cu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, lds)) != hipSuccess) return e;
    if (per_cu < 1) per_cu = 1;
    grid = cus * per_cu;
    grid = ((grid + kXcds - 1) / kXcds) * kXcds;
    cache[key] = grid;
  } else {
    grid = itc->second;
  }
  out->grid = grid;
  out->lds = lds;
  return hipSuccess;
}

}  // namespace
}  // namespace moe
