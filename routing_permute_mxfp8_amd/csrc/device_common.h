// Device helpers shared by the routing, permute and grouped-GEMM kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
// Native 16-byte vector (HIP's uint4 is a class with a union inside and is kept in
// scratch memory by the optimizer when held in arrays across branches).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// FP8 element formats, indexed by the MFMA operand-type code (cbsz / blgp):
// 0 = FLOAT8_E4M3FN, 1 = FLOAT8_E5M2.
template <int FMT> struct Fp8;
template <> struct Fp8<0> {
  static constexpr int emax = 8;          // exponent of the largest normal (448 = 1.75 * 2^8)
  static constexpr float maxv = 448.0f;
};
template <> struct Fp8<1> {
  static constexpr int emax = 15;         // 57344 = 1.75 * 2^15
  static constexpr float maxv = 57344.0f;
};
// 2 = FLOAT4_E2M1 (MXFP4; permute output only): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
template <> struct Fp8<2> {
  static constexpr int emax = 2;          // 6 = 1.5 * 2^2
  static constexpr float maxv = 6.0f;
};

// E2M1 code (sign 0x8) of a scaled float: round to the nearest of the eight
// magnitudes, ties to the even code, saturating at 6; the sign is kept (negative
// values that round to 0 give code 0x8, as the FP8 conversions do). The comparisons
// against the midpoints 0.25, 0.75, ... are exact in fp32.
__device__ __forceinline__ uint32_t fp4_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 31) << 3;
  const float a = fabsf(y);
  uint32_t c;
  if (a <= 0.25f) c = 0;         // tie 0.25 -> 0
  else if (a < 0.75f) c = 1;     // tie 0.75 -> 2
  else if (a <= 1.25f) c = 2;    // tie 1.25 -> 2
  else if (a < 1.75f) c = 3;     // tie 1.75 -> 4
  else if (a <= 2.5f) c = 4;     // tie 2.5 -> 4
  else if (a < 3.5f) c = 5;      // tie 3.5 -> 6
  else if (a <= 5.0f) c = 6;     // tie 5 -> 6
  else c = 7;                    // 6 and above (saturated)
  return sign | c;
}

// E8M0 scale byte of an MX group (MegaMoE A8W8-FP stage 1 takes one shared exponent
// per 32 elements; the OCP MX rule gives it): clamp(floor(log2(amax)) - emax + 127, 0, 254).
// amax >= 0 and finite. For a normal float the biased exponent field is
// floor(log2) + 127, so the byte is field - emax; zero and subnormal amax give a
// negative value, clamped to 0. The upper clamp is never reached (field <= 254).
template <int FMT>
__device__ __forceinline__ int mx_scale_byte(float amax) {
  int field = (__float_as_int(amax) >> 23) & 0xff;
  int b = field - Fp8<FMT>::emax;
  return b < 0 ? 0 : b;
}

// 1 / 2^(b - 127) = 2^(127 - b) as a float (b in [0, 246] keeps it a normal float).
__device__ __forceinline__ float mx_inv_scale(int b) { return __int_as_float((254 - b) << 23); }

// Two floats (already divided by the group scale) -> two FP8 codes in the low
// (HI = false) or high (HI = true) half of `old`. Values are clamped to +-max first,
// then converted by the hardware (round to nearest even, sign kept, subnormals kept).
template <int FMT, bool HI>
__device__ __forceinline__ int cvt_pk(float a, float b, int old) {
  const float m = Fp8<FMT>::maxv;
  a = fminf(fmaxf(a, -m), m);
  b = fminf(fmaxf(b, -m), m);
  if constexpr (FMT == 0)
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
  else
    return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
}

// Four scaled floats -> one dword of FP8 codes (element 0 in the lowest byte).
template <int FMT>
__device__ __forceinline__ uint32_t pack4(float a, float b, float c, float d) {
  int w = cvt_pk<FMT, false>(a, b, 0);
  w = cvt_pk<FMT, true>(c, d, w);
  return (uint32_t)w;
}

// Max over the 4 lanes of a DPP quad (lanes 4q..4q+3) of non-negative float bits.
__device__ __forceinline__ int quad_max_bits(int v) {
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  return v;
}

// bf16 / fp16 / fp32 -> float.
__device__ __forceinline__ float bf16_to_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
// Two floats to bf16, round to nearest even, as one gfx950 V_CVT_PK_BF16_F32 (a in the
// low half); the same bits as f_to_bf16 for every finite value.
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, bf2_t));
}

__device__ __forceinline__ uint16_t f_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Block-scaled MFMA, 16x16 output, K = 128 (two FP8 operands of the same format).
// Operand lane layout (lane l, group g = l / 16, row r = l % 16), measured on gfx950:
//   register bytes 0..15  hold K [16g, 16g + 16) of row r,
//   register bytes 16..31 hold K [64 + 16g, 64 + 16g + 16),
//   scale byte 0 of lane l is the E8M0 scale of K-block g (K [32g, 32g + 32)) of row r.
// So with K-contiguous rows in memory a lane loads 16 bytes at 16g and 16 bytes at
// 64 + 16g of each 128-wide K step, and the scale dword of the step shifted right by 8g.
// Output: lane l holds C[4g + i][r] for i = 0..3 (A rows = C rows, B rows = C columns).
template <int FMT>
__device__ __forceinline__ v4f mfma_mx16(const v8i& a, const v8i& b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT, FMT, 0, sa, 0, sb);
}

// Operand format codes of the block-scaled MFMA: 0 FP8 E4M3FN, 1 FP8 E5M2, 4 FP4 E2M1.
// An FP4 operand (measured on gfx950) uses register bytes 0..15 only: lane l holds
// K [32g, 32g + 32) of row r, element 2j in the low nibble of byte j, i.e. the 16
// bytes at byte offset 16g of the row's packed K step; the scale byte is as for FP8.
constexpr int kFmtFp4 = 4;

template <int FA, int FB>
__device__ __forceinline__ v4f mfma_mx16_ab(const v8i& a, const v8i& b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, sa, 0, sb);
}

__device__ __forceinline__ v8i join_operand(u32x4 lo, u32x4 hi) {
  v8i r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  return r;
}

__device__ __forceinline__ v8i load_mx_operand(const uint8_t* row_k0, int g) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(row_k0 + 16 * g);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(row_k0 + 64 + 16 * g);
  return join_operand(lo, hi);
}

// ---- tiled token layout ------------------------------------------------------------
// An FP8 matrix of R rows (R a multiple of 16) and K columns (K a multiple of 128) in
// the operand order of the MFMA above: 16-row x 128-K tiles of 2 KB,
//   codes  [R/16][K/128][2 halves][64 lanes][16 B]: lane l = (g, r) of half h holds
//          row 16T + r, K bytes [128 s + 64 h + 16 g, +16),
//   scales [R/16][ceil(K/512)][64 lanes][4 B]: byte j of lane (g, r) in quad q is the
//          E8M0 scale of row 16T + r, K-block g of step 4q + j (0 past the last step).
// Rows of one expert start at a multiple of 16 (each expert is padded to whole tiles).
__device__ __forceinline__ int64_t t16_codes(int64_t tile, int ks, int step) {
  return ((tile * ks + step) * 2) * 1024;
}
__device__ __forceinline__ int64_t t16_scales(int64_t tile, int kq, int quad) { return (tile * kq + quad) * 256; }

}  // namespace moe
