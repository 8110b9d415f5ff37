// Grouped GEMMs of the MX expert FFN for layers whose experts hold many rows: the
// weight stream goes HBM -> LDS several K steps ahead of its use.
//
// MegaMoE README, "A8W8-FP quantization scenario" (and "A8W4-FP"):
//   stage 2  G_e = DQ(X^_e).DQ(W1_e^(G)), U_e = DQ(X^_e).DQ(W1_e^(U)), A_e = act(G_e, U_e),
//            A^_e, S_A,e = Q_MX(A_e) with the FP8 type of stage 1;
//   stage 3  O_e = DQ(A^_e).DQ(W2_e).
// Weights as in "MXFP quantization scenario constraints": weight1 (E, 2I, H) with the gate
// branch in the first I output channels and the up branch in the last I, weight2 (E, H, I),
// K-contiguous rows, one E8M0 scale per 32 (ND layout or the library's packed layout).
//
// Why a second kernel: when an expert has a few hundred rows the GEMM reads each weight
// byte once and does ~2 * rows flops with it, below the MI355X ridge (~625 flop/B), so it
// is bound by the weight stream. Streaming the weights into registers (gmm.hip) leaves
// room for one K step of prefetch next to hundreds of accumulators, and each step then
// waits one loaded-HBM round trip. Here the weights go into a ring of LDS slots by
// direct-to-LDS loads issued kLead steps ahead, continuously across work items, and
// the register file holds the accumulators and the (L2-resident) token operands.
//
// Work item = (chunk of up to 4 * kRT 16-row token tiles of one expert, channel block of
// kCB 16-channel weight tiles). GMM1: 6 gate tiles and the 6 matching up tiles (96 gate
// channels, so the activation is lane-local); GMM2: 12 consecutive output tiles. A block
// is 4 waves, one per SIMD, persistent, XCD-aware (the channel blocks of one chunk run
// at the same time on one XCD and share its L2 for the token tiles). Wave w owns the
// chunk's token tiles w, w + 4, w + 8, ... (up to kRT), loads them into registers three
// K steps ahead, and multiplies them with all kCB weight tiles of the step read from LDS
// (V_MFMA_SCALE_F32_16X16X128_F8F6F4, weights in the A slot: a lane holds 4 consecutive
// channels of one token row). A wave runs the MFMAs of RT tiles every step whether or
// not the chunk has them (tiles past its end load zeros, their results are not
// stored): the chunk-size classes (RT = 2, 4, 5) keep that close to the chunk's own
// tiles, so a chunk of a few rows costs little more than its weight stream.
//
// Per K step and wave: one fixed vmcnt wait (this step's weight slot, landed by every
// wave's own loads) and one barrier (every wave's loads have landed; every wave is done
// with the slot about to be refilled) -- with six LDS slots (kLead + 2, where they fit)
// the wait and the barrier come every second step and cover two steps' slots (the
// waves then drift apart by up to a step between barriers); then the token loads of step + 3 and this wave's
// share of the weight loads of step + kLead (always the same number of each, so the
// wait count is a constant: loads past the last step read valid addresses again, and
// those of token tiles past the chunk's end fall outside the chunk's buffer resource,
// whose range check returns zeros without touching memory); then the MFMAs. The epilogue of an item (activation and
// requantization, or the O rows) runs after its last K step, while the next item's loads
// are in flight. The item descriptions live in scalar registers, read through the scalar
// cache an item ahead: an LDS read in the K loop would have to wait for every
// direct-to-LDS load in flight (the compiler cannot tell which bytes those loads write),
// draining the pipeline each step.

#include <algorithm>
#include <climits>

#include "device_common.h"
#include "gmm_device.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kCB = 12;         // 16-channel weight tiles per channel block (192 channels)
constexpr int kRT = 5;          // most token tiles per wave: a chunk holds up to 20 tiles (320 rows)
constexpr int kLead = 4;        // weight loads run kLead steps ahead
constexpr int kTokLead = 3;     // token loads run three steps ahead (four register sets)

// LDS: kSlots weight code slots (one K step of the channel block each), then two scale
// groups (the E8M0 scales of four K steps: the block's weight tiles, then the chunk's
// token tiles), loaded once per four steps.
template <int WF, bool PACKED>
struct StreamW {
  static constexpr bool kFp4 = WF == kFmtFp4;
  static constexpr int kCode = kFp4 ? 1024 : 2048;   // bytes of one 16-channel x 128-K tile
  static constexpr int kHalves = kFp4 ? 1 : 2;       // 1 KB loads per tile
  static constexpr int kSlotBytes = kCB * kCode;
  // a weight tile's scales of four steps: the packed layout's 256-byte block (lane l's
  // dword, byte s = step s), or 16 ND bytes per lane (row l % 16, byte 4 s + b = block b
  // of step s; the four lanes of a row load the same bytes)
  static constexpr int kWsTile = PACKED ? kTileScaleBytes : 1024;
  static constexpr int kTsOff = kCB * kWsTile;       // token scales in a group
  static constexpr int kGroupBytes = kTsOff + 4 * kRT * kTileScaleBytes;
  // weight slots: kLead + 2 where they fit in LDS (the barrier every second step), else
  // kLead + 1 (a barrier every step)
  static constexpr int kSlots = 6 * kSlotBytes + 2 * kGroupBytes <= 160 * 1024 ? 6 : 5;
  static constexpr int kGroups = kSlots * kSlotBytes;   // offset of the two scale groups
  static constexpr int kLds = kGroups + 2 * kGroupBytes;
  static constexpr int kDma = (kCB / 4) * kHalves;   // weight code loads per wave and step
  // Step h issues T(h + 3) (2 RT ops) before its MFMAs, W(h + 4) (kDma ops) between
  // two of its MFMA groups, and, when h = 0 mod 4, the scale group S of steps h + 4 ..
  // h + 7 after a later group. The prologue is steps -4..-1 of the same pattern (S0, W0,
  // T0 W1, T1 W2, T2 W3). At the top of step g the weight codes W(g) and the scales of
  // step g (both issued in step g - 4 or earlier) must have landed; the ops issued after
  // them are at least three whole steps' worth without scale loads, so vmcnt(kWait)
  // covers both from step 0 on (vector memory loads complete in order). The compiler's
  // own wait for the token registers of step g comes after that.
  // (kTokLoads = 2 RT per wave and step: lo and hi half of each of its RT token tiles)
  template <int RT>
  static constexpr int kWait = 3 * (kDma + 2 * RT);
  // With six slots the wait at the top of an even step g also covers W(g + 1), issued in
  // step g - 3: the ops after it are at least two whole steps' worth (the scales of
  // steps g and g + 1 belong to one group, issued in step g - 4 or earlier).
  template <int RT>
  static constexpr int kWaitPair = 2 * (kDma + 2 * RT);
  static_assert(kWait<kRT> <= 63, "vmcnt holds at most 63");
  static_assert(kLds <= 160 * 1024, "LDS per workgroup");
};

struct StreamArgs {
  const uint8_t* tok;           // tiled token codes [padded rows, K]
  const uint8_t* toks;          // tiled token scales
  const uint8_t* w;             // weights [G, N, K] (ND or packed)
  const uint8_t* ws;            // weight scales
  const int4* tiles;            // chunks {group, padded row0, rows, sorted row0}
  const int* tile_count;
  int K;                        // contraction: hidden (GMM1) or A's width (GMM2)
  int N;                        // output channels: 2I (GMM1) or hidden (GMM2)
  int inter;                    // GMM1: I
  uint8_t* aq;                  // GMM1: tiled A^ codes [padded rows, A width]
  uint8_t* sa;                  // GMM1: tiled A^ scales
  float* h1;                    // GMM1: optional fp32 [rows, 2I] (sorted rows)
  ActParams act;
  float* o;                     // GMM2: fp32 O rows [rows, N] (sorted rows), or
  uint16_t* o16;                // GMM2: bf16 O rows
  // A shared expert folded into the launch: group sh_first (INT_MAX: none) takes its
  // weights from w + sh_first N K + sh_wdelta (codes) and the matching scales address +
  // sh_sdelta, i.e. from the shared expert's own weights; its rows live in the same token,
  // A^ and O buffers as the routed experts' (after theirs).
  int sh_first;
  int64_t sh_wdelta, sh_sdelta;
};



// The item's weight tile q (0..kCB-1) of channel block cb, clamped into the expert (the
// tiles of a partial last block repeat the last one; their results are not stored).
template <int GMM>
__device__ __forceinline__ int block_tile(int cb, int q, int n16, int i16) {
  if constexpr (GMM == 1) {
    const int h = q < kCB / 2 ? q : q - kCB / 2;
    const int gt = min(cb * (kCB / 2) + h, i16 - 1);
    return q < kCB / 2 ? gt : i16 + gt;
  } else {
    return min(cb * kCB + q, n16 - 1);
  }
}

// Buffer descriptor word 3 for raw (untyped) buffer loads on CDNA.
constexpr int kRsrcWord3 = 0x00020000;
// Cache-policy operand of a buffer load: non-temporal (the weight codes are streamed once
// per chunk; a plain streaming read measured ~6.3 TB/s, a non-temporal one ~7.1 TB/s).
constexpr int kNonTemporal = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// A work item: the chunk's expert, first padded row, rows and first sorted row (one entry
// of the chunk list), and the channel block.
struct Item {
  int e, row0, nrows, srow0, cb;
};

typedef __attribute__((address_space(4))) const int const_int;

// Item `it` of the flattened (chunk, channel block) list. The chunk list is read-only in
// this kernel and the index is wave-uniform, so the loads go through the scalar cache:
// they count on the LDS/scalar counter, not on the vector memory counter that the K
// loop's explicit waits count the pipeline's own loads on.
__device__ __forceinline__ Item load_item(const int4* tiles, int it, int ncb) {
  const int jc = it / ncb;
  const const_int* q = (const const_int*)(tiles + jc);
  return Item{q[0], q[1], q[2], q[3], it - jc * ncb};
}

// A stream `lead` steps ahead of compute step kc of the current item: the current item's
// step kc + lead while that is below ks, else the next item's step kc + lead - ks. Past
// the block's last item it stays on that item's last step (the next item is then the
// current one), so every step issues the same loads. Selects, no branches: a branch per
// stream and step cuts the K loop into blocks the scheduler handles badly.
struct Ahead {
  Item d;
  int k;
};

__device__ __forceinline__ Ahead ahead(const Item& cur, const Item& nxt, bool last, int kc, int lead, int ks) {
  const int k = kc + lead;
  const bool wrap = k >= ks;
  Ahead a;
  a.d.e = wrap ? nxt.e : cur.e;
  a.d.row0 = wrap ? nxt.row0 : cur.row0;
  a.d.nrows = wrap ? nxt.nrows : cur.nrows;
  a.d.srow0 = wrap ? nxt.srow0 : cur.srow0;
  a.d.cb = wrap ? nxt.cb : cur.cb;
  a.k = wrap ? (last ? ks - 1 : k - ks) : k;
  return a;
}

// Token tiles of wave `wave` in a chunk of nrows rows: tiles wave, wave + 4, ... < ntt.
__device__ __forceinline__ int wave_tiles(int nrows, int wave) {
  const int ntt = (nrows + 15) >> 4;
  return ntt > wave ? (ntt - wave + 3) >> 2 : 0;
}

// Per-lane byte offsets of the loads (the same for every tile and step): the lane's 16
// code bytes and its 4 scale bytes of a tile, in the packed layouts (weights and tokens)
// or in the ND weight rows (row l % 16 of the tile).
struct LaneOffsets {
  int code, scale;              // tiled / packed layouts
  int wcode, wscale;            // weights (ND: row-major rows)
};

template <bool PACKED, int WF>
__device__ __forceinline__ LaneOffsets lane_offsets(int K, int lane) {
  LaneOffsets o;
  o.code = 16 * lane;
  o.scale = 4 * lane;
  const int g = lane >> 4, r = lane & 15;
  if constexpr (PACKED) {
    o.wcode = o.code;
    o.wscale = o.scale;
  } else {
    o.wcode = r * (WF == kFmtFp4 ? K >> 1 : K) + 16 * g;
    o.wscale = r * (K >> 5);
  }
  return o;
}

// The weight loads of step k of item c: buffer descriptors of expert c.e's codes and
// scales (direct-to-LDS loads through them stay inside that expert's weights).
struct WeightStep {
  __amdgpu_buffer_rsrc_t wr, sr;
  int cb, k;
};

template <int WF, bool PACKED>
__device__ __forceinline__ WeightStep weight_step(const StreamArgs& p, const Item& c, int k, int n16) {
  using SW = StreamW<WF, PACKED>;
  const int K = p.K, kq = ((K >> 7) + 3) >> 2;
  const int64_t cbytes = (int64_t)p.N * (SW::kFp4 ? K >> 1 : K);
  const int64_t sbytes = PACKED ? (int64_t)n16 * kq * kTileScaleBytes : (int64_t)p.N * (K >> 5);
  // the shared expert's weights by an added offset, not a select of two pointers (the
  // compiler turns that into a branch, which cuts the K loop into blocks)
  const int64_t m = -(int64_t)(c.e == p.sh_first);
  return WeightStep{rsrc(p.w + c.e * cbytes + (p.sh_wdelta & m), cbytes),
                    rsrc(p.ws + c.e * sbytes + (p.sh_sdelta & m), sbytes), c.cb, k};
}

// This wave's i-th weight tile of a step (tile wave + 4 i of the channel block): its code
// halves into `slot`.
template <int GMM, bool PACKED, int WF>
__device__ __forceinline__ void issue_weight_tile(const WeightStep& L, int i, uint8_t* slot, int K, int n16, int i16,
                                                  const LaneOffsets& lo, int wave) {
  using SW = StreamW<WF, PACKED>;
  const int ks = K >> 7;
  const int q = wave + 4 * i;
  const int tile = block_tile<GMM>(L.cb, q, n16, i16);
#pragma unroll
  for (int h = 0; h < SW::kHalves; ++h) {
    int so;
    if constexpr (PACKED)
      so = (tile * ks + L.k) * SW::kCode + h * 1024;
    else if constexpr (SW::kFp4)
      so = tile * 16 * (K >> 1) + 64 * L.k;
    else
      so = tile * 16 * K + 128 * L.k + 64 * h;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(L.wr, (lds_void_ptr)(slot + q * SW::kCode + h * 1024), 16, lo.wcode, so,
                                             0, kNonTemporal);
  }
}

// All of this wave's weight code loads of step k of item c into `slot`.
template <int GMM, bool PACKED, int WF>
__device__ __forceinline__ void issue_weights(const StreamArgs& p, const Item& c, int k, uint8_t* slot, int n16,
                                              int i16, const LaneOffsets& lo, int wave) {
  const WeightStep L = weight_step<WF, PACKED>(p, c, k, n16);
#pragma unroll
  for (int i = 0; i < kCB / 4; ++i) issue_weight_tile<GMM, PACKED, WF>(L, i, slot, p.K, n16, i16, lo, wave);
}

// The token loads of step k of item c: descriptors of exactly the chunk's tiles (a wave's
// tiles past the chunk's end are addressed one past its last tile: the range check
// returns zero codes and scales for them, measured on gfx950 for register and
// direct-to-LDS buffer loads, with no memory traffic; zero operands also draw less power).
struct TokenStep {
  __amdgpu_buffer_rsrc_t tr, sr;
  int ntt, k;
};

__device__ __forceinline__ TokenStep token_step(const StreamArgs& p, const Item& c, int k, int ks, int kq) {
  const int ntt = (c.nrows + 15) >> 4;
  const int64_t tile0 = c.row0 >> 4;
  return TokenStep{rsrc(p.tok + tile0 * ks * 2048, (int64_t)ntt * ks * 2048),
                   rsrc(p.toks + tile0 * kq * kTileScaleBytes, (int64_t)ntt * kq * kTileScaleBytes), ntt, k};
}

__device__ __forceinline__ int wave_tile(const TokenStep& L, int j, int wave) {
  return 4 * j + wave < L.ntt ? 4 * j + wave : L.ntt;
}

// This wave's j-th token tile of a step (chunk tile 4 j + wave): its codes into registers.
__device__ __forceinline__ void issue_token_tile(const TokenStep& L, int j, int ks, int wave, const LaneOffsets& lo,
                                                 v8i& t) {
  const int so = (wave_tile(L, j, wave) * ks + L.k) * 2048;
  const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(L.tr, lo.code, so, 0);
  const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(L.tr, lo.code, so + 1024, 0);
  t = join_operand(a, b);
}

// All of this wave's token tiles of step k of item c.
template <int RT>
__device__ __forceinline__ void issue_tokens(const StreamArgs& p, const Item& c, int k, int ks, int kq, int wave,
                                             const LaneOffsets& lo, v8i (&t)[RT]) {
  const TokenStep L = token_step(p, c, k, ks, kq);
#pragma unroll
  for (int j = 0; j < RT; ++j) issue_token_tile(L, j, ks, wave, lo, t[j]);
}

// This wave's share of the scale group of steps k .. k + 3 of item c (k = 0 mod 4) into
// `group`: the scales of its weight tiles wave + 4 i and of its token tiles 4 j + wave.
template <int GMM, bool PACKED, int WF, int RT>
__device__ __forceinline__ void issue_scales(const StreamArgs& p, const Item& c, int k, uint8_t* group, int ks, int kq,
                                             int n16, int i16, const LaneOffsets& lo, int wave) {
  using SW = StreamW<WF, PACKED>;
  const WeightStep W = weight_step<WF, PACKED>(p, c, k, n16);
  const TokenStep T = token_step(p, c, k, ks, kq);
  const int K = p.K, g4 = k >> 2;
#pragma unroll
  for (int i = 0; i < kCB / 4; ++i) {
    const int q = wave + 4 * i;
    const int tile = block_tile<GMM>(c.cb, q, n16, i16);
    const int so = PACKED ? (tile * kq + g4) * kTileScaleBytes : tile * 16 * (K >> 5) + 16 * g4;
    if constexpr (PACKED)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(W.sr, (lds_void_ptr)(group + q * SW::kWsTile), 4, lo.wscale, so, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(W.sr, (lds_void_ptr)(group + q * SW::kWsTile), 16, lo.wscale, so, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < RT; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(T.sr, (lds_void_ptr)(group + SW::kTsOff + (4 * j + wave) * kTileScaleBytes),
                                             4, lo.scale, (wave_tile(T, j, wave) * kq + g4) * kTileScaleBytes, 0, 0);
}

// MFMAs of one K step for the wave's first NW token tiles: for each weight tile q (read
// from the LDS slot, the next one's read issued before this one's MFMAs), NW MFMAs, then
// between(q): the loads of later steps go out in small groups between the MFMA groups, so
// that a wave whose loads wait for room in the memory pipeline still keeps its matrix
// core busy. The E8M0 scales come from the step's scale group (byte k % 4 of a packed or
// token dword; byte lane / 16 of the ND dword of step k % 4). ZERO_C: the MFMAs take a
// zero C operand (an item's first step) instead of the accumulators.
template <int FMT, bool PACKED, int WF, int NW, bool ZERO_C, class Between>
__device__ __forceinline__ void step_mfma(v4f (&acc)[kCB][NW], const uint8_t* slot, const uint8_t* group, int k,
                                          int lane, int wave, const v8i (&t)[NW], Between&& between) {
  using SW = StreamW<WF, PACKED>;
  const int sh = 8 * (k & 3);
  int tsc[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j)
    tsc[j] = (int)((uint32_t)reinterpret_cast<const int*>(group + SW::kTsOff + (4 * j + wave) * kTileScaleBytes)[lane] >>
                   sh);
  v8i a[2];
  int sa[2];
  auto read = [&](int q, v8i& v, int& s) {
    const uint8_t* tile = slot + q * SW::kCode;
    if constexpr (SW::kFp4) {
      const u32x4 lo = reinterpret_cast<const u32x4*>(tile)[lane];
      v = join_operand(lo, lo);   // an FP4 operand uses register bytes 0..15 only
    } else {
      v = join_operand(reinterpret_cast<const u32x4*>(tile)[lane], reinterpret_cast<const u32x4*>(tile + 1024)[lane]);
    }
    if constexpr (PACKED)
      s = (int)((uint32_t)reinterpret_cast<const int*>(group + q * SW::kWsTile)[lane] >> sh);
    else
      s = (int)((uint32_t)reinterpret_cast<const int*>(group + q * SW::kWsTile)[4 * lane + (k & 3)] >> (8 * (lane >> 4)));
  };
  read(0, a[0], sa[0]);
#pragma unroll
  for (int q = 0; q < kCB; ++q) {
    if (q + 1 < kCB) read(q + 1, a[(q + 1) & 1], sa[(q + 1) & 1]);
#pragma unroll
    for (int j = 0; j < NW; ++j)
      acc[q][j] = mfma_mx16_ab<WF, FMT>(a[q & 1], t[j], ZERO_C ? v4f{0.f, 0.f, 0.f, 0.f} : acc[q][j], sa[q & 1], tsc[j]);
    between(q);
    __builtin_amdgcn_sched_barrier(0);   // keep the weight tile reads one tile ahead, not all hoisted
  }
}

// MX-quantize one 32-channel group (act[jj][i] = channel c + 16 jj + 4 g + i of row r of
// token tile tl, c a multiple of 32) and store it into the tiled A layout (K = A's width,
// ks2 K steps).
template <int FMT>
__device__ __forceinline__ void store_a_group(const float (&act)[2][4], uint8_t* __restrict__ aq,
                                              uint8_t* __restrict__ sa, int64_t tl, int ks2, int c, int g, int r) {
  int m = 0;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, __float_as_int(fabsf(act[jj][i])));
  m = max_over_rows(m);
  const int b = mx_scale_byte<FMT>(__int_as_float(m));
  const float inv = mx_inv_scale(b);
  const int s2 = c >> 7, half = (c >> 6) & 1, sub = (c >> 4) & 3;
  uint8_t* ob = aq + t16_codes(tl, ks2, s2) + half * 1024;
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const uint32_t codes = pack4<FMT>(act[jj][0] * inv, act[jj][1] * inv, act[jj][2] * inv, act[jj][3] * inv);
    *reinterpret_cast<uint32_t*>(ob + ((sub + jj) * 16 + r) * 16 + 4 * g) = codes;
  }
  if (g == 0) sa[t16_scales(tl, (ks2 + 3) >> 2, s2 >> 2) + (((c >> 5) & 3) * 16 + r) * 4 + (s2 & 3)] = (uint8_t)b;
}

// GMM1 epilogue of an item: acc[q][j][i] = H1[row 16 t + r][channel 4 g + i of tile q]
// for the wave's token tile t = 4 j + wave; tiles 0..5 gate, 6..11 the matching up tiles.
// The lane index, computed afresh for the epilogue by an asm the compiler cannot merge with
// the K loop's copy. Values the epilogue derives from it (store offsets) are then computed
// in the epilogue rather than hoisted out of the item loop, and the loop's own copy need
// not survive into the epilogue: a spilled copy would have to be reloaded there, and the
// wait for that reload would also wait for every load the pipeline has in flight.
__device__ __forceinline__ int epilogue_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

template <int FMT, int EPI, bool H1, int RT>
__device__ __forceinline__ void epilogue1(const StreamArgs& p, const Item& c, v4f (&acc)[kCB][RT], int nw,
                                          int wave) {
  const int lane = epilogue_lane();
  const int g = lane >> 4, r = lane & 15;
  const int i16 = p.inter >> 4;
  const int aw = EPI == kActGelu ? 2 * p.inter : p.inter;
  const int ks2 = aw >> 7;
  uint8_t* const aq = p.aq;
  uint8_t* const sa = p.sa;
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    if (j >= nw) break;                        // uniform per wave
    const int t = 4 * j + wave;
    const int64_t tl = (int64_t)(c.row0 >> 4) + t;
#pragma unroll
    for (int pg = 0; pg < kCB / 4; ++pg) {     // 32-channel groups of the block's gate channels
      const int gt = c.cb * (kCB / 2) + 2 * pg;   // first gate tile of the group
      if (gt >= i16) break;                    // partial last block (uniform)
      const int ch = 16 * gt;
      __builtin_amdgcn_sched_barrier(0);       // one group at a time: its 16 accumulators in VGPRs
      if constexpr (EPI == kActGelu) {
        float ag[2][4], au[2][4];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ag[jj][i] = gelu_act(acc[2 * pg + jj][j][i]);
            au[jj][i] = gelu_act(acc[kCB / 2 + 2 * pg + jj][j][i]);
          }
        store_a_group<FMT>(ag, aq, sa, tl, ks2, ch, g, r);
        store_a_group<FMT>(au, aq, sa, tl, ks2, p.inter + ch, g, r);
      } else {
        float a2[2][4];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            a2[jj][i] = gated_act<EPI>(acc[2 * pg + jj][j][i], acc[kCB / 2 + 2 * pg + jj][j][i], p.act);
        store_a_group<FMT>(a2, aq, sa, tl, ks2, ch, g, r);
      }
      const int rr = 16 * t + r;
      if (H1 && c.e != p.sh_first && rr < c.nrows) {   // h1: the routed experts' rows only
        float* row = p.h1 + (int64_t)(c.srow0 + rr) * 2 * p.inter;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int cg = ch + 16 * jj + 4 * g;
          *reinterpret_cast<float4*>(row + cg) = make_float4(acc[2 * pg + jj][j][0], acc[2 * pg + jj][j][1],
                                                             acc[2 * pg + jj][j][2], acc[2 * pg + jj][j][3]);
          const v4f& u = acc[kCB / 2 + 2 * pg + jj][j];
          *reinterpret_cast<float4*>(row + p.inter + cg) = make_float4(u[0], u[1], u[2], u[3]);
        }
      }
    }
  }
}

// GMM2 epilogue: acc[q][j][i] = O[row 16 t + r][channel 16 (12 cb + q) + 4 g + i].
// bf16 O: the lanes exchange halves of two tiles so that each stores 16 bytes (GMM2 of
// the prefill-shaped layer 8% faster than with 8-byte stores: the store instructions of
// an item, not its bytes, were the cost).
template <bool OBF16, int RT>
__device__ __forceinline__ void epilogue2(const StreamArgs& p, const Item& c, v4f (&acc)[kCB][RT], int nw,
                                          int wave) {
  const int lane = epilogue_lane();
  const int g = lane >> 4, r = lane & 15;
  const int n16 = p.N >> 4;
  float* const o = p.o;
  uint16_t* const o16 = p.o16;
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    if (j >= nw) break;
    const int rr = 16 * (4 * j + wave) + r;
    const bool row_ok = rr < c.nrows;         // the same for the four lanes of row r
    const int64_t row = (int64_t)(c.srow0 + rr) * p.N;
    if constexpr (OBF16) {
      // tiles q, q + 1: after one row swap per dword a lane of row g holds 8 contiguous
      // channels, 4 (g & 2) .. + 7 of tile q + (g & 1) (n16 is even: pairs never straddle
      // the end of hidden)
#pragma unroll
      for (int q = 0; q < kCB; q += 2) {
        const int tile = c.cb * kCB + q;
        if (tile >= n16) break;                  // partial last block (uniform)
        __builtin_amdgcn_sched_barrier(0);
        v4f x = acc[q][j], y = acc[q + 1][j];
        asm volatile("" : "+v"(x), "+v"(y));     // through vector registers
        const auto lo = __builtin_amdgcn_permlane16_swap(bf16x2(x[0], x[1]), bf16x2(y[0], y[1]), false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap(bf16x2(x[2], x[3]), bf16x2(y[2], y[3]), false, false);
        if (row_ok) {
          const int64_t at = row + 16 * (tile + (g & 1)) + 4 * (g & 2);
          *reinterpret_cast<u32x4*>(o16 + at) = u32x4{lo[0], hi[0], lo[1], hi[1]};
        }
      }
    } else {
      if (!row_ok) continue;                    // per lane; no cross-lane work below
#pragma unroll
      for (int q = 0; q < kCB; ++q) {
        const int tile = c.cb * kCB + q;
        if (tile >= n16) break;                  // partial last block (uniform)
        __builtin_amdgcn_sched_barrier(0);
        const int64_t at = row + 16 * tile + 4 * g;
        v4f x = acc[q][j];
        asm volatile("" : "+v"(x));   // through vector registers, as the bf16 path
        *reinterpret_cast<float4*>(o + at) = make_float4(x[0], x[1], x[2], x[3]);
      }
    }
  }
}

template <int RT>
__device__ __forceinline__ void zero_acc(v4f (&acc)[kCB][RT]) {
#pragma unroll
  for (int q = 0; q < kCB; ++q)
#pragma unroll
    for (int j = 0; j < RT; ++j) acc[q][j] = v4f{0.f, 0.f, 0.f, 0.f};
}

// The kernel body gets the LDS area twice, as two restrict pointers: one that the
// direct-to-LDS loads go through, one for every read. The compiler then does not make
// each LDS read wait for every direct-to-LDS load in flight (it cannot tell which bytes
// such a load writes); the reads of a weight slot are ordered after its loads by the
// explicit wait and barrier at the top of each K step, with a compiler-level memory fence
// after the barrier.
// The channel blocks of an item's chunk.
template <int GMM>
__device__ __forceinline__ int channel_blocks(const StreamArgs& p) {
  return GMM == 1 ? ((p.inter >> 4) + kCB / 2 - 1) / (kCB / 2) : ((p.N >> 4) + kCB - 1) / kCB;
}

// The items first, first + stride, ... < last of the chunk list `tiles`.
template <int FMT, bool PACKED, int WF, int GMM, int EPI, bool OBF16, bool H1, int RT>
__device__ __forceinline__ void stream_body(const StreamArgs& p, const int4* tiles, int first, int stride, int last,
                                            uint8_t* __restrict__ lds, const uint8_t* __restrict__ ldsr);

template <int FMT, bool PACKED, int WF, int GMM, int EPI, bool OBF16, bool H1, int RT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void gmm_stream_kernel(StreamArgs p) {
  extern __shared__ __align__(16) uint8_t lds_area[];
  int first, stride, last;
  block_items(*p.tile_count * channel_blocks<GMM>(p), &first, &stride, &last);
  stream_body<FMT, PACKED, WF, GMM, EPI, OBF16, H1, RT>(p, p.tiles, first, stride, last, lds_area, lds_area);
}

// The three chunk-size classes in one launch, each by the instance of its token tiles a
// wave, one class after the other (most tiles first). Each XCD takes a contiguous share
// of every class's items, and the XCD's workgroups deal its items round robin, the deal
// continuing from class to class: a workgroup left with one item fewer of a class gets
// the next class's first items, so every workgroup ends within about one item of the
// others (one launch a class leaves the last round of each class part-empty).
template <int FMT, int WF, int GMM, int EPI, bool OBF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void gmm_stream_classes_kernel(StreamArgs p, StreamClasses cl) {
  static_assert(kStreamClasses == 3 && kStreamClassRT[2] == kRT, "classes of 2, 4 and 5 token tiles a wave");
  extern __shared__ __align__(16) uint8_t lds_area[];
  const int ncb = channel_blocks<GMM>(p);
  const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds, per = gridDim.x / kXcds;
  int dealt = 0;   // items of the earlier classes dealt on this XCD, modulo per
  auto phase = [&]<int C>(std::integral_constant<int, C>) {
    const int total = cl.count[C] * ncb;
    const int lo = (int)(((int64_t)total * xcd) / kXcds), hi = (int)(((int64_t)total * (xcd + 1)) / kXcds);
    const int first = lo + (j - dealt + per) % per;
    if (first < hi) {   // uniform per workgroup
      stream_body<FMT, true, WF, GMM, EPI, OBF16, false, kStreamClassRT[C]>(p, cl.tiles + C * cl.stride, first, per,
                                                                           hi, lds_area, lds_area);
      __syncthreads();   // every wave is done with the LDS slots before the next class's prologue fills them
    }
    dealt = (dealt + (hi - lo)) % per;
  };
  phase(std::integral_constant<int, 2>());
  phase(std::integral_constant<int, 1>());
  phase(std::integral_constant<int, 0>());
}

template <int FMT, bool PACKED, int WF, int GMM, int EPI, bool OBF16, bool H1, int RT>
__device__ __forceinline__ void stream_body(const StreamArgs& p, const int4* tiles, int first, int stride, int last,
                                            uint8_t* __restrict__ lds, const uint8_t* __restrict__ ldsr) {
  using SW = StreamW<WF, PACKED>;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ks = p.K >> 7, kq = (ks + 3) >> 2;
  const int n16 = p.N >> 4, i16 = p.inter >> 4;
  const LaneOffsets lofs = lane_offsets<PACKED, WF>(p.K, lane);
  const int ncb = channel_blocks<GMM>(p);
  const int count = first < last ? (last - first + stride - 1) / stride : 0;
  if (count == 0) return;

  v4f acc[kCB][RT];
  zero_acc(acc);
  v8i t0[RT], t1[RT], t2[RT], t3[RT];

  // items n (cur), n + 1 (nxt) and n + 2 (nn, read an item early so that its scalar loads
  // have landed when it becomes nxt); past the last item each repeats the last one
  Item cur = load_item(tiles, first, ncb);
  Item nxt = count > 1 ? load_item(tiles, first + stride, ncb) : cur;
  Item nn = count > 2 ? load_item(tiles, first + 2 * stride, ncb) : nxt;

  // prologue: the loads of steps -4..-1 in the steady state's order, S0 (the scale group
  // of steps 0..3), W0, T0 W1, T1 W2, T2 W3 (all in item 0: ks >= 4)
  uint8_t* const groups = lds + SW::kGroups;
  const uint8_t* const groups_r = ldsr + SW::kGroups;
  issue_scales<GMM, PACKED, WF, RT>(p, cur, 0, groups, ks, kq, n16, i16, lofs, wave);
  issue_weights<GMM, PACKED, WF>(p, cur, 0, lds, n16, i16, lofs, wave);
  issue_tokens<RT>(p, cur, 0, ks, kq, wave, lofs, t0);
  issue_weights<GMM, PACKED, WF>(p, cur, 1, lds + SW::kSlotBytes, n16, i16, lofs, wave);
  issue_tokens<RT>(p, cur, 1, ks, kq, wave, lofs, t1);
  issue_weights<GMM, PACKED, WF>(p, cur, 2, lds + 2 * SW::kSlotBytes, n16, i16, lofs, wave);
  issue_tokens<RT>(p, cur, 2, ks, kq, wave, lofs, t2);
  issue_weights<GMM, PACKED, WF>(p, cur, 3, lds + 3 * SW::kSlotBytes, n16, i16, lofs, wave);
  int wslot = 4;   // slot of the next weight loads
  int cslot = 0;   // slot of the next compute step
  int grp = 0;     // scale group of the next compute step

  static_assert(kTokLead == 3, "the item loop below rotates four token register sets");
  constexpr int kWeightsAfter = 5;
  static_assert(kWeightsAfter + 1 < kCB, "the loads of a step go out between its MFMA groups");
  for (int n = 0; n < count; ++n) {
    const bool last_item = n + 1 >= count;
    // K step kc of item n with the token registers of set (tc); the token loads of
    // kc + kTokLead go into set (tn), the set the previous step used; a step kc = 0 mod 4
    // also loads the scale group of steps kc + 4 .. kc + 7 into the other group.
    // (even: kc is even; with six slots only even steps wait and meet the barrier)
    auto step = [&]<bool ZERO_C>(std::integral_constant<bool, ZERO_C>, int kc, bool group_start, bool even, v8i(&tc)[RT],
                                 v8i(&tn)[RT]) {
      constexpr bool kPaired = SW::kSlots == 6;
      if (!kPaired || even) {
        wait_vmcnt<kPaired ? SW::template kWaitPair<RT> : SW::template kWait<RT>>();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
      const Ahead at = ahead(cur, nxt, last_item, kc, kTokLead, ks);
      const TokenStep tl = token_step(p, at.d, at.k, ks, kq);
      const Ahead aw = ahead(cur, nxt, last_item, kc, kLead, ks);
      const WeightStep wl = weight_step<WF, PACKED>(p, aw.d, aw.k, n16);
      uint8_t* const wdst = lds + wslot * SW::kSlotBytes;
      wslot = wslot == SW::kSlots - 1 ? 0 : wslot + 1;
      __builtin_amdgcn_sched_barrier(0);
      // the token loads before the MFMAs; the weight codes after MFMA group kWeightsAfter,
      // the scale group after the next one (placements measured best: the loads of a
      // step spread over it, and a clean register allocation of the K loop)
#pragma unroll
      for (int j = 0; j < RT; ++j) issue_token_tile(tl, j, ks, wave, lofs, tn[j]);
      __builtin_amdgcn_sched_barrier(0);
      auto between = [&](int q) {
        if (q == kWeightsAfter) {
#pragma unroll
          for (int i = 0; i < kCB / 4; ++i)
            issue_weight_tile<GMM, PACKED, WF>(wl, i, wdst, p.K, n16, i16, lofs, wave);
        } else if (q == kWeightsAfter + 1 && group_start) {
          issue_scales<GMM, PACKED, WF, RT>(p, aw.d, aw.k, groups + (grp ^ 1) * SW::kGroupBytes, ks, kq, n16, i16, lofs,
                                        wave);
        }
      };
      step_mfma<FMT, PACKED, WF, RT, ZERO_C>(acc, ldsr + cslot * SW::kSlotBytes, groups_r + grp * SW::kGroupBytes, kc,
                                             lane, wave, tc, between);
      cslot = cslot == SW::kSlots - 1 ? 0 : cslot + 1;
    };
    // K steps of item n (a multiple of 4): t0..t3 in turn, the first step uses t0. The
    // GMM2 instances of at most four tiles a wave start an item with a zero C operand in
    // its first step's MFMAs rather than a zeroing pass after the previous item (measured
    // ~1.5% off GMM2; in GMM1 the peeled first group measured slower, and the five-tile
    // instances then spill registers).
    constexpr bool kZeroC = GMM == 2 && RT < 5;
    const std::integral_constant<bool, false> accum;
    int k0 = 0;
    if constexpr (kZeroC) {
      const std::integral_constant<bool, true> zero_c;
      step(zero_c, 0, true, true, t0, t3);
      step(accum, 1, false, false, t1, t0);
      step(accum, 2, false, true, t2, t1);
      step(accum, 3, false, false, t3, t2);
      grp ^= 1;
      k0 = 4;
    }
    for (int k = k0; k < ks; k += 4) {
      step(accum, k, true, true, t0, t3);
      step(accum, k + 1, false, false, t1, t0);
      step(accum, k + 2, false, true, t2, t1);
      step(accum, k + 3, false, false, t3, t2);
      grp ^= 1;
    }
    const int nw = wave_tiles(cur.nrows, wave);
    if constexpr (GMM == 1)
      epilogue1<FMT, EPI, H1, RT>(p, cur, acc, nw, wave);
    else
      epilogue2<OBF16, RT>(p, cur, acc, nw, wave);
    if constexpr (!kZeroC) zero_acc(acc);
    cur = nxt;
    nxt = nn;
    if (n + 3 < count) nn = load_item(tiles, first + (n + 3) * stride, ncb);
  }
  wait_vmcnt<0>();   // no direct-to-LDS load still writes when the workgroup's LDS is released
}

}  // namespace

#ifndef MOE_STREAM_KERNEL_ONLY   // (defined by single-instance builds that inspect the kernel's code)
namespace {

template <int FMT, bool PACKED, int WF, int GMM, int EPI, bool OBF16, bool H1, int RT = kRT>
hipError_t stream_go(const StreamArgs& a, hipStream_t st) {
  auto kern = gmm_stream_kernel<FMT, PACKED, WF, GMM, EPI, OBF16, H1, RT>;
  LaunchShape ls;
  hipError_t e = persistent_shape(kern, StreamW<WF, PACKED>::kLds, &ls);
  if (e != hipSuccess) return e;
  kern<<<ls.grid, 256, ls.lds, st>>>(a);
  return hipGetLastError();
}

// GMM1: one instance per activation, and one with the h1 parity output (storing h1 from
// the epilogue costs the fast instance its clean register allocation).
template <int FMT, bool PACKED, int WF, bool H1>
hipError_t stream_gmm1_act(const StreamArgs& a, int kind, hipStream_t st) {
  switch (kind) {
    case 1: return stream_go<FMT, PACKED, WF, 1, 1, false, H1>(a, st);
    case 2: return stream_go<FMT, PACKED, WF, 1, 2, false, H1>(a, st);
    case 3: return stream_go<FMT, PACKED, WF, 1, 3, false, H1>(a, st);
    case kActGelu: return stream_go<FMT, PACKED, WF, 1, kActGelu, false, H1>(a, st);
    default: return stream_go<FMT, PACKED, WF, 1, 0, false, H1>(a, st);
  }
}

template <int FMT, bool PACKED, int WF>
hipError_t stream_gmm1(const StreamArgs& a, int kind, hipStream_t st) {
  return a.h1 ? stream_gmm1_act<FMT, PACKED, WF, true>(a, kind, st) : stream_gmm1_act<FMT, PACKED, WF, false>(a, kind, st);
}

template <int FMT, bool PACKED, int WF>
hipError_t stream_gmm2(const StreamArgs& a, hipStream_t st) {
  return a.o16 ? stream_go<FMT, PACKED, WF, 2, 0, true, false>(a, st)
               : stream_go<FMT, PACKED, WF, 2, 0, false, false>(a, st);
}

// The folded shared expert's weights as offsets from where group sh.group's weights
// would sit in the routed experts' arrays.
template <bool PACKED>
void set_shared_t(StreamArgs& a, const SharedGroups& sh, bool fp4) {
  a.sh_first = INT_MAX;
  a.sh_wdelta = a.sh_sdelta = 0;
  if (!sh.w) return;
  const int64_t K = a.K, kq = ((K >> 7) + 3) >> 2;
  const int64_t cbytes = (int64_t)a.N * (fp4 ? K >> 1 : K);
  const int64_t sbytes = PACKED ? (int64_t)(a.N >> 4) * kq * kTileScaleBytes : (int64_t)a.N * (K >> 5);
  a.sh_first = sh.group;
  a.sh_wdelta = (int64_t)((uintptr_t)sh.w - (uintptr_t)(a.w + sh.group * cbytes));
  a.sh_sdelta = (int64_t)((uintptr_t)sh.ws - (uintptr_t)(a.ws + sh.group * sbytes));
}

void set_shared(StreamArgs& a, const SharedGroups& sh, int wfp4, int packed) {
  if (packed)
    set_shared_t<true>(a, sh, wfp4 != 0);
  else
    set_shared_t<false>(a, sh, wfp4 != 0);
}

// The chunk classes in one launch (gmm_stream_classes_kernel).
template <int FMT, int WF, int GMM, int EPI, bool OBF16>
hipError_t stream_classes(const StreamArgs& a, const StreamClasses& cl, hipStream_t st) {
  auto kern = gmm_stream_classes_kernel<FMT, WF, GMM, EPI, OBF16>;
  LaunchShape ls;
  hipError_t e = persistent_shape(kern, StreamW<WF, true>::kLds, &ls);
  if (e != hipSuccess) return e;
  kern<<<ls.grid, 256, ls.lds, st>>>(a, cl);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gmm1_stream(const Gmm1Params& p, hipStream_t st) {
  StreamArgs a{};
  a.tok = p.xq; a.toks = p.sx; a.w = p.w; a.ws = p.ws; a.tiles = p.tiles; a.tile_count = p.tile_count;
  a.K = p.hidden; a.N = 2 * p.inter; a.inter = p.inter; a.aq = p.aq; a.sa = p.sa; a.h1 = p.h1; a.act = p.act;
  set_shared(a, p.shared, p.wfp4, p.packed);
  // chunk classes: the packed FP8 SwiGLU instance without the h1 output
  if (p.classes.tiles && p.packed && !p.wfp4 && !p.h1 && p.act.kind == 0) {
    if (p.act.clamp == __builtin_huge_valf())
      return p.fmt == 0 ? stream_classes<0, 0, 1, kActSwigluNoClamp, false>(a, p.classes, st)
                        : stream_classes<1, 1, 1, kActSwigluNoClamp, false>(a, p.classes, st);
    return p.fmt == 0 ? stream_classes<0, 0, 1, 0, false>(a, p.classes, st)
                      : stream_classes<1, 1, 1, 0, false>(a, p.classes, st);
  }
  if (p.wfp4) {
    if (p.fmt != 0) return hipErrorInvalidValue;
    return p.packed ? stream_gmm1<0, true, kFmtFp4>(a, p.act.kind, st) : stream_gmm1<0, false, kFmtFp4>(a, p.act.kind, st);
  }
  if (p.fmt == 0) return p.packed ? stream_gmm1<0, true, 0>(a, p.act.kind, st) : stream_gmm1<0, false, 0>(a, p.act.kind, st);
  return p.packed ? stream_gmm1<1, true, 1>(a, p.act.kind, st) : stream_gmm1<1, false, 1>(a, p.act.kind, st);
}

hipError_t launch_gmm2_stream(const Gmm2Params& p, hipStream_t st) {
  StreamArgs a{};
  a.tok = p.aq; a.toks = p.sa; a.w = p.w; a.ws = p.ws; a.tiles = p.tiles; a.tile_count = p.tile_count;
  a.K = p.inter; a.N = p.hidden; a.inter = p.inter; a.o = p.o; a.o16 = p.o16;
  set_shared(a, p.shared, p.wfp4, p.packed);
  // chunk classes: the packed FP8 instance with bf16 O rows
  if (p.classes.tiles && p.packed && !p.wfp4 && p.o16)
    return p.fmt == 0 ? stream_classes<0, 0, 2, 0, true>(a, p.classes, st)
                      : stream_classes<1, 1, 2, 0, true>(a, p.classes, st);
  if (p.wfp4) {
    if (p.fmt != 0) return hipErrorInvalidValue;
    return p.packed ? stream_gmm2<0, true, kFmtFp4>(a, st) : stream_gmm2<0, false, kFmtFp4>(a, st);
  }
  if (p.fmt == 0) return p.packed ? stream_gmm2<0, true, 0>(a, st) : stream_gmm2<0, false, 0>(a, st);
  return p.packed ? stream_gmm2<1, true, 1>(a, st) : stream_gmm2<1, false, 1>(a, st);
}
#endif

}  // namespace moe
