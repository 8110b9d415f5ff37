// Grouped GEMMs of the MX expert FFN on gfx950 block-scaled MFMA.
//
// MegaMoE README, "A8W8-FP quantization scenario":
//   stage 2  G_e = DQ(X^_e).DQ(W1_e^(G)), U_e = DQ(X^_e).DQ(W1_e^(U)), A_e = SiLU(G_e)*U_e
//            (swiglu of the activation formulas, no clamp), then A^_e, S_A,e = Q_MX(A_e)
//            with the FP8 type of stage 1;
//   stage 3  O_e = DQ(A^_e).DQ(W2_e);
//   stage 4  Y[i] = sum_k W[i,k] O[pi(i,k)] (+ the shared experts' outputs).
// Weight layout (MXFP quantization scenario constraints): weight1 (E, 2I, H), weight2
// (E, H, I), every output channel a K-contiguous row with one E8M0 scale per 32; the
// first I channels of weight1 are the gate branch, the last I the up branch.
//
// These kernels take layers whose experts hold at most 128 rows on average (decode-
// shaped); layers with more rows per expert take the LDS-streaming kernels of
// gmm_stream.hip (gmm_token_tiles chooses).
//
// Design (one kernel per GEMM, persistent):
// * Work item = (token chunk of one expert, channel block). A chunk holds up to 16*NT
//   rows of one expert, NT = 1, 2, 4 or 8 (device-built tile list, no host readback of
//   the counts).
// * Each wave owns 64 output channels (GMM1: 32 gate + the matching 32 up channels) and
//   streams their weights from HBM straight into VGPRs exactly once per chunk, with a
//   two-step register prefetch. The chunk's token rows are staged per K step into LDS
//   (double-buffered, laid out exactly as the MFMA operand so every ds_read_b128 is
//   conflict-free) and shared by the block's waves.
// * V_MFMA_SCALE_F32_16X16X128_F8F6F4 with the E8M0 scales applied by the matrix core.
//   GMM1 puts the weights in the A slot (output rows = channels): a lane then holds the
//   gate and up values of the same channels, so SwiGLU is lane-local and the 32-channel
//   MX group of the requantization is the lane's 8 values plus 3 lanes (xor 16 / 32).
//   GMM2 puts the tokens in the A slot (output rows = tokens): a lane group then holds
//   16 consecutive channels of one token, stored as one 32-byte (bf16) or 64-byte (fp32)
//   piece of that token's O row with plain stores; the weighted combine reads the rows
//   back per token (combine.hip), in a fixed order.
// * Blocks are persistent and XCD-aware: block b runs on XCD b % 8 and takes items from
//   that XCD's contiguous share of the item list, so the channel blocks of one expert run
//   together on one XCD and share its L2 for the token rows.
// * Weights are read either in the pages' layout (ND) or in an MFMA-native packed layout
//   (built once by moe_mx_pack_weights, the analog of the pages' fractal weight formats):
//   16-channel x 128-K blocks of 2 KB in lane order, so each load instruction of a wave
//   reads 1 KB of contiguous memory, with the scales of 4 K steps in one dword per lane.

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>

#include "device_common.h"
#include "gmm_device.h"
#include "internal.h"

namespace moe {
namespace {

// ---- the K loop shared by both GEMMs ---------------------------------------------
// Loads issued in K step s, numbered: first the weights of step s + WPF (per weight
// tile: operand lo half, hi half, scale dword; from HBM into the VGPR buffer that step
// uses), then the token tiles of step s + 2 (per tile this wave stages: lo half, hi
// half, scale dword; from L2 into ring slot (s + 2) % 3). WPF (weight prefetch
// distance) is 2: three weight buffers fit in the registers beside the accumulators of
// up to 8 token tiles; MXFP4 weights in chunks of up to 2 tiles take WPF = 3 (four
// buffers; the half-size FP4 loads keep half the bytes in flight: GMM1 of the MXFP4
// decode-shaped layer 2.6% faster; with FP8 weights the fourth buffer spills). At the
// top of step s the weights and token tiles of step s must have landed; the newest
// batch (step s + 1's) may be in flight: one fixed vmcnt (with WPF = 3 too: the batch
// issued in step s - 2 holds the token tiles of step s and is followed by one batch).
template <int NT, int WF> struct WeightPrefetch { static constexpr int value = WF == kFmtFp4 && NT <= 2 ? 3 : 2; };

template <int NT, int WF, int QW>
struct Batch {
  static constexpr int kWeights = QW * WeightFmt<WF>::kParts;
  static constexpr int kTokens = 3 * StageLayout<NT>::kPerWave;
  static constexpr int kLoads = kWeights + kTokens;
  static constexpr int kInFlight = WeightPrefetch<NT, WF>::value >= 2 ? kLoads : kTokens;
};

// NTW: the weight codes with non-temporal loads (streamed once per chunk; GMM1 measured
// 5% faster on the decode-shaped layer with them, GMM2 3% slower, so GMM1 only).
template <int NT, bool PACKED, int WF, int QW, bool NTW, int K_SLOT>
__device__ __forceinline__ void load_slot(v8i (&aload)[QW], int (&sload)[QW], const WPtr<PACKED> (&wp)[QW], int wstep,
                                          const uint8_t* tok, const uint8_t* toks, int ks, int row0, int ntt,
                                          int tstep, uint8_t* slot, int wave, int lane) {
  constexpr int kW = Batch<NT, WF, QW>::kWeights;
  if constexpr (K_SLOT < kW) {
    constexpr int kParts = WeightFmt<WF>::kParts;
    constexpr int q = K_SLOT / kParts, part = K_SLOT % kParts;
    const int g = lane >> 4;
    if constexpr (part == kParts - 1) {
      if constexpr (PACKED)
        sload[q] = (int)*reinterpret_cast<const uint32_t*>(wp[q].s + (wstep >> 2) * kTileScaleBytes);
      else
        sload[q] = (int)*reinterpret_cast<const uint32_t*>(wp[q].s + 4 * wstep);
    } else {
      const uint8_t* src;
      if constexpr (PACKED)
        src = wp[q].d + (int64_t)wstep * WeightFmt<WF>::kStepBytes + part * 1024 + lane * 16;
      else if constexpr (WeightFmt<WF>::kFp4)
        src = wp[q].d + 64 * wstep + 16 * g;
      else
        src = wp[q].d + 128 * wstep + part * 64 + 16 * g;
      const u32x4 v = NTW ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src))
                          : *reinterpret_cast<const u32x4*>(src);
#pragma unroll
      for (int j = 0; j < 4; ++j) aload[q][4 * part + j] = (int)v[j];
    }
  } else {
    // Tile wave + 4 i of the chunk (clamped to its last tile: a wave past the end
    // re-stages that tile, writing the same bytes another wave writes).
    constexpr int i = (K_SLOT - kW) / 3, part = (K_SLOT - kW) % 3;
    const int t = min(wave + 4 * i, ntt - 1);
    const int64_t tile = (int64_t)(row0 >> 4) + t;
    if constexpr (part == 2)
      lds_dma4(toks + t16_scales(tile, (ks + 3) >> 2, tstep >> 2) + 4 * lane, slot + NT * kTileBytes + t * kTileScaleBytes);
    else
      lds_dma16(tok + t16_codes(tile, ks, tstep) + part * 1024 + 16 * lane, slot + t * kTileBytes + part * 1024);
  }
}

template <int NT, bool PACKED, int WF, int QW, bool NTW, int K0, int... I>
__device__ __forceinline__ void load_slots(std::integer_sequence<int, I...>, v8i (&aload)[QW], int (&sload)[QW],
                                           const WPtr<PACKED> (&wp)[QW], int wstep, const uint8_t* tok,
                                           const uint8_t* toks, int ks, int row0, int ntt, int tstep, uint8_t* slot,
                                           int wave, int lane) {
  (load_slot<NT, PACKED, WF, QW, NTW, K0 + I>(aload, sload, wp, wstep, tok, toks, ks, row0, ntt, tstep, slot, wave, lane), ...);
}

// One K step s, with its weights in (acur, scur) and its token tiles in ring slot
// s % 3 (`cur`):
//  1. wait until the loads of step s have landed and meet the barrier: every wave's
//     token tiles of step s are then in LDS, and every wave is done with slot
//     (s + 2) % 3, read in step s - 1;
//  2. issue the weights of step s + WPF into (aload, sload) and the token tiles of step
//     s + 2 into slot (s + 2) % 3 (past the last step the last one is re-read: in
//     bounds, unused);
//  3. the MFMAs of step s.
// All NT token tiles are multiplied whatever the chunk's tile count ntt: the MFMA
// sequence is straight-line code in which the LDS reads of tile t+1 are issued before
// the MFMAs of tile t. Tiles in [ntt, NT) hold stale LDS bytes; their accumulators are
// never stored (idle tiles of a partial chunk cost MFMA time only).
// Load placement: with one wave per SIMD the MFMA pipe idles whenever the wave's
// in-order issue waits, and a burst of loads waits for the CU's vector memory unit. So
// for chunks of 4 or more tiles the loads are spread one after each MFMA (scheduling
// fences keep them there); loads that do not fit, and all loads of small chunks, go
// first.
// WEIGHTS_A: weights in the MFMA A slot (GMM1), else tokens in the A slot (GMM2).
template <int FMT, int NT, bool PACKED, bool WEIGHTS_A, int WF, int QW>
__device__ __forceinline__ void k_step(int s, int ks, int cur, v4f (&acc)[QW][NT], const WPtr<PACKED> (&wp)[QW],
                                       const v8i (&acur)[QW], const int (&scur)[QW], v8i (&aload)[QW],
                                       int (&sload)[QW], const uint8_t* tok, const uint8_t* toks, int row0, int ntt,
                                       uint8_t* lds, int wave, int lane) {
  constexpr int kLoads = Batch<NT, WF, QW>::kLoads;
  constexpr int kTop = NT < 4 ? kLoads : (kLoads > QW * NT ? kLoads - QW * NT : 0);
  constexpr int kBuf = StageLayout<NT>::kBufBytes;
  wait_vmcnt<Batch<NT, WF, QW>::kInFlight>();
  block_barrier<NT>();
  const int wstep = min(s + WeightPrefetch<NT, WF>::value, ks - 1), tstep = min(s + 2, ks - 1);
  uint8_t* slot = lds + (cur == 0 ? 2 : cur - 1) * kBuf;   // (cur + 2) % 3
  const uint8_t* buf = lds + cur * kBuf;
  load_slots<NT, PACKED, WF, QW, WEIGHTS_A, 0>(std::make_integer_sequence<int, kTop>{}, aload, sload, wp, wstep, tok, toks, ks, row0,
                            ntt, tstep, slot, wave, lane);
  int sw[QW];
#pragma unroll
  for (int q = 0; q < QW; ++q) sw[q] = weight_scale<PACKED>(scur[q], s, lane);
  v8i b[2];
  int sb[2];
  stage_read<NT>(buf, 0, s, lane, b[0], sb[0]);
  [&]<int... T>(std::integer_sequence<int, T...>) {
    ([&] {
      constexpr int t = T;
      if constexpr (t + 1 < NT) stage_read<NT>(buf, t + 1, s, lane, b[(t + 1) & 1], sb[(t + 1) & 1]);
      [&]<int... Q>(std::integer_sequence<int, Q...>) {
        ([&] {
          constexpr int q = Q;
          if constexpr (WEIGHTS_A)
            acc[q][t] = mfma_mx16_ab<WF, FMT>(acur[q], b[t & 1], acc[q][t], sw[q], sb[t & 1]);
          else
            acc[q][t] = mfma_mx16_ab<FMT, WF>(b[t & 1], acur[q], acc[q][t], sb[t & 1], sw[q]);
          constexpr int k = kTop + QW * t + q;
          if constexpr (k < kLoads) {
            load_slot<NT, PACKED, WF, QW, WEIGHTS_A, k>(aload, sload, wp, wstep, tok, toks, ks, row0, ntt, tstep, slot, wave, lane);
            __builtin_amdgcn_sched_barrier(0);
          }
        }(), ...);
      }(std::make_integer_sequence<int, QW>{});
    }(), ...);
  }(std::make_integer_sequence<int, NT>{});
}

// The K loop of one chunk with WPF = 2. Three weight register buffers rotate with the step (roles
// fixed in the unrolled three-step body: step s uses a0 and loads into a2, s + 1 uses a1
// and loads into a0, s + 2 uses a2 and loads into a1); the ring slot is a runtime
// index. The r = ks % 3 leftover steps run first, and batches 0 and 1 go into the
// buffers that make the rotation line up when the loop starts at step r (no buffer is
// copied: a copy would wait for its load). (With the leftover steps after the loop the
// register allocator permutes the accumulators across the loop body instead.) At the
// end every load has landed and every wave is past its last LDS read, so the next
// chunk may reuse the ring.
template <int FMT, int NT, bool PACKED, bool WEIGHTS_A, int WF, int QW>
__device__ __forceinline__ void k_loop_pf2(v4f (&acc)[QW][NT], const WPtr<PACKED> (&wp)[QW], const uint8_t* tok,
                                       const uint8_t* toks, int K, int row0, int ntt, uint8_t* lds, int wave,
                                       int lane) {
  constexpr int kL = Batch<NT, WF, QW>::kLoads;
  constexpr int kBuf = StageLayout<NT>::kBufBytes;
  const int ks = K >> 7, r = ks % 3, s1 = min(1, ks - 1);
  v8i a0[QW], a1[QW], a2[QW];
  int c0[QW], c1[QW], c2[QW];
  auto seq = std::make_integer_sequence<int, kL>{};
  if (r == 0) {
    load_slots<NT, PACKED, WF, QW, WEIGHTS_A, 0>(seq, a0, c0, wp, 0, tok, toks, ks, row0, ntt, 0, lds, wave, lane);
    load_slots<NT, PACKED, WF, QW, WEIGHTS_A, 0>(seq, a1, c1, wp, s1, tok, toks, ks, row0, ntt, s1, lds + kBuf, wave, lane);
  } else if (r == 1) {
    load_slots<NT, PACKED, WF, QW, WEIGHTS_A, 0>(seq, a2, c2, wp, 0, tok, toks, ks, row0, ntt, 0, lds, wave, lane);
    load_slots<NT, PACKED, WF, QW, WEIGHTS_A, 0>(seq, a0, c0, wp, s1, tok, toks, ks, row0, ntt, s1, lds + kBuf, wave, lane);
  } else {
    load_slots<NT, PACKED, WF, QW, WEIGHTS_A, 0>(seq, a1, c1, wp, 0, tok, toks, ks, row0, ntt, 0, lds, wave, lane);
    load_slots<NT, PACKED, WF, QW, WEIGHTS_A, 0>(seq, a2, c2, wp, s1, tok, toks, ks, row0, ntt, s1, lds + kBuf, wave, lane);
  }
  int s = 0, cur = 0;
  if (r == 1) {
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(0, ks, 0, acc, wp, a2, c2, a1, c1, tok, toks, row0, ntt, lds, wave, lane);
    s = 1;
    cur = 1;
  } else if (r == 2) {
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(0, ks, 0, acc, wp, a1, c1, a0, c0, tok, toks, row0, ntt, lds, wave, lane);
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(1, ks, 1, acc, wp, a2, c2, a1, c1, tok, toks, row0, ntt, lds, wave, lane);
    s = 2;
    cur = 2;
  }
  for (; s < ks; s += 3) {
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(s, ks, cur, acc, wp, a0, c0, a2, c2, tok, toks, row0, ntt, lds, wave, lane);
    cur = cur == 2 ? 0 : cur + 1;
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(s + 1, ks, cur, acc, wp, a1, c1, a0, c0, tok, toks, row0, ntt, lds, wave, lane);
    cur = cur == 2 ? 0 : cur + 1;
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(s + 2, ks, cur, acc, wp, a2, c2, a1, c1, tok, toks, row0, ntt, lds, wave, lane);
    cur = cur == 2 ? 0 : cur + 1;
  }
  wait_vmcnt<0>();
  __syncthreads();
}

// The K loop of one chunk with WPF = 3: four weight register buffers with fixed roles in
// the unrolled four-step body (a0 -> a3, a1 -> a0, a2 -> a1, a3 -> a2: the buffer a step
// uses, then the one it loads the weights of step + 3 into); the ks % 4 leftover steps
// run first from buffers chosen so that the roles line up at the loop's first step. The
// prologue loads weights 0, 1, 2 and the token tiles of steps 0 and 1.
template <int FMT, int NT, bool PACKED, bool WEIGHTS_A, int WF, int QW>
__device__ __forceinline__ void k_loop_pf3(v4f (&acc)[QW][NT], const WPtr<PACKED> (&wp)[QW], const uint8_t* tok,
                                           const uint8_t* toks, int K, int row0, int ntt, uint8_t* lds, int wave,
                                           int lane) {
  constexpr int kL = Batch<NT, WF, QW>::kLoads;
  constexpr int kW = Batch<NT, WF, QW>::kWeights;
  constexpr int kBuf = StageLayout<NT>::kBufBytes;
  const int ks = K >> 7, r = ks % 4, s1 = min(1, ks - 1), s2 = min(2, ks - 1);
  v8i a0[QW], a1[QW], a2[QW], a3[QW];
  int c0[QW], c1[QW], c2[QW], c3[QW];
  auto seq = std::make_integer_sequence<int, kL>{};
  auto wseq = std::make_integer_sequence<int, kW>{};
  auto pro = [&](v8i (&x0)[QW], int (&y0)[QW], v8i (&x1)[QW], int (&y1)[QW], v8i (&x2)[QW], int (&y2)[QW]) {
    load_slots<NT, PACKED, WF, QW, WEIGHTS_A, 0>(seq, x0, y0, wp, 0, tok, toks, ks, row0, ntt, 0, lds, wave, lane);
    load_slots<NT, PACKED, WF, QW, WEIGHTS_A, 0>(seq, x1, y1, wp, s1, tok, toks, ks, row0, ntt, s1, lds + kBuf, wave,
                                                 lane);
    load_slots<NT, PACKED, WF, QW, WEIGHTS_A, 0>(wseq, x2, y2, wp, s2, tok, toks, ks, row0, ntt, s2, lds, wave, lane);
  };
  if (r == 0)
    pro(a0, c0, a1, c1, a2, c2);
  else if (r == 1)
    pro(a3, c3, a0, c0, a1, c1);
  else if (r == 2)
    pro(a2, c2, a3, c3, a0, c0);
  else
    pro(a1, c1, a2, c2, a3, c3);
  int s = 0, cur = 0;
  if (r == 1) {
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(0, ks, 0, acc, wp, a3, c3, a2, c2, tok, toks, row0, ntt, lds, wave, lane);
    s = 1;
    cur = 1;
  } else if (r == 2) {
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(0, ks, 0, acc, wp, a2, c2, a1, c1, tok, toks, row0, ntt, lds, wave, lane);
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(1, ks, 1, acc, wp, a3, c3, a2, c2, tok, toks, row0, ntt, lds, wave, lane);
    s = 2;
    cur = 2;
  } else if (r == 3) {
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(0, ks, 0, acc, wp, a1, c1, a0, c0, tok, toks, row0, ntt, lds, wave, lane);
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(1, ks, 1, acc, wp, a2, c2, a1, c1, tok, toks, row0, ntt, lds, wave, lane);
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(2, ks, 2, acc, wp, a3, c3, a2, c2, tok, toks, row0, ntt, lds, wave, lane);
    s = 3;
    cur = 0;
  }
  for (; s < ks; s += 4) {
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(s, ks, cur, acc, wp, a0, c0, a3, c3, tok, toks, row0, ntt, lds, wave, lane);
    cur = cur == 2 ? 0 : cur + 1;
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(s + 1, ks, cur, acc, wp, a1, c1, a0, c0, tok, toks, row0, ntt, lds, wave,
                                               lane);
    cur = cur == 2 ? 0 : cur + 1;
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(s + 2, ks, cur, acc, wp, a2, c2, a1, c1, tok, toks, row0, ntt, lds, wave,
                                               lane);
    cur = cur == 2 ? 0 : cur + 1;
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(s + 3, ks, cur, acc, wp, a3, c3, a2, c2, tok, toks, row0, ntt, lds, wave,
                                               lane);
    cur = cur == 2 ? 0 : cur + 1;
  }
  wait_vmcnt<0>();
  __syncthreads();
}

// The K loop of one chunk with WPF = 1: weights of step 0 and token tiles of steps 0 and
// 1 first; if ks is odd, step 0 alone (its weight buffers then swap by copies); then
// the steps two at a time (the two weight buffers alternate, roles fixed in the
// unrolled body). Then as above.
template <int FMT, int NT, bool PACKED, bool WEIGHTS_A, int WF, int QW>
__device__ __forceinline__ void k_loop_pf1(v4f (&acc)[QW][NT], const WPtr<PACKED> (&wp)[QW], const uint8_t* tok,
                                           const uint8_t* toks, int K, int row0, int ntt, uint8_t* lds, int wave,
                                           int lane) {
  constexpr int kW = Batch<NT, WF, QW>::kWeights, kT = Batch<NT, WF, QW>::kTokens;
  constexpr int kBuf = StageLayout<NT>::kBufBytes;
  const int ks = K >> 7;
  v8i a0[QW], a1[QW];
  int c0[QW], c1[QW];
  load_slots<NT, PACKED, WF, QW, WEIGHTS_A, 0>(std::make_integer_sequence<int, kW + kT>{}, a0, c0, wp, 0, tok, toks, ks, row0, ntt, 0,
                            lds, wave, lane);
  load_slots<NT, PACKED, WF, QW, WEIGHTS_A, kW>(std::make_integer_sequence<int, kT>{}, a1, c1, wp, 0, tok, toks, ks, row0, ntt,
                             min(1, ks - 1), lds + kBuf, wave, lane);
  int s = 0, cur = 0;
  if (ks & 1) {
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(0, ks, 0, acc, wp, a0, c0, a1, c1, tok, toks, row0, ntt, lds, wave, lane);
#pragma unroll
    for (int q = 0; q < QW; ++q) {
      a0[q] = a1[q];
      c0[q] = c1[q];
    }
    s = 1;
    cur = 1;
  }
  for (; s < ks; s += 2) {
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(s, ks, cur, acc, wp, a0, c0, a1, c1, tok, toks, row0, ntt, lds, wave, lane);
    cur = cur == 2 ? 0 : cur + 1;
    k_step<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(s + 1, ks, cur, acc, wp, a1, c1, a0, c0, tok, toks, row0, ntt, lds, wave, lane);
    cur = cur == 2 ? 0 : cur + 1;
  }
  wait_vmcnt<0>();
  __syncthreads();
}

template <int FMT, int NT, bool PACKED, bool WEIGHTS_A, int WF, int QW>
__device__ __forceinline__ void k_loop(v4f (&acc)[QW][NT], const WPtr<PACKED> (&wp)[QW], const uint8_t* tok,
                                       const uint8_t* toks, int K, int row0, int ntt, uint8_t* lds, int wave,
                                       int lane) {
  if constexpr (WeightPrefetch<NT, WF>::value == 3)
    k_loop_pf3<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(acc, wp, tok, toks, K, row0, ntt, lds, wave, lane);
  else if constexpr (WeightPrefetch<NT, WF>::value == 2)
    k_loop_pf2<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(acc, wp, tok, toks, K, row0, ntt, lds, wave, lane);
  else
    k_loop_pf1<FMT, NT, PACKED, WEIGHTS_A, WF, QW>(acc, wp, tok, toks, K, row0, ntt, lds, wave, lane);
}

// Occupancy targets: small token chunks (decode) want several waves per SIMD to keep
// many weight loads in flight; 256-row chunks need the whole register file for 256
// accumulators.
template <int NT> struct WavesPerEU { static constexpr int value = NT <= 2 ? 2 : 1; };

// ---- GMM1 + activation + MX requantization --------------------------------------
template <int FMT, int NT, bool PACKED, int EPI, int WF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WavesPerEU<NT>::value)))
void gmm1_swiglu_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ sx, const uint8_t* __restrict__ w,
    const uint8_t* __restrict__ ws, const int4* __restrict__ tiles, const int* __restrict__ tile_count, int hidden,
    int inter, uint8_t* __restrict__ aq, uint8_t* __restrict__ sa, float* __restrict__ h1, ActParams act_p) {
  extern __shared__ __align__(16) uint8_t lds[];
  // wave index as a scalar: every per-wave address (LDS slots, tiles) stays in SGPRs
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int ncb = inter >> 7;                 // 128 gate channels per block
  const int n16 = (2 * inter) >> 4;            // 16-channel tiles per expert
  int it, stride, last;
  block_items(*tile_count * ncb, &it, &stride, &last);
  for (; it < last; it += stride) {
    const int j = it / ncb, cb = it - j * ncb;
    const int4 tile = tiles[j];
    const int e = tile.x, row0 = tile.y, nrows = tile.z, srow0 = tile.w;
    const int ntt = (nrows + 15) >> 4;
    const int n0 = cb * 128 + wave * 32;       // first gate channel of this wave
    WPtr<PACKED> wp[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ct = (q < 2 ? n0 : inter + n0 - 32) / 16 + q;   // q = 0,1 gate; 2,3 up
      wp[q] = weight_tile<PACKED, WF>(w, ws, (int64_t)e * n16 + ct, hidden, lane);
    }
    v4f acc[4][NT];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[q][t] = v4f{0.f, 0.f, 0.f, 0.f};
    k_loop<FMT, NT, PACKED, true, WF, 4>(acc, wp, xq, sx, hidden, row0, ntt, lds, wave, lane);

    // A^ goes out in the tiled layout with K = inter (2 inter for gelu), where this
    // block's 128 gate channels are exactly K step cb: the wave's 32 channels are half
    // wave/2 of it, lane groups 2 (wave % 2) + jj, byte 4g + i, and its MX group is
    // K-block `wave`. For gelu the up half's channels are K step cb + inter/128.
    // Every row of the tile is written: rows past the chunk are zero tokens (the tiled
    // X holds zeros there), so they requantize to code 0 and scale 0.
    const int ks2 = (EPI == kActGelu ? 2 * inter : inter) >> 7, kq2 = (ks2 + 3) >> 2;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntt) continue;                   // uniform per wave
      const int rr = 16 * t + r;
      const int64_t tl = (int64_t)(row0 >> 4) + t;
      if constexpr (EPI == kActGelu) {
        float ag[2][4], au[2][4];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ag[jj][i] = gelu_act(acc[jj][t][i]);
            au[jj][i] = gelu_act(acc[2 + jj][t][i]);
          }
        store_group<FMT>(ag, aq, sa, tl, ks2, kq2, cb, wave, g, r);
        store_group<FMT>(au, aq, sa, tl, ks2, kq2, cb + (inter >> 7), wave, g, r);
      } else {
        float a2[2][4];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            a2[jj][i] = gated_act<EPI>(acc[jj][t][i], acc[2 + jj][t][i], act_p);
        store_group<FMT>(a2, aq, sa, tl, ks2, kq2, cb, wave, g, r);
      }
      if (h1 && rr < nrows) {
        const int64_t row = srow0 + rr;
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

// ---- GMM2 ---------------------------------------------------------------------------
// O rows (sorted-row order; fp32, or bf16 with OBF16: the rows the combine receives when
// each expert's output is sent as BF16) go out with plain stores; the weighted combine
// reads them back per token (combine.hip). Combining here with fp32 atomics would send every
// add to memory: a token's K rows are computed on different XCDs, whose L2s are not
// coherent, so device-scope atomics are not resolved in L2.
// QW 16-channel weight tiles per wave: 4 (256 channels a block).
template <int NT> struct Gmm2Tiles { static constexpr int value = 4; };

template <int FMT, int NT, bool PACKED, int WF, bool OBF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WavesPerEU<NT>::value)))
void gmm2_kernel(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ sa, const uint8_t* __restrict__ w,
    const uint8_t* __restrict__ ws, const int4* __restrict__ tiles, const int* __restrict__ tile_count, int hidden,
    int inter, float* __restrict__ o, uint16_t* __restrict__ o16) {
  constexpr int QW = Gmm2Tiles<NT>::value;
  extern __shared__ __align__(16) uint8_t lds[];
  // wave index as a scalar: every per-wave address (LDS slots, tiles) stays in SGPRs
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int n16 = hidden >> 4;
  const int ncb = (n16 + 4 * QW - 1) / (4 * QW);   // 64 QW channels per block (16 QW per wave)
  int it, stride, last;
  block_items(*tile_count * ncb, &it, &stride, &last);
  for (; it < last; it += stride) {
    const int j = it / ncb, cb = it - j * ncb;
    const int4 tile = tiles[j];
    const int e = tile.x, row0 = tile.y, nrows = tile.z, srow0 = tile.w;
    const int ntt = (nrows + 15) >> 4;
    // This wave's first 16-channel tile. In the last block, tiles past hidden take the
    // last tile's weights (in bounds; the wave still stages tokens and meets the
    // barriers) and are not stored; with QW = 4 (hidden % 256 == 128) a whole wave is off.
    const int t0 = (cb * 4 + wave) * QW;
    const int nq = min(QW, n16 - t0);            // tiles of this wave inside hidden (may be <= 0)
    WPtr<PACKED> wp[QW];
#pragma unroll
    for (int q = 0; q < QW; ++q) {
      const int tq = QW == 4 ? (nq > 0 ? t0 : 0) + q : min(t0 + q, n16 - 1);
      wp[q] = weight_tile<PACKED, WF>(w, ws, (int64_t)e * n16 + tq, inter, lane);
    }
    v4f acc[QW][NT];
#pragma unroll
    for (int q = 0; q < QW; ++q)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[q][t] = v4f{0.f, 0.f, 0.f, 0.f};
    k_loop<FMT, NT, PACKED, false, WF, QW>(acc, wp, aq, sa, inter, row0, ntt, lds, wave, lane);

    // acc[q][t][i] = O[token row 16t + 4g + i][channel 16 (t0 + q) + r]
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= ntt || nq <= 0) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * t + 4 * g + i;
        if (rr >= nrows) continue;
        const int64_t at = (int64_t)(srow0 + rr) * hidden + 16 * t0 + r;
#pragma unroll
        for (int q = 0; q < QW; ++q) {
          if (QW != 4 && q >= nq) continue;      // QW = 4: a wave is all on or all off
          if constexpr (OBF16)
            o16[at + 16 * q] = f_to_bf16(acc[q][t][i]);
          else
            o[at + 16 * q] = acc[q][t][i];
        }
      }
    }
  }
}

// ---- packing of weights into the MFMA-native layout -----------------------------
// codes [G, N, K] -> packed [G][N/16][K/128][2][64][16 B]: tile (g, n16, s), half h, lane l
// holds row n16*16 + l%16, K bytes [128 s + 64 h + 16 (l/16), +16).
// scales [G, N, K/32] -> packed [G][N/16][ceil(K/512)][64][4 B]: byte j of lane l = the
// scale of row n16*16 + l%16, K block 4 (4 q + j) + l/16 (0 beyond the last K step).
__global__ void pack_codes_kernel(const uint8_t* __restrict__ codes, uint8_t* __restrict__ packed, int64_t pieces,
                                  int N, int K) {
  const int ks = K >> 7;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < pieces; p += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(p & 63);
    const int h = (int)((p >> 6) & 1);
    const int64_t blk = p >> 7;                 // (g * N/16 + n16) * ks + s
    const int s = (int)(blk % ks);
    const int64_t tile = blk / ks;              // g * N/16 + n16
    const int64_t row = tile * 16 + (l & 15);   // flat row over [G * N]
    const u32x4 v = *reinterpret_cast<const u32x4*>(codes + row * K + 128 * s + 64 * h + 16 * (l >> 4));
    reinterpret_cast<u32x4*>(packed)[p] = v;
  }
}

// MXFP4 codes [G, N, K/2] (two a byte) -> packed [G][N/16][K/128][64][16 B]: tile (g, n16, s),
// lane l holds row n16*16 + l%16, bytes [64 s + 16 (l/16), +16) of the row (K [128 s + 32 (l/16), +32)).
__global__ void pack_codes_fp4_kernel(const uint8_t* __restrict__ codes, uint8_t* __restrict__ packed,
                                      int64_t pieces, int K) {
  const int ks = K >> 7;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < pieces; p += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(p & 63);
    const int64_t blk = p >> 6;                 // (g * N/16 + n16) * ks + s
    const int s = (int)(blk % ks);
    const int64_t tile = blk / ks;
    const int64_t row = tile * 16 + (l & 15);
    const u32x4 v = *reinterpret_cast<const u32x4*>(codes + row * (K >> 1) + 64 * s + 16 * (l >> 4));
    reinterpret_cast<u32x4*>(packed)[p] = v;
  }
}

__global__ void pack_scales_kernel(const uint8_t* __restrict__ scales, uint32_t* __restrict__ packed, int64_t words,
                                   int N, int K) {
  const int ks = K >> 7, kq = (ks + 3) >> 2, kb = K >> 5;
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < words; p += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(p & 63);
    const int64_t blk = p >> 6;                 // (g * N/16 + n16) * kq + q
    const int q = (int)(blk % kq);
    const int64_t tile = blk / kq;
    const int64_t row = tile * 16 + (l & 15);
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = 4 * q + j;
      if (s < ks) word |= (uint32_t)scales[row * kb + 4 * s + (l >> 4)] << (8 * j);
    }
    packed[p] = word;
  }
}

template <int FMT, int NT, bool PACKED, int EPI, int WF>
hipError_t gmm1_go(const Gmm1Params& p, hipStream_t st) {
  auto kern = gmm1_swiglu_kernel<FMT, NT, PACKED, EPI, WF>;
  LaunchShape ls;
  hipError_t e = persistent_shape(kern, kRing * StageLayout<NT>::kBufBytes, &ls);
  if (e != hipSuccess) return e;
  kern<<<ls.grid, 256, ls.lds, st>>>(p.xq, p.sx, p.w, p.ws, p.tiles, p.tile_count, p.hidden, p.inter, p.aq, p.sa,
                                     p.h1, p.act);
  return hipGetLastError();
}

template <int FMT, int NT, bool PACKED, int WF, bool OBF16>
hipError_t gmm2_go(const Gmm2Params& p, hipStream_t st) {
  auto kern = gmm2_kernel<FMT, NT, PACKED, WF, OBF16>;
  LaunchShape ls;
  hipError_t e = persistent_shape(kern, kRing * StageLayout<NT>::kBufBytes, &ls);
  if (e != hipSuccess) return e;
  kern<<<ls.grid, 256, ls.lds, st>>>(p.aq, p.sa, p.w, p.ws, p.tiles, p.tile_count, p.hidden, p.inter, p.o, p.o16);
  return hipGetLastError();
}

template <int FMT, bool PACKED, int EPI, int WF>
hipError_t gmm1_epi(const Gmm1Params& p, hipStream_t st) {
  switch (p.tt) {
    case 1: return gmm1_go<FMT, 1, PACKED, EPI, WF>(p, st);
    case 2: return gmm1_go<FMT, 2, PACKED, EPI, WF>(p, st);
    case 4: return gmm1_go<FMT, 4, PACKED, EPI, WF>(p, st);
    case 8: return gmm1_go<FMT, 8, PACKED, EPI, WF>(p, st);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT, bool PACKED, int WF>
hipError_t gmm1_nt(const Gmm1Params& p, hipStream_t st) {
  switch (p.act.kind) {
    case 1: return gmm1_epi<FMT, PACKED, 1, WF>(p, st);
    case 2: return gmm1_epi<FMT, PACKED, 2, WF>(p, st);
    case 3: return gmm1_epi<FMT, PACKED, 3, WF>(p, st);
    case kActGelu: return gmm1_epi<FMT, PACKED, kActGelu, WF>(p, st);
    default: return gmm1_epi<FMT, PACKED, 0, WF>(p, st);
  }
}

template <int FMT, bool PACKED, int WF, bool OBF16>
hipError_t gmm2_tt(const Gmm2Params& p, hipStream_t st) {
  switch (p.tt) {
    case 1: return gmm2_go<FMT, 1, PACKED, WF, OBF16>(p, st);
    case 2: return gmm2_go<FMT, 2, PACKED, WF, OBF16>(p, st);
    case 4: return gmm2_go<FMT, 4, PACKED, WF, OBF16>(p, st);
    case 8: return gmm2_go<FMT, 8, PACKED, WF, OBF16>(p, st);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT, bool PACKED, int WF>
hipError_t gmm2_nt(const Gmm2Params& p, hipStream_t st) {
  return p.o16 ? gmm2_tt<FMT, PACKED, WF, true>(p, st) : gmm2_tt<FMT, PACKED, WF, false>(p, st);
}

}  // namespace

int gmm_token_tiles(int64_t rows, int64_t groups, int64_t hidden, int64_t inter, int64_t aw) {
  const double avg = groups > 0 ? (double)rows / (double)groups : (double)rows;
  if (avg <= 16.0) return 1;
  if (avg <= 32.0) return 2;
  if (avg <= 64.0) return 4;
  if (avg <= 128.0) return 8;
  // Experts of a few hundred rows (a prefill-shaped layer: 256 +- 16 rows per expert):
  // 320-row chunks on the LDS-streaming kernels, so that every such expert is one chunk
  // and its weights are read once.
  const bool even = (hidden / 128) % 4 == 0 && (aw / 128) % 4 == 0 && (inter / 128) % 4 == 0;
  const bool small = 2 * inter * hidden < (int64_t(1) << 31) && hidden * aw < (int64_t(1) << 31);
  return even && small ? kStreamTiles : 8;
}

// MXFP4 weights (the pages' A8W4-FP scenario) pair with E4M3 tokens only.
hipError_t launch_gmm1(const Gmm1Params& p, hipStream_t st) {
  if (p.tt == kStreamTiles) return launch_gmm1_stream(p, st);
  if (p.wfp4) {
    if (p.fmt != 0) return hipErrorInvalidValue;
    return p.packed ? gmm1_nt<0, true, kFmtFp4>(p, st) : gmm1_nt<0, false, kFmtFp4>(p, st);
  }
  if (p.fmt == 0) return p.packed ? gmm1_nt<0, true, 0>(p, st) : gmm1_nt<0, false, 0>(p, st);
  return p.packed ? gmm1_nt<1, true, 1>(p, st) : gmm1_nt<1, false, 1>(p, st);
}

hipError_t launch_gmm2(const Gmm2Params& p, hipStream_t st) {
  if (p.tt == kStreamTiles) return launch_gmm2_stream(p, st);
  if (p.wfp4) {
    if (p.fmt != 0) return hipErrorInvalidValue;
    return p.packed ? gmm2_nt<0, true, kFmtFp4>(p, st) : gmm2_nt<0, false, kFmtFp4>(p, st);
  }
  if (p.fmt == 0) return p.packed ? gmm2_nt<0, true, 0>(p, st) : gmm2_nt<0, false, 0>(p, st);
  return p.packed ? gmm2_nt<1, true, 1>(p, st) : gmm2_nt<1, false, 1>(p, st);
}

hipError_t launch_pack_weights(const uint8_t* codes, const uint8_t* scales, int64_t groups, int64_t n, int64_t k,
                               uint8_t* packed, uint8_t* packed_scales, hipStream_t st) {
  const int64_t pieces = groups * n * k / 16;
  const int64_t words = groups * (n / 16) * (((k >> 7) + 3) >> 2) * 64;
  int64_t b1 = std::min<int64_t>((pieces + 255) / 256, 65536), b2 = std::min<int64_t>((words + 255) / 256, 65536);
  if (b1 < 1) b1 = 1;
  if (b2 < 1) b2 = 1;
  pack_codes_kernel<<<(unsigned)b1, 256, 0, st>>>(codes, packed, pieces, (int)n, (int)k);
  pack_scales_kernel<<<(unsigned)b2, 256, 0, st>>>(scales, reinterpret_cast<uint32_t*>(packed_scales), words, (int)n,
                                                   (int)k);
  return hipGetLastError();
}

hipError_t launch_pack_weights_fp4(const uint8_t* codes, const uint8_t* scales, int64_t groups, int64_t n, int64_t k,
                                   uint8_t* packed, uint8_t* packed_scales, hipStream_t st) {
  const int64_t pieces = groups * n * k / 32;   // 16-byte pieces of the [G, N, K/2] codes
  const int64_t words = groups * (n / 16) * (((k >> 7) + 3) >> 2) * 64;
  int64_t b1 = std::min<int64_t>((pieces + 255) / 256, 65536), b2 = std::min<int64_t>((words + 255) / 256, 65536);
  if (b1 < 1) b1 = 1;
  if (b2 < 1) b2 = 1;
  pack_codes_fp4_kernel<<<(unsigned)b1, 256, 0, st>>>(codes, packed, pieces, (int)k);
  pack_scales_kernel<<<(unsigned)b2, 256, 0, st>>>(scales, reinterpret_cast<uint32_t*>(packed_scales), words, (int)n,
                                                   (int)k);
  return hipGetLastError();
}

}  // namespace moe
