// Routing on gfx950: stable counting sort of the flattened expert ids.
//
// MoeInitRoutingV3 README, 计算公式 1-3 and 6: keyValueSort(expertIdx, rowIdx), the
// inverse scatter expandedRowIdx[sortedRowIdx[i]] = i, the per-expert histogram, and
// availableIdxNum = number of ids inside the active expert range. moe_token_permute
// article, 功能说明 / 确定性计算: the sort is stable, so ties keep ascending flat row.
//
// Expert ids are small integers (E <= 10240), so the sort is a three-pass counting
// sort instead of a comparison sort:
//   1. route_count   one workgroup per chunk of flat rows, LDS histogram over the
//                    active experts, written expert-major (hist[a][c]);
//   2. route_scan    one wave per expert: exclusive scan of its row counts over the
//                    chunks (base[a][c] = rows of expert a in chunks < c) and its total;
//      route_offsets one workgroup: exclusive scan of the totals over the experts
//                    (offsets, per-expert counts / cumsum, availableIdxNum). The first
//                    sorted position of (chunk c, expert a) is offsets[a] + base[a][c].
//                    When the histogram fits in LDS (A * chunks <= kFusedScan) both run
//                    as one workgroup (route_scan_fused), one launch instead of two;
//   3. route_scatter one wave per chunk walks its rows in order, 64 at a time. The rank
//                    of a row among the earlier lanes with the same expert comes from a
//                    bit-sliced match: one ballot per bit of the expert id, AND-ed per
//                    lane (bit set ? ballot : ~ballot), then mbcnt below the lane. An LDS
//                    cursor per expert carries the running position across steps.
// Block path, for chunks of up to 1024 rows over at most 512 active experts: one thread
// per row in both passes (route_count_block, route_scatter_block), each wave ranking its
// 64 rows at once, per-wave counts scanned over the waves in LDS; when the histogram is
// small (at most 64 chunks, or at most two experts per wave) the scatter pass also
// derives its chunk's first positions from it, so the scan pass disappears (two
// launches in all).
// Positions are relative to the start of the active segment [s, e).

#include <climits>

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

template <typename KeyT>
__global__ __launch_bounds__(256) void route_count(const KeyT* __restrict__ keys, int64_t flat, int s,
                                                   int A, int chunk, int* __restrict__ hist) {
  extern __shared__ int lds_hist[];
  const int c = blockIdx.x;
  for (int a = threadIdx.x; a < A; a += blockDim.x) lds_hist[a] = 0;
  __syncthreads();
  const int64_t lo = (int64_t)c * chunk;
  const int64_t hi = min(flat, lo + chunk);
  for (int64_t r = lo + threadIdx.x; r < hi; r += blockDim.x) {
    const int64_t a = (int64_t)keys[r] - s;
    if (a >= 0 && a < A) atomicAdd(&lds_hist[a], 1);
  }
  __syncthreads();
  for (int a = threadIdx.x; a < A; a += blockDim.x) hist[(int64_t)a * gridDim.x + c] = lds_hist[a];
}

// Inclusive scan (sum, or max when MAX) of one int per thread over a 1024-thread block:
// a shuffle scan within each wave, a scan of the 16 wave totals by wave 0, then each
// wave adds the totals before it (three barriers). Leaves every thread's inclusive value
// in part[t] (the block total in part[1023]) for the callers that read another thread's.
template <bool MAX = false>
__device__ int block_inclusive_scan_1024(int v, int* part) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  constexpr int kId = MAX ? INT_MIN : 0;
  auto op = [](int a, int b) { return MAX ? max(a, b) : a + b; };
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x = op(x, y);
  }
  if (lane == 63) part[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? part[lane] : kId;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int y = __shfl_up(w, d);
      if (lane >= d) w = op(w, y);
    }
    if (lane < 16) part[lane] = w;
  }
  __syncthreads();
  if (wave > 0) x = op(part[wave - 1], x);
  __syncthreads();   // every read of the wave totals is done before part is overwritten
  part[t] = x;
  __syncthreads();
  return x;
}

// Exclusive scan of one expert's chunk counts (one wave per expert, 64 chunks per step,
// shuffle scan within the wave, the running total carried across steps).
__global__ __launch_bounds__(64) void route_scan(const int* __restrict__ hist, int nch, int* __restrict__ base,
                                                 int* __restrict__ totals) {
  const int a = blockIdx.x, lane = threadIdx.x;
  const int* h = hist + (int64_t)a * nch;
  int* b = base + (int64_t)a * nch;
  int carry = 0;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int c = c0 + lane;
    const int v = c < nch ? h[c] : 0;
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int x = __shfl_up(incl, d);
      if (lane >= d) incl += x;
    }
    if (c < nch) b[c] = carry + incl - v;
    carry += __shfl(incl, 63);
  }
  if (lane == 0) totals[a] = carry;
}

// Exclusive scan over the experts of the totals held by every thread in tot[a0, a1)
// (the thread's contiguous share), writing the routing summaries. part: 1024 ints.
__device__ void offsets_from_totals(const int* tot, int A, int* part, int* __restrict__ offsets, int64_t* avail64,
                                    int64_t* expert_tokens, int tokens_type, int32_t* token_nums32) {
  const int t = threadIdx.x;
  const int P = (A + 1023) / 1024;
  const int a0 = min(A, t * P), a1 = min(A, a0 + P);
  int sum = 0;
  for (int a = a0; a < a1; ++a) sum += tot[a];
  const int incl = block_inclusive_scan_1024(sum, part);
  int run = incl - sum;
  for (int a = a0; a < a1; ++a) {
    const int cnt = tot[a];
    offsets[a] = run;
    run += cnt;
    if (expert_tokens) expert_tokens[a] = tokens_type == 1 ? (int64_t)cnt : (int64_t)run;
    if (token_nums32) token_nums32[a] = cnt;
  }
  if (t == 1023) {
    offsets[A] = part[1023];
    if (avail64) *avail64 = part[1023];
  }
}

constexpr int kFusedScan = 14336;   // ints (histogram + totals) route_scan_fused holds in LDS (56 KB)

// route_scan + route_offsets in one workgroup of 16 waves: the histogram is loaded into
// LDS with coalesced loads; each expert's chunk counts are scanned by one thread (32 or
// fewer chunks) or one wave (experts wave, wave + 16, ...); then the totals are scanned
// over the experts.
__global__ __launch_bounds__(1024) void route_scan_fused(const int* __restrict__ hist, int nch, int A,
                                                         int* __restrict__ base, int* __restrict__ offsets,
                                                         int64_t* avail64, int64_t* expert_tokens, int tokens_type,
                                                         int32_t* token_nums32) {
  __shared__ int part[1024];
  extern __shared__ int lds[];   // hist [A * nch], then totals [A]
  int* tot = lds + A * nch;
  const int L = A * nch;
  for (int j = threadIdx.x; j < L; j += 1024) lds[j] = hist[j];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (nch <= 32) {   // few chunks: one thread per expert walks its chunk counts
    for (int a = threadIdx.x; a < A; a += 1024) {
      const int* h = lds + a * nch;
      int* b = base + (int64_t)a * nch;
      int run = 0;
      for (int c = 0; c < nch; ++c) {
        b[c] = run;
        run += h[c];
      }
      tot[a] = run;
    }
  }
  for (int a = nch <= 32 ? A : wave; a < A; a += 16) {
    const int* h = lds + a * nch;
    int* b = base + (int64_t)a * nch;
    int carry = 0;
    for (int c0 = 0; c0 < nch; c0 += 64) {
      const int c = c0 + lane;
      const int v = c < nch ? h[c] : 0;
      int incl = v;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int x = __shfl_up(incl, d);
        if (lane >= d) incl += x;
      }
      if (c < nch) b[c] = carry + incl - v;
      carry += __shfl(incl, 63);
    }
    if (lane == 0) tot[a] = carry;
  }
  __syncthreads();
  offsets_from_totals(tot, A, part, offsets, avail64, expert_tokens, tokens_type, token_nums32);
}

__global__ __launch_bounds__(1024) void route_offsets(const int* __restrict__ totals, int A, int* __restrict__ offsets,
                                                      int64_t* avail64, int64_t* expert_tokens, int tokens_type,
                                                      int32_t* token_nums32) {
  __shared__ int part[1024];
  offsets_from_totals(totals, A, part, offsets, avail64, expert_tokens, tokens_type, token_nums32);
}

template <typename KeyT>
__global__ __launch_bounds__(64) void route_scatter(
    const KeyT* __restrict__ keys, int64_t flat, int topk, int s, int A, int nbits, int chunk,
    const int* __restrict__ base, const int* __restrict__ offsets, int32_t* __restrict__ scat,
    int32_t* __restrict__ gath, int32_t* __restrict__ gath_fill, int32_t* __restrict__ row_token,
    float* __restrict__ row_weight, const void* __restrict__ topk_w, int topk_w_bf16) {
  extern __shared__ int cursor[];  // A
  const int c = blockIdx.x;
  const int lane = threadIdx.x;
  for (int a = lane; a < A; a += 64) cursor[a] = offsets[a] + base[(int64_t)a * gridDim.x + c];
  __syncthreads();
  const int64_t lo = (int64_t)c * chunk;
  const int64_t hi = min(flat, lo + chunk);
  // The keys of 16 steps (1024 rows) are loaded before they are walked, so the walk
  // pays the memory latency once per 1024 rows instead of once per 64.
  constexpr int kPre = 16;
  for (int64_t r1 = lo; r1 < hi; r1 += 64 * kPre) {
    int ak[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int64_t r = r1 + 64 * u + lane;
      int a = A;  // sentinel for rows outside the active range (and past the end)
      if (r < hi) {
        const int64_t d = (int64_t)keys[r] - s;
        if (d >= 0 && d < A) a = (int)d;
      }
      ak[u] = a;
    }
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int64_t r0 = r1 + 64 * u;
      if (r0 >= hi) break;   // uniform
      const int64_t r = r0 + lane;
      const bool valid = r < hi;
      const int a = ak[u];
      const bool act = a < A;
      uint64_t match = __ballot(act);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = (a >> b) & 1;
        const uint64_t bal = __ballot(bit);
        match &= bit ? bal : ~bal;
      }
      const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(match >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)match, 0));
      const int total = __popcll(match);
      int pos = -1;
      if (act) pos = cursor[a] + rank;
      // Within one wave LDS accesses complete in program order: every lane has read its
      // cursor before the last lane of each expert advances it.
      if (act && rank == total - 1) cursor[a] = pos + 1;
      if (valid) scat[r] = pos;
      if (act) {
        if (gath) gath[pos] = (int32_t)r;
        if (row_token) row_token[pos] = (int32_t)(r / topk);
        if (row_weight) {
          float w;
          if (topk_w_bf16) w = bf16_to_f(reinterpret_cast<const uint16_t*>(topk_w)[r]);
          else w = reinterpret_cast<const float*>(topk_w)[r];
          row_weight[pos] = w;
        }
      }
    }
  }
  if (gath_fill) {
    const int avail = offsets[A];
    for (int64_t p = avail + (int64_t)c * 64 + lane; p < flat; p += (int64_t)gridDim.x * 64) gath_fill[p] = -1;
  }
}

// ---- block path: chunks of at most 1024 rows over at most 512 active experts -------
// One thread per row. Each wave ranks its 64 rows by expert with the bit-sliced match
// of route_scatter (rank = matching lanes below, count = matching lanes); per-wave
// counts of every expert go to LDS ([waves][A]).
constexpr int kBlockMaxActive = 512;
// Histogram entries (A * chunks) up to which the scatter pass may derive its chunk's
// first positions from the histogram itself instead of a separate scan pass.
constexpr int kScanInScatter = 16384;
// Chunk counts per expert up to which one thread walks them in global memory (beyond:
// one wave per expert, 64 chunk counts a step and a shuffle reduction). Counts staged in
// LDS are always walked by one thread per expert.
constexpr int kThreadScan = 64;

// Dynamic LDS of the block path's scatter pass: per-wave counts [waves][A], first
// positions [A], totals [A], wave sums [waves + 1].
size_t scatter_lds(int A, int chunk) {
  return sizeof(int) * ((size_t)(chunk / 64) * A + (size_t)2 * A + chunk / 64 + 1);
}

// Whether the scanning scatter pass stages the chunk counts in LDS (16-bit each, the
// histogram's [A][nch] layout) after those buffers: for 17-64 chunks (the walks of up to
// 16 chunks read global memory about as fast; longer LDS walks are latency-bound, where
// one wave per expert reads global memory faster), when all of it stays within 64 KB.
__host__ __device__ inline bool scatter_stages(int A, int nch, int nw) {
  const int64_t base = (int64_t)4 * ((int64_t)nw * A + 2 * A + nw + 1);
  return nch > 16 && nch <= 64 && base + (int64_t)2 * A * nch <= 65536;
}

template <typename KeyT>
__device__ __forceinline__ void block_rank(const KeyT* __restrict__ keys, int64_t r, bool valid, int s, int A,
                                           int nbits, int* a_out, int* rank_out, int* count_out) {
  int a = A;  // sentinel for rows outside the active range (and past the end)
  if (valid) {
    const int64_t d = (int64_t)keys[r] - s;
    if (d >= 0 && d < A) a = (int)d;
  }
  uint64_t match = __ballot(a < A);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (a >> b) & 1;
    const uint64_t bal = __ballot(bit);
    match &= bit ? bal : ~bal;
  }
  *a_out = a;
  *rank_out = __builtin_amdgcn_mbcnt_hi((uint32_t)(match >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)match, 0));
  *count_out = __popcll(match);
}

// Counting pass of the block path: hist[a][c] = sum over the waves of their counts.
template <typename KeyT>
__global__ __launch_bounds__(1024) void route_count_block(const KeyT* __restrict__ keys, int64_t flat, int s, int A,
                                                          int nbits, int chunk, int* __restrict__ hist) {
  extern __shared__ int wcnt[];  // [waves][A]
  const int nw = blockDim.x >> 6;
  const int c = blockIdx.x, tid = threadIdx.x, wave = tid >> 6;
  for (int i = tid; i < nw * A; i += blockDim.x) wcnt[i] = 0;
  const int64_t r = (int64_t)c * chunk + tid;
  int a, rank, cnt;
  block_rank(keys, r, tid < chunk && r < flat, s, A, nbits, &a, &rank, &cnt);
  __syncthreads();
  if (a < A && rank == cnt - 1) wcnt[wave * A + a] = cnt;
  __syncthreads();
  for (int ex = tid; ex < A; ex += blockDim.x) {
    int sum = 0;
    for (int w = 0; w < nw; ++w) sum += wcnt[w * A + ex];
    hist[(int64_t)ex * gridDim.x + c] = sum;
  }
}

// Scatter pass of the block path. The chunk's first position of expert a is
// offsets[a] + base[a][c]; with SCAN the workgroup derives both from the histogram
// (rows of a in chunks < c, one thread or one wave per expert; exclusive scan of the
// per-expert totals),
// and workgroup 0 writes the routing summaries route_scan_fused would. The per-wave
// counts are then turned into per-wave first positions by a scan over the waves.
template <typename KeyT, bool SCAN>
__global__ __launch_bounds__(1024) void route_scatter_block(
    const KeyT* __restrict__ keys, int64_t flat, int topk, int s, int A, int nbits, int chunk,
    const int* __restrict__ hist, const int* __restrict__ base, int* __restrict__ offsets, int64_t* avail64,
    int64_t* expert_tokens, int tokens_type, int32_t* token_nums32, int32_t* __restrict__ scat,
    int32_t* __restrict__ gath, int32_t* __restrict__ gath_fill, int32_t* __restrict__ row_token,
    float* __restrict__ row_weight, const void* __restrict__ topk_w, int topk_w_bf16) {
  extern __shared__ int sh[];
  const int nw = blockDim.x >> 6;
  int* wcnt = sh;              // [waves][A]: counts, then first positions
  int* pre = wcnt + nw * A;    // [A] first position of (this chunk, expert)
  int* tot = pre + A;          // [A] rows per expert (SCAN)
  int* part = tot + A;         // [waves + 1] scan of the per-thread sums (SCAN)
  const int c = blockIdx.x, nch = gridDim.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < nw * A; i += blockDim.x) wcnt[i] = 0;
  const int64_t r = (int64_t)c * chunk + tid;
  const bool valid = tid < chunk && r < flat;
  int a, rank, cnt;
  block_rank(keys, r, valid, s, A, nbits, &a, &rank, &cnt);
  const bool act = a < A;
  int avail;
  if constexpr (SCAN) {
    // The chunk counts (each at most the chunk's 1024 rows) into LDS as 16-bit values when
    // they fit (scatter_stages); the walks below then read LDS instead of waiting on one
    // global load after another.
    const bool staged = scatter_stages(A, nch, nw);
    uint16_t* hl = reinterpret_cast<uint16_t*>(part + nw + 1);
    if (staged) {   // flat copy, eight loads in flight per thread
      const int n = A * nch;
      for (int i0 = 0; i0 < n; i0 += 8 * (int)blockDim.x) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * (int)blockDim.x + tid;
          v[u] = i < n ? hist[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * (int)blockDim.x + tid;
          if (i < n) hl[i] = (uint16_t)v[u];
        }
      }
      __syncthreads();
      // one thread per expert walks its row, starting at chunk ex % nch so that the threads
      // of a wave read different banks (the sums do not depend on the order)
      for (int ex = tid; ex < A; ex += blockDim.x) {
        const uint16_t* h = hl + ex * nch;
        int before = 0, total = 0;
        int cc = ex % nch;
        for (int j = 0; j < nch; ++j) {
          const int v = h[cc];
          total += v;
          if (cc < c) before += v;
          cc = cc + 1 == nch ? 0 : cc + 1;
        }
        pre[ex] = before;
        tot[ex] = total;
      }
    } else if (nch <= kThreadScan) {   // one thread per expert walks its chunk counts
      for (int ex = tid; ex < A; ex += blockDim.x) {
        const int* h = hist + (int64_t)ex * nch;
        int before = 0, total = 0;
        for (int cc = 0; cc < nch; ++cc) {
          const int v = h[cc];
          total += v;
          if (cc < c) before += v;
        }
        pre[ex] = before;
        tot[ex] = total;
      }
    } else {   // one wave per expert
      for (int ex = wave; ex < A; ex += nw) {
        const int* h = hist + (int64_t)ex * nch;
        int before = 0, total = 0;
        for (int cc = lane; cc < nch; cc += 64) {
          const int v = h[cc];
          total += v;
          if (cc < c) before += v;
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
          before += __shfl_xor(before, d);
          total += __shfl_xor(total, d);
        }
        if (lane == 0) {
          pre[ex] = before;
          tot[ex] = total;
        }
      }
    }
    __syncthreads();
    // exclusive scan of the totals over the experts: thread t takes experts [a0, a1)
    const int P = (A + blockDim.x - 1) / blockDim.x;
    const int a0 = min(A, tid * P), a1 = min(A, a0 + P);
    int sum = 0;
    for (int e = a0; e < a1; ++e) sum += tot[e];
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int x = __shfl_up(incl, d);
      if (lane >= d) incl += x;
    }
    if (lane == 63) part[wave] = incl;
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int w = 0; w < nw; ++w) {
        const int v = part[w];
        part[w] = run;
        run += v;
      }
      part[nw] = run;
    }
    __syncthreads();
    int run = part[wave] + incl - sum;
    for (int e = a0; e < a1; ++e) {
      const int n_e = tot[e];
      pre[e] += run;
      if (c == 0) {
        offsets[e] = run;
        if (expert_tokens) expert_tokens[e] = tokens_type == 1 ? (int64_t)n_e : (int64_t)(run + n_e);
        if (token_nums32) token_nums32[e] = n_e;
      }
      run += n_e;
    }
    avail = part[nw];
    if (c == 0 && tid == 0) {
      offsets[A] = avail;
      if (avail64) *avail64 = avail;
    }
  } else {
    for (int ex = tid; ex < A; ex += blockDim.x) pre[ex] = offsets[ex] + base[(int64_t)ex * nch + c];
    avail = offsets[A];
  }
  __syncthreads();
  if (act && rank == cnt - 1) wcnt[wave * A + a] = cnt;
  __syncthreads();
  for (int ex = tid; ex < A; ex += blockDim.x) {
    int run = pre[ex];
    for (int w = 0; w < nw; ++w) {
      const int v = wcnt[w * A + ex];
      wcnt[w * A + ex] = run;
      run += v;
    }
  }
  __syncthreads();
  const int pos = act ? wcnt[wave * A + a] + rank : -1;
  if (valid) scat[r] = pos;
  if (act) {
    if (gath) gath[pos] = (int32_t)r;
    if (row_token) row_token[pos] = (int32_t)(r / topk);
    if (row_weight) {
      float w;
      if (topk_w_bf16) w = bf16_to_f(reinterpret_cast<const uint16_t*>(topk_w)[r]);
      else w = reinterpret_cast<const float*>(topk_w)[r];
      row_weight[pos] = w;
    }
  }
  if (gath_fill)
    for (int64_t p = avail + (int64_t)c * blockDim.x + tid; p < flat; p += (int64_t)nch * blockDim.x)
      gath_fill[p] = -1;
}

template <typename KeyT>
hipError_t routing_block_path(const RouteParams& p, int A, int nbits, hipStream_t stream) {
  const KeyT* keys = (const KeyT*)p.keys;
  const size_t wl = sizeof(int) * (size_t)(p.chunk / 64) * (size_t)A;
  route_count_block<KeyT><<<p.nch, p.chunk, wl, stream>>>(keys, p.flat, p.s, A, nbits, p.chunk, p.hist);
  // in-kernel scan only where it is short: at most 64 chunk counts per thread (thread per
  // expert) or at most two experts per wave (wave per expert)
  const bool scan_here = (p.nch <= 64 && (int64_t)A * p.nch <= kScanInScatter) || A <= 2 * (p.chunk / 64);
  const size_t sl = scatter_lds(A, p.chunk);
  if (scan_here) {
    const size_t sls = sl + (scatter_stages(A, p.nch, p.chunk / 64) ? (size_t)2 * A * p.nch : 0);
    route_scatter_block<KeyT, true><<<p.nch, p.chunk, sls, stream>>>(
        keys, p.flat, p.topk, p.s, A, nbits, p.chunk, p.hist, p.base, p.offsets, p.avail64, p.expert_tokens,
        p.tokens_type, p.token_nums32, p.scat, p.gath, p.gath_fill, p.row_token, p.row_weight, p.topk_w,
        p.topk_w_bf16);
    return hipGetLastError();
  }
  if ((int64_t)A * p.nch + A + 1 <= kFusedScan) {
    route_scan_fused<<<1, 1024, sizeof(int) * ((size_t)A * p.nch + A + 1), stream>>>(
        p.hist, p.nch, A, p.base, p.offsets, p.avail64, p.expert_tokens, p.tokens_type, p.token_nums32);
  } else {
    route_scan<<<A, 64, 0, stream>>>(p.hist, p.nch, p.base, p.totals);
    route_offsets<<<1, 1024, 0, stream>>>(p.totals, A, p.offsets, p.avail64, p.expert_tokens, p.tokens_type,
                                          p.token_nums32);
  }
  route_scatter_block<KeyT, false><<<p.nch, p.chunk, sl, stream>>>(
      keys, p.flat, p.topk, p.s, A, nbits, p.chunk, p.hist, p.base, p.offsets, p.avail64, p.expert_tokens,
      p.tokens_type, p.token_nums32, p.scat, p.gath, p.gath_fill, p.row_token, p.row_weight, p.topk_w,
      p.topk_w_bf16);
  return hipGetLastError();
}

// key_value form of the per-expert counts (MoeInitRoutingV3 README, expertTokensNumType
// 2): rows (expert id, count) of the active experts with a non-zero count, ascending,
// then zero rows up to `rows` (one workgroup; thread t takes a contiguous share of the
// experts, a block scan of the non-zero flags gives each row's place).
__global__ __launch_bounds__(1024) void route_key_value(const int* __restrict__ offsets, int A, int s, int rows,
                                                        int64_t* __restrict__ out) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int P = (A + 1023) / 1024;
  const int a0 = min(A, t * P), a1 = min(A, a0 + P);
  int nz = 0;
  for (int a = a0; a < a1; ++a) nz += offsets[a + 1] > offsets[a];
  const int incl = block_inclusive_scan_1024(nz, part);
  int row = incl - nz;
  for (int a = a0; a < a1; ++a) {
    const int cnt = offsets[a + 1] - offsets[a];
    if (cnt > 0 && row < rows) {
      out[2 * (int64_t)row] = s + a;
      out[2 * (int64_t)row + 1] = cnt;
      ++row;
    }
  }
  for (int r = part[1023] + t; r < rows; r += 1024) {
    out[2 * (int64_t)r] = 0;
    out[2 * (int64_t)r + 1] = 0;
  }
}

// Offsets are clamped into [0, rows] and made non-decreasing, and at most max_tiles
// tiles are written, so caller-given offsets can never send a GEMM out of bounds.
// Each group is padded to whole 16-row tiles in the tiled token layout: its padded
// start is the sum of the padded sizes of the groups before it.
// One 1024-thread workgroup; returns the number of chunks written (block-uniform).
__device__ int build_tiles_block(const int* __restrict__ offsets, int G, int rows, int tm, int max_tiles,
                                 int4* __restrict__ tiles, int* part) {
  const int t = threadIdx.x;
  const int P = (G + 1023) / 1024;
  const int g0 = min(G, t * P), g1 = min(G, g0 + P);
  auto off = [&](int g) { return min(max(offsets[g], 0), rows); };
  // start of this thread's first group: max of the clamped offsets [0, g0]
  int local = 0;
  for (int g = g0; g < g1; ++g) local = max(local, off(g));
  block_inclusive_scan_1024<true>(local, part);
  const int before = t > 0 ? part[t - 1] : 0;
  __syncthreads();
  const int start = g0 < g1 ? max(before, off(g0)) : 0;
  int ntiles = 0, npad = 0;
  int prev = start;
  for (int g = g0; g < g1; ++g) {
    const int nxt = max(prev, off(g + 1));
    ntiles += (nxt - prev + tm - 1) / tm;
    npad += (nxt - prev + 15) & ~15;
    prev = nxt;
  }
  const int tiles_incl = block_inclusive_scan_1024(ntiles, part);
  const int total = part[1023];
  __syncthreads();
  const int pad_incl = block_inclusive_scan_1024(npad, part);
  int run = tiles_incl - ntiles;
  int pad = pad_incl - npad;
  prev = start;
  for (int g = g0; g < g1; ++g) {
    const int nxt = max(prev, off(g + 1));
    const int cnt = nxt - prev;
    for (int i = 0; i * tm < cnt; ++i) {
      if (run < max_tiles) tiles[run] = make_int4(g, pad + i * tm, min(tm, cnt - i * tm), prev + i * tm);
      ++run;
    }
    pad += (cnt + 15) & ~15;
    prev = nxt;
  }
  return min(total, max_tiles);
}

__global__ __launch_bounds__(1024) void build_tiles_kernel(const int* __restrict__ offsets, int G, int rows, int tm,
                                                           int max_tiles, int4* __restrict__ tiles,
                                                           int* __restrict__ count) {
  __shared__ int part[1024];
  const int n = build_tiles_block(offsets, G, rows, tm, max_tiles, tiles, part);
  if (threadIdx.x == 0) *count = n;
}

// Chunks c < nt of one group over `rows` rows in chunks of tm rows: {group, prow0 + c tm,
// rows in the chunk, srow0 + c tm}, written to out[c].
__device__ void group_chunks(int rows, int tm, int group, int prow0, int srow0, int4* __restrict__ out) {
  const int nt = (rows + tm - 1) / tm;
  for (int c = threadIdx.x; c < nt; c += blockDim.x)
    out[c] = make_int4(group, prow0 + c * tm, min(tm, rows - c * tm), srow0 + c * tm);
}

// One wave: a stable split of chunks[0, n) by the token tiles a wave needs, ceil(tiles /
// 4), into the classes of kStreamClassRT (class c at out + c stride, out_count[c]).
__device__ void split_chunks_wave(const int4* __restrict__ chunks, int n, int stride, int4* __restrict__ out,
                                  int* __restrict__ out_count) {
  const int lane = threadIdx.x & 63;
  int base[kStreamClasses] = {};
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    const bool valid = i < n;
    const int4 c = valid ? chunks[i] : make_int4(0, 0, 0, 0);
    const int rt = (((c.z + 15) >> 4) + 3) >> 2;
    int cls = kStreamClasses - 1;
#pragma unroll
    for (int k = kStreamClasses - 2; k >= 0; --k)
      if (rt <= kStreamClassRT[k]) cls = k;
#pragma unroll
    for (int k = 0; k < kStreamClasses; ++k) {
      const uint64_t m = __ballot(valid && cls == k);
      if (valid && cls == k) out[k * stride + base[k] + __popcll(m & ((1ull << lane) - 1))] = c;
      base[k] += __popcll(m);
    }
  }
  if (lane == 0)
    for (int k = 0; k < kStreamClasses; ++k) out_count[k] = base[k];
}

// All chunk lists of one layer call in one workgroup (see ChunkListParams).
__global__ __launch_bounds__(1024) void chunk_lists_kernel(ChunkListParams p) {
  __shared__ int part[1024];
  const int routed = build_tiles_block(p.offsets, p.groups, p.rows, p.tm, p.max_tiles, p.tiles, part);
  if (threadIdx.x == 0) *p.count = routed;
  int all = routed;
  if (p.count_all) {   // the folded shared expert's chunks right after the routed ones
    group_chunks(p.sh_rows, p.sh_tm, p.sh_group, p.sh_prow0, p.sh_srow0, p.tiles + routed);
    all = routed + (p.sh_rows + p.sh_tm - 1) / p.sh_tm;
    if (threadIdx.x == 0) *p.count_all = all;
  }
  if (p.sh_tiles) {    // the shared expert's own list: rows [0, sh_rows) of group 0
    group_chunks(p.sh_rows, p.sh_tm, 0, 0, 0, p.sh_tiles);
    if (threadIdx.x == 0) *p.sh_count = (p.sh_rows + p.sh_tm - 1) / p.sh_tm;
  }
  if (p.cls_tiles) {
    __syncthreads();   // the chunk list above is written by the whole workgroup, read by wave 0
    if (threadIdx.x < 64) split_chunks_wave(p.tiles, min(all, p.cls_stride), p.cls_stride, p.cls_tiles, p.cls_count);
  }
}

}  // namespace

hipError_t launch_routing(const RouteParams& p, hipStream_t stream) {
  const int A = p.e - p.s;
  int nbits = 0;
  while ((1 << nbits) <= A) ++nbits;  // bits of the sentinel value A
  if (A >= 1 && A <= kBlockMaxActive && p.chunk <= 1024)
    return p.key_is64 ? routing_block_path<int64_t>(p, A, nbits, stream)
                      : routing_block_path<int32_t>(p, A, nbits, stream);
  const size_t lds_a = sizeof(int) * (size_t)(A > 0 ? A : 1);
  if (A > 0) {
    if (p.key_is64)
      route_count<int64_t><<<p.nch, 256, lds_a, stream>>>((const int64_t*)p.keys, p.flat, p.s, A, p.chunk, p.hist);
    else
      route_count<int32_t><<<p.nch, 256, lds_a, stream>>>((const int32_t*)p.keys, p.flat, p.s, A, p.chunk, p.hist);
  }
  if ((int64_t)A * p.nch + A + 1 <= kFusedScan) {
    route_scan_fused<<<1, 1024, sizeof(int) * ((size_t)A * p.nch + A + 1), stream>>>(
        p.hist, p.nch, A, p.base, p.offsets, p.avail64, p.expert_tokens, p.tokens_type, p.token_nums32);
  } else {
    route_scan<<<A, 64, 0, stream>>>(p.hist, p.nch, p.base, p.totals);
    route_offsets<<<1, 1024, 0, stream>>>(p.totals, A, p.offsets, p.avail64, p.expert_tokens, p.tokens_type,
                                          p.token_nums32);
  }
  if (p.key_is64)
    route_scatter<int64_t><<<p.nch, 64, lds_a, stream>>>(
        (const int64_t*)p.keys, p.flat, p.topk, p.s, A, nbits, p.chunk, p.base, p.offsets, p.scat, p.gath,
        p.gath_fill, p.row_token, p.row_weight, p.topk_w, p.topk_w_bf16);
  else
    route_scatter<int32_t><<<p.nch, 64, lds_a, stream>>>(
        (const int32_t*)p.keys, p.flat, p.topk, p.s, A, nbits, p.chunk, p.base, p.offsets, p.scat, p.gath,
        p.gath_fill, p.row_token, p.row_weight, p.topk_w, p.topk_w_bf16);
  return hipGetLastError();
}

hipError_t launch_key_value(const int* offsets, int active, int s, int rows, int64_t* out, hipStream_t stream) {
  route_key_value<<<1, 1024, 0, stream>>>(offsets, active, s, rows, out);
  return hipGetLastError();
}

hipError_t launch_chunk_lists(const ChunkListParams& p, hipStream_t stream) {
  chunk_lists_kernel<<<1, 1024, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_build_tiles(const int* offsets, int groups, int rows, int tm, int max_tiles, int4* tiles,
                              int* count, hipStream_t stream) {
  build_tiles_kernel<<<1, 1024, 0, stream>>>(offsets, groups, rows, tm, max_tiles, tiles, count);
  return hipGetLastError();
}

}  // namespace moe
