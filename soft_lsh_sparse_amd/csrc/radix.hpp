// Block-level building blocks of the radix selects (top-k and the
// threshold estimate of the decode queries): lane prefix counts, block scans
// and the search of a 2048-bin histogram for the bin that holds the n-th
// largest element.
#pragma once

#include "common.hpp"

namespace socket_lsh {

constexpr int kHistBins = 2048;

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lane_prefix(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Exclusive scan of one uint32 per thread over the block; returns the
// thread's exclusive prefix and writes the block total to *total. Wave scans
// with DPP; the wave totals are scanned by the first wave the same way.
// `scratch` needs blockDim/64 + 1 words. Contains __syncthreads().
template <int NT>
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch,
                                                uint32_t* total) {
  constexpr int NWV = NT / 64;
  static_assert(NWV <= 64, "one wave scans the wave totals");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan_dpp(v);
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const uint32_t t = lane < NWV ? scratch[lane] : 0u;
    const uint32_t inc = wave_inclusive_scan_dpp(t);
    if (lane < NWV) scratch[lane] = inc - t;
    if (lane == 63) scratch[NWV] = inc;
  }
  __syncthreads();
  const uint32_t res = scratch[wave] + x - v;
  *total = scratch[NWV];
  __syncthreads();
  return res;
}

// Exclusive scans of two uint32 per thread over the block at once (same
// synchronisations as one); totals to *ta and *tb. `scratch` needs
// 2 * (blockDim/64 + 1) words. Contains __syncthreads().
template <int NT>
__device__ inline void block_exclusive_scan2(uint32_t a, uint32_t b, uint32_t* scratch,
                                             uint32_t* ea, uint32_t* eb, uint32_t* ta,
                                             uint32_t* tb) {
  constexpr int NWV = NT / 64;
  static_assert(NWV <= 64, "one wave scans the wave totals");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t* sa = scratch;
  uint32_t* sb = scratch + NWV + 1;
  const uint32_t xa = wave_inclusive_scan_dpp(a), xb = wave_inclusive_scan_dpp(b);
  if (lane == 63) {
    sa[wave] = xa;
    sb[wave] = xb;
  }
  __syncthreads();
  if (wave == 0) {
    const uint32_t va = lane < NWV ? sa[lane] : 0u, vb = lane < NWV ? sb[lane] : 0u;
    const uint32_t ia = wave_inclusive_scan_dpp(va), ib = wave_inclusive_scan_dpp(vb);
    if (lane < NWV) {
      sa[lane] = ia - va;
      sb[lane] = ib - vb;
    }
    if (lane == 63) {
      sa[NWV] = ia;
      sb[NWV] = ib;
    }
  }
  __syncthreads();
  *ea = sa[wave] + xa - a;
  *eb = sb[wave] + xb - b;
  *ta = sa[NWV];
  *tb = sb[NWV];
  __syncthreads();
}

// Given a 2048-bin histogram (global or LDS), find the bin holding the
// need-th largest element (need >= 1): the bin b with count(> b) < need <=
// count(>= b). Writes b, count(> b) and the sum of the bins to out[0..2]
// (out[0..1] stay 0 when the bins hold fewer than need elements).
template <int NT>
__device__ inline void find_threshold_bin(const uint32_t* bins, uint32_t need,
                                   uint32_t* scratch, uint32_t* out) {
  constexpr int PER = kHistBins / NT;
  if (threadIdx.x == 0) {
    out[0] = 0;
    out[1] = 0;
  }
  // thread t owns bins 2047 - (t*PER + i), i.e. bins in descending order
  uint32_t cnt[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    cnt[i] = bins[kHistBins - 1 - (threadIdx.x * PER + i)];
    sum += cnt[i];
  }
  uint32_t total;
  uint32_t run = block_exclusive_scan<NT>(sum, scratch, &total);
  if (threadIdx.x == 0) out[2] = total;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (run < need && run + cnt[i] >= need) {
      out[0] = kHistBins - 1 - (threadIdx.x * PER + i);
      out[1] = run;
    }
    run += cnt[i];
  }
  __syncthreads();
}

}  // namespace socket_lsh
