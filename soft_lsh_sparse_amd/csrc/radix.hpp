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

// Given a 2048-bin histogram (global or LDS), find the bin holding the
// need-th largest element (need >= 1, need <= sum of bins): the bin b with
// count(> b) < need <= count(>= b). Writes b and count(> b) to out[0..1].
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

// The need-th largest (1 <= need <= number of valid values) of the values
// u[i] (where valid[i]) that the block's threads hold, PER each: a radix
// select with digits of 11, 11 and 10 bits over the 2048-bin LDS histogram
// h. scratch needs NT/64 + 3 words. Every thread gets the result. Contains
// __syncthreads().
template <int NT, int PER>
__device__ inline uint32_t block_select_nth(const uint32_t (&u)[PER], const bool (&valid)[PER],
                                            uint32_t need, uint32_t* h, uint32_t* scratch) {
  uint32_t* res = scratch + NT / 64 + 1;
  uint32_t prefix = 0;  // u >> 21, then u >> 10, of the values still in the running
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int pshift = pass == 1 ? 21 : 10;
    const uint32_t dmask = pass == 2 ? 1023u : 2047u;
    for (int i = threadIdx.x; i < kHistBins; i += NT) h[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (valid[i] && (pass == 0 || (u[i] >> pshift) == prefix))
        atomicAdd(&h[(u[i] >> shift) & dmask], 1u);
    }
    __syncthreads();
    find_threshold_bin<NT>(h, need, scratch, res);
    prefix = (prefix << (pass == 2 ? 10 : 11)) | res[0];
    need -= res[1];
  }
  return prefix;
}

}  // namespace socket_lsh
