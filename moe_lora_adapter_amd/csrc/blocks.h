// Block lookup shared by the fused kernels: the align outputs give, per
// slot, num_tokens_post_padded / block_m blocks; blocks are numbered over all
// slots in slot order.
#pragma once

#include "common.h"
#include "internal.h"

namespace mlr {

// Number of blocks over all slots (every lane gets it).
__device__ __forceinline__ int count_blocks(const FusedParams& p) {
  int run = 0;
  for (int c0 = 0; c0 < p.L; c0 += kWave) {
    const int sl = c0 + lane_id();
    const int nbk = sl < p.L ? p.ntpp[sl] / p.B : 0;
    run += lane_value(wave_incl_scan(nbk), kWave - 1);
  }
  return run;
}

// Block counts of the first 64 slots, read once and kept in registers: the
// block count over all slots and the slot lookup then need no second read of
// num_tokens_post_padded (more than 64 slots fall back to the loops above and
// below).
struct BlockScan {
  int nbk;    // blocks of slot lane_id()
  int incl;   // inclusive prefix of nbk over the lanes
  int total;  // blocks over all slots
};

__device__ __forceinline__ BlockScan scan_blocks(const FusedParams& p) {
  BlockScan sc;
  if (p.L <= kWave) {
    const int sl = lane_id();
    sc.nbk = sl < p.L ? p.ntpp[sl] / p.B : 0;
    sc.incl = wave_incl_scan(sc.nbk);
    sc.total = lane_value(sc.incl, kWave - 1);
  } else {
    sc.nbk = sc.incl = 0;
    sc.total = count_blocks(p);
  }
  sc.total = __builtin_amdgcn_readfirstlane(sc.total);
  return sc;
}

// Block g (g < total) -> slot l and block b inside the slot.  Every lane of
// the wavefront gets the same answer.
__device__ __forceinline__ void find_block(const FusedParams& p, int g, int& l, int& b) {
  int run = 0;
  for (int c0 = 0; c0 < p.L; c0 += kWave) {
    const int sl = c0 + lane_id();
    const int nbk = sl < p.L ? p.ntpp[sl] / p.B : 0;
    const int incl = wave_incl_scan(nbk) + run;
    const uint64_t hit = __ballot(incl > g);
    if (hit) {
      const int first = __builtin_ctzll(hit);
      l = c0 + first;
      b = g - (lane_value(incl, first) - lane_value(nbk, first));
      return;
    }
    run = lane_value(incl, kWave - 1);
  }
  l = b = 0;
}

// Workgroup id -> (unit, split).  The units are cut into 8 contiguous ranges
// of nearly equal size, range x for XCD x (workgroup i runs on XCD i % 8);
// the splits of a unit take adjacent ids of one XCD.  Consecutive units --
// the blocks of one (slot, expert) group, and the slices of a block -- thus
// share an L2.  Returns false for a workgroup with no unit.
__device__ __forceinline__ bool map_unit_xcd(int id, int units, int n_split, int& unit, int& split) {
  const int x = id % kXcds, slot = id / kXcds;
  const int lo = int(int64_t(x) * units / kXcds), hi = int(int64_t(x + 1) * units / kXcds);
  const int local = slot / n_split;
  split = slot - local * n_split;
  unit = lo + local;
  return unit < hi;
}

// The same lookup from the registers of scan_blocks.
__device__ __forceinline__ void find_block(const FusedParams& p, const BlockScan& sc, int g, int& l,
                                           int& b) {
  if (p.L <= kWave) {
    const uint64_t hit = __ballot(sc.incl > g);
    const int first = hit ? __builtin_ctzll(hit) : 0;
    l = first;
    b = g - (lane_value(sc.incl, first) - lane_value(sc.nbk, first));
  } else {
    find_block(p, g, l, b);
  }
  l = __builtin_amdgcn_readfirstlane(l);
  b = __builtin_amdgcn_readfirstlane(b);
}

}  // namespace mlr
