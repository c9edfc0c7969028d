// On-chip grouping of the routed pairs, for the align-free path.
//
// The pages' naive block assignment (vLLM PR #42290 summary, the dispatch
// fragment of the one-shot kernel: a grid over tokens x top-k, slices and
// active slots) lets a decode batch skip the align launch and hand each
// (token, k) pair to its own program.  Here every workgroup of the fused
// kernel reads topk_ids and the token -> slot mapping itself (one pair per
// thread, at most 1024 pairs) and forms the same blocks the align step would:
// the valid pairs of one (slot, expert) group in ascending pair order, cut
// into blocks of block_m pairs.  Groups are numbered by their first pair
// rather than by (slot, expert); a block holds the same pairs in the same
// order either way, so the fused arithmetic does not change.  block_m = 1 is
// the pages' one-pair-per-program assignment.
//
// Pairs with equal keys inside a wavefront are found by voting on the key
// bits.  Up to 64 pairs, every wavefront holds all of them (lane = pair) and
// forms the groups, their block counts and the block numbering in registers,
// with no LDS table and no barrier but the one that publishes the block's
// pair ids.  Beyond that, the wavefront leaders (lowest lane of each key)
// meet in a small LDS hash table, where the first pair and the size of each
// group collect by atomic min and add.  Neither depends on the order of the
// atomics, so the numbering is deterministic.
#pragma once

#include <limits.h>

#include "common.h"
#include "internal.h"

namespace mlr {

constexpr int kGroupThreads = 1024;  // one pair per thread
constexpr int kGroupHashBits = 11;
constexpr int kGroupHash = 1 << kGroupHashBits;  // at most 1024 keys: half full at most

struct GroupLds {
  int key[kGroupHash];    // -1 = empty
  int first[kGroupHash];  // lowest pair index of the group
  int cnt[kGroupHash];    // pairs of the group
  int wsum[kGroupThreads / kWave];
  int sel[2];             // the workgroup's block: group key, block within the group
};

// What a thread keeps about its own pair between the two phases.
struct PairGroup {
  int key;   // l * E + e, or -1 for an invalid pair
  int excl;  // blocks of the groups that start before this pair (group leaders only)
  int nblk;  // blocks of this pair's group if the pair is its first, else 0
};

// Phase 1 (every thread of a kGroupThreads workgroup): group the pairs;
// returns the number of blocks over all groups.  Contains barriers.
__device__ inline int group_pairs(const FusedParams& p, GroupLds& g, PairGroup& pg) {
  const int t = threadIdx.x, lane = lane_id(), w = wave_id();
  const bool one_wave = p.numel <= kWave;
  const int pair = one_wave ? lane : t;
  // both loads are issued before either is used (one memory round trip): the
  // validity test is a select, not a branch the second load could sink into
  int l = -1, e = -1;
  if (pair < p.numel) {
    l = p.mapping[pair / p.topk];
    e = p.topk_ids[pair];
  }
  const bool ok = (unsigned(l) < unsigned(p.L)) & (unsigned(e) < unsigned(p.E));
  const int key = ok ? l * p.E + e : -1;
  const uint64_t valid = __ballot(key >= 0);
  const uint64_t peers = match_key(key, valid, p.nbits);
  const int src = key >= 0 ? __builtin_ctzll(peers) : lane;  // the wavefront leader of the key
  if (one_wave) {
    const int nblk = (key >= 0 && src == lane) ? (__popcll(peers) + p.B - 1) / p.B : 0;
    const int incl = wave_incl_scan(nblk);
    pg.key = key;
    pg.excl = incl - nblk;
    pg.nblk = nblk;
    return __builtin_amdgcn_readfirstlane(__shfl(incl, kWave - 1));
  }
  for (int i = t; i < kGroupHash; i += kGroupThreads) {
    g.key[i] = -1;
    g.first[i] = INT_MAX;
    g.cnt[i] = 0;
  }
  __syncthreads();
  int slot = 0;
  if (key >= 0 && src == lane) {
    uint32_t h = (uint32_t(key) * 2654435761u) >> (32 - kGroupHashBits);
    for (;;) {  // at most 1024 keys in 2048 entries: a free or equal entry is always found
      const int old = atomicCAS(&g.key[h], -1, key);
      if (old == -1 || old == key) break;
      h = (h + 1) & (kGroupHash - 1);
    }
    slot = int(h);
    atomicMin(&g.first[h], t);
    atomicAdd(&g.cnt[h], __popcll(peers));
  }
  slot = __shfl(slot, src);
  __syncthreads();
  const bool lead = key >= 0 && g.first[slot] == t;
  const int nblk = lead ? (g.cnt[slot] + p.B - 1) / p.B : 0;
  const int incl = wave_incl_scan(nblk);
  if (lane == kWave - 1) g.wsum[w] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kGroupThreads / kWave; ++i) {
    const int v = g.wsum[i];
    total += v;
    before += i < w ? v : 0;
  }
  pg.key = key;
  pg.excl = before + incl - nblk;
  pg.nblk = nblk;
  return __builtin_amdgcn_readfirstlane(total);
}

// Phase 2 (every thread): block gi (< the total of phase 1) -> slot l, expert
// e and its pair ids in ids[0..B), ascending, padded with numel.  Contains
// barriers.
__device__ inline void group_block(const FusedParams& p, GroupLds& g, const PairGroup& pg, int gi,
                                   int* ids, int& l, int& e) {
  const int t = threadIdx.x, lane = lane_id(), w = wave_id();
  if (p.numel <= kWave) {
    // the group leader whose block range holds gi, found in registers
    const uint64_t hit = __ballot(gi >= pg.excl && gi < pg.excl + pg.nblk);
    const int src = hit ? __builtin_ctzll(hit) : 0;
    const int key = __builtin_amdgcn_readfirstlane(__shfl(pg.key, src));
    const int b = __builtin_amdgcn_readfirstlane(gi - __shfl(pg.excl, src));
    const bool match = pg.key == key;
    const uint64_t m = __ballot(match);
    if (w == 0) {
      for (int i = lane; i < p.B; i += kWave) ids[i] = p.numel;
      const int rank = __popcll(m & lanes_below(lane)) - b * p.B;
      if (match && rank >= 0 && rank < p.B) ids[rank] = lane;
    }
    __syncthreads();
    l = key / p.E;
    e = key - l * p.E;
    return;
  }
  if (gi >= pg.excl && gi < pg.excl + pg.nblk) {
    g.sel[0] = pg.key;
    g.sel[1] = gi - pg.excl;
  }
  for (int i = t; i < p.B; i += kGroupThreads) ids[i] = p.numel;
  __syncthreads();
  const int key = __builtin_amdgcn_readfirstlane(g.sel[0]);
  const int b = __builtin_amdgcn_readfirstlane(g.sel[1]);
  const bool match = pg.key == key;
  const uint64_t m = __ballot(match);
  if (lane == 0) g.wsum[w] = __popcll(m);
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int i = 0; i < kGroupThreads / kWave; ++i) before += i < w ? g.wsum[i] : 0;
  const int rank = before + __popcll(m & lanes_below(lane)) - b * p.B;
  if (match && rank >= 0 && rank < p.B) ids[rank] = t;
  __syncthreads();
  l = key / p.E;
  e = key - l * p.E;
}

}  // namespace mlr
