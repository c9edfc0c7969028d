// On-chip grouping of the routed pairs, for the align-free path.
//
// The pages' naive block assignment (vLLM PR #42290 summary, the dispatch
// fragment of the one-shot kernel: a grid over tokens x top-k, slices and
// active slots) lets a decode batch skip the align launch and hand each
// (token, k) pair to its own program.  Here every workgroup of the fused
// kernel reads topk_ids and the token -> slot mapping itself (at most 1024
// pairs) and forms the same blocks the align step would: the valid pairs of
// one (slot, expert) group in ascending pair order, cut into blocks of
// block_m pairs.  Groups are numbered by their first pair rather than by
// (slot, expert); a block holds the same pairs in the same order either way,
// so the fused arithmetic does not change.  block_m = 1 is the pages'
// one-pair-per-program assignment.
//
// Pairs with equal keys inside a wavefront are found by voting on the key
// bits.  Up to 64 pairs, every wavefront holds all of them (lane = pair) and
// forms the groups, their block counts and the block numbering in registers,
// with no LDS table and no barrier but the one that publishes the block's
// pair ids.  Beyond that, a workgroup of T threads takes the pairs in
// 1024 / T steps of T (pair = step * T + thread, so the 16 wavefront-sized
// pieces of the pair range are numbered in pair order), and the wavefront
// leaders (lowest lane of each key in a piece) meet in a small LDS hash
// table, where the first pair and the size of each group collect by atomic
// min and add.  Neither depends on the order of the atomics, so the
// numbering is deterministic.
#pragma once

#include <limits.h>

#include "common.h"
#include "internal.h"

namespace mlr {

constexpr int kGroupPairs = 1024;                  // most pairs grouped
constexpr int kGroupPieces = kGroupPairs / kWave;  // wavefront-sized pieces of the pairs
constexpr int kGroupHashBits = 11;
constexpr int kGroupHash = 1 << kGroupHashBits;  // at most 1024 keys: half full at most
static_assert(kGroupPairs == kNaiveMaxPairs, "grouping capacity");

struct GroupLds {
  int key[kGroupHash];    // -1 = empty
  int first[kGroupHash];  // lowest pair index of the group
  int cnt[kGroupHash];    // pairs of the group
  int wsum[kGroupPieces];
  int sel[2];             // the workgroup's block: group key, block within the group
};

// What a thread keeps about its pairs between the two phases (step c holds
// pair c * T + thread; with at most 64 pairs only step 0, pair = lane).
template <int T>
struct PairGroup {
  static constexpr int R = kGroupPairs / T;
  int key[R];   // l * E + e, or -1 for an invalid pair
  int excl[R];  // blocks of the groups that start before this pair (group leaders only)
  int nblk[R];  // blocks of this pair's group if the pair is its first, else 0
};

// Phase 1 (every thread of a T-thread workgroup): group the pairs; returns
// the number of blocks over all groups.  Contains barriers.
template <int T>
__device__ inline int group_pairs(const FusedParams& p, GroupLds& g, PairGroup<T>& pg) {
  static_assert(T % kWave == 0 && kGroupPairs % T == 0, "workgroup size");
  constexpr int R = PairGroup<T>::R, W = T / kWave;
  const int t = threadIdx.x, lane = lane_id(), w = wave_id();
  const bool one_wave = p.numel <= kWave;
  // every load is issued before any is used (one memory round trip): the
  // validity test is a select, not a branch a later load could sink into
  int l[R], e[R];
#pragma unroll
  for (int c = 0; c < R; ++c) {
    const int pair = one_wave ? (c == 0 ? lane : kGroupPairs) : c * T + t;
    l[c] = e[c] = -1;
    if (pair < p.numel) {
      l[c] = p.mapping[pair / p.topk];
      e[c] = p.topk_ids[pair];
    }
  }
  uint64_t peers[R];
  int src[R];
#pragma unroll
  for (int c = 0; c < R; ++c) {
    const bool ok = (unsigned(l[c]) < unsigned(p.L)) & (unsigned(e[c]) < unsigned(p.E));
    pg.key[c] = ok ? l[c] * p.E + e[c] : -1;
    pg.excl[c] = pg.nblk[c] = 0;
    peers[c] = match_key(pg.key[c], __ballot(ok), p.nbits);
    src[c] = ok ? __builtin_ctzll(peers[c]) : lane;  // the leader of the key in this piece
  }
  if (one_wave) {
    const int nblk = (pg.key[0] >= 0 && src[0] == lane) ? (__popcll(peers[0]) + p.B - 1) / p.B : 0;
    const int incl = wave_incl_scan(nblk);
    pg.excl[0] = incl - nblk;
    pg.nblk[0] = nblk;
    return lane_value(incl, kWave - 1);
  }
  for (int i = t; i < kGroupHash; i += T) {
    g.key[i] = -1;
    g.first[i] = INT_MAX;
    g.cnt[i] = 0;
  }
  __syncthreads();
  int slot[R];
#pragma unroll
  for (int c = 0; c < R; ++c) {
    const int key = pg.key[c];
    slot[c] = 0;
    if (key >= 0 && src[c] == lane) {
      uint32_t h = (uint32_t(key) * 2654435761u) >> (32 - kGroupHashBits);
      for (;;) {  // at most 1024 keys in 2048 entries: a free or equal entry is always found
        const int old = atomicCAS(&g.key[h], -1, key);
        if (old == -1 || old == key) break;
        h = (h + 1) & (kGroupHash - 1);
      }
      slot[c] = int(h);
      atomicMin(&g.first[h], c * T + t);
      atomicAdd(&g.cnt[h], __popcll(peers[c]));
    }
    slot[c] = __shfl(slot[c], src[c]);
  }
  __syncthreads();
  int incl[R];
#pragma unroll
  for (int c = 0; c < R; ++c) {
    const bool lead = pg.key[c] >= 0 && g.first[slot[c]] == c * T + t;
    pg.nblk[c] = lead ? (g.cnt[slot[c]] + p.B - 1) / p.B : 0;
    incl[c] = wave_incl_scan(pg.nblk[c]);
    if (lane == kWave - 1) g.wsum[c * W + w] = incl[c];
  }
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int i = 0; i < kGroupPieces; ++i) {
    const int v = g.wsum[i];
#pragma unroll
    for (int c = 0; c < R; ++c) pg.excl[c] += i < c * W + w ? v : 0;
    total += v;
  }
#pragma unroll
  for (int c = 0; c < R; ++c) pg.excl[c] += incl[c] - pg.nblk[c];
  return __builtin_amdgcn_readfirstlane(total);
}

// Phase 2 for at most 64 pairs, run by the one wavefront that ran phase 1:
// block gi -> slot l, expert e and its pair ids in ids[0..B), ascending,
// padded with numel.  No barrier: the caller publishes ids.
template <int T>
__device__ inline void group_block_wave(const FusedParams& p, const PairGroup<T>& pg, int gi,
                                        int* ids, int& l, int& e) {
  const int lane = lane_id();
  const uint64_t hit = __ballot(gi >= pg.excl[0] && gi < pg.excl[0] + pg.nblk[0]);
  const int src = hit ? __builtin_ctzll(hit) : 0;
  const int key = lane_value(pg.key[0], src);
  const int b = gi - lane_value(pg.excl[0], src);
  const bool match = pg.key[0] == key;
  const uint64_t m = __ballot(match);
  for (int i = lane; i < p.B; i += kWave) ids[i] = p.numel;
  const int rank = __popcll(m & lanes_below(lane)) - b * p.B;
  if (match && rank >= 0 && rank < p.B) ids[rank] = lane;
  l = key / p.E;
  e = key - l * p.E;
}

// Phase 2 (every thread): block gi (< the total of phase 1) -> slot l, expert
// e and its pair ids in ids[0..B), ascending, padded with numel.  Contains
// barriers.
template <int T>
__device__ inline void group_block(const FusedParams& p, GroupLds& g, const PairGroup<T>& pg,
                                   int gi, int* ids, int& l, int& e) {
  constexpr int R = PairGroup<T>::R, W = T / kWave;
  const int t = threadIdx.x, lane = lane_id(), w = wave_id();
  if (p.numel <= kWave) {
    // the group leader whose block range holds gi, found in registers
    const uint64_t hit = __ballot(gi >= pg.excl[0] && gi < pg.excl[0] + pg.nblk[0]);
    const int src = hit ? __builtin_ctzll(hit) : 0;
    const int key = lane_value(pg.key[0], src);
    const int b = gi - lane_value(pg.excl[0], src);
    const bool match = pg.key[0] == key;
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
#pragma unroll
  for (int c = 0; c < R; ++c) {
    if (gi >= pg.excl[c] && gi < pg.excl[c] + pg.nblk[c]) {
      g.sel[0] = pg.key[c];
      g.sel[1] = gi - pg.excl[c];
    }
  }
  for (int i = t; i < p.B; i += T) ids[i] = p.numel;
  __syncthreads();
  const int key = __builtin_amdgcn_readfirstlane(g.sel[0]);
  const int b = __builtin_amdgcn_readfirstlane(g.sel[1]);
  uint64_t m[R];
#pragma unroll
  for (int c = 0; c < R; ++c) {
    m[c] = __ballot(pg.key[c] == key);
    if (lane == 0) g.wsum[c * W + w] = __popcll(m[c]);
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < R; ++c) {
    int before = 0;
#pragma unroll
    for (int i = 0; i < kGroupPieces; ++i) before += i < c * W + w ? g.wsum[i] : 0;
    const int rank = before + __popcll(m[c] & lanes_below(lane)) - b * p.B;
    if (pg.key[c] == key && rank >= 0 && rank < p.B) ids[rank] = c * T + t;
  }
  __syncthreads();
  l = key / p.E;
  e = key - l * p.E;
}

}  // namespace mlr
