// One-wavefront align step, shared by the align kernel and the fused kernels
// that run it beside their own work (fused_moe_lora_with_align).
#pragma once

#include <limits.h>

#include "common.h"
#include "internal.h"

namespace mlr {

// At most 64 pairs and 64 slots (decode batches): lane = pair.  Equal keys
// are found by voting on the key bits; a group's start in its slot is the sum
// of the padded sizes of the same slot's groups with smaller keys (their
// leaders are read lane by lane), a pair's place is that start plus the
// number of lower lanes with its key.  Everything stays in registers: no LDS,
// no barrier, one round trip to read the routing.

// Called by the 64 lanes of one wavefront.
__device__ __forceinline__ void align_wave_body(const AlignParams& a) {
  const int lane = lane_id();
  int l = -1, e = -1;
  if (lane < a.numel) {  // both loads issued before either is used
    l = int(unsigned(a.mapping[lane / a.topk]) - unsigned(a.l0));
    e = a.topk_ids[lane];
  }
  const bool ok = (unsigned(l) < unsigned(a.L)) & (unsigned(e) < unsigned(a.E));
  const int key = ok ? l * a.E + e : -1;
  const int slot = ok ? l : -1;
  const uint64_t peers = match_key(key, __ballot(ok), a.nbits);
  const bool lead = ok && (peers & lanes_below(lane)) == 0;
  const int cnt = ok ? __popcll(peers) : 0;
  const int pad = lead ? (cnt + a.B - 1) / a.B * a.B : 0;  // 0 unless this lane leads a group
  int off = 0;
  for (int j = 0; j < kWave; ++j) {
    const int kj = __builtin_amdgcn_readlane(key, j);
    const int sj = __builtin_amdgcn_readlane(slot, j);
    const int pj = __builtin_amdgcn_readlane(pad, j);
    off += (sj == slot && kj < key) ? pj : 0;
  }
  if (ok) {
    const int goff = __shfl(off, __builtin_ctzll(peers));
    a.sorted[l * a.cap + goff + __popcll(peers & lanes_below(lane))] = lane;
  }
  if (lead) {  // the group's expert ids and padding sentinels
    int32_t* erow = a.eids + l * a.nb + off / a.B;
    for (int b = 0; b < pad / a.B; ++b) erow[b] = e;
    int32_t* srow = a.sorted + l * a.cap + off;
    for (int i = cnt; i < pad; ++i) srow[i] = a.numel;
  }
  // lane = slot: padded total, the active list and its count
  int tot = 0;
  for (int j = 0; j < kWave; ++j) {
    const int sj = __builtin_amdgcn_readlane(slot, j);
    const int pj = __builtin_amdgcn_readlane(pad, j);
    tot += sj == lane ? pj : 0;
  }
  const bool in = lane < a.L;
  if (in) a.ntpp[lane] = tot;
  const uint64_t act = __ballot(in && tot > 0);
  const int nact = __popcll(act);
  if (a.lora_ids) {  // entries [0, nact) get the active slots, [nact, L) get -1: disjoint stores
    if (in && tot > 0) a.lora_ids[__popcll(act & lanes_below(lane))] = lane;
    if (in && lane >= nact) a.lora_ids[lane] = -1;
  }
  if (a.nact && lane == 0) *a.nact = nact;
}

// fused_moe_lora_with_align: one workgroup of the fused kernel writes the
// align outputs with its first wavefront; the fused workgroups form their
// blocks on chip and never read those outputs, so the two run side by side.
// The align goes to the first workgroup the unit mapping leaves without work,
// `idle`, which then does nothing else; when every workgroup has work (idle
// is past the grid) workgroup 0 runs it before its own.  (A workgroup added
// to the launch for it was dispatched after all others and, on a full XCD,
// waited for a compute unit to free up: +2 to +5 us.)  Returns true when this
// workgroup has no fused work left (every thread of it: the caller returns
// before any barrier).
__device__ __forceinline__ bool side_align(const FusedParams& p, int idle) {
  if (p.al_sorted == nullptr) return false;
  const bool spare = idle < int(gridDim.x);
  if (int(blockIdx.x) != (spare ? idle : 0)) return false;
  if (threadIdx.x < kWave) {
    AlignParams a{};
    a.topk_ids = p.topk_ids;
    a.mapping = p.mapping;
    a.sorted = p.al_sorted;
    a.eids = p.al_eids;
    a.ntpp = p.al_ntpp;
    a.lora_ids = p.al_lora_ids;
    a.nact = p.al_nact;
    a.numel = p.numel;
    a.topk = p.topk;
    a.E = p.E;
    a.L = p.L;
    a.LE = p.L * p.E;
    a.B = p.B;
    a.nbits = p.nbits;
    a.cap = p.cap;
    a.nb = p.nb;
    align_wave_body(a);
  }
  return spare;
}

// The first workgroup index map_unit_xcd leaves without a unit.  XCD x
// holds units [x units / 8, (x + 1) units / 8), so XCD 0 holds the fewest,
// units / 8, and its first index past them, 8 (units / 8) n_split, is below
// the first idle index x + 8 (its count) n_split of every other XCD x.
__device__ __forceinline__ int first_idle_xcd(int units, int n_split) {
  return units / kXcds * n_split * kXcds;
}

}  // namespace mlr
