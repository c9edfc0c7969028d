// Align step on gfx950: per LoRA slot, bucket the (token, k) pairs by expert,
// pad each bucket to block_m, in canonical order (ascending pair index inside
// a bucket, ascending expert per slot).
//
// The pages (vLLM PR #29257 "Lora MoE Align Improvements", Purpose) keep a
// shared-memory variant for few experts and add a global-memory variant for
// many.  Here the split is by problem size instead:
//   * small problems: ONE workgroup does histogram, scan, layout and scatter
//     with every table in LDS (one launch: decode batches are latency bound);
//   * large problems: tiles of pairs over many workgroups; each tile keeps its
//     per-wave histograms in LDS and only its per-key totals go to global
//     memory, followed by a per-key scan over tiles, one layout workgroup and a
//     tile scatter.
// Both paths are deterministic: a pair's position is its group's start plus
// the number of earlier pairs of the same group, found by wavefront votes on
// the key bits (no atomics decide an order).
#include <algorithm>

#include "align_wave.h"
#include "common.h"
#include "internal.h"

namespace mlr {

constexpr int kLdsInts = 16384;  // 64 KiB of LDS per workgroup

__device__ __forceinline__ int pair_key(const AlignParams& a, int p) {
  const int m = p / a.topk;
  const int l = a.mapping[m];
  const int e = a.topk_ids[p];
  return (unsigned(l) < unsigned(a.L) && unsigned(e) < unsigned(a.E)) ? l * a.E + e : -1;
}

// One wavefront counts pairs [s0, s1) into row[key] (LDS).  If keys is not
// null the pair keys are also kept there (LDS, indexed by pair) for the
// placement pass.
__device__ void count_segment(const AlignParams& a, int s0, int s1, int* row, int* keys) {
  for (int base = s0; base < s1; base += kWave) {
    const int p = base + lane_id();
    if (p < s1) {
      const int key = pair_key(a, p);
      if (keys) keys[p] = key;
      if (key >= 0) atomicAdd(&row[key], 1);
    }
  }
}

// One wavefront places pairs [s0, s1).  row[key] holds the position of the
// next pair of that key; the lowest lane of each equal-key set advances it.
// Keys come from LDS when keys is not null, else are recomputed.
__device__ void scatter_segment(const AlignParams& a, int s0, int s1, int* row, const int* keys) {
  const int lane = lane_id();
  for (int base = s0; base < s1; base += kWave) {
    const int p = base + lane;
    const int key = p < s1 ? (keys ? keys[p] : pair_key(a, p)) : -1;
    const uint64_t valid = __ballot(key >= 0);
    if (valid == 0) continue;
    const uint64_t peers = match_key(key, valid, a.nbits);
    if (key >= 0) {
      const uint64_t below = peers & lanes_below(lane);
      const int pos = row[key] + __popcll(below);
      const int l = key / a.E;
      a.sorted[l * a.cap + pos] = p;
      if (below == 0) row[key] = pos + __popcll(peers);
    }
  }
}

// Expert ids and padding sentinels of group `key`, which starts at o within
// its slot and holds c pairs.  Both runs are consecutive, so lpk lanes share
// a group (block_m / 4 of them: at most three stores each) and a store
// instruction touches a few cache lines instead of one per lane.
__device__ __forceinline__ void fill_group(const AlignParams& a, int key, int o, int c, int sl,
                                           int lpk) {
  const int l = key / a.E, e = key - l * a.E;
  const int P = (c + a.B - 1) / a.B * a.B;
  int32_t* srow = a.sorted + l * a.cap + o;
  int32_t* erow = a.eids + l * a.nb + o / a.B;
  for (int blk = sl; blk < P / a.B; blk += lpk) erow[blk] = e;
  for (int i = c + sl; i < P; i += lpk) srow[i] = a.numel;
}

// From per-key pair counts: padded group starts (within the slot) in off[],
// slot starts in sb[0..L], and the outputs num_tokens_post_padded,
// lora_ids, num_active and (with `fill`) expert_ids and padding sentinels.
// All threads of the workgroup call it (barriers inside).  tot may live in
// LDS or in global memory written by this workgroup before the call (the
// barriers order it).
__device__ void layout_groups(const AlignParams& a, const int* tot, int* off, int* sb,
                              int* wtot, bool fill) {
  const int tid = threadIdx.x;
  for (int key = tid; key < a.LE; key += blockDim.x) {
    const int c = tot[key];
    off[key] = (c + a.B - 1) / a.B * a.B;
  }
  __syncthreads();
  const int total = block_excl_scan(off, a.LE, wtot);
  for (int l = tid; l <= a.L; l += blockDim.x) sb[l] = l < a.L ? off[l * a.E] : total;
  __syncthreads();
  if (fill) {
    const int lpk = a.B / 4;
    const int sub = lane_id() / lpk, sl = lane_id() % lpk;
    const int stride = (blockDim.x / kWave) * (kWave / lpk);
    for (int key = wave_id() * (kWave / lpk) + sub; key < a.LE; key += stride)
      fill_group(a, key, off[key] - sb[key / a.E], tot[key], sl, lpk);
    __syncthreads();
  }
  for (int key = tid; key < a.LE; key += blockDim.x) off[key] -= sb[key / a.E];
  for (int l = tid; l < a.L; l += blockDim.x) a.ntpp[l] = sb[l + 1] - sb[l];
  if (wave_id() == 0 && (a.lora_ids || a.nact)) {
    const int lane = lane_id();
    int run = 0;
    for (int c0 = 0; c0 < a.L; c0 += kWave) {
      const int l = c0 + lane;
      const bool act = l < a.L && sb[l + 1] > sb[l];
      const uint64_t mk = __ballot(act);
      if (act && a.lora_ids) a.lora_ids[run + __popcll(mk & lanes_below(lane))] = l;
      run += __popcll(mk);
    }
    if (a.lora_ids)
      for (int i = run + lane; i < a.L; i += kWave) a.lora_ids[i] = -1;
    if (a.nact && lane == 0) *a.nact = run;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- one wavefront
// (align_wave.h)
__global__ void __launch_bounds__(kWave) align_wave_kernel(AlignParams a) { align_wave_body(a); }

// ---------------------------------------------------------------- one workgroup
__global__ void __launch_bounds__(1024) align_single_kernel(AlignParams a) {
  extern __shared__ int smem[];
  int* cnt = smem;                // [W][LE]: wave histograms, then positions
  int* tot = cnt + a.W * a.LE;    // [LE]
  int* off = tot + a.LE;          // [LE]
  int* sb = off + a.LE;           // [L + 1]
  int* wtot = sb + a.L + 1;       // [17]
  int* keys = wtot + 17;          // [numel]: each pair's key, read once
  const int tid = threadIdx.x, w = wave_id();
  for (int i = tid; i < a.W * a.LE; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  const int s0 = w * a.seg, s1 = min(a.numel, s0 + a.seg);
  if (w < a.W) count_segment(a, s0, s1, cnt + w * a.LE, keys);
  __syncthreads();
  for (int key = tid; key < a.LE; key += blockDim.x) {
    int run = 0;
    for (int q = 0; q < a.W; ++q) {
      const int c = cnt[q * a.LE + key];
      cnt[q * a.LE + key] = run;
      run += c;
    }
    tot[key] = run;
  }
  __syncthreads();
  layout_groups(a, tot, off, sb, wtot, true);
  for (int i = tid; i < a.W * a.LE; i += blockDim.x) cnt[i] += off[i % a.LE];
  __syncthreads();
  if (w < a.W) scatter_segment(a, s0, s1, cnt + w * a.LE, keys);
}

// ---------------------------------------------------------------- tiles
__global__ void __launch_bounds__(1024) align_tile_count_kernel(AlignParams a) {
  extern __shared__ int smem[];
  int* cnt = smem;  // [W][LE]
  const int tid = threadIdx.x, w = wave_id(), t = blockIdx.x;
  for (int i = tid; i < a.W * a.LE; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  const int s0 = (t * a.W + w) * a.seg, s1 = min(a.numel, s0 + a.seg);
  if (s0 < s1) count_segment(a, s0, s1, cnt + w * a.LE, nullptr);
  __syncthreads();
  for (int key = tid; key < a.LE; key += blockDim.x) {
    int sum = 0;
    for (int q = 0; q < a.W; ++q) sum += cnt[q * a.LE + key];
    a.tile_cnt[t * a.LE + key] = sum;
  }
}

// One workgroup: per key, the exclusive prefix of the tile counts over tiles
// (written back in place) and the total (key_tot), then the layout of all
// groups; the expert ids and padding sentinels are left to the tile
// scatter, spread over its workgroups (one workgroup issuing every group's
// stores was the slow part here).  The counts of kPrefixBatch tiles are
// loaded before any is summed.
constexpr int kPrefixBatch = 32;
__global__ void __launch_bounds__(1024) align_meta_kernel(AlignParams a) {
  extern __shared__ int smem[];
  int* off = smem;            // [LE]
  int* sb = off + a.LE;       // [L + 1]
  int* wtot = sb + a.L + 1;   // [17]
  for (int key = threadIdx.x; key < a.LE; key += blockDim.x) {
    int run = 0;
    for (int t0 = 0; t0 < a.ntiles; t0 += kPrefixBatch) {
      int v[kPrefixBatch];
#pragma unroll
      for (int i = 0; i < kPrefixBatch; ++i)
        v[i] = t0 + i < a.ntiles ? a.tile_cnt[(t0 + i) * a.LE + key] : 0;
#pragma unroll
      for (int i = 0; i < kPrefixBatch; ++i) {
        if (t0 + i < a.ntiles) a.tile_cnt[(t0 + i) * a.LE + key] = run;
        run += v[i];
      }
    }
    a.key_tot[key] = run;
  }
  layout_groups(a, a.key_tot, off, sb, wtot, false);
  for (int key = threadIdx.x; key < a.LE; key += blockDim.x) a.key_off[key] = off[key];
}

__global__ void __launch_bounds__(1024) align_tile_scatter_kernel(AlignParams a) {
  extern __shared__ int smem[];
  int* cnt = smem;  // [W][LE]
  const int tid = threadIdx.x, w = wave_id(), t = blockIdx.x;
  for (int i = tid; i < a.W * a.LE; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  const int s0 = (t * a.W + w) * a.seg, s1 = min(a.numel, s0 + a.seg);
  if (s0 < s1) count_segment(a, s0, s1, cnt + w * a.LE, nullptr);
  __syncthreads();
  for (int key = tid; key < a.LE; key += blockDim.x) {
    int run = a.key_off[key] + a.tile_cnt[t * a.LE + key];
    for (int q = 0; q < a.W; ++q) {
      const int c = cnt[q * a.LE + key];
      cnt[q * a.LE + key] = run;
      run += c;
    }
  }
  __syncthreads();
  if (s0 < s1) scatter_segment(a, s0, s1, cnt + w * a.LE, nullptr);
  // expert ids and padding sentinels of this tile's share of the groups
  const int per = (a.LE + a.ntiles - 1) / a.ntiles;
  const int k0 = t * per, k1 = min(a.LE, k0 + per);
  const int lpk = a.B / 4;
  const int sub = lane_id() / lpk, sl = lane_id() % lpk;
  const int stride = (blockDim.x / kWave) * (kWave / lpk);
  for (int key = k0 + w * (kWave / lpk) + sub; key < k1; key += stride)
    fill_group(a, key, a.key_off[key], a.key_tot[key], sl, lpk);
}

// ---------------------------------------------------------------- host
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

AlignPlan plan_align(int64_t numel, int E, int L, int B) {
  (void)B;
  AlignPlan pl{};
  if (numel <= kAlignWaveMaxPairs && L <= kAlignWaveMaxSlots) {
    pl.wave = true;
    pl.threads = kWave;
    return pl;
  }
  const int64_t LE = int64_t(L) * E;
  const int64_t fixed = 2 * LE + L + 1 + 17 + numel;   // tot, off, sb, wtot, keys
  const int64_t wmax_single = (kLdsInts - fixed) / LE;
  if (numel <= 4096 && wmax_single >= 1) {
    pl.single = true;
    int64_t W = std::min<int64_t>({16, std::max<int64_t>(1, cdiv(numel, kWave)), wmax_single});
    int64_t seg = cdiv(std::max<int64_t>(numel, 1), W);
    seg = cdiv(seg, kWave) * kWave;
    W = std::max<int64_t>(1, cdiv(numel, seg));
    pl.W = int(W);
    pl.seg = int(seg);
    pl.ntiles = 1;
    pl.threads = 16 * kWave;  // all waves help with the layout and the padding
    pl.lds_bytes = size_t((W * LE + fixed) * 4);
    pl.ws_bytes = 0;
    return pl;
  }
  pl.single = false;
  const int64_t W = std::min<int64_t>(16, kLdsInts / LE);
  const int64_t max_tiles = std::max<int64_t>(1, std::min<int64_t>(1024, (int64_t(1) << 18) / LE));
  int64_t ntiles = std::min<int64_t>(max_tiles, cdiv(numel, W * kWave));
  ntiles = std::max<int64_t>(ntiles, 1);
  int64_t seg = std::max<int64_t>(kWave, cdiv(cdiv(numel, ntiles * W), kWave) * kWave);
  ntiles = std::max<int64_t>(1, cdiv(numel, W * seg));
  pl.W = int(W);
  pl.seg = int(seg);
  pl.ntiles = int(ntiles);
  pl.threads = int(W * kWave);
  pl.lds_bytes = size_t(W * LE * 4);
  pl.meta_lds_bytes = size_t((LE + L + 1 + 17) * 4);
  pl.ws_bytes = (ntiles * LE + 2 * LE) * 4;
  return pl;
}

hipError_t launch_align(const AlignPlan& pl, const AlignParams& a, hipStream_t st) {
  if (pl.wave) {
    hipLaunchKernelGGL(align_wave_kernel, dim3(1), dim3(kWave), 0, st, a);
    return hipGetLastError();
  }
  if (pl.single) {
    hipLaunchKernelGGL(align_single_kernel, dim3(1), dim3(pl.threads), pl.lds_bytes, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(align_tile_count_kernel, dim3(pl.ntiles), dim3(pl.threads), pl.lds_bytes,
                     st, a);
  hipLaunchKernelGGL(align_meta_kernel, dim3(1), dim3(1024), pl.meta_lds_bytes, st, a);
  hipLaunchKernelGGL(align_tile_scatter_kernel, dim3(pl.ntiles), dim3(pl.threads),
                     pl.lds_bytes, st, a);
  return hipGetLastError();
}

}  // namespace mlr
