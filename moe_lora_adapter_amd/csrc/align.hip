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

// Most per-wave count rows of the tile scatter (its wavefronts per
// workgroup); can be overridden when building to re-tune.
#ifndef MLR_ALIGN_MAX_ROWS
#define MLR_ALIGN_MAX_ROWS 16
#endif

__device__ __forceinline__ int pair_key(const AlignParams& a, int p) {
  const int m = p / a.topk;
  const int l = int(unsigned(a.mapping[m]) - unsigned(a.l0));  // wraps: out of range stays out
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
// A tile is `seg` consecutive pairs (the last one shorter); tile t is handled
// by workgroup t of the count and of the scatter kernel.  Every lane loads the
// keys of kKeyBatch of its pairs before it uses any, so a wavefront waits for
// memory once per 64 * kKeyBatch pairs instead of once per 64.
constexpr int kKeyBatch = 16;
constexpr int kKeyChunk = kKeyBatch * kWave;

// Keys of pairs base + 64 i + lane (i < kKeyBatch); -1 for a pair at or past
// s1 (s1 > base) or one outside every group.  The loads are unconditional
// (addresses clamped into [base, s1)) so that all of them are in flight
// together.
__device__ __forceinline__ void load_keys(const AlignParams& a, int64_t base, int s1,
                                          int (&key)[kKeyBatch]) {
  const int lane = lane_id();
  int e[kKeyBatch], l[kKeyBatch];
#pragma unroll
  for (int i = 0; i < kKeyBatch; ++i) {
    const int p = int(min<int64_t>(base + i * kWave + lane, s1 - 1));
    e[i] = a.topk_ids[p];
    l[i] = int(unsigned(a.mapping[p / a.topk]) - unsigned(a.l0));
  }
#pragma unroll
  for (int i = 0; i < kKeyBatch; ++i) {
    const bool in = base + i * kWave + lane < s1 && unsigned(l[i]) < unsigned(a.L) &&
                    unsigned(e[i]) < unsigned(a.E);
    key[i] = in ? l[i] * a.E + e[i] : -1;
  }
}

// One wavefront's pairs of one 64-pair step, keys known: positions from
// row[key] (the next free position of each key), the lowest lane of each
// equal-key set advancing it.
__device__ __forceinline__ void place_step(const AlignParams& a, int* row, int key, int p) {
  const int lane = lane_id();
  const uint64_t valid = __ballot(key >= 0);
  if (valid == 0) return;
  const uint64_t peers = match_key(key, valid, a.nbits);
  if (key >= 0) {
    const uint64_t below = peers & lanes_below(lane);
    const int pos = row[key] + __popcll(below);
    const int l = key / a.E;
    a.sorted[l * a.cap + pos] = p;
    if (below == 0) row[key] = pos + __popcll(peers);
  }
}

// Per tile: the pair count of every key (one LDS histogram shared by the
// workgroup) to tile_cnt[t][key].
__global__ void __launch_bounds__(1024) align_tile_count_kernel(AlignParams a) {
  extern __shared__ int hist[];  // [LE]
  const int tid = threadIdx.x, t = blockIdx.x;
  const int nw = blockDim.x / kWave, w = wave_id();
  for (int i = tid; i < a.LE; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  const int64_t t0 = int64_t(t) * a.seg;
  const int t1 = int(min<int64_t>(a.numel, t0 + a.seg));
  for (int64_t base = t0 + w * kKeyChunk; base < t1; base += nw * kKeyChunk) {
    int key[kKeyBatch];
    load_keys(a, base, t1, key);
#pragma unroll
    for (int i = 0; i < kKeyBatch; ++i)
      if (key[i] >= 0) atomicAdd(&hist[key[i]], 1);
  }
  __syncthreads();
  int* out = a.tile_cnt + int64_t(t) * a.LE;
  for (int key = tid; key < a.LE; key += blockDim.x) out[key] = hist[key];
}

// Per key, the exclusive prefix of its tile counts over tiles (in place) and
// its total (key_tot).  A workgroup takes 64 consecutive keys (lane = key, so
// every load reads 256 contiguous bytes of a tile's row) and its Q
// wavefronts split the tiles into runs; each run's counts are loaded a batch
// at a time before any is used, and the runs' sums are combined in LDS.
__global__ void __launch_bounds__(1024) align_prefix_kernel(AlignParams a) {
  __shared__ int part[16][kWave];
  const int lane = lane_id(), q = wave_id(), Q = blockDim.x / kWave;
  const int key = blockIdx.x * kWave + lane;
  const bool live = key < a.LE;
  const int chunk = (a.ntiles + Q - 1) / Q;
  const int ta = min(a.ntiles, q * chunk), tb = min(a.ntiles, ta + chunk);
  int* col = a.tile_cnt + (live ? key : 0);
  int sum = 0;
  for (int t = ta; t < tb; t += kKeyBatch) {
    int v[kKeyBatch];
#pragma unroll
    for (int i = 0; i < kKeyBatch; ++i) v[i] = col[int64_t(min(t + i, tb - 1)) * a.LE];
#pragma unroll
    for (int i = 0; i < kKeyBatch; ++i) sum += t + i < tb ? v[i] : 0;
  }
  part[q][lane] = sum;
  __syncthreads();
  int run = 0, total = 0;
  for (int u = 0; u < Q; ++u) {
    const int c = part[u][lane];
    run += u < q ? c : 0;
    total += c;
  }
  if (!live) return;
  for (int t = ta; t < tb; t += kKeyBatch) {
    int v[kKeyBatch];
#pragma unroll
    for (int i = 0; i < kKeyBatch; ++i) v[i] = col[int64_t(min(t + i, tb - 1)) * a.LE];
#pragma unroll
    for (int i = 0; i < kKeyBatch; ++i) {
      if (t + i < tb) {
        col[int64_t(t + i) * a.LE] = run;
        run += v[i];
      }
    }
  }
  if (q == 0) a.key_tot[key] = total;
}

// Exclusive prefix sum in place of a[0..n) in LDS, each thread taking a
// contiguous run of about n / blockDim entries (two barriers in all, against
// three per blockDim entries for block_excl_scan).  Returns the total.
__device__ int block_excl_scan_runs(int* a, int n, int* wtot) {
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int nw = blockDim.x / kWave;
  const int r = (n + blockDim.x - 1) / blockDim.x;
  const int i0 = min(n, tid * r), i1 = min(n, i0 + r);
  int s = 0;
  for (int i = i0; i < i1; ++i) s += a[i];
  const int incl = wave_incl_scan(s);
  if (lane == kWave - 1) wtot[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int t = lane < nw ? wtot[lane] : 0;
    const int ti = wave_incl_scan(t);
    if (lane < nw) wtot[lane] = ti - t;
    if (lane == nw - 1) wtot[16] = ti;
  }
  __syncthreads();
  int run = wtot[w] + incl - s;
  for (int i = i0; i < i1; ++i) {
    const int v = a[i];
    a[i] = run;
    run += v;
  }
  const int total = wtot[16];
  __syncthreads();
  return total;
}

// Per tile, W = blockDim / 64 wavefronts, wave w owning pairs
// [t seg + w segw, + segw) of the tile:
//   1. per-wave counts (LDS rows), while the key totals are in flight;
//   2. the layout of every group from the key totals (each workgroup computes
//      it: padded sizes, one scan, slot starts), and each row turned into the
//      next free position of every key for that wave (group start in the
//      slot + pairs of the key in earlier tiles + in earlier waves of this
//      tile);
//   3. the placement;
//   4. the expert ids and padding sentinels of this tile's share of the
//      groups; workgroup 0 also writes num_tokens_post_padded and the active
//      slot list.
__global__ void __launch_bounds__(1024) align_tile_scatter_kernel(AlignParams a) {
  extern __shared__ int smem[];
  int* off = smem;               // [LE]: padded sizes, then group starts in the slot
  int* sb = off + a.LE;          // [L + 1]: slot starts in the scan
  int* wtot = sb + a.L + 1;      // [17]
  int* cnt = wtot + 17;          // [W][LE]
  const int tid = threadIdx.x, w = wave_id(), t = blockIdx.x, W = blockDim.x / kWave;
  const int64_t s0 = int64_t(t) * a.seg + int64_t(w) * a.segw;
  const int t1 = int(min<int64_t>(a.numel, (int64_t(t) + 1) * a.seg));
  const int s1 = int(min<int64_t>(t1, s0 + a.segw));
  int key0[kKeyBatch];           // keys of the wave's first chunk, kept for both passes
  if (s0 < s1) load_keys(a, s0, s1, key0);
  int tv[8];                     // the first key totals of this thread, in flight meanwhile
#pragma unroll
  for (int i = 0; i < 8; ++i) tv[i] = a.key_tot[min(tid + i * int(blockDim.x), a.LE - 1)];
  for (int i = tid; i < W * a.LE; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  int* row = cnt + w * a.LE;
  for (int64_t base = s0; base < s1; base += kKeyChunk) {
    int key[kKeyBatch];
    if (base == s0) {
#pragma unroll
      for (int i = 0; i < kKeyBatch; ++i) key[i] = key0[i];
    } else {
      load_keys(a, base, s1, key);
    }
#pragma unroll
    for (int i = 0; i < kKeyBatch; ++i)
      if (key[i] >= 0) atomicAdd(&row[key[i]], 1);
  }
  // padded group sizes, then their scan: group starts, slot starts
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (tid + i * int(blockDim.x) < a.LE) off[tid + i * blockDim.x] = (tv[i] + a.B - 1) / a.B * a.B;
  for (int k0 = tid + 8 * blockDim.x; k0 < a.LE; k0 += blockDim.x * 8) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = a.key_tot[min(k0 + i * int(blockDim.x), a.LE - 1)];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (k0 + i * int(blockDim.x) < a.LE) off[k0 + i * blockDim.x] = (v[i] + a.B - 1) / a.B * a.B;
  }
  __syncthreads();
  const int total = block_excl_scan_runs(off, a.LE, wtot);
  for (int l = tid; l <= a.L; l += blockDim.x) sb[l] = l < a.L ? off[l * a.E] : total;
  __syncthreads();
  const int* tc = a.tile_cnt + int64_t(t) * a.LE;
  for (int k0 = tid; k0 < a.LE; k0 += blockDim.x * 8) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = tc[min(k0 + i * int(blockDim.x), a.LE - 1)];
    for (int i = 0; i < 8; ++i) {
      const int key = k0 + i * blockDim.x;
      if (key >= a.LE) break;
      int c[16];                 // the W rows' counts of this key, read together
#pragma unroll
      for (int q = 0; q < 16; ++q) c[q] = q < W ? cnt[q * a.LE + key] : 0;
      int run = off[key] - sb[key / a.E] + v[i];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (q < W) {
          cnt[q * a.LE + key] = run;
          run += c[q];
        }
      }
    }
  }
  __syncthreads();
  for (int64_t base = s0; base < s1; base += kKeyChunk) {
    int key[kKeyBatch];
    if (base == s0) {
#pragma unroll
      for (int i = 0; i < kKeyBatch; ++i) key[i] = key0[i];
    } else {
      load_keys(a, base, s1, key);
    }
#pragma unroll
    for (int i = 0; i < kKeyBatch; ++i)
      place_step(a, row, key[i], int(base + i * kWave + lane_id()));
  }
  // expert ids and padding sentinels of this tile's share of the groups
  const int per = (a.LE + a.ntiles - 1) / a.ntiles;
  const int k0 = t * per, k1 = min(a.LE, k0 + per);
  const int lpk = a.B / 4;
  const int sub = lane_id() / lpk, sl = lane_id() % lpk;
  const int stride = W * (kWave / lpk);
  for (int key = k0 + w * (kWave / lpk) + sub; key < k1; key += stride)
    fill_group(a, key, off[key] - sb[key / a.E], a.key_tot[key], sl, lpk);
  if (t == 0) {
    for (int l = tid; l < a.L; l += blockDim.x) a.ntpp[l] = sb[l + 1] - sb[l];
    if (w == 0 && (a.lora_ids || a.nact)) {
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
  }
}

// ---------------------------------------------------------------- host
static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Most LDS bytes one workgroup may take on the current device (cached).
static int lds_per_block() {
  constexpr int kMaxDevices = 64;
  static int cache[kMaxDevices] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return kLdsInts * 4;
  if (dev < kMaxDevices && cache[dev] > 0) return cache[dev];
  int bytes = 0;
  if (hipDeviceGetAttribute(&bytes, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
      bytes <= 0)
    bytes = kLdsInts * 4;
  if (dev < kMaxDevices) cache[dev] = bytes;
  return bytes;
}

// Tiles of at least kMinTile pairs; at most 2^20 / (L E) of them, so that the
// per-tile counts fit a fixed workspace bound (4 MiB).
#ifndef MLR_ALIGN_MIN_TILE
#define MLR_ALIGN_MIN_TILE 512
#endif
constexpr int64_t kMinTile = MLR_ALIGN_MIN_TILE;

AlignPlan plan_align(int64_t numel, int E, int L, int B) {
  (void)B;
  AlignPlan pl{};
  pl.pass_slots = L;
  if (numel <= kAlignWaveMaxPairs && L <= kAlignWaveMaxSlots) {
    pl.wave = true;   // keys are matched by votes: any key range in one pass
    pl.threads = kWave;
    return pl;
  }
  // The LDS tables hold at most kAlignPassKeys (slot, expert) keys; more
  // slots are taken in passes over slot ranges (each pass reads every pair
  // and keeps those of its slots).
  if (int64_t(L) * E > kAlignPassKeys) pl.pass_slots = std::max(1, kAlignPassKeys / E);
  L = pl.pass_slots;
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
  const int64_t max_tiles = std::max<int64_t>(1, std::min<int64_t>(1024, (int64_t(1) << 20) / LE));
  int64_t tile = std::max<int64_t>(kMinTile, cdiv(numel, max_tiles));
  tile = cdiv(tile, kWave) * kWave;
  pl.seg = int(tile);
  pl.ntiles = int(cdiv(numel, tile));
  pl.threads = int(std::min<int64_t>(1024, tile));               // count kernel
  pl.lds_bytes = size_t(LE * 4);
  pl.ws_bytes = (int64_t(pl.ntiles) + 1) * LE * 4;   // tile counts, then key totals
  return pl;
}

// Active slots from num_tokens_post_padded (one wavefront): ascending, then -1.
__global__ void __launch_bounds__(kWave) align_active_kernel(const int32_t* ntpp, int L,
                                                             int32_t* lora_ids, int32_t* nact) {
  const int lane = lane_id();
  int run = 0;
  for (int c0 = 0; c0 < L; c0 += kWave) {
    const int l = c0 + lane;
    const bool act = l < L && ntpp[l] > 0;
    const uint64_t mk = __ballot(act);
    if (act && lora_ids) lora_ids[run + __popcll(mk & lanes_below(lane))] = l;
    run += __popcll(mk);
  }
  if (lora_ids)
    for (int i = run + lane; i < L; i += kWave) lora_ids[i] = -1;
  if (nact && lane == 0) *nact = run;
}

hipError_t launch_align_active(const int32_t* ntpp, int L, int32_t* lora_ids, int32_t* nact,
                               hipStream_t st) {
  hipLaunchKernelGGL(align_active_kernel, dim3(1), dim3(kWave), 0, st, ntpp, L, lora_ids, nact);
  return hipGetLastError();
}

hipError_t launch_align(const AlignPlan& pl, AlignParams a, hipStream_t st) {
  if (pl.wave) {
    hipLaunchKernelGGL(align_wave_kernel, dim3(1), dim3(kWave), 0, st, a);
    return hipGetLastError();
  }
  if (pl.single) {
    hipLaunchKernelGGL(align_single_kernel, dim3(1), dim3(pl.threads), pl.lds_bytes, st, a);
    return hipGetLastError();
  }
  // prefix kernel: 64 keys per workgroup, enough wavefronts (at most 16)
  // that each sums at most 16 tiles where the tile count allows
  const int prefix_waves = int(std::min<int64_t>(16, cdiv(a.ntiles, kKeyBatch)));
  // scatter kernel: as many per-wave rows as LDS holds beside the layout
  // tables (at most 16), each wave owning an equal run of the tile (a
  // multiple of 64 pairs)
  const int64_t fixed_ints = int64_t(a.LE) + a.L + 1 + 17;
  auto fit_rows = [&](int64_t lds_bytes) {
    int w = int(std::max<int64_t>(
        1, std::min<int64_t>(MLR_ALIGN_MAX_ROWS, (lds_bytes / 4 - fixed_ints) / a.LE)));
    w = int(std::min<int64_t>(w, cdiv(a.seg, kWave)));
    a.segw = int(cdiv(cdiv(a.seg, w), kWave) * kWave);
    a.W = int(cdiv(a.seg, a.segw));
  };
  fit_rows(lds_per_block());
  if ((fixed_ints + int64_t(a.W) * a.LE) * 4 > kLdsInts * 4 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(align_tile_scatter_kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          int((fixed_ints + int64_t(a.W) * a.LE) * 4)) != hipSuccess) {
    (void)hipGetLastError();   // keep within the 64 KiB every launch may take
    fit_rows(kLdsInts * 4);
  }
  const size_t scatter_lds = size_t(fixed_ints + int64_t(a.W) * a.LE) * 4;
  hipLaunchKernelGGL(align_tile_count_kernel, dim3(pl.ntiles), dim3(pl.threads), pl.lds_bytes,
                     st, a);
  hipLaunchKernelGGL(align_prefix_kernel, dim3(unsigned(cdiv(a.LE, kWave))),
                     dim3(prefix_waves * kWave), 0, st, a);
  hipLaunchKernelGGL(align_tile_scatter_kernel, dim3(pl.ntiles), dim3(a.W * kWave), scatter_lds,
                     st, a);
  return hipGetLastError();
}

}  // namespace mlr
