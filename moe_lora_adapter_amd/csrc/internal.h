// Host-side declarations shared by the translation units of libmoelora.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlr {

// ---------------------------------------------------------------- align
struct AlignParams {
  const int32_t* topk_ids;
  const int32_t* mapping;
  int32_t* sorted;    // [L, cap]
  int32_t* eids;      // [L, nb]
  int32_t* ntpp;      // [L]
  int32_t* lora_ids;  // [L] or null
  int32_t* nact;      // [1] or null
  int32_t* tile_cnt;  // [ntiles, LE]  (multi-workgroup path)
  int32_t* key_tot;   // [LE]
  int32_t numel, topk, E, L, LE, B, nbits;
  int32_t cap, nb;
  int32_t W;       // waves that own a pair segment, per workgroup
  int32_t seg;     // single workgroup: pairs per wave; tiles: pairs per tile
  int32_t ntiles;  // workgroups of the tile kernels
  int32_t segw;    // tile scatter: pairs per wave (multiple of 64)
  int32_t l0;      // first slot of this pass: slots [l0, l0 + L) of the call,
                   // whose rows sorted / eids / ntpp point at
};

struct AlignPlan {
  bool wave;         // one wavefront does everything (at most 64 pairs and 64 slots)
  bool single;       // one workgroup does everything
  int W, seg, ntiles;
  int threads;       // block size of the single / tile count kernels
  size_t lds_bytes;  // dynamic LDS of the single / tile count kernels
  int64_t ws_bytes;  // device workspace (0 for the single path)
  int pass_slots;    // slots per pass: the call's L, or fewer when L * E keys
                     // exceed what the LDS tables of one pass hold
};

// The one-wavefront align (lane = pair, lane = slot) takes at most this many.
constexpr int kAlignWaveMaxPairs = 64;
constexpr int kAlignWaveMaxSlots = 64;
// (slot, expert) keys one pass of the LDS-table align paths takes.
constexpr int kAlignPassKeys = 8192;

AlignPlan plan_align(int64_t numel, int E, int L, int B);
hipError_t launch_align(const AlignPlan& plan, AlignParams a, hipStream_t st);
// lora_ids / num_active from num_tokens_post_padded (after passes that
// wrote them for slot ranges without those outputs).
hipError_t launch_align_active(const int32_t* ntpp, int L, int32_t* lora_ids, int32_t* nact,
                               hipStream_t st);

// ---------------------------------------------------------------- fused
struct FusedParams {
  const uint16_t* x;
  const uint16_t* a;   // [S, L, E, r, K]
  const uint16_t* b;   // [S, L, E, Ns, r]
  const int32_t* sorted;
  const int32_t* eids;
  const int32_t* ntpp;
  const int32_t* topk_ids;  // align-free path: [numel]
  const int32_t* mapping;   // align-free path: [numel / topk]
  const float* w;      // [numel] or null
  uint16_t* y;         // [numel, N]
  int32_t x_per_pair, mul, add;
  int32_t numel, topk, K, Ns, S, E, L, r, B, N;
  int32_t cap, nb;
  int32_t units;       // upper bound on blocks, times S
  int32_t xcd_cus;     // compute units per XCD of the current device
  int32_t naive;       // 1: blocks formed on chip from topk_ids and mapping (no align outputs)
  int32_t nbits;       // align-free path: bits of a key l * E + e
  // fused_moe_lora_with_align: the align outputs one workgroup writes
  // beside the fused work; null when there is none
  int32_t* al_sorted;
  int32_t* al_eids;
  int32_t* al_ntpp;
  int32_t* al_lora_ids;
  int32_t* al_nact;
  int32_t* xch;        // stream kernel: K-split exchange area (xch.h; null: no K split)
  int32_t xch_nslot;   // slots the exchange area holds (its layout depends on this alone)
  int32_t xch_passes;  // exchange slots per unit: one per pass of kXchRows rows
  int32_t peer_wait;   // stream kernel: polls for a peer's partial before computing it here
  float* ws;           // two-kernel path: partial rank vectors, fp32 [kz, S, numel, r]
  int32_t kz;          // two-kernel path: K splits of the shrink
  int32_t kchunk;      // two-kernel path: K per split (a multiple of 32)
};

// Largest rank of the two-kernel path, and the ranks of one shrink workgroup.
constexpr int kMaxRankTwoKernel = 512;
constexpr int kTwoKernelRankGroup = 128;

// Polls for a peer's partial in the stream kernel's K split before the
// workgroup computes it itself (each poll is one round trip plus a short
// sleep, about 0.7 us).
constexpr int kDefaultPeerWait = 64;

// Most pairs the align-free path groups (one per thread of a workgroup).
constexpr int64_t kNaiveMaxPairs = 1024;

// Upper bound on the number of blocks over all slots: every non-empty
// (slot, expert) group adds at most block_m - 1 padding entries.
inline int64_t max_total_blocks(int64_t numel, int64_t LE, int64_t B) {
  const int64_t groups = numel < LE ? numel : LE;
  return (numel + groups * (B - 1)) / B;
}

// Compute units per XCD of the current device (cached per device).
int xcd_compute_units();

hipError_t launch_fused_valu(FusedParams p, hipStream_t st);
hipError_t launch_fused_mfma(FusedParams p, hipStream_t st);
hipError_t launch_fused_stream(FusedParams p, hipStream_t st);
// Slots of the K-split exchange a launch of `units` units uses (one per unit
// and pass of four rows).
inline int64_t exchange_passes(int64_t block_m) { return (block_m + 3) / 4; }
bool stream_supported(int64_t M, int64_t numel, int64_t K, int64_t N, int r, int x_per_pair);
// Whether the vector variant runs the stream kernel for these sizes.
bool valu_takes_stream(int64_t M, int64_t numel, int64_t K, int64_t N, int r, int x_per_pair);
bool mfma_supported(int r, int B);
// Two-kernel path: K splits of the shrink for these sizes, and the launch of
// shrink then expand (p.ws, p.kz, p.kchunk set by the caller).
int two_kernel_splits(int64_t units_bound, int64_t K, int r);
hipError_t launch_two_kernel(FusedParams p, hipStream_t st);
bool two_kernel_fits(int64_t x_bytes, int64_t r, int64_t K, int64_t Ns);

// ---------------------------------------------------------------- join step
hipError_t launch_accumulate(uint16_t* y, const uint16_t* d, int64_t n, hipStream_t st);
bool mfma_fits(int64_t x_bytes, int64_t y_bytes, int64_t r, int64_t K, int64_t Ns);

}  // namespace mlr
