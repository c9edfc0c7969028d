// Fused shrink + expand with vector loads and wavefront reductions (the
// decode-sized path).  One workgroup handles one (block, slice, column split):
//
//   shrink  v[i][j] = sum_t X[row_i][t] A[j][t].  The wavefronts form RGW row
//           groups x KP partitions of K.  A wavefront owns JW rows of A and
//           walks its part of K in 16-byte chunks, lanes side by side (one
//           wavefront load reads 1 KiB of one A row).  All row loads of a step
//           are issued before any is used, so every lane keeps up to 16 loads
//           in flight.  bf16 pairs are multiplied with v_dot2; the 64 lane
//           partials are folded with a reduce-scatter butterfly and the KP
//           partial sums are added in LDS.
//   v       stays on chip (LDS, fp32); it never goes to global memory.
//   expand  d[i][n] = sum_j v[i][j] B[n][j].  For r in {8,...,128} the B tile
//           of the split (consecutive rows n, r contiguous) is read as one
//           coalesced stream of 16-byte chunks; a lane always sees the same
//           8 ranks, keeps those v values in registers, and the partial sums
//           of one row are folded over the r/8 lanes that share it.  Other
//           ranks take one thread per column.
//
// The prhub summary of vLLM PR #42290 (implementation steps) describes the
// one-shot kernel: x loaded once, multiplied by lora_a, the rank-sized result
// kept in registers and multiplied by lora_b, written over or added onto the
// output.  Here several workgroups share a block by splitting its output
// columns (each redoes the small shrink), so that a decode batch with few
// active groups still spreads over the chip.  The split count is chosen on
// the device from the number of blocks actually present, and the splits of a
// block get workgroup ids of equal residue mod 8, which places them on one XCD
// where they re-read A from its L2.
#include <algorithm>

#include "blocks.h"
#include "common.h"
#include "align_wave.h"
#include "groups.h"
#include "internal.h"

// Launch shape.  The defaults were picked by timing the decode shapes on
// MI355X; they can be overridden when building to re-tune.
#ifndef MLR_VALU_LOADS       // A rows loaded per wavefront per step (x RG <= 32)
#define MLR_VALU_LOADS 16
#endif
#ifndef MLR_VALU_MIN_COLS    // fewest output columns per split
#define MLR_VALU_MIN_COLS 256
#endif
#ifndef MLR_VALU_OCC         // workgroups per compute unit the split count plans for
#define MLR_VALU_OCC 1
#endif

// Two workgroup sizes: 512 threads for rank 16, 1024 for the other ranks.
// Measured on MI355X (graph-timed per call): 512 threads on the
// gpt-oss-120b-like decode w13 9.9 us against 11.4, w2 9.5 against 10.9, and
// 23.2 against 32.0 at 64 tokens; 1024 threads for ranks 8, 24 and 64
// (K > 4096), where 512 were 7 to 12 percent slower.
namespace mlr {
namespace valu1024 {
#define MLR_VALU_T 1024
#include "fused_valu_body.h"
#undef MLR_VALU_T
}  // namespace valu1024
namespace valu512 {
#define MLR_VALU_T 512
#define MLR_VALU_R16_ONLY
#include "fused_valu_body.h"
#undef MLR_VALU_R16_ONLY
#undef MLR_VALU_T
}  // namespace valu512

#ifndef MLR_VALU_STREAM  // decode shapes the stream kernel supports go there
#define MLR_VALU_STREAM 1
#endif

// r = 16 stays here: the stream has few stages per workgroup and the
// register-batch kernel was measured faster (gpt-oss-120b-like decode w13
// 12.4 vs 13.4 us; re-measured later, 7.5 vs 13.3 one launch and 7.2 vs
// 12.7 sorted); from r = 32 on the stream kernel is (20b-like a2..a4:
// 27.8 vs 33.8 us).  stream_supported() admits r in {32, 64, 128}.
bool valu_takes_stream(int64_t M, int64_t numel, int64_t K, int64_t N, int r, int x_per_pair) {
  return MLR_VALU_STREAM && stream_supported(M, numel, K, N, r, x_per_pair);
}

hipError_t launch_fused_valu(FusedParams p, hipStream_t st) {
  if (valu_takes_stream(p.numel / p.topk, p.numel, p.K, p.N, p.r, p.x_per_pair))
    return launch_fused_stream(p, st);
  return p.r == 16 ? valu512::launch_valu(p, st) : valu1024::launch_valu(p, st);
}

}  // namespace mlr
