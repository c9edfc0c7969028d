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
#include "internal.h"

namespace mlr {

// Launch shape.  The defaults were picked by timing the decode shapes on
// MI355X; they can be overridden when building to re-tune.
#ifndef MLR_VALU_THREADS
#define MLR_VALU_THREADS 1024
#endif
#ifndef MLR_VALU_WG_TARGET   // working workgroups to aim for
#define MLR_VALU_WG_TARGET 192
#endif
#ifndef MLR_VALU_LOADS       // A rows loaded per wavefront per step (x RG <= 32)
#define MLR_VALU_LOADS 16
#endif
#ifndef MLR_VALU_MIN_COLS    // fewest output columns per split
#define MLR_VALU_MIN_COLS 256
#endif
constexpr int kThreads = MLR_VALU_THREADS;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxB = 128;
constexpr int kMaxR = 128;
constexpr int kMaxRG = 4;    // X rows per group

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Sum NV per-lane values over the wavefront.  On return the lane holds the
// total of value index `which`; lanes whose index bits agree hold the same.
template <int NV>
__device__ __forceinline__ float reduce_scatter(float (&v)[NV], int& which) {
  static_assert(NV >= 1 && NV <= kWave && (NV & (NV - 1)) == 0, "NV: power of two <= 64");
  const int lane = lane_id();
  which = 0;
  int o = kWave / 2;
#pragma unroll
  for (int half = NV / 2; half >= 1; half >>= 1, o >>= 1) {
    const bool up = lane & o;
    // select on the values (bit masks), not on array indices: an index
    // select would turn v into a dynamically indexed (scratch) array
    const uint32_t m = up ? 0xffffffffu : 0u;
#pragma unroll
    for (int q = 0; q < half; ++q) {
      const uint32_t lo = __float_as_uint(v[q]), hi = __float_as_uint(v[q + half]);
      const float send = __uint_as_float((lo & m) | (hi & ~m));
      const float keep = __uint_as_float((hi & m) | (lo & ~m));
      v[q] = keep + __shfl_xor(send, o);
    }
    if (up) which += half;
  }
  float t = v[0];
  for (; o >= 1; o >>= 1) t += __shfl_xor(t, o);
  return t;
}

struct ShrinkShape {
  int rgw;    // row groups of wavefronts
  int kp;     // K partitions
};

// One wavefront: JW rows of A starting at j0 (rows >= r are loaded clamped and
// dropped), K chunks [c0, c1), RG X rows.  Writes RG x JW partial sums to
// part[(i) * r + j] of its K partition.
template <int RG, int JW>
__device__ __forceinline__ void shrink_wave(const FusedParams& p, const uint16_t* __restrict__ A,
                                            const uint16_t* const (&xr)[kMaxRG], int j0, int c0,
                                            int c1, float* part) {
  const int lane = lane_id();
  float acc[RG * JW];
#pragma unroll
  for (int q = 0; q < RG * JW; ++q) acc[q] = 0.f;
  const uint16_t* arow[JW];
#pragma unroll
  for (int jj = 0; jj < JW; ++jj) arow[jj] = A + int64_t(min(j0 + jj, p.r - 1)) * p.K;
#pragma unroll 1
  for (int c = c0 + lane; c < c1; c += kWave) {
    uint4 av[JW];
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) av[jj] = ld16(arow[jj] + c * 8);
    uint4 xv[RG];
#pragma unroll
    for (int i = 0; i < RG; ++i) xv[i] = ld16(xr[i] + c * 8);
    // every load of the step is issued before the first product waits
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jj = 0; jj < JW; ++jj)
#pragma unroll
      for (int i = 0; i < RG; ++i) acc[i * JW + jj] = dot8_bf16(av[jj], xv[i], acc[i * JW + jj]);
  }
  int which;
  const float t = reduce_scatter<RG * JW>(acc, which);
  if ((lane & (kWave / (RG * JW) - 1)) == 0) {
    const int i = which / JW, j = j0 + which % JW;
    if (j < p.r) part[i * p.r + j] = t;
  }
}

// v[i][j] for the RG rows of a group into s_v (fp32, row stride kMaxR).
template <int RG, int JW>
__device__ __forceinline__ void shrink_group(const FusedParams& p, const uint16_t* __restrict__ A,
                                             const int* s_row, int nr, ShrinkShape sh,
                                             float* s_part, float* s_v) {
  constexpr int JL = JW < MLR_VALU_LOADS ? JW : MLR_VALU_LOADS;
  constexpr int JB = (RG * JL > 32) ? 32 / RG : JL;
  const int w = wave_id();
  const int rg = w % sh.rgw, kpi = w / sh.rgw;
  const uint16_t* xr[kMaxRG];
#pragma unroll
  for (int i = 0; i < kMaxRG; ++i)
    xr[i] = p.x + int64_t(__builtin_amdgcn_readfirstlane(s_row[i < nr ? i : 0])) * p.K;
  const int K8 = p.K >> 3;
  if (kpi < sh.kp) {
    const int per = (K8 + sh.kp - 1) / sh.kp;
    const int c0 = kpi * per, c1 = min(K8, c0 + per);
    for (int j0 = rg * JW; j0 < p.r; j0 += sh.rgw * JW)
      for (int jb = j0; jb < min(j0 + JW, p.r); jb += JB)
        shrink_wave<RG, JB>(p, A, xr, jb, c0, c1, s_part + kpi * RG * p.r);
  }
  __syncthreads();
  for (int t = threadIdx.x; t < nr * p.r; t += kThreads) {
    const int i = t / p.r, j = t - i * p.r;
    float sum = 0.f;
    for (int q = 0; q < sh.kp; ++q) sum += s_part[(q * RG + i) * p.r + j];
    s_v[i * kMaxR + j] = sum;
  }
  __syncthreads();
}

// Per-row output scale: the routed weight, or 1.
template <int RG>
__device__ __forceinline__ void row_scales(const FusedParams& p, const int* s_pair, int nr,
                                           float (&wt)[RG]) {
#pragma unroll
  for (int i = 0; i < RG; ++i) wt[i] = (p.mul && i < nr) ? p.w[s_pair[i]] : 1.f;
}

// Y[pair, col] = bf16(w * d + (add ? y : 0)) for the valid rows of a group;
// y holds the bf16 input values, loaded earlier.
template <int RG>
__device__ __forceinline__ void store_out(const FusedParams& p, const int* s_pair, int nr,
                                          int col, const float (&d)[RG], const float (&wt)[RG],
                                          const uint16_t (&y)[RG]) {
#pragma unroll
  for (int i = 0; i < RG; ++i) {
    if (i < nr) {
      float val = d[i] * wt[i];
      if (p.add) val += bf16_to_f32(y[i]);
      p.y[int64_t(s_pair[i]) * p.N + col] = f32_to_bf16(val);
    }
  }
}

template <int RG>
__device__ __forceinline__ void load_y(const FusedParams& p, const int* s_pair, int nr, int col,
                                       uint16_t (&y)[RG]) {
#pragma unroll
  for (int i = 0; i < RG; ++i)
    y[i] = (p.add && i < nr) ? p.y[int64_t(s_pair[i]) * p.N + col] : uint16_t(0);
}

// Expand for r == 8 * CPR: the B tile rows [n0, n1) read as one coalesced
// stream of 16-byte chunks.  Chunk q of the tile is row q / CPR, ranks
// 8 * (q % CPR) .. +8; since the thread count is a multiple of CPR a thread
// always sees the same eight ranks.  The row sums land in LDS (s_d), and the
// epilogue then reads Y and writes it back in 16-byte pieces (8 columns per
// thread), the Y reads issued before the B chunks are consumed.
constexpr int kRowsPerBatch = 2048;

template <int RG, int CPR>
__device__ __forceinline__ void expand_stream(const FusedParams& p, const uint16_t* __restrict__ Bm,
                                              const int* s_pair, int nr, const float* s_v, int s,
                                              int n0, int n1, float* s_d) {
  // chunk loads in flight per thread; one batch covers at most kRowsPerBatch rows
  constexpr int NB0 = RG <= 2 ? 16 : 8;
  constexpr int NBR = kRowsPerBatch * CPR / kThreads;
  constexpr int NB = NB0 < NBR ? NB0 : (NBR > 0 ? NBR : 1);
  const int tid = threadIdx.x;
  const int jc = tid % CPR;
  float vr[RG][8];
#pragma unroll
  for (int i = 0; i < RG; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q) vr[i][q] = s_v[i * kMaxR + jc * 8 + q];
  float wt[RG];
  row_scales<RG>(p, s_pair, nr, wt);
  const uint16_t* tile = Bm + int64_t(n0) * p.r;
  const int nchunks = (n1 - n0) * CPR;
  const int col0 = s * p.Ns + n0;
#pragma unroll 1
  for (int base = 0; base < nchunks; base += NB * kThreads) {
    const int rows = min(NB * kThreads, nchunks - base) / CPR;  // columns in this batch
    const int row0 = base / CPR;
    // epilogue task of this thread: row i, 8 columns starting at 8 * c8
    const int c8n = rows / 8;
    const int task_i = tid / max(c8n, 1), task_c = tid - task_i * max(c8n, 1);
    const bool has_task = c8n > 0 && task_i < nr;
    uint4 yv = make_uint4(0, 0, 0, 0);
    uint16_t* yp = nullptr;
    if (has_task) {
      yp = p.y + int64_t(s_pair[task_i]) * p.N + col0 + row0 + task_c * 8;
      if (p.add) yv = *reinterpret_cast<const uint4*>(yp);
    }
    uint4 bv[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int q = min(base + k * kThreads + tid, nchunks - 1);
      bv[k] = ld16(tile + int64_t(q) * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int q = base + k * kThreads + tid;
      const uint4 b4 = bv[k];
      const float b[8] = {bf16_lo(b4.x), bf16_hi(b4.x), bf16_lo(b4.y), bf16_hi(b4.y),
                          bf16_lo(b4.z), bf16_hi(b4.z), bf16_lo(b4.w), bf16_hi(b4.w)};
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        float d = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) d += vr[i][t] * b[t];
#pragma unroll
        for (int o = CPR / 2; o >= 1; o >>= 1) d += __shfl_xor(d, o);
        if (jc == 0 && q < nchunks) s_d[i * kRowsPerBatch + q / CPR - row0] = d;
      }
    }
    __syncthreads();
    if (has_task) {
      const float* dd = s_d + task_i * kRowsPerBatch + task_c * 8;
      const float w = wt[task_i];
      const uint32_t in[4] = {yv.x, yv.y, yv.z, yv.w};
      uint32_t outw[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        float lo = dd[2 * h] * w, hi = dd[2 * h + 1] * w;
        if (p.add) {
          lo += bf16_lo(in[h]);
          hi += bf16_hi(in[h]);
        }
        outw[h] = uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
      }
      *reinterpret_cast<uint4*>(yp) = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    }
    __syncthreads();
  }
}

// Expand for any other rank: one thread per output column.
template <int RG>
__device__ __forceinline__ void expand_columns(const FusedParams& p, const uint16_t* __restrict__ Bm,
                                               const int* s_pair, int nr, const float* s_v, int s,
                                               int n0, int n1) {
  float wt[RG];
  row_scales<RG>(p, s_pair, nr, wt);
#pragma unroll 1
  for (int n = n0 + int(threadIdx.x); n < n1; n += kThreads) {
    uint16_t yv[RG];
    load_y<RG>(p, s_pair, nr, s * p.Ns + n, yv);
    const uint16_t* brow = Bm + int64_t(n) * p.r;
    float d[RG];
#pragma unroll
    for (int i = 0; i < RG; ++i) d[i] = 0.f;
    for (int j = 0; j < p.r; ++j) {
      const float bj = bf16_to_f32(brow[j]);
#pragma unroll
      for (int i = 0; i < RG; ++i) d[i] += s_v[i * kMaxR + j] * bj;
    }
    store_out<RG>(p, s_pair, nr, s * p.Ns + n, d, wt, yv);
  }
}

template <int RG, int JW, int CPR>
__global__ void __launch_bounds__(kThreads) fused_valu_kernel(FusedParams p, ShrinkShape sh) {
  __shared__ int s_pair[kMaxB];
  __shared__ int s_row[kMaxB];
  __shared__ float s_v[kMaxRG * kMaxR];
  __shared__ float s_part[kMaxRG * 256];
  __shared__ float s_d[CPR > 0 ? RG * kRowsPerBatch : 1];

  // The blocks present decide the split count: enough working workgroups to
  // fill the chip, at least MLR_VALU_MIN_COLS columns each.
  const int total = __builtin_amdgcn_readfirstlane(count_blocks(p));
  const int units = total * p.S;
  const int u8 = (units + kXcds - 1) / kXcds * kXcds;
  const int max_split = max(1, p.Ns / MLR_VALU_MIN_COLS);
  const int n_split = min(max_split, max(1, (MLR_VALU_WG_TARGET + u8 - 1) / max(u8, 1)));
  // workgroup -> (split, unit), split-major; equal unit residue mod 8 = same XCD
  const int id = blockIdx.x;
  const int split = id / max(u8, 1), unit = id - split * u8;
  if (unit >= units || split >= n_split) return;
  const int nsz = ((p.Ns + n_split - 1) / n_split + 7) / 8 * 8;
  const int n0 = split * nsz;
  if (n0 >= p.Ns) return;
  const int n1 = min(p.Ns, n0 + nsz);
  const int g = unit / p.S, s = unit - g * p.S;
  int l, b;
  find_block(p, g, l, b);
  l = __builtin_amdgcn_readfirstlane(l);
  b = __builtin_amdgcn_readfirstlane(b);
  const int e = __builtin_amdgcn_readfirstlane(p.eids[l * p.nb + b]);
  const int64_t wsel = (int64_t(s) * p.L + l) * p.E + e;
  const uint16_t* A = p.a + wsel * p.r * p.K;
  const uint16_t* Bm = p.b + wsel * p.Ns * p.r;

  const int tid = threadIdx.x;
  int valid = 0;
  if (tid < p.B) {
    const int pid = p.sorted[l * p.cap + b * p.B + tid];
    valid = pid < p.numel;
    s_pair[tid] = pid;
    s_row[tid] = valid ? (p.x_per_pair ? pid : pid / p.topk) : 0;
  }
  // valid rows form a prefix of the block (sentinels only pad a group's end)
  const int nv = __builtin_amdgcn_readfirstlane(__syncthreads_count(valid));

  // rows in groups of RG (a group with fewer valid rows repeats row 0 and
  // drops its sums)
  for (int g0 = 0; g0 < nv; g0 += RG) {
    const int nr = min(RG, nv - g0);
    shrink_group<RG, JW>(p, A, s_row + g0, nr, sh, s_part, s_v);
      if constexpr (CPR > 0)
      expand_stream<RG, CPR>(p, Bm, s_pair + g0, nr, s_v, s, n0, n1, s_d);
    else
      expand_columns<RG>(p, Bm, s_pair + g0, nr, s_v, s, n0, n1);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Pipelined variant for r in {8, ..., 128} and blocks of at most two valid
// rows per group (the decode case).  512 threads; every thread works through
// one stream: its A chunks (the shrink) followed by its B chunks (the
// expand), 16 loads per stage, two stages in flight.  The B chunks of the
// first expand stage are already loading while the last shrink stage is
// multiplied and v is finished, so the step from shrink to expand costs no
// memory round trip; the Y values of the epilogue are loaded right after the
// block metadata.
constexpr int kPThreads = 512;
constexpr int kPWaves = kPThreads / kWave;
constexpr int kDepth = 16;        // 16-byte loads per thread and stage
constexpr int kPMaxCols = 2048;   // output columns per workgroup (s_d size)
#ifndef MLR_PIPE_WG_TARGET
#define MLR_PIPE_WG_TARGET 240
#endif

struct PipeCtx {
  const uint16_t* A;
  const uint16_t* tile;   // B rows [n0, n1) of this split
  int n0, n1, s;
  int nchunks;            // (n1 - n0) * CPR
};

// One pass over rows [g0, g0 + nr) of a block (nr <= RG): the shrink stream
// over A, then the expand stream over the B tile, two stages of D loads per
// thread in flight.
template <int RG, int JW, int CPR, int D>
__device__ __forceinline__ void pipe_rows(const FusedParams& p, const PipeCtx& c,
                                          const int* s_pair, const int* s_row, int g0, int nr,
                                          float* s_part, float* s_v, float* s_d) {
  static_assert(JW <= D && D <= kDepth && RG * JW <= 32, "stage shape");
  const int tid = threadIdx.x, w = wave_id(), lane = lane_id();
  // wave arrangement: rgw groups of JW rows x kp partitions of K
  const int rgw = min(kPWaves, (p.r + JW - 1) / JW);  // rgw * JW >= r: callers ensure r <= 8 * JW
  const int kp = max(1, kPWaves / rgw);
  const int rgi = w % rgw, kpi = w / rgw;
  const bool shrinker = kpi < kp;
  const int K8 = p.K >> 3;
  const int per = (K8 + kp - 1) / kp;
  const int c0 = shrinker ? kpi * per : 0;
  const int c1 = shrinker ? min(K8, c0 + per) : 0;
  const int nA = (c1 - c0 + kWave - 1) / kWave;
  const int j0 = rgi * JW;
  const int jlast = p.r - 1;
  const __amdgpu_buffer_rsrc_t a_rs = make_rsrc(c.A, uint32_t(p.r) * p.K * 2u);
  const __amdgpu_buffer_rsrc_t b_rs = make_rsrc(c.tile, uint32_t(c.nchunks) * 16u);
  const __amdgpu_buffer_rsrc_t none_rs = make_rsrc(c.tile, 0u);
  const int nB = (c.nchunks + D * kPThreads - 1) / (D * kPThreads);
  const int ns = nA + nB;
  const int jc = tid % CPR;
  const int ncol8 = (c.n1 - c.n0) / 8;
  const int col0 = c.s * p.Ns + c.n0;

  __amdgpu_buffer_rsrc_t x_rs[RG];
#pragma unroll
  for (int i = 0; i < RG; ++i)
    x_rs[i] = make_rsrc(p.x + int64_t(__builtin_amdgcn_readfirstlane(s_row[g0 + (i < nr ? i : 0)])) * p.K,
                        uint32_t(p.K) * 2u);
  // epilogue tasks: (row i, columns 8 * c8 .. +8), up to NT per thread; the
  // Y values are loaded now and used at the end
  constexpr int NT = (RG * (kPMaxCols / 8) + kPThreads - 1) / kPThreads;
  const int ntask = nr * ncol8;
  uint4 yv[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int t = tid + u * kPThreads;
    yv[u] = make_uint4(0, 0, 0, 0);
    if (t < ntask && p.add) {
      const int ti = t / ncol8, tc = t - ti * ncol8;
      yv[u] = *reinterpret_cast<const uint4*>(p.y + int64_t(s_pair[g0 + ti]) * p.N + col0 + tc * 8);
    }
  }

  float acc[RG * JW];
#pragma unroll
  for (int q = 0; q < RG * JW; ++q) acc[q] = 0.f;
  // this lane's eight ranks of v as bf16 pairs, split v = hi + lo (hi the
  // nearest bf16, lo the nearest bf16 of the remainder): the expand then
  // runs on v_dot2 with the raw B pairs, to about 2^-17 relative of fp32 v
  uint32_t vhi[RG][4], vlo[RG][4];

  // One stage = D + RG loads, the same instruction sequence for shrink
  // and expand stages (only the descriptors and offsets differ), so the
  // compiler can count outstanding loads exactly.  Expand stages point the
  // X loads at an empty descriptor (they read zero and touch no memory).
  auto issue = [&](int st, uint4 (&buf)[D], uint4 (&xb)[RG]) {
    const bool is_a = st < nA;
    const uint32_t cb = uint32_t(min(c0 + lane + kWave * st, max(c1 - 1, 0))) * 16u;
    const uint32_t bb = uint32_t((st - nA) * (D * kPThreads) + tid) * 16u;
    const __amdgpu_buffer_rsrc_t rs = is_a ? a_rs : b_rs;
#pragma unroll
    for (int k = 0; k < D; ++k) {
      const uint32_t voff = is_a ? cb : bb + uint32_t(k * kPThreads) * 16u;
      const uint32_t soff = is_a ? uint32_t(min(j0 + min(k, JW - 1), jlast)) * uint32_t(p.K) * 2u : 0u;
      buf[k] = buf_ld16(rs, voff, soff);
    }
#pragma unroll
    for (int i = 0; i < RG; ++i) xb[i] = buf_ld16(is_a ? x_rs[i] : none_rs, cb, 0u);
  };
  auto finish_shrink = [&]() {
    if (shrinker) {
      int which;
      const float t = reduce_scatter<RG * JW>(acc, which);
      if ((lane & (kWave / (RG * JW) - 1)) == 0) {
        const int i = which / JW, j = j0 + which % JW;
        if (j < p.r) s_part[(kpi * RG + i) * p.r + j] = t;
      }
    }
    lds_barrier();
    for (int t = tid; t < nr * p.r; t += kPThreads) {
      const int i = t / p.r, j = t - i * p.r;
      float sum = 0.f;
      for (int q = 0; q < kp; ++q) sum += s_part[(q * RG + i) * p.r + j];
      s_v[i * kMaxR + j] = sum;
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < RG; ++i)
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float a = s_v[i * kMaxR + jc * 8 + 2 * h], b = s_v[i * kMaxR + jc * 8 + 2 * h + 1];
        const uint16_t ah = f32_to_bf16(a), bh = f32_to_bf16(b);
        const uint16_t al = f32_to_bf16(a - bf16_to_f32(ah)), bl = f32_to_bf16(b - bf16_to_f32(bh));
        vhi[i][h] = uint32_t(ah) | (uint32_t(bh) << 16);
        vlo[i][h] = uint32_t(al) | (uint32_t(bl) << 16);
      }
  };
  auto consume = [&](int st, const uint4 (&buf)[D], const uint4 (&xb)[RG]) {
    if (st < nA) {
      if (c0 + lane + kWave * st < c1) {
#pragma unroll
        for (int jj = 0; jj < JW; ++jj)
#pragma unroll
          for (int i = 0; i < RG; ++i) acc[i * JW + jj] = dot8_bf16(buf[jj], xb[i], acc[i * JW + jj]);
      }
      return;
    }
    const int base = (st - nA) * (D * kPThreads);
#pragma unroll
    for (int k = 0; k < D; ++k) {
      const int q = base + k * kPThreads + tid;
      const uint32_t bw[4] = {buf[k].x, buf[k].y, buf[k].z, buf[k].w};
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        float d = 0.f;
#pragma unroll
        for (int h = 0; h < 4; ++h) d = dot2_bf16(bw[h], vlo[i][h], dot2_bf16(bw[h], vhi[i][h], d));
#pragma unroll
        for (int o = CPR / 2; o >= 1; o >>= 1) d += __shfl_xor(d, o);
        if (jc == 0 && q < c.nchunks) s_d[i * kPMaxCols + q / CPR] = d;
      }
    }
  };

  // two stages in flight; v is finished right after the last shrink stage
  // is consumed, while the first expand stage is still loading
  uint4 buf0[D], buf1[D], xb0[RG], xb1[RG];
  issue(0, buf0, xb0);
  if (nA == 0) finish_shrink();
  for (int st = 0; st < ns; st += 2) {
    if (st + 1 < ns) issue(st + 1, buf1, xb1);
    __builtin_amdgcn_sched_barrier(0);
    consume(st, buf0, xb0);
    if (st == nA - 1) finish_shrink();
    if (st + 2 < ns) issue(st + 2, buf0, xb0);
    __builtin_amdgcn_sched_barrier(0);
    if (st + 1 < ns) {
      consume(st + 1, buf1, xb1);
      if (st + 1 == nA - 1) finish_shrink();
    }
  }
  lds_barrier();
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int t = tid + u * kPThreads;
    if (t < ntask) {
      const int ti = t / ncol8, tc = t - ti * ncol8;
      const float* dd = s_d + ti * kPMaxCols + tc * 8;
      const int pair = s_pair[g0 + ti];
      const float wt = p.mul ? p.w[pair] : 1.f;
      const uint32_t in[4] = {yv[u].x, yv[u].y, yv[u].z, yv[u].w};
      uint32_t outw[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        float lo = dd[2 * h] * wt, hi = dd[2 * h + 1] * wt;
        if (p.add) {
          lo += bf16_lo(in[h]);
          hi += bf16_hi(in[h]);
        }
        outw[h] = uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
      }
      *reinterpret_cast<uint4*>(p.y + int64_t(pair) * p.N + col0 + tc * 8) =
          make_uint4(outw[0], outw[1], outw[2], outw[3]);
    }
  }
  __syncthreads();
}

// Blocks of up to two valid rows take the 2-row pass (16 A rows per
// wavefront); larger blocks are taken four rows at a time (8 A rows per
// wavefront), so every decode block is one pass.
template <int CPR>
__global__ void __launch_bounds__(kPThreads) fused_valu_pipe_kernel(FusedParams p) {
  __shared__ int s_pair[kMaxB];
  __shared__ int s_row[kMaxB];
  __shared__ float s_v[4 * kMaxR];
  __shared__ float s_part[4 * 8 * kDepth];   // kp * RG * r <= 8 * RG * JW <= 8 * 32
  __shared__ float s_d[4 * kPMaxCols];

  const int total = __builtin_amdgcn_readfirstlane(count_blocks(p));
  const int units = total * p.S;
  const int u8 = (units + kXcds - 1) / kXcds * kXcds;
  const int min_split = (p.Ns + kPMaxCols - 1) / kPMaxCols;
  const int max_split = max(min_split, p.Ns / MLR_VALU_MIN_COLS);
  const int n_split = min(max_split, max(min_split, MLR_PIPE_WG_TARGET / max(u8, 1)));
  const int id = blockIdx.x;
  const int split = id / max(u8, 1), unit = id - split * u8;
  if (unit >= units || split >= n_split) return;
  const int nsz = ((p.Ns + n_split - 1) / n_split + 7) / 8 * 8;
  const int n0 = split * nsz;
  if (n0 >= p.Ns) return;
  const int n1 = min(p.Ns, n0 + nsz);
  const int g = unit / p.S, s = unit - g * p.S;
  int l, b;
  find_block(p, g, l, b);
  l = __builtin_amdgcn_readfirstlane(l);
  b = __builtin_amdgcn_readfirstlane(b);
  const int e = __builtin_amdgcn_readfirstlane(p.eids[l * p.nb + b]);
  const int64_t wsel = (int64_t(s) * p.L + l) * p.E + e;
  PipeCtx c;
  c.A = p.a + wsel * p.r * p.K;
  c.tile = p.b + wsel * p.Ns * p.r + int64_t(n0) * p.r;
  c.n0 = n0;
  c.n1 = n1;
  c.s = s;
  c.nchunks = (n1 - n0) * CPR;

  const int tid = threadIdx.x;
  int valid = 0;
  if (tid < p.B) {
    const int pid = p.sorted[l * p.cap + b * p.B + tid];
    valid = pid < p.numel;
    s_pair[tid] = pid;
    s_row[tid] = valid ? (p.x_per_pair ? pid : pid / p.topk) : 0;
  }
  const int nv = __builtin_amdgcn_readfirstlane(__syncthreads_count(valid));
  // the 4-row pass covers 8 wavefronts x 8 A rows = 64 ranks; r = 128 (CPR
  // 16) takes 2-row passes
  if (nv <= 2 || CPR > 8) {
    for (int g0 = 0; g0 < nv; g0 += 2)
      pipe_rows<2, 16, CPR, 16>(p, c, s_pair, s_row, g0, min(2, nv - g0), s_part, s_v, s_d);
  } else {
    for (int g0 = 0; g0 < nv; g0 += 4)
      pipe_rows<4, 8, CPR, 8>(p, c, s_pair, s_row, g0, min(4, nv - g0), s_part, s_v, s_d);
  }
}

template <int JW, int CPR>
static void launch(const FusedParams& p, ShrinkShape sh, int rg, dim3 grid, hipStream_t st) {
  if (rg == 2)
    hipLaunchKernelGGL((fused_valu_kernel<2, JW, CPR>), grid, dim3(kThreads), 0, st, p, sh);
  else
    hipLaunchKernelGGL((fused_valu_kernel<4, JW, CPR>), grid, dim3(kThreads), 0, st, p, sh);
}

hipError_t launch_fused_valu(FusedParams p, hipStream_t st) {
  // rows of A per wavefront and the wave arrangement
  int jw = 1;
  while (jw < p.r && jw < 16) jw <<= 1;
  ShrinkShape sh;
  sh.rgw = std::min(kWaves, (p.r + jw - 1) / jw);
  sh.kp = std::max(1, kWaves / sh.rgw);
  // grid: the most working workgroups any block count can ask for, plus the
  // padding of the unit count to a multiple of 8 per split
  const int64_t units_pad = (int64_t(p.units) + kXcds - 1) / kXcds * kXcds;
  const int64_t grid = MLR_VALU_WG_TARGET + units_pad;
  const int cpr = (p.r % 8 == 0 && ((p.r / 8) & (p.r / 8 - 1)) == 0) ? p.r / 8 : 0;
  // X rows per group: 2 when blocks are expected to hold few valid rows
  const int64_t groups = std::min<int64_t>(p.numel, int64_t(p.L) * p.E);
  const int rg = (p.numel <= 2 * groups + groups / 2) ? 2 : 4;
  if (rg == 2 && cpr > 0) {
    // pipelined kernel (decode-sized blocks)
    const dim3 pgrid(unsigned(MLR_PIPE_WG_TARGET + units_pad));
    switch (cpr) {
      case 1: hipLaunchKernelGGL(fused_valu_pipe_kernel<1>, pgrid, dim3(kPThreads), 0, st, p); break;
      case 2: hipLaunchKernelGGL(fused_valu_pipe_kernel<2>, pgrid, dim3(kPThreads), 0, st, p); break;
      case 4: hipLaunchKernelGGL(fused_valu_pipe_kernel<4>, pgrid, dim3(kPThreads), 0, st, p); break;
      case 8: hipLaunchKernelGGL(fused_valu_pipe_kernel<8>, pgrid, dim3(kPThreads), 0, st, p); break;
      default: hipLaunchKernelGGL(fused_valu_pipe_kernel<16>, pgrid, dim3(kPThreads), 0, st, p); break;
    }
    return hipGetLastError();
  }
#define MLR_CASE(JW_, CPR_) \
  if (jw == JW_ && cpr == CPR_) { launch<JW_, CPR_>(p, sh, rg, dim3(unsigned(grid)), st); return hipGetLastError(); }
  MLR_CASE(16, 16)
  MLR_CASE(16, 8)
  MLR_CASE(16, 4)
  MLR_CASE(16, 2)
  MLR_CASE(8, 1)
  MLR_CASE(16, 0)
  MLR_CASE(8, 0)
  MLR_CASE(4, 0)
  MLR_CASE(2, 0)
  MLR_CASE(1, 0)
#undef MLR_CASE
  return hipErrorInvalidValue;
}

}  // namespace mlr
