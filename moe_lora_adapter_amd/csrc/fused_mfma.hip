// Fused shrink + expand on bf16 MFMA tiles (the prefill-sized path).
//
// One workgroup (4 wavefronts) handles one (block, slice, column split); the
// rows of a block are taken up to 64 at a time (a "pass"), in 1, 2 or 4 row
// tiles of 16 depending on how many of them hold valid pairs.
//
//   shrink  V[rows x r] = X[rows x K] . A[s,l,e][r x K]^T on
//           v_mfma_f32_16x16x32_bf16.  K is streamed in stages of 64 (128 when
//           the four wavefronts split K) through a ring of three LDS slots
//           filled by buffer loads that write LDS directly: two stages are in
//           flight while the third is multiplied, and no VGPR holds the
//           staged data.  Rows of a stage are stored with their 16-byte chunks
//           XOR-permuted by the row index, so the MFMA operand reads of 16
//           rows spread over the LDS banks.  Loads past the end of a buffer
//           return zero, which pads invalid rows, ranks >= r and the K tail.
//   v       goes to LDS as two bf16 parts, V = V_hi + V_lo (V_hi = bf16(V),
//           V_lo = bf16(V - V_hi)); it never leaves the chip.
//   expand  every wavefront holds both parts of V for all rows of the pass as
//           MFMA operands and takes a share of the output columns.  The
//           product is formed transposed, D^T = B[cols] . (V_hi + V_lo)^T (two
//           MFMAs per k-step, so v enters with about 16 significant bits
//           rather than bf16's 8), so that a lane ends with four
//           consecutive output columns of one row: the routed weight, the
//           add onto Y and the bf16 rounding happen in registers and Y is
//           read and written 8 bytes per lane.  B and Y of the next column
//           group are loaded while the current one is multiplied.
//
// Operand layouts of v_mfma_f32_16x16x32_bf16 (wave64): lane l supplies row
// l % 16 of A and column l % 16 of B, each with eight consecutive k values
// starting at 8 * (l / 16) (any k order works as long as A and B agree, since
// the instruction sums over k); the 16x16 fp32 result has element i of lane l
// at row 4 * (l / 16) + i, column l % 16.
//
// The prhub summary of vLLM PR #42290 (implementation steps, key source
// fragment) describes the one-shot kernel: x loaded once, shrink by lora_a,
// the rank vector kept on chip (BLOCK_R, rank <= 128), expand by lora_b,
// written over or added onto the output.
#include <algorithm>

#include "blocks.h"
#include "common.h"
#include "dma.h"
#include "align_wave.h"
#include "groups.h"
#include "internal.h"

namespace mlr {
namespace {

#ifndef MLR_MFMA_THREADS
#define MLR_MFMA_THREADS 256
#endif
constexpr int kThreadsM = MLR_MFMA_THREADS;
constexpr int kWavesM = kThreadsM / kWave;
constexpr int kPassRows = 64;
constexpr int kMaxIdsM = 128;  // largest block_m
constexpr int64_t kMaxXBytes = int64_t(1) << 31;

#ifndef MLR_MFMA_CTW_BUDGET  // expand: column tiles per wavefront and group x row tiles x k-steps
#define MLR_MFMA_CTW_BUDGET 8
#endif
#ifndef MLR_MFMA_MIN_COLS
#define MLR_MFMA_MIN_COLS 256
#endif
#ifndef MLR_MFMA_STAGE_BYTES  // most bytes of X and A rows per ring stage
#define MLR_MFMA_STAGE_BYTES 24576
#endif
#ifndef MLR_MFMA_OCCUPANCY  // workgroups per compute unit the split count assumes
#define MLR_MFMA_OCCUPANCY 2
#endif

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Shrink layout of a pass with MT row tiles and RT rank tiles (16 each).
// The 4 wavefronts are arranged as MT row tiles x WR rank groups x WK parts
// of K; a wavefront owns one row tile and TR rank tiles.
template <int MT, int RT>
struct Shrink {
  static constexpr int RB = 16 * MT;                                // rows
  static constexpr int RP = 16 * RT;                                // A rows staged
  static constexpr int WR = RT < kWavesM / MT ? RT : kWavesM / MT;  // rank groups
  static constexpr int WK = kWavesM / (MT * WR);                    // K parts
  static constexpr int TR = (RT + WR - 1) / WR;                     // rank tiles per wave
  // K per stage: the largest power of two (at least 32 per K part) whose
  // stage of X and A rows stays within MLR_MFMA_STAGE_BYTES; small stages
  // leave a pass bound by the fixed cost of each ring step
  static constexpr int kt(int k) {
    return (k < 512 && (RB + RP) * 2 * k * 2 <= MLR_MFMA_STAGE_BYTES) ? kt(2 * k) : k;
  }
  static constexpr int KT = kt(32 * WK > 64 ? 32 * WK : 64);
  static constexpr int CPR = KT / 8;                                // chunks per staged row
  static constexpr int KSW = KT / WK / 32;                          // k-steps per wave, stage
  static constexpr int XI = RB * CPR / kWave;                       // DMA instrs for X
  static constexpr int AI = RP * CPR / kWave;                       // DMA instrs for A
  static constexpr int IPW = (XI + AI + kWavesM - 1) / kWavesM;     // per wavefront
  static constexpr int BYTES = kWavesM * IPW * kWave * 16;          // slot size
  static_assert(KSW >= 1 && (RB * CPR) % kWave == 0 && (RP * CPR) % kWave == 0, "layout");
};

template <int RT>
struct Slots {
  static constexpr int KS = (RT + 1) / 2;   // expand k-steps of 32 ranks
  static constexpr int RK = 32 * KS;
  static constexpr int VP = RK + 8;         // bf16 pitch of V rows in LDS
  static constexpr int a = Shrink<1, RT>::BYTES, b = Shrink<2, RT>::BYTES, c = Shrink<4, RT>::BYTES;
  static constexpr int ab = a > b ? a : b;
  static constexpr int BYTES = ab > c ? ab : c;
  static_assert(kPassRows * VP * 2 <= BYTES, "V must fit in one slot");
  static_assert(kThreadsM * 4 * ((RT + 3) / 4) * 4 <= BYTES, "partials must fit in one slot");
};

struct PassCtx {
  i32x4_t xr, ar;               // DMA sources: x, A[s,l,e]
  __amdgpu_buffer_rsrc_t br;    // B[s,l,e]
  __amdgpu_buffer_rsrc_t yr;    // y
  uint8_t* ring;                // three slots of Slots<RT>::BYTES
  uint32_t ring_lds;            // LDS byte address of ring
  const int* s_row;    // X row per pass row, -1 = none
  const int* s_pair;   // pair per pass row, numel = none
  const float* s_wt;   // routed weight per pass row (1 when not applied)
  int s, n0, n1;
};

// Per-lane DMA source of this wavefront's instructions (fixed over K).
template <int IPW>
struct DmaSrc {
  int base[IPW];  // element offset of the chunk's row, -1 = zero fill
  int c8[IPW];    // k offset of the chunk inside a stage
};

template <int MT, int RT>
__device__ __forceinline__ void dma_plan(const FusedParams& p, const PassCtx& c, DmaSrc<Shrink<MT, RT>::IPW>& d) {
  using S = Shrink<MT, RT>;
  const int w = wave_id(), lane = lane_id();
#pragma unroll
  for (int i = 0; i < S::IPW; ++i) {
    const int ins = w + kWavesM * i;
    const int chunk = ins * kWave + lane;
    const int q = chunk / S::CPR, j = chunk % S::CPR;
    d.c8[i] = 8 * (j ^ (q & 7));
    int base = -1;
    if (ins < S::XI) {
      const int xr = c.s_row[q];
      if (xr >= 0) base = xr * p.K;
    } else if (ins < S::XI + S::AI) {
      const int jr = q - S::RB;
      if (jr < p.r) base = jr * p.K;
    }
    d.base[i] = base;
  }
}

template <int MT, int RT>
__device__ __forceinline__ void dma_issue(const FusedParams& p, const PassCtx& c, const DmaSrc<Shrink<MT, RT>::IPW>& d,
                                          int stage, uint32_t slot_lds) {
  using S = Shrink<MT, RT>;
  const int w = wave_id();
  const int k0 = stage * S::KT;
#pragma unroll
  for (int i = 0; i < S::IPW; ++i) {
    const int ins = w + kWavesM * i;
    const int k = k0 + d.c8[i];
    const uint32_t off = (d.base[i] >= 0 && k < p.K) ? uint32_t(d.base[i] + k) * 2u : kOob;
    dma16(ins < S::XI ? c.xr : c.ar, slot_lds + ins * (kWave * 16), off);
  }
}

// MFMAs of one staged K slice for this wavefront's tiles.
template <int MT, int RT>
__device__ __forceinline__ void shrink_compute(const uint8_t* slot, f32x4_t (&acc)[Shrink<MT, RT>::TR]) {
  using S = Shrink<MT, RT>;
  // all four wavefronts have a tile unless WR does not divide the rank tiles
  constexpr bool kAllBusy = MT * S::WR * S::WK == kWavesM;
  constexpr bool kAllRanks = RT % S::WR == 0;
  const int w = wave_id(), lane = lane_id();
  if (!kAllBusy && w >= MT * S::WR * S::WK) return;
  const int mt = w % MT, wr = (w / MT) % S::WR, kp = w / (MT * S::WR);
  const int lr = lane & 15, lq = lane >> 4;
  const uint4* st = reinterpret_cast<const uint4*>(slot);
#pragma unroll
  for (int ks = 0; ks < S::KSW; ++ks) {
    const int ch = 4 * (kp * S::KSW + ks) + lq;
    const int qx = 16 * mt + lr;
    const uint4 xa = st[qx * S::CPR + (ch ^ (qx & 7))];
#pragma unroll
    for (int tr = 0; tr < S::TR; ++tr) {
      const int rt = wr + tr * S::WR;
      if (kAllRanks || rt < RT) {
        const int qa = S::RB + 16 * rt + lr;
        const uint4 ab = st[qa * S::CPR + (ch ^ (qa & 7))];
        acc[tr] = mfma16(xa, ab, acc[tr]);
      }
    }
  }
}

// One ring step: stage t is complete once at most one later stage of this
// wavefront is still loading; then stage t + 2 goes into the slot of t - 1,
// which every wavefront has finished with (it passed the barrier).
template <int MT, int RT>
__device__ __forceinline__ void shrink_step(const FusedParams& p, const PassCtx& c, const DmaSrc<Shrink<MT, RT>::IPW>& d,
                                            int t, int nst, f32x4_t (&acc)[Shrink<MT, RT>::TR]) {
  using S = Shrink<MT, RT>;
  constexpr int SB = Slots<RT>::BYTES;
  if (t + 1 < nst) stage_barrier<S::IPW>();
  else stage_barrier<0>();
  const int cur = t % 3, nxt = (t + 2) % 3;
  if (t + 2 < nst) dma_issue<MT, RT>(p, c, d, t + 2, c.ring_lds + nxt * SB);
  shrink_compute<MT, RT>(c.ring + cur * SB, acc);
}

// Expand geometry of a pass with MT row tiles and KS k-steps: column groups
// of NCG columns; wavefront w multiplies column tiles w + kWavesM i (i < CTW)
// of a group for all MT row tiles.  The scaled delta of a group crosses LDS
// once (fp32, DP floats per row, two buffers) so that Y is read and written
// in 16-byte chunks of 8 columns laid along the rows: thread t takes chunks
// t + kThreadsM i (i < YC) of the group, CPRW to a row, and a wavefront
// instruction covers 64 / CPRW whole rows of NCG columns.  Y pieces of 8 bytes
// per lane, 16 rows to an instruction (the MFMA result layout), ran at about
// 60% of the rate of this layout on MI355X.
template <int MT, int KS>
struct Expand {
  static constexpr int CTW0 = MLR_MFMA_CTW_BUDGET / (MT * KS);
  static constexpr int CTW = CTW0 < 1 ? 1 : (CTW0 > 4 ? 4 : CTW0);  // column tiles per wavefront
  static constexpr int NCG = 16 * kWavesM * CTW;                     // columns per group
  static constexpr int RB = 16 * MT;                                 // rows
  static constexpr int CPRW = NCG / 8;                               // 16-byte chunks per row
  static constexpr int YC = RB * CPRW / kThreadsM;                   // chunks per thread
  static constexpr int DP = NCG + 4;                                 // fp32 pitch of a delta row
  static constexpr int DBYTES = RB * DP * 4;                         // one delta buffer
  static_assert(YC >= 1 && YC * kThreadsM == RB * CPRW, "whole chunks per thread");
};
// the two delta buffers of the largest group (64 rows x 128 or 32 x 256 columns)
constexpr int kDeltaBytes = 2 * 64 * (128 + 4) * 4;

// 16-byte chunk j of a delta row is stored at chunk j ^ bit 3 of j: the two
// chunks a thread reads for its 8 columns then fall in different bank groups
// from those of its neighbours.
__device__ __forceinline__ int dswz(int j) { return j ^ ((j >> 3) & 1); }

// B chunks (MFMA layout) and Y chunks (row layout) of one column group.
template <int MT, int KS>
struct ExpandRegs {
  uint4 b[Expand<MT, KS>::CTW][KS];
  uint4 y[Expand<MT, KS>::YC];
};

// Row-layout chunks of this thread: Y element offset of the chunk's row
// (slice column 0), -1 for a row without a pair (y stays below 2 GiB, so
// offsets fit 32 bits); column of the chunk in a group.
template <int MT, int KS>
struct YChunks {
  int row[Expand<MT, KS>::YC];
  int col[Expand<MT, KS>::YC];
};

// Byte offset of a Y chunk in the buffer resource; past its range (reads
// zero, stores dropped) for a row without a pair or a column past the split.
template <int MT, int KS>
__device__ __forceinline__ uint32_t ychunk_off(const PassCtx& c, const YChunks<MT, KS>& yc, int i, int nb) {
  const int n = nb + yc.col[i];
  return (yc.row[i] >= 0 && n < c.n1) ? uint32_t(yc.row[i] + n) * 2u : kOob;
}

// Loads of column group nb: every load is issued (out-of-range B and Y
// chunks read as zero through the buffer resources), so no load sits behind a
// per-lane branch.
template <int MT, int KS>
__device__ __forceinline__ void expand_load(const FusedParams& p, const PassCtx& c, int nb,
                                            const YChunks<MT, KS>& yc, ExpandRegs<MT, KS>& r) {
  using X = Expand<MT, KS>;
  const int w = wave_id(), lane = lane_id();
  const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int i = 0; i < X::CTW; ++i) {
    const int n = nb + 16 * (w + kWavesM * i) + lr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int j = 32 * ks + 8 * lq;
      const uint32_t off = (n < c.n1 && j < p.r) ? uint32_t(n * p.r + j) * 2u : kOob;
      r.b[i][ks] = buf_ld16(c.br, off, 0);
    }
  }
  // Y is read once and written once: both accesses are non-temporal (loads
  // and stores together measured 2-11 % faster on the prefill and dense
  // shapes; either one alone, within 2 %)
  if (p.add) {
#pragma unroll
    for (int i = 0; i < X::YC; ++i) r.y[i] = buf_ld16<kNonTemporal>(c.yr, ychunk_off(c, yc, i, nb), 0);
  }
}

// MFMAs of column group nb; the delta, scaled by the routed weight, goes to
// LDS buffer dl.  The MFMA result D^T[16 columns x 16 rows] leaves each lane
// four consecutive columns of one row: one 16-byte LDS write.
template <int MT, int KS>
__device__ __forceinline__ void expand_mfma(const float (&wt)[MT], const uint4 (&va)[MT][KS],
                                            const uint4 (&vl)[MT][KS], const ExpandRegs<MT, KS>& r,
                                            float* dl) {
  using X = Expand<MT, KS>;
  const int w = wave_id(), lane = lane_id();
  const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int i = 0; i < X::CTW; ++i) {
    const int j = 4 * (w + kWavesM * i) + lq;  // 16-byte chunk of the delta row
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      f32x4_t dt = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        dt = mfma16(r.b[i][ks], va[m][ks], dt);
        dt = mfma16(r.b[i][ks], vl[m][ks], dt);
      }
      const float4 o = make_float4(dt[0] * wt[m], dt[1] * wt[m], dt[2] * wt[m], dt[3] * wt[m]);
      *reinterpret_cast<float4*>(dl + (16 * m + lr) * X::DP + 4 * dswz(j)) = o;
    }
  }
}

// Epilogue of column group nb in the row layout: Y (+)= delta, one rounding.
template <int MT, int KS>
__device__ __forceinline__ void expand_store(const FusedParams& p, const PassCtx& c, int nb,
                                             const YChunks<MT, KS>& yc, const ExpandRegs<MT, KS>& r,
                                             const float* dl) {
  using X = Expand<MT, KS>;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < X::YC; ++i) {
    const int q = t + kThreadsM * i, row = q / X::CPRW, cj = q % X::CPRW;
    const float4 d0 = *reinterpret_cast<const float4*>(dl + row * X::DP + 4 * dswz(2 * cj));
    const float4 d1 = *reinterpret_cast<const float4*>(dl + row * X::DP + 4 * dswz(2 * cj + 1));
    float o[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
    if (p.add) {
      const uint32_t yw[4] = {r.y[i].x, r.y[i].y, r.y[i].z, r.y[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] += bf16_lo(yw[e]);
        o[2 * e + 1] += bf16_hi(yw[e]);
      }
    }
    uint32_t ow[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      ow[e] = pack_bf16x2(o[2 * e], o[2 * e + 1]);
    buf_st16<kNonTemporal>(make_uint4(ow[0], ow[1], ow[2], ow[3]), c.yr, ychunk_off(c, yc, i, nb), 0);
  }
}

template <int MT, int RT>
__device__ __forceinline__ void run_pass(const FusedParams& p, const PassCtx& c) {
  using S = Shrink<MT, RT>;
  using SS = Slots<RT>;
  constexpr int KS = SS::KS, VP = SS::VP;
  const int tid = threadIdx.x, w = wave_id(), lane = lane_id();
  const int lr = lane & 15, lq = lane >> 4;

  // ---------------- shrink
  DmaSrc<S::IPW> d;
  dma_plan<MT, RT>(p, c, d);
  const int nst = (p.K + S::KT - 1) / S::KT;
  dma_issue<MT, RT>(p, c, d, 0, c.ring_lds);
  if (nst > 1) dma_issue<MT, RT>(p, c, d, 1, c.ring_lds + SS::BYTES);
  f32x4_t acc[S::TR];
#pragma unroll
  for (int i = 0; i < S::TR; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < nst; ++t) shrink_step<MT, RT>(p, c, d, t, nst, acc);
  stage_barrier<0>();  // every wavefront is done with the ring

  // K parts -> one sum (slot 1 holds the partials of parts 1..WK-1)
  const bool owner = w < MT * S::WR;
  if constexpr (S::WK > 1) {
    float* part = reinterpret_cast<float*>(c.ring + SS::BYTES);
    if (!owner && w < MT * S::WR * S::WK) {
#pragma unroll
      for (int i = 0; i < S::TR; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) part[((w * S::TR + i) * 4 + e) * kWave + lane] = acc[i][e];
    }
    stage_barrier<0>();
    if (owner) {
#pragma unroll
      for (int kp = 1; kp < S::WK; ++kp) {
        const int src = w + kp * MT * S::WR;
#pragma unroll
        for (int i = 0; i < S::TR; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][e] += part[((src * S::TR + i) * 4 + e) * kWave + lane];
      }
    }
  }
  // V -> bf16 rows: the high parts in slot 0, the low parts in slot 2 (slot 1
  // may still be read for partials), both zero from RP up to RK
  uint16_t* s_v = reinterpret_cast<uint16_t*>(c.ring);
  uint16_t* s_vl = reinterpret_cast<uint16_t*>(c.ring + 2 * SS::BYTES);
  if (owner) {
    const int mt = w % MT, wr = (w / MT) % S::WR;
#pragma unroll
    for (int i = 0; i < S::TR; ++i) {
      const int rt = wr + i * S::WR;
      if (rt < RT) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int at = (16 * mt + 4 * lq + e) * VP + 16 * rt + lr;
          const uint16_t hi = f32_to_bf16(acc[i][e]);
          s_v[at] = hi;
          s_vl[at] = f32_to_bf16(acc[i][e] - bf16_to_f32(hi));
        }
      }
    }
  }
  if constexpr (SS::RK > S::RP) {
    for (int i = tid; i < S::RB * (SS::RK - S::RP); i += kThreadsM) {
      const int at = (i / (SS::RK - S::RP)) * VP + S::RP + i % (SS::RK - S::RP);
      s_v[at] = 0;
      s_vl[at] = 0;
    }
  }
  stage_barrier<0>();

  // ---------------- expand
  using X = Expand<MT, KS>;
  static_assert(2 * X::DBYTES <= kDeltaBytes, "delta buffers");
  ExpandRegs<MT, KS> cur, nxt;
  uint4 va[MT][KS], vl[MT][KS];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int at = (16 * m + lr) * VP + 32 * ks + 8 * lq;
      va[m][ks] = *reinterpret_cast<const uint4*>(s_v + at);
      vl[m][ks] = *reinterpret_cast<const uint4*>(s_vl + at);
    }
  // routed weight of this lane's row in each row tile (MFMA layout)
  float wt[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) wt[m] = c.s_wt[16 * m + lr];
  // row layout: the Y row of each of this thread's chunks
  YChunks<MT, KS> yc;
#pragma unroll
  for (int i = 0; i < X::YC; ++i) {
    const int q = tid + kThreadsM * i, row = q / X::CPRW;
    const int pid = c.s_pair[row];
    yc.row[i] = pid < p.numel ? pid * p.N + c.s * p.Ns : -1;
    yc.col[i] = 8 * (q % X::CPRW);
  }
  expand_load<MT, KS>(p, c, c.n0, yc, cur);
  // the delta buffers take the ring's place: every wavefront holds V in registers
  stage_barrier<63>();
  float* dl0 = reinterpret_cast<float*>(c.ring);
  float* dl1 = reinterpret_cast<float*>(c.ring + X::DBYTES);
  for (int nb = c.n0; nb < c.n1; nb += 2 * X::NCG) {
    if (nb + X::NCG < c.n1) expand_load<MT, KS>(p, c, nb + X::NCG, yc, nxt);
    expand_mfma<MT, KS>(wt, va, vl, cur, dl0);
    stage_barrier<63>();  // the group's delta is in LDS; loads stay in flight
    expand_store<MT, KS>(p, c, nb, yc, cur, dl0);
    if (nb + X::NCG >= c.n1) break;
    if (nb + 2 * X::NCG < c.n1) expand_load<MT, KS>(p, c, nb + 2 * X::NCG, yc, cur);
    expand_mfma<MT, KS>(wt, va, vl, nxt, dl1);
    stage_barrier<63>();
    expand_store<MT, KS>(p, c, nb + X::NCG, yc, nxt, dl1);
  }
  stage_barrier<0>();  // V (slot 0) and the row tables are reused by the next pass
}

// How the work of a (block, slice) unit is spread when the units leave
// compute units idle: n_split column ranges and n_rs row parts (16-row
// multiples) per unit, each a workgroup of its own.  A column split re-reads
// the unit's X rows and A; a row part re-reads A and B.  Among the splittings
// that keep every workgroup in one round (xcd_cus * MLR_MFMA_OCCUPANCY slots
// per XCD), the one that moves the fewest bytes per workgroup wins -- for
// the dense projections (few blocks of full rows, small rank, large K) that
// is row parts, where column splits would stream the same X rows many times.
// With every slot taken there is one workgroup per unit.
__device__ __forceinline__ void pick_splits(const FusedParams& p, int total, int per_xcd, int& n_rs,
                                            int& n_split) {
  const int cap = p.xcd_cus * MLR_MFMA_OCCUPANCY;
  const int max_split = max(1, p.Ns / MLR_MFMA_MIN_COLS);
  const int room = max(1, cap / max(per_xcd, 1));
  n_rs = 1;
  n_split = min(max_split, room);
  if (room < 2) return;
  // rows a block holds on average (valid rows form each block's prefix)
  const float rows = float(min(p.B, (p.numel + total - 1) / max(total, 1)));
  const float K = float(p.K), r = float(p.r), Ns = float(p.Ns);
  auto cost = [&](int rs, int cs) {
    const float pr = rows / rs, pc = Ns / cs;
    return pr * K * 2.f + r * K * 2.f + pc * r * 2.f + pr * pc * 2.f * (p.add ? 2.f : 1.f);
  };
  float best = cost(1, n_split);
  for (int rs = 2; rs <= 8 && 16 * rs <= p.B && rows >= 16.f * rs && rs <= room; rs *= 2) {
    const int cs = min(max_split, room / rs);
    const float c = cost(rs, cs);
    if (c < best) {
      best = c;
      n_rs = rs;
      n_split = cs;
    }
  }
}

// NAIVE: the blocks are formed on chip from topk_ids and the mapping (the
// align-free path) instead of being read from the align outputs.
template <int RT, bool NAIVE>
__global__ void __launch_bounds__(kThreadsM) __attribute__((amdgpu_waves_per_eu(2))) fused_mfma_kernel(FusedParams p) {
  __shared__ __align__(16) uint8_t ring[3 * Slots<RT>::BYTES > kDeltaBytes ? 3 * Slots<RT>::BYTES : kDeltaBytes];
  __shared__ int s_row[kPassRows];
  __shared__ int s_pair[kPassRows];
  __shared__ float s_wt[kPassRows];
  __shared__ int s_ids[NAIVE ? kMaxIdsM : 1];  // pair ids of the block (align-free path)
  static_assert(sizeof(GroupLds) <= sizeof(ring), "the grouping tables borrow the ring");

  // units = (block, slice); the split count gives every working workgroup a
  // slot (MLR_MFMA_OCCUPANCY per compute unit), at least MLR_MFMA_MIN_COLS
  // columns each
  GroupLds& gl = *reinterpret_cast<GroupLds*>(ring);  // free until the first stage is loaded
  PairGroup<kThreadsM> pg;
  BlockScan sc;
  int total;
  if constexpr (NAIVE) {
    total = group_pairs(p, gl, pg);
  } else {
    sc = scan_blocks(p);
    total = sc.total;
  }
  const int units = total * p.S;
  const int per_xcd = (units + kXcds - 1) / kXcds;
  int n_rs, n_split;
  pick_splits(p, total, per_xcd, n_rs, n_split);
  if constexpr (NAIVE) {  // fused_moe_lora_with_align: the align outputs
    if (side_align(p, first_idle_xcd(units * n_rs, n_split))) return;
  }
  int sub, split;
  if (!map_unit_xcd(blockIdx.x, units * n_rs, n_split, sub, split)) return;
  const int unit = sub / n_rs, rpart = sub - unit * n_rs;
  const int prows = p.B / n_rs;  // rows of the block this workgroup takes
  const int nsz = ((p.Ns + n_split - 1) / n_split + 15) / 16 * 16;
  const int n0 = split * nsz;
  if (n0 >= p.Ns) return;
  const int n1 = min(p.Ns, n0 + nsz);
  const int g = unit / p.S, s = unit - g * p.S;
  int l, e, b = 0;
  if constexpr (NAIVE) {
    group_block(p, gl, pg, g, s_ids, l, e);
  } else {
    find_block(p, sc, g, l, b);
    e = __builtin_amdgcn_readfirstlane(p.eids[l * p.nb + b]);
  }
  const int64_t wsel = (int64_t(s) * p.L + l) * p.E + e;

  PassCtx c;
  const int64_t x_rows = p.x_per_pair ? int64_t(p.numel) : int64_t(p.numel / p.topk);
  c.xr = dma_rsrc(p.x, uint32_t(x_rows * p.K * 2));
  c.ar = dma_rsrc(p.a + wsel * p.r * p.K, uint32_t(p.r * p.K * 2));
  c.br = make_rsrc(p.b + wsel * p.Ns * p.r, uint32_t(p.Ns * p.r * 2));
  c.yr = make_rsrc(p.y, uint32_t(int64_t(p.numel) * p.N * 2));
  c.ring = ring;
  c.ring_lds = lds_address(ring);
  c.s_row = s_row;
  c.s_pair = s_pair;
  c.s_wt = s_wt;
  c.s = s;
  c.n0 = n0;
  c.n1 = n1;

  const int tid = threadIdx.x;
  const int rend = (rpart + 1) * prows;
  for (int r0 = rpart * prows; r0 < rend; r0 += kPassRows) {
    if (tid < kPassRows) {
      int pid = p.numel, xr = -1;
      float wv = 1.f;
      if (r0 + tid < rend) {
        pid = NAIVE ? s_ids[r0 + tid] : p.sorted[l * p.cap + b * p.B + r0 + tid];
        if (pid < p.numel) {
          xr = p.x_per_pair ? pid : pid / p.topk;
          if (p.mul) wv = p.w[pid];
        } else {
          pid = p.numel;
        }
      }
      s_pair[tid] = pid;
      s_row[tid] = xr;
      s_wt[tid] = wv;
    }
    // valid rows are a prefix of the block (sentinels only pad a group's end)
    const int nv = __builtin_amdgcn_readfirstlane(__syncthreads_count(tid < kPassRows && s_row[tid] >= 0));
    if (nv == 0) break;
    if (nv <= 16) run_pass<1, RT>(p, c);
    else if (nv <= 32) run_pass<2, RT>(p, c);
    else run_pass<4, RT>(p, c);
  }
}

}  // namespace

// B rows are read as 16-byte chunks of 8 ranks, so r must be a multiple of 8.
bool mfma_supported(int r, int B) {
  return r >= 8 && r <= 16 * 8 && r % 8 == 0 && B >= 16 && B <= 128;
}

// Every buffer the kernel reads through a buffer resource stays below 2 GiB,
// so that one offset past the end (kOob) is out of range for all of them (y
// is held to the same limit).
bool mfma_fits(int64_t x_bytes, int64_t y_bytes, int64_t r, int64_t K, int64_t Ns) {
  return x_bytes <= kMaxXBytes && y_bytes <= kMaxXBytes && r * K * 2 <= kMaxXBytes &&
         r * Ns * 2 <= kMaxXBytes;
}

hipError_t launch_fused_mfma(FusedParams p, hipStream_t st) {
  const int rt = (p.r + 15) / 16;
  // grid: 8 XCD ranges of ceil(units / 8) units times the split count, which
  // the kernel keeps within xcd_cus * MLR_MFMA_OCCUPANCY slots per XCD
  const int64_t per_xcd = (int64_t(p.units) + kXcds - 1) / kXcds;
  const int64_t slots = std::max<int64_t>(per_xcd, int64_t(p.xcd_cus) * MLR_MFMA_OCCUPANCY);
  const dim3 grid(unsigned(kXcds * slots));
#define MLR_MFMA_CASE(RT_)                                                                       \
  case RT_:                                                                                      \
    if (p.naive) hipLaunchKernelGGL((fused_mfma_kernel<RT_, true>), grid, dim3(kThreadsM), 0, st, p); \
    else hipLaunchKernelGGL((fused_mfma_kernel<RT_, false>), grid, dim3(kThreadsM), 0, st, p);       \
    break;
  switch (rt) {
    MLR_MFMA_CASE(1)
    MLR_MFMA_CASE(2)
    MLR_MFMA_CASE(3)
    MLR_MFMA_CASE(4)
    MLR_MFMA_CASE(5)
    MLR_MFMA_CASE(6)
    MLR_MFMA_CASE(7)
    MLR_MFMA_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef MLR_MFMA_CASE
  return hipGetLastError();
}

}  // namespace mlr
