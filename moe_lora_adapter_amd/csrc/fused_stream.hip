// Fused shrink + expand for decode-sized blocks as one continuous stream.
//
// One 1024-thread workgroup handles one (block, slice, column split) and up
// to ROWS rows at a time (4; 8 as a build option where K <= 3072, not with
// the K split).  Its whole weight traffic -- the A matrix (r x K),
// then the split's B columns (cols x r) -- flows through one ring of LDS
// slots filled by direct-to-LDS buffer loads, 16 KiB per stage, NS - 1 stages
// in flight.  The B stages start loading while the last A stages are being
// multiplied, so the weight stream does not stop between shrink and expand
// (loading A in register batches and then B leaves HBM idle between the two
// bursts).  The arithmetic is on v_mfma_f32_16x16x32_bf16: with one MFMA per
// wavefront and stage the vector ALUs stay out of the way of the stream (the
// same loop with v_dot2 products was bound by their issue).
//
//   before the ring  X rows (rows x K) and the Y values of the split
//                    (rows x cols) are loaded into LDS the same way, only
//                    the pass's valid rows.
//   A stage          K range [t KT, (t+1) KT) of all r rows: 16 (rank tile,
//                    k-step) products, one per wavefront, V^T[16 ranks x 16
//                    rows] += A[16 x 32] X^T[32 x 16] (rows >= ROWS zero;
//                    valid rows < row < ROWS stale and never stored).
//   after A          the k-step partials of each rank tile are added through
//                    LDS and v goes to LDS as two bf16 parts, v = hi + lo
//                    (hi = bf16(v), lo = bf16(v - hi)); never to memory.
//   B stage          NCS consecutive columns of B: D^T[16 cols x 16 cols'] =
//                    B[16 x 32 ranks] W^T, where the 16 MFMA columns of W
//                    carry V_hi of the pass rows in columns 0..ROWS-1 and
//                    V_lo of the same rows in columns ROWS..2 ROWS-1.  Adding
//                    column i + ROWS of the result onto column i (one lane
//                    shuffle) gives B (V_hi + V_lo)^T: v enters with about 16
//                    significant bits instead of bf16's 8, at no extra MFMA.
//                    A lane then ends with four
//                    consecutive columns of one row, which it scales by the
//                    routed weight, adds to the Y values held in LDS and
//                    rounds to bf16 there.
//   epilogue         the Y rows of the split go back to memory in 16-byte
//                    pieces.
// Staged rows keep their 16-byte chunks XOR-permuted by the row (A) or
// column (B) index so the 16 rows of an MFMA operand read spread over the
// LDS banks.
//
// The prhub summary of vLLM PR #42290 (implementation steps) describes the
// one-shot kernel this follows: x loaded once, multiplied by lora_a, the
// rank-sized result kept on chip and multiplied by lora_b, written over or
// added onto the output.
#include <algorithm>

#include "blocks.h"
#include "common.h"
#include "dma.h"
#include "align_wave.h"
#include "groups.h"
#include "internal.h"
#include "xch.h"

namespace mlr {
namespace {

constexpr int kST = 1024;                   // threads
constexpr int kRows = 4;                    // X rows per pass
constexpr int kStage = 16384;               // bytes per ring stage
constexpr int kStageChunks = kStage / 16;   // 1024
constexpr int kIPS = kStageChunks / kST;    // DMA instructions per thread and stage
static_assert(kIPS == 1, "a stage is one 16-byte chunk per thread");
constexpr int kXBytes = 32768;              // X rows of a four-row pass: kRows * K * 2
// Eight rows per pass (MLR_STREAM_ROWS8) where K allows (the K split keeps
// four: its exchange slot holds four rows): a block of five to eight rows
// then streams its weights once instead of twice.  X rows of such a pass:
// 8 * K * 2 bytes.
constexpr int kRows8 = 8;
constexpr int kXBytes8 = 49152;
constexpr int kMaxCols = 2048;              // output columns per workgroup
constexpr int kMaxIds = 128;                // largest block_m
constexpr int kMaxPeers = kXchPeers;       // most workgroups one K split spans
constexpr int64_t kMaxBufBytes = int64_t(1) << 31;

// Ring depth: slots - 1 stages in flight per workgroup.  Four slots (48 KiB
// in flight) measured fastest on MI355X with B non-temporal; deeper rings add
// contention among the 228 streaming workgroups (20b-like decode a6, kernel
// us with 3 / 4 / 5 / 6 slots: 22.5 / 22.2 / 23.1 / 23.8 one launch, 22.0 /
// 21.5 / 22.3 / 23.0 sorted; w2 a6 18.1 / 17.6 / 19.0 / 19.8).
#ifndef MLR_STREAM_SLOTS
#define MLR_STREAM_SLOTS 4
#endif
constexpr int kSlots = MLR_STREAM_SLOTS;
static_assert(kSlots >= 3 && kSlots <= 8, "ring slots");

// With the K split, B stages are issued up to this many slots minus one
// ahead from the exchange on: the exchange's round trip (3 to 4 us under the
// streaming load) then passes while B keeps streaming into the ring.  The
// slot count is what LDS leaves room for beside the exchange's buffers.
template <int R>
constexpr int kSlotsXch() { return R <= 64 ? 5 : 4; }

// Eight rows per pass (build option, off by default): it removes the second
// pass of blocks with five to eight rows, but gained nothing clear on the
// default decode step and made a captured dual-stream decode layer slower
// (421 against 409 us; 880 against 520 with the LoRA side enqueued first).
#ifndef MLR_STREAM_ROWS8
#define MLR_STREAM_ROWS8 0
#endif
#ifndef MLR_STREAM_MIN_COLS
#define MLR_STREAM_MIN_COLS 256
#endif

// Wait for the ring stage whose loads were followed by `later` stages.
template <int L>
__device__ __forceinline__ void wait_stage(int later) {
  if constexpr (L < 0) {
    stage_barrier<0>();
  } else {
    if (later == L) stage_barrier<L * kIPS>();
    else wait_stage<L - 1>(later);
  }
}

// Wait until at most n (1 <= n <= N) vector memory operations of this
// wavefront are outstanding, then meet the workgroup.
template <int N>
__device__ __forceinline__ void wait_counts(int n) {
  if constexpr (N <= 0) {
    stage_barrier<0>();
  } else {
    if (n == N) stage_barrier<N>();
    else wait_counts<N - 1>(n);
  }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Lane i of every 16-lane row gets the value of lane i + ROWS of the same
// row (DPP row shift left; lanes past the row's end get 0): a VALU lane move,
// with no trip through the LDS crossbar.
template <int ROWS>
__device__ __forceinline__ float lane_plus_rows(float v) {
  static_assert(ROWS >= 1 && ROWS <= 15, "DPP row shift distance");
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x100 + ROWS, 0xf, 0xf, true));
}

// Stage geometry for rank R (32, 64 or 128).
template <int R>
struct Geo {
  static constexpr int KT = kStage / 2 / R;     // K per A stage
  static constexpr int CPRK = KT / 8;           // chunks per A row in a stage (>= 8)
  static constexpr int RT = R / 16;             // rank tiles
  static constexpr int KSA = KT / 32 / 1;       // k-steps per A stage
  static constexpr int NCS = kStage / 2 / R;    // columns per B stage
  static constexpr int CPR = R / 8;             // chunks per B column
  static constexpr int SW = CPR < 8 ? CPR : 8;  // B chunk permutation width
  static constexpr int CT = NCS / 16;           // column tiles per B stage
  static constexpr int KS = (R + 31) / 32;      // expand k-steps (ranks padded to 32)
  static_assert(RT * KSA == kST / kWave, "one (rank tile, k-step) per wavefront");
  static_assert(CPRK >= 8, "A chunk permutation needs 8 chunks per row");
};

// Loads of ring stage t into slot `lds`: the workgroup's nA stages of A
// (K stages ka0, ka0 + 1, ...), then its B stages.  B is read by this
// workgroup only and goes in as non-temporal (evict-first) loads; A stays
// with the default policy, since the unit's other column splits read it from
// L2.  Measured on the 20b-like decode w13, a2..a6: 0.3 to 1.3 us faster
// with B non-temporal, 0.3 us slower at a1; with A non-temporal as well,
// slower.
template <int R>
__device__ __forceinline__ void issue_stage(const FusedParams& p, i32x4_t ar, i32x4_t br, int t,
                                            int nA, int ka0, int ncols, uint32_t lds) {
  using G = Geo<R>;
  const int q = threadIdx.x;  // one 16-byte chunk per thread and stage
  const uint32_t dst = lds + wave_id() * kWave * 16;
  if (t < nA) {
    const int j = q / G::CPRK, cs = q % G::CPRK;
    const int kk = (ka0 + t) * G::KT + 8 * (cs ^ (j & 7));
    dma16(ar, dst, kk < p.K ? uint32_t(j * p.K + kk) * 2u : kOob);
  } else {
    const int col = q / G::CPR, js = q % G::CPR;
    const int n = (t - nA) * G::NCS + col;
    const int jc = js ^ (col & (G::SW - 1));
    dma16<true>(br, dst, n < ncols ? uint32_t(n * R + 8 * jc) * 2u : kOob);
  }
}

// Adds the k-step partials of each rank tile through LDS: afterwards the
// wavefronts w < RT hold, lane (lr, lq), v[row lr][16 w + 4 lq + i] in acc[i]
// (summed over the A stages this workgroup multiplied).
template <int R>
__device__ __forceinline__ void reduce_ksteps(f32x4_t& acc, float* s_part) {
  using G = Geo<R>;
  const int w = wave_id(), lane = lane_id();
  stage_barrier<63>();  // earlier readers of s_part are done
#pragma unroll
  for (int i = 0; i < 4; ++i) s_part[(w * 4 + i) * kWave + lane] = acc[i];
  stage_barrier<63>();
  if (w < G::RT) {
#pragma unroll
    for (int k = 1; k < G::KSA; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += s_part[((w + k * G::RT) * 4 + i) * kWave + lane];
  }
}

// The MFMAs of A stages [k0, k1) with A read from memory instead of the ring:
// the same operands in the same order as the ring path, so the partial is
// the same bit for bit.  Used for a peer whose partial did not arrive.
template <int R>
__device__ __forceinline__ f32x4_t a_partial_direct(const FusedParams& p, __amdgpu_buffer_rsrc_t a_rsrc,
                                                    const uint8_t* xs, int k0, int k1) {
  using G = Geo<R>;
  const int w = wave_id(), lane = lane_id(), lr = lane & 15, lq = lane >> 4;
  const int j = 16 * (w % G::RT) + lr, c = 4 * (w / G::RT) + lq;
  const int K8 = p.K / 8;
  const uint4 zero4 = make_uint4(0, 0, 0, 0);
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int t = k0; t < k1; ++t) {
    const int kk = t * G::KT + 8 * c;
    const uint4 a = buf_ld16(a_rsrc, kk < p.K ? uint32_t(j * p.K + kk) * 2u : kOob, 0);
    const int xc = t * (G::KT / 8) + c;
    const uint4 x = (lr < kRows && xc < K8) ? reinterpret_cast<const uint4*>(xs)[lr * K8 + xc] : zero4;
    acc = mfma16(a, x, acc);
  }
  return acc;
}

// The K split of one pass (exchange protocol and area: xch.h).  The peers
// -- the C workgroups of a unit, one per column split -- each multiply an
// equal share of the A stages, publish their partial, and form
// v = P_0 + P_1 + ... + P_{C-1} in peer order, so all peers hold the same v.
// A partial not complete after `peer_wait` polls is computed here from A in
// memory (the same bits), so no wait depends on another workgroup being
// resident.

// The wavefronts w < RT hold, lane (lr, lq), v[row lr][16 w + 4 lq + i].
template <int R>
__device__ __forceinline__ void publish_partial(const XchSlot& x, const f32x4_t& acc, int split,
                                                uint32_t tag) {
  using G = Geo<R>;
  const int w = wave_id(), lane = lane_id(), lr = lane & 15, lq = lane >> 4;
  if (w < G::RT && lr < kRows) {
#pragma unroll
    for (int i = 0; i < 4; ++i) xch_put(x, split, lr, 16 * w + 4 * lq + i, acc[i], tag);
  }
}

// All peers' words polled at once by the holders, the values parked in LDS
// (s_peer[peer][row][rank]); s_miss collects the peers whose partial did not
// arrive, which are then computed here.  v is then summed in peer order.
template <int R>
__device__ __forceinline__ void gather_partials(const FusedParams& p, const XchSlot& x, f32x4_t& acc,
                                                float* s_part, float* s_peer, int* s_miss,
                                                const uint8_t* xs, __amdgpu_buffer_rsrc_t a_rsrc,
                                                int split, int C, int nA_all, uint32_t tag) {
  using G = Geo<R>;
  const int w = wave_id(), lane = lane_id(), lr = lane & 15, lq = lane >> 4;
  const bool holder = w < G::RT && lr < kRows;
  float* mine = s_peer + lr * R + 16 * w + 4 * lq;  // + q * kRows * R
  if (w < G::RT) {
    uint32_t pending = 0;
#pragma unroll
    for (int q = 0; q < kMaxPeers; ++q)
      if (holder && q < C && q != split) pending |= 1u << q;
    for (int n = 0; n < p.peer_wait && __ballot(pending != 0) != 0; ++n) {
#pragma unroll
      for (int q = 0; q < kMaxPeers; ++q) {
        if ((pending >> q) & 1u) {
          uint64_t wd[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) wd[i] = xch_get(x, q, lr, 16 * w + 4 * lq + i);
          bool ok = true;
#pragma unroll
          for (int i = 0; i < 4; ++i) ok = ok && xch_tagged(wd[i], tag);
          if (ok) {
#pragma unroll
            for (int i = 0; i < 4; ++i) mine[q * kRows * R + i] = xch_value(wd[i]);
            pending &= ~(1u << q);
          }
        }
      }
      if (__ballot(pending != 0) != 0) __builtin_amdgcn_s_sleep(8);
    }
    if (pending) atomicOr(s_miss, int(pending));
    if (holder) {
#pragma unroll
      for (int i = 0; i < 4; ++i) mine[split * kRows * R + i] = acc[i];
    }
  }
  stage_barrier<63>();
  const int miss = __builtin_amdgcn_readfirstlane(*s_miss);
  if (miss) {
    stage_barrier<0>();  // X, and everything else in flight, has landed
    for (int q = 0; q < C; ++q) {  // rare: a peer's partial computed here instead
      if (!((miss >> q) & 1)) continue;
      f32x4_t pq = a_partial_direct<R>(p, a_rsrc, xs, q * nA_all / C, (q + 1) * nA_all / C);
      reduce_ksteps<R>(pq, s_part);
      if (holder) {
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[q * kRows * R + i] = pq[i];
      }
    }
  }
  if (holder) {
    f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < C; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] += mine[q * kRows * R + i];
    acc = v;
  }
}

// NAIVE: the blocks are formed on chip from topk_ids and the mapping (the
// align-free path) instead of being read from the align outputs.  XCH: the
// K split (an exchange area is given); its own instantiation, so the state
// it keeps does not crowd the registers of the kernel without it (the
// shared build spilled scalar registers into vector lanes on every stage:
// +2 us on the 20b-like decode).
template <int R, bool NAIVE, bool XCH, int ROWS>
__global__ void __launch_bounds__(kST) fused_stream_kernel(FusedParams p) {
  using G = Geo<R>;
  static_assert(ROWS == kRows || (ROWS == kRows8 && !XCH), "rows per pass");
  constexpr int XB = ROWS == kRows ? kXBytes : kXBytes8;  // X rows of a pass
  constexpr int YB = ROWS * kMaxCols * 2;                 // the split's Y values of a pass
  constexpr int VP = 32 * G::KS + 8;  // bf16 pitch of the v rows
  // ring slots: kSlots, or with the K split a deeper ring that holds the B
  // stages loaded while the peers' partials are awaited
  constexpr int NS = XCH ? kSlotsXch<R>() : kSlots;
  // slots the stream runs ahead through (with the K split, until the exchange)
  constexpr int SA = NS < kSlots ? NS : kSlots;
  __shared__ __align__(16) uint8_t ring[NS * kStage];
  __shared__ __align__(16) uint8_t xs[XB];
  __shared__ __align__(16) uint8_t ys[YB];
  __shared__ __align__(16) uint16_t s_vb[ROWS * VP];  // v, bf16 high part
  __shared__ __align__(16) uint16_t s_vl[ROWS * VP];  // v, bf16 low part
  __shared__ int s_pair[ROWS];
  __shared__ int s_row[ROWS];
  __shared__ float s_w[ROWS];
  __shared__ int s_ids[NAIVE ? kMaxIds : 1];  // pair ids of the block (align-free path)
  __shared__ uint2 s_dummy[kWave];            // stores of lanes with no output
  __shared__ __align__(16) float s_part[XCH ? kST * 4 : 4];  // k-step partials (K split)
  static_assert(kST * 4 * 4 <= XB, "k-step partials fit the X buffer");
  __shared__ int s_miss;                      // K split: peers whose partial did not arrive
  __shared__ float s_peer[XCH ? kMaxPeers * ROWS * R : 1];  // K split: the peers' partials
  __shared__ uint32_t s_tag;                  // K split: this call's tag in the pass's slot
  __shared__ __align__(16) uint32_t s_left[XCH ? kXchPeers : 1];  // K split: the slot's left words
  __shared__ int s_grp1[4];                   // one-wavefront grouping: blocks, slot, expert,
                                              // valid rows of the first pass
  static_assert(2 * ROWS <= 16, "V_hi and V_lo share the 16 columns of one MFMA operand");
  static_assert(sizeof(GroupLds) <= sizeof(ring), "the grouping tables borrow the ring");

  // units = (block, slice); split count: a compute unit per working
  // workgroup, at least MLR_STREAM_MIN_COLS and at most kMaxCols columns each
  GroupLds& gl = *reinterpret_cast<GroupLds*>(ring);  // free until the first stage is loaded
  PairGroup<kST> pg;
  BlockScan sc;
  int total;
  // Up to 64 pairs the grouping is one wavefront's work (a pair per lane):
  // wavefront 0 does it alone while the others wait, rather than all 16
  // repeating it four to a SIMD.  The same holds for the block lookup of up
  // to 64 slots; wavefront 0 then also sets the first pass's rows.
  const bool one_wave = NAIVE && p.numel <= kWave;
  const bool rows_first = NAIVE ? one_wave : p.L <= kWave;
  if constexpr (NAIVE) {
    if (one_wave) {
      if (wave_id() == 0) {
        const int t = group_pairs(p, gl, pg);  // no barrier on this path
        if (lane_id() == 0) s_grp1[0] = t;
      }
      __syncthreads();
      total = __builtin_amdgcn_readfirstlane(s_grp1[0]);
    } else {
      total = group_pairs(p, gl, pg);
    }
  } else {
    sc = scan_blocks(p);
    total = sc.total;
  }
  const int units = total * p.S;
  const int per_xcd = (units + kXcds - 1) / kXcds;
  const int need = (p.Ns + kMaxCols - 1) / kMaxCols;
  const int max_split = max(need, p.Ns / MLR_STREAM_MIN_COLS);
  const int n_split = min(max_split, max(need, p.xcd_cus / max(per_xcd, 1)));
  if constexpr (NAIVE) {  // fused_moe_lora_with_align: the align outputs
    if (side_align(p, first_idle_xcd(units, n_split))) return;
  }
  int unit, split;
  if (!map_unit_xcd(blockIdx.x, units, n_split, unit, split)) return;
  const int nsz = ((p.Ns + n_split - 1) / n_split + 7) / 8 * 8;
  const int n0 = split * nsz;
  if (n0 >= p.Ns) return;
  const int n1 = min(p.Ns, n0 + nsz);
  const int ncols = n1 - n0;
  const int g = unit / p.S, s = unit - g * p.S;
  int l, e;
  const int32_t* srow = nullptr;
  int id0 = p.numel;
  // The block's pair ids of the first pass -> the pass's rows, written to LDS
  // (lanes < ROWS of the calling wavefront); returns the valid rows.
  auto first_rows = [&](int id) {
    const int lane = lane_id();
    int pid = p.numel, xrow = -1;
    float wv = 1.f;
    if (lane < ROWS && lane < p.B && id < p.numel) {
      pid = id;
      xrow = p.x_per_pair ? id : id / p.topk;
      if (p.mul) wv = p.w[id];
    }
    if (lane < ROWS) {
      s_pair[lane] = pid;
      s_row[lane] = xrow;
      s_w[lane] = wv;
    }
    return __popcll(__ballot(lane < ROWS && xrow >= 0));
  };
  if constexpr (NAIVE) {
    if (rows_first) {
      if (wave_id() == 0) {
        group_block_wave(p, pg, g, s_ids, l, e);
        // the first pass's rows too, so that one barrier publishes both
        const int lane = lane_id();
        const int nr0 = first_rows(lane < ROWS && lane < p.B ? s_ids[lane] : p.numel);
        if (lane == 0) {
          s_grp1[1] = l;
          s_grp1[2] = e;
          s_grp1[3] = nr0;
        }
      }
      __syncthreads();
      l = __builtin_amdgcn_readfirstlane(s_grp1[1]);
      e = __builtin_amdgcn_readfirstlane(s_grp1[2]);
    } else {
      group_block(p, gl, pg, g, s_ids, l, e);
    }
  } else if (rows_first) {
    // wavefront 0 looks the block up, reads its expert and first pair ids and
    // sets the first pass's rows; one barrier publishes them
    if (wave_id() == 0) {
      int b;
      find_block(p, sc, g, l, b);
      srow = p.sorted + l * p.cap + b * p.B;
      const int lane = lane_id();
      const int id = (lane < ROWS && lane < p.B) ? srow[lane] : p.numel;
      e = __builtin_amdgcn_readfirstlane(p.eids[l * p.nb + b]);
      const int nr0 = first_rows(id);
      if (lane == 0) {
        s_grp1[1] = l;
        s_grp1[2] = e;
        s_grp1[3] = nr0;
      }
    }
    __syncthreads();
    l = __builtin_amdgcn_readfirstlane(s_grp1[1]);
    e = __builtin_amdgcn_readfirstlane(s_grp1[2]);
  } else {
    int b;
    find_block(p, sc, g, l, b);
    // the first pass's pair ids are loaded before the expert id is waited for
    srow = p.sorted + l * p.cap + b * p.B;
    id0 = (threadIdx.x < ROWS && int(threadIdx.x) < p.B) ? srow[threadIdx.x] : p.numel;
    e = __builtin_amdgcn_readfirstlane(p.eids[l * p.nb + b]);
  }
  const int64_t wsel = (int64_t(s) * p.L + l) * p.E + e;
  const i32x4_t ar = dma_rsrc(p.a + wsel * R * p.K, uint32_t(R * p.K * 2));
  const i32x4_t br = dma_rsrc(p.b + wsel * p.Ns * R + int64_t(n0) * R, uint32_t(ncols * R * 2));
  const int64_t x_rows = p.x_per_pair ? int64_t(p.numel) : int64_t(p.numel / p.topk);
  const i32x4_t xr = dma_rsrc(p.x, uint32_t(x_rows * p.K * 2));
  const int64_t col0 = int64_t(s) * p.Ns + n0;
  const i32x4_t yr = dma_rsrc(p.y + col0, uint32_t((int64_t(p.numel) * p.N - col0) * 2));
  const uint32_t ring_lds = lds_address(ring);
  const uint32_t xs_lds = lds_address(xs);
  const uint32_t ys_lds = lds_address(ys);

  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int lr = lane & 15, lq = lane >> 4;
  const int K8 = p.K / 8, c8 = ncols / 8;
  // K split: with an exchange area, the C workgroups of the unit (one per
  // column split with columns) each multiply stages [ka0, ka0 + nA) of the
  // nA_all A stages and meet before the expand
  const int C = (p.Ns + nsz - 1) / nsz;
  // (a unit past the slots the area holds -- only when more slots are active
  // than the call's max_active_loras promised -- multiplies all of A itself)
  const bool xch = XCH && C > 1 && C <= kMaxPeers && (unit + 1) * p.xch_passes <= p.xch_nslot;
  const int nA_all = (p.K + G::KT - 1) / G::KT;
  const int ka0 = xch ? split * nA_all / C : 0;
  const int nA = xch ? (split + 1) * nA_all / C - ka0 : nA_all;
  const int nB = (ncols + G::NCS - 1) / G::NCS, T = nA + nB;
  const int TA = xch ? nA : T;  // stages issued ahead until the exchange
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(p.a + wsel * R * p.K, uint32_t(R * p.K * 2));
  const uint4 zero4 = make_uint4(0, 0, 0, 0);

  // The first pass's first A stage loads while the pass is set up: it needs
  // only the expert and the ring (whose grouping tables are done with).  The
  // pass then issues X, Y and the later stages, so the first wait still finds
  // exactly one stage issued after the one it waits for.
  if (TA > 0) issue_stage<R>(p, ar, br, 0, nA, ka0, ncols, ring_lds);

  for (int g0 = 0; g0 < p.B; g0 += ROWS) {
    // K split: the pass's slot
    const XchSlot xs_slot = xch ? xch_slot(p.xch, p.xch_nslot, unit * p.xch_passes + g0 / ROWS) : XchSlot{};
    // K split: the slot's `left` words go to LDS by a direct load issued now
    // (two lanes of wavefront 0, after the pass's first stage): no register
    // holds them and nothing waits for them before the exchange, which reads
    // them; the first stage's wait covers them
    if (xch && w == 0 && lane < 2) {
      const i32x4_t lr4 = dma_rsrc(xs_slot.left, 4 * kXchPeers);
      dma16(lr4, lds_address(s_left), uint32_t(16 * lane));
    }
    const bool rows_set = rows_first && g0 == 0;  // set with the block, before its barrier
    if (!rows_set && tid < ROWS) {
      int pid = p.numel, xrow = -1;
      float wv = 1.f;
      if (g0 + tid < p.B) {
        const int id = NAIVE ? s_ids[g0 + tid] : (g0 == 0 ? id0 : srow[g0 + tid]);
        if (id < p.numel) {
          pid = id;
          xrow = p.x_per_pair ? id : id / p.topk;
          if (p.mul) wv = p.w[id];
        }
      }
      s_pair[tid] = pid;
      s_row[tid] = xrow;
      s_w[tid] = wv;
    }
    for (int i = tid; i < ROWS * VP; i += kST) s_vb[i] = s_vl[i] = 0;
    // valid rows are a prefix of the block (sentinels only pad a group's end)
    const int nr = rows_set ? __builtin_amdgcn_readfirstlane(s_grp1[3])
                            : __builtin_amdgcn_readfirstlane(
                                  __syncthreads_count(tid < ROWS && s_row[tid] >= 0));
    if (nr == 0) {  // (a block's first pass always has a row: only later passes end here)
      stage_barrier<0>();
      break;
    }

    // X rows (row stride K / 8 chunks) and the split's Y values (row stride
    // ncols / 8 chunks) into LDS: 64 chunks per instruction, only
    // instructions that start inside the data (both buffers are multiples
    // of 64 chunks, so a last partial instruction still fits).  (Loading Y
    // after the first stage instead, since the expand is the first to need
    // it, measured 4 us slower on the 20b-like decode.)
    // Only the pass's nr valid rows are staged.  The rows past them keep what
    // the buffers held: each row of the products depends on its own X row
    // and v row only, and rows past nr are never stored.
    for (int q0 = w * kWave; q0 < nr * K8; q0 += kST) {
      const int q = q0 + lane, i = q / K8, c = q % K8;
      const int xrow = i < ROWS ? s_row[i] : -1;
      const uint32_t off = (q < nr * K8 && xrow >= 0) ? uint32_t(xrow * p.K + 8 * c) * 2u : kOob;
      dma16(xr, xs_lds + q0 * 16, off);
    }
    for (int q0 = w * kWave; q0 < nr * c8; q0 += kST) {
      const int q = q0 + lane, i = q / c8, c = q % c8;
      const int pid = i < ROWS ? s_pair[i] : p.numel;
      const uint32_t off = (q < nr * c8 && p.add && pid < p.numel)
                               ? uint32_t(int64_t(pid) * p.N + 8 * c) * 2u : kOob;
      dma16(yr, ys_lds + q0 * 16, off);
    }
    for (int t = g0 == 0 ? 1 : 0; t < SA - 1 && t < TA; ++t)
      issue_stage<R>(p, ar, br, t, nA, ka0, ncols, ring_lds + t * kStage);

    // wavefront w: A rank tile rt and k-step ka of every A stage
    const int rt = w % G::RT, ka = w / G::RT;
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint4 vop[G::KS];
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) vop[ks] = zero4;
    const float wrow = lr < ROWS ? s_w[lr] : 0.f;

    // stage t's wait and the next stage's issue (the ring's step)
    auto ring_step = [&](int t) {
      // stage t (and, at t = 0, the X rows issued before it): the later
      // stages stay in flight, so the ring never drains to empty
      // (with the K split the A stages drain before the exchange)
      const int lim = t < nA ? TA : T;
      if constexpr (!XCH) {
        wait_stage<SA - 2>(min(SA - 2, lim - 1 - t));
        if (t + SA - 1 < lim)
          issue_stage<R>(p, ar, br, t + SA - 1, nA, ka0, ncols,
                         ring_lds + ((t + SA - 1) % NS) * kStage);
      } else {
        // stages issued ahead of t: SA - 1, or NS - 1 from the exchange on
        const int ahead = (xch && t >= nA) ? NS - 1 : SA - 1;
        wait_stage<NS - 2>(min(ahead - 1, lim - 1 - t));
        if (xch && t == nA && tid == 0) {
          // every read of the slot by this workgroup has returned (its values
          // are in s_vb / s_vl): leave it
          xch_leave(xs_slot, split, s_tag);
        }
        if (t + ahead < lim)
          issue_stage<R>(p, ar, br, t + ahead, nA, ka0, ncols, ring_lds + ((t + ahead) % NS) * kStage);
      }
    };
    // ---- shrink, the A stages: V^T[rank tile rt] += A[16 ranks x 32 k] . X^T
    for (int t = 0; t < nA; ++t) {
      ring_step(t);
      const uint4* st = reinterpret_cast<const uint4*>(ring + (t % NS) * kStage);
      const int j = 16 * rt + lr, c = 4 * ka + lq;
      const uint4 a = st[j * G::CPRK + (c ^ (j & 7))];
      const int xc = (ka0 + t) * (G::KT / 8) + c;
      // one 16-byte read at a clamped index, then the select (a read
      // guarded by the condition became four masked 4-byte reads)
      const uint4 xv = reinterpret_cast<const uint4*>(xs)[min(lr, ROWS - 1) * K8 + min(xc, K8 - 1)];
      const uint4 x = (lr < ROWS && xc < K8) ? xv : zero4;
      acc = mfma16(a, x, acc);
    }
    {
      // the A stages are multiplied: v for rows < ROWS into s_vb / s_vl
      // (the k-step partials go through the X buffer, which only the K
      // split's fallback still reads)
      if (xch && tid == 0) {
        uint32_t m = 0;
#pragma unroll
        for (int q = 0; q < kXchPeers; ++q) m = s_left[q] > m ? s_left[q] : m;
        s_tag = m + 1u;
        s_miss = 0;
      }
      reduce_ksteps<R>(acc, XCH ? s_part : reinterpret_cast<float*>(xs));
      if (xch) {
        const uint32_t tag = __builtin_amdgcn_readfirstlane(s_tag);
        // the wavefronts holding v publish; then every wavefront issues
        // the next NS - 1 B stages, which stream while the holders wait
        // for the peers' partials (their polls retire after those loads)
        publish_partial<R>(xs_slot, acc, split, tag);
        for (int u = nA; u < nA + NS - 1 && u < T; ++u)
          issue_stage<R>(p, ar, br, u, nA, ka0, ncols, ring_lds + (u % NS) * kStage);
        gather_partials<R>(p, xs_slot, acc, s_part, s_peer, &s_miss, xs, a_rsrc, split, C, nA_all, tag);
      }
      // lane (lr, lq) of wavefront w < RT holds v[row lr][16 w + 4 lq + i]
      if (w < G::RT && lr < ROWS) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint16_t hi = f32_to_bf16(acc[i]);
          s_vb[lr * VP + 16 * w + 4 * lq + i] = hi;
          s_vl[lr * VP + 16 * w + 4 * lq + i] = f32_to_bf16(acc[i] - bf16_to_f32(hi));
        }
      }
    }
    // ---- expand, the B stages: D^T[16 cols x 16 rows] = B[16 cols x 32 ranks] . V^T
    // (a loop of its own, so that the expand's operands do not share
    // registers with the shrink's and move between them at every stage)
    for (int t = nA; t < T; ++t) {
      ring_step(t);
      const uint4* st = reinterpret_cast<const uint4*>(ring + (t % NS) * kStage);
      const int u = t - nA;
      if (u == 0) {
        // operand column lr: V_hi of row lr (lr < ROWS), V_lo of row
        // lr - ROWS (ROWS <= lr < 2 ROWS), else zero
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
          const int row = lr < ROWS ? lr : (lr < 2 * ROWS ? lr - ROWS : 0);
          const uint16_t* src = lr < ROWS ? s_vb : s_vl;
          const uint4 vv = *reinterpret_cast<const uint4*>(src + row * VP + 32 * ks + 8 * lq);
          vop[ks] = lr < 2 * ROWS ? vv : zero4;
        }
      }
      for (int ct = w; ct < G::CT; ct += kST / kWave) {
        const int col = 16 * ct + lr;
        // lane (lr, lq): row lr, columns 16 ct + 4 lq .. + 3 of this stage.
        // Its Y values are read before the products so the read's latency
        // hides behind them (lanes with nothing to write read row 0,
        // column 0 and drop it).
        const int n = u * G::NCS + 16 * ct + 4 * lq;
        const bool live = lr < nr && n < ncols;
        uint2* yp = reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(ys) +
                                             (live ? lr * ncols + n : 0));
        const uint2 yv = *yp;
        f32x4_t dt = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < G::KS; ++ks) {
          const int jc = 4 * ks + lq;
          const uint4 bb = jc < G::CPR ? st[col * G::CPR + (jc ^ (col & (G::SW - 1)))] : zero4;
          dt = mfma16(bb, vop[ks], dt);
        }
        // lane (lr, lq) adds the V_lo product of its row, held ROWS lanes up
#pragma unroll
        for (int i = 0; i < 4; ++i) dt[i] += lane_plus_rows<ROWS>(dt[i]);
        // every lane forms and stores its result -- lanes with nothing to
        // write into a dummy LDS slot -- so no branch exists that the Y read
        // and the arithmetic could be sunk into (below the products)
        const float ya = p.add ? 1.f : 0.f;
        const float o[4] = {dt[0] * wrow + ya * bf16_lo(yv.x), dt[1] * wrow + ya * bf16_hi(yv.x),
                            dt[2] * wrow + ya * bf16_lo(yv.y), dt[3] * wrow + ya * bf16_hi(yv.y)};
        const uint2 out = make_uint2(pack_bf16x2(o[0], o[1]),
                                     pack_bf16x2(o[2], o[3]));
        *(live ? yp : &s_dummy[lane]) = out;
      }
    }
    __syncthreads();
    // ---- epilogue: Y rows of the split, 16 bytes per thread and step
    for (int q = tid; q < nr * c8; q += kST) {
      const int i = q / c8, c = q % c8;
      const uint4 v = reinterpret_cast<const uint4*>(ys)[i * c8 + c];
      *reinterpret_cast<uint4*>(p.y + int64_t(s_pair[i]) * p.N + col0 + 8 * c) = v;
    }
    __syncthreads();  // s_* tables, xs, ys and the ring are reused by the next pass
  }
}

}  // namespace

// The stream kernel takes r in {32, 64, 128}, X rows of a pass that fit
// kXBytes, and buffers below 2 GiB (kOob must lie past each of them).
bool stream_supported(int64_t M, int64_t numel, int64_t K, int64_t N, int r, int x_per_pair) {
  if (r != 32 && r != 64 && r != 128) return false;
  if (int64_t(kRows) * K * 2 > kXBytes) return false;
  const int64_t x_bytes = (x_per_pair ? numel : M) * K * 2;
  return x_bytes <= kMaxBufBytes && numel * N * 2 <= kMaxBufBytes && r * K * 2 <= kMaxBufBytes;
}

static_assert(kRows == kXchRows, "a pass of the stream kernel is one exchange slot");

hipError_t launch_fused_stream(FusedParams p, hipStream_t st) {
  // grid: 8 XCD ranges of ceil(units / 8) units times the split count, which
  // the kernel keeps within xcd_cus per XCD unless the column limit needs more
  const int64_t per_xcd = (int64_t(p.units) + kXcds - 1) / kXcds;
  const int64_t need = (p.Ns + kMaxCols - 1) / kMaxCols;
  const int64_t slots = std::max<int64_t>(per_xcd * need, p.xcd_cus);
  const dim3 grid(unsigned(kXcds * slots));
  // eight rows per pass where the X rows fit (not with the K split)
#if MLR_STREAM_ROWS8
  // eight rows per pass where the X rows fit (not with the K split)
  const bool rows8 = !p.xch && int64_t(kRows8) * p.K * 2 <= kXBytes8;
#define MLR_STREAM_CASE(R_)                                                                  \
  case R_:                                                                                   \
    if (p.xch) hipLaunchKernelGGL((fused_stream_kernel<R_, false, true, kRows>), grid, dim3(kST), 0, st, p); \
    else if (p.naive && rows8) hipLaunchKernelGGL((fused_stream_kernel<R_, true, false, kRows8>), grid, dim3(kST), 0, st, p); \
    else if (p.naive) hipLaunchKernelGGL((fused_stream_kernel<R_, true, false, kRows>), grid, dim3(kST), 0, st, p); \
    else if (rows8) hipLaunchKernelGGL((fused_stream_kernel<R_, false, false, kRows8>), grid, dim3(kST), 0, st, p); \
    else hipLaunchKernelGGL((fused_stream_kernel<R_, false, false, kRows>), grid, dim3(kST), 0, st, p); \
    break;
#else
#define MLR_STREAM_CASE(R_)                                                                  \
  case R_:                                                                                   \
    if (p.xch) hipLaunchKernelGGL((fused_stream_kernel<R_, false, true, kRows>), grid, dim3(kST), 0, st, p); \
    else if (p.naive) hipLaunchKernelGGL((fused_stream_kernel<R_, true, false, kRows>), grid, dim3(kST), 0, st, p); \
    else hipLaunchKernelGGL((fused_stream_kernel<R_, false, false, kRows>), grid, dim3(kST), 0, st, p); \
    break;
#endif
  switch (p.r) {
    MLR_STREAM_CASE(32)
    MLR_STREAM_CASE(64)
    MLR_STREAM_CASE(128)
    default: return hipErrorInvalidValue;
  }
#undef MLR_STREAM_CASE
  return hipGetLastError();
}

}  // namespace mlr
