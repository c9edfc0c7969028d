// The register-batch kernel, its helpers and its launcher, for one
// workgroup size: included by fused_valu.hip once per size, each time inside
// a namespace of its own with MLR_VALU_T (threads per workgroup) defined, and
// MLR_VALU_R16_ONLY defined where only rank 16 is launched.  No include guard
// on purpose.
constexpr int kThreads = MLR_VALU_T;
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
      v[q] = keep + butterfly_partner(send, o);
    }
    if (up) which += half;
  }
  float t = v[0];
#pragma unroll
  for (; o >= 1; o >>= 1) t += butterfly_partner(t, o);
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

constexpr int kRowsPerBatch = 2 * kThreads;  // columns of one expand batch (at most)
// one epilogue task (one row, 8 columns) per thread covers a batch
static_assert(kMaxRG * kRowsPerBatch / 8 <= kThreads, "epilogue tasks exceed the threads");

// The loads of one expand batch: this thread's B chunks and the Y piece of
// its epilogue task.  They do not depend on v, so the first batch can be in
// flight with A.
template <int NB>
struct ExpandBatch {
  uint4 bv[NB];
  uint4 yv;
};

template <int RG, int CPR>
struct ExpandGeom {
  static constexpr int NB0 = RG <= 2 ? 16 : 8;            // chunk loads in flight per thread
  static constexpr int NBR = kRowsPerBatch * CPR / kThreads;
  static constexpr int NB = NB0 < NBR ? NB0 : (NBR > 0 ? NBR : 1);
};

// Epilogue task of this thread in the batch starting at chunk `base`: row
// task_i, 8 columns from 8 task_c; none when the batch has fewer than 8
// columns or the row is past nr.
struct ExpandTask {
  int row0, rows, task_i, task_c;
  bool has;
};

template <int CPR>
__device__ __forceinline__ ExpandTask expand_task(int base, int nchunks, int NBT, int nr) {
  ExpandTask t;
  t.rows = min(NBT, nchunks - base) / CPR;  // columns in this batch
  t.row0 = base / CPR;
  const int c8n = t.rows / 8;
  t.task_i = int(threadIdx.x) / max(c8n, 1);
  t.task_c = int(threadIdx.x) - t.task_i * max(c8n, 1);
  t.has = c8n > 0 && t.task_i < nr;
  return t;
}

template <int RG, int CPR>
__device__ __forceinline__ void expand_issue(const FusedParams& p, const uint16_t* __restrict__ tile,
                                             const int* s_pair, int nr, int col0, int base,
                                             int nchunks, ExpandBatch<ExpandGeom<RG, CPR>::NB>& eb) {
  constexpr int NB = ExpandGeom<RG, CPR>::NB;
  const int tid = threadIdx.x;
  const ExpandTask t = expand_task<CPR>(base, nchunks, NB * kThreads, nr);
  eb.yv = make_uint4(0, 0, 0, 0);
  if (t.has && p.add)
    eb.yv = *reinterpret_cast<const uint4*>(p.y + int64_t(s_pair[t.task_i]) * p.N + col0 + t.row0 +
                                            t.task_c * 8);
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int q = min(base + k * kThreads + tid, nchunks - 1);
    eb.bv[k] = ld16(tile + int64_t(q) * 8);
  }
}

// Expand for r == 8 * CPR: the B tile rows [n0, n1) read as one coalesced
// stream of 16-byte chunks.  Chunk q of the tile is row q / CPR, ranks
// 8 * (q % CPR) .. +8; since the thread count is a multiple of CPR a thread
// always sees the same eight ranks.  The row sums land in LDS (s_d), and the
// epilogue then reads Y and writes it back in 16-byte pieces (8 columns per
// thread), the Y reads issued before the B chunks are consumed.  With FIRST,
// `first` holds the loads of the first batch, issued by the caller
// (expand_issue).

// One batch of the expand from its loads: row sums into s_d, then the
// epilogue (Y (+)= w d, one rounding) of this thread's task.
template <int RG, int CPR>
__device__ __forceinline__ void expand_batch(const FusedParams& p, const int* s_pair, int nr,
                                             const float (&vr)[RG][8], const float (&wt)[RG],
                                             int col0, int base, int nchunks, float* s_d,
                                             const ExpandBatch<ExpandGeom<RG, CPR>::NB>& eb) {
  constexpr int NB = ExpandGeom<RG, CPR>::NB;
  const int tid = threadIdx.x;
  const int jc = tid % CPR;
  const ExpandTask t = expand_task<CPR>(base, nchunks, NB * kThreads, nr);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int q = base + k * kThreads + tid;
    const uint4 b4 = eb.bv[k];
    const float b[8] = {bf16_lo(b4.x), bf16_hi(b4.x), bf16_lo(b4.y), bf16_hi(b4.y),
                        bf16_lo(b4.z), bf16_hi(b4.z), bf16_lo(b4.w), bf16_hi(b4.w)};
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      float d = 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) d += vr[i][u] * b[u];
#pragma unroll
      for (int o = CPR / 2; o >= 1; o >>= 1) d += butterfly_partner(d, o);
      if (jc == 0 && q < nchunks) s_d[i * kRowsPerBatch + q / CPR - t.row0] = d;
    }
  }
  __syncthreads();
  if (t.has) {
    uint16_t* yp = p.y + int64_t(s_pair[t.task_i]) * p.N + col0 + t.row0 + t.task_c * 8;
    const float* dd = s_d + t.task_i * kRowsPerBatch + t.task_c * 8;
    const float w = wt[t.task_i];
    const uint32_t in[4] = {eb.yv.x, eb.yv.y, eb.yv.z, eb.yv.w};
    uint32_t outw[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float lo = dd[2 * h] * w, hi = dd[2 * h + 1] * w;
      if (p.add) {
        lo += bf16_lo(in[h]);
        hi += bf16_hi(in[h]);
      }
      outw[h] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<uint4*>(yp) = make_uint4(outw[0], outw[1], outw[2], outw[3]);
  }
  __syncthreads();
}

template <int RG, int CPR, bool FIRST>
__device__ __forceinline__ void expand_stream(const FusedParams& p, const uint16_t* __restrict__ Bm,
                                              const int* s_pair, int nr, const float* s_v, int s,
                                              int n0, int n1, float* s_d,
                                              const ExpandBatch<ExpandGeom<RG, CPR>::NB>& first) {
  constexpr int NB = ExpandGeom<RG, CPR>::NB;
  const int jc = int(threadIdx.x) % CPR;
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
  int base = 0;
  if constexpr (FIRST) {
    expand_batch<RG, CPR>(p, s_pair, nr, vr, wt, col0, 0, nchunks, s_d, first);
    base = NB * kThreads;
  }
#pragma unroll 1
  for (; base < nchunks; base += NB * kThreads) {
    ExpandBatch<NB> eb;
    expand_issue<RG, CPR>(p, tile, s_pair, nr, col0, base, nchunks, eb);
    expand_batch<RG, CPR>(p, s_pair, nr, vr, wt, col0, base, nchunks, s_d, eb);
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

// Rows [0, nv) of one block in groups of RG (a group with fewer valid rows
// repeats row 0 and drops its sums).
template <int RG, int JW, int CPR>
__device__ __forceinline__ void valu_rows(const FusedParams& p, const uint16_t* A, const uint16_t* Bm,
                                          const int* s_row, const int* s_pair, int nv,
                                          ShrinkShape sh, float* s_part, float* s_v, float* s_d,
                                          int s, int n0, int n1) {
  for (int g0 = 0; g0 < nv; g0 += RG) {
    const int nr = min(RG, nv - g0);
    if constexpr (CPR > 0) {
      // with 512 threads the expand's first B and Y loads go out with A's
      // (with 1024 the registers they would hold through the shrink spill)
      constexpr bool kEarly = kThreads <= 512;
      ExpandBatch<ExpandGeom<RG, CPR>::NB> first;
      if constexpr (kEarly)
        expand_issue<RG, CPR>(p, Bm + int64_t(n0) * p.r, s_pair + g0, nr, s * p.Ns + n0, 0,
                              (n1 - n0) * CPR, first);
      shrink_group<RG, JW>(p, A, s_row + g0, nr, sh, s_part, s_v);
      expand_stream<RG, CPR, kEarly>(p, Bm, s_pair + g0, nr, s_v, s, n0, n1, s_d, first);
    } else {
      shrink_group<RG, JW>(p, A, s_row + g0, nr, sh, s_part, s_v);
      expand_columns<RG>(p, Bm, s_pair + g0, nr, s_v, s, n0, n1);
    }
    __syncthreads();
  }
}

// Blocks of up to two valid rows take 2-row groups; larger blocks take
// 4-row groups (one pass over A and B per group).
// NAIVE: the blocks are formed on chip from topk_ids and the mapping (the
// align-free path) instead of being read from the align outputs.
template <int JW, int CPR, bool NAIVE>
__global__ void __launch_bounds__(kThreads, MLR_VALU_OCC * kThreads / 256) fused_valu_kernel(FusedParams p, ShrinkShape sh) {
  constexpr int RG = 4;  // LDS sized for the larger group
  __shared__ int s_pair[kMaxB];
  __shared__ int s_row[kMaxB];
  __shared__ float s_v[kMaxRG * kMaxR];
  __shared__ float s_part[kMaxRG * 256];
  __shared__ float s_d[CPR > 0 ? RG * kRowsPerBatch : 1];
  __shared__ __align__(16) uint8_t s_grp[NAIVE ? sizeof(GroupLds) : 1];
  __shared__ int s_one[4];  // one-wavefront lookup: blocks, slot, expert, valid rows
  GroupLds& gl = *reinterpret_cast<GroupLds*>(s_grp);

  // The blocks present decide the split count: as many column splits (of at
  // least MLR_VALU_MIN_COLS columns) as give every working workgroup a compute
  // unit of its own.  Unit u goes to XCD u % 8, so an XCD holds
  // ceil(units / 8) * n_split of them; a second workgroup on a compute unit
  // was measured to cost far more than a split saves.
  PairGroup<kThreads> pg;
  BlockScan sc;
  int total;
  // Up to 64 pairs (align-free) or 64 slots (sorted) the grouping and the
  // block lookup are one wavefront's work: wavefront 0 does them, and sets
  // the block's rows, while the others wait, rather than all 16 repeating
  // them four to a SIMD.
  const bool one_wave = NAIVE ? p.numel <= kWave : p.L <= kWave;
  if constexpr (NAIVE) {
    if (one_wave) {
      if (wave_id() == 0) {
        const int t = group_pairs(p, gl, pg);  // no barrier on this path
        if (lane_id() == 0) s_one[0] = t;
      }
      __syncthreads();
      total = __builtin_amdgcn_readfirstlane(s_one[0]);
    } else {
      total = group_pairs(p, gl, pg);
    }
  } else {
    sc = scan_blocks(p);
    total = sc.total;
  }
  const int units = total * p.S;
  const int per_xcd = (units + kXcds - 1) / kXcds;
  const int u8 = per_xcd * kXcds;
  const int max_split = max(1, p.Ns / MLR_VALU_MIN_COLS);
  const int n_split = min(max_split, max(1, p.xcd_cus * MLR_VALU_OCC / max(per_xcd, 1)));
  if constexpr (NAIVE) {  // fused_moe_lora_with_align: the align outputs (the first
    // index with no unit: unit `units` of split 0, else split n_split's first)
    if (side_align(p, units < u8 ? units : n_split * u8)) return;
  }
  // workgroup -> (split, unit), split-major; equal unit residue mod 8 = same XCD
  const int id = blockIdx.x;
  const int split = id / max(u8, 1), unit = id - split * u8;
  if (unit >= units || split >= n_split) return;
  const int nsz = ((p.Ns + n_split - 1) / n_split + 7) / 8 * 8;
  const int n0 = split * nsz;
  if (n0 >= p.Ns) return;
  const int n1 = min(p.Ns, n0 + nsz);
  const int g = unit / p.S, s = unit - g * p.S;
  int l, e, nv;
  if (one_wave) {
    if (wave_id() == 0) {
      int b = 0;
      if constexpr (NAIVE) {
        group_block_wave(p, pg, g, s_pair, l, e);  // pair ids straight into s_pair
      } else {
        find_block(p, sc, g, l, b);
        e = __builtin_amdgcn_readfirstlane(p.eids[l * p.nb + b]);
      }
      // the block's rows (lane 0 takes part in every step, so it counts all)
      int cnt = 0;
      for (int i = lane_id(); i < p.B; i += kWave) {
        const int pid = NAIVE ? s_pair[i] : p.sorted[l * p.cap + b * p.B + i];
        const bool valid = pid < p.numel;
        s_pair[i] = pid;
        s_row[i] = valid ? (p.x_per_pair ? pid : pid / p.topk) : 0;
        cnt += __popcll(__ballot(valid));
      }
      if (lane_id() == 0) {
        s_one[1] = l;
        s_one[2] = e;
        s_one[3] = cnt;
      }
    }
    __syncthreads();
    l = __builtin_amdgcn_readfirstlane(s_one[1]);
    e = __builtin_amdgcn_readfirstlane(s_one[2]);
    nv = __builtin_amdgcn_readfirstlane(s_one[3]);
  } else {
    int b = 0;
    if constexpr (NAIVE) {
      group_block(p, gl, pg, g, s_pair, l, e);  // pair ids straight into s_pair
    } else {
      find_block(p, sc, g, l, b);
      e = __builtin_amdgcn_readfirstlane(p.eids[l * p.nb + b]);
    }
    const int tid = threadIdx.x;
    int valid = 0;
    if (tid < p.B) {
      const int pid = NAIVE ? s_pair[tid] : p.sorted[l * p.cap + b * p.B + tid];
      valid = pid < p.numel;
      s_pair[tid] = pid;
      s_row[tid] = valid ? (p.x_per_pair ? pid : pid / p.topk) : 0;
    }
    // valid rows form a prefix of the block (sentinels only pad a group's end)
    nv = __builtin_amdgcn_readfirstlane(__syncthreads_count(valid));
  }
  const int64_t wsel = (int64_t(s) * p.L + l) * p.E + e;
  const uint16_t* A = p.a + wsel * p.r * p.K;
  const uint16_t* Bm = p.b + wsel * p.Ns * p.r;

  // one-row blocks (most of a decode batch's) get their own instantiation:
  // a two-row group would repeat the row's loads and products (120b-like
  // decode, kernel us: w13 7.5 -> 7.3, w2 7.5 -> 6.8 one launch)
  if (nv <= 1)
    valu_rows<1, JW, CPR>(p, A, Bm, s_row, s_pair, nv, sh, s_part, s_v, s_d, s, n0, n1);
  else if (nv <= 2)
    valu_rows<2, JW, CPR>(p, A, Bm, s_row, s_pair, nv, sh, s_part, s_v, s_d, s, n0, n1);
  else
    valu_rows<4, JW, CPR>(p, A, Bm, s_row, s_pair, nv, sh, s_part, s_v, s_d, s, n0, n1);
}

template <int JW, int CPR>
static void launch(const FusedParams& p, ShrinkShape sh, dim3 grid, hipStream_t st) {
  if (p.naive) hipLaunchKernelGGL((fused_valu_kernel<JW, CPR, true>), grid, dim3(kThreads), 0, st, p, sh);
  else hipLaunchKernelGGL((fused_valu_kernel<JW, CPR, false>), grid, dim3(kThreads), 0, st, p, sh);
}

// The kernel for these sizes (not the stream kernel's), launched on st.
hipError_t launch_valu(const FusedParams& p, hipStream_t st) {
  // rows of A per wavefront and the wave arrangement
  int jw = 1;
  while (jw < p.r && jw < 16) jw <<= 1;
  ShrinkShape sh;
  sh.rgw = std::min(kWaves, (p.r + jw - 1) / jw);
  sh.kp = std::max(1, kWaves / sh.rgw);
  // grid: covers split * u8 + unit for every split count the kernel can pick:
  // u8 <= units_pad with one split, and n_split * u8 <= 8 * xcd_cus * OCC with more.
  const int64_t units_pad = (int64_t(p.units) + kXcds - 1) / kXcds * kXcds;
  const int64_t grid = std::max<int64_t>(units_pad, int64_t(kXcds) * p.xcd_cus * MLR_VALU_OCC);
  const int cpr = (p.r % 8 == 0 && ((p.r / 8) & (p.r / 8 - 1)) == 0) ? p.r / 8 : 0;
#define MLR_CASE(JW_, CPR_) \
  if (jw == JW_ && cpr == CPR_) { launch<JW_, CPR_>(p, sh, dim3(unsigned(grid)), st); return hipGetLastError(); }
  MLR_CASE(16, 2)
#ifndef MLR_VALU_R16_ONLY
  MLR_CASE(16, 16)
  MLR_CASE(16, 8)
  MLR_CASE(16, 4)
  MLR_CASE(8, 1)
  MLR_CASE(16, 0)
  MLR_CASE(8, 0)
  MLR_CASE(4, 0)
  MLR_CASE(2, 0)
  MLR_CASE(1, 0)
#endif
#undef MLR_CASE
  return hipErrorInvalidValue;
}

