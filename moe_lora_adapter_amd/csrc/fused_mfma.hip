// Fused shrink + expand on bf16 MFMA tiles (the prefill-sized path).
//
// One workgroup (4 wavefronts) handles one (block, slice, column split).
// Rows of a block are taken 64 at a time:
//
//   shrink  V[64 x RP] = X_rows[64 x K] . A[s,l,e][RP x K]^T with
//           v_mfma_f32_16x16x32_bf16.  K advances in tiles of 64: the X rows
//           (gathered through sorted_token_ids) and the A rows are staged in
//           LDS, the next tile is fetched into registers while the current
//           one is multiplied.  Wavefront w owns output rows 16w..16w+15 and
//           all RP = r rounded up to 16 columns.
//   v       rounded to bf16 into LDS (the expand's A operand), zero padded to
//           RK = r rounded up to 32; it never leaves the chip.
//   expand  D[64 x 16] per wavefront and column tile = V . B[cols][RK]^T,
//           wavefront w taking columns 16w..16w+15 of every 64-column tile,
//           with V held in registers and B read straight from global memory
//           (each B element is read once).  The epilogue scales by the routed
//           weight and adds onto Y (add_inputs) before the bf16 store.
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
#include "internal.h"

namespace mlr {
namespace {

constexpr int kThreadsM = 256;
constexpr int kTileM = 64;    // rows per row tile
constexpr int kTileK = 64;    // K per staged tile
constexpr int kPitch = kTileK + 8;  // LDS row pitch (bf16) of X / A tiles
constexpr int kMaxRP = 128;
constexpr int kVPitch = kMaxRP + 8;  // LDS row pitch (bf16) of V

#ifndef MLR_MFMA_WG_TARGET
#define MLR_MFMA_WG_TARGET 512
#endif
#ifndef MLR_MFMA_MIN_COLS
#define MLR_MFMA_MIN_COLS 256
#endif

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Register staging of one K tile: X rows (64 x 64) and A rows (RP x 64), as
// 16-byte chunks; each thread holds XC + AC chunks.
template <int RT>
struct TileRegs {
  static constexpr int XC = kTileM * (kTileK / 8) / kThreadsM;                   // 2
  static constexpr int ACN = ((RT * 16) * (kTileK / 8) + kThreadsM - 1) / kThreadsM;  // ceil
  uint4 x[XC];
  uint4 a[ACN];
};

// Chunk c of a [rows x 8] chunk grid: row c / 8, chunk c % 8.
template <int RT>
__device__ __forceinline__ void fetch_tile(const FusedParams& p, const uint16_t* __restrict__ A,
                                           const int* s_row, int k0, TileRegs<RT>& t) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < TileRegs<RT>::XC; ++q) {
    const int c = q * kThreadsM + tid;
    const int row = c >> 3, k = k0 + (c & 7) * 8;
    const int xr = s_row[row];
    t.x[q] = (xr >= 0 && k < p.K) ? ldg16(p.x + int64_t(xr) * p.K + k) : make_uint4(0, 0, 0, 0);
  }
  constexpr int RP = RT * 16;
#pragma unroll
  for (int q = 0; q < TileRegs<RT>::ACN; ++q) {
    const int c = q * kThreadsM + tid;
    const int j = c >> 3, k = k0 + (c & 7) * 8;
    const bool ok = c < RP * 8 && j < p.r && k < p.K;
    t.a[q] = ok ? ldg16(A + int64_t(j) * p.K + k) : make_uint4(0, 0, 0, 0);
  }
}

template <int RT>
__device__ __forceinline__ void store_tile(const TileRegs<RT>& t, uint16_t* s_x, uint16_t* s_a) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < TileRegs<RT>::XC; ++q) {
    const int c = q * kThreadsM + tid;
    *reinterpret_cast<uint4*>(s_x + (c >> 3) * kPitch + (c & 7) * 8) = t.x[q];
  }
  constexpr int RP = RT * 16;
#pragma unroll
  for (int q = 0; q < TileRegs<RT>::ACN; ++q) {
    const int c = q * kThreadsM + tid;
    if (c < RP * 8) *reinterpret_cast<uint4*>(s_a + (c >> 3) * kPitch + (c & 7) * 8) = t.a[q];
  }
}

template <int RT, int KS>
__global__ void __launch_bounds__(kThreadsM) fused_mfma_kernel(FusedParams p) {
  constexpr int RP = RT * 16;
  constexpr int RK = KS * 32;
  __shared__ int s_pair[kTileM];
  __shared__ int s_row[kTileM];
  __shared__ __align__(16) uint16_t s_x[kTileM * kPitch];
  __shared__ __align__(16) uint16_t s_a[RP * kPitch];
  __shared__ __align__(16) uint16_t s_v[kTileM * kVPitch];

  const int total = __builtin_amdgcn_readfirstlane(count_blocks(p));
  const int units = total * p.S;
  const int u8 = (units + kXcds - 1) / kXcds * kXcds;
  const int max_split = max(1, p.Ns / MLR_MFMA_MIN_COLS);
  const int n_split = min(max_split, max(1, (MLR_MFMA_WG_TARGET + u8 - 1) / max(u8, 1)));
  const int id = blockIdx.x;
  const int split = id / max(u8, 1), unit = id - split * u8;
  if (unit >= units || split >= n_split) return;
  const int nsz = ((p.Ns + n_split - 1) / n_split + 15) / 16 * 16;
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

  const int tid = threadIdx.x, w = wave_id(), lane = lane_id();
  const int lr = lane & 15, lq = lane >> 4;

  for (int rt0 = 0; rt0 < p.B; rt0 += kTileM) {
    // rows of this tile: X row index (-1 = no row) and pair index
    if (tid < kTileM) {
      int pid = p.numel, xr = -1;
      if (rt0 + tid < p.B) {
        pid = p.sorted[l * p.cap + b * p.B + rt0 + tid];
        if (pid < p.numel) xr = p.x_per_pair ? pid : pid / p.topk;
      }
      s_pair[tid] = pid;
      s_row[tid] = xr;
    }
    const int nv = __builtin_amdgcn_readfirstlane(__syncthreads_count(tid < kTileM && s_row[tid] >= 0 ? 1 : 0));
    if (nv == 0) break;  // only sentinels from here on

    // ---------------- shrink
    f32x4_t acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    TileRegs<RT> regs;
    fetch_tile<RT>(p, A, s_row, 0, regs);
    for (int k0 = 0; k0 < p.K; k0 += kTileK) {
      __syncthreads();  // previous tile fully consumed
      store_tile<RT>(regs, s_x, s_a);
      __syncthreads();
      if (k0 + kTileK < p.K) fetch_tile<RT>(p, A, s_row, k0 + kTileK, regs);
#pragma unroll
      for (int ks = 0; ks < kTileK / 32; ++ks) {
        const uint4 xa = *reinterpret_cast<const uint4*>(s_x + (16 * w + lr) * kPitch + ks * 32 + lq * 8);
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          const uint4 ab = *reinterpret_cast<const uint4*>(s_a + (16 * t + lr) * kPitch + ks * 32 + lq * 8);
          acc[t] = mfma16(xa, ab, acc[t]);
        }
      }
    }
    // V (fp32, MFMA layout) -> bf16 rows of s_v, zero past RP up to RK
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s_v[(16 * w + 4 * lq + i) * kVPitch + 16 * t + lr] = f32_to_bf16(acc[t][i]);
    if constexpr (RK > RP) {
      for (int c = tid; c < kTileM * (RK - RP); c += kThreadsM)
        s_v[(c / (RK - RP)) * kVPitch + RP + c % (RK - RP)] = 0;
    }
    __syncthreads();

    // ---------------- expand: V (all 64 rows) in registers as MFMA A operands
    uint4 va[4][KS];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        va[rt][ks] = *reinterpret_cast<const uint4*>(s_v + (16 * rt + lr) * kVPitch + ks * 32 + lq * 8);
    float wrow[4][4];
    int prow[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * rt + 4 * lq + i;
        const int pid = s_pair[row];
        prow[rt][i] = pid;
        wrow[rt][i] = (p.mul && pid < p.numel) ? p.w[pid] : 1.f;
      }
    const int col_base = s * p.Ns;
    for (int nt = n0 + 16 * w; nt < n1; nt += 64) {
      const int n = nt + lr;
      uint4 bb[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int j = ks * 32 + lq * 8;
        bb[ks] = (n < n1 && j < p.r) ? ldg16(Bm + int64_t(n) * p.r + j) : make_uint4(0, 0, 0, 0);
      }
      uint16_t yin[4][4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pid = prow[rt][i];
          yin[rt][i] = (p.add && pid < p.numel && n < n1) ? p.y[int64_t(pid) * p.N + col_base + n] : uint16_t(0);
        }
      f32x4_t d[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        d[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) d[rt] = mfma16(va[rt][ks], bb[ks], d[rt]);
      }
      if (n < n1) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int pid = prow[rt][i];
            if (pid < p.numel) {
              float val = d[rt][i] * wrow[rt][i];
              if (p.add) val += bf16_to_f32(yin[rt][i]);
              p.y[int64_t(pid) * p.N + col_base + n] = f32_to_bf16(val);
            }
          }
      }
    }
    __syncthreads();  // s_row / s_pair / s_v reused by the next row tile
  }
}

// RT = ceil(r / 16) row tiles of the shrink, KS = ceil(r / 32) K steps of the
// expand; KS is fixed by RT.
template <int RT>
void launch_rt(const FusedParams& p, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL((fused_mfma_kernel<RT, (RT + 1) / 2>), grid, dim3(kThreadsM), 0, st, p);
}

}  // namespace

// B rows are read as 16-byte chunks of 8 ranks, so r must be a multiple of 8.
bool mfma_supported(int r, int B) {
  return r >= 8 && r <= kMaxRP && r % 8 == 0 && B >= 16 && B <= 128;
}

hipError_t launch_fused_mfma(FusedParams p, hipStream_t st) {
  const int rt = (p.r + 15) / 16;
  const int64_t units_pad = (int64_t(p.units) + kXcds - 1) / kXcds * kXcds;
  const dim3 grid(unsigned(MLR_MFMA_WG_TARGET + units_pad));
  switch (rt) {
    case 1: launch_rt<1>(p, grid, st); break;
    case 2: launch_rt<2>(p, grid, st); break;
    case 3: launch_rt<3>(p, grid, st); break;
    case 4: launch_rt<4>(p, grid, st); break;
    case 5: launch_rt<5>(p, grid, st); break;
    case 6: launch_rt<6>(p, grid, st); break;
    case 7: launch_rt<7>(p, grid, st); break;
    default: launch_rt<8>(p, grid, st); break;
  }
  return hipGetLastError();
}

}  // namespace mlr
