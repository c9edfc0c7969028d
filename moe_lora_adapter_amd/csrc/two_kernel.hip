// Two-kernel shrink / expand: the rank vector goes through memory.
//
// The pages describe the path the one-shot kernel replaces (prhub summary of
// vLLM PR #42290, motivation: shrink and expand as two kernels with the
// intermediate written back to HBM; key source fragment: the one-shot kernel
// takes ranks up to 128 and leaves larger ranks to the two-kernel path; the
// PR #32005 diff shows the two launches, `_fused_moe_lora_shrink`
// with a `split_k` and `_fused_moe_lora_expand` with a column `offset`).  Here
// it is the path for ranks up to 512 and the comparator of the fused kernels.
//
//   shrink  one workgroup per (block, slice, group of 128 ranks, K split):
//           V^T[16 ranks x 16 rows] += A[16 ranks x 32 k] X^T[32 k x 16 rows]
//           on v_mfma_f32_16x16x32_bf16, two 16-rank tiles per wavefront, row
//           tiles of up to 64 rows per pass.  The X rows of a 128-wide K chunk
//           are staged once in LDS for all wavefronts (double buffered, the
//           next chunk loading during this one); each wavefront loads its A
//           rows straight into registers.  The partial sums of a K split go to their own slice of
//           the workspace, fp32 [split][slice][pair][rank]: the split gives a
//           decode batch enough workgroups without atomics, and the expand
//           adds the splits in a fixed order, so the result is deterministic.
//   expand  one workgroup per (block, slice, column split): the rank vectors
//           of up to 64 rows are summed over the splits and staged in LDS as
//           bf16 high and low parts (v = hi + lo); every wavefront takes four
//           16-column tiles of a 256-column group and accumulates
//           D^T = B[cols x r] (V_hi + V_lo)^T over all ranks, B straight from
//           memory (the next k-step's B loaded while the current one is
//           multiplied); the routed weight, the add onto Y and the bf16
//           rounding follow in registers.
// Blocks are found on the device from the align outputs, as in the fused
// kernels, and both launches depend on M alone.
#include <algorithm>

#include "blocks.h"
#include "common.h"
#include "dma.h"
#include "internal.h"

namespace mlr {
namespace {

constexpr int kT2 = 256;                // threads of both kernels
constexpr int kW2 = kT2 / kWave;        // wavefronts
constexpr int kPass2 = 64;              // rows per pass (four row tiles)
constexpr int kTilesPerWave = 2;        // shrink: 16-rank tiles per wavefront
constexpr int kRankGroup = 16 * kW2 * kTilesPerWave;  // ranks per shrink workgroup
static_assert(kRankGroup == kTwoKernelRankGroup, "rank group of the host-side bounds");
constexpr int kKC = 128;                // shrink: K per staged X chunk
constexpr int kCPR = kKC / 8;           // 16-byte chunks per X row of a chunk
constexpr int kXP = kKC + 8;            // bf16 pitch of a staged X row (bank spread)
constexpr int kXLoads = kPass2 * kCPR / kT2;  // X chunks per thread and K chunk
static_assert(kPass2 * kCPR % kT2 == 0, "X staging covers the rows evenly");
constexpr int kCT2 = 4;                 // expand: column tiles per wavefront and group
constexpr int kNCG2 = 16 * kW2 * kCT2;  // expand: columns per group
constexpr int64_t kMaxBuf = int64_t(1) << 31;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Block g of the align outputs -> slot, expert and the pair ids of pass r0
// (rows r0 .. r0 + 63 of the block) into s_pair / s_row; returns the valid rows.
__device__ __forceinline__ int load_pass_rows(const FusedParams& p, int l, int b, int r0,
                                              int* s_pair, int* s_row, float* s_wt) {
  const int tid = threadIdx.x;
  if (tid < kPass2) {
    int pid = p.numel, xr = -1;
    float wv = 1.f;
    if (r0 + tid < p.B) {
      const int id = p.sorted[l * p.cap + b * p.B + r0 + tid];
      if (id < p.numel) {
        pid = id;
        xr = p.x_per_pair ? id : id / p.topk;
        if (s_wt && p.mul) wv = p.w[id];
      }
    }
    s_pair[tid] = pid;
    s_row[tid] = xr;
    if (s_wt) s_wt[tid] = wv;
  }
  // valid rows are a prefix of the block (sentinels only pad a group's end)
  return __builtin_amdgcn_readfirstlane(__syncthreads_count(tid < kPass2 && s_row[tid] >= 0));
}

__global__ void __launch_bounds__(kT2) lora_shrink_kernel(FusedParams p) {
  __shared__ __align__(16) uint16_t s_x[2][kPass2 * kXP];  // X rows of a K chunk, two buffers
  __shared__ int s_pair[kPass2];
  __shared__ int s_row[kPass2];
  const BlockScan sc = scan_blocks(p);
  const int groups = (p.r + kRankGroup - 1) / kRankGroup;
  const int units = sc.total * p.S * groups * p.kz;
  int unit, split;
  if (!map_unit_xcd(blockIdx.x, units, 1, unit, split)) return;
  // unit -> (block, slice, rank group, K split), K split fastest
  const int kz = unit % p.kz;
  int rest = unit / p.kz;
  const int rg = rest % groups;
  rest /= groups;
  const int s = rest % p.S, g = rest / p.S;
  int l, b;
  find_block(p, sc, g, l, b);
  const int e = __builtin_amdgcn_readfirstlane(p.eids[l * p.nb + b]);
  const int64_t wsel = (int64_t(s) * p.L + l) * p.E + e;
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(p.a + wsel * p.r * p.K, uint32_t(p.r * p.K * 2));
  const int64_t x_rows = p.x_per_pair ? int64_t(p.numel) : int64_t(p.numel / p.topk);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x, uint32_t(x_rows * p.K * 2));
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id(), lr = lane & 15, lq = lane >> 4;
  const int k0 = kz * p.kchunk, k1 = min(p.K, k0 + p.kchunk);
  float* wsz = p.ws + (int64_t(kz) * p.S + s) * p.numel * p.r;
  // this lane's A rows: rank tiles 2 w and 2 w + 1 of the group
  int arow[kTilesPerWave];
#pragma unroll
  for (int t = 0; t < kTilesPerWave; ++t) arow[t] = rg * kRankGroup + 16 * (kTilesPerWave * w + t) + lr;

  for (int r0 = 0; r0 < p.B; r0 += kPass2) {
    const int nv = load_pass_rows(p, l, b, r0, s_pair, s_row, nullptr);
    if (nv == 0) break;
    const int mt = (nv + 15) / 16;
    // X staging: thread tid copies chunks q = tid + kT2 i of the K chunk, row
    // q / kCPR, 16-byte column q % kCPR (rows past nv and columns past k1 as zero)
    int xsrc[kXLoads];
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      const int q = tid + kT2 * i, row = q / kCPR;
      xsrc[i] = row < nv ? s_row[row] : -1;
    }
    auto load_x = [&](int kc, uint4 (&reg)[kXLoads]) {
#pragma unroll
      for (int i = 0; i < kXLoads; ++i) {
        const int q = tid + kT2 * i, kk = kc + 8 * (q % kCPR);
        reg[i] = buf_ld16(xr, (xsrc[i] >= 0 && kk < k1) ? uint32_t(xsrc[i] * p.K + kk) * 2u : kOob, 0);
      }
    };
    auto store_x = [&](int buf, const uint4 (&reg)[kXLoads]) {
#pragma unroll
      for (int i = 0; i < kXLoads; ++i) {
        const int q = tid + kT2 * i;
        *reinterpret_cast<uint4*>(&s_x[buf][(q / kCPR) * kXP + 8 * (q % kCPR)]) = reg[i];
      }
    };
    auto load_a = [&](int kc, uint4 (&a)[kTilesPerWave][kKC / 32]) {
#pragma unroll
      for (int t = 0; t < kTilesPerWave; ++t)
#pragma unroll
        for (int u = 0; u < kKC / 32; ++u) {
          const int kk = kc + 32 * u + 8 * lq;
          a[t][u] = buf_ld16(ar, (kk < k1 && arow[t] < p.r) ? uint32_t(arow[t] * p.K + kk) * 2u : kOob, 0);
        }
    };
    f32x4_t acc[kTilesPerWave][4];
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[t][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint4 xreg[kXLoads];
    uint4 a[kTilesPerWave][kKC / 32], anxt[kTilesPerWave][kKC / 32];
    load_a(k0, a);
    load_x(k0, xreg);
    store_x(0, xreg);
    __syncthreads();
    int buf = 0;
    for (int kc = k0; kc < k1; kc += kKC) {
      const bool more = kc + kKC < k1;
      if (more) {  // the next chunk's X and A, in flight during this one
        load_x(kc + kKC, xreg);
        load_a(kc + kKC, anxt);
      }
#pragma unroll
      for (int u = 0; u < kKC / 32; ++u)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (m < mt) {
            const uint4 xo = *reinterpret_cast<const uint4*>(&s_x[buf][(16 * m + lr) * kXP + 32 * u + 8 * lq]);
#pragma unroll
            for (int t = 0; t < kTilesPerWave; ++t) acc[t][m] = mfma16(a[t][u], xo, acc[t][m]);
          }
        }
      if (more) store_x(buf ^ 1, xreg);
      __syncthreads();  // the other buffer is filled; this one may be overwritten next
      buf ^= 1;
#pragma unroll
      for (int t = 0; t < kTilesPerWave; ++t)
#pragma unroll
        for (int u = 0; u < kKC / 32; ++u) a[t][u] = anxt[t][u];
    }
    // lane (lr, lq) holds V[row 16 m + lr][ranks of tile (2 w + t): 4 lq .. 4 lq + 3]
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int j0 = rg * kRankGroup + 16 * (kTilesPerWave * w + t) + 4 * lq;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int row = 16 * m + lr;
        if (m < mt && row < nv && j0 < p.r) {
          float* dst = wsz + int64_t(s_pair[row]) * p.r + j0;
          if ((p.r & 3) == 0) {
            *reinterpret_cast<float4*>(dst) =
                make_float4(acc[t][m][0], acc[t][m][1], acc[t][m][2], acc[t][m][3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (j0 + i < p.r) dst[i] = acc[t][m][i];
          }
        }
      }
    }
    __syncthreads();  // row tables are reused by the next pass
  }
}

// RP: ranks padded to a multiple of 32 that the LDS copy of V is sized for.
template <int RP>
__global__ void __launch_bounds__(kT2) __attribute__((amdgpu_waves_per_eu(RP <= 256 ? 2 : 1)))
lora_expand_kernel(FusedParams p) {
  constexpr int VP = RP + 8;  // bf16 pitch of the V rows
  __shared__ __align__(16) uint16_t s_vh[kPass2 * VP];
  __shared__ __align__(16) uint16_t s_vl[kPass2 * VP];
  __shared__ int s_pair[kPass2];
  __shared__ int s_row[kPass2];
  __shared__ float s_wt[kPass2];

  const BlockScan sc = scan_blocks(p);
  const int units = sc.total * p.S;
  const int per_xcd = (units + kXcds - 1) / kXcds;
  const int max_split = max(1, p.Ns / kNCG2);
  const int n_split = min(max_split, max(1, p.xcd_cus * 2 / max(per_xcd, 1)));
  int unit, split;
  if (!map_unit_xcd(blockIdx.x, units, n_split, unit, split)) return;
  const int nsz = ((p.Ns + n_split - 1) / n_split + 15) / 16 * 16;
  const int n0 = split * nsz;
  if (n0 >= p.Ns) return;
  const int n1 = min(p.Ns, n0 + nsz);
  const int g = unit / p.S, s = unit - g * p.S;
  int l, b;
  find_block(p, sc, g, l, b);
  const int e = __builtin_amdgcn_readfirstlane(p.eids[l * p.nb + b]);
  const int64_t wsel = (int64_t(s) * p.L + l) * p.E + e;
  const uint16_t* bmat = p.b + wsel * p.Ns * p.r;
  const __amdgpu_buffer_rsrc_t br = make_rsrc(bmat, uint32_t(p.Ns * p.r * 2));
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id(), lr = lane & 15, lq = lane >> 4;
  const int KS = (p.r + 31) / 32;
  const int64_t zstride = int64_t(p.S) * p.numel * p.r;
  const float* wss = p.ws + int64_t(s) * p.numel * p.r;

  for (int r0 = 0; r0 < p.B; r0 += kPass2) {
    const int nv = load_pass_rows(p, l, b, r0, s_pair, s_row, s_wt);
    if (nv == 0) break;
    const int mt = (nv + 15) / 16;
    // V of the pass rows: the K splits added in order, then hi / lo parts
    for (int q = tid; q < kPass2 * RP; q += kT2) {
      const int i = q / RP, j = q - i * RP;
      float v = 0.f;
      if (i < nv && j < p.r) {
        const float* src = wss + int64_t(s_pair[i]) * p.r + j;
        for (int z = 0; z < p.kz; ++z) v += src[z * zstride];
      }
      const uint16_t hi = f32_to_bf16(v);
      s_vh[i * VP + j] = hi;
      s_vl[i * VP + j] = f32_to_bf16(v - bf16_to_f32(hi));
    }
    __syncthreads();
    int64_t yrow[4];
    bool rv[4];
    float wt[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int pid = s_pair[16 * m + lr];
      rv[m] = m < mt && pid < p.numel;
      yrow[m] = rv[m] ? int64_t(pid) * p.N + int64_t(s) * p.Ns : 0;
      wt[m] = s_wt[16 * m + lr];
    }
    for (int nb = n0; nb < n1; nb += kNCG2) {
      // Y of this lane's rows and columns first: their latency hides behind the products
      uint2 yv[kCT2][4];
#pragma unroll
      for (int i = 0; i < kCT2; ++i) {
        const int n = nb + 16 * (w + kW2 * i) + 4 * lq;
#pragma unroll
        for (int m = 0; m < 4; ++m)
          yv[i][m] = (p.add && rv[m] && n < n1) ? *reinterpret_cast<const uint2*>(p.y + yrow[m] + n)
                                                : make_uint2(0, 0);
      }
      f32x4_t acc[kCT2][4];
#pragma unroll
      for (int i = 0; i < kCT2; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[i][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      uint4 bcur[kCT2], bnxt[kCT2];
      // B chunk of 8 ranks; a chunk that would run past the end of its row
      // (r not a multiple of 8) is read element by element: as one 16-byte
      // load it would also run past the matrix for the last column, where the
      // buffer range check zeroes the whole access
      auto load_b = [&](int ks, uint4 (&dst)[kCT2]) {
#pragma unroll
        for (int i = 0; i < kCT2; ++i) {
          const int col = nb + 16 * (w + kW2 * i) + lr;
          const int j = 32 * ks + 8 * lq;
          if (j + 8 <= p.r || col >= n1 || j >= p.r) {
            dst[i] = buf_ld16(br, (col < n1 && j < p.r) ? uint32_t(col * p.r + j) * 2u : kOob, 0);
          } else {
            const uint16_t* src = bmat + int64_t(col) * p.r + j;
            uint32_t h[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) h[q] = j + q < p.r ? src[q] : 0u;
            dst[i] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                h[6] | (h[7] << 16));
          }
        }
      };
      load_b(0, bcur);
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) load_b(ks + 1, bnxt);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (m < mt) {
            const int at = (16 * m + lr) * VP + 32 * ks + 8 * lq;
            const uint4 vh = *reinterpret_cast<const uint4*>(s_vh + at);
            const uint4 vl = *reinterpret_cast<const uint4*>(s_vl + at);
#pragma unroll
            for (int i = 0; i < kCT2; ++i) {
              acc[i][m] = mfma16(bcur[i], vh, acc[i][m]);
              acc[i][m] = mfma16(bcur[i], vl, acc[i][m]);
            }
          }
        }
#pragma unroll
        for (int i = 0; i < kCT2; ++i) bcur[i] = bnxt[i];
      }
      // lane (lr, lq): row 16 m + lr, columns 16 (w + 4 i) + 4 lq .. + 3
#pragma unroll
      for (int i = 0; i < kCT2; ++i) {
        const int n = nb + 16 * (w + kW2 * i) + 4 * lq;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (rv[m] && n < n1) {
            float o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = acc[i][m][q] * wt[m];
            if (p.add) {
              o[0] += bf16_lo(yv[i][m].x);
              o[1] += bf16_hi(yv[i][m].x);
              o[2] += bf16_lo(yv[i][m].y);
              o[3] += bf16_hi(yv[i][m].y);
            }
            *reinterpret_cast<uint2*>(p.y + yrow[m] + n) =
                make_uint2(pack_bf16x2(o[0], o[1]),
                           pack_bf16x2(o[2], o[3]));
          }
        }
      }
    }
    __syncthreads();  // V and the row tables are reused by the next pass
  }
}

}  // namespace

// K splits: enough shrink workgroups to give every compute unit two (by the
// bound on blocks), each split at least 256 of K, at most 8 splits.
int two_kernel_splits(int64_t units_bound, int64_t K, int r) {
  const int64_t groups = (r + kRankGroup - 1) / kRankGroup;
  const int64_t wgs = std::max<int64_t>(1, units_bound * groups);
  int kz = int(std::min<int64_t>(8, (2 * 256 + wgs - 1) / wgs));
  kz = int(std::min<int64_t>(kz, std::max<int64_t>(1, K / 256)));
  return std::max(1, kz);
}

hipError_t launch_two_kernel(FusedParams p, hipStream_t st) {
  if (p.r > kMaxRankTwoKernel) return hipErrorInvalidValue;
  const int64_t groups = (p.r + kRankGroup - 1) / kRankGroup;
  const int64_t shrink_units = int64_t(p.units) * groups * p.kz;  // p.units = blocks x S bound
  const dim3 g1(unsigned((shrink_units + kXcds - 1) / kXcds * kXcds));
  hipLaunchKernelGGL(lora_shrink_kernel, g1, dim3(kT2), 0, st, p);
  const hipError_t e1 = hipGetLastError();
  if (e1 != hipSuccess) return e1;
  const int64_t per_xcd = (int64_t(p.units) + kXcds - 1) / kXcds;
  const int64_t slots = std::max<int64_t>(per_xcd, int64_t(p.xcd_cus) * 2);
  const dim3 g2(unsigned(kXcds * slots));
  const int rp = (p.r + 31) / 32 * 32;
  if (rp <= 32) hipLaunchKernelGGL(lora_expand_kernel<32>, g2, dim3(kT2), 0, st, p);
  else if (rp <= 64) hipLaunchKernelGGL(lora_expand_kernel<64>, g2, dim3(kT2), 0, st, p);
  else if (rp <= 128) hipLaunchKernelGGL(lora_expand_kernel<128>, g2, dim3(kT2), 0, st, p);
  else if (rp <= 256) hipLaunchKernelGGL(lora_expand_kernel<256>, g2, dim3(kT2), 0, st, p);
  else hipLaunchKernelGGL(lora_expand_kernel<512>, g2, dim3(kT2), 0, st, p);
  return hipGetLastError();
}

bool two_kernel_fits(int64_t x_bytes, int64_t r, int64_t K, int64_t Ns) {
  return x_bytes <= kMaxBuf && r * K * 2 <= kMaxBuf && r * Ns * 2 <= kMaxBuf;
}

}  // namespace mlr
