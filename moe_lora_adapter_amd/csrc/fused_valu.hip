// Fused shrink + expand with vector loads and wavefront reductions (the
// decode-sized path).  One workgroup handles one (block, slice, column split):
//
//   shrink  v[i][j] = sum_t X[row_i][t] A[j][t]   -- lanes walk K in 16-byte
//           chunks (coalesced: a wavefront reads 1 KiB of one A row per load),
//           each wave owns a few A rows at a time, bf16 pairs are multiplied
//           with v_dot2, and the 64 lane partials are folded with a
//           reduce-scatter butterfly so one pass yields RG*JW sums;
//   v       stays in LDS (fp32), never in global memory;
//   expand  d[i][n] = sum_j v[i][j] B[n][j]        -- one thread per output
//           column n of this split; Y is read (add_inputs) and written with
//           consecutive columns on consecutive lanes.
//
// The prhub summary of vLLM PR #42290 (implementation steps) describes the
// one-shot kernel: x loaded once, multiplied by lora_a, the rank-sized result
// kept in registers and multiplied by lora_b, written over or added onto the
// output.  This kernel keeps that shape; the column split (several
// workgroups per block, each redoing the small shrink) gives a decode batch
// enough workgroups to pull HBM bandwidth, and workgroup ids are mapped so the
// splits of one block land on the same XCD and re-read A from its L2.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace mlr {

constexpr int kValuThreads = 256;
constexpr int kValuWaves = kValuThreads / kWave;
constexpr int kRG = 4;   // X rows per group
constexpr int kJW = 4;   // A rows per wave per pass
constexpr int kMaxB = 128;
constexpr int kMaxR = 128;

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Block g (over all active slots, in slot order) -> slot l, block b in slot.
// Every lane of the calling wavefront gets the same answer.
__device__ __forceinline__ bool find_block(const FusedParams& p, int g, int& l, int& b) {
  int run = 0;
  for (int c0 = 0; c0 < p.L; c0 += kWave) {
    const int sl = c0 + lane_id();
    const int nbk = sl < p.L ? p.ntpp[sl] / p.B : 0;
    const int incl = wave_incl_scan(nbk) + run;
    const uint64_t hit = __ballot(incl > g);
    if (hit) {
      const int first = __builtin_ctzll(hit);
      l = c0 + first;
      b = g - (__shfl(incl, first) - __shfl(nbk, first));
      return true;
    }
    run = __shfl(incl, kWave - 1);
  }
  return false;
}

// Sum NV per-lane values over the wavefront.  On return the lane holds the
// total of value index `which`; lanes whose index bits agree hold the same.
template <int NV>
__device__ __forceinline__ float reduce_scatter(float (&v)[NV], int& which) {
  const int lane = lane_id();
  which = 0;
  int o = kWave / 2;
#pragma unroll
  for (int half = NV / 2; half >= 1; half >>= 1, o >>= 1) {
    const bool up = lane & o;
#pragma unroll
    for (int q = 0; q < half; ++q) {
      const float send = up ? v[q] : v[q + half];
      const float keep = up ? v[q + half] : v[q];
      v[q] = keep + __shfl_xor(send, o);
    }
    if (up) which += half;
  }
  float t = v[0];
  for (; o >= 1; o >>= 1) t += __shfl_xor(t, o);
  return t;
}

__device__ void shrink_group(const FusedParams& p, const uint16_t* __restrict__ A,
                             const int* s_row, int nr, float* s_v) {
  const int K8 = p.K >> 3;
  const int w = wave_id(), lane = lane_id();
  const uint16_t* xr[kRG];
#pragma unroll
  for (int i = 0; i < kRG; ++i) xr[i] = p.x + int64_t(s_row[i < nr ? i : 0]) * p.K;
  for (int jb = w * kJW; jb < p.r; jb += kValuWaves * kJW) {
    float acc[kRG * kJW];
#pragma unroll
    for (int q = 0; q < kRG * kJW; ++q) acc[q] = 0.f;
    const int jn = min(kJW, p.r - jb);
    for (int c = lane; c < K8; c += kWave) {
      uint4 xv[kRG];
#pragma unroll
      for (int i = 0; i < kRG; ++i) xv[i] = ld16(xr[i] + c * 8);
#pragma unroll
      for (int jj = 0; jj < kJW; ++jj) {
        if (jj < jn) {
          const uint4 av = ld16(A + int64_t(jb + jj) * p.K + c * 8);
#pragma unroll
          for (int i = 0; i < kRG; ++i) acc[i * kJW + jj] = dot8_bf16(av, xv[i], acc[i * kJW + jj]);
        }
      }
    }
    int which;
    const float t = reduce_scatter<kRG * kJW>(acc, which);
    if ((lane & (kWave / (kRG * kJW) - 1)) == 0) {
      const int i = which / kJW, jj = which % kJW;
      if (i < nr && jj < jn) s_v[i * kMaxR + jb + jj] = t;
    }
  }
}

__device__ void expand_group(const FusedParams& p, const uint16_t* __restrict__ Bm,
                             const int* s_pair, int nr, const float* s_v, int s, int n0,
                             int n1) {
  for (int n = n0 + int(threadIdx.x); n < n1; n += kValuThreads) {
    const uint16_t* brow = Bm + int64_t(n) * p.r;
    float acc[kRG];
#pragma unroll
    for (int i = 0; i < kRG; ++i) acc[i] = 0.f;
    if ((p.r & 7) == 0) {
      for (int j0 = 0; j0 < p.r; j0 += 8) {
        const uint4 bv = ld16(brow + j0);
        const float bf[8] = {bf16_lo(bv.x), bf16_hi(bv.x), bf16_lo(bv.y), bf16_hi(bv.y),
                             bf16_lo(bv.z), bf16_hi(bv.z), bf16_lo(bv.w), bf16_hi(bv.w)};
#pragma unroll
        for (int i = 0; i < kRG; ++i) {
          if (i < nr) {
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[i] += s_v[i * kMaxR + j0 + q] * bf[q];
          }
        }
      }
    } else {
      for (int j = 0; j < p.r; ++j) {
        const float bj = bf16_to_f32(brow[j]);
#pragma unroll
        for (int i = 0; i < kRG; ++i)
          if (i < nr) acc[i] += s_v[i * kMaxR + j] * bj;
      }
    }
#pragma unroll
    for (int i = 0; i < kRG; ++i) {
      if (i < nr) {
        const int pair = s_pair[i];
        float val = acc[i];
        if (p.mul) val *= p.w[pair];
        uint16_t* yp = p.y + int64_t(pair) * p.N + s * p.Ns + n;
        if (p.add) val += bf16_to_f32(*yp);
        *yp = f32_to_bf16(val);
      }
    }
  }
}

__global__ void __launch_bounds__(kValuThreads) fused_valu_kernel(FusedParams p) {
  __shared__ int s_pair[kMaxB];
  __shared__ int s_row[kMaxB];
  __shared__ float s_v[kRG * kMaxR];

  // workgroup id -> (unit, split); the splits of one unit share an XCD
  const int id = blockIdx.x;
  const int xcd = id % kXcds, q = id / kXcds;
  const int unit = (q / p.n_split) * kXcds + xcd;
  const int split = q % p.n_split;
  if (unit >= p.units) return;
  const int g = unit / p.S, s = unit - g * p.S;
  const int n0 = split * p.nsz;
  if (n0 >= p.Ns) return;
  const int n1 = min(p.Ns, n0 + p.nsz);
  int l, b;
  if (!find_block(p, g, l, b)) return;
  const int e = p.eids[l * p.nb + b];

  const int tid = threadIdx.x;
  int valid = 0;
  if (tid < p.B) {
    const int pid = p.sorted[l * p.cap + b * p.B + tid];
    valid = pid < p.numel;
    s_pair[tid] = pid;
    s_row[tid] = valid ? (p.x_per_pair ? pid : pid / p.topk) : 0;
  }
  // valid rows form a prefix of the block (sentinels only pad a group's end)
  const int nv = __syncthreads_count(valid);

  const int64_t wsel = (int64_t(s) * p.L + l) * p.E + e;
  const uint16_t* A = p.a + wsel * p.r * p.K;
  const uint16_t* Bm = p.b + wsel * p.Ns * p.r;
  for (int g0 = 0; g0 < nv; g0 += kRG) {
    const int nr = min(kRG, nv - g0);
    shrink_group(p, A, s_row + g0, nr, s_v);
    __syncthreads();
    expand_group(p, Bm, s_pair + g0, nr, s_v, s, n0, n1);
    __syncthreads();
  }
}

hipError_t launch_fused_valu(FusedParams p, hipStream_t st) {
  // enough workgroups to keep every CU streaming: aim for ~512 in total
  int n_split = (512 + p.units - 1) / p.units;
  const int max_split = std::max(1, p.Ns / 256);
  n_split = std::max(1, std::min(n_split, max_split));
  p.n_split = n_split;
  p.nsz = ((p.Ns + n_split - 1) / n_split + 7) / 8 * 8;
  const int64_t units_pad = (int64_t(p.units) + kXcds - 1) / kXcds * kXcds;
  const int64_t grid = units_pad * n_split;
  hipLaunchKernelGGL(fused_valu_kernel, dim3(unsigned(grid)), dim3(kValuThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace mlr
