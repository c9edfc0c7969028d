// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlr {

constexpr int kWave = 64;  // CDNA wavefront width
constexpr int kXcds = 8;   // MI355X: 8 accelerator complex dies, 32 CUs each

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
// Wavefront index within the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return (uint64_t(1) << lane) - 1;
}

// DPP move of a lane value (VALU, no trip through the LDS crossbar): the
// result of a lane whose source lies outside the pattern, or whose row is
// not in row_mask, is 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_move(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, false);
}

// The partner of this lane in a butterfly at distance O (a power of two
// below 64): lane ^ O, except that O = 4 pairs lane i with i ^ 7 inside
// each group of 8 (DPP's half-row mirror).  Both differ from the lane in
// bit log2(O) and agree on the bits above it, so a sum or reduce-scatter
// over the levels O = 32, 16, ..., 1 pairs the same halves either way.
// O = 32 and 16 are gfx950's lane-swap instructions, 8 a row rotation, 4, 2
// and 1 DPP within a row.
template <int O>
__device__ __forceinline__ uint32_t butterfly_partner(uint32_t v) {
  static_assert(O == 1 || O == 2 || O == 4 || O == 8 || O == 16 || O == 32, "distance");
  if constexpr (O == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane_id() & 32) ? r[0] : r[1];
  } else if constexpr (O == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane_id() & 16) ? r[0] : r[1];
  } else if constexpr (O == 8) {
    return uint32_t(dpp_move<0x128>(int(v)));  // row_ror:8
  } else if constexpr (O == 4) {
    return uint32_t(dpp_move<0x141>(int(v)));  // row_half_mirror
  } else if constexpr (O == 2) {
    return uint32_t(dpp_move<0x4e>(int(v)));   // quad_perm [2,3,0,1]
  } else {
    return uint32_t(dpp_move<0xb1>(int(v)));   // quad_perm [1,0,3,2]
  }
}

__device__ __forceinline__ float butterfly_partner(float v, int o) {
  const uint32_t u = __float_as_uint(v);
  // o is a constant wherever this is called from an unrolled loop
  switch (o) {
    case 32: return __uint_as_float(butterfly_partner<32>(u));
    case 16: return __uint_as_float(butterfly_partner<16>(u));
    case 8: return __uint_as_float(butterfly_partner<8>(u));
    case 4: return __uint_as_float(butterfly_partner<4>(u));
    case 2: return __uint_as_float(butterfly_partner<2>(u));
    default: return __uint_as_float(butterfly_partner<1>(u));
  }
}

// Inclusive prefix sum over the 64 lanes of a wavefront: shifts by 1, 2, 4
// and 8 inside each row of 16 lanes, then the last lane of row 0 added to row
// 1 and of row 2 to row 3, then the last lane of row 1 to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_move<0x111>(v);       // row_shr:1
  v += dpp_move<0x112>(v);       // row_shr:2
  v += dpp_move<0x114>(v);       // row_shr:4
  v += dpp_move<0x118>(v);       // row_shr:8
  v += dpp_move<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_move<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// The value of lane `src` (wave-uniform) in every lane.
__device__ __forceinline__ int lane_value(int v, int src) {
  return __builtin_amdgcn_readlane(v, src);
}


// Mask of the lanes (among `active`) whose key equals this lane's key, found
// by voting on each key bit in turn.  Keys are below 2^nbits.
__device__ __forceinline__ uint64_t match_key(int key, uint64_t active, int nbits) {
  uint64_t peers = active;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t ones = __ballot(bit);
    peers &= bit ? ones : ~ones;
  }
  return peers;
}

// Workgroup barrier that orders LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global loads (a __syncthreads() fence
// would drain those too and stall a load pipeline at every barrier).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt, expcnt untouched
  __builtin_amdgcn_s_barrier();
}

// Exclusive prefix sum, in place, of a[0..n) held in LDS, by the whole
// workgroup (blockDim.x a multiple of 64, at most 1024).  `wtot` is LDS
// scratch of at least 17 ints.  Returns the total to every thread.  Contains
// barriers: every thread of the block must call it.
__device__ inline int block_excl_scan(int* a, int n, int* wtot) {
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int nw = blockDim.x / kWave;
  int carry = 0;
  for (int base = 0; base < n; base += blockDim.x) {
    const int i = base + tid;
    const int v = i < n ? a[i] : 0;
    const int incl = wave_incl_scan(v);
    if (lane == kWave - 1) wtot[w] = incl;
    __syncthreads();
    if (w == 0) {
      const int t = lane < nw ? wtot[lane] : 0;
      const int ti = wave_incl_scan(t);
      if (lane < nw) wtot[lane] = ti - t;
      if (lane == nw - 1) wtot[16] = ti;
    }
    __syncthreads();
    if (i < n) a[i] = carry + wtot[w] + incl - v;
    carry += wtot[16];
    __syncthreads();
  }
  return carry;
}

// bf16 <-> fp32.  Widening is exact (the bf16 bits are the upper half of the
// binary32 value).  Narrowing rounds to nearest, ties to even, from the IEEE
// definition; NaN stays a quiet NaN.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// f32 -> bf16, rounded to nearest even, subnormals kept, NaN stays NaN: one
// v_cvt_pk_bf16_f32 (gfx950), which rounds exactly as adding 0x7fff plus the
// kept lowest bit to the f32 pattern and truncating does, for every finite
// input.  The pair form converts two values with one instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// lo in bits 0..15, hi in bits 16..31
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Raw buffer access: a wave-uniform descriptor (base, byte range) in scalar
// registers, a 32-bit per-lane byte offset and a wave-uniform byte offset.
// Reads past the range return zero.  Word 3 is the gfx9-family format word.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}
// Cache policy of a buffer access (the instruction's aux bits): 0 = default,
// kNonTemporal = nt (evict-first, for data a kernel touches once).
constexpr int kNonTemporal = 2;
template <int AUX = 0>
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, int(voff), int(soff), AUX);
  return make_uint4(uint32_t(v.x), uint32_t(v.y), uint32_t(v.z), uint32_t(v.w));
}

// Stores past the range are dropped.
template <int AUX = 0>
__device__ __forceinline__ void buf_st16(uint4 v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const i32x4_t d = {int(v.x), int(v.y), int(v.z), int(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(d, r, int(voff), int(soff), AUX);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// acc + a.lo*b.lo + a.hi*b.hi on two packed bf16 pairs (v_dot2 on gfx950).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// 8 bf16 x 8 bf16 dot product added onto acc.
__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b, float acc) {
  acc = dot2_bf16(a.x, b.x, acc);
  acc = dot2_bf16(a.y, b.y, acc);
  acc = dot2_bf16(a.z, b.z, acc);
  acc = dot2_bf16(a.w, b.w, acc);
  return acc;
}

}  // namespace mlr
