// The K-split exchange of the decode kernels: the workgroups that share a
// unit (its column splits, the "peers") each multiply a share of A's K range
// and meet to add their partial rank vectors, instead of every one of them
// reading all of A.
//
// Area layout, fixed by the number of slots the caller's workspace holds
// (never by the sizes of a call, so one workspace serves calls of any size):
//   uint32 left[nslot][kXchPeers]   the tag with which each peer last left the slot
//   uint64 words[nslot][kXchPeers][kXchRows][kXchMaxRank]   (from a 16-byte boundary)
// A word is an fp32 partial value in its low half and the tag of the call
// that wrote it in its high half.  A call's tag in a slot is one more than
// the largest `left` word of the slot, read when the pass starts; a peer
// writes its `left` word with its tag once it has read all it needs from the
// slot (a plain store: no atomic whose return would have to be waited for).
// Every peer that writes words in a slot also leaves it, so the largest
// `left` word is at least every tag ever written in the slot, and the next
// call's tag exceeds them all: a stale word never carries the current tag,
// whichever unit, rank or peer count used the slot before.  A consumer
// therefore polls the values themselves -- no flag, no fence, no wait
// between data and its announcement.  (A peer that starts after another has
// already left reads a larger tag than its peers used; it then finds none of
// their words and computes their partials itself, and they its -- the same
// bits, only later.)  Zero-filled before first use, the area is reused as it
// is, also inside a captured graph; calls that may overlap must not share an
// area.  (Tags are 32-bit: a slot used 2^32 times would wrap.)
//
// Stores are relaxed atomics at agent scope.  A consumer polls with
// non-temporal loads, which skip this compute unit's L1 (a plain load can
// hit a stale L1 line forever) and read the L2 the peers of a unit share
// (they run on one XCD): under a full streaming load a published word was
// seen 3.3 us after its store that way, against 4.3 us with agent-scope
// loads; idle, 0.7 and 0.6 us (MI355X, measured).  A peer on another XCD
// may keep reading its own L2's stale copy; it then computes the partial
// itself, with the same bits.  The `left` words are read with plain loads
// when a pass starts: every value a previous call stored is visible to a
// later kernel, and a store of the current call may or may not be seen,
// which the protocol allows.  Release / acquire fences at agent scope would
// order plain accesses instead, but each one writes back or invalidates a
// whole L2 (20 to 30 us per exchange, measured).
#pragma once

#include <stdint.h>

#include "common.h"

namespace mlr {

constexpr int kXchPeers = 8;       // most workgroups one K split spans
constexpr int kXchRows = 4;        // rows of one pass
constexpr int kXchMaxRank = 128;
constexpr int64_t kXchSlotWords = int64_t(kXchPeers) * kXchRows * kXchMaxRank;

__host__ __device__ inline int64_t xch_words_offset(int64_t nslot) {
  return (4 * kXchPeers * nslot + 15) / 16 * 16;
}
__host__ __device__ inline int64_t xch_area_bytes(int64_t nslot) {
  return xch_words_offset(nslot) + nslot * kXchSlotWords * 8;
}
// The most slots an area of `bytes` holds.
inline int64_t xch_slots_in(int64_t bytes) {
  int64_t n = bytes / (4 * kXchPeers + kXchSlotWords * 8);
  while (n > 0 && xch_area_bytes(n) > bytes) --n;
  return n;
}

struct XchSlot {
  uint32_t* left;   // [kXchPeers]
  uint64_t* words;  // [kXchPeers][kXchRows][kXchMaxRank]
};

__device__ __forceinline__ XchSlot xch_slot(int32_t* area, int nslot, int slot) {
  XchSlot x;
  x.left = reinterpret_cast<uint32_t*>(area) + int64_t(slot) * kXchPeers;
  x.words = reinterpret_cast<uint64_t*>(reinterpret_cast<uint8_t*>(area) + xch_words_offset(nslot)) +
            int64_t(slot) * kXchSlotWords;
  return x;
}

// The largest `left` word of the slot (one thread; the loads are issued
// together).  The call's tag is this + 1.
__device__ __forceinline__ uint32_t xch_last_tag(const XchSlot& x) {
  static_assert(kXchPeers == 8, "two 16-byte loads");
  const uint4 a = reinterpret_cast<const uint4*>(x.left)[0];
  const uint4 b = reinterpret_cast<const uint4*>(x.left)[1];
  const uint32_t t[kXchPeers] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t m = 0;
#pragma unroll
  for (int q = 0; q < kXchPeers; ++q) m = t[q] > m ? t[q] : m;
  return m;
}

__device__ __forceinline__ uint64_t* xch_word(const XchSlot& x, int peer, int row, int j) {
  return x.words + (peer * kXchRows + row) * kXchMaxRank + j;
}

__device__ __forceinline__ void xch_put(const XchSlot& x, int peer, int row, int j, float v, uint32_t tag) {
  const uint64_t word = uint64_t(__float_as_uint(v)) | (uint64_t(tag) << 32);
  __hip_atomic_store(xch_word(x, peer, row, j), word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t xch_get(const XchSlot& x, int peer, int row, int j) {
  return __builtin_nontemporal_load(xch_word(x, peer, row, j));
}

__device__ __forceinline__ bool xch_tagged(uint64_t word, uint32_t tag) { return uint32_t(word >> 32) == tag; }
__device__ __forceinline__ float xch_value(uint64_t word) { return __uint_as_float(uint32_t(word)); }

// One thread, after every read of the slot by its workgroup has returned.
__device__ __forceinline__ void xch_leave(const XchSlot& x, int peer, uint32_t tag) {
  __hip_atomic_store(x.left + peer, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace mlr
