// C ABI of the MoE-LoRA hot path: argument checks, sizing, dispatch.
// Every check runs on the host before any HIP call; a failing check returns
// a negative status with nothing launched and nothing written.
#include <stdint.h>

#include <algorithm>

#include "../../include/moe_lora.h"
#include "common.h"
#include "internal.h"
#include "xch.h"

using namespace mlr;

namespace {

constexpr int64_t kMaxE = 1024;
constexpr int64_t kMaxL = 1024;
constexpr int64_t kMaxLE = int64_t(1) << 20;
constexpr int64_t kMaxRank = 128;
constexpr int64_t kInt32Max = 2147483647;

bool block_m_ok(int64_t b) { return b == 16 || b == 32 || b == 64 || b == 128; }
bool naive_block_m_ok(int64_t b) { return b >= 1 && b <= 128 && (b & (b - 1)) == 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared size checks of the calls.  On success fills numel and cap.
// `naive`: the block sizes of the align-free path.
int check_sizes(int64_t M, int64_t topk, int64_t E, int64_t L, int64_t block_m,
                int64_t* numel_out, int64_t* cap_out, bool naive = false) {
  if (M < 0 || topk < 1 || E < 1 || L < 1) return MOE_LORA_ERR_INVALID;
  if (E > kMaxE || L > kMaxL || L * E > kMaxLE ||
      !(naive ? naive_block_m_ok(block_m) : block_m_ok(block_m)))
    return MOE_LORA_ERR_UNSUPPORTED;
  if (topk > kInt32Max || M > kInt32Max / topk) return MOE_LORA_ERR_UNSUPPORTED;
  const int64_t numel = M * topk;
  const int64_t groups = std::min(E, numel);
  const int64_t bound = numel + groups * (block_m - 1);
  const int64_t cap = (bound + block_m - 1) / block_m * block_m;
  if (bound + block_m >= kInt32Max || L * cap >= kInt32Max) return MOE_LORA_ERR_UNSUPPORTED;
  *numel_out = numel;
  *cap_out = cap;
  return MOE_LORA_OK;
}

// Whether the MFMA kernel can take these sizes (rank, block size and the
// byte ranges its buffer resources address).
bool mfma_ok(int64_t M, int64_t numel, int64_t K, int64_t Ns, int64_t N, int r, int block_m,
             int x_per_pair) {
  const int64_t x_bytes = (x_per_pair ? numel : M) * K * 2;
  return mfma_supported(r, block_m) && mfma_fits(x_bytes, numel * N * 2, r, K, Ns);
}

// The kernel that runs; the sizes have been checked.
int pick_variant(int64_t M, int64_t numel, int64_t K, int64_t Ns, int64_t N, int64_t E, int64_t L,
                 int r, int block_m, int x_per_pair, int variant) {
  if (variant != MOE_LORA_VARIANT_AUTO) return variant;
  // Expected valid rows per (slot, expert) group: below one half, most
  // blocks hold one or two rows and the vector kernel, which streams A and B
  // with no padded rows, is faster; from there on the MFMA kernel is
  // (measured on MI355X: gpt-oss-20b-like w13 at 0.33 rows per group 28 vs
  // 33 us, at 1.3 rows per group 82 vs 60 us).  Rank 16 runs the 512-thread
  // vector kernel, faster up to and including two rows per group
  // (gpt-oss-120b-like w13 at 0.5 / 1 / 2 rows per group 23.2 / 45.1 / 54.2 us
  // against MFMA 27.7 / 48.1 / 54.7; w2 at 1 row 22.5 against 27.7).
  const bool rows = r == 16 ? numel > 2 * L * E : 2 * numel >= L * E;
  const bool mfma = mfma_ok(M, numel, K, Ns, N, r, block_m, x_per_pair) && rows;
  return mfma ? MOE_LORA_VARIANT_MFMA : MOE_LORA_VARIANT_VALU;
}

int nbits_for(int64_t keys) {
  int n = 0;
  while ((int64_t(1) << n) < keys) ++n;
  return n;
}

}  // namespace

namespace mlr {

// The device's compute units over its XCDs; each device is queried once.  Two
// threads that race on the first call store the same value.
int xcd_compute_units() {
  constexpr int kMaxDevices = 64;
  static int cache[kMaxDevices] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices && cache[dev] > 0) return cache[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  const int per = cus / kXcds;
  if (dev < kMaxDevices) cache[dev] = per;
  return per;
}

}  // namespace mlr

extern "C" {

const char* moe_lora_status_string(int status) {
  switch (status) {
    case MOE_LORA_OK: return "ok";
    case MOE_LORA_ERR_INVALID: return "invalid argument";
    case MOE_LORA_ERR_UNSUPPORTED: return "unsupported size or option";
    case MOE_LORA_ERR_WORKSPACE: return "workspace too small";
    case MOE_LORA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int64_t moe_lora_align_capacity(int64_t M, int32_t topk, int32_t E, int32_t block_m) {
  int64_t numel, cap;
  const int rc = check_sizes(M, topk, E, 1, block_m, &numel, &cap);
  return rc != MOE_LORA_OK ? rc : cap;
}

int64_t moe_lora_align_workspace_size(int64_t M, int32_t topk, int32_t E, int32_t L,
                                       int32_t block_m) {
  int64_t numel, cap;
  const int rc = check_sizes(M, topk, E, L, block_m, &numel, &cap);
  if (rc != MOE_LORA_OK) return rc;
  return plan_align(numel, E, L, block_m).ws_bytes;
}

}  // extern "C"

// The align call with its workspace (null when `ws_bytes` is 0): checks,
// plan, launch.
static int align_call(const int32_t* topk_ids, const int32_t* token_lora_mapping, int64_t M,
                      int32_t topk, int32_t E, int32_t L, int32_t block_m,
                      int32_t* sorted_token_ids, int32_t* expert_ids,
                      int32_t* num_tokens_post_padded, int32_t* lora_ids,
                      int32_t* num_active_loras, void* workspace, int64_t workspace_bytes,
                      void* stream) {
  int64_t numel, cap;
  const int rc = check_sizes(M, topk, E, L, block_m, &numel, &cap);
  if (rc != MOE_LORA_OK) return rc;
  // arrays of zero size (everything but num_tokens_post_padded when M == 0)
  // may be null
  if (!num_tokens_post_padded || workspace_bytes < 0) return MOE_LORA_ERR_INVALID;
  if (numel > 0 && (!topk_ids || !token_lora_mapping || !sorted_token_ids || !expert_ids))
    return MOE_LORA_ERR_INVALID;
  // numel == 0 still launches: every slot's metadata is written (all empty)
  const AlignPlan plan = plan_align(numel, E, L, block_m);
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return MOE_LORA_ERR_WORKSPACE;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const bool passes = plan.pass_slots < L;  // slot ranges, one pass each
  for (int32_t l0 = 0; l0 < L; l0 += plan.pass_slots) {
    const int32_t Lp = std::min<int32_t>(plan.pass_slots, L - l0);
    AlignParams a{};
    a.topk_ids = topk_ids;
    a.mapping = token_lora_mapping;
    a.l0 = l0;
    a.sorted = sorted_token_ids ? sorted_token_ids + int64_t(l0) * cap : nullptr;
    a.eids = expert_ids ? expert_ids + int64_t(l0) * (cap / block_m) : nullptr;
    a.ntpp = num_tokens_post_padded + l0;
    a.lora_ids = passes ? nullptr : lora_ids;
    a.nact = passes ? nullptr : num_active_loras;
    a.numel = int32_t(numel);
    a.topk = topk;
    a.E = E;
    a.L = Lp;
    a.LE = Lp * E;
    a.B = block_m;
    a.nbits = nbits_for(int64_t(Lp) * E);
    a.cap = int32_t(cap);
    a.nb = int32_t(cap / block_m);
    a.W = plan.W;
    a.seg = plan.seg;
    a.ntiles = plan.ntiles;
    if (!plan.single && !plan.wave) {
      int32_t* ws = static_cast<int32_t*>(workspace);
      a.tile_cnt = ws;
      a.key_tot = ws + int64_t(plan.ntiles) * a.LE;
    }
    if (launch_align(plan, a, st) != hipSuccess) return MOE_LORA_ERR_HIP;
  }
  if (passes && (lora_ids || num_active_loras) &&
      launch_align_active(num_tokens_post_padded, L, lora_ids, num_active_loras, st) != hipSuccess)
    return MOE_LORA_ERR_HIP;
  return MOE_LORA_OK;
}

extern "C" {

int moe_lora_align(const int32_t* topk_ids, const int32_t* token_lora_mapping, int64_t M,
                   int32_t topk, int32_t E, int32_t L, int32_t block_m,
                   int32_t* sorted_token_ids, int32_t* expert_ids,
                   int32_t* num_tokens_post_padded, int32_t* lora_ids,
                   int32_t* num_active_loras, void* workspace, int64_t workspace_bytes,
                   void* stream) {
  return align_call(topk_ids, token_lora_mapping, M, topk, E, L, block_m, sorted_token_ids,
                    expert_ids, num_tokens_post_padded, lora_ids, num_active_loras, workspace,
                    workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- no-allocation align
// The scratch of moe_lora_align_noalloc: one copy per GPU, alive until the
// process ends.  Host code never passes this name to a kernel (on the host it
// is only a stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) int32_t scratch[MOE_LORA_ALIGN_NOALLOC_SCRATCH_BYTES / 4];

namespace {

constexpr int kMaxScratchDevices = 64;
void* g_scratch_ptr[kMaxScratchDevices] = {nullptr};

// The current device's scratch address, looked up once per device (with that
// device current).  Two threads that race on the first call store the same
// address.  Null when the lookup fails.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  if (g_scratch_ptr[dev]) return g_scratch_ptr[dev];
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  g_scratch_ptr[dev] = ptr;
  return ptr;
}

}  // namespace

extern "C" {

int moe_lora_align_noalloc(const int32_t* topk_ids, const int32_t* token_lora_mapping, int64_t M,
                           int32_t topk, int32_t E, int32_t L, int32_t block_m,
                           int32_t* sorted_token_ids, int32_t* expert_ids,
                           int32_t* num_tokens_post_padded, int32_t* lora_ids,
                           int32_t* num_active_loras, void* stream) {
  // sizes first: a rejected call makes no HIP call at all
  int64_t numel, cap;
  const int rc = check_sizes(M, topk, E, L, block_m, &numel, &cap);
  if (rc != MOE_LORA_OK) return rc;
  const int64_t need = plan_align(numel, E, L, block_m).ws_bytes;
  if (need > MOE_LORA_ALIGN_NOALLOC_SCRATCH_BYTES) return MOE_LORA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_address();
    if (!ws) return MOE_LORA_ERR_HIP;
  }
  return align_call(topk_ids, token_lora_mapping, M, topk, E, L, block_m, sorted_token_ids,
                    expert_ids, num_tokens_post_padded, lora_ids, num_active_loras, ws,
                    need > 0 ? MOE_LORA_ALIGN_NOALLOC_SCRATCH_BYTES : 0, stream);
}

// The K-split exchange area the sorted-path call needs (0: its kernel has no
// use for one), or a negative status for sizes the call would reject.
static int64_t fused_exchange_bytes(int64_t M, int32_t topk, int32_t K, int32_t Ns, int32_t S,
                                    int32_t E, int32_t L, int32_t r, int32_t block_m,
                                    int32_t x_per_pair, int32_t variant) {
  const int v = fused_moe_lora_variant(M, topk, K, Ns, S, E, L, r, block_m, x_per_pair, variant);
  if (v < 0) return v;
  const int64_t numel = M * topk, N = int64_t(S) * Ns;
  if (v == MOE_LORA_VARIANT_MFMA || numel == 0 || !valu_takes_stream(M, numel, K, N, r, x_per_pair))
    return 0;
  const int64_t units = max_total_blocks(numel, int64_t(L) * E, block_m) * S;
  return xch_area_bytes(units * exchange_passes(block_m));
}

static int fused_sorted(const uint16_t* x, int32_t x_per_pair, const uint16_t* lora_a,
                        const uint16_t* lora_b, const int32_t* sorted_token_ids,
                        const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                        int32_t max_active_loras,
                        const float* topk_weights, int32_t mul_routed_weight, int32_t add_inputs,
                        int64_t M, int32_t topk, int32_t K, int32_t Ns, int32_t S, int32_t E,
                        int32_t L, int32_t r, int32_t block_m, uint16_t* y, int32_t variant,
                        int32_t* xch, int64_t xch_bytes, int32_t peer_wait, void* stream) {
  int64_t numel, cap;
  const int rc = check_sizes(M, topk, E, L, block_m, &numel, &cap);
  if (rc != MOE_LORA_OK) return rc;
  if (K < 8 || Ns < 8 || S < 1 || r < 1 || (K & 7) || (Ns & 7)) return MOE_LORA_ERR_INVALID;
  if ((x_per_pair != 0 && x_per_pair != 1) || (mul_routed_weight != 0 && mul_routed_weight != 1) ||
      (add_inputs != 0 && add_inputs != 1) || variant < 0 || variant > 2)
    return MOE_LORA_ERR_INVALID;
  if (r > kMaxRank) return MOE_LORA_ERR_UNSUPPORTED;
  const int64_t N = int64_t(S) * Ns;
  if (N > kInt32Max || numel * N / N != numel) return MOE_LORA_ERR_UNSUPPORTED;
  if (variant == MOE_LORA_VARIANT_MFMA && !mfma_ok(M, numel, K, Ns, N, r, block_m, x_per_pair))
    return MOE_LORA_ERR_UNSUPPORTED;
  if (max_active_loras < 0 || max_active_loras > L) return MOE_LORA_ERR_INVALID;
  // no pair, or no active slot: nothing is read or written, nothing launched
  if (numel == 0 || max_active_loras == 0) return MOE_LORA_OK;
  if (!x || !lora_a || !lora_b || !sorted_token_ids || !expert_ids ||
      !num_tokens_post_padded || !y || (mul_routed_weight && !topk_weights))
    return MOE_LORA_ERR_INVALID;
  if (!aligned16(x) || !aligned16(lora_a) || !aligned16(lora_b) || !aligned16(y))
    return MOE_LORA_ERR_INVALID;
  // the grid covers the blocks at most max_active_loras slots can hold
  const int64_t gmax = max_total_blocks(numel, int64_t(max_active_loras) * E, block_m);
  const int64_t units = gmax * S;
  if (units * 64 > kInt32Max) return MOE_LORA_ERR_UNSUPPORTED;

  FusedParams p{};
  p.x = x;
  p.a = lora_a;
  p.b = lora_b;
  p.sorted = sorted_token_ids;
  p.eids = expert_ids;
  p.ntpp = num_tokens_post_padded;
  p.w = topk_weights;
  p.y = y;
  p.x_per_pair = x_per_pair;
  p.mul = mul_routed_weight;
  p.add = add_inputs;
  p.numel = int32_t(numel);
  p.topk = topk;
  p.K = K;
  p.Ns = Ns;
  p.S = S;
  p.E = E;
  p.L = L;
  p.r = r;
  p.B = block_m;
  p.N = int32_t(N);
  p.cap = int32_t(cap);
  p.nb = int32_t(cap / block_m);
  p.units = int32_t(units);
  p.xcd_cus = xcd_compute_units();
  p.xch = xch;
  p.xch_nslot = xch ? int32_t(std::min<int64_t>(xch_slots_in(xch_bytes), kInt32Max)) : 0;
  p.xch_passes = int32_t(exchange_passes(block_m));
  p.peer_wait = peer_wait < 0 ? kDefaultPeerWait : peer_wait;

  const bool use_mfma =
      pick_variant(M, numel, K, Ns, N, E, L, r, block_m, x_per_pair, variant) == MOE_LORA_VARIANT_MFMA;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t err = use_mfma ? launch_fused_mfma(p, st) : launch_fused_valu(p, st);
  return err == hipSuccess ? MOE_LORA_OK : MOE_LORA_ERR_HIP;
}

int fused_moe_lora(const uint16_t* x, int32_t x_per_pair, const uint16_t* lora_a,
                   const uint16_t* lora_b, const int32_t* sorted_token_ids,
                   const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                   int32_t max_active_loras, const float* topk_weights,
                   int32_t mul_routed_weight, int32_t add_inputs,
                   int64_t M, int32_t topk, int32_t K, int32_t Ns, int32_t S, int32_t E,
                   int32_t L, int32_t r, int32_t block_m, uint16_t* y, int32_t variant,
                   void* stream) {
  return fused_sorted(x, x_per_pair, lora_a, lora_b, sorted_token_ids, expert_ids,
                      num_tokens_post_padded, max_active_loras, topk_weights, mul_routed_weight,
                      add_inputs, M, topk, K, Ns, S, E, L, r, block_m, y, variant, nullptr, 0, 0,
                      stream);
}

int64_t fused_moe_lora_workspace_bytes(int64_t M, int32_t topk, int32_t K, int32_t Ns, int32_t S,
                                       int32_t E, int32_t L, int32_t r, int32_t block_m,
                                       int32_t x_per_pair, int32_t variant) {
  return fused_exchange_bytes(M, topk, K, Ns, S, E, L, r, block_m, x_per_pair, variant);
}

int fused_moe_lora_ws(const uint16_t* x, int32_t x_per_pair, const uint16_t* lora_a,
                      const uint16_t* lora_b, const int32_t* sorted_token_ids,
                      const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                      int32_t max_active_loras, const float* topk_weights,
                      int32_t mul_routed_weight, int32_t add_inputs,
                      int64_t M, int32_t topk, int32_t K, int32_t Ns, int32_t S, int32_t E,
                      int32_t L, int32_t r, int32_t block_m, uint16_t* y, int32_t variant,
                      void* workspace, int64_t workspace_bytes, int32_t peer_wait, void* stream) {
  const int64_t need = fused_exchange_bytes(M, topk, K, Ns, S, E, L, r, block_m, x_per_pair, variant);
  if (need < 0) return int(need);
  if (workspace_bytes < 0) return MOE_LORA_ERR_INVALID;
  // max_active_loras == 0 launches nothing (fused_sorted), so no area is needed
  if (need > 0 && max_active_loras != 0 &&
      (!workspace || !aligned16(workspace) || workspace_bytes < need))
    return MOE_LORA_ERR_WORKSPACE;
  return fused_sorted(x, x_per_pair, lora_a, lora_b, sorted_token_ids, expert_ids,
                      num_tokens_post_padded, max_active_loras, topk_weights, mul_routed_weight,
                      add_inputs, M, topk, K, Ns, S, E, L, r, block_m, y, variant,
                      need > 0 ? static_cast<int32_t*>(workspace) : nullptr, workspace_bytes,
                      peer_wait, stream);
}

static_assert(kAlignWaveMaxPairs == MOE_LORA_WITH_ALIGN_MAX_PAIRS &&
                  kAlignWaveMaxSlots == MOE_LORA_WITH_ALIGN_MAX_SLOTS,
              "the header's limits are the one-wavefront align's");

// The align-free launch shared by fused_moe_lora_naive and
// fused_moe_lora_with_align (al: the align outputs one workgroup writes,
// or null); sizes and pointers of the fused part are checked here.
static int naive_launch(const uint16_t* x, int32_t x_per_pair, const uint16_t* lora_a,
                        const uint16_t* lora_b, const int32_t* topk_ids,
                        const int32_t* token_lora_mapping, const float* topk_weights,
                        int32_t mul_routed_weight, int32_t add_inputs, int64_t M, int32_t topk,
                        int32_t K, int32_t Ns, int32_t S, int32_t E, int32_t L, int32_t r,
                        int32_t block_m, uint16_t* y, int32_t variant, const AlignParams* al,
                        void* stream) {
  int64_t numel, cap;
  const int rc = check_sizes(M, topk, E, L, block_m, &numel, &cap, true);
  if (rc != MOE_LORA_OK) return rc;
  if (K < 8 || Ns < 8 || S < 1 || r < 1 || (K & 7) || (Ns & 7)) return MOE_LORA_ERR_INVALID;
  if ((x_per_pair != 0 && x_per_pair != 1) || (mul_routed_weight != 0 && mul_routed_weight != 1) ||
      (add_inputs != 0 && add_inputs != 1) || variant < 0 || variant > 2)
    return MOE_LORA_ERR_INVALID;
  if (r > kMaxRank || numel > kNaiveMaxPairs) return MOE_LORA_ERR_UNSUPPORTED;
  const int64_t N = int64_t(S) * Ns;
  if (N > kInt32Max || numel * N / N != numel) return MOE_LORA_ERR_UNSUPPORTED;
  if (variant == MOE_LORA_VARIANT_MFMA && !mfma_ok(M, numel, K, Ns, N, r, block_m, x_per_pair))
    return MOE_LORA_ERR_UNSUPPORTED;
  if (numel == 0) return MOE_LORA_OK;  // no pair: nothing is read or written
  if (!x || !lora_a || !lora_b || !topk_ids || !token_lora_mapping || !y ||
      (mul_routed_weight && !topk_weights))
    return MOE_LORA_ERR_INVALID;
  if (!aligned16(x) || !aligned16(lora_a) || !aligned16(lora_b) || !aligned16(y))
    return MOE_LORA_ERR_INVALID;
  const int64_t units = max_total_blocks(numel, int64_t(L) * E, block_m) * S;
  if (units * 64 > kInt32Max) return MOE_LORA_ERR_UNSUPPORTED;

  FusedParams p{};
  p.x = x;
  p.a = lora_a;
  p.b = lora_b;
  p.topk_ids = topk_ids;
  p.mapping = token_lora_mapping;
  p.w = topk_weights;
  p.y = y;
  p.x_per_pair = x_per_pair;
  p.mul = mul_routed_weight;
  p.add = add_inputs;
  p.numel = int32_t(numel);
  p.topk = topk;
  p.K = K;
  p.Ns = Ns;
  p.S = S;
  p.E = E;
  p.L = L;
  p.r = r;
  p.B = block_m;
  p.N = int32_t(N);
  p.units = int32_t(units);
  p.xcd_cus = xcd_compute_units();
  p.naive = 1;
  p.nbits = nbits_for(int64_t(L) * E);
  if (al) {
    p.al_sorted = al->sorted;
    p.al_eids = al->eids;
    p.al_ntpp = al->ntpp;
    p.al_lora_ids = al->lora_ids;
    p.al_nact = al->nact;
    p.cap = al->cap;
    p.nb = al->nb;
  }
  const bool use_mfma =
      pick_variant(M, numel, K, Ns, N, E, L, r, block_m, x_per_pair, variant) == MOE_LORA_VARIANT_MFMA;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t err = use_mfma ? launch_fused_mfma(p, st) : launch_fused_valu(p, st);
  return err == hipSuccess ? MOE_LORA_OK : MOE_LORA_ERR_HIP;
}

int fused_moe_lora_naive(const uint16_t* x, int32_t x_per_pair, const uint16_t* lora_a,
                         const uint16_t* lora_b, const int32_t* topk_ids,
                         const int32_t* token_lora_mapping, const float* topk_weights,
                         int32_t mul_routed_weight, int32_t add_inputs, int64_t M, int32_t topk,
                         int32_t K, int32_t Ns, int32_t S, int32_t E, int32_t L, int32_t r,
                         int32_t block_m, uint16_t* y, int32_t variant, void* stream) {
  return naive_launch(x, x_per_pair, lora_a, lora_b, topk_ids, token_lora_mapping, topk_weights,
                      mul_routed_weight, add_inputs, M, topk, K, Ns, S, E, L, r, block_m, y,
                      variant, nullptr, stream);
}

int fused_moe_lora_with_align(const int32_t* topk_ids, const int32_t* token_lora_mapping,
                              int64_t M, int32_t topk, int32_t E, int32_t L, int32_t block_m,
                              int32_t* sorted_token_ids, int32_t* expert_ids,
                              int32_t* num_tokens_post_padded, int32_t* lora_ids,
                              int32_t* num_active_loras, const uint16_t* x, int32_t x_per_pair,
                              const uint16_t* lora_a, const uint16_t* lora_b,
                              const float* topk_weights, int32_t mul_routed_weight,
                              int32_t add_inputs, int32_t K, int32_t Ns, int32_t S, int32_t r,
                              uint16_t* y, int32_t variant, void* stream) {
  // the align step's own rules (block_m as moe_lora_align takes it), then the
  // one-wavefront limits of the align that rides along
  int64_t numel, cap;
  const int rc = check_sizes(M, topk, E, L, block_m, &numel, &cap);
  if (rc != MOE_LORA_OK) return rc;
  if (numel > kAlignWaveMaxPairs || L > kAlignWaveMaxSlots) return MOE_LORA_ERR_UNSUPPORTED;
  if (!num_tokens_post_padded) return MOE_LORA_ERR_INVALID;
  if (numel > 0 && (!sorted_token_ids || !expert_ids)) return MOE_LORA_ERR_INVALID;
  // the fused part's checks, without a launch (the pointers too)
  const int vrc = fused_moe_lora_variant(M, topk, K, Ns, S, E, L, r, block_m, x_per_pair, variant);
  if (vrc < 0) return vrc;
  if ((mul_routed_weight != 0 && mul_routed_weight != 1) || (add_inputs != 0 && add_inputs != 1))
    return MOE_LORA_ERR_INVALID;
  if (numel == 0)  // no fused work: the align alone writes the (empty) outputs
    return moe_lora_align(topk_ids, token_lora_mapping, M, topk, E, L, block_m, sorted_token_ids,
                          expert_ids, num_tokens_post_padded, lora_ids, num_active_loras, nullptr,
                          0, stream);
  AlignParams al{};
  al.sorted = sorted_token_ids;
  al.eids = expert_ids;
  al.ntpp = num_tokens_post_padded;
  al.lora_ids = lora_ids;
  al.nact = num_active_loras;
  al.cap = int32_t(cap);
  al.nb = int32_t(cap / block_m);
  return naive_launch(x, x_per_pair, lora_a, lora_b, topk_ids, token_lora_mapping, topk_weights,
                      mul_routed_weight, add_inputs, M, topk, K, Ns, S, E, L, r, block_m, y,
                      variant, &al, stream);
}

}  // extern "C"

namespace {

// Checks of the two-kernel call; fills the launch plan (kz, kchunk, units,
// workspace bytes).  Returns a status.
struct TwoPlan {
  int64_t numel, cap, N, units, ws_bytes;
  int kz, kchunk;
};

int plan_two_kernel(int64_t M, int32_t topk, int32_t K, int32_t Ns, int32_t S, int32_t E,
                    int32_t L, int32_t r, int32_t block_m, int32_t x_per_pair, TwoPlan* t) {
  const int rc = check_sizes(M, topk, E, L, block_m, &t->numel, &t->cap);
  if (rc != MOE_LORA_OK) return rc;
  if (K < 8 || Ns < 8 || S < 1 || r < 1 || (K & 7) || (Ns & 7)) return MOE_LORA_ERR_INVALID;
  if (x_per_pair != 0 && x_per_pair != 1) return MOE_LORA_ERR_INVALID;
  if (r > kMaxRankTwoKernel) return MOE_LORA_ERR_UNSUPPORTED;
  t->N = int64_t(S) * Ns;
  if (t->N > kInt32Max || t->numel * t->N / t->N != t->numel) return MOE_LORA_ERR_UNSUPPORTED;
  const int64_t x_bytes = (x_per_pair ? t->numel : M) * K * 2;
  if (!two_kernel_fits(x_bytes, r, K, Ns)) return MOE_LORA_ERR_UNSUPPORTED;
  t->units = max_total_blocks(t->numel, int64_t(L) * E, block_m) * S;
  t->kz = two_kernel_splits(t->units, K, r);
  const int64_t per = (K + t->kz - 1) / t->kz;
  t->kchunk = int((per + 31) / 32 * 32);
  const int64_t groups = (r + kTwoKernelRankGroup - 1) / kTwoKernelRankGroup;
  if (t->units * groups * t->kz * 64 > kInt32Max) return MOE_LORA_ERR_UNSUPPORTED;
  t->ws_bytes = int64_t(t->kz) * S * t->numel * r * 4;
  return MOE_LORA_OK;
}

}  // namespace

extern "C" {

int64_t fused_moe_lora_two_kernel_workspace_bytes(int64_t M, int32_t topk, int32_t K, int32_t Ns,
                                                  int32_t S, int32_t E, int32_t L, int32_t r,
                                                  int32_t block_m, int32_t x_per_pair) {
  TwoPlan t;
  const int rc = plan_two_kernel(M, topk, K, Ns, S, E, L, r, block_m, x_per_pair, &t);
  return rc != MOE_LORA_OK ? rc : t.ws_bytes;
}

int fused_moe_lora_two_kernel(const uint16_t* x, int32_t x_per_pair, const uint16_t* lora_a,
                              const uint16_t* lora_b, const int32_t* sorted_token_ids,
                              const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                              int32_t max_active_loras, const float* topk_weights,
                              int32_t mul_routed_weight,
                              int32_t add_inputs, int64_t M, int32_t topk, int32_t K, int32_t Ns,
                              int32_t S, int32_t E, int32_t L, int32_t r, int32_t block_m,
                              uint16_t* y, void* workspace, int64_t workspace_bytes,
                              void* stream) {
  TwoPlan t;
  const int rc = plan_two_kernel(M, topk, K, Ns, S, E, L, r, block_m, x_per_pair, &t);
  if (rc != MOE_LORA_OK) return rc;
  if ((mul_routed_weight != 0 && mul_routed_weight != 1) || (add_inputs != 0 && add_inputs != 1) ||
      workspace_bytes < 0 || max_active_loras < 0 || max_active_loras > L)
    return MOE_LORA_ERR_INVALID;
  // no pair, or no active slot: nothing is read or written, nothing launched
  if (t.numel == 0 || max_active_loras == 0) return MOE_LORA_OK;
  if (!x || !lora_a || !lora_b || !sorted_token_ids || !expert_ids ||
      !num_tokens_post_padded || !y || (mul_routed_weight && !topk_weights))
    return MOE_LORA_ERR_INVALID;
  if (!aligned16(x) || !aligned16(lora_a) || !aligned16(lora_b) || !aligned16(y))
    return MOE_LORA_ERR_INVALID;
  if (!workspace || workspace_bytes < t.ws_bytes || !aligned16(workspace))
    return MOE_LORA_ERR_WORKSPACE;

  FusedParams p{};
  p.x = x;
  p.a = lora_a;
  p.b = lora_b;
  p.sorted = sorted_token_ids;
  p.eids = expert_ids;
  p.ntpp = num_tokens_post_padded;
  p.w = topk_weights;
  p.y = y;
  p.x_per_pair = x_per_pair;
  p.mul = mul_routed_weight;
  p.add = add_inputs;
  p.numel = int32_t(t.numel);
  p.topk = topk;
  p.K = K;
  p.Ns = Ns;
  p.S = S;
  p.E = E;
  p.L = L;
  p.r = r;
  p.B = block_m;
  p.N = int32_t(t.N);
  p.cap = int32_t(t.cap);
  p.nb = int32_t(t.cap / block_m);
  // the grid covers the blocks at most max_active_loras slots can hold
  p.units = int32_t(max_total_blocks(t.numel, int64_t(max_active_loras) * E, block_m) * S);
  p.xcd_cus = xcd_compute_units();
  p.ws = static_cast<float*>(workspace);
  p.kz = t.kz;
  p.kchunk = t.kchunk;
  const hipError_t err = launch_two_kernel(p, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? MOE_LORA_OK : MOE_LORA_ERR_HIP;
}

int moe_lora_accumulate(uint16_t* y, const uint16_t* delta, int64_t n, void* stream) {
  if (n < 0) return MOE_LORA_ERR_INVALID;
  if (n == 0) return MOE_LORA_OK;
  if (!y || !delta || !aligned16(y) || !aligned16(delta)) return MOE_LORA_ERR_INVALID;
  const hipError_t err = launch_accumulate(y, delta, n, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? MOE_LORA_OK : MOE_LORA_ERR_HIP;
}

int fused_moe_lora_variant(int64_t M, int32_t topk, int32_t K, int32_t Ns, int32_t S, int32_t E,
                           int32_t L, int32_t r, int32_t block_m, int32_t x_per_pair,
                           int32_t variant) {
  int64_t numel, cap;
  const int rc = check_sizes(M, topk, E, L, block_m, &numel, &cap);
  if (rc != MOE_LORA_OK) return rc;
  if (K < 8 || Ns < 8 || S < 1 || r < 1 || (K & 7) || (Ns & 7)) return MOE_LORA_ERR_INVALID;
  const int64_t N = int64_t(S) * Ns;
  if (N > kInt32Max || numel * N / N != numel) return MOE_LORA_ERR_UNSUPPORTED;
  if ((x_per_pair != 0 && x_per_pair != 1) || variant < 0 || variant > 2) return MOE_LORA_ERR_INVALID;
  if (r > kMaxRank) return MOE_LORA_ERR_UNSUPPORTED;
  if (variant == MOE_LORA_VARIANT_MFMA && !mfma_ok(M, numel, K, Ns, N, r, block_m, x_per_pair))
    return MOE_LORA_ERR_UNSUPPORTED;
  return pick_variant(M, numel, K, Ns, N, E, L, r, block_m, x_per_pair, variant);
}

const char* fused_moe_lora_kernel_name(int64_t M, int32_t topk, int32_t K, int32_t Ns, int32_t S,
                                       int32_t E, int32_t L, int32_t r, int32_t block_m,
                                       int32_t x_per_pair, int32_t variant) {
  const int v = fused_moe_lora_variant(M, topk, K, Ns, S, E, L, r, block_m, x_per_pair, variant);
  if (v < 0) return nullptr;
  if (v == MOE_LORA_VARIANT_MFMA) return "fused_mfma_kernel";
  const int64_t numel = M * topk, N = int64_t(S) * Ns;
  return valu_takes_stream(M, numel, K, N, r, x_per_pair) ? "fused_stream_kernel"
                                                          : "fused_valu_kernel";
}

}  // extern "C"
