/*
 * moe_lora.h -- C ABI of the MI355X (gfx950) MoE-LoRA hot path.
 *
 * Two operations, both hand-written HIP kernels:
 *
 *   moe_lora_align  -- per LoRA slot, group the routed (token, k) pairs by
 *                      expert and pad every group to block_m (vLLM PR #29257
 *                      "Lora MoE Align Improvements", Purpose).
 *   fused_moe_lora  -- Y[m,k,:] (+)= (X[m] A[s,l,e]^T) B[s,l,e]^T per slice s,
 *                      with l = token_lora_mapping[m], e = topk_ids[m,k], the
 *                      rank-r vector kept on chip, optional routed weight
 *                      (prhub summary of vLLM PR #42290, implementation
 *                      steps and key source fragment).
 *
 * Conventions for every call below:
 *   - Pointers marked [device] are device (HBM) addresses; the caller owns
 *     and allocates every buffer.  The library allocates no memory, keeps no
 *     pointer after a call returns, and never synchronises.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     on it asynchronously; results are visible to later work on that stream.
 *   - All index arrays are int32 (a type mismatch on token_lora_mapping was
 *     flagged as undefined behaviour in the review of PR #29257).
 *   - Arguments are validated on the host before any HIP call.  A negative
 *     status means nothing was launched and no output was written.
 *   - M = 0 is valid: moe_lora_align still writes every slot's metadata
 *     (all slots empty), fused_moe_lora returns MOE_LORA_OK at once.  Arrays
 *     of zero size may then be NULL.
 *   - Calls on different streams may overlap if their outputs are disjoint.
 *
 * Limits: 1 <= E <= 1024 (the expert limit asked for in the review of PR
 * #29257), 1 <= L <= 1024 (so L*E <= 2^20), block_m in {16, 32, 64, 128},
 * 1 <= r <= 128 (the one-shot kernel's compile-time rank bound in the prhub
 * summary of PR #42290, here an error code instead of an assert),
 * M*topk + min(E, M*topk)*(block_m-1) < 2^31 and L * capacity < 2^31.
 */
#ifndef MOE_LORA_H
#define MOE_LORA_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_LORA_API __attribute__((visibility("default")))
#else
#define MOE_LORA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum moe_lora_status {
    MOE_LORA_OK = 0,
    MOE_LORA_ERR_INVALID = -1,     /* null pointer, negative size, bad flag,
                                      misaligned pointer, K or Ns not % 8   */
    MOE_LORA_ERR_UNSUPPORTED = -2, /* outside the limits listed above       */
    MOE_LORA_ERR_WORKSPACE = -3,   /* align workspace smaller than needed   */
    MOE_LORA_ERR_HIP = -4          /* a HIP launch or query failed          */
};

/* Human-readable name of a status code (static string, never NULL). */
MOE_LORA_API const char *moe_lora_status_string(int status);

/*
 * Row length `cap` of each slot in sorted_token_ids:
 *     round_up(numel + min(E, numel) * (block_m - 1), block_m),
 * numel = M * topk.  No slot can need more: each non-empty expert group adds
 * at most block_m - 1 padding entries.  expert_ids rows hold cap / block_m
 * entries.  Returns a negative status for invalid sizes.  Host only.
 */
MOE_LORA_API int64_t moe_lora_align_capacity(int64_t M, int32_t topk, int32_t E, int32_t block_m);

/*
 * Bytes of device workspace moe_lora_align needs for these sizes (0 when
 * the single-workgroup path is taken).  Returns a negative status for
 * invalid sizes.  Host only.
 */
MOE_LORA_API int64_t moe_lora_align_workspace_size(int64_t M, int32_t topk, int32_t E,
                                       int32_t L, int32_t block_m);

/*
 * moe_lora_align -- the align step (vLLM PR #29257, Purpose: an LDS variant
 * for few experts and a global-memory variant for many; one routine serves
 * the LoRA case and, with L = 1 and a zero mapping, the plain MoE case).
 *
 * Inputs  [device]:
 *   topk_ids            int32 [M, topk]   expert of pair p = m*topk + k
 *   token_lora_mapping  int32 [M]         slot of token m; -1 = no adapter
 * Outputs [device]:
 *   sorted_token_ids    int32 [L, cap]    slot l's row: for each expert e in
 *                       ascending order, the pairs p with (l, e) in ascending
 *                       p, then the sentinel numel = M*topk up to a multiple
 *                       of block_m.  Entries from num_tokens_post_padded[l]
 *                       to cap are not written.
 *   expert_ids          int32 [L, cap/block_m]  expert of each block of
 *                       block_m entries in that row (entries past the slot's
 *                       blocks are not written).
 *   num_tokens_post_padded int32 [L]      padded length of each slot's row.
 *   lora_ids            int32 [L] or NULL the slots with at least one pair,
 *                       ascending, then -1 (the active-slot list of vLLM PR
 *                       #32005).
 *   num_active_loras    int32 [1] or NULL how many slots are active.
 *   workspace           [device] scratch of moe_lora_align_workspace_size()
 *                       bytes (may be NULL when that is 0); contents on entry
 *                       do not matter.
 * Pairs whose slot is outside [0, L) (including -1) or whose expert is
 * outside [0, E) are skipped; nothing traps on device.  The result does not
 * depend on thread timing: the same inputs give the same bytes.  When L*E is
 * above 8192 (slot, expert) keys (and the call is not a one-wavefront one of
 * at most 64 pairs and 64 slots), the work runs as several launches over
 * ranges of 8192/E slots, each reading every pair, then one that lists the
 * active slots; the workspace is sized for one range.
 */
MOE_LORA_API int moe_lora_align(const int32_t *topk_ids, const int32_t *token_lora_mapping,
                   int64_t M, int32_t topk, int32_t E, int32_t L,
                   int32_t block_m, int32_t *sorted_token_ids,
                   int32_t *expert_ids, int32_t *num_tokens_post_padded,
                   int32_t *lora_ids, int32_t *num_active_loras,
                   void *workspace, int64_t workspace_bytes, void *stream);

/* Bytes of the device scratch moe_lora_align_noalloc owns on each GPU. */
#define MOE_LORA_ALIGN_NOALLOC_SCRATCH_BYTES (8 * 1024 * 1024)

/*
 * moe_lora_align_noalloc -- moe_lora_align for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same arguments
 * without the workspace, the same outputs bit for bit.  The scratch the
 * multi-workgroup path needs (per-tile key counts and per-key totals) lives
 * in a static device array of MOE_LORA_ALIGN_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it has run on until the process ends; its
 * address is looked up once per device.  The call allocates nothing.
 *   - Every call on one GPU shares that array: calls that may overlap on one
 *     GPU (other streams, other threads) race and must not be issued.
 *     Calls in stream order are fine; nothing in the array needs clearing
 *     (its contents on entry do not matter).
 *   - MOE_LORA_ERR_WORKSPACE (nothing launched) when the sizes need more
 *     scratch than that (moe_lora_align_workspace_size() above the limit;
 *     no size the limits of this header allow does today).
 *   - MOE_LORA_ERR_HIP when the scratch's address cannot be found.
 * Other arguments, statuses and outputs as moe_lora_align.
 */
MOE_LORA_API int moe_lora_align_noalloc(const int32_t *topk_ids,
                   const int32_t *token_lora_mapping, int64_t M, int32_t topk,
                   int32_t E, int32_t L, int32_t block_m, int32_t *sorted_token_ids,
                   int32_t *expert_ids, int32_t *num_tokens_post_padded,
                   int32_t *lora_ids, int32_t *num_active_loras, void *stream);

/* Kernel choice for fused_moe_lora. */
enum moe_lora_variant {
    MOE_LORA_VARIANT_AUTO = 0, /* chosen from the expected rows per block */
    MOE_LORA_VARIANT_VALU = 1, /* vector loads + wavefront reductions     */
    MOE_LORA_VARIANT_MFMA = 2  /* LDS-staged bf16 MFMA tiles              */
};

/*
 * fused_moe_lora -- shrink and expand in one kernel, the rank-r vector
 * never leaving the chip (prhub summary of vLLM PR #42290; slices and the
 * routed weight as in the fused_moe_lora signature of the PR #32005 diff).
 *
 * For every valid pair p = m*topk + k in the align outputs, with its slot l
 * (the row of sorted_token_ids it sits in) and expert e (its block's
 * expert_ids entry), and every slice s < S:
 *     v[j] = sum_t X[row, t] * A[s,l,e,j,t]      row = p if x_per_pair else m
 *     d[n] = sum_j v[j] * B[s,l,e,n,j]           (fp32 accumulation)
 *     d[n] *= topk_weights[p]                    if mul_routed_weight
 *     Y[p, s*Ns+n] = bf16(add_inputs ? Y[p, s*Ns+n] + d[n] : d[n])  (RNE)
 * Rows of pairs that are in no slot are not touched.
 *
 * Inputs  [device]:
 *   x          bf16 [M, K], or [M*topk, K] when x_per_pair (w2-style input)
 *   lora_a     bf16 [S, L, E, r, K]
 *   lora_b     bf16 [S, L, E, Ns, r]
 *   sorted_token_ids, expert_ids, num_tokens_post_padded: as produced by
 *              moe_lora_align for the same M, topk, E, L, block_m.
 * [host] max_active_loras: at most this many slots have a non-empty row (the
 *              pages' max_loras grid bound, vLLM PR #32005 diff; pass L when
 *              unknown).  0 returns MOE_LORA_OK with nothing launched or read
 *              (the no-LoRA batch, the pages' no_lora_flag); otherwise the
 *              launch covers the blocks that many slots can hold.  With more
 *              slots active than promised, blocks past that bound are not
 *              computed.  MOE_LORA_ERR_INVALID outside [0, L].  (The kernels
 *              find the active slots from num_tokens_post_padded on the
 *              device, so the lora_ids list is not an argument.)
 *   topk_weights fp32 [M, topk]; may be NULL when mul_routed_weight == 0.
 * In/out [device]:
 *   y          bf16 [M, topk, S*Ns]
 * x, lora_a, lora_b and y must be 16-byte aligned; K and Ns multiples of 8.
 * The grid covers only blocks of active slots: a workgroup finds its slot
 * from num_tokens_post_padded, and the launch size depends on M alone, not
 * on how many slots are active.  Results are deterministic (no atomics).
 * `variant` is a moe_lora_variant; both kernels compute the same function.
 */
MOE_LORA_API int fused_moe_lora(const uint16_t *x, int32_t x_per_pair,
                   const uint16_t *lora_a, const uint16_t *lora_b,
                   const int32_t *sorted_token_ids, const int32_t *expert_ids,
                   const int32_t *num_tokens_post_padded, int32_t max_active_loras,
                   const float *topk_weights, int32_t mul_routed_weight,
                   int32_t add_inputs, int64_t M, int32_t topk, int32_t K,
                   int32_t Ns, int32_t S, int32_t E, int32_t L, int32_t r,
                   int32_t block_m, uint16_t *y, int32_t variant, void *stream);

/*
 * fused_moe_lora_ws -- fused_moe_lora with a workspace: the same arguments,
 * the same function and, for given sizes, the same result bit for bit
 * whatever the timing.  With the workspace the decode stream kernel (VALU
 * variant, r in {32, 64, 128}) splits the shrink's K range among the
 * workgroups that share a
 * (block, slice) -- one per column range of the expand -- instead of having
 * each of them read all of A: each multiplies an equal share of K,
 * publishes its fp32 partial rank vectors in the workspace, and all of them
 * add the partials in the same order, so the rank vector never reaches
 * memory in bf16 and is identical in every workgroup.  (The split-K shrink
 * of the pages' two-kernel path -- prhub summary of vLLM PR #42290,
 * implementation steps -- applied inside the one-shot kernel.)
 *   workspace    [device] at least fused_moe_lora_workspace_bytes() bytes,
 *                16-byte aligned and ZERO-FILLED before its first use.  Its
 *                layout depends on workspace_bytes alone, not on the sizes
 *                of a call: reused as it is (also inside a captured graph),
 *                one workspace serves calls of any size it is large enough
 *                for, provided it is always passed with the same
 *                workspace_bytes (zero-fill it again before passing another
 *                size).  Two calls that may run at the same time must not
 *                share one.  May be NULL when the size is 0 (then this is
 *                fused_moe_lora).
 *   peer_wait    polls (about 0.5 us each) for another workgroup's partial
 *                before this workgroup computes that partial itself, from A
 *                in memory and with the same bits; no workgroup waits on
 *                another beyond that, so the call completes even when the
 *                workgroups of a unit are not resident together.  Negative:
 *                the default (64).  0: every workgroup computes every partial.
 * MOE_LORA_ERR_WORKSPACE when a workspace is needed and is NULL, misaligned
 * or smaller than the size; other statuses as fused_moe_lora.
 */
MOE_LORA_API int fused_moe_lora_ws(const uint16_t *x, int32_t x_per_pair,
                   const uint16_t *lora_a, const uint16_t *lora_b,
                   const int32_t *sorted_token_ids, const int32_t *expert_ids,
                   const int32_t *num_tokens_post_padded, int32_t max_active_loras,
                   const float *topk_weights, int32_t mul_routed_weight,
                   int32_t add_inputs, int64_t M, int32_t topk, int32_t K,
                   int32_t Ns, int32_t S, int32_t E, int32_t L, int32_t r,
                   int32_t block_m, uint16_t *y, int32_t variant,
                   void *workspace, int64_t workspace_bytes, int32_t peer_wait,
                   void *stream);

/*
 * fused_moe_lora_workspace_bytes -- [host, no HIP call] bytes of the
 * workspace fused_moe_lora_ws uses for these sizes: 0 when its kernel has no
 * use for one, else the exchange area of the K split (an upper bound over
 * the blocks these sizes can produce).  Negative status for sizes
 * fused_moe_lora would reject.
 */
MOE_LORA_API int64_t fused_moe_lora_workspace_bytes(int64_t M, int32_t topk, int32_t K,
                   int32_t Ns, int32_t S, int32_t E, int32_t L, int32_t r,
                   int32_t block_m, int32_t x_per_pair, int32_t variant);

/*
 * fused_moe_lora_variant -- [host, no HIP call] the kernel that
 * fused_moe_lora runs for these sizes and `variant`: MOE_LORA_VARIANT_VALU
 * or MOE_LORA_VARIANT_MFMA, AUTO resolved the way fused_moe_lora resolves
 * it.  Returns a negative status when fused_moe_lora would reject the sizes,
 * x_per_pair or the variant (MOE_LORA_ERR_UNSUPPORTED for MFMA when r is not
 * a multiple of 8 in [8, 128], block_m > 128, or x, y, an A matrix or a B
 * matrix exceeds 2 GiB).
 */
MOE_LORA_API int fused_moe_lora_variant(int64_t M, int32_t topk, int32_t K, int32_t Ns,
                   int32_t S, int32_t E, int32_t L, int32_t r, int32_t block_m,
                   int32_t x_per_pair, int32_t variant);

/*
 * fused_moe_lora_kernel_name -- [host, no HIP call] name of the GPU kernel
 * that fused_moe_lora launches for these sizes and `variant` (as profilers
 * print it, without template arguments): "fused_stream_kernel" (decode
 * blocks: A and B streamed through one LDS ring), "fused_valu_kernel"
 * (decode blocks, other ranks or K) or "fused_mfma_kernel" (prefill
 * blocks).  A static string; NULL when fused_moe_lora_variant would return a
 * negative status.
 */
MOE_LORA_API const char *fused_moe_lora_kernel_name(int64_t M, int32_t topk, int32_t K,
                   int32_t Ns, int32_t S, int32_t E, int32_t L, int32_t r, int32_t block_m,
                   int32_t x_per_pair, int32_t variant);

/* Most (token, k) pairs fused_moe_lora_naive takes (M * topk). */
#define MOE_LORA_NAIVE_MAX_PAIRS 1024

/*
 * fused_moe_lora_naive -- fused_moe_lora without the align step, for decode
 * batches: the naive block assignment of the one-shot kernel (prhub summary
 * of vLLM PR #42290, the dispatch fragment: a grid over tokens x top-k,
 * slices and active slots, chosen instead of sorted_token_ids).
 *
 * Computes exactly the function of fused_moe_lora, with each pair's slot and
 * expert read from token_lora_mapping and topk_ids as moe_lora_align reads
 * them (pairs whose slot is outside [0, L) or whose expert is outside [0, E)
 * are skipped; their Y rows are not touched).  Every workgroup forms the
 * (slot, expert) groups on chip and cuts each into blocks of block_m pairs,
 * ascending: the blocks moe_lora_align would produce for this block_m, so
 * for block_m in {16, 32, 64, 128} the result is bit-identical to
 * moe_lora_align followed by fused_moe_lora with the same variant.
 * block_m = 1 gives every valid pair its own block (the weights of a group
 * are then read once per pair).
 *
 * Inputs  [device]:
 *   x, lora_a, lora_b, topk_weights, y: as for fused_moe_lora.
 *   topk_ids             int32 [M, topk]
 *   token_lora_mapping   int32 [M]
 * Sizes: as for fused_moe_lora, except block_m, a power of two in [1, 128]
 * (the MFMA variant takes block_m >= 16; AUTO picks it under the same rule as
 * fused_moe_lora, and fused_moe_lora_kernel_name / fused_moe_lora_variant
 * answer for block_m >= 16; smaller blocks always run the vector variant).
 * Returns MOE_LORA_ERR_UNSUPPORTED when M * topk > MOE_LORA_NAIVE_MAX_PAIRS
 * (larger batches go through moe_lora_align); other errors as for
 * fused_moe_lora.  No workspace; deterministic.
 */
MOE_LORA_API int fused_moe_lora_naive(const uint16_t *x, int32_t x_per_pair,
                   const uint16_t *lora_a, const uint16_t *lora_b,
                   const int32_t *topk_ids, const int32_t *token_lora_mapping,
                   const float *topk_weights, int32_t mul_routed_weight,
                   int32_t add_inputs, int64_t M, int32_t topk, int32_t K,
                   int32_t Ns, int32_t S, int32_t E, int32_t L, int32_t r,
                   int32_t block_m, uint16_t *y, int32_t variant, void *stream);

/* Most pairs and slots fused_moe_lora_with_align takes. */
#define MOE_LORA_WITH_ALIGN_MAX_PAIRS 64
#define MOE_LORA_WITH_ALIGN_MAX_SLOTS 64

/*
 * fused_moe_lora_with_align -- the whole path in one launch: the outputs of
 * moe_lora_align (prhub summary of vLLM PR #42290's align kernel; vLLM PR
 * #29257, Purpose) and the result of fused_moe_lora for the same inputs, for
 * decode batches of at most MOE_LORA_WITH_ALIGN_MAX_PAIRS pairs and
 * MOE_LORA_WITH_ALIGN_MAX_SLOTS slots.  The fused workgroups form their
 * blocks on chip, as fused_moe_lora_naive does, and one workgroup the
 * fused work leaves idle writes the align outputs beside them (nothing reads
 * them in this call), so the align costs no launch of its own and no wait.  The outputs are those of
 * moe_lora_align, bit for bit; y is that of fused_moe_lora_naive with the
 * same block_m, bit for bit.
 *   Inputs as moe_lora_align (topk_ids .. block_m) and as fused_moe_lora
 *   (x .. r, y, variant); outputs sorted_token_ids .. num_active_loras as
 *   moe_lora_align (lora_ids and num_active_loras may be NULL); no
 *   workspace.  block_m as moe_lora_align takes it.  MOE_LORA_ERR_UNSUPPORTED
 *   beyond the pair or slot limit; other statuses as the two calls.  M == 0
 *   writes the (empty) align outputs and touches no y.
 */
MOE_LORA_API int fused_moe_lora_with_align(const int32_t *topk_ids,
                   const int32_t *token_lora_mapping, int64_t M, int32_t topk,
                   int32_t E, int32_t L, int32_t block_m,
                   int32_t *sorted_token_ids, int32_t *expert_ids,
                   int32_t *num_tokens_post_padded, int32_t *lora_ids,
                   int32_t *num_active_loras, const uint16_t *x, int32_t x_per_pair,
                   const uint16_t *lora_a, const uint16_t *lora_b,
                   const float *topk_weights, int32_t mul_routed_weight,
                   int32_t add_inputs, int32_t K, int32_t Ns, int32_t S, int32_t r,
                   uint16_t *y, int32_t variant, void *stream);

/* Largest rank fused_moe_lora_two_kernel takes. */
#define MOE_LORA_TWO_KERNEL_MAX_RANK 512

/*
 * fused_moe_lora_two_kernel_workspace_bytes -- [host, no HIP call] bytes of
 * device workspace fused_moe_lora_two_kernel needs for these sizes (the
 * fp32 rank vectors of every pair and slice, once per K split); a negative
 * status when fused_moe_lora_two_kernel would reject the sizes.
 */
MOE_LORA_API int64_t fused_moe_lora_two_kernel_workspace_bytes(int64_t M, int32_t topk,
                   int32_t K, int32_t Ns, int32_t S, int32_t E, int32_t L, int32_t r,
                   int32_t block_m, int32_t x_per_pair);

/*
 * fused_moe_lora_two_kernel -- the same function as fused_moe_lora, computed
 * by two kernels with the rank vectors in memory: the path the one-shot
 * kernel replaces (prhub summary of vLLM PR #42290: motivation, and its key
 * source fragment, where ranks above 128 are left to the two-kernel path; the shrink
 * and expand launches of the PR #32005 diff).  Takes ranks up to
 * MOE_LORA_TWO_KERNEL_MAX_RANK, past fused_moe_lora's 128.
 *
 * A shrink kernel writes, for every valid pair p and slice s, the fp32 rank
 * vector v[j] = sum_t X[row, t] A[s,l,e,j,t] into the workspace (in K splits,
 * one workspace slice each); an expand kernel adds the splits in a fixed
 * order and writes Y[p, s*Ns+n] = bf16(add ? Y + w d[n] : w d[n]) with
 * d[n] = sum_j v[j] B[s,l,e,n,j] (v enters the bf16 products as a bf16
 * high / low pair).  Two launches on `stream`, in that order.
 *
 * Arguments as for fused_moe_lora (the align outputs of the same M, topk, E,
 * L, block_m), plus:
 *   workspace   [device] at least fused_moe_lora_two_kernel_workspace_bytes()
 *               bytes, 16-byte aligned; contents on entry do not matter,
 *               contents on return are the rank vectors (unspecified rows for
 *               pairs in no slot).  MOE_LORA_ERR_WORKSPACE when too small.
 * MOE_LORA_ERR_UNSUPPORTED for r > MOE_LORA_TWO_KERNEL_MAX_RANK or when x, an
 * A matrix or a B matrix exceeds 2 GiB.  Deterministic (no atomics).
 */
MOE_LORA_API int fused_moe_lora_two_kernel(const uint16_t *x, int32_t x_per_pair,
                   const uint16_t *lora_a, const uint16_t *lora_b,
                   const int32_t *sorted_token_ids, const int32_t *expert_ids,
                   const int32_t *num_tokens_post_padded, int32_t max_active_loras,
                   const float *topk_weights, int32_t mul_routed_weight,
                   int32_t add_inputs, int64_t M, int32_t topk, int32_t K,
                   int32_t Ns, int32_t S, int32_t E, int32_t L, int32_t r,
                   int32_t block_m, uint16_t *y, void *workspace,
                   int64_t workspace_bytes, void *stream);

/*
 * moe_lora_accumulate -- y[i] = bf16(y[i] + delta[i]) for i < n, the sum in
 * fp32, rounded to nearest even once: the join of the dual-stream path (prhub
 * summary of vLLM PR #42290, implementation step 2 and the TritonExperts
 * fragment: the base MoE GEMM on the default stream, fused_moe_lora with
 * add_inputs = 0 into a zero-filled delta buffer on an auxiliary stream, the
 * delta added onto the base output once both streams have met).  The caller
 * orders the streams (an event recorded on the auxiliary stream and waited
 * for on `stream`).
 * [device] y, delta: bf16 [n], 16-byte aligned, not overlapping.  n == 0
 * does nothing; MOE_LORA_ERR_INVALID for n < 0, null or misaligned pointers.
 */
MOE_LORA_API int moe_lora_accumulate(uint16_t *y, const uint16_t *delta, int64_t n,
                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LORA_H */
