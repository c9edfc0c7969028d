/*
 * oracle.c -- plain CPU reference of the MoE-LoRA hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no source with the HIP library.
 *
 * What it computes, and where the pages define it:
 *
 *  oracle_align -- the align step (vLLM PR #29257 "Lora MoE Align
 *    Improvements", Purpose: per LoRA slot, the (token, k) pairs are grouped
 *    by expert and every group is padded to BLOCK_M; the LoRA and non-LoRA
 *    cases share one routine).  Outputs are the three arrays the pages hand
 *    to the fused kernel (sorted_token_ids and expert_ids viewed per slot as
 *    [max_loras, -1], and num_tokens_post_padded; PR #32005 diff of
 *    tests/lora/test_fused_moe_lora_kernel.py), plus the list of active slots
 *    that the active-LoRA grid of PR #32005 indexes with lora_ids.
 *    Readings taken where the pages are silent: padding entries hold
 *    numel = M*topk; inside a group pairs are in ascending flat index
 *    p = m*topk + k; groups are in ascending expert id; an empty group takes
 *    no space; a token with mapping -1 (or any id outside [0, L)) and an
 *    expert id outside [0, E) are skipped.
 *
 *  oracle_fused -- the fused shrink+expand (prhub summary of vLLM PR #42290,
 *    implementation steps and key source fragment: x is multiplied by lora_a,
 *    the rank-sized result is multiplied by lora_b, and the product either
 *    overwrites or is added onto the output, ADD_INPUTS; the routed weight is
 *    optional, mul_routed_weight in the PR #32005 diff).  For every valid pair
 *    p = (m, k) with slot l and expert e, and every slice s:
 *        v[j]  = sum_t X[row, t] * A[s, l, e, j, t]         (row = m, or p)
 *        d[n]  = sum_j v[j] * B[s, l, e, n, j]
 *        d[n] *= w[m, k]                      when mul_routed_weight
 *        Y[p, s*Ns + n] = (add ? Y_in[p, s*Ns + n] : 0) + d[n]
 *    Invalid pairs keep Y_in.  Arithmetic is in double: every bf16 value is
 *    widened exactly, products of two bf16 values are exact in double, and the
 *    sums are taken in the order written above (t ascending, then j
 *    ascending).  The result is not rounded back to bf16.
 *
 * The fused routine never reads the align outputs: it walks the pairs
 * directly, so a comparison against it also checks the align -> fused hand-off
 * of the HIP path.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact widening of a bf16 bit pattern: its 16 bits are the upper half of an
 * IEEE binary32 value. */
static double bf16_to_double(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Per-slot row length of sorted_token_ids: the largest padded total one slot
 * can reach, numel + min(E, numel) * (block_m - 1), rounded up to block_m. */
int64_t oracle_capacity(int64_t M, int32_t topk, int32_t E, int32_t block_m)
{
    int64_t numel = M * (int64_t)topk;
    int64_t groups = E < numel ? (int64_t)E : numel;
    int64_t bound = numel + groups * (block_m - 1);
    return (bound + block_m - 1) / block_m * block_m;
}

/* Returns 0 on success, -1 on allocation failure. */
int oracle_align(const int32_t *topk_ids, const int32_t *token_lora_mapping,
                 int64_t M, int32_t topk, int32_t E, int32_t L, int32_t block_m,
                 int64_t cap,
                 int32_t *sorted_token_ids,        /* [L, cap]            */
                 int32_t *expert_ids,              /* [L, cap / block_m]  */
                 int32_t *num_tokens_post_padded,  /* [L]                 */
                 int32_t *lora_ids,                /* [L]                 */
                 int32_t *num_active)              /* [1]                 */
{
    int64_t numel = M * (int64_t)topk;
    int64_t nb = cap / block_m;
    int64_t groups = (int64_t)L * E;
    int64_t *count = calloc((size_t)groups, sizeof *count);
    int64_t *start = calloc((size_t)groups, sizeof *start);
    int64_t *cursor = calloc((size_t)groups, sizeof *cursor);
    if (!count || !start || !cursor) {
        free(count); free(start); free(cursor);
        return -1;
    }

    /* 1. how many valid pairs fall in each (slot, expert) group */
    for (int64_t p = 0; p < numel; ++p) {
        int64_t m = p / topk;
        int32_t l = token_lora_mapping[m];
        int32_t e = topk_ids[p];
        if (l < 0 || l >= L || e < 0 || e >= E)
            continue;
        count[(int64_t)l * E + e] += 1;
    }

    /* 2. padded sizes and group starts, experts in ascending order per slot */
    for (int32_t l = 0; l < L; ++l) {
        int64_t offset = 0;
        for (int32_t e = 0; e < E; ++e) {
            int64_t c = count[(int64_t)l * E + e];
            int64_t padded = (c + block_m - 1) / block_m * block_m;
            start[(int64_t)l * E + e] = offset;
            offset += padded;
        }
        num_tokens_post_padded[l] = (int32_t)offset;
    }

    /* 3. the expert of every block */
    for (int32_t l = 0; l < L; ++l) {
        for (int32_t e = 0; e < E; ++e) {
            int64_t c = count[(int64_t)l * E + e];
            int64_t padded = (c + block_m - 1) / block_m * block_m;
            int64_t first = start[(int64_t)l * E + e] / block_m;
            for (int64_t b = first; b < first + padded / block_m; ++b)
                expert_ids[(int64_t)l * nb + b] = e;
        }
    }

    /* 4. place every valid pair, walking p upwards */
    for (int64_t g = 0; g < groups; ++g)
        cursor[g] = start[g];
    for (int64_t p = 0; p < numel; ++p) {
        int64_t m = p / topk;
        int32_t l = token_lora_mapping[m];
        int32_t e = topk_ids[p];
        if (l < 0 || l >= L || e < 0 || e >= E)
            continue;
        int64_t g = (int64_t)l * E + e;
        sorted_token_ids[(int64_t)l * cap + cursor[g]] = (int32_t)p;
        cursor[g] += 1;
    }

    /* 5. fill each group's padding with the sentinel numel */
    for (int32_t l = 0; l < L; ++l) {
        for (int32_t e = 0; e < E; ++e) {
            int64_t g = (int64_t)l * E + e;
            int64_t padded = (count[g] + block_m - 1) / block_m * block_m;
            for (int64_t i = start[g] + count[g]; i < start[g] + padded; ++i)
                sorted_token_ids[(int64_t)l * cap + i] = (int32_t)numel;
        }
    }

    /* 6. active slots (non-empty), ascending, then -1 */
    int32_t n = 0;
    for (int32_t l = 0; l < L; ++l)
        if (num_tokens_post_padded[l] > 0)
            lora_ids[n++] = l;
    *num_active = n;
    for (int32_t l = n; l < L; ++l)
        lora_ids[l] = -1;

    free(count); free(start); free(cursor);
    return 0;
}

/* One valid pair: writes its S*Ns outputs into out_row (double). */
static void fused_one_pair(const uint16_t *x, int32_t x_per_pair,
                           const uint16_t *lora_a, const uint16_t *lora_b,
                           int64_t p, int64_t m, int32_t l, int32_t e,
                           const float *topk_weights, int32_t mul, int32_t add,
                           int32_t K, int32_t Ns, int32_t S, int32_t E, int32_t L,
                           int32_t r, const uint16_t *y_in_row, double *out_row,
                           double *v)
{
    int64_t row = x_per_pair ? p : m;
    const uint16_t *xr = x + row * (int64_t)K;
    for (int32_t s = 0; s < S; ++s) {
        const uint16_t *A = lora_a + (((int64_t)s * L + l) * E + e) * (int64_t)r * K;
        const uint16_t *B = lora_b + (((int64_t)s * L + l) * E + e) * (int64_t)Ns * r;
        for (int32_t j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int32_t t = 0; t < K; ++t)
                acc += bf16_to_double(xr[t]) * bf16_to_double(A[(int64_t)j * K + t]);
            v[j] = acc;
        }
        for (int32_t n = 0; n < Ns; ++n) {
            double d = 0.0;
            for (int32_t j = 0; j < r; ++j)
                d += v[j] * bf16_to_double(B[(int64_t)n * r + j]);
            if (mul)
                d *= (double)topk_weights[p];
            int64_t col = (int64_t)s * Ns + n;
            double base = add ? bf16_to_double(y_in_row[col]) : 0.0;
            out_row[col] = base + d;
        }
    }
}

/*
 * Full output: out[numel, S*Ns] (double).  Rows of invalid pairs hold Y_in.
 * If pairs != NULL, only the listed pairs are computed and out has
 * [n_pairs, S*Ns] rows, in the order of the list (a pair that is not valid
 * gets its Y_in row).  Returns 0, or -1 on allocation failure.
 */
int oracle_fused(const uint16_t *x, int32_t x_per_pair,
                 const uint16_t *lora_a, const uint16_t *lora_b,
                 const int32_t *topk_ids, const int32_t *token_lora_mapping,
                 const float *topk_weights, int32_t mul_routed_weight,
                 int32_t add_inputs, int64_t M, int32_t topk, int32_t K,
                 int32_t Ns, int32_t S, int32_t E, int32_t L, int32_t r,
                 const uint16_t *y_in, const int64_t *pairs, int64_t n_pairs,
                 double *out)
{
    int64_t numel = M * (int64_t)topk;
    int64_t N = (int64_t)S * Ns;
    int64_t count = pairs ? n_pairs : numel;
    int failed = 0;

#pragma omp parallel
    {
        double *v = malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
        if (!v) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < count; ++i) {
            int64_t p = pairs ? pairs[i] : i;
            double *out_row = out + i * N;
            const uint16_t *y_in_row = y_in + p * N;
            int64_t m = p / topk;
            int32_t l = token_lora_mapping[m];
            int32_t e = topk_ids[p];
            if (!v || l < 0 || l >= L || e < 0 || e >= E) {
                for (int64_t c = 0; c < N; ++c)
                    out_row[c] = bf16_to_double(y_in_row[c]);
                continue;
            }
            fused_one_pair(x, x_per_pair, lora_a, lora_b, p, m, l, e,
                           topk_weights, mul_routed_weight, add_inputs, K, Ns,
                           S, E, L, r, y_in_row, out_row, v);
        }
        free(v);
    }
    return failed ? -1 : 0;
}
