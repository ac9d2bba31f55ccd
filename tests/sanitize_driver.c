/* Drives the fp64 oracle, the host block allocator and the host input checks through
 * small seeded cases so that an AddressSanitizer / UndefinedBehaviorSanitizer build can
 * watch every path: decode, contiguous decode, prefill, append (with fp8 per-head
 * scales), block copy, widening and the E4M3 encoder; allocator acquire, share,
 * release, reserve with copy-on-write, fork, truncate and rejected calls; table, query
 * range and slot checks.  Exits 0 when every call returned what it should (the
 * sanitizers abort the process on a finding). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../include/paged_attention.h"

int oracle_decode_paged_hs(const void *q, int q_dtype, const void *k_pool, const void *v_pool,
                           int kv_dtype, double k_scale, double v_scale,
                           const float *k_head_scales, const float *v_head_scales, int num_seqs,
                           int num_q_heads, int num_kv_heads, int head_dim, int num_blocks,
                           const int32_t *block_tables, int max_blocks_per_seq,
                           const int32_t *context_lens, float scale, double *out, double *wsum,
                           int num_threads);
int oracle_prefill_paged_hs(const void *q, int q_dtype, const void *k_pool, const void *v_pool,
                            int kv_dtype, double k_scale, double v_scale,
                            const float *k_head_scales, const float *v_head_scales,
                            int num_seqs, const int32_t *query_start, int num_q_heads,
                            int num_kv_heads, int head_dim, int num_blocks,
                            const int32_t *block_tables, int max_blocks_per_seq,
                            const int32_t *context_lens, float scale, double *out,
                            double *wsum, int num_threads);
int oracle_decode_contig(const void *q, const void *k, const void *v, int dtype, int num_seqs,
                         int num_q_heads, int num_kv_heads, int head_dim, int s_max,
                         const int32_t *context_lens, float scale, double *out, double *wsum,
                         int num_threads);
int oracle_cache_append_hs(void *k_pool, void *v_pool, int kv_dtype, int act_dtype,
                           float k_scale, float v_scale, const float *k_head_scales,
                           const float *v_head_scales, int num_blocks, int num_kv_heads,
                           int head_dim, const void *k_new, const void *v_new,
                           const int32_t *slot_mapping, int num_tokens);
int oracle_copy_blocks(void *k_pool, void *v_pool, int dtype, int num_blocks, int num_kv_heads,
                       int head_dim, const int32_t *pairs, int num_pairs);
int oracle_widen(const void *src, int dtype, size_t n, double *dst);
void oracle_encode_e4m3(const float *src, size_t n, uint8_t *dst);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double urand(void)
{
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

static int oracle_cases(void)
{
    enum { NB = 9, HKV = 2, HQ = 6, D = 16, B = 3, MAXB = 3 };
    float kf[NB * HKV * 16 * D], vf[NB * HKV * D * 16], qf[B * HQ * D];
    for (size_t i = 0; i < sizeof kf / sizeof kf[0]; ++i) kf[i] = (float)urand();
    for (size_t i = 0; i < sizeof vf / sizeof vf[0]; ++i) vf[i] = (float)urand();
    for (size_t i = 0; i < sizeof qf / sizeof qf[0]; ++i) qf[i] = (float)urand();
    int32_t tables[B * MAXB] = {4, 1, 7, 0, 8, 2, 5, 3, 6};
    int32_t ctx[B] = {37, 0, 48};
    double out[B * HQ * D], wsum[B * HQ];
    CHECK(oracle_decode_paged_hs(qf, 0, kf, vf, 0, 1.0, 1.0, NULL, NULL, B, HQ, HKV, D, NB, tables,
                                 MAXB, ctx, 0.25f, out, wsum, 2) == 0);
    CHECK(wsum[HQ] == 0.0 && wsum[0] > 0.999);
    int32_t bad[B * MAXB] = {4, 1, 99, 0, 8, 2, 5, 3, 6};
    CHECK(oracle_decode_paged_hs(qf, 0, kf, vf, 0, 1.0, 1.0, NULL, NULL, B, HQ, HKV, D, NB, bad,
                                 MAXB, ctx, 0.25f, out, wsum, 1) == -2);
    /* fp8 pools with per-head scales (one unusable), f16 q */
    uint8_t k8[NB * HKV * 16 * D], v8[NB * HKV * D * 16];
    oracle_encode_e4m3(kf, sizeof k8, k8);
    oracle_encode_e4m3(vf, sizeof v8, v8);
    uint16_t q16[B * HQ * D];
    for (size_t i = 0; i < sizeof q16 / sizeof q16[0]; ++i) q16[i] = (uint16_t)(0x3C00 ^ (i & 0x3FF));
    float ks[HKV] = {0.02f, 0.0f}, vs[HKV] = {0.01f, 0.03f};
    CHECK(oracle_decode_paged_hs(q16, 1, k8, v8, 3, 1.0, 1.0, ks, vs, B, HQ, HKV, D, NB, tables,
                                 MAXB, ctx, 0.25f, out, wsum, 3) == 0);
    CHECK(out[(size_t)(HQ - 1) * D] != out[(size_t)(HQ - 1) * D]);   /* head 1 poisoned: NaN */
    /* append rows of f16 into the fp8 pool through slots, one padded, one past the pool */
    int32_t slots[4] = {4 * 16 + 3, -1, 8 * 16 + 15, NB * 16};
    uint16_t kn[4 * HKV * D], vn[4 * HKV * D];
    for (size_t i = 0; i < sizeof kn / sizeof kn[0]; ++i) { kn[i] = (uint16_t)(0x3800 + i); vn[i] = (uint16_t)(0x3400 + i); }
    CHECK(oracle_cache_append_hs(k8, v8, 3, 1, 1.0f, 1.0f, ks, vs, NB, HKV, D, kn, vn, slots, 3) == 0);
    CHECK(oracle_cache_append_hs(k8, v8, 3, 1, 1.0f, 1.0f, ks, vs, NB, HKV, D, kn, vn, slots, 4) == -2);
    /* prefill: chunks of 5, 0 and 48 query rows */
    int32_t qs[B + 1] = {0, 5, 5, 53};
    static float qp[53 * HQ * D];
    for (size_t i = 0; i < sizeof qp / sizeof qp[0]; ++i) qp[i] = (float)urand();
    static double pout[53 * HQ * D], pw[53 * HQ];
    CHECK(oracle_prefill_paged_hs(qp, 0, kf, vf, 0, 1.0, 1.0, NULL, NULL, B, qs, HQ, HKV, D, NB,
                                  tables, MAXB, ctx, 0.25f, pout, pw, 2) == 0);
    /* contiguous cache, block copy, widening */
    static float kc[B * HKV * 48 * D], vc[B * HKV * 48 * D];
    for (size_t i = 0; i < sizeof kc / sizeof kc[0]; ++i) { kc[i] = (float)urand(); vc[i] = (float)urand(); }
    CHECK(oracle_decode_contig(qf, kc, vc, 0, B, HQ, HKV, D, 48, ctx, 0.25f, out, wsum, 2) == 0);
    int32_t pairs[6] = {1, 0, -1, 3, 2, 9};
    CHECK(oracle_copy_blocks(kf, vf, 0, NB, HKV, D, pairs, 3) == 0);
    double wide[256];
    uint8_t codes[256];
    for (int i = 0; i < 256; ++i) codes[i] = (uint8_t)i;
    CHECK(oracle_widen(codes, 3, 256, wide) == 0);
    return 0;
}

static int allocator_cases(void)
{
    CHECK(pa_allocator_create(0) == NULL);
    pa_block_allocator *a = pa_allocator_create(12);
    CHECK(a != NULL && pa_allocator_num_free(a) == 12);
    int32_t ids[12];
    CHECK(pa_allocator_acquire(a, 13, ids) == PA_ERR_OUT_OF_BLOCKS && pa_allocator_num_free(a) == 12);
    int32_t row[8], row2[8], slots[40], pairs[2], ncopy = -1;
    for (int i = 0; i < 8; ++i) row[i] = row2[i] = -1;
    CHECK(pa_seq_reserve(a, row, 8, 0, 35, slots, pairs, &ncopy) == PA_OK && ncopy == 0);
    CHECK(pa_allocator_num_free(a) == 9);
    CHECK(pa_seq_fork(a, row, row2, 8, 35) == PA_OK && pa_allocator_ref_count(a, row[0]) == 2);
    CHECK(pa_seq_reserve(a, row2, 8, 35, 1, slots, pairs, &ncopy) == PA_OK && ncopy == 1);
    CHECK(pa_seq_reserve(a, row, 8, 35, 200, slots, pairs, &ncopy) == PA_ERR_INVALID_ARG);
    CHECK(pa_seq_truncate(a, row2, 8, 36, 0) == PA_OK);
    CHECK(pa_seq_truncate(a, row, 8, 35, 17) == PA_OK);
    CHECK(pa_allocator_share(a, row, 2) == PA_OK && pa_allocator_release(a, row, 2) == PA_OK);
    int32_t badid = 99;
    CHECK(pa_allocator_release(a, &badid, 1) != PA_OK);
    CHECK(pa_seq_truncate(a, row, 8, 17, 0) == PA_OK && pa_allocator_num_free(a) == 12);
    pa_allocator_destroy(a);
    return 0;
}

static int validate_cases(void)
{
    int32_t bt[2 * 4] = {5, 7, 2, -1, 1, 99, -3, 0};
    int32_t cl[2] = {37, 16}, bad = 0;
    CHECK(pa_validate_decode_tables(2, bt, 4, cl, 64, 8, &bad) == PA_OK && bad == -1);
    cl[1] = 17;
    CHECK(pa_validate_decode_tables(2, bt, 4, cl, 64, 8, &bad) == PA_ERR_INVALID_ARG && bad == 1);
    cl[1] = 16;
    int32_t qs[3] = {0, 5, 12};
    CHECK(pa_validate_prefill_batch(2, qs, 12, 8, bt, 4, cl, 64, 8, &bad) == PA_OK);
    qs[2] = 13;
    CHECK(pa_validate_prefill_batch(2, qs, 12, 8, bt, 4, cl, 64, 8, &bad) == PA_ERR_INVALID_ARG);
    int32_t slots[5] = {3, -1, 17, 127, 3};
    CHECK(pa_validate_slots(slots, 4, 8, &bad) == PA_OK);
    CHECK(pa_validate_slots(slots, 5, 8, &bad) == PA_ERR_INVALID_ARG && bad == 4);
    CHECK(pa_validate_slots(slots, 5, 0, NULL) == PA_ERR_INVALID_ARG);
    /* row 0 reads 5, 7, 2; row 1 reads 1: nothing shared; row 1 reading 2 shares it */
    CHECK(pa_tables_share_blocks(2, bt, 4, cl) == 0);
    bt[4] = 2;
    CHECK(pa_tables_share_blocks(2, bt, 4, cl) == 1);
    CHECK(pa_tables_share_blocks(0, NULL, 4, NULL) == 0);
    CHECK(pa_tables_share_blocks(2, NULL, 4, cl) == -1);
    return 0;
}

int main(void)
{
    if (oracle_cases() || allocator_cases() || validate_cases())
        return 1;
    printf("sanitized oracle and allocator cases passed\n");
    return 0;
}
