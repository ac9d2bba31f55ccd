/*
 * oracle.c -- plain, slow, fp64 CPU reference for paged attention (decode and prefill).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path never
 * links, imports or calls it, and it shares no source, header or table with the
 * GPU kernels.
 *
 * What it computes (sources are the four web pages on paged KV caches):
 *
 *  - Paged KV storage: the KV cache is cut into fixed 16-token physical blocks and a
 *    per-request block table maps logical block -> physical block
 *    (LLM-101-CN "推理优化", section "物理块与逻辑块"; 16 tokens per block also in
 *    "大模型推理的三维本质原理解析与工程实践", section on PagedAttention).
 *    Token t of a request lives in physical block table[t / 16] at row t % 16
 *    (same page, PagedAttentionManager.get_kv_cache; "LLM应用 12 推理优化",
 *    PagedKVCache.update: page index = seq_idx // page_size, offset = seq_idx % page_size).
 *
 *  - Attention of one decode query: softmax(q . K^T / sqrt(d_h)) . V
 *    (LLM-101-CN "推理优化", section "Chunked Prefill", standard attention with the
 *    1/sqrt(head_dim) factor).  Here the scale is the caller's fp32 value, widened.
 *
 *  - GQA: q-heads are split into contiguous groups, each group reads one KV head
 *    ("大模型推理的三维本质原理解析与工程实践", section 6 GQA): kv_head = h / (Hq/Hkv).
 *
 *  - Paged prefill: the queries of a prompt chunk attend to the cache over the same
 *    block tables, each to its own prefix (causal); a decode query is the one-row case
 *    (oracle_prefill_paged_ex below gives the sources).
 *
 * It is written as the plain definition: resolve each token through the table, form
 * every score, take the maximum, exponentiate, sum, weight V, divide once.  It does
 * NOT use the pages' per-page combine or online softmax; the tests check those forms
 * against this one.  Every (sequence, q-head) is summed in logical token order, so
 * the result does not depend on the thread count or on where blocks sit in the pool.
 *
 * Storage layouts read here (element = 4 bytes for f32, 2 for f16/bf16, 1 for fp8):
 *   q        [B][Hq][d]
 *   k_pool   [num_blocks][Hkv][16][d]   (token-major inside a block)
 *   v_pool   [num_blocks][Hkv][d][16]   (token-minor inside a block)
 *   block_tables [B][max_blocks_per_seq] int32, context_lens [B] int32
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BLOCK 16

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2, ORACLE_FP8_E4M3 = 3 };

/* IEEE binary16 -> double, written from the format's definition:
 * sign | 5-bit exponent (bias 15) | 10-bit fraction.                                */
static double widen_f16_bits(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);                    /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(frac | 0x400), expo - 25);    /* 1.frac * 2^(expo-15)    */
    return sign ? -v : v;
}

/* bfloat16 -> double: a bf16 value is the top half of an IEEE binary32.           */
static double widen_bf16_bits(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3 ("E4M3FN") -> double: sign | 4-bit exponent (bias 7) | 3-bit fraction;
 * no infinities, S.1111.111 is NaN; largest finite magnitude 448.                   */
static double widen_e4m3_bits(uint8_t c)
{
    int sign = (c >> 7) & 1;
    int expo = (c >> 3) & 0xf;
    int frac = c & 0x7;
    double v;
    if (expo == 15 && frac == 7)
        v = NAN;
    else if (expo == 0)
        v = ldexp((double)frac, -9);                     /* subnormal: frac * 2^-9 */
    else
        v = ldexp((double)(frac | 0x8), expo - 10);      /* 1.frac * 2^(expo-7)   */
    return sign ? -v : v;
}

/* float -> E4M3 code: round to nearest, ties to even, magnitudes >= 448 saturate to
 * 448, NaN stays NaN.  Written from the format's value set: subnormals are integer
 * multiples of 2^-9 below 2^-6; a normal value in [2^k, 2^(k+1)) has 8 steps.         */
static uint8_t encode_e4m3(float x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x))
        return sign | 0x7f;
    float a = fabsf(x);
    if (a >= 448.0f)
        return sign | 0x7e;
    if (a < 0.015625f) {                            /* below 2^-6 */
        float steps = rintf(a * 512.0f);            /* exact scaling, then RNE */
        return sign | (uint8_t)steps;               /* 8 steps = smallest normal */
    }
    int e;
    (void)frexpf(a, &e);                            /* a in [2^(e-1), 2^e) */
    int k = e - 1;
    float steps = rintf(ldexpf(a, 3 - k));          /* in [8, 16] */
    if (steps == 16.0f) {
        k += 1;
        steps = 8.0f;
    }
    return sign | (uint8_t)(((k + 7) << 3) | ((int)steps - 8));
}

static size_t elem_bytes(int dtype)
{
    return dtype == ORACLE_F32 ? 4 : (dtype == ORACLE_FP8_E4M3 ? 1 : 2);
}

static double widen_at(const void *base, size_t idx, int dtype)
{
    if (dtype == ORACLE_FP8_E4M3)
        return widen_e4m3_bits(((const uint8_t *)base)[idx]);
    if (dtype == ORACLE_F32) {
        float f;
        memcpy(&f, (const char *)base + 4 * idx, 4);
        return (double)f;
    }
    uint16_t bits;
    memcpy(&bits, (const char *)base + 2 * idx, 2);
    return dtype == ORACLE_F16 ? widen_f16_bits(bits) : widen_bf16_bits(bits);
}

int oracle_widen(const void *src, int dtype, size_t n, double *dst)
{
    if (dtype < ORACLE_F32 || dtype > ORACLE_FP8_E4M3)
        return -1;
    for (size_t i = 0; i < n; ++i)
        dst[i] = widen_at(src, i, dtype);
    return 0;
}

/* E4M3 codes of n floats (the quantiser the fp8 append uses).                        */
void oracle_encode_e4m3(const float *src, size_t n, uint8_t *dst)
{
    for (size_t i = 0; i < n; ++i)
        dst[i] = encode_e4m3(src[i]);
}

/* KV cache size 2 * L * H * d_h * S * B * dtype_size
 * (LLM-101-CN "推理优化", section "KV Cache 的显存计算").                             */
uint64_t oracle_kv_cache_bytes(uint64_t layers, uint64_t kv_heads, uint64_t head_dim,
                               uint64_t seq_len, uint64_t batch, uint64_t dtype_size)
{
    return 2ull * layers * kv_heads * head_dim * seq_len * batch * dtype_size;
}

/* ---------------------------------------------------------------- attention core */

/* Attention of one query row over n keys given by two accessor callbacks.
 * Plain two-pass form: scores, max, exp, sum, weighted V, one final divide.       */
typedef struct {
    const void *q_row;        /* d elements of q_dtype */
    int q_dtype, d;
    double scale;
    int n;                    /* number of keys */
    double *scores;           /* scratch, n entries */
    /* key/value element accessors */
    double (*key)(const void *ctx, int t, int e);
    double (*val)(const void *ctx, int t, int e);
    const void *ctx;
} attn_job;

static void attend(const attn_job *J, double *out, double *wsum)
{
    const int d = J->d, n = J->n;
    if (n == 0) {                 /* empty context: defined as a zero output */
        for (int e = 0; e < d; ++e)
            out[e] = 0.0;
        *wsum = 0.0;
        return;
    }
    double m = -INFINITY;
    for (int t = 0; t < n; ++t) {
        double dot = 0.0;
        for (int e = 0; e < d; ++e)
            dot += widen_at(J->q_row, (size_t)e, J->q_dtype) * J->key(J->ctx, t, e);
        J->scores[t] = J->scale * dot;
        if (J->scores[t] > m)
            m = J->scores[t];
    }
    double z = 0.0;
    for (int t = 0; t < n; ++t) {
        J->scores[t] = exp(J->scores[t] - m);      /* scores now hold the weights w_t */
        z += J->scores[t];
    }
    for (int e = 0; e < d; ++e) {
        double acc = 0.0;
        for (int t = 0; t < n; ++t)
            acc += J->scores[t] * J->val(J->ctx, t, e);
        out[e] = acc / z;
    }
    double s = 0.0;
    for (int t = 0; t < n; ++t)
        s += J->scores[t] / z;
    *wsum = s;
}

/* ----------------------------------------------------------- paged accessors */

typedef struct {
    const void *k_pool, *v_pool;
    int dtype, hkv, d, kv_head;
    double k_scale, v_scale;   /* stored value x scale = K, V (1 unless fp8) */
    const int32_t *table_row;  /* logical block -> physical block */
} paged_ctx;

static double paged_key(const void *c, int t, int e)
{
    const paged_ctx *P = (const paged_ctx *)c;
    size_t phys = (size_t)P->table_row[t / ORACLE_BLOCK];
    size_t off = (size_t)(t % ORACLE_BLOCK);
    size_t idx = ((phys * P->hkv + P->kv_head) * ORACLE_BLOCK + off) * P->d + e;
    return widen_at(P->k_pool, idx, P->dtype) * P->k_scale;
}

static double paged_val(const void *c, int t, int e)
{
    const paged_ctx *P = (const paged_ctx *)c;
    size_t phys = (size_t)P->table_row[t / ORACLE_BLOCK];
    size_t off = (size_t)(t % ORACLE_BLOCK);
    size_t idx = ((phys * P->hkv + P->kv_head) * P->d + e) * ORACLE_BLOCK + off;
    return widen_at(P->v_pool, idx, P->dtype) * P->v_scale;
}

/* ------------------------------------------------------- contiguous accessors */

typedef struct {
    const void *k, *v;        /* [B][Hkv][S][d] each, dtype elements */
    int dtype, hkv, d, s_max, seq, kv_head;
    double k_scale, v_scale;
} contig_ctx;

static double contig_key(const void *c, int t, int e)
{
    const contig_ctx *C = (const contig_ctx *)c;
    size_t idx = (((size_t)C->seq * C->hkv + C->kv_head) * C->s_max + t) * C->d + e;
    return widen_at(C->k, idx, C->dtype) * C->k_scale;
}

static double contig_val(const void *c, int t, int e)
{
    const contig_ctx *C = (const contig_ctx *)c;
    size_t idx = (((size_t)C->seq * C->hkv + C->kv_head) * C->s_max + t) * C->d + e;
    return widen_at(C->v, idx, C->dtype) * C->v_scale;
}

/* ---------------------------------------------------------------- threading */

typedef struct {
    int paged;                 /* 1: paged pool, 0: contiguous cache */
    const void *q;
    const void *k, *v;
    int dtype, q_dtype;        /* K/V storage type, q type */
    double k_scale, v_scale;
    int B, hq, hkv, d, num_blocks, max_blocks, s_max;
    const int32_t *tables, *ctx_lens;
    double scale;
    double *out, *wsum;
    int nthreads;
    /* prefill only (NULL / 0 for decode): query rows of sequence b are
     * q_start[b] .. q_start[b+1]-1 of q [num_tokens][Hq][d]                          */
    const int32_t *q_start;
    int num_tokens;
    /* fp8 pools: a scale per kv-head (NULL: k_scale / v_scale for every head)        */
    const float *k_head_scales, *v_head_scales;
} decode_args;

/* A usable scale is finite and > 0.                                                  */
static int scale_ok(double s) { return s > 0.0 && isfinite(s); }

/* Sequence that owns query row `tok` (q_start is non-decreasing, q_start[0] = 0).    */
static int owner_of(const int32_t *q_start, int B, int tok)
{
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (q_start[mid] <= tok)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

typedef struct {
    const decode_args *A;
    int tid;
} worker_arg;

static void *decode_worker(void *p)
{
    const worker_arg *W = (const worker_arg *)p;
    const decode_args *A = W->A;
    const int group = A->hq / A->hkv;
    int cap = A->paged ? A->max_blocks * ORACLE_BLOCK : A->s_max;
    double *scores = (double *)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
    if (!scores)
        return (void *)1;
    /* units (query row, q-head) are dealt round-robin; each unit is self-contained.
     * Decode has one query row per sequence, the sequence's newest token, which sees
     * the whole context.  Prefill row r of sequence b is token ctx - q_len + i of it
     * (i = r - q_start[b]; the chunk was appended before attending) and sees tokens
     * 0 .. ctx - q_len + i: its own prefix, itself included.                         */
    const int rows = A->q_start ? A->num_tokens : A->B;
    for (int u = W->tid; u < rows * A->hq; u += A->nthreads) {
        int r = u / A->hq, h = u % A->hq;
        int b = A->q_start ? owner_of(A->q_start, A->B, r) : r;
        int n = A->ctx_lens[b];
        if (A->q_start) {
            int q_len = A->q_start[b + 1] - A->q_start[b];
            int pos = n - q_len + (r - A->q_start[b]);
            n = pos < 0 ? 0 : pos + 1;
        }
        int kvh = h / group;
        /* K of kv-head kvh = stored value x its scale (V likewise): the head's entry of
         * a per-head array when one is given, else the pool's one scale.  The FP8
         * format scales a tensor ("Deep dive into vLLM 06", FP8 section); a per-head
         * array treats each head's slice of the cache as its own tensor.  A head whose
         * scale is unusable has no defined attention: its rows are NaN.               */
        double ks = A->k_head_scales ? (double)A->k_head_scales[kvh] : A->k_scale;
        double vs = A->v_head_scales ? (double)A->v_head_scales[kvh] : A->v_scale;
        if (!scale_ok(ks) || !scale_ok(vs)) {
            for (int e = 0; e < A->d; ++e)
                A->out[(size_t)u * A->d + e] = NAN;
            A->wsum[u] = NAN;
            continue;
        }
        attn_job J;
        J.q_row = (const char *)A->q + ((size_t)r * A->hq + h) * A->d * elem_bytes(A->q_dtype);
        J.q_dtype = A->q_dtype;
        J.d = A->d;
        J.scale = A->scale;
        J.n = n;
        J.scores = scores;
        paged_ctx pc;
        contig_ctx cc;
        if (A->paged) {
            pc.k_pool = A->k; pc.v_pool = A->v; pc.dtype = A->dtype; pc.hkv = A->hkv;
            pc.d = A->d; pc.kv_head = kvh; pc.k_scale = ks; pc.v_scale = vs;
            pc.table_row = A->tables + (size_t)b * A->max_blocks;
            J.key = paged_key; J.val = paged_val; J.ctx = &pc;
        } else {
            cc.k = A->k; cc.v = A->v; cc.dtype = A->dtype; cc.hkv = A->hkv; cc.d = A->d;
            cc.s_max = A->s_max; cc.seq = b; cc.kv_head = kvh;
            cc.k_scale = ks; cc.v_scale = vs;
            J.key = contig_key; J.val = contig_val; J.ctx = &cc;
        }
        attend(&J, A->out + (size_t)u * A->d, A->wsum + u);
    }
    free(scores);
    return NULL;
}

static int run_decode(decode_args *A)
{
    if (A->nthreads < 1)
        A->nthreads = 1;
    if (A->nthreads > 1024)
        A->nthreads = 1024;
    pthread_t th[1024];
    worker_arg wa[1024];
    int started = 0, rc = 0;
    for (int i = 0; i < A->nthreads; ++i) {
        wa[i].A = A;
        wa[i].tid = i;
        if (A->nthreads == 1)
            break;
        if (pthread_create(&th[i], NULL, decode_worker, &wa[i]) != 0) {
            rc = -3;
            break;
        }
        ++started;
    }
    if (A->nthreads == 1)
        return decode_worker(&wa[0]) ? -3 : 0;
    for (int i = 0; i < started; ++i) {
        void *r = NULL;
        pthread_join(th[i], &r);
        if (r)
            rc = -3;
    }
    return rc;
}

static int check_common(int dtype, int B, int hq, int hkv, int d)
{
    if (dtype < ORACLE_F32 || dtype > ORACLE_FP8_E4M3)
        return -1;
    if (B < 0 || hq <= 0 || hkv <= 0 || d <= 0 || hq % hkv != 0)
        return -1;
    return 0;
}

/* Paged decode attention.  q has type q_dtype; K/V are stored as kv_dtype and read
 * as stored value x k_scale (x v_scale); for fp8 pools q_dtype is f16 or bf16, for the
 * others it equals kv_dtype and the scales are 1.  out [B][Hq][d] and wsum [B][Hq]
 * (sum of the normalised softmax weights of each row) are fp64.  Returns 0, or -1 on
 * bad shapes, -2 when a context length or a block-table entry it would read is out
 * of range.                                                                          */
int oracle_decode_paged_hs(const void *q, int q_dtype, const void *k_pool, const void *v_pool,
                           int kv_dtype, double k_scale, double v_scale,
                           const float *k_head_scales, const float *v_head_scales, int num_seqs,
                           int num_q_heads, int num_kv_heads, int head_dim, int num_blocks,
                           const int32_t *block_tables, int max_blocks_per_seq,
                           const int32_t *context_lens, float scale, double *out, double *wsum,
                           int num_threads)
{
    if (check_common(kv_dtype, num_seqs, num_q_heads, num_kv_heads, head_dim) ||
        check_common(q_dtype, num_seqs, num_q_heads, num_kv_heads, head_dim) ||
        q_dtype == ORACLE_FP8_E4M3)
        return -1;
    for (int b = 0; b < num_seqs; ++b) {
        int n = context_lens[b];
        if (n < 0 || n > max_blocks_per_seq * ORACLE_BLOCK)
            return -2;
        for (int lb = 0; lb < (n + ORACLE_BLOCK - 1) / ORACLE_BLOCK; ++lb) {
            int32_t p = block_tables[(size_t)b * max_blocks_per_seq + lb];
            if (p < 0 || p >= num_blocks)
                return -2;
        }
    }
    decode_args A = {1, q, k_pool, v_pool, kv_dtype, q_dtype, k_scale, v_scale, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, 0,
                     block_tables, context_lens, (double)scale, out, wsum, num_threads};
    A.k_head_scales = k_head_scales;
    A.v_head_scales = v_head_scales;
    return run_decode(&A);
}

/* The same with one scale pair for the whole pool.                                   */
int oracle_decode_paged_ex(const void *q, int q_dtype, const void *k_pool, const void *v_pool,
                           int kv_dtype, double k_scale, double v_scale, int num_seqs,
                           int num_q_heads, int num_kv_heads, int head_dim, int num_blocks,
                           const int32_t *block_tables, int max_blocks_per_seq,
                           const int32_t *context_lens, float scale, double *out, double *wsum,
                           int num_threads)
{
    return oracle_decode_paged_hs(q, q_dtype, k_pool, v_pool, kv_dtype, k_scale, v_scale, NULL,
                                  NULL, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                  num_blocks, block_tables, max_blocks_per_seq, context_lens,
                                  scale, out, wsum, num_threads);
}

/* Paged prefill attention (a prompt chunk, or several, over the paged cache).
 * LLM-101-CN "推理优化", section "Chunked Prefill": a chunk's queries attend to the
 * cached K/V of the earlier chunks joined with the chunk's own K/V, with the same
 * 1/sqrt(d_h)-scaled softmax; its mixed-batch section runs the requests of one batch
 * with different chunk lengths.  "Deep dive into vLLM 06", section 4.2: one forward
 * computes every position from its own known prefix, i.e. the causal rule.
 * Query rows of sequence b are q_start[b] .. q_start[b+1]-1 of q [T][Hq][d]
 * (q_start has B + 1 entries, non-decreasing, q_start[0] = 0, q_start[B] = T).  The
 * chunk is already in the pool, counted in context_lens[b]; its i-th query is token
 * ctx - q_len + i and attends to tokens 0 .. ctx - q_len + i.  A query with no key
 * (q_len > ctx) gives a zero row.  out [T][Hq][d], wsum [T][Hq] fp64.  Returns 0, -1
 * on bad shapes, -2 on an out-of-range context length, block-table entry or q_start.  */
int oracle_prefill_paged_hs(const void *q, int q_dtype, const void *k_pool, const void *v_pool,
                            int kv_dtype, double k_scale, double v_scale,
                            const float *k_head_scales, const float *v_head_scales,
                            int num_seqs, const int32_t *query_start, int num_q_heads,
                            int num_kv_heads, int head_dim, int num_blocks,
                            const int32_t *block_tables, int max_blocks_per_seq,
                            const int32_t *context_lens, float scale, double *out,
                            double *wsum, int num_threads)
{
    if (check_common(kv_dtype, num_seqs, num_q_heads, num_kv_heads, head_dim) ||
        check_common(q_dtype, num_seqs, num_q_heads, num_kv_heads, head_dim) ||
        q_dtype == ORACLE_FP8_E4M3 || num_seqs < 1)
        return -1;
    if (query_start[0] != 0)
        return -2;
    for (int b = 0; b < num_seqs; ++b) {
        int n = context_lens[b];
        if (query_start[b + 1] < query_start[b])
            return -2;
        if (n < 0 || n > max_blocks_per_seq * ORACLE_BLOCK)
            return -2;
        for (int lb = 0; lb < (n + ORACLE_BLOCK - 1) / ORACLE_BLOCK; ++lb) {
            int32_t p = block_tables[(size_t)b * max_blocks_per_seq + lb];
            if (p < 0 || p >= num_blocks)
                return -2;
        }
    }
    decode_args A = {1, q, k_pool, v_pool, kv_dtype, q_dtype, k_scale, v_scale, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, max_blocks_per_seq, 0,
                     block_tables, context_lens, (double)scale, out, wsum, num_threads,
                     query_start, query_start[num_seqs]};
    A.k_head_scales = k_head_scales;
    A.v_head_scales = v_head_scales;
    return run_decode(&A);
}

int oracle_prefill_paged_ex(const void *q, int q_dtype, const void *k_pool, const void *v_pool,
                            int kv_dtype, double k_scale, double v_scale, int num_seqs,
                            const int32_t *query_start, int num_q_heads, int num_kv_heads,
                            int head_dim, int num_blocks, const int32_t *block_tables,
                            int max_blocks_per_seq, const int32_t *context_lens, float scale,
                            double *out, double *wsum, int num_threads)
{
    return oracle_prefill_paged_hs(q, q_dtype, k_pool, v_pool, kv_dtype, k_scale, v_scale, NULL,
                                   NULL, num_seqs, query_start, num_q_heads, num_kv_heads,
                                   head_dim, num_blocks, block_tables, max_blocks_per_seq,
                                   context_lens, scale, out, wsum, num_threads);
}

/* Same with q and K/V all of one type and unit scales.                             */
int oracle_decode_paged(const void *q, const void *k_pool, const void *v_pool, int dtype,
                        int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                        int num_blocks, const int32_t *block_tables, int max_blocks_per_seq,
                        const int32_t *context_lens, float scale, double *out, double *wsum,
                        int num_threads)
{
    return oracle_decode_paged_ex(q, dtype, k_pool, v_pool, dtype, 1.0, 1.0, num_seqs,
                                  num_q_heads, num_kv_heads, head_dim, num_blocks, block_tables,
                                  max_blocks_per_seq, context_lens, scale, out, wsum,
                                  num_threads);
}

/* The same attention over an ordinary contiguous cache k, v [B][Hkv][S_max][d] of
 * kv_dtype (read as value x scale), q of q_dtype.                                     */
int oracle_decode_contig_hs(const void *q, int q_dtype, const void *k, const void *v,
                            int kv_dtype, double k_scale, double v_scale,
                            const float *k_head_scales, const float *v_head_scales,
                            int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                            int s_max, const int32_t *context_lens, float scale, double *out,
                            double *wsum, int num_threads)
{
    if (check_common(kv_dtype, num_seqs, num_q_heads, num_kv_heads, head_dim) ||
        check_common(q_dtype, num_seqs, num_q_heads, num_kv_heads, head_dim) ||
        q_dtype == ORACLE_FP8_E4M3)
        return -1;
    for (int b = 0; b < num_seqs; ++b)
        if (context_lens[b] < 0 || context_lens[b] > s_max)
            return -2;
    decode_args A = {0, q, k, v, kv_dtype, q_dtype, k_scale, v_scale, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, 0, 0, s_max, NULL, context_lens, (double)scale,
                     out, wsum, num_threads};
    A.k_head_scales = k_head_scales;
    A.v_head_scales = v_head_scales;
    return run_decode(&A);
}

int oracle_decode_contig_ex(const void *q, int q_dtype, const void *k, const void *v,
                            int kv_dtype, double k_scale, double v_scale, int num_seqs,
                            int num_q_heads, int num_kv_heads, int head_dim, int s_max,
                            const int32_t *context_lens, float scale, double *out,
                            double *wsum, int num_threads)
{
    return oracle_decode_contig_hs(q, q_dtype, k, v, kv_dtype, k_scale, v_scale, NULL, NULL,
                                   num_seqs, num_q_heads, num_kv_heads, head_dim, s_max,
                                   context_lens, scale, out, wsum, num_threads);
}

int oracle_decode_contig(const void *q, const void *k, const void *v, int dtype, int num_seqs,
                         int num_q_heads, int num_kv_heads, int head_dim, int s_max,
                         const int32_t *context_lens, float scale, double *out, double *wsum,
                         int num_threads)
{
    return oracle_decode_contig_ex(q, dtype, k, v, dtype, 1.0, 1.0, num_seqs, num_q_heads,
                                   num_kv_heads, head_dim, s_max, context_lens, scale, out,
                                   wsum, num_threads);
}

/* Cache append: new row i goes to slot s = slot_mapping[i], i.e. physical block
 * s / 16, row s % 16 (the page/offset split of "LLM应用 12 推理优化",
 * PagedKVCache.update, and the write-into-the-last-page rule of LLM-101-CN
 * "推理优化", KVCachePool.write_tokens).  A negative slot means "no row".
 * k_new, v_new: [T][Hkv][d] of act_dtype.  When the pool has the new rows' type the
 * bytes are copied unchanged.  An fp8 pool stores encode_e4m3(x / scale), the
 * division done in fp32 (the KV-cache write fused with quantisation that "Deep dive
 * into vLLM 06" lists among vLLM's fused kernels).  Returns -2 on a slot past the pool. */
int oracle_cache_append_hs(void *k_pool, void *v_pool, int kv_dtype, int act_dtype,
                           float k_scale, float v_scale, const float *k_head_scales,
                           const float *v_head_scales, int num_blocks, int num_kv_heads,
                           int head_dim, const void *k_new, const void *v_new,
                           const int32_t *slot_mapping, int num_tokens)
{
    if (check_common(kv_dtype, 1, num_kv_heads, num_kv_heads, head_dim) || num_tokens < 0 ||
        check_common(act_dtype, 1, num_kv_heads, num_kv_heads, head_dim))
        return -1;
    const int quantise = kv_dtype == ORACLE_FP8_E4M3;
    if (!quantise && act_dtype != kv_dtype)
        return -1;
    if (quantise && act_dtype != ORACLE_F16 && act_dtype != ORACLE_BF16)
        return -1;
    const size_t eb = elem_bytes(kv_dtype);
    for (int i = 0; i < num_tokens; ++i) {
        int32_t s = slot_mapping[i];
        if (s < 0)
            continue;
        if ((int64_t)s >= (int64_t)num_blocks * ORACLE_BLOCK)
            return -2;
        size_t blk = (size_t)(s / ORACLE_BLOCK), off = (size_t)(s % ORACLE_BLOCK);
        for (int h = 0; h < num_kv_heads; ++h) {
            /* the row's kv-head scale: its per-head entry, else the pool's            */
            float ks = k_head_scales ? k_head_scales[h] : k_scale;
            float vs = v_head_scales ? v_head_scales[h] : v_scale;
            for (int e = 0; e < head_dim; ++e) {
                size_t src = ((size_t)i * num_kv_heads + h) * head_dim + e;
                size_t kdst = ((blk * num_kv_heads + h) * ORACLE_BLOCK + off) * head_dim + e;
                size_t vdst = ((blk * num_kv_heads + h) * head_dim + e) * ORACLE_BLOCK + off;
                if (quantise) {
                    float kx = (float)widen_at(k_new, src, act_dtype);
                    float vx = (float)widen_at(v_new, src, act_dtype);
                    /* an unusable scale quantises to the NaN code                     */
                    ((uint8_t *)k_pool)[kdst] = scale_ok(ks) ? encode_e4m3(kx / ks) : 0x7F;
                    ((uint8_t *)v_pool)[vdst] = scale_ok(vs) ? encode_e4m3(vx / vs) : 0x7F;
                } else {
                    memcpy((char *)k_pool + kdst * eb, (const char *)k_new + src * eb, eb);
                    memcpy((char *)v_pool + vdst * eb, (const char *)v_new + src * eb, eb);
                }
            }
        }
    }
    return 0;
}

int oracle_cache_append_ex(void *k_pool, void *v_pool, int kv_dtype, int act_dtype,
                           float k_scale, float v_scale, int num_blocks, int num_kv_heads,
                           int head_dim, const void *k_new, const void *v_new,
                           const int32_t *slot_mapping, int num_tokens)
{
    return oracle_cache_append_hs(k_pool, v_pool, kv_dtype, act_dtype, k_scale, v_scale, NULL,
                                  NULL, num_blocks, num_kv_heads, head_dim, k_new, v_new,
                                  slot_mapping, num_tokens);
}

int oracle_cache_append(void *k_pool, void *v_pool, int dtype, int num_blocks,
                        int num_kv_heads, int head_dim, const void *k_new, const void *v_new,
                        const int32_t *slot_mapping, int num_tokens)
{
    return oracle_cache_append_ex(k_pool, v_pool, dtype, dtype, 1.0f, 1.0f, num_blocks,
                                  num_kv_heads, head_dim, k_new, v_new, slot_mapping,
                                  num_tokens);
}

/* Copy-on-write's copy: for each pair, block src of both pools is copied to block dst
 * as exact bytes (every kv-head; a block of a pool is Hkv * 16 * d elements).  Pairs
 * with an id outside the pool are skipped.                                           */
int oracle_copy_blocks(void *k_pool, void *v_pool, int dtype, int num_blocks, int num_kv_heads,
                       int head_dim, const int32_t *pairs, int num_pairs)
{
    if (check_common(dtype, 1, num_kv_heads, num_kv_heads, head_dim) || num_pairs < 0)
        return -1;
    const size_t bytes = (size_t)num_kv_heads * ORACLE_BLOCK * head_dim * elem_bytes(dtype);
    for (int i = 0; i < num_pairs; ++i) {
        int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
        if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks)
            continue;
        memmove((char *)k_pool + (size_t)dst * bytes, (const char *)k_pool + (size_t)src * bytes,
                bytes);
        memmove((char *)v_pool + (size_t)dst * bytes, (const char *)v_pool + (size_t)src * bytes,
                bytes);
    }
    return 0;
}
