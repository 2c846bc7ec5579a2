/*
 * CSA2 hot-path ORACLE: a plain, slow CPU statement of what the path computes.
 *
 * This file is test infrastructure.  Only the test-suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code, header, table or helper with the GPU library.
 *
 * Sources (the pages are cited by title and section):
 *   [R]  "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
 *        (the report), sections 2.3, 2.3.1, 2.3.2, 2.4.4, 4.2.1.
 *   [N4] reading note "DeepSeek V4.1 Flash: Pushing the Limits of KV Cache
 *        Compression" (papers.chlience.com), section
 *        "CSA2：共享存储、刷新选择和逐层计算分别控制" (CSA2: shared storage,
 *        refreshed selection and per-layer computation), its mode table and
 *        its decoder search-range / read-range table.
 *   [C3] course notes "3. 通用基础设施" (3. General infrastructure),
 *        section 3.2.2 SWA Bounded Replay, window equation.
 *   OCP  OCP Microscaling Formats (MX) v1.0 -- [R] 2.4.4 names "OCP-standard
 *        MXFP4" for the FP4 caches.
 *
 * Where the pages leave a step open, the plain reading is taken; every such
 * reading is listed in the design notes of the repository.  The readings that
 * shape this file:
 *   - index score  score(t,j) = 2^(ek_j-127) * sum_h w[t,h] * ReLU(d_h * 2^(eq_th-127)),
 *     d_h = exact dot product of the decoded q and k rows ("lightweight indexer
 *     that scores the main KV entries using indexer Q and indexer K", [R] 2.3;
 *     the per-head weights w come with the indexer of DeepSeek-V4's CSA, which
 *     [R] 2.3.1 says Full mode inherits).  The head sum is evaluated in fp32 as
 *     acc = +0; for h = 0..H-1: acc = fmaf(w[t,h], r_h, acc)  (one IEEE fused
 *     multiply-add per head, round to nearest even).  That order is a convention.
 *   - index score in the report's indexer format (OCP MXFP4 for indexer q and
 *     indexer K, [R] 2.4.4: one E8M0 per 32 channels on both sides): the block
 *     scales enter the dot product, d_h = sum_b 2^(eq_thb + ek_jb - 254) *
 *     (dot of block b), exact; then r_h = ReLU(d_h), the same fmaf head sum, and
 *     no per-entry factor after it.
 *   - Top-K: the first min(K, visible) entries under (score descending,
 *     position ascending); returned in ascending position order, -1 padded.
 *   - block pool: blocks of 8 aligned at position 0; a block's score is the
 *     maximum score over its visible positions; the first min(2048, #blocks)
 *     blocks under (block score descending, block ascending) are kept
 *     ([R] 2.3.2, [N4] decoder indexer paragraph).
 *   - attention: one softmax over the union of the selected entries and the
 *     SWA window, scale 1/sqrt(512), keys = values = the 512-channel latent.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -pthread (the explicit fmaf is the
 * only fused operation).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Formats (OCP MX v1.0; [R] 2.4.4)                                           */
/* ------------------------------------------------------------------------ */

/* E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
 * exponent 0 is subnormal: 0.5 * m. */
double orc_e2m1(uint8_t nibble) {
    int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E8M0: 2^(code-127); code 255 is NaN. */
double orc_e8m0(uint8_t code) {
    if (code == 255) return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* E4M3 "FN": sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
 * S.1111.111 is NaN, there are no infinities. */
double orc_e4m3(uint8_t code) {
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* bf16: the top 16 bits of an IEEE binary32. */
float orc_bf16(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ------------------------------------------------------------------------ */
/* Visibility ([R] 2.3: entry j of a ratio-m cache is built from the m tokens  */
/* jm .. jm+m-1, with no overlap between entries)                             */
/* ------------------------------------------------------------------------ */

/* Entry j is visible to the query at token position t when every token it
 * was built from is at or before t:  (j+1)*m - 1 <= t.  Returns how many of
 * the n_entries are visible (they are always a prefix 0..vis-1). */
int64_t orc_visible(int64_t n_entries, int64_t t, int m) {
    if (t < 0) return 0;
    int64_t v = (t + 1) / m;
    return v < n_entries ? v : n_entries;
}

/* ------------------------------------------------------------------------ */
/* Parallel-for over independent rows (no effect on any value)                */
/* ------------------------------------------------------------------------ */

typedef void (*row_fn)(void* ctx, int64_t i);
typedef struct { row_fn fn; void* ctx; int64_t n; int64_t next; pthread_mutex_t mu; } pool_t;

static void* pool_worker(void* p) {
    pool_t* P = (pool_t*)p;
    for (;;) {
        pthread_mutex_lock(&P->mu);
        int64_t i = P->next++;
        pthread_mutex_unlock(&P->mu);
        if (i >= P->n) break;
        P->fn(P->ctx, i);
    }
    return NULL;
}

static void parallel_for(int64_t n, int nthreads, row_fn fn, void* ctx) {
    if (nthreads <= 1 || n <= 1) {
        for (int64_t i = 0; i < n; ++i) fn(ctx, i);
        return;
    }
    if (nthreads > 512) nthreads = 512;
    pool_t P;
    P.fn = fn; P.ctx = ctx; P.n = n; P.next = 0;
    pthread_mutex_init(&P.mu, NULL);
    pthread_t th[512];
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, pool_worker, &P);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&P.mu);
}

/* ------------------------------------------------------------------------ */
/* Batch description shared by the calls below.                              */
/* ------------------------------------------------------------------------ */
/* row_seq[r]   : sequence of query row r
 * q_pos[r]     : token position t of query row r
 * entry_off[b] : first entry of sequence b in the packed caches; entry_off[n_seq] = total
 * ratio        : compression ratio m                                          */

/* ------------------------------------------------------------------------ */
/* Index score ([R] 2.3 indexer; [R] 2.3.1 Full/Reindex; [R] 2.3.2 pool)      */
/* ------------------------------------------------------------------------ */

enum { ORC_Q_FP4 = 0, ORC_Q_FP8 = 1, ORC_Q_MXFP4 = 2 };

typedef struct {
    const int32_t *row_seq, *q_pos;
    const int64_t* entry_off;
    int ratio, H, q_fmt;
    const uint8_t *q, *q_sc;
    const float* w;
    const uint8_t *k, *k_sc;
    const int32_t* cand;
    int64_t cand_stride;
    float* scores;
    int64_t score_stride, n_slots;
    int status;
} score_ctx;

/* Integer image of an indexer-q element: value * 2^qshift is an integer.
 * E2M1 values are multiples of 0.5 (qshift 1); E4M3 values are multiples of
 * 2^-9 (qshift 9). */
static int64_t q_int(const score_ctx* c, int64_t row, int h, int ch) {
    if (c->q_fmt == ORC_Q_FP4 || c->q_fmt == ORC_Q_MXFP4) {
        uint8_t byte = c->q[(row * c->H + h) * 64 + ch / 2];
        uint8_t nib = (ch & 1) ? (byte >> 4) : (byte & 15);
        return (int64_t)llround(orc_e2m1(nib) * 2.0);
    } else {
        uint8_t code = c->q[(row * c->H + h) * 128 + ch];
        return (int64_t)llround(orc_e4m3(code) * 512.0);
    }
}

static int64_t k_int(const score_ctx* c, int64_t e, int ch) {
    uint8_t byte = c->k[e * 64 + ch / 2];
    uint8_t nib = (ch & 1) ? (byte >> 4) : (byte & 15);
    return (int64_t)llround(orc_e2m1(nib) * 2.0);
}

/* The report's MXFP4 indexer format: q [T][H][64 B] with q_sc [T][H][4] and
 * K [N][64 B] with k_sc [N][4], one E8M0 per 32 channels on both sides (OCP
 * MX v1.0: a block's value is 2^(scale - 127) times its E2M1 elements).  Block
 * b of head h contributes 2^(eq + ek - 254) times its integer dot product / 4;
 * the blocks are summed exactly in integers at the smallest block exponent,
 * so d_h is the exact dot product of the decoded rows. */
static float score_one_mx(const score_ctx* c, int64_t r, int64_t e, const int64_t* qi, const int64_t* kv) {
    float acc = 0.0f;
    for (int h = 0; h < c->H; ++h) {
        int64_t part[4], mag[4];
        int ex[4], emin = 1 << 30;
        for (int b = 0; b < 4; ++b) {
            part[b] = 0;
            mag[b] = 0;
            for (int ch = 32 * b; ch < 32 * b + 32; ++ch) {
                const int64_t p = qi[h * 128 + ch] * kv[ch];
                part[b] += p;
                mag[b] += p < 0 ? -p : p;
            }
            ex[b] = (int)c->q_sc[(r * c->H + h) * 4 + b] + (int)c->k_sc[e * 4 + b] - 254;
            if (ex[b] < emin) emin = ex[b];
        }
        int64_t dot = 0, total = 0; /* d_h = dot * 2^(emin - 2) */
        for (int b = 0; b < 4; ++b) {
            int sh = ex[b] - emin;
            if (sh > 30) { ((score_ctx*)c)->status = 2; sh = 30; }
            dot += part[b] * ((int64_t)1 << sh);
            total += mag[b] * ((int64_t)1 << sh);
        }
        /* Every partial sum of the products, in any order, lies within the sum
         * of their magnitudes; below 2^24 units of the finest block grid each
         * is exact in binary32, so d_h is the same in every summation order.
         * Beyond it (block scales spread wide, even when the blocks cancel)
         * an accumulation in binary32 may round, and the score is not pinned. */
        if (total >= (1LL << 24)) ((score_ctx*)c)->status = 2;
        float d = (float)ldexp((double)dot, emin - 2);
        acc = fmaf(c->w[r * c->H + h], fmaxf(d, 0.0f), acc);
    }
    return acc;
}

/* score of one (query row, local entry j), or -inf when j is not visible. */
static float score_one(const score_ctx* c, int64_t r, int64_t j, const int64_t* qi /* [H][128] */) {
    int b = c->row_seq[r];
    int64_t n = c->entry_off[b + 1] - c->entry_off[b];
    int64_t vis = orc_visible(n, c->q_pos[r], c->ratio);
    if (j < 0 || j >= vis) return -INFINITY;
    int64_t e = c->entry_off[b] + j;
    int64_t kv[128];
    for (int ch = 0; ch < 128; ++ch) kv[ch] = k_int(c, e, ch);
    if (c->q_fmt == ORC_Q_MXFP4) return score_one_mx(c, r, e, qi, kv);
    int qshift = (c->q_fmt == ORC_Q_FP4) ? 1 : 9;
    float acc = 0.0f;
    for (int h = 0; h < c->H; ++h) {
        int64_t dot = 0, total = 0; /* exact: sum of integer products, and of their magnitudes */
        for (int ch = 0; ch < 128; ++ch) {
            const int64_t p = qi[h * 128 + ch] * kv[ch];
            dot += p;
            total += p < 0 ? -p : p;
        }
        /* d_h = dot * 2^-(qshift+1).  Every partial sum in any order lies
         * within the sum of magnitudes; below 2^24 units all of them are exact
         * in binary32, which the value bounds of both query formats ensure
         * (FP4: at most 128 * 144 units; E4M3 with |q| <= 16: at most
         * 128 * 8192 * 12 units). */
        if (total >= (1LL << 24)) ((score_ctx*)c)->status = 2;
        float d = (float)ldexp((double)dot, -(qshift + 1));
        float sq = (float)orc_e8m0(c->q_sc[r * c->H + h]);
        float rh = fmaxf(d, 0.0f) * sq; /* ReLU, then the query row's power-of-two scale */
        acc = fmaf(c->w[r * c->H + h], rh, acc);
    }
    return acc * (float)orc_e8m0(c->k_sc[e]);
}

/* Work item = (row, chunk of 65,536 slots): scores are independent of each
 * other, so splitting a row changes nothing but the number of busy threads. */
#define SCORE_CHUNK 65536

static void score_item(void* p, int64_t item) {
    const score_ctx* c = (const score_ctx*)p;
    int64_t nchunk = (c->n_slots + SCORE_CHUNK - 1) / SCORE_CHUNK;
    if (nchunk < 1) nchunk = 1;
    int64_t r = item / nchunk, ch0 = (item % nchunk) * SCORE_CHUNK;
    int b = c->row_seq[r];
    int64_t n = c->entry_off[b + 1] - c->entry_off[b];
    int64_t ns = c->cand ? c->n_slots : n;
    if (ch0 >= ns) return;
    int64_t ch1 = ch0 + SCORE_CHUNK < ns ? ch0 + SCORE_CHUNK : ns;
    int64_t* qi = (int64_t*)malloc(sizeof(int64_t) * (size_t)c->H * 128);
    for (int h = 0; h < c->H; ++h)
        for (int ch = 0; ch < 128; ++ch) qi[h * 128 + ch] = q_int(c, r, h, ch);
    float* out = c->scores + r * c->score_stride;
    for (int64_t s = ch0; s < ch1; ++s) {
        int64_t j = c->cand ? c->cand[r * c->cand_stride + s] : s;
        out[s] = score_one(c, r, j, qi);
    }
    free(qi);
}

/* Scores for every query row.  Without a candidate list, slot s of row r is
 * entry s of the row's sequence (slots 0..N_b-1 are written).  With one, slot
 * s is entry cand[r][s] (-1 = empty) and n_slots slots are written.  Entries
 * that are not visible, and empty slots, get -inf.  Returns 0, or 2 when a
 * dot product fell outside the range where binary32 holds it exactly. */
int orc_index_score(int64_t total_q, const int32_t* row_seq, const int32_t* q_pos, const int64_t* entry_off,
                    int ratio, int H, int q_fmt, const uint8_t* q, const uint8_t* q_sc, const float* w,
                    const uint8_t* k, const uint8_t* k_sc, const int32_t* cand, int64_t cand_stride,
                    int64_t n_slots, float* scores, int64_t score_stride, int nthreads) {
    /* without a candidate list the caller passes n_slots = the largest N_b */
    score_ctx c = {row_seq, q_pos, entry_off, ratio, H, q_fmt, q, q_sc, w, k, k_sc,
                   cand, cand_stride, scores, score_stride, n_slots, 0};
    int64_t nchunk = (n_slots + SCORE_CHUNK - 1) / SCORE_CHUNK;
    if (nchunk < 1) nchunk = 1;
    parallel_for(total_q * nchunk, nthreads, score_item, &c);
    return c.status;
}

/* ------------------------------------------------------------------------ */
/* Top-K ([R] 2.3: "selects the Top-K entries for each query"; K = 512 in     */
/* [R] 4.2.1).  Plain definition: sort everything, keep the first K.          */
/* ------------------------------------------------------------------------ */

typedef struct { float s; int64_t pos; } sp_t;

static int cmp_score_desc_pos_asc(const void* a, const void* b) {
    const sp_t* x = (const sp_t*)a;
    const sp_t* y = (const sp_t*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->pos < y->pos) ? -1 : (x->pos > y->pos);
}

static int cmp_i32_asc(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x < y) ? -1 : (x > y);
}

typedef struct {
    const float* scores;
    int64_t score_stride;
    const int64_t* n_valid; /* slots 0..n_valid[r]-1 take part */
    const int32_t* cand;    /* slot -> position, NULL: slot == position */
    int64_t cand_stride;
    int K;
    int32_t* idx;
} topk_ctx;

static void topk_row(void* p, int64_t r) {
    const topk_ctx* c = (const topk_ctx*)p;
    int64_t n = c->n_valid[r];
    sp_t* a = (sp_t*)malloc(sizeof(sp_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t s = 0; s < n; ++s) {
        a[s].s = c->scores[r * c->score_stride + s];
        a[s].pos = c->cand ? c->cand[r * c->cand_stride + s] : s;
    }
    qsort(a, (size_t)n, sizeof(sp_t), cmp_score_desc_pos_asc);
    int64_t take = n < c->K ? n : c->K;
    int32_t* out = c->idx + r * c->K;
    for (int64_t i = 0; i < take; ++i) out[i] = (int32_t)a[i].pos;
    qsort(out, (size_t)take, sizeof(int32_t), cmp_i32_asc);
    for (int64_t i = take; i < c->K; ++i) out[i] = -1;
    free(a);
}

void orc_topk(int64_t total_q, const float* scores, int64_t score_stride, const int64_t* n_valid,
              const int32_t* cand, int64_t cand_stride, int K, int32_t* idx, int nthreads) {
    topk_ctx c = {scores, score_stride, n_valid, cand, cand_stride, K, idx};
    parallel_for(total_q, nthreads, topk_row, &c);
}

/* ------------------------------------------------------------------------ */
/* Block pool ([R] 2.3.2 Hierarchical Sparse Indexer; [N4] decoder indexer:   */
/* both selections come from the same position scores and are independent)  */
/* ------------------------------------------------------------------------ */

typedef struct {
    const float* scores;
    int64_t score_stride;
    const int64_t* vis;
    int block, max_blocks;
    int32_t *blocks, *pool_pos, *pool_count;
} pool_ctx;

static void pool_row(void* p, int64_t r) {
    const pool_ctx* c = (const pool_ctx*)p;
    int64_t vis = c->vis[r];
    int64_t nb = (vis + c->block - 1) / c->block; /* blocks with at least one visible position */
    sp_t* a = (sp_t*)malloc(sizeof(sp_t) * (size_t)(nb > 0 ? nb : 1));
    for (int64_t b = 0; b < nb; ++b) {
        float m = -INFINITY;
        for (int64_t j = b * c->block; j < (b + 1) * c->block && j < vis; ++j) {
            float s = c->scores[r * c->score_stride + j];
            if (s > m) m = s;
        }
        a[b].s = m;
        a[b].pos = b;
    }
    qsort(a, (size_t)nb, sizeof(sp_t), cmp_score_desc_pos_asc);
    int64_t take = nb < c->max_blocks ? nb : c->max_blocks;
    int32_t* ob = c->blocks + r * c->max_blocks;
    for (int64_t i = 0; i < take; ++i) ob[i] = (int32_t)a[i].pos;
    qsort(ob, (size_t)take, sizeof(int32_t), cmp_i32_asc);
    for (int64_t i = take; i < c->max_blocks; ++i) ob[i] = -1;
    int32_t* op = c->pool_pos + r * (int64_t)c->max_blocks * c->block;
    int64_t cnt = 0;
    for (int64_t i = 0; i < take; ++i)
        for (int64_t j = (int64_t)ob[i] * c->block; j < ((int64_t)ob[i] + 1) * c->block && j < vis; ++j) op[cnt++] = (int32_t)j;
    for (int64_t i = cnt; i < (int64_t)c->max_blocks * c->block; ++i) op[i] = -1;
    c->pool_count[r] = (int32_t)cnt;
    free(a);
}

void orc_block_pool(int64_t total_q, const float* scores, int64_t score_stride, const int64_t* vis, int block,
                    int max_blocks, int32_t* blocks, int32_t* pool_pos, int32_t* pool_count, int nthreads) {
    pool_ctx c = {scores, score_stride, vis, block, max_blocks, blocks, pool_pos, pool_count};
    parallel_for(total_q, nthreads, pool_row, &c);
}

/* ------------------------------------------------------------------------ */
/* Gather + dequantise ([R] 2.4.4: cached values are dequantised before       */
/* attention; [N4] Figure 4 reading: "Selection" reads the selected entries)  */
/* ------------------------------------------------------------------------ */

/* Main-KV entry e, channel c, for the two scale formats:
 *   fmt 0 (OCP MXFP4):  E2M1(kv[e][c]) * 2^(sc[e][c/32] - 127), 16 scale bytes per row;
 *   fmt 1 ([R] 2.4.4):  E2M1(kv[e][c]) * E4M3(sc[e][c/16]), 32 scale bytes per row
 *                       (NVFP4's layout without its second-level global scale).
 * Either product has at most six significant bits, so it is exact in bf16. */
static double kv_value(const uint8_t* kv, const uint8_t* kv_sc, int kv_fmt, int64_t e, int ch) {
    uint8_t byte = kv[e * 256 + ch / 2];
    uint8_t nib = (ch & 1) ? (byte >> 4) : (byte & 15);
    if (kv_fmt == 1) return orc_e2m1(nib) * orc_e4m3(kv_sc[e * 32 + ch / 16]);
    return orc_e2m1(nib) * orc_e8m0(kv_sc[e * 16 + ch / 32]);
}

/* out[r][s][c] as bf16 bits; rows for idx == -1 are zero.  The value has at
 * most two significant bits with an E8M0 scale and at most six with an E4M3
 * scale, so it is exact in bf16 either way: the bits are those of the
 * binary32 value with the low half dropped (which is zero). */
void orc_gather_dequant(int64_t total_q, const int32_t* row_seq, const int64_t* entry_off, const uint8_t* kv,
                        const uint8_t* kv_sc, int kv_fmt, const int32_t* idx, int K, uint16_t* out) {
    for (int64_t r = 0; r < total_q; ++r)
        for (int s = 0; s < K; ++s) {
            int32_t j = idx[r * K + s];
            uint16_t* o = out + (r * K + s) * 512;
            for (int ch = 0; ch < 512; ++ch) {
                if (j < 0) { o[ch] = 0; continue; }
                float f = (float)kv_value(kv, kv_sc, kv_fmt, entry_off[row_seq[r]] + j, ch);
                uint32_t u;
                memcpy(&u, &f, 4);
                o[ch] = (uint16_t)(u >> 16);
            }
        }
}

/* ------------------------------------------------------------------------ */
/* Sparse latent attention ([R] 2.3: each query attends to the selected       */
/* entries together with the layer-local SWA KV; [N4] Figure 4 reading: the   */
/* selected main KV is concatenated with the SWA KV for core attention;      */
/* [C3] 3.2.2: query i sees SWA keys [max(s, i-W+1), i])                      */
/* ------------------------------------------------------------------------ */

typedef struct {
    const int32_t *row_seq, *q_pos;
    const int64_t* entry_off;
    const uint16_t* q; /* [total_q][Hm][512] bf16 */
    int Hm;
    const uint8_t *kv, *kv_sc;
    int kv_fmt;
    const int32_t* idx;
    int K;
    const void* swa; /* swa_fmt 0: [rows][512] bf16; 1: [rows][528] MXFP8 (512 E4M3 codes, 16 E8M0 scales) */
    int swa_fmt;
    const int64_t* swa_row_off;
    const int32_t* swa_pos0;
    int W;
    const int32_t* replay_s;
    double scale;
    float *out, *lse;
} attn_ctx;

static void attn_row(void* p, int64_t r) {
    const attn_ctx* c = (const attn_ctx*)p;
    int b = c->row_seq[r];
    int64_t t = c->q_pos[r];
    int64_t s0 = c->replay_s ? c->replay_s[b] : 0;
    int64_t u_lo = t - c->W + 1;
    if (u_lo < s0) u_lo = s0;
    int64_t n_swa = t - u_lo + 1;
    if (n_swa < 0) n_swa = 0;
    int64_t nk = c->K + n_swa;
    double* keys = (double*)malloc(sizeof(double) * (size_t)nk * 512);
    int64_t n = 0;
    for (int s = 0; s < c->K; ++s) {
        int32_t j = c->idx[r * c->K + s];
        if (j < 0) continue;
        for (int ch = 0; ch < 512; ++ch)
            keys[n * 512 + ch] = kv_value(c->kv, c->kv_sc, c->kv_fmt, c->entry_off[b] + j, ch);
        ++n;
    }
    for (int64_t u = u_lo; u <= t; ++u) {
        int64_t row = c->swa_row_off[b] + (u - c->swa_pos0[b]);
        for (int ch = 0; ch < 512; ++ch) {
            if (c->swa_fmt == 1) { /* OCP MXFP8: E4M3 element times the E8M0 scale of its 32 channels */
                const uint8_t* rb = (const uint8_t*)c->swa + row * 528;
                keys[n * 512 + ch] = orc_e4m3(rb[ch]) * orc_e8m0(rb[512 + ch / 32]);
            } else {
                keys[n * 512 + ch] = (double)orc_bf16(((const uint16_t*)c->swa)[row * 512 + ch]);
            }
        }
        ++n;
    }
    double* logit = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int h = 0; h < c->Hm; ++h) {
        const uint16_t* qh = c->q + (r * c->Hm + h) * 512;
        double mx = -INFINITY;
        for (int64_t i = 0; i < n; ++i) {
            double d = 0.0;
            for (int ch = 0; ch < 512; ++ch) d += (double)orc_bf16(qh[ch]) * keys[i * 512 + ch];
            logit[i] = d * c->scale;
            if (logit[i] > mx) mx = logit[i];
        }
        double den = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            logit[i] = exp(logit[i] - mx); /* now the unnormalised weight of key i */
            den += logit[i];
        }
        float* o = c->out + (r * c->Hm + h) * 512;
        for (int ch = 0; ch < 512; ++ch) {
            double acc = 0.0;
            for (int64_t i = 0; i < n; ++i) acc += logit[i] * keys[i * 512 + ch];
            o[ch] = n > 0 ? (float)(acc / den) : 0.0f;
        }
        if (c->lse) c->lse[r * c->Hm + h] = n > 0 ? (float)(mx + log(den)) : -INFINITY;
    }
    free(logit);
    free(keys);
}

void orc_sparse_attn(int64_t total_q, const int32_t* row_seq, const int32_t* q_pos, const int64_t* entry_off,
                     const uint16_t* q, int Hm, const uint8_t* kv, const uint8_t* kv_sc, int kv_fmt, const int32_t* idx,
                     int K,
                     const void* swa, int swa_fmt, const int64_t* swa_row_off, const int32_t* swa_pos0, int W,
                     const int32_t* replay_s, double scale, float* out, float* lse, int nthreads) {
    attn_ctx c = {row_seq, q_pos, entry_off, q, Hm, kv, kv_sc, kv_fmt, idx, K, swa, swa_fmt, swa_row_off, swa_pos0, W, replay_s,
                  scale, out, lse};
    parallel_for(total_q, nthreads, attn_row, &c);
}

/* ------------------------------------------------------------------------ */
/* Cache append ([R] 2.4.4: the main KV is quantised after RoPE, all 512     */
/* channels including the rotated part; [R] 4.2.1: RoPE sub-dimension 64).   */
/* ------------------------------------------------------------------------ */
/* Readings: the rotated part is channels 448..511, pairs (448 + 2i, 449 + 2i)
 * turned by the caller's angle of pair i (cos, sin given per entry), each
 * output one fp32 product difference or sum with no fused multiply-add.  The
 * quantiser's decisions are taken in fp32 on correctly rounded quotients:
 *   E4M3/16 (kv_fmt 1): X = E4M3(fl32(amax / 6)) to nearest even (2^-9 where
 *     that is 0), codes E2M1(fl32(x / X)) to nearest even, saturating at 6;
 *   MXFP4/32 (kv_fmt 0, OCP MX v1.0): X = 2^(floor(log2 amax) - 2), at least
 *     2^-127 (2^0 for an all-zero block), codes E2M1(x / X) to nearest even,
 *     saturating at 6. */

/* nearest of a finite set of non-negative grid values (ties to the even
 * code, i.e. the one whose last mantissa bit is 0) -- written as a search
 * over the grid so that it follows the definition rather than a bit trick */
static int nearest_code(double a, const double* grid, int n) {
    int best = 0;
    for (int i = 1; i < n; ++i) {
        double db = fabs(a - grid[best]), di = fabs(a - grid[i]);
        if (di < db || (di == db && (i & 1) == 0 && (best & 1) == 1)) best = i;
    }
    return best;
}

static uint8_t e2m1_rne(float q) {
    static const double g[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    int c = nearest_code(fabs((double)q), g, 8); /* beyond 6 the nearest is 6: saturation */
    return (uint8_t)(c | (q < 0.0f ? 8 : 0));
}

static uint8_t e4m3_rne_pos(float q) { /* q >= 0; codes 0..126 (126 = 448) */
    static double g[127];
    static int ready = 0;
    if (!ready) { for (int i = 0; i < 127; ++i) g[i] = orc_e4m3((uint8_t)i); ready = 1; }
    return (uint8_t)nearest_code((double)q, g, 127);
}

static int floor_log2_f(float a) { int e; frexpf(a, &e); return e - 1; }

/* RoPE on one latent v[512] in place: pair i = (448 + 2i, 449 + 2i) turned by
 * cs_e[2i] = cos, cs_e[2i + 1] = sin of its angle, each product rounded to
 * fp32 on its own, then one rounded difference or sum. */
static void rope_latent(float* v, const float* cs_e) {
    for (int i = 0; i < 32; ++i) {
        float a = v[448 + 2 * i], b = v[449 + 2 * i];
        float co = cs_e[2 * i], si = cs_e[2 * i + 1];
        float ac = a * co, bs = b * si, as = a * si, bc = b * co;
        v[448 + 2 * i] = ac - bs;
        v[449 + 2 * i] = as + bc;
    }
}

/* Append n entries: x [n][512] fp32 latents before RoPE, cs [n][32][2] the
 * cos and sin of each pair's angle, dst [n] the cache row of each entry.
 * Writes kv_fp4 [rows][256] and kv_sc [rows][16] (kv_fmt 0) or [rows][32]
 * (kv_fmt 1).  Returns 0, or 1 for a bad format or a row outside [0, rows). */
int orc_kv_append(int64_t n, const float* x, const float* cs, const int64_t* dst, int kv_fmt, int64_t rows,
                  uint8_t* kv_fp4, uint8_t* kv_sc) {
    if (kv_fmt != 0 && kv_fmt != 1) return 1;
    for (int64_t e = 0; e < n; ++e) {
        if (dst[e] < 0 || dst[e] >= rows) return 1;
        float v[512];
        for (int c = 0; c < 512; ++c) v[c] = x[e * 512 + c];
        rope_latent(v, cs + e * 64);
        uint8_t* codes = kv_fp4 + dst[e] * 256;
        int bl = kv_fmt == 1 ? 16 : 32;
        for (int b0 = 0; b0 < 512; b0 += bl) {
            float amax = 0.0f;
            for (int c = b0; c < b0 + bl; ++c) amax = fmaxf(amax, fabsf(v[c]));
            float X;
            if (kv_fmt == 1) {
                uint8_t sc = e4m3_rne_pos(amax / 6.0f);
                if (sc == 0) sc = 1;
                kv_sc[dst[e] * 32 + b0 / 16] = sc;
                X = (float)orc_e4m3(sc);
            } else {
                int se = amax > 0.0f ? floor_log2_f(amax) - 2 : 0;
                if (se < -127) se = -127; /* the E8M0 range */
                kv_sc[dst[e] * 16 + b0 / 32] = (uint8_t)(se + 127);
                X = ldexpf(1.0f, se);
            }
            for (int c = b0; c < b0 + bl; c += 2) {
                uint8_t lo = e2m1_rne(v[c] / X), hi = e2m1_rne(v[c + 1] / X);
                codes[c / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Compressor (reading note "DeepSeek V4.1 Flash: Pushing the Limits of KV   */
/* Cache Compression": C_l = H W^KV are the KV entries and Z_l = H W^Z their */
/* compression weights; CSA2 drops V4's overlapping windows and absolute     */
/* position embedding).  Reading: entry j combines its m tokens jm..jm+m-1,  */
/* per channel, with the softmax over those tokens of Z:                     */
/*   e[j][c] = sum_i exp(Z[jm+i][c]) C[jm+i][c] / sum_i exp(Z[jm+i][c]).     */
/* In double, rounded to float at the end.                                   */
/* ------------------------------------------------------------------------ */
int orc_compress(int64_t n_entries, int m, const float* c_tok, const float* z_tok, float* out) {
    if (n_entries < 0 || m < 1) return 1;
    for (int64_t j = 0; j < n_entries; ++j)
        for (int c = 0; c < 512; ++c) {
            double mx = -INFINITY;
            for (int i = 0; i < m; ++i) mx = fmax(mx, (double)z_tok[(j * m + i) * 512 + c]);
            double num = 0.0, den = 0.0;
            for (int i = 0; i < m; ++i) {
                double w = exp((double)z_tok[(j * m + i) * 512 + c] - mx);
                num += w * (double)c_tok[(j * m + i) * 512 + c];
                den += w;
            }
            out[j * 512 + c] = (float)(num / den);
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Indexer-K projection (reading note "DeepSeek V4.1 Flash: Pushing the      */
/* Limits of KV Cache Compression", configuration section: indexer K is      */
/* projected directly from the main KV; [R] 2.4.4: indexer keys in MXFP4).   */
/* Readings: y[o] = sum_k x[k] W[k][o] over the 512 channels of the entry as */
/* stored before quantisation (after RoPE: when cs is given, x is the entry  */
/* before RoPE and is first turned as the append turns it), evaluated as the */
/* fp32 chain acc = +0;                                                      */
/* acc = fmaf(x[k], W[k][o], acc) for k ascending (a convention, like the    */
/* head sum); then E2M1 codes with the OCP MX scale 2^(floor(log2 amax) - 2) */
/* (at least 2^-127; 1 for an all-zero block) per row (k_fmt 0: the default  */
/* layout, one E8M0 per row) or per 32 channels (k_fmt 1: MXFP4), to nearest */
/* even, saturating at 6.                                                    */
/* ------------------------------------------------------------------------ */
int orc_index_k_project(int64_t n, const float* x, const float* cs /* [n][32][2] or NULL */, const float* W,
                        const int64_t* dst, int k_fmt, int64_t rows, uint8_t* k_fp4, uint8_t* k_sc,
                        float* y_out /* [n][128] or NULL */) {
    if (k_fmt != 0 && k_fmt != 1) return 1;
    for (int64_t e = 0; e < n; ++e) {
        if (dst[e] < 0 || dst[e] >= rows) return 1;
        float v[512];
        for (int c = 0; c < 512; ++c) v[c] = x[e * 512 + c];
        if (cs) rope_latent(v, cs + e * 64);
        float y[128];
        for (int o = 0; o < 128; ++o) {
            float acc = 0.0f;
            for (int k = 0; k < 512; ++k) acc = fmaf(v[k], W[k * 128 + o], acc);
            y[o] = acc;
            if (y_out) y_out[e * 128 + o] = acc;
        }
        int bl = k_fmt == 1 ? 32 : 128;
        for (int b0 = 0; b0 < 128; b0 += bl) {
            float amax = 0.0f;
            for (int c = b0; c < b0 + bl; ++c) amax = fmaxf(amax, fabsf(y[c]));
            int se = amax > 0.0f ? floor_log2_f(amax) - 2 : 0;
            if (se < -127) se = -127;
            if (k_fmt == 1) k_sc[dst[e] * 4 + b0 / 32] = (uint8_t)(se + 127);
            else k_sc[dst[e]] = (uint8_t)(se + 127);
            for (int c = b0; c < b0 + bl; c += 2) {
                uint8_t lo = e2m1_rne(ldexpf(y[c], -se)), hi = e2m1_rne(ldexpf(y[c + 1], -se));
                k_fp4[dst[e] * 64 + c / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* RoPE and cast around attention (the report's kernel flow names a fused    */
/* "RoPE-attention-RoPE-cast" kernel: the query is rotated before attention, */
/* the output's rotated part is turned back after it, and the result is     */
/* cast).  Reading: the rotated channels and pairs of the append (448..511,  */
/* pairs (448 + 2i, 449 + 2i), caller-given cos/sin per row and pair; with   */
/* `inverse` the angle is negated: sin -> -sin), fp32 products without       */
/* fusion, then every channel to bf16 to nearest even.                      */
/* ------------------------------------------------------------------------ */
/* binary32 -> bf16 (binary32's sign and 8-bit exponent, 7 stored fraction
 * bits) to nearest, ties to even, written from the format: a finite value is
 * a multiple of its binade's bf16 spacing 2^(e-7) (e = max(floor(log2|x|),
 * -126), the subnormal spacing below 2^-126); the multiple is rounded to the
 * nearest integer, ties to the even one, and a result of 2^128 or more is an
 * infinity.  Infinities stay.  A NaN stays a NaN: sign and leading payload
 * bits kept, quiet bit set. */
static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);
    if (isinf(f)) return (uint16_t)(sign | 0x7F80u);
    const double a = fabs((double)f);
    if (a == 0.0) return sign;
    int e = ilogb(a);
    if (e < -126) e = -126;
    const double unit = ldexp(1.0, e - 7);
    const double q = a / unit;          /* exact: a has at most 24 significant bits */
    double r = floor(q);
    const double frac = q - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) == 1.0)) r += 1.0;
    const double v = r * unit;
    if (v >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    const float vf = (float)v;          /* exact: v has at most 8 significant bits */
    uint32_t vb;
    memcpy(&vb, &vf, 4);
    return (uint16_t)(sign | (vb >> 16));
}

int orc_rope_cast(int64_t n_rows, int heads, const float* in, const float* cs, int inverse, uint16_t* out) {
    if (n_rows < 0 || heads < 1) return 1;
    for (int64_t r = 0; r < n_rows; ++r)
        for (int h = 0; h < heads; ++h) {
            const float* v = in + (r * heads + h) * 512;
            uint16_t* o = out + (r * heads + h) * 512;
            for (int c = 0; c < 448; ++c) o[c] = f32_to_bf16_rne(v[c]);
            for (int i = 0; i < 32; ++i) {
                float a = v[448 + 2 * i], b = v[449 + 2 * i];
                float co = cs[(r * 32 + i) * 2], si = cs[(r * 32 + i) * 2 + 1];
                if (inverse) si = -si;
                float ac = a * co, bs = b * si, as = a * si, bc = b * co;
                o[448 + 2 * i] = f32_to_bf16_rne(ac - bs);
                o[449 + 2 * i] = f32_to_bf16_rne(as + bc);
            }
        }
    return 0;
}
