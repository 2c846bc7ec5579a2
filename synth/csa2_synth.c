/*
 * Seeded synthetic inputs for the CSA2 hot path: shared by the GPU tests, the
 * benchmark and the CPU oracle's tests as *input data*.  Nothing here computes
 * any step of the method (no scoring, selection, dequantisation or attention);
 * it only draws random numbers and encodes them into the cache formats.
 *
 * Random numbers: a counter-based generator.  Element i of tensor `tid` under
 * seed s is  h = mix(mix(s + GOLDEN * (tid + 1)) + i)  with mix() the SplitMix64
 * finaliser (Steele, Lea, Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014).  The output therefore does not depend on how the
 * work is split over threads.
 *   U(0,1)  = (h >> 40) * 2^-24
 *   N(0,1)  = Box-Muller on u1 = ((h >> 40) + 1) * 2^-24, u2 = ((h >> 16) & 0xFFFFFF) * 2^-24
 *
 * Encoders (the OCP Microscaling Formats v1.0 spec, which the report names as
 * "OCP-standard MXFP4"):
 *   E2M1 code  s<<3 | e<<1 | m ; element 2i in the low nibble of byte i.
 *   E8M0 code  e -> 2^(e-127); a block's scale X = 2^(floor(log2 amax) - emax)
 *              with emax = 2 for E2M1 and 3 (a stricter bound, |x/X| < 16)
 *              for the E4M3 indexer queries.
 *   rounding   round-to-nearest-even onto the target grid, saturating.
 *   bf16       round-to-nearest-even of the fp32 value.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

static inline uint64_t hash3(uint64_t seed, uint64_t tid, uint64_t i) {
    return mix64(mix64(seed + GOLDEN * (tid + 1)) + i);
}

static inline double unif(uint64_t h) { return (double)(h >> 40) * 0x1p-24; }

static inline double normal(uint64_t h) {
    double u1 = (double)((h >> 40) + 1) * 0x1p-24;
    double u2 = (double)((h >> 16) & 0xFFFFFFULL) * 0x1p-24;
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

/* ---- encoders ---------------------------------------------------------- */

/* |v| rounded to nearest-even on the E2M1 magnitude grid {0,.5,1,1.5,2,3,4,6}
 * (saturating), returned as the 3-bit magnitude code e<<1|m. */
static uint8_t e2m1_mag_code(double a) {
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    if (a >= 6.0) return 7;
    int lo = 0;
    while (lo < 7 && grid[lo + 1] <= a) ++lo;
    if (lo == 7) return 7;
    double dlo = a - grid[lo], dhi = grid[lo + 1] - a;
    if (dlo < dhi) return (uint8_t)lo;
    if (dhi < dlo) return (uint8_t)(lo + 1);
    return (uint8_t)((lo & 1) ? lo + 1 : lo); /* tie: even mantissa bit */
}

static uint8_t e2m1_code(double v) {
    uint8_t c = e2m1_mag_code(fabs(v));
    return (uint8_t)(((v < 0 && c != 0) ? 8 : 0) | c);
}

/* E4M3 (OCP "FN" variant: bias 7, no infinities, max 448) round-to-nearest-even. */
static uint8_t e4m3_code(double v) {
    uint8_t s = v < 0 ? 0x80 : 0;
    double a = fabs(v);
    if (a >= 448.0) return (uint8_t)(s | 0x7E);
    /* subnormals: multiples of 2^-9 below 2^-6 */
    if (a < 0x1p-6) {
        double q = a * 512.0; /* units of 2^-9 */
        double f = floor(q), r = q - f;
        long m = (long)f;
        if (r > 0.5 || (r == 0.5 && (m & 1))) ++m;
        if (m == 8) return (uint8_t)(s | 0x08); /* rounds up to min normal */
        return (uint8_t)(s | m);
    }
    int e;
    frexp(a, &e); /* a = f * 2^e, f in [0.5,1) -> unbiased exponent e-1 */
    int ue = e - 1;
    double q = ldexp(a, 3 - ue); /* in [8,16) */
    double f = floor(q), r = q - f;
    long m = (long)f;
    if (r > 0.5 || (r == 0.5 && (m & 1))) ++m;
    if (m == 16) { m = 8; ++ue; }
    int be = ue + 7;
    if (be > 15 || (be == 15 && m - 8 == 7)) return (uint8_t)(s | 0x7E);
    return (uint8_t)(s | (be << 3) | (m - 8));
}

/* value of an E4M3 code (finite codes only) */
static double e4m3_value(uint8_t c) {
    int e = (c >> 3) & 15, m = c & 7;
    double mag = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
    return (c & 0x80) ? -mag : mag;
}

static uint16_t bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* floor(log2(a)) for a > 0, exactly (frexp is exact). */
static int ilog2_floor(double a) {
    int e;
    frexp(a, &e);
    return e - 1;
}

/* ---- threaded row loops -------------------------------------------------- */

typedef struct {
    int kind; /* 0 normal f32, 1 uniform f32, 2 bf16 normal, 3 mxfp4 rows, 4 e4m3 rows, 5 e2m1 + e4m3/16 rows */
    uint64_t seed, tid;
    int64_t row0, nrows;
    int row_len, block;
    void* out;
    uint8_t* scales;
    int64_t lo, hi; /* [lo,hi) range of rows (kind 3,4) or elements handled */
} job_t;

static void run_range(const job_t* j, int64_t lo, int64_t hi) {
    switch (j->kind) {
    case 0: {
        float* o = (float*)j->out;
        for (int64_t i = lo; i < hi; ++i) o[i] = (float)normal(hash3(j->seed, j->tid, (uint64_t)(j->row0 + i)));
        break;
    }
    case 1: {
        float* o = (float*)j->out;
        for (int64_t i = lo; i < hi; ++i) o[i] = (float)unif(hash3(j->seed, j->tid, (uint64_t)(j->row0 + i)));
        break;
    }
    case 2: {
        uint16_t* o = (uint16_t*)j->out;
        for (int64_t i = lo; i < hi; ++i)
            o[i] = bf16_rne((float)normal(hash3(j->seed, j->tid, (uint64_t)(j->row0 + i))));
        break;
    }
    case 3: { /* MXFP4 rows: row_len values, one E8M0 scale per `block` values */
        uint8_t* o = (uint8_t*)j->out;
        int nb = j->row_len / j->block;
        double* v = (double*)malloc(sizeof(double) * (size_t)j->row_len);
        for (int64_t r = lo; r < hi; ++r) {
            uint64_t base = (uint64_t)(j->row0 + r) * (uint64_t)j->row_len;
            for (int c = 0; c < j->row_len; ++c) v[c] = normal(hash3(j->seed, j->tid, base + (uint64_t)c));
            uint8_t* orow = o + r * (j->row_len / 2);
            for (int b = 0; b < nb; ++b) {
                double amax = 0.0;
                for (int c = 0; c < j->block; ++c) amax = fmax(amax, fabs(v[b * j->block + c]));
                int se = amax > 0.0 ? ilog2_floor(amax) - 2 : 0;
                if (se < -127) se = -127;
                if (se > 127) se = 127;
                j->scales[r * nb + b] = (uint8_t)(se + 127);
                for (int c = 0; c < j->block; c += 2) {
                    int idx = b * j->block + c;
                    uint8_t lo4 = e2m1_code(ldexp(v[idx], -se));
                    uint8_t hi4 = e2m1_code(ldexp(v[idx + 1], -se));
                    orow[idx / 2] = (uint8_t)(lo4 | (hi4 << 4));
                }
            }
        }
        free(v);
        break;
    }
    case 4: { /* E4M3 rows with one E8M0 scale per row, |x/X| < 16 */
        uint8_t* o = (uint8_t*)j->out;
        double* v = (double*)malloc(sizeof(double) * (size_t)j->row_len);
        for (int64_t r = lo; r < hi; ++r) {
            uint64_t base = (uint64_t)(j->row0 + r) * (uint64_t)j->row_len;
            double amax = 0.0;
            for (int c = 0; c < j->row_len; ++c) {
                v[c] = normal(hash3(j->seed, j->tid, base + (uint64_t)c));
                amax = fmax(amax, fabs(v[c]));
            }
            int se = amax > 0.0 ? ilog2_floor(amax) - 3 : 0;
            j->scales[r] = (uint8_t)(se + 127);
            for (int c = 0; c < j->row_len; ++c) o[r * j->row_len + c] = e4m3_code(ldexp(v[c], -se));
        }
        free(v);
        break;
    }
    case 7: { /* MXFP8 rows: E4M3 elements with one E8M0 scale per 32, stored inline:
               * row = row_len code bytes then row_len/32 scale bytes; X = 2^(floor(log2 amax) - 8) */
        uint8_t* o = (uint8_t*)j->out;
        int nb = j->row_len / 32, stride = j->row_len + nb;
        double* v = (double*)malloc(sizeof(double) * (size_t)j->row_len);
        for (int64_t r = lo; r < hi; ++r) {
            uint64_t base = (uint64_t)(j->row0 + r) * (uint64_t)j->row_len;
            for (int c = 0; c < j->row_len; ++c) v[c] = normal(hash3(j->seed, j->tid, base + (uint64_t)c));
            uint8_t* orow = o + r * stride;
            for (int b = 0; b < nb; ++b) {
                double amax = 0.0;
                for (int c = 0; c < 32; ++c) amax = fmax(amax, fabs(v[b * 32 + c]));
                int se = amax > 0.0 ? ilog2_floor(amax) - 8 : -127;
                if (se < -127) se = -127;
                if (se > 127) se = 127;
                orow[j->row_len + b] = (uint8_t)(se + 127);
                for (int c = 0; c < 32; ++c) orow[b * 32 + c] = e4m3_code(ldexp(v[b * 32 + c], -se));
            }
        }
        free(v);
        break;
    }
    case 6: {
        double* o = (double*)j->out;
        for (int64_t i = lo; i < hi; ++i) o[i] = normal(hash3(j->seed, j->tid, (uint64_t)(j->row0 + i)));
        break;
    }
    case 5: { /* E2M1 rows with one E4M3 scale per 16 values: X = E4M3(amax / 6) (RNE), a block
               * whose X would be 0 takes the smallest step 2^-9; values E2M1(x / X) (RNE, saturating) */
        uint8_t* o = (uint8_t*)j->out;
        int nb = j->row_len / 16;
        double* v = (double*)malloc(sizeof(double) * (size_t)j->row_len);
        for (int64_t r = lo; r < hi; ++r) {
            uint64_t base = (uint64_t)(j->row0 + r) * (uint64_t)j->row_len;
            for (int c = 0; c < j->row_len; ++c) v[c] = normal(hash3(j->seed, j->tid, base + (uint64_t)c));
            uint8_t* orow = o + r * (j->row_len / 2);
            for (int b = 0; b < nb; ++b) {
                double amax = 0.0;
                for (int c = 0; c < 16; ++c) amax = fmax(amax, fabs(v[b * 16 + c]));
                uint8_t sc = e4m3_code(amax / 6.0);
                if ((sc & 0x7F) == 0) sc = 0x01;
                j->scales[r * nb + b] = sc;
                double X = e4m3_value(sc);
                for (int c = 0; c < 16; c += 2) {
                    int idx = b * 16 + c;
                    uint8_t lo4 = e2m1_code(v[idx] / X);
                    uint8_t hi4 = e2m1_code(v[idx + 1] / X);
                    orow[idx / 2] = (uint8_t)(lo4 | (hi4 << 4));
                }
            }
        }
        free(v);
        break;
    }
    }
}

static void* worker(void* p) {
    job_t* j = (job_t*)p;
    run_range(j, j->lo, j->hi);
    return NULL;
}

static int g_threads = 0;

void csa2synth_set_threads(int n) { g_threads = n; }

static void run(job_t* proto, int64_t count) {
    int nt = g_threads > 0 ? g_threads : 8;
    if (count < 4096) nt = 1;
    if (nt > 256) nt = 256;
    pthread_t th[256];
    job_t jobs[256];
    int64_t per = (count + nt - 1) / nt;
    int started = 0;
    for (int t = 0; t < nt; ++t) {
        jobs[t] = *proto;
        jobs[t].lo = t * per;
        jobs[t].hi = (t + 1) * per < count ? (t + 1) * per : count;
        if (jobs[t].lo >= jobs[t].hi) break;
        if (nt == 1) {
            worker(&jobs[t]);
        } else {
            pthread_create(&th[t], NULL, worker, &jobs[t]);
            ++started;
        }
    }
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
}

/* ---- exported fillers ---------------------------------------------------- */

/* out[i] = N(0,1) sample for element (off + i) of tensor tid. */
void csa2synth_normal_f32(uint64_t seed, uint64_t tid, int64_t off, int64_t n, float* out) {
    job_t j = {0};
    j.kind = 0; j.seed = seed; j.tid = tid; j.row0 = off; j.out = out;
    run(&j, n);
}

/* the same N(0,1) draws in double (what the encoders quantise), for tests */
void csa2synth_normal_f64(uint64_t seed, uint64_t tid, int64_t off, int64_t n, double* out) {
    job_t j = {0};
    j.kind = 6; j.seed = seed; j.tid = tid; j.row0 = off; j.out = out;
    run(&j, n);
}

void csa2synth_uniform_f32(uint64_t seed, uint64_t tid, int64_t off, int64_t n, float* out) {
    job_t j = {0};
    j.kind = 1; j.seed = seed; j.tid = tid; j.row0 = off; j.out = out;
    run(&j, n);
}

void csa2synth_normal_bf16(uint64_t seed, uint64_t tid, int64_t off, int64_t n, uint16_t* out) {
    job_t j = {0};
    j.kind = 2; j.seed = seed; j.tid = tid; j.row0 = off; j.out = out;
    run(&j, n);
}

/* nrows rows of row_len N(0,1) values (rows row0.. of tensor tid), encoded as
 * packed E2M1 codes [nrows][row_len/2] with E8M0 scales [nrows][row_len/block]. */
int csa2synth_mxfp4_rows(uint64_t seed, uint64_t tid, int64_t row0, int64_t nrows, int row_len, int block,
                         uint8_t* codes, uint8_t* scales) {
    if (row_len <= 0 || block <= 0 || row_len % block || block % 2) return 1;
    job_t j = {0};
    j.kind = 3; j.seed = seed; j.tid = tid; j.row0 = row0; j.row_len = row_len; j.block = block;
    j.out = codes; j.scales = scales;
    run(&j, nrows);
    return 0;
}

/* nrows rows of row_len N(0,1) values encoded as E4M3 [nrows][row_len] with
 * one E8M0 scale per row chosen so that |x/X| < 16. */
int csa2synth_e4m3_rows(uint64_t seed, uint64_t tid, int64_t row0, int64_t nrows, int row_len, uint8_t* codes,
                        uint8_t* scales) {
    if (row_len <= 0) return 1;
    job_t j = {0};
    j.kind = 4; j.seed = seed; j.tid = tid; j.row0 = row0; j.row_len = row_len;
    j.out = codes; j.scales = scales;
    run(&j, nrows);
    return 0;
}

/* nrows rows of row_len N(0,1) values as packed E2M1 codes [nrows][row_len/2]
 * with one E4M3 scale per 16 values [nrows][row_len/16] (the report's main-KV
 * cache format, section 2.4.4: NVFP4's layout without its global scale). */
int csa2synth_e2m1_e4m3_rows(uint64_t seed, uint64_t tid, int64_t row0, int64_t nrows, int row_len, uint8_t* codes,
                             uint8_t* scales) {
    if (row_len <= 0 || row_len % 16) return 1;
    job_t j = {0};
    j.kind = 5; j.seed = seed; j.tid = tid; j.row0 = row0; j.row_len = row_len;
    j.out = codes; j.scales = scales;
    run(&j, nrows);
    return 0;
}

/* nrows rows of row_len N(0,1) values as OCP MXFP8 (E4M3 elements, one E8M0
 * scale per 32), each row its row_len code bytes followed by its row_len/32
 * scale bytes: [nrows][row_len + row_len/32] u8. */
int csa2synth_mxfp8_rows(uint64_t seed, uint64_t tid, int64_t row0, int64_t nrows, int row_len, uint8_t* rows) {
    if (row_len <= 0 || row_len % 32) return 1;
    job_t j = {0};
    j.kind = 7; j.seed = seed; j.tid = tid; j.row0 = row0; j.row_len = row_len;
    j.out = rows;
    run(&j, nrows);
    return 0;
}

/* Single-value encoders, exported so that tests can pin them. */
uint8_t csa2synth_encode_e2m1(double v) { return e2m1_code(v); }
uint8_t csa2synth_encode_e4m3(double v) { return e4m3_code(v); }
uint16_t csa2synth_encode_bf16(float v) { return bf16_rne(v); }
uint64_t csa2synth_hash(uint64_t seed, uint64_t tid, uint64_t i) { return hash3(seed, tid, i); }
