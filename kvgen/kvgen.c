/*
 * kvgen.c - seeded synthetic fp16 KV-cache generator.
 *
 * Shared input source for the oracle, the HIP path, the tests and the bench.
 * It holds none of the codec's arithmetic: it only draws numbers and writes
 * fp16 bit patterns in the layout [L][2][T][C] (layer, K|V, token, channel),
 * the kv_shape (layers, 2, tokens, kv_heads, head_dim) of the CacheGen/LMCache
 * write-up, "3.2 Validation and testing", with heads and head_dim flattened.
 *
 * Model of one series (layer l, tensor kv, channel c):
 *     x_0 = e_0 / sqrt(1 - rho^2),   x_t = rho * x_{t-1} + e_t      (double)
 *     value_t = s_c * x_t, clamped to +-65504, then double -> fp32 -> fp16 (RNE)
 * with e_t ~ N(0,1) (Box-Muller) or Student-t(3) = Z / sqrt((Z1^2+Z2^2+Z3^2)/3),
 * and s_c = a * (b/a)^U (log-uniform), multiplied by `outlier_mul` on a set of
 * round(outlier_frac * C) channels per (l, kv) picked by a partial Fisher-Yates
 * shuffle.
 *
 * Random numbers: every series has its own xoshiro256** stream (Vigna,
 * "Scrambled linear pseudorandom number generators", 2018/2021) whose 256-bit
 * state is filled by splitmix64 (Steele, Lea, Flood 2014) from a 64-bit key
 * built from (seed, purpose, l, kv, c).  Uniforms take the top 53 bits.
 * The output does not depend on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    uint64_t s[4];
} xo256;

static uint64_t splitmix64_next(uint64_t *x)
{
    uint64_t z = (*x += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static uint64_t rotl64(uint64_t x, int k) { return (x << k) | (x >> (64 - k)); }

static uint64_t xo_next(xo256 *g)
{
    uint64_t *s = g->s;
    uint64_t result = rotl64(s[1] * 5u, 7) * 9u;
    uint64_t t = s[1] << 17;
    s[2] ^= s[0];
    s[3] ^= s[1];
    s[1] ^= s[2];
    s[0] ^= s[3];
    s[2] ^= t;
    s[3] = rotl64(s[3], 45);
    return result;
}

enum { PURPOSE_SCALE = 1, PURPOSE_OUTLIER = 2, PURPOSE_INNOV = 3 };

static void xo_seed(xo256 *g, uint64_t seed, uint64_t purpose, uint64_t l, uint64_t kv, uint64_t c)
{
    /* key: disjoint bit fields, then mixed by splitmix64 */
    uint64_t x = seed * 0xD1342543DE82EF95ull;
    x ^= (purpose << 60) ^ (l << 40) ^ (kv << 39) ^ c;
    for (int i = 0; i < 4; ++i) g->s[i] = splitmix64_next(&x);
}

static double uniform01(xo256 *g) { return (double)(xo_next(g) >> 11) * 0x1.0p-53; }

/* Box-Muller: one pair of uniforms gives two independent N(0,1) draws; the
 * second is kept for the next call on the same series. */
typedef struct {
    xo256 g;
    double spare;
    int has_spare;
} normal_src;

static double normal01(normal_src *n)
{
    if (n->has_spare) {
        n->has_spare = 0;
        return n->spare;
    }
    double u1 = uniform01(&n->g), u2 = uniform01(&n->g);
    double rad = sqrt(-2.0 * log(1.0 - u1));
    double ang = 6.283185307179586476925 * u2;
    n->spare = rad * sin(ang);
    n->has_spare = 1;
    return rad * cos(ang);
}

static double student_t3(normal_src *n)
{
    double z = normal01(n);
    double z1 = normal01(n), z2 = normal01(n), z3 = normal01(n);
    return z / sqrt((z1 * z1 + z2 * z2 + z3 * z3) / 3.0);
}

/* fp32 -> fp16 bit pattern, round to nearest even; input finite, |f| <= 65504 */
static uint16_t gen_f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t sign = (u >> 16) & 0x8000u;
    uint32_t mag = u & 0x7FFFFFFFu;
    if (mag >= 0x477FF000u) return (uint16_t)(sign | 0x7BFFu); /* clamp (only 65504 reaches here) */
    if (mag < 0x38800000u) {                                   /* below 2^-14: fp16 subnormal */
        /* value * 2^24 rounded to an integer, exact in double */
        float a;
        memcpy(&a, &mag, 4);
        double m = rint((double)a * 16777216.0);
        return (uint16_t)(sign | (uint32_t)m);
    }
    uint32_t e = (mag >> 23) - 127 + 15;
    uint32_t mant = mag & 0x7FFFFFu;
    uint32_t h = (e << 10) | (mant >> 13);
    uint32_t rest = mant & 0x1FFFu;
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1; /* carry into exponent is correct */
    return (uint16_t)(sign | h);
}

typedef struct {
    int32_t L, C;
    int64_t T;
    double rho;
    int32_t innov; /* 0 = normal, 1 = student-t(3) */
    double scale_lo, scale_hi;
    double outlier_frac, outlier_mul;
    uint64_t seed;
} kvgen_params;

typedef struct {
    const kvgen_params *p;
    uint16_t *out;
    int64_t n_jobs; /* jobs = (l, kv, channel block) */
    int64_t next;
    pthread_mutex_t mu;
    int64_t saturated;
} gen_shared;

enum { CBLK = 64 };

static void gen_job(const kvgen_params *p, uint16_t *out, int64_t job, int64_t *sat)
{
    int64_t nblk = (p->C + CBLK - 1) / CBLK;
    int64_t lk = job / nblk, blk = job % nblk;
    int l = (int)(lk / 2), kv = (int)(lk % 2);
    int c0 = (int)(blk * CBLK), c1 = c0 + CBLK < p->C ? c0 + CBLK : p->C;
    int nc = c1 - c0;

    /* outlier channels of this (l, kv): partial Fisher-Yates over all C */
    int n_out = (int)floor(p->outlier_frac * p->C + 0.5);
    unsigned char *is_out = NULL;
    if (n_out > 0) {
        int *perm = (int *)malloc(sizeof(int) * p->C);
        is_out = (unsigned char *)calloc(p->C, 1);
        xo256 g;
        xo_seed(&g, p->seed, PURPOSE_OUTLIER, l, kv, 0);
        for (int i = 0; i < p->C; ++i) perm[i] = i;
        for (int i = 0; i < n_out; ++i) {
            int j = i + (int)(uniform01(&g) * (p->C - i));
            int t = perm[i];
            perm[i] = perm[j];
            perm[j] = t;
            is_out[perm[i]] = 1;
        }
        free(perm);
    }

    double scale[CBLK], x[CBLK];
    normal_src g[CBLK];
    for (int i = 0; i < nc; ++i) {
        int c = c0 + i;
        xo256 gs;
        xo_seed(&gs, p->seed, PURPOSE_SCALE, l, kv, c);
        double u = uniform01(&gs);
        scale[i] = p->scale_lo * pow(p->scale_hi / p->scale_lo, u);
        if (is_out && is_out[c]) scale[i] *= p->outlier_mul;
        xo_seed(&g[i].g, p->seed, PURPOSE_INNOV, l, kv, c);
        g[i].has_spare = 0;
        g[i].spare = 0.0;
    }
    free(is_out);

    double stat = 1.0 / sqrt(1.0 - p->rho * p->rho);
    uint16_t *base = out + (int64_t)lk * p->T * p->C;
    int64_t s = 0;
    for (int64_t t = 0; t < p->T; ++t) {
        uint16_t *row = base + t * p->C;
        for (int i = 0; i < nc; ++i) {
            double e = p->innov ? student_t3(&g[i]) : normal01(&g[i]);
            x[i] = (t == 0) ? e * stat : p->rho * x[i] + e;
            double v = scale[i] * x[i];
            if (v > 65504.0) { v = 65504.0; ++s; }
            if (v < -65504.0) { v = -65504.0; ++s; }
            row[c0 + i] = gen_f32_to_f16((float)v);
        }
    }
    *sat += s;
}

static void *gen_worker(void *arg)
{
    gen_shared *sh = (gen_shared *)arg;
    int64_t sat = 0;
    for (;;) {
        pthread_mutex_lock(&sh->mu);
        int64_t job = sh->next++;
        pthread_mutex_unlock(&sh->mu);
        if (job >= sh->n_jobs) break;
        gen_job(sh->p, sh->out, job, &sat);
    }
    pthread_mutex_lock(&sh->mu);
    sh->saturated += sat;
    pthread_mutex_unlock(&sh->mu);
    return NULL;
}

/* Fill out[L][2][T][C] (fp16 bit patterns).  Returns the number of clamped
 * values (>= 0) or -1 on a bad argument. */
int64_t kvgen_generate(const kvgen_params *p, uint16_t *out, int n_threads)
{
    if (!p || !out || p->L < 1 || p->C < 1 || p->T < 0 || p->rho <= -1.0 || p->rho >= 1.0 ||
        !(p->scale_lo > 0.0) || !(p->scale_hi >= p->scale_lo))
        return -1;
    if (p->T == 0) return 0;
    gen_shared sh;
    sh.p = p;
    sh.out = out;
    sh.n_jobs = (int64_t)p->L * 2 * ((p->C + CBLK - 1) / CBLK);
    sh.next = 0;
    sh.saturated = 0;
    pthread_mutex_init(&sh.mu, NULL);
    if (n_threads < 1) n_threads = 1;
    if (n_threads > 256) n_threads = 256;
    pthread_t th[256];
    int started = 0;
    for (int i = 1; i < n_threads; ++i)
        if (pthread_create(&th[started], NULL, gen_worker, &sh) == 0) ++started;
    gen_worker(&sh);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&sh.mu);
    return sh.saturated;
}

/* FNV-1a 64 over a byte buffer (input checksum for logs). */
uint64_t kvgen_fnv1a64(const void *buf, int64_t n)
{
    const unsigned char *b = (const unsigned char *)buf;
    uint64_t h = 0xcbf29ce484222325ull;
    for (int64_t i = 0; i < n; ++i) {
        h ^= b[i];
        h *= 0x100000001b3ull;
    }
    return h;
}
