/*
 * Exercise of the C oracle (oracle/la_oracle.c) for the sanitizer builds of
 * the CPU test suite: varlen batches with empty requests, grouped kv heads,
 * snapshots at and past a request's end, tree verify, several worker threads
 * and the argument errors.  Built with -fsanitize=address,undefined (and
 * separately with -fsanitize=thread); any report fails the test.  It also
 * checks that the threaded result equals the single-threaded one bit for bit
 * and that one small case matches the unrolled recurrence
 * S_t = e^{-l(t+1)} S_0 + sum_{s<=t} e^{-l(t-s)} k_s v_s^T, o_t = q_t S_t / sqrt(d).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int la_oracle_alibi_slopes(int num_heads, int layer_id, int num_layers, float *slopes);
int la_oracle_run(int batch, int heads, int kv_heads, int dim, const int64_t *cu_seqlens,
                  const double *q, const double *k, const double *v,
                  const double *init_states, const double *slopes,
                  const int64_t *track_lens, double *out, double *final_states,
                  double *track_states, int num_threads);
int la_oracle_tree(int batch, int num_draft, int heads, int kv_heads, int dim,
                   const double *q, const double *k, const double *v,
                   const double *init_states, const double *slopes, const int32_t *parents,
                   double *out, double *states, int num_threads);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double rnd(void) /* uniform in [-1, 1), splitmix64 */
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) / 4503599627370496.0 - 1.0;
}

static double *vec(size_t n)
{
    double *p = (double *)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i)
        p[i] = rnd();
    return p;
}

#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            return 1;                                                     \
        }                                                                 \
    } while (0)

int main(void)
{
    /* varlen batch: lengths 5, 0, 9, 1; H = 4 query heads over 2 kv heads, d = 8 */
    enum { B = 4, H = 4, HK = 2, D = 8 };
    const int64_t cu[B + 1] = {0, 5, 5, 14, 15};
    const int64_t T = cu[B];
    double *q = vec((size_t)T * H * D), *k = vec((size_t)T * HK * D), *v = vec((size_t)T * HK * D);
    double *s0 = vec((size_t)B * H * D * D);
    float sl32[H];
    double sl[H];
    CHECK(la_oracle_alibi_slopes(H, 1, 3, sl32) == 0);
    for (int h = 0; h < H; ++h)
        sl[h] = sl32[h];
    const int64_t tl[B] = {5, 0, 4, 3}; /* at the end, the prefix, inside, past the end */
    double *o1 = vec((size_t)T * H * D), *f1 = vec((size_t)B * H * D * D), *t1 = vec((size_t)B * H * D * D);
    double *o3 = vec((size_t)T * H * D), *f3 = vec((size_t)B * H * D * D), *t3 = vec((size_t)B * H * D * D);
    memcpy(t3, t1, (size_t)B * H * D * D * sizeof(double)); /* untouched entries must match too */
    CHECK(la_oracle_run(B, H, HK, D, cu, q, k, v, s0, sl, tl, o1, f1, t1, 1) == 0);
    CHECK(la_oracle_run(B, H, HK, D, cu, q, k, v, s0, sl, tl, o3, f3, t3, 3) == 0);
    CHECK(memcmp(o1, o3, (size_t)T * H * D * sizeof(double)) == 0);
    CHECK(memcmp(f1, f3, (size_t)B * H * D * D * sizeof(double)) == 0);
    CHECK(memcmp(t1, t3, (size_t)B * H * D * D * sizeof(double)) == 0);

    /* request 2, head 3 (kv head 1): the unrolled recurrence at its last token */
    {
        const int b = 2, h = 3, hk = 1;
        const int64_t n = cu[b + 1] - cu[b], t = n - 1;
        double o[D] = {0};
        for (int j = 0; j < D; ++j) {
            for (int i = 0; i < D; ++i) {
                double s = exp(-sl[h] * (double)(t + 1)) * s0[(((size_t)b * H + h) * D + i) * D + j];
                for (int64_t u = 0; u <= t; ++u)
                    s += exp(-sl[h] * (double)(t - u)) * k[((cu[b] + u) * HK + hk) * D + i] *
                         v[((cu[b] + u) * HK + hk) * D + j];
                o[j] += q[((cu[b] + t) * H + h) * D + i] * s;
            }
            o[j] /= sqrt((double)D);
            CHECK(fabs(o[j] - o1[((cu[b] + t) * H + h) * D + j]) <= 1e-12 * (1.0 + fabs(o[j])));
        }
    }

    /* tree verify: 3 requests x 4 drafts, parents chain / star / mixed */
    {
        enum { TB = 3, N = 4 };
        const int32_t par[TB * N] = {-1, 0, 1, 2, -1, -1, -1, -1, -1, 0, 0, 2};
        double *tq = vec((size_t)TB * N * H * D), *tk = vec((size_t)TB * N * HK * D);
        double *tv = vec((size_t)TB * N * HK * D), *ts0 = vec((size_t)TB * H * D * D);
        double *out1 = vec((size_t)TB * N * H * D), *st1 = vec((size_t)TB * N * H * D * D);
        double *out4 = vec((size_t)TB * N * H * D), *st4 = vec((size_t)TB * N * H * D * D);
        CHECK(la_oracle_tree(TB, N, H, HK, D, tq, tk, tv, ts0, sl, par, out1, st1, 1) == 0);
        CHECK(la_oracle_tree(TB, N, H, HK, D, tq, tk, tv, ts0, sl, par, out4, st4, 4) == 0);
        CHECK(memcmp(out1, out4, (size_t)TB * N * H * D * sizeof(double)) == 0);
        CHECK(memcmp(st1, st4, (size_t)TB * N * H * D * D * sizeof(double)) == 0);
        const int32_t bad[TB * N] = {-1, 0, 1, 3, -1, -1, -1, -1, -1, 0, 0, 2};
        CHECK(la_oracle_tree(TB, N, H, HK, D, tq, tk, tv, ts0, sl, bad, out1, st1, 2) != 0);
        free(tq), free(tk), free(tv), free(ts0), free(out1), free(st1), free(out4), free(st4);
    }

    /* argument errors: rejected before any work */
    const int64_t cu_bad[3] = {0, 4, 2};
    CHECK(la_oracle_run(2, H, HK, D, cu_bad, q, k, v, s0, sl, NULL, o1, f1, NULL, 2) != 0);
    CHECK(la_oracle_run(B, H, 3, D, cu, q, k, v, s0, sl, NULL, o1, f1, NULL, 2) != 0);
    CHECK(la_oracle_run(B, H, HK, D, cu, q, k, v, s0, sl, tl, o1, f1, NULL, 2) != 0);
    CHECK(la_oracle_run(B, H, HK, D, cu, NULL, k, v, s0, sl, NULL, o1, f1, NULL, 2) != 0);
    CHECK(la_oracle_alibi_slopes(0, 0, 1, sl32) != 0);
    CHECK(la_oracle_alibi_slopes(4, 2, 2, sl32) != 0);
    /* an empty batch is fine */
    const int64_t cu0[1] = {0};
    CHECK(la_oracle_run(0, H, HK, D, cu0, NULL, NULL, NULL, s0, sl, NULL, NULL, f1, NULL, 4) == 0);

    free(q), free(k), free(v), free(s0), free(o1), free(f1), free(t1), free(o3), free(f3), free(t3);
    puts("oracle driver ok");
    return 0;
}
