/*
 * la_oracle.c -- plain fp64 CPU oracle for Lightning-style segmented linear
 * attention (seg_la).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library; its inputs are the seeded synthetic tensors,
 * never values produced by the GPU path.
 *
 * Citations name the web page "SGLang Lightning Attention 能力矩阵与 seg_la
 * 线性注意力测试覆盖深度解析" (www.2kiu.com/news/4599301) as [LA-page] and
 * its sections by their headings.
 *
 * What it computes ([LA-page] §独立参考实现：逐 token 递推公式, the per-token
 * recurrence), for every request b and head h, over that request's tokens t in
 * order:
 *
 *     S   <- S * exp(-slope_h) + outer(k_t, v_t)      (decay first, then add)
 *     o_t  = (q_t @ S) * head_dim^-0.5                (uses the updated S)
 *
 * S is d_k x d_v: row i is indexed by the key feature, column j by the value
 * feature, so q contracts the row index.  The state before the first token
 * is the request's slot of the state pool (the prefix state injected in the
 * same section), and the final state is returned per request.  Every step is
 * the definition written out in double precision, one token at a time; the
 * only parallelism is across independent (request, head) pairs.
 *
 * The ALiBi slope rule ([LA-page] same section, slope bullet: slopes times
 * (1 - layer_id/(L-1) + 1e-5), or times (1 + 1e-5) when L = 1) is taken with
 * the geometric ALiBi sequence of Press, Smith & Lewis, "Train Short, Test
 * Long" (ICLR 2022): for n heads a power of two, slope_i = 2^(-8(i+1)/n);
 * otherwise the first m = 2^floor(log2 n) slopes of the m-head sequence
 * followed by every other slope of the 2m-head sequence.  The factor is
 * applied in double and the product rounded once to fp32, the precision the
 * kernels receive.
 *
 * Parity status: every function here is pinned by the CPU tests (closed form,
 * slope-0 cumulative sum, hand-derived worked example, orientation, large
 * slope, split invariance, linearity, published ALiBi values).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define LA_ORACLE_OK 0
#define LA_ORACLE_BAD_ARG 1
#define LA_ORACLE_NO_MEM 2

/* Slope for head i of an n-head ALiBi model (Press et al., geometric rule). */
static double alibi_slope(int n, int i)
{
    int m = 1;
    while (m * 2 <= n)
        m *= 2;
    if (i < m)
        return pow(2.0, -8.0 * (double)(i + 1) / (double)m);
    /* heads beyond the largest power of two: every other slope of the
       2m-head sequence, starting at its first element */
    int j = i - m;
    return pow(2.0, -8.0 * (double)(2 * j + 1) / (double)(2 * m));
}

/* Per-head slopes for layer `layer_id` of `num_layers`, rounded once to fp32.
   Returns nonzero on an invalid argument. */
int la_oracle_alibi_slopes(int num_heads, int layer_id, int num_layers, float *slopes)
{
    if (num_heads <= 0 || num_layers <= 0 || layer_id < 0 || layer_id >= num_layers || !slopes)
        return LA_ORACLE_BAD_ARG;
    double factor;
    if (num_layers == 1)
        factor = 1.0 + 1e-5;
    else
        factor = 1.0 - (double)layer_id / (double)(num_layers - 1) + 1e-5;
    for (int h = 0; h < num_heads; ++h)
        slopes[h] = (float)(alibi_slope(num_heads, h) * factor);
    return LA_ORACLE_OK;
}

typedef struct {
    int batch, heads, dim;
    const int64_t *cu_seqlens; /* [batch+1] */
    const double *q, *k, *v;   /* [T, heads, dim] */
    const double *init;        /* [batch, heads, dim, dim] initial states */
    const double *slopes;      /* [heads] */
    double *out;               /* [T, heads, dim] */
    double *final_state;       /* [batch, heads, dim, dim] */
    int64_t next;              /* next (request, head) pair to take */
    pthread_mutex_t lock;
    int status;
} job_t;

/* One (request, head) pair: the recurrence, token by token. */
static void run_pair(const job_t *jb, int b, int h, double *S)
{
    const int H = jb->heads, d = jb->dim;
    const double decay = exp(-jb->slopes[h]);
    const double scale = 1.0 / sqrt((double)d);
    const size_t sdd = (size_t)d * d;

    memcpy(S, jb->init + ((size_t)b * H + h) * sdd, sdd * sizeof(double));
    for (int64_t t = jb->cu_seqlens[b]; t < jb->cu_seqlens[b + 1]; ++t) {
        const double *qt = jb->q + ((size_t)t * H + h) * d;
        const double *kt = jb->k + ((size_t)t * H + h) * d;
        const double *vt = jb->v + ((size_t)t * H + h) * d;
        double *ot = jb->out + ((size_t)t * H + h) * d;
        /* state update: decay, then add the outer product k_t v_t^T */
        for (int i = 0; i < d; ++i)
            for (int j = 0; j < d; ++j)
                S[(size_t)i * d + j] = S[(size_t)i * d + j] * decay + kt[i] * vt[j];
        /* output from the updated state: o_j = scale * sum_i q_i S_ij */
        for (int j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i)
                acc += qt[i] * S[(size_t)i * d + j];
            ot[j] = acc * scale;
        }
    }
    memcpy(jb->final_state + ((size_t)b * H + h) * sdd, S, sdd * sizeof(double));
}

static void *worker(void *arg)
{
    job_t *jb = (job_t *)arg;
    const int64_t pairs = (int64_t)jb->batch * jb->heads;
    double *S = (double *)malloc((size_t)jb->dim * jb->dim * sizeof(double));
    if (!S) {
        pthread_mutex_lock(&jb->lock);
        jb->status = LA_ORACLE_NO_MEM;
        pthread_mutex_unlock(&jb->lock);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&jb->lock);
        int64_t p = jb->next++;
        pthread_mutex_unlock(&jb->lock);
        if (p >= pairs)
            break;
        run_pair(jb, (int)(p / jb->heads), (int)(p % jb->heads), S);
    }
    free(S);
    return NULL;
}

/*
 * Run the recurrence over a packed varlen batch.
 *   cu_seqlens [batch+1]: request b owns tokens cu_seqlens[b] .. cu_seqlens[b+1]-1
 *   q, k, v, out  [T, heads, dim] row-major, T = cu_seqlens[batch]
 *   init_states, final_states [batch, heads, dim, dim]: the state before the
 *       first token and after the last one (a zero-length request returns its
 *       initial state unchanged)
 *   slopes [heads]
 * Threads: `num_threads` workers take (request, head) pairs from a shared
 * counter.  Returns 0 on success.
 */
int la_oracle_run(int batch, int heads, int dim, const int64_t *cu_seqlens,
                  const double *q, const double *k, const double *v,
                  const double *init_states, const double *slopes,
                  double *out, double *final_states, int num_threads)
{
    if (batch < 0 || heads <= 0 || dim <= 0 || !cu_seqlens || !init_states || !slopes || !final_states)
        return LA_ORACLE_BAD_ARG;
    if (cu_seqlens[0] != 0)
        return LA_ORACLE_BAD_ARG;
    for (int b = 0; b < batch; ++b)
        if (cu_seqlens[b + 1] < cu_seqlens[b])
            return LA_ORACLE_BAD_ARG;
    if (cu_seqlens[batch] > 0 && (!q || !k || !v || !out))
        return LA_ORACLE_BAD_ARG;
    if (num_threads < 1)
        num_threads = 1;
    if ((int64_t)num_threads > (int64_t)batch * heads)
        num_threads = (int)((int64_t)batch * heads > 0 ? (int64_t)batch * heads : 1);

    job_t jb;
    jb.batch = batch;
    jb.heads = heads;
    jb.dim = dim;
    jb.cu_seqlens = cu_seqlens;
    jb.q = q;
    jb.k = k;
    jb.v = v;
    jb.init = init_states;
    jb.slopes = slopes;
    jb.out = out;
    jb.final_state = final_states;
    jb.next = 0;
    jb.status = LA_ORACLE_OK;
    pthread_mutex_init(&jb.lock, NULL);

    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)num_threads);
    if (!tid) {
        pthread_mutex_destroy(&jb.lock);
        return LA_ORACLE_NO_MEM;
    }
    int started = 0;
    for (int i = 0; i < num_threads; ++i) {
        if (pthread_create(&tid[i], NULL, worker, &jb) != 0)
            break;
        ++started;
    }
    if (started == 0)
        worker(&jb);
    for (int i = 0; i < started; ++i)
        pthread_join(tid[i], NULL);
    free(tid);
    pthread_mutex_destroy(&jb.lock);
    return jb.status;
}
