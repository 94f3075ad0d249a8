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
 * Grouped heads: with kv_heads < heads, query head h reads key/value head
 * h / (heads / kv_heads) (contiguous groups, the usual grouped-query layout);
 * state and slope stay per query head.  The pages only say that the reference
 * kernel rejects qo_heads != kv_heads ([LA-page] §输入与配置覆盖); this is the
 * plainest extension of the recurrence to that case.
 *
 * State tracking ([LA-page] §额外覆盖：mamba 状态跟踪与布局鲁棒性): with
 * track_lens given, the state of request b once its first track_lens[b]
 * tokens have been absorbed (the prefix state itself for 0) is copied out as
 * a snapshot; a track length outside [0, len] takes no snapshot.
 *
 * Tree verify ([LA-page] §生产环境不支持 item 3 and the Next Work item on tree
 * verify: every draft token forks from the saved state of its parent): draft
 * j of request b has parent p = parents[b][j], either -1 (the request's
 * committed state) or an earlier draft p < j.  Its state is
 *     S_j = S_p * exp(-slope_h) + outer(k_j, v_j),   o_j = (q_j @ S_j) * d^-0.5
 * with S_{-1} the initial state, and every S_j is kept.  Parents (-1, 0, 1,
 * ..., k-2) give the chain.
 *
 * Parity status: every function here is pinned by the CPU tests (closed form,
 * slope-0 cumulative sum, hand-derived worked example, orientation, large
 * slope, split invariance, linearity, published ALiBi values, grouped-head
 * closed form, snapshot closed form, tree path closed form).
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
    int batch, heads, kv_heads, dim;
    const int64_t *cu_seqlens; /* [batch+1] */
    const double *q;           /* [T, heads, dim] */
    const double *k, *v;       /* [T, kv_heads, dim] */
    const double *init;        /* [batch, heads, dim, dim] initial states */
    const double *slopes;      /* [heads] */
    const int64_t *track_lens; /* [batch] or NULL */
    double *out;               /* [T, heads, dim] */
    double *final_state;       /* [batch, heads, dim, dim] */
    double *track_state;       /* [batch, heads, dim, dim] or NULL */
    /* tree verify (cu_seqlens unused): request b owns tokens b*num_draft .. */
    int num_draft;
    const int32_t *parents;    /* [batch, num_draft] or NULL (varlen recurrence) */
    double *draft_state;       /* [batch, num_draft, heads, dim, dim] */
    int64_t next;              /* next (request, head) pair to take */
    pthread_mutex_t lock;
    int status;
} job_t;

/* S <- S * decay + outer(k_t, v_t), then o_t = scale * q_t @ S */
static void step(double *S, int d, double decay, double scale,
                 const double *qt, const double *kt, const double *vt, double *ot)
{
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

/* One (request, head) pair: the recurrence, token by token. */
static void run_pair(const job_t *jb, int b, int h, double *S)
{
    const int H = jb->heads, HK = jb->kv_heads, d = jb->dim;
    const int hk = h / (H / HK); /* key/value head of query head h */
    const double decay = exp(-jb->slopes[h]);
    const double scale = 1.0 / sqrt((double)d);
    const size_t sdd = (size_t)d * d;
    const int64_t t0 = jb->cu_seqlens[b], t1 = jb->cu_seqlens[b + 1];
    const int64_t tl = jb->track_lens ? jb->track_lens[b] : -1;
    double *snap = jb->track_state ? jb->track_state + ((size_t)b * H + h) * sdd : NULL;

    memcpy(S, jb->init + ((size_t)b * H + h) * sdd, sdd * sizeof(double));
    for (int64_t t = t0; t < t1; ++t) {
        if (snap && t - t0 == tl) /* track_len tokens absorbed */
            memcpy(snap, S, sdd * sizeof(double));
        step(S, d, decay, scale, jb->q + ((size_t)t * H + h) * d, jb->k + ((size_t)t * HK + hk) * d,
             jb->v + ((size_t)t * HK + hk) * d, jb->out + ((size_t)t * H + h) * d);
    }
    if (snap && tl == t1 - t0)
        memcpy(snap, S, sdd * sizeof(double));
    memcpy(jb->final_state + ((size_t)b * H + h) * sdd, S, sdd * sizeof(double));
}

/* One (request, head) pair of a tree verify: each draft starts from a copy of
   its parent's saved state (or the initial state) and takes one step. */
static void tree_pair(const job_t *jb, int b, int h, double *S)
{
    const int H = jb->heads, HK = jb->kv_heads, d = jb->dim, n = jb->num_draft;
    const int hk = h / (H / HK);
    const double decay = exp(-jb->slopes[h]);
    const double scale = 1.0 / sqrt((double)d);
    const size_t sdd = (size_t)d * d;

    for (int j = 0; j < n; ++j) {
        const int p = jb->parents[(size_t)b * n + j];
        const double *from = p < 0 ? jb->init + ((size_t)b * H + h) * sdd
                                   : jb->draft_state + (((size_t)b * n + p) * H + h) * sdd;
        memcpy(S, from, sdd * sizeof(double));
        const size_t t = (size_t)b * n + j;
        step(S, d, decay, scale, jb->q + (t * H + h) * d, jb->k + (t * HK + hk) * d,
             jb->v + (t * HK + hk) * d, jb->out + (t * H + h) * d);
        memcpy(jb->draft_state + (((size_t)b * n + j) * H + h) * sdd, S, sdd * sizeof(double));
    }
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
        if (jb->parents)
            tree_pair(jb, (int)(p / jb->heads), (int)(p % jb->heads), S);
        else
            run_pair(jb, (int)(p / jb->heads), (int)(p % jb->heads), S);
    }
    free(S);
    return NULL;
}

static int run_job(job_t *jb, int num_threads)
{
    const int64_t pairs = (int64_t)jb->batch * jb->heads;
    if (num_threads < 1)
        num_threads = 1;
    if ((int64_t)num_threads > pairs)
        num_threads = (int)(pairs > 0 ? pairs : 1);
    jb->next = 0;
    jb->status = LA_ORACLE_OK;
    pthread_mutex_init(&jb->lock, NULL);
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)num_threads);
    if (!tid) {
        pthread_mutex_destroy(&jb->lock);
        return LA_ORACLE_NO_MEM;
    }
    int started = 0;
    for (int i = 0; i < num_threads; ++i) {
        if (pthread_create(&tid[i], NULL, worker, jb) != 0)
            break;
        ++started;
    }
    if (started == 0)
        worker(jb);
    for (int i = 0; i < started; ++i)
        pthread_join(tid[i], NULL);
    free(tid);
    pthread_mutex_destroy(&jb->lock);
    return jb->status;
}

/*
 * Run the recurrence over a packed varlen batch.
 *   cu_seqlens [batch+1]: request b owns tokens cu_seqlens[b] .. cu_seqlens[b+1]-1
 *   q, out  [T, heads, dim]; k, v [T, kv_heads, dim] row-major, T = cu_seqlens[batch];
 *       kv_heads divides heads
 *   init_states, final_states [batch, heads, dim, dim]: the state before the
 *       first token and after the last one (a zero-length request returns its
 *       initial state unchanged)
 *   slopes [heads]
 *   track_lens [batch] and track_states [batch, heads, dim, dim]: both NULL, or
 *       the snapshot of each request after track_lens[b] tokens (entries of
 *       requests whose track length is outside [0, len] are left as they are)
 * Threads: `num_threads` workers take (request, head) pairs from a shared
 * counter.  Returns 0 on success.
 */
int la_oracle_run(int batch, int heads, int kv_heads, int dim, const int64_t *cu_seqlens,
                  const double *q, const double *k, const double *v,
                  const double *init_states, const double *slopes,
                  const int64_t *track_lens, double *out, double *final_states,
                  double *track_states, int num_threads)
{
    if (batch < 0 || heads <= 0 || kv_heads <= 0 || heads % kv_heads || dim <= 0 || !cu_seqlens ||
        !init_states || !slopes || !final_states)
        return LA_ORACLE_BAD_ARG;
    if (!track_lens != !track_states)
        return LA_ORACLE_BAD_ARG;
    if (cu_seqlens[0] != 0)
        return LA_ORACLE_BAD_ARG;
    for (int b = 0; b < batch; ++b)
        if (cu_seqlens[b + 1] < cu_seqlens[b])
            return LA_ORACLE_BAD_ARG;
    if (cu_seqlens[batch] > 0 && (!q || !k || !v || !out))
        return LA_ORACLE_BAD_ARG;

    job_t jb;
    memset(&jb, 0, sizeof(jb));
    jb.batch = batch;
    jb.heads = heads;
    jb.kv_heads = kv_heads;
    jb.dim = dim;
    jb.cu_seqlens = cu_seqlens;
    jb.q = q;
    jb.k = k;
    jb.v = v;
    jb.init = init_states;
    jb.slopes = slopes;
    jb.track_lens = track_lens;
    jb.out = out;
    jb.final_state = final_states;
    jb.track_state = track_states;
    return run_job(&jb, num_threads);
}

/*
 * Tree verify.  Request b owns draft tokens b*num_draft .. b*num_draft+num_draft-1
 * of q, out [batch*num_draft, heads, dim] and k, v [batch*num_draft, kv_heads, dim];
 * parents [batch, num_draft] with parents[b][j] in [-1, j); init_states
 * [batch, heads, dim, dim]; states [batch, num_draft, heads, dim, dim] receives
 * the state after every draft.  Returns 0 on success.
 */
int la_oracle_tree(int batch, int num_draft, int heads, int kv_heads, int dim,
                   const double *q, const double *k, const double *v,
                   const double *init_states, const double *slopes, const int32_t *parents,
                   double *out, double *states, int num_threads)
{
    if (batch < 0 || num_draft <= 0 || heads <= 0 || kv_heads <= 0 || heads % kv_heads || dim <= 0 ||
        !init_states || !slopes || !parents || !states)
        return LA_ORACLE_BAD_ARG;
    if (batch > 0 && (!q || !k || !v || !out))
        return LA_ORACLE_BAD_ARG;
    for (int64_t i = 0; i < (int64_t)batch * num_draft; ++i) {
        const int j = (int)(i % num_draft);
        if (parents[i] < -1 || parents[i] >= j)
            return LA_ORACLE_BAD_ARG;
    }
    job_t jb;
    memset(&jb, 0, sizeof(jb));
    jb.batch = batch;
    jb.heads = heads;
    jb.kv_heads = kv_heads;
    jb.dim = dim;
    jb.q = q;
    jb.k = k;
    jb.v = v;
    jb.init = init_states;
    jb.slopes = slopes;
    jb.out = out;
    jb.num_draft = num_draft;
    jb.parents = parents;
    jb.draft_state = states;
    return run_job(&jb, num_threads);
}
