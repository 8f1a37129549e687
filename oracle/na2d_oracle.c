/*
 * na2d_oracle.c -- plain, slow, obviously-correct CPU oracle for the forward
 * and backward passes of 2D (dilated) Neighborhood Attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
 * the CPU-baseline leg of the benchmark may load this code.  It shares no
 * source, header, table or helper with the HIP library; it is compiled with
 * gcc on its own and loaded through ctypes.
 *
 * What it computes (all arithmetic in double):
 *
 *   For every batch b, head h and query pixel (i, j) of an H x W map:
 *
 *   1. Neighbourhood (sources: NAT model doc, Overview -- NA is a pixel-wise
 *      operation restricting self attention to the nearest neighbouring
 *      pixels; NAT repository README, introduction -- NA equals dot-product
 *      self attention when the neighbourhood is as large as the image, and the
 *      edges are special cases; DiNAT walk-through blog, section "What is
 *      DiNAT" -- dilation samples a neighbour every d pixels and the number of
 *      attended tokens is fixed by kernel_size alone).
 *
 *      Reading adopted for the edges: the k x k window is shifted inward so it
 *      stays inside the map; every query keeps exactly k*k neighbours.  Only
 *      this reading makes the README's "equals self attention at full size"
 *      statement true for edge pixels.
 *
 *      Reading adopted for dilation: pixels are split into d*d residue classes
 *      (i mod d, j mod d); each class is a strided sub-grid, and the window is
 *      placed and clamped inside the query's own sub-grid.  A class with
 *      residue ry holds ceil((H - ry) / d) rows.
 *
 *        ry = i mod d, ci = i div d, Ly = ceil((H - ry)/d),
 *        sy = clamp(ci - k div 2, 0, Ly - k),
 *        neighbour row of window row a = ry + (sy + a) * d,  a in [0, k)
 *      (the same on columns with j, W).
 *
 *   2. Scores (source: DiNAT walk-through blog, section "What is DiNAT", the
 *      module calls natten2dqkrpb(query, key, rpb, kernel_size, dilation)):
 *        S[n] = (sum_e q[e] * key_n[e]) / sqrt(D) + rpb[h][dy_n + k-1][dx_n + k-1]
 *      for n = a*k + c, where (dy_n, dx_n) is the key-minus-query offset
 *      counted in sub-grid steps; the bias table has (2k-1) x (2k-1) entries
 *      per head, exactly the range of offsets the clamped window can produce.
 *      rpb == NULL means a zero bias.
 *
 *   3. Softmax over the k*k neighbour axis (same passage, softmax(dim=-1)),
 *      computed with the maximum subtracted.
 *
 *   4. Output (same passage, natten2dav(attn, value, kernel_size, dilation)):
 *        out[e] = sum_n P[n] * value_n[e].
 *
 *   5. Log-sum-exp (optional): the natural log of step 3's denominator,
 *        lse = ln sum_n exp(S[n]) = Smax + ln sum_n exp(S[n] - Smax).
 *
 * The function returns, per requested query, the output row and optionally
 * the scores S, the probabilities P, the log-sum-exp, the flat neighbour
 * pixel index of every window slot and the arg-max of S (lowest n wins
 * ties).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS 1
#define ORACLE_NO_MEMORY 2

/* Window start, in sub-grid steps, of a query at sub-grid coordinate c in a
 * residue class of length len: the window is centred on the query and then
 * shifted inward until it fits. */
static int oracle_window_start(int c, int len, int ks)
{
    int s = c - ks / 2;
    if (s < 0)
        s = 0;
    if (s > len - ks)
        s = len - ks;
    return s;
}

typedef struct {
    const double *q, *k, *v, *rpb;
    int B, heads, H, W, D, ks, dil;
    const int64_t *qidx;
    int64_t first, last; /* range of positions in the query list */
    double *out, *scores, *probs, *lse;
    int32_t *nbr, *argmax;
} oracle_job;

static void oracle_one_query(const oracle_job *jb, int64_t pos, double *s, double *p)
{
    const int W = jb->W, H = jb->H, D = jb->D, ks = jb->ks, d = jb->dil;
    const int nk = ks * ks;
    const int64_t flat = jb->qidx ? jb->qidx[pos] : pos; /* index over B*heads*H*W */
    const int64_t plane = flat / ((int64_t)H * W);       /* b*heads + h */
    const int pix = (int)(flat % ((int64_t)H * W));
    const int i = pix / W, j = pix % W;
    const int h = (int)(plane % jb->heads);

    const int ry = i % d, ci = i / d, Ly = (H - ry + d - 1) / d;
    const int rx = j % d, cj = j / d, Lx = (W - rx + d - 1) / d;
    const int sy = oracle_window_start(ci, Ly, ks);
    const int sx = oracle_window_start(cj, Lx, ks);

    const double *qrow = jb->q + flat * D;
    const double *kplane = jb->k + plane * (int64_t)H * W * D;
    const double *vplane = jb->v + plane * (int64_t)H * W * D;
    const double scale = 1.0 / sqrt((double)D);

    double smax = -INFINITY;
    int amax = 0;
    for (int a = 0; a < ks; ++a) {
        for (int c = 0; c < ks; ++c) {
            const int n = a * ks + c;
            const int ni = ry + (sy + a) * d;
            const int nj = rx + (sx + c) * d;
            const double *krow = kplane + ((int64_t)ni * W + nj) * D;
            double dot = 0.0;
            for (int e = 0; e < D; ++e)
                dot += qrow[e] * krow[e];
            double bias = 0.0;
            if (jb->rpb) {
                const int dy = (sy + a) - ci; /* key minus query, sub-grid steps */
                const int dx = (sx + c) - cj;
                const int side = 2 * ks - 1;
                bias = jb->rpb[((int64_t)h * side + (dy + ks - 1)) * side + (dx + ks - 1)];
            }
            s[n] = dot * scale + bias;
            if (s[n] > smax) { /* strict: the lowest n wins a tie */
                smax = s[n];
                amax = n;
            }
            if (jb->nbr)
                jb->nbr[pos * nk + n] = ni * W + nj;
        }
    }
    double sum = 0.0;
    for (int n = 0; n < nk; ++n) {
        p[n] = exp(s[n] - smax);
        sum += p[n];
    }
    for (int n = 0; n < nk; ++n)
        p[n] /= sum;
    if (jb->lse)
        jb->lse[pos] = smax + log(sum);

    double *orow = jb->out + pos * D;
    for (int e = 0; e < D; ++e)
        orow[e] = 0.0;
    for (int a = 0; a < ks; ++a) {
        for (int c = 0; c < ks; ++c) {
            const int n = a * ks + c;
            const int ni = ry + (sy + a) * d;
            const int nj = rx + (sx + c) * d;
            const double *vrow = vplane + ((int64_t)ni * W + nj) * D;
            for (int e = 0; e < D; ++e)
                orow[e] += p[n] * vrow[e];
        }
    }
    if (jb->scores)
        memcpy(jb->scores + pos * nk, s, sizeof(double) * nk);
    if (jb->probs)
        memcpy(jb->probs + pos * nk, p, sizeof(double) * nk);
    if (jb->argmax)
        jb->argmax[pos] = amax;
}

static void *oracle_worker(void *arg)
{
    const oracle_job *jb = (const oracle_job *)arg;
    const int nk = jb->ks * jb->ks;
    double *s = (double *)malloc(sizeof(double) * nk);
    double *p = (double *)malloc(sizeof(double) * nk);
    if (s && p)
        for (int64_t pos = jb->first; pos < jb->last; ++pos)
            oracle_one_query(jb, pos, s, p);
    free(s);
    free(p);
    return (s && p) ? NULL : (void *)1;
}

/*
 * q, k, v: [B, heads, H, W, D] doubles, contiguous.  rpb: [heads, 2k-1, 2k-1]
 * or NULL.  qidx: nq flat query indices in [0, B*heads*H*W), or NULL for all
 * queries in order.  Outputs are indexed by position in that list:
 * out [nq, D]; scores, probs [nq, k*k] (optional); lse [nq] (optional);
 * nbr [nq, k*k] flat pixel index i*W+j (optional); argmax [nq] (optional).
 */
int na2d_oracle_forward(const double *q, const double *k, const double *v, const double *rpb,
                        int B, int heads, int H, int W, int D, int ks, int dil,
                        const int64_t *qidx, int64_t nq,
                        double *out, double *scores, double *probs, double *lse,
                        int32_t *nbr, int32_t *argmax, int nthreads)
{
    if (!q || !k || !v || !out || B < 1 || heads < 1 || H < 1 || W < 1 || D < 1 ||
        ks < 1 || (ks % 2) == 0 || dil < 1 || H < ks * dil || W < ks * dil)
        return ORACLE_BAD_ARGS;
    const int64_t total = (int64_t)B * heads * H * W;
    if (!qidx)
        nq = total;
    if (nq < 0)
        return ORACLE_BAD_ARGS;
    if (qidx)
        for (int64_t t = 0; t < nq; ++t)
            if (qidx[t] < 0 || qidx[t] >= total)
                return ORACLE_BAD_ARGS;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (nq < nthreads)
        nthreads = nq > 0 ? (int)nq : 1;

    oracle_job jobs[256];
    pthread_t tids[256];
    int created[256];
    const int64_t chunk = (nq + nthreads - 1) / nthreads;
    int failed = 0;
    for (int t = 0; t < nthreads; ++t) {
        oracle_job *jb = &jobs[t];
        jb->q = q; jb->k = k; jb->v = v; jb->rpb = rpb;
        jb->B = B; jb->heads = heads; jb->H = H; jb->W = W; jb->D = D;
        jb->ks = ks; jb->dil = dil; jb->qidx = qidx;
        jb->first = (int64_t)t * chunk;
        jb->last = jb->first + chunk < nq ? jb->first + chunk : nq;
        jb->out = out; jb->scores = scores; jb->probs = probs; jb->lse = lse;
        jb->nbr = nbr; jb->argmax = argmax;
        created[t] = 0;
        if (jb->first >= jb->last)
            continue;
        if (pthread_create(&tids[t], NULL, oracle_worker, jb) == 0)
            created[t] = 1;
        else if (oracle_worker(jb)) /* could not spawn: run it here */
            failed = 1;
    }
    for (int t = 0; t < nthreads; ++t) {
        if (!created[t])
            continue;
        void *rc = NULL;
        pthread_join(tids[t], &rc);
        if (rc)
            failed = 1;
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Backward pass: the chain rule through the four steps above, in double.
 * With L = sum over all outputs of out * dout (dout given), for every query
 * with window keys n and probabilities P[n] (recomputed as in the forward):
 *
 *   dP[n]   = sum_e dout[e] * value_n[e]
 *   Dq      = sum_n P[n] * dP[n]               (softmax Jacobian, one row)
 *   dS[n]   = P[n] * (dP[n] - Dq)
 *   dq[e]   = sum_n dS[n] * key_n[e] / sqrt(D)
 *   dk_n[e] += dS[n] * q[e] / sqrt(D)          for every query whose window holds n
 *   dv_n[e] += P[n] * dout[e]                  likewise
 *   drpb[h][dy_n + k-1][dx_n + k-1] += dS[n]
 *
 * Threads own whole (batch, head) planes, so the scatter into dk and dv never
 * races; each thread sums its bias gradient into its own table and the tables
 * are added in thread order at the end (deterministic).
 */
typedef struct {
    const double *q, *k, *v, *rpb, *dout;
    int B, heads, H, W, D, ks, dil;
    int64_t plane0, plane1;
    double *dq, *dk, *dv, *drpb; /* drpb: this thread's own table */
} oracle_bwd_job;

static void *oracle_bwd_worker(void *arg)
{
    const oracle_bwd_job *jb = (const oracle_bwd_job *)arg;
    const int H = jb->H, W = jb->W, D = jb->D, ks = jb->ks, d = jb->dil;
    const int nk = ks * ks, side = 2 * ks - 1;
    const int64_t hw = (int64_t)H * W;
    const double scale = 1.0 / sqrt((double)D);
    double *s = (double *)malloc(sizeof(double) * nk);
    double *p = (double *)malloc(sizeof(double) * nk);
    double *dp = (double *)malloc(sizeof(double) * nk);
    int64_t *nb = (int64_t *)malloc(sizeof(int64_t) * nk);
    int *boff = (int *)malloc(sizeof(int) * nk);
    if (!s || !p || !dp || !nb || !boff) {
        free(s); free(p); free(dp); free(nb); free(boff);
        return (void *)1;
    }
    for (int64_t plane = jb->plane0; plane < jb->plane1; ++plane) {
        const int h = (int)(plane % jb->heads);
        const int64_t base = plane * hw * D;
        for (int i = 0; i < H; ++i) {
            for (int j = 0; j < W; ++j) {
                const int ry = i % d, ci = i / d, Ly = (H - ry + d - 1) / d;
                const int rx = j % d, cj = j / d, Lx = (W - rx + d - 1) / d;
                const int sy = oracle_window_start(ci, Ly, ks);
                const int sx = oracle_window_start(cj, Lx, ks);
                const double *qrow = jb->q + base + ((int64_t)i * W + j) * D;
                const double *grow = jb->dout + base + ((int64_t)i * W + j) * D;
                double smax = -INFINITY;
                for (int a = 0; a < ks; ++a)
                    for (int c = 0; c < ks; ++c) {
                        const int n = a * ks + c;
                        const int ni = ry + (sy + a) * d, nj = rx + (sx + c) * d;
                        nb[n] = base + ((int64_t)ni * W + nj) * D;
                        boff[n] = ((sy + a) - ci + ks - 1) * side + ((sx + c) - cj + ks - 1);
                        double dot = 0.0;
                        for (int e = 0; e < D; ++e)
                            dot += qrow[e] * jb->k[nb[n] + e];
                        s[n] = dot * scale + (jb->rpb ? jb->rpb[(int64_t)h * side * side + boff[n]] : 0.0);
                        if (s[n] > smax)
                            smax = s[n];
                    }
                double sum = 0.0;
                for (int n = 0; n < nk; ++n) {
                    p[n] = exp(s[n] - smax);
                    sum += p[n];
                }
                double dq_dot = 0.0; /* Dq */
                for (int n = 0; n < nk; ++n) {
                    p[n] /= sum;
                    double g = 0.0;
                    for (int e = 0; e < D; ++e)
                        g += grow[e] * jb->v[nb[n] + e];
                    dp[n] = g;
                    dq_dot += p[n] * g;
                }
                double *dqrow = jb->dq + base + ((int64_t)i * W + j) * D;
                for (int e = 0; e < D; ++e)
                    dqrow[e] = 0.0;
                for (int n = 0; n < nk; ++n) {
                    const double ds = p[n] * (dp[n] - dq_dot);
                    for (int e = 0; e < D; ++e) {
                        dqrow[e] += ds * jb->k[nb[n] + e] * scale;
                        jb->dk[nb[n] + e] += ds * qrow[e] * scale;
                        jb->dv[nb[n] + e] += p[n] * grow[e];
                    }
                    jb->drpb[(int64_t)h * side * side + boff[n]] += ds;
                }
            }
        }
    }
    free(s); free(p); free(dp); free(nb); free(boff);
    return NULL;
}

/*
 * q, k, v, dout: [B, heads, H, W, D] doubles, contiguous; rpb as in the
 * forward (NULL = zero bias).  Writes dq, dk, dv ([B, heads, H, W, D]) and
 * drpb ([heads, 2k-1, 2k-1], the gradient of the bias table; written also
 * when rpb is NULL).
 */
int na2d_oracle_backward(const double *q, const double *k, const double *v, const double *rpb,
                         const double *dout, int B, int heads, int H, int W, int D, int ks,
                         int dil, double *dq, double *dk, double *dv, double *drpb,
                         int nthreads)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || !drpb || B < 1 || heads < 1 ||
        H < 1 || W < 1 || D < 1 || ks < 1 || (ks % 2) == 0 || dil < 1 || H < ks * dil ||
        W < ks * dil)
        return ORACLE_BAD_ARGS;
    const int64_t planes = (int64_t)B * heads;
    const int64_t n = planes * H * W * D;
    const int side = 2 * ks - 1;
    const int64_t nb = (int64_t)heads * side * side;
    memset(dk, 0, sizeof(double) * n);
    memset(dv, 0, sizeof(double) * n);
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (planes < nthreads)
        nthreads = (int)planes;
    double *tables = (double *)calloc((size_t)nthreads * nb, sizeof(double));
    if (!tables)
        return ORACLE_NO_MEMORY;
    oracle_bwd_job jobs[256];
    pthread_t tids[256];
    int created[256];
    const int64_t chunk = (planes + nthreads - 1) / nthreads;
    int failed = 0;
    for (int t = 0; t < nthreads; ++t) {
        oracle_bwd_job *jb = &jobs[t];
        jb->q = q; jb->k = k; jb->v = v; jb->rpb = rpb; jb->dout = dout;
        jb->B = B; jb->heads = heads; jb->H = H; jb->W = W; jb->D = D;
        jb->ks = ks; jb->dil = dil;
        jb->plane0 = (int64_t)t * chunk;
        jb->plane1 = jb->plane0 + chunk < planes ? jb->plane0 + chunk : planes;
        jb->dq = dq; jb->dk = dk; jb->dv = dv; jb->drpb = tables + (int64_t)t * nb;
        created[t] = 0;
        if (jb->plane0 >= jb->plane1)
            continue;
        if (pthread_create(&tids[t], NULL, oracle_bwd_worker, jb) == 0)
            created[t] = 1;
        else if (oracle_bwd_worker(jb))
            failed = 1;
    }
    for (int t = 0; t < nthreads; ++t) {
        if (!created[t])
            continue;
        void *rc = NULL;
        pthread_join(tids[t], &rc);
        if (rc)
            failed = 1;
    }
    for (int64_t e = 0; e < nb; ++e) {
        double acc = 0.0;
        for (int t = 0; t < nthreads; ++t)
            acc += tables[(int64_t)t * nb + e];
        drpb[e] = acc;
    }
    free(tables);
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* 1 when H, W, kernel size and dilation form a valid problem. */
int na2d_oracle_valid(int H, int W, int ks, int dil)
{
    return ks >= 1 && (ks % 2) == 1 && dil >= 1 && H >= ks * dil && W >= ks * dil;
}
