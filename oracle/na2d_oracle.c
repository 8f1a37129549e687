/*
 * na2d_oracle.c -- plain, slow, obviously-correct CPU oracle for the forward
 * pass of 2D (dilated) Neighborhood Attention.
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
 * The function returns, per requested query, the output row and optionally
 * the scores S, the probabilities P, the flat neighbour pixel index of every
 * window slot and the arg-max of S (lowest n wins ties).
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
    double *out, *scores, *probs;
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
 * out [nq, D]; scores, probs [nq, k*k] (optional); nbr [nq, k*k] flat pixel
 * index i*W+j (optional); argmax [nq] (optional).
 */
int na2d_oracle_forward(const double *q, const double *k, const double *v, const double *rpb,
                        int B, int heads, int H, int W, int D, int ks, int dil,
                        const int64_t *qidx, int64_t nq,
                        double *out, double *scores, double *probs,
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
        jb->out = out; jb->scores = scores; jb->probs = probs;
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

/* 1 when H, W, kernel size and dilation form a valid problem. */
int na2d_oracle_valid(int H, int W, int ks, int dil)
{
    return ks >= 1 && (ks % 2) == 1 && dil >= 1 && H >= ks * dil && W >= ks * dil;
}
