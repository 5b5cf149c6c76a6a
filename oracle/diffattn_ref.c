/*
 * diffattn_ref.c -- fp64 CPU oracle of the differential-attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file or the library built from it.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg use it.  It shares no
 * code, header or constant with the HIP library.
 *
 * What it computes (sources: the DiffTransformer.py page of
 * Differential-Transformer-PyTorch, MultiHeadDifferentialAttention.forward and
 * RMSNorm.forward; the LlamaDiffSdpaAttention.py gist, forward; the unilm pull
 * request "Add an isolated implementation of FlashDiffAttention",
 * alternative_forward):
 *
 *   lambda_h = exp(sum_c lq1_h[c]*lk1_h[c]) - exp(sum_c lq2_h[c]*lk2_h[c])
 *              + lambda_init
 *              (one set of vectors shared by all heads, or one per head as
 *              the DiffTransformer page keeps them: lq1_h = lq1 + h*stride)
 *   optional rotary prologue (the pull request's apply_rotary_emb with
 *   interleaved=True on every d-wide half-head of q and k): the pair
 *   (x[2j], x[2j+1]) of a row at sequence position p is turned by the angle
 *   of table row p, column j;
 *   for every packed sequence s (tokens a .. a+n-1), head h, row i:
 *     g      = h / (H / Hkv)                  (GQA: contiguous head groups)
 *     map m in {1,2}: x_j = <Qm[a+i,h], Km[a+j,g]> / sqrt(d), j in J(i)
 *                     J(i) = {0..i} when causal, else {0..n-1}
 *                     A_m  = softmax_j(x_j)
 *     pre    = sum_j (A_1[j] - lambda_h * A_2[j]) * V[a+j, g, :]   (2d wide)
 *     out    = pre / sqrt(mean_c pre[c]^2 + eps) * w * (1 - lambda_init)
 *
 * Against a key/value cache (diffattn_ref_fwd_kv; the Llama gist's forward
 * appends the new keys and values to the cache before attending), sequence s
 * has nq new queries and nk >= nq keys, the queries' own keys last; causal
 * row i sees keys {0 .. nk - nq + i}, the bottom-right alignment of the pull
 * request's mask (upper triangle above diagonal 1 + src_len - tgt_len).
 * With nq = nk this is the prefill above.
 *
 * Each softmax is taken the plain two-pass way (maximum, then exponentials
 * and their sum), every operation in IEEE double.  Inputs arrive as fp32
 * arrays: every bf16 or fp32 input value is exactly representable there, and
 * each is widened to double before use.
 *
 * Parity of every function here is pinned by the CPU tests against an mpmath
 * brute force of the materialised form, torch's scaled_dot_product_attention
 * and rms_norm on special inputs, and closed forms (row 0, uniform attention,
 * identical maps, lambda = 0).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* The decaying initial value of lambda for a layer at 1-based depth, as the
 * DiffTransformer model builds its layers (DiffTransformer.__init__). */
double diffattn_ref_lambda_init(int depth)
{
    return 0.8 - 0.6 * exp(-0.3 * (double)(depth - 1));
}

/* The re-parameterised lambda (MultiHeadDifferentialAttention.forward) of
 * one set of four length-d vectors.  The Llama gist and the pull request's
 * alternative_forward share one set among all heads; the DiffTransformer page
 * keeps one set per head. */
double diffattn_ref_lambda(const float *lq1, const float *lk1,
                           const float *lq2, const float *lk2, int d,
                           double lambda_init)
{
    double dot1 = 0.0, dot2 = 0.0;
    for (int c = 0; c < d; ++c) {
        dot1 += (double)lq1[c] * (double)lk1[c];
        dot2 += (double)lq2[c] * (double)lk2[c];
    }
    return exp(dot1) - exp(dot2) + lambda_init;
}

/* lambda of every head: lam[h] from the vectors at offset h * stride
 * (stride 0: the same vectors for every head). */
static void lambda_per_head(const float *lq1, const float *lk1,
                            const float *lq2, const float *lk2, int64_t stride,
                            int H, int d, double lambda_init, double *lam)
{
    for (int h = 0; h < H; ++h) {
        const int64_t o = (int64_t)h * stride;
        lam[h] = diffattn_ref_lambda(lq1 + o, lk1 + o, lq2 + o, lk2 + o, d,
                                     lambda_init);
    }
}

/* Rotary position tables (the pull request passes them as rel_pos, built by
 * RotaryEmbedding(head_dim, base, interleaved=True)): row p holds
 * cos(p * theta_j) and sin(p * theta_j), j < d/2.  cos == NULL: no rotation
 * (the inputs are already rotated). */
typedef struct {
    const float *cos;
    const float *sin;
    int64_t len;
    int round_bf16;   /* store rotated rows as bf16, as a bf16 pipeline does */
} rope_t;

/* x rounded to the nearest bfloat16 (ties to even), by way of the nearest
 * float: the value a bf16 tensor holds after a float result is stored. */
static double to_bf16(double x)
{
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, sizeof(u));
    u += 0x7fffu + ((u >> 16) & 1u);
    u &= 0xffff0000u;
    memcpy(&f, &u, sizeof(f));
    return (double)f;
}

/* One d-wide half-head row x at sequence position pos, rotated the
 * interleaved way: the pair (x[2j], x[2j+1]) is turned by the angle whose
 * cosine and sine are row pos, column j of the tables (the complex number
 * x[2j] + i x[2j+1] times exp(i angle)).  Widened to double; with
 * round_bf16 the rotated values are then rounded to bfloat16, since the
 * pull request's pipeline stores the rotated q and k in its bf16 storage
 * type before the attention reads them. */
static void row_rot(const float *x, int d, const rope_t *rp, int64_t pos,
                    double *out)
{
    if (!rp->cos) {
        for (int c = 0; c < d; ++c)
            out[c] = (double)x[c];
        return;
    }
    const float *cr = rp->cos + pos * (int64_t)(d / 2);
    const float *sr = rp->sin + pos * (int64_t)(d / 2);
    for (int j = 0; j < d / 2; ++j) {
        const double x0 = (double)x[2 * j], x1 = (double)x[2 * j + 1];
        const double c = (double)cr[j], sn = (double)sr[j];
        out[2 * j] = x0 * c - x1 * sn;
        out[2 * j + 1] = x0 * sn + x1 * c;
    }
    if (rp->round_bf16)
        for (int c = 0; c < d; ++c)
            out[c] = to_bf16(out[c]);
}

/* Softmax of one attention map over the keys j in [0, nkeys) that start at
 * key token ka, for query token qt (sequence position qpos; key j sits at
 * position j) of head h: writes the probabilities into p[0..nkeys).
 * qd and kd are scratch of d doubles. */
static void softmax_map(const float *q, const float *k, int64_t qt, int64_t qpos,
                        int64_t ka, int64_t nkeys, int h, int g, int map, int H,
                        int Hkv, int d, const rope_t *rp, double *qd,
                        double *kd, double *p)
{
    row_rot(q + ((qt * H + h) * 2 + map) * (int64_t)d, d, rp, qpos, qd);
    const double scale = 1.0 / sqrt((double)d);
    double mx = -INFINITY;
    for (int64_t j = 0; j < nkeys; ++j) {
        row_rot(k + (((ka + j) * Hkv + g) * 2 + map) * (int64_t)d, d, rp, j, kd);
        double x = 0.0;
        for (int c = 0; c < d; ++c)
            x += qd[c] * kd[c];
        x *= scale;
        p[j] = x;
        if (x > mx)
            mx = x;
    }
    double z = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        p[j] = exp(p[j] - mx);
        z += p[j];
    }
    for (int64_t j = 0; j < nkeys; ++j)
        p[j] /= z;
}

/* One output row (query token qt at sequence position qpos, head h) over
 * the nkeys keys that start at key token ka, into o[0..2d).  sc is
 * caller-provided scratch of 2 nkeys + 4d doubles. */
static void diff_row(const float *q, const float *k, const float *v,
                     double lam, double lambda_init, const float *w, double eps,
                     int64_t qt, int64_t qpos, int64_t ka, int64_t nkeys, int h,
                     int H, int Hkv, int d, const rope_t *rp, double *sc,
                     double *o)
{
    const int g = h / (H / Hkv);
    const int dv = 2 * d;
    double *p1 = sc, *p2 = sc + nkeys, *pre = sc + 2 * nkeys;
    double *qd = pre + dv, *kd = qd + d;
    softmax_map(q, k, qt, qpos, ka, nkeys, h, g, 0, H, Hkv, d, rp, qd, kd, p1);
    softmax_map(q, k, qt, qpos, ka, nkeys, h, g, 1, H, Hkv, d, rp, qd, kd, p2);
    for (int c = 0; c < dv; ++c)
        pre[c] = 0.0;
    for (int64_t j = 0; j < nkeys; ++j) {
        const double coef = p1[j] - lam * p2[j];
        const float *vrow = v + ((ka + j) * Hkv + g) * (int64_t)dv;
        for (int c = 0; c < dv; ++c)
            pre[c] += coef * (double)vrow[c];
    }
    double ss = 0.0;
    for (int c = 0; c < dv; ++c)
        ss += pre[c] * pre[c];
    const double rms = sqrt(ss / (double)dv + eps);
    for (int c = 0; c < dv; ++c) {
        const double wc = w ? (double)w[c] : 1.0;
        o[c] = pre[c] / rms * wc * (1.0 - lambda_init);
    }
}

/* Keys visible to row i (0-based) of a sequence of n tokens attending to
 * itself: its prefix when causal, the whole sequence otherwise. */
static int64_t prefill_keys(int causal, int64_t i, int64_t n)
{
    return causal ? i + 1 : n;
}

static int check_args(const int32_t *cu, int nseq, int64_t T, int H, int Hkv,
                      int d)
{
    if (nseq < 0 || T < 0 || H < 1 || Hkv < 1 || d < 1 || H % Hkv != 0)
        return -1;
    if (!cu)
        return -1;
    if (cu[0] != 0 || cu[nseq] != T)
        return -1;
    for (int s = 0; s < nseq; ++s)
        if (cu[s + 1] < cu[s])
            return -1;
    return 0;
}

static int64_t max_len(const int32_t *cu, int nseq)
{
    int64_t m = 0;
    for (int s = 0; s < nseq; ++s)
        if (cu[s + 1] - cu[s] > m)
            m = cu[s + 1] - cu[s];
    return m;
}

/* Full forward pass: out[T, H, 2d] in double.  cu_seqlens[nseq+1] holds the
 * packed sequence boundaries (host).  rope_cos / rope_sin: rotary tables
 * [rope_len, d/2] (rope_len >= the longest sequence) or NULL for inputs that
 * are already rotated; rope_round_bf16 rounds the rotated rows to bf16.
 * nthreads <= 0 uses the OpenMP default.
 * Returns 0, or -1 on malformed arguments, -2 if scratch memory is short. */
int diffattn_ref_fwd(const float *q, const float *k, const float *v,
                     const float *lq1, const float *lk1, const float *lq2,
                     const float *lk2, int64_t lambda_stride,
                     double lambda_init, const float *w, double eps, int causal,
                     const int32_t *cu_seqlens, int nseq, int64_t T, int H,
                     int Hkv, int d, const float *rope_cos,
                     const float *rope_sin, int64_t rope_len, int rope_round_bf16,
                     double *out, int nthreads)
{
    if (check_args(cu_seqlens, nseq, T, H, Hkv, d) || lambda_stride < 0)
        return -1;
    const rope_t rp = {rope_cos, rope_sin, rope_len, rope_round_bf16};
    if (rope_cos && (!rope_sin || d % 2 || rope_len < max_len(cu_seqlens, nseq)))
        return -1;
    double *lam = malloc(sizeof(double) * (size_t)H);
    if (!lam)
        return -2;
    lambda_per_head(lq1, lk1, lq2, lk2, lambda_stride, H, d, lambda_init, lam);
    const int64_t nmax = max_len(cu_seqlens, nseq);
    const int64_t nrows = T * H;
    int err = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *scratch = malloc(sizeof(double) * (size_t)(2 * nmax + 4 * d + 1));
        if (!scratch) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = -2;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 8)
#endif
        for (int64_t r = 0; r < nrows; ++r) {
            if (!scratch)
                continue;
            const int64_t t = r / H;
            const int h = (int)(r % H);
            int s = 0;
            while (cu_seqlens[s + 1] <= t)
                ++s;
            const int64_t a = cu_seqlens[s];
            const int64_t n = cu_seqlens[s + 1] - a;
            diff_row(q, k, v, lam[h], lambda_init, w, eps, t, t - a, a,
                     prefill_keys(causal, t - a, n), h, H, Hkv, d, &rp,
                     scratch, out + r * 2 * (int64_t)d);
        }
        free(scratch);
    }
    free(lam);
    return err;
}

/* Selected rows only: row r is (token tok[r], head head[r]); writes
 * out_rows[nrows, 2d].  Used to check full-size runs on a sample. */
int diffattn_ref_rows(const float *q, const float *k, const float *v,
                      const float *lq1, const float *lk1, const float *lq2,
                      const float *lk2, int64_t lambda_stride,
                      double lambda_init, const float *w, double eps,
                      int causal, const int32_t *cu_seqlens, int nseq,
                      int64_t T, int H, int Hkv, int d, const float *rope_cos,
                      const float *rope_sin, int64_t rope_len,
                      int rope_round_bf16, const int64_t *tok,
                      const int32_t *head, int64_t nrows, double *out_rows,
                      int nthreads)
{
    if (check_args(cu_seqlens, nseq, T, H, Hkv, d) || lambda_stride < 0)
        return -1;
    const rope_t rp = {rope_cos, rope_sin, rope_len, rope_round_bf16};
    if (rope_cos && (!rope_sin || d % 2 || rope_len < max_len(cu_seqlens, nseq)))
        return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (tok[r] < 0 || tok[r] >= T || head[r] < 0 || head[r] >= H)
            return -1;
    double *lam = malloc(sizeof(double) * (size_t)H);
    if (!lam)
        return -2;
    lambda_per_head(lq1, lk1, lq2, lk2, lambda_stride, H, d, lambda_init, lam);
    const int64_t nmax = max_len(cu_seqlens, nseq);
    int err = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *scratch = malloc(sizeof(double) * (size_t)(2 * nmax + 4 * d + 1));
        if (!scratch) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = -2;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t r = 0; r < nrows; ++r) {
            if (!scratch)
                continue;
            const int64_t t = tok[r];
            int s = 0;
            while (cu_seqlens[s + 1] <= t)
                ++s;
            const int64_t a = cu_seqlens[s];
            const int64_t n = cu_seqlens[s + 1] - a;
            diff_row(q, k, v, lam[head[r]], lambda_init, w, eps, t, t - a, a,
                     prefill_keys(causal, t - a, n), head[r], H, Hkv, d, &rp,
                     scratch, out_rows + r * 2 * (int64_t)d);
        }
        free(scratch);
    }
    free(lam);
    return err;
}

/* New queries against a key/value cache: sequence s has nq = cu_q[s+1] -
 * cu_q[s] query tokens (in q) and nk = cu_k[s+1] - cu_k[s] key tokens (in k,
 * v; the queries' own keys are the last nq of them).  Causal alignment is
 * bottom-right, as the pull request's alternative_forward builds its mask
 * with triu(-inf, 1 + src_len - tgt_len): query i sees keys j <= nk - nq + i.
 * Not causal: every key of the sequence.  out[Tq, H, 2d].  Returns 0, -1 on
 * malformed arguments (including causal with nq > nk), -2 without memory. */
int diffattn_ref_fwd_kv(const float *q, const float *k, const float *v,
                        const float *lq1, const float *lk1, const float *lq2,
                        const float *lk2, int64_t lambda_stride,
                        double lambda_init, const float *w, double eps,
                        int causal, const int32_t *cu_q, const int32_t *cu_k,
                        int nseq, int64_t Tq, int64_t Tk, int H, int Hkv, int d,
                        double *out, int nthreads)
{
    if (check_args(cu_q, nseq, Tq, H, Hkv, d) || check_args(cu_k, nseq, Tk, H, Hkv, d) ||
        lambda_stride < 0)
        return -1;
    for (int s = 0; s < nseq; ++s) {
        const int64_t nq = cu_q[s + 1] - cu_q[s], nk = cu_k[s + 1] - cu_k[s];
        if ((causal && nq > nk) || (nq > 0 && nk == 0))
            return -1;
    }
    double *lam = malloc(sizeof(double) * (size_t)H);
    if (!lam)
        return -2;
    lambda_per_head(lq1, lk1, lq2, lk2, lambda_stride, H, d, lambda_init, lam);
    const int64_t nmax = max_len(cu_k, nseq);
    const rope_t no_rope = {NULL, NULL, 0, 0};
    const int64_t nrows = Tq * H;
    int err = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *scratch = malloc(sizeof(double) * (size_t)(2 * nmax + 4 * d + 1));
        if (!scratch) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = -2;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 8)
#endif
        for (int64_t r = 0; r < nrows; ++r) {
            if (!scratch)
                continue;
            const int64_t t = r / H;
            const int h = (int)(r % H);
            int s = 0;
            while (cu_q[s + 1] <= t)
                ++s;
            const int64_t nq = cu_q[s + 1] - cu_q[s];
            const int64_t nk = cu_k[s + 1] - cu_k[s];
            const int64_t i = t - cu_q[s];
            const int64_t nkeys = causal ? nk - nq + i + 1 : nk;
            diff_row(q, k, v, lam[h], lambda_init, w, eps, t, nk - nq + i,
                     cu_k[s], nkeys, h, H, Hkv, d, &no_rope, scratch,
                     out + r * 2 * (int64_t)d);
        }
        free(scratch);
    }
    free(lam);
    return err;
}

/* Backward of the prefill (inputs already rotated; no rotary prologue).
 * Given the output gradient dy[T, H, 2d], writes in double:
 *   dq[T, H, 2, d], dk[T, Hkv, 2, d], dv[T, Hkv, 2d];
 *   dlq1, dlk1, dlq2, dlk2: gradients of the lambda vectors, laid out like
 *     them (lambda_stride 0: one set of d; else H sets, stride apart);
 *   dw[2d]: gradient of the RMSNorm weight (of a weight of ones when w is
 *     NULL);
 *   dlam_head[H]: dlambda_h, and dlam_scale[H]: the sum over the head's rows
 *     of |dpre| |O_2| (Euclidean norms), which bounds how much a relative
 *     error in O_2 or dpre can move dlambda_h (the sum can cancel).
 * The chain, per row (token i, head h) of the forward above:
 *   g = dy * w * (1 - lambda_init);  r = 1 / sqrt(mean(pre^2) + eps)
 *   dpre = r g - r^3 pre <g, pre> / (2d);   dw += dy * pre * r * (1 - lambda_init)
 *   dO_1 = dpre;  dO_2 = -lambda dpre;  dlambda_h += -<dpre, O_2>
 *   per map m: D_m = <dO_m, O_m>;  dS_m[j] = P_m[j] (<dO_m, V_j> - D_m)
 *     dQ_m[i] += scale sum_j dS_m[j] K_m[j];  dK_m[j] += scale dS_m[j] Q_m[i]
 *     dV[j] += P_m[j] dO_m
 *   lambda = exp(a) - exp(b) + lambda_init with a = <lq1, lk1>, b = <lq2, lk2>:
 *     dlq1 = dlambda e^a lk1, dlk1 = dlambda e^a lq1,
 *     dlq2 = -dlambda e^b lk2, dlk2 = -dlambda e^b lq2
 * Work is split by (sequence, KV head), so every dk/dv element has one
 * writer; dlambda and dw are summed per task and reduced in task order.
 * Returns 0, -1 on malformed arguments, -2 without memory. */
int diffattn_ref_bwd(const float *q, const float *k, const float *v,
                     const float *lq1, const float *lk1, const float *lq2,
                     const float *lk2, int64_t lambda_stride, double lambda_init,
                     const float *w, double eps, int causal,
                     const int32_t *cu_seqlens, int nseq, int64_t T, int H,
                     int Hkv, int d, const float *dy, double *dq, double *dk,
                     double *dv, double *dlq1, double *dlk1, double *dlq2,
                     double *dlk2, double *dw, double *dlam_head,
                     double *dlam_scale, int nthreads)
{
    if (check_args(cu_seqlens, nseq, T, H, Hkv, d) || lambda_stride < 0)
        return -1;
    const int G = H / Hkv, dv2 = 2 * d;
    const int64_t ntask = (int64_t)nseq * Hkv;
    double *lam = malloc(sizeof(double) * (size_t)H);
    double *tdl = calloc((size_t)(ntask * H), sizeof(double));   /* dlambda per task, head */
    double *tds = calloc((size_t)(ntask * H), sizeof(double));   /* its scale */
    double *tdw = calloc((size_t)(ntask * dv2), sizeof(double)); /* dw per task */
    if (!lam || !tdl || !tdw || !tds) {
        free(lam);
        free(tdl);
        free(tdw);
        free(tds);
        return -2;
    }
    lambda_per_head(lq1, lk1, lq2, lk2, lambda_stride, H, d, lambda_init, lam);
    memset(dq, 0, sizeof(double) * (size_t)(T * H * 2 * d));
    memset(dk, 0, sizeof(double) * (size_t)(T * Hkv * 2 * d));
    memset(dv, 0, sizeof(double) * (size_t)(T * Hkv * dv2));
    const int64_t nmax = max_len(cu_seqlens, nseq);
    const double scale = 1.0 / sqrt((double)d);
    int err = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        /* p1, p2 [nmax]; o1, o2, pre, do1, do2 [2d] */
        double *sc = malloc(sizeof(double) * (size_t)(2 * nmax + 5 * dv2 + 1));
        if (!sc) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = -2;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t task = 0; task < ntask; ++task) {
            if (!sc)
                continue;
            const int s = (int)(task / Hkv), g = (int)(task % Hkv);
            const int64_t a = cu_seqlens[s], n = cu_seqlens[s + 1] - a;
            double *p[2] = {sc, sc + nmax};
            double *o[2] = {sc + 2 * nmax, sc + 2 * nmax + dv2};
            double *pre = o[1] + dv2, *dO[2] = {pre + dv2, pre + 2 * dv2};
            for (int h = g * G; h < (g + 1) * G; ++h) {
                for (int64_t i = 0; i < n; ++i) {
                    const int64_t t = a + i, nk = prefill_keys(causal, i, n);
                    /* forward of the row: both maps, O_m normalised */
                    for (int m = 0; m < 2; ++m) {
                        const float *qr = q + ((t * H + h) * 2 + m) * (int64_t)d;
                        double mx = -INFINITY;
                        for (int64_t j = 0; j < nk; ++j) {
                            const float *kr = k + (((a + j) * Hkv + g) * 2 + m) * (int64_t)d;
                            double x = 0.0;
                            for (int c = 0; c < d; ++c)
                                x += (double)qr[c] * (double)kr[c];
                            p[m][j] = x * scale;
                            if (p[m][j] > mx)
                                mx = p[m][j];
                        }
                        double z = 0.0;
                        for (int64_t j = 0; j < nk; ++j) {
                            p[m][j] = exp(p[m][j] - mx);
                            z += p[m][j];
                        }
                        for (int c = 0; c < dv2; ++c)
                            o[m][c] = 0.0;
                        for (int64_t j = 0; j < nk; ++j) {
                            p[m][j] /= z;
                            const float *vr = v + ((a + j) * Hkv + g) * (int64_t)dv2;
                            for (int c = 0; c < dv2; ++c)
                                o[m][c] += p[m][j] * (double)vr[c];
                        }
                    }
                    double ss = 0.0;
                    for (int c = 0; c < dv2; ++c) {
                        pre[c] = o[0][c] - lam[h] * o[1][c];
                        ss += pre[c] * pre[c];
                    }
                    const double r = 1.0 / sqrt(ss / (double)dv2 + eps);
                    /* RMSNorm, weight and scale backward */
                    const float *dyr = dy + (t * H + h) * (int64_t)dv2;
                    double gp = 0.0;
                    for (int c = 0; c < dv2; ++c) {
                        const double wc = w ? (double)w[c] : 1.0;
                        gp += (double)dyr[c] * wc * (1.0 - lambda_init) * pre[c];
                        tdw[task * dv2 + c] += (double)dyr[c] * pre[c] * r * (1.0 - lambda_init);
                    }
                    double dl = 0.0, nd = 0.0, no = 0.0;
                    for (int c = 0; c < dv2; ++c) {
                        const double wc = w ? (double)w[c] : 1.0;
                        const double gc = (double)dyr[c] * wc * (1.0 - lambda_init);
                        const double dp = r * gc - r * r * r * pre[c] * gp / (double)dv2;
                        dO[0][c] = dp;
                        dO[1][c] = -lam[h] * dp;
                        dl -= dp * o[1][c];
                        nd += dp * dp;
                        no += o[1][c] * o[1][c];
                    }
                    tdl[task * H + h] += dl;
                    tds[task * H + h] += sqrt(nd) * sqrt(no);
                    /* both softmax maps */
                    for (int m = 0; m < 2; ++m) {
                        double D = 0.0;
                        for (int c = 0; c < dv2; ++c)
                            D += dO[m][c] * o[m][c];
                        const float *qr = q + ((t * H + h) * 2 + m) * (int64_t)d;
                        double *dqr = dq + ((t * H + h) * 2 + m) * (int64_t)d;
                        for (int64_t j = 0; j < nk; ++j) {
                            const float *vr = v + ((a + j) * Hkv + g) * (int64_t)dv2;
                            double dpj = 0.0;
                            for (int c = 0; c < dv2; ++c)
                                dpj += dO[m][c] * (double)vr[c];
                            const double ds = p[m][j] * (dpj - D);
                            const float *kr = k + (((a + j) * Hkv + g) * 2 + m) * (int64_t)d;
                            double *dkr = dk + (((a + j) * Hkv + g) * 2 + m) * (int64_t)d;
                            for (int c = 0; c < d; ++c) {
                                dqr[c] += scale * ds * (double)kr[c];
                                dkr[c] += scale * ds * (double)qr[c];
                            }
                            double *dvr = dv + ((a + j) * Hkv + g) * (int64_t)dv2;
                            for (int c = 0; c < dv2; ++c)
                                dvr[c] += p[m][j] * dO[m][c];
                        }
                    }
                }
            }
        }
        free(sc);
    }
    if (!err) {
        /* reduce in task order; lambda-vector gradients by the chain rule */
        for (int c = 0; c < dv2; ++c) {
            double acc = 0.0;
            for (int64_t t2 = 0; t2 < ntask; ++t2)
                acc += tdw[t2 * dv2 + c];
            dw[c] = acc;
        }
        for (int h = 0; h < H; ++h) {
            double a2 = 0.0, s2 = 0.0;
            for (int64_t t2 = 0; t2 < ntask; ++t2) {
                a2 += tdl[t2 * H + h];
                s2 += tds[t2 * H + h];
            }
            dlam_head[h] = a2;
            dlam_scale[h] = s2;
        }
        const int nsets = lambda_stride ? H : 1;
        for (int st = 0; st < nsets; ++st) {
            double dlam = 0.0;
            for (int h = 0; h < H; ++h)
                if (!lambda_stride || h == st)
                    for (int64_t t2 = 0; t2 < ntask; ++t2)
                        dlam += tdl[t2 * H + h];
            const int64_t off = (int64_t)st * lambda_stride;
            double a1 = 0.0, b1 = 0.0;
            for (int c = 0; c < d; ++c) {
                a1 += (double)lq1[off + c] * (double)lk1[off + c];
                b1 += (double)lq2[off + c] * (double)lk2[off + c];
            }
            const double ea = exp(a1), eb = exp(b1);
            for (int c = 0; c < d; ++c) {
                dlq1[off + c] = dlam * ea * (double)lk1[off + c];
                dlk1[off + c] = dlam * ea * (double)lq1[off + c];
                dlq2[off + c] = -dlam * eb * (double)lk2[off + c];
                dlk2[off + c] = -dlam * eb * (double)lq2[off + c];
            }
        }
    }
    free(lam);
    free(tdl);
    free(tdw);
    free(tds);
    return err;
}

/* The backward quantities of one row (token t at sequence position i of a
 * sequence starting at token a, head h, KV head g): for both maps the
 * natural log-sum-exp of the scaled scores over the nk visible keys, dO_m
 * (2d each) and D_m = <dO_m, O_m>.  p is scratch of nk doubles, o of 4d. */
static void bwd_row_stats(const float *q, const float *k, const float *v,
                          double lam, double lambda_init, const float *w,
                          double eps, const float *dy, int64_t t, int64_t a,
                          int64_t nk, int h, int g, int H, int Hkv, int d,
                          double *p, double *o, double lse[2],
                          double *dO /* [2][2d] */, double D[2])
{
    const int dv2 = 2 * d;
    const double scale = 1.0 / sqrt((double)d);
    for (int m = 0; m < 2; ++m) {
        const float *qr = q + ((t * H + h) * 2 + m) * (int64_t)d;
        double mx = -INFINITY;
        for (int64_t j = 0; j < nk; ++j) {
            const float *kr = k + (((a + j) * Hkv + g) * 2 + m) * (int64_t)d;
            double x = 0.0;
            for (int c = 0; c < d; ++c)
                x += (double)qr[c] * (double)kr[c];
            p[j] = x * scale;
            if (p[j] > mx)
                mx = p[j];
        }
        double z = 0.0;
        for (int64_t j = 0; j < nk; ++j)
            z += exp(p[j] - mx);
        lse[m] = mx + log(z);
        double *om = o + m * dv2;
        for (int c = 0; c < dv2; ++c)
            om[c] = 0.0;
        for (int64_t j = 0; j < nk; ++j) {
            const double pj = exp(p[j] - lse[m]);
            const float *vr = v + ((a + j) * Hkv + g) * (int64_t)dv2;
            for (int c = 0; c < dv2; ++c)
                om[c] += pj * (double)vr[c];
        }
    }
    double ss = 0.0, gp = 0.0;
    const float *dyr = dy + (t * H + h) * (int64_t)dv2;
    for (int c = 0; c < dv2; ++c) {
        const double pre = o[c] - lam * o[dv2 + c];
        ss += pre * pre;
    }
    const double r = 1.0 / sqrt(ss / (double)dv2 + eps);
    for (int c = 0; c < dv2; ++c) {
        const double pre = o[c] - lam * o[dv2 + c];
        gp += (double)dyr[c] * (w ? (double)w[c] : 1.0) * (1.0 - lambda_init) * pre;
    }
    D[0] = D[1] = 0.0;
    for (int c = 0; c < dv2; ++c) {
        const double pre = o[c] - lam * o[dv2 + c];
        const double gc = (double)dyr[c] * (w ? (double)w[c] : 1.0) * (1.0 - lambda_init);
        const double dp = r * gc - r * r * r * pre * gp / (double)dv2;
        dO[c] = dp;
        dO[dv2 + c] = -lam * dp;
        D[0] += dO[c] * o[c];
        D[1] += dO[dv2 + c] * o[dv2 + c];
    }
}

/* Gradients on a sample, for checking full-size runs: dq of the rows
 * (tok_q[r], head_q[r]) into dq_out[nq][2][d], and dk, dv of the key rows
 * (tok_k[r], kvhead_k[r]) into dk_out[nk][2][d], dv_out[nk][2d]; same
 * inputs and definitions as diffattn_ref_bwd.  A sampled key needs every
 * row of its sequence and group that can see it; each such row's
 * statistics are computed once and applied to all sampled keys of that
 * (sequence, KV head).  Returns 0, -1 on malformed arguments, -2 without
 * memory. */
int diffattn_ref_bwd_sample(const float *q, const float *k, const float *v,
                            const float *lq1, const float *lk1,
                            const float *lq2, const float *lk2,
                            int64_t lambda_stride, double lambda_init,
                            const float *w, double eps, int causal,
                            const int32_t *cu_seqlens, int nseq, int64_t T,
                            int H, int Hkv, int d, const float *dy,
                            int64_t nrq, const int64_t *tok_q,
                            const int32_t *head_q, double *dq_out,
                            int64_t nrk, const int64_t *tok_k,
                            const int32_t *kvhead_k, double *dk_out,
                            double *dv_out, int nthreads)
{
    if (check_args(cu_seqlens, nseq, T, H, Hkv, d) || lambda_stride < 0)
        return -1;
    for (int64_t r = 0; r < nrq; ++r)
        if (tok_q[r] < 0 || tok_q[r] >= T || head_q[r] < 0 || head_q[r] >= H)
            return -1;
    for (int64_t r = 0; r < nrk; ++r)
        if (tok_k[r] < 0 || tok_k[r] >= T || kvhead_k[r] < 0 || kvhead_k[r] >= Hkv)
            return -1;
    const int G = H / Hkv, dv2 = 2 * d;
    const double scale = 1.0 / sqrt((double)d);
    double *lam = malloc(sizeof(double) * (size_t)H);
    if (!lam)
        return -2;
    lambda_per_head(lq1, lk1, lq2, lk2, lambda_stride, H, d, lambda_init, lam);
    const int64_t nmax = max_len(cu_seqlens, nseq);
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#else
    nthreads = 1;
#endif
    /* per-thread accumulators of the sampled keys' dk and dv */
    const int64_t per = nrk * (2 * d + dv2);
    double *acc = calloc((size_t)(nthreads * per + 1), sizeof(double));
    int err = acc ? 0 : -2;
    /* work items: sampled query rows, then (row token, head) pairs that some
     * sampled key needs */
    const int64_t nitems = nrq + T * H;
#ifdef _OPENMP
#pragma omp parallel num_threads(nthreads)
#endif
    {
#ifdef _OPENMP
        const int tid = omp_get_thread_num();
#else
        const int tid = 0;
#endif
        double *sc = malloc(sizeof(double) * (size_t)(nmax + 4 * dv2 + 8));
        if (!sc || !acc) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = -2;
        }
#ifdef _OPENMP
#pragma omp for schedule(static, 1)
#endif
        for (int64_t it = 0; it < nitems; ++it) {
            if (!sc || !acc)
                continue;
            int64_t t;
            int h;
            if (it < nrq) {
                t = tok_q[it];
                h = head_q[it];
            } else {
                t = (it - nrq) / H;
                h = (int)((it - nrq) % H);
            }
            const int g = h / G;
            int s = 0;
            while (cu_seqlens[s + 1] <= t)
                ++s;
            const int64_t a = cu_seqlens[s], n = cu_seqlens[s + 1] - a, i = t - a;
            const int64_t nk = prefill_keys(causal, i, n);
            if (it >= nrq) {
                /* does any sampled key of this sequence and group see row i? */
                int need = 0;
                for (int64_t r = 0; r < nrk && !need; ++r)
                    need = kvhead_k[r] == g && tok_k[r] >= a && tok_k[r] - a < nk;
                if (!need)
                    continue;
            }
            double *p = sc, *o = sc + nmax, *dO = o + 2 * dv2;
            double lse[2], D[2];
            bwd_row_stats(q, k, v, lam[h], lambda_init, w, eps, dy, t, a, nk, h, g,
                          H, Hkv, d, p, o, lse, dO, D);
            if (it < nrq) {
                double *dqr = dq_out + it * 2 * (int64_t)d;
                for (int m = 0; m < 2; ++m) {
                    for (int c = 0; c < d; ++c)
                        dqr[m * d + c] = 0.0;
                    const float *qr = q + ((t * H + h) * 2 + m) * (int64_t)d;
                    for (int64_t j = 0; j < nk; ++j) {
                        const float *kr = k + (((a + j) * Hkv + g) * 2 + m) * (int64_t)d;
                        const float *vr = v + ((a + j) * Hkv + g) * (int64_t)dv2;
                        double x = 0.0, dp = 0.0;
                        for (int c = 0; c < d; ++c)
                            x += (double)qr[c] * (double)kr[c];
                        for (int c = 0; c < dv2; ++c)
                            dp += dO[m * dv2 + c] * (double)vr[c];
                        const double ds = exp(x * scale - lse[m]) * (dp - D[m]);
                        for (int c = 0; c < d; ++c)
                            dqr[m * d + c] += scale * ds * (double)kr[c];
                    }
                }
                continue;
            }
            double *my = acc + tid * per;
            for (int64_t r = 0; r < nrk; ++r) {
                if (kvhead_k[r] != g || tok_k[r] < a || tok_k[r] - a >= nk)
                    continue;
                const int64_t j = tok_k[r];
                const float *vr = v + (j * Hkv + g) * (int64_t)dv2;
                double *dkr = my + r * (2 * d + dv2), *dvr = dkr + 2 * d;
                for (int m = 0; m < 2; ++m) {
                    const float *qr = q + ((t * H + h) * 2 + m) * (int64_t)d;
                    const float *kr = k + ((j * Hkv + g) * 2 + m) * (int64_t)d;
                    double x = 0.0, dp = 0.0;
                    for (int c = 0; c < d; ++c)
                        x += (double)qr[c] * (double)kr[c];
                    for (int c = 0; c < dv2; ++c)
                        dp += dO[m * dv2 + c] * (double)vr[c];
                    const double pj = exp(x * scale - lse[m]);
                    const double ds = pj * (dp - D[m]);
                    for (int c = 0; c < d; ++c)
                        dkr[m * d + c] += scale * ds * (double)qr[c];
                    for (int c = 0; c < dv2; ++c)
                        dvr[c] += pj * dO[m * dv2 + c];
                }
            }
        }
        free(sc);
    }
    if (!err) {
        for (int64_t r = 0; r < nrk; ++r) {
            for (int c = 0; c < 2 * d; ++c) {
                double x = 0.0;
                for (int th = 0; th < nthreads; ++th)
                    x += acc[th * per + r * (2 * d + dv2) + c];
                dk_out[r * 2 * d + c] = x;
            }
            for (int c = 0; c < dv2; ++c) {
                double x = 0.0;
                for (int th = 0; th < nthreads; ++th)
                    x += acc[th * per + r * (2 * d + dv2) + 2 * d + c];
                dv_out[r * dv2 + c] = x;
            }
        }
    }
    free(acc);
    free(lam);
    return err;
}

/* Number of OpenMP threads a parallel region with nthreads <= 0 would use. */
int diffattn_ref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
