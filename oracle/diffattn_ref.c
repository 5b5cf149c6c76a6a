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

/* Number of OpenMP threads a parallel region with nthreads <= 0 would use. */
int diffattn_ref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
