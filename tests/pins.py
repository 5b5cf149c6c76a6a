"""Checks that pin the fp64 oracle to something other than itself.

Each ``pin_*`` function takes a loaded oracle library (``oracle.load(path)``)
and raises ``AssertionError`` when the oracle disagrees with:

* an mpmath brute force of the materialised form of the DiffTransformer.py
  page (MultiHeadDifferentialAttention.forward: two full masked score
  matrices, two softmaxes, their lambda-weighted difference times V, then the
  per-head RMSNorm and the (1 - lambda_init) scale), at 50 digits on tiny
  inputs;
* torch's ``scaled_dot_product_attention`` and ``rms_norm`` in fp64 (library
  routines), composed the way the LlamaDiffSdpaAttention.py gist composes two
  SDPA calls (attn1 - lambda * attn2, then subln, then the scale), with the
  library's own GQA broadcast (``enable_gqa``: head h reads KV head h // G,
  as ``repeat_kv`` does on that page);
* closed forms: lambda at special vectors, row 0 of every sequence, uniform
  attention (K = 0), identical maps with lambda = 1;
* invariants: causality, packing, GQA = MHA with repeated K/V, odd symmetry
  in V, the row-sampling entry point.

The same pins run against deliberately broken copies of the oracle source
(``tests/test_oracle_mutants.py``) to show that each plausible mistake fails
at least one of them.
"""

from __future__ import annotations

import math

import mpmath
import numpy as np
import torch
import torch.nn.functional as F

import oracle


# --------------------------------------------------------------------------
# tiny seeded inputs (fp32 values; the oracle widens them exactly)

def tiny_inputs(seed, seqlens, H, Hkv, d, q_scale=1.0, v_scale=1.0):
    rng = np.random.default_rng(seed)
    T = int(sum(seqlens))
    q = (rng.standard_normal((T, H, 2, d)) * q_scale).astype(np.float32)
    k = rng.standard_normal((T, Hkv, 2, d)).astype(np.float32)
    v = (rng.standard_normal((T, Hkv, 2 * d)) * v_scale).astype(np.float32)
    lv = [(0.3 * rng.standard_normal(d)).astype(np.float32) for _ in range(4)]
    w = (0.5 + rng.random(2 * d)).astype(np.float32)
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    return q, k, v, lv, w, cu


def run(lib, q, k, v, lv, lam_init, w, eps, causal, cu):
    return oracle.fwd(q, k, v, *lv, lam_init, w, eps, causal, cu, lib=lib)


# --------------------------------------------------------------------------
# mpmath brute force of the materialised two-map form

def brute_mpmath(q, k, v, lv, lam_init, w, eps, causal, cu, dps=50, cu_k=None,
                 rope=None):
    """With ``cu_k``, sequence s has its queries at ``cu[s]..`` and its keys
    at ``cu_k[s]..`` and a causal row i sees keys j <= i + nk - nq: the
    lower triangle of the pull request's mask, which puts -inf above
    diagonal 1 + src_len - tgt_len.  With ``rope`` = (cos, sin) tables, q and
    k rows at sequence position p are first multiplied, as complex numbers
    x[2j] + i x[2j+1], by cos[p, j] + i sin[p, j]."""
    mpmath.mp.dps = dps
    if cu_k is None:
        cu_k = cu
    if rope is not None:
        q, k = _rotate_mp(q, cu, rope), _rotate_mp(k, cu_k, rope)
    T, H, _, d = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    mpf = mpmath.mpf

    def lam_of(vecs):
        lq1, lk1, lq2, lk2 = [[mpf(float(x)) for x in a] for a in vecs]
        return (mpmath.exp(mpmath.fsum(a * b for a, b in zip(lq1, lk1)))
                - mpmath.exp(mpmath.fsum(a * b for a, b in zip(lq2, lk2)))
                + mpf(lam_init))
    if np.asarray(lv[0]).ndim == 2:     # one set of vectors per head
        lams = [lam_of([a[h] for a in lv]) for h in range(H)]
    else:
        lams = [lam_of(lv)] * H
    scaling = 1 / mpmath.sqrt(d)
    out = np.zeros((T, H, 2 * d))
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        n = b - a
        ka = int(cu_k[s])
        nk = int(cu_k[s + 1]) - ka
        for h in range(H):
            g = h // G
            lam = lams[h]
            A = []
            for m in range(2):
                Am = []
                for i in range(n):
                    row = []
                    for j in range(nk):
                        if causal and j > i + nk - n:
                            row.append(mpmath.ninf)
                            continue
                        x = mpmath.fsum(_mp(q[a + i, h, m, c])
                                        * _mp(k[ka + j, g, m, c])
                                        for c in range(d))
                        row.append(x * scaling)
                    mx = max(x for x in row if x != mpmath.ninf)
                    e = [mpmath.exp(x - mx) if x != mpmath.ninf else mpf(0)
                         for x in row]
                    z = mpmath.fsum(e)
                    Am.append([x / z for x in e])
                A.append(Am)
            for i in range(n):
                pre = []
                for c in range(2 * d):
                    pre.append(mpmath.fsum((A[0][i][j] - lam * A[1][i][j])
                                           * mpf(float(v[ka + j, g, c]))
                                           for j in range(nk)))
                rms = mpmath.sqrt(mpmath.fsum(x * x for x in pre) / (2 * d)
                                  + mpf(eps))
                for c in range(2 * d):
                    wc = mpf(1) if w is None else mpf(float(w[c]))
                    out[a + i, h, c] = float(pre[c] / rms * wc * (1 - mpf(lam_init)))
    return out


def _mp(x):
    return x if isinstance(x, mpmath.mpf) else mpmath.mpf(float(x))


def _rotate_mp(x, cu, rope):
    """Rotated copy of x [T, heads, 2, d] as an object array of mpf."""
    cos, sin = (np.asarray(t, dtype=np.float64) for t in rope)
    T, nh, two, d = x.shape
    out = np.empty(x.shape, dtype=object)
    for s in range(len(cu) - 1):
        for t in range(int(cu[s]), int(cu[s + 1])):
            p = t - int(cu[s])
            for hh in range(nh):
                for m in range(two):
                    for j in range(d // 2):
                        z = (mpmath.mpc(float(x[t, hh, m, 2 * j]), float(x[t, hh, m, 2 * j + 1]))
                             * mpmath.mpc(cos[p, j], sin[p, j]))
                        out[t, hh, m, 2 * j] = z.real
                        out[t, hh, m, 2 * j + 1] = z.imag
    return out


def pin_brute_force(lib):
    cases = [
        # seed, seqlens, H, Hkv, d, causal, q_scale
        (1, (4, 6), 4, 2, 3, True, 1.0),
        (2, (5,), 2, 2, 2, False, 1.0),
        (3, (3, 1, 5), 2, 1, 4, True, 1.0),
        (4, (6,), 2, 1, 2, True, 800.0),    # scores beyond exp()'s double range
        (5, (4, 5), 4, 2, 3, True, 1.0),    # one set of lambda vectors per head
    ]
    for seed, seqlens, H, Hkv, d, causal, qs in cases:
        q, k, v, lv, w, cu = tiny_inputs(seed, seqlens, H, Hkv, d, q_scale=qs)
        if seed == 5:
            rng = np.random.default_rng(55)
            lv = [(0.4 * rng.standard_normal((H, d))).astype(np.float32)
                  for _ in range(4)]
        lam_init = 0.8 - 0.6 * math.exp(-0.3 * (seed + 2))
        got = run(lib, q, k, v, lv, lam_init, w, 1e-5, causal, cu)
        ref = brute_mpmath(q, k, v, lv, lam_init, w, 1e-5, causal, cu)
        err = np.max(np.abs(got - ref))
        assert np.all(np.isfinite(got)), f"non-finite oracle output, case {seed}"
        assert err < 1e-12, f"brute force case {seed}: max-abs {err:.3e}"


# --------------------------------------------------------------------------
# library routines: torch SDPA + rms_norm in fp64

def sdpa_diff(q, k, v, lam, lam_init, w, eps, causal, cu, cu_k=None):
    """The two-call composition with torch library routines, per sequence.
    With ``cu_k`` the keys of sequence s are ``cu_k[s]..`` and the causal
    mask is an explicit bottom-right lower triangle (torch.tril at offset
    nk - nq)."""
    if cu_k is None:
        cu_k = cu
    qt = torch.from_numpy(q).double()
    kt = torch.from_numpy(k).double()
    vt = torch.from_numpy(v).double()
    T, H, _, d = q.shape
    out = torch.zeros(T, H, 2 * d, dtype=torch.float64)
    wt = None if w is None else torch.from_numpy(w).double()
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        ka, kb = int(cu_k[s]), int(cu_k[s + 1])
        if b == a:
            continue
        # [1, heads, n, width]
        q1 = qt[a:b, :, 0].permute(1, 0, 2).unsqueeze(0)
        q2 = qt[a:b, :, 1].permute(1, 0, 2).unsqueeze(0)
        k1 = kt[ka:kb, :, 0].permute(1, 0, 2).unsqueeze(0)
        k2 = kt[ka:kb, :, 1].permute(1, 0, 2).unsqueeze(0)
        vv = vt[ka:kb].permute(1, 0, 2).unsqueeze(0)
        sc = 1.0 / math.sqrt(d)
        if kb - ka == b - a:
            kw = dict(is_causal=causal)
        else:
            mask = torch.ones(b - a, kb - ka, dtype=torch.bool)
            kw = dict(attn_mask=mask.tril((kb - ka) - (b - a)) if causal else None)
        o1 = F.scaled_dot_product_attention(q1, k1, vv, scale=sc,
                                            enable_gqa=True, **kw)
        o2 = F.scaled_dot_product_attention(q2, k2, vv, scale=sc,
                                            enable_gqa=True, **kw)
        lam_t = torch.as_tensor(np.asarray(lam, dtype=np.float64)).reshape(-1, 1, 1)
        o = o1 - lam_t * o2
        o = F.rms_norm(o, (2 * d,), weight=wt, eps=eps) * (1.0 - lam_init)
        out[a:b] = o[0].permute(1, 0, 2)
    return out.numpy()


def pin_sdpa_lambda_zero(lib):
    """lambda = 0 (lambda_init = 0, equal vector pairs): plain causal softmax
    attention of map 1 followed by RMSNorm."""
    q, k, v, lv, w, cu = tiny_inputs(11, (37, 64, 9), 8, 2, 16)
    lv = [lv[0], lv[1], lv[0], lv[1]]
    got = run(lib, q, k, v, lv, 0.0, w, 1e-5, True, cu)
    q2 = q.copy()
    q2[:, :, 1] = 0.0  # map 2 is multiplied by lambda = 0
    ref = sdpa_diff(q2, k, v, 0.0, 0.0, w, 1e-5, True, cu)
    err = np.max(np.abs(got - ref))
    assert err < 1e-10, f"lambda=0 vs SDPA: max-abs {err:.3e}"


def pin_sdpa_per_head_lambda(lib):
    """One set of lambda vectors per head (the DiffTransformer page's
    parameter shape), against the library composition with a per-head
    lambda."""
    H, Hkv, d = 8, 2, 16
    q, k, v, lv, w, cu = tiny_inputs(17, (41, 30), H, Hkv, d)
    rng = np.random.default_rng(170)
    lv = [(0.3 * rng.standard_normal((H, d))).astype(np.float32) for _ in range(4)]
    lam_init = 0.8 - 0.6 * math.exp(-0.3 * 4)
    lam = np.array([math.exp(float(np.dot(lv[0][h].astype(np.float64), lv[1][h])))
                    - math.exp(float(np.dot(lv[2][h].astype(np.float64), lv[3][h])))
                    + lam_init for h in range(H)])
    got = run(lib, q, k, v, lv, lam_init, w, 1e-5, True, cu)
    ref = sdpa_diff(q, k, v, lam, lam_init, w, 1e-5, True, cu)
    err = np.max(np.abs(got - ref))
    assert err < 1e-10, f"per-head lambda vs SDPA: max-abs {err:.3e}"
    # identical per-head sets equal the shared set, bitwise
    shared = [x[3] for x in lv]
    rep = [np.repeat(x[None, :], H, axis=0) for x in shared]
    assert np.array_equal(run(lib, q, k, v, rep, lam_init, w, 1e-5, True, cu),
                          run(lib, q, k, v, shared, lam_init, w, 1e-5, True, cu))


def pin_sdpa_two_maps(lib):
    for causal in (True, False):
        for H, Hkv in ((8, 2), (4, 4), (6, 1)):
            q, k, v, lv, w, cu = tiny_inputs(12 + H, (33, 70), H, Hkv, 16)
            lam_init = 0.8 - 0.6 * math.exp(-0.3 * 7)
            lam = (math.exp(float(np.dot(lv[0].astype(np.float64), lv[1])))
                   - math.exp(float(np.dot(lv[2].astype(np.float64), lv[3])))
                   + lam_init)
            got = run(lib, q, k, v, lv, lam_init, w, 1e-5, causal, cu)
            ref = sdpa_diff(q, k, v, lam, lam_init, w, 1e-5, causal, cu)
            err = np.max(np.abs(got - ref))
            assert err < 1e-10, (f"two-map vs SDPA (H={H}, Hkv={Hkv}, "
                                 f"causal={causal}): max-abs {err:.3e}")


# --------------------------------------------------------------------------
# closed forms

def pin_lambda_closed_forms(lib):
    assert oracle.lambda_init(1, lib=lib) == 0.8 - 0.6, "lambda_init(1)"
    assert abs(oracle.lambda_init(1, lib=lib) - 0.2) < 1e-15
    assert abs(oracle.lambda_init(10 ** 6, lib=lib) - 0.8) < 1e-15
    # strictly increasing in depth
    vals = [oracle.lambda_init(l, lib=lib) for l in range(1, 40)]
    assert all(b > a for a, b in zip(vals, vals[1:]))
    d = 8
    z = np.zeros(d, np.float32)
    e0 = np.zeros(d, np.float32)
    e0[0] = 1.0
    e1 = np.zeros(d, np.float32)
    e1[1] = 1.0
    # both dot products zero: exp(0) - exp(0) + lambda_init
    assert oracle.lam(z, z, z, z, 0.3, lib=lib) == 0.3
    assert oracle.lam(e0, e1, e1, e0, 0.3, lib=lib) == 0.3
    # first dot product one, second zero: e - 1 + lambda_init
    got = oracle.lam(e0, e0, z, z, 0.25, lib=lib)
    assert abs(got - (math.e - 1.0 + 0.25)) < 1e-15, got
    # second dot product two, first zero: 1 - e^2 + lambda_init
    two = 2 * e1
    got = oracle.lam(z, z, two, e1, 0.5, lib=lib)
    assert abs(got - (1.0 - math.e ** 2 + 0.5)) < 1e-14, got


def pin_row0_closed_form(lib):
    """Causal row 0 of a sequence sees only key 0, so both maps put weight 1
    on V[a]: pre = (1 - lambda) V[a]."""
    for v_scale in (1.0, 3e-3):
        q, k, v, lv, w, cu = tiny_inputs(21, (5, 17, 1, 40), 4, 2, 8,
                                         v_scale=v_scale)
        lam_init = 0.55
        lam = (math.exp(float(np.dot(lv[0].astype(np.float64), lv[1])))
               - math.exp(float(np.dot(lv[2].astype(np.float64), lv[3])))
               + lam_init)
        got = run(lib, q, k, v, lv, lam_init, w, 1e-5, True, cu)
        for s in range(len(cu) - 1):
            a = int(cu[s])
            for h in range(4):
                g = h // 2
                pre = (1.0 - lam) * v[a, g].astype(np.float64)
                ref = (pre / math.sqrt(np.mean(pre * pre) + 1e-5)
                       * w.astype(np.float64) * (1.0 - lam_init))
                err = np.max(np.abs(got[a, h] - ref))
                assert err < 1e-12, f"row0 seq {s} head {h}: {err:.3e}"


def pin_uniform_attention(lib):
    """K = 0 makes every score zero, so each map is the uniform average over
    the visible keys: pre_i = (1 - lambda) * mean_{j in J(i)} V_j."""
    for causal in (True, False):
        q, k, v, lv, w, cu = tiny_inputs(31, (50, 3, 77), 4, 1, 8)
        k[:] = 0.0
        lam_init = 0.7
        lam = (math.exp(float(np.dot(lv[0].astype(np.float64), lv[1])))
               - math.exp(float(np.dot(lv[2].astype(np.float64), lv[3])))
               + lam_init)
        got = run(lib, q, k, v, lv, lam_init, w, 1e-5, causal, cu)
        for s in range(len(cu) - 1):
            a, b = int(cu[s]), int(cu[s + 1])
            vv = v[a:b, 0].astype(np.float64)
            if causal:
                mean = np.cumsum(vv, axis=0) / np.arange(1, b - a + 1)[:, None]
            else:
                mean = np.broadcast_to(vv.mean(axis=0), vv.shape)
            pre = (1.0 - lam) * mean
            ref = (pre / np.sqrt(np.mean(pre * pre, axis=1, keepdims=True) + 1e-5)
                   * w.astype(np.float64) * (1.0 - lam_init))
            for h in range(4):
                err = np.max(np.abs(got[a:b, h] - ref))
                assert err < 1e-12, f"uniform seq {s} head {h}: {err:.3e}"


def pin_identical_maps(lib):
    """Q2 = Q1, K2 = K1 and lambda = 1 cancel the two maps exactly."""
    q, k, v, lv, w, cu = tiny_inputs(41, (20, 13), 4, 2, 8)
    q[:, :, 1] = q[:, :, 0]
    k[:, :, 1] = k[:, :, 0]
    lv = [lv[0], lv[1], lv[0], lv[1]]
    got = run(lib, q, k, v, lv, 1.0, w, 1e-5, True, cu)
    assert np.all(got == 0.0), "identical maps with lambda = 1 must give 0"
    # and with lambda != 1 they give RMSNorm((1 - lambda) * attention), whose
    # sign is that of (1 - lambda): flip it and the output flips
    a = run(lib, q, k, v, lv, 0.5, w, 1e-5, True, cu)
    b = run(lib, q, k, v, lv, 1.5, w, 1e-5, True, cu)
    assert np.max(np.abs(a / (1 - 0.5) + b / (1 - 1.5))) < 1e-12


# --------------------------------------------------------------------------
# invariants

def pin_causality(lib):
    q, k, v, lv, w, cu = tiny_inputs(51, (30,), 2, 1, 4)
    base = run(lib, q, k, v, lv, 0.4, w, 1e-5, True, cu)
    for cut in (0, 7, 29):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        q2[cut + 1:] += 3.0
        k2[cut + 1:] -= 2.0
        v2[cut + 1:] *= -5.0
        got = run(lib, q2, k2, v2, lv, 0.4, w, 1e-5, True, cu)
        assert np.array_equal(got[:cut + 1], base[:cut + 1]), f"cut {cut}"
        if cut + 1 < 30:
            assert not np.allclose(got[cut + 1:], base[cut + 1:])


def pin_packing(lib):
    seqlens = (9, 1, 25, 4)
    q, k, v, lv, w, cu = tiny_inputs(61, seqlens, 4, 2, 4)
    for causal in (True, False):
        packed = run(lib, q, k, v, lv, 0.3, w, 1e-5, causal, cu)
        for s in range(len(seqlens)):
            a, b = int(cu[s]), int(cu[s + 1])
            one = run(lib, q[a:b], k[a:b], v[a:b], lv, 0.3, w, 1e-5, causal,
                      np.array([0, b - a], np.int32))
            assert np.array_equal(one, packed[a:b]), f"seq {s}"


def pin_gqa_equals_repeated(lib):
    q, k, v, lv, w, cu = tiny_inputs(71, (19, 8), 6, 2, 4)
    got = run(lib, q, k, v, lv, 0.3, w, 1e-5, True, cu)
    kr = np.repeat(k, 3, axis=1)   # KV head g serves heads 3g .. 3g+2
    vr = np.repeat(v, 3, axis=1)
    ref = run(lib, q, kr, vr, lv, 0.3, w, 1e-5, True, cu)
    assert np.array_equal(got, ref)


def pin_odd_in_v(lib):
    q, k, v, lv, w, cu = tiny_inputs(81, (12, 12), 2, 2, 4)
    a = run(lib, q, k, v, lv, 0.3, w, 1e-5, True, cu)
    b = run(lib, q, k, -v, lv, 0.3, w, 1e-5, True, cu)
    assert np.array_equal(a, -b)


def pin_rows_entry(lib):
    q, k, v, lv, w, cu = tiny_inputs(91, (10, 23), 4, 2, 4)
    full = run(lib, q, k, v, lv, 0.3, w, 1e-5, True, cu)
    toks = np.array([0, 9, 10, 11, 32, 5, 20], np.int64)
    heads = np.array([0, 3, 1, 2, 3, 0, 1], np.int32)
    got = oracle.rows(q, k, v, *lv, 0.3, toks, heads, w, 1e-5, True, cu, lib=lib)
    assert np.array_equal(got, full[toks, heads])


# --------------------------------------------------------------------------
# rotary prologue (the pull request's interleaved apply_rotary_emb)

def rope_tables(length, d, base=10000.0, offset=0):
    import workloads
    c, s_ = workloads.rope_tables(length, d, base, offset)
    return c.numpy(), s_.numpy()


def rotate_torch(x, cu, rope):
    """q or k [T, heads, 2, d] rotated with torch complex arithmetic
    (view_as_complex on consecutive pairs times cos + i sin of the row's
    sequence position), fp64."""
    cos, sin = (torch.from_numpy(np.asarray(t, dtype=np.float64)) for t in rope)
    xt = torch.from_numpy(np.asarray(x, dtype=np.float64))
    T, nh, two, d = xt.shape
    pos = torch.cat([torch.arange(int(cu[s + 1] - cu[s])) for s in range(len(cu) - 1)])
    z = torch.view_as_complex(xt.reshape(T, nh, two, d // 2, 2).contiguous())
    rot = torch.complex(cos, sin)[pos]                             # [T, d/2]
    out = torch.view_as_real(z * rot[:, None, None, :]).reshape(T, nh, two, d)
    return out.numpy()


def pin_rope_brute_force(lib):
    cases = [
        # seed, seqlens, H, Hkv, d, causal
        (201, (4, 6), 4, 2, 4, True),
        (202, (5,), 2, 1, 6, False),
    ]
    for seed, seqlens, H, Hkv, d, causal in cases:
        q, k, v, lv, w, cu = tiny_inputs(seed, seqlens, H, Hkv, d)
        rope = rope_tables(max(seqlens), d, base=3.0)
        got = oracle.fwd(q, k, v, *lv, 0.45, w, 1e-5, causal, cu, lib=lib, rope=rope)
        ref = brute_mpmath(q, k, v, lv, 0.45, w, 1e-5, causal, cu, rope=rope)
        err = np.max(np.abs(got - ref))
        assert err < 1e-12, f"rope brute force case {seed}: max-abs {err:.3e}"


def pin_rope_sdpa(lib):
    """Rotation by torch complex arithmetic, then the library composition of
    two SDPA calls, against the oracle's fused rotary prologue (varlen, GQA,
    positions restart in every sequence)."""
    H, Hkv, d = 8, 2, 16
    q, k, v, lv, w, cu = tiny_inputs(210, (45, 1, 70), H, Hkv, d)
    rope = rope_tables(80, d)
    lam_init = 0.8 - 0.6 * math.exp(-0.3 * 5)
    lam = (math.exp(float(np.dot(lv[0].astype(np.float64), lv[1])))
           - math.exp(float(np.dot(lv[2].astype(np.float64), lv[3])))
           + lam_init)
    for causal in (True, False):
        got = oracle.fwd(q, k, v, *lv, lam_init, w, 1e-5, causal, cu, lib=lib,
                         rope=rope)
        ref = sdpa_diff(rotate_torch(q, cu, rope), rotate_torch(k, cu, rope), v,
                        lam, lam_init, w, 1e-5, causal, cu)
        err = np.max(np.abs(got - ref))
        assert err < 1e-10, f"rope vs SDPA (causal={causal}): max-abs {err:.3e}"
    # rows entry point with the same prologue
    toks = np.array([0, 44, 45, 46, 115], np.int64)
    heads = np.array([0, 7, 3, 1, 5], np.int32)
    full = oracle.fwd(q, k, v, *lv, lam_init, w, 1e-5, True, cu, lib=lib, rope=rope)
    got = oracle.rows(q, k, v, *lv, lam_init, toks, heads, w, 1e-5, True, cu,
                      lib=lib, rope=rope)
    assert np.array_equal(got, full[toks, heads])


def pin_rope_identity_and_shift(lib):
    """cos = 1, sin = 0 rotates nothing (bitwise equal to no prologue); and
    rotating every position by the same extra angle leaves every score, so
    every output, unchanged (scores depend on position differences only)."""
    H, Hkv, d = 4, 2, 8
    q, k, v, lv, w, cu = tiny_inputs(220, (17, 30), H, Hkv, d)
    ones = np.ones((30, d // 2), np.float32)
    zeros = np.zeros((30, d // 2), np.float32)
    plain = run(lib, q, k, v, lv, 0.3, w, 1e-5, True, cu)
    ident = oracle.fwd(q, k, v, *lv, 0.3, w, 1e-5, True, cu, lib=lib,
                       rope=(ones, zeros))
    assert np.array_equal(plain, ident)
    a = oracle.fwd(q, k, v, *lv, 0.3, w, 1e-5, True, cu, lib=lib,
                   rope=rope_tables(30, d, base=7.0))
    b = oracle.fwd(q, k, v, *lv, 0.3, w, 1e-5, True, cu, lib=lib,
                   rope=rope_tables(30, d, base=7.0, offset=1000))
    # the tables are rounded to fp32 at different angles: ~1e-7 apart
    err = np.max(np.abs(a - b))
    assert err < 1e-5, f"rope shift invariance: {err:.3e}"
    assert np.max(np.abs(a - plain)) > 1e-3, "rotation had no effect"


def pin_rope_bf16_storage(lib):
    """With rope_round_bf16 the oracle equals, bitwise, the plain oracle on
    q and k rotated in fp64 (same products, same order) and stored as bf16
    by torch's own conversion (a library routine)."""
    H, Hkv, d = 4, 2, 16
    q, k, v, lv, w, cu = tiny_inputs(230, (40, 9), H, Hkv, d)
    rope = rope_tables(40, d, base=20.0)
    got = oracle.fwd(q, k, v, *lv, 0.5, w, 1e-5, True, cu, lib=lib, rope=rope,
                     rope_round_bf16=True)

    def rot_bf16(x):
        cos, sin = (np.asarray(t, dtype=np.float64) for t in rope)
        pos = np.concatenate([np.arange(int(cu[s + 1] - cu[s])) for s in range(len(cu) - 1)])
        x0 = x[..., 0::2].astype(np.float64)
        x1 = x[..., 1::2].astype(np.float64)
        c = cos[pos][:, None, None, :]
        s_ = sin[pos][:, None, None, :]
        out = np.empty(x.shape, np.float64)
        out[..., 0::2] = x0 * c - x1 * s_
        out[..., 1::2] = x0 * s_ + x1 * c
        return torch.from_numpy(out).to(torch.bfloat16).float().numpy()

    ref = run(lib, rot_bf16(q), rot_bf16(k), v, lv, 0.5, w, 1e-5, True, cu)
    assert np.array_equal(got, ref)
    plain = oracle.fwd(q, k, v, *lv, 0.5, w, 1e-5, True, cu, lib=lib, rope=rope)
    assert np.max(np.abs(plain - got)) > 1e-6, "rounding had no effect"


# --------------------------------------------------------------------------
# backward

def autograd_composition(q, k, v, lv, lam_init, w, eps, causal, cu, dy):
    """Gradients of <dy, out> by torch autograd in fp64 through the library
    composition: lambda from the vectors, two SDPA calls per sequence (GQA
    through enable_gqa), their difference, rms_norm with the weight, the
    (1 - lambda_init) scale."""
    f = lambda x: torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)
    qt, kt, vt, wt = f(q), f(k), f(v), f(w)
    lt = [f(x) for x in lv]
    a = (lt[0] * lt[1]).sum(-1)
    b = (lt[2] * lt[3]).sum(-1)
    lam = torch.exp(a) - torch.exp(b) + lam_init
    T, H, _, d = q.shape
    sc = 1.0 / math.sqrt(d)
    outs = []
    for s in range(len(cu) - 1):
        a0, b0 = int(cu[s]), int(cu[s + 1])
        if b0 == a0:
            continue
        seg = lambda x, m: x[a0:b0, :, m].permute(1, 0, 2).unsqueeze(0)
        vv = vt[a0:b0].permute(1, 0, 2).unsqueeze(0)
        o1 = F.scaled_dot_product_attention(seg(qt, 0), seg(kt, 0), vv,
                                            is_causal=causal, scale=sc, enable_gqa=True)
        o2 = F.scaled_dot_product_attention(seg(qt, 1), seg(kt, 1), vv,
                                            is_causal=causal, scale=sc, enable_gqa=True)
        o = o1 - lam.reshape(-1, 1, 1) * o2
        o = F.rms_norm(o, (2 * d,), weight=wt, eps=eps) * (1.0 - lam_init)
        outs.append(o[0].permute(1, 0, 2))
    y = torch.cat(outs, 0)
    (y * torch.from_numpy(np.asarray(dy, dtype=np.float64))).sum().backward()
    g = {"dq": qt.grad, "dk": kt.grad, "dv": vt.grad, "dw": wt.grad}
    for name, t in zip(("dlq1", "dlk1", "dlq2", "dlk2"), lt):
        g[name] = t.grad
    return {kk: x.numpy() for kk, x in g.items()}


def pin_bwd_autograd(lib):
    cases = [
        # seed, seqlens, H, Hkv, d, causal, per-head lambda
        (301, (9, 1, 14), 4, 2, 8, True, False),
        (302, (11, 6), 6, 2, 4, False, False),
        (303, (7, 12), 4, 1, 8, True, True),
    ]
    for seed, seqlens, H, Hkv, d, causal, per_head in cases:
        q, k, v, lv, w, cu = tiny_inputs(seed, seqlens, H, Hkv, d)
        if per_head:
            rng = np.random.default_rng(seed + 1)
            lv = [(0.3 * rng.standard_normal((H, d))).astype(np.float32) for _ in range(4)]
        dy = np.random.default_rng(seed + 2).standard_normal((q.shape[0], H, 2 * d)).astype(np.float32)
        lam_init = 0.8 - 0.6 * math.exp(-0.3 * (seed - 300))
        got = oracle.bwd(q, k, v, *lv, lam_init, dy, w, 1e-5, causal, cu, lib=lib)
        ref = autograd_composition(q, k, v, lv, lam_init, w, 1e-5, causal, cu, dy)
        # dlambda per head reproduces the vector gradients by the chain rule
        aux = got["aux"]
        for hh in range(H if per_head else 1):
            sel = (lambda x: x[hh]) if per_head else (lambda x: x)
            dl = aux["dlam_head"][hh] if per_head else aux["dlam_head"].sum()
            ea = math.exp(float(np.dot(sel(lv[0]).astype(np.float64), sel(lv[1]))))
            assert np.max(np.abs(dl * ea * sel(lv[1]) - sel(ref["dlq1"]))) < 1e-9
            assert np.all(aux["dlam_scale"] >= np.abs(aux["dlam_head"]) - 1e-12)
        for name in ref:
            err = np.max(np.abs(got[name] - ref[name]))
            assert err < 1e-9, f"bwd vs autograd case {seed} {name}: max-abs {err:.3e}"


def pin_bwd_finite_differences(lib):
    """Central differences of <dy, oracle forward> along +-1 directions
    scaled by 2^-10 (exact in fp32 for these inputs) against <grad, u>."""
    H, Hkv, d = 4, 2, 4
    for causal in (True, False):
        q, k, v, lv, w, cu = tiny_inputs(310 + causal, (7, 5), H, Hkv, d)
        dy = np.random.default_rng(311).standard_normal((12, H, 2 * d)).astype(np.float32)
        lam_init = 0.35
        g = oracle.bwd(q, k, v, *lv, lam_init, dy, w, 1e-5, causal, cu, lib=lib)
        base = dict(q=q, k=k, v=v, lq1=lv[0], lk1=lv[1], lq2=lv[2], lk2=lv[3], w=w)
        eps = 2.0 ** -10

        def loss(x):
            out = oracle.fwd(x["q"], x["k"], x["v"], x["lq1"], x["lk1"], x["lq2"],
                             x["lk2"], lam_init, x["w"], 1e-5, causal, cu, lib=lib)
            return float(np.sum(out * dy.astype(np.float64)))

        rng = np.random.default_rng(312)
        for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("w", "dw"),
                            ("lq1", "dlq1"), ("lk1", "dlk1"), ("lq2", "dlq2"),
                            ("lk2", "dlk2")):
            u = rng.choice([-1.0, 1.0], size=base[name].shape).astype(np.float32)
            xp, xm = dict(base), dict(base)
            xp[name] = (base[name] + np.float32(eps) * u).astype(np.float32)
            xm[name] = (base[name] - np.float32(eps) * u).astype(np.float32)
            fd = (loss(xp) - loss(xm)) / (2 * eps)
            an = float(np.sum(g[gname] * u))
            assert abs(fd - an) <= 1e-4 * max(1.0, abs(an)), \
                f"finite differences {name} causal={causal}: {fd:.8f} vs {an:.8f}"


def pin_bwd_sample(lib):
    """The sampling entry point equals the full backward on the sampled
    rows and keys (only the summation order of dk, dv differs)."""
    for causal in (True, False):
        q, k, v, lv, w, cu = tiny_inputs(320 + causal, (13, 1, 20), 6, 2, 4)
        dy = np.random.default_rng(321).standard_normal((34, 6, 8)).astype(np.float32)
        full = oracle.bwd(q, k, v, *lv, 0.4, dy, w, 1e-5, causal, cu, lib=lib)
        tq = np.array([0, 12, 13, 14, 33, 20], np.int64)
        hq = np.array([0, 5, 3, 2, 1, 4], np.int32)
        tk = np.array([0, 5, 12, 13, 14, 20, 33], np.int64)
        gk = np.array([0, 1, 1, 0, 1, 0, 1], np.int32)
        got = oracle.bwd_sample(q, k, v, *lv, 0.4, dy, (tq, hq), (tk, gk), w, 1e-5,
                                causal, cu, lib=lib)
        assert np.max(np.abs(got["dq"] - full["dq"][tq, hq])) < 1e-12
        assert np.max(np.abs(got["dk"] - full["dk"][tk, gk])) < 1e-12
        assert np.max(np.abs(got["dv"] - full["dv"][tk, gk])) < 1e-12


# --------------------------------------------------------------------------
# new queries against a key/value cache

def kv_inputs(seed, nq, nk, H, Hkv, d, q_scale=1.0):
    """Queries of ``sum(nq)`` tokens, keys/values of ``sum(nk)`` tokens."""
    rng = np.random.default_rng(seed)
    Tq, Tk = int(sum(nq)), int(sum(nk))
    q = (rng.standard_normal((Tq, H, 2, d)) * q_scale).astype(np.float32)
    k = rng.standard_normal((Tk, Hkv, 2, d)).astype(np.float32)
    v = rng.standard_normal((Tk, Hkv, 2 * d)).astype(np.float32)
    lv = [(0.3 * rng.standard_normal(d)).astype(np.float32) for _ in range(4)]
    w = (0.5 + rng.random(2 * d)).astype(np.float32)
    cq = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(nk)]).astype(np.int32)
    return q, k, v, lv, w, cq, ck


def run_kv(lib, q, k, v, lv, lam_init, w, eps, causal, cq, ck):
    return oracle.fwd_kv(q, k, v, *lv, lam_init, w, eps, causal, cq, ck, lib=lib)


def pin_kv_brute_force(lib):
    cases = [
        # seed, query lengths, key lengths, H, Hkv, d, causal
        (101, (1, 3), (5, 7), 4, 2, 3, True),
        (102, (2, 4), (6, 3), 2, 1, 2, False),   # more queries than keys
        (103, (1, 1, 2), (1, 4, 2), 2, 2, 4, True),
        (104, (3,), (9,), 4, 1, 2, True),
    ]
    for seed, nq, nk, H, Hkv, d, causal in cases:
        q, k, v, lv, w, cq, ck = kv_inputs(seed, nq, nk, H, Hkv, d)
        if seed == 104:                        # one set of vectors per head
            rng = np.random.default_rng(1040)
            lv = [(0.4 * rng.standard_normal((H, d))).astype(np.float32)
                  for _ in range(4)]
        lam_init = 0.8 - 0.6 * math.exp(-0.3 * (seed - 100))
        got = run_kv(lib, q, k, v, lv, lam_init, w, 1e-5, causal, cq, ck)
        ref = brute_mpmath(q, k, v, lv, lam_init, w, 1e-5, causal, cq, cu_k=ck)
        err = np.max(np.abs(got - ref))
        assert np.all(np.isfinite(got)), f"non-finite oracle output, case {seed}"
        assert err < 1e-12, f"kv brute force case {seed}: max-abs {err:.3e}"


def pin_kv_sdpa(lib):
    for causal in (True, False):
        q, k, v, lv, w, cq, ck = kv_inputs(110, (1, 5, 16, 2), (40, 5, 100, 77),
                                           8, 2, 16)
        lam_init = 0.8 - 0.6 * math.exp(-0.3 * 11)
        lam = (math.exp(float(np.dot(lv[0].astype(np.float64), lv[1])))
               - math.exp(float(np.dot(lv[2].astype(np.float64), lv[3])))
               + lam_init)
        got = run_kv(lib, q, k, v, lv, lam_init, w, 1e-5, causal, cq, ck)
        ref = sdpa_diff(q, k, v, lam, lam_init, w, 1e-5, causal, cq, cu_k=ck)
        err = np.max(np.abs(got - ref))
        assert err < 1e-10, f"kv vs SDPA (causal={causal}): max-abs {err:.3e}"


def pin_kv_prefill_tail(lib):
    """The last nq rows of a causal prefill are nq new queries against the
    whole sequence as their cache (same arithmetic, so bitwise)."""
    seqlens = (12, 1, 30)
    tails = (4, 1, 7)
    q, k, v, lv, w, cu = tiny_inputs(120, seqlens, 4, 2, 4)
    full = run(lib, q, k, v, lv, 0.35, w, 1e-5, True, cu)
    rows = np.concatenate([np.arange(int(cu[s + 1]) - tails[s], int(cu[s + 1]))
                           for s in range(len(seqlens))])
    cq = np.concatenate([[0], np.cumsum(tails)]).astype(np.int32)
    got = run_kv(lib, q[rows], k, v, lv, 0.35, w, 1e-5, True, cq, cu)
    assert np.array_equal(got, full[rows])
    # nq = nk is the prefill itself, causal or not
    for causal in (True, False):
        assert np.array_equal(run_kv(lib, q, k, v, lv, 0.35, w, 1e-5, causal, cu, cu),
                              run(lib, q, k, v, lv, 0.35, w, 1e-5, causal, cu))


def pin_kv_single_key(lib):
    """One query against a one-key cache (or the cache's first key only,
    causal with nq = nk): pre = (1 - lambda) V[key]."""
    q, k, v, lv, w, cq, ck = kv_inputs(130, (1, 1), (1, 1), 2, 1, 4)
    lam_init = 0.45
    lam = (math.exp(float(np.dot(lv[0].astype(np.float64), lv[1])))
           - math.exp(float(np.dot(lv[2].astype(np.float64), lv[3])))
           + lam_init)
    got = run_kv(lib, q, k, v, lv, lam_init, w, 1e-5, True, cq, ck)
    for s in range(2):
        pre = (1.0 - lam) * v[s, 0].astype(np.float64)
        ref = pre / math.sqrt(np.mean(pre * pre) + 1e-5) * w * (1.0 - lam_init)
        assert np.max(np.abs(got[s] - ref)) < 1e-12


ALL_PINS = [
    pin_lambda_closed_forms,
    pin_brute_force,
    pin_sdpa_lambda_zero,
    pin_sdpa_two_maps,
    pin_sdpa_per_head_lambda,
    pin_row0_closed_form,
    pin_uniform_attention,
    pin_identical_maps,
    pin_causality,
    pin_packing,
    pin_gqa_equals_repeated,
    pin_odd_in_v,
    pin_rows_entry,
    pin_rope_brute_force,
    pin_rope_sdpa,
    pin_rope_identity_and_shift,
    pin_rope_bf16_storage,
    pin_bwd_autograd,
    pin_bwd_finite_differences,
    pin_bwd_sample,
    pin_kv_brute_force,
    pin_kv_sdpa,
    pin_kv_prefill_tail,
    pin_kv_single_key,
]
