"""How far the two maps of an output row cancel before the RMSNorm: the
conditioning that scales the bf16 bar of the parity tests for such rows.
Not from the pages (they state no bound for this case): the scaling follows
from the bf16 rounding of the probabilities, which the RMSNorm divides by
rms(pre).  A row whose ratio r is below RATIO_REF is held to the bar times
0.2 / r, never more than CAP times the bar; rows that would need more fail.
The logic of such rows is pinned separately, by fp32 twins of the same
inputs at the fp32 bar."""

import copy

import numpy as np
import torch

import oracle

RATIO_REF = 0.2   # rows with a smaller cancellation ratio get a wider bar
CAP = 4.0         # ... at most this many times the plain bar


def bar_factor(ratio):
    """The bar multiplier of a row with cancellation ratio ``ratio``:
    0.2 / ratio below RATIO_REF, capped at CAP, else 1."""
    return float(min(CAP, max(1.0, RATIO_REF / max(ratio, 1e-300))))


def cancellation_ratio(inp, t, h):
    """rms(pre) / sum_j (P_1j + |lambda| P_2j) rms(V_j) of output row (token
    t, head h), in fp64 from the definition: how far the two maps' weighted
    sums of V cancel before the RMSNorm.  Rounding the probabilities P_mj to
    bf16 (the PV operand) moves pre by up to 2^-9 times the denominator, so
    the RMSNorm turns it into an output error of about 2^-9 / ratio."""
    cu = inp.cu_seqlens.tolist()
    s = max(j for j in range(len(cu) - 1) if cu[j] <= t)
    a, b = cu[s], cu[s + 1]
    H, Hkv, d = inp.q.shape[1], inp.k.shape[1], inp.q.shape[3]
    g = h // (H // Hkv)
    J = slice(a, t + 1) if inp.causal else slice(a, b)
    q, k, v = inp.q.double(), inp.k.double(), inp.v.double()
    lv = [x if x.dim() == 1 else x[h] for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
    lam = oracle.lam(*lv, oracle.lambda_init(inp.depth))
    o, w = [], []
    for m in range(2):
        x = (k[J, g, m] @ q[t, h, m]) / d ** 0.5
        pr = torch.softmax(x, dim=0)
        o.append(pr @ v[J, g])
        w.append(pr)
    pre = o[0] - lam * o[1]
    contrib = ((w[0] + abs(lam) * w[1]) * v[J, g].pow(2).mean(1).sqrt()).sum()
    return float(pre.pow(2).mean().sqrt() / contrib)


def rows_within_bar(got, ref, tol, bf16, inp, log=print):
    """Every output row of the forward within tol; for bf16 storage, a row
    whose two maps cancel (cancellation_ratio below 0.2) is held to tol
    times bar_factor(ratio) instead (at most CAP times tol): the RMSNorm
    divides the fixed bf16 rounding of the probabilities (the PV operand) by
    rms(pre).  inp supplies the rows' inputs for the ratio (already rotated
    when the kernel rotates).  Returns (largest row error, number of rows
    that needed the wider bar)."""
    g = got.float().cpu().double().numpy()
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    if not ref.size:
        return 0.0, 0
    row_err = np.abs(g - ref).max(axis=2)
    relaxed = 0
    for t, h in np.argwhere(row_err > tol):
        assert bf16, (t, h, row_err[t, h])
        ratio = cancellation_ratio(inp, int(t), int(h))
        f = bar_factor(ratio)
        log(f"row (token {t}, head {h}): max-abs {row_err[t, h]:.3e}, "
            f"cancellation ratio {ratio:.4f}, bar x{f:.2f}")
        assert row_err[t, h] <= tol * f, (
            f"row (token {t}, head {h}): {row_err[t, h]:.3e} > {tol * f:.3e}")
        relaxed += 1
    return float(row_err.max()), relaxed


def _seq_ratios(inp, a, b, h, g, lam):
    """[n] cancellation ratios of the rows of head h over tokens a..b-1, and
    [n] the number of keys each row sees (whole score matrices)."""
    H, Hkv, d = inp.q.shape[1], inp.k.shape[1], inp.q.shape[3]
    n = b - a
    q, k, v = inp.q.double(), inp.k.double(), inp.v.double()
    mask = torch.ones(n, n, dtype=torch.bool)
    if inp.causal:
        mask = torch.tril(mask)
    o, w = [], []
    for m in range(2):
        x = (q[a:b, h, m] @ k[a:b, g, m].T) / d ** 0.5
        pr = torch.softmax(x.masked_fill(~mask, float("-inf")), dim=1)
        o.append(pr @ v[a:b, g])
        w.append(pr)
    pre = o[0] - lam * o[1]
    contrib = (w[0] + abs(lam) * w[1]) @ v[a:b, g].pow(2).mean(1).sqrt()
    return (pre.pow(2).mean(1).sqrt() / contrib).numpy(), mask.sum(1).numpy()


def row_factors(inp):
    """[T, H] bar multipliers of the backward's output rows: bar_factor of
    each row's cancellation ratio, except 1 for rows that see a single key
    (their probabilities are exactly 1, so there is no rounding for the
    RMSNorm to amplify).  Whole score matrices: for small shapes."""
    cu = inp.cu_seqlens.tolist()
    T, H, Hkv = inp.q.shape[0], inp.q.shape[1], inp.k.shape[1]
    G = H // Hkv
    lam0 = oracle.lambda_init(inp.depth)
    out = np.ones((T, H))
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b == a:
            continue
        for h in range(H):
            lv = [x if x.dim() == 1 else x[h] for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
            lam = oracle.lam(*lv, lam0)
            r, nvis = _seq_ratios(inp, a, b, h, h // G, lam)
            f = np.minimum(CAP, np.maximum(1.0, RATIO_REF / np.maximum(r, 1e-300)))
            f[nvis == 1] = 1.0
            out[a:b, h] = f
    return out


def key_factors(inp, rf):
    """[T, Hkv] bar multipliers of dk and dv: for key j of KV head g, the
    largest row factor among the rows (token t, head of group g) that see
    key j -- t >= j in its sequence when causal, every t of the sequence
    otherwise."""
    cu = inp.cu_seqlens.tolist()
    T, H, Hkv = inp.q.shape[0], inp.q.shape[1], inp.k.shape[1]
    G = H // Hkv
    grp = rf.reshape(T, Hkv, G).max(axis=2)            # [T, Hkv]
    out = np.ones((T, Hkv))
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if b == a:
            continue
        if inp.causal:   # max over t >= j: a reversed running maximum
            out[a:b] = np.maximum.accumulate(grp[a:b][::-1], axis=0)[::-1]
        else:
            out[a:b] = grp[a:b].max(axis=0, keepdims=True)
    return out


def turn(x, pos, rope):
    """Rows of x ([N, ...heads, d]) turned as the rotary prologue turns
    them: pair (x[2j], x[2j+1]) of row n by (cos, sin)[pos[n], j], in fp64,
    stored back in x's type."""
    cos, sin = (t.double() for t in rope)
    pos = torch.as_tensor(pos).long()
    c, s_ = cos[pos], sin[pos]                                   # [N, d/2]
    xd = x.double()
    x0, x1 = xd[..., 0::2], xd[..., 1::2]
    shape = (xd.shape[0],) + (1,) * (xd.dim() - 2) + (c.shape[1],)
    cc, ss = c.reshape(shape), s_.reshape(shape)
    y = torch.empty_like(xd)
    y[..., 0::2] = x0 * cc - x1 * ss
    y[..., 1::2] = x0 * ss + x1 * cc
    return y.to(x.dtype)


def rotated(inp, rope):
    """A copy of inp whose q and k rows are turned as the rotary prologue
    turns them: the row at position p of its sequence by (cos, sin)[p],
    stored back in the input's type."""
    cu = inp.cu_seqlens.tolist()
    pos = torch.cat([torch.arange(cu[s + 1] - cu[s]) for s in range(len(cu) - 1)]).long()
    out = copy.copy(inp)
    out.q, out.k = turn(inp.q, pos, rope), turn(inp.k, pos, rope)
    return out
