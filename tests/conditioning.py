"""How far the two maps of an output row cancel before the RMSNorm: the
conditioning that scales the bf16 bar of the parity tests for such rows.
Not from the pages (they state no bound for this case): the bar's scaling
follows from the bf16 rounding of the probabilities, and the constant is
set with a margin over seeded sweeps."""

import copy

import numpy as np
import torch

import oracle


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


def group_floor(inp):
    """[nseq, Hkv]: the smallest cancellation_ratio over the rows (token,
    head) of each (sequence, KV group), in fp64 from the definition (whole
    score matrices: for the small shapes of the random tests)."""
    cu = inp.cu_seqlens.tolist()
    H, Hkv, d = inp.q.shape[1], inp.k.shape[1], inp.q.shape[3]
    G = H // Hkv
    lam0 = oracle.lambda_init(inp.depth)
    q, k, v = inp.q.double(), inp.k.double(), inp.v.double()
    out = torch.ones(len(cu) - 1, Hkv, dtype=torch.float64)
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        n = b - a
        if n == 0:
            continue
        mask = torch.ones(n, n, dtype=torch.bool)
        if inp.causal:
            mask = torch.tril(mask)
        for g in range(Hkv):
            worst = 1.0
            for h in range(g * G, (g + 1) * G):
                lv = [x if x.dim() == 1 else x[h] for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
                lam = oracle.lam(*lv, lam0)
                o, w = [], []
                for m in range(2):
                    x = (q[a:b, h, m] @ k[a:b, g, m].T) / d ** 0.5
                    pr = torch.softmax(x.masked_fill(~mask, float("-inf")), dim=1)
                    o.append(pr @ v[a:b, g])
                    w.append(pr)
                pre = o[0] - lam * o[1]
                contrib = (w[0] + abs(lam) * w[1]) @ v[a:b, g].pow(2).mean(1).sqrt()
                ratio = pre.pow(2).mean(1).sqrt() / contrib
                worst = min(worst, float(ratio.min()))
            out[s, g] = worst
    return out.numpy()


def rows_within_bar(got, ref, tol, bf16, inp, log=print):
    """Every output row of the forward within tol; for bf16 storage, a row
    whose two maps cancel (cancellation_ratio below 0.2) is held to tol
    times 0.2 / that ratio instead: the RMSNorm divides the fixed bf16
    rounding of the probabilities (the PV operand) by rms(pre).  inp
    supplies the rows' inputs for the ratio (already rotated when the
    kernel rotates).  Returns the largest row error."""
    g = got.float().cpu().double().numpy()
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    if not ref.size:
        return 0.0
    row_err = np.abs(g - ref).max(axis=2)
    for t, h in np.argwhere(row_err > tol):
        assert bf16, (t, h, row_err[t, h])
        ratio = cancellation_ratio(inp, int(t), int(h))
        log(f"row (token {t}, head {h}): max-abs {row_err[t, h]:.3e}, "
            f"cancellation ratio {ratio:.4f}")
        assert ratio < 0.2 and row_err[t, h] <= tol * 0.2 / ratio
    return float(row_err.max())


def rotated(inp, rope):
    """A copy of inp whose q and k rows are turned as the rotary prologue
    turns them: pair (x[2j], x[2j+1]) of the row at position p of its
    sequence by (cos, sin)[p, j], stored back in the input's type."""
    cos, sin = (t.double() for t in rope)
    cu = inp.cu_seqlens.tolist()
    pos = torch.cat([torch.arange(cu[s + 1] - cu[s]) for s in range(len(cu) - 1)]).long()
    c, s_ = cos[pos], sin[pos]                                   # [T, d/2]

    def turn(x):
        x = x.double()
        x0, x1 = x[..., 0::2], x[..., 1::2]
        shape = (x.shape[0],) + (1,) * (x.dim() - 2) + (c.shape[1],)
        cc, ss = c.reshape(shape), s_.reshape(shape)
        y = torch.empty_like(x)
        y[..., 0::2] = x0 * cc - x1 * ss
        y[..., 1::2] = x0 * ss + x1 * cc
        return y.to(inp.q.dtype)

    out = copy.copy(inp)
    out.q, out.k = turn(inp.q), turn(inp.k)
    return out
