"""How far the two maps of an output row cancel before the RMSNorm: the
conditioning that scales the bf16 bar of the parity tests for such rows."""

import torch

import oracle


def cancellation_ratio(inp, t, h):
    """rms(pre) / rms(O_1) of output row (token t, head h), in fp64 from the
    definition: how far the two maps cancel before the RMSNorm."""
    cu = inp.cu_seqlens.tolist()
    s = max(j for j in range(len(cu) - 1) if cu[j] <= t)
    a, b = cu[s], cu[s + 1]
    H, Hkv, d = inp.q.shape[1], inp.k.shape[1], inp.q.shape[3]
    g = h // (H // Hkv)
    J = slice(a, t + 1) if inp.causal else slice(a, b)
    q, k, v = inp.q.double(), inp.k.double(), inp.v.double()
    lv = [x if x.dim() == 1 else x[h] for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
    lam = oracle.lam(*lv, oracle.lambda_init(inp.depth))
    o = []
    for m in range(2):
        x = (k[J, g, m] @ q[t, h, m]) / d ** 0.5
        pr = torch.softmax(x, dim=0)
        o.append(pr @ v[J, g])
    pre = o[0] - lam * o[1]
    return float(pre.pow(2).mean().sqrt() / o[0].pow(2).mean().sqrt())


def group_floor(inp):
    """[nseq, Hkv]: the smallest rms(pre)/rms(O_1) over the rows (token,
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
                o = []
                for m in range(2):
                    x = (q[a:b, h, m] @ k[a:b, g, m].T) / d ** 0.5
                    pr = torch.softmax(x.masked_fill(~mask, float("-inf")), dim=1)
                    o.append(pr @ v[a:b, g])
                pre = o[0] - lam * o[1]
                ratio = pre.pow(2).mean(1).sqrt() / o[0].pow(2).mean(1).sqrt()
                worst = min(worst, float(ratio.min()))
            out[s, g] = worst
    return out.numpy()
