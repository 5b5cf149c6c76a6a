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
