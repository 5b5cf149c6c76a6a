"""The cancellation ratio used by the parity tests, pinned to its closed form
on the CPU."""

import torch

import oracle
from conditioning import cancellation_ratio
from workloads import custom, make_inputs


def test_cancellation_ratio_first_row_closed_form():
    """At the first token of a causal sequence both maps put all weight on
    V[0], so pre = (1 - lambda) V[0] and the ratio is
    |1 - lambda| / (1 + |lambda|) exactly (CPU only)."""
    wl = custom("ratio", "bf16", (3, 5), 4, 2, 16, depth=3, seed=5)
    inp = make_inputs(wl)
    g = torch.Generator().manual_seed(6)
    inp.lq1, inp.lk1, inp.lq2, inp.lk2 = [0.4 * torch.randn(4, 16, generator=g)
                                          for _ in range(4)]
    lam0 = oracle.lambda_init(inp.depth)
    for t in (0, 3):
        for h in range(4):
            lam = oracle.lam(inp.lq1[h], inp.lk1[h], inp.lq2[h], inp.lk2[h], lam0)
            want = abs(1 - lam) / (1 + abs(lam))
            assert abs(cancellation_ratio(inp, t, h) - want) < 1e-9


def test_group_floor_equals_rowwise_minimum():
    """The per-(sequence, KV group) minimum, from whole score matrices, equals
    the minimum of the row-by-row ratio (CPU only)."""
    import numpy as np
    from conditioning import group_floor
    for causal in (True, False):
        wl = custom("floor", "bf16", (5, 9, 0, 4), 4, 2, 16, depth=3, causal=causal, seed=2)
        inp = make_inputs(wl)
        g = torch.Generator().manual_seed(1)
        inp.lq1, inp.lk1, inp.lq2, inp.lk2 = [0.5 * torch.randn(4, 16, generator=g)
                                              for _ in range(4)]
        floor = group_floor(inp)
        cu = inp.cu_seqlens.tolist()
        brute = np.ones_like(floor)
        for s in range(len(cu) - 1):
            for t in range(cu[s], cu[s + 1]):
                for h in range(4):
                    brute[s, h // 2] = min(brute[s, h // 2], cancellation_ratio(inp, t, h))
        assert np.abs(floor - brute).max() < 1e-12


def test_rotated_copy_matches_the_oracle_rotary_path():
    """Attention on rows turned by `rotated` equals the oracle's own rotary
    prologue with bf16 storage of the rotated rows (CPU only)."""
    import numpy as np
    from conditioning import rotated
    from workloads import rope_tables
    wl = custom("rot", "bf16", (7, 0, 12), 4, 2, 16, depth=2, seed=4)
    inp = make_inputs(wl)
    rope = rope_tables(20, 16, base=50.0)
    lam0 = oracle.lambda_init(inp.depth)
    ref = oracle.fwd(inp.q, inp.k, inp.v, inp.lq1, inp.lk1, inp.lq2, inp.lk2, lam0, inp.w,
                     inp.eps, inp.causal, inp.cu_seqlens, rope=rope, rope_round_bf16=True)
    r = rotated(inp, rope)
    got = oracle.fwd(r.q, r.k, r.v, r.lq1, r.lk1, r.lq2, r.lk2, lam0, r.w, r.eps, r.causal,
                     r.cu_seqlens)
    assert np.abs(got - ref).max() < 1e-12
