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


def test_bar_factor_is_capped():
    """Rows that cancel get 0.2 / ratio times the bar, never more than 4x
    (CPU only)."""
    from conditioning import CAP, bar_factor
    assert CAP == 4.0
    assert bar_factor(0.5) == 1.0 and bar_factor(0.2) == 1.0
    assert abs(bar_factor(0.1) - 2.0) < 1e-12
    assert bar_factor(0.05) == 4.0 and bar_factor(1e-9) == 4.0 and bar_factor(0.0) == 4.0


def _case(causal, seed):
    wl = custom("factors", "bf16", (5, 9, 0, 4, 1), 4, 2, 16, depth=3, causal=causal, seed=seed)
    inp = make_inputs(wl)
    g = torch.Generator().manual_seed(seed + 1)
    # vectors at 0.5 scale: heads with lambda near 1, so some rows cancel
    inp.lq1, inp.lk1, inp.lq2, inp.lk2 = [0.5 * torch.randn(4, 16, generator=g)
                                          for _ in range(4)]
    return inp


def test_row_factors_equal_rowwise_ratios():
    """The backward's per-row multipliers, from whole score matrices, equal
    bar_factor of the row-by-row ratio, and 1 where a row sees one key
    (CPU only)."""
    import numpy as np
    from conditioning import bar_factor, row_factors
    seen_wide = False
    for causal in (True, False):
        for seed in (2, 3, 4):
            inp = _case(causal, seed)
            rf = row_factors(inp)
            cu = inp.cu_seqlens.tolist()
            for s in range(len(cu) - 1):
                for t in range(cu[s], cu[s + 1]):
                    single = (t == cu[s]) if causal else (cu[s + 1] - cu[s] == 1)
                    for h in range(4):
                        want = 1.0 if single else bar_factor(cancellation_ratio(inp, t, h))
                        assert abs(rf[t, h] - want) < 1e-9, (causal, seed, t, h)
                        seen_wide |= want > 1.0
            assert rf.max() <= 4.0
    assert seen_wide   # the cases do reach the wider bar


def test_key_factors_take_the_worst_row_that_sees_the_key():
    """dk/dv multiplier of key j = max of the row factors of the group's rows
    that see j (brute force over rows; CPU only)."""
    import numpy as np
    from conditioning import key_factors
    for causal in (True, False):
        inp = _case(causal, 7)
        T = inp.q.shape[0]
        rng = np.random.default_rng(0)
        rf = rng.uniform(1.0, 4.0, (T, 4))
        kf = key_factors(inp, rf)
        cu = inp.cu_seqlens.tolist()
        for s in range(len(cu) - 1):
            for j in range(cu[s], cu[s + 1]):
                for g in range(2):
                    rows = [(t, h) for t in range(cu[s], cu[s + 1])
                            for h in (2 * g, 2 * g + 1) if (t >= j or not causal)]
                    assert kf[j, g] == max(rf[t, h] for t, h in rows)


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
