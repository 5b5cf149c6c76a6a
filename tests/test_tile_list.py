"""The compact tile list of the prefill kernel's scheduler, restated on the
host: for packed sequences (at most 64) each workgroup finds its query tile
from cu_seqlens alone.  Level t lists query tile t of every sequence that
has one (in sequence order, each for all GH KV-group/head-block pairs);
levels run from the deepest down, so the longest causal work starts first.
cnt(t) = sum over sequences of max(0, nt_s - t) counts the entries at level
t or above; workgroup i (entry q = i // GH) takes the largest t with
cnt(t) > q and, within it, the (q - cnt(t + 1))-th sequence that has a
tile there.  The grid is sized by the bound T // bm + nseq.  These checks
run the same search over random length mixes: every existing tile exactly
once, levels non-increasing along the grid, and the workgroups past the
last tile at its end.  (The kernel's own output over such mixes is checked
against the oracle by the GPU parity tests.)"""

import numpy as np
import pytest


def entry(i, cnt, nt, GH):
    """The kernel's search for workgroup i; cnt[t] = cnt(t) for
    t = 0 .. ntile_q."""
    q, grp = divmod(i, GH)
    level = -1
    for t in range(len(cnt) - 1):   # the kernel: one ballot per 64 levels
        if cnt[t] > q:
            level = t
    if level < 0:
        return None
    k = q - cnt[level + 1]
    seqs = [s for s, n in enumerate(nt) if n > level]
    return level, seqs[k], grp


@pytest.mark.parametrize("seed", range(40))
def test_compact_tile_list_covers_every_tile_once(seed):
    rng = np.random.default_rng(seed)
    nseq = int(rng.integers(1, 65))
    hi = int(rng.choice([100, 700, 5000]))
    lens = [int(x) for x in rng.integers(0, hi, nseq)]
    lens[int(rng.integers(nseq))] = max(1, max(lens))
    bm = int(rng.choice([32, 64, 128, 256]))
    GH = int(rng.choice([1, 2, 4, 8]))
    T = sum(lens)
    ntile_q = -(-max(lens) // bm)
    nt = [min(-(-n // bm), ntile_q) for n in lens]
    grid = min(ntile_q * nseq, T // bm + nseq) * GH
    cnt = [sum(max(0, n - t) for n in nt) for t in range(ntile_q + 1)]
    got = [entry(i, cnt, nt, GH) for i in range(grid)]
    live = [g for g in got if g is not None]
    want = {(t, s, g) for s, n in enumerate(nt) for t in range(n) for g in range(GH)}
    assert len(live) == len(want) and set(live) == want
    levels = [g[0] for g in live]
    assert all(a >= b for a, b in zip(levels, levels[1:]))
    first_exit = next((i for i, g in enumerate(got) if g is None), len(got))
    assert all(g is None for g in got[first_exit:])
