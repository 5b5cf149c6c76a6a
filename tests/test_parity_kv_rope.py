"""Rotary embedding at decode time, through the C ABI: the cache update
(diffattn_kv_append) and the new queries' rotation inside diffattn_fwd_kv,
against the fp64 oracle.  The LlamaDiffSdpaAttention.py gist's forward
turns the step's queries and keys at their position ids, appends the keys
and values to the cache, then attends; the rotation itself is the one the
FlashDiffAttention pull request's test applies (interleaved pairs of each
d-wide half-head).

Bars: attention outputs max-abs 2e-2 (bf16 storage); rotated cache rows
within one unit in the last place of the storage type of the fp64 rotation
plus the fp32 rounding of the rotation's two terms (the kernel rotates in
fp32 and rounds once), copied rows and values bitwise.  bf16 tables give bitwise the output of fp32 tables holding the
same values.  All tests need an MI355X.
"""

import numpy as np
import pytest
import torch

import oracle
from conditioning import turn
from workloads import custom, custom_kv, make_inputs, make_kv_inputs, rope_tables

pytestmark = pytest.mark.gpu

TOL = 2e-2
DEV = torch.device("cuda:0")


def _da():
    import differential_attention_amd as da
    return da


def announce(msg):
    print(f"[parity-kv-rope] {msg}", flush=True)


def c(t):
    return t.to(DEV).contiguous()


def positions(cu_q, cu_k):
    """Absolute position nk - nq + i of every new token, packed."""
    cq, ck = cu_q.tolist(), cu_k.tolist()
    return torch.cat([torch.arange(ck[s + 1] - ck[s] - (cq[s + 1] - cq[s]),
                                   ck[s + 1] - ck[s]) for s in range(len(cq) - 1)]).long()


def tables(length, d, kind):
    """Strongly turning tables (base 50); kind "bf16" rounds them to bf16."""
    rc, rs = rope_tables(length, d, base=50.0)
    if kind == "bf16":
        rc, rs = rc.bfloat16(), rs.bfloat16()
    return rc, rs


def fwd_kv(inp, rope=None, noalloc=False):
    da = _da()
    lv = [c(x) for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
    f = da.fwd_kv_noalloc if noalloc else da.fwd_kv
    out = f(c(inp.q), c(inp.k), c(inp.v), *lv, da.lambda_init(inp.depth), c(inp.w),
            inp.eps, inp.causal, cu_seqlens_q=c(inp.cu_q), cu_seqlens_k=c(inp.cu_k),
            max_seqlen_q=inp.max_q, max_seqlen_k=inp.max_k,
            rope=None if rope is None else tuple(c(t) for t in rope))
    torch.cuda.synchronize()
    return out


def max_abs(gpu_out, ref):
    got = gpu_out.float().cpu().double().numpy()
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    return float(np.max(np.abs(got - ref))) if ref.size else 0.0


RAGGED = [
    ((1, 3, 5, 16, 2), (37, 100, 250, 600, 2)),
    ((1, 1, 1), (1, 31, 33)),
    ((8, 0, 4), (8, 50, 4)),
]


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("H,Hkv,d", [(8, 2, 64), (4, 4, 32), (12, 4, 64)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("case", range(len(RAGGED)))
def test_queries_rotated_at_their_positions(kind, H, Hkv, d, causal, case):
    """fwd_kv with tables equals the oracle on queries turned at nk - nq + i
    (the cache keys are taken as already rotated)."""
    ql, kl = RAGGED[case]
    wl = custom_kv("kv_rope", "bf16", ql, kl, H=H, Hkv=Hkv, d=d, depth=6,
                   causal=causal, seed=300 + case)
    inp = make_kv_inputs(wl)
    rope = tables(max(kl), d, kind)
    out = fwd_kv(inp, rope)
    qr = turn(inp.q, positions(inp.cu_q, inp.cu_k), tuple(t.float() for t in rope))
    ref = oracle.fwd_kv(qr, inp.k, inp.v, inp.lq1, inp.lk1, inp.lq2, inp.lk2,
                        oracle.lambda_init(inp.depth), inp.w, inp.eps, inp.causal,
                        inp.cu_q.numpy(), inp.cu_k.numpy())
    err = max_abs(out, ref)
    announce(f"case {case} {kind} tables H={H} Hkv={Hkv} d={d} causal={causal}: "
             f"max-abs {err:.3e}")
    assert err <= TOL


def test_bf16_tables_equal_fp32_tables_of_the_same_values():
    ql, kl = RAGGED[0]
    wl = custom_kv("kv_rope_tab", "bf16", ql, kl, H=8, Hkv=2, d=64, depth=3, seed=310)
    inp = make_kv_inputs(wl)
    rb = tables(max(kl), 64, "bf16")
    a = fwd_kv(inp, rb)
    b = fwd_kv(inp, tuple(t.float() for t in rb))
    assert torch.equal(a, b)


def test_rope_no_alloc_equals_workspace_path():
    ql, kl = RAGGED[0]
    wl = custom_kv("kv_rope_na", "bf16", ql, kl, H=8, Hkv=2, d=64, depth=3, seed=311)
    inp = make_kv_inputs(wl)
    rope = tables(max(kl), 64, "f32")
    assert torch.equal(fwd_kv(inp, rope), fwd_kv(inp, rope, noalloc=True))


def ulp(x, dtype):
    """One unit in the last place of |x| in dtype (fp64 values)."""
    mant = 7 if dtype == torch.bfloat16 else 23
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))
    return np.exp2(e - mant)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [16, 32, 64])
@pytest.mark.parametrize("kind", ["f32", "bf16", None])
def test_append_places_and_rotates(dtype, d, kind):
    """New keys and values land in the last nq rows of each sequence's
    cache region, keys turned at their positions; every other row is left
    as it was."""
    da = _da()
    ql, kl = (3, 0, 1, 7, 2), (40, 5, 1, 7, 300)
    Hkv = 3
    g = torch.Generator().manual_seed(d + (0 if kind is None else len(kind)))
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(ql)]), dtype=torch.int32)
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(kl)]), dtype=torch.int32)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    k_new = torch.randn(Tq, Hkv, 2, d, generator=g).to(dtype)
    v_new = torch.randn(Tq, Hkv, 2 * d, generator=g).to(dtype)
    k_old = torch.randn(Tk, Hkv, 2, d, generator=g).to(dtype)
    v_old = torch.randn(Tk, Hkv, 2 * d, generator=g).to(dtype)
    rope = None if kind is None else tables(max(kl), d, kind)
    kc, vc = c(k_old), c(v_old)
    da.kv_append(c(k_new), c(v_new), kc, vc, cu_seqlens_q=c(cu_q), cu_seqlens_k=c(cu_k),
                 max_seqlen_k=max(kl),
                 rope=None if rope is None else tuple(c(t) for t in rope))
    torch.cuda.synchronize()
    kc, vc = kc.cpu(), vc.cpu()
    rows = torch.cat([torch.arange(int(cu_k[s + 1]) - ql[s], int(cu_k[s + 1]))
                      for s in range(len(ql))]).long()
    others = torch.ones(Tk, dtype=torch.bool)
    others[rows] = False
    assert torch.equal(kc[others], k_old[others]) and torch.equal(vc[others], v_old[others])
    assert torch.equal(vc[rows], v_new)
    if rope is None:
        assert torch.equal(kc[rows], k_new)
        return
    ref = turn(k_new.double(), positions(cu_q, cu_k),
               tuple(t.float() for t in rope)).numpy()          # fp64 rotation
    got = kc[rows].double().numpy()
    # one unit of the stored type, plus the fp32 rounding of the two terms
    # of the rotation (a pair can cancel to far below its terms)
    x = k_new.double().numpy()
    mag = np.repeat(np.hypot(x[..., 0::2], x[..., 1::2]), 2, axis=-1)
    bound = ulp(ref, dtype) + 2 * ulp(mag, torch.float32)
    rounded = torch.from_numpy(ref).to(dtype).double().numpy()
    exact = float(np.mean(got == rounded))
    worst = float(np.max(np.abs(got - ref) / bound))
    announce(f"append {dtype} d={d} {kind} tables: worst {worst:.2f} of the bound, "
             f"{100 * exact:.2f}% rounded as the fp64 value")
    assert worst <= 1.0


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("H,Hkv,d", [(16, 4, 64), (6, 2, 32)])
def test_decode_step_equals_rotary_prefill_rows(kind, H, Hkv, d):
    """A whole decode step with rotary tables -- the prompt's keys appended
    (and turned) sequence by sequence, then the step's new keys, then the
    new queries against the cache -- gives the rows of the oracle's causal
    prefill with its own rotary prologue at those tokens."""
    da = _da()
    lens, news = (700, 65, 257, 3), (1, 4, 16, 3)
    wl = custom("rope_step", "bf16", lens, H=H, Hkv=Hkv, d=d, depth=7, seed=17 + d)
    pf = make_inputs(wl)
    rope = tables(max(lens), d, kind)
    rdev = tuple(c(t) for t in rope)
    cu = pf.cu_seqlens.tolist()
    k_cache = torch.zeros_like(c(pf.k))
    v_cache = torch.zeros_like(c(pf.v))
    # the prompt: each sequence's first L - n tokens, positions from 0
    for s, (L, n) in enumerate(zip(lens, news)):
        P = L - n
        if P == 0:
            continue
        a = cu[s]
        da.kv_append(c(pf.k[a:a + P]), c(pf.v[a:a + P]), k_cache[a:a + P], v_cache[a:a + P],
                     nseq=1, rope=rdev)
    # the step: the last n tokens of every sequence
    new_rows = torch.cat([torch.arange(cu[s + 1] - n, cu[s + 1])
                          for s, n in enumerate(news)]).long()
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(news)]), dtype=torch.int32)
    da.kv_append(c(pf.k[new_rows]), c(pf.v[new_rows]), k_cache, v_cache,
                 cu_seqlens_q=c(cu_q), cu_seqlens_k=c(pf.cu_seqlens),
                 max_seqlen_k=max(lens), rope=rdev)
    lv = [c(x) for x in (pf.lq1, pf.lk1, pf.lq2, pf.lk2)]
    out = da.fwd_kv(c(pf.q[new_rows]), k_cache, v_cache, *lv, da.lambda_init(wl.depth),
                    c(pf.w), wl.eps, True, cu_seqlens_q=c(cu_q),
                    cu_seqlens_k=c(pf.cu_seqlens), max_seqlen_q=max(news),
                    max_seqlen_k=max(lens), rope=rdev)
    torch.cuda.synchronize()
    heads = np.arange(H, dtype=np.int32)
    toks = np.repeat(new_rows.numpy(), H)
    ref = oracle.rows(pf.q, pf.k, pf.v, pf.lq1, pf.lk1, pf.lq2, pf.lk2,
                      oracle.lambda_init(wl.depth), toks, np.tile(heads, new_rows.numel()),
                      pf.w, wl.eps, True, pf.cu_seqlens,
                      rope=tuple(t.float() for t in rope), rope_round_bf16=True)
    err = max_abs(out.reshape(-1, 2 * d), ref.reshape(-1, 2 * d))
    announce(f"decode step {kind} tables H={H} Hkv={Hkv} d={d}: max-abs {err:.3e}")
    assert err <= TOL
