"""Parity of the cache path on long query chunks with the fp64 oracle:
diffattn_fwd_kv calls whose bounds make the split-KV kernels' rows x keys
cost outweigh the prefill kernel's run on that kernel with the keys' own
boundaries -- over whole key ranges (no workspace), or over key splits
merged by the combine kernel when whole ranges would leave CUs idle.  The
tests read the path from diffattn_fwd_kv_path.

A chunk is the method's attention for the nq newest tokens of a sequence of
nk: query i sees keys 0 .. nk - nq + i under the causal mask, all nk keys
without it -- so a prompt cut into chunks gives, chunk by chunk, the rows of
its one-shot prefill.  The oracle's fwd_kv states that row by row; at full
size the prefill rows of the oracle (oracle.rows) stand in for it on sampled
tokens.

Tolerance: bf16 storage, max-abs 2e-2 over every compared element.  All
tests need an MI355X.
"""

import numpy as np
import pytest
import torch

import oracle
from conditioning import turn
from workloads import (WORKLOADS, custom, custom_kv, make_inputs, make_kv_inputs,
                       rope_tables)

pytestmark = pytest.mark.gpu

TOL = 2e-2
DEV = torch.device("cuda:0")


def _da():
    import differential_attention_amd as da
    return da


def announce(msg):
    print(f"[parity-kv-chunk] {msg}", flush=True)


def c(t):
    return t.to(DEV).contiguous()


def path(inp, max_q=None):
    """The kernels the call runs: 0 split-KV, 1 prefill kernel, 2 prefill
    kernel on key splits."""
    Tq, H, _, d = inp.q.shape
    Tk, Hkv = inp.k.shape[:2]
    return _da().kv_path(inp.cu_q.numel() - 1, max_q or inp.max_q, inp.max_k, H, Hkv, d,
                         Tq=Tq, Tk=Tk)


def on_every_path(inp, ref, what, **kw):
    """The call on the library's own path and on each forced one (key splits
    where there are more than 256 keys to split), against ref."""
    paths = [None, 0, 1] + ([2] if inp.max_k > 256 else [])
    for pth in paths:
        err = max_abs(gpu_kv(inp, on_path=pth, **kw), ref)
        announce(f"{what}, path {'auto ' + str(path(inp)) if pth is None else pth}: "
                 f"max-abs {err:.3e}")
        assert err <= TOL


def gpu_kv(inp, lam=None, rope=None, uniform=False, noalloc=False, out=None, max_q=None,
           on_path=None, workspace=None, max_k=None):
    da = _da()
    lv = [c(x) for x in (lam if lam is not None else (inp.lq1, inp.lk1, inp.lq2, inp.lk2))]
    kw = {}
    if uniform:
        kw["nseq"] = inp.cu_q.numel() - 1
    else:
        kw.update(cu_seqlens_q=c(inp.cu_q), cu_seqlens_k=c(inp.cu_k),
                  max_seqlen_q=max_q or inp.max_q, max_seqlen_k=max_k or inp.max_k)
    if rope is not None:
        kw["rope"] = tuple(c(t) for t in rope)
    if out is not None:
        kw["out"] = out
    if on_path is not None:
        kw["path"] = on_path
    if workspace is not None:
        kw["workspace"] = workspace
    f = da.fwd_kv_noalloc if noalloc else da.fwd_kv
    res = f(c(inp.q), c(inp.k), c(inp.v), *lv, da.lambda_init(inp.depth), c(inp.w),
            inp.eps, inp.causal, **kw)
    torch.cuda.synchronize()
    return res


def oracle_kv(inp, lam=None, q=None):
    lv = lam if lam is not None else (inp.lq1, inp.lk1, inp.lq2, inp.lk2)
    return oracle.fwd_kv(inp.q if q is None else q, inp.k, inp.v, *lv,
                         oracle.lambda_init(inp.depth), inp.w, inp.eps, inp.causal,
                         inp.cu_q.numpy(), inp.cu_k.numpy())


def max_abs(gpu_out, ref):
    got = gpu_out.float().cpu().double().numpy()
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    return float(np.max(np.abs(got - ref))) if ref.size else 0.0


def positions(cu_q, cu_k):
    """Absolute position nk - nq + i of every new token, packed."""
    cq, ck = cu_q.tolist(), cu_k.tolist()
    return torch.cat([torch.arange(ck[s + 1] - ck[s] - (cq[s + 1] - cq[s]),
                                   ck[s + 1] - ck[s]) for s in range(len(cq) - 1)]).long()


# ---------------------------------------------------------------------------
# shapes, masks and edge cases at sizes the oracle finishes in seconds

CHUNKS = [
    # query lengths, key lengths: a long chunk beside one-token decodes, an
    # empty query set, a chunk that is its whole sequence (nq == nk) and
    # ragged tails of the 64- and 128-row tiles
    ((200, 1, 0, 130, 257), (1000, 700, 50, 130, 1100)),
    ((128,), (128,)),
    ((300, 129), (301, 1500)),
    ((1000, 3), (1000, 4)),
]


@pytest.mark.parametrize("H,Hkv,d", [(8, 2, 64), (4, 4, 32), (12, 4, 64), (16, 1, 64),
                                     (10, 5, 32)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("case", range(len(CHUNKS)))
def test_chunk_ragged_matrix(H, Hkv, d, causal, case):
    """Every path on each case (key splits where there are more than 256
    keys to split), and the library's own choice bitwise equal to running
    the path it reports."""
    ql, kl = CHUNKS[case]
    wl = custom_kv("chunk", "bf16", ql, kl, H=H, Hkv=Hkv, d=d, depth=5, causal=causal,
                   seed=700 + case)
    inp = make_kv_inputs(wl)
    inp.w.copy_(0.5 + torch.rand(2 * d, generator=torch.Generator().manual_seed(case)))
    ref = oracle_kv(inp)
    outs = {}
    for pth in (0, 1, 2):
        if pth == 2 and max(kl) <= 256:
            continue
        outs[pth] = gpu_kv(inp, on_path=pth)
        err = max_abs(outs[pth], ref)
        announce(f"case {case} H={H} Hkv={Hkv} d={d} causal={causal} path {pth}: "
                 f"max-abs {err:.3e}")
        assert err <= TOL
    auto = path(inp)
    assert torch.equal(gpu_kv(inp), outs[auto])


def test_paths_on_the_same_call():
    """max_seqlen_q is an upper bound (at most Tq), and with the other sizes
    it picks the path: 8 queries per sequence under a bound of 8 take the
    prefill kernel on key splits, under a loose bound the split-KV kernels.
    Every path met meets the bar on the same data."""
    wl = custom_kv("paths", "bf16", (8,) * 8, (4096,) * 8, H=16, Hkv=4, d=64, depth=3,
                   seed=710)
    inp = make_kv_inputs(wl)
    bounds = {}
    for b in (8, 16, 32, 64):
        bounds.setdefault(path(inp, b), b)
    assert 0 in bounds and 2 in bounds
    ref = oracle_kv(inp)
    for pth, b in sorted(bounds.items()):
        err = max_abs(gpu_kv(inp, max_q=b), ref)
        announce(f"bound {b} (path {pth}): max-abs {err:.3e}")
        assert err <= TOL


def test_many_sequences_on_key_splits():
    """More than 64 sequences, with empty ones and caches of every length up
    to several splits, on each path: a split slot finds its sequence by the
    kernels' scan of cu_seqlens_k across 64-sequence steps, and a sequence
    without keys owns no slot."""
    rng = np.random.default_rng(740)
    nseq = 150
    kl = [int(x) for x in rng.integers(1, 2500, nseq)]
    ql = [int(min(q, k)) for q, k in zip(rng.integers(0, 40, nseq), kl)]
    for s in (0, 63, 64, 100, 149):   # empty sequences, on and off step edges
        ql[s], kl[s] = 0, 0
    ql[70] = 0                         # keys only
    wl = custom_kv("many", "bf16", tuple(ql), tuple(kl), H=8, Hkv=2, d=64, depth=4, seed=741)
    inp = make_kv_inputs(wl)
    on_every_path(inp, oracle_kv(inp), f"{nseq} sequences, Tk={sum(kl)}")


def test_uniform_chunks_without_boundaries():
    wl = custom_kv("uni", "bf16", (160,) * 3, (500,) * 3, H=16, Hkv=4, d=64, depth=6,
                   seed=711)
    inp = make_kv_inputs(wl)
    ref = oracle_kv(inp)
    for pth in (None, 0, 1, 2):
        a = gpu_kv(inp, uniform=True, on_path=pth)
        assert torch.equal(a, gpu_kv(inp, on_path=pth))
        err = max_abs(a, ref)
        announce(f"uniform chunks, path {pth}: max-abs {err:.3e}")
        assert err <= TOL


def test_more_queries_than_keys_noncausal():
    wl = custom_kv("nc", "bf16", (300, 150), (100, 2), H=8, Hkv=2, d=64, causal=False,
                   seed=712)
    inp = make_kv_inputs(wl)
    on_every_path(inp, oracle_kv(inp), "nq > nk, non-causal")


def test_large_logits():
    wl = custom_kv("big", "bf16", (600, 140), (3000, 5000), H=8, Hkv=2, d=64, depth=2,
                   seed=713)
    inp = make_kv_inputs(wl, q_scale=30.0)
    on_every_path(inp, oracle_kv(inp), "large logits")


def test_per_head_lambda():
    wl = custom_kv("ph", "bf16", (400, 2), (900, 70), H=8, Hkv=2, d=64, depth=4, seed=714)
    inp = make_kv_inputs(wl)
    g = torch.Generator().manual_seed(715)
    lam = [0.2 * torch.randn(wl.H, wl.d, generator=g) for _ in range(4)]
    on_every_path(inp, oracle_kv(inp, lam=lam), "per-head lambda", lam=lam)


@pytest.mark.parametrize("ql,kl", [((700, 64), (4000, 64)), ((16,) * 8, (4096,) * 8),
                                   ((64,) * 8, (4096,) * 8), ((2000,), (2000,))])
def test_deterministic_no_alloc_and_output_bounds(ql, kl):
    """Bitwise equal on repeated calls; rows around a provided output are
    left untouched.  The no-allocation entry point gives the same bits on
    the prefill kernel alone and when the workspace bound fits its static
    scratch; when key splits' partials would not fit, it takes the plan of a
    call given a workspace of the scratch's size (same bar, another
    rounding order), and those bits."""
    da = _da()
    wl = custom_kv("det", "bf16", ql, kl, H=16, Hkv=4, d=64, depth=8, seed=716)
    inp = make_kv_inputs(wl)
    pth = path(inp)
    assert pth in (1, 2)
    a = gpu_kv(inp)
    assert torch.equal(a, gpu_kv(inp))
    na = gpu_kv(inp, noalloc=True)
    need = da.kv_workspace_size(len(ql), max(ql), max(kl), 16, 4, 64)
    if pth == 1 or need <= da.KV_SCRATCH_BYTES:
        assert torch.equal(a, na)
    else:
        ws = torch.empty(da.KV_SCRATCH_BYTES, dtype=torch.uint8, device=DEV)
        assert torch.equal(gpu_kv(inp, workspace=ws), na)
    ref = oracle_kv(inp)
    e1, e2 = max_abs(a, ref), max_abs(na, ref)
    announce(f"path {pth}, workspace bound {need / 2**20:.1f} MiB: max-abs {e1:.3e}, "
             f"no-alloc {e2:.3e}")
    assert e1 <= TOL and e2 <= TOL
    out = torch.full((inp.q.shape[0] + 2, 16, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    gpu_kv(inp, out=out[1:-1])
    assert torch.all(out[0] == 7.0) and torch.all(out[-1] == 7.0)
    assert torch.equal(out[1:-1], a)


# ---------------------------------------------------------------------------
# rotary chunks: the queries turn at their absolute positions nk - nq + i

@pytest.mark.parametrize("nq,nk,bq,bk", [(64, 8192, 100, 8192), (512, 4096, 1024, 4096),
                                         (100, 4097, 100, 8192)])
def test_workspace_of_larger_bounds_serves_a_smaller_call(nq, nk, bq, bk):
    """A workspace sized for larger bounds (a serving loop's one
    allocation) runs a call whose own first choice of key splits would need
    more: the call takes the cheapest split plan that fits, which is what
    the forced key-split path gives with the same workspace."""
    da = _da()
    nseq, H, Hkv, d = 2, 16, 4, 64
    W = da.kv_workspace_size(nseq, bq, bk, H, Hkv, d)
    first = da.kv_plan(nseq, nq, nk, H, Hkv, d)
    capped = da.kv_plan(nseq, nq, nk, H, Hkv, d, workspace_bytes=W)
    announce(f"{nseq} x ({nq} vs {nk}) in a workspace for ({bq} vs {bk}): {W / 2**20:.1f} MiB; "
             f"first choice {first}, with it {capped}")
    assert first[1] > W >= capped[1] and capped[0] in (1, 2)
    wl = custom_kv("wsbound", "bf16", (nq,) * nseq, (nk,) * nseq, H=H, Hkv=Hkv, d=d, depth=6,
                   seed=731)
    inp = make_kv_inputs(wl)
    ws = torch.empty(W, dtype=torch.uint8, device=DEV)
    got = gpu_kv(inp, workspace=ws)
    assert torch.equal(got, gpu_kv(inp, workspace=ws, on_path=capped[0]))
    err = max_abs(got, oracle_kv(inp))
    announce(f"max-abs vs oracle {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("H,Hkv,d", [(8, 2, 64), (4, 4, 32), (12, 4, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_rotary_chunks(kind, H, Hkv, d, causal):
    ql, kl = CHUNKS[0]
    wl = custom_kv("chunk_rope", "bf16", ql, kl, H=H, Hkv=Hkv, d=d, depth=6, causal=causal,
                   seed=720)
    inp = make_kv_inputs(wl)
    rc, rs = rope_tables(max(kl), d, base=50.0)
    rope = (rc.bfloat16(), rs.bfloat16()) if kind == "bf16" else (rc, rs)
    qr = turn(inp.q, positions(inp.cu_q, inp.cu_k), tuple(t.float() for t in rope))
    ref = oracle_kv(inp, q=qr)
    for pth in (None, 0, 1, 2):
        err = max_abs(gpu_kv(inp, rope=rope, on_path=pth), ref)
        announce(f"rotary {kind} H={H} Hkv={Hkv} d={d} causal={causal} path {pth}: "
                 f"max-abs {err:.3e}")
        assert err <= TOL


@pytest.mark.parametrize("on_path", [None, 1, 2])
@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_chunked_rotary_prefill_equals_prefill_rows(kind, on_path):
    """A prompt run as a chunked prefill -- each chunk's keys appended
    (turned) to the cache, then its queries against the cache so far --
    gives the rows of the oracle's one-shot causal prefill with its own
    rotary prologue."""
    da = _da()
    lens, H, Hkv, d = (1000, 300, 700), 16, 4, 64
    cuts = (0, 300, 429, 1000)                   # chunk boundaries per sequence
    wl = custom("chunked", "bf16", lens, H=H, Hkv=Hkv, d=d, depth=7, seed=721)
    pf = make_inputs(wl)
    rc, rs = rope_tables(max(lens), d, base=50.0)
    rope = (rc.bfloat16(), rs.bfloat16()) if kind == "bf16" else (rc, rs)
    rdev = tuple(c(t) for t in rope)
    cu = pf.cu_seqlens.tolist()
    kc, vc = torch.zeros_like(c(pf.k)), torch.zeros_like(c(pf.v))
    out = torch.zeros((pf.q.shape[0], H, 2 * d), dtype=torch.bfloat16, device=DEV)
    lv = [c(x) for x in (pf.lq1, pf.lk1, pf.lq2, pf.lk2)]
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        # chunk [lo, hi) of every sequence (clipped to its length)
        ql = [max(0, min(hi, L) - lo) for L in lens]
        kl = [min(hi, L) for L in lens]
        rows = torch.cat([torch.arange(cu[s] + lo, cu[s] + lo + n)
                          for s, n in enumerate(ql)]).long()
        cu_q = torch.tensor(np.concatenate([[0], np.cumsum(ql)]), dtype=torch.int32)
        cu_k = torch.tensor(np.concatenate([[0], np.cumsum(kl)]), dtype=torch.int32)
        # the cache holds each sequence's first kl tokens, packed
        krows = torch.cat([torch.arange(cu[s], cu[s] + n) for s, n in enumerate(kl)]).long()
        kcur, vcur = kc[krows.to(DEV)], vc[krows.to(DEV)]
        da.kv_append(c(pf.k[rows]), c(pf.v[rows]), kcur, vcur, cu_seqlens_q=c(cu_q),
                     cu_seqlens_k=c(cu_k), max_seqlen_k=max(kl), rope=rdev)
        kc[krows.to(DEV)], vc[krows.to(DEV)] = kcur, vcur
        o = da.fwd_kv(c(pf.q[rows]), kcur, vcur, *lv, da.lambda_init(wl.depth), c(pf.w),
                      wl.eps, True, cu_seqlens_q=c(cu_q), cu_seqlens_k=c(cu_k),
                      max_seqlen_q=max(ql), max_seqlen_k=max(kl), rope=rdev, path=on_path)
        out[rows.to(DEV)] = o
    torch.cuda.synchronize()
    toks = np.arange(pf.q.shape[0], dtype=np.int64)
    heads = np.arange(H, dtype=np.int32)
    ref = oracle.rows(pf.q, pf.k, pf.v, pf.lq1, pf.lk1, pf.lq2, pf.lk2,
                      oracle.lambda_init(wl.depth), np.repeat(toks, H),
                      np.tile(heads, toks.size), pf.w, wl.eps, True, pf.cu_seqlens,
                      rope=tuple(t.float() for t in rope), rope_round_bf16=True)
    err = max_abs(out.reshape(-1, 2 * d), ref.reshape(-1, 2 * d))
    announce(f"chunked rotary prefill ({kind} tables, path {on_path}): max-abs {err:.3e}")
    assert err <= TOL


# ---------------------------------------------------------------------------
# full size: the last quarter of the 8 x 4096 prefill as one chunk

def test_full_size_chunk_of_the_headline_prefill():
    """The last 1024 tokens of each of the 8 x 4096 prefill's sequences as a
    chunk against all 4096 keys (16 heads, 4 KV heads, d = 64): every head
    of one token in four, and of every token of the first and last 128 of
    each chunk, against the oracle's prefill rows."""
    da = _da()
    wl = WORKLOADS["llama1b_b8_n4096"]
    pf = make_inputs(wl)
    B, N, n = 8, 4096, 1024
    rows = torch.cat([torch.arange(s * N + N - n, s * N + N) for s in range(B)]).long()
    cu_q = torch.arange(0, B + 1, dtype=torch.int32) * n
    lv = [c(x) for x in (pf.lq1, pf.lk1, pf.lq2, pf.lk2)]
    assert da.kv_path(B, n, N, wl.H, wl.Hkv, wl.d) in (1, 2)
    announce("8 x (1024 vs 4096) chunk: full-size GPU run")
    out = da.fwd_kv(c(pf.q[rows]), c(pf.k), c(pf.v), *lv, da.lambda_init(wl.depth),
                    c(pf.w), wl.eps, True, cu_seqlens_q=c(cu_q),
                    cu_seqlens_k=c(pf.cu_seqlens), max_seqlen_q=n, max_seqlen_k=N)
    torch.cuda.synchronize()
    pick = set(range(0, B * n, 4))
    for s in range(B):
        pick |= set(range(s * n, s * n + 128)) | set(range(s * n + n - 128, s * n + n))
    pick = np.array(sorted(pick), np.int64)
    toks = rows.numpy()[pick]
    rows_t = np.repeat(toks, wl.H)
    rows_h = np.tile(np.arange(wl.H, dtype=np.int32), toks.size)
    ref = oracle.rows(pf.q, pf.k, pf.v, pf.lq1, pf.lk1, pf.lq2, pf.lk2,
                      oracle.lambda_init(wl.depth), rows_t, rows_h, pf.w, wl.eps, True,
                      pf.cu_seqlens)
    got = out[torch.from_numpy(np.repeat(pick, wl.H)).to(DEV),
              torch.from_numpy(rows_h).long().to(DEV)]
    err = max_abs(got, ref)
    announce(f"8 x (1024 vs 4096) chunk: {rows_t.size} rows, max-abs {err:.3e}")
    assert err <= TOL


def test_full_size_long_context_chunk_on_key_splits():
    """One 32768-token sequence whose last 1024 tokens form the chunk (16
    heads, 4 KV heads, d = 64): too few query tiles to fill the GPU, so the
    keys are split and merged.  Every head of one token in eight, and of the
    chunk's first and last 64 tokens, against the oracle's prefill rows."""
    da = _da()
    N, n, H, Hkv, d = 32768, 1024, 16, 4, 64
    wl = custom("long_chunk", "bf16", (N,), H=H, Hkv=Hkv, d=d, depth=12, seed=730)
    pf = make_inputs(wl)
    assert da.kv_path(1, n, N, H, Hkv, d) == 2
    rows = torch.arange(N - n, N)
    lv = [c(x) for x in (pf.lq1, pf.lk1, pf.lq2, pf.lk2)]
    announce("1 x (1024 vs 32768) chunk on key splits: full-size GPU run")
    out = da.fwd_kv(c(pf.q[rows]), c(pf.k), c(pf.v), *lv, da.lambda_init(wl.depth),
                    c(pf.w), wl.eps, True, nseq=1)
    torch.cuda.synchronize()
    pick = np.array(sorted(set(range(0, n, 8)) | set(range(64)) | set(range(n - 64, n))),
                    np.int64)
    toks = rows.numpy()[pick]
    rows_t = np.repeat(toks, H)
    rows_h = np.tile(np.arange(H, dtype=np.int32), toks.size)
    ref = oracle.rows(pf.q, pf.k, pf.v, pf.lq1, pf.lk1, pf.lq2, pf.lk2,
                      oracle.lambda_init(wl.depth), rows_t, rows_h, pf.w, wl.eps, True,
                      pf.cu_seqlens)
    got = out[torch.from_numpy(np.repeat(pick, H)).to(DEV),
              torch.from_numpy(rows_h).long().to(DEV)]
    err = max_abs(got, ref)
    announce(f"1 x (1024 vs 32768): {rows_t.size} rows, max-abs {err:.3e}")
    assert err <= TOL
