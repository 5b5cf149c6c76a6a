"""Parity of the key/value-cache path (diffattn_fwd_kv, through the C ABI)
with the fp64 oracle's ``fwd_kv``.

Tolerance: bf16 storage, max-abs 2e-2 over every compared element (outputs
upcast to fp64).  All tests need an MI355X.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import KV_WORKLOADS, custom_kv, make_kv_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _da():
    import differential_attention_amd as da
    return da


def announce(msg):
    print(f"[parity-kv] {msg}", flush=True)


def gpu_kv(inp, lam=None, out=None, workspace=None, stream=None, uniform=False):
    da = _da()
    dev = torch.device("cuda:0")
    c = lambda t: t.to(dev).contiguous()
    lv = [c(x) for x in (lam if lam is not None else
                         (inp.lq1, inp.lk1, inp.lq2, inp.lk2))]
    kw = {}
    if uniform:
        kw["nseq"] = inp.cu_q.numel() - 1
    else:
        kw.update(cu_seqlens_q=c(inp.cu_q), cu_seqlens_k=c(inp.cu_k),
                  max_seqlen_q=inp.max_q, max_seqlen_k=inp.max_k)
    res = da.fwd_kv(c(inp.q), c(inp.k), c(inp.v), *lv,
                    da.lambda_init(inp.depth), c(inp.w), inp.eps, inp.causal,
                    workspace=workspace, out=out, stream=stream, **kw)
    torch.cuda.synchronize()
    return res


def oracle_kv(inp, lam=None, seqs=None):
    lv = lam if lam is not None else (inp.lq1, inp.lk1, inp.lq2, inp.lk2)
    cq, ck = inp.cu_q.numpy(), inp.cu_k.numpy()
    if seqs is None:
        return oracle.fwd_kv(inp.q, inp.k, inp.v, *lv,
                             oracle.lambda_init(inp.depth), inp.w, inp.eps,
                             inp.causal, cq, ck)
    # a subset of the sequences, each computed on its own slice
    outs = []
    for s in seqs:
        qa, qb, ka, kb = int(cq[s]), int(cq[s + 1]), int(ck[s]), int(ck[s + 1])
        outs.append(oracle.fwd_kv(inp.q[qa:qb], inp.k[ka:kb], inp.v[ka:kb],
                                  *lv, oracle.lambda_init(inp.depth), inp.w,
                                  inp.eps, inp.causal, [0, qb - qa],
                                  [0, kb - ka]))
    return outs


def max_abs(gpu_out, ref):
    got = gpu_out.float().cpu().double().numpy()
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    return float(np.max(np.abs(got - ref))) if ref.size else 0.0


# ---------------------------------------------------------------------------
# the three cache workloads

@pytest.mark.parametrize("name", ["decode_b8_kv4097", "decode_b64_kv8192"])
def test_decode_workloads_full(name):
    wl = KV_WORKLOADS[name]
    announce(f"{name}: full output vs oracle")
    inp = make_kv_inputs(wl)
    out = gpu_kv(inp)
    err = max_abs(out, oracle_kv(inp))
    announce(f"{name}: max-abs {err:.3e}")
    assert err <= TOL


def test_decode_varlen_sampled_sequences():
    wl = KV_WORKLOADS["decode_varlen_b32_q4"]
    inp = make_kv_inputs(wl)
    out = gpu_kv(inp)
    lens = np.asarray(wl.k_lens)
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 7, 19,
                   wl.nseq - 1})
    announce(f"decode_varlen_b32_q4: sequences {seqs} vs oracle")
    refs = oracle_kv(inp, seqs=seqs)
    cq = wl.cu_q()
    err = 0.0
    for s, ref in zip(seqs, refs):
        err = max(err, max_abs(out[int(cq[s]):int(cq[s + 1])], ref))
    announce(f"decode_varlen_b32_q4: max-abs {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("name", sorted(KV_WORKLOADS))
def test_decode_workloads_uniform_closed_form(name):
    """K = 0 makes both maps uniform over the visible keys: row i of a
    sequence is RMSNorm((1 - lambda) * mean of V over keys 0 .. nk - nq + i),
    computable for every row by prefix sums."""
    wl = KV_WORKLOADS[name]
    announce(f"{name}: K=0 closed form on every row")
    inp = make_kv_inputs(wl)
    inp.k.zero_()
    out = gpu_kv(inp).float().cpu().numpy()
    lam_init = oracle.lambda_init(wl.depth)
    lam = oracle.lam(inp.lq1, inp.lk1, inp.lq2, inp.lk2, lam_init)
    v = inp.v.float().numpy().astype(np.float64)
    cq, ck = wl.cu_q(), wl.cu_k()
    G = wl.H // wl.Hkv
    err = 0.0
    for s in range(wl.nseq):
        nq, nk = int(cq[s + 1] - cq[s]), int(ck[s + 1] - ck[s])
        pref = np.cumsum(v[int(ck[s]):int(ck[s + 1])], axis=0)
        for i in range(nq):
            cnt = nk - nq + i + 1
            pre = (1.0 - lam) * pref[cnt - 1] / cnt            # [Hkv, 2d]
            ref = (pre / np.sqrt(np.mean(pre * pre, axis=1, keepdims=True) + wl.eps)
                   * (1.0 - lam_init))
            got = out[int(cq[s]) + i].reshape(wl.Hkv, G, -1)
            err = max(err, float(np.max(np.abs(got - ref[:, None, :]))))
    announce(f"{name}: max-abs {err:.3e}")
    assert err <= TOL


# ---------------------------------------------------------------------------
# shapes, masks and edge cases at sizes the oracle finishes in seconds

RAGGED = [
    # query lengths, key lengths (ragged tails, splits, masks)
    ((1, 3, 5, 16, 2), (37, 100, 250, 600, 2)),
    ((1, 1, 1), (1, 31, 33)),
    ((8, 0, 4), (8, 50, 4)),            # nq == nk (a prefill); an empty query set
]


@pytest.mark.parametrize("H,Hkv", [(8, 2), (4, 4), (16, 1), (12, 4), (10, 5)])
@pytest.mark.parametrize("d", [64, 32])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("case", range(len(RAGGED)))
def test_ragged_matrix(H, Hkv, d, causal, case):
    ql, kl = RAGGED[case]
    wl = custom_kv("ragged", "bf16", ql, kl, H=H, Hkv=Hkv, d=d, depth=5,
                   causal=causal, seed=100 + case)
    inp = make_kv_inputs(wl)
    inp.w.copy_(0.5 + torch.rand(2 * d, generator=torch.Generator().manual_seed(case)))
    out = gpu_kv(inp)
    err = max_abs(out, oracle_kv(inp))
    announce(f"ragged case {case} H={H} Hkv={Hkv} d={d} causal={causal}: "
             f"max-abs {err:.3e}")
    assert err <= TOL


def test_many_sequences_split_scan():
    """More than 64 sequences, with empty ones, uneven caches and a total
    large enough for splits longer than the minimum: every sequence's
    splits are found by the kernels' scan of cu_seqlens_k across several
    64-sequence steps."""
    rng = np.random.default_rng(21)
    nseq = 150
    kl = [int(x) for x in rng.integers(1, 6000, nseq)]
    ql = [int(x) for x in rng.integers(1, 4, nseq)]
    for s in (0, 63, 64, 100):       # empty sequences, on and off step edges
        ql[s], kl[s] = 0, 0
    ql[70] = 0                       # no query, keys only
    wl = custom_kv("many", "bf16", tuple(ql), tuple(kl), H=8, Hkv=2, d=64,
                   depth=4, seed=21)
    inp = make_kv_inputs(wl)
    err = max_abs(gpu_kv(inp), oracle_kv(inp))
    announce(f"many sequences (Tk={sum(kl)}): max-abs {err:.3e}")
    assert err <= TOL


def test_one_split_per_sequence():
    """More sequences x KV heads than the split plan's wave budget (300 x 4
    against 1024): every sequence becomes a single split of the longest
    cache's length, whatever its own length, including empty ones."""
    rng = np.random.default_rng(31)
    nseq = 300
    kl = [int(x) for x in rng.integers(1, 400, nseq)]
    ql = [int(x) for x in rng.integers(1, 3, nseq)]
    for s in (5, 64, 299):
        ql[s], kl[s] = 0, 0
    wl = custom_kv("one_split", "bf16", tuple(ql), tuple(kl), H=8, Hkv=4, d=64,
                   depth=5, seed=31)
    inp = make_kv_inputs(wl)
    err = max_abs(gpu_kv(inp), oracle_kv(inp))
    announce(f"one split per sequence (Tk={sum(kl)}): max-abs {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("d", [64, 32])
def test_long_cache_many_splits(d):
    """One long sequence with several new queries: many key splits per row
    block (over a hundred: the combine kernel's widest grouping, several
    rounds per thread), and the causal limit inside the last split."""
    wl = custom_kv("long", "bf16", (7,), (20000,), H=16, Hkv=4, d=d, depth=3,
                   seed=7)
    inp = make_kv_inputs(wl)
    err = max_abs(gpu_kv(inp), oracle_kv(inp))
    announce(f"long cache d={d}: max-abs {err:.3e}")
    assert err <= TOL


def test_large_logits():
    """Scores far beyond exp()'s range: the lazily raised maximum and the
    log-sum-exp merge across splits must stay finite and exact."""
    wl = custom_kv("big", "bf16", (1, 4), (3000, 5000), H=8, Hkv=2, d=64,
                   depth=2, seed=3)
    inp = make_kv_inputs(wl, q_scale=30.0)
    err = max_abs(gpu_kv(inp), oracle_kv(inp))
    announce(f"large logits: max-abs {err:.3e}")
    assert err <= TOL


def test_per_head_lambda():
    wl = custom_kv("ph", "bf16", (1, 2, 3), (300, 70, 1000), H=8, Hkv=2, d=64,
                   depth=4, seed=11)
    inp = make_kv_inputs(wl)
    g = torch.Generator().manual_seed(12)
    lam = [0.2 * torch.randn(wl.H, wl.d, generator=g) for _ in range(4)]
    err = max_abs(gpu_kv(inp, lam=lam), oracle_kv(inp, lam=lam))
    announce(f"per-head lambda: max-abs {err:.3e}")
    assert err <= TOL


def test_uniform_lengths_without_boundaries():
    wl = custom_kv("uni", "bf16", (2,) * 5, (700,) * 5, H=16, Hkv=4, d=64,
                   depth=6, seed=13)
    inp = make_kv_inputs(wl)
    a = gpu_kv(inp, uniform=True)
    b = gpu_kv(inp)
    assert torch.equal(a, b)
    err = max_abs(a, oracle_kv(inp))
    announce(f"uniform lengths: max-abs {err:.3e}")
    assert err <= TOL


def test_decode_of_last_token_matches_prefill_row():
    """The last query of a causal prefill and the same query decoded against
    the whole sequence as cache are the same row of the method."""
    da = _da()
    from workloads import custom, make_inputs
    wl = custom("pf", "bf16", (900,), H=16, Hkv=4, d=64, depth=8, seed=21)
    pf = make_inputs(wl)
    dev = torch.device("cuda:0")
    c = lambda t: t.to(dev).contiguous()
    lv = [c(x) for x in (pf.lq1, pf.lk1, pf.lq2, pf.lk2)]
    full = da.fwd(c(pf.q), c(pf.k), c(pf.v), *lv, da.lambda_init(8), c(pf.w),
                  1e-5, True, c(pf.cu_seqlens), max_seqlen=900)
    last = da.fwd_kv(c(pf.q[-1:]), c(pf.k), c(pf.v), *lv, da.lambda_init(8),
                     c(pf.w), 1e-5, True, nseq=1)
    torch.cuda.synchronize()
    ref = oracle.fwd(pf.q, pf.k, pf.v, pf.lq1, pf.lk1, pf.lq2, pf.lk2,
                     oracle.lambda_init(8), pf.w, 1e-5, True,
                     pf.cu_seqlens)[-1:]
    e1, e2 = max_abs(full[-1:], ref), max_abs(last, ref)
    announce(f"last token: prefill {e1:.3e}, decode {e2:.3e}")
    assert e1 <= TOL and e2 <= TOL


def test_deterministic_and_workspace_reuse():
    """Bitwise equal on repeated calls; the workspace needs no clearing
    between calls of different sizes, and a smaller call leaves rows past
    its output untouched."""
    da = _da()
    big = custom_kv("a", "bf16", (3, 1), (4000, 2500), H=16, Hkv=4, d=64,
                    depth=8, seed=31)
    small = custom_kv("b", "bf16", (1,), (333,), H=16, Hkv=4, d=64, depth=8,
                      seed=32)
    ib, ism = make_kv_inputs(big), make_kv_inputs(small)
    need = da.kv_workspace_size(2, 3, 4000, 16, 4, 64)
    ws = torch.full((need,), 0x7f, dtype=torch.uint8, device="cuda:0")
    a1 = gpu_kv(ib, workspace=ws)
    s1 = gpu_kv(ism, workspace=ws)
    a2 = gpu_kv(ib, workspace=ws)
    assert torch.equal(a1, a2)
    assert max_abs(s1, oracle_kv(ism)) <= TOL
    assert max_abs(a1, oracle_kv(ib)) <= TOL
    # the canary around a provided output survives
    out = torch.full((ism.q.shape[0] + 2, 16, 128), 7.0, dtype=torch.bfloat16,
                     device="cuda:0")
    gpu_kv(ism, out=out[1:-1], workspace=ws)
    assert torch.all(out[0] == 7.0) and torch.all(out[-1] == 7.0)
    assert torch.equal(out[1:-1], s1)


def test_small_workspace_rejected():
    da = _da()
    wl = custom_kv("w", "bf16", (1,), (500,), H=16, Hkv=4, d=64, seed=41)
    inp = make_kv_inputs(wl)
    ws = torch.empty(64, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(da.DiffAttnError):
        gpu_kv(inp, workspace=ws)


def test_stream_argument():
    wl = custom_kv("st", "bf16", (2, 1), (600, 900), H=16, Hkv=4, d=64, seed=51)
    inp = make_kv_inputs(wl)
    st = torch.cuda.Stream()
    a = gpu_kv(inp, stream=st)
    b = gpu_kv(inp)
    assert torch.equal(a, b)


def test_more_queries_than_keys_noncausal():
    wl = custom_kv("nc", "bf16", (5, 40), (2, 3), H=8, Hkv=2, d=64,
                   causal=False, seed=61)
    inp = make_kv_inputs(wl)
    err = max_abs(gpu_kv(inp), oracle_kv(inp))
    announce(f"nq > nk, non-causal: max-abs {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("i", range(12))
def test_random_shapes(i):
    """Seeded random cache shapes: sequence counts, query and cache lengths
    (empty sequences included), head groupings, d, masking, shared or
    per-head lambda."""
    rng = np.random.default_rng(4000 + i)
    nseq = int(rng.integers(1, 9))
    d = int(rng.choice([32, 64]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4, 8]))
    causal = bool(rng.integers(0, 2))
    ql = [int(x) for x in rng.integers(0, 6, nseq)]
    kl = [int(x) for x in rng.integers(1, 3000, nseq)]
    kl = [max(k, q) if causal else k for q, k in zip(ql, kl)]
    if sum(ql) == 0:
        ql[0] = 1
    wl = custom_kv("random", "bf16", tuple(ql), tuple(kl), H=Hkv * G, Hkv=Hkv, d=d,
                   depth=1 + i, causal=causal, seed=5000 + i)
    inp = make_kv_inputs(wl)
    lam = None
    if rng.integers(0, 2):
        g = torch.Generator().manual_seed(6000 + i)
        lam = [0.2 * torch.randn(Hkv * G, d, generator=g) for _ in range(4)]
    err = max_abs(gpu_kv(inp, lam=lam), oracle_kv(inp, lam=lam))
    announce(f"random case {i}: q {ql} k {kl} H={Hkv * G} Hkv={Hkv} d={d} "
             f"causal={causal} per-head={lam is not None}: max-abs {err:.3e}")
    assert err <= TOL
