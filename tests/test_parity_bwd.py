"""Parity of the backward pass (diffattn_fwd_train + diffattn_bwd, through
the C ABI) with the fp64 oracle's ``bwd``.

Gradients have very different scales from tensor to tensor, so the bar is
relative: max|got - ref| <= 2e-2 * max|ref| for dq, dk, dv and dw -- the
forward's 2e-2 on O(1) outputs; dq, dk and dv come from contractions with
bf16 operands (P, dS, dO_m) and are stored in bf16.  The lambda-vector
gradients are dlambda times a vector, and dlambda = -sum over rows of
<dpre, O_2> can cancel to far below its terms, each of which carries the
forward's bf16 rounding of P; their error is bounded instead by 2^-7 (two
bf16 roundings) times the oracle's sum over rows of |dpre| |O_2|, times the
vector factor.

fp32 storage (and bf16 at d = 16) runs the exact kernels, fp32 throughout:
with fp32 inputs every gradient, the lambda-vector ones included, is held
to 2e-5 of the same scales (fp32 sums over at most a few thousand terms sit
near 1e-6).  Every bf16 random case also runs as an fp32 twin (the same
values in fp32 storage) against that bar, which shows the bf16 cases' error
is the operand rounding and not a slip of the arithmetic.  All tests need an
MI355X.
"""

import numpy as np
import pytest
import torch

import oracle
from conditioning import key_factors, row_factors
from launch_shape import prefill_sub_blocks
from workloads import WORKLOADS, custom, make_inputs

pytestmark = pytest.mark.gpu

REL = {"dq": 2e-2, "dk": 2e-2, "dv": 2e-2, "dlq1": 2.0 ** -7, "dlk1": 2.0 ** -7,
       "dlq2": 2.0 ** -7, "dlk2": 2.0 ** -7, "dw": 2e-2}
REL32 = {name: 2e-5 for name in REL}


def fp32_twin(inp, dy):
    """The same input values in fp32 storage (bf16 -> fp32 is exact)."""
    import copy
    twin = copy.copy(inp)
    twin.q, twin.k, twin.v = inp.q.float(), inp.k.float(), inp.v.float()
    return twin, dy.float()


def announce(msg):
    print(f"[parity-bwd] {msg}", flush=True)


def dout_for(inp, seed):
    g = torch.Generator().manual_seed(seed)
    T, H, _, d = inp.q.shape
    return torch.randn(T, H, 2 * d, generator=g).to(inp.q.dtype)


def gpu_grads(inp, dy, w=True, repeat=1):
    import differential_attention_amd as da
    dev = torch.device("cuda:0")
    c = lambda t: t.to(dev).contiguous()
    lv = [c(x) for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
    wt = c(inp.w) if w else None
    kw = dict(subln_weight=wt, eps=inp.eps, causal=inp.causal,
              cu_seqlens=c(inp.cu_seqlens), max_seqlen=inp.max_seqlen)
    q, k, v = c(inp.q), c(inp.k), c(inp.v)
    lam0 = da.lambda_init(inp.depth)
    out, lse, o12 = da.fwd_train(q, k, v, *lv, lam0, **kw)
    res = [da.bwd(q, k, v, *lv, lam0, c(dy), lse, o12, **kw) for _ in range(repeat)]
    torch.cuda.synchronize()
    return out, res


def oracle_grads(inp, dy, w=True):
    return oracle.bwd(inp.q, inp.k, inp.v, inp.lq1, inp.lk1, inp.lq2, inp.lk2,
                      oracle.lambda_init(inp.depth), dy, inp.w if w else None,
                      inp.eps, inp.causal, inp.cu_seqlens)


def conditioning_factors(inp):
    """Bar multipliers of dq ([T, H], per output row) and of dk, dv ([T,
    Hkv], per key): a row whose two maps cancel before the RMSNorm
    (cancellation ratio r below 0.2) amplifies the bf16 rounding of P that
    the training forward's saved O_m carry, once in pre and again through
    the RMSNorm backward, by about 1 / r.  Its dq row gets 0.2 / r (at most
    4x), and so does every key it sees in dk and dv; rows that see a single
    key (P exactly 1) keep the plain bar."""
    rf = row_factors(inp)
    return rf, key_factors(inp, rf)


def compare(got, ref, tag, inp=None, rel=REL):
    """dq, dk, dv, dw: max-abs relative to the tensor's largest magnitude
    (with inp given, dq, dk and dv elementwise against the bar times the
    multiplier of their row or key, conditioning_factors).
    The lambda-vector gradients all carry the factor dlambda (a sum over
    rows that can cancel), so their error is measured against the oracle's
    dlambda_scale instead: the sum over rows of |dpre| |O_2|, times the
    vector factor (e^a |lk1| for dlq1, and so on)."""
    errs = {}
    aux = ref["aux"]
    fac = conditioning_factors(inp) if inp is not None else None
    widened = 0
    for name, r in ref.items():
        if name == "aux":
            continue
        gv = got[name].float().cpu().double().numpy()
        assert np.all(np.isfinite(gv)), f"{tag}: non-finite {name}"
        if name.startswith("dl"):
            # |d vector| = |dlambda| * |factor|: bound it by scale * |factor|
            dl = aux["dlam_head"].sum() if r.ndim == 1 else aux["dlam_head"][:, None]
            sc = aux["dlam_scale"].sum() if r.ndim == 1 else aux["dlam_scale"][:, None]
            factor = np.abs(r) / np.maximum(np.abs(dl), 1e-300)
            bound = sc * factor + 1e-30
            errs[name] = float(np.max(np.abs(gv - r) / bound))
        else:
            scale = max(float(np.max(np.abs(r))), 1e-30)
            e = np.abs(gv - r)
            if fac is not None and name in ("dq", "dk", "dv"):
                f = fac[0] if name == "dq" else fac[1]           # [T, heads]
                # elements beyond the plain bar are the ones the wider bar admits
                widened += int(np.sum(e > rel[name] * scale))
                e = e / f.reshape(f.shape + (1,) * (e.ndim - 2))
            errs[name] = float(np.max(e)) / scale
    announce(f"{tag}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()) +
             (f"; {widened} elements past the plain bar" if widened else ""))
    for name, err in errs.items():
        assert err <= rel[name], f"{tag}: {name} relative max-abs {err:.3e}"
    return max(errs[n] / rel[n] for n in errs)


RAGGED = (1, 0, 31, 32, 33, 63, 64, 65, 127, 200, 7)


@pytest.mark.parametrize("d", [64, 32])
@pytest.mark.parametrize("H,Hkv", [(4, 2), (8, 2), (3, 1), (16, 4), (10, 5), (8, 8)])
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_ragged(d, H, Hkv, causal):
    wl = custom("bwd", "bf16", RAGGED, H, Hkv, d, depth=6, causal=causal,
                seed=H * 10 + d)
    inp = make_inputs(wl)
    inp.w = torch.linspace(0.5, 1.5, 2 * d)
    dy = dout_for(inp, 7)
    _, (got,) = gpu_grads(inp, dy)
    worst = compare(got, oracle_grads(inp, dy), f"d={d} H={H} Hkv={Hkv} causal={causal}")
    announce(f"ragged d={d} H={H} Hkv={Hkv} causal={causal}: worst err / bar {worst:.3f}")


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 32), ("f32", 32), ("bf16", 16)])
def test_bwd_ragged_64_query_slots(dtype, d):
    """Many short sequences: the training forward on its 64-query
    instantiation, then the backward."""
    lens = RAGGED * 11
    assert prefill_sub_blocks(16, 4, len(lens), max(lens), sum(lens)) == 2
    wl = custom("bwd_many", dtype, lens, 16, 4, d, depth=4, causal=True, seed=d + 90)
    inp = make_inputs(wl)
    inp.w = torch.linspace(0.5, 1.5, 2 * d)
    dy = dout_for(inp, 27)
    _, (got,) = gpu_grads(inp, dy)
    tag = f"ragged x11 {dtype} d={d}"
    worst = compare(got, oracle_grads(inp, dy), tag, inp=inp,
                    rel=REL32 if dtype == "f32" else REL)
    announce(f"{tag}: worst err / bar {worst:.3f}")


# the exact kernels: fp32 storage at every d, bf16 at d = 16
@pytest.mark.parametrize("dtype,d", [("f32", 16), ("f32", 32), ("f32", 64), ("bf16", 16)])
@pytest.mark.parametrize("H,Hkv", [(4, 2), (3, 1), (10, 5), (8, 8)])
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_exact_path_ragged(dtype, d, H, Hkv, causal):
    wl = custom("bwd_exact", dtype, RAGGED, H, Hkv, d, depth=5, causal=causal,
                seed=H * 10 + d + 1)
    inp = make_inputs(wl)
    inp.w = torch.linspace(0.5, 1.5, 2 * d)
    dy = dout_for(inp, 17)
    _, (got,) = gpu_grads(inp, dy)
    tag = f"exact {dtype} d={d} H={H} Hkv={Hkv} causal={causal}"
    worst = compare(got, oracle_grads(inp, dy), tag, inp=inp,
                    rel=REL32 if dtype == "f32" else REL)
    announce(f"{tag}: worst err / bar {worst:.3f}")


@pytest.mark.parametrize("i", range(8))
def test_bwd_exact_path_random(i):
    """Seeded random shapes on the exact kernels, per-head lambda in half of
    them, longer sequences than the ragged matrix (up to 1500 keys)."""
    rng = np.random.default_rng(7500 + i)
    dtype, d = [("f32", 64), ("f32", 32), ("f32", 16), ("bf16", 16)][i % 4]
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4]))
    lens = tuple(int(x) for x in rng.integers(0, 1500, int(rng.integers(1, 4))))
    if sum(lens) == 0:
        lens = lens + (9,)
    causal = bool(rng.integers(0, 2))
    wl = custom("bwd_exact_random", dtype, lens, Hkv * G, Hkv, d, depth=3 + i,
                causal=causal, seed=8500 + i)
    inp = make_inputs(wl)
    if rng.integers(0, 2):
        g = torch.Generator().manual_seed(9500 + i)
        inp.lq1, inp.lk1, inp.lq2, inp.lk2 = [0.3 * torch.randn(Hkv * G, d, generator=g)
                                              for _ in range(4)]
    dy = dout_for(inp, 40 + i)
    _, (got,) = gpu_grads(inp, dy)
    tag = f"exact random {i}: {dtype} lens {lens} H={Hkv * G} Hkv={Hkv} d={d} causal={causal}"
    worst = compare(got, oracle_grads(inp, dy), tag, inp=inp,
                    rel=REL32 if dtype == "f32" else REL)
    announce(f"{tag}: worst err / bar {worst:.3f}")


def test_bwd_embed2048_full():
    """The pull request's test shape (B=2, N=512, 16 heads, 4 KV heads) in
    full: several query and key tiles per sequence."""
    inp = make_inputs(WORKLOADS["embed2048_b2_n512"])
    dy = dout_for(inp, 11)
    out, (got,) = gpu_grads(inp, dy)
    worst = compare(got, oracle_grads(inp, dy), "embed2048")
    announce(f"embed2048: worst err / bar {worst:.3f}")


def test_bwd_long_sequences():
    """8 sequences of 1024 tokens (8 tiles each way), GQA 4."""
    wl = custom("bwd_long", "bf16", (1024,) * 8, 16, 4, 64, depth=8, seed=12)
    inp = make_inputs(wl)
    dy = dout_for(inp, 13)
    _, (got,) = gpu_grads(inp, dy)
    worst = compare(got, oracle_grads(inp, dy), "8 x 1024")
    announce(f"8 x 1024: worst err / bar {worst:.3f}")


def test_bwd_per_head_lambda_no_weight():
    wl = custom("bwd_ph", "bf16", (150, 90), 8, 2, 64, depth=4, seed=14)
    inp = make_inputs(wl)
    g = torch.Generator().manual_seed(15)
    inp.lq1, inp.lk1, inp.lq2, inp.lk2 = [0.3 * torch.randn(8, 64, generator=g)
                                          for _ in range(4)]
    dy = dout_for(inp, 16)
    _, (got,) = gpu_grads(inp, dy, w=False)
    worst = compare(got, oracle_grads(inp, dy, w=False), "per-head lambda")
    announce(f"per-head lambda, no weight: worst err / bar {worst:.3f}")


def test_training_forward_matches_forward():
    """The training forward's output equals the plain forward bitwise, and
    its saved state reproduces the output: RMSNorm(O_1 - lambda O_2)."""
    import differential_attention_amd as da
    wl = custom("train", "bf16", (300, 41), 16, 4, 64, depth=8, seed=17)
    inp = make_inputs(wl)
    dev = torch.device("cuda:0")
    c = lambda t: t.to(dev).contiguous()
    lv = [c(x) for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
    lam0 = da.lambda_init(8)
    out, lse, o12 = da.fwd_train(c(inp.q), c(inp.k), c(inp.v), *lv, lam0, c(inp.w),
                                 1e-5, True, c(inp.cu_seqlens), max_seqlen=300)
    plain = da.fwd(c(inp.q), c(inp.k), c(inp.v), *lv, lam0, c(inp.w), 1e-5, True,
                   c(inp.cu_seqlens), max_seqlen=300)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    lam = oracle.lam(inp.lq1, inp.lk1, inp.lq2, inp.lk2, lam0)
    o = o12.double().cpu()
    pre = o[:, :, 0] - lam * o[:, :, 1]
    y = pre / torch.sqrt((pre * pre).mean(-1, keepdim=True) + 1e-5) * (1 - lam0)
    assert float((y - out.double().cpu()).abs().max()) < 2e-2
    assert torch.all(torch.isfinite(lse))


def test_bwd_deterministic():
    wl = custom("bwd_det", "bf16", (333, 128, 5), 16, 4, 64, depth=3, seed=18)
    inp = make_inputs(wl)
    dy = dout_for(inp, 19)
    _, (a, b) = gpu_grads(inp, dy, repeat=2)
    for name in a:
        assert torch.equal(a[name], b[name]), name


def test_bwd_small_workspace_rejected():
    import differential_attention_amd as da
    wl = custom("bwd_ws", "bf16", (64,), 4, 2, 64, seed=20)
    inp = make_inputs(wl)
    dev = torch.device("cuda:0")
    c = lambda t: t.to(dev).contiguous()
    lv = [c(x) for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
    out, lse, o12 = da.fwd_train(c(inp.q), c(inp.k), c(inp.v), *lv, 0.3)
    with pytest.raises(da.DiffAttnError):
        da.bwd(c(inp.q), c(inp.k), c(inp.v), *lv, 0.3, torch.zeros_like(out), lse,
               o12, workspace=torch.empty(256, dtype=torch.uint8, device=dev))


def _tile_rows(starts, width, heads):
    t = np.concatenate([np.arange(a, a + width) for a in starts]).astype(np.int64)
    return np.repeat(t, heads), np.tile(np.arange(heads, dtype=np.int32), t.size)


@pytest.mark.parametrize("name", ["llama1b_b8_n4096", "long_b1_n32768"])
def test_bwd_full_size_sampled(name):
    """The benchmark's training-step configuration at full size: dq of whole
    128-row query tiles (every head) and dk, dv of whole 128-key tiles
    (every KV head) against the oracle's sampling entry (which recomputes
    every row that can see a sampled key).  8 x 4096: query and key tiles
    at the start, the middle and the end of every sequence.  One 32768-token
    sequence: query tiles at the start, middle and end; key tiles near the
    end only (a key at position j needs all 32768 - j rows that see it, so
    early keys would cost the oracle the whole backward of the sequence).
    Bar: 2e-2 of the sample's largest magnitude per tensor."""
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    gen = torch.Generator().manual_seed(1)
    dy = torch.randn(wl.T, wl.H, 2 * wl.d, generator=gen).to(torch.bfloat16)
    _, (got,) = gpu_grads(inp, dy)
    n = wl.max_seqlen
    qst = [s * n + o for s in range(wl.nseq) for o in (0, n // 2 - 64, n - 128)]
    if wl.nseq > 1:
        kst = qst
    else:
        kst = [n - 1024, n - 128]
    tq, hq = _tile_rows(qst, 128, wl.H)
    tk, gk = _tile_rows(kst, 128, wl.Hkv)
    announce(f"{name}: full-size backward, {tq.size} dq rows, {tk.size} dk/dv keys")
    ref = oracle.bwd_sample(inp.q, inp.k, inp.v, inp.lq1, inp.lk1, inp.lq2, inp.lk2,
                            oracle.lambda_init(wl.depth), dy, (tq, hq), (tk, gk),
                            inp.w, inp.eps, inp.causal, inp.cu_seqlens)
    dev_idx = lambda a: torch.from_numpy(np.asarray(a, np.int64)).cuda()
    sel = {"dq": got["dq"][dev_idx(tq), dev_idx(hq)],
           "dk": got["dk"][dev_idx(tk), dev_idx(gk)],
           "dv": got["dv"][dev_idx(tk), dev_idx(gk)]}
    errs = {}
    for key in ("dq", "dk", "dv"):
        gv = sel[key].float().cpu().double().numpy()
        assert np.all(np.isfinite(gv))
        errs[key] = float(np.max(np.abs(gv - ref[key]))) / float(np.max(np.abs(ref[key])))
    announce(f"{name}: " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for key, e in errs.items():
        assert e <= 2e-2, f"{name}: {key} relative max-abs {e:.3e}"


# 74, 83 and 156 each hold a row whose maps cancel (the second or third
# token of a sequence), held to the conditioning-scaled bar
@pytest.mark.parametrize("i", list(range(24)) + [74, 83, 156])
def test_bwd_random_shapes(i):
    """Seeded random shapes for the backward: sequence mixes, head
    groupings, d, masking, per-head lambda with or without the weight."""
    rng = np.random.default_rng(7000 + i)
    d = int(rng.choice([32, 64]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4]))
    lens = tuple(int(x) for x in rng.integers(0, 400, int(rng.integers(1, 5))))
    if sum(lens) == 0:
        lens = lens + (9,)
    causal = bool(rng.integers(0, 2))
    wl = custom("bwd_random", "bf16", lens, Hkv * G, Hkv, d, depth=2 + i, causal=causal,
                seed=8000 + i)
    inp = make_inputs(wl)
    use_w = bool(rng.integers(0, 2))
    if use_w:
        inp.w = torch.from_numpy(rng.uniform(0.5, 1.5, 2 * d)).float()
    if rng.integers(0, 2):
        g = torch.Generator().manual_seed(9000 + i)
        inp.lq1, inp.lk1, inp.lq2, inp.lk2 = [0.3 * torch.randn(Hkv * G, d, generator=g)
                                              for _ in range(4)]
    dy = dout_for(inp, 10 + i)
    _, (got,) = gpu_grads(inp, dy, w=use_w)
    ref = oracle_grads(inp, dy, w=use_w)
    tag = f"random {i}: lens {lens} H={Hkv * G} Hkv={Hkv} d={d} causal={causal}"
    worst = compare(got, ref, tag, inp=inp)
    announce(f"random case {i}: worst err / bar {worst:.3f}")
    twin, dy32 = fp32_twin(inp, dy)
    _, (got32,) = gpu_grads(twin, dy32, w=use_w)
    worst32 = compare(got32, ref, "fp32 twin of " + tag, inp=twin, rel=REL32)
    announce(f"random case {i}, fp32 twin: worst err / bar {worst32:.3f}")


@pytest.mark.parametrize("w", [True, False])
def test_autograd_function_matches_the_raw_calls(w):
    """diff_attention under autograd: its output is the training forward's
    and its gradients are diffattn_bwd's, bitwise."""
    import differential_attention_amd as da
    wl = custom("autograd", "bf16", (300, 65, 129), 8, 2, 64, depth=5, seed=71)
    inp = make_inputs(wl)
    dev = torch.device("cuda:0")
    c = lambda t: t.to(dev).contiguous()
    q, k, v = (c(x).requires_grad_() for x in (inp.q, inp.k, inp.v))
    lv = [c(x).requires_grad_() for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
    wt = c(inp.w).requires_grad_() if w else None
    lam0 = da.lambda_init(wl.depth)
    kw = dict(subln_weight=wt, eps=wl.eps, causal=True, cu_seqlens=c(inp.cu_seqlens),
              max_seqlen=wl.max_seqlen)
    out = da.diff_attention(q, k, v, *lv, lam0, **kw)
    dy = c(dout_for(inp, 72))
    out.backward(dy)
    torch.cuda.synchronize()
    with torch.no_grad():
        raw = [x.detach() for x in (q, k, v, *lv)]
        kw2 = dict(kw, subln_weight=None if wt is None else wt.detach())
        ref_out, lse, o12 = da.fwd_train(*raw, lam0, **kw2)
        g = da.bwd(*raw, lam0, dy, lse, o12, **kw2)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), ref_out)
    for name, t in zip(("dq", "dk", "dv", "dlq1", "dlk1", "dlq2", "dlk2"), (q, k, v, *lv)):
        assert torch.equal(t.grad, g[name]), name
    if w:
        assert torch.equal(wt.grad, g["dw"])
    announce(f"autograd (weight {w}): output and gradients equal the raw calls")
