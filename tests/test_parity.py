"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances (max-abs over every compared element, outputs upcast to fp64):
fp32 storage 1e-4, bf16 storage 2e-2.  All tests need an MI355X.
"""

import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from conditioning import rows_within_bar
from launch_shape import compact_list, prefill_sub_blocks
from workloads import WORKLOADS, custom, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _da():
    import differential_attention_amd as da
    return da


def gpu_run(inp, out=None, stream=None, causal=None, max_seqlen=None):
    da = _da()
    dev = torch.device("cuda:0")
    c = lambda t: t.to(dev).contiguous()
    res = da.fwd(c(inp.q), c(inp.k), c(inp.v), c(inp.lq1), c(inp.lk1),
                 c(inp.lq2), c(inp.lk2), da.lambda_init(inp.depth),
                 c(inp.w), inp.eps, inp.causal if causal is None else causal,
                 c(inp.cu_seqlens),
                 max_seqlen=inp.max_seqlen if max_seqlen is None else max_seqlen,
                 out=out, stream=stream)
    torch.cuda.synchronize()
    return res


def oracle_full(inp):
    return oracle.fwd(inp.q, inp.k, inp.v, inp.lq1, inp.lk1, inp.lq2, inp.lk2,
                      oracle.lambda_init(inp.depth), inp.w, inp.eps,
                      inp.causal, inp.cu_seqlens)


def oracle_rows(inp, toks, heads):
    return oracle.rows(inp.q, inp.k, inp.v, inp.lq1, inp.lk1, inp.lq2, inp.lk2,
                       oracle.lambda_init(inp.depth), toks, heads, inp.w,
                       inp.eps, inp.causal, inp.cu_seqlens)


def max_abs(gpu_out, ref):
    got = gpu_out.float().cpu().double().numpy()
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    return float(np.max(np.abs(got - ref))) if ref.size else 0.0


def announce(msg):
    print(f"[parity] {msg}", flush=True)


# ---------------------------------------------------------------------------
# the five workloads

@pytest.mark.parametrize("name", ["tiny_f32", "embed2048_b2_n512"])
def test_small_workloads_full(name):
    wl = WORKLOADS[name]
    announce(f"{name}: full output vs oracle")
    inp = make_inputs(wl)
    out = gpu_run(inp)
    err = max_abs(out, oracle_full(inp))
    announce(f"{name}: max-abs {err:.3e}")
    assert err <= TOL[wl.dtype]


@pytest.mark.parametrize("name", ["llama1b_b8_n4096", "varlen_t65536"])
def test_large_workloads_every_row(name):
    """The benchmark's launch at full size, every output row (all tokens,
    all heads) against the oracle at the bf16 bar."""
    wl = WORKLOADS[name]
    announce(f"{name}: full-size GPU run, every row vs oracle")
    inp = make_inputs(wl)
    out = gpu_run(inp)
    err = max_abs(out, oracle_full(inp))
    announce(f"{name}: {wl.T * wl.H} rows, max-abs {err:.3e}")
    assert err <= TOL[wl.dtype]


def test_long_workload_dense_blocks_and_one_token_in_four():
    """The 32768-token sequence at full size: every head of one token in
    four, and of every token in blocks of 256 at the start, the middle and
    the end (several 64-row query tiles and 128-key tiles each), against the
    oracle at the bf16 bar."""
    wl = WORKLOADS["long_b1_n32768"]
    announce("long_b1_n32768: full-size GPU run, 1 token in 4 + dense blocks vs oracle")
    inp = make_inputs(wl)
    out = gpu_run(inp)
    n = wl.T
    toks = set(range(0, n, 4))
    for lo in (0, n // 2 - 128, n - 256):
        toks |= set(range(lo, lo + 256))
    toks = np.array(sorted(toks), np.int64)
    rows_t = np.repeat(toks, wl.H)
    rows_h = np.tile(np.arange(wl.H, dtype=np.int32), toks.size)
    ref = oracle_rows(inp, rows_t, rows_h)
    got = out[torch.from_numpy(rows_t).cuda(), torch.from_numpy(rows_h).long().cuda()]
    err = max_abs(got, ref)
    announce(f"long_b1_n32768: {rows_t.size} rows, max-abs {err:.3e}")
    assert err <= TOL[wl.dtype]


@pytest.mark.parametrize("name", ["llama1b_b8_n4096", "long_b1_n32768",
                                  "varlen_t65536"])
def test_large_workloads_uniform_closed_form(name):
    """K = 0: every map is the uniform average over the visible prefix, so
    each output row has a closed form computable for every row by prefix
    sums.  Checks every row of the full-size launch."""
    wl = WORKLOADS[name]
    announce(f"{name}: K=0 closed form on every row")
    inp = make_inputs(wl)
    inp.k.zero_()
    out = gpu_run(inp).float().cpu().numpy()
    lam_init = oracle.lambda_init(wl.depth)
    lam = oracle.lam(inp.lq1, inp.lk1, inp.lq2, inp.lk2, lam_init)
    G = wl.H // wl.Hkv
    cu = wl.cu_seqlens()
    worst = 0.0
    for s in range(wl.nseq):
        a, b = int(cu[s]), int(cu[s + 1])
        vv = inp.v[a:b].float().numpy().astype(np.float64)      # [n, Hkv, 2d]
        mean = np.cumsum(vv, axis=0) / np.arange(1, b - a + 1)[:, None, None]
        pre = (1.0 - lam) * mean
        ref = pre / np.sqrt(np.mean(pre * pre, axis=2, keepdims=True) + wl.eps)
        ref = ref * (1.0 - lam_init)
        ref = np.repeat(ref, G, axis=1)                          # [n, H, 2d]
        worst = max(worst, float(np.max(np.abs(out[a:b] - ref))))
    announce(f"{name}: max-abs {worst:.3e}")
    assert worst <= TOL[wl.dtype]


# ---------------------------------------------------------------------------
# edge cases and structure

RAGGED = (1, 0, 31, 32, 33, 63, 64, 65, 127, 200, 0, 7)


@pytest.mark.parametrize("dtype,d", [("f32", 16), ("bf16", 64), ("f32", 64),
                                     ("bf16", 16), ("bf16", 32), ("f32", 32)])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 2), (8, 2), (16, 2), (3, 1), (10, 5), (8, 8)])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged_varlen(dtype, d, H, Hkv, causal):
    wl = custom("ragged", dtype, RAGGED, H, Hkv, d, depth=5, causal=causal,
                seed=H * 100 + d)
    announce(f"ragged {dtype} d={d} H={H} Hkv={Hkv} causal={causal}")
    inp = make_inputs(wl)
    inp.w = torch.linspace(0.5, 1.5, 2 * d)
    out = gpu_run(inp)
    err = max_abs(out, oracle_full(inp))
    assert err <= TOL[dtype], f"max-abs {err:.3e}"


# Small shapes launch the 32-query instantiation (fewer than 512 workgroups
# of 64-query slots); many short ragged sequences keep the 64-query one at
# sizes the oracle finishes at once.
RAGGED_MANY = RAGGED * 11


@pytest.mark.parametrize("dtype,d", [("f32", 16), ("bf16", 64), ("f32", 64),
                                     ("bf16", 16), ("bf16", 32), ("f32", 32)])
@pytest.mark.parametrize("H,Hkv", [(4, 4), (16, 4), (6, 2)])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged_varlen_64_query_slots(dtype, d, H, Hkv, causal):
    assert prefill_sub_blocks(H, Hkv, len(RAGGED_MANY), max(RAGGED_MANY),
                              sum(RAGGED_MANY)) == 2
    wl = custom("ragged_many", dtype, RAGGED_MANY, H, Hkv, d, depth=7, causal=causal,
                seed=H * 100 + d + 1)
    announce(f"ragged x11 {dtype} d={d} H={H} Hkv={Hkv} causal={causal}")
    inp = make_inputs(wl)
    inp.w = torch.linspace(1.5, 0.5, 2 * d)
    out = gpu_run(inp)
    err = max_abs(out, oracle_full(inp))
    assert err <= TOL[dtype], f"max-abs {err:.3e}"


# Sequences long and short, a few empty: the compact tile list over more
# than 64 query-tile levels (its level search runs over several 64-lane
# chunks), on both instantiations.
COMPACT = (6000, 1, 100, 0, 3000, 70, 2049, 64, 0, 65)


@pytest.mark.parametrize("H,Hkv,sub", [(16, 4, 2), (4, 1, 1)])
def test_compact_tile_list(H, Hkv, sub):
    T = sum(COMPACT)
    assert compact_list(H, Hkv, len(COMPACT), max(COMPACT), T)
    assert prefill_sub_blocks(H, Hkv, len(COMPACT), max(COMPACT), T) == sub
    wl = custom("compact", "bf16", COMPACT, H, Hkv, 64, depth=6, causal=True,
                seed=H + 300)
    announce(f"compact tile list H={H} Hkv={Hkv}: every row")
    inp = make_inputs(wl)
    err, relaxed = rows_within_bar(gpu_run(inp), oracle_full(inp), TOL["bf16"], True, inp,
                                   announce)
    announce(f"compact tile list H={H}: max-abs {err:.3e}, {relaxed} rows on the wider bar")


def test_ragged_shapes_take_32_query_slots():
    """The ragged matrix above runs on the other instantiation."""
    for H, Hkv in [(2, 2), (4, 2), (8, 2), (16, 2), (3, 1), (10, 5), (8, 8)]:
        assert prefill_sub_blocks(H, Hkv, len(RAGGED), max(RAGGED), sum(RAGGED)) == 1


def test_fp32_path_at_d64_gqa4():
    """The embed-2048 shape computed end to end in fp32 storage."""
    wl = custom("f32_d64", "f32", (512, 300, 212), 16, 4, 64, depth=12)
    announce("f32 d=64 GQA x4 varlen")
    inp = make_inputs(wl)
    err = max_abs(gpu_run(inp), oracle_full(inp))
    announce(f"max-abs {err:.3e}")
    assert err <= 1e-4


def test_large_logits_bf16():
    """Scores with standard deviation ~8 exercise the running-max rescale."""
    wl = custom("large_logits", "bf16", (512, 777), 16, 4, 64, depth=3)
    inp = make_inputs(wl, q_scale=8.0)
    err = max_abs(gpu_run(inp), oracle_full(inp))
    announce(f"large logits max-abs {err:.3e}")
    assert err <= 2e-2


def test_large_logits_f32():
    wl = custom("large_logits32", "f32", (300, 129), 4, 2, 16, depth=3)
    inp = make_inputs(wl, q_scale=16.0)
    err = max_abs(gpu_run(inp), oracle_full(inp))
    assert err <= 1e-4


def test_single_token_sequences():
    wl = custom("ones", "bf16", (1,) * 37, 8, 2, 64, depth=2)
    inp = make_inputs(wl)
    err = max_abs(gpu_run(inp), oracle_full(inp))
    assert err <= 2e-2


def test_uniform_lengths_without_cu_seqlens():
    da = _da()
    wl = WORKLOADS["embed2048_b2_n512"]
    inp = make_inputs(wl)
    dev = torch.device("cuda:0")
    c = lambda t: t.to(dev).contiguous()
    out = da.fwd(c(inp.q), c(inp.k), c(inp.v), c(inp.lq1), c(inp.lk1),
                 c(inp.lq2), c(inp.lk2), da.lambda_init(wl.depth), None,
                 wl.eps, True, None, nseq=2)
    torch.cuda.synchronize()
    ref = gpu_run(inp)
    assert torch.equal(out, ref)


def test_empty_input():
    da = _da()
    dev = torch.device("cuda:0")
    q = torch.empty(0, 4, 2, 64, dtype=torch.bfloat16, device=dev)
    k = torch.empty(0, 2, 2, 64, dtype=torch.bfloat16, device=dev)
    v = torch.empty(0, 2, 128, dtype=torch.bfloat16, device=dev)
    lv = torch.zeros(64, device=dev)
    out = da.fwd(q, k, v, lv, lv, lv, lv, 0.2, cu_seqlens=torch.zeros(
        2, dtype=torch.int32, device=dev), max_seqlen=0)
    assert out.shape == (0, 4, 128)


def test_identical_maps_lambda_one_is_zero():
    wl = custom("ident", "bf16", (300, 64), 8, 2, 64, depth=4)
    inp = make_inputs(wl)
    inp.q[:, :, 1] = inp.q[:, :, 0]
    inp.k[:, :, 1] = inp.k[:, :, 0]
    inp.lq2, inp.lk2 = inp.lq1.clone(), inp.lk1.clone()
    da = _da()
    dev = torch.device("cuda:0")
    c = lambda t: t.to(dev).contiguous()
    out = da.fwd(c(inp.q), c(inp.k), c(inp.v), c(inp.lq1), c(inp.lk1),
                 c(inp.lq2), c(inp.lk2), 1.0, None, 1e-5, True,
                 c(inp.cu_seqlens), max_seqlen=300)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.float()) == 0


def test_deterministic_and_in_bounds():
    wl = WORKLOADS["embed2048_b2_n512"]
    inp = make_inputs(wl)
    n = wl.T * wl.H * 2 * wl.d
    pad = 4096
    dev = torch.device("cuda:0")
    buf = torch.full((n + 2 * pad,), 12345.0, dtype=torch.bfloat16, device=dev)
    out = buf[pad:pad + n].view(wl.T, wl.H, 2 * wl.d)
    gpu_run(inp, out=out)
    first = out.clone()
    gpu_run(inp, out=out)
    assert torch.equal(first, out), "two runs differ"
    assert torch.all(buf[:pad] == 12345.0) and torch.all(buf[pad + n:] == 12345.0)


def test_causality_bitwise():
    wl = custom("causal", "bf16", (200,), 4, 1, 64, depth=3)
    inp = make_inputs(wl)
    base = gpu_run(inp).clone()
    cut = 77
    inp.q[cut + 1:] += 1.0
    inp.k[cut + 1:] -= 1.0
    inp.v[cut + 1:] *= -3.0
    got = gpu_run(inp)
    assert torch.equal(got[:cut + 1], base[:cut + 1])


def test_gqa_equals_repeated_kv():
    wl = custom("gqa", "bf16", (150, 90), 8, 2, 64, depth=6)
    inp = make_inputs(wl)
    a = gpu_run(inp).clone()
    inp.k = inp.k.repeat_interleave(4, dim=1).contiguous()
    inp.v = inp.v.repeat_interleave(4, dim=1).contiguous()
    b = gpu_run(inp)
    assert torch.equal(a, b)


def test_stream_argument():
    wl = WORKLOADS["embed2048_b2_n512"]
    inp = make_inputs(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = gpu_run(inp, stream=s)
    s.synchronize()
    assert torch.equal(out, gpu_run(inp))


@pytest.mark.parametrize("dtype,d,H,Hkv", [("bf16", 64, 16, 4), ("f32", 16, 4, 2),
                                           ("bf16", 32, 6, 3)])
def test_per_head_lambda(dtype, d, H, Hkv):
    """One set of lambda vectors per head, as the DiffTransformer page keeps
    them ([H, d], lambda_stride = d)."""
    wl = custom("per_head", dtype, (200, 77, 130), H, Hkv, d, depth=9, seed=d)
    inp = make_inputs(wl)
    g = torch.Generator().manual_seed(1234 + d)
    inp.lq1, inp.lk1, inp.lq2, inp.lk2 = [
        0.3 * torch.randn(H, d, generator=g) for _ in range(4)]
    announce(f"per-head lambda {dtype} d={d} H={H} Hkv={Hkv}")
    err = max_abs(gpu_run(inp), oracle_full(inp))
    announce(f"per-head lambda max-abs {err:.3e}")
    assert err <= TOL[dtype]


# ---------------------------------------------------------------------------
# seeded random shapes: sequence mixes whose tile counts are odd and even,
# partial last tiles seen by some waves of a workgroup and not others, every
# head-grouping, both maskings, with and without per-head lambda (vectors at
# 0.2 scale, so some heads get lambda near 1 and some rows nearly cancel:
# case 65 has one such row, token 1 of a sequence in a head with lambda
# 0.9885).  Every bf16 case also runs as its fp32 twin -- the same input
# values in fp32 storage through the fp32 kernel -- at the fp32 bar on every
# row, which pins the rows where bf16 is ill-conditioned.

def random_case(i):
    rng = np.random.default_rng(1000 + i)
    dtype, d = [("bf16", 64), ("bf16", 64), ("bf16", 32), ("bf16", 16), ("f32", 16)][i % 5]
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4, 8]))
    lens = tuple(int(x) for x in rng.integers(0, 700, int(rng.integers(1, 6))))
    return dtype, d, Hkv * G, Hkv, lens, bool(rng.integers(0, 2)), bool(rng.integers(0, 2))


def fp32_twin(inp):
    """The same input values in fp32 storage (bf16 -> fp32 is exact)."""
    import copy
    twin = copy.copy(inp)
    twin.q, twin.k, twin.v = inp.q.float(), inp.k.float(), inp.v.float()
    return twin


@pytest.mark.parametrize("i", range(70))
def test_random_shapes(i):
    dtype, d, H, Hkv, lens, causal, per_head = random_case(i)
    if sum(lens) == 0:
        lens = lens + (5,)
    wl = custom("random", dtype, lens, H, Hkv, d, depth=1 + i % 12, causal=causal,
                seed=2000 + i)
    announce(f"random case {i}: {dtype} d={d} H={H} Hkv={Hkv} lens={lens} "
             f"causal={causal} per-head lambda={per_head}")
    inp = make_inputs(wl)
    if per_head:
        g = torch.Generator().manual_seed(3000 + i)
        inp.lq1, inp.lk1, inp.lq2, inp.lk2 = [0.2 * torch.randn(H, d, generator=g)
                                              for _ in range(4)]
    ref = oracle_full(inp)
    err, relaxed = rows_within_bar(gpu_run(inp), ref, TOL[dtype], dtype == "bf16", inp,
                                   announce)
    announce(f"random case {i}: max-abs {err:.3e}, {relaxed} rows on the wider bar")
    if dtype == "bf16":
        err32 = max_abs(gpu_run(fp32_twin(inp)), ref)
        announce(f"random case {i}: fp32 twin max-abs {err32:.3e}")
        assert err32 <= TOL["f32"]
