"""Parity of the fused rotary prologue (diffattn_fwd with rope tables)
with the fp64 oracle's rotary prologue.

The pull request's test rotates q and k with apply_rotary_emb(...,
interleaved=True) on every d-wide half-head before the attention call and
stores the result in its bf16 storage type; the kernel does the same on the
fly (positions restart in every packed sequence), and the oracle is asked
to round the rotated rows to bf16 for bf16 inputs.  Tolerances as for the
plain forward: max-abs 1e-4 (fp32 storage), 2e-2 (bf16).  All tests need an
MI355X.
"""

import numpy as np
import pytest
import torch

import oracle
from conditioning import rotated, rows_within_bar
from workloads import WORKLOADS, custom, make_inputs, rope_tables
from launch_shape import prefill_sub_blocks

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def announce(msg):
    print(f"[parity-rope] {msg}", flush=True)


def gpu_run(inp, rope, max_seqlen=None):
    import differential_attention_amd as da
    dev = torch.device("cuda:0")
    c = lambda t: t.to(dev).contiguous()
    out = da.fwd(c(inp.q), c(inp.k), c(inp.v), c(inp.lq1), c(inp.lk1),
                 c(inp.lq2), c(inp.lk2), da.lambda_init(inp.depth), c(inp.w),
                 inp.eps, inp.causal, c(inp.cu_seqlens),
                 max_seqlen=inp.max_seqlen if max_seqlen is None else max_seqlen,
                 rope=None if rope is None else tuple(c(t) for t in rope))
    torch.cuda.synchronize()
    return out


def oracle_full(inp, rope):
    return oracle.fwd(inp.q, inp.k, inp.v, inp.lq1, inp.lk1, inp.lq2, inp.lk2,
                      oracle.lambda_init(inp.depth), inp.w, inp.eps,
                      inp.causal, inp.cu_seqlens, rope=rope,
                      rope_round_bf16=inp.q.dtype == torch.bfloat16)


def max_abs(gpu_out, ref):
    got = gpu_out.float().cpu().double().numpy()
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    return float(np.max(np.abs(got - ref))) if ref.size else 0.0


RAGGED = (1, 0, 31, 32, 33, 63, 64, 65, 127, 200, 0, 7)


@pytest.mark.parametrize("dtype,d", [("f32", 16), ("bf16", 64), ("f32", 64),
                                     ("bf16", 16), ("bf16", 32)])
@pytest.mark.parametrize("H,Hkv", [(4, 2), (16, 2), (3, 1)])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged_varlen_rope(dtype, d, H, Hkv, causal):
    wl = custom("ragged_rope", dtype, RAGGED, H, Hkv, d, depth=5,
                causal=causal, seed=H * 100 + d + 7)
    inp = make_inputs(wl)
    inp.w = torch.linspace(0.5, 1.5, 2 * d)
    # a small base turns every pair noticeably within 200 positions
    rope = rope_tables(256, d, base=50.0)
    err = max_abs(gpu_run(inp, rope), oracle_full(inp, rope))
    announce(f"ragged {dtype} d={d} H={H} Hkv={Hkv} causal={causal}: max-abs {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 16), ("bf16", 32), ("f32", 64),
                                     ("bf16", 16)])
@pytest.mark.parametrize("lens", [RAGGED, RAGGED * 11])
def test_bf16_tables(dtype, d, lens):
    """Tables stored in bf16 (as the pull request's test caches them): the
    output equals, bitwise, that of fp32 tables holding the same values, on
    both instantiations of the prefill, and the oracle's with those values."""
    wl = custom("rope_bf16_tables", dtype, lens, 16, 4, d, depth=4, seed=d + 51)
    inp = make_inputs(wl)
    rb = tuple(t.bfloat16() for t in rope_tables(256, d, base=50.0))
    rf = tuple(t.float() for t in rb)
    a, b = gpu_run(inp, rb), gpu_run(inp, rf)
    assert torch.equal(a, b)
    err = max_abs(a, oracle_full(inp, rf))
    announce(f"bf16 tables {dtype} d={d} {len(lens)} sequences: max-abs {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,d", [("f32", 16), ("bf16", 64), ("bf16", 32), ("f32", 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged_varlen_rope_64_query_slots(dtype, d, causal):
    """Many short sequences: the 64-query instantiation with the rotation."""
    lens = RAGGED * 11
    assert prefill_sub_blocks(16, 4, len(lens), max(lens), sum(lens)) == 2
    wl = custom("ragged_rope_many", dtype, lens, 16, 4, d, depth=9, causal=causal,
                seed=d + 70)
    inp = make_inputs(wl)
    inp.w = torch.linspace(1.5, 0.5, 2 * d)
    rope = rope_tables(256, d, base=50.0)
    err = max_abs(gpu_run(inp, rope), oracle_full(inp, rope))
    announce(f"ragged x11 {dtype} d={d} causal={causal}: max-abs {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,d,H,Hkv", [("bf16", 64, 10, 5), ("bf16", 64, 16, 8),
                                           ("f32", 16, 8, 8), ("bf16", 32, 9, 3),
                                           ("f32", 64, 10, 5), ("bf16", 16, 24, 8)])
def test_many_kv_heads_rope(dtype, d, H, Hkv):
    """The K rotation takes each chunk position of a token through its
    2 Hkv half-heads eight at a time: Hkv = 3 leaves a partial group, Hkv = 5
    and 8 need a second one."""
    wl = custom("kvheads_rope", dtype, (300, 1, 129, 64), H, Hkv, d, depth=3,
                causal=True, seed=H * 10 + Hkv + d)
    inp = make_inputs(wl)
    inp.w = torch.linspace(0.5, 1.5, 2 * d)
    rope = rope_tables(320, d, base=50.0)
    err = max_abs(gpu_run(inp, rope), oracle_full(inp, rope))
    announce(f"kv heads {dtype} d={d} H={H} Hkv={Hkv}: max-abs {err:.3e}")
    assert err <= TOL[dtype]


def test_identity_tables_bitwise():
    """cos = 1, sin = 0: the rotated path must reproduce the plain one bit
    for bit (x * 1 - y * 0 is exact)."""
    wl = custom("ident_rope", "bf16", (300, 77, 1), 16, 4, 64, depth=8, seed=3)
    inp = make_inputs(wl)
    ones = torch.ones(300, 32)
    zeros = torch.zeros(300, 32)
    a = gpu_run(inp, (ones, zeros))
    b = gpu_run(inp, None)
    assert torch.equal(a, b)


def test_rotation_changes_output():
    wl = custom("chg_rope", "bf16", (300,), 16, 4, 64, depth=8, seed=4)
    inp = make_inputs(wl)
    a = gpu_run(inp, rope_tables(300, 64))
    b = gpu_run(inp, None)
    assert float((a.float() - b.float()).abs().max()) > 0.05


@pytest.mark.parametrize("name", ["llama1b_b8_n4096", "long_b1_n32768"])
def test_large_workloads_rope_sampled(name):
    """The benchmark's rotary configuration (base 10000, tables as long as
    the longest sequence) at full size, on sampled rows."""
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    rope = rope_tables(wl.max_seqlen, wl.d)
    out = gpu_run(inp, rope)
    rng = np.random.default_rng(5)
    cu = wl.cu_seqlens()
    toks = []
    for s in range(wl.nseq):
        a, n = int(cu[s]), int(cu[s + 1] - cu[s])
        local = {0, 1, 63, 64, 127, 128, n // 2, n - 1} | set(
            int(x) for x in rng.integers(0, n, 6 if wl.nseq > 1 else 40))
        toks += [a + i for i in sorted(local) if 0 <= i < n]
    toks = np.array(toks, np.int64)
    heads = ((np.arange(toks.size) * 7) % wl.H).astype(np.int32)
    ref = oracle.rows(inp.q, inp.k, inp.v, inp.lq1, inp.lk1, inp.lq2, inp.lk2,
                      oracle.lambda_init(wl.depth), toks, heads, inp.w,
                      inp.eps, inp.causal, inp.cu_seqlens, rope=rope,
                      rope_round_bf16=True)
    got = out[torch.from_numpy(toks).cuda(), torch.from_numpy(heads).long().cuda()]
    err = max_abs(got, ref)
    announce(f"{name} +rope: {toks.size} rows, max-abs {err:.3e}")
    assert err <= 2e-2


def test_longer_tables_and_per_head_lambda():
    wl = custom("rope_ph", "bf16", (130, 250), 8, 2, 64, depth=6, seed=9)
    inp = make_inputs(wl)
    g = torch.Generator().manual_seed(99)
    inp.lq1, inp.lk1, inp.lq2, inp.lk2 = [0.3 * torch.randn(8, 64, generator=g)
                                          for _ in range(4)]
    rope = rope_tables(4096, 64, base=500.0)
    err = max_abs(gpu_run(inp, rope), oracle_full(inp, rope))
    announce(f"longer tables, per-head lambda: max-abs {err:.3e}")
    assert err <= 2e-2


def test_short_tables_rejected():
    import differential_attention_amd as da
    wl = custom("short_rope", "bf16", (100,), 4, 2, 64, seed=1)
    inp = make_inputs(wl)
    with pytest.raises(da.DiffAttnError):
        gpu_run(inp, rope_tables(99, 64))


@pytest.mark.parametrize("i", range(24))
def test_random_shapes_rope(i):
    """Seeded random shapes through the rotary prologue: sequence mixes
    (positions restart in every sequence), head groupings, the five (dtype,
    d) instantiations, masking, table bases and lengths, shared or per-head
    lambda; rows whose maps cancel held to the conditioning-scaled bar
    (capped at 4x), and every bf16 case run again as its fp32 twin at the
    fp32 bar."""
    rng = np.random.default_rng(5000 + i)
    dtype, d = [("bf16", 64), ("bf16", 32), ("bf16", 16), ("f32", 16), ("f32", 64)][i % 5]
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4]))
    lens = tuple(int(x) for x in rng.integers(0, 600, int(rng.integers(1, 6))))
    if sum(lens) == 0:
        lens = lens + (5,)
    causal = bool(rng.integers(0, 2))
    wl = custom("random_rope", dtype, lens, Hkv * G, Hkv, d, depth=1 + i % 10, causal=causal,
                seed=6000 + i)
    inp = make_inputs(wl)
    if rng.integers(0, 2):
        g = torch.Generator().manual_seed(7000 + i)
        inp.lq1, inp.lk1, inp.lq2, inp.lk2 = [0.2 * torch.randn(Hkv * G, d, generator=g)
                                              for _ in range(4)]
    base = float(rng.choice([50.0, 500.0, 10000.0]))
    rope = rope_tables(max(lens) + int(rng.integers(0, 50)), d, base=base)
    announce(f"random case {i}: {dtype} d={d} H={Hkv * G} Hkv={Hkv} lens={lens} "
             f"causal={causal} base={base}")
    err, relaxed = rows_within_bar(gpu_run(inp, rope), oracle_full(inp, rope), TOL[dtype],
                                   dtype == "bf16", rotated(inp, rope), announce)
    announce(f"random case {i}: max-abs {err:.3e}, {relaxed} rows on the wider bar")
    if dtype == "bf16":
        # the same values in fp32 storage: the rotation then stays in fp32
        # on both sides, held to the fp32 bar on every row
        import copy
        twin = copy.copy(inp)
        twin.q, twin.k, twin.v = inp.q.float(), inp.k.float(), inp.v.float()
        err32 = max_abs(gpu_run(twin, rope), oracle_full(twin, rope))
        announce(f"random case {i}: fp32 twin max-abs {err32:.3e}")
        assert err32 <= TOL["f32"]
