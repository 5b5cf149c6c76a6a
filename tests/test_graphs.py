"""Every entry point allocates nothing, never synchronises and launches only
kernels on the caller's stream, so a call can be captured into a HIP graph
(torch.cuda.CUDAGraph) and replayed.  Each test captures a call, replays it
several times with the program's own eager work and synchronisations in
between, changes an input in place between replays, and checks every
replay bitwise against an eager call on the same inputs.  All tests need
an MI355X.
"""

import pytest
import torch

import differential_attention_amd as da
from workloads import custom, custom_kv, make_inputs, make_kv_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def announce(msg):
    print(f"[graphs] {msg}", flush=True)


def capture(fn):
    """Warm up on a side stream, then capture fn() into a graph; returns the
    graph and what fn returned during capture (its static outputs)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = fn()
    torch.cuda.synchronize()
    return g, res


def eager_noise():
    """Unrelated eager work with a synchronisation, between replays."""
    x = torch.randn(1 << 20, device=DEV)
    (x * 3 + 1).sum().item()


def replay_and_check(g, static_out, eager, mutate, name, rounds=3):
    for i in range(rounds):
        if i == rounds - 1:
            mutate()            # a changed input must show in the replay
        eager_noise()
        ref = eager()
        g.replay()
        torch.cuda.synchronize()
        outs = static_out if isinstance(static_out, (list, tuple)) else [static_out]
        refs = ref if isinstance(ref, (list, tuple)) else [ref]
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), f"{name}: replay {i} differs from the eager call"
    announce(f"{name}: {rounds} replays bitwise equal to eager calls")


def dev_inputs(wl):
    inp = make_inputs(wl)
    c = lambda t: t.to(DEV).contiguous()
    return (c(inp.q), c(inp.k), c(inp.v), [c(x) for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)],
            c(inp.w), c(inp.cu_seqlens), inp)


@pytest.mark.parametrize("rope", [False, True])
def test_fwd_graph(rope):
    wl = custom("graph", "bf16", (200, 33, 512, 1), H=8, Hkv=2, d=64, depth=3, seed=5)
    q, k, v, lv, w, cu, inp = dev_inputs(wl)
    lam0 = da.lambda_init(wl.depth)
    tabs, ws = None, None
    if rope:
        pos = torch.arange(wl.max_seqlen, dtype=torch.float64)[:, None]
        inv = 10000.0 ** (-torch.arange(0, wl.d, 2, dtype=torch.float64) / wl.d)
        tabs = (torch.cos(pos * inv).float().to(DEV).contiguous(),
                torch.sin(pos * inv).float().to(DEV).contiguous())
        ws = torch.empty(da.fwd_workspace_size(q.dtype, q.shape[0], wl.Hkv, wl.d, True),
                         dtype=torch.uint8, device=DEV)
    out = torch.empty((q.shape[0], wl.H, 2 * wl.d), dtype=q.dtype, device=DEV)
    kw = dict(subln_weight=w, eps=wl.eps, causal=True, cu_seqlens=cu,
              max_seqlen=wl.max_seqlen, rope=tabs)
    g, static = capture(lambda: da.fwd(q, k, v, *lv, lam0, out=out, workspace=ws, **kw))

    def eager():
        return da.fwd(q, k, v, *lv, lam0,
                      workspace=None if ws is None else torch.empty_like(ws), **kw)

    replay_and_check(g, static, eager, lambda: q.mul_(-0.5), f"fwd rope={rope}")


def test_fwd_kv_graph():
    wl = custom_kv("graph", "bf16", (1, 3, 2), (700, 40, 1500), H=16, Hkv=4, d=64,
                   depth=2, seed=6)
    inp = make_kv_inputs(wl)
    c = lambda t: t.to(DEV).contiguous()
    q, k, v = c(inp.q), c(inp.k), c(inp.v)
    lv = [c(x) for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
    cq, ck = c(inp.cu_q), c(inp.cu_k)
    lam0 = da.lambda_init(wl.depth)
    nseq = cq.numel() - 1
    ws = torch.empty(da.kv_workspace_size(nseq, inp.max_q, inp.max_k, wl.H, wl.Hkv, wl.d),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty((q.shape[0], wl.H, 2 * wl.d), dtype=q.dtype, device=DEV)
    kw = dict(subln_weight=c(inp.w), eps=wl.eps, causal=True, cu_seqlens_q=cq,
              cu_seqlens_k=ck, max_seqlen_q=inp.max_q, max_seqlen_k=inp.max_k)
    g, static = capture(lambda: da.fwd_kv(q, k, v, *lv, lam0, workspace=ws, out=out, **kw))
    replay_and_check(g, static, lambda: da.fwd_kv(q, k, v, *lv, lam0, **kw),
                     lambda: v.mul_(2.0), "fwd_kv")


def test_decode_step_with_rotary_graph():
    """A rotary decode step -- the step's keys turned into the cache, then
    the new queries turned and attending -- captured as one graph."""
    from workloads import rope_tables
    wl = custom_kv("graph_rope", "bf16", (1, 3, 2), (700, 40, 1500), H=16, Hkv=4, d=64,
                   depth=3, seed=16)
    inp = make_kv_inputs(wl)
    c = lambda t: t.to(DEV).contiguous()
    q, kc, vc = c(inp.q), c(inp.k), c(inp.v)
    g_ = torch.Generator().manual_seed(17)
    k_new = c(torch.randn(q.shape[0], wl.Hkv, 2, wl.d, generator=g_).to(q.dtype))
    v_new = c(torch.randn(q.shape[0], wl.Hkv, 2 * wl.d, generator=g_).to(q.dtype))
    lv = [c(x) for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
    cq, ck = c(inp.cu_q), c(inp.cu_k)
    rope = tuple(c(t) for t in rope_tables(inp.max_k, wl.d, base=50.0))
    lam0 = da.lambda_init(wl.depth)
    nseq = cq.numel() - 1
    ws = torch.empty(da.kv_workspace_size(nseq, inp.max_q, inp.max_k, wl.H, wl.Hkv, wl.d),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty((q.shape[0], wl.H, 2 * wl.d), dtype=q.dtype, device=DEV)
    kw = dict(subln_weight=c(inp.w), eps=wl.eps, causal=True, cu_seqlens_q=cq,
              cu_seqlens_k=ck, max_seqlen_q=inp.max_q, max_seqlen_k=inp.max_k, rope=rope)

    def step(**extra):
        da.kv_append(k_new, v_new, kc, vc, cu_seqlens_q=cq, cu_seqlens_k=ck,
                     max_seqlen_k=inp.max_k, rope=rope)
        return da.fwd_kv(q, kc, vc, *lv, lam0, **kw, **extra)

    g, static = capture(lambda: step(workspace=ws, out=out))
    replay_and_check(g, static, step, lambda: k_new.mul_(2.0), "rotary decode step")


@pytest.mark.parametrize("path", [None, da.KV_PATH_PREFILL, da.KV_PATH_PREFILL_SPLIT])
def test_chunked_prefill_step_graph(path):
    """A rotary chunked-prefill step -- the chunk's keys turned into the
    cache, then its queries attending on the prefill kernel (whole key
    ranges, or key splits merged by the combine kernel) -- captured as one
    graph."""
    from workloads import rope_tables
    wl = custom_kv("graph_chunk", "bf16", (200, 64, 1), (1200, 300, 900), H=16, Hkv=4, d=64,
                   depth=5, seed=18)
    inp = make_kv_inputs(wl)
    c = lambda t: t.to(DEV).contiguous()
    q, kc, vc = c(inp.q), c(inp.k), c(inp.v)
    g_ = torch.Generator().manual_seed(19)
    k_new = c(torch.randn(q.shape[0], wl.Hkv, 2, wl.d, generator=g_).to(q.dtype))
    v_new = c(torch.randn(q.shape[0], wl.Hkv, 2 * wl.d, generator=g_).to(q.dtype))
    lv = [c(x) for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
    cq, ck = c(inp.cu_q), c(inp.cu_k)
    rope = tuple(c(t) for t in rope_tables(inp.max_k, wl.d, base=50.0))
    lam0 = da.lambda_init(wl.depth)
    nseq = cq.numel() - 1
    need = (da.kv_workspace_size(nseq, inp.max_q, inp.max_k, wl.H, wl.Hkv, wl.d) if path is None
            else da.kv_path_workspace_size(path, nseq, inp.max_q, inp.max_k, wl.H, wl.Hkv,
                                           wl.d))
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
    out = torch.empty((q.shape[0], wl.H, 2 * wl.d), dtype=q.dtype, device=DEV)
    kw = dict(subln_weight=c(inp.w), eps=wl.eps, causal=True, cu_seqlens_q=cq,
              cu_seqlens_k=ck, max_seqlen_q=inp.max_q, max_seqlen_k=inp.max_k, rope=rope,
              path=path)

    def step(**extra):
        da.kv_append(k_new, v_new, kc, vc, cu_seqlens_q=cq, cu_seqlens_k=ck,
                     max_seqlen_k=inp.max_k, rope=rope)
        return da.fwd_kv(q, kc, vc, *lv, lam0, **kw, **extra)

    g, static = capture(lambda: step(workspace=ws, out=out))
    replay_and_check(g, static, step, lambda: q.mul_(-1.5), f"chunked prefill step path={path}")


def test_training_step_graph():
    wl = custom("graph", "bf16", (300, 65, 129), H=8, Hkv=2, d=64, depth=4, seed=7)
    q, k, v, lv, w, cu, inp = dev_inputs(wl)
    lam0 = da.lambda_init(wl.depth)
    dy = torch.randn((q.shape[0], wl.H, 2 * wl.d), generator=torch.Generator().manual_seed(8))
    dy = dy.to(q.dtype).to(DEV).contiguous()
    ws = torch.empty(da.bwd_workspace_size(q.dtype, q.shape[0], wl.H, wl.d), dtype=torch.uint8,
                     device=DEV)
    kw = dict(subln_weight=w, eps=wl.eps, causal=True, cu_seqlens=cu, max_seqlen=wl.max_seqlen)
    names = ("dq", "dk", "dv", "dlq1", "dlk1", "dlq2", "dlk2", "dw")

    def step(workspace):
        out, lse, o12 = da.fwd_train(q, k, v, *lv, lam0, **kw)
        gr = da.bwd(q, k, v, *lv, lam0, dy, lse, o12, workspace=workspace, **kw)
        return [out, lse, o12] + [gr[n] for n in names]

    g, static = capture(lambda: step(ws))
    replay_and_check(g, static, lambda: step(torch.empty_like(ws)), lambda: k.mul_(0.75),
                     "training step")
