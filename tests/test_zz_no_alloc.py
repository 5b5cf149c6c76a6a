"""diffattn_fwd_kv_noalloc, the cache path on the library's static device
scratch, against diffattn_fwd_kv with a caller's workspace, both through the
C ABI.  The two share their kernels and split plan, so the outputs must be
bitwise equal; each is also held to the oracle at the bf16 bar (2e-2).

Two calls in a row, the second on a smaller input, check that what the
first call leaves in the shared scratch does not leak into the second; a
third repeats the first input after the smaller one.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import custom_kv, make_kv_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2


def announce(msg):
    print(f"[no-alloc] {msg}", flush=True)


def _run(inp, noalloc):
    import differential_attention_amd as da
    dev = torch.device("cuda:0")
    c = lambda t: t.to(dev).contiguous()
    lv = [c(x) for x in (inp.lq1, inp.lk1, inp.lq2, inp.lk2)]
    H, d = inp.q.shape[1], inp.q.shape[3]
    # NaN canary: every row must be written
    out = torch.full((inp.q.shape[0], H, 2 * d), float("nan"),
                     dtype=inp.q.dtype, device=dev)
    args = (c(inp.q), c(inp.k), c(inp.v), *lv, da.lambda_init(inp.depth),
            c(inp.w), inp.eps, inp.causal)
    kw = dict(cu_seqlens_q=c(inp.cu_q), cu_seqlens_k=c(inp.cu_k),
              max_seqlen_q=inp.max_q, max_seqlen_k=inp.max_k, out=out)
    if noalloc:
        da.fwd_kv_noalloc(*args, **kw)
    else:
        # a workspace filled with garbage: its contents must not matter
        need = da.kv_workspace_size(inp.cu_q.numel() - 1, inp.max_q,
                                    inp.max_k, H, inp.k.shape[1], d)
        ws = torch.full((need,), 0x7f, dtype=torch.uint8, device=dev)
        da.fwd_kv(*args, workspace=ws, **kw)
    torch.cuda.synchronize()
    return out.cpu()


def _oracle(inp):
    return oracle.fwd_kv(inp.q, inp.k, inp.v, inp.lq1, inp.lk1, inp.lq2,
                         inp.lk2, oracle.lambda_init(inp.depth), inp.w,
                         inp.eps, inp.causal, inp.cu_q.numpy(),
                         inp.cu_k.numpy())


def test_noalloc_equals_workspace_path_on_two_calls():
    import differential_attention_amd as da
    big = custom_kv("noalloc_big", "bf16", (1, 4, 2, 3, 1, 4),
                    (5000, 300, 4097, 77, 12000, 1500), H=16, Hkv=4, d=64,
                    depth=8, seed=11)
    small = custom_kv("noalloc_small", "bf16", (2, 1, 3), (130, 40, 3),
                      H=8, Hkv=2, d=32, depth=3, seed=12)
    for wl in (big, small):
        need = da.kv_workspace_size(wl.nseq, wl.max_q, wl.max_k, wl.H,
                                    wl.Hkv, wl.d)
        assert 0 < need <= da.KV_SCRATCH_BYTES
    inputs = [make_kv_inputs(big), make_kv_inputs(small)]
    refs = [_oracle(x) for x in inputs]
    # noalloc on big, then on small, then big again
    for i, which in enumerate((0, 1, 0)):
        inp = inputs[which]
        announce(f"call {i}: {(big, small)[which].name}")
        got = _run(inp, noalloc=True)
        want = _run(inp, noalloc=False)
        assert not torch.isnan(got.float()).any()
        assert torch.equal(got, want), "no-alloc output differs from the workspace path"
        err = float(np.max(np.abs(got.float().double().numpy() - refs[which])))
        announce(f"call {i}: bitwise equal, max-abs vs oracle {err:.3e}")
        assert err <= TOL


def test_noalloc_rejects_oversized_without_writing():
    import differential_attention_amd as da
    dev = torch.device("cuda:0")
    # (2 query rows: the split-KV path is the only one, and its partials do
    # not fit the scratch)
    nseq, nq, nk, H, Hkv, d = 4096, 2, 128, 16, 4, 64
    assert da.kv_workspace_size(nseq, nq, nk, H, Hkv, d) > da.KV_SCRATCH_BYTES
    q = torch.zeros(nseq * nq, H, 2, d, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(nseq * nk, Hkv, 2, d, dtype=torch.bfloat16, device=dev)
    v = torch.zeros(nseq * nk, Hkv, 2 * d, dtype=torch.bfloat16, device=dev)
    lv = [torch.zeros(d, device=dev) for _ in range(4)]
    out = torch.full((nseq * nq, H, 2 * d), 3.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(da.DiffAttnError) as e:
        da.fwd_kv_noalloc(q, k, v, *lv, 0.5, nseq=nseq, out=out)
    assert e.value.status == da.ETOOLARGE
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
