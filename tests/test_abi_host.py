"""The C-ABI library on the host: it loads, exports every declared symbol
and rejects malformed arguments before touching a device (CPU only)."""

import ctypes
import os
import re

import pytest

import differential_attention_amd as da

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "diffattn.h")
FAKE = 0x1000   # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(diffattn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return da.library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "diffattn_fwd" in names and len(names) >= 6
    for name in names:
        assert hasattr(lib, name), f"{name} declared in diffattn.h but not exported"


def test_abi_version_matches_header(lib):
    m = re.search(r"#define DIFFATTN_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.diffattn_abi_version() == int(m.group(1))


def test_strerror(lib):
    for st in (0, -1, -2, -3, -4, 12345):
        assert isinstance(da.strerror(st), str) and da.strerror(st)


def test_lambda_init_schedule():
    assert abs(da.lambda_init(1) - 0.2) < 1e-15
    assert abs(da.lambda_init(10 ** 6) - 0.8) < 1e-15


def test_fwd_workspace_size():
    import torch
    assert da.fwd_workspace_size(torch.bfloat16, 64, 4, 64, False) == 0
    assert da.fwd_workspace_size(torch.bfloat16, 64, 4, 64, True) >= 64 * 4 * 128 * 2
    assert da.fwd_workspace_size(torch.float32, 64, 4, 64, True) >= 64 * 4 * 128 * 4


def test_supported():
    import torch
    assert da.supported(torch.bfloat16, 64)
    assert da.supported(torch.float32, 16)
    assert da.supported(torch.float32, 32)
    assert not da.supported(torch.bfloat16, 48)


def test_check_cu_seqlens():
    assert da.check_cu_seqlens([0, 3, 3, 10], 10, 7)
    assert not da.check_cu_seqlens([0, 3, 3, 10], 10, 6)     # length 7 > max
    assert not da.check_cu_seqlens([0, 5, 4, 10], 10, 10)    # decreasing
    assert not da.check_cu_seqlens([1, 5, 10], 10, 10)       # cu[0] != 0
    assert not da.check_cu_seqlens([0, 5, 9], 10, 10)        # cu[nseq] != T


def call(**over):
    a = dict(dtype=da.BF16, q=FAKE, k=FAKE, v=FAKE, lq1=FAKE, lk1=FAKE,
             lq2=FAKE, lk2=FAKE, lambda_stride=0, lambda_init_value=0.2,
             subln_weight=0,
             eps=1e-5, causal=1, cu_seqlens=0, nseq=2, max_seqlen=0, T=64,
             H=16, Hkv=4, d=64, rope_cos=0, rope_sin=0, rope_len=0,
             rope_dtype=0, workspace=0, workspace_bytes=0, out=FAKE, stream=0)
    a.update(over)
    return da.fwd_ptr(**a)


@pytest.mark.parametrize("over,status", [
    (dict(dtype=7), da.EINVAL),
    (dict(H=6, Hkv=4), da.EINVAL),
    (dict(Hkv=0), da.EINVAL),
    (dict(T=-1), da.EINVAL),
    (dict(causal=2), da.EINVAL),
    (dict(eps=-1.0), da.EINVAL),
    (dict(eps=float("nan")), da.EINVAL),
    (dict(lambda_init_value=float("inf")), da.EINVAL),
    (dict(lambda_stride=-1), da.EINVAL),
    (dict(lambda_stride=63), da.EINVAL),        # stride below d
    (dict(d=48), da.EUNSUPPORTED),
    (dict(dtype=da.F32, d=48), da.EUNSUPPORTED),
    (dict(q=0), da.EINVAL),
    (dict(out=0), da.EINVAL),
    (dict(lk2=0), da.EINVAL),
    (dict(q=FAKE + 8), da.EINVAL),             # not 16-byte aligned
    (dict(nseq=0), da.EINVAL),
    (dict(nseq=3), da.EINVAL),                 # T % nseq != 0 without cu
    (dict(max_seqlen=31), da.EINVAL),          # must equal T / nseq
    (dict(cu_seqlens=FAKE, max_seqlen=0), da.EINVAL),
    (dict(cu_seqlens=FAKE, max_seqlen=65), da.EINVAL),
    (dict(rope_cos=FAKE, rope_len=32), da.EINVAL),               # sin missing
    (dict(rope_cos=FAKE, rope_sin=FAKE, rope_len=31, workspace=FAKE,
          workspace_bytes=1 << 20), da.EINVAL),                     # < max_seqlen
    (dict(rope_cos=FAKE + 8, rope_sin=FAKE, rope_len=32, workspace=FAKE,
          workspace_bytes=1 << 20), da.EINVAL),                     # alignment
    (dict(rope_cos=FAKE, rope_sin=FAKE, rope_len=32), da.EINVAL),   # no workspace
    (dict(rope_cos=FAKE, rope_sin=FAKE, rope_len=32, workspace=FAKE,
          workspace_bytes=100), da.EINVAL),                         # workspace too small
    (dict(rope_cos=FAKE, rope_sin=FAKE, rope_len=32, rope_dtype=5, workspace=FAKE,
          workspace_bytes=1 << 20), da.EINVAL),                     # table type
    (dict(T=0, q=0, k=0, v=0, out=0), da.OK),  # empty: nothing launched
])
def test_validation_before_any_device_work(over, status):
    assert call(**over) == status


# --------------------------------------------------------------------------
# the key/value-cache entry point

def test_supported_kv():
    import torch
    assert da.supported_kv(torch.bfloat16, 64)
    assert da.supported_kv(torch.bfloat16, 32)
    assert not da.supported_kv(torch.bfloat16, 16)
    assert not da.supported_kv(torch.float32, 64)


def test_kv_workspace_size():
    small = da.kv_workspace_size(8, 1, 4097, 16, 4, 64)
    big = da.kv_workspace_size(64, 1, 8192, 16, 4, 64)
    assert 0 < small < big
    assert da.kv_workspace_size(8, 1, 4097, 16, 5, 64) == 0   # H % Hkv
    assert da.kv_workspace_size(0, 1, 4097, 16, 4, 64) == 0
    # more queries need more partial rows
    assert da.kv_workspace_size(8, 4, 4097, 16, 4, 64) > small


def test_check_cu_seqlens_kv():
    ok = da.check_cu_seqlens_kv
    assert ok([0, 1, 3], [0, 10, 12], 3, 12, 2, 10)
    assert not ok([0, 1, 3], [0, 10, 12], 3, 12, 1, 10)     # nq 2 > max
    assert not ok([0, 1, 3], [0, 10, 11], 3, 11, 2, 10)     # causal nq > nk
    assert ok([0, 1, 3], [0, 10, 11], 3, 11, 2, 10, causal=False)
    assert not ok([0, 1, 3], [0, 0, 12], 3, 12, 2, 12, causal=False)  # nk = 0
    assert not ok([0, 1, 3], [0, 10, 12], 3, 13, 2, 10)     # cu_k[nseq] != Tk


def call_kv(**over):
    a = dict(dtype=da.BF16, q=FAKE, k=FAKE, v=FAKE, lq1=FAKE, lk1=FAKE,
             lq2=FAKE, lk2=FAKE, lambda_stride=0, lambda_init_value=0.7,
             subln_weight=0, eps=1e-5, causal=1, cu_seqlens_q=0,
             cu_seqlens_k=0, nseq=8, max_seqlen_q=0, max_seqlen_k=0, Tq=8,
             Tk=8 * 4097, H=16, Hkv=4, d=64, rope_cos=0, rope_sin=0,
             rope_len=0, rope_dtype=0, workspace=FAKE,
             workspace_bytes=1 << 30, out=FAKE, stream=0)
    a.update(over)
    return da.fwd_kv_ptr(**a)


@pytest.mark.parametrize("over,status", [
    (dict(dtype=7), da.EINVAL),
    (dict(H=6, Hkv=4), da.EINVAL),
    (dict(Tq=-1), da.EINVAL),
    (dict(causal=2), da.EINVAL),
    (dict(eps=-1.0), da.EINVAL),
    (dict(lambda_init_value=float("nan")), da.EINVAL),
    (dict(lambda_stride=63), da.EINVAL),
    (dict(dtype=da.F32), da.EUNSUPPORTED),
    (dict(d=16), da.EUNSUPPORTED),
    (dict(cu_seqlens_q=FAKE), da.EINVAL),          # one boundary array only
    (dict(Tq=12), da.EINVAL),                      # Tq % nseq
    (dict(Tk=8 * 4097 + 1), da.EINVAL),            # Tk % nseq
    (dict(Tq=8 * 5000), da.EINVAL),                # causal: nq > nk
    (dict(Tk=0), da.EINVAL),                       # queries without keys
    (dict(q=0), da.EINVAL),
    (dict(workspace=0), da.EINVAL),
    (dict(workspace=FAKE + 4), da.EINVAL),         # not 16-byte aligned
    (dict(workspace_bytes=1024), da.EINVAL),       # smaller than required
    (dict(cu_seqlens_q=FAKE, cu_seqlens_k=FAKE, max_seqlen_q=9), da.EINVAL),
    (dict(cu_seqlens_q=FAKE, cu_seqlens_k=FAKE, max_seqlen_q=1,
          max_seqlen_k=8 * 4097 + 1), da.EINVAL),  # bound beyond Tk
    (dict(rope_cos=FAKE), da.EINVAL),              # one table only
    (dict(rope_cos=FAKE, rope_sin=FAKE, rope_len=4097, rope_dtype=7), da.EINVAL),
    (dict(rope_cos=FAKE, rope_sin=FAKE, rope_len=4096), da.EINVAL),   # < max_seqlen_k
    (dict(rope_cos=FAKE + 8, rope_sin=FAKE, rope_len=4097), da.EINVAL),
    (dict(Tq=0, q=0, out=0), da.OK),               # no query rows
])
def test_kv_validation_before_any_device_work(over, status):
    assert call_kv(**over) == status


def call_kv_noalloc(**over):
    a = dict(dtype=da.BF16, q=FAKE, k=FAKE, v=FAKE, lq1=FAKE, lk1=FAKE,
             lq2=FAKE, lk2=FAKE, lambda_stride=0, lambda_init_value=0.7,
             subln_weight=0, eps=1e-5, causal=1, cu_seqlens_q=0,
             cu_seqlens_k=0, nseq=8, max_seqlen_q=0, max_seqlen_k=0, Tq=8,
             Tk=8 * 4097, H=16, Hkv=4, d=64, rope_cos=0, rope_sin=0,
             rope_len=0, rope_dtype=0, out=FAKE, stream=0)
    a.update(over)
    return da.fwd_kv_noalloc_ptr(**a)


def test_kv_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define DIFFATTN_KV_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == da.KV_SCRATCH_BYTES
    # the three decode workloads fit the static scratch
    for nseq, mq, mk in ((8, 1, 4097), (64, 1, 8192), (32, 4, 31196)):
        assert 0 < da.kv_workspace_size(nseq, mq, mk, 16, 4, 64) <= da.KV_SCRATCH_BYTES


@pytest.mark.parametrize("over,status", [
    (dict(dtype=7), da.EINVAL),
    (dict(H=6, Hkv=4), da.EINVAL),
    (dict(causal=2), da.EINVAL),
    (dict(dtype=da.F32), da.EUNSUPPORTED),
    (dict(Tq=12), da.EINVAL),                      # Tq % nseq
    (dict(Tk=0), da.EINVAL),                       # queries without keys
    (dict(q=0), da.EINVAL),
    (dict(out=FAKE + 4), da.EINVAL),               # not 16-byte aligned
    (dict(rope_cos=FAKE, rope_sin=FAKE, rope_len=100), da.EINVAL),  # < max_seqlen_k
    (dict(Tq=0, q=0, out=0), da.OK),               # no query rows
    # split partials beyond the static scratch: 4096 sequences x 2 queries x
    # 16 heads against 128 keys each (a decode-sized call, too few query rows
    # for the prefill kernel)
    (dict(nseq=4096, Tq=4096 * 2, Tk=4096 * 128), da.ETOOLARGE),
])
def test_kv_noalloc_validation_before_any_device_work(over, status):
    assert call_kv_noalloc(**over) == status


def call_append(**over):
    a = dict(dtype=da.BF16, k_new=FAKE, v_new=FAKE, cu_seqlens_q=0,
             cu_seqlens_k=0, nseq=8, max_seqlen_k=0, Tq=8, Tk=8 * 4097,
             Hkv=4, d=64, rope_cos=0, rope_sin=0, rope_len=0, rope_dtype=0,
             k_cache=FAKE, v_cache=FAKE, stream=0)
    a.update(over)
    return da.kv_append_ptr(**a)


@pytest.mark.parametrize("over,status", [
    (dict(dtype=7), da.EINVAL),
    (dict(Hkv=0), da.EINVAL),
    (dict(nseq=0), da.EINVAL),
    (dict(d=48), da.EUNSUPPORTED),
    (dict(cu_seqlens_q=FAKE), da.EINVAL),          # one boundary array only
    (dict(Tq=12), da.EINVAL),                      # Tq % nseq
    (dict(Tq=8 * 5000), da.EINVAL),                # nq > nk
    (dict(k_cache=0), da.EINVAL),
    (dict(v_new=FAKE + 4), da.EINVAL),             # not 16-byte aligned
    (dict(rope_cos=FAKE), da.EINVAL),              # one table only
    (dict(rope_cos=FAKE, rope_sin=FAKE, rope_len=4096), da.EINVAL),  # < nk
    (dict(rope_cos=FAKE, rope_sin=FAKE, rope_len=4097, rope_dtype=3), da.EINVAL),
    (dict(cu_seqlens_q=FAKE, cu_seqlens_k=FAKE, max_seqlen_k=8 * 4097 + 1), da.EINVAL),
    (dict(Tq=0, k_new=0, v_new=0), da.OK),         # nothing to append
])
def test_kv_append_validation_before_any_device_work(over, status):
    assert call_append(**over) == status


def test_kv_noalloc_too_large_matches_workspace_size():
    need = da.kv_workspace_size(4096, 2, 128, 16, 4, 64)
    assert need > da.KV_SCRATCH_BYTES
    # no path fits the scratch: the split-KV path is the only one below 4
    # query rows
    assert da.kv_plan(4096, 2, 128, 16, 4, 64, workspace_bytes=da.KV_SCRATCH_BYTES) == (0, need)
    assert da.kv_workspace_size(64, 1, 4096, 16, 4, 64) <= da.KV_SCRATCH_BYTES
    # with 4 query rows the prefill kernel alone (no scratch) takes over
    assert da.kv_workspace_size(4096, 4, 128, 16, 4, 64) > da.KV_SCRATCH_BYTES
    assert da.kv_plan(4096, 4, 128, 16, 4, 64, workspace_bytes=da.KV_SCRATCH_BYTES) == (1, 0)


@pytest.mark.parametrize("nseq,mq,mk,H,Hkv,d,path", [
    (8, 1024, 4096, 16, 4, 64, 1),   # chunked prefill of the 8 x 4096 prompts
    (8, 4096, 4096, 16, 4, 64, 1),   # the whole prompt as one chunk
    (5, 257, 1100, 12, 4, 64, 1),    # G = 3
    (1, 1024, 32768, 16, 4, 64, 2),  # one long context: too few query tiles
    (1, 64, 32768, 16, 4, 64, 2),
    (8, 64, 4096, 16, 4, 64, 2),
    (8, 16, 4096, 16, 4, 64, 2),     # speculative tokens
    (8, 128, 4096, 8, 8, 64, 2),     # G = 1
])
def test_long_chunks_take_the_prefill_kernel(nseq, mq, mk, H, Hkv, d, path):
    """Query chunks whose split-KV cost (rows x keys) outweighs the prefill
    kernel's run on it: over whole key ranges when the grid fills the GPU,
    else over key splits."""
    assert da.kv_path(nseq, mq, mk, H, Hkv, d) == path


@pytest.mark.parametrize("nseq,mq,mk,H,Hkv,d,Tq,Tk", [
    (8, 1, 4097, 16, 4, 64, None, None),     # decode steps
    (64, 1, 8192, 16, 4, 64, None, None),
    (32, 4, 31196, 16, 4, 64, 128, 539306),  # the varlen step: its cache total
    (8, 3, 4096, 16, 4, 64, None, None),     # below 4 query rows
    (8, 16, 4096, 16, 4, 64, 16, 32768),     # a loose bound on 2 queries each
    (4096, 4, 128, 16, 4, 64, None, None),
])
def test_decode_shapes_keep_the_split_path(nseq, mq, mk, H, Hkv, d, Tq, Tk):
    assert da.kv_path(nseq, mq, mk, H, Hkv, d, Tq=Tq, Tk=Tk) == 0
    assert da.kv_workspace_size(nseq, mq, mk, H, Hkv, d) > 0


def test_kv_path_rejects_what_the_call_rejects():
    assert da.kv_path(8, 64, 4096, 16, 5, 64) == -1    # H % Hkv
    assert da.kv_path(8, 64, 4096, 16, 4, 16) == -1    # d not compiled
    assert da.kv_path(0, 64, 4096, 16, 4, 64) == -1
    assert da.kv_path(8, 64, 4096, 16, 4, 64, Tq=0) == -1


def call_kv_on_path(path, **over):
    a = dict(dtype=da.BF16, q=FAKE, k=FAKE, v=FAKE, lq1=FAKE, lk1=FAKE,
             lq2=FAKE, lk2=FAKE, lambda_stride=0, lambda_init_value=0.7,
             subln_weight=0, eps=1e-5, causal=1, cu_seqlens_q=0,
             cu_seqlens_k=0, nseq=8, max_seqlen_q=0, max_seqlen_k=0, Tq=8 * 64,
             Tk=8 * 4096, H=16, Hkv=4, d=64, rope_cos=0, rope_sin=0,
             rope_len=0, rope_dtype=0, workspace=FAKE,
             workspace_bytes=1 << 30, out=FAKE, stream=0)
    a.update(over)
    return da.fwd_kv_on_path_ptr(path, **a)


@pytest.mark.parametrize("path,over,status", [
    (3, {}, da.EINVAL),                      # no such path
    (-2, {}, da.EINVAL),
    (2, dict(Tk=8 * 200), da.EINVAL),        # 200 keys: nothing to split
    (0, dict(workspace_bytes=64), da.EINVAL),
    (2, dict(workspace_bytes=64), da.EINVAL),
    (1, dict(dtype=da.F32), da.EUNSUPPORTED),
    (1, dict(Tq=0, q=0, out=0), da.OK),      # no query rows
])
def test_kv_on_path_validation_before_any_device_work(path, over, status):
    assert call_kv_on_path(path, **over) == status


def test_path_workspace_sizes():
    assert da.kv_path_workspace_size(1, 8, 64, 4096, 16, 4, 64) == 0
    assert da.kv_path_workspace_size(0, 8, 64, 4096, 16, 4, 64) > 0
    assert da.kv_path_workspace_size(2, 8, 64, 4096, 16, 4, 64) > 0
    assert da.kv_path_workspace_size(2, 8, 64, 200, 16, 4, 64) == 0   # nothing to split
    assert da.kv_path_workspace_size(3, 8, 64, 4096, 16, 4, 64) == 0


@pytest.mark.parametrize("d", [64, 32])
def test_workspace_of_the_bounds_serves_every_call_within_them(d):
    """A workspace of kv_workspace_size(bounds) bytes fits the plan of
    every call with smaller bounds: the call takes the cheapest plan whose
    partials fit, which is its first choice whenever that fits."""
    H, Hkv = 16, 4
    changed = 0
    for nseq in (1, 2, 3, 8):
        for Mq, Mk in ((4, 4096), (64, 8192), (100, 8192), (100, 32768), (1024, 4096),
                       (2048, 32768)):
            W = da.kv_workspace_size(nseq, Mq, Mk, H, Hkv, d)
            for mq in (1, 3, 4, 5, 16, 33, 64, 100, 512, 1024, 2048):
                for mk in (mq, 256, 257, 1000, 4096, 4097, 8192, 16384, 32768):
                    if mq > Mq or mk > Mk or mk < mq:
                        continue
                    path, need = da.kv_plan(nseq, mq, mk, H, Hkv, d, workspace_bytes=W)
                    first = da.kv_plan(nseq, mq, mk, H, Hkv, d)
                    assert path in (0, 1, 2) and need <= W, (nseq, Mq, Mk, mq, mk)
                    if first[1] <= W:
                        assert (path, need) == first
                    else:
                        changed += 1
    # (some calls within the bounds do want more than the bounds' own plan)
    assert changed > 0


def test_plan_follows_the_workspace_given():
    # one 32768-key context's last 1024 queries: key splits first choice
    first = da.kv_plan(1, 1024, 32768, 16, 4, 64)
    assert first[0] == 2 and first[1] > 0
    # with no workspace: the prefill kernel alone
    assert da.kv_plan(1, 1024, 32768, 16, 4, 64, workspace_bytes=0) == (1, 0)
    # with half the first choice's bytes: another split plan that fits
    path, need = da.kv_plan(1, 1024, 32768, 16, 4, 64, workspace_bytes=first[1] // 2)
    assert path in (1, 2) and need <= first[1] // 2
    # decode keeps the split-KV path whatever the workspace; its need is
    # reported even when the workspace is smaller (the call refuses it)
    dec = da.kv_plan(8, 1, 4097, 16, 4, 64)
    assert dec[0] == 0 and dec[1] == da.kv_workspace_size(8, 1, 4097, 16, 4, 64)
    assert da.kv_plan(8, 1, 4097, 16, 4, 64, workspace_bytes=0) == dec


def test_workspace_bound_covers_either_path():
    """The workspace bound holds the split-KV plan and, where a call within
    the bounds may run on key splits, that plan too."""
    from_split_only = da.kv_workspace_size(8, 3, 4096, 16, 4, 64)
    assert da.kv_workspace_size(8, 64, 4096, 16, 4, 64) >= from_split_only


# --------------------------------------------------------------------------
# training forward and backward

def test_supported_bwd_and_workspace():
    import torch
    for dt in (torch.bfloat16, torch.float32):
        for d in (16, 32, 64):
            assert da.supported_bwd(dt, d)
        assert not da.supported_bwd(dt, 48)
    assert not da.library().diffattn_supported_bwd(9, 64)
    bf, f32 = torch.bfloat16, torch.float32
    assert da.bwd_workspace_size(bf, 4096, 16, 64) > da.bwd_workspace_size(bf, 1024, 16, 64) > 0
    assert da.bwd_workspace_size(bf, -1, 16, 64) == 0
    assert da.bwd_workspace_size(f32, 1024, 16, 48) == 0
    # the exact path (fp32, and bf16 at d = 16) keeps dpre [T, H, 2d] in fp32,
    # the MFMA path in bf16
    assert (da.bwd_workspace_size(f32, 1024, 16, 64) - da.bwd_workspace_size(bf, 1024, 16, 64)
            == 1024 * 16 * 128 * 2)
    assert da.bwd_workspace_size(bf, 1024, 16, 16) == da.bwd_workspace_size(f32, 1024, 16, 16)


def call_bwd(**over):
    a = [da.BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0.3, None, 1e-5, 1,
         None, 2, 0, 64, 16, 4, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
         FAKE, FAKE, None, FAKE, 1 << 30, None]
    names = ["dtype", "q", "k", "v", "lq1", "lk1", "lq2", "lk2", "lstride",
             "lam", "w", "eps", "causal", "cu", "nseq", "max_seqlen", "T", "H",
             "Hkv", "d", "dout", "lse", "o12", "dq", "dk", "dv", "dlq1", "dlk1",
             "dlq2", "dlk2", "dw", "ws", "ws_bytes", "stream"]
    for k2, v2 in over.items():
        a[names.index(k2)] = v2
    return da.library().diffattn_bwd(*a)


@pytest.mark.parametrize("over,status", [
    (dict(dtype=9), da.EINVAL),
    (dict(dtype=da.F32, d=48), da.EUNSUPPORTED),
    (dict(d=48), da.EUNSUPPORTED),
    (dict(d=128), da.EUNSUPPORTED),
    (dict(H=6), da.EINVAL),
    (dict(H=512, Hkv=4), da.EINVAL),            # more heads than supported
    (dict(causal=3), da.EINVAL),
    (dict(lstride=10), da.EINVAL),
    (dict(T=63), da.EINVAL),                    # T % nseq
    (dict(dq=None), da.EINVAL),
    (dict(dlk2=None), da.EINVAL),
    (dict(o12=FAKE + 4), da.EINVAL),            # alignment
    (dict(ws_bytes=100), da.EINVAL),
    (dict(T=0, q=None, k=None, v=None), da.OK),  # nothing to do
])
def test_bwd_validation_before_any_device_work(over, status):
    assert call_bwd(**over) == status


def test_fwd_train_validation():
    lib = da.library()
    args = [da.BF16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0.3, None, 1e-5, 1,
            None, 2, 0, 64, 16, 4, 64, FAKE, None, FAKE, None]
    assert lib.diffattn_fwd_train(*args) == da.EINVAL           # lse missing
    args[21] = FAKE
    args[22] = FAKE + 4
    assert lib.diffattn_fwd_train(*args) == da.EINVAL           # o12 misaligned
