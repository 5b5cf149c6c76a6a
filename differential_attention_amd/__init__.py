"""Python binding of libdiffattn, the MI355X differential-attention forward.

Argument marshalling only: tensors become device pointers and sizes, the
stream comes from torch, and every step of the computation runs in the HIP
kernels of ``libdiffattn.so`` behind the C ABI declared in
``include/diffattn.h``.  PyTorch is used for device memory and streams.

There is no fallback: if the library is missing, or the call fails, this
module raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["fwd", "fwd_ptr", "fwd_workspace_size", "fwd_kv", "fwd_kv_ptr", "kv_workspace_size",
           "kv_path", "kv_plan", "KV_PATH_SPLIT_KV", "KV_PATH_PREFILL",
           "KV_PATH_PREFILL_SPLIT", "fwd_kv_on_path_ptr", "kv_path_workspace_size",
           "fwd_kv_noalloc", "fwd_kv_noalloc_ptr", "KV_SCRATCH_BYTES",
           "fwd_train", "bwd", "bwd_workspace_size", "supported_bwd",
           "kv_append", "kv_append_ptr", "diff_attention", "DiffAttnFunction",
           "lambda_init", "supported", "supported_kv", "check_cu_seqlens",
           "check_cu_seqlens_kv", "library", "LIBRARY", "DiffAttnError",
           "BF16", "F32"]

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libdiffattn.so")

OK, EINVAL, EUNSUPPORTED, EHIP, ETOOLARGE = 0, -1, -2, -3, -4
# size of the static device array behind diffattn_fwd_kv_noalloc
# (DIFFATTN_KV_SCRATCH_BYTES in include/diffattn.h)
KV_SCRATCH_BYTES = 32 << 20
BF16, F32 = 0, 1
_DTYPES = {torch.bfloat16: BF16, torch.float32: F32}


class DiffAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


_lib: Optional[ctypes.CDLL] = None


def library() -> ctypes.CDLL:
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise RuntimeError(
            f"{LIBRARY} is missing: build it with "
            "`python differential_attention_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIBRARY)
    vp, f32p, i32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.diffattn_fwd.argtypes = [
        ctypes.c_int, vp, vp, vp, f32p, f32p, f32p, f32p, i32, ctypes.c_float,
        f32p, ctypes.c_float, ctypes.c_int, i32p, i32, i32, i32, i32, i32, i32,
        vp, vp, i32, ctypes.c_int, vp, ctypes.c_size_t, vp, vp]
    lib.diffattn_fwd_workspace_size.argtypes = [ctypes.c_int, i32, i32, i32, ctypes.c_int]
    lib.diffattn_fwd_workspace_size.restype = ctypes.c_size_t
    lib.diffattn_fwd.restype = ctypes.c_int
    lib.diffattn_fwd_kv.argtypes = [
        ctypes.c_int, vp, vp, vp, f32p, f32p, f32p, f32p, i32, ctypes.c_float,
        f32p, ctypes.c_float, ctypes.c_int, i32p, i32p, i32, i32, i32, i32,
        i32, i32, i32, i32, vp, vp, i32, ctypes.c_int, vp, ctypes.c_size_t,
        vp, vp]
    lib.diffattn_fwd_kv.restype = ctypes.c_int
    lib.diffattn_fwd_kv_on_path.argtypes = [ctypes.c_int] + lib.diffattn_fwd_kv.argtypes
    lib.diffattn_fwd_kv_on_path.restype = ctypes.c_int
    lib.diffattn_fwd_kv_path_workspace_size.argtypes = [ctypes.c_int] + [i32] * 6
    lib.diffattn_fwd_kv_path_workspace_size.restype = ctypes.c_size_t
    lib.diffattn_fwd_kv_noalloc.argtypes = [
        ctypes.c_int, vp, vp, vp, f32p, f32p, f32p, f32p, i32, ctypes.c_float,
        f32p, ctypes.c_float, ctypes.c_int, i32p, i32p, i32, i32, i32, i32,
        i32, i32, i32, i32, vp, vp, i32, ctypes.c_int, vp, vp]
    lib.diffattn_fwd_kv_noalloc.restype = ctypes.c_int
    lib.diffattn_kv_append.argtypes = [
        ctypes.c_int, vp, vp, i32p, i32p, i32, i32, i32, i32, i32, i32,
        vp, vp, i32, ctypes.c_int, vp, vp, vp]
    lib.diffattn_kv_append.restype = ctypes.c_int
    lib.diffattn_fwd_kv_workspace_size.argtypes = [i32] * 6
    lib.diffattn_fwd_kv_workspace_size.restype = ctypes.c_size_t
    lib.diffattn_fwd_kv_path.argtypes = [i32] * 8 + [ctypes.c_size_t,
                                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.diffattn_fwd_kv_path.restype = ctypes.c_int
    lib.diffattn_supported_kv.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.diffattn_supported_kv.restype = ctypes.c_int
    lib.diffattn_check_cu_seqlens_kv.argtypes = [
        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32), i32,
        i32, i32, i32, i32, ctypes.c_int]
    lib.diffattn_check_cu_seqlens_kv.restype = ctypes.c_int
    lib.diffattn_fwd_train.argtypes = [
        ctypes.c_int, vp, vp, vp, f32p, f32p, f32p, f32p, i32, ctypes.c_float,
        f32p, ctypes.c_float, ctypes.c_int, i32p, i32, i32, i32, i32, i32, i32,
        vp, vp, vp, vp]
    lib.diffattn_fwd_train.restype = ctypes.c_int
    lib.diffattn_bwd.argtypes = [
        ctypes.c_int, vp, vp, vp, f32p, f32p, f32p, f32p, i32, ctypes.c_float,
        f32p, ctypes.c_float, ctypes.c_int, i32p, i32, i32, i32, i32, i32, i32,
        vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.diffattn_bwd.restype = ctypes.c_int
    lib.diffattn_bwd_workspace_size.argtypes = [ctypes.c_int, i32, i32, i32]
    lib.diffattn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.diffattn_supported_bwd.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.diffattn_supported_bwd.restype = ctypes.c_int
    lib.diffattn_lambda_init.argtypes = [ctypes.c_int]
    lib.diffattn_lambda_init.restype = ctypes.c_double
    lib.diffattn_supported.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.diffattn_supported.restype = ctypes.c_int
    lib.diffattn_check_cu_seqlens.argtypes = [ctypes.POINTER(ctypes.c_int32),
                                              i32, i32, i32]
    lib.diffattn_check_cu_seqlens.restype = ctypes.c_int
    lib.diffattn_strerror.argtypes = [ctypes.c_int]
    lib.diffattn_strerror.restype = ctypes.c_char_p
    lib.diffattn_abi_version.argtypes = []
    lib.diffattn_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return library().diffattn_strerror(int(status)).decode()


def lambda_init(depth: int) -> float:
    """Initial lambda of a layer at 1-based ``depth`` (computed by the
    library)."""
    return float(library().diffattn_lambda_init(int(depth)))


def supported(dtype: torch.dtype, d: int) -> bool:
    return bool(library().diffattn_supported(_DTYPES[dtype], int(d)))


def check_cu_seqlens(cu_host, T: int, max_seqlen: int) -> bool:
    """Host-side precondition check of a CPU copy of cu_seqlens."""
    cu = torch.as_tensor(cu_host, dtype=torch.int32).contiguous().cpu()
    ptr = ctypes.cast(cu.data_ptr(), ctypes.POINTER(ctypes.c_int32))
    return library().diffattn_check_cu_seqlens(ptr, cu.numel() - 1, int(T),
                                               int(max_seqlen)) == OK


def supported_kv(dtype: torch.dtype, d: int) -> bool:
    return bool(library().diffattn_supported_kv(_DTYPES[dtype], int(d)))


def check_cu_seqlens_kv(cu_q_host, cu_k_host, Tq: int, Tk: int,
                        max_seqlen_q: int, max_seqlen_k: int,
                        causal: bool = True) -> bool:
    """Host-side precondition check of CPU copies of both boundaries."""
    cq = torch.as_tensor(cu_q_host, dtype=torch.int32).contiguous().cpu()
    ck = torch.as_tensor(cu_k_host, dtype=torch.int32).contiguous().cpu()
    if cq.numel() != ck.numel():
        return False
    P = ctypes.POINTER(ctypes.c_int32)
    return library().diffattn_check_cu_seqlens_kv(
        ctypes.cast(cq.data_ptr(), P), ctypes.cast(ck.data_ptr(), P),
        cq.numel() - 1, int(Tq), int(Tk), int(max_seqlen_q),
        int(max_seqlen_k), int(bool(causal))) == OK


def kv_workspace_size(nseq: int, max_seqlen_q: int, max_seqlen_k: int,
                      H: int, Hkv: int, d: int) -> int:
    """Bytes of device workspace ``fwd_kv`` needs (0: sizes rejected)."""
    return int(library().diffattn_fwd_kv_workspace_size(
        int(nseq), int(max_seqlen_q), int(max_seqlen_k), int(H), int(Hkv),
        int(d)))


# the kernels fwd_kv runs (kv_path)
KV_PATH_SPLIT_KV = 0       # split-KV partial kernel + combine kernel
KV_PATH_PREFILL = 1        # the prefill kernel alone (no workspace)
KV_PATH_PREFILL_SPLIT = 2  # the prefill kernel on key splits + combine kernel


def kv_plan(nseq: int, max_seqlen_q: int, max_seqlen_k: int, H: int, Hkv: int,
            d: int, Tq: Optional[int] = None, Tk: Optional[int] = None,
            workspace_bytes: Optional[int] = None) -> tuple:
    """(path, bytes): the kernels ``fwd_kv`` runs for these bounds and totals
    given a workspace of ``workspace_bytes`` (None: as large as the
    library's first choice needs), and the workspace bytes that plan uses
    (KV_PATH_*; path -1: sizes rejected).  Tq and Tk default to nseq equal
    sequences."""
    Tq = nseq * max_seqlen_q if Tq is None else Tq
    Tk = nseq * max_seqlen_k if Tk is None else Tk
    cap = (1 << 64) - 1 if workspace_bytes is None else int(workspace_bytes)
    need = ctypes.c_size_t(0)
    path = int(library().diffattn_fwd_kv_path(
        int(nseq), int(max_seqlen_q), int(max_seqlen_k), int(Tq), int(Tk), int(H), int(Hkv),
        int(d), cap, ctypes.byref(need)))
    return path, int(need.value)


def kv_path(nseq: int, max_seqlen_q: int, max_seqlen_k: int, H: int, Hkv: int,
            d: int, Tq: Optional[int] = None, Tk: Optional[int] = None,
            workspace_bytes: Optional[int] = None) -> int:
    """Which kernels ``fwd_kv`` runs (the path of ``kv_plan``)."""
    return kv_plan(nseq, max_seqlen_q, max_seqlen_k, H, Hkv, d, Tq, Tk, workspace_bytes)[0]


def fwd_kv_ptr(dtype: int, q: int, k: int, v: int, lq1: int, lk1: int,
               lq2: int, lk2: int, lambda_stride: int,
               lambda_init_value: float, subln_weight: int, eps: float,
               causal: int, cu_seqlens_q: int, cu_seqlens_k: int, nseq: int,
               max_seqlen_q: int, max_seqlen_k: int, Tq: int, Tk: int, H: int,
               Hkv: int, d: int, rope_cos: int, rope_sin: int, rope_len: int,
               rope_dtype: int, workspace: int, workspace_bytes: int,
               out: int, stream: int) -> int:
    """The raw cache entry point on integer device addresses; returns the
    status."""
    return library().diffattn_fwd_kv(
        int(dtype), q or None, k or None, v or None, lq1 or None, lk1 or None,
        lq2 or None, lk2 or None, int(lambda_stride), float(lambda_init_value),
        subln_weight or None, float(eps), int(causal), cu_seqlens_q or None,
        cu_seqlens_k or None, int(nseq), int(max_seqlen_q), int(max_seqlen_k),
        int(Tq), int(Tk), int(H), int(Hkv), int(d), rope_cos or None,
        rope_sin or None, int(rope_len), int(rope_dtype), workspace or None,
        int(workspace_bytes), out or None, stream or None)


def fwd_kv_on_path_ptr(path: int, dtype: int, q: int, k: int, v: int, lq1: int, lk1: int,
                       lq2: int, lk2: int, lambda_stride: int,
                       lambda_init_value: float, subln_weight: int, eps: float,
                       causal: int, cu_seqlens_q: int, cu_seqlens_k: int, nseq: int,
                       max_seqlen_q: int, max_seqlen_k: int, Tq: int, Tk: int, H: int,
                       Hkv: int, d: int, rope_cos: int, rope_sin: int, rope_len: int,
                       rope_dtype: int, workspace: int, workspace_bytes: int,
                       out: int, stream: int) -> int:
    """diffattn_fwd_kv_on_path on integer device addresses; returns the
    status."""
    return library().diffattn_fwd_kv_on_path(
        int(path), int(dtype), q or None, k or None, v or None, lq1 or None, lk1 or None,
        lq2 or None, lk2 or None, int(lambda_stride), float(lambda_init_value),
        subln_weight or None, float(eps), int(causal), cu_seqlens_q or None,
        cu_seqlens_k or None, int(nseq), int(max_seqlen_q), int(max_seqlen_k),
        int(Tq), int(Tk), int(H), int(Hkv), int(d), rope_cos or None,
        rope_sin or None, int(rope_len), int(rope_dtype), workspace or None,
        int(workspace_bytes), out or None, stream or None)


def kv_path_workspace_size(path: int, nseq: int, max_seqlen_q: int, max_seqlen_k: int,
                           H: int, Hkv: int, d: int) -> int:
    """Bytes of device workspace ``fwd_kv(path=...)`` needs (0: path 1, or
    sizes rejected)."""
    return int(library().diffattn_fwd_kv_path_workspace_size(
        int(path), int(nseq), int(max_seqlen_q), int(max_seqlen_k), int(H), int(Hkv),
        int(d)))


def fwd_kv_noalloc_ptr(dtype: int, q: int, k: int, v: int, lq1: int,
                       lk1: int, lq2: int, lk2: int, lambda_stride: int,
                       lambda_init_value: float, subln_weight: int,
                       eps: float, causal: int, cu_seqlens_q: int,
                       cu_seqlens_k: int, nseq: int, max_seqlen_q: int,
                       max_seqlen_k: int, Tq: int, Tk: int, H: int, Hkv: int,
                       d: int, rope_cos: int, rope_sin: int, rope_len: int,
                       rope_dtype: int, out: int, stream: int) -> int:
    """The raw no-allocation cache entry point (static device scratch) on
    integer device addresses; returns the status."""
    return library().diffattn_fwd_kv_noalloc(
        int(dtype), q or None, k or None, v or None, lq1 or None, lk1 or None,
        lq2 or None, lk2 or None, int(lambda_stride), float(lambda_init_value),
        subln_weight or None, float(eps), int(causal), cu_seqlens_q or None,
        cu_seqlens_k or None, int(nseq), int(max_seqlen_q), int(max_seqlen_k),
        int(Tq), int(Tk), int(H), int(Hkv), int(d), rope_cos or None,
        rope_sin or None, int(rope_len), int(rope_dtype), out or None,
        stream or None)


def kv_append_ptr(dtype: int, k_new: int, v_new: int, cu_seqlens_q: int,
                  cu_seqlens_k: int, nseq: int, max_seqlen_k: int, Tq: int,
                  Tk: int, Hkv: int, d: int, rope_cos: int, rope_sin: int,
                  rope_len: int, rope_dtype: int, k_cache: int, v_cache: int,
                  stream: int) -> int:
    """The raw cache-update entry point on integer device addresses;
    returns the status."""
    return library().diffattn_kv_append(
        int(dtype), k_new or None, v_new or None, cu_seqlens_q or None,
        cu_seqlens_k or None, int(nseq), int(max_seqlen_k), int(Tq), int(Tk),
        int(Hkv), int(d), rope_cos or None, rope_sin or None, int(rope_len),
        int(rope_dtype), k_cache or None, v_cache or None, stream or None)


def fwd_ptr(dtype: int, q: int, k: int, v: int, lq1: int, lk1: int, lq2: int,
            lk2: int, lambda_stride: int, lambda_init_value: float,
            subln_weight: int, eps: float, causal: int, cu_seqlens: int,
            nseq: int, max_seqlen: int, T: int, H: int, Hkv: int, d: int,
            rope_cos: int, rope_sin: int, rope_len: int, rope_dtype: int,
            workspace: int, workspace_bytes: int, out: int, stream: int) -> int:
    """The raw C entry point on integer device addresses; returns the
    status."""
    return library().diffattn_fwd(
        int(dtype), q or None, k or None, v or None, lq1 or None, lk1 or None,
        lq2 or None, lk2 or None, int(lambda_stride), float(lambda_init_value),
        subln_weight or None, float(eps), int(causal), cu_seqlens or None,
        int(nseq), int(max_seqlen), int(T), int(H), int(Hkv), int(d),
        rope_cos or None, rope_sin or None, int(rope_len), int(rope_dtype),
        workspace or None, int(workspace_bytes), out or None, stream or None)


def fwd_workspace_size(dtype: torch.dtype, T: int, Hkv: int, d: int,
                       rope: bool) -> int:
    """Bytes of workspace ``fwd`` needs (the rotated K when ``rope``)."""
    return int(library().diffattn_fwd_workspace_size(
        _DTYPES[dtype], int(T), int(Hkv), int(d), int(bool(rope))))


def _dev(t: torch.Tensor, name: str, device, dtype=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
        lambda_q1: torch.Tensor, lambda_k1: torch.Tensor,
        lambda_q2: torch.Tensor, lambda_k2: torch.Tensor,
        lambda_init: float, subln_weight: Optional[torch.Tensor] = None,
        eps: float = 1e-5, causal: bool = True,
        cu_seqlens: Optional[torch.Tensor] = None,
        max_seqlen: Optional[int] = None, nseq: Optional[int] = None,
        out: Optional[torch.Tensor] = None,
        stream: Optional[torch.cuda.Stream] = None,
        rope: Optional[tuple] = None,
        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Differential-attention forward on the GPU.

    q [T, H, 2, d], k [T, Hkv, 2, d], v [T, Hkv, 2d] (bf16 or fp32, one
    device); lambda vectors fp32 [d] (one set for all heads) or [H, d] (one
    set per head); subln_weight fp32 [2d] or None;
    cu_seqlens int32 [nseq + 1] on the device, or None for ``nseq`` (default
    1) sequences of equal length.  ``max_seqlen`` bounds every sequence
    length; when cu_seqlens is given without it, it is read back from the
    device (a synchronising copy).  ``rope`` = (cos, sin) fp32 device tables
    [len, d/2] applies the interleaved rotary prologue to q and k in the
    kernel (positions restart in every sequence); it needs a device uint8
    ``workspace`` of ``fwd_workspace_size(...)`` bytes for the rotated K,
    allocated through torch when None.  Returns ``out`` [T, H, 2d].
    """
    if q.dim() != 4 or q.shape[2] != 2:
        raise ValueError("q must be [T, H, 2, d]")
    T, H, _, d = q.shape
    if k.dim() != 4 or k.shape[0] != T or k.shape[2:] != (2, d):
        raise ValueError("k must be [T, Hkv, 2, d]")
    Hkv = k.shape[1]
    if tuple(v.shape) != (T, Hkv, 2 * d):
        raise ValueError("v must be [T, Hkv, 2d]")
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    args = [_dev(q, "q", dev), _dev(k, "k", dev, q.dtype),
            _dev(v, "v", dev, q.dtype)]
    per_head = lambda_q1.dim() == 2
    for name, lv in (("lambda_q1", lambda_q1), ("lambda_k1", lambda_k1),
                     ("lambda_q2", lambda_q2), ("lambda_k2", lambda_k2)):
        want = (H, d) if per_head else (d,)
        if tuple(lv.shape) != want:
            raise ValueError(f"{name} must be {list(want)}")
        args.append(_dev(lv, name, dev, torch.float32))
    lambda_stride = d if per_head else 0
    w_ptr = 0
    if subln_weight is not None:
        if subln_weight.numel() != 2 * d:
            raise ValueError("subln_weight must have 2d elements")
        w_ptr = _dev(subln_weight, "subln_weight", dev, torch.float32)
    cu_ptr = 0
    if cu_seqlens is not None:
        cu_ptr = _dev(cu_seqlens, "cu_seqlens", dev, torch.int32)
        nseq = cu_seqlens.numel() - 1
        if max_seqlen is None:
            cu_host = cu_seqlens.cpu()
            max_seqlen = int((cu_host[1:] - cu_host[:-1]).max()) if nseq > 0 else 0
    else:
        nseq = 1 if nseq is None else int(nseq)
        if max_seqlen is None:
            max_seqlen = T // nseq if nseq > 0 else 0
    rc_ptr = rs_ptr = rope_len = rope_dtype = ws_ptr = ws_bytes = 0
    if rope is not None:
        rc_ptr, rs_ptr, rope_len, rope_dtype = _rope_args(rope, d, dev)
        if workspace is None:
            workspace = torch.empty(max(fwd_workspace_size(q.dtype, T, Hkv, d, True), 16),
                                    dtype=torch.uint8, device=dev)
        ws_ptr = _dev(workspace, "workspace", dev)
        ws_bytes = workspace.numel()
    if out is None:
        out = torch.empty((T, H, 2 * d), dtype=q.dtype, device=dev)
    elif tuple(out.shape) != (T, H, 2 * d):
        raise ValueError("out must be [T, H, 2d]")
    out_ptr = _dev(out, "out", dev, q.dtype)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = fwd_ptr(_DTYPES[q.dtype], args[0], args[1], args[2], args[3],
                     args[4], args[5], args[6], lambda_stride, lambda_init,
                     w_ptr, eps,
                     int(bool(causal)), cu_ptr, nseq, max_seqlen, T, H, Hkv, d,
                     rc_ptr, rs_ptr, rope_len, rope_dtype, ws_ptr, ws_bytes,
                     out_ptr, stream.cuda_stream)
    if st != OK:
        raise DiffAttnError(st, "diffattn_fwd")
    return out


def _rope_args(rope, d, dev):
    """(cos, sin) tables [len, d/2], both fp32 or both bf16, on the device:
    their pointers, length and DIFFATTN dtype."""
    rc, rs = rope
    if rc.dim() != 2 or rc.shape[1] != d // 2 or tuple(rs.shape) != tuple(rc.shape):
        raise ValueError("rope tables must be two [len, d/2] tensors")
    if rc.dtype not in _DTYPES or rs.dtype != rc.dtype:
        raise ValueError("rope tables must both be float32 or both bfloat16")
    return (_dev(rc, "rope cos", dev, rc.dtype), _dev(rs, "rope sin", dev, rc.dtype),
            rc.shape[0], _DTYPES[rc.dtype])


def _lambda_args(lvs, H, d, dev):
    per_head = lvs[0].dim() == 2
    ptrs = []
    for name, lv in zip(("lambda_q1", "lambda_k1", "lambda_q2", "lambda_k2"), lvs):
        want = (H, d) if per_head else (d,)
        if tuple(lv.shape) != want:
            raise ValueError(f"{name} must be {list(want)}")
        ptrs.append(_dev(lv, name, dev, torch.float32))
    return ptrs, (d if per_head else 0)


def fwd_kv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
           lambda_q1: torch.Tensor, lambda_k1: torch.Tensor,
           lambda_q2: torch.Tensor, lambda_k2: torch.Tensor,
           lambda_init: float, subln_weight: Optional[torch.Tensor] = None,
           eps: float = 1e-5, causal: bool = True,
           cu_seqlens_q: Optional[torch.Tensor] = None,
           cu_seqlens_k: Optional[torch.Tensor] = None,
           max_seqlen_q: Optional[int] = None,
           max_seqlen_k: Optional[int] = None, nseq: Optional[int] = None,
           workspace: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None,
           stream: Optional[torch.cuda.Stream] = None,
           rope: Optional[tuple] = None, path: Optional[int] = None) -> torch.Tensor:
    """New queries against a key/value cache on the GPU (bottom-right causal).

    q [Tq, H, 2, d]; k [Tk, Hkv, 2, d], v [Tk, Hkv, 2d] (bf16); lambda
    vectors fp32 [d] or [H, d]; cu_seqlens_q / cu_seqlens_k int32
    [nseq + 1] on the device, both or neither (neither: ``nseq`` equal
    sequences).  When the bounds are not given they are read back from the
    device (a synchronising copy).  ``workspace`` is a device uint8 tensor of
    at least ``kv_workspace_size(...)`` bytes; one is allocated through
    torch when it is None and the call needs one (``kv_path``: not on the
    prefill kernel alone).  ``rope`` = (cos, sin) device tables [len, d/2]
    (fp32 or bf16) rotates each new query at its absolute position
    nk - nq + i; the cached keys are taken as already rotated (``kv_append``
    writes them so).  ``path`` (KV_PATH_*) runs those kernels instead of the
    library's choice (diffattn_fwd_kv_on_path).  Returns ``out`` [Tq, H, 2d].
    """
    return _kv_call(q, k, v, (lambda_q1, lambda_k1, lambda_q2, lambda_k2),
                    lambda_init, subln_weight, eps, causal, cu_seqlens_q,
                    cu_seqlens_k, max_seqlen_q, max_seqlen_k, nseq, out,
                    stream, workspace, noalloc=False, rope=rope, path=path)


def fwd_kv_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   lambda_q1: torch.Tensor, lambda_k1: torch.Tensor,
                   lambda_q2: torch.Tensor, lambda_k2: torch.Tensor,
                   lambda_init: float,
                   subln_weight: Optional[torch.Tensor] = None,
                   eps: float = 1e-5, causal: bool = True,
                   cu_seqlens_q: Optional[torch.Tensor] = None,
                   cu_seqlens_k: Optional[torch.Tensor] = None,
                   max_seqlen_q: Optional[int] = None,
                   max_seqlen_k: Optional[int] = None,
                   nseq: Optional[int] = None,
                   out: Optional[torch.Tensor] = None,
                   stream: Optional[torch.cuda.Stream] = None,
                   rope: Optional[tuple] = None) -> torch.Tensor:
    """``fwd_kv`` through ``diffattn_fwd_kv_noalloc``: the library's static
    device scratch (``KV_SCRATCH_BYTES`` per GPU) replaces the workspace, so
    the call allocates nothing when ``out`` and both bounds are given.
    Calls overlapping in time on one GPU race on that scratch."""
    return _kv_call(q, k, v, (lambda_q1, lambda_k1, lambda_q2, lambda_k2),
                    lambda_init, subln_weight, eps, causal, cu_seqlens_q,
                    cu_seqlens_k, max_seqlen_q, max_seqlen_k, nseq, out,
                    stream, None, noalloc=True, rope=rope)


def _kv_call(q, k, v, lvs, lambda_init, subln_weight, eps, causal,
             cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, nseq,
             out, stream, workspace, noalloc, rope=None, path=None):
    if q.dim() != 4 or q.shape[2] != 2:
        raise ValueError("q must be [Tq, H, 2, d]")
    Tq, H, _, d = q.shape
    if k.dim() != 4 or k.shape[2:] != (2, d):
        raise ValueError("k must be [Tk, Hkv, 2, d]")
    Tk, Hkv = k.shape[0], k.shape[1]
    if tuple(v.shape) != (Tk, Hkv, 2 * d):
        raise ValueError("v must be [Tk, Hkv, 2d]")
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    qp, kp, vp_ = (_dev(q, "q", dev), _dev(k, "k", dev, q.dtype),
                   _dev(v, "v", dev, q.dtype))
    lptrs, lambda_stride = _lambda_args(lvs, H, d, dev)
    w_ptr = 0
    if subln_weight is not None:
        if subln_weight.numel() != 2 * d:
            raise ValueError("subln_weight must have 2d elements")
        w_ptr = _dev(subln_weight, "subln_weight", dev, torch.float32)
    if (cu_seqlens_q is None) != (cu_seqlens_k is None):
        raise ValueError("give both cu_seqlens_q and cu_seqlens_k, or neither")
    cq_ptr = ck_ptr = 0
    if cu_seqlens_q is not None:
        if cu_seqlens_q.numel() != cu_seqlens_k.numel():
            raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
        cq_ptr = _dev(cu_seqlens_q, "cu_seqlens_q", dev, torch.int32)
        ck_ptr = _dev(cu_seqlens_k, "cu_seqlens_k", dev, torch.int32)
        nseq = cu_seqlens_q.numel() - 1
        if max_seqlen_q is None:
            c = cu_seqlens_q.cpu()
            max_seqlen_q = int((c[1:] - c[:-1]).max()) if nseq > 0 else 0
        if max_seqlen_k is None:
            c = cu_seqlens_k.cpu()
            max_seqlen_k = int((c[1:] - c[:-1]).max()) if nseq > 0 else 0
    else:
        nseq = 1 if nseq is None else int(nseq)
        max_seqlen_q = Tq // nseq if nseq > 0 else 0
        max_seqlen_k = Tk // nseq if nseq > 0 else 0
    if not noalloc and path is not None:
        need = kv_path_workspace_size(path, nseq, max(max_seqlen_q, 1),
                                      max(max_seqlen_k, 1), H, Hkv, d)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_ptr = 0 if workspace is None else _dev(workspace, "workspace", dev)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    elif not noalloc:
        need = kv_workspace_size(nseq, max(max_seqlen_q, 1),
                                 max(max_seqlen_k, 1), H, Hkv, d)
        if workspace is None and (need == 0 or kv_path(
                nseq, max(max_seqlen_q, 1), max(max_seqlen_k, 1), H, Hkv, d,
                max(Tq, 1), max(Tk, 1)) == KV_PATH_PREFILL):
            ws_ptr, ws_bytes = 0, 0      # the prefill kernel alone: no workspace
        else:
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=dev)
            ws_ptr = _dev(workspace, "workspace", dev)
            ws_bytes = workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty((Tq, H, 2 * d), dtype=q.dtype, device=dev)
    elif tuple(out.shape) != (Tq, H, 2 * d):
        raise ValueError("out must be [Tq, H, 2d]")
    out_ptr = _dev(out, "out", dev, q.dtype)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    rargs = (0, 0, 0, 0) if rope is None else _rope_args(rope, d, dev)
    common = (_DTYPES[q.dtype], qp, kp, vp_, *lptrs, lambda_stride,
              lambda_init, w_ptr, eps, int(bool(causal)), cq_ptr, ck_ptr,
              nseq, max_seqlen_q, max_seqlen_k, Tq, Tk, H, Hkv, d, *rargs)
    with torch.cuda.device(dev):
        if noalloc:
            st = fwd_kv_noalloc_ptr(*common, out_ptr, stream.cuda_stream)
        elif path is not None:
            st = fwd_kv_on_path_ptr(path, *common, ws_ptr, ws_bytes, out_ptr,
                                    stream.cuda_stream)
        else:
            st = fwd_kv_ptr(*common, ws_ptr, ws_bytes, out_ptr,
                            stream.cuda_stream)
    if st != OK:
        raise DiffAttnError(st, "diffattn_fwd_kv_noalloc" if noalloc
                            else "diffattn_fwd_kv_on_path" if path is not None
                            else "diffattn_fwd_kv")
    return out


def kv_append(k_new: torch.Tensor, v_new: torch.Tensor,
              k_cache: torch.Tensor, v_cache: torch.Tensor,
              cu_seqlens_q: Optional[torch.Tensor] = None,
              cu_seqlens_k: Optional[torch.Tensor] = None,
              max_seqlen_k: Optional[int] = None, nseq: Optional[int] = None,
              rope: Optional[tuple] = None,
              stream: Optional[torch.cuda.Stream] = None) -> None:
    """The cache update of a decode step, in place: the nq new tokens of
    each sequence (k_new [Tq, Hkv, 2, d], v_new [Tq, Hkv, 2d]) go to the
    last nq rows of its region of k_cache [Tk, Hkv, 2, d] / v_cache
    [Tk, Hkv, 2d]; with ``rope`` = (cos, sin) the keys are rotated at their
    positions nk - nq + i.  Boundaries as for ``fwd_kv``."""
    if k_new.dim() != 4 or k_new.shape[2] != 2:
        raise ValueError("k_new must be [Tq, Hkv, 2, d]")
    Tq, Hkv, _, d = k_new.shape
    if tuple(v_new.shape) != (Tq, Hkv, 2 * d):
        raise ValueError("v_new must be [Tq, Hkv, 2d]")
    if k_cache.dim() != 4 or tuple(k_cache.shape[1:]) != (Hkv, 2, d):
        raise ValueError("k_cache must be [Tk, Hkv, 2, d]")
    Tk = k_cache.shape[0]
    if tuple(v_cache.shape) != (Tk, Hkv, 2 * d):
        raise ValueError("v_cache must be [Tk, Hkv, 2d]")
    if k_new.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {k_new.dtype}")
    dev = k_new.device
    dt = k_new.dtype
    ptrs = [_dev(k_new, "k_new", dev, dt), _dev(v_new, "v_new", dev, dt)]
    if (cu_seqlens_q is None) != (cu_seqlens_k is None):
        raise ValueError("give both cu_seqlens_q and cu_seqlens_k, or neither")
    cq_ptr = ck_ptr = 0
    if cu_seqlens_q is not None:
        if cu_seqlens_q.numel() != cu_seqlens_k.numel():
            raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
        cq_ptr = _dev(cu_seqlens_q, "cu_seqlens_q", dev, torch.int32)
        ck_ptr = _dev(cu_seqlens_k, "cu_seqlens_k", dev, torch.int32)
        nseq = cu_seqlens_q.numel() - 1
        if max_seqlen_k is None:
            c = cu_seqlens_k.cpu()
            max_seqlen_k = int((c[1:] - c[:-1]).max()) if nseq > 0 else 0
    else:
        nseq = 1 if nseq is None else int(nseq)
        max_seqlen_k = Tk // nseq if nseq > 0 else 0
    rargs = (0, 0, 0, 0) if rope is None else _rope_args(rope, d, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = kv_append_ptr(_DTYPES[dt], *ptrs, cq_ptr, ck_ptr, nseq, max_seqlen_k,
                           Tq, Tk, Hkv, d, *rargs, _dev(k_cache, "k_cache", dev, dt),
                           _dev(v_cache, "v_cache", dev, dt), stream.cuda_stream)
    if st != OK:
        raise DiffAttnError(st, "diffattn_kv_append")


def supported_bwd(dtype: torch.dtype, d: int) -> bool:
    return bool(library().diffattn_supported_bwd(_DTYPES[dtype], int(d)))


def bwd_workspace_size(dtype: torch.dtype, T: int, H: int, d: int) -> int:
    return int(library().diffattn_bwd_workspace_size(_DTYPES[dtype], int(T), int(H), int(d)))


def _seq_args(T, cu_seqlens, max_seqlen, nseq, dev):
    if cu_seqlens is not None:
        cu_ptr = _dev(cu_seqlens, "cu_seqlens", dev, torch.int32)
        nseq = cu_seqlens.numel() - 1
        if max_seqlen is None:
            c = cu_seqlens.cpu()
            max_seqlen = int((c[1:] - c[:-1]).max()) if nseq > 0 else 0
        return cu_ptr, nseq, max_seqlen
    nseq = 1 if nseq is None else int(nseq)
    return 0, nseq, (T // nseq if nseq > 0 else 0)


def fwd_train(q, k, v, lambda_q1, lambda_k1, lambda_q2, lambda_k2,
              lambda_init: float, subln_weight=None, eps: float = 1e-5,
              causal: bool = True, cu_seqlens=None, max_seqlen=None, nseq=None,
              stream=None):
    """Training forward: returns ``(out, lse, o12)`` where ``lse``
    [T, H, 2] and ``o12`` [T, H, 2, 2d] (fp32) are what ``bwd`` needs."""
    T, H, _, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    lptrs, lstride = _lambda_args((lambda_q1, lambda_k1, lambda_q2, lambda_k2), H, d, dev)
    w_ptr = 0 if subln_weight is None else _dev(subln_weight, "subln_weight", dev, torch.float32)
    cu_ptr, nseq, max_seqlen = _seq_args(T, cu_seqlens, max_seqlen, nseq, dev)
    out = torch.empty((T, H, 2 * d), dtype=q.dtype, device=dev)
    lse = torch.empty((T, H, 2), dtype=torch.float32, device=dev)
    o12 = torch.empty((T, H, 2, 2 * d), dtype=torch.float32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = library().diffattn_fwd_train(
            _DTYPES[q.dtype], _dev(q, "q", dev), _dev(k, "k", dev, q.dtype),
            _dev(v, "v", dev, q.dtype), *lptrs, lstride, float(lambda_init),
            w_ptr or None, float(eps), int(bool(causal)), cu_ptr or None, nseq,
            max_seqlen, T, H, Hkv, d, out.data_ptr() or None,
            lse.data_ptr() or None, o12.data_ptr() or None, stream.cuda_stream)
    if st != OK:
        raise DiffAttnError(st, "diffattn_fwd_train")
    return out, lse, o12


def bwd(q, k, v, lambda_q1, lambda_k1, lambda_q2, lambda_k2,
        lambda_init: float, dout, lse, o12, subln_weight=None,
        eps: float = 1e-5, causal: bool = True, cu_seqlens=None,
        max_seqlen=None, nseq=None, workspace=None, stream=None) -> dict:
    """Backward of the prefill: gradients of sum(dout * out) as a dict with
    ``dq``, ``dk``, ``dv`` (storage type), ``dlq1`` .. ``dlk2`` (fp32, shaped
    like the lambda vectors) and ``dw`` (fp32 [2d])."""
    T, H, _, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    lvs = (lambda_q1, lambda_k1, lambda_q2, lambda_k2)
    lptrs, lstride = _lambda_args(lvs, H, d, dev)
    w_ptr = 0 if subln_weight is None else _dev(subln_weight, "subln_weight", dev, torch.float32)
    cu_ptr, nseq, max_seqlen = _seq_args(T, cu_seqlens, max_seqlen, nseq, dev)
    g = {"dq": torch.empty_like(q), "dk": torch.empty_like(k),
         "dv": torch.empty_like(v)}
    # (the library writes every element of these when T > 0; zeros only for
    # T == 0, where it writes nothing -- so a captured call records no fill)
    alloc = torch.zeros_like if T == 0 else torch.empty_like
    for name, lv in zip(("dlq1", "dlk1", "dlq2", "dlk2"), lvs):
        g[name] = alloc(lv)
    g["dw"] = alloc(torch.empty(2 * d, dtype=torch.float32, device=dev))
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_size(q.dtype, T, H, d), 16),
                                dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    ptr = lambda t: t.data_ptr() or None
    with torch.cuda.device(dev):
        st = library().diffattn_bwd(
            _DTYPES[q.dtype], _dev(q, "q", dev), _dev(k, "k", dev, q.dtype),
            _dev(v, "v", dev, q.dtype), *lptrs, lstride, float(lambda_init),
            w_ptr or None, float(eps), int(bool(causal)), cu_ptr or None, nseq,
            max_seqlen, T, H, Hkv, d, _dev(dout, "dout", dev, q.dtype),
            _dev(lse, "lse", dev, torch.float32), _dev(o12, "o12", dev, torch.float32),
            ptr(g["dq"]), ptr(g["dk"]), ptr(g["dv"]), ptr(g["dlq1"]),
            ptr(g["dlk1"]), ptr(g["dlq2"]), ptr(g["dlk2"]), ptr(g["dw"]),
            _dev(workspace, "workspace", dev), workspace.numel(),
            stream.cuda_stream)
    if st != OK:
        raise DiffAttnError(st, "diffattn_bwd")
    return g


class DiffAttnFunction(torch.autograd.Function):
    """Differential attention as a differentiable op: the forward through
    ``diffattn_fwd_train``, the backward through ``diffattn_bwd`` (inputs
    already rotated; gradients for q, k, v, the four lambda vectors and the
    RMSNorm weight).  Call it through ``diff_attention``."""

    @staticmethod
    def forward(ctx, q, k, v, lambda_q1, lambda_k1, lambda_q2, lambda_k2,
                subln_weight, lambda_init, eps, causal, cu_seqlens, max_seqlen, nseq):
        kw = dict(subln_weight=subln_weight, eps=eps, causal=causal,
                  cu_seqlens=cu_seqlens, max_seqlen=max_seqlen, nseq=nseq)
        out, lse, o12 = fwd_train(q, k, v, lambda_q1, lambda_k1, lambda_q2,
                                  lambda_k2, lambda_init, **kw)
        ctx.save_for_backward(q, k, v, lambda_q1, lambda_k1, lambda_q2, lambda_k2, lse, o12)
        ctx.lambda_init = lambda_init
        ctx.kw = kw
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, lq1, lk1, lq2, lk2, lse, o12 = ctx.saved_tensors
        g = bwd(q, k, v, lq1, lk1, lq2, lk2, ctx.lambda_init, dout.contiguous(),
                lse, o12, **ctx.kw)
        w = ctx.kw["subln_weight"]
        dw = g["dw"].view_as(w) if w is not None and ctx.needs_input_grad[7] else None
        return (g["dq"], g["dk"], g["dv"], g["dlq1"], g["dlk1"], g["dlq2"],
                g["dlk2"], dw, None, None, None, None, None, None)


def diff_attention(q, k, v, lambda_q1, lambda_k1, lambda_q2, lambda_k2,
                   lambda_init: float, subln_weight=None, eps: float = 1e-5,
                   causal: bool = True, cu_seqlens=None, max_seqlen=None,
                   nseq=None) -> torch.Tensor:
    """Differentiable forward (autograd through ``DiffAttnFunction``); the
    arguments are those of ``fwd_train`` (q and k post-rotary)."""
    return DiffAttnFunction.apply(q, k, v, lambda_q1, lambda_k1, lambda_q2,
                                  lambda_k2, subln_weight, lambda_init, eps,
                                  causal, cu_seqlens, max_seqlen, nseq)
