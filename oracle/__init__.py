"""fp64 CPU oracle of the differential-attention forward pass (ctypes binding).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only users.  The product path (the
``differential_attention_amd`` package and its HIP library) never imports
this package, and this package never imports that one; the only module both
sides share is the seeded input generator ``workloads``.

The arithmetic lives in ``diffattn_ref.c`` (plain C, IEEE double, OpenMP over
output rows); see its header for the formula and the pages it follows.
``build()`` compiles it with gcc into ``libdiffattn_ref.so`` beside it.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "diffattn_ref.c")
LIBRARY = os.path.join(_HERE, "libdiffattn_ref.so")


def build(source: str = SOURCE, output: str = LIBRARY, extra=()) -> str:
    """Compile the oracle with gcc (IEEE semantics: no fast-math)."""
    # (a temporary of this process's own, so concurrent builds -- parallel
    # test workers -- each replace the library whole)
    tmp = f"{output}.{os.getpid()}.tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Werror", *extra, source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


_lib_cache = {}


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library at ``path``."""
    if path in _lib_cache:
        return _lib_cache[path]
    if path == LIBRARY and not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.diffattn_ref_lambda_init.argtypes = [ctypes.c_int]
    lib.diffattn_ref_lambda_init.restype = ctypes.c_double
    lib.diffattn_ref_lambda.argtypes = [f32p, f32p, f32p, f32p, ctypes.c_int,
                                        ctypes.c_double]
    lib.diffattn_ref_lambda.restype = ctypes.c_double
    common = [f32p, f32p, f32p, f32p, f32p, f32p, f32p, ctypes.c_int64,
              ctypes.c_double, f32p, ctypes.c_double, ctypes.c_int, i32p,
              ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
              ctypes.c_int, f32p, f32p, ctypes.c_int64, ctypes.c_int]
    lib.diffattn_ref_fwd.argtypes = common + [f64p, ctypes.c_int]
    lib.diffattn_ref_fwd.restype = ctypes.c_int
    lib.diffattn_ref_rows.argtypes = common + [i64p, i32p, ctypes.c_int64, f64p,
                                               ctypes.c_int]
    lib.diffattn_ref_rows.restype = ctypes.c_int
    lib.diffattn_ref_fwd_kv.argtypes = (
        [f32p] * 7 + [ctypes.c_int64, ctypes.c_double, f32p, ctypes.c_double,
                      ctypes.c_int, i32p, i32p, ctypes.c_int, ctypes.c_int64,
                      ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                      f64p, ctypes.c_int])
    lib.diffattn_ref_fwd_kv.restype = ctypes.c_int
    lib.diffattn_ref_bwd.argtypes = (
        [f32p] * 7 + [ctypes.c_int64, ctypes.c_double, f32p, ctypes.c_double,
                      ctypes.c_int, i32p, ctypes.c_int, ctypes.c_int64,
                      ctypes.c_int, ctypes.c_int, ctypes.c_int, f32p]
        + [f64p] * 10 + [ctypes.c_int])
    lib.diffattn_ref_bwd.restype = ctypes.c_int
    lib.diffattn_ref_bwd_sample.argtypes = (
        [f32p] * 7 + [ctypes.c_int64, ctypes.c_double, f32p, ctypes.c_double,
                      ctypes.c_int, i32p, ctypes.c_int, ctypes.c_int64,
                      ctypes.c_int, ctypes.c_int, ctypes.c_int, f32p,
                      ctypes.c_int64, i64p, i32p, f64p,
                      ctypes.c_int64, i64p, i32p, f64p, f64p, ctypes.c_int])
    lib.diffattn_ref_bwd_sample.restype = ctypes.c_int
    lib.diffattn_ref_max_threads.argtypes = []
    lib.diffattn_ref_max_threads.restype = ctypes.c_int
    _lib_cache[path] = lib
    return lib


def _f32(x) -> np.ndarray:
    """Any array-like (numpy, torch CPU tensor of fp32 or bf16) as a
    contiguous fp32 numpy array; bf16 -> fp32 is exact."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float32).contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def lambda_init(depth: int, lib: Optional[ctypes.CDLL] = None) -> float:
    return (lib or load()).diffattn_ref_lambda_init(int(depth))


def lam(lq1, lk1, lq2, lk2, lambda_init_value: float,
        lib: Optional[ctypes.CDLL] = None) -> float:
    a = [_f32(x).reshape(-1) for x in (lq1, lk1, lq2, lk2)]
    d = a[0].size
    assert all(x.size == d for x in a)
    return (lib or load()).diffattn_ref_lambda(
        *[_ptr(x, ctypes.c_float) for x in a], d, float(lambda_init_value))


def _common(q, k, v, lq1, lk1, lq2, lk2, lambda_init_value, w, eps, causal,
            cu_seqlens, rope=None, rope_round_bf16=False):
    qa, ka, va = _f32(q), _f32(k), _f32(v)
    T, H, two, d = qa.shape
    assert two == 2
    Hkv = ka.shape[1]
    assert ka.shape == (T, Hkv, 2, d) and va.shape == (T, Hkv, 2 * d)
    # lambda vectors: [d] shared by all heads, or [H, d] one set per head
    lv = [_f32(x) for x in (lq1, lk1, lq2, lk2)]
    per_head = lv[0].ndim == 2
    assert all(x.shape == ((H, d) if per_head else (d,)) for x in lv)
    lstride = d if per_head else 0
    wa = None if w is None else _f32(w).reshape(-1)
    if wa is not None:
        assert wa.size == 2 * d
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int32)
    else:
        try:
            import torch
            if isinstance(cu_seqlens, torch.Tensor):
                cu_seqlens = cu_seqlens.cpu().numpy()
        except ImportError:  # pragma: no cover
            pass
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    if rope is None:
        rc = rs = None
        rope_len = 0
    else:
        rc, rs = (_f32(x) for x in rope)
        assert rc.shape == rs.shape and rc.ndim == 2 and rc.shape[1] == d // 2
        rope_len = rc.shape[0]
    keep = (qa, ka, va, lv, wa, cu, rc, rs)
    args = [_ptr(qa, ctypes.c_float), _ptr(ka, ctypes.c_float),
            _ptr(va, ctypes.c_float)] + [_ptr(x, ctypes.c_float) for x in lv]
    args += [int(lstride), float(lambda_init_value),
             None if wa is None else _ptr(wa, ctypes.c_float),
             float(eps), int(bool(causal)), _ptr(cu, ctypes.c_int32),
             int(cu.size - 1), int(T), int(H), int(Hkv), int(d),
             None if rc is None else _ptr(rc, ctypes.c_float),
             None if rs is None else _ptr(rs, ctypes.c_float), int(rope_len),
             int(bool(rope_round_bf16))]
    return keep, args, (T, H, d)


def fwd(q, k, v, lq1, lk1, lq2, lk2, lambda_init_value: float, w=None,
        eps: float = 1e-5, causal: bool = True, cu_seqlens=None,
        nthreads: int = 0, lib: Optional[ctypes.CDLL] = None,
        rope=None, rope_round_bf16: bool = False) -> np.ndarray:
    """Whole output ``[T, H, 2d]`` in fp64.  Layouts as in ``workloads``;
    the lambda vectors are ``[d]`` (shared) or ``[H, d]`` (per head);
    ``rope`` = (cos, sin) tables ``[len, d/2]`` rotates q and k first
    (``rope_round_bf16``: and stores the rotated rows as bf16, as a bf16
    pipeline does)."""
    keep, args, (T, H, d) = _common(q, k, v, lq1, lk1, lq2, lk2,
                                    lambda_init_value, w, eps, causal,
                                    cu_seqlens, rope, rope_round_bf16)
    out = np.empty((T, H, 2 * d), dtype=np.float64)
    rc = (lib or load()).diffattn_ref_fwd(*args, _ptr(out, ctypes.c_double),
                                          int(nthreads))
    del keep
    if rc != 0:
        raise ValueError(f"diffattn_ref_fwd failed with status {rc}")
    return out


def rows(q, k, v, lq1, lk1, lq2, lk2, lambda_init_value: float,
         tokens: Sequence[int], heads: Sequence[int], w=None, eps: float = 1e-5,
         causal: bool = True, cu_seqlens=None, nthreads: int = 0,
         lib: Optional[ctypes.CDLL] = None, rope=None,
         rope_round_bf16: bool = False) -> np.ndarray:
    """Output rows ``[len(tokens), 2d]`` in fp64 for (token, head) pairs."""
    keep, args, (T, H, d) = _common(q, k, v, lq1, lk1, lq2, lk2,
                                    lambda_init_value, w, eps, causal,
                                    cu_seqlens, rope, rope_round_bf16)
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    hd = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    assert tok.shape == hd.shape and tok.ndim == 1
    out = np.empty((tok.size, 2 * d), dtype=np.float64)
    rc = (lib or load()).diffattn_ref_rows(
        *args, _ptr(tok, ctypes.c_int64), _ptr(hd, ctypes.c_int32),
        int(tok.size), _ptr(out, ctypes.c_double), int(nthreads))
    del keep
    if rc != 0:
        raise ValueError(f"diffattn_ref_rows failed with status {rc}")
    return out


def _cu(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def fwd_kv(q, k, v, lq1, lk1, lq2, lk2, lambda_init_value: float, w=None,
           eps: float = 1e-5, causal: bool = True, cu_seqlens_q=None,
           cu_seqlens_k=None, nthreads: int = 0,
           lib: Optional[ctypes.CDLL] = None) -> np.ndarray:
    """New queries against a key/value cache, in fp64: q ``[Tq, H, 2, d]``,
    k ``[Tk, Hkv, 2, d]``, v ``[Tk, Hkv, 2d]``; sequence s owns query tokens
    ``cu_seqlens_q[s] ..`` and key tokens ``cu_seqlens_k[s] ..`` (one
    sequence of all tokens when both are None).  Causal rows are aligned
    bottom-right.  Returns ``[Tq, H, 2d]``."""
    qa, ka, va = _f32(q), _f32(k), _f32(v)
    Tq, H, two, d = qa.shape
    Tk, Hkv = ka.shape[0], ka.shape[1]
    assert two == 2 and ka.shape == (Tk, Hkv, 2, d)
    assert va.shape == (Tk, Hkv, 2 * d)
    lv = [_f32(x) for x in (lq1, lk1, lq2, lk2)]
    per_head = lv[0].ndim == 2
    assert all(x.shape == ((H, d) if per_head else (d,)) for x in lv)
    wa = None if w is None else _f32(w).reshape(-1)
    cq = _cu([0, Tq] if cu_seqlens_q is None else cu_seqlens_q)
    ck = _cu([0, Tk] if cu_seqlens_k is None else cu_seqlens_k)
    if cq.size != ck.size:
        raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
    out = np.empty((Tq, H, 2 * d), dtype=np.float64)
    rc = (lib or load()).diffattn_ref_fwd_kv(
        _ptr(qa, ctypes.c_float), _ptr(ka, ctypes.c_float),
        _ptr(va, ctypes.c_float), *[_ptr(x, ctypes.c_float) for x in lv],
        int(d if per_head else 0), float(lambda_init_value),
        None if wa is None else _ptr(wa, ctypes.c_float), float(eps),
        int(bool(causal)), _ptr(cq, ctypes.c_int32), _ptr(ck, ctypes.c_int32),
        int(cq.size - 1), int(Tq), int(Tk), int(H), int(Hkv), int(d),
        _ptr(out, ctypes.c_double), int(nthreads))
    if rc != 0:
        raise ValueError(f"diffattn_ref_fwd_kv failed with status {rc}")
    return out


def bwd(q, k, v, lq1, lk1, lq2, lk2, lambda_init_value: float, dy, w=None,
        eps: float = 1e-5, causal: bool = True, cu_seqlens=None,
        nthreads: int = 0, lib: Optional[ctypes.CDLL] = None) -> dict:
    """Gradients of <dy, fwd(...)> in fp64: ``dq``, ``dk``, ``dv`` in the
    input layouts, ``dlq1``.. ``dlk2`` shaped like the lambda vectors and
    ``dw`` [2d] (the RMSNorm weight; of ones when ``w`` is None); plus, under
    ``aux``, ``dlam_head`` [H] (dlambda per head) and ``dlam_scale`` [H]
    (sum over the head's rows of |dpre| |O_2|, the size a relative error in
    those factors can move dlambda by)."""
    keep, args, (T, H, d) = _common(q, k, v, lq1, lk1, lq2, lk2,
                                    lambda_init_value, w, eps, causal,
                                    cu_seqlens)
    Hkv = _f32(k).shape[1]
    dya = _f32(dy)
    assert dya.shape == (T, H, 2 * d)
    lshape = _f32(lq1).shape
    out = {"dq": np.empty((T, H, 2, d)), "dk": np.empty((T, Hkv, 2, d)),
           "dv": np.empty((T, Hkv, 2 * d)), "dlq1": np.zeros(lshape),
           "dlk1": np.zeros(lshape), "dlq2": np.zeros(lshape),
           "dlk2": np.zeros(lshape), "dw": np.empty(2 * d)}
    aux = {"dlam_head": np.empty(H), "dlam_scale": np.empty(H)}
    order = ["dq", "dk", "dv", "dlq1", "dlk1", "dlq2", "dlk2", "dw"]
    # the rotary arguments of the forward entry points are not part of this one
    rc = (lib or load()).diffattn_ref_bwd(
        *args[:-4], _ptr(dya, ctypes.c_float),
        *[_ptr(out[kk], ctypes.c_double) for kk in order],
        _ptr(aux["dlam_head"], ctypes.c_double),
        _ptr(aux["dlam_scale"], ctypes.c_double), int(nthreads))
    del keep
    if rc != 0:
        raise ValueError(f"diffattn_ref_bwd failed with status {rc}")
    out["aux"] = aux
    return out


def bwd_sample(q, k, v, lq1, lk1, lq2, lk2, lambda_init_value: float, dy,
               rows_q, rows_k, w=None, eps: float = 1e-5, causal: bool = True,
               cu_seqlens=None, nthreads: int = 0,
               lib: Optional[ctypes.CDLL] = None) -> dict:
    """Backward on a sample: ``dq`` [len(rows_q), 2, d] for rows_q = (tokens,
    heads) and ``dk`` [len(rows_k), 2, d], ``dv`` [len(rows_k), 2d] for
    rows_k = (key tokens, KV heads), as ``bwd`` defines them."""
    keep, args, (T, H, d) = _common(q, k, v, lq1, lk1, lq2, lk2,
                                    lambda_init_value, w, eps, causal,
                                    cu_seqlens)
    dya = _f32(dy)
    tq = np.ascontiguousarray(np.asarray(rows_q[0], dtype=np.int64))
    hq = np.ascontiguousarray(np.asarray(rows_q[1], dtype=np.int32))
    tk = np.ascontiguousarray(np.asarray(rows_k[0], dtype=np.int64))
    gk = np.ascontiguousarray(np.asarray(rows_k[1], dtype=np.int32))
    out = {"dq": np.empty((tq.size, 2, d)), "dk": np.empty((tk.size, 2, d)),
           "dv": np.empty((tk.size, 2 * d))}
    rc = (lib or load()).diffattn_ref_bwd_sample(
        *args[:-4], _ptr(dya, ctypes.c_float),
        int(tq.size), _ptr(tq, ctypes.c_int64), _ptr(hq, ctypes.c_int32),
        _ptr(out["dq"], ctypes.c_double),
        int(tk.size), _ptr(tk, ctypes.c_int64), _ptr(gk, ctypes.c_int32),
        _ptr(out["dk"], ctypes.c_double), _ptr(out["dv"], ctypes.c_double),
        int(nthreads))
    del keep
    if rc != 0:
        raise ValueError(f"diffattn_ref_bwd_sample failed with status {rc}")
    return out


def max_threads(lib: Optional[ctypes.CDLL] = None) -> int:
    return (lib or load()).diffattn_ref_max_threads()
