"""Seeded synthetic inputs for the differential-attention forward pass.

This module holds no arithmetic of the method itself: it only draws random
tensors, fixes the packed memory layout and names the five workload shapes.
Both the fp64 oracle (through the tests) and the HIP library (through the
tests and the benchmark) consume exactly what it returns, so the two sides see
bit-identical inputs.

Layout (token-major, contiguous), with T tokens, H differential heads, Hkv
key/value heads and half-head width d:

    q   [T, H,   2, d]   q[:, h, 0] is Q1 of head h, q[:, h, 1] is Q2
    k   [T, Hkv, 2, d]   k[:, g, 0] is K1 of KV head g, k[:, g, 1] is K2
    v   [T, Hkv, 2d]     one V shared by both maps
    out [T, H,   2d]

This is the head-major split of the DiffTransformer page
("MultiHeadDifferentialAttention.forward": each head's 2d-wide projection is
chunked into a first half for map 1 and a second half for map 2) laid out the
way the FlashDiffAttention pull request packs it (2H half-heads of width d,
"new_impl" / "alternative_forward").

Draw order (one ``torch.Generator`` seeded with ``seed``): q, k, v from a
standard normal in fp32, then the four lambda vectors lambda_q1, lambda_k1,
lambda_q2, lambda_k2 from N(0, 0.1^2) in fp32 (the Llama diff-attention gist
initialises them with ``normal_(mean=0, std=0.1)``). bf16 workloads round q, k
and v to bf16 after drawing; the lambda vectors stay fp32.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str              # "f32" or "bf16": storage type of q, k, v, out
    seqlens: tuple          # one entry per packed sequence
    H: int
    Hkv: int
    d: int
    depth: int
    causal: bool = True
    eps: float = 1e-5
    seed: int = 0
    description: str = ""

    @property
    def T(self) -> int:
        return int(sum(self.seqlens))

    @property
    def nseq(self) -> int:
        return len(self.seqlens)

    @property
    def max_seqlen(self) -> int:
        return int(max(self.seqlens)) if self.seqlens else 0

    def cu_seqlens(self) -> np.ndarray:
        cu = np.zeros(self.nseq + 1, dtype=np.int32)
        cu[1:] = np.cumsum(np.asarray(self.seqlens, dtype=np.int64))
        return cu

    def flops(self) -> float:
        """FLOP count under the stated convention: per unmasked (query, key)
        pair and head, two QK^T maps of 2d FLOP each plus two PV
        accumulations of 2*2d FLOP each, i.e. 12*d; a causal sequence of
        length n contributes n^2/2 pairs, a full one n^2."""
        pairs = sum((n * n) / 2.0 if self.causal else float(n * n) for n in self.seqlens)
        return 12.0 * self.d * self.H * pairs


def varlen_lengths(total: int, lo: int, hi: int, seed: int = 0) -> List[int]:
    """Sequence lengths drawn uniformly from [lo, hi] with
    ``numpy.random.default_rng(seed)`` until their sum reaches ``total``; the
    last length is cut so that the sum is exactly ``total``."""
    rng = np.random.default_rng(seed)
    out: List[int] = []
    s = 0
    while s < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - s)
        out.append(n)
        s += n
    return out


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", "f32", (64,), H=2, Hkv=2, d=16, depth=1,
        description="fp32, B=1, N=64, 2 diff heads (no GQA), d=16, depth 1"),
    "embed2048_b2_n512": Workload(
        "embed2048_b2_n512", "bf16", (512, 512), H=16, Hkv=4, d=64, depth=12,
        description="bf16, B=2, N=512, 16 diff heads, 4 KV heads, d=64, depth 12"),
    "llama1b_b8_n4096": Workload(
        "llama1b_b8_n4096", "bf16", (4096,) * 8, H=16, Hkv=4, d=64, depth=8,
        description="bf16, B=8, N=4096, 16 diff heads, 4 KV heads, d=64, depth 8"),
    "long_b1_n32768": Workload(
        "long_b1_n32768", "bf16", (32768,), H=16, Hkv=4, d=64, depth=16,
        description="bf16, B=1, N=32768, 16 diff heads, 4 KV heads, d=64, depth 16"),
    "varlen_t65536": Workload(
        "varlen_t65536", "bf16", tuple(varlen_lengths(65536, 128, 4096, 0)),
        H=16, Hkv=4, d=64, depth=24,
        description="bf16 varlen, 65536 tokens, lengths uniform in [128,4096], "
                    "16 diff heads, 4 KV heads, d=64, depth 24"),
}

HEADLINE = "llama1b_b8_n4096"


def _randn(gen: torch.Generator, *shape) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32)


@dataclasses.dataclass
class Inputs:
    """Host tensors of one workload; q/k/v in the storage dtype, everything
    else fp32 (cu_seqlens int32). ``depth`` is the 1-based layer depth from
    which each side derives lambda_init itself."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    lq1: torch.Tensor
    lk1: torch.Tensor
    lq2: torch.Tensor
    lk2: torch.Tensor
    w: torch.Tensor
    cu_seqlens: torch.Tensor
    depth: int
    eps: float
    causal: bool
    max_seqlen: int


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(wl: Workload, seed: Optional[int] = None,
                q_scale: float = 1.0) -> Inputs:
    """Draw the inputs of ``wl`` on the CPU in the fixed order."""
    gen = torch.Generator("cpu")
    gen.manual_seed(wl.seed if seed is None else seed)
    T, H, Hkv, d = wl.T, wl.H, wl.Hkv, wl.d
    dt = torch_dtype(wl.dtype)
    q = _randn(gen, T, H, 2, d)
    if q_scale != 1.0:
        q = q * q_scale
    q = q.to(dt)
    k = _randn(gen, T, Hkv, 2, d).to(dt)
    v = _randn(gen, T, Hkv, 2 * d).to(dt)
    lq1 = 0.1 * _randn(gen, d)
    lk1 = 0.1 * _randn(gen, d)
    lq2 = 0.1 * _randn(gen, d)
    lk2 = 0.1 * _randn(gen, d)
    w = torch.ones(2 * d, dtype=torch.float32)
    cu = torch.from_numpy(wl.cu_seqlens())
    return Inputs(q, k, v, lq1, lk1, lq2, lk2, w, cu,
                  wl.depth, wl.eps, wl.causal, wl.max_seqlen)


def rope_tables(length: int, d: int, base: float = 10000.0, offset: int = 0):
    """Rotary tables ``(cos, sin)``, each fp32 ``[length, d/2]``: row p,
    column j holds cos / sin of (p + offset) * base^(-2j/d), the frequencies
    RotaryEmbedding(head_dim=d, base) uses in the pull request's test
    (computed in float64, rounded once to fp32)."""
    j = np.arange(d // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * j / d)
    ang = np.outer(np.arange(length, dtype=np.float64) + offset, inv_freq)
    return (torch.from_numpy(np.cos(ang).astype(np.float32)),
            torch.from_numpy(np.sin(ang).astype(np.float32)))


# --------------------------------------------------------------------------
# new queries against a key/value cache (decoding)

@dataclasses.dataclass(frozen=True)
class KvWorkload:
    """Sequence s has ``q_lens[s]`` new queries and ``k_lens[s]`` cached keys
    (the new tokens' own keys being the last ``q_lens[s]`` of them).  Queries
    are packed ``[Tq, H, 2, d]``, the caches ``[Tk, Hkv, 2, d]`` and
    ``[Tk, Hkv, 2d]``, each by its own cu_seqlens."""
    name: str
    dtype: str
    q_lens: tuple
    k_lens: tuple
    H: int
    Hkv: int
    d: int
    depth: int
    causal: bool = True
    eps: float = 1e-5
    seed: int = 0
    description: str = ""

    @property
    def nseq(self) -> int:
        return len(self.q_lens)

    @property
    def Tq(self) -> int:
        return int(sum(self.q_lens))

    @property
    def Tk(self) -> int:
        return int(sum(self.k_lens))

    @property
    def max_q(self) -> int:
        return int(max(self.q_lens)) if self.q_lens else 0

    @property
    def max_k(self) -> int:
        return int(max(self.k_lens)) if self.k_lens else 0

    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    def cu_k(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.k_lens)]).astype(np.int32)

    def bytes(self) -> float:
        """Bytes a call must move at least: read q, k, v once, write out."""
        es = 2 if self.dtype == "bf16" else 4
        return float(es * (2 * self.Tq * self.H * 2 * self.d
                           + 2 * self.Tk * self.Hkv * 2 * self.d))

    def flops(self) -> float:
        """12*d FLOP per visible (query, key) pair and head, as for the
        prefill."""
        pairs = 0
        for nq, nk in zip(self.q_lens, self.k_lens):
            if self.causal:
                pairs += sum(nk - nq + i + 1 for i in range(nq))
            else:
                pairs += nq * nk
        return 12.0 * self.d * self.H * pairs


KV_WORKLOADS = {
    "decode_b8_kv4097": KvWorkload(
        "decode_b8_kv4097", "bf16", (1,) * 8, (4097,) * 8, H=16, Hkv=4, d=64,
        depth=8,
        description="bf16 decode step after the B=8, N=4096 prefill: one new "
                    "query per sequence against 4097 cached keys, 16 diff "
                    "heads, 4 KV heads, d=64"),
    "decode_b64_kv8192": KvWorkload(
        "decode_b64_kv8192", "bf16", (1,) * 64, (8192,) * 64, H=16, Hkv=4,
        d=64, depth=8,
        description="bf16 decode step, 64 sequences x 8192 cached keys "
                    "(1 GiB of K/V), one new query each, 16 diff heads, "
                    "4 KV heads, d=64"),
    "decode_varlen_b32_q4": KvWorkload(
        "decode_varlen_b32_q4", "bf16", (4,) * 32,
        tuple(int(x) for x in np.random.default_rng(1).integers(1024, 32769, 32)),
        H=16, Hkv=4, d=64, depth=8,
        description="bf16 multi-token decode: 32 sequences, 4 new queries "
                    "each, cache lengths uniform in [1024, 32768], 16 diff "
                    "heads, 4 KV heads, d=64"),
    "chunk_b8_q1024_kv4096": KvWorkload(
        "chunk_b8_q1024_kv4096", "bf16", (1024,) * 8, (4096,) * 8, H=16, Hkv=4,
        d=64, depth=8,
        description="bf16 chunked prefill: the last 1024 tokens of each of "
                    "the 8 x 4096 prompts as one chunk against its 4096 "
                    "keys (bottom-right causal), 16 diff heads, 4 KV heads, "
                    "d=64"),
    "chunk_b1_q1024_kv32768": KvWorkload(
        "chunk_b1_q1024_kv32768", "bf16", (1024,), (32768,), H=16, Hkv=4,
        d=64, depth=8,
        description="bf16 chunked prefill of one long context: its last "
                    "1024 tokens against 32768 keys (bottom-right causal), "
                    "16 diff heads, 4 KV heads, d=64 -- too few query "
                    "tiles to fill the GPU, so the keys are split"),
}

KV_HEADLINE = "decode_b64_kv8192"


@dataclasses.dataclass
class KvInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    lq1: torch.Tensor
    lk1: torch.Tensor
    lq2: torch.Tensor
    lk2: torch.Tensor
    w: torch.Tensor
    cu_q: torch.Tensor
    cu_k: torch.Tensor
    depth: int
    eps: float
    causal: bool
    max_q: int
    max_k: int


def make_kv_inputs(wl: KvWorkload, seed: Optional[int] = None,
                   q_scale: float = 1.0) -> KvInputs:
    """Draw the inputs of ``wl`` on the CPU: q, k, v (standard normal, fp32
    then rounded to the storage type), then the four lambda vectors
    (N(0, 0.1^2)), from one generator seeded with ``seed``."""
    gen = torch.Generator("cpu")
    gen.manual_seed(wl.seed if seed is None else seed)
    H, Hkv, d = wl.H, wl.Hkv, wl.d
    dt = torch_dtype(wl.dtype)
    q = _randn(gen, wl.Tq, H, 2, d)
    if q_scale != 1.0:
        q = q * q_scale
    q = q.to(dt)
    k = _randn(gen, wl.Tk, Hkv, 2, d).to(dt)
    v = _randn(gen, wl.Tk, Hkv, 2 * d).to(dt)
    lq1 = 0.1 * _randn(gen, d)
    lk1 = 0.1 * _randn(gen, d)
    lq2 = 0.1 * _randn(gen, d)
    lk2 = 0.1 * _randn(gen, d)
    w = torch.ones(2 * d, dtype=torch.float32)
    return KvInputs(q, k, v, lq1, lk1, lq2, lk2, w,
                    torch.from_numpy(wl.cu_q()), torch.from_numpy(wl.cu_k()),
                    wl.depth, wl.eps, wl.causal, wl.max_q, wl.max_k)


def custom_kv(name: str, dtype: str, q_lens, k_lens, H: int, Hkv: int, d: int,
              depth: int = 1, causal: bool = True, eps: float = 1e-5,
              seed: int = 0) -> KvWorkload:
    """An ad-hoc cache workload for edge-case tests."""
    return KvWorkload(name, dtype, tuple(int(n) for n in q_lens),
                      tuple(int(n) for n in k_lens), H=H, Hkv=Hkv, d=d,
                      depth=depth, causal=causal, eps=eps, seed=seed)


def custom(name: str, dtype: str, seqlens, H: int, Hkv: int, d: int,
           depth: int = 1, causal: bool = True, eps: float = 1e-5,
           seed: int = 0) -> Workload:
    """An ad-hoc workload for edge-case tests."""
    return Workload(name, dtype, tuple(int(n) for n in seqlens), H=H, Hkv=Hkv,
                    d=d, depth=depth, causal=causal, eps=eps, seed=seed)
