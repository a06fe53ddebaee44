"""Seeded synthetic inputs: the only code shared by the HIP path's tests and
the oracle's.  It draws random numbers and nothing else -- none of the
attention arithmetic lives here.

Recipe: a CPU ``torch.Generator`` seeded with the preset's seed draws
standard-normal float32 tensors in the order Q, K, V, dO (each contiguous
[B, H, N, d]; K and V use H_kv heads; for the split presets Q has N_q rows
and K, V have N_k; packed variable-length batches are [H, total, d], their
lengths drawn first from a generator of their own); bf16 presets round those
values to bfloat16 (round to nearest even).  The same rounded values feed the GPU and,
upcast exactly to float64, the oracle.
"""

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Preset:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str  # "bf16" or "fp32"
    causal: bool
    seed: int
    backward: bool = False

    @property
    def scale(self):
        return self.d ** -0.5

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def describe(self):
        return (f"{self.name}: B={self.B} H_q={self.Hq} H_kv={self.Hkv} N={self.N} d={self.d} "
                f"{self.dtype} {'causal' if self.causal else 'non-causal'} seed={self.seed}")


PRESETS = {
    p.name: p
    for p in [
        Preset("c1", 1, 1, 1, 128, 64, "fp32", False, 101),
        Preset("c2", 8, 16, 16, 2048, 128, "bf16", True, 201),
        Preset("c3a", 2, 16, 16, 8192, 128, "bf16", True, 301),
        Preset("c3b", 2, 32, 32, 8192, 64, "bf16", True, 302),
        Preset("c4a", 4, 32, 8, 4096, 128, "bf16", True, 401),
        Preset("c4b", 4, 32, 1, 4096, 128, "bf16", True, 402),
        Preset("c4c", 4, 8, 8, 2048, 256, "bf16", True, 403),
        Preset("c5", 4, 16, 16, 4096, 64, "bf16", True, 501, backward=True),
    ]
}


def make(B, Hq, Hkv, N, d, dtype=torch.bfloat16, seed=0, with_grad=False):
    """Q, K, V (and dO when ``with_grad``) as CPU tensors of ``dtype``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, Hq, N, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    out = [q, k, v]
    if with_grad:
        out.append(torch.randn((B, Hq, N, d), generator=g, dtype=torch.float32))
    return tuple(t.to(dtype) for t in out)


@dataclass(frozen=True)
class SplitPreset:
    """N_q queries against N_k keys (split key/value forward workloads)."""

    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    seed: int
    dtype: str = "bf16"

    @property
    def scale(self):
        return self.d ** -0.5

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def describe(self):
        return (f"{self.name}: B={self.B} H_q={self.Hq} H_kv={self.Hkv} N_q={self.Nq} N_k={self.Nk} d={self.d} "
                f"{self.dtype} {'causal' if self.causal else 'non-causal'} seed={self.seed}")


# Decoding steps (one query per head against a long key/value cache), with
# grouped heads (4 query heads per kv head) and without.
SPLIT_PRESETS = {
    p.name: p
    for p in [
        SplitPreset("s1", 4, 32, 8, 1, 16384, 128, True, 601),
        SplitPreset("s2", 8, 16, 16, 1, 8192, 128, True, 602),
        SplitPreset("s3", 1, 8, 8, 16, 32768, 64, True, 603),
    ]
}


def make_split(B, Hq, Hkv, Nq, Nk, d, dtype=torch.bfloat16, seed=0):
    """Q [B, Hq, Nq, d], K and V [B, Hkv, Nk, d], drawn in that order."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, Hq, Nq, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, Nk, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, Nk, d), generator=g, dtype=torch.float32)
    return tuple(t.to(dtype) for t in (q, k, v))


def make_split_preset(p):
    return make_split(p.B, p.Hq, p.Hkv, p.Nq, p.Nk, p.d, p.torch_dtype, p.seed)


def make_preset(p, with_grad=None):
    return make(p.B, p.Hq, p.Hkv, p.N, p.d, p.torch_dtype, p.seed, p.backward if with_grad is None else with_grad)


@dataclass(frozen=True)
class VarlenPreset:
    """Packed sequences of different lengths: ``total`` tokens per head, the
    lengths drawn log-uniformly in [lo, hi] (``varlen_lengths``)."""

    name: str
    total: int
    lo: int
    hi: int
    Hq: int
    Hkv: int
    d: int
    causal: bool
    seed: int
    dtype: str = "bf16"

    @property
    def scale(self):
        return self.d ** -0.5

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def lengths(self):
        return varlen_lengths(self.total, self.lo, self.hi, self.seed)

    def describe(self):
        n = self.lengths
        return (f"{self.name}: {len(n)} sequences, total={self.total} lengths {self.lo}..{self.hi} "
                f"(longest {max(n)}) H_q={self.Hq} H_kv={self.Hkv} d={self.d} {self.dtype} "
                f"{'causal' if self.causal else 'non-causal'} seed={self.seed}")


# The fwd+bwd workload's token count (8 x 2048 per head) as a ragged pack of
# sequences of 128..4096 tokens.
VARLEN_PRESETS = {
    p.name: p
    for p in [
        VarlenPreset("v1", 16384, 128, 4096, 16, 16, 128, True, 701),
        VarlenPreset("v2", 16384, 128, 4096, 16, 16, 64, True, 702),
    ]
}


def varlen_lengths(total, lo, hi, seed):
    """Sequence lengths drawn log-uniformly in [lo, hi] (a torch generator
    seeded with ``seed``) until they sum to ``total``; the last one is cut to
    fit."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 7919)
    lens, s = [], 0
    while s < total:
        u = float(torch.rand((), generator=g))
        n = min(int(round(lo * (hi / lo) ** u)), total - s)
        lens.append(n)
        s += n
    return lens


def make_varlen(lengths, Hq, Hkv, d, dtype=torch.bfloat16, seed=0, with_grad=False):
    """Packed Q [Hq, total, d], K and V [Hkv, total, d] (and dO like Q when
    ``with_grad``), drawn in that order, plus the offsets cu_seqlens (int32,
    CPU, len(lengths) + 1 entries)."""
    total = int(sum(lengths))
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((Hq, total, d), generator=g, dtype=torch.float32)
    k = torch.randn((Hkv, total, d), generator=g, dtype=torch.float32)
    v = torch.randn((Hkv, total, d), generator=g, dtype=torch.float32)
    out = [q, k, v]
    if with_grad:
        out.append(torch.randn((Hq, total, d), generator=g, dtype=torch.float32))
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if lengths:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return (*[t.to(dtype) for t in out], cu)


def make_varlen_preset(p, with_grad=True):
    return make_varlen(p.lengths, p.Hq, p.Hkv, p.d, p.torch_dtype, p.seed, with_grad)
