"""Workload shapes and seeded generators for SOCKET decode inputs.

Layouts (all contiguous, row-major):
  Q  [B, Hq, d]            query of the current decode step
  K  [B, Hkv, N, d]        cached keys
  V  [B, Hkv, N, d]        cached values
  R  [d, L*P]              random hyperplanes; column l*P + j is bit j of table l

Distributions (the SOCKET pages evaluate on real models with LongBench and
RULER; those need weights and datasets, so these seeded tensors stand in for
them with Llama-3-8B attention shapes):
  * Q, R ~ N(0, 1).
  * K ~ N(0, 1); optionally a few outlier channels (chosen once per seed and
    shared by every head and token) are multiplied by a constant.
  * V is either N(0, 1) or a uniformly random direction whose length is drawn
    from LogNormal(0, 0.5).
  * Optionally a few "planted" keys per (batch, KV head) at distinct seeded
    positions: key = |q| * (0.9 * q_hat + sqrt(1 - 0.81) * w_hat), where q_hat
    is the unit step-0 query of the first query head of the group and w_hat a
    random unit vector orthogonal to it, so cos(key, q) = 0.9 exactly in real
    arithmetic. Planted rows replace the whole key row (no outlier scaling).

Values are drawn in float32 and rounded to bfloat16 (round-to-nearest-even)
when the workload is bf16. Every tensor gets its own seed derived from
(base seed, workload name, tensor tag, layer, step), so a tensor can be
regenerated alone on any device.
"""

from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    N: int
    dtype: str  # "f32" or "bf16"
    L: int
    P: int
    tau: float
    k: int
    steps: int = 1
    outlier_channels: int = 0
    outlier_scale: float = 1.0
    lognormal_v: bool = False
    planted: int = 0
    decode: bool = True

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def C(self) -> int:
        return self.L * self.P

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def kk(self) -> int:
        return min(self.k, self.N)


WORKLOADS = {
    # Tiny fp32 decode: one head, d=64, 1024 keys, 8 tables of 4 bits.
    "tiny_fp32_1k": Workload("tiny_fp32_1k", B=1, Hq=1, Hkv=1, d=64, N=1024,
                             dtype="f32", L=8, P=4, tau=0.5, k=64),
    # Llama-3-8B attention shape (32 query / 8 KV heads, d=128) at 32K keys.
    "llama3_8b_32k": Workload("llama3_8b_32k", B=1, Hq=32, Hkv=8, d=128,
                              N=32768, dtype="bf16", L=32, P=8, tau=0.3,
                              k=1024, outlier_channels=4, outlier_scale=8.0,
                              lognormal_v=True, planted=16),
    # Same shape at 128K keys, batch 4, 256 decode steps with fresh queries.
    "llama3_8b_128k_b4": Workload("llama3_8b_128k_b4", B=4, Hq=32, Hkv=8,
                                  d=128, N=131072, dtype="bf16", L=32, P=8,
                                  tau=0.3, k=4096, steps=256,
                                  outlier_channels=4, outlier_scale=8.0,
                                  lognormal_v=True, planted=16),
    # Prefill hashing only: 8 KV heads x 128K keys, 64 tables of 8 bits.
    "prefill_hash_128k": Workload("prefill_hash_128k", B=1, Hq=8, Hkv=8,
                                  d=128, N=131072, dtype="bf16", L=64, P=8,
                                  tau=1.0, k=1, decode=False),
    # One million keys, 64 tables of 6 bits.
    "llama3_8b_1m": Workload("llama3_8b_1m", B=1, Hq=32, Hkv=8, d=128,
                             N=1048576, dtype="bf16", L=64, P=6, tau=0.2,
                             k=16384, outlier_channels=4, outlier_scale=8.0,
                             lognormal_v=True, planted=16),
}


def custom_workload(base: str | None = None, **kw) -> Workload:
    """A workload with explicit sizes, optionally starting from a named one."""
    if base is not None:
        return replace(WORKLOADS[base], **kw)
    defaults = dict(name="custom", B=1, Hq=1, Hkv=1, d=64, N=256, dtype="f32",
                    L=4, P=4, tau=0.5, k=16)
    defaults.update(kw)
    return Workload(**defaults)


def seed_for(base_seed: int, workload: str, tag: str, layer: int = 0,
             step: int = 0) -> int:
    key = f"{base_seed}/{workload}/{tag}/{layer}/{step}".encode()
    return zlib.crc32(key) * 2654435761 % (2 ** 62)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, device, seed):
    return torch.randn(shape, generator=_gen(device, seed), device=device,
                       dtype=torch.float32)


def make_query(w: Workload, device="cpu", seed: int = 0, step: int = 0,
               layer: int = 0) -> torch.Tensor:
    """Q [B, Hq, d] for one decode step."""
    q = _randn((w.B, w.Hq, w.d), device, seed_for(seed, w.name, "q", layer, step))
    return q.to(w.torch_dtype)


def make_hyperplanes(w: Workload, device="cpu", seed: int = 0,
                     layer: int = 0) -> torch.Tensor:
    """R [d, L*P] ~ N(0, 1)."""
    r = _randn((w.d, w.C), device, seed_for(seed, w.name, "r", layer))
    return r.to(w.torch_dtype)


def make_keys_values(w: Workload, device="cpu", seed: int = 0,
                     layer: int = 0):
    """(K, V) each [B, Hkv, N, d] in the workload dtype."""
    shape = (w.B, w.Hkv, w.N, w.d)
    K = _randn(shape, device, seed_for(seed, w.name, "k", layer))
    if w.outlier_channels > 0:
        perm = torch.randperm(w.d, generator=_gen("cpu", seed_for(
            seed, w.name, "outliers", layer)))
        ch = perm[: w.outlier_channels].to(device)
        K[..., ch] *= w.outlier_scale
    V = _randn(shape, device, seed_for(seed, w.name, "v", layer))
    if w.lognormal_v:
        length = torch.exp(0.5 * _randn((w.B, w.Hkv, w.N, 1), device,
                                        seed_for(seed, w.name, "vlen", layer)))
        V = V / V.norm(dim=-1, keepdim=True).clamp_min(1e-30) * length
    if w.planted > 0 and w.N > 0:
        q0 = _randn((w.B, w.Hq, w.d), device,
                    seed_for(seed, w.name, "q", layer, 0))
        gpos = _gen("cpu", seed_for(seed, w.name, "planted_pos", layer))
        wdir = _randn((w.B, w.Hkv, w.planted, w.d), device,
                      seed_for(seed, w.name, "planted_dir", layer))
        n_plant = min(w.planted, w.N)
        for b in range(w.B):
            for g in range(w.Hkv):
                pos = torch.randperm(w.N, generator=gpos)[:n_plant].to(device)
                q = q0[b, g * w.G].double()
                qn = q.norm()
                qhat = q / qn
                wv = wdir[b, g, :n_plant].double()
                wv = wv - (wv @ qhat)[:, None] * qhat[None, :]
                wv = wv / wv.norm(dim=-1, keepdim=True)
                rows = qn * (0.9 * qhat[None, :] + math.sqrt(1 - 0.81) * wv)
                K[b, g, pos] = rows.float()
    return K.to(w.torch_dtype), V.to(w.torch_dtype)


def planted_positions(w: Workload, seed: int = 0, layer: int = 0):
    """Positions of the planted keys, [B, Hkv, planted] (CPU int64)."""
    gpos = _gen("cpu", seed_for(seed, w.name, "planted_pos", layer))
    n_plant = min(w.planted, w.N)
    out = torch.empty((w.B, w.Hkv, n_plant), dtype=torch.int64)
    for b in range(w.B):
        for g in range(w.Hkv):
            out[b, g] = torch.randperm(w.N, generator=gpos)[:n_plant]
    return out


def make_decode_inputs(w: Workload, device="cpu", seed: int = 0,
                       step: int = 0, layer: int = 0):
    """(Q, K, V, R) for one decode step of the workload."""
    K, V = make_keys_values(w, device, seed, layer)
    Q = make_query(w, device, seed, step, layer)
    R = make_hyperplanes(w, device, seed, layer)
    return Q, K, V, R
