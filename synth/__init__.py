"""Seeded synthetic inputs for attention over a resident KV-cache prefix.

This module only draws numbers: it holds none of the attention, merge, selection
or quantization arithmetic. Both the fp64 oracle (tests) and the HIP path (tests,
bench) take their inputs from here, so both sides see the same fp16 bits.

Recipe (numpy PCG64 via ``default_rng``):
  * every tensor is drawn as ``standard_normal`` in fp64 and cast to fp16 with
    round-to-nearest-even (numpy's cast), or to fp32 (``dtype="float32"``, for
    fp32-resident slots: same draws, more mantissa bits kept);
  * draw order per (config, layer): Q, K, V, suffix K, suffix V, then extras
    (per-channel K scales, needle block choice);
  * the tiny dense case uses seed 0; every other case uses seed ``[case, layer]``;
  * "per-channel outlier" K (decode and mlx4g32 shapes) multiplies K by a
    ``lognormal(0, 0.5)`` factor of shape ``[H_kv, D]`` before the fp16 cast;
  * the long-context sparse case plants needle blocks: ``rng.choice(nb, n_needles,
    replace=False)`` picks the blocks, and every key in them gets ``+3 * u`` added,
    with ``u`` the unit vector along the sum of the (fp16-rounded) query heads that
    map to the key's kv-head - a +3 sigma shift along the query direction.

Shapes follow the pages (Shared KV Cache Serving, Stage 2 wire forms; ATTEND.* command
table): Q ``[H_q, M, D]``, resident K/V ``[H_kv, N, D]`` (the STORE layout), suffix
K/V ``[H_kv, S_suf, D]``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Case:
    """One workload shape. ``head_map`` None means q-head h reads kv-head h // (H_q // H_kv)."""
    name: str
    case_id: int
    H_q: int
    H_kv: int
    N: int
    D: int
    M: int = 1
    S_suf: int = 0
    layers: int = 1
    k_channel_scale: bool = False
    B: int = 0
    K_top: int = 0
    n_needles: int = 0
    kv_format: str = "fp16"          # "fp16" or "mlx4g32" (resident format)

    def head_map(self) -> np.ndarray:
        r = self.H_q // self.H_kv
        return (np.arange(self.H_q, dtype=np.int32) // r).astype(np.int32)


# The five workload shapes.
TINY = Case("tiny dense prefix attention H=2 N=128 D=64 M=1", 1, 2, 2, 128, 64)
DECODE = Case("decode H=8 N=2048 D=128 M=1, 32 layers", 2, 8, 8, 2048, 128,
              layers=32, k_channel_scale=True)
PREFILL = Case("fused batched-Q prefill H_q=24 H_kv=8 N=4096 M=S_suf=512 D=128", 3,
               24, 8, 4096, 128, M=512, S_suf=512)
MLX4_DECODE = Case("mlx4g32 decode H_q=24 H_kv=8 N=32768 D=128 M=1", 4, 24, 8, 32768, 128,
                   k_channel_scale=True, kv_format="mlx4g32")
SPARSE = Case("sparse-auto H_q=8 H_kv=1 N=65536 D=256 B=64 K_top=8 S_suf=64 M=1", 5,
              8, 1, 65536, 256, S_suf=64, B=64, K_top=8, n_needles=8)

CASES = {c.case_id: c for c in (TINY, DECODE, PREFILL, MLX4_DECODE, SPARSE)}


@dataclass
class Inputs:
    Q: np.ndarray                     # fp16 [H_q, M, D]
    K: np.ndarray                     # fp16 [H_kv, N, D]
    V: np.ndarray                     # fp16 [H_kv, N, D]
    K_suf: Optional[np.ndarray] = None  # fp16 [H_kv, S_suf, D]
    V_suf: Optional[np.ndarray] = None
    head_map: Optional[np.ndarray] = None  # int32 [H_q]
    needles: Optional[np.ndarray] = None   # int64 [H_kv, n_needles] sorted block ids
    extras: dict = field(default_factory=dict)


def rng_for(case: Case, layer: int = 0) -> np.random.Generator:
    if case.case_id == 1:
        return np.random.default_rng(0)
    return np.random.default_rng([case.case_id, layer])


def _normal(rng: np.random.Generator, shape, dtype) -> np.ndarray:
    return rng.standard_normal(shape).astype(dtype)


def generate(case: Case, layer: int = 0, *, N: Optional[int] = None,
             M: Optional[int] = None, S_suf: Optional[int] = None,
             H_q: Optional[int] = None, H_kv: Optional[int] = None,
             D: Optional[int] = None, n_needles: Optional[int] = None,
             seed=None, dtype: str = "float16") -> Inputs:
    """Draw the inputs of ``case`` for ``layer``; keyword overrides shrink a shape
    (same recipe, same draw order) for tests that need a smaller instance. ``dtype``
    is the element type of every returned tensor (float16, or float32)."""
    dt = np.dtype(dtype)
    H_q = case.H_q if H_q is None else H_q
    H_kv = case.H_kv if H_kv is None else H_kv
    N = case.N if N is None else N
    D = case.D if D is None else D
    M = case.M if M is None else M
    S_suf = case.S_suf if S_suf is None else S_suf
    rng = rng_for(case, layer) if seed is None else np.random.default_rng(seed)

    Qd = rng.standard_normal((H_q, M, D))
    Kd = rng.standard_normal((H_kv, N, D))
    Vd = rng.standard_normal((H_kv, N, D))
    Ks = Vs = None
    if S_suf > 0:
        Ks = _normal(rng, (H_kv, S_suf, D), dt)
        Vs = _normal(rng, (H_kv, S_suf, D), dt)
    if case.k_channel_scale:
        c = rng.lognormal(0.0, 0.5, size=(H_kv, D))
        Kd = Kd * c[:, None, :]
    Q = Qd.astype(dt)
    r = max(1, H_q // H_kv)
    head_map = (np.arange(H_q) // r).astype(np.int32)
    needles = None
    n_needles = case.n_needles if n_needles is None else n_needles
    if n_needles > 0 and case.B > 0:
        nb = -(-N // case.B)
        picks = []
        for g in range(H_kv):
            blocks = np.sort(rng.choice(nb, min(n_needles, nb), replace=False))
            picks.append(blocks)
            qsum = Q[head_map == g, 0, :].astype(np.float64).sum(axis=0)
            u = qsum / np.linalg.norm(qsum)
            for b in blocks:
                Kd[g, b * case.B:min((b + 1) * case.B, N), :] += 3.0 * u
        needles = np.stack(picks)
    K = Kd.astype(dt)
    V = Vd.astype(dt)
    return Inputs(Q=Q, K=K, V=V, K_suf=Ks, V_suf=Vs, head_map=head_map, needles=needles)


def random_head_map(H_q: int, H_kv: int, seed: int) -> np.ndarray:
    """An arbitrary (non-h//r) q-head -> kv-head map; when H_q >= H_kv every kv-head is used."""
    rng = np.random.default_rng(seed)
    m = rng.integers(0, H_kv, size=H_q).astype(np.int32)
    if H_q >= H_kv:
        m[rng.permutation(H_q)[:H_kv]] = np.arange(H_kv, dtype=np.int32)
    return m


def mlx4_records(n_tokens: int, kv_dim: int, seed) -> np.ndarray:
    """Random V-store records of the mlx4g32 tier (the per-token layout of the V-store
    page, "The mlx4g32 tier": kv_dim/8 little-endian uint32 code words, then kv_dim/32
    fp16 scales, then kv_dim/32 fp16 biases) -> uint8 [n_tokens, 5 * kv_dim / 8].

    Every field is drawn directly (no encoder runs): code words uniform over all 32-bit
    values, scales |N(0, 1)| * 0.25 and biases N(0, 1) - 2, both cast to fp16 (finite,
    scales >= 0), so the dequantized values spread over roughly [-4, 4]."""
    if kv_dim % 32:
        raise ValueError("kv_dim must be a multiple of 32")
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 2 ** 32, size=(n_tokens, kv_dim // 8), dtype=np.uint64)
    codes = codes.astype("<u4")
    scales = (np.abs(rng.standard_normal((n_tokens, kv_dim // 32))) * 0.25).astype("<f2")
    biases = (rng.standard_normal((n_tokens, kv_dim // 32)) - 2.0).astype("<f2")
    return np.concatenate([codes.view(np.uint8).reshape(n_tokens, -1),
                           scales.view(np.uint8).reshape(n_tokens, -1),
                           biases.view(np.uint8).reshape(n_tokens, -1)], axis=1)
