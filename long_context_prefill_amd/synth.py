"""Seeded synthetic inputs for causal-prefill attention workloads.

This module only draws inputs.  It holds none of the attention method's
arithmetic; both the CPU oracle (through the tests) and the HIP path consume the
arrays it returns, so nothing here may depend on either of them.

The pages measure on Llama-3.1-8B and Qwen3-8B prefill at up to 128K tokens
over RULER, LongBench v2 and InfiniteBench ("S2O: Early Stopping for Sparse
Attention via Online Permutation", gist.science technical summary, section
"Résultats Expérimentaux").  None of those weights or suites is available, so
these generators stand in for them.  They plant the structures the pages name
as the reason importance ordering pays off: vertical stripes (a few keys that
every query attends to), attention sinks at the first positions and a local
band near the diagonal (same summary, "Classement par Segment" and
"Signification et Revendications").

Recipe per (batch b, KV group g), with ``rng = default_rng([20260226, seed, b, g])``
and draws in this order: u, stripe positions, band knots, K, V, then the G query
heads of the group.

* structure ``"stripes"`` / ``"stripes+band"``:
  - K, V, Q ~ N(0, 1) in fp32;
  - u is a seeded unit vector; K rows at the sinks 0..3 and at ``n_stripes``
    positions drawn without replacement from [4, N) get ``+4u``; every Q row
    gets ``+2u``;
  - ``"stripes+band"`` adds ``c * w(t)`` to Q[t] and K[t], where w is a unit
    direction field, piecewise linear between seeded unit knots every 128
    tokens and renormalised, and ``c**2 = 1.5 * sqrt(d + 4)``.  Near the
    diagonal this raises the logit by about 1.5 * |Q_i| / sqrt(d), the size a
    key shifted by 1.5 along the query direction would give; the boost fades
    to ~0 beyond a few hundred tokens.
* structure ``"uniform"``: Q, K ~ N(0, 0.1**2), V ~ N(0, 1), nothing planted.

bf16 inputs are the fp32 draws rounded to nearest-even and stored as uint16
bit patterns.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

SEED_ROOT = 20260226
SINKS = (0, 1, 2, 3)
BAND_KNOT_STRIDE = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention-layer workload."""

    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    dtype: str  # "f32" or "bf16"
    tile_m: int
    tile_n: int
    seg_len: int
    taus: Tuple[float, ...]
    structure: str  # "stripes", "stripes+band" or "uniform"
    n_stripes: int
    seed: int
    softmax_scale: Optional[float] = None  # None: 1/sqrt(d)

    @property
    def scale(self) -> float:
        if self.softmax_scale is not None:
            return float(self.softmax_scale)
        return float(1.0 / np.sqrt(self.d))


def _llama8b(name, N, seg_len, taus, structure, seed):
    return Workload(name=name, B=1, Hq=32, Hkv=8, N=N, d=128, dtype="bf16",
                    tile_m=128, tile_n=64, seg_len=seg_len, taus=taus,
                    structure=structure,
                    n_stripes=int(round(0.01 * N)) if structure != "uniform" else 0,
                    seed=seed)


TAU_SWEEP = (1e-1, 3e-2, 1e-2, 5e-3, 3e-3, 2e-3, 1.5e-3, 1.2e-3, 1e-3, 7e-4, 5e-4, 3e-4, 1e-4, 0.0)

WORKLOADS: Dict[str, Workload] = {
    # one fp32 head, 2048 tokens; the whole sequence is one segment (dense)
    "tiny_f32_n2048": Workload("tiny_f32_n2048", 1, 1, 1, 2048, 64, "f32", 64, 64,
                               2048, (1e-3,), "stripes", 32, 0),
    # the same inputs with 512-token segments, so index lists and early stop occur
    "tiny_f32_n2048_s512": Workload("tiny_f32_n2048_s512", 1, 1, 1, 2048, 64, "f32",
                                    64, 64, 512, (1e-3, 0.0), "stripes", 32, 0),
    # Llama-3.1-8B attention-layer shape (32 Q heads, 8 KV heads, d=128)
    "llama8b_n16k": _llama8b("llama8b_n16k", 16384, 4096, (1e-2, 1e-3, 1e-4),
                             "stripes+band", 1),
    "llama8b_n64k": _llama8b("llama8b_n64k", 65536, 8192, (1e-3,), "stripes+band", 2),
    "llama8b_n128k": _llama8b("llama8b_n128k", 131072, 8192, TAU_SWEEP,
                              "stripes+band", 3),
    # near-uniform attention: no planted structure
    "uniform_n128k": _llama8b("uniform_n128k", 131072, 8192, (0.0, 1e-3), "uniform", 4),
}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); return uint16 bit patterns.

    Inputs must be finite.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _unit(v: np.ndarray) -> np.ndarray:
    return v / np.linalg.norm(v, axis=-1, keepdims=True)


def _band_field(knots: np.ndarray, N: int) -> np.ndarray:
    t = np.arange(N)
    k0 = t // BAND_KNOT_STRIDE
    frac = ((t % BAND_KNOT_STRIDE) / BAND_KNOT_STRIDE).astype(np.float32)[:, None]
    w = (1.0 - frac) * knots[k0] + frac * knots[k0 + 1]
    return _unit(w).astype(np.float32)


def _draw_group(rng, N, d, G, structure, n_stripes):
    """One KV group's K, V and its G query heads, fp32."""
    if structure == "uniform":
        k = (0.1 * rng.standard_normal((N, d), dtype=np.float32)).astype(np.float32)
        v = rng.standard_normal((N, d), dtype=np.float32)
        q = (0.1 * rng.standard_normal((G, N, d), dtype=np.float32)).astype(np.float32)
        return q, k, v
    u = _unit(rng.standard_normal(d)).astype(np.float32)
    stripes = rng.choice(np.arange(len(SINKS), N), size=min(n_stripes, N - len(SINKS)),
                         replace=False)
    knots = None
    if structure == "stripes+band":
        n_knots = N // BAND_KNOT_STRIDE + 2
        knots = _unit(rng.standard_normal((n_knots, d))).astype(np.float32)
    elif structure != "stripes":
        raise ValueError(f"unknown structure {structure!r}")
    k = rng.standard_normal((N, d), dtype=np.float32)
    v = rng.standard_normal((N, d), dtype=np.float32)
    q = rng.standard_normal((G, N, d), dtype=np.float32)
    marked = np.concatenate([np.array(SINKS[:min(len(SINKS), N)]), stripes])
    k[marked] += 4.0 * u
    q += 2.0 * u
    if knots is not None:
        c = np.float32(np.sqrt(1.5 * np.sqrt(d + 4.0)))
        w = _band_field(knots, N)
        k += c * w
        q += c * w[None]
    return q, k, v


def make_inputs(w: Workload, seed: int | None = None):
    """Draw Q [B,Hq,N,d], K and V [B,Hkv,N,d] for workload ``w``.

    Returns a dict with ``q``, ``k``, ``v`` as numpy arrays in storage form
    (float32, or uint16 bf16 bit patterns) and ``workload``.
    """
    seed = w.seed if seed is None else seed
    G = w.Hq // w.Hkv
    store = np.float32 if w.dtype == "f32" else np.uint16
    q = np.empty((w.B, w.Hq, w.N, w.d), dtype=store)
    k = np.empty((w.B, w.Hkv, w.N, w.d), dtype=store)
    v = np.empty((w.B, w.Hkv, w.N, w.d), dtype=store)
    conv = (lambda a: a.astype(np.float32)) if w.dtype == "f32" else bf16_bits_from_f32
    for b in range(w.B):
        for g in range(w.Hkv):
            rng = np.random.default_rng([SEED_ROOT, seed, b, g])
            qg, kg, vg = _draw_group(rng, w.N, w.d, G, w.structure, w.n_stripes)
            k[b, g] = conv(kg)
            v[b, g] = conv(vg)
            for i in range(G):
                q[b, g * G + i] = conv(qg[i])
    return {"q": q, "k": k, "v": v, "workload": w}


def custom_workload(B=1, Hq=1, Hkv=1, N=256, d=64, dtype="f32", tile_m=64, tile_n=64,
                    seg_len=128, structure="stripes", n_stripes=8, seed=100,
                    taus=(1e-3,), name="custom", scale=None) -> Workload:
    """A small workload for tests (shapes chosen by the caller; scale None is 1/sqrt(d))."""
    return Workload(name, B, Hq, Hkv, N, d, dtype, tile_m, tile_n, seg_len,
                    tuple(taus), structure, n_stripes, seed, scale)
