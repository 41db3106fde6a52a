"""Seeded synthetic inputs for the product-key memory layer.

This module holds no arithmetic of the method (no scoring, selection, weighting,
gathering or gradient): it only draws the arrays a caller would hand to the
layer, so that the GPU library and the CPU oracle receive identical bytes.
Both the tests and ``bench.py`` use it; neither the oracle nor the GPU library
imports it.

Workloads (shapes follow the memory sizes the pages discuss: 512^2 and 1024^2
slots, a 1600-dim model, batches of 32 x 512 tokens):

  tiny-fp32            T=64,    H=1, d_k=32,  n=32,   k=4,  d_v=16,   fp32
  proj-fp32            T=4096,  H=1, d_k=512, n=128,  k=16, d_v=512,  fp32
  base-bf16            T=16384, H=4, d_k=512, n=512,  k=32, d_v=1024, bf16
  base-bf16-zipf-bwd   as base-bf16, Zipf(1.1) query bias, forward+backward
  large-bf16-zipf-bwd  T=16384, H=8, d_k=512, n=1024, k=32, d_v=1600, bf16, fwd+bwd

Recipes (std is the second argument of every normal):
  * tiny-fp32: q, sub-keys, values all N(0, 1).
  * proj-fp32: x ~ N(0,1) [T, 512], W ~ N(0, 512^-0.5) [512, 512]; the caller-side
    query network is the projection q = x W^T (computed in float64, rounded to
    float32); sub-keys uniform on the unit sphere of dimension d_k/2; values
    N(0, d_v^-0.5).
  * base-bf16: z ~ N(0,1) [T, H, d_k] standardised per feature over the tokens
    (batch-norm style, no affine); sub-keys on the unit sphere; values
    N(0, d_v^-0.5) = N(0, 1/32).
  * *-zipf-bwd: before standardising, each (token, head) query gets a bias
    beta * (C[h,0,i*] ++ C[h,1,j*]) towards one slot (i*, j*) = divmod(pi(r), n),
    where the rank r ~ Zipf(1.1) on 1..n^2 and pi is a fixed seeded permutation
    of the slots; beta = 4.  The upstream gradient dy ~ N(0, 1) [T, d_v].
  * bf16 arrays are rounded from float32 to nearest-even on the host and kept
    as raw uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    d_k: int
    n: int
    k: int
    d_v: int
    dtype: str            # "fp32" or "bf16"
    seed: int
    query: str            # "normal", "projection", "standardised"
    zipf: float = 0.0     # 0 = no slot bias
    zipf_beta: float = 4.0
    backward: bool = False
    d_model: int = 0      # projection input width ("projection" queries)

    @property
    def half(self) -> int:
        return self.d_k // 2

    @property
    def slots(self) -> int:
        return self.n * self.n


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny-fp32", T=64, H=1, d_k=32, n=32, k=4, d_v=16, dtype="fp32",
                 seed=1001, query="normal"),
        Workload("proj-fp32", T=4096, H=1, d_k=512, n=128, k=16, d_v=512, dtype="fp32",
                 seed=1002, query="projection", d_model=512),
        Workload("base-bf16", T=16384, H=4, d_k=512, n=512, k=32, d_v=1024, dtype="bf16",
                 seed=1003, query="standardised"),
        Workload("base-bf16-zipf-bwd", T=16384, H=4, d_k=512, n=512, k=32, d_v=1024,
                 dtype="bf16", seed=1004, query="standardised", zipf=1.1, backward=True),
        Workload("large-bf16-zipf-bwd", T=16384, H=8, d_k=512, n=1024, k=32, d_v=1600,
                 dtype="bf16", seed=1005, query="standardised", zipf=1.1, backward=True),
    ]
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); raw uint16 patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    step = 1 << 24
    flat_u, flat_o = u.reshape(-1), out.reshape(-1)
    for s in range(0, flat_u.size, step):        # chunked: bounded temporaries
        c = flat_u[s:s + step]
        rounded = c + np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1))
        flat_o[s:s + step] = (rounded >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of raw bfloat16 patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _unit_sphere(rng: np.random.Generator, shape) -> np.ndarray:
    v = rng.standard_normal(shape, dtype=np.float64)
    v /= np.linalg.norm(v, axis=-1, keepdims=True)
    return v.astype(np.float32)


def _normal32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _standardise(z: np.ndarray) -> np.ndarray:
    """Batch-norm style: zero mean, unit variance per feature over the tokens."""
    z = z.astype(np.float64)
    z -= z.mean(axis=0, keepdims=True)
    z /= z.std(axis=0, keepdims=True)
    return z.astype(np.float32)


def zipf_slots(rng: np.random.Generator, count: int, slots: int, s: float) -> np.ndarray:
    """`count` slots drawn by rank r ~ p(r) proportional to r^-s on 1..slots,
    mapped through a seeded permutation of the slots."""
    ranks = np.arange(1, slots + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** -s)
    cdf /= cdf[-1]
    r = np.searchsorted(cdf, rng.random(count), side="right")
    r = np.minimum(r, slots - 1)
    perm = rng.permutation(slots)
    return perm[r].astype(np.int64)


def make(workload, T: int | None = None, seed: int | None = None,
         with_dy: bool | None = None) -> dict:
    """Draw the inputs of a workload (a name or a Workload).

    T overrides the token count (same recipe and seed, fewer or more tokens).
    Returns a dict with numpy arrays q [T,H,d_k], keys [H,2,n,d_k/2],
    values [n*n, d_v], optionally dy [T, d_v] (float32 or uint16=bf16 bits,
    per the workload dtype), the float32 versions under *_f32, the Zipf target
    slots (if any) and the Workload itself under "w".
    """
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    if T is not None:
        w = dataclasses.replace(w, T=T)
    rng = np.random.default_rng(w.seed if seed is None else seed)
    half = w.half

    if w.query == "normal":
        keys = _normal32(rng, (w.H, 2, w.n, half), 1.0)
        values = _normal32(rng, (w.slots, w.d_v), 1.0)
    else:
        keys = _unit_sphere(rng, (w.H, 2, w.n, half))
        values = _normal32(rng, (w.slots, w.d_v), w.d_v ** -0.5)

    target = None
    if w.query == "normal":
        q = _normal32(rng, (w.T, w.H, w.d_k), 1.0)
    elif w.query == "projection":
        x = rng.standard_normal((w.T, w.d_model), dtype=np.float64)
        W = rng.standard_normal((w.H * w.d_k, w.d_model), dtype=np.float64) * w.d_model ** -0.5
        q = (x @ W.T).astype(np.float32).reshape(w.T, w.H, w.d_k)
    elif w.query == "standardised":
        z = rng.standard_normal((w.T, w.H * w.d_k), dtype=np.float32)
        if w.zipf > 0:
            target = zipf_slots(rng, w.T * w.H, w.slots, w.zipf).reshape(w.T, w.H)
            i_star, j_star = np.divmod(target, w.n)
            z = z.reshape(w.T, w.H, w.d_k)
            for h in range(w.H):
                z[:, h, :half] += np.float32(w.zipf_beta) * keys[h, 0, i_star[:, h]]
                z[:, h, half:] += np.float32(w.zipf_beta) * keys[h, 1, j_star[:, h]]
            z = z.reshape(w.T, w.H * w.d_k)
        q = _standardise(z).reshape(w.T, w.H, w.d_k)
    else:
        raise ValueError(w.query)

    want_dy = w.backward if with_dy is None else with_dy
    dy = _normal32(rng, (w.T, w.d_v), 1.0) if want_dy else None

    out = dict(w=w, q_f32=q, keys_f32=keys, values_f32=values, dy_f32=dy, target=target)
    if w.dtype == "bf16":
        out["q"] = bf16_bits(q)
        out["keys"] = bf16_bits(keys)
        out["values"] = bf16_bits(values)
        out["dy"] = bf16_bits(dy) if dy is not None else None
        # the float32 views hold exactly the rounded values the kernels see
        out["q_f32"] = bf16_to_f32(out["q"])
        out["keys_f32"] = bf16_to_f32(out["keys"])
        out["values_f32"] = None          # 4x the table; widen on demand
        out["dy_f32"] = bf16_to_f32(out["dy"]) if dy is not None else None
    else:
        out["q"], out["keys"], out["values"], out["dy"] = q, keys, values, dy
    return out


def token_subset(T: int, count: int, seed: int) -> np.ndarray:
    """Sorted seeded subset of token ids (used to bound oracle work)."""
    rng = np.random.default_rng(seed)
    count = min(count, T)
    return np.sort(rng.choice(T, size=count, replace=False)).astype(np.int64)


def custom(T: int, H: int, n: int, k: int, d_k: int, d_v: int, dtype: str = "fp32",
           seed: int = 0, kind: str = "normal", with_dy: bool = True) -> dict:
    """Small seeded problems for edge cases, same dict layout as make().

    kind: "normal"     all N(0, 1)
          "integer"    q in {-3..3}, sub-keys in {-2..2} (exact float arithmetic,
                       many exactly tied scores), values N(0, 1)
          "dup"        normal, with duplicated sub-key rows in both codebooks
          "right_zero" normal, with the right half of every query set to 0
    """
    w = Workload(f"custom-{kind}", T=T, H=H, d_k=d_k, n=n, k=k, d_v=d_v, dtype=dtype,
                 seed=seed, query=kind, backward=with_dy)
    rng = np.random.default_rng(seed)
    half = d_k // 2
    if kind == "integer":
        q = rng.integers(-3, 4, size=(T, H, d_k)).astype(np.float32)
        keys = rng.integers(-2, 3, size=(H, 2, n, half)).astype(np.float32)
    else:
        q = rng.standard_normal((T, H, d_k), dtype=np.float32)
        keys = rng.standard_normal((H, 2, n, half), dtype=np.float32)
    if kind == "dup" and n >= 3:
        keys[:, 0, n - 1] = keys[:, 0, 0]
        keys[:, 1, 1] = keys[:, 1, n - 2]
    if kind == "right_zero":
        q[:, :, half:] = 0.0
    values = rng.standard_normal((n * n, d_v), dtype=np.float32)
    dy = rng.standard_normal((T, d_v), dtype=np.float32) if with_dy else None
    out = dict(w=w, target=None)
    if dtype == "bf16":
        out["q"], out["keys"], out["values"] = bf16_bits(q), bf16_bits(keys), bf16_bits(values)
        out["dy"] = bf16_bits(dy) if dy is not None else None
    else:
        out["q"], out["keys"], out["values"], out["dy"] = q, keys, values, dy
    return out
