"""Seeded synthetic workloads for the prefill attention core.

This module only draws inputs: it holds none of the method's arithmetic, so the
test suite and the benchmark can feed the same arrays to the HIP library and to
the CPU oracle.

Shapes follow the pages' workloads: dense single-sequence prefill at positions
0..T-1 in token-major ``[T, heads*head_dim]`` f32 (memra-engine 0.130.0
``src/forward.rs``, ``Model::forward``), Qwen3-style head geometry, and a packed
mixed-length batch whose positions restart per sequence.

Draw order for every workload (numpy PCG64 seeded with ``seed``): Q, K, V as
standard normals (drawn in f64, stored as f32), then ``w_q = 1 + 0.1 N(0,1)``
and ``w_k`` likewise (f32), then -- only when ``outlier_frac > 0`` -- the
outlier tokens, ``ceil(outlier_frac * T)`` distinct token indices drawn without
replacement.  An outlier token has all of its K heads multiplied by 8
(:func:`with_outlier_keys`), exact in f32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    seq_lens: tuple
    n_head: int
    n_head_kv: int
    head_dim: int
    rope_dim: int
    rope_freq_base: float
    rms_eps: float
    seed: int
    causal: bool = True
    outlier_frac: float = 0.0
    scale: float = field(default=None)  # None -> 1/sqrt(head_dim)

    @property
    def T(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def softmax_scale(self) -> float:
        return float(self.scale) if self.scale is not None else 1.0 / math.sqrt(self.head_dim)

    @property
    def seq_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seq_lens)]).astype(np.int32)

    @property
    def n_seqs(self) -> int:
        return len(self.seq_lens)

    def causal_pairs(self) -> int:
        """Visible (query, key) pairs per head."""
        if self.causal:
            return int(sum(L * (L + 1) // 2 for L in self.seq_lens))
        return int(sum(L * L for L in self.seq_lens))

    def attn_flops(self) -> int:
        """Algorithmic FLOPs of the two contractions, masked work not counted:
        2 FLOPs per multiply-add, head_dim multiply-adds per visible pair for
        each of Q.K and P.V, for every query head."""
        return 4 * self.head_dim * self.n_head * self.causal_pairs()

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads, plus the T = 8192 target shape with the 8B-like heads.
CONFIGS = {
    "tiny": Workload("tiny", (16,), 4, 2, 64, 64, 1e6, 1e-6, seed=1000, scale=1.0 / 8.0),
    "qwen3_0p6b": Workload("qwen3_0p6b", (512,), 16, 8, 128, 128, 1e6, 1e-6, seed=2000),
    "qwen3_8b": Workload("qwen3_8b", (4096,), 32, 8, 128, 128, 1e6, 1e-6, seed=3000),
    "long": Workload("long", (16384,), 32, 8, 128, 128, 1e6, 1e-6, seed=4000, outlier_frac=0.01),
    "mixed": Workload("mixed", (128, 256, 512, 1024, 2048, 3000, 4096, 5000), 16, 4, 128, 64,
                      1e4, 1e-6, seed=5000),
    "prefill_8192": Workload("prefill_8192", (8192,), 32, 8, 128, 128, 1e6, 1e-6, seed=17192),
}


def sweep_workload(T: int) -> Workload:
    """8B-like heads at length T (seed 9000 + T)."""
    return Workload(f"sweep_{T}", (T,), 32, 8, 128, 128, 1e6, 1e-6, seed=9000 + T)


@dataclass
class Inputs:
    q: np.ndarray        # [T, n_head*head_dim] f32
    k: np.ndarray        # [T, n_head_kv*head_dim] f32
    v: np.ndarray        # [T, n_head_kv*head_dim] f32
    wq: np.ndarray       # [head_dim] f32
    wk: np.ndarray       # [head_dim] f32
    outliers: np.ndarray  # sorted int64 token indices (may be empty)


def make_inputs(w: Workload) -> Inputs:
    rng = np.random.default_rng(w.seed)
    T, H, Hkv, d = w.T, w.n_head, w.n_head_kv, w.head_dim
    q = rng.standard_normal((T, H * d)).astype(np.float32)
    k = rng.standard_normal((T, Hkv * d)).astype(np.float32)
    v = rng.standard_normal((T, Hkv * d)).astype(np.float32)
    wq = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    wk = (1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    n_out = int(math.ceil(w.outlier_frac * T)) if w.outlier_frac > 0 else 0
    if n_out:
        outliers = np.sort(rng.choice(T, size=n_out, replace=False)).astype(np.int64)
    else:
        outliers = np.zeros(0, dtype=np.int64)
    return Inputs(q, k, v, wq, wk, outliers)


def with_outlier_keys(k: np.ndarray, outliers: np.ndarray, factor: float = 8.0) -> np.ndarray:
    """A copy of ``k`` whose outlier token rows (every head) are scaled by ``factor``."""
    k2 = np.array(k, copy=True)
    if outliers.size:
        k2[outliers] *= np.float32(factor)
    return k2


def sample_rows(w: Workload, n_random: int = 64, seed: int = 0) -> np.ndarray:
    """Query rows to check at full size: each sequence's first, second and last rows,
    the rows on either side of every 32- and 64-row tile edge near the sequence ends,
    and ``n_random`` uniformly drawn rows.  Sorted, unique."""
    rng = np.random.default_rng(seed)
    rows = set()
    offs = w.seq_offsets
    for s in range(w.n_seqs):
        a, b = int(offs[s]), int(offs[s + 1])
        if b <= a:
            continue
        for r in (a, a + 1, a + 31, a + 32, a + 63, a + 64, b - 65, b - 64, b - 33, b - 32, b - 1):
            if a <= r < b:
                rows.add(r)
    rows.update(int(x) for x in rng.integers(0, w.T, size=n_random))
    return np.array(sorted(rows), dtype=np.int64)


def tile_edge_rows(w: Workload, seed: int = 0) -> np.ndarray:
    """Query rows that touch every tile of every sequence: the rows on both sides of each
    32-row edge (32j - 1 and 32j, counted from the sequence's start; the 64-row edges
    among them), its last row, and one uniformly drawn row inside each 32-row block.
    Sorted, unique."""
    rng = np.random.default_rng(seed)
    rows = set()
    offs = w.seq_offsets
    for s in range(w.n_seqs):
        a, b = int(offs[s]), int(offs[s + 1])
        if b <= a:
            continue
        for j in range(a, b, 32):
            rows.update(r for r in (j - 1, j) if a <= r < b)
            rows.add(int(j + rng.integers(0, min(32, b - j))))
        rows.add(b - 1)
    return np.array(sorted(rows), dtype=np.int64)


def q8_store(rows: int, heads: int, head_dim: int, seed: int, spread: float = 45.0,
             scale: float = 0.022):
    """Random contents of an 8-bit K/V (or Q) store, shaped like quantised normal rows:
    ``codes [rows, heads*head_dim]`` int8 and ``scales [rows, heads]`` f32.

    Draw order (numpy PCG64 seeded with ``seed``): codes as ``N(0, spread^2)`` rounded to
    integers and clipped to -127..127; then one position per (row, head) and a sign, where
    the code is set to +-127 (every quantised row has its largest magnitude on the top
    code); then scales ``scale * exp(0.1 N(0,1))``.  ``spread = 45`` and ``scale = 0.022``
    match unit-variance rows of 128 values."""
    rng = np.random.default_rng(seed)
    c = np.clip(np.rint(rng.normal(0.0, spread, size=(rows, heads, head_dim))), -127, 127)
    top = rng.integers(0, head_dim, size=(rows, heads))
    sign = np.where(rng.integers(0, 2, size=(rows, heads)) == 1, 127, -127)
    np.put_along_axis(c, top[..., None], sign[..., None], axis=2)
    scales = (scale * np.exp(0.1 * rng.standard_normal((rows, heads)))).astype(np.float32)
    return c.astype(np.int8).reshape(rows, heads * head_dim), scales
