"""Seeded synthetic inputs for token-level cross-entropy.

This module only builds inputs: logit matrices, labels and per-workload
settings.  It holds none of the loss arithmetic, so both the GPU tests and the
float64 oracle can take their inputs from it.

The five workloads stand in for the pages' training runs (fms-acceleration PR
#79, tables "Improvements to Full Finetuning" and "FLAN (6000 samples) with
PaddingFree": Mistral-7B, batch 4, padding-free packed FLAN/alpaca batches);
no dataset or model weights are used.  Logits are i.i.d. normal, which gives
the same bytes, shapes and value ranges as real lm-head outputs.

Recipe (all draws from numpy PCG64):
  * logits are drawn in blocks of BLOCK_ROWS rows; block b uses the seed
    sequence (seed, 1, b), so any subset of rows can be regenerated alone and
    blocks can be drawn in parallel.  Each value is a float64 standard normal
    times sigma, rounded to float32 (nearest-even), then to the storage format
    (nearest-even).  16-bit formats are returned as uint16 bit patterns.
  * labels, ignored rows, sequence lengths and spikes come from the seed
    sequence (seed, 2), in that order.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK_ROWS = 64
IGNORE_INDEX = -100


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    N: int
    V: int
    dtype: str            # 'f32' | 'bf16' | 'f16'
    sigma: float
    ignore_frac: float
    dloss: float = 1.0
    chunk: int = 0
    labels_kind: str = "uniform"   # 'uniform' | 'zipf' | 'packed'
    zipf_s: float = 1.1
    spike_frac: float = 0.0
    spike_value: float = 60.0
    pack_min: int = 64
    pack_max: int = 1024

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    1: Workload("tiny-f32", 1, 64, 1000, "f32", 1.0, 0.10),
    2: Workload("mistral7b-b4s1024-bf16", 2, 4096, 32000, "bf16", 2.0, 0.05),
    3: Workload("packed-8192-bf16", 3, 8192, 32000, "bf16", 2.0, 0.15, labels_kind="packed"),
    4: Workload("llama3-vocab128k-bf16", 4, 8192, 128256, "bf16", 3.0, 0.05, chunk=65536,
                labels_kind="zipf"),
    5: Workload("stress-f16", 5, 16384, 49152, "f16", 30.0, 0.20, dloss=0.5, spike_frac=0.10),
}


def custom(name: str, seed: int, N: int, V: int, dtype: str, sigma: float = 2.0,
           ignore_frac: float = 0.05, **kw) -> Workload:
    """A workload of any shape with the same recipe (for edge and tile tests)."""
    return Workload(name, seed, N, V, dtype, sigma, ignore_frac, **kw)


# ---------------------------------------------------------------------------
# storage-format conversion of generated values (input construction only)
# ---------------------------------------------------------------------------

def _f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16      # nearest-even on the dropped half
    return u.astype(np.uint16)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> float32 (nearest-even) -> storage format (nearest-even)."""
    f = x64.astype(np.float32)
    if dtype == "f32":
        return f
    if dtype == "bf16":
        return _f32_to_bf16_bits(f)
    if dtype == "f16":
        return f.astype(np.float16).view(np.uint16)
    raise ValueError(dtype)


def storage_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


# ---------------------------------------------------------------------------
# labels and row structure
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Plan:
    labels: np.ndarray            # int64 [N]
    seq_starts: np.ndarray        # int64, first row of each packed sequence (packed only)
    spike_rows: np.ndarray        # int64 rows given a spike
    spike_cols: np.ndarray        # int64 column of each spike


def plan(w: Workload) -> Plan:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 2])))
    N, V = w.N, w.V
    if w.labels_kind == "zipf":
        k = np.arange(V, dtype=np.float64)
        wts = (k + 1.0) ** (-w.zipf_s)
        cdf = np.cumsum(wts)
        cdf /= cdf[-1]
        u = rng.random(N)
        labels = np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int64)
    else:
        labels = rng.integers(0, V, size=N, dtype=np.int64)
    seq_starts = np.zeros(0, np.int64)
    if w.labels_kind == "packed":
        starts, pos = [], 0
        while pos < N:
            starts.append(pos)
            pos += int(rng.integers(w.pack_min, w.pack_max + 1))
        seq_starts = np.asarray(starts, np.int64)
        labels[seq_starts] = IGNORE_INDEX
        others = np.setdiff1d(np.arange(N, dtype=np.int64), seq_starts)
        k_ign = int(round(w.ignore_frac * N))
        ign = rng.choice(others, size=min(k_ign, others.size), replace=False)
    else:
        k_ign = int(round(w.ignore_frac * N))
        ign = rng.choice(N, size=k_ign, replace=False)
    labels[ign] = IGNORE_INDEX
    spike_rows = np.zeros(0, np.int64)
    spike_cols = np.zeros(0, np.int64)
    if w.spike_frac > 0:
        valid = np.flatnonzero(labels != IGNORE_INDEX)
        k_sp = min(int(round(w.spike_frac * N)), valid.size)
        spike_rows = rng.choice(valid, size=k_sp, replace=False).astype(np.int64)
        half = k_sp // 2
        cols = labels[spike_rows].copy()
        # the second half: a uniform column other than the label
        other = rng.integers(0, V - 1, size=k_sp - half, dtype=np.int64)
        other = other + (other >= cols[half:])
        cols[half:] = other
        spike_cols = cols
    return Plan(labels, seq_starts, spike_rows, spike_cols)


# ---------------------------------------------------------------------------
# logits
# ---------------------------------------------------------------------------

def _block(w: Workload, b: int) -> np.ndarray:
    r0 = b * BLOCK_ROWS
    r1 = min(w.N, r0 + BLOCK_ROWS)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 1, b])))
    x = rng.standard_normal((r1 - r0) * w.V)
    x *= w.sigma
    return to_storage(x, w.dtype).reshape(r1 - r0, w.V)


def _apply_spikes(w: Workload, p: Plan, rows: np.ndarray, out: np.ndarray) -> None:
    if p.spike_rows.size == 0:
        return
    val = to_storage(np.array([w.spike_value]), w.dtype)[0]
    pos = {int(r): i for i, r in enumerate(rows)}
    for r, c in zip(p.spike_rows, p.spike_cols):
        i = pos.get(int(r))
        if i is not None:
            out[i, c] = val


def logits(w: Workload, rows=None, p: Plan | None = None, threads: int | None = None,
           out: np.ndarray | None = None) -> np.ndarray:
    """Logit rows (all when rows is None) as a [len(rows), V] storage array."""
    p = p or plan(w)
    if rows is None:
        rows = np.arange(w.N, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    if out is None:
        out = np.empty((rows.size, w.V), storage_dtype(w.dtype))
    blocks = sorted(set((rows // BLOCK_ROWS).tolist()))
    threads = threads or min(16, os.cpu_count() or 1)
    full = rows.size == w.N and np.array_equal(rows, np.arange(w.N))

    def work(b):
        blk = _block(w, b)
        if full:
            out[b * BLOCK_ROWS: b * BLOCK_ROWS + blk.shape[0]] = blk
        else:
            sel = np.flatnonzero(rows // BLOCK_ROWS == b)
            out[sel] = blk[rows[sel] - b * BLOCK_ROWS]

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, blocks))
    _apply_spikes(w, p, rows, out)
    return out


def make(w: Workload, threads: int | None = None):
    """(logits [N, V] storage array, Plan) for the whole workload."""
    p = plan(w)
    return logits(w, None, p, threads), p


# ---------------------------------------------------------------------------
# LM-head projection inputs: hidden states h [N, H] and the weight W [V, H] of
# a bias-free linear layer (the Mistral-7B head: hidden 4096, vocabulary
# 32000).  Hidden values are standard normal; weights are normal with
# standard deviation sigma_w / sqrt(H), so the logits h W^T have standard
# deviation ~sigma_w, like the cross-entropy workloads above.
# Recipe: hidden rows in blocks of BLOCK_ROWS drawn from (seed, 3, b), weight
# rows from (seed, 4, b), labels and ignored rows from (seed, 2); every value
# is rounded float64 -> float32 -> storage format (nearest-even).
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class LinearWorkload:
    name: str
    seed: int
    N: int
    H: int
    V: int
    dtype: str
    sigma_w: float = 2.0
    ignore_frac: float = 0.05
    dloss: float = 1.0
    chunk_rows: int = 0  # 0: the library's default (4096 rows)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


LINEAR_WORKLOADS = {
    1: LinearWorkload("mistral7b-lmhead-b4s1024-bf16", 6, 4096, 4096, 32000, "bf16"),
    # a Llama-3-8B head (hidden 4096, vocabulary 128256) over the large-vocabulary cross-entropy
    # shape's 8192 rows (numbered as that shape, 4): g alone is 2.1 GB, the logits the fused path never stores
    4: LinearWorkload("llama3-lmhead-b8s1024-bf16", 7, 8192, 4096, 128256, "bf16"),
}


def _normal_rows(seed: int, stream: int, rows: int, cols: int, scale: float, dtype: str, threads: int):
    out = np.empty((rows, cols), storage_dtype(dtype))

    def work(b):
        r0 = b * BLOCK_ROWS
        n = min(BLOCK_ROWS, rows - r0)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence((seed, stream, b))))
        out[r0:r0 + n] = to_storage(rng.standard_normal((n, cols)) * scale, dtype)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, range((rows + BLOCK_ROWS - 1) // BLOCK_ROWS)))
    return out


def linear_inputs(lw: LinearWorkload, threads: int | None = None):
    """(hidden [N, H], weight [V, H], labels [N]) storage arrays."""
    threads = threads or min(16, os.cpu_count() or 1)
    h = _normal_rows(lw.seed, 3, lw.N, lw.H, 1.0, lw.dtype, threads)
    w = _normal_rows(lw.seed, 4, lw.V, lw.H, lw.sigma_w / np.sqrt(lw.H), lw.dtype, threads)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence((lw.seed, 2))))
    y = rng.integers(0, lw.V, lw.N)
    ign = rng.choice(lw.N, int(round(lw.ignore_frac * lw.N)), replace=False)
    y[ign] = IGNORE_INDEX
    return h, w, y


@dataclasses.dataclass(frozen=True)
class NormWorkload:
    """RMSNorm over the hidden states: N token rows of H elements, a weight of
    H elements and an upstream gradient of the output's shape."""
    name: str
    seed: int
    N: int
    H: int
    dtype: str
    eps: float = 1e-5

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


NORM_WORKLOADS = {
    # a Mistral-7B decoder norm (hidden 4096, eps 1e-5) over batch 4 x sequence 1024
    1: NormWorkload("mistral7b-rmsnorm-b4s1024-bf16", 8, 4096, 4096, "bf16"),
}


def norm_inputs(nw: NormWorkload, threads: int | None = None):
    """(x [N, H], weight [H], dy [N, H]) storage arrays: x and dy iid N(0, 1),
    the weight 1 + N(0, 0.25^2) (a trained norm's weights sit around one)."""
    threads = threads or min(16, os.cpu_count() or 1)
    x = _normal_rows(nw.seed, 5, nw.N, nw.H, 1.0, nw.dtype, threads)
    dy = _normal_rows(nw.seed, 6, nw.N, nw.H, 1.0, nw.dtype, threads)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence((nw.seed, 7))))
    w = to_storage(1.0 + 0.25 * rng.standard_normal(nw.H), nw.dtype)
    return x, w, dy


@dataclasses.dataclass(frozen=True)
class RopeWorkload:
    """Rotary embedding of one attention layer's q and k over a padding-free
    packed batch: T tokens, Hq query heads and Hk key heads of head_dim D;
    positions restart at every packed sequence (lengths uniform in
    [min_len, max_len], the last one cut at T)."""
    name: str
    seed: int
    T: int
    Hq: int
    Hk: int
    D: int
    dtype: str
    base: float = 10000.0
    min_len: int = 64
    max_len: int = 1024

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


ROPE_WORKLOADS = {
    # Mistral-7B attention: 32 query heads, 8 key heads, head_dim 128, rope base 10000
    1: RopeWorkload("mistral7b-rope-packed4096-bf16", 9, 4096, 32, 8, 128, "bf16"),
}


def packed_positions(seed: int, T: int, min_len: int, max_len: int) -> np.ndarray:
    """Positions of a packed batch: 0, 1, ... restarting at each sequence."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence((seed, 10))))
    out, n = [], 0
    while n < T:
        L = int(min(rng.integers(min_len, max_len + 1), T - n))
        out.append(np.arange(L, dtype=np.int64))
        n += L
    return np.concatenate(out)


def rope_inputs(rw: RopeWorkload, threads: int | None = None):
    """(q [T, Hq, D], k [T, Hk, D], positions [T]) storage arrays, q and k iid N(0, 1)."""
    threads = threads or min(16, os.cpu_count() or 1)
    q = _normal_rows(rw.seed, 11, rw.T, rw.Hq * rw.D, 1.0, rw.dtype, threads).reshape(rw.T, rw.Hq, rw.D)
    k = _normal_rows(rw.seed, 12, rw.T, rw.Hk * rw.D, 1.0, rw.dtype, threads).reshape(rw.T, rw.Hk, rw.D)
    return q, k, packed_positions(rw.seed, rw.T, rw.min_len, rw.max_len)
