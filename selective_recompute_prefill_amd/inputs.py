"""Seeded synthetic workloads for the selective-recompute prefill layer.

This module only draws random numbers and lays out integer index arrays. It holds
none of the layer's arithmetic: no rotary embedding, no projection, no deviation,
no selection and no attention. Both the fp64 CPU oracle and the HIP library are fed
from here; whatever a workload needs beyond raw draws (the chunk-local caches) is
produced by each side from these draws.

Workload recipe (the shapes follow the pages' RAG setups: 512-token chunks and six
retrieved chunks in the CacheBlend walkthrough, 16K-token inputs and a 20% ratio in
the CacheClip paper's latency table, 15% as CacheBlend's quality floor):

* hidden X ~ N(0, 1) of shape [T, H] (query tail included);
* W_q, W_k, W_v ~ N(0, 1/H), each stored as [out_features, H];
* per cached row, noise n ~ N(0, 1) of shape [H] and a scale eps ~ lognormal(-3, 1),
  i.i.d. over rows, so the chunk caches are the projection of X + eps * n encoded at
  the chunk-local positions (the perturbation stands in for the missing cross-chunk
  attention of an independently encoded chunk);
* draw order X, W_q, W_k, W_v, n, eps, then permutations; multi-layer stacks draw
  X then (W_q, W_k, W_v, n, eps) per layer; the seed is 20260000 + config id;
* external importance scores (selection by a small model's scores) come from
  draw_scores, a stream of their own: units of 1-6 rows at a lognormal(0, 0.5)
  level with 2% per-row jitter.

Storage: fp32 workloads keep float32 arrays; bf16 workloads keep uint16 bit patterns
(value rounded to float32, then to bfloat16, each round-to-nearest-even). The
encode input X + eps*n is returned in float64 and is never rounded.

Layout (CacheClip paper, section 4.1, "Position ID rearrangement"; CacheBlend
walkthrough, "Selective KV recompute"): rows are partitioned into requests
(req_offsets, CSR) and into segments (chunk_offsets, CSR). A segment is either a
cached chunk, whose first row was encoded at position chunk_src_pos[c], or a fresh
segment (chunk_src_pos[c] = -1) such as the query tail, which has no cache. With a
shared prefix, the first chunk carries the one kept prefix copy and was encoded at
position 0; every later chunk was encoded right after its own (dropped) prefix copy,
at position P. Global positions are 0..n-1 within each request.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

SEED_BASE = 20260000


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and selection parameters of one synthetic workload."""

    name: str
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str  # "f32" or "bf16"
    prefix: int  # shared-prefix rows kept in front of the first chunk (0 = none)
    chunk_lens: tuple  # rows per chunk (per request, before permutation)
    n_query: int  # fresh query-tail rows per request
    n_req: int = 1
    ratio: float = 0.2
    ratios: tuple = ()  # per-layer ratios for stacks; empty = (ratio,)
    window: int = 0  # sliding-window grouping size (0 = off)
    tau: int = 0  # grouping density threshold
    n_layers: int = 1
    rope_base: float = 10000.0
    shared_chunks: bool = False  # all requests draw from one chunk pool, permuted
    seed: int = SEED_BASE

    @property
    def qdim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kvdim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def rows_per_req(self) -> int:
        return self.prefix + sum(self.chunk_lens) + self.n_query

    @property
    def ctx_per_req(self) -> int:
        return self.prefix + sum(self.chunk_lens)

    @property
    def total_rows(self) -> int:
        return self.n_req * self.rows_per_req

    def layer_ratios(self) -> tuple:
        return tuple(self.ratios) if self.ratios else (self.ratio,) * self.n_layers

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


# The five workloads (shapes, sizes and ratios of the pages' setups), by id.
WORKLOADS: Dict[int, Spec] = {
    0: Spec("tiny-fp32", 256, 4, 2, 64, "f32", prefix=32, chunk_lens=(128,) * 4,
            n_query=32, ratio=0.20, seed=SEED_BASE + 0),
    1: Spec("llama3-8b-layer", 4096, 32, 8, 128, "bf16", prefix=0,
            chunk_lens=(512,) * 6, n_query=64, ratio=0.15, seed=SEED_BASE + 1),
    2: Spec("14b-16k-grouped", 5120, 40, 8, 128, "bf16", prefix=32,
            chunk_lens=(512,) * 32, n_query=96, ratio=0.20, window=8, tau=4,
            seed=SEED_BASE + 2),
    3: Spec("70b-4layer-gradual", 8192, 64, 8, 128, "bf16", prefix=0,
            chunk_lens=(512,) * 8, n_query=64, ratio=0.30,
            ratios=(0.30, 0.15, 0.15, 0.15), n_layers=4, seed=SEED_BASE + 3),
    4: Spec("8b-batch16x8k", 4096, 32, 8, 128, "bf16", prefix=0,
            chunk_lens=(512,) * 16, n_query=0, n_req=16, ratio=0.20,
            shared_chunks=True, seed=SEED_BASE + 4),
}

# Ratios swept on the batched workload.
BATCH_RATIOS = (0.05, 0.10, 0.20, 0.35, 0.50)


def small_spec(name: str = "mini", **kw) -> Spec:
    """A small bf16 workload the oracle finishes in well under a second: two
    requests, ragged chunk lengths, several GEMM/attention tiles per request."""
    base = dict(hidden=512, n_heads=8, n_kv_heads=2, head_dim=128, dtype="bf16",
                prefix=16, chunk_lens=(200, 137, 250), n_query=45, n_req=2,
                ratio=0.2, seed=SEED_BASE + 100)
    base.update(kw)
    return Spec(name, **base)


# --------------------------------------------------------------------------- #
# storage helpers (bit-level format conversion only)
# --------------------------------------------------------------------------- #

def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float -> bfloat16 bit patterns (uint16): round to float32, then to bf16,
    both round-to-nearest-even. NaN is not expected in generated data."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float array to the workload's storage format."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16_bits(x)
    raise ValueError(dtype)


def stored_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of a stored array to float64 (used to build encode inputs)."""
    if dtype == "f32":
        return a.astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------- #
# layout
# --------------------------------------------------------------------------- #

@dataclasses.dataclass
class Layout:
    req_offsets: np.ndarray  # int32 [n_req+1]
    chunk_offsets: np.ndarray  # int32 [n_segments+1]
    chunk_src_pos: np.ndarray  # int32 [n_segments], -1 for fresh segments
    positions: np.ndarray  # int32 [T]
    # bookkeeping for the generator itself
    chunk_ids: np.ndarray  # int32 [n_segments]: pool chunk id, -1 fresh
    max_position: int

    @property
    def n_req(self) -> int:
        return len(self.req_offsets) - 1

    @property
    def total_rows(self) -> int:
        return int(self.req_offsets[-1])


def make_layout(spec: Spec, perms: Optional[Sequence[Sequence[int]]] = None) -> Layout:
    """CSR layout of requests and segments. perms[r] permutes the chunk order of
    request r (the pool chunk placed in each slot)."""
    req_off = [0]
    seg_off = [0]
    seg_src: List[int] = []
    seg_id: List[int] = []
    pos: List[np.ndarray] = []
    n_ch = len(spec.chunk_lens)
    for r in range(spec.n_req):
        order = list(perms[r]) if perms is not None else list(range(n_ch))
        row = req_off[-1]
        p = 0
        for slot, cid in enumerate(order):
            ln = spec.chunk_lens[cid]
            if slot == 0 and spec.prefix:
                ln += spec.prefix
                src = 0  # the one kept prefix copy: encoded together at 0
            else:
                src = spec.prefix  # encoded right after its own prefix copy
            seg_src.append(src)
            seg_id.append(cid)
            row += ln
            p += ln
            seg_off.append(row)
        if spec.n_query:
            seg_src.append(-1)
            seg_id.append(-1)
            row += spec.n_query
            p += spec.n_query
            seg_off.append(row)
        pos.append(np.arange(p, dtype=np.int32))
        req_off.append(row)
    positions = np.concatenate(pos) if pos else np.zeros(0, np.int32)
    max_pos = int(max(positions.max(initial=0) + 1, spec.prefix + max(spec.chunk_lens, default=0)))
    return Layout(np.asarray(req_off, np.int32), np.asarray(seg_off, np.int32),
                  np.asarray(seg_src, np.int32), positions.astype(np.int32),
                  np.asarray(seg_id, np.int32), max_pos)


def cached_rows(layout: Layout) -> np.ndarray:
    """Row ids covered by cached segments, ascending (bookkeeping, no arithmetic)."""
    out = []
    for c in range(len(layout.chunk_src_pos)):
        if layout.chunk_src_pos[c] >= 0:
            out.append(np.arange(layout.chunk_offsets[c], layout.chunk_offsets[c + 1]))
    return np.concatenate(out).astype(np.int64) if out else np.zeros(0, np.int64)


def encode_positions(layout: Layout) -> np.ndarray:
    """Position at which each cached row was encoded (-1 for fresh rows)."""
    src = np.full(layout.total_rows, -1, np.int64)
    for c in range(len(layout.chunk_src_pos)):
        s = int(layout.chunk_src_pos[c])
        if s >= 0:
            a, b = int(layout.chunk_offsets[c]), int(layout.chunk_offsets[c + 1])
            src[a:b] = s + np.arange(b - a)
    return src


# --------------------------------------------------------------------------- #
# draws
# --------------------------------------------------------------------------- #

@dataclasses.dataclass
class LayerDraws:
    w_qkv: np.ndarray  # stored [(nh+2nkv)*d, H]: Q rows, then K rows, then V rows
    noise: np.ndarray  # float64 [n_cache_rows, H]
    eps: np.ndarray  # float64 [n_cache_rows]


@dataclasses.dataclass
class Workload:
    spec: Spec
    layout: Layout
    hidden: np.ndarray  # stored [T, H]
    layers: List[LayerDraws]
    # For shared-chunk workloads, noise/eps are drawn per pool row and
    # cache_row_of[j] maps batch row j to its pool row (-1 for fresh rows);
    # otherwise pool rows are the batch's cached rows in order.
    cache_row_of: np.ndarray

    def encode_input(self, layer: int = 0, x_full: Optional[np.ndarray] = None) -> np.ndarray:
        """float64 [T, H] input the chunk caches of `layer` were encoded from:
        (x + eps * n) on cached rows, where x is the stored hidden upcast
        (layer 0) or the caller-supplied full-prefill hidden of that layer.
        Fresh rows are zero (they have no cache)."""
        ld = self.layers[layer]
        x = stored_to_f64(self.hidden, self.spec.dtype) if x_full is None else x_full
        out = np.zeros((self.layout.total_rows, self.spec.hidden), np.float64)
        m = self.cache_row_of >= 0
        rows = np.nonzero(m)[0]
        pr = self.cache_row_of[rows]
        out[rows] = x[rows] + ld.eps[pr, None] * ld.noise[pr]
        return out


def _normal(rng, shape, std=1.0):
    return rng.standard_normal(shape) * std


def paged_layout(layout: "Layout", block_rows: int = 16, seed: int = 1, spare: int = 5):
    """A block pool for the layout's cache rows (Cache-Craft summary, section 4: each
    chunk maps to 16-token memory blocks, padded at its end): segment c takes
    ceil(len_c / block_rows) blocks, placed at shuffled pool positions among `spare`
    unused ones. Returns seg_block (int32 [n_chunks], index of each segment's first
    table entry), block_table (int32), the pool row of every batch row (int64 [T])
    and the pool's row count. Index arrays only."""
    co = np.asarray(layout.chunk_offsets, np.int64)
    lens = np.diff(co)
    nb = (lens + block_rows - 1) // block_rows
    seg_block = np.concatenate([[0], np.cumsum(nb)[:-1]]).astype(np.int32)
    total = int(nb.sum())
    rng = np.random.default_rng(seed)
    table = rng.permutation(total + spare)[:total].astype(np.int32)
    slot = np.zeros(layout.total_rows, np.int64)
    for c in range(len(lens)):
        i = np.arange(lens[c])
        slot[co[c] + i] = table[seg_block[c] + i // block_rows] * block_rows + i % block_rows
    return seg_block, table, slot, (total + spare) * block_rows


def draw_scores(n_rows: int, seed: int, unit_max: int = 6, spread: float = 0.5,
                jitter: float = 0.02) -> np.ndarray:
    """Seeded per-row importance scores as a small auxiliary model would hand them
    over (deep-layer hidden-state norms, SpecCache notes 2.2; attention column means,
    CacheClip paper 4.2): positive, and shaped into multi-token units of 1..unit_max
    rows that share a lognormal(0, spread) level up to a relative jitter, so that
    smooth spans and sharp edges both occur. float32 [n_rows]; the draws only."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(1, unit_max + 1, n_rows + 1)
    levels = rng.lognormal(0.0, spread, n_rows + 1)
    base = np.repeat(levels, lens)[:n_rows]
    noise = rng.standard_normal(n_rows)
    return (base * (1.0 + jitter * noise)).astype(np.float32)


def generate(spec: Spec) -> Workload:
    """Draw the workload of `spec` (deterministic for its seed)."""
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    H = spec.hidden
    wstd = 1.0 / np.sqrt(H)

    if spec.shared_chunks:
        pool_lens = spec.chunk_lens
        pool_off = np.concatenate([[0], np.cumsum(pool_lens)]).astype(np.int64)
        x_pool = _normal(rng, (int(pool_off[-1]), H))
        layers = []
        for _ in range(spec.n_layers):
            wq = _normal(rng, (spec.qdim, H), wstd)
            wk = _normal(rng, (spec.kvdim, H), wstd)
            wv = _normal(rng, (spec.kvdim, H), wstd)
            n = _normal(rng, (int(pool_off[-1]), H))
            eps = rng.lognormal(-3.0, 1.0, int(pool_off[-1]))
            layers.append(LayerDraws(store(np.concatenate([wq, wk, wv]), spec.dtype), n, eps))
        perms = [rng.permutation(len(pool_lens)) for _ in range(spec.n_req)]
        layout = make_layout(spec, perms)
        T = layout.total_rows
        cache_row_of = np.full(T, -1, np.int64)
        x_rows = np.zeros(T, np.int64)
        has_x = np.zeros(T, bool)
        for c in range(len(layout.chunk_src_pos)):
            cid = int(layout.chunk_ids[c])
            a, b = int(layout.chunk_offsets[c]), int(layout.chunk_offsets[c + 1])
            if cid >= 0:
                cache_row_of[a:b] = pool_off[cid] + np.arange(b - a)
                x_rows[a:b] = cache_row_of[a:b]
                has_x[a:b] = True
        if not has_x.all():
            raise ValueError("shared-chunk workloads carry no query tail")
        hidden = store(x_pool, spec.dtype)[x_rows]
        return Workload(spec, layout, hidden, layers, cache_row_of)

    layout = make_layout(spec)
    T = layout.total_rows
    x = _normal(rng, (T, H))
    cached = cached_rows(layout)
    layers = []
    for _ in range(spec.n_layers):
        wq = _normal(rng, (spec.qdim, H), wstd)
        wk = _normal(rng, (spec.kvdim, H), wstd)
        wv = _normal(rng, (spec.kvdim, H), wstd)
        n = _normal(rng, (len(cached), H))
        eps = rng.lognormal(-3.0, 1.0, len(cached))
        layers.append(LayerDraws(store(np.concatenate([wq, wk, wv]), spec.dtype), n, eps))
    cache_row_of = np.full(T, -1, np.int64)
    cache_row_of[cached] = np.arange(len(cached))
    return Workload(spec, layout, store(x, spec.dtype), layers, cache_row_of)
