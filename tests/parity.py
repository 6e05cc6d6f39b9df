"""Helpers of the parity tests: oracle-side inputs, tolerances, selection checks.

All expected values come from the fp64 oracle on the same stored inputs the GPU
sees; nothing here reads a GPU result back into an oracle input."""
from __future__ import annotations

import numpy as np

from oracle import ref
from selective_recompute_prefill_amd import inputs

# Tolerances: rel-L2 and max-abs per output, by storage dtype.
TOL = {"bf16": (1e-2, 3e-2), "f32": (1e-5, 1e-5)}
# The fixed max-abs bound holds for unit-scale operands (|K|, |V| below about 4 on
# the workloads' selections). bf16 rounding errors grow with the magnitude of the
# operands (a store of v errs by up to |v| 2^-9; rounded queries and probabilities
# perturb an attention row in proportion to its values), so where large-magnitude
# rows stay in the cache the bound scales: max-abs <= bound * max(1, mag / MAG_UNIT),
# mag = the stored value itself for K/V, the largest |V| among the row's visible keys
# for attention.
MAG_UNIT = 4.0
NEAR_TIE = 1e-4  # relative deviation gap below which two candidates may swap


def oracle_caches(w: inputs.Workload, layer: int = 0, x_full=None):
    """Stored chunk caches of `layer`: the oracle encodes (x + eps n) at the encode
    positions in fp64, then the values are rounded to the storage dtype."""
    spec, lay = w.spec, w.layout
    src = inputs.encode_positions(lay)
    cr = src >= 0
    wq = ref.widen(w.layers[layer].w_qkv, spec.dtype)
    xe = w.encode_input(layer, x_full)
    T = lay.total_rows
    kc = np.zeros((T, spec.n_kv_heads, spec.head_dim))
    vc = np.zeros_like(kc)
    if cr.any():
        kc[cr], vc[cr] = ref.encode_kv(xe[cr], wq, src[cr], spec.n_heads, spec.n_kv_heads,
                                       spec.head_dim, spec.rope_base)
    return inputs.store(kc, spec.dtype), inputs.store(vc, spec.dtype)


def oracle_layer(spec, lay, hidden_st, wq_st, kc_st, vc_st, **kw):
    """Oracle layer on stored inputs (widened exactly to fp64)."""
    args = dict(hidden=ref.widen(hidden_st, spec.dtype), w_qkv=ref.widen(wq_st, spec.dtype),
                k_cache=ref.widen(kc_st, spec.dtype), v_cache=ref.widen(vc_st, spec.dtype),
                req_offsets=lay.req_offsets, chunk_offsets=lay.chunk_offsets,
                chunk_src_pos=lay.chunk_src_pos, positions=lay.positions,
                n_heads=spec.n_heads, n_kv=spec.n_kv_heads, head_dim=spec.head_dim,
                rope_base=spec.rope_base, ratio=spec.ratio, window=spec.window, tau=spec.tau)
    args.update(kw)
    return ref.fuse_layer(**args)


def gpu_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return ref.widen(a, dtype)


def assert_close(got: np.ndarray, want: np.ndarray, dtype: str, what: str, mag=None):
    rl, ma = TOL[dtype]
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if want.size == 0:
        return
    err = got - want
    nrm = np.linalg.norm(want)
    rel = np.linalg.norm(err) / (nrm if nrm > 0 else 1.0)
    bound = ma * np.maximum(1.0, np.broadcast_to(mag, want.shape) / MAG_UNIT) if mag is not None \
        else np.full(want.shape, ma)
    worst = int(np.argmax(np.abs(err) - bound))
    mx, bw = float(np.abs(err).flat[worst]), float(bound.flat[worst])
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert rel <= rl and mx <= bw, (f"{what}: rel-L2 {rel:.3e} (<= {rl}), abs err {mx:.3e} at "
                                    f"|value| {abs(float(want.flat[worst])):.3g} (<= {bw:.3e})")


def visible_vmax(v_cache: np.ndarray, rows: np.ndarray, req_offsets, n_heads: int) -> np.ndarray:
    """[len(rows), n_heads, 1]: the largest |V| of head h's KV group over the keys row
    j sees (its request's rows up to j; positions ascend with rows in a request)."""
    nkv = v_cache.shape[1]
    m = np.abs(v_cache).max(axis=2)  # [T, nkv]
    pm = np.empty_like(m)
    for r in range(len(req_offsets) - 1):
        a, b = int(req_offsets[r]), int(req_offsets[r + 1])
        if b > a:
            pm[a:b] = np.maximum.accumulate(m[a:b], axis=0)
    g = (np.arange(n_heads) * nkv) // n_heads
    return pm[np.asarray(rows, np.int64)][:, g][:, :, None]


def check_selection(gpu_sel: np.ndarray, ref_out: dict, req_of_row: np.ndarray, what: str):
    """The GPU's selected set equals the oracle's except for near-ties: each request
    selects exactly as many rows as in the oracle's result, and every row in the
    symmetric difference is a candidate whose oracle deviation lies within NEAR_TIE
    (relative) of its request's k-th largest. Returns the swapped rows."""
    ga = np.asarray(gpu_sel, np.int64)
    gb = np.asarray(ref_out["sel_idx"], np.int64)
    n_req = int(req_of_row.max(initial=-1)) + 1
    ca = np.bincount(req_of_row[ga], minlength=n_req)
    cb = np.bincount(req_of_row[gb], minlength=n_req)
    bad = np.nonzero(ca != cb)[0]
    assert len(bad) == 0, (f"{what}: request {int(bad[0])} selects {int(ca[bad[0]])} rows, the "
                           f"oracle {int(cb[bad[0]])}")
    a, b = set(ga.tolist()), set(gb.tolist())
    sym = sorted(a ^ b)
    for j in sym:
        r = int(req_of_row[j])
        dk = ref_out["kth"][r]
        dj = ref_out["dev"][j]
        assert np.isfinite(dj) and np.isfinite(dk) and dk > 0, f"{what}: row {j} differs and is not a scored candidate"
        assert abs(dj - dk) / dk < NEAR_TIE, f"{what}: row {j} differs (dev {dj} vs k-th {dk})"
    return sym


def attn_tile_rows(dtype: str, n_heads: int, n_kv: int) -> int:
    """Selected rows per attention work-group tile of the library for this shape:
    bf16 packs the (query, head) pairs of a KV group into 256 columns, so
    floor(256 / G) queries for G = n_heads / n_kv; fp32 takes 32."""
    return 256 // (n_heads // n_kv) if dtype == "bf16" else 32


def tile_sample(sel_offsets, tile_rows: int, extra: int = 16, seed: int = 0) -> np.ndarray:
    """Positions into sel_idx that hit every attention tile: the first and last row
    of each tile of each request (tiles are runs of tile_rows selected rows from the
    request's first one), plus `extra` seeded positions inside tiles."""
    off = np.asarray(sel_offsets, np.int64)
    pos = []
    for r in range(len(off) - 1):
        a, b = int(off[r]), int(off[r + 1])
        for t in range(a, b, tile_rows):
            pos += [t, min(t + tile_rows, b) - 1]
    n = int(off[-1])
    if n and extra:
        pos += np.random.default_rng(seed).integers(0, n, extra).tolist()
    return np.unique(np.asarray(pos, np.int64))


def csr_ok(sel: np.ndarray, off: np.ndarray, req_offsets: np.ndarray):
    """Selected rows ascend inside each request and lie in it."""
    for r in range(len(req_offsets) - 1):
        s = sel[off[r]:off[r + 1]]
        assert np.all(np.diff(s) > 0)
        if len(s):
            assert s[0] >= req_offsets[r] and s[-1] < req_offsets[r + 1]
