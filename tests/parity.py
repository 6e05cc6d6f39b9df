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
# the workloads' selections). A bf16 store of a value v errs by up to |v| 2^-9, so
# where large-magnitude rows stay in the cache (a choice by external scores) the
# bound on cache rows scales: max-abs <= bound * max(1, |v| / MAG_UNIT), which is
# 3.8 times the storage rounding. Attention rows there use the derived bound below.
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


# Attention with a choice by external scores (high-noise rows stay in the cache).
# The kernel rounds to bf16 (u = 2^-9, round to nearest even) the queries, the keys
# and values as the cache stores them, the probabilities that enter the PV product,
# and the output. To first order the output error of row j, head h is
#   sum_i p_i (v_i - o) ds_i + sum_i p_i v_i (g_i + e_i) + o n,
# ds_i = (q (a) . k_i + q . k_i (b_i)) / sqrt(d) with relative rounding errors a (of
# the query, shared by every key), b_i, g_i, e_i, n. Taking them independent and
# uniform on [-u, u] (variance u^2 / 3) gives a standard deviation per output element
# (attn_sigma). Where the fixed max-abs bound does not hold, an element may err by up
# to ATTN_Z of those deviations: a simulation of these rounding points reproduces the
# kernel's errors and stays within 5.2 deviations wherever they exceed 3e-2.
BF16_U = 2.0 ** -9
ATTN_Z = 8.0


def attn_sigma(q: np.ndarray, K: np.ndarray, V: np.ndarray, o: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Standard deviation [nh, d] of the bf16 rounding error of one attention row (model
    above): q [nh, d] the row's roped query, K/V [T, nkv, d] the fused caches, o
    [nh, d] the exact output, keys the rows it sees. All from the oracle (fp64)."""
    nh, d = q.shape
    nkv = K.shape[1]
    cs = 1.0 / np.sqrt(d)
    out = np.zeros_like(o)
    for h in range(nh):
        g = (h * nkv) // nh
        k, v = K[keys, g], V[keys, g]
        s = (k @ q[h]) * cs
        p = np.exp(s - s.max())
        p /= p.sum()
        dv = v - o[h][None, :]
        gq = cs * (k.T @ (p[:, None] * dv))                     # d(o) / d(q), [d, d]
        q_term = ((q[h] ** 2)[:, None] * gq ** 2).sum(0)
        k_term = cs ** 2 * (((p ** 2) * ((k * q[h][None, :]) ** 2).sum(1))[:, None] * dv ** 2).sum(0)
        pv_term = 2.0 * ((p ** 2)[:, None] * v ** 2).sum(0)
        out[h] = np.sqrt(BF16_U ** 2 / 3.0 * (q_term + k_term + pv_term + o[h] ** 2))
    return out


def assert_attention_bf16_scores(got: np.ndarray, want: np.ndarray, q: np.ndarray, K: np.ndarray,
                                 V: np.ndarray, rows: np.ndarray, req_offsets, positions, what: str):
    """Attention rows of a choice by external scores: rel-L2 <= 1e-2 overall; max-abs
    <= 3e-2, or <= ATTN_Z x attn_sigma where that is larger (computed only for rows
    that exceed 3e-2). got/want/q: [n, nh, d] for the selected rows `rows`."""
    rl, ma = TOL["bf16"]
    got = np.asarray(got, np.float64)
    assert got.shape == want.shape and np.isfinite(got).all(), what
    if want.size == 0:
        return
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    assert rel <= rl, f"{what}: rel-L2 {rel:.3e} (<= {rl})"
    err = np.abs(got - want)
    req_of = np.searchsorted(np.asarray(req_offsets), rows, side="right") - 1
    pos = np.asarray(positions)
    for i in np.nonzero(err.reshape(len(rows), -1).max(axis=1) > ma)[0]:
        j, r = int(rows[i]), int(req_of[i])
        span = np.arange(int(req_offsets[r]), int(req_offsets[r + 1]))
        keys = span[pos[span] <= pos[j]]
        bound = np.maximum(ma, ATTN_Z * attn_sigma(q[i], K, V, want[i], keys))
        worst = np.unravel_index(int(np.argmax(err[i] - bound)), bound.shape)
        assert err[i][worst] <= bound[worst], (
            f"{what}: row {j} head {worst[0]} abs err {err[i][worst]:.3e} at |value| "
            f"{abs(want[i][worst]):.3g} (<= max(3e-2, {ATTN_Z:g} sigma) = {bound[worst]:.3e})")


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
