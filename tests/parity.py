"""Helpers of the parity tests: oracle-side inputs, tolerances, selection checks.

All expected values come from the fp64 oracle on the same stored inputs the GPU
sees; nothing here reads a GPU result back into an oracle input."""
from __future__ import annotations

import numpy as np

from oracle import ref
from selective_recompute_prefill_amd import inputs

# Tolerances: rel-L2 and max-abs per output, by storage dtype.
TOL = {"bf16": (1e-2, 3e-2), "f32": (1e-5, 1e-5)}
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


def assert_close(got: np.ndarray, want: np.ndarray, dtype: str, what: str):
    rl, ma = TOL[dtype]
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if want.size == 0:
        return
    err = got - want
    nrm = np.linalg.norm(want)
    rel = np.linalg.norm(err) / (nrm if nrm > 0 else 1.0)
    mx = np.abs(err).max()
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert rel <= rl and mx <= ma, f"{what}: rel-L2 {rel:.3e} (<= {rl}), max-abs {mx:.3e} (<= {ma})"


def check_selection(gpu_sel: np.ndarray, ref_out: dict, req_of_row: np.ndarray, what: str):
    """The GPU's selected set equals the oracle's except for near-ties: every row in
    the symmetric difference is a candidate whose oracle deviation lies within
    NEAR_TIE (relative) of its request's k-th largest. Returns the swapped rows."""
    a, b = set(gpu_sel.tolist()), set(ref_out["sel_idx"].tolist())
    sym = sorted(a ^ b)
    for j in sym:
        r = int(req_of_row[j])
        dk = ref_out["kth"][r]
        dj = ref_out["dev"][j]
        assert np.isfinite(dj) and np.isfinite(dk) and dk > 0, f"{what}: row {j} differs and is not a scored candidate"
        assert abs(dj - dk) / dk < NEAR_TIE, f"{what}: row {j} differs (dev {dj} vs k-th {dk})"
    return sym


def csr_ok(sel: np.ndarray, off: np.ndarray, req_offsets: np.ndarray):
    """Selected rows ascend inside each request and lie in it."""
    for r in range(len(req_offsets) - 1):
        s = sel[off[r]:off[r + 1]]
        assert np.all(np.diff(s) > 0)
        if len(s):
            assert s[0] >= req_offsets[r] and s[-1] < req_offsets[r + 1]
