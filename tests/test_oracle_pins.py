"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values worked by
hand from the pages (tests/golden), closed forms, brute-force definitions on tiny
inputs, or an independent library formulation (complex arithmetic for the rotary
embedding, torch's scaled_dot_product_attention for attention). CPU only."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import ref
from selective_recompute_prefill_amd import inputs


# --------------------------------------------------------------------------- #
# rotary embedding
# --------------------------------------------------------------------------- #

def _rope_complex(x, pos, base):
    """Rotate-half RoPE as complex multiplication: pair (x_i, x_{i+d/2}) is the
    complex number x_i + 1j x_{i+d/2}, multiplied by exp(1j * pos * base^(-2i/d))."""
    d = x.shape[-1]
    h = d // 2
    z = x[..., :h] + 1j * x[..., h:]
    freq = np.array([base ** (-(2.0 * i) / d) for i in range(h)])
    rot = np.exp(1j * np.outer(pos, freq))[:, None, :]
    w = z * rot
    return np.concatenate([w.real, w.imag], axis=-1)


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((37, 3, 64))
    pos = rng.integers(0, 20000, 37)
    np.testing.assert_allclose(ref.rope(x, pos, 10000.0), _rope_complex(x, pos, 10000.0),
                               rtol=0, atol=1e-11)


def test_rope_group_properties():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 2, 128))
    a = rng.integers(-9000, 9000, 50)
    b = rng.integers(-9000, 9000, 50)
    # identity at 0, composition, inverse, orthogonality (norm per rotation pair)
    np.testing.assert_array_equal(ref.rope(x, np.zeros(50, int), 1e4), x)
    np.testing.assert_allclose(ref.rope(ref.rope(x, a, 1e4), b, 1e4), ref.rope(x, a + b, 1e4),
                               atol=1e-11)
    np.testing.assert_allclose(ref.rope(ref.rope(x, a, 1e4), -a, 1e4), x, atol=1e-11)
    y = ref.rope(x, a, 1e4)
    pair = lambda t: t[..., :64] ** 2 + t[..., 64:] ** 2
    np.testing.assert_allclose(pair(y), pair(x), rtol=1e-12)


def test_rope_scores_depend_only_on_relative_distance():
    # CacheBlend walkthrough, "Selective KV recompute": a RoPE score between two
    # tokens depends on their distance, not on where they sit.
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    s = lambda pq, pk: float((ref.rope(q, [pq], 1e4) * ref.rope(k, [pk], 1e4)).sum())
    for pq, pk, shift in [(100, 37, 5000), (16000, 3, 123), (7, 7, 9999)]:
        assert abs(s(pq, pk) - s(pq + shift, pk + shift)) < 1e-10


def test_rerotation_equals_direct_encode():
    # A chunk encoded at local positions and moved by R(pos - src) equals the
    # same chunk encoded at its global positions.
    spec = inputs.small_spec(dtype="f32")
    w = inputs.generate(spec)
    lay = w.layout
    src = inputs.encode_positions(lay)
    cr = src >= 0
    x = inputs.stored_to_f64(w.hidden, "f32")[cr]
    wq = ref.widen(w.layers[0].w_qkv, "f32")
    kl, _ = ref.encode_kv(x, wq, src[cr], spec.n_heads, spec.n_kv_heads, spec.head_dim, 1e4)
    kg, _ = ref.encode_kv(x, wq, lay.positions[cr], spec.n_heads, spec.n_kv_heads,
                          spec.head_dim, 1e4)
    moved = ref.rerotate(kl, lay.positions[cr].astype(np.int64), src[cr], 1e4)
    np.testing.assert_allclose(moved, kg, atol=1e-11)
    assert np.abs(kl - kg).max() > 1e-2  # the relocation is not a no-op


# --------------------------------------------------------------------------- #
# deviation closed form
# --------------------------------------------------------------------------- #

def _unrounded_layer(spec):
    w = inputs.generate(spec)
    lay = w.layout
    src = inputs.encode_positions(lay)
    cr = src >= 0
    x = inputs.stored_to_f64(w.hidden, spec.dtype)
    wq = ref.widen(w.layers[0].w_qkv, spec.dtype)
    xe = w.encode_input(0)
    T = lay.total_rows
    kc = np.zeros((T, spec.n_kv_heads, spec.head_dim))
    vc = np.zeros_like(kc)
    kc[cr], vc[cr] = ref.encode_kv(xe[cr], wq, src[cr], spec.n_heads, spec.n_kv_heads,
                                   spec.head_dim, spec.rope_base)
    return w, x, wq, kc, vc


def _layer_kwargs(spec, w, x, wq, kc, vc, **kw):
    lay = w.layout
    base = dict(hidden=x, w_qkv=wq, k_cache=kc, v_cache=vc, req_offsets=lay.req_offsets,
                chunk_offsets=lay.chunk_offsets, chunk_src_pos=lay.chunk_src_pos,
                positions=lay.positions, n_heads=spec.n_heads, n_kv=spec.n_kv_heads,
                head_dim=spec.head_dim, rope_base=spec.rope_base, ratio=spec.ratio,
                window=spec.window, tau=spec.tau)
    base.update(kw)
    return base


def test_deviation_closed_form():
    # cached = R(src) W (x + eps n) moved by R(pos - src); fresh = R(pos) W x, so the
    # deviation is eps * sqrt(|W_k n|^2 + |W_v n|^2) exactly (orthogonal R).
    spec = inputs.WORKLOADS[0]
    w, x, wq, kc, vc = _unrounded_layer(spec)
    out = ref.fuse_layer(**_layer_kwargs(spec, w, x, wq, kc, vc))
    ld = w.layers[0]
    qd, kvd = spec.qdim, spec.kvdim
    wk, wv = wq[qd:qd + kvd], wq[qd + kvd:]
    rows = np.nonzero(w.cache_row_of >= 0)[0]
    pr = w.cache_row_of[rows]
    n = ld.noise[pr]
    closed = ld.eps[pr] * np.sqrt(((n @ wk.T) ** 2).sum(1) + ((n @ wv.T) ** 2).sum(1))
    np.testing.assert_allclose(out["dev"][rows], closed, rtol=1e-10)
    closed_v = ld.eps[pr] * np.sqrt(((n @ wv.T) ** 2).sum(1))
    out_v = ref.fuse_layer(**_layer_kwargs(spec, w, x, wq, kc, vc, dev_mode="v"))
    np.testing.assert_allclose(out_v["dev"][rows], closed_v, rtol=1e-10)
    assert np.all(np.isnan(out["dev"][w.cache_row_of < 0]))


# --------------------------------------------------------------------------- #
# top-k
# --------------------------------------------------------------------------- #

def test_topk_counts_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "topk_counts.json")))
    for c in g["cases"]:
        assert ref.topk_count(c["ratio"], c["n"], 10 ** 9) == c["k"], c
    assert ref.topk_count(0.5, 100, 7) == 7  # clamped to the candidates


def _brute_topk(dev, rows, k):
    sel = []
    for i in range(len(rows)):
        rank = sum(1 for j in range(len(rows))
                   if dev[j] > dev[i] or (dev[j] == dev[i] and rows[j] < rows[i]))
        if rank < k:
            sel.append(rows[i])
    return sorted(sel)


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 30))
    rows = np.sort(rng.choice(200, n, replace=False))
    dev = rng.integers(0, 5, n).astype(np.float64)  # many exact ties
    if seed % 2:
        dev = dev + rng.random(n)
    for k in sorted({0, 1, n // 3, n - 1, n}):
        k = max(k, 0)
        assert list(ref.topk_rows(dev, rows, k)) == _brute_topk(dev, rows, k)


# --------------------------------------------------------------------------- #
# grouping
# --------------------------------------------------------------------------- #

def test_grouping_figure6(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "fig6_grouping.json")))
    assert ref.group_windows(g["candidates"], g["seq_len"], g["w"], g["tau"]) == g["expected"]
    for c in g["cases"]:
        assert ref.group_windows(c["candidates"], c["seq_len"], c["w"], c["tau"]) == c["expected"], c


def _brute_grouping(cands, n, w, tau):
    # slot p is recomputed iff some window start t in [p-w+1, p] is a candidate,
    # fits in the sequence, and holds at least tau candidates.
    c = set(cands)
    out = []
    for p in range(n):
        for t in range(max(0, p - w + 1), p + 1):
            if t in c and t + w <= n and len([j for j in range(t, t + w) if j in c]) >= tau:
                out.append(p)
                break
    return out


@pytest.mark.parametrize("seed", range(10))
def test_grouping_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 60))
    w = int(rng.integers(1, 10))
    tau = int(rng.integers(1, w + 1))
    cands = sorted(rng.choice(n, int(rng.integers(0, n + 1)), replace=False).tolist())
    got = ref.group_windows(cands, n, w, tau)
    assert got == _brute_grouping(cands, n, w, tau)
    # properties: the kept set is a union of whole windows and keeps no isolated
    # candidate; every candidate in a passing window is kept.
    kept = set(got)
    for c in cands:
        if c + w <= n and sum(1 for j in range(c, c + w) if j in cands) >= tau:
            assert all(j in kept for j in range(c, c + w))


# --------------------------------------------------------------------------- #
# attention
# --------------------------------------------------------------------------- #

def test_attention_two_keys_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "attention_two_keys.json")))
    k = np.asarray(g["k"])[:, None, :]
    v = np.asarray(g["v"])[:, None, :]
    q = np.stack([np.zeros(2), np.asarray(g["q_row2"])])[:, None, :]
    rows = np.array([0, 2])
    o = ref.attention(q, rows, k, v, np.zeros(3, int), np.arange(3))
    np.testing.assert_allclose(o[1, 0], g["expected_row2"], atol=1e-12)
    np.testing.assert_allclose(o[0, 0], g["expected_row0"], atol=1e-12)


def test_attention_properties():
    rng = np.random.default_rng(7)
    T, nh, nkv, d = 40, 4, 2, 16
    k = rng.standard_normal((T, nkv, d))
    v = rng.standard_normal((T, nkv, d))
    req = np.zeros(T, int)
    pos = np.arange(T)
    rows = np.array([0, 5, 17, 39])
    q = rng.standard_normal((4, nh, d))
    # weights sum to one: constant V returns the constant
    o1 = ref.attention(q, rows, k, np.ones_like(v) * 3.5, req, pos)
    np.testing.assert_allclose(o1, 3.5, atol=1e-12)
    # a query that sees one key returns that key's value
    o = ref.attention(q, rows, k, v, req, pos)
    for h in range(nh):
        np.testing.assert_allclose(o[0, h], v[0, (h * nkv) // nh], atol=1e-12)
    # q = 0 gives the mean of the visible values
    oz = ref.attention(np.zeros_like(q), rows, k, v, req, pos)
    for i, j in enumerate(rows):
        for h in range(nh):
            np.testing.assert_allclose(oz[i, h], v[:j + 1, (h * nkv) // nh].mean(0), atol=1e-12)


def _sdpa(q, k, v, causal=True):
    """torch reference: q [n, nh, d], k/v [n, nkv, d] -> [n, nh, d], float64."""
    nh, nkv = q.shape[1], k.shape[1]
    rep = nh // nkv
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(rep, 0).contiguous()
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(rep, 0).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal)
    return o.permute(1, 0, 2).numpy()


def test_attention_matches_sdpa_mha_and_gqa():
    rng = np.random.default_rng(8)
    T, d = 50, 32
    for nh, nkv in [(4, 4), (8, 2)]:
        q = rng.standard_normal((T, nh, d))
        k = rng.standard_normal((T, nkv, d))
        v = rng.standard_normal((T, nkv, d))
        o = ref.attention(q, np.arange(T), k, v, np.zeros(T, int), np.arange(T))
        np.testing.assert_allclose(o, _sdpa(q, k, v), atol=1e-12)


# --------------------------------------------------------------------------- #
# whole layer: reductions at ratio 0 and ratio 1, batching, chain
# --------------------------------------------------------------------------- #

def _torch_rope(x, pos, base):
    d = x.shape[-1]
    h = d // 2
    freq = torch.tensor([base ** (-(2.0 * i) / d) for i in range(h)], dtype=torch.float64)
    ang = torch.outer(torch.as_tensor(pos, dtype=torch.float64), freq)
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]
    z = torch.complex(x[..., :h], x[..., h:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def _full_prefill_torch(x, wq, spec, req_offsets, positions):
    """Full prefill of every row with torch ops only (independent of the oracle)."""
    xt = torch.from_numpy(x)
    w = torch.from_numpy(wq)
    qd, kvd, d = spec.qdim, spec.kvdim, spec.head_dim
    n = x.shape[0]
    q = (xt @ w[:qd].T).reshape(n, spec.n_heads, d)
    k = (xt @ w[qd:qd + kvd].T).reshape(n, spec.n_kv_heads, d)
    v = (xt @ w[qd + kvd:].T).reshape(n, spec.n_kv_heads, d)
    q = _torch_rope(q, positions, spec.rope_base)
    k = _torch_rope(k, positions, spec.rope_base)
    o = np.zeros((n, spec.n_heads, d))
    for r in range(len(req_offsets) - 1):
        a, b = req_offsets[r], req_offsets[r + 1]
        o[a:b] = _sdpa(q[a:b].numpy(), k[a:b].numpy(), v[a:b].numpy())
    return k.numpy(), v.numpy(), o


def test_ratio_one_equals_full_prefill():
    spec = inputs.small_spec(dtype="f32", hidden=256, n_heads=4, n_kv_heads=2, head_dim=64,
                             chunk_lens=(40, 33, 51), prefix=8, n_query=9)
    w, x, wq, kc, vc = _unrounded_layer(spec)
    out = ref.fuse_layer(**_layer_kwargs(spec, w, x, wq, kc, vc, ratio=1.0))
    lay = w.layout
    assert np.array_equal(out["sel_idx"], np.arange(lay.total_rows))
    kf, vf, of = _full_prefill_torch(x, wq, spec, lay.req_offsets, lay.positions)
    np.testing.assert_allclose(out["k_cache"], kf, atol=1e-10)
    np.testing.assert_allclose(out["v_cache"], vf, atol=1e-10)
    np.testing.assert_allclose(out["attn_out"], of, atol=1e-10)


def test_ratio_zero_is_rerotated_cache():
    spec = inputs.small_spec(dtype="f32", hidden=256, n_query=0)
    w, x, wq, kc, vc = _unrounded_layer(spec)
    out = ref.fuse_layer(**_layer_kwargs(spec, w, x, wq, kc, vc, ratio=0.0))
    assert len(out["sel_idx"]) == 0 and out["attn_out"].shape[0] == 0
    src = inputs.encode_positions(w.layout)
    rerot = ref.rerotate(kc, w.layout.positions.astype(np.int64), src, spec.rope_base)
    assert np.array_equal(out["k_cache"], rerot)
    assert np.array_equal(out["v_cache"], vc)


def test_ratio_zero_with_query_tail_recomputes_only_the_tail():
    spec = inputs.small_spec(dtype="f32", hidden=256)
    w, x, wq, kc, vc = _unrounded_layer(spec)
    out = ref.fuse_layer(**_layer_kwargs(spec, w, x, wq, kc, vc, ratio=0.0))
    fresh = np.nonzero(w.cache_row_of < 0)[0]
    assert np.array_equal(out["sel_idx"], fresh)


def test_batch_equals_concatenated_requests():
    spec = inputs.small_spec(dtype="f32", hidden=256)
    w, x, wq, kc, vc = _unrounded_layer(spec)
    lay = w.layout
    full = ref.fuse_layer(**_layer_kwargs(spec, w, x, wq, kc, vc))
    for r in range(lay.n_req):
        a, b = int(lay.req_offsets[r]), int(lay.req_offsets[r + 1])
        segs = [c for c in range(len(lay.chunk_src_pos))
                if a <= lay.chunk_offsets[c] < b]
        one = ref.fuse_layer(**_layer_kwargs(
            spec, w, x[a:b], wq, kc[a:b], vc[a:b],
            req_offsets=np.array([0, b - a]),
            chunk_offsets=np.concatenate([lay.chunk_offsets[segs], [b]]) - a,
            chunk_src_pos=lay.chunk_src_pos[segs], positions=lay.positions[a:b]))
        s0, s1 = full["sel_offsets"][r], full["sel_offsets"][r + 1]
        assert np.array_equal(full["sel_idx"][s0:s1] - a, one["sel_idx"])
        np.testing.assert_allclose(full["attn_out"][s0:s1], one["attn_out"], atol=1e-13)
        np.testing.assert_allclose(full["k_cache"][a:b], one["k_cache"], atol=1e-13)


def test_selection_tracks_noise_scale():
    # The deviation of a layer-1 token is eps * |W n|: with eps lognormal(-3, 1) the
    # top-k set must be dominated by the largest-eps tokens.
    spec = inputs.WORKLOADS[0]
    w, x, wq, kc, vc = _unrounded_layer(spec)
    out = ref.fuse_layer(**_layer_kwargs(spec, w, x, wq, kc, vc))
    rows = np.nonzero(w.cache_row_of >= 0)[0]
    eps = w.layers[0].eps[w.cache_row_of[rows]]
    top_eps = set(rows[np.argsort(-eps)[:109]].tolist())
    sel = set(out["sel_idx"].tolist()) & set(rows.tolist())
    assert len(sel) == 109
    assert len(sel & top_eps) >= 90


def test_grouped_layer_windows_cover_selection():
    spec = inputs.small_spec(dtype="f32", hidden=256, window=8, tau=4, ratio=0.3)
    w, x, wq, kc, vc = _unrounded_layer(spec)
    out = ref.fuse_layer(**_layer_kwargs(spec, w, x, wq, kc, vc))
    lay = w.layout
    sel = set(out["sel_idx"].tolist())
    fresh = set(np.nonzero(w.cache_row_of < 0)[0].tolist())
    assert fresh <= sel
    # every selected cached row lies in a window that starts on a top-k member
    s0 = set(out["s0"].tolist())
    for j in sel - fresh:
        assert any((j - t) in s0 for t in range(spec.window))


def test_chain_all_recompute_equals_full_stack():
    spec = inputs.small_spec(dtype="f32", hidden=256, n_heads=4, n_kv_heads=2, head_dim=64,
                             chunk_lens=(30, 41), prefix=0, n_query=7, n_req=1, n_layers=3,
                             ratios=(1.0, 1.0, 1.0))
    w = inputs.generate(spec)
    lay = w.layout
    src = inputs.encode_positions(lay)
    cr = src >= 0
    x = inputs.stored_to_f64(w.hidden, "f32")
    layers = []
    for l in range(spec.n_layers):
        wq = ref.widen(w.layers[l].w_qkv, "f32")
        kc = np.zeros((lay.total_rows, spec.n_kv_heads, spec.head_dim))
        vc = np.zeros_like(kc)
        kc[cr], vc[cr] = ref.encode_kv(w.encode_input(l, x_full=x)[cr], wq, src[cr],
                                       spec.n_heads, spec.n_kv_heads, spec.head_dim, 1e4)
        layers.append(dict(w_qkv=wq, k_cache=kc, v_cache=vc))
    outs = ref.fuse_stack(hidden=x, layers=layers, req_offsets=lay.req_offsets,
                          chunk_offsets=lay.chunk_offsets, chunk_src_pos=lay.chunk_src_pos,
                          positions=lay.positions, n_heads=spec.n_heads,
                          n_kv=spec.n_kv_heads, head_dim=spec.head_dim, rope_base=1e4,
                          ratios=spec.layer_ratios())
    # direct stack with torch ops
    h = x.copy()
    for l in range(spec.n_layers):
        _, _, o = _full_prefill_torch(h, layers[l]["w_qkv"], spec, lay.req_offsets, lay.positions)
        np.testing.assert_allclose(outs[l]["attn_out"], o, atol=1e-10)
        y = torch.from_numpy(h + o.reshape(h.shape[0], -1))
        h = (y / torch.sqrt((y * y).mean(1, keepdim=True) + 1e-6)).numpy()


def test_gradual_filtering_shrinks():
    spec = inputs.small_spec(dtype="f32", hidden=256, n_heads=4, n_kv_heads=2, head_dim=64,
                             n_layers=3, ratios=(0.3, 0.15, 0.15))
    w = inputs.generate(spec)
    lay = w.layout
    src = inputs.encode_positions(lay)
    cr = src >= 0
    x = inputs.stored_to_f64(w.hidden, "f32")
    layers = []
    for l in range(spec.n_layers):
        wq = ref.widen(w.layers[l].w_qkv, "f32")
        kc = np.zeros((lay.total_rows, spec.n_kv_heads, spec.head_dim))
        vc = np.zeros_like(kc)
        kc[cr], vc[cr] = ref.encode_kv(w.encode_input(l, x_full=x)[cr], wq, src[cr],
                                       spec.n_heads, spec.n_kv_heads, spec.head_dim, 1e4)
        layers.append(dict(w_qkv=wq, k_cache=kc, v_cache=vc))
    outs = ref.fuse_stack(hidden=x, layers=layers, req_offsets=lay.req_offsets,
                          chunk_offsets=lay.chunk_offsets, chunk_src_pos=lay.chunk_src_pos,
                          positions=lay.positions, n_heads=spec.n_heads,
                          n_kv=spec.n_kv_heads, head_dim=spec.head_dim, rope_base=1e4,
                          ratios=spec.layer_ratios())
    fresh = set(np.nonzero(~cr)[0].tolist())
    prev = None
    for o in outs:
        s = set(o["sel_idx"].tolist()) - fresh
        if prev is not None:
            assert s <= prev
        prev = s
    n_ctx = [int(cr[lay.req_offsets[r]:lay.req_offsets[r + 1]].sum()) for r in range(lay.n_req)]
    assert len(set(outs[0]["sel_idx"].tolist()) - fresh) == sum(
        ref.topk_count(0.3, n, n) for n in n_ctx)


# --------------------------------------------------------------------------- #
# chain step and storage widening
# --------------------------------------------------------------------------- #

def test_residual_rmsnorm_golden(golden_dir):
    # hand-worked rows (tests/golden/rmsnorm.json): the residual adds, the mean (not
    # the sum) of squares is taken, eps sits inside the square root
    with open(os.path.join(golden_dir, "rmsnorm.json")) as fh:
        g = json.load(fh)
    for case in g["cases"]:
        x = np.asarray([case["x"]], np.float64)
        o = np.asarray([case["o"]], np.float64)
        got = ref.residual_rmsnorm(x, o, case["eps"])[0]
        np.testing.assert_allclose(got, case["expected"], rtol=1e-14, atol=0, err_msg=case["what"])


def test_residual_rmsnorm_rows_are_independent_and_scale_free():
    # each row is normalised on its own (a batch equals its rows one by one); with
    # eps = 0 the output has unit RMS and does not change when y is scaled
    rng = np.random.default_rng(17)
    x = rng.standard_normal((5, 24)) * np.array([1e-2, 1, 3, 50, 7])[:, None]
    o = rng.standard_normal((5, 24))
    both = ref.residual_rmsnorm(x, o, 0.0)
    for i in range(5):
        np.testing.assert_array_equal(both[i], ref.residual_rmsnorm(x[i:i + 1], o[i:i + 1], 0.0)[0])
    np.testing.assert_allclose(np.sqrt((both ** 2).mean(axis=1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(ref.residual_rmsnorm(3.5 * x, 3.5 * o, 0.0), both, rtol=1e-14)


def test_widen_bf16_bit_patterns():
    # bfloat16 = the upper 16 bits of an IEEE binary32: sign, 8 exponent bits, 7
    # mantissa bits; hand-decoded patterns
    cases = {
        0x3F80: 1.0,                       # exponent 127, mantissa 0
        0xC000: -2.0,                      # sign, exponent 128
        0x4049: 3.140625,                  # 2 * (1 + 1/2 + 1/16 + 1/128)
        0x3E80: 0.25,                      # exponent 125
        0x0000: 0.0,
        0x0001: 2.0 ** -133,               # smallest subnormal: 2^-126 * 2^-7
        0x007F: (127 / 128) * 2.0 ** -126,  # largest subnormal
        0x0080: 2.0 ** -126,               # smallest normal
        0x7F7F: (2 - 2 ** -7) * 2.0 ** 127,  # largest finite
        0x7F80: np.inf,
        0xFF80: -np.inf,
    }
    bits = np.array(list(cases), np.uint16)
    got = ref.widen(bits, "bf16")
    assert got.dtype == np.float64
    np.testing.assert_array_equal(got, np.array(list(cases.values())))
    neg_zero = ref.widen(np.array([0x8000], np.uint16), "bf16")[0]
    assert neg_zero == 0.0 and np.signbit(neg_zero)


def test_widen_bf16_matches_torch_for_every_pattern():
    # every non-NaN bit pattern against torch's own bfloat16 -> float64 conversion
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = ref.widen(bits, "bf16")
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_widen_f32_is_exact():
    x = np.array([1.0, -0.0, 3.4028234663852886e38, 1.401298464324817e-45, np.inf], np.float32)
    got = ref.widen(x, "f32")
    assert got.dtype == np.float64
    np.testing.assert_array_equal(got, x.astype(np.float64))
    with pytest.raises(ValueError):
        ref.widen(x, "fp8")


def _chain_layers(spec, w, x):
    lay = w.layout
    src = inputs.encode_positions(lay)
    cr = src >= 0
    layers = []
    for l in range(spec.n_layers):
        wq = ref.widen(w.layers[l].w_qkv, "f32")
        kc = np.zeros((lay.total_rows, spec.n_kv_heads, spec.head_dim))
        vc = np.zeros_like(kc)
        kc[cr], vc[cr] = ref.encode_kv(w.encode_input(l, x_full=x)[cr], wq, src[cr],
                                       spec.n_heads, spec.n_kv_heads, spec.head_dim, 1e4)
        layers.append(dict(w_qkv=wq, k_cache=kc, v_cache=vc))
    return layers


def test_given_layers_after_a_full_check_equal_the_full_stack():
    # check_flag off on layers 2 and 3 (CacheBlend walkthrough, "Implementation"):
    # they recompute the rows handed to them; after a first layer that recomputes
    # every row, the whole chain is a full prefill stack, computed here directly
    spec = inputs.small_spec(dtype="f32", hidden=256, n_heads=4, n_kv_heads=2, head_dim=64,
                             chunk_lens=(30, 41), prefix=0, n_query=7, n_req=1, n_layers=3,
                             ratios=(1.0, 0.1, 0.0))
    w = inputs.generate(spec)
    lay = w.layout
    x = inputs.stored_to_f64(w.hidden, "f32")
    layers = _chain_layers(spec, w, x)
    outs = ref.fuse_stack(hidden=x, layers=layers, req_offsets=lay.req_offsets,
                          chunk_offsets=lay.chunk_offsets, chunk_src_pos=lay.chunk_src_pos,
                          positions=lay.positions, n_heads=spec.n_heads, n_kv=spec.n_kv_heads,
                          head_dim=spec.head_dim, rope_base=1e4, ratios=spec.layer_ratios(),
                          modes=("topk", "given", "given"))
    h = x.copy()
    for l in range(spec.n_layers):
        assert len(outs[l]["sel_idx"]) == lay.total_rows
        _, _, o = _full_prefill_torch(h, layers[l]["w_qkv"], spec, lay.req_offsets, lay.positions)
        np.testing.assert_allclose(outs[l]["attn_out"], o, atol=1e-10)
        y = torch.from_numpy(h + o.reshape(h.shape[0], -1))
        h = (y / torch.sqrt((y * y).mean(1, keepdim=True) + 1e-6)).numpy()


def test_given_layers_keep_the_last_checked_selection():
    # check on layers 1-2, then pass the indices on: layers 3 and 4 select exactly
    # layer 2's rows although their own ratio would keep fewer
    spec = inputs.small_spec(dtype="f32", hidden=256, n_heads=4, n_kv_heads=2, head_dim=64,
                             n_layers=4, ratios=(0.3, 0.15, 0.05, 0.05))
    w = inputs.generate(spec)
    lay = w.layout
    x = inputs.stored_to_f64(w.hidden, "f32")
    layers = _chain_layers(spec, w, x)
    kw = dict(hidden=x, layers=layers, req_offsets=lay.req_offsets, chunk_offsets=lay.chunk_offsets,
              chunk_src_pos=lay.chunk_src_pos, positions=lay.positions, n_heads=spec.n_heads,
              n_kv=spec.n_kv_heads, head_dim=spec.head_dim, rope_base=1e4, ratios=spec.layer_ratios())
    given = ref.fuse_stack(modes=("topk", "topk", "given", "given"), **kw)
    checked = ref.fuse_stack(**kw)
    for l in (0, 1):  # identical up to the last check layer
        np.testing.assert_array_equal(given[l]["sel_idx"], checked[l]["sel_idx"])
    for l in (2, 3):
        np.testing.assert_array_equal(given[l]["sel_idx"], given[1]["sel_idx"])
        assert len(checked[l]["sel_idx"]) < len(given[l]["sel_idx"])
