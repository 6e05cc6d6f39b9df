"""GPU checks of the paged cache layout (blocks of block_rows rows reached through a
block table, each segment padded to whole blocks; the Cache-Craft summary, section
4, uses 16-token blocks).

Every paged run is compared with the fp64 oracle exactly as a contiguous run is
(selection with near-ties and per-request sizes, K/V caches, deviations, attention),
with its padding rows filled with large values that must come back untouched. The
layout only changes where cache rows live, so on top of that a paged run must give,
bit for bit, what the same layer gives on contiguous caches."""
import sys

import numpy as np
import pytest
import torch

from selective_recompute_prefill_amd import inputs
from selective_recompute_prefill_amd import srp as S
from selective_recompute_prefill_amd.device import LayerCall, download, ints, upload

from parity import oracle_caches
from test_gpu_layer import POISON, _scores_case, paged_call, run_case, to_pool

pytestmark = pytest.mark.gpu

B = 16


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_both(spec, sel_kw_fn, what, w=None, seed=1, block_rows=B):
    """The same layer on contiguous caches and on a block pool: bit-equal results."""
    w = w or inputs.generate(spec)
    lay = w.layout
    kc, vc = oracle_caches(w)
    seg_block, table, slot, pool_rows = inputs.paged_layout(lay, block_rows, seed)
    hid, wq = upload(w.hidden, spec.dtype), upload(w.layers[0].w_qkv, spec.dtype)
    _say(f"[gpu] paged {what}: T={lay.total_rows}, blocks of {block_rows}, pool rows {pool_rows}")
    flat = LayerCall(spec, lay)
    k1, v1 = upload(kc, spec.dtype), upload(vc, spec.dtype)
    flat.fuse(flat.select(**sel_kw_fn()), hid, wq, k1, v1)
    paged = paged_call(spec, lay, block_rows, seg_block, table)
    S.srp_validate_batch(paged.batch)
    k2 = upload(to_pool(kc, slot, pool_rows, spec.dtype), spec.dtype)
    v2 = upload(to_pool(vc, slot, pool_rows, spec.dtype), spec.dtype)
    paged.fuse(paged.select(**sel_kw_fn()), hid, wq, k2, v2)
    torch.cuda.synchronize()
    a, b = flat.results(), paged.results()
    for key in ("sel_idx", "sel_offsets", "attn_out"):
        assert np.array_equal(a[key], b[key]), f"{what}: {key} differs"
    assert np.array_equal(a["dev"], b["dev"], equal_nan=True), f"{what}: deviations differ"
    kf, vf, kp, vp = download(k1), download(v1), download(k2), download(v2)
    assert np.array_equal(kp[slot], kf) and np.array_equal(vp[slot], vf), f"{what}: cache rows differ"
    pad = np.setdiff1d(np.arange(pool_rows), slot)
    poison = inputs.store(np.full(1, POISON), spec.dtype)[0]
    assert np.all(kp[pad] == poison) and np.all(vp[pad] == poison), f"{what}: padding rows touched"


def test_paged_topk_grouped():
    spec = inputs.small_spec(window=8, tau=4)
    run_both(spec, lambda: dict(ratio=spec.ratio, window=8, tau=4), "grouped")
    run_case(spec, what="paged grouped", paged=(B, 1))


def test_paged_fp32():
    spec = inputs.small_spec(dtype="f32")
    run_both(spec, lambda: dict(ratio=0.25), "fp32")
    run_case(spec, sel_kw=dict(ratio=0.25), what="paged fp32", paged=(B, 1))


def test_paged_scores_and_fresh_all():
    spec = inputs.small_spec()
    T = inputs.generate(spec).layout.total_rows
    sc_np = inputs.draw_scores(T, 31)
    sc = torch.as_tensor(sc_np, device="cuda")
    spans = dict(span_max=16, tau_smooth=0.4, tau_cover=0.7)
    run_both(spec, lambda: dict(ratio=0.2, mode=S.SRP_SEL_SCORES, scores=sc, **spans), "scores")
    _scores_case(spec, sc_np, dict(ratio=0.2, **spans), "paged scores", paged=(B, 1))
    run_both(spec, lambda: dict(ratio=0.2, fresh_all=True), "fresh-all", seed=2)
    run_case(spec, sel_kw=dict(ratio=0.2, fresh_all=True), oracle_kw=dict(fresh_all=True),
             what="paged fresh-all", paged=(B, 2))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_paged_v_only_deviation(dtype):
    spec = inputs.small_spec(dtype=dtype)
    run_both(spec, lambda: dict(ratio=0.2, dev_mode=S.SRP_DEV_V), f"v-only {dtype}")
    run_case(spec, sel_kw=dict(ratio=0.2, dev_mode=S.SRP_DEV_V), oracle_kw=dict(dev_mode="v"),
             what=f"paged v-only {dtype}", paged=(B, 1))


def test_paged_candidate_list():
    spec = inputs.small_spec()
    lay = inputs.generate(spec).layout
    cand = np.concatenate([np.arange(lay.req_offsets[r], lay.req_offsets[r + 1])[::2]
                           for r in range(lay.n_req)])
    off = np.searchsorted(cand, lay.req_offsets)
    c_t, o_t = ints(cand), ints(off)
    run_both(spec, lambda: dict(ratio=0.15, cand=c_t, cand_offsets=o_t), "cand")
    for mode, omode in [(S.SRP_SEL_TOPK, "topk"), (S.SRP_SEL_GIVEN, "given")]:
        run_case(spec, sel_kw=dict(ratio=0.15, mode=mode, cand=c_t, cand_offsets=o_t),
                 oracle_kw=dict(mode=omode, cand=cand), what=f"paged cand-{omode}", paged=(B, 1))


@pytest.mark.parametrize("block_rows", [1, 5, 64, 300])
def test_paged_other_block_sizes(block_rows):
    """Blocks of 1, 5, 64 and 300 rows (the layout takes any size): a block smaller
    than a copy piece, one that splits rows of a 64-row attention tile unevenly, one
    as large as a tile, and one larger than some segments (the 137-row chunk)."""
    spec = inputs.small_spec(window=8, tau=4)
    run_both(spec, lambda: dict(ratio=spec.ratio, window=8, tau=4), f"grouped b{block_rows}",
             seed=block_rows, block_rows=block_rows)
    run_case(spec, what=f"paged grouped b{block_rows}", paged=(block_rows, block_rows))
    fspec = inputs.small_spec(dtype="f32")
    run_case(fspec, sel_kw=dict(ratio=0.3), what=f"paged fp32 b{block_rows}", paged=(block_rows, 7))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_paged_rerotate(dtype):
    from oracle import ref
    from parity import assert_close
    spec = inputs.small_spec(dtype=dtype)
    w = inputs.generate(spec)
    lay = w.layout
    kc, _ = oracle_caches(w)
    seg_block, table, slot, pool_rows = inputs.paged_layout(lay, B, 3)
    flat = LayerCall(spec, lay)
    k1 = upload(kc, dtype)
    S.srp_rerotate_kv(flat.dims, flat.batch, k1)
    paged = paged_call(spec, lay, B, seg_block, table)
    k2 = upload(to_pool(kc, slot, pool_rows, dtype), dtype)
    S.srp_rerotate_kv(paged.dims, paged.batch, k2)
    torch.cuda.synchronize()
    kf, kp = download(k1), download(k2)
    assert np.array_equal(kp[slot], kf)
    pad = np.setdiff1d(np.arange(pool_rows), slot)
    assert np.all(kp[pad] == inputs.store(np.full(1, POISON), dtype)[0])
    # and against the oracle's re-rotation
    _, src = ref.row_layout(lay.req_offsets, lay.chunk_offsets, lay.chunk_src_pos, lay.total_rows)
    want = ref.rerotate(ref.widen(kc, dtype), lay.positions.astype(np.int64), src, spec.rope_base)
    assert_close(ref.widen(kp[slot], dtype), want, dtype, "paged rerotate")


def test_validate_rejects_shared_pool_rows():
    spec = inputs.small_spec()
    lay = inputs.generate(spec).layout
    seg_block, table, _, _ = inputs.paged_layout(lay, B, 4)
    bad = table.copy()
    bad[1] = bad[0]  # two blocks at one place
    call = paged_call(spec, lay, B, seg_block, bad)
    with pytest.raises(S.SrpError) as e:
        S.srp_validate_batch(call.batch)
    assert e.value.code == S.SRP_E_BATCH


def test_paged_head_dim_64_gqa8():
    """Head dim 64 with eight query heads per KV head: the gathered K rows, the V
    transpose from the pool and the projection epilogue at the other head size."""
    spec = inputs.small_spec(hidden=1024, n_heads=16, n_kv_heads=2, head_dim=64)
    run_both(spec, lambda: dict(ratio=0.25), "d64 g8")
    run_case(spec, sel_kw=dict(ratio=0.25), what="paged d64 g8", paged=(B, 1))
