"""GPU checks of the paged cache layout (16-row blocks reached through a block table,
each segment padded to whole blocks, as in the Cache-Craft summary, section 4).

The layout only changes where cache rows live, so a layer run on a block pool must
give, bit for bit, what the same layer gives on contiguous caches: the same
selection, attention rows and deviations, and pool rows holding exactly the
contiguous run's cache rows. Padding rows of the pool are filled with large values
and must come back untouched (nothing reads or writes them)."""
import sys

import numpy as np
import pytest
import torch

from selective_recompute_prefill_amd import inputs
from selective_recompute_prefill_amd import srp as S
from selective_recompute_prefill_amd.device import LayerCall, download, ints, upload

from parity import oracle_caches

pytestmark = pytest.mark.gpu

B = 16
POISON = 1000.0


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def paged_map(lay, seed):
    return inputs.paged_layout(lay, B, seed)


def to_pool(a, slot, pool_rows, dtype):
    shape = (pool_rows,) + a.shape[1:]
    pool = inputs.store(np.full(shape, POISON), dtype)
    pool[slot] = a
    return pool


def paged_call(spec, lay, seg_block, table):
    call = LayerCall(spec, lay)
    call.seg_block = ints(seg_block)
    call.block_table = ints(table)
    call.batch = S.make_batch(call.req_offsets, call.chunk_offsets, call.chunk_src_pos, call.positions,
                              total_rows=lay.total_rows, max_req_rows=call.max_req_rows,
                              max_position=lay.max_position, block_rows=B, seg_block=call.seg_block,
                              block_table=call.block_table)
    return call


def run_both(spec, sel_kw_fn, what, w=None, seed=1):
    w = w or inputs.generate(spec)
    lay = w.layout
    kc, vc = oracle_caches(w)
    seg_block, table, slot, pool_rows = paged_map(lay, seed)
    hid, wq = upload(w.hidden, spec.dtype), upload(w.layers[0].w_qkv, spec.dtype)
    _say(f"[gpu] paged {what}: T={lay.total_rows}, pool rows {pool_rows}")
    flat = LayerCall(spec, lay)
    k1, v1 = upload(kc, spec.dtype), upload(vc, spec.dtype)
    flat.fuse(flat.select(**sel_kw_fn()), hid, wq, k1, v1)
    paged = paged_call(spec, lay, seg_block, table)
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


def test_paged_fp32():
    spec = inputs.small_spec(dtype="f32")
    run_both(spec, lambda: dict(ratio=0.25), "fp32")


def test_paged_scores_and_fresh_all():
    spec = inputs.small_spec()
    T = inputs.generate(spec).layout.total_rows
    sc = torch.as_tensor(inputs.draw_scores(T, 31), device="cuda")
    run_both(spec, lambda: dict(ratio=0.2, mode=S.SRP_SEL_SCORES, scores=sc, span_max=16, tau_smooth=0.4,
                                tau_cover=0.7), "scores")
    run_both(spec, lambda: dict(ratio=0.2, fresh_all=True), "fresh-all", seed=2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_paged_v_only_deviation(dtype):
    spec = inputs.small_spec(dtype=dtype)
    run_both(spec, lambda: dict(ratio=0.2, dev_mode=S.SRP_DEV_V), f"v-only {dtype}")


def test_paged_candidate_list():
    spec = inputs.small_spec()
    lay = inputs.generate(spec).layout
    cand = np.concatenate([np.arange(lay.req_offsets[r], lay.req_offsets[r + 1])[::2]
                           for r in range(lay.n_req)])
    off = np.searchsorted(cand, lay.req_offsets)
    c_t, o_t = ints(cand), ints(off)
    run_both(spec, lambda: dict(ratio=0.15, cand=c_t, cand_offsets=o_t), "cand")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_paged_rerotate(dtype):
    spec = inputs.small_spec(dtype=dtype)
    w = inputs.generate(spec)
    lay = w.layout
    kc, _ = oracle_caches(w)
    seg_block, table, slot, pool_rows = paged_map(lay, 3)
    flat = LayerCall(spec, lay)
    k1 = upload(kc, dtype)
    S.srp_rerotate_kv(flat.dims, flat.batch, k1)
    paged = paged_call(spec, lay, seg_block, table)
    k2 = upload(to_pool(kc, slot, pool_rows, dtype), dtype)
    S.srp_rerotate_kv(paged.dims, paged.batch, k2)
    torch.cuda.synchronize()
    kf, kp = download(k1), download(k2)
    assert np.array_equal(kp[slot], kf)
    pad = np.setdiff1d(np.arange(pool_rows), slot)
    assert np.all(kp[pad] == inputs.store(np.full(1, POISON), dtype)[0])


def test_validate_rejects_shared_pool_rows():
    spec = inputs.small_spec()
    lay = inputs.generate(spec).layout
    seg_block, table, _, _ = paged_map(lay, 4)
    bad = table.copy()
    bad[1] = bad[0]  # two blocks at one place
    call = paged_call(spec, lay, seg_block, bad)
    with pytest.raises(S.SrpError) as e:
        S.srp_validate_batch(call.batch)
    assert e.value.code == S.SRP_E_BATCH


def test_paged_head_dim_64_gqa8():
    """Head dim 64 with eight query heads per KV head: the gathered K rows, the V
    transpose from the pool and the projection epilogue at the other head size."""
    spec = inputs.small_spec(hidden=1024, n_heads=16, n_kv_heads=2, head_dim=64)
    run_both(spec, lambda: dict(ratio=0.25), "d64 g8")
