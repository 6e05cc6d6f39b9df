"""GPU checks of srp_fuse_layer_noalloc, the entry point for callers that cannot
allocate: its outputs must match srp_fuse_layer's on the same inputs (selection
exact up to near-ties, with equal sizes per request; K/V caches, deviations and
attention within the dtype's tolerance), over consecutive calls that shrink the
input and change the shape, so that each call runs on what the last one left in
the static scratch array."""
import sys

import numpy as np
import pytest
import torch

from oracle import ref
from selective_recompute_prefill_amd import inputs
from selective_recompute_prefill_amd import srp as S
from selective_recompute_prefill_amd.device import LayerCall, download, ints, upload

from parity import NEAR_TIE, assert_close, csr_ok, oracle_caches

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _pair(spec, sel_kw, what):
    """The layer through srp_fuse_layer (reference) and srp_fuse_layer_noalloc."""
    w = inputs.generate(spec)
    lay = w.layout
    kc, vc = oracle_caches(w)
    hid, wq = upload(w.hidden, spec.dtype), upload(w.layers[0].w_qkv, spec.dtype)
    ratio = sel_kw.pop("ratio")

    def run(noalloc, kw):
        call = LayerCall(spec, lay)
        k, v = upload(kc, spec.dtype), upload(vc, spec.dtype)
        sel = S.make_select(ratio, **kw)
        if noalloc:
            S.srp_fuse_layer_noalloc(call.dims, call.batch, sel, hid, wq, k, v, call.sel_idx,
                                     call.sel_offsets, call.attn_out, call.dev_out)
            assert call.workspace is None
        else:
            call.fuse(sel, hid, wq, k, v)
        torch.cuda.synchronize()
        r = call.results()
        r["k"], r["v"] = download(k), download(v)
        return r

    _say(f"[gpu] noalloc {what}: T={lay.total_rows}")
    a, b = run(False, sel_kw), run(True, sel_kw)
    csr_ok(b["sel_idx"], b["sel_offsets"], lay.req_offsets)
    assert np.array_equal(a["sel_offsets"], b["sel_offsets"]), f"{what}: selected rows per request differ"
    if not np.array_equal(a["sel_idx"], b["sel_idx"]):
        # near-ties only: the two top-k sets (grouping off) may differ only in rows
        # within NEAR_TIE of the reference's k-th largest deviation; the outputs are
        # then compared with both entry points given the reference's selection
        _, src = ref.row_layout(lay.req_offsets, lay.chunk_offsets, lay.chunk_src_pos, lay.total_rows)
        req = np.searchsorted(lay.req_offsets, np.arange(lay.total_rows), side="right") - 1
        kw0 = dict(sel_kw, window=0, tau=0)
        a0, b0 = run(False, kw0), run(True, kw0)
        assert np.array_equal(a0["sel_offsets"], b0["sel_offsets"]), f"{what}: top-k sizes differ"
        sym = sorted(set(a0["sel_idx"].tolist()) ^ set(b0["sel_idx"].tolist()))
        assert sym, f"{what}: equal top-k sets grouped differently"
        for j in sym:
            top = a0["sel_idx"][(req[a0["sel_idx"]] == req[j]) & (src[a0["sel_idx"]] >= 0)]
            kth = a0["dev"][top].min()
            assert abs(a0["dev"][j] - kth) / kth < NEAR_TIE, f"{what}: row {j} differs and is no near-tie"
        cached = a["sel_idx"][src[a["sel_idx"]] >= 0]
        off = np.searchsorted(cached, lay.req_offsets)
        given = dict(mode=S.SRP_SEL_GIVEN, cand=ints(cached), cand_offsets=ints(off))
        a, b = run(False, given), run(True, given)
        assert np.array_equal(a["sel_idx"], b["sel_idx"])
    dt = spec.dtype
    assert np.array_equal(np.isnan(a["dev"]), np.isnan(b["dev"]))
    m = np.isfinite(a["dev"])
    if m.any():
        rel = np.abs(a["dev"][m] - b["dev"][m]) / np.maximum(a["dev"][m], 1e-30)
        assert rel.max() < 1e-4, f"{what}: deviation rel diff {rel.max():.2e}"
    assert_close(ref.widen(b["k"], dt), ref.widen(a["k"], dt), dt, what + " K cache")
    assert_close(ref.widen(b["v"], dt), ref.widen(a["v"], dt), dt, what + " V cache")
    assert_close(ref.widen(b["attn_out"], dt), ref.widen(a["attn_out"], dt), dt, what + " attention")


def test_noalloc_matches_workspace_entry_point_over_shrinking_calls():
    # 1: the 8B-shaped layer (3136 rows); 2: a smaller two-request layer with
    # grouping; 3: head dim 64 (the rotary table is rebuilt); 4: fp32
    _pair(inputs.WORKLOADS[1], dict(ratio=0.15), "llama3-8b-layer")
    _pair(inputs.small_spec(window=8, tau=4), dict(ratio=0.2, window=8, tau=4), "mini grouped")
    _pair(inputs.small_spec(head_dim=64, n_heads=8, n_kv_heads=4), dict(ratio=0.3), "mini d64")
    _pair(inputs.WORKLOADS[0], dict(ratio=0.2), "tiny fp32")


def test_noalloc_rejects_a_layer_beyond_its_scratch():
    spec = inputs.WORKLOADS[2]  # 16,512 rows at hidden 5120: more than 128 MiB
    lay = inputs.make_layout(spec)
    call = LayerCall(spec, lay)
    hid = torch.empty((1,), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(S.SrpError) as e:
        S.srp_fuse_layer_noalloc(call.dims, call.batch, S.make_select(0.2), hid, hid, hid, hid, call.sel_idx,
                                 call.sel_offsets, call.attn_out, None)
    assert e.value.code == S.SRP_E_WORKSPACE
