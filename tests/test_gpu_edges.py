"""GPU parity at the edges of the input space: a request larger than the LDS-resident
selection holds (the global-memory selection path, with and without grouping), an
empty batch, empty / one-row / cache-only / query-only requests in one batch, a
batch without any cached row, and more requests than one 1024-thread block covers. Compared with the fp64 oracle as in the other
parity tests."""
import copy
import sys

import numpy as np
import pytest
import torch

from oracle import ref
from selective_recompute_prefill_amd import inputs
from selective_recompute_prefill_amd import srp as S
from selective_recompute_prefill_amd.device import LayerCall, download, upload

from parity import assert_close, check_selection, csr_ok, oracle_caches, oracle_layer
from test_gpu_layer import run_case

pytestmark = pytest.mark.gpu

LDS_ROWS = 22528  # rows of one request the LDS-resident selection holds


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def custom_workload(requests, dtype="bf16", hidden=256, n_heads=4, n_kv=2, head_dim=64, seed=7):
    """A workload over an explicit layout: requests = [[(rows, src or -1), ...], ...]
    (segments in order; src = encode position of the segment's first row, -1 fresh).
    Draws come from a one-chunk workload of the same total size."""
    T = sum(n for req in requests for n, _ in req)
    spec = inputs.small_spec("edges", hidden=hidden, n_heads=n_heads, n_kv_heads=n_kv, head_dim=head_dim,
                             dtype=dtype, prefix=0, chunk_lens=(max(T, 1),), n_query=0, n_req=1,
                             seed=inputs.SEED_BASE + 200 + seed)
    w = inputs.generate(spec)
    req_off, seg_off, seg_src, pos = [0], [0], [], []
    for req in requests:
        p = 0
        for n, src in req:
            seg_off.append(seg_off[-1] + n)
            seg_src.append(src)
            pos.append(np.arange(p, p + n, dtype=np.int32))
            p += n
        req_off.append(seg_off[-1])
    if not seg_src:  # an empty batch still has one (empty) segment
        seg_off.append(0)
        seg_src.append(0)
    positions = np.concatenate(pos) if pos else np.zeros(0, np.int32)
    max_pos = int(max([positions.max(initial=0) + 1] + [s + n for req in requests for n, s in req if s >= 0] + [1]))
    lay = inputs.Layout(np.asarray(req_off, np.int32), np.asarray(seg_off, np.int32),
                        np.asarray(seg_src, np.int32), positions, np.zeros(len(seg_src), np.int32), max_pos)
    w2 = copy.copy(w)
    w2.layout = lay
    w2.hidden = w.hidden[:T] if T else w.hidden[:0]
    src = inputs.encode_positions(lay)
    w2.cache_row_of = np.where(src >= 0, np.arange(T), -1).astype(np.int64)
    return spec, w2


def test_request_beyond_lds_selection_uses_global_path():
    # 47 chunks of 512 rows + a 64-row query tail: 24,128 rows in one request
    spec = inputs.small_spec("big-request", hidden=256, n_heads=4, n_kv_heads=2, head_dim=64,
                             prefix=0, chunk_lens=(512,) * 47, n_query=64, n_req=1, ratio=0.2)
    w = inputs.generate(spec)
    lay = w.layout
    assert lay.total_rows > LDS_ROWS
    kc, vc = oracle_caches(w)
    req, src = ref.row_layout(lay.req_offsets, lay.chunk_offsets, lay.chunk_src_pos, lay.total_rows)
    for window, tau in [(0, 0), (8, 4)]:
        call = LayerCall(spec, lay)
        k, v = upload(kc, "bf16"), upload(vc, "bf16")
        _say(f"[gpu] big request T={lay.total_rows} window={window}")
        call.fuse(call.select(0.2, window=window, tau=tau), upload(w.hidden, "bf16"),
                  upload(w.layers[0].w_qkv, "bf16"), k, v)
        torch.cuda.synchronize()
        got = call.results()
        csr_ok(got["sel_idx"], got["sel_offsets"], lay.req_offsets)
        sample = np.unique(np.linspace(0, len(got["sel_idx"]) - 1, 40).astype(np.int64))
        okw = dict(ratio=0.2, window=window, tau=tau)
        if window == 0:
            want = oracle_layer(spec, lay, w.hidden, w.layers[0].w_qkv, kc, vc, attn_sample=sample, **okw)
            check_selection(got["sel_idx"], want, req, "big request top-k")
            assert len(got["sel_idx"]) == ref.topk_count(0.2, int((src >= 0).sum()), 10 ** 9) + 64
            s0 = np.setdiff1d(got["sel_idx"], np.nonzero(src < 0)[0])
        else:
            # the GPU's grouping of its own top-k set (from the ungrouped run)
            seq = np.nonzero(src >= 0)[0]
            kept = ref.group_windows(np.searchsorted(seq, s0), len(seq), 8, 4)
            assert np.array_equal(got["sel_idx"], np.union1d(seq[np.asarray(kept)], np.nonzero(src < 0)[0]))
        want = oracle_layer(spec, lay, w.hidden, w.layers[0].w_qkv, kc, vc, sel_override=got["sel_idx"],
                            attn_sample=sample, **okw)
        assert_close(ref.widen(download(k), "bf16"), want["k_cache"], "bf16", "big request K")
        assert_close(ref.widen(download(v), "bf16"), want["v_cache"], "bf16", "big request V")
        ga = ref.widen(got["attn_out"], "bf16")
        assert_close(ga[sample], want["attn_out"][sample], "bf16", "big request attention (sampled)")
    # external scores need the request resident in LDS
    call = LayerCall(spec, lay)
    sc = torch.ones(lay.total_rows, dtype=torch.float32, device="cuda")
    with pytest.raises(S.SrpError) as e:
        call.ensure_workspace(call.select(0.2, mode=S.SRP_SEL_SCORES, scores=sc))
    assert e.value.code == S.SRP_E_UNSUPPORTED


def test_empty_batch():
    spec, w = custom_workload([[]])
    call = LayerCall(spec, w.layout)
    k = torch.zeros((1, spec.n_kv_heads, spec.head_dim), dtype=torch.bfloat16, device="cuda")
    call.fuse(call.select(0.2), upload(np.zeros((1, spec.hidden), np.uint16), "bf16"),
              upload(w.layers[0].w_qkv, "bf16"), k, k.clone())
    torch.cuda.synchronize()
    got = call.results()
    assert list(got["sel_offsets"]) == [0, 0] and len(got["sel_idx"]) == 0


@pytest.mark.parametrize("window", [0, 4])
def test_empty_one_row_cache_only_and_query_only_requests(window):
    requests = [
        [],                                  # empty request
        [(1, -1)],                           # one fresh row
        [(5, 0)],                            # five cached rows, no query
        [(40, 0), (3, -1), (33, 40), (9, -1)],  # a missing chunk in the middle and a tail
        [],                                  # empty again
        [(7, 100)],                          # encoded far from its global position
    ]
    spec, w = custom_workload(requests)
    kc, vc = oracle_caches(w)
    run_case(spec, w=w, lay=w.layout, kc_st=kc, vc_st=vc,
             sel_kw=dict(ratio=0.3, window=window, tau=2 if window else 0), what=f"edge requests w{window}")


def test_no_cached_rows():
    spec, w = custom_workload([[(50, -1)], [(17, -1), (9, -1)]])
    kc, vc = oracle_caches(w)
    got, want, _ = run_case(spec, w=w, lay=w.layout, kc_st=kc, vc_st=vc, sel_kw=dict(ratio=0.5),
                            what="all fresh")
    assert len(got["sel_idx"]) == w.layout.total_rows  # everything recomputed


@pytest.mark.parametrize("n_req", [63, 64])
@pytest.mark.parametrize("fresh_all", [False, True])
def test_request_table_in_lanes_boundary(n_req, fresh_all):
    """63 and 64 requests of mixed sizes (empty ones included): below 64 the
    scatter keeps the request tables one entry per lane and finds a row's
    request with a ballot, from 64 on it searches them in memory."""
    requests = [[] if i % 9 == 4 else [(5 + (i * 7) % 23, 0), (1 + i % 3, -1)] for i in range(n_req)]
    spec, w = custom_workload(requests, seed=11)
    kc, vc = oracle_caches(w)
    sel_kw, okw = dict(ratio=0.3), {}
    if fresh_all:
        sel_kw["fresh_all"] = okw["fresh_all"] = True
    got, _, _ = run_case(spec, w=w, lay=w.layout, kc_st=kc, vc_st=vc, sel_kw=sel_kw, oracle_kw=okw,
                         what=f"{n_req} requests fresh_all={fresh_all}")
    assert len(got["sel_offsets"]) == n_req + 1


def test_more_requests_than_one_block():
    """1100 requests (every hundredth long, the rest three cached rows and one
    fresh one): the CSR offsets and the attention tile list are built in two
    passes of a 1024-thread block."""
    requests = [[(120, 0), (40, -1)] if i % 100 == 0 else [(3, 0), (1, -1)] for i in range(1100)]
    spec, w = custom_workload(requests, seed=9)
    kc, vc = oracle_caches(w)
    _say(f"[gpu] {len(requests)} requests, T={w.layout.total_rows}")
    got, _, _ = run_case(spec, w=w, lay=w.layout, kc_st=kc, vc_st=vc, sel_kw=dict(ratio=0.34),
                         what="1100 requests")
    assert len(got["sel_offsets"]) == 1101
