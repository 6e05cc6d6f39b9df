"""GPU checks of srp_fuse_stack, the stack executor that loads each layer's chunk
caches from page-locked host memory on a copy stream while earlier layers compute.

The executor only orders existing kernels, so its results must equal, bit for bit,
the same layers run one by one through srp_fuse_layer and srp_residual_rmsnorm with
the caches already on the device; with the copies in line on the compute stream
too. Against the fp64 oracle's stack (gradual filtering with the residual RMSNorm
chain) selections must agree and values stay within the bf16 tolerance."""
import sys

import numpy as np
import pytest
import torch

from oracle import ref
from selective_recompute_prefill_amd import inputs
from selective_recompute_prefill_amd import srp as S
from selective_recompute_prefill_amd.device import LayerCall, download, upload

from parity import assert_close, check_selection, csr_ok, oracle_caches

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _pinned(a: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return t.pin_memory()


def _stack_spec(**kw):
    base = dict(hidden=1024, n_heads=8, n_kv_heads=2, head_dim=128, n_layers=4,
                ratios=(0.3, 0.15, 0.15, 0.15), ratio=0.3)
    base.update(kw)
    return inputs.small_spec("stack", **base)


def _serial(spec, lay, call, w, caches, first_kw, modes=None):
    """The reference chain: one srp_fuse_layer + srp_residual_rmsnorm per layer
    (modes[l] for l >= 1: SRP_SEL_TOPK checks the layer, SRP_SEL_GIVEN passes the
    previous selection on)."""
    T = lay.total_rows
    h = upload(w.hidden, "bf16")
    kcs, vcs = [], []
    prev_i = torch.empty_like(call.sel_idx)
    prev_o = torch.empty_like(call.sel_offsets)
    steps = []  # each chain step's hidden before and after, with the layer's output
    for l in range(spec.n_layers):
        kc, vc = upload(caches[l][0], "bf16"), upload(caches[l][1], "bf16")
        if l == 0:
            sel = call.select(spec.layer_ratios()[0], **first_kw)
        else:
            prev_i.copy_(call.sel_idx)
            prev_o.copy_(call.sel_offsets)
            mode = S.SRP_SEL_TOPK if modes is None else modes[l]
            sel = call.select(spec.layer_ratios()[l], mode=mode, cand=prev_i, cand_offsets=prev_o)
        call.fuse(sel, h, upload(w.layers[l].w_qkv, "bf16"), kc, vc, dev_out=False)
        torch.cuda.synchronize()
        before = download(h)
        S.srp_residual_rmsnorm(call.dims, h, call.attn_out, call.sel_idx, call.sel_offsets, lay.n_req, T)
        torch.cuda.synchronize()
        r = call.results()
        steps.append(dict(before=before, after=download(h), attn=r["attn_out"], sel_idx=r["sel_idx"]))
        kcs.append(kc)
        vcs.append(vc)
    torch.cuda.synchronize()
    r = call.results()
    return dict(sel_idx=r["sel_idx"], sel_offsets=r["sel_offsets"], attn=r["attn_out"],
                hidden=download(h), k=[download(k) for k in kcs], v=[download(v) for v in vcs], steps=steps)


def _stacked(spec, lay, w, caches, first_kw, copy_stream, modes=None):
    """The same chain through srp_fuse_stack with the caches in pinned host memory."""
    T = lay.total_rows
    call = LayerCall(spec, lay)
    first = call.select(spec.layer_ratios()[0], **first_kw)
    h = upload(w.hidden, "bf16")
    ws_n = S.srp_stack_workspace_size(call.dims, call.batch, first)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    keep, layers, kcs, vcs = [], [], [], []
    for l in range(spec.n_layers):
        kh, vh = _pinned(caches[l][0]), _pinned(caches[l][1])
        kc = torch.empty((T, spec.n_kv_heads, spec.head_dim), dtype=torch.bfloat16, device="cuda")
        vc = torch.empty_like(kc)
        wq = upload(w.layers[l].w_qkv, "bf16")
        keep += [kh, vh, wq]
        kcs.append(kc)
        vcs.append(vc)
        layers.append(S.make_layer(wq, kc, vc, spec.layer_ratios()[l], k_host=kh, v_host=vh,
                                   mode=S.SRP_SEL_TOPK if modes is None else modes[l]))
    S.srp_fuse_stack(call.dims, call.batch, first, layers, h, 1e-6, call.sel_idx, call.sel_offsets,
                     call.attn_out, ws, ws_n, None, copy_stream)
    torch.cuda.synchronize()
    r = call.results()
    return dict(sel_idx=r["sel_idx"], sel_offsets=r["sel_offsets"], attn=r["attn_out"],
                hidden=download(h), k=[download(k) for k in kcs], v=[download(v) for v in vcs])


def _check_chain_steps(ser):
    """Each chain step of the serial run against the oracle's residual RMSNorm on the
    same stored inputs: the selected rows within the bf16 tolerance of one layer, every
    other row unchanged."""
    for l, st in enumerate(ser["steps"]):
        s = st["sel_idx"]
        x = ref.widen(st["before"], "bf16")
        want = ref.residual_rmsnorm(x[s], ref.widen(st["attn"], "bf16").reshape(len(s), -1))
        got = ref.widen(st["after"], "bf16")
        assert_close(got[s], want, "bf16", f"chain step {l}")
        rest = np.ones(len(x), bool)
        rest[s] = False
        assert np.array_equal(st["after"][rest], st["before"][rest]), f"chain step {l}: unselected rows changed"


def _same(a, b, what):
    for key in ("sel_idx", "sel_offsets", "attn", "hidden"):
        assert np.array_equal(a[key], b[key]), f"{what}: {key} differs"
    for l in range(len(a["k"])):
        assert np.array_equal(a["k"][l], b["k"][l]), f"{what}: K cache of layer {l} differs"
        assert np.array_equal(a["v"][l], b["v"][l]), f"{what}: V cache of layer {l} differs"


@pytest.mark.parametrize("first", ["topk", "grouped", "check-two-layers"])
def test_stack_equals_serial_layers_and_oracle(first):
    """check-two-layers: layers 1 and 2 check (rank by deviation), layers 3 and 4
    recompute the indices layer 2 chose (CacheBlend walkthrough, "Implementation":
    the per-layer check_flag with the carried indices)."""
    spec = _stack_spec()
    w = inputs.generate(spec)
    lay = w.layout
    caches = [oracle_caches(w, l) for l in range(spec.n_layers)]
    first_kw = dict(window=8, tau=4) if first == "grouped" else {}
    modes = None
    if first == "check-two-layers":
        modes = [S.SRP_SEL_TOPK, S.SRP_SEL_TOPK, S.SRP_SEL_GIVEN, S.SRP_SEL_GIVEN]
    _say(f"[gpu] stack {first}: T={lay.total_rows}, {spec.n_layers} layers")
    ser = _serial(spec, lay, LayerCall(spec, lay), w, caches, first_kw, modes)
    _check_chain_steps(ser)
    side = torch.cuda.Stream()
    piped = _stacked(spec, lay, w, caches, first_kw, side, modes)
    _same(piped, ser, "copy stream")
    inline = _stacked(spec, lay, w, caches, first_kw, None, modes)
    _same(inline, ser, "copies in line")

    # the oracle's stack on the same stored inputs (hidden rounded to bf16 between layers)
    rb = lambda y: ref.widen(inputs.store(y, "bf16"), "bf16")
    outs = ref.fuse_stack(hidden=ref.widen(w.hidden, "bf16"),
                          layers=[dict(w_qkv=ref.widen(w.layers[l].w_qkv, "bf16"),
                                       k_cache=ref.widen(caches[l][0], "bf16"),
                                       v_cache=ref.widen(caches[l][1], "bf16"))
                                  for l in range(spec.n_layers)],
                          req_offsets=lay.req_offsets, chunk_offsets=lay.chunk_offsets,
                          chunk_src_pos=lay.chunk_src_pos, positions=lay.positions,
                          n_heads=spec.n_heads, n_kv=spec.n_kv_heads, head_dim=spec.head_dim,
                          rope_base=spec.rope_base, ratios=spec.layer_ratios(),
                          window=first_kw.get("window", 0), tau=first_kw.get("tau", 0), round_hidden=rb,
                          modes=None if modes is None else ["topk" if m == S.SRP_SEL_TOPK else "given"
                                                            for m in modes])
    if modes is not None:  # the passed-on layers keep layer 2's rows
        assert np.array_equal(outs[3]["sel_idx"], outs[1]["sel_idx"])
    last = outs[-1]
    req, _ = ref.row_layout(lay.req_offsets, lay.chunk_offsets, lay.chunk_src_pos, lay.total_rows)
    csr_ok(piped["sel_idx"], piped["sel_offsets"], lay.req_offsets)
    assert np.array_equal(piped["sel_idx"], last["sel_idx"]), "last layer's selection differs from the oracle"
    for l, o in enumerate(outs):
        assert_close(ref.widen(piped["k"][l], "bf16"), o["k_cache"], "bf16", f"layer {l} K cache")
        assert_close(ref.widen(piped["v"][l], "bf16"), o["v_cache"], "bf16", f"layer {l} V cache")
    assert_close(ref.widen(piped["attn"], "bf16"), last["attn_out"], "bf16", "last layer attention")
    x = ref.widen(w.hidden, "bf16").copy()
    for o in outs:  # the oracle's hidden after every chain step
        s = o["sel_idx"]
        x[s] = rb(ref.residual_rmsnorm(o["hidden_in"][s], o["attn_out"].reshape(len(s), -1)))
    # the hidden state went through every layer's chain step: each adds its layer's
    # output error (and a bf16 rounding) to the residual, so the max-abs bound is one
    # layer's bound per chained layer; rel-L2 keeps the single-layer bound (every step
    # on its own inputs is held to one layer's bound by _check_chain_steps)
    got_h = ref.widen(piped["hidden"], "bf16")
    err = np.abs(got_h - x)
    assert np.linalg.norm(got_h - x) / np.linalg.norm(x) <= 1e-2
    assert err.max() <= 3e-2 * spec.n_layers, f"stack output hidden: max-abs {err.max():.3e}"


def test_stack_single_layer_without_host_caches():
    """One layer whose cache is already on the device: the executor reduces to
    srp_fuse_layer followed by the chain step."""
    spec = _stack_spec(n_layers=1, ratios=(0.2,), ratio=0.2)
    w = inputs.generate(spec)
    lay = w.layout
    caches = [oracle_caches(w, 0)]
    ser = _serial(spec, lay, LayerCall(spec, lay), w, caches, {})
    _check_chain_steps(ser)
    call = LayerCall(spec, lay)
    first = call.select(0.2)
    h = upload(w.hidden, "bf16")
    kc, vc = upload(caches[0][0], "bf16"), upload(caches[0][1], "bf16")
    n = S.srp_stack_workspace_size(call.dims, call.batch, first)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    S.srp_fuse_stack(call.dims, call.batch, first, [S.make_layer(upload(w.layers[0].w_qkv, "bf16"), kc, vc, 0.2)],
                     h, 1e-6, call.sel_idx, call.sel_offsets, call.attn_out, ws, n)
    torch.cuda.synchronize()
    r = call.results()
    got = dict(sel_idx=r["sel_idx"], sel_offsets=r["sel_offsets"], attn=r["attn_out"], hidden=download(h),
               k=[download(kc)], v=[download(vc)])
    _same(got, ser, "single layer")
