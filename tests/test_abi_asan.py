"""The C ABI's host code under AddressSanitizer (CPU only): a debug build of the
library with the host pass instrumented runs every host-checkable path (argument
checks and their messages, workspace sizes over many shapes, the controller, the
no-allocation variant's size limit, the stack executor's checks) in a subprocess
that preloads the ASan runtime; any heap, stack or global overflow aborts it."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r'''
import ctypes, itertools
from selective_recompute_prefill_amd import srp as S
L = S.lib()
assert S.srp_version().startswith("libsrp")
n = ctypes.c_size_t(0)
for (H, nh, nkv, d), dt, T, nreq, bl in itertools.product(
        [(256, 4, 2, 64), (5120, 40, 8, 128), (8192, 64, 8, 128), (512, 8, 8, 128)],
        [S.SRP_BF16, S.SRP_F32], [0, 1, 577, 16512], [1, 3], [0, 16]):
    dims = S.make_dims(H, nh, nkv, d, 1e4, dt)
    b = S.Batch(nreq, 2, T, max(T, 1), T + 64, 8, 8, 8, 8, bl, 8 if bl else None, 8 if bl else None)
    for sel in (S.make_select(0.2), S.make_select(0.3, window=8, tau=4), S.make_select(0.1, dev_mode=S.SRP_DEV_V)):
        assert L.srp_workspace_size(ctypes.byref(dims), ctypes.byref(b), ctypes.byref(sel), ctypes.byref(n)) == 0
        assert n.value > 0
        assert L.srp_stack_workspace_size(ctypes.byref(dims), ctypes.byref(b), ctypes.byref(sel), ctypes.byref(n)) == 0
# every rejected argument leaves a message
dims = S.make_dims(5120, 40, 8, 128)
b = S.Batch(1, 2, 100, 100, 200, 8, 8, 8, 8, 0, None, None)
bad = [
    (S.make_dims(5120, 40, 8, 96), b, S.make_select(0.2)),
    (S.make_dims(5120, 40, 7, 128), b, S.make_select(0.2)),
    (S.make_dims(5120, 72, 8, 128), b, S.make_select(0.2)),
    (dims, S.Batch(0, 2, 100, 100, 200, 8, 8, 8, 8, 0, None, None), S.make_select(0.2)),
    (dims, S.Batch(1, 2, 100, 100, 200, 8, 8, 8, 8, 16, None, None), S.make_select(0.2)),
    (dims, b, S.make_select(1.5)),
    (dims, b, S.make_select(0.2, window=8, tau=9)),
    (dims, b, S.make_select(0.2, mode=S.SRP_SEL_GIVEN)),
    (dims, b, S.make_select(0.2, span_max=16)),
    (dims, b, S.make_select(0.2, mode=S.SRP_SEL_SCORES, scores=8, span_max=2000)),
]
for dd, bb, ss in bad:
    rc = L.srp_workspace_size(ctypes.byref(dd), ctypes.byref(bb), ctypes.byref(ss), ctypes.byref(n))
    assert rc < 0 and len(L.srp_last_error()) > 0, rc
    rc = L.srp_fuse_layer(ctypes.byref(dd), ctypes.byref(bb), ctypes.byref(ss), 8, 8, 8, 8, 8, 8, 8, None, 8, 1 << 40, None)
    assert rc < 0 and len(L.srp_last_error()) > 0, rc
# workspace too small, NULL tensors, the no-allocation variant's limit
sel = S.make_select(0.2)
assert L.srp_fuse_layer(ctypes.byref(dims), ctypes.byref(b), ctypes.byref(sel), 8, 8, 8, 8, 8, 8, 8, None, 8, 16, None) == S.SRP_E_WORKSPACE
assert L.srp_fuse_layer(ctypes.byref(dims), ctypes.byref(b), ctypes.byref(sel), None, 8, 8, 8, 8, 8, 8, None, 8, 1 << 40, None) == S.SRP_E_INVALID
big = S.Batch(1, 2, 16512, 16512, 16512, 8, 8, 8, 8, 0, None, None)
assert L.srp_fuse_layer_noalloc(ctypes.byref(dims), ctypes.byref(big), ctypes.byref(sel), 8, 8, 8, 8, 8, 8, 8, None, None) == S.SRP_E_WORKSPACE
# controller and stack checks
r = ctypes.c_double(0)
assert L.srp_controller_ratio(1.2, 0.3, 0.15, ctypes.byref(r)) == 0 and abs(r.value - 0.25) < 1e-12
assert L.srp_controller_ratio(0.0, 0.3, 0.15, ctypes.byref(r)) == S.SRP_E_INVALID
lay = (S.Layer * 2)(S.make_layer(8, 8, 8, 0.3), S.make_layer(8, 8, 8, 0.15, mode=7))
assert L.srp_fuse_stack(ctypes.byref(dims), ctypes.byref(b), ctypes.byref(sel), 2, lay, 8, ctypes.c_float(1e-6), 8, 8, 8, 8, 1 << 40, None, None) == S.SRP_E_INVALID
for i in range(-2, S.SRP_N_STAGES + 2):
    L.srp_profile_stage_name(i)
assert "libclang_rt.asan" in open("/proc/self/maps").read(), "the ASan runtime is not loaded"
print("asan host paths ok")
'''


def test_host_paths_under_address_sanitizer():
    from selective_recompute_prefill_amd import build_asan as BA
    lib = BA.build_asan()
    # the host code is instrumented (it reports through the runtime's entry points)
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in nm
    env = dict(os.environ, SRP_LIB=lib, LD_PRELOAD=BA.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1", PYTHONPATH=ROOT)
    p = subprocess.run([sys.executable, "-c", SCRIPT], env=env, capture_output=True, text=True, timeout=600)
    assert p.returncode == 0 and "asan host paths ok" in p.stdout, p.stdout[-2000:] + p.stderr[-4000:]
