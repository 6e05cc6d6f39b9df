"""Device buffers for one layer call: uploads a workload's arrays to HBM as torch
tensors and calls libsrp through the binding. torch is used for device memory and
streams only; every step of the layer runs in libsrp's kernels."""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import srp as S
from .inputs import Layout, Spec


def torch_dtype(dtype: str) -> torch.dtype:
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def srp_dtype(dtype: str) -> int:
    return S.SRP_BF16 if dtype == "bf16" else S.SRP_F32


def upload(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Stored array (float32, or bf16 bit patterns as uint16) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def download(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> stored numpy format (bf16 as uint16 bit patterns)."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def ints(a, device="cuda") -> torch.Tensor:
    return torch.as_tensor(np.asarray(a, np.int32), dtype=torch.int32, device=device)


class LayerCall:
    """Layout tensors, outputs and workspace of srp_fuse_layer for one batch."""

    def __init__(self, spec: Spec, layout: Layout, device="cuda"):
        self.spec = spec
        self.layout = layout
        self.dims = S.make_dims(spec.hidden, spec.n_heads, spec.n_kv_heads, spec.head_dim,
                                spec.rope_base, srp_dtype(spec.dtype))
        self.req_offsets = ints(layout.req_offsets, device)
        self.chunk_offsets = ints(layout.chunk_offsets, device)
        self.chunk_src_pos = ints(layout.chunk_src_pos, device)
        self.positions = ints(layout.positions, device)
        T = layout.total_rows
        ro = layout.req_offsets
        self.max_req_rows = int(max(np.diff(ro).max(initial=0), 1))
        self.batch = S.make_batch(self.req_offsets, self.chunk_offsets, self.chunk_src_pos,
                                  self.positions, total_rows=T, max_req_rows=self.max_req_rows,
                                  max_position=layout.max_position)
        td = torch_dtype(spec.dtype)
        self.sel_idx = torch.full((max(T, 1),), -1, dtype=torch.int32, device=device)
        self.sel_offsets = torch.zeros(layout.n_req + 1, dtype=torch.int32, device=device)
        self.attn_out = torch.zeros((max(T, 1), spec.n_heads, spec.head_dim), dtype=td, device=device)
        self.dev_out = torch.zeros(max(T, 1), dtype=torch.float32, device=device)
        self.workspace: Optional[torch.Tensor] = None
        self.device = device

    def select(self, ratio: float, **kw) -> S.Select:
        return S.make_select(ratio, **kw)

    def ensure_workspace(self, sel: S.Select) -> int:
        n = S.srp_workspace_size(self.dims, self.batch, sel)
        if self.workspace is None or self.workspace.numel() < n:
            self.workspace = torch.empty(n, dtype=torch.uint8, device=self.device)
        return n

    def fuse(self, sel: S.Select, hidden, w_qkv, k_cache, v_cache, dev_out=True, stream=None):
        n = self.ensure_workspace(sel)
        S.srp_fuse_layer(self.dims, self.batch, sel, hidden, w_qkv, k_cache, v_cache,
                         self.sel_idx, self.sel_offsets, self.attn_out,
                         self.dev_out if dev_out else None, self.workspace, n, stream)

    def results(self) -> Dict[str, np.ndarray]:
        off = self.sel_offsets.cpu().numpy().astype(np.int64)
        n = int(off[-1])
        return dict(sel_idx=self.sel_idx[:n].cpu().numpy().astype(np.int64), sel_offsets=off,
                    attn_out=download(self.attn_out[:n]), dev=self.dev_out.cpu().numpy())


def encode_cache(spec: Spec, layout: Layout, x_enc: torch.Tensor, w_qkv: torch.Tensor,
                 src_positions: np.ndarray, device="cuda"):
    """Chunk caches of the cached rows encoded on the device at their encode positions
    (srp_encode_kv); fresh rows are left zero."""
    T = layout.total_rows
    td = torch_dtype(spec.dtype)
    k = torch.zeros((T, spec.n_kv_heads, spec.head_dim), dtype=td, device=device)
    v = torch.zeros_like(k)
    rows = np.nonzero(src_positions >= 0)[0]
    if len(rows) == 0:
        return k, v
    dims = S.make_dims(spec.hidden, spec.n_heads, spec.n_kv_heads, spec.head_dim, spec.rope_base,
                       srp_dtype(spec.dtype))
    idx = torch.as_tensor(rows, dtype=torch.long, device=device)
    xr = x_enc.index_select(0, idx).contiguous()
    pos = ints(src_positions[rows], device)
    kr = torch.empty((len(rows), spec.n_kv_heads, spec.head_dim), dtype=td, device=device)
    vr = torch.empty_like(kr)
    S.srp_encode_kv(dims, len(rows), layout.max_position, xr, w_qkv, pos, kr, vr)
    k.index_copy_(0, idx, kr)
    v.index_copy_(0, idx, vr)
    return k, v
