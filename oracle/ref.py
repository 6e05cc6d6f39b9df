"""fp64 CPU oracle of the selective-recompute prefill layer ("KV cache fusor").

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute
this module: only the tests, the package smoke check and the CPU-baseline leg of the
benchmark use it. It shares no code with the HIP library (no kernels, headers,
tables or helpers); the two meet only in the seeded input generator, which holds
none of the layer's arithmetic.

Everything here is plain numpy float64, written for a reader to check against the
pages by eye; speed is not a goal. Each function names the passage it follows:

* "CacheBlend walkthrough" = the CacheBlend blog post (sarpat.github.io), sections
  "Selective KV recompute", "Picking the tokens to recompute", "The chicken-and-egg
  problem", "Implementation".
* "CacheClip paper" = arXiv 2510.10129, sections 4.1-4.3; "CacheClip walkthrough" =
  the CacheClip blog post, sections 6.1-6.3 (Figure 6 and the grouping pseudo-code).
* "SpecCache notes" = the SpecCache reading notes, sections 2.1-2.2.
* "Cache-Craft summary" = the Cache-Craft abstract page, sections 3.4 and 4.

Where the pages are silent, garbled or disagree, the reading taken is stated at the
function and listed, with every other reading, in the design notes of the repo.

Parity status: every function is pinned by the CPU tests (closed forms, brute
force, library cross-checks, the grouping figure; for span completion, hand-worked
cases, a characterisation of the segmentation and a cross-check of the external-score
mode against deviation-ranked top-k; for the chain step, hand-worked rows; for bf16
widening, hand-decoded bit patterns and torch's conversion of every pattern). The intermediate layers of the
multi-layer chain are pinned only through the invariants of the single layer and
the all-recompute reduction of the whole stack.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

# --------------------------------------------------------------------------- #
# storage formats
# --------------------------------------------------------------------------- #


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored array -> exact float64. bf16 is held as uint16 bit patterns."""
    if dtype == "f32":
        return np.asarray(a, np.float32).astype(np.float64)
    if dtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------- #
# rotary position embedding
# --------------------------------------------------------------------------- #


def rope_inv_freq(head_dim: int, base: float) -> np.ndarray:
    """Frequencies base^(-2i/d), i < d/2, in float64 (RoFormer, cited by the
    CacheBlend walkthrough, "Selective KV recompute")."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / head_dim)


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate x [n, heads, d] by positions pos [n] (rotate-half pairing of
    element i with element i + d/2). The angle is pos * inv_freq_i."""
    d = x.shape[-1]
    half = d // 2
    theta = np.asarray(pos, np.float64)[:, None] * rope_inv_freq(d, base)[None, :]
    c = np.cos(theta)[:, None, :]
    s = np.sin(theta)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# --------------------------------------------------------------------------- #
# layout
# --------------------------------------------------------------------------- #


def row_layout(req_offsets, chunk_offsets, chunk_src_pos, total_rows: int):
    """Per-row request id and encode position (-1 = fresh row without cache).

    A cached segment's rows were encoded at consecutive positions starting at
    chunk_src_pos[c] (CacheClip paper, section 4.1: each chunk was precomputed from
    the same offset after the shared prefix)."""
    req = np.full(total_rows, -1, np.int64)
    for r in range(len(req_offsets) - 1):
        req[req_offsets[r]:req_offsets[r + 1]] = r
    src = np.full(total_rows, -1, np.int64)
    for c in range(len(chunk_src_pos)):
        a, b = int(chunk_offsets[c]), int(chunk_offsets[c + 1])
        if chunk_src_pos[c] >= 0:
            src[a:b] = int(chunk_src_pos[c]) + np.arange(b - a)
    return req, src


# --------------------------------------------------------------------------- #
# the steps of one layer
# --------------------------------------------------------------------------- #


def project_q(x: np.ndarray, w_qkv: np.ndarray, n_heads: int, n_kv: int, d: int):
    """Q = x W_q^T (rows of w_qkv: Q, then K, then V), shaped [n, heads, d]."""
    qd = n_heads * d
    return (x @ w_qkv[:qd].T).reshape(x.shape[0], n_heads, d)


def project_kv(x: np.ndarray, w_qkv: np.ndarray, n_heads: int, n_kv: int, d: int):
    """K, V = x W_k^T, x W_v^T (rows of w_qkv: Q, then K, then V)."""
    qd, kvd = n_heads * d, n_kv * d
    wk, wv = w_qkv[qd:qd + kvd], w_qkv[qd + kvd:qd + 2 * kvd]
    n = x.shape[0]
    return (x @ wk.T).reshape(n, n_kv, d), (x @ wv.T).reshape(n, n_kv, d)


def project(x: np.ndarray, w_qkv: np.ndarray, n_heads: int, n_kv: int, d: int):
    """Q, K, V = x W_q^T, x W_k^T, x W_v^T."""
    return (project_q(x, w_qkv, n_heads, n_kv, d),) + project_kv(x, w_qkv, n_heads, n_kv, d)


def encode_kv(x: np.ndarray, w_qkv: np.ndarray, pos: np.ndarray, n_heads: int,
              n_kv: int, d: int, base: float):
    """Offline chunk cache: K = R(pos) W_k x and V = W_v x for each row, at the
    positions the rows are encoded at (CacheClip walkthrough, Figure 4, offline
    phase; chunk-local positions)."""
    k, v = project_kv(x, w_qkv, n_heads, n_kv, d)
    return rope(k, pos, base), v


def rerotate(k_cache: np.ndarray, positions: np.ndarray, src: np.ndarray, base: float):
    """Move each cached key from its encode position to its global position by one
    rotation R(pos - src) (CacheBlend walkthrough, "Selective KV recompute": under
    RoPE a score depends only on relative distance, so relocating a chunk is a single
    multiplication of its K by a rotation; SpecCache notes 2.1, positional recovery).
    Fresh rows (src = -1) are returned unchanged."""
    out = k_cache.copy()
    m = src >= 0
    out[m] = rope(k_cache[m], positions[m] - src[m], base)
    return out


def kv_deviation(k_new, v_new, k_old, v_old, mode: str = "kv") -> np.ndarray:
    """Per-token KV deviation: L2 norm of (recomputed - cached) over the token's K and
    V rows of every KV head (CacheBlend walkthrough, "Selective KV recompute"; the
    formula itself was lost from the page, and the L2-over-K-and-V reading is taken).
    mode "v" keeps only the V term (the CacheClip paper's account of CacheBlend
    comparing value matrices)."""
    n = k_new.shape[0]
    dv = ((v_new - v_old) ** 2).reshape(n, -1).sum(axis=1)
    if mode == "v":
        return np.sqrt(dv)
    dk = ((k_new - k_old) ** 2).reshape(n, -1).sum(axis=1)
    return np.sqrt(dk + dv)


def topk_count(ratio: float, n_ctx: int, n_cand: int, rule: str = "round") -> int:
    """Top-k size from the recompute ratio, clamped to the number of candidates.
    rule "round": k = round(ratio * N) with halves rounded up (CacheClip walkthrough,
    section 6.2: k = round(recomp_ratio * N)); rule "ceil": K = ceil(rho * N)
    (SpecCache notes 2.2). N = cached rows of the request; the product is taken in
    float64."""
    x = float(ratio) * n_ctx
    if rule == "ceil":
        k = np.ceil(x)
    elif rule == "round":
        k = np.floor(x + 0.5)
    else:
        raise ValueError(rule)
    return int(min(k, n_cand))


def topk_rows(dev: np.ndarray, rows: np.ndarray, k: int) -> np.ndarray:
    """The k rows with the largest deviation; equal deviations go to the lower row
    index. Returned ascending. (CacheBlend walkthrough, "Implementation": the tokens
    with the largest deviation become the new selection.)"""
    if k <= 0:
        return np.zeros(0, np.int64)
    order = np.lexsort((rows, -dev))  # primary: -dev ascending; secondary: row
    return np.sort(rows[order[:k]])


def group_windows(cand_seq: Sequence[int], seq_len: int, w: int, tau: int) -> List[int]:
    """Sliding-window grouping over a sequence of seq_len token slots (CacheClip
    paper 4.3; CacheClip walkthrough 6.3, Figure 6). Windows have size w and move
    with step 1, so a window is identified by its first slot; only windows whose
    first slot is a candidate are evaluated, and only those lying wholly inside the
    sequence. The candidate count inside a window is its local density; a window
    of density >= tau adds all of its w slots (gaps included) to the result.
    Candidates that no such window covers are dropped."""
    cand = sorted(set(int(c) for c in cand_seq))
    member = np.zeros(seq_len, bool)
    member[cand] = True
    keep = np.zeros(seq_len, bool)
    for start in cand:
        if start + w > seq_len:
            continue
        if int(member[start:start + w].sum()) >= tau:
            keep[start:start + w] = True
    return [int(i) for i in np.nonzero(keep)[0]]


# --------------------------------------------------------------------------- #
# span completion of a score-ranked selection
# --------------------------------------------------------------------------- #


def normalise_scores(score: np.ndarray) -> np.ndarray:
    """Min-max normalisation of a token score sequence to [0, 1] (SpecCache notes 2.3,
    span segmentation). Constant scores give 0/0 = NaN everywhere (IEEE); the span
    rule below then merges nothing."""
    s = np.asarray(score, np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        return (s - s.min()) / (s.max() - s.min())


def relative_change(norm: np.ndarray) -> np.ndarray:
    """delta_i = |I~_{i+1} - I~_i| / I~_i for consecutive tokens of the sequence
    (SpecCache notes 2.3), evaluated in IEEE float64: a token at the minimum gives
    +inf (or NaN when its successor is also at the minimum)."""
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.abs(norm[1:] - norm[:-1]) / norm[:-1]


def segment_spans(score: np.ndarray, tau_smooth: float, max_len: int) -> List[tuple]:
    """Split a token sequence into spans [u, v] (inclusive) of locally smooth scores
    (SpecCache notes 2.3): walking left to right, the next token joins the current
    span while delta < tau_smooth holds (a NaN delta does not hold) and the span is
    shorter than max_len; otherwise a new span starts at that token."""
    n = len(score)
    if n == 0:
        return []
    delta = relative_change(normalise_scores(score))
    spans = []
    u = 0
    for i in range(n - 1):
        if delta[i] < tau_smooth and i - u + 1 < max_len:
            continue
        spans.append((u, i))
        u = i + 1
    spans.append((u, n - 1))
    return spans


def complete_spans(score: np.ndarray, init: np.ndarray, tau_smooth: float, max_len: int,
                   tau_cover: float) -> np.ndarray:
    """Coverage-based span completion (SpecCache notes 2.3): a span whose share of
    initially selected tokens, |T_init & [u, v]| / (v - u + 1) in float64, is at least
    tau_cover is added whole; the result is T_init united with those spans."""
    init = np.asarray(init, bool)
    out = init.copy()
    for u, v in segment_spans(score, tau_smooth, max_len):
        cover = float(init[u:v + 1].sum()) / float(v - u + 1)
        if cover >= tau_cover:
            out[u:v + 1] = True
    return out


def budget_cap(score: np.ndarray, chosen: np.ndarray, m: int) -> np.ndarray:
    """Global budget after span completion (SpecCache notes 2.3): when more than m
    tokens are chosen, keep the m with the highest score (equal scores: the earlier
    token) and drop the rest."""
    chosen = np.asarray(chosen, bool)
    if chosen.sum() <= m:
        return chosen.copy()
    idx = np.nonzero(chosen)[0]
    keep = topk_rows(np.asarray(score, np.float64)[idx], idx, m)
    out = np.zeros_like(chosen)
    out[keep] = True
    return out


def attention(q: np.ndarray, q_rows: np.ndarray, k: np.ndarray, v: np.ndarray,
              req: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Causal grouped-query attention of selected query rows over the full fused
    cache (CacheBlend walkthrough, "Selective KV recompute": only the selected rows
    of the attention matrix are computed, each row complete over every earlier token
    of its request). q [nq, nh, d] for rows q_rows; k, v [T, nkv, d]. Head h reads
    KV head floor(h * nkv / nh); scale 1/sqrt(d); key i is visible to query j when
    both lie in one request and pos_i <= pos_j."""
    nq, nh, d = q.shape
    nkv = k.shape[1]
    out = np.zeros((nq, nh, d), np.float64)
    for r in np.unique(req[q_rows]) if nq else []:
        qsel = np.nonzero(req[q_rows] == r)[0]
        keys = np.nonzero(req == r)[0]
        visible = positions[keys][None, :] <= positions[q_rows[qsel]][:, None]
        for h in range(nh):
            g = (h * nkv) // nh
            s = (q[qsel, h, :] @ k[keys, g, :].T) / np.sqrt(d)
            s = np.where(visible, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[qsel, h, :] = p @ v[keys, g, :]
    return out


def residual_rmsnorm(x: np.ndarray, o: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """Chain step between stacked layers: RMSNorm(x + o) with unit weight (the
    reading taken for the multi-layer workload; the pages give no block internals)."""
    y = x + o
    return y / np.sqrt((y * y).mean(axis=1, keepdims=True) + eps)


# --------------------------------------------------------------------------- #
# one fused layer
# --------------------------------------------------------------------------- #


def _score_selection(score_r: np.ndarray, c_r: np.ndarray, n_ctx: int, ratio: float,
                     k_rule: str, window: int, tau: int, span_max: int, tau_smooth: float,
                     tau_cover: float, cap_ratio: float):
    """Selection of one request's candidates c_r (ascending rows) from external token
    scores score_r (SpecCache notes 2.2-2.3; CacheClip paper 4.2-4.3 for the scores
    with window grouping): T_init = the top K by score, then optional window grouping
    or span completion over the candidate sequence, then the optional budget cap.
    Returns (T_init rows, selected rows)."""
    k = topk_count(ratio, n_ctx, len(c_r), k_rule)
    s0 = topk_rows(score_r, c_r, k)
    if span_max > 0:
        init = np.isin(c_r, s0)
        chosen = complete_spans(score_r, init, tau_smooth, span_max, tau_cover)
        if cap_ratio > 0:
            chosen = budget_cap(score_r, chosen, topk_count(cap_ratio, n_ctx, len(c_r), k_rule))
        return s0, c_r[chosen]
    if window > 0:
        slot = {int(j): i for i, j in enumerate(c_r)}
        kept = group_windows([slot[int(j)] for j in s0], len(c_r), window, tau)
        return s0, (c_r[np.asarray(kept, np.int64)] if kept else np.zeros(0, np.int64))
    return s0, s0


def fuse_layer(*, hidden, w_qkv, k_cache, v_cache, req_offsets, chunk_offsets,
               chunk_src_pos, positions, n_heads, n_kv, head_dim, rope_base,
               ratio, mode: str = "topk", window: int = 0, tau: int = 0,
               dev_mode: str = "kv", cand: Optional[np.ndarray] = None,
               sel_override: Optional[np.ndarray] = None,
               attn_sample: Optional[np.ndarray] = None, k_rule: str = "round",
               scores: Optional[np.ndarray] = None, span_max: int = 0,
               tau_smooth: float = 0.4, tau_cover: float = 0.7, cap_ratio: float = 0.0,
               fresh_all: bool = False) -> Dict[str, np.ndarray]:
    """One selective-recompute layer, all float64 (CacheBlend walkthrough,
    "Selective KV recompute" and "Implementation"; CacheClip paper 4.1-4.3; SpecCache
    notes 2.1-2.3).

    Inputs are float64 arrays (already widened from storage). cand = candidate rows
    (None = every cached row). mode "topk" scores candidates by KV deviation and keeps
    the top k per request (k from ratio * N_ctx by k_rule); mode "given" keeps the
    candidates as they are; mode "scores" ranks the candidates by the caller's
    per-row scores instead (no deviation is needed to choose, so only the selected
    rows are recomputed), with window grouping or span completion (span_max > 0,
    tau_smooth, tau_cover, cap_ratio = budget as a ratio of N_ctx, 0 = none).
    fresh_all: every recomputed row takes its fresh K/V, not only the selected ones
    (CacheBlend walkthrough, "The chicken-and-egg problem": the figure of gradual
    filtering shows every candidate of a layer recomputed). sel_override replaces
    the selected set (used to compare downstream stages on another implementation's
    selection). Returns the selected rows (ascending, fresh rows included),
    per-request offsets, the fused caches, the attention output rows and the per-row
    deviation (NaN where not scored; in mode "scores", the deviation of the
    recomputed cached rows)."""
    T = hidden.shape[0]
    d = head_dim
    if (window > 0 or span_max > 0) and cand is not None:
        raise ValueError("grouping scans the whole cached sequence: cand must be None")
    req, src = row_layout(req_offsets, chunk_offsets, chunk_src_pos, T)
    cached = src >= 0
    fresh = ~cached
    pos = np.asarray(positions, np.int64)
    n_req = len(req_offsets) - 1

    # 1. positional recovery of every cached key
    k_tilde = rerotate(k_cache, pos, src, rope_base)

    # 2. candidate set C
    if cand is None:
        is_cand = cached.copy()
    else:
        is_cand = np.zeros(T, bool)
        is_cand[np.asarray(cand, np.int64)] = True
        is_cand &= cached

    # 2b. with external scores the selection comes first; C shrinks to it
    sel_parts = []
    s0_parts = []
    kth = []
    if mode == "scores":
        score = np.asarray(scores, np.float64)
        for r in range(n_req):
            rows_r = np.arange(req_offsets[r], req_offsets[r + 1])
            c_r = rows_r[is_cand[rows_r]]
            n_ctx = int(cached[rows_r].sum())
            s0, s = _score_selection(score[c_r], c_r, n_ctx, ratio, k_rule, window, tau,
                                     span_max, tau_smooth, tau_cover, cap_ratio)
            s0_parts.append(s0)
            kth.append(score[s0].min() if len(s0) else np.nan)
            sel_parts.append(np.union1d(s, rows_r[fresh[rows_r]]))
        is_cand = np.zeros(T, bool)
        for s in sel_parts:
            is_cand[s] = True
        is_cand &= cached

    # 2c. the rows recomputed: C plus fresh rows
    rec = np.nonzero(is_cand | fresh)[0]
    kf, vf = project_kv(hidden[rec], w_qkv, n_heads, n_kv, d)
    kf = rope(kf, pos[rec], rope_base)
    k_new = np.zeros_like(k_cache)
    v_new = np.zeros_like(v_cache)
    k_new[rec], v_new[rec] = kf, vf

    # 3. deviation of every candidate
    dev = np.full(T, np.nan)
    ci = np.nonzero(is_cand)[0]
    if len(ci):
        dev[ci] = kv_deviation(k_new[ci], v_new[ci], k_tilde[ci], v_cache[ci], dev_mode)

    # 4. selection per request
    if mode != "scores":
        for r in range(n_req):
            rows_r = np.arange(req_offsets[r], req_offsets[r + 1])
            c_r = rows_r[is_cand[rows_r]]
            n_ctx = int(cached[rows_r].sum())
            if mode == "given":
                s0 = c_r
                kth.append(np.nan)
            elif mode == "topk":
                k = topk_count(ratio, n_ctx, len(c_r), k_rule)
                s0 = topk_rows(dev[c_r], c_r, k)
                kth.append(dev[s0].min() if len(s0) else np.nan)
            else:
                raise ValueError(mode)
            s0_parts.append(s0)
            if window > 0:
                seq = rows_r[cached[rows_r]]  # the request's cached tokens, in order
                slot = {int(j): i for i, j in enumerate(seq)}
                kept = group_windows([slot[int(j)] for j in s0], len(seq), window, tau)
                s = seq[np.asarray(kept, np.int64)] if kept else np.zeros(0, np.int64)
            else:
                s = s0
            sel_parts.append(np.union1d(s, rows_r[fresh[rows_r]]))
    if sel_override is not None:
        sel = np.asarray(sel_override, np.int64)
    else:
        sel = np.concatenate(sel_parts) if sel_parts else np.zeros(0, np.int64)
    sel_offsets = np.zeros(len(req_offsets), np.int64)
    for r in range(n_req):
        sel_offsets[r + 1] = sel_offsets[r] + int(np.sum(req[sel] == r))

    # 5. expand: selected rows (every recomputed row with fresh_all) take their
    #    recomputed K/V, the rest keep the cache
    if sel_override is not None:
        missing = np.setdiff1d(sel, rec)
        if len(missing):  # an override may name rows that were not recomputed
            km, vm = project_kv(hidden[missing], w_qkv, n_heads, n_kv, d)
            k_new[missing], v_new[missing] = rope(km, pos[missing], rope_base), vm
    k_out = k_tilde.copy()
    v_out = v_cache.copy()
    upd = np.union1d(sel, rec) if fresh_all else sel
    k_out[upd] = k_new[upd]
    v_out[upd] = v_new[upd]

    # 6. queries of the selected rows and their attention over the fused cache
    #    (attn_sample: positions into the selection whose rows are evaluated;
    #    the others are left NaN -- a cost cut for large tests)
    if attn_sample is None:
        q = project_q(hidden[sel], w_qkv, n_heads, n_kv, d)
        q = rope(q, pos[sel], rope_base)
        attn = attention(q, sel, k_out, v_out, req, pos)
    else:
        idx = np.asarray(attn_sample, np.int64)
        q = project_q(hidden[sel[idx]], w_qkv, n_heads, n_kv, d)
        q = rope(q, pos[sel[idx]], rope_base)
        attn = np.full((len(sel), n_heads, d), np.nan)
        attn[idx] = attention(q, sel[idx], k_out, v_out, req, pos)

    return dict(sel_idx=sel, sel_offsets=sel_offsets, k_cache=k_out, v_cache=v_out,
                attn_out=attn, dev=dev, s0=(np.concatenate(s0_parts) if s0_parts
                                            else np.zeros(0, np.int64)),
                kth=np.asarray(kth), k_tilde=k_tilde, q=q)


def fuse_stack(*, hidden, layers: Sequence[dict], req_offsets, chunk_offsets,
               chunk_src_pos, positions, n_heads, n_kv, head_dim, rope_base,
               ratios: Sequence[float], window: int = 0, tau: int = 0,
               dev_mode: str = "kv", rms_eps: float = 1e-6,
               round_hidden=None, k_rule: str = "round", fresh_all: bool = False,
               first_kw: Optional[dict] = None,
               modes: Optional[Sequence[str]] = None) -> List[Dict[str, np.ndarray]]:
    """Gradual filtering across stacked layers (CacheBlend walkthrough, "The
    chicken-and-egg problem": layer 1 scores every token, each later layer scores
    only the previous layer's selection, so the set only shrinks; the fusor is
    sequential, "The system"). layers[l] = dict(w_qkv, k_cache, v_cache) in float64.
    Between layers x[j] <- RMSNorm(x[j] + o[j]) on the selected rows; rows outside
    the selection are not read again. round_hidden, if given, is applied to the new
    hidden rows (the storage rounding of a bf16 model's hidden state). k_rule and
    fresh_all apply to every layer; first_kw holds further selection settings of
    layer 1 only (e.g. mode "scores" with its scores and span settings). modes[l]
    for l >= 1 is the layer's check flag (CacheBlend walkthrough, "Implementation":
    a layer either checks, "topk", or reuses the indices it is handed, "given");
    None = every layer checks."""
    x = hidden.copy()
    outs = []
    cand = None
    for l, lw in enumerate(layers):
        o = fuse_layer(hidden=x, w_qkv=lw["w_qkv"], k_cache=lw["k_cache"],
                       v_cache=lw["v_cache"], req_offsets=req_offsets,
                       chunk_offsets=chunk_offsets, chunk_src_pos=chunk_src_pos,
                       positions=positions, n_heads=n_heads, n_kv=n_kv,
                       head_dim=head_dim, rope_base=rope_base, ratio=ratios[l],
                       **dict(dict(mode="topk" if l == 0 or modes is None else modes[l],
                                   window=window if l == 0 else 0, tau=tau,
                                   dev_mode=dev_mode, cand=cand, k_rule=k_rule,
                                   fresh_all=fresh_all),
                              **((first_kw or {}) if l == 0 else {})))
        o["hidden_in"] = x.copy()
        sel = o["sel_idx"]
        y = residual_rmsnorm(x[sel], o["attn_out"].reshape(len(sel), -1), rms_eps)
        if round_hidden is not None:
            y = round_hidden(y)
        x[sel] = y
        outs.append(o)
        _, src = row_layout(req_offsets, chunk_offsets, chunk_src_pos, x.shape[0])
        cand = sel[src[sel] >= 0]
    return outs


def controller_ratio(full_layer_ms: float, load_ms: float, r_floor: float = 0.15) -> float:
    """Recompute ratio of the loading controller (CacheBlend walkthrough, "Making the
    recompute free"): the recompute delay of ratio r is r times the profiled full
    prefill of the layer, the load delay is the layer's KV bytes over the measured
    load throughput; the ratio that makes the two equal, raised to the quality floor
    r* (15% on the page) and capped at 1 (everything recomputed)."""
    r_equal = load_ms / full_layer_ms
    return float(min(max(r_equal, r_floor), 1.0))


def load_ms(kv_bytes: float, gbps: float) -> float:
    """Load delay in ms: bytes over throughput (GB/s = 1e9 bytes/s)."""
    return kv_bytes / (gbps * 1e9) * 1e3


def full_prefill_layer(*, hidden, w_qkv, req_offsets, positions, n_heads, n_kv,
                       head_dim, rope_base):
    """Reference layer with nothing reused: Q/K/V of every row at its global
    position, causal attention of every row (the CacheBlend walkthrough's full
    recompute, the quality reference)."""
    T = hidden.shape[0]
    req = np.zeros(T, np.int64)
    for r in range(len(req_offsets) - 1):
        req[req_offsets[r]:req_offsets[r + 1]] = r
    pos = np.asarray(positions, np.int64)
    q, k, v = project(hidden, w_qkv, n_heads, n_kv, head_dim)
    q, k = rope(q, pos, rope_base), rope(k, pos, rope_base)
    rows = np.arange(T)
    return dict(q=q, k=k, v=v, attn_out=attention(q, rows, k, v, req, pos))
