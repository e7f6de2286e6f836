"""Attention under AKV visibility, naive float64.  (Oracle: test infrastructure only.)

Attention itself is the textbook definition: for query i, head h,
    o[i,h] = sum_j softmax_j( <q_ih, k_jg> * scale ) v_jg,   g = h // (Hq/Hkv),
with q and k RoPE-rotated to their positions; scale = 1/sqrt(d) unless given.

Three forms of the same result:
  attention_replay   token by token over replay_tokens' visible lists:
                     [P1] "three cache operations" (§3.3) -- append computes
                     the new token against the current active cache.
  segment_attention  one batched pass per repos stretch with an explicit
                     boolean mask: [P1] "single-prefill restore with
                     segment-batch attention" (§4.2, App. A.1.1, Fig. 10) --
                     queries are cut at drop/repos points into segments; each
                     segment attends causally to its own tokens and to the
                     active cache earlier segments left; a dropped entry stays
                     visible to the segments that used it and is hidden from
                     later ones; with repos, per-stretch key versions are
                     built by key rotation and value copy.
                     The mask is vis(i, j) = j <= i < D_j, with D_j the
                     boundary at which j was dropped; the key j is used at the
                     position it holds in the stretch of query i.
  decode             one query per request over a gathered key list: [P1]
                     "serving flow" / Fig. 12 (App. A.4.1) -- decode reads only
                     the active cache.
Also `repos` (batched key re-rotation, [P1] §3.3 / §4.2 A.1.2: rotation only,
values untouched) and `decode_after_ops` (decode continuing a replayed state).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .replay import replay_tokens, replay_events
from .rope import rope, rotate, HALF


def _softmax_attend(qh, kk, vv, scale, mask=None):
    """qh [n, d], kk [m, d], vv [m, d] -> (o [n, d], lse [n]) in float64.
    Rows whose mask is all False give NaN (no key to attend to)."""
    s = (qh @ kk.T) * scale
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    z = p.sum(axis=1, keepdims=True)
    o = (p @ vv) / z
    lse = (m + np.log(z))[:, 0]
    return o, lse


def attention_replay(q_raw, k_raw, v, ops, base=150000.0, layout=HALF, scale=None):
    """Literal token-by-token definition.  Inputs [T, H, d] (any float dtype).
    Returns (o [T, Hq, d], lse [T, Hq]) in float64.  Tiny inputs only."""
    q_raw = np.asarray(q_raw, np.float64)
    k_raw = np.asarray(k_raw, np.float64)
    v = np.asarray(v, np.float64)
    T, hq, d = q_raw.shape
    hkv = k_raw.shape[1]
    grp = hq // hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    records, _ = replay_tokens(ops)
    o = np.empty((T, hq, d))
    lse = np.empty((T, hq))
    for i, (pi, vis) in enumerate(records):
        js = np.asarray([j for j, _ in vis])
        ps = np.asarray([p for _, p in vis])
        qi = rope(q_raw[i], np.full(hq, pi), base, layout)            # [hq, d]
        kr = rope(k_raw[js], ps, base, layout)                        # [n, hkv, d]
        for h in range(hq):
            g = h // grp
            oo, ll = _softmax_attend(qi[h:h + 1], kr[:, g], v[js, g], scale)
            o[i, h], lse[i, h] = oo[0], ll[0]
    return o, lse


def visibility_mask(ev, e):
    """Explicit boolean mask of repos stretch e: rows = its own tokens,
    columns = [version rows] ++ [own tokens].  Returns (mask, key_tok, key_pos)."""
    tb, te, src = ev.epochs[e]
    own = np.arange(tb, te)
    key_tok = np.concatenate([src, own])
    key_pos = np.concatenate([np.arange(src.size), ev.tok_pos[own]])
    key_drop = ev.tok_drop[key_tok]
    i = own[:, None]
    mask = (key_tok[None, :] <= i) & (i < key_drop[None, :])
    return mask, key_tok, key_pos


def _pool_map(fn, items, threads):
    """fn over items, on a thread pool when threads > 1 (numpy releases the GIL in
    its array kernels); results in item order."""
    items = list(items)
    if threads <= 1 or len(items) <= 1:
        return [fn(x) for x in items]
    with ThreadPoolExecutor(max_workers=min(threads, len(items))) as ex:
        return list(ex.map(fn, items))


def segment_attention(q_raw, k_raw, v, ops=None, ev=None, base=150000.0, layout=HALF,
                      scale=None, rows=None, chunk=64, compact=False, threads=1):
    """Batched (restore-prefill) definition with an explicit mask per stretch.

    rows: optional sorted array of query token indices to compute (others are
    left NaN).  Returns (o [T, Hq, d], lse [T, Hq]) float64, or with compact=True
    only the requested rows, (o [len(rows), Hq, d], lse [len(rows), Hq]).
    threads > 1 spreads the independent (query chunk, head) products and the key
    rotation of each stretch (in blocks of rows) over a thread pool; every element
    is computed exactly as in the single-threaded walk."""
    if ev is None:
        ev = replay_events(ops)
    T, hq, d = q_raw.shape
    hkv = k_raw.shape[1]
    grp = hq // hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    if rows is None:
        rows = np.arange(T)
        compact = False
    rows = np.asarray(rows, np.int64)
    slot = np.full(T, -1, np.int64)           # output row of each requested token
    slot[rows] = np.arange(rows.size) if compact else rows
    n_out = rows.size if compact else T
    o = np.full((n_out, hq, d), np.nan)
    lse = np.full((n_out, hq), np.nan)
    want = slot >= 0
    kblk = 8192
    for e, (tb, te, src) in enumerate(ev.epochs):
        qrows = np.nonzero(want[tb:te])[0] + tb
        if qrows.size == 0:
            continue
        own = np.arange(tb, te)
        key_tok = np.concatenate([src, own])
        key_pos = np.concatenate([np.arange(src.size), ev.tok_pos[own]])
        key_drop = ev.tok_drop[key_tok]
        parts = _pool_map(lambda a: rope(np.asarray(k_raw[key_tok[a:a + kblk]], np.float64),
                                         key_pos[a:a + kblk], base, layout),
                          range(0, key_tok.size, kblk), threads)
        kr = np.concatenate(parts)                                     # [m, hkv, d]
        vv = np.asarray(v[key_tok], np.float64)
        for c0 in range(0, qrows.size, chunk):
            qi = qrows[c0:c0 + chunk]
            qr = rope(np.asarray(q_raw[qi], np.float64), ev.tok_pos[qi], base, layout)  # [n, hq, d]
            mask = (key_tok[None, :] <= qi[:, None]) & (qi[:, None] < key_drop[None, :])

            def one_head(h):
                g = h // grp
                return _softmax_attend(qr[:, h], kr[:, g], vv[:, g], scale, mask)

            for h, (oo, ll) in enumerate(_pool_map(one_head, range(hq), threads)):
                o[slot[qi], h] = oo
                lse[slot[qi], h] = ll
    return o, lse


def decode(q, k_rows, v_rows, indptr, scale=None):
    """One query token per request.  q [B, Hq, d] (already at its position),
    k_rows/v_rows [sum n, Hkv, d] = the gathered keys/values of each request in
    order, indptr [B+1].  Returns (o [B, Hq, d], lse [B, Hq]) float64."""
    q = np.asarray(q, np.float64)
    B, hq, d = q.shape
    hkv = k_rows.shape[1]
    grp = hq // hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    o = np.empty((B, hq, d))
    lse = np.empty((B, hq))
    for b in range(B):
        kk = np.asarray(k_rows[indptr[b]:indptr[b + 1]], np.float64)
        vv = np.asarray(v_rows[indptr[b]:indptr[b + 1]], np.float64)
        for g in range(hkv):
            oo, ll = _softmax_attend(q[b, g * grp:(g + 1) * grp], kk[:, g], vv[:, g], scale)
            o[b, g * grp:(g + 1) * grp] = oo
            lse[b, g * grp:(g + 1) * grp] = ll
    return o, lse


def decode_after_ops(q_new, k_new, v_new, k_raw, v, ops, base=150000.0, layout=HALF, scale=None):
    """Decode of one new token after the op sequence: the raw query/key of the
    new token are placed at p_next; it attends to the final active cache at
    its final positions plus its own KV."""
    _, (act, pos, p_next) = replay_tokens(ops)
    act = np.asarray(act, np.int64)
    kk = np.concatenate([rope(np.asarray(k_raw, np.float64)[act], np.asarray(pos), base, layout),
                         rope(np.asarray(k_new, np.float64)[None], [p_next], base, layout)])
    vv = np.concatenate([np.asarray(v, np.float64)[act], np.asarray(v_new, np.float64)[None]])
    qq = rope(np.asarray(q_new, np.float64), np.full(q_new.shape[0], p_next), base, layout)
    return decode(qq[None], kk, vv, np.array([0, kk.shape[0]]), scale)


def repos(k_rows, pos_from, pos_to, base=150000.0, layout=HALF):
    """Batched repos: key n (already at position pos_from[n]) moves to
    pos_to[n].  Values are not touched.  Returns float64 [n, H, d]."""
    return rotate(np.asarray(k_rows, np.float64), pos_from, pos_to, base, layout)
