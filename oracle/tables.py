"""Plan tables derived from the replay and the explicit mask.  (Oracle: test infrastructure only.)

These are the integer tables the GPU library's plan compiler must reproduce
bit for bit.  Here every one is read off the replay (replay_events) or off
the explicit boolean mask of each repos stretch, tile by tile.

  T1 tok_pos[T]        position of each token when appended ([P1] §3.3)
  T2 tok_drop[T]       boundary token index at which it was dropped, or INT32_MAX
  T3 segments          (begin, end, stretch) of each maximal run of tokens with
                       no drop/repos boundary inside ([P1] §4.2: queries are cut
                       at drop/repos points)
  T4 stretches         (tok_begin, tok_end, r, ver_offset) per repos stretch
                       that appends tokens
  T5 versions          (src token, from_pos = tok_pos[src], to_pos = v) for the
                       r keys active right after the stretch's repos ([P1] §4.2,
                       App. A.1.1: per-segment KV versions by key rotation and
                       value copy)
  T6 tile classes      per (stretch, q-tile): ascending non-empty k-tiles and
                       their class, FULL (every pair visible) or PARTIAL.  Query
                       tiles of bq tokens start at the stretch's first token; key
                       tiles of bk run over the version rows from 0, then restart
                       at the stretch's own tokens.  Key slots past the end of a
                       part count as not visible; query rows past the stretch's
                       end are ignored.
  T7 final             active tokens, their positions, p_next
"""
from __future__ import annotations

import numpy as np

from .replay import replay_events, NEVER

EMPTY, PARTIAL, FULL = 0, 1, 2


def _virtual_keys(ev, e, bk):
    """Key token / drop arrays of stretch e laid out on the tiled virtual axis:
    version part padded to a multiple of bk, then the own part padded likewise.
    Padding slots get token = drop = -1 (never visible)."""
    tb, te, src = ev.epochs[e]
    own = np.arange(tb, te)
    nvt = -(-src.size // bk)
    not_ = -(-own.size // bk)
    tok = np.full((nvt + not_) * bk, -1, np.int64)
    drp = np.full((nvt + not_) * bk, -1, np.int64)
    tok[:src.size] = src
    drp[:src.size] = ev.tok_drop[src]
    tok[nvt * bk:nvt * bk + own.size] = own
    drp[nvt * bk:nvt * bk + own.size] = ev.tok_drop[own]
    return tok, drp, nvt, not_


def _classify(mask_blocks):
    """mask_blocks [rows, ntiles, bk] -> class per tile."""
    anyv = mask_blocks.any(axis=(0, 2))
    allv = mask_blocks.all(axis=(0, 2))
    return np.where(allv, FULL, np.where(anyv, PARTIAL, EMPTY))


def tile_classes(ev, bq, bk):
    """Return (items [n,2] = (stretch, q-tile), ptr [n+1], k_tile [m], cls [m])."""
    items, ptr, kts, cls = [], [0], [], []
    for e, (tb, te, src) in enumerate(ev.epochs):
        tok, drp, nvt, not_ = _virtual_keys(ev, e, bk)
        valid = tok >= 0
        for qt in range(-(-(te - tb) // bq)):
            i = np.arange(tb + qt * bq, min(te, tb + (qt + 1) * bq))[:, None]
            mask = valid[None, :] & (tok[None, :] <= i) & (i < drp[None, :])
            c = _classify(mask.reshape(i.shape[0], nvt + not_, bk))
            nz = np.nonzero(c)[0]
            items.append((e, qt))
            kts.append(nz)
            cls.append(c[nz])
            ptr.append(ptr[-1] + nz.size)
    return (np.asarray(items, np.int64).reshape(-1, 2), np.asarray(ptr, np.int64),
            np.concatenate(kts) if kts else np.zeros(0, np.int64),
            np.concatenate(cls) if cls else np.zeros(0, np.int64))


def tile_class_of(ev, e, qt, kt, bq, bk):
    """Class of one tile, from the explicit mask (for spot checks on large plans)."""
    tb, te, src = ev.epochs[e]
    tok, drp, nvt, not_ = _virtual_keys(ev, e, bk)
    sl = slice(kt * bk, (kt + 1) * bk)
    t, dd = tok[sl], drp[sl]
    i = np.arange(tb + qt * bq, min(te, tb + (qt + 1) * bq))[:, None]
    mask = (t[None, :] >= 0) & (t[None, :] <= i) & (i < dd[None, :])
    return int(_classify(mask[:, None, :])[0])


def plan_tables(ops=None, ev=None, bq=64, bk=64, with_tiles=True):
    if ev is None:
        ev = replay_events(ops)
    T = ev.T
    cuts = sorted({0, T} | {b for b in ev.boundaries if 0 < b < T})
    ep_of = ev.epoch_of_token()
    segs = np.asarray([(a, b, ep_of[a]) for a, b in zip(cuts[:-1], cuts[1:]) if b > a],
                      np.int64).reshape(-1, 3)
    stretches, vers = [], []
    off = 0
    for (tb, te, src) in ev.epochs:
        stretches.append((tb, te, src.size, off))
        for v, j in enumerate(src):
            vers.append((j, ev.tok_pos[j], v))
        off += src.size
    out = {
        "tok_pos": ev.tok_pos.copy(),
        "tok_drop": np.minimum(ev.tok_drop, NEVER),
        "segments": segs,
        "epochs": np.asarray(stretches, np.int64).reshape(-1, 4),
        "versions": np.asarray(vers, np.int64).reshape(-1, 3),
        "final_tok": ev.final[0],
        "final_pos": ev.final[1],
        "p_next": ev.final[2],
        "visible_pairs": ev.visible_pairs,
    }
    if with_tiles:
        items, ptr, kt, cls = tile_classes(ev, bq, bk)
        out.update(items=items, tile_ptr=ptr, tile_k=kt, tile_cls=cls)
    return out
