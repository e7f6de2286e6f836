"""Python binding of libakv (ctypes).  Argument marshalling only.

Every computation runs in libakv.so (host plan compiler + HIP kernels for
gfx950).  This module checks tensor shapes/dtypes/devices, passes raw
pointers and the current HIP stream, and raises AkvError on a non-zero status.
There is no fallback: if the library is missing, importing this module fails.

Names mirror the C entry points in include/akv.h.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional, Sequence

import numpy as np
# torch ships its own HIP runtime under the same soname as the system one.  Loading
# it first makes libakv.so bind to that copy; loading libakv.so first would map a
# second HIP runtime, whose launches then find no device for torch's allocations.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("AKV_LIB", os.path.join(_HERE, "libakv.so"))
if not os.path.exists(LIB_PATH):
    raise ImportError(f"libakv.so not found at {LIB_PATH}: build it with "
                      "`python -m segmented_attention_seq_amd.build` (no CPU fallback exists)")
_lib = C.CDLL(LIB_PATH)

OK, EINVAL, EOPSEQ, EUNSUPPORTED, EHIP, ENOMEM, ENOSPACE = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1
ROPE_HALF, ROPE_INTERLEAVED = 0, 1
OP_APPEND, OP_DROP, OP_REPOS = 0, 1, 2
TILE_PARTIAL, TILE_FULL = 1, 2


class AkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.akv_last_error().decode()
        super().__init__(f"{where}: {_lib.akv_status_string(status).decode()} ({status}): {msg}")


class akv_op(C.Structure):
    _fields_ = [("kind", C.c_int32), ("reserved", C.c_int32), ("a", C.c_int64), ("b", C.c_int64)]


class akv_plan_info(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("n_tokens", "n_segments", "n_epochs", "n_versions",
                                          "n_items", "n_tiles", "n_full", "n_partial",
                                          "visible_pairs", "n_final", "p_next")] + \
               [("bq", C.c_int32), ("bk", C.c_int32), ("device_bytes", C.c_uint64), ("n_runs", C.c_int64)]


_P32 = C.POINTER(C.c_int32)


class akv_cache_match_info(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("n_tokens", "n_matched", "n_resident", "restore_from",
                                         "n_final", "p_next")]


class akv_cache_stats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("n_slots", "n_free", "n_resident", "n_locked", "n_nodes",
                                         "n_tree_tokens", "n_marks", "n_frontier")]


class akv_plan_tables(C.Structure):
    _fields_ = [(n, _P32) for n in ("tok_pos", "tok_drop", "segments", "epochs", "versions",
                                     "items", "tile_ptr", "tiles", "item_order", "final_tok",
                                     "final_pos", "ver_run", "run_delta")]


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_vp, _i32, _i64, _u64, _f32, _f64 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint64, C.c_float, C.c_double
_sig("akv_status_string", C.c_char_p, C.c_int)
_sig("akv_last_error", C.c_char_p)
_sig("akv_version", C.c_char_p)
_sig("akv_ops_from_messages", C.c_int, _i32, _vp, _i32, _vp, _vp, _i32, _vp, C.POINTER(akv_op), _i64,
     C.POINTER(_i64))
_sig("akv_build_visibility", C.c_int, C.POINTER(akv_op), _i64, _i32, _i32, C.POINTER(_vp))
_sig("akv_plan_info_get", C.c_int, _vp, C.POINTER(akv_plan_info))
_sig("akv_plan_tables_get", C.c_int, _vp, C.POINTER(akv_plan_tables))
_sig("akv_plan_upload", C.c_int, _vp, _vp, _u64, _vp)
_sig("akv_plan_destroy", None, _vp)
_sig("akv_rope_repos", C.c_int, _vp, _vp, C.c_int, _i64, _i32, _i32, _vp, _vp, _vp, _f64, C.c_int, _vp)
_sig("akv_kv_reuse", C.c_int, _vp, _vp, _vp, _vp, C.c_int, _i64, _i32, _i32, _vp, _vp, _vp, _f64, C.c_int, _vp)
_sig("akv_rope_apply", C.c_int, _vp, _vp, _vp, _vp, C.c_int, _i32, _i32, _f64, C.c_int, _vp)
_sig("akv_build_kv_versions", C.c_int, _vp, _vp, _vp, _vp, _vp, _vp, C.c_int, _i32, _i32, _f64, C.c_int, _vp)
_sig("akv_segment_attention", C.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, C.c_int, _i32, _i32,
     _i32, _f32, _vp)
_sig("akv_segment_attention_rope", C.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, C.c_int, _i32, _i32,
     _i32, _f32, _f64, C.c_int, _vp)
_sig("akv_decode_workspace_bytes", _u64, _i32, _i32, _i32, _i32, _i64)
_sig("akv_decode_attention", C.c_int, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _f32, C.c_int,
     _vp, _vp, _vp, _u64, _vp)
_sig("akv_rot_table_bytes", C.c_uint64, _vp, _i32)
_sig("akv_segment_attention_fused", C.c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, C.c_int, _i32, _i32, _i32, _f32,
     C.c_double, C.c_int, _vp, _u64, _vp)
_sig("akv_decode_attention_noalloc", C.c_int, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _f32, C.c_int,
     _vp, _vp, _vp)
_sig("akv_cache_create", C.c_int, _i32, C.POINTER(_vp))
_sig("akv_cache_destroy", None, _vp)
_sig("akv_cache_match", C.c_int, _vp, _vp, _i64, _vp, _i64, _i32, _vp, _vp, C.POINTER(akv_cache_match_info))
_sig("akv_cache_alloc", C.c_int, _vp, _i32, _vp)
_sig("akv_cache_insert", C.c_int, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i64)
_sig("akv_cache_unlock", C.c_int, _vp, _vp, _i64)
_sig("akv_cache_stats_get", C.c_int, _vp, C.POINTER(akv_cache_stats))
_sig("akv_attention_bq", _i32, _i32, _i32)

EXPORTED = ["akv_status_string", "akv_last_error", "akv_version", "akv_ops_from_messages",
            "akv_build_visibility", "akv_plan_info_get", "akv_plan_tables_get", "akv_plan_upload",
            "akv_plan_destroy", "akv_rope_repos", "akv_kv_reuse", "akv_rope_apply", "akv_build_kv_versions",
            "akv_segment_attention", "akv_segment_attention_rope", "akv_decode_workspace_bytes", "akv_decode_attention",
            "akv_decode_attention_noalloc", "akv_rot_table_bytes", "akv_segment_attention_fused",
            "akv_cache_create", "akv_cache_destroy", "akv_cache_match", "akv_cache_alloc",
            "akv_cache_insert", "akv_cache_unlock", "akv_cache_stats_get", "akv_attention_bq"]


def _check(status: int, where: str):
    if status != OK:
        raise AkvError(status, where)


def version() -> str:
    return _lib.akv_version().decode()


def lib_path() -> str:
    return LIB_PATH


# ---------------------------------------------------------------- A1: host plan

def ops_from_messages(msg_len: Sequence[int], drop: Optional[Dict[int, Sequence[int]]] = None,
                      reposition: Sequence[int] = ()) -> np.ndarray:
    """Operate-after request -> canonical op array (structured numpy, fields kind/a/b)."""
    ml = np.ascontiguousarray(msg_len, np.int32)
    pairs = [(int(k), int(j)) for k, js in (drop or {}).items() for j in js]
    da = np.ascontiguousarray([p[0] for p in pairs], np.int32)
    dt = np.ascontiguousarray([p[1] for p in pairs], np.int32)
    ra = np.ascontiguousarray(list(reposition), np.int32)
    n = _i64(0)
    args = (len(ml), ml.ctypes.data, len(pairs), da.ctypes.data, dt.ctypes.data, len(ra), ra.ctypes.data)
    _check(_lib.akv_ops_from_messages(*args, None, 0, C.byref(n)), "akv_ops_from_messages")
    ops = (akv_op * max(n.value, 1))()
    _check(_lib.akv_ops_from_messages(*args, ops, n.value, C.byref(n)), "akv_ops_from_messages")
    return np.ctypeslib.as_array(ops)[: n.value].copy()


def ops_array(ops) -> np.ndarray:
    """List of (kind, a[, b]) tuples -> akv_op structured array."""
    out = (akv_op * max(len(ops), 1))()
    for i, op in enumerate(ops):
        out[i].kind = op[0]
        out[i].a = op[1] if len(op) > 1 else 0
        out[i].b = op[2] if len(op) > 2 else 0
    return np.ctypeslib.as_array(out)[: len(ops)].copy()


def _ops_arg(ops):
    ops = ops if isinstance(ops, np.ndarray) else ops_array(ops)
    ops = np.ascontiguousarray(ops)
    return ops, (ops.ctypes.data if len(ops) else None), len(ops)


def _i32_arg(x):
    a = np.ascontiguousarray(x, np.int32)
    return a, (a.ctypes.data if a.size else None), a.size


class CacheIndex:
    """KV cache index (akv_cache_*): extended radix tree over token + op histories,
    position versions per token, drop-aware eviction over n_slots pool rows."""

    def __init__(self, n_slots: int):
        h = _vp()
        _check(_lib.akv_cache_create(int(n_slots), C.byref(h)), "akv_cache_create")
        self._h = h

    def __del__(self, _destroy=_lib.akv_cache_destroy):
        # the library function is bound at definition time: module globals may
        # already be cleared when this runs at interpreter exit
        if getattr(self, "_h", None):
            _destroy(self._h)
            self._h = None

    def match(self, tok, ops, lock: bool = False):
        """-> (slot int32[T], pos int32[T], info dict)."""
        tk, tp, n = _i32_arg(tok)
        ops, op_p, n_ops = _ops_arg(ops)
        slot = np.empty(n, np.int32)
        pos = np.empty(n, np.int32)
        info = akv_cache_match_info()
        _check(_lib.akv_cache_match(self._h, tp, n, op_p, n_ops, int(bool(lock)),
                                    slot.ctypes.data if n else None, pos.ctypes.data if n else None,
                                    C.byref(info)), "akv_cache_match")
        return slot, pos, {f: getattr(info, f) for f, _ in info._fields_}

    def alloc(self, n: int) -> np.ndarray:
        out = np.empty(max(int(n), 0), np.int32)
        _check(_lib.akv_cache_alloc(self._h, int(n), out.ctypes.data if out.size else None),
               "akv_cache_alloc")
        return out

    def insert(self, tok, ops, ver_token, ver_pos, ver_slot):
        tk, tp, n = _i32_arg(tok)
        ops, op_p, n_ops = _ops_arg(ops)
        vt, vtp, nv = _i32_arg(ver_token)
        vp, vpp, nv2 = _i32_arg(ver_pos)
        vs, vsp, nv3 = _i32_arg(ver_slot)
        if not nv == nv2 == nv3:
            raise ValueError("version arrays differ in length")
        _check(_lib.akv_cache_insert(self._h, tp, n, op_p, n_ops, vtp, vpp, vsp, nv), "akv_cache_insert")

    def unlock(self, slots):
        s, sp, n = _i32_arg(slots)
        _check(_lib.akv_cache_unlock(self._h, sp, n), "akv_cache_unlock")

    def stats(self) -> Dict[str, int]:
        st = akv_cache_stats()
        _check(_lib.akv_cache_stats_get(self._h, C.byref(st)), "akv_cache_stats_get")
        return {f: getattr(st, f) for f, _ in st._fields_}


class Plan:
    """Host restore plan (akv_build_visibility).  Immutable once built."""

    def __init__(self, ops: np.ndarray, bq: int = 64, bk: int = 64):
        ops = np.ascontiguousarray(ops)
        h = _vp()
        ptr = ops.ctypes.data_as(C.POINTER(akv_op)) if len(ops) else None
        _check(_lib.akv_build_visibility(ptr, len(ops), bq, bk, C.byref(h)), "akv_build_visibility")
        self._h = h
        info = akv_plan_info()
        _check(_lib.akv_plan_info_get(h, C.byref(info)), "akv_plan_info_get")
        self.info = {f: getattr(info, f) for f, _ in akv_plan_info._fields_}
        self._dev = {}

    @property
    def handle(self):
        return self._h

    def __del__(self, _destroy=_lib.akv_plan_destroy):
        # bound at definition time, as in CacheIndex.__del__
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            _destroy(h)
            self._h = None

    def tables(self) -> Dict[str, np.ndarray]:
        v = akv_plan_tables()
        _check(_lib.akv_plan_tables_get(self._h, C.byref(v)), "akv_plan_tables_get")
        i = self.info

        def arr(p, n, cols=None):
            if n == 0:
                return np.zeros((0,) if cols is None else (0, cols), np.int32)
            a = np.ctypeslib.as_array(p, shape=(n * (cols or 1),)).copy()
            return a if cols is None else a.reshape(n, cols)
        t = {
            "tok_pos": arr(v.tok_pos, i["n_tokens"]),
            "tok_drop": arr(v.tok_drop, i["n_tokens"]),
            "segments": arr(v.segments, i["n_segments"], 3),
            "epochs": arr(v.epochs, i["n_epochs"], 4),
            "versions": arr(v.versions, i["n_versions"], 3),
            "items": arr(v.items, i["n_items"], 2),
            "tile_ptr": arr(v.tile_ptr, i["n_items"] + 1),
            "tiles": arr(v.tiles, i["n_tiles"]),
            "item_order": arr(v.item_order, i["n_items"]),
            "final_tok": arr(v.final_tok, i["n_final"]),
            "final_pos": arr(v.final_pos, i["n_final"]),
            "ver_run": arr(v.ver_run, i["n_versions"]),
            "run_delta": arr(v.run_delta, i["n_runs"]),
        }
        return t

    def upload(self, device=None):
        """Copy the device image into a torch uint8 tensor on `device` (cached)."""
        import torch
        dev = torch.device(device if device is not None else "cuda")
        key = str(dev)
        if key not in self._dev:
            buf = torch.empty(max(int(self.info["device_bytes"]), 256), dtype=torch.uint8, device=dev)
            _check(_lib.akv_plan_upload(self._h, buf.data_ptr(), buf.numel(), _stream(dev)),
                   "akv_plan_upload")
            torch.cuda.current_stream(dev).synchronize()
            self._dev[key] = buf
        return self._dev[key]


def attention_bq(hq: int, hkv: int) -> int:
    """Plan query tile the bf16 attention runs fastest with (akv_attention_bq)."""
    return int(_lib.akv_attention_bq(hq, hkv))


def build_visibility(ops, bq: int = 64, bk: int = 64) -> Plan:
    if not isinstance(ops, np.ndarray):
        ops = ops_array(ops)
    return Plan(ops, bq, bk)


# ---------------------------------------------------------------- GPU entry points

def _stream(dev=None):
    import torch
    return C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _req(t, name, dtype=None, shape=None, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.data_ptr()


def rope_repos(out, inp, pos_to, pos_from=None, gather=None, base: float = 150000.0,
               layout: int = ROPE_HALF):
    """out[n] = R((pos_to[n] - pos_from[n]) theta) inp[gather[n] or n].
    inp [rows, H, d]; out [n, H, d]; index tensors int32 on the same device."""
    import torch
    n, H, d = out.shape
    dev = out.device
    _req(out, "out", inp.dtype, device=dev)
    _req(inp, "inp", device=dev)
    if inp.shape[1:] != out.shape[1:]:
        raise ValueError("inp/out head shapes differ")
    if gather is None and inp.shape[0] != n:
        raise ValueError("without gather, inp and out need the same row count")
    p_to = _req(pos_to, "pos_to", torch.int32, (n,), dev)
    p_from = _req(pos_from, "pos_from", torch.int32, (n,), dev) if pos_from is not None else None
    g = _req(gather, "gather", torch.int32, (n,), dev) if gather is not None else None
    _check(_lib.akv_rope_repos(out.data_ptr(), inp.data_ptr(), _dtype_code(out), n, H, d, g, p_from,
                               p_to, base, layout, _stream(dev)), "akv_rope_repos")
    return out


def kv_reuse(k_out, v_out, k_pool, v_pool, gather, pos_from, pos_to, base: float = 150000.0,
             layout: int = ROPE_HALF):
    """Reuse path: k_out[n] = R((pos_to[n] - pos_from[n]) theta) k_pool[gather[n]],
    v_out[n] = v_pool[gather[n]].  Pools [rows, H, d]; outputs [n, H, d]."""
    import torch
    n, H, d = k_out.shape
    dev = k_out.device
    _req(k_out, "k_out", k_pool.dtype, device=dev)
    _req(v_out, "v_out", k_pool.dtype, (n, H, d), dev)
    _req(k_pool, "k_pool", device=dev)
    _req(v_pool, "v_pool", k_pool.dtype, tuple(k_pool.shape), dev)
    if k_pool.shape[1:] != k_out.shape[1:]:
        raise ValueError("pool/output head shapes differ")
    g = _req(gather, "gather", torch.int32, (n,), dev)
    p_from = _req(pos_from, "pos_from", torch.int32, (n,), dev)
    p_to = _req(pos_to, "pos_to", torch.int32, (n,), dev)
    _check(_lib.akv_kv_reuse(k_out.data_ptr(), v_out.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                             _dtype_code(k_out), n, H, d, g, p_from, p_to, base, layout, _stream(dev)),
           "akv_kv_reuse")
    return k_out, v_out


def rope_apply(plan: Plan, out, inp, base: float = 150000.0, layout: int = ROPE_HALF):
    """Rotate raw [T, H, d] rows to their append positions (plan T1)."""
    T, H, d = inp.shape
    dev = inp.device
    if T != plan.info["n_tokens"]:
        raise ValueError("row count differs from the plan's token count")
    _req(inp, "inp", device=dev)
    _req(out, "out", inp.dtype, tuple(inp.shape), dev)
    _check(_lib.akv_rope_apply(plan.handle, plan.upload(dev).data_ptr(), out.data_ptr(), inp.data_ptr(),
                               _dtype_code(inp), H, d, base, layout, _stream(dev)), "akv_rope_apply")
    return out


def build_kv_versions(plan: Plan, k, v, k_ver, v_ver, base: float = 150000.0, layout: int = ROPE_HALF):
    T, H, d = k.shape
    dev = k.device
    nv = plan.info["n_versions"]
    _req(k, "k", device=dev)
    _req(v, "v", k.dtype, tuple(k.shape), dev)
    _req(k_ver, "k_ver", k.dtype, (nv, H, d), dev)
    _req(v_ver, "v_ver", k.dtype, (nv, H, d), dev)
    _check(_lib.akv_build_kv_versions(plan.handle, plan.upload(dev).data_ptr(), k.data_ptr(), v.data_ptr(),
                                      k_ver.data_ptr(), v_ver.data_ptr(), _dtype_code(k), H, d, base,
                                      layout, _stream(dev)), "akv_build_kv_versions")


def segment_attention(plan: Plan, q, k, v, k_ver, v_ver, out, lse=None, scale: float = 0.0,
                      rope_base: Optional[float] = None, layout: int = ROPE_HALF):
    """Segment attention (akv_segment_attention).  With rope_base set, q is raw and
    is rotated to its append positions inside the attention
    (akv_segment_attention_rope)."""
    import torch
    T, hq, d = q.shape
    hkv = k.shape[1]
    dev = q.device
    nv = plan.info["n_versions"]
    if T != plan.info["n_tokens"]:
        raise ValueError("token count differs from the plan")
    _req(q, "q", device=dev)
    _req(k, "k", q.dtype, (T, hkv, d), dev)
    _req(v, "v", q.dtype, (T, hkv, d), dev)
    kvp = vvp = None
    if nv:
        kvp = _req(k_ver, "k_ver", q.dtype, (nv, hkv, d), dev)
        vvp = _req(v_ver, "v_ver", q.dtype, (nv, hkv, d), dev)
    _req(out, "out", q.dtype, (T, hq, d), dev)
    lp = _req(lse, "lse", torch.float32, (T, hq), dev) if lse is not None else None
    if rope_base is None:
        _check(_lib.akv_segment_attention(plan.handle, plan.upload(dev).data_ptr(), q.data_ptr(), k.data_ptr(),
                                          v.data_ptr(), kvp, vvp, out.data_ptr(), lp, _dtype_code(q), hq, hkv,
                                          d, scale, _stream(dev)), "akv_segment_attention")
    else:
        _check(_lib.akv_segment_attention_rope(plan.handle, plan.upload(dev).data_ptr(), q.data_ptr(),
                                               k.data_ptr(), v.data_ptr(), kvp, vvp, out.data_ptr(), lp,
                                               _dtype_code(q), hq, hkv, d, scale, float(rope_base), layout,
                                               _stream(dev)), "akv_segment_attention_rope")
    return out


def rot_table_bytes(plan: Plan, d: int) -> int:
    return int(_lib.akv_rot_table_bytes(plan.handle, d))


def segment_attention_fused(plan: Plan, q_raw, k, v, out, lse=None, scale: float = 0.0,
                            rope_base: float = 150000.0, layout: int = ROPE_HALF, ws=None):
    """Segment attention with version rows rotated while key tiles are staged
    (akv_segment_attention_fused): raw queries, keys rotated to their append
    positions, values; no version buffers."""
    import torch
    T, hq, d = q_raw.shape
    hkv = k.shape[1]
    dev = q_raw.device
    if T != plan.info["n_tokens"]:
        raise ValueError("token count differs from the plan")
    _req(q_raw, "q_raw", device=dev)
    _req(k, "k", q_raw.dtype, (T, hkv, d), dev)
    _req(v, "v", q_raw.dtype, (T, hkv, d), dev)
    _req(out, "out", q_raw.dtype, (T, hq, d), dev)
    lp = _req(lse, "lse", torch.float32, (T, hq), dev) if lse is not None else None
    need = rot_table_bytes(plan, d)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    wp, wn = (None, 0) if ws is None else (_req(ws, "ws", device=dev), ws.numel() * ws.element_size())
    _check(_lib.akv_segment_attention_fused(plan.handle, plan.upload(dev).data_ptr(), q_raw.data_ptr(), k.data_ptr(),
                                            v.data_ptr(), out.data_ptr(), lp, _dtype_code(q_raw), hq, hkv, d,
                                            scale, float(rope_base), layout, wp, wn, _stream(dev)),
           "akv_segment_attention_fused")
    return out


def decode_workspace_bytes(batch: int, hq: int, hkv: int, d: int, max_n: int) -> int:
    return int(_lib.akv_decode_workspace_bytes(batch, hq, hkv, d, max_n))


def decode_attention(q, k_pool, v_pool, indptr, indices, max_n: int, out, lse=None, ws=None,
                     scale: float = 0.0):
    import torch
    B, hq, d = q.shape
    hkv = k_pool.shape[1]
    dev = q.device
    _req(q, "q", torch.bfloat16, device=dev)
    _req(k_pool, "k_pool", torch.bfloat16, device=dev)
    _req(v_pool, "v_pool", torch.bfloat16, tuple(k_pool.shape), dev)
    _req(indptr, "indptr", torch.int32, (B + 1,), dev)
    _req(indices, "indices", torch.int32, device=dev)
    _req(out, "out", torch.bfloat16, (B, hq, d), dev)
    lp = _req(lse, "lse", torch.float32, (B, hq), dev) if lse is not None else None
    need = decode_workspace_bytes(B, hq, hkv, d, max_n)
    if ws is None:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
    _req(ws, "ws", device=dev)
    nbytes = ws.numel() * ws.element_size()
    _check(_lib.akv_decode_attention(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), indptr.data_ptr(),
                                     indices.data_ptr(), B, hq, hkv, d, max_n, scale, BF16, out.data_ptr(),
                                     lp, ws.data_ptr(), nbytes, _stream(dev)), "akv_decode_attention")
    return out


def decode_attention_noalloc(q, k_pool, v_pool, indptr, indices, max_n: int, out, lse=None,
                             scale: float = 0.0):
    """decode_attention on the library's fixed per-device scratch (no workspace is
    allocated or passed); calls on one device must not overlap."""
    import torch
    B, hq, d = q.shape
    hkv = k_pool.shape[1]
    dev = q.device
    _req(q, "q", torch.bfloat16, device=dev)
    _req(k_pool, "k_pool", torch.bfloat16, device=dev)
    _req(v_pool, "v_pool", torch.bfloat16, tuple(k_pool.shape), dev)
    _req(indptr, "indptr", torch.int32, (B + 1,), dev)
    _req(indices, "indices", torch.int32, device=dev)
    _req(out, "out", torch.bfloat16, (B, hq, d), dev)
    lp = _req(lse, "lse", torch.float32, (B, hq), dev) if lse is not None else None
    _check(_lib.akv_decode_attention_noalloc(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), indptr.data_ptr(),
                                             indices.data_ptr(), B, hq, hkv, d, max_n, scale, BF16,
                                             out.data_ptr(), lp, _stream(dev)), "akv_decode_attention_noalloc")
    return out


def restore(plan: Plan, q_raw, k_raw, v, base: float = 150000.0, layout: int = ROPE_HALF,
            with_lse: bool = False, scale: float = 0.0, bufs: Optional[dict] = None, fuse_q: bool = True,
            fused_versions: bool = False):
    """Restore prefill: RoPE-apply K to its append positions, build the per-stretch
    KV versions, run segment attention, which rotates the raw queries as it loads
    them (fuse_q=False: RoPE-apply Q into a rotated copy first).  With
    fused_versions, no version buffers are built: the attention rotates version
    rows as it stages key tiles.  Returns (out, lse or None).  `bufs` may hold
    preallocated q_rot/k_rot/k_ver/v_ver/out/lse/rot_ws tensors."""
    import torch
    T, hq, d = q_raw.shape
    hkv = k_raw.shape[1]
    dev, dt = q_raw.device, q_raw.dtype
    nv = int(plan.info["n_versions"])
    b = {} if bufs is None else bufs
    if fused_versions:
        kr = b.get("k_rot")
        kr = torch.empty_like(k_raw) if kr is None else kr
        out = b.get("out")
        out = torch.empty_like(q_raw) if out is None else out
        lse = b.get("lse")
        if with_lse and lse is None:
            lse = torch.empty((T, hq), dtype=torch.float32, device=dev)
        rope_apply(plan, kr, k_raw, base, layout)
        segment_attention_fused(plan, q_raw, kr, v, out, lse if with_lse else None, scale, base, layout,
                                b.get("rot_ws"))
        return out, (lse if with_lse else None)
    qr = None
    if not fuse_q:
        qr = b.get("q_rot")
        qr = torch.empty_like(q_raw) if qr is None else qr
    kr = b.get("k_rot")
    kr = torch.empty_like(k_raw) if kr is None else kr
    kv = b.get("k_ver")
    kv = torch.empty((nv, hkv, d), dtype=dt, device=dev) if kv is None else kv
    vv = b.get("v_ver")
    vv = torch.empty((nv, hkv, d), dtype=dt, device=dev) if vv is None else vv
    out = b.get("out")
    out = torch.empty_like(q_raw) if out is None else out
    lse = b.get("lse")
    if with_lse and lse is None:
        lse = torch.empty((T, hq), dtype=torch.float32, device=dev)
    rope_apply(plan, kr, k_raw, base, layout)
    if nv:
        build_kv_versions(plan, kr, v, kv, vv, base, layout)
    if fuse_q:
        segment_attention(plan, q_raw, kr, v, kv, vv, out, lse if with_lse else None, scale, base, layout)
    else:
        rope_apply(plan, qr, q_raw, base, layout)
        segment_attention(plan, qr, kr, v, kv, vv, out, lse if with_lse else None, scale)
    return out, (lse if with_lse else None)
