"""Thin ctypes binding of liboasiskv (include/oasiskv.h), same names as the C ABI.

Argument marshalling only: torch tensors and numpy arrays become raw pointers,
streams become hipStream_t handles, a non-zero status becomes an OasisError
carrying the library's message.  Every step of the decode path runs in the HIP
library; if it is not built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liboasiskv.so")

OASIS_OK = 0
OASIS_EINVAL = -1
OASIS_EHIP = -2
OASIS_EUNSUPPORTED = -3
OASIS_F32 = 0
OASIS_BF16 = 1


class OasisError(RuntimeError):
    def __init__(self, func: str, code: int, msg: str):
        super().__init__(f"{func} failed ({code}): {msg}")
        self.code = code


class oasis_shape(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in (
        "batch", "kv_heads", "group", "head_dim", "block_size", "max_blocks",
        "budget_blocks", "n_draft", "fetch_cap", "dtype")]


class oasis_launch_options(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in (
        "attn_waves", "attn_pf", "attn_splits", "score_tpw", "step_order", "step_launches", "attn_merge")]


LAUNCH_OPTION_FIELDS = tuple(f for f, _ in oasis_launch_options._fields_)


class oasis_transfer(ctypes.Structure):
    _fields_ = [("host_tier", ctypes.c_void_p), ("pool", ctypes.c_void_p), ("fetch", ctypes.c_void_p),
                ("n_fetch", ctypes.c_void_p)]


class oasis_select_job(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("scores", "ctx_len", "sel", "block_to_slot", "slot_to_block", "fetch",
                                               "n_fetch", "evict", "attend", "n_attend")]


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_int = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes); status-returning functions use c_int.
SIGNATURES = {
    "oasis_create": (_int, [ctypes.POINTER(oasis_shape), ctypes.POINTER(_vp)]),
    "oasis_create_with_options": (_int, [ctypes.POINTER(oasis_shape), ctypes.POINTER(oasis_launch_options),
                                         ctypes.POINTER(_vp)]),
    "oasis_get_launch_options": (_int, [_vp, ctypes.POINTER(oasis_launch_options)]),
    "oasis_destroy": (_int, [_vp]),
    "oasis_last_error": (ctypes.c_char_p, []),
    "oasis_version": (_int, []),
    "oasis_page_bytes": (_sz, [_vp]),
    "oasis_meta_bytes": (_sz, [_vp]),
    "oasis_pool_bytes": (_sz, [_vp]),
    "oasis_host_tier_bytes": (_sz, [_vp]),
    "oasis_workspace_bytes": (_sz, [_vp]),
    "oasis_pack_pages": (_int, [_vp, _vp, _vp, _vp, _i32, _i32, _vp]),
    "oasis_host_tier_append": (_int, [_vp, _vp, _vp, _vp, _vp]),
    "oasis_block_meta_build": (_int, [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp]),
    "oasis_block_meta_update": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "oasis_block_meta_build_rows": (_int, [_vp, _vp, _i32, _i32, _vp, _vp, _vp]),
    "oasis_block_meta_export": (_int, [_vp, _vp, _vp, _vp]),
    "oasis_block_meta_import": (_int, [_vp, _vp, _vp, _vp]),
    "oasis_lookahead_score": (_int, [_vp, _vp, _vp, _vp, _vp, _vp]),
    "oasis_topk_select": (_int, [_vp, _vp, _vp, _vp, _vp]),
    "oasis_verify_score": (_int, [_vp, _vp, _vp, _vp, _vp, _vp]),
    "oasis_admit": (_int, [_vp] * 9),
    "oasis_resident_diff_cap_evict": (_int, [_vp] * 11),
    "oasis_select_and_diff": (_int, [_vp] * 12),
    "oasis_fetch_issue": (_int, [_vp, _vp, _vp, _vp, _vp, _vp]),
    "oasis_sparse_paged_decode_attn": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "oasis_decode_step": (_int, [_vp] * 18),
    "oasis_decode_step_gather": (_int, [_vp] * 17 + [ctypes.POINTER(oasis_transfer), _vp]),
    "oasis_decode_step_append": (_int, [_vp] * 20),
    "oasis_decode_step_carry": (_int, [_vp] * 11 + [ctypes.POINTER(oasis_select_job),
                                                     ctypes.POINTER(oasis_transfer), _vp]),
    "oasis_sparse_paged_decode_attn_list": (_int, [_vp] * 9),
    "oasis_sparse_paged_decode_attn_noalloc": (_int, [_vp] * 8),
    "oasis_attend_and_score": (_int, [_vp] * 14),
    "oasis_attn_combine": (_int, [_vp] * 4),
    "oasis_select_diff_combine": (_int, [_vp] * 14),
    "oasis_select_and_diff_lru": (_int, [_vp] * 7 + [_i32] + [_vp] * 6),
    "oasis_select_diff_combine_lru": (_int, [_vp] * 7 + [_i32] + [_vp] * 8),
    "oasis_fetch_gather": (_int, [_vp, _vp, _vp, _vp, _vp, _vp]),
}

_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m lookahead_sparse_kv_draft_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _ptr(x):
    """Raw address of a torch tensor / numpy array / int (None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(name: str, code: int):
    if code != OASIS_OK:
        msg = load().oasis_last_error().decode(errors="replace")
        raise OasisError(name, code, msg)


def _call(name: str, *args):
    code = getattr(load(), name)(*args)
    _check(name, code)


# ----------------------------------------------------------------- handle
def oasis_create(batch, kv_heads, group, head_dim, max_blocks, budget_blocks, n_draft, fetch_cap,
                 dtype, block_size=16) -> int:
    s = oasis_shape(batch=batch, kv_heads=kv_heads, group=group, head_dim=head_dim,
                    block_size=block_size, max_blocks=max_blocks, budget_blocks=budget_blocks,
                    n_draft=n_draft, fetch_cap=fetch_cap, dtype=dtype)
    h = _vp()
    _call("oasis_create", ctypes.byref(s), ctypes.byref(h))
    return h.value


def oasis_create_with_options(batch, kv_heads, group, head_dim, max_blocks, budget_blocks, n_draft, fetch_cap,
                              dtype, options=None, block_size=16) -> int:
    """options: a dict of oasis_launch_options fields (missing fields = 0, the default)."""
    s = oasis_shape(batch=batch, kv_heads=kv_heads, group=group, head_dim=head_dim,
                    block_size=block_size, max_blocks=max_blocks, budget_blocks=budget_blocks,
                    n_draft=n_draft, fetch_cap=fetch_cap, dtype=dtype)
    o = None
    if options is not None:
        unknown = set(options) - set(LAUNCH_OPTION_FIELDS)
        if unknown:
            raise ValueError(f"unknown launch options {sorted(unknown)}")
        o = oasis_launch_options(**{k: int(v) for k, v in options.items()})
    h = _vp()
    _call("oasis_create_with_options", ctypes.byref(s), None if o is None else ctypes.byref(o), ctypes.byref(h))
    return h.value


def oasis_get_launch_options(h) -> dict:
    o = oasis_launch_options()
    _call("oasis_get_launch_options", h, ctypes.byref(o))
    return {f: getattr(o, f) for f in LAUNCH_OPTION_FIELDS}


def oasis_destroy(h):
    _call("oasis_destroy", h)


def oasis_last_error() -> str:
    return load().oasis_last_error().decode(errors="replace")


def oasis_version() -> int:
    return load().oasis_version()


def oasis_page_bytes(h) -> int:
    return load().oasis_page_bytes(h)


def oasis_meta_bytes(h) -> int:
    return load().oasis_meta_bytes(h)


def oasis_pool_bytes(h) -> int:
    return load().oasis_pool_bytes(h)


def oasis_host_tier_bytes(h) -> int:
    return load().oasis_host_tier_bytes(h)


def oasis_workspace_bytes(h) -> int:
    return load().oasis_workspace_bytes(h)


# ----------------------------------------------------------------- host side
def oasis_pack_pages(h, k, v, blocks, n_blocks, unit, pages):
    _call("oasis_pack_pages", h, _ptr(k), _ptr(v), _ptr(blocks), n_blocks, unit, _ptr(pages))


def oasis_host_tier_append(h, k_new, v_new, pos, host_tier):
    _call("oasis_host_tier_append", h, _ptr(k_new), _ptr(v_new), _ptr(pos), _ptr(host_tier))


def oasis_fetch_gather(h, host_tier, pool, fetch, n_fetch, stream=None):
    _call("oasis_fetch_gather", h, _ptr(host_tier), _ptr(pool), _ptr(fetch), _ptr(n_fetch), _stream(stream))


def oasis_fetch_issue(h, host_tier, pool, fetch_host, n_fetch_host, stream=None):
    _call("oasis_fetch_issue", h, _ptr(host_tier), _ptr(pool), _ptr(fetch_host), _ptr(n_fetch_host),
          _stream(stream))


# ----------------------------------------------------------------- device side
def oasis_block_meta_build(h, pages, page_ids, count, ctx_len, meta, pool=None, block_to_slot=None,
                           stream=None):
    _call("oasis_block_meta_build", h, _ptr(pages), _ptr(page_ids), count, _ptr(ctx_len), _ptr(meta),
          _ptr(pool), _ptr(block_to_slot), _stream(stream))


def oasis_block_meta_build_rows(h, k_rows, tok_begin, tok_end, ctx_len, meta, stream=None):
    _call("oasis_block_meta_build_rows", h, _ptr(k_rows), tok_begin, tok_end, _ptr(ctx_len), _ptr(meta),
          _stream(stream))


def oasis_block_meta_export(h, meta, meta_logical, stream=None):
    _call("oasis_block_meta_export", h, _ptr(meta), _ptr(meta_logical), _stream(stream))


def oasis_block_meta_import(h, meta_logical, meta, stream=None):
    _call("oasis_block_meta_import", h, _ptr(meta_logical), _ptr(meta), _stream(stream))


def oasis_block_meta_update(h, k_new, v_new, ctx_len_in, ctx_len_out, meta, pool, block_to_slot,
                            stream=None):
    _call("oasis_block_meta_update", h, _ptr(k_new), _ptr(v_new), _ptr(ctx_len_in), _ptr(ctx_len_out),
          _ptr(meta), _ptr(pool), _ptr(block_to_slot), _stream(stream))


def oasis_lookahead_score(h, q, meta, ctx_len, scores, stream=None):
    _call("oasis_lookahead_score", h, _ptr(q), _ptr(meta), _ptr(ctx_len), _ptr(scores), _stream(stream))


def oasis_topk_select(h, scores, ctx_len, sel, stream=None):
    _call("oasis_topk_select", h, _ptr(scores), _ptr(ctx_len), _ptr(sel), _stream(stream))


def oasis_resident_diff_cap_evict(h, sel, scores, block_to_slot, slot_to_block, fetch, n_fetch, evict,
                                  attend=None, n_attend=None, stream=None):
    _call("oasis_resident_diff_cap_evict", h, _ptr(sel), _ptr(scores), _ptr(block_to_slot),
          _ptr(slot_to_block), _ptr(fetch), _ptr(n_fetch), _ptr(evict), _ptr(attend), _ptr(n_attend),
          _stream(stream))


def oasis_select_and_diff(h, scores, ctx_len, sel, block_to_slot, slot_to_block, fetch, n_fetch, evict,
                          attend=None, n_attend=None, stream=None):
    _call("oasis_select_and_diff", h, _ptr(scores), _ptr(ctx_len), _ptr(sel), _ptr(block_to_slot),
          _ptr(slot_to_block), _ptr(fetch), _ptr(n_fetch), _ptr(evict), _ptr(attend), _ptr(n_attend),
          _stream(stream))


def oasis_sparse_paged_decode_attn(h, q, pool, sel, block_to_slot, ctx_len, out, workspace, stream=None):
    _call("oasis_sparse_paged_decode_attn", h, _ptr(q), _ptr(pool), _ptr(sel), _ptr(block_to_slot),
          _ptr(ctx_len), _ptr(out), _ptr(workspace), _stream(stream))


def oasis_decode_step(h, q, pool, meta, ctx_attn, ctx_score, sel, block_to_slot, slot_to_block, scores, out,
                      workspace, fetch, n_fetch, evict, attend=None, n_attend=None, stream=None):
    _call("oasis_decode_step", h, _ptr(q), _ptr(pool), _ptr(meta), _ptr(ctx_attn), _ptr(ctx_score), _ptr(sel),
          _ptr(block_to_slot), _ptr(slot_to_block), _ptr(scores), _ptr(out), _ptr(workspace), _ptr(fetch),
          _ptr(n_fetch), _ptr(evict), _ptr(attend), _ptr(n_attend), _stream(stream))


def oasis_sparse_paged_decode_attn_noalloc(h, q, pool, sel, block_to_slot, ctx_len, out, stream=None):
    _call("oasis_sparse_paged_decode_attn_noalloc", h, _ptr(q), _ptr(pool), _ptr(sel), _ptr(block_to_slot),
          _ptr(ctx_len), _ptr(out), _stream(stream))


def oasis_decode_step_append(h, q, pool, meta, ctx_in, ctx_out, sel, block_to_slot, slot_to_block, scores, out,
                             workspace, fetch, n_fetch, evict, attend, n_attend, k_new, v_new, stream=None):
    _call("oasis_decode_step_append", h, _ptr(q), _ptr(pool), _ptr(meta), _ptr(ctx_in), _ptr(ctx_out), _ptr(sel),
          _ptr(block_to_slot), _ptr(slot_to_block), _ptr(scores), _ptr(out), _ptr(workspace), _ptr(fetch),
          _ptr(n_fetch), _ptr(evict), _ptr(attend), _ptr(n_attend), _ptr(k_new), _ptr(v_new), _stream(stream))


def oasis_decode_step_gather(h, q, pool, meta, ctx_attn, ctx_score, sel, block_to_slot, slot_to_block, scores, out,
                             workspace, fetch, n_fetch, evict, attend=None, n_attend=None, transfer=None,
                             stream=None):
    """transfer: (host_tier, pool, fetch, n_fetch) of another layer, or None."""
    tr = None
    if transfer is not None:
        tr = oasis_transfer(*(_ptr(x) for x in transfer))
    _call("oasis_decode_step_gather", h, _ptr(q), _ptr(pool), _ptr(meta), _ptr(ctx_attn), _ptr(ctx_score), _ptr(sel),
          _ptr(block_to_slot), _ptr(slot_to_block), _ptr(scores), _ptr(out), _ptr(workspace), _ptr(fetch),
          _ptr(n_fetch), _ptr(evict), _ptr(attend), _ptr(n_attend), None if tr is None else ctypes.byref(tr),
          _stream(stream))


def oasis_decode_step_carry(h, q, pool, meta, ctx_attn, ctx_score, attend, n_attend, scores, out, workspace,
                            job=None, transfer=None, stream=None):
    """job: (scores, ctx_len, sel, block_to_slot, slot_to_block, fetch, n_fetch, evict, attend, n_attend) of
    another state, or None; transfer: (host_tier, pool, fetch, n_fetch) of another layer, or None."""
    jb = None if job is None else oasis_select_job(*(_ptr(x) for x in job))
    tr = None if transfer is None else oasis_transfer(*(_ptr(x) for x in transfer))
    _call("oasis_decode_step_carry", h, _ptr(q), _ptr(pool), _ptr(meta), _ptr(ctx_attn), _ptr(ctx_score),
          _ptr(attend), _ptr(n_attend), _ptr(scores), _ptr(out), _ptr(workspace),
          None if jb is None else ctypes.byref(jb), None if tr is None else ctypes.byref(tr), _stream(stream))


def oasis_sparse_paged_decode_attn_list(h, q, pool, attend, n_attend, ctx_len, out, workspace, stream=None):
    _call("oasis_sparse_paged_decode_attn_list", h, _ptr(q), _ptr(pool), _ptr(attend), _ptr(n_attend),
          _ptr(ctx_len), _ptr(out), _ptr(workspace), _stream(stream))


def oasis_attend_and_score(h, q, pool, meta, ctx_attn, ctx_score, sel, block_to_slot, attend, n_attend, scores, out,
                           workspace, stream=None):
    _call("oasis_attend_and_score", h, _ptr(q), _ptr(pool), _ptr(meta), _ptr(ctx_attn), _ptr(ctx_score), _ptr(sel),
          _ptr(block_to_slot), _ptr(attend), _ptr(n_attend), _ptr(scores), _ptr(out), _ptr(workspace),
          _stream(stream))


def oasis_attn_combine(h, workspace, out, stream=None):
    _call("oasis_attn_combine", h, _ptr(workspace), _ptr(out), _stream(stream))


def oasis_select_diff_combine(h, scores, ctx_score, sel, block_to_slot, slot_to_block, fetch, n_fetch, evict,
                              attend, n_attend, out, workspace, stream=None):
    _call("oasis_select_diff_combine", h, _ptr(scores), _ptr(ctx_score), _ptr(sel), _ptr(block_to_slot),
          _ptr(slot_to_block), _ptr(fetch), _ptr(n_fetch), _ptr(evict), _ptr(attend), _ptr(n_attend), _ptr(out),
          _ptr(workspace), _stream(stream))


def oasis_select_and_diff_lru(h, scores, ctx_len, sel, block_to_slot, slot_to_block, slot_last_use, step, fetch,
                              n_fetch, evict, attend=None, n_attend=None, stream=None):
    _call("oasis_select_and_diff_lru", h, _ptr(scores), _ptr(ctx_len), _ptr(sel), _ptr(block_to_slot),
          _ptr(slot_to_block), _ptr(slot_last_use), int(step), _ptr(fetch), _ptr(n_fetch), _ptr(evict),
          _ptr(attend), _ptr(n_attend), _stream(stream))


def oasis_select_diff_combine_lru(h, scores, ctx_score, sel, block_to_slot, slot_to_block, slot_last_use, step,
                                  fetch, n_fetch, evict, attend, n_attend, out, workspace, stream=None):
    _call("oasis_select_diff_combine_lru", h, _ptr(scores), _ptr(ctx_score), _ptr(sel), _ptr(block_to_slot),
          _ptr(slot_to_block), _ptr(slot_last_use), int(step), _ptr(fetch), _ptr(n_fetch), _ptr(evict),
          _ptr(attend), _ptr(n_attend), _ptr(out), _ptr(workspace), _stream(stream))


def oasis_verify_score(h, q, meta, ctx_len, scores, stream=None):
    _call("oasis_verify_score", h, _ptr(q), _ptr(meta), _ptr(ctx_len), _ptr(scores), _stream(stream))


def oasis_admit(h, k_rows, v_rows, ctx_len, host_tier, meta, pool=None, block_to_slot=None, stream=None):
    _call("oasis_admit", h, _ptr(k_rows), _ptr(v_rows), _ptr(ctx_len), _ptr(host_tier), _ptr(meta), _ptr(pool),
          _ptr(block_to_slot), _stream(stream))
