"""Python binding of libflashblock.so (the C ABI in include/flashblock.h).

Argument marshalling only: every step of the FlashBlock step and the LoSA-style sparse
path runs in the library's HIP kernels.  torch tensors supply device memory and the
current HIP stream.  There is no fallback: if the shared library is missing every call
raises.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflashblock.so")

FB_BF16, FB_F32 = 0, 1
STATUS = {0: "FB_OK", 1: "FB_ERR_INVALID_ARG", 2: "FB_ERR_UNSUPPORTED", 3: "FB_ERR_WORKSPACE",
          4: "FB_ERR_CACHE_INVALID", 5: "FB_ERR_HIP"}
FB_FLAG_CHECK_CACHE = 1   # fb_shape.flags: debug check that every reused cache row was written
EXPORTS = ("fb_status_string", "fb_workspace_size", "fb_prefix_attn", "fb_block_attn", "fb_lse_merge",
           "fb_step", "fb_step_threshold", "fb_step_noalloc", "fb_mask_threshold", "fb_mask_similarity", "fb_head_cosine", "losa_meta_bytes",
           "losa_workspace_size", "losa_union_capacity", "losa_page_meta", "losa_select_union", "losa_step",
           "fb_residual_workspace_size", "fb_residual_step", "fb_append_block", "losa_page_meta_append",
           "fb_block_workspace_size", "fb_block_run", "fb_prefix_attn_varlen_workspace_size",
           "fb_prefix_attn_varlen")
FB_RULE_THRESHOLD, FB_RULE_SIMILARITY = 0, 1


class FlashBlockError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class FbShape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("h_q", C.c_int32), ("h_kv", C.c_int32), ("head_dim", C.c_int32),
                ("block", C.c_int32), ("cu_seqlens_k", C.c_void_p), ("seqlen_k", C.c_int32),
                ("max_seqlen_k", C.c_int32), ("dtype", C.c_int32), ("softmax_scale", C.c_float),
                ("num_splits", C.c_int32), ("flags", C.c_uint32)]


class LosaShape(C.Structure):
    _fields_ = [("s", FbShape), ("page_size", C.c_int32), ("topk", C.c_int32), ("n_active", C.c_int32),
                ("max_pages", C.c_int32)]


class ResidualShape(C.Structure):
    _fields_ = [("s", FbShape), ("page_size", C.c_int32), ("max_pages", C.c_int32), ("max_sel", C.c_int32)]


class VarlenShape(C.Structure):
    _fields_ = [("s", FbShape), ("cu_seqlens_q", C.c_void_p), ("total_q", C.c_int32)]


class BlockPlan(C.Structure):
    _fields_ = [("n_steps", C.c_int32), ("rule", C.c_int32), ("tau", C.c_int32), ("gamma", C.c_float)]


class FbTrace(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_begin", "attn_end", "merge_begin", "merge_end",
                                           "select_begin", "select_end")]


_lib = None


def load(path: str | None = None):
    """Load the shared library (raises FileNotFoundError when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(f"{p} is missing; build it with `python -m cached_kv_prefix_amd.build`")
    lib = C.CDLL(p)
    vp, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
    sp, lp, tp = C.POINTER(FbShape), C.POINTER(LosaShape), C.POINTER(FbTrace)
    rp = C.POINTER(ResidualShape)
    bp = C.POINTER(BlockPlan)
    vlp = C.POINTER(VarlenShape)
    sig = {
        "fb_status_string": (C.c_char_p, [i32]),
        "fb_workspace_size": (sz, [sp]),
        "fb_prefix_attn": (i32, [sp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "fb_block_attn": (i32, [sp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "fb_lse_merge": (i32, [i64, i32, vp, vp, vp, vp, vp, i32, vp, vp]),
        "fb_step": (i32, [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, tp, vp]),
        "fb_step_noalloc": (i32, [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "fb_step_threshold": (i32, [sp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, sz, tp, vp]),
        "fb_mask_threshold": (i32, [vp, i32, i32, i32, vp, vp]),
        "fb_mask_similarity": (i32, [vp, f32, i64, vp, vp]),
        "fb_head_cosine": (i32, [i32, i32, i32, i32, vp, vp, vp, vp]),
        "losa_meta_bytes": (sz, [lp]),
        "losa_workspace_size": (sz, [lp]),
        "losa_union_capacity": (i32, [lp]),
        "losa_page_meta": (i32, [lp, vp, vp, vp, vp]),
        "losa_select_union": (i32, [lp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "losa_step": (i32, [lp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, tp, vp]),
        "fb_residual_workspace_size": (sz, [rp]),
        "fb_residual_step": (i32, [rp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, tp, vp]),
        "fb_append_block": (i32, [sp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "losa_page_meta_append": (i32, [lp, i32, vp, vp, vp, vp]),
        "fb_block_workspace_size": (sz, [sp]),
        "fb_prefix_attn_varlen_workspace_size": (sz, [vlp]),
        "fb_prefix_attn_varlen": (i32, [vlp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "fb_block_run": (i32, [sp, bp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


# ----------------------------------------------------------------------------- helpers

def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _check(st: int, where: str):
    if st != 0:
        raise FlashBlockError(st, where)


def dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FB_BF16
    if t.dtype == torch.float32:
        return FB_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def make_shape(batch, h_q, h_kv, head_dim, block, *, dtype=FB_BF16, seqlen_k=0, cu_seqlens_k=None,
               max_seqlen_k=0, softmax_scale=0.0, num_splits=0, flags=0) -> FbShape:
    return FbShape(batch, h_q, h_kv, head_dim, block,
                   None if cu_seqlens_k is None else C.c_void_p(cu_seqlens_k.data_ptr()),
                   seqlen_k, max_seqlen_k, dtype, softmax_scale, num_splits, flags)


def make_losa_shape(shape: FbShape, page_size=16, topk=64, n_active=8, max_pages=None) -> LosaShape:
    if max_pages is None:
        n = shape.max_seqlen_k if shape.cu_seqlens_k else shape.seqlen_k
        max_pages = max(1, -(-n // page_size))
    return LosaShape(shape, page_size, topk, n_active, max_pages)


def make_residual_shape(shape: FbShape, page_size=16, max_sel=None, max_pages=None) -> ResidualShape:
    if max_pages is None:
        n = shape.max_seqlen_k if shape.cu_seqlens_k else shape.seqlen_k
        max_pages = max(1, -(-n // page_size))
    return ResidualShape(shape, page_size, max_pages, max_pages if max_sel is None else max_sel)


def make_trace(**events) -> FbTrace:
    """torch.cuda.Event objects (enable_timing=True) by field name."""
    tr = FbTrace()
    for k, e in events.items():
        setattr(tr, k, C.c_void_p(e.cuda_event))
    return tr


# ------------------------------------------------------------------------- entry points

def workspace_size(shape: FbShape) -> int:
    return int(load().fb_workspace_size(C.byref(shape)))


def prefix_attn(shape, q, k, v, a_out, l_out, ws, stream=None):
    _check(load().fb_prefix_attn(C.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(a_out), _ptr(l_out),
                                 _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "fb_prefix_attn")


def block_attn(shape, q, k_blk, v_blk, a_in, l_in, ws, stream=None):
    _check(load().fb_block_attn(C.byref(shape), _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(a_in), _ptr(l_in),
                                _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "fb_block_attn")


def lse_merge(a_out, l_out, a_in, l_in, a_full, l_full=None, stream=None):
    d = a_out.shape[-1]
    rows = a_out.numel() // d if d else 0
    _check(load().fb_lse_merge(rows, d, _ptr(a_out), _ptr(l_out), _ptr(a_in), _ptr(l_in), _ptr(a_full),
                               dtype_code(a_full), _ptr(l_full), _stream(stream)), "fb_lse_merge")


def step(shape, q, k, v, k_blk, v_blk, reuse_mask, cache_a, cache_l, a_full, l_full, ws, trace=None,
         stream=None):
    _check(load().fb_step(C.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(k_blk), _ptr(v_blk), _ptr(reuse_mask),
                          _ptr(cache_a), _ptr(cache_l), _ptr(a_full), _ptr(l_full), _ptr(ws),
                          0 if ws is None else ws.numel() * ws.element_size(),
                          None if trace is None else C.byref(trace), _stream(stream)), "fb_step")


def step_noalloc(shape, q, k, v, k_blk, v_blk, reuse_mask, cache_a, cache_l, a_full, l_full, stream=None):
    """fb_step without a workspace: the partials go to the library's static per-GPU array."""
    _check(load().fb_step_noalloc(C.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(k_blk), _ptr(v_blk),
                                  _ptr(reuse_mask), _ptr(cache_a), _ptr(cache_l), _ptr(a_full), _ptr(l_full),
                                  _stream(stream)), "fb_step_noalloc")


def step_threshold(shape, q, k, v, k_blk, v_blk, m_updated, tau, cache_a, cache_l, a_full, l_full, ws,
                   trace=None, stream=None):
    _check(load().fb_step_threshold(C.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(k_blk), _ptr(v_blk),
                                    _ptr(m_updated), tau, _ptr(cache_a), _ptr(cache_l), _ptr(a_full),
                                    _ptr(l_full), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                    None if trace is None else C.byref(trace), _stream(stream)),
           "fb_step_threshold")


def mask_threshold(m_updated, tau, h_q, mask, stream=None):
    _check(load().fb_mask_threshold(_ptr(m_updated), tau, m_updated.numel(), h_q, _ptr(mask), _stream(stream)),
           "fb_mask_threshold")


def mask_similarity(sim, gamma, mask, stream=None):
    _check(load().fb_mask_similarity(_ptr(sim), gamma, sim.numel(), _ptr(mask), _stream(stream)),
           "fb_mask_similarity")


def head_cosine(a_prev, a_cur, sim, stream=None):
    b, B, h, d = a_prev.shape
    _check(load().fb_head_cosine(b, B, h, d, _ptr(a_prev), _ptr(a_cur), _ptr(sim), _stream(stream)),
           "fb_head_cosine")


def losa_meta_bytes(ls: LosaShape) -> int:
    return int(load().losa_meta_bytes(C.byref(ls)))


def losa_workspace_size(ls: LosaShape) -> int:
    return int(load().losa_workspace_size(C.byref(ls)))


def losa_union_capacity(ls: LosaShape) -> int:
    return int(load().losa_union_capacity(C.byref(ls)))


def losa_page_meta(ls, k, kmin, kmax, stream=None):
    _check(load().losa_page_meta(C.byref(ls), _ptr(k), _ptr(kmin), _ptr(kmax), _stream(stream)), "losa_page_meta")


def losa_select_union(ls, q_cur, q_prev, kmin, kmax, active, topk_pages, union_pages, union_count, ws,
                      stream=None):
    _check(load().losa_select_union(C.byref(ls), _ptr(q_cur), _ptr(q_prev), _ptr(kmin), _ptr(kmax), _ptr(active),
                                    _ptr(topk_pages), _ptr(union_pages), _ptr(union_count), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)), "losa_select_union")


def losa_step(ls, q_cur, q_prev, k, v, k_blk, v_blk, kmin, kmax, cache_a, cache_l, a_full, l_full, active,
              topk_pages, union_pages, union_count, ws, trace=None, stream=None):
    _check(load().losa_step(C.byref(ls), _ptr(q_cur), _ptr(q_prev), _ptr(k), _ptr(v), _ptr(k_blk), _ptr(v_blk),
                            _ptr(kmin), _ptr(kmax), _ptr(cache_a), _ptr(cache_l), _ptr(a_full), _ptr(l_full),
                            _ptr(active), _ptr(topk_pages), _ptr(union_pages), _ptr(union_count), _ptr(ws),
                            ws.numel() * ws.element_size(), None if trace is None else C.byref(trace),
                            _stream(stream)), "losa_step")


def residual_workspace_size(rs: ResidualShape) -> int:
    return int(load().fb_residual_workspace_size(C.byref(rs)))


def residual_step(rs, q, k, v, k_blk, v_blk, sel_pages, sel_count, reuse_mask, cache_a, cache_l, a_full, l_full,
                  ws, trace=None, stream=None):
    _check(load().fb_residual_step(C.byref(rs), _ptr(q), _ptr(k), _ptr(v), _ptr(k_blk), _ptr(v_blk),
                                   _ptr(sel_pages), _ptr(sel_count), _ptr(reuse_mask), _ptr(cache_a),
                                   _ptr(cache_l), _ptr(a_full), _ptr(l_full), _ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(),
                                   None if trace is None else C.byref(trace), _stream(stream)),
           "fb_residual_step")


def append_block(shape, k, v, k_blk, v_blk, k_out, v_out, cu_out=None, stream=None):
    _check(load().fb_append_block(C.byref(shape), _ptr(k), _ptr(v), _ptr(k_blk), _ptr(v_blk), _ptr(k_out),
                                  _ptr(v_out), _ptr(cu_out), _stream(stream)), "fb_append_block")


def losa_page_meta_append(ls, n_appended, k, kmin, kmax, stream=None):
    _check(load().losa_page_meta_append(C.byref(ls), n_appended, _ptr(k), _ptr(kmin), _ptr(kmax), _stream(stream)),
           "losa_page_meta_append")


def block_workspace_size(shape) -> int:
    return int(load().fb_block_workspace_size(C.byref(shape)))


def block_run(shape, plan, q_steps, k, v, k_blk_steps, v_blk_steps, m_steps, cache_a, cache_l, a_full_steps,
              l_full_steps, masks, sims, ws, stream=None):
    _check(load().fb_block_run(C.byref(shape), C.byref(plan), _ptr(q_steps), _ptr(k), _ptr(v), _ptr(k_blk_steps),
                               _ptr(v_blk_steps), _ptr(m_steps), _ptr(cache_a), _ptr(cache_l), _ptr(a_full_steps),
                               _ptr(l_full_steps), _ptr(masks), _ptr(sims), _ptr(ws),
                               0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)), "fb_block_run")


def make_varlen_shape(shape: FbShape, cu_seqlens_q, total_q: int) -> VarlenShape:
    return VarlenShape(shape, C.c_void_p(cu_seqlens_q.data_ptr()), total_q)


def prefix_attn_varlen_workspace_size(vs) -> int:
    return int(load().fb_prefix_attn_varlen_workspace_size(C.byref(vs)))


def prefix_attn_varlen(vs, q, k, v, a_out, l_out, ws, stream=None):
    _check(load().fb_prefix_attn_varlen(C.byref(vs), _ptr(q), _ptr(k), _ptr(v), _ptr(a_out), _ptr(l_out), _ptr(ws),
                                        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "fb_prefix_attn_varlen")
