"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function
include/flashblock.h declares, sizes its workspace from the shape alone, and rejects bad
arguments with the documented status before anything is enqueued."""
import ctypes as C
import os
import re

import pytest

import cached_kv_prefix_amd as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "flashblock.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:fb|losa)_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = fb.load()
    names = header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(fb.EXPORTS)


def test_status_strings():
    lib = fb.load()
    assert lib.fb_status_string(0) == b"ok"
    assert lib.fb_status_string(3) == b"workspace too small"
    assert lib.fb_status_string(4) == b"a reused cache row was never written"
    assert lib.fb_status_string(99) == b"unknown status"


def dllm_shape(**kw):
    base = dict(batch=1, h_q=32, h_kv=32, head_dim=128, block=32, seqlen_k=32768)
    base.update(kw)
    return fb.make_shape(**base)


def test_workspace_size_depends_on_shape_only():
    a = fb.workspace_size(dllm_shape())
    assert a == fb.workspace_size(dllm_shape()) and a > 0
    # 32 heads x 32 rows x 128 dims x 4 B per prefix chunk + stats; more chunks, more bytes
    s1 = fb.workspace_size(dllm_shape(num_splits=1))
    s32 = fb.workspace_size(dllm_shape(num_splits=32))
    assert s1 < s32
    assert s32 >= 32 * 32 * 32 * 128 * 4


def test_workspace_size_zero_on_invalid_shape():
    assert fb.workspace_size(dllm_shape(h_kv=5)) == 0
    assert fb.workspace_size(dllm_shape(head_dim=96)) == 0


class Fake:
    """Stand-in for a device tensor: only a pointer value (never dereferenced on error)."""
    def __init__(self, ptr=0x10000, n=1 << 30):
        self.p, self.n = ptr, n

    def data_ptr(self):
        return self.p

    def numel(self):
        return self.n

    def element_size(self):
        return 1


def call_step(shape, **over):
    lib = fb.load()
    args = dict(q=Fake(), k=Fake(), v=Fake(), kb=Fake(), vb=Fake(), mask=None, ca=Fake(), cl=Fake(), af=Fake(),
                lf=None, ws=Fake(), ws_bytes=1 << 40)
    args.update(over)
    p = lambda t: None if t is None else C.c_void_p(t.data_ptr())
    return lib.fb_step(C.byref(shape), p(args["q"]), p(args["k"]), p(args["v"]), p(args["kb"]), p(args["vb"]),
                       p(args["mask"]), p(args["ca"]), p(args["cl"]), p(args["af"]), p(args["lf"]), p(args["ws"]),
                       args["ws_bytes"], None, None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(kb=None), 1), (dict(ca=None), 1), (dict(af=None), 1),
    (dict(q=Fake(0x10004)), 1),                  # misaligned
    (dict(ws_bytes=16), 3), (dict(ws=None), 3),
])
def test_step_rejects_bad_pointers(over, code):
    assert call_step(dllm_shape(), **over) == code


def test_step_noalloc_refuses_before_launch():
    """fb_step_noalloc: an invalid shape returns fb_step's error and a shape whose workspace
    is larger than the static array returns FB_ERR_WORKSPACE, both before any device call."""
    lib = fb.load()
    p = lambda x: C.c_void_p(x)
    args = [p(0x10000)] * 5 + [None] + [p(0x10000)] * 3 + [None, None]
    bad = dllm_shape(h_kv=3)
    assert lib.fb_step_noalloc(C.byref(bad), *args) == 1
    big = fb.make_shape(1, 12, 12, 128, 4680, seqlen_k=32760)   # about 84 MiB of partials
    assert fb.workspace_size(big) > 64 << 20
    assert lib.fb_step_noalloc(C.byref(big), *args) == 3


@pytest.mark.parametrize("kw,code", [
    (dict(h_kv=3), 1), (dict(batch=0), 1), (dict(block=0), 1), (dict(head_dim=96), 2),
    (dict(flags=2), 1), (dict(flags=3), 1), (dict(num_splits=-1), 1), (dict(seqlen_k=-5), 1), (dict(softmax_scale=-1.0), 1),
    (dict(softmax_scale=float("inf")), 1), (dict(dtype=7), 1), (dict(dtype=fb.FB_F32, head_dim=512), 2),
])
def test_step_rejects_bad_shapes(kw, code):
    assert call_step(dllm_shape(**kw)) == code


def test_prefix_rejects_bad_args_before_launch():
    lib = fb.load()
    s = dllm_shape()
    r = lib.fb_prefix_attn(C.byref(s), C.c_void_p(0x10000), None, None, C.c_void_p(0x10000), C.c_void_p(0x10000),
                           C.c_void_p(0x10000), 1 << 40, None)
    assert r == 1


def test_lse_merge_validation():
    lib = fb.load()
    assert lib.fb_lse_merge(-1, 128, None, None, None, None, None, 0, None, None) == 1
    assert lib.fb_lse_merge(0, 128, None, None, None, None, None, 0, None, None) == 0   # nothing to do
    assert lib.fb_lse_merge(4, 0, None, None, None, None, None, 0, None, None) == 1
    assert lib.fb_lse_merge(4, 512, None, None, None, None, None, 0, None, None) == 2
    assert lib.fb_lse_merge(4, 128, None, None, None, None, None, 0, None, None) == 1


def losa_shape(**kw):
    s = dllm_shape(block=64, seqlen_k=131072)
    base = dict(page_size=16, topk=64, n_active=8)
    base.update(kw)
    return fb.make_losa_shape(s, **base)


def test_losa_sizes():
    ls = losa_shape()
    assert ls.max_pages == 8192
    assert fb.losa_meta_bytes(ls) == 32 * 128 * 8192 * 2          # 64 MiB each for kmin / kmax
    assert fb.losa_union_capacity(ls) == 8 * 64                   # |A| * G * topk
    assert fb.losa_workspace_size(ls) >= 32 * 8 * 8192 * 8        # fp64 page scores
    assert fb.losa_workspace_size(losa_shape(n_active=65)) == 0   # |A| > B
    assert fb.losa_workspace_size(fb.make_losa_shape(dllm_shape(block=64, seqlen_k=131072), max_pages=100)) == 0


def test_losa_select_rejects_small_workspace():
    lib = fb.load()
    ls = losa_shape()
    f = C.c_void_p(0x10000)
    r = lib.losa_select_union(C.byref(ls), f, f, f, f, f, f, f, f, f, 64, None)
    assert r == 3


def test_mask_validation():
    lib = fb.load()
    assert lib.fb_mask_threshold(None, 4, 1, 32, None, None) == 1
    assert lib.fb_mask_similarity(None, 0.95, 0, None, None) == 0
    assert lib.fb_mask_similarity(None, 0.95, 4, None, None) == 1
    assert lib.fb_head_cosine(0, 32, 32, 128, None, None, None, None) == 1


def residual_shape(**kw):
    s = dllm_shape(block=64, seqlen_k=131072)
    base = dict(page_size=16, max_sel=512)
    base.update(kw)
    return fb.make_residual_shape(s, **base)


def test_residual_sizes_and_shape_checks():
    rs = residual_shape()
    assert rs.max_pages == 8192
    w = fb.residual_workspace_size(rs)
    assert w == fb.residual_workspace_size(residual_shape()) and w >= 32 * 8192 * 4   # complement lists
    assert fb.residual_workspace_size(residual_shape(max_sel=0)) == 0
    assert fb.residual_workspace_size(residual_shape(max_sel=9000)) == 0            # > max_pages
    assert fb.residual_workspace_size(residual_shape(max_pages=100)) == 0           # prefix needs 8192
    assert fb.residual_workspace_size(residual_shape(max_pages=70000, max_sel=10)) == 0   # above 65536
    assert fb.residual_workspace_size(residual_shape(page_size=0, max_pages=1, max_sel=1)) == 0


def test_residual_step_rejects_bad_args_before_launch():
    lib = fb.load()
    rs = residual_shape()
    f = C.c_void_p(0x10000)
    n = fb.residual_workspace_size(rs)
    call = lambda sp=f, sc=f, ws=f, nb=n, q=f: lib.fb_residual_step(C.byref(rs), q, f, f, f, f, sp, sc, None, f, f, f,
                                                                   None, ws, nb, None, None)
    assert call(sp=None) == 1 and call(sc=None) == 1 and call(q=None) == 1
    assert call(q=C.c_void_p(0x10002)) == 1
    assert call(nb=n - 1) == 3 and call(ws=None) == 3
    bad = residual_shape(max_sel=0)
    assert lib.fb_residual_step(C.byref(bad), f, f, f, f, f, f, f, None, f, f, f, None, f, n, None, None) == 1


def test_lifecycle_validation():
    lib = fb.load()
    f = C.c_void_p(0x10000)
    s = dllm_shape(batch=2)
    # in place with more than one sequence would move the later sequences
    assert lib.fb_append_block(C.byref(s), f, f, f, f, f, f, None, None) == 1
    g = C.c_void_p(0x20000)
    assert lib.fb_append_block(C.byref(s), f, f, f, f, g, f, None, None) == 1      # only k in place
    assert lib.fb_append_block(C.byref(s), f, f, None, f, g, g, None, None) == 1
    plan = fb.BlockPlan(0, fb.FB_RULE_THRESHOLD, 4, 0.0)
    n = fb.block_workspace_size(s)
    assert n > fb.workspace_size(s)
    args = [f, f, f, f, f, f, f, f, f, None, f, None, f, n, None]
    assert lib.fb_block_run(C.byref(s), C.byref(plan), *args) == 1                  # no steps
    plan = fb.BlockPlan(4, 7, 4, 0.0)
    assert lib.fb_block_run(C.byref(s), C.byref(plan), *args) == 1                  # unknown rule
    plan = fb.BlockPlan(4, fb.FB_RULE_THRESHOLD, 4, 0.0)
    a2 = list(args)
    a2[5] = None
    assert lib.fb_block_run(C.byref(s), C.byref(plan), *a2) == 1                    # threshold without M
    a3 = list(args)
    a3[13] = n - 1
    assert lib.fb_block_run(C.byref(s), C.byref(plan), *a3) == 3
    ls = losa_shape()
    assert lib.losa_page_meta_append(C.byref(ls), 0, f, f, f, None) == 1


def test_varlen_validation():
    lib = fb.load()
    s = dllm_shape(batch=6, block=128)
    f = C.c_void_p(0x10000)
    vs = fb.VarlenShape(s, f, 6 * 128 + 1)                      # more rows than batch * B_max
    assert lib.fb_prefix_attn_varlen_workspace_size(C.byref(vs)) == 0
    vs = fb.VarlenShape(s, None, 10)
    assert lib.fb_prefix_attn_varlen_workspace_size(C.byref(vs)) == 0
    vs = fb.VarlenShape(s, f, 252)
    n = lib.fb_prefix_attn_varlen_workspace_size(C.byref(vs))
    assert n > fb.workspace_size(s)
    assert lib.fb_prefix_attn_varlen(C.byref(vs), f, f, f, f, f, f, n - 1, None) == 3
    assert lib.fb_prefix_attn_varlen(C.byref(vs), None, f, f, f, f, f, n, None) == 1
    vs0 = fb.VarlenShape(s, f, 0)
    assert lib.fb_prefix_attn_varlen(C.byref(vs0), None, None, None, None, None, None, 0, None) == 0


def test_grid_size_limits_are_rejected_before_launch():
    """Sizes whose launch grid would not fit return FB_ERR_UNSUPPORTED instead of wrapping."""
    lib = fb.load()
    f = C.c_void_p(0x10000)
    assert lib.fb_lse_merge(1 << 34, 128, f, f, f, f, f, 0, None, None) == 2
    assert lib.fb_mask_similarity(f, 0.9, 1 << 40, f, None) == 2
    assert lib.fb_mask_threshold(f, 4, 1 << 30, 1 << 10, f, None) == 2
    assert lib.fb_head_cosine(1 << 16, 4, 1 << 16, 128, f, f, f, None) == 2
    ls = fb.make_losa_shape(fb.make_shape(65535, 1024, 1024, 128, 1024, seqlen_k=16), page_size=16, topk=1,
                            n_active=1024, max_pages=1)
    assert fb.losa_workspace_size(ls) == 0


def ceiling_header_functions():
    text = open(os.path.join(ROOT, "include", "fb_ceiling.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fbc_[a-z_0-9]+)\s*\(", text)))


def test_ceiling_library_exports_every_declared_function():
    from cached_kv_prefix_amd import ceiling
    lib = ceiling.load()
    names = ceiling_header_functions()
    assert names == sorted(ceiling.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_ceiling_argument_checks_launch_nothing():
    """Invalid arguments return 1 before any launch (so these run without a GPU)."""
    from cached_kv_prefix_amd import ceiling
    lib = ceiling.load()
    buf, sink = C.c_void_p(0x10000), C.c_void_p(0x20000)
    assert lib.fbc_stream_read(None, 1024, 4, 0, sink, None) == 1
    assert lib.fbc_stream_read(buf, 1024, 4, 0, None, None) == 1
    assert lib.fbc_stream_read(buf, 0, 4, 0, sink, None) == 1
    assert lib.fbc_stream_read(buf, 1000, 4, 0, sink, None) == 1          # not a multiple of 16 bytes
    assert lib.fbc_stream_read(buf, 1024, 0, 0, sink, None) == 1
    assert lib.fbc_stream_read(buf, 1024, 65537, 0, sink, None) == 1
    assert lib.fbc_stream_read(C.c_void_p(0x10008), 1024, 4, 0, sink, None) == 1   # misaligned
    assert lib.fbc_mfma_loop(4, 10, 1.0, 1.0, None, None) == 1
    assert lib.fbc_mfma_loop(0, 10, 1.0, 1.0, sink, None) == 1
    assert lib.fbc_mfma_loop(65537, 10, 1.0, 1.0, sink, None) == 1
    assert lib.fbc_mfma_loop(4, 0, 1.0, 1.0, sink, None) == 1
    assert lib.fbc_mfma_loop(4, 262145, 1.0, 1.0, sink, None) == 1
    assert lib.fbc_stream_read(buf, 1024, 4, 2, sink, None) == 1       # nontemporal is 0 or 1
    assert lib.fbc_mfma_valu(0, 0, 4, 10, 1.0, None, None) == 1
    assert lib.fbc_mfma_valu(4, 4, 4, 10, 1.0, sink, None) == 1        # no such mode
    assert lib.fbc_mfma_valu(-1, 4, 4, 10, 1.0, sink, None) == 1
    assert lib.fbc_mfma_valu(2, 0, 4, 10, 1.0, sink, None) == 1        # a vector stream needs operations
    assert lib.fbc_mfma_valu(1, 3, 4, 10, 1.0, sink, None) == 1
    assert lib.fbc_mfma_valu(3, 16, 4, 10, 1.0, sink, None) == 1
    assert lib.fbc_mfma_valu(2, 4, 0, 10, 1.0, sink, None) == 1
    assert lib.fbc_mfma_valu(2, 4, 65537, 10, 1.0, sink, None) == 1
    assert lib.fbc_mfma_valu(2, 4, 4, 0, 1.0, sink, None) == 1
    assert lib.fbc_mfma_valu(2, 4, 4, 262145, 1.0, sink, None) == 1
