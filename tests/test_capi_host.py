"""Host-only checks of the C ABI: the library loads without a GPU, exports
every function include/moe_fp8.h declares, and rejects invalid requests with
the documented status before touching the HIP runtime."""

import ctypes
import os
import re

import pytest

import block_fp8_mixture_amd as moe
from block_fp8_mixture_amd import _binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe_fp8.h")
OK, INVALID, UNSUPPORTED, CAPACITY = 0, 1, 2, 3
NULL = None
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    return moe.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_six_entry_points():
    names = declared_functions()
    for fn in ("moe_align", "moe_act_quant", "moe_grouped_gemm_fp8", "moe_silu_mul_quant",
               "moe_topk_combine", "moe_forward"):
        assert fn in names


def test_library_exports_every_declared_function(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_min_row_cap(lib):
    assert moe.moe_min_row_cap(4096, 8, 32, 16) == 32768 + 32 * 15
    assert moe.moe_min_row_cap(4, 8, 288, 16) == 32 + 32 * 15
    assert moe.moe_min_row_cap(8, 2, 4, 16) == 64      # 16 pairs on 4 experts: at most 4 x 16 rows
    assert moe.moe_min_row_cap(3, 1, 8, 4) == 12       # 3 pairs: at most 3 segments of 4
    assert moe.moe_min_row_cap(0, 8, 4, 16) == 0
    assert moe.moe_min_row_cap(5, 0, 4, 16) == -1
    assert moe.moe_min_row_cap(1 << 30, 64, 4, 16) == -1


def test_status_strings(lib):
    assert moe.moe_status_string(0) == "ok"
    assert moe.moe_status_string(3) == "capacity too small"
    assert moe.moe_status_string(99) == "unknown status"


def test_align_validation(lib):
    f = lib.moe_align
    args = dict(ids=FAKE, t_cap=4, live=NULL, k=8, e=288, a=16, rc=512)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["ids"], a["t_cap"], a["live"], a["k"], a["e"], 0, a["a"], a["rc"], FAKE, FAKE,
                 FAKE, FAKE, NULL)
    assert call(k=0) == INVALID
    assert call(k=65) == INVALID
    assert call(a=0) == INVALID
    assert call(e=0) == INVALID
    assert call(t_cap=-1) == INVALID
    assert call(e=1025) == UNSUPPORTED
    assert call(rc=511) == CAPACITY
    assert call(ids=NULL) == INVALID
    assert f(FAKE, 4, NULL, 8, 288, 0, 16, 512, NULL, FAKE, FAKE, FAKE, NULL) == INVALID


def test_act_quant_validation(lib):
    f = lib.moe_act_quant
    assert f(FAKE, 4, NULL, 100, 0, 0, FAKE, FAKE, NULL) == INVALID    # hidden not a multiple of 128
    assert f(FAKE, 4, NULL, 256, 3, 0, FAKE, FAKE, NULL) == INVALID    # unknown format
    assert f(FAKE, 4, NULL, 256, 0, 2, FAKE, FAKE, NULL) == INVALID    # unknown rounding
    assert f(NULL, 4, NULL, 256, 0, 0, FAKE, FAKE, NULL) == INVALID
    assert f(FAKE, 4, NULL, 256, 0, 1, FAKE, NULL, NULL) == INVALID
    assert f(NULL, 0, NULL, 256, 0, 1, NULL, NULL, NULL) == OK         # nothing to do, nothing launched


def test_gemm_validation(lib):
    f = lib.moe_grouped_gemm_fp8

    def call(n=256, k=256, fmt=0, div=1, e=4, rc=64, mr=0, a=FAKE, c=FAKE, w=FAKE):
        return f(a, FAKE, fmt, 64, NULL, div, w, FAKE, FAKE, FAKE, e, rc, mr, n, k, c, NULL, NULL)
    assert call(n=200) == INVALID
    assert call(k=0) == INVALID
    assert call(fmt=7) == INVALID
    assert call(div=0) == INVALID
    assert call(e=0) == INVALID
    assert call(e=2000) == UNSUPPORTED
    assert call(mr=-1) == INVALID
    assert call(a=NULL) == INVALID
    assert call(w=NULL) == INVALID
    assert call(rc=0, a=NULL, c=NULL) == OK


def test_silu_mul_quant_validation(lib):
    f = lib.moe_silu_mul_quant

    def call(inter=256, act=0, lim=7.0, fmt=0, rc=64, gu=FAKE, rnd=0):
        return f(gu, inter, FAKE, FAKE, 4, rc, act, lim, fmt, rnd, FAKE, FAKE, NULL)
    assert call(inter=100) == INVALID
    assert call(act=3) == INVALID
    assert call(act=1, lim=0.0) == INVALID
    assert call(act=2, lim=-1.0) == INVALID
    assert call(act=1, lim=float("nan")) == INVALID
    assert call(fmt=5) == INVALID
    assert call(rnd=-1) == INVALID
    assert call(gu=NULL) == INVALID
    assert call(rc=1 << 24, inter=1 << 15) == INVALID  # 2^32 groups
    assert call(rc=0, gu=NULL) == OK


def test_combine_validation(lib):
    f = lib.moe_topk_combine
    assert f(FAKE, 64, FAKE, FAKE, 4, NULL, 0, 256, FAKE, NULL) == INVALID
    assert f(FAKE, 64, FAKE, FAKE, 4, NULL, 8, 200, FAKE, NULL) == INVALID
    assert f(FAKE, 64, NULL, FAKE, 4, NULL, 8, 256, FAKE, NULL) == INVALID
    assert f(NULL, 0, NULL, NULL, 0, NULL, 8, 256, NULL, NULL) == OK


def _problem(**kw):
    d = dict(num_experts=32, hidden=7168, inter=2048, topk=8, t_cap=4096, align_rows=16,
             row_cap=0, scale_fmt=0, act=0, clamp_limit=float("inf"), rounding=0, expert_start=0,
             expert_cap=0, weight_fmt=0)
    d.update(kw)
    return B._Problem(**d)


def test_workspace_plan_layout(lib):
    for fmt in (0, 2):
        p = _problem(scale_fmt=fmt)
        lay = B._Layout()
        assert lib.moe_workspace_plan(ctypes.byref(p), ctypes.byref(lay)) == OK
        R = lay.row_cap
        assert R == 32768 + 32 * 15
        sb = 1 if fmt == 2 else 4
        spans = [("expert_counts", 32 * 4), ("expert_offsets", 33 * 4), ("row_to_pair", R * 4),
                 ("pair_to_row", 4096 * 8 * 4), ("xq", 4096 * 7168), ("xs", 56 * 4096 * sb),
                 ("c1", R * 4096 * 2), ("hq", R * 2048), ("hs", 16 * R * sb), ("y", R * 7168 * 2)]
        end = 0
        for name, size in spans:
            start = getattr(lay, name)
            assert start % 256 == 0 and start >= end, name
            end = start + size
        assert lay.total >= end
        assert lib.moe_workspace_bytes(ctypes.byref(p)) == lay.total


def test_forward_validation(lib):
    lay = B._Layout()
    assert lib.moe_workspace_plan(ctypes.byref(_problem(hidden=100)), ctypes.byref(lay)) == INVALID
    assert lib.moe_workspace_plan(ctypes.byref(_problem(row_cap=100)), ctypes.byref(lay)) == CAPACITY
    assert lib.moe_workspace_plan(ctypes.byref(_problem(act=1, clamp_limit=0.0)),
                                  ctypes.byref(lay)) == INVALID
    assert lib.moe_workspace_plan(ctypes.byref(_problem(num_experts=4096)),
                                  ctypes.byref(lay)) == UNSUPPORTED
    assert lib.moe_workspace_bytes(ctypes.byref(_problem(inter=0))) == 0
    assert lib.moe_workspace_plan(ctypes.byref(_problem(rounding=2)), ctypes.byref(lay)) == INVALID
    assert lib.moe_workspace_plan(ctypes.byref(_problem(rounding=1)), ctypes.byref(lay)) == OK
    # FC2-input groups (row_cap * inter / 128) are indexed in 32 bits
    assert lib.moe_workspace_plan(ctypes.byref(_problem(row_cap=1 << 24, inter=1 << 15)),
                                  ctypes.byref(lay)) == INVALID
    p = _problem()
    t = B._Tensors(*([FAKE.value] * 9))
    need = lib.moe_workspace_bytes(ctypes.byref(p))
    assert lib.moe_forward(ctypes.byref(p), ctypes.byref(t), FAKE, need - 1, NULL) == CAPACITY
    assert lib.moe_forward(ctypes.byref(p), ctypes.byref(t), NULL, need, NULL) == INVALID
    t0 = B._Tensors(*([FAKE.value] * 8 + [None]))
    assert lib.moe_forward(ctypes.byref(p), ctypes.byref(t0), FAKE, need, NULL) == INVALID
    assert lib.moe_forward(ctypes.byref(_problem(t_cap=0)), ctypes.byref(t), FAKE, need, NULL) == OK


def test_decode_plan_lays_out_act_and_fc1_decode_validates(lib):
    # decode-sized problem: the plan lays out act [R, I] fp32 at the end
    p = _problem(num_experts=288, hidden=4096, inter=512, topk=8, t_cap=4)
    lay = B._Layout()
    assert lib.moe_workspace_plan(ctypes.byref(p), ctypes.byref(lay)) == OK
    assert lay.act % 256 == 0 and lay.act >= lay.y + lay.row_cap * 4096 * 2
    assert lay.total >= lay.act + lay.row_cap * 512 * 4
    # 4096 tokens: no act buffer (act == total)
    big = B._Layout()
    assert lib.moe_workspace_plan(ctypes.byref(_problem()), ctypes.byref(big)) == OK
    assert big.act == big.status
    need = lib.moe_workspace_bytes(ctypes.byref(p))
    t = B._Tensors(*([FAKE.value] * 9))
    f = lib.moe_fc1_decode
    assert f(ctypes.byref(_problem()), ctypes.byref(t), FAKE, big.total, NULL) == UNSUPPORTED
    assert f(ctypes.byref(p), ctypes.byref(t), FAKE, need - 1, NULL) == CAPACITY
    assert f(ctypes.byref(p), ctypes.byref(t), NULL, need, NULL) == INVALID
    tx = B._Tensors(None, *([FAKE.value] * 8))
    assert f(ctypes.byref(p), ctypes.byref(tx), FAKE, need, NULL) == INVALID
    # 8 tokens at H = 6144 fit the decode path but not FC1's resident activations
    p8 = _problem(num_experts=256, hidden=6144, inter=256, topk=8, t_cap=8)
    l8 = B._Layout()
    assert lib.moe_workspace_plan(ctypes.byref(p8), ctypes.byref(l8)) == OK and l8.act < l8.status
    assert f(ctypes.byref(p8), ctypes.byref(t), FAKE, l8.total, NULL) == UNSUPPORTED


def _header_macros(prefix):
    return {m: int(v) for m, v in re.findall(r"#define (" + prefix + r"[A-Z0-9_]+) (\d+)", open(HEADER).read())}


def test_python_mirrors_of_header_limits():
    g = _header_macros("MOE_GEMM_")
    assert moe.GEMM_TILES == {"stream_tile_m": g["MOE_GEMM_STREAM_TILE_M"],
                              "stream_max_rows": g["MOE_GEMM_STREAM_MAX_ROWS"],
                              "tiled_tile_m": g["MOE_GEMM_TILED_TILE_M"],
                              "col_tile": g["MOE_GEMM_COL_TILE"]}
    d = _header_macros("MOE_DECODE_")
    assert moe.DECODE_LIMITS == {"max_pairs": d["MOE_DECODE_MAX_PAIRS"],
                                 "fc2_row_bytes": d["MOE_DECODE_FC2_ROW_BYTES"],
                                 "fc2_max_scales": d["MOE_DECODE_FC2_MAX_SCALES"],
                                 "layer_token_bytes": d["MOE_DECODE_LAYER_TOKEN_BYTES"],
                                 "layer_max_scales": d["MOE_DECODE_LAYER_MAX_SCALES"]}


def test_decode_layer_applies_matches_the_workspace_plan(lib):
    # The one-launch layer is a form of the decode path: whenever it applies,
    # the plan lays out the decode path's act buffer.
    for t_cap, k, h, i in [(4, 8, 4096, 512), (1, 8, 4096, 512), (8, 8, 6144, 256),
                           (16, 4, 3584, 256), (8, 8, 7168, 256), (32, 2, 512, 128)]:
        lay = moe.moe_workspace_plan(288, h, i, k, t_cap)
        if moe.decode_layer_applies(t_cap, k, h, i):
            assert lay["act"] < lay["status"], (t_cap, k, h, i)
    assert moe.decode_layer_applies(8, 8, 6144, 256)       # 49 KB of token codes
    assert not moe.decode_layer_applies(9, 7, 7168, 256)   # 64.6 KB
    assert not moe.decode_layer_applies(4, 8, 4096, 2048)  # FC2 input rows too large
    # MXFP4 weights: the one-launch layer (and with it the act buffer) exactly
    # when the FP8 conditions hold and H and I are multiples of 256
    for t_cap, k, h, i in [(4, 8, 4096, 512), (1, 8, 6144, 256), (8, 8, 6144, 256), (4, 8, 4224, 512),
                           (4, 8, 4096, 384), (32, 2, 512, 128), (8, 8, 7168, 256), (4, 8, 4096, 2048)]:
        lay = moe.moe_workspace_plan(288, h, i, k, t_cap, weight_fmt="mxfp4")
        applies = moe.decode_layer_applies(t_cap, k, h, i, "mxfp4")
        assert applies == (moe.decode_layer_applies(t_cap, k, h, i) and h % 256 == 0 and i % 256 == 0)
        assert applies == (lay["act"] < lay["status"]), (t_cap, k, h, i)


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [ctypes.POINTER(B._Problem), ctypes.POINTER(B._Tensors),
                                        ctypes.c_void_p]
    t = B._Tensors(*([FAKE.value] * 9))
    big = _problem()  # the 4096-token layer needs about 1 GB of workspace
    assert lib.moe_workspace_bytes(ctypes.byref(big)) > _header_macros("MOE_NOALLOC_")["MOE_NOALLOC_SCRATCH_BYTES"]
    assert lib.moe_forward_noalloc(ctypes.byref(big), ctypes.byref(t), NULL) == CAPACITY
    assert lib.moe_forward_noalloc(ctypes.byref(_problem(hidden=100)), ctypes.byref(t), NULL) == INVALID
    assert lib.moe_forward_noalloc(ctypes.byref(_problem(t_cap=4)), None, NULL) == INVALID
    assert moe.NOALLOC_SCRATCH_BYTES == _header_macros("MOE_NOALLOC_")["MOE_NOALLOC_SCRATCH_BYTES"]


def test_batched_layout_validation(lib):
    lay = B._Layout()
    p = _problem(t_cap=512, expert_cap=64)
    assert lib.moe_workspace_plan(ctypes.byref(p), ctypes.byref(lay)) == OK
    assert lay.row_cap == 32 * 64
    assert lay.act == lay.status  # no decode path on the batched layout
    assert lay.overflow % 256 == 0 and lay.overflow + 4 <= lay.total
    assert lib.moe_workspace_plan(ctypes.byref(_problem(t_cap=512, expert_cap=64, row_cap=2047)),
                                  ctypes.byref(lay)) == INVALID
    assert lib.moe_workspace_plan(ctypes.byref(_problem(t_cap=512, expert_cap=-1)),
                                  ctypes.byref(lay)) == INVALID
    assert lib.moe_workspace_plan(ctypes.byref(_problem(expert_cap=1 << 26)), ctypes.byref(lay)) == INVALID
    # a decode-sized batched problem takes no decode path either
    pd = _problem(num_experts=288, hidden=4096, inter=512, t_cap=4, expert_cap=4)
    assert lib.moe_workspace_plan(ctypes.byref(pd), ctypes.byref(lay)) == OK and lay.act == lay.status
    fa = lib.moe_align_batched
    assert fa(FAKE, 4, NULL, 8, 32, 0, 0, FAKE, FAKE, FAKE, NULL, NULL) == INVALID   # cap 0
    assert fa(FAKE, 4, NULL, 8, 2000, 0, 4, FAKE, FAKE, FAKE, NULL, NULL) == UNSUPPORTED
    assert fa(FAKE, 4, NULL, 8, 32, 0, 4, NULL, FAKE, FAKE, NULL, NULL) == INVALID
    fg = lib.moe_grouped_gemm_fp8_masked
    assert fg(FAKE, FAKE, 0, 64, NULL, 1, FAKE, FAKE, FAKE, 4, 0, 256, 256, FAKE, NULL, NULL) == INVALID
    assert fg(FAKE, FAKE, 0, 64, NULL, 1, FAKE, FAKE, NULL, 4, 16, 256, 256, FAKE, NULL, NULL) == INVALID
    assert fg(FAKE, FAKE, 0, 64, NULL, 1, FAKE, FAKE, FAKE, 4, 16, 200, 256, FAKE, NULL, NULL) == INVALID
    fs = lib.moe_silu_mul_quant_masked
    assert fs(FAKE, 256, FAKE, 4, 0, 0, 7.0, 0, 0, FAKE, FAKE, NULL) == INVALID
    assert fs(FAKE, 256, FAKE, 2000, 4, 0, 7.0, 0, 0, FAKE, FAKE, NULL) == UNSUPPORTED
    assert fs(FAKE, 256, NULL, 4, 4, 0, 7.0, 0, 0, FAKE, FAKE, NULL) == INVALID


def test_silu_mul_quant_rejects_more_experts_than_its_table(lib):
    f = lib.moe_silu_mul_quant
    assert f(FAKE, 256, FAKE, FAKE, 1025, 64, 0, 7.0, 0, 0, FAKE, FAKE, NULL) == UNSUPPORTED


def test_mxfp4_gemm_validation(lib):
    f = lib.moe_grouped_gemm_mxfp4

    def call(n=256, k=256, fmt=0, div=1, e=4, rc=64, cap=0, a=FAKE, c=FAKE, w=FAKE, ws=FAKE,
             counts=FAKE, offsets=FAKE, a_rows=64, mr=0):
        return f(a, FAKE, fmt, a_rows, NULL, div, w, ws, counts, offsets, cap, e, rc, mr, n, k, c, NULL)
    assert call(n=200) == INVALID
    assert call(k=64) == INVALID
    assert call(fmt=7) == INVALID
    assert call(div=0) == INVALID
    assert call(e=0) == INVALID
    assert call(e=2000) == UNSUPPORTED
    assert call(a=NULL) == INVALID
    assert call(w=NULL) == INVALID
    assert call(ws=NULL) == INVALID
    assert call(counts=NULL) == INVALID
    assert call(offsets=NULL) == INVALID          # the aligned layout reads offsets
    assert call(a_rows=0) == INVALID              # rows to compute but no A rows
    assert call(cap=16, rc=63) == INVALID         # batched: row_cap must be E * cap
    assert call(cap=-1) == INVALID
    assert call(mr=-1) == INVALID
    assert call(rc=0, a=NULL, c=NULL) == OK


def test_forward_weight_format_field(lib):
    lay = B._Layout()
    assert lib.moe_workspace_plan(ctypes.byref(_problem(weight_fmt=2)), ctypes.byref(lay)) == INVALID
    assert lib.moe_workspace_plan(ctypes.byref(_problem(weight_fmt=1)), ctypes.byref(lay)) == OK
    # MXFP4 weights take the decode path's one-launch layer (the act rows are
    # laid out) when H and I are multiples of 256 (a stage is two K blocks),
    # and the general schedule otherwise
    pd = _problem(num_experts=288, hidden=4096, inter=512, t_cap=4, weight_fmt=1)
    assert lib.moe_workspace_plan(ctypes.byref(pd), ctypes.byref(lay)) == OK and lay.act < lay.status
    pd8 = _problem(num_experts=288, hidden=4096, inter=512, t_cap=4, weight_fmt=0)
    assert lib.moe_workspace_plan(ctypes.byref(pd8), ctypes.byref(lay)) == OK and lay.act < lay.status
    for h, i in ((4096 + 128, 512), (4096, 384), (256, 128)):
        pn = _problem(num_experts=64, hidden=h, inter=i, t_cap=4, weight_fmt=1)
        assert lib.moe_workspace_plan(ctypes.byref(pn), ctypes.byref(lay)) == OK and lay.act == lay.status, (h, i)
        pn8 = _problem(num_experts=64, hidden=h, inter=i, t_cap=4, weight_fmt=0)
        assert lib.moe_workspace_plan(ctypes.byref(pn8), ctypes.byref(lay)) == OK and lay.act < lay.status, (h, i)
    # FC1 of the decode path on its own serves FP8 weights only
    t = B._Tensors(*([FAKE.value] * 9))
    assert lib.moe_workspace_plan(ctypes.byref(pd), ctypes.byref(lay)) == OK
    assert lib.moe_fc1_decode(ctypes.byref(pd), ctypes.byref(t), FAKE, lay.total, NULL) == UNSUPPORTED
