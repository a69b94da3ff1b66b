"""Host-only checks of the Python binding: every wrapper validates shapes,
dtypes and devices of its tensors and raises ValueError before anything is
enqueued (so a mismatched tensor can never become an out-of-bounds device
access), and moe_forward accepts topk_w=None. CPU tensors stand in for device
tensors: the shape checks come first, the GPU check last."""

import pytest
import torch

import block_fp8_mixture_amd as moe

E, H, I, K, T = 4, 256, 128, 2, 8


def _layer(**over):
    t = dict(
        x=torch.zeros((T, H), dtype=torch.bfloat16),
        topk_ids=torch.zeros((T, K), dtype=torch.int32),
        topk_w=torch.ones((T, K), dtype=torch.float32),
        w1=torch.zeros((E, 2 * I, H), dtype=torch.uint8),
        w1_scales=torch.ones((E, 2 * I // 128, H // 128), dtype=torch.float32),
        w2=torch.zeros((E, H, I), dtype=torch.uint8),
        w2_scales=torch.ones((E, H // 128, I // 128), dtype=torch.float32),
    )
    t.update(over)
    return t


def _forward(**over):
    t = _layer(**over)
    return moe.moe_forward(t["x"], t["topk_ids"], t["topk_w"], t["w1"], t["w1_scales"], t["w2"],
                           t["w2_scales"])


@pytest.mark.parametrize("name,bad", [
    ("topk_ids", torch.zeros((T + 1, K), dtype=torch.int32)),
    ("topk_w", torch.ones((T, K + 1), dtype=torch.float32)),
    ("w1", torch.zeros((E, 2 * I, H + 128), dtype=torch.uint8)),
    ("w1_scales", torch.ones((E, 2 * I // 128, H // 128 + 1), dtype=torch.float32)),
    ("w2", torch.zeros((E, H, 2 * I), dtype=torch.uint8)),
    ("w2_scales", torch.ones((E + 1, H // 128, I // 128), dtype=torch.float32)),
])
def test_forward_rejects_mismatched_shapes(name, bad):
    with pytest.raises(ValueError):
        _forward(**{name: bad})


def test_forward_accepts_none_weights_and_then_requires_gpu_tensors():
    # topk_w=None is substituted by ones; with every shape right, the only
    # remaining complaint for CPU tensors is the device.
    with pytest.raises(ValueError, match="GPU"):
        _forward(topk_w=None)


def test_forward_rejects_wrong_out_shape():
    t = _layer()
    with pytest.raises(ValueError, match="out"):
        moe.moe_forward(t["x"], t["topk_ids"], t["topk_w"], t["w1"], t["w1_scales"], t["w2"],
                        t["w2_scales"], out=torch.zeros((T, H + 1), dtype=torch.int16))


def test_gemm_rejects_mismatched_shapes():
    a = torch.zeros((64, 256), dtype=torch.uint8)
    sa = torch.ones((2, 64), dtype=torch.float32)
    w = torch.zeros((3, 128, 256), dtype=torch.uint8)
    ws = torch.ones((3, 1, 2), dtype=torch.float32)
    cnt = torch.zeros(3, dtype=torch.int32)
    off = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="a_scales"):
        moe.moe_grouped_gemm_fp8(a, torch.ones((2, 63), dtype=torch.float32), "fp32", w, ws, cnt,
                                 off, 64)
    with pytest.raises(ValueError, match="w_scales"):
        moe.moe_grouped_gemm_fp8(a, sa, "fp32", w, torch.ones((3, 2, 2), dtype=torch.float32), cnt,
                                 off, 64)
    with pytest.raises(ValueError, match="counts"):
        moe.moe_grouped_gemm_fp8(a, sa, "fp32", w, ws, torch.zeros(2, dtype=torch.int32), off, 64)
    with pytest.raises(ValueError, match="offsets"):
        moe.moe_grouped_gemm_fp8(a, sa, "fp32", w, ws, cnt, torch.zeros(3, dtype=torch.int32), 64)
    with pytest.raises(ValueError, match="out"):
        moe.moe_grouped_gemm_fp8(a, sa, "fp32", w, ws, cnt, off, 64,
                                 out=torch.zeros((63, 128), dtype=torch.int16))
    with pytest.raises(ValueError, match="row map"):
        moe.moe_grouped_gemm_fp8(a, sa, "fp32", w, ws, cnt, off, 65)
    with pytest.raises(ValueError, match="a_row_map"):
        moe.moe_grouped_gemm_fp8(a, sa, "fp32", w, ws, cnt, off, 80,
                                 a_row_map=torch.zeros(79, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        moe.moe_grouped_gemm_fp8(a, sa, "fp32", w, ws, cnt, off, 64)


def test_stage_wrappers_reject_mismatched_shapes():
    x = torch.zeros((T, H), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="xs"):
        moe.moe_act_quant(x, "fp32", xs=torch.ones((H // 128, T + 1), dtype=torch.float32))
    with pytest.raises(ValueError, match="xq"):
        moe.moe_act_quant(x, "fp32", xq=torch.zeros((T, H - 1), dtype=torch.uint8))
    gu = torch.zeros((32, 2 * I), dtype=torch.bfloat16)
    cnt = torch.zeros(E, dtype=torch.int32)
    with pytest.raises(ValueError, match="offsets"):
        moe.moe_silu_mul_quant(gu, cnt, torch.zeros(E, dtype=torch.int32))
    with pytest.raises(ValueError, match="hs"):
        moe.moe_silu_mul_quant(gu, cnt, torch.zeros(E + 1, dtype=torch.int32),
                               hs=torch.ones((1, 31), dtype=torch.float32))
    y = torch.zeros((32, H), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="pair_to_row"):
        moe.moe_topk_combine(y, torch.zeros(T * K - 1, dtype=torch.int32),
                             torch.ones((T, K), dtype=torch.float32))
    with pytest.raises(ValueError, match="out"):
        moe.moe_topk_combine(y, torch.zeros(T * K, dtype=torch.int32),
                             torch.ones((T, K), dtype=torch.float32),
                             out=torch.zeros((T, H + 1), dtype=torch.int16))
    ids = torch.zeros((T, K), dtype=torch.int32)
    with pytest.raises(ValueError, match="row_to_pair"):
        moe.moe_align(ids, E, 16, row_cap=64,
                      out={"counts": torch.zeros(E, dtype=torch.int32),
                           "offsets": torch.zeros(E + 1, dtype=torch.int32),
                           "row_to_pair": torch.zeros(63, dtype=torch.int32),
                           "pair_to_row": torch.zeros(T * K, dtype=torch.int32)})


def test_workspace_plan_lays_out_barrier_status_slots():
    for t_cap, h, i in [(4, 4096, 512), (4096, 7168, 2048)]:
        lay = moe.moe_workspace_plan(288, h, i, 8, t_cap)
        assert lay["status"] % 256 == 0
        assert lay["status"] >= lay["y"] + lay["row_cap"] * h * 2
        assert lay["status"] + 1024 * 4 <= lay["total"]
        if lay["act"] < lay["status"]:  # the decode path's act buffer
            assert lay["status"] >= lay["act"] + lay["row_cap"] * i * 4
        else:
            assert lay["act"] == lay["status"]


def test_spin_limit_round_trips():
    old = moe.moe_barrier_spin_limit(-1)
    try:
        assert moe.moe_barrier_spin_limit(123) == -1
        assert moe.moe_barrier_spin_limit(old) == 123
    finally:
        moe.moe_barrier_spin_limit(old)
    assert old == 1 << 21


def _mx_layer(**over):
    t = dict(
        w1=torch.zeros((E, 2 * I, H // 2), dtype=torch.uint8),
        w1_scales=torch.full((E, 2 * I, H // 32), 127, dtype=torch.uint8),
        w2=torch.zeros((E, H, I // 2), dtype=torch.uint8),
        w2_scales=torch.full((E, H, I // 32), 127, dtype=torch.uint8),
    )
    t.update(over)
    return _layer(**t)


@pytest.mark.parametrize("name,bad", [
    ("w1", torch.zeros((E, 2 * I, H), dtype=torch.uint8)),              # FP8 width
    ("w1_scales", torch.ones((E, 2 * I // 128, H // 128), dtype=torch.float32)),
    ("w2", torch.zeros((E, H, I), dtype=torch.uint8)),
    ("w2_scales", torch.full((E, H, I // 32 + 1), 127, dtype=torch.uint8)),
])
def test_mxfp4_forward_rejects_mismatched_shapes(name, bad):
    t = _mx_layer(**{name: bad})
    with pytest.raises((ValueError, TypeError)):  # a wrong dtype is a TypeError
        moe.moe_forward(t["x"], t["topk_ids"], t["topk_w"], t["w1"], t["w1_scales"], t["w2"],
                        t["w2_scales"], weight_fmt="mxfp4")


def test_mxfp4_forward_shapes_pass_and_then_require_gpu_tensors():
    t = _mx_layer()
    with pytest.raises(ValueError, match="GPU"):
        moe.moe_forward(t["x"], t["topk_ids"], t["topk_w"], t["w1"], t["w1_scales"], t["w2"],
                        t["w2_scales"], weight_fmt="mxfp4")
    with pytest.raises(ValueError, match="weight_fmt"):
        moe.moe_forward(t["x"], t["topk_ids"], t["topk_w"], t["w1"], t["w1_scales"], t["w2"],
                        t["w2_scales"], weight_fmt="fp4")


def test_mxfp4_gemm_rejects_mismatched_shapes():
    a = torch.zeros((64, 256), dtype=torch.uint8)
    sa = torch.ones((2, 64), dtype=torch.float32)
    w = torch.zeros((3, 128, 128), dtype=torch.uint8)
    ws = torch.full((3, 128, 8), 127, dtype=torch.uint8)
    cnt = torch.zeros(3, dtype=torch.int32)
    off = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="K"):
        moe.moe_grouped_gemm_mxfp4(torch.zeros((64, 128), dtype=torch.uint8), sa, "fp32", w, ws,
                                   cnt, off, 64)
    with pytest.raises(ValueError, match="w_scales"):
        moe.moe_grouped_gemm_mxfp4(a, sa, "fp32", w, torch.full((3, 128, 2), 127, dtype=torch.uint8),
                                   cnt, off, 64)
    with pytest.raises(TypeError, match="w_scales"):
        moe.moe_grouped_gemm_mxfp4(a, sa, "fp32", w, ws.float(), cnt, off, 64)
    with pytest.raises(ValueError, match="offsets"):
        moe.moe_grouped_gemm_mxfp4(a, sa, "fp32", w, ws, cnt, None, 64)
    with pytest.raises(ValueError, match="out"):
        moe.moe_grouped_gemm_mxfp4(a, sa, "fp32", w, ws, cnt, off, 64,
                                   out=torch.zeros((64, 127), dtype=torch.int16))
    with pytest.raises(ValueError, match="GPU"):
        moe.moe_grouped_gemm_mxfp4(a, sa, "fp32", w, ws, cnt, off, 64)
    with pytest.raises(ValueError, match="GPU"):  # batched: counts = masked_m, no offsets
        moe.moe_grouped_gemm_mxfp4(a, sa, "fp32", w, ws, cnt, expert_cap=16)
