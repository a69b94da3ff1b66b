"""ctypes marshalling for libmoefp8.so. No arithmetic of the layer lives here."""

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmoefp8.so"

SCALE_FMTS = {"fp32": 0, "pow2": 1, "ue8m0": 2}
ROUNDINGS = {"divide": 0, "reciprocal": 1}
ACTS = {"swiglu": 0, "swiglu_clamp": 1, "swiglu_clamp_after_silu": 2}
WEIGHT_FMTS = {"e4m3": 0, "mxfp4": 1}
# Row-tile geometry of the grouped GEMM (mirrors the header's macros), used to
# interpret the tiles_visited counter.
GEMM_TILES = {"stream_tile_m": 16, "stream_max_rows": 64, "tiled_tile_m": 256, "col_tile": 128}
# Limits of moe_forward's decode path and of its one-launch form (mirrors the
# header's MOE_DECODE_* macros).
DECODE_LIMITS = {"max_pairs": 64, "fc2_row_bytes": 24576, "fc2_max_scales": 256,
                 "layer_token_bytes": 61440, "layer_max_scales": 512}


def decode_layer_applies(t_cap, topk, hidden, inter, weight_fmt="e4m3"):
    """Whether moe_forward runs this problem (aligned layout) as its one-launch
    decode layer; with MXFP4 weights H and I must also be multiples of 256."""
    d, p = DECODE_LIMITS, t_cap * topk
    if _weight_fmt(weight_fmt) == 1 and (hidden % 256 or inter % 256):
        return False
    return (1 <= p <= d["max_pairs"] and p * (inter + 16) <= d["fc2_row_bytes"]
            and p * (inter // 128) <= d["fc2_max_scales"] and hidden % 16 == 0
            and t_cap * (hidden + 16) <= d["layer_token_bytes"]
            and t_cap * (hidden // 128) <= d["layer_max_scales"])

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "capacity too small",
           4: "HIP runtime error"}

_lock = threading.Lock()
_lib = None

_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_f32 = ctypes.c_float


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)} ({status})")


class _Problem(ctypes.Structure):
    _fields_ = [("num_experts", _i32), ("hidden", _i32), ("inter", _i32), ("topk", _i32),
                ("t_cap", _i32), ("align_rows", _i32), ("row_cap", _i32),
                ("scale_fmt", ctypes.c_int), ("act", ctypes.c_int), ("clamp_limit", _f32),
                ("rounding", ctypes.c_int), ("expert_start", _i32), ("expert_cap", _i32),
                ("weight_fmt", ctypes.c_int)]


class _Tensors(ctypes.Structure):
    _fields_ = [("x", _vp), ("topk_ids", _vp), ("topk_w", _vp), ("t_live_dev", _vp),
                ("w1", _vp), ("w1_scales", _vp), ("w2", _vp), ("w2_scales", _vp),
                ("out", _vp)]


class _Layout(ctypes.Structure):
    _fields_ = [("expert_counts", ctypes.c_size_t), ("expert_offsets", ctypes.c_size_t),
                ("row_to_pair", ctypes.c_size_t), ("pair_to_row", ctypes.c_size_t),
                ("xq", ctypes.c_size_t), ("xs", ctypes.c_size_t), ("c1", ctypes.c_size_t),
                ("hq", ctypes.c_size_t), ("hs", ctypes.c_size_t), ("y", ctypes.c_size_t),
                ("act", ctypes.c_size_t), ("status", ctypes.c_size_t),
                ("overflow", ctypes.c_size_t), ("total", ctypes.c_size_t), ("row_cap", _i32)]


_SIGNATURES = {
    "moe_min_row_cap": (_i32, [_i32, _i32, _i32, _i32]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_align": (ctypes.c_int, [_vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                 _vp]),
    "moe_align_batched": (ctypes.c_int, [_vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                         _vp, _vp]),
    "moe_grouped_gemm_mxfp4": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i32, _vp, _i32, _vp, _vp,
                                              _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp,
                                              _vp]),
    "moe_grouped_gemm_fp8_masked": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i32, _vp, _i32, _vp,
                                                   _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp,
                                                   _vp]),
    "moe_silu_mul_quant_masked": (ctypes.c_int, [_vp, _i32, _vp, _i32, _i32, ctypes.c_int, _f32,
                                                 ctypes.c_int, ctypes.c_int, _vp, _vp, _vp]),
    "moe_act_quant": (ctypes.c_int, [_vp, _i32, _vp, _i32, ctypes.c_int, ctypes.c_int, _vp, _vp,
                                     _vp]),
    "moe_grouped_gemm_fp8": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i32, _vp, _i32, _vp, _vp,
                                            _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                            _vp]),
    "moe_silu_mul_quant": (ctypes.c_int, [_vp, _i32, _vp, _vp, _i32, _i32, ctypes.c_int, _f32,
                                          ctypes.c_int, ctypes.c_int, _vp, _vp, _vp]),
    "moe_topk_combine": (ctypes.c_int, [_vp, _i32, _vp, _vp, _i32, _vp, _i32, _i32, _vp, _vp]),
    "moe_workspace_plan": (ctypes.c_int, [ctypes.POINTER(_Problem), ctypes.POINTER(_Layout)]),
    "moe_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(_Problem)]),
    "moe_forward": (ctypes.c_int, [ctypes.POINTER(_Problem), ctypes.POINTER(_Tensors), _vp,
                                   ctypes.c_size_t, _vp]),
    "moe_fc1_decode": (ctypes.c_int, [ctypes.POINTER(_Problem), ctypes.POINTER(_Tensors), _vp,
                                      ctypes.c_size_t, _vp]),
    "moe_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(_Problem), ctypes.POINTER(_Tensors), _vp]),
    "moe_barrier_timeouts": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32)]),
    "moe_barrier_spin_limit": (_i32, [_i32]),
}


def library_path():
    return os.path.join(_HERE, _LIB_NAME)


def load_library():
    """Load libmoefp8.so from the package directory (raises if it is not built)."""
    global _lib
    with _lock:
        if _lib is None:
            path = library_path()
            if not os.path.exists(path):
                raise ImportError(f"{path} is not built; run python -m block_fp8_mixture_amd.build")
            lib = ctypes.CDLL(path)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def _check(fn, status):
    if status != 0:
        raise MoeError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype, device=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    return t


def _shape(t, name, shape):
    """Raises ValueError unless tensor ``t`` has exactly ``shape``."""
    if tuple(t.shape) != tuple(int(d) for d in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _min_numel(t, name, n):
    if t.numel() < n:
        raise ValueError(f"{name} needs at least {n} elements, has {t.numel()}")
    return t


def _same_device(*tensors):
    """All given tensors on one GPU (checked after every shape, so shape errors
    are reported first)."""
    devs = {t.device for t in tensors if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors live on different devices: {sorted(map(str, devs))}")
    if any(d.type != "cuda" for d in devs):
        raise ValueError("tensors must be GPU tensors")


def _fmt(fmt):
    if fmt not in SCALE_FMTS:
        raise ValueError(f"scale format must be one of {list(SCALE_FMTS)}")
    return SCALE_FMTS[fmt]


def _rounding(rounding):
    if rounding not in ROUNDINGS:
        raise ValueError(f"rounding must be one of {list(ROUNDINGS)}")
    return ROUNDINGS[rounding]


def _scale_dtype(fmt):
    return torch.uint8 if fmt == "ue8m0" else torch.float32


def _live(t_live):
    if t_live is None:
        return None
    _need(t_live, "t_live", torch.int32)
    if t_live.numel() != 1 or not t_live.is_cuda:
        raise ValueError("t_live must be a one-element int32 GPU tensor")
    return _ptr(t_live)


def _bf16_view(t, name):
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return _need(t, name, torch.int16)


def moe_min_row_cap(t_cap, topk, num_experts, align_rows):
    return int(load_library().moe_min_row_cap(t_cap, topk, num_experts, align_rows))


def moe_status_string(status):
    return load_library().moe_status_string(status).decode()


def moe_align(topk_ids, num_experts, align_rows=16, row_cap=None, t_live=None, out=None,
              expert_start=0):
    """Routing alignment. Returns dict(counts, offsets, row_to_pair, pair_to_row).
    Local expert ids are ``topk_ids - expert_start``."""
    lib = load_library()
    ids = _need(topk_ids, "topk_ids", torch.int32, ndim=2)
    t_cap, topk = ids.shape
    if row_cap is None:
        row_cap = moe_min_row_cap(t_cap, topk, num_experts, align_rows)
    dev = ids.device
    if out is None:
        out = {
            "counts": torch.empty(num_experts, dtype=torch.int32, device=dev),
            "offsets": torch.empty(num_experts + 1, dtype=torch.int32, device=dev),
            "row_to_pair": torch.empty(max(row_cap, 1), dtype=torch.int32, device=dev),
            "pair_to_row": torch.empty(max(t_cap * topk, 1), dtype=torch.int32, device=dev),
        }
    for k, n in (("counts", num_experts), ("offsets", num_experts + 1),
                 ("row_to_pair", row_cap), ("pair_to_row", t_cap * topk)):
        _min_numel(_need(out[k], k, torch.int32), k, n)
    _same_device(ids, *out.values())
    st = lib.moe_align(_ptr(ids), t_cap, _live(t_live), topk, num_experts, expert_start,
                       align_rows, row_cap, _ptr(out["counts"]), _ptr(out["offsets"]),
                       _ptr(out["row_to_pair"]), _ptr(out["pair_to_row"]), _stream())
    _check("moe_align", st)
    return out


def moe_align_batched(topk_ids, num_experts, expert_cap, t_live=None, out=None, expert_start=0):
    """Routing into the batched masked-M layout ([E, expert_cap] rows). Returns
    dict(masked_m, row_to_pair, pair_to_row, overflow)."""
    lib = load_library()
    ids = _need(topk_ids, "topk_ids", torch.int32, ndim=2)
    t_cap, topk = ids.shape
    dev = ids.device
    if out is None:
        out = {
            "masked_m": torch.empty(num_experts, dtype=torch.int32, device=dev),
            "row_to_pair": torch.empty(max(num_experts * expert_cap, 1), dtype=torch.int32, device=dev),
            "pair_to_row": torch.empty(max(t_cap * topk, 1), dtype=torch.int32, device=dev),
            "overflow": torch.empty(1, dtype=torch.int32, device=dev),
        }
    for k, n in (("masked_m", num_experts), ("row_to_pair", num_experts * expert_cap),
                 ("pair_to_row", t_cap * topk), ("overflow", 1)):
        _min_numel(_need(out[k], k, torch.int32), k, n)
    _same_device(ids, *out.values())
    st = lib.moe_align_batched(_ptr(ids), t_cap, _live(t_live), topk, num_experts, expert_start,
                               expert_cap, _ptr(out["masked_m"]), _ptr(out["row_to_pair"]),
                               _ptr(out["pair_to_row"]), _ptr(out["overflow"]), _stream())
    _check("moe_align_batched", st)
    return out


def moe_act_quant(x, fmt="fp32", t_live=None, xq=None, xs=None, rounding="divide"):
    """Per-token 1x128 quantization. Returns (xq uint8 [t_cap, H], xs [H/128, t_cap])."""
    lib = load_library()
    xb = _bf16_view(x, "x")
    if xb.dim() != 2:
        raise ValueError("x must be [t_cap, hidden]")
    t_cap, hidden = xb.shape
    if xq is None:
        xq = torch.empty((t_cap, hidden), dtype=torch.uint8, device=xb.device)
    if xs is None:
        xs = torch.empty((hidden // 128, t_cap), dtype=_scale_dtype(fmt), device=xb.device)
    _shape(_need(xq, "xq", torch.uint8), "xq", (t_cap, hidden))
    _shape(_need(xs, "xs", _scale_dtype(fmt)), "xs", (hidden // 128, t_cap))
    _same_device(xb, xq, xs)
    st = lib.moe_act_quant(_ptr(xb), t_cap, _live(t_live), hidden, _fmt(fmt), _rounding(rounding),
                           _ptr(xq), _ptr(xs), _stream())
    _check("moe_act_quant", st)
    return xq, xs


def moe_grouped_gemm_fp8(a, a_scales, fmt, w, w_scales, counts, offsets, row_cap,
                         a_row_map=None, a_row_div=1, max_rows_per_expert=0, out=None,
                         tiles_visited=None):
    """Grouped FP8 GEMM over live rows. ``w`` is uint8 [E, N, K]; returns BF16 bits
    (int16) [row_cap, N]."""
    lib = load_library()
    _need(a, "a", torch.uint8, ndim=2)
    _need(a_scales, "a_scales", _scale_dtype(fmt), ndim=2)
    _need(w, "w", torch.uint8, ndim=3)
    _need(w_scales, "w_scales", torch.float32, ndim=3)
    num_experts, n, k = w.shape
    a_rows = a.shape[0]
    if a.shape[1] != k:
        raise ValueError("a and w disagree on K")
    _shape(a_scales, "a_scales", (k // 128, a_rows))
    _shape(w_scales, "w_scales", (num_experts, n // 128, k // 128))
    _shape(_need(counts, "counts", torch.int32), "counts", (num_experts,))
    _shape(_need(offsets, "offsets", torch.int32), "offsets", (num_experts + 1,))
    if out is None:
        out = torch.empty((max(row_cap, 1), n), dtype=torch.int16, device=a.device)
    ob = _bf16_view(out, "out")
    if ob.dim() != 2 or ob.shape[1] != n or ob.shape[0] < row_cap:
        raise ValueError(f"out must be [>= {row_cap}, {n}], got {tuple(ob.shape)}")
    if a_row_map is not None:
        _min_numel(_need(a_row_map, "a_row_map", torch.int32), "a_row_map", row_cap)
    elif a_rows < row_cap:
        raise ValueError("without a row map, a needs row_cap rows")
    if tiles_visited is not None:
        _min_numel(_need(tiles_visited, "tiles_visited", torch.int32), "tiles_visited", 1)
    _same_device(a, a_scales, w, w_scales, counts, offsets, ob, a_row_map, tiles_visited)
    st = lib.moe_grouped_gemm_fp8(_ptr(a), _ptr(a_scales), _fmt(fmt), a_rows, _ptr(a_row_map),
                                  a_row_div, _ptr(w), _ptr(w_scales), _ptr(counts),
                                  _ptr(offsets), num_experts, row_cap, max_rows_per_expert, n, k,
                                  _ptr(ob), _ptr(tiles_visited), _stream())
    _check("moe_grouped_gemm_fp8", st)
    return out


def moe_grouped_gemm_mxfp4(a, a_scales, fmt, w, w_scales, counts, offsets=None, row_cap=None,
                           a_row_map=None, a_row_div=1, expert_cap=0, max_rows_per_expert=0,
                           out=None):
    """Grouped GEMM with MXFP4 weights over live rows. ``w`` is uint8 [E, N, K/2]
    packed E2M1 codes, ``w_scales`` uint8 [E, N, K/32] E8M0 bytes. With
    ``expert_cap`` > 0 the batched layout (``counts`` = masked_m, no offsets,
    row_cap = E * expert_cap). Returns BF16 bits (int16) [row_cap, N]."""
    lib = load_library()
    _need(a, "a", torch.uint8, ndim=2)
    _need(a_scales, "a_scales", _scale_dtype(fmt), ndim=2)
    _need(w, "w", torch.uint8, ndim=3)
    _need(w_scales, "w_scales", torch.uint8, ndim=3)
    num_experts, n, k2 = w.shape
    k = 2 * k2
    a_rows = a.shape[0]
    if a.shape[1] != k:
        raise ValueError("a and w disagree on K")
    _shape(a_scales, "a_scales", (k // 128, a_rows))
    _shape(w_scales, "w_scales", (num_experts, n, k // 32))
    _shape(_need(counts, "counts", torch.int32), "counts", (num_experts,))
    if expert_cap > 0:
        row_cap = num_experts * expert_cap if row_cap is None else row_cap
        offsets = None
    else:
        if offsets is None or row_cap is None:
            raise ValueError("the aligned layout needs offsets and row_cap")
        _shape(_need(offsets, "offsets", torch.int32), "offsets", (num_experts + 1,))
    if out is None:
        out = torch.empty((max(row_cap, 1), n), dtype=torch.int16, device=a.device)
    ob = _bf16_view(out, "out")
    if ob.dim() != 2 or ob.shape[1] != n or ob.shape[0] < row_cap:
        raise ValueError(f"out must be [>= {row_cap}, {n}], got {tuple(ob.shape)}")
    if a_row_map is not None:
        _min_numel(_need(a_row_map, "a_row_map", torch.int32), "a_row_map", row_cap)
    elif a_rows < row_cap:
        raise ValueError("without a row map, a needs row_cap rows")
    _same_device(a, a_scales, w, w_scales, counts, offsets, ob, a_row_map)
    st = lib.moe_grouped_gemm_mxfp4(_ptr(a), _ptr(a_scales), _fmt(fmt), a_rows, _ptr(a_row_map),
                                    a_row_div, _ptr(w), _ptr(w_scales), _ptr(counts),
                                    _ptr(offsets), int(expert_cap), num_experts, row_cap,
                                    int(max_rows_per_expert), n, k, _ptr(ob), _stream())
    _check("moe_grouped_gemm_mxfp4", st)
    return out


def moe_grouped_gemm_fp8_masked(a, a_scales, fmt, w, w_scales, masked_m, expert_cap,
                                a_row_map=None, a_row_div=1, out=None, tiles_visited=None):
    """Grouped FP8 GEMM on the batched masked-M layout: expert e's live rows are
    [e*cap, e*cap + masked_m[e]). Returns BF16 bits (int16) [E*cap, N]."""
    lib = load_library()
    _need(a, "a", torch.uint8, ndim=2)
    _need(a_scales, "a_scales", _scale_dtype(fmt), ndim=2)
    _need(w, "w", torch.uint8, ndim=3)
    _need(w_scales, "w_scales", torch.float32, ndim=3)
    num_experts, n, k = w.shape
    rows = num_experts * expert_cap
    a_rows = a.shape[0]
    if a.shape[1] != k:
        raise ValueError("a and w disagree on K")
    _shape(a_scales, "a_scales", (k // 128, a_rows))
    _shape(w_scales, "w_scales", (num_experts, n // 128, k // 128))
    _shape(_need(masked_m, "masked_m", torch.int32), "masked_m", (num_experts,))
    if out is None:
        out = torch.empty((max(rows, 1), n), dtype=torch.int16, device=a.device)
    ob = _bf16_view(out, "out")
    if ob.dim() != 2 or ob.shape[1] != n or ob.shape[0] < rows:
        raise ValueError(f"out must be [>= {rows}, {n}], got {tuple(ob.shape)}")
    if a_row_map is not None:
        _min_numel(_need(a_row_map, "a_row_map", torch.int32), "a_row_map", rows)
    elif a_rows < rows:
        raise ValueError("without a row map, a needs num_experts * expert_cap rows")
    if tiles_visited is not None:
        _min_numel(_need(tiles_visited, "tiles_visited", torch.int32), "tiles_visited", 1)
    _same_device(a, a_scales, w, w_scales, masked_m, ob, a_row_map, tiles_visited)
    st = lib.moe_grouped_gemm_fp8_masked(_ptr(a), _ptr(a_scales), _fmt(fmt), a_rows,
                                         _ptr(a_row_map), a_row_div, _ptr(w), _ptr(w_scales),
                                         _ptr(masked_m), num_experts, expert_cap, n, k, _ptr(ob),
                                         _ptr(tiles_visited), _stream())
    _check("moe_grouped_gemm_fp8_masked", st)
    return out


def moe_silu_mul_quant_masked(gate_up, masked_m, expert_cap, act="swiglu",
                              clamp_limit=float("inf"), fmt="fp32", hq=None, hs=None,
                              rounding="divide"):
    """SiLU(gate)*up + 1x128 FP8 quantization on the batched masked-M layout.
    Returns (hq uint8 [E*cap, I], hs [I/128, E*cap])."""
    lib = load_library()
    gu = _bf16_view(gate_up, "gate_up")
    _need(masked_m, "masked_m", torch.int32, ndim=1)
    num_experts = masked_m.shape[0]
    rows = num_experts * expert_cap
    if gu.dim() != 2 or gu.shape[1] % 2 or gu.shape[0] != rows:
        raise ValueError(f"gate_up must be [{rows}, 2 * inter], got {tuple(gu.shape)}")
    inter = gu.shape[1] // 2
    if hq is None:
        hq = torch.empty((rows, inter), dtype=torch.uint8, device=gu.device)
    if hs is None:
        hs = torch.empty((inter // 128, rows), dtype=_scale_dtype(fmt), device=gu.device)
    _shape(_need(hq, "hq", torch.uint8), "hq", (rows, inter))
    _shape(_need(hs, "hs", _scale_dtype(fmt)), "hs", (inter // 128, rows))
    _same_device(gu, masked_m, hq, hs)
    if act not in ACTS:
        raise ValueError(f"act must be one of {list(ACTS)}")
    st = lib.moe_silu_mul_quant_masked(_ptr(gu), inter, _ptr(masked_m), num_experts, expert_cap,
                                       ACTS[act], float(clamp_limit), _fmt(fmt),
                                       _rounding(rounding), _ptr(hq), _ptr(hs), _stream())
    _check("moe_silu_mul_quant_masked", st)
    return hq, hs


def moe_silu_mul_quant(gate_up, counts, offsets, act="swiglu", clamp_limit=float("inf"),
                       fmt="fp32", hq=None, hs=None, rounding="divide"):
    """SiLU(gate)*up + 1x128 FP8 quantization of live rows.
    Returns (hq uint8 [row_cap, I], hs [I/128, row_cap])."""
    lib = load_library()
    gu = _bf16_view(gate_up, "gate_up")
    if gu.dim() != 2 or gu.shape[1] % 2:
        raise ValueError("gate_up must be [row_cap, 2 * inter]")
    row_cap, two_i = gu.shape
    inter = two_i // 2
    _need(counts, "counts", torch.int32, ndim=1)
    num_experts = counts.shape[0]
    _shape(_need(offsets, "offsets", torch.int32), "offsets", (num_experts + 1,))
    if hq is None:
        hq = torch.empty((row_cap, inter), dtype=torch.uint8, device=gu.device)
    if hs is None:
        hs = torch.empty((inter // 128, row_cap), dtype=_scale_dtype(fmt), device=gu.device)
    _shape(_need(hq, "hq", torch.uint8), "hq", (row_cap, inter))
    _shape(_need(hs, "hs", _scale_dtype(fmt)), "hs", (inter // 128, row_cap))
    _same_device(gu, counts, offsets, hq, hs)
    if act not in ACTS:
        raise ValueError(f"act must be one of {list(ACTS)}")
    st = lib.moe_silu_mul_quant(_ptr(gu), inter, _ptr(counts), _ptr(offsets), num_experts,
                                row_cap, ACTS[act], float(clamp_limit), _fmt(fmt),
                                _rounding(rounding), _ptr(hq), _ptr(hs), _stream())
    _check("moe_silu_mul_quant", st)
    return hq, hs


def moe_topk_combine(y, pair_to_row, topk_w, t_live=None, out=None):
    """Top-k weighted sum of expert rows. Returns BF16 bits (int16) [t_cap, H]."""
    lib = load_library()
    yb = _bf16_view(y, "y")
    if yb.dim() != 2:
        raise ValueError("y must be [row_cap, hidden]")
    row_cap, hidden = yb.shape
    w = _need(topk_w, "topk_w", torch.float32, ndim=2)
    t_cap, topk = w.shape
    _min_numel(_need(pair_to_row, "pair_to_row", torch.int32), "pair_to_row", t_cap * topk)
    if out is None:
        out = torch.empty((t_cap, hidden), dtype=torch.int16, device=yb.device)
    ob = _shape(_bf16_view(out, "out"), "out", (t_cap, hidden))
    _same_device(yb, pair_to_row, w, ob)
    st = lib.moe_topk_combine(_ptr(yb), row_cap, _ptr(pair_to_row), _ptr(w), t_cap, _live(t_live),
                              topk, hidden, _ptr(ob), _stream())
    _check("moe_topk_combine", st)
    return out


def _weight_fmt(weight_fmt):
    if weight_fmt not in WEIGHT_FMTS:
        raise ValueError(f"weight_fmt must be one of {list(WEIGHT_FMTS)}")
    return WEIGHT_FMTS[weight_fmt]


def _problem(num_experts, hidden, inter, topk, t_cap, align_rows, row_cap, fmt, act, clamp_limit,
             rounding="divide", expert_start=0, expert_cap=0, weight_fmt="e4m3"):
    if act not in ACTS:
        raise ValueError(f"act must be one of {list(ACTS)}")
    return _Problem(num_experts, hidden, inter, topk, t_cap, align_rows, row_cap or 0, _fmt(fmt),
                    ACTS[act], float(clamp_limit), _rounding(rounding), int(expert_start),
                    int(expert_cap), _weight_fmt(weight_fmt))


def moe_workspace_plan(num_experts, hidden, inter, topk, t_cap, align_rows=16, row_cap=0,
                       fmt="fp32", act="swiglu", clamp_limit=float("inf"), rounding="divide",
                       expert_start=0, expert_cap=0, weight_fmt="e4m3"):
    """Byte offsets of every intermediate in the forward workspace (dict)."""
    lib = load_library()
    prob = _problem(num_experts, hidden, inter, topk, t_cap, align_rows, row_cap, fmt, act,
                    clamp_limit, rounding, expert_start, expert_cap, weight_fmt)
    lay = _Layout()
    _check("moe_workspace_plan", lib.moe_workspace_plan(ctypes.byref(prob), ctypes.byref(lay)))
    return {name: getattr(lay, name) for name, _ in _Layout._fields_}


def moe_workspace_bytes(num_experts, hidden, inter, topk, t_cap, align_rows=16, row_cap=0,
                        fmt="fp32", act="swiglu", clamp_limit=float("inf"), rounding="divide",
                        expert_start=0, expert_cap=0, weight_fmt="e4m3"):
    lib = load_library()
    prob = _problem(num_experts, hidden, inter, topk, t_cap, align_rows, row_cap, fmt, act,
                    clamp_limit, rounding, expert_start, expert_cap, weight_fmt)
    return int(lib.moe_workspace_bytes(ctypes.byref(prob)))


def _check_layer_tensors(xb, topk_ids, w1, w1_scales, w2=None, w2_scales=None, weight_fmt="e4m3"):
    """Shapes and devices of the layer's inputs; returns (num_experts, inter, topk)."""
    t_cap, hidden = xb.shape
    _weight_fmt(weight_fmt)
    mx = weight_fmt == "mxfp4"
    _need(topk_ids, "topk_ids", torch.int32, ndim=2)
    if topk_ids.shape[0] != t_cap:
        raise ValueError(f"topk_ids has {topk_ids.shape[0]} rows, x has {t_cap}")
    _need(w1, "w1", torch.uint8, ndim=3)
    num_experts, two_i, h1 = w1.shape
    if h1 != (hidden // 2 if mx else hidden) or two_i % 256:
        raise ValueError(f"w1 must be [E, 2*inter, {hidden // 2 if mx else hidden}], got {tuple(w1.shape)}")
    inter = two_i // 2
    if mx:
        _shape(_need(w1_scales, "w1_scales", torch.uint8), "w1_scales", (num_experts, two_i, hidden // 32))
    else:
        _shape(_need(w1_scales, "w1_scales", torch.float32), "w1_scales",
               (num_experts, two_i // 128, hidden // 128))
    if w2 is not None:
        if mx:
            _shape(_need(w2, "w2", torch.uint8), "w2", (num_experts, hidden, inter // 2))
            _shape(_need(w2_scales, "w2_scales", torch.uint8), "w2_scales",
                   (num_experts, hidden, inter // 32))
        else:
            _shape(_need(w2, "w2", torch.uint8), "w2", (num_experts, hidden, inter))
            _shape(_need(w2_scales, "w2_scales", torch.float32), "w2_scales",
                   (num_experts, hidden // 128, inter // 128))
    return num_experts, inter, topk_ids.shape[1]


def moe_forward(x, topk_ids, topk_w, w1, w1_scales, w2, w2_scales, fmt="fp32", act="swiglu",
                clamp_limit=float("inf"), align_rows=16, row_cap=0, t_live=None, out=None,
                workspace=None, rounding="divide", expert_start=0, expert_cap=0,
                weight_fmt="e4m3"):
    """The whole expert layer. Returns (out BF16 bits int16 [t_cap, H], workspace uint8).
    ``topk_w=None`` weights every routed pair by one. ``weight_fmt="mxfp4"``:
    w1/w2 are packed E2M1 codes [E, rows, cols/2] with E8M0 scale bytes
    [E, rows, cols/32]."""
    lib = load_library()
    xb = _bf16_view(x, "x")
    if xb.dim() != 2:
        raise ValueError("x must be [t_cap, hidden]")
    t_cap, hidden = xb.shape
    num_experts, inter, topk = _check_layer_tensors(xb, topk_ids, w1, w1_scales, w2, w2_scales,
                                                    weight_fmt)
    if topk_w is None:
        topk_w = torch.ones((t_cap, topk), dtype=torch.float32, device=xb.device)
    _shape(_need(topk_w, "topk_w", torch.float32), "topk_w", (t_cap, topk))
    prob = _problem(num_experts, hidden, inter, topk, t_cap, align_rows, row_cap, fmt, act,
                    clamp_limit, rounding, expert_start, expert_cap, weight_fmt)
    need = int(lib.moe_workspace_bytes(ctypes.byref(prob)))
    if need == 0:
        lay = _Layout()
        _check("moe_workspace_plan", lib.moe_workspace_plan(ctypes.byref(prob), ctypes.byref(lay)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=xb.device)
    _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty((t_cap, hidden), dtype=torch.int16, device=xb.device)
    ob = _shape(_bf16_view(out, "out"), "out", (t_cap, hidden))
    if t_live is not None:
        _shape(_need(t_live, "t_live", torch.int32), "t_live", (1,))
    _same_device(xb, topk_ids, topk_w, w1, w1_scales, w2, w2_scales, ob, workspace, t_live)
    tens = _Tensors(_ptr(xb), _ptr(topk_ids), _ptr(topk_w), _live(t_live), _ptr(w1),
                    _ptr(w1_scales), _ptr(w2), _ptr(w2_scales), _ptr(ob))
    st = lib.moe_forward(ctypes.byref(prob), ctypes.byref(tens), _ptr(workspace),
                         workspace.numel(), _stream())
    _check("moe_forward", st)
    return out, workspace


# Bytes of the library's static workspace behind moe_forward_noalloc (mirrors
# the header's MOE_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


def moe_forward_noalloc(x, topk_ids, topk_w, w1, w1_scales, w2, w2_scales, fmt="fp32",
                        act="swiglu", clamp_limit=float("inf"), align_rows=16, row_cap=0,
                        t_live=None, out=None, rounding="divide", expert_start=0, expert_cap=0,
                        weight_fmt="e4m3"):
    """moe_forward with the library's static per-device workspace instead of a
    caller buffer (for callers that cannot allocate; the call allocates nothing
    when ``out`` and ``topk_w`` are given). Calls on one device must not overlap.
    Returns out (BF16 bits int16 [t_cap, H])."""
    lib = load_library()
    xb = _bf16_view(x, "x")
    if xb.dim() != 2:
        raise ValueError("x must be [t_cap, hidden]")
    t_cap, hidden = xb.shape
    num_experts, inter, topk = _check_layer_tensors(xb, topk_ids, w1, w1_scales, w2, w2_scales,
                                                    weight_fmt)
    if topk_w is None:
        topk_w = torch.ones((t_cap, topk), dtype=torch.float32, device=xb.device)
    _shape(_need(topk_w, "topk_w", torch.float32), "topk_w", (t_cap, topk))
    if out is None:
        out = torch.empty((t_cap, hidden), dtype=torch.int16, device=xb.device)
    ob = _shape(_bf16_view(out, "out"), "out", (t_cap, hidden))
    if t_live is not None:
        _shape(_need(t_live, "t_live", torch.int32), "t_live", (1,))
    _same_device(xb, topk_ids, topk_w, w1, w1_scales, w2, w2_scales, ob, t_live)
    prob = _problem(num_experts, hidden, inter, topk, t_cap, align_rows, row_cap, fmt, act,
                    clamp_limit, rounding, expert_start, expert_cap, weight_fmt)
    tens = _Tensors(_ptr(xb), _ptr(topk_ids), _ptr(topk_w), _live(t_live), _ptr(w1),
                    _ptr(w1_scales), _ptr(w2), _ptr(w2_scales), _ptr(ob))
    _check("moe_forward_noalloc", lib.moe_forward_noalloc(ctypes.byref(prob), ctypes.byref(tens),
                                                          _stream()))
    return out


def moe_fc1_decode(x, topk_ids, w1, w1_scales, inter, fmt="fp32", act="swiglu",
                   clamp_limit=float("inf"), align_rows=16, row_cap=0, t_live=None,
                   workspace=None, rounding="divide", expert_start=0):
    """The decode path's first launch alone (routing, activation quantization and
    FC1 with SiLU(gate)*up), writing moe_forward's workspace. Returns the workspace."""
    lib = load_library()
    xb = _bf16_view(x, "x")
    if xb.dim() != 2:
        raise ValueError("x must be [t_cap, hidden]")
    t_cap, hidden = xb.shape
    num_experts, w_inter, topk = _check_layer_tensors(xb, topk_ids, w1, w1_scales)
    if w_inter != inter:
        raise ValueError("w1 shape disagrees with inter")
    prob = _problem(num_experts, hidden, inter, topk, t_cap, align_rows, row_cap,
                    fmt, act, clamp_limit, rounding, expert_start)
    need = int(lib.moe_workspace_bytes(ctypes.byref(prob)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=xb.device)
    _need(workspace, "workspace", torch.uint8)
    if t_live is not None:
        _shape(_need(t_live, "t_live", torch.int32), "t_live", (1,))
    _same_device(xb, topk_ids, w1, w1_scales, workspace, t_live)
    tens = _Tensors(_ptr(xb), _ptr(topk_ids), None, _live(t_live), _ptr(w1), _ptr(w1_scales),
                    None, None, None)
    st = lib.moe_fc1_decode(ctypes.byref(prob), ctypes.byref(tens), _ptr(workspace),
                            workspace.numel(), _stream())
    _check("moe_fc1_decode", st)
    return workspace


def moe_barrier_timeouts():
    """Waits at the one-launch decode layer's grid barrier that gave up on the
    current device (sticky count; nonzero means some launch's outputs are unreliable)."""
    lib = load_library()
    n = ctypes.c_uint32(0)
    _check("moe_barrier_timeouts", lib.moe_barrier_timeouts(ctypes.byref(n)))
    return int(n.value)


def moe_barrier_spin_limit(polls):
    """Sets the polls per wait of the one-launch decode layer's grid barrier for
    later launches (negative: every wait gives up at once); returns the old value."""
    return int(load_library().moe_barrier_spin_limit(int(polls)))
