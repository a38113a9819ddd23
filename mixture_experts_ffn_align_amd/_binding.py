"""ctypes binding over libmoe_ffn.so (the C ABI declared in include/moe_ffn.h).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch supplies device memory and the current stream. If the library has
not been built this module raises on first use; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; MOE_FFN_LIBRARY names another build of the same sources
# (the host-sanitizer build of the tests, for one).
LIB_PATH = os.environ.get("MOE_FFN_LIBRARY") or os.path.join(_PKG, "libmoe_ffn.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "moe_ffn.h")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_CAPACITY = 3
MOE_ERR_WORKSPACE = 4
MOE_ERR_HIP = 5

MOE_W_INT4_AWQ = 0
MOE_W_MXFP8 = 1

MOE_PATH_AUTO = 0
MOE_PATH_DECODE = 1
MOE_PATH_GROUPED = 2

_c_i32 = ctypes.c_int32
_c_size = ctypes.c_size_t
_c_ptr = ctypes.c_void_p


class moe_weights(ctypes.Structure):
    _fields_ = [("fmt", _c_i32), ("group", _c_i32), ("q", _c_ptr), ("scale", _c_ptr),
                ("zero", _c_ptr)]


class moe_ffn_desc(ctypes.Structure):
    _fields_ = [("M", _c_i32), ("H", _c_i32), ("I", _c_i32), ("E", _c_i32), ("k", _c_i32),
                ("b", _c_i32), ("w13", moe_weights), ("w2", moe_weights), ("path", _c_i32),
                ("max_workgroups", _c_i32), ("expert_base", _c_i32)]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        super().__init__(f"{where}: {status_str(status)} (status {status})")


_SIGNATURES = {
    "moe_align_capacity": (_c_size, [_c_i32, _c_i32, _c_i32, _c_i32]),
    "moe_align": (_c_i32, [_c_ptr, _c_i32, _c_i32, _c_i32, _c_i32, _c_ptr, _c_ptr, _c_ptr,
                           _c_size, _c_ptr]),
    "moe_align_ex": (_c_i32, [_c_ptr, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_ptr, _c_ptr, _c_ptr,
                              _c_size, _c_ptr, _c_size, _c_ptr]),
    "moe_align_ex_workspace_size": (_c_i32, [_c_i32, _c_i32, _c_i32, ctypes.POINTER(_c_size)]),
    "moe_ffn_workspace_size": (_c_i32, [ctypes.POINTER(moe_ffn_desc), ctypes.POINTER(_c_size)]),
    "moe_ffn_forward": (_c_i32, [ctypes.POINTER(moe_ffn_desc), _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                 _c_ptr, _c_size, _c_ptr]),
    "moe_ffn_forward_aligned": (_c_i32, [ctypes.POINTER(moe_ffn_desc), _c_ptr, _c_ptr, _c_ptr,
                                         _c_ptr, _c_ptr, _c_ptr, _c_size, _c_ptr, _c_ptr,
                                         _c_size, _c_ptr]),
    "moe_ffn_forward_noalloc": (_c_i32, [ctypes.POINTER(moe_ffn_desc), _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                         _c_ptr]),
    "moe_ffn_noalloc_max_bytes": (_c_size, []),
    "moe_ffn_forward_capture": (_c_i32, [ctypes.POINTER(moe_ffn_desc), _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                         _c_ptr, _c_size, _c_ptr, _c_ptr]),
    "moe_ffn_forward_profiled": (_c_i32, [ctypes.POINTER(moe_ffn_desc), _c_ptr, _c_ptr, _c_ptr,
                                          _c_ptr, _c_ptr, _c_size, _c_ptr,
                                          ctypes.POINTER(_c_ptr), _c_i32]),
    "moe_ffn_gate_up": (_c_i32, [ctypes.POINTER(moe_ffn_desc), _c_ptr, _c_ptr, _c_ptr, _c_size,
                                 _c_ptr]),
    "moe_ffn_down_combine": (_c_i32, [ctypes.POINTER(moe_ffn_desc), _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                      _c_size, _c_ptr]),
    "moe_ffn_gate_up_batched": (_c_i32, [ctypes.POINTER(moe_ffn_desc), _c_ptr, _c_ptr, _c_i32, _c_ptr,
                                         _c_ptr, _c_ptr]),
    "moe_ffn_down_batched": (_c_i32, [ctypes.POINTER(moe_ffn_desc), _c_ptr, _c_ptr, _c_ptr, _c_i32,
                                      _c_ptr, _c_ptr]),
    "moe_ffn_kernel_count": (_c_i32, [ctypes.POINTER(moe_ffn_desc)]),
    "moe_ffn_kernel_name": (ctypes.c_char_p, [ctypes.POINTER(moe_ffn_desc), _c_i32]),
    "moe_ffn_intermediate": (_c_i32, [ctypes.POINTER(moe_ffn_desc), ctypes.POINTER(_c_size),
                                      ctypes.POINTER(_c_size), ctypes.POINTER(_c_i32)]),
    "moe_ffn_route_outputs": (_c_i32, [ctypes.POINTER(moe_ffn_desc), ctypes.POINTER(_c_size)]),
    "moe_ffn_auto_decode_max_m": (_c_i32, []),
    "moe_ffn_resolved_path": (_c_i32, [ctypes.POINTER(moe_ffn_desc)]),
    "moe_status_str": (ctypes.c_char_p, [_c_i32]),
}

_lib = None
_bench_lib = None
BENCH_LIB_PATH = os.path.join(_PKG, "libmoe_bench.so")
BENCH_HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "moe_bench.h")
_BENCH_SIGNATURES = {
    "moe_bench_stream_read": (_c_i32, [_c_ptr, _c_size, _c_ptr, _c_i32, _c_i32, ctypes.POINTER(_c_i32), _c_ptr,
                                       _c_ptr, _c_ptr]),
    "moe_bench_copy": (_c_i32, [_c_ptr, _c_ptr, _c_size, _c_i32, _c_ptr, _c_ptr, _c_ptr]),
    "moe_bench_mfma": (_c_i32, [_c_i32, _c_i32, _c_i32, _c_i32, _c_ptr, ctypes.POINTER(ctypes.c_double), _c_ptr,
                                _c_ptr, _c_ptr]),
}


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mixture_experts_ffn_align_amd.build` (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def bench_lib() -> ctypes.CDLL:
    """The measurement kernels (include/moe_bench.h); raises if not built."""
    global _bench_lib
    if _bench_lib is None:
        if not os.path.exists(BENCH_LIB_PATH):
            raise RuntimeError(f"{BENCH_LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_ffn_align_amd.build`")
        L = ctypes.CDLL(BENCH_LIB_PATH)
        for name, (res, args) in _BENCH_SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _bench_lib = L
    return _bench_lib


def declared_symbols(header: str = HEADER_PATH, macro: str = "MOE_API") -> list[str]:
    """Entry points a header declares (include/moe_ffn.h by default)."""
    with open(header) as f:
        text = f.read()
    return re.findall(macro + r"\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)


def status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _expect(name, t, dtype, shape, device=None):
    """Check that tensor ``t`` is a contiguous ``dtype`` tensor of ``shape`` on a
    GPU (on ``device`` when given) before its pointer goes to the library: the
    kernels read raw memory, so a wrong dtype or a short buffer would misread
    or run past its end instead of failing."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be on a GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    return t.device


def _check_layer_io(desc, x=None, topk_ids=None, topk_w=None, y=None, ws=None):
    """dtype / shape checks of a layer call's tensors against ``desc``, then
    the device checks (all on one GPU)."""
    import torch
    M, H, k = desc.M, desc.H, desc.k
    specs = [("x", x, torch.bfloat16, (M, H)), ("topk_ids", topk_ids, torch.int32, (M, k)),
             ("topk_w", topk_w, torch.float32, (M, k)), ("y", y, torch.float32, (M, H)),
             ("ws", ws, torch.uint8, None)]
    specs = [s for s in specs if s[1] is not None]
    for name, t, dtype, shape in specs:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
        if t.dtype != dtype:
            raise TypeError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    for name, t, dtype, shape in specs:
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
    dev = None
    for name, t, dtype, shape in specs:
        dev = _expect(name, t, dtype, tuple(t.shape), dev)


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def moe_align_capacity(M: int, k: int, E: int, b: int) -> int:
    return int(lib().moe_align_capacity(M, k, E, b))


def moe_align(topk_ids, E: int, b: int, sorted_route_ids, expert_block_ids, num_padded,
              stream=None, check: bool = True) -> int:
    M, k = topk_ids.shape
    st = lib().moe_align(_ptr(topk_ids), M, k, E, b, _ptr(sorted_route_ids),
                         _ptr(expert_block_ids), _ptr(num_padded),
                         sorted_route_ids.numel(), _stream(stream))
    if check:
        _check(st, "moe_align")
    return st


def moe_align_ex_workspace_size(M: int, k: int, E: int) -> int:
    n = _c_size(0)
    _check(lib().moe_align_ex_workspace_size(M, k, E, ctypes.byref(n)), "moe_align_ex_workspace_size")
    return int(n.value)


def moe_align_ex(topk_ids, E: int, expert_base: int, b: int, sorted_route_ids, expert_block_ids,
                 num_padded, ws=None, stream=None, check: bool = True) -> int:
    M, k = topk_ids.shape
    st = lib().moe_align_ex(_ptr(topk_ids), M, k, E, expert_base, b, _ptr(sorted_route_ids),
                            _ptr(expert_block_ids), _ptr(num_padded), sorted_route_ids.numel(),
                            _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                            _stream(stream))
    if check:
        _check(st, "moe_align_ex")
    return st


def weights_struct(fmt: int, group: int, q, scale, zero) -> moe_weights:
    return moe_weights(fmt, group, _ptr(q), _ptr(scale), _ptr(zero))


def make_desc(M: int, H: int, I: int, E: int, k: int, b: int, w13: moe_weights,
              w2: moe_weights, path: int = MOE_PATH_AUTO, max_workgroups: int = 0,
              expert_base: int = 0) -> moe_ffn_desc:
    return moe_ffn_desc(M, H, I, E, k, b, w13, w2, path, max_workgroups, expert_base)


def moe_ffn_workspace_size(desc: moe_ffn_desc, check: bool = True):
    n = _c_size(0)
    st = lib().moe_ffn_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if check:
        _check(st, "moe_ffn_workspace_size")
        return int(n.value)
    return st, int(n.value)


def moe_ffn_forward(desc: moe_ffn_desc, x, topk_ids, topk_w, y, ws, stream=None,
                    check: bool = True) -> int:
    _check_layer_io(desc, x, topk_ids, topk_w, y, ws)
    st = lib().moe_ffn_forward(ctypes.byref(desc), _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(y),
                               _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                               _stream(stream))
    if check:
        _check(st, "moe_ffn_forward")
    return st


def moe_ffn_forward_noalloc(desc: moe_ffn_desc, x, topk_ids, topk_w, y, stream=None,
                            check: bool = True) -> int:
    """moe_ffn_forward on the library's static per-GPU scratch (no workspace)."""
    _check_layer_io(desc, x, topk_ids, topk_w, y)
    st = lib().moe_ffn_forward_noalloc(ctypes.byref(desc), _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(y),
                                       _stream(stream))
    if check:
        _check(st, "moe_ffn_forward_noalloc")
    return st


def moe_ffn_noalloc_max_bytes() -> int:
    return int(lib().moe_ffn_noalloc_max_bytes())


def moe_ffn_forward_aligned(desc: moe_ffn_desc, x, topk_ids, topk_w, sorted_route_ids,
                            expert_block_ids, num_padded, y, ws, stream=None,
                            check: bool = True) -> int:
    import torch
    _check_layer_io(desc, x, topk_ids, topk_w, y, ws)
    cap = sorted_route_ids.numel()
    _expect("sorted_route_ids", sorted_route_ids, torch.int32, (cap,), x.device)
    _expect("expert_block_ids", expert_block_ids, torch.int32, (cap // max(desc.b, 1),), x.device)
    _expect("num_padded", num_padded, torch.int32, (1,), x.device)
    st = lib().moe_ffn_forward_aligned(
        ctypes.byref(desc), _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(sorted_route_ids),
        _ptr(expert_block_ids), _ptr(num_padded), sorted_route_ids.numel(), _ptr(y), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream))
    if check:
        _check(st, "moe_ffn_forward_aligned")
    return st


def moe_ffn_forward_capture(desc: moe_ffn_desc, x, topk_ids, topk_w, y, ws, w13_out, stream=None) -> None:
    """moe_ffn_forward that also writes the W13 outputs (gate, up) of every valid
    route into w13_out, fp32 [M*k, 2I]."""
    import torch
    _check_layer_io(desc, x, topk_ids, topk_w, y, ws)
    _expect("w13_out", w13_out, torch.float32, (desc.M * desc.k, 2 * desc.I), x.device)
    _check(lib().moe_ffn_forward_capture(ctypes.byref(desc), _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(y),
                                         _ptr(ws), ws.numel() * ws.element_size(), _ptr(w13_out),
                                         _stream(stream)), "moe_ffn_forward_capture")


def moe_ffn_forward_profiled(desc: moe_ffn_desc, x, topk_ids, topk_w, y, ws, events,
                             stream=None) -> None:
    """``events`` are torch.cuda.Event(enable_timing=True) objects, two per
    kernel: events[2i] and events[2i + 1] take kernel i's start and end."""
    _check_layer_io(desc, x, topk_ids, topk_w, y, ws)
    for e in events:
        if int(e.cuda_event) == 0:   # torch creates the HIP event on first record
            e.record()
    handles = (_c_ptr * len(events))(*[int(e.cuda_event) for e in events])
    st = lib().moe_ffn_forward_profiled(ctypes.byref(desc), _ptr(x), _ptr(topk_ids), _ptr(topk_w),
                                        _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                        _stream(stream), handles, len(events))
    _check(st, "moe_ffn_forward_profiled")


def moe_ffn_gate_up(desc: moe_ffn_desc, x, topk_ids, ws, stream=None) -> None:
    _check_layer_io(desc, x, topk_ids, None, None, ws)
    _check(lib().moe_ffn_gate_up(ctypes.byref(desc), _ptr(x), _ptr(topk_ids), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)), "moe_ffn_gate_up")


def moe_ffn_down_combine(desc: moe_ffn_desc, topk_ids, topk_w, y, ws, stream=None) -> None:
    _check_layer_io(desc, None, topk_ids, topk_w, y, ws)
    _check(lib().moe_ffn_down_combine(ctypes.byref(desc), _ptr(topk_ids), _ptr(topk_w), _ptr(y),
                                      _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_ffn_down_combine")


def moe_ffn_gate_up_batched(desc: moe_ffn_desc, xb, counts, a16, a_scale, stream=None) -> None:
    """xb [E, capacity, H] bf16, counts [E] int32 (device), a16 [E, capacity, I]
    fp16 and a_scale [E, capacity, ceil(I/128), 4] fp32 (intermediate format 2)."""
    import torch
    E, cap = desc.E, xb.shape[1] if xb.dim() == 3 else -1
    dev = _expect("xb", xb, torch.bfloat16, (E, cap, desc.H))
    _expect("counts", counts, torch.int32, (E,), dev)
    _expect("a16", a16, torch.float16, (E, cap, desc.I), dev)
    _expect("a_scale", a_scale, torch.float32, (E, cap, -(-desc.I // 128), 4), dev)
    _check(lib().moe_ffn_gate_up_batched(ctypes.byref(desc), _ptr(xb), _ptr(counts), xb.shape[1],
                                         _ptr(a16), _ptr(a_scale), _stream(stream)),
           "moe_ffn_gate_up_batched")


def moe_ffn_down_batched(desc: moe_ffn_desc, a16, a_scale, counts, yb, stream=None) -> None:
    """a16 [E, capacity, I] fp16 and a_scale [E, capacity, ceil(I/128), 4] fp32, counts [E]
    int32, yb [E, capacity, H] fp32."""
    import torch
    E, cap = desc.E, a16.shape[1] if a16.dim() == 3 else -1
    dev = _expect("a16", a16, torch.float16, (E, cap, desc.I))
    _expect("a_scale", a_scale, torch.float32, (E, cap, -(-desc.I // 128), 4), dev)
    _expect("counts", counts, torch.int32, (E,), dev)
    _expect("yb", yb, torch.float32, (E, cap, desc.H), dev)
    _check(lib().moe_ffn_down_batched(ctypes.byref(desc), _ptr(a16), _ptr(a_scale), _ptr(counts),
                                      a16.shape[1], _ptr(yb), _stream(stream)),
           "moe_ffn_down_batched")


def moe_ffn_kernel_count(desc: moe_ffn_desc) -> int:
    return int(lib().moe_ffn_kernel_count(ctypes.byref(desc)))


def moe_ffn_kernel_name(desc: moe_ffn_desc, i: int) -> str | None:
    r = lib().moe_ffn_kernel_name(ctypes.byref(desc), i)
    return None if r is None else r.decode()


def moe_ffn_intermediate(desc: moe_ffn_desc) -> tuple[int, int, int]:
    """(offset, aux_offset, format) of the intermediate in the workspace."""
    off, aux, fmt = _c_size(0), _c_size(0), _c_i32(0)
    _check(lib().moe_ffn_intermediate(ctypes.byref(desc), ctypes.byref(off), ctypes.byref(aux),
                                      ctypes.byref(fmt)), "moe_ffn_intermediate")
    return int(off.value), int(aux.value), int(fmt.value)


def moe_ffn_route_outputs(desc: moe_ffn_desc) -> int:
    """Offset of the grouped path's routed-W2 rows (fp32 [M*k][H]) in the workspace."""
    off = _c_size(0)
    _check(lib().moe_ffn_route_outputs(ctypes.byref(desc), ctypes.byref(off)), "moe_ffn_route_outputs")
    return int(off.value)


def moe_ffn_auto_decode_max_m() -> int:
    return int(lib().moe_ffn_auto_decode_max_m())


def moe_ffn_resolved_path(desc: moe_ffn_desc) -> int:
    """The path moe_ffn_forward takes for `desc` (-1 if it is rejected)."""
    return int(lib().moe_ffn_resolved_path(ctypes.byref(desc)))
