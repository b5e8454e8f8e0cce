"""Python binding of the C ABI in include/moe_layer.h (ctypes).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe_layer.so.  Tensors are torch tensors (device memory and streams come
from PyTorch); each function has the name of the C entry point it calls and
raises MoeError when that entry point returns a non-OK status.  There is no
fallback: if the library is not built, importing this module fails.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_layer.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m moe_layer_router_amd.build` "
                      "(or __graft_entry__.build())")

# PyTorch ships its own HIP runtime with the same soname (libamdhip64.so.7).
# Importing torch first makes the dynamic loader bind this library to that
# already-loaded runtime, so device pointers and streams from torch are valid
# here; loading the library first would put two HIP runtimes in the process.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

# moe_status
MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_HIP = 4
# moe_dtype
MOE_DTYPE_BF16 = 0
MOE_DTYPE_FP8_E4M3 = 1
MOE_DTYPE_FP4_E2M1 = 2
MOE_DTYPE_F32 = 3
# moe_mode
MOE_MODE_MEGA = 0
MOE_MODE_SEPARATE = 1
# flags
MOE_FLAG_ROUTING_GIVEN = 1
MOE_FLAG_TRACE = 2
MOE_TRACE_GROUPS = 1024
MOE_TRACE_FIELDS = 8
# moe_weight_layout
MOE_LAYOUT_ROW_MAJOR = 0
MOE_LAYOUT_TILED = 1
# moe_inter_scale
MOE_INTER_SCALE_F32 = 0
MOE_INTER_SCALE_POW2 = 1
# moe_weight_scale
MOE_WSCALE_BLOCK = 0
MOE_WSCALE_CHANNEL = 1
# moe_peak_kind
MOE_PEAK_KINDS = {"mfma16_fp8_fp8": 0, "mfma16_fp4_fp8": 1, "mfma16_fp4_fp4": 2, "mfma16_bf16": 3,
                  "mfma32_fp8_fp8": 4, "mfma32_fp4_fp8": 5}
# moe_pack_weights `which`
MOE_WEIGHTS_GATE_UP = 0
MOE_WEIGHTS_DOWN = 1

DTYPES = {"bf16": MOE_DTYPE_BF16, "fp8": MOE_DTYPE_FP8_E4M3, "fp4": MOE_DTYPE_FP4_E2M1, "f32": MOE_DTYPE_F32}
MODES = {"mega": MOE_MODE_MEGA, "separate": MOE_MODE_SEPARATE}


class MoeDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("I", ctypes.c_int32), ("top_k", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("weight_dtype", ctypes.c_int32), ("mode", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("weight_layout", ctypes.c_int32), ("inter_scale", ctypes.c_int32),
                ("weight_scale", ctypes.c_int32)]


class MoeWorkspaceRegions(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("logits", "perm", "row_of", "offsets", "inter", "inter_scales", "staging", "trace", "total")]


class MoeError(RuntimeError):
    def __init__(self, status, func):
        self.status = status
        super().__init__(f"{func}: {moe_status_string(status)}: {moe_last_error()}")


_P = ctypes.c_void_p
_lib.moe_abi_version.restype = ctypes.c_int32
_lib.moe_abi_version.argtypes = []
_lib.moe_workspace_size.restype = ctypes.c_size_t
_lib.moe_workspace_size.argtypes = [ctypes.POINTER(MoeDesc)]
_lib.moe_route_workspace_size.restype = ctypes.c_size_t
_lib.moe_route_workspace_size.argtypes = [ctypes.POINTER(MoeDesc)]
_lib.moe_permute_workspace_size.restype = ctypes.c_size_t
_lib.moe_permute_workspace_size.argtypes = [ctypes.POINTER(MoeDesc)]
_lib.moe_get_workspace_regions.restype = ctypes.c_int
_lib.moe_get_workspace_regions.argtypes = [ctypes.POINTER(MoeDesc), ctypes.POINTER(MoeWorkspaceRegions)]
_lib.moe_validate.restype = ctypes.c_int
_lib.moe_validate.argtypes = [ctypes.POINTER(MoeDesc)] + [_P] * 11 + [_P, ctypes.c_size_t]
_lib.moe_forward.restype = ctypes.c_int
_lib.moe_forward.argtypes = [ctypes.POINTER(MoeDesc)] + [_P] * 13 + [_P, ctypes.c_size_t, _P]
_lib.moe_quantize_input.restype = ctypes.c_int
_lib.moe_quantize_input.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P]
_lib.moe_quantize_e5m6.restype = ctypes.c_int
_lib.moe_quantize_e5m6.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P]
_lib.moe_dequantize_e5m6.restype = ctypes.c_int
_lib.moe_dequantize_e5m6.argtypes = [ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P]
_lib.moe_backward_workspace_size.restype = ctypes.c_size_t
_lib.moe_backward_workspace_size.argtypes = [ctypes.POINTER(MoeDesc)]
_lib.moe_backward.restype = ctypes.c_int
_lib.moe_backward.argtypes = [ctypes.POINTER(MoeDesc)] + [_P] * 13 + [ctypes.c_size_t, _P]
_lib.moe_forward_static.restype = ctypes.c_int
_lib.moe_forward_static.argtypes = [ctypes.POINTER(MoeDesc)] + [_P] * 13 + [_P]
_lib.moe_route.restype = ctypes.c_int
_lib.moe_route.argtypes = [ctypes.POINTER(MoeDesc)] + [_P] * 7 + [_P, ctypes.c_size_t, _P]
_lib.moe_permute.restype = ctypes.c_int
_lib.moe_permute.argtypes = [ctypes.POINTER(MoeDesc)] + [_P] * 4 + [_P, ctypes.c_size_t, _P]
_lib.moe_pack_weights.restype = ctypes.c_int
_lib.moe_pack_weights.argtypes = [ctypes.POINTER(MoeDesc), ctypes.c_int32] + [_P] * 4 + [_P]
_lib.moe_peak_mfma_flops.restype = ctypes.c_double
_lib.moe_peak_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
_lib.moe_peak_mfma.restype = ctypes.c_int
_lib.moe_peak_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]
_lib.moe_peak_hbm_read.restype = ctypes.c_int
_lib.moe_peak_hbm_read.argtypes = [_P, ctypes.c_size_t, ctypes.c_int32, _P, _P]
_lib.moe_status_string.restype = ctypes.c_char_p
_lib.moe_status_string.argtypes = [ctypes.c_int]
_lib.moe_last_error.restype = ctypes.c_char_p
_lib.moe_last_error.argtypes = []


LAYOUTS = {"row_major": MOE_LAYOUT_ROW_MAJOR, "tiled": MOE_LAYOUT_TILED}
INTER_SCALES = {"f32": MOE_INTER_SCALE_F32, "pow2": MOE_INTER_SCALE_POW2}
WEIGHT_SCALES = {"block": MOE_WSCALE_BLOCK, "channel": MOE_WSCALE_CHANNEL}


def make_desc(T, H, E, I, top_k, act="fp8", weight="fp8", mode="mega", flags=0, layout="tiled",
              inter_scale="f32", wscale="block") -> MoeDesc:
    return MoeDesc(T, H, E, I, top_k, DTYPES[act], DTYPES[weight], MODES.get(mode, mode), flags,
                   LAYOUTS.get(layout, layout), INTER_SCALES.get(inter_scale, inter_scale),
                   WEIGHT_SCALES.get(wscale, wscale))


def _ptr(t):
    """Device (or host) address of a tensor, an int address, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t):
    return t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, func):
    if status != MOE_OK:
        raise MoeError(status, func)


def moe_abi_version() -> int:
    return _lib.moe_abi_version()


def moe_status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def moe_last_error() -> str:
    return _lib.moe_last_error().decode()


def moe_workspace_size(desc: MoeDesc) -> int:
    return _lib.moe_workspace_size(ctypes.byref(desc))


def moe_route_workspace_size(desc: MoeDesc) -> int:
    return _lib.moe_route_workspace_size(ctypes.byref(desc))


def moe_permute_workspace_size(desc: MoeDesc) -> int:
    return _lib.moe_permute_workspace_size(ctypes.byref(desc))


def moe_get_workspace_regions(desc: MoeDesc) -> dict:
    r = MoeWorkspaceRegions()
    _check(_lib.moe_get_workspace_regions(ctypes.byref(desc), ctypes.byref(r)), "moe_get_workspace_regions")
    return {n: getattr(r, n) for n, _ in MoeWorkspaceRegions._fields_}


def moe_validate(desc, x, x_scales, router_w, router_bias, w_gate_up, w_gate_up_scales,
                 w_down, w_down_scales, y, topk_ids, topk_weights, workspace, workspace_bytes=None) -> int:
    """Returns the status (does not raise); pointers may be tensors or ints."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else _nbytes(workspace)
    return _lib.moe_validate(ctypes.byref(desc), _ptr(x), _ptr(x_scales), _ptr(router_w), _ptr(router_bias),
                             _ptr(w_gate_up), _ptr(w_gate_up_scales), _ptr(w_down), _ptr(w_down_scales),
                             _ptr(y), _ptr(topk_ids), _ptr(topk_weights), _ptr(workspace), workspace_bytes)


def moe_forward(desc, x, x_scales, router_w, router_bias, w_gate_up, w_gate_up_scales, w_down,
                w_down_scales, y, topk_ids, topk_weights, expert_offsets, perm, workspace, stream=None):
    st = _lib.moe_forward(ctypes.byref(desc), _ptr(x), _ptr(x_scales), _ptr(router_w), _ptr(router_bias),
                          _ptr(w_gate_up), _ptr(w_gate_up_scales), _ptr(w_down), _ptr(w_down_scales),
                          _ptr(y), _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_offsets), _ptr(perm),
                          _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check(st, "moe_forward")


def moe_forward_static(desc, x, x_scales, router_w, router_bias, w_gate_up, w_gate_up_scales, w_down,
                       w_down_scales, y, topk_ids, topk_weights, expert_offsets, perm, stream=None):
    st = _lib.moe_forward_static(ctypes.byref(desc), _ptr(x), _ptr(x_scales), _ptr(router_w), _ptr(router_bias),
                                 _ptr(w_gate_up), _ptr(w_gate_up_scales), _ptr(w_down), _ptr(w_down_scales),
                                 _ptr(y), _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_offsets), _ptr(perm),
                                 _stream(stream))
    _check(st, "moe_forward_static")


MOE_STATIC_WORKSPACE_BYTES = 64 << 20


def moe_backward_workspace_size(desc) -> int:
    return _lib.moe_backward_workspace_size(ctypes.byref(desc))


def moe_backward(desc, x, router_w, w_gate_up, w_down, topk_ids, topk_weights, dy, dx, dw_gate_up, dw_down,
                 dw_router, dbias, workspace, stream=None):
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.moe_backward(ctypes.byref(desc), _ptr(x), _ptr(router_w), _ptr(w_gate_up), _ptr(w_down),
                             _ptr(topk_ids), _ptr(topk_weights), _ptr(dy), _ptr(dx), _ptr(dw_gate_up),
                             _ptr(dw_down), _ptr(dw_router), _ptr(dbias), _ptr(workspace), nbytes,
                             _stream(stream)), "moe_backward")


def moe_quantize_input(x, xq, x_scales, scale_mode="f32", stream=None):
    """x: [T, H] bfloat16 or float32 tensor; xq [T, H] uint8; x_scales [T, H/128] float32."""
    import torch
    T, H = x.shape
    in_dtype = MOE_DTYPE_BF16 if x.dtype == torch.bfloat16 else MOE_DTYPE_F32
    _check(_lib.moe_quantize_input(T, H, in_dtype, INTER_SCALES.get(scale_mode, scale_mode), _ptr(x), _ptr(xq),
                                   _ptr(x_scales), _stream(stream)), "moe_quantize_input")


def moe_quantize_e5m6(x, xq, x_scales, scale_mode="f32", stream=None):
    """x: [T, H] bfloat16 or float32 tensor; xq [T, 3H/2] uint8; x_scales [T, H/128] float32."""
    import torch
    T, H = x.shape
    in_dtype = MOE_DTYPE_BF16 if x.dtype == torch.bfloat16 else MOE_DTYPE_F32
    _check(_lib.moe_quantize_e5m6(T, H, in_dtype, INTER_SCALES.get(scale_mode, scale_mode), _ptr(x), _ptr(xq),
                                  _ptr(x_scales), _stream(stream)), "moe_quantize_e5m6")


def moe_dequantize_e5m6(xq, x_scales, out, stream=None):
    """xq [T, 3H/2] uint8, x_scales [T, H/128] float32 -> out [T, H] float32."""
    T, H = out.shape
    _check(_lib.moe_dequantize_e5m6(T, H, _ptr(xq), _ptr(x_scales), _ptr(out), _stream(stream)),
           "moe_dequantize_e5m6")


def moe_route(desc, x, x_scales, router_w, router_bias, logits, topk_ids, topk_weights, workspace,
              stream=None):
    st = _lib.moe_route(ctypes.byref(desc), _ptr(x), _ptr(x_scales), _ptr(router_w), _ptr(router_bias),
                        _ptr(logits), _ptr(topk_ids), _ptr(topk_weights), _ptr(workspace), _nbytes(workspace),
                        _stream(stream))
    _check(st, "moe_route")


def moe_permute(desc, topk_ids, expert_offsets, perm, row_of, workspace, stream=None):
    st = _lib.moe_permute(ctypes.byref(desc), _ptr(topk_ids), _ptr(expert_offsets), _ptr(perm), _ptr(row_of),
                          _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check(st, "moe_permute")


def moe_pack_weights(desc, which, src, src_scales, dst, dst_scales, stream=None):
    st = _lib.moe_pack_weights(ctypes.byref(desc), which, _ptr(src), _ptr(src_scales), _ptr(dst), _ptr(dst_scales),
                               _stream(stream))
    _check(st, "moe_pack_weights")


def moe_peak_mfma_flops(kind, iters, blocks) -> float:
    return _lib.moe_peak_mfma_flops(MOE_PEAK_KINDS.get(kind, kind), iters, blocks)


def moe_peak_mfma(kind, iters, blocks, sink, cycles, stream=None):
    _check(_lib.moe_peak_mfma(MOE_PEAK_KINDS.get(kind, kind), iters, blocks, _ptr(sink), _ptr(cycles),
                              _stream(stream)), "moe_peak_mfma")


def moe_peak_hbm_read(buf, nbytes, blocks, sink, stream=None):
    _check(_lib.moe_peak_hbm_read(_ptr(buf), nbytes, blocks, _ptr(sink), _stream(stream)), "moe_peak_hbm_read")


def exported_symbols():
    """Names of the C entry points this binding wraps (for ABI checks)."""
    return ["moe_abi_version", "moe_workspace_size", "moe_forward_static", "moe_quantize_input", "moe_route_workspace_size",
            "moe_permute_workspace_size", "moe_get_workspace_regions", "moe_validate", "moe_forward", "moe_route",
            "moe_permute", "moe_pack_weights", "moe_status_string", "moe_last_error",
            "moe_peak_mfma_flops", "moe_peak_mfma", "moe_peak_hbm_read", "moe_backward_workspace_size",
            "moe_backward", "moe_quantize_e5m6", "moe_dequantize_e5m6"]
