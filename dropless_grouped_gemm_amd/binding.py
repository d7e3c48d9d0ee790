"""Thin Python binding of libmoe's C ABI (argument marshalling only).

Every function here has the name of the C entry point it calls and does nothing
but turn torch tensors into device pointers, pick the current HIP stream and
raise on a non-zero status; every step of the layer runs in the HIP kernels of
libmoe.so.  PyTorch provides device memory and streams.  There is no fallback:
if the library is missing, ``lib()`` raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch  # loads the HIP runtime libmoe.so links against (same soname)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")
# the same library built with MOE_DEBUG (kernels report the indices they skip or clamp)
DEBUG_LIB_PATH = os.path.join(HERE, "libmoe_debug.so")

MOE_OK, MOE_EINVAL, MOE_ENOTSUP, MOE_EWORKSPACE, MOE_EHIP = 0, 1, 2, 3, 4
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
MOE_OP_GATEUP_SWIGLU, MOE_OP_DOWN = 0, 1
(MOE_DBG_BLOCK_TABLE, MOE_DBG_BLOCK_COUNT, MOE_DBG_POSITION, MOE_DBG_GATHER_ROW,
 MOE_DBG_EXPERT_ID) = 0x1, 0x2, 0x4, 0x8, 0x10

ENTRY_POINTS = ("moe_status_str", "moe_max_blocks", "moe_max_rows", "moe_workspace_bytes",
                "moe_workspace_layout", "moe_route", "moe_build_offsets", "moe_permute",
                "moe_build_offsets_noalloc", "moe_build_offsets_noalloc_capacity",
                "moe_build_offsets_scratch_bytes",
                "moe_grouped_gemm", "moe_grouped_gemm_shared", "moe_grouped_gemm_gather",
                "moe_combine", "moe_layer_fwd", "moe_quantize_fp8", "moe_dequantize_fp8",
                "moe_grouped_gemm_fp8", "moe_fp8_workspace_bytes", "moe_layer_fwd_fp8",
                "moe_combine_bwd", "moe_swiglu_bwd", "moe_grouped_gemm_dgrad",
                "moe_grouped_gemm_wgrad", "moe_grouped_gemm_wgrad_workspace_bytes",
                "moe_router_bwd", "moe_router_bwd_workspace_bytes",
                "moe_grouped_gemm_dgrad_workspace_bytes",
                "moe_bwd_workspace_bytes",
                "moe_bwd_workspace_layout", "moe_layer_bwd", "moe_debug_flags",
                "moe_grouped_gemm_fp8_workspace_bytes")


class moe_shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "d", "E", "k", "d_e", "n_groups", "topk_groups", "renormalize",
                 "block_m", "d_e_shared", "dtype", "unpadded")]


_LAYOUT_FIELDS = ("logits", "topk_idx", "topk_w", "counts", "offsets", "padded_offsets",
                  "block_meta", "num_blocks", "pos", "row_src", "err_flag", "x_perm", "act", "y",
                  "shared_act", "shared_out", "scratch", "total")


class moe_ws_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in _LAYOUT_FIELDS]


_BWD_LAYOUT_FIELDS = ("dy", "dact", "dgu", "x_perm", "dx_perm", "dtopk_w", "dlogits",
                      "shared_dact", "shared_dgu", "shared_dx", "router_dx", "router_scratch",
                      "wgrad_sched", "w2_t", "w13_t", "ws2_t", "ws13_t", "total")


class moe_bwd_ws_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in _BWD_LAYOUT_FIELDS]


class MoEError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({status_str(status)})")


_lib = None
_debug_lib = None
_active = None   # the library the wrappers call inside debug_library()


def lib():
    """Load libmoe.so once; raise if it has not been built.  Inside debug_library() the
    debug variant instead."""
    global _lib
    if _active is not None:
        return _active
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def debug_lib():
    """Load libmoe_debug.so once; raise if it has not been built."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _load(DEBUG_LIB_PATH)
    return _debug_lib


@contextlib.contextmanager
def debug_library():
    """Every wrapper called inside the block runs libmoe_debug.so."""
    global _active
    prev = _active
    _active = debug_lib()
    try:
        yield _active
    finally:
        _active = prev


def _load(path):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m dropless_grouped_gemm_amd.build`")
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    S = ctypes.POINTER(moe_shape)
    L.moe_status_str.argtypes = [ctypes.c_int32]
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_max_blocks.argtypes = [S]
    L.moe_max_blocks.restype = ctypes.c_int32
    L.moe_max_rows.argtypes = [S]
    L.moe_max_rows.restype = ctypes.c_int64
    L.moe_workspace_bytes.argtypes = [S]
    L.moe_workspace_bytes.restype = ctypes.c_size_t
    L.moe_workspace_layout.argtypes = [S, ctypes.POINTER(moe_ws_layout)]
    L.moe_workspace_layout.restype = ctypes.c_int32
    L.moe_route.argtypes = [S, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.moe_route.restype = ctypes.c_int32
    L.moe_build_offsets.argtypes = [S, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.moe_build_offsets.restype = ctypes.c_int32
    L.moe_build_offsets_noalloc.argtypes = [S, P, P, P, P, P, P, P, P, P, P]
    L.moe_build_offsets_noalloc.restype = ctypes.c_int32
    L.moe_build_offsets_noalloc_capacity.argtypes = []
    L.moe_build_offsets_noalloc_capacity.restype = ctypes.c_size_t
    L.moe_build_offsets_scratch_bytes.argtypes = [S]
    L.moe_build_offsets_scratch_bytes.restype = ctypes.c_size_t
    L.moe_permute.argtypes = [S, P, P, P, P]
    L.moe_permute.restype = ctypes.c_int32
    L.moe_grouped_gemm.argtypes = [S, ctypes.c_int32, P, P, P, P, P, ctypes.c_int32, P, P]
    L.moe_grouped_gemm.restype = ctypes.c_int32
    L.moe_grouped_gemm_shared.argtypes = [S, ctypes.c_int32, P, P, P, P, P, ctypes.c_int32, P,
                                          P, P, P, P, P]
    L.moe_grouped_gemm_shared.restype = ctypes.c_int32
    L.moe_grouped_gemm_gather.argtypes = [S, P, P, P, P, P, P, ctypes.c_int32, P, P, P, P, P]
    L.moe_grouped_gemm_gather.restype = ctypes.c_int32
    L.moe_quantize_fp8.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P, P]
    L.moe_quantize_fp8.restype = ctypes.c_int32
    L.moe_dequantize_fp8.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P, P]
    L.moe_dequantize_fp8.restype = ctypes.c_int32
    L.moe_fp8_workspace_bytes.argtypes = [S]
    L.moe_fp8_workspace_bytes.restype = ctypes.c_size_t
    L.moe_grouped_gemm_fp8.argtypes = [S, ctypes.c_int32, P, P, P, P, P, P, P, ctypes.c_int32,
                                       P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.moe_grouped_gemm_fp8_workspace_bytes.argtypes = [S]
    L.moe_grouped_gemm_fp8_workspace_bytes.restype = ctypes.c_size_t
    L.moe_grouped_gemm_fp8.restype = ctypes.c_int32
    L.moe_layer_fwd_fp8.argtypes = [S] + [P] * 19 + [ctypes.c_size_t, P]
    L.moe_layer_fwd_fp8.restype = ctypes.c_int32
    L.moe_combine.argtypes = [S, P, P, P, P, P, P]
    L.moe_combine.restype = ctypes.c_int32
    L.moe_layer_fwd.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.moe_layer_fwd.restype = ctypes.c_int32
    L.moe_combine_bwd.argtypes = [S, P, P, P, P, P, P, P]
    L.moe_combine_bwd.restype = ctypes.c_int32
    L.moe_swiglu_bwd.argtypes = [S, P, P, P, P, P, P, P, ctypes.c_int32, P, P, P, P, P, P, P]
    L.moe_swiglu_bwd.restype = ctypes.c_int32
    L.moe_grouped_gemm_dgrad.argtypes = [S, ctypes.c_int32, P, P, P, P, P, ctypes.c_int32, P, P,
                                         ctypes.c_size_t, P]
    L.moe_grouped_gemm_dgrad_workspace_bytes.argtypes = [S, ctypes.c_int32]
    L.moe_grouped_gemm_dgrad_workspace_bytes.restype = ctypes.c_size_t
    L.moe_grouped_gemm_dgrad.restype = ctypes.c_int32
    L.moe_grouped_gemm_wgrad.argtypes = [S, ctypes.c_int32, P, P, P, P, P, P, P,
                                         ctypes.c_size_t, P]
    L.moe_grouped_gemm_wgrad_workspace_bytes.argtypes = [S]
    L.moe_grouped_gemm_wgrad_workspace_bytes.restype = ctypes.c_size_t
    L.moe_grouped_gemm_wgrad.restype = ctypes.c_int32
    L.moe_router_bwd.argtypes = [S] + [P] * 11 + [ctypes.c_size_t, P]
    L.moe_router_bwd_workspace_bytes.argtypes = [S]
    L.moe_router_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.moe_router_bwd.restype = ctypes.c_int32
    L.moe_bwd_workspace_bytes.argtypes = [S]
    L.moe_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.moe_bwd_workspace_layout.argtypes = [S, ctypes.POINTER(moe_bwd_ws_layout)]
    L.moe_bwd_workspace_layout.restype = ctypes.c_int32
    L.moe_layer_bwd.argtypes = ([S] + [P] * 12 + [ctypes.c_size_t] + [P] * 11 +
                                [ctypes.c_size_t, P])
    L.moe_layer_bwd.restype = ctypes.c_int32
    L.moe_debug_flags.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32]
    L.moe_debug_flags.restype = ctypes.c_int32
    return L


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def make_shape(T, d, E, k, d_e, block_m, dtype="bf16", n_groups=0, topk_groups=0,
               renormalize=False, d_e_shared=0, unpadded=False) -> moe_shape:
    dt = {"bf16": MOE_DTYPE_BF16, "fp32": MOE_DTYPE_F32, torch.bfloat16: MOE_DTYPE_BF16,
          torch.float32: MOE_DTYPE_F32}[dtype]
    return moe_shape(T, d, E, k, d_e, n_groups, topk_groups, int(bool(renormalize)), block_m,
                     d_e_shared, dt, int(bool(unpadded)))


def shape_of_config(cfg) -> moe_shape:
    """moe_shape of a workloads.MoEConfig."""
    return make_shape(cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_e, cfg.block_m, cfg.dtype, cfg.n_groups,
                      cfg.topk_groups, cfg.renormalize, cfg.d_e_shared, cfg.unpadded)


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, status):
    if status != MOE_OK:
        raise MoEError(fn, status)


# ---------------------------------------------------------------------------
# Host-only helpers
# ---------------------------------------------------------------------------
def moe_max_blocks(shape: moe_shape) -> int:
    return lib().moe_max_blocks(ctypes.byref(shape))


def moe_max_rows(shape: moe_shape) -> int:
    return lib().moe_max_rows(ctypes.byref(shape))


def moe_debug_flags(clear: bool = True) -> int:
    """MOE_DBG_* bits the debug library's kernels set on the current device since the last
    clear (synchronises the device); raises MoEError(MOE_ENOTSUP) on the release library."""
    v = ctypes.c_uint32(0)
    _check("moe_debug_flags", lib().moe_debug_flags(ctypes.byref(v), int(bool(clear))))
    return v.value


def moe_workspace_bytes(shape: moe_shape) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(shape))


def moe_workspace_layout(shape: moe_shape) -> dict:
    L = moe_ws_layout()
    _check("moe_workspace_layout", lib().moe_workspace_layout(ctypes.byref(shape), ctypes.byref(L)))
    return {n: getattr(L, n) for n in _LAYOUT_FIELDS}


def alloc_workspace(shape: moe_shape, device="cuda", fp8: bool = False) -> torch.Tensor:
    """A workspace for moe_layer_fwd (fp8=False) or moe_layer_fwd_fp8 (fp8=True)."""
    n = moe_fp8_workspace_bytes(shape) if fp8 else moe_workspace_bytes(shape)
    if n == 0:
        raise MoEError("moe_fp8_workspace_bytes" if fp8 else "moe_workspace_bytes", MOE_EINVAL)
    return torch.empty(n, dtype=torch.uint8, device=device)


def ws_view(ws: torch.Tensor, shape: moe_shape, name: str, dtype: torch.dtype, shape_out):
    """A typed view of one intermediate inside a moe_layer_fwd workspace."""
    off = moe_workspace_layout(shape)[name]
    n = 1
    for s in shape_out:
        n *= s
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype).view(*shape_out)


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------
def moe_route(shape, x, w_gate, bias, logits, topk_idx, topk_w, ws, stream=None):
    _check("moe_route", lib().moe_route(ctypes.byref(shape), _p(x), _p(w_gate), _p(bias),
                                        _p(logits), _p(topk_idx), _p(topk_w), _p(ws),
                                        ws.numel() if ws is not None else 0, _stream(stream)))


def moe_build_offsets(shape, topk_idx, counts, offsets, padded_offsets, block_meta, num_blocks,
                      pos, row_src, err_flag, ws, stream=None):
    _check("moe_build_offsets", lib().moe_build_offsets(
        ctypes.byref(shape), _p(topk_idx), _p(counts), _p(offsets), _p(padded_offsets),
        _p(block_meta), _p(num_blocks), _p(pos), _p(row_src), _p(err_flag), _p(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))


def moe_build_offsets_noalloc(shape, topk_idx, counts, offsets, padded_offsets, block_meta,
                              num_blocks, pos, row_src, err_flag, stream=None):
    _check("moe_build_offsets_noalloc", lib().moe_build_offsets_noalloc(
        ctypes.byref(shape), _p(topk_idx), _p(counts), _p(offsets), _p(padded_offsets),
        _p(block_meta), _p(num_blocks), _p(pos), _p(row_src), _p(err_flag), _stream(stream)))


def moe_build_offsets_noalloc_capacity() -> int:
    return lib().moe_build_offsets_noalloc_capacity()


def moe_build_offsets_scratch_bytes(shape: moe_shape) -> int:
    return lib().moe_build_offsets_scratch_bytes(ctypes.byref(shape))


def moe_permute(shape, x, pos, x_perm, stream=None):
    _check("moe_permute", lib().moe_permute(ctypes.byref(shape), _p(x), _p(pos), _p(x_perm),
                                            _stream(stream)))


def moe_grouped_gemm(shape, op, A, B0, B1, block_meta, num_blocks, max_blocks, C, stream=None):
    _check("moe_grouped_gemm", lib().moe_grouped_gemm(
        ctypes.byref(shape), op, _p(A), _p(B0), _p(B1), _p(block_meta), _p(num_blocks),
        int(max_blocks), _p(C), _stream(stream)))


def moe_grouped_gemm_shared(shape, op, A, B0, B1, block_meta, num_blocks, max_blocks, C,
                            A_shared, B0_shared, B1_shared, C_shared, stream=None):
    _check("moe_grouped_gemm_shared", lib().moe_grouped_gemm_shared(
        ctypes.byref(shape), op, _p(A), _p(B0), _p(B1), _p(block_meta), _p(num_blocks),
        int(max_blocks), _p(C), _p(A_shared), _p(B0_shared), _p(B1_shared), _p(C_shared),
        _stream(stream)))


def moe_grouped_gemm_gather(shape, x, row_src, w1, w3, block_meta, num_blocks, max_blocks, act,
                            ws1=None, ws3=None, shared_act=None, stream=None):
    _check("moe_grouped_gemm_gather", lib().moe_grouped_gemm_gather(
        ctypes.byref(shape), _p(x), _p(row_src), _p(w1), _p(w3), _p(block_meta), _p(num_blocks),
        int(max_blocks), _p(act), _p(ws1), _p(ws3), _p(shared_act), _stream(stream)))


def gather_supported(shape) -> bool:
    """moe_grouped_gemm_gather (and so moe_layer_fwd's fused permute) applies: bf16,
    d % 32 == 0 and gathered rows addressable with 32-bit byte offsets."""
    return (shape.dtype == MOE_DTYPE_BF16 and shape.d % 32 == 0
            and shape.T * shape.d * 2 + 4096 < 2 ** 32)


def moe_quantize_fp8(w, q, scales, stream=None):
    """w: bf16 [E, K, N] (or [K, N]); q: uint8 of the same shape; scales: fp32
    [E, ceil(K/128), ceil(N/128)]."""
    E, K, N = (1,) + tuple(w.shape) if w.dim() == 2 else tuple(w.shape)
    _check("moe_quantize_fp8", lib().moe_quantize_fp8(E, K, N, _p(w), _p(q), _p(scales),
                                                      _stream(stream)))


def moe_dequantize_fp8(q, scales, w, stream=None):
    """q: uint8 [E, K, N] (or [K, N]); scales: fp32 [E, ceil(K/128), ceil(N/128)];
    w: bf16 of q's shape, written."""
    E, K, N = (1,) + tuple(q.shape) if q.dim() == 2 else tuple(q.shape)
    _check("moe_dequantize_fp8", lib().moe_dequantize_fp8(E, K, N, _p(q), _p(scales), _p(w),
                                                          _stream(stream)))


def dequantize_fp8(q, scales, stream=None):
    """The bf16 weights (code * block scale, rounded to nearest even) of an fp8 pair."""
    w = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    moe_dequantize_fp8(q, scales, w, stream)
    return w


def moe_fp8_workspace_bytes(shape: moe_shape) -> int:
    return lib().moe_fp8_workspace_bytes(ctypes.byref(shape))


def fp8_dequantises(shape: moe_shape) -> bool:
    """moe_layer_fwd_fp8 dequantises the weights into its workspace and runs the bf16
    kernels: where the routed rows M = T * k reach 256 * min(E, M) (the header's rule)."""
    M = shape.T * shape.k
    return M > 0 and M >= 256 * min(shape.E, M)


def fp8_scale_shape(w_shape):
    """Scale array shape for a weight of shape [E, K, N] (or [K, N])."""
    *e, K, N = w_shape
    return tuple(e) + (-(-K // 128), -(-N // 128))


def quantize_fp8(w, stream=None):
    """(codes, scales) of a bf16 weight tensor, on its device."""
    q = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    s = torch.empty(fp8_scale_shape(w.shape), dtype=torch.float32, device=w.device)
    moe_quantize_fp8(w, q, s, stream)
    return q, s


def moe_grouped_gemm_fp8(shape, op, A, Q0, S0, Q1, S1, block_meta, num_blocks, max_blocks,
                         row_src, C, A_shared=None, Q0_shared=None, S0_shared=None,
                         Q1_shared=None, S1_shared=None, C_shared=None, ws=None, stream=None):
    """ws: None, or a uint8 tensor of moe_grouped_gemm_fp8_workspace_bytes(shape) bytes."""
    _check("moe_grouped_gemm_fp8", lib().moe_grouped_gemm_fp8(
        ctypes.byref(shape), op, _p(A), _p(Q0), _p(S0), _p(Q1), _p(S1), _p(block_meta),
        _p(num_blocks), int(max_blocks), _p(row_src), _p(C), _p(A_shared), _p(Q0_shared),
        _p(S0_shared), _p(Q1_shared), _p(S1_shared), _p(C_shared), _p(ws),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream)))


def moe_grouped_gemm_fp8_workspace_bytes(shape) -> int:
    return lib().moe_grouped_gemm_fp8_workspace_bytes(ctypes.byref(shape))


def alloc_fp8_gemm_workspace(shape, device="cuda") -> torch.Tensor:
    """The optional scratch of moe_grouped_gemm_fp8 (uninitialised: every byte read is
    first written by the same call)."""
    return torch.empty(moe_grouped_gemm_fp8_workspace_bytes(shape), dtype=torch.uint8,
                       device=device)


def moe_layer_fwd_fp8(shape, x, w_gate, bias, q1, s1, q3, s3, q2, s2, qs1, ss1, qs3, ss3,
                      qs2, ss2, topk_idx_in, topk_w_in, out, ws, stream=None):
    _check("moe_layer_fwd_fp8", lib().moe_layer_fwd_fp8(
        ctypes.byref(shape), _p(x), _p(w_gate), _p(bias), _p(q1), _p(s1), _p(q3), _p(s3),
        _p(q2), _p(s2), _p(qs1), _p(ss1), _p(qs3), _p(ss3), _p(qs2), _p(ss2), _p(topk_idx_in),
        _p(topk_w_in), _p(out), _p(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def fp8_supported(shape) -> bool:
    """The fp8-weight path applies: bf16 activations, 128-row blocks, d, d_e (and
    d_e_shared) multiples of 32 and at most 32768."""
    dims = [shape.d, shape.d_e] + ([shape.d_e_shared] if shape.d_e_shared else [])
    return (shape.dtype == MOE_DTYPE_BF16 and shape.block_m == 128
            and all(v % 32 == 0 and v <= 32768 for v in dims))


def moe_combine(shape, y, pos, topk_w, shared_out, out, stream=None):
    _check("moe_combine", lib().moe_combine(ctypes.byref(shape), _p(y), _p(pos), _p(topk_w),
                                            _p(shared_out), _p(out), _stream(stream)))


def moe_layer_fwd(shape, x, w_gate, bias, w1, w3, w2, ws1, ws3, ws2, topk_idx_in, topk_w_in,
                  out, ws, stream=None):
    _check("moe_layer_fwd", lib().moe_layer_fwd(
        ctypes.byref(shape), _p(x), _p(w_gate), _p(bias), _p(w1), _p(w3), _p(w2), _p(ws1),
        _p(ws3), _p(ws2), _p(topk_idx_in), _p(topk_w_in), _p(out), _p(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------
def moe_bwd_workspace_bytes(shape: moe_shape) -> int:
    return lib().moe_bwd_workspace_bytes(ctypes.byref(shape))


def moe_bwd_workspace_layout(shape: moe_shape) -> dict:
    L = moe_bwd_ws_layout()
    _check("moe_bwd_workspace_layout",
           lib().moe_bwd_workspace_layout(ctypes.byref(shape), ctypes.byref(L)))
    return {n: getattr(L, n) for n in _BWD_LAYOUT_FIELDS}


def alloc_bwd_workspace(shape: moe_shape, device="cuda") -> torch.Tensor:
    if moe_max_blocks(shape) < 0:                 # invalid shape
        raise MoEError("moe_bwd_workspace_bytes", MOE_EINVAL)
    n = moe_bwd_workspace_bytes(shape)            # 0 for T == 0: nothing to hold
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def bwd_ws_view(ws: torch.Tensor, shape: moe_shape, name: str, dtype: torch.dtype, shape_out):
    """A typed view of one intermediate inside a moe_layer_bwd workspace."""
    off = moe_bwd_workspace_layout(shape)[name]
    n = 1
    for v in shape_out:
        n *= v
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype).view(*shape_out)


def backward_supported(shape) -> bool:
    """The backward kernels' conditions (mirrors the library's own checks)."""
    return (shape.dtype == MOE_DTYPE_BF16 and shape.d % 32 == 0 and shape.d_e % 32 == 0
            and shape.d_e_shared % 32 == 0 and shape.d <= 8192)


def moe_combine_bwd(shape, dout, y, pos, topk_w, dy, dtopk_w, stream=None):
    _check("moe_combine_bwd", lib().moe_combine_bwd(
        ctypes.byref(shape), _p(dout), _p(y), _p(pos), _p(topk_w), _p(dy), _p(dtopk_w),
        _stream(stream)))


def moe_swiglu_bwd(shape, A, row_src, w1, w3, dact, block_meta, num_blocks, max_blocks, dgu,
                   x_shared=None, ws1=None, ws3=None, dact_shared=None, dgu_shared=None,
                   stream=None):
    _check("moe_swiglu_bwd", lib().moe_swiglu_bwd(
        ctypes.byref(shape), _p(A), _p(row_src), _p(w1), _p(w3), _p(dact), _p(block_meta),
        _p(num_blocks), max_blocks, _p(dgu), _p(x_shared), _p(ws1), _p(ws3), _p(dact_shared),
        _p(dgu_shared), _stream(stream)))


def moe_grouped_gemm_dgrad_workspace_bytes(shape, op) -> int:
    return lib().moe_grouped_gemm_dgrad_workspace_bytes(ctypes.byref(shape), op)


def moe_grouped_gemm_dgrad(shape, op, dC, B0, B1, block_meta, num_blocks, max_blocks, dA,
                           ws=None, stream=None):
    """ws: None - the weights are read transposed in place; a device buffer of
    moe_grouped_gemm_dgrad_workspace_bytes(shape, op) bytes - transposed into it first."""
    _check("moe_grouped_gemm_dgrad", lib().moe_grouped_gemm_dgrad(
        ctypes.byref(shape), op, _p(dC), _p(B0), _p(B1), _p(block_meta), _p(num_blocks),
        max_blocks, _p(dA), _p(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def moe_grouped_gemm_wgrad_workspace_bytes(shape: moe_shape) -> int:
    return lib().moe_grouped_gemm_wgrad_workspace_bytes(ctypes.byref(shape))


def moe_grouped_gemm_wgrad(shape, op, A, dC, counts, padded_offsets, dB0, dB1, ws=None,
                           stream=None):
    """ws: None (static order) or a uint8 device tensor of at least
    moe_grouped_gemm_wgrad_workspace_bytes(shape) bytes (work queue, largest expert
    first)."""
    _check("moe_grouped_gemm_wgrad", lib().moe_grouped_gemm_wgrad(
        ctypes.byref(shape), op, _p(A), _p(dC), _p(counts), _p(padded_offsets), _p(dB0),
        _p(dB1), _p(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def moe_router_bwd_workspace_bytes(shape: moe_shape) -> int:
    return lib().moe_router_bwd_workspace_bytes(ctypes.byref(shape))


def moe_router_bwd(shape, x, w_gate, logits, topk_idx, dtopk_w, dlogits, dw_gate, dbias, dx_in,
                   dx_out, ws=None, stream=None):
    """ws: scratch of moe_router_bwd_workspace_bytes(shape) bytes (allocated here when
    None)."""
    if ws is None:
        n = moe_router_bwd_workspace_bytes(shape)
        ws = torch.empty(n, dtype=torch.uint8, device=x.device) if n else None
    _check("moe_router_bwd", lib().moe_router_bwd(
        ctypes.byref(shape), _p(x), _p(w_gate), _p(logits), _p(topk_idx), _p(dtopk_w),
        _p(dlogits), _p(dw_gate), _p(dbias), _p(dx_in), _p(dx_out), _p(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))


def moe_layer_bwd(shape, x, w_gate, w1, w3, w2, ws1, ws3, ws2, topk_idx_in, topk_w_in, dout,
                  fwd_ws, dx, dw1, dw3, dw2, dws1, dws3, dws2, dw_gate, dbias, dtopk_w, ws,
                  stream=None):
    _check("moe_layer_bwd", lib().moe_layer_bwd(
        ctypes.byref(shape), _p(x), _p(w_gate), _p(w1), _p(w3), _p(w2), _p(ws1), _p(ws3),
        _p(ws2), _p(topk_idx_in), _p(topk_w_in), _p(dout), _p(fwd_ws),
        fwd_ws.numel() if fwd_ws is not None else 0, _p(dx), _p(dw1), _p(dw3), _p(dw2),
        _p(dws1), _p(dws3), _p(dws2), _p(dw_gate), _p(dbias), _p(dtopk_w), _p(ws),
        ws.numel() if ws is not None else 0, _stream(stream)))
