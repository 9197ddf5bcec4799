"""Python binding of ``libvattn.so``: head-major, non-causal attention on MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/vattn.h``.  PyTorch supplies
device memory and the current HIP stream.  There is no CPU fallback: if the
library is missing, importing this package raises.

    import torch, non_causal_flash_amd as vattn
    out = vattn.forward(q, k, v)            # q, k, v: cuda float32 [H, N, d]

``q``, ``k``, ``v`` (and ``out``) may also be strided views with the same
strides and a contiguous last dimension, e.g. a patch-major ``[N, H, d]``
tensor seen as ``x.transpose(0, 1)``; those go through
``vattn_forward_strided``.  float16 tensors go through ``vattn_forward_f16``.

With a rotary table (``rope_table(n_patches, rope_dims, base)``, built once
per set of positions), ``forward(q, k, v, rope=table)`` rotates Q and K
(NeoX pairs) inside the kernel: ``vattn_forward_rope`` /
``vattn_forward_rope_f16``.
"""
from __future__ import annotations

import ctypes
import os

# torch first: its bundled HIP runtime (soname libamdhip64.so.7) then serves
# libvattn.so too, so the stream handles torch hands out are valid for it.
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvattn.so")

VATTN_OK = 0
VATTN_ERR_NULL = 1
VATTN_ERR_SIZE = 2
VATTN_ERR_HEAD_DIM = 3
VATTN_ERR_ALIGN = 4
VATTN_ERR_ALIAS = 5
VATTN_ERR_HIP = 6
VATTN_ERR_ARG = 7
VATTN_ERR_ROPE = 8

PRECISION = {"auto": 0, "fast": 1, "split": 2}

# Symbols declared in include/vattn.h.
EXPORTS = ("vattn_forward", "vattn_forward_precision", "vattn_forward_strided",
           "vattn_forward_f16", "vattn_rope_table", "vattn_forward_rope",
           "vattn_forward_rope_f16", "vattn_status_string", "vattn_last_hip_error",
           "vattn_launch_shape")

# Workgroup shapes (vattn_shape in vattn.h).
SHAPE_SPLIT_KEYS = 1
SHAPE_4_WAVES = 4
SHAPE_8_WAVES = 8
SHAPE_16_WAVES = 16


class VattnError(RuntimeError):
    def __init__(self, status: int, lib):
        self.status = status
        msg = lib.vattn_status_string(status).decode()
        if status == VATTN_ERR_HIP:
            msg += " (hipError_t %d)" % lib.vattn_last_hip_error()
        super().__init__("vattn status %d: %s" % (status, msg))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libvattn.so is not built (%s); run `python non_causal_flash_amd/build.py`"
            % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.vattn_forward.argtypes = [vp, vp, vp, vp, ci, ci, ci, vp]
    lib.vattn_forward.restype = ci
    lib.vattn_forward_precision.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, vp]
    lib.vattn_forward_precision.restype = ci
    ll = ctypes.c_longlong
    lib.vattn_forward_strided.argtypes = [vp, vp, vp, vp, ci, ci, ci, ll, ll, ci, vp]
    lib.vattn_forward_strided.restype = ci
    lib.vattn_forward_f16.argtypes = [vp, vp, vp, vp, ci, ci, ci, ll, ll, ci, vp]
    lib.vattn_forward_f16.restype = ci
    lib.vattn_rope_table.argtypes = [vp, ci, ci, ctypes.c_float, vp, ci, vp]
    lib.vattn_rope_table.restype = ci
    lib.vattn_forward_rope.argtypes = [vp, vp, vp, vp, ci, ci, ci, ll, ll, ci, vp, ci, vp]
    lib.vattn_forward_rope.restype = ci
    lib.vattn_forward_rope_f16.argtypes = [vp, vp, vp, vp, ci, ci, ci, ll, ll, ci, vp, ci, vp]
    lib.vattn_forward_rope_f16.restype = ci
    lib.vattn_status_string.argtypes = [ci]
    lib.vattn_status_string.restype = ctypes.c_char_p
    lib.vattn_last_hip_error.argtypes = []
    lib.vattn_last_hip_error.restype = ci
    lib.vattn_launch_shape.argtypes = [ci, ci, ci, ci, ci]
    lib.vattn_launch_shape.restype = ci
    return lib


lib = _load()


def _mode(precision: str | int) -> int:
    """C precision code of "auto", "fast" or "split" (an int passes through:
    the library rejects unknown codes with VATTN_ERR_ARG)."""
    if isinstance(precision, str):
        if precision not in PRECISION:
            raise ValueError("precision must be one of %s, got %r"
                             % (sorted(PRECISION), precision))
        return PRECISION[precision]
    return int(precision)


def forward_raw(q_ptr: int, k_ptr: int, v_ptr: int, out_ptr: int, n_heads: int,
                n_patches: int, head_dim: int, stream: int = 0,
                precision: str | int = "auto") -> int:
    """Direct call of ``vattn_forward_precision`` with raw device pointers.
    Returns the status code (no exception)."""
    mode = _mode(precision)
    return lib.vattn_forward_precision(q_ptr or None, k_ptr or None, v_ptr or None,
                                       out_ptr or None, int(n_heads), int(n_patches),
                                       int(head_dim), mode, stream or None)


def forward_strided_raw(q_ptr: int, k_ptr: int, v_ptr: int, out_ptr: int, n_heads: int,
                        n_patches: int, head_dim: int, stride_head: int, stride_patch: int,
                        stream: int = 0, precision: str | int = "auto") -> int:
    """Direct call of ``vattn_forward_strided`` (strides in floats); returns
    the status code."""
    mode = _mode(precision)
    return lib.vattn_forward_strided(q_ptr or None, k_ptr or None, v_ptr or None,
                                     out_ptr or None, int(n_heads), int(n_patches),
                                     int(head_dim), int(stride_head), int(stride_patch),
                                     mode, stream or None)


def forward_f16_raw(q_ptr: int, k_ptr: int, v_ptr: int, out_ptr: int, n_heads: int,
                    n_patches: int, head_dim: int, stride_head: int, stride_patch: int,
                    stream: int = 0, precision: str | int = "auto") -> int:
    """Direct call of ``vattn_forward_f16`` (f16 tensors, strides in
    elements); returns the status code."""
    mode = _mode(precision)
    return lib.vattn_forward_f16(q_ptr or None, k_ptr or None, v_ptr or None,
                                 out_ptr or None, int(n_heads), int(n_patches),
                                 int(head_dim), int(stride_head), int(stride_patch),
                                 mode, stream or None)


def rope_table_raw(table_ptr: int, n_positions: int, rope_dims: int, base: float,
                   factors=None, pos_offset: int = 0, stream: int = 0) -> int:
    """Direct call of ``vattn_rope_table``; ``factors`` is a host sequence of
    rope_dims/2 floats or None.  Returns the status code."""
    fac = None
    if factors is not None:
        vals = [float(x) for x in factors]
        # the library reads rope_dims/2 values from this host array
        if len(vals) != int(rope_dims) // 2 or len(vals) == 0:
            raise ValueError("factors must hold rope_dims/2 = %d values, got %d"
                             % (int(rope_dims) // 2, len(vals)))
        fac = (ctypes.c_float * len(vals))(*vals)
    return lib.vattn_rope_table(table_ptr or None, int(n_positions), int(rope_dims),
                                float(base),
                                None if fac is None else ctypes.cast(fac, ctypes.c_void_p),
                                int(pos_offset), stream or None)


def forward_rope_raw(q_ptr: int, k_ptr: int, v_ptr: int, out_ptr: int, n_heads: int,
                     n_patches: int, head_dim: int, stride_head: int, stride_patch: int,
                     rope_dims: int, table_ptr: int, stream: int = 0,
                     precision: str | int = "auto", f16: bool = False) -> int:
    """Direct call of ``vattn_forward_rope`` (or ``vattn_forward_rope_f16``);
    returns the status code."""
    mode = _mode(precision)
    fn = lib.vattn_forward_rope_f16 if f16 else lib.vattn_forward_rope
    return fn(q_ptr or None, k_ptr or None, v_ptr or None, out_ptr or None, int(n_heads),
              int(n_patches), int(head_dim), int(stride_head), int(stride_patch),
              int(rope_dims), table_ptr or None, mode, stream or None)


def rope_table(n_positions: int, rope_dims: int, base: float = 10000.0, factors=None,
               pos_offset: int = 0, device=None,
               stream: torch.cuda.Stream | None = None) -> torch.Tensor:
    """(cos, sin) table of the NeoX rotary angles, float32
    ``[n_positions, rope_dims // 2, 2]`` on ``device`` (default: current):
    row n is position ``pos_offset + n``, pair i turns by
    pos * base^(-2i/rope_dims) / factors[i].  Enqueued on ``stream``."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None \
        else torch.device(device)
    table = torch.empty((int(n_positions), int(rope_dims) // 2, 2), dtype=torch.float32,
                        device=dev)
    with torch.cuda.device(dev):
        s = stream if stream is not None else torch.cuda.current_stream()
        rc = rope_table_raw(table.data_ptr(), n_positions, rope_dims, base, factors,
                            pos_offset, s.cuda_stream)
    if rc != VATTN_OK:
        raise VattnError(rc, lib)
    return table


def launch_shape(n_heads: int, n_patches: int, head_dim: int, rope: bool = False,
                 cu_count: int = 256) -> int:
    """Workgroup shape ``vattn_launch_shape`` picks (host-only, no device):
    SHAPE_SPLIT_KEYS, SHAPE_4_WAVES, SHAPE_8_WAVES or SHAPE_16_WAVES, or a
    negative status for invalid sizes."""
    return lib.vattn_launch_shape(int(n_heads), int(n_patches), int(head_dim), int(bool(rope)),
                                  int(cu_count))


def vattn_forward(q_ptr: int, k_ptr: int, v_ptr: int, out_ptr: int, n_heads: int,
                  n_patches: int, head_dim: int, stream: int = 0) -> int:
    """Direct call of the C entry point ``vattn_forward``; returns its status."""
    return lib.vattn_forward(q_ptr or None, k_ptr or None, v_ptr or None,
                             out_ptr or None, int(n_heads), int(n_patches),
                             int(head_dim), stream or None)


def _check(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype not in (torch.float32, torch.float16):
        raise TypeError("%s must be float32 or float16, got %s" % (name, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on a HIP device" % name)
    if t.dim() != 3:
        raise ValueError("%s must be [n_heads, n_patches, head_dim]" % name)
    if t.shape[2] > 1 and t.stride(2) != 1:
        raise ValueError("%s must have a contiguous last (head_dim) dimension" % name)


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            out: torch.Tensor | None = None, precision: str = "auto",
            stream: torch.cuda.Stream | None = None,
            rope: torch.Tensor | None = None) -> torch.Tensor:
    """out[h] = softmax(q[h] @ k[h]^T) @ v[h] for every head (no scale inside).

    q, k, v, out: float32 (or all float16) [n_heads, n_patches, head_dim] on one device,
    head_dim <= 64, last dimension contiguous and the same strides for all
    four (contiguous head-major tensors, or e.g. patch-major [N, H, d]
    tensors viewed as ``x.transpose(0, 1)``).  ``out`` defaults to a new
    tensor with q's strides.  ``rope``: a table from ``rope_table`` with at
    least n_patches rows; q and k are then rotated (patch i with row i)
    inside the kernel.  Enqueued on ``stream`` (default: torch's current
    stream); returns ``out`` without synchronising.
    """
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch.Tensor" % name)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v dtypes differ: %s %s %s" % (q.dtype, k.dtype, v.dtype))
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, name)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v shapes differ: %s %s %s" % (q.shape, k.shape, v.shape))
    if out is None:
        out = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
    _check(out, "out")
    if out.dtype != q.dtype:
        raise TypeError("out dtype %s != %s" % (out.dtype, q.dtype))
    if out.shape != q.shape:
        raise ValueError("out shape %s != %s" % (out.shape, q.shape))
    devs = {q.device, k.device, v.device, out.device}
    if len(devs) != 1:
        raise ValueError("tensors on different devices: %s" % devs)
    h, n, d = q.shape
    strides = {t.stride()[:2] for t in (q, k, v, out)}
    if len(strides) != 1:
        raise ValueError("q, k, v and out must share their strides: %s" % strides)
    sh, sn = strides.pop()
    if rope is not None:
        if not isinstance(rope, torch.Tensor) or rope.dtype != torch.float32 or \
                rope.dim() != 3 or rope.shape[2] != 2 or not rope.is_contiguous():
            raise ValueError("rope must be a contiguous float32 [positions, rope_dims/2, 2] "
                             "table from rope_table()")
        if rope.device != q.device:
            raise ValueError("rope table on %s, tensors on %s" % (rope.device, q.device))
        if rope.shape[0] < n:
            raise ValueError("rope table has %d rows for %d patches" % (rope.shape[0], n))
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream()
        if rope is not None:
            rc = forward_rope_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  h, n, d, sh, sn, 2 * rope.shape[1], rope.data_ptr(),
                                  s.cuda_stream, precision, f16=q.dtype == torch.float16)
        elif q.dtype == torch.float16:
            rc = forward_f16_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 h, n, d, sh, sn, s.cuda_stream, precision)
        elif q.is_contiguous():
            rc = forward_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             h, n, d, s.cuda_stream, precision)
        else:
            rc = forward_strided_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     h, n, d, sh, sn, s.cuda_stream, precision)
    if rc != VATTN_OK:
        raise VattnError(rc, lib)
    return out
