"""fp32 GEMM and GEMV on one AMD Instinct MI355X, through libmm's C ABI.

The functions named like the C entry points (mm_gemm_f32, mm_gemv_f32, ...)
marshal their arguments and call libmm.so; every step of the computation runs in
the library's HIP kernels. Pointer arguments accept a device address (int) or a
torch tensor on the GPU; `stream` accepts a hipStream_t address (int), a
torch.cuda.Stream, or None for torch's current stream on the current device.

gemm(A, B, out=None), gemv(A, x, out=None), conv2d(x, w, ...) etc. are conveniences for torch tensors:
they check dtypes, devices and strides, allocate the output with torch when none
is given, and call the C entry points. PyTorch only provides device memory and
streams here.

There is no fallback: if libmm.so is missing or fails to load, every call raises.
Build it with `python -m tiled_gemm_gemv_amd.build`.
"""
import ctypes
import os

# the library build.py writes (not imported from there, so that `python -m
# tiled_gemm_gemv_amd.build` runs the module once)
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmm.so")

MM_OK = 0
MM_ERR_INVALID_ARG = 1
MM_ERR_NO_DEVICE = 2
MM_ERR_LAUNCH = 3


class MMError(RuntimeError):
    """A libmm call returned a non-zero status."""

    def __init__(self, status, where, detail=""):
        self.status = status
        text = _lib_or_none().mm_status_string(status).decode() if _lib_or_none() else str(status)
        msg = f"{where}: {text} (status {status})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)


_lib = None


def _lib_or_none():
    return _lib


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libmm.so (once). Raises OSError if it is missing or cannot be loaded."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise OSError(f"{_LIB_PATH} is not built; run `python -m tiled_gemm_gemv_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.mm_gemm_f32.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.mm_gemm_f32.restype = ci
    lib.mm_gemm_f32_config.argtypes = [ci, i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.mm_gemm_f32_config.restype = ci
    lib.mm_gemm_f32_num_configs.argtypes = []
    lib.mm_gemm_f32_num_configs.restype = ci
    lib.mm_gemm_f32_config_name.argtypes = [ci]
    lib.mm_gemm_f32_config_name.restype = ctypes.c_char_p
    lib.mm_gemm_f32_select.argtypes = [i64, i64, i64]
    lib.mm_gemm_f32_select.restype = ci
    lib.mm_gemm_f32_batched.argtypes = [i64, i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64,
                                        i64, vp]
    lib.mm_gemm_f32_batched.restype = ci
    for name in ("mm_gemm_bf16", "mm_gemm_f16"):
        getattr(lib, name).argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
        getattr(lib, name).restype = ci
    for name in ("mm_gemm_bf16_config", "mm_gemm_f16_config"):
        getattr(lib, name).argtypes = [ci, i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
        getattr(lib, name).restype = ci
    lib.mm_gemm_h16_num_configs.argtypes = []
    lib.mm_gemm_h16_num_configs.restype = ci
    lib.mm_gemm_h16_config_name.argtypes = [ci]
    lib.mm_gemm_h16_config_name.restype = ctypes.c_char_p
    lib.mm_gemm_h16_select.argtypes = [i64, i64, i64]
    lib.mm_gemm_h16_select.restype = ci
    lib.mm_gemv_f32.argtypes = [i64, i64, vp, vp, vp, vp]
    lib.mm_gemv_t_f32.argtypes = [i64, i64, vp, vp, vp, vp]
    lib.mm_gemv_t_f32.restype = ci
    lib.mm_gemm_f32_workspace_bytes.argtypes = [i64, i64, i64]
    lib.mm_gemm_f32_workspace_bytes.restype = i64
    lib.mm_gemm_f32_ws.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.mm_gemm_f32_ws.restype = ci
    lib.mm_gemm_f32_ws_static.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.mm_gemm_f32_ws_static.restype = ci
    lib.mm_gemv_t_f32_workspace_bytes.argtypes = [i64, i64]
    lib.mm_gemv_t_f32_workspace_bytes.restype = i64
    lib.mm_gemv_t_f32_ws.argtypes = [i64, i64, vp, vp, vp, vp, i64, vp]
    lib.mm_gemv_t_f32_ws.restype = ci
    lib.mm_gemv_f32.restype = ci
    conv_args = [i64] * 13 + [vp, vp, vp, vp]
    lib.mm_conv2d_f32.argtypes = conv_args
    lib.mm_conv2d_f32.restype = ci
    lib.mm_conv2d_f32_config.argtypes = [ci] + conv_args
    lib.mm_conv2d_f32_config.restype = ci
    lib.mm_conv2d_out_dim.argtypes = [i64] * 5
    lib.mm_conv2d_out_dim.restype = i64
    lib.mm_conv2d_f32_num_configs.argtypes = []
    lib.mm_conv2d_f32_num_configs.restype = ci
    lib.mm_conv2d_f32_config_name.argtypes = [ci]
    lib.mm_conv2d_f32_config_name.restype = ctypes.c_char_p
    lib.mm_conv2d_f32_select.argtypes = [i64] * 13
    lib.mm_conv2d_f32_select.restype = ci
    lib.mm_status_string.argtypes = [ci]
    lib.mm_status_string.restype = ctypes.c_char_p
    lib.mm_last_error.argtypes = []
    lib.mm_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ----------------------------------------------------------------- marshalling

def _addr(p):
    """Device address of an int, None or torch tensor."""
    if p is None:
        return None
    if isinstance(p, int):
        return p or None
    if hasattr(p, "data_ptr"):
        return p.data_ptr() or None
    raise TypeError(f"expected a device address or a tensor, got {type(p).__name__}")


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(s, int):
        return s or None
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream or None
    raise TypeError(f"expected a stream address or torch.cuda.Stream, got {type(s).__name__}")


def _check(status, where):
    if status != MM_OK:
        raise MMError(status, where, load().mm_last_error().decode())


# ------------------------------------------------------- C entry points by name

def mm_gemm_f32(M, N, K, A, lda, B, ldb, C, ldc, stream=None):
    """C = A x B (row-major, leading dimensions lda, ldb, ldc). Raises MMError."""
    lib = load()
    _check(lib.mm_gemm_f32(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc,
                           _stream(stream)), "mm_gemm_f32")


def mm_gemm_f32_config(cfg, M, N, K, A, lda, B, ldb, C, ldc, stream=None):
    """mm_gemm_f32 with tile configuration `cfg` forced. Raises MMError."""
    lib = load()
    _check(lib.mm_gemm_f32_config(cfg, M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc,
                                  _stream(stream)), "mm_gemm_f32_config")


def mm_gemm_f32_batched(batch, M, N, K, A, lda, stride_a, B, ldb, stride_b, C, ldc, stride_c,
                        stream=None):
    """C_b = A_b x B_b for b < batch, operands offset by b * stride. Raises MMError."""
    lib = load()
    _check(lib.mm_gemm_f32_batched(batch, M, N, K, _addr(A), lda, stride_a, _addr(B), ldb,
                                   stride_b, _addr(C), ldc, stride_c, _stream(stream)),
           "mm_gemm_f32_batched")


def mm_gemm_bf16(M, N, K, A, lda, B, ldb, C, ldc, stream=None):
    """C (fp32) = A x B with bf16 A and B. Raises MMError."""
    lib = load()
    _check(lib.mm_gemm_bf16(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc,
                            _stream(stream)), "mm_gemm_bf16")


def mm_gemm_f16(M, N, K, A, lda, B, ldb, C, ldc, stream=None):
    """C (fp32) = A x B with fp16 A and B. Raises MMError."""
    lib = load()
    _check(lib.mm_gemm_f16(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc,
                           _stream(stream)), "mm_gemm_f16")


def mm_gemm_bf16_config(cfg, M, N, K, A, lda, B, ldb, C, ldc, stream=None):
    lib = load()
    _check(lib.mm_gemm_bf16_config(cfg, M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc,
                                   _stream(stream)), "mm_gemm_bf16_config")


def mm_gemm_f16_config(cfg, M, N, K, A, lda, B, ldb, C, ldc, stream=None):
    lib = load()
    _check(lib.mm_gemm_f16_config(cfg, M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc,
                                  _stream(stream)), "mm_gemm_f16_config")


def mm_gemm_h16_num_configs():
    return load().mm_gemm_h16_num_configs()


def mm_gemm_h16_config_name(cfg):
    name = load().mm_gemm_h16_config_name(cfg)
    return name.decode() if name is not None else None


def mm_gemm_h16_select(M, N, K):
    return load().mm_gemm_h16_select(M, N, K)


def mm_gemv_f32(M, N, A, x, y, stream=None):
    """y = A x (A M x N with packed rows). Raises MMError."""
    lib = load()
    _check(lib.mm_gemv_f32(M, N, _addr(A), _addr(x), _addr(y), _stream(stream)), "mm_gemv_f32")


def mm_gemv_t_f32(M, N, A, x, y, stream=None):
    """y = A^T x (A M x N with packed rows, x of M, y of N). Raises MMError."""
    lib = load()
    _check(lib.mm_gemv_t_f32(M, N, _addr(A), _addr(x), _addr(y), _stream(stream)),
           "mm_gemv_t_f32")


def mm_gemm_f32_workspace_bytes(M, N, K):
    """Bytes of workspace mm_gemm_f32_ws needs for (M, N, K); -1 for invalid sizes."""
    return load().mm_gemm_f32_workspace_bytes(M, N, K)


def mm_gemm_f32_ws(M, N, K, A, lda, B, ldb, C, ldc, workspace, workspace_bytes, stream=None):
    """C = A B, splitting K across workgroups through `workspace` where that pays.
    Raises MMError."""
    lib = load()
    _check(lib.mm_gemm_f32_ws(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc, _addr(workspace),
                              workspace_bytes, _stream(stream)), "mm_gemm_f32_ws")


def mm_gemm_f32_ws_static(M, N, K, A, lda, B, ldb, C, ldc, stream=None):
    """mm_gemm_f32_ws with the library's static device scratch (MM_STATIC_SCRATCH_BYTES per
    GPU) as its workspace: allocates nothing. Calls that overlap on one GPU race.
    Raises MMError."""
    lib = load()
    _check(lib.mm_gemm_f32_ws_static(M, N, K, _addr(A), lda, _addr(B), ldb, _addr(C), ldc,
                                     _stream(stream)), "mm_gemm_f32_ws_static")


MM_STATIC_SCRATCH_BYTES = 16 * 1024 * 1024  # as include/mm.h defines it


def mm_gemv_t_f32_workspace_bytes(M, N):
    """Bytes of workspace mm_gemv_t_f32_ws needs for (M, N); -1 for invalid sizes."""
    return load().mm_gemv_t_f32_workspace_bytes(M, N)


def mm_gemv_t_f32_ws(M, N, A, x, y, workspace, workspace_bytes, stream=None):
    """y = A^T x reading A along whole rows, partial sums in `workspace`. Raises MMError."""
    lib = load()
    _check(lib.mm_gemv_t_f32_ws(M, N, _addr(A), _addr(x), _addr(y), _addr(workspace), workspace_bytes,
                                _stream(stream)), "mm_gemv_t_f32_ws")


def mm_gemm_f32_num_configs():
    return load().mm_gemm_f32_num_configs()


def mm_gemm_f32_config_name(cfg):
    name = load().mm_gemm_f32_config_name(cfg)
    return name.decode() if name is not None else None


def mm_gemm_f32_select(M, N, K):
    return load().mm_gemm_f32_select(M, N, K)


def mm_conv2d_f32(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, x, w, y, stream=None):
    """2-D convolution, x N x C x H x W, w K x C x R x S, y N x K x P x Q (packed).
    Raises MMError."""
    lib = load()
    _check(lib.mm_conv2d_f32(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, _addr(x), _addr(w),
                             _addr(y), _stream(stream)), "mm_conv2d_f32")


def mm_conv2d_f32_config(cfg, N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, x, w, y, stream=None):
    lib = load()
    _check(lib.mm_conv2d_f32_config(cfg, N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, _addr(x),
                                    _addr(w), _addr(y), _stream(stream)), "mm_conv2d_f32_config")


def mm_conv2d_out_dim(in_, filter_, stride, pad, dil):
    return load().mm_conv2d_out_dim(in_, filter_, stride, pad, dil)


def mm_conv2d_f32_num_configs():
    return load().mm_conv2d_f32_num_configs()


def mm_conv2d_f32_config_name(cfg):
    name = load().mm_conv2d_f32_config_name(cfg)
    return name.decode() if name is not None else None


def mm_conv2d_f32_select(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw):
    return load().mm_conv2d_f32_select(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw)


def mm_status_string(status):
    return load().mm_status_string(status).decode()


def mm_last_error():
    return load().mm_last_error().decode()


# ----------------------------------------------------- torch-tensor front ends

def _on_device(device, **tensors):
    """Raise ValueError unless every given tensor is on `device` (a host tensor's address
    handed to a kernel would fault the GPU)."""
    for name, t in tensors.items():
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _workspace_bytes(ws, device):
    """Size in bytes of a workspace tensor, which must be contiguous and on `device`."""
    if not hasattr(ws, "data_ptr"):
        raise TypeError(f"workspace must be a torch.Tensor, got {type(ws).__name__}")
    if ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, the operands on {device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws.numel() * ws.element_size()


def _matrix(t, name, dtypes=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    dtypes = dtypes or (torch.float32,)
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    ld = t.stride(0) if rows > 1 else max(cols, 1)
    if ld < max(cols, 1):
        raise ValueError(f"{name} row stride {ld} is below its width {cols}")
    return ld


def gemm_workspace(M, N, K, device):
    """A device buffer of the size mm_gemm_f32_ws needs for (M, N, K) (None if none)."""
    import torch
    n = mm_gemm_f32_workspace_bytes(M, N, K)
    if n < 0:
        raise ValueError(f"invalid sizes {M} x {N} x {K}")
    return torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None


def gemm(A, B, out=None, config=None, stream=None, workspace=None):
    """out = A @ B for fp32 GPU tensors (any row strides, unit column stride). With
    `workspace` (a device tensor of at least mm_gemm_f32_workspace_bytes bytes, e.g. from
    gemm_workspace) it runs mm_gemm_f32_ws; with workspace="static", mm_gemm_f32_ws_static
    (the library's own device scratch; calls that overlap on one GPU race)."""
    import torch
    lda = _matrix(A, "A")
    ldb = _matrix(B, "B")
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {tuple(A.shape)} x {tuple(B.shape)}")
    if B.device != A.device:
        raise ValueError("A and B are on different devices")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(M, N)}")
    ldc = _matrix(out, "out")
    _on_device(A.device, out=out)
    if workspace is not None and config is not None:
        raise ValueError("a workspace and a forced config do not go together")
    with torch.cuda.device(A.device):
        if isinstance(workspace, str):
            if workspace != "static":
                raise ValueError(f"workspace must be a tensor or 'static', got {workspace!r}")
            mm_gemm_f32_ws_static(M, N, K, A, lda, B, ldb, out, ldc, stream)
        elif workspace is not None:
            mm_gemm_f32_ws(M, N, K, A, lda, B, ldb, out, ldc, workspace,
                           _workspace_bytes(workspace, A.device), stream)
        elif config is None:
            mm_gemm_f32(M, N, K, A, lda, B, ldb, out, ldc, stream)
        else:
            mm_gemm_f32_config(config, M, N, K, A, lda, B, ldb, out, ldc, stream)
    return out


def gemm_batched(A, B, out=None, stream=None):
    """out[b] = A[b] @ B[b] for 3-D fp32 GPU tensors (batch, rows, cols) whose last
    dimension has unit stride; a batch stride of 0 (e.g. from expand) shares an operand."""
    import torch
    for t, name in ((A, "A"), (B, "B")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 3:
            raise TypeError(f"{name} must be a 3-D float32 tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU")
    batch, M, K = A.shape
    batch2, K2, N = B.shape
    if batch2 != batch or K2 != K:
        raise ValueError(f"shapes differ: {tuple(A.shape)} x {tuple(B.shape)}")
    if out is None:
        out = torch.empty((batch, M, N), dtype=torch.float32, device=A.device)
    lda = _matrix(A[0] if batch else A.new_empty((M, K)), "A")
    ldb = _matrix(B[0] if batch else B.new_empty((K, N)), "B")
    ldc = _matrix(out[0] if batch else out.new_empty((M, N)), "out")
    _on_device(A.device, B=B, out=out)
    with torch.cuda.device(A.device):
        mm_gemm_f32_batched(batch, M, N, K, A, lda, A.stride(0), B, ldb, B.stride(0), out, ldc,
                            out.stride(0), stream)
    return out


def gemm16(A, B, out=None, config=None, stream=None):
    """out (fp32) = A @ B for bf16 or fp16 GPU tensors A and B of the same dtype."""
    import torch
    lda = _matrix(A, "A", (torch.bfloat16, torch.float16))
    ldb = _matrix(B, "B", (A.dtype,))
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {tuple(A.shape)} x {tuple(B.shape)}")
    if B.device != A.device:
        raise ValueError("A and B are on different devices")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(M, N)}")
    ldc = _matrix(out, "out")
    _on_device(A.device, out=out)
    bf = A.dtype == torch.bfloat16
    with torch.cuda.device(A.device):
        if config is None:
            (mm_gemm_bf16 if bf else mm_gemm_f16)(M, N, K, A, lda, B, ldb, out, ldc, stream)
        else:
            (mm_gemm_bf16_config if bf else mm_gemm_f16_config)(config, M, N, K, A, lda, B, ldb,
                                                                 out, ldc, stream)
    return out


def gemv(A, x, out=None, stream=None):
    """out = A @ x for an fp32 GPU matrix with packed rows and a contiguous vector."""
    import torch
    _matrix(A, "A")
    M, N = A.shape
    if not A.is_contiguous():
        raise ValueError("A must have packed rows (contiguous)")
    if x.dtype != torch.float32 or x.dim() != 1 or x.shape[0] != N or not x.is_contiguous():
        raise ValueError(f"x must be a contiguous float32 vector of {N} entries")
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=A.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (M,) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous float32 vector of {M} entries")
    _on_device(A.device, x=x, out=out)
    with torch.cuda.device(A.device):
        mm_gemv_f32(M, N, A, x, out, stream)
    return out


def gemv_t_workspace(M, N, device):
    """A device buffer of the size mm_gemv_t_f32_ws needs for (M, N) (None if none)."""
    import torch
    n = mm_gemv_t_f32_workspace_bytes(M, N)
    if n < 0:
        raise ValueError(f"invalid sizes {M} x {N}")
    return torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None


def gemv_t(A, x, out=None, workspace=None, stream=None):
    """out = A.T @ x for an fp32 GPU matrix with packed rows and a contiguous vector.
    With `workspace` (a device tensor of at least mm_gemv_t_f32_workspace_bytes bytes,
    e.g. from gemv_t_workspace) it runs mm_gemv_t_f32_ws."""
    import torch
    _matrix(A, "A")
    M, N = A.shape
    if not A.is_contiguous():
        raise ValueError("A must have packed rows (contiguous)")
    if x.dtype != torch.float32 or x.dim() != 1 or x.shape[0] != M or not x.is_contiguous():
        raise ValueError(f"x must be a contiguous float32 vector of {M} entries")
    if out is None:
        out = torch.empty(N, dtype=torch.float32, device=A.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (N,) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous float32 vector of {N} entries")
    _on_device(A.device, x=x, out=out)
    with torch.cuda.device(A.device):
        if workspace is None:
            mm_gemv_t_f32(M, N, A, x, out, stream)
        else:
            mm_gemv_t_f32_ws(M, N, A, x, out, workspace, _workspace_bytes(workspace, A.device), stream)
    return out


def conv2d(x, w, stride=(1, 1), pad=(0, 0), dilation=(1, 1), out=None, config=None, stream=None):
    """out = the 2-D convolution of x (N x C x H x W) with w (K x C x R x S), both
    contiguous fp32 GPU tensors; out is N x K x P x Q (allocated if not given)."""
    import torch
    for t, name in ((x, "x"), (w, "w")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.dim() != 4:
            raise TypeError(f"{name} must be a 4-D float32 tensor")
        if t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if w.device != x.device:
        raise ValueError("x and w are on different devices")
    N, C, H, W = x.shape
    K, C2, R, S = w.shape
    if C2 != C:
        raise ValueError(f"channel counts differ: x has {C}, w has {C2}")
    (sh, sw), (ph, pw), (dh, dw) = stride, pad, dilation
    P = mm_conv2d_out_dim(H, R, sh, ph, dh)
    Q = mm_conv2d_out_dim(W, S, sw, pw, dw)
    if P < 1 or Q < 1:
        raise ValueError("invalid convolution geometry (the filter must fit the padded input)")
    if out is None:
        out = torch.empty((N, K, P, Q), dtype=torch.float32, device=x.device)
    if (out.dtype != torch.float32 or tuple(out.shape) != (N, K, P, Q) or not out.is_contiguous()
            or out.device != x.device):
        raise ValueError(f"out must be a contiguous float32 tensor of shape {(N, K, P, Q)}")
    with torch.cuda.device(x.device):
        if config is None:
            mm_conv2d_f32(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, x, w, out, stream)
        else:
            mm_conv2d_f32_config(config, N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, x, w, out,
                                 stream)
    return out
