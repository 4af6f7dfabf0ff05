"""int8_gemm_linear_amd -- MI355X (gfx950) quantized linear-layer GEMM.

Thin Python binding over the C ABI of ``libqlinear.so`` (``include/qlinear.h``):
argument marshalling only.  Every step of the computation runs in the HIP
kernels of the library; there is no CPU or PyTorch fallback, and every call
raises ImportError when the library has not been built
(``python -m int8_gemm_linear_amd.build``).  PyTorch supplies device memory
and the current stream.

    Y = scaled_mm(a_q, a_scale, b_q, b_scale)          # FP8_Dynamic / W8A8_INT8
    Y = block_scaled_mm(a_q, a_scale, b_q, b_scale)    # Block_FP8

``a_q`` [M,K] and ``b_q`` [N,K] (torch.float8_e4m3fn or torch.int8, rows
K-contiguous); fp32 scales ``a_scale`` [M] and ``b_scale`` [N], or for the
block format ``a_scale`` [M, K/128] and ``b_scale`` [N/128, K/128]; the
result is bfloat16 [M,N].  Formats per "Building a High-Performance and
Portable vLLM Linear Backend with Helion", section "Helion Linear Backend /
Scope".
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import asdict, dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlinear.so")

E4M3, INT8 = 0, 1
TOKEN_CHANNEL, BLOCK128 = 0, 1
KERNEL_STREAM, KERNEL_TILE, KERNEL_STREAM_LDS, KERNEL_GEMV, KERNEL_STREAM_TOK = 0, 1, 2, 3, 4
STANDARD, SWAP_AB = 0, 1
REDUCE_TWO_PASS, REDUCE_LAST_ARRIVER = 0, 1

_STATUS = {0: "ok", 1: "null pointer", 2: "bad shape", 3: "bad leading dimension",
           4: "misaligned pointer", 5: "workspace", 6: "bad config", 7: "config file",
           8: "HIP launch failed", 9: "bad argument"}


class QlinError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_lib().qlin_status_string(status).decode()} (status {status})")


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "kernel", "variant", "tile_m", "tile_n", "tile_k", "waves_n", "waves_k",
        "stages", "split_k", "reduce")]


@dataclass(frozen=True)
class Config:
    """One launch configuration (mirrors ``qlin_config``)."""
    kernel: int
    variant: int
    tile_m: int
    tile_n: int
    tile_k: int
    waves_n: int
    waves_k: int
    stages: int
    split_k: int = 1
    reduce: int = REDUCE_LAST_ARRIVER

    def _c(self) -> _Cfg:
        return _Cfg(**asdict(self))

    @staticmethod
    def _from_c(c: _Cfg) -> "Config":
        return Config(**{f: getattr(c, f) for f, _ in _Cfg._fields_})

    def replace(self, **kw) -> "Config":
        d = asdict(self)
        d.update(kw)
        return Config(**d)


_LIB = None


def _check_single_hip_runtime():
    # torch ships its own libamdhip64; the library must bind to that same
    # runtime (it does: both carry the soname libamdhip64.so.7 and torch is
    # loaded first).  Two runtimes in one process would not share streams.
    try:
        with open("/proc/self/maps") as f:
            paths = {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    except OSError:
        return
    if len(paths) > 1:
        raise ImportError("two HIP runtimes are mapped into this process: " + ", ".join(sorted(paths)))


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m int8_gemm_linear_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    _check_single_hip_runtime()
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    I = ctypes.c_int
    CP = ctypes.POINTER(_Cfg)
    lib.qlin_scaled_mm_cfg.argtypes = [I, I64, I64, I64, P, I64, P, P, I64, P, P, I64, P, SZ, P, CP]
    lib.qlin_scaled_mm_cfg.restype = I
    lib.qlin_scaled_mm.argtypes = [I, I64, I64, I64, P, I64, P, P, I64, P, P, I64, P, SZ, P]
    lib.qlin_scaled_mm.restype = I
    lib.qlin_block_scaled_mm_cfg.argtypes = [I64, I64, I64, P, I64, P, P, I64, P, P, I64, P, SZ, P, CP]
    lib.qlin_block_scaled_mm_cfg.restype = I
    lib.qlin_block_scaled_mm.argtypes = [I64, I64, I64, P, I64, P, P, I64, P, P, I64, P, SZ, P]
    lib.qlin_block_scaled_mm.restype = I
    lib.qlin_int8_accumulate.argtypes = [I64, I64, I64, P, I64, P, I64, P, I64, P, SZ, P, CP]
    lib.qlin_int8_accumulate.restype = I
    lib.qlin_select_config.argtypes = [I, I, I64, I64, I64, CP]
    lib.qlin_select_config.restype = I
    lib.qlin_check_config.argtypes = [I, I, I64, I64, I64, CP]
    lib.qlin_check_config.restype = I
    lib.qlin_workspace_size.argtypes = [I, I, I64, I64, I64, CP]
    lib.qlin_workspace_size.restype = SZ
    lib.qlin_kernel_instance.argtypes = [ctypes.c_int32, CP, ctypes.POINTER(ctypes.c_int32)]
    lib.qlin_kernel_instance.restype = I
    lib.qlin_load_config_table.argtypes = [ctypes.c_char_p]
    lib.qlin_load_config_table.restype = I
    lib.qlin_config_table_size.argtypes = []
    lib.qlin_config_table_size.restype = ctypes.c_int32
    lib.qlin_status_string.argtypes = [I]
    lib.qlin_status_string.restype = ctypes.c_char_p
    lib.qlin_abi_version.argtypes = []
    lib.qlin_abi_version.restype = ctypes.c_int32
    lib.qlin_scaled_mm_noalloc.argtypes = [I, I, I64, I64, I64, P, I64, P, P, I64, P, P, I64, P]
    lib.qlin_scaled_mm_noalloc.restype = I
    lib.qlin_stream_capture_id.argtypes = [P, ctypes.POINTER(ctypes.c_ulonglong)]
    lib.qlin_stream_capture_id.restype = ctypes.c_int32
    lib.qlin_quant_per_token.argtypes = [I, I64, I64, P, I64, P, I64, P, P]
    lib.qlin_quant_per_token.restype = I
    lib.qlin_quant_per_group128.argtypes = [I64, I64, P, I64, P, I64, P, P]
    lib.qlin_quant_per_group128.restype = I
    F = ctypes.c_float
    lib.qlin_grouped_scaled_mm.argtypes = [I, I64, P, I64, I64, I64, P, I64, P, P, I64, I64, P, I64,
                                           P, I64, P, CP]
    lib.qlin_grouped_scaled_mm.restype = I
    lib.qlin_grouped_block_scaled_mm.argtypes = [I64, P, I64, I64, I64, P, I64, P, P, I64, I64, P,
                                                 I64, P, I64, P, CP]
    lib.qlin_grouped_block_scaled_mm.restype = I
    lib.qlin_select_grouped_config.argtypes = [I, I, I64, I64, I64, CP]
    lib.qlin_select_grouped_config.restype = I
    lib.qlin_rms_norm_dynamic_per_token_quant.argtypes = [I, I64, I64, P, I64, P, I64, P, F, P, I64, P, P]
    lib.qlin_rms_norm_dynamic_per_token_quant.restype = I
    lib.qlin_rms_norm_per_block_quant.argtypes = [I64, I64, P, I64, P, I64, P, F, P, I64, P, P]
    lib.qlin_rms_norm_per_block_quant.restype = I
    lib.qlin_silu_and_mul_dynamic_per_token_quant.argtypes = [I, I64, I64, P, I64, P, I64, P, P]
    lib.qlin_silu_and_mul_dynamic_per_token_quant.restype = I
    lib.qlin_silu_and_mul_per_block_quant.argtypes = [I64, I64, P, I64, P, I64, P, P]
    lib.qlin_silu_and_mul_per_block_quant.restype = I
    _LIB = lib
    return lib


def lib():
    """The loaded ctypes handle of libqlinear.so."""
    return _lib()


# ---------------------------------------------------------------------------
# Split-K workspaces.  A workspace's counter region must hold zeros before
# its first use, and a HIP graph keeps using the workspace address it was
# captured with, so:
#  * eager calls use one zeroed buffer per (device, stream): calls on
#    different streams never share one;
#  * each graph capture gets buffers of its own, allocated and zeroed inside
#    the capture (torch's allocator serves them from the graph's pool and the
#    zero fill is a kernel node that runs before the first call of every
#    replay), so eager calls and other graphs never touch them;
#  * a buffer is never freed once a call has used it: when a call needs more,
#    a larger one replaces it and the old one is kept, because a graph
#    captured earlier may still replay with its address.
# Calls that may overlap in time on one stream cannot exist; graphs that may
# replay concurrently on different streams were captured separately and hold
# separate buffers.  A caller may always pass its own `workspace=` instead.
# ---------------------------------------------------------------------------
_WS: dict = {}
_WS_KEPT: list = []
COUNTER_BYTES = 128 * 1024      # the workspace's leading counter region (include/qlinear.h)


def _capture_id(stream) -> int:
    cid = ctypes.c_ulonglong(0)
    r = _lib().qlin_stream_capture_id(ctypes.c_void_p(stream.cuda_stream), ctypes.byref(cid))
    if r < 0:
        raise RuntimeError("could not query the stream's capture state")
    return int(cid.value) if r == 1 else 0


def workspace_for(nbytes: int, device: torch.device, stream=None) -> torch.Tensor | None:
    """A zeroed-counter workspace of at least `nbytes` for calls on `stream`
    (the device's current stream by default)."""
    if nbytes == 0:
        return None
    dev = device.index if device.index is not None else torch.cuda.current_device()
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    key = (dev, int(stream.cuda_stream), _capture_id(stream))
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        size = max(nbytes, 1 << 20, 2 * buf.numel() if buf is not None else 0)
        with torch.cuda.stream(stream):
            # only the counter region must start at zero (a fill kernel; the
            # split partials are always written before they are read)
            new = torch.empty(size, dtype=torch.uint8, device=torch.device("cuda", dev))
            new[:COUNTER_BYTES].zero_()
        if buf is not None:
            _WS_KEPT.append(buf)
        _WS[key] = buf = new
    return buf


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float8_e4m3fn:
        return E4M3
    if t.dtype == torch.int8:
        return INT8
    raise TypeError(f"operands must be float8_e4m3fn or int8, got {t.dtype}")


def _rows(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.stride(0)


def _scale(t: torch.Tensor, shape, name: str) -> torch.Tensor:
    if t.dtype != torch.float32 or not t.is_cuda:
        raise ValueError(f"{name} must be a float32 device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _call(fn, args, what):
    st = fn(*args)
    if st != 0:
        raise QlinError(st, what)


def scaled_mm(a_q, a_scale, b_q, b_scale, out=None, config: Config | None = None, workspace=None):
    """FP8_Dynamic (e4m3) or W8A8_INT8 (int8): bf16 [M,N] = sA[m] sB[n] (A B^T)."""
    dt = _dt(a_q)
    if b_q.dtype != a_q.dtype:
        raise TypeError("A and B must have the same dtype")
    lda, ldb = _rows(a_q, "a_q"), _rows(b_q, "b_q")
    M, K = a_q.shape
    N = b_q.shape[0]
    if b_q.shape[1] != K:
        raise ValueError("A is [M,K] and B must be [N,K]")
    _scale(a_scale, (M,), "a_scale")
    _scale(b_scale, (N,), "b_scale")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device)
    elif out.dtype != torch.bfloat16 or out.dim() != 2 or out.stride(1) != 1 or tuple(out.shape) != (M, N):
        raise ValueError("out must be a bf16 [M,N] tensor with contiguous rows")
    stream = torch.cuda.current_stream(a_q.device)
    c = config._c() if config is not None else None
    wsz = _lib().qlin_workspace_size(TOKEN_CHANNEL, dt, M, N, K, ctypes.byref(c) if c else None)
    ws = workspace if workspace is not None else workspace_for(wsz, a_q.device, stream)
    args = [dt, M, N, K, a_q.data_ptr(), lda, a_scale.data_ptr(), b_q.data_ptr(), ldb,
            b_scale.data_ptr(), out.data_ptr(), out.stride(0),
            ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
            stream.cuda_stream]
    if c is None:
        _call(_lib().qlin_scaled_mm, args, "qlin_scaled_mm")
    else:
        _call(_lib().qlin_scaled_mm_cfg, args + [ctypes.byref(c)], "qlin_scaled_mm_cfg")
    return out


def _bf16_rows(x: torch.Tensor, name: str) -> int:
    if x.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {x.dtype}")
    return _rows(x, name)


def quant_per_token(x, dtype=torch.float8_e4m3fn, out=None, scale=None):
    """Dynamic per-token quantization of bf16 activations x [M,K]: returns
    (codes [M,K] of `dtype` (float8_e4m3fn or int8), scales float32 [M]),
    scale = amax/448 (e4m3) or amax/127 (int8), codes = nearest-even of
    x/scale, clamped.  The outputs are scaled_mm's a_q and a_scale."""
    ldx = _bf16_rows(x, "x")
    M, K = x.shape
    dt = E4M3 if dtype == torch.float8_e4m3fn else (INT8 if dtype == torch.int8 else None)
    if dt is None:
        raise TypeError("dtype must be float8_e4m3fn or int8")
    if out is None:
        out = torch.empty((M, K), dtype=dtype, device=x.device)
    elif out.dtype != dtype or tuple(out.shape) != (M, K) or out.stride(1) != 1:
        raise ValueError("out must be a [M,K] tensor of dtype with contiguous rows")
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _scale(scale, (M,), "scale")
    stream = torch.cuda.current_stream(x.device)
    _call(_lib().qlin_quant_per_token, [dt, M, K, x.data_ptr(), ldx, out.data_ptr(), out.stride(0),
                                        scale.data_ptr(), stream.cuda_stream], "qlin_quant_per_token")
    return out, scale


def quant_per_group128(x, out=None, scale=None):
    """Per-token-group (1x128) e4m3 quantization of bf16 activations x [M,K]:
    returns (codes float8_e4m3fn [M,K], scales float32 [M, K/128]), the
    a_q and a_scale of block_scaled_mm."""
    ldx = _bf16_rows(x, "x")
    M, K = x.shape
    if out is None:
        out = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=x.device)
    elif out.dtype != torch.float8_e4m3fn or tuple(out.shape) != (M, K) or out.stride(1) != 1:
        raise ValueError("out must be a float8_e4m3fn [M,K] tensor with contiguous rows")
    if scale is None:
        scale = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    _scale(scale, (M, K // 128), "scale")
    stream = torch.cuda.current_stream(x.device)
    _call(_lib().qlin_quant_per_group128, [M, K, x.data_ptr(), ldx, out.data_ptr(), out.stride(0),
                                           scale.data_ptr(), stream.cuda_stream],
          "qlin_quant_per_group128")
    return out, scale


def _codes_out(out, dtype, M, K, device):
    if out is None:
        return torch.empty((M, K), dtype=dtype, device=device)
    if out.dtype != dtype or tuple(out.shape) != (M, K) or out.stride(1) != 1:
        raise ValueError(f"out must be a {dtype} [M,K] tensor with contiguous rows")
    return out


def _code_dtype(dtype):
    dt = E4M3 if dtype == torch.float8_e4m3fn else (INT8 if dtype == torch.int8 else None)
    if dt is None:
        raise TypeError("dtype must be float8_e4m3fn or int8")
    return dt


def _rms_args(x, weight, residual):
    ldx = _bf16_rows(x, "x")
    M, K = x.shape
    if weight.dtype != torch.bfloat16 or not weight.is_cuda or weight.dim() != 1 or weight.numel() != K or \
            weight.stride(0) != 1:
        raise ValueError("weight must be a contiguous bfloat16 vector of K elements")
    ldr = 0
    if residual is not None:
        ldr = _bf16_rows(residual, "residual")
        if tuple(residual.shape) != (M, K):
            raise ValueError("residual must be [M,K]")
    return ldx, M, K, ldr


def rms_norm_dynamic_per_token_quant(x, weight, eps=1e-6, dtype=torch.float8_e4m3fn,
                                     residual=None, out=None, scale=None):
    """RMS norm of bf16 x [M,K] with bf16 weight [K] (after x += residual,
    rounded to bf16 and written back into `residual`, when one is given),
    then dynamic per-token quantization: returns (codes [M,K], scales [M])."""
    ldx, M, K, ldr = _rms_args(x, weight, residual)
    dt = _code_dtype(dtype)
    out = _codes_out(out, dtype, M, K, x.device)
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _scale(scale, (M,), "scale")
    stream = torch.cuda.current_stream(x.device)
    _call(_lib().qlin_rms_norm_dynamic_per_token_quant,
          [dt, M, K, x.data_ptr(), ldx, None if residual is None else residual.data_ptr(), ldr,
           weight.data_ptr(), float(eps), out.data_ptr(), out.stride(0), scale.data_ptr(),
           stream.cuda_stream], "qlin_rms_norm_dynamic_per_token_quant")
    return out, scale


def rms_norm_per_block_quant(x, weight, eps=1e-6, residual=None, out=None, scale=None):
    """RMS norm as above, then per-token-group (1x128) e4m3 quantization:
    returns (codes float8_e4m3fn [M,K], scales float32 [M, K/128])."""
    ldx, M, K, ldr = _rms_args(x, weight, residual)
    out = _codes_out(out, torch.float8_e4m3fn, M, K, x.device)
    if scale is None:
        scale = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    _scale(scale, (M, K // 128), "scale")
    stream = torch.cuda.current_stream(x.device)
    _call(_lib().qlin_rms_norm_per_block_quant,
          [M, K, x.data_ptr(), ldx, None if residual is None else residual.data_ptr(), ldr,
           weight.data_ptr(), float(eps), out.data_ptr(), out.stride(0), scale.data_ptr(),
           stream.cuda_stream], "qlin_rms_norm_per_block_quant")
    return out, scale


def _silu_args(x):
    ldx = _bf16_rows(x, "x")
    M, K2 = x.shape
    if K2 % 2:
        raise ValueError("x must be [M, 2K] (gate | up)")
    return ldx, M, K2 // 2


def silu_and_mul_dynamic_per_token_quant(x, dtype=torch.float8_e4m3fn, out=None, scale=None):
    """SiLU(gate) * up of bf16 x [M, 2K] (gate | up), then dynamic per-token
    quantization: returns (codes [M,K], scales [M])."""
    ldx, M, K = _silu_args(x)
    dt = _code_dtype(dtype)
    out = _codes_out(out, dtype, M, K, x.device)
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _scale(scale, (M,), "scale")
    stream = torch.cuda.current_stream(x.device)
    _call(_lib().qlin_silu_and_mul_dynamic_per_token_quant,
          [dt, M, K, x.data_ptr(), ldx, out.data_ptr(), out.stride(0), scale.data_ptr(),
           stream.cuda_stream], "qlin_silu_and_mul_dynamic_per_token_quant")
    return out, scale


def silu_and_mul_per_block_quant(x, out=None, scale=None):
    """SiLU(gate) * up, then per-token-group (1x128) e4m3 quantization:
    returns (codes float8_e4m3fn [M,K], scales float32 [M, K/128])."""
    ldx, M, K = _silu_args(x)
    out = _codes_out(out, torch.float8_e4m3fn, M, K, x.device)
    if scale is None:
        scale = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    _scale(scale, (M, K // 128), "scale")
    stream = torch.cuda.current_stream(x.device)
    _call(_lib().qlin_silu_and_mul_per_block_quant,
          [M, K, x.data_ptr(), ldx, out.data_ptr(), out.stride(0), scale.data_ptr(),
           stream.cuda_stream], "qlin_silu_and_mul_per_block_quant")
    return out, scale


def block_scaled_mm(a_q, a_scale, b_q, b_scale, out=None, config: Config | None = None,
                    workspace=None):
    """Block_FP8: bf16 [M,N] = sum_g sA[m,g] sB[n/128,g] (A B^T over group g)."""
    if a_q.dtype != torch.float8_e4m3fn or b_q.dtype != torch.float8_e4m3fn:
        raise TypeError("block_scaled_mm takes float8_e4m3fn operands")
    lda, ldb = _rows(a_q, "a_q"), _rows(b_q, "b_q")
    M, K = a_q.shape
    N = b_q.shape[0]
    if b_q.shape[1] != K:
        raise ValueError("A is [M,K] and B must be [N,K]")
    G = K // 128
    _scale(a_scale, (M, G), "a_scale")
    _scale(b_scale, (N // 128, G), "b_scale")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device)
    elif out.dtype != torch.bfloat16 or out.dim() != 2 or out.stride(1) != 1 or tuple(out.shape) != (M, N):
        raise ValueError("out must be a bf16 [M,N] tensor with contiguous rows")
    stream = torch.cuda.current_stream(a_q.device)
    c = config._c() if config is not None else None
    wsz = _lib().qlin_workspace_size(BLOCK128, E4M3, M, N, K, ctypes.byref(c) if c else None)
    ws = workspace if workspace is not None else workspace_for(wsz, a_q.device, stream)
    args = [M, N, K, a_q.data_ptr(), lda, a_scale.data_ptr(), b_q.data_ptr(), ldb,
            b_scale.data_ptr(), out.data_ptr(), out.stride(0),
            ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
            stream.cuda_stream]
    if c is None:
        _call(_lib().qlin_block_scaled_mm, args, "qlin_block_scaled_mm")
    else:
        _call(_lib().qlin_block_scaled_mm_cfg, args + [ctypes.byref(c)], "qlin_block_scaled_mm_cfg")
    return out


def scaled_mm_noalloc(a_q, a_scale, b_q, b_scale, out, block: bool = False):
    """scaled_mm (block=False) or block_scaled_mm (block=True) through the
    library's allocation-free entry point: the split-K workspace is the
    library's own per-GPU device array, and `out` must be given (nothing is
    allocated).  Calls that overlap in time on one GPU must not be issued."""
    dt = _dt(a_q)
    if b_q.dtype != a_q.dtype:
        raise TypeError("A and B must have the same dtype")
    if block and dt != E4M3:
        raise TypeError("block scaling takes float8_e4m3fn operands")
    lda, ldb = _rows(a_q, "a_q"), _rows(b_q, "b_q")
    M, K = a_q.shape
    N = b_q.shape[0]
    if b_q.shape[1] != K:
        raise ValueError("A is [M,K] and B must be [N,K]")
    if block:
        _scale(a_scale, (M, K // 128), "a_scale")
        _scale(b_scale, (N // 128, K // 128), "b_scale")
    else:
        _scale(a_scale, (M,), "a_scale")
        _scale(b_scale, (N,), "b_scale")
    if out is None or out.dtype != torch.bfloat16 or out.dim() != 2 or out.stride(1) != 1 or \
            tuple(out.shape) != (M, N):
        raise ValueError("out must be a bf16 [M,N] tensor with contiguous rows")
    stream = torch.cuda.current_stream(a_q.device)
    _call(_lib().qlin_scaled_mm_noalloc,
          [BLOCK128 if block else TOKEN_CHANNEL, dt, M, N, K, a_q.data_ptr(), lda, a_scale.data_ptr(),
           b_q.data_ptr(), ldb, b_scale.data_ptr(), out.data_ptr(), out.stride(0), stream.cuda_stream],
          "qlin_scaled_mm_noalloc")
    return out


def _grouped_args(a_q, b_q, group_offsets, out):
    if b_q.dim() != 3 or b_q.stride(2) != 1 or not b_q.is_cuda:
        raise ValueError("b_q must be a [G,N,K] device tensor with contiguous rows")
    G, N, K = b_q.shape
    lda = _rows(a_q, "a_q")
    if a_q.shape[1] != K:
        raise ValueError("A is [rows,K] and B must be [G,N,K]")
    if group_offsets.dtype != torch.int32 or group_offsets.dim() != 1 or \
            group_offsets.numel() != G + 1 or not group_offsets.is_cuda or \
            not group_offsets.is_contiguous():
        raise ValueError("group_offsets must be a contiguous int32 device tensor of G+1 values")
    rows = a_q.shape[0]
    if out is None:
        out = torch.empty((rows, N), dtype=torch.bfloat16, device=a_q.device)
    elif out.dtype != torch.bfloat16 or out.dim() != 2 or out.stride(1) != 1 or \
            tuple(out.shape) != (rows, N):
        raise ValueError("out must be a bf16 [rows,N] tensor with contiguous rows")
    return G, N, K, lda, rows, out


def grouped_scaled_mm(a_q, a_scale, b_q, b_scale, group_offsets, max_rows: int, out=None,
                      config: Config | None = None):
    """Grouped (mixture-of-experts) FP8_Dynamic / W8A8_INT8: expert g computes
    rows group_offsets[g] .. group_offsets[g+1]-1 of A [rows,K] against its
    weights b_q[g] [N,K] with scales b_scale[g] [N]; bf16 out [rows,N].
    max_rows bounds any expert's row count."""
    dt = _dt(a_q)
    if b_q.dtype != a_q.dtype:
        raise TypeError("A and B must have the same dtype")
    G, N, K, lda, rows, out = _grouped_args(a_q, b_q, group_offsets, out)
    _scale(a_scale, (rows,), "a_scale")
    _scale(b_scale, (G, N), "b_scale")
    c = config._c() if config is not None else None
    stream = torch.cuda.current_stream(a_q.device)
    _call(_lib().qlin_grouped_scaled_mm,
          [dt, G, group_offsets.data_ptr(), int(max_rows), N, K, a_q.data_ptr(), lda,
           a_scale.data_ptr(), b_q.data_ptr(), b_q.stride(1), b_q.stride(0), b_scale.data_ptr(), N,
           out.data_ptr(), out.stride(0), stream.cuda_stream, ctypes.byref(c) if c else None],
          "qlin_grouped_scaled_mm")
    return out


def grouped_block_scaled_mm(a_q, a_scale, b_q, b_scale, group_offsets, max_rows: int, out=None,
                            config: Config | None = None):
    """Grouped Block_FP8: as grouped_scaled_mm with a_scale [rows, K/128] and
    b_scale [G, N/128, K/128]."""
    if a_q.dtype != torch.float8_e4m3fn or b_q.dtype != torch.float8_e4m3fn:
        raise TypeError("grouped_block_scaled_mm takes float8_e4m3fn operands")
    G, N, K, lda, rows, out = _grouped_args(a_q, b_q, group_offsets, out)
    _scale(a_scale, (rows, K // 128), "a_scale")
    _scale(b_scale, (G, N // 128, K // 128), "b_scale")
    c = config._c() if config is not None else None
    stream = torch.cuda.current_stream(a_q.device)
    _call(_lib().qlin_grouped_block_scaled_mm,
          [G, group_offsets.data_ptr(), int(max_rows), N, K, a_q.data_ptr(), lda,
           a_scale.data_ptr(), b_q.data_ptr(), b_q.stride(1), b_q.stride(0), b_scale.data_ptr(),
           (N // 128) * (K // 128), out.data_ptr(), out.stride(0), stream.cuda_stream,
           ctypes.byref(c) if c else None], "qlin_grouped_block_scaled_mm")
    return out


def int8_accumulate(a_q, b_q, config: Config | None = None, out=None):
    """Test hook: raw int32 A B^T of int8 operands (no scaling, no rounding)."""
    if a_q.dtype != torch.int8 or b_q.dtype != torch.int8:
        raise TypeError("int8_accumulate takes int8 operands")
    lda, ldb = _rows(a_q, "a_q"), _rows(b_q, "b_q")
    M, K = a_q.shape
    N = b_q.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.int32, device=a_q.device)
    stream = torch.cuda.current_stream(a_q.device)
    c = config._c() if config is not None else None
    wsz = _lib().qlin_workspace_size(TOKEN_CHANNEL, INT8, M, N, K, ctypes.byref(c) if c else None)
    ws = workspace_for(wsz, a_q.device, stream)
    _call(_lib().qlin_int8_accumulate,
          [M, N, K, a_q.data_ptr(), lda, b_q.data_ptr(), ldb, out.data_ptr(), out.stride(0),
           ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
           stream.cuda_stream, ctypes.byref(c) if c else None], "qlin_int8_accumulate")
    return out


FORMATS = {"fp8": (TOKEN_CHANNEL, E4M3), "int8": (TOKEN_CHANNEL, INT8), "block_fp8": (BLOCK128, E4M3)}


def select_config(fmt: str, M: int, N: int, K: int) -> Config:
    sc, dt = FORMATS[fmt]
    c = _Cfg()
    _call(_lib().qlin_select_config, [sc, dt, M, N, K, ctypes.byref(c)], "qlin_select_config")
    return Config._from_c(c)


def select_grouped_config(fmt: str, max_rows: int, N: int, K: int) -> Config:
    """The config a grouped call uses by default (split_k = 1)."""
    sc, dt = FORMATS[fmt]
    c = _Cfg()
    _call(_lib().qlin_select_grouped_config, [sc, dt, max_rows, N, K, ctypes.byref(c)],
          "qlin_select_grouped_config")
    return Config._from_c(c)


def check_config(fmt: str, M: int, N: int, K: int, config: Config) -> int:
    sc, dt = FORMATS[fmt]
    c = config._c()
    return _lib().qlin_check_config(sc, dt, M, N, K, ctypes.byref(c))


def workspace_size(fmt: str, M: int, N: int, K: int, config: Config | None = None) -> int:
    sc, dt = FORMATS[fmt]
    c = config._c() if config is not None else None
    return _lib().qlin_workspace_size(sc, dt, M, N, K, ctypes.byref(c) if c else None)


def kernel_instances():
    """[(Config, fmt_mask)] of every built kernel instance (bit0 fp8, bit1 int8, bit2 block)."""
    out = []
    i = 0
    c = _Cfg()
    m = ctypes.c_int32()
    while _lib().qlin_kernel_instance(i, ctypes.byref(c), ctypes.byref(m)) == 0:
        out.append((Config._from_c(c), m.value))
        i += 1
    return out


def instances_for(fmt: str):
    bit = {"fp8": 1, "int8": 2, "block_fp8": 4}[fmt]
    return [c for c, m in kernel_instances() if m & bit]


def load_config_table(path: str | None):
    _call(_lib().qlin_load_config_table, [path.encode() if path else None], "qlin_load_config_table")


def config_table_size() -> int:
    return _lib().qlin_config_table_size()


def abi_version() -> int:
    return _lib().qlin_abi_version()
