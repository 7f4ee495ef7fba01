"""Thin Python binding of libfp8bs (C ABI in include/fp8bs.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory (tensors) and the current stream.
Importing this module loads ``libfp8bs.so`` from the package directory and
raises ``ImportError`` if it has not been built (there is no fallback).
"""

import contextlib
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8bs.so")

OK, ERR_NULL, ERR_SHAPE, ERR_LAYOUT, ERR_DTYPE, ERR_WORKSPACE, ERR_HIP = range(7)
OUT_F32, OUT_BF16 = 0, 1
A_E4M3, A_BF16 = 0, 1
OP_QUANT_ACT, OP_QUANT_W, OP_GEMM_E4M3, OP_GEMM_BF16, OP_GROUPED_GEMM = range(5)
NOALLOC_SCRATCH_BYTES = 8 * 1024 * 1024  # FP8BS_NOALLOC_SCRATCH_BYTES
DELAY_TILE, DELAY_TENSOR = 0, 1

EXPORTS = (
    "fp8_quant_act_1x128",
    "fp8_quant_act_1x128_delayed",
    "fp8_quant_act_128x1_t",
    "fp8_quant_w_128x128",
    "fp8_quant_w_128x128_t",
    "fp8_quant_linear",
    "fp8_block_gemm",
    "fp8_block_gemm_bf16_noalloc",
    "fp8_block_grouped_gemm",
    "fp8_block_gemm_e4m3_out",
    "fp8_block_grouped_gemm_e4m3_out",
    "fp8_block_gemm_rowscaled",
    "fp8_block_kgrouped_gemm_rowscaled",
    "fp8bs_workspace_bytes",
    "fp8bs_status_string",
    "fp8bs_last_hip_error",
)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t

_SIGNATURES = {
    "fp8_quant_act_1x128": ([_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p], _int),
    "fp8_quant_act_1x128_delayed": ([_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _int, _p, _i64,
                                     _i64, _i64, _p, _p], _int),
    "fp8_quant_w_128x128": ([_p, _i64, _i64, _i64, _p, _i64, _p, _p], _int),
    "fp8_quant_w_128x128_t": ([_p, _i64, _i64, _i64, _p, _i64, _p, _p, _i64, _p, _p], _int),
    "fp8_quant_act_128x1_t": ([_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p], _int),
    "fp8_quant_linear": ([_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p, _i64, _i64, _p, _i64,
                          _p, _p], _int),
    "fp8_block_gemm_rowscaled": ([_p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _int, _i64,
                                  _i64, _i64, _p], _int),
    "fp8_block_kgrouped_gemm_rowscaled": ([_p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _i64, _i64,
                                           _int, _p, _i64, _i64, _i64, _i64, _p], _int),
    "fp8_block_gemm": ([_int, _p, _i64, _p, _i64, _p, _i64, _p, _p, _i64, _int,
                        _i64, _i64, _i64, _p, _sz, _p], _int),
    "fp8_block_gemm_bf16_noalloc": ([_p, _i64, _p, _i64, _p, _i64, _p, _p, _i64, _int, _i64,
                                     _i64, _i64, _p], _int),
    "fp8_block_grouped_gemm": ([_p, _i64, _p, _i64, _p, _i64, _i64, _p, _p, _i64, _int,
                                _p, _i64, _i64, _i64, _i64, _p, _sz, _p], _int),
    "fp8_block_gemm_e4m3_out": ([_int, _p, _i64, _p, _i64, _p, _i64, _p, _p, _i64, _p, _i64,
                                 _i64, _i64, _i64, _p, _sz, _p], _int),
    "fp8_block_grouped_gemm_e4m3_out": ([_p, _i64, _p, _i64, _p, _i64, _i64, _p, _p, _i64, _p,
                                         _i64, _p, _i64, _i64, _i64, _i64, _p, _sz, _p], _int),
    "fp8bs_workspace_bytes": ([_int, _i64, _i64, _i64, _i64], _sz),
    "fp8bs_status_string": ([_int], ctypes.c_char_p),
    "fp8bs_last_hip_error": ([], _int),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m fp8_block_scaled_05_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


class Fp8bsError(RuntimeError):
    def __init__(self, status, where):
        msg = lib.fp8bs_status_string(status).decode()
        if status == ERR_HIP:
            msg += f" (hipError_t {lib.fp8bs_last_hip_error()})"
        super().__init__(f"{where}: status {status}: {msg}")
        self.status = status


def _check(status, where):
    if status != OK:
        raise Fp8bsError(status, where)


# The current stream's raw handle: torch's private accessor returns it
# without building a Stream object (about 2 us less per call on MI355X hosts).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_NO_SWITCH = contextlib.nullcontext()


def _stream(t):
    if _raw_stream is not None:
        return _raw_stream(t.device.index)
    return torch.cuda.current_stream(t.device).cuda_stream


def _on(device):
    """Make ``device`` current for a call (the library's HIP calls act on the
    current device); no switch when it already is."""
    if device.index == torch.cuda.current_device():
        return _NO_SWITCH
    return torch.cuda.device(device)


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _need_device(*ts):
    devices = set()
    for t in ts:
        if t is None:
            continue
        d = t.device
        if d.type != "cuda":
            raise ValueError("libfp8bs works on GPU tensors only")
        devices.add(d)
    if len(devices) > 1:
        raise ValueError("all tensors of a call must be on one GPU, got "
                         f"{sorted(map(str, devices))}")


def _mat(t, name, rows, cols, dtype, ld=None):
    """Check that the caller's 2-D row-major tensor ``t`` (if given) holds
    ``rows`` x ``cols`` elements of ``dtype``: the library receives only its
    pointer and row stride, so a smaller tensor would be read or written
    past its end on the device.  ``ld``: the row stride the layout fixes."""
    if t is None:
        return
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    shape = t.shape
    if len(shape) != 2 or shape[0] < rows or shape[1] < cols:
        raise ValueError(f"{name} must be a 2-D tensor of at least [{rows}][{cols}], "
                         f"got {list(shape)}")
    if shape[0] == 0 or shape[1] == 0:
        return  # nothing is read or written; an empty tensor's strides are arbitrary
    row, col = t.stride()
    if shape[1] > 1 and col != 1:
        raise ValueError(f"{name} must have unit column stride")
    if rows > 1 and row < cols:
        raise ValueError(f"{name} rows overlap (row stride {row} < {cols})")
    if ld is not None and rows > 1 and row != ld:
        raise ValueError(f"{name} must have row stride {ld}, got {row}")


def _rowmajor(t, name):
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


def _ld(t):
    # leading dimension of a row-major 2-D tensor (its row stride)
    return t.stride(0) if t.dim() == 2 else t.shape[-1]


def _k_of(K, name):
    if K <= 0 or K % 128 != 0:
        raise ValueError(f"{name}: K = {K} must be a positive multiple of 128")
    return K // 128


def _offsets(group_offsets, G):
    if group_offsets.dtype != torch.int32:
        raise ValueError("group_offsets must be int32")
    if group_offsets.dim() != 1 or group_offsets.numel() != G + 1:
        raise ValueError(f"group_offsets must be a vector of G + 1 = {G + 1} entries")


def workspace_bytes(op, M, N, K, G=0):
    return int(lib.fp8bs_workspace_bytes(op, M, N, K, G))


def fp8_quant_act_1x128(x, q=None, s=None, lds=None):
    """bf16 [M][K] -> (E4M3 codes uint8 [M][K], scales fp32 [K/128][lds]).

    ``s[kb, m]`` is the scale of row m's tile kb (``lds >= M``, default M).
    """
    _mat(x, "x", 0, 0, torch.bfloat16)
    M, K = x.shape
    KB = _k_of(K, "fp8_quant_act_1x128")
    _mat(q, "q", M, K, torch.uint8)
    _mat(s, "s", KB, M, torch.float32)
    _need_device(x, q, s)
    ldx = _rowmajor(x, "x") if M else K
    if q is None:
        q = torch.empty(M, K, dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty(KB, lds or M, dtype=torch.float32, device=x.device)
    with _on(x.device):
        _check(lib.fp8_quant_act_1x128(_ptr(x), M, K, ldx, _ptr(q), _ld(q), _ptr(s), s.stride(0),
                                       _stream(x)), "fp8_quant_act_1x128")
    return q, s


def fp8_quant_act_1x128_delayed(x, hist, step, mode="tile", q=None, s=None, stats=None):
    """Delayed (history-based) scaling of bf16 [M][K] per 1x128 tile.

    ``hist``: float32 history ring on the device, updated in place;
    ``mode="tile"``: [H][K/128][ldh] (ldh >= M), ``mode="tensor"``: [H + 2].
    ``step``: t = 0, 1, 2, ... in order.  ``stats``: optional int32/uint32 [2]
    device tensor accumulating (clipped, flushed) counts.
    Returns ``(q, s)`` as ``fp8_quant_act_1x128``.
    """
    _mat(x, "x", 0, 0, torch.bfloat16)
    if hist.dtype != torch.float32:
        raise ValueError("hist must be float32")
    M, K = x.shape
    KB = _k_of(K, "fp8_quant_act_1x128_delayed")
    _mat(q, "q", M, K, torch.uint8)
    _mat(s, "s", KB, M, torch.float32)
    if mode == "tile":
        if hist.dim() != 3 or hist.shape[1] != KB or hist.shape[2] < M or not hist.is_contiguous():
            raise ValueError(f"per-tile history must be a contiguous [H][{KB}][ldh >= {M}]")
        H, ldh, m = hist.shape[0], hist.shape[2], DELAY_TILE
    elif mode == "tensor":
        if hist.dim() != 1 or hist.shape[0] < 3 or not hist.is_contiguous():
            raise ValueError("per-tensor history must be a contiguous [H + 2], H >= 1")
        H, ldh, m = hist.shape[0] - 2, 0, DELAY_TENSOR
    else:
        raise ValueError("mode must be 'tile' or 'tensor'")
    if stats is not None and (stats.dtype not in (torch.int32, torch.uint32) or
                              stats.numel() < 2 or not stats.is_contiguous()):
        raise ValueError("stats must be a contiguous int32/uint32 tensor of 2 counters")
    _need_device(x, hist, q, s, stats)
    ldx = _rowmajor(x, "x") if M else K
    if q is None:
        q = torch.empty(M, K, dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty(KB, M, dtype=torch.float32, device=x.device)
    with _on(x.device):
        _check(lib.fp8_quant_act_1x128_delayed(_ptr(x), M, K, ldx, _ptr(q), _ld(q), _ptr(s),
                                               s.stride(0), m, _ptr(hist), ldh, H, step,
                                               _ptr(stats), _stream(x)),
               "fp8_quant_act_1x128_delayed")
    return q, s


def fp8_quant_w_128x128(w, q=None, s=None):
    """bf16 [N][K] -> (E4M3 codes uint8 [N][K], scales fp32 [ceil(N/128)][K/128])."""
    _mat(w, "w", 0, 0, torch.bfloat16)
    N, K = w.shape
    KB = _k_of(K, "fp8_quant_w_128x128")
    _mat(q, "q", N, K, torch.uint8)
    _mat(s, "s", (N + 127) // 128, KB, torch.float32, ld=KB)
    _need_device(w, q, s)
    ldw = _rowmajor(w, "w") if N else K
    if q is None:
        q = torch.empty(N, K, dtype=torch.uint8, device=w.device)
    if s is None:
        s = torch.empty((N + 127) // 128, KB, dtype=torch.float32, device=w.device)
    with _on(w.device):
        _check(lib.fp8_quant_w_128x128(_ptr(w), N, K, ldw, _ptr(q), _ld(q), _ptr(s), _stream(w)),
               "fp8_quant_w_128x128")
    return q, s


def fp8_quant_linear(x, w, q=None, s=None, qw=None, sw=None):
    """Both operands of y = x . W^T in one launch: returns ``(q, s, qw, sw)``,
    exactly ``fp8_quant_act_1x128(x)`` and ``fp8_quant_w_128x128(w)``."""
    _mat(x, "x", 0, 0, torch.bfloat16)
    _mat(w, "w", 0, 0, torch.bfloat16)
    M, K = x.shape
    N, Kw = w.shape
    if Kw != K:
        raise ValueError(f"x has K={K} columns but w has {Kw}")
    KB = _k_of(K, "fp8_quant_linear")
    _mat(q, "q", M, K, torch.uint8)
    _mat(s, "s", KB, M, torch.float32)
    _mat(qw, "qw", N, K, torch.uint8)
    _mat(sw, "sw", (N + 127) // 128, KB, torch.float32, ld=KB)
    _need_device(x, w, q, s, qw, sw)
    ldx = _rowmajor(x, "x") if M else K
    ldw = _rowmajor(w, "w") if N else K
    if q is None:
        q = torch.empty(M, K, dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty(KB, M, dtype=torch.float32, device=x.device)
    if qw is None:
        qw = torch.empty(N, K, dtype=torch.uint8, device=w.device)
    if sw is None:
        sw = torch.empty((N + 127) // 128, KB, dtype=torch.float32, device=w.device)
    with _on(x.device):
        _check(lib.fp8_quant_linear(_ptr(x), M, K, ldx, _ptr(q), _ld(q), _ptr(s), s.stride(0),
                                    _ptr(w), N, ldw, _ptr(qw), _ld(qw), _ptr(sw), _stream(x)),
               "fp8_quant_linear")
    return q, s, qw, sw


def fp8_quant_w_128x128_t(w, q=None, s=None, qt=None, st=None):
    """bf16 [N][K] -> (q [N][K], s [N/128][K/128], qt [K][N], st [K/128][N/128]):
    the weight's codes and scales for the forward GEMM and, transposed, for
    the data-gradient GEMM dX = dY . W (``fp8_block_gemm(qdy, sdy, qt, st)``)."""
    _mat(w, "w", 0, 0, torch.bfloat16)
    N, K = w.shape
    KB = _k_of(K, "fp8_quant_w_128x128_t")
    if N % 128 != 0:
        raise ValueError(f"fp8_quant_w_128x128_t: N = {N} must be a multiple of 128")
    NB = N // 128
    _mat(q, "q", N, K, torch.uint8)
    _mat(s, "s", NB, KB, torch.float32, ld=KB)
    _mat(qt, "qt", K, N, torch.uint8)
    _mat(st, "st", KB, NB, torch.float32, ld=NB)
    _need_device(w, q, s, qt, st)
    ldw = _rowmajor(w, "w") if N else K
    dev = w.device
    q = torch.empty(N, K, dtype=torch.uint8, device=dev) if q is None else q
    s = torch.empty(NB, KB, dtype=torch.float32, device=dev) if s is None else s
    qt = torch.empty(K, N, dtype=torch.uint8, device=dev) if qt is None else qt
    st = torch.empty(KB, NB, dtype=torch.float32, device=dev) if st is None else st
    with _on(w.device):
        _check(lib.fp8_quant_w_128x128_t(_ptr(w), N, K, ldw, _ptr(q), _ld(q), _ptr(s), _ptr(qt),
                                         _ld(qt), _ptr(st), _stream(w)), "fp8_quant_w_128x128_t")
    return q, s, qt, st


def fp8_quant_act_128x1_t(x, qt=None, st=None):
    """bf16 [M][N] -> (qt uint8 [N][M], st fp32 [M/128][N]): groups of 128
    consecutive rows per column, codes transposed (the operands of the
    weight-gradient GEMM)."""
    _mat(x, "x", 0, 0, torch.bfloat16)
    M, N = x.shape
    if M % 128 != 0 or N % 128 != 0:
        raise ValueError(f"fp8_quant_act_128x1_t: M = {M} and N = {N} must be multiples of 128")
    _mat(qt, "qt", N, M, torch.uint8)
    _mat(st, "st", M // 128, N, torch.float32)
    _need_device(x, qt, st)
    ldx = _rowmajor(x, "x") if M else N
    if qt is None:
        qt = torch.empty(N, M, dtype=torch.uint8, device=x.device)
    if st is None:
        st = torch.empty(M // 128, N, dtype=torch.float32, device=x.device)
    with _on(x.device):
        _check(lib.fp8_quant_act_128x1_t(_ptr(x), M, N, ldx, _ptr(qt), _ld(qt), _ptr(st),
                                         st.stride(0), _stream(x)), "fp8_quant_act_128x1_t")
    return qt, st


def fp8_block_gemm_rowscaled(a, sa, b, sb, out=None, out_dtype=torch.float32):
    """C[M][N] = A . B^T with one scale per row and 128-K group on both
    operands (sa [K/128][ldsa], sb [K/128][ldsb]); the weight-gradient GEMM
    dW = dY^T . X with (a, sa), (b, sb) from ``fp8_quant_act_128x1_t``."""
    _mat(a, "a", 0, 0, torch.uint8)
    M, K = a.shape
    KB = _k_of(K, "fp8_block_gemm_rowscaled")
    N = b.shape[0]
    _mat(b, "b", N, K, torch.uint8)
    _mat(sa, "sa", KB, M, torch.float32)
    _mat(sb, "sb", KB, N, torch.float32)
    if out is not None:
        _mat(out, "out", M, N, out.dtype)
    _need_device(a, sa, b, sb, out)
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=a.device)
    with _on(a.device):
        _check(lib.fp8_block_gemm_rowscaled(_ptr(a), _ld(a), _ptr(sa), sa.stride(0), _ptr(b),
                                            _ld(b), _ptr(sb), sb.stride(0), _ptr(out), _ld(out),
                                            _out_kind(out.dtype), M, N, K, _stream(a)),
               "fp8_block_gemm_rowscaled")
    return out


def fp8_block_kgrouped_gemm_rowscaled(a, sa, b, sb, group_offsets, out=None,
                                      out_dtype=torch.float32):
    """MoE weight gradients in one launch: out[g] = A[:, t0:t1] . B[:, t0:t1]^T
    over expert g's token columns [t0, t1) = group_offsets[g:g+2]
    (multiples of 128).  ``a`` [M][T], ``b`` [N][T] from
    ``fp8_quant_act_128x1_t``; returns ``out`` [G][M][N]."""
    _mat(a, "a", 0, 0, torch.uint8)
    M, T = a.shape
    if T % 128 != 0:
        raise ValueError(f"fp8_block_kgrouped_gemm_rowscaled: T = {T} must be a multiple of 128")
    N = b.shape[0]
    G = group_offsets.shape[0] - 1
    _offsets(group_offsets, G)
    _mat(b, "b", N, T, torch.uint8)
    _mat(sa, "sa", T // 128, M, torch.float32)
    _mat(sb, "sb", T // 128, N, torch.float32)
    if out is not None:
        if (out.dim() != 3 or out.shape[0] < G or out.shape[1] < M or out.shape[2] < N or
                out.stride(2) != 1):
            raise ValueError(f"out must be [G >= {G}][M >= {M}][N >= {N}] with unit column "
                             "stride")
    _need_device(a, sa, b, sb, group_offsets, out)
    if out is None:
        out = torch.empty(G, M, N, dtype=out_dtype, device=a.device)
    with _on(a.device):
        _check(lib.fp8_block_kgrouped_gemm_rowscaled(
            _ptr(a), _ld(a), _ptr(sa), sa.stride(0), _ptr(b), _ld(b), _ptr(sb), sb.stride(0),
            _ptr(out), out.stride(1), out.stride(0), _out_kind(out.dtype), _ptr(group_offsets),
            G, M, N, T, _stream(a)), "fp8_block_kgrouped_gemm_rowscaled")
    return out


def _out_kind(dtype):
    if dtype == torch.bfloat16:
        return OUT_BF16
    if dtype == torch.float32:
        return OUT_F32
    raise ValueError("output must be float32 or bfloat16")


def _a_kind(a):
    if a.dtype == torch.uint8:
        return A_E4M3
    if a.dtype == torch.bfloat16:
        return A_BF16
    raise ValueError("a must be uint8 (E4M3 codes) or bfloat16")


def _dense_operands(where, a, sa, b, sb):
    """Sizes of a dense GEMM call after checking its operand tensors."""
    a_kind = _a_kind(a)
    _mat(a, "a", 0, 0, a.dtype)
    M, K = a.shape
    KB = _k_of(K, where)
    N = b.shape[0] if b.dim() == 2 else -1
    _mat(b, "b", N, K, torch.uint8)
    if a_kind == A_E4M3 and sa is None:
        raise ValueError("E4M3 codes need their scales sa")
    _mat(sa, "sa", KB, M, torch.float32)
    _mat(sb, "sb", (N + 127) // 128, KB, torch.float32, ld=KB)
    return a_kind, M, N, K


def _workspace(a_kind, M, N, K, workspace, device):
    ws_need = workspace_bytes(OP_GEMM_BF16, M, N, K) if a_kind == A_BF16 else 0
    if ws_need and workspace is None:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return workspace, ws_bytes


def fp8_block_gemm(a, sa, b, sb, out=None, out_dtype=torch.bfloat16, workspace=None):
    """C[M][N] = A . B^T with per-tile/per-block scales and FP32 promotion.

    ``a`` uint8 E4M3 codes with input scales ``sa`` [K/128][ldsa], or
    bfloat16 (quantized inside the call; ``sa`` is then an optional output of
    the scales).  ``b`` uint8 [N][K], ``sb`` fp32 [ceil(N/128)][K/128].
    """
    a_kind, M, N, K = _dense_operands("fp8_block_gemm", a, sa, b, sb)
    if out is not None:
        _mat(out, "out", M, N, out.dtype)
    _need_device(a, sa, b, sb, out, workspace)
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=a.device)
    workspace, ws_bytes = _workspace(a_kind, M, N, K, workspace, a.device)
    ldsa = sa.stride(0) if sa is not None else 0
    with _on(a.device):
        _check(lib.fp8_block_gemm(a_kind, _ptr(a), _ld(a), _ptr(sa), ldsa, _ptr(b), _ld(b),
                                  _ptr(sb), _ptr(out), _ld(out), _out_kind(out.dtype), M, N, K,
                                  _ptr(workspace), ws_bytes, _stream(a)), "fp8_block_gemm")
    return out


def fp8_block_gemm_bf16_noalloc(a, sa, b, sb, out):
    """``fp8_block_gemm`` with a bf16 ``a`` quantized into the library's own
    fixed device buffer: the library allocates nothing, and neither does this
    wrapper (``out`` [M][N] fp32 or bf16 is the caller's; ``sa``
    [K/128][ldsa], optional, receives the scales).  Calls that overlap on one
    GPU share that buffer and race."""
    if a.dtype != torch.bfloat16:
        raise ValueError("a must be bfloat16")
    if out is None:
        raise ValueError("out must be given (this entry point allocates nothing)")
    _, M, N, K = _dense_operands("fp8_block_gemm_bf16_noalloc", a, sa, b, sb)
    _mat(out, "out", M, N, out.dtype)
    _need_device(a, sa, b, sb, out)
    ldsa = sa.stride(0) if sa is not None else 0
    with _on(a.device):
        _check(lib.fp8_block_gemm_bf16_noalloc(_ptr(a), _ld(a), _ptr(sa), ldsa, _ptr(b), _ld(b),
                                               _ptr(sb), _ptr(out), _ld(out),
                                               _out_kind(out.dtype), M, N, K, _stream(a)),
               "fp8_block_gemm_bf16_noalloc")
    return out


def _grouped_operands(where, a, sa, b, sb, group_offsets):
    """Sizes of a grouped GEMM call after checking its operand tensors."""
    _mat(a, "a", 0, 0, torch.uint8)
    M_total, K = a.shape
    KB = _k_of(K, where)
    if b.dtype != torch.uint8 or b.dim() != 3 or b.shape[2] < K or b.stride(2) != 1:
        raise ValueError(f"b must be uint8 [G][N][>= {K}] with unit column stride")
    G, N, _ = b.shape
    _offsets(group_offsets, G)
    _mat(sa, "sa", KB, M_total, torch.float32)
    NB = (N + 127) // 128
    if (sb.dtype != torch.float32 or sb.dim() != 3 or list(sb.shape) != [G, NB, KB] or
            not sb.is_contiguous()):
        raise ValueError(f"sb must be a contiguous float32 [{G}][{NB}][{KB}]")
    return M_total, G, N, K


def fp8_block_grouped_gemm(a, sa, b, sb, group_offsets, out=None, out_dtype=torch.bfloat16):
    """Grouped (MoE) block GEMM.

    ``a`` uint8 [M_total][K] rows sorted by expert, ``sa`` fp32 [K/128][ldsa];
    ``b`` uint8 [G][N][K]; ``sb`` fp32 [G][ceil(N/128)][K/128];
    ``group_offsets`` int32 [G+1] on the device.
    """
    M_total, G, N, K = _grouped_operands("fp8_block_grouped_gemm", a, sa, b, sb, group_offsets)
    if out is not None:
        _mat(out, "out", M_total, N, out.dtype)
    _need_device(a, sa, b, sb, group_offsets, out)
    if out is None:
        out = torch.empty(M_total, N, dtype=out_dtype, device=a.device)
    with _on(a.device):
        _check(lib.fp8_block_grouped_gemm(_ptr(a), _ld(a), _ptr(sa), sa.stride(0), _ptr(b),
                                          b.stride(1), b.stride(0), _ptr(sb), _ptr(out), _ld(out),
                                          _out_kind(out.dtype), _ptr(group_offsets), G, M_total, N,
                                          K, None, 0, _stream(a)), "fp8_block_grouped_gemm")
    return out


def _e4m3_check(M, N, qc, sc):
    if N % 128 != 0:
        raise ValueError(f"E4M3 output needs N = {N} to be a multiple of 128")
    _mat(qc, "qc", M, N, torch.uint8)
    _mat(sc, "sc", N // 128, M, torch.float32)


def _e4m3_outputs(M, N, qc, sc, device):
    if qc is None:
        qc = torch.empty(M, N, dtype=torch.uint8, device=device)
    if sc is None:
        sc = torch.empty(N // 128, M, dtype=torch.float32, device=device)
    return qc, sc


def fp8_block_gemm_e4m3_out(a, sa, b, sb, qc=None, sc=None, workspace=None):
    """As ``fp8_block_gemm``, with C quantized per 1x128 tile along N.

    Returns ``(qc, sc)``: E4M3 codes uint8 [M][N] and scales fp32
    [N/128][ldsc] (``sc[nb, m]``), the layout ``fp8_block_gemm`` takes as
    its activation input.
    """
    a_kind, M, N, K = _dense_operands("fp8_block_gemm_e4m3_out", a, sa, b, sb)
    _e4m3_check(M, N, qc, sc)
    _need_device(a, sa, b, sb, qc, sc, workspace)
    qc, sc = _e4m3_outputs(M, N, qc, sc, a.device)
    workspace, ws_bytes = _workspace(a_kind, M, N, K, workspace, a.device)
    ldsa = sa.stride(0) if sa is not None else 0
    with _on(a.device):
        _check(lib.fp8_block_gemm_e4m3_out(a_kind, _ptr(a), _ld(a), _ptr(sa), ldsa, _ptr(b),
                                           _ld(b), _ptr(sb), _ptr(qc), _ld(qc), _ptr(sc),
                                           sc.stride(0), M, N, K, _ptr(workspace), ws_bytes,
                                           _stream(a)),
               "fp8_block_gemm_e4m3_out")
    return qc, sc


def fp8_block_grouped_gemm_e4m3_out(a, sa, b, sb, group_offsets, qc=None, sc=None):
    """As ``fp8_block_grouped_gemm``, with C quantized per 1x128 tile along N.

    Returns ``(qc, sc)`` as ``fp8_block_gemm_e4m3_out``.
    """
    M_total, G, N, K = _grouped_operands("fp8_block_grouped_gemm_e4m3_out", a, sa, b, sb,
                                         group_offsets)
    _e4m3_check(M_total, N, qc, sc)
    _need_device(a, sa, b, sb, group_offsets, qc, sc)
    qc, sc = _e4m3_outputs(M_total, N, qc, sc, a.device)
    with _on(a.device):
        _check(lib.fp8_block_grouped_gemm_e4m3_out(_ptr(a), _ld(a), _ptr(sa), sa.stride(0), _ptr(b),
                                                   b.stride(1), b.stride(0), _ptr(sb), _ptr(qc),
                                                   _ld(qc), _ptr(sc), sc.stride(0),
                                                   _ptr(group_offsets), G, M_total, N, K, None, 0,
                                                   _stream(a)),
               "fp8_block_grouped_gemm_e4m3_out")
    return qc, sc
