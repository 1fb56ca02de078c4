"""Python binding of libqgemv_q4 (gfx950 HIP kernels behind a C ABI).

The functions here have the names of the C entry points declared in
include/qgemv_q4.h.  They only marshal arguments: they check dtype, device,
contiguity and byte lengths of torch tensors (the C side receives raw
pointers that carry no size), allocate outputs when none are given, and pass
``torch.cuda.current_stream()`` as the stream.  Every step of the computation
runs in the library's kernels; if the library is missing, importing this
module raises.

torch is imported before the library is loaded so that the process keeps a
single HIP runtime (torch's ``libamdhip64``, which the library then binds to).
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the CDLL load, see module doc)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("QG_LIB_PATH", os.path.join(_HERE, "lib", "libqgemv_q4.so"))

QG_OK, QG_EINVAL, QG_ELAUNCH = 0, 1, 2
# bits of qg_set_kernel_mask (include/qgemv_q4.h)
QG_KERNEL_KSLICED, QG_KERNEL_XR, QG_KERNEL_MMA = 1, 2, 4
QG_KERNEL_ALL = QG_KERNEL_KSLICED | QG_KERNEL_XR | QG_KERNEL_MMA

# Entry points declared in include/qgemv_q4.h: name -> (restype, argtypes)
_P = ctypes.c_void_p
_I = ctypes.c_int64
SIGNATURES = {
    "qg_last_error": (ctypes.c_char_p, []),
    "qgemv_q4_0": (ctypes.c_int, [_P, _P, _P, _I, _I, _I, _P]),
    "qgemv_q4_k": (ctypes.c_int, [_P, _P, _P, _I, _I, _I, _P]),
    "qgemv_dual_q4_0": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _P]),
    "qmm_affine_t": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "qmm_affine_t_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "qkv_split_f32": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "qgemv_q4_k_multi": (ctypes.c_int, [_P, _P, _P, _P, _I, _P, _I, _I, _P]),
    "qmm_affine_t_packed": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "qmm_affine_t_qkv": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "qg_set_mfma_min_m": (ctypes.c_int, [_I]),
    "qg_get_mfma_min_m": (ctypes.c_int64, []),
    "qg_set_kernel_mask": (ctypes.c_int, [ctypes.c_uint32]),
    "qg_get_kernel_mask": (ctypes.c_uint32, []),
}


class QGError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libqgemv_q4 not built ({LIB_PATH} missing); run `python gemm_qgemv_q4_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def last_error() -> str:
    return (_lib.qg_last_error() or b"").decode()


def _check(status: int):
    if status != QG_OK:
        raise QGError(status, last_error())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(name, t, dtype, nbytes=None, numel=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} dtype {t.dtype} != {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if nbytes is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} too small: need {nbytes} bytes, have {t.numel() * t.element_size()}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} element_count {t.numel()} != {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _out(name, y, shape, like):
    if y is None:
        return torch.empty(shape, dtype=torch.float32, device=like.device)
    _dev(name, y, torch.float32, numel=int(torch.Size(shape).numel()))
    return y


def _mk(x, k):
    if x.dim() == 1:
        if x.numel() != k:
            raise ValueError(f"x has {x.numel()} elements, expected K={k}")
        return 1
    if x.shape[-1] != k:
        raise ValueError(f"x last dim {x.shape[-1]} != K={k}")
    return x.numel() // k


def qgemv_q4_0(w: torch.Tensor, x: torch.Tensor, n: int, k: int, y: torch.Tensor | None = None):
    """y[M, N] = x[M, K] * W^T, W in Q4_0 blocks (uint8, N*K/32*18 bytes)."""
    m = _mk(x, k)
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    pw = _dev("w", w, torch.uint8, nbytes=n * (k // 32) * 18)
    px = _dev("x", x, torch.float32, numel=m * k)
    y = _out("y", y, (m, n), x)
    _check(_lib.qgemv_q4_0(pw, px, ctypes.c_void_p(y.data_ptr()), m, n, k, _stream(x)))
    return y


def qgemv_q4_k(w: torch.Tensor, x: torch.Tensor, n: int, k: int, y: torch.Tensor | None = None):
    """y[M, N] = x[M, K] * W^T, W in Q4_K super-blocks (uint8, N*K/256*144 bytes)."""
    m = _mk(x, k)
    if k % 256:
        raise ValueError("K must be a multiple of 256")
    pw = _dev("w", w, torch.uint8, nbytes=n * (k // 256) * 144)
    px = _dev("x", x, torch.float32, numel=m * k)
    y = _out("y", y, (m, n), x)
    _check(_lib.qgemv_q4_k(pw, px, ctypes.c_void_p(y.data_ptr()), m, n, k, _stream(x)))
    return y


def qgemv_dual_q4_0(w_a: torch.Tensor, w_b: torch.Tensor, x: torch.Tensor, n: int, k: int,
                    y_a: torch.Tensor | None = None, y_b: torch.Tensor | None = None):
    """(x W_a^T, x W_b^T) in one pass; bitwise equal to two qgemv_q4_0 calls."""
    m = _mk(x, k)
    if k % 32:
        raise ValueError("K must be a multiple of 32")
    nb = n * (k // 32) * 18
    pa = _dev("w_a", w_a, torch.uint8, nbytes=nb)
    pb = _dev("w_b", w_b, torch.uint8, nbytes=nb)
    px = _dev("x", x, torch.float32, numel=m * k)
    y_a = _out("y_a", y_a, (m, n), x)
    y_b = _out("y_b", y_b, (m, n), x)
    _check(_lib.qgemv_dual_q4_0(pa, pb, px, ctypes.c_void_p(y_a.data_ptr()),
                                ctypes.c_void_p(y_b.data_ptr()), m, n, k, _stream(x)))
    return y_a, y_b


def qmm_affine_t(x: torch.Tensor, q: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
                 group_size: int, y: torch.Tensor | None = None):
    """y[M, N] = x[M, K] * (scales * q + biases)^T with u8 codes q[N, K]."""
    if q.dim() != 2:
        raise ValueError("q must be [N, K]")
    n, k = q.shape
    m = _mk(x, k)
    if group_size <= 0 or k % group_size:
        raise ValueError("K must be divisible by group_size")
    g = n * (k // group_size)
    px = _dev("x", x, torch.float32, numel=m * k)
    pq = _dev("q_int", q, torch.uint8, numel=n * k)
    ps = _dev("scales", scales, torch.float32, numel=g)
    pb = _dev("biases", biases, torch.float32, numel=g)
    y = _out("y", y, (m, n), x)
    _check(_lib.qmm_affine_t(px, pq, ps, pb, ctypes.c_void_p(y.data_ptr()), m, n, k, group_size,
                             _stream(x)))
    return y


def qmm_affine_t_noalloc(x: torch.Tensor, q: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
                         group_size: int, y: torch.Tensor):
    """qmm_affine_t without any allocation: the caller passes the output y[M, N],
    and the matrix-core path uses the library's static scratch (16 MiB per GPU)."""
    if q.dim() != 2:
        raise ValueError("q must be [N, K]")
    n, k = q.shape
    m = _mk(x, k)
    if group_size <= 0 or k % group_size:
        raise ValueError("K must be divisible by group_size")
    g = n * (k // group_size)
    px = _dev("x", x, torch.float32, numel=m * k)
    pq = _dev("q_int", q, torch.uint8, numel=n * k)
    ps = _dev("scales", scales, torch.float32, numel=g)
    pb = _dev("biases", biases, torch.float32, numel=g)
    py = _dev("y", y, torch.float32, numel=m * n)
    _check(_lib.qmm_affine_t_noalloc(px, pq, ps, pb, py, m, n, k, group_size, _stream(x)))
    return y


def qgemv_q4_k_multi(ws, x: torch.Tensor, ns, k: int, y: torch.Tensor | None = None, ys=None):
    """Parts of a fused Q4_K projection in one launch: part p (weights ws[p],
    ns[p] rows) writes columns [sum(ns[:p]), sum(ns[:p+1])) of one shared
    output y[M, sum(ns)], or, when ``ys`` is given, its own output ys[p][M, ns[p]]."""
    parts = len(ws)
    if parts != len(ns) or parts < 1:
        raise ValueError("ws and ns must be non-empty lists of the same length")
    m = _mk(x, k)
    if k % 256:
        raise ValueError("K must be a multiple of 256")
    px = _dev("x", x, torch.float32, numel=m * k)
    pw = [_dev(f"ws[{i}]", w, torch.uint8, nbytes=n * (k // 256) * 144) for i, (w, n) in enumerate(zip(ws, ns))]
    total = sum(ns)
    if ys is None:
        y = _out("y", y, (m, total), x)
        col = [sum(ns[:i]) for i in range(parts)]
        py = [ctypes.c_void_p(y.data_ptr() + 4 * c) for c in col]
        ldy = [total] * parts
        result = y
    else:
        if len(ys) != parts:
            raise ValueError("ys must have one output per part")
        ys = [_out(f"ys[{i}]", t, (m, n), x) for i, (t, n) in enumerate(zip(ys, ns))]
        py = [ctypes.c_void_p(t.data_ptr()) for t in ys]
        ldy = list(ns)
        result = ys
    arr_w = (ctypes.c_void_p * parts)(*pw)
    arr_y = (ctypes.c_void_p * parts)(*py)
    arr_n = (ctypes.c_int64 * parts)(*ns)
    arr_l = (ctypes.c_int64 * parts)(*ldy)
    _check(_lib.qgemv_q4_k_multi(arr_w, arr_y, arr_n, arr_l, parts, px, m, k, _stream(x)))
    return result


def qmm_affine_t_packed(x: torch.Tensor, w_packed: torch.Tensor, scales: torch.Tensor,
                        biases: torch.Tensor, group_size: int, y: torch.Tensor | None = None):
    """y[M, N] = x * (scales * q + biases)^T with the 4-bit codes packed eight per
    32-bit word: w_packed[N, K/8] (int32 or uint32; code of element 8*kp + j in
    bits 4j..4j+3 of word kp)."""
    if w_packed.dim() != 2:
        raise ValueError("w_packed must be [N, K/8]")
    if w_packed.dtype not in (torch.int32, torch.uint32):
        raise ValueError(f"w_packed dtype {w_packed.dtype} is not a 32-bit integer")
    n, k = w_packed.shape[0], w_packed.shape[1] * 8
    m = _mk(x, k)
    if group_size <= 0 or k % group_size:
        raise ValueError("K must be divisible by group_size")
    g = n * (k // group_size)
    px = _dev("x", x, torch.float32, numel=m * k)
    pw = _dev("w_packed", w_packed, w_packed.dtype, numel=n * (k // 8))
    ps = _dev("scales", scales, torch.float32, numel=g)
    pb = _dev("biases", biases, torch.float32, numel=g)
    y = _out("y", y, (m, n), x)
    _check(_lib.qmm_affine_t_packed(px, pw, ps, pb, ctypes.c_void_p(y.data_ptr()), m, n, k, group_size,
                                    _stream(x)))
    return y


def qmm_affine_t_qkv(x: torch.Tensor, q: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
                     group_size: int, q_sp: int, k_sp: int, v_sp: int,
                     q_out: torch.Tensor | None = None, k_out: torch.Tensor | None = None,
                     v_out: torch.Tensor | None = None):
    """The affine product of a fused [q_sp + k_sp + v_sp, K] weight written
    straight into contiguous q[M, q_sp], k[M, k_sp], v[M, v_sp]; bitwise equal
    to qmm_affine_t followed by qkv_split_f32."""
    if q.dim() != 2:
        raise ValueError("q must be [N, K]")
    n, k = q.shape
    if n != q_sp + k_sp + v_sp:
        raise ValueError(f"q has {n} rows, spans add up to {q_sp + k_sp + v_sp}")
    m = _mk(x, k)
    if group_size <= 0 or k % group_size:
        raise ValueError("K must be divisible by group_size")
    g = n * (k // group_size)
    px = _dev("x", x, torch.float32, numel=m * k)
    pq = _dev("q_int", q, torch.uint8, numel=n * k)
    ps = _dev("scales", scales, torch.float32, numel=g)
    pb = _dev("biases", biases, torch.float32, numel=g)
    q_out = _out("q_out", q_out, (m, q_sp), x)
    k_out = _out("k_out", k_out, (m, k_sp), x)
    v_out = _out("v_out", v_out, (m, v_sp), x)
    _check(_lib.qmm_affine_t_qkv(px, pq, ps, pb, ctypes.c_void_p(q_out.data_ptr()),
                                 ctypes.c_void_p(k_out.data_ptr()), ctypes.c_void_p(v_out.data_ptr()),
                                 m, k, group_size, q_sp, k_sp, v_sp, _stream(x)))
    return q_out, k_out, v_out


def qkv_split_f32(qkv: torch.Tensor, seq: int, q_sp: int, k_sp: int, v_sp: int,
                  q: torch.Tensor | None = None, k: torch.Tensor | None = None,
                  v: torch.Tensor | None = None):
    """Split qkv[seq, q_sp+k_sp+v_sp] into contiguous q, k, v."""
    ch = q_sp + k_sp + v_sp
    pqkv = _dev("qkv", qkv, torch.float32, nbytes=seq * ch * 4)
    q = _out("q", q, (seq, q_sp), qkv)
    k = _out("k", k, (seq, k_sp), qkv)
    v = _out("v", v, (seq, v_sp), qkv)
    _check(_lib.qkv_split_f32(pqkv, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                              ctypes.c_void_p(v.data_ptr()), seq, q_sp, k_sp, v_sp, _stream(qkv)))
    return q, k, v


def qg_set_mfma_min_m(m: int) -> None:
    _check(_lib.qg_set_mfma_min_m(m))


def qg_get_mfma_min_m() -> int:
    return int(_lib.qg_get_mfma_min_m())


def qg_set_kernel_mask(mask: int) -> None:
    _check(_lib.qg_set_kernel_mask(mask))


def qg_get_kernel_mask() -> int:
    return int(_lib.qg_get_kernel_mask())


class kernels:
    """Context manager that sets the kernel mask (and optionally the matrix-core
    threshold) for the calls inside it and restores both afterwards."""

    def __init__(self, mask: int | None = None, mfma_min_m: int | None = None):
        self.mask, self.min_m = mask, mfma_min_m

    def __enter__(self):
        self.old = (qg_get_kernel_mask(), qg_get_mfma_min_m())
        if self.mask is not None:
            qg_set_kernel_mask(self.mask)
        if self.min_m is not None:
            qg_set_mfma_min_m(self.min_m)
        return self

    def __exit__(self, *exc):
        qg_set_kernel_mask(self.old[0])
        qg_set_mfma_min_m(self.old[1])
        return False


raw = _lib  # the loaded C library, for callers that pass raw pointers
