"""ctypes binding of libsgemm_strided.so (the C ABI in include/sgemm_strided.h).

Argument marshalling only: every step of the product runs in the HIP
library.  If the library has not been built, every call raises; there is no
other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsgemm_strided.so")

PATH_AUTO, PATH_MFMA, PATH_WAVE, PATH_GENERIC = 0, 1, 2, 3
PATH_NAMES = {PATH_AUTO: "auto", PATH_MFMA: "mfma", PATH_WAVE: "wave", PATH_GENERIC: "generic"}

STATUS = {
    0: "SGEMM_OK",
    -1: "SGEMM_ERR_INVALID_SIZE",
    -2: "SGEMM_ERR_INVALID_STRIDE",
    -3: "SGEMM_ERR_NULL_POINTER",
    -4: "SGEMM_ERR_C_ALIAS",
    -5: "SGEMM_ERR_UNSUPPORTED",
    -6: "SGEMM_ERR_HIP",
    -7: "SGEMM_ERR_INVALID_PATH",
    -8: "SGEMM_ERR_WORKSPACE",
}

# Every symbol include/sgemm_strided.h declares.
EXPORTS = ("sgemm_strided_batched", "sgemm_strided_batched_path", "sgemm_strided_batched_ex",
           "sgemm_strided_batched_ex_path", "sgemm_strided_batched2", "sgemm_strided_batched2_path",
           "sgemm_strided_batched_splitk", "sgemm_splitk_describe",
           "sgemm_sqnorms", "sgemm_pairwise_sqdist", "sgemm_pairwise_sqdist_noalloc",
           "sgemm_attention", "sgemm_attention_path", "sgemm_attention_splitkv", "sgemm_attention_splitkv_describe",
           "sgemm_attention_describe",
           "sgemm_plan_describe", "sgemm_plan_describe2", "sgemm_status_string", "sgemm_last_error")


class SgemmError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int),
        ("transposed", ctypes.c_int),
        ("tile_m", ctypes.c_int),
        ("tile_n", ctypes.c_int),
        ("tile_k", ctypes.c_int),
        ("waves", ctypes.c_int),
        ("vec_a", ctypes.c_int),
        ("vec_b", ctypes.c_int),
        ("a_kfast", ctypes.c_int),
        ("b_kfast", ctypes.c_int),
        ("launches", ctypes.c_int),
        ("fixed_offsets", ctypes.c_int),
        ("workgroups", ctypes.c_int64),
        ("kernel", ctypes.c_char * 64),
    ]

    def as_dict(self) -> dict:
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["kernel"] = self.kernel.decode()
        d["path_name"] = PATH_NAMES.get(self.path, str(self.path))
        return d


class SplitkInfo(ctypes.Structure):
    _fields_ = [
        ("splits", ctypes.c_int),
        ("launches", ctypes.c_int),
        ("kc", ctypes.c_int64),
        ("k_last", ctypes.c_int64),
        ("workspace_floats", ctypes.c_int64),
        ("parts", PlanInfo),
    ]

    def as_dict(self) -> dict:
        d = {name: getattr(self, name) for name, _ in self._fields_ if name != "parts"}
        d["parts"] = self.parts.as_dict()
        return d


_i64, _f32, _int, _vp = ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_void_p
_GEMM_ARGS = [_i64, _i64, _i64, _i64, _f32,
              _vp, _i64, _i64, _i64,
              _vp, _i64, _i64, _i64,
              _int,
              _vp, _i64, _i64, _i64]

_EX_ARGS = [_i64, _i64, _i64, _i64, _f32,
            _vp, _i64, _i64, _i64,
            _vp, _i64, _i64, _i64,
            _f32,
            _vp, _i64, _i64, _i64,
            _vp, _i64, _i64,
            _vp, _i64, _i64]

_B2_ARGS = [_i64, _i64, _i64, _i64, _i64, _f32,
            _vp, _i64, _i64, _i64, _i64, _i64,
            _vp, _i64, _i64, _i64, _i64, _i64,
            _int,
            _vp, _i64, _i64, _i64, _i64]

_ATTN_ARGS = [_i64, _i64, _i64, _i64, _i64, _f32, _int,
              _vp, _i64, _i64, _i64, _i64,
              _vp, _i64, _i64, _i64, _i64, _i64,
              _vp, _i64, _i64, _i64, _i64,
              _vp, _i64, _i64, _i64, _i64]

_lib = None


def load(path: str = LIB_PATH):
    """Load (once) and return the library; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library not built: {path} is missing. Build it with "
            "`python -m strided_fp32_gemm_amd.build` (or __graft_entry__.build()).")
    lib = ctypes.CDLL(path)
    lib.sgemm_strided_batched.restype = _int
    lib.sgemm_strided_batched.argtypes = _GEMM_ARGS + [_vp]
    lib.sgemm_strided_batched_path.restype = _int
    lib.sgemm_strided_batched_path.argtypes = _GEMM_ARGS + [_int, _vp]
    lib.sgemm_strided_batched_ex.restype = _int
    lib.sgemm_strided_batched_ex.argtypes = _EX_ARGS + [_vp]
    lib.sgemm_strided_batched_ex_path.restype = _int
    lib.sgemm_strided_batched_ex_path.argtypes = _EX_ARGS + [_int, _vp]
    lib.sgemm_strided_batched2.restype = _int
    lib.sgemm_strided_batched2.argtypes = _B2_ARGS + [_vp]
    lib.sgemm_strided_batched2_path.restype = _int
    lib.sgemm_strided_batched2_path.argtypes = _B2_ARGS + [_int, _vp]
    lib.sgemm_attention.restype = _int
    lib.sgemm_attention.argtypes = _ATTN_ARGS + [_vp]
    lib.sgemm_attention_path.restype = _int
    lib.sgemm_attention_path.argtypes = _ATTN_ARGS + [_int, _vp]
    lib.sgemm_attention_splitkv.restype = _int
    lib.sgemm_attention_splitkv.argtypes = _ATTN_ARGS + [_vp, _i64, _vp]
    lib.sgemm_attention_splitkv_describe.restype = _int
    lib.sgemm_attention_splitkv_describe.argtypes = _ATTN_ARGS + [_i64, _int, ctypes.POINTER(_i64),
                                                                  ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
    lib.sgemm_attention_describe.restype = _int
    lib.sgemm_attention_describe.argtypes = _ATTN_ARGS + [_int, ctypes.POINTER(PlanInfo)]
    lib.sgemm_sqnorms.restype = _int
    lib.sgemm_sqnorms.argtypes = [_i64, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp]
    lib.sgemm_pairwise_sqdist.restype = _int
    lib.sgemm_pairwise_sqdist.argtypes = [_i64, _i64, _i64, _i64,
                                          _vp, _i64, _i64, _i64,
                                          _vp, _i64, _i64, _i64,
                                          _vp, _i64, _i64, _i64,
                                          _vp, _i64, _vp]
    lib.sgemm_pairwise_sqdist_noalloc.restype = _int
    lib.sgemm_pairwise_sqdist_noalloc.argtypes = [_i64, _i64, _i64, _i64,
                                                  _vp, _i64, _i64, _i64,
                                                  _vp, _i64, _i64, _i64,
                                                  _vp, _i64, _i64, _i64,
                                                  _vp]
    lib.sgemm_plan_describe.restype = _int
    lib.sgemm_plan_describe.argtypes = _GEMM_ARGS + [_int, _int, ctypes.POINTER(PlanInfo)]
    lib.sgemm_strided_batched_splitk.restype = _int
    lib.sgemm_strided_batched_splitk.argtypes = _GEMM_ARGS + [_vp, _i64, _vp]
    lib.sgemm_splitk_describe.restype = _int
    lib.sgemm_splitk_describe.argtypes = _GEMM_ARGS + [_vp, _i64, _int, ctypes.POINTER(SplitkInfo)]
    lib.sgemm_plan_describe2.restype = _int
    lib.sgemm_plan_describe2.argtypes = _B2_ARGS + [_int, _int, ctypes.POINTER(PlanInfo)]
    lib.sgemm_status_string.restype = ctypes.c_char_p
    lib.sgemm_status_string.argtypes = [_int]
    lib.sgemm_last_error.restype = ctypes.c_char_p
    lib.sgemm_last_error.argtypes = []
    _lib = lib
    return lib


def _ptr(x) -> int:
    """Device address of a pointer-like argument: an int, None, or anything
    with data_ptr() (a torch tensor)."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    raise TypeError(f"expected a device pointer or tensor, got {type(x).__name__}")


def _stream(s) -> int:
    if s is None:
        return 0
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    raise TypeError(f"expected a stream handle, got {type(s).__name__}")


def _check(status: int):
    if status != 0:
        raise SgemmError(status, load().sgemm_last_error().decode())


def _gemm_list(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch, sB_row,
               sB_col, accumulate, C, sC_batch, sC_row, sC_col):
    return [int(batch), int(m), int(n), int(k), float(alpha),
            _ptr(A), int(sA_batch), int(sA_row), int(sA_col),
            _ptr(B), int(sB_batch), int(sB_row), int(sB_col),
            int(bool(accumulate)),
            _ptr(C), int(sC_batch), int(sC_row), int(sC_col)]


def sgemm_strided_batched(batch, m, n, k, alpha,
                          A, sA_batch, sA_row, sA_col,
                          B, sB_batch, sB_row, sB_col,
                          accumulate,
                          C, sC_batch, sC_row, sC_col,
                          stream=None) -> None:
    """C <- alpha*A*B (+C) through the C ABI; strides in elements."""
    args = _gemm_list(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch,
                      sB_row, sB_col, accumulate, C, sC_batch, sC_row, sC_col)
    _check(load().sgemm_strided_batched(*args, _stream(stream)))


def sgemm_strided_batched_path(batch, m, n, k, alpha,
                               A, sA_batch, sA_row, sA_col,
                               B, sB_batch, sB_row, sB_col,
                               accumulate,
                               C, sC_batch, sC_row, sC_col,
                               path, stream=None) -> None:
    """Same as sgemm_strided_batched with the kernel family forced."""
    args = _gemm_list(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch,
                      sB_row, sB_col, accumulate, C, sC_batch, sC_row, sC_col)
    _check(load().sgemm_strided_batched_path(*args, int(path), _stream(stream)))


def _ex_list(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch, sB_row, sB_col,
             beta, C, sC_batch, sC_row, sC_col, row_add, sR_batch, sR_row, col_add, sL_batch,
             sL_col):
    return [int(batch), int(m), int(n), int(k), float(alpha),
            _ptr(A), int(sA_batch), int(sA_row), int(sA_col),
            _ptr(B), int(sB_batch), int(sB_row), int(sB_col),
            float(beta),
            _ptr(C), int(sC_batch), int(sC_row), int(sC_col),
            _ptr(row_add), int(sR_batch), int(sR_row),
            _ptr(col_add), int(sL_batch), int(sL_col)]


def sgemm_strided_batched_ex(batch, m, n, k, alpha,
                             A, sA_batch, sA_row, sA_col,
                             B, sB_batch, sB_row, sB_col,
                             beta,
                             C, sC_batch, sC_row, sC_col,
                             row_add=None, sR_batch=0, sR_row=0,
                             col_add=None, sL_batch=0, sL_col=0,
                             stream=None) -> None:
    """C <- alpha*A*B + beta*C + row_add[b,i] + col_add[b,j] through the C
    ABI (beta 0 never reads C; None drops a vector term)."""
    args = _ex_list(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch, sB_row,
                    sB_col, beta, C, sC_batch, sC_row, sC_col, row_add, sR_batch, sR_row,
                    col_add, sL_batch, sL_col)
    _check(load().sgemm_strided_batched_ex(*args, _stream(stream)))


def sgemm_strided_batched_ex_path(batch, m, n, k, alpha,
                                  A, sA_batch, sA_row, sA_col,
                                  B, sB_batch, sB_row, sB_col,
                                  beta,
                                  C, sC_batch, sC_row, sC_col,
                                  row_add=None, sR_batch=0, sR_row=0,
                                  col_add=None, sL_batch=0, sL_col=0,
                                  path=PATH_AUTO, stream=None) -> None:
    """sgemm_strided_batched_ex with the kernel family forced."""
    args = _ex_list(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch, sB_row,
                    sB_col, beta, C, sC_batch, sC_row, sC_col, row_add, sR_batch, sR_row,
                    col_add, sL_batch, sL_col)
    _check(load().sgemm_strided_batched_ex_path(*args, int(path), _stream(stream)))


def _b2_list(nb_outer, nb_inner, m, n, k, alpha, A, sA_outer, sA_inner, gA, sA_row, sA_col,
             B, sB_outer, sB_inner, gB, sB_row, sB_col, accumulate,
             C, sC_outer, sC_inner, sC_row, sC_col):
    return [int(nb_outer), int(nb_inner), int(m), int(n), int(k), float(alpha),
            _ptr(A), int(sA_outer), int(sA_inner), int(gA), int(sA_row), int(sA_col),
            _ptr(B), int(sB_outer), int(sB_inner), int(gB), int(sB_row), int(sB_col),
            int(bool(accumulate)),
            _ptr(C), int(sC_outer), int(sC_inner), int(sC_row), int(sC_col)]


def sgemm_strided_batched2(nb_outer, nb_inner, m, n, k, alpha,
                           A, sA_outer, sA_inner, gA, sA_row, sA_col,
                           B, sB_outer, sB_inner, gB, sB_row, sB_col,
                           accumulate,
                           C, sC_outer, sC_inner, sC_row, sC_col,
                           stream=None) -> None:
    """C[o,i] <- alpha*A[o,i//gA]*B[o,i//gB] (+C[o,i]) over two batch levels
    through the C ABI; strides in elements."""
    args = _b2_list(nb_outer, nb_inner, m, n, k, alpha, A, sA_outer, sA_inner, gA, sA_row, sA_col,
                    B, sB_outer, sB_inner, gB, sB_row, sB_col, accumulate,
                    C, sC_outer, sC_inner, sC_row, sC_col)
    _check(load().sgemm_strided_batched2(*args, _stream(stream)))


def sgemm_strided_batched2_path(nb_outer, nb_inner, m, n, k, alpha,
                                A, sA_outer, sA_inner, gA, sA_row, sA_col,
                                B, sB_outer, sB_inner, gB, sB_row, sB_col,
                                accumulate,
                                C, sC_outer, sC_inner, sC_row, sC_col,
                                path=PATH_AUTO, stream=None) -> None:
    """sgemm_strided_batched2 with the kernel family forced."""
    args = _b2_list(nb_outer, nb_inner, m, n, k, alpha, A, sA_outer, sA_inner, gA, sA_row, sA_col,
                    B, sB_outer, sB_inner, gB, sB_row, sB_col, accumulate,
                    C, sC_outer, sC_inner, sC_row, sC_col)
    _check(load().sgemm_strided_batched2_path(*args, int(path), _stream(stream)))


def _attn_list(nb_outer, nb_inner, tq, tk, d, alpha, causal,
               Q, sQ_outer, sQ_inner, sQ_row, sQ_col,
               K, sK_outer, sK_inner, g, sK_row, sK_col,
               V, sV_outer, sV_inner, sV_row, sV_col,
               O, sO_outer, sO_inner, sO_row, sO_col):
    return [int(nb_outer), int(nb_inner), int(tq), int(tk), int(d), float(alpha), int(bool(causal)),
            _ptr(Q), int(sQ_outer), int(sQ_inner), int(sQ_row), int(sQ_col),
            _ptr(K), int(sK_outer), int(sK_inner), int(g), int(sK_row), int(sK_col),
            _ptr(V), int(sV_outer), int(sV_inner), int(sV_row), int(sV_col),
            _ptr(O), int(sO_outer), int(sO_inner), int(sO_row), int(sO_col)]


def sgemm_attention(nb_outer, nb_inner, tq, tk, d, alpha, causal,
                    Q, sQ_outer, sQ_inner, sQ_row, sQ_col,
                    K, sK_outer, sK_inner, g, sK_row, sK_col,
                    V, sV_outer, sV_inner, sV_row, sV_col,
                    O, sO_outer, sO_inner, sO_row, sO_col, stream=None) -> None:
    """O <- softmax(alpha Q K^T [causal]) V over two batch levels, fused,
    through the C ABI (K and V head i//g for query head i)."""
    args = _attn_list(nb_outer, nb_inner, tq, tk, d, alpha, causal, Q, sQ_outer, sQ_inner, sQ_row,
                      sQ_col, K, sK_outer, sK_inner, g, sK_row, sK_col, V, sV_outer, sV_inner, sV_row,
                      sV_col, O, sO_outer, sO_inner, sO_row, sO_col)
    _check(load().sgemm_attention(*args, _stream(stream)))


def sgemm_attention_path(nb_outer, nb_inner, tq, tk, d, alpha, causal,
                         Q, sQ_outer, sQ_inner, sQ_row, sQ_col,
                         K, sK_outer, sK_inner, g, sK_row, sK_col,
                         V, sV_outer, sV_inner, sV_row, sV_col,
                         O, sO_outer, sO_inner, sO_row, sO_col, path=PATH_AUTO, stream=None) -> None:
    """sgemm_attention with the kernel forced (PATH_AUTO, PATH_MFMA, PATH_GENERIC)."""
    args = _attn_list(nb_outer, nb_inner, tq, tk, d, alpha, causal, Q, sQ_outer, sQ_inner, sQ_row,
                      sQ_col, K, sK_outer, sK_inner, g, sK_row, sK_col, V, sV_outer, sV_inner, sV_row,
                      sV_col, O, sO_outer, sO_inner, sO_row, sO_col)
    _check(load().sgemm_attention_path(*args, int(path), _stream(stream)))


def sgemm_attention_splitkv(nb_outer, nb_inner, tq, tk, d, alpha, causal,
                            Q, sQ_outer, sQ_inner, sQ_row, sQ_col,
                            K, sK_outer, sK_inner, g, sK_row, sK_col,
                            V, sV_outer, sV_inner, sV_row, sV_col,
                            O, sO_outer, sO_inner, sO_row, sO_col,
                            workspace, workspace_floats, stream=None) -> None:
    """Fused attention with the keys split across the GPU through `workspace`
    (decode-shaped calls) through the C ABI."""
    args = _attn_list(nb_outer, nb_inner, tq, tk, d, alpha, causal, Q, sQ_outer, sQ_inner, sQ_row, sQ_col,
                      K, sK_outer, sK_inner, g, sK_row, sK_col, V, sV_outer, sV_inner, sV_row, sV_col,
                      O, sO_outer, sO_inner, sO_row, sO_col)
    _check(load().sgemm_attention_splitkv(*args, _ptr(workspace), int(workspace_floats), _stream(stream)))


def sgemm_attention_splitkv_describe(nb_outer, nb_inner, tq, tk, d, alpha, causal,
                                     Q, sQ_outer, sQ_inner, sQ_row, sQ_col,
                                     K, sK_outer, sK_inner, g, sK_row, sK_col,
                                     V, sV_outer, sV_inner, sV_row, sV_col,
                                     O, sO_outer, sO_inner, sO_row, sO_col,
                                     workspace_floats=-1, num_cus=256) -> dict:
    """The split sgemm_attention_splitkv would make: chunks, chunk_keys and
    workspace_floats (all 0: not split).  workspace_floats < 0 asks what
    the planned split needs."""
    args = _attn_list(nb_outer, nb_inner, tq, tk, d, alpha, causal, Q, sQ_outer, sQ_inner, sQ_row, sQ_col,
                      K, sK_outer, sK_inner, g, sK_row, sK_col, V, sV_outer, sV_inner, sV_row, sV_col,
                      O, sO_outer, sO_inner, sO_row, sO_col)
    ch, ck, fl = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(load().sgemm_attention_splitkv_describe(*args, int(workspace_floats), int(num_cus), ctypes.byref(ch),
                                                   ctypes.byref(ck), ctypes.byref(fl)))
    return {"chunks": ch.value, "chunk_keys": ck.value, "workspace_floats": fl.value}


def sgemm_attention_describe(nb_outer, nb_inner, tq, tk, d, alpha, causal,
                             Q, sQ_outer, sQ_inner, sQ_row, sQ_col,
                             K, sK_outer, sK_inner, g, sK_row, sK_col,
                             V, sV_outer, sV_inner, sV_row, sV_col,
                             O, sO_outer, sO_inner, sO_row, sO_col, path=PATH_AUTO) -> dict:
    """The plan of a sgemm_attention_path call (no device access)."""
    info = PlanInfo()
    args = _attn_list(nb_outer, nb_inner, tq, tk, d, alpha, causal, Q, sQ_outer, sQ_inner, sQ_row,
                      sQ_col, K, sK_outer, sK_inner, g, sK_row, sK_col, V, sV_outer, sV_inner, sV_row,
                      sV_col, O, sO_outer, sO_inner, sO_row, sO_col)
    _check(load().sgemm_attention_describe(*args, int(path), ctypes.byref(info)))
    return info.as_dict()


def sgemm_sqnorms(batch, count, length, X, sX_batch, sX_item, sX_elem, out, sO_batch, sO_item,
                  stream=None) -> None:
    """out[b,i] <- sum_p X[b,i,p]^2 through the C ABI."""
    _check(load().sgemm_sqnorms(int(batch), int(count), int(length), _ptr(X), int(sX_batch),
                                int(sX_item), int(sX_elem), _ptr(out), int(sO_batch),
                                int(sO_item), _stream(stream)))


def sgemm_pairwise_sqdist(batch, m, n, k,
                          X, sX_batch, sX_row, sX_col,
                          Y, sY_batch, sY_row, sY_col,
                          D, sD_batch, sD_row, sD_col,
                          workspace, workspace_floats, stream=None) -> None:
    """D[b,i,j] <- |X[b,i,:] - Y[b,j,:]|^2 through the C ABI; `workspace`
    holds batch*m + nY*n floats (nY = 1 when sY_batch == 0, else batch)."""
    _check(load().sgemm_pairwise_sqdist(int(batch), int(m), int(n), int(k),
                                        _ptr(X), int(sX_batch), int(sX_row), int(sX_col),
                                        _ptr(Y), int(sY_batch), int(sY_row), int(sY_col),
                                        _ptr(D), int(sD_batch), int(sD_row), int(sD_col),
                                        _ptr(workspace), int(workspace_floats), _stream(stream)))


# Norm floats the allocation-free distance entry point can hold
# (SGEMM_SCRATCH_FLOATS of the public header).
SCRATCH_FLOATS = 1 << 20


def sgemm_pairwise_sqdist_noalloc(batch, m, n, k,
                                  X, sX_batch, sX_row, sX_col,
                                  Y, sY_batch, sY_row, sY_col,
                                  D, sD_batch, sD_row, sD_col, stream=None) -> None:
    """sgemm_pairwise_sqdist with the norms in the library's fixed device
    scratch (no workspace; batch*m + nY*n <= SCRATCH_FLOATS)."""
    _check(load().sgemm_pairwise_sqdist_noalloc(int(batch), int(m), int(n), int(k),
                                                _ptr(X), int(sX_batch), int(sX_row), int(sX_col),
                                                _ptr(Y), int(sY_batch), int(sY_row), int(sY_col),
                                                _ptr(D), int(sD_batch), int(sD_row), int(sD_col),
                                                _stream(stream)))


def sgemm_plan_describe(batch, m, n, k, alpha,
                        A, sA_batch, sA_row, sA_col,
                        B, sB_batch, sB_row, sB_col,
                        accumulate,
                        C, sC_batch, sC_row, sC_col,
                        path=PATH_AUTO, num_cus=256) -> dict:
    """The plan the library would launch (no device access when num_cus > 0)."""
    info = PlanInfo()
    args = _gemm_list(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch,
                      sB_row, sB_col, accumulate, C, sC_batch, sC_row, sC_col)
    _check(load().sgemm_plan_describe(*args, int(path), int(num_cus), ctypes.byref(info)))
    return info.as_dict()


def sgemm_strided_batched_splitk(batch, m, n, k, alpha,
                                 A, sA_batch, sA_row, sA_col,
                                 B, sB_batch, sB_row, sB_col,
                                 accumulate,
                                 C, sC_batch, sC_row, sC_col,
                                 workspace, workspace_floats,
                                 stream=None) -> None:
    """C <- alpha*A*B (+C) with k split across workgroups, partials in
    `workspace` (device memory of workspace_floats floats) through the C ABI."""
    args = _gemm_list(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch,
                      sB_row, sB_col, accumulate, C, sC_batch, sC_row, sC_col)
    _check(load().sgemm_strided_batched_splitk(*args, _ptr(workspace), int(workspace_floats),
                                               _stream(stream)))


def sgemm_splitk_describe(batch, m, n, k, alpha,
                          A, sA_batch, sA_row, sA_col,
                          B, sB_batch, sB_row, sB_col,
                          accumulate,
                          C, sC_batch, sC_row, sC_col,
                          workspace=None, workspace_floats=-1, num_cus=256) -> dict:
    """What sgemm_strided_batched_splitk would launch; workspace_floats < 0
    asks for the workspace the best split needs (no device access when
    num_cus > 0)."""
    info = SplitkInfo()
    args = _gemm_list(batch, m, n, k, alpha, A, sA_batch, sA_row, sA_col, B, sB_batch,
                      sB_row, sB_col, accumulate, C, sC_batch, sC_row, sC_col)
    _check(load().sgemm_splitk_describe(*args, _ptr(workspace), int(workspace_floats), int(num_cus),
                                        ctypes.byref(info)))
    return info.as_dict()


def sgemm_plan_describe2(nb_outer, nb_inner, m, n, k, alpha,
                         A, sA_outer, sA_inner, gA, sA_row, sA_col,
                         B, sB_outer, sB_inner, gB, sB_row, sB_col,
                         accumulate,
                         C, sC_outer, sC_inner, sC_row, sC_col,
                         path=PATH_AUTO, num_cus=256) -> dict:
    """The plan of a sgemm_strided_batched2 call (no device access when
    num_cus > 0)."""
    info = PlanInfo()
    args = _b2_list(nb_outer, nb_inner, m, n, k, alpha, A, sA_outer, sA_inner, gA, sA_row, sA_col,
                    B, sB_outer, sB_inner, gB, sB_row, sB_col, accumulate,
                    C, sC_outer, sC_inner, sC_row, sC_col)
    _check(load().sgemm_plan_describe2(*args, int(path), int(num_cus), ctypes.byref(info)))
    return info.as_dict()


def sgemm_status_string(status: int) -> str:
    return load().sgemm_status_string(int(status)).decode()


def sgemm_last_error() -> str:
    return load().sgemm_last_error().decode()
