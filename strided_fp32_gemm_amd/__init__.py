"""Strided, batched fp32 matrix product for AMD Instinct MI355X (gfx950).

    C <- alpha * A @ B   (+ C when accumulate)

over a batch, with every operand given by a pointer and (batch, row, col)
element strides; a transposed operand is the same memory with its row and
column strides exchanged (StaleyNET "GPU Implementation", section "The
matrix product").  Around it: a general epilogue (beta, per-row and
per-column terms), squared norms and distances, two batch levels with
grouped inputs, and fused attention softmax(alpha Q K^T) V.  The computation
runs in hand-written HIP kernels behind a C ABI (include/sgemm_strided.h);
this package only marshals arguments.  PyTorch is used for device memory and
streams.
"""
from . import _binding  # noqa: F401
from ._binding import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    PATH_AUTO,
    PATH_GENERIC,
    PATH_MFMA,
    PATH_NAMES,
    PATH_WAVE,
    SCRATCH_FLOATS,
    SgemmError,
    load,
    sgemm_attention,
    sgemm_attention_describe,
    sgemm_attention_path,
    sgemm_attention_splitkv,
    sgemm_attention_splitkv_describe,
    sgemm_last_error,
    sgemm_pairwise_sqdist,
    sgemm_pairwise_sqdist_noalloc,
    sgemm_plan_describe,
    sgemm_plan_describe2,
    sgemm_splitk_describe,
    sgemm_sqnorms,
    sgemm_status_string,
    sgemm_strided_batched,
    sgemm_strided_batched2,
    sgemm_strided_batched2_path,
    sgemm_strided_batched_ex,
    sgemm_strided_batched_ex_path,
    sgemm_strided_batched_splitk,
    sgemm_strided_batched_path,
)


def _strides3(t, name):
    if t.dim() == 2:
        return 1, (0, t.stride(0), t.stride(1)), tuple(t.shape)
    if t.dim() == 3:
        return t.shape[0], tuple(t.stride()), tuple(t.shape[1:])
    raise ValueError(f"{name} must be 2-D or 3-D, got {t.dim()}-D")


def sgemm(A, B, C, alpha: float = 1.0, accumulate: bool = False, path: int = PATH_AUTO,
          stream=None, splitk: bool = False):
    """C <- alpha*A@B (+C) for torch float32 views on one GPU.

    A is [batch,] m x k, B is [batch,] k x n, C is [batch,] m x n; any of them
    may be a strided or transposed view (``W.t()`` passes W with exchanged
    strides, no copy).  A 2-D operand next to 3-D ones is broadcast over the
    batch (batch stride 0).  Runs on ``stream`` (default: torch's current
    stream) and returns C.

    splitk=True goes through sgemm_strided_batched_splitk (k split across
    workgroups, for small outputs over a deep k): the workspace the library's
    plan asks for is allocated here with torch (the library allocates
    nothing); ``path`` does not apply.
    """
    import torch

    for t, nm in ((A, "A"), (B, "B"), (C, "C")):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{nm} must be a torch.Tensor")
        if t.dtype != torch.float32:
            raise TypeError(f"{nm} must be float32, got {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError(f"{nm} must be on the GPU")
    if not (A.device == B.device == C.device):
        raise ValueError("A, B and C must be on the same device")
    ba, sa, (m, k) = _strides3(A, "A")
    bb, sb, (k2, n) = _strides3(B, "B")
    bc, sc, (m2, n2) = _strides3(C, "C")
    if k != k2 or m != m2 or n != n2:
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    batch = max(ba, bb, bc)
    for b_, nm in ((ba, "A"), (bb, "B")):
        if b_ not in (1, batch):
            raise ValueError(f"{nm} batch {b_} does not match {batch}")
    if bc != batch:
        raise ValueError(f"C batch {bc} does not match {batch}")
    if ba == 1 and batch > 1:
        sa = (0, sa[1], sa[2])
    if bb == 1 and batch > 1:
        sb = (0, sb[1], sb[2])
    if stream is None:
        stream = torch.cuda.current_stream(C.device)
    with torch.cuda.device(C.device):
        if splitk:
            plan = sgemm_splitk_describe(batch, m, n, k, alpha, A, *sa, B, *sb, accumulate, C, *sc, num_cus=0)
            floats = plan["workspace_floats"]
            work = torch.empty(floats, dtype=torch.float32, device=C.device) if floats else None
            sgemm_strided_batched_splitk(batch, m, n, k, alpha, A, *sa, B, *sb, accumulate, C, *sc,
                                         work, floats, stream=stream)
            if work is not None:
                # The workspace must outlive the enqueued launches on `stream`.
                work.record_stream(stream if isinstance(stream, torch.cuda.Stream) else
                                   torch.cuda.ExternalStream(_binding._stream(stream)))
        else:
            sgemm_strided_batched_path(batch, m, n, k, alpha, A, *sa, B, *sb, accumulate, C, *sc,
                                       path=path, stream=stream)
    return C


def attention(Q, K, V, O, alpha: float = None, causal: bool = False, stream=None, splitkv: bool = True):
    """O <- softmax(alpha Q K^T [causal]) V for torch float32 views on one GPU.

    Q and O are [outer, heads, tq, d], K and V [outer, kv_heads, tk, d], any
    strides (a token-major cache [outer, t, heads, d] passes as
    ``x.transpose(1, 2)``, no copy); query head i reads KV head
    i // (heads // kv_heads).  alpha defaults to 1/sqrt(d).  With
    splitkv=True (the default) a decode-shaped call goes through
    sgemm_attention_splitkv with the workspace its plan asks for, allocated
    here with torch; any other call, and splitkv=False, through
    sgemm_attention.  Runs on ``stream`` (default: torch's current stream)
    and returns O.
    """
    import math
    import torch

    for t, nm in ((Q, "Q"), (K, "K"), (V, "V"), (O, "O")):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{nm} must be a torch.Tensor")
        if t.dtype != torch.float32 or t.device.type != "cuda" or t.dim() != 4:
            raise ValueError(f"{nm} must be a 4-D float32 tensor on the GPU")
    if not (Q.device == K.device == V.device == O.device):
        raise ValueError("Q, K, V and O must be on the same device")
    no, h, tq, d = Q.shape
    hk, tk = K.shape[1], K.shape[2]
    if tuple(O.shape) != (no, h, tq, d) or tuple(K.shape) != (no, hk, tk, d) or tuple(V.shape) != (no, hk, tk, d):
        raise ValueError(f"shape mismatch: Q {tuple(Q.shape)}, K {tuple(K.shape)}, V {tuple(V.shape)}, "
                         f"O {tuple(O.shape)}")
    if hk == 0 or h % hk:
        raise ValueError(f"{h} query heads do not split evenly over {hk} KV heads")
    g = h // hk
    if alpha is None:
        alpha = 1.0 / math.sqrt(d) if d else 1.0
    args = [no, h, tq, tk, d, alpha, int(causal), Q, *Q.stride(), K, K.stride(0), K.stride(1), g,
            K.stride(2), K.stride(3), V, *V.stride(), O, *O.stride()]
    if stream is None:
        stream = torch.cuda.current_stream(O.device)
    with torch.cuda.device(O.device):
        plan = sgemm_attention_splitkv_describe(*args, num_cus=0) if splitkv else {"chunks": 0}
        if plan["chunks"]:
            floats = plan["workspace_floats"]
            work = torch.empty(floats, dtype=torch.float32, device=O.device)
            sgemm_attention_splitkv(*args, work, floats, stream=stream)
            # The workspace must outlive the enqueued launches on `stream`.
            work.record_stream(stream if isinstance(stream, torch.cuda.Stream) else
                               torch.cuda.ExternalStream(_binding._stream(stream)))
        else:
            sgemm_attention(*args, stream=stream)
    return O
