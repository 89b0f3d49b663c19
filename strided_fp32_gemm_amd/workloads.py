"""Seeded synthetic inputs for the strided, batched fp32 product.

This module only draws numbers and lays them out in memory; it performs none
of the product's arithmetic.  Both sides of every parity check (the HIP
library and the CPU oracle) receive the very same host bytes from here.

Recipe (stated once, used everywhere):
  * numpy ``SeedSequence(2024)`` -- the seed kael's device tests use (kael
    book ch. 09 "CUDA backend", section "How it is tested") -- is spawned once
    per workload, and each workload's child is spawned once per tensor; every
    tensor is drawn from its own ``Generator(PCG64)``.
  * Values are drawn in float64 and rounded to float32 on the host.
  * "Stored" arrays are row-major and contiguous; a transposed read is the
    stored array with its row and column strides exchanged (StaleyNET
    "GPU Implementation", section "The matrix product").
  * Strides are (batch, row, col), counted in float elements.

The five workloads mirror the users of the product the pages name: a tiny
square product, a linear layer y = x W^T with W read transposed (rvllm post,
section "Matmuls go to cuBLAS"), both attention products over all heads and
sequences in one batch with 1/sqrt(head_dim) folded into alpha (same
section), a spectrogram-style product against a shared DFT basis (StaleyNET
"GPU Implementation", "The matrix product" names the spectrogram), and a large
square product with A read transposed, alpha = 0.5 and accumulation.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

ROOT_SEED = 2024

# Benchmark workloads.
WORKLOADS = ("square64", "linear_xWt", "attn_qk", "attn_pv", "spectrogram", "square4096_acc",
             "linear_bwd_dx", "linear_bwd_dw", "linear_xT", "linear_bias", "sqdist",
             "attn_qk_gqa", "attn_pv_gqa", "attn_fused", "attn_fused_causal", "skinny_xWt",
             "linear_dw_deep", "attn_decode")
# Entry point each workload goes through: "plain" (sgemm_strided_batched),
# "ex" (sgemm_strided_batched_ex), "dist" (sgemm_pairwise_sqdist) or
# "batched2" (sgemm_strided_batched2), "attention" (sgemm_attention) or
# "splitk" (sgemm_strided_batched_splitk, with the workspace its plan asks for)
# or "attention_splitkv" (sgemm_attention_splitkv, likewise).
KINDS = {"linear_bias": "ex", "sqdist": "dist", "attn_qk_gqa": "batched2",
         "attn_pv_gqa": "batched2", "attn_fused": "attention", "attn_fused_causal": "attention",
         "linear_dw_deep": "splitk", "attn_decode": "attention_splitkv"}


def kind(name: str) -> str:
    return KINDS.get(name, "plain")


# Children of the root seed, in spawn order (the two halves of the linear
# layer's backward pass share one draw of dy, W and x).
SEED_NAMES = ("square64", "linear_xWt", "attn_qk", "attn_pv", "spectrogram", "square4096_acc",
              "linear_bwd", "linear_xT", "linear_bias", "sqdist", "attn_qk_gqa", "attn_pv_gqa",
              "attn_fused", "skinny_xWt", "linear_dw_deep", "attn_decode")


@dataclasses.dataclass
class Operand:
    """A flat float32 host storage plus the (batch, row, col) strides of the
    logical matrix view over it."""
    storage: np.ndarray
    strides: tuple

    @property
    def s_batch(self):
        return self.strides[0]

    @property
    def s_row(self):
        return self.strides[1]

    @property
    def s_col(self):
        return self.strides[2]


@dataclasses.dataclass
class Vector:
    """A flat float32 host storage plus the (batch, index) strides of a
    batch of vectors over it (the general epilogue's row / column terms)."""
    storage: np.ndarray
    strides: tuple


@dataclasses.dataclass
class Problem:
    """One call: C <- alpha*A*B (+C) over batch x (m x k)(k x n), or, when
    `beta`, `row` or `col` is given, the general epilogue C <- alpha*A*B +
    beta*C + row[b,i] + col[b,j] (sgemm_strided_batched_ex)."""
    name: str
    batch: int
    m: int
    n: int
    k: int
    alpha: float
    accumulate: bool
    A: Operand
    B: Operand
    C: Operand          # storage holds C_old (read only when accumulating)
    notes: str = ""
    beta: float = None  # None: 1 if accumulate else 0, plain entry point
    row: Vector = None
    col: Vector = None

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.m * self.n * self.k

    @property
    def is_ex(self) -> bool:
        return self.beta is not None or self.row is not None or self.col is not None

    @property
    def beta_value(self) -> float:
        return self.beta if self.beta is not None else (1.0 if self.accumulate else 0.0)

    def ex_call_args(self, a, b, c, r=None, l=None):
        """Positional argument list of sgemm_strided_batched_ex (without the
        stream) with the storages replaced by a, b, c and the vectors by r, l
        (None when the problem has no such term)."""
        sr = self.row.strides if self.row is not None else (0, 0)
        sl = self.col.strides if self.col is not None else (0, 0)
        return [self.batch, self.m, self.n, self.k, self.alpha,
                a, *self.A.strides, b, *self.B.strides, self.beta_value, c, *self.C.strides,
                r, *sr, l, *sl]

    def call_args(self, a, b, c):
        """Positional argument list of the entry point with the three storages
        replaced by `a`, `b`, `c` (pointers or arrays)."""
        return [self.batch, self.m, self.n, self.k, self.alpha,
                a, *self.A.strides, b, *self.B.strides,
                int(self.accumulate), c, *self.C.strides]


def _children(name: str):
    idx = SEED_NAMES.index(name)
    return np.random.SeedSequence(ROOT_SEED).spawn(len(SEED_NAMES))[idx]


def _gens(name: str, count: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in _children(name).spawn(count)]


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32).ravel())


def square64() -> Problem:
    """1 x 64x64x64, A and B row-major U[-1,1], alpha 1, no accumulate."""
    ga, gb, gc = _gens("square64", 3)
    A = _f32(ga.uniform(-1.0, 1.0, (64, 64)))
    B = _f32(gb.uniform(-1.0, 1.0, (64, 64)))
    C = np.zeros(64 * 64, np.float32)
    return Problem("square64", 1, 64, 64, 64, 1.0, False,
                   Operand(A, (4096, 64, 1)), Operand(B, (4096, 64, 1)), Operand(C, (4096, 64, 1)))


def linear_xWt() -> Problem:
    """y = x W^T: x [2048][960] N(0,1), W stored [2560][960] N(0,0.02) and
    read transposed (B[p][j] = W[j][p], strides (0, 1, 960))."""
    gx, gw = _gens("linear_xWt", 2)
    x = _f32(gx.normal(0.0, 1.0, (2048, 960)))
    W = _f32(gw.normal(0.0, 0.02, (2560, 960)))
    y = np.zeros(2048 * 2560, np.float32)
    return Problem("linear_xWt", 1, 2048, 2560, 960, 1.0, False,
                   Operand(x, (0, 960, 1)), Operand(W, (0, 1, 960)), Operand(y, (0, 2560, 1)))


def attn_qk() -> Problem:
    """S = (1/8) Q K^T for 8 sequences x 15 heads = 120 batches, head-major
    [120][512][64]; K read transposed (strides (32768, 1, 64))."""
    gq, gk = _gens("attn_qk", 2)
    Q = _f32(gq.normal(0.0, 1.0, (120, 512, 64)))
    K = _f32(gk.normal(0.0, 1.0, (120, 512, 64)))
    S = np.zeros(120 * 512 * 512, np.float32)
    return Problem("attn_qk", 120, 512, 512, 64, 1.0 / math.sqrt(64.0), False,
                   Operand(Q, (32768, 64, 1)), Operand(K, (32768, 1, 64)),
                   Operand(S, (262144, 512, 1)))


def attn_pv() -> Problem:
    """O = P V: P [120][512][512] i.i.d. U[0, 1/512] (softmax-like row scale,
    not renormalised), V [120][512][64] N(0,1)."""
    gp, gv = _gens("attn_pv", 2)
    P = _f32(gp.uniform(0.0, 1.0 / 512.0, (120, 512, 512)))
    V = _f32(gv.normal(0.0, 1.0, (120, 512, 64)))
    O = np.zeros(120 * 512 * 64, np.float32)
    return Problem("attn_pv", 120, 512, 64, 512, 1.0, False,
                   Operand(P, (262144, 512, 1)), Operand(V, (32768, 64, 1)),
                   Operand(O, (32768, 64, 1)))


SPEC_BATCH, SPEC_FRAMES, SPEC_WIN, SPEC_HOP, SPEC_BINS = 4, 4096, 512, 128, 257
SPEC_RATE = 16000.0


def dft_basis(win: int = SPEC_WIN, bins: int = SPEC_BINS) -> np.ndarray:
    """[win][2*bins] real DFT basis: column j < bins is cos(2 pi j t / win),
    column bins + j is sin(2 pi j t / win); computed in fp64, rounded to fp32."""
    t = np.arange(win, dtype=np.float64)[:, None]
    j = np.arange(bins, dtype=np.float64)[None, :]
    ang = 2.0 * math.pi * ((t * j) % win) / win
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def spectrogram() -> Problem:
    """frames [4][4096][512] of a 3-tone signal plus N(0, 0.1) noise (hop 128)
    times the shared basis [512][514] (batch stride 0)."""
    gs = _gens("spectrogram", 2)
    gsig, gnoise = gs
    length = (SPEC_FRAMES - 1) * SPEC_HOP + SPEC_WIN
    s = np.arange(length, dtype=np.float64)
    frames = np.empty((SPEC_BATCH, SPEC_FRAMES, SPEC_WIN), np.float64)
    starts = np.arange(SPEC_FRAMES)[:, None] * SPEC_HOP + np.arange(SPEC_WIN)[None, :]
    for b in range(SPEC_BATCH):
        amp = gsig.uniform(0.1, 1.0, 3)
        freq = gsig.uniform(50.0, 4000.0, 3)
        phase = gsig.uniform(0.0, 2.0 * math.pi, 3)
        x = sum(amp[q] * np.sin(2.0 * math.pi * freq[q] * s / SPEC_RATE + phase[q]) for q in range(3))
        x = x + gnoise.normal(0.0, 0.1, length)
        frames[b] = x[starts]
    n = 2 * SPEC_BINS
    C = np.zeros(SPEC_BATCH * SPEC_FRAMES * n, np.float32)
    return Problem("spectrogram", SPEC_BATCH, SPEC_FRAMES, n, SPEC_WIN, 1.0, False,
                   Operand(_f32(frames), (SPEC_FRAMES * SPEC_WIN, SPEC_WIN, 1)),
                   Operand(_f32(dft_basis()), (0, n, 1)),
                   Operand(C, (SPEC_FRAMES * n, n, 1)))


def square4096_acc(batch: int = 4, size: int = 4096) -> Problem:
    """4 x 4096^3: A stored transposed [batch][k][m] and read with swapped
    strides, B row-major, all U[-1,1]; C_old U[-1,1], alpha 0.5, accumulate."""
    ga, gb, gc = _gens("square4096_acc", 3)
    s2 = size * size
    A = _f32(ga.uniform(-1.0, 1.0, batch * s2))
    B = _f32(gb.uniform(-1.0, 1.0, batch * s2))
    C = _f32(gc.uniform(-1.0, 1.0, batch * s2))
    return Problem("square4096_acc", batch, size, size, size, 0.5, True,
                   Operand(A, (s2, 1, size)), Operand(B, (s2, size, 1)), Operand(C, (s2, size, 1)))


def _linear_bwd_tensors():
    gy, gw, gx = _gens("linear_bwd", 3)
    dy = _f32(gy.normal(0.0, 1.0, (2048, 2560)))
    W = _f32(gw.normal(0.0, 0.02, (2560, 960)))
    x = _f32(gx.normal(0.0, 1.0, (2048, 960)))
    return dy, W, x


def linear_bwd_dx() -> Problem:
    """Backward of the linear layer y = x W^T, input gradient: dx = dy W
    (the left gradient dC B^T of "PyTorch demystified 3", Opt. 4, with B =
    W^T).  dy [2048][2560] N(0,1) row-major (k-fast), W stored [2560][960]
    N(0,0.02) read as stored (n-fast), dx [2048][960]."""
    dy, W, _ = _linear_bwd_tensors()
    dx = np.zeros(2048 * 960, np.float32)
    return Problem("linear_bwd_dx", 1, 2048, 960, 2560, 1.0, False,
                   Operand(dy, (0, 2560, 1)), Operand(W, (0, 960, 1)), Operand(dx, (0, 960, 1)))


def linear_bwd_dw() -> Problem:
    """Backward of the linear layer, weight gradient in W's own layout:
    dW = dy^T x (the right gradient A^T dC of the same page, transposed to
    match W [2560][960]).  dy read transposed (A[i][p] = dy[p][i], m-fast),
    x [2048][960] N(0,1) row-major (n-fast), same dy as linear_bwd_dx."""
    dy, _, x = _linear_bwd_tensors()
    dW = np.zeros(2560 * 960, np.float32)
    return Problem("linear_bwd_dw", 1, 2560, 960, 2048, 1.0, False,
                   Operand(dy, (0, 1, 2560)), Operand(x, (0, 960, 1)), Operand(dW, (0, 960, 1)))


def linear_xT() -> Problem:
    """The fourth transpose case at the linear layer's size: y = x W^T with
    the activations stored feature-major, x^T [960][2048] (A m-fast), and W
    stored [2560][960] read transposed (B k-fast)."""
    gx, gw = _gens("linear_xT", 2)
    xT = _f32(gx.normal(0.0, 1.0, (960, 2048)))
    W = _f32(gw.normal(0.0, 0.02, (2560, 960)))
    y = np.zeros(2048 * 2560, np.float32)
    return Problem("linear_xT", 1, 2048, 2560, 960, 1.0, False,
                   Operand(xT, (0, 1, 2048)), Operand(W, (0, 1, 960)), Operand(y, (0, 2560, 1)))


def linear_bias() -> Problem:
    """The linear layer with its bias fused into the product's epilogue
    ("PyTorch demystified 3", "Comparison with cuBLAS and outlook"): y = x W^T
    + b, x [2048][960] N(0,1), W stored [2560][960] N(0,0.02) read
    transposed, b [2560] N(0,1) added to every row (a column term)."""
    gx, gw, gb = _gens("linear_bias", 3)
    x = _f32(gx.normal(0.0, 1.0, (2048, 960)))
    W = _f32(gw.normal(0.0, 0.02, (2560, 960)))
    bias = _f32(gb.normal(0.0, 1.0, 2560))
    y = np.zeros(2048 * 2560, np.float32)
    return Problem("linear_bias", 1, 2048, 2560, 960, 1.0, False,
                   Operand(x, (0, 960, 1)), Operand(W, (0, 1, 960)), Operand(y, (0, 2560, 1)),
                   beta=0.0, col=Vector(bias, (0, 1)))


def skinny_xWt() -> Problem:
    """A skinny product: y = x W^T for 4 rows, x [4][4096] N(0,1), W stored
    [16384][4096] N(0,0.02) and read transposed (B k-fast), y [4][16384].
    Not a size the pages print: it is the skinny case of the wavefront
    fallback (a few rows, a long k, one large operand streamed once) at a
    size where HBM rather than launch overhead bounds it."""
    gx, gw = _gens("skinny_xWt", 2)
    x = _f32(gx.normal(0.0, 1.0, (4, 4096)))
    W = _f32(gw.normal(0.0, 0.02, (16384, 4096)))
    y = np.zeros(4 * 16384, np.float32)
    return Problem("skinny_xWt", 1, 4, 16384, 4096, 1.0, False,
                   Operand(x, (0, 4096, 1)), Operand(W, (0, 1, 4096)), Operand(y, (0, 16384, 1)))


def linear_dw_deep() -> Problem:
    """The weight gradient of a narrow layer over many tokens: dW = dy^T x
    (the right gradient A^T dC of "PyTorch demystified 3", Opt. 4), dy
    [16384][256] N(0,1) read transposed (A[i][p] = dy[p][i], m-fast), x
    [16384][256] N(0,1) row-major (n-fast), dW [256][256].  Not a size the
    pages print: a small output (16 tiles of 64 x 64) over a deep
    contraction, the case the split-k entry point serves."""
    gy, gx = _gens("linear_dw_deep", 2)
    dy = _f32(gy.normal(0.0, 1.0, (16384, 256)))
    x = _f32(gx.normal(0.0, 1.0, (16384, 256)))
    dW = np.zeros(256 * 256, np.float32)
    return Problem("linear_dw_deep", 1, 256, 256, 16384, 1.0, False,
                   Operand(dy, (0, 1, 256)), Operand(x, (0, 256, 1)), Operand(dW, (0, 256, 1)))


@dataclasses.dataclass
class DistProblem:
    """Squared distances D[b,i,j] = |X[b,i,:] - Y[b,j,:]|^2 between the rows
    of X [batch][m][k] and of Y [batch][n][k] (sgemm_pairwise_sqdist).  The
    FLOP count is the product's, 2*batch*m*n*k."""
    name: str
    batch: int
    m: int
    n: int
    k: int
    X: Operand
    Y: Operand
    D: Operand

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.m * self.n * self.k

    @property
    def workspace_floats(self) -> int:
        ny = 1 if self.Y.strides[0] == 0 else self.batch
        return self.batch * self.m + ny * self.n

    def call_args(self, x, y, d, ws):
        return [self.batch, self.m, self.n, self.k, x, *self.X.strides, y, *self.Y.strides,
                d, *self.D.strides, ws, self.workspace_floats]


def sqdist() -> DistProblem:
    """The tokenizer's distance table (StaleyNET "GPU Implementation", "The
    matrix product"): 4 x 4096 frame vectors of 512 features, N(0,1), against
    one shared codebook of 1024 entries, N(0,1) (batch stride 0).  The sizes
    are assumed; the page gives none."""
    gx, gy = _gens("sqdist", 2)
    X = _f32(gx.normal(0.0, 1.0, (4, 4096, 512)))
    Y = _f32(gy.normal(0.0, 1.0, (1024, 512)))
    D = np.zeros(4 * 4096 * 1024, np.float32)
    return DistProblem("sqdist", 4, 4096, 1024, 512, Operand(X, (4096 * 512, 512, 1)),
                       Operand(Y, (0, 512, 1)), Operand(D, (4096 * 1024, 1024, 1)))


@dataclasses.dataclass
class Operand2:
    """A flat float32 host storage plus the (outer, inner, row, col) strides
    of a two-level batch of matrices over it, and the group divisor of the
    inner level (entry i of the inner level reads matrix i // group)."""
    storage: np.ndarray
    strides: tuple
    group: int = 1


@dataclasses.dataclass
class Problem2:
    """One sgemm_strided_batched2 call: C[o,i] <- alpha * A[o, i//gA] @
    B[o, i//gB] (+C[o,i]) for o < nb_outer, i < nb_inner."""
    name: str
    nb_outer: int
    nb_inner: int
    m: int
    n: int
    k: int
    alpha: float
    accumulate: bool
    A: Operand2
    B: Operand2
    C: Operand2
    notes: str = ""

    @property
    def batch(self) -> int:
        return self.nb_outer * self.nb_inner

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.m * self.n * self.k

    def call_args(self, a, b, c):
        """Positional arguments of sgemm_strided_batched2 (and of the
        oracle's two-level product) with the storages replaced by a, b, c."""
        (ao, ai, ar, ac), (bo, bi, br, bc) = self.A.strides, self.B.strides
        return [self.nb_outer, self.nb_inner, self.m, self.n, self.k, self.alpha,
                a, ao, ai, self.A.group, ar, ac, b, bo, bi, self.B.group, br, bc,
                int(self.accumulate), c, *self.C.strides]


def layout2(nb_outer: int, count: int, rows: int, cols: int, order: str, transposed: bool = False):
    """Storage size and (outer, inner, row, col) strides of nb_outer x count
    matrices of rows x cols.  order "heads" stores [outer][count][r][c]
    (head-major); "tokens" stores [outer][r][count][c] (a [sequence][token]
    [head][dim] buffer, rows = tokens).  `transposed` reads the stored
    matrices transposed: the stored matrix is cols x rows and the row and
    column strides are exchanged."""
    sr, sc = (cols, rows) if transposed else (rows, cols)
    per = sr * count * sc
    if order == "heads":
        st = (per, sr * sc, sc, 1)
    elif order == "tokens":
        st = (per, sc, count * sc, 1)
    else:
        raise ValueError(order)
    if transposed:
        st = (st[0], st[1], st[3], st[2])
    return per * nb_outer, st


# SmolLM2-360M, the model the rvllm post runs: 15 query heads share 5
# key/value heads (3 per group), head_dim 64.
GQA_Q_HEADS, GQA_KV_HEADS, GQA_HEAD_DIM = 15, 5, 64
GQA_SEQS, GQA_TOKENS = 8, 512


def attn_qk_gqa() -> Problem2:
    """S = (1/8) Q K^T straight from the token-major projections: Q
    [8][512][15][64] and K [8][512][5][64] N(0,1), three query heads per KV
    head (gB = 3), S written head-major [8][15][512][512].  The same work as
    attn_qk, without the transposing copies and with 5 K heads instead of 15."""
    gq, gk = _gens("attn_qk_gqa", 2)
    no, h, hk, t, d = GQA_SEQS, GQA_Q_HEADS, GQA_KV_HEADS, GQA_TOKENS, GQA_HEAD_DIM
    nq, sq = layout2(no, h, t, d, "tokens")
    nk, sk = layout2(no, hk, d, t, "tokens", transposed=True)
    ns, ss = layout2(no, h, t, t, "heads")
    Q = _f32(gq.normal(0.0, 1.0, nq))
    K = _f32(gk.normal(0.0, 1.0, nk))
    S = np.zeros(ns, np.float32)
    return Problem2("attn_qk_gqa", no, h, t, t, d, 1.0 / math.sqrt(d), False,
                    Operand2(Q, sq), Operand2(K, sk, h // hk), Operand2(S, ss))


def attn_pv_gqa() -> Problem2:
    """O = P V written token-major: P [8][15][512][512] i.i.d. U[0, 1/512]
    (as attn_pv), V [8][512][5][64] N(0,1) shared by 3 query heads each
    (gB = 3), O [8][512][15][64] -- the layout the output projection reads,
    with no transposing copy."""
    gp, gv = _gens("attn_pv_gqa", 2)
    no, h, hk, t, d = GQA_SEQS, GQA_Q_HEADS, GQA_KV_HEADS, GQA_TOKENS, GQA_HEAD_DIM
    n_p, sp = layout2(no, h, t, t, "heads")
    nv, sv = layout2(no, hk, t, d, "tokens")
    n_o, so = layout2(no, h, t, d, "tokens")
    P = _f32(gp.uniform(0.0, 1.0 / t, n_p))
    V = _f32(gv.normal(0.0, 1.0, nv))
    O = np.zeros(n_o, np.float32)
    return Problem2("attn_pv_gqa", no, h, t, d, t, 1.0, False,
                    Operand2(P, sp), Operand2(V, sv, h // hk), Operand2(O, so))


@dataclasses.dataclass
class AttnProblem:
    """One sgemm_attention call: O[o,i] <- softmax(alpha Q[o,i] K[o,i//g]^T,
    causal or not) V[o,i//g] for o < nb_outer, i < nb_inner; Q, O are
    tq x d, K, V are tk x d.  Strides are (outer, inner, row, col)."""
    name: str
    nb_outer: int
    nb_inner: int
    tq: int
    tk: int
    d: int
    g: int
    alpha: float
    causal: bool
    Q: Operand2
    K: Operand2
    V: Operand2
    O: Operand2

    @property
    def batch(self) -> int:
        return self.nb_outer * self.nb_inner

    @property
    def visible_pairs(self) -> int:
        """(query, key) pairs the definition sums over, per (o, i)."""
        if not self.causal:
            return self.tq * self.tk
        shift = self.tk - self.tq
        return sum(min(q + shift + 1, self.tk) for q in range(self.tq))

    @property
    def flops(self) -> int:
        """The two products' multiply-adds over the visible pairs (2*d each
        for the scores and for P V)."""
        return 4 * self.d * self.batch * self.visible_pairs

    def call_args(self, q, k, v, o):
        """Positional arguments of sgemm_attention (and of the oracle's
        attention) with the storages replaced by q, k, v, o."""
        (ko, ki, kr, kc) = self.K.strides
        return [self.nb_outer, self.nb_inner, self.tq, self.tk, self.d, self.alpha, int(self.causal),
                q, *self.Q.strides, k, ko, ki, self.g, kr, kc, v, *self.V.strides, o, *self.O.strides]


def _attn_fused(name: str, causal: bool) -> AttnProblem:
    """The whole attention of one layer, fused: Q [8][512][15][64], K and V
    [8][512][5][64] token-major N(0,1), three query heads per KV head, alpha
    1/8, O [8][512][15][64] token-major (zero-filled)."""
    gq, gk, gv = _gens("attn_fused", 3)
    no, h, hk, t, d = GQA_SEQS, GQA_Q_HEADS, GQA_KV_HEADS, GQA_TOKENS, GQA_HEAD_DIM
    nq, sq = layout2(no, h, t, d, "tokens")
    nk, sk = layout2(no, hk, t, d, "tokens")
    Q = _f32(gq.normal(0.0, 1.0, nq))
    K = _f32(gk.normal(0.0, 1.0, nk))
    V = _f32(gv.normal(0.0, 1.0, nk))
    O = np.zeros(nq, np.float32)
    return AttnProblem(name, no, h, t, t, d, h // hk, 1.0 / math.sqrt(d), causal,
                       Operand2(Q, sq), Operand2(K, sk), Operand2(V, sk), Operand2(O, sq))


def attn_fused() -> AttnProblem:
    """Scores, softmax and P V in one launch over the attn_qk / attn_pv sizes
    (8 sequences x 15 query heads x 512 tokens, head_dim 64) with 5 KV heads;
    no mask."""
    return _attn_fused("attn_fused", False)


def attn_decode() -> AttnProblem:
    """One decode step of the same layer over a 4096-token context: for each
    of 8 sequences and 15 query heads one new query (the last position,
    causal) against a KV cache of 4096 positions, 5 KV heads (three query
    heads each), head_dim 64, token-major Q [8][1][15][64] and K, V
    [8][4096][5][64] N(0,1), alpha 1/8, O zero-filled; through
    sgemm_attention_splitkv.  The context length is not one the pages
    print: the cache is long enough that reading it, 84 MB, sets the time."""
    gq, gk, gv = _gens("attn_decode", 3)
    no, h, hk, d, ctx = GQA_SEQS, GQA_Q_HEADS, GQA_KV_HEADS, GQA_HEAD_DIM, 4096
    nq, sq = layout2(no, h, 1, d, "tokens")
    nk, sk = layout2(no, hk, ctx, d, "tokens")
    Q = _f32(gq.normal(0.0, 1.0, nq))
    K = _f32(gk.normal(0.0, 1.0, nk))
    V = _f32(gv.normal(0.0, 1.0, nk))
    O = np.zeros(nq, np.float32)
    return AttnProblem("attn_decode", no, h, 1, ctx, d, h // hk, 1.0 / math.sqrt(d), True,
                       Operand2(Q, sq), Operand2(K, sk), Operand2(V, sk), Operand2(O, sq))


def attn_fused_causal() -> AttnProblem:
    """attn_fused with the causal mask of a prefill (query q sees keys <= q);
    the same draw of Q, K, V."""
    return _attn_fused("attn_fused_causal", True)


BUILDERS = {
    "square64": square64,
    "linear_xWt": linear_xWt,
    "attn_qk": attn_qk,
    "attn_pv": attn_pv,
    "spectrogram": spectrogram,
    "square4096_acc": square4096_acc,
    "linear_bwd_dx": linear_bwd_dx,
    "linear_bwd_dw": linear_bwd_dw,
    "linear_xT": linear_xT,
    "linear_bias": linear_bias,
    "sqdist": sqdist,
    "attn_qk_gqa": attn_qk_gqa,
    "attn_pv_gqa": attn_pv_gqa,
    "attn_fused": attn_fused,
    "attn_fused_causal": attn_fused_causal,
    "skinny_xWt": skinny_xWt,
    "linear_dw_deep": linear_dw_deep,
    "attn_decode": attn_decode,
}


def workload(name: str):
    return BUILDERS[name]()


def algorithmic_bytes(p) -> int:
    """Bytes one call must move at least: every input element read once and
    every output element written once (plus C read when it is accumulated).
    A batch-stride-0 operand counts once."""
    if isinstance(p, AttnProblem):
        kv = -(-p.nb_inner // p.g)
        return 4 * p.nb_outer * (2 * p.nb_inner * p.tq * p.d + 2 * kv * p.tk * p.d)
    if isinstance(p, DistProblem):
        ny = 1 if p.Y.strides[0] == 0 else p.batch
        return 4 * (p.batch * p.m * p.k + ny * p.n * p.k + p.batch * p.m * p.n)
    if isinstance(p, Problem2):
        na, nb = -(-p.nb_inner // p.A.group), -(-p.nb_inner // p.B.group)
        a = p.nb_outer * na * p.m * p.k
        b = p.nb_outer * nb * p.k * p.n
        return 4 * (a + b + p.batch * p.m * p.n * (2 if p.accumulate else 1))
    a = (1 if p.A.strides[0] == 0 else p.batch) * p.m * p.k
    b = (1 if p.B.strides[0] == 0 else p.batch) * p.k * p.n
    c = p.batch * p.m * p.n * (2 if p.beta_value != 0 else 1)
    vec = 0
    if p.row is not None:
        vec += (1 if p.row.strides[0] == 0 else p.batch) * p.m
    if p.col is not None:
        vec += (1 if p.col.strides[0] == 0 else p.batch) * p.n
    return 4 * (a + b + c + vec)


# ---------------------------------------------------------------------------
# Parametric problems for parity tests.
# ---------------------------------------------------------------------------

def layout_strides(rows: int, cols: int, contiguous: str, pad: int = 0, batch_gap: int = 0):
    """Storage size and (batch, row, col) strides of a rows x cols logical
    matrix stored with `contiguous` in {"row", "col"}: "row" means the column
    index is the fast one (row-major), "col" means stored transposed.  `pad`
    adds unused elements after every stored line, `batch_gap` after every
    matrix."""
    if contiguous == "row":
        ld = cols + pad
        per = rows * ld
        return per + batch_gap, (per + batch_gap, ld, 1)
    if contiguous == "col":
        ld = rows + pad
        per = cols * ld
        return per + batch_gap, (per + batch_gap, 1, ld)
    raise ValueError(contiguous)


def random_problem(seed: int, batch: int, m: int, n: int, k: int, *,
                   a_major: str = "row", b_major: str = "row", c_major: str = "row",
                   alpha: float = 1.0, accumulate: bool = False,
                   pad: int = 0, b_broadcast: bool = False,
                   dist: str = "uniform", name: str = "random") -> Problem:
    """Random problem with the requested storage orders.

    dist: "uniform" U[-1,1]; "normal" N(0,1); "int" integers in [-3, 3]
    (every partial sum is exact in fp32, so the result is unique);
    "ones" every A and B entry 1.0.
    """
    ss = np.random.SeedSequence([ROOT_SEED, seed])
    ga, gb, gc = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(3)]

    def draw(g, count):
        if dist == "uniform":
            return _f32(g.uniform(-1.0, 1.0, count))
        if dist == "normal":
            return _f32(g.normal(0.0, 1.0, count))
        if dist == "int":
            return _f32(g.integers(-3, 4, count))
        if dist == "ones":
            return np.ones(count, np.float32)
        raise ValueError(dist)

    per_a, sa = layout_strides(m, k, a_major, pad, pad)
    per_b, sb = layout_strides(k, n, b_major, pad, pad)
    per_c, sc = layout_strides(m, n, c_major, pad, pad)
    nb_b = 1 if b_broadcast else batch
    if b_broadcast:
        sb = (0, sb[1], sb[2])
    A = draw(ga, max(per_a * batch, 1))
    B = draw(gb, max(per_b * nb_b, 1))
    if dist == "int":
        C = _f32(gc.integers(-3, 4, max(per_c * batch, 1)))
    else:
        C = _f32(gc.uniform(-1.0, 1.0, max(per_c * batch, 1)))
    return Problem(name, batch, m, n, k, alpha, accumulate,
                   Operand(A, sa), Operand(B, sb), Operand(C, sc))


def random_problem2(seed: int, nb_outer: int, nb_inner: int, m: int, n: int, k: int, *,
                    gA: int = 1, gB: int = 1, a_order: str = "tokens", a_trans: bool = False,
                    b_order: str = "tokens", b_trans: bool = False, c_order: str = "heads",
                    c_trans: bool = False, alpha: float = 1.0, accumulate: bool = False, dist: str = "normal",
                    name: str = "random2") -> Problem2:
    """Random two-level problem: A holds ceil(nb_inner/gA) matrices per outer
    entry, B ceil(nb_inner/gB), C nb_inner, each laid out by layout2 with the
    given order and transposition.  dist as for random_problem."""
    ss = np.random.SeedSequence([ROOT_SEED, 2, seed])
    ga, gb, gc = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(3)]

    def draw(g, count):
        count = max(count, 1)
        if dist == "uniform":
            return _f32(g.uniform(-1.0, 1.0, count))
        if dist == "normal":
            return _f32(g.normal(0.0, 1.0, count))
        if dist == "int":
            return _f32(g.integers(-3, 4, count))
        raise ValueError(dist)

    na, sa = layout2(nb_outer, -(-nb_inner // gA), m, k, a_order, a_trans)
    nb, sb = layout2(nb_outer, -(-nb_inner // gB), k, n, b_order, b_trans)
    nc, sc = layout2(nb_outer, nb_inner, m, n, c_order, c_trans)
    A, B = draw(ga, na), draw(gb, nb)
    C = _f32(gc.integers(-3, 4, max(nc, 1))) if dist == "int" else _f32(gc.uniform(-1.0, 1.0, max(nc, 1)))
    return Problem2(name, nb_outer, nb_inner, m, n, k, alpha, accumulate,
                    Operand2(A, sa, gA), Operand2(B, sb, gB), Operand2(C, sc))


def random_attention(seed: int, nb_outer: int, nb_inner: int, tq: int, tk: int, d: int, *,
                     g: int = 1, causal: bool = False, order: str = "tokens", alpha: float = None,
                     scale: float = 1.0, o_fill: float = 0.0, name: str = "random_attn") -> AttnProblem:
    """Random attention problem: Q, K, V N(0, scale^2) stored head-major or
    token-major (layout2), ceil(nb_inner/g) KV heads, O filled with o_fill;
    alpha defaults to 1/sqrt(d)."""
    ss = np.random.SeedSequence([ROOT_SEED, 3, seed])
    gq, gk, gv = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(3)]
    hk = -(-nb_inner // g)
    nq, sq = layout2(nb_outer, nb_inner, tq, d, order)
    nk, sk = layout2(nb_outer, hk, tk, d, order)
    Q = _f32(gq.normal(0.0, scale, max(nq, 1)))
    K = _f32(gk.normal(0.0, scale, max(nk, 1)))
    V = _f32(gv.normal(0.0, 1.0, max(nk, 1)))
    O = np.full(max(nq, 1), o_fill, np.float32)
    a = 1.0 / math.sqrt(d) if alpha is None else alpha
    return AttnProblem(name, nb_outer, nb_inner, tq, tk, d, g, a, causal,
                       Operand2(Q, sq), Operand2(K, sk), Operand2(V, sk), Operand2(O, sq))
