"""Weight-only block-INT4 MatMul (MatMulNBits contract) for AMD MI355X.

Thin Python binding over libmnb's C ABI (include/mnb.h).  This module only
checks torch tensors (device, dtype, shape, contiguity), allocates outputs with
torch, and passes raw pointers and the current HIP stream; every step of the
computation runs in the library's gfx950 kernels.  There is no fallback path:
a missing library raises.

    Y[M][N] = A[M][K] x dequant(B)[K][N] (+ bias)
    dequant(B)[k][n] = (q[n][k] - zp[n][k // block_size]) * scale[n][k // block_size]

Storage follows MatMulNBits: packed weights [N][nb][block_size/2] uint8 with
the low nibble holding the even k, scales [N][nb] in the activation dtype,
packed zero points [N][ceil(nb/2)] uint8 (default 8 when absent).
"""

from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence as TSeq, Tuple

import torch

from ._lib import BF16, F32, Desc, MatmulArgs, MnbError, check, lib  # noqa: F401

__all__ = [
    "Desc", "MnbError", "make_desc", "validate", "packed_weight_bytes",
    "scale_bytes", "zero_point_bytes", "gemv_max_k", "pack", "gemv", "gemm",
    "dequant", "PackedWeight", "Sequence", "version", "import_qdq", "qdq_is_native",
    "gather_rows", "argmax", "gemv_silu_mul", "workspace_bytes",
    "argmax_workspace_bytes", "workspace", "gemm_noalloc", "gemm_silu_mul",
    "gemm_silu_workspace_bytes", "gemv_rmsnorm", "PersistentStep",
]

_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}


def _code(dtype: torch.dtype) -> int:
    if dtype not in _DTYPES:
        raise TypeError(f"activation dtype must be float32 or bfloat16, got {dtype}")
    return _DTYPES[dtype]


def make_desc(K: int, N: int, block_size: int = 32,
              act_dtype: torch.dtype = torch.float32,
              has_zero_points: bool = False, accuracy_level: int = 4,
              bits: int = 4) -> Desc:
    return Desc(K=int(K), N=int(N), bits=int(bits), block_size=int(block_size),
                act_dtype=_code(act_dtype), has_zero_points=int(bool(has_zero_points)),
                accuracy_level=int(accuracy_level), reserved=0)


def validate(desc: Desc, M: int = 1) -> None:
    check(lib().mnb_validate(ctypes.byref(desc), int(M)), "mnb_validate")


def packed_weight_bytes(desc: Desc) -> int:
    return int(lib().mnb_packed_weight_bytes(ctypes.byref(desc)))


def scale_bytes(desc: Desc) -> int:
    return int(lib().mnb_scale_bytes(ctypes.byref(desc)))


def zero_point_bytes(desc: Desc) -> int:
    return int(lib().mnb_zero_point_bytes(ctypes.byref(desc)))


def gemv_max_k(desc: Desc) -> int:
    return int(lib().mnb_gemv_max_k(ctypes.byref(desc)))


def workspace_bytes(desc: Desc, M: int) -> int:
    """Workspace bytes mnb_gemm needs for (desc, M); 0 when none."""
    return int(lib().mnb_workspace_bytes(ctypes.byref(desc), int(M)))


def argmax_workspace_bytes(M: int, N: int) -> int:
    return int(lib().mnb_argmax_workspace_bytes(int(M), int(N)))


def workspace(nbytes: int, device="cuda") -> Optional[torch.Tensor]:
    """A caller-owned workspace of at least nbytes (None when nbytes is 0).
    torch's allocator returns 256-byte aligned blocks, as the library needs."""
    if nbytes <= 0:
        return None
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device)


def _ws(t: Optional[torch.Tensor], need: int, device):
    """(pointer, size) of the given workspace, or of a fresh one when none is
    given (the library itself never allocates)."""
    if need <= 0:
        return None, 0, t
    if t is None:
        t = workspace(need, device)
    _need(t, "workspace", torch.uint8)
    return ctypes.c_void_p(t.data_ptr()), t.numel(), t


def version() -> str:
    return lib().mnb_version().decode()


# ---- tensor plumbing ---------------------------------------------------------

def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: Optional[torch.Tensor], name: str, dtype: torch.dtype,
          numel: Optional[int] = None, shape: Optional[Tuple[int, ...]] = None):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _nb(K: int, bs: int) -> int:
    return -(-K // bs)


# ---- entry points --------------------------------------------------------------

def pack(q: torch.Tensor, zp: Optional[torch.Tensor] = None, block_size: int = 32,
         act_dtype: torch.dtype = torch.float32, stream=None
         ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Pack logical weights q[N][K] (uint8, 0..15) and optional zero points
    zp[N][nb] (uint8) into MatMulNBits storage on the GPU."""
    N, K = q.shape
    d = make_desc(K, N, block_size, act_dtype, zp is not None)
    _need(q, "q", torch.uint8, shape=(N, K))
    if zp is not None:
        _need(zp, "zp", torch.uint8, shape=(N, _nb(K, block_size)))
    b = torch.empty(packed_weight_bytes(d) or 1, dtype=torch.uint8, device=q.device)
    zpp = None
    if zp is not None:
        zpp = torch.empty(zero_point_bytes(d) or 1, dtype=torch.uint8, device=q.device)
    check(lib().mnb_pack(ctypes.byref(d), _ptr(q), _ptr(zp), _ptr(b), _ptr(zpp),
                         _stream(stream)), "mnb_pack")
    return b, zpp


def _matmul(fn: str, a: torch.Tensor, b_packed: torch.Tensor, scales: torch.Tensor,
            zp_packed: Optional[torch.Tensor], bias: Optional[torch.Tensor],
            K: int, N: int, block_size: int, out: Optional[torch.Tensor],
            stream, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    if a.dim() == 1:
        a = a.view(1, -1)
    M = a.shape[0]
    d = make_desc(K, N, block_size, a.dtype, zp_packed is not None)
    _need(a, "a", a.dtype, shape=(M, K))
    _need(b_packed, "b_packed", torch.uint8, numel=packed_weight_bytes(d))
    _need(scales, "scales", a.dtype, numel=N * _nb(K, block_size))
    if zp_packed is not None:
        _need(zp_packed, "zp_packed", torch.uint8, numel=zero_point_bytes(d))
    if bias is not None:
        _need(bias, "bias", torch.float32, numel=N)
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    _need(out, "out", a.dtype, shape=(M, N))
    f = getattr(lib(), fn)
    if fn == "mnb_gemm_noalloc":
        check(f(ctypes.byref(d), M, _ptr(a), _ptr(b_packed), _ptr(scales), _ptr(zp_packed),
                _ptr(bias), _ptr(out), _stream(stream)), fn)
    elif fn == "mnb_gemm":
        wp, wn, keep = _ws(ws, workspace_bytes(d, M), a.device)
        check(f(ctypes.byref(d), M, _ptr(a), _ptr(b_packed), _ptr(scales), _ptr(zp_packed),
                _ptr(bias), _ptr(out), wp, wn, _stream(stream)), fn)
        if keep is not None and ws is None and stream is not None:
            keep.record_stream(stream)     # freed only after the work on that stream
    else:
        check(f(ctypes.byref(d), M, _ptr(a), _ptr(b_packed), _ptr(scales), _ptr(zp_packed),
                _ptr(bias), _ptr(out), _stream(stream)), fn)
    return out


def gemv(a, b_packed, scales, zp_packed=None, bias=None, *, K, N, block_size,
         out=None, stream=None) -> torch.Tensor:
    """Decode GEMV: a is [1][K] (or [K]); returns y [1][N] in a's dtype."""
    return _matmul("mnb_gemv", a, b_packed, scales, zp_packed, bias, K, N, block_size,
                   out, stream)


def gemm(a, b_packed, scales, zp_packed=None, bias=None, *, K, N, block_size,
         out=None, stream=None, workspace=None) -> torch.Tensor:
    """Prefill GEMM: a is [M][K]; returns y [M][N] in a's dtype.  workspace:
    a uint8 device tensor of at least workspace_bytes(desc, M) bytes, or None
    to have one allocated through torch for this call."""
    return _matmul("mnb_gemm", a, b_packed, scales, zp_packed, bias, K, N, block_size,
                   out, stream, workspace)


def gemm_noalloc(a, b_packed, scales, zp_packed=None, bias=None, *, K, N, block_size,
                 out=None, stream=None) -> torch.Tensor:
    """mnb_gemm_noalloc: the prefill GEMM with its split-K partials in the
    library's static per-GPU array (no workspace; calls that may overlap on
    one GPU race on that array).  `out` should be given by callers that must
    not allocate."""
    return _matmul("mnb_gemm_noalloc", a, b_packed, scales, zp_packed, bias, K, N, block_size,
                   out, stream)


DEQUANT_F32, DEQUANT_BF16, DEQUANT_INT8 = 0, 1, 2


def dequant(b_packed, scales, zp_packed=None, *, K, N, block_size,
            act_dtype=torch.float32, out_kind=DEQUANT_F32, stream=None) -> torch.Tensor:
    """Test hook: dequantized weights w[N][K] (float32, bfloat16, or the int8
    integers q - zp)."""
    d = make_desc(K, N, block_size, act_dtype, zp_packed is not None)
    _need(b_packed, "b_packed", torch.uint8, numel=packed_weight_bytes(d))
    if out_kind != DEQUANT_INT8:
        _need(scales, "scales", act_dtype, numel=N * _nb(K, block_size))
    odt = {DEQUANT_F32: torch.float32, DEQUANT_BF16: torch.bfloat16,
           DEQUANT_INT8: torch.int8}[out_kind]
    w = torch.empty((N, K), dtype=odt, device=b_packed.device)
    check(lib().mnb_dequant(ctypes.byref(d), _ptr(b_packed), _ptr(scales),
                            _ptr(zp_packed), int(out_kind), _ptr(w), _stream(stream)),
          "mnb_dequant")
    return w


# ---- prepared plans and step driver ---------------------------------------------

def import_qdq(w_q: torch.Tensor, scales_q: torch.Tensor, zp_q: Optional[torch.Tensor],
               *, K: int, N: int, block_size: int = 32, axis: int = 0, stream=None
               ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Normalize a blocked UINT4 DequantizeLinear weight into MatMulNBits
    storage.  axis 0: W [K][N], scales/zero points [nb][N]; axis 1: W [N][K]
    (tied embedding / LM head), scales/zero points [N][nb].  w_q and zp_q are
    flat uint8 streams (row-major elements, low nibble first); zp_q None means
    zero point 0.  Returns (b_packed, scales [N][nb], zp_packed)."""
    nb = _nb(K, block_size)
    d = make_desc(K, N, block_size, scales_q.dtype, True)
    _need(w_q, "w_q", torch.uint8, numel=(K * N + 1) // 2)
    _need(scales_q, "scales_q", scales_q.dtype, numel=nb * N)
    if zp_q is not None:
        _need(zp_q, "zp_q", torch.uint8, numel=(nb * N + 1) // 2)
    dev = w_q.device
    b = torch.empty(packed_weight_bytes(d), dtype=torch.uint8, device=dev)
    s = torch.empty((N, nb), dtype=scales_q.dtype, device=dev)
    z = torch.empty(zero_point_bytes(d), dtype=torch.uint8, device=dev)
    check(lib().mnb_import_qdq(ctypes.byref(d), int(axis), _ptr(w_q), _ptr(scales_q), _ptr(zp_q),
                               _ptr(b), _ptr(s), _ptr(z), _stream(stream)), "mnb_import_qdq")
    return b, s, z


def qdq_is_native(K: int, N: int, block_size: int = 32, axis: int = 1,
                  has_zero_points: bool = True) -> bool:
    """True when the axis-1 QDQ bytes already are MatMulNBits storage."""
    d = make_desc(K, N, block_size, torch.float32, has_zero_points)
    return bool(lib().mnb_qdq_is_native(ctypes.byref(d), int(axis)))


def gather_rows(ids: torch.Tensor, b_packed, scales, zp_packed=None, *, K: int, N: int,
                block_size: int, out=None, stream=None) -> torch.Tensor:
    """Tied-embedding lookup: rows ids of dequant(B)^T, [len(ids)][K] in the
    scales' dtype (ids int64; negative ids count from the end)."""
    d = make_desc(K, N, block_size, scales.dtype, zp_packed is not None)
    _need(ids, "ids", torch.int64)
    T = ids.numel()
    _need(b_packed, "b_packed", torch.uint8, numel=packed_weight_bytes(d))
    _need(scales, "scales", scales.dtype, numel=N * _nb(K, block_size))
    if zp_packed is not None:
        _need(zp_packed, "zp_packed", torch.uint8, numel=zero_point_bytes(d))
    if out is None:
        out = torch.empty((T, K), dtype=scales.dtype, device=scales.device)
    _need(out, "out", scales.dtype, shape=(T, K))
    check(lib().mnb_gather_rows(ctypes.byref(d), _ptr(ids), T, _ptr(b_packed), _ptr(scales),
                                _ptr(zp_packed), _ptr(out), _stream(stream)), "mnb_gather_rows")
    return out


def argmax(x: torch.Tensor, out=None, stream=None, workspace=None) -> torch.Tensor:
    """Row-wise greedy ArgMax (first maximum; a NaN counts as largest) of a
    float32 or bfloat16 [M][N] (or [N]) tensor; returns int64 [M].
    workspace: at least argmax_workspace_bytes(M, N) bytes, or None."""
    if x.dim() == 1:
        x = x.view(1, -1)
    M, N = x.shape
    _need(x, "x", x.dtype, shape=(M, N))
    if out is None:
        out = torch.empty(M, dtype=torch.int64, device=x.device)
    _need(out, "out", torch.int64, numel=M)
    wp, wn, keep = _ws(workspace, argmax_workspace_bytes(M, N), x.device)
    check(lib().mnb_argmax(_code(x.dtype), M, N, _ptr(x), _ptr(out), wp, wn, _stream(stream)),
          "mnb_argmax")
    if keep is not None and workspace is None and stream is not None:
        keep.record_stream(stream)
    return out


def gemv_silu_mul(a, b_packed, scales, zp_packed=None, bias=None, *, K, N, block_size,
                  out=None, stream=None) -> torch.Tensor:
    """Fused gate||up decode projection: B has N = 2I columns (gate, then
    up); returns h [1][I] = silu(y[:I]) * y[I:] with y = a x dequant(B) + bias."""
    if a.dim() == 1:
        a = a.view(1, -1)
    d = make_desc(K, N, block_size, a.dtype, zp_packed is not None)
    _need(a, "a", a.dtype, shape=(1, K))
    _need(b_packed, "b_packed", torch.uint8, numel=packed_weight_bytes(d))
    _need(scales, "scales", a.dtype, numel=N * _nb(K, block_size))
    if zp_packed is not None:
        _need(zp_packed, "zp_packed", torch.uint8, numel=zero_point_bytes(d))
    if bias is not None:
        _need(bias, "bias", torch.float32, numel=N)
    if out is None:
        out = torch.empty((1, N // 2), dtype=a.dtype, device=a.device)
    _need(out, "out", a.dtype, numel=N // 2)
    check(lib().mnb_gemv_silu_mul(ctypes.byref(d), 1, _ptr(a), _ptr(b_packed), _ptr(scales),
                                  _ptr(zp_packed), _ptr(bias), _ptr(out), _stream(stream)),
          "mnb_gemv_silu_mul")
    return out


def gemm_silu_workspace_bytes(desc: Desc, M: int) -> int:
    return int(lib().mnb_gemm_silu_workspace_bytes(ctypes.byref(desc), int(M)))


def gemm_silu_mul(a, b_packed, scales, zp_packed=None, bias=None, *, K, N, block_size,
                  out=None, stream=None, workspace=None) -> torch.Tensor:
    """Gated gate||up projection for any M: B has N = 2I columns (gate, then
    up); returns h [M][I] = silu(y[:, :I]) * y[:, I:] with y = a x dequant(B)
    + bias.  workspace: at least gemm_silu_workspace_bytes(desc, M) bytes, or
    None to have one allocated through torch."""
    if a.dim() == 1:
        a = a.view(1, -1)
    M = a.shape[0]
    d = make_desc(K, N, block_size, a.dtype, zp_packed is not None)
    _need(a, "a", a.dtype, shape=(M, K))
    _need(b_packed, "b_packed", torch.uint8, numel=packed_weight_bytes(d))
    _need(scales, "scales", a.dtype, numel=N * _nb(K, block_size))
    if zp_packed is not None:
        _need(zp_packed, "zp_packed", torch.uint8, numel=zero_point_bytes(d))
    if bias is not None:
        _need(bias, "bias", torch.float32, numel=N)
    if out is None:
        out = torch.empty((M, N // 2), dtype=a.dtype, device=a.device)
    _need(out, "out", a.dtype, numel=M * (N // 2))
    wp, wn, keep = _ws(workspace, gemm_silu_workspace_bytes(d, M), a.device)
    check(lib().mnb_gemm_silu_mul(ctypes.byref(d), M, _ptr(a), _ptr(b_packed), _ptr(scales),
                                  _ptr(zp_packed), _ptr(bias), _ptr(out), wp, wn, _stream(stream)),
          "mnb_gemm_silu_mul")
    if keep is not None and workspace is None and stream is not None:
        keep.record_stream(stream)
    return out


def gemv_rmsnorm(x, gamma, eps, b_packed, scales, zp_packed=None, bias=None, *, K, N, block_size,
                 out=None, stream=None) -> torch.Tensor:
    """Decode projection of an RMS-normalized row: y = (x / sqrt(mean(x^2) +
    eps) * gamma) x dequant(B) (+ bias), the normalization fused into the
    GEMV's input staging.  x [1][K] (or [K]) and gamma [K] share the
    activation dtype."""
    if x.dim() == 1:
        x = x.view(1, -1)
    d = make_desc(K, N, block_size, x.dtype, zp_packed is not None)
    _need(x, "x", x.dtype, shape=(1, K))
    _need(gamma, "gamma", x.dtype, numel=K)
    _need(b_packed, "b_packed", torch.uint8, numel=packed_weight_bytes(d))
    _need(scales, "scales", x.dtype, numel=N * _nb(K, block_size))
    if zp_packed is not None:
        _need(zp_packed, "zp_packed", torch.uint8, numel=zero_point_bytes(d))
    if bias is not None:
        _need(bias, "bias", torch.float32, numel=N)
    if out is None:
        out = torch.empty((1, N), dtype=x.dtype, device=x.device)
    _need(out, "out", x.dtype, numel=N)
    check(lib().mnb_gemv_rmsnorm(ctypes.byref(d), 1, _ptr(x), _ptr(gamma), float(eps), _ptr(b_packed),
                                 _ptr(scales), _ptr(zp_packed), _ptr(bias), _ptr(out), _stream(stream)),
          "mnb_gemv_rmsnorm")
    return out


class PackedWeight:
    """A prepared weight-only plan: packed weights, scales, optional packed
    zero points and optional fp32 bias of one (possibly fused) projection."""

    def __init__(self, K: int, N: int, block_size: int, act_dtype: torch.dtype,
                 b_packed: torch.Tensor, scales: torch.Tensor,
                 zp_packed: Optional[torch.Tensor] = None,
                 bias: Optional[torch.Tensor] = None):
        self.K, self.N, self.block_size, self.act_dtype = K, N, block_size, act_dtype
        self.b_packed, self.scales, self.zp_packed, self.bias = b_packed, scales, zp_packed, bias
        self.desc = make_desc(K, N, block_size, act_dtype, zp_packed is not None)
        _need(b_packed, "b_packed", torch.uint8, numel=packed_weight_bytes(self.desc))
        _need(scales, "scales", act_dtype, numel=N * _nb(K, block_size))
        if zp_packed is not None:
            _need(zp_packed, "zp_packed", torch.uint8, numel=zero_point_bytes(self.desc))
        if bias is not None:
            _need(bias, "bias", torch.float32, numel=N)

    @classmethod
    def from_logical(cls, q: torch.Tensor, scales: torch.Tensor,
                     zp: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                     block_size: int = 32, stream=None) -> "PackedWeight":
        N, K = q.shape
        b, zpp = pack(q, zp, block_size, scales.dtype, stream)
        return cls(K, N, block_size, scales.dtype, b, scales.contiguous(), zpp, bias)

    @property
    def weight_bytes(self) -> int:
        return (self.b_packed.numel() + self.scales.numel() * self.scales.element_size()
                + (0 if self.zp_packed is None else self.zp_packed.numel()))

    def matmul(self, a: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None,
               workspace: Optional[torch.Tensor] = None):
        """y = a x dequant(B) (+ bias): the decode GEMV for one row within the
        register kernel's K, the prefill GEMM otherwise."""
        one = a.dim() == 1 or a.shape[0] == 1
        if one and self.K <= gemv_max_k(self.desc):
            return gemv(a, self.b_packed, self.scales, self.zp_packed, self.bias, K=self.K,
                        N=self.N, block_size=self.block_size, out=out, stream=stream)
        return gemm(a, self.b_packed, self.scales, self.zp_packed, self.bias, K=self.K,
                    N=self.N, block_size=self.block_size, out=out, stream=stream,
                    workspace=workspace)

    def args(self, a: torch.Tensor, y: torch.Tensor) -> MatmulArgs:
        M = 1 if a.dim() == 1 else a.shape[0]
        _need(a, "a", self.act_dtype, numel=M * self.K)
        _need(y, "y", self.act_dtype, numel=M * self.N)
        return MatmulArgs(desc=self.desc, M=M, a=a.data_ptr(),
                          b_packed=self.b_packed.data_ptr(),
                          scales=self.scales.data_ptr(),
                          zp_packed=None if self.zp_packed is None else self.zp_packed.data_ptr(),
                          bias=None if self.bias is None else self.bias.data_ptr(),
                          y=y.data_ptr())


class Sequence:
    """An ordered list of projections run back to back on one stream (a decode
    or prefill step), either eagerly or as one captured HIP graph.  The caller
    keeps every tensor alive while the sequence exists.  The sequence owns
    one workspace for its split products (sized by the library's query) for
    eager runs, and a second one for its captured graph, so that a replay and
    eager runs never share partial sums."""

    def __init__(self, items: TSeq[Tuple[PackedWeight, torch.Tensor, torch.Tensor]]):
        self._keep: List = list(items)
        n = len(self._keep)
        self._args = (MatmulArgs * max(n, 1))()
        for i, (w, a, y) in enumerate(self._keep):
            self._args[i] = w.args(a, y)
        self.n = n
        self._graph = None
        self.workspace_bytes = int(lib().mnb_sequence_workspace_bytes(self._args, n))
        dev = self._keep[0][1].device if n else "cuda"
        self._ws = workspace(self.workspace_bytes, dev)
        self._graph_ws = None

    @staticmethod
    def _wsargs(t):
        return (None, 0) if t is None else (ctypes.c_void_p(t.data_ptr()), t.numel())

    def run(self, stream=None) -> None:
        check(lib().mnb_matmul_sequence(self._args, self.n, *self._wsargs(self._ws), _stream(stream)),
              "mnb_matmul_sequence")

    def capture(self) -> None:
        g = ctypes.c_void_p()
        if self._graph_ws is None and self.workspace_bytes:
            self._graph_ws = workspace(self.workspace_bytes, self._keep[0][1].device)
        check(lib().mnb_graph_create(self._args, self.n, *self._wsargs(self._graph_ws), ctypes.byref(g)),
              "mnb_graph_create")
        self._graph = g

    def replay(self, stream=None) -> None:
        if self._graph is None:
            raise RuntimeError("capture() first")
        check(lib().mnb_graph_launch(self._graph, _stream(stream)), "mnb_graph_launch")

    def close(self) -> None:
        if self._graph is not None:
            check(lib().mnb_graph_destroy(self._graph), "mnb_graph_destroy")
            self._graph = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class PersistentStep:
    """A decode step (every projection M == 1) as one cooperative launch of
    the library's persistent step kernel: each projection reads its input
    only after every workgroup has written the previous projection's output.
    The caller keeps every tensor alive while the step exists; the step owns
    the workspace that holds its arrival counters and projection table."""

    def __init__(self, items: TSeq[Tuple[PackedWeight, torch.Tensor, torch.Tensor]]):
        self._keep: List = list(items)
        n = len(self._keep)
        self._args = (MatmulArgs * max(n, 1))()
        for i, (w, a, y) in enumerate(self._keep):
            self._args[i] = w.args(a, y)
        self.n = n
        self._h = None
        self.workspace_bytes = int(lib().mnb_step_workspace_bytes(self._args, n))
        if self.workspace_bytes == 0:
            # the same checks again, for the library's reason
            check(lib().mnb_step_create(self._args, n, None, 0, ctypes.byref(ctypes.c_void_p())),
                  "mnb_step_create")
        dev = self._keep[0][1].device
        self._ws = workspace(self.workspace_bytes, dev)
        h = ctypes.c_void_p()
        check(lib().mnb_step_create(self._args, n, ctypes.c_void_p(self._ws.data_ptr()), self._ws.numel(),
                                    ctypes.byref(h)), "mnb_step_create")
        self._h = h

    def launch(self, stream=None) -> None:
        check(lib().mnb_step_launch(self._h, _stream(stream)), "mnb_step_launch")

    def trace_buffer(self) -> torch.Tensor:
        """Turns on the phase timestamps of later launches and returns their
        buffer: int64 [workgroups][entries][5] of the 100 MHz device clock
        (before the wait for the previous entry, after it, row staged, sums
        complete, outputs acknowledged)."""
        n = int(lib().mnb_step_trace_bytes(self._h)) // 8
        t = torch.zeros(n, dtype=torch.int64, device=self._keep[0][1].device)
        check(lib().mnb_step_set_trace(self._h, ctypes.c_void_p(t.data_ptr()), 8 * n), "mnb_step_set_trace")
        self._trace = t
        return t.view(-1, self.n, 5)

    def check(self, stream=None) -> None:
        """Synchronizes the stream; raises if a launch gave up waiting."""
        check(lib().mnb_step_check(self._h, _stream(stream)), "mnb_step_check")

    def close(self) -> None:
        if self._h is not None:
            check(lib().mnb_step_destroy(self._h), "mnb_step_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

