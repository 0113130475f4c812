"""Python handle on the CPU oracle (``mnb_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this module; the product package never imports it.

The functions below only marshal numpy arrays into the C library; every
computation happens in ``mnb_oracle.c``. Arrays are numpy: bfloat16 data is
carried as uint16 bit patterns.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mnb_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F32, BF16 = 0, 1


def build(src: str = SRC, out: str = LIB, quiet: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", out, src, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + r.stdout + r.stderr)
    return out


class Oracle:
    """ctypes bindings of one compiled oracle library."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"{path} is missing; build it with oracle.build()")
        self.lib = L = ctypes.CDLL(path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        L.oracle_n_blocks.argtypes = [i64, i64]
        L.oracle_n_blocks.restype = i64
        L.oracle_contract_ok.argtypes = [i64, i64, i64, i64]
        L.oracle_contract_ok.restype = ctypes.c_int
        L.oracle_pack_weights.argtypes = [i64, i64, i64, vp, vp]
        L.oracle_unpack_weights.argtypes = [i64, i64, i64, vp, vp]
        L.oracle_pack_zero_points.argtypes = [i64, i64, vp, vp]
        L.oracle_unpack_zero_points.argtypes = [i64, i64, vp, vp]
        L.oracle_round_to_f32.argtypes = [i64, vp, vp]
        L.oracle_round_to_bf16.argtypes = [i64, vp, vp]
        L.oracle_dequant.argtypes = [i64, i64, i64, vp, vp, ctypes.c_int, vp,
                                     vp]
        L.oracle_dequant_int.argtypes = [i64, i64, i64, vp, vp, vp]
        L.oracle_matmul.argtypes = [i64, i64, i64, i64, ctypes.c_int, vp, vp,
                                    vp, vp, vp, vp, vp, ctypes.c_int]
        L.oracle_qdq_unpack.argtypes = [i64, vp, vp]
        L.oracle_qdq_dequant.argtypes = [i64, i64, i64, ctypes.c_int, vp, vp,
                                         ctypes.c_int, vp, vp]
        L.oracle_qdq_import.argtypes = [i64, i64, i64, ctypes.c_int, vp, vp,
                                        i64, vp, vp, vp, vp]
        L.oracle_silu_mul.argtypes = [i64, vp, vp, vp]
        L.oracle_rmsnorm.argtypes = [i64, i64, ctypes.c_int, vp, vp, ctypes.c_double, vp]
        L.oracle_matmul_f64a.argtypes = [i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_argmax.argtypes = [i64, i64, ctypes.c_int, vp, vp]
        for f in ("oracle_pack_weights", "oracle_unpack_weights",
                  "oracle_pack_zero_points", "oracle_unpack_zero_points",
                  "oracle_round_to_f32", "oracle_round_to_bf16",
                  "oracle_dequant", "oracle_dequant_int", "oracle_matmul"):
            getattr(L, f).restype = None

    # -- helpers ------------------------------------------------------------
    @staticmethod
    def _p(x: Optional[np.ndarray]):
        if x is None:
            return None
        assert x.flags["C_CONTIGUOUS"], "oracle inputs must be contiguous"
        return x.ctypes.data_as(ctypes.c_void_p)

    @staticmethod
    def _dtype_code(x: np.ndarray) -> int:
        if x.dtype == np.float32:
            return F32
        if x.dtype == np.uint16:
            return BF16
        raise TypeError(f"expected float32 or uint16 (bf16 bits), got {x.dtype}")

    def n_blocks(self, K: int, bs: int) -> int:
        return int(self.lib.oracle_n_blocks(K, bs))

    def contract_ok(self, K: int, N: int, bits: int, bs: int) -> bool:
        return bool(self.lib.oracle_contract_ok(K, N, bits, bs))

    # -- packing --------------------------------------------------------------
    def pack_weights(self, q: np.ndarray, bs: int) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.uint8)
        N, K = q.shape
        out = np.empty(N * self.n_blocks(K, bs) * (bs // 2), np.uint8)
        self.lib.oracle_pack_weights(K, N, bs, self._p(q), self._p(out))
        return out

    def unpack_weights(self, packed: np.ndarray, K: int, N: int,
                       bs: int) -> np.ndarray:
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        assert packed.size == N * self.n_blocks(K, bs) * (bs // 2)
        q = np.empty((N, K), np.uint8)
        self.lib.oracle_unpack_weights(K, N, bs, self._p(packed), self._p(q))
        return q

    def pack_zero_points(self, zp: np.ndarray) -> np.ndarray:
        zp = np.ascontiguousarray(zp, dtype=np.uint8)
        N, nb = zp.shape
        out = np.empty(N * ((nb + 1) // 2), np.uint8)
        self.lib.oracle_pack_zero_points(N, nb, self._p(zp), self._p(out))
        return out

    def unpack_zero_points(self, packed: np.ndarray, N: int,
                           nb: int) -> np.ndarray:
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        assert packed.size == N * ((nb + 1) // 2)
        zp = np.empty((N, nb), np.uint8)
        self.lib.oracle_unpack_zero_points(N, nb, self._p(packed),
                                           self._p(zp))
        return zp

    # -- conversions ----------------------------------------------------------
    def round_to_f32(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, np.float32)
        self.lib.oracle_round_to_f32(x.size, self._p(x), self._p(out))
        return out

    def round_to_bf16(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, np.uint16)
        self.lib.oracle_round_to_bf16(x.size, self._p(x), self._p(out))
        return out

    # -- dequantization ---------------------------------------------------------
    def dequant(self, q: np.ndarray, zp: Optional[np.ndarray],
                scales: np.ndarray, bs: int) -> np.ndarray:
        """Exact binary64 w[N][K] = (q - zp) * s."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        N, K = q.shape
        nb = self.n_blocks(K, bs)
        scales = np.ascontiguousarray(scales)
        assert scales.shape == (N, nb)
        if zp is not None:
            zp = np.ascontiguousarray(zp, dtype=np.uint8)
            assert zp.shape == (N, nb)
        w = np.empty((N, K), np.float64)
        self.lib.oracle_dequant(K, N, bs, self._p(q), self._p(zp),
                                self._dtype_code(scales), self._p(scales),
                                self._p(w))
        return w

    def dequant_int(self, q: np.ndarray, zp: Optional[np.ndarray],
                    bs: int) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.uint8)
        N, K = q.shape
        if zp is not None:
            zp = np.ascontiguousarray(zp, dtype=np.uint8)
        out = np.empty((N, K), np.int8)
        self.lib.oracle_dequant_int(K, N, bs, self._p(q), self._p(zp),
                                    self._p(out))
        return out

    # -- matmul -----------------------------------------------------------------
    def matmul(self, a: np.ndarray, q: np.ndarray, zp: Optional[np.ndarray],
               scales: np.ndarray, bs: int, bias: Optional[np.ndarray] = None,
               nthreads: int = 1):
        """Return (y, S): binary64 [M][N] results and tolerance scales."""
        a = np.ascontiguousarray(a)
        q = np.ascontiguousarray(q, dtype=np.uint8)
        scales = np.ascontiguousarray(scales)
        M, K = a.shape
        N, K2 = q.shape
        assert K == K2, (a.shape, q.shape)
        nb = self.n_blocks(K, bs)
        assert scales.shape == (N, nb), scales.shape
        code = self._dtype_code(a)
        assert self._dtype_code(scales) == code, "scales share A's dtype"
        if zp is not None:
            zp = np.ascontiguousarray(zp, dtype=np.uint8)
            assert zp.shape == (N, nb)
        if bias is not None:
            bias = np.ascontiguousarray(bias, dtype=np.float32)
            assert bias.shape == (N,)
        y = np.empty((M, N), np.float64)
        S = np.empty((M, N), np.float64)
        self.lib.oracle_matmul(M, K, N, bs, code, self._p(a), self._p(q),
                               self._p(zp), self._p(scales), self._p(bias),
                               self._p(y), self._p(S), int(nthreads))
        return y, S


    # -- RMSNorm into the projection input ------------------------------------
    def rmsnorm(self, x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
        """binary64 a[m][k] = x / sqrt(mean_k x^2 + eps) * gamma[k]."""
        x = np.ascontiguousarray(x)
        gamma = np.ascontiguousarray(gamma)
        M, K = x.shape
        code = self._dtype_code(x)
        assert self._dtype_code(gamma) == code and gamma.shape == (K,)
        a = np.empty((M, K), np.float64)
        self.lib.oracle_rmsnorm(M, K, code, self._p(x), self._p(gamma), float(eps), self._p(a))
        return a

    def matmul_f64a(self, a: np.ndarray, q: np.ndarray, zp: Optional[np.ndarray],
                    scales: np.ndarray, bs: int, bias: Optional[np.ndarray] = None):
        """(y, S) of binary64 activations a [M][K] against the quantized
        weight (scales float32 or bfloat16 bit patterns)."""
        a = np.ascontiguousarray(a, dtype=np.float64)
        q = np.ascontiguousarray(q, dtype=np.uint8)
        scales = np.ascontiguousarray(scales)
        M, K = a.shape
        N, K2 = q.shape
        assert K == K2
        nb = self.n_blocks(K, bs)
        assert scales.shape == (N, nb)
        if zp is not None:
            zp = np.ascontiguousarray(zp, dtype=np.uint8)
            assert zp.shape == (N, nb)
        if bias is not None:
            bias = np.ascontiguousarray(bias, dtype=np.float32)
        y = np.empty((M, N), np.float64)
        S = np.empty((M, N), np.float64)
        self.lib.oracle_matmul_f64a(M, K, N, bs, self._dtype_code(scales), self._p(a), self._p(q),
                                    self._p(zp), self._p(scales), self._p(bias), self._p(y), self._p(S))
        return y, S

    # -- the QDQ encoding -----------------------------------------------------
    def qdq_unpack(self, packed: np.ndarray, count: int) -> np.ndarray:
        """Elements 0..count-1 of a flat low-nibble-first UINT4 stream."""
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        assert packed.size >= (count + 1) // 2
        out = np.empty(count, np.uint8)
        self.lib.oracle_qdq_unpack(count, self._p(packed), self._p(out))
        return out

    def qdq_dequant(self, w_q: np.ndarray, zp_q: Optional[np.ndarray],
                    scales_q: np.ndarray, K: int, N: int, bs: int,
                    axis: int) -> np.ndarray:
        """DequantizeLinear of the QDQ tensors: exact binary64 [K][N]."""
        w_q = np.ascontiguousarray(w_q, dtype=np.uint8)
        scales_q = np.ascontiguousarray(scales_q)
        nb = self.n_blocks(K, bs)
        assert w_q.size == (K * N + 1) // 2 and scales_q.size == nb * N
        if zp_q is not None:
            zp_q = np.ascontiguousarray(zp_q, dtype=np.uint8)
            assert zp_q.size == (nb * N + 1) // 2
        out = np.empty((K, N), np.float64)
        self.lib.oracle_qdq_dequant(K, N, bs, axis, self._p(w_q), self._p(zp_q),
                                    self._dtype_code(scales_q), self._p(scales_q),
                                    self._p(out))
        return out

    def qdq_import(self, w_q: np.ndarray, zp_q: Optional[np.ndarray],
                   scales_q: np.ndarray, K: int, N: int, bs: int, axis: int):
        """(b_packed, scales [N][nb], zp_packed) in the MatMulNBits storage."""
        w_q = np.ascontiguousarray(w_q, dtype=np.uint8)
        scales_q = np.ascontiguousarray(scales_q)
        nb = self.n_blocks(K, bs)
        assert w_q.size == (K * N + 1) // 2 and scales_q.size == nb * N
        if zp_q is not None:
            zp_q = np.ascontiguousarray(zp_q, dtype=np.uint8)
            assert zp_q.size == (nb * N + 1) // 2
        b = np.empty(N * nb * (bs // 2), np.uint8)
        s = np.empty((N, nb), scales_q.dtype)
        z = np.empty(N * ((nb + 1) // 2), np.uint8)
        self.lib.oracle_qdq_import(K, N, bs, axis, self._p(w_q), self._p(zp_q),
                                   scales_q.itemsize, self._p(scales_q), self._p(b),
                                   self._p(s), self._p(z))
        return b, s, z

    # -- epilogues ----------------------------------------------------------------
    def silu_mul(self, gate: np.ndarray, up: np.ndarray) -> np.ndarray:
        gate = np.ascontiguousarray(gate, dtype=np.float64)
        up = np.ascontiguousarray(up, dtype=np.float64)
        assert gate.shape == up.shape
        h = np.empty(gate.shape, np.float64)
        self.lib.oracle_silu_mul(gate.size, self._p(gate), self._p(up), self._p(h))
        return h

    def argmax(self, x: np.ndarray) -> np.ndarray:
        """Row-wise greedy ArgMax of float32 or bfloat16 (uint16 bits) rows."""
        x = np.ascontiguousarray(x)
        if x.ndim == 1:
            x = x[None]
        M, N = x.shape
        idx = np.empty(M, np.int64)
        self.lib.oracle_argmax(M, N, self._dtype_code(x), self._p(x), self._p(idx))
        return idx


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built in-tree (built on first use when missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB):
            build()
        _default = Oracle(LIB)
    return _default
