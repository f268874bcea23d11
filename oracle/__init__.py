"""The CPU oracle for paged-KV attention decode.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library's code shares
nothing with it, and nothing in the GPU library imports it.

  * `paged_decode` -- fp64 gather + textbook softmax attention (oracle.c);
  * `replay`       -- integer replays of block allocation, slots and split-K
                      partitions (replay.py).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import replay  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

F16, BF16, FP8 = 0, 1, 3


def compile_c(src: str, out: str) -> str:
    """gcc build of an oracle source: plain IEEE double, no FMA contraction."""
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                           "-ffp-contract=off", "-fno-fast-math", src, "-o", tmp, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
        compile_c(SRC_PATH, LIB_PATH)
    return LIB_PATH


class OracleLib:
    """ctypes view of one build of oracle.c (tests may load a planted-mistake copy)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_paged_decode.argtypes = [i, i, i, i, i, i, i, i, i, P, P, P, P, P, P, P,
                                            ctypes.c_float, P, P, i]
        lib.oracle_paged_decode.restype = i
        lib.oracle_paged_decode_kv.argtypes = [i, i, i, i, i, i, i, i, i, i, P, P, P, P, P, P, P, P, P,
                                               ctypes.c_float, P, P, i]
        lib.oracle_paged_decode_kv.restype = i
        lib.oracle_fp8_encode.argtypes = [ctypes.c_float]
        lib.oracle_fp8_encode.restype = ctypes.c_uint8
        lib.oracle_fp8_encode_array.argtypes = [P, ctypes.c_int64, P]
        lib.oracle_fp8_encode_array.restype = None
        lib.oracle_quantize_fp8.argtypes = [P, i, i, i, i, P, P]
        lib.oracle_quantize_fp8.restype = None
        lib.oracle_paged_prefill.argtypes = [i, i, i, i, i, i, i, i, i, P, P, P, P, P, P, ctypes.c_float, P, P, i]
        lib.oracle_paged_prefill.restype = i
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = i
        lib.oracle_decode_value.argtypes = [ctypes.c_uint16, i]
        lib.oracle_decode_value.restype = ctypes.c_double
        self.lib = lib
        self.path = path

    def max_threads(self) -> int:
        return self.lib.oracle_max_threads()

    def decode_value(self, bits: int, dtype: int) -> float:
        return self.lib.oracle_decode_value(bits, dtype)

    def fp8_encode(self, x) -> np.ndarray:
        """Nearest E4M3 codes (saturating, ties to even) of fp32 values."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint8)
        self.lib.oracle_fp8_encode_array(_ptr(x), x.size, _ptr(out))
        return out

    def quantize_fp8(self, src_bits, src_dtype: int, ntok: int):
        """One (block, kv head) tile [bs][D] of 16-bit values -> (E4M3 codes [bs][D], fp32 scale)."""
        src = np.ascontiguousarray(src_bits, dtype=np.uint16)
        bs, D = src.shape
        codes = np.empty((bs, D), dtype=np.uint8)
        sc = np.empty(1, dtype=np.float32)
        self.lib.oracle_quantize_fp8(_ptr(src), src_dtype, ntok, bs, D, _ptr(codes), _ptr(sc))
        return codes, np.float32(sc[0])

    def paged_decode(self, q_bits, k_bits, v_bits, block_tables, context_lens, scale, *,
                     num_kv_heads, block_size, dtype, tok_lo=None, tok_hi=None,
                     nthreads=None, table_width=None, kv_dtype=None, k_scale=None, v_scale=None):
        """fp64 reference output [B][Hq][D] and lse [B][Hq] (natural log).

        q_bits [B][Hq][D]: raw uint16 storage of fp16 (dtype=F16) or bf16
        (dtype=BF16) values.  k_bits/v_bits [NB][Hkv][bs][D]: the same storage
        as q, or with kv_dtype=FP8 uint8 E4M3 codes with fp32 k_scale/v_scale
        [NB][Hkv].  block_tables int32 [B][W], context_lens int32 [B].  scale:
        the fp32 scale the GPU call receives.
        """
        kv_dtype = dtype if kv_dtype is None else kv_dtype
        kvt = np.uint8 if kv_dtype == FP8 else np.uint16
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        k_bits = np.ascontiguousarray(k_bits, dtype=kvt)
        v_bits = np.ascontiguousarray(v_bits, dtype=kvt)
        if kv_dtype == FP8:
            k_scale = np.ascontiguousarray(k_scale, dtype=np.float32)
            v_scale = np.ascontiguousarray(v_scale, dtype=np.float32)
            assert k_scale.shape == v_scale.shape == (k_bits.shape[0], num_kv_heads)
        else:
            k_scale = v_scale = None
        tables = np.ascontiguousarray(block_tables, dtype=np.int32)
        ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
        B, Hq, D = q_bits.shape
        NB = k_bits.shape[0]
        assert k_bits.shape == (NB, num_kv_heads, block_size, D) == v_bits.shape
        assert tables.ndim == 2 and tables.shape[0] == B and ctx.shape == (B,)
        lo = None if tok_lo is None else np.ascontiguousarray(tok_lo, dtype=np.int32)
        hi = None if tok_hi is None else np.ascontiguousarray(tok_hi, dtype=np.int32)
        out = np.empty((B, Hq, D), dtype=np.float64)
        lse = np.empty((B, Hq), dtype=np.float64)
        width = tables.shape[1] if table_width is None else table_width
        nt = self.max_threads() if nthreads is None else int(nthreads)
        rc = self.lib.oracle_paged_decode_kv(
            B, Hq, num_kv_heads, D, block_size, NB, tables.shape[1], width, dtype, kv_dtype,
            _ptr(q_bits), _ptr(k_bits), _ptr(v_bits), _ptr(k_scale), _ptr(v_scale), _ptr(tables), _ptr(ctx),
            _ptr(lo), _ptr(hi), ctypes.c_float(scale), _ptr(out), _ptr(lse), nt)
        if rc != 0:
            raise ValueError(f"oracle_paged_decode failed with status {rc}")
        return out, lse


    def paged_prefill(self, q_bits, k_bits, v_bits, block_tables, context_lens, cu_q, scale, *,
                      num_kv_heads, block_size, dtype, nthreads=None, table_width=None):
        """fp64 chunked-prefill output [total_q][Hq][D] and lse [total_q][Hq] (natural log).

        q_bits [total_q][Hq][D] (16-bit storage): rows cu_q[s] .. cu_q[s+1]-1 are
        sequence s's chunk, the last tokens of its context_lens[s]-token context.
        """
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        k_bits = np.ascontiguousarray(k_bits, dtype=np.uint16)
        v_bits = np.ascontiguousarray(v_bits, dtype=np.uint16)
        tables = np.ascontiguousarray(block_tables, dtype=np.int32)
        ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
        cu = np.ascontiguousarray(cu_q, dtype=np.int32)
        T, Hq, D = q_bits.shape
        B = ctx.shape[0]
        assert cu.shape == (B + 1,) and cu[-1] == T and tables.shape[0] == B
        NB = k_bits.shape[0]
        out = np.empty((T, Hq, D), dtype=np.float64)
        lse = np.empty((T, Hq), dtype=np.float64)
        width = tables.shape[1] if table_width is None else table_width
        nt = self.max_threads() if nthreads is None else int(nthreads)
        rc = self.lib.oracle_paged_prefill(B, Hq, num_kv_heads, D, block_size, NB, tables.shape[1], width, dtype,
                                           _ptr(q_bits), _ptr(k_bits), _ptr(v_bits), _ptr(tables), _ptr(ctx),
                                           _ptr(cu), ctypes.c_float(scale), _ptr(out), _ptr(lse), nt)
        if rc != 0:
            raise ValueError(f"oracle_paged_prefill failed with status {rc}")
        return out, lse


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


_default = None


def default() -> OracleLib:
    global _default
    if _default is None:
        _default = OracleLib(build())
    return _default


def max_threads() -> int:
    return default().max_threads()


def decode_value(bits: int, dtype: int) -> float:
    return default().decode_value(bits, dtype)


def paged_decode(*args, **kw):
    return default().paged_decode(*args, **kw)


def paged_prefill(*args, **kw):
    return default().paged_prefill(*args, **kw)


def fp8_encode(x):
    return default().fp8_encode(x)


def quantize_fp8(src_bits, src_dtype, ntok):
    return default().quantize_fp8(src_bits, src_dtype, ntok)


def _bits16(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def paged_decode_workload(wl, q, k, v, lib: OracleLib = None, **kw):
    """Oracle on a DecodeWorkload with torch tensors q, k, v (any device)."""
    dt = BF16 if wl.dtype == "bf16" else F16
    lib = default() if lib is None else lib
    return lib.paged_decode(_bits16(q), _bits16(k), _bits16(v), wl.block_tables, wl.context_lens,
                        wl.scale, num_kv_heads=wl.num_kv_heads, block_size=wl.block_size,
                        dtype=dt, **kw)
