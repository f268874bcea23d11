"""Thin Python binding of libpkv.so (include/pkv.h): argument marshalling only.

Every step of the path runs in the HIP library.  Tensors are passed by device
pointer; the stream is torch's current stream unless one is given.  If the
library is missing, loading fails with an error: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")

PKV_OK, PKV_EINVAL, PKV_ENOMEM, PKV_EUNSUPPORTED, PKV_EHIP, PKV_EWORKSPACE = 0, -1, -2, -3, -4, -5
PKV_F16, PKV_BF16, PKV_F32, PKV_FP8_E4M3 = 0, 1, 2, 3
PKV_FUSE_MAX_ITEMS = 320   # appended sequences kv_append_decode folds into the split kernel (include/pkv.h)

# Every entry point include/pkv.h declares.
EXPORTS = (
    "pkv_last_error", "pkv_version",
    "kv_block_pool_create", "kv_block_pool_destroy", "kv_seq_add", "kv_seq_import", "kv_seq_fork",
    "kv_seq_free", "kv_seq_info", "kv_pool_stats", "kv_reserve", "kv_append", "kv_append_tokens", "kv_write_tables",
    "kv_validate_tables", "kv_block_pool_attach_host_tier", "kv_seq_offload", "kv_seq_restore",
    "kv_host_tier_stats", "kv_block_pool_set_fp8_scales", "kv_quantize_fp8", "paged_attn_decode_fp8",
    "paged_attn_decode_partials_fp8", "paged_attn_prefill", "paged_attn_partition_size", "paged_attn_grid_waves", "paged_attn_workspace_bytes",
    "paged_attn_decode", "paged_attn_decode_partials", "paged_attn_merge", "paged_attn_plan",
    "paged_attn_decode_noalloc", "paged_attn_decode_launches", "pkv_read_probe",
    "kv_block_pool_attach_host_tier_fp8", "paged_attn_decode_partials_timed", "kv_append_decode",
)


class PkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"pkv status {code}: {msg}")
        self.code = code


class PoolDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_blocks", "block_size", "num_kv_heads", "head_dim", "kv_dtype", "max_seqs",
        "max_blocks_per_seq")]


class PrefillDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size", "num_blocks", "table_stride",
        "total_q", "max_context_len", "q_dtype", "kv_dtype", "out_dtype")]


class AttnDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_q_heads", "num_kv_heads", "head_dim", "block_size", "num_blocks",
        "table_stride", "max_context_len", "partition_size", "q_dtype", "kv_dtype", "out_dtype", "num_waves")]


_lib = None


def load(path: str = LIB_PATH):
    """Load libpkv.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_268_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    PI32 = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "pkv_last_error": ([], ctypes.c_char_p),
        "pkv_version": ([], ctypes.c_char_p),
        "kv_block_pool_create": ([ctypes.POINTER(PoolDesc), P, P, P, ctypes.POINTER(P)], ctypes.c_int),
        "kv_block_pool_destroy": ([P], None),
        "kv_seq_add": ([P, PI32], ctypes.c_int),
        "kv_seq_import": ([P, I32, P, I32, PI32], ctypes.c_int),
        "kv_seq_fork": ([P, I32, PI32], ctypes.c_int),
        "kv_seq_free": ([P, I32], ctypes.c_int),
        "kv_seq_info": ([P, I32, PI32, P, I32, PI32], ctypes.c_int),
        "kv_pool_stats": ([P, PI32, PI32, I32, PI32], ctypes.c_int),
        "kv_reserve": ([P, I32, P, P], ctypes.c_int),
        "kv_append": ([P, I32, P, P, P, P, P, P], ctypes.c_int),
        "kv_write_tables": ([P, P, P, P], ctypes.c_int),
        "kv_append_tokens": ([P, I32, P, P, P, P, P, P, P], ctypes.c_int),
        "kv_validate_tables": ([I32, P, I32, I32, P, I32, I32], ctypes.c_int),
        "kv_block_pool_attach_host_tier": ([P, I32, P, P], ctypes.c_int),
        "kv_block_pool_attach_host_tier_fp8": ([P, I32, P, P, P, P], ctypes.c_int),
        "kv_seq_offload": ([P, I32, P, I32, P], ctypes.c_int),
        "kv_seq_restore": ([P, I32, P, P], ctypes.c_int),
        "kv_host_tier_stats": ([P, PI32, I32, PI32], ctypes.c_int),
        "kv_block_pool_set_fp8_scales": ([P, P, P, P, P], ctypes.c_int),
        "kv_quantize_fp8": ([I32, P, P, P, I32, P, P, P, P, I32, I32, I32, P], ctypes.c_int),
        "paged_attn_decode_fp8": ([ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, ctypes.c_float, P, P, P, SZ, P],
                                  ctypes.c_int),
        "paged_attn_decode_partials_fp8": ([ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, ctypes.c_float, P, P, P,
                                            SZ, P], ctypes.c_int),
        "paged_attn_decode_partials_timed": ([ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, ctypes.c_float, P, P,
                                              P, SZ, P, P, P], ctypes.c_int),
        "kv_append_decode": ([P, I32, P, P, P, P, P, ctypes.POINTER(AttnDesc), P, ctypes.c_float, P, P, P, SZ, P, P, P],
                             ctypes.c_int),
        "paged_attn_partition_size": ([ctypes.POINTER(AttnDesc)], I32),
        "paged_attn_grid_waves": ([ctypes.POINTER(AttnDesc)], I32),
        "paged_attn_decode_launches": ([ctypes.POINTER(AttnDesc)], I32),
        "pkv_read_probe": ([P, SZ, I32, I32, P, P], ctypes.c_int),
        "paged_attn_workspace_bytes": ([ctypes.POINTER(AttnDesc)], SZ),
        "paged_attn_decode": ([ctypes.POINTER(AttnDesc), P, P, P, P, P, ctypes.c_float, P, P, P, SZ, P],
                              ctypes.c_int),
        "paged_attn_decode_partials": ([ctypes.POINTER(AttnDesc), P, P, P, P, P, ctypes.c_float, P, P, P, SZ, P],
                                       ctypes.c_int),
        "paged_attn_merge": ([ctypes.POINTER(AttnDesc), P, P, P, P, SZ, P], ctypes.c_int),
        "paged_attn_decode_noalloc": ([ctypes.POINTER(AttnDesc), P, P, P, P, P, ctypes.c_float, P, P, P],
                                      ctypes.c_int),
        "paged_attn_prefill": ([ctypes.POINTER(PrefillDesc), P, P, P, P, P, P, ctypes.c_float, P, P, P], ctypes.c_int),
        "paged_attn_plan": ([ctypes.POINTER(AttnDesc), P, P, I64, ctypes.POINTER(I64)], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def last_error() -> str:
    return load().pkv_last_error().decode()


def check(rc: int):
    if rc != PKV_OK:
        raise PkvError(rc, last_error())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def dtype_code(t) -> int:
    """Library dtype of a tensor; uint8 storage means E4M3 codes."""
    import torch
    return {torch.float16: PKV_F16, torch.bfloat16: PKV_BF16, torch.float32: PKV_F32,
            torch.uint8: PKV_FP8_E4M3}[t.dtype]


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------

def attn_desc(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, table_stride,
              max_context_len, partition_size=0, dtype=PKV_BF16, out_dtype=PKV_F32, num_waves=0,
              kv_dtype=None) -> AttnDesc:
    return AttnDesc(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, table_stride,
                    max_context_len, partition_size, dtype, dtype if kv_dtype is None else kv_dtype, out_dtype,
                    num_waves)


def desc_for(q, k_cache, block_tables, max_context_len, partition_size=0, out_dtype=None, num_waves=0) -> AttnDesc:
    B, Hq, D = q.shape
    NB, Hkv, bs, D2 = k_cache.shape
    assert D == D2
    od = PKV_F32 if out_dtype is None else out_dtype
    return attn_desc(B, Hq, Hkv, D, bs, NB, block_tables.stride(0), max_context_len, partition_size,
                     dtype_code(q), od, num_waves, kv_dtype=dtype_code(k_cache))


def partition_size(desc: AttnDesc) -> int:
    r = load().paged_attn_partition_size(ctypes.byref(desc))
    if r < 0:
        check(r)
    return r


def grid_waves(desc: AttnDesc) -> int:
    r = load().paged_attn_grid_waves(ctypes.byref(desc))
    if r < 0:
        check(r)
    return r


def decode_launches(desc: AttnDesc) -> int:
    """Launches of paged_attn_decode: 1 if no pair can span several segments, else 2 (split, merge)."""
    r = load().paged_attn_decode_launches(ctypes.byref(desc))
    if r < 0:
        check(r)
    return r


def workspace_bytes(desc: AttnDesc) -> int:
    return load().paged_attn_workspace_bytes(ctypes.byref(desc))


def workspace_views(desc: AttnDesc, ws):
    """(hdr int32, seg_out float [rows][GC][D], seg_lse float [rows][GC]) views of a uint8 workspace
    tensor, following the layout include/pkv.h documents for paged_attn_workspace_bytes."""
    import torch
    B, Hq, Hkv, D = desc.num_seqs, desc.num_q_heads, desc.num_kv_heads, desc.head_dim
    P, mc = desc.partition_size, desc.max_context_len
    hw = 2 if desc.kv_dtype == PKV_FP8_E4M3 and Hkv % 2 == 0 else 1
    GC = Hq // Hkv * hw
    pairs = B * (Hkv // hw)
    chunks = pairs * max(1, -(-mc // P)) if P > 0 else grid_waves(desc)
    rows = max(chunks + pairs, 1)
    up = lambda x: (x + 255) // 256 * 256
    hb, ob = up(4 * (3 + B)), up(rows * GC * D * 4)
    assert hb + ob + up(rows * GC * 4) == workspace_bytes(desc)
    hdr = ws[:4 * (3 + B)].view(torch.int32)
    seg_out = ws[hb:hb + rows * GC * D * 4].view(torch.float32).view(rows, GC, D)
    seg_lse = ws[hb + ob:hb + ob + rows * GC * 4].view(torch.float32).view(rows, GC)
    return hdr, seg_out, seg_lse


def alloc_workspace(desc: AttnDesc, device):
    """A workspace for `desc` (zero-filled; the library needs no particular contents)."""
    import torch
    n = workspace_bytes(desc)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, max_context_len: int, *,
           out=None, lse=None, partition_size: int = 0, workspace=None, stream=None, out_dtype=None,
           num_waves: int = 0, desc: Optional[AttnDesc] = None):
    """paged_attn_decode.  Returns out (allocated as fp32 unless given)."""
    import torch
    if desc is None:
        od = out_dtype if out_dtype is not None else (dtype_code(out) if out is not None else PKV_F32)
        desc = desc_for(q, k_cache, block_tables, max_context_len, partition_size, od, num_waves)
    if out is None:
        tdt = {PKV_F32: torch.float32, PKV_F16: torch.float16, PKV_BF16: torch.bfloat16}[desc.out_dtype]
        out = torch.empty(q.shape, dtype=tdt, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(desc, q.device)
    check(load().paged_attn_decode(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(block_tables), _ptr(context_lens), ctypes.c_float(scale), _ptr(out),
                                   _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def decode_noalloc(desc, q, k_cache, v_cache, block_tables, context_lens, scale, out, lse=None, stream=None):
    """paged_attn_decode_noalloc: the decode with the library's static scratch as its workspace."""
    check(load().paged_attn_decode_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                           _ptr(block_tables), _ptr(context_lens), ctypes.c_float(scale),
                                           _ptr(out), _ptr(lse), _stream(stream)))


def decode_partials(desc, q, k_cache, v_cache, block_tables, context_lens, scale, out, lse, workspace,
                    stream=None):
    check(load().paged_attn_decode_partials(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(block_tables), _ptr(context_lens), ctypes.c_float(scale),
                                            _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                            _stream(stream)))


def decode_partials_timed(desc, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, scale, out, lse,
                          workspace, start, stop, stream=None):
    """paged_attn_decode_partials_timed: start / stop are LaunchEvents stamped by the split dispatch itself
    (k_scale = v_scale = None for 16-bit K/V)."""
    check(load().paged_attn_decode_partials_timed(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                  _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
                                                  _ptr(context_lens), ctypes.c_float(scale), _ptr(out), _ptr(lse),
                                                  _ptr(workspace), workspace.numel(), start.handle, stop.handle,
                                                  _stream(stream)))


_hip = None


def _hip_runtime():
    """The HIP runtime this process already uses (the one libpkv.so and torch are linked against)."""
    global _hip
    if _hip is None:
        load()
        path = "libamdhip64.so"
        with open("/proc/self/maps") as f:
            for line in f:
                name = line.split()[-1]
                if os.path.basename(name).startswith("libamdhip64.so"):
                    path = name
                    break
        h = ctypes.CDLL(path)
        h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        _hip = h
    return _hip


class LaunchEvent:
    """A HIP event with timing, created on the current device, for paged_attn_decode_partials_timed."""

    def __init__(self):
        self.handle = ctypes.c_void_p()
        rc = _hip_runtime().hipEventCreate(ctypes.byref(self.handle))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed (hipError {rc})")

    def elapsed_ms(self, stop: "LaunchEvent") -> float:
        """Milliseconds from this event to stop (waits for stop)."""
        h = _hip_runtime()
        rc = h.hipEventSynchronize(stop.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventSynchronize failed (hipError {rc})")
        t = ctypes.c_float()
        rc = h.hipEventElapsedTime(ctypes.byref(t), self.handle, stop.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed (hipError {rc})")
        return float(t.value)

    def __del__(self):
        if _hip is not None and self.handle:
            _hip.hipEventDestroy(self.handle)
            self.handle = ctypes.c_void_p()


def decode_fp8(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, scale: float,
               max_context_len: int, *, out=None, lse=None, partition_size: int = 0, workspace=None, stream=None,
               out_dtype=None, num_waves: int = 0, desc: Optional[AttnDesc] = None):
    """paged_attn_decode_fp8: k_cache / v_cache uint8 E4M3 codes, k_scale / v_scale float [NB][Hkv]."""
    import torch
    if desc is None:
        od = out_dtype if out_dtype is not None else (dtype_code(out) if out is not None else PKV_F32)
        desc = desc_for(q, k_cache, block_tables, max_context_len, partition_size, od, num_waves)
    if out is None:
        tdt = {PKV_F32: torch.float32, PKV_F16: torch.float16, PKV_BF16: torch.bfloat16}[desc.out_dtype]
        out = torch.empty(q.shape, dtype=tdt, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(desc, q.device)
    check(load().paged_attn_decode_fp8(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                       _ptr(v_scale), _ptr(block_tables), _ptr(context_lens), ctypes.c_float(scale),
                                       _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def decode_partials_fp8(desc, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, scale, out, lse,
                        workspace, stream=None):
    check(load().paged_attn_decode_partials_fp8(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                                _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), _ptr(context_lens),
                                                ctypes.c_float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                                workspace.numel(), _stream(stream)))


def quantize_fp8(items, src_k, src_v, dst_k, dst_v, k_scale, v_scale, stream=None):
    """kv_quantize_fp8: items device int32 [n][3] (source block, destination block, used rows)."""
    n = items.shape[0]
    NB, Hkv, bs, D = src_k.shape
    check(load().kv_quantize_fp8(n, _ptr(items), _ptr(src_k), _ptr(src_v), dtype_code(src_k), _ptr(dst_k),
                                 _ptr(dst_v), _ptr(k_scale), _ptr(v_scale), Hkv, bs, D, _stream(stream)))


def prefill(q, k_cache, v_cache, block_tables, context_lens, cu_seqlens_q, scale: float, max_context_len: int, *,
            out=None, lse=None, out_dtype=None, stream=None, desc: Optional[PrefillDesc] = None):
    """paged_attn_prefill.  q [total_q][Hq][D]; cu_seqlens_q device int32 [B + 1].  Returns out."""
    import torch
    T, Hq, D = q.shape
    NB, Hkv, bs, D2 = k_cache.shape
    assert D == D2
    if desc is None:
        od = out_dtype if out_dtype is not None else (dtype_code(out) if out is not None else PKV_F32)
        desc = PrefillDesc(context_lens.shape[0], Hq, Hkv, D, bs, NB, block_tables.stride(0), T, max_context_len,
                           dtype_code(q), dtype_code(k_cache), od)
    if out is None:
        tdt = {PKV_F32: torch.float32, PKV_F16: torch.float16, PKV_BF16: torch.bfloat16}[desc.out_dtype]
        out = torch.empty(q.shape, dtype=tdt, device=q.device)
    check(load().paged_attn_prefill(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                    _ptr(context_lens), _ptr(cu_seqlens_q), ctypes.c_float(scale), _ptr(out), _ptr(lse),
                                    _stream(stream)))
    return out


def merge(desc, context_lens, out, lse, workspace, stream=None):
    check(load().paged_attn_merge(ctypes.byref(desc), _ptr(context_lens), _ptr(out), _ptr(lse),
                                  _ptr(workspace), workspace.numel(), _stream(stream)))


def plan(desc: AttnDesc, context_lens_host) -> np.ndarray:
    """Segments (seq, kv_head, slot, tok_lo, tok_hi) of the split as an int32 [n][5] array."""
    ctx = _i32(context_lens_host)
    n = ctypes.c_int64(0)
    lib = load()
    check(lib.paged_attn_plan(ctypes.byref(desc), ctx.ctypes.data, None, 0, ctypes.byref(n)))
    items = np.zeros((n.value, 5), dtype=np.int32)
    check(lib.paged_attn_plan(ctypes.byref(desc), ctx.ctypes.data, items.ctypes.data, n.value, ctypes.byref(n)))
    return items


def read_probe(buf, workgroups: int, nontemporal: bool, sink, stream=None):
    """pkv_read_probe: one streaming read of the device tensor buf (its whole 16 KiB pieces)."""
    check(load().pkv_read_probe(_ptr(buf), buf.numel() * buf.element_size(), workgroups, 1 if nontemporal else 0,
                                _ptr(sink), _stream(stream)))


def validate_tables(block_tables_host, context_lens_host, num_blocks: int, block_size: int,
                    table_width: Optional[int] = None):
    tab = _i32(block_tables_host)
    ctx = _i32(context_lens_host)
    w = tab.shape[1] if table_width is None else table_width
    check(load().kv_validate_tables(tab.shape[0], tab.ctypes.data, tab.shape[1], w, ctx.ctypes.data,
                                    num_blocks, block_size))


# ---------------------------------------------------------------------------
# Block pool
# ---------------------------------------------------------------------------

class BlockPool:
    """kv_block_pool_* over caller-owned k_cache / v_cache (device tensors or None)."""

    def __init__(self, num_blocks, block_size, num_kv_heads, head_dim, kv_dtype, max_seqs,
                 max_blocks_per_seq, k_cache=None, v_cache=None, alloc_order: Optional[Sequence[int]] = None):
        self.lib = load()
        self.desc = PoolDesc(num_blocks, block_size, num_kv_heads, head_dim, kv_dtype, max_seqs,
                             max_blocks_per_seq)
        order = None if alloc_order is None else _i32(alloc_order)
        self._order = order
        h = ctypes.c_void_p()
        check(self.lib.kv_block_pool_create(ctypes.byref(self.desc), _ptr(k_cache), _ptr(v_cache),
                                            None if order is None else order.ctypes.data, ctypes.byref(h)))
        self.handle = h
        self.k_cache, self.v_cache = k_cache, v_cache

    def close(self):
        if self.handle:
            self.lib.kv_block_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self) -> int:
        s = ctypes.c_int32()
        check(self.lib.kv_seq_add(self.handle, ctypes.byref(s)))
        return s.value

    def import_seq(self, length: int, blocks) -> int:
        b = _i32(blocks)
        s = ctypes.c_int32()
        check(self.lib.kv_seq_import(self.handle, length, b.ctypes.data if b.size else None, b.size,
                                     ctypes.byref(s)))
        return s.value

    def fork(self, src: int) -> int:
        s = ctypes.c_int32()
        check(self.lib.kv_seq_fork(self.handle, src, ctypes.byref(s)))
        return s.value

    def free(self, seq: int):
        check(self.lib.kv_seq_free(self.handle, seq))

    def info(self, seq: int):
        ln, nb = ctypes.c_int32(), ctypes.c_int32()
        check(self.lib.kv_seq_info(self.handle, seq, ctypes.byref(ln), None, 0, ctypes.byref(nb)))
        ids = np.zeros(nb.value, dtype=np.int32)
        check(self.lib.kv_seq_info(self.handle, seq, ctypes.byref(ln), ids.ctypes.data if nb.value else None,
                                   nb.value, ctypes.byref(nb)))
        return ln.value, ids.tolist()

    def stats(self, block: int = -1):
        nf, ns, rc = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(-1)
        check(self.lib.kv_pool_stats(self.handle, ctypes.byref(nf), ctypes.byref(ns), block, ctypes.byref(rc)))
        return nf.value, ns.value, rc.value

    def reserve(self, seq_ids) -> np.ndarray:
        ids = _i32(seq_ids)
        items = np.zeros((ids.size, 7), dtype=np.int32)
        check(self.lib.kv_reserve(self.handle, ids.size, ids.ctypes.data if ids.size else None,
                                  items.ctypes.data if ids.size else None))
        return items

    def append(self, seq_ids, k_new, v_new, block_tables, context_lens, stream=None):
        ids = _i32(seq_ids)
        check(self.lib.kv_append(self.handle, ids.size, ids.ctypes.data if ids.size else None, _ptr(k_new),
                                 _ptr(v_new), _ptr(block_tables), _ptr(context_lens), _stream(stream)))

    def append_decode(self, seq_ids, k_new, v_new, block_tables, context_lens, desc, q, scale, out, lse, workspace,
                      start=None, stop=None, stream=None):
        """kv_append_decode: append one token to each listed sequence and decode (16-bit pools); start / stop:
        LaunchEvents for the split dispatch, or None."""
        ids = _i32(seq_ids)
        check(self.lib.kv_append_decode(self.handle, ids.size, ids.ctypes.data if ids.size else None, _ptr(k_new),
                                        _ptr(v_new), _ptr(block_tables), _ptr(context_lens), ctypes.byref(desc),
                                        _ptr(q), ctypes.c_float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                        workspace.numel(), start.handle if start else None,
                                        stop.handle if stop else None, _stream(stream)))

    def append_tokens(self, seq_ids, counts, k_new, v_new, block_tables, context_lens, stream=None):
        ids, cnt = _i32(seq_ids), _i32(counts)
        assert ids.size == cnt.size
        check(self.lib.kv_append_tokens(self.handle, ids.size, ids.ctypes.data if ids.size else None,
                                        cnt.ctypes.data if cnt.size else None, _ptr(k_new), _ptr(v_new),
                                        _ptr(block_tables), _ptr(context_lens), _stream(stream)))

    def write_tables(self, block_tables, context_lens, stream=None):
        check(self.lib.kv_write_tables(self.handle, _ptr(block_tables), _ptr(context_lens), _stream(stream)))

    def set_fp8_scales(self, k_scale, v_scale, k_init, v_init):
        """8-bit pools: device scales [NB][Hkv] and default scales of new blocks [Hkv]."""
        check(self.lib.kv_block_pool_set_fp8_scales(self.handle, _ptr(k_scale), _ptr(v_scale), _ptr(k_init),
                                                    _ptr(v_init)))
        self._fp8_scales = (k_scale, v_scale, k_init, v_init)

    # -- host tier ----------------------------------------------------------
    def attach_host_tier(self, num_host_blocks: int, k_host, v_host):
        """k_host / v_host: pinned CPU tensors [num_host_blocks][Hkv][bs][D] (torch pin_memory=True)."""
        check(self.lib.kv_block_pool_attach_host_tier(self.handle, num_host_blocks, _ptr(k_host), _ptr(v_host)))
        self.k_host, self.v_host = k_host, v_host

    def attach_host_tier_fp8(self, num_host_blocks: int, k_host, v_host, k_scale_host, v_scale_host):
        """8-bit pools: pinned uint8 codes [num_host_blocks][Hkv][bs][D] and pinned float32 scales
        [num_host_blocks][Hkv] for K and V."""
        check(self.lib.kv_block_pool_attach_host_tier_fp8(self.handle, num_host_blocks, _ptr(k_host), _ptr(v_host),
                                                          _ptr(k_scale_host), _ptr(v_scale_host)))
        self.k_host, self.v_host = k_host, v_host
        self.k_scale_host, self.v_scale_host = k_scale_host, v_scale_host

    def offload(self, seq_ids, gpu_window: int, stream=None):
        ids = _i32(seq_ids)
        check(self.lib.kv_seq_offload(self.handle, ids.size, ids.ctypes.data if ids.size else None, gpu_window,
                                      _stream(stream)))

    def restore(self, seq_ids, stream=None):
        ids = _i32(seq_ids)
        check(self.lib.kv_seq_restore(self.handle, ids.size, ids.ctypes.data if ids.size else None,
                                      _stream(stream)))

    def host_stats(self, block: int = -1):
        nf, rc = ctypes.c_int32(), ctypes.c_int32(-1)
        check(self.lib.kv_host_tier_stats(self.handle, ctypes.byref(nf), block, ctypes.byref(rc)))
        return nf.value, rc.value
