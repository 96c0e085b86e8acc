"""ctypes binding of libloopvq.so (argument marshalling only).

Every function keeps the C name.  Tensors must already live where the C ABI
expects them (device tensors on the current HIP device, except the host RoPE
table), with the documented dtype and a contiguous layout.  Work is enqueued
on torch's current stream.  A nonzero status raises LoopVQError.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libloopvq.so")

LOOPVQ_DTYPE_F32 = 0
LOOPVQ_DTYPE_BF16 = 1


class LoopVQError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({loopvq_status_string(status)})")
        self.status = status


class loopvq_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("D", "c", "Tc", "T", "bits", "K", "H_kv", "H_q", "page_size", "x_dtype", "io_dtype",
                 "per_group")]

    @classmethod
    def make(cls, D, c, Tc, T, bits, H_kv, H_q, page_size, x_dtype="bf16", io_dtype="bf16", per_group=0):
        dt = {"f32": LOOPVQ_DTYPE_F32, "bf16": LOOPVQ_DTYPE_BF16}
        return cls(D, c, Tc, T, bits, 1 << bits, H_kv, H_q, page_size,
                   dt.get(x_dtype, x_dtype), dt.get(io_dtype, io_dtype), int(per_group))

    @property
    def n_codebooks(self):
        """Codebooks per (block, KV head, K|V): 1, or D/c with one per channel group."""
        return self.D // self.c if self.per_group else 1

    @property
    def G(self):
        return self.c * self.Tc

    @property
    def n_blocks(self):
        return self.T // self.Tc

    @property
    def row_bytes(self):
        return self.D // self.c * self.bits // 8


class loopvq_bf16_window(ctypes.Structure):
    _fields_ = [("kv", ctypes.c_void_p), ("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
                ("n_sink", ctypes.c_void_p), ("win_start", ctypes.c_void_p)]


class loopvq_tasq(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("perm", ctypes.c_void_p), ("sigma", ctypes.c_void_p),
                ("sigma_stride", ctypes.c_int64)]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m decode_attention_loopvq_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int32
        D = ctypes.POINTER(loopvq_dims)
        L.loopvq_status_string.restype = ctypes.c_char_p
        L.loopvq_status_string.argtypes = [ctypes.c_int]
        L.loopvq_row_bytes.restype = ctypes.c_int
        L.loopvq_row_bytes.argtypes = [D]
        L.loopvq_build_codebook_slices.restype = ctypes.c_int
        L.loopvq_build_codebook_slices.argtypes = [D, P, P, P, P]
        L.loopvq_rope_table.restype = ctypes.c_int
        L.loopvq_rope_table.argtypes = [I, I, ctypes.c_double, P]
        L.loopvq_rope_table_floats.restype = ctypes.c_size_t
        L.loopvq_rope_table_floats.argtypes = [I, I]
        L.loopvq_encode.restype = ctypes.c_int
        L.loopvq_encode.argtypes = [D, I, I, I, P, P, P, P, P, P, ctypes.c_int64, P, P]
        L.loopvq_encode_pages.restype = ctypes.c_int
        L.loopvq_encode_pages.argtypes = [D, I, I, I, P, ctypes.c_int64, P, P, P, P, P, ctypes.c_int64, P]
        L.loopvq_decode_workspace_bytes.restype = ctypes.c_size_t
        L.loopvq_decode_workspace_bytes.argtypes = [D, I, I]
        L.loopvq_decode_attn.restype = ctypes.c_int
        L.loopvq_decode_attn.argtypes = [D, I, I, P, P, P, P, I, P, I, P, I, ctypes.c_float,
                                         P, P, P, ctypes.c_size_t, P]
        L.loopvq_decode_attn_noalloc.restype = ctypes.c_int
        L.loopvq_decode_attn_noalloc.argtypes = [D, I, I, P, P, P, P, I, P, I, P, I, ctypes.c_float, P, P, P]
        L.loopvq_decode_split.restype = ctypes.c_int
        L.loopvq_decode_split.argtypes = [D, I, I, P, P, P, P, I, P, I, P, I, ctypes.c_float, P,
                                          ctypes.c_size_t, P]
        L.loopvq_decode_combine.restype = ctypes.c_int
        L.loopvq_decode_combine.argtypes = [D, I, P, I, P, P, P, ctypes.c_size_t, P]
        L.loopvq_decode_attn_window.restype = ctypes.c_int
        L.loopvq_decode_attn_window.argtypes = [D, I, I, P, P, P, P, I, P, I, P, I,
                                                ctypes.POINTER(loopvq_bf16_window), ctypes.c_float,
                                                P, P, P, ctypes.c_size_t, P]
        L.loopvq_encode_tasq_workspace_bytes.restype = ctypes.c_size_t
        L.loopvq_encode_tasq_workspace_bytes.argtypes = [D, I, I]
        L.loopvq_encode_tasq.restype = ctypes.c_int
        L.loopvq_encode_tasq.argtypes = [D, I, I, I, P, P, ctypes.POINTER(loopvq_tasq), P, P, P, P,
                                         ctypes.c_int64, P, ctypes.c_size_t, P]
        L.loopvq_decode_attn_tasq.restype = ctypes.c_int
        L.loopvq_decode_attn_tasq.argtypes = [D, I, I, P, P, P, P, I, P, I, P, I, ctypes.POINTER(loopvq_tasq),
                                              ctypes.POINTER(loopvq_bf16_window), ctypes.c_float,
                                              P, P, P, ctypes.c_size_t, P]
        L.loopvq_kmeans_workspace_bytes.restype = ctypes.c_size_t
        L.loopvq_kmeans_workspace_bytes.argtypes = [D, I]
        L.loopvq_kmeans_update.restype = ctypes.c_int
        L.loopvq_kmeans_update.argtypes = [D, I, I, I, P, P, P, P, ctypes.c_int64, P, P, P, P, ctypes.c_size_t, P]
        _lib = L
    return _lib


EXPORTED = ("loopvq_status_string", "loopvq_row_bytes", "loopvq_build_codebook_slices",
            "loopvq_rope_table", "loopvq_rope_table_floats", "loopvq_encode", "loopvq_encode_pages",
            "loopvq_decode_workspace_bytes",
            "loopvq_decode_attn", "loopvq_decode_attn_noalloc", "loopvq_decode_split", "loopvq_decode_combine",
            "loopvq_decode_attn_window", "loopvq_encode_tasq_workspace_bytes", "loopvq_encode_tasq",
            "loopvq_decode_attn_tasq", "loopvq_kmeans_workspace_bytes", "loopvq_kmeans_update")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, what: str):
    if status != 0:
        raise LoopVQError(status, what)


def _need(t: torch.Tensor, dtype, name: str, device: bool = True):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _io_dtype(dims: loopvq_dims):
    return torch.float32 if dims.io_dtype == LOOPVQ_DTYPE_F32 else torch.bfloat16


def _decode_inputs(dims: loopvq_dims, q: torch.Tensor, index_cache: torch.Tensor, slices: torch.Tensor,
                   rope_table: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                   max_pos: Optional[int]) -> int:
    """Dtype, placement and shape checks shared by the decode calls; returns B."""
    _need(q, _io_dtype(dims), "q"); _need(index_cache, torch.uint8, "index_cache")
    _need(slices, torch.float16, "slices"); _need(rope_table, torch.float32, "rope_table")
    _need(block_table, torch.int32, "block_table"); _need(seq_lens, torch.int32, "seq_lens")
    if q.dim() != 3 or tuple(q.shape[1:]) != (dims.H_q, dims.D):
        raise ValueError(f"q must be [B][{dims.H_q}][{dims.D}], got {tuple(q.shape)}")
    B = q.shape[0]
    if seq_lens.numel() < B:
        raise ValueError(f"seq_lens holds {seq_lens.numel()} entries for {B} requests")
    if block_table.dim() != 2 or block_table.shape[0] < B:
        raise ValueError("block_table must be [B][max_pages]")
    if max_pos is None:
        raise ValueError("max_pos (positions covered by rope_table) is required")
    if rope_table.numel() < int(lib().loopvq_rope_table_floats(int(max_pos), int(dims.D))):
        raise ValueError(f"rope_table holds {rope_table.numel()} floats, fewer than {max_pos} positions need")
    return B


def _decode_outputs(dims: loopvq_dims, B: int, out: torch.Tensor, lse: Optional[torch.Tensor]) -> None:
    _need(out, _io_dtype(dims), "out")
    if tuple(out.shape) != (B, dims.H_q, dims.D):
        raise ValueError(f"out must be [{B}][{dims.H_q}][{dims.D}], got {tuple(out.shape)}")
    if lse is not None:
        _need(lse, torch.float32, "lse")
        if tuple(lse.shape) != (B, dims.H_q):
            raise ValueError(f"lse must be [{B}][{dims.H_q}], got {tuple(lse.shape)}")


def _workspace(dims: loopvq_dims, B: int, max_seq_len: int, workspace: Optional[torch.Tensor], device):
    need = loopvq_decode_workspace_bytes(dims, B, max_seq_len)
    if workspace is None:
        return torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    _need(workspace, torch.uint8, "workspace")
    return workspace


def loopvq_status_string(status: int) -> str:
    return lib().loopvq_status_string(int(status)).decode()


def loopvq_row_bytes(dims: loopvq_dims) -> int:
    r = lib().loopvq_row_bytes(ctypes.byref(dims))
    if r < 0:
        raise LoopVQError(r, "loopvq_row_bytes")
    return r


def loopvq_build_codebook_slices(dims: loopvq_dims, cb: torch.Tensor, slices=None, hsq=None):
    """cb [n_blocks][H_kv][2]([D/c])[K][G] fp16 -> (slices [T][H_kv][2]([D/c])[K][c] fp16, hsq fp32)."""
    _need(cb, torch.float16, "cb")
    ng = (dims.n_codebooks,) if dims.per_group else ()
    if slices is None:
        slices = torch.empty((dims.T, dims.H_kv, 2) + ng + (dims.K, dims.c), dtype=torch.float16, device=cb.device)
    if hsq is None:
        hsq = torch.empty((dims.n_blocks, dims.H_kv, 2) + ng + (dims.K,), dtype=torch.float32, device=cb.device)
    _check(lib().loopvq_build_codebook_slices(ctypes.byref(dims), _ptr(cb), _ptr(slices), _ptr(hsq),
                                              _stream()), "loopvq_build_codebook_slices")
    return slices, hsq


def loopvq_rope_table(max_pos: int, D: int, base: float = 10000.0) -> torch.Tensor:
    """Host table (float32, loopvq_rope_table_floats(max_pos, D) values) in the decode kernel's layout."""
    t = torch.empty(int(lib().loopvq_rope_table_floats(int(max_pos), int(D))), dtype=torch.float32)
    _check(lib().loopvq_rope_table(int(max_pos), int(D), float(base), _ptr(t) if max_pos > 0 else None),
           "loopvq_rope_table")
    return t


def loopvq_encode(dims: loopvq_dims, xk: torch.Tensor, xv: torch.Tensor, cb: torch.Tensor,
                  hsq: torch.Tensor, slot_mapping: torch.Tensor, index_cache: torch.Tensor,
                  first_block: int = 0, n_blocks: Optional[int] = None,
                  block_stride_bytes: Optional[int] = None,
                  near_tie_count: Optional[torch.Tensor] = None) -> None:
    """Encode xk, xv [n_blocks*Tc][n_tok][H_kv][D] into index_cache (uint8).

    cb / hsq hold all blocks of the layer; index_cache holds the cache of
    `first_block` first, the next block `block_stride_bytes` later.
    near_tie_count: None, or a device int32 tensor whose first element the
    call adds its near-tie count to (the caller zeroes it).
    """
    xdt = torch.float32 if dims.x_dtype == LOOPVQ_DTYPE_F32 else torch.bfloat16
    _need(xk, xdt, "xk"); _need(xv, xdt, "xv")
    _need(cb, torch.float16, "cb"); _need(hsq, torch.float32, "hsq")
    _need(slot_mapping, torch.int32, "slot_mapping"); _need(index_cache, torch.uint8, "index_cache")
    if near_tie_count is not None:
        _need(near_tie_count, torch.int32, "near_tie_count")
        if near_tie_count.numel() < 1:
            raise ValueError("near_tie_count must hold one element")
    if n_blocks is None:
        n_blocks = xk.shape[0] // dims.Tc
    n_tok = xk.shape[1]
    if xk.shape != xv.shape or xk.shape[0] != n_blocks * dims.Tc or slot_mapping.numel() != n_tok:
        raise ValueError("encode: inconsistent shapes")
    if block_stride_bytes is None:
        block_stride_bytes = index_cache.numel() // max(n_blocks, 1) if n_blocks > 1 else 0
    _check(lib().loopvq_encode(ctypes.byref(dims), n_tok, first_block, n_blocks, _ptr(xk), _ptr(xv),
                               _ptr(cb), _ptr(hsq), _ptr(slot_mapping), _ptr(index_cache),
                               int(block_stride_bytes), _ptr(near_tie_count), _stream()), "loopvq_encode")


def loopvq_encode_pages(dims: loopvq_dims, kv_pages: torch.Tensor, src_slot: torch.Tensor, cb: torch.Tensor,
                        hsq: torch.Tensor, slot_mapping: torch.Tensor, index_cache: torch.Tensor,
                        first_block: int = 0, n_blocks: Optional[int] = None,
                        block_stride_bytes: Optional[int] = None) -> None:
    """Code the tokens src_slot of bf16 page pools kv_pages [steps][num_pages][H_kv][2][8][D] (loop
    steps of blocks first_block.. in order) into index_cache, as loopvq_encode would."""
    _need(kv_pages, torch.bfloat16, "kv_pages"); _need(src_slot, torch.int32, "src_slot")
    _need(cb, torch.float16, "cb"); _need(hsq, torch.float32, "hsq")
    _need(slot_mapping, torch.int32, "slot_mapping"); _need(index_cache, torch.uint8, "index_cache")
    if n_blocks is None:
        n_blocks = kv_pages.shape[0] // dims.Tc
    if kv_pages.dim() != 6 or kv_pages.shape[0] < n_blocks * dims.Tc or slot_mapping.numel() != src_slot.numel():
        raise ValueError("encode_pages: inconsistent shapes")
    if block_stride_bytes is None:
        block_stride_bytes = index_cache.numel() // max(n_blocks, 1) if n_blocks > 1 else 0
    step_stride = kv_pages[0].numel()
    _check(lib().loopvq_encode_pages(ctypes.byref(dims), int(src_slot.numel()), first_block, n_blocks,
                                     _ptr(kv_pages), int(step_stride), _ptr(src_slot), _ptr(cb), _ptr(hsq),
                                     _ptr(slot_mapping), _ptr(index_cache), int(block_stride_bytes), _stream()),
           "loopvq_encode_pages")


def loopvq_decode_workspace_bytes(dims: loopvq_dims, B: int, max_seq_len: int) -> int:
    return int(lib().loopvq_decode_workspace_bytes(ctypes.byref(dims), int(B), int(max_seq_len)))


def loopvq_decode_attn(dims: loopvq_dims, t: int, q: torch.Tensor, index_cache: torch.Tensor,
                       slices: torch.Tensor, rope_table: torch.Tensor, block_table: torch.Tensor,
                       seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float = 0.0,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, max_pos: Optional[int] = None):
    """Decode attention at loop step t; returns (out [B][H_q][D], lse [B][H_q] or None)."""
    B = _decode_inputs(dims, q, index_cache, slices, rope_table, block_table, seq_lens, max_pos)
    if out is None:
        out = torch.empty((B, dims.H_q, dims.D), dtype=_io_dtype(dims), device=q.device)
    _decode_outputs(dims, B, out, lse)
    workspace = _workspace(dims, B, max_seq_len, workspace, q.device)
    max_pages = block_table.shape[1]
    _check(lib().loopvq_decode_attn(ctypes.byref(dims), int(t), B, _ptr(q), _ptr(index_cache),
                                    _ptr(slices), _ptr(rope_table), int(max_pos), _ptr(block_table),
                                    int(max_pages), _ptr(seq_lens), int(max_seq_len), float(sm_scale),
                                    _ptr(out), _ptr(lse), _ptr(workspace), int(workspace.numel()),
                                    _stream()), "loopvq_decode_attn")
    return out, lse


NOALLOC_SCRATCH_BYTES = 8 << 20   # LOOPVQ_NOALLOC_SCRATCH_BYTES


def loopvq_decode_attn_noalloc(dims: loopvq_dims, t: int, q: torch.Tensor, index_cache: torch.Tensor,
                               slices: torch.Tensor, rope_table: torch.Tensor, block_table: torch.Tensor,
                               seq_lens: torch.Tensor, max_seq_len: int, out: torch.Tensor,
                               lse: Optional[torch.Tensor] = None, sm_scale: float = 0.0,
                               max_pos: Optional[int] = None) -> None:
    """loopvq_decode_attn with its split partials in the library's fixed device scratch: the C call
    allocates nothing (out and lse are the caller's tensors)."""
    B = _decode_inputs(dims, q, index_cache, slices, rope_table, block_table, seq_lens, max_pos)
    _decode_outputs(dims, B, out, lse)
    _check(lib().loopvq_decode_attn_noalloc(ctypes.byref(dims), int(t), B, _ptr(q), _ptr(index_cache),
                                            _ptr(slices), _ptr(rope_table), int(max_pos), _ptr(block_table),
                                            int(block_table.shape[1]), _ptr(seq_lens), int(max_seq_len),
                                            float(sm_scale), _ptr(out), _ptr(lse), _stream()),
           "loopvq_decode_attn_noalloc")


def loopvq_decode_split(dims: loopvq_dims, t: int, q: torch.Tensor, index_cache: torch.Tensor,
                        slices: torch.Tensor, rope_table: torch.Tensor, block_table: torch.Tensor,
                        seq_lens: torch.Tensor, max_seq_len: int, workspace: torch.Tensor,
                        sm_scale: float = 0.0, max_pos: Optional[int] = None) -> None:
    """Split-K pass of decode attention; partials are left in `workspace`."""
    _decode_inputs(dims, q, index_cache, slices, rope_table, block_table, seq_lens, max_pos)
    _need(workspace, torch.uint8, "workspace")
    max_pages = block_table.shape[1]
    _check(lib().loopvq_decode_split(ctypes.byref(dims), int(t), q.shape[0], _ptr(q), _ptr(index_cache),
                                     _ptr(slices), _ptr(rope_table), int(max_pos), _ptr(block_table),
                                     int(max_pages), _ptr(seq_lens), int(max_seq_len), float(sm_scale),
                                     _ptr(workspace), int(workspace.numel()), _stream()), "loopvq_decode_split")


def loopvq_decode_combine(dims: loopvq_dims, B: int, seq_lens: torch.Tensor, max_seq_len: int,
                          workspace: torch.Tensor, out: torch.Tensor,
                          lse: Optional[torch.Tensor] = None) -> None:
    """Merge the split partials in `workspace` into out (and lse)."""
    _need(seq_lens, torch.int32, "seq_lens"); _need(workspace, torch.uint8, "workspace")
    if seq_lens.numel() < B:
        raise ValueError(f"seq_lens holds {seq_lens.numel()} entries for {B} requests")
    _decode_outputs(dims, int(B), out, lse)
    _check(lib().loopvq_decode_combine(ctypes.byref(dims), int(B), _ptr(seq_lens), int(max_seq_len), _ptr(out),
                                       _ptr(lse), _ptr(workspace), int(workspace.numel()), _stream()),
           "loopvq_decode_combine")


def loopvq_decode_attn_window(dims: loopvq_dims, t: int, q: torch.Tensor, index_cache: torch.Tensor,
                              slices: torch.Tensor, rope_table: torch.Tensor, block_table: torch.Tensor,
                              seq_lens: torch.Tensor, max_seq_len: int, kv_bf16: torch.Tensor,
                              page_table: torch.Tensor, n_sink: torch.Tensor, win_start: torch.Tensor,
                              sm_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                              lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                              max_pos: Optional[int] = None):
    """Decode attention over coded pages plus bf16 sink / recent-window pages.

    kv_bf16 [num_pages][H_kv][2][8][D] bf16 pages of loop step t; page_table
    [B][max_pages] int32 (bf16 token u of a request in page u // 8, slot u % 8);
    n_sink, win_start [B] int32.  Returns (out, lse).
    """
    B = _decode_inputs(dims, q, index_cache, slices, rope_table, block_table, seq_lens, max_pos)
    _need(kv_bf16, torch.bfloat16, "kv_bf16"); _need(page_table, torch.int32, "page_table")
    _need(n_sink, torch.int32, "n_sink"); _need(win_start, torch.int32, "win_start")
    if n_sink.numel() < B or win_start.numel() < B or page_table.dim() != 2 or page_table.shape[0] < B:
        raise ValueError("n_sink, win_start need B entries and page_table B rows")
    if out is None:
        out = torch.empty((B, dims.H_q, dims.D), dtype=_io_dtype(dims), device=q.device)
    _decode_outputs(dims, B, out, lse)
    workspace = _workspace(dims, B, max_seq_len, workspace, q.device)
    max_pages = block_table.shape[1]
    win = loopvq_bf16_window(kv_bf16.data_ptr(), page_table.data_ptr(),
                             page_table.shape[1] if page_table.dim() == 2 else 0,
                             n_sink.data_ptr(), win_start.data_ptr())
    _check(lib().loopvq_decode_attn_window(ctypes.byref(dims), int(t), B, _ptr(q), _ptr(index_cache),
                                           _ptr(slices), _ptr(rope_table), int(max_pos), _ptr(block_table),
                                           int(max_pages), _ptr(seq_lens), int(max_seq_len), ctypes.byref(win),
                                           float(sm_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                           int(workspace.numel()), _stream()), "loopvq_decode_attn_window")
    return out, lse


def _tasq_struct(dims: loopvq_dims, w: torch.Tensor, perm: torch.Tensor, sigma: torch.Tensor) -> loopvq_tasq:
    """w [T][H_kv][D] fp32, perm [T/Tc][H_kv][D/2] int32, sigma [T][n_slots] fp16 (device tensors)."""
    _need(w, torch.float32, "tasq w"); _need(perm, torch.int32, "tasq perm"); _need(sigma, torch.float16, "sigma")
    if tuple(w.shape) != (dims.T, dims.H_kv, dims.D) or tuple(perm.shape) != (dims.n_blocks, dims.H_kv, dims.D // 2):
        raise ValueError("tasq: w must be [T][H_kv][D] and perm [T/Tc][H_kv][D/2]")
    if sigma.dim() != 2 or sigma.shape[0] != dims.T:
        raise ValueError("sigma must be [T][n_slots]")
    return loopvq_tasq(w.data_ptr(), perm.data_ptr(), sigma.data_ptr(), int(sigma.shape[1]))


def loopvq_encode_tasq_workspace_bytes(dims: loopvq_dims, n_tok: int, n_blocks: int) -> int:
    return int(lib().loopvq_encode_tasq_workspace_bytes(ctypes.byref(dims), int(n_tok), int(n_blocks)))


def loopvq_encode_tasq(dims: loopvq_dims, xk: torch.Tensor, xv: torch.Tensor, w: torch.Tensor,
                       perm: torch.Tensor, sigma: torch.Tensor, cb: torch.Tensor, hsq: torch.Tensor,
                       slot_mapping: torch.Tensor, index_cache: torch.Tensor, first_block: int = 0,
                       n_blocks: Optional[int] = None, block_stride_bytes: Optional[int] = None,
                       workspace: Optional[torch.Tensor] = None) -> None:
    """loopvq_encode with TaSQ-coded keys; writes each token's fp16 sigma of every coded loop step
    into sigma [T][n_slots] at its slot.  cb holds codebooks of u for the keys."""
    xdt = torch.float32 if dims.x_dtype == LOOPVQ_DTYPE_F32 else torch.bfloat16
    _need(xk, xdt, "xk"); _need(xv, xdt, "xv")
    _need(cb, torch.float16, "cb"); _need(hsq, torch.float32, "hsq")
    _need(slot_mapping, torch.int32, "slot_mapping"); _need(index_cache, torch.uint8, "index_cache")
    tq = _tasq_struct(dims, w, perm, sigma)
    if n_blocks is None:
        n_blocks = xk.shape[0] // dims.Tc
    n_tok = xk.shape[1]
    if xk.shape != xv.shape or xk.shape[0] != n_blocks * dims.Tc or slot_mapping.numel() != n_tok:
        raise ValueError("encode_tasq: inconsistent shapes")
    if block_stride_bytes is None:
        block_stride_bytes = index_cache.numel() // max(n_blocks, 1) if n_blocks > 1 else 0
    need = loopvq_encode_tasq_workspace_bytes(dims, n_tok, n_blocks)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=xk.device)
    _check(lib().loopvq_encode_tasq(ctypes.byref(dims), n_tok, first_block, n_blocks, _ptr(xk), _ptr(xv),
                                    ctypes.byref(tq), _ptr(cb), _ptr(hsq), _ptr(slot_mapping), _ptr(index_cache),
                                    int(block_stride_bytes), _ptr(workspace), int(workspace.numel()), _stream()),
           "loopvq_encode_tasq")


def loopvq_decode_attn_tasq(dims: loopvq_dims, t: int, q: torch.Tensor, index_cache: torch.Tensor,
                            slices: torch.Tensor, rope_table: torch.Tensor, block_table: torch.Tensor,
                            seq_lens: torch.Tensor, max_seq_len: int, w: torch.Tensor, perm: torch.Tensor,
                            sigma: torch.Tensor, window: Optional[tuple] = None, sm_scale: float = 0.0,
                            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, max_pos: Optional[int] = None):
    """Decode attention at loop step t over TaSQ-coded keys; window = (kv_bf16, page_table, n_sink,
    win_start) adds the bf16 sink and recent window.  Returns (out, lse)."""
    B = _decode_inputs(dims, q, index_cache, slices, rope_table, block_table, seq_lens, max_pos)
    tq = _tasq_struct(dims, w, perm, sigma)
    if out is None:
        out = torch.empty((B, dims.H_q, dims.D), dtype=_io_dtype(dims), device=q.device)
    _decode_outputs(dims, B, out, lse)
    workspace = _workspace(dims, B, max_seq_len, workspace, q.device)
    win = None
    if window is not None:
        kv_bf16, page_table, n_sink, win_start = window
        _need(kv_bf16, torch.bfloat16, "kv_bf16"); _need(page_table, torch.int32, "page_table")
        _need(n_sink, torch.int32, "n_sink"); _need(win_start, torch.int32, "win_start")
        if n_sink.numel() < B or win_start.numel() < B or page_table.dim() != 2 or page_table.shape[0] < B:
            raise ValueError("n_sink, win_start need B entries and page_table B rows")
        win = loopvq_bf16_window(kv_bf16.data_ptr(), page_table.data_ptr(), page_table.shape[1],
                                 n_sink.data_ptr(), win_start.data_ptr())
    max_pages = block_table.shape[1]
    _check(lib().loopvq_decode_attn_tasq(ctypes.byref(dims), int(t), B, _ptr(q), _ptr(index_cache),
                                         _ptr(slices), _ptr(rope_table), int(max_pos), _ptr(block_table),
                                         int(max_pages), _ptr(seq_lens), int(max_seq_len), ctypes.byref(tq),
                                         None if win is None else ctypes.byref(win), float(sm_scale),
                                         _ptr(out), _ptr(lse), _ptr(workspace), int(workspace.numel()),
                                         _stream()), "loopvq_decode_attn_tasq")
    return out, lse


def loopvq_kmeans_workspace_bytes(dims: loopvq_dims, n_blocks: int) -> int:
    return int(lib().loopvq_kmeans_workspace_bytes(ctypes.byref(dims), int(n_blocks)))


def loopvq_kmeans_update(dims: loopvq_dims, xk: torch.Tensor, xv: torch.Tensor, slot_mapping: torch.Tensor,
                         index_cache: torch.Tensor, cb: torch.Tensor, cb_out: Optional[torch.Tensor] = None,
                         err: Optional[torch.Tensor] = None, first_block: int = 0, n_blocks: Optional[int] = None,
                         block_stride_bytes: Optional[int] = None, workspace: Optional[torch.Tensor] = None):
    """Codebook half of a Lloyd iteration after loopvq_encode assigned the codes; returns (cb_out, err)."""
    xdt = torch.float32 if dims.x_dtype == LOOPVQ_DTYPE_F32 else torch.bfloat16
    _need(xk, xdt, "xk"); _need(xv, xdt, "xv"); _need(cb, torch.float16, "cb")
    _need(slot_mapping, torch.int32, "slot_mapping"); _need(index_cache, torch.uint8, "index_cache")
    if n_blocks is None:
        n_blocks = xk.shape[0] // dims.Tc
    n_tok = xk.shape[1]
    if xk.shape != xv.shape or xk.shape[0] != n_blocks * dims.Tc or slot_mapping.numel() != n_tok:
        raise ValueError("kmeans_update: inconsistent shapes")
    if block_stride_bytes is None:
        block_stride_bytes = index_cache.numel() // max(n_blocks, 1) if n_blocks > 1 else 0
    if cb_out is None:
        cb_out = torch.empty_like(cb)
    _need(cb_out, torch.float16, "cb_out")
    if err is None:
        err = torch.zeros((dims.n_blocks, dims.H_kv, 2, 2), dtype=torch.float64, device=cb.device)
    _need(err, torch.float64, "err")
    need = loopvq_kmeans_workspace_bytes(dims, n_blocks)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=cb.device)
    _check(lib().loopvq_kmeans_update(ctypes.byref(dims), n_tok, first_block, n_blocks, _ptr(xk), _ptr(xv),
                                      _ptr(slot_mapping), _ptr(index_cache), int(block_stride_bytes), _ptr(cb),
                                      _ptr(cb_out), _ptr(err), _ptr(workspace), int(workspace.numel()), _stream()),
           "loopvq_kmeans_update")
    return cb_out, err
