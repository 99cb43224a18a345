"""Python binding of libattn (fused attention for MI355X / gfx950).

Thin ctypes marshalling over the C ABI declared in include/libattn.h: torch
tensors are checked for device, dtype, shape and contiguity, turned into
pointers and sizes, and the call is enqueued on torch's current HIP stream.
Every step of the computation runs in the HIP kernels of libattn.so; there is
no fallback path. If the shared library is missing, loading fails loudly.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os

__all__ = ["attn_fwd", "attn_decode_paged", "attn_fwd_paged", "attn_cache_append", "attn_cache_append_fp8",
           "attn_decode_paged_fp8", "attn_fwd_paged_fp8", "attn_fwd_fp8", "attn_cache_append_rope",
           "attn_fwd_paged_rope", "attn_decode_paged_rope", "attn_decode_workspace_bytes",
           "attn_gemm_splitk", "attn_decode_paged_noalloc", "attn_status_str", "attn_last_error", "AttnError", "lib",
           "LIB_PATH", "EXPORTS",
           "BLOCK_SIZE", "decode_workspace"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")
LIB_SINGLE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_single.so")
EXPORTS = ("attn_fwd", "attn_decode_paged", "attn_fwd_paged", "attn_cache_append", "attn_cache_append_fp8",
           "attn_decode_paged_fp8", "attn_fwd_paged_fp8", "attn_fwd_fp8", "attn_cache_append_rope",
           "attn_fwd_paged_rope", "attn_decode_paged_rope", "attn_decode_workspace_bytes", "attn_gemm_splitk",
           "attn_gemm_splitk_cfg", "attn_decode_paged_noalloc", "attn_status_str", "attn_last_error")
BLOCK_SIZE = 16

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3
ATTN_F16, ATTN_BF16 = 0, 1

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{attn_status_str(status)}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libattn.so (built in-tree by tiled_attention_02_amd.build)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def single_buffer_library():
    """Routes the calls made inside the block to libattn_single.so: the same library built with the
    prefill's debug key loop (one K and one V buffer, nothing overlapped), whose results must equal the
    pipelined kernel's bit for bit. Test use only."""
    global _lib
    prev = lib()
    _lib = _load(LIB_SINGLE_PATH)
    try:
        yield _lib
    finally:
        _lib = prev


_loaded = {}


def _load(path) -> ctypes.CDLL:
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m tiled_attention_02_amd.build` "
                          "(the HIP library is required; there is no fallback)")
    L = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i, vp]
    L.attn_fwd.restype = i
    L.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    L.attn_decode_paged.restype = i
    L.attn_fwd_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, i, vp]
    L.attn_fwd_paged.restype = i
    L.attn_cache_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp]
    L.attn_cache_append.restype = i
    L.attn_cache_append_fp8.argtypes = [vp, vp, vp, vp, f, f, vp, vp, vp, i, i, i, i, i, i, i, i, vp]
    L.attn_cache_append_fp8.restype = i
    L.attn_decode_paged_fp8.argtypes = [vp, vp, vp, f, f, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    L.attn_decode_paged_fp8.restype = i
    L.attn_fwd_fp8.argtypes = [vp, vp, vp, f, f, f, vp, vp, i, i, i, i, i, i, f, i, vp, i, vp]
    L.attn_fwd_fp8.restype = i
    L.attn_fwd_paged_fp8.argtypes = [vp, vp, vp, f, f, vp, i, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, i,
                                     vp]
    L.attn_fwd_paged_fp8.restype = i
    L.attn_cache_append_rope.argtypes = [vp, vp, vp, vp, vp, i, vp, vp, vp, i, i, i, i, i, i, i, i, vp]
    L.attn_cache_append_rope.restype = i
    L.attn_fwd_paged_rope.argtypes = [vp, vp, vp, vp, i, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, i, vp]
    L.attn_fwd_paged_rope.restype = i
    L.attn_decode_paged_rope.argtypes = [vp, vp, vp, vp, i, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    L.attn_decode_paged_rope.restype = i
    L.attn_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    L.attn_decode_paged_noalloc.restype = i
    L.attn_decode_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_gemm_splitk.argtypes = [vp, vp, vp, i, i, i, i, vp]
    L.attn_gemm_splitk.restype = i
    L.attn_gemm_splitk_cfg.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, vp]
    L.attn_gemm_splitk_cfg.restype = i
    L.attn_status_str.argtypes = [i]
    L.attn_status_str.restype = ctypes.c_char_p
    L.attn_last_error.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    _loaded[path] = L
    return L


def attn_status_str(status: int) -> str:
    return lib().attn_status_str(int(status)).decode()


def attn_last_error() -> str:
    return lib().attn_last_error().decode()


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float16:
        return ATTN_F16
    raise TypeError(f"libattn takes bfloat16 or float16 tensors, got {t.dtype}")


def _check(cond, msg):
    if not cond:
        raise ValueError(msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


@contextlib.contextmanager
def _on(first, *others):
    """Makes the device of `first` current for a library call (the C library launches on the current HIP
    device) after checking that every other tensor argument lives on that device."""
    import torch
    dev = first.device
    for t in others:
        if t is not None:
            _check(t.device == dev, f"every tensor must be on {dev} (found one on {t.device})")
    with torch.cuda.device(dev):
        yield


def _raise(status):
    if status != ATTN_OK:
        raise AttnError(status, attn_last_error())


def attn_fwd(q, k, v, scale: float | None = None, causal: bool = False, seq_lens=None, out=None, lse=None,
             need_lse: bool = True):
    """Fused attention forward. q [B,Hq,Tq,D], k/v [B,Hkv,Tk,D] on the GPU (bf16 or fp16).

    Returns (o [B,Hq,Tq,D] like q, lse [B,Hq,Tq] float32 or None). seq_lens is an
    int32 device tensor [B] for ragged batches (requires Tq == Tk).
    """
    import torch
    dt = _dtype_code(q)
    _check(q.is_cuda and k.is_cuda and v.is_cuda, "q, k, v must be GPU tensors")
    _check(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v must be 4-D [B,H,T,D]")
    _check(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v must share a dtype")
    _check(q.is_contiguous() and k.is_contiguous() and v.is_contiguous(), "q, k, v must be contiguous")
    B, Hq, Tq, D = q.shape
    _check(k.shape[0] == B and k.shape[3] == D and v.shape == k.shape, "k/v shape mismatch")
    Hkv, Tk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous() and out.is_cuda, "bad out")
    if need_lse and lse is None:
        lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse.shape == (B, Hq, Tq) and lse.dtype == torch.float32 and lse.is_contiguous(), "bad lse")
    if seq_lens is not None:
        _check(seq_lens.is_cuda and seq_lens.dtype == torch.int32 and seq_lens.numel() == B
               and seq_lens.is_contiguous(), "seq_lens must be a contiguous int32 GPU tensor [B]")
    with _on(q, k, v, out, lse, seq_lens):
        st = lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Tq, Tk, D,
                            ctypes.c_float(scale), int(bool(causal)), _ptr(seq_lens), dt, _stream(q.device))
    _raise(st)
    return out, lse


def attn_fwd_fp8(q, k, v, q_scale: float, k_scale: float, v_scale: float, scale: float | None = None,
                 causal: bool = False, seq_lens=None, out_dtype=None, out=None, lse=None, need_lse: bool = True):
    """Prefill attention on E4M3 inputs: q [B,Hq,Tq,D], k/v [B,Hkv,Tk,D] uint8 codes (an entry means
    value(code) * its scale). Returns (o [B,Hq,Tq,D] in out_dtype (bfloat16 default), lse float32 or None)."""
    import torch
    _check(q.is_cuda and k.is_cuda and v.is_cuda, "q, k, v must be GPU tensors")
    _check(q.dtype == torch.uint8 and k.dtype == torch.uint8 and v.dtype == torch.uint8, "q, k, v: uint8 E4M3 codes")
    _check(q.dim() == 4 and k.dim() == 4 and v.shape == k.shape, "q, k, v must be 4-D [B,H,T,D]")
    _check(q.is_contiguous() and k.is_contiguous() and v.is_contiguous(), "q, k, v must be contiguous")
    B, Hq, Tq, D = q.shape
    _check(k.shape[0] == B and k.shape[3] == D, "k/v shape mismatch")
    Hkv, Tk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    od = torch.bfloat16 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, Hq, Tq, D), dtype=od, device=q.device)
    dt = _dtype_code(out)
    _check(out.shape == (B, Hq, Tq, D) and out.is_contiguous() and out.is_cuda, "bad out")
    if need_lse and lse is None:
        lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    if seq_lens is not None:
        _check(seq_lens.is_cuda and seq_lens.dtype == torch.int32 and seq_lens.numel() == B
               and seq_lens.is_contiguous(), "seq_lens must be a contiguous int32 GPU tensor [B]")
    with _on(q, k, v, out, lse, seq_lens):
        st = lib().attn_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), ctypes.c_float(q_scale), ctypes.c_float(k_scale),
                                ctypes.c_float(v_scale), _ptr(out), _ptr(lse), B, Hq, Hkv, Tq, Tk, D, ctypes.c_float(scale),
                                int(bool(causal)), _ptr(seq_lens), dt, _stream(q.device))
    _raise(st)
    return out, lse


def attn_decode_workspace_bytes(B: int, Hq: int, Hkv: int, D: int, max_blocks_per_seq: int,
                                block_size: int = BLOCK_SIZE):
    return int(lib().attn_decode_workspace_bytes(B, Hq, Hkv, D, max_blocks_per_seq, block_size))


_workspaces = {}


def decode_workspace(device, nbytes: int):
    """A decode workspace of at least nbytes on device, kept per (device, stream) and reused."""
    import torch
    key = (str(device), torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def attn_decode_paged(q, k_cache, v_cache, block_table, ctx_lens, scale: float | None = None, out=None,
                      lse=None, workspace=None, need_lse: bool = True, rope=None):
    """Paged one-token decode. q [B,Hq,D]; caches [num_blocks,Hkv,16,D]; block_table int32
    [B,max_blocks]; ctx_lens int32 [B]. rope: optional float32 table [max_pos, D] (cos | sin halves):
    the query is rotated at position ctx - 1. Returns (o [B,Hq,D], lse [B,Hq] float32 or None)."""
    return _decode(q, k_cache, v_cache, None, block_table, ctx_lens, scale, out, lse, workspace, need_lse, rope)


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, ctx_lens, scale: float | None = None, out=None,
                              lse=None):
    """attn_decode_paged with the library's static per-GPU scratch instead of a workspace (no allocation in
    the library; out / lse may be passed in so that the call allocates nothing at all). Calls that overlap on
    one GPU race; the split partials of one call must fit in 32 MiB."""
    import torch
    dt = _dtype_code(q)
    _check(q.dim() == 3 and k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "bad q / cache rank or shape")
    _check(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype, "q and caches must share a dtype")
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (block_table, "block_table"),
                 (ctx_lens, "ctx_lens")):
        _check(t.is_cuda and t.is_contiguous(), f"{n} must be a contiguous GPU tensor")
    _check(block_table.dtype == torch.int32 and ctx_lens.dtype == torch.int32, "block_table/ctx_lens: int32")
    B, Hq, D = q.shape
    NB, Hkv, bs, Dk = k_cache.shape
    _check(Dk == D, "head size mismatch")
    _check(block_table.dim() == 2 and block_table.shape[0] == B and ctx_lens.numel() == B, "table shape")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous(), "bad out")
    if lse is not None:
        _check(lse.shape == (B, Hq) and lse.dtype == torch.float32 and lse.is_contiguous(), "bad lse")
    with _on(q, k_cache, v_cache, block_table, ctx_lens, out, lse):
        st = lib().attn_decode_paged_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                             _ptr(ctx_lens), _ptr(out), _ptr(lse), B, Hq, Hkv, D, bs,
                                             block_table.shape[1], NB, ctypes.c_float(scale), dt, _stream(q.device))
    _raise(st)
    return out, lse


def attn_decode_paged_fp8(q, k_cache, v_cache, k_scale: float, v_scale: float, block_table, ctx_lens,
                          scale: float | None = None, out=None, lse=None, workspace=None, need_lse: bool = True):
    """Paged one-token decode over E4M3 caches (uint8 [num_blocks,Hkv,16,D]; an entry means
    value(code) * k_scale or * v_scale). q, o bf16 or fp16."""
    return _decode(q, k_cache, v_cache, (k_scale, v_scale), block_table, ctx_lens, scale, out, lse, workspace,
                   need_lse, None)


def _check_rope(rope, D):
    import torch
    _check(rope.is_cuda and rope.dtype == torch.float32 and rope.is_contiguous() and rope.dim() == 2
           and rope.shape[1] == D, "rope must be a contiguous float32 GPU tensor [max_pos, D]")
    return rope.shape[0]


def _decode(q, k_cache, v_cache, scales, block_table, ctx_lens, scale, out, lse, workspace, need_lse, rope):
    import torch
    dt = _dtype_code(q)
    _check(q.dim() == 3 and k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "bad q / cache rank or shape")
    if scales is None:
        _check(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype, "q and caches must share a dtype")
    else:
        _check(k_cache.dtype == torch.uint8 and v_cache.dtype == torch.uint8, "E4M3 caches must be uint8 tensors")
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (block_table, "block_table"),
                 (ctx_lens, "ctx_lens")):
        _check(t.is_cuda and t.is_contiguous(), f"{n} must be a contiguous GPU tensor")
    _check(block_table.dtype == torch.int32 and ctx_lens.dtype == torch.int32, "block_table/ctx_lens: int32")
    B, Hq, D = q.shape
    NB, Hkv, bs, Dk = k_cache.shape
    _check(Dk == D, "head size mismatch")
    _check(block_table.dim() == 2 and block_table.shape[0] == B and ctx_lens.numel() == B, "table shape")
    maxb = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if need_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = attn_decode_workspace_bytes(B, Hq, Hkv, D, maxb, bs)
    if workspace is None:
        workspace = decode_workspace(q.device, need)
    tail = (_ptr(out), _ptr(lse), B, Hq, Hkv, D, bs, maxb, NB, ctypes.c_float(scale), dt, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(q.device))
    with _on(q, k_cache, v_cache, block_table, ctx_lens, out, lse, workspace, rope):
        if rope is not None:
            st = lib().attn_decode_paged_rope(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(rope), _check_rope(rope, D),
                                              _ptr(block_table), _ptr(ctx_lens), *tail)
        elif scales is None:
            st = lib().attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(ctx_lens), *tail)
        else:
            st = lib().attn_decode_paged_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.c_float(scales[0]),
                                             ctypes.c_float(scales[1]), _ptr(block_table), _ptr(ctx_lens), *tail)
    _raise(st)
    return out, lse


def _check_paged(caches, dtype, D):
    import torch
    k_cache, v_cache = caches
    _check(k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "caches must be [num_blocks, Hkv, 16, D]")
    _check(k_cache.dtype == dtype and v_cache.dtype == dtype, "caches must share the dtype of the inputs")
    _check(k_cache.shape[3] == D, "head size mismatch")
    _check(k_cache.is_cuda and v_cache.is_cuda and k_cache.is_contiguous() and v_cache.is_contiguous(),
           "caches must be contiguous GPU tensors")
    return k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]


def _check_i32(t, n, name, optional=False):
    import torch
    if t is None:
        _check(optional, f"{name} is required")
        return
    _check(t.is_cuda and t.dtype == torch.int32 and t.is_contiguous() and t.numel() == n,
           f"{name} must be a contiguous int32 GPU tensor of {n} elements")


def attn_fwd_paged(q, k_cache, v_cache, block_table, ctx_lens, q_lens=None, scale: float | None = None,
                   causal: bool = True, out=None, lse=None, need_lse: bool = True, rope=None):
    """Chunked prefill through the paged cache. q [B,Hq,Tq,D]: row i of sequence b is position
    ctx_lens[b] - q_lens[b] + i (q_lens None: all Tq rows). rope: optional float32 table [max_pos, D]
    (query rows rotated at their positions). Returns (o like q, lse [B,Hq,Tq] or None)."""
    return _fwd_paged(q, k_cache, v_cache, None, block_table, ctx_lens, q_lens, scale, causal, out, lse, need_lse,
                      rope)


def attn_fwd_paged_fp8(q, k_cache, v_cache, k_scale: float, v_scale: float, block_table, ctx_lens, q_lens=None,
                       scale: float | None = None, causal: bool = True, out=None, lse=None, need_lse: bool = True,
                       rope=None):
    """Chunked prefill over E4M3 caches (uint8 [num_blocks,Hkv,16,D]; an entry means value(code) * scale)."""
    return _fwd_paged(q, k_cache, v_cache, (k_scale, v_scale), block_table, ctx_lens, q_lens, scale, causal, out,
                      lse, need_lse, rope)


def _fwd_paged(q, k_cache, v_cache, scales, block_table, ctx_lens, q_lens, scale, causal, out, lse, need_lse, rope):
    import torch
    dt = _dtype_code(q)
    _check(q.is_cuda and q.dim() == 4 and q.is_contiguous(), "q must be a contiguous 4-D GPU tensor")
    B, Hq, Tq, D = q.shape
    NB, Hkv, bs = _check_paged((k_cache, v_cache), q.dtype if scales is None else torch.uint8, D)
    _check(block_table.dim() == 2 and block_table.shape[0] == B, "block_table must be [B, max_blocks]")
    _check_i32(block_table, block_table.numel(), "block_table")
    _check_i32(ctx_lens, B, "ctx_lens")
    _check_i32(q_lens, B, "q_lens", optional=True)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _check(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous() and out.is_cuda, "bad out")
    if need_lse and lse is None:
        lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse.shape == (B, Hq, Tq) and lse.dtype == torch.float32 and lse.is_contiguous(), "bad lse")
    tail = (_ptr(block_table), _ptr(ctx_lens), _ptr(q_lens), _ptr(out), _ptr(lse), B, Hq, Hkv, Tq, D, bs,
            block_table.shape[1], NB, ctypes.c_float(scale), int(bool(causal)), dt, _stream(q.device))
    with _on(q, k_cache, v_cache, block_table, ctx_lens, q_lens, out, lse, rope):
        if scales is not None:
            max_pos = _check_rope(rope, D) if rope is not None else 0
            st = lib().attn_fwd_paged_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.c_float(scales[0]),
                                          ctypes.c_float(scales[1]), _ptr(rope), max_pos, *tail)
        elif rope is not None:
            st = lib().attn_fwd_paged_rope(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(rope), _check_rope(rope, D), *tail)
        else:
            st = lib().attn_fwd_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), *tail)
    _raise(st)
    return out, lse


def attn_cache_append(k_new, v_new, k_cache, v_cache, block_table, start_pos, new_lens=None, rope=None):
    """Write k_new/v_new [B,Hkv,Tnew,D] into the paged caches in place: token i < new_lens[b]
    becomes position start_pos[b] + i of sequence b (new_lens None: all Tnew tokens)."""
    dt = _dtype_code(k_new)
    _check(k_new.is_cuda and k_new.dim() == 4 and v_new.shape == k_new.shape and v_new.dtype == k_new.dtype
           and k_new.is_contiguous() and v_new.is_contiguous() and v_new.is_cuda,
           "k_new / v_new must be contiguous GPU tensors of one shape [B,Hkv,Tnew,D]")
    B, Hkv, Tnew, D = k_new.shape
    NB, Hc, bs = _check_paged((k_cache, v_cache), k_new.dtype, D)
    _check(Hc == Hkv, "kv head count mismatch")
    _check(block_table.dim() == 2 and block_table.shape[0] == B, "block_table must be [B, max_blocks]")
    _check_i32(block_table, block_table.numel(), "block_table")
    _check_i32(start_pos, B, "start_pos")
    _check_i32(new_lens, B, "new_lens", optional=True)
    tail = (_ptr(block_table), _ptr(start_pos), _ptr(new_lens), B, Hkv, Tnew, D, bs, block_table.shape[1], NB, dt,
            _stream(k_new.device))
    with _on(k_new, v_new, k_cache, v_cache, block_table, start_pos, new_lens, rope):
        if rope is not None:
            st = lib().attn_cache_append_rope(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(rope),
                                              _check_rope(rope, D), *tail)
        else:
            st = lib().attn_cache_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), *tail)
    _raise(st)


def attn_cache_append_fp8(k_new, v_new, k_cache, v_cache, k_scale: float, v_scale: float, block_table, start_pos,
                          new_lens=None):
    """Quantize k_new/v_new [B,Hkv,Tnew,D] (bf16 / fp16) to E4M3 codes of x / scale and write them into the
    uint8 caches [num_blocks,Hkv,16,D] in place (token i < new_lens[b] -> position start_pos[b] + i)."""
    import torch
    dt = _dtype_code(k_new)
    _check(k_new.is_cuda and k_new.dim() == 4 and v_new.shape == k_new.shape and v_new.dtype == k_new.dtype
           and k_new.is_contiguous() and v_new.is_contiguous() and v_new.is_cuda,
           "k_new / v_new must be contiguous GPU tensors of one shape [B,Hkv,Tnew,D]")
    B, Hkv, Tnew, D = k_new.shape
    NB, Hc, bs = _check_paged((k_cache, v_cache), torch.uint8, D)
    _check(Hc == Hkv, "kv head count mismatch")
    _check(block_table.dim() == 2 and block_table.shape[0] == B, "block_table must be [B, max_blocks]")
    _check_i32(block_table, block_table.numel(), "block_table")
    _check_i32(start_pos, B, "start_pos")
    _check_i32(new_lens, B, "new_lens", optional=True)
    with _on(k_new, v_new, k_cache, v_cache, block_table, start_pos, new_lens):
        st = lib().attn_cache_append_fp8(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), ctypes.c_float(k_scale),
                                         ctypes.c_float(v_scale), _ptr(block_table), _ptr(start_pos), _ptr(new_lens), B,
                                         Hkv, Tnew, D, bs, block_table.shape[1], NB, dt, _stream(k_new.device))
    _raise(st)


def attn_gemm_splitk(x, w, out=None, config=None):
    """Linear-layer product y = x w^T (no bias): x [M, K], w [N, K] (bf16 or fp16, contiguous, on the GPU),
    K % 8 == 0. config: None for the tuned/default configuration, or (rows, waves, unroll).
    Returns y [M, N] like x."""
    import torch
    dt = _dtype_code(x)
    _check(x.dim() == 2 and w.dim() == 2 and x.shape[1] == w.shape[1], "x [M, K] and w [N, K] required")
    _check(w.dtype == x.dtype, "x and w must share a dtype")
    for t, n in ((x, "x"), (w, "w")):
        _check(t.is_cuda and t.is_contiguous(), f"{n} must be a contiguous GPU tensor")
    M, K = x.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check(out.shape == (M, N) and out.dtype == x.dtype and out.is_contiguous(), "out must be [M, N] like x")
    with _on(x, w, out):
        if config is None:
            st = lib().attn_gemm_splitk(_ptr(x), _ptr(w), _ptr(out), M, N, K, dt, _stream(x.device))
        else:
            rows, waves, unroll = config
            st = lib().attn_gemm_splitk_cfg(_ptr(x), _ptr(w), _ptr(out), M, N, K, dt, rows, waves, unroll,
                                            _stream(x.device))
    _raise(st)
    return out
