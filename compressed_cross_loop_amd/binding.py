"""Thin Python binding of liblla.so (C ABI in include/lla.h).

Argument marshalling only: torch tensors are passed as device pointers and
the current torch stream as the HIP stream.  Every step of the decode path
runs in the library's HIP kernels; if the library is missing this module
raises at import time rather than falling back to anything else.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblla.so")

LLA_OK = 0
LLA_ERR_INVALID_ARGUMENT = 1
LLA_ERR_UNSUPPORTED = 2
LLA_ERR_WORKSPACE_TOO_SMALL = 3
LLA_ERR_HIP = 4
LLA_F32 = 0
LLA_BF16 = 1
LLA_FLAG_GENERIC = 1
LLA_FLAG_FUSED = 2     # absorbed / HLA reads: one fused launch per call (small batch x context)

_DTYPES = {torch.float32: LLA_F32, torch.bfloat16: LLA_BF16}
_TORCH = {LLA_F32: torch.float32, LLA_BF16: torch.bfloat16}


class LlaSetDesc(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("groups", ctypes.c_int32), ("r_k", ctypes.c_int32), ("r_v", ctypes.c_int32),
                ("loop_first", ctypes.c_int32), ("loop_last", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("rope_baked", ctypes.c_int32),
                ("rope_base", ctypes.c_float), ("dtype", ctypes.c_int32), ("latent_fp8", ctypes.c_int32)]


class LlaStore(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("max_pages_per_seq", ctypes.c_int32)]


class LlaDecodeArgs(ctypes.Structure):
    _fields_ = [("loop", ctypes.c_int32), ("window", ctypes.c_int32),
                ("max_pos_hint", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("pos", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("k_cur", ctypes.c_void_p), ("v_cur", ctypes.c_void_p),
                ("ring_k", ctypes.c_void_p), ("ring_v", ctypes.c_void_p),
                ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("scan_events", ctypes.c_void_p)]


class LlaKvDesc(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("rope_base", ctypes.c_float), ("dtype", ctypes.c_int32)]


class LlaKvCache(ctypes.Structure):
    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("max_pages_per_seq", ctypes.c_int32)]


class LlaFullDecodeArgs(ctypes.Structure):
    _fields_ = [("max_pos_hint", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("pos", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("k_cur", ctypes.c_void_p), ("v_cur", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("scan_events", ctypes.c_void_p)]


class LlaParallelArgs(ctypes.Structure):
    _fields_ = [("loop", ctypes.c_int32), ("window", ctypes.c_int32), ("n_max", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("n_tok", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("A", ctypes.c_void_p), ("B", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("attn_events", ctypes.c_void_p)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run python3 compressed_cross_loop_amd/build.py first")
lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.POINTER
lib.lla_write_latents.restype = ctypes.c_int
lib.lla_write_latents.argtypes = [_P(LlaSetDesc), _P(LlaStore), ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
lib.lla_write_workspace_bytes.restype = ctypes.c_size_t
lib.lla_write_workspace_bytes.argtypes = [_P(LlaSetDesc), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
for _name in ("lla_decode_reconstruct", "lla_decode_absorbed", "hla_decode_windowed"):
    _f = getattr(lib, _name)
    _f.restype = ctypes.c_int
    _f.argtypes = [_P(LlaSetDesc), _P(LlaStore), ctypes.c_int32, _P(LlaDecodeArgs), ctypes.c_void_p]
lib.lla_decode_workspace_bytes.restype = ctypes.c_size_t
lib.lla_decode_workspace_bytes.argtypes = [_P(LlaSetDesc), ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32]
lib.lla_decode_plan_splits.restype = ctypes.c_int32
lib.lla_decode_plan_splits.argtypes = [_P(LlaSetDesc), ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
lib.lla_decode_full_cache.restype = ctypes.c_int
lib.lla_decode_full_cache.argtypes = [_P(LlaKvDesc), _P(LlaKvCache), ctypes.c_int32, _P(LlaFullDecodeArgs),
                                      ctypes.c_void_p]
lib.lla_full_decode_workspace_bytes.restype = ctypes.c_size_t
lib.lla_full_decode_workspace_bytes.argtypes = [_P(LlaKvDesc), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
lib.lla_full_decode_plan_splits.restype = ctypes.c_int32
lib.lla_full_decode_plan_splits.argtypes = [_P(LlaKvDesc), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
lib.hla_attention_parallel.restype = ctypes.c_int
lib.hla_attention_parallel.argtypes = [_P(LlaSetDesc), _P(LlaStore), ctypes.c_int32, _P(LlaParallelArgs),
                                       ctypes.c_void_p]
lib.lla_parallel_workspace_bytes.restype = ctypes.c_size_t
lib.lla_parallel_workspace_bytes.argtypes = [_P(LlaSetDesc), ctypes.c_int32, ctypes.c_int32]
lib.lla_decode_scan_kernel.restype = ctypes.c_char_p
lib.lla_decode_scan_kernel.argtypes = [_P(LlaSetDesc), ctypes.c_int32, ctypes.c_int32]
lib.hla_decode_windowed_noalloc.restype = ctypes.c_int
lib.hla_decode_windowed_noalloc.argtypes = [_P(LlaSetDesc), _P(LlaStore), ctypes.c_int32, _P(LlaDecodeArgs),
                                            ctypes.c_void_p]
lib.lla_decode_scan_kernel_for_store.restype = ctypes.c_char_p
lib.lla_decode_scan_kernel_for_store.argtypes = [_P(LlaSetDesc), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_int32]
lib.lla_check_indices.restype = ctypes.c_int
lib.lla_check_indices.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int32]
lib.lla_bytes_per_token.restype = ctypes.c_size_t
lib.lla_bytes_per_token.argtypes = [_P(LlaSetDesc)]
lib.lla_status_string.restype = ctypes.c_char_p
lib.lla_status_string.argtypes = [ctypes.c_int]
lib.lla_abi_version.restype = ctypes.c_int32
lib.lla_abi_version.argtypes = []

ABI_VERSION = 5   # include/lla.h LLA_ABI_VERSION this binding marshals for
if lib.lla_abi_version() != ABI_VERSION:
    raise ImportError(f"{LIB_PATH} has ABI version {lib.lla_abi_version()}, the binding expects {ABI_VERSION}: "
                      "rebuild it (python3 compressed_cross_loop_amd/build.py)")


class LlaError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(f"lla status {status}: {lib.lla_status_string(status).decode()}")


def _check(status):
    if status != LLA_OK:
        raise LlaError(status)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to liblla must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def set_desc(*, n_heads, head_dim, groups, r_k, r_v, loop_first, loop_last, page_size=64,
             rope_baked=0, rope_base=0.0, dtype=LLA_BF16, latent_fp8=0):
    if isinstance(dtype, torch.dtype):
        dtype = _DTYPES[dtype]
    return LlaSetDesc(n_heads, head_dim, groups, r_k, r_v, loop_first, loop_last, page_size,
                      rope_baked, rope_base, dtype, latent_fp8)


def store_bytes(desc, n_pages):
    """Bytes of a latent store of n_pages pages for this set."""
    G, P, R = desc.groups, desc.page_size, desc.r_k + desc.r_v
    if desc.latent_fp8:
        return n_pages * G * (P // 16) * (16 * R + 128)
    return n_pages * G * P * R * (2 if desc.dtype == LLA_BF16 else 4)


def store(pages, block_table, max_pages_per_seq=None):
    if max_pages_per_seq is None:
        max_pages_per_seq = block_table.shape[-1]
    st = LlaStore(_ptr(pages), _ptr(block_table), int(max_pages_per_seq))
    st._keep = (pages, block_table)   # the struct holds raw pointers: keep the tensors alive with it
    return st


def lla_abi_version():
    return lib.lla_abi_version()


def lla_status_string(status):
    return lib.lla_status_string(status).decode()


def lla_bytes_per_token(desc):
    return lib.lla_bytes_per_token(ctypes.byref(desc))


def lla_write_workspace_bytes(desc, batch, n_tok, d_in):
    return lib.lla_write_workspace_bytes(ctypes.byref(desc), batch, n_tok, d_in)


def lla_decode_workspace_bytes(desc, batch, max_pos, window, splits=0):
    return lib.lla_decode_workspace_bytes(ctypes.byref(desc), batch, max_pos, window, splits)


def lla_decode_plan_splits(desc, batch, max_pos, window, splits=0, entry=1):
    return lib.lla_decode_plan_splits(ctypes.byref(desc), batch, max_pos, window, splits, entry)


def lla_check_indices(pos, block_table, n_pages, page_size):
    """Host check of positions and block-table entries (CPU int32 tensors or
    arrays); returns the status (LLA_OK or LLA_ERR_INVALID_ARGUMENT)."""
    import numpy as _np
    pos = _np.ascontiguousarray(_np.asarray(pos, dtype=_np.int32))
    bt = _np.ascontiguousarray(_np.asarray(block_table, dtype=_np.int32))
    return lib.lla_check_indices(pos.ctypes.data, int(pos.shape[0]), bt.ctypes.data, int(bt.shape[1]),
                                 int(page_size), int(n_pages))


def lla_decode_scan_kernel(desc, entry, flags=0):
    """Latent-scan kernel family a decode call launches (entry 0 reconstruct,
    1 absorbed, 2 HLA windowed); None on invalid arguments."""
    r = lib.lla_decode_scan_kernel(ctypes.byref(desc), entry, flags)
    return None if r is None else r.decode()


def lla_decode_scan_kernel_for_store(desc, entry, max_pos_hint, max_pages_per_seq, flags=0):
    """The scan kernel family a decode call launches on a store whose block
    table has max_pages_per_seq columns; None on invalid arguments."""
    r = lib.lla_decode_scan_kernel_for_store(ctypes.byref(desc), entry, flags, max_pos_hint, max_pages_per_seq)
    return None if r is None else r.decode()


def lla_write_latents(desc, st, *, pos, x, enc, workspace=None, stream=None):
    """pos [B, n_tok] int32, x [B, n_tok, n_loops, G, d_in], enc [n_loops, G, r_k+r_v, d_in]."""
    batch, n_tok = int(pos.shape[0]), int(pos.shape[1])
    d_in = int(x.shape[-1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.lla_write_latents(ctypes.byref(desc), ctypes.byref(st), batch, n_tok, _ptr(pos),
                                 _ptr(x), d_in, _ptr(enc), _ptr(workspace), ws_bytes,
                                 _stream(stream)))


def decode_args(*, loop, window, pos, q, k_cur, v_cur, ring_k, ring_v, A, B, out, workspace,
                max_pos_hint, splits=0, flags=0, scan_events=None):
    """scan_events: optional ctypes array of two hipEvent_t handles."""
    ws_bytes = 0 if workspace is None or isinstance(workspace, int) else \
        workspace.numel() * workspace.element_size()
    ev = ctypes.cast(scan_events, ctypes.c_void_p) if scan_events is not None else None
    args = LlaDecodeArgs(loop, window, int(max_pos_hint), splits, flags, _ptr(pos), _ptr(q),
                         _ptr(k_cur), _ptr(v_cur), _ptr(ring_k), _ptr(ring_v), _ptr(A), _ptr(B),
                         _ptr(out), _ptr(workspace), ws_bytes, ev)
    # the struct holds raw pointers: keep every tensor (temporaries included) alive with it
    args._keep = (pos, q, k_cur, v_cur, ring_k, ring_v, A, B, out, workspace)
    return args


def _decode(fn, desc, st, batch, args, stream):
    _check(fn(ctypes.byref(desc), ctypes.byref(st), batch, ctypes.byref(args), _stream(stream)))


def lla_decode_reconstruct(desc, st, batch, args, stream=None):
    _decode(lib.lla_decode_reconstruct, desc, st, batch, args, stream)


def lla_decode_absorbed(desc, st, batch, args, stream=None):
    _decode(lib.lla_decode_absorbed, desc, st, batch, args, stream)


def hla_decode_windowed(desc, st, batch, args, stream=None):
    _decode(lib.hla_decode_windowed, desc, st, batch, args, stream)


NOALLOC_SCRATCH_BYTES = 32 << 20   # include/lla.h LLA_NOALLOC_SCRATCH_BYTES


def hla_decode_windowed_noalloc(desc, st, batch, args, stream=None):
    """hla_decode_windowed with the library's per-GPU scratch array as the
    workspace: build `args` with workspace=None."""
    _decode(lib.hla_decode_windowed_noalloc, desc, st, batch, args, stream)


# ---------------------------------------------------------------- full cache
def kv_desc(*, n_heads, head_dim, page_size=64, rope_base=0.0, dtype=LLA_BF16):
    if isinstance(dtype, torch.dtype):
        dtype = _DTYPES[dtype]
    return LlaKvDesc(n_heads, head_dim, page_size, rope_base, dtype)


def kv_cache(k_pages, v_pages, block_table, max_pages_per_seq=None):
    if max_pages_per_seq is None:
        max_pages_per_seq = block_table.shape[-1]
    c = LlaKvCache(_ptr(k_pages), _ptr(v_pages), _ptr(block_table), int(max_pages_per_seq))
    c._keep = (k_pages, v_pages, block_table)   # raw pointers: keep the tensors alive with it
    return c


def full_decode_args(*, pos, q, k_cur, v_cur, out, workspace, max_pos_hint, splits=0, flags=0,
                     scan_events=None):
    ws_bytes = 0 if workspace is None or isinstance(workspace, int) else \
        workspace.numel() * workspace.element_size()
    ev = ctypes.cast(scan_events, ctypes.c_void_p) if scan_events is not None else None
    args = LlaFullDecodeArgs(int(max_pos_hint), splits, flags, _ptr(pos), _ptr(q), _ptr(k_cur),
                             _ptr(v_cur), _ptr(out), _ptr(workspace), ws_bytes, ev)
    args._keep = (pos, q, k_cur, v_cur, out, workspace)
    return args


def lla_decode_full_cache(desc, cache, batch, args, stream=None):
    _check(lib.lla_decode_full_cache(ctypes.byref(desc), ctypes.byref(cache), batch, ctypes.byref(args),
                                     _stream(stream)))


def lla_full_decode_workspace_bytes(desc, batch, max_pos, splits=0):
    return lib.lla_full_decode_workspace_bytes(ctypes.byref(desc), batch, max_pos, splits)


def lla_full_decode_plan_splits(desc, batch, max_pos, splits=0):
    return lib.lla_full_decode_plan_splits(ctypes.byref(desc), batch, max_pos, splits)


def parallel_args(*, loop, window, n_tok, q, k, v, A, B, out, workspace, flags=0, attn_events=None):
    """n_tok [batch] int32; q, k, v, out [batch, n_max, H, d_h]; A [H, d_h, r_k]; B = B_t^T [H, d_h, r_v];
    attn_events: optional ctypes array of two hipEvent_t handles."""
    ws_bytes = 0 if workspace is None or isinstance(workspace, int) else \
        workspace.numel() * workspace.element_size()
    ev = ctypes.cast(attn_events, ctypes.c_void_p) if attn_events is not None else None
    args = LlaParallelArgs(loop, window, int(q.shape[1]), flags, _ptr(n_tok), _ptr(q), _ptr(k), _ptr(v), _ptr(A),
                           _ptr(B), _ptr(out), _ptr(workspace), ws_bytes, ev)
    args._keep = (n_tok, q, k, v, A, B, out, workspace)
    return args


def hla_attention_parallel(desc, st, batch, args, stream=None):
    _check(lib.hla_attention_parallel(ctypes.byref(desc), ctypes.byref(st), batch, ctypes.byref(args),
                                      _stream(stream)))


def lla_parallel_workspace_bytes(desc, batch, n_max):
    return lib.lla_parallel_workspace_bytes(ctypes.byref(desc), batch, n_max)


def torch_dtype(desc):
    return _TORCH[desc.dtype]
