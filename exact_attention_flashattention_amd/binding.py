"""Thin ctypes binding over libattn.so (argument marshalling only).

Each function has the name of the C entry point it calls and takes torch
tensors that already live on the GPU; every step of the computation runs in
the library's HIP kernels. If the shared library is missing the first call
raises ``AttnLibraryMissing``: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("ATTN_LIB", os.path.join(HERE, "libattn.so"))

ATTN_OK = 0
ATTN_F32, ATTN_BF16 = 0, 1
ATTN_BNHD, ATTN_BHND = 0, 1
LAYOUTS = {"BNHD": ATTN_BNHD, "BHND": ATTN_BHND}

class AttnVariant(ctypes.Structure):
    """struct attn_variant: window (0 = none), n_sink initial positions kept
    visible with a window, sinks = device fp32 [Hq] sink logits or NULL."""
    _fields_ = [("window", ctypes.c_int), ("n_sink", ctypes.c_int), ("sinks", ctypes.c_void_p)]


# (name, restype, argtypes) for every symbol declared in include/attn.h
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_var = ctypes.POINTER(AttnVariant)
SIGNATURES = [
    ("attn_prefill", _i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]),
    ("attn_prefill_ex", _i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _i, _var, _vp]),
    ("attn_decode_num_splits", _i, [_i, _i, _i, _i]),
    ("attn_decode_workspace_size", _sz, [_i, _i, _i, _i, _i, _i]),
    ("attn_decode", _i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp, _sz,
                         _vp]),
    ("attn_decode_ex", _i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _var, _vp,
                            _sz, _vp]),
    ("attn_decode_noalloc", _i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    ("attn_kv_append", _i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp]),
    ("attn_prefill_paged", _i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                                _i, _i, _f, _var, _vp]),
    ("attn_backward_workspace_size", _sz, [_i, _i, _i]),
    ("attn_backward", _i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp,
                           _sz, _vp]),
    ("attn_decode_mla_num_splits", _i, [_i, _i, _i, _i]),
    ("attn_decode_mla_workspace_size", _sz, [_i, _i, _i, _i]),
    ("attn_decode_mla", _i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    ("attn_gather_pages", _i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp]),
    ("attn_status_string", ctypes.c_char_p, [_i]),
    ("attn_version", _i, []),
]


class AttnLibraryMissing(RuntimeError):
    pass


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libattn.so once and declare every exported signature."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise AttnLibraryMissing(
                f"{LIB_PATH} is not built; run `python -m exact_attention_flashattention_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().attn_status_string(status).decode()


attn_status_string = status_string


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return getattr(stream, "cuda_stream", stream)


def _scratch(nbytes: int, device, stream):
    """fp32 scratch for one call, allocated on the stream the call's kernels
    run on. The caching allocator keys a freed block by the stream it was
    allocated on, so when the tensor is dropped right after the enqueue its
    memory is only handed to later work on that same stream, which runs after
    these kernels (a block allocated on another stream could be reused there
    while the kernels still write it)."""
    import torch
    if stream is None:
        ts = torch.cuda.current_stream(device)
    elif isinstance(stream, torch.cuda.Stream):
        ts = stream
    else:
        ts = torch.cuda.ExternalStream(int(stream), device=device)
    with torch.cuda.stream(ts):
        return torch.empty(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device=device)


def _check(status: int, where: str) -> None:
    if status != ATTN_OK:
        raise AttnError(status, where)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _variant(window: int, n_sink: int, sinks, Hq: int):
    """A pointer to an attn_variant, or None when no variant is asked for.
    The struct is returned with the pointer so it outlives the call."""
    import torch
    if not window and not n_sink and sinks is None:
        return None, None
    ptr = None
    if sinks is not None:
        if sinks.dtype != torch.float32 or tuple(sinks.shape) != (Hq,):
            raise ValueError("sinks must be float32 [Hq]")
        ptr = _dev(sinks, "sinks")
    v = AttnVariant(int(window), int(n_sink), ptr)
    return ctypes.pointer(v), v


def attn_prefill_ex(q, k, v, o=None, *, causal: bool = True, scale: Optional[float] = None,
                    layout: str = "BNHD", lse=None, window: int = 0, n_sink: int = 0, sinks=None,
                    stream=None):
    """Causal (or full) GQA attention. q [B,N,Hq,d] / [B,Hq,N,d] and k, v with
    Hkv heads, bf16 or fp32 (all alike). window / n_sink / sinks select the
    attn_variant options (bf16 only). Returns o (allocated if not given)."""
    import torch
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {list(LAYOUTS)}")
    if q.dim() != 4 or k.shape != v.shape or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D and k, v alike")
    if layout == "BNHD":
        B, N, Hq, d = q.shape
        Hkv = k.shape[2]
        ok = k.shape[0] == B and k.shape[1] == N and k.shape[3] == d
    else:
        B, Hq, N, d = q.shape
        Hkv = k.shape[1]
        ok = k.shape[0] == B and k.shape[2] == N and k.shape[3] == d
    if not ok:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)}")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share a dtype")
    dtype = {torch.bfloat16: ATTN_BF16, torch.float32: ATTN_F32}.get(q.dtype)
    if dtype is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if o is None:
        o = torch.empty_like(q)
    elif o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("o must match q")
    if scale is None:
        scale = d ** -0.5
    lse_ptr = None
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, N):
            raise ValueError("lse must be float32 [B, Hq, N]")
        lse_ptr = _dev(lse, "lse")
    var, _keep = _variant(window, n_sink, sinks, Hq)
    st = lib().attn_prefill_ex(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), lse_ptr,
                               B, N, Hq, Hkv, d, float(scale), int(bool(causal)), dtype,
                               LAYOUTS[layout], var, _stream(stream))
    _check(st, "attn_prefill_ex")
    return o


def attn_prefill(q, k, v, o=None, *, causal: bool = True, scale: Optional[float] = None, stream=None):
    """bf16 [B, N, H, d] prefill (the attn_prefill entry point)."""
    import torch
    if q.dtype != torch.bfloat16 or q.dim() != 4:
        raise ValueError("attn_prefill takes bf16 [B, N, H, d] tensors")
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, N, Hkv, d) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k, v must be bf16 [B, N, Hkv, d]")
    if o is None:
        o = torch.empty_like(q)
    st = lib().attn_prefill(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), B, N, Hq, Hkv, d,
                            float(d ** -0.5 if scale is None else scale), int(bool(causal)), _stream(stream))
    _check(st, "attn_prefill")
    return o


def attn_decode_num_splits(B: int, Hkv: int, max_pages_per_seq: int, num_splits: int = 0) -> int:
    s = lib().attn_decode_num_splits(B, Hkv, max_pages_per_seq, num_splits)
    _check(min(s, 0), "attn_decode_num_splits")
    return s


def attn_decode_workspace_size(B: int, Hq: int, Hkv: int, d: int, max_pages_per_seq: int,
                               num_splits: int = 0) -> int:
    return int(lib().attn_decode_workspace_size(B, Hq, Hkv, d, max_pages_per_seq, num_splits))


def attn_decode(q, k_pages, v_pages, block_table, seq_lens, o=None, *, scale: Optional[float] = None,
                num_splits: int = 0, workspace=None, stream=None):
    """Paged decode. q [B,Hq,d] bf16; pools [num_pages,16,Hkv,d] bf16;
    block_table int32 [B,max_pages]; seq_lens int32 [B]. Returns o [B,Hq,d]."""
    return _decode(q, k_pages, v_pages, block_table, seq_lens, o, scale, num_splits, workspace,
                   stream, None)


def attn_decode_ex(q, k_pages, v_pages, block_table, seq_lens, o=None, *, scale: Optional[float] = None,
                   num_splits: int = 0, window: int = 0, n_sink: int = 0, sinks=None, workspace=None,
                   stream=None):
    """attn_decode with the attn_variant options (window, n_sink, sinks)."""
    return _decode(q, k_pages, v_pages, block_table, seq_lens, o, scale, num_splits, workspace,
                   stream, (window, n_sink, sinks))


def _decode(q, k_pages, v_pages, block_table, seq_lens, o, scale, num_splits, workspace, stream, variant):
    import torch
    if q.dtype != torch.bfloat16 or k_pages.dtype != torch.bfloat16 or v_pages.dtype != torch.bfloat16:
        raise ValueError("decode takes bf16 q and pools")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    B, Hq, d = q.shape
    num_pages, page_size, Hkv, d2 = k_pages.shape
    if d2 != d or v_pages.shape != k_pages.shape:
        raise ValueError("pool shape mismatch")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    mpps = block_table.shape[1]
    if o is None:
        o = torch.empty_like(q)
    need = attn_decode_workspace_size(B, Hq, Hkv, d, mpps, num_splits)
    if workspace is None:
        workspace = _scratch(need, q.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    args = (_dev(q, "q"), _dev(k_pages, "k_pages"), _dev(v_pages, "v_pages"),
            _dev(block_table, "block_table"), _dev(seq_lens, "seq_lens"), _dev(o, "o"),
            B, Hq, Hkv, d, page_size, mpps, num_pages, float(d ** -0.5 if scale is None else scale),
            num_splits, ATTN_BF16)
    tail = (_dev(workspace, "workspace"), ws_bytes, _stream(stream))
    if variant is None:
        st = lib().attn_decode(*args, *tail)
        _check(st, "attn_decode")
    else:
        var, _keep = _variant(*variant, Hq)
        st = lib().attn_decode_ex(*args, var, *tail)
        _check(st, "attn_decode_ex")
    return o


ATTN_NOALLOC_SCRATCH_BYTES = 16 << 20


def attn_decode_noalloc(q, k_pages, v_pages, block_table, seq_lens, o, *, scale: Optional[float] = None,
                        num_splits: int = 0, stream=None):
    """attn_decode whose split partials go to the library's fixed per-GPU
    scratch (no workspace, nothing allocated by the call); o [B, Hq, d] bf16
    must be passed. Calls that overlap in time on one GPU must not be issued."""
    import torch
    if q.dtype != torch.bfloat16 or k_pages.dtype != torch.bfloat16 or v_pages.dtype != torch.bfloat16:
        raise ValueError("decode takes bf16 q and pools")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    B, Hq, d = q.shape
    num_pages, page_size, Hkv, d2 = k_pages.shape
    if d2 != d or v_pages.shape != k_pages.shape:
        raise ValueError("pool shape mismatch")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    if o is None or o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("o must be given, bf16 [B, Hq, d]")
    st = lib().attn_decode_noalloc(_dev(q, "q"), _dev(k_pages, "k_pages"), _dev(v_pages, "v_pages"),
                                   _dev(block_table, "block_table"), _dev(seq_lens, "seq_lens"), _dev(o, "o"),
                                   B, Hq, Hkv, d, page_size, block_table.shape[1], num_pages,
                                   float(d ** -0.5 if scale is None else scale), num_splits, ATTN_BF16,
                                   _stream(stream))
    _check(st, "attn_decode_noalloc")
    return o


def _check_pool(k_pages, v_pages, block_table, B):
    import torch
    if k_pages.dtype != torch.bfloat16 or v_pages.shape != k_pages.shape or v_pages.dtype != k_pages.dtype:
        raise ValueError("k_pages and v_pages must be bf16 [num_pages, 16, Hkv, d] alike")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages]")


def attn_kv_append(k_new, v_new, k_pages, v_pages, block_table, cu_new, start_pos, *,
                   max_new: Optional[int] = None, stream=None):
    """Write new tokens k_new/v_new [T, Hkv, d] (sequence b owns rows
    cu_new[b] .. cu_new[b+1]-1, starting at cache position start_pos[b]) into
    the bf16 page pools, in place. max_new defaults to the longest chunk
    (read from cu_new on the host)."""
    import torch
    B = start_pos.shape[0]
    _check_pool(k_pages, v_pages, block_table, B)
    if cu_new.dtype != torch.int32 or start_pos.dtype != torch.int32 or cu_new.shape != (B + 1,):
        raise ValueError("cu_new must be int32 [B + 1] and start_pos int32 [B]")
    T, Hkv, d = k_new.shape
    if v_new.shape != k_new.shape or k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise ValueError("k_new, v_new must be bf16 [T, Hkv, d] alike")
    num_pages, page_size, Hkv2, d2 = k_pages.shape
    if (Hkv2, d2) != (Hkv, d):
        raise ValueError("pool and new rows disagree on Hkv or d")
    if max_new is None:
        max_new = int((cu_new[1:] - cu_new[:-1]).max().item()) if B else 0
    st = lib().attn_kv_append(_dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_pages, "k_pages"),
                              _dev(v_pages, "v_pages"), _dev(block_table, "block_table"),
                              _dev(cu_new, "cu_new"), _dev(start_pos, "start_pos"), B, Hkv, d,
                              page_size, block_table.shape[1], num_pages, T, max_new, _stream(stream))
    _check(st, "attn_kv_append")


def attn_prefill_paged(q, k_pages, v_pages, block_table, cu_q, seq_lens, o=None, *,
                       max_q_len: Optional[int] = None, scale: Optional[float] = None, lse=None,
                       window: int = 0, n_sink: int = 0, sinks=None, stream=None):
    """Chunk queries q [T, Hq, d] bf16 (sequence b owns rows cu_q[b] ..
    cu_q[b+1]-1, at positions seq_lens[b] - c_b ..) against the paged cache.
    Returns o [T, Hq, d]; lse, if given, is float32 [Hq, T]. max_q_len
    defaults to the longest chunk (read from cu_q on the host)."""
    import torch
    B = seq_lens.shape[0]
    _check_pool(k_pages, v_pages, block_table, B)
    if cu_q.dtype != torch.int32 or seq_lens.dtype != torch.int32 or cu_q.shape != (B + 1,):
        raise ValueError("cu_q must be int32 [B + 1] and seq_lens int32 [B]")
    if q.dtype != torch.bfloat16 or q.dim() != 3:
        raise ValueError("q must be bf16 [T, Hq, d]")
    T, Hq, d = q.shape
    num_pages, page_size, Hkv, d2 = k_pages.shape
    if d2 != d:
        raise ValueError("pool and q disagree on d")
    if o is None:
        o = torch.empty_like(q)
    elif o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("o must match q")
    if max_q_len is None:
        max_q_len = int((cu_q[1:] - cu_q[:-1]).max().item()) if B else 0
    lse_ptr = None
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (Hq, T):
            raise ValueError("lse must be float32 [Hq, T]")
        lse_ptr = _dev(lse, "lse")
    var, _keep = _variant(window, n_sink, sinks, Hq)
    st = lib().attn_prefill_paged(_dev(q, "q"), _dev(k_pages, "k_pages"), _dev(v_pages, "v_pages"),
                                  _dev(block_table, "block_table"), _dev(cu_q, "cu_q"),
                                  _dev(seq_lens, "seq_lens"), _dev(o, "o"), lse_ptr, B, Hq, Hkv, d,
                                  page_size, block_table.shape[1], num_pages, T, max_q_len,
                                  float(d ** -0.5 if scale is None else scale), var, _stream(stream))
    _check(st, "attn_prefill_paged")
    return o


def attn_backward_workspace_size(B: int, N: int, Hq: int) -> int:
    return int(lib().attn_backward_workspace_size(B, N, Hq))


def attn_backward(q, k, v, o, dout, lse, dq=None, dk=None, dv=None, *, causal: bool = True,
                  scale: Optional[float] = None, layout: str = "BNHD", workspace=None, stream=None):
    """Gradients (dq, dk, dv) of the bf16 prefill given dout; o and lse
    ([B, Hq, N] fp32) are the forward's outputs. Returns (dq, dk, dv)."""
    import torch
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {list(LAYOUTS)}")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        if t.dtype != torch.bfloat16 or t.dim() != 4:
            raise ValueError(f"{n} must be a bf16 4-D tensor")
    if o.shape != q.shape or dout.shape != q.shape or v.shape != k.shape:
        raise ValueError("o and dout must match q, v must match k")
    if layout == "BNHD":
        B, N, Hq, d = q.shape
        Hkv = k.shape[2]
    else:
        B, Hq, N, d = q.shape
        Hkv = k.shape[1]
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("lse must be float32 [B, Hq, N]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = attn_backward_workspace_size(B, N, Hq)
    if workspace is None:
        workspace = _scratch(need, q.device, stream)
    st = lib().attn_backward(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dev(dout, "dout"),
                             _dev(lse, "lse"), _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"), B, N, Hq,
                             Hkv, d, float(d ** -0.5 if scale is None else scale), int(bool(causal)),
                             LAYOUTS[layout], _dev(workspace, "workspace"),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "attn_backward")
    return dq, dk, dv


def attn_decode_mla_num_splits(B: int, Hq: int, max_pages_per_seq: int, num_splits: int = 0) -> int:
    s = lib().attn_decode_mla_num_splits(B, Hq, max_pages_per_seq, num_splits)
    _check(min(s, 0), "attn_decode_mla_num_splits")
    return s


def attn_decode_mla_workspace_size(B: int, Hq: int, max_pages_per_seq: int, num_splits: int = 0) -> int:
    return int(lib().attn_decode_mla_workspace_size(B, Hq, max_pages_per_seq, num_splits))


def attn_decode_mla(q, kv_pages, block_table, seq_lens, o=None, *, scale: Optional[float] = None,
                    d_c: int = 512, num_splits: int = 0, workspace=None, stream=None):
    """Absorbed-MLA decode. q [B, Hq, 576] bf16; kv_pages [num_pages, 16, 576]
    bf16; returns o [B, Hq, 512]. The default scale is 1/sqrt(128 + 64)."""
    import torch
    if q.dtype != torch.bfloat16 or kv_pages.dtype != torch.bfloat16:
        raise ValueError("q and kv_pages must be bf16")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    B, Hq, dk = q.shape
    num_pages, page_size, dk2 = kv_pages.shape
    if dk2 != dk:
        raise ValueError("q and kv_pages disagree on the row width")
    mpps = block_table.shape[1]
    if o is None:
        o = torch.empty((B, Hq, d_c), dtype=q.dtype, device=q.device)
    need = attn_decode_mla_workspace_size(B, Hq, mpps, num_splits)
    if workspace is None:
        workspace = _scratch(need, q.device, stream)
    st = lib().attn_decode_mla(_dev(q, "q"), _dev(kv_pages, "kv_pages"), _dev(block_table, "block_table"),
                               _dev(seq_lens, "seq_lens"), _dev(o, "o"), B, Hq, d_c, dk - d_c, page_size, mpps,
                               num_pages, float((128 + 64) ** -0.5 if scale is None else scale), num_splits,
                               _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                               _stream(stream))
    _check(st, "attn_decode_mla")
    return o


def attn_gather_pages(pages, block_table, seq_lens, max_len: int, out=None, stream=None):
    """Materialise [B, max_len, Hkv, d] from a page pool through the block table."""
    import torch
    num_pages, page_size, Hkv, d = pages.shape
    B = block_table.shape[0]
    if out is None:
        out = torch.zeros((B, max_len, Hkv, d), dtype=pages.dtype, device=pages.device)
    st = lib().attn_gather_pages(_dev(pages, "pages"), _dev(block_table, "block_table"),
                                 _dev(seq_lens, "seq_lens"), _dev(out, "out"), B, Hkv, d, page_size,
                                 block_table.shape[1], num_pages, max_len, pages.element_size(),
                                 _stream(stream))
    _check(st, "attn_gather_pages")
    return out
