"""Python binding of libpkvattn: causal GQA prefill, contiguous/paged decode, MLA latent decode.

Argument marshalling only. Every function takes torch tensors that already
live on the GPU, checks that they are dense and of one supported dtype, reads
their sizes, and calls the C entry point of the same name in
``libpkvattn.so`` on the current torch stream. All arithmetic runs in the HIP
kernels; there is no CPU path. If the library is missing, every call raises.

The library is loaded after ``torch`` so that it binds to the HIP runtime
torch already loaded (both name ``libamdhip64.so.7``), which makes torch's
stream handles valid arguments.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

__all__ = [
    "PkvaError",
    "library_path",
    "lib",
    "header_symbols",
    "attn_prefill",
    "attn_prefill_varlen",
    "attn_decode_contig",
    "attn_decode_paged",
    "attn_decode_paged_noalloc",
    "attn_decode_contig_ext",
    "attn_decode_paged_ext",
    "Arms",
    "attn_decode_workspace_size",
    "mla_decode_latent",
    "mla_decode_workspace_size",
    "mla_decode_latent_paged",
    "mla_absorb_q",
    "mla_up_proj",
    "kv_append",
    "mla_append_latent",
    "status_string",
    "F32",
    "BF16",
]

F32 = 0
BF16 = 1
_HERE = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_HERE), "include", "pkvattn.h")
_LIB = None


class Arms(ctypes.Structure):
    """``pkva_arms``: the optional arms of one attention layer (see pkvattn.h)."""
    _fields_ = [("window", ctypes.c_int), ("softcap", ctypes.c_float),
                ("alibi_slopes", ctypes.c_void_p), ("sinks", ctypes.c_void_p),
                ("v_head_dim", ctypes.c_int)]


class PkvaError(RuntimeError):
    """A non-zero status from the library; ``.status`` holds the code."""

    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: status {status} ({status_string(status)})")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, "libpkvattn.so")


def lib():
    """The loaded ``libpkvattn.so`` (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        import torch  # noqa: F401  -- bind to torch's HIP runtime first
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m paged_kv_attention_causal_amd.csrc.build`")
        L = ctypes.CDLL(path)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.pkva_status_string.restype = ctypes.c_char_p
        L.pkva_status_string.argtypes = [i32]
        L.pkva_version.restype = ctypes.c_char_p
        L.pkva_version.argtypes = []
        L.attn_prefill.restype = i32
        L.attn_prefill.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                                   vp, i32, i32, i32, i32, vp]
        L.attn_prefill_varlen.restype = i32
        L.attn_prefill_varlen.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, i32, i32,
                                          f32, vp, i32, i32, i32, i32, vp]
        L.attn_decode_workspace_size.restype = sz
        L.attn_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.attn_decode_contig.restype = i32
        L.attn_decode_contig.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, i32, i32, f32,
                                         vp, sz, vp]
        L.attn_decode_paged.restype = i32
        L.attn_decode_paged.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, i32, i32, i32,
                                        vp, i32, f32, vp, sz, vp]
        ap = ctypes.POINTER(Arms)
        L.attn_decode_contig_ext.restype = i32
        L.attn_decode_contig_ext.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, i32, i32,
                                             f32, ap, vp, sz, vp]
        L.attn_decode_paged_ext.restype = i32
        L.attn_decode_paged_ext.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, i32, i32,
                                            i32, vp, i32, f32, ap, vp, sz, vp]
        L.attn_decode_paged_noalloc.restype = i32
        L.attn_decode_paged_noalloc.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, i32,
                                                i32, i32, vp, i32, f32, vp]
        L.mla_decode_latent_paged.restype = i32
        L.mla_decode_latent_paged.argtypes = [i32, vp, vp, vp, i32, i32, i32, i32, vp, i32, i32,
                                              i32, vp, i32, f32, vp, sz, vp]
        L.mla_absorb_q.restype = i32
        L.mla_absorb_q.argtypes = [i32, vp, vp, vp, i32, i32, i32, i32, i32, vp]
        L.mla_up_proj.restype = i32
        L.mla_up_proj.argtypes = [i32, vp, vp, vp, i32, i32, i32, i32, vp]
        L.kv_append.restype = i32
        L.kv_append.argtypes = [i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, i32, i32, i32,
                                i32, vp]
        L.mla_append_latent.restype = i32
        L.mla_append_latent.argtypes = [i32, vp, vp, vp, i32, i32, i32, vp, f32, vp, i32, i32, i32,
                                        i32, vp]
        L.mla_decode_workspace_size.restype = sz
        L.mla_decode_workspace_size.argtypes = [i32, i32, i32, i32]
        L.mla_decode_latent.restype = i32
        L.mla_decode_latent.argtypes = [i32, vp, vp, vp, i32, i32, i32, i32, vp, i32, i32, f32,
                                        vp, sz, vp]
        _LIB = L
    return _LIB


def header_symbols() -> list:
    """Names of the functions ``include/pkvattn.h`` declares."""
    with open(_HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def status_string(status: int) -> str:
    try:
        return lib().pkva_status_string(int(status)).decode()
    except Exception:  # pragma: no cover - the library itself is missing
        return "unknown"


def _check(fn: str, status: int):
    if status != 0:
        raise PkvaError(fn, status)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}: use float32 or bfloat16")


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t) -> int:
    return t.data_ptr()


def _stream(t, stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _i32(t, name):
    import torch
    _dev(t, name)
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return t


def attn_prefill(q, k, v, *, seq_kv: int, position_offset: int, attention_scale: float,
                 block_table=None, block_size: int = 0, out=None, stream=None):
    """Causal GQA prefill; returns ``o`` ``[B, seq_q, H, D]`` (see ``attn_prefill`` in pkvattn.h).

    Contiguous: ``k``/``v`` are ``[B, kv_capacity, Hkv, D]``. Paged: ``k``/``v`` are pools
    ``[num_blocks, block_size, Hkv, D]`` and ``block_table`` is int32 ``[B, max_blocks]``.
    """
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    if k.dtype != q.dtype or v.dtype != q.dtype or k.shape != v.shape:
        raise ValueError("q, k, v must share a dtype and k, v a shape")
    B, seq_q, H, D = q.shape
    Hkv = k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out")
    if block_table is not None:
        _i32(block_table, "block_table")
        nb, bs = k.shape[0], k.shape[1]
        if block_size and block_size != bs:
            raise ValueError("block_size disagrees with the pool shape")
        st = lib().attn_prefill(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hkv, D,
                                seq_q, seq_kv, position_offset, attention_scale,
                                _ptr(block_table), block_table.shape[1], bs, nb, 0,
                                _stream(q, stream))
    else:
        st = lib().attn_prefill(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hkv, D,
                                seq_q, seq_kv, position_offset, attention_scale, None, 0, 0, 0,
                                k.shape[1], _stream(q, stream))
    _check("attn_prefill", st)
    return out


def attn_prefill_varlen(q, k, v, cu_seqlens_q, seq_kv, *, max_seq_q: int, attention_scale: float,
                        block_table=None, out=None, stream=None):
    """Causal GQA prefill of a ragged batch; returns ``o`` ``[total_q, H, D]``.

    ``q`` packs every sequence's chunk ``[total_q, H, D]``; ``cu_seqlens_q`` (int32
    ``[B + 1]``) gives each sequence's first row; ``seq_kv`` (int32 ``[B]``) its keys, the
    chunk being the last of them. Paged: ``k``/``v`` pools ``[num_blocks, block_size, Hkv, D]``
    with ``block_table``; contiguous: ``[B, capacity, Hkv, D]``.
    """
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    _i32(cu_seqlens_q, "cu_seqlens_q")
    _i32(seq_kv, "seq_kv")
    if k.dtype != q.dtype or v.dtype != q.dtype or k.shape != v.shape:
        raise ValueError("q, k, v must share a dtype and k, v a shape")
    total_q, H, D = q.shape
    B = seq_kv.shape[0]
    if cu_seqlens_q.shape[0] != B + 1:
        raise ValueError("cu_seqlens_q must hold batch + 1 entries")
    Hkv = k.shape[2]
    out = torch.empty_like(q) if out is None else _dev(out, "out")
    if block_table is not None:
        _i32(block_table, "block_table")
        st = lib().attn_prefill_varlen(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H,
                                       Hkv, D, _ptr(cu_seqlens_q), _ptr(seq_kv), total_q, max_seq_q,
                                       attention_scale, _ptr(block_table), block_table.shape[1],
                                       k.shape[1], k.shape[0], 0, _stream(q, stream))
    else:
        st = lib().attn_prefill_varlen(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H,
                                       Hkv, D, _ptr(cu_seqlens_q), _ptr(seq_kv), total_q, max_seq_q,
                                       attention_scale, None, 0, 0, 0, k.shape[1],
                                       _stream(q, stream))
    _check("attn_prefill_varlen", st)
    return out


def attn_decode_workspace_size(batch, n_heads, n_kv_heads, head_dim, max_seq_len) -> int:
    return int(lib().attn_decode_workspace_size(batch, n_heads, n_kv_heads, head_dim, max_seq_len))


def _workspace(nbytes, like, workspace):
    import torch
    if workspace is None:
        workspace = torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=like.device)
    _dev(workspace, "workspace")
    return workspace


def attn_decode_contig(q, k_cache, v_cache, seq_lens, *, max_seq_len: int, attention_scale: float,
                       out=None, workspace=None, stream=None):
    """Single-token decode over ``[B, capacity, Hkv, D]`` caches; returns ``o`` ``[B, H, D]``."""
    import torch
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    _i32(seq_lens, "seq_lens")
    B, H, D = q.shape
    Hkv = k_cache.shape[2]
    out = torch.empty_like(q) if out is None else _dev(out, "out")
    nbytes = attn_decode_workspace_size(B, H, Hkv, D, max_seq_len)
    workspace = _workspace(nbytes, q, workspace)
    st = lib().attn_decode_contig(_dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                  B, H, Hkv, D, _ptr(seq_lens), k_cache.shape[1], max_seq_len,
                                  attention_scale, _ptr(workspace), workspace.numel(),
                                  _stream(q, stream))
    _check("attn_decode_contig", st)
    return out


def attn_decode_paged(q, k_pool, v_pool, block_table, seq_lens, *, max_seq_len: int,
                      attention_scale: float, out=None, workspace=None, stream=None):
    """Single-token decode over ``[num_blocks, block_size, Hkv, D]`` pools; returns ``[B, H, D]``."""
    import torch
    for t, n in ((q, "q"), (k_pool, "k_pool"), (v_pool, "v_pool")):
        _dev(t, n)
    _i32(block_table, "block_table")
    _i32(seq_lens, "seq_lens")
    B, H, D = q.shape
    nb, bs, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    out = torch.empty_like(q) if out is None else _dev(out, "out")
    nbytes = attn_decode_workspace_size(B, H, Hkv, D, max_seq_len)
    workspace = _workspace(nbytes, q, workspace)
    st = lib().attn_decode_paged(_dtype_code(q), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(out),
                                 B, H, Hkv, D, _ptr(block_table), block_table.shape[1], bs, nb,
                                 _ptr(seq_lens), max_seq_len, attention_scale, _ptr(workspace),
                                 workspace.numel(), _stream(q, stream))
    _check("attn_decode_paged", st)
    return out


def _arms(q, v, window, softcap, alibi, sinks):
    import torch
    H = q.shape[1]
    for t, n in ((alibi, "alibi"), (sinks, "sinks")):
        if t is not None:
            _dev(t, n)
            if t.dtype != torch.float32 or t.numel() != H:
                raise ValueError(f"{n} must be float32 [n_heads]")
    return Arms(int(window), float(softcap), None if alibi is None else _ptr(alibi),
                None if sinks is None else _ptr(sinks), int(v.shape[-1]))


def attn_decode_contig_ext(q, k_cache, v_cache, seq_lens, *, max_seq_len: int,
                           attention_scale: float, window: int = 0, softcap: float = 0.0,
                           alibi=None, sinks=None, out=None, workspace=None, stream=None):
    """:func:`attn_decode_contig` with a layer's arms; ``v_cache`` rows may be narrower
    than ``k_cache`` rows. Returns ``[B, H, v_head_dim]``."""
    import torch
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    _i32(seq_lens, "seq_lens")
    B, H, D = q.shape
    Hkv, Dv = k_cache.shape[2], v_cache.shape[3]
    arms = _arms(q, v_cache, window, softcap, alibi, sinks)
    if out is None:
        out = torch.empty((B, H, Dv), dtype=q.dtype, device=q.device)
    _dev(out, "out")
    workspace = _workspace(attn_decode_workspace_size(B, H, Hkv, Dv, max_seq_len), q, workspace)
    st = lib().attn_decode_contig_ext(_dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(out), B, H, Hkv, D, _ptr(seq_lens), k_cache.shape[1],
                                      max_seq_len, attention_scale, ctypes.byref(arms),
                                      _ptr(workspace), workspace.numel(), _stream(q, stream))
    _check("attn_decode_contig_ext", st)
    return out


def attn_decode_paged_ext(q, k_pool, v_pool, block_table, seq_lens, *, max_seq_len: int,
                          attention_scale: float, window: int = 0, softcap: float = 0.0,
                          alibi=None, sinks=None, out=None, workspace=None, stream=None):
    """:func:`attn_decode_paged` with a layer's arms. Returns ``[B, H, v_head_dim]``."""
    import torch
    for t, n in ((q, "q"), (k_pool, "k_pool"), (v_pool, "v_pool")):
        _dev(t, n)
    _i32(block_table, "block_table")
    _i32(seq_lens, "seq_lens")
    B, H, D = q.shape
    nb, bs, Hkv, Dv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2], v_pool.shape[3]
    arms = _arms(q, v_pool, window, softcap, alibi, sinks)
    if out is None:
        out = torch.empty((B, H, Dv), dtype=q.dtype, device=q.device)
    _dev(out, "out")
    workspace = _workspace(attn_decode_workspace_size(B, H, Hkv, Dv, max_seq_len), q, workspace)
    st = lib().attn_decode_paged_ext(_dtype_code(q), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                     _ptr(out), B, H, Hkv, D, _ptr(block_table),
                                     block_table.shape[1], bs, nb, _ptr(seq_lens), max_seq_len,
                                     attention_scale, ctypes.byref(arms), _ptr(workspace),
                                     workspace.numel(), _stream(q, stream))
    _check("attn_decode_paged_ext", st)
    return out


def attn_decode_paged_noalloc(q, k_pool, v_pool, block_table, seq_lens, *, max_seq_len: int,
                              attention_scale: float, out, stream=None):
    """:func:`attn_decode_paged` on the library's static scratch: allocates nothing.

    ``out`` must be given (``[B, H, D]``, the dtype of ``q``). Calls that overlap
    on one device share the scratch and must be ordered by the caller.
    """
    for t, n in ((q, "q"), (k_pool, "k_pool"), (v_pool, "v_pool"), (out, "out")):
        _dev(t, n)
    _i32(block_table, "block_table")
    _i32(seq_lens, "seq_lens")
    B, H, D = q.shape
    nb, bs, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    st = lib().attn_decode_paged_noalloc(_dtype_code(q), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                         _ptr(out), B, H, Hkv, D, _ptr(block_table),
                                         block_table.shape[1], bs, nb, _ptr(seq_lens), max_seq_len,
                                         attention_scale, _stream(q, stream))
    _check("attn_decode_paged_noalloc", st)
    return out


def mla_decode_workspace_size(batch, n_heads, kv_lora_rank, max_seq_len) -> int:
    return int(lib().mla_decode_workspace_size(batch, n_heads, kv_lora_rank, max_seq_len))


def mla_decode_latent(q_abs, latent, seq_lens, *, kv_lora_rank: int, max_seq_len: int,
                      attention_scale: float, out=None, workspace=None, stream=None):
    """Absorbed MLA decode; ``q_abs`` ``[B, H, R+P]``, ``latent`` ``[B, cap, R+P]`` -> ``[B, H, R]``."""
    import torch
    _dev(q_abs, "q_abs")
    _dev(latent, "latent")
    _i32(seq_lens, "seq_lens")
    B, H, W = q_abs.shape
    P = W - kv_lora_rank
    if out is None:
        out = torch.empty((B, H, kv_lora_rank), dtype=q_abs.dtype, device=q_abs.device)
    _dev(out, "out")
    nbytes = mla_decode_workspace_size(B, H, kv_lora_rank, max_seq_len)
    workspace = _workspace(nbytes, q_abs, workspace)
    st = lib().mla_decode_latent(_dtype_code(q_abs), _ptr(q_abs), _ptr(latent), _ptr(out), B, H,
                                 kv_lora_rank, P, _ptr(seq_lens), latent.shape[1], max_seq_len,
                                 attention_scale, _ptr(workspace), workspace.numel(),
                                 _stream(q_abs, stream))
    _check("mla_decode_latent", st)
    return out


def mla_decode_latent_paged(q_abs, latent_pool, block_table, seq_lens, *, kv_lora_rank: int,
                            max_seq_len: int, attention_scale: float, out=None, workspace=None,
                            stream=None):
    """:func:`mla_decode_latent` over a pool ``[num_blocks, block_size, R + P]``."""
    import torch
    _dev(q_abs, "q_abs")
    _dev(latent_pool, "latent_pool")
    _i32(block_table, "block_table")
    _i32(seq_lens, "seq_lens")
    B, H, W = q_abs.shape
    P = W - kv_lora_rank
    if out is None:
        out = torch.empty((B, H, kv_lora_rank), dtype=q_abs.dtype, device=q_abs.device)
    _dev(out, "out")
    workspace = _workspace(mla_decode_workspace_size(B, H, kv_lora_rank, max_seq_len), q_abs,
                           workspace)
    st = lib().mla_decode_latent_paged(_dtype_code(q_abs), _ptr(q_abs), _ptr(latent_pool),
                                       _ptr(out), B, H, kv_lora_rank, P, _ptr(block_table),
                                       block_table.shape[1], latent_pool.shape[1],
                                       latent_pool.shape[0], _ptr(seq_lens), max_seq_len,
                                       attention_scale, _ptr(workspace), workspace.numel(),
                                       _stream(q_abs, stream))
    _check("mla_decode_latent_paged", st)
    return out


def mla_absorb_q(q, k_b, *, out=None, stream=None):
    """``q`` ``[B, H, nope + P]``, ``k_b`` ``[H, R, nope]`` -> ``q_abs`` ``[B, H, R + P]``."""
    import torch
    _dev(q, "q")
    _dev(k_b, "k_b")
    B, H, W = q.shape
    _, R, nope = k_b.shape
    if out is None:
        out = torch.empty((B, H, R + W - nope), dtype=q.dtype, device=q.device)
    _dev(out, "out")
    st = lib().mla_absorb_q(_dtype_code(q), _ptr(q), _ptr(k_b), _ptr(out), B, H, nope, W - nope, R,
                            _stream(q, stream))
    _check("mla_absorb_q", st)
    return out


def mla_up_proj(o_lat, v_b, *, out=None, stream=None):
    """``o_lat`` ``[B, H, R]``, ``v_b`` ``[H, v_dim, R]`` -> ``[B, H, v_dim]``."""
    import torch
    _dev(o_lat, "o_lat")
    _dev(v_b, "v_b")
    B, H, R = o_lat.shape
    vd = v_b.shape[1]
    if out is None:
        out = torch.empty((B, H, vd), dtype=o_lat.dtype, device=o_lat.device)
    _dev(out, "out")
    st = lib().mla_up_proj(_dtype_code(o_lat), _ptr(o_lat), _ptr(v_b), _ptr(out), B, H, R, vd,
                           _stream(o_lat, stream))
    _check("mla_up_proj", st)
    return out


def kv_append(k_new, v_new, k_cache, v_cache, positions, *, block_table=None, stream=None):
    """Write ``k_new``/``v_new`` ``[B, n_new, Hkv, D]`` into the cache at ``positions[b] + i``.

    Contiguous: ``k_cache``/``v_cache`` are ``[B, capacity, Hkv, D]``. Paged: they are pools
    ``[num_blocks, block_size, Hkv, D]`` and ``block_table`` is int32 ``[B, max_blocks]``.
    """
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    _i32(positions, "positions")
    if k_new.shape != v_new.shape or k_cache.shape != v_cache.shape:
        raise ValueError("k and v must share shapes")
    if any(t.dtype != k_new.dtype for t in (v_new, k_cache, v_cache)):
        raise ValueError("k and v must share a dtype")
    B, n_new, Hkv, D = k_new.shape
    if tuple(k_cache.shape[2:]) != (Hkv, D):
        raise ValueError("cache rows must be [n_kv_heads, head_dim]")
    if block_table is not None:
        _i32(block_table, "block_table")
        st = lib().kv_append(_dtype_code(k_new), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                             _ptr(v_cache), B, Hkv, D, n_new, _ptr(positions), _ptr(block_table),
                             block_table.shape[1], k_cache.shape[1], k_cache.shape[0], 0,
                             _stream(k_new, stream))
    else:
        st = lib().kv_append(_dtype_code(k_new), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                             _ptr(v_cache), B, Hkv, D, n_new, _ptr(positions), None, 0, 0, 0,
                             k_cache.shape[1], _stream(k_new, stream))
    _check("kv_append", st)


def mla_append_latent(c_new, k_rot_new, latent, positions, *, rope_theta: float,
                      block_table=None, stream=None):
    """Write ``[c_new | rope(k_rot_new)]`` at token ``positions[b]`` of the latent cache.

    ``c_new`` ``[B, R]``, ``k_rot_new`` ``[B, P]`` (unrotated). Contiguous: ``latent`` is
    ``[B, capacity, R + P]``; paged: a pool ``[num_blocks, block_size, R + P]`` with ``block_table``.
    """
    for t, n in ((c_new, "c_new"), (k_rot_new, "k_rot_new"), (latent, "latent")):
        _dev(t, n)
    _i32(positions, "positions")
    if k_rot_new.dtype != c_new.dtype or latent.dtype != c_new.dtype:
        raise ValueError("c_new, k_rot_new and latent must share a dtype")
    B, R = c_new.shape
    P = k_rot_new.shape[1]
    if latent.shape[-1] != R + P:
        raise ValueError("latent rows must be kv_lora_rank + qk_rope_head_dim wide")
    if block_table is not None:
        _i32(block_table, "block_table")
        st = lib().mla_append_latent(_dtype_code(c_new), _ptr(c_new), _ptr(k_rot_new), _ptr(latent),
                                     B, R, P, _ptr(positions), rope_theta, _ptr(block_table),
                                     block_table.shape[1], latent.shape[1], latent.shape[0], 0,
                                     _stream(c_new, stream))
    else:
        st = lib().mla_append_latent(_dtype_code(c_new), _ptr(c_new), _ptr(k_rot_new), _ptr(latent),
                                     B, R, P, _ptr(positions), rope_theta, None, 0, 0, 0,
                                     latent.shape[1], _stream(c_new, stream))
    _check("mla_append_latent", st)
