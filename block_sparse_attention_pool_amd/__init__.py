"""Python binding of libsda (top-k block-sparse decode attention, gfx950).

Argument marshalling only: every step runs in the HIP kernels of libsda.so.
torch supplies device memory and the current stream.  The functions carry
the C names; each checks dtypes, contiguity and devices, derives the sizes
from the tensor shapes, allocates outputs and workspace when they are not
given, and raises SdaError when the library returns a non-zero status.

Layouts (bf16 given as torch.bfloat16, int32 as torch.int32):
  K, V      [B, H_kv, T_cap, d]      k_tilde   [B, H_kv, NB_cap, d] bfloat16
  f         [B, NQ, H_kv, d]         q         [B, NQ, H_q, d]
  block_idx [B, NQ, H_kv, n_sel_max] n_sel     [B, NQ, H_kv]
  out       [B, NQ, H_q, d] float32  lse       [B, NQ, H_q] float32
"""
import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsda.so")

SDA_GROUP_EXACT = 0
SDA_GROUP_SHARED_REP = 1
BLOCK = 64

_c_void_p = ctypes.c_void_p
_c_int = ctypes.c_int
_c_float = ctypes.c_float
_c_size_t = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/sda.h
_SIGNATURES = {
    "sda_status_string": (ctypes.c_char_p, [_c_int]),
    "sda_last_error": (ctypes.c_char_p, []),
    "sda_version": (ctypes.c_char_p, []),
    "sda_update_compressed_keys": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                                            _c_int, _c_int, _c_int, _c_int, _c_void_p]),
    "sda_update_compressed_keys_strided": (_c_int, [_c_void_p] * 4 + [_c_int] * 8 + [_c_void_p]),
    "sda_score_select_workspace": (_c_size_t, [_c_int] * 5),
    "sda_score_select_pooled_workspace": (_c_size_t, [_c_int] * 6),
    "sda_score_select_pooled": (_c_int, [_c_void_p] * 3 + [_c_int] * 11 + [_c_void_p] * 4 + [_c_size_t, _c_void_p]),
    "sda_score_select": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                  _c_int, _c_int, _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p,
                                  _c_void_p, _c_size_t, _c_void_p]),
    "sda_score_select_multihead_workspace": (_c_size_t, [_c_int] * 6),
    "sda_score_select_multihead": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int,
                                            _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                            _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size_t,
                                            _c_void_p]),
    "sda_score_select_multihead_pooled_workspace": (_c_size_t, [_c_int] * 7),
    "sda_score_select_multihead_pooled": (_c_int, [_c_void_p] * 3 + [_c_int] * 12 + [_c_float] + [_c_void_p] * 4
                                          + [_c_size_t, _c_void_p]),
    "sda_sparse_decode_workspace": (_c_size_t, [_c_int] * 7),
    "sda_sparse_decode": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                                   _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                   _c_void_p, _c_void_p, _c_int, _c_void_p, _c_size_t, _c_void_p]),
    "sda_grouped_decode_workspace": (_c_size_t, [_c_int] * 10),
    "sda_grouped_decode": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                                    _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float, _c_int,
                                    _c_int, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_void_p, _c_size_t,
                                    _c_void_p]),
    "sda_nsa_decode_workspace": (_c_size_t, [_c_int] * 11),
    "sda_nsa_decode": (_c_int, [_c_void_p] * 8 + [_c_int] * 5 + [_c_void_p] + [_c_int] * 5 + [_c_float]
                       + [_c_int] * 2 + [_c_void_p] * 4 + [_c_size_t, _c_void_p]),
    "sda_gather_blocks": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_int,
                                   _c_int, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_void_p]),
    "sda_decode_step_workspace": (_c_size_t, [_c_int] * 8),
    "sda_decode_step_is_fused": (_c_int, [_c_int] * 8),
    "sda_decode_step": (_c_int, [_c_void_p] * 6 + [_c_int] * 6 + [_c_float, _c_void_p, _c_void_p, _c_int]
                        + [_c_void_p] * 3 + [_c_int] * 5 + [_c_void_p] * 4 + [_c_int] * 2
                        + [_c_void_p, _c_size_t, _c_void_p]),
    "sda_nsa_chain_workspace": (_c_size_t, [_c_int] * 11),
    "sda_nsa_chain": (_c_int, [_c_void_p] * 2 + [_c_int] + [_c_void_p] + [_c_int] * 12 + [_c_float]
                      + [_c_void_p] * 3 + [_c_size_t, _c_void_p]),
    "sda_offload_chain_workspace": (_c_size_t, [_c_int] * 9),
    "sda_offload_chain": (_c_int, [_c_void_p, _c_int, _c_void_p] + [_c_int] * 8 + [_c_float, _c_void_p, _c_int]
                          + [_c_void_p] * 2 + [_c_size_t] + [_c_void_p] * 2),
    "sda_prefill_select": (_c_int, [_c_void_p] * 3 + [_c_int] * 10 + [_c_void_p] * 3),
    "sda_prefill_attention_workspace": (_c_size_t, [_c_int] * 7),
    "sda_prefill_attention": (_c_int, [_c_void_p] * 6 + [_c_int] * 8 + [_c_float, _c_int] + [_c_void_p] * 3
                              + [_c_size_t, _c_void_p]),
    "sda_decode_step_noalloc": (_c_int, [_c_void_p] * 6 + [_c_int] * 6 + [_c_float, _c_void_p, _c_void_p, _c_int]
                                + [_c_void_p] * 3 + [_c_int] * 5 + [_c_void_p] * 4 + [_c_int] * 2
                                + [_c_void_p]),
}

_lib = None


class SdaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{status_string(status) if _lib else status}: {msg}")
        self.status = status


def lib():
    """The loaded libsda.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_pool_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGNATURES)


def status_string(s):
    return lib().sda_status_string(int(s)).decode()


def last_error():
    return lib().sda_last_error().decode()


def version():
    return lib().sda_version().decode()


def _check(st):
    if st != 0:
        raise SdaError(st, last_error())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    return torch.cuda.current_stream().cuda_stream


def _need(t, name, dtype, shape=None):
    """Check a tensor argument: type, dtype, exact shape (None entries match
    any size; an int for shape means only that many dims) and contiguity.
    The C ABI cannot see buffer sizes, so every size the kernels index by is
    checked here; placement is checked by _on_gpu / _on_host once all shapes
    have passed."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if isinstance(shape, int):
        if t.dim() != shape:
            raise ValueError(f"{name} must have {shape} dims, got shape {tuple(t.shape)}")
    elif shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(w) != n for w, n in zip(shape, t.shape)):
            want = tuple("*" if w is None else int(w) for w in shape)
            raise ValueError(f"{name} must have shape {want}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(**tensors):
    """Every given tensor (None skipped) lives on the current GPU."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.device.index != torch.cuda.current_device():
            raise ValueError(f"{name} is on {t.device}, the current device is cuda:{torch.cuda.current_device()}")


def _on_host(**tensors):
    for name, t in tensors.items():
        if t.is_cuda:
            raise ValueError(f"{name} must be a host tensor")


def _opt(t, name, dtype, shape):
    if t is not None:
        _need(t, name, dtype, shape)


def _workspace(nbytes, device, ws=None):
    """Caller's workspace (a contiguous tensor of at least nbytes bytes), or a
    new zero-filled one (the split decode keeps arrival counters in it that
    must start at zero)."""
    if ws is not None:
        if not isinstance(ws, torch.Tensor) or not ws.is_contiguous():
            raise ValueError("ws must be a contiguous tensor")
        have = ws.numel() * ws.element_size()
        if have < nbytes:
            raise ValueError(f"ws holds {have} bytes, {nbytes} needed")
        return ws, have
    if nbytes == 0:
        return None, 0
    return torch.zeros(nbytes, dtype=torch.uint8, device=device), nbytes


class PreparedCall:
    """A library call whose ctypes arguments are converted once.

    run() re-sends them with the current (or given) stream, so a decode loop
    pays only the foreign-call cost per launch.  The tensors the call was
    prepared with must stay alive and keep their storage."""

    def __init__(self, name, args, keep):
        self._fn = getattr(lib(), name)
        self._args = list(args)
        self._keep = keep
        self.name = name

    def run(self, stream=None):
        self._args[-1] = _stream(stream)
        _check(self._fn(*self._args))


def prepare(fn_py, *a, **kw):
    """Run a binding function's checks and allocations without launching and
    return (PreparedCall, outputs); supported for sda_score_select,
    sda_sparse_decode and sda_decode_step."""
    kw["_prepare"] = True
    return fn_py(*a, **kw)


# ---------------------------------------------------------------------------

def sda_update_compressed_keys(k, k_tilde, len_old, len_new, max_new_tokens, stream=None):
    """Recompute the mean-pooled block keys touched by tokens [len_old, len_new)."""
    _need(k, "k", torch.bfloat16, 4)
    B, H, T_cap, d = k.shape
    _need(k_tilde, "k_tilde", torch.bfloat16, (B, H, None, d))
    _need(len_old, "len_old", torch.int32, (B,))
    _need(len_new, "len_new", torch.int32, (B,))
    _on_gpu(k=k, k_tilde=k_tilde, len_old=len_old, len_new=len_new)
    _check(lib().sda_update_compressed_keys(_ptr(k), _ptr(k_tilde), _ptr(len_old), _ptr(len_new),
                                            int(max_new_tokens), B, H, d, T_cap, k_tilde.shape[2],
                                            _stream(stream)))
    return k_tilde


def _select_outputs(B, NQ, H, n_sel_max, block_idx, n_sel, dev, suffix=""):
    if block_idx is None:
        block_idx = torch.empty((B, NQ, H, n_sel_max), dtype=torch.int32, device=dev)
    if n_sel is None:
        n_sel = torch.empty((B, NQ, H), dtype=torch.int32, device=dev)
    _need(block_idx, "block_idx" + suffix, torch.int32, (B, NQ, H, n_sel_max))
    _need(n_sel, "n_sel" + suffix, torch.int32, (B, NQ, H))
    return block_idx, n_sel


def sda_score_select(f, k_tilde, seq_len, n_init, n_local, top_k, n_sel_max=None, block_idx=None,
                     n_sel=None, scores=None, ws=None, stream=None, _prepare=False):
    """Indexer scores, exact top-k and block-set assembly; returns (block_idx, n_sel)."""
    _need(f, "f", torch.bfloat16, 4)
    B, NQ, H, d = f.shape
    _need(k_tilde, "k_tilde", torch.bfloat16, (B, H, None, d))
    _need(seq_len, "seq_len", torch.int32, (B,))
    NB_cap = k_tilde.shape[2]
    if n_sel_max is None:
        n_sel_max = block_idx.shape[-1] if block_idx is not None else n_init + n_local + top_k
    block_idx, n_sel = _select_outputs(B, NQ, H, n_sel_max, block_idx, n_sel, f.device)
    _opt(scores, "scores", torch.float32, (B, NQ, H, NB_cap))
    ws, wsb = _workspace(lib().sda_score_select_workspace(B, NQ, H, NB_cap, top_k), f.device, ws)
    _on_gpu(f=f, k_tilde=k_tilde, seq_len=seq_len, block_idx=block_idx, n_sel=n_sel, scores=scores, ws=ws)
    args = (_ptr(f), _ptr(k_tilde), _ptr(seq_len), B, NQ, H, d, NB_cap, n_init, n_local,
            top_k, n_sel_max, _ptr(block_idx), _ptr(n_sel), _ptr(scores), _ptr(ws), wsb, None)
    if _prepare:
        return PreparedCall("sda_score_select", args, (f, k_tilde, seq_len, block_idx, n_sel, scores, ws)), \
            (block_idx, n_sel)
    _check(lib().sda_score_select(*args[:-1], _stream(stream)))
    return block_idx, n_sel


def sda_update_compressed_keys_strided(k, k_tilde, len_old, len_new, max_new_tokens, window, stride,
                                       stream=None):
    """Recompute the overlapping compressed keys (kernel `window`, stride
    `stride`) touched by tokens [len_old, len_new); k_tilde is [B, H_kv, NC_cap, d]."""
    _need(k, "k", torch.bfloat16, 4)
    B, H, T_cap, d = k.shape
    _need(k_tilde, "k_tilde", torch.bfloat16, (B, H, None, d))
    _need(len_old, "len_old", torch.int32, (B,))
    _need(len_new, "len_new", torch.int32, (B,))
    _on_gpu(k=k, k_tilde=k_tilde, len_old=len_old, len_new=len_new)
    _check(lib().sda_update_compressed_keys_strided(_ptr(k), _ptr(k_tilde), _ptr(len_old), _ptr(len_new),
                                                    int(max_new_tokens), B, H, d, T_cap, k_tilde.shape[2],
                                                    int(window), int(stride), _stream(stream)))
    return k_tilde


def sda_score_select_pooled(f, k_tilde, seq_len, window, stride, n_init, n_local, top_k, n_sel_max=None,
                            block_idx=None, n_sel=None, scores=None, ws=None, stream=None):
    """Indexer scores on overlapping compressed keys, max-pooled onto the
    64-token blocks, then top-k and block sets; returns (block_idx, n_sel).
    scores (optional) is [B, NQ, H_kv, ceil(NC_cap * stride / 64)] float32."""
    _need(f, "f", torch.bfloat16, 4)
    B, NQ, H, d = f.shape
    _need(k_tilde, "k_tilde", torch.bfloat16, (B, H, None, d))
    _need(seq_len, "seq_len", torch.int32, (B,))
    NC_cap = k_tilde.shape[2]
    if n_sel_max is None:
        n_sel_max = block_idx.shape[-1] if block_idx is not None else n_init + n_local + top_k
    block_idx, n_sel = _select_outputs(B, NQ, H, n_sel_max, block_idx, n_sel, f.device)
    _opt(scores, "scores", torch.float32, (B, NQ, H, -(-NC_cap * int(stride) // BLOCK)))
    nbytes = lib().sda_score_select_pooled_workspace(B, NQ, H, NC_cap, int(stride), top_k)
    ws, wsb = _workspace(nbytes, f.device, ws)
    _on_gpu(f=f, k_tilde=k_tilde, seq_len=seq_len, block_idx=block_idx, n_sel=n_sel, scores=scores, ws=ws)
    _check(lib().sda_score_select_pooled(_ptr(f), _ptr(k_tilde), _ptr(seq_len), B, NQ, H, d, NC_cap, int(window),
                                         int(stride), n_init, n_local, top_k, n_sel_max, _ptr(block_idx),
                                         _ptr(n_sel), _ptr(scores), _ptr(ws), wsb, _stream(stream)))
    return block_idx, n_sel


def sda_score_select_multihead(q, k_tilde, seq_len, n_init, n_local, top_k, tau, H_kv=None, n_sel_max=None,
                               block_idx=None, n_sel=None, scores=None, ws=None, stream=None):
    """G-head softmax-sum selector (comparator); returns (block_idx, n_sel)."""
    _need(q, "q", torch.bfloat16, 4)
    B, NQ, H_q, d = q.shape
    _need(k_tilde, "k_tilde", torch.bfloat16, (B, H_kv, None, d))
    _need(seq_len, "seq_len", torch.int32, (B,))
    H = k_tilde.shape[1]
    NB_cap = k_tilde.shape[2]
    if n_sel_max is None:
        n_sel_max = block_idx.shape[-1] if block_idx is not None else n_init + n_local + top_k
    block_idx, n_sel = _select_outputs(B, NQ, H, n_sel_max, block_idx, n_sel, q.device)
    _opt(scores, "scores", torch.float32, (B, NQ, H, NB_cap))
    nbytes = lib().sda_score_select_multihead_workspace(B, NQ, H_q, H, NB_cap, top_k)
    ws, wsb = _workspace(nbytes, q.device, ws)
    _on_gpu(q=q, k_tilde=k_tilde, seq_len=seq_len, block_idx=block_idx, n_sel=n_sel, scores=scores, ws=ws)
    _check(lib().sda_score_select_multihead(_ptr(q), _ptr(k_tilde), _ptr(seq_len), B, NQ, H_q, H, d, NB_cap,
                                            n_init, n_local, top_k, n_sel_max, float(tau), _ptr(block_idx),
                                            _ptr(n_sel), _ptr(scores), _ptr(ws), wsb, _stream(stream)))
    return block_idx, n_sel


def sda_score_select_multihead_pooled(q, k_tilde, seq_len, window, stride, n_init, n_local, top_k, tau, H_kv=None,
                                      n_sel_max=None, block_idx=None, n_sel=None, scores=None, ws=None, stream=None):
    """InfLLM-V2's G-head selector on overlapping compressed keys (kernel
    `window`, stride `stride`): per-head softmax over the entries, sum over
    the heads, max-pool onto the 64-token blocks, then top-k; returns
    (block_idx, n_sel)."""
    _need(q, "q", torch.bfloat16, 4)
    B, NQ, H_q, d = q.shape
    _need(k_tilde, "k_tilde", torch.bfloat16, (B, H_kv, None, d))
    _need(seq_len, "seq_len", torch.int32, (B,))
    H = k_tilde.shape[1]
    NC_cap = k_tilde.shape[2]
    if n_sel_max is None:
        n_sel_max = block_idx.shape[-1] if block_idx is not None else n_init + n_local + top_k
    block_idx, n_sel = _select_outputs(B, NQ, H, n_sel_max, block_idx, n_sel, q.device)
    _opt(scores, "scores", torch.float32, (B, NQ, H, -(-NC_cap * int(stride) // BLOCK)))
    nbytes = lib().sda_score_select_multihead_pooled_workspace(B, NQ, H_q, H, NC_cap, int(stride), top_k)
    ws, wsb = _workspace(nbytes, q.device, ws)
    _on_gpu(q=q, k_tilde=k_tilde, seq_len=seq_len, block_idx=block_idx, n_sel=n_sel, scores=scores, ws=ws)
    _check(lib().sda_score_select_multihead_pooled(_ptr(q), _ptr(k_tilde), _ptr(seq_len), B, NQ, H_q, H, d, NC_cap,
                                                   int(window), int(stride), n_init, n_local, top_k, n_sel_max,
                                                   float(tau), _ptr(block_idx), _ptr(n_sel), _ptr(scores), _ptr(ws),
                                                   wsb, _stream(stream)))
    return block_idx, n_sel


def _attn_inputs(q, k, v, seq_len, block_idx, n_sel, NQ_lists=None):
    """Checks shared by the decode calls; returns (B, NQ, H_q, d, H_kv, T_cap, n_sel_max)."""
    _need(q, "q", torch.bfloat16, 4)
    B, NQ, H_q, d = q.shape
    _need(k, "k", torch.bfloat16, (B, None, None, d))
    H_kv, T_cap = k.shape[1], k.shape[2]
    _need(v, "v", torch.bfloat16, tuple(k.shape))
    _need(seq_len, "seq_len", torch.int32, (B,))
    _need(block_idx, "block_idx", torch.int32, (B, NQ if NQ_lists is None else NQ_lists, H_kv, None))
    _need(n_sel, "n_sel", torch.int32, (B, NQ if NQ_lists is None else NQ_lists, H_kv))
    if H_q % H_kv:
        raise ValueError(f"H_q={H_q} is not a multiple of H_kv={H_kv}")
    return B, NQ, H_q, d, H_kv, T_cap, block_idx.shape[3]


def _attn_outputs(B, NQ, H_q, d, out, lse, dev, lse_tail=()):
    if out is None:
        out = torch.empty((B, NQ, H_q, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, NQ, H_q) + lse_tail, dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, NQ, H_q, d))
    _need(lse, "lse", torch.float32, (B, NQ, H_q) + lse_tail)
    return out, lse


def sda_sparse_decode(q, k, v, seq_len, block_idx, n_sel, scale=None, out=None, lse=None, slot=None,
                      split_k=0, ws=None, stream=None, _prepare=False):
    """Block-sparse decode attention; returns (out, lse)."""
    B, NQ, H_q, d, H_kv, T_cap, n_sel_max = _attn_inputs(q, k, v, seq_len, block_idx, n_sel)
    _opt(slot, "slot", torch.int32, tuple(block_idx.shape))
    if scale is None:
        scale = d ** -0.5
    out, lse = _attn_outputs(B, NQ, H_q, d, out, lse, q.device)
    nbytes = lib().sda_sparse_decode_workspace(B, NQ, H_q, H_kv, n_sel_max, d, int(split_k))
    ws, wsb = _workspace(nbytes, q.device, ws)
    _on_gpu(q=q, k=k, v=v, seq_len=seq_len, block_idx=block_idx, n_sel=n_sel, slot=slot, out=out, lse=lse, ws=ws)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(seq_len), _ptr(block_idx), _ptr(n_sel),
            n_sel_max, _ptr(slot), T_cap, B, NQ, H_q, H_kv, d, float(scale), _ptr(out),
            _ptr(lse), int(split_k), _ptr(ws), wsb, None)
    if _prepare:
        return PreparedCall("sda_sparse_decode", args, (q, k, v, seq_len, block_idx, n_sel, out, lse, slot, ws)), \
            (out, lse)
    _check(lib().sda_sparse_decode(*args[:-1], _stream(stream)))
    return out, lse


def sda_decode_step(q, k, v, seq_len, block_idx, n_sel, f_next, k_tilde_next, seq_len_next, n_init, n_local,
                    top_k, n_sel_max_next=None, block_idx_next=None, n_sel_next=None, scale=None, out=None,
                    lse=None, split_k=0, k_tilde_cur=None, len_old_cur=None, max_new_tokens_cur=1, ws=None,
                    stream=None, _prepare=False, _noalloc=False):
    """Layer l's decode plus layer l+1's selection (same results as
    sda_score_select for l+1 then sda_sparse_decode for l) and, with
    k_tilde_cur, the refresh of layer l's compressed keys for the tokens
    [len_old_cur, seq_len); returns (out, lse, block_idx_next, n_sel_next)."""
    B, NQ, H_q, d, H_kv, T_cap, n_sel_max = _attn_inputs(q, k, v, seq_len, block_idx, n_sel)
    if NQ != 1:
        raise ValueError("sda_decode_step takes one query per sequence")
    _need(f_next, "f_next", torch.bfloat16, (B, 1, H_kv, d))
    _need(k_tilde_next, "k_tilde_next", torch.bfloat16, (B, H_kv, None, d))
    _need(seq_len_next, "seq_len_next", torch.int32, (B,))
    NB_cap_next = k_tilde_next.shape[2]
    if n_sel_max_next is None:
        n_sel_max_next = block_idx_next.shape[-1] if block_idx_next is not None else n_init + n_local + top_k
    if scale is None:
        scale = d ** -0.5
    dev = q.device
    out, lse = _attn_outputs(B, 1, H_q, d, out, lse, dev)
    block_idx_next, n_sel_next = _select_outputs(B, 1, H_kv, n_sel_max_next, block_idx_next, n_sel_next, dev,
                                                  "_next")
    NB_cap_cur = 0
    if k_tilde_cur is not None:
        _need(k_tilde_cur, "k_tilde_cur", torch.bfloat16, (B, H_kv, None, d))
        _need(len_old_cur, "len_old_cur", torch.int32, (B,))
        NB_cap_cur = k_tilde_cur.shape[2]
    if _noalloc:
        ws, wsb = None, 0
    else:
        nbytes = lib().sda_decode_step_workspace(B, H_q, H_kv, d, n_sel_max, int(split_k), NB_cap_next, top_k)
        ws, wsb = _workspace(nbytes, dev, ws)
    _on_gpu(q=q, k=k, v=v, seq_len=seq_len, block_idx=block_idx, n_sel=n_sel, f_next=f_next,
            k_tilde_next=k_tilde_next, seq_len_next=seq_len_next, out=out, lse=lse, block_idx_next=block_idx_next,
            n_sel_next=n_sel_next, k_tilde_cur=k_tilde_cur, len_old_cur=len_old_cur, ws=ws)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(seq_len), _ptr(block_idx), _ptr(n_sel), n_sel_max, T_cap, B, H_q,
            H_kv, d, float(scale), _ptr(out), _ptr(lse), int(split_k), _ptr(f_next), _ptr(k_tilde_next),
            _ptr(seq_len_next), NB_cap_next, n_init, n_local, top_k, n_sel_max_next, _ptr(block_idx_next),
            _ptr(n_sel_next), _ptr(k_tilde_cur), _ptr(len_old_cur), int(max_new_tokens_cur), NB_cap_cur)
    args = args + ((None,) if _noalloc else (_ptr(ws), wsb, None))
    outs = (out, lse, block_idx_next, n_sel_next)
    name = "sda_decode_step_noalloc" if _noalloc else "sda_decode_step"
    if _prepare:
        return PreparedCall(name, args, (q, k, v, seq_len, block_idx, n_sel, f_next, k_tilde_next, seq_len_next, ws,
                                         k_tilde_cur, len_old_cur) + outs), outs
    _check(getattr(lib(), name)(*args[:-1], _stream(stream)))
    return outs


def sda_decode_step_noalloc(q, k, v, seq_len, block_idx, n_sel, f_next, k_tilde_next, seq_len_next, n_init,
                            n_local, top_k, **kw):
    """sda_decode_step without a workspace: the library's static per-device
    scratch holds the split partials, counters and candidate lists (for
    callers that cannot allocate).  Same arguments and results as
    sda_decode_step, minus ws; calls that overlap on one GPU race."""
    if "ws" in kw:
        raise TypeError("sda_decode_step_noalloc takes no workspace")
    return sda_decode_step(q, k, v, seq_len, block_idx, n_sel, f_next, k_tilde_next, seq_len_next, n_init, n_local,
                           top_k, _noalloc=True, **kw)


def sda_grouped_decode(q, k, v, seq_len, block_idx, n_sel, group_C, mode=SDA_GROUP_EXACT, scale=None,
                       NB_cap=None, out=None, lse=None, union_count=None, split_k=0, ws=None, stream=None):
    """SSV grouped verification decode; returns (out, lse, union_count)."""
    B, NQ, H_q, d, H_kv, T_cap, n_sel_max = _attn_inputs(q, k, v, seq_len, block_idx, n_sel)
    if NB_cap is None:
        NB_cap = -(-T_cap // BLOCK)
    if scale is None:
        scale = d ** -0.5
    if int(group_C) < 1:
        raise ValueError("group_C must be >= 1")
    n_groups = -(-NQ // int(group_C))
    out, lse = _attn_outputs(B, NQ, H_q, d, out, lse, q.device)
    if union_count is None:
        union_count = torch.empty((B, n_groups, H_kv), dtype=torch.int32, device=q.device)
    _need(union_count, "union_count", torch.int32, (B, n_groups, H_kv))
    nbytes = lib().sda_grouped_decode_workspace(B, NQ, H_q, H_kv, n_sel_max, d, int(NB_cap), int(group_C),
                                                int(mode), int(split_k))
    ws, wsb = _workspace(nbytes, q.device, ws)
    _on_gpu(q=q, k=k, v=v, seq_len=seq_len, block_idx=block_idx, n_sel=n_sel, out=out, lse=lse,
            union_count=union_count, ws=ws)
    _check(lib().sda_grouped_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(seq_len), _ptr(block_idx), _ptr(n_sel),
                                    n_sel_max, T_cap, int(NB_cap), B, NQ, H_q, H_kv, d, float(scale),
                                    int(group_C), int(mode), _ptr(out), _ptr(lse), _ptr(union_count),
                                    int(split_k), _ptr(ws), wsb, _stream(stream)))
    return out, lse, union_count


def sda_nsa_decode(q, k, v, k_cmp, v_cmp, seq_len, block_idx, n_sel, gates, cmp_stride, window, group_C=1,
                   mode=SDA_GROUP_EXACT, scale=None, out=None, lse=None, union_count=None, ws=None, stream=None):
    """NSA verification output (compressed, selected-block and window branches,
    gated sum) in one launch; returns (out, lse [B, NQ, H_q, 3], union_count).
    group_C up to 32 and group_C * G up to 128 rows in either mode (two or
    more queries per KV head run on row tiles that load the compressed cache
    and the window once per tile)."""
    B, NQ, H_q, d, H, T_cap, n_sel_max = _attn_inputs(q, k, v, seq_len, block_idx, n_sel)
    _need(k_cmp, "k_cmp", torch.bfloat16, (B, H, None, d))
    _need(v_cmp, "v_cmp", torch.bfloat16, tuple(k_cmp.shape))
    _need(gates, "gates", torch.float32, (B, NQ, H_q, 3))
    NC_cap = k_cmp.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if int(group_C) < 1:
        raise ValueError("group_C must be >= 1")
    out, lse = _attn_outputs(B, NQ, H_q, d, out, lse, q.device, lse_tail=(3,))
    n_groups = -(-NQ // int(group_C))
    if union_count is None and group_C > 1:
        union_count = torch.empty((B, n_groups, H), dtype=torch.int32, device=q.device)
    _opt(union_count, "union_count", torch.int32, (B, n_groups, H))
    nbytes = lib().sda_nsa_decode_workspace(B, NQ, H_q, H, n_sel_max, d, T_cap, NC_cap, int(window), int(group_C),
                                            int(mode))
    ws, wsb = _workspace(nbytes, q.device, ws)
    _on_gpu(q=q, k=k, v=v, k_cmp=k_cmp, v_cmp=v_cmp, seq_len=seq_len, block_idx=block_idx, n_sel=n_sel,
            gates=gates, out=out, lse=lse, union_count=union_count, ws=ws)
    _check(lib().sda_nsa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(k_cmp), _ptr(v_cmp), _ptr(seq_len), _ptr(block_idx),
                                _ptr(n_sel), n_sel_max, T_cap, NC_cap, int(cmp_stride), int(window), _ptr(gates), B,
                                NQ, H_q, H, d, float(scale), int(group_C), int(mode), _ptr(out), _ptr(lse),
                                _ptr(union_count), _ptr(ws), wsb, _stream(stream)))
    return out, lse, union_count


class NsaLayer(ctypes.Structure):
    """sda_nsa_layer of the C ABI: one layer's tensors in a refresh/reuse chain."""
    _fields_ = [(n, _c_void_p) for n in ("q", "k", "v", "k_cmp", "v_cmp", "k_route", "f_route", "gates", "out",
                                         "lse")]


def sda_nsa_chain(layers, refresh, seq_len, top_n, cmp_stride, window, group_C=1, mode=SDA_GROUP_EXACT, scale=None,
                  block_idx_cache=None, n_sel_cache=None, ws=None, stream=None, _prepare=False):
    """Refresh/reuse chain of NSA verification layers: refresh layers route
    (top_n blocks per row from f_route . k_route) and cache the lists, every
    layer runs the three-branch NSA output with the cached lists.  `layers`
    is a list of dicts with q, k, v, k_cmp, v_cmp, gates (and k_route,
    f_route on refresh layers; out, lse optional); returns
    ([(out, lse) per layer], block_idx_cache, n_sel_cache)."""
    L = len(layers)
    if L < 1 or len(refresh) != L:
        raise ValueError("one refresh flag per layer, at least one layer")
    y0 = layers[0]
    _need(y0["q"], "q", torch.bfloat16, 4)
    B, NQ, H_q, d = y0["q"].shape
    _need(y0["k"], "k", torch.bfloat16, (B, None, None, d))
    H, T_cap = y0["k"].shape[1], y0["k"].shape[2]
    _need(y0["k_cmp"], "k_cmp", torch.bfloat16, (B, H, None, d))
    NC_cap = y0["k_cmp"].shape[2]
    NB_cap = -(-T_cap // BLOCK)
    _need(seq_len, "seq_len", torch.int32, (B,))
    if H_q % H:
        raise ValueError(f"H_q={H_q} is not a multiple of H_kv={H}")
    dev = y0["q"].device
    if block_idx_cache is None:
        block_idx_cache = torch.empty((B, NQ, H, top_n), dtype=torch.int32, device=dev)
    if n_sel_cache is None:
        n_sel_cache = torch.empty((B, NQ, H), dtype=torch.int32, device=dev)
    _need(block_idx_cache, "block_idx_cache", torch.int32, (B, NQ, H, top_n))
    _need(n_sel_cache, "n_sel_cache", torch.int32, (B, NQ, H))
    arr = (NsaLayer * L)()
    outs, keep = [], []
    for j, y in enumerate(layers):
        _need(y["q"], f"layers[{j}].q", torch.bfloat16, (B, NQ, H_q, d))
        for n in ("k", "v"):
            _need(y[n], f"layers[{j}].{n}", torch.bfloat16, (B, H, T_cap, d))
        for n in ("k_cmp", "v_cmp"):
            _need(y[n], f"layers[{j}].{n}", torch.bfloat16, (B, H, NC_cap, d))
        _need(y["gates"], f"layers[{j}].gates", torch.float32, (B, NQ, H_q, 3))
        if refresh[j]:
            _need(y["k_route"], f"layers[{j}].k_route", torch.bfloat16, (B, H, NB_cap, d))
            _need(y["f_route"], f"layers[{j}].f_route", torch.bfloat16, (B, NQ, H, d))
        out, lse = _attn_outputs(B, NQ, H_q, d, y.get("out"), y.get("lse"), dev, lse_tail=(3,))
        outs.append((out, lse))
        ts = dict(q=y["q"], k=y["k"], v=y["v"], k_cmp=y["k_cmp"], v_cmp=y["v_cmp"], gates=y["gates"], out=out,
                  lse=lse, k_route=y.get("k_route") if refresh[j] else None,
                  f_route=y.get("f_route") if refresh[j] else None)
        _on_gpu(**{f"layers[{j}].{n}": t for n, t in ts.items()})
        for n, t in ts.items():
            setattr(arr[j], n, _ptr(t))
        keep.append(ts)
    flags = (ctypes.c_uint8 * L)(*[1 if x else 0 for x in refresh])
    if scale is None:
        scale = d ** -0.5
    nbytes = lib().sda_nsa_chain_workspace(B, NQ, H_q, H, d, T_cap, NC_cap, int(window), int(top_n), int(group_C),
                                           int(mode))
    ws, wsb = _workspace(nbytes, dev, ws)
    _on_gpu(seq_len=seq_len, block_idx_cache=block_idx_cache, n_sel_cache=n_sel_cache, ws=ws)
    args = (ctypes.addressof(arr), ctypes.addressof(flags), L, _ptr(seq_len), B, NQ, H_q, H, d, T_cap, NC_cap,
            int(cmp_stride), int(window), int(top_n), int(group_C), int(mode), float(scale), _ptr(block_idx_cache),
            _ptr(n_sel_cache), _ptr(ws), wsb, None)
    res = (outs, block_idx_cache, n_sel_cache)
    if _prepare:
        return PreparedCall("sda_nsa_chain", args, (arr, flags, keep, seq_len, block_idx_cache, n_sel_cache, ws)), res
    _check(lib().sda_nsa_chain(*args[:-1], _stream(stream)))
    return res


class OffloadLayer(ctypes.Structure):
    """sda_offload_layer of the C ABI: one layer of the offloaded decode chain."""
    _fields_ = [(n, _c_void_p) for n in ("k_host", "v_host", "k_tilde", "q", "f", "out", "lse")]


def sda_offload_chain(layers, seq_len, n_init, n_local, top_k, f_first, prefetch_workgroups=64, scale=None,
                      block_idx=None, ws=None, stream=None, side_stream=None, _prepare=False):
    """Offloaded-KV decode through L layers with the persistent prefetch pool:
    each layer's blocks are chosen one layer ahead, copied from pinned host
    memory by the pool on `side_stream` while the previous layer attends,
    and attended from a device stage.  `layers`: dicts with k_host, v_host
    (pinned CPU bf16 [B, H_kv, T_cap, d]), k_tilde, q, f (GPU), out and lse
    optional.  Returns ([(out, lse) per layer], block_idx [L, B, 1, H_kv, n],
    ws); the int32 at byte 8 of ws is non-zero if a transfer wait gave up."""
    L = len(layers)
    if L < 1:
        raise ValueError("at least one layer")
    y0 = layers[0]
    _need(y0["k_host"], "k_host", torch.bfloat16, 4)
    B, H, T_cap, d = y0["k_host"].shape
    _need(y0["q"], "q", torch.bfloat16, (B, 1, None, d))
    H_q = y0["q"].shape[2]
    if H_q % H:
        raise ValueError(f"H_q={H_q} is not a multiple of H_kv={H}")
    NB_cap = -(-T_cap // BLOCK)
    nsm = n_init + n_local + top_k
    _need(seq_len, "seq_len", torch.int32, (B,))
    _need(f_first, "f_first", torch.bfloat16, (B, 1, H, d))
    dev = y0["q"].device
    if block_idx is None:
        block_idx = torch.empty((L, B, 1, H, nsm), dtype=torch.int32, device=dev)
    _need(block_idx, "block_idx", torch.int32, (L, B, 1, H, nsm))
    arr = (OffloadLayer * L)()
    outs, keep = [], []
    for j, y in enumerate(layers):
        for n in ("k_host", "v_host"):
            _need(y[n], f"layers[{j}].{n}", torch.bfloat16, (B, H, T_cap, d))
            _on_host(**{f"layers[{j}].{n}": y[n]})
            if not y[n].is_pinned():
                raise ValueError(f"layers[{j}].{n} must be pinned host memory")
        _need(y["k_tilde"], f"layers[{j}].k_tilde", torch.bfloat16, (B, H, NB_cap, d))
        _need(y["q"], f"layers[{j}].q", torch.bfloat16, (B, 1, H_q, d))
        _need(y["f"], f"layers[{j}].f", torch.bfloat16, (B, 1, H, d))
        out, lse = _attn_outputs(B, 1, H_q, d, y.get("out"), y.get("lse"), dev)
        outs.append((out, lse))
        dv = dict(k_tilde=y["k_tilde"], q=y["q"], f=y["f"], out=out, lse=lse)
        _on_gpu(**{f"layers[{j}].{n}": t for n, t in dv.items()})
        for n, t in list(dv.items()) + [("k_host", y["k_host"]), ("v_host", y["v_host"])]:
            setattr(arr[j], n, _ptr(t))
        keep.append((dv, y["k_host"], y["v_host"]))
    if scale is None:
        scale = d ** -0.5
    nbytes = lib().sda_offload_chain_workspace(L, B, H_q, H, d, T_cap, n_init, n_local, top_k)
    ws, wsb = _workspace(nbytes, dev, ws)
    _on_gpu(seq_len=seq_len, f_first=f_first, block_idx=block_idx, ws=ws)
    if side_stream is None:
        side_stream = torch.cuda.Stream()
    args = [ctypes.addressof(arr), L, _ptr(seq_len), B, H_q, H, d, T_cap, n_init, n_local, top_k, float(scale),
            _ptr(f_first), int(prefetch_workgroups), _ptr(block_idx), _ptr(ws), wsb, None, _stream(side_stream)]
    res = (outs, block_idx, ws)
    if _prepare:
        # the stream argument is the second to last here: PreparedCall fills the last one
        raise ValueError("sda_offload_chain runs eagerly (it starts a pool on a second stream)")
    args[-2] = _stream(stream)
    _check(lib().sda_offload_chain(*args))
    return res


def sda_prefill_select(f, k_tilde, seq_len, pos0, n_init, n_local, top_k, n_sel_max=None, block_idx=None,
                       n_sel=None, stream=None):
    """Block sets of every query position of a prefill chunk (query r at
    position pos0 + r chooses as a decode step at length pos0 + r + 1);
    returns (block_idx, n_sel)."""
    _need(f, "f", torch.bfloat16, 4)
    B, NQ, H, d = f.shape
    _need(k_tilde, "k_tilde", torch.bfloat16, (B, H, None, d))
    _need(seq_len, "seq_len", torch.int32, (B,))
    if n_sel_max is None:
        n_sel_max = block_idx.shape[-1] if block_idx is not None else n_init + n_local + top_k
    block_idx, n_sel = _select_outputs(B, NQ, H, n_sel_max, block_idx, n_sel, f.device)
    _on_gpu(f=f, k_tilde=k_tilde, seq_len=seq_len, block_idx=block_idx, n_sel=n_sel)
    _check(lib().sda_prefill_select(_ptr(f), _ptr(k_tilde), _ptr(seq_len), B, NQ, H, d, k_tilde.shape[2], int(pos0),
                                    n_init, n_local, top_k, n_sel_max, _ptr(block_idx), _ptr(n_sel),
                                    _stream(stream)))
    return block_idx, n_sel


def sda_prefill_attention(q, k, v, seq_len, block_idx, n_sel, pos0, scale=None, NB_cap=None, out=None, lse=None,
                          ws=None, stream=None):
    """Causal block-sparse attention of every query position of a prefill
    chunk over its own blocks; returns (out, lse)."""
    B, NQ, H_q, d, H_kv, T_cap, n_sel_max = _attn_inputs(q, k, v, seq_len, block_idx, n_sel)
    if NB_cap is None:
        NB_cap = -(-T_cap // BLOCK)
    if scale is None:
        scale = d ** -0.5
    out, lse = _attn_outputs(B, NQ, H_q, d, out, lse, q.device)
    nbytes = lib().sda_prefill_attention_workspace(B, NQ, H_q, H_kv, n_sel_max, d, int(NB_cap))
    ws, wsb = _workspace(nbytes, q.device, ws)
    _on_gpu(q=q, k=k, v=v, seq_len=seq_len, block_idx=block_idx, n_sel=n_sel, out=out, lse=lse, ws=ws)
    _check(lib().sda_prefill_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(seq_len), _ptr(block_idx), _ptr(n_sel),
                                       n_sel_max, T_cap, int(NB_cap), B, NQ, H_q, H_kv, d, float(scale), int(pos0),
                                       _ptr(out), _ptr(lse), _ptr(ws), wsb, _stream(stream)))
    return out, lse


def sda_gather_blocks(k_host, v_host, block_idx, n_sel, k_stage=None, v_stage=None, slot=None,
                      max_workgroups=0, stream=None):
    """Copy the selected blocks of pinned host K/V into a device stage.

    k_host, v_host: pinned CPU bf16 [B, H_kv, T_cap, d]; block_idx [B, 1, H_kv, n_sel_max]
    or [B, H_kv, n_sel_max]; returns (k_stage, v_stage, slot) with slot shaped like block_idx."""
    _need(k_host, "k_host", torch.bfloat16, 4)
    B, H_kv, T_cap, d = k_host.shape
    _need(v_host, "v_host", torch.bfloat16, tuple(k_host.shape))
    if block_idx.dim() == 4:
        _need(block_idx, "block_idx", torch.int32, (B, 1, H_kv, None))
        _need(n_sel, "n_sel", torch.int32, (B, 1, H_kv))
    else:
        _need(block_idx, "block_idx", torch.int32, (B, H_kv, None))
        _need(n_sel, "n_sel", torch.int32, (B, H_kv))
    n_sel_max = block_idx.shape[-1]
    dev = block_idx.device
    if k_stage is None:
        k_stage = torch.empty((B, H_kv, n_sel_max * BLOCK, d), dtype=torch.bfloat16, device=dev)
    if v_stage is None:
        v_stage = torch.empty((B, H_kv, n_sel_max * BLOCK, d), dtype=torch.bfloat16, device=dev)
    if slot is None:
        slot = torch.empty(block_idx.shape, dtype=torch.int32, device=dev)
    _need(k_stage, "k_stage", torch.bfloat16, (B, H_kv, n_sel_max * BLOCK, d))
    _need(v_stage, "v_stage", torch.bfloat16, (B, H_kv, n_sel_max * BLOCK, d))
    _need(slot, "slot", torch.int32, tuple(block_idx.shape))
    _on_host(k_host=k_host, v_host=v_host)
    if not (k_host.is_pinned() and v_host.is_pinned()):
        raise ValueError("k_host and v_host must be pinned host memory")
    _on_gpu(block_idx=block_idx, n_sel=n_sel, k_stage=k_stage, v_stage=v_stage, slot=slot)
    _check(lib().sda_gather_blocks(_ptr(k_host), _ptr(v_host), _ptr(block_idx), _ptr(n_sel), n_sel_max, B,
                                   H_kv, d, T_cap, _ptr(k_stage), _ptr(v_stage), _ptr(slot),
                                   int(max_workgroups), _stream(stream)))
    return k_stage, v_stage, slot
