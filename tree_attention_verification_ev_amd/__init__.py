"""Python binding of libev.so: one-pass verification of a drafted token tree on MI355X.

Thin ctypes marshalling over the C ABI declared in include/ev.h.  Every function has the
name of the C entry point it calls and takes torch tensors that already live on the GPU;
torch provides device memory and the current HIP stream, nothing else.  All arithmetic
happens in the HIP kernels of libev.so; there is no host fallback: if the library is not
built or cannot be loaded, every call raises.

Outputs and workspace may be passed in (preallocated) or are allocated here with
torch.empty.  With check=True a call synchronises and raises EvError when the device
status word reports a data error; the default leaves the call asynchronous.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libev.so")

EV_OK = 0
EV_F32, EV_BF16, EV_INT4 = 0, 1, 2
STATUS_NAMES = {
    0: "EV_OK", 1: "EV_ERR_NULL", 2: "EV_ERR_SHAPE", 3: "EV_ERR_DTYPE", 4: "EV_ERR_WORKSPACE",
    5: "EV_ERR_ARG", 6: "EV_ERR_LAUNCH", 7: "EV_ERR_SCRATCH", 101: "EV_DERR_PARENT",
    102: "EV_DERR_BOUNDS",
    103: "EV_DERR_TOKEN", 104: "EV_DERR_PATH", 105: "EV_DERR_WIDTH",
}
EXPORTED = (
    "ev_tree_mask_build", "ev_tree_attention_workspace", "ev_tree_attention",
    "ev_tree_attention_noalloc", "ev_tree_attention_noalloc_limit", "ev_tree_mask_attention",
    "ev_accept_workspace", "ev_accept_greedy", "ev_accept_rejection",
    "ev_accept_greedy_compact", "ev_accept_rejection_compact",
    "ev_accept_sampled_workspace", "ev_accept_sampled", "ev_kv_compact",
    "ev_kv_compact_remap_workspace", "ev_kv_compact_remap",
    "ev_draft_tree_workspace", "ev_draft_tree_expand", "ev_draft_tree_finalize",
    "ev_status_string",
)
# include/ev_peaks.h: calibration kernels (box-measured peaks), not part of the pass
EXPORTED_PEAKS = ("ev_peak_mfma_bf16", "ev_peak_copy", "ev_peak_read")


class EvError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS_NAMES.get(code, code)} ({_status_text(code)})")


class EvKvDesc(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("paged", ctypes.c_int32), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("n_layers", ctypes.c_int32), ("layer_stride", ctypes.c_int64), ("cap", ctypes.c_int64),
        ("block_table", ctypes.c_void_p), ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("n_blocks", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
    ]


_lib = None
_P, _I32, _I64, _F32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """The loaded libev.so (raises EvError-free OSError/RuntimeError when absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m tree_attention_verification_ev_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        kv = ctypes.POINTER(EvKvDesc)
        sigs = {
            "ev_tree_mask_build": (_I32, [_P, _I32, _I32, _P, _P, _P, _P]),
            "ev_tree_attention_workspace": (_SZ, [kv, _I32, _I32, _I32, _I64]),
            "ev_tree_attention": (_I32, [_P, kv, _P, _P, _I32, _I32, _I32, _I64, _F32, _P, _P, _P,
                                         _SZ, _P, _P]),
            "ev_tree_attention_noalloc": (_I32, [_P, kv, _P, _P, _I32, _I32, _I32, _I64, _F32, _P,
                                                 _P, _P, _P]),
            "ev_tree_attention_noalloc_limit": (_SZ, []),
            "ev_tree_mask_attention": (_I32, [_P, kv, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _F32,
                                              _P, _P, _P, _SZ, _P, _P]),
            "ev_accept_workspace": (_SZ, [_I32, _I32, _I32]),
            "ev_accept_greedy": (_I32, [_P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P, _P]),
            "ev_accept_rejection": (_I32, [_P, _P, _P, _I32, _I32, _I32, _F32, _P, _P, _P, _P, _P,
                                           _SZ, _P, _P]),
            "ev_accept_greedy_compact": (_I32, [_P, _P, _P, _I32, _I32, _I32, _P, _P, _P, kv, _P,
                                                _P, _P, _SZ, _P, _P]),
            "ev_accept_rejection_compact": (_I32, [_P, _P, _P, _I32, _I32, _I32, _F32, _P, _P, _P,
                                                   _P, kv, _P, _P, _P, _SZ, _P, _P]),
            "ev_accept_sampled_workspace": (_SZ, [_I32, _I32, _I32]),
            "ev_accept_sampled": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _F32, _F32, _P, _I32,
                                         _P, _P, _P, _P, _SZ, _P, _P]),
            "ev_kv_compact": (_I32, [kv, _P, _P, _P, _I32, _I32, _P, _P, _P]),
            "ev_kv_compact_remap_workspace": (_SZ, [_I32]),
            "ev_kv_compact_remap": (_I32, [kv, _P, _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P,
                                           _P]),
            "ev_draft_tree_workspace": (_SZ, [_I32, _I32, _I32]),
            "ev_draft_tree_expand": (_I32, [_P, _I32, _I32, _I32, _I32, _F32, _I32, _P, _P, _P,
                                            _P, _SZ, _P, _P]),
            "ev_draft_tree_finalize": (_I32, [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _SZ,
                                              _P]),
            "ev_status_string": (ctypes.c_char_p, [_I32]),
            "ev_peak_mfma_bf16": (_I32, [_I32, _I32, _P, _P]),
            "ev_peak_copy": (_I32, [_P, _P, _SZ, _P]),
            "ev_peak_read": (_I32, [_P, _SZ, _P, _I32, _P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _status_text(code: int) -> str:
    try:
        return lib().ev_status_string(code).decode()
    except Exception:  # library missing while formatting an error
        return "?"


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _finish(code: int, where: str, status: Optional[torch.Tensor], check: bool):
    if code != EV_OK:
        raise EvError(code, where)
    if check and status is not None:
        torch.cuda.current_stream(status.device).synchronize()
        dev_code = int(status.item())
        if dev_code != EV_OK:
            raise EvError(dev_code, where)


def _status_word(device, status):
    return torch.zeros(1, dtype=torch.int32, device=device) if status is None else status


class KvCache:
    """A KV cache layout plus the ctypes descriptor handed to the library.

    contiguous: k, v [B][Hkv][cap][d] (or [n_layers][B][Hkv][cap][d] with layered=True)
    paged:      k, v [n_blocks][Hkv][block_size][d] (or with a leading layer axis) and
                block_table int32 [B][max_blocks_per_seq]
    INT4:       k, v uint8 with d/2 bytes per row (two 4-bit values each) and k_scale,
                v_scale float32 of the same shape without the last axis.
    """

    def __init__(self, k: torch.Tensor, v: torch.Tensor, block_table: Optional[torch.Tensor] = None,
                 layered: bool = False, k_scale: Optional[torch.Tensor] = None,
                 v_scale: Optional[torch.Tensor] = None):
        _dev(k, "k")
        _dev(v, "v")
        if k.shape != v.shape or k.dtype != v.dtype:
            raise ValueError("k and v must have the same shape and dtype")
        if k.dtype == torch.float32:
            dtype = EV_F32
        elif k.dtype == torch.bfloat16:
            dtype = EV_BF16
        elif k.dtype == torch.uint8:
            dtype = EV_INT4
            _dev(k_scale, "k_scale", torch.float32)
            _dev(v_scale, "v_scale", torch.float32)
            if tuple(k_scale.shape) != tuple(k.shape[:-1]) or tuple(v_scale.shape) != tuple(k.shape[:-1]):
                raise ValueError("INT4 scales must have the cache's shape without its last axis")
        else:
            raise ValueError(f"unsupported KV dtype {k.dtype}")
        layer_shape = k.shape[1:] if layered else k.shape
        n_layers = k.shape[0] if layered else 1
        per_value = 2 if dtype == EV_INT4 else 1         # values per stored element
        layer_stride = k.stride(0) * per_value if layered else 0
        self.k, self.v, self.block_table, self.layered = k, v, block_table, layered
        self.k_scale, self.v_scale = k_scale, v_scale
        self.paged = block_table is not None
        d = layer_shape[-1] * per_value
        hkv = layer_shape[1]
        desc = EvKvDesc()
        desc.dtype, desc.n_kv_heads, desc.head_dim, desc.paged = dtype, hkv, d, int(self.paged)
        desc.k, desc.v = k.data_ptr(), v.data_ptr()
        desc.n_layers, desc.layer_stride = n_layers, layer_stride
        if dtype == EV_INT4:
            desc.k_scale, desc.v_scale = k_scale.data_ptr(), v_scale.data_ptr()
        if self.paged:
            _dev(block_table, "block_table", torch.int32)
            desc.cap = 0
            desc.block_table = block_table.data_ptr()
            desc.block_size = layer_shape[2]
            desc.max_blocks_per_seq = block_table.shape[1]
            desc.n_blocks = layer_shape[0]
        else:
            desc.cap = layer_shape[2]
            desc.block_table = None
            desc.block_size = desc.max_blocks_per_seq = desc.n_blocks = 0
        self.desc = desc
        # logical slots one sequence can hold
        self.capacity = (desc.max_blocks_per_seq * desc.block_size) if self.paged else desc.cap
        self.dtype = k.dtype
        self.n_kv_heads = hkv
        self.head_dim = d

    def ref(self):
        return ctypes.byref(self.desc)


def ev_tree_mask_build(parent: torch.Tensor, anc_mask: Optional[torch.Tensor] = None,
                       depth: Optional[torch.Tensor] = None, dev_status: Optional[torch.Tensor] = None,
                       check: bool = False):
    """Ancestor bitmasks (int64 view of uint64) and depths of parent[B][T]."""
    _dev(parent, "parent", torch.int32)
    B, T = parent.shape
    dev = parent.device
    anc_mask = torch.empty((B, T), dtype=torch.int64, device=dev) if anc_mask is None else anc_mask
    depth = torch.empty((B, T), dtype=torch.int32, device=dev) if depth is None else depth
    status = _status_word(dev, dev_status)
    code = lib().ev_tree_mask_build(_ptr(parent), B, T, _ptr(anc_mask), _ptr(depth), _ptr(status),
                                    _stream(dev))
    _finish(code, "ev_tree_mask_build", status, check)
    return anc_mask, depth


def ev_tree_attention_workspace(kv: KvCache, B: int, T: int, Hq: int,
                                max_prefix_len: Optional[int] = None) -> int:
    """Workspace bytes of ev_tree_attention; max_prefix_len defaults to what the cache holds."""
    mpl = kv.capacity - T if max_prefix_len is None else max_prefix_len
    return int(lib().ev_tree_attention_workspace(kv.ref(), B, T, Hq, max(0, int(mpl))))


def ev_tree_attention(q: torch.Tensor, kv: KvCache, prefix_len: torch.Tensor, anc_mask: torch.Tensor,
                      sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                      lse: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                      dev_status: Optional[torch.Tensor] = None, check: bool = False,
                      max_prefix_len: Optional[int] = None):
    """Tree-masked attention; returns (out [B][T][Hq][d], lse [B][T][Hq] float32).

    max_prefix_len: an upper bound of prefix_len (host int); the work is split over its
    key range, so pass the batch's longest prefix.  When omitted, the cache's capacity
    less T is used: always valid, but the split then spans the whole cache."""
    _dev(q, "q", torch.bfloat16 if kv.dtype == torch.uint8 else kv.dtype)
    _dev(prefix_len, "prefix_len", torch.int32)
    _dev(anc_mask, "anc_mask", torch.int64)
    B, T, Hq, d = q.shape
    dev = q.device
    if sm_scale is None:
        sm_scale = d ** -0.5
    mpl = max(0, kv.capacity - T) if max_prefix_len is None else int(max_prefix_len)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    need = ev_tree_attention_workspace(kv, B, T, Hq, mpl)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    status = _status_word(dev, dev_status)
    code = lib().ev_tree_attention(_ptr(q), kv.ref(), _ptr(prefix_len), _ptr(anc_mask), B, T, Hq,
                                   mpl, float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
                                   _ptr(status), _stream(dev))
    _finish(code, "ev_tree_attention", status, check)
    return out, lse


def ev_tree_mask_attention(q: torch.Tensor, kv: KvCache, prefix_len: torch.Tensor,
                           parent: torch.Tensor, sm_scale: Optional[float] = None,
                           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                           anc_mask: Optional[torch.Tensor] = None, depth: Optional[torch.Tensor] = None,
                           ws: Optional[torch.Tensor] = None, dev_status: Optional[torch.Tensor] = None,
                           check: bool = False, max_prefix_len: Optional[int] = None):
    """ev_tree_mask_build and ev_tree_attention in one call; returns (out, lse, anc_mask, depth).
    depth is only written when given (or returned as None)."""
    _dev(q, "q", torch.bfloat16 if kv.dtype == torch.uint8 else kv.dtype)
    _dev(prefix_len, "prefix_len", torch.int32)
    _dev(parent, "parent", torch.int32)
    B, T, Hq, d = q.shape
    dev = q.device
    if sm_scale is None:
        sm_scale = d ** -0.5
    mpl = max(0, kv.capacity - T) if max_prefix_len is None else int(max_prefix_len)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    anc_mask = torch.empty((B, T), dtype=torch.int64, device=dev) if anc_mask is None else anc_mask
    need = ev_tree_attention_workspace(kv, B, T, Hq, mpl)
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    status = _status_word(dev, dev_status)
    code = lib().ev_tree_mask_attention(_ptr(q), kv.ref(), _ptr(prefix_len), _ptr(parent),
                                        _ptr(anc_mask), _ptr(depth), B, T, Hq, mpl, float(sm_scale),
                                        _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _ptr(status),
                                        _stream(dev))
    _finish(code, "ev_tree_mask_attention", status, check)
    return out, lse, anc_mask, depth


def ev_tree_attention_noalloc(q: torch.Tensor, kv: KvCache, prefix_len: torch.Tensor,
                              anc_mask: torch.Tensor, sm_scale: Optional[float] = None,
                              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                              dev_status: Optional[torch.Tensor] = None, check: bool = False,
                              max_prefix_len: Optional[int] = None):
    """ev_tree_attention through the entry point that allocates nothing (its split partials
    live in the library's fixed per-GPU array).  Pass out, lse and dev_status to make the
    call itself allocation-free; otherwise they are allocated here."""
    _dev(q, "q", torch.bfloat16 if kv.dtype == torch.uint8 else kv.dtype)
    _dev(prefix_len, "prefix_len", torch.int32)
    _dev(anc_mask, "anc_mask", torch.int64)
    B, T, Hq, d = q.shape
    dev = q.device
    if sm_scale is None:
        sm_scale = d ** -0.5
    mpl = max(0, kv.capacity - T) if max_prefix_len is None else int(max_prefix_len)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=dev) if lse is None else lse
    status = _status_word(dev, dev_status)
    code = lib().ev_tree_attention_noalloc(_ptr(q), kv.ref(), _ptr(prefix_len), _ptr(anc_mask), B, T,
                                           Hq, mpl, float(sm_scale), _ptr(out), _ptr(lse),
                                           _ptr(status), _stream(dev))
    _finish(code, "ev_tree_attention_noalloc", status, check)
    return out, lse


def ev_tree_attention_noalloc_limit() -> int:
    return int(lib().ev_tree_attention_noalloc_limit())


def ev_accept_workspace(B: int, T: int, V: int) -> int:
    return int(lib().ev_accept_workspace(B, T, V))


def _accept_outputs(B, T, dev, accept_len, path, out_tokens):
    accept_len = torch.empty(B, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    path = torch.empty((B, T), dtype=torch.int32, device=dev) if path is None else path
    out_tokens = torch.empty((B, T), dtype=torch.int32, device=dev) if out_tokens is None else out_tokens
    return accept_len, path, out_tokens


def ev_accept_greedy(logits: torch.Tensor, tokens: torch.Tensor, parent: torch.Tensor,
                     accept_len=None, path=None, out_tokens=None, ws=None, dev_status=None,
                     check: bool = False):
    """Greedy acceptance; returns (accept_len [B], path [B][T], out_tokens [B][T])."""
    _dev(logits, "logits", torch.float32)
    _dev(tokens, "tokens", torch.int32)
    _dev(parent, "parent", torch.int32)
    B, T, V = logits.shape
    dev = logits.device
    accept_len, path, out_tokens = _accept_outputs(B, T, dev, accept_len, path, out_tokens)
    if ws is None:
        ws = torch.zeros(max(1, ev_accept_workspace(B, T, V)), dtype=torch.uint8, device=dev)
    status = _status_word(dev, dev_status)
    code = lib().ev_accept_greedy(_ptr(logits), _ptr(tokens), _ptr(parent), B, T, V, _ptr(accept_len),
                                  _ptr(path), _ptr(out_tokens), _ptr(ws), ws.numel() * ws.element_size(),
                                  _ptr(status), _stream(dev))
    _finish(code, "ev_accept_greedy", status, check)
    return accept_len, path, out_tokens


def ev_accept_rejection(logits: torch.Tensor, tokens: torch.Tensor, parent: torch.Tensor,
                        temperature: float, uniforms: torch.Tensor, accept_len=None, path=None,
                        out_tokens=None, ws=None, dev_status=None, check: bool = False):
    """Rejection-sampling acceptance; returns (accept_len, path, out_tokens)."""
    _dev(logits, "logits", torch.float32)
    _dev(tokens, "tokens", torch.int32)
    _dev(parent, "parent", torch.int32)
    _dev(uniforms, "uniforms", torch.float64)
    B, T, V = logits.shape
    dev = logits.device
    accept_len, path, out_tokens = _accept_outputs(B, T, dev, accept_len, path, out_tokens)
    if ws is None:
        ws = torch.zeros(max(1, ev_accept_workspace(B, T, V)), dtype=torch.uint8, device=dev)
    status = _status_word(dev, dev_status)
    code = lib().ev_accept_rejection(_ptr(logits), _ptr(tokens), _ptr(parent), B, T, V,
                                     float(temperature), _ptr(uniforms), _ptr(accept_len), _ptr(path),
                                     _ptr(out_tokens), _ptr(ws), ws.numel() * ws.element_size(),
                                     _ptr(status), _stream(dev))
    _finish(code, "ev_accept_rejection", status, check)
    return accept_len, path, out_tokens


def ev_accept_greedy_compact(logits: torch.Tensor, tokens: torch.Tensor, parent: torch.Tensor,
                             kv: KvCache, prefix_len: torch.Tensor, accept_len=None, path=None,
                             out_tokens=None, new_len=None, ws=None, dev_status=None,
                             check: bool = False):
    """Greedy acceptance and compaction of each accepted path in one call; returns
    (accept_len, path, out_tokens, new_len)."""
    return _accept_compact(False, logits, tokens, parent, None, None, kv, prefix_len, accept_len,
                           path, out_tokens, new_len, ws, dev_status, check)


def ev_accept_rejection_compact(logits: torch.Tensor, tokens: torch.Tensor, parent: torch.Tensor,
                                temperature: float, uniforms: torch.Tensor, kv: KvCache,
                                prefix_len: torch.Tensor, accept_len=None, path=None,
                                out_tokens=None, new_len=None, ws=None, dev_status=None,
                                check: bool = False):
    """Rejection acceptance and compaction of each accepted path in one call; returns
    (accept_len, path, out_tokens, new_len)."""
    return _accept_compact(True, logits, tokens, parent, temperature, uniforms, kv, prefix_len,
                           accept_len, path, out_tokens, new_len, ws, dev_status, check)


def _accept_compact(rej, logits, tokens, parent, temperature, uniforms, kv, prefix_len, accept_len,
                    path, out_tokens, new_len, ws, dev_status, check):
    _dev(logits, "logits", torch.float32)
    _dev(tokens, "tokens", torch.int32)
    _dev(parent, "parent", torch.int32)
    _dev(prefix_len, "prefix_len", torch.int32)
    B, T, V = logits.shape
    dev = logits.device
    accept_len, path, out_tokens = _accept_outputs(B, T, dev, accept_len, path, out_tokens)
    new_len = torch.empty(B, dtype=torch.int32, device=dev) if new_len is None else new_len
    if ws is None:
        ws = torch.zeros(max(1, ev_accept_workspace(B, T, V)), dtype=torch.uint8, device=dev)
    status = _status_word(dev, dev_status)
    ws_bytes = ws.numel() * ws.element_size()
    if rej:
        _dev(uniforms, "uniforms", torch.float64)
        name = "ev_accept_rejection_compact"
        code = lib().ev_accept_rejection_compact(
            _ptr(logits), _ptr(tokens), _ptr(parent), B, T, V, float(temperature), _ptr(uniforms),
            _ptr(accept_len), _ptr(path), _ptr(out_tokens), kv.ref(), _ptr(prefix_len),
            _ptr(new_len), _ptr(ws), ws_bytes, _ptr(status), _stream(dev))
    else:
        name = "ev_accept_greedy_compact"
        code = lib().ev_accept_greedy_compact(
            _ptr(logits), _ptr(tokens), _ptr(parent), B, T, V, _ptr(accept_len), _ptr(path),
            _ptr(out_tokens), kv.ref(), _ptr(prefix_len), _ptr(new_len), _ptr(ws), ws_bytes,
            _ptr(status), _stream(dev))
    _finish(code, name, status, check)
    return accept_len, path, out_tokens, new_len


def ev_accept_sampled_workspace(B: int, T: int, V: int) -> int:
    return int(lib().ev_accept_sampled_workspace(B, T, V))


def ev_accept_sampled(logits: torch.Tensor, draft_logits: torch.Tensor, tokens: torch.Tensor,
                      parent: torch.Tensor, temperature: float, draft_temperature: float,
                      uniforms: torch.Tensor, max_children: int, accept_len=None, path=None,
                      out_tokens=None, ws=None, dev_status=None, check: bool = False):
    """Acceptance of drafts sampled from a draft distribution; returns
    (accept_len, path, out_tokens).  ws must be zero-filled before its first use."""
    _dev(logits, "logits", torch.float32)
    _dev(draft_logits, "draft_logits", torch.float32)
    _dev(tokens, "tokens", torch.int32)
    _dev(parent, "parent", torch.int32)
    _dev(uniforms, "uniforms", torch.float64)
    B, T, V = logits.shape
    if tuple(draft_logits.shape) != (B, T, V):
        raise ValueError("draft_logits must have the shape of logits")
    dev = logits.device
    accept_len, path, out_tokens = _accept_outputs(B, T, dev, accept_len, path, out_tokens)
    if ws is None:
        ws = torch.zeros(max(1, ev_accept_sampled_workspace(B, T, V)), dtype=torch.uint8, device=dev)
    status = _status_word(dev, dev_status)
    code = lib().ev_accept_sampled(_ptr(logits), _ptr(draft_logits), _ptr(tokens), _ptr(parent),
                                   B, T, V, float(temperature), float(draft_temperature),
                                   _ptr(uniforms), int(max_children), _ptr(accept_len), _ptr(path),
                                   _ptr(out_tokens), _ptr(ws), ws.numel() * ws.element_size(),
                                   _ptr(status), _stream(dev))
    _finish(code, "ev_accept_sampled", status, check)
    return accept_len, path, out_tokens


def ev_kv_compact(kv: KvCache, prefix_len: torch.Tensor, path: torch.Tensor, accept_len: torch.Tensor,
                  new_len: Optional[torch.Tensor] = None, dev_status=None, check: bool = False):
    """Move the accepted path's KV next to the prefix in place; returns new_len [B]."""
    _dev(prefix_len, "prefix_len", torch.int32)
    _dev(path, "path", torch.int32)
    _dev(accept_len, "accept_len", torch.int32)
    B, T = path.shape
    dev = path.device
    new_len = torch.empty(B, dtype=torch.int32, device=dev) if new_len is None else new_len
    status = _status_word(dev, dev_status)
    code = lib().ev_kv_compact(kv.ref(), _ptr(prefix_len), _ptr(path), _ptr(accept_len), B, T,
                               _ptr(new_len), _ptr(status), _stream(dev))
    _finish(code, "ev_kv_compact", status, check)
    return new_len


def ev_kv_compact_remap_workspace(B: int) -> int:
    return int(lib().ev_kv_compact_remap_workspace(B))


def ev_kv_compact_remap(kv: "KvCache", prefix_len: torch.Tensor, path: torch.Tensor,
                        accept_len: torch.Tensor, new_len=None, freed=None, freed_count=None,
                        copied=None, ws=None, dev_status=None, check: bool = False):
    """Zero-copy pruning of a paged cache: remaps kv's block table in place (copying rows
    only where the moves do not fill aligned blocks); returns (new_len [B], freed
    [B][max_blocks_per_seq], freed_count [B], copied [B])."""
    _dev(prefix_len, "prefix_len", torch.int32)
    _dev(path, "path", torch.int32)
    _dev(accept_len, "accept_len", torch.int32)
    if kv.block_table is None:
        raise ValueError("ev_kv_compact_remap needs a paged cache")
    B, T = path.shape
    dev = path.device
    e = lambda *s: torch.empty(s, dtype=torch.int32, device=dev)
    new_len = e(B) if new_len is None else new_len
    freed = e(B, kv.block_table.shape[1]) if freed is None else freed
    freed_count = e(B) if freed_count is None else freed_count
    copied = e(B) if copied is None else copied
    if ws is None:
        ws = torch.empty(max(1, ev_kv_compact_remap_workspace(B)), dtype=torch.uint8, device=dev)
    status = _status_word(dev, dev_status)
    code = lib().ev_kv_compact_remap(kv.ref(), _ptr(prefix_len), _ptr(path), _ptr(accept_len), B, T,
                                     _ptr(new_len), _ptr(freed), _ptr(freed_count), _ptr(copied),
                                     _ptr(ws), ws.numel(), _ptr(status), _stream(dev))
    _finish(code, "ev_kv_compact_remap", status, check)
    return new_len, freed, freed_count, copied


def ev_draft_tree_workspace(B: int, beam: int, V: int) -> int:
    return int(lib().ev_draft_tree_workspace(B, beam, V))


def ev_draft_tree_expand(draft_logits: torch.Tensor, depth: int, temperature: float, k_max: int,
                         ws: torch.Tensor, frontier_tokens=None, frontier_slots=None,
                         frontier_count=None, dev_status=None, check: bool = False):
    """One depth of the draft-tree beam expansion over draft_logits [B][beam][V]; returns
    the next frontier (tokens [B][beam], parent slots [B][beam], counts [B]).  ws carries
    the tree between calls (zero-filled before the first tree, one tree at a time)."""
    _dev(draft_logits, "draft_logits", torch.float32)
    _dev(ws, "ws", torch.uint8)
    B, W, V = draft_logits.shape
    dev = draft_logits.device
    if frontier_tokens is None:
        frontier_tokens = torch.empty((B, W), dtype=torch.int32, device=dev)
    if frontier_slots is None:
        frontier_slots = torch.empty((B, W), dtype=torch.int32, device=dev)
    if frontier_count is None:
        frontier_count = torch.empty(B, dtype=torch.int32, device=dev)
    status = _status_word(dev, dev_status)
    code = lib().ev_draft_tree_expand(_ptr(draft_logits), B, W, V, int(depth), float(temperature),
                                      int(k_max), _ptr(frontier_tokens), _ptr(frontier_slots),
                                      _ptr(frontier_count), _ptr(ws), ws.numel(), _ptr(status),
                                      _stream(dev))
    _finish(code, "ev_draft_tree_expand", status, check)
    return frontier_tokens, frontier_slots, frontier_count


def ev_draft_tree_finalize(root_tokens: torch.Tensor, beam: int, V: int, n_nodes: int,
                           ws: torch.Tensor, parent=None, tokens=None, tree_size=None):
    """The tree after the expansions so far; returns (parent [B][n_nodes], tokens
    [B][n_nodes], tree_size [B])."""
    _dev(root_tokens, "root_tokens", torch.int32)
    _dev(ws, "ws", torch.uint8)
    B = root_tokens.shape[0]
    dev = root_tokens.device
    if parent is None:
        parent = torch.empty((B, n_nodes), dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, n_nodes), dtype=torch.int32, device=dev)
    if tree_size is None:
        tree_size = torch.empty(B, dtype=torch.int32, device=dev)
    code = lib().ev_draft_tree_finalize(_ptr(root_tokens), B, int(beam), int(V), int(n_nodes),
                                        _ptr(parent), _ptr(tokens), _ptr(tree_size), _ptr(ws),
                                        ws.numel(), _stream(dev))
    _finish(code, "ev_draft_tree_finalize", None, False)
    return parent, tokens, tree_size


def ev_status_string(code: int) -> str:
    return lib().ev_status_string(code).decode()


def ev_peak_mfma_bf16(n_workgroups: int, iters: int, sink: torch.Tensor) -> None:
    """Enqueue the bf16 matrix-core loop (n_workgroups * 4 * iters * 4 * 32768 flops)."""
    _dev(sink, "sink", torch.float32)
    if sink.numel() < n_workgroups:
        raise ValueError("sink needs one float per workgroup")
    _finish(lib().ev_peak_mfma_bf16(n_workgroups, iters, sink.data_ptr(), _stream(sink.device)),
            "ev_peak_mfma_bf16", None, False)


def ev_peak_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    """Enqueue a copy of src's bytes into dst (16-byte pieces)."""
    _dev(src, "src")
    _dev(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    _finish(lib().ev_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream(src.device)),
            "ev_peak_copy", None, False)


def ev_peak_read(src: torch.Tensor, sink: torch.Tensor) -> None:
    """Enqueue a read of src's bytes by sink.numel() workgroups (one uint32 each into sink)."""
    _dev(src, "src")
    _dev(sink, "sink", torch.int32)
    _finish(lib().ev_peak_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(),
                               sink.numel(), _stream(src.device)), "ev_peak_read", None, False)


__all__ = ["KvCache", "EvError", "EvKvDesc", "lib", "LIB_PATH", *EXPORTED, *EXPORTED_PEAKS]
