"""Python binding of libddt (ctypes).  Argument marshalling only: every step
of the chain runs in the HIP kernels behind the C ABI declared in
include/ddt.h.  PyTorch provides device memory and the current stream.

The library must be built (``python -m block_diffusion_draft_vocab_amd.build``);
loading fails loudly otherwise -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libddt.so")
_lib = None

DDT_OK, DDT_EINVAL, DDT_EUNSUPPORTED, DDT_EWORKSPACE, DDT_ELAUNCH = range(5)

_c = ctypes
_P = _c.c_void_p
_I = _c.c_int
_I64 = _c.c_int64
_F = _c.c_float
_SZ = _c.c_size_t

# exported symbol -> (restype, argtypes)
SIGNATURES = {
    "ddt_abi_version": (_I, []),
    "ddt_status_string": (_c.c_char_p, [_I]),
    "ddt_topk_logprobs_workspace_size": (_SZ, [_I, _I, _I]),
    "ddt_topk_logprobs": (_I, [_P, _I64, _I, _I, _I, _F, _P, _P, _P, _P, _SZ, _P]),
    "ddt_topk_logprobs_noalloc": (_I, [_P, _I64, _I, _I, _I, _F, _P, _P, _P, _P]),
    "ddt_lmhead_topk_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "ddt_lmhead_topk": (_I, [_P, _P, _I, _I, _I, _I, _F, _P, _P, _P, _P, _SZ, _P]),
    "ddt_tree_rope_kv": (_I, [_P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _F, _P,
                              _P]),
    "ddt_argmax_workspace_size": (_SZ, [_I, _I]),
    "ddt_argmax": (_I, [_P, _I64, _I, _I, _P, _P, _P, _SZ, _P]),
    "ddt_build_tree_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "ddt_build_tree": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "ddt_masked_attention_workspace_size": (_SZ, [_P]),
    "ddt_masked_attention": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "ddt_packed_block_attention": (_I, [_P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "ddt_accept_compact": (_I, [_P, _P, _P, _I, _P, _I, _I, _P, _P, _P, _P, _I, _I64, _I, _I,
                                _P, _P, _P, _P, _P]),
}


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", _I), ("hq", _I), ("hkv", _I), ("head_dim", _I), ("n_q_max", _I),
                ("mask_words", _I), ("max_kv_len", _I), ("scale", _F)]


class DdtError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load().ddt_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} returned {status} ({msg})")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libddt.so once; raise if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -m block_diffusion_draft_vocab_amd.build` (no CPU fallback exists)")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(fn: str, status: int) -> None:
    if status != DDT_OK:
        raise DdtError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _on_stream(fn):
    """Run an entry point with ``stream=`` as torch's current stream, so the
    outputs and the workspace it allocates belong to the stream its kernels
    run on (the caching allocator then cannot hand their blocks to other
    work before those kernels finish)."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, **kw)
    return wrapper


def _need(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError("workspace too small")
    return ws, ws.numel() * ws.element_size()


# ---------------------------------------------------------------- stage 1
def topk_workspace_size(n_rows: int, vocab: int, k: int) -> int:
    return int(load().ddt_topk_logprobs_workspace_size(n_rows, vocab, k))


@_on_stream
def topk_logprobs(logits: torch.Tensor, k: int, inv_temperature: float = 1.0, *,
                  vocab: Optional[int] = None, ids=None, logp=None, lse=None, workspace=None,
                  want_lse: bool = True):
    lib = load()
    if logits.dim() != 2 or logits.dtype != torch.float32 or not logits.is_cuda:
        raise ValueError("logits must be a device float32 [rows, ld] tensor")
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    rows, ld = logits.shape[0], logits.stride(0)
    vocab = logits.shape[1] if vocab is None else vocab
    dev = logits.device
    ids = torch.empty(rows, k, dtype=torch.int32, device=dev) if ids is None else ids
    logp = torch.empty(rows, k, dtype=torch.float32, device=dev) if logp is None else logp
    if want_lse and lse is None:
        lse = torch.empty(rows, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(topk_workspace_size(rows, vocab, k), dev, workspace)
    st = lib.ddt_topk_logprobs(_ptr(logits), ld, rows, vocab, k, float(inv_temperature),
                               _ptr(ids), _ptr(logp), _ptr(lse), _ptr(ws), wsb, _stream())
    _check("ddt_topk_logprobs", st)
    return ids, logp, lse


@_on_stream
def topk_logprobs_noalloc(logits: torch.Tensor, k: int, inv_temperature: float = 1.0, *,
                          vocab: Optional[int] = None, ids=None, logp=None, lse=None,
                          want_lse: bool = True):
    """topk_logprobs through ddt_topk_logprobs_noalloc: the library's own
    per-device scratch instead of a workspace (outputs still allocated here
    unless given)."""
    lib = load()
    if logits.dim() != 2 or logits.dtype != torch.float32 or not logits.is_cuda:
        raise ValueError("logits must be a device float32 [rows, ld] tensor")
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    rows, ld = logits.shape[0], logits.stride(0)
    vocab = logits.shape[1] if vocab is None else vocab
    dev = logits.device
    ids = torch.empty(rows, k, dtype=torch.int32, device=dev) if ids is None else ids
    logp = torch.empty(rows, k, dtype=torch.float32, device=dev) if logp is None else logp
    if want_lse and lse is None:
        lse = torch.empty(rows, dtype=torch.float32, device=dev)
    st = lib.ddt_topk_logprobs_noalloc(_ptr(logits), ld, rows, vocab, k, float(inv_temperature),
                                       _ptr(ids), _ptr(logp), _ptr(lse), _stream())
    _check("ddt_topk_logprobs_noalloc", st)
    return ids, logp, lse


# ---------------------------------------------------------------- fused LM head
def lmhead_topk_workspace_size(n_rows: int, hidden: int, vocab: int, k: int) -> int:
    return int(load().ddt_lmhead_topk_workspace_size(n_rows, hidden, vocab, k))


@_on_stream
def lmhead_topk(hidden_states: torch.Tensor, weight: torch.Tensor, k: int,
                inv_temperature: float = 1.0, *, ids=None, logp=None, lse=None, workspace=None,
                want_lse: bool = True):
    """Top-k ids / log-probs of softmax(inv_temperature * hidden_states . weight^T)
    per row, without materialising the logits.  hidden_states bf16 [rows, hidden],
    weight bf16 [vocab, hidden] (the LM head), both contiguous on the device."""
    lib = load()
    _need(hidden_states, torch.bfloat16, "hidden_states")
    _need(weight, torch.bfloat16, "weight")
    if hidden_states.dim() != 2 or weight.dim() != 2 or hidden_states.shape[1] != weight.shape[1]:
        raise ValueError("need hidden_states [rows, hidden] and weight [vocab, hidden]")
    rows, hidden = hidden_states.shape
    vocab = weight.shape[0]
    dev = hidden_states.device
    ids = torch.empty(rows, k, dtype=torch.int32, device=dev) if ids is None else ids
    logp = torch.empty(rows, k, dtype=torch.float32, device=dev) if logp is None else logp
    if want_lse and lse is None:
        lse = torch.empty(rows, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(lmhead_topk_workspace_size(rows, hidden, vocab, k), dev, workspace)
    st = lib.ddt_lmhead_topk(_ptr(hidden_states), _ptr(weight), rows, hidden, vocab, k,
                             float(inv_temperature), _ptr(ids), _ptr(logp), _ptr(lse), _ptr(ws),
                             wsb, _stream())
    _check("ddt_lmhead_topk", st)
    return ids, logp, lse


# ---------------------------------------------------------------- tree RoPE + KV
@_on_stream
def tree_rope_kv(node_depth: torch.Tensor, n_nodes: torch.Tensor, prefix_len: torch.Tensor,
                 kv_base: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                 v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 rope_base: float = 1.0e6, *, positions=None, want_positions: bool = True):
    """Positions P + depth for the tree slots, rotary embedding of q (in place)
    and of the new k, and the scatter of k / v into the cache rows P + slot.
    Returns positions i32 [batch, n_max] (or None)."""
    lib = load()
    _need(node_depth, torch.int32, "node_depth")
    _need(n_nodes, torch.int32, "n_nodes")
    _need(prefix_len, torch.int32, "prefix_len")
    _need(kv_base, torch.int64, "kv_base")
    for t, nm in ((q, "q"), (k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"),
                  (v_cache, "v_cache")):
        _need(t, torch.bfloat16, nm)
    batch, n_max, hq, D = q.shape
    hkv = k_new.shape[2]
    if tuple(k_new.shape) != (batch, n_max, hkv, D) or tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("k_new / v_new must be [batch, n_max, hkv, D]")
    if k_cache.shape[-2:] != (hkv, D) or v_cache.shape[-2:] != (hkv, D):
        raise ValueError("caches must be [rows, hkv, D]")
    if want_positions and positions is None:
        positions = torch.empty(batch, n_max, dtype=torch.int32, device=q.device)
    st = lib.ddt_tree_rope_kv(_ptr(node_depth), _ptr(n_nodes), batch, n_max, _ptr(prefix_len),
                              _ptr(kv_base), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                              _ptr(v_cache), hq, hkv, D, float(rope_base), _ptr(positions),
                              _stream())
    _check("ddt_tree_rope_kv", st)
    return positions


# ---------------------------------------------------------------- target argmax
def argmax_workspace_size(n_rows: int, vocab: int) -> int:
    return int(load().ddt_argmax_workspace_size(n_rows, vocab))


@_on_stream
def argmax(logits: torch.Tensor, *, vocab: Optional[int] = None, ids=None, maxv=None,
           want_max: bool = False, workspace=None):
    """Per-row arg-max (smallest id among the maxima) of device float32 logits.
    Returns (ids i32 [rows], max f32 [rows] or None)."""
    lib = load()
    if logits.dim() != 2 or logits.dtype != torch.float32 or not logits.is_cuda:
        raise ValueError("logits must be a device float32 [rows, ld] tensor")
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    rows, ld = logits.shape[0], logits.stride(0)
    vocab = logits.shape[1] if vocab is None else vocab
    dev = logits.device
    ids = torch.empty(rows, dtype=torch.int32, device=dev) if ids is None else ids
    if want_max and maxv is None:
        maxv = torch.empty(rows, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(argmax_workspace_size(rows, vocab), dev, workspace)
    st = lib.ddt_argmax(_ptr(logits), ld, rows, vocab, _ptr(ids), _ptr(maxv), _ptr(ws), wsb,
                        _stream())
    _check("ddt_argmax", st)
    return ids, maxv


# ---------------------------------------------------------------- stage 2
@_on_stream
def build_tree(topk_logp: torch.Tensor, topk_ids: torch.Tensor, root_token: torch.Tensor,
               batch: int, L: int, k_tree: int, budget: int, *, out=None, want_score=True):
    lib = load()
    _need(topk_logp, torch.float32, "topk_logp")
    _need(topk_ids, torch.int32, "topk_ids")
    _need(root_token, torch.int32, "root_token")
    k = topk_logp.shape[1]
    if topk_logp.shape[0] != batch * L or topk_ids.shape != topk_logp.shape:
        raise ValueError("top-K tables must be [batch*L, k]")
    n_max = budget + 1
    W = (n_max + 63) // 64
    dev = topk_logp.device
    if out is None:
        out = {
            "n_nodes": torch.empty(batch, dtype=torch.int32, device=dev),
            "token": torch.empty(batch, n_max, dtype=torch.int32, device=dev),
            "parent": torch.empty(batch, n_max, dtype=torch.int32, device=dev),
            "depth": torch.empty(batch, n_max, dtype=torch.int32, device=dev),
            "score": torch.empty(batch, n_max, dtype=torch.float32, device=dev) if want_score else None,
            "mask": torch.empty(batch, n_max, W, dtype=torch.int64, device=dev),
        }
    st = lib.ddt_build_tree(_ptr(topk_logp), _ptr(topk_ids), _ptr(root_token), batch, L, k,
                            k_tree, budget, _ptr(out["n_nodes"]), _ptr(out["token"]),
                            _ptr(out["parent"]), _ptr(out["depth"]), _ptr(out.get("score")),
                            _ptr(out["mask"]), None, 0, _stream())
    _check("ddt_build_tree", st)
    return out


# ---------------------------------------------------------------- stage 3
def attn_desc(batch, hq, hkv, head_dim, n_q_max, max_kv_len, mask_words=0, scale=0.0):
    return AttnDesc(batch, hq, hkv, head_dim, n_q_max, mask_words, max_kv_len, scale)


def attention_workspace_size(desc: AttnDesc) -> int:
    return int(load().ddt_masked_attention_workspace_size(ctypes.byref(desc)))


@_on_stream
def masked_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                     kv_base: torch.Tensor, prefix_len: torch.Tensor, n_q: torch.Tensor,
                     own_mask: Optional[torch.Tensor] = None, *, max_kv_len: int,
                     scale: float = 0.0, out=None, lse=None, want_lse=False, workspace=None,
                     block_len: int = 0):
    """q bf16 [b, n_q_max, hq, D]; k/v bf16 [rows, hkv, D]; own_mask int64
    [b, n_q_max, W] (bit patterns) or None for the dense drafter block.
    block_len > 0 (no mask): packed drafter blocks, each query sees the prefix
    and only its own block of block_len own rows."""
    lib = load()
    _need(q, torch.bfloat16, "q")
    _need(k_cache, torch.bfloat16, "k_cache")
    _need(v_cache, torch.bfloat16, "v_cache")
    _need(kv_base, torch.int64, "kv_base")
    _need(prefix_len, torch.int32, "prefix_len")
    _need(n_q, torch.int32, "n_q")
    b, n_q_max, hq, D = q.shape
    hkv = k_cache.shape[1]
    W = 0
    if own_mask is not None:
        _need(own_mask, torch.int64, "own_mask")
        W = own_mask.shape[2]
    desc = attn_desc(b, hq, hkv, D, n_q_max, max_kv_len, W, scale)
    out = torch.empty_like(q) if out is None else out
    if want_lse and lse is None:
        lse = torch.empty(b, n_q_max, hq, dtype=torch.float32, device=q.device)
    ws, wsb = _workspace(attention_workspace_size(desc), q.device, workspace)
    if block_len:
        if own_mask is not None:
            raise ValueError("block_len and own_mask are exclusive")
        st = lib.ddt_packed_block_attention(ctypes.byref(desc), int(block_len), _ptr(q),
                                            _ptr(k_cache), _ptr(v_cache), _ptr(kv_base),
                                            _ptr(prefix_len), _ptr(n_q), _ptr(out), _ptr(lse),
                                            _ptr(ws), wsb, _stream())
        _check("ddt_packed_block_attention", st)
        return (out, lse) if want_lse else out
    st = lib.ddt_masked_attention(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(kv_base), _ptr(prefix_len), _ptr(n_q), _ptr(own_mask),
                                  _ptr(out), _ptr(lse), _ptr(ws), wsb, _stream())
    _check("ddt_masked_attention", st)
    return (out, lse) if want_lse else out


# ---------------------------------------------------------------- stage 4
@_on_stream
def accept_compact(node_token: torch.Tensor, node_parent: torch.Tensor, n_nodes: torch.Tensor,
                   target: torch.Tensor, L: int, k_cache: Optional[torch.Tensor],
                   v_cache: Optional[torch.Tensor], kv_base: Optional[torch.Tensor],
                   prefix_len: torch.Tensor, *, n_layers: Optional[int] = None,
                   layer_stride: Optional[int] = None, hkv: Optional[int] = None,
                   head_dim: Optional[int] = None, out=None):
    """k_cache/v_cache bf16 [n_layers, rows, hkv, D] (edited in place) or None."""
    lib = load()
    for t, nm in ((node_token, "node_token"), (node_parent, "node_parent"),
                  (n_nodes, "n_nodes"), (target, "target"), (prefix_len, "prefix_len")):
        _need(t, torch.int32, nm)
    batch, n_max = node_token.shape
    if k_cache is not None:
        _need(k_cache, torch.bfloat16, "k_cache")
        _need(v_cache, torch.bfloat16, "v_cache")
        _need(kv_base, torch.int64, "kv_base")
        n_layers = k_cache.shape[0] if n_layers is None else n_layers
        layer_stride = k_cache.stride(0) if layer_stride is None else layer_stride
        hkv = k_cache.shape[2] if hkv is None else hkv
        head_dim = k_cache.shape[3] if head_dim is None else head_dim
    else:
        n_layers, layer_stride = 0, 0
        hkv = hkv or 1
        head_dim = head_dim or 8
    dev = node_token.device
    if out is None:
        out = {
            "accept_len": torch.empty(batch, dtype=torch.int32, device=dev),
            "accepted": torch.empty(batch, L + 1, dtype=torch.int32, device=dev),
            "bonus": torch.empty(batch, dtype=torch.int32, device=dev),
            "new_len": torch.empty(batch, dtype=torch.int32, device=dev),
        }
    st = lib.ddt_accept_compact(_ptr(node_token), _ptr(node_parent), _ptr(n_nodes), n_max,
                                _ptr(target), batch, L, _ptr(k_cache), _ptr(v_cache),
                                _ptr(kv_base), _ptr(prefix_len), n_layers, layer_stride, hkv,
                                head_dim, _ptr(out["accept_len"]), _ptr(out["accepted"]),
                                _ptr(out["bonus"]), _ptr(out["new_len"]), _stream())
    _check("ddt_accept_compact", st)
    return out
