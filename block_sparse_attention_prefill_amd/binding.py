"""ctypes binding of libseer.so: the C-ABI of include/seer.h with the same names.

Argument marshalling only -- every step of the path runs in the HIP library.
Torch tensors provide device memory and the current HIP stream.  If the
library is missing the calls raise instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libseer.so")

SEER_OK = 0
SEER_MASK_THRESHOLD = 0
SEER_MASK_TOPK = 1
BLOCK = 64

EXPORTED = (
    "seer_status_string", "seer_version", "seer_topk_budget", "seer_build_mask",
    "seer_sparse_prefill_workspace_size", "seer_sparse_prefill", "seer_sparse_prefill_block",
    "seer_pooled_attn_map_workspace_size", "seer_pooled_attn_map", "seer_pooled_target_mse",
    "seer_attn_gate_workspace_size", "seer_attn_gate_scores", "seer_attn_gate_mask_workspace_size",
    "seer_attn_gate_mask_pass_workspace_size",
    "seer_attn_gate_mask", "seer_attn_gate_decode_keys_workspace_size", "seer_attn_gate_decode_keys",
    "seer_attn_gate_decode_scores", "seer_attn_gate_decode_mask", "seer_build_mask_decode",
    "seer_sparse_decode_workspace_size", "seer_sparse_decode", "seer_build_mask_need",
    "seer_validate_lists", "seer_list_flags_status", "seer_sparse_prefill_noalloc",
)

SEER_LIST_BAD_COUNT = 1
SEER_LIST_BAD_ENTRY = 2
SEER_LIST_REPEAT = 4
SEER_LIST_UNSORTED = 8
SEER_LIST_CAPACITY = 16

_lib = None


class SeerError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libseer.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m block_sparse_attention_prefill_amd.build`"
            " (there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    c_int, c_float, c_double, c_size, c_void = (ctypes.c_int, ctypes.c_float, ctypes.c_double,
                                                ctypes.c_size_t, ctypes.c_void_p)
    lib.seer_status_string.restype = ctypes.c_char_p
    lib.seer_status_string.argtypes = [c_int]
    lib.seer_version.restype = c_int
    lib.seer_version.argtypes = []
    lib.seer_topk_budget.restype = c_int
    lib.seer_topk_budget.argtypes = [c_int, c_double, c_int]
    lib.seer_build_mask.restype = c_int
    lib.seer_build_mask.argtypes = [c_void, c_int, c_int, c_int, c_int, c_int, c_float, c_double,
                                    c_int, c_void, c_void, c_int, c_void]
    lib.seer_build_mask_need.restype = c_int
    lib.seer_build_mask_need.argtypes = [c_void, c_int, c_int, c_int, c_int, c_int, c_float,
                                         c_double, c_int, c_void, c_void, c_void, c_int, c_void]
    lib.seer_validate_lists.restype = c_int
    lib.seer_validate_lists.argtypes = [c_void, c_void, c_void, c_int, c_int, c_int, c_int,
                                        c_void, c_void, c_void]
    lib.seer_sparse_prefill_noalloc.restype = c_int
    lib.seer_sparse_prefill_noalloc.argtypes = [c_void, c_void, c_void, c_int, c_int, c_int, c_int,
                                                c_int, c_float, c_void, c_void, c_int, c_void,
                                                c_void]
    lib.seer_list_flags_status.restype = c_int
    lib.seer_list_flags_status.argtypes = [c_int]
    lib.seer_sparse_prefill_workspace_size.restype = c_size
    lib.seer_sparse_prefill_workspace_size.argtypes = [c_int, c_int, c_int, c_int]
    lib.seer_sparse_prefill.restype = c_int
    lib.seer_sparse_prefill.argtypes = [c_void, c_void, c_void, c_int, c_int, c_int, c_int, c_int,
                                        c_float, c_void, c_void, c_int, c_void, c_void, c_size,
                                        c_void]
    lib.seer_sparse_prefill_block.restype = c_int
    lib.seer_sparse_prefill_block.argtypes = [c_void, c_void, c_void, c_int, c_int, c_int, c_int,
                                              c_int, c_float, c_int, c_void, c_void, c_int,
                                              c_void, c_void, c_size, c_void]
    lib.seer_pooled_attn_map_workspace_size.restype = c_size
    lib.seer_pooled_attn_map_workspace_size.argtypes = [c_int, c_int, c_int]
    lib.seer_pooled_attn_map.restype = c_int
    lib.seer_pooled_attn_map.argtypes = [c_void, c_void, c_void, c_int, c_int, c_int, c_int, c_int,
                                         c_float, c_void, c_void, c_void, c_size, c_void]
    lib.seer_attn_gate_workspace_size.restype = c_size
    lib.seer_attn_gate_workspace_size.argtypes = [c_int, c_int, c_int, c_int, c_int]
    lib.seer_attn_gate_scores.restype = c_int
    lib.seer_attn_gate_scores.argtypes = [c_void, c_void, c_int, c_int, c_int, c_int, c_int,
                                          c_void, c_void, c_int, c_float, c_float, c_void,
                                          c_void, c_size, c_void]
    lib.seer_attn_gate_mask_workspace_size.restype = c_size
    lib.seer_attn_gate_mask_workspace_size.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int]
    lib.seer_attn_gate_mask_pass_workspace_size.restype = c_size
    lib.seer_attn_gate_mask_pass_workspace_size.argtypes = [c_int, c_int, c_int, c_int, c_int,
                                                            c_int]
    lib.seer_attn_gate_mask.restype = c_int
    lib.seer_attn_gate_mask.argtypes = [c_void, c_void, c_int, c_int, c_int, c_int, c_int,
                                        c_void, c_void, c_int, c_float, c_float, c_int, c_float,
                                        c_double, c_int, c_void, c_void, c_int, c_void, c_void,
                                        c_size, c_void]
    lib.seer_pooled_target_mse.restype = c_int
    lib.seer_pooled_target_mse.argtypes = [c_void, c_void, c_int, c_int, c_int, c_void, c_void,
                                           c_void, c_void]
    lib.seer_attn_gate_decode_keys_workspace_size.restype = c_size
    lib.seer_attn_gate_decode_keys_workspace_size.argtypes = [c_int] * 5
    lib.seer_attn_gate_decode_keys.restype = c_int
    lib.seer_attn_gate_decode_keys.argtypes = [c_void, c_void, c_int, c_int, c_int, c_int,
                                               c_void, c_int, c_float, c_int, c_int, c_void,
                                               c_void, c_size, c_void]
    lib.seer_attn_gate_decode_scores.restype = c_int
    lib.seer_attn_gate_decode_scores.argtypes = [c_void, c_void, c_void, c_int, c_int, c_int,
                                                 c_int, c_int, c_void, c_int, c_float, c_float,
                                                 c_int, c_void, c_void]
    lib.seer_attn_gate_decode_mask.restype = c_int
    lib.seer_attn_gate_decode_mask.argtypes = [c_void, c_void, c_void, c_int, c_int, c_int, c_int,
                                               c_int, c_void, c_int, c_float, c_float, c_int,
                                               c_int, c_float, c_int, c_int, c_void, c_void, c_int,
                                               c_void, c_void]
    lib.seer_build_mask_decode.restype = c_int
    lib.seer_build_mask_decode.argtypes = [c_void, c_void, c_int, c_int, c_int, c_int, c_int,
                                           c_float, c_int, c_int, c_void, c_void, c_int, c_void]
    lib.seer_sparse_decode_workspace_size.restype = c_size
    lib.seer_sparse_decode_workspace_size.argtypes = [c_int] * 8
    lib.seer_sparse_decode.restype = c_int
    lib.seer_sparse_decode.argtypes = [c_void, c_void, c_void, c_void, c_int, c_int, c_int, c_int,
                                       c_int, c_float, c_int, c_void, c_void, c_int, c_int,
                                       c_void, c_void, c_size, c_void]
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != SEER_OK:
        raise SeerError(fn, status, load().seer_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: Tuple[int, ...]) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    # The calls launch on a stream of the current device (and the no-allocation
    # entry point takes its scratch from the current device).
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, not on the current device "
                         f"cuda:{torch.cuda.current_device()} (use torch.cuda.device(...))")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def version() -> int:
    return load().seer_version()


def topk_budget(nqb: int, density: float, keep_sink: bool) -> int:
    return load().seer_topk_budget(nqb, float(density), int(bool(keep_sink)))


def seer_build_mask(scores: torch.Tensor, mode: int, threshold: float, density: float,
                    keep_sink: bool, max_k: int, kv_idx: Optional[torch.Tensor] = None,
                    kv_cnt: Optional[torch.Tensor] = None, stream=None):
    """scores fp32 [B,H,nQB,nKB] -> (kv_idx int32 [B,H,nQB,max_k], kv_cnt int32 [B,H,nQB])."""
    lib = load()
    b, h, nqb, nkb = scores.shape
    _need(scores, "scores", torch.float32, (b, h, nqb, nkb))
    if kv_idx is None:
        kv_idx = torch.empty((b, h, nqb, max_k), dtype=torch.int32, device=scores.device)
    if kv_cnt is None:
        kv_cnt = torch.empty((b, h, nqb), dtype=torch.int32, device=scores.device)
    _need(kv_idx, "kv_idx", torch.int32, (b, h, nqb, max_k))
    _need(kv_cnt, "kv_cnt", torch.int32, (b, h, nqb))
    _check("seer_build_mask", lib.seer_build_mask(
        _ptr(scores), b, h, nqb, nkb, int(mode), float(threshold), float(density),
        int(bool(keep_sink)), _ptr(kv_idx), _ptr(kv_cnt), int(max_k), _stream(stream)))
    return kv_idx, kv_cnt


def seer_build_mask_need(scores: torch.Tensor, mode: int, threshold: float, density: float,
                         keep_sink: bool, max_k: int, kv_idx: Optional[torch.Tensor] = None,
                         kv_cnt: Optional[torch.Tensor] = None,
                         kv_need: Optional[torch.Tensor] = None, stream=None):
    """seer_build_mask plus kv_need int32 [B,H,nQB] (blocks selected before any cut
    to max_k): returns (kv_idx, kv_cnt, kv_need)."""
    lib = load()
    b, h, nqb, nkb = scores.shape
    _need(scores, "scores", torch.float32, (b, h, nqb, nkb))
    dev = scores.device
    kv_idx = torch.empty((b, h, nqb, max_k), dtype=torch.int32, device=dev) if kv_idx is None \
        else kv_idx
    kv_cnt = torch.empty((b, h, nqb), dtype=torch.int32, device=dev) if kv_cnt is None else kv_cnt
    kv_need = torch.empty((b, h, nqb), dtype=torch.int32, device=dev) if kv_need is None \
        else kv_need
    _need(kv_idx, "kv_idx", torch.int32, (b, h, nqb, max_k))
    _need(kv_cnt, "kv_cnt", torch.int32, (b, h, nqb))
    _need(kv_need, "kv_need", torch.int32, (b, h, nqb))
    _check("seer_build_mask_need", lib.seer_build_mask_need(
        _ptr(scores), b, h, nqb, nkb, int(mode), float(threshold), float(density),
        int(bool(keep_sink)), _ptr(kv_idx), _ptr(kv_cnt), _ptr(kv_need), int(max_k),
        _stream(stream)))
    return kv_idx, kv_cnt, kv_need


def seer_validate_lists(kv_idx: torch.Tensor, kv_cnt: torch.Tensor,
                        kv_need: Optional[torch.Tensor] = None, row_flags: bool = False,
                        stream=None):
    """Flag bits of block lists kv_idx [B,H,nB,max_k] / kv_cnt [B,H,nB]: returns the
    device int32 [1] OR of all rows, and the per-row flags [B,H,nB] if asked."""
    lib = load()
    b, h, nb, max_k = kv_idx.shape
    _need(kv_idx, "kv_idx", torch.int32, (b, h, nb, max_k))
    _need(kv_cnt, "kv_cnt", torch.int32, (b, h, nb))
    if kv_need is not None:
        _need(kv_need, "kv_need", torch.int32, (b, h, nb))
    flags = torch.empty((1,), dtype=torch.int32, device=kv_idx.device)
    rows = torch.empty((b, h, nb), dtype=torch.int32, device=kv_idx.device) if row_flags else None
    _check("seer_validate_lists", lib.seer_validate_lists(
        _ptr(kv_idx), _ptr(kv_cnt), _ptr(kv_need), b, h, nb, int(max_k), _ptr(rows),
        _ptr(flags), _stream(stream)))
    return (flags, rows) if row_flags else flags


def list_flags_status(flags: int) -> int:
    """The status code a set of list flags amounts to (host only)."""
    return load().seer_list_flags_status(int(flags))


def sparse_prefill_workspace_size(b: int, hq: int, hkv: int, t: int) -> int:
    return load().seer_sparse_prefill_workspace_size(b, hq, hkv, t)


def pooled_attn_map_workspace_size(b: int, hq: int, t: int) -> int:
    return load().seer_pooled_attn_map_workspace_size(b, hq, t)


def attn_gate_workspace_size(b: int, hq: int, hkv: int, t: int, dg: int) -> int:
    return load().seer_attn_gate_workspace_size(b, hq, hkv, t, dg)


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator hands out 512-byte aligned blocks.
    return torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=device)


def _caller_workspace(ws: torch.Tensor) -> torch.Tensor:
    """A workspace the caller passed: device memory of the current device, one
    contiguous block (the library checks its size and alignment itself)."""
    if not ws.is_cuda:
        raise ValueError("workspace must be a GPU tensor")
    if ws.device.index != torch.cuda.current_device():
        raise ValueError(f"workspace is on {ws.device}, not on the current device")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws


def _qkv_dims(q, k, v):
    b, hq, t, d = q.shape
    hkv = k.shape[1]
    _need(q, "q", torch.bfloat16, (b, hq, t, d))
    _need(k, "k", torch.bfloat16, (b, hkv, t, d))
    _need(v, "v", torch.bfloat16, (b, hkv, t, d))
    return b, hq, hkv, t, d


def _sparse_args(q, k, v, kv_idx, kv_cnt, block, sm_scale, out, workspace):
    lib = load()
    b, hq, hkv, t, d = _qkv_dims(q, k, v)
    nb = (t + block - 1) // block
    max_k = kv_idx.shape[-1]
    _need(kv_idx, "kv_idx", torch.int32, (b, hq, nb, max_k))
    _need(kv_cnt, "kv_cnt", torch.int32, (b, hq, nb))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, (b, hq, t, d))
    need = lib.seer_sparse_prefill_workspace_size(b, hq, hkv, t)
    if workspace is None:
        workspace = _workspace(need, q.device)
    else:
        _caller_workspace(workspace)
    scale = (1.0 / d ** 0.5) if sm_scale is None else float(sm_scale)
    return lib, (b, hq, hkv, t, d, scale), int(max_k), out, workspace


def seer_sparse_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_idx: torch.Tensor,
                        kv_cnt: torch.Tensor, sm_scale: Optional[float] = None,
                        out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Block-sparse causal prefill.  q [B,Hq,T,D], k/v [B,Hkv,T,D] bf16 -> O bf16."""
    lib, dims, max_k, out, workspace = _sparse_args(q, k, v, kv_idx, kv_cnt, BLOCK, sm_scale, out,
                                                    workspace)
    _check("seer_sparse_prefill", lib.seer_sparse_prefill(
        _ptr(q), _ptr(k), _ptr(v), *dims, _ptr(kv_idx), _ptr(kv_cnt), max_k, _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def seer_sparse_prefill_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                kv_idx: torch.Tensor, kv_cnt: torch.Tensor, out: torch.Tensor,
                                sm_scale: Optional[float] = None, stream=None) -> torch.Tensor:
    """seer_sparse_prefill without a workspace (the library's static scratch holds
    the work list); `out` is the caller's bf16 [B,Hq,T,D] output."""
    lib = load()
    b, hq, hkv, t, d = _qkv_dims(q, k, v)
    nb = (t + BLOCK - 1) // BLOCK
    max_k = kv_idx.shape[-1]
    _need(kv_idx, "kv_idx", torch.int32, (b, hq, nb, max_k))
    _need(kv_cnt, "kv_cnt", torch.int32, (b, hq, nb))
    _need(out, "out", torch.bfloat16, (b, hq, t, d))
    scale = (1.0 / d ** 0.5) if sm_scale is None else float(sm_scale)
    _check("seer_sparse_prefill_noalloc", lib.seer_sparse_prefill_noalloc(
        _ptr(q), _ptr(k), _ptr(v), b, hq, hkv, t, d, scale, _ptr(kv_idx), _ptr(kv_cnt),
        int(max_k), _ptr(out), _stream(stream)))
    return out


def seer_sparse_prefill_block(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                              kv_idx: torch.Tensor, kv_cnt: torch.Tensor, block: int,
                              sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """seer_sparse_prefill with lists of `block`-token blocks (64 or 128):
    kv_idx [B,Hq,ceil(T/block),max_k], kv_cnt [B,Hq,ceil(T/block)]."""
    lib, dims, max_k, out, workspace = _sparse_args(q, k, v, kv_idx, kv_cnt, int(block), sm_scale,
                                                    out, workspace)
    _check("seer_sparse_prefill_block", lib.seer_sparse_prefill_block(
        _ptr(q), _ptr(k), _ptr(v), *dims, int(block), _ptr(kv_idx), _ptr(kv_cnt), max_k,
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def seer_pooled_attn_map(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                         amap: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None):
    """Dense causal pass -> (O bf16 [B,Hq,T,D], A fp32 [B,Hq,nQB,nQB])."""
    lib = load()
    b, hq, hkv, t, d = _qkv_dims(q, k, v)
    nqb = (t + BLOCK - 1) // BLOCK
    if out is None:
        out = torch.empty_like(q)
    if amap is None:
        amap = torch.empty((b, hq, nqb, nqb), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16, (b, hq, t, d))
    _need(amap, "amap", torch.float32, (b, hq, nqb, nqb))
    need = lib.seer_pooled_attn_map_workspace_size(b, hq, t)
    if workspace is None:
        workspace = _workspace(need, q.device)
    else:
        _caller_workspace(workspace)
    scale = (1.0 / d ** 0.5) if sm_scale is None else float(sm_scale)
    _check("seer_pooled_attn_map", lib.seer_pooled_attn_map(
        _ptr(q), _ptr(k), _ptr(v), b, hq, hkv, t, d, scale, _ptr(out), _ptr(amap),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, amap


def seer_pooled_target_mse(amap: torch.Tensor, gate: Optional[torch.Tensor] = None,
                           target: Optional[torch.Tensor] = None, row_sse: Optional[torch.Tensor] = None,
                           loss: Optional[torch.Tensor] = None, stream=None):
    """amap fp32 [B,H,nQB,nQB] -> (target, row_sse, loss); the last two are None without gate.

    target may be amap itself (normalised in place)."""
    lib = load()
    b, h, nqb, nkb = amap.shape
    _need(amap, "amap", torch.float32, (b, h, nqb, nqb))
    if gate is not None:
        _need(gate, "gate", torch.float32, (b, h, nqb, nqb))
    if target is None:
        target = torch.empty_like(amap)
    _need(target, "target", torch.float32, (b, h, nqb, nqb))
    if gate is not None:
        if row_sse is None:
            row_sse = torch.empty((b, h, nqb), dtype=torch.float32, device=amap.device)
        if loss is None:
            loss = torch.empty((1,), dtype=torch.float32, device=amap.device)
        _need(row_sse, "row_sse", torch.float32, (b, h, nqb))
        _need(loss, "loss", torch.float32, (1,))
    else:
        row_sse = loss = None
    _check("seer_pooled_target_mse", lib.seer_pooled_target_mse(
        _ptr(amap), _ptr(gate), b, h, nqb, _ptr(target), _ptr(row_sse), _ptr(loss),
        _stream(stream)))
    return target, row_sse, loss


def seer_attn_gate_scores(q: torch.Tensor, k: torch.Tensor, wq: torch.Tensor, wk: torch.Tensor,
                          scale: Optional[float] = None, rope_base: float = 10000.0,
                          scores: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """AttnGate soft block scores [B,Hq,nQB,nQB] fp32 from q [B,Hq,T,D], k [B,Hkv,T,D]
    (bf16, before RoPE) and weights wq [Hq,D,Dg], wk [Hkv,2D,Dg] (fp32)."""
    lib = load()
    b, hq, hkv, t, d = _qkv_dims(q, k, k)
    dg = wq.shape[-1]
    nqb = (t + BLOCK - 1) // BLOCK
    _need(wq, "wq", torch.float32, (hq, d, dg))
    _need(wk, "wk", torch.float32, (hkv, 2 * d, dg))
    if scores is None:
        scores = torch.empty((b, hq, nqb, nqb), dtype=torch.float32, device=q.device)
    _need(scores, "scores", torch.float32, (b, hq, nqb, nqb))
    need = lib.seer_attn_gate_workspace_size(b, hq, hkv, t, dg)
    if workspace is None:
        workspace = _workspace(need, q.device)
    else:
        _caller_workspace(workspace)
    sc = (1.0 / dg ** 0.5) if scale is None else float(scale)
    _check("seer_attn_gate_scores", lib.seer_attn_gate_scores(
        _ptr(q), _ptr(k), b, hq, hkv, t, d, _ptr(wq), _ptr(wk), int(dg), sc, float(rope_base),
        _ptr(scores), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return scores


def attn_gate_mask_workspace_size(b: int, hq: int, hkv: int, t: int, dg: int,
                                  with_scores: bool) -> int:
    return load().seer_attn_gate_mask_workspace_size(b, hq, hkv, t, dg, int(bool(with_scores)))


def attn_gate_mask_pass_workspace_size(b: int, hq: int, hkv: int, t: int, dg: int,
                                        pass_tiles: int) -> int:
    return load().seer_attn_gate_mask_pass_workspace_size(b, hq, hkv, t, dg, int(pass_tiles))


def seer_attn_gate_mask(q: torch.Tensor, k: torch.Tensor, wq: torch.Tensor, wk: torch.Tensor,
                        mode: int, threshold: float, density: float, keep_sink: bool, max_k: int,
                        scale: Optional[float] = None, rope_base: float = 10000.0,
                        return_scores: bool = False, kv_idx: Optional[torch.Tensor] = None,
                        kv_cnt: Optional[torch.Tensor] = None,
                        scores: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None,
                        pass_tiles: Optional[int] = None, stream=None):
    """AttnGate scores straight into block lists: (kv_idx [B,Hq,nQB,max_k], kv_cnt
    [B,Hq,nQB], scores [B,Hq,nQB,nQB] or None).  Scores are written only when
    return_scores is set or a scores buffer is passed.  Without scores, pass_tiles
    sizes the allocated workspace for passes of that many 64-block tile rows
    (memory linear in T); the lists are the same."""
    lib = load()
    b, hq, hkv, t, d = _qkv_dims(q, k, k)
    dg = wq.shape[-1]
    nqb = (t + BLOCK - 1) // BLOCK
    _need(wq, "wq", torch.float32, (hq, d, dg))
    _need(wk, "wk", torch.float32, (hkv, 2 * d, dg))
    if scores is None and return_scores:
        scores = torch.empty((b, hq, nqb, nqb), dtype=torch.float32, device=q.device)
    if scores is not None:
        _need(scores, "scores", torch.float32, (b, hq, nqb, nqb))
    if kv_idx is None:
        kv_idx = torch.empty((b, hq, nqb, max_k), dtype=torch.int32, device=q.device)
    if kv_cnt is None:
        kv_cnt = torch.empty((b, hq, nqb), dtype=torch.int32, device=q.device)
    _need(kv_idx, "kv_idx", torch.int32, (b, hq, nqb, max_k))
    _need(kv_cnt, "kv_cnt", torch.int32, (b, hq, nqb))
    if scores is None and pass_tiles is not None:
        need = lib.seer_attn_gate_mask_pass_workspace_size(b, hq, hkv, t, dg, int(pass_tiles))
    else:
        need = lib.seer_attn_gate_mask_workspace_size(b, hq, hkv, t, dg, int(scores is not None))
    if workspace is None:
        workspace = _workspace(need, q.device)
    else:
        _caller_workspace(workspace)
    sc = (1.0 / dg ** 0.5) if scale is None else float(scale)
    _check("seer_attn_gate_mask", lib.seer_attn_gate_mask(
        _ptr(q), _ptr(k), b, hq, hkv, t, d, _ptr(wq), _ptr(wk), int(dg), sc, float(rope_base),
        int(mode), float(threshold), float(density), int(bool(keep_sink)), _ptr(kv_idx),
        _ptr(kv_cnt), int(max_k), _ptr(scores), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return kv_idx, kv_cnt, scores


def attn_gate_decode_keys_workspace_size(b: int, hkv: int, tmax: int, d: int,
                                         block: int) -> int:
    return load().seer_attn_gate_decode_keys_workspace_size(b, hkv, tmax, d, block)


def seer_attn_gate_decode_keys(k_cache: torch.Tensor, kv_len: torch.Tensor, wk: torch.Tensor,
                               block: int = BLOCK, rope_base: float = 10000.0,
                               last_block_only: bool = False,
                               k_gate: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None,
                               stream=None) -> torch.Tensor:
    """Gate keys K~ [B,Hkv,nKB,Dg] fp32 of k_cache [B,Hkv,Tmax,D] (bf16, before RoPE) for
    the blocks below kv_len int32 [B]; with last_block_only only each sequence's last
    block is (re)computed in the given k_gate."""
    lib = load()
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [B,Hkv,Tmax,D]")
    b, hkv, tmax, d = k_cache.shape
    dg = wk.shape[-1]
    nkb = (tmax + block - 1) // block
    _need(k_cache, "k_cache", torch.bfloat16, (b, hkv, tmax, d))
    _need(kv_len, "kv_len", torch.int32, (b,))
    _need(wk, "wk", torch.float32, (hkv, 2 * d, dg))
    if k_gate is None:
        if last_block_only:
            raise ValueError("last_block_only updates an existing k_gate")
        k_gate = torch.empty((b, hkv, nkb, dg), dtype=torch.float32, device=k_cache.device)
    _need(k_gate, "k_gate", torch.float32, (b, hkv, nkb, dg))
    if workspace is None and not last_block_only:
        workspace = _workspace(lib.seer_attn_gate_decode_keys_workspace_size(
            b, hkv, tmax, d, int(block)), k_cache.device)
    elif workspace is not None:
        _caller_workspace(workspace)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("seer_attn_gate_decode_keys", lib.seer_attn_gate_decode_keys(
        _ptr(k_cache), _ptr(kv_len), b, hkv, tmax, d, _ptr(wk), int(dg), float(rope_base),
        int(block), int(bool(last_block_only)), _ptr(k_gate), _ptr(workspace), nbytes,
        _stream(stream)))
    return k_gate


def seer_attn_gate_decode_scores(q: torch.Tensor, k_gate: torch.Tensor, kv_len: torch.Tensor,
                                 wq: torch.Tensor, tmax: int, block: int = BLOCK,
                                 scale: Optional[float] = None, rope_base: float = 10000.0,
                                 scores: Optional[torch.Tensor] = None,
                                 stream=None) -> torch.Tensor:
    """Per-token gate scores [B,Hq,nKB] fp32 for q [B,Hq,D] (bf16, before RoPE) from the
    gate keys k_gate [B,Hkv,nKB,Dg] of a cache of tmax slots; kv_len int32 [B]."""
    lib = load()
    if q.dim() != 3 or k_gate.dim() != 4:
        raise ValueError("q must be [B,Hq,D] and k_gate [B,Hkv,nKB,Dg]")
    b, hq, d = q.shape
    hkv, nkb, dg = k_gate.shape[1], k_gate.shape[2], k_gate.shape[3]
    if nkb != (tmax + block - 1) // block:
        raise ValueError(f"k_gate has {nkb} blocks, a cache of {tmax} slots has "
                         f"{(tmax + block - 1) // block}")
    _need(q, "q", torch.bfloat16, (b, hq, d))
    _need(k_gate, "k_gate", torch.float32, (b, hkv, nkb, dg))
    _need(kv_len, "kv_len", torch.int32, (b,))
    _need(wq, "wq", torch.float32, (hq, d, dg))
    if scores is None:
        scores = torch.empty((b, hq, nkb), dtype=torch.float32, device=q.device)
    _need(scores, "scores", torch.float32, (b, hq, nkb))
    sc = (1.0 / dg ** 0.5) if scale is None else float(scale)
    _check("seer_attn_gate_decode_scores", lib.seer_attn_gate_decode_scores(
        _ptr(q), _ptr(k_gate), _ptr(kv_len), b, hq, hkv, tmax, d, _ptr(wq), int(dg), sc,
        float(rope_base), int(block), _ptr(scores), _stream(stream)))
    return scores


def seer_attn_gate_decode_mask(q: torch.Tensor, k_gate: torch.Tensor, kv_len: torch.Tensor,
                               wq: torch.Tensor, tmax: int, mode: int, threshold: float,
                               k_blocks: int, keep_sink: bool, max_k: int, block: int = BLOCK,
                               scale: Optional[float] = None, rope_base: float = 10000.0,
                               return_scores: bool = False,
                               kv_idx: Optional[torch.Tensor] = None,
                               kv_cnt: Optional[torch.Tensor] = None,
                               scores: Optional[torch.Tensor] = None, stream=None):
    """Per-token gate scores and decode lists in one pass: the lists of
    seer_build_mask_decode on seer_attn_gate_decode_scores's rows ->
    (kv_idx int32 [B,Hq,max_k], kv_cnt int32 [B,Hq], scores [B,Hq,nKB] or None)."""
    lib = load()
    if q.dim() != 3 or k_gate.dim() != 4:
        raise ValueError("q must be [B,Hq,D] and k_gate [B,Hkv,nKB,Dg]")
    b, hq, d = q.shape
    hkv, nkb, dg = k_gate.shape[1], k_gate.shape[2], k_gate.shape[3]
    if nkb != (tmax + block - 1) // block:
        raise ValueError(f"k_gate has {nkb} blocks, a cache of {tmax} slots has "
                         f"{(tmax + block - 1) // block}")
    _need(q, "q", torch.bfloat16, (b, hq, d))
    _need(k_gate, "k_gate", torch.float32, (b, hkv, nkb, dg))
    _need(kv_len, "kv_len", torch.int32, (b,))
    _need(wq, "wq", torch.float32, (hq, d, dg))
    if kv_idx is None:
        kv_idx = torch.empty((b, hq, max_k), dtype=torch.int32, device=q.device)
    if kv_cnt is None:
        kv_cnt = torch.empty((b, hq), dtype=torch.int32, device=q.device)
    _need(kv_idx, "kv_idx", torch.int32, (b, hq, max_k))
    _need(kv_cnt, "kv_cnt", torch.int32, (b, hq))
    if return_scores and scores is None:
        scores = torch.empty((b, hq, nkb), dtype=torch.float32, device=q.device)
    if scores is not None:
        _need(scores, "scores", torch.float32, (b, hq, nkb))
    sc = (1.0 / dg ** 0.5) if scale is None else float(scale)
    _check("seer_attn_gate_decode_mask", lib.seer_attn_gate_decode_mask(
        _ptr(q), _ptr(k_gate), _ptr(kv_len), b, hq, hkv, tmax, d, _ptr(wq), int(dg), sc,
        float(rope_base), int(block), int(mode), float(threshold), int(k_blocks),
        int(bool(keep_sink)), _ptr(kv_idx), _ptr(kv_cnt), int(max_k), _ptr(scores),
        _stream(stream)))
    return kv_idx, kv_cnt, scores


def seer_build_mask_decode(scores: torch.Tensor, kv_len: torch.Tensor, block: int, mode: int,
                           threshold: float, k_blocks: int, keep_sink: bool, max_k: int,
                           kv_idx: Optional[torch.Tensor] = None,
                           kv_cnt: Optional[torch.Tensor] = None, stream=None):
    """Decode lists: scores fp32 [B,H,nKB], kv_len int32 [B] ->
    (kv_idx int32 [B,H,max_k], kv_cnt int32 [B,H])."""
    lib = load()
    b, h, nkb = scores.shape
    _need(scores, "scores", torch.float32, (b, h, nkb))
    _need(kv_len, "kv_len", torch.int32, (b,))
    if kv_idx is None:
        kv_idx = torch.empty((b, h, max_k), dtype=torch.int32, device=scores.device)
    if kv_cnt is None:
        kv_cnt = torch.empty((b, h), dtype=torch.int32, device=scores.device)
    _need(kv_idx, "kv_idx", torch.int32, (b, h, max_k))
    _need(kv_cnt, "kv_cnt", torch.int32, (b, h))
    _check("seer_build_mask_decode", lib.seer_build_mask_decode(
        _ptr(scores), _ptr(kv_len), b, h, nkb, int(block), int(mode), float(threshold),
        int(k_blocks), int(bool(keep_sink)), _ptr(kv_idx), _ptr(kv_cnt), int(max_k),
        _stream(stream)))
    return kv_idx, kv_cnt


def sparse_decode_workspace_size(b: int, hq: int, hkv: int, tmax: int, d: int, list_heads: int,
                                 max_k: int, block: int) -> int:
    return load().seer_sparse_decode_workspace_size(b, hq, hkv, tmax, d, list_heads, max_k,
                                                    block)


def seer_sparse_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       kv_len: torch.Tensor, kv_idx: torch.Tensor, kv_cnt: torch.Tensor,
                       block: int = BLOCK, sm_scale: Optional[float] = None,
                       out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Block-sparse decode: q [B,Hq,D], cache [B,Hkv,Tmax,D] (bf16), kv_len int32 [B],
    lists [B,H,max_k] / [B,H] with H = Hq or Hkv -> O bf16 [B,Hq,D]."""
    lib = load()
    b, hq, d = q.shape
    hkv, tmax = k_cache.shape[1], k_cache.shape[2]
    _need(q, "q", torch.bfloat16, (b, hq, d))
    _need(k_cache, "k_cache", torch.bfloat16, (b, hkv, tmax, d))
    _need(v_cache, "v_cache", torch.bfloat16, (b, hkv, tmax, d))
    _need(kv_len, "kv_len", torch.int32, (b,))
    lh, max_k = kv_idx.shape[1], kv_idx.shape[2]
    _need(kv_idx, "kv_idx", torch.int32, (b, lh, max_k))
    _need(kv_cnt, "kv_cnt", torch.int32, (b, lh))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, (b, hq, d))
    if workspace is None:
        workspace = _workspace(sparse_decode_workspace_size(b, hq, hkv, tmax, d, lh, max_k,
                                                            int(block)), q.device)
    else:
        _caller_workspace(workspace)
    scale = (1.0 / d ** 0.5) if sm_scale is None else float(sm_scale)
    _check("seer_sparse_decode", lib.seer_sparse_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(kv_len), b, hq, hkv, tmax, d, scale,
        int(block), _ptr(kv_idx), _ptr(kv_cnt), lh, max_k, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out
