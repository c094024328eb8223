"""Python binding of the MI355X decode-attention library (argument marshalling only).

Every function has the name of the C entry point it calls (include/attn_decode.h)
and takes torch tensors that already live on the GPU. The binding checks dtypes,
shapes and contiguity, allocates outputs/workspaces when the caller passes none,
and hands raw pointers plus torch's current HIP stream to the C library. All
arithmetic runs in the HIP kernels; there is no CPU or PyTorch fallback, and a
missing library raises.
"""

from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import _lib
from ._lib import ATTN_BF16, ATTN_F32, load

__all__ = [
    "AttnError", "load",
    "attn_kv_cache_bytes", "attn_mla_cache_bytes",
    "attn_decode_gqa_plan", "attn_decode_gqa_workspace_bytes", "attn_decode_gqa",
    "attn_decode_gqa_noalloc", "attn_decode_gqa_split", "attn_decode_gqa_split_merge",
    "attn_decode_gqa_partial", "attn_decode_merge",
    "attn_decode_mla_plan", "attn_decode_mla_workspace_bytes", "attn_decode_mla",
    "attn_decode_mla_partial",
    "attn_decode_gqa_step", "attn_kv_append", "attn_decode_mla_step", "attn_latent_append",
    "attn_decode_gqa_window", "attn_decode_gqa_paged", "attn_kv_append_paged",
    "attn_decode_mla_paged", "attn_latent_append_paged",
    "attn_mla_absorb_q", "attn_mla_up_v",
]


class AttnError(RuntimeError):
    """A non-zero attn_status returned by the C library."""

    def __init__(self, status: int, where: str):
        self.status = int(status)
        super().__init__(f"{where}: {_lib.status_str(status)} ({status})")


def _check(st: int, where: str) -> None:
    if st != _lib.ATTN_OK:
        raise AttnError(st, where)


_DT = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}: expected float32 or bfloat16")
    return _DT[t.dtype]


def _dev(*ts: torch.Tensor) -> torch.device:
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    return dev


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _lens(seq_lens: torch.Tensor, B: int) -> None:
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,):
        raise ValueError(f"seq_lens must be int32 of shape ({B},)")


# ----------------------------------------------------------------------------- helpers

def attn_kv_cache_bytes(n_layers: int, n_kv_heads: int, head_dim: int, seq_len: int,
                        batch: int = 1, bytes_per_elem: int = 2) -> int:
    """Exact KV-cache bytes: K and V, each [batch, kv_heads, seq, head_dim], per layer."""
    return int(load().attn_kv_cache_bytes(n_layers, n_kv_heads, head_dim, seq_len, batch,
                                          bytes_per_elem))


def attn_mla_cache_bytes(n_layers: int, d_c: int, d_r: int, seq_len: int, batch: int = 1,
                         bytes_per_elem: int = 2) -> int:
    """Exact MLA cache bytes: one (d_c + d_r)-wide row per token per layer per sequence."""
    return int(load().attn_mla_cache_bytes(n_layers, d_c, d_r, seq_len, batch, bytes_per_elem))


def attn_decode_gqa_plan(B: int, h_q: int, h_kv: int, D: int, T_max: int, dtype=torch.bfloat16):
    """(partition_size, num_partitions, workspace_bytes) the library picks for a shape."""
    P, NP, ws = ctypes.c_int(), ctypes.c_int(), ctypes.c_size_t()
    _check(load().attn_decode_gqa_plan(B, h_q, h_kv, D, T_max, _DT[dtype], ctypes.byref(P),
                                       ctypes.byref(NP), ctypes.byref(ws)), "attn_decode_gqa_plan")
    return P.value, NP.value, ws.value


def attn_decode_gqa_workspace_bytes(B, h_q, h_kv, D, T_max, dtype=torch.bfloat16) -> int:
    return int(load().attn_decode_gqa_workspace_bytes(B, h_q, h_kv, D, T_max, _DT[dtype]))


def attn_decode_mla_plan(B: int, H: int, d_c: int, d_r: int, T_max: int):
    P, NP, ws = ctypes.c_int(), ctypes.c_int(), ctypes.c_size_t()
    _check(load().attn_decode_mla_plan(B, H, d_c, d_r, T_max, ctypes.byref(P), ctypes.byref(NP),
                                       ctypes.byref(ws)), "attn_decode_mla_plan")
    return P.value, NP.value, ws.value


def attn_decode_mla_workspace_bytes(B, H, d_c, d_r, T_max) -> int:
    return int(load().attn_decode_mla_workspace_bytes(B, H, d_c, d_r, T_max))


# ----------------------------------------------------------------------------- GQA

def _gqa_shapes(q, k_cache, v_cache):
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B,h_q,D], k_cache and v_cache [B,h_kv,T_max,D]")
    B, h_q, D = q.shape
    if k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("q and k_cache disagree on B or D")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q, k_cache and v_cache must share one dtype")
    return B, h_q, k_cache.shape[1], D, k_cache.shape[2]


def attn_decode_gqa(q, k_cache, v_cache, seq_lens, scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """One decode step of MHA/GQA/MQA. Returns out [B, h_q, D] in q's dtype."""
    B, h_q, h_kv, D, T_max = _gqa_shapes(q, k_cache, v_cache)
    dev = _dev(q, k_cache, v_cache, seq_lens)
    _lens(seq_lens, B)
    dt = _dt(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    need = attn_decode_gqa_workspace_bytes(B, h_q, h_kv, D, T_max, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(out, workspace)
    _check(load().attn_decode_gqa(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), B, h_q,
                                  h_kv, D, T_max, scale, dt, _ptr(out), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(dev)),
           "attn_decode_gqa")
    return out


def attn_decode_gqa_noalloc(q, k_cache, v_cache, seq_lens, scale: Optional[float] = None,
                            out: Optional[torch.Tensor] = None):
    """attn_decode_gqa with the library's static device scratch as the workspace (no
    allocation in the call; only `out` is allocated here when the caller passes none)."""
    B, h_q, h_kv, D, T_max = _gqa_shapes(q, k_cache, v_cache)
    dev = _dev(q, k_cache, v_cache, seq_lens)
    _lens(seq_lens, B)
    dt = _dt(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _dev(out)
    _check(load().attn_decode_gqa_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), B, h_q,
                                          h_kv, D, T_max, scale, dt, _ptr(out), _stream(dev)),
           "attn_decode_gqa_noalloc")
    return out


def _gqa_split_call(fn_name, q, k_cache, v_cache, seq_lens, workspace, scale, out):
    B, h_q, h_kv, D, T_max = _gqa_shapes(q, k_cache, v_cache)
    dev = _dev(q, k_cache, v_cache, seq_lens)
    _lens(seq_lens, B)
    dt = _dt(q)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, workspace)
    _check(getattr(load(), fn_name)(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), B, h_q,
                                    h_kv, D, T_max, scale, dt, _ptr(out), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(dev)),
           fn_name)
    return out


def attn_decode_gqa_split(q, k_cache, v_cache, seq_lens, workspace: torch.Tensor,
                          scale: Optional[float] = None, out: Optional[torch.Tensor] = None):
    """Stage 1 of attn_decode_gqa's work-balanced split (bf16 storage, every supported D and g):
    writes the partials into `workspace` (attn_decode_gqa_workspace_bytes bytes); `out` is
    checked, not written."""
    _gqa_split_call("attn_decode_gqa_split", q, k_cache, v_cache, seq_lens, workspace, scale, out)


def attn_decode_gqa_split_merge(q, k_cache, v_cache, seq_lens, workspace: torch.Tensor,
                                scale: Optional[float] = None, out: Optional[torch.Tensor] = None):
    """Stage 2 of the split: merges the partials stage 1 left in `workspace` into
    out [B, h_q, D] (returned)."""
    return _gqa_split_call("attn_decode_gqa_split_merge", q, k_cache, v_cache, seq_lens, workspace,
                           scale, out)


def attn_decode_gqa_window(q, k_cache, v_cache, seq_lens, window: int, scale: Optional[float] = None,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Sliding-window decode: each row attends over its last `window` positions.
    Returns out [B, h_q, D] in q's dtype."""
    B, h_q, h_kv, D, T_max = _gqa_shapes(q, k_cache, v_cache)
    dev = _dev(q, k_cache, v_cache, seq_lens)
    _lens(seq_lens, B)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    window = int(window)
    need = attn_decode_gqa_workspace_bytes(B, h_q, h_kv, D, max(1, min(window, T_max)), q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(out, workspace)
    _check(load().attn_decode_gqa_window(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), B,
                                         h_q, h_kv, D, T_max, window, scale, _dt(q), _ptr(out),
                                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         _stream(dev)), "attn_decode_gqa_window")
    return out


def _new_rows(k_new, v_new, B, h_kv, D, dtype):
    if tuple(k_new.shape) != (B, h_kv, D) or tuple(v_new.shape) != (B, h_kv, D):
        raise ValueError(f"k_new and v_new must be [{B}, {h_kv}, {D}]")
    if k_new.dtype != dtype or v_new.dtype != dtype:
        raise TypeError("k_new and v_new must have the caches' dtype")


def attn_decode_gqa_step(q, k_new, v_new, k_cache, v_cache, seq_lens, scale: Optional[float] = None,
                         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Append k_new/v_new [B,h_kv,D] at row seq_lens[b] of the caches (in place), then attend
    over seq_lens[b] + 1 positions. seq_lens (lengths before the step) is not modified.
    Returns out [B, h_q, D] in q's dtype."""
    B, h_q, h_kv, D, T_max = _gqa_shapes(q, k_cache, v_cache)
    dev = _dev(q, k_new, v_new, k_cache, v_cache, seq_lens)
    _lens(seq_lens, B)
    _new_rows(k_new, v_new, B, h_kv, D, q.dtype)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    need = attn_decode_gqa_workspace_bytes(B, h_q, h_kv, D, T_max, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(out, workspace)
    _check(load().attn_decode_gqa_step(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(seq_lens), B, h_q, h_kv, D, T_max, scale,
                                       _dt(q), _ptr(out), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(dev)),
           "attn_decode_gqa_step")
    return out


def attn_kv_append(k_new, v_new, k_cache, v_cache, seq_lens) -> None:
    """Copy k_new/v_new [B,h_kv,D] into row seq_lens[b] of k_cache/v_cache (in place)."""
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("expected k_cache and v_cache [B,h_kv,T_max,D] of one dtype")
    B, h_kv, T_max, D = k_cache.shape
    dev = _dev(k_new, v_new, k_cache, v_cache, seq_lens)
    _lens(seq_lens, B)
    _new_rows(k_new, v_new, B, h_kv, D, k_cache.dtype)
    _check(load().attn_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(seq_lens), B, h_kv, D, T_max, _dt(k_cache), _stream(dev)),
           "attn_kv_append")


def attn_decode_gqa_partial(q, k_cache, v_cache, seq_lens, partition_size: int,
                            scale: Optional[float] = None, part_out=None, part_lse=None):
    """Stage 1 with an explicit partition size. Returns (part_out [B,h_q,NP,D], part_lse [B,h_q,NP])."""
    B, h_q, h_kv, D, T_max = _gqa_shapes(q, k_cache, v_cache)
    dev = _dev(q, k_cache, v_cache, seq_lens)
    _lens(seq_lens, B)
    NP = -(-T_max // int(partition_size)) if partition_size > 0 else 1
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if part_out is None:
        part_out = torch.empty((B, h_q, NP, D), dtype=torch.float32, device=dev)
    if part_lse is None:
        part_lse = torch.empty((B, h_q, NP), dtype=torch.float32, device=dev)
    _dev(part_out, part_lse)
    _check(load().attn_decode_gqa_partial(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                          B, h_q, h_kv, D, T_max, scale, _dt(q), int(partition_size),
                                          _ptr(part_out), _ptr(part_lse), _stream(dev)),
           "attn_decode_gqa_partial")
    return part_out, part_lse


def attn_decode_merge(part_out, part_lse, seq_lens, T_max: int, partition_size: int,
                      out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None):
    """Stage 2: merge [B,H,NP,Dv] partials into out [B,H,Dv]."""
    if part_out.dim() != 4 or part_lse.shape != part_out.shape[:3]:
        raise ValueError("expected part_out [B,H,NP,Dv] and part_lse [B,H,NP]")
    B, H, NP, Dv = part_out.shape
    dev = _dev(part_out, part_lse, seq_lens)
    _lens(seq_lens, B)
    if NP != -(-int(T_max) // int(partition_size)):
        raise ValueError("part_out's partition count does not match T_max / partition_size")
    if out is None:
        out = torch.empty((B, H, Dv), dtype=out_dtype, device=dev)
    _dev(out)
    _check(load().attn_decode_merge(_ptr(part_out), _ptr(part_lse), _ptr(seq_lens), B, H, Dv,
                                    int(T_max), int(partition_size), _DT[out.dtype], _ptr(out),
                                    _stream(dev)), "attn_decode_merge")
    return out


# ----------------------------------------------------------------------------- MLA

def _mla_shapes(q_nope, q_rope, latent):
    if q_nope.dim() != 3 or q_rope.dim() != 3 or latent.dim() != 3:
        raise ValueError("expected q_nope [B,H,d_c], q_rope [B,H,d_r], latent [B,T_max,d_c+d_r]")
    B, H, d_c = q_nope.shape
    d_r = q_rope.shape[2]
    if q_rope.shape[:2] != (B, H) or latent.shape[0] != B or latent.shape[2] != d_c + d_r:
        raise ValueError("q_nope, q_rope and latent disagree on B, H or widths")
    for t in (q_nope, q_rope, latent):
        if t.dtype != torch.bfloat16:
            raise TypeError("MLA inputs must be bfloat16")
    return B, H, d_c, d_r, latent.shape[1]


def attn_decode_mla(q_nope_absorbed, q_rope, latent_cache, seq_lens, scale: float,
                    out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """One absorbed-MLA decode step. Returns out [B, H, d_c] bf16."""
    B, H, d_c, d_r, T_max = _mla_shapes(q_nope_absorbed, q_rope, latent_cache)
    dev = _dev(q_nope_absorbed, q_rope, latent_cache, seq_lens)
    _lens(seq_lens, B)
    if out is None:
        out = torch.empty((B, H, d_c), dtype=torch.bfloat16, device=dev)
    need = attn_decode_mla_workspace_bytes(B, H, d_c, d_r, T_max)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(out, workspace)
    _check(load().attn_decode_mla(_ptr(q_nope_absorbed), _ptr(q_rope), _ptr(latent_cache),
                                  _ptr(seq_lens), B, H, d_c, d_r, T_max, float(scale), _ptr(out),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(dev)), "attn_decode_mla")
    return out


def attn_decode_mla_partial(q_nope_absorbed, q_rope, latent_cache, seq_lens, scale: float,
                            partition_size: int, part_out=None, part_lse=None):
    B, H, d_c, d_r, T_max = _mla_shapes(q_nope_absorbed, q_rope, latent_cache)
    dev = _dev(q_nope_absorbed, q_rope, latent_cache, seq_lens)
    _lens(seq_lens, B)
    NP = -(-T_max // int(partition_size)) if partition_size > 0 else 1
    if part_out is None:
        part_out = torch.empty((B, H, NP, d_c), dtype=torch.float32, device=dev)
    if part_lse is None:
        part_lse = torch.empty((B, H, NP), dtype=torch.float32, device=dev)
    _dev(part_out, part_lse)
    _check(load().attn_decode_mla_partial(_ptr(q_nope_absorbed), _ptr(q_rope), _ptr(latent_cache),
                                          _ptr(seq_lens), B, H, d_c, d_r, T_max, float(scale),
                                          int(partition_size), _ptr(part_out), _ptr(part_lse),
                                          _stream(dev)), "attn_decode_mla_partial")
    return part_out, part_lse


def attn_decode_mla_step(q_nope_absorbed, q_rope, latent_new, latent_cache, seq_lens, scale: float,
                         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Append latent_new [B, d_c+d_r] at row seq_lens[b] of latent_cache (in place), then attend
    over seq_lens[b] + 1 positions. Returns out [B, H, d_c] bf16."""
    B, H, d_c, d_r, T_max = _mla_shapes(q_nope_absorbed, q_rope, latent_cache)
    dev = _dev(q_nope_absorbed, q_rope, latent_new, latent_cache, seq_lens)
    _lens(seq_lens, B)
    if tuple(latent_new.shape) != (B, d_c + d_r) or latent_new.dtype != torch.bfloat16:
        raise ValueError(f"latent_new must be bfloat16 [{B}, {d_c + d_r}]")
    if out is None:
        out = torch.empty((B, H, d_c), dtype=torch.bfloat16, device=dev)
    need = attn_decode_mla_workspace_bytes(B, H, d_c, d_r, T_max)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(out, workspace)
    _check(load().attn_decode_mla_step(_ptr(q_nope_absorbed), _ptr(q_rope), _ptr(latent_new),
                                       _ptr(latent_cache), _ptr(seq_lens), B, H, d_c, d_r, T_max,
                                       float(scale), _ptr(out), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(dev)),
           "attn_decode_mla_step")
    return out


def attn_latent_append(latent_new, latent_cache, seq_lens, d_c: int = 512) -> None:
    """Copy latent_new [B, d_c+d_r] into row seq_lens[b] of latent_cache [B,T_max,d_c+d_r] (in place)."""
    if latent_cache.dim() != 3 or latent_cache.dtype != torch.bfloat16:
        raise ValueError("expected a bfloat16 latent_cache [B, T_max, d_c + d_r]")
    B, T_max, W = latent_cache.shape
    dev = _dev(latent_new, latent_cache, seq_lens)
    _lens(seq_lens, B)
    if tuple(latent_new.shape) != (B, W) or latent_new.dtype != torch.bfloat16:
        raise ValueError(f"latent_new must be bfloat16 [{B}, {W}]")
    _check(load().attn_latent_append(_ptr(latent_new), _ptr(latent_cache), _ptr(seq_lens), B,
                                     int(d_c), W - int(d_c), T_max, _stream(dev)),
           "attn_latent_append")


# ----------------------------------------------------------------------------- paged caches

def _table(block_table, B):
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be int32 [{B}, max_pages]")
    return block_table.shape[1]


def attn_decode_gqa_paged(q, k_pages, v_pages, block_table, seq_lens, scale: Optional[float] = None,
                          out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Decode over pages k_pages/v_pages [num_pages, h_kv, page_size, D]; block_table int32
    [B, max_pages] maps sequence b's logical page i to a physical page. Returns out [B,h_q,D]."""
    if q.dim() != 3 or k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("expected q [B,h_q,D] and pages [num_pages,h_kv,page_size,D]")
    B, h_q, D = q.shape
    num_pages, h_kv, page_size, Dk = k_pages.shape
    if Dk != D or not (q.dtype == k_pages.dtype == v_pages.dtype):
        raise ValueError("q and the pages disagree on D or dtype")
    dev = _dev(q, k_pages, v_pages, block_table, seq_lens)
    _lens(seq_lens, B)
    max_pages = _table(block_table, B)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    need = attn_decode_gqa_workspace_bytes(B, h_q, h_kv, D, max_pages * page_size, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(out, workspace)
    _check(load().attn_decode_gqa_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                        _ptr(seq_lens), B, h_q, h_kv, D, num_pages, page_size,
                                        max_pages, scale, _dt(q), _ptr(out), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(dev)),
           "attn_decode_gqa_paged")
    return out


def attn_kv_append_paged(k_new, v_new, k_pages, v_pages, block_table, seq_lens) -> None:
    """Write k_new/v_new [B,h_kv,D] at logical position seq_lens[b] of the paged caches (in place)."""
    num_pages, h_kv, page_size, D = k_pages.shape
    B = k_new.shape[0]
    dev = _dev(k_new, v_new, k_pages, v_pages, block_table, seq_lens)
    _lens(seq_lens, B)
    max_pages = _table(block_table, B)
    _new_rows(k_new, v_new, B, h_kv, D, k_pages.dtype)
    _check(load().attn_kv_append_paged(_ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages),
                                       _ptr(block_table), _ptr(seq_lens), B, h_kv, D, num_pages,
                                       page_size, max_pages, _dt(k_pages), _stream(dev)),
           "attn_kv_append_paged")


def attn_decode_mla_paged(q_nope_absorbed, q_rope, latent_pages, block_table, seq_lens, scale: float,
                          out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Absorbed MLA over latent pages [num_pages, page_size, d_c+d_r] bf16. Returns out [B,H,d_c]."""
    if q_nope_absorbed.dim() != 3 or q_rope.dim() != 3 or latent_pages.dim() != 3:
        raise ValueError("expected q_nope [B,H,d_c], q_rope [B,H,d_r], pages [num_pages,page_size,d_c+d_r]")
    B, H, d_c = q_nope_absorbed.shape
    d_r = q_rope.shape[2]
    num_pages, page_size, W = latent_pages.shape
    if W != d_c + d_r:
        raise ValueError("latent page rows must be d_c + d_r wide")
    for t in (q_nope_absorbed, q_rope, latent_pages):
        if t.dtype != torch.bfloat16:
            raise TypeError("MLA inputs must be bfloat16")
    dev = _dev(q_nope_absorbed, q_rope, latent_pages, block_table, seq_lens)
    _lens(seq_lens, B)
    max_pages = _table(block_table, B)
    if out is None:
        out = torch.empty((B, H, d_c), dtype=torch.bfloat16, device=dev)
    need = attn_decode_mla_workspace_bytes(B, H, d_c, d_r, max_pages * page_size)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(out, workspace)
    _check(load().attn_decode_mla_paged(_ptr(q_nope_absorbed), _ptr(q_rope), _ptr(latent_pages),
                                        _ptr(block_table), _ptr(seq_lens), B, H, d_c, d_r, num_pages,
                                        page_size, max_pages, float(scale), _ptr(out), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(dev)),
           "attn_decode_mla_paged")
    return out


def attn_latent_append_paged(latent_new, latent_pages, block_table, seq_lens, d_c: int = 512) -> None:
    """Write latent_new [B, d_c+d_r] at logical position seq_lens[b] of the latent pages (in place)."""
    num_pages, page_size, W = latent_pages.shape
    B = latent_new.shape[0]
    dev = _dev(latent_new, latent_pages, block_table, seq_lens)
    _lens(seq_lens, B)
    max_pages = _table(block_table, B)
    if tuple(latent_new.shape) != (B, W) or latent_new.dtype != torch.bfloat16:
        raise ValueError(f"latent_new must be bfloat16 [{B}, {W}]")
    _check(load().attn_latent_append_paged(_ptr(latent_new), _ptr(latent_pages), _ptr(block_table),
                                           _ptr(seq_lens), B, int(d_c), W - int(d_c), num_pages,
                                           page_size, max_pages, _stream(dev)),
           "attn_latent_append_paged")


# ----------------------------------------------------------------------------- MLA absorption products

def _bf16_3d(*ts):
    for t in ts:
        if t.dtype != torch.bfloat16 or t.dim() != 3:
            raise ValueError("expected bfloat16 tensors of rank 3")


def attn_mla_absorb_q(q_nope, w_uk, out: Optional[torch.Tensor] = None):
    """q_nope [B,H,d_h] and W_UK [H,d_c,d_h] -> q_lat [B,H,d_c] (bf16, fp32 accumulation)."""
    _bf16_3d(q_nope, w_uk)
    B, H, d_h = q_nope.shape
    if w_uk.shape[0] != H or w_uk.shape[2] != d_h:
        raise ValueError("W_UK must be [H, d_c, d_h]")
    d_c = w_uk.shape[1]
    dev = _dev(q_nope, w_uk)
    if out is None:
        out = torch.empty((B, H, d_c), dtype=torch.bfloat16, device=dev)
    _dev(out)
    _check(load().attn_mla_absorb_q(_ptr(q_nope), _ptr(w_uk), _ptr(out), B, H, d_h, d_c, _stream(dev)),
           "attn_mla_absorb_q")
    return out


def attn_mla_up_v(o_lat, w_uv, out: Optional[torch.Tensor] = None):
    """o_lat [B,H,d_c] and W_UV [H,d_c,d_v] -> out [B,H,d_v] (bf16, fp32 accumulation)."""
    _bf16_3d(o_lat, w_uv)
    B, H, d_c = o_lat.shape
    if w_uv.shape[0] != H or w_uv.shape[1] != d_c:
        raise ValueError("W_UV must be [H, d_c, d_v]")
    d_v = w_uv.shape[2]
    dev = _dev(o_lat, w_uv)
    if out is None:
        out = torch.empty((B, H, d_v), dtype=torch.bfloat16, device=dev)
    _dev(out)
    _check(load().attn_mla_up_v(_ptr(o_lat), _ptr(w_uv), _ptr(out), B, H, d_c, d_v, _stream(dev)),
           "attn_mla_up_v")
    return out
