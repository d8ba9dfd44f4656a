"""Python binding of the attention library: argument marshalling only.

Tensors are torch device tensors (torch supplies device memory and the current
HIP stream); every step of the computation runs in the library's HIP kernels.
Names follow the C ABI in include/fa.h.
"""
from __future__ import annotations

import math

import torch

from . import _lib


def _launch(ref: torch.Tensor, tensors, fn, *args):
    """Call library entry point ``fn`` with ``args`` and the current stream of ``ref``'s
    device, with that device current; ``ref`` must be a GPU tensor and every tensor
    passed must live on its device."""
    for t in tensors:
        if t is not None and t.device != ref.device:
            raise ValueError(f"all tensors must be on {ref.device} (got one on {t.device})")
    if ref.device.type != "cuda":
        raise ValueError(f"tensors must be GPU tensors (got {ref.device}); there is no CPU path")
    with torch.cuda.device(ref.device):
        return fn(*args, torch.cuda.current_stream(ref.device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int, shape=None) -> None:
    """Check a tensor argument's type, dtype, rank and contiguity; with ``shape`` its exact
    shape too (every output is checked this way, so an undersized caller-supplied buffer
    is rejected before any launch). Devices are checked by ``_launch``."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor (got shape {tuple(t.shape)})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _scale(scale, d: int) -> float:
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, scale=None,
        out: torch.Tensor | None = None, lse: torch.Tensor | None = None, return_lse: bool = True,
        out_f32: bool = False):
    """Exact attention forward. q [B,Sq,Hq,d], k/v [B,Skv,Hkv,d] bf16 -> (o, lse).

    o has q's shape (bf16, or fp32 with ``out_f32``); lse is fp32 [B,Hq,Sq] (None
    when ``return_lse`` is False).
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4)
    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Skv, Hkv, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k/v shape {tuple(k.shape)}/{tuple(v.shape)} does not match q {tuple(q.shape)}")
    odt = torch.float32 if out_f32 else torch.bfloat16
    if out is None:
        out = torch.empty((B, Sq, Hq, d), dtype=odt, device=q.device)
    _need(out, "out", odt, 4, (B, Sq, Hq, d))
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 3, (B, Hq, Sq))
    lib = _lib.load()
    fn = lib.fa_fwd_f32out if out_f32 else lib.fa_fwd
    st = _launch(q, (q, k, v, out, lse), fn,
                 q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                 lse.data_ptr() if lse is not None else None, B, Hq, Hkv, Sq, Skv, d, int(bool(causal)),
                 _scale(scale, d))
    _lib.check(st, "fa_fwd_f32out" if out_f32 else "fa_fwd")
    return out, lse


def decode_default_splits(B: int, Hkv: int, Skv: int, d: int) -> int:
    return int(_lib.load().fa_decode_default_splits(B, Hkv, Skv, d))


def decode_workspace_bytes(B: int, Hq: int, d: int, num_splits: int) -> int:
    return int(_lib.load().fa_decode_workspace_bytes(B, Hq, d, num_splits))


def decode_chunk_bounds(Skv: int, num_splits: int) -> list:
    """Key ranges of the chunks fa_decode / fa_decode_partials cut from a contiguous cache
    (see include/fa.h; the paged decode cuts chunks of falling size instead)."""
    tiles = (Skv + 63) // 64
    L = 64 * ((tiles + num_splits - 1) // num_splits)
    return [min(Skv, c * L) for c in range(num_splits)] + [Skv]


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, scale=None,
           num_splits: int = 0, workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
           lse: torch.Tensor | None = None):
    """Split-KV decode. q [B,Hq,d], caches [B,Skv,Hkv,d] bf16 -> (o [B,Hq,d] bf16, lse [B,Hq] fp32)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, Hq, d = q.shape
    Skv, Hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Skv, Hkv, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache shape does not match q")
    ns = num_splits if num_splits > 0 else decode_default_splits(B, Hkv, Skv, d)
    need = decode_workspace_bytes(B, Hq, d, ns)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16, 3, (B, Hq, d))
    _need(lse, "lse", torch.float32, 2, (B, Hq))
    st = _launch(q, (q, k_cache, v_cache, out, lse, workspace), _lib.load().fa_decode,
                 q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv,
                 Skv, d, _scale(scale, d), ns, workspace.data_ptr(), workspace.numel() * workspace.element_size())
    _lib.check(st, "fa_decode")
    return out, lse


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, scale=None,
                   num_splits: int = 0, out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Split-KV decode whose partials live in the library's per-GPU scratch (fa_decode_noalloc):
    the library allocates nothing. Pass ``out`` and ``lse`` to keep the call allocation-free
    on this side too. Calls that overlap on one GPU race (see include/fa.h)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, Hq, d = q.shape
    Skv, Hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Skv, Hkv, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache/v_cache shape does not match q")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16, 3, (B, Hq, d))
    _need(lse, "lse", torch.float32, 2, (B, Hq))
    st = _launch(q, (q, k_cache, v_cache, out, lse), _lib.load().fa_decode_noalloc,
                 q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv,
                 Skv, d, _scale(scale, d), int(num_splits))
    _lib.check(st, "fa_decode_noalloc")
    return out, lse


def decode_partials(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, num_splits: int,
                    scale=None):
    """Chunk partials only: (part_o fp32 [B,Hq,n,d], part_lse fp32 [B,Hq,n])."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    B, Hq, d = q.shape
    Skv, Hkv = k_cache.shape[1], k_cache.shape[2]
    part_o = torch.empty((B, Hq, num_splits, d), dtype=torch.float32, device=q.device)
    part_lse = torch.empty((B, Hq, num_splits), dtype=torch.float32, device=q.device)
    st = _launch(q, (q, k_cache, v_cache, part_o, part_lse), _lib.load().fa_decode_partials,
                 q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), part_o.data_ptr(), part_lse.data_ptr(), B,
                 Hq, Hkv, Skv, d, _scale(scale, d), num_splits)
    _lib.check(st, "fa_decode_partials")
    return part_o, part_lse


def decode_combine(part_o: torch.Tensor, part_lse: torch.Tensor):
    """Merge chunk partials: part_o [B,Hq,n,d], part_lse [B,Hq,n] fp32 -> (o bf16 [B,Hq,d], lse [B,Hq])."""
    _need(part_o, "part_o", torch.float32, 4)
    _need(part_lse, "part_lse", torch.float32, 3)
    B, Hq, n, d = part_o.shape
    if tuple(part_lse.shape) != (B, Hq, n):
        raise ValueError("part_lse shape does not match part_o")
    out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=part_o.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=part_o.device)
    st = _launch(part_o, (part_o, part_lse, out, lse), _lib.load().fa_decode_combine,
                 part_o.data_ptr(), part_lse.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, d, n)
    _lib.check(st, "fa_decode_combine")
    return out, lse


def decode_paged_default_splits(B: int, Hkv: int, max_len: int, d: int) -> int:
    """Split count fa_decode_paged uses when num_splits <= 0 (see include/fa.h)."""
    ns = decode_default_splits(B, Hkv, max_len, d)
    return max(ns, min(64, (max_len + 2047) // 2048))


def decode_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                 seq_lens: torch.Tensor, scale=None, num_splits: int = 0, workspace: torch.Tensor | None = None,
                 out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Split-KV decode over a paged cache (see fa_decode_paged in include/fa.h).

    q [B,Hq,d] bf16; k_pages, v_pages [num_pages, page_size, Hkv, d] bf16; block_table
    [B, max_blocks] int32; seq_lens [B] int32 -> (o [B,Hq,d] bf16, lse [B,Hq] fp32).
    """
    _need(q, "q", torch.bfloat16, 3)
    _need(k_pages, "k_pages", torch.bfloat16, 4)
    _need(v_pages, "v_pages", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    B, Hq, d = q.shape
    num_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if tuple(k_pages.shape) != (num_pages, page_size, Hkv, d) or tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("k_pages/v_pages shape does not match q")
    if block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table / seq_lens must have one row per sequence")
    max_blocks = block_table.shape[1]
    ns = num_splits if num_splits > 0 else decode_paged_default_splits(B, Hkv, max_blocks * page_size, d)
    if workspace is None:
        workspace = torch.empty(decode_workspace_bytes(B, Hq, d, ns), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16, 3, (B, Hq, d))
    _need(lse, "lse", torch.float32, 2, (B, Hq))
    st = _launch(q, (q, k_pages, v_pages, block_table, seq_lens, out, lse, workspace), _lib.load().fa_decode_paged,
                 q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
                 seq_lens.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, d, page_size, max_blocks,
                 num_pages, _scale(scale, d), ns, workspace.data_ptr(),
                 workspace.numel() * workspace.element_size())
    _lib.check(st, "fa_decode_paged")
    return out, lse


def bwd_workspace_bytes(B: int, Hq: int, Sq: int) -> int:
    return int(_lib.load().fa_bwd_workspace_bytes(B, Hq, Sq))


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
        causal: bool = False, scale=None, workspace: torch.Tensor | None = None, dq: torch.Tensor | None = None,
        dk: torch.Tensor | None = None, dv: torch.Tensor | None = None):
    """Attention backward (see fa_bwd in include/fa.h).

    q, o, dout [B,Sq,Hq,d] bf16; k, v [B,Skv,Hkv,d] bf16; lse [B,Hq,Sq] fp32 from ``fwd``
    -> (dq [B,Sq,Hq,d], dk, dv [B,Skv,Hkv,d]) bf16.
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, n, torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Skv, Hkv, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k/v shape {tuple(k.shape)}/{tuple(v.shape)} does not match q {tuple(q.shape)}")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("o / dout / lse shapes do not match q")
    if workspace is None:
        workspace = torch.empty(bwd_workspace_bytes(B, Hq, Sq), dtype=torch.uint8, device=q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n, shp in ((dq, "dq", q.shape), (dk, "dk", k.shape), (dv, "dv", k.shape)):
        _need(t, n, torch.bfloat16, 4)
        if tuple(t.shape) != tuple(shp):
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {tuple(shp)}")
    st = _launch(q, (q, k, v, o, lse, dout, dq, dk, dv, workspace), _lib.load().fa_bwd,
                 q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                 dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Sq, Skv, d, int(bool(causal)),
                 _scale(scale, d), workspace.data_ptr(), workspace.numel() * workspace.element_size())
    _lib.check(st, "fa_bwd")
    return dq, dk, dv


def fwd_fp8(q8: torch.Tensor, k8: torch.Tensor, vt8: torch.Tensor, q_scale: torch.Tensor, k_scale: torch.Tensor,
            v_scale: torch.Tensor, skv: int | None = None, causal: bool = False, scale=None,
            out: torch.Tensor | None = None, lse: torch.Tensor | None = None, return_lse: bool = True):
    """Attention forward on fp8 (e4m3) codes (see fa_fwd_fp8 in include/fa.h).

    q8 [B,Sq,Hq,d], k8 [B,Skv,Hkv,d], vt8 [B,Hkv,d,ldv] uint8; q_scale [B,Hq], k_scale and
    v_scale [B,Hkv] fp32 -> (o bf16 [B,Sq,Hq,d], lse fp32 [B,Hq,Sq]). ``skv`` defaults to
    k8.shape[1].
    """
    _need(q8, "q8", torch.uint8, 4)
    _need(k8, "k8", torch.uint8, 4)
    _need(vt8, "vt8", torch.uint8, 4)
    B, Sq, Hq, d = q8.shape
    Skv, Hkv = k8.shape[1], k8.shape[2]
    if skv is not None and skv != Skv:
        raise ValueError("skv must equal k8.shape[1]")
    if tuple(k8.shape) != (B, Skv, Hkv, d) or tuple(vt8.shape[:3]) != (B, Hkv, d):
        raise ValueError("k8 / vt8 shapes do not match q8")
    ldv = vt8.shape[3]
    for t, n, shp in ((q_scale, "q_scale", (B, Hq)), (k_scale, "k_scale", (B, Hkv)), (v_scale, "v_scale", (B, Hkv))):
        _need(t, n, torch.float32, 2)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {shp}")
    if out is None:
        out = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=q8.device)
    _need(out, "out", torch.bfloat16, 4, (B, Sq, Hq, d))
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q8.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 3, (B, Hq, Sq))
    st = _launch(q8, (q8, k8, vt8, q_scale, k_scale, v_scale, out, lse), _lib.load().fa_fwd_fp8,
                 q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), q_scale.data_ptr(), k_scale.data_ptr(),
                 v_scale.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None, B, Hq, Hkv, Sq,
                 Skv, ldv, d, int(bool(causal)), _scale(scale, d))
    _lib.check(st, "fa_fwd_fp8")
    return out, lse


def bpt_workspace_bytes(B: int, S: int, block_rows: int, Hq: int, d: int, d_ff: int) -> int:
    return int(_lib.load().fa_bpt_workspace_bytes(B, S, block_rows, Hq, d, d_ff))


def bpt_layer(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, w1: torch.Tensor, b1: torch.Tensor,
              w2: torch.Tensor, b2: torch.Tensor, causal: bool = False, scale=None, block_rows: int = 2048,
              workspace: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """Attention + feed-forward network, blockwise (see fa_bpt_layer in include/fa.h).

    q [B,S,Hq,d], k/v [B,S,Hkv,d], w1 [d_ff, Hq*d], b1 [d_ff], w2 [Hq*d, d_ff], b2 [Hq*d]
    (linear-layer [out, in] weights), all bf16 -> y bf16 [B, S, Hq*d].
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4)
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, S, Hkv, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k/v must be [B, S, Hkv, d] with q's B, S, d")
    dm = Hq * d
    _need(w1, "w1", torch.bfloat16, 2)
    _need(w2, "w2", torch.bfloat16, 2)
    _need(b1, "b1", torch.bfloat16, 1)
    _need(b2, "b2", torch.bfloat16, 1)
    d_ff = w1.shape[0]
    if tuple(w1.shape) != (d_ff, dm) or tuple(w2.shape) != (dm, d_ff) or tuple(b1.shape) != (d_ff,) \
            or tuple(b2.shape) != (dm,):
        raise ValueError("feed-forward weights do not match d_model = Hq * d")
    need = bpt_workspace_bytes(B, S, block_rows, Hq, d, d_ff)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, S, dm), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, 3, (B, S, dm))
    st = _launch(q, (q, k, v, w1, b1, w2, b2, out, workspace), _lib.load().fa_bpt_layer,
                 q.data_ptr(), k.data_ptr(), v.data_ptr(), w1.data_ptr(), b1.data_ptr(), w2.data_ptr(),
                 b2.data_ptr(), out.data_ptr(), B, Hq, Hkv, S, d, d_ff, int(bool(causal)), _scale(scale, d),
                 block_rows, workspace.data_ptr(), workspace.numel() * workspace.element_size())
    _lib.check(st, "fa_bpt_layer")
    return out
