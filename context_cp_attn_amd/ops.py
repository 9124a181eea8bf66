"""Thin torch binding of the C ABI: shape checks and argument marshalling only.

Every function launches on torch's current HIP stream and returns without
synchronizing.  All arithmetic happens in the HIP kernels of libcp_attn.
"""

from __future__ import annotations

import ctypes
import os

import torch

from . import _lib

# CP_ATTN_DEBUG=1: every attention call first checks its position / segment arrays
# on the device (cp_attn_check_args), synchronizes, and raises ValueError on a
# violation.  Off by default: the check costs a synchronization per call.
DEBUG = os.environ.get("CP_ATTN_DEBUG", "0") == "1"

_DT = {torch.bfloat16: _lib.CP_DTYPE_BF16, torch.float32: _lib.CP_DTYPE_F32}


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _opt_i32(t, name, n):
    if t is None:
        return None
    _dev(t, name, torch.int32)
    if t.numel() != n:
        raise ValueError(f"{name} has {t.numel()} entries, expected {n}")
    return t


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def make_args(q, k, *, causal=True, q_offset=0, k_offset=0, q_pos=None, k_pos=None, q_seg=None,
              k_seg=None, window=0, scale=0.0) -> _lib.AttnArgs:
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B,Sq,Hq,D] and k/v [B,Sk,Hkv,D]")
    if q.dtype not in _DT:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    _opt_i32(q_pos, "q_pos", Sq)
    _opt_i32(k_pos, "k_pos", Sk)
    _opt_i32(q_seg, "q_seg", B * Sq)
    _opt_i32(k_seg, "k_seg", B * Sk)
    return _lib.AttnArgs(B, Sq, Sk, Hq, Hkv, D, _DT[q.dtype], int(causal), int(q_offset),
                         int(k_offset), _ptr(q_pos), _ptr(k_pos), _ptr(q_seg), _ptr(k_seg),
                         int(window), float(scale))


_CHECK_BITS = {
    1: "q_pos must be strictly increasing and >= 0",
    2: "k_pos must be strictly increasing and >= 0",
    4: "q_seg must be non-decreasing along each batch row",
    8: "k_seg must be non-decreasing along each batch row",
}


def check_attn_args(q, k, **mask) -> list[str]:
    """The preconditions the attention kernels rely on, checked on the device.

    Returns one message per violated rule (empty list: all hold).  Synchronizes.
    """
    a = make_args(q, k, **mask)
    flags = torch.empty(1, device=q.device, dtype=torch.int32)
    _lib.check(_lib.load().cp_attn_check_args(ctypes.byref(a), flags.data_ptr(), _stream()))
    f = int(flags.item())
    return [msg for bit, msg in _CHECK_BITS.items() if f & bit]


def _debug_check(q, k, mask):
    if DEBUG:
        errs = check_attn_args(q, k, **mask)
        if errs:
            raise ValueError("; ".join(errs))


def _check_qkv(q, k, v):
    _dev(q, "q")
    _dev(k, "k", q.dtype)
    _dev(v, "v", q.dtype)
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")


def fwd_workspace(q, k, **mask) -> torch.Tensor | None:
    """Workspace for attn_fwd's split path on this problem (None if it does not split)."""
    n = _lib.load().cp_attn_fwd_workspace_size(ctypes.byref(make_args(q, k, **mask)))
    return torch.empty(n, device=q.device, dtype=torch.uint8) if n else None


def attn_fwd(q, k, v, *, out=None, lse=None, workspace=None, **mask):
    """(out [B,Sq,Hq,D] q.dtype, lse [B,Hq,Sq] fp32) of one attention block.

    mask keywords: causal, q_offset, k_offset, q_pos, k_pos, q_seg, k_seg, window, scale.
    workspace: None allocates what cp_attn_fwd_workspace_size asks for (the split
    path for small grids); a uint8 tensor is used as given; False calls cp_attn_fwd,
    which never splits.
    """
    _check_qkv(q, k, v)
    a = make_args(q, k, **mask)
    _debug_check(q, k, mask)
    B, Sq, Hq, _ = q.shape
    out = torch.empty_like(q) if out is None else _dev(out, "out", q.dtype)
    lse = torch.empty(B, Hq, Sq, device=q.device, dtype=torch.float32) if lse is None else _dev(lse, "lse", torch.float32)
    if out.shape != q.shape or lse.shape != (B, Hq, Sq):
        raise ValueError("out/lse shape mismatch")
    lib = _lib.load()
    if workspace is False:
        _lib.check(lib.cp_attn_fwd(ctypes.byref(a), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                   out.data_ptr(), lse.data_ptr(), _stream()))
        return out, lse
    if workspace is None:
        n = lib.cp_attn_fwd_workspace_size(ctypes.byref(a))
        workspace = torch.empty(n, device=q.device, dtype=torch.uint8) if n else None
    ws_ptr, ws_n = (None, 0) if workspace is None else (_dev(workspace, "workspace").data_ptr(), workspace.numel())
    _lib.check(lib.cp_attn_fwd_ws(ctypes.byref(a), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  out.data_ptr(), lse.data_ptr(), ws_ptr, ws_n, _stream()))
    return out, lse


def attn_fwd_merge(q, k, v, out_acc, lse_acc, **mask):
    """Fused ring step, in place: (out_acc, lse_acc) <- merge((out_acc, lse_acc), attn_fwd(q, k, v)).

    out_acc [B,Sq,Hq,D] fp32, lse_acc [B,Hq,Sq] fp32; the block result is merged in
    fp32.  Same mask keywords as attn_fwd.
    """
    _check_qkv(q, k, v)
    a = make_args(q, k, **mask)
    _debug_check(q, k, mask)
    B, Sq, Hq, _ = q.shape
    _dev(out_acc, "out_acc", torch.float32)
    _dev(lse_acc, "lse_acc", torch.float32)
    if out_acc.shape != q.shape or lse_acc.shape != (B, Hq, Sq):
        raise ValueError("out_acc/lse_acc shape mismatch")
    lib = _lib.load()
    _lib.check(lib.cp_attn_fwd_merge(ctypes.byref(a), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     out_acc.data_ptr(), lse_acc.data_ptr(), _stream()))
    return out_acc, lse_acc


def bwd_workspace(q, k, **mask) -> torch.Tensor:
    a = make_args(q, k, **mask)
    n = _lib.load().cp_attn_bwd_workspace_size(ctypes.byref(a))
    return torch.empty(max(n, 16), device=q.device, dtype=torch.uint8)


def attn_bwd(q, k, v, out, lse, dout, *, dq=None, dk=None, dv=None, accumulate=False, workspace=None,
             rows_ready=False, **mask):
    """(dq, dk, dv) float32 of one attention block given the rows' final (out, lse).

    rows_ready: ``workspace`` still holds the per-row values an earlier call with the
    same out, lse and dout (and the same query shape) derived (cp_attn_bwd_rows_ready)."""
    _check_qkv(q, k, v)
    _dev(out, "out", q.dtype)
    _dev(dout, "dout", q.dtype)
    _dev(lse, "lse", torch.float32)
    a = make_args(q, k, **mask)
    _debug_check(q, k, mask)
    f32 = dict(device=q.device, dtype=torch.float32)
    if accumulate and (dq is None or dk is None or dv is None):
        raise ValueError("accumulate needs dq, dk and dv")
    dq = torch.empty(q.shape, **f32) if dq is None else _dev(dq, "dq", torch.float32)
    dk = torch.empty(k.shape, **f32) if dk is None else _dev(dk, "dk", torch.float32)
    dv = torch.empty(v.shape, **f32) if dv is None else _dev(dv, "dv", torch.float32)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("dq, dk, dv must be shaped like q, k, v")
    if out.shape != q.shape or dout.shape != q.shape or lse.shape != (q.shape[0], q.shape[2], q.shape[1]):
        raise ValueError("out/dout must be shaped like q and lse [B,Hq,Sq]")
    lib = _lib.load()
    need = lib.cp_attn_bwd_workspace_size(ctypes.byref(a))
    if rows_ready and workspace is None:
        raise ValueError("rows_ready needs the workspace of an earlier call")
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=q.device, dtype=torch.uint8)
    fn = lib.cp_attn_bwd_rows_ready if rows_ready else lib.cp_attn_bwd
    _lib.check(fn(ctypes.byref(a), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                               out.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                               dk.data_ptr(), dv.data_ptr(), int(bool(accumulate)),
                               workspace.data_ptr(), workspace.numel(), _stream()))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, out, lse, dout, dq, dk, dv, *, accumulate=False, **mask):
    """attn_bwd into the caller's dq, dk, dv with the library's own device scratch
    (cp_attn_bwd_noalloc): no device memory is allocated, here or in the library.
    Calls that may overlap on one device race on that scratch."""
    _check_qkv(q, k, v)
    _dev(out, "out", q.dtype)
    _dev(dout, "dout", q.dtype)
    _dev(lse, "lse", torch.float32)
    for t, n, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _dev(t, n, torch.float32)
        if t.shape != ref.shape:
            raise ValueError(f"{n} must be shaped like {n[1]} {tuple(ref.shape)}, got {tuple(t.shape)}")
    if out.shape != q.shape or dout.shape != q.shape or lse.shape != (q.shape[0], q.shape[2], q.shape[1]):
        raise ValueError("out/dout must be shaped like q and lse [B,Hq,Sq]")
    a = make_args(q, k, **mask)
    _debug_check(q, k, mask)
    _lib.check(_lib.load().cp_attn_bwd_noalloc(ctypes.byref(a), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                               out.data_ptr(), lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                               dk.data_ptr(), dv.data_ptr(), int(bool(accumulate)), _stream()))
    return dq, dk, dv


def lse_merge(out_acc, lse_acc, out_blk, lse_blk):
    """In place: (out_acc, lse_acc) <- merge((out_acc, lse_acc), (out_blk, lse_blk))."""
    _dev(out_acc, "out_acc", torch.float32)
    _dev(lse_acc, "lse_acc", torch.float32)
    _dev(out_blk, "out_blk")
    _dev(lse_blk, "lse_blk", torch.float32)
    if out_blk.dtype not in _DT or out_acc.shape != out_blk.shape or lse_acc.shape != lse_blk.shape:
        raise ValueError("merge shape/dtype mismatch")
    B, S, H, D = out_acc.shape
    if lse_acc.shape != (B, H, S):
        raise ValueError("lse must be [B,H,S]")
    _lib.check(_lib.load().cp_lse_merge(B, S, H, D, out_acc.data_ptr(), lse_acc.data_ptr(),
                                        out_blk.data_ptr(), lse_blk.data_ptr(), _DT[out_blk.dtype],
                                        _stream()))
    return out_acc, lse_acc


def ulysses_relayout(x, P, out=None):
    """[P][B][S/P][H][D] -> [P][B][S][H/P][D] (sequence -> head, all ranks)."""
    _dev(x, "x")
    if x.dim() != 5 or x.shape[0] != P:
        raise ValueError("x must be [P][B][S/P][H][D]")
    _, B, Sp, H, D = x.shape
    if H % P:
        raise _lib.CpError(_lib.CP_ERR_INVALID, f"heads {H} not divisible by the Ulysses degree {P}")
    out = torch.empty(P, B, Sp * P, H // P, D, device=x.device, dtype=x.dtype) if out is None else _dev(out, "out", x.dtype)
    _lib.check(_lib.load().cp_ulysses_relayout(x.data_ptr(), out.data_ptr(), P, B, Sp * P, H, D,
                                               x.element_size(), _stream()))
    return out


def ulysses_relayout_inv(y, P, out=None):
    """[P][B][S][H/P][D] -> [P][B][S/P][H][D] (head -> sequence, all ranks)."""
    _dev(y, "y")
    if y.dim() != 5 or y.shape[0] != P:
        raise ValueError("y must be [P][B][S][H/P][D]")
    _, B, S, Hp, D = y.shape
    if S % P:
        raise _lib.CpError(_lib.CP_ERR_INVALID, f"seqlen {S} not divisible by the Ulysses degree {P}")
    out = torch.empty(P, B, S // P, Hp * P, D, device=y.device, dtype=y.dtype) if out is None else _dev(out, "out", y.dtype)
    _lib.check(_lib.load().cp_ulysses_relayout_inv(y.data_ptr(), out.data_ptr(), P, B, S, Hp * P, D,
                                                   y.element_size(), _stream()))
    return out


def ulysses_relayout_ex(x, P, *, groups=1, rep=1, inverse=False, out=None):
    """General Ulysses relayout of ``groups`` independent groups with every head
    replicated ``rep`` times (head j of the replicated set = head j // rep).

    forward: x [G][P][B][S/P][H][D] -> [G][P][B][S][H*rep/P][D]
    inverse: x [G][P][B][S][H*rep/P][D] -> [G][P][B][S/P][H][D]; with rep > 1 the
    copies of each head are summed (float32 gradients).
    """
    _dev(x, "x")
    if x.dim() != 6 or x.shape[0] != groups or x.shape[1] != P:
        raise ValueError("x must be [G][P][B][...][...][D]")
    G, _, B, s_in, h_in, D = x.shape
    if not inverse:
        S, H = s_in * P, h_in
        if (H * rep) % P:
            raise _lib.CpError(_lib.CP_ERR_INVALID, f"heads {H} x rep {rep} not divisible by {P}")
        shape = (G, P, B, S, H * rep // P, D)
    else:
        S, H = s_in, h_in * P // rep
        if S % P or (h_in * P) % rep:
            raise _lib.CpError(_lib.CP_ERR_INVALID, "sequence or replicated heads not divisible")
        shape = (G, P, B, S // P, H, D)
    out = torch.empty(shape, device=x.device, dtype=x.dtype) if out is None else _dev(out, "out", x.dtype)
    if tuple(out.shape) != shape:
        raise ValueError(f"out must be {shape}")
    a = _lib.RelayoutArgs(groups=G, P=P, batch=B, seqlen=S, heads=H, head_dim=D, elem_bytes=x.element_size(),
                          rep=rep, inverse=int(bool(inverse)))
    _lib.check(_lib.load().cp_ulysses_relayout_ex(ctypes.byref(a), x.data_ptr(), out.data_ptr(), _stream()))
    return out


def pad_rows(x, seqlen_out, fill=0, out=None):
    """x [B][S][...] -> [B][seqlen_out][...]: the first min(S, seqlen_out) rows
    copied, rows beyond S filled with the 32-bit word ``fill`` (0 for data, a fresh
    segment id for int32 segment ids); seqlen_out < S truncates."""
    _dev(x, "x")
    if x.dim() < 2:
        raise ValueError("x must be [B][S][...]")
    B, S = x.shape[0], x.shape[1]
    row_bytes = (x[0, 0].numel() if x.dim() > 2 else 1) * x.element_size()
    shape = (B, seqlen_out) + tuple(x.shape[2:])
    out = torch.empty(shape, device=x.device, dtype=x.dtype) if out is None else _dev(out, "out", x.dtype)
    if tuple(out.shape) != shape:
        raise ValueError(f"out must be {shape}")
    _lib.check(_lib.load().cp_pad_rows(x.data_ptr(), out.data_ptr(), B, S, seqlen_out, row_bytes,
                                       int(fill) & 0xFFFFFFFF, _stream()))
    return out


DUAL_CHUNK_SWAP, STRIPED = 0, 1


def zigzag_reorder(x, P, inverse=False, strategy=DUAL_CHUNK_SWAP, out=None):
    """Load-balancing reorder of x [B][S][...] along S into the P ranks' shares in rank
    order; inverse undoes it.  strategy DUAL_CHUNK_SWAP (zigzag chunks r, 2P-1-r) or
    STRIPED (tokens r, r+P, ...)."""
    _dev(x, "x")
    if x.dim() < 2:
        raise ValueError("x must be [B][S][...]")
    B, S = x.shape[0], x.shape[1]
    row_bytes = x[0, 0].numel() * x.element_size() if x.numel() else 0
    out = torch.empty_like(x) if out is None else _dev(out, "out", x.dtype)
    _lib.check(_lib.load().cp_zigzag_reorder(x.data_ptr(), out.data_ptr(), B, S, row_bytes, P,
                                             int(strategy), int(bool(inverse)), _stream()))
    return out
