"""Thin ctypes binding of libpackattn.so (argument marshalling only).

Every function has the name of the C entry point it calls (``include/packattn.h``)
and does no arithmetic of its own: it checks tensor placement, dtypes and
shapes, allocates the outputs with torch (device memory and streams are all
torch provides here), passes raw device pointers and the current HIP stream,
and raises :class:`PackAttnError` on a negative status.  There is no CPU
fallback: if the library is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpackattn.so")

PA_F32, PA_BF16 = 0, 1
_DTYPES = {torch.float32: PA_F32, torch.bfloat16: PA_BF16}


class PackAttnError(RuntimeError):
    """A negative status returned by libpackattn."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {pa_status_str(status)} ({status})")


class PaDualConstraint(ctypes.Structure):
    """Mirror of ``pa_dual_constraint``."""

    _fields_ = [("m_mem", ctypes.c_double), ("m_comp", ctypes.c_double), ("p", ctypes.c_double),
                ("tokens_per_frame", ctypes.c_int32)]


class PaBlockMask(ctypes.Structure):
    """Mirror of ``pa_block_mask`` (host descriptor of device storage)."""

    _fields_ = [
        ("nq", ctypes.c_int32), ("nkv", ctypes.c_int32),
        ("block_q", ctypes.c_int32), ("block_kv", ctypes.c_int32),
        ("nq_tiles", ctypes.c_int32), ("nkv_tiles", ctypes.c_int32),
        ("tile_class", ctypes.c_void_p),
        ("q_ptr", ctypes.c_void_p), ("q_cols", ctypes.c_void_p),
        ("kv_ptr", ctypes.c_void_p), ("kv_rows", ctypes.c_void_p),
        ("q_order", ctypes.c_void_p), ("kv_order", ctypes.c_void_p),
        ("pair_off", ctypes.c_void_p), ("pair_len", ctypes.c_void_p),
        ("pair_ent", ctypes.c_void_p),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()' from the repository root)")
    lib = ctypes.CDLL(LIB_PATH)
    i32, f32, vp, sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    pm = ctypes.POINTER(PaBlockMask)
    sig = {
        "pa_status_str": (ctypes.c_char_p, [i32]),
        "seq_ids_from_valid_frames": (i32, [vp, i32, i32, i32, vp, vp]),
        "build_block_mask_bytes": (sz, [i32, i32, i32, i32]),
        "build_block_mask": (i32, [vp, i32, vp, i32, i32, i32, vp, sz, pm, vp]),
        "attn_packed_fwd": (i32, [i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, pm, vp, vp,
                                  vp]),
        "attn_packed_bwd_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "attn_packed_bwd": (i32, [i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp,
                                  pm, vp, vp, vp, vp, sz, vp]),
        "attn_packed_bwd_preprocess": (i32, [i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]),
        "attn_packed_bwd_dq": (i32, [i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp, vp,
                                     sz, vp, vp, pm, vp, vp]),
        "attn_packed_bwd_dkdv": (i32, [i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp, sz,
                                       vp, vp, pm, vp, vp, vp]),
        "plan_token_packs": (i32, [vp, i32, ctypes.c_int64, vp, vp]),
        "seq_ids_from_lengths": (i32, [vp, i32, i32, vp, vp, vp]),
        "adaln_fwd": (i32, [i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "adaln_bwd_workspace_bytes": (sz, [i32, i32, i32]),
        "adaln_bwd": (i32, [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                            vp]),
        "length_bucket_rank_size": (sz, [i32, i32]),
        "length_bucket_batches": (i32, [vp, i32, ctypes.c_uint64, i32, i32, i32, i32, vp, i32,
                                        i32, vp, vp, vp, vp]),
        "dual_constraint_batch": (i32, [ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                        ctypes.c_double]),
        "fit_step_cost": (i32, [vp, vp, vp, i32, ctypes.c_double, ctypes.c_double, vp]),
        "masked_mse_workspace_bytes": (sz, [i32]),
        "masked_mse_fwd": (i32, [i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
        "masked_mse_bwd": (i32, [i32, i32, i32, vp, vp, vp, vp, f32, vp, vp]),
        "masked_mse_fwd_bwd": (i32, [i32, i32, i32, vp, vp, vp, f32, vp, vp, vp, sz, vp]),
        "pa_test_set_handover_spin_limit": (i32, [i32]),
        "pa_handover_failures": (i32, [i32]),
        "attn_packed_bwd_noalloc_max_bytes": (sz, []),
        "attn_packed_bwd_noalloc": (i32, [i32, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp,
                                          vp, vp, pm, vp, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def pa_status_str(status: int) -> str:
    return _lib.pa_status_str(int(status)).decode()


def pa_test_set_handover_spin_limit(limit: int) -> int:
    """Test hook: bound of the dK/dV kernel's P hand-over wait for later launches
    (a negative limit restores the default); returns the previous bound."""
    return int(_lib.pa_test_set_handover_spin_limit(int(limit)))


def pa_handover_failures(reset: bool = False) -> int:
    """Count of dK/dV waves whose P hand-over wait ran out (their dv rows are
    NaN) on the current device since load or the last reset; synchronous."""
    n = int(_lib.pa_handover_failures(1 if reset else 0))
    if n < 0:
        raise PackAttnError(n, "pa_handover_failures")
    return n


def _check(status: int, where: str) -> None:
    if status != 0:
        raise PackAttnError(status, where)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None, device=None, shape=None) -> None:
    """Check placement, layout, dtype and (when given) the exact shape: the C ABI
    receives bare pointers, so a buffer of the wrong size must be refused here."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


# --------------------------------------------------------------------- seq ids
def seq_ids_from_valid_frames(valid_frames: torch.Tensor, frames_padded: int,
                              tokens_per_frame: int, out: Optional[torch.Tensor] = None
                              ) -> torch.Tensor:
    """int32 ids ``[B * frames_padded * tokens_per_frame]`` on the same device."""
    _need(valid_frames, "valid_frames", torch.int32)
    B = valid_frames.numel()
    n = B * int(frames_padded) * int(tokens_per_frame)
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=valid_frames.device)
    _need(out, "out", torch.int32, valid_frames.device)
    if out.numel() != n:
        raise ValueError(f"out has {out.numel()} elements, expected {n}")
    _check(_lib.seq_ids_from_valid_frames(valid_frames.data_ptr(), B, int(frames_padded),
                                          int(tokens_per_frame), out.data_ptr(),
                                          _stream(valid_frames)), "seq_ids_from_valid_frames")
    return out


# --------------------------------------------------------------------- block mask
class BlockMask:
    """Owns the device storage of a block mask and its C descriptor."""

    def __init__(self, storage: torch.Tensor, desc: PaBlockMask):
        self.storage = storage
        self.desc = desc

    @property
    def nq_tiles(self) -> int:
        return self.desc.nq_tiles

    @property
    def nkv_tiles(self) -> int:
        return self.desc.nkv_tiles

    def _view(self, ptr: int, n: int, dtype) -> torch.Tensor:
        off = ptr - self.storage.data_ptr()
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.storage[off:off + nbytes].view(dtype)

    def tile_class(self) -> torch.Tensor:
        d = self.desc
        return self._view(d.tile_class, d.nq_tiles * d.nkv_tiles, torch.uint8).view(
            d.nq_tiles, d.nkv_tiles)

    def csr(self):
        """``(q_ptr, q_cols, kv_ptr, kv_rows)`` as device views (lists trimmed)."""
        d = self.desc
        q_ptr = self._view(d.q_ptr, d.nq_tiles + 1, torch.int32)
        kv_ptr = self._view(d.kv_ptr, d.nkv_tiles + 1, torch.int32)
        nnz_q = int(q_ptr[-1].item())
        nnz_kv = int(kv_ptr[-1].item())
        return (q_ptr, self._view(d.q_cols, nnz_q, torch.int32), kv_ptr,
                self._view(d.kv_rows, nnz_kv, torch.int32))

    def orders(self):
        d = self.desc
        return (self._view(d.q_order, d.nq_tiles, torch.int32),
                self._view(d.kv_order, d.nkv_tiles, torch.int32))

    def pairs(self):
        """``(pair_off [npairs + 1], pair_len [npairs], pair_ent)`` as device views
        (entries up to pair_off[-1], the room reserved; a pair's list is
        pair_ent[off : off + len])."""
        d = self.desc
        npairs = (d.nq_tiles + 1) // 2
        off = self._view(d.pair_off, npairs + 1, torch.int32)
        total = int(off[-1].item())
        return (off, self._view(d.pair_len, npairs, torch.int32),
                self._view(d.pair_ent, total, torch.int32))


def build_block_mask_bytes(nq: int, nkv: int, block_q: int = 128, block_kv: int = 128) -> int:
    return int(_lib.build_block_mask_bytes(int(nq), int(nkv), int(block_q), int(block_kv)))


def build_block_mask(q_seq_id: torch.Tensor, kv_seq_id: torch.Tensor, block_q: int = 128,
                     block_kv: int = 128, storage: Optional[torch.Tensor] = None) -> BlockMask:
    _need(q_seq_id, "q_seq_id", torch.int32)
    _need(kv_seq_id, "kv_seq_id", torch.int32, q_seq_id.device)
    nq, nkv = q_seq_id.numel(), kv_seq_id.numel()
    nbytes = build_block_mask_bytes(nq, nkv, block_q, block_kv)
    if nbytes == 0:
        raise PackAttnError(-2, "build_block_mask_bytes")
    if storage is None:
        storage = torch.empty(nbytes, dtype=torch.uint8, device=q_seq_id.device)
    _need(storage, "storage", torch.uint8, q_seq_id.device)
    if storage.dim() != 1:
        raise ValueError("storage must be a flat uint8 tensor")
    desc = PaBlockMask()
    _check(_lib.build_block_mask(q_seq_id.data_ptr(), nq, kv_seq_id.data_ptr(), nkv,
                                 int(block_q), int(block_kv), storage.data_ptr(),
                                 storage.numel(), ctypes.byref(desc), _stream(q_seq_id)),
           "build_block_mask")
    return BlockMask(storage, desc)


# --------------------------------------------------------------------- attention
def _attn_shapes(q, k, v):
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [tokens, heads, head_dim]")
    if k.shape != v.shape or q.shape[1:] != k.shape[1:]:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be float32 or all bfloat16")
    return q.shape[0], k.shape[0], q.shape[1], q.shape[2]


def attn_packed_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_seq_id: torch.Tensor,
                    kv_seq_id: torch.Tensor, mask: BlockMask, scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Returns ``(o [nq, H, d] like q, lse [H, nq] float32)``."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, device=q.device)
    _need(q_seq_id, "q_seq_id", torch.int32, q.device)
    _need(kv_seq_id, "kv_seq_id", torch.int32, q.device)
    nq, nkv, H, d = _attn_shapes(q, k, v)
    if q_seq_id.numel() != nq or kv_seq_id.numel() != nkv:
        raise ValueError("seq id lengths do not match q / k")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((H, nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, "out", q.dtype, q.device, q.shape)
    _need(lse_t, "lse", torch.float32, q.device, (H, nq))
    _check(_lib.attn_packed_fwd(_DTYPES[q.dtype], nq, nkv, H, d, float(scale), q.data_ptr(),
                                k.data_ptr(), v.data_ptr(), q_seq_id.data_ptr(),
                                kv_seq_id.data_ptr(), ctypes.byref(mask.desc), o.data_ptr(),
                                lse_t.data_ptr(), _stream(q)), "attn_packed_fwd")
    return o, lse_t


def attn_packed_bwd_workspace_bytes(dtype: torch.dtype, nq: int, nkv: int, heads: int,
                                    head_dim: int) -> int:
    return int(_lib.attn_packed_bwd_workspace_bytes(_DTYPES[dtype], int(nq), int(nkv),
                                                    int(heads), int(head_dim)))


def attn_packed_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                    dout: torch.Tensor, lse: torch.Tensor, q_seq_id: torch.Tensor,
                    kv_seq_id: torch.Tensor, mask: BlockMask, scale: Optional[float] = None,
                    workspace: Optional[torch.Tensor] = None, grads=None
                    ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Returns ``(dq, dk, dv)`` with the shapes and dtype of ``(q, k, v)``."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _need(t, name, q.dtype, q.device)
    _need(lse, "lse", torch.float32, q.device)
    _need(q_seq_id, "q_seq_id", torch.int32, q.device)
    _need(kv_seq_id, "kv_seq_id", torch.int32, q.device)
    nq, nkv, H, d = _attn_shapes(q, k, v)
    if o.shape != q.shape or dout.shape != q.shape or tuple(lse.shape) != (H, nq):
        raise ValueError("o / dout / lse shapes do not match q")
    if q_seq_id.numel() != nq or kv_seq_id.numel() != nkv:
        raise ValueError("seq id lengths do not match q / k")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = grads
    _need(dq, "dq", q.dtype, q.device, q.shape)
    _need(dk, "dk", q.dtype, q.device, k.shape)
    _need(dv, "dv", q.dtype, q.device, v.shape)
    nbytes = attn_packed_bwd_workspace_bytes(q.dtype, nq, nkv, H, d)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, q.device)
    _check(_lib.attn_packed_bwd(_DTYPES[q.dtype], nq, nkv, H, d, float(scale), q.data_ptr(),
                                k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                lse.data_ptr(), q_seq_id.data_ptr(), kv_seq_id.data_ptr(),
                                ctypes.byref(mask.desc), dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                _stream(q)), "attn_packed_bwd")
    return dq, dk, dv


def attn_packed_bwd_noalloc_max_bytes() -> int:
    return int(_lib.attn_packed_bwd_noalloc_max_bytes())


def attn_packed_bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                            dout: torch.Tensor, lse: torch.Tensor, q_seq_id: torch.Tensor,
                            kv_seq_id: torch.Tensor, mask: BlockMask,
                            scale: Optional[float] = None, grads=None
                            ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """attn_packed_bwd with the library's fixed per-device workspace (the C entry
    point allocates nothing; pass ``grads`` to allocate nothing here either)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _need(t, name, q.dtype, q.device)
    nq, nkv, H, d = _attn_shapes(q, k, v)
    _need(lse, "lse", torch.float32, q.device, (H, nq))
    _need(q_seq_id, "q_seq_id", torch.int32, q.device, (nq,))
    _need(kv_seq_id, "kv_seq_id", torch.int32, q.device, (nkv,))
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o / dout shapes do not match q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = grads
    _need(dq, "dq", q.dtype, q.device, q.shape)
    _need(dk, "dk", q.dtype, q.device, k.shape)
    _need(dv, "dv", q.dtype, q.device, v.shape)
    _check(_lib.attn_packed_bwd_noalloc(_DTYPES[q.dtype], nq, nkv, H, d, float(scale),
                                        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        dout.data_ptr(), lse.data_ptr(), q_seq_id.data_ptr(),
                                        kv_seq_id.data_ptr(), ctypes.byref(mask.desc),
                                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _stream(q)),
           "attn_packed_bwd_noalloc")
    return dq, dk, dv


def attn_packed_bwd_preprocess(o: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor,
                               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fill the backward workspace (row sums of ``dout * o`` and the LSE in log2 units)."""
    _need(o, "o")
    _need(dout, "dout", o.dtype, o.device)
    _need(lse, "lse", torch.float32, o.device)
    if o.dtype not in _DTYPES or o.dim() != 3 or dout.shape != o.shape:
        raise ValueError("o and dout must be matching [nq, H, d] float32/bfloat16 tensors")
    nq, H, d = o.shape
    if tuple(lse.shape) != (H, nq):
        raise ValueError("lse must be [H, nq]")
    nbytes = attn_packed_bwd_workspace_bytes(o.dtype, nq, 1, H, d)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=o.device)
    _need(workspace, "workspace", torch.uint8, o.device)
    _check(_lib.attn_packed_bwd_preprocess(_DTYPES[o.dtype], nq, H, d, o.data_ptr(),
                                           dout.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                                           workspace.numel(), _stream(o)),
           "attn_packed_bwd_preprocess")
    return workspace


def _stage_args(q, k, v, dout, lse, workspace, q_seq_id, kv_seq_id, scale):
    nq, nkv, H, d = _attn_shapes(q, k, v)
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _need(t, name, q.dtype, q.device)
    _need(lse, "lse", torch.float32, q.device, (H, nq))
    _need(workspace, "workspace", torch.uint8, q.device)
    _need(q_seq_id, "q_seq_id", torch.int32, q.device, (nq,))
    _need(kv_seq_id, "kv_seq_id", torch.int32, q.device, (nkv,))
    if dout.shape != q.shape:
        raise ValueError("dout must match q")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return nq, nkv, H, d, float(scale)


def attn_packed_bwd_dq(q, k, v, o, dout, lse, workspace, q_seq_id, kv_seq_id, mask: BlockMask,
                       scale: Optional[float] = None, dq: Optional[torch.Tensor] = None):
    """The row terms (into ``workspace``, for attn_packed_bwd_dkdv) and dq."""
    nq, nkv, H, d, scale = _stage_args(q, k, v, dout, lse, workspace, q_seq_id, kv_seq_id, scale)
    _need(o, "o", q.dtype, q.device, q.shape)
    dq = torch.empty_like(q) if dq is None else dq
    _need(dq, "dq", q.dtype, q.device, q.shape)
    _check(_lib.attn_packed_bwd_dq(_DTYPES[q.dtype], nq, nkv, H, d, scale, q.data_ptr(),
                                   k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                   lse.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                   q_seq_id.data_ptr(), kv_seq_id.data_ptr(),
                                   ctypes.byref(mask.desc), dq.data_ptr(), _stream(q)),
           "attn_packed_bwd_dq")
    return dq


def attn_packed_bwd_dkdv(q, k, v, dout, lse, workspace, q_seq_id, kv_seq_id, mask: BlockMask,
                         scale: Optional[float] = None, dk: Optional[torch.Tensor] = None,
                         dv: Optional[torch.Tensor] = None):
    nq, nkv, H, d, scale = _stage_args(q, k, v, dout, lse, workspace, q_seq_id, kv_seq_id, scale)
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dk, "dk", q.dtype, q.device, k.shape)
    _need(dv, "dv", q.dtype, q.device, v.shape)
    _check(_lib.attn_packed_bwd_dkdv(_DTYPES[q.dtype], nq, nkv, H, d, scale, q.data_ptr(),
                                     k.data_ptr(), v.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                                     workspace.data_ptr(), workspace.numel(),
                                     q_seq_id.data_ptr(), kv_seq_id.data_ptr(),
                                     ctypes.byref(mask.desc), dk.data_ptr(), dv.data_ptr(),
                                     _stream(q)), "attn_packed_bwd_dkdv")
    return dk, dv


# ------------------------------------------------------------ unpadded packing
def plan_token_packs(lengths, budget: int):
    """Host next-fit plan: returns (pack index per episode as an int32 numpy
    array, number of packs)."""
    import numpy as np
    arr = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
    pack_of = np.empty(len(arr), dtype=np.int32)
    n = ctypes.c_int32(0)
    _check(_lib.plan_token_packs(arr.ctypes.data if len(arr) else None, len(arr), int(budget),
                                 pack_of.ctypes.data if len(arr) else None, ctypes.byref(n)),
           "plan_token_packs")
    return pack_of, int(n.value)


def seq_ids_from_lengths(lengths: torch.Tensor, n_tokens: int,
                         out: Optional[torch.Tensor] = None, offsets: bool = False):
    """int32 ids ``[n_tokens]`` of an unpadded pack (and the episode offsets
    ``[B + 1]`` when ``offsets`` is true)."""
    _need(lengths, "lengths", torch.int32)
    B = lengths.numel()
    if out is None:
        out = torch.empty(int(n_tokens), dtype=torch.int32, device=lengths.device)
    _need(out, "out", torch.int32, lengths.device)
    if out.numel() != int(n_tokens):
        raise ValueError(f"out has {out.numel()} elements, expected {n_tokens}")
    off = torch.empty(B + 1, dtype=torch.int32, device=lengths.device) if offsets else None
    _check(_lib.seq_ids_from_lengths(lengths.data_ptr() if B else None, B, int(n_tokens),
                                     out.data_ptr() if n_tokens else None,
                                     off.data_ptr() if off is not None else None,
                                     _stream(lengths)), "seq_ids_from_lengths")
    return (out, off) if offsets else out


# ----------------------------------------------------------------- masked loss
def masked_mse_workspace_bytes(n: int) -> int:
    return int(_lib.masked_mse_workspace_bytes(int(n)))


def _loss_args(pred, target, seq_id, workspace):
    _need(pred, "pred")
    if pred.dtype not in _DTYPES or pred.dim() != 2:
        raise ValueError("pred must be a [n, C] float32/bfloat16 tensor")
    _need(target, "target", pred.dtype, pred.device)
    _need(seq_id, "seq_id", torch.int32, pred.device)
    n, c = pred.shape
    if target.shape != pred.shape or seq_id.numel() != n:
        raise ValueError("target must match pred and seq_id must have one id per row")
    if workspace is None:
        workspace = torch.empty(max(masked_mse_workspace_bytes(n), 1), dtype=torch.uint8,
                                device=pred.device)
    _need(workspace, "workspace", torch.uint8, pred.device)
    return n, c, workspace


def masked_mse_fwd(pred: torch.Tensor, target: torch.Tensor, seq_id: torch.Tensor,
                   stats: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 ``stats[4]`` = (loss, sum of squared errors, n_valid, 2/(n_valid*C))."""
    n, c, workspace = _loss_args(pred, target, seq_id, workspace)
    stats = torch.empty(4, dtype=torch.float32, device=pred.device) if stats is None else stats
    _need(stats, "stats", torch.float32, pred.device, (4,))
    _check(_lib.masked_mse_fwd(_DTYPES[pred.dtype], n, c, pred.data_ptr(), target.data_ptr(),
                               seq_id.data_ptr(), stats.data_ptr(), workspace.data_ptr(),
                               workspace.numel(), _stream(pred)), "masked_mse_fwd")
    return stats


def masked_mse_bwd(pred: torch.Tensor, target: torch.Tensor, seq_id: torch.Tensor,
                   stats: torch.Tensor, upstream: float = 1.0,
                   dpred: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gradient of the loss w.r.t. ``pred`` (times ``upstream``), from forward ``stats``."""
    n, c, _ = _loss_args(pred, target, seq_id, torch.empty(1, dtype=torch.uint8,
                                                            device=pred.device))
    _need(stats, "stats", torch.float32, pred.device, (4,))
    dpred = torch.empty_like(pred) if dpred is None else dpred
    _need(dpred, "dpred", pred.dtype, pred.device, pred.shape)
    _check(_lib.masked_mse_bwd(_DTYPES[pred.dtype], n, c, pred.data_ptr(), target.data_ptr(),
                               seq_id.data_ptr(), stats.data_ptr(), float(upstream),
                               dpred.data_ptr(), _stream(pred)), "masked_mse_bwd")
    return dpred


def masked_mse_fwd_bwd(pred: torch.Tensor, target: torch.Tensor, seq_id: torch.Tensor,
                       upstream: float = 1.0, stats: Optional[torch.Tensor] = None,
                       dpred: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None
                       ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Loss stats and gradient in one pass over ``pred`` and ``target``."""
    n, c, workspace = _loss_args(pred, target, seq_id, workspace)
    stats = torch.empty(4, dtype=torch.float32, device=pred.device) if stats is None else stats
    dpred = torch.empty_like(pred) if dpred is None else dpred
    _need(stats, "stats", torch.float32, pred.device, (4,))
    _need(dpred, "dpred", pred.dtype, pred.device, pred.shape)
    _check(_lib.masked_mse_fwd_bwd(_DTYPES[pred.dtype], n, c, pred.data_ptr(), target.data_ptr(),
                                   seq_id.data_ptr(), float(upstream), stats.data_ptr(),
                                   dpred.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                   _stream(pred)), "masked_mse_fwd_bwd")
    return stats, dpred


# ----------------------------------------------------------------------- AdaLN
def _adaln_args(x, seq_id, seg_offsets):
    _need(x, "x")
    if x.dtype not in _DTYPES or x.dim() != 2:
        raise ValueError("x must be a [n, D] float32/bfloat16 tensor")
    _need(seq_id, "seq_id", torch.int32, x.device)
    _need(seg_offsets, "seg_offsets", torch.int32, x.device)
    n, d = x.shape
    if seq_id.numel() != n:
        raise ValueError("seq_id must have one id per row")
    return n, d, seg_offsets.numel() - 1


def adaln_fwd(x: torch.Tensor, seq_id: torch.Tensor, seg_offsets: torch.Tensor,
              shift: torch.Tensor, scale: torch.Tensor, eps: float = 1e-6,
              out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Returns ``(y, mean, rstd)``: y like x, mean / rstd fp32 ``[n]``."""
    n, d, n_seg = _adaln_args(x, seq_id, seg_offsets)
    for name, t in (("shift", shift), ("scale", scale)):
        _need(t, name, torch.float32, x.device)
        if tuple(t.shape) != (n_seg, d):
            raise ValueError(f"{name} must be [{n_seg}, {d}]")
    if out is None:
        y = torch.empty_like(x)
        mean = torch.empty(n, dtype=torch.float32, device=x.device)
        rstd = torch.empty(n, dtype=torch.float32, device=x.device)
    else:
        y, mean, rstd = out
    _need(y, "y", x.dtype, x.device, x.shape)
    _need(mean, "mean", torch.float32, x.device, (n,))
    _need(rstd, "rstd", torch.float32, x.device, (n,))
    _check(_lib.adaln_fwd(_DTYPES[x.dtype], n, d, n_seg, float(eps), x.data_ptr(),
                          seq_id.data_ptr(), seg_offsets.data_ptr(), shift.data_ptr(),
                          scale.data_ptr(), y.data_ptr(), mean.data_ptr(), rstd.data_ptr(),
                          _stream(x)), "adaln_fwd")
    return y, mean, rstd


def adaln_bwd_workspace_bytes(n: int, d: int, n_seg: int) -> int:
    return int(_lib.adaln_bwd_workspace_bytes(int(n), int(d), int(n_seg)))


def adaln_bwd(x: torch.Tensor, dy: torch.Tensor, seq_id: torch.Tensor,
              seg_offsets: torch.Tensor, scale: torch.Tensor, mean: torch.Tensor,
              rstd: torch.Tensor, workspace: Optional[torch.Tensor] = None,
              out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Returns ``(dx, d_shift, d_scale)``."""
    n, d, n_seg = _adaln_args(x, seq_id, seg_offsets)
    _need(dy, "dy", x.dtype, x.device)
    if dy.shape != x.shape:
        raise ValueError("dy must match x")
    _need(scale, "scale", torch.float32, x.device, (n_seg, d))
    _need(mean, "mean", torch.float32, x.device, (n,))
    _need(rstd, "rstd", torch.float32, x.device, (n,))
    if out is None:
        dx = torch.empty_like(x)
        d_shift = torch.empty((n_seg, d), dtype=torch.float32, device=x.device)
        d_scale = torch.empty((n_seg, d), dtype=torch.float32, device=x.device)
    else:
        dx, d_shift, d_scale = out
    _need(dx, "dx", x.dtype, x.device, x.shape)
    _need(d_shift, "d_shift", torch.float32, x.device, (n_seg, d))
    _need(d_scale, "d_scale", torch.float32, x.device, (n_seg, d))
    nbytes = adaln_bwd_workspace_bytes(n, d, n_seg)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _need(workspace, "workspace", torch.uint8, x.device)
    _check(_lib.adaln_bwd(_DTYPES[x.dtype], n, d, n_seg, x.data_ptr(), dy.data_ptr(),
                          seq_id.data_ptr(), seg_offsets.data_ptr(), scale.data_ptr(),
                          mean.data_ptr(), rstd.data_ptr(), dx.data_ptr(), d_shift.data_ptr(),
                          d_scale.data_ptr(), workspace.data_ptr(), workspace.numel(),
                          _stream(x)), "adaln_bwd")
    return dx, d_shift, d_scale


# -------------------------------------------------------------- batch planning
def length_bucket_batches(frames, seed: int, epoch: int, pool_size: int, pad_multiple: int = 8,
                          batch_size: int = 4, dual=None, rank: int = 0, world_size: int = 1):
    """One rank's batches for one epoch (host).  ``dual = (m_mem, m_comp, p,
    tokens_per_frame)`` with ``batch_size = 0`` sizes batches by the dual
    constraint.  Returns (list of episode-index lists, padded frames per batch)."""
    import numpy as np
    fr = np.ascontiguousarray(np.asarray(frames, dtype=np.int32))
    n = len(fr)
    cap = int(_lib.length_bucket_rank_size(n, int(world_size)))
    eps = np.empty(max(cap, 1), np.int32)
    ptr = np.empty(cap + 1, np.int32)
    bfr = np.empty(max(cap, 1), np.int32)
    nb = ctypes.c_int32(0)
    d = None
    if dual is not None:
        d = PaDualConstraint(float(dual[0]), float(dual[1]), float(dual[2]), int(dual[3]))
    _check(_lib.length_bucket_batches(fr.ctypes.data if n else None, n, int(seed) & (2**64 - 1),
                                      int(epoch), int(pool_size), int(pad_multiple),
                                      int(batch_size), ctypes.byref(d) if d is not None else None,
                                      int(rank), int(world_size), eps.ctypes.data,
                                      ptr.ctypes.data, bfr.ctypes.data, ctypes.byref(nb)),
           "length_bucket_batches")
    k = nb.value
    batches = [eps[ptr[b]:ptr[b + 1]].tolist() for b in range(k)]
    return batches, bfr[:k].tolist()


def dual_constraint_batch(seq_len: float, m_mem: float, m_comp: float, p: float) -> int:
    r = int(_lib.dual_constraint_batch(float(seq_len), float(m_mem), float(m_comp), float(p)))
    _check(min(r, 0), "dual_constraint_batch")
    return r


def fit_step_cost(B, S, t, p_lo: float = 1.0, p_hi: float = 3.0):
    """Least-squares fit of t ~ a + b * B * S^p (host); returns (a, b, p)."""
    import numpy as np
    arrs = [np.ascontiguousarray(np.asarray(v, dtype=np.float64)) for v in (B, S, t)]
    out = np.empty(3, np.float64)
    _check(_lib.fit_step_cost(arrs[0].ctypes.data, arrs[1].ctypes.data, arrs[2].ctypes.data,
                              len(arrs[2]), float(p_lo), float(p_hi), out.ctypes.data),
           "fit_step_cost")
    return float(out[0]), float(out[1]), float(out[2])
