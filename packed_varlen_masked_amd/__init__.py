"""Python binding of libflashmask_mi355.so (FlashMask forward over packed
variable-length sequences on MI355X).

Argument marshalling only: every step of the path runs in the HIP library.
PyTorch supplies device memory and the current HIP stream.  There is no
fallback: if the library is missing or fails to load, importing this package
raises.

Entry points mirror include/fm_api.h:
  tile_config, auto_split, workspace_layout, workspace_size,
  preprocess_mask, build_worklist, build_plan, attn_fwd, attn_fwd_noalloc,
  attn_bwd, rope_qk_, read_status.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libflashmask_mi355.so")

FM_OK, FM_E_INVAL, FM_E_UNSUPPORTED, FM_E_WORKSPACE, FM_E_HIP = 0, 1, 2, 3, 4
FM_BF16, FM_F32 = 0, 1
FM_FLAG_NO_SKIP, FM_FLAG_PLAN_READY = 0x1, 0x2
FM_STATUS_CU0, FM_STATUS_ORDER, FM_STATUS_CUN, FM_STATUS_CAP, FM_STATUS_POS = 0x1, 0x2, 0x4, 0x8, 0x10
FULL, PARTIAL, UNMASKED = 0, 1, 2
ITEM_FIELDS = ("seq", "head", "q_tile", "kb_begin", "kb_end", "split_idx", "n_splits", "cost",
               "seq_start", "seq_end", "kb_base", "split0_slot", "zero0", "zero1", "zero2", "zero3")
ITEM_WORDS = len(ITEM_FIELDS)

_ERRNAMES = {FM_E_INVAL: "FM_E_INVAL", FM_E_UNSUPPORTED: "FM_E_UNSUPPORTED",
             FM_E_WORKSPACE: "FM_E_WORKSPACE", FM_E_HIP: "FM_E_HIP"}


class FMError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s: %s" % (_ERRNAMES.get(code, str(code)), msg))
        self.code = code


class WsLayout(ctypes.Structure):
    _fields_ = [("bytes", ctypes.c_size_t),
                ("off_hdr", ctypes.c_size_t), ("off_kb_off", ctypes.c_size_t),
                ("off_extrema", ctypes.c_size_t), ("off_items", ctypes.c_size_t),
                ("off_tile_class", ctypes.c_size_t), ("off_scratch", ctypes.c_size_t),
                ("off_partial", ctypes.c_size_t), ("off_merge", ctypes.c_size_t),
                ("scratch_bytes", ctypes.c_size_t),
                ("partial_bytes", ctypes.c_size_t),
                ("kb_cap", ctypes.c_int64), ("item_cap", ctypes.c_int64),
                ("map_cap", ctypes.c_int64), ("slot_cap", ctypes.c_int64),
                ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("max_kb_per_item", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("%s is missing: build it with `python packed_varlen_masked_amd/build.py` "
                          "(or __graft_entry__.build())" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, U, SZ, F, U64 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint,
                                ctypes.c_size_t, ctypes.c_float, ctypes.c_uint64)
    sig = {
        "fm_last_error": (ctypes.c_char_p, []),
        "fm_version": (I, []),
        "fm_self_check": (I, []),
        "fm_get_tile_config": (I, [I, I, P, P]),
        "fm_auto_split": (I, [I64, I, I, I, I]),
        "fm_workspace_layout": (I, [I64, I, I, I, I, I, I, I, P]),
        "fm_workspace_size": (SZ, [I64, I, I, I, I, I]),
        "fm_worklist_scratch_size": (SZ, [I64, I, I, I, I, I]),
        "fm_preprocess_mask": (I, [P, I, I, P, I, I64, I, P, P, I64, P, P, P]),
        "fm_build_worklist": (I, [P, I, I64, I, I, I, P, P, P, I, I, P, I64, P, P, P, I64, P, SZ, P]),
        "fm_build_plan": (I, [P, I, I64, I, I, I, P, I, I, I, I, I, I, P, SZ, P]),
        "fm_attn_fwd": (I, [P, P, P, I, I64, I, I, P, I, P, I, I, F, P, P, I, I, I, P, SZ, U, P]),
        "fm_read_status": (I, [P, P, P]),
        "fm_fused_path": (I, [I64, I, I, I, I, I, I, I, U]),
        "fm_bwd_workspace_size": (SZ, [I64, I, I, I, I]),
        "fm_attn_bwd": (I, [P, P, P, P, P, P, I, I64, I, I, P, I, P, I, I, F, P, P, P, P, SZ, P]),
        "fm_rope_qk": (I, [P, P, I, I64, I, I, I, P, I, P, P, I64, I, P, P]),
        "fm_attn_fwd_dropout": (I, [P, P, P, I, I64, I, I, P, I, P, I, I, F, P, P, I, I, I, P, SZ, U, F, U64, U64, P]),
        "fm_attn_bwd_dropout": (I, [P, P, P, P, P, P, I, I64, I, I, P, I, P, I, I, F, P, P, P, P, SZ, F, U64, U64, P]),
        "fm_attn_fwd_noalloc": (I, [P, P, P, I, I64, I, I, P, I, P, I, I, F, P, P, I, I, I, U, P]),
        "fm_attn_bwd_streams": (I, [P, P, P, P, P, P, I, I64, I, I, P, I, P, I, I, F, P, P, P, P, SZ, P, P, P, P]),
        "fm_attn_bwd_dropout_streams": (I, [P, P, P, P, P, P, I, I64, I, I, P, I, P, I, I, F, P, P, P, P, SZ, F, U64,
                                            U64, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("fm_last_error", "fm_version", "fm_self_check", "fm_get_tile_config", "fm_auto_split",
            "fm_workspace_layout", "fm_workspace_size", "fm_worklist_scratch_size",
            "fm_preprocess_mask", "fm_build_worklist", "fm_build_plan", "fm_attn_fwd",
            "fm_read_status", "fm_fused_path", "fm_bwd_workspace_size", "fm_attn_bwd", "fm_rope_qk",
            "fm_attn_fwd_dropout", "fm_attn_bwd_dropout", "fm_attn_fwd_noalloc", "fm_attn_bwd_streams",
            "fm_attn_bwd_dropout_streams")
NOALLOC_SCRATCH_BYTES = 64 << 20   # FM_NOALLOC_SCRATCH_BYTES


def _check(rc: int):
    if rc != FM_OK:
        raise FMError(rc, _lib.fm_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return FM_BF16
    if dt == torch.float32:
        return FM_F32
    raise FMError(FM_E_UNSUPPORTED, "dtype %s (bf16 and fp32 are built)" % dt)


def _workspace(ws: torch.Tensor, device) -> torch.Tensor:
    """A caller's workspace: a contiguous uint8 CUDA tensor on `device` (its
    numel() is then its size in bytes)."""
    if ws.dtype != torch.uint8 or not ws.is_contiguous() or not ws.is_cuda or ws.device != device:
        raise FMError(FM_E_INVAL, "workspace must be a contiguous uint8 CUDA tensor on the inputs' device")
    return ws


def _i32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.int32 or not t.is_contiguous() or not t.is_cuda:
        raise FMError(FM_E_INVAL, "%s must be a contiguous int32 CUDA tensor" % name)
    return t


# ---------------------------------------------------------------- queries
def version() -> int:
    return _lib.fm_version()


def self_check() -> None:
    """Host-only check of the kernels' fixed copy tables (no GPU needed)."""
    _check(_lib.fm_self_check())


def tile_config(dtype: torch.dtype, head_dim: int):
    bq, bk = ctypes.c_int(), ctypes.c_int()
    _check(_lib.fm_get_tile_config(_dtype_code(dtype), head_dim, ctypes.byref(bq), ctypes.byref(bk)))
    return bq.value, bk.value


def auto_split(N: int, B: int, H: int, dtype: torch.dtype, head_dim: int) -> int:
    s = _lib.fm_auto_split(N, B, H, _dtype_code(dtype), head_dim)
    if s < 0:
        raise FMError(FM_E_INVAL, "bad sizes")
    return s


def fused_path(N: int, B: int, H: int, head_dim: int, dtype: torch.dtype, n_vec: int, causal: bool,
               max_kb_per_item: int = -1, flags: int = 0) -> bool:
    """True if attn_fwd takes the fused one-launch path for these sizes."""
    r = _lib.fm_fused_path(N, B, H, head_dim, _dtype_code(dtype), n_vec, int(causal), max_kb_per_item, flags)
    if r < 0:
        raise FMError(FM_E_INVAL, "bad sizes")
    return r == 1


def workspace_layout(N: int, B: int, H: int, head_dim: int, block_q: int, block_k: int,
                     max_kb_per_item: int = 0, want_class_map: bool = False) -> WsLayout:
    lay = WsLayout()
    _check(_lib.fm_workspace_layout(N, B, H, head_dim, block_q, block_k, max_kb_per_item,
                                    int(want_class_map), ctypes.byref(lay)))
    return lay


def workspace_size(N: int, B: int, H: int, head_dim: int, dtype: torch.dtype, max_kb_per_item: int = -1) -> int:
    n = _lib.fm_workspace_size(N, B, H, head_dim, _dtype_code(dtype), max_kb_per_item)
    if n == 0:
        raise FMError(FM_E_INVAL, "bad sizes")
    return n


# ------------------------------------------------------------ plan stages
def preprocess_mask(startend: torch.Tensor, n_vec: int, causal: bool, cu_seqlens: torch.Tensor,
                    N: int, block_k: int):
    """Returns (kb_off [B+1], extrema [n_kb, 8], status) as device tensors;
    extrema is cut to the real block count (one host sync)."""
    cu = _i32(cu_seqlens, "cu_seqlens")
    B = cu.numel() - 1
    if N > 0:
        _i32(startend, "startend")
    dev = cu.device
    cap = -(-N // block_k) + B
    kb_off = torch.empty(B + 1, dtype=torch.int32, device=dev)
    ext = torch.empty(cap, 8, dtype=torch.int32, device=dev)
    scal = torch.zeros(2, dtype=torch.int32, device=dev)  # n_kblocks, status
    _check(_lib.fm_preprocess_mask(_ptr(startend) if N > 0 else None, n_vec, int(causal), _ptr(cu), B, N,
                                   block_k, _ptr(kb_off), _ptr(ext), cap, _ptr(scal[0:1]),
                                   ctypes.c_void_p(scal.data_ptr() + 4), _stream()))
    nkb, status = (int(x) for x in scal.cpu())
    return kb_off, ext[:nkb], status


def build_worklist(cu_seqlens: torch.Tensor, N: int, H: int, block_q: int, block_k: int,
                   kb_off: torch.Tensor, extrema: torch.Tensor, status: int, causal: bool,
                   max_kb_per_item: int = 0, want_class_map: bool = True):
    """Returns dict(items [n_items, 16], class_counts [3], tile_class (uint8) or None)."""
    cu = _i32(cu_seqlens, "cu_seqlens")
    B = cu.numel() - 1
    dev = cu.device
    lay = workspace_layout(N, B, H, 1, block_q, block_k, max_kb_per_item, want_class_map)
    scratch = torch.empty(max(lay.scratch_bytes, 1), dtype=torch.uint8, device=dev)
    items = torch.empty(lay.item_cap, ITEM_WORDS, dtype=torch.int32, device=dev)
    n_items = torch.zeros(1, dtype=torch.int32, device=dev)
    counts = torch.zeros(3, dtype=torch.int64, device=dev)
    st = torch.tensor([status], dtype=torch.int32, device=dev)
    tc = torch.empty(max(lay.map_cap, 1), dtype=torch.uint8, device=dev) if want_class_map else None
    ext = extrema.contiguous() if extrema.numel() else torch.empty(1, 8, dtype=torch.int32, device=dev)
    _check(_lib.fm_build_worklist(_ptr(cu), B, N, H, block_q, block_k, _ptr(kb_off), _ptr(ext), _ptr(st),
                                  int(causal), max_kb_per_item, _ptr(items), lay.item_cap, _ptr(n_items),
                                  _ptr(counts), _ptr(tc), lay.map_cap if tc is not None else 0,
                                  _ptr(scratch), scratch.numel(), _stream()))
    n = int(n_items.item())
    return {"items": items[:n], "class_counts": counts, "tile_class": tc, "status": int(st.item())}


@dataclasses.dataclass
class Plan:
    """A workspace holding the extrema and the work list for one
    (cu_seqlens, mask, H, tiles, split); reusable by every layer."""
    workspace: torch.Tensor
    layout: WsLayout
    N: int
    B: int
    H: int
    head_dim: int
    dtype: torch.dtype
    causal: bool
    n_vec: int
    max_kb_per_item: int

    def header(self):
        h = self.workspace[:256].view(torch.int32).cpu()
        return {"status": int(h[0]), "n_kblocks": int(h[1]), "n_items": int(h[2]),
                "sched_counter": int(h[3]), "n_slots": int(h[4]), "n_merge": int(h[5]),
                "class_counts": self.workspace[64:88].view(torch.int64).cpu().tolist()}

    def _view(self, off, n, dt, shape):
        esz = torch.empty(0, dtype=dt).element_size()
        return self.workspace[off:off + n * esz].view(dt).view(*shape)

    def kb_off(self):
        return self._view(self.layout.off_kb_off, self.B + 1, torch.int32, (self.B + 1,))

    def extrema(self, n_kb):
        return self._view(self.layout.off_extrema, n_kb * 8, torch.int32, (n_kb, 8))

    def items(self, n_items):
        return self._view(self.layout.off_items, n_items * ITEM_WORDS, torch.int32, (n_items, ITEM_WORDS))

    def tile_class(self, n):
        return self._view(self.layout.off_tile_class, n, torch.uint8, (n,))


def _resolve(N, B, H, D, dtype, block_q, block_k, max_kb_per_item):
    dq, dk = tile_config(dtype, D)
    bq, bk = (block_q or dq), (block_k or dk)
    S = auto_split(N, B, H, dtype, D) if max_kb_per_item < 0 else max_kb_per_item
    if dtype == torch.float32:
        S = 0
    return bq, bk, S


def build_plan(cu_seqlens: torch.Tensor, startend: torch.Tensor, n_vec: int, causal: bool, N: int,
               H: int, head_dim: int, dtype: torch.dtype, block_q: int = 0, block_k: int = 0,
               max_kb_per_item: int = -1, want_class_map: bool = False) -> Plan:
    cu = _i32(cu_seqlens, "cu_seqlens")
    B = cu.numel() - 1
    bq, bk, S = _resolve(N, B, H, head_dim, dtype, block_q, block_k, max_kb_per_item)
    lay = workspace_layout(N, B, H, head_dim, bq, bk, S, want_class_map)
    ws = torch.zeros(lay.bytes, dtype=torch.uint8, device=cu.device)
    _check(_lib.fm_build_plan(_ptr(cu), B, N, H, head_dim, _dtype_code(dtype),
                              _ptr(startend) if N > 0 else None, n_vec, int(causal), bq, bk, S,
                              int(want_class_map), _ptr(ws), ws.numel(), _stream()))
    return Plan(ws, lay, N, B, H, head_dim, dtype, causal, n_vec, S)


def build_plan_into(plan: Plan, cu_seqlens: torch.Tensor, startend: torch.Tensor) -> Plan:
    """Rebuilds `plan` in place (same sizes, new cu_seqlens / mask values);
    allocates nothing."""
    cu = _i32(cu_seqlens, "cu_seqlens")
    lay = plan.layout
    _check(_lib.fm_build_plan(_ptr(cu), plan.B, plan.N, plan.H, plan.head_dim, _dtype_code(plan.dtype),
                              _ptr(startend) if plan.N > 0 else None, plan.n_vec, int(plan.causal),
                              lay.block_q, lay.block_k, plan.max_kb_per_item, int(lay.off_tile_class != 0),
                              _ptr(plan.workspace), plan.workspace.numel(), _stream()))
    return plan


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
             startend: torch.Tensor, n_vec: int, causal: bool, scale: Optional[float] = None,
             plan: Optional[Plan] = None, max_kb_per_item: int = -1, block_q: int = 0,
             block_k: int = 0, flags: int = 0, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             dropout_p: float = 0.0, seed: int = 0, offset: int = 0):
    """FlashMask forward.  q, k, v: [N, H, D] bf16 or fp32 (contiguous, same
    device); cu_seqlens int32 [B+1]; startend int32 [n_vec, N] (global row
    indices).  dropout_p > 0 (bf16): attention dropout with the Philox mask
    of (seed, offset).  Returns (out [N, H, D], softmax_lse fp32 [H, N])."""
    if q.shape != k.shape or q.shape != v.shape or q.dim() != 3:
        raise FMError(FM_E_INVAL, "q, k, v must share one [N, H, D] shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise FMError(FM_E_INVAL, "q, k, v must share one dtype")
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        if not t.is_contiguous() or not t.is_cuda:
            raise FMError(FM_E_INVAL, "%s must be a contiguous CUDA tensor" % nm)
    N, H, D = q.shape
    cu = _i32(cu_seqlens, "cu_seqlens")
    B = cu.numel() - 1
    if N > 0:
        _i32(startend, "startend")
        if tuple(startend.shape) != (n_vec, N):
            raise FMError(FM_E_INVAL, "startend must be [n_vec, N] = [%d, %d]" % (n_vec, N))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if plan is not None:
        bq, bk, S = plan.layout.block_q, plan.layout.block_k, plan.max_kb_per_item
        ws = plan.workspace
        flags |= FM_FLAG_PLAN_READY
    else:
        bq, bk, S = _resolve(N, B, H, D, q.dtype, block_q, block_k, max_kb_per_item)
        if workspace is None:
            lay = workspace_layout(N, B, H, D, bq, bk, S, False)
            ws = torch.zeros(lay.bytes, dtype=torch.uint8, device=q.device)
        else:
            ws = _workspace(workspace, q.device)
    if out is None:
        out = torch.empty_like(q)
    elif (out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or not out.is_cuda
          or out.device != q.device):
        raise FMError(FM_E_INVAL, "out must be a contiguous CUDA tensor with q's shape, dtype and device")
    if lse is None:
        lse = torch.empty(H, N, dtype=torch.float32, device=q.device)
    elif (lse.dtype != torch.float32 or tuple(lse.shape) != (H, N) or not lse.is_contiguous() or not lse.is_cuda
          or lse.device != q.device):
        raise FMError(FM_E_INVAL, "lse must be a contiguous fp32 CUDA tensor [H, N] = [%d, %d] on q's device" % (H, N))
    if dropout_p > 0.0:
        _check(_lib.fm_attn_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), N, H, D, _ptr(cu), B,
                                        _ptr(startend) if N > 0 else None, n_vec, int(causal),
                                        ctypes.c_float(scale), _ptr(out), _ptr(lse), bq, bk, S, _ptr(ws),
                                        ws.numel(), flags, ctypes.c_float(dropout_p), seed, offset, _stream()))
    else:
        _check(_lib.fm_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), N, H, D, _ptr(cu), B,
                                _ptr(startend) if N > 0 else None, n_vec, int(causal), ctypes.c_float(scale),
                                _ptr(out), _ptr(lse), bq, bk, S, _ptr(ws), ws.numel(), flags, _stream()))
    return out, lse


def attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                     startend: torch.Tensor, n_vec: int, causal: bool, out: torch.Tensor, lse: torch.Tensor,
                     scale: Optional[float] = None, max_kb_per_item: int = -1, block_q: int = 0,
                     block_k: int = 0, flags: int = 0):
    """fm_attn_fwd_noalloc: the forward with the library's own per-device
    workspace array; neither this call nor the library allocates anything,
    so out [N, H, D] and lse fp32 [H, N] come from the caller.  Calls that
    can overlap on one GPU race on the array."""
    if q.shape != k.shape or q.shape != v.shape or q.dim() != 3:
        raise FMError(FM_E_INVAL, "q, k, v must share one [N, H, D] shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise FMError(FM_E_INVAL, "q, k, v must share one dtype")
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        if not t.is_contiguous() or not t.is_cuda:
            raise FMError(FM_E_INVAL, "%s must be a contiguous CUDA tensor" % nm)
    N, H, D = q.shape
    if (out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or not out.is_cuda
            or out.device != q.device):
        raise FMError(FM_E_INVAL, "out must be a contiguous CUDA tensor with q's shape, dtype and device")
    if (lse.dtype != torch.float32 or tuple(lse.shape) != (H, N) or not lse.is_contiguous() or not lse.is_cuda
            or lse.device != q.device):
        raise FMError(FM_E_INVAL, "lse must be a contiguous fp32 CUDA tensor [H, N] = [%d, %d] on q's device" % (H, N))
    cu = _i32(cu_seqlens, "cu_seqlens")
    B = cu.numel() - 1
    if N > 0:
        _i32(startend, "startend")
        if tuple(startend.shape) != (n_vec, N):
            raise FMError(FM_E_INVAL, "startend must be [n_vec, N] = [%d, %d]" % (n_vec, N))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check(_lib.fm_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q.dtype), N, H, D, _ptr(cu), B,
                                    _ptr(startend) if N > 0 else None, n_vec, int(causal), ctypes.c_float(scale),
                                    _ptr(out), _ptr(lse), block_q, block_k, max_kb_per_item, flags, _stream()))
    return out, lse


def bwd_workspace_size(N: int, B: int, H: int, head_dim: int, dtype: torch.dtype) -> int:
    n = _lib.fm_bwd_workspace_size(N, B, H, head_dim, _dtype_code(dtype))
    if n == 0:
        raise FMError(FM_E_INVAL, "bad sizes for the backward: %s" % _lib.fm_last_error().decode())
    return n


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
             dout: torch.Tensor, cu_seqlens: torch.Tensor, startend: torch.Tensor, n_vec: int, causal: bool,
             scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
             dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
             dv: Optional[torch.Tensor] = None, dropout_p: float = 0.0, seed: int = 0, offset: int = 0,
             dq_stream: Optional[torch.cuda.Stream] = None):
    """FlashMask backward.  q, k, v, out, dout: [N, H, D] bf16 (contiguous,
    same device); lse fp32 [H, N] from the forward; cu_seqlens and startend
    as for attn_fwd.  dq_stream: a second stream of the caller's on which
    the dQ launches overlap the dK/dV ones (fm_attn_bwd_streams,
    fm_attn_bwd_dropout_streams; the fork and join events are this
    binding's).
    Returns (dq, dk, dv) [N, H, D] bf16."""
    ts = ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout"))
    for t, nm in ts:
        if t.dim() != 3 or t.shape != q.shape:
            raise FMError(FM_E_INVAL, "%s must have q's [N, H, D] shape" % nm)
        if t.dtype != q.dtype:
            raise FMError(FM_E_INVAL, "%s must have q's dtype" % nm)
        if not t.is_contiguous() or not t.is_cuda:
            raise FMError(FM_E_INVAL, "%s must be a contiguous CUDA tensor" % nm)
    N, H, D = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (H, N) or not lse.is_contiguous():
        raise FMError(FM_E_INVAL, "lse must be contiguous fp32 [H, N]")
    cu = _i32(cu_seqlens, "cu_seqlens")
    B = cu.numel() - 1
    if N > 0:
        _i32(startend, "startend")
        if tuple(startend.shape) != (n_vec, N):
            raise FMError(FM_E_INVAL, "startend must be [n_vec, N] = [%d, %d]" % (n_vec, N))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = torch.zeros(bwd_workspace_size(N, B, H, D, q.dtype), dtype=torch.uint8, device=q.device)
    else:
        workspace = _workspace(workspace, q.device)
    if not lse.is_cuda or lse.device != q.device:
        raise FMError(FM_E_INVAL, "lse must be on q's device")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if (t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous() or not t.is_cuda
                or t.device != q.device):
            raise FMError(FM_E_INVAL, "%s must be a contiguous CUDA tensor with q's shape, dtype and device" % nm)
    common = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _dtype_code(q.dtype), N, H, D,
              _ptr(cu), B, _ptr(startend) if N > 0 else None, n_vec, int(causal), ctypes.c_float(scale),
              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel())
    if dropout_p > 0.0:
        if dq_stream is not None:
            fork, join = _bwd_events(q.device)
            _check(_lib.fm_attn_bwd_dropout_streams(*common, ctypes.c_float(dropout_p), seed, offset, _stream(),
                                                    ctypes.c_void_p(dq_stream.cuda_stream),
                                                    ctypes.c_void_p(fork.cuda_event), ctypes.c_void_p(join.cuda_event)))
        else:
            _check(_lib.fm_attn_bwd_dropout(*common, ctypes.c_float(dropout_p), seed, offset, _stream()))
    elif dq_stream is not None:
        fork, join = _bwd_events(q.device)
        _check(_lib.fm_attn_bwd_streams(*common, _stream(), ctypes.c_void_p(dq_stream.cuda_stream),
                                        ctypes.c_void_p(fork.cuda_event), ctypes.c_void_p(join.cuda_event)))
    else:
        _check(_lib.fm_attn_bwd(*common, _stream()))
    return dq, dk, dv


_EVENTS = {}


def _bwd_events(device):
    """The binding's fork and join events for fm_attn_bwd_streams, one pair
    per device (created, and their handles materialised, on first use)."""
    key = torch.device(device).index
    if key not in _EVENTS:
        evs = (torch.cuda.Event(), torch.cuda.Event())
        for e in evs:
            e.record()   # creates the underlying event
        torch.cuda.current_stream().synchronize()
        _EVENTS[key] = evs
    return _EVENTS[key]


def rope_qk_(q: Optional[torch.Tensor], k: Optional[torch.Tensor], cu_seqlens: torch.Tensor,
             cos: torch.Tensor, sin: torch.Tensor, inverse: bool = False,
             status: Optional[torch.Tensor] = None):
    """Rotary embedding of packed q [N, Hq, D] and k [N, Hk, D] in place
    (bf16 or fp32, contiguous; either may be None), positions restarting in
    every sample of cu_seqlens; cos, sin: fp32 [max_pos, D/2].  inverse=True
    negates sin (the backward).  status: optional int32 [1] device tensor
    that receives FM_STATUS_POS for positions outside the tables."""
    ref = q if q is not None else k
    if ref is None:
        raise FMError(FM_E_INVAL, "q and k are both None")
    N, _, D = ref.shape
    for t, nm in ((q, "q"), (k, "k")):
        if t is not None and (t.dim() != 3 or t.shape[0] != N or t.shape[2] != D or t.dtype != ref.dtype
                              or not t.is_contiguous() or not t.is_cuda):
            raise FMError(FM_E_INVAL, "%s must be a contiguous CUDA [N, H, D] tensor like the other" % nm)
    for t, nm in ((cos, "cos"), (sin, "sin")):
        if t.dtype != torch.float32 or t.dim() != 2 or t.shape[1] != D // 2 or not t.is_contiguous():
            raise FMError(FM_E_INVAL, "%s must be contiguous fp32 [max_pos, D/2]" % nm)
    if cos.shape != sin.shape:
        raise FMError(FM_E_INVAL, "cos and sin must have one shape")
    cu = _i32(cu_seqlens, "cu_seqlens")
    if status is not None and (status.dtype != torch.int32 or status.numel() < 1 or not status.is_cuda):
        raise FMError(FM_E_INVAL, "status must be an int32 CUDA tensor")
    _check(_lib.fm_rope_qk(_ptr(q), _ptr(k), _dtype_code(ref.dtype), N, 0 if q is None else q.shape[1],
                           0 if k is None else k.shape[1], D, _ptr(cu), cu.numel() - 1, _ptr(cos), _ptr(sin),
                           cos.shape[0], int(bool(inverse)), _ptr(status), _stream()))
    return q, k


def read_status(workspace: torch.Tensor) -> int:
    st = ctypes.c_int32()
    _check(_lib.fm_read_status(_ptr(workspace), _stream(), ctypes.byref(st)))
    return st.value
