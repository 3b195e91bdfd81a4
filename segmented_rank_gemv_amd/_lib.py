"""ctypes declarations of include/lora_sgmv.h and thin wrappers with the same names."""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "liblora_sgmv.so")

DTYPE_F32, DTYPE_BF16 = 0, 1
FAMILY_QKV, FAMILY_O, FAMILY_GATE_UP, FAMILY_DOWN = 0, 1, 2, 3
PATH_AUTO, PATH_VALU, PATH_MFMA, PATH_FUSED = 0, 1, 2, 3
_TARGET_BITS = {"q": 1, "k": 2, "v": 4, "o": 8}
_DTYPES = {"f32": DTYPE_F32, "bf16": DTYPE_BF16}


class LoraError(Exception):
    """A non-zero lora_status_t.  Codes 1-4 (bad argument, invalid adapter,
    slot out of range, capacity) and 7-8 (no free slot, adapter not active)
    also derive from ValueError."""

    def __init__(self, code: int, name: str, where: str):
        super().__init__(f"{where}: {name} ({code})")
        self.code = code
        self.name = name


class _LoraValueError(LoraError, ValueError):
    pass


class _LoraDims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_lora_rank", ctypes.c_int32), ("max_num_loras", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("intermediate_size", ctypes.c_int32)]


class _LoraRouting(ctypes.Structure):
    _fields_ = [("lora_ids", ctypes.c_void_p), ("grouped_offsets", ctypes.c_void_p),
                ("num_groups", ctypes.c_int32), ("end", ctypes.c_int64),
                ("host_lora_ids", ctypes.c_void_p), ("host_grouped_offsets", ctypes.c_void_p),
                ("token_rows", ctypes.c_void_p), ("num_rows", ctypes.c_int64)]


MAX_HOST_GROUPS = 64


class _LoraOptions(ctypes.Structure):
    _fields_ = [("long_delta", ctypes.c_int32), ("fused_max_tokens", ctypes.c_int32), ("splitk_short", ctypes.c_int32),
                ("fused_feature_tile", ctypes.c_int32), ("fused_k_rotation", ctypes.c_int32),
                ("fold_slabs", ctypes.c_int32)]


@dataclass(frozen=True)
class LoraOptions:
    """Tuning choices of lora_sgmv_delta (lora_options_t).  -1 (0 for
    fused_feature_tile) keeps the library default; none changes what is
    computed, only which kernels compute it."""
    long_delta: int = -1
    fused_max_tokens: int = -1
    splitk_short: int = -1
    fused_feature_tile: int = 0
    fused_k_rotation: int = -1
    fold_slabs: int = -1

    def c(self) -> _LoraOptions:
        return _LoraOptions(self.long_delta, self.fused_max_tokens, self.splitk_short,
                            self.fused_feature_tile, self.fused_k_rotation, self.fold_slabs)


class LoraRouting:
    """The routing triple of a batch for the device calls: lora_ids and
    grouped_offsets as int32 GPU tensors, `end` and the group count on the
    host, and (by default) host copies of the two arrays, which the library
    passes to the kernels as launch arguments.  For per-token routing,
    token_rows (int32 GPU tensor, sorted position -> row of x and y) and
    num_rows (rows of x and y) are set as well."""

    def __init__(self, lora_ids, grouped_offsets, num_groups: int, end: int,
                 host_lora_ids: Optional[np.ndarray] = None,
                 host_grouped_offsets: Optional[np.ndarray] = None,
                 token_rows=None, num_rows: int = 0):
        self.token_rows = token_rows
        self.num_rows = int(num_rows)
        self.lora_ids = lora_ids
        self.grouped_offsets = grouped_offsets
        self.num_groups = int(num_groups)
        self.end = int(end)
        self.host_lora_ids = None if host_lora_ids is None else np.ascontiguousarray(host_lora_ids, np.int32)
        self.host_grouped_offsets = (None if host_grouped_offsets is None
                                     else np.ascontiguousarray(host_grouped_offsets, np.int32))

    @classmethod
    def from_host(cls, routing: Dict[str, object], device="cuda", host_copy: bool = True,
                  device_arrays: bool = True):
        """Upload a lora_build_routing result; keep host copies if host_copy."""
        import torch
        ids = np.ascontiguousarray(routing["lora_ids"], np.int32)
        offs = np.ascontiguousarray(routing["grouped_offsets"], np.int32)
        d_ids = d_offs = None
        if device_arrays:
            d_ids = torch.from_numpy(ids if ids.size else np.zeros(1, np.int32)).to(device)
            d_offs = torch.from_numpy(offs).to(device)
        rows, n_rows = None, 0
        if "token_indices_sorted" in routing:
            idx = np.ascontiguousarray(routing["token_indices_sorted"][:routing["end"]], np.int32)
            rows = torch.from_numpy(idx if idx.size else np.zeros(1, np.int32)).to(device)
            n_rows = len(routing["token_indices_sorted"])
        return cls(d_ids, d_offs, routing["num_groups"], routing["end"],
                   ids if host_copy else None, offs if host_copy else None, rows, n_rows)

    def c(self) -> _LoraRouting:
        r = _LoraRouting()
        r.lora_ids = None if self.lora_ids is None else _dev_ptr(self.lora_ids, "lora_ids")
        r.grouped_offsets = None if self.grouped_offsets is None else _dev_ptr(self.grouped_offsets,
                                                                             "grouped_offsets")
        r.num_groups = self.num_groups
        r.end = self.end
        r.host_lora_ids = None if self.host_lora_ids is None else self.host_lora_ids.ctypes.data
        r.host_grouped_offsets = (None if self.host_grouped_offsets is None
                                  else self.host_grouped_offsets.ctypes.data)
        r.token_rows = None if self.token_rows is None else _dev_ptr(self.token_rows, "token_rows")
        r.num_rows = self.num_rows
        return r


@dataclass(frozen=True)
class LoraDims:
    """Model and LoRA capacity dimensions.  The defaults of max_lora_rank and
    max_num_loras are the pages' LoRAConfig defaults (16 and 1)."""
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    max_lora_rank: int = 16
    max_num_loras: int = 1
    dtype: str = "bf16"
    intermediate_size: int = 0  # MLP width; 0 = MLP not targeted

    def c(self) -> _LoraDims:
        return _LoraDims(self.hidden, self.n_heads, self.n_kv_heads, self.head_dim,
                         self.max_lora_rank, self.max_num_loras, _DTYPES[self.dtype],
                         self.intermediate_size)


def library_path() -> str:
    """The library this process loads: liblora_sgmv.so next to this file."""
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run segmented_rank_gemv_amd.build.build()")
    lib = ctypes.CDLL(path)
    P, i32, i64, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
    D = ctypes.POINTER(_LoraDims)
    lib.lora_abi_version.restype = i32
    lib.lora_abi_version.argtypes = []
    lib.lora_status_string.restype = ctypes.c_char_p
    lib.lora_status_string.argtypes = [i32]
    lib.lora_family_shape.restype = i32
    lib.lora_family_shape.argtypes = [D, i32, P, P, P, P]
    lib.lora_pack_adapter.restype = i32
    lib.lora_pack_adapter.argtypes = [D, i32, ctypes.c_float, i32, i32, u32] + [P] * 12
    lib.lora_pack_family.restype = i32
    lib.lora_pack_family.argtypes = [D, i32, i32, ctypes.c_float, i32, i32, u32, P, P, P, P]
    lib.lora_build_routing.restype = i32
    lib.lora_build_routing.argtypes = [i32, P, P, i32, P, P, P, P, P, P]
    lib.lora_build_token_routing.restype = i32
    lib.lora_build_token_routing.argtypes = [i32, P, i32, P, P, P, P, P]
    lib.lora_sgmv_workspace_bytes.restype = i32
    lib.lora_sgmv_workspace_bytes.argtypes = [D, i32, i64, ctypes.POINTER(ctypes.c_size_t)]
    RT = ctypes.POINTER(_LoraRouting)
    lib.lora_sgmv_shrink.restype = i32
    lib.lora_sgmv_shrink.argtypes = [D, i32, P, i64, P, RT, P, P, ctypes.c_size_t, i32, P]
    lib.lora_sgmv_expand.restype = i32
    lib.lora_sgmv_expand.argtypes = [D, i32, P, P, P, RT, P, i64, i32, P]
    lib.lora_sgmv_delta.restype = i32
    lib.lora_sgmv_delta.argtypes = [D, i32, P, i64, P, P, P, RT, P, i64, P, ctypes.c_size_t, i32,
                                    ctypes.POINTER(_LoraOptions), P]
    lib.lora_sgmv_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.lora_sgmv_noalloc_scratch_bytes.argtypes = []
    lib.lora_sgmv_delta_noalloc.restype = i32
    lib.lora_sgmv_delta_noalloc.argtypes = [D, i32, P, i64, P, P, P, RT, P, i64, i32,
                                            ctypes.POINTER(_LoraOptions), P]
    lib.lora_pack_bias.restype = i32
    lib.lora_pack_bias.argtypes = [D, i32, u32, P, P]
    I32P, I64P = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    lib.lora_cache_create.restype = i32
    lib.lora_cache_create.argtypes = [i32, i32, ctypes.POINTER(P)]
    lib.lora_cache_destroy.restype = None
    lib.lora_cache_destroy.argtypes = [P]
    lib.lora_cache_activate.restype = i32
    lib.lora_cache_activate.argtypes = [P, i64, I32P, I32P, I64P]
    lib.lora_cache_activate_batch.restype = i32
    lib.lora_cache_activate_batch.argtypes = [P, i32, P, P, P, P, I32P]
    lib.lora_cache_unload.restype = i32
    lib.lora_cache_unload.argtypes = [P, i64, I32P]
    lib.lora_cache_pin.restype = i32
    lib.lora_cache_pin.argtypes = [P, i64, i32, I32P, I32P, I64P]
    lib.lora_cache_lookup.restype = i32
    lib.lora_cache_lookup.argtypes = [P, i64, I32P]
    lib.lora_cache_slot_table.restype = i32
    lib.lora_cache_slot_table.argtypes = [P, i32, P, P]
    lib.lora_write_slot.restype = i32
    lib.lora_write_slot.argtypes = [D, i32] + [P] * 8 + [P]
    lib.lora_reset_slot.restype = i32
    lib.lora_reset_slot.argtypes = [D, i32] + [P] * 4 + [P]
    _lib = lib
    return lib


def lora_status_string(code: int) -> str:
    return _load().lora_status_string(int(code)).decode()


def _check(code: int, where: str):
    if code != 0:
        name = lora_status_string(code)
        cls = _LoraValueError if (1 <= code <= 4 or code in (7, 8)) else LoraError
        raise cls(code, name, where)


def lora_abi_version() -> int:
    return int(_load().lora_abi_version())


def _np_ptr(a: Optional[np.ndarray]) -> Optional[int]:
    return None if a is None else a.ctypes.data


# ----------------------------------------------------------------------------- host
def lora_family_shape(dims: LoraDims, family: int) -> Tuple[int, int, Tuple[int, ...], int]:
    """(in_features, n_slices, slice_widths, out_features)."""
    i = np.zeros(1, np.int32)
    n = np.zeros(1, np.int32)
    w = np.zeros(4, np.int32)
    o = np.zeros(1, np.int32)
    dc = dims.c()
    _check(_load().lora_family_shape(ctypes.byref(dc), family, _np_ptr(i), _np_ptr(n), _np_ptr(w),
                                     _np_ptr(o)), "lora_family_shape")
    return int(i[0]), int(n[0]), tuple(int(v) for v in w[:int(n[0])]), int(o[0])


family_shape = lora_family_shape


def a_tiled_shape(rows: int, K: int) -> Tuple[int, int, int, int]:
    """Shape [blocks, K/8, 16, 8] of one slot of an A stack in the device
    layout (rows rounded up to a multiple of 16)."""
    return ((rows + 15) // 16, K // 8, 16, 8)


def untile_a(a: np.ndarray, rows: int) -> np.ndarray:
    """Device-layout A slot(s) [..., blocks, K/8, 16, 8] -> logical
    [..., rows, K] (drops the zero rows added up to a multiple of 16)."""
    nb, p = a.shape[-4], a.shape[-3]
    lead = a.shape[:-4]
    m = np.swapaxes(a, -3, -2).reshape(*lead, nb * 16, p * 8)
    return m[..., :rows, :]


def tile_a(a: np.ndarray) -> np.ndarray:
    """Logical A [..., rows, K] -> device layout [..., blocks, K/8, 16, 8]."""
    rows, K = a.shape[-2], a.shape[-1]
    nb = (rows + 15) // 16
    lead = a.shape[:-2]
    pad = np.zeros((*lead, nb * 16, K), a.dtype)
    pad[..., :rows, :] = a
    return np.ascontiguousarray(np.swapaxes(pad.reshape(*lead, nb, 16, K // 8, 8), -3, -2))


def lora_pack_adapter(dims: LoraDims, rank: int, lora_alpha: float, use_rslora: bool,
                      bias_none: bool, targets: Sequence[str],
                      weights: Dict[str, Tuple[np.ndarray, np.ndarray]],
                      target_mask: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Pack one adapter of one layer; returns host arrays A_qkv, B_qkv, A_o,
    B_o (uint16 bf16 patterns or float32).  A_qkv and A_o come in the device's
    tiled layout (a_tiled_shape; untile_a gives the logical [rows, K])."""
    R = dims.max_lora_rank
    nq, nkv = dims.n_heads * dims.head_dim, dims.n_kv_heads * dims.head_dim
    st = np.uint16 if dims.dtype == "bf16" else np.float32
    out = {"A_qkv": np.empty(a_tiled_shape(3 * R, dims.hidden), st),
           "B_qkv": np.empty((nq + 2 * nkv, R), st),
           "A_o": np.empty(a_tiled_shape(R, nq), st), "B_o": np.empty((dims.hidden, R), st)}
    if target_mask is None:
        target_mask = 0
        for t in targets:
            target_mask |= _TARGET_BITS[t]
    keep = []
    ptrs = []
    for i, p in enumerate("qkvo"):
        if (target_mask >> i) & 1 and p in weights:
            a = np.ascontiguousarray(weights[p][0], dtype=np.float32)
            b = np.ascontiguousarray(weights[p][1], dtype=np.float32)
            keep += [a, b]
            ptrs += [_np_ptr(a), _np_ptr(b)]
        else:
            ptrs += [None, None]
    dc = dims.c()
    _check(_load().lora_pack_adapter(ctypes.byref(dc), int(rank), float(lora_alpha),
                                     int(bool(use_rslora)), int(bool(bias_none)), int(target_mask),
                                     *ptrs, _np_ptr(out["A_qkv"]), _np_ptr(out["B_qkv"]),
                                     _np_ptr(out["A_o"]), _np_ptr(out["B_o"])),
           "lora_pack_adapter")
    return out


def lora_pack_family(dims: LoraDims, family: int, rank: int, lora_alpha: float, use_rslora: bool,
                     bias_none: bool, slices: Sequence[Optional[Tuple[np.ndarray, np.ndarray]]]
                     ) -> Dict[str, np.ndarray]:
    """Pack one adapter's projections of one family: slices[s] = (lora_A
    [rank, in], lora_B [width_s, rank]) in the family's slice order, or None
    for an untargeted slice.  Returns {"A": tiled A, "B": [out, R]}."""
    in_f, n_s, widths, out_f = lora_family_shape(dims, family)
    if len(slices) != n_s:
        raise ValueError(f"family {family} has {n_s} slices")
    R = dims.max_lora_rank
    st = np.uint16 if dims.dtype == "bf16" else np.float32
    out = {"A": np.empty(a_tiled_shape(n_s * R, in_f), st), "B": np.empty((out_f, R), st)}
    keep, mask = [], 0
    a_ptrs = (ctypes.c_void_p * max(n_s, 1))()
    b_ptrs = (ctypes.c_void_p * max(n_s, 1))()
    for i, sl in enumerate(slices):
        if sl is None:
            continue
        a = np.ascontiguousarray(sl[0], dtype=np.float32)
        b = np.ascontiguousarray(sl[1], dtype=np.float32)
        keep += [a, b]
        a_ptrs[i], b_ptrs[i] = _np_ptr(a), _np_ptr(b)
        mask |= 1 << i
    dc = dims.c()
    _check(_load().lora_pack_family(ctypes.byref(dc), int(family), int(rank), float(lora_alpha),
                                    int(bool(use_rslora)), int(bool(bias_none)), mask,
                                    ctypes.cast(a_ptrs, ctypes.c_void_p), ctypes.cast(b_ptrs, ctypes.c_void_p),
                                    _np_ptr(out["A"]), _np_ptr(out["B"])),
           "lora_pack_family")
    return out


def lora_pack_bias(dims: LoraDims, family: int, slices: Sequence[Optional[np.ndarray]]) -> np.ndarray:
    """Pack one adapter's LoRA bias of one family: slices[s] = bias [width_s]
    in the family's slice order, or None (zero).  Stored as given (only B
    carries the scaling); returns [out] in the stack dtype (uint16 bf16
    patterns or float32)."""
    in_f, n_s, widths, out_f = lora_family_shape(dims, family)
    if len(slices) != n_s:
        raise ValueError(f"family {family} has {n_s} slices")
    st = np.uint16 if dims.dtype == "bf16" else np.float32
    out = np.empty(out_f, st)
    keep, mask = [], 0
    ptrs = (ctypes.c_void_p * max(n_s, 1))()
    for i, b in enumerate(slices):
        if b is None:
            continue
        b = np.ascontiguousarray(b, dtype=np.float32).reshape(-1)
        if b.size != widths[i]:
            raise ValueError(f"bias slice {i} must have {widths[i]} entries")
        keep.append(b)
        ptrs[i] = _np_ptr(b)
        mask |= 1 << i
    dc = dims.c()
    _check(_load().lora_pack_bias(ctypes.byref(dc), int(family), mask, ctypes.cast(ptrs, ctypes.c_void_p),
                                  _np_ptr(out)), "lora_pack_bias")
    return out


def lora_build_routing(request_slot: np.ndarray, row_offsets: np.ndarray,
                       max_num_loras: int) -> Dict[str, object]:
    slots = np.ascontiguousarray(request_slot, dtype=np.int32)
    offs = np.ascontiguousarray(row_offsets, dtype=np.int64)
    n = slots.size
    if offs.size != n + 1:
        raise ValueError("row_offsets must have num_requests + 1 entries")
    L = int(max_num_loras)
    perm = np.zeros(max(n, 1), np.int32)
    srt = np.zeros(n + 1, np.int64)
    ids = np.zeros(max(L, 1), np.int32)
    goffs = np.zeros(max(L, 1) + 1, np.int32)
    G = np.zeros(1, np.int32)
    end = np.zeros(1, np.int64)
    _check(_load().lora_build_routing(n, _np_ptr(slots), _np_ptr(offs), L, _np_ptr(perm),
                                      _np_ptr(srt), _np_ptr(ids), _np_ptr(goffs), _np_ptr(G),
                                      _np_ptr(end)), "lora_build_routing")
    g = int(G[0])
    return {"perm": perm[:n].copy(), "sorted_offsets": srt, "lora_ids": ids[:g].copy(),
            "grouped_offsets": goffs[:g + 1].copy(), "num_groups": g, "end": int(end[0])}


def lora_build_token_routing(token_slot: np.ndarray, max_num_loras: int) -> Dict[str, object]:
    """Per-token routing: token_slot[t] is token t's slot (-1 = none).
    Returns token_indices_sorted (sorted position -> token), lora_ids,
    grouped_offsets, num_groups and end."""
    slots = np.ascontiguousarray(token_slot, dtype=np.int32).reshape(-1)
    n = slots.size
    L = int(max_num_loras)
    idx = np.zeros(max(n, 1), np.int32)
    ids = np.zeros(max(L, 1), np.int32)
    goffs = np.zeros(max(L, 1) + 1, np.int32)
    G = np.zeros(1, np.int32)
    end = np.zeros(1, np.int64)
    _check(_load().lora_build_token_routing(n, _np_ptr(slots), L, _np_ptr(idx), _np_ptr(ids), _np_ptr(goffs),
                                            _np_ptr(G), _np_ptr(end)), "lora_build_token_routing")
    g = int(G[0])
    return {"token_indices_sorted": idx[:n].copy(), "lora_ids": ids[:g].copy(),
            "grouped_offsets": goffs[:g + 1].copy(), "num_groups": g, "end": int(end[0])}


def lora_sgmv_workspace_bytes(dims: LoraDims, family: int, max_tokens: int) -> int:
    out = ctypes.c_size_t(0)
    dc = dims.c()
    _check(_load().lora_sgmv_workspace_bytes(ctypes.byref(dc), family, int(max_tokens),
                                             ctypes.byref(out)), "lora_sgmv_workspace_bytes")
    return int(out.value)


# ----------------------------------------------------------------------------- device
def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dev_ptr(t, what: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor")
    return t.data_ptr()


def _row_stride(t, what: str) -> int:
    if t.dim() != 2:
        raise ValueError(f"{what} must be a 2-D tensor")
    if t.numel() == 0:
        return int(t.shape[1])
    if t.stride(1) != 1:
        raise ValueError(f"{what} must have unit column stride")
    return int(t.stride(0)) if t.shape[0] > 1 else int(max(t.stride(0), t.shape[1]))


def lora_sgmv_shrink(dims: LoraDims, family: int, x, A_stack, routing: LoraRouting, u,
                     workspace=None, path: int = PATH_AUTO, stream=None) -> None:
    """u[:end] = per-segment A[slot] . x (fp32), asynchronously on the stream."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dc, rc = dims.c(), routing.c()
    _check(_load().lora_sgmv_shrink(ctypes.byref(dc), family, _dev_ptr(x, "x"), _row_stride(x, "x"),
                                     _dev_ptr(A_stack, "A_stack"), ctypes.byref(rc), _dev_ptr(u, "u"),
                                     _dev_ptr(workspace, "workspace"), ws_bytes, int(path),
                                     _stream_handle(stream)),
           "lora_sgmv_shrink")


def lora_sgmv_expand(dims: LoraDims, family: int, u, B_stack, routing: LoraRouting, y,
                     path: int = PATH_AUTO, stream=None, bias=None) -> None:
    """y[:end] += per-segment B[slot] . u (+ bias[slot] when a bias stack
    [L, out] is given), in place, asynchronously on the stream."""
    dc, rc = dims.c(), routing.c()
    _check(_load().lora_sgmv_expand(ctypes.byref(dc), family, _dev_ptr(u, "u"),
                                     _dev_ptr(B_stack, "B_stack"), _dev_ptr(bias, "bias"), ctypes.byref(rc),
                                     _dev_ptr(y, "y"), _row_stride(y, "y"), int(path),
                                     _stream_handle(stream)),
           "lora_sgmv_expand")


def lora_sgmv_delta(dims: LoraDims, family: int, x, A_stack, B_stack, routing: LoraRouting, y,
                    workspace, path: int = PATH_AUTO, stream=None, bias=None,
                    options: Optional[LoraOptions] = None) -> None:
    """y[:end] += per-segment B[slot] . (A[slot] . x) (+ bias[slot] when a
    bias stack [L, out] is given), shrink and expand in one call.  workspace
    may be None where the one-kernel path runs; options: LoraOptions or None
    (the library defaults)."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dc, rc = dims.c(), routing.c()
    oc = None if options is None else ctypes.byref(options.c())
    _check(_load().lora_sgmv_delta(ctypes.byref(dc), family, _dev_ptr(x, "x"), _row_stride(x, "x"),
                                    _dev_ptr(A_stack, "A_stack"), _dev_ptr(B_stack, "B_stack"),
                                    _dev_ptr(bias, "bias"), ctypes.byref(rc), _dev_ptr(y, "y"),
                                    _row_stride(y, "y"),
                                    _dev_ptr(workspace, "workspace"), ws_bytes, int(path), oc,
                                    _stream_handle(stream)),
           "lora_sgmv_delta")


def lora_sgmv_noalloc_scratch_bytes() -> int:
    """Bytes of the device scratch array lora_sgmv_delta_noalloc uses."""
    return int(_load().lora_sgmv_noalloc_scratch_bytes())


def lora_sgmv_delta_noalloc(dims: LoraDims, family: int, x, A_stack, B_stack, routing: LoraRouting, y,
                            path: int = PATH_AUTO, stream=None, bias=None,
                            options: Optional[LoraOptions] = None) -> None:
    """lora_sgmv_delta without a workspace argument: the partial sums go to
    the library's own device scratch array; nothing is allocated."""
    dc, rc = dims.c(), routing.c()
    oc = None if options is None else ctypes.byref(options.c())
    _check(_load().lora_sgmv_delta_noalloc(ctypes.byref(dc), family, _dev_ptr(x, "x"), _row_stride(x, "x"),
                                            _dev_ptr(A_stack, "A_stack"), _dev_ptr(B_stack, "B_stack"),
                                            _dev_ptr(bias, "bias"), ctypes.byref(rc), _dev_ptr(y, "y"),
                                            _row_stride(y, "y"), int(path), oc, _stream_handle(stream)),
           "lora_sgmv_delta_noalloc")


def packed_to_torch(a: np.ndarray):
    """Host packed array (uint16 bf16 patterns or float32) -> CPU torch tensor of
    the matching dtype, sharing no memory with `a`."""
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).copy())


# ----------------------------------------------------------------------------- slot cache
CACHE_LRU, CACHE_NO_EVICT = 0, 1


class LoraSlotCache:
    """Host slot cache (lora_cache_*): which adapter id holds which slot."""

    def __init__(self, num_slots: int, policy: int = CACHE_LRU):
        self._h = ctypes.c_void_p()
        _check(_load().lora_cache_create(int(num_slots), int(policy), ctypes.byref(self._h)), "lora_cache_create")
        self.num_slots = int(num_slots)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.lora_cache_destroy(h)
            self._h = None

    def activate(self, adapter_id: int) -> Tuple[int, bool, int]:
        """(slot, needs_load, evicted adapter id or -1)."""
        s, l, e = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
        _check(_load().lora_cache_activate(self._h, int(adapter_id), ctypes.byref(s), ctypes.byref(l),
                                           ctypes.byref(e)), "lora_cache_activate")
        return s.value, bool(l.value), e.value

    def activate_batch(self, adapter_ids) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """(request_slot int32[n], load_slots int32[k], load_ids int64[k])."""
        ids = np.ascontiguousarray(adapter_ids, np.int64)
        n = len(ids)
        rs = np.zeros(max(n, 1), np.int32)
        ls = np.zeros(max(n, 1), np.int32)
        li = np.zeros(max(n, 1), np.int64)
        k = ctypes.c_int32()
        _check(_load().lora_cache_activate_batch(self._h, n, _np_ptr(ids) if n else None, _np_ptr(rs),
                                                 _np_ptr(ls), _np_ptr(li), ctypes.byref(k)),
               "lora_cache_activate_batch")
        return rs[:n].copy(), ls[:k.value].copy(), li[:k.value].copy()

    def unload(self, adapter_id: int) -> int:
        s = ctypes.c_int32()
        _check(_load().lora_cache_unload(self._h, int(adapter_id), ctypes.byref(s)), "lora_cache_unload")
        return s.value

    def pin(self, adapter_id: int, pinned: bool = True) -> Tuple[int, bool, int]:
        s, l, e = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
        _check(_load().lora_cache_pin(self._h, int(adapter_id), 1 if pinned else 0, ctypes.byref(s),
                                      ctypes.byref(l), ctypes.byref(e)), "lora_cache_pin")
        return s.value, bool(l.value), e.value

    def lookup(self, adapter_id: int) -> int:
        s = ctypes.c_int32()
        _check(_load().lora_cache_lookup(self._h, int(adapter_id), ctypes.byref(s)), "lora_cache_lookup")
        return s.value

    def slot_table(self) -> Tuple[np.ndarray, np.ndarray]:
        ids = np.zeros(self.num_slots, np.int64)
        pinned = np.zeros(self.num_slots, np.uint8)
        _check(_load().lora_cache_slot_table(self._h, self.num_slots, _np_ptr(ids), _np_ptr(pinned)),
               "lora_cache_slot_table")
        return ids, pinned


def lora_write_slot(dims: LoraDims, slot: int, packed, stacks, stream=None) -> None:
    """Copy one adapter's packed host tensors (lora_pack_adapter's dict, or
    host torch tensors with the same keys) into slot `slot` of the four
    device stacks {"A_qkv", "B_qkv", "A_o", "B_o"}, asynchronously."""
    keys = ("A_qkv", "B_qkv", "A_o", "B_o")
    src = []
    for k in keys:
        a = packed[k]
        if isinstance(a, np.ndarray):
            if not a.flags["C_CONTIGUOUS"]:
                raise ValueError(f"{k} must be contiguous")
            src.append(_np_ptr(a))
        else:
            if a.is_cuda or not a.is_contiguous():
                raise ValueError(f"{k} must be a contiguous host tensor")
            src.append(a.data_ptr())
    dc = dims.c()
    _check(_load().lora_write_slot(ctypes.byref(dc), int(slot), *src,
                                   *[_dev_ptr(stacks[k], k) for k in keys], _stream_handle(stream)),
           "lora_write_slot")


def lora_reset_slot(dims: LoraDims, slot: int, stacks, stream=None) -> None:
    """Zero slot `slot` of the four device stacks, asynchronously."""
    keys = ("A_qkv", "B_qkv", "A_o", "B_o")
    dc = dims.c()
    _check(_load().lora_reset_slot(ctypes.byref(dc), int(slot), *[_dev_ptr(stacks[k], k) for k in keys],
                                   _stream_handle(stream)), "lora_reset_slot")
