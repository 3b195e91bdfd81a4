"""ctypes binding of the C oracle (lora_oracle.c) plus the per-request driver.

TEST INFRASTRUCTURE (see the package docstring).  The driver evaluates the
delta request by request, in arrival order, from the packed slot tensors; it
never uses the routing it can also compute, so the routing is checked on its
own and the forward only depends on each request's slot.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lora_oracle.c")
_LIB = os.path.join(_HERE, "liblora_oracle.so")

DTYPE_CODE = {"f32": 0, "bf16": 1}
TARGET_BITS = {"q": 1, "k": 2, "v": 4, "o": 8}


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what} failed with code {code}")
        self.code = code


def library_path() -> str:
    return _LIB


def build() -> str:
    """Compile the oracle with gcc (plain C, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", _SRC, "-o", _LIB, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("ORACLE_LIB")  # lets the mutation test load a planted-mistake build
    if not path:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, u32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_double
    lib.oracle_scaling.restype = f64
    lib.oracle_scaling.argtypes = [f64, i32, i32]
    lib.oracle_bf16_round.restype = ctypes.c_uint16
    lib.oracle_bf16_round.argtypes = [ctypes.c_float]
    lib.oracle_bf16_round_array.restype = None
    lib.oracle_bf16_round_array.argtypes = [P, P, i64]
    lib.oracle_pack_adapter.restype = i32
    lib.oracle_pack_adapter.argtypes = [i32, i32, i32, i32, i32, i32, i32, f64, i32, i32, u32,
                                        P, P, P, P, P, P]
    lib.oracle_pack_family.restype = i32
    lib.oracle_pack_family.argtypes = [i32, i32, P, i32, i32, i32, f64, i32, i32, u32, P, P, P, P]
    lib.oracle_route.restype = i32
    lib.oracle_route.argtypes = [i32, P, P, i32, P, P, P, P, P, P]
    lib.oracle_delta.restype = i32
    lib.oracle_delta.argtypes = [i32, i32, i32, P, i32, P, P, P, P, P, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ---------------------------------------------------------------------------
def scaling(alpha: float, r: int, use_rslora: bool) -> float:
    return float(_load().oracle_scaling(float(alpha), int(r), int(bool(use_rslora))))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns (round to nearest, ties to even)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().oracle_bf16_round_array(_ptr(a), _ptr(out), a.size)
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def stack_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_to_f64(a) if dtype == "bf16" else np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
def pack_adapter(hidden: int, n_heads: int, n_kv_heads: int, head_dim: int, max_rank: int,
                 dtype: str, rank: int, alpha: float, use_rslora: bool, bias_none: bool,
                 targets: Sequence[str],
                 weights: Dict[str, Tuple[np.ndarray, np.ndarray]],
                 target_mask: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Pack one adapter; returns {"A_qkv", "B_qkv", "A_o", "B_o"} in the stack
    dtype (uint16 bit patterns for bf16, float32 for f32)."""
    lib = _load()
    nq, nkv = n_heads * head_dim, n_kv_heads * head_dim
    R = max_rank
    st = np.uint16 if dtype == "bf16" else np.float32
    out = {
        "A_qkv": np.zeros((3 * R, hidden), dtype=st),
        "B_qkv": np.zeros((nq + 2 * nkv, R), dtype=st),
        "A_o": np.zeros((R, nq), dtype=st),
        "B_o": np.zeros((hidden, R), dtype=st),
    }
    if target_mask is None:
        target_mask = 0
        for t in targets:
            target_mask |= TARGET_BITS[t]
    keep = []
    a_ptrs = (ctypes.c_void_p * 4)()
    b_ptrs = (ctypes.c_void_p * 4)()
    for i, p in enumerate("qkvo"):
        if p in weights and (target_mask >> i) & 1:
            a = np.ascontiguousarray(weights[p][0], dtype=np.float32)
            b = np.ascontiguousarray(weights[p][1], dtype=np.float32)
            keep += [a, b]
            a_ptrs[i] = _ptr(a)
            b_ptrs[i] = _ptr(b)
    code = lib.oracle_pack_adapter(hidden, n_heads, n_kv_heads, head_dim, R, DTYPE_CODE[dtype],
                                   int(rank), float(alpha), int(bool(use_rslora)),
                                   int(bool(bias_none)), int(target_mask),
                                   ctypes.cast(a_ptrs, ctypes.c_void_p),
                                   ctypes.cast(b_ptrs, ctypes.c_void_p),
                                   _ptr(out["A_qkv"]), _ptr(out["B_qkv"]), _ptr(out["A_o"]),
                                   _ptr(out["B_o"]))
    if code != 0:
        raise OracleError(code, "pack")
    return out


def pack_family(in_f: int, widths: Sequence[int], max_rank: int, dtype: str, rank: int, alpha: float,
                use_rslora: bool, bias_none: bool,
                slices: Sequence[Optional[Tuple[np.ndarray, np.ndarray]]]) -> Dict[str, np.ndarray]:
    """Pack one adapter's slices of one family: {"A" [n_s R, in_f], "B" [sum widths, R]}
    in the stack dtype (logical layout)."""
    lib = _load()
    n_s = len(widths)
    R = max_rank
    st = np.uint16 if dtype == "bf16" else np.float32
    out = {"A": np.zeros((n_s * R, in_f), dtype=st), "B": np.zeros((int(sum(widths)), R), dtype=st)}
    keep, mask = [], 0
    a_ptrs = (ctypes.c_void_p * n_s)()
    b_ptrs = (ctypes.c_void_p * n_s)()
    for i, sl in enumerate(slices):
        if sl is None:
            continue
        a = np.ascontiguousarray(sl[0], dtype=np.float32)
        b = np.ascontiguousarray(sl[1], dtype=np.float32)
        keep += [a, b]
        a_ptrs[i], b_ptrs[i] = _ptr(a), _ptr(b)
        mask |= 1 << i
    w = np.ascontiguousarray(widths, dtype=np.int32)
    code = lib.oracle_pack_family(int(in_f), n_s, _ptr(w), R, DTYPE_CODE[dtype], int(rank), float(alpha),
                                  int(bool(use_rslora)), int(bool(bias_none)), mask,
                                  ctypes.cast(a_ptrs, ctypes.c_void_p), ctypes.cast(b_ptrs, ctypes.c_void_p),
                                  _ptr(out["A"]), _ptr(out["B"]))
    if code != 0:
        raise OracleError(code, "pack_family")
    return out


def pack_bias(widths: Sequence[int], dtype: str, slices: Sequence[Optional[np.ndarray]]) -> np.ndarray:
    """One adapter's LoRA bias of one family, [sum widths] in the stack dtype.

    [vLLM] "vLLM LoRA 实现深度解析" §5.3 activate_adapter: set_lora receives
    the bias beside A and B, and the scaling is folded into B alone
    (optimize); [MAX-lora] LoRAType BIAS: a bias attached to B.  So the bias
    is the slices' biases concatenated in slice order (the same order as B's
    rows, [MAX-lora] QKV fusion), zero for a slice the adapter has none for,
    cast to the stack dtype.
    """
    if len(slices) != len(widths):
        raise OracleError(1, "pack_bias")
    parts = []
    for w, b in zip(widths, slices):
        parts.append(np.zeros(int(w)) if b is None else np.asarray(b, dtype=np.float32).reshape(int(w)))
    cat = np.concatenate(parts).astype(np.float32) if parts else np.zeros(0, np.float32)
    return bf16_round(cat) if dtype == "bf16" else cat


def route(slots: np.ndarray, row_offsets: np.ndarray, max_num_loras: int) -> Dict[str, object]:
    lib = _load()
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    offs = np.ascontiguousarray(row_offsets, dtype=np.int64)
    n = slots.size
    if offs.size != n + 1:
        raise OracleError(1, "route")
    L = int(max_num_loras)
    perm = np.zeros(max(n, 1), dtype=np.int32)
    sorted_offsets = np.zeros(n + 1, dtype=np.int64)
    ids = np.zeros(max(L, 1), dtype=np.int32)
    goffs = np.zeros(max(L, 1) + 1, dtype=np.int32)
    G = np.zeros(1, dtype=np.int32)
    end = np.zeros(1, dtype=np.int64)
    code = lib.oracle_route(n, _ptr(slots), _ptr(offs), L, _ptr(perm), _ptr(sorted_offsets),
                            _ptr(ids), _ptr(goffs), _ptr(G), _ptr(end))
    if code != 0:
        raise OracleError(code, "route")
    g = int(G[0])
    return {"perm": perm[:n].copy(), "sorted_offsets": sorted_offsets, "lora_ids": ids[:g].copy(),
            "grouped_offsets": goffs[:g + 1].copy(), "num_groups": g, "end": int(end[0])}


def delta(x: np.ndarray, A: np.ndarray, B: np.ndarray, y_in: np.ndarray,
          widths: Sequence[int], R: int) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 (u, y_out) for tokens x [n, in] of one adapter (A [n_s R, in], B [sum w, R])."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    A = np.ascontiguousarray(A, dtype=np.float64)
    B = np.ascontiguousarray(B, dtype=np.float64)
    y_in = np.ascontiguousarray(y_in, dtype=np.float64)
    w = np.ascontiguousarray(widths, dtype=np.int32)
    n, fin = x.shape
    n_s = w.size
    u = np.zeros((n, n_s * R), dtype=np.float64)
    y = np.zeros((n, int(w.sum())), dtype=np.float64)
    if n == 0:
        return u, y
    code = lib.oracle_delta(n, fin, n_s, _ptr(w), int(R), _ptr(x), _ptr(A), _ptr(B), _ptr(y_in),
                            _ptr(u), _ptr(y))
    if code != 0:
        raise OracleError(code, "delta")
    return u, y


def reference_family(x: np.ndarray, y_in: np.ndarray, row_offsets: np.ndarray, slots: np.ndarray,
                     A_stack: np.ndarray, B_stack: np.ndarray, widths: Sequence[int], R: int,
                     dtype: str, requests: Optional[Sequence[int]] = None,
                     token_rows: Optional[Dict[int, np.ndarray]] = None,
                     bias_stack: Optional[np.ndarray] = None):
    """Reference (y_ref fp64, u fp64) for one projection family of a batch.

    x, y_in are float arrays in arrival order ([T, in], [T, out]); A_stack,
    B_stack are the packed stacks [L, ...] in the stack dtype.  Each LoRA
    request gets y_in + B[slot] (A[slot] x) token by token, plus
    bias_stack[slot] when a bias stack [L, out] is given (the LoRA layer's
    bias, [vLLM] §5.3 set_lora); base requests get y_in unchanged.
    `requests` restricts the work to some requests and `token_rows` to some
    rows of each (rows relative to the request).
    Returns dicts keyed by request index: {i: (rows, y_ref, u or None)}.
    """
    out = {}
    n_req = len(slots)
    todo = range(n_req) if requests is None else requests
    cache = {}
    for i in todo:
        a, b = int(row_offsets[i]), int(row_offsets[i + 1])
        rows = np.arange(b - a) if token_rows is None or i not in token_rows else np.asarray(token_rows[i])
        yi = np.asarray(y_in[a + rows], dtype=np.float64)
        s = int(slots[i])
        if s < 0:
            out[i] = (rows, yi.copy(), None)
            continue
        if s not in cache:
            cache[s] = (stack_to_f64(A_stack[s], dtype), stack_to_f64(B_stack[s], dtype))
        Af, Bf = cache[s]
        u, y = delta(np.asarray(x[a + rows], dtype=np.float64), Af, Bf, yi, widths, R)
        if bias_stack is not None:
            y = y + stack_to_f64(bias_stack[s], dtype)[None, :]
        out[i] = (rows, y, u)
    return out
