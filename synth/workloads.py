"""Workload definitions and seeded draws (see the package docstring for scope).

Value distributions are written N(mean, variance):
A ~ N(0, 1/in_features), B ~ N(0, 0.02), x ~ N(0, 1), y ~ N(0, 1).

Every draw comes from its own counter-addressed numpy stream
``default_rng([seed, stream, layer, slot])`` so that any layer or slot can be
regenerated alone, in any order, with identical results.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Tuple

import numpy as np

PROJECTIONS = ("q", "k", "v", "o")
MLP_PROJECTIONS = ("gate", "up", "down")

# stream ids of the counter-addressed generators
_S_REQ, _S_RANK, _S_ADAPTER, _S_ACT, _S_MLP_ADAPTER, _S_MLP_ACT, _S_BIAS = 1, 2, 3, 4, 5, 6, 7

B_VARIANCE = 0.02


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    max_lora_rank: int
    max_num_loras: int
    dtype: str            # "f32" or "bf16"
    n_layers: int
    lora_alpha: float
    use_rslora: bool
    seed: int
    intermediate: int = 0  # MLP width (gate/up output, down input); 0 = attention only

    @property
    def nq(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def nkv(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def n_qkv(self) -> int:
        return self.nq + 2 * self.nkv

    def proj_shape(self, p: str) -> Tuple[int, int]:
        """(in_features, out_features) of projection p."""
        if p == "q":
            return self.hidden, self.nq
        if p in ("k", "v"):
            return self.hidden, self.nkv
        if p in ("gate", "up"):
            return self.hidden, self.intermediate
        if p == "down":
            return self.intermediate, self.hidden
        if p == "o":
            return self.nq, self.hidden
        raise KeyError(p)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in (
        Workload("tiny", "fp32 toy attention block, 3 requests 5/3/4 tokens on slots 0/1/base",
                 hidden=128, n_heads=8, n_kv_heads=8, head_dim=16, max_lora_rank=16,
                 max_num_loras=2, dtype="f32", n_layers=1, lora_alpha=8.0, use_rslora=False,
                 seed=1001),
        Workload("decode", "Llama-3-8B attention, 256 one-token requests, 8 slots, ranks 8/16, 25% base",
                 hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128, max_lora_rank=16,
                 max_num_loras=8, dtype="bf16", n_layers=1, lora_alpha=16.0, use_rslora=False,
                 seed=1002),
        Workload("prefill", "Llama-3-8B attention, 16 requests of 128..2048 tokens, 4 slots round-robin, 2 base",
                 hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128, max_lora_rank=16,
                 max_num_loras=4, dtype="bf16", n_layers=1, lora_alpha=32.0, use_rslora=False,
                 seed=1003),
        Workload("mixed", "hidden 5120 attention, 192 decode + 8 prefill requests, 32 Zipf slots, ranks 8..64",
                 hidden=5120, n_heads=40, n_kv_heads=8, head_dim=128, max_lora_rank=64,
                 max_num_loras=32, dtype="bf16", n_layers=1, lora_alpha=16.0, use_rslora=False,
                 seed=1004),
        Workload("mlp", "Llama-3-8B MLP (4096 -> 2 x 14336 -> 4096), 256 one-token requests, 8 slots, ranks 8/16, 25% base",
                 hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128, max_lora_rank=16,
                 max_num_loras=8, dtype="bf16", n_layers=1, lora_alpha=16.0, use_rslora=False,
                 seed=1006, intermediate=14336),
        Workload("stack", "32-layer Llama-3-8B attention, 4096 tokens in 32 requests, 16 slots, rsLoRA r=32",
                 hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128, max_lora_rank=32,
                 max_num_loras=16, dtype="bf16", n_layers=32, lora_alpha=16.0, use_rslora=True,
                 seed=1005),
    )
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def _rng(w: Workload, stream: int, layer: int = 0, slot: int = 0) -> np.random.Generator:
    return np.random.default_rng([w.seed, stream, layer, slot])


def _rescale_lengths(raw: np.ndarray, total: int) -> np.ndarray:
    """Scale positive integers to sum exactly `total`: floor, then hand the
    remainder out by largest fractional part (ties to the lower index)."""
    exact = raw.astype(np.float64) * total / raw.sum()
    base = np.floor(exact).astype(np.int64)
    rem = total - int(base.sum())
    frac = exact - base
    order = sorted(range(len(raw)), key=lambda i: (-frac[i], i))
    for i in order[:rem]:
        base[i] += 1
    return base


def draw_requests(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Request lengths (int64) and slot ids (int32, -1 = base) in arrival order."""
    rng = _rng(w, _S_REQ)
    L = w.max_num_loras
    if w.name == "tiny":
        lengths = np.array([5, 3, 4], dtype=np.int64)
        slots = np.array([0, 1, -1], dtype=np.int32)
    elif w.name in ("decode", "mlp"):
        n = 256
        lengths = np.ones(n, dtype=np.int64)
        slots = rng.integers(0, L, size=n).astype(np.int32)
        base = rng.permutation(n)[:64]
        slots[base] = -1
    elif w.name == "prefill":
        n = 16
        lengths = rng.integers(128, 2049, size=n).astype(np.int64)
        slots = np.array([i % L for i in range(14)] + [-1, -1], dtype=np.int32)
    elif w.name == "mixed":
        lengths = np.array([1] * 192 + [104] * 8, dtype=np.int64)
        p = (np.arange(L) + 1.0) ** -1.1
        p /= p.sum()
        slots = rng.choice(L, size=200, p=p).astype(np.int32)
        base = rng.choice(200, size=20, replace=False)
        slots[base] = -1
        order = rng.permutation(200)
        lengths, slots = lengths[order], slots[order]
    elif w.name == "stack":
        raw = rng.integers(32, 225, size=32)
        lengths = _rescale_lengths(raw, 4096)
        slots = np.array([i % L for i in range(28)] + [-1] * 4, dtype=np.int32)
    else:
        raise KeyError(w.name)
    return lengths, slots


def draw_ranks(w: Workload) -> np.ndarray:
    """Adapter rank of each slot (int32[max_num_loras])."""
    rng = _rng(w, _S_RANK)
    L = w.max_num_loras
    if w.name in ("decode", "mlp"):
        return rng.choice(np.array([8, 16]), size=L).astype(np.int32)
    if w.name == "mixed":
        return rng.choice(np.array([8, 16, 32, 64]), size=L).astype(np.int32)
    fixed = {"tiny": 4, "prefill": 16, "stack": 32}[w.name]
    return np.full(L, fixed, dtype=np.int32)


def draw_adapter(w: Workload, layer: int, slot: int, rank: int) -> Dict[str, Tuple[np.ndarray, np.ndarray]]:
    """Unscaled fp32 PEFT matrices of one adapter in one layer:
    {p: (lora_A [rank, in_p], lora_B [out_p, rank])} for p in q, k, v, o."""
    rng = _rng(w, _S_ADAPTER, layer, slot)
    out = {}
    for p in PROJECTIONS:
        fin, fout = w.proj_shape(p)
        a = rng.standard_normal((rank, fin), dtype=np.float32) * np.float32(1.0 / np.sqrt(fin))
        b = rng.standard_normal((fout, rank), dtype=np.float32) * np.float32(np.sqrt(B_VARIANCE))
        out[p] = (a.astype(np.float32), b.astype(np.float32))
    return out


def draw_bias(w: Workload, layer: int, slot: int, projections=PROJECTIONS) -> Dict[str, np.ndarray]:
    """Unscaled fp32 LoRA biases of one adapter in one layer: {p: bias [out_p]}.
    Their spread (4 sqrt(B_VARIANCE)) is of the order of a rank-16 delta."""
    rng = _rng(w, _S_BIAS, layer, slot)
    out = {}
    for p in projections:
        _, fout = w.proj_shape(p)
        out[p] = (rng.standard_normal(fout, dtype=np.float32) * np.float32(4.0 * np.sqrt(B_VARIANCE))
                  ).astype(np.float32)
    return out


def _to_dtype_values(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 draws rounded to the nearest bf16 number (ties to even) when the
    workload is bf16; the draws are finite, so no NaN or overflow case."""
    if dtype == "f32":
        return a
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    keep_odd = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + keep_odd) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def draw_activations(w: Workload, layer: int, n_tokens: int) -> Dict[str, np.ndarray]:
    """x and base y of both projection families for one layer, tokens in arrival order.

    Returns float32 arrays whose values are exactly representable in the
    workload dtype: x_qkv [T, hidden], y_qkv [T, nq + 2 nkv], x_o [T, nq], y_o [T, hidden].
    """
    rng = _rng(w, _S_ACT, layer)
    shapes = {
        "x_qkv": (n_tokens, w.hidden),
        "y_qkv": (n_tokens, w.n_qkv),
        "x_o": (n_tokens, w.nq),
        "y_o": (n_tokens, w.hidden),
    }
    return {k: _to_dtype_values(rng.standard_normal(s, dtype=np.float32), w.dtype)
            for k, s in shapes.items()}


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16 numbers
    (low 16 bits zero).  Raises if any value would need rounding."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not exactly representable in bf16")
    return (u >> np.uint32(16)).astype(np.uint16)


def draw_mlp_adapter(w: Workload, layer: int, slot: int, rank: int) -> Dict[str, Tuple[np.ndarray, np.ndarray]]:
    """Unscaled fp32 PEFT matrices of one adapter's MLP projections in one
    layer: {p: (lora_A [rank, in_p], lora_B [out_p, rank])} for p in gate, up, down."""
    if w.intermediate <= 0:
        raise ValueError("workload has no MLP")
    rng = _rng(w, _S_MLP_ADAPTER, layer, slot)
    out = {}
    for p in MLP_PROJECTIONS:
        fin, fout = w.proj_shape(p)
        a = rng.standard_normal((rank, fin), dtype=np.float32) * np.float32(1.0 / np.sqrt(fin))
        b = rng.standard_normal((fout, rank), dtype=np.float32) * np.float32(np.sqrt(B_VARIANCE))
        out[p] = (a.astype(np.float32), b.astype(np.float32))
    return out


def draw_mlp_activations(w: Workload, layer: int, n_tokens: int) -> Dict[str, np.ndarray]:
    """x and base y of the two MLP families, tokens in arrival order:
    x_gu [T, hidden], y_gu [T, 2 intermediate], x_down [T, intermediate], y_down [T, hidden]."""
    rng = _rng(w, _S_MLP_ACT, layer)
    shapes = {
        "x_gu": (n_tokens, w.hidden),
        "y_gu": (n_tokens, 2 * w.intermediate),
        "x_down": (n_tokens, w.intermediate),
        "y_down": (n_tokens, w.hidden),
    }
    return {k: _to_dtype_values(rng.standard_normal(s, dtype=np.float32), w.dtype)
            for k, s in shapes.items()}
