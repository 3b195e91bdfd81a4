"""Oracle side of the every-row check of the 32-layer stack workload, run in
worker processes on the CPU.

A worker regenerates one layer's inputs from the workload's seeds (synth),
packs that layer's adapters with the oracle's own pack, evaluates the oracle
for every request of both families, and compares with the GPU result the
test process wrote to a file (bf16 bit patterns of y in arrival order, and
optionally fp32 u).  It imports neither torch nor the GPU library, so the
workers start as fresh interpreters that never touch the GPU.
"""

from __future__ import annotations

import os
from typing import Dict

import numpy as np

import oracle
import synth

TOL_BF16 = 1e-2   # max relative error of y (bf16 in, fp32 accumulate)
U_TOL_BF16 = 1e-4


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max_i |g_i - r_i| / max(|r_i|, rho), rho = RMS of the reference."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rho = float(np.sqrt(np.mean(ref * ref)))
    den = np.maximum(np.abs(ref), rho if rho > 0 else 1.0)
    return float(np.max(np.abs(got - ref) / den))


def oracle_stacks(w: synth.Workload, layer: int, ranks) -> Dict[str, np.ndarray]:
    st = {k: [] for k in ("A_qkv", "B_qkv", "A_o", "B_o")}
    for s in range(w.max_num_loras):
        pk = oracle.pack_adapter(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank, w.dtype,
                                 int(ranks[s]), w.lora_alpha, w.use_rslora, True, "qkvo",
                                 synth.draw_adapter(w, layer, s, int(ranks[s])))
        for k in st:
            st[k].append(pk[k])
    return {k: np.stack(v) for k, v in st.items()}


def check_layer(job) -> dict:
    """job: (workload name, layer, path of the GPU result .npz).  The file
    holds y_qkv / y_o as uint16 bf16 patterns [T, out] in arrival order and,
    when present, u_qkv / u_o fp32 [T, C] (rows of base requests unused).
    Returns the worst errors of the layer and whether every base row is
    bit-identical to its input; deletes the file."""
    name, layer, path = job
    w = synth.get_workload(name)
    lengths, slots = synth.draw_requests(w)
    ranks = synth.draw_ranks(w)
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(offs[-1])
    st = oracle_stacks(w, layer, ranks)
    acts = synth.draw_activations(w, layer, T)
    with np.load(path) as f:
        gpu = {k: f[k] for k in f.files}
    os.remove(path)
    out = {"layer": layer, "base_rows_identical": True}
    R = w.max_lora_rank
    for fam, xk, yk, ak, bk, uk, widths in (
            ("qkv", "x_qkv", "y_qkv", "A_qkv", "B_qkv", "u_qkv", [w.nq, w.nkv, w.nkv]),
            ("o", "x_o", "y_o", "A_o", "B_o", "u_o", [w.hidden])):
        ref = oracle.reference_family(acts[xk], acts[yk], offs, slots, st[ak], st[bk], widths, R, w.dtype)
        y = oracle.bf16_to_f64(gpu[yk])
        got, want, ug, ur = [], [], [], []
        for i, (rows, yref, uref) in ref.items():
            a = int(offs[i])
            g = y[a + rows]
            if uref is None:
                if not np.array_equal(g, yref):
                    out["base_rows_identical"] = False
                continue
            got.append(g)
            want.append(yref)
            if uk in gpu:
                ug.append(gpu[uk][a + rows])
                ur.append(uref)
        out["rows_" + fam] = int(sum(len(g) for g in got))
        out["y_rel_" + fam] = rel_err(np.concatenate(got), np.concatenate(want))
        out["u_rel_" + fam] = rel_err(np.concatenate(ug), np.concatenate(ur)) if ug else None
    return out
