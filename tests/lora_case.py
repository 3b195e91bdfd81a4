"""Helpers shared by the GPU tests: run one layer of a workload through the
C-ABI library and compare it with the oracle.

The GPU side packs with lora_pack_adapter, routes with lora_build_routing,
lays x/y out in its own sorted order and runs lora_sgmv_shrink /
lora_sgmv_expand.  The oracle side evaluates each request in arrival order.
Results are compared request by request.
"""

from __future__ import annotations

import sys
from typing import Dict, Optional, Sequence

import numpy as np

import oracle
import synth
import segmented_rank_gemv_amd as srg

TOL = {"f32": 1e-5, "bf16": 1e-2}   # max relative error of y (see rel_err)
U_TOL = {"f32": 1e-5, "bf16": 1e-4}  # diagnostic bound on the rank-space intermediate


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def dims_of(w: synth.Workload) -> srg.LoraDims:
    return srg.LoraDims(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank,
                        w.max_num_loras, w.dtype)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max_i |g_i - r_i| / max(|r_i|, rho), rho = RMS of the reference."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rho = float(np.sqrt(np.mean(ref * ref)))
    den = np.maximum(np.abs(ref), rho if rho > 0 else 1.0)
    return float(np.max(np.abs(got - ref) / den))


def pack_stacks(w: synth.Workload, layer: int, ranks: np.ndarray, targets="qkvo",
                zero_B: bool = False, with_ref: bool = True) -> Dict[str, np.ndarray]:
    """Stacks [L, ...] of one layer: A_qkv / B_qkv / A_o / B_o packed by the
    product library (device layout, for the GPU) and, under "ref" (unless
    with_ref is false), the same adapters packed by the oracle (logical
    layout, for the reference)."""
    d = dims_of(w)
    out = {k: [] for k in ("A_qkv", "B_qkv", "A_o", "B_o")}
    ref = {k: [] for k in out}
    for s in range(w.max_num_loras):
        weights = synth.draw_adapter(w, layer, s, int(ranks[s]))
        if zero_B:
            weights = {p: (a, np.zeros_like(b)) for p, (a, b) in weights.items()}
        pk = srg.lora_pack_adapter(d, int(ranks[s]), w.lora_alpha, w.use_rslora, True, targets, weights)
        for k in out:
            out[k].append(pk[k])
        if with_ref:
            po = oracle.pack_adapter(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank, w.dtype,
                                     int(ranks[s]), w.lora_alpha, w.use_rslora, True, targets, weights)
            for k in ref:
                ref[k].append(po[k])
    stacks = {k: np.stack(v) for k, v in out.items()}
    if with_ref:
        stacks["ref"] = {k: np.stack(v) for k, v in ref.items()}
    return stacks


def pack_bias_stacks(w: synth.Workload, layer: int, targets="qkvo") -> Dict[str, np.ndarray]:
    """Bias stacks [L, out] of one layer: bias_qkv / bias_o packed by the
    product library and, under "ref", by the oracle."""
    d = dims_of(w)
    fams = (("bias_qkv", srg.FAMILY_QKV, "qkv"), ("bias_o", srg.FAMILY_O, "o"))
    out = {k: [] for k, _, _ in fams}
    ref = {k: [] for k, _, _ in fams}
    for s in range(w.max_num_loras):
        b = synth.draw_bias(w, layer, s)
        for key, fam, projs in fams:
            sl = [b[p] if p in targets else None for p in projs]
            out[key].append(srg.lora_pack_bias(d, fam, sl))
            widths = srg.lora_family_shape(d, fam)[2]
            ref[key].append(oracle.pack_bias(widths, w.dtype, sl))
    stacks = {k: np.stack(v) for k, v in out.items()}
    stacks["ref"] = {k: np.stack(v) for k, v in ref.items()}
    return stacks


def to_dev(a: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        if a.dtype == np.uint16:
            bits = a
        else:
            bits = synth.bf16_bits(a)
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def from_dev(t) -> np.ndarray:
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).numpy().view(np.uint16)
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return t.numpy().astype(np.float32)


class GpuLayer:
    """One layer (both families) of one batch on the GPU."""

    def __init__(self, w: synth.Workload, stacks: Dict[str, np.ndarray], lengths: np.ndarray,
                 slots: np.ndarray, acts: Dict[str, np.ndarray], pad_rows: int = 0,
                 pad_cols: int = 0, bias: Optional[Dict[str, np.ndarray]] = None):
        import torch
        self.w = w
        self.dims = dims_of(w)
        self.lengths = np.asarray(lengths, np.int64)
        self.slots = np.asarray(slots, np.int32)
        self.offs = np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int64)
        self.rt = srg.lora_build_routing(self.slots, self.offs, w.max_num_loras)
        perm = self.rt["perm"]
        self.tok_order = (np.concatenate([np.arange(self.offs[p], self.offs[p + 1]) for p in perm])
                          if len(perm) else np.zeros(0, np.int64)).astype(np.int64)
        self.T = int(self.offs[-1])
        self.end = self.rt["end"]
        self.G = self.rt["num_groups"]
        self.st = {k: to_dev(v, w.dtype) for k, v in stacks.items() if k != "ref"}
        self.bias = None if bias is None else {k: to_dev(v, w.dtype) for k, v in bias.items() if k != "ref"}
        # routing with host copies (kernel-argument routing) and device-only
        self.routing = {"host": srg.LoraRouting.from_host(self.rt, host_copy=True),
                        "device": srg.LoraRouting.from_host(self.rt, host_copy=False)}
        self.dev = {}
        self.shape = {}
        for fam, xk, yk in ((srg.FAMILY_QKV, "x_qkv", "y_qkv"), (srg.FAMILY_O, "x_o", "y_o")):
            fin, n_s, widths, fout = srg.lora_family_shape(self.dims, fam)
            self.shape[fam] = (fin, n_s, widths, fout)
            for key, width in ((xk, fin), (yk, fout)):
                host = acts[key][self.tok_order]
                # optional padding: wider rows (stride tests) and extra rows past T
                buf = np.zeros((self.T + pad_rows, width + pad_cols), np.float32)
                buf[:self.T, :width] = host
                if pad_rows:
                    buf[self.T:, :width] = 7.0
                full = to_dev(buf, w.dtype)
                self.dev[key] = full[:, :width] if pad_cols else full
                self.dev[key + "_full"] = full
        self.u = {}
        self.ws = {}
        for fam in (srg.FAMILY_QKV, srg.FAMILY_O):
            C = self.shape[fam][1] * w.max_lora_rank
            self.u[fam] = torch.full((max(self.end, 1), C), float("nan"), dtype=torch.float32, device="cuda")
            nb = srg.lora_sgmv_workspace_bytes(self.dims, fam, max(self.end, 1))
            self.ws[fam] = torch.full((max(nb, 16) // 4 + 4,), -1, dtype=torch.int32, device="cuda")

    def run(self, path: int = srg.PATH_AUTO, families=(srg.FAMILY_QKV, srg.FAMILY_O),
            fused: bool = False, routing: str = "host", options=None, noalloc: bool = False):
        """fused=False: lora_sgmv_shrink then lora_sgmv_expand (u checked);
        fused=True: lora_sgmv_delta (u stays internal), with `options`
        (srg.LoraOptions or None), or with noalloc lora_sgmv_delta_noalloc.
        routing: "host" (host copies passed, kernel-argument routing) or
        "device"."""
        rt = self.routing[routing]
        for fam in families:
            xk, yk = ("x_qkv", "y_qkv") if fam == srg.FAMILY_QKV else ("x_o", "y_o")
            A = self.st["A_qkv" if fam == srg.FAMILY_QKV else "A_o"]
            B = self.st["B_qkv" if fam == srg.FAMILY_QKV else "B_o"]
            bias = None if self.bias is None else self.bias["bias_qkv" if fam == srg.FAMILY_QKV else "bias_o"]
            if fused:
                log(f"  launch delta family={fam} path={path} routing={routing} end={self.end} G={self.G}"
                    f" bias={bias is not None} noalloc={noalloc}")
                if noalloc:
                    srg.lora_sgmv_delta_noalloc(self.dims, fam, self.dev[xk], A, B, rt, self.dev[yk], path,
                                                bias=bias, options=options)
                else:
                    srg.lora_sgmv_delta(self.dims, fam, self.dev[xk], A, B, rt, self.dev[yk], self.ws[fam], path,
                                        bias=bias, options=options)
                continue
            log(f"  launch shrink+expand family={fam} path={path} routing={routing} end={self.end} G={self.G}"
                f" bias={bias is not None}")
            srg.lora_sgmv_shrink(self.dims, fam, self.dev[xk], A, rt, self.u[fam], self.ws[fam], path)
            srg.lora_sgmv_expand(self.dims, fam, self.u[fam], B, rt, self.dev[yk], path, bias=bias)
        import torch
        torch.cuda.synchronize()

    def y_arrival(self, key: str) -> np.ndarray:
        ys = from_dev(self.dev[key])
        out = np.empty_like(ys[:self.T])
        out[self.tok_order] = ys[:self.T]
        return out

    def u_arrival(self, fam) -> np.ndarray:
        us = from_dev(self.u[fam])[:self.end]
        out = np.full((self.T, us.shape[1]), np.nan, np.float32)
        out[self.tok_order[:self.end]] = us
        return out


def oracle_layer(w: synth.Workload, stacks: Dict[str, np.ndarray], lengths, slots, acts,
                 requests: Optional[Sequence[int]] = None, token_rows=None,
                 bias: Optional[Dict[str, np.ndarray]] = None):
    """Oracle reference of both families: {family: {request: (rows, y_ref, u)}}."""
    offs = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    R = w.max_lora_rank
    st = stacks["ref"]
    bq = None if bias is None else bias["ref"]["bias_qkv"]
    bo = None if bias is None else bias["ref"]["bias_o"]
    ref = {}
    ref[srg.FAMILY_QKV] = oracle.reference_family(acts["x_qkv"], acts["y_qkv"], offs, slots,
                                                  st["A_qkv"], st["B_qkv"],
                                                  [w.nq, w.nkv, w.nkv], R, w.dtype, requests, token_rows, bq)
    ref[srg.FAMILY_O] = oracle.reference_family(acts["x_o"], acts["y_o"], offs, slots, st["A_o"],
                                                st["B_o"], [w.hidden], R, w.dtype, requests, token_rows, bo)
    return ref


def compare(w: synth.Workload, gl: GpuLayer, ref, check_u: bool = True):
    """Returns (max y rel err, max u rel err) over both families and asserts
    base requests' rows are bit-identical to y_in."""
    worst_y, worst_u = 0.0, 0.0
    for fam, yk in ((srg.FAMILY_QKV, "y_qkv"), (srg.FAMILY_O, "y_o")):
        y = gl.y_arrival(yk)
        u = gl.u_arrival(fam) if check_u else None
        got_all, ref_all, ug, ur = [], [], [], []
        for i, (rows, yref, uref) in ref[fam].items():
            a = int(gl.offs[i])
            g = y[a + rows]
            if uref is None:
                assert np.array_equal(g.astype(np.float64), yref), f"base request {i} rows changed"
                continue
            got_all.append(g)
            ref_all.append(yref)
            if check_u:
                ug.append(u[a + rows])
                ur.append(uref)
        if got_all:
            worst_y = max(worst_y, rel_err(np.concatenate(got_all), np.concatenate(ref_all)))
            if check_u:
                worst_u = max(worst_u, rel_err(np.concatenate(ug), np.concatenate(ur)))
    return worst_y, worst_u
