#!/usr/bin/env python3
"""Benchmark of the segment-routed multi-adapter LoRA delta on one MI355X.

A step is one batch through the whole hot path: host routing of the batch
(lora_build_routing), upload of the routing arrays, then for every layer the
fused-QKV delta (shrink + expand) and the o_proj delta (shrink + expand), by
default through lora_sgmv_delta (one call per family; on decode batches that
is one kernel).  Adapters are packed (lora_pack_adapter) once, at activation,
before timing.

Default workload: Llama-3-8B attention (hidden 4096, 32 heads, 8 kv heads,
head_dim 128), 256 one-token decode requests, 8 adapter slots with ranks 8/16
padded to 16, 25% base requests, bf16 data with fp32 accumulation, run over
64 distinct layer replicas per step so that no layer's data is still in the
256 MB last-level cache when it is read again.

Output: one JSON line (rank 0).  `value` = LoRA-routed tokens x layers per
second (tokens through one layer's q/k/v/o delta per second).

Options that change the work: --bias (every adapter also carries a LoRA
bias), --token-routing (per-token routing: x and y stay in token order and
the kernels gather and scatter rows through the sorted token indices, built
and uploaded every step), --workload, --api, --path.

Phases:
  1. timed steps, the layer loop captured once in a HIP graph and replayed
     (host routing + routing upload stay eager every step);
  2. per call kind, the call over all layers back to back between two HIP
     events on the launch stream: average duration per call -> roofline of
     the dominant call (algorithmic bytes / duration);
  3. the CPU oracle on a bounded sample of the same workload (one core).

Counter runs (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE):
  bench.py --counters delta_qkv [--workload ...]       (GPU, under rocprofv3)
  bench.py --traffic-from FETCH.csv WRITE.csv --traffic-kind delta_qkv
writes profiles/traffic.json (HBM bytes per call, calibrated against a plain
256 MiB copy in the same run), which the roofline line reports as `traffic`
while the kernel source is unchanged.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
REPLICAS = {"tiny": 1, "decode": 64, "prefill": 4, "mixed": 8, "stack": 32, "mlp": 32}
KERNEL_SRC = os.path.join(ROOT, "segmented_rank_gemv_amd", "csrc", "lora_sgmv.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


UPLOAD_PIECE = 4096  # int32 entries per host-to-device copy of the token indices
GRAPH_CALLS = 16     # least calls per captured graph when timing one call kind
PREFILL_LAYERS = 4   # layer replicas of the prefill leg of the default run


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode", choices=list(REPLICAS))
    p.add_argument("--layers", type=int, default=0, help="override layer replicas per step")
    p.add_argument("--path", default="auto", choices=["auto", "valu", "mfma", "fused"])
    p.add_argument("--api", default="delta", choices=["delta", "split"],
                   help="delta: lora_sgmv_delta per family; split: lora_sgmv_shrink + lora_sgmv_expand")
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--bias", action="store_true", help="every adapter also carries a LoRA bias per projection")
    p.add_argument("--token-routing", action="store_true",
                   help="per-token routing: x and y stay in token order; each step builds the token "
                        "routing (lora_build_token_routing) and uploads the sorted token indices")
    p.add_argument("--device-routing", action="store_true",
                   help="kernels read the routing from device memory only (no host copies)")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-prefill", action="store_true",
                   help="skip the prefill leg that the default (decode) run also measures")
    p.add_argument("--counters", metavar="KIND", default=None,
                   help="counter-collection run: a plain copy of COPY_MIB MiB (calibration), then the "
                        "call KIND (e.g. delta_qkv) over every layer twice; no timing, no JSON line")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                   help="write profiles/traffic.json from the counter_collection.csv files of two "
                        "--counters runs (FETCH_SIZE, then WRITE_SIZE); needs no GPU")
    p.add_argument("--traffic-kind", default="delta_qkv")
    p.add_argument("--counter-summary", nargs="+", metavar="CSV", default=None,
                   help="print per-kernel means of the counters in rocprofv3 --pmc counter_collection.csv "
                        "files and the derived MFMA / VALU / L2 figures; needs no GPU")
    p.add_argument("--trace-summary", nargs=2, metavar=("STATS_CSV", "TRACE_CSV"), default=None,
                   help="print the kernel table of a rocprofv3 --kernel-trace --stats -f csv run, the "
                        "library's kernels split by launch grid and, when the run also had --marker-trace "
                        "(p_marker_api_trace.csv next to TRACE_CSV), by timed call kind; needs no GPU")
    return p.parse_args()


COPY_MIB = 256


def summarize_traffic(args):
    """HBM bytes per call of one call kind from rocprofv3 --pmc runs.

    FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the library's kernels are
    scaled by the ratio known bytes / counter value of a plain copy kernel of
    COPY_MIB MiB measured in the same run; a call of several kernels (split
    shrink + slab reduction, or the two-kernel delta) adds its kernels."""
    import csv
    from collections import defaultdict

    def read(path, counter):
        lib, copy = defaultdict(list), []
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"])
                name = r["Kernel_Name"]
                if "lora::" in name:
                    lib[name].append(v)
                elif "copyBuffer" in name and v * 1024 >= 0.25 * COPY_MIB * 2**20:
                    copy.append(v)
        if not copy or not lib:
            raise SystemExit(f"{path}: no calibration copy or no library kernel with {counter}")
        return lib, float(np.mean(copy))

    fetch, fetch_copy = read(args.traffic_from[0], "FETCH_SIZE")
    write, write_copy = read(args.traffic_from[1], "WRITE_SIZE")
    known = COPY_MIB * 2**20
    f_fac, w_fac = known / (fetch_copy * 1024), known / (write_copy * 1024)
    kern = {}
    total = 0.0
    for name in sorted(fetch):
        fk, wk = float(np.mean(fetch[name])), float(np.mean(write.get(name, [0.0])))
        b = fk * 1024 * f_fac + wk * 1024 * w_fac
        kern[name] = {"dispatches": len(fetch[name]), "fetch_kib": fk, "write_kib": wk, "hbm_bytes": b}
        total += b
    out = {"kernel_sha": kernel_sha(),
           "copy_calibration": {"bytes": known, "fetch_kib": fetch_copy, "write_kib": write_copy,
                                "fetch_factor": f_fac, "write_factor": w_fac},
           "kernels": {f"{args.workload}:{args.traffic_kind}": {"hbm_bytes_per_launch": total,
                                                                "per_kernel": kern}}}
    old = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            old = json.load(fh)
    if old.get("kernel_sha") == out["kernel_sha"]:
        old.setdefault("kernels", {}).update(out["kernels"])
        old["copy_calibration"] = out["copy_calibration"]
        out = old
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out["kernels"]), flush=True)


MI355X_SIMDS = 256 * 4  # compute units x SIMDs per CU
MI355X_XCDS = 8
L2_LINE = 128           # bytes per L1 -> L2 read request (one cache line)


def counter_summary(paths):
    """Per-kernel means of every counter in rocprofv3 --pmc CSV files (the
    library's kernels only) and derived figures:
      mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x SIMDs):
        the share of the kernel's time the matrix cores were busy, chip-wide;
      mfma_bf16_flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (the counter
        counts adds and multiplies in units of 512) per dispatch;
      l1_to_l2_read_bytes = TCP_TCC_READ_REQ_sum x 128 (one line per request);
      l2_hit_rate = TCC_HIT / (TCC_HIT + TCC_MISS)."""
    import csv
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(list))
    dur = defaultdict(list)
    for path in paths:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                if "lora::" not in name:
                    continue
                short = name.split("(anonymous namespace)::")[1].split("(lora")[0] if "namespace)::" in name else name
                key = f"{short} grid={r.get('Grid_Size', '?')}"
                vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
                try:
                    dur[key].append((float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) * 1e-3)
                except (KeyError, ValueError):
                    pass
    out = {}
    for key in sorted(vals):
        c = {k: float(np.mean(v)) for k, v in vals[key].items()}
        d = {"counters": c, "dispatches": max(len(v) for v in vals[key].values())}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and c.get("GRBM_GUI_ACTIVE"):
            # GRBM_GUI_ACTIVE accumulates over the 8 XCDs (it reads 8x the
            # dispatch's duration x clock); the MFMA busy cycles over all SIMDs
            d["mfma_busy"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / MI355X_XCDS * MI355X_SIMDS)
        if "TCP_TCC_READ_REQ_sum" in c:
            d["l1_to_l2_read_bytes"] = c["TCP_TCC_READ_REQ_sum"] * L2_LINE
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
            d["mfma_bf16_flops"] = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        if "TCC_HIT_sum" in c and c.get("TCC_HIT_sum", 0) + c.get("TCC_MISS_sum", 0) > 0:
            d["l2_hit_rate"] = c["TCC_HIT_sum"] / (c["TCC_HIT_sum"] + c["TCC_MISS_sum"])
        out[key] = d
        print(key, json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()
                               if k != "counters"}), json.dumps({k: round(v, 1) for k, v in c.items()}),
              flush=True)
    return out


def _short_kernel(name, width=62):
    name = name.replace("(anonymous namespace)::", "")
    name = name.split("(lora::")[0]
    if name.endswith("(long)"):
        name = name[:-len("(long)")]
    return name[:width]


def trace_summary(stats_csv, trace_csv):
    """The kernel statistics of a rocprofv3 --kernel-trace --stats -f csv run
    (every dispatch of the run), then the library's kernels split by launch
    grid (workgroups x workgroup size), which separates the families and
    call kinds that share one kernel instantiation with different grids.
    With the run's marker trace (--marker-trace: the marker_api_trace.csv
    file beside trace_csv), also the library's dispatches inside each range
    that the per-call timing opens around one call kind ("workload:kind"):
    the per-kind figures that the bench line's avg_launch_us is measured on,
    also where two call kinds share a kernel and a grid."""
    import csv
    import glob
    import statistics
    from collections import defaultdict
    print(f"{'kernel':62s} {'calls':>8s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>8s}")
    with open(stats_csv) as fh:
        for r in csv.DictReader(fh):
            print(f"{_short_kernel(r['Name']):62s} {int(r['Calls']):8d} {float(r['AverageNs']) / 1e3:10.2f} "
                  f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):8.2f}")
    print()
    print("Library kernels split by launch grid (workgroups x workgroup size):")
    print()
    grids = defaultdict(list)
    with open(trace_csv) as fh:
        for r in csv.DictReader(fh):
            if "lora::" not in r["Kernel_Name"]:
                continue
            wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r.get("Workgroup_Size_Z", 1))
            n = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) // wg
            grids[(_short_kernel(r["Kernel_Name"]), n, wg)].append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"{'kernel':62s} {'wgs':>6s} {'wg':>5s} {'calls':>7s} {'avg_us':>10s} {'median_us':>10s}")
    for (n, nwg, wg), d in sorted(grids.items(), key=lambda kv: -len(kv[1])):
        print(f"{n:62s} {nwg:6d} {wg:5d} {len(d):7d} {statistics.mean(d):10.2f} {statistics.median(d):10.2f}")
    markers = sorted(glob.glob(os.path.join(os.path.dirname(os.path.abspath(trace_csv)), "*marker_api_trace.csv")))
    if not markers:
        return
    ranges = []
    with open(markers[0]) as fh:
        for r in csv.DictReader(fh):
            if ":" in r["Function"]:
                ranges.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Function"]))
    ranges.sort()
    kinds = defaultdict(list)
    with open(trace_csv) as fh:
        for r in csv.DictReader(fh):
            if "lora::" not in r["Kernel_Name"]:
                continue
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            hit = [name for (a, b, name) in ranges if a <= t0 and t1 <= b]
            if hit:
                kinds[(hit[-1], _short_kernel(r["Kernel_Name"]))].append((t1 - t0) / 1e3)
    print()
    print("Library kernels inside the per-call timing ranges (workload:call kind):")
    print()
    print(f"{'range':24s} {'kernel':62s} {'calls':>7s} {'avg_us':>10s} {'median_us':>10s}")
    for (rng, n), d in sorted(kinds.items()):
        print(f"{rng:24s} {n:62s} {len(d):7d} {statistics.mean(d):10.2f} {statistics.median(d):10.2f}")


def cpu_identity() -> str:
    """The host CPU as /proc/cpuinfo names it: model name, vendor, family,
    model and stepping (some virtual machines shorten the model name)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if not line.strip():
                    break
                k, _, v = line.partition(":")
                fields.setdefault(k.strip(), v.strip())
    except OSError:
        return "unknown"
    return (f"{fields.get('model name', '?')} ({fields.get('vendor_id', '?')}, family "
            f"{fields.get('cpu family', '?')}, model {fields.get('model', '?')}, stepping "
            f"{fields.get('stepping', '?')})")


def kernel_sha() -> str:
    """Hash of the kernel source's code: comments, trailing blanks and empty
    lines removed, so that an edit of a comment keeps counter figures taken
    with the same code valid."""
    with open(KERNEL_SRC, encoding="utf-8") as f:
        src = f.read()
    tok = re.compile(r'("(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\')|//[^\n]*|/\*.*?\*/', re.S)
    code = tok.sub(lambda m: m.group(1) or "", src)
    lines = [ln.rstrip() for ln in code.splitlines()]
    return hashlib.sha256("\n".join(ln for ln in lines if ln).encode()).hexdigest()[:16]


def run_workload(args, torch, synth, srg, dev, log):
    """One workload on the GPU: pack its adapters, lay out its layers, time
    args.steps whole steps (phase 1) and every call kind (phase 2).  Returns
    the measurements and the objects the extra legs reuse, or None for a
    counter-collection run."""
    path = {"auto": srg.PATH_AUTO, "valu": srg.PATH_VALU, "mfma": srg.PATH_MFMA,
            "fused": srg.PATH_FUSED}[args.path]
    w = synth.get_workload(args.workload)
    n_layers = args.layers or REPLICAS[args.workload]
    if args.workload == "stack" and not args.layers:
        n_layers = w.n_layers
    mlp = w.intermediate > 0
    dims = srg.LoraDims(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, w.max_lora_rank,
                        w.max_num_loras, w.dtype, w.intermediate)
    # projection families of the workload: (family, name, x, y, A stack, B stack, PEFT projections)
    if mlp:
        FAMS = ((srg.FAMILY_GATE_UP, "gu", "x_gu", "y_gu", "A_gu", "B_gu", ("gate", "up")),
                (srg.FAMILY_DOWN, "down", "x_down", "y_down", "A_down", "B_down", ("down",)))
    else:
        FAMS = ((srg.FAMILY_QKV, "qkv", "x_qkv", "y_qkv", "A_qkv", "B_qkv", ("q", "k", "v")),
                (srg.FAMILY_O, "o", "x_o", "y_o", "A_o", "B_o", ("o",)))
    lengths, slots = synth.draw_requests(w)
    ranks = synth.draw_ranks(w)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(offsets[-1])
    L, R = w.max_num_loras, w.max_lora_rank
    bf16 = w.dtype == "bf16"
    tdt = torch.bfloat16 if bf16 else torch.float32

    # routing once to lay the batch out in sorted order (the serving layer
    # sorts its batch once; the timed steps still route on the host)
    token_slot = np.repeat(slots, lengths).astype(np.int32)
    if args.token_routing:
        # the batch stays in token order; the kernels gather and scatter rows
        rt0 = srg.lora_build_token_routing(token_slot, L)
        order = np.arange(T)
    else:
        rt0 = srg.lora_build_routing(slots, offsets, L)
        order = np.concatenate([np.arange(offsets[p], offsets[p + 1]) for p in rt0["perm"]])
    end, G = rt0["end"], rt0["num_groups"]
    fam_shape = {fm[0]: srg.lora_family_shape(dims, fm[0]) for fm in FAMS}
    proj_desc = "gate/up/down" if mlp else "q/k/v/o"
    log(f"workload={w.name} T={T} end={end} G={G} layers={n_layers}")

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        if bf16:
            return torch.from_numpy(synth.bf16_bits(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    # ---- activation: pack every slot of every layer, upload stacks and data
    t_pack = 0.0
    n_pack = 0
    layers = []
    for l in range(n_layers):
        st = {k: [] for fm in FAMS for k in fm[4:6]}
        for s in range(L):
            if mlp:
                wts = synth.draw_mlp_adapter(w, l, s, int(ranks[s]))
                t0 = time.perf_counter()
                pk = {}
                for f, nm, xk, yk, ak, bk, projs in FAMS:
                    r = srg.lora_pack_family(dims, f, int(ranks[s]), w.lora_alpha, w.use_rslora, True,
                                             [wts[p] for p in projs])
                    pk[ak], pk[bk] = r["A"], r["B"]
            else:
                wts = synth.draw_adapter(w, l, s, int(ranks[s]))
                t0 = time.perf_counter()
                pk = srg.lora_pack_adapter(dims, int(ranks[s]), w.lora_alpha, w.use_rslora, True, "qkvo", wts)
            if args.bias:
                bias = synth.draw_bias(w, l, s, tuple(p for fm in FAMS for p in fm[6]))
                for f, nm, xk, yk, ak, bk, projs in FAMS:
                    pk["bias_" + nm] = srg.lora_pack_bias(dims, f, [bias[p] for p in projs])
                    st.setdefault("bias_" + nm, [])
            t_pack += time.perf_counter() - t0
            n_pack += 1
            for k in st:
                st[k].append(pk[k])
        acts = synth.draw_mlp_activations(w, l, T) if mlp else synth.draw_activations(w, l, T)
        layer = {k: to_dev(np.stack(v)) for k, v in st.items()}
        for fm in FAMS:
            for k in fm[2:4]:
                layer[k] = to_dev(np.ascontiguousarray(acts[k][order]))
        layers.append(layer)
        if (l + 1) % 16 == 0:
            log(f"  prepared {l + 1}/{n_layers} layers")
    u = {f: torch.zeros((max(end, 1), fam_shape[f][1] * R), dtype=torch.float32, device=dev)
         for f in fam_shape}
    ws = {f: torch.zeros(max(srg.lora_sgmv_workspace_bytes(dims, f, max(end, 1)), 16) // 4 + 4,
                         dtype=torch.int32, device=dev) for f in fam_shape}
    ids_dev = torch.zeros(L, dtype=torch.int32, device=dev)
    offs_dev = torch.zeros(L + 1, dtype=torch.int32, device=dev)
    ids_pin = torch.zeros(L, dtype=torch.int32).pin_memory()
    offs_pin = torch.zeros(L + 1, dtype=torch.int32).pin_memory()
    # the routing the kernels see: device arrays (refreshed every step) plus,
    # unless --device-routing, host copies passed as launch arguments
    rows_dev = torch.zeros(max(end, 1), dtype=torch.int32, device=dev)
    rows_pin = torch.zeros(max(end, 1), dtype=torch.int32).pin_memory()
    routing = srg.LoraRouting(ids_dev, offs_dev, G, end,
                              None if args.device_routing else rt0["lora_ids"],
                              None if args.device_routing else rt0["grouped_offsets"],
                              rows_dev if args.token_routing else None, T)

    def route_and_upload():
        rt = (srg.lora_build_token_routing(token_slot, L) if args.token_routing
              else srg.lora_build_routing(slots, offsets, L))
        assert rt["end"] == end and rt["num_groups"] == G
        assert np.array_equal(rt["lora_ids"], rt0["lora_ids"])
        assert np.array_equal(rt["grouped_offsets"], rt0["grouped_offsets"])
        ids_pin[:G].copy_(torch.from_numpy(rt["lora_ids"]))
        offs_pin[:G + 1].copy_(torch.from_numpy(rt["grouped_offsets"]))
        ids_dev.copy_(ids_pin, non_blocking=True)
        offs_dev.copy_(offs_pin, non_blocking=True)
        if args.token_routing:
            assert np.array_equal(rt["token_indices_sorted"], rt0["token_indices_sorted"])
            rows_pin[:end].copy_(torch.from_numpy(rt["token_indices_sorted"][:end]))
            # in pieces of 16 KB: a larger pinned copy blocks the host until
            # the stream drains (measured), which would serialise the steps
            for c0 in range(0, max(end, 1), UPLOAD_PIECE):
                rows_dev[c0:c0 + UPLOAD_PIECE].copy_(rows_pin[c0:c0 + UPLOAD_PIECE], non_blocking=True)

    if args.api == "delta":
        KINDS = tuple("delta_" + fm[1] for fm in FAMS)
    else:
        KINDS = tuple(k + "_" + fm[1] for fm in FAMS for k in ("shrink", "expand"))
    BY_NAME = {fm[1]: fm for fm in FAMS}

    def call(kind, ly):
        f, nm, xk, yk, ak, bk, _ = BY_NAME[kind.split("_", 1)[1]]
        bias = ly.get("bias_" + nm)
        if kind.startswith("delta"):
            srg.lora_sgmv_delta(dims, f, ly[xk], ly[ak], ly[bk], routing, ly[yk], ws[f], path, bias=bias)
        elif kind.startswith("shrink"):
            srg.lora_sgmv_shrink(dims, f, ly[xk], ly[ak], routing, u[f], ws[f], path)
        else:
            srg.lora_sgmv_expand(dims, f, u[f], ly[bk], routing, ly[yk], path, bias=bias)

    def layer_pass(ly):
        for kind in KINDS:
            call(kind, ly)

    def all_layers():
        for ly in layers:
            layer_pass(ly)

    stream = torch.cuda.Stream()
    if args.counters:
        # counter-collection run: calibration copy, then only the counted
        # call, twice per layer (no other call runs in this process)
        src = torch.ones(COPY_MIB * 2**20 // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            route_and_upload()
            for _ in range(3):
                dst.copy_(src)
            for _ in range(2):
                for ly in layers:
                    call(args.counters, ly)
        torch.cuda.synchronize()
        log(f"counters: copy {COPY_MIB} MiB x 3, {args.counters} x {2 * n_layers}")
        return None

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        route_and_upload()
        all_layers()  # first eager pass (also loads the code objects)
    torch.cuda.synchronize()

    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            all_layers()
        torch.cuda.synchronize()

    host_route_s = [0.0]

    def step():
        t0 = time.perf_counter()
        route_and_upload()
        host_route_s[0] += time.perf_counter() - t0
        if graph is not None:
            graph.replay()
        else:
            all_layers()

    # ---- phase 1: timed steps
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        host_route_s[0] = 0.0
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    log(f"phase 1: {ms_per_step:.4f} ms/step")

    # ---- phase 2: per-call durations with HIP events on the launch stream.
    # For every call kind the same call runs over all layers back to back
    # (cold data, as in the step) between one pair of events.  With graphs
    # (the default, as in the timed step) each kind's sequence is one
    # captured graph, so the events time the kernels as the step launches
    # them; without, a bounded spin kernel (torch.cuda._sleep) runs first so
    # that the host has queued the whole eager sequence before the GPU
    # reaches it, so the events time the kernels and not the host's launch
    # rate.
    ev_reps = max(1, min(args.steps, 20))
    # at least GRAPH_CALLS calls per captured graph (passes over the layers
    # repeated), so that the graph launch itself is a small part of each
    # timed sequence
    passes = max(1, -(-GRAPH_CALLS // n_layers)) if graph is not None else 1
    total_ms = {k: 0.0 for k in KINDS}
    kind_graphs = {}
    if graph is not None:
        for kind in KINDS:
            kg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(kg, stream=stream):
                for _ in range(passes):
                    for ly in layers:
                        call(kind, ly)
            kind_graphs[kind] = kg
        torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        route_and_upload()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for ly in layers:
            call(KINDS[0], ly)
        enqueue_s = time.perf_counter() - t0
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(1_000_000)
        e1.record()
        torch.cuda.synchronize()
        s_per_cycle = max(e0.elapsed_time(e1) * 1e-3 / 1e6, 1e-12)
        spin = int(min(3.0 * enqueue_s / s_per_cycle + 1e5, 2e10))
        for _ in range(ev_reps):
            for kind in KINDS:
                # a named range (ROCTX) around each timed sequence, so that a
                # profiler's marker trace attributes its kernels to the kind
                torch.cuda.nvtx.range_push(f"{args.workload}:{kind}")
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda._sleep(spin)
                a.record()
                if kind in kind_graphs:
                    kind_graphs[kind].replay()
                else:
                    for ly in layers:
                        call(kind, ly)
                b.record()
                torch.cuda.synchronize()
                torch.cuda.nvtx.range_pop()
                total_ms[kind] += a.elapsed_time(b)
    avg_us = {k: 1e3 * total_ms[k] / (ev_reps * n_layers * (passes if k in kind_graphs else 1)) for k in KINDS}
    log("phase 2: " + " ".join(f"{k}={v:.2f}us" for k, v in avg_us.items()))

    # algorithmic bytes per call (u, the rank-space intermediate, counted for
    # the split calls that move it through memory; not for the delta call)
    b = 2 if bf16 else 4
    kbytes, kflops = {}, {}
    for f, nm, *_ in FAMS:
        fin, n_s, widths, fout = fam_shape[f]
        C = n_s * R
        x_b, a_b = end * fin * b, G * C * fin * b
        b_b, y_b = G * fout * R * b, 2 * end * fout * b
        if args.bias:
            b_b += G * fout * b  # the groups' bias rows
        u_b = end * C * 4
        kbytes["shrink_" + nm] = x_b + a_b + u_b
        kbytes["expand_" + nm] = u_b + b_b + y_b
        kbytes["delta_" + nm] = x_b + a_b + b_b + y_b
        kflops["shrink_" + nm] = 2 * end * C * fin
        kflops["expand_" + nm] = 2 * end * fout * R
        kflops["delta_" + nm] = kflops["shrink_" + nm] + kflops["expand_" + nm]
    fam_bytes = sum(kbytes["delta_" + nm] for _, nm, *_ in FAMS)
    dominant = max(KINDS, key=lambda k: avg_us[k])
    achieved = kbytes[dominant] / (avg_us[dominant] * 1e-6) / 1e9

    traffic = None
    try:
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        key = f"{w.name}:{dominant}"
        if not args.bias and tr.get("kernel_sha") == kernel_sha() and key in tr.get("kernels", {}):
            traffic = tr["kernels"][key]["hbm_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        traffic = None

    value = end * n_layers / (ms_per_step * 1e-3)
    e2e_gbs = fam_bytes * n_layers / (ms_per_step * 1e-3) / 1e9

    del kind_graphs, graph
    return {"w": w, "n_layers": n_layers, "mlp": mlp, "dims": dims, "FAMS": FAMS, "lengths": lengths,
            "slots": slots, "ranks": ranks, "offsets": offsets, "T": T, "L": L, "R": R, "bf16": bf16,
            "end": end, "G": G, "fam_shape": fam_shape, "proj_desc": proj_desc, "layers": layers,
            "stream": stream, "ms_per_step": ms_per_step, "host_route_s": host_route_s[0], "KINDS": KINDS,
            "avg_us": avg_us, "kbytes": kbytes, "kflops": kflops, "fam_bytes": fam_bytes, "dominant": dominant,
            "achieved": achieved, "traffic": traffic, "value": value, "e2e_gbs": e2e_gbs, "t_pack": t_pack,
            "n_pack": n_pack, "graph_calls": passes * n_layers}


def main():
    args = parse()
    if args.traffic_from:
        summarize_traffic(args)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.gpus != 1:
        print(f"bench.py: this benchmark measures one GPU; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding is a design note only)", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import synth
    import segmented_rank_gemv_amd as srg

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)

    ctx = run_workload(args, torch, synth, srg, dev, log)
    if ctx is None:
        return
    w, n_layers, mlp, dims, FAMS = ctx["w"], ctx["n_layers"], ctx["mlp"], ctx["dims"], ctx["FAMS"]
    lengths, slots, ranks, offsets, T = ctx["lengths"], ctx["slots"], ctx["ranks"], ctx["offsets"], ctx["T"]
    L, R, bf16, end, G = ctx["L"], ctx["R"], ctx["bf16"], ctx["end"], ctx["G"]
    fam_shape, proj_desc, layers, stream = ctx["fam_shape"], ctx["proj_desc"], ctx["layers"], ctx["stream"]
    KINDS, avg_us, kbytes, kflops = ctx["KINDS"], ctx["avg_us"], ctx["kbytes"], ctx["kflops"]
    dominant, achieved, traffic = ctx["dominant"], ctx["achieved"], ctx["traffic"]
    ms_per_step, value, e2e_gbs = ctx["ms_per_step"], ctx["value"], ctx["e2e_gbs"]

    # ---- the prefill workload beside the decode headline (default run only):
    # the same call through lora_sgmv_delta on the Llama-3-8B prefill batch
    prefill = None
    if (args.workload == "decode" and not args.no_prefill and not args.layers and not args.bias
            and not args.token_routing and not args.device_routing and args.path == "auto" and args.api == "delta"):
        pargs = argparse.Namespace(**{**vars(args), "workload": "prefill", "layers": PREFILL_LAYERS,
                                      "steps": min(args.steps, 40), "warmup": min(args.warmup, 5)})
        pre = run_workload(pargs, torch, synth, srg, dev, log)
        prefill = {"workload": "prefill", "lora_tokens": pre["end"], "tokens": pre["T"], "groups": pre["G"],
                   "layers_per_step": pre["n_layers"], "ms_per_step": pre["ms_per_step"],
                   "value": pre["value"], "unit": "LoRA tokens x layers / s (q/k/v/o delta)",
                   "end_to_end_GBps": pre["e2e_gbs"], "frac": pre["e2e_gbs"] / HBM_PEAK_GBS,
                   "calls": {k: {"avg_us": pre["avg_us"][k], "bytes": pre["kbytes"][k],
                                 "GBps": pre["kbytes"][k] / (pre["avg_us"][k] * 1e-6) / 1e9,
                                 "frac": pre["kbytes"][k] / (pre["avg_us"][k] * 1e-6) / 1e9 / HBM_PEAK_GBS}
                             for k in pre["KINDS"]},
                   "calls_per_timed_graph": pre["graph_calls"]}
        log(f"prefill: {pre['ms_per_step']:.4f} ms/step ({PREFILL_LAYERS} layers), "
            + " ".join(f"{k}={v['avg_us']:.2f}us ({v['frac']:.3f})" for k, v in prefill["calls"].items()))
        del pre
        torch.cuda.empty_cache()

    # ---- reference streams (outside the step): what plain device kernels
    # reach on this GPU, beside the 8 TB/s nameplate -- an in-place add over
    # 1 GiB of bf16 (read + write, like the expand's y) and a row-wise max
    # over the same bytes (read only, like the shrink's x)
    stream_ref = None
    if not args.counters:
        big = torch.empty(2**29, dtype=torch.bfloat16, device=dev).normal_()
        rows2d = big.view(-1, 4096)

        def ev_time(fn, reps=10):
            fn()
            torch.cuda.synchronize()
            ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ea.record()
            for _ in range(reps):
                fn()
            eb.record()
            torch.cuda.synchronize()
            return ea.elapsed_time(eb) * 1e-3 / reps

        nbytes = big.numel() * 2
        t_rw = ev_time(lambda: big.add_(1.0))
        t_rd = ev_time(lambda: rows2d.amax(dim=1))
        stream_ref = {"inplace_add_GBps": 2 * nbytes / t_rw / 1e9, "row_max_read_GBps": nbytes / t_rd / 1e9,
                      "bytes": nbytes}
        del big, rows2d
        torch.cuda.empty_cache()
        # launch-sized legs: one in-place add per launch moving as many bytes
        # (read + write) as one call of each kind of the headline workload,
        # over 64 rotating buffers, captured in one graph: what a single
        # plain launch over that many bytes reaches here
        legs = {}
        for kind in KINDS:
            moved = kbytes[kind]
            elems = max(8, int(moved // 4) // 8 * 8)  # bf16 elements of one buffer (read + write = moved)
            bufs = [torch.zeros(elems, dtype=torch.bfloat16, device=dev) for _ in range(64)]
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                for b in bufs:
                    b.add_(1.0)
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=stream):
                    for b in bufs:
                        b.add_(1.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 10
            ea.record()
            for _ in range(reps):
                g.replay()
            eb.record()
            torch.cuda.synchronize()
            us = 1e3 * ea.elapsed_time(eb) / (reps * len(bufs))
            legs[kind] = {"bytes": 4 * elems, "avg_us": us, "GBps": 4 * elems / (us * 1e-6) / 1e9,
                          "frac": 4 * elems / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                          "kernel_vs_reference": avg_us[kind] / us}
            del bufs, g
        torch.cuda.empty_cache()
        stream_ref["launch_sized_inplace_add"] = legs
        log("launch-sized in-place add: " + " ".join(f"{k}: {v['bytes'] / 1e6:.2f} MB {v['avg_us']:.2f}us "
                                                      f"({v['frac']:.3f}; call/ref {v['kernel_vs_reference']:.2f})"
                                                      for k, v in legs.items()))
        log(f"reference streams: in-place add {stream_ref['inplace_add_GBps']:.0f} GB/s, "
            f"row max read {stream_ref['row_max_read_GBps']:.0f} GB/s")

    # ---- adapter activation (outside the step): the slot cache's decisions
    # for a stream of batches over twice as many adapters as slots, and the
    # host-to-device writes of one adapter into one slot of every layer
    # (lora_write_slot from pinned host memory, timed with events on the
    # stream).  Each slot is rewritten with the adapter it already holds, so
    # the stacks are unchanged.
    activation = None
    if L > 1 and not mlp:
        cache = srg.LoraSlotCache(L)
        crng = np.random.default_rng(5)
        nb, loads = 2000, 0
        t0 = time.perf_counter()
        for _ in range(nb):
            ids = crng.integers(-1, 2 * L, size=len(slots))
            keep = [a for a in dict.fromkeys(ids.tolist()) if a >= 0][:L]
            ids = np.where(np.isin(ids, keep), ids, -1)
            loads += len(cache.activate_batch(ids)[1])
        cache_us = 1e6 * (time.perf_counter() - t0) / nb
        wl = min(n_layers, 16)
        pinned = []
        for l in range(wl):
            s0 = l % L
            pk = srg.lora_pack_adapter(dims, int(ranks[s0]), w.lora_alpha, w.use_rslora, True, "qkvo",
                                       synth.draw_adapter(w, l, s0, int(ranks[s0])))
            pinned.append((s0, {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16 if v.dtype == np.uint16
                                                                                  else np.float32)).pin_memory()
                                for k, v in pk.items()}))
        slot_bytes = sum(v.numel() * v.element_size() for v in pinned[0][1].values())
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 4
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            ea.record(stream)
            for _ in range(reps):
                for l, (s0, pk) in enumerate(pinned):
                    srg.lora_write_slot(dims, s0, pk, {k: layers[l][k] for k in ("A_qkv", "B_qkv", "A_o", "B_o")},
                                        stream=stream)
            eb.record(stream)
        torch.cuda.synchronize()
        write_us = 1e3 * ea.elapsed_time(eb) / (reps * wl)
        activation = {"slots": L, "batches": nb, "loads_per_batch": loads / nb,
                      "cache_us_per_batch": cache_us, "slot_bytes_per_layer": slot_bytes,
                      "write_us_per_slot_layer": write_us,
                      "h2d_GBps": slot_bytes / (write_us * 1e-6) / 1e9}
        log(f"activation: cache {cache_us:.2f} us/batch, write {write_us:.2f} us/slot-layer "
            f"({activation['h2d_GBps']:.1f} GB/s)")

    # ---- phase 3: CPU oracle on a bounded sample: whole layers (both
    # families) of the same workload, cycling over a few distinct layers and
    # rotating which requests a layer's row budget covers, until about
    # --cpu-seconds of oracle time has been spent
    cpu = None
    if not args.no_cpu:
        import oracle
        tokens_done, t_cpu, n_calls = 0, 0.0, 0
        prepared = []
        n_distinct = min(n_layers, 4)
        lora_req = [i for i in range(len(slots)) if slots[i] >= 0]
        # bound the rows per call for the long workloads (about 0.1-1 s each)
        f0 = FAMS[0][0]
        budget = max(1, int(2e8 // (fam_shape[f0][0] * fam_shape[f0][1] * R + fam_shape[f0][3] * R)))
        # the oracle is single-threaded C; run it on one host CPU (this
        # thread's affinity only, restored afterwards)
        host_cpus = os.sched_getaffinity(0)
        pin_cpu = min(host_cpus)
        os.sched_setaffinity(0, {pin_cpu})
        while t_cpu < args.cpu_seconds and n_calls < 100000:
            l = n_calls % n_distinct
            if l >= len(prepared):
                st = {k: [] for fm in FAMS for k in fm[4:6]}
                for s in range(L):
                    if mlp:
                        wts = synth.draw_mlp_adapter(w, l, s, int(ranks[s]))
                        pk = {}
                        for f, nm, xk, yk, ak, bk, projs in FAMS:
                            fin, _, widths, _ = fam_shape[f]
                            r = oracle.pack_family(fin, widths, R, w.dtype, int(ranks[s]), w.lora_alpha,
                                                   w.use_rslora, True, [wts[p] for p in projs])
                            pk[ak], pk[bk] = r["A"], r["B"]
                    else:
                        pk = oracle.pack_adapter(w.hidden, w.n_heads, w.n_kv_heads, w.head_dim, R, w.dtype,
                                                 int(ranks[s]), w.lora_alpha, w.use_rslora, True, "qkvo",
                                                 synth.draw_adapter(w, l, s, int(ranks[s])))
                    if args.bias:
                        bias = synth.draw_bias(w, l, s, tuple(p for fm in FAMS for p in fm[6]))
                        for f, nm, xk, yk, ak, bk, projs in FAMS:
                            pk["bias_" + nm] = oracle.pack_bias(list(fam_shape[f][2]), w.dtype,
                                                                [bias[p] for p in projs])
                            st.setdefault("bias_" + nm, [])
                    for k in st:
                        st[k].append(pk[k])
                acts_l = synth.draw_mlp_activations(w, l, T) if mlp else synth.draw_activations(w, l, T)
                prepared.append(({k: np.stack(v) for k, v in st.items()}, acts_l))
            st, acts = prepared[l]
            order_req = lora_req[n_calls % len(lora_req):] + lora_req[:n_calls % len(lora_req)]
            rows, left = {}, budget
            for i in order_req:
                n = int(lengths[i])
                rows[i] = np.arange(min(n, max(left, 0)))
                left -= len(rows[i])
            reqs = [i for i in order_req if len(rows[i])]
            t0 = time.perf_counter()
            for f, nm, xk, yk, ak, bk, _ in FAMS:
                oracle.reference_family(acts[xk], acts[yk], offsets, slots, st[ak], st[bk],
                                        list(fam_shape[f][2]), R, w.dtype, reqs, rows, st.get("bias_" + nm))
            t_cpu += time.perf_counter() - t0
            tokens_done += sum(len(rows[i]) for i in reqs)
            n_calls += 1
        os.sched_setaffinity(0, host_cpus)
        cpu = {"value": tokens_done / t_cpu, "unit": "LoRA tokens x layers / s", "cores": 1,
               "kind": "oracle", "cpu_model": cpu_identity(), "pinned_cpu": pin_cpu,
               "host_cpus_available": len(host_cpus),
               "sample": f"{tokens_done} LoRA-routed token rows through the {proj_desc} delta of one layer "
                         f"({n_calls} oracle passes over {len(prepared)} distinct layers of the same "
                         f"workload, at most {budget} rows per pass), fp64, one thread pinned to host "
                         f"CPU {pin_cpu}, {t_cpu:.1f} s"}
        log(f"phase 3: oracle {cpu['value']:.1f} tokens x layers/s")

    out = {
        "metric": "LoRA-delta tokens/s + achieved HBM GB/s (% of peak), Llama-8B QKV shape",
        "value": value,
        "unit": f"LoRA tokens x layers / s ({proj_desc} delta)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "host_routing_us_per_step": 1e6 * ctx["host_route_s"] / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded; adapters, activations and routing drawn per layer)",
        "config": {"workload": w.name, "hidden": w.hidden, "n_heads": w.n_heads,
                   "intermediate": w.intermediate if mlp else None,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "requests": int(len(slots)),
                   "tokens": T, "lora_tokens": end, "groups": G, "max_num_loras": L,
                   "max_lora_rank": R, "layers_per_step": n_layers, "path": args.path,
                   "api": args.api, "routing": "device" if args.device_routing else "host+device",
                   "token_routing": bool(args.token_routing),
                   "hip_graph": not args.no_graph, "lora_bias": bool(args.bias)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": dominant,
                     "algorithmic_bytes_per_launch": kbytes[dominant],
                     "avg_launch_us": avg_us[dominant]},
        "calls": {k: {"avg_us": avg_us[k], "bytes": kbytes[k], "flops": kflops[k],
                      "GBps": kbytes[k] / (avg_us[k] * 1e-6) / 1e9,
                      "frac": kbytes[k] / (avg_us[k] * 1e-6) / 1e9 / HBM_PEAK_GBS} for k in KINDS},
        "calls_per_timed_graph": ctx["graph_calls"],
        "prefill": prefill,
        "end_to_end_GBps": e2e_gbs,
        "stream_reference": stream_ref,
        "pack_ms_per_adapter_layer": 1e3 * ctx["t_pack"] / max(ctx["n_pack"], 1),
        "activation": activation,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
