"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Workloads (synthetic, seeded; shapes of the pages' attention blocks):
tiny (fp32), decode, prefill, mixed (bf16) at full size with every request
checked; the 32-layer stack at full size with every row of every layer.
Every path (auto, VALU, MFMA) runs where it applies.  Edge cases: empty and
base-only batches, the pages' base-only routing form, zero-length requests,
ragged segment lengths around the tile size, zero B, rows at and past `end`,
strided x/y, determinism and batch-composition invariance.
"""

import numpy as np
import pytest

import synth
import segmented_rank_gemv_amd as srg
from lora_case import (TOL, U_TOL, GpuLayer, compare, dims_of, log, oracle_layer, pack_stacks,
                       rel_err)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


PATHS = {"auto": srg.PATH_AUTO, "valu": srg.PATH_VALU, "mfma": srg.PATH_MFMA}
DELTA_PATHS = {**PATHS, "fused": srg.PATH_FUSED}
_CACHE = {}


def fused_applies(w) -> bool:
    """The one-kernel delta needs bf16 and a rank of 16 or 32 (every
    workload here has slice widths that are multiples of 32)."""
    return w.dtype == "bf16" and w.max_lora_rank in (16, 32)


def workload_case(name, layer=0):
    key = (name, layer)
    if key not in _CACHE:
        w = synth.get_workload(name)
        lengths, slots = synth.draw_requests(w)
        ranks = synth.draw_ranks(w)
        stacks = pack_stacks(w, layer, ranks)
        acts = synth.draw_activations(w, layer, int(lengths.sum()))
        ref = oracle_layer(w, stacks, lengths, slots, acts)
        _CACHE[key] = (w, lengths, slots, stacks, acts, ref)
    return _CACHE[key]


@pytest.mark.parametrize("api", ["split", "delta", "delta_reduce", "delta_nofold", "split_devroute"])
@pytest.mark.parametrize("path", list(DELTA_PATHS))
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "mixed"])
def test_full_workload_parity(name, path, api):
    """split: lora_sgmv_shrink + lora_sgmv_expand (u checked too); delta:
    lora_sgmv_delta (AUTO takes the one-kernel path on decode batches);
    delta_reduce: lora_sgmv_delta on the two-kernel path with its slabs folded
    by the reduce kernel before the expand (fold_slabs 1; by default no batch
    folds); delta_nofold: the same path with the expand reading every slab
    itself; split_devroute: split with the
    routing read from the device arrays only.  path fused: lora_sgmv_delta
    forced onto the one-kernel path."""
    w, lengths, slots, stacks, acts, ref = workload_case(name)
    if path == "mfma" and w.dtype != "bf16":
        pytest.skip("MFMA path is bf16 only")
    if path == "fused" and api != "delta":
        pytest.skip("the one-kernel path exists for lora_sgmv_delta only")
    if path == "fused" and not fused_applies(w):
        pytest.skip("one-kernel path needs bf16 and rank 16 or 32 (error path tested separately)")
    opts = None
    if api in ("delta_reduce", "delta_nofold"):
        opts = srg.LoraOptions(fused_max_tokens=0, fold_slabs=1 if api == "delta_reduce" else 0)
    log(f"[parity] workload={name} path={path} api={api} T={int(lengths.sum())}")
    gl = GpuLayer(w, stacks, lengths, slots, acts)
    gl.run(DELTA_PATHS[path], fused=api.startswith("delta"), routing="device" if api.endswith("devroute") else "host",
           options=opts)
    ey, eu = compare(w, gl, ref, check_u=api.startswith("split"))
    log(f"[parity] workload={name} path={path} api={api} y_rel={ey:.3e} u_rel={eu:.3e}")
    assert ey <= TOL[w.dtype]
    assert eu <= U_TOL[w.dtype]


def test_stack_every_row_every_layer(tmp_path):
    """All 32 layers of the stack workload at full size (rsLoRA rank 32, 4096
    tokens, the last 4 requests base), every row of every request of both
    families against the oracle: 3 630 LoRA rows x (6 144 + 4 096) outputs
    per layer, and every base row bit-identical.  Even layers run the split
    calls (u checked too), odd layers lora_sgmv_delta; every third layer reads
    the routing from the device arrays only.  The oracle runs in spawned
    worker processes on the CPU (stack_check.py), which regenerate each
    layer's inputs from its seeds, while this process runs the next layer on
    the GPU."""
    import multiprocessing as mp
    import os
    import stack_check

    w = synth.get_workload("stack")
    lengths, slots = synth.draw_requests(w)
    ranks = synth.draw_ranks(w)
    T = int(lengths.sum())
    nproc = max(1, min(16, len(os.sched_getaffinity(0))))
    log(f"[stack] {w.n_layers} layers, T={T}, oracle workers={nproc}")
    results = []
    with mp.get_context("spawn").Pool(nproc) as pool:
        pending = []
        for layer in range(w.n_layers):
            stacks = pack_stacks(w, layer, ranks, with_ref=False)
            acts = synth.draw_activations(w, layer, T)
            split = layer % 2 == 0
            gl = GpuLayer(w, stacks, lengths, slots, acts)
            gl.run(srg.PATH_AUTO, fused=not split, routing="device" if layer % 3 == 0 else "host")
            data = {"y_qkv": synth.bf16_bits(gl.y_arrival("y_qkv")), "y_o": synth.bf16_bits(gl.y_arrival("y_o"))}
            if split:
                data["u_qkv"] = gl.u_arrival(srg.FAMILY_QKV)
                data["u_o"] = gl.u_arrival(srg.FAMILY_O)
            path = str(tmp_path / f"layer{layer}.npz")
            np.savez(path, **data)
            del gl, data, acts
            pending.append(pool.apply_async(stack_check.check_layer, (("stack", layer, path),)))
            log(f"[stack] layer={layer} done on the GPU ({'split' if split else 'delta'})")
        for p in pending:
            r = p.get(timeout=900)
            log(f"[stack] layer={r['layer']} y_rel qkv={r['y_rel_qkv']:.3e} o={r['y_rel_o']:.3e}"
                f" u_rel qkv={r['u_rel_qkv']} o={r['u_rel_o']} rows={r['rows_qkv']}")
            results.append(r)
    assert len(results) == w.n_layers
    lora_rows = int(lengths[slots >= 0].sum())
    for r in results:
        assert r["base_rows_identical"], r
        assert r["rows_qkv"] == lora_rows and r["rows_o"] == lora_rows, r
        assert r["y_rel_qkv"] <= TOL[w.dtype] and r["y_rel_o"] <= TOL[w.dtype], r
        if r["layer"] % 2 == 0:
            assert r["u_rel_qkv"] <= U_TOL[w.dtype] and r["u_rel_o"] <= U_TOL[w.dtype], r
    log(f"[stack] worst y_rel={max(max(r['y_rel_qkv'], r['y_rel_o']) for r in results):.3e}")


# ----------------------------------------------------------------------------- edge cases
def small_bf16(L=4, R=16):
    base = synth.get_workload("decode")
    return synth.Workload(**{**base.__dict__, "name": "decode", "hidden": 512, "n_heads": 4,
                             "n_kv_heads": 2, "head_dim": 128, "max_lora_rank": R,
                             "max_num_loras": L})


def run_custom(w, lengths, slots, path, ranks=None, targets="qkvo", zero_B=False, pad_rows=0,
               pad_cols=0, layer=0):
    lengths = np.asarray(lengths, np.int64)
    slots = np.asarray(slots, np.int32)
    ranks = np.full(w.max_num_loras, min(8, w.max_lora_rank), np.int32) if ranks is None else ranks
    stacks = pack_stacks(w, layer, ranks, targets, zero_B)
    acts = synth.draw_activations(w, layer, int(lengths.sum()))
    gl = GpuLayer(w, stacks, lengths, slots, acts, pad_rows, pad_cols)
    gl.run(path)
    ref = oracle_layer(w, stacks, lengths, slots, acts)
    return gl, ref, acts


@pytest.mark.parametrize("routing", ["host", "device"])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("path", list(DELTA_PATHS))
def test_ragged_segments_around_tile_size(path, fused, routing):
    if path == "fused" and not fused:
        pytest.skip("the one-kernel path exists for lora_sgmv_delta only")
    w = small_bf16(L=8)
    lengths = np.array([1, 15, 16, 17, 63, 64, 65, 127, 129, 3, 0, 200], np.int64)
    slots = np.array([0, 1, 2, 3, 4, 5, 6, 7, 0, -1, 3, 1], np.int32)
    log(f"[ragged] path={path} fused={fused}")
    stacks = pack_stacks(w, 0, np.full(w.max_num_loras, 8, np.int32))
    acts = synth.draw_activations(w, 0, int(lengths.sum()))
    gl = GpuLayer(w, stacks, lengths, slots, acts)
    gl.run(DELTA_PATHS[path], fused=fused, routing=routing)
    ey, eu = compare(w, gl, oracle_layer(w, stacks, lengths, slots, acts), check_u=not fused)
    assert ey <= TOL["bf16"] and eu <= U_TOL["bf16"]


@pytest.mark.parametrize("R", [16, 32])
@pytest.mark.parametrize("path", ["fused", "auto"])
def test_one_kernel_delta_odd_widths_and_long_k(R, path):
    """One-kernel delta on shapes that exercise its tiling: K = 4640 (QKV) and
    4608 (O) give more K steps per wave than one batch and a K tail; slice
    widths 4608 / 1152 / 1152 and an o_proj width of 4640 give feature tiles
    of 128 and 32.  Groups of 1..33 tokens (balanced 16-token tiles), a base
    request and an empty one; AUTO takes the one-kernel path since no group
    is longer than 32 (except the 33-token one, which sends AUTO to the
    two-kernel path)."""
    base = synth.get_workload("decode")
    w = synth.Workload(**{**base.__dict__, "hidden": 4640, "n_heads": 16, "n_kv_heads": 4,
                          "head_dim": 288, "max_lora_rank": R, "max_num_loras": 6})
    lengths = np.array([1, 2, 16, 17, 31, 33, 5, 0, 9], np.int64)
    slots = np.array([0, 1, 2, 3, 4, 5, -1, 0, 1], np.int32)
    if path == "auto":
        lengths = lengths[lengths != 33]
        slots = slots[:len(lengths)]
    stacks = pack_stacks(w, 0, np.array([R, R // 2, 8, R, 8, R], np.int32))
    acts = synth.draw_activations(w, 0, int(lengths.sum()))
    log(f"[one-kernel] R={R} path={path}")
    gl = GpuLayer(w, stacks, lengths, slots, acts)
    gl.run(DELTA_PATHS[path], fused=True)
    ey, _ = compare(w, gl, oracle_layer(w, stacks, lengths, slots, acts), check_u=False)
    log(f"[one-kernel] R={R} path={path} y_rel={ey:.3e}")
    assert ey <= TOL["bf16"]


@pytest.mark.parametrize("R", [16, 32])
@pytest.mark.parametrize("hidden,heads,kv,hd", [(4096, 32, 8, 128), (2080, 16, 16, 130)])
def test_one_kernel_delta_x_through_lds(R, hidden, heads, kv, hd):
    """One-kernel delta with x staged through LDS (K <= 4096): K = 4096 gives
    every wave a full 256-element range; K = 2080 gives 160-element ranges
    (lanes past the range load a clamped piece that must not contribute) and
    32-feature tiles.  Groups of 1..32 tokens: tiles of 1..16 rows (rows past
    the tile load a clamped row that must not be stored)."""
    base = synth.get_workload("decode")
    w = synth.Workload(**{**base.__dict__, "hidden": hidden, "n_heads": heads, "n_kv_heads": kv,
                          "head_dim": hd, "max_lora_rank": R, "max_num_loras": 5})
    lengths = np.array([1, 7, 16, 17, 32, 3, 0, 2], np.int64)
    slots = np.array([0, 1, 2, 3, 4, -1, 2, 0], np.int32)
    stacks = pack_stacks(w, 0, np.array([R, 8, R // 2, R, 8], np.int32))
    acts = synth.draw_activations(w, 0, int(lengths.sum()))
    log(f"[x-lds] R={R} hidden={hidden}")
    gl = GpuLayer(w, stacks, lengths, slots, acts)
    gl.run(srg.PATH_FUSED, fused=True)
    ey, _ = compare(w, gl, oracle_layer(w, stacks, lengths, slots, acts), check_u=False)
    log(f"[x-lds] R={R} hidden={hidden} y_rel={ey:.3e}")
    assert ey <= TOL["bf16"]


@pytest.mark.parametrize("path", ["auto", "valu", "mfma"])
def test_largest_rank(path):
    """max_lora_rank 128 (the largest the kernels accept): the QKV shrink
    spans six 64-column groups, the expand runs on the VALU path (MFMA
    expand stops at rank 64) and the one-kernel path does not apply."""
    w = small_bf16(L=3, R=128)
    lengths = np.array([5, 70, 1, 33], np.int64)
    slots = np.array([2, 0, -1, 1], np.int32)
    if path == "mfma":
        # the forced MFMA path needs an MFMA expand: rank 128 is rejected up front
        stacks = pack_stacks(w, 0, np.array([128, 100, 7], np.int32))
        acts = synth.draw_activations(w, 0, int(lengths.sum()))
        gl = GpuLayer(w, stacks, lengths, slots, acts)
        with pytest.raises(srg.LoraError):
            srg.lora_sgmv_expand(gl.dims, srg.FAMILY_QKV, gl.u[srg.FAMILY_QKV], gl.st["B_qkv"],
                                 gl.routing["host"], gl.dev["y_qkv"], srg.PATH_MFMA)
        return
    gl, ref, _ = run_custom(w, lengths, slots, PATHS[path], ranks=np.array([128, 100, 7], np.int32))
    ey, eu = compare(w, gl, ref)
    log(f"[rank128] path={path} y_rel={ey:.3e} u_rel={eu:.3e}")
    assert ey <= TOL["bf16"] and eu <= U_TOL["bf16"]


def test_one_kernel_path_rejected_where_it_does_not_apply():
    """PATH_FUSED: an error (no launch) for fp32, for rank 64 and for the
    split calls; y stays as it was."""
    import torch
    cases = [synth.get_workload("tiny"), small_bf16(L=2, R=64)]
    for w in cases:
        lengths, slots = np.array([3, 2], np.int64), np.array([0, 1], np.int32)
        stacks = pack_stacks(w, 0, np.full(w.max_num_loras, 4, np.int32))
        acts = synth.draw_activations(w, 0, 5)
        gl = GpuLayer(w, stacks, lengths, slots, acts)
        y0 = gl.dev["y_qkv"].clone()
        with pytest.raises(srg.LoraError):
            srg.lora_sgmv_delta(gl.dims, srg.FAMILY_QKV, gl.dev["x_qkv"], gl.st["A_qkv"], gl.st["B_qkv"],
                                gl.routing["host"], gl.dev["y_qkv"], gl.ws[srg.FAMILY_QKV], srg.PATH_FUSED)
        torch.cuda.synchronize()
        assert torch.equal(gl.dev["y_qkv"], y0)
    w = small_bf16(L=2, R=16)
    stacks = pack_stacks(w, 0, np.full(2, 4, np.int32))
    gl = GpuLayer(w, stacks, np.array([3], np.int64), np.array([1], np.int32), synth.draw_activations(w, 0, 3))
    with pytest.raises(srg.LoraError):
        srg.lora_sgmv_shrink(gl.dims, srg.FAMILY_QKV, gl.dev["x_qkv"], gl.st["A_qkv"], gl.routing["host"],
                             gl.u[srg.FAMILY_QKV], gl.ws[srg.FAMILY_QKV], srg.PATH_FUSED)
    with pytest.raises(srg.LoraError):
        srg.lora_sgmv_expand(gl.dims, srg.FAMILY_QKV, gl.u[srg.FAMILY_QKV], gl.st["B_qkv"], gl.routing["host"],
                             gl.dev["y_qkv"], srg.PATH_FUSED)


@pytest.mark.parametrize("path", ["auto", "valu"])
def test_tiny_fp32_odd_shapes(path):
    w = synth.Workload(**{**synth.get_workload("tiny").__dict__, "hidden": 72, "n_heads": 3,
                          "n_kv_heads": 1, "head_dim": 24, "max_lora_rank": 8, "max_num_loras": 3})
    lengths = [2, 0, 70, 1, 9]
    slots = [2, 0, 1, -1, 2]
    gl, ref, _ = run_custom(w, lengths, slots, PATHS[path], ranks=np.array([3, 8, 5], np.int32))
    ey, eu = compare(w, gl, ref)
    assert ey <= TOL["f32"] and eu <= U_TOL["f32"]


def test_empty_and_base_only_batches_are_noops():
    w = small_bf16()
    for lengths, slots in (([], []), ([3, 4], [-1, -1])):
        gl, ref, acts = run_custom(w, lengths, slots, srg.PATH_AUTO)
        assert gl.end == 0 and gl.G == 0
        if len(lengths):
            assert np.array_equal(gl.y_arrival("y_qkv"), acts["y_qkv"])
            assert np.array_equal(gl.y_arrival("y_o"), acts["y_o"])


def test_pages_base_only_form_leaves_y_unchanged():
    """The base-only fallback routes every token to slot 0 holding an all-zero
    adapter; y must come back bit-identical."""
    w = small_bf16(L=2)
    lengths = np.array([5, 70], np.int64)
    stacks = pack_stacks(w, 0, np.full(2, 8, np.int32), targets="")
    acts = synth.draw_activations(w, 0, 75)
    gl = GpuLayer(w, stacks, lengths, np.array([0, 0], np.int32), acts)
    gl.run(srg.PATH_AUTO)
    assert gl.G == 1 and gl.end == 75
    assert np.array_equal(gl.y_arrival("y_qkv"), acts["y_qkv"])
    assert np.array_equal(gl.y_arrival("y_o"), acts["y_o"])


@pytest.mark.parametrize("path", list(PATHS))
def test_zero_B_gives_zero_delta(path):
    w = small_bf16()
    gl, ref, acts = run_custom(w, [3, 40, 90], [0, 1, 2], PATHS[path], zero_B=True)
    assert np.array_equal(gl.y_arrival("y_qkv"), acts["y_qkv"])
    assert np.array_equal(gl.y_arrival("y_o"), acts["y_o"])


def test_rows_past_end_untouched_and_strided_buffers():
    w = small_bf16()
    gl, ref, acts = run_custom(w, [7, 33, 2, 5], [1, 0, -1, 1], srg.PATH_AUTO, pad_rows=9, pad_cols=8)
    ey, _ = compare(w, gl, ref)
    assert ey <= TOL["bf16"]
    from lora_case import from_dev
    for key in ("y_qkv_full", "y_o_full"):
        full = from_dev(gl.dev[key])
        assert np.all(full[gl.T:] [:, :-8] == 7.0)   # padded rows past the batch
        assert np.all(full[:, -8:] == 0.0)            # padded columns


def test_missing_projection_slice_unchanged():
    w = small_bf16()
    gl, ref, acts = run_custom(w, [10, 80], [0, 1], srg.PATH_AUTO, targets="qv")
    y = gl.y_arrival("y_qkv")
    k = slice(w.nq, w.nq + w.nkv)
    assert np.array_equal(y[:, k], acts["y_qkv"][:, k])
    assert np.array_equal(gl.y_arrival("y_o"), acts["y_o"])
    ey, _ = compare(w, gl, ref)
    assert ey <= TOL["bf16"]


def test_padding_invariance_on_gpu():
    """rank-8 adapters in R=8 and R=64 stacks give the same result within tolerance."""
    res = []
    for R in (8, 64):
        w = small_bf16(L=2, R=R)
        gl, ref, acts = run_custom(w, [20, 70], [0, 1], srg.PATH_AUTO, ranks=np.array([8, 8], np.int32))
        res.append(gl.y_arrival("y_qkv"))
    assert rel_err(res[1], res[0]) <= TOL["bf16"]


def test_deterministic_and_batch_composition_invariant():
    w = small_bf16()
    lengths = np.array([30, 1, 90, 4], np.int64)
    slots = np.array([2, 0, 2, 1], np.int32)
    stacks = pack_stacks(w, 0, np.full(w.max_num_loras, 8, np.int32))
    acts = synth.draw_activations(w, 0, int(lengths.sum()))
    a = GpuLayer(w, stacks, lengths, slots, acts)
    a.run(srg.PATH_AUTO)
    b = GpuLayer(w, stacks, lengths, slots, acts)
    b.run(srg.PATH_AUTO)
    assert np.array_equal(a.y_arrival("y_qkv"), b.y_arrival("y_qkv"))
    assert np.array_equal(a.y_arrival("y_o"), b.y_arrival("y_o"))
    # request 2 (tokens 31..120) alone, with the same rows, vs inside the batch
    alone_acts = {k: v[31:121] for k, v in acts.items()}
    c = GpuLayer(w, stacks, np.array([90]), np.array([2], np.int32), alone_acts)
    c.run(srg.PATH_AUTO)
    for key in ("y_qkv", "y_o"):
        assert rel_err(c.y_arrival(key), a.y_arrival(key)[31:121]) <= TOL["bf16"]


def test_host_side_argument_errors_launch_nothing():
    w = small_bf16()
    d = dims_of(w)
    x = torch.zeros((4, w.hidden), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((w.max_num_loras, 3 * w.max_lora_rank, w.hidden), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(1, dtype=torch.int32, device="cuda")
    offs = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    rt = srg.LoraRouting(ids, offs, 1, 4)
    u = torch.zeros((4, 3 * w.max_lora_rank), dtype=torch.float32, device="cuda")
    # misaligned x (one element in)
    with pytest.raises(srg.LoraError) as e:
        srg.lora_sgmv_shrink(d, srg.FAMILY_QKV, x.view(-1)[1:1 + 3 * w.hidden].view(3, w.hidden), A, rt, u)
    assert e.value.code == 1
    # workspace too small for a split-K launch
    with pytest.raises(srg.LoraError) as e:
        srg.lora_sgmv_shrink(d, srg.FAMILY_QKV, x, A, rt, u, torch.zeros(4, dtype=torch.int32, device="cuda"))
    assert e.value.code in (1, 4)
    # more groups than slots
    with pytest.raises(srg.LoraError) as e:
        srg.lora_sgmv_shrink(d, srg.FAMILY_QKV, x, A, srg.LoraRouting(ids, offs, w.max_num_loras + 1, 4), u)
    assert e.value.code == 1
    # host routing copies that disagree with end, or carry a bad slot id
    with pytest.raises(srg.LoraError) as e:
        srg.lora_sgmv_shrink(d, srg.FAMILY_QKV, x, A, srg.LoraRouting(ids, offs, 1, 4, np.array([0]),
                                                                      np.array([0, 3])), u)
    assert e.value.code == 1
    with pytest.raises(srg.LoraError) as e:
        srg.lora_sgmv_shrink(d, srg.FAMILY_QKV, x, A, srg.LoraRouting(ids, offs, 1, 4, np.array([w.max_num_loras]),
                                                                      np.array([0, 4])), u)
    assert e.value.code == 3
    # MFMA forced on fp32
    d32 = srg.LoraDims(**{**d.__dict__, "dtype": "f32"})
    with pytest.raises(srg.LoraError) as e:
        srg.lora_sgmv_expand(d32, srg.FAMILY_O, u, A, rt, x, srg.PATH_MFMA)
    assert e.value.code == 1
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["decode", "stack_decode"])
def test_fused_launch_shapes_bit_identical(name):
    """The one-kernel delta's launch choices do not change its arithmetic:
    every feature tile width (128, 256 or 512 features per workgroup, or the
    launcher's own pick) and the wave K-range rotation on or off give the same
    bits, and each of them matches the oracle.  The partial sums over the K
    ranges are added in K-range order whatever wave computed them, and each
    output feature's expand is the same sum whatever its tile.  stack_decode:
    the rank-32 stack adapters on a decode-shaped batch (one token per request)."""
    if name == "decode":
        w, lengths, slots, stacks, acts, ref = workload_case("decode")
    else:
        w = synth.get_workload("stack")
        rng = np.random.default_rng(11)
        lengths = np.ones(160, np.int64)
        slots = np.where(rng.random(160) < 0.2, -1, rng.integers(0, w.max_num_loras, 160)).astype(np.int32)
        stacks = pack_stacks(w, 3, synth.draw_ranks(w))
        acts = synth.draw_activations(w, 3, int(lengths.sum()))
        ref = oracle_layer(w, stacks, lengths, slots, acts)
    outs = {}
    for feat in ("", "512", "256", "128"):
        for krot in ("1", "0"):
            opts = srg.LoraOptions(fused_feature_tile=int(feat or 0), fused_k_rotation=int(krot))
            log(f"[fused-shapes] workload={name} feat={feat or 'auto'} krot={krot}")
            gl = GpuLayer(w, stacks, lengths, slots, acts)
            gl.run(srg.PATH_FUSED, fused=True, options=opts)
            ey, _ = compare(w, gl, ref, check_u=False)
            assert ey <= TOL[w.dtype], (feat, krot, ey)
            outs[(feat, krot)] = (gl.y_arrival("y_qkv"), gl.y_arrival("y_o"))
    first = outs[("", "1")]
    for key, (yq, yo) in outs.items():
        assert np.array_equal(yq.view(np.uint32), first[0].view(np.uint32)), key
        assert np.array_equal(yo.view(np.uint32), first[1].view(np.uint32)), key


@pytest.mark.parametrize("path", ["auto", "fused"])
def test_one_kernel_delta_takes_a_null_workspace(path):
    """The one-kernel path touches no workspace, so lora_sgmv_delta accepts
    NULL there: the decode batch gives the same bits as with a workspace."""
    w, lengths, slots, stacks, acts, ref = workload_case("decode")
    a = GpuLayer(w, stacks, lengths, slots, acts)
    a.run(DELTA_PATHS[path], fused=True)
    b = GpuLayer(w, stacks, lengths, slots, acts)
    b.ws = {k: None for k in b.ws}
    b.run(DELTA_PATHS[path], fused=True)
    ey, _ = compare(w, b, ref, check_u=False)
    assert ey <= TOL[w.dtype]
    for key in ("y_qkv", "y_o"):
        assert np.array_equal(a.y_arrival(key).view(np.uint32), b.y_arrival(key).view(np.uint32))
