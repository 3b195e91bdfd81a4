"""GPU parity of the one-kernel delta for long groups: lora_sgmv_delta's AUTO
path on prefill-sized batches (the batch fills the chip without splitting
K), or any batch with the long_delta option.  Each workgroup computes the
shrink and the expand of a piece of at most 64 tokens; x and y move as
whole lines through per-wave LDS regions.  Checked against the oracle on
ragged groups (pieces of 1..64 tokens, empty and base requests), every rank
it takes (16, 32, 64), a K whose last wave range ends mid-chunk, an output
width that leaves the last wave a short run, LoRA bias, padded and strided
buffers, per-token routing and the MLP families; and AUTO on the prefill
workload is shown to take it."""

import numpy as np
import pytest

import synth
import segmented_rank_gemv_amd as srg
from lora_case import (TOL, GpuLayer, compare, log, oracle_layer, pack_bias_stacks, pack_stacks)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LONG = srg.LoraOptions(long_delta=1)
NO_LONG = srg.LoraOptions(long_delta=0)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dims(hidden, heads, kv, hd, R, L):
    base = synth.get_workload("decode")
    return synth.Workload(**{**base.__dict__, "hidden": hidden, "n_heads": heads, "n_kv_heads": kv,
                             "head_dim": hd, "max_lora_rank": R, "max_num_loras": L})


def run_case(w, lengths, slots, ranks, options, bias=False, pad_rows=0, pad_cols=0, layer=0):
    lengths = np.asarray(lengths, np.int64)
    slots = np.asarray(slots, np.int32)
    stacks = pack_stacks(w, layer, np.asarray(ranks, np.int32))
    bs = pack_bias_stacks(w, layer) if bias else None
    acts = synth.draw_activations(w, layer, int(lengths.sum()))
    gl = GpuLayer(w, stacks, lengths, slots, acts, pad_rows=pad_rows, pad_cols=pad_cols, bias=bs)
    gl.run(srg.PATH_AUTO, fused=True, options=options)
    ey, _ = compare(w, gl, oracle_layer(w, stacks, lengths, slots, acts, bias=bs), check_u=False)
    if pad_rows or pad_cols:
        for key in ("y_qkv", "y_o"):
            full = gl.dev[key + "_full"].float().cpu().numpy()
            width = acts[key].shape[1]
            assert np.all(full[gl.T:, :width] == 7.0), key
            assert np.all(full[:, width:] == 0.0), key
    return ey, gl


RAGGED = (np.array([1, 15, 16, 17, 63, 64, 65, 127, 129, 3, 0, 200, 49], np.int64),
          np.array([0, 1, 2, 3, 4, 5, 0, 1, 2, -1, 3, 1, -1], np.int32))


@pytest.mark.parametrize("R", [16, 32, 64])
@pytest.mark.parametrize("bias", [False, True])
def test_long_delta_ragged(R, bias):
    """Ragged groups around the 64-token piece, an empty request, base
    requests; padded rows and columns stay untouched.  QKV takes the long
    delta at rank 16 (u has 48 columns) and falls back to the two-kernel
    path above; o_proj takes it at every rank."""
    w = dims(512, 4, 2, 128, R, 6)
    lengths, slots = RAGGED
    log(f"[long] ragged R={R} bias={bias}")
    ey, _ = run_case(w, lengths, slots, [R, R // 2, 8, R, 8, R], LONG, bias=bias, pad_rows=3, pad_cols=64)
    log(f"[long] ragged R={R} bias={bias} y_rel={ey:.3e}")
    assert ey <= TOL["bf16"]


def test_long_delta_k_tail_and_short_last_wave():
    """K = 4672 gives 608-element wave ranges, the last one ending halfway
    through a 64-element chunk; an o_proj width of 4672 gives 640-feature
    runs per wave and a 192-feature run for the last wave."""
    w = dims(4672, 8, 2, 128, 16, 4)
    lengths = np.array([300, 64, 1, 129, 0, 77], np.int64)
    slots = np.array([0, 1, 2, 3, 1, -1], np.int32)
    ey, _ = run_case(w, lengths, slots, [16, 8, 16, 12], LONG)
    log(f"[long] K tail y_rel={ey:.3e}")
    assert ey <= TOL["bf16"]


def test_prefill_auto_takes_the_long_delta():
    """On the prefill workload AUTO without a workspace takes the long delta
    (only the one-kernel paths accept that); with one it takes the two-kernel
    path for QKV (u of 48 columns) and the long delta for O (16).  Every
    result is bit-identical to the forced long delta and to the forced
    two-kernel path (same K order and reduction tree in the shrink, same
    operand layout in the expand)."""
    w = synth.get_workload("prefill")
    lengths, slots = synth.draw_requests(w)
    ranks = synth.draw_ranks(w)
    stacks = pack_stacks(w, 1, ranks)
    acts = synth.draw_activations(w, 1, int(lengths.sum()))
    ref = oracle_layer(w, stacks, lengths, slots, acts)
    ys = {}
    for name, opts, ws in (("auto", None, False), ("auto-ws", None, True), ("long", LONG, False),
                           ("two-kernel", NO_LONG, True)):
        gl = GpuLayer(w, stacks, lengths, slots, acts)
        if not ws:
            gl.ws = {k: None for k in gl.ws}
        gl.run(srg.PATH_AUTO, fused=True, options=opts)
        ey, _ = compare(w, gl, ref, check_u=False)
        log(f"[long] prefill {name} y_rel={ey:.3e}")
        assert ey <= TOL["bf16"], name
        ys[name] = (gl.y_arrival("y_qkv").view(np.uint32), gl.y_arrival("y_o").view(np.uint32))
    for name in ("auto-ws", "long", "two-kernel"):
        assert np.array_equal(ys["auto"][0], ys[name][0]) and np.array_equal(ys["auto"][1], ys[name][1]), name
    gl = GpuLayer(w, stacks, lengths, slots, acts)
    gl.ws = {k: None for k in gl.ws}
    with pytest.raises(ValueError):
        gl.run(srg.PATH_AUTO, fused=True, options=NO_LONG)


def test_long_delta_per_token_routing():
    """Per-token routing (rows gathered and scattered through the sorted
    token indices) on the prefill batch with its tokens shuffled, padded and
    strided buffers."""
    import test_gpu_token_routing as tr
    w, token_slot, stacks, acts = tr.token_case("prefill", True)
    log(f"[long] per-token routing T={len(token_slot)}")
    ys, _ = tr.run_tokens(w, stacks, token_slot, acts, "auto", "delta", pad_rows=5, pad_cols=64, options=LONG)
    ey = tr.check(w, stacks, token_slot, acts, ys, pad_rows=5, pad_cols=64)
    log(f"[long] per-token routing y_rel={ey:.3e}")
    assert ey <= TOL["bf16"]


@pytest.mark.parametrize("fam", [srg.FAMILY_GATE_UP, srg.FAMILY_DOWN])
def test_long_delta_mlp_families(fam):
    """The MLP families (gate_up: two 14 336-wide slices, u of 32 columns;
    down: K = 14 336) on a prefill-shaped batch, with a LoRA bias."""
    import test_gpu_mlp as mlp
    w = synth.get_workload("mlp")
    lengths = np.array([200, 64, 1, 333, 0, 90, 17], np.int64)
    slots = np.array([0, 1, 2, 3, 4, -1, 5], np.int32)
    ranks = np.array([16, 8, 16, 12, 16, 8, 16, 8], np.int32)
    ey = mlp.run_family(w, fam, lengths, slots, ranks, "auto", True, with_bias=True, options=LONG)
    log(f"[long] mlp family={fam} y_rel={ey:.3e}")
    assert ey <= TOL["bf16"]
