"""GPU parity of the split-K delta for short groups: lora_sgmv_delta on AUTO
runs the one-kernel delta's shrink half with K split over workgroups into
fp32 slabs, then the expand kernel, when a batch has only short groups but
the one-kernel launch would be slow (a long K, or a wide output).  The MLP
decode batch takes it by default (test_gpu_mlp.py); here it is forced with
the splitk_short option onto the attention families and checked against the
oracle: the Llama-3-8B decode batch, a rank-32 decode batch on the stack's
adapters, ragged short groups with a LoRA bias, per-token routing with
padded strided buffers."""

import numpy as np
import pytest

import synth
import segmented_rank_gemv_amd as srg
from lora_case import (TOL, GpuLayer, compare, log, oracle_layer, pack_bias_stacks, pack_stacks)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def decode_case(name):
    if name == "decode":
        w = synth.get_workload("decode")
        lengths, slots = synth.draw_requests(w)
        ranks = synth.draw_ranks(w)
        layer = 0
    else:
        # the stack's rank-32 rsLoRA adapters on a batch of one-token requests
        w = synth.get_workload("stack")
        rng = np.random.default_rng(17)
        lengths = np.ones(176, np.int64)
        slots = np.where(rng.random(176) < 0.2, -1, rng.integers(0, w.max_num_loras, 176)).astype(np.int32)
        ranks = synth.draw_ranks(w)
        layer = 5
    stacks = pack_stacks(w, layer, ranks)
    acts = synth.draw_activations(w, layer, int(lengths.sum()))
    return w, lengths, slots, stacks, acts


@pytest.mark.parametrize("name", ["decode", "stack_decode"])
def test_forced_splitk_short_matches_oracle(name):
    w, lengths, slots, stacks, acts = decode_case(name)
    ref = oracle_layer(w, stacks, lengths, slots, acts)
    out = {}
    for mode in ("1", "0"):
        log(f"[splitk-short] workload={name} forced={mode} T={int(lengths.sum())}")
        gl = GpuLayer(w, stacks, lengths, slots, acts)
        gl.run(srg.PATH_AUTO, fused=True, options=srg.LoraOptions(splitk_short=int(mode)))
        ey, _ = compare(w, gl, ref, check_u=False)
        log(f"[splitk-short] workload={name} forced={mode} y_rel={ey:.3e}")
        assert ey <= TOL[w.dtype], (mode, ey)
        out[mode] = gl.y_arrival("y_qkv")
    # the two paths add the K partial sums in different orders: close, and
    # not required to be bit-identical
    assert np.allclose(out["1"], out["0"], rtol=2e-2, atol=2e-2)


@pytest.mark.parametrize("R", [16, 32])
def test_forced_splitk_short_ragged_with_bias(R):
    """Short groups of 1..32 tokens (ragged tiles of the 16-token table, an
    empty request, base requests in between) with a LoRA bias."""
    base = synth.get_workload("decode")
    w = synth.Workload(**{**base.__dict__, "hidden": 1024, "n_heads": 8, "n_kv_heads": 2, "head_dim": 128,
                          "max_lora_rank": R, "max_num_loras": 6})
    lengths = np.array([1, 15, 16, 17, 31, 32, 0, 3, 9, 24, 2], np.int64)
    slots = np.array([0, 1, 2, 3, 4, 5, 2, -1, 0, 1, -1], np.int32)
    stacks = pack_stacks(w, 0, np.full(w.max_num_loras, min(8, R), np.int32))
    bias = pack_bias_stacks(w, 0)
    acts = synth.draw_activations(w, 0, int(lengths.sum()))
    log(f"[splitk-short] ragged R={R} T={int(lengths.sum())}")
    gl = GpuLayer(w, stacks, lengths, slots, acts, pad_rows=5, pad_cols=16, bias=bias)
    gl.run(srg.PATH_AUTO, fused=True, options=srg.LoraOptions(splitk_short=1))
    ey, _ = compare(w, gl, oracle_layer(w, stacks, lengths, slots, acts, bias=bias), check_u=False)
    log(f"[splitk-short] ragged R={R} y_rel={ey:.3e}")
    assert ey <= TOL[w.dtype]
    # the padding rows past the batch and the columns past each row are untouched
    for key in ("y_qkv", "y_o"):
        full = gl.dev[key + "_full"].float().cpu().numpy()
        width = acts[key].shape[1]
        assert np.all(full[gl.T:, :width] == 7.0)
        assert np.all(full[:, width:] == 0.0)


def test_forced_splitk_short_per_token_routing():
    """Per-token routing (x gathered, y scattered through the sorted token
    indices) on the decode batch with its slots shuffled over the batch."""
    import test_gpu_token_routing as tr
    w, token_slot, stacks, acts = tr.token_case("decode", True)
    log(f"[splitk-short] per-token routing T={len(token_slot)}")
    ys, _ = tr.run_tokens(w, stacks, token_slot, acts, "auto", "delta", pad_rows=3, pad_cols=8,
                          options=srg.LoraOptions(splitk_short=1))
    ey = tr.check(w, stacks, token_slot, acts, ys, pad_rows=3, pad_cols=8)
    log(f"[splitk-short] per-token routing y_rel={ey:.3e}")
    assert ey <= TOL[w.dtype]

