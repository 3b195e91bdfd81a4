"""GPU parity with a LoRA bias per slot: y = y_in + B[slot] (A[slot] x) +
bias[slot] for LoRA-routed rows, y_in for base rows, against the oracle.

Covers every expand variant the bias is added in: the VALU expand (fp32 and
bf16), the MFMA expand for R = 16 (B fragments from memory), R = 32 and 64
(B staged in LDS), R = 48 (register-resident B), the one-kernel decode delta
(R = 16 and 32), each through lora_sgmv_expand and lora_sgmv_delta, on the
full-size workloads and on ragged segments around the tile size; untargeted
slices carry no bias; a zero B leaves exactly the bias."""

import numpy as np
import pytest

import oracle
import synth
import segmented_rank_gemv_amd as srg
from lora_case import TOL, GpuLayer, compare, from_dev, log, oracle_layer, pack_bias_stacks, pack_stacks

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PATHS = {"auto": srg.PATH_AUTO, "valu": srg.PATH_VALU, "mfma": srg.PATH_MFMA, "fused": srg.PATH_FUSED}
_CACHE = {}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def fused_applies(w) -> bool:
    return w.dtype == "bf16" and w.max_lora_rank in (16, 32)


def bias_case(name):
    if name not in _CACHE:
        w = synth.get_workload(name)
        lengths, slots = synth.draw_requests(w)
        ranks = synth.draw_ranks(w)
        stacks = pack_stacks(w, 0, ranks)
        bias = pack_bias_stacks(w, 0)
        acts = synth.draw_activations(w, 0, int(lengths.sum()))
        ref = oracle_layer(w, stacks, lengths, slots, acts, bias=bias)
        _CACHE[name] = (w, lengths, slots, stacks, bias, acts, ref)
    return _CACHE[name]


@pytest.mark.parametrize("api", ["split", "delta"])
@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "mixed"])
def test_bias_full_workload_parity(name, path, api):
    w, lengths, slots, stacks, bias, acts, ref = bias_case(name)
    if path == "mfma" and w.dtype != "bf16":
        pytest.skip("MFMA path is bf16 only")
    if path == "fused" and (api != "delta" or not fused_applies(w)):
        pytest.skip("the one-kernel path is lora_sgmv_delta's, for bf16 and rank 16 or 32")
    log(f"[bias] workload={name} path={path} api={api} T={int(lengths.sum())}")
    gl = GpuLayer(w, stacks, lengths, slots, acts, bias=bias)
    gl.run(PATHS[path], fused=api == "delta")
    ey, _ = compare(w, gl, ref, check_u=False)
    log(f"[bias] workload={name} path={path} api={api} y_rel={ey:.3e}")
    assert ey <= TOL[w.dtype]


def small_bf16(R, L=8):
    base = synth.get_workload("decode")
    return synth.Workload(**{**base.__dict__, "hidden": 512, "n_heads": 4, "n_kv_heads": 2,
                             "head_dim": 128, "max_lora_rank": R, "max_num_loras": L})


@pytest.mark.parametrize("api", ["split", "delta"])
@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("R", [8, 16, 32, 48, 64])
def test_bias_ragged_every_rank(R, path, api):
    """Segments around the tile size, a base request and an empty one; the
    adapters target q and o only, so the k and v slices carry no bias."""
    w = small_bf16(R)
    if path == "mfma" and R % 16:
        pytest.skip("the MFMA path needs a rank that is a multiple of 16 (rejected otherwise)")
    if path == "fused" and (api != "delta" or not fused_applies(w)):
        pytest.skip("the one-kernel path is lora_sgmv_delta's, for bf16 and rank 16 or 32")
    if path == "fused":
        lengths = np.array([1, 15, 16, 17, 32, 3, 0, 20], np.int64)
        slots = np.array([0, 1, 2, 3, 4, -1, 5, 7], np.int32)
    else:
        lengths = np.array([1, 15, 16, 17, 63, 64, 65, 127, 129, 3, 0, 200], np.int64)
        slots = np.array([0, 1, 2, 3, 4, 5, 6, 7, 0, -1, 3, 1], np.int32)
    ranks = np.array([min(R, r) for r in (8, 8, 4, 8, 8, 2, 8, 8)], np.int32)
    stacks = pack_stacks(w, 0, ranks, targets="qo")
    bias = pack_bias_stacks(w, 0, targets="qo")
    acts = synth.draw_activations(w, 0, int(lengths.sum()))
    log(f"[bias-ragged] R={R} path={path} api={api}")
    gl = GpuLayer(w, stacks, lengths, slots, acts, bias=bias)
    gl.run(PATHS[path], fused=api == "delta")
    ref = oracle_layer(w, stacks, lengths, slots, acts, bias=bias)
    ey, _ = compare(w, gl, ref, check_u=False)
    log(f"[bias-ragged] R={R} path={path} api={api} y_rel={ey:.3e}")
    assert ey <= TOL[w.dtype]
    kv = bias["ref"]["bias_qkv"][:, w.nq:]
    assert not kv.any()


@pytest.mark.parametrize("path", ["valu", "mfma", "fused"])
def test_bias_with_zero_B_adds_exactly_the_bias(path):
    """B = 0: each LoRA row becomes round(y_in + bias) (fp32 sum of two bf16
    values, rounded once), base rows stay y_in."""
    w = small_bf16(16)
    lengths = np.array([5, 3, 17, 1], np.int64)
    slots = np.array([2, -1, 0, 2], np.int32)
    stacks = pack_stacks(w, 0, np.full(w.max_num_loras, 8, np.int32), zero_B=True)
    bias = pack_bias_stacks(w, 0)
    acts = synth.draw_activations(w, 0, int(lengths.sum()))
    gl = GpuLayer(w, stacks, lengths, slots, acts, bias=bias)
    gl.run(PATHS[path], fused=True)
    offs = gl.offs
    for key, bk in (("y_qkv", "bias_qkv"), ("y_o", "bias_o")):
        got = gl.y_arrival(key)
        b = oracle.stack_to_f64(bias["ref"][bk], w.dtype).astype(np.float32)
        for i in range(len(lengths)):
            rows = slice(int(offs[i]), int(offs[i + 1]))
            yin = acts[key][rows]
            want = yin if slots[i] < 0 else (yin + b[slots[i]][None, :]).astype(np.float32)
            if slots[i] >= 0:
                want = from_dev(torch.from_numpy(want).to(torch.bfloat16))
            assert np.array_equal(got[rows], want), (path, key, i)
