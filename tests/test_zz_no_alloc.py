"""lora_sgmv_delta_noalloc, the variant of lora_sgmv_delta for callers that
cannot allocate device memory: its partial sums go to the library's own
device scratch array instead of a caller workspace.  Checked against
lora_sgmv_delta with a caller workspace (the same kernels: the same bits) on
two calls in a row, the second with a smaller batch, on every kind of
launch that uses scratch (the two-kernel path's K-split partial sums, and
the split-K form of the one-kernel path) and on one that uses none; the
smaller batch also against the oracle.  The capacity limit is checked on
the host, before any launch."""

import ctypes

import numpy as np
import pytest

import synth
import segmented_rank_gemv_amd as srg
from segmented_rank_gemv_amd import _lib
from lora_case import TOL, GpuLayer, compare, log, oracle_layer, pack_stacks


def _case(name, keep=None, layer=0):
    w = synth.get_workload(name)
    lengths, slots = synth.draw_requests(w)
    if keep is not None:
        lengths, slots = lengths[:keep], slots[:keep]
    stacks = pack_stacks(w, layer, synth.draw_ranks(w))
    acts = synth.draw_activations(w, layer, int(lengths.sum()))
    return w, lengths, slots, stacks, acts


def _same_bits(a: GpuLayer, b: GpuLayer):
    for key in ("y_qkv", "y_o"):
        ya, yb = a.y_arrival(key), b.y_arrival(key)
        assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32)), key


def _check_pair(name, keep, path, options, with_oracle):
    w, lengths, slots, stacks, acts = _case(name, keep)
    log(f"[noalloc] workload={name} requests={len(lengths)} T={int(lengths.sum())} path={path} options={options}")
    ref = GpuLayer(w, stacks, lengths, slots, acts)
    ref.run(path, fused=True, options=options)
    got = GpuLayer(w, stacks, lengths, slots, acts)
    got.run(path, fused=True, options=options, noalloc=True)
    _same_bits(ref, got)
    if with_oracle:
        ey, _ = compare(w, got, oracle_layer(w, stacks, lengths, slots, acts), check_u=False)
        log(f"[noalloc] workload={name} y_rel={ey:.3e}")
        assert ey <= TOL[w.dtype]


@pytest.mark.gpu
@pytest.mark.parametrize("first,second,path,options", [
    # prefill: AUTO's one-kernel delta for long groups (no scratch)
    (("prefill", None), ("prefill", 5), srg.PATH_AUTO, None),
    # two-kernel path: the shrink's K-split partial sums live in the scratch
    (("stack", None), ("stack", 8), srg.PATH_AUTO, None),
    (("mixed", None), ("mixed", 60), srg.PATH_MFMA, None),
    # one-kernel path in its split-K form (partial sums in the scratch)
    (("decode", None), ("decode", 100), srg.PATH_AUTO, srg.LoraOptions(splitk_short=1)),
    # one-kernel path proper: no scratch at all
    (("decode", None), ("decode", 70), srg.PATH_FUSED, None),
])
def test_noalloc_matches_delta_on_two_calls(first, second, path, options):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert srg.lora_sgmv_noalloc_scratch_bytes() == 64 << 20
    _check_pair(first[0], first[1], path, options, with_oracle=False)
    _check_pair(second[0], second[1], path, options, with_oracle=True)


def test_noalloc_capacity_checked_before_launch():
    """A batch whose partial sums exceed the scratch (mixed-batch dims,
    rank 64: 100 000 LoRA tokens x 192 fp32 columns = 76.8 MB > 64 MiB) is
    refused with LORA_ERR_CAPACITY before anything is launched; the device
    pointers are fake and never dereferenced (no GPU needed)."""
    lib = _lib._load()
    fake = 0x7F0000000000
    d = srg.LoraDims(5120, 40, 8, 128, 64, 32, "bf16").c()
    ids = np.array([3], np.int32)
    offs = np.array([0, 100000], np.int32)
    r = _lib._LoraRouting()
    r.lora_ids, r.grouped_offsets, r.num_groups, r.end = fake, fake, 1, 100000
    r.host_lora_ids, r.host_grouped_offsets = ids.ctypes.data, offs.ctypes.data
    assert srg.lora_sgmv_workspace_bytes(srg.LoraDims(5120, 40, 8, 128, 64, 32, "bf16"), srg.FAMILY_QKV,
                                         100000) > 64 << 20
    st = lib.lora_sgmv_delta_noalloc(ctypes.byref(d), srg.FAMILY_QKV, fake, 5120, fake, fake, None,
                                     ctypes.byref(r), fake, 7168, srg.PATH_AUTO, None, None)
    assert st == 4
