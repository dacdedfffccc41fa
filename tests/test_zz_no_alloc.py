"""kda_chunk_forward_noalloc (the forward with the library's fixed device
scratch as its workspace) against kda_chunk_forward with a caller-allocated
workspace: two calls in a row, the second on a smaller input (the scratch
then holds the first call's data), then the fp32 path and 300 packed
sequences.  Both entry
points take the same cut into segments on these shapes (the best cut fits
the scratch), so their results are bit-identical."""
import pytest
import torch

import gated_delta_rule_105_amd as kda
import synth
from gpu_util import note

pytestmark = pytest.mark.gpu


def _compare(name, inp):
    args = (inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    kw = dict(h0=inp["h0"], cu_seqlens=inp["cu_seqlens"])
    note(f"chunk_forward_noalloc {name}")
    o_ref, ht_ref = kda.chunk_forward(*args, **kw)
    o = torch.full_like(o_ref, float("nan"))
    ht = torch.full_like(ht_ref, float("nan"))
    kda.chunk_forward_noalloc(*args, o=o, ht=ht, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), name
    assert torch.equal(ht, ht_ref), name


def test_noalloc_matches_forward_two_calls():
    big = synth.prefill_inputs(1, 4096, 16, 128, 128, "bf16", wid=1, h0=True, device="cuda")
    _compare("bf16 B1 T4096 H16 d128 (48 MiB of segment records)", big)
    del big
    small = synth.prefill_inputs(1, 0, 4, 128, 128, "bf16", wid=220, h0=True, lengths=[300, 1, 0, 1000, 64],
                                 device="cuda")
    _compare("bf16 packed [300, 1, 0, 1000, 64] H4 d128", small)
    f32 = synth.prefill_inputs(2, 200, 3, 64, 64, "f32", wid=221, h0=True, device="cuda")
    _compare("f32 B2 T200 H3 d64", f32)
    many = synth.prefill_inputs(1, 0, 2, 128, 128, "bf16", wid=222, h0=True,
                                lengths=synth.packed_lengths(222, 300, 0, 200), device="cuda")
    _compare("bf16 300 packed sequences H2 d128", many)
