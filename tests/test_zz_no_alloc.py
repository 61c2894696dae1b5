"""ep_decode_batch_noalloc: the allocation-free entry point against ep_decode_batch.

The entry point decodes with the library's static device scratch instead of a
caller workspace.  Two calls in a row (the second with a smaller batch, so it
runs over what the first left in the scratch) must give outputs and tile
statuses identical, byte for byte, to ep_decode_batch on its own workspace; a
batch whose workspace exceeds the scratch is rejected before any GPU work.
"""
import numpy as np
import pytest
import torch

import synthgen

pytestmark = pytest.mark.gpu

ep = pytest.importorskip("dit_weight_compression_amd")
from dit_weight_compression_amd import encoder  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.lib()


def _packed(shapes):
    out = []
    for i, (r, c, bpp, route, V) in enumerate(shapes):
        W = synthgen.student_t_weights(r, c, 900 + i, bf16=True).numpy()
        ct = encoder.encode(W, bpp, V=V, route=route, threads=8)
        out.append(ep.PackedTensor.from_arrays(ct, device="cuda"))
    return out


def _statuses(packed):
    return [torch.full((max(p.T, 1),), -7, dtype=torch.int32, device="cuda") for p in packed]


def _compare(packed, kinds):
    ref, ref_st = ep.decode_batch(packed, kinds, with_status=True)
    outs = ep.alloc_outputs(packed, kinds, "cuda")
    for o in outs:
        o.view(torch.uint8).fill_(0xA5)                 # nothing left over from the reference
    sts = _statuses(packed)
    ep.decode_batch_noalloc(packed, kinds, outs, sts)
    torch.cuda.synchronize()
    for i, (p, a, b, sa, sb) in enumerate(zip(packed, ref, outs, ref_st, sts)):
        assert torch.equal(sa[: p.T], sb[: p.T]), f"tensor {i}: tile statuses differ"
        assert bool((sb[: p.T] == 0).all()), f"tensor {i}: tile status {sb[: p.T].unique().tolist()}"
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"tensor {i} ({p.rows}x{p.cols}): outputs differ"


def test_two_calls_in_a_row_match_the_workspace_entry_point():
    # first call: several layouts, routes and output kinds, ragged last tiles
    first = _packed([(1024, 1536, 4.0, "direct", 0), (768, 1024, 8.0, "direct", 0),
                     (1000, 1032, 3.0, "direct", 455), (512, 2048, 5.0, "fp8", 0),
                     (640, 768, 2.0, "int8", 0), (256, 512, 6.0, "direct", 64)])
    kinds1 = ["bf16", "bf16", "fp32", "fp8", "int8", "fp16"]
    assert ep.workspace_size(first) <= ep.NOALLOC_SCRATCH_BYTES
    _compare(first, kinds1)
    # second call: a smaller batch over the first call's leftovers in the scratch
    second = _packed([(200, 520, 4.0, "direct", 33), (96, 256, 7.0, "direct", 0)])
    assert ep.workspace_size(second) < ep.workspace_size(first)
    _compare(second, ["bf16", "lattice2x"])


def test_batch_beyond_the_scratch_is_rejected_before_any_work():
    one = _packed([(512, 1024, 4.0, "direct", 32)])[0]
    base = ep.workspace_size([one])
    per = ep.workspace_size([one, one]) - base          # what each further tensor adds
    n = (ep.NOALLOC_SCRATCH_BYTES - base) // per + 3
    packed = [one] * n
    assert ep.workspace_size(packed) > ep.NOALLOC_SCRATCH_BYTES
    outs = [torch.zeros((one.rows, one.cols), dtype=torch.int16, device="cuda") for _ in range(n)]
    with pytest.raises(ep.EpError) as e:
        ep.decode_batch_noalloc(packed, "bf16", outs)
    assert e.value.status == ep.EP_ERR_WORKSPACE
    assert "static" in str(e.value) and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert all(int(o.abs().sum()) == 0 for o in outs[:4])     # nothing was written
    # the entry point still works after the rejection
    _compare([one], ["bf16"])
