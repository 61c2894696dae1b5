"""A captured ep_decode_batch_noalloc call replays byte for byte.

A batch of at most 6 tensors passes its descriptors to the table build as
kernel arguments and decodes in the library's static scratch, so the call
records only kernel launches.  The graph is replayed several times; between
replays the outputs and statuses are overwritten and an eager call decodes a
different batch through the same scratch, so every replay has to rebuild the
tables, the schedule and the flags from its own arguments.  Every replay must
equal the eager decode of the same batch, tile statuses included.
"""
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


def _packed(shapes, seed0):
    out = []
    for i, (r, c, bpp, route, V) in enumerate(shapes):
        W = synthgen.student_t_weights(r, c, seed0 + i, bf16=True).numpy()
        ct = encoder.encode(W, bpp, V=V, route=route, threads=8)
        out.append(ep.PackedTensor.from_arrays(ct, device="cuda"))
    return out


def _statuses(packed, fill):
    return [torch.full((max(p.T, 1),), fill, dtype=torch.int32, device="cuda") for p in packed]


def test_captured_noalloc_call_replays_byte_for_byte():
    # packed (fp16 byte entries), hybrid b = 11 and b = 12, FP8 and INT8 routes, a ragged tile size
    packed = _packed([(1024, 1536, 4.0, "direct", 0), (512, 1024, 6.2, "direct", 0),
                      (768, 1024, 8.0, "direct", 0), (512, 2048, 5.0, "fp8", 0),
                      (640, 768, 2.0, "int8", 0), (1000, 1032, 3.0, "direct", 455)], 1300)
    kinds = ["bf16", "bf16", "fp16", "fp8", "int8", "fp32"]
    assert len(packed) <= 6 and ep.workspace_size(packed) <= ep.NOALLOC_SCRATCH_BYTES
    ref, ref_st = ep.decode_batch(packed, kinds, with_status=True)
    other = _packed([(300, 520, 4.0, "direct", 33), (96, 256, 7.0, "direct", 0)], 1400)
    outs = ep.alloc_outputs(packed, kinds, "cuda")
    sts = _statuses(packed, -7)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ep.decode_batch_noalloc(packed, kinds, outs, sts, stream=s)     # eager, on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ep.decode_batch_noalloc(packed, kinds, outs, sts, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.view(torch.uint8).fill_(0x5A + rep)
        for t in sts:
            t.fill_(-9)
        ep.decode_batch_noalloc(other, "bf16", ep.alloc_outputs(other, ["bf16"] * len(other), "cuda"))  # same scratch
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (p, a, b, sa, sb) in enumerate(zip(packed, ref, outs, ref_st, sts)):
            assert torch.equal(sa[: p.T], sb[: p.T]), f"replay {rep}, tensor {i}: tile statuses differ"
            assert bool((sb[: p.T] == 0).all()), f"replay {rep}, tensor {i}: status {sb[: p.T].unique().tolist()}"
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}, tensor {i}: outputs differ"
