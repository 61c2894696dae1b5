"""Reconstruct-then-GEMM: the decoded weight feeds a library BF16 GEMM.

The compressed linear call (decode into a scratch buffer, then y = x W^T)
must give exactly the output of the same GEMM on the oracle's decoded weight.
"""
import numpy as np
import pytest
import torch

import oracle
import synthgen

pytestmark = pytest.mark.gpu

ep = pytest.importorskip("dit_weight_compression_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.lib()


@pytest.mark.parametrize("tokens", [1, 77, 256])
def test_compressed_linear_matches_gemm_on_oracle_weight(tokens):
    W = synthgen.student_t_weights(384, 1024, 31).numpy()
    ct = oracle.encode(W, 4.0)
    ref_w, _ = oracle.decode(ct, "bf16")
    w_res = torch.from_numpy(ref_w.view(np.int16)).view(torch.bfloat16).to("cuda")
    p = ep.PackedTensor.from_arrays(ct)
    scratch = torch.empty((ct.rows, ct.cols), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ep.workspace_size([p]), dtype=torch.uint8, device="cuda")
    x = torch.randn(tokens, ct.cols, generator=torch.Generator().manual_seed(tokens)).to(torch.bfloat16).cuda()
    for _ in range(2):   # reuse of the scratch buffer and workspace
        ep.decode_batch([p], "bf16", outs=[scratch], workspace=ws)
        y = torch.matmul(x, scratch.t())
        torch.cuda.synchronize()
        assert torch.equal(y, torch.matmul(x, w_res.t()))
