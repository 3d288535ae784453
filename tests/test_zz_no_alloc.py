"""The allocation-free greedy entry point (tkq_gemv_argmax_static) against
tkq_gemv_argmax on the same prepared launches, through the C ABI: the
logits bit-identical and the same token, on two calls in a row where the
second launch is smaller (fewer matrices and tiles) than the first, so the
second reads slots the first also wrote."""

import numpy as np
import pytest

from gemm_tkq_gemv_amd import inputs
from helpers import gpu_or_skip

pytestmark = pytest.mark.gpu


def _batch(torch, tkq, shapes, seed):
    items = []
    for i, (N, K) in enumerate(shapes):
        W = inputs.normal_matrix((seed, i, N, K), N, K)
        codes, meta = tkq.pack_int4_g128(torch.from_numpy(W).cuda())
        x = torch.from_numpy(inputs.normal_vector((seed, 50 + i, K), K)).cuda()
        items.append(dict(codes=codes, meta=meta, x=x, N=N, K=K,
                          y=torch.full((N,), float("nan"), dtype=torch.float16, device="cuda")))
    return items


def _compare(torch, tkq, items, target):
    """(token, y of every item) from both entry points on the same inputs."""
    ref = tkq.GemvBatch("int4", items)
    tok_ref = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    ref.run_argmax(target, tok_ref, ref.greedy_scratch().fill_(-1))
    torch.cuda.synchronize()
    y_ref = [it["y"].clone() for it in items]
    for it in items:
        it["y"].fill_(float("nan"))
    torch.cuda.synchronize()
    st = tkq.GemvBatch("int4", items)
    tok = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    st.run_argmax_static(target, tok)
    torch.cuda.synchronize()
    assert int(tok.item()) == int(tok_ref.item()), (int(tok.item()), int(tok_ref.item()))
    for a, b in zip(y_ref, items):
        assert torch.equal(a.view(torch.int16), b["y"].view(torch.int16))
    assert 0 <= int(tok.item()) < items[target]["N"]
    return int(tok.item()), st.tiles


def test_static_argmax_matches_scratch_argmax_twice():
    torch = gpu_or_skip()
    from gemm_tkq_gemv_amd import tkq
    big = _batch(torch, tkq, [(896, 896), (4864, 896), (151936, 896)], 61)
    tok1, tiles1 = _compare(torch, tkq, big, 2)
    small = _batch(torch, tkq, [(3000, 896), (128, 4864)], 62)
    tok2, tiles2 = _compare(torch, tkq, small, 0)
    assert tiles2 < tiles1
    # the token is the first argmax of the stored logits
    y = small[0]["y"].float().cpu().numpy()
    assert tok2 == int(np.argmax(y))
