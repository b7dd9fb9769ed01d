"""lmhead_argmax_noalloc (no allocation: the argmax state lives in the
library's static device scratch) against lmhead_argmax (caller workspace),
through the C ABI: bit-identical indices and maximum logits, on two calls in
a row, the second with a smaller input."""
import numpy as np
import pytest
import torch

import oracle
import speculative_verify_amd as svq
from speculative_verify_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    svq.load()
    yield
    torch.cuda.synchronize()


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def both(case, seed, row_ids=None):
    codes, scales, X, rows = synth.make_lmhead(case, seed)
    blob = dev(svq.pack_int4_grouped(codes, scales))
    Xd = dev(X)
    rid = None if row_ids is None else dev(row_ids)
    M, N, K = case.M, case.N, case.K
    out = []
    for noalloc in (True, False):
        idx = torch.full((M,), -7, dtype=torch.int32, device="cuda")
        mx = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            svq.lmhead_argmax_noalloc(blob, Xd, M, N, K, idx, mx, row_ids=rid)
        else:
            ws = torch.zeros(svq.lmhead_workspace_bytes(M), dtype=torch.uint8, device="cuda")
            svq.lmhead_argmax(blob, Xd, M, N, K, idx, mx, ws, row_ids=rid)
        torch.cuda.synchronize()
        out.append((idx.cpu().numpy(), mx.cpu().numpy().view(np.int32)))
    return out, rows, codes, scales, X


def test_noalloc_head_matches_workspace_head_on_two_calls():
    # First call: a full verify block over a 40,000-row head (K = 4096);
    # second: 3 rows over 5,000 rows at K = 1024, with a row -> token map.
    big = synth.Case("noalloc_big", "lmhead", 16, 40000, 4096)
    small = synth.Case("noalloc_small", "lmhead", 3, 5000, 1024)
    print("lmhead_argmax_noalloc M=16 N=40000 K=4096", flush=True)
    (a, b), rows, _, _, _ = both(big, 900)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(a[0], rows.astype(np.int32))
    print("lmhead_argmax_noalloc M=3 N=5000 K=1024", flush=True)
    rid = (7 + 5 * np.arange(small.N)).astype(np.int32)
    (a, b), rows, codes, scales, X = both(small, 901, row_ids=rid)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    r = oracle.argmax_w4a16(codes, scales, X, row_ids=rid)
    assert np.array_equal(a[0], r["out"])


def test_noalloc_head_unplanted_and_single_row():
    # Random rows (no planted maximum) and the M = 1 kernel: still identical
    # to the workspace call, bit for bit.
    for M, N, K in ((1, 248320 // 8, 4096), (16, 7777, 512), (1, 17, 128)):
        rng = np.random.default_rng(M * 1000 + N)
        codes, scales = synth.int4_weights(rng, N, K)
        X = synth.activations(rng, M, K)
        blob, Xd = dev(svq.pack_int4_grouped(codes, scales)), dev(X)
        res = []
        for noalloc in (True, False):
            idx = torch.empty(M, dtype=torch.int32, device="cuda")
            mx = torch.empty(M, dtype=torch.float32, device="cuda")
            if noalloc:
                svq.lmhead_argmax_noalloc(blob, Xd, M, N, K, idx, mx)
            else:
                ws = torch.zeros(svq.lmhead_workspace_bytes(M), dtype=torch.uint8, device="cuda")
                svq.lmhead_argmax(blob, Xd, M, N, K, idx, mx, ws)
            torch.cuda.synchronize()
            res.append(torch.cat([idx, mx.view(torch.int32)]).cpu().numpy())
        assert np.array_equal(res[0], res[1]), (M, N, K)


def test_noalloc_rejects_blocks_beyond_its_scratch():
    t = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(svq.SvqError, match="SHAPE"):
        svq.lmhead_argmax_noalloc(torch.zeros(svq.int4_packed_bytes(16, 128), dtype=torch.uint8, device="cuda"),
                                  torch.zeros(17 * 128, dtype=torch.int16, device="cuda"), 17, 16, 128,
                                  t, t.view(torch.float32))
