"""Offline quantizers carried through the HIP kernels, and W4A16 rows whose
codes are zero, against the fp64 oracle, through the C ABI on MI355X.

Quantizer chains: the library's host quantizers produce codes, signs and
scales (checked bit-exact against the oracle's quantizers on the CPU), the
library packs them, and the kernels' outputs must meet the bound
|y_gpu - y_oracle| <= 2e-3 * sum_k |w_nk x_k| + 1e-5 against the oracle's
layer applied to the oracle's own quantizer outputs.
  * Efficient Qwen Competition report, sec. 2.1: trained weights go back
    onto the frozen INT4 grid at packing time and are served as W4A16.
  * ShiftAddQwen README, "Output-aware fit" (greedy plus alternating least
    squares sign-plane fit) and "Method / Format" (sa* storage: u8 codes per
    plane and group, one fp16 d per 256-weight super-block).

Zero codes: a row (or group) whose INT4 codes are all zero has the exact
value 0 and a bound of 1e-5, whatever its scale and activations.
"""
import numpy as np
import pytest
import torch

import oracle
import speculative_verify_amd as svq
from speculative_verify_amd import synth

pytestmark = pytest.mark.gpu

REL, ABS = 2e-3, 1e-5


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    svq.load()
    yield
    torch.cuda.synchronize()


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.bfloat16).double().cpu().numpy()


def check_close(y_gpu, y, a, what):
    err = np.abs(y_gpu - y)
    tol = REL * a + ABS
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside bound; worst ratio "
                           f"{(err / tol).max():.3g} at {np.unravel_index((err / tol).argmax(), err.shape)}")


def check_close_or_rounded(y_gpu, y, a, what):
    """The bound, or, where half a bf16 ulp of the exact value exceeds it (|y|
    close to sum |w x|, so that no bf16 value can meet it), the bf16
    round-to-nearest-even of the exact value; either bf16 neighbour only when
    the exact value lies within the bound of their midpoint."""
    tol = REL * a + ABS
    ok = np.abs(y_gpu - y) <= tol
    ay = np.abs(y)
    pos = ay > 0
    e = np.floor(np.log2(np.where(pos, ay, 1.0)))
    ulp = np.exp2(e - 7)
    lo = np.floor(ay / ulp) * ulp
    hi = lo + ulp
    mid = lo + ulp / 2
    even_lo = (np.floor(ay / ulp) % 2) == 0
    rne = np.where(ay < mid, lo, np.where(ay > mid, hi, np.where(even_lo, lo, hi)))
    g = np.abs(y_gpu)
    same_sign = np.sign(y_gpu) == np.sign(y)
    rounded = pos & same_sign & ((g == rne) | ((np.abs(ay - mid) <= tol) & ((g == lo) | (g == hi))))
    bad = ~(ok | rounded)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} neither within the bound nor correctly rounded; "
                           f"first at {np.argwhere(bad)[0]}")


def weights(rng, N, K, scale):
    """bf16 bits [N][K], w ~ N(0, scale^2): stands in for trained weights."""
    return synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * scale).astype(np.float32))


def run_w4a16(blob, X, N, K):
    M = X.shape[0]
    Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    if M == 1:
        svq.gemv_w4a16(blob, dev(X), Y, N, K)
    else:
        svq.gemm_smallm_w4a16(blob, dev(X), Y, M, N, K)
    torch.cuda.synchronize()
    return bf16_host(Y)


# ---------------------------------------------------------------------------
# Quantizer -> pack -> kernel chains

@pytest.mark.parametrize("M", [1, 16, 24, 40])
def test_requantized_int4_through_the_kernels(M):
    rng = np.random.default_rng(700 + M)
    N, K = 1000, 4096
    _, scales = synth.int4_weights(rng, N, K)        # frozen group scales
    w = weights(rng, N, K, 0.05)                    # |w / s| reaches past 8: clamping is exercised
    codes = svq.quantize_int4_frozen(w, scales)
    ocodes = oracle.requant_int4(w, scales)
    assert np.array_equal(codes, ocodes)
    assert (codes == -8).any() and (codes == 7).any()
    X = synth.activations(rng, M, K)
    Y, A = oracle.linear_w4a16(ocodes, scales, X)
    print(f"requant chain M={M}", flush=True)
    blob = dev(svq.pack_int4_grouped(codes, scales))
    check_close(run_w4a16(blob, X, N, K), Y, A, f"requant chain M={M}")


@pytest.mark.parametrize("P,M", [(1, 1), (3, 1), (3, 16), (4, 5), (2, 40)])
def test_fitted_planes_through_the_kernels(P, M):
    rng = np.random.default_rng(720 + 10 * P + M)
    N, K = 600, 4096
    w = weights(rng, N, K, 0.02)
    signs, alpha = svq.fit_binary_planes(w, P=P, iters=10)
    osigns, _, oalpha = oracle.fit_planes(w, P=P, iters=10)
    assert np.array_equal(signs, osigns) and np.array_equal(alpha, oalpha)
    X = synth.activations(rng, M, K)
    Y, A = oracle.linear_binplane(osigns, oalpha, X)
    blob = dev(svq.pack_binary_planes(signs, alpha))
    out = torch.empty((M, N), dtype=torch.int16, device="cuda")
    print(f"plane fit chain P={P} M={M}", flush=True)
    if M == 1:
        svq.gemv_binplane(blob, dev(X), out, N, K, P)
    else:
        svq.gemm_smallm_binplane(blob, dev(X), out, M, N, K, P)
    torch.cuda.synchronize()
    check_close(bf16_host(out), Y, A, f"plane fit chain P={P} M={M}")


@pytest.mark.parametrize("G,P,M", [(64, 3, 1), (128, 3, 1), (256, 3, 1), (64, 3, 16), (128, 2, 16),
                                   (256, 6, 16), (128, 3, 33)])
def test_fitted_snapped_sa_through_the_kernels(G, P, M):
    rng = np.random.default_rng(740 + G + 10 * P + M)
    N, K = 600, 4096
    w = weights(rng, N, K, 0.02)
    signs, alpha = svq.fit_binary_planes(w, P=P, G=G, iters=10)
    codes, d = svq.snap_sa_scales(alpha, G=G)
    osigns, _, oalpha = oracle.fit_planes(w, P=P, G=G, iters=10)
    ocodes, od = oracle.snap_sa(oalpha, G=G)
    assert np.array_equal(signs, osigns) and np.array_equal(codes, ocodes) and np.array_equal(d, od)
    X = synth.activations(rng, M, K)
    Y, A = oracle.linear_sa(osigns, ocodes, od, X, G=G)
    blob = dev(svq.pack_sa(signs, codes, d, G=G))
    out = torch.empty((M, N), dtype=torch.int16, device="cuda")
    print(f"sa chain G={G} P={P} M={M}", flush=True)
    if M == 1:
        svq.gemv_sa(blob, dev(X), out, N, K, P, G=G)
    else:
        svq.gemm_smallm_sa(blob, dev(X), out, M, N, K, P, G=G)
    torch.cuda.synchronize()
    check_close(bf16_host(out), Y, A, f"sa chain G={G} P={P} M={M}")


# ---------------------------------------------------------------------------
# Rows of zero codes

def zero_code_case(rng, N, K, M):
    """Rows 0-127: every code zero.  Rows 128-255: one code in 64 nonzero.
    Rows 256-: uniform codes.  Scale 1.0 everywhere.  Activations N(0, 1)
    with 8 outliers of magnitude 96-112 per row of X."""
    codes = rng.integers(-8, 8, size=(N, K), dtype=np.int8)
    codes[:128] = 0
    sparse = np.zeros((128, K), np.int8)
    for n in range(128):
        at = rng.choice(K, size=K // 64, replace=False)
        sparse[n, at] = rng.choice(np.r_[-8:0, 1:8], size=K // 64).astype(np.int8)
    codes[128:256] = sparse
    scales = np.full((N, K // 128), 0x3F80, np.uint16)  # bf16 1.0
    Xf = rng.standard_normal((M, K)).astype(np.float32)
    for m in range(M):
        at = rng.choice(K, size=8, replace=False)
        Xf[m, at] = rng.choice([-1.0, 1.0], size=8) * rng.uniform(96, 112, size=8)
    return codes, scales, synth.f32_to_bf16_bits(Xf)


@pytest.mark.parametrize("M", [1, 5, 16, 24, 40, 64])
def test_zero_code_rows_are_exact(M):
    # M = 1: the mat-vec; 2-16: the verify mat-mul; 17-32: its two-m-tile
    # form; 33-64: the kernel that streams X.  The 136 carried by each decoded
    # code must cancel exactly where the codes are zero.
    rng = np.random.default_rng(760 + M)
    N, K = 384, 4096
    codes, scales, X = zero_code_case(rng, N, K, M)
    Y, A = oracle.linear_w4a16(codes, scales, X)
    assert (Y[:, :128] == 0).all() and (A[:, :128] == 0).all()
    print(f"zero-code rows M={M}", flush=True)
    blob = dev(svq.pack_int4_grouped(codes, scales))
    got = run_w4a16(blob, X, N, K)
    assert (got[:, :128] == 0).all(), f"{int((got[:, :128] != 0).sum())} all-zero-code outputs are not 0"
    # A sparse row whose nonzero codes meet an outlier has |y| close to
    # sum |w x|: there the bf16 output's own rounding can exceed the bound.
    check_close_or_rounded(got, Y, A, f"zero-code rows M={M}")


@pytest.mark.parametrize("M", [1, 16])
def test_zero_code_rows_in_the_head(M):
    # The heads run the same kernels with the argmax epilogue: a head whose
    # rows are all zero codes but one planted row reports that row with its
    # logit, and a head of only zero-code rows reports row 0 with logit 0
    # (every logit is exactly 0; the lowest index wins the tie).
    rng = np.random.default_rng(780 + M)
    N, K = 4096, 4096
    codes = np.zeros((N, K), np.int8)
    scales = np.full((N, K // 128), 0x3F80, np.uint16)
    Xf = rng.standard_normal((M, K)).astype(np.float32)
    Xf[:, :8] = 100.0
    X = synth.f32_to_bf16_bits(Xf)
    ws = torch.zeros(svq.lmhead_workspace_bytes(M), dtype=torch.uint8, device="cuda")
    idx = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    mx = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    svq.lmhead_argmax(dev(svq.pack_int4_grouped(codes, scales)), dev(X), M, N, K, idx, mx, ws)
    torch.cuda.synchronize()
    assert (idx.cpu().numpy() == 0).all()
    assert (mx.cpu().numpy() == 0).all()
    rows = synth.plant_rows(rng, codes, scales, X)
    r = oracle.argmax_w4a16(codes, scales, X)
    assert np.array_equal(r["idx"], rows.astype(np.int32))
    svq.lmhead_argmax(dev(svq.pack_int4_grouped(codes, scales)), dev(X), M, N, K, idx, mx, ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), rows.astype(np.int32))
    check_close(mx.double().cpu().numpy(), r["zmax"], r["amax"], "zero-code head maxlogit")
