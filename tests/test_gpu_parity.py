"""HIP path vs the fp64 oracle, through the C ABI, on MI355X.

Bar: codes/indices bit-exact; every float output within
|y_gpu - y_oracle| <= 2e-3 * sum_k |w_nk x_k| + 1e-5 (y_oracle unrounded fp64).
Sizes run from ragged tails and multi-tile cases the oracle finishes in
seconds up to the full workload shapes, in the launch shapes the bench uses.
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


def check_close(y_gpu: np.ndarray, y: np.ndarray, a: np.ndarray, what: str):
    err = np.abs(y_gpu - y)
    tol = REL * a + ABS
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside bound; worst ratio "
                           f"{(err / tol).max():.3g} at {np.unravel_index((err / tol).argmax(), err.shape)}")
    return float((err / tol).max())


def run_gemv_w4a16(codes, scales, x):
    N, K = codes.shape
    blob = dev(svq.pack_int4_grouped(codes, scales))
    y = torch.empty(N, dtype=torch.int16, device="cuda")
    svq.gemv_w4a16(blob, dev(x), y, N, K)
    torch.cuda.synchronize()
    return bf16_host(y)


def run_gemv_binplane(signs, alpha, x):
    P, N, K = signs.shape
    blob = dev(svq.pack_binary_planes(signs, alpha))
    y = torch.empty(N, dtype=torch.int16, device="cuda")
    svq.gemv_binplane(blob, dev(x), y, N, K, P)
    torch.cuda.synchronize()
    return bf16_host(y)


def run_gemm_w4a16(codes, scales, X):
    N, K = codes.shape
    M = X.shape[0]
    blob = dev(svq.pack_int4_grouped(codes, scales))
    Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    svq.gemm_smallm_w4a16(blob, dev(X), Y, M, N, K)
    torch.cuda.synchronize()
    return bf16_host(Y)


def run_gemm_binplane(signs, alpha, X):
    P, N, K = signs.shape
    M = X.shape[0]
    blob = dev(svq.pack_binary_planes(signs, alpha))
    Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    svq.gemm_smallm_binplane(blob, dev(X), Y, M, N, K, P)
    torch.cuda.synchronize()
    return bf16_host(Y)


def run_gemv_sa(signs, codes, d, x, G):
    P, N, K = signs.shape
    blob = dev(svq.pack_sa(signs, codes, d, G=G))
    y = torch.empty(N, dtype=torch.int16, device="cuda")
    svq.gemv_sa(blob, dev(x), y, N, K, P, G=G)
    torch.cuda.synchronize()
    return bf16_host(y)


def run_gemm_sa(signs, codes, d, X, G):
    P, N, K = signs.shape
    M = X.shape[0]
    blob = dev(svq.pack_sa(signs, codes, d, G=G))
    Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    svq.gemm_smallm_sa(blob, dev(X), Y, M, N, K, P, G=G)
    torch.cuda.synchronize()
    return bf16_host(Y)


def run_lmhead(codes, scales, X, row_ids=None, blob=None, N=None, K=None):
    if codes is not None:
        N, K = codes.shape
    M = X.shape[0]
    if blob is None:
        blob = dev(svq.pack_int4_grouped(codes, scales))
    idx = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    mx = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(svq.lmhead_workspace_bytes(M), dtype=torch.uint8, device="cuda")
    svq.lmhead_argmax(blob, dev(X), M, N, K, idx, mx, ws,
                      row_ids=None if row_ids is None else dev(row_ids))
    torch.cuda.synchronize()
    return idx.cpu().numpy(), mx.double().cpu().numpy()


# ---------------------------------------------------------------------------
# W4A16 mat-vec (M = 1)

@pytest.mark.parametrize("case,seed", [(synth.TINY_W4A16, 0), (synth.TINY_W4A16, 1),
                                       (synth.DECODE_W4A16, 0), (synth.DECODE_W4A16, 2)])
def test_gemv_w4a16_configs(case, seed):
    codes, scales, x = synth.make_w4a16(case, seed)
    y, a = oracle.linear_w4a16(codes, scales, x)
    print(f"gemv_w4a16 {case.name} seed={seed}", flush=True)
    check_close(run_gemv_w4a16(codes, scales, x), y[0], a[0], case.name)


@pytest.mark.parametrize("N,K", [(1, 128), (17, 128), (100, 256), (1000, 384), (333, 1152), (2049, 2048),
                                 (77, 8192), (4001, 4096)])
def test_gemv_w4a16_ragged(N, K):
    rng = np.random.default_rng(N + K)
    codes, scales = synth.int4_weights(rng, N, K)
    x = synth.activations(rng, 1, K)
    y, a = oracle.linear_w4a16(codes, scales, x)
    check_close(run_gemv_w4a16(codes, scales, x), y[0], a[0], f"N={N} K={K}")


def test_gemv_w4a16_onehot_unit_scale_is_exact():
    # s = 1, x = e_k: y[n] = c[n][k] exactly, for every k position of two tiles.
    N, K = 40, 256
    rng = np.random.default_rng(5)
    codes = rng.integers(-8, 8, size=(N, K), dtype=np.int8)
    scales = np.full((N, K // 128), 0x3F80, np.uint16)
    blob = dev(svq.pack_int4_grouped(codes, scales))
    y = torch.empty(N, dtype=torch.int16, device="cuda")
    for k in range(K):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = 0x3F80
        svq.gemv_w4a16(blob, dev(x), y, N, K)
        assert np.array_equal(bf16_host(y), codes[:, k].astype(np.float64)), k


# ---------------------------------------------------------------------------
# Binary-plane mat-vec (M = 1)

@pytest.mark.parametrize("seed", [0, 1])
def test_gemv_binplane_config(seed):
    case = synth.DECODE_BINPLANE
    signs, alpha, x = synth.make_binplane(case, seed)
    y, a = oracle.linear_binplane(signs, alpha, x)
    print(f"gemv_binplane {case.name} seed={seed}", flush=True)
    check_close(run_gemv_binplane(signs, alpha, x), y[0], a[0], case.name)


@pytest.mark.parametrize("N,K,P", [(1, 128, 1), (23, 256, 2), (300, 384, 3), (129, 512, 4), (77, 1024, 5),
                                   (64, 2048, 6), (1500, 4096, 3), (45, 6144, 3)])
def test_gemv_binplane_ragged(N, K, P):
    rng = np.random.default_rng(N + K + P)
    signs, alpha = synth.binplane_weights(rng, N, K, P=P)
    x = synth.activations(rng, 1, K)
    y, a = oracle.linear_binplane(signs, alpha, x)
    check_close(run_gemv_binplane(signs, alpha, x), y[0], a[0], f"N={N} K={K} P={P}")


@pytest.mark.parametrize("kind", ["w4a16", "binplane", "sa"])
def test_gemv_wide_matrices(kind):
    # Above three row tiles per CU every mat-vec runs one workgroup a CU with
    # a two-tile ring (N = 20000: 1250 row tiles, a ragged last tile and a
    # partial last ring round on some workgroups).
    N, K = 20000, 4096
    rng = np.random.default_rng(4242)
    x = synth.activations(rng, 1, K)
    print(f"gemv wide {kind} N={N} K={K}", flush=True)
    if kind == "w4a16":
        codes, scales = synth.int4_weights(rng, N, K)
        y, a = oracle.linear_w4a16(codes, scales, x)
        got = run_gemv_w4a16(codes, scales, x)
    elif kind == "binplane":
        signs, alpha = synth.binplane_weights(rng, N, K, P=3)
        y, a = oracle.linear_binplane(signs, alpha, x)
        got = run_gemv_binplane(signs, alpha, x)
    else:
        signs, codes, d = synth.sa_weights(rng, N, K, P=3, G=128)
        y, a = oracle.linear_sa(signs, codes, d, x, G=128)
        got = run_gemv_sa(signs, codes, d, x, G=128)
    check_close(got, y[0], a[0], f"wide {kind}")


def test_gemv_binplane_onehot_unit_plane_is_exact():
    N, K = 20, 256
    rng = np.random.default_rng(6)
    signs, _ = synth.binplane_weights(rng, N, K, P=1)
    alpha = np.full((1, N, K // 128), 0x3C00, np.uint16)
    blob = dev(svq.pack_binary_planes(signs, alpha))
    y = torch.empty(N, dtype=torch.int16, device="cuda")
    for k in range(K):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = 0x3F80
        svq.gemv_binplane(blob, dev(x), y, N, K, 1)
        assert np.array_equal(bf16_host(y), signs[0, :, k].astype(np.float64)), k


def test_three_planes_match_int4_on_odd_codes_across_kernels():
    rng = np.random.default_rng(8)
    N, K = 500, 1024
    codes = (2 * rng.integers(-4, 4, size=(N, K)) + 1).astype(np.int8)
    _, scales = synth.int4_weights(rng, N, K)
    s = synth.bf16_bits_to_f32(scales)
    alpha = synth.f32_to_f16_bits(np.stack([4 * s, 2 * s, s]))
    c = codes.astype(np.int64)
    b1 = np.where(c > 0, 1, -1)
    b2 = np.where(c - 4 * b1 > 0, 1, -1)
    signs = np.stack([b1, b2, c - 4 * b1 - 2 * b2]).astype(np.int8)
    x = synth.activations(rng, 1, K)
    y, a = oracle.linear_w4a16(codes, scales, x)
    check_close(run_gemv_w4a16(codes, scales, x), y[0], a[0], "int4 gemv")
    check_close(run_gemv_binplane(signs, alpha, x), y[0], a[0], "binplane gemv")
    X = synth.activations(rng, 16, K)
    Y, A = oracle.linear_w4a16(codes, scales, X)
    check_close(run_gemm_w4a16(codes, scales, X), Y, A, "int4 gemm")
    check_close(run_gemm_binplane(signs, alpha, X), Y, A, "binplane gemm")


# ---------------------------------------------------------------------------
# Verify-block GEMMs (M <= 16)

@pytest.mark.parametrize("case", synth.VERIFY_W4A16, ids=lambda c: c.name)
def test_gemm_w4a16_configs(case):
    codes, scales, X = synth.make_w4a16(case, 0)
    Y, A = oracle.linear_w4a16(codes, scales, X)
    print(f"gemm_w4a16 {case.name}", flush=True)
    check_close(run_gemm_w4a16(codes, scales, X), Y, A, case.name)


@pytest.mark.parametrize("case", synth.VERIFY_BINPLANE, ids=lambda c: c.name)
def test_gemm_binplane_configs(case):
    signs, alpha, X = synth.make_binplane(case, 0)
    Y, A = oracle.linear_binplane(signs, alpha, X)
    print(f"gemm_binplane {case.name}", flush=True)
    check_close(run_gemm_binplane(signs, alpha, X), Y, A, case.name)


@pytest.mark.parametrize("M", list(range(1, 17)))
def test_gemm_m_sweep_and_rows_match_gemv(M):
    rng = np.random.default_rng(100 + M)
    N, K = 150, 640
    codes, scales = synth.int4_weights(rng, N, K)
    signs, alpha = synth.binplane_weights(rng, N, K, P=3)
    X = synth.activations(rng, M, K)
    Y, A = oracle.linear_w4a16(codes, scales, X)
    Yg = run_gemm_w4a16(codes, scales, X)
    check_close(Yg, Y, A, f"gemm w4a16 M={M}")
    Yb, Ab = oracle.linear_binplane(signs, alpha, X)
    check_close(run_gemm_binplane(signs, alpha, X), Yb, Ab, f"gemm binplane M={M}")
    # every row of the block meets the bound against the M = 1 result of that row
    for m in range(M):
        y1, a1 = oracle.linear_w4a16(codes, scales, X[m:m + 1])
        check_close(Yg[m], y1[0], a1[0], f"row {m}")


@pytest.mark.parametrize("M,N,K", [(16, 200, 8192), (7, 96, 6144), (16, 33, 4224)])
def test_gemm_wide_k(M, N, K):
    # K above 4096 takes the 12- and 16-wave workgroups.
    rng = np.random.default_rng(M + N + K)
    codes, scales = synth.int4_weights(rng, N, K)
    signs, alpha = synth.binplane_weights(rng, N, K, P=3)
    X = synth.activations(rng, M, K)
    Y, A = oracle.linear_w4a16(codes, scales, X)
    check_close(run_gemm_w4a16(codes, scales, X), Y, A, f"gemm w4a16 M={M} N={N} K={K}")
    Yb, Ab = oracle.linear_binplane(signs, alpha, X)
    check_close(run_gemm_binplane(signs, alpha, X), Yb, Ab, f"gemm binplane M={M} N={N} K={K}")
    case = synth.Case("t", "lmhead", M, N, K)
    hc, hs, hX, rows = synth.make_lmhead(case, M + K)
    idx, mx = run_lmhead(hc, hs, hX)
    assert np.array_equal(idx, rows.astype(np.int32))


# Blocks of 16 < M <= 64 rows (the kernel that streams X with the weights).

@pytest.mark.parametrize("M", [17, 20, 24, 31, 32, 33, 40, 47, 48, 56, 63, 64])
def test_gemm_w4a16_midm_ragged(M):  # "midm": 16 < M <= 64
    rng = np.random.default_rng(300 + M)
    N, K = 1000 + 37 * M, 1152
    codes, scales = synth.int4_weights(rng, N, K)
    X = synth.activations(rng, M, K)
    Y, A = oracle.linear_w4a16(codes, scales, X)
    print(f"gemm_smallm_w4a16 M={M} N={N} K={K}", flush=True)
    check_close(run_gemm_w4a16(codes, scales, X), Y, A, f"M={M}")


@pytest.mark.parametrize("M,N,K", [(64, 12288, 4096), (64, 4096, 4096), (32, 12288, 4096), (48, 4096, 4096),
                                   (64, 1, 128), (17, 33, 8192), (64, 300, 256)])
def test_gemm_w4a16_midm_shapes(M, N, K):
    rng = np.random.default_rng(M + N + K)
    codes, scales = synth.int4_weights(rng, N, K)
    X = synth.activations(rng, M, K)
    print(f"gemm_smallm_w4a16 M={M} N={N} K={K}", flush=True)
    got = run_gemm_w4a16(codes, scales, X)
    Y, A = oracle.linear_w4a16(codes, scales, X)
    check_close(got, Y, A, f"M={M} N={N} K={K}")


def test_gemm_w4a16_midm_many_blocks_per_workgroup():
    # 2063 row tiles: blocks of four tiles, several blocks per workgroup, a
    # ragged last tile; checked on a sample of output rows.
    rng = np.random.default_rng(77)
    M, N, K = 64, 33000, 1024
    codes, scales = synth.int4_weights(rng, N, K)
    X = synth.activations(rng, M, K)
    got = run_gemm_w4a16(codes, scales, X)
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(N - 70, N), rng.integers(0, N, 600)]))
    Y, A = oracle.linear_w4a16(codes[rows], scales[rows], X)
    check_close(got[:, rows], Y, A, "M=64 N=33000 sample")


@pytest.mark.parametrize("M,N,K", [(24, 20000, 1024), (32, 40000, 4096), (17, 16400, 2048)])
def test_gemm_w4a16_two_mtiles_many_tiles_per_workgroup(M, N, K):
    # 17..32 rows at K <= 4096 keep both m-tiles in registers; here every
    # workgroup owns several row tiles (with a two-tile ring where the
    # registers allow one), checked on a sample of output rows.
    rng = np.random.default_rng(M + N + K)
    codes, scales = synth.int4_weights(rng, N, K)
    X = synth.activations(rng, M, K)
    print(f"gemm_smallm_w4a16 M={M} N={N} K={K}", flush=True)
    got = run_gemm_w4a16(codes, scales, X)
    rows = np.unique(np.concatenate([np.arange(0, 48), np.arange(N - 40, N), rng.integers(0, N, 400)]))
    Y, A = oracle.linear_w4a16(codes[rows], scales[rows], X)
    check_close(got[:, rows], Y, A, f"M={M} N={N} K={K} sample")


@pytest.mark.parametrize("M,N,K,P", [(17, 300, 512, 3), (40, 1000, 1024, 2), (64, 4096, 4096, 3), (64, 77, 2048, 6),
                                   (40, 700, 8192, 3), (24, 300, 6144, 6)])
def test_gemm_planes_midm(M, N, K, P):
    # Sign planes (fp16 alphas and sa* codes) above 16 rows, each row against
    # the oracle: the 16-row tiles of the block on workgroups of their own at
    # K <= 4096, the streaming kernel that decodes each weight tile once for
    # all m-tiles above.
    rng = np.random.default_rng(M * 7 + N + K + P)
    signs, alpha = synth.binplane_weights(rng, N, K, P=P)
    X = synth.activations(rng, M, K)
    Y, A = oracle.linear_binplane(signs, alpha, X)
    print(f"gemm_smallm_binplane M={M} N={N} K={K} P={P}", flush=True)
    check_close(run_gemm_binplane(signs, alpha, X), Y, A, f"binplane M={M}")
    G = (64, 128, 256)[M % 3]
    s2, codes, d = synth.sa_weights(rng, N, K, max(P, 2), G)
    Y, A = oracle.linear_sa(s2, codes, d, X, G=G)
    check_close(run_gemm_sa(s2, codes, d, X, G), Y, A, f"sa M={M} G={G}")


@pytest.mark.parametrize("kind", ["planes", "sa"])
def test_gemm_planes_midm_every_m(kind):
    # Every block height 17..64 (two, three and four m-tiles, ragged last
    # m-tile) on a ragged N, P cycling through 1..6 (2..6 for sa*) and G
    # through 64, 128, 256.
    rng = np.random.default_rng(4100 + len(kind))
    N, K = 333, 1024
    for M in range(17, 65):
        P = 1 + M % 6 if kind == "planes" else 2 + M % 5
        X = synth.activations(rng, M, K)
        if kind == "planes":
            signs, alpha = synth.binplane_weights(rng, N, K, P=P)
            Y, A = oracle.linear_binplane(signs, alpha, X)
            got = run_gemm_binplane(signs, alpha, X)
        else:
            G = (64, 128, 256)[M % 3]
            signs, codes, d = synth.sa_weights(rng, N, K, P, G)
            Y, A = oracle.linear_sa(signs, codes, d, X, G=G)
            got = run_gemm_sa(signs, codes, d, X, G)
        check_close(got, Y, A, f"{kind} M={M} P={P}")


@pytest.mark.parametrize("K", [2048, 4096])
def test_gemm_planes_two_mtiles(K):
    # Blocks of 17..32 rows at K <= 4096 with up to four planes (and sa* at
    # G >= 128) keep both m-tiles of X in registers; K = 2048 and 4096 take
    # two and four column tiles a wave.  Several tiles a workgroup
    # (N = 9000), a ragged last tile and a ragged second m-tile.
    rng = np.random.default_rng(4150 + K)
    N = 9000
    for M, P in [(17, 1), (24, 3), (32, 4), (29, 2)]:
        X = synth.activations(rng, M, K)
        signs, alpha = synth.binplane_weights(rng, N, K, P=P)
        Y, A = oracle.linear_binplane(signs, alpha, X)
        print(f"two m-tiles planes K={K} M={M} P={P}", flush=True)
        check_close(run_gemm_binplane(signs, alpha, X), Y, A, f"planes K={K} M={M} P={P}")
    for M, P, G in [(17, 2, 128), (32, 3, 256), (25, 4, 128)]:
        X = synth.activations(rng, M, K)
        s2, c2, d2 = synth.sa_weights(rng, N, K, P, G)
        Y, A = oracle.linear_sa(s2, c2, d2, X, G=G)
        print(f"two m-tiles sa K={K} M={M} P={P} G={G}", flush=True)
        check_close(run_gemm_sa(s2, c2, d2, X, G), Y, A, f"sa K={K} M={M} P={P} G={G}")


@pytest.mark.parametrize("M", [65, 100, 128, 193])
def test_gemm_above_64_rows(M):
    # Blocks above 64 rows (prefill chunks) run as consecutive launches of 64
    # rows; every row against the oracle, all three storages.
    rng = np.random.default_rng(4200 + M)
    N, K = 203, 1024
    X = synth.activations(rng, M, K)
    codes, scales = synth.int4_weights(rng, N, K)
    Y, A = oracle.linear_w4a16(codes, scales, X)
    print(f"M={M} above one launch: w4a16", flush=True)
    check_close(run_gemm_w4a16(codes, scales, X), Y, A, f"w4a16 M={M}")
    signs, alpha = synth.binplane_weights(rng, N, K, P=3)
    Y, A = oracle.linear_binplane(signs, alpha, X)
    check_close(run_gemm_binplane(signs, alpha, X), Y, A, f"planes M={M}")
    G = (64, 128, 256)[M % 3]
    s2, c2, d2 = synth.sa_weights(rng, N, K, 4, G)
    Y, A = oracle.linear_sa(s2, c2, d2, X, G=G)
    check_close(run_gemm_sa(s2, c2, d2, X, G), Y, A, f"sa M={M} G={G}")


@pytest.mark.parametrize("M,N,K,P", [(40, 40000, 1024, 3), (64, 20000, 2048, 2), (24, 33333, 512, 4)])
def test_gemm_planes_midm_many_blocks_per_workgroup(M, N, K, P):
    # Enough row tiles that every workgroup walks many of them (at K <= 4096
    # each 16-row tile of the block on workgroups of its own; the ragged
    # last m-tile of M = 40 and 24).
    rng = np.random.default_rng(M + N + K + P)
    signs, alpha = synth.binplane_weights(rng, N, K, P=P)
    X = synth.activations(rng, M, K)
    Y, A = oracle.linear_binplane(signs, alpha, X)
    print(f"planes midm many blocks M={M} N={N} K={K} P={P}", flush=True)
    check_close(run_gemm_binplane(signs, alpha, X), Y, A, f"planes M={M} N={N}")
    G = 64 if P % 2 else 128
    s2, codes, d = synth.sa_weights(rng, N, K, max(P, 2), G)
    Y, A = oracle.linear_sa(s2, codes, d, X, G=G)
    check_close(run_gemm_sa(s2, codes, d, X, G), Y, A, f"sa M={M} N={N}")


@pytest.mark.parametrize("M,N,K,P", [(40, 20000, 6144, 3), (64, 13000, 8192, 2)])
def test_gemm_planes_midm_streaming_many_blocks(M, N, K, P):
    # Above K = 4096 the streaming kernel: every workgroup walks several
    # blocks (grid-stride over blocks, the X and weight cursors crossing
    # block boundaries); checked on a sample of output rows.
    rng = np.random.default_rng(M + N + K + P)
    signs, alpha = synth.binplane_weights(rng, N, K, P=P)
    X = synth.activations(rng, M, K)
    rows = np.unique(np.concatenate([np.arange(0, 48), np.arange(N - 40, N), rng.integers(0, N, 400)]))
    print(f"planes streaming many blocks M={M} N={N} K={K} P={P}", flush=True)
    got = run_gemm_binplane(signs, alpha, X)
    Y, A = oracle.linear_binplane(signs[:, rows], alpha[:, rows], X)
    check_close(got[:, rows], Y, A, f"planes M={M} N={N} K={K} sample")
    G = 128 if P % 2 else 64
    s2, codes, d = synth.sa_weights(rng, N, K, max(P, 2), G)
    got = run_gemm_sa(s2, codes, d, X, G)
    Y, A = oracle.linear_sa(s2[:, rows], codes[:, rows], d[rows], X, G=G)
    check_close(got[:, rows], Y, A, f"sa M={M} N={N} K={K} G={G} sample")


@pytest.mark.parametrize("kind,M,N,K", [("w4a16", 47, 20000, 2048), ("w4a16", 18, 40, 4096), ("w4a16", 64, 12000, 4096),
                                        ("planes", 33, 9000, 4096), ("planes", 50, 35, 1024),
                                        ("sa", 64, 5000, 4096), ("sa", 20, 1000, 4096)])
def test_gemm_msplit_layouts(kind, M, N, K):
    # Blocks of 17..64 rows at K <= 4096 as 16-row tiles on workgroups of
    # their own: ragged last m-tiles (47, 33, 50, 18, 20 rows), workgroups
    # that own many row tiles (N = 20000, 12000, 9000), and workgroups that
    # own none (N = 40 and 35: fewer row tiles than workgroups per m-tile);
    # checked on a sample of output rows.
    rng = np.random.default_rng(M * 31 + N + K)
    X = synth.activations(rng, M, K)
    rows = np.unique(np.concatenate([np.arange(0, min(N, 48)), np.arange(max(0, N - 40), N), rng.integers(0, N, 300)]))
    print(f"msplit {kind} M={M} N={N} K={K}", flush=True)
    if kind == "w4a16":
        codes, scales = synth.int4_weights(rng, N, K)
        got = run_gemm_w4a16(codes, scales, X)
        Y, A = oracle.linear_w4a16(codes[rows], scales[rows], X)
    elif kind == "planes":
        signs, alpha = synth.binplane_weights(rng, N, K, P=3)
        got = run_gemm_binplane(signs, alpha, X)
        Y, A = oracle.linear_binplane(signs[:, rows], alpha[:, rows], X)
    else:
        signs, codes, d = synth.sa_weights(rng, N, K, 3, 128)
        got = run_gemm_sa(signs, codes, d, X, 128)
        Y, A = oracle.linear_sa(signs[:, rows], codes[:, rows], d[rows], X, G=128)
    check_close(got[:, rows], Y, A, f"{kind} M={M} N={N} K={K} sample")


@pytest.mark.parametrize("M,P", [(20, 1), (33, 3), (64, 6)])
def test_gemm_planes_midm_onehot_unit_alpha_is_exact(M, P):
    # Unit alphas and x = one-hot rows: each output is sum_p b_p[n][k_m], a
    # small integer, exactly -- pins every (row, k) position and m-tile of
    # the block kernel.
    rng = np.random.default_rng(M * 10 + P)
    N, K = 96, 2048
    signs = (1 - 2 * rng.integers(0, 2, size=(P, N, K))).astype(np.int8)
    alpha = np.full((P, N, K // 128), 0x3C00, np.uint16)  # fp16 1.0
    ks = rng.choice(K, size=M, replace=False)
    X = np.zeros((M, K), np.uint16)
    X[np.arange(M), ks] = 0x3F80  # bf16 1.0
    want = signs[:, :, ks].sum(axis=0).T.astype(np.float64)  # [M][N]
    got = run_gemm_binplane(signs, alpha, X)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("M", [33, 64])
def test_gemm_w4a16_midm_onehot_unit_scale_is_exact(M):
    # Row m of X is e_{k_m}: Y[m][n] = c[n][k_m] exactly, for every m-tile.
    N, K = 48, 512
    rng = np.random.default_rng(90 + M)
    codes = rng.integers(-8, 8, size=(N, K), dtype=np.int8)
    scales = np.full((N, K // 128), 0x3F80, np.uint16)
    blob = dev(svq.pack_int4_grouped(codes, scales))
    Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    for base in range(0, K, 64):
        ks = [(base + 3 * m) % K for m in range(M)]
        X = np.zeros((M, K), np.uint16)
        X[np.arange(M), ks] = 0x3F80
        svq.gemm_smallm_w4a16(blob, dev(X), Y, M, N, K)
        assert np.array_equal(bf16_host(Y), codes[:, ks].T.astype(np.float64)), base


def test_gemm_onehot_unit_scale_is_exact():
    # Row m of X is e_{k_m}; Y[m][n] = c[n][k_m] exactly (checks both MFMA operand layouts).
    N, K, M = 48, 256, 16
    rng = np.random.default_rng(9)
    codes = rng.integers(-8, 8, size=(N, K), dtype=np.int8)
    scales = np.full((N, K // 128), 0x3F80, np.uint16)
    signs, _ = synth.binplane_weights(rng, N, K, P=1)
    alpha = np.full((1, N, K // 128), 0x3C00, np.uint16)
    blob = dev(svq.pack_int4_grouped(codes, scales))
    bblob = dev(svq.pack_binary_planes(signs, alpha))
    Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    for base in range(0, K, M):
        ks = [(base + 5 * m) % K for m in range(M)]
        X = np.zeros((M, K), np.uint16)
        X[np.arange(M), ks] = 0x3F80
        svq.gemm_smallm_w4a16(blob, dev(X), Y, M, N, K)
        assert np.array_equal(bf16_host(Y), codes[:, ks].T.astype(np.float64)), base
        svq.gemm_smallm_binplane(bblob, dev(X), Y, M, N, K, 1)
        assert np.array_equal(bf16_host(Y), signs[0][:, ks].T.astype(np.float64)), base


# ---------------------------------------------------------------------------
# sa* storage (u8 scale codes per plane and group, fp16 d per super-block)

@pytest.mark.parametrize("G", [64, 128, 256])
def test_gemv_sa_decode_shape(G):
    case = synth.Case(f"decode_sa_p3_g{G}", "sa", 1, 12288, 4096, P=3, G=G)
    signs, codes, d, x = synth.make_sa(case, 0)
    y, a = oracle.linear_sa(signs, codes, d, x, G=G)
    print(f"gemv_sa {case.name}", flush=True)
    check_close(run_gemv_sa(signs, codes, d, x, G), y[0], a[0], case.name)


@pytest.mark.parametrize("N,K,P,G", [(1, 256, 2, 64), (23, 512, 3, 128), (300, 768, 4, 256), (129, 1024, 5, 64),
                                     (77, 2048, 6, 128), (1500, 4096, 3, 256), (45, 6144, 3, 64),
                                     (33, 8192, 2, 128), (64, 4352, 6, 256)])
def test_gemv_sa_ragged(N, K, P, G):
    rng = np.random.default_rng(N + K + P + G)
    signs, codes, d = synth.sa_weights(rng, N, K, P, G)
    x = synth.activations(rng, 1, K)
    y, a = oracle.linear_sa(signs, codes, d, x, G=G)
    check_close(run_gemv_sa(signs, codes, d, x, G), y[0], a[0], f"N={N} K={K} P={P} G={G}")


@pytest.mark.parametrize("N,G", [(4096, 128), (12288, 128), (4096, 64), (4096, 256)])
def test_gemm_sa_verify_shapes(N, G):
    case = synth.Case(f"verify_sa_p3_m16_n{N}_g{G}", "sa", 16, N, 4096, P=3, G=G)
    signs, codes, d, X = synth.make_sa(case, 0)
    Y, A = oracle.linear_sa(signs, codes, d, X, G=G)
    print(f"gemm_smallm_sa {case.name}", flush=True)
    check_close(run_gemm_sa(signs, codes, d, X, G), Y, A, case.name)


@pytest.mark.parametrize("M", list(range(1, 17)))
def test_gemm_sa_m_sweep_and_rows_match_gemv(M):
    G = (64, 128, 256)[M % 3]
    P = 2 + M % 5
    rng = np.random.default_rng(200 + M)
    N, K = 150, 768
    signs, codes, d = synth.sa_weights(rng, N, K, P, G)
    X = synth.activations(rng, M, K)
    Y, A = oracle.linear_sa(signs, codes, d, X, G=G)
    Yg = run_gemm_sa(signs, codes, d, X, G)
    check_close(Yg, Y, A, f"gemm sa M={M} P={P} G={G}")
    y0 = run_gemv_sa(signs, codes, d, X[:1], G)
    check_close(y0, Y[0], A[0], f"gemv sa row 0 P={P} G={G}")


@pytest.mark.parametrize("M,N,K,G", [(16, 200, 8192, 64), (7, 96, 6144, 128), (16, 33, 4352, 256)])
def test_gemm_sa_wide_k(M, N, K, G):
    rng = np.random.default_rng(M + N + K + G)
    signs, codes, d = synth.sa_weights(rng, N, K, 3, G)
    X = synth.activations(rng, M, K)
    Y, A = oracle.linear_sa(signs, codes, d, X, G=G)
    check_close(run_gemm_sa(signs, codes, d, X, G), Y, A, f"gemm sa M={M} N={N} K={K} G={G}")


@pytest.mark.parametrize("G", [64, 128, 256])
def test_sa_onehot_with_unit_d_is_exact(G):
    # d = 1 and codes <= 40 over three planes: y = sum_p a_p b_p is an integer of
    # magnitude <= 120, exact in bf16, for x = e_k at every k of two super-blocks
    # (mat-vec), and for 16 different k per launch (mat-mul).
    N, K, P = 40, 512, 3
    rng = np.random.default_rng(11 + G)
    signs, _, _ = synth.sa_weights(rng, N, K, P, G)
    codes = rng.integers(0, 41, size=(P, N, K // G)).astype(np.uint8)
    d = np.full((N, K // 256), 0x3C00, np.uint16)
    blob = dev(svq.pack_sa(signs, codes, d, G=G))
    k = np.arange(K)
    want = sum(codes[p][:, k // G].astype(np.int64) * signs[p].astype(np.int64) for p in range(P))
    y = torch.empty(N, dtype=torch.int16, device="cuda")
    for kk in range(K):
        x = np.zeros((1, K), np.uint16)
        x[0, kk] = 0x3F80
        svq.gemv_sa(blob, dev(x), y, N, K, P, G=G)
        assert np.array_equal(bf16_host(y), want[:, kk].astype(np.float64)), kk
    M = 16
    Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    for base in range(0, K, M):
        ks = [(base + 7 * m) % K for m in range(M)]
        X = np.zeros((M, K), np.uint16)
        X[np.arange(M), ks] = 0x3F80
        svq.gemm_smallm_sa(blob, dev(X), Y, M, N, K, P, G=G)
        assert np.array_equal(bf16_host(Y), want[:, ks].T.astype(np.float64)), base


def test_sa_codes_4_2_1_match_int4_on_odd_codes():
    # With codes (4, 2, 1) and d = the super-block's INT4 scale, the three sign
    # planes of an odd code c carry s * c: both sa kernels meet the bound
    # against the W4A16 oracle.
    rng = np.random.default_rng(12)
    N, K = 300, 1024
    codes4 = (2 * rng.integers(-4, 4, size=(N, K)) + 1).astype(np.int8)
    _, s_sb = synth.int4_weights(rng, N, K, G=256)
    scales = np.repeat(s_sb, 2, axis=1)
    d = synth.f32_to_f16_bits(synth.bf16_bits_to_f32(s_sb))
    c = codes4.astype(np.int64)
    b1 = np.where(c > 0, 1, -1)
    b2 = np.where(c - 4 * b1 > 0, 1, -1)
    signs = np.stack([b1, b2, c - 4 * b1 - 2 * b2]).astype(np.int8)
    sa_codes = np.empty((3, N, K // 64), np.uint8)
    sa_codes[0], sa_codes[1], sa_codes[2] = 4, 2, 1
    X = synth.activations(rng, 16, K)
    Y, A = oracle.linear_w4a16(codes4, scales, X)
    check_close(run_gemv_sa(signs, sa_codes, d, X[:1], 64), Y[0], A[0], "sa gemv")
    check_close(run_gemm_sa(signs, sa_codes, d, X, 64), Y, A, "sa gemm")


# ---------------------------------------------------------------------------
# Output rounding and accumulation quality

def bf16_rne_candidates(v: np.ndarray, slack: np.ndarray):
    """The bf16 value(s) a correctly rounded result may take for exact v > 0."""
    e = np.floor(np.log2(v))
    ulp = np.exp2(e - 7)
    lo = np.floor(v / ulp) * ulp
    hi = lo + ulp
    mid = lo + ulp / 2
    even_lo = (np.floor(v / ulp) % 2) == 0
    pick = np.where(v < mid, lo, np.where(v > mid, hi, np.where(even_lo, lo, hi)))
    either = np.abs(v - mid) <= slack
    return pick, lo, hi, either


@pytest.mark.parametrize("kind", ["w4a16_gemv", "w4a16_gemm", "binplane_gemv", "binplane_gemm", "sa_gemv",
                                  "sa_gemm"])
def test_sign_coherent_outputs_are_correctly_rounded(kind):
    # x > 0 and every weight positive: |y| = sum |w x|.  The result must be the
    # bf16 round-to-nearest-even of the exact sum (either neighbour only when the
    # exact sum lies within 4e-5 * |y| of a rounding midpoint).
    rng = np.random.default_rng(10)
    N, K, M = 256, 4096, 16
    X = synth.f32_to_bf16_bits(np.abs(rng.standard_normal((M, K))).astype(np.float32) + 0.01)
    if kind.startswith("w4a16"):
        codes = np.full((N, K), 7, np.int8)
        codes[::3] = 5
        _, scales = synth.int4_weights(rng, N, K)
        Y, A = oracle.linear_w4a16(codes, scales, X)
        got = run_gemv_w4a16(codes, scales, X[:1])[None] if kind.endswith("gemv") else \
            run_gemm_w4a16(codes, scales, X)
    elif kind.startswith("binplane"):
        signs = np.ones((3, N, K), np.int8)
        _, alpha = synth.binplane_weights(rng, N, K, P=3)
        Y, A = oracle.linear_binplane(signs, alpha, X)
        got = run_gemv_binplane(signs, alpha, X[:1])[None] if kind.endswith("gemv") else \
            run_gemm_binplane(signs, alpha, X)
    else:
        _, codes, d = synth.sa_weights(rng, N, K, 3, 64)
        signs = np.ones((3, N, K), np.int8)
        Y, A = oracle.linear_sa(signs, codes, d, X, G=64)
        got = run_gemv_sa(signs, codes, d, X[:1], 64)[None] if kind.endswith("gemv") else \
            run_gemm_sa(signs, codes, d, X, 64)
    Y = Y[: got.shape[0]]
    pick, lo, hi, either = bf16_rne_candidates(Y, 4e-5 * Y)
    ok = (got == pick) | (either & ((got == lo) | (got == hi)))
    assert ok.all(), f"{(~ok).sum()} outputs not correctly rounded"


def test_results_are_bitwise_deterministic():
    case = synth.DECODE_W4A16
    codes, scales, x = synth.make_w4a16(case, 3)
    a = run_gemv_w4a16(codes, scales, x)
    b = run_gemv_w4a16(codes, scales, x)
    assert np.array_equal(a, b)
    X = synth.activations(np.random.default_rng(4), 16, case.K)
    assert np.array_equal(run_gemm_w4a16(codes, scales, X), run_gemm_w4a16(codes, scales, X))


# ---------------------------------------------------------------------------
# LM head with fused argmax

_PLANTED = {}


def planted_head(case, seed=0):
    """A planted head case with its oracle result and packed device blob,
    kept for the next test (the full-vocabulary heads take seconds to draw
    and check): (X, rows, oracle result, blob)."""
    key = (case.name, seed)
    if key not in _PLANTED:
        _PLANTED.clear()
        print(f"lmhead {case.name}: generating", flush=True)
        codes, scales, X, rows = synth.make_lmhead(case, seed)
        r = oracle.argmax_w4a16(codes, scales, X)
        blob = dev(svq.pack_int4_grouped(codes, scales))
        del codes, scales
        _PLANTED[key] = (X, rows, r, blob)
    return _PLANTED[key]


@pytest.mark.parametrize("case", synth.LMHEAD, ids=lambda c: c.name)
def test_lmhead_planted_configs(case):
    X, rows, r, blob = planted_head(case)
    assert np.array_equal(r["idx"], rows.astype(np.int32))
    tol = REL * r["amax"] + ABS
    assert np.all(r["zmax"] - r["zsecond"] > 10 * tol), "planted margin too small"
    print(f"lmhead {case.name}: running", flush=True)
    idx, mx = run_lmhead(None, None, X, blob=blob, N=case.N, K=case.K)
    assert np.array_equal(idx, rows.astype(np.int32))
    check_close(mx, r["zmax"], r["amax"], "maxlogit")


@pytest.mark.parametrize("levels", [None, "2"])
def test_lmhead_verify_greedy_full_vocab(levels, monkeypatch):
    # The verify step exactly as the bench times it: M = 16 query rows over
    # the full 248,320-row head at K = 4096 (61 row tiles a workgroup, so the
    # one-level argmax completion by default; "2" forces the two-level one),
    # greedy acceptance fused.  Drafts are the planted target tokens with one
    # rejected position, or all accepted.
    case = synth.LMHEAD[3]
    assert (case.M, case.N, case.K) == (16, 248320, 4096)
    X, rows, r, blob = planted_head(case)
    monkeypatch.delenv("SVQ_ARGMAX_LEVELS", raising=False)
    if levels is not None:
        monkeypatch.setenv("SVQ_ARGMAX_LEVELS", levels)
    M, N, K = case.M, case.N, case.K
    t_ids = rows.astype(np.int32)
    Xd = dev(X)
    ws = torch.zeros(svq.lmhead_workspace_bytes(M), dtype=torch.uint8, device="cuda")
    for bad in (0, 6, 14, None):
        d = t_ids[:-1].copy()
        if bad is not None:
            d[bad] = (d[bad] + 1) % N
        idx = torch.full((M,), -1, dtype=torch.int32, device="cuda")
        mx = torch.zeros(M, dtype=torch.float32, device="cuda")
        tau = torch.zeros(1, dtype=torch.int32, device="cuda")
        print(f"lmhead_verify_greedy full vocab levels={levels} rejected={bad}", flush=True)
        svq.lmhead_verify_greedy(blob, Xd, M, N, K, dev(d), idx, mx, tau, ws)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), t_ids)
        check_close(mx.double().cpu().numpy(), r["zmax"], r["amax"], "verify maxlogit")
        want = oracle.verify_greedy(t_ids, d)
        assert want == (M if bad is None else bad + 1)
        assert int(tau.item()) == want, bad
        assert int(ws.count_nonzero().item()) == 0


def test_lmhead_row_ids_and_ties():
    rng = np.random.default_rng(21)
    case = synth.Case("t", "lmhead", 4, 3000, 1024)
    codes, scales, X, rows = synth.make_lmhead(case, 21)
    # Copy each planted row to a lower index in a different tile: the tie goes low.
    for m in range(case.M):
        dst = int(rng.integers(0, rows[m])) if rows[m] > 0 else None
        if dst is not None and dst not in rows:
            codes[dst] = codes[rows[m]]
            scales[dst] = scales[rows[m]]
    rid = rng.permutation(200000)[: case.N].astype(np.int32)
    r = oracle.argmax_w4a16(codes, scales, X, row_ids=rid)
    idx, mx = run_lmhead(codes, scales, X, row_ids=rid)
    assert np.array_equal(idx, r["out"])
    for m in range(case.M):  # single-row queries take the M = 1 path
        i1, _ = run_lmhead(codes, scales, X[m:m + 1], row_ids=rid)
        assert i1[0] == r["out"][m]


@pytest.mark.parametrize("M", [1, 5, 16])
def test_lmhead_unplanted_pick_is_a_valid_maximum(M):
    # Without planting, near-ties are possible: any index whose exact logit is
    # within the two tolerances of the exact maximum is a correct greedy pick.
    rng = np.random.default_rng(30 + M)
    N, K = 20000, 2048
    codes, scales = synth.int4_weights(rng, N, K)
    X = synth.activations(rng, M, K)
    Z, A = oracle.linear_w4a16(codes, scales, X)
    idx, mx = run_lmhead(codes, scales, X)
    for m in range(M):
        best = int(np.argmax(Z[m]))
        tol = lambda n: REL * A[m, n] + ABS
        g = int(idx[m])
        assert Z[m, g] >= Z[m, best] - tol(g) - tol(best), (m, g, best)
        assert abs(mx[m] - Z[m, g]) <= tol(g)


def test_lmhead_single_row_and_ragged_vocab():
    rng = np.random.default_rng(40)
    for N in (1, 15, 17, 1001):
        codes, scales = synth.int4_weights(rng, N, 256)
        X = synth.activations(rng, 3, 256)
        r = oracle.argmax_w4a16(codes, scales, X)
        idx, mx = run_lmhead(codes, scales, X)
        Z, A = oracle.linear_w4a16(codes, scales, X)
        for m in range(3):
            g = int(idx[m])
            assert 0 <= g < N
            assert Z[m, g] >= r["zmax"][m] - 2 * (REL * A[m].max() + ABS)


def test_lmhead_workspace_counter_is_reusable():
    # One zeroed workspace serves many calls of different M and N; it is
    # all zero again after every call.
    rng = np.random.default_rng(50)
    ws = torch.zeros(svq.lmhead_workspace_bytes(16), dtype=torch.uint8, device="cuda")
    for it in range(6):
        M = (1, 16, 3, 1, 16, 7)[it]
        N = (5000, 2000, 16, 70000, 40000, 999)[it]
        case = synth.Case("t", "lmhead", M, N, 512)
        codes, scales, X, rows = synth.make_lmhead(case, 100 + it)
        blob = dev(svq.pack_int4_grouped(codes, scales))
        idx = torch.full((M,), -1, dtype=torch.int32, device="cuda")
        mx = torch.zeros(M, dtype=torch.float32, device="cuda")
        svq.lmhead_argmax(blob, dev(X), M, N, 512, idx, mx, ws)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), rows.astype(np.int32)), it
        assert int(ws.count_nonzero().item()) == 0, it


# ---------------------------------------------------------------------------
# Greedy acceptance of a verified block

def test_verify_greedy_matches_oracle():
    rng = np.random.default_rng(60)
    cases = []
    for M in range(1, 17):
        for a in range(M):  # accepted drafts
            t = rng.integers(0, 1000, M).astype(np.int32)
            d = t[:-1].copy()
            if a < M - 1:
                d[a] = t[a] + 1
            cases.append((t, d))
    t = np.array([4, -1, 7], np.int32)
    cases.append((t, np.array([4, 0], np.int32)))
    tau = torch.zeros(1, dtype=torch.int32, device="cuda")
    for t, d in cases:
        M = t.shape[0]
        svq.verify_greedy(dev(t), dev(d) if M > 1 else None, M, tau)
        torch.cuda.synchronize()
        assert int(tau.item()) == oracle.verify_greedy(t, d), (t, d)


@pytest.mark.parametrize("M,N", [(16, 4096), (5, 32768), (1, 2000)])
def test_lmhead_verify_greedy_planted(M, N):
    case = synth.Case("t", "lmhead", M, N, 1024)
    codes, scales, X, rows = synth.make_lmhead(case, 70 + M)
    rid = (5 + 3 * np.arange(N)).astype(np.int32)
    t_ids = rid[rows].astype(np.int32)
    blob = dev(svq.pack_int4_grouped(codes, scales))
    ws = torch.zeros(svq.lmhead_workspace_bytes(M), dtype=torch.uint8, device="cuda")
    idx = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    mx = torch.zeros(M, dtype=torch.float32, device="cuda")
    tau = torch.zeros(1, dtype=torch.int32, device="cuda")
    Xd, rd = dev(X), dev(rid)
    for bad in list(range(M - 1)) + [None]:
        d = t_ids[:-1].copy()
        if bad is not None:
            d[bad] += 1
        svq.lmhead_verify_greedy(blob, Xd, M, N, 1024, dev(d) if M > 1 else None, idx, mx, tau, ws,
                                 row_ids=rd)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), t_ids)
        want = oracle.verify_greedy(t_ids, d)
        assert want == (M if bad is None else bad + 1)
        assert int(tau.item()) == want, bad
        assert int(ws.count_nonzero().item()) == 0


# ---------------------------------------------------------------------------
# Sign-plane head

@pytest.mark.parametrize("M,N,K,P", [(1, 5000, 4096, 3), (16, 32768, 4096, 3), (5, 777, 1024, 2),
                                     (16, 300, 6144, 4), (1, 64, 256, 1)])
def test_lmhead_binplane_planted(M, N, K, P):
    case = synth.Case("t", "lmhead", M, N, K, P=P)
    signs, alpha, X, rows = synth.make_lmhead_binplane(case, 80 + M + P)
    rid = (11 + 2 * np.arange(N)).astype(np.int32)
    r = oracle.argmax_binplane(signs, alpha, X, row_ids=rid)
    assert np.array_equal(r["idx"], rows.astype(np.int32))
    blob = dev(svq.pack_binary_planes(signs, alpha))
    idx = torch.full((M,), -1, dtype=torch.int32, device="cuda")
    mx = torch.zeros(M, dtype=torch.float32, device="cuda")
    ws = torch.zeros(svq.lmhead_workspace_bytes(M), dtype=torch.uint8, device="cuda")
    print(f"lmhead_argmax_binplane M={M} N={N} K={K} P={P}", flush=True)
    svq.lmhead_argmax_binplane(blob, dev(X), M, N, K, P, idx, mx, ws, row_ids=dev(rid))
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), r["out"])
    check_close(mx.double().cpu().numpy(), r["zmax"], r["amax"], "binplane head max")
    assert int(ws.count_nonzero().item()) == 0


# ---------------------------------------------------------------------------
# Launch-shape independence: the workgroup count, the ring depth and the
# workgroups per CU change which workgroup computes a tile and how far ahead
# it loads, never the arithmetic (each tile's per-wave partials are combined
# in wave order), so every output must be bit-identical under every setting
# of the tuning knobs.  The heads' argmax completion in one level or two
# (SVQ_ARGMAX_LEVELS) changes only the order of max operations.

_KNOBS = [{}, {"SVQ_WG_PER_CU": "1"}, {"SVQ_WG_PER_CU": "3"}, {"SVQ_PIPE_DEPTH": "1"}, {"SVQ_PIPE_DEPTH": "3"},
          {"SVQ_GRID_MAX": "37"}, {"SVQ_ARGMAX_LEVELS": "1"}, {"SVQ_ARGMAX_LEVELS": "2"},
          {"SVQ_ARGMAX_LEVELS": "2", "SVQ_GRID_MAX": "5"}]


def _under_knobs(fn, monkeypatch):
    outs = []
    for knobs in _KNOBS:
        for k in ("SVQ_WG_PER_CU", "SVQ_PIPE_DEPTH", "SVQ_GRID_MAX", "SVQ_ARGMAX_LEVELS"):
            monkeypatch.delenv(k, raising=False)
        for k, v in knobs.items():
            monkeypatch.setenv(k, v)
        outs.append((knobs, fn()))
        torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("kind,M", [("w4a16", 1), ("w4a16", 16), ("w4a16", 5), ("binplane", 1), ("binplane", 16),
                                    ("sa", 1), ("sa", 16), ("head", 1), ("head", 16), ("bphead", 1),
                                    ("bphead", 16), ("verify", 16), ("w4a16", 40), ("w4a16", 24),
                                    ("binplane", 64), ("sa", 33)])
def test_outputs_do_not_depend_on_launch_shape(kind, M, monkeypatch):
    N, K, P, G = 5008, 4096, 3, 64  # 313 row tiles (the device generators need whole tiles)
    X = synth.device_activations(M, K, 11).view(torch.int16)
    if kind in ("w4a16", "head", "verify"):
        blob = synth.device_int4_blob(N, K, 12)
    elif kind in ("binplane", "bphead"):
        blob = synth.device_binplane_blob(N, K, P, 13)
    else:
        blob = synth.device_sa_blob(N, K, P, G, 14)

    # Drafts for the verify call: the greedy tokens of a first call with the
    # eighth one changed, so tau = 8 whatever the knobs.
    draft = None
    if kind == "verify":
        idx0 = torch.empty(M, dtype=torch.int32, device="cuda")
        mx0 = torch.empty(M, dtype=torch.float32, device="cuda")
        ws0 = torch.zeros(svq.lmhead_workspace_bytes(M), dtype=torch.uint8, device="cuda")
        svq.lmhead_argmax(blob, X, M, N, K, idx0, mx0, ws0)
        draft = idx0[:-1].clone()
        draft[7] = (draft[7] + 1) % N

    def call():
        if kind in ("head", "bphead", "verify"):
            idx = torch.empty(M, dtype=torch.int32, device="cuda")
            mx = torch.empty(M, dtype=torch.float32, device="cuda")
            ws = torch.zeros(svq.lmhead_workspace_bytes(M), dtype=torch.uint8, device="cuda")
            tau = torch.zeros(1, dtype=torch.int32, device="cuda")
            if kind == "head":
                svq.lmhead_argmax(blob, X, M, N, K, idx, mx, ws)
            elif kind == "verify":
                svq.lmhead_verify_greedy(blob, X, M, N, K, draft, idx, mx, tau, ws)
                assert int(tau.item()) == 8
            else:
                svq.lmhead_argmax_binplane(blob, X, M, N, K, P, idx, mx, ws)
            return torch.cat([idx.view(torch.int32), mx.view(torch.int32), tau]).cpu().numpy()
        Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
        if kind == "w4a16":
            (svq.gemv_w4a16(blob, X, Y, N, K) if M == 1 else svq.gemm_smallm_w4a16(blob, X, Y, M, N, K))
        elif kind == "binplane":
            (svq.gemv_binplane(blob, X, Y, N, K, P) if M == 1 else svq.gemm_smallm_binplane(blob, X, Y, M, N, K, P))
        else:
            (svq.gemv_sa(blob, X, Y, N, K, P, G) if M == 1 else svq.gemm_smallm_sa(blob, X, Y, M, N, K, P, G))
        return Y.cpu().numpy()

    print(f"launch-shape independence {kind} M={M}", flush=True)
    outs = _under_knobs(call, monkeypatch)
    ref = outs[0][1]
    for knobs, out in outs[1:]:
        assert np.array_equal(out, ref), f"{kind} M={M}: outputs differ under {knobs}"


@pytest.mark.parametrize("kind,M,N", [("w4a16", 64, 3008), ("w4a16", 47, 704), ("planes", 40, 3008),
                                      ("planes", 20, 2000), ("sa", 64, 1200), ("sa", 33, 3008)])
def test_msplit_block_equals_its_16_row_slices(kind, M, N):
    # A block of 17..64 rows at K <= 4096 with no more row tiles than CUs runs
    # as 16-row m-tiles of the M <= 16 kernel in one launch: the same
    # arithmetic per output as separate calls on each 16-row slice, so the
    # outputs must match those calls bit for bit.
    K, P, G = 4096, 3, 128
    X = synth.device_activations(M, K, 31 + M).view(torch.int16)
    if kind == "w4a16":
        blob = synth.device_int4_blob(N, K, 32)
    elif kind == "planes":
        blob = synth.device_binplane_blob(N, K, P, 33)
    else:
        blob = synth.device_sa_blob(N, K, P, G, 34)

    def run(Xs, m):
        Y = torch.empty((m, N), dtype=torch.int16, device="cuda")
        if kind == "w4a16":
            svq.gemm_smallm_w4a16(blob, Xs, Y, m, N, K)
        elif kind == "planes":
            svq.gemm_smallm_binplane(blob, Xs, Y, m, N, K, P)
        else:
            svq.gemm_smallm_sa(blob, Xs, Y, m, N, K, P, G)
        return Y

    print(f"m-split {kind} M={M} N={N} against its slices", flush=True)
    whole = run(X, M).cpu().numpy()
    for m0 in range(0, M, 16):
        m = min(16, M - m0)
        part = run(X[m0:m0 + m].contiguous(), m).cpu().numpy()
        assert np.array_equal(whole[m0:m0 + m], part), f"{kind} M={M}: rows {m0}..{m0 + m - 1} differ"


# ---------------------------------------------------------------------------
# Seeded sweep over random shapes: every linear call at random M (1..64), N,
# K (up to 8192, so both workgroup widths), P and G, against the oracle.

@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_random_shapes_against_the_oracle(seed):
    rng = np.random.default_rng(1000 + seed)
    for c in range(12):
        kind = ("w4a16", "binplane", "sa")[c % 3]
        M = int(rng.choice([1, 2, 5, 16, 17, 33, 64]))
        if kind == "sa":
            G, K, P = int(rng.choice([64, 128, 256])), 256 * int(rng.integers(1, 33)), int(rng.integers(2, 7))
        else:
            G, K, P = 128, 128 * int(rng.integers(1, 65)), int(rng.integers(1, 7))
        N = int(rng.integers(1, 1500))
        what = f"seed {seed} case {c}: {kind} M={M} N={N} K={K} P={P} G={G}"
        print(what, flush=True)
        X = synth.activations(rng, M, K)
        if kind == "w4a16":
            codes, scales = synth.int4_weights(rng, N, K)
            Y, A = oracle.linear_w4a16(codes, scales, X)
            Yg = run_gemv_w4a16(codes, scales, X)[None] if M == 1 else run_gemm_w4a16(codes, scales, X)
        elif kind == "binplane":
            signs, alpha = synth.binplane_weights(rng, N, K, P=P)
            Y, A = oracle.linear_binplane(signs, alpha, X)
            Yg = run_gemv_binplane(signs, alpha, X)[None] if M == 1 else run_gemm_binplane(signs, alpha, X)
        else:
            signs, codes, d = synth.sa_weights(rng, N, K, P, G)
            Y, A = oracle.linear_sa(signs, codes, d, X, G=G)
            Yg = run_gemv_sa(signs, codes, d, X, G)[None] if M == 1 else run_gemm_sa(signs, codes, d, X, G)
        check_close(Yg, Y, A, what)


# ---------------------------------------------------------------------------
# HIP graph replay: the calls captured once and replayed give the eager
# results, replay after replay, with eager work between the replays (the
# head's workspace counters reset themselves in the launch that completes the
# argmax, so consecutive replays start from a clean workspace).

def test_graph_replay_matches_eager_and_oracle():
    rng = np.random.default_rng(31)
    N, NH, K, P, M = 2048, 8192, 4096, 3, 16
    codes, scales = synth.int4_weights(rng, N, K)
    signs, alpha = synth.binplane_weights(rng, N, K, P=P)
    hc, hs = synth.int4_weights(rng, NH, K)
    X = synth.activations(rng, M, K)
    rows = synth.plant_rows(rng, hc, hs, X)
    w4 = dev(svq.pack_int4_grouped(codes, scales))
    bp = dev(svq.pack_binary_planes(signs, alpha))
    hb = dev(svq.pack_int4_grouped(hc, hs))
    Xd = dev(X)
    draft = torch.from_numpy(rows[:-1].astype(np.int32)).cuda()
    draft[5] = (draft[5] + 1) % NH  # the sixth drafted token is rejected: tau = 6
    ws = torch.zeros(svq.lmhead_workspace_bytes(M), dtype=torch.uint8, device="cuda")

    def outputs():
        return {"y1": torch.empty(N, dtype=torch.int16, device="cuda"),
                "p1": torch.empty(N, dtype=torch.int16, device="cuda"),
                "Y": torch.empty((M, N), dtype=torch.int16, device="cuda"),
                "PY": torch.empty((M, N), dtype=torch.int16, device="cuda"),
                "idx": torch.empty(M, dtype=torch.int32, device="cuda"),
                "mx": torch.empty(M, dtype=torch.float32, device="cuda"),
                "vidx": torch.empty(M, dtype=torch.int32, device="cuda"),
                "vmx": torch.empty(M, dtype=torch.float32, device="cuda"),
                "tau": torch.empty(1, dtype=torch.int32, device="cuda")}

    def run(o):
        svq.gemv_w4a16(w4, Xd[0], o["y1"], N, K)
        svq.gemv_binplane(bp, Xd[0], o["p1"], N, K, P)
        svq.gemm_smallm_w4a16(w4, Xd, o["Y"], M, N, K)
        svq.gemm_smallm_binplane(bp, Xd, o["PY"], M, N, K, P)
        svq.lmhead_argmax(hb, Xd, M, NH, K, o["idx"], o["mx"], ws)
        svq.lmhead_verify_greedy(hb, Xd, M, NH, K, draft, o["vidx"], o["vmx"], o["tau"], ws)

    eager = outputs()
    run(eager)
    torch.cuda.synchronize()
    ref = {k: v.cpu() for k, v in eager.items()}

    # The eager results against the oracle first.
    y, a = oracle.linear_w4a16(codes, scales, X[:1])
    check_close(ref["y1"].view(torch.bfloat16).double().numpy(), y[0], a[0], "gemv_w4a16")
    y, a = oracle.linear_binplane(signs, alpha, X[:1])
    check_close(ref["p1"].view(torch.bfloat16).double().numpy(), y[0], a[0], "gemv_binplane")
    y, a = oracle.linear_w4a16(codes, scales, X)
    check_close(ref["Y"].view(torch.bfloat16).double().numpy(), y, a, "gemm_w4a16")
    y, a = oracle.linear_binplane(signs, alpha, X)
    check_close(ref["PY"].view(torch.bfloat16).double().numpy(), y, a, "gemm_binplane")
    rh = oracle.argmax_w4a16(hc, hs, X)
    assert np.array_equal(rh["idx"], rows.astype(np.int32))
    assert np.array_equal(ref["idx"].numpy(), rows.astype(np.int32))
    assert np.array_equal(ref["vidx"].numpy(), rows.astype(np.int32))
    want = oracle.verify_greedy(rows.astype(np.int32), draft.cpu().numpy())
    assert want == 6 and int(ref["tau"][0]) == want
    check_close(ref["mx"].double().numpy(), rh["zmax"], rh["amax"], "maxlogit")

    graph_out = outputs()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(graph_out)
    torch.cuda.synchronize()
    other = outputs()
    for rep in range(4):
        for v in graph_out.values():
            v.fill_(-1)  # a fill kernel, not a memset node: outside the graph
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in graph_out.items():
            assert torch.equal(v.cpu(), ref[k]), f"replay {rep}: {k} differs from the eager result"
        run(other)  # eager work on the same workspace between replays
        torch.cuda.synchronize()
        for k, v in other.items():
            assert torch.equal(v.cpu(), ref[k]), f"eager after replay {rep}: {k} differs"
    del graph
