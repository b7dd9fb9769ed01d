"""Pins for the fp64 CPU oracle, against facts fixed outside the oracle itself.

Each test checks the oracle against a closed form, an invariant, a library
routine on a special case, or a hand-worked fixture, chosen so that a plausible
slip in the oracle (a dropped term, a wrong sign, a wrong group or k index, a
transposed operand, the wrong plane's scale) fails at least one of them.
"""
import numpy as np
import pytest
import torch

import oracle
from speculative_verify_amd import synth
from conftest import read_golden_bytes

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
BF16_ONE = 0x3F80
F16_ONE = 0x3C00


def onehot_x(K, k, value_bits=BF16_ONE):
    x = np.zeros((1, K), np.uint16)
    x[0, k] = value_bits
    return x


# ---- scalar decoders -------------------------------------------------------

def test_bf16_decode_matches_torch_for_every_pattern():
    ours = oracle.bf16_values(ALL16)
    ref = torch.from_numpy(ALL16.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_f16_decode_matches_numpy_for_every_pattern():
    ours = oracle.f16_values(ALL16)
    ref = ALL16.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero and the extreme subnormal / normal values
    assert oracle.f16_values(np.array([0x8000], np.uint16))[0] == 0.0
    assert np.signbit(oracle.f16_values(np.array([0x8000], np.uint16))[0])
    assert oracle.f16_values(np.array([0x0001], np.uint16))[0] == 2.0 ** -24
    assert oracle.f16_values(np.array([0x7BFF], np.uint16))[0] == 65504.0


# ---- W4A16 ------------------------------------------------------------------

def test_w4a16_onehot_selects_one_code_times_its_group_scale():
    rng = np.random.default_rng(1)
    N, K = 7, 384
    codes, scales = synth.int4_weights(rng, N, K)
    s = oracle.bf16_values(scales)
    for k in range(K):
        for vbits in (BF16_ONE, 0xBFC0):  # 1.0 and -1.5
            v = oracle.bf16_values(np.array([vbits], np.uint16))[0]
            y, a = oracle.linear_w4a16(codes, scales, onehot_x(K, k, vbits))
            want = v * s[:, k // 128] * codes[:, k].astype(np.float64)
            assert np.array_equal(y[0], want), k
            assert np.array_equal(a[0], np.abs(want)), k


def test_w4a16_unit_scales_reduce_to_integer_matmul():
    rng = np.random.default_rng(2)
    M, N, K = 3, 33, 512
    codes = rng.integers(-8, 8, size=(N, K), dtype=np.int8)
    scales = np.full((N, K // 128), BF16_ONE, np.uint16)
    xi = rng.integers(-3, 4, size=(M, K)).astype(np.int64)
    xbits = synth.f32_to_bf16_bits(xi.astype(np.float32))
    y, a = oracle.linear_w4a16(codes, scales, xbits)
    want = xi @ codes.astype(np.int64).T
    assert np.array_equal(y, want.astype(np.float64))
    assert np.array_equal(a, (np.abs(xi) @ np.abs(codes.astype(np.int64)).T).astype(np.float64))


def test_w4a16_sign_coherent_closed_form():
    rng = np.random.default_rng(3)
    N, K = 5, 512
    codes = np.full((N, K), 7, np.int8)
    _, scales = synth.int4_weights(rng, N, K)
    x = synth.f32_to_bf16_bits(np.abs(rng.standard_normal((1, K))).astype(np.float32) + 0.01)
    y, a = oracle.linear_w4a16(codes, scales, x)
    xv = oracle.bf16_values(x)[0]
    s = oracle.bf16_values(scales)
    want = np.array([sum(7.0 * s[n, g] * xv[g * 128:(g + 1) * 128].sum()
                         for g in range(K // 128)) for n in range(N)])
    assert np.allclose(y[0], want, rtol=1e-14, atol=0)
    assert np.array_equal(y, a)


def test_w4a16_additive_over_groups():
    rng = np.random.default_rng(4)
    M, N, K = 2, 9, 640
    codes, scales = synth.int4_weights(rng, N, K)
    x = synth.activations(rng, M, K)
    y, a = oracle.linear_w4a16(codes, scales, x)
    parts = np.zeros_like(y)
    for g in range(K // 128):
        sg = np.zeros_like(scales)
        sg[:, g] = scales[:, g]
        yg, _ = oracle.linear_w4a16(codes, sg, x)
        parts += yg
    assert np.allclose(parts, y, rtol=0, atol=1e-12 * a.max())
    assert np.all(a >= np.abs(y))


# ---- binary planes -----------------------------------------------------------

def test_binplane_single_unit_plane_is_a_signed_sum():
    rng = np.random.default_rng(5)
    M, N, K = 2, 17, 256
    signs, _ = synth.binplane_weights(rng, N, K, P=1)
    alpha = np.full((1, N, K // 128), F16_ONE, np.uint16)
    xi = rng.integers(-5, 6, size=(M, K)).astype(np.int64)
    y, a = oracle.linear_binplane(signs, alpha, synth.f32_to_bf16_bits(xi.astype(np.float32)))
    assert np.array_equal(y, (xi @ signs[0].astype(np.int64).T).astype(np.float64))
    assert np.array_equal(a, (np.abs(xi).sum(axis=1)[:, None] * np.ones((1, N))).astype(np.float64))


def test_binplane_onehot_is_sum_of_plane_scales_times_signs():
    rng = np.random.default_rng(6)
    N, K, P = 6, 256, 3
    signs, alpha = synth.binplane_weights(rng, N, K, P=P)
    al = oracle.f16_values(alpha)
    for k in range(K):
        y, a = oracle.linear_binplane(signs, alpha, onehot_x(K, k))
        want = sum(al[p, :, k // 128] * signs[p, :, k] for p in range(P))
        assert np.array_equal(y[0], want), k
        assert np.array_equal(a[0], np.abs(want)), k


def planes_from_odd_codes(codes):
    """Three sign planes with c = 4 b1 + 2 b2 + b3 for odd c in [-7, 7]."""
    c = codes.astype(np.int64)
    b1 = np.where(c > 0, 1, -1)
    r = c - 4 * b1
    b2 = np.where(r > 0, 1, -1)
    b3 = r - 2 * b2
    assert np.all(np.abs(b3) == 1)
    assert np.array_equal(4 * b1 + 2 * b2 + b3, c)
    return np.stack([b1, b2, b3]).astype(np.int8)


def test_three_planes_reproduce_odd_int4_codes():
    rng = np.random.default_rng(7)
    M, N, K = 3, 21, 512
    codes = (2 * rng.integers(-4, 4, size=(N, K)) + 1).astype(np.int8)  # odd in [-7, 7]
    _, scales = synth.int4_weights(rng, N, K)
    s = synth.bf16_bits_to_f32(scales)
    alpha = synth.f32_to_f16_bits(np.stack([4 * s, 2 * s, s]))
    # every bf16 scale in [0.005, 0.02] and its 2x, 4x are exact in fp16
    assert np.array_equal(oracle.f16_values(alpha), np.stack([4 * s, 2 * s, s]).astype(np.float64))
    x = synth.activations(rng, M, K)
    y4, a4 = oracle.linear_w4a16(codes, scales, x)
    yb, ab = oracle.linear_binplane(planes_from_odd_codes(codes), alpha, x)
    assert np.allclose(yb, y4, rtol=0, atol=1e-13 * a4.max())
    assert np.allclose(ab, a4, rtol=1e-14, atol=0)


# ---- sa* storage: u8 scale codes times one fp16 d per 256-weight super-block ----

def sa_alpha_exact(codes, d, G):
    """fp16 alpha[p][n][g] = d[n][g*G/256] * a[p][n][g], asserted exact in fp16
    (the pins below pick d so that it is)."""
    P, N, ng = codes.shape
    dv = oracle.f16_values(d)
    al = np.empty((P, N, ng), np.float64)
    for g in range(ng):
        al[:, :, g] = dv[None, :, (g * G) // 256] * codes[:, :, g].astype(np.float64)
    bits = synth.f32_to_f16_bits(al.astype(np.float32))
    assert np.array_equal(oracle.f16_values(bits), al)
    return bits


def exact_d(rng, N, K):
    """fp16 d values 2^e * (1 + j/4): times any u8 code they stay exact in fp16."""
    e = rng.integers(-14, -9, size=(N, K // 256))
    j = rng.integers(0, 4, size=(N, K // 256))
    return synth.f32_to_f16_bits((np.ldexp(1.0, e) * (1 + j / 4)).astype(np.float32))


@pytest.mark.parametrize("G", [64, 128, 256])
def test_sa_equals_plane_layer_with_alpha_d_times_code(G):
    rng = np.random.default_rng(20 + G)
    M, N, K, P = 3, 11, 768, 4
    signs, codes, _ = synth.sa_weights(rng, N, K, P, G)
    codes[:, 0, 0] = 0  # a zero code drops its plane's group
    codes[:, 1, :] = 255
    d = exact_d(rng, N, K)
    x = synth.activations(rng, M, K)
    y, a = oracle.linear_sa(signs, codes, d, x, G=G)
    yb, ab = oracle.linear_binplane(signs, sa_alpha_exact(codes, d, G), x, G=G)
    assert np.array_equal(y, yb)
    assert np.array_equal(a, ab)


def test_sa_hand_worked_example():
    signs = np.ones((2, 1, 512), np.int8)
    signs[0, 0, [0, 200, 300]] = -1
    signs[1, 0, [129, 511]] = -1
    codes = np.array([[[1, 2, 3, 255, 4, 0, 9, 10]], [[16, 0, 128, 7, 1, 1, 1, 1]]], np.uint8)
    d = np.array([[0x3C00, 0xC000]], np.uint16)  # fp16 1.0, -2.0
    x = np.full((1, 512), BF16_ONE, np.uint16)
    y, _ = oracle.linear_sa(signs, codes, d, x, G=64)
    assert y[0, 0] == 22164.0
    assert oracle.pack_sa(signs, codes, d, G=64).tobytes() == read_golden_bytes("sa_n1_k512_p2_g64.txt")


def test_sa_three_planes_with_codes_4_2_1_reproduce_odd_int4():
    # c = 4 b1 + 2 b2 + b3 for odd c, so codes (4, 2, 1) under d = s give s * c.
    rng = np.random.default_rng(27)
    M, N, K = 2, 13, 512
    codes4 = (2 * rng.integers(-4, 4, size=(N, K)) + 1).astype(np.int8)
    _, s_sb = synth.int4_weights(rng, N, K, G=256)      # one bf16 scale per super-block
    scales = np.repeat(s_sb, 2, axis=1)                   # the same scale on both 128-groups
    d = synth.f32_to_f16_bits(synth.bf16_bits_to_f32(s_sb))
    assert np.array_equal(oracle.f16_values(d), oracle.bf16_values(s_sb))
    sa_codes = np.empty((3, N, K // 128), np.uint8)
    sa_codes[0], sa_codes[1], sa_codes[2] = 4, 2, 1
    x = synth.activations(rng, M, K)
    y4, a4 = oracle.linear_w4a16(codes4, scales, x)
    ys, as_ = oracle.linear_sa(planes_from_odd_codes(codes4), sa_codes, d, x, G=128)
    assert np.allclose(ys, y4, rtol=0, atol=1e-13 * a4.max())
    assert np.allclose(as_, a4, rtol=1e-14, atol=0)


def test_sa_group_size_reductions():
    # Equal codes on the two halves of a group make G = 64 the G = 128 layer,
    # and equal codes on a super-block's two groups make G = 128 the G = 256 one.
    rng = np.random.default_rng(28)
    M, N, K, P = 2, 9, 1024, 3
    signs, c256, d = synth.sa_weights(rng, N, K, P, G=256)
    x = synth.activations(rng, M, K)
    y256, a256 = oracle.linear_sa(signs, c256, d, x, G=256)
    c128 = np.repeat(c256, 2, axis=2)
    y128, a128 = oracle.linear_sa(signs, c128, d, x, G=128)
    y64, a64 = oracle.linear_sa(signs, np.repeat(c128, 2, axis=2), d, x, G=64)
    for yy, aa in ((y128, a128), (y64, a64)):
        assert np.allclose(yy, y256, rtol=0, atol=1e-13 * a256.max())
        assert np.allclose(aa, a256, rtol=1e-13, atol=0)
    # ... and different codes on the halves change the result
    c64 = np.repeat(c128, 2, axis=2)
    c64[0, :, 1] = c64[0, :, 1] // 2
    y64b, _ = oracle.linear_sa(signs, c64, d, x, G=64)
    assert not np.allclose(y64b, y256, rtol=0, atol=1e-6 * a256.max())


@pytest.mark.parametrize("G", [64, 128, 256])
def test_sa_brute_force_dense_matmul(G):
    rng = np.random.default_rng(30 + G)
    M, N, K, P = 4, 7, 512, 5
    signs, codes, d = synth.sa_weights(rng, N, K, P, G)
    x = synth.activations(rng, M, K)
    dv = ALL16.view(np.float16).astype(np.float64)[d]          # numpy's own fp16 decode
    xv = x.astype(np.uint32) << 16
    xv = xv.view(np.float32).astype(np.float64)
    k = np.arange(K)
    W = np.zeros((N, K))
    for p in range(P):
        W += dv[:, k // 256] * codes[p][:, k // G].astype(np.float64) * signs[p].astype(np.float64)
    want = xv @ W.T
    y, a = oracle.linear_sa(signs, codes, d, x, G=G)
    assert np.allclose(y, want, rtol=0, atol=1e-12 * a.max())
    assert np.allclose(a, np.abs(xv) @ np.abs(W).T, rtol=1e-12, atol=0)


def test_sa_pack_places_every_code_and_d_in_its_own_slot():
    N, K, P, G = 18, 512, 2, 64
    signs = np.ones((P, N, K), np.int8)
    sign_bytes = 32 * (K // 8) * P
    codes = np.zeros((P, N, K // G), np.uint8)
    d = np.zeros((N, K // 256), np.uint16)
    assert not np.any(oracle.pack_sa(signs, codes, d, G=G))
    seen = set()
    for p in range(P):
        for n in range(N):
            for g in range(K // G):
                c = codes.copy()
                c[p, n, g] = 0xA5
                nz = np.flatnonzero(oracle.pack_sa(signs, c, d, G=G))
                assert len(nz) == 1 and nz[0] >= sign_bytes
                seen.add(int(nz[0]))
    for n in range(N):
        for j in range(K // 256):
            dd = d.copy()
            dd[n, j] = 0x1234
            blob = oracle.pack_sa(signs, codes, dd, G=G)
            nz = np.flatnonzero(blob)
            assert len(nz) == 2 and nz[1] == nz[0] + 1 and nz[0] % 2 == 0
            assert blob[nz[0]] == 0x34 and blob[nz[1]] == 0x12
            seen.add(int(nz[0]))
    assert len(seen) == P * N * (K // G) + N * (K // 256)


# ---- offline quantizers ------------------------------------------------------

def test_f16_encode_rounds_like_numpy_at_every_midpoint():
    # Every finite positive fp16 value, the midpoints between neighbours (ties
    # to even) and points just beside them: numpy's float64 -> float16 cast is
    # correctly rounded.
    finite = ALL16[(ALL16 & 0x7C00) != 0x7C00].view(np.float16).astype(np.float64)
    pos = np.unique(finite[finite >= 0])
    mids = (pos[:-1] + pos[1:]) / 2
    v = np.concatenate([pos, mids, np.nextafter(mids, 0), np.nextafter(mids, 1), [65519.0, 65520.0, 1e6]])
    v = np.concatenate([v, -v])
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f16_bits(v), want)


def test_requant_round_trips_dequantized_codes():
    # bf16(s * c) is within 2^-9 |c| of s * c, so rounding w / s returns c.
    rng = np.random.default_rng(40)
    N, K = 8, 512
    codes = np.tile(np.arange(-8, 8, dtype=np.int8), (N, K // 16))
    rng.shuffle(codes, axis=1)
    _, scales = synth.int4_weights(rng, N, K)
    s = synth.bf16_bits_to_f32(scales)
    w = synth.f32_to_bf16_bits(np.repeat(s, 128, axis=1) * codes.astype(np.float32))
    assert np.array_equal(oracle.requant_int4(w, scales), codes)


def test_requant_is_the_nearest_grid_point():
    # Brute force over the 16 grid points (ties to the even code), including
    # weights far outside the grid (clamped to its ends) and zero scales.
    rng = np.random.default_rng(41)
    N, K = 6, 256
    _, scales = synth.int4_weights(rng, N, K)
    scales[2, 1] = 0
    s = oracle.bf16_values(scales)
    w = synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.15).astype(np.float32))
    wv = oracle.bf16_values(w)
    got = oracle.requant_int4(w, scales)
    grid = np.arange(-8, 8)
    for n in range(N):
        for k in range(K):
            sv = s[n, k // 128]
            if sv == 0:
                assert got[n, k] == 0
                continue
            dist = np.abs(wv[n, k] - sv * grid)
            best = grid[dist == dist.min()]
            want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
            assert got[n, k] == want, (n, k)


def test_requant_half_way_goes_to_the_even_code():
    s = np.full((1, 1), 0x3C80, np.uint16)      # bf16 2^-6
    c = np.arange(-8, 7)
    w = synth.f32_to_bf16_bits(((c + 0.5) * 2.0 ** -6).astype(np.float32))[None, :]
    w = np.pad(w, ((0, 0), (0, 128 - w.shape[1])))
    got = oracle.requant_int4(w, s)[0, :len(c)]
    assert np.array_equal(got, np.where(c % 2 == 0, c, c + 1))


@pytest.mark.parametrize("iters", [0, 3])
def test_fit_one_plane_is_mean_abs_and_sign(iters):
    rng = np.random.default_rng(42)
    N, K = 5, 256
    w = synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    w[0, :3] = 0
    wv = oracle.bf16_values(w)
    signs, a64, a16 = oracle.fit_planes(w, P=1, G=128, iters=iters)
    assert np.array_equal(signs[0], np.where(wv < 0, -1, 1))
    want = np.abs(wv).reshape(N, 2, 128).mean(axis=2)
    assert np.allclose(a64[0], want, rtol=1e-15, atol=0)
    assert np.array_equal(a16[0], want.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("iters", [0, 5])
def test_fit_recovers_exact_superincreasing_planes(iters):
    # w = 2^-3 b1 + 2^-4 b2 + 2^-5 b3 (each alpha above the sum of the later
    # ones): the greedy pass already finds the signs (its mean-|r| scales are
    # biased by the planes' overlap), and the least-squares rounds then give
    # the scales exactly.
    rng = np.random.default_rng(43)
    N, K, P = 4, 384, 3
    b = np.where(rng.integers(0, 2, size=(P, N, K)) == 1, -1, 1).astype(np.int8)
    b[:, :, 0] = 1  # every group sees both signs of every plane below
    b[:, :, 1] = -1
    al = np.array([2.0 ** -3, 2.0 ** -4, 2.0 ** -5])
    wv = np.tensordot(al, b.astype(np.float64), axes=1)
    w = synth.f32_to_bf16_bits(wv.astype(np.float32))
    assert np.array_equal(oracle.bf16_values(w), wv)
    signs, a64, _ = oracle.fit_planes(w, P=P, G=128, iters=iters)
    assert np.array_equal(signs, b)
    want = np.broadcast_to(al[:, None, None], a64.shape)
    if iters == 0:
        # greedy: alpha_1 = mean |w| = 2^-3 + (overlap of plane 1 with 2, 3) / 128
        b64 = b.astype(np.float64)
        over = (al[1] * (b64[0] * b64[1]).reshape(N, 3, 128).sum(2)
                + al[2] * (b64[0] * b64[2]).reshape(N, 3, 128).sum(2)) / 128
        assert np.allclose(a64[0], al[0] + over, rtol=1e-15, atol=0)
        assert np.all(np.abs(a64 - want) < al[2])
    else:
        assert np.allclose(a64, want, rtol=1e-13, atol=0)


def fit_error(w, signs, a64, G):
    wv = oracle.bf16_values(w)
    P, N, K = signs.shape
    approx = np.zeros((N, K))
    for p in range(P):
        approx += np.repeat(a64[p], G, axis=1) * signs[p]
    return ((wv - approx) ** 2).reshape(N, K // G, G).sum(axis=2)


@pytest.mark.parametrize("P,G", [(2, 64), (3, 128), (4, 256)])
def test_fit_rounds_never_increase_the_error(P, G):
    rng = np.random.default_rng(44 + P)
    N, K = 6, 512
    w = synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    errs = [fit_error(w, *oracle.fit_planes(w, P=P, G=G, iters=it)[:2], G) for it in (0, 1, 2, 5, 20)]
    for a, b in zip(errs, errs[1:]):
        assert np.all(b <= a * (1 + 1e-12)), (P, G)
    # the greedy fit is rarely a fixed point already: most groups, and the total, improve
    assert np.mean(errs[-1] < errs[0] * (1 - 1e-9)) > 0.5 and errs[-1].sum() < errs[0].sum()


def test_fit_fixed_point_is_least_squares_and_nearest_codes():
    # After enough rounds the fit stops moving: alpha is the least-squares
    # solution for its signs (numpy lstsq) and every weight's sign vector is a
    # nearest one for that alpha (enumeration of all 2^P vectors).
    rng = np.random.default_rng(45)
    N, K, P, G = 3, 256, 3, 64
    w = synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    wv = oracle.bf16_values(w)
    signs, a64, _ = oracle.fit_planes(w, P=P, G=G, iters=60)
    s2, a2, _ = oracle.fit_planes(w, P=P, G=G, iters=61)
    assert np.array_equal(signs, s2) and np.allclose(a64, a2, rtol=1e-12, atol=0)
    combos = np.array([[1 - 2 * ((c >> p) & 1) for p in range(P)] for c in range(1 << P)])
    for n in range(N):
        for g in range(K // G):
            B = signs[:, n, g * G:(g + 1) * G].astype(np.float64)
            x = wv[n, g * G:(g + 1) * G]
            ls = np.linalg.lstsq(B.T, x, rcond=None)[0]
            assert np.allclose(np.abs(ls), a64[:, n, g], rtol=1e-9, atol=1e-15)
            vals = combos @ a64[:, n, g]
            for k in range(G):
                d = np.abs(x[k] - vals)
                assert abs(x[k] - B[:, k] @ a64[:, n, g]) <= d.min() * (1 + 1e-12) + 1e-18


def test_snap_recovers_codes_on_a_power_of_two_grid():
    # alpha = d0 * a0 with d0 a power of two and a0 reaching 255 in every
    # super-block: the snap returns exactly (a0, d0).
    rng = np.random.default_rng(46)
    P, N, K, G = 3, 5, 512, 64
    a0 = rng.integers(0, 256, size=(P, N, K // G)).astype(np.uint8)
    a0[0, :, 0] = 255
    a0[1, :, 4] = 255
    d0 = 2.0 ** -12
    alpha = synth.f32_to_f16_bits((a0.astype(np.float64) * d0).astype(np.float32))
    assert np.array_equal(oracle.f16_values(alpha), a0 * d0)
    codes, d = oracle.snap_sa(alpha, G=G)
    assert np.array_equal(codes, a0)
    assert np.all(oracle.f16_values(d) == d0)


def test_snap_error_is_at_most_half_a_step():
    rng = np.random.default_rng(47)
    P, N, K, G = 4, 7, 768, 128
    _, alpha = synth.binplane_weights(rng, N, K, P=P, G=G)
    codes, d = oracle.snap_sa(alpha, G=G)
    al = oracle.f16_values(alpha)
    dv = np.repeat(oracle.f16_values(d), 256 // G, axis=1)[None]
    err = np.abs(al - dv * codes)
    clamped = codes == 255
    assert np.all(err[~clamped] <= dv.repeat(P, 0)[~clamped] / 2 * (1 + 1e-12))
    # the largest scale of each super-block maps to 254 or 255
    top = codes.reshape(P, N, K // 256, 256 // G).max(axis=(0, 3))
    assert np.all(top >= 254)


# ---- greedy argmax -----------------------------------------------------------

def test_argmax_finds_planted_rows_with_closed_form_logit():
    case = synth.Case("t", "lmhead", 4, 300, 512)
    codes, scales, x, rows = synth.make_lmhead(case, seed=11)
    r = oracle.argmax_w4a16(codes, scales, x)
    assert np.array_equal(r["idx"], rows.astype(np.int32))
    xv = oracle.bf16_values(x)
    for m in range(case.M):
        s = oracle.bf16_values(scales[rows[m]])
        want = sum(s[g] * 7.0 * np.abs(xv[m, g * 128:(g + 1) * 128]).sum()
                   for g in range(case.K // 128))
        assert r["zmax"][m] == pytest.approx(want, rel=1e-14)
        assert r["amax"][m] == pytest.approx(want, rel=1e-14)
        assert r["zsecond"][m] < r["zmax"][m]


def test_binplane_argmax_finds_planted_rows_with_closed_form_logit():
    case = synth.Case("t", "lmhead", 3, 250, 384, P=3)
    signs, alpha, x, rows = synth.make_lmhead_binplane(case, seed=15)
    r = oracle.argmax_binplane(signs, alpha, x)
    assert np.array_equal(r["idx"], rows.astype(np.int32))
    xv = oracle.bf16_values(x)
    for m in range(case.M):
        want = 0.0
        for g in range(case.K // 128):
            sx = np.abs(xv[m, g * 128:(g + 1) * 128]).sum()
            want += sum(oracle.f16_values(alpha[p, rows[m], g:g + 1])[0] * sx for p in range(case.P))
        assert r["zmax"][m] == pytest.approx(want, rel=1e-14)
        assert r["zsecond"][m] < r["zmax"][m]


def test_argmax_ties_go_to_lowest_index_and_row_ids_map():
    case = synth.Case("t", "lmhead", 2, 64, 256)
    codes, scales, x, rows = synth.make_lmhead(case, seed=12)
    lo, hi = 3, 40
    for m in range(case.M):
        codes[[lo, hi]] = codes[rows[m]]
        scales[[lo, hi]] = scales[rows[m]]
        rid = (1000 + 7 * np.arange(case.N)).astype(np.int32)
        r = oracle.argmax_w4a16(codes, scales, x[m:m + 1], row_ids=rid)
        assert r["idx"][0] == min(lo, rows[m])
        assert r["out"][0] == rid[r["idx"][0]]
        assert r["zsecond"][0] == r["zmax"][0]


def test_argmax_agrees_with_first_occurrence_argmax_of_logits():
    rng = np.random.default_rng(13)
    M, N, K = 5, 97, 256
    codes, scales = synth.int4_weights(rng, N, K)
    x = synth.activations(rng, M, K)
    y, _ = oracle.linear_w4a16(codes, scales, x)
    r = oracle.argmax_w4a16(codes, scales, x)
    assert np.array_equal(r["idx"], np.argmax(y, axis=1).astype(np.int32))
    assert np.array_equal(r["zmax"], y.max(axis=1))


# ---- greedy acceptance ---------------------------------------------------------
# Hand-worked cases of the acceptance rule (DFlash summary sec. 4.1): the block
# is [anchor, d_1 .. d_{M-1}], target[j] predicts the token after row j, drafts
# are accepted in order while target[j] == d_{j+1}, and tau = accepted + 1.
VERIFY_CASES = [
    # (target, draft, tau, why)
    ([5], [], 1, "no drafts: only the target's own token"),
    ([7, 8, 9, 4], [7, 8, 9], 4, "every draft accepted, plus the bonus token t_3"),
    ([7, 8, 9, 4], [1, 8, 9], 1, "first draft rejected"),
    ([7, 8, 9, 4], [7, 2, 9], 2, "second draft rejected"),
    ([7, 8, 9, 4], [7, 8, 3], 3, "last draft rejected"),
    ([1, 2, 3], [9, 2], 1, "a later match after a rejection does not count"),
    ([-1, 5, 6], [0, 5], 1, "a row without a valid maximum ends the prefix"),
    ([3, -1, 6], [3, 0], 2, "... also after accepted drafts"),
    (list(range(16)), list(range(15)), 16, "full 16-row block accepted"),
]


@pytest.mark.parametrize("target,draft,tau,why", VERIFY_CASES)
def test_verify_greedy_hand_cases(target, draft, tau, why):
    assert oracle.verify_greedy(np.array(target), np.array(draft)) == tau, why


def test_verify_greedy_on_planted_head_blocks():
    # End to end: the planted rows fix the target tokens, so drafts copied from
    # them are accepted up to the first planted mismatch.
    case = synth.Case("t", "lmhead", 6, 200, 256)
    codes, scales, x, rows = synth.make_lmhead(case, seed=14)
    t = oracle.argmax_w4a16(codes, scales, x)["out"]
    assert np.array_equal(t, rows.astype(np.int32))
    for bad in range(case.M - 1):
        draft = t[:-1].copy()
        draft[bad] = (draft[bad] + 1) % case.N
        assert oracle.verify_greedy(t, draft) == bad + 1
    assert oracle.verify_greedy(t, t[:-1]) == case.M


# ---- packed layouts -----------------------------------------------------------

def test_int4_pack_matches_hand_worked_bytes():
    codes = ((np.arange(128) % 16) - 8).astype(np.int8)[None, :]
    scales = np.array([[BF16_ONE]], np.uint16)
    assert oracle.pack_int4(codes, scales).tobytes() == read_golden_bytes("int4_n1_k128.txt")


def test_binplane_pack_matches_hand_worked_bytes():
    signs = np.ones((2, 1, 128), np.int8)
    signs[0, 0, [0, 1, 42, 127]] = -1
    signs[1, 0, 64] = -1
    alpha = np.array([[[F16_ONE]], [[0x3800]]], np.uint16)
    got = oracle.pack_binplane(signs, alpha).tobytes()
    assert got == read_golden_bytes("binplane_n1_k128_p2.txt")


def test_int4_pack_places_every_code_in_its_own_nibble():
    N, K = 20, 256
    seen = {}
    scales = np.zeros((N, K // 128), np.uint16)
    code_bytes = ((N + 15) // 16 * 16) * K // 2
    base = oracle.pack_int4(np.full((N, K), -8, np.int8), scales)[:code_bytes]
    pad = base != 0  # padded rows hold code 0 (nibble 8)
    for n in range(N):
        for k in range(K):
            codes = np.full((N, K), -8, np.int8)
            codes[n, k] = 7
            blob = oracle.pack_int4(codes, scales)[:code_bytes]
            diff = np.flatnonzero(blob != base)
            assert len(diff) == 1
            nib = (int(blob[diff[0]]) >> 4, int(blob[diff[0]]) & 15)
            assert nib in ((15, 0), (0, 15))
            key = (int(diff[0]), nib)
            assert key not in seen
            seen[key] = (n, k)
    assert not np.any(pad[: 16 * K // 2 * (N // 16)])  # full tiles carry no padding


def test_binplane_pack_places_every_sign_in_its_own_bit():
    N, K, P = 18, 256, 2
    alpha = np.zeros((P, N, K // 128), np.uint16)
    nbytes = ((N + 15) // 16 * 16) * K // 8 * P
    seen = set()
    for p in range(P):
        for n in range(N):
            for k in range(K):
                signs = np.ones((P, N, K), np.int8)
                signs[p, n, k] = -1
                blob = oracle.pack_binplane(signs, alpha)[:nbytes]
                nz = np.flatnonzero(blob)
                assert len(nz) == 1 and bin(int(blob[nz[0]])).count("1") == 1
                key = (int(nz[0]), int(blob[nz[0]]))
                assert key not in seen
                seen.add(key)
    assert len(seen) == P * N * K
