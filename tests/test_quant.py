"""The library's offline quantizers against the oracle (bit-exact codes,
signs and fp16 scales on seeded inputs), their argument checks, and the
quantize -> pack -> layer chain through the oracle's layer definitions."""
import numpy as np
import pytest

import oracle
import speculative_verify_amd as svq
from speculative_verify_amd import synth


def weights(rng, N, K, scale=0.02):
    return synth.f32_to_bf16_bits((rng.standard_normal((N, K)) * scale).astype(np.float32))


@pytest.mark.parametrize("N,K,G", [(1, 128, 128), (37, 512, 128), (16, 768, 64), (9, 1024, 256)])
def test_requant_matches_oracle(N, K, G):
    rng = np.random.default_rng(N + K + G)
    _, scales = synth.int4_weights(rng, N, K, G=G)
    scales[0, 0] = 0
    w = weights(rng, N, K, 0.05)
    w[:, 5] = 0x8000  # -0.0
    got = svq.quantize_int4_frozen(w, scales, G=G)
    assert np.array_equal(got, oracle.requant_int4(w, scales, G=G))


@pytest.mark.parametrize("N,K,G,P,iters", [(3, 128, 128, 1, 0), (5, 256, 64, 2, 3), (7, 512, 128, 3, 10),
                                           (4, 512, 256, 4, 10), (3, 256, 64, 6, 5), (2, 256, 128, 5, 40)])
def test_fit_matches_oracle(N, K, G, P, iters):
    rng = np.random.default_rng(N * 10 + K + G + P + iters)
    w = weights(rng, N, K)
    w[0, :G // 2] = 0                      # zeros: sign +1, and a group with repeated values
    w[1 % N, G:2 * G] = w[1 % N, 0]
    signs, alpha = svq.fit_binary_planes(w, P=P, G=G, iters=iters)
    os_, _, oa = oracle.fit_planes(w, P=P, G=G, iters=iters)
    assert np.array_equal(signs, os_)
    assert np.array_equal(alpha, oa)


def test_fit_thread_count_independent():
    rng = np.random.default_rng(3)
    w = weights(rng, 300, 256)
    a = svq.fit_binary_planes(w, P=3, G=128, iters=5)
    b = svq.fit_binary_planes(w[:70], P=3, G=128, iters=5)  # a different split over threads
    assert np.array_equal(a[0][:, :70], b[0]) and np.array_equal(a[1][:, :70], b[1])


@pytest.mark.parametrize("N,K,G,P", [(5, 256, 64, 2), (11, 512, 128, 3), (4, 1024, 256, 6)])
def test_snap_matches_oracle(N, K, G, P):
    rng = np.random.default_rng(N + K + G + P)
    _, alpha = synth.binplane_weights(rng, N, K, P=P, G=G)
    alpha[:, 0, :] = 0                      # an all-zero super-block: d = 0, codes 0
    codes, d = svq.snap_sa_scales(alpha, G=G)
    oc, od = oracle.snap_sa(alpha, G=G)
    assert np.array_equal(codes, oc) and np.array_equal(d, od)


def test_fit_then_snap_then_pack_is_a_valid_sa_layer():
    # The offline chain of the sa* storage: fit, snap, pack; the packed blob
    # unpacks to the fitted signs and snapped scales, and the sa layer stays
    # close to the unsnapped plane layer.
    rng = np.random.default_rng(5)
    N, K, P, G = 24, 512, 3, 64
    w = weights(rng, N, K)
    signs, alpha = svq.fit_binary_planes(w, P=P, G=G, iters=10)
    codes, d = svq.snap_sa_scales(alpha, G=G)
    blob = svq.pack_sa(signs, codes, d, G=G)
    s2, c2, d2 = svq.unpack_sa(blob, N, K, P, G=G)
    assert np.array_equal(s2, signs) and np.array_equal(c2, codes) and np.array_equal(d2, d)
    x = synth.activations(rng, 4, K)
    y_sa, a_sa = oracle.linear_sa(signs, codes, d, x, G=G)
    y_bp, _ = oracle.linear_binplane(signs, alpha, x, G=G)
    # each scale moves by at most half a code step: |d a - alpha| <= d / 2 <= max alpha / 510
    assert np.all(np.abs(y_sa - y_bp) <= a_sa * (1 / 255))


def test_quantizer_argument_checks():
    lib = svq.load()
    buf = np.zeros(1 << 16, np.uint8)
    A = buf.ctypes.data
    assert lib.quantize_int4_frozen(None, A, 1, 128, 128, A) == -1
    assert lib.quantize_int4_frozen(A, A, 1, 100, 128, A) == -2
    assert lib.quantize_int4_frozen(A, A, 1, 128, 32, A) == -2
    assert lib.fit_binary_planes(A, 1, 128, 128, 0, 1, A, A) == -2
    assert lib.fit_binary_planes(A, 1, 128, 128, 7, 1, A, A) == -2
    assert lib.fit_binary_planes(A, 1, 128, 128, 2, -1, A, A) == -2
    assert lib.fit_binary_planes(A, 0, 128, 128, 2, 1, A, A) == -2
    assert lib.snap_sa_scales(A, 1, 384, 128, 2, A, A) == -2
    neg = np.zeros((2, 1, 2), np.uint16)
    neg[1, 0, 1] = 0xBC00  # -1.0
    with pytest.raises(svq.SvqError) as e:
        svq.snap_sa_scales(neg, G=128)
    assert e.value.code == -4 and "p=1, n=0, g=1" in str(e.value)
