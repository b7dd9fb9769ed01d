"""Host packers of the C ABI against the oracle's element-wise layout
statement (bit-exact), plus round trips and range checks."""
import numpy as np
import pytest

import oracle
import speculative_verify_amd as svq
from speculative_verify_amd import synth
from conftest import read_golden_bytes


@pytest.mark.parametrize("N,K", [(1, 128), (16, 128), (17, 256), (45, 384), (64, 1024), (130, 512)])
def test_int4_pack_bit_exact_vs_oracle(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    codes, scales = synth.int4_weights(rng, N, K)
    blob = svq.pack_int4_grouped(codes, scales)
    assert blob.nbytes == svq.int4_packed_bytes(N, K)
    assert np.array_equal(blob, oracle.pack_int4(codes, scales))
    c2, s2 = svq.unpack_int4_grouped(blob, N, K)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


@pytest.mark.parametrize("N,K,P", [(1, 128, 1), (16, 128, 3), (19, 256, 2), (33, 512, 3), (40, 256, 6),
                                   (64, 384, 5), (17, 128, 4)])
def test_binplane_pack_bit_exact_vs_oracle(N, K, P):
    rng = np.random.default_rng(N * 1000 + K + P)
    signs, alpha = synth.binplane_weights(rng, N, K, P=P)
    blob = svq.pack_binary_planes(signs, alpha)
    assert blob.nbytes == svq.binplane_packed_bytes(N, K, P)
    assert np.array_equal(blob, oracle.pack_binplane(signs, alpha))
    s2, a2 = svq.unpack_binary_planes(blob, N, K, P)
    assert np.array_equal(s2, signs) and np.array_equal(a2, alpha)


@pytest.mark.parametrize("N,K,P,G", [(1, 256, 2, 64), (16, 256, 3, 128), (19, 512, 2, 256), (33, 768, 6, 64),
                                     (40, 1024, 5, 128), (17, 512, 4, 256), (64, 256, 3, 64)])
def test_sa_pack_bit_exact_vs_oracle(N, K, P, G):
    rng = np.random.default_rng(N * 1000 + K + P + G)
    signs, codes, d = synth.sa_weights(rng, N, K, P, G)
    blob = svq.pack_sa(signs, codes, d, G=G)
    assert blob.nbytes == svq.sa_packed_bytes(N, K, P, G)
    assert np.array_equal(blob, oracle.pack_sa(signs, codes, d, G=G))
    s2, c2, d2 = svq.unpack_sa(blob, N, K, P, G=G)
    assert np.array_equal(s2, signs) and np.array_equal(c2, codes) and np.array_equal(d2, d)


def test_sa_pack_rejects_bad_arguments():
    lib = svq.load()
    buf = np.zeros(1 << 16, np.uint8)
    s = np.ones((2, 1, 512), np.int8)
    c = np.zeros((2, 1, 8), np.uint8)
    d = np.zeros((1, 2), np.uint16)
    assert lib.pack_sa(s.ctypes.data, c.ctypes.data, d.ctypes.data, 1, 384, 128, 2, buf.ctypes.data) == -2
    assert lib.pack_sa(s.ctypes.data, c.ctypes.data, d.ctypes.data, 1, 512, 32, 2, buf.ctypes.data) == -2
    assert lib.pack_sa(s.ctypes.data, c.ctypes.data, d.ctypes.data, 1, 512, 64, 1, buf.ctypes.data) == -2
    assert lib.pack_sa(s.ctypes.data, c.ctypes.data, d.ctypes.data, 1, 512, 64, 7, buf.ctypes.data) == -2
    assert lib.pack_sa(s.ctypes.data, None, d.ctypes.data, 1, 512, 64, 2, buf.ctypes.data) == -1
    s[1, 0, 300] = 2
    with pytest.raises(svq.SvqError) as e:
        svq.pack_sa(s, c, d, G=64)
    assert e.value.code == -4 and "p=1, n=0, k=300" in str(e.value)
    assert svq.sa_packed_bytes(1, 384, 2, 128) == 0 and svq.sa_packed_bytes(1, 512, 1, 128) == 0


def test_golden_blobs():
    codes = ((np.arange(128) % 16) - 8).astype(np.int8)[None, :]
    blob = svq.pack_int4_grouped(codes, np.array([[0x3F80]], np.uint16))
    assert blob.tobytes() == read_golden_bytes("int4_n1_k128.txt")
    signs = np.ones((2, 1, 128), np.int8)
    signs[0, 0, [0, 1, 42, 127]] = -1
    signs[1, 0, 64] = -1
    blob = svq.pack_binary_planes(signs, np.array([[[0x3C00]], [[0x3800]]], np.uint16))
    assert blob.tobytes() == read_golden_bytes("binplane_n1_k128_p2.txt")
    signs = np.ones((2, 1, 512), np.int8)
    signs[0, 0, [0, 200, 300]] = -1
    signs[1, 0, [129, 511]] = -1
    codes = np.array([[[1, 2, 3, 255, 4, 0, 9, 10]], [[16, 0, 128, 7, 1, 1, 1, 1]]], np.uint8)
    blob = svq.pack_sa(signs, codes, np.array([[0x3C00, 0xC000]], np.uint16), G=64)
    assert blob.tobytes() == read_golden_bytes("sa_n1_k512_p2_g64.txt")


def test_every_code_value_at_every_tile_position_round_trips():
    # 16 rows x 256 k: each (row, k) slot sees all 16 code values across 16 packs.
    N, K = 16, 256
    scales = np.zeros((N, K // 128), np.uint16)
    base = (np.arange(N)[:, None] + np.arange(K)[None, :]) % 16
    for shift in range(16):
        codes = (((base + shift) % 16) - 8).astype(np.int8)
        blob = svq.pack_int4_grouped(codes, scales)
        assert np.array_equal(blob, oracle.pack_int4(codes, scales))
        assert np.array_equal(svq.unpack_int4_grouped(blob, N, K)[0], codes)


def test_every_sign_pattern_per_byte_round_trips():
    # Each group of 8 consecutive k of each row takes all 256 sign patterns.
    N, K, P = 16, 256, 1
    pats = np.arange(256, dtype=np.uint8)
    bits = np.unpackbits(pats[:, None], axis=1, bitorder="little")  # [256][8]
    flat = np.resize(bits, (N * K // 8, 8)).reshape(N, K)
    signs = (1 - 2 * flat.astype(np.int8))[None]
    alpha = np.zeros((P, N, K // 128), np.uint16)
    blob = svq.pack_binary_planes(signs, alpha)
    assert np.array_equal(blob, oracle.pack_binplane(signs, alpha))
    assert np.array_equal(svq.unpack_binary_planes(blob, N, K, P)[0], signs)


def test_pack_rejects_out_of_range_codes_and_signs():
    codes = np.zeros((3, 128), np.int8)
    codes[2, 77] = 8
    with pytest.raises(svq.SvqError) as e:
        svq.pack_int4_grouped(codes, np.zeros((3, 1), np.uint16))
    assert e.value.code == -4 and "n=2, k=77" in str(e.value)
    signs = np.ones((2, 3, 128), np.int8)
    signs[1, 0, 5] = 0
    with pytest.raises(svq.SvqError) as e:
        svq.pack_binary_planes(signs, np.zeros((2, 3, 1), np.uint16))
    assert e.value.code == -4 and "p=1, n=0, k=5" in str(e.value)


def test_pack_rejects_bad_shapes():
    lib = svq.load()
    buf = np.zeros(4096, np.uint8)
    c = np.zeros((1, 192), np.int8)
    s = np.zeros((1, 2), np.uint16)
    assert lib.pack_int4_grouped(c.ctypes.data, s.ctypes.data, 1, 192, 128, buf.ctypes.data) == -2
    assert lib.pack_int4_grouped(c.ctypes.data, s.ctypes.data, 1, 128, 64, buf.ctypes.data) == -2
    assert lib.pack_int4_grouped(None, s.ctypes.data, 1, 128, 128, buf.ctypes.data) == -1
    assert lib.pack_binary_planes(c.ctypes.data, s.ctypes.data, 1, 128, 128, 7, buf.ctypes.data) == -2
    assert svq.int4_packed_bytes(0, 128) == 0 and svq.binplane_packed_bytes(5, 128, 0) == 0
