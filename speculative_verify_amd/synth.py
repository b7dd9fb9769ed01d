"""Seeded synthetic inputs for the low-bit linear layers.

This module only draws random numbers and stores them in the bit formats the
layers consume (int8 codes/signs, bf16 scales, fp16 plane scales, bf16
activations).  It holds none of the layers' arithmetic, so both the CPU oracle
tests and the HIP tests/bench can use it.

Draw order for every case (numpy ``default_rng(seed)``, PCG64):
  1. INT4 codes ``integers(-8, 8)`` (uniform in [-8, 7])
     -- or sign bits ``integers(0, 2)`` per (plane, row, k), b = 1 - 2*bit;
  2. scales ``uniform(0.005, 0.02)`` per (row, group) rounded to bf16 (RNE)
     -- or alpha_1 ``uniform(0.01, 0.03)``, alpha_{p+1} = alpha_p *
     ``uniform(0.3, 0.6)`` per (row, group), each rounded to fp16 (RNE)
     -- or, for the sa* storage, u8 scale codes a_1 ``integers(128, 256)``,
     a_{p+1} = floor(a_p * ``uniform(0.3, 0.6)``) per (row, group), then
     one fp16 d ``uniform(6e-5, 2e-4)`` per (row, 256-weight super-block);
  3. activations ``standard_normal`` (float32) rounded to bf16 (RNE);
  4. planted head rows, if asked for: M distinct rows, uniform in [0, N).

The shapes stand in for the workloads the pages describe: hidden size
K = 4096, an MLP width N = 12288, a verify block of M = 16 drafted positions,
a full vocabulary of 248,320 rows and a trimmed head of 32,768 rows.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

GROUP = 128


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even), as bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f32_to_f16_bits(a) -> np.ndarray:
    """Round float32 values to IEEE binary16 (round-to-nearest-even), as bits."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def int4_weights(rng, N: int, K: int, G: int = GROUP, smin: float = 0.005,
                 smax: float = 0.02):
    """codes int8 [N][K] uniform in [-8, 7]; scales bf16 bits [N][K/G]."""
    codes = rng.integers(-8, 8, size=(N, K), dtype=np.int8)
    scales = f32_to_bf16_bits(rng.uniform(smin, smax, size=(N, K // G)).astype(np.float32))
    return codes, scales


def binplane_weights(rng, N: int, K: int, P: int = 3, G: int = GROUP,
                     a1=(0.01, 0.03), ratio=(0.3, 0.6)):
    """signs int8 [P][N][K] in {-1,+1} (Bernoulli 0.5); alpha fp16 bits [P][N][K/G]."""
    bits = rng.integers(0, 2, size=(P, N, K), dtype=np.int8)
    signs = (1 - 2 * bits).astype(np.int8)
    del bits
    ng = K // G
    alpha = np.empty((P, N, ng), np.float32)
    alpha[0] = rng.uniform(a1[0], a1[1], size=(N, ng))
    for p in range(1, P):
        alpha[p] = alpha[p - 1] * rng.uniform(ratio[0], ratio[1], size=(N, ng))
    return signs, f32_to_f16_bits(alpha)


def sa_weights(rng, N: int, K: int, P: int = 3, G: int = GROUP, a1=(128, 256),
               ratio=(0.3, 0.6), d_range=(6e-5, 2e-4)):
    """signs int8 [P][N][K] in {-1,+1}; u8 scale codes [P][N][K/G]; fp16 bits
    d [N][K/256].  Plane p+1's codes are plane p's times U(ratio), floored."""
    assert K % 256 == 0 and 256 % G == 0
    bits = rng.integers(0, 2, size=(P, N, K), dtype=np.int8)
    signs = (1 - 2 * bits).astype(np.int8)
    del bits
    ng = K // G
    codes = np.empty((P, N, ng), np.uint8)
    codes[0] = rng.integers(a1[0], a1[1], size=(N, ng))
    for p in range(1, P):
        codes[p] = np.floor(codes[p - 1] * rng.uniform(ratio[0], ratio[1], size=(N, ng)))
    d = f32_to_f16_bits(rng.uniform(d_range[0], d_range[1], size=(N, K // 256)).astype(np.float32))
    return signs, codes, d


def activations(rng, M: int, K: int) -> np.ndarray:
    """bf16 bits [M][K], x ~ N(0, 1)."""
    return f32_to_bf16_bits(rng.standard_normal(size=(M, K), dtype=np.float32))


def plant_rows(rng, codes: np.ndarray, scales: np.ndarray, x: np.ndarray,
               factor: float = 3.0) -> np.ndarray:
    """Plant one row per query so the head's argmax is unambiguous.

    For query m a row r_m is drawn (distinct, uniform in [0, N)); its codes
    become +7 where x[m][k] has a clear sign bit and -7 where it is set, and
    its scales become ``factor`` times the drawn ones (rounded to bf16).
    Edits ``codes``/``scales`` in place and returns the planted rows [M].
    """
    M = x.shape[0]
    N = codes.shape[0]
    rows = rng.choice(N, size=M, replace=False).astype(np.int64)
    for m in range(M):
        neg = (x[m] & 0x8000) != 0
        codes[rows[m]] = np.where(neg, -7, 7).astype(np.int8)
        scales[rows[m]] = f32_to_bf16_bits(factor * bf16_bits_to_f32(scales[rows[m]]))
    return rows


def plant_rows_binplane(rng, signs: np.ndarray, alpha: np.ndarray, x: np.ndarray,
                        factor: float = 3.0) -> np.ndarray:
    """Sign-plane counterpart of plant_rows: for query m a distinct row r_m gets
    b = +1 on every plane where x[m][k] has a clear sign bit and -1 where it is
    set, and its plane scales become ``factor`` times the drawn ones (fp16).
    Edits ``signs``/``alpha`` in place and returns the planted rows [M]."""
    M = x.shape[0]
    N = signs.shape[1]
    rows = rng.choice(N, size=M, replace=False).astype(np.int64)
    for m in range(M):
        neg = (x[m] & 0x8000) != 0
        signs[:, rows[m]] = np.where(neg, -1, 1).astype(np.int8)[None, :]
        a = alpha[:, rows[m]].astype(np.uint16).view(np.float16).astype(np.float32)
        alpha[:, rows[m]] = f32_to_f16_bits(factor * a)
    return rows


@dataclass(frozen=True)
class Case:
    """One synthetic workload shape."""
    name: str
    kind: str          # "w4a16" | "binplane" | "sa" | "lmhead"
    M: int
    N: int
    K: int
    P: int = 0
    G: int = GROUP

    @property
    def groups(self) -> int:
        return self.K // self.G


# The five workload shapes (the first is small enough for quick oracle runs).
TINY_W4A16 = Case("tiny_w4a16_m1_k256_n512", "w4a16", 1, 512, 256)
DECODE_W4A16 = Case("decode_w4a16_m1_k4096_n12288", "w4a16", 1, 12288, 4096)
DECODE_BINPLANE = Case("decode_binplane_p3_m1_k4096_n12288", "binplane", 1, 12288, 4096, P=3)
VERIFY_W4A16 = (Case("verify_w4a16_m16_k4096_n4096", "w4a16", 16, 4096, 4096),
                Case("verify_w4a16_m16_k4096_n12288", "w4a16", 16, 12288, 4096))
VERIFY_BINPLANE = (Case("verify_binplane_p3_m16_k4096_n4096", "binplane", 16, 4096, 4096, P=3),
                   Case("verify_binplane_p3_m16_k4096_n12288", "binplane", 16, 12288, 4096, P=3))
LMHEAD = (Case("lmhead_trim_m1_k4096_n32768", "lmhead", 1, 32768, 4096),
          Case("lmhead_trim_m16_k4096_n32768", "lmhead", 16, 32768, 4096),
          Case("lmhead_full_m1_k4096_n248320", "lmhead", 1, 248320, 4096),
          Case("lmhead_full_m16_k4096_n248320", "lmhead", 16, 248320, 4096))


def make_w4a16(case: Case, seed: int = 0):
    rng = np.random.default_rng(seed)
    codes, scales = int4_weights(rng, case.N, case.K, case.G)
    x = activations(rng, case.M, case.K)
    return codes, scales, x


def make_binplane(case: Case, seed: int = 0):
    rng = np.random.default_rng(seed)
    signs, alpha = binplane_weights(rng, case.N, case.K, case.P, case.G)
    x = activations(rng, case.M, case.K)
    return signs, alpha, x


def make_sa(case: Case, seed: int = 0):
    rng = np.random.default_rng(seed)
    signs, codes, d = sa_weights(rng, case.N, case.K, case.P, case.G)
    x = activations(rng, case.M, case.K)
    return signs, codes, d, x


def make_lmhead(case: Case, seed: int = 0):
    rng = np.random.default_rng(seed)
    codes, scales = int4_weights(rng, case.N, case.K, case.G)
    x = activations(rng, case.M, case.K)
    rows = plant_rows(rng, codes, scales, x)
    return codes, scales, x, rows


def make_lmhead_binplane(case: Case, seed: int = 0):
    rng = np.random.default_rng(seed)
    signs, alpha = binplane_weights(rng, case.N, case.K, case.P, case.G)
    x = activations(rng, case.M, case.K)
    rows = plant_rows_binplane(rng, signs, alpha, x)
    return signs, alpha, x, rows


def device_int4_blob(N: int, K: int, seed: int, G: int = GROUP, smin: float = 0.005,
                     smax: float = 0.02, device: str = "cuda"):
    """A packed INT4 blob drawn directly on the device (for timing runs).

    Uniform random code bytes give uniform nibbles, i.e. codes uniform in
    [-8, 7] whatever the byte layout; the scale section gets bf16 values
    uniform in [smin, smax].  Needs N % 16 == 0 (no padding rows) and K/G a
    multiple of 4 (no padded scale entries), so the sections are contiguous.
    """
    assert N % 16 == 0 and K % G == 0 and (K // G) % 4 == 0
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    code_bytes = N * K // 2
    blob = torch.empty(code_bytes + N * (K // G) * 2, dtype=torch.uint8, device=device)
    blob[:code_bytes] = torch.randint(0, 256, (code_bytes,), generator=gen, dtype=torch.uint8,
                                      device=device)
    s = torch.empty(N * (K // G), dtype=torch.float32, device=device).uniform_(smin, smax, generator=gen)
    blob[code_bytes:] = s.to(torch.bfloat16).view(torch.uint8)
    return blob


def device_binplane_blob(N: int, K: int, P: int, seed: int, G: int = GROUP, a1=(0.01, 0.03),
                         ratio=(0.3, 0.6), device: str = "cuda"):
    """A packed sign-plane blob drawn on the device: Bernoulli(0.5) sign bits,
    alpha_1 ~ U(a1), alpha_{p+1} = alpha_p * U(ratio), fp16.  N % 16 == 0 and
    (K/G) % 4 == 0, as for device_int4_blob."""
    assert N % 16 == 0 and K % G == 0 and (K // G) % 4 == 0
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    sign_bytes = N * K // 8 * P
    ng = K // G
    blob = torch.empty(sign_bytes + P * N * ng * 2, dtype=torch.uint8, device=device)
    blob[:sign_bytes] = torch.randint(0, 256, (sign_bytes,), generator=gen, dtype=torch.uint8,
                                      device=device)
    a = torch.empty((P, N * ng), dtype=torch.float32, device=device)
    a[0].uniform_(a1[0], a1[1], generator=gen)
    for p in range(1, P):
        a[p] = a[p - 1] * torch.empty(N * ng, device=device).uniform_(ratio[0], ratio[1], generator=gen)
    blob[sign_bytes:] = a.to(torch.float16).reshape(-1).view(torch.uint8)
    return blob


def device_sa_blob(N: int, K: int, P: int, G: int, seed: int, a1=(128, 256), ratio=(0.3, 0.6),
                   d_range=(6e-5, 2e-4), device: str = "cuda"):
    """A packed sa blob drawn on the device, with the distributions of
    sa_weights: Bernoulli(0.5) sign bits, u8 codes a_1 ~ U{a1}, a_{p+1} =
    floor(a_p * U(ratio)), fp16 d ~ U(d_range).  N % 16 == 0 and K/128 a
    multiple of 4, so the code and d rows carry no padding."""
    assert N % 16 == 0 and K % 512 == 0 and 256 % G == 0
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    sign_bytes = N * K // 8 * P
    ng, ns = K // G, K // 256
    blob = torch.empty(sign_bytes + P * N * ng + N * ns * 2, dtype=torch.uint8, device=device)
    blob[:sign_bytes] = torch.randint(0, 256, (sign_bytes,), generator=gen, dtype=torch.uint8, device=device)
    a = torch.empty((P, N * ng), dtype=torch.float32, device=device)
    a[0] = torch.randint(a1[0], a1[1], (N * ng,), generator=gen, device=device).float()
    for p in range(1, P):
        u = torch.empty(N * ng, device=device).uniform_(ratio[0], ratio[1], generator=gen)
        a[p] = torch.floor(a[p - 1] * u)
    blob[sign_bytes:sign_bytes + P * N * ng] = a.to(torch.uint8).reshape(-1)
    d = torch.empty(N * ns, dtype=torch.float32, device=device).uniform_(d_range[0], d_range[1], generator=gen)
    blob[sign_bytes + P * N * ng:] = d.to(torch.float16).view(torch.uint8)
    return blob


def device_activations(M: int, K: int, seed: int, device: str = "cuda"):
    """bf16 activations x ~ N(0, 1), [M][K], drawn on the device."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn((M, K), generator=gen, device=device).to(torch.bfloat16)
