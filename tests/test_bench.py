"""bench.py's host-side contract (no GPU): the refusal of more than one GPU
and the algorithmic byte counts its GB/s figures divide by."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2" in r.stderr and "one GPU" in r.stderr
    assert r.stdout == ""


def test_linear_bytes_count_codes_scales_activations_and_outputs():
    # K = 4096, groups of 128: 0.5 B per INT4 code, a bf16 scale per (row,
    # group), bf16 x in and y out.
    assert bench.alg_bytes_linear("w4a16", 1, 12288) == 12288 * 2048 + 12288 * 32 * 2 + 4096 * 2 + 12288 * 2
    assert bench.alg_bytes_linear("w4a16", 1, 12288) == 25_985_024
    assert bench.alg_bytes_linear("w4a16", 16, 4096) == 8_912_896
    assert bench.alg_bytes_linear("w4a16", 16, 12288) == 26_476_544
    # P sign bits per weight and an fp16 alpha per (plane, row, group).
    assert bench.alg_bytes_linear("binplane", 1, 12288, 3) == 21_266_432
    assert bench.alg_bytes_linear("binplane", 16, 4096, 3) == 7_340_032
    assert bench.alg_bytes_linear("binplane", 16, 12288, 3) == 21_757_952


def test_head_bytes_replace_the_output_by_index_and_max():
    assert bench.alg_bytes_head(1, 32768) == 69_214_216
    assert bench.alg_bytes_head(16, 32768) == 69_337_216
    assert bench.alg_bytes_head(1, 248320) == 524_460_040
    assert bench.alg_bytes_head(16, 248320) == 524_583_040
    # The sign-plane head: P bits per weight and an fp16 alpha per (plane,
    # row, group) instead of the nibble and the bf16 scale.
    assert bench.alg_bytes_head_binplane(1, 32768, 3) == 32768 * 512 * 3 + 3 * 32768 * 32 * 2 + 8192 + 8
    # No logits are stored: the fused head moves M * N * 4 bytes less than
    # a mat-mul writing fp32 logits would.
    assert bench.alg_bytes_head(16, 248320) < bench.alg_bytes_linear("w4a16", 16, 248320)


def test_sa_bytes_count_code_bytes_and_superblock_scales():
    # 3 sign planes (18,874,368 B), one u8 code per (plane, row, group of G),
    # one fp16 d per (row, 256 weights), x and y.
    signs = 12288 * 4096 // 8 * 3
    assert bench.alg_bytes_sa(1, 12288, 3, 128) == signs + 3 * 12288 * 32 + 12288 * 16 * 2 + 8192 + 24576
    assert bench.alg_bytes_sa(1, 12288, 3, 128) == 20_480_000
    assert bench.alg_bytes_sa(1, 12288, 3, 64) - bench.alg_bytes_sa(1, 12288, 3, 128) == 3 * 12288 * 32
    # Cheaper than the fp16-alpha storage at G = 128 (one byte per alpha
    # instead of two, plus the shared d).
    assert bench.alg_bytes_sa(16, 12288, 3, 128) < bench.alg_bytes_linear("binplane", 16, 12288, 3)
