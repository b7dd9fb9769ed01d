"""The C-ABI library loads, exports every symbol include/svq.h declares, and
rejects bad arguments before touching a device (no GPU needed)."""
import ctypes
import os
import re

import pytest
import torch

import speculative_verify_amd as svq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "svq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["pack_int4_grouped", "pack_binary_planes", "gemv_w4a16", "gemv_binplane",
                 "gemm_smallm_w4a16", "gemm_smallm_binplane", "lmhead_argmax", "lmhead_verify_greedy",
                 "verify_greedy", "svq_last_error", "pack_sa", "gemv_sa", "gemm_smallm_sa", "lmhead_argmax_noalloc"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(svq.lib_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_sizes():
    assert svq.int4_packed_bytes(12288, 4096) == 25165824 + 786432
    assert svq.binplane_packed_bytes(12288, 4096, 3) == 18874368 + 2359296
    assert svq.int4_packed_bytes(248320, 4096) == 508559360 + 15892480
    assert svq.int4_packed_bytes(32768, 4096) == 69206016 - 2097152 + 2097152  # 67108864 + 2097152
    assert svq.lmhead_workspace_bytes(16) >= 16 * 8 and svq.lmhead_workspace_bytes(17) == 0
    # sa at P = 3: signs + 3 code bytes per (row, 128 weights) + one fp16 d per (row, 256 weights)
    assert svq.sa_packed_bytes(12288, 4096, 3, 128) == 18874368 + 3 * 12288 * 32 + 12288 * 16 * 2
    assert svq.sa_packed_bytes(12288, 4096, 3, 64) == 18874368 + 3 * 12288 * 64 + 12288 * 16 * 2
    assert svq.sa_packed_bytes(12288, 4096, 3, 256) == 18874368 + 3 * 12288 * 16 + 12288 * 16 * 2


A = 0x100000  # an aligned address that is never dereferenced: validation fails first


@pytest.mark.parametrize("call,code", [
    (lambda l: l.gemv_w4a16(None, A, A, 16, 128, 128, None), -1),
    (lambda l: l.gemv_w4a16(A, A, A, 0, 128, 128, None), -2),
    (lambda l: l.gemv_w4a16(A, A, A, 16, 100, 128, None), -2),
    (lambda l: l.gemv_w4a16(A, A, A, 16, 128 * 65, 128, None), -2),
    (lambda l: l.gemv_w4a16(A, A, A, 16, 128, 64, None), -2),
    (lambda l: l.gemv_w4a16(A + 8, A, A, 16, 128, 128, None), -3),
    (lambda l: l.gemv_w4a16(A, A + 4, A, 16, 128, 128, None), -3),
    (lambda l: l.gemv_w4a16(A, A, A + 1, 16, 128, 128, None), -3),
    (lambda l: l.gemv_binplane(A, A, A, 16, 128, 128, 0, None), -2),
    (lambda l: l.gemv_binplane(A, A, A, 16, 128, 128, 7, None), -2),
    (lambda l: l.gemm_smallm_w4a16(A, A, A, 0, 16, 128, 128, None), -2),
    (lambda l: l.gemm_smallm_w4a16(A, A, A, 65537, 16, 128, 128, None), -2),
    (lambda l: l.gemm_smallm_binplane(A, A, A, 65537, 16, 128, 128, 3, None), -2),
    (lambda l: l.gemm_smallm_binplane(A, A, A, 4, 16, 128, 128, 0, None), -2),
    (lambda l: l.lmhead_argmax(A, A, 2, 16, 128, 128, None, A, A, None, 0, None), -5),
    (lambda l: l.lmhead_argmax(A, A, 2, 16, 128, 128, None, A, A, A, 8, None), -5),
    (lambda l: l.lmhead_argmax(A, A, 2, 16, 128, 128, None, A, None, A, 1 << 20, None), -1),
    (lambda l: l.lmhead_argmax(A, A, 2, 16, 128, 128, A + 2, A, A, A, 1 << 20, None), -3),
    (lambda l: l.verify_greedy(None, A, 2, A, None), -1),
    (lambda l: l.verify_greedy(A, None, 2, A, None), -1),
    (lambda l: l.verify_greedy(A, A, 0, A, None), -2),
    (lambda l: l.verify_greedy(A, A, 17, A, None), -2),
    (lambda l: l.verify_greedy(A + 2, A, 2, A, None), -3),
    (lambda l: l.lmhead_verify_greedy(A, A, 2, 16, 128, 128, None, A, A, A, None, A, 1 << 20, None), -1),
    (lambda l: l.lmhead_verify_greedy(A, A, 2, 16, 128, 128, None, None, A, A, A, A, 1 << 20, None), -1),
    (lambda l: l.lmhead_verify_greedy(A, A, 2, 16, 128, 128, None, A, A, A, A, None, 0, None), -5),
    (lambda l: l.lmhead_argmax_binplane(A, A, 2, 16, 128, 128, 0, None, A, A, A, 1 << 20, None), -2),
    (lambda l: l.lmhead_argmax_binplane(A, A, 2, 16, 128, 128, 7, None, A, A, A, 1 << 20, None), -2),
    (lambda l: l.lmhead_argmax_binplane(A, A, 2, 16, 128, 128, 3, None, A, A, None, 0, None), -5),
    (lambda l: l.gemv_sa(None, A, A, 16, 256, 128, 3, None), -1),
    (lambda l: l.gemv_sa(A, A, A, 16, 384, 128, 3, None), -2),
    (lambda l: l.gemv_sa(A, A, A, 16, 256, 32, 3, None), -2),
    (lambda l: l.gemv_sa(A, A, A, 16, 256, 128, 1, None), -2),
    (lambda l: l.gemv_sa(A, A, A, 16, 256, 128, 7, None), -2),
    (lambda l: l.gemv_sa(A, A, A, 16, 256 * 33, 128, 3, None), -2),
    (lambda l: l.gemv_sa(A + 8, A, A, 16, 256, 128, 3, None), -3),
    (lambda l: l.gemm_smallm_sa(A, A, A, 65537, 16, 256, 64, 2, None), -2),
    (lambda l: l.gemm_smallm_sa(A, A, A, 4, 16, 256, 512, 2, None), -2),
    (lambda l: l.gemm_smallm_sa(A, A + 2, A, 4, 16, 256, 256, 2, None), -3),
    (lambda l: l.lmhead_argmax_noalloc(A, A, 17, 16, 128, 128, None, A, A, None), -2),
    (lambda l: l.lmhead_argmax_noalloc(A, A, 0, 16, 128, 128, None, A, A, None), -2),
    (lambda l: l.lmhead_argmax_noalloc(A, A, 2, 16, 128, 128, None, A, None, None), -1),
    (lambda l: l.lmhead_argmax_noalloc(A, A, 2, 16, 128, 128, A + 2, A, A, None), -3),
    (lambda l: l.svq_stream_read(A, 100, A, 0, None), -2),
    (lambda l: l.svq_stream_read(A, 1024, A, 9, None), -2),
])
def test_argument_validation(call, code):
    lib = svq.load()
    assert call(lib) == code
    assert lib.svq_last_error().decode()


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the no-device error path")
def test_no_device_is_a_hip_error_not_a_crash():
    lib = svq.load()
    rc = lib.gemv_w4a16(A, A, A, 16, 128, 128, None)
    assert rc == -6
    assert "hip" in lib.svq_last_error().decode().lower()


# The Python binding checks every tensor's byte size against what the call
# reads or writes before anything reaches the library: an undersized tensor
# or a 1-byte dtype where 2-byte values are expected raises ValueError, and
# no launch happens (these are CPU tensors, which never reach a launch).
def _t(n, dtype=torch.int16):
    return torch.zeros(n, dtype=dtype)


N_, K_, P_ = 32, 256, 3


@pytest.mark.parametrize("what,call", [
    ("packed", lambda: svq.gemv_w4a16(_t(10, torch.uint8), _t(K_), _t(N_), N_, K_)),
    ("x", lambda: svq.gemv_w4a16(_t(svq.int4_packed_bytes(N_, K_), torch.uint8), _t(K_, torch.uint8), _t(N_),
                                 N_, K_)),
    ("y", lambda: svq.gemv_w4a16(_t(svq.int4_packed_bytes(N_, K_), torch.uint8), _t(K_), _t(N_ - 1), N_, K_)),
    ("packed", lambda: svq.gemv_binplane(_t(svq.binplane_packed_bytes(N_, K_, P_) - 1, torch.uint8), _t(K_),
                                         _t(N_), N_, K_, P_)),
    ("packed", lambda: svq.gemv_sa(_t(svq.sa_packed_bytes(N_, K_, P_) - 1, torch.uint8), _t(K_), _t(N_),
                                   N_, K_, P_)),
    ("X", lambda: svq.gemm_smallm_w4a16(_t(svq.int4_packed_bytes(N_, K_), torch.uint8), _t(16 * K_ - 1),
                                        _t(16 * N_), 16, N_, K_)),
    ("Y", lambda: svq.gemm_smallm_w4a16(_t(svq.int4_packed_bytes(N_, K_), torch.uint8), _t(16 * K_),
                                        _t(16 * N_, torch.uint8), 16, N_, K_)),
    ("Y", lambda: svq.gemm_smallm_binplane(_t(svq.binplane_packed_bytes(N_, K_, P_), torch.uint8), _t(40 * K_),
                                           _t(39 * N_), 40, N_, K_, P_)),
    ("X", lambda: svq.gemm_smallm_sa(_t(svq.sa_packed_bytes(N_, K_, P_), torch.uint8), _t(3 * K_), _t(4 * N_),
                                     4, N_, K_, P_)),
    ("argmax", lambda: svq.lmhead_argmax(_t(svq.int4_packed_bytes(N_, K_), torch.uint8), _t(4 * K_),
                                         4, N_, K_, _t(3, torch.int32), _t(4, torch.float32), _t(4352, torch.uint8))),
    ("maxlogit", lambda: svq.lmhead_argmax(_t(svq.int4_packed_bytes(N_, K_), torch.uint8), _t(4 * K_),
                                           4, N_, K_, _t(4, torch.int32), _t(4, torch.int16),
                                           _t(4352, torch.uint8))),
    ("row_ids", lambda: svq.lmhead_argmax(_t(svq.int4_packed_bytes(N_, K_), torch.uint8), _t(4 * K_),
                                          4, N_, K_, _t(4, torch.int32), _t(4, torch.float32),
                                          _t(4352, torch.uint8), row_ids=_t(N_ - 1, torch.int32))),
    ("packed", lambda: svq.lmhead_argmax_binplane(_t(100, torch.uint8), _t(K_), 1, N_, K_, P_,
                                                  _t(1, torch.int32), _t(1, torch.float32), _t(4352, torch.uint8))),
    ("draft_ids", lambda: svq.lmhead_verify_greedy(_t(svq.int4_packed_bytes(N_, K_), torch.uint8), _t(16 * K_),
                                                   16, N_, K_, _t(14, torch.int32), _t(16, torch.int32),
                                                   _t(16, torch.float32), _t(1, torch.int32),
                                                   _t(4352, torch.uint8))),
    ("accept_len", lambda: svq.lmhead_verify_greedy(_t(svq.int4_packed_bytes(N_, K_), torch.uint8), _t(16 * K_),
                                                    16, N_, K_, _t(15, torch.int32), _t(16, torch.int32),
                                                    _t(16, torch.float32), _t(0, torch.int32),
                                                    _t(4352, torch.uint8))),
    ("target_ids", lambda: svq.verify_greedy(_t(4, torch.int32), _t(4, torch.int32), 5, _t(1, torch.int32))),
    ("src", lambda: svq.svq_stream_read(_t(8, torch.uint8), 16, _t(8, torch.int32))),
])
def test_binding_rejects_undersized_tensors(what, call):
    with pytest.raises(ValueError, match=what):
        call()
