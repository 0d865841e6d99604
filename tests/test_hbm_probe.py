"""The HBM probe library (libhbm_probe.so) that bench.py's calibration mode
times: its argument checks on the host, and on the GPU that every kind moves
exactly the bytes it claims to (the ceilings it reports are only as good as
that)."""
import ctypes
import os

import pytest
# torch first: its HIP runtime and the one the probe library links share a
# soname, so whichever loads first serves both; loading the probe library
# first would hand torch a runtime other than the one it ships with
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBE = os.path.join(ROOT, "frame_wise_gated_amd", "libhbm_probe.so")


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(PROBE):
        pytest.fail(f"{PROBE} is missing: build it with `python -m frame_wise_gated_amd.build`")
    lib = ctypes.CDLL(PROBE)
    lib.hbm_probe.restype = ctypes.c_int
    lib.hbm_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                              ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("kind, src, dst, nbytes, blocks", [
    (6, 4096, 4096, 1 << 20, 32),        # no such kind
    (-1, 4096, 4096, 1 << 20, 32),
    (0, 4096, 4096, 100, 32),            # not a multiple of 16 bytes
    (2, 4104, 4096, 1 << 20, 32),        # misaligned source
    (2, 4096, 4104, 1 << 20, 32),        # misaligned destination
    (2, None, 4096, 1 << 20, 32),        # a copy needs a source
    (1, 4096, None, 1 << 20, 32),        # a write needs a destination
    (3, 4096, 4096, 1 << 20, 33),        # spans: bytes must be whole 32 KB steps per workgroup
    (5, 4096, 4096, (1 << 20) + 16, 32),
])
def test_probe_rejects_bad_arguments_before_any_launch(probe, kind, src, dst, nbytes, blocks):
    # fake addresses: the checks return before anything touches them
    assert probe.hbm_probe(kind, src, dst, nbytes, blocks, 0, None) == 1


@pytest.mark.gpu
@pytest.mark.parametrize("kind, nt", [(2, 0), (2, 1), (5, 0), (5, 1)])
def test_probe_copies_are_exact(probe, kind, nt):
    n = 1 << 20  # bytes: 32 workgroups x one 32 KB span each for kind 5
    src = torch.randint(0, 2**31 - 1, (n // 4,), dtype=torch.int32, device="cuda:0")
    dst = torch.zeros_like(src)
    st = torch.cuda.current_stream().cuda_stream
    assert probe.hbm_probe(kind, src.data_ptr(), dst.data_ptr(), n, 32, nt, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.gpu
@pytest.mark.parametrize("nt", [0, 1])
def test_probe_write_fills_its_pattern(probe, nt):
    n = 1 << 20
    dst = torch.zeros(n // 4, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    assert probe.hbm_probe(1, None, dst.data_ptr(), n, 32, nt, st) == 0
    torch.cuda.synchronize()
    v = 0x01234567
    want = torch.tensor([v, v ^ 1, v ^ 2, v ^ 3], dtype=torch.int32).repeat(n // 16)
    assert torch.equal(dst.cpu(), want)


@pytest.mark.gpu
@pytest.mark.parametrize("kind", [0, 3, 4])
def test_probe_reads_leave_the_sink_alone(probe, kind):
    # every word is the same, so the XOR the reads fold their data into is 0
    # and never the value that would make them store to the sink
    n = 1 << 20
    src = torch.full((n // 4,), 7, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    assert probe.hbm_probe(kind, src.data_ptr(), sink.data_ptr(), n, 32, 1, st) == 0
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
