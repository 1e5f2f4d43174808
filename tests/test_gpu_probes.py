"""The bfloat16 matrix-core instruction checked for exact integer block
sums: a small integer weight stored as bfloat16, times an int8 activation
code, summed over one 32-element block in fp32 from an fp32 start value,
must give the exact integer whenever every partial sum stays below 2^24 in
magnitude.  This is a property of the device that a bfloat16 form of the
integer block partials would rest on (no layer kernel uses that form); the
expected values are integer matrix products computed here."""

import ctypes
import os

import numpy as np
import pytest
import torch

from tests.gpu_common import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def probes():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    L = ctypes.CDLL(os.path.join(ROOT, "quantized_routed_expert_sigmoid_amd", "libcolibri_probes.so"))
    L.colibri_probe_mfma_bf16_block.argtypes = [ctypes.c_void_p] * 5
    return L


def _bf16_bits(v):
    """bfloat16 bit patterns of integer values that bfloat16 holds exactly."""
    f = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    assert np.all((f & 0xFFFF) == 0), "value not exact in bfloat16"
    return (f >> 16).astype(np.uint16)


def _mfma(probes, a, b, c):
    da = torch.from_numpy(_bf16_bits(a).view(np.int16)).cuda()
    db = torch.from_numpy(_bf16_bits(b).view(np.int16)).cuda()
    dc = torch.from_numpy(np.ascontiguousarray(c, dtype=np.float32)).cuda()
    dd = torch.empty(16, 16, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert probes.colibri_probe_mfma_bf16_block(da.data_ptr(), db.data_ptr(), dc.data_ptr(), dd.data_ptr(), st) == 0
    torch.cuda.synchronize()
    return dd.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("case", ["int4_offset", "int2_offset", "int8_extremes", "signed_int4_start"])
def test_bf16_mfma_block_sums_exact(probes, case):
    say(f"bf16 block sums case={case}")
    rng = np.random.default_rng(sum(map(ord, case)))
    for trial in range(8):
        x = rng.integers(-127, 128, size=(32, 16)).astype(np.int64)   # activation codes, K x tokens
        if trial == 0:
            x[:] = 127
        elif trial == 1:
            x[:] = -127
        if case in ("int4_offset", "int2_offset"):
            # weight w stored as 128 + (w + 2^(b-1)), the start value takes out
            # (128 + 2^(b-1)) times the token's code sum: the exact partial
            half = 8 if case == "int4_offset" else 2
            w = rng.integers(-half, half, size=(16, 32)).astype(np.int64)
            if trial == 0:
                w[:] = half - 1
            a = 128 + w + half
            c = np.broadcast_to(-(128 + half) * x.sum(axis=0), (16, 16)).astype(np.int64)
        elif case == "int8_extremes":
            w = rng.choice([-127, 127], size=(16, 32)).astype(np.int64)
            a, c = w, np.zeros((16, 16), np.int64)
        else:
            w = rng.integers(-8, 8, size=(16, 32)).astype(np.int64)
            a = w
            c = rng.integers(-(1 << 22), 1 << 22, size=(16, 16)).astype(np.int64)
        d = _mfma(probes, a, x, c)
        want = c + a @ x
        assert np.max(np.abs(want)) < (1 << 24)
        assert np.array_equal(d, want.astype(np.float64)), f"trial {trial}"
        if case in ("int4_offset", "int2_offset"):
            assert np.array_equal(d, (w @ x).astype(np.float64))
