"""Exhaustive device checks of the arithmetic the codec kernels use for their
shared-divisor divisions (each must give the same bits as the IEEE operation
it replaces):

* recip_rn, the hardware reciprocal plus one correction with the exact
  residual, against 1.0f / d for every normal fp32 d below 2^126, where 1/d
  is normal too (2^23 mantissas x 252 exponents);
* div_rn, RN(a * rh) plus one correction from the exact remainder, against
  a / d for every divisor mantissa and, by default, 64 slices of 1024
  consecutive numerator patterns spread over [1, 4) (5.5e11 quotients). With
  TQ_FULL_DIVISION_CHECK=1 it runs over every numerator pattern in [1, 4):
  all 1.4e14 quotients, about a minute on one MI355X.

* sqrt_rn_large, the hardware square root moved to a neighbour by the signs
  of exact residuals, against the IEEE square root for every x in
  [2^-96, 2^128) and +inf (the TQ3 norm clamps anything smaller to 1e-8).

Each check also counts the errors of the uncorrected step, to show that it
sees a wrong result."""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "randomized_hadamard_lloyd_amd", "libtqprobe.so")
ONE = 127 << 23          # bit pattern of 1.0f
SPAN_1_4 = 2 << 23       # patterns in [1, 4)


@pytest.fixture(scope="module")
def probe():
    lib = ctypes.CDLL(PROBE)
    lib.tqprobe_recip_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.tqprobe_sqrt_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.tqprobe_div_check.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32,
                                      ctypes.c_int, ctypes.c_void_p]
    return lib


def _stream():
    return torch.cuda.current_stream("cuda:0").cuda_stream


def test_recip_rn_matches_ieee_for_every_normal_divisor(probe):
    cnt = torch.zeros(3, dtype=torch.int64, device="cuda:0")
    assert probe.tqprobe_recip_check(cnt.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    total, bad, raw = cnt.cpu().tolist()
    assert total == 252 * (1 << 23)
    assert bad == 0, f"{bad} reciprocals differ from 1.0f / d"
    assert raw > 0


def _div_mismatches(probe, base, span, corrected):
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    assert probe.tqprobe_div_check(cnt.data_ptr(), base, span, corrected, _stream()) == 0
    torch.cuda.synchronize()
    return int(cnt.item())


def test_div_rn_matches_ieee(probe):
    if os.environ.get("TQ_FULL_DIVISION_CHECK") == "1":
        slices = [(ONE + s * (1 << 17), 1 << 17) for s in range(SPAN_1_4 >> 17)]
    else:
        step = SPAN_1_4 // 64
        slices = [(ONE + s * step + (s * 7919) % (step - 1024), 1024) for s in range(64)]
    for base, span in slices:
        bad = _div_mismatches(probe, base, span, 1)
        assert bad == 0, f"{bad} quotients differ from a / d for numerators {base:#x} + {span}"


def test_div_check_sees_the_uncorrected_product(probe):
    assert _div_mismatches(probe, ONE, 1024, 0) > 0


def test_sqrt_rn_large_matches_ieee(probe):
    cnt = torch.zeros(3, dtype=torch.int64, device="cuda:0")
    assert probe.tqprobe_sqrt_check(cnt.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    total, bad, raw = cnt.cpu().tolist()
    assert total == 224 * (1 << 23) + 1
    assert bad == 0, f"{bad} square roots differ from the IEEE result"
    assert raw > 0
