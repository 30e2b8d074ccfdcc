"""Exhaustive device checks of arithmetic shortcuts the codec kernels rely on
(each must give the same bits as the IEEE operation it replaces).

recip_rn: the hardware reciprocal plus one correction with the exact
residual, against the IEEE quotient 1.0f / d, for every normal fp32 d below
2^126, where 1/d is normal too (2^23 mantissas x 252 exponents); the raw hardware reciprocal is
counted too, to show that the check sees a wrong result."""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "randomized_hadamard_lloyd_amd", "libtqprobe.so")


def test_recip_rn_matches_ieee_for_every_normal_divisor():
    lib = ctypes.CDLL(PROBE)
    lib.tqprobe_recip_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    cnt = torch.zeros(3, dtype=torch.int64, device="cuda:0")
    stream = torch.cuda.current_stream("cuda:0").cuda_stream
    assert lib.tqprobe_recip_check(cnt.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    total, bad, raw = cnt.cpu().tolist()
    assert total == 252 * (1 << 23)
    assert bad == 0, f"{bad} reciprocals differ from 1.0f / d"
    assert raw > 0
