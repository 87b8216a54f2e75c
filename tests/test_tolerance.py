"""The parity bound's allowance for results stored in bfloat16, checked on the host."""
import numpy as np
import torch

from test_gpu_parity import _half_ulp_bf16


def test_half_ulp_bounds_bf16_storage_rounding_tightly():
    gen = torch.Generator().manual_seed(0)
    # float32 values, as the kernels round them (float64 -> bfloat16 in torch goes through
    # float32 and can round twice)
    x = torch.randn(200000, generator=gen, dtype=torch.float32) * 8
    x[:4] = torch.tensor([0.0, 1.0, -4.0, 3.0 + 2.0 ** -7])      # exact, exact, exact, a tie
    err = (x.to(torch.bfloat16).double() - x.double()).abs().numpy()
    h = _half_ulp_bf16(x.double().numpy())
    assert (err <= h).all()
    assert err[:3].max() == 0.0 and err[3] == h[3]
    assert (err / np.where(h > 0, h, 1.0)).max() > 0.99
