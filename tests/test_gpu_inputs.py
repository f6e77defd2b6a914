"""The device fill reproduces the host generator bit for bit (GPU)."""
import numpy as np
import pytest
import torch

from hils_inputs.configs import LazyNormalBF16
from hils_inputs.device import fill_normal
from hils_inputs.gen import normal_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,dtype", [(1000003, torch.bfloat16), (4099, torch.float32), (7, torch.bfloat16)])
def test_device_fill_matches_host(n, dtype):
    assert torch.cuda.is_available()
    t = torch.empty(n, dtype=dtype, device="cuda")
    fill_normal(t, 7, "k", offset=123456789)
    torch.cuda.synchronize()
    want = normal_f32(7, 2, np.arange(123456789, 123456789 + n, dtype=np.uint64))
    if dtype == torch.bfloat16:
        got = t.view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(got, f32_to_bf16_bits(want))
    else:
        np.testing.assert_array_equal(t.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_lazy_view_matches_device_cache():
    shape = (2, 3, 4096, 128)
    t = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    fill_normal(t, 5, "v")
    lz = LazyNormalBF16(5, "v", shape)
    got = t[1, 2, 1000:1064].float().cpu().numpy()
    np.testing.assert_array_equal(got, lz[1, 2][1000:1064])
