"""quantize_linear_layers: the user-level selection of the path (page
"Online Quantization", Parameters table: method, ignored_layers,
activation_scheme). Argument refusals run on the CPU; the conversion and the
converted model's forward run on the GPU."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from w8a8_int8_dynamic_amd import W8A8Linear, quantize_linear_layers


def _model(device="cpu", dtype=torch.float32):
    torch.manual_seed(0)
    return torch.nn.Sequential(
        torch.nn.Linear(256, 512), torch.nn.GELU(),
        torch.nn.Sequential(torch.nn.Linear(512, 128), torch.nn.Linear(128, 64, bias=False)),
    ).to(device=device, dtype=dtype)


def test_refusals_on_the_host():
    m = _model()
    with pytest.raises(ValueError, match="method"):
        quantize_linear_layers(m, method="mxfp4")
    with pytest.raises(ValueError, match="dynamic"):
        quantize_linear_layers(m, activation_scheme="static")
    with pytest.raises(ValueError, match="GPU"):          # a CPU layer is not converted silently
        quantize_linear_layers(m)
    # every Linear ignored: nothing to convert, the model comes back as it was
    same = quantize_linear_layers(m, ignored_layers=["0", "2.*"])
    assert same is m and all(isinstance(x, torch.nn.Linear) for x in (m[0], m[2][0], m[2][1]))


@pytest.mark.gpu
@pytest.mark.parametrize("method", ["int8", "fp8"])
def test_convert_and_run(method):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ref = _model("cuda", torch.bfloat16)
    m = _model("cuda", torch.bfloat16)
    x = torch.randn(3, 40, 256, device="cuda", generator=torch.Generator("cuda").manual_seed(1))
    x = x.to(torch.bfloat16)
    direct = W8A8Linear.from_float(m[0].weight.detach(), m[0].bias.detach(), scheme=method)
    out = quantize_linear_layers(m, method=method, ignored_layers=["2.1"])
    assert out is m
    assert isinstance(m[0], W8A8Linear) and isinstance(m[2][0], W8A8Linear)
    assert isinstance(m[2][1], torch.nn.Linear) and not isinstance(m[2][1], W8A8Linear)
    assert m[0].scheme == method
    # the first layer equals W8A8Linear built directly, bit for bit
    assert torch.equal(m[0](x).view(torch.int16), direct(x).view(torch.int16))
    # the whole model stays close to its float twin (fp32 reference)
    with torch.no_grad():
        y = m(x).float()
        r = ref.float()(x.float())
    rel = (torch.linalg.norm(y - r) / torch.linalg.norm(r)).item()
    bound = 0.03 if method == "int8" else 0.10      # e4m3 keeps 3 mantissa bits
    assert y.shape == (3, 40, 64) and np.isfinite(rel) and rel < bound, rel
    # a layer whose in_features is not a multiple of 16 is refused by name
    odd = torch.nn.Sequential(torch.nn.Linear(40, 8)).cuda()
    with pytest.raises(ValueError, match="'0'"):
        quantize_linear_layers(odd, method=method)
