"""One LayerNorm step through the C ABI (aut_layernorm, the kernel in front of
qkv, fc1 and the projector; LayerNorm with bias: cubic.dev wiki, "Audio
Encoder Component").

* fp32 output against the float64 oracle's ``layer_norm`` (fp32 statistics:
  relative error a few float32 units);
* bf16 output bit-identical to the fp32 output rounded to nearest even (the
  same fp32 values, one conversion);
* MX-fp8 output (the operand the fp8 qkv / fc1 / projector products read):
  codes and scale codes bit-identical to the oracle's ``mx_quantize`` of the
  kernel's own fp32 output, i.e. the producer's block maximum (a butterfly
  over the 8 lanes of a block), scale exponent and e4m3 rounding are checked
  code by code.
"""
import numpy as np
import pytest

import oracle
from gpu_common import torch_mod

pytestmark = pytest.mark.gpu


def ln_inputs(R, d, seed):
    """Rows with an offset and a spread that vary over many binades, plus a
    constant row (zero variance: the output is beta exactly) and a row with
    one large outlier (a block maximum far above its neighbours)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, d)) * np.exp2(rng.integers(-6, 7, (R, 1))) + rng.standard_normal((R, 1)) * 3
    if R > 2:
        x[1] = 0.75
        x[2, d // 3] = 500.0
    g = 1.0 + 0.3 * rng.standard_normal(d)
    b = 0.1 * rng.standard_normal(d)
    return x.astype(np.float32), g.astype(np.float32), b.astype(np.float32)


def run(R, d, dtype, seed):
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    x, g, b = ln_inputs(R, d, seed)
    xd, gd, bd = (torch.from_numpy(a).cuda() for a in (x, g, b))
    y = aut.layernorm(xd, gd, bd, dtype)
    torch.cuda.synchronize()
    return x, g, b, y


@pytest.mark.parametrize("R,d", [(1, 256), (37, 200), (1000, 1280), (14673, 1280), (300, 2048)])
def test_layernorm_fp32_vs_oracle(R, d):
    print(f"case: layernorm fp32 R={R} d={d}", flush=True)
    x, g, b, y = run(R, d, "fp32", seed=R + d)
    ref = oracle.layer_norm(x.astype(np.float64), g.astype(np.float64), b.astype(np.float64))
    got = y.double().cpu().numpy()
    scale = np.abs(g).max() * np.sqrt(d) + np.abs(b).max()
    err = float(np.abs(got - ref).max())
    print(f"[layernorm fp32 {R}x{d}] max abs err {err:.3e} (bound scale {scale:.1f})", flush=True)
    assert np.isfinite(got).all()
    assert err <= 4e-6 * scale
    if R > 2:
        assert np.array_equal(got[1].astype(np.float32), b)   # constant row: beta exactly


@pytest.mark.parametrize("R,d", [(37, 200), (1000, 1280)])
def test_layernorm_bf16_is_rounded_fp32(R, d):
    torch = torch_mod()
    print(f"case: layernorm bf16 R={R} d={d}", flush=True)
    _, _, _, y32 = run(R, d, "fp32", seed=7 * R + d)
    _, _, _, y16 = run(R, d, "bf16", seed=7 * R + d)
    assert torch.equal(y16, y32.to(torch.bfloat16))


@pytest.mark.parametrize("R,d", [(1, 128), (37, 1024), (1000, 1280), (14673, 1280), (300, 2048)])
def test_layernorm_mx_producer_bit_exact(R, d):
    from packed_windowed_attention_amd import aut
    print(f"case: layernorm fp8 R={R} d={d}", flush=True)
    _, _, _, y32 = run(R, d, "fp32", seed=3 * R + d)
    _, _, _, (codes, scales) = run(R, d, "fp8", seed=3 * R + d)
    rc, rs = oracle.mx_quantize(y32.double().cpu().numpy())
    got_c = codes.cpu().numpy()
    got_s = aut.mx_scales_rowmajor(scales.cpu().numpy(), R, d)
    nbad = int(np.count_nonzero(got_c != rc))
    print(f"[layernorm fp8 {R}x{d}] code mismatches {nbad}, scale mismatches "
          f"{int(np.count_nonzero(got_s != rs))}", flush=True)
    assert nbad == 0
    assert np.array_equal(got_s, rs)


def test_layernorm_argument_checks():
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    x = torch.zeros((4, 96), device="cuda")
    g = torch.ones(96, device="cuda")
    with pytest.raises(RuntimeError) as e:          # fp8 needs d a multiple of 128
        aut.layernorm(x, g, torch.zeros(96, device="cuda"), "fp8")
    assert "AUT_ERR_UNSUPPORTED" in str(e.value)
    with pytest.raises(ValueError):
        aut.layernorm(x, g[:50], g[:50], "fp32")
