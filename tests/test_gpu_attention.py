"""One window-attention step through the C ABI (aut_attention, the kernel the
forward uses; m-star AuTAttention: SDPA per window from cu_seqlens, no mask
inside a window and nothing across windows).

* fp32 inputs and outputs against the float64 oracle's ``window_attention``;
* bf16 inputs with fp32 outputs against the oracle, within the rounding of
  the probabilities to bf16 for the second product;
* bf16 outputs bit-identical to those fp32 outputs rounded to nearest even;
* MX-fp8 outputs (the operand of an fp8 out-projection): codes and scale codes
  bit-identical to the oracle's ``mx_quantize`` of the kernel's own fp32
  outputs, i.e. the producer's block maximum (lane swaps over the four lane
  groups that hold a query row), scale exponent and e4m3 rounding are checked
  code by code;
* the order the windows are taken in changes no bit.

Windows cover the kernel's key-tile paths: 1, 2, 13, 16, 17, 33, 52, 64, 65,
96 (every tile masked), 97 and 112 (eighth tile skipped), 113, 117 and 128
(eighth tile masked); and the wide workload's 171 windows (14 673 rows,
20 heads).
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from gpu_common import torch_mod

pytestmark = pytest.mark.gpu

RAGGED = [104, 1, 2, 13, 16, 17, 52, 96, 97, 112, 113, 117, 128, 104, 33, 64, 65]


def inputs(lens, heads, seed, bf16):
    """qkv [T, 3 d]: q and k ~ N(0, 1.5^2) (scaled scores with a spread of a
    few units, so the softmax is neither flat nor one-hot), v ~ N(0, 1);
    bf16-representable values when the kernel reads bf16."""
    torch = torch_mod()
    rng = np.random.default_rng(seed)
    T, d = int(sum(lens)), 64 * heads
    qkv = rng.standard_normal((T, 3 * d)).astype(np.float32)
    qkv[:, :2 * d] *= 1.5
    t = torch.from_numpy(qkv)
    if bf16:
        t = t.to(torch.bfloat16)
        qkv = t.float().numpy()
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return qkv.astype(np.float64), t.cuda(), cu


def device_tables(cu, order):
    torch = torch_mod()
    return (torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda(),
            torch.from_numpy(np.asarray(order, dtype=np.int32)).cuda())


def longest_first(lens):
    return np.argsort(-np.asarray(lens), kind="stable")


def reference(qkv, cu, heads):
    d = 64 * heads
    return oracle.window_attention(qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:], cu, heads)


def run(t, cu, order, heads, out_dtype):
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    dcu, dord = device_tables(cu, order)
    y = aut.attention(t, dcu, dord, heads, out_dtype)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("heads", [4, 20])
def test_attention_fp32_vs_oracle(heads):
    print(f"case: attention fp32, {len(RAGGED)} ragged windows, {heads} heads", flush=True)
    qkv, t, cu = inputs(RAGGED, heads, seed=heads, bf16=False)
    y = run(t, cu, longest_first(RAGGED), heads, "fp32").double().cpu().numpy()
    ref = reference(qkv, cu, heads)
    rms = np.sqrt(np.mean(ref * ref))
    err = float(np.max(np.abs(y - ref) / np.maximum(np.abs(ref), rms)))
    print(f"[attention fp32 h{heads}] rel err {err:.3e}", flush=True)
    assert np.isfinite(y).all()
    assert err <= 1e-4


@pytest.mark.parametrize("heads", [4, 20])
def test_attention_bf16_vs_oracle(heads):
    """bf16 inputs, fp32 outputs: the probabilities enter the second product
    rounded to bf16 (relative error at most 2^-9 each) while the normaliser
    sums them unrounded, so |out - ref| <= 2^-9 max|v|, plus fp32 rounding
    (at most 1e-4 max|v| here)."""
    print(f"case: attention bf16 -> fp32, {len(RAGGED)} ragged windows, {heads} heads", flush=True)
    qkv, t, cu = inputs(RAGGED, heads, seed=10 + heads, bf16=True)
    y = run(t, cu, longest_first(RAGGED), heads, "fp32").double().cpu().numpy()
    ref = reference(qkv, cu, heads)
    vmax = float(np.abs(qkv[:, 128 * heads:]).max())
    err = float(np.abs(y - ref).max())
    bound = (2.0 ** -9 + 1e-4) * vmax
    print(f"[attention bf16 h{heads}] max abs err {err:.3e}, bound {bound:.3e}", flush=True)
    assert err <= bound


@pytest.mark.parametrize("heads", [4, 20])
def test_attention_bf16_is_rounded_fp32(heads):
    torch = torch_mod()
    print(f"case: attention bf16 -> bf16 against bf16 -> fp32, {heads} heads", flush=True)
    _, t, cu = inputs(RAGGED, heads, seed=20 + heads, bf16=True)
    order = longest_first(RAGGED)
    y32 = run(t, cu, order, heads, "fp32")
    y16 = run(t, cu, order, heads, "bf16")
    assert torch.equal(y16, y32.to(torch.bfloat16))


def check_mx(t, cu, lens, heads, what):
    from packed_windowed_attention_amd import aut
    order = longest_first(lens)
    y32 = run(t, cu, order, heads, "fp32")
    codes, scales = run(t, cu, order, heads, "fp8")
    T, d = y32.shape
    rc, rs = oracle.mx_quantize(y32.double().cpu().numpy())
    got_c = codes.cpu().numpy()
    got_s = aut.mx_scales_rowmajor(scales.cpu().numpy(), T, d)
    nbad = int(np.count_nonzero(got_c != rc))
    print(f"[{what}] code mismatches {nbad}, scale mismatches {int(np.count_nonzero(got_s != rs))}",
          flush=True)
    assert nbad == 0
    assert np.array_equal(got_s, rs)


@pytest.mark.parametrize("heads", [4, 20])
def test_attention_mx_producer_bit_exact(heads):
    print(f"case: attention bf16 -> fp8, {len(RAGGED)} ragged windows, {heads} heads", flush=True)
    _, t, cu = inputs(RAGGED, heads, seed=30 + heads, bf16=True)
    check_mx(t, cu, RAGGED, heads, f"attention fp8 h{heads}")


def test_attention_wide_windows():
    """The wide workload's 171 windows (14 673 rows, 20 heads), random bf16
    qkv: every output against the oracle, and the MX-fp8 producer bit-exact
    over the whole output."""
    opl = oracle.plan(si.feature_lens("wide"), si.model_config("wide"))
    cu_w = np.asarray(opl["cu_seqlens"], dtype=np.int32)
    lens = np.diff(cu_w)
    print(f"case: attention bf16, wide windows ({len(lens)} windows, {cu_w[-1]} rows)", flush=True)
    qkv, t, cu = inputs(lens, 20, seed=41, bf16=True)
    assert np.array_equal(cu, cu_w)
    y = run(t, cu, longest_first(lens), 20, "fp32").double().cpu().numpy()
    ref = reference(qkv, cu, 20)
    vmax = float(np.abs(qkv[:, 2560:]).max())
    err = float(np.abs(y - ref).max())
    print(f"[attention wide] max abs err {err:.3e}", flush=True)
    assert err <= (2.0 ** -9 + 1e-4) * vmax
    check_mx(t, cu, lens, 20, "attention fp8 wide")


def test_attention_window_order_changes_no_bit():
    torch = torch_mod()
    print("case: attention bf16, longest-first against a random window order", flush=True)
    _, t, cu = inputs(RAGGED, 20, seed=50, bf16=True)
    perm = np.random.default_rng(51).permutation(len(RAGGED))
    a = run(t, cu, longest_first(RAGGED), 20, "bf16")
    b = run(t, cu, perm, 20, "bf16")
    assert torch.equal(a, b)
