"""Incremental (streaming) encode through the C ABI: a live request whose
audio arrives in pieces, re-encoded from its first non-final window at each
step, ends bit-identical to the batch encode, and rows that are final are
never rewritten (windows are independent: m-star module summary; openarchlab
"1A", section 4).  At every arrival the rows written so far are also checked
against the float64 oracle's forward of the request as it stands (its first
n frames), and the final output against the oracle's forward of the whole
request, at the mode's tolerance (fp32: relative 1e-4; bf16: max-abs 2e-2 and
per-token cosine 0.999; MX-fp8: within the quantisation noise bound of the
oracle with the same products quantised)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth_inputs as si
from gpu_common import check, forward, pack, small_cfg, torch_mod
from test_gpu_fp8 import check_fp8

pytestmark = pytest.mark.gpu

ARRIVALS = [150, 420, 800, 1010, 1650, 2400, 2630]
FP8_MASK = 63


def check_vs_oracle(g, feats, n, P, cfg_d, dtype, what):
    """Rows g against the oracle's forward of the request's first n frames."""
    f = np.ascontiguousarray(feats[:, :, :n])
    ref, _ = oracle.forward(f, np.array([n]), P, cfg_d)
    ref = ref[:g.shape[0]]
    if dtype == "fp8":
        ref_q, _ = oracle.forward(f, np.array([n]), P, cfg_d, fp8=FP8_MASK)
        check_fp8(g, ref_q[:g.shape[0]], ref, what)
    else:
        check(g, ref, dtype, what)


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp8"])
def test_stream_equals_batch(dtype):
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    cfg_d = small_cfg(dtype)
    if dtype == "fp8":
        cfg_d["fp8_gemms"] = FP8_MASK
    L = ARRIVALS[-1]
    lens = np.array([L])
    feats = si.mel_features(lens, seed=31)
    P = si.params(cfg_d, seed=31, std=0.05)
    cfg, packed = pack(cfg_d, P)
    print(f"case: stream {dtype} L={L} arrivals={ARRIVALS}", flush=True)
    y_batch, _ = forward(cfg_d, lens, feats, packed=packed, cfg=cfg)
    T = y_batch.shape[0]
    T_max = feats.shape[2]
    # frames not yet arrived hold NaN: any read of them would show in the output
    fbuf = torch.full((cfg_d["num_mel_bins"], T_max), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full((T, cfg_d["output_dim"]), float("nan"), dtype=torch.float32, device="cuda")
    ws = aut.stream_workspace(cfg, L, dtype)
    wf = 0
    prev = out.cpu().numpy()
    for n in ARRIVALS:
        fbuf[:, :n] = torch.from_numpy(np.ascontiguousarray(feats[0, :, :n])).cuda()
        sp = aut.stream_plan(cfg, n, wf)
        wf_new = aut.encode_stream(cfg, fbuf, n, wf, packed, dtype, out, ws)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        r0, r1 = sp["row_begin"], sp["row_begin"] + sp["rows"]
        print(f"[stream {dtype}] frames {n}: rows {r0}..{r1}, final windows {wf} -> {wf_new}", flush=True)
        assert np.isfinite(o[r0:r1]).all()
        # rows of windows already final were not touched
        np.testing.assert_array_equal(o[:r0], prev[:r0])
        # rows final now equal the batch result bit for bit
        rf = sp["row_begin"] + 104 * (wf_new - wf)
        np.testing.assert_array_equal(o[:rf], y_batch[:rf])
        # every row written so far against the oracle on the frames received
        check_vs_oracle(o[:r1].astype(np.float64), feats, n, P, cfg_d, dtype, f"stream {dtype} at {n} frames")
        wf = wf_new
        prev = o
    final = out.cpu().numpy()
    np.testing.assert_array_equal(final, y_batch)
    check_vs_oracle(final.astype(np.float64), feats, L, P, cfg_d, dtype, f"stream {dtype} final")


def test_stream_argument_checks():
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    cfg_d = small_cfg("fp32")
    cfg, packed = pack(cfg_d, si.params(cfg_d, seed=1))
    fbuf = torch.zeros((128, 1000), dtype=torch.float32, device="cuda")
    out = torch.zeros((200, cfg_d["output_dim"]), dtype=torch.float32, device="cuda")
    ws = aut.stream_workspace(cfg, 1000, "fp32")
    for frames, wf in ((1200, 0), (900, 2)):   # more frames than T_max; windows not complete
        with pytest.raises(RuntimeError) as e:
            aut.encode_stream(cfg, fbuf, frames, wf, packed, "fp32", out, ws)
        assert "AUT_ERR_INVALID_ARG" in str(e.value)
    # nothing left to encode: no launch, no error
    assert aut.encode_stream(cfg, fbuf, 800, 1, packed, "fp32", out, ws) == 1
