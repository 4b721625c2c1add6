"""aut_encode_noalloc through the C ABI: the forward on the library's own
device scratch (for callers that cannot allocate device memory) gives, bit
for bit, what aut_encode gives with a caller workspace, on two calls in a row
(the second with a smaller batch, over scratch the first one left behind),
in fp32, bf16 and MX-fp8."""
import numpy as np
import pytest

import synth_inputs as si
from gpu_common import features_dev, pack, small_cfg, torch_mod

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp8"])
def test_noalloc_equals_encode(dtype):
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    cfg_d = small_cfg(dtype, encoder_layers=2)
    P = si.params(cfg_d, seed=41, std=0.05)
    cfg, packed = pack(cfg_d, P)
    for lens in (np.array([1737, 250, 0, 801, 3000]), np.array([420, 37])):
        print(f"case: noalloc {dtype} lens {list(lens)}", flush=True)
        feats = si.mel_features(lens, seed=int(lens.sum()))
        fd = features_dev(feats)
        ref, pl = aut.encode(cfg, fd, lens, packed, dtype)
        out = torch.full((pl.total_tokens, cfg_d["output_dim"]), float("nan"), device="cuda")
        got, pl2 = aut.encode_noalloc(cfg, fd, lens, packed, dtype, out=out)
        torch.cuda.synchronize()
        assert pl2.copy()[1] == pl.copy()[1]
        assert got.data_ptr() == out.data_ptr()
        g, r = got.cpu().numpy(), ref.cpu().numpy()
        print(f"[noalloc {dtype}] {pl.total_tokens} tokens, identical: {np.array_equal(g, r)}", flush=True)
        assert np.isfinite(g).all()
        assert np.array_equal(g, r)


def test_noalloc_wide_model_batch():
    """d_model 1280, 24 layers, C 480 (the full-width model) on a batch that
    fits the scratch at conv_chunksize 16: two calls, the second smaller."""
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    cfg_d, _, _, P = si.workload("wide")
    cfg_d = dict(cfg_d, conv_chunksize=16)
    cfg, packed = pack(cfg_d, P)
    for lens in (np.array([3000, 1250, 2999]), np.array([900])):
        pl = aut.plan(cfg, lens)
        print(f"case: noalloc wide lens {list(lens)}, workspace {aut.workspace_bytes(cfg, pl, 'bf16')} bytes",
              flush=True)
        feats = si.mel_features(lens, seed=int(lens.sum()))
        fd = features_dev(feats)
        ref, _ = aut.encode(cfg, fd, lens, packed, "bf16")
        got, _ = aut.encode_noalloc(cfg, fd, lens, packed, "bf16")
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), ref.cpu().numpy())
