"""aut_encode_planned inside a captured HIP graph (the header documents it as
capturable: kernels only, no allocation, synchronisation or host copy).

The graph is replayed several times with the program's own eager work and
synchronisations in between; every replay must equal the eager forward bit
for bit (same kernels, same launch shapes, so the same arithmetic)."""
import numpy as np
import pytest

import synth_inputs as si
from gpu_common import features_dev, pack, small_cfg, torch_mod

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,mask", [("fp32", 0), ("bf16", 0), ("fp8", 63)])
def test_graph_replay_matches_eager(dtype, mask):
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    cfg_d = small_cfg(dtype, fp8_gemms=mask)
    lens = np.array([250, 0, 800, 37, 1737])
    feats = si.mel_features(lens, seed=41)
    P = si.params(cfg_d, seed=41, std=0.05)
    print(f"case: graph replay {dtype} mask {mask}", flush=True)
    cfg, packed = pack(cfg_d, P)
    fd = features_dev(feats)
    pl = aut.plan(cfg, lens)
    ws = aut.workspace(cfg, pl, dtype)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        aut.plan_upload(pl, ws, stream=side)
        eager = torch.empty((pl.total_tokens, cfg_d["output_dim"]), device="cuda")
        aut.encode_planned(cfg, pl, fd, packed, dtype, eager, ws, stream=side)
    torch.cuda.synchronize()
    ref = eager.cpu().numpy()

    out = torch.full_like(eager, float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        aut.encode_planned(cfg, pl, fd, packed, dtype, out, ws,
                           stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        # eager work between replays, on the same buffers' device
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.isfinite(got).all(), f"replay {rep}: non-finite output"
        assert np.array_equal(got, ref), f"replay {rep}: max diff {np.abs(got - ref).max()}"
        del junk
    print(f"[graph {dtype} mask {mask}] 3 replays bit-identical to eager ({pl.total_tokens} tokens)",
          flush=True)
