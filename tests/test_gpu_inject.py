"""Audio rows into the decoder's embedding sequence ("Audio Encoder Component",
cubic.dev wiki, Data Flow and Integration) through the C ABI, bit-exact against
the oracle for fp32 and bf16 sequences."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_common import torch_mod

pytestmark = pytest.mark.gpu

PAD = 151676


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("n_audio,S", [(1, 3), (759, 1000), (14673, 15200)])
def test_inject_matches_oracle(dtype, n_audio, S):
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    rng = np.random.default_rng(n_audio)
    D = 2048
    print(f"case: inject {dtype} n_audio={n_audio} S={S}", flush=True)
    ids = rng.integers(0, 150000, size=S).astype(np.int32)
    pos = np.sort(rng.choice(S, size=n_audio, replace=False))
    ids[pos] = PAD
    audio = rng.normal(size=(n_audio, D)).astype(np.float32)
    emb = rng.normal(size=(S, D)).astype(np.float32)
    if dtype == "bf16":
        emb = oracle.bf16_round(emb)
    rows = torch.tensor(aut.audio_rows(ids, PAD, n_audio), dtype=torch.int32, device="cuda")
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    dst = torch.from_numpy(emb).cuda().to(tdt)
    aut.inject_audio(torch.from_numpy(audio).cuda(), rows, dst, dtype)
    torch.cuda.synchronize()
    got = dst.float().cpu().numpy().astype(np.float64)
    ref = oracle.inject_audio(emb, ids, PAD, audio.astype(np.float64), dtype)
    np.testing.assert_array_equal(got, ref)
