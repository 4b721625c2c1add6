"""Log-mel front end through the C ABI against the oracle's Whisper-style
log-mel, and the whole path audio -> log-mel -> encoder against the oracle."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth_inputs as si
from gpu_common import check, forward, pack, small_cfg, torch_mod

pytestmark = pytest.mark.gpu

# fp32 DFT and filterbank on the matrix cores against float64: the relative
# error of a bin's power is ~ sqrt(400) x 6e-8 x (frame energy / bin power),
# i.e. 1e-6 for typical bins and larger only for bins far below their frame's
# energy; log10 turns a relative error e into e / ln 10 and the scaling divides
# by 4 (measured on the speech-like stand-in: max 5e-6, mean 1e-7)
LOGMEL_ABS_TOL = 1e-4
LOGMEL_MEAN_TOL = 1e-6


def test_logmel_vs_oracle():
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    n = np.array([16000, 161 * 160 + 57, 80000, 201, 0, 32123])
    audio = si.audio_samples(n, seed=5)
    print(f"case: logmel samples={list(n)}", flush=True)
    tables = aut.logmel_tables()
    feats = aut.logmel(torch.from_numpy(audio).cuda(), n, tables)
    torch.cuda.synchronize()
    got = feats.cpu().numpy().astype(np.float64)
    for b in range(len(n)):
        nf = int(n[b]) // 160
        assert np.isfinite(got[b, :, :nf]).all()
        if nf == 0:
            continue
        ref = oracle.log_mel(audio[b, :n[b]].astype(np.float64))
        err = np.abs(got[b, :, :nf] - ref)
        print(f"[logmel {b}] frames {nf}: max abs {err.max():.3e} mean abs {err.mean():.3e}", flush=True)
        assert err.max() <= LOGMEL_ABS_TOL and err.mean() <= LOGMEL_MEAN_TOL
        # untouched past the request's frames
        assert (got[b, :, nf:] == 0).all()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_audio_to_encoder(dtype):
    """16 kHz audio -> GPU log-mel -> GPU encoder against oracle log-mel ->
    oracle encoder (both halves' own tolerances hold end to end)."""
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    cfg_d = small_cfg(dtype)
    n = np.array([3 * 16000 + 123, 9 * 16000, 20000])
    audio = si.audio_samples(n, seed=6)
    P = si.params(cfg_d, seed=6, std=0.05)
    print(f"case: audio->encoder {dtype} samples={list(n)}", flush=True)
    feats = aut.logmel(torch.from_numpy(audio).cuda(), n, aut.logmel_tables())
    lens = n // 160
    cfg, packed = pack(cfg_d, P)
    out, _ = aut.encode(cfg, feats, lens, packed, dtype)
    torch.cuda.synchronize()
    T_max = feats.shape[2]
    ref_feats = np.zeros((len(n), 128, T_max))
    for b in range(len(n)):
        ref_feats[b, :, :lens[b]] = oracle.log_mel(audio[b, :n[b]].astype(np.float64))
    ref, _ = oracle.forward(ref_feats, lens, P, cfg_d)
    check(out.double().cpu().numpy(), ref, dtype, "audio->encoder")


def test_logmel_argument_checks():
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    tables = aut.logmel_tables()
    audio = torch.zeros((2, 1000), dtype=torch.float32, device="cuda")
    for lens, T_max in (([150, 1000], 8), ([1000, 1001], 8), ([1000, 1000], 4), ([1000, 1000], 6)):
        with pytest.raises(RuntimeError) as e:
            aut.logmel(audio, lens, tables, T_max=T_max)
        assert "AUT_ERR_INVALID_ARG" in str(e.value)
