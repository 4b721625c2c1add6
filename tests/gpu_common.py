"""Helpers for the GPU tests: device upload, the forward through the C ABI,
and the comparison metrics with their tolerances."""
from __future__ import annotations

import functools

import numpy as np

import synth_inputs as si

# fp32 mode: max_i |g_i - r_i| / max(|r_i|, rms(r)) over the whole output
FP32_REL_TOL = 1e-4
# bf16 mode: max-abs error and per-token cosine similarity
BF16_ABS_TOL = 2e-2
BF16_COS_TOL = 0.999


def torch_mod():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("these tests need a GPU")
    return torch


def small_cfg(dtype="fp32", **kw):
    cfg = dict(num_mel_bins=128, n_window=50, n_window_infer=800, conv_chunksize=500,
               output_dim=128, max_source_positions=1500, d_model=256, encoder_layers=2,
               encoder_attention_heads=4, encoder_ffn_dim=512, downsample_hidden_size=32,
               conv_out_bias=False, dtype=dtype)
    cfg.update(kw)
    return cfg


def to_device(P: dict):
    torch = torch_mod()
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in P.items()}


def pack(cfg_d: dict, P: dict):
    from packed_windowed_attention_amd import aut
    cfg = aut.config(cfg_d)
    dev = to_device(P)
    packed = aut.weights_pack(cfg, dev, cfg_d["dtype"])
    del dev
    return cfg, packed


def features_dev(feats: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(feats)).cuda()


def forward(cfg_d, lens, feats, P=None, packed=None, cfg=None):
    """Whole forward through aut_encode; returns (out float64 numpy, plan)."""
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    if packed is None:
        cfg, packed = pack(cfg_d, P)
    out, pl = aut.encode(cfg, features_dev(feats), lens, packed, cfg_d["dtype"])
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), pl


def rel_err(g, r):
    r = np.asarray(r, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r)) if r.size else 1.0
    den = np.maximum(np.abs(r), rms)
    return float(np.max(np.abs(g - r) / den)) if r.size else 0.0


def token_cos(g, r):
    num = np.sum(g * r, axis=1)
    den = np.linalg.norm(g, axis=1) * np.linalg.norm(r, axis=1)
    return num / np.maximum(den, 1e-30)


def check_fp32(g, r, what=""):
    e = rel_err(g, r)
    print(f"[{what}] fp32 rel err {e:.3e} (normwise {np.abs(g - r).max() / max(np.abs(r).max(), 1e-30):.3e})",
          flush=True)
    assert np.isfinite(g).all()
    assert e <= FP32_REL_TOL, f"{what}: rel err {e}"


def check_bf16(g, r, what=""):
    assert np.isfinite(g).all()
    mx = float(np.abs(g - r).max()) if r.size else 0.0
    cmin = float(token_cos(g, r).min()) if r.size else 1.0
    print(f"[{what}] bf16 max-abs {mx:.3e} min cos {cmin:.6f} (ref max {np.abs(r).max():.3f})", flush=True)
    assert mx <= BF16_ABS_TOL, f"{what}: max-abs {mx}"
    assert cmin >= BF16_COS_TOL, f"{what}: min cosine {cmin}"


def check(g, r, dtype, what=""):
    (check_fp32 if dtype == "fp32" else check_bf16)(g, r, what)


@functools.lru_cache(maxsize=2)
def workload(name):
    return si.workload(name)


def sample_windows(pl_oracle: dict, seed: int, n_random: int = 4, at_least: int = 8):
    """First, last, shortest, longest partial and n_random random windows,
    topped up with further random ones until at least ``at_least`` distinct
    windows (or all of them) are picked."""
    wl = pl_oracle["window_lengths"]
    nw = len(wl)
    pick = {0, nw - 1, int(np.argmin(wl))}
    partial = [w for w in range(nw) if wl[w] < max(wl)]
    if partial:
        pick.add(max(partial, key=lambda w: (wl[w], -w)))
    rng = np.random.default_rng(seed)
    order = [int(x) for x in rng.permutation(nw)]
    pick.update(order[:min(n_random, nw)])
    for w in order[min(n_random, nw):]:
        if len(pick) >= min(at_least, nw):
            break
        pick.add(w)
    return sorted(pick)
