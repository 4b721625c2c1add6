"""Seeded synthetic inputs for the AuT encoder forward pass.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark.  It holds *no* arithmetic of the method itself: it only draws the
request lengths, the log-mel features and the parameters, and names the five
workloads.  Everything the encoder computes lives on each side separately.

Workloads (model sizes from the AuTEncoderConfig field list and defaults of the
m-star ``aut_encoder`` API page; the request length mixes are synthetic
stand-ins for a read-speech test set's utterance lengths, and N(-4, 2) noise
stands in for real log-mel values):

====  =========================================  ==============================
name  requests / lengths                         model
====  =========================================  ==============================
tiny  1 x 8 s                                    1 layer, d 1280, C 128, fp32
rag   4 x (3.0, 8.0, 17.37, 30.0) s              18 layers, d 1024, C 128, bf16
wide  64 x U[5, 30] s                            24 layers, d 1280, C 480, bf16
long  1 x 1200 s                                 24 layers, d 1280, C 480, bf16
conc  512 x lognormal(ln 7, 0.6) in [0.5, 35] s  24 layers, d 1280, C 480, bf16
====  =========================================  ==============================

Random streams: workload k (1-based) uses base seed ``k - 1`` and numpy's PCG64
through ``default_rng([seed, stream])`` with stream 0 = lengths, 1 = mel,
2 = parameters, so that changing one never shifts another.
"""
from __future__ import annotations

import numpy as np

MEL_BINS = 128

# ---------------------------------------------------------------------------
# model shapes
# ---------------------------------------------------------------------------

_BASE = dict(
    num_mel_bins=128,
    n_window=50,
    n_window_infer=800,
    conv_chunksize=500,
    output_dim=2048,
    max_source_positions=1500,
    conv_out_bias=False,
)


def model_config(name: str) -> dict:
    """Model hyper-parameters of a named workload (field names follow
    AuTEncoderConfig on the m-star API page)."""
    if name == "tiny":
        m = dict(d_model=1280, encoder_layers=1, encoder_attention_heads=20,
                 encoder_ffn_dim=5120, downsample_hidden_size=128, dtype="fp32")
    elif name == "rag":
        m = dict(d_model=1024, encoder_layers=18, encoder_attention_heads=16,
                 encoder_ffn_dim=4096, downsample_hidden_size=128, dtype="bf16")
    elif name in ("wide", "long", "conc"):
        m = dict(d_model=1280, encoder_layers=24, encoder_attention_heads=20,
                 encoder_ffn_dim=5120, downsample_hidden_size=480, dtype="bf16")
    else:
        raise KeyError(name)
    out = dict(_BASE)
    out.update(m)
    return out


WORKLOADS = ("tiny", "rag", "wide", "long", "conc")


def workload_seed(name: str) -> int:
    return WORKLOADS.index(name)


def seconds_to_frames(seconds) -> np.ndarray:
    """100 mel frames per second, rounded half up (17.37 s -> 1737 frames)."""
    s = np.asarray(seconds, dtype=np.float64)
    return np.floor(100.0 * s + 0.5).astype(np.int64)


def feature_lens(name: str) -> np.ndarray:
    """Per-request mel lengths (frames) of a named workload, int64."""
    seed = workload_seed(name)
    rng = np.random.default_rng([seed, 0])
    if name == "tiny":
        sec = [8.0]
    elif name == "rag":
        sec = [3.0, 8.0, 17.37, 30.0]
    elif name == "wide":
        sec = rng.uniform(5.0, 30.0, 64)
    elif name == "long":
        sec = [1200.0]
    elif name == "conc":
        sec = np.clip(rng.lognormal(np.log(7.0), 0.6, 512), 0.5, 35.0)
    else:
        raise KeyError(name)
    return seconds_to_frames(sec)


def mel_features(lens, seed: int, pad_value: float = float("nan"),
                 t_max: int | None = None) -> np.ndarray:
    """Log-mel stand-in: i.i.d. N(-4, 2) float32 in a [B, 128, T_max] buffer.

    Frames at or beyond a request's length hold ``pad_value`` (NaN by default),
    so that any use of the padding shows up at once.
    """
    lens = np.asarray(lens, dtype=np.int64)
    B = len(lens)
    T = int(lens.max()) if t_max is None else int(t_max)
    T = max(T, 1)
    rng = np.random.default_rng([seed, 1])
    x = np.full((B, MEL_BINS, T), pad_value, dtype=np.float32)
    for b in range(B):
        L = int(lens[b])
        if L:
            x[b, :, :L] = rng.normal(-4.0, 2.0, size=(MEL_BINS, L)).astype(np.float32)
    return x


def audio_samples(n_samples, seed: int, s_max: int | None = None) -> np.ndarray:
    """16 kHz mono stand-in for speech: Gaussian noise under a slowly varying,
    log-normal envelope (pauses down to ~1e-4 of the loud parts) plus a few
    steady tones, float32 [B, S_max]; samples past a request's length are 0."""
    n = np.asarray(n_samples, dtype=np.int64)
    B = len(n)
    S = max(int(n.max()) if B else 1, 1) if s_max is None else int(s_max)
    rng = np.random.default_rng([seed, 3])
    x = np.zeros((B, S), dtype=np.float32)
    for b in range(B):
        L = int(n[b])
        if not L:
            continue
        knots = rng.normal(0.0, 2.0, size=L // 1600 + 2)
        env = np.exp(np.interp(np.arange(L) / 1600.0, np.arange(knots.size), knots))
        t = np.arange(L) / 16000.0
        tones = sum(rng.uniform(0.05, 0.3) * np.sin(2 * np.pi * rng.uniform(80, 7000) * t + rng.uniform(0, 6.3))
                    for _ in range(3))
        x[b, :L] = (0.1 * env * rng.normal(size=L) + tones).astype(np.float32)
    return x


def param_shapes(cfg: dict) -> list[tuple[str, tuple]]:
    """Parameter roles in generation order, PyTorch layouts ([out, in(, kH, kW)])."""
    C = cfg["downsample_hidden_size"]
    d = cfg["d_model"]
    F = cfg["encoder_ffn_dim"]
    O = cfg["output_dim"]
    fbins = cfg["num_mel_bins"]
    for _ in range(3):
        fbins = (fbins + 1) // 2
    shapes = [
        ("conv1_w", (C, 1, 3, 3)), ("conv1_b", (C,)),
        ("conv2_w", (C, C, 3, 3)), ("conv2_b", (C,)),
        ("conv3_w", (C, C, 3, 3)), ("conv3_b", (C,)),
        ("conv_out_w", (d, C * fbins)),
    ]
    if cfg.get("conv_out_bias", False):
        shapes.append(("conv_out_b", (d,)))
    for i in range(cfg["encoder_layers"]):
        p = f"layers.{i}."
        shapes += [
            (p + "ln1_g", (d,)), (p + "ln1_b", (d,)),
            (p + "qkv_w", (3 * d, d)), (p + "qkv_b", (3 * d,)),
            (p + "o_w", (d, d)), (p + "o_b", (d,)),
            (p + "ln2_g", (d,)), (p + "ln2_b", (d,)),
            (p + "fc1_w", (F, d)), (p + "fc1_b", (F,)),
            (p + "fc2_w", (d, F)), (p + "fc2_b", (d,)),
        ]
    shapes += [
        ("ln_post_g", (d,)), ("ln_post_b", (d,)),
        ("proj1_w", (d, d)), ("proj1_b", (d,)),
        ("proj2_w", (O, d)), ("proj2_b", (O,)),
    ]
    return shapes


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Float32 values made bf16-representable (round to nearest even).

    Used only to prepare *inputs* (parameters) for bf16 workloads, so both the
    oracle and the device path start from the same representable values.
    Finite inputs only (generated parameters are never NaN or Inf).
    """
    out = np.array(a, dtype=np.float32, copy=True)
    u = out.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return out


def params(cfg: dict, seed: int, std: float = 0.02) -> dict[str, np.ndarray]:
    """Synthetic parameters: weights and biases ~ N(0, std); LayerNorm gain
    1 + N(0, std), LayerNorm shift ~ N(0, std).  float32, bf16-representable
    when the workload's dtype is bf16 or fp8 (whose other operands are bf16)."""
    rng = np.random.default_rng([seed, 2])
    out = {}
    for name, shape in param_shapes(cfg):
        a = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
        if name.endswith("_g"):
            a = a + np.float32(1.0)
        if cfg.get("dtype") in ("bf16", "fp8"):
            a = round_to_bf16(a)
        out[name] = a.astype(np.float32, copy=False)
    return out


def workload(name: str, with_params: bool = True):
    """(cfg, feature_lens, features, params) of a named workload."""
    cfg = model_config(name)
    seed = workload_seed(name)
    lens = feature_lens(name)
    feats = mel_features(lens, seed)
    w = params(cfg, seed) if with_params else None
    return cfg, lens, feats, w
