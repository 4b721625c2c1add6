"""Pins of the oracle's arithmetic against things other than itself.

Each ``check_*`` function compares one oracle function with a library routine
(torch float64 on the CPU), a closed form, or an exact invariant, and returns
the largest deviation.  ``test_planted_mistakes`` then plants plausible
mistakes in the oracle (a transposed kernel, a dropped bias, a causal mask, a
wrong variance, a swapped flatten order, ...) and requires the corresponding
check to catch each one: the pins are shown to be able to fail.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
import oracle.aut_oracle as ao
import synth_inputs as si

RNG = np.random.default_rng(1234)


def small_cfg(**kw):
    cfg = dict(num_mel_bins=128, n_window=50, n_window_infer=800, conv_chunksize=500,
               output_dim=96, max_source_positions=1500, d_model=128, encoder_layers=2,
               encoder_attention_heads=2, encoder_ffn_dim=256, downsample_hidden_size=8,
               conv_out_bias=False, dtype="fp32")
    cfg.update(kw)
    return cfg


# ---------------------------------------------------------------------------
# checks: each returns a max deviation
# ---------------------------------------------------------------------------


def check_gelu():
    x = np.linspace(-8, 8, 4001)
    ref = Fn.gelu(torch.from_numpy(x), approximate="none").numpy()
    e1 = np.abs(ao.gelu(x) - ref).max()
    # exact identities: gelu(x) - gelu(-x) = x, gelu(0) = 0
    e2 = np.abs(ao.gelu(x) - ao.gelu(-x) - x).max()
    return max(e1, e2, abs(ao.gelu(np.array(0.0))))


def check_pe():
    d = 1280
    D = d // 2
    pe = ao.sinusoid_table(1500, d)
    j = np.arange(1500)
    errs = [
        np.abs(pe[0, :D]).max(),
        np.abs(pe[0, D:] - 1).max(),
        np.abs(pe[:, 0] - np.sin(j)).max(),
        np.abs(pe[:, D] - np.cos(j)).max(),
        np.abs(pe[:, D - 1] - np.sin(j * 1e-4)).max(),
        np.abs(pe[:, 2 * D - 1] - np.cos(j * 1e-4)).max(),
        np.abs(pe[:, :D] ** 2 + pe[:, D:] ** 2 - 1).max(),
    ]
    # frequencies form a geometric progression from 1 down to 1e-4
    freq = np.arcsin(pe[1, :D])  # row 1 holds sin(tau_i), tau_i <= 1 < pi/2
    ratio = freq[1:] / freq[:-1]
    errs.append(np.abs(ratio - 1e-4 ** (1.0 / (D - 1))).max())
    return max(errs)


def check_conv():
    errs = []
    for cin, cout, H, W in [(1, 5, 128, 100), (3, 4, 9, 7), (2, 2, 64, 50), (4, 3, 32, 25)]:
        x = RNG.standard_normal((cin, H, W))
        w = RNG.standard_normal((cout, cin, 3, 3))
        b = RNG.standard_normal(cout)
        ref = Fn.conv2d(torch.from_numpy(x)[None], torch.from_numpy(w), torch.from_numpy(b),
                        stride=2, padding=1)[0].numpy()
        got = ao.conv2d_k3s2p1(x, w, b)
        if got.shape != ref.shape:
            return float("inf")
        errs.append(np.abs(got - ref).max())
    # special case: centre-tap identity kernel = stride-2 subsampling
    x = RNG.standard_normal((3, 11, 10))
    w = np.zeros((3, 3, 3, 3))
    for i in range(3):
        w[i, i, 1, 1] = 1.0
    errs.append(np.abs(ao.conv2d_k3s2p1(x, w, np.zeros(3)) - x[:, ::2, ::2]).max())
    return max(errs)


def check_ln():
    x = RNG.standard_normal((17, 96)) * 3 + 1.5
    g = RNG.standard_normal(96)
    b = RNG.standard_normal(96)
    ref = Fn.layer_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), torch.from_numpy(b),
                        eps=1e-5).numpy()
    e1 = np.abs(ao.layer_norm(x, g, b) - ref).max()
    # a constant row normalises to the shift exactly
    c = np.full((2, 96), 3.25)
    e2 = np.abs(ao.layer_norm(c, g, b) - b).max()
    return max(e1, e2)


def sdpa_windows(q, k, v, cu, H):
    out = torch.zeros(q.shape, dtype=torch.float64)
    hd = q.shape[1] // H
    for w in range(len(cu) - 1):
        s, e = cu[w], cu[w + 1]

        def heads(t):
            return torch.from_numpy(t[s:e]).reshape(e - s, H, hd).transpose(0, 1)[None]
        o = Fn.scaled_dot_product_attention(heads(q), heads(k), heads(v), is_causal=False)
        out[s:e] = o[0].transpose(0, 1).reshape(e - s, H * hd)
    return out.numpy()


def check_attn():
    T, H, hd = 230, 3, 64
    q, k, v = (RNG.standard_normal((T, H * hd)) for _ in range(3))
    cu = [0, 104, 105, 200, 230]
    e1 = np.abs(ao.window_attention(q, k, v, cu, H) - sdpa_windows(q, k, v, cu, H)).max()
    # one window over everything = dense attention
    e2 = np.abs(ao.window_attention(q, k, v, [0, T], H) - sdpa_windows(q, k, v, [0, T], H)).max()
    # a length-1 window returns v; equal keys return the mean of v
    e3 = np.abs(ao.window_attention(q, k, v, cu, H)[104] - v[104]).max()
    keq = np.tile(k[:1], (T, 1))
    o = ao.window_attention(q, keq, v, [0, 50, T], H)
    e4 = max(np.abs(o[:50] - v[:50].mean(0)).max(), np.abs(o[50:] - v[50:].mean(0)).max())
    return max(e1, e2, e3, e4)


def torch_forward(features, lens, P, cfg):
    """Independent float64 composition of torch library routines: chunks are
    cut with reshape and convolved as a batch, tokens flattened with
    permute/reshape, attention by scaled_dot_product_attention per window."""
    t = {k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in P.items()}
    d, H = cfg["d_model"], cfg["encoder_attention_heads"]
    D = d // 2
    inv = torch.exp(-math.log(10000.0) / (D - 1) * torch.arange(D, dtype=torch.float64))
    pos = torch.arange(13, dtype=torch.float64)[:, None] * inv[None]
    pe = torch.cat([pos.sin(), pos.cos()], 1)
    rows, wl = [], []
    for b, L in enumerate(lens):
        L = int(L)
        if L == 0:
            continue
        n = -(-L // 100)
        x = torch.zeros(128, n * 100, dtype=torch.float64)
        x[:, :L] = torch.from_numpy(features[b, :, :L].astype(np.float64))
        x = x.reshape(128, n, 100).permute(1, 0, 2)[:, None]          # [n, 1, 128, 100]
        for i in (1, 2, 3):
            x = Fn.gelu(Fn.conv2d(x, t[f"conv{i}_w"], t[f"conv{i}_b"], stride=2, padding=1))
        n_, C, Fq, Tq = x.shape
        u = x.permute(0, 3, 1, 2).reshape(n, Tq, C * Fq)              # [n, 13, C*16]
        e = Fn.linear(u, t["conv_out_w"], t.get("conv_out_b")) + pe
        ntok = 13 * (L // 100) + -(-(L % 100) // 8)
        rows.append(e.reshape(n * 13, d)[:ntok] if L % 100 == 0 else
                    torch.cat([e[:-1].reshape(-1, d), e[-1, :ntok - 13 * (n - 1)]]))
        wl += [104] * (ntok // 104) + ([ntok % 104] if ntok % 104 else [])
    x = torch.cat(rows)
    cu = np.cumsum([0] + wl)
    for i in range(cfg["encoder_layers"]):
        p = f"layers.{i}."
        h = Fn.layer_norm(x, (d,), t[p + "ln1_g"], t[p + "ln1_b"], eps=1e-5)
        qkv = Fn.linear(h, t[p + "qkv_w"], t[p + "qkv_b"])
        q, k, v = qkv.split(d, dim=1)
        o = torch.from_numpy(sdpa_windows(q.numpy(), k.numpy(), v.numpy(), cu, H))
        x = x + Fn.linear(o, t[p + "o_w"], t[p + "o_b"])
        h = Fn.layer_norm(x, (d,), t[p + "ln2_g"], t[p + "ln2_b"], eps=1e-5)
        x = x + Fn.linear(Fn.gelu(Fn.linear(h, t[p + "fc1_w"], t[p + "fc1_b"])), t[p + "fc2_w"], t[p + "fc2_b"])
    y = Fn.layer_norm(x, (d,), t["ln_post_g"], t["ln_post_b"], eps=1e-5)
    y = Fn.linear(Fn.gelu(Fn.linear(y, t["proj1_w"], t["proj1_b"])), t["proj2_w"], t["proj2_b"])
    return y.numpy()


COMP = {}


def composition_case(bias=False):
    key = bias
    if key not in COMP:
        cfg = small_cfg(conv_out_bias=bias)
        lens = np.array([250, 0, 800, 37, 1010])
        feats = si.mel_features(lens, seed=7)
        P = si.params(cfg, seed=7, std=0.1)
        COMP[key] = (cfg, lens, feats, P, torch_forward(feats, lens, P, cfg))
    return COMP[key]


def check_composition(bias=False):
    cfg, lens, feats, P, ref = composition_case(bias)
    got, _ = ao.forward(feats, lens, P, cfg)
    if got.shape != ref.shape:
        return float("inf")
    return np.abs(got - ref).max() / np.abs(ref).max()


# ---------------------------------------------------------------------------
# tests
# ---------------------------------------------------------------------------


def test_gelu():
    assert check_gelu() < 1e-14


def test_sinusoid_closed_form():
    assert check_pe() < 1e-9


def test_conv_vs_torch():
    assert check_conv() < 1e-12


def test_layer_norm_vs_torch():
    assert check_ln() < 1e-12


def test_window_attention_vs_sdpa():
    assert check_attn() < 1e-12


@pytest.mark.parametrize("bias", [False, True])
def test_whole_path_vs_torch_composition(bias):
    assert check_composition(bias) < 1e-12


def test_partial_chunk_is_padded_to_full_chunk():
    """m-star ``frontend``: the last piece is zero-padded to a full chunk,
    convolved, then trimmed.  Convolving only the 37 valid frames gives a
    different last token (GELU(bias) != 0 in the padded region)."""
    cfg = small_cfg(encoder_layers=0)
    lens = np.array([137])
    feats = si.mel_features(lens, seed=3)
    P = si.params(cfg, seed=3, std=0.1)
    hid, pl = ao.frontend(feats, lens, P, cfg)
    assert hid.shape[0] == 13 + 5
    img = np.zeros((1, 128, 100))
    img[0, :, :37] = feats[0, :, 100:137]
    a = ao.conv_stem(img, P)
    want = ao.flatten_tokens(a, 5) @ P["conv_out_w"].T.astype(np.float64) + ao.sinusoid_table(13, 128)[:5]
    assert np.abs(hid[13:] - want).max() < 1e-12
    short = ao.conv_stem(img[:, :, :37], P)
    alt = ao.flatten_tokens(short, 5) @ P["conv_out_w"].T.astype(np.float64) + ao.sinusoid_table(13, 128)[:5]
    assert np.abs(alt[:4] - want[:4]).max() < 1e-12      # early tokens agree
    assert np.abs(alt[4] - want[4]).max() > 1e-3         # the last one does not


def test_padding_contents_ignored():
    cfg = small_cfg(encoder_layers=1)
    lens = np.array([137, 301])
    a = si.mel_features(lens, seed=5, pad_value=np.nan)
    b = si.mel_features(lens, seed=5, pad_value=0.0)
    c = si.mel_features(lens, seed=5, pad_value=1e30, t_max=400)
    P = si.params(cfg, seed=5)
    ya, _ = ao.forward(a, lens, P, cfg)
    yb, _ = ao.forward(b, lens, P, cfg)
    yc, _ = ao.forward(c, lens, P, cfg)
    assert np.isfinite(ya).all()
    assert np.array_equal(ya, yb) and np.array_equal(ya, yc)


def test_window_isolation_bitwise():
    """openarchlab "1A", section 4: perturbing one window's spectrogram leaves
    every other window's output unchanged (deviation 0.00e+00)."""
    cfg = small_cfg()
    lens = np.array([1737, 300])
    feats = si.mel_features(lens, seed=11)
    P = si.params(cfg, seed=11, std=0.05)
    y0, pl = ao.forward(feats, lens, P, cfg)
    cu = pl["cu_seqlens"]
    f2 = feats.copy()
    f2[0, :, 800:1600] += 0.5            # window 1 of request 0 = frames 800..1599
    y1, _ = ao.forward(f2, lens, P, cfg)
    changed = [w for w in range(len(cu) - 1) if not np.array_equal(y0[cu[w]:cu[w + 1]], y1[cu[w]:cu[w + 1]])]
    assert changed == [1]


def test_stream_suffix_equals_batch():
    """Windows are independent (m-star module summary; openarchlab "1A",
    section 4), so encoding a request's frames from a window boundary on gives
    exactly its rows from that window's first row on: the basis of the
    incremental encode."""
    cfg = small_cfg()
    L = 1850
    feats = si.mel_features(np.array([L]), seed=9)
    P = si.params(cfg, seed=9, std=0.05)
    y, _ = ao.forward(feats, np.array([L]), P, cfg)
    for wf in (1, 2):
        sub = np.ascontiguousarray(feats[:, :, 800 * wf:])
        ys, _ = ao.forward(sub, np.array([L - 800 * wf]), P, cfg)
        np.testing.assert_array_equal(ys, y[104 * wf:])


def test_request_permutation():
    cfg = small_cfg(encoder_layers=1)
    lens = np.array([250, 800, 37])
    feats = si.mel_features(lens, seed=2)
    P = si.params(cfg, seed=2)
    y, pl = ao.forward(feats, lens, P, cfg)
    perm = [2, 0, 1]
    y2, pl2 = ao.forward(feats[perm], lens[perm], P, cfg)
    off = np.cumsum([0] + pl["tokens_per_request"])
    rows = np.concatenate([np.arange(off[b], off[b + 1]) for b in perm])
    assert np.array_equal(y[rows], y2)


def test_forward_windows_exact():
    cfg = small_cfg()
    lens = np.array([1737, 300, 0, 905])
    feats = si.mel_features(lens, seed=4)
    P = si.params(cfg, seed=4, std=0.05)
    y, pl = ao.forward(feats, lens, P, cfg)
    nw = len(pl["cu_seqlens"]) - 1
    part = ao.forward_windows(feats, lens, P, cfg, range(nw))
    for w, (r0, yw) in part.items():
        np.testing.assert_array_equal(yw, y[r0:r0 + yw.shape[0]])


# planted mistakes: each must make its pin fail


def check_power():
    import torch
    x = np.random.default_rng(41).normal(size=7 * 160 + 91)
    ref = torch.stft(torch.from_numpy(x), 400, 160, window=torch.hann_window(400, dtype=torch.float64),
                     center=True, pad_mode="reflect", return_complex=True)
    ref = (ref.abs() ** 2)[:, :-1].numpy().T
    got = ao.power_spectrum(x)
    if got.shape != ref.shape:
        return float("inf")
    return float(np.abs(got - ref).max() / np.abs(ref).max())


def check_mel_scale():
    e1 = np.abs(ao.hz_to_mel(np.array([0.0, 500.0, 1000.0, 6400.0])) - np.array([0.0, 7.5, 15.0, 42.0])).max()
    f = np.linspace(0, 8000, 321)
    e2 = np.abs(ao.mel_to_hz(ao.hz_to_mel(f)) - f).max()
    return float(max(e1, e2))


def check_fbank():
    w = ao.mel_filterbank(128)
    pts = ao.mel_to_hz(np.linspace(0.0, float(ao.hz_to_mel(8000.0)), 130))
    freqs = np.linspace(0, 8000, 201)
    tri = w * ((pts[2:] - pts[:-2]) / 2.0)[:, None]
    inside = (freqs >= pts[1]) & (freqs <= pts[128])
    return float(np.abs(tri.sum(axis=0)[inside] - 1.0).max())


def check_log_mel():
    import torch
    rng = np.random.default_rng(43)
    # a loud part and silence: a dynamic range well over the floor's 8 decades
    x = np.concatenate([rng.normal(size=3200) * 1000.0, np.zeros(1600)])
    spec = torch.stft(torch.from_numpy(x), 400, 160, window=torch.hann_window(400, dtype=torch.float64),
                      center=True, pad_mode="reflect", return_complex=True)[:, :-1]
    mel = torch.from_numpy(ao.mel_filterbank(128)) @ (spec.abs() ** 2)
    lg = torch.clamp(mel, min=1e-10).log10()
    lg = torch.maximum(lg, lg.max() - 8.0)
    ref = ((lg + 4.0) / 4.0).numpy()
    got = ao.log_mel(x)
    e = float(np.abs(got - ref).max()) if got.shape == ref.shape else float("inf")
    return max(e, abs(ao.frames_for_samples(16000) - 100) * 1.0)


def torch_mx_round(x, block=32):
    """MX-fp8 round trip built independently: the block exponent by a search
    over every E8M0 value, the element rounding by torch's float8_e4m3fn."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    xb = x.reshape(-1, block)
    out = np.empty_like(xb)
    for i, blk in enumerate(xb):
        amax = np.abs(blk).max()
        e = -127
        while e < 127 and amax > 448.0 * 2.0 ** e:
            e += 1
        t = torch.from_numpy((blk / 2.0 ** e).astype(np.float32)).to(torch.float8_e4m3fn)
        out[i] = t.to(torch.float64).numpy() * 2.0 ** e
    return out.reshape(x.shape)


def check_e4m3_round():
    """the direct rounding against the code table, value by value"""
    r = np.random.default_rng(12)
    x = r.uniform(-1, 1, 50000) * np.exp2(r.integers(-14, 9, 50000))
    vals = ao.e4m3_decode(np.arange(127))
    x = np.concatenate([x[np.abs(x) <= 448], (vals[1:] + vals[:-1]) / 2, -vals, [0.0]])
    return float(np.abs(ao.e4m3_round(x) - ao.e4m3_decode(ao.e4m3_encode(x))).max())


def check_e4m3():
    r = np.random.default_rng(5)
    x = (r.uniform(-1, 1, 20000) * np.exp2(r.integers(-12, 9, 20000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    vals = ao.e4m3_decode(np.arange(127)).astype(np.float32)
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)        # exact in fp32
    x = np.concatenate([x, mids, -mids, vals])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return float(np.count_nonzero(ao.e4m3_encode(x.astype(np.float64)) != ref))


def check_mx():
    r = np.random.default_rng(6)
    x = r.standard_normal((24, 128)) * np.exp2(r.integers(-20, 20, (24, 1)))
    x[3, 32:64] = 0.0
    x[5, :32] = 448.0 * 2.0 ** -3              # block maximum exactly on a scale boundary
    # e4m3 rounding is scale-free except below the normal range: blocks whose
    # first value dwarfs the rest put the others into the subnormal range
    x[7:12] = r.standard_normal((5, 128)) * 2.0 ** -14
    x[7:12, ::32] = 1.0
    x = x.astype(np.float32).astype(np.float64)
    ref = torch_mx_round(x)
    worst = 0.0
    # the value path (mx_round) and the code path (quantize, then dequantize)
    for f in (ao.mx_round, lambda v: ao.mx_dequantize(*ao.mx_quantize(v))):
        try:
            got = f(x)
        except ValueError:                      # an element past the e4m3 range
            return float("inf")
        d = np.abs(got - ref).reshape(-1, 32)
        worst = max(worst, float((d / np.abs(x).reshape(-1, 32).max(1, keepdims=True).clip(1e-300)).max()))
    return worst


def check_linear_mx():
    r = np.random.default_rng(7)
    x = r.standard_normal((16, 96)).astype(np.float32).astype(np.float64)
    w = (r.standard_normal((40, 96)) * 0.02).astype(np.float32).astype(np.float64)
    b = r.standard_normal(40)
    ref = torch_mx_round(x) @ torch_mx_round(w).T + b
    return float(np.abs(ao.linear_mx(x, w, b) - ref).max())


def check_conv_mx():
    """conv2d_k3s2p1_mx against an explicit im2col product, k = tap * C + c,
    rounded with the torch-built MX quantizer."""
    r = np.random.default_rng(13)
    x = r.standard_normal((64, 7, 6))
    x[:16] *= 2.0 ** -16        # the blocks matter only where they mix magnitudes
    x = x.astype(np.float32).astype(np.float64)
    w = (r.standard_normal((5, 64, 3, 3)) * 0.1).astype(np.float32).astype(np.float64)
    b = r.standard_normal(5)
    Ho, Wo = 4, 3
    xp = np.pad(x, ((0, 0), (1, 1), (1, 1)))
    cols = np.zeros((Ho * Wo, 9 * 64))
    for oy in range(Ho):
        for ox in range(Wo):
            for kh in range(3):
                for kw in range(3):
                    t = 3 * kh + kw
                    cols[oy * Wo + ox, t * 64:(t + 1) * 64] = xp[:, 2 * oy + kh, 2 * ox + kw]
    wm = np.zeros((5, 9 * 64))
    for kh in range(3):
        for kw in range(3):
            t = 3 * kh + kw
            wm[:, t * 64:(t + 1) * 64] = w[:, :, kh, kw]
    ref = (torch_mx_round(cols) @ torch_mx_round(wm).T + b).T.reshape(5, Ho, Wo)
    return float(np.abs(ao.conv2d_k3s2p1_mx(x, w, b) - ref).max())


def check_conv_out_mx():
    """conv_out on MX-fp8 against an explicit reorder to f * C + c."""
    r = np.random.default_rng(14)
    C, F = 64, 16
    u = r.standard_normal((7, C * F))
    u[:, 0::2] *= 2.0 ** -16    # even bins (index c * F + f, F even) tiny
    u = u.astype(np.float32).astype(np.float64)
    w = (r.standard_normal((9, C * F)) * 0.05).astype(np.float32).astype(np.float64)
    b = r.standard_normal(9)
    ub = np.zeros_like(u)
    wb = np.zeros_like(w)
    for f in range(F):
        for c in range(C):
            ub[:, f * C + c] = u[:, c * F + f]
            wb[:, f * C + c] = w[:, c * F + f]
    ref = torch_mx_round(ub) @ torch_mx_round(wb).T + b
    return float(np.abs(ao.linear_conv_out_mx(u, w, b, F) - ref).max())


MUTATIONS = {
    "conv kernel transposed": ("conv2d_k3s2p1", lambda orig: (lambda x, w, b: orig(x, np.swapaxes(w, 2, 3), b)), check_conv),
    "conv bias dropped": ("conv2d_k3s2p1", lambda orig: (lambda x, w, b: orig(x, w, np.zeros_like(b))), check_conv),
    "ln unbiased variance": ("layer_norm", lambda orig: (lambda x, g, b, eps=1e-5: (x - x.mean(-1, keepdims=True)) / np.sqrt(x.var(-1, ddof=1, keepdims=True) + eps) * g + b), check_ln),
    "ln gain/shift swapped": ("layer_norm", lambda orig: (lambda x, g, b, eps=1e-5: orig(x, b, g, eps)), check_ln),
    "attention scale 1/hd": ("window_attention", lambda orig: (lambda q, k, v, cu, H: orig(q * (1.0 / 8.0), k, v, cu, H)), check_attn),
    "attention causal": ("window_attention", lambda orig: _causal_attn, check_attn),
    "attention across windows": ("window_attention", lambda orig: (lambda q, k, v, cu, H: orig(q, k, v, [cu[0], cu[-1]], H)), check_attn),
    "pe sin/cos swapped": ("sinusoid_table", lambda orig: (lambda n, c: np.roll(orig(n, c), c // 2, axis=1)), check_pe),
    "pe increment ln/D": ("sinusoid_table", lambda orig: _pe_wrong_inc, check_pe),
    "gelu tanh approx": ("gelu", lambda orig: (lambda x: 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))), check_gelu),
    "flatten f-major": ("flatten_tokens", lambda orig: (lambda a3, vt: a3[:, :, :vt].transpose(2, 1, 0).reshape(vt, -1)), check_composition),
    "linear bias dropped": ("linear", lambda orig: (lambda x, w, b=None: orig(x, w, None)), check_composition),
    "post-LN layer order": ("encoder_layer", lambda orig: _post_ln_layer, check_composition),
    "qkv split k/v swapped": ("window_attention", lambda orig: (lambda q, k, v, cu, H: orig(q, v, k, cu, H)), check_composition),
    "positions not chunk-local": ("sinusoid_table", lambda orig: (lambda n, c: orig(n + 1, c)[1:]), check_composition),
    "magnitude instead of power": ("power_spectrum", lambda orig: (lambda a: np.sqrt(orig(a))), check_power),
    "symmetric Hann": ("hann", lambda orig: (lambda n=400: 0.5 - 0.5 * np.cos(2 * np.pi * np.arange(n) / (n - 1))), check_power),
    "HTK mel scale": ("hz_to_mel", lambda orig: (lambda f: 2595.0 * np.log10(1.0 + np.asarray(f, dtype=np.float64) / 700.0)), check_mel_scale),
    "filterbank not unit area": ("mel_filterbank", lambda orig: (lambda n=128: orig(n) / orig(n).max(axis=1, keepdims=True)), check_fbank),
    "last frame kept": ("frames_for_samples", lambda orig: (lambda n: int(n) // 160 + 1), check_log_mel),
    "natural log": ("log_mel", lambda orig: _log_mel_ln, check_log_mel),
    "floor at max - 10": ("log_mel", lambda orig: _log_mel_floor10, check_log_mel),
    "e4m3 truncated": ("e4m3_encode", lambda orig: _e4m3_trunc, check_e4m3),
    "e4m3 ties away from zero": ("e4m3_encode", lambda orig: (lambda x: orig(np.clip(np.asarray(x, dtype=np.float64) * (1 + 2.0 ** -40), -448, 448))), check_e4m3),
    "mx block of 16": ("MX_BLOCK", lambda orig: 16, check_mx),
    "e4m3 round half up": ("e4m3_round", lambda orig: (lambda x: _e4m3_round_half_up(x)), check_e4m3_round),
    "e4m3 round no subnormal floor": ("e4m3_round", lambda orig: _e4m3_round_no_subnormal, check_mx),
    "mx floor exponent rule": ("mx_block_exponent", lambda orig: (lambda a: np.where(np.asarray(a) > 0, np.floor(np.log2(np.where(np.asarray(a) > 0, a, 1.0))) - 8, -127).astype(np.int64)), check_mx),
    "mx scale bias 128": ("mx_dequantize", lambda orig: (lambda c, sc: orig(c, np.asarray(sc, dtype=np.int64) - 1)), check_mx),
    "mx weights left unquantized": ("linear_mx", lambda orig: (lambda x, w, b=None: ao.linear(ao.mx_round(x), w, b)), check_linear_mx),
    "conv mx blocks across taps": ("conv2d_k3s2p1_mx", lambda orig: _conv_mx_c_major, check_conv_mx),
    "conv_out mx channel-major blocks": ("linear_conv_out_mx", lambda orig: (lambda u, w, b, F: ao.linear_mx(u, w, b)), check_conv_out_mx),
}


def _conv_mx_c_major(x, w, b):
    """planted: the contraction blocks taken in the channel-major order c * 9 + tap"""
    cin, H, W = x.shape
    Ho, Wo = ao.conv_out_len(H), ao.conv_out_len(W)
    xp = np.pad(x, ((0, 0), (1, 1), (1, 1)))
    cols = np.stack([xp[:, kh:kh + 2 * Ho:2, kw:kw + 2 * Wo:2] for kh in range(3) for kw in range(3)], 1)
    cols = cols.reshape(cin * 9, Ho * Wo).T                    # k = c * 9 + tap
    wm = w.reshape(w.shape[0], cin * 9)
    return (ao.mx_round(cols) @ ao.mx_round(wm).T + b).T.reshape(-1, Ho, Wo)


def _e4m3_round_half_up(x):
    x = np.asarray(x, dtype=np.float64)
    _, E = np.frexp(x)
    q = np.maximum(E - 1, -6) - 3
    return np.sign(x) * np.ldexp(np.floor(np.ldexp(np.abs(x), -q) + 0.5), q)


def _e4m3_round_no_subnormal(x):
    x = np.asarray(x, dtype=np.float64)
    _, E = np.frexp(x)
    q = E - 1 - 3
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)


def _e4m3_trunc(x):
    x = np.asarray(x, dtype=np.float64)
    vals = ao.e4m3_decode(np.arange(127))
    code = np.searchsorted(vals, np.abs(x), side="right") - 1
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def _log_mel_ln(audio, n_mels=128):
    p = ao.power_spectrum(audio)
    lg = np.log(np.maximum(ao.mel_filterbank(n_mels) @ p.T, 1e-10))
    lg = np.maximum(lg, lg.max() - 8.0)
    return (lg + 4.0) / 4.0


def _log_mel_floor10(audio, n_mels=128):
    p = ao.power_spectrum(audio)
    lg = np.log10(np.maximum(ao.mel_filterbank(n_mels) @ p.T, 1e-10))
    lg = np.maximum(lg, lg.max() - 10.0)
    return (lg + 4.0) / 4.0


def _causal_attn(q, k, v, cu, H):
    T, d = q.shape
    hd = d // H
    out = np.zeros((T, d))
    for w in range(len(cu) - 1):
        s, e = cu[w], cu[w + 1]
        for h in range(H):
            c = slice(h * hd, (h + 1) * hd)
            sc = q[s:e, c] @ k[s:e, c].T / math.sqrt(hd)
            sc = sc + np.triu(np.full((e - s, e - s), -np.inf), 1)
            out[s:e, c] = ao.softmax(sc) @ v[s:e, c]
    return out


def _pe_wrong_inc(n, c):
    D = c // 2
    tau = np.exp(-math.log(10000.0) / D * np.arange(D))
    t = np.arange(n)[:, None] * tau[None]
    return np.concatenate([np.sin(t), np.cos(t)], 1)


def _post_ln_layer(x, cu, P, i, cfg, fp8=0):
    p = f"layers.{i}."
    d = cfg["d_model"]
    qkv = ao.linear(x, P[p + "qkv_w"], P[p + "qkv_b"])
    o = ao.window_attention(qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:], cu, cfg["encoder_attention_heads"])
    x = ao.layer_norm(x + ao.linear(o, P[p + "o_w"], P[p + "o_b"]), P[p + "ln1_g"], P[p + "ln1_b"])
    f = ao.gelu(ao.linear(x, P[p + "fc1_w"], P[p + "fc1_b"]))
    return ao.layer_norm(x + ao.linear(f, P[p + "fc2_w"], P[p + "fc2_b"]), P[p + "ln2_g"], P[p + "ln2_b"])


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes(name, monkeypatch):
    attr, make, check = MUTATIONS[name]
    orig = getattr(ao, attr)
    composition_case(False)  # reference computed before patching
    monkeypatch.setattr(ao, attr, make(orig))
    err = check()
    assert err > 1e-6, f"pin did not catch: {name} (err={err})"


# ---------------------------------------------------------------------------
# audio rows into the decoder sequence
# ---------------------------------------------------------------------------


def test_inject_audio_worked_example():
    """Placeholders take the audio rows in order; other rows keep their text
    embedding; the count must match."""
    PAD = 151676
    ids = [9, PAD, 4, PAD, PAD, 7]
    emb = np.arange(6 * 3, dtype=np.float64).reshape(6, 3)
    aud = -np.arange(1, 10, dtype=np.float64).reshape(3, 3)
    out = ao.inject_audio(emb, ids, PAD, aud)
    expect = np.array([[0, 1, 2], [-1, -2, -3], [6, 7, 8], [-4, -5, -6], [-7, -8, -9], [15, 16, 17]],
                      dtype=np.float64)
    np.testing.assert_array_equal(out, expect)
    np.testing.assert_array_equal(ao.audio_rows(ids, PAD, 3), [1, 3, 4])
    with pytest.raises(ValueError):
        ao.audio_rows(ids, PAD, 2)
    with pytest.raises(ValueError):
        ao.inject_audio(emb, ids, PAD, aud[:2])


def test_bf16_round_vs_torch():
    """Round-to-nearest-even to bfloat16 against torch's conversion, including
    ties and values at the edges of the exponent range."""
    torch = pytest.importorskip("torch")
    x = np.concatenate([RNG.normal(size=4000) * 10.0 ** RNG.integers(-30, 30, 4000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.0e38, 1e-40, 0.0])])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ao.bf16_round(x32), ref)


# ---------------------------------------------------------------------------
# log-mel front end
# ---------------------------------------------------------------------------


def test_log_mel_page_rates():
    """16 kHz mono in, 100 frames per second, 128 bins out (cubic.dev wiki,
    Processing Pipeline; m-star module summary)."""
    x = RNG.normal(size=16000)
    assert ao.frames_for_samples(16000) == 100
    assert ao.log_mel(x).shape == (128, 100)
    assert ao.power_spectrum(RNG.normal(size=800 * 160 + 37)).shape == (800, 201)


def test_mel_scale_special_points():
    """Slaney scale: 0 Hz -> 0, 1 kHz -> 15 mel (end of the linear part),
    6.4 kHz -> 42 mel (one factor 6.4 above 1 kHz = 27 mel), and round trips."""
    np.testing.assert_allclose(ao.hz_to_mel([0.0, 1000.0, 6400.0]), [0.0, 15.0, 42.0], atol=1e-12)
    np.testing.assert_allclose(ao.hz_to_mel(500.0), 7.5, atol=1e-12)
    f = np.linspace(0, 8000, 321)
    np.testing.assert_allclose(ao.mel_to_hz(ao.hz_to_mel(f)), f, atol=1e-9)


def test_mel_filterbank_structure():
    """Triangles with unit area: scaled back by (upper - lower) / 2 they form a
    partition of unity between the first and last centre frequency, each
    non-zero only between its neighbours' centres, peaking at its own."""
    w = ao.mel_filterbank(128)
    assert w.shape == (128, 201) and (w >= 0).all()
    pts = ao.mel_to_hz(np.linspace(0.0, float(ao.hz_to_mel(8000.0)), 130))
    freqs = np.linspace(0, 8000, 201)
    tri = w * ((pts[2:] - pts[:-2]) / 2.0)[:, None]
    inside = (freqs >= pts[1]) & (freqs <= pts[128])
    np.testing.assert_allclose(tri.sum(axis=0)[inside], 1.0, atol=1e-12)
    for m in range(128):
        nz = np.nonzero(w[m])[0]
        if nz.size:
            assert freqs[nz].min() > pts[m] - 1e-9 and freqs[nz].max() < pts[m + 2] + 1e-9
            assert abs(freqs[nz[np.argmax(w[m, nz])]] - pts[m + 1]) <= 20.0 + 1e-9


def test_power_spectrum_vs_torch_stft():
    """Framing, window and DFT against torch.stft (centred, reflect padding,
    periodic Hann, last frame dropped)."""
    torch = pytest.importorskip("torch")
    x = RNG.normal(size=7 * 160 + 91)
    ref = torch.stft(torch.from_numpy(x), 400, 160, window=torch.hann_window(400, dtype=torch.float64),
                     center=True, pad_mode="reflect", return_complex=True)
    ref = (ref.abs() ** 2)[:, :-1].numpy().T
    np.testing.assert_allclose(ao.power_spectrum(x), ref, rtol=1e-10, atol=1e-9)


def test_power_spectrum_pure_tone():
    """A cosine on DFT bin k: in every frame away from the edges the power sits
    in bins k-1, k, k+1 with the Hann window's closed-form weights
    (N/4 * A)^2 and (N/8 * A)^2."""
    A, k = 0.3, 25
    n = np.arange(50 * 160)
    x = A * np.cos(2 * np.pi * k * n / 400)
    p = ao.power_spectrum(x)[5:-5]
    np.testing.assert_allclose(p[:, k], (400 / 4 * A) ** 2, rtol=1e-9)
    np.testing.assert_allclose(p[:, k - 1], (400 / 8 * A) ** 2, rtol=1e-9)
    np.testing.assert_allclose(p[:, k + 1], (400 / 8 * A) ** 2, rtol=1e-9)
    rest = np.delete(p, [k - 1, k, k + 1], axis=1)
    assert rest.max() < 1e-18 * p[:, k].max() + 1e-20


def test_log_mel_floor_and_scale():
    """Silence: every value log10(1e-10) = -10 -> (-10 + 4) / 4 = -1.5; the floor
    keeps the dynamic range to 8 (in log10 units, 2 after the scaling)."""
    np.testing.assert_array_equal(ao.log_mel(np.zeros(3200)), np.full((128, 20), -1.5))
    y = ao.log_mel(RNG.normal(size=32000) * np.exp(RNG.normal(size=32000) * 3))
    assert y.max() - y.min() <= 2.0 + 1e-12
    torch = pytest.importorskip("torch")
    x = RNG.normal(size=4800)
    spec = torch.stft(torch.from_numpy(x), 400, 160, window=torch.hann_window(400, dtype=torch.float64),
                      center=True, pad_mode="reflect", return_complex=True)[:, :-1]
    mel = torch.from_numpy(ao.mel_filterbank(128)) @ (spec.abs() ** 2)
    lg = torch.clamp(mel, min=1e-10).log10()
    lg = torch.maximum(lg, lg.max() - 8.0)
    np.testing.assert_allclose(ao.log_mel(x), ((lg + 4.0) / 4.0).numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# MX-fp8 products (OCP 8-bit floating point and Microscaling formats)
# ---------------------------------------------------------------------------


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = ao.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    # closed forms of the format: largest finite, smallest subnormal and normal, one, NaNs
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and np.count_nonzero(np.isnan(got)) == 2
    assert np.all(np.diff(got[:127]) > 0)


def test_e4m3_encode_vs_torch():
    assert check_e4m3() == 0


def test_e4m3_round_equals_code_table():
    assert check_e4m3_round() == 0


def test_e4m3_ties_to_even():
    x = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 432.0, -1.0625, 0.0])
    assert list(ao.e4m3_encode(x)) == [0x38, 0x3A, 0x00, 0x02, 0x7E, 0xB8, 0x00]
    with pytest.raises(ValueError):
        ao.e4m3_encode(np.array([449.0]))


def test_mx_block_exponent_brute_force():
    r = np.random.default_rng(8)
    a = np.concatenate([r.uniform(0, 1, 400) * np.exp2(r.integers(-60, 60, 400)),
                        448.0 * np.exp2(np.arange(-20, 20, dtype=np.float64)),
                        np.nextafter(448.0 * np.exp2(np.arange(-20, 20, dtype=np.float64)), np.inf),
                        [0.0, 1e-300, 1e300]])
    got = ao.mx_block_exponent(a)
    for ai, e in zip(a, got):
        want = -127
        while want < 127 and ai > 448.0 * 2.0 ** want:
            want += 1
        assert e == want, (ai, e, want)


def test_mx_quantize_matches_independent_build():
    assert check_mx() == 0


def test_mx_quantize_bounds_and_representable_identity():
    r = np.random.default_rng(9)
    x = r.standard_normal((64, 256))
    codes, sc = ao.mx_quantize(x)
    v = ao.e4m3_decode(codes).reshape(64, 8, 32)
    amax = np.abs(v).max(-1)
    assert np.all((amax >= 224) & (amax <= 448))             # the smallest scale that fits
    q = ao.mx_dequantize(codes, sc)
    rel = np.abs(q - x) / np.abs(x)
    assert rel[np.abs(x) > np.repeat(np.abs(x).reshape(64, 8, 32).max(-1), 32, 1) / 2**6].max() <= 2.0 ** -4
    # MX-representable input: the round trip is the identity
    assert np.array_equal(ao.mx_round(q), q)
    assert np.array_equal(ao.linear_mx(q, q[:16]), q @ q[:16].T)


def test_linear_mx_vs_independent_build():
    assert check_linear_mx() < 1e-12


def test_conv_mx_vs_im2col():
    assert check_conv_mx() < 1e-12


def test_conv_out_mx_vs_reorder():
    assert check_conv_out_mx() < 1e-12


def test_stem_mx_is_one_per_pixel_quantisation():
    """The three MX-fp8 stem products see the same rounding of an activation:
    conv2 / conv3 on MX operands equal the exact convolution of the input
    rounded per pixel (blocks of 32 channels) with the weights rounded per tap
    over input channels; conv_out on MX operands equals the exact product of
    the per-pixel-rounded stem output, flattened c * 16 + f, with the weight
    rounded over each bin's 32-channel groups."""
    r = np.random.default_rng(21)
    C, F, T = 64, 16, 5
    x = r.standard_normal((C, 9, 8)) * np.exp2(r.integers(-8, 8, (C, 1, 1)))
    w = r.standard_normal((7, C, 3, 3)) * 0.05
    b = r.standard_normal(7)
    wq = np.zeros_like(w)
    for kh in range(3):
        for kw in range(3):
            wq[:, :, kh, kw] = torch_mx_round(w[:, :, kh, kw])
    ref = ao.conv2d_k3s2p1(ao.mx_round_pixels(x), wq, b)
    assert np.abs(ao.conv2d_k3s2p1_mx(x, w, b) - ref).max() < 1e-12
    a3 = r.standard_normal((C, F, T)) * np.exp2(r.integers(-8, 8, (C, 1, 1)))
    wo = r.standard_normal((9, C * F)) * 0.05
    u = ao.flatten_tokens(a3, T)
    uq = ao.flatten_tokens(ao.mx_round_pixels(a3), T)
    woq = np.zeros_like(wo)
    for f in range(F):
        cols = np.arange(C) * F + f
        woq[:, cols] = torch_mx_round(wo[:, cols])
    ref = uq @ woq.T
    assert np.abs(ao.linear_conv_out_mx(u, wo, None, F) - ref).max() < 1e-12


def test_fp8_encoder_masks():
    cfg = small_cfg(encoder_layers=1, downsample_hidden_size=32)
    lens = np.array([420], dtype=np.int32)
    feats = si.mel_features(lens, seed=3)
    P = si.params(cfg, seed=4)
    base, _ = ao.forward(feats, lens, P, cfg)
    same, _ = ao.forward(feats, lens, P, cfg, fp8=0)
    assert np.array_equal(base, same)
    cos_all = None
    for bit in (ao.FP8_QKV, ao.FP8_OUT, ao.FP8_FC1, ao.FP8_FC2, ao.FP8_PROJ, ao.FP8_CONV, ao.FP8_ALL):
        out, _ = ao.forward(feats, lens, P, cfg, fp8=bit)
        assert not np.array_equal(out, base)
        cos = (out * base).sum(1) / np.linalg.norm(out, axis=1) / np.linalg.norm(base, axis=1)
        assert cos.min() > 0.99, (bit, cos.min())
        if bit == ao.FP8_ALL:
            cos_all = cos.min()
    assert cos_all < 0.99999
