"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Stage-wise on a small ragged configuration (fp32 and bf16), then every named
workload: the tiny fp32 one and the ragged bf16 one on their whole output,
the three large bf16 ones on a seeded sample of windows that the oracle
computes exactly (windows are independent end to end).
Tolerances: fp32 max_i |g - r| / max(|r_i|, rms r) <= 1e-4; bf16 max-abs
<= 2e-2 and per-token cosine >= 0.999; the plan is compared exactly.
"""
import numpy as np
import pytest

import oracle
import synth_inputs as si
from gpu_common import (check, forward, pack, features_dev, sample_windows, small_cfg, torch_mod,
                        workload)

pytestmark = pytest.mark.gpu

SMALL_LENS = np.array([250, 0, 800, 37, 1737, 5, 100, 101])


def small_case(dtype, **kw):
    cfg = small_cfg(dtype, **kw)
    feats = si.mel_features(SMALL_LENS, seed=21)
    P = si.params(cfg, seed=21, std=0.05)
    return cfg, SMALL_LENS, feats, P


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_small_stages(dtype):
    """frontend, encode and the whole forward separately."""
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    cfg_d, lens, feats, P = small_case(dtype)
    print(f"case: small {dtype} lens={list(lens)}", flush=True)
    cfg, packed = pack(cfg_d, P)
    pl = aut.plan(cfg, lens)
    ws = aut.workspace(cfg, pl, dtype)
    aut.plan_upload(pl, ws)
    T = pl.total_tokens
    hid = torch.empty((T, cfg_d["d_model"]), dtype=torch.float32, device="cuda")
    aut.frontend(cfg, pl, features_dev(feats), packed, dtype, hid, ws)
    torch.cuda.synchronize()
    ref_hid, opl = oracle.frontend(feats, lens, P, cfg_d)
    assert pl.copy()[1] == opl["cu_seqlens"]
    check(hid.double().cpu().numpy(), ref_hid, dtype, "frontend")

    out = torch.empty((T, cfg_d["output_dim"]), dtype=torch.float32, device="cuda")
    aut.encode_packed(cfg, pl, torch.from_numpy(ref_hid.astype(np.float32)).cuda(), packed, dtype, out, ws)
    torch.cuda.synchronize()
    ref_enc = oracle.encode(ref_hid.astype(np.float32).astype(np.float64), opl["cu_seqlens"], P, cfg_d)
    check(out.double().cpu().numpy(), ref_enc, dtype, "encode")

    y, _ = forward(cfg_d, lens, feats, packed=packed, cfg=cfg)
    ref, _ = oracle.forward(feats, lens, P, cfg_d)
    check(y, ref, dtype, "forward")


def test_small_conv_out_bias():
    cfg_d, lens, feats, P = small_case("fp32")
    cfg_d = dict(cfg_d, conv_out_bias=True)
    P = si.params(cfg_d, seed=22, std=0.05)
    y, _ = forward(cfg_d, lens, feats, P)
    ref, _ = oracle.forward(feats, lens, P, cfg_d)
    check(y, ref, "fp32", "conv_out bias")


@pytest.mark.parametrize("lens", [[1], [7, 8, 9], [99, 100, 101], [800, 801, 1599, 1600, 1601]])
def test_edge_lengths(lens):
    cfg_d = small_cfg("fp32", encoder_layers=1)
    lens = np.array(lens)
    feats = si.mel_features(lens, seed=5)
    P = si.params(cfg_d, seed=5, std=0.05)
    y, pl = forward(cfg_d, lens, feats, P)
    ref, opl = oracle.forward(feats, lens, P, cfg_d)
    assert pl.copy()[1] == opl["cu_seqlens"]
    check(y, ref, "fp32", f"lens {list(lens)}")


@pytest.mark.parametrize("n_window_infer,dtype", [(100, "bf16"), (400, "fp32"), (900, "bf16")])
def test_window_sizes(n_window_infer, dtype):
    """Windows of 13, 52 and 117 tokens (1, 4 and 9 chunks; 117 is the largest
    that fits the 128-key attention tile), ragged requests with partial last
    chunks and windows: the whole output against the oracle."""
    cfg_d = small_cfg(dtype, n_window_infer=n_window_infer)
    lens = np.array([250, 0, 1737, 37, 901, 2600])
    feats = si.mel_features(lens, seed=61)
    P = si.params(cfg_d, seed=61, std=0.05)
    print(f"case: window of {13 * n_window_infer // 100} tokens, {dtype}", flush=True)
    y, pl = forward(cfg_d, lens, feats, P)
    ref, opl = oracle.forward(feats, lens, P, cfg_d)
    assert pl.copy()[1] == opl["cu_seqlens"]
    assert max(np.diff(opl["cu_seqlens"])) == 13 * n_window_infer // 100
    check(y, ref, dtype, f"window {13 * n_window_infer // 100} tokens")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_attention_key_tile_paths(dtype):
    """Windows on each side of the attention kernel's key-tile boundaries: 96
    (every tile masked), 97 and 112 (the eighth key tile skipped, the seventh
    masked), 113 and 117 (all eight tiles, the last masked), with 117-token
    windows (9 chunks) and single-chunk leftovers; the whole output against the
    oracle."""
    cfg_d = small_cfg(dtype, n_window_infer=900)
    lens = np.array([740, 748, 864, 872, 900, 1764, 1])
    feats = si.mel_features(lens, seed=67)
    P = si.params(cfg_d, seed=67, std=0.05)
    print(f"case: key-tile paths, {dtype}", flush=True)
    y, pl = forward(cfg_d, lens, feats, P)
    ref, opl = oracle.forward(feats, lens, P, cfg_d)
    assert pl.copy()[1] == opl["cu_seqlens"]
    wl = sorted(set(np.diff(opl["cu_seqlens"]).tolist()))
    assert {96, 97, 112, 113, 117, 1} <= set(wl), wl
    check(y, ref, dtype, f"key-tile paths, windows {wl}")


@pytest.mark.parametrize("n_window,n_window_infer,dtype", [(25, 400, "fp32"), (60, 960, "bf16"),
                                                          (10, 160, "bf16")])
def test_chunk_sizes(n_window, n_window_infer, dtype):
    """Chunks of 50, 120 and 20 frames (7, 15 and 3 tokens per chunk, windows of
    8 chunks): other stem geometries and position counts, whole output."""
    cfg_d = small_cfg(dtype, n_window=n_window, n_window_infer=n_window_infer)
    lens = np.array([250, 0, 1737, 37, 901])
    feats = si.mel_features(lens, seed=67)
    P = si.params(cfg_d, seed=67, std=0.05)
    print(f"case: chunks of {2 * n_window} frames, {dtype}", flush=True)
    y, pl = forward(cfg_d, lens, feats, P)
    ref, opl = oracle.forward(feats, lens, P, cfg_d)
    assert pl.copy()[1] == opl["cu_seqlens"]
    check(y, ref, dtype, f"chunks of {2 * n_window} frames")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_odd_widths(dtype):
    """d_model 192 (3 heads), FFN 200, 24 conv channels, output 72: column
    tails in every GEMM tile, a k tail in fc2 (K = 200), conv taps of 24
    channels inside a 64-wide k step; whole output."""
    cfg_d = small_cfg(dtype, d_model=192, encoder_attention_heads=3, encoder_ffn_dim=200,
                      downsample_hidden_size=24, output_dim=72)
    lens = np.array([250, 0, 1737, 37, 901])
    feats = si.mel_features(lens, seed=71)
    P = si.params(cfg_d, seed=71, std=0.05)
    print(f"case: odd widths, {dtype}", flush=True)
    y, pl = forward(cfg_d, lens, feats, P)
    ref, opl = oracle.forward(feats, lens, P, cfg_d)
    assert pl.copy()[1] == opl["cu_seqlens"]
    check(y, ref, dtype, f"odd widths {dtype}")


def test_empty_batch():
    from packed_windowed_attention_amd import aut
    cfg_d = small_cfg("fp32", encoder_layers=1)
    P = si.params(cfg_d, seed=1)
    cfg, packed = pack(cfg_d, P)
    feats = features_dev(si.mel_features([0, 0], seed=1))
    out, pl = aut.encode(cfg, feats, [0, 0], packed, "fp32")
    assert pl.total_tokens == 0 and out.shape[0] == 0


def test_padding_contents_ignored():
    """Buffer contents past each length (NaN, zeros, huge values) never matter."""
    cfg_d, lens, _, P = small_case("bf16")
    cfg, packed = pack(cfg_d, P)
    outs = []
    for pad, tmax in [(np.nan, None), (0.0, None), (1e30, 2000)]:
        feats = si.mel_features(lens, seed=21, pad_value=pad, t_max=tmax)
        y, _ = forward(cfg_d, lens, feats, packed=packed, cfg=cfg)
        outs.append(y)
    assert np.isfinite(outs[0]).all()
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_tiny_fp32():
    """1 request of 8 s, 1 layer d 1280, C 128, fp32: whole output."""
    cfg_d, lens, feats, P = workload("tiny")
    print("case: tiny fp32", flush=True)
    y, pl = forward(cfg_d, lens, feats, P)
    ref, opl = oracle.forward(feats, lens, P, cfg_d)
    assert pl.copy()[1] == opl["cu_seqlens"] == [0, 104]
    check(y, ref, "fp32", "tiny")


def test_rag_bf16():
    """4 ragged requests, 18 layers d 1024: whole output."""
    cfg_d, lens, feats, P = workload("rag")
    print("case: rag bf16", flush=True)
    y, pl = forward(cfg_d, lens, feats, P)
    ref, opl = oracle.forward(feats, lens, P, cfg_d)
    # the printed cu_seqlens of 3.0, 8.0, 17.37 and 30.0 s (tokens 39, 104,
    # 226, 390; windows of 104 tokens per request, then the remainder)
    assert pl.copy()[1] == opl["cu_seqlens"] == [0, 39, 143, 247, 351, 369, 473, 577, 681, 759]
    check(y, ref, "bf16", "rag")


@pytest.mark.parametrize("name", ["wide", "long", "conc"])
def test_large_sampled_windows(name):
    """Full-size bf16 forward; the oracle recomputes a seeded sample of windows."""
    cfg_d, lens, feats, P = workload(name)
    print(f"case: {name} bf16 full size, sampled windows", flush=True)
    y, pl = forward(cfg_d, lens, feats, P)
    opl = oracle.plan(lens, cfg_d)
    assert pl.copy()[1] == opl["cu_seqlens"]
    assert np.isfinite(y).all()
    wins = sample_windows(opl, seed=si.workload_seed(name))
    assert len(wins) >= 8, wins
    print(f"[{name}] windows {wins}", flush=True)
    res = oracle.forward_windows(feats, lens, P, cfg_d, wins)
    for w, (r0, ref) in res.items():
        check(y[r0:r0 + ref.shape[0]], ref, "bf16", f"{name} window {w} (rows {r0}+{ref.shape[0]})")


def wrap_band_windows(T, lda_elems, elem_bytes, cu):
    """Windows holding rows that a 256-row GEMM tile would lose if its A
    descriptor took the rest of the matrix, (T - m0) * lda bytes, as a 32-bit
    count: where that count wraps past 2^32 to less than the tile's own span,
    the tile's rows beyond the wrapped count read as zero."""
    row_bytes = lda_elems * elem_bytes
    rows = []
    for m0 in range(0, T, 256):
        rest = (T - m0) * row_bytes
        if rest >= 1 << 32 and rest % (1 << 32) < 256 * row_bytes:
            first = m0 + -(-(rest % (1 << 32)) // row_bytes)
            rows += list(range(first, min(m0 + 256, T)))
    return sorted({int(np.searchsorted(cu, r, side="right") - 1) for r in rows})


def test_max_batch_sampled_windows():
    """One 35 000 s request, 455 000 tokens in one bf16 batch (13.8 GiB of
    workspace): past the size where a GEMM tile's A descriptor count, the rest
    of the matrix in bytes, no longer fits 32 bits (fc2's A is T x 5120 bf16,
    2^32 bytes at 419 430 rows). The windows of the rows a wrapped count would
    have cut are recomputed by the oracle, with the first, a middle and the
    last window; only the sampled rows leave the GPU."""
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    cfg_d, _, _, P = workload("wide")
    lens = np.array([3_500_000])
    feats = si.mel_features(lens, seed=77)
    opl = oracle.plan(lens, cfg_d)
    cu = np.asarray(opl["cu_seqlens"])
    T = int(cu[-1])
    assert T == 455_000
    band = wrap_band_windows(T, cfg_d["encoder_ffn_dim"], 2, cu)
    assert band, "the sample must include rows past a wrap of the 32-bit count"
    wins = sorted({0, len(cu) // 2, len(cu) - 2} | set(band))
    print(f"case: max batch bf16, T={T}, windows {wins}", flush=True)
    cfg, packed = pack(cfg_d, P)
    out, pl = aut.encode(cfg, features_dev(feats), lens, packed, "bf16")
    torch.cuda.synchronize()
    assert pl.copy()[1] == opl["cu_seqlens"]
    res = oracle.forward_windows(feats, lens, P, cfg_d, wins)
    for w, (r0, ref) in res.items():
        g = out[r0:r0 + ref.shape[0]].double().cpu().numpy()
        check(g, ref, "bf16", f"max batch window {w} (rows {r0}+{ref.shape[0]})")


def test_wide_bench_launch_config():
    """The wide workload in the launch configuration bench.py times (conv-stem
    batches as large as the library allows), seeded sample of windows."""
    cfg_d, lens, feats, P = workload("wide")
    cfg_d = dict(cfg_d, conv_chunksize=4096)
    print("case: wide bf16, bench launch configuration, sampled windows", flush=True)
    y, pl = forward(cfg_d, lens, feats, P)
    opl = oracle.plan(lens, cfg_d)
    assert pl.copy()[1] == opl["cu_seqlens"]
    assert np.isfinite(y).all()
    wins = sample_windows(opl, seed=si.workload_seed("wide") + 7)
    assert len(wins) >= 8, wins
    res = oracle.forward_windows(feats, lens, P, cfg_d, wins)
    for w, (r0, ref) in res.items():
        check(y[r0:r0 + ref.shape[0]], ref, "bf16", f"wide/bench window {w} (rows {r0}+{ref.shape[0]})")


def test_window_isolation_bitwise():
    """openarchlab "1A", section 4: change one window's spectrogram, every other
    window's output must not move at all (0.00e+00)."""
    cfg_d, lens, feats, P = workload("rag")
    cfg, packed = pack(cfg_d, P)
    y0, pl = forward(cfg_d, lens, feats, packed=packed, cfg=cfg)
    cu = pl.copy()[1]
    f2 = feats.copy()
    f2[3, :, 800:1600] += 0.25   # request 3, window 1 (frames 800..1599)
    y1, _ = forward(cfg_d, lens, f2, packed=packed, cfg=cfg)
    changed = [w for w in range(len(cu) - 1) if not np.array_equal(y0[cu[w]:cu[w + 1]], y1[cu[w]:cu[w + 1]])]
    target = 1 + 1 + 3 + 1          # windows of requests 0..2 come first (1 + 1 + 3)
    assert changed == [target], changed
    dev = max(np.abs(y0[cu[w]:cu[w + 1]] - y1[cu[w]:cu[w + 1]]).max() for w in range(len(cu) - 1) if w != target)
    print(f"isolation: max deviation outside the perturbed window {dev:.2e}", flush=True)
    assert dev == 0.0


def test_batch_composition_bitwise():
    """A request's output rows do not depend on what else is in the batch, bit
    for bit: the wide batch (14 673 rows; its layer GEMMs run 288 x 256 and
    256 x 320 tiles, its conv GEMMs 256 x 256) against three of its requests
    encoded alone (a few hundred rows; narrower tiles). Every GEMM output sums
    its k steps in the same order in every tile shape, and every other step
    works per row or per window (m-star module summary: attention stays
    inside each window)."""
    cfg_d, lens, feats, P = workload("wide")
    cfg, packed = pack(cfg_d, P)
    y, pl = forward(cfg_d, lens, feats, packed=packed, cfg=cfg)
    off = np.concatenate([[0], np.cumsum(pl.copy()[0])])
    for b in (0, len(lens) // 2, len(lens) - 1):
        print(f"case: request {b} alone ({off[b + 1] - off[b]} rows) against the wide batch", flush=True)
        yb, _ = forward(cfg_d, lens[b:b + 1], feats[b:b + 1], packed=packed, cfg=cfg)
        assert yb.shape == (off[b + 1] - off[b], y.shape[1])
        assert np.array_equal(yb, y[off[b]:off[b + 1]]), b


@pytest.mark.parametrize("dtype,mask", [("bf16", 0), ("fp8", 32)])
def test_conv_batch_size_bitwise(dtype, mask):
    """conv_chunksize only sets how many chunks one conv-stem launch takes
    (memory), and the library picks batch sizes below it that fill the conv
    GEMMs' rounds of tiles: the wide workload's whole output is bit-identical
    whether the stem runs in two batches (~700 chunks) or in thirteen (<= 97)."""
    cfg_d, lens, feats, P = workload("wide")
    cfg_d = dict(cfg_d, dtype=dtype, fp8_gemms=mask)
    ys = []
    for cs in (4096, 97):
        print(f"case: wide {dtype} mask {mask}, conv_chunksize {cs}", flush=True)
        y, _ = forward(dict(cfg_d, conv_chunksize=cs), lens, feats, P)
        ys.append(y)
    assert np.isfinite(ys[0]).all()
    assert np.array_equal(ys[0], ys[1])


def test_run_twice_bitwise():
    """Full-width workload twice: identical bits (no order-dependent reductions)."""
    cfg_d, lens, feats, P = workload("wide")
    cfg, packed = pack(cfg_d, P)
    y0, _ = forward(cfg_d, lens, feats, packed=packed, cfg=cfg)
    y1, _ = forward(cfg_d, lens, feats, packed=packed, cfg=cfg)
    assert np.array_equal(y0, y1)


def test_planned_matches_encode():
    """aut_encode_planned after one aut_plan_upload equals aut_encode, also on
    a second call (the plan is reused, as in a replayed graph)."""
    from packed_windowed_attention_amd import aut
    torch = torch_mod()
    cfg_d, lens, feats, P = small_case("bf16")
    cfg, packed = pack(cfg_d, P)
    y, _ = forward(cfg_d, lens, feats, packed=packed, cfg=cfg)
    pl = aut.plan(cfg, lens)
    ws = aut.workspace(cfg, pl, "bf16")
    aut.plan_upload(pl, ws)
    fd = features_dev(feats)
    for _ in range(2):
        out = torch.full((pl.total_tokens, cfg_d["output_dim"]), float("nan"), device="cuda")
        aut.encode_planned(cfg, pl, fd, packed, "bf16", out, ws)
        torch.cuda.synchronize()
        assert np.array_equal(out.double().cpu().numpy(), y)
