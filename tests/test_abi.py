"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and its host-only calls (configuration, plan, sizes, argument
checks) behave as documented.  No call here launches GPU work: every error
path tested returns before the first launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth_inputs as si
from packed_windowed_attention_amd import aut

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "aut.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:aut_status|void|const char\*)\s+(aut_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    L = aut.lib()
    names = declared_functions()
    assert len(names) == len(aut.SIGNATURES) == 32
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(aut.SIGNATURES), "binding and header disagree"


def test_config_default_matches_page_defaults():
    import json
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))
    d = gold["config_defaults"]["value"]
    c = aut.config()
    for k in aut.CONFIG_FIELDS:
        if k in d:
            assert getattr(c, k) == d[k], k
    assert c.conv_out_bias == 0 and abs(c.ln_eps - 1e-5) < 1e-12


@pytest.mark.parametrize("name", si.WORKLOADS)
def test_plan_bit_exact_vs_oracle(name):
    cfg_d = si.model_config(name)
    lens = si.feature_lens(name)
    pl = aut.plan(aut.config(cfg_d), lens)
    tpr, cu, chunks = pl.copy()
    op = oracle.plan(lens, cfg_d)
    assert tpr == op["tokens_per_request"]
    assert cu == op["cu_seqlens"]
    assert chunks == [tuple(c) for c in op["chunks"]]
    assert pl.total_tokens == op["total_tokens"]


@pytest.mark.parametrize("lens", [[0], [1], [99, 100, 101], [0, 5, 0, 100, 0], list(range(0, 1700, 37)),
                                  [120000], [800] * 3 + [801]])
def test_plan_edge_cases_vs_oracle(lens):
    cfg_d = si.model_config("rag")
    pl = aut.plan(aut.config(cfg_d), lens)
    tpr, cu, chunks = pl.copy()
    op = oracle.plan(lens, cfg_d)
    assert (tpr, cu, chunks) == (op["tokens_per_request"], op["cu_seqlens"], [tuple(c) for c in op["chunks"]])


def test_plan_random_lengths_vs_oracle():
    rng = np.random.default_rng(99)
    cfg_d = si.model_config("wide")
    for _ in range(20):
        lens = rng.integers(0, 5000, size=rng.integers(1, 40))
        pl = aut.plan(aut.config(cfg_d), lens)
        tpr, cu, chunks = pl.copy()
        op = oracle.plan(lens, cfg_d)
        assert cu == op["cu_seqlens"] and tpr == op["tokens_per_request"]
        assert chunks == [tuple(c) for c in op["chunks"]]


def status_of(fn):
    with pytest.raises(aut.AutError) as e:
        fn()
    return e.value.status


def test_config_errors():
    assert status_of(lambda: aut.config_check(aut.config(d_model=1000, encoder_attention_heads=16))) == 2
    assert status_of(lambda: aut.config_check(aut.config(n_window_infer=750))) == 2
    assert status_of(lambda: aut.config_check(aut.config(n_window_infer=1600))) == 2   # 208 tokens
    assert status_of(lambda: aut.config_check(aut.config(num_mel_bins=80))) == 2
    assert status_of(lambda: aut.config_check(aut.config(downsample_hidden_size=100))) == 2
    assert status_of(lambda: aut.config_check(aut.config(d_model=0))) == 1
    assert status_of(lambda: aut.plan(aut.config(), [100, -1])) == 1
    assert status_of(lambda: aut.weights_bytes(aut.config(), 7)) == 1


def test_sizes():
    cfg = aut.config(si.model_config("wide"))
    n_params = sum(int(np.prod(s)) for _, s in si.param_shapes(si.model_config("wide")))
    wb = aut.weights_bytes(cfg, "bf16")
    assert 2 * n_params <= wb <= 2 * n_params + 4 * 10 ** 7
    assert aut.weights_bytes(cfg, "fp32") >= 4 * n_params
    pl = aut.plan(cfg, si.feature_lens("wide"))
    ws = aut.workspace_bytes(cfg, pl, "bf16")
    T, d = pl.total_tokens, cfg.d_model
    assert ws >= T * d * 4 + T * 3 * d * 2 + T * cfg.encoder_ffn_dim * 2


def test_missing_weight_reported_before_launch():
    cfg = aut.config(si.model_config("tiny"))
    w = aut.AutWeightPtrs()
    nbytes = aut.weights_bytes(cfg, "fp32")
    st = aut.lib().aut_weights_pack(ctypes.byref(cfg), ctypes.byref(w), 0, ctypes.c_void_p(256),
                                    nbytes, None)
    assert st == 3
    assert b"conv1_w" in aut.lib().aut_last_error()
    # every scalar given but one per-layer entry missing: the message names it
    for n in aut._SCALAR_W + aut._TAIL_W:
        setattr(w, n, 4096)
    arrs = []
    for n in aut.LAYER_W:
        arr = (ctypes.c_void_p * 1)(4096 if n != "fc2_b" else None)
        arrs.append(arr)
        setattr(w, n, ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)))
    st = aut.lib().aut_weights_pack(ctypes.byref(cfg), ctypes.byref(w), 0, ctypes.c_void_p(256),
                                    nbytes, None)
    assert st == 3 and b"layers.0.fc2_b" in aut.lib().aut_last_error()
    # destination too small
    st = aut.lib().aut_weights_pack(ctypes.byref(cfg), ctypes.byref(w), 0, ctypes.c_void_p(256),
                                    nbytes - 1, None)
    assert st == 4


def test_encode_argument_checks_before_launch():
    cfg = aut.config(si.model_config("tiny"))
    lens = (ctypes.c_int32 * 2)(800, 900)
    fake = ctypes.c_void_p(4096)
    L = aut.lib()
    # a length beyond T_max
    st = L.aut_encode(ctypes.byref(cfg), fake, 850, lens, 2, fake, 0, fake, fake, 1 << 40, None)
    assert st == 1 and b"T_max" in L.aut_last_error()
    # workspace too small
    st = L.aut_encode(ctypes.byref(cfg), fake, 900, lens, 2, fake, 0, fake, fake, 1024, None)
    assert st == 4
    # unknown dtype
    st = L.aut_encode(ctypes.byref(cfg), fake, 900, lens, 2, fake, 5, fake, fake, 1 << 40, None)
    assert st == 1
    # a plan made for another configuration
    pl = aut.plan(aut.config(si.model_config("rag")), [800])
    st = L.aut_encode_planned(ctypes.byref(cfg), pl.handle, fake, 900, fake, 0, fake, fake, 1 << 40, None)
    assert st == 1
    # an empty batch is a no-op that needs no buffers at all
    z = (ctypes.c_int32 * 1)(0)
    assert L.aut_encode(ctypes.byref(cfg), None, 0, z, 1, None, 0, None, None, 0, None) == 0
    assert L.aut_encode(ctypes.byref(cfg), None, 0, z, 0, None, 0, None, None, 0, None) == 0


def _oracle_tokens(L, cfg_d):
    return oracle.plan([L], cfg_d)["tokens_per_request"][0]


def test_stream_plan_vs_oracle():
    """aut_stream_plan against the oracle's plan: window k of a request starts at
    frame 800 k and row 104 k; the frames from there form a request of their own
    with the remaining rows (chunk-aligned start)."""
    cfg_d = si.model_config("wide")
    cfg = aut.config(cfg_d)
    rng = np.random.default_rng(5)
    lens = [0, 1, 99, 100, 101, 799, 800, 801, 1599, 1600, 1601, 2630] + [int(x) for x in rng.integers(0, 12000, 30)]
    for L in lens:
        opl = oracle.plan([L], cfg_d)
        cu = opl["cu_seqlens"]
        complete = L // 800
        assert complete == sum(1 for w in range(len(cu) - 1) if cu[w + 1] - cu[w] == 104 and (w + 1) * 800 <= L)
        for wf in sorted({0, complete // 2, complete}):
            sp = aut.stream_plan(cfg, L, wf)
            assert sp["frame_begin"] == 800 * wf
            assert sp["row_begin"] == (cu[wf] if wf < len(cu) else cu[-1])
            assert sp["rows"] == _oracle_tokens(L, cfg_d) - sp["row_begin"]
            assert sp["rows"] == _oracle_tokens(L - 800 * wf, cfg_d)
            assert sp["windows_final_after"] == complete


def test_stream_plan_errors():
    cfg = aut.config(si.model_config("wide"))
    for L, wf in ((100, 1), (1599, 2), (-1, 0), (800, -1)):
        with pytest.raises(RuntimeError) as e:
            aut.stream_plan(cfg, L, wf)
        assert "AUT_ERR_INVALID_ARG" in str(e.value)


def test_stream_workspace_covers_each_step():
    """The one-request workspace for max_frames covers the plan of any step."""
    cfg_d = si.model_config("rag")
    cfg = aut.config(cfg_d)
    lib = aut.lib()
    import ctypes as ct
    for mx in (1, 800, 2630, 12000):
        n = ct.c_size_t()
        assert lib.aut_stream_workspace_bytes(ct.byref(cfg), mx, aut.DTYPES["bf16"], ct.byref(n)) == 0
        for L in (1, mx // 3, mx):
            assert aut.workspace_bytes(cfg, aut.plan(cfg, [L]), "bf16") <= n.value


@pytest.mark.parametrize("dtype,mask", [("bf16", 0), ("fp8", 63)])
def test_workspace_never_shrinks_as_a_request_grows(dtype, mask):
    """A workspace sized for one request covers every shorter request (what a
    stream's steps rely on): the full-width model at the default conv batch
    size and at the largest, over lengths around the chunk counts where the
    conv batches change size."""
    cfg_d = dict(si.model_config("wide"), fp8_gemms=mask)
    for cs in (500, 8192):
        cfg = aut.config(dict(cfg_d, conv_chunksize=cs))
        prev = 0
        for L in list(range(100, 2000, 97)) + list(range(40000, 160000, 3100)):
            n = aut.workspace_bytes(cfg, aut.plan(cfg, [L]), dtype)
            assert n >= prev, (cs, L, n, prev)
            prev = n


def test_audio_rows_vs_oracle():
    """aut_audio_rows (host) against the oracle's placeholder positions."""
    rng = np.random.default_rng(17)
    PAD = 151676
    for n in (0, 1, 5, 300, 4000):
        ids = rng.integers(0, 150000, size=n + 37).astype(np.int32)
        pos = np.sort(rng.choice(n + 37, size=n, replace=False))
        ids[pos] = PAD
        assert aut.audio_rows(ids, PAD, n) == [int(x) for x in oracle.audio_rows(ids, PAD, n)]
    with pytest.raises(RuntimeError) as e:
        aut.audio_rows([1, PAD, 2], PAD, 2)
    assert "AUT_ERR_INVALID_ARG" in str(e.value)


def test_inject_argument_checks_before_launch():
    lib = aut.lib()
    import ctypes as ct
    ok_ptr = ct.c_void_p(16)
    assert lib.aut_inject_audio(None, None, 0, 2048, None, 0, 0, None) == 0      # nothing to do
    assert lib.aut_inject_audio(None, ok_ptr, 4, 2048, ok_ptr, 10, 0, None) == 1  # NULL audio
    assert lib.aut_inject_audio(ok_ptr, ok_ptr, 4, 2046, ok_ptr, 10, 0, None) == 1  # dim % 4
    assert lib.aut_inject_audio(ok_ptr, ok_ptr, -1, 2048, ok_ptr, 10, 0, None) == 1
    assert lib.aut_inject_audio(ok_ptr, ok_ptr, 4, 2048, ok_ptr, 10, 7, None) == 1  # dtype


# ---------------------------------------------------------------------------
# MX-fp8 (AUT_FP8): sizes and argument checks, host only
# ---------------------------------------------------------------------------


def test_fp8_config_default_and_range():
    c = aut.config()
    assert c.fp8_gemms == aut.FP8_ALL == 63
    aut.config_check(aut.config(fp8_gemms=0))
    with pytest.raises(aut.AutError) as e:
        aut.config_check(aut.config(fp8_gemms=64))
    assert e.value.status == 1


def test_mx_scale_bytes():
    for rows, K in [(1, 128), (16, 128), (17, 1280), (14673, 5120), (0, 256)]:
        assert aut.mx_scale_bytes(rows, K) == (rows + 15) // 16 * 16 * K // 32
    for K in (0, 64, 1000):
        with pytest.raises(aut.AutError):
            aut.mx_scale_bytes(16, K)


def test_fp8_weight_bytes_follow_the_mask():
    cfg_d = si.model_config("wide")
    d, F, O = cfg_d["d_model"], cfg_d["encoder_ffn_dim"], cfg_d["output_dim"]
    L = cfg_d["encoder_layers"]
    bf = aut.weights_bytes(aut.config(cfg_d), "bf16")
    full = aut.weights_bytes(aut.config(cfg_d, fp8_gemms=aut.FP8_ALL & ~aut.FP8_CONV), "fp8")
    none = aut.weights_bytes(aut.config(cfg_d, fp8_gemms=0), "fp8")
    assert none == bf
    # each fp8 weight: 1 byte + 1/32 of a scale byte per element instead of 2 bytes
    per_layer = 3 * d * d + d * d + 2 * F * d
    elems = L * per_layer + d * d + O * d
    saved = bf - full
    assert abs(saved - elems * (1 - 1 / 32)) < 256 * (6 * L + 4)   # up to 256-byte alignment per array


def test_fp8_conv_weight_bytes():
    # conv2 / conv3 [C][9 cp] and conv_out [d][16 cp] codes, cp = C rounded up to 128
    cfg_d = si.model_config("wide")
    C, d = cfg_d["downsample_hidden_size"], cfg_d["d_model"]
    cp = (C + 127) // 128 * 128
    a = aut.weights_bytes(aut.config(cfg_d, fp8_gemms=aut.FP8_ALL), "fp8")
    b = aut.weights_bytes(aut.config(cfg_d, fp8_gemms=aut.FP8_ALL & ~aut.FP8_CONV), "fp8")
    conv_bf16 = (2 * C * 9 * C + d * 16 * C) * 2
    conv_f8 = (2 * C * 9 * cp + d * 16 * cp) * (1 + 1 / 32)
    assert abs((b - a) - (conv_bf16 - conv_f8)) < 256 * 8


def test_fp8_conv_needs_32_channel_blocks():
    cfg_d = dict(si.model_config("tiny"), downsample_hidden_size=40)
    with pytest.raises(aut.AutError) as e:
        aut.weights_bytes(aut.config(cfg_d, fp8_gemms=aut.FP8_ALL), "fp8")
    assert e.value.status == 2
    aut.weights_bytes(aut.config(cfg_d, fp8_gemms=aut.FP8_ALL & ~aut.FP8_CONV), "fp8")


def test_fp8_needs_128_multiples():
    cfg_d = dict(si.model_config("tiny"))
    cfg_d.update(d_model=192, encoder_attention_heads=3)
    with pytest.raises(aut.AutError) as e:
        aut.weights_bytes(aut.config(cfg_d), "fp8")
    assert e.value.status == 2
    aut.weights_bytes(aut.config(cfg_d), "bf16")


def test_mx_primitive_argument_checks():
    L = aut.lib()
    assert L.aut_mx_quantize(None, 4, 100, None, None, None) == 1
    assert L.aut_mx_quantize(None, 0, 128, None, None, None) == 0      # nothing to do
    assert L.aut_mx_matmul(None, None, 4, None, None, 6, 128, None, None) == 2   # N % 4
    assert L.aut_mx_matmul(None, None, 4, None, None, 8, 96, None, None) == 1    # K % 128
    assert L.aut_mx_matmul(None, None, 4, None, None, 8, 128, None, None) == 1   # NULL


def test_attention_argument_checks_before_launch():
    """aut_attention refuses bad counts, dtype pairs, head counts, NULL and
    misaligned pointers on the host, before any GPU call."""
    L = aut.lib()
    fp32, bf16, fp8 = (aut.DTYPES[k] for k in ("fp32", "bf16", "fp8"))
    p = 4096  # a non-NULL, 16-byte aligned stand-in (never dereferenced: the checks fail first)
    assert L.aut_attention(p, -1, 20, p, p, 1, bf16, bf16, p, None, None) == 1          # rows < 0
    assert L.aut_attention(p, 10, 20, p, p, -1, bf16, bf16, p, None, None) == 1         # windows < 0
    assert L.aut_attention(p, 10, 20, p, p, 1, fp32, bf16, p, None, None) == 2          # fp32 -> bf16
    assert L.aut_attention(p, 10, 20, p, p, 1, fp32, fp8, p, p, None) == 2              # fp32 -> fp8
    assert L.aut_attention(p, 10, 0, p, p, 1, bf16, bf16, p, None, None) == 2           # no head
    assert L.aut_attention(p, 10, 3, p, p, 1, bf16, fp8, p, p, None) == 2               # odd heads, fp8
    assert L.aut_attention(p, 10, 65, p, p, 1, bf16, bf16, p, None, None) == 2          # too many heads
    assert L.aut_attention(None, 0, 20, None, None, 0, bf16, bf16, None, None, None) == 0  # nothing to do
    assert L.aut_attention(None, 10, 20, p, p, 1, bf16, bf16, p, None, None) == 1       # NULL qkv
    assert L.aut_attention(p, 10, 2, p, p, 1, bf16, fp8, p, None, None) == 1            # NULL scales
    assert L.aut_attention(p + 8, 10, 20, p, p, 1, bf16, bf16, p, None, None) == 1      # misaligned qkv
    assert L.aut_attention(p, 10, 20, p + 2, p, 1, bf16, bf16, p, None, None) == 1      # misaligned table


def test_mx_scale_layout_reindex():
    # the binding's reindexing matches the documented formula, entry by entry
    rows, K = 37, 256
    flat = np.arange(aut.mx_scale_bytes(rows, K)) % 251
    rm = aut.mx_scales_rowmajor(flat, rows, K)
    for r in (0, 15, 16, 36):
        for kb in range(K // 32):
            assert rm[r, kb] == flat[((r // 16) * (K // 128) + kb // 4) * 64 + (kb % 4) * 16 + r % 16]


def test_encode_noalloc_rejects_a_batch_past_its_scratch():
    """aut_encode_noalloc refuses, before any GPU call, a batch whose
    workspace exceeds the library's device scratch, naming both sizes."""
    cfg = aut.config(si.model_config("wide"), conv_chunksize=500)
    lens = (ctypes.c_int32 * 1)(120000)          # 1200 s of audio: several GiB of workspace
    fake = ctypes.c_void_p(256)
    st = aut.lib().aut_encode_noalloc(ctypes.byref(cfg), fake, 120000, lens, 1, fake,
                                      aut.DTYPES["bf16"], fake, None)
    msg = aut.lib().aut_last_error().decode()
    assert aut.STATUS.get(st) == "AUT_ERR_WORKSPACE_TOO_SMALL", (st, msg)
    assert "device scratch" in msg and str(256 << 20) in msg
