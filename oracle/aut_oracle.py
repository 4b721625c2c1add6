"""CPU oracle of the AuT audio-encoder forward pass (test infrastructure).

Plain, slow, float64 numpy.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may use this module; the product path never does.
It shares no code with the HIP library and imports nothing from it.

What it follows (the pages are cited by title and section):

* "mstar.model.components.aut_encoder" (m-star API page), module summary:
  1 s chunks of 2*n_window frames; three stride-2 Conv2d layers (100 frames ->
  13 tokens); linear conv_out; the same 13 sinusoidal positions per chunk;
  valid tokens packed into one [total_tokens, d_model] sequence; attention
  within windows of n_window_infer frames (8 s -> 104 tokens), block-diagonal,
  bidirectional, no cache; final LayerNorm and a two-layer GELU projector.
  ``frontend``: the last piece is zero-padded to a full chunk, convolved and
  trimmed back to its valid tokens.  ``tokens_for_frames``: 13 per full chunk
  plus three stride-2 convolutions' worth of the remainder.
  ``window_lengths``: full windows, then the remainder.  SDPA per window from
  cu_seqlens is the attention's definition.  q/k/v are fused into qkv_proj.
* "1A - AuT Audio Encoder" (openarchlab course), section 3: Conv2d(k=3, s=2,
  p=1) maps L to floor((L+1)/2); 128 bins -> 16; flatten C_conv x 16 and a
  linear conv_out to d_model; non-causal attention inside cu_seqlens segments;
  projector Linear(d -> d) + GELU + Linear(d -> 2048).
* "Audio Encoder Component" (cubic.dev wiki), Transformer Encoder Layers:
  LayerNorm with bias (not RMSNorm); sinusoidal positions computed, not loaded.

Readings where the pages are silent: Whisper-style [sin | cos] table with increment
ln(10000)/(d/2 - 1); chunk-local positions 0..k-1; exact (erf) GELU after each
conv, fc1 and proj1; LayerNorm eps 1e-5 with population variance; pre-LN
residual order; attention scale 1/sqrt(head_dim); flatten index c*16 + f;
conv_out without bias unless one is given; H axis = mel bin, W axis = time;
padding beyond a request's length is treated as zero whatever it holds.

Parity pins: see tests/test_oracle_pins.py.  Every function below is pinned by
at least one test against a library routine, a closed form, a value printed on
the pages, or an exact invariant.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

# ---------------------------------------------------------------------------
# plan (host arithmetic only)
# ---------------------------------------------------------------------------


def conv_out_len(n: int) -> int:
    """Output length of Conv2d(kernel 3, stride 2, padding 1) along one axis:
    floor((n + 1) / 2) -- openarchlab "1A", section 3 formula."""
    return (n + 1) // 2


def chunk_frames(cfg: dict) -> int:
    """Frames per chunk: 2 * n_window (m-star API page, module summary)."""
    return 2 * cfg["n_window"]


def tokens_for_frames(num_frames: int, cfg: dict) -> int:
    """m-star ``tokens_for_frames``: per full chunk the three-conv output
    length of a full chunk; for the remainder, three halvings of its length."""
    cf = chunk_frames(cfg)
    per_chunk = conv_out_len(conv_out_len(conv_out_len(cf)))
    full, rem = divmod(int(num_frames), cf)
    return full * per_chunk + conv_out_len(conv_out_len(conv_out_len(rem)))


def window_tokens(cfg: dict) -> int:
    """Tokens per attention window: n_window_infer frames is a whole number of
    chunks (8 s = 8 chunks -> 104 tokens on the m-star page)."""
    cf = chunk_frames(cfg)
    if cfg["n_window_infer"] % cf:
        raise ValueError("n_window_infer must be a multiple of 2*n_window")
    per_chunk = tokens_for_frames(cf, cfg)
    return per_chunk * (cfg["n_window_infer"] // cf)


def window_lengths(num_tokens: int, cfg: dict) -> list[int]:
    """m-star ``window_lengths``: full windows, then the remainder (if any)."""
    wt = window_tokens(cfg)
    full, rem = divmod(int(num_tokens), wt)
    return [wt] * full + ([rem] if rem else [])


def plan(feature_lens, cfg: dict) -> dict:
    """m-star ``layout``: tokens per request and cu_seqlens for a batch, plus
    the chunk table the frontend walks.

    Packed row order: request, then chunk, then token within the chunk.
    Windows never span two requests; an empty request adds nothing.
    """
    cf = chunk_frames(cfg)
    chunks = []            # (request, first frame, valid frames, valid tokens, first row)
    tokens_per_request = []
    cu = [0]
    row = 0
    for b, L in enumerate(feature_lens):
        L = int(L)
        if L < 0:
            raise ValueError("negative feature length")
        n_chunks = -(-L // cf)
        t_req = 0
        for c in range(n_chunks):
            vf = min(cf, L - c * cf)
            vt = tokens_for_frames(vf, cfg)
            chunks.append((b, c * cf, vf, vt, row))
            row += vt
            t_req += vt
        assert t_req == tokens_for_frames(L, cfg)
        tokens_per_request.append(t_req)
        for wl in window_lengths(t_req, cfg):
            cu.append(cu[-1] + wl)
    return dict(
        chunks=chunks,
        tokens_per_request=tokens_per_request,
        cu_seqlens=cu,
        total_tokens=row,
        window_lengths=[cu[i + 1] - cu[i] for i in range(len(cu) - 1)],
    )


# ---------------------------------------------------------------------------
# elementary operations
# ---------------------------------------------------------------------------


def gelu(x):
    """Exact GELU, x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)) ('gelu' in
    AuTEncoderConfig.activation_function)."""
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def sinusoid_table(length: int, channels: int) -> np.ndarray:
    """Fixed sinusoidal position table [length, channels] (wiki "Positional
    Embeddings": computed, not loaded).  Whisper-style: row j, column i < D is
    sin(j * tau_i), column D + i is cos(j * tau_i), tau_i = 10000^(-i/(D-1)),
    D = channels / 2."""
    if channels % 2:
        raise ValueError("channels must be even")
    D = channels // 2
    inc = math.log(10000.0) / (D - 1)
    tau = np.exp(-inc * np.arange(D, dtype=np.float64))
    t = np.arange(length, dtype=np.float64)[:, None] * tau[None, :]
    return np.concatenate([np.sin(t), np.cos(t)], axis=1)


def conv2d_k3s2p1(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """2-D cross-correlation, kernel 3x3, stride 2, zero padding 1 (openarchlab
    "1A", glossary and section 3), plus bias.

    x [Cin, H, W], w [Cout, Cin, 3, 3], b [Cout] -> [Cout, floor((H+1)/2),
    floor((W+1)/2)].  out[o, y, t] = b[o] + sum_{i, kh, kw} w[o, i, kh, kw] *
    xpad[i, 2y + kh, 2t + kw], written as a sum over the nine taps of a
    channel contraction.
    """
    cin, H, W = x.shape
    Ho, Wo = conv_out_len(H), conv_out_len(W)
    xp = np.zeros((cin, H + 2, W + 2), dtype=np.float64)
    xp[:, 1:H + 1, 1:W + 1] = x
    out = np.zeros((w.shape[0], Ho, Wo), dtype=np.float64)
    for kh in range(3):
        for kw in range(3):
            patch = xp[:, kh:kh + 2 * Ho:2, kw:kw + 2 * Wo:2]        # [Cin, Ho, Wo]
            out += np.tensordot(w[:, :, kh, kw].astype(np.float64), patch, axes=(1, 0))
    out += np.asarray(b, dtype=np.float64)[:, None, None]
    return out


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = 1e-5):
    """LayerNorm with bias over the last axis: population variance, eps inside
    the square root (wiki: "LayerNorm with bias")."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def linear(x: np.ndarray, w: np.ndarray, b=None) -> np.ndarray:
    """y = x W^T (+ b), W in [out, in] layout."""
    y = x @ np.asarray(w, dtype=np.float64).T
    if b is not None:
        y = y + np.asarray(b, dtype=np.float64)
    return y


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    m = s.max(axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=axis, keepdims=True)


def window_attention(q, k, v, cu_seqlens, num_heads: int) -> np.ndarray:
    """SDPA per window (m-star AuTAttention, unbound case): for each segment
    [s, e) of cu_seqlens and each head, softmax(Q K^T / sqrt(hd)) V with no
    mask inside the segment and nothing across segments (bidirectional,
    is_causal = False)."""
    T, d = q.shape
    hd = d // num_heads
    out = np.zeros((T, d), dtype=np.float64)
    scale = 1.0 / math.sqrt(hd)
    for w in range(len(cu_seqlens) - 1):
        s, e = int(cu_seqlens[w]), int(cu_seqlens[w + 1])
        for h in range(num_heads):
            cols = slice(h * hd, (h + 1) * hd)
            qh, kh, vh = q[s:e, cols], k[s:e, cols], v[s:e, cols]
            p = softmax((qh @ kh.T) * scale, axis=-1)
            out[s:e, cols] = p @ vh
    return out


# ---------------------------------------------------------------------------
# 8-bit matrix products: MX-fp8 operands
# ---------------------------------------------------------------------------
# The pages run 8-bit variants of the encoder and judge them by the per-token
# cosine similarity to the full-precision one (soniqo "Qwen3-ASR" transcribe
# guide, es, section "Codificador CoreML (Neural Engine)": an INT8-palettised
# encoder at cosine > 0.999; the 8-, 5- and 4-bit MLX rows of its performance
# table).  Those formats are weight-only and Apple-specific.  The reading taken
# here is the 8-bit format the gfx950 matrix cores multiply at twice the bf16
# rate, OCP MX-fp8 (OCP "Microscaling Formats (MX) v1.0"): both operands of a
# product in e4m3 (OCP "8-bit Floating Point" E4M3: sign, 4 exponent bits with
# bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 = NaN,
# largest finite 448), every 32 consecutive values along the contraction axis
# sharing one power-of-two scale stored as E8M0 (scale = 2^(code - 127)).  The
# MX format leaves the choice of scale to the quantizer; here it is the
# smallest power of two s with max|x| / s <= 448 over the block (no element
# saturates), and each x / s goes to the nearest e4m3 value, ties to the even
# code.  Everything outside the products stays as in the unquantized path.

E4M3_MAX = 448.0
MX_BLOCK = 32
FP8_QKV, FP8_OUT, FP8_FC1, FP8_FC2, FP8_PROJ, FP8_CONV = 1, 2, 4, 8, 16, 32
FP8_ALL = 63


def e4m3_decode(codes) -> np.ndarray:
    """Value of each e4m3 code (uint8): exponent field 0 is subnormal,
    (m / 8) 2^-6; otherwise (1 + m / 8) 2^(e - 7); S.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 code of each |x| <= 448 (ties to the even code; -0.0 and
    +0.0 both give code 0 after a zero round: the sign of a zero is kept)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX) or np.any(np.isnan(x)):
        raise ValueError("e4m3_encode: |x| > 448 or NaN")
    vals = e4m3_decode(np.arange(127))                     # 0 .. 448, ascending
    a = np.abs(x)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, 126)   # vals[hi] >= a
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == vals[hi], hi, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def e4m3_round(x) -> np.ndarray:
    """The value ``e4m3_encode`` picks, computed directly: |x| <= 448 rounded
    to a multiple of its binade's spacing 2^(max(E, -6) - 3), E = floor(log2
    |x|) (3 mantissa bits; below 2^-6 the fixed subnormal spacing 2^-9), ties
    to even by np.rint, sign kept."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_round: |x| > 448")
    _, E = np.frexp(x)                       # |x| = m 2^E, m in [0.5, 1)
    q = np.maximum(E - 1, -6) - 3
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)


def mx_block_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e, within the E8M0 range
    [-127, 127]; an all-zero block takes -127."""
    a = np.asarray(amax, dtype=np.float64)
    safe = np.where(a > 0, a, E4M3_MAX)
    e = np.ceil(np.log2(safe / E4M3_MAX))
    e = np.where(safe > E4M3_MAX * np.exp2(e), e + 1, e)            # log2 rounding
    e = np.where(safe <= E4M3_MAX * np.exp2(e - 1), e - 1, e)
    e = np.where(a > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def mx_quantize(x):
    """x [..., K] with K a multiple of 32 -> (e4m3 codes uint8 [..., K],
    E8M0 scale codes uint8 [..., K / 32]), blocks along the last axis."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("mx_quantize: K must be a multiple of 32")
    xb = x.reshape(x.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    e = mx_block_exponent(np.abs(xb).max(axis=-1))
    codes = e4m3_encode(xb / np.exp2(e)[..., None])
    return codes.reshape(x.shape), (e + 127).astype(np.uint8)


def mx_dequantize(codes, scales) -> np.ndarray:
    c = np.asarray(codes)
    K = c.shape[-1]
    v = e4m3_decode(c).reshape(c.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    s = np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)
    return (v * s[..., None]).reshape(c.shape)


def mx_round(x) -> np.ndarray:
    """x after an MX-fp8 round trip, mx_dequantize(*mx_quantize(x)), computed
    on values: each block's scale exponent, then e4m3_round of x / 2^e."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("mx_round: K must be a multiple of 32")
    xb = x.reshape(x.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    e = mx_block_exponent(np.abs(xb).max(axis=-1))[..., None]
    return np.ldexp(e4m3_round(np.ldexp(xb, -e)), e).reshape(x.shape)


_MX_WEIGHTS: dict = {}


def linear_conv_out_mx(u: np.ndarray, w: np.ndarray, b, F: int) -> np.ndarray:
    """conv_out on MX-fp8 operands.  u holds the token features in the
    channel-major flatten c * F + f (the pairing of features and weight
    columns is unchanged).  Reading: every activation of the conv stem is
    quantised once, per pixel, in blocks of 32 consecutive channels: that is
    the only blocking the conv2 and conv3 contractions admit (their 32-value
    blocks run over channels within one tap, i.e. within one input pixel), and
    conv_out reads the same kind of tensor, the stem's last activation, so its
    blocks are those of the same rule: for token j, the 32-channel groups of
    one frequency bin f.  A dot product does not depend on the order of its
    terms, so the flatten order fixes which weight meets which feature but not
    how the contraction is blocked; the weight blocks are the matching sets of
    columns, {c * F + f : c in one group of 32}.  Both sides are therefore
    rounded in the order f * C + c and put back."""
    u = np.asarray(u, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    C = u.shape[1] // F
    perm = (np.arange(C)[None, :] * F + np.arange(F)[:, None]).reshape(-1)   # f * C + c -> c * F + f
    uq = np.empty_like(u)
    uq[:, perm] = mx_round(u[:, perm])
    wq = np.empty_like(w)
    wq[:, perm] = mx_round(w[:, perm])
    return linear(uq, wq, b)


def mx_round_pixels(a: np.ndarray) -> np.ndarray:
    """MX-fp8 round trip of a stem activation [C, H, W]: every pixel's C
    channel values in blocks of 32 consecutive channels (C a multiple of 32)."""
    a = np.asarray(a, dtype=np.float64)
    C = a.shape[0]
    return mx_round(a.reshape(C, -1).T).T.reshape(a.shape)


def _mx_weight(w) -> np.ndarray:
    """mx_round of a parameter array, remembered per array object (a
    parameter is rounded once however many windows or calls use it)."""
    hit = _MX_WEIGHTS.get(id(w))
    if hit is None or hit[0] is not w:
        if len(_MX_WEIGHTS) > 512:
            _MX_WEIGHTS.clear()
        hit = (w, mx_round(np.asarray(w, dtype=np.float64)))
        _MX_WEIGHTS[id(w)] = hit
    return hit[1]


def conv2d_k3s2p1_mx(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """``conv2d_k3s2p1`` as a product with MX-fp8 operands.  Its contraction
    axis is (tap, input channel): for each of the nine taps the strided input
    patch meets w[:, :, kh, kw] over the channels, so the blocks of 32 run over
    consecutive channels of one tap (C_in a multiple of 32), on both sides."""
    cin, H, W = x.shape
    if cin % MX_BLOCK:
        raise ValueError("conv2d_k3s2p1_mx: input channels must be a multiple of 32")
    Ho, Wo = conv_out_len(H), conv_out_len(W)
    xp = np.zeros((cin, H + 2, W + 2), dtype=np.float64)
    xp[:, 1:H + 1, 1:W + 1] = x
    out = np.zeros((w.shape[0], Ho, Wo), dtype=np.float64)
    for kh in range(3):
        for kw in range(3):
            patch = xp[:, kh:kh + 2 * Ho:2, kw:kw + 2 * Wo:2]            # [Cin, Ho, Wo]
            pq = mx_round(patch.reshape(cin, -1).T).T.reshape(patch.shape)
            wq = mx_round(np.asarray(w[:, :, kh, kw], dtype=np.float64))  # [Cout, Cin]
            out += np.tensordot(wq, pq, axes=(1, 0))
    out += np.asarray(b, dtype=np.float64)[:, None, None]
    return out


def linear_mx(x: np.ndarray, w: np.ndarray, b=None) -> np.ndarray:
    """``linear`` with both operands MX-fp8 rounded along the contraction axis
    (rows of x, rows of W in its [out, in] layout); exact products and sums."""
    return linear(mx_round(x), _mx_weight(w), b)


# ---------------------------------------------------------------------------
# the encoder
# ---------------------------------------------------------------------------


def chunk_image(features: np.ndarray, b: int, frame0: int, valid: int, cfg: dict):
    """One chunk as a 1-channel image [1, mel, chunk_frames]: the valid frames
    of request b, then zeros (the m-star ``frontend`` zero-pads the last piece
    to a full chunk).  Buffer contents past the length are never read."""
    cf = chunk_frames(cfg)
    img = np.zeros((1, cfg["num_mel_bins"], cf), dtype=np.float64)
    img[0, :, :valid] = features[b, :, frame0:frame0 + valid]
    return img


def conv_stem(img: np.ndarray, P: dict, fp8: int = 0) -> np.ndarray:
    """Three Conv2d(k3, s2, p1) layers, each followed by GELU:
    [1, 128, 100] -> [C, 16, 13].  FP8_CONV: conv2 and conv3 (conv1 has one
    input channel: no contraction to speak of) on MX-fp8 operands."""
    conv = conv2d_k3s2p1_mx if fp8 & FP8_CONV else conv2d_k3s2p1
    a = gelu(conv2d_k3s2p1(img, P["conv1_w"], P["conv1_b"]))
    a = gelu(conv(a, P["conv2_w"], P["conv2_b"]))
    a = gelu(conv(a, P["conv3_w"], P["conv3_b"]))
    return a


def flatten_tokens(a3: np.ndarray, vt: int) -> np.ndarray:
    """The first vt time columns of the stem output [C, 16, 13] as token rows
    [vt, C * 16], flattened channel-major: u_j[c * 16 + f] = a3[c, f, j]
    (openarchlab "1A", section 3: flatten C_conv x 16)."""
    C, Fq, _ = a3.shape
    return a3[:, :, :vt].transpose(2, 0, 1).reshape(vt, C * Fq)


def frontend(features, feature_lens, P: dict, cfg: dict, chunk_ids=None, fp8: int = 0):
    """m-star ``frontend``: chunk, pad, convolve, conv_out, add positions,
    keep the valid tokens.  Returns ([rows, d_model], the plan); ``chunk_ids``
    restricts the work to some chunks (rows returned in chunk order).
    FP8_CONV: conv2, conv3 and conv_out on MX-fp8 operands, each stem
    activation quantised per pixel in blocks of 32 channels (see
    ``linear_conv_out_mx``)."""
    pl = plan(feature_lens, cfg)
    d = cfg["d_model"]
    pe = sinusoid_table(cfg["max_source_positions"], d)
    ids = range(len(pl["chunks"])) if chunk_ids is None else chunk_ids
    rows = []
    for ci in ids:
        b, f0, vf, vt, _ = pl["chunks"][ci]
        a3 = conv_stem(chunk_image(features, b, f0, vf, cfg), P, fp8)  # [C, 16, 13]
        u = flatten_tokens(a3, vt)
        if fp8 & FP8_CONV:
            e = linear_conv_out_mx(u, P["conv_out_w"], P.get("conv_out_b"), a3.shape[1])
        else:
            e = linear(u, P["conv_out_w"], P.get("conv_out_b"))
        e = e + pe[:vt]
        rows.append(e)
    if rows:
        return np.concatenate(rows, axis=0), pl
    return np.zeros((0, d)), pl


def _lin(fp8: int, bit: int):
    """The product of one GEMM class: MX-fp8 operands when its bit is set."""
    return linear_mx if fp8 & bit else linear


def encoder_layer(x: np.ndarray, cu_seqlens, P: dict, i: int, cfg: dict, fp8: int = 0):
    """One pre-LN layer: x += Attn(LN1 x); x += FFN(LN2 x) with
    FFN(y) = fc2(GELU(fc1 y)).  qkv rows are [q; k; v].  ``fp8``: FP8_* bits
    of the products that take MX-fp8 operands."""
    p = f"layers.{i}."
    d = cfg["d_model"]
    h = layer_norm(x, P[p + "ln1_g"], P[p + "ln1_b"])
    qkv = _lin(fp8, FP8_QKV)(h, P[p + "qkv_w"], P.get(p + "qkv_b"))
    q, k, v = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    o = window_attention(q, k, v, cu_seqlens, cfg["encoder_attention_heads"])
    x = x + _lin(fp8, FP8_OUT)(o, P[p + "o_w"], P.get(p + "o_b"))
    h = layer_norm(x, P[p + "ln2_g"], P[p + "ln2_b"])
    f = gelu(_lin(fp8, FP8_FC1)(h, P[p + "fc1_w"], P.get(p + "fc1_b")))
    x = x + _lin(fp8, FP8_FC2)(f, P[p + "fc2_w"], P.get(p + "fc2_b"))
    return x


def encode(hidden: np.ndarray, cu_seqlens, P: dict, cfg: dict, fp8: int = 0) -> np.ndarray:
    """m-star ``encode``: the layer stack and projector over a packed
    sequence, (total_tokens, d_model) -> (total_tokens, output_dim)."""
    x = np.asarray(hidden, dtype=np.float64)
    for i in range(cfg["encoder_layers"]):
        x = encoder_layer(x, cu_seqlens, P, i, cfg, fp8)
    y = layer_norm(x, P["ln_post_g"], P["ln_post_b"])
    y = gelu(_lin(fp8, FP8_PROJ)(y, P["proj1_w"], P.get("proj1_b")))
    return _lin(fp8, FP8_PROJ)(y, P["proj2_w"], P.get("proj2_b"))


def forward(features, feature_lens, P: dict, cfg: dict, fp8: int = 0):
    """m-star ``forward``: (output [total_tokens, output_dim], layout)."""
    hidden, pl = frontend(features, feature_lens, P, cfg, fp8=fp8)
    return encode(hidden, pl["cu_seqlens"], P, cfg, fp8), pl


def window_chunks(pl: dict, cfg: dict) -> list[list[int]]:
    """Chunk ids of each window: a window is a whole number of chunks of one
    request, because window_tokens is a multiple of the tokens per chunk."""
    cu = pl["cu_seqlens"]
    out = []
    ci = 0
    for w in range(len(cu) - 1):
        s, e = cu[w], cu[w + 1]
        ids = []
        while ci < len(pl["chunks"]) and pl["chunks"][ci][4] < e:
            assert pl["chunks"][ci][4] >= s
            ids.append(ci)
            ci += 1
        out.append(ids)
    return out


def forward_windows(features, feature_lens, P: dict, cfg: dict, windows, fp8: int = 0):
    """Exact output rows of selected windows only.

    Windows are independent end to end (block-diagonal attention, per-row
    everything else), so a window's rows depend on its own chunks alone.
    Returns {window id: (first row, [rows, output_dim])}.
    """
    pl = plan(feature_lens, cfg)
    wch = window_chunks(pl, cfg)
    res = {}
    for w in windows:
        ids = wch[w]
        hidden, _ = frontend(features, feature_lens, P, cfg, chunk_ids=ids, fp8=fp8)
        n = hidden.shape[0]
        res[w] = (pl["cu_seqlens"][w], encode(hidden, [0, n], P, cfg, fp8))
    return res


# ---------------------------------------------------------------------------
# after the encoder: audio rows into the decoder's embedding sequence
# ---------------------------------------------------------------------------


def audio_rows(ids, pad_id: int, n_audio: int) -> np.ndarray:
    """Positions of the <|audio_pad|> placeholders in a token-id sequence, in
    order ("Audio Encoder Component", cubic.dev wiki, Data Flow and Integration:
    the audio features go into the text sequence at the placeholder positions,
    not appended).  There must be exactly one placeholder per audio row."""
    ids = np.asarray(ids)
    pos = np.nonzero(ids == pad_id)[0]
    if len(pos) != n_audio:
        raise ValueError(f"{len(pos)} placeholders for {n_audio} audio rows")
    return pos


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float64/float32 -> the nearest bfloat16 value (ties to even), as float32:
    keep the top 16 bits of the float32 pattern after adding the rounding bias
    0x7FFF plus the lowest kept bit (NaN inputs are not expected here)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def inject_audio(embeds: np.ndarray, ids, pad_id: int, audio: np.ndarray, out_dtype="fp32"):
    """The decoder's input sequence: row i is the text embedding `embeds[i]`
    unless ids[i] is the placeholder, in which case it is the next audio row
    (same passage as ``audio_rows``).  out_dtype "bf16": every row stored as
    bfloat16 (round to nearest even), the text rows being bf16 already."""
    pos = audio_rows(ids, pad_id, audio.shape[0])
    out = np.array(embeds, dtype=np.float64, copy=True)
    out[pos] = audio
    if out_dtype == "bf16":
        out = bf16_round(out).astype(np.float64)
    return out


# ---------------------------------------------------------------------------
# before the encoder: Whisper-style log-mel of 16 kHz mono audio
# ---------------------------------------------------------------------------
# The pages fix 16 kHz mono input, 128 mel bins and 100 frames per second
# ("Audio Encoder Component", cubic.dev wiki, Processing Pipeline; m-star
# module summary: a Whisper-style log-mel input).  Everything else is the
# published Whisper front end, taken as the reading: a 400-sample periodic
# Hann window and 400-point DFT every 160 samples, frames centred by reflect
# padding of 200 samples, the last frame dropped (N // 160 frames); the power
# spectrum; a Slaney-scale, Slaney-normalised triangular mel filterbank over
# 0..8000 Hz; log10 of max(mel, 1e-10); a floor at (the request's maximum - 8);
# then (x + 4) / 4.

SAMPLE_RATE = 16000
N_FFT = 400
HOP = 160


def hz_to_mel(f):
    """Slaney mel scale: linear 3/200 mel per Hz below 1 kHz (15 mel at 1 kHz),
    logarithmic above, 27 mel per factor 6.4."""
    f = np.asarray(f, dtype=np.float64)
    lin = 3.0 * f / 200.0
    log = 15.0 + 27.0 * np.log(np.maximum(f, 1e-300) / 1000.0) / np.log(6.4)
    return np.where(f >= 1000.0, log, lin)


def mel_to_hz(m):
    m = np.asarray(m, dtype=np.float64)
    return np.where(m >= 15.0, 1000.0 * np.exp((m - 15.0) * np.log(6.4) / 27.0), 200.0 * m / 3.0)


def mel_filterbank(n_mels: int = 128) -> np.ndarray:
    """[n_mels, N_FFT // 2 + 1] triangles between n_mels + 2 points equally spaced
    in mel from 0 Hz to the Nyquist frequency, each scaled to unit area
    (2 / (upper edge - lower edge))."""
    freqs = np.linspace(0.0, SAMPLE_RATE / 2.0, N_FFT // 2 + 1)
    pts = mel_to_hz(np.linspace(0.0, float(hz_to_mel(SAMPLE_RATE / 2.0)), n_mels + 2))
    w = np.zeros((n_mels, freqs.size))
    for m in range(n_mels):
        lo, c, hi = pts[m], pts[m + 1], pts[m + 2]
        rise = (freqs - lo) / (c - lo)
        fall = (hi - freqs) / (hi - c)
        w[m] = np.maximum(0.0, np.minimum(rise, fall)) * (2.0 / (hi - lo))
    return w


def hann(n: int = N_FFT) -> np.ndarray:
    """Periodic Hann window (the DFT-even form)."""
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * np.arange(n) / n)


def frames_for_samples(n_samples: int) -> int:
    return int(n_samples) // HOP


def power_spectrum(audio) -> np.ndarray:
    """[N // HOP, N_FFT // 2 + 1] |DFT|^2 of the windowed, centred frames."""
    x = np.asarray(audio, dtype=np.float64)
    nf = frames_for_samples(x.size)
    if nf == 0:
        return np.zeros((0, N_FFT // 2 + 1))
    if x.size <= N_FFT // 2:
        raise ValueError("reflect padding needs more than N_FFT / 2 samples")
    xp = np.pad(x, N_FFT // 2, mode="reflect")
    fr = np.stack([xp[f * HOP:f * HOP + N_FFT] for f in range(nf)]) * hann()
    return np.abs(np.fft.rfft(fr, axis=1)) ** 2


def log_mel(audio, n_mels: int = 128) -> np.ndarray:
    """[n_mels, N // HOP] Whisper-style log-mel of one request."""
    p = power_spectrum(audio)
    if p.shape[0] == 0:
        return np.zeros((n_mels, 0))
    mel = mel_filterbank(n_mels) @ p.T
    lg = np.log10(np.maximum(mel, 1e-10))
    lg = np.maximum(lg, lg.max() - 8.0)
    return (lg + 4.0) / 4.0
