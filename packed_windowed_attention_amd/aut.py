"""Python binding of libaut.so (the C ABI in include/aut.h).

Argument marshalling only: every step of the forward pass runs in the HIP
library.  PyTorch provides device memory and the stream.  There is no CPU
fallback: if the library cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libaut.so")

AUT_OK = 0
STATUS = {0: "AUT_OK", 1: "AUT_ERR_INVALID_ARG", 2: "AUT_ERR_UNSUPPORTED",
          3: "AUT_ERR_MISSING_WEIGHT", 4: "AUT_ERR_WORKSPACE_TOO_SMALL", 5: "AUT_ERR_HIP"}
DTYPES = {"fp32": 0, "bf16": 1, "fp8": 2}
KERNEL_CLASSES = ["conv1", "conv_gemm", "conv_out", "layernorm", "gemm", "attention", "logmel",
                  "gemm_fp8"]
# aut_config.fp8_gemms bits (the products on MX-fp8 operands under "fp8")
FP8_QKV, FP8_OUT, FP8_FC1, FP8_FC2, FP8_PROJ, FP8_CONV = 1, 2, 4, 8, 16, 32
FP8_ALL = 63

CONFIG_FIELDS = ["d_model", "encoder_layers", "encoder_attention_heads", "encoder_ffn_dim",
                 "num_mel_bins", "n_window", "n_window_infer", "conv_chunksize",
                 "downsample_hidden_size", "output_dim", "max_source_positions", "conv_out_bias"]


class AutConfig(ctypes.Structure):
    _fields_ = ([(f, c_int32) for f in CONFIG_FIELDS] + [("ln_eps", c_float)]
                + [("fp8_gemms", c_int32)])


class AutChunk(ctypes.Structure):
    _fields_ = [("request", c_int32), ("frame0", c_int32), ("valid_frames", c_int32),
                ("valid_tokens", c_int32), ("row0", c_int32)]


_SCALAR_W = ["conv1_w", "conv1_b", "conv2_w", "conv2_b", "conv3_w", "conv3_b",
             "conv_out_w", "conv_out_b"]
LAYER_W = ["ln1_g", "ln1_b", "qkv_w", "qkv_b", "o_w", "o_b", "ln2_g", "ln2_b",
           "fc1_w", "fc1_b", "fc2_w", "fc2_b"]
_TAIL_W = ["ln_post_g", "ln_post_b", "proj1_w", "proj1_b", "proj2_w", "proj2_b"]


class AutWeightPtrs(ctypes.Structure):
    _fields_ = ([(n, c_void_p) for n in _SCALAR_W] + [(n, POINTER(c_void_p)) for n in LAYER_W]
                + [(n, c_void_p) for n in _TAIL_W])


class AutKernelStats(ctypes.Structure):
    _fields_ = [("launches", c_int64), ("total_ms", c_double), ("flops", c_double), ("bytes", c_double)]


# name -> (restype, argtypes); the exported symbols of include/aut.h
SIGNATURES = {
    "aut_config_default": (c_int, [POINTER(AutConfig)]),
    "aut_config_check": (c_int, [POINTER(AutConfig)]),
    "aut_plan": (c_int, [POINTER(AutConfig), POINTER(c_int32), c_int32, POINTER(c_void_p)]),
    "aut_plan_counts": (c_int, [c_void_p, POINTER(c_int64), POINTER(c_int32), POINTER(c_int32)]),
    "aut_plan_copy": (c_int, [c_void_p, POINTER(c_int32), POINTER(c_int32), POINTER(AutChunk)]),
    "aut_plan_destroy": (None, [c_void_p]),
    "aut_weights_bytes": (c_int, [POINTER(AutConfig), c_int, POINTER(c_size_t)]),
    "aut_weights_pack": (c_int, [POINTER(AutConfig), POINTER(AutWeightPtrs), c_int, c_void_p,
                                 c_size_t, c_void_p]),
    "aut_workspace_bytes": (c_int, [POINTER(AutConfig), c_void_p, c_int, POINTER(c_size_t)]),
    "aut_plan_upload": (c_int, [c_void_p, c_void_p, c_size_t, c_void_p]),
    "aut_encode": (c_int, [POINTER(AutConfig), c_void_p, c_int32, POINTER(c_int32), c_int32,
                           c_void_p, c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
    "aut_encode_planned": (c_int, [POINTER(AutConfig), c_void_p, c_void_p, c_int32, c_void_p,
                                   c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
    "aut_frontend": (c_int, [POINTER(AutConfig), c_void_p, c_void_p, c_int32, c_void_p, c_int,
                             c_void_p, c_void_p, c_size_t, c_void_p]),
    "aut_encode_packed": (c_int, [POINTER(AutConfig), c_void_p, c_void_p, c_void_p, c_int,
                                  c_void_p, c_void_p, c_size_t, c_void_p]),
    "aut_stream_plan": (c_int, [POINTER(AutConfig), c_int32, c_int32, POINTER(c_int32),
                                POINTER(c_int32), POINTER(c_int32), POINTER(c_int32)]),
    "aut_stream_workspace_bytes": (c_int, [POINTER(AutConfig), c_int32, c_int, POINTER(c_size_t)]),
    "aut_encode_stream": (c_int, [POINTER(AutConfig), c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                  c_int, c_void_p, c_void_p, c_size_t, c_void_p, POINTER(c_int32)]),
    "aut_audio_rows": (c_int, [POINTER(c_int32), c_int64, c_int32, c_int64, POINTER(c_int32)]),
    "aut_inject_audio": (c_int, [c_void_p, c_void_p, c_int64, c_int32, c_void_p, c_int64, c_int,
                                 c_void_p]),
    "aut_logmel_tables_bytes": (c_int, [POINTER(c_size_t)]),
    "aut_logmel_tables_init": (c_int, [c_void_p, c_size_t, c_void_p]),
    "aut_logmel_workspace_bytes": (c_int, [c_int32, POINTER(c_size_t)]),
    "aut_logmel": (c_int, [c_void_p, c_int32, POINTER(c_int32), c_int32, c_void_p, c_void_p, c_int32,
                           c_void_p, c_size_t, c_void_p]),
    "aut_mx_scale_bytes": (c_int, [c_int64, c_int32, POINTER(c_size_t)]),
    "aut_mx_quantize": (c_int, [c_void_p, c_int64, c_int32, c_void_p, c_void_p, c_void_p]),
    "aut_mx_matmul": (c_int, [c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_int32, c_int32,
                              c_void_p, c_void_p]),
    "aut_encode_noalloc": (c_int, [POINTER(AutConfig), c_void_p, c_int32, POINTER(c_int32), c_int32, c_void_p,
                                    c_int, c_void_p, c_void_p]),
    "aut_attention": (c_int, [c_void_p, c_int64, c_int32, c_void_p, c_void_p, c_int32, c_int, c_int,
                              c_void_p, c_void_p, c_void_p]),
    "aut_layernorm": (c_int, [c_void_p, c_int64, c_int32, c_void_p, c_void_p, c_float, c_int, c_void_p,
                               c_void_p, c_void_p]),
    "aut_profile_enable": (c_int, [c_int]),
    "aut_profile_collect": (c_int, [POINTER(AutKernelStats)]),
    "aut_last_error": (c_char_p, []),
}

_lib = None


def lib():
    """The loaded libaut.so (built first if it is not there yet)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        # PyTorch ships its own HIP runtime under the same soname as the
        # system one this library links: load it first, so that the process
        # has one runtime.  (With the library loaded first, the system runtime
        # came in beside PyTorch's own libraries, and every launch from the
        # library failed with "no ROCm-capable device" while torch ran.)
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class AutError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def _check(st: int):
    if st != AUT_OK:
        msg = lib().aut_last_error()
        raise AutError(st, msg.decode() if msg else "")


def _dtype(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    return DTYPES[dtype]


def config(cfg: dict | None = None, **over) -> AutConfig:
    """aut_config from the library defaults, then a dict of AuTEncoderConfig
    fields (unknown keys ignored), then keyword overrides."""
    c = AutConfig()
    _check(lib().aut_config_default(byref(c)))
    src = dict(cfg or {})
    src.update(over)
    for f in CONFIG_FIELDS:
        if f in src:
            setattr(c, f, int(src[f]))
    if "ln_eps" in src:
        c.ln_eps = float(src["ln_eps"])
    if "fp8_gemms" in src:
        c.fp8_gemms = int(src["fp8_gemms"])
    return c


def config_check(cfg: AutConfig):
    _check(lib().aut_config_check(byref(cfg)))


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream)


def _ptr(t):
    return c_void_p(t.data_ptr()) if t is not None else c_void_p(0)


class Plan:
    """Owner of an aut_plan_t handle (host memory, freed with the object)."""

    def __init__(self, cfg: AutConfig, feature_lens):
        lens = [int(x) for x in feature_lens]
        arr = (c_int32 * max(1, len(lens)))(*lens)
        h = c_void_p()
        _check(lib().aut_plan(byref(cfg), arr, len(lens), byref(h)))
        self.handle = h
        self.cfg = cfg
        self.B = len(lens)
        tot, nw, nc = c_int64(), c_int32(), c_int32()
        _check(lib().aut_plan_counts(h, byref(tot), byref(nw), byref(nc)))
        self.total_tokens, self.n_windows, self.n_chunks = tot.value, nw.value, nc.value

    def copy(self):
        """(tokens_per_request, cu_seqlens, chunks as list of 5-tuples)."""
        tpr = (c_int32 * max(1, self.B))()
        cu = (c_int32 * (self.n_windows + 1))()
        ch = (AutChunk * max(1, self.n_chunks))()
        _check(lib().aut_plan_copy(self.handle, tpr, cu, ch))
        chunks = [(c.request, c.frame0, c.valid_frames, c.valid_tokens, c.row0)
                  for c in ch[:self.n_chunks]]
        return list(tpr[:self.B]), list(cu), chunks

    @property
    def cu_seqlens(self):
        return self.copy()[1]

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.aut_plan_destroy(h)
            self.handle = None


def plan(cfg: AutConfig, feature_lens) -> Plan:
    """aut_plan: host-only layout of one packed forward."""
    return Plan(cfg, feature_lens)


def weights_bytes(cfg: AutConfig, dtype) -> int:
    n = c_size_t()
    _check(lib().aut_weights_bytes(byref(cfg), _dtype(dtype), byref(n)))
    return n.value


def weights_pack(cfg: AutConfig, params: dict, dtype, device="cuda", stream=None):
    """aut_weights_pack: fp32 PyTorch-layout device tensors (names as in
    synth_inputs.param_shapes) -> a packed uint8 device tensor.  Missing names
    are passed as NULL so that the library reports them."""
    import torch
    L = cfg.encoder_layers
    w = AutWeightPtrs()
    keep = []
    for n in _SCALAR_W + _TAIL_W:
        t = params.get(n)
        setattr(w, n, t.data_ptr() if t is not None else None)
    for n in LAYER_W:
        arr = (c_void_p * max(1, L))()
        for i in range(L):
            t = params.get(f"layers.{i}.{n}")
            arr[i] = t.data_ptr() if t is not None else None
        keep.append(arr)
        setattr(w, n, ctypes.cast(arr, POINTER(c_void_p)))
    nbytes = weights_bytes(cfg, dtype)
    out = torch.empty(nbytes, dtype=torch.uint8, device=device)
    sp = _stream_ptr(stream)
    _check(lib().aut_weights_pack(byref(cfg), byref(w), _dtype(dtype), _ptr(out), nbytes, sp))
    # the sources only need to live until the pack kernels have read them
    (stream or torch.cuda.current_stream()).synchronize()
    return out


def workspace_bytes(cfg: AutConfig, pl: Plan, dtype) -> int:
    n = c_size_t()
    _check(lib().aut_workspace_bytes(byref(cfg), pl.handle, _dtype(dtype), byref(n)))
    return n.value


def workspace(cfg: AutConfig, pl: Plan, dtype, device="cuda"):
    import torch
    return torch.empty(max(1, workspace_bytes(cfg, pl, dtype)), dtype=torch.uint8, device=device)


def plan_upload(pl: Plan, ws, stream=None):
    _check(lib().aut_plan_upload(pl.handle, _ptr(ws), ws.numel(), _stream_ptr(stream)))


def _check_features(features, cfg: AutConfig, n_requests: int):
    """The kernels read features[b, :, :len_b] for every request b: the
    tensor must hold that many requests and cfg.num_mel_bins rows each."""
    if str(features.dtype) != "torch.float32":
        raise TypeError("features must be float32")
    if features.dim() != 3 or not features.is_contiguous():
        raise ValueError("features must be a contiguous [B, mel, T_max] tensor")
    if features.shape[0] < n_requests:
        raise ValueError(f"features holds {features.shape[0]} requests, the lengths name {n_requests}")
    if features.shape[1] != cfg.num_mel_bins:
        raise ValueError(f"features has {features.shape[1]} mel bins, the configuration {cfg.num_mel_bins}")


def _check_f32(t, rows: int, cols: int, what: str, device=None):
    """A caller-supplied fp32 buffer the kernels write (or read) rows x cols of."""
    if t is None:
        raise ValueError(f"{what} is missing")
    if str(t.dtype) != "torch.float32" or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous float32 tensor")
    if t.numel() < rows * cols:
        raise ValueError(f"{what} holds {t.numel()} values, needs {rows} x {cols}")
    if device is not None and t.device != device:
        raise ValueError(f"{what} is on {t.device}, the features on {device}")


def _check_bytes(t, need: int, what: str):
    if t is None or str(t.dtype) != "torch.uint8" or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous uint8 tensor")
    if t.numel() < need:
        raise ValueError(f"{what} holds {t.numel()} bytes, needs {need}")


def encode(cfg: AutConfig, features, feature_lens, packed, dtype, out=None, ws=None, stream=None):
    """aut_encode: the whole forward; returns (out [T, output_dim] fp32, plan)."""
    import torch
    lens = [int(x) for x in feature_lens]
    _check_features(features, cfg, len(lens))
    pl = Plan(cfg, feature_lens)
    if out is None:
        out = torch.empty((pl.total_tokens, cfg.output_dim), dtype=torch.float32, device=features.device)
    _check_f32(out, pl.total_tokens, cfg.output_dim, "out", features.device)
    if ws is None:
        ws = workspace(cfg, pl, dtype, device=features.device)
    _check_bytes(ws, workspace_bytes(cfg, pl, dtype), "ws")
    _check_bytes(packed, weights_bytes(cfg, dtype), "packed")
    arr = (c_int32 * max(1, len(lens)))(*lens)
    _check(lib().aut_encode(byref(cfg), _ptr(features), features.shape[2], arr, len(lens),
                            _ptr(packed), _dtype(dtype), _ptr(out), _ptr(ws), ws.numel(),
                            _stream_ptr(stream)))
    return out, pl


def encode_noalloc(cfg: AutConfig, features, feature_lens, packed, dtype, out=None, stream=None):
    """aut_encode_noalloc: the whole forward on the library's device scratch
    (no workspace argument); returns (out [T, output_dim] fp32, plan)."""
    import torch
    lens = [int(x) for x in feature_lens]
    _check_features(features, cfg, len(lens))
    pl = Plan(cfg, feature_lens)
    if out is None:
        out = torch.empty((pl.total_tokens, cfg.output_dim), dtype=torch.float32, device=features.device)
    _check_f32(out, pl.total_tokens, cfg.output_dim, "out", features.device)
    _check_bytes(packed, weights_bytes(cfg, dtype), "packed")
    arr = (c_int32 * max(1, len(lens)))(*lens)
    _check(lib().aut_encode_noalloc(byref(cfg), _ptr(features), features.shape[2], arr, len(lens),
                                    _ptr(packed), _dtype(dtype), _ptr(out), _stream_ptr(stream)))
    return out, pl


def encode_planned(cfg: AutConfig, pl: Plan, features, packed, dtype, out, ws, stream=None):
    """aut_encode_planned: kernels only, for a plan already uploaded into ws."""
    _check_features(features, cfg, pl.B)
    _check_f32(out, pl.total_tokens, cfg.output_dim, "out", features.device)
    _check_bytes(ws, workspace_bytes(cfg, pl, dtype), "ws")
    _check_bytes(packed, weights_bytes(cfg, dtype), "packed")
    _check(lib().aut_encode_planned(byref(cfg), pl.handle, _ptr(features), features.shape[2],
                                    _ptr(packed), _dtype(dtype), _ptr(out), _ptr(ws), ws.numel(),
                                    _stream_ptr(stream)))
    return out


def frontend(cfg: AutConfig, pl: Plan, features, packed, dtype, hidden, ws, stream=None):
    """aut_frontend: features -> packed hidden [T, d_model] fp32 (plan uploaded)."""
    _check_features(features, cfg, pl.B)
    _check_f32(hidden, pl.total_tokens, cfg.d_model, "hidden", features.device)
    _check_bytes(ws, workspace_bytes(cfg, pl, dtype), "ws")
    _check_bytes(packed, weights_bytes(cfg, dtype), "packed")
    _check(lib().aut_frontend(byref(cfg), pl.handle, _ptr(features), features.shape[2],
                              _ptr(packed), _dtype(dtype), _ptr(hidden), _ptr(ws), ws.numel(),
                              _stream_ptr(stream)))
    return hidden


def encode_packed(cfg: AutConfig, pl: Plan, hidden, packed, dtype, out, ws, stream=None):
    """aut_encode_packed: layer stack + projector over packed hidden (plan uploaded)."""
    _check_f32(hidden, pl.total_tokens, cfg.d_model, "hidden")
    _check_f32(out, pl.total_tokens, cfg.output_dim, "out", hidden.device)
    _check_bytes(ws, workspace_bytes(cfg, pl, dtype), "ws")
    _check_bytes(packed, weights_bytes(cfg, dtype), "packed")
    _check(lib().aut_encode_packed(byref(cfg), pl.handle, _ptr(hidden), _ptr(packed),
                                   _dtype(dtype), _ptr(out), _ptr(ws), ws.numel(),
                                   _stream_ptr(stream)))
    return out


def stream_plan(cfg: AutConfig, frames_total: int, windows_final: int) -> dict:
    """aut_stream_plan: frame/row range of one incremental-encode step."""
    f0, r0, rows, after = c_int32(), c_int32(), c_int32(), c_int32()
    _check(lib().aut_stream_plan(byref(cfg), int(frames_total), int(windows_final), byref(f0),
                                 byref(r0), byref(rows), byref(after)))
    return dict(frame_begin=f0.value, row_begin=r0.value, rows=rows.value,
                windows_final_after=after.value)


def stream_workspace(cfg: AutConfig, max_frames: int, dtype, device="cuda"):
    """Workspace for every step of a request of up to max_frames frames."""
    import torch
    n = c_size_t()
    _check(lib().aut_stream_workspace_bytes(byref(cfg), int(max_frames), _dtype(dtype), byref(n)))
    return torch.empty(max(1, n.value), dtype=torch.uint8, device=device)


def encode_stream(cfg: AutConfig, features, frames_total: int, windows_final: int, packed, dtype,
                  out, ws, stream=None) -> int:
    """aut_encode_stream: re-encode a live request from its first non-final
    window; features [mel, T_max] fp32 on the device, out the request's output
    rows.  Returns the new count of final windows."""
    if str(features.dtype) != "torch.float32" or features.dim() != 2 or not features.is_contiguous():
        raise ValueError("features must be a contiguous float32 [mel, T_max] tensor")
    if features.shape[0] != cfg.num_mel_bins:
        raise ValueError(f"features has {features.shape[0]} mel bins, the configuration {cfg.num_mel_bins}")
    # the request's output rows for the frames received so far
    rows = Plan(cfg, [int(frames_total)]).total_tokens if int(frames_total) >= 0 else 0
    _check_f32(out, rows, cfg.output_dim, "out", features.device)
    _check_bytes(packed, weights_bytes(cfg, dtype), "packed")
    after = c_int32()
    _check(lib().aut_encode_stream(byref(cfg), _ptr(features), features.shape[1], int(frames_total),
                                   int(windows_final), _ptr(packed), _dtype(dtype), _ptr(out),
                                   _ptr(ws), ws.numel(), _stream_ptr(stream), byref(after)))
    return after.value


def logmel_tables(device="cuda", stream=None):
    """aut_logmel_tables_bytes + aut_logmel_tables_init: the constant tables on the device."""
    import torch
    n = c_size_t()
    _check(lib().aut_logmel_tables_bytes(byref(n)))
    t = torch.empty(n.value, dtype=torch.uint8, device=device)
    _check(lib().aut_logmel_tables_init(_ptr(t), n.value, _stream_ptr(stream)))
    return t


def logmel(audio, sample_lens, tables, features=None, T_max=None, ws=None, stream=None):
    """aut_logmel: audio fp32 [B, S_max] on the device -> features [B, 128, T_max]
    (frames past a request's count are left as they are; a new buffer is zeroed)."""
    import torch
    lens = [int(x) for x in sample_lens]
    B = len(lens)
    if T_max is None:
        T_max = max([n // 160 for n in lens] + [1])
        T_max = (T_max + 3) // 4 * 4
    if features is None:
        features = torch.zeros((B, 128, T_max), dtype=torch.float32, device=audio.device)
    if ws is None:
        n = c_size_t()
        _check(lib().aut_logmel_workspace_bytes(B, byref(n)))
        ws = torch.empty(max(1, n.value), dtype=torch.uint8, device=audio.device)
    arr = (c_int32 * max(1, B))(*lens)
    _check(lib().aut_logmel(_ptr(audio), audio.shape[1], arr, B, _ptr(tables), _ptr(features),
                            features.shape[2], _ptr(ws), ws.numel(), _stream_ptr(stream)))
    return features


def audio_rows(ids, pad_id: int, n_audio: int) -> list:
    """aut_audio_rows: placeholder positions of a token-id sequence (host)."""
    ids = [int(x) for x in ids]
    arr = (c_int32 * max(1, len(ids)))(*ids)
    rows = (c_int32 * max(1, int(n_audio)))()
    _check(lib().aut_audio_rows(arr, len(ids), int(pad_id), int(n_audio), rows))
    return list(rows)[:int(n_audio)]


def inject_audio(audio, rows, dst, dst_dtype, stream=None):
    """aut_inject_audio: dst[rows[j]] = audio[j] on the device (rows: int32 device tensor)."""
    if str(rows.dtype) != "torch.int32":
        raise TypeError("rows must be int32")
    _check(lib().aut_inject_audio(_ptr(audio), _ptr(rows), rows.numel(), audio.shape[1], _ptr(dst),
                                  dst.shape[0], _dtype(dst_dtype), _stream_ptr(stream)))
    return dst


def profile_enable(on: bool):
    _check(lib().aut_profile_enable(1 if on else 0))


def profile_collect() -> dict:
    """{class name: dict(launches, total_ms, flops, bytes)} since the last collect."""
    st = (AutKernelStats * len(KERNEL_CLASSES))()
    _check(lib().aut_profile_collect(st))
    return {n: dict(launches=s.launches, total_ms=s.total_ms, flops=s.flops, bytes=s.bytes)
            for n, s in zip(KERNEL_CLASSES, st)}


def mx_scale_bytes(rows: int, K: int) -> int:
    n = c_size_t()
    _check(lib().aut_mx_scale_bytes(int(rows), int(K), byref(n)))
    return n.value


def mx_quantize(x, stream=None):
    """aut_mx_quantize: fp32 [R, K] on the device -> (e4m3 codes uint8 [R, K],
    scale codes uint8 in the kernels' layout, mx_scale_bytes(R, K) bytes)."""
    if str(x.dtype) != "torch.float32" or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D float32 tensor")
    import torch
    R, K = x.shape
    codes = torch.empty((R, K), dtype=torch.uint8, device=x.device)
    scales = torch.empty(max(1, mx_scale_bytes(R, K)), dtype=torch.uint8, device=x.device)
    _check(lib().aut_mx_quantize(_ptr(x), R, K, _ptr(codes), _ptr(scales), _stream_ptr(stream)))
    return codes, scales


def mx_scales_rowmajor(scales, rows: int, K: int):
    """The kernels' scale layout as [rows, K / 32] (host-side reindexing)."""
    import numpy as np
    s = np.asarray(scales)
    r = np.arange(rows)[:, None]
    kb = np.arange(K // 32)[None, :]
    idx = ((r // 16) * (K // 128) + kb // 4) * 64 + (kb % 4) * 16 + r % 16
    return s[idx]


def mx_matmul(a_codes, a_scales, b_codes, b_scales, out=None, stream=None):
    """aut_mx_matmul: out fp32 [M, N] = A B^T on MX-fp8 operands (codes
    [M, K] and [N, K] with their scales in the kernels' layout)."""
    import torch
    M, K = a_codes.shape
    N = b_codes.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a_codes.device)
    _check(lib().aut_mx_matmul(_ptr(a_codes), _ptr(a_scales), M, _ptr(b_codes), _ptr(b_scales), N,
                               K, _ptr(out), _stream_ptr(stream)))
    return out


def attention(qkv, cu_seqlens, window_order, heads: int, out_dtype=None, stream=None):
    """aut_attention: qkv [R, 3 d] (float32 or bfloat16, contiguous, on the
    device) with device int32 cu_seqlens [n + 1] and window_order [n] ->
    out [R, d] in out_dtype ("fp32", "bf16" or, from bf16 qkv, "fp8": e4m3
    codes uint8 [R, d] and scale codes in the MX layout).  Default out_dtype:
    qkv's.  Rows outside every window are returned as zero."""
    import torch
    if qkv.dim() != 2 or not qkv.is_contiguous() or qkv.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("qkv must be a contiguous 2-D float32 or bfloat16 tensor")
    in_dt = "fp32" if qkv.dtype == torch.float32 else "bf16"
    out_dtype = out_dtype or in_dt
    R = qkv.shape[0]
    d = 64 * int(heads)
    if qkv.shape[1] != 3 * d:
        raise ValueError(f"qkv has {qkv.shape[1]} columns, 3 x 64 x heads = {3 * d} expected")
    for t in (cu_seqlens, window_order):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous() or t.device != qkv.device:
            raise ValueError("cu_seqlens and window_order must be contiguous int32 vectors on qkv's device")
    n = window_order.numel()
    if cu_seqlens.numel() != n + 1:
        raise ValueError("cu_seqlens must hold one more entry than window_order")
    odt = _dtype(out_dtype)
    scales = None
    if odt == DTYPES["fp8"]:
        out = torch.zeros((R, d), dtype=torch.uint8, device=qkv.device)
        nsc = mx_scale_bytes(R, d) if d % 128 == 0 else 1
        scales = torch.zeros(max(1, nsc), dtype=torch.uint8, device=qkv.device)
    else:
        out = torch.zeros((R, d), dtype=torch.float32 if odt == DTYPES["fp32"] else torch.bfloat16,
                          device=qkv.device)
    _check(lib().aut_attention(_ptr(qkv), R, int(heads), _ptr(cu_seqlens), _ptr(window_order), n,
                               _dtype(in_dt), odt, _ptr(out), _ptr(scales) if scales is not None else None,
                               _stream_ptr(stream)))
    return (out, scales) if scales is not None else out


def layernorm(x, gamma, beta, dtype="fp32", eps=1e-5, stream=None):
    """aut_layernorm: fp32 [R, d] rows on the device -> fp32 / bf16 [R, d],
    or for "fp8" (e4m3 codes uint8 [R, d], scale codes in the MX layout)."""
    import torch
    if str(x.dtype) != "torch.float32" or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D float32 tensor")
    R, d = x.shape
    for t in (gamma, beta):
        if str(t.dtype) != "torch.float32" or t.numel() != d or not t.is_contiguous() or t.device != x.device:
            raise ValueError("gamma and beta must be contiguous float32 [d] tensors on x's device")
    dt = _dtype(dtype)
    scales = None
    if dt == DTYPES["fp8"]:
        y = torch.empty((R, d), dtype=torch.uint8, device=x.device)
        # (a d the library refuses gets a placeholder: the call reports it)
        nsc = mx_scale_bytes(R, d) if d > 0 and d % 128 == 0 else 1
        scales = torch.zeros(max(1, nsc), dtype=torch.uint8, device=x.device)
    else:
        y = torch.empty((R, d), dtype=torch.float32 if dt == DTYPES["fp32"] else torch.bfloat16,
                        device=x.device)
    _check(lib().aut_layernorm(_ptr(x), R, d, _ptr(gamma), _ptr(beta), float(eps), dt, _ptr(y),
                               _ptr(scales) if scales is not None else None, _stream_ptr(stream)))
    return (y, scales) if scales is not None else y
