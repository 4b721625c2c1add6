/*
 * aut.h -- C ABI of the AuT audio-encoder forward pass on MI355X (gfx950).
 *
 * The encoder: a 128-bin log-mel at 100 frames/s is cut into 1 s chunks of
 * 2 * n_window frames, each chunk goes through three stride-2 Conv2d + GELU
 * layers and a linear conv_out, gets the chunk-local sinusoidal positions,
 * and the valid tokens of every chunk are packed into one
 * [total_tokens, d_model] sequence; a pre-LN stack of LayerNorm-with-bias
 * encoder layers attends bidirectionally inside windows of n_window_infer
 * frames (8 s -> 104 tokens) and a final LayerNorm + Linear/GELU/Linear
 * projector maps every token to output_dim.  Sources: "mstar.model.
 * components.aut_encoder" (m-star API page, module summary and the
 * AuTEncoder / AuTEncoderConfig / AuTLayout entries) and "1A - AuT Audio
 * Encoder" (openarchlab course, sections 1 and 3).
 *
 * Conventions for every call below:
 *  - Every function returns aut_status; AUT_OK is 0.  On any other value
 *    aut_last_error() returns a message for the calling thread.  No C++
 *    exception crosses this interface.
 *  - "device" pointers are HIP device memory on the current device; "host"
 *    pointers are ordinary host memory.  The caller owns every buffer
 *    (features, parameters, packed parameters, workspace, outputs) and the
 *    stream.  The library never allocates or frees device memory and never
 *    synchronises the device, except where a call says so.  Host-to-device
 *    copies of host arguments (plan tables, lengths) go through one pinned
 *    host buffer per device that the library keeps (see aut_plan_upload).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - All argument checks happen before the first launch: a call that fails
 *    validation has enqueued nothing.
 *  - A batch without tokens (B = 0, or every length 0) is valid: the forward
 *    calls enqueue nothing and need no device buffers (they may be NULL).
 *  - Asynchronous faults of launched work surface as AUT_ERR_HIP from a later
 *    call (or from the caller's own synchronisation).
 */
#ifndef AUT_H_
#define AUT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AUT_OK = 0,
  AUT_ERR_INVALID_ARG = 1,         /* NULL handle/pointer, negative or too long length, bad dtype */
  AUT_ERR_UNSUPPORTED = 2,         /* a configuration the kernels do not implement */
  AUT_ERR_MISSING_WEIGHT = 3,      /* a required parameter pointer is NULL (message names it) */
  AUT_ERR_WORKSPACE_TOO_SMALL = 4, /* workspace or destination smaller than required */
  AUT_ERR_HIP = 5                  /* a HIP runtime call failed */
} aut_status;

/* Arithmetic type of the matrix products.  AUT_FP32: every operand and every
 * activation is fp32.  AUT_BF16: GEMM/conv/attention operands are bf16
 * (round to nearest even), accumulation, LayerNorm statistics, softmax and
 * the residual stream stay fp32.  AUT_FP8: as AUT_BF16, except that the
 * encoder-layer and projector products named by aut_config.fp8_gemms take
 * MX-fp8 operands (OCP Microscaling formats: e4m3 elements, one power-of-two
 * E8M0 scale per 32 consecutive values along the contraction axis, the
 * smallest scale with no element above 448, elements rounded to nearest
 * even), quantized by the kernel that produces each operand; accumulation
 * stays fp32.  The 8-bit variants on the pages (soniqo "Qwen3-ASR" transcribe
 * guide: the INT8 CoreML encoder, the 8/5/4-bit MLX rows of the performance
 * table) are weight-only formats of Apple hardware; this is the 8-bit format
 * the gfx950 matrix cores multiply at twice the bf16 rate.  Requires d_model
 * and encoder_ffn_dim multiples of 128. */
typedef enum { AUT_FP32 = 0, AUT_BF16 = 1, AUT_FP8 = 2 } aut_dtype;

/* aut_config.fp8_gemms bits: the products that run on MX-fp8 under AUT_FP8. */
enum {
  AUT_FP8_QKV = 1,   /* fused q/k/v projection (operand: LayerNorm 1 output) */
  AUT_FP8_OUT = 2,   /* attention output projection (operand: attention output) */
  AUT_FP8_FC1 = 4,   /* FFN fc1 (operand: LayerNorm 2 output) */
  AUT_FP8_FC2 = 8,   /* FFN fc2 (operand: GELU(fc1) output) */
  AUT_FP8_PROJ = 16, /* projector proj1 and proj2 */
  AUT_FP8_CONV = 32, /* conv stem: conv2, conv3 (blocks of 32 channels of one tap) and conv_out
                        (32 channels of one frequency bin); needs downsample_hidden_size a
                        multiple of 32 */
  AUT_FP8_ALL = 63
};

/* Model hyper-parameters.  Field names and defaults follow AuTEncoderConfig
 * on the m-star API page; ln_eps and conv_out_bias are additions (LayerNorm
 * epsilon 1e-5, conv_out without bias by default).
 * Supported: num_mel_bins = 128; d_model = 64 * encoder_attention_heads,
 * d_model a multiple of 64 and <= 2048; n_window_infer a multiple of
 * 2 * n_window; tokens per window <= 128; downsample_hidden_size a multiple
 * of 8; encoder_ffn_dim and output_dim multiples of 8. */
typedef struct {
  int32_t d_model;                /* 1024 */
  int32_t encoder_layers;         /* 24 */
  int32_t encoder_attention_heads;/* 16 */
  int32_t encoder_ffn_dim;        /* 4096 */
  int32_t num_mel_bins;           /* 128 */
  int32_t n_window;               /* 50: a chunk is 2 * n_window frames */
  int32_t n_window_infer;         /* 800 frames per attention window */
  int32_t conv_chunksize;         /* 500: chunks per conv-stem batch (memory only) */
  int32_t downsample_hidden_size; /* 480: conv channels C */
  int32_t output_dim;             /* 2048 */
  int32_t max_source_positions;   /* 1500: sinusoid table length */
  int32_t conv_out_bias;          /* 0: conv_out has no bias; 1: it has one */
  float ln_eps;                   /* 1e-5 */
  int32_t fp8_gemms;              /* AUT_FP8_* bits, read under AUT_FP8 only; default AUT_FP8_ALL */
} aut_config;

/* One chunk of the plan: which request it belongs to, its first mel frame,
 * how many frames of it are real (<= 2 * n_window), how many tokens it keeps,
 * and the packed row of its first token. */
typedef struct {
  int32_t request;
  int32_t frame0;
  int32_t valid_frames;
  int32_t valid_tokens;
  int32_t row0;
} aut_chunk;

typedef struct aut_plan aut_plan_t;

/* Parameters as produced by a PyTorch-layout model, all fp32 *device*
 * pointers: conv weights [C_out, C_in, 3, 3] (conv1: C_in = 1), linear
 * weights [out, in].  Per-layer fields are *host* arrays holding
 * encoder_layers device pointers each.  qkv_w stacks the q, k and v
 * projections row-wise ([3 d, d], rows q then k then v), as the m-star page's
 * fused qkv_proj does.  Every pointer is required except conv_out_b, which is
 * read only when conv_out_bias = 1. */
typedef struct {
  const float* conv1_w;  const float* conv1_b;
  const float* conv2_w;  const float* conv2_b;
  const float* conv3_w;  const float* conv3_b;
  const float* conv_out_w; const float* conv_out_b;   /* [d, C * 16], index c * 16 + f */
  const float* const* ln1_g; const float* const* ln1_b;
  const float* const* qkv_w; const float* const* qkv_b;
  const float* const* o_w;   const float* const* o_b;
  const float* const* ln2_g; const float* const* ln2_b;
  const float* const* fc1_w; const float* const* fc1_b;
  const float* const* fc2_w; const float* const* fc2_b;
  const float* ln_post_g; const float* ln_post_b;
  const float* proj1_w; const float* proj1_b;          /* [d, d] */
  const float* proj2_w; const float* proj2_b;          /* [output_dim, d] */
} aut_weight_ptrs;

/* Fills *cfg with the AuTEncoderConfig defaults (m-star API page). */
aut_status aut_config_default(aut_config* cfg);

/* Checks a configuration against what the kernels implement
 * (AUT_ERR_UNSUPPORTED with a reason otherwise). */
aut_status aut_config_check(const aut_config* cfg);

/* Host-only layout of one packed forward (m-star AuTEncoder.layout and
 * tokens_for_frames / window_lengths): per request, ceil(L / chunk) chunks,
 * tokens = three ceiling halvings of each chunk's valid frames (13 for a full
 * 100-frame chunk), windows of window_tokens (104) then the remainder; windows
 * never span requests; packed rows ordered request, chunk, token.
 * feature_lens: host int32[B], each >= 0 (0 = an empty request with no
 * tokens and no window).  B >= 0.  Never touches the GPU.  The handle is
 * library-owned host memory, freed by aut_plan_destroy. */
aut_status aut_plan(const aut_config* cfg, const int32_t* feature_lens, int32_t B,
                    aut_plan_t** out);

/* Sizes of a plan; any output pointer may be NULL. */
aut_status aut_plan_counts(const aut_plan_t* plan, int64_t* total_tokens, int32_t* n_windows,
                           int32_t* n_chunks);

/* Copies a plan into host arrays; any may be NULL.  tokens_per_request:
 * int32[B]; cu_seqlens: int32[n_windows + 1] (window starts, then the total);
 * chunks: aut_chunk[n_chunks]. */
aut_status aut_plan_copy(const aut_plan_t* plan, int32_t* tokens_per_request, int32_t* cu_seqlens,
                         aut_chunk* chunks);

void aut_plan_destroy(aut_plan_t* plan);

/* Bytes of the packed-parameter buffer for (cfg, dtype). */
aut_status aut_weights_bytes(const aut_config* cfg, aut_dtype dtype, size_t* bytes);

/* Converts PyTorch-layout fp32 parameters into the kernels' layout and dtype
 * in the caller's device buffer `dst` (aut_weights_bytes bytes), and computes
 * the sinusoid position table into it (positions are computed, never loaded:
 * cubic.dev wiki, "Positional Embeddings").  A NULL required pointer gives
 * AUT_ERR_MISSING_WEIGHT naming the field (the m-star load_weights refuses to
 * leave a parameter unloaded).  Asynchronous on `stream`; the sources must
 * stay valid until the stream has passed this work. */
aut_status aut_weights_pack(const aut_config* cfg, const aut_weight_ptrs* src, aut_dtype dtype,
                            void* dst, size_t dst_bytes, void* stream);

/* Device workspace bytes a forward of `plan` needs (plan tables, conv-stem
 * batch buffers, residual stream and layer activations). */
aut_status aut_workspace_bytes(const aut_config* cfg, const aut_plan_t* plan, aut_dtype dtype,
                               size_t* bytes);

/* Copies the plan's tables into the workspace: into a library-owned pinned
 * host buffer (one per device, grown on demand, kept until the process ends),
 * then one asynchronous H2D copy on `stream`.  The plan may be destroyed as
 * soon as this returns.  Before reusing the pinned buffer the call waits, on
 * the host, for the previous upload's copy out of it to finish.  Must precede
 * aut_encode_planned / aut_frontend / aut_encode_packed with the same plan and
 * workspace; it is the step kept outside a captured graph (the m-star page
 * builds the attention plan outside the graph). */
aut_status aut_plan_upload(const aut_plan_t* plan, void* workspace, size_t workspace_bytes,
                           void* stream);

/* The whole forward (m-star AuTEncoder.forward): plan, upload, frontend,
 * encoder stack, projector.
 * features: device fp32 [B, num_mel_bins, T_max], time fastest; frames at or
 *   past feature_lens[b] are never read (treated as zero).
 * feature_lens: host int32[B], 0 <= L <= T_max.
 * packed: the aut_weights_pack buffer of the same cfg and dtype.
 * out: device fp32 [total_tokens, output_dim], packed row order.
 * workspace: device, >= aut_workspace_bytes for this batch.
 * Asynchronous on `stream`; the plan upload goes through aut_plan_upload's
 * pinned buffer, so the temporary plan is freed before the call returns. */
aut_status aut_encode(const aut_config* cfg, const float* features, int32_t T_max,
                      const int32_t* feature_lens, int32_t B, const void* packed, aut_dtype dtype,
                      float* out, void* workspace, size_t workspace_bytes, void* stream);

/* aut_encode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same plan and kernels, with the workspace in a library-owned device
 * scratch array of 256 MiB per GPU (allocated with the library's code object
 * when it is loaded on that GPU, held until the process ends) instead of a
 * caller buffer.  Neither it nor anything it calls allocates device or pinned
 * memory; the plan tables are copied from the plan's host memory directly
 * (pageable), so the call may wait for the stream's earlier work.
 * Returns AUT_ERR_WORKSPACE_TOO_SMALL, before touching the GPU, for a batch
 * whose aut_workspace_bytes exceeds 256 MiB (e.g. d_model 1280 with C 480
 * fits about 300 s of audio per call at conv_chunksize 16).  All calls on one
 * GPU share its scratch: calls that overlap in time on one GPU (other streams
 * or threads) race and must be serialised by the caller.  Arguments as
 * aut_encode, without the workspace.  Keep aut_profile_enable off: its timing
 * events are created on demand. */
aut_status aut_encode_noalloc(const aut_config* cfg, const float* features, int32_t T_max,
                              const int32_t* feature_lens, int32_t B, const void* packed,
                              aut_dtype dtype, float* out, void* stream);

/* Kernels only, for a plan already uploaded into `workspace`: no allocation,
 * no synchronisation, no host-to-device copy, so it can be captured in a HIP
 * graph and replayed.  Arguments as aut_encode. */
aut_status aut_encode_planned(const aut_config* cfg, const aut_plan_t* plan, const float* features,
                              int32_t T_max, const void* packed, aut_dtype dtype, float* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* The frontend alone (m-star AuTEncoder.frontend): features -> packed chunk
 * embeddings with positions, hidden: device fp32 [total_tokens, d_model].
 * Requires the plan uploaded into `workspace`. */
aut_status aut_frontend(const aut_config* cfg, const aut_plan_t* plan, const float* features,
                        int32_t T_max, const void* packed, aut_dtype dtype, float* hidden,
                        void* workspace, size_t workspace_bytes, void* stream);

/* The layer stack and projector over a packed sequence (m-star
 * AuTEncoder.encode): hidden device fp32 [total_tokens, d_model] (read only)
 * -> out device fp32 [total_tokens, output_dim], attention blocks from the
 * plan's cu_seqlens.  Requires the plan uploaded into `workspace`. */
aut_status aut_encode_packed(const aut_config* cfg, const aut_plan_t* plan, const float* hidden,
                             const void* packed, aut_dtype dtype, float* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Incremental (streaming) encode of one live request.
 *
 * A window covers its own n_window_infer frames (8 chunks; m-star
 * AuTEncoderConfig.window_lengths: windows never span requests or other
 * frames) and attention is block-diagonal over windows (m-star module
 * summary; openarchlab "1A", section 4: perturbing one window leaves every
 * other window's output unchanged).  So once a request holds all
 * n_window_infer frames of a window, that window's output rows are final, and
 * a caller that appends audio re-encodes only the frames from the first
 * window that was not final at its previous step.  The result equals the
 * batch encode of the whole request, bit for bit.
 * ------------------------------------------------------------------------ */

/* Host-only arithmetic for one step.  frames_total >= 0 frames received so
 * far; windows_final >= 0 windows already emitted as final (at most the
 * complete windows in frames_total, else AUT_ERR_INVALID_ARG).  Outputs (any
 * may be NULL):
 *   frame_begin         = windows_final * n_window_infer, first frame to encode;
 *   row_begin           = windows_final * window tokens, its first output row;
 *   rows                = output rows from row_begin to the request's end
 *                         (0 when nothing is left to encode);
 *   windows_final_after = complete windows in frames_total. */
aut_status aut_stream_plan(const aut_config* cfg, int32_t frames_total, int32_t windows_final,
                           int32_t* frame_begin, int32_t* row_begin, int32_t* rows,
                           int32_t* windows_final_after);

/* Workspace bytes that cover every step of a request of up to max_frames
 * frames (the workspace of a one-request plan of max_frames frames). */
aut_status aut_stream_workspace_bytes(const aut_config* cfg, int32_t max_frames, aut_dtype dtype,
                                      size_t* bytes);

/* One step: encodes frames [frame_begin, frames_total) of the request whose
 * log-mel is `features` (device fp32 [num_mel_bins, T_max], time fastest,
 * T_max >= frames_total) and writes output rows [row_begin, row_begin + rows)
 * of `out` (device fp32, the request's output, [tokens(frames_total),
 * output_dim] or longer).  Rows before row_begin are not touched.  The
 * workspace must hold aut_stream_workspace_bytes for frames_total frames.
 * Stream use and synchronisation as aut_encode.  *windows_final_after (may
 * be NULL) receives the new count of final windows. */
aut_status aut_encode_stream(const aut_config* cfg, const float* features, int32_t T_max,
                             int32_t frames_total, int32_t windows_final, const void* packed,
                             aut_dtype dtype, float* out, void* workspace, size_t workspace_bytes,
                             void* stream, int32_t* windows_final_after);

/* ------------------------------------------------------------------------
 * Before the encoder: Whisper-style log-mel of 16 kHz mono audio
 * ("Audio Encoder Component", cubic.dev wiki, Processing Pipeline: 16 kHz
 * mono audio becomes a 128-bin mel spectrogram; m-star module summary: a
 * Whisper-style log-mel input at 100 frames/s).  Beyond what the pages fix,
 * the published Whisper front end: 400-sample periodic Hann window and
 * 400-point DFT every 160 samples on reflect-padded centred frames
 * (sample_len / 160 frames), power spectrum, Slaney mel filterbank over
 * 0..8000 Hz, log10 of max(mel, 1e-10), floor at the request's maximum - 8,
 * then (x + 4) / 4.
 * ------------------------------------------------------------------------ */

/* Bytes of the constant tables (window x DFT, mel filterbank), and filling
 * them on the device (once; caller-owned device buffer, 256-byte aligned). */
aut_status aut_logmel_tables_bytes(size_t* bytes);
aut_status aut_logmel_tables_init(void* tables, size_t bytes, void* stream);

/* Workspace bytes for B requests. */
aut_status aut_logmel_workspace_bytes(int32_t B, size_t* bytes);

/* audio: device fp32 [B, S_max] (request b's samples first, sample_lens[b] of
 * them, host int32, each 0 or > 200 and <= S_max); features: device fp32
 * [B, 128, T_max], T_max >= max(sample_lens) / 160 and a multiple of 4 for the
 * 16-byte stores; frames past a request's count are not written.  Copies the
 * lengths into the workspace through the pinned buffer (sample_lens may be
 * freed when the call returns); asynchronous on `stream`. */
aut_status aut_logmel(const float* audio, int32_t S_max, const int32_t* sample_lens, int32_t B,
                      const void* tables, float* features, int32_t T_max, void* workspace,
                      size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * After the encoder: audio rows into the decoder's embedding sequence
 * ("Audio Encoder Component", cubic.dev wiki, Data Flow and Integration: the
 * audio features are placed at the <|audio_pad|> placeholder positions of the
 * text sequence, not appended).
 * ------------------------------------------------------------------------ */

/* Host only: the positions of the n_ids-long token sequence `ids` (host) that
 * hold pad_id, in order, into rows (host, n_audio entries).  The count must
 * equal n_audio (one placeholder per audio row), else AUT_ERR_INVALID_ARG. */
aut_status aut_audio_rows(const int32_t* ids, int64_t n_ids, int32_t pad_id, int64_t n_audio,
                          int32_t* rows);

/* dst[rows[j]] = audio[j] for j < n_audio: audio device fp32 [n_audio, dim]
 * (e.g. one request's rows of the encoder output), rows device int32
 * [n_audio] (from aut_audio_rows), dst device [dst_rows, dim] of dst_dtype
 * (fp32 copy, or bf16 rounded to nearest even); other rows of dst are not
 * touched, and entries of rows outside [0, dst_rows) are skipped.  dim must be
 * a multiple of 4 and audio/dst 16-byte aligned.  Asynchronous on `stream`. */
aut_status aut_inject_audio(const float* audio, const int32_t* rows, int64_t n_audio, int32_t dim,
                            void* dst, int64_t dst_rows, aut_dtype dst_dtype, void* stream);

/* ------------------------------------------------------------------------
 * MX-fp8 operands (the AUT_FP8 products) as primitives: the conversion the
 * packing and the operand-producing kernels apply, and one product.
 * Format: OCP Microscaling MX-fp8, e4m3 codes (OCP 8-bit floating point) and
 * one E8M0 scale code per 32 consecutive values of a row, scale 2^(code-127),
 * the smallest power of two with no element above 448; elements rounded to
 * nearest even.  Scale layout of an operand with R rows and K columns (K a
 * multiple of 128): rows padded to a multiple of 16; the scale of row r, block
 * kb (columns 32 kb .. 32 kb + 31) is byte
 *   ((r / 16) * (K / 128) + kb / 4) * 64 + (kb % 4) * 16 + r % 16,
 * i.e. per 16 rows and 128 columns the 64 bytes one scaled matrix instruction
 * takes, in lane order.
 * ------------------------------------------------------------------------ */

/* Bytes of the scale array of an operand with `rows` rows and K columns:
 * ceil(rows / 16) * 16 * K / 32.  K must be a positive multiple of 128. */
aut_status aut_mx_scale_bytes(int64_t rows, int32_t K, size_t* bytes);

/* x: device fp32 [rows, K], row-major, 16-byte aligned -> codes: device uint8
 * [rows, K] (16-byte aligned), scales: device, aut_mx_scale_bytes(rows, K)
 * bytes (the padding rows get scale code 0).  |x| must be finite.
 * Asynchronous on `stream`. */
aut_status aut_mx_quantize(const float* x, int64_t rows, int32_t K, uint8_t* codes, uint8_t* scales,
                           void* stream);

/* out: device fp32 [M, N] = A B^T with A = (a_codes [M, K], a_scales) and
 * B = (b_codes [N, K], b_scales) as produced by aut_mx_quantize; products
 * exact, sums in fp32.  K a multiple of 128, N a multiple of 4, codes and out
 * 16-byte aligned.  Asynchronous on `stream`. */
aut_status aut_mx_matmul(const uint8_t* a_codes, const uint8_t* a_scales, int64_t M,
                         const uint8_t* b_codes, const uint8_t* b_scales, int32_t N, int32_t K,
                         float* out, void* stream);

/* ------------------------------------------------------------------------
 * One LayerNorm step on its own: the normalisation in front of qkv, fc1 and
 * the projector (LayerNorm with bias, not RMSNorm: cubic.dev wiki, "Audio
 * Encoder Component", encoder-layer description), with the kernel the
 * forward uses.  Per row of d values: y = (x - mean) / sqrt(var + eps) *
 * gamma + beta, population variance, fp32 statistics (two passes: the mean,
 * then the mean of squared deviations).
 *   x:      device fp32 [rows, d], row-major, 16-byte aligned
 *   gamma,  device fp32 [d] each
 *   beta:
 *   dtype:  AUT_FP32: y is fp32 [rows, d];
 *           AUT_BF16: y is bf16 [rows, d], each value the fp32 result
 *                     rounded to nearest even;
 *           AUT_FP8:  y is e4m3 codes [rows, d] and y_scales holds the scale
 *                     codes (aut_mx_scale_bytes(rows, d) bytes, the MX
 *                     layout above): each 32-value block of a row quantised
 *                     from the fp32 results as aut_mx_quantize would; d a
 *                     multiple of 128.  The scale bytes of the padding rows
 *                     past `rows` are not written.
 * d a multiple of 4, at most 2048; y 8-byte aligned.  The caller owns every
 * buffer.  Returns INVALID_ARG for NULL pointers, misalignment or a
 * negative count, UNSUPPORTED for a d outside these limits.  Asynchronous on
 * `stream`. */
aut_status aut_layernorm(const float* x, int64_t rows, int32_t d, const float* gamma,
                         const float* beta, float eps, aut_dtype dtype, void* y,
                         uint8_t* y_scales, void* stream);

/* ------------------------------------------------------------------------
 * One window-attention step on its own, with the kernel the forward uses:
 * for every window [s, e) of cu_seqlens and every head h, softmax(Q K^T /
 * sqrt(64)) V over the window's own rows only, bidirectional, with no mask
 * inside the window and nothing across windows (m-star API page, module
 * summary and AuTAttention: SDPA per window from cu_seqlens; openarchlab
 * "1A", section 3: is_causal = False).  Head dimension 64, d = 64 heads.
 *   qkv:          device [rows, 3 d] in in_dtype, row-major: q in columns
 *                 [0, d), k in [d, 2d), v in [2d, 3d); head h owns columns
 *                 [64 h, 64 h + 64) of each; 16-byte aligned
 *   cu_seqlens:   device int32 [n_windows + 1], window w = rows
 *                 [cu[w], cu[w + 1]), at most 128 rows each
 *   window_order: device int32 [n_windows], a permutation of the windows:
 *                 the order the kernel takes them in (longest first fills
 *                 the machine best); results do not depend on it
 *   in -> out:    AUT_FP32 -> AUT_FP32; AUT_BF16 -> AUT_BF16 (each value the
 *                 fp32 result rounded to nearest even), AUT_FP32 (those fp32
 *                 results) or AUT_FP8 (e4m3 codes [rows, d] and, in
 *                 out_scales, aut_mx_scale_bytes(rows, d) scale bytes in the
 *                 MX layout above, each 32-value block of a row quantised
 *                 from the fp32 results as aut_mx_quantize would; heads
 *                 even)
 *   out:          device [rows, d] of out_dtype, 16-byte aligned
 * Rows of no window are not written.  A window outside rows [0, rows), longer
 * than 128 rows or named by an order entry outside [0, n_windows) is skipped
 * (its rows are not written).  heads from 1 to 64, rows below 2^31.  The
 * caller owns every buffer.  Returns INVALID_ARG for NULL pointers,
 * misalignment or negative counts, UNSUPPORTED for other dtype pairs, head
 * counts or row counts.  Asynchronous on `stream`. */
aut_status aut_attention(const void* qkv, int64_t rows, int32_t heads, const int32_t* cu_seqlens,
                         const int32_t* window_order, int32_t n_windows, aut_dtype in_dtype,
                         aut_dtype out_dtype, void* out, uint8_t* out_scales, void* stream);

/* Kernel classes for the optional per-launch timing below. */
typedef enum {
  AUT_K_CONV1 = 0,     /* conv1 (+GELU), fp32 vector ALU */
  AUT_K_CONV_GEMM = 1, /* conv2 / conv3 implicit GEMM (+bias, GELU) */
  AUT_K_CONV_OUT = 2,  /* conv_out GEMM (+bias, positions, pack) */
  AUT_K_LAYERNORM = 3, /* LayerNorm rows -> GEMM operand */
  AUT_K_GEMM = 4,      /* qkv / out_proj / fc1 / fc2 / proj1 / proj2 */
  AUT_K_ATTENTION = 5, /* window attention */
  AUT_K_LOGMEL = 6,    /* log-mel front end (DFT + filterbank + log, floor pass) */
  AUT_K_GEMM_FP8 = 7,  /* the AUT_K_GEMM products on MX-fp8 operands */
  AUT_K_COUNT = 8
} aut_kernel_class;

typedef struct {
  int64_t launches;
  double total_ms;  /* summed launch durations from HIP events around each launch */
  double flops;     /* algorithmic flops of those launches (valid work only) */
  double bytes;     /* algorithmic HBM bytes of those launches (each operand once) */
} aut_kernel_stats;

/* Turns per-launch timing on (1) or off (0).  While on, every launch is
 * bracketed by two HIP events recorded on the launch's own stream. */
aut_status aut_profile_enable(int on);

/* Waits for the recorded events, adds their durations into
 * stats[AUT_K_COUNT] (overwritten), and clears the records. */
aut_status aut_profile_collect(aut_kernel_stats* stats);

/* Message describing the last non-OK status returned on this thread. */
const char* aut_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* AUT_H_ */
