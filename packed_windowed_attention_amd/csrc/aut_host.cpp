// Host layer of the AuT encoder library: configuration checks, the plan
// (m-star AuTEncoder.layout), parameter packing, workspace layout, the
// launch sequence of one forward, and optional per-launch event timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "aut_internal.h"

namespace {

thread_local char g_err[1024] = "";

aut_status fail(aut_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

#define HIPCHK(expr)                                                                      \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess) return fail(AUT_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int half_up(int n) { return (n + 1) / 2; }  // Conv2d(k3, s2, p1) output length

// activation element size: fp32, or bf16 (also under AUT_FP8, whose MX-fp8
// operands take one byte plus 1/32 of a scale byte per element and fit in the
// same buffers)
size_t esize(aut_dtype dt) { return dt == AUT_FP32 ? 4 : 2; }

// the arithmetic of everything that is not an MX-fp8 product
aut_dtype base_dtype(aut_dtype dt) { return dt == AUT_FP8 ? AUT_BF16 : dt; }

}  // namespace

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------

struct aut_plan {
  aut_config cfg;
  aut::Geometry geo;
  int32_t B = 0;
  std::vector<int32_t> lens;
  std::vector<int32_t> tokens_per_request;
  std::vector<aut_chunk> chunks;
  std::vector<int32_t> rowmap;   // per packed row: chunk * tokens_per_chunk + j
  std::vector<int32_t> cu;       // n_windows + 1
  std::vector<int32_t> worder;   // windows, longest first (ties by index)
  int64_t total = 0;
  double sum_len2 = 0;           // sum over windows of L^2
};

namespace aut {

Geometry geometry(const aut_config& c) {
  Geometry g;
  g.mel = c.num_mel_bins;
  g.cf = 2 * c.n_window;
  g.h1 = half_up(g.mel);
  g.w1 = half_up(g.cf);
  g.h2 = half_up(g.h1);
  g.w2 = half_up(g.w1);
  g.h3 = half_up(g.h2);
  g.w3 = half_up(g.w2);
  g.C = c.downsample_hidden_size;
  g.d = c.d_model;
  g.H = c.encoder_attention_heads;
  g.hd = g.H > 0 ? g.d / g.H : 0;
  g.F = c.encoder_ffn_dim;
  g.out = c.output_dim;
  g.layers = c.encoder_layers;
  g.chunks_per_window = g.cf > 0 ? c.n_window_infer / g.cf : 0;
  g.window_tokens = g.w3 * g.chunks_per_window;
  return g;
}

// ---------------------------------------------------------------------------
// per-launch timing
// ---------------------------------------------------------------------------

namespace {

struct ProfRecord {
  hipEvent_t start, stop;
  aut_kernel_class cls;
  double flops, bytes;
};

std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_prof;
std::vector<hipEvent_t> g_event_pool;
hipEvent_t g_pending_start = nullptr;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

void prof_begin(hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return;
  g_pending_start = take_event();
  if (g_pending_start) (void)hipEventRecord(g_pending_start, s);
}

void prof_end(hipStream_t s, aut_kernel_class cls, double flops, double bytes) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on || !g_pending_start) return;
  hipEvent_t stop = take_event();
  if (!stop) return;
  (void)hipEventRecord(stop, s);
  g_prof.push_back(ProfRecord{g_pending_start, stop, cls, flops, bytes});
  g_pending_start = nullptr;
}

}  // namespace aut

using aut::Geometry;

// ---------------------------------------------------------------------------
// configuration
// ---------------------------------------------------------------------------

extern "C" aut_status aut_config_default(aut_config* cfg) {
  if (!cfg) return fail(AUT_ERR_INVALID_ARG, "cfg is NULL");
  cfg->d_model = 1024;
  cfg->encoder_layers = 24;
  cfg->encoder_attention_heads = 16;
  cfg->encoder_ffn_dim = 4096;
  cfg->num_mel_bins = 128;
  cfg->n_window = 50;
  cfg->n_window_infer = 800;
  cfg->conv_chunksize = 500;
  cfg->downsample_hidden_size = 480;
  cfg->output_dim = 2048;
  cfg->max_source_positions = 1500;
  cfg->conv_out_bias = 0;
  cfg->ln_eps = 1e-5f;
  cfg->fp8_gemms = AUT_FP8_ALL;
  return AUT_OK;
}

extern "C" aut_status aut_config_check(const aut_config* c) {
  if (!c) return fail(AUT_ERR_INVALID_ARG, "cfg is NULL");
  if (c->encoder_layers < 0 || c->d_model <= 0 || c->encoder_attention_heads <= 0 ||
      c->encoder_ffn_dim <= 0 || c->num_mel_bins <= 0 || c->n_window <= 0 ||
      c->n_window_infer <= 0 || c->conv_chunksize <= 0 || c->downsample_hidden_size <= 0 ||
      c->output_dim <= 0 || c->max_source_positions <= 0)
    return fail(AUT_ERR_INVALID_ARG, "configuration sizes must be positive");
  if (!(c->ln_eps > 0.f)) return fail(AUT_ERR_INVALID_ARG, "ln_eps must be positive");
  if (c->conv_out_bias != 0 && c->conv_out_bias != 1)
    return fail(AUT_ERR_INVALID_ARG, "conv_out_bias must be 0 or 1");
  if (c->fp8_gemms < 0 || c->fp8_gemms > AUT_FP8_ALL)
    return fail(AUT_ERR_INVALID_ARG, "fp8_gemms must be a combination of AUT_FP8_* bits");
  Geometry g = aut::geometry(*c);
  if (c->num_mel_bins != 128) return fail(AUT_ERR_UNSUPPORTED, "num_mel_bins must be 128");
  if (g.cf > 256) return fail(AUT_ERR_UNSUPPORTED, "2 * n_window must be <= 256");
  if (c->n_window_infer % g.cf)
    return fail(AUT_ERR_UNSUPPORTED, "n_window_infer (%d) must be a multiple of 2 * n_window (%d)",
                c->n_window_infer, g.cf);
  if (g.window_tokens > 128)
    return fail(AUT_ERR_UNSUPPORTED, "tokens per window (%d) must be <= 128", g.window_tokens);
  if (c->d_model != 64 * c->encoder_attention_heads)
    return fail(AUT_ERR_UNSUPPORTED, "head_dim must be 64 (d_model = 64 * heads)");
  if (c->d_model > 2048) return fail(AUT_ERR_UNSUPPORTED, "d_model must be <= 2048");
  if (g.C % 8 || g.C > 1024)
    return fail(AUT_ERR_UNSUPPORTED, "downsample_hidden_size must be a multiple of 8, <= 1024");
  if (c->encoder_ffn_dim % 8 || c->output_dim % 8)
    return fail(AUT_ERR_UNSUPPORTED, "encoder_ffn_dim and output_dim must be multiples of 8");
  if (c->max_source_positions < g.w3)
    return fail(AUT_ERR_UNSUPPORTED, "max_source_positions must cover the tokens of one chunk");
  if (c->conv_chunksize > 8192) return fail(AUT_ERR_UNSUPPORTED, "conv_chunksize must be <= 8192");
  return AUT_OK;
}

// ---------------------------------------------------------------------------
// plan
// ---------------------------------------------------------------------------

static const int64_t kMaxRows = 8000000;

extern "C" aut_status aut_plan(const aut_config* cfg, const int32_t* feature_lens, int32_t B,
                               aut_plan_t** out) {
  if (!out) return fail(AUT_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  aut_status st = aut_config_check(cfg);
  if (st != AUT_OK) return st;
  if (B < 0) return fail(AUT_ERR_INVALID_ARG, "B must be >= 0");
  if (B > 0 && !feature_lens) return fail(AUT_ERR_INVALID_ARG, "feature_lens is NULL");
  for (int b = 0; b < B; ++b)
    if (feature_lens[b] < 0) return fail(AUT_ERR_INVALID_ARG, "feature_lens[%d] = %d < 0", b, feature_lens[b]);

  aut_plan_t* p = new (std::nothrow) aut_plan_t();
  if (!p) return fail(AUT_ERR_INVALID_ARG, "out of host memory");
  p->cfg = *cfg;
  p->geo = aut::geometry(*cfg);
  const Geometry& g = p->geo;
  p->B = B;
  p->lens.assign(feature_lens, feature_lens + B);
  p->cu.push_back(0);
  int64_t row = 0;
  for (int b = 0; b < B; ++b) {
    const int L = feature_lens[b];
    const int nch = (L + g.cf - 1) / g.cf;
    int64_t treq = 0;
    for (int c = 0; c < nch; ++c) {
      const int vf = std::min(g.cf, L - c * g.cf);
      // tokens kept: the length of three stride-2 halvings of the valid frames
      const int vt = half_up(half_up(half_up(vf)));
      aut_chunk ch{b, c * g.cf, vf, vt, (int32_t)row};
      const int32_t cid = (int32_t)p->chunks.size();
      p->chunks.push_back(ch);
      for (int j = 0; j < vt; ++j) p->rowmap.push_back(cid * g.w3 + j);
      row += vt;
      treq += vt;
      if (row > kMaxRows) {
        delete p;
        return fail(AUT_ERR_UNSUPPORTED, "more than %lld tokens in one batch", (long long)kMaxRows);
      }
    }
    p->tokens_per_request.push_back((int32_t)treq);
    // windows: full windows of window_tokens, then the remainder
    for (int64_t s = 0; s < treq; s += g.window_tokens) {
      const int64_t len = std::min<int64_t>(g.window_tokens, treq - s);
      p->cu.push_back(p->cu.back() + (int32_t)len);
      p->sum_len2 += (double)len * (double)len;
    }
  }
  p->total = row;
  const int nw = (int)p->cu.size() - 1;
  p->worder.resize(nw);
  for (int w = 0; w < nw; ++w) p->worder[w] = w;
  std::stable_sort(p->worder.begin(), p->worder.end(), [&](int a, int b) {
    return (p->cu[a + 1] - p->cu[a]) > (p->cu[b + 1] - p->cu[b]);
  });
  *out = p;
  return AUT_OK;
}

extern "C" aut_status aut_plan_counts(const aut_plan_t* plan, int64_t* total_tokens,
                                      int32_t* n_windows, int32_t* n_chunks) {
  if (!plan) return fail(AUT_ERR_INVALID_ARG, "plan is NULL");
  if (total_tokens) *total_tokens = plan->total;
  if (n_windows) *n_windows = (int32_t)plan->cu.size() - 1;
  if (n_chunks) *n_chunks = (int32_t)plan->chunks.size();
  return AUT_OK;
}

extern "C" aut_status aut_plan_copy(const aut_plan_t* plan, int32_t* tokens_per_request,
                                    int32_t* cu_seqlens, aut_chunk* chunks) {
  if (!plan) return fail(AUT_ERR_INVALID_ARG, "plan is NULL");
  if (tokens_per_request && plan->B)
    memcpy(tokens_per_request, plan->tokens_per_request.data(), sizeof(int32_t) * plan->B);
  if (cu_seqlens) memcpy(cu_seqlens, plan->cu.data(), sizeof(int32_t) * plan->cu.size());
  if (chunks && !plan->chunks.empty())
    memcpy(chunks, plan->chunks.data(), sizeof(aut_chunk) * plan->chunks.size());
  return AUT_OK;
}

extern "C" void aut_plan_destroy(aut_plan_t* plan) { delete plan; }

// ---------------------------------------------------------------------------
// packed parameters
// ---------------------------------------------------------------------------

namespace {

// A GEMM weight [rows, cols] is bf16/fp32, or under AUT_FP8 with its class
// bit set, MX-fp8 codes at *_w and scales at *_s.
struct LayerOff {
  size_t ln1_g, ln1_b, qkv_w, qkv_b, o_w, o_b, ln2_g, ln2_b, fc1_w, fc1_b, fc2_w, fc2_b;
  size_t qkv_s, o_s, fc1_s, fc2_s;
};

struct PackLayout {
  size_t conv1_w, conv1_b, conv2_w, conv2_b, conv3_w, conv3_b, conv_out_w, conv_out_b, pe;
  size_t conv2_s, conv3_s, conv_out_s;  // AUT_FP8_CONV: MX scales of the conv-stem weights
  std::vector<LayerOff> layers;
  size_t ln_post_g, ln_post_b, proj1_w, proj1_b, proj2_w, proj2_b;
  size_t proj1_s, proj2_s;
  size_t total;
};

// channels per pixel of the MX-fp8 conv-stem activations: a multiple of 128,
// so that a 128-code k step of the implicit convolution stays within one tap
int conv_cp(const Geometry& g) { return (g.C + 127) / 128 * 128; }

// the AUT_FP8_* bits in force for a dtype
int fp8_mask(const aut_config& c, aut_dtype dt) { return dt == AUT_FP8 ? c.fp8_gemms : 0; }

PackLayout pack_layout(const Geometry& g, aut_dtype dt, int f8) {
  PackLayout L;
  size_t off = 0;
  const size_t es = esize(dt);
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  // a GEMM weight: codes and scales when its class runs on MX-fp8
  auto wmat = [&](size_t& w, size_t& sc, size_t rows, size_t cols, int bit) {
    if (f8 & bit) {
      w = take(rows * cols);
      sc = take(aut::mx_scale_bytes((long)rows, (int)cols));
    } else {
      w = take(rows * cols * es);
      sc = 0;
    }
  };
  const size_t C = g.C, d = g.d, F = g.F, O = g.out;
  L.conv1_w = take(C * 9 * 4);
  L.conv1_b = take(C * 4);
  L.conv2_s = L.conv3_s = L.conv_out_s = 0;
  if (f8 & AUT_FP8_CONV) {
    const size_t cp = conv_cp(g);
    L.conv2_w = take(C * 9 * cp);
    L.conv2_s = take(aut::mx_scale_bytes((long)C, (int)(9 * cp)));
    L.conv2_b = take(C * 4);
    L.conv3_w = take(C * 9 * cp);
    L.conv3_s = take(aut::mx_scale_bytes((long)C, (int)(9 * cp)));
    L.conv3_b = take(C * 4);
    L.conv_out_w = take(d * g.h3 * cp);
    L.conv_out_s = take(aut::mx_scale_bytes((long)d, (int)(g.h3 * cp)));
  } else {
    L.conv2_w = take(C * 9 * C * es);
    L.conv2_b = take(C * 4);
    L.conv3_w = take(C * 9 * C * es);
    L.conv3_b = take(C * 4);
    L.conv_out_w = take(d * g.h3 * C * es);
  }
  L.conv_out_b = take(d * 4);
  L.pe = take((size_t)g.w3 * d * 4);
  L.layers.resize(g.layers);
  for (int i = 0; i < g.layers; ++i) {
    LayerOff& l = L.layers[i];
    l.ln1_g = take(d * 4);
    l.ln1_b = take(d * 4);
    wmat(l.qkv_w, l.qkv_s, 3 * d, d, AUT_FP8_QKV);
    l.qkv_b = take(3 * d * 4);
    wmat(l.o_w, l.o_s, d, d, AUT_FP8_OUT);
    l.o_b = take(d * 4);
    l.ln2_g = take(d * 4);
    l.ln2_b = take(d * 4);
    wmat(l.fc1_w, l.fc1_s, F, d, AUT_FP8_FC1);
    l.fc1_b = take(F * 4);
    wmat(l.fc2_w, l.fc2_s, d, F, AUT_FP8_FC2);
    l.fc2_b = take(d * 4);
  }
  L.ln_post_g = take(d * 4);
  L.ln_post_b = take(d * 4);
  wmat(L.proj1_w, L.proj1_s, d, d, AUT_FP8_PROJ);
  L.proj1_b = take(d * 4);
  wmat(L.proj2_w, L.proj2_s, O, d, AUT_FP8_PROJ);
  L.proj2_b = take(O * 4);
  L.total = off;
  return L;
}

bool valid_dtype(aut_dtype dt) { return dt == AUT_FP32 || dt == AUT_BF16 || dt == AUT_FP8; }

// what the MX-fp8 products need of the sizes: k steps of 128 for every
// product whose operand is d_model or encoder_ffn_dim wide
aut_status check_dtype(const aut_config& c, aut_dtype dt) {
  if (!valid_dtype(dt)) return fail(AUT_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (dt == AUT_FP8 && (c.d_model % 128 || c.encoder_ffn_dim % 128))
    return fail(AUT_ERR_UNSUPPORTED, "AUT_FP8 needs d_model and encoder_ffn_dim multiples of 128");
  if (dt == AUT_FP8 && (c.fp8_gemms & AUT_FP8_CONV) && c.downsample_hidden_size % 32)
    return fail(AUT_ERR_UNSUPPORTED, "AUT_FP8_CONV needs downsample_hidden_size a multiple of 32");
  return AUT_OK;
}

}  // namespace

extern "C" aut_status aut_weights_bytes(const aut_config* cfg, aut_dtype dtype, size_t* bytes) {
  aut_status st = aut_config_check(cfg);
  if (st != AUT_OK) return st;
  if ((st = check_dtype(*cfg, dtype)) != AUT_OK) return st;
  if (!bytes) return fail(AUT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = pack_layout(aut::geometry(*cfg), dtype, fp8_mask(*cfg, dtype)).total;
  return AUT_OK;
}

extern "C" aut_status aut_weights_pack(const aut_config* cfg, const aut_weight_ptrs* w,
                                       aut_dtype dt, void* dst, size_t dst_bytes, void* stream) {
  aut_status st = aut_config_check(cfg);
  if (st != AUT_OK) return st;
  if ((st = check_dtype(*cfg, dt)) != AUT_OK) return st;
  if (!w) return fail(AUT_ERR_INVALID_ARG, "weights is NULL");
  if (!dst) return fail(AUT_ERR_INVALID_ARG, "dst is NULL");
  const Geometry g = aut::geometry(*cfg);
  const int f8 = fp8_mask(*cfg, dt);
  const PackLayout L = pack_layout(g, dt, f8);
  if (dst_bytes < L.total)
    return fail(AUT_ERR_WORKSPACE_TOO_SMALL, "packed buffer has %zu bytes, needs %zu", dst_bytes,
                L.total);

  // every parameter must be present before anything is launched
#define NEED(ptr, name)                                                       \
  do {                                                                        \
    if (!(ptr)) return fail(AUT_ERR_MISSING_WEIGHT, "missing parameter %s", name); \
  } while (0)
  NEED(w->conv1_w, "conv1_w"); NEED(w->conv1_b, "conv1_b");
  NEED(w->conv2_w, "conv2_w"); NEED(w->conv2_b, "conv2_b");
  NEED(w->conv3_w, "conv3_w"); NEED(w->conv3_b, "conv3_b");
  NEED(w->conv_out_w, "conv_out_w");
  if (cfg->conv_out_bias) NEED(w->conv_out_b, "conv_out_b");
  NEED(w->ln_post_g, "ln_post_g"); NEED(w->ln_post_b, "ln_post_b");
  NEED(w->proj1_w, "proj1_w"); NEED(w->proj1_b, "proj1_b");
  NEED(w->proj2_w, "proj2_w"); NEED(w->proj2_b, "proj2_b");
  if (g.layers > 0) {
    NEED(w->ln1_g, "ln1_g"); NEED(w->ln1_b, "ln1_b"); NEED(w->qkv_w, "qkv_w"); NEED(w->qkv_b, "qkv_b");
    NEED(w->o_w, "o_w"); NEED(w->o_b, "o_b"); NEED(w->ln2_g, "ln2_g"); NEED(w->ln2_b, "ln2_b");
    NEED(w->fc1_w, "fc1_w"); NEED(w->fc1_b, "fc1_b"); NEED(w->fc2_w, "fc2_w"); NEED(w->fc2_b, "fc2_b");
  }
  char nm[64];
  for (int i = 0; i < g.layers; ++i) {
#define NEEDL(f)                                                                           \
  do {                                                                                     \
    if (!w->f[i]) {                                                                        \
      snprintf(nm, sizeof(nm), "layers.%d.%s", i, #f);                                     \
      return fail(AUT_ERR_MISSING_WEIGHT, "missing parameter %s", nm);                     \
    }                                                                                      \
  } while (0)
    NEEDL(ln1_g); NEEDL(ln1_b); NEEDL(qkv_w); NEEDL(qkv_b); NEEDL(o_w); NEEDL(o_b);
    NEEDL(ln2_g); NEEDL(ln2_b); NEEDL(fc1_w); NEEDL(fc1_b); NEEDL(fc2_w); NEEDL(fc2_b);
#undef NEEDL
  }
#undef NEED

  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)dst;
  const aut_dtype bdt = base_dtype(dt);
  auto vec = [&](const float* src, size_t off, int n) {
    return aut::launch_pack(src, base + off, AUT_FP32, aut::PACK_CAST, 1, n, 0, 0, s);
  };
  auto mat = [&](const float* src, size_t off, int rows, int cols) {
    return aut::launch_pack(src, base + off, bdt, aut::PACK_CAST, rows, cols, 0, 0, s);
  };
  // a GEMM weight, MX-fp8 when its class bit is set
  auto gmat = [&](const float* src, size_t off, size_t off_s, int rows, int cols, int bit) {
    if (f8 & bit)
      return aut::launch_mx_quantize(src, cols, rows, cols, (uint8_t*)(base + off),
                                     (uint8_t*)(base + off_s), s);
    return mat(src, off, rows, cols);
  };
  const int C = g.C, d = g.d, F = g.F;
  HIPCHK(aut::launch_pack(w->conv1_w, base + L.conv1_w, AUT_FP32, aut::PACK_CAST, C, 9, 0, 0, s));
  HIPCHK(vec(w->conv1_b, L.conv1_b, C));
  if (f8 & AUT_FP8_CONV) {
    const int cp = conv_cp(g);
    HIPCHK(aut::launch_mx_quantize_gather(w->conv2_w, aut::PACK_CONV, C, C, cp, 1,
                                          (uint8_t*)(base + L.conv2_w), (uint8_t*)(base + L.conv2_s), s));
    HIPCHK(aut::launch_mx_quantize_gather(w->conv3_w, aut::PACK_CONV, C, C, cp, 1,
                                          (uint8_t*)(base + L.conv3_w), (uint8_t*)(base + L.conv3_s), s));
    HIPCHK(aut::launch_mx_quantize_gather(w->conv_out_w, aut::PACK_CONV_OUT, d, C, cp, g.h3,
                                          (uint8_t*)(base + L.conv_out_w),
                                          (uint8_t*)(base + L.conv_out_s), s));
  } else {
    HIPCHK(aut::launch_pack(w->conv2_w, base + L.conv2_w, bdt, aut::PACK_CONV, C, 9 * C, C, 0, s));
    HIPCHK(aut::launch_pack(w->conv3_w, base + L.conv3_w, bdt, aut::PACK_CONV, C, 9 * C, C, 0, s));
    HIPCHK(aut::launch_pack(w->conv_out_w, base + L.conv_out_w, bdt, aut::PACK_CONV_OUT, d,
                            g.h3 * C, C, g.h3, s));
  }
  HIPCHK(vec(w->conv2_b, L.conv2_b, C));
  HIPCHK(vec(w->conv3_b, L.conv3_b, C));
  if (cfg->conv_out_bias) HIPCHK(vec(w->conv_out_b, L.conv_out_b, d));
  HIPCHK(aut::launch_pe_table((float*)(base + L.pe), g.w3, d, s));
  for (int i = 0; i < g.layers; ++i) {
    const LayerOff& l = L.layers[i];
    HIPCHK(vec(w->ln1_g[i], l.ln1_g, d));
    HIPCHK(vec(w->ln1_b[i], l.ln1_b, d));
    HIPCHK(gmat(w->qkv_w[i], l.qkv_w, l.qkv_s, 3 * d, d, AUT_FP8_QKV));
    HIPCHK(vec(w->qkv_b[i], l.qkv_b, 3 * d));
    HIPCHK(gmat(w->o_w[i], l.o_w, l.o_s, d, d, AUT_FP8_OUT));
    HIPCHK(vec(w->o_b[i], l.o_b, d));
    HIPCHK(vec(w->ln2_g[i], l.ln2_g, d));
    HIPCHK(vec(w->ln2_b[i], l.ln2_b, d));
    HIPCHK(gmat(w->fc1_w[i], l.fc1_w, l.fc1_s, F, d, AUT_FP8_FC1));
    HIPCHK(vec(w->fc1_b[i], l.fc1_b, F));
    HIPCHK(gmat(w->fc2_w[i], l.fc2_w, l.fc2_s, d, F, AUT_FP8_FC2));
    HIPCHK(vec(w->fc2_b[i], l.fc2_b, d));
  }
  HIPCHK(vec(w->ln_post_g, L.ln_post_g, d));
  HIPCHK(vec(w->ln_post_b, L.ln_post_b, d));
  HIPCHK(gmat(w->proj1_w, L.proj1_w, L.proj1_s, d, d, AUT_FP8_PROJ));
  HIPCHK(vec(w->proj1_b, L.proj1_b, d));
  HIPCHK(gmat(w->proj2_w, L.proj2_w, L.proj2_s, g.out, d, AUT_FP8_PROJ));
  HIPCHK(vec(w->proj2_b, L.proj2_b, g.out));
  return AUT_OK;
}

// ---------------------------------------------------------------------------
// workspace
// ---------------------------------------------------------------------------

namespace {

struct WsLayout {
  size_t chunks, rowmap, cu, worder;
  size_t a1, a2, a3;
  size_t a1_s, a2_s, a3_s;  // AUT_FP8_CONV: MX scales of the conv-stem activations
  // a3 holds every chunk's conv3 output, so that conv_out runs once over all
  // tokens (a full grid) rather than once per conv batch; false when that
  // buffer would pass the 2 GiB of the GEMM's 32-bit gather offsets
  bool a3_all;
  size_t x, xn, qkv, o, h;
  size_t xn_s, o_s, h_s;  // AUT_FP8: MX scales of xn, o and h
  size_t total;
  int nb;  // chunks per conv-stem batch
};

// Chunks per conv-stem batch, at most cap.  A conv GEMM's grid runs in
// rounds of one tile per CU, so a batch whose tile count just passes a
// multiple of the CU count pays a nearly empty last round.  Among batch sizes
// from cap down to cap / 2, at most 512 of them (batches of that size, the
// rest in a last one), this
// takes the one with the least estimated conv2 + conv3 time, ties to the
// larger size.  Results do not depend on it: every output pixel sums its k
// steps in the same order in any batch.
int conv_batch_chunks(int nch, int cap, const Geometry& g, bool f8) {
  if (nch <= 0 || cap <= 1) return cap;
  auto t = [&](int n) {
    return aut::gemm_conv_time_model(n * g.h2 * g.w2, g.C, f8) +
           aut::gemm_conv_time_model(n * g.h3 * g.w3, g.C, f8);
  };
  int best = cap;
  double best_t = 0.0;
  for (int n = cap; n >= std::max(std::max(1, cap / 2), cap - 511); --n) {
    const int full = nch / n, rest = nch - full * n;
    const double tn = full * t(n) + (rest ? t(rest) : 0.0);
    if (n == cap || tn < best_t * (1.0 - 1e-9)) {
      best = n;
      best_t = tn;
    }
  }
  return best;
}

WsLayout ws_layout(const aut_plan_t& p, aut_dtype dt) {
  const Geometry& g = p.geo;
  WsLayout W;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  const size_t es = esize(dt);
  const size_t T = (size_t)p.total;
  const size_t nch = p.chunks.size();
  const size_t nw = p.cu.size() - 1;
  // chunks per conv-stem batch: conv_chunksize, also kept small enough that
  // the batch's conv1 output stays below 2 GiB (32-bit buffer offsets); an
  // MX-fp8 stem stores cp one-byte codes per pixel
  const bool f8c = dt == AUT_FP8 && (p.cfg.fp8_gemms & AUT_FP8_CONV);
  const size_t cs = f8c ? std::max<size_t>(g.C * es, (size_t)conv_cp(g)) : g.C * es;
  const size_t per_chunk = (size_t)g.h1 * g.w1 * cs;
  const size_t max_nb = std::max<size_t>(1, ((size_t)1 << 31) / per_chunk - 1);
  const size_t cap = std::min<size_t>(std::min<size_t>((size_t)p.cfg.conv_chunksize, nch), max_nb);
  W.nb = dt != AUT_FP32 ? conv_batch_chunks((int)nch, (int)cap, g, f8c) : (int)cap;
  // the batch buffers hold cap chunks, not the chosen W.nb <= cap: cap never
  // shrinks as the plan grows, so a workspace sized for a plan covers every
  // plan with fewer chunks (a stream's steps use the whole request's size)
  const size_t nb = cap;
  W.chunks = take(nch * sizeof(aut_chunk));
  W.rowmap = take(T * 4);
  W.cu = take((nw + 1) * 4);
  W.worder = take(nw * 4);
  W.a3_all = nch * g.h3 * g.w3 * cs < ((size_t)1 << 31);
  const size_t n3 = W.a3_all ? nch : nb;  // chunks held in a3
  W.a1 = take(nb * g.h1 * g.w1 * cs);
  W.a2 = take(nb * g.h2 * g.w2 * cs);
  W.a3 = take(n3 * g.h3 * g.w3 * cs);
  W.a1_s = W.a2_s = W.a3_s = 0;
  if (f8c) {
    const size_t spp = (size_t)conv_cp(g) / 32;  // scale bytes per pixel
    W.a1_s = take(nb * g.h1 * g.w1 * spp);
    W.a2_s = take(nb * g.h2 * g.w2 * spp);
    W.a3_s = take(n3 * g.h3 * g.w3 * spp);
  }
  W.x = take(T * g.d * 4);
  W.xn = take(T * g.d * es);
  W.qkv = take(T * 3 * g.d * es);
  W.o = take(T * g.d * es);
  W.h = take(T * std::max(g.F, g.d) * es);
  W.xn_s = W.o_s = W.h_s = 0;
  if (dt == AUT_FP8 && T > 0) {
    W.xn_s = take(aut::mx_scale_bytes((long)T, g.d));
    W.o_s = take(aut::mx_scale_bytes((long)T, g.d));
    W.h_s = take(aut::mx_scale_bytes((long)T, std::max(g.F, g.d)));
  }
  W.total = off;
  return W;
}

aut_status check_common(const aut_config* cfg, const aut_plan_t* plan, aut_dtype dt,
                        const void* packed, void* ws, size_t ws_bytes, WsLayout* W) {
  aut_status st = aut_config_check(cfg);
  if (st != AUT_OK) return st;
  if (!plan) return fail(AUT_ERR_INVALID_ARG, "plan is NULL");
  if ((st = check_dtype(*cfg, dt)) != AUT_OK) return st;
  if (memcmp(cfg, &plan->cfg, sizeof(aut_config)) != 0)
    return fail(AUT_ERR_INVALID_ARG, "plan was made for a different configuration");
  *W = ws_layout(*plan, dt);
  if (plan->total > 0) {
    if (!packed) return fail(AUT_ERR_MISSING_WEIGHT, "packed parameters are NULL");
    if (!ws) return fail(AUT_ERR_INVALID_ARG, "workspace is NULL");
  }
  if (plan->total > 0 && ws_bytes < W->total)
    return fail(AUT_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws_bytes,
                W->total);
  return AUT_OK;
}

}  // namespace

extern "C" aut_status aut_workspace_bytes(const aut_config* cfg, const aut_plan_t* plan,
                                          aut_dtype dtype, size_t* bytes) {
  aut_status st = aut_config_check(cfg);
  if (st != AUT_OK) return st;
  if (!plan) return fail(AUT_ERR_INVALID_ARG, "plan is NULL");
  if ((st = check_dtype(*cfg, dtype)) != AUT_OK) return st;
  if (!bytes) return fail(AUT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = ws_layout(*plan, dtype).total;
  return AUT_OK;
}

namespace {

// Pinned staging of plan uploads, one buffer per device.  A copy from
// pageable host memory makes the calling thread wait until the stream has
// drained (the runtime stages it synchronously), which leaves the GPU idle
// between forwards; from pinned memory the copy is queued like a kernel.  The
// event marks the end of the last copy out of the buffer: the host waits for
// it before writing the buffer again (in steady state it has long passed).
struct PlanStaging {
  char* host = nullptr;
  size_t cap = 0;
  hipEvent_t done = nullptr;
};
std::mutex g_stage_mu;
std::vector<PlanStaging> g_stage;

// Host data -> device `dst` (bytes) through the device's pinned staging
// buffer: `fill` writes the image into the buffer, then one queued copy.
template <typename Fill>
aut_status upload_pinned(void* dst, size_t bytes, hipStream_t s, Fill fill) {
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_stage_mu);
  if ((int)g_stage.size() <= dev) g_stage.resize(dev + 1);
  PlanStaging& st = g_stage[dev];
  if (st.done) HIPCHK(hipEventSynchronize(st.done));
  else HIPCHK(hipEventCreateWithFlags(&st.done, hipEventDisableTiming));
  if (st.cap < bytes) {
    if (st.host) HIPCHK(hipHostFree(st.host));
    st.host = nullptr;
    st.cap = 0;
    const size_t cap = std::max<size_t>(align256(bytes + bytes / 4), (size_t)1 << 20);
    HIPCHK(hipHostMalloc((void**)&st.host, cap, hipHostMallocDefault));
    st.cap = cap;
  }
  fill(st.host);
  HIPCHK(hipMemcpyAsync(dst, st.host, bytes, hipMemcpyHostToDevice, s));
  HIPCHK(hipEventRecord(st.done, s));
  return AUT_OK;
}

}  // namespace

extern "C" aut_status aut_plan_upload(const aut_plan_t* plan, void* ws, size_t ws_bytes,
                                      void* stream) {
  if (!plan) return fail(AUT_ERR_INVALID_ARG, "plan is NULL");
  const WsLayout W = ws_layout(*plan, AUT_FP32);  // table offsets do not depend on dtype
  const size_t need = W.worder + plan->worder.size() * 4;
  if (plan->total == 0) return AUT_OK;
  if (!ws) return fail(AUT_ERR_INVALID_ARG, "workspace is NULL");
  if (ws_bytes < need) return fail(AUT_ERR_WORKSPACE_TOO_SMALL, "workspace too small for the plan");
  // the four tables are consecutive pieces of the workspace: one image, one copy
  return upload_pinned((char*)ws + W.chunks, need - W.chunks, (hipStream_t)stream, [&](char* h) {
    memcpy(h, plan->chunks.data(), plan->chunks.size() * sizeof(aut_chunk));
    memcpy(h + (W.rowmap - W.chunks), plan->rowmap.data(), plan->rowmap.size() * 4);
    memcpy(h + (W.cu - W.chunks), plan->cu.data(), plan->cu.size() * 4);
    memcpy(h + (W.worder - W.chunks), plan->worder.data(), plan->worder.size() * 4);
  });
}

// ---------------------------------------------------------------------------
// the forward pass
// ---------------------------------------------------------------------------

namespace {

struct Ctx {
  const aut_plan_t* p;
  const Geometry* g;
  aut_dtype dt;  // arithmetic outside the MX-fp8 products (bf16 under AUT_FP8)
  const PackLayout* P;
  const WsLayout* W;
  const char* pk;  // packed parameters
  char* ws;        // workspace
  hipStream_t s;
  int f8;          // AUT_FP8_* bits of the products on MX-fp8 operands
};

template <typename X>
const X* pk_at(const Ctx& c, size_t off) { return reinterpret_cast<const X*>(c.pk + off); }

aut_status gemm(const Ctx& c, aut_kernel_class cls, const aut::GemmArgs& a, int amode, int epi,
                double bytes) {
  aut::prof_begin(c.s);
  hipError_t e = aut::launch_gemm(a, amode, epi, c.dt, c.s);
  if (e != hipSuccess) return fail(AUT_ERR_HIP, "gemm launch failed: %s", hipGetErrorString(e));
  aut::prof_end(c.s, cls, 2.0 * a.M * (double)a.N * a.K, bytes);
  return AUT_OK;
}

aut_status gemm_f8(const Ctx& c, aut_kernel_class cls, const aut::GemmArgs& a, int amode, int epi,
                   double bytes) {
  aut::prof_begin(c.s);
  hipError_t e = aut::launch_gemm_f8(a, amode, epi, c.s);
  if (e != hipSuccess) return fail(AUT_ERR_HIP, "fp8 gemm launch failed: %s", hipGetErrorString(e));
  aut::prof_end(c.s, cls, 2.0 * a.M * (double)a.N * a.K, bytes);
  return AUT_OK;
}

aut::GemmArgs plain_args(const void* A, const void* B, int M, int N, int K, const float* bias,
                         void* out, long ldo) {
  aut::GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.A = A; a.lda = K; a.B = B; a.ldb = K;
  a.M = M; a.N = N; a.K = K;
  a.bias = bias; a.out = out; a.ldo = ldo;
  return a;
}

// frontend: features -> hidden [T, d] fp32.  Under AUT_FP8_CONV the stem's
// activations are MX-fp8 codes, cp channels per pixel (zero past C), with
// row-major scales per pixel, and conv2, conv3 and conv_out run on them.
aut_status run_frontend(const Ctx& c, const float* feat, int T_max, float* hidden) {
  const aut_plan_t& p = *c.p;
  const Geometry& g = *c.g;
  const WsLayout& W = *c.W;
  const PackLayout& P = *c.P;
  const size_t es = esize(c.dt);
  const bool f8 = c.f8 & AUT_FP8_CONV;
  const int cp = conv_cp(g);
  const size_t cs = f8 ? (size_t)cp : (size_t)g.C * es;  // bytes per pixel of the stem activations
  const int nch = (int)p.chunks.size();
  const int* d_chunks = (const int*)(c.ws + W.chunks);
  const int* d_rowmap = (const int*)(c.ws + W.rowmap);
  // conv_out + positions: tokens [r0, r1), whose conv3 rows are chunks
  // [first, first + count) of a3
  auto conv_out = [&](int r0, int r1, int first, int count) -> aut_status {
    if (r1 <= r0) return AUT_OK;
    aut::GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.A = c.ws + W.a3;
    a.B = c.pk + P.conv_out_w;
    a.M = r1 - r0;
    a.N = g.d;
    a.rowmap = d_rowmap + r0;
    a.rowmap_base = first * g.w3;
    a.tpc = g.w3;
    a.bias = p.cfg.conv_out_bias ? pk_at<float>(c, P.conv_out_b) : nullptr;
    a.out = hidden + (size_t)r0 * g.d;
    a.ldo = g.d;
    a.pe = pk_at<float>(c, P.pe);
    if (f8) {
      a.lda = (long)g.h3 * cp;
      a.ldb = (long)g.h3 * cp;
      a.K = g.h3 * cp;
      a.a_bytes = (size_t)count * g.w3 * g.h3 * cp;
      a.a_scale = (const uint8_t*)(c.ws + W.a3_s);
      a.a_scale_ld = g.h3 * cp / 32;
      a.a_scale_bytes = (size_t)count * g.w3 * g.h3 * (cp / 32);
      a.b_scale = (const uint8_t*)(c.pk + P.conv_out_s);
      const double bytes = ((double)a.M * a.K + (double)g.d * a.K) * (1.0 + 1.0 / 32) +
                           (double)a.M * g.d * 4;
      return gemm_f8(c, AUT_K_CONV_OUT, a, aut::A_ROWMAP, aut::EPI_PE, bytes);
    }
    a.lda = (long)g.h3 * g.C;
    a.ldb = (long)g.h3 * g.C;
    a.K = g.h3 * g.C;
    a.a_bytes = (size_t)count * g.w3 * g.h3 * g.C * es;
    const double bytes = ((double)a.M * a.K + (double)g.d * a.K) * es + (double)a.M * g.d * 4;
    return gemm(c, AUT_K_CONV_OUT, a, aut::A_ROWMAP, aut::EPI_PE, bytes);
  };
  for (int c0 = 0; c0 < nch; c0 += W.nb) {
    const int n = std::min(W.nb, nch - c0);
    // conv1 + GELU
    aut::prof_begin(c.s);
    hipError_t e = aut::launch_conv1(feat, T_max, d_chunks, c0, n, pk_at<float>(c, P.conv1_w),
                                     pk_at<float>(c, P.conv1_b), c.ws + W.a1, f8 ? AUT_FP8 : c.dt,
                                     g, c.s, f8 ? (uint8_t*)(c.ws + W.a1_s) : nullptr, cp);
    if (e != hipSuccess) return fail(AUT_ERR_HIP, "conv1 launch failed: %s", hipGetErrorString(e));
    aut::prof_end(c.s, AUT_K_CONV1, 2.0 * 9 * g.C * (double)g.h1 * g.w1 * n,
                  (double)n * g.mel * g.cf * 4 + (double)n * g.h1 * g.w1 * cs);
    // conv2, conv3: implicit GEMMs over the whole (padded) chunks
    for (int layer = 2; layer <= 3; ++layer) {
      aut::GemmArgs a;
      memset(&a, 0, sizeof(a));
      const bool l2 = layer == 2;
      a.A = c.ws + (l2 ? W.a1 : W.a2);
      a.B = c.pk + (l2 ? P.conv2_w : P.conv3_w);
      a.hin = l2 ? g.h1 : g.h2;
      a.win = l2 ? g.w1 : g.w2;
      a.hout = l2 ? g.h2 : g.h3;
      a.wout = l2 ? g.w2 : g.w3;
      a.xmajor = l2 ? 0 : 1;  // conv3 output stored [chunk][x][y][c] for the token flatten
      a.M = n * a.hout * a.wout;
      a.N = g.C;
      a.bias = pk_at<float>(c, l2 ? P.conv2_b : P.conv3_b);
      // conv3 writes at the batch's chunk offset when a3 holds every chunk
      const size_t a3_first = W.a3_all ? (size_t)c0 * g.h3 * g.w3 : 0;  // pixel offset
      a.out = c.ws + (l2 ? W.a2 : W.a3 + a3_first * cs);
      aut_status st;
      if (f8) {
        a.cin = cp;
        a.K = 9 * cp;
        a.ldb = 9 * cp;
        a.a_bytes = (size_t)n * a.hin * a.win * cp;
        a.a_scale = (const uint8_t*)(c.ws + (l2 ? W.a1_s : W.a2_s));
        a.a_scale_ld = cp / 32;
        a.a_scale_bytes = (size_t)n * a.hin * a.win * (cp / 32);
        a.b_scale = (const uint8_t*)(c.pk + (l2 ? P.conv2_s : P.conv3_s));
        a.ldo = cp;
        a.n_store = cp;
        a.out_scale = (uint8_t*)(c.ws + (l2 ? W.a2_s : W.a3_s + a3_first * (cp / 32)));
        a.out_scale_rowmajor = 1;
        const double bytes = ((double)n * a.hin * a.win + (double)a.M) * cp * (1.0 + 1.0 / 32) +
                             (double)g.C * a.K * (1.0 + 1.0 / 32);
        st = gemm_f8(c, AUT_K_CONV_GEMM, a, aut::A_CONV, aut::EPI_GELU_MX, bytes);
      } else {
        a.cin = g.C;
        a.K = 9 * g.C;
        a.ldb = 9 * g.C;
        a.a_bytes = (size_t)n * a.hin * a.win * g.C * es;
        a.ldo = g.C;
        const double bytes = ((double)n * a.hin * a.win * g.C + (double)g.C * a.K +
                              (double)a.M * g.C) * es;
        st = gemm(c, AUT_K_CONV_GEMM, a, aut::A_CONV, aut::EPI_STORE_GELU, bytes);
      }
      if (st != AUT_OK) return st;
    }
    // conv_out + positions over the batch's valid tokens (here only when a3
    // holds one batch; otherwise once over all tokens below)
    if (!W.a3_all) {
      const int r0 = p.chunks[c0].row0;
      const int r1 = (c0 + n < nch) ? p.chunks[c0 + n].row0 : (int)p.total;
      const aut_status st = conv_out(r0, r1, c0, n);
      if (st != AUT_OK) return st;
    }
  }
  if (W.a3_all && p.total > 0) return conv_out(0, (int)p.total, 0, nch);
  return AUT_OK;
}

// LayerNorm into the next product's operand: MX-fp8 (codes in y, scales in
// ysc) when ysc is given
aut_status layernorm(const Ctx& c, const float* x, size_t g_off, size_t b_off, void* y,
                     uint8_t* ysc = nullptr) {
  const int T = (int)c.p->total, d = c.g->d;
  aut::prof_begin(c.s);
  hipError_t e = aut::launch_layernorm(x, pk_at<float>(c, g_off), pk_at<float>(c, b_off), y, T, d,
                                       c.p->cfg.ln_eps, ysc ? AUT_FP8 : c.dt, c.s, ysc);
  if (e != hipSuccess) return fail(AUT_ERR_HIP, "layernorm launch failed: %s", hipGetErrorString(e));
  aut::prof_end(c.s, AUT_K_LAYERNORM, 8.0 * T * d,
                (double)T * d * (4 + (ysc ? 1.0 + 1.0 / 32 : (double)esize(c.dt))));
  return AUT_OK;
}

// encoder stack + projector: ws.x (fp32 residual, in place) -> out [T, out].
// A product on MX-fp8 operands (its AUT_FP8_* bit set) gets its activation
// operand from the kernel that produces it (LayerNorm, attention or the GELU
// epilogue of fc1 / proj1) as codes plus scales, and its weight as packed.
aut_status run_encode(const Ctx& c, float* out) {
  const aut_plan_t& p = *c.p;
  const Geometry& g = *c.g;
  const WsLayout& W = *c.W;
  const PackLayout& P = *c.P;
  const int T = (int)p.total;
  if (T == 0) return AUT_OK;
  const int d = g.d, F = g.F;
  const double es = (double)esize(c.dt);
  const double e8 = 1.0 + 1.0 / 32;  // bytes per MX-fp8 element with its scale
  float* x = (float*)(c.ws + W.x);
  void* xn = c.ws + W.xn;
  void* qkv = c.ws + W.qkv;
  void* o = c.ws + W.o;
  void* h = c.ws + W.h;
  uint8_t* xn_s = (uint8_t*)(c.ws + W.xn_s);
  uint8_t* o_s = (uint8_t*)(c.ws + W.o_s);
  uint8_t* h_s = (uint8_t*)(c.ws + W.h_s);
  const bool f_qkv = c.f8 & AUT_FP8_QKV, f_out = c.f8 & AUT_FP8_OUT;
  const bool f_fc1 = c.f8 & AUT_FP8_FC1, f_fc2 = c.f8 & AUT_FP8_FC2;
  const bool f_proj = c.f8 & AUT_FP8_PROJ;
  // one product: MX-fp8 operands (scales of A and B) or the base dtype
  // (out_s: the output's scales when the epilogue writes MX-fp8)
  auto prod = [&](bool f8, aut::GemmArgs a, const uint8_t* a_s, size_t b_s, int epi,
                  uint8_t* out_s, double bytes_base, double bytes_f8) {
    a.out_scale = out_s;
    if (!f8) return gemm(c, AUT_K_GEMM, a, aut::A_PLAIN, epi, bytes_base);
    a.a_scale = a_s;
    a.b_scale = (const uint8_t*)(c.pk + b_s);
    return gemm_f8(c, AUT_K_GEMM_FP8, a, aut::A_PLAIN, epi, bytes_f8);
  };
  aut_status st;
  for (int i = 0; i < g.layers; ++i) {
    const LayerOff& l = P.layers[i];
    if ((st = layernorm(c, x, l.ln1_g, l.ln1_b, xn, f_qkv ? xn_s : nullptr)) != AUT_OK) return st;
    st = prod(f_qkv, plain_args(xn, c.pk + l.qkv_w, T, 3 * d, d, pk_at<float>(c, l.qkv_b), qkv, 3 * d),
              xn_s, l.qkv_s, aut::EPI_STORE, nullptr,
              ((double)T * d + 3.0 * d * d + 3.0 * T * d) * es,
              ((double)T * d + 3.0 * d * d) * e8 + 3.0 * T * d * es);
    if (st != AUT_OK) return st;
    aut::prof_begin(c.s);
    hipError_t e = aut::launch_attention(qkv, o, (const int*)(c.ws + W.cu),
                                         (const int*)(c.ws + W.worder), (int)p.cu.size() - 1, g.H,
                                         d, f_out ? AUT_FP8 : c.dt, c.s, f_out ? o_s : nullptr, T);
    if (e != hipSuccess) return fail(AUT_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
    aut::prof_end(c.s, AUT_K_ATTENTION, 4.0 * d * p.sum_len2, 3.0 * T * d * es + T * d * (f_out ? e8 : es));
    st = prod(f_out, plain_args(o, c.pk + l.o_w, T, d, d, pk_at<float>(c, l.o_b), x, d), o_s, l.o_s,
              aut::EPI_RESID, nullptr, ((double)T * d + (double)d * d) * es + 8.0 * T * d,
              ((double)T * d + (double)d * d) * e8 + 8.0 * T * d);
    if (st != AUT_OK) return st;
    if ((st = layernorm(c, x, l.ln2_g, l.ln2_b, xn, f_fc1 ? xn_s : nullptr)) != AUT_OK) return st;
    // fc1 writes GELU(.) as the operand of fc2: MX-fp8 when fc2 runs on it
    st = prod(f_fc1, plain_args(xn, c.pk + l.fc1_w, T, F, d, pk_at<float>(c, l.fc1_b), h, F), xn_s,
              l.fc1_s, f_fc2 ? aut::EPI_GELU_MX : aut::EPI_STORE_GELU, f_fc2 ? h_s : nullptr,
              ((double)T * d + (double)F * d) * es + (double)T * F * (f_fc2 ? e8 : es),
              ((double)T * d + (double)F * d) * e8 + (double)T * F * (f_fc2 ? e8 : es));
    if (st != AUT_OK) return st;
    st = prod(f_fc2, plain_args(h, c.pk + l.fc2_w, T, d, F, pk_at<float>(c, l.fc2_b), x, d), h_s,
              l.fc2_s, aut::EPI_RESID, nullptr, ((double)T * F + (double)d * F) * es + 8.0 * T * d,
              ((double)T * F + (double)d * F) * e8 + 8.0 * T * d);
    if (st != AUT_OK) return st;
  }
  if ((st = layernorm(c, x, P.ln_post_g, P.ln_post_b, xn, f_proj ? xn_s : nullptr)) != AUT_OK) return st;
  st = prod(f_proj, plain_args(xn, c.pk + P.proj1_w, T, d, d, pk_at<float>(c, P.proj1_b), h, d), xn_s,
            P.proj1_s, f_proj ? aut::EPI_GELU_MX : aut::EPI_STORE_GELU, f_proj ? h_s : nullptr,
            (2.0 * T * d + (double)d * d) * es, (2.0 * T * d + (double)d * d) * e8);
  if (st != AUT_OK) return st;
  st = prod(f_proj, plain_args(h, c.pk + P.proj2_w, T, g.out, d, pk_at<float>(c, P.proj2_b), out, g.out),
            h_s, P.proj2_s, aut::EPI_STORE_F32, nullptr,
            ((double)T * d + (double)g.out * d) * es + 4.0 * T * g.out,
            ((double)T * d + (double)g.out * d) * e8 + 4.0 * T * g.out);
  return st;
}

aut_status check_features(const float* features, int32_t T_max, const aut_plan_t& p) {
  if (T_max < 0) return fail(AUT_ERR_INVALID_ARG, "T_max must be >= 0");
  for (int b = 0; b < p.B; ++b)
    if (p.lens[b] > T_max)
      return fail(AUT_ERR_INVALID_ARG, "feature_lens[%d] = %d exceeds T_max = %d", b, p.lens[b], T_max);
  if (p.total > 0 && !features) return fail(AUT_ERR_INVALID_ARG, "features is NULL");
  return AUT_OK;
}

}  // namespace

extern "C" aut_status aut_encode_planned(const aut_config* cfg, const aut_plan_t* plan,
                                         const float* features, int32_t T_max, const void* packed,
                                         aut_dtype dt, float* out, void* ws, size_t ws_bytes,
                                         void* stream) {
  WsLayout W;
  aut_status st = check_common(cfg, plan, dt, packed, ws, ws_bytes, &W);
  if (st != AUT_OK) return st;
  if ((st = check_features(features, T_max, *plan)) != AUT_OK) return st;
  if (plan->total > 0 && !out) return fail(AUT_ERR_INVALID_ARG, "out is NULL");
  if (plan->total == 0) return AUT_OK;
  const PackLayout P = pack_layout(plan->geo, dt, fp8_mask(plan->cfg, dt));
  Ctx c{plan, &plan->geo, base_dtype(dt), &P, &W, (const char*)packed, (char*)ws,
        (hipStream_t)stream, fp8_mask(plan->cfg, dt)};
  if ((st = run_frontend(c, features, T_max, (float*)((char*)ws + W.x))) != AUT_OK) return st;
  return run_encode(c, out);
}

extern "C" aut_status aut_frontend(const aut_config* cfg, const aut_plan_t* plan,
                                   const float* features, int32_t T_max, const void* packed,
                                   aut_dtype dt, float* hidden, void* ws, size_t ws_bytes,
                                   void* stream) {
  WsLayout W;
  aut_status st = check_common(cfg, plan, dt, packed, ws, ws_bytes, &W);
  if (st != AUT_OK) return st;
  if ((st = check_features(features, T_max, *plan)) != AUT_OK) return st;
  if (plan->total > 0 && !hidden) return fail(AUT_ERR_INVALID_ARG, "hidden is NULL");
  if (plan->total == 0) return AUT_OK;
  const PackLayout P = pack_layout(plan->geo, dt, fp8_mask(plan->cfg, dt));
  Ctx c{plan, &plan->geo, base_dtype(dt), &P, &W, (const char*)packed, (char*)ws,
        (hipStream_t)stream, fp8_mask(plan->cfg, dt)};
  return run_frontend(c, features, T_max, hidden);
}

extern "C" aut_status aut_encode_packed(const aut_config* cfg, const aut_plan_t* plan,
                                        const float* hidden, const void* packed, aut_dtype dt,
                                        float* out, void* ws, size_t ws_bytes, void* stream) {
  WsLayout W;
  aut_status st = check_common(cfg, plan, dt, packed, ws, ws_bytes, &W);
  if (st != AUT_OK) return st;
  if (plan->total == 0) return AUT_OK;
  if (!hidden || !out) return fail(AUT_ERR_INVALID_ARG, "hidden or out is NULL");
  const PackLayout P = pack_layout(plan->geo, dt, fp8_mask(plan->cfg, dt));
  Ctx c{plan, &plan->geo, base_dtype(dt), &P, &W, (const char*)packed, (char*)ws,
        (hipStream_t)stream, fp8_mask(plan->cfg, dt)};
  HIPCHK(hipMemcpyAsync((char*)ws + W.x, hidden, (size_t)plan->total * plan->geo.d * 4,
                        hipMemcpyDeviceToDevice, c.s));
  return run_encode(c, out);
}

extern "C" aut_status aut_encode(const aut_config* cfg, const float* features, int32_t T_max,
                                 const int32_t* feature_lens, int32_t B, const void* packed,
                                 aut_dtype dt, float* out, void* ws, size_t ws_bytes, void* stream) {
  aut_plan_t* plan = nullptr;
  aut_status st = aut_plan(cfg, feature_lens, B, &plan);
  if (st != AUT_OK) return st;
  WsLayout W;
  st = check_common(cfg, plan, dt, packed, ws, ws_bytes, &W);
  if (st == AUT_OK) st = check_features(features, T_max, *plan);
  if (st == AUT_OK && plan->total > 0 && !out) st = fail(AUT_ERR_INVALID_ARG, "out is NULL");
  // the upload copies the tables out of the plan before it returns
  if (st == AUT_OK) st = aut_plan_upload(plan, ws, ws_bytes, stream);
  if (st == AUT_OK)
    st = aut_encode_planned(cfg, plan, features, T_max, packed, dt, out, ws, ws_bytes, stream);
  aut_plan_destroy(plan);
  return st;
}

extern "C" aut_status aut_encode_noalloc(const aut_config* cfg, const float* features, int32_t T_max,
                                         const int32_t* feature_lens, int32_t B, const void* packed,
                                         aut_dtype dt, float* out, void* stream) {
  aut_plan_t* plan = nullptr;
  aut_status st = aut_plan(cfg, feature_lens, B, &plan);
  if (st != AUT_OK) return st;
  st = check_dtype(*cfg, dt);
  // the size check is host arithmetic and comes before any HIP call
  if (st == AUT_OK) {
    const size_t need = ws_layout(*plan, dt).total;
    if (need > aut::scratch_bytes())
      st = fail(AUT_ERR_WORKSPACE_TOO_SMALL,
                "this batch needs %zu bytes of device scratch; aut_encode_noalloc holds %zu "
                "(smaller batches, or a smaller conv_chunksize, fit)",
                need, aut::scratch_bytes());
  }
  void* ws = nullptr;
  if (st == AUT_OK && plan->total > 0) {
    hipError_t e = aut::scratch_ptr(&ws);
    if (e != hipSuccess) st = fail(AUT_ERR_HIP, "device scratch lookup failed: %s", hipGetErrorString(e));
  }
  WsLayout W;
  if (st == AUT_OK && plan->total > 0) {
    st = check_common(cfg, plan, dt, packed, ws, aut::scratch_bytes(), &W);
    if (st == AUT_OK) st = check_features(features, T_max, *plan);
    if (st == AUT_OK && !out) st = fail(AUT_ERR_INVALID_ARG, "out is NULL");
  }
  if (st == AUT_OK && plan->total > 0) {
    // the plan tables straight from the plan's host memory (pageable: the
    // runtime has consumed the source when each copy returns), no staging
    hipStream_t s = (hipStream_t)stream;
    char* d = (char*)ws;
    hipError_t e = hipMemcpyAsync(d + W.chunks, plan->chunks.data(), plan->chunks.size() * sizeof(aut_chunk),
                                  hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(d + W.rowmap, plan->rowmap.data(), plan->rowmap.size() * 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(d + W.cu, plan->cu.data(), plan->cu.size() * 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(d + W.worder, plan->worder.data(), plan->worder.size() * 4, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) st = fail(AUT_ERR_HIP, "plan upload failed: %s", hipGetErrorString(e));
  }
  if (st == AUT_OK && plan->total > 0)
    st = aut_encode_planned(cfg, plan, features, T_max, packed, dt, out, ws, aut::scratch_bytes(), stream);
  aut_plan_destroy(plan);
  return st;
}

// ---------------------------------------------------------------------------
// incremental (streaming) encode of one request
// ---------------------------------------------------------------------------

namespace {

// output rows of a request of L frames: full chunks of w3 tokens plus the
// three stride-2 halvings of a partial chunk's frames
int64_t request_tokens(const Geometry& g, int64_t L) {
  const int64_t full = L / g.cf;
  const int rem = (int)(L - full * g.cf);
  return full * g.w3 + (rem ? half_up(half_up(half_up(rem))) : 0);
}

}  // namespace

extern "C" aut_status aut_stream_plan(const aut_config* cfg, int32_t frames_total,
                                      int32_t windows_final, int32_t* frame_begin,
                                      int32_t* row_begin, int32_t* rows,
                                      int32_t* windows_final_after) {
  aut_status st = aut_config_check(cfg);
  if (st != AUT_OK) return st;
  if (frames_total < 0) return fail(AUT_ERR_INVALID_ARG, "frames_total = %d < 0", frames_total);
  const Geometry g = aut::geometry(*cfg);
  const int fpw = g.cf * g.chunks_per_window;  // frames per window (n_window_infer)
  const int complete = frames_total / fpw;
  if (windows_final < 0 || windows_final > complete)
    return fail(AUT_ERR_INVALID_ARG, "windows_final = %d outside [0, %d] for %d frames",
                windows_final, complete, frames_total);
  const int64_t f0 = (int64_t)windows_final * fpw;
  const int64_t r0 = (int64_t)windows_final * g.window_tokens;
  if (frame_begin) *frame_begin = (int32_t)f0;
  if (row_begin) *row_begin = (int32_t)r0;
  if (rows) *rows = (int32_t)(request_tokens(g, frames_total) - r0);
  if (windows_final_after) *windows_final_after = complete;
  return AUT_OK;
}

extern "C" aut_status aut_stream_workspace_bytes(const aut_config* cfg, int32_t max_frames,
                                                 aut_dtype dtype, size_t* bytes) {
  if (!bytes) return fail(AUT_ERR_INVALID_ARG, "bytes is NULL");
  if (max_frames < 0) return fail(AUT_ERR_INVALID_ARG, "max_frames = %d < 0", max_frames);
  aut_plan_t* plan = nullptr;
  aut_status st = aut_plan(cfg, &max_frames, 1, &plan);
  if (st != AUT_OK) return st;
  st = aut_workspace_bytes(cfg, plan, dtype, bytes);
  aut_plan_destroy(plan);
  return st;
}

extern "C" aut_status aut_encode_stream(const aut_config* cfg, const float* features,
                                        int32_t T_max, int32_t frames_total,
                                        int32_t windows_final, const void* packed, aut_dtype dt,
                                        float* out, void* ws, size_t ws_bytes, void* stream,
                                        int32_t* windows_final_after) {
  int32_t f0 = 0, r0 = 0, rows = 0, after = 0;
  aut_status st = aut_stream_plan(cfg, frames_total, windows_final, &f0, &r0, &rows, &after);
  if (st != AUT_OK) return st;
  if (frames_total > T_max)
    return fail(AUT_ERR_INVALID_ARG, "frames_total = %d exceeds T_max = %d", frames_total, T_max);
  if (rows > 0) {
    if (!features) return fail(AUT_ERR_INVALID_ARG, "features is NULL");
    if (!out) return fail(AUT_ERR_INVALID_ARG, "out is NULL");
    // the frames from f0 on form a request of their own: same mel rows (row
    // stride T_max), chunk-aligned start, so the same chunks, windows and
    // chunk-local positions as in the whole request
    const int32_t len = frames_total - f0;
    st = aut_encode(cfg, features + f0, T_max, &len, 1, packed, dt,
                    out + (size_t)r0 * cfg->output_dim, ws, ws_bytes, stream);
    if (st != AUT_OK) return st;
  }
  if (windows_final_after) *windows_final_after = after;
  return AUT_OK;
}

// ---------------------------------------------------------------------------
// log-mel front end
// ---------------------------------------------------------------------------

extern "C" aut_status aut_logmel_tables_bytes(size_t* bytes) {
  if (!bytes) return fail(AUT_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = aut::logmel_table_floats() * sizeof(float);
  return AUT_OK;
}

extern "C" aut_status aut_logmel_tables_init(void* tables, size_t bytes, void* stream) {
  if (!tables) return fail(AUT_ERR_INVALID_ARG, "tables is NULL");
  if (bytes < aut::logmel_table_floats() * sizeof(float))
    return fail(AUT_ERR_WORKSPACE_TOO_SMALL, "tables buffer has %zu bytes, needs %zu", bytes,
                aut::logmel_table_floats() * sizeof(float));
  if ((size_t)tables & 15) return fail(AUT_ERR_INVALID_ARG, "tables must be 16-byte aligned");
  hipError_t e = aut::launch_logmel_tables((float*)tables, (hipStream_t)stream);
  if (e != hipSuccess) return fail(AUT_ERR_HIP, "log-mel table launch failed: %s", hipGetErrorString(e));
  return AUT_OK;
}

extern "C" aut_status aut_logmel_workspace_bytes(int32_t B, size_t* bytes) {
  if (!bytes) return fail(AUT_ERR_INVALID_ARG, "bytes is NULL");
  if (B < 0) return fail(AUT_ERR_INVALID_ARG, "B must be >= 0");
  *bytes = align256((size_t)B * 4) + align256((size_t)B * 4);
  return AUT_OK;
}

extern "C" aut_status aut_logmel(const float* audio, int32_t S_max, const int32_t* sample_lens,
                                 int32_t B, const void* tables, float* features, int32_t T_max,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (B < 0) return fail(AUT_ERR_INVALID_ARG, "B must be >= 0");
  if (B == 0) return AUT_OK;
  if (!sample_lens) return fail(AUT_ERR_INVALID_ARG, "sample_lens is NULL");
  int max_frames = 0;
  for (int b = 0; b < B; ++b) {
    const int n = sample_lens[b];
    if (n < 0 || n > S_max)
      return fail(AUT_ERR_INVALID_ARG, "sample_lens[%d] = %d outside [0, S_max = %d]", b, n, S_max);
    if (n > 0 && n <= aut::LM_NFFT / 2)
      return fail(AUT_ERR_INVALID_ARG, "sample_lens[%d] = %d: reflect padding needs more than %d samples",
                  b, n, aut::LM_NFFT / 2);
    max_frames = std::max(max_frames, n / aut::LM_HOP);
  }
  if (max_frames > T_max)
    return fail(AUT_ERR_INVALID_ARG, "T_max = %d is below %d frames", T_max, max_frames);
  if (T_max % 4) return fail(AUT_ERR_INVALID_ARG, "T_max must be a multiple of 4");
  if (!audio || !tables || !features || !ws) return fail(AUT_ERR_INVALID_ARG, "NULL buffer");
  if (((size_t)features & 15) || ((size_t)tables & 15))
    return fail(AUT_ERR_INVALID_ARG, "features and tables must be 16-byte aligned");
  size_t need = 0;
  aut_logmel_workspace_bytes(B, &need);
  if (ws_bytes < need) return fail(AUT_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  int* lens_dev = (int*)ws;
  unsigned* mx = (unsigned*)((char*)ws + align256((size_t)B * 4));
  // the host lengths may go away after the call: copied out before it returns
  aut_status ust = upload_pinned(lens_dev, (size_t)B * 4, s,
                                 [&](char* h) { memcpy(h, sample_lens, (size_t)B * 4); });
  if (ust != AUT_OK) return ust;
  aut::prof_begin(s);
  hipError_t e = aut::launch_logmel(audio, S_max, lens_dev, B, max_frames, (const float*)tables, features, T_max,
                         mx, s);
  if (e != hipSuccess) return fail(AUT_ERR_HIP, "log-mel launch failed: %s", hipGetErrorString(e));
  double frames = 0;
  for (int b = 0; b < B; ++b) frames += sample_lens[b] / aut::LM_HOP;
  const int bins = 16 * aut::LM_BIN_TILES;
  aut::prof_end(s, AUT_K_LOGMEL, frames * 2.0 * aut::LM_NFFT * 2 * bins + frames * 2.0 * bins * aut::LM_MELS,
                frames * aut::LM_HOP * 4.0 + frames * aut::LM_MELS * 4.0 * 3);
  return AUT_OK;
}

// ---------------------------------------------------------------------------
// audio rows into the decoder sequence
// ---------------------------------------------------------------------------

extern "C" aut_status aut_audio_rows(const int32_t* ids, int64_t n_ids, int32_t pad_id,
                                     int64_t n_audio, int32_t* rows) {
  if (n_ids < 0 || n_audio < 0) return fail(AUT_ERR_INVALID_ARG, "negative length");
  if (n_ids > 0 && !ids) return fail(AUT_ERR_INVALID_ARG, "ids is NULL");
  if (n_audio > 0 && !rows) return fail(AUT_ERR_INVALID_ARG, "rows is NULL");
  if (n_ids > INT32_MAX) return fail(AUT_ERR_UNSUPPORTED, "sequence longer than 2^31 - 1");
  int64_t k = 0;
  for (int64_t i = 0; i < n_ids; ++i)
    if (ids[i] == pad_id) {
      if (k < n_audio) rows[k] = (int32_t)i;
      ++k;
    }
  if (k != n_audio)
    return fail(AUT_ERR_INVALID_ARG, "%lld placeholders for %lld audio rows", (long long)k,
                (long long)n_audio);
  return AUT_OK;
}

extern "C" aut_status aut_inject_audio(const float* audio, const int32_t* rows, int64_t n_audio,
                                       int32_t dim, void* dst, int64_t dst_rows,
                                       aut_dtype dst_dtype, void* stream) {
  if (n_audio < 0 || dst_rows < 0) return fail(AUT_ERR_INVALID_ARG, "negative length");
  if (dst_dtype != AUT_FP32 && dst_dtype != AUT_BF16) return fail(AUT_ERR_INVALID_ARG, "bad dtype");
  if (n_audio == 0) return AUT_OK;
  if (!audio || !rows || !dst) return fail(AUT_ERR_INVALID_ARG, "NULL buffer");
  if (dim <= 0 || dim % 4) return fail(AUT_ERR_INVALID_ARG, "dim = %d must be a positive multiple of 4", dim);
  if (((size_t)audio & 15) || ((size_t)dst & 15))
    return fail(AUT_ERR_INVALID_ARG, "audio and dst must be 16-byte aligned");
  hipError_t e = aut::launch_inject(audio, rows, (long)n_audio, dim, dst, (long)dst_rows, dst_dtype,
                                    (hipStream_t)stream);
  if (e != hipSuccess) return fail(AUT_ERR_HIP, "inject launch failed: %s", hipGetErrorString(e));
  return AUT_OK;
}

// ---------------------------------------------------------------------------
// MX-fp8 primitives
// ---------------------------------------------------------------------------

extern "C" aut_status aut_mx_scale_bytes(int64_t rows, int32_t K, size_t* bytes) {
  if (!bytes) return fail(AUT_ERR_INVALID_ARG, "bytes is NULL");
  if (rows < 0 || K <= 0 || K % 128)
    return fail(AUT_ERR_INVALID_ARG, "need rows >= 0 and K a positive multiple of 128");
  *bytes = aut::mx_scale_bytes((long)rows, K);
  return AUT_OK;
}

extern "C" aut_status aut_mx_quantize(const float* x, int64_t rows, int32_t K, uint8_t* codes,
                                      uint8_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 128)
    return fail(AUT_ERR_INVALID_ARG, "need rows >= 0 and K a positive multiple of 128");
  if (rows == 0) return AUT_OK;
  if (!x || !codes || !scales) return fail(AUT_ERR_INVALID_ARG, "NULL pointer");
  if (((size_t)x & 15) || ((size_t)codes & 15))
    return fail(AUT_ERR_INVALID_ARG, "x and codes must be 16-byte aligned");
  if (rows * (int64_t)K >= ((int64_t)1 << 40)) return fail(AUT_ERR_INVALID_ARG, "too large");
  hipError_t e = aut::launch_mx_quantize(x, K, (long)rows, K, codes, scales, (hipStream_t)stream);
  if (e != hipSuccess) return fail(AUT_ERR_HIP, "mx quantize launch failed: %s", hipGetErrorString(e));
  return AUT_OK;
}

extern "C" aut_status aut_mx_matmul(const uint8_t* a_codes, const uint8_t* a_scales, int64_t M,
                                    const uint8_t* b_codes, const uint8_t* b_scales, int32_t N,
                                    int32_t K, float* out, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || K % 128)
    return fail(AUT_ERR_INVALID_ARG, "need M, N >= 0 and K a positive multiple of 128");
  if (M == 0 || N == 0) return AUT_OK;
  if (N % 4) return fail(AUT_ERR_UNSUPPORTED, "N must be a multiple of 4");
  if (!a_codes || !a_scales || !b_codes || !b_scales || !out)
    return fail(AUT_ERR_INVALID_ARG, "NULL pointer");
  if (((size_t)a_codes & 15) || ((size_t)b_codes & 15) || ((size_t)out & 15))
    return fail(AUT_ERR_INVALID_ARG, "codes and out must be 16-byte aligned");
  // 32-bit buffer offsets inside the kernel
  if (M * (int64_t)K >= ((int64_t)1 << 31) || (int64_t)N * K >= ((int64_t)1 << 31) ||
      M > ((int64_t)1 << 30))
    return fail(AUT_ERR_UNSUPPORTED, "operands of 2 GiB or more");
  aut::GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.A = a_codes; a.lda = K; a.B = b_codes; a.ldb = K;
  a.M = (int)M; a.N = N; a.K = K;
  a.out = out; a.ldo = N;
  a.a_scale = a_scales; a.b_scale = b_scales;
  hipError_t e = aut::launch_gemm_f8(a, aut::A_PLAIN, aut::EPI_STORE_F32, (hipStream_t)stream);
  if (e != hipSuccess) return fail(AUT_ERR_HIP, "mx matmul launch failed: %s", hipGetErrorString(e));
  return AUT_OK;
}

extern "C" aut_status aut_layernorm(const float* x, int64_t rows, int32_t d, const float* gamma,
                                    const float* beta, float eps, aut_dtype dtype, void* y,
                                    uint8_t* y_scales, void* stream) {
  if (rows < 0) return fail(AUT_ERR_INVALID_ARG, "rows = %lld is negative", (long long)rows);
  if (dtype != AUT_FP32 && dtype != AUT_BF16 && dtype != AUT_FP8)
    return fail(AUT_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (d <= 0 || d % 4 || d > 2048 || (dtype == AUT_FP8 && d % 128))
    return fail(AUT_ERR_UNSUPPORTED, "d = %d: need a multiple of 4 (of 128 for fp8), at most 2048", d);
  if (rows >= ((int64_t)1 << 31)) return fail(AUT_ERR_UNSUPPORTED, "rows = %lld: at most 2^31 - 1", (long long)rows);
  if (rows == 0) return AUT_OK;
  if (!x || !gamma || !beta || !y || (dtype == AUT_FP8 && !y_scales))
    return fail(AUT_ERR_INVALID_ARG, "NULL pointer");
  if (((size_t)x & 15) || ((size_t)y & 7) || ((size_t)gamma & 15) || ((size_t)beta & 15))
    return fail(AUT_ERR_INVALID_ARG, "x, gamma and beta must be 16-byte aligned, y 8-byte aligned");
  hipError_t e = aut::launch_layernorm(x, gamma, beta, y, (int)rows, d, eps, dtype, (hipStream_t)stream,
                                       y_scales);
  if (e != hipSuccess) return fail(AUT_ERR_HIP, "layernorm launch failed: %s", hipGetErrorString(e));
  return AUT_OK;
}

extern "C" aut_status aut_attention(const void* qkv, int64_t rows, int32_t heads,
                                    const int32_t* cu_seqlens, const int32_t* window_order,
                                    int32_t n_windows, aut_dtype in_dtype, aut_dtype out_dtype,
                                    void* out, uint8_t* out_scales, void* stream) {
  if (rows < 0 || n_windows < 0)
    return fail(AUT_ERR_INVALID_ARG, "rows = %lld and n_windows = %d must not be negative",
                (long long)rows, n_windows);
  const bool ok_pair = (in_dtype == AUT_FP32 && out_dtype == AUT_FP32) ||
                       (in_dtype == AUT_BF16 && (out_dtype == AUT_BF16 || out_dtype == AUT_FP32 ||
                                                 out_dtype == AUT_FP8));
  if (!ok_pair)
    return fail(AUT_ERR_UNSUPPORTED, "dtypes (%d -> %d): fp32 -> fp32, bf16 -> bf16, fp32 or fp8",
                (int)in_dtype, (int)out_dtype);
  if (heads <= 0 || heads > 64 || (out_dtype == AUT_FP8 && heads % 2))
    return fail(AUT_ERR_UNSUPPORTED, "heads = %d: 1 to 64 (even for fp8 output)", heads);
  if (rows >= ((int64_t)1 << 31)) return fail(AUT_ERR_UNSUPPORTED, "rows = %lld: at most 2^31 - 1", (long long)rows);
  if (rows == 0 || n_windows == 0) return AUT_OK;
  if (!qkv || !cu_seqlens || !window_order || !out || (out_dtype == AUT_FP8 && !out_scales))
    return fail(AUT_ERR_INVALID_ARG, "NULL pointer");
  if (((size_t)qkv & 15) || ((size_t)out & 15) || ((size_t)cu_seqlens & 3) || ((size_t)window_order & 3))
    return fail(AUT_ERR_INVALID_ARG, "qkv and out must be 16-byte aligned, the tables 4-byte aligned");
  const int d = 64 * heads;
  const aut_dtype kdt = out_dtype == AUT_FP8 ? AUT_FP8 : in_dtype;
  hipError_t e = aut::launch_attention(qkv, out, cu_seqlens, window_order, n_windows, heads, d, kdt,
                                       (hipStream_t)stream, out_scales, (int)rows,
                                       in_dtype == AUT_BF16 && out_dtype == AUT_FP32);
  if (e != hipSuccess) return fail(AUT_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  return AUT_OK;
}

// ---------------------------------------------------------------------------
// timing and errors
// ---------------------------------------------------------------------------

extern "C" aut_status aut_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(aut::g_prof_mu);
  aut::g_prof_on = on != 0;
  return AUT_OK;
}

extern "C" aut_status aut_profile_collect(aut_kernel_stats* stats) {
  if (!stats) return fail(AUT_ERR_INVALID_ARG, "stats is NULL");
  std::lock_guard<std::mutex> lk(aut::g_prof_mu);
  for (int k = 0; k < AUT_K_COUNT; ++k) stats[k] = aut_kernel_stats{0, 0.0, 0.0, 0.0};
  aut_status st = AUT_OK;
  for (auto& r : aut::g_prof) {
    if (st == AUT_OK) {
      hipError_t e = hipEventSynchronize(r.stop);
      float ms = 0.f;
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
      if (e != hipSuccess) {
        st = fail(AUT_ERR_HIP, "event timing failed: %s", hipGetErrorString(e));
      } else {
        aut_kernel_stats& k = stats[r.cls];
        k.launches += 1;
        k.total_ms += ms;
        k.flops += r.flops;
        k.bytes += r.bytes;
      }
    }
    aut::g_event_pool.push_back(r.start);
    aut::g_event_pool.push_back(r.stop);
  }
  aut::g_prof.clear();
  return st;
}

extern "C" const char* aut_last_error(void) { return g_err; }
