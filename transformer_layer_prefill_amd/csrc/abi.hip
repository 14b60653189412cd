// C-ABI entry points: argument validation, workspace layout and the launch
// sequence of one layer / one chunk.  See include/tlp.h for the contract.
//
// Launch sequence of a layer (oxibonsai-kernels metal_prefill.rs,
// encode_layer_prefill steps 1-7), all on the caller's stream, no host sync:
//   rmsnorm (+ fp32 copy of the residual) -> QKV GEMM -> QK-norm/RoPE/KV store
//   -> attention -> O GEMM (+ residual, fp32) -> rmsnorm -> gate/up GEMM with
//   SwiGLU -> down GEMM (+ residual)
// The chunk driver (turbospark-runtime llama/prefill.rs,
// prefill_chunk_real_llama_dense) runs that per micro-batch and per layer,
// keeping the residual stream in fp32 between layers.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/tlp.h"
#include "launch.h"

// A caller-owned pipeline handle (tlp_pipeline_create): the second stream and
// the events that let tlp_prefill_chunk keep two micro-batches in flight.
struct tlp_pipeline {
  int device = -1;
  int max_layers = 0;
  hipStream_t second = nullptr;
  std::vector<hipEvent_t> ev;   // [2][max_layers] K/V-stored events, then start, end
};

namespace {

thread_local std::string g_last_error;

tlp_status fail(tlp_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
tlp_status fail(tlp_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

size_t elt_size(const tlp_config& c) { return c.dtype == TLP_F32 ? 4 : 2; }

tlp_status check_config(const tlp_config* c) {
  if (!c) return fail(TLP_ERR_NULL, "config is NULL");
  if (c->dtype != TLP_F32 && c->dtype != TLP_BF16)
    return fail(TLP_ERR_UNSUPPORTED, "dtype %d is not TLP_F32 or TLP_BF16", c->dtype);
  if (c->wformat != TLP_W_DENSE && c->wformat != TLP_W_SIGN1_G128)
    return fail(TLP_ERR_UNSUPPORTED, "wformat %d is not a tlp_wformat", c->wformat);
  if (c->wformat == TLP_W_SIGN1_G128 && c->dtype != TLP_BF16)
    return fail(TLP_ERR_UNSUPPORTED, "1-bit weights need dtype TLP_BF16");
  if (c->kv_format != TLP_KV_ACT && c->kv_format != TLP_KV_F16)
    return fail(TLP_ERR_UNSUPPORTED, "kv_format %d is not a tlp_kv_format", c->kv_format);
  if (c->kv_format == TLP_KV_F16 && c->dtype != TLP_BF16)
    return fail(TLP_ERR_UNSUPPORTED, "an fp16 KV cache needs dtype TLP_BF16");
  if (c->hidden <= 0 || c->intermediate <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
      c->max_seq <= 0 || c->n_layers <= 0)
    return fail(TLP_ERR_SHAPE, "sizes must be positive");
  if (c->hidden > 16384)
    return fail(TLP_ERR_UNSUPPORTED, "hidden %d above 16384", c->hidden);
  if (c->hidden % 8 || c->intermediate % 8)
    return fail(TLP_ERR_SHAPE, "hidden (%d) and intermediate (%d) must be multiples of 8",
                c->hidden, c->intermediate);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(TLP_ERR_SHAPE, "head_dim %d is not 64 or 128", c->head_dim);
  if (c->n_q_heads % c->n_kv_heads)
    return fail(TLP_ERR_SHAPE, "n_q_heads %d is not a multiple of n_kv_heads %d",
                c->n_q_heads, c->n_kv_heads);
  const int g = c->n_q_heads / c->n_kv_heads;
  if (!(g == 1 || g == 2 || g == 4 || g % 4 == 0))
    return fail(TLP_ERR_UNSUPPORTED, "heads per kv group %d is not 1, 2 or a multiple of 4", g);
  if (c->wformat == TLP_W_SIGN1_G128 &&
      (c->hidden % 128 || c->intermediate % 128 || (c->n_q_heads * c->head_dim) % 128))
    return fail(TLP_ERR_SHAPE, "1-bit weights need every K (hidden, intermediate, nq*hd) "
                               "to be a multiple of 128");
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps))
    return fail(TLP_ERR_SHAPE, "rms_eps must be finite and >= 0");
  return TLP_OK;
}

// Whether a micro-batch of n rows takes the skinny projections (decode steps
// and short batches with bf16 activations, dense or 1-bit weights).
bool skinny_path(const tlp_config& c, int n) {
  return c.dtype == TLP_BF16 && n <= tlp::kSkinnyMaxM;
}

// fp32 elements of the PART region for any micro-batch of at most m rows
// (bf16 path): split-K slices of the QKV, output and down projections (and of
// gate/up on the skinny path), or the split-KV partial results of attention
// (the two are never live at once).
size_t part_elems(const tlp_config& c, int m) {
  if (c.dtype != TLP_BF16) return 0;
  using namespace tlp;
  const int H = c.hidden, I = c.intermediate, qd = c.n_q_heads * c.head_dim;
  const int qkv = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  size_t best = 0;
  auto take = [&](size_t v) { if (v > best) best = v; };
  for (int r = 1; r <= m; ++r) {
    if (skinny_path(c, r)) {
      take(static_cast<size_t>(skinny_splits(qkv, H, c.wformat == TLP_W_SIGN1_G128)) * qkv * r);
      take(static_cast<size_t>(skinny_splits(H, qd, c.wformat == TLP_W_SIGN1_G128)) * H * r);
      take(static_cast<size_t>(skinny_splits(2 * I, H, c.wformat == TLP_W_SIGN1_G128)) * 2 * I * r);
      take(static_cast<size_t>(skinny_splits(H, I, c.wformat == TLP_W_SIGN1_G128)) * H * r);
    } else {
      const int a = gemm_partial_splits(r, H, qd);
      const int b = gemm_partial_splits(r, H, I);
      take(static_cast<size_t>(a > b ? a : b) * H * r);
      take(static_cast<size_t>(gemm_partial_splits(r, qkv, H)) * qkv * r);
    }
    take(attention_split_floats(r, c.max_seq, c.n_q_heads, c.n_kv_heads, c.head_dim));
  }
  return best;
}

struct Layout {
  size_t off[TLP_WS_COUNT];
  size_t total;
  size_t part_floats;   // capacity of the PART region
};

Layout layout_of(const tlp_config& c, int m) {
  const size_t e = elt_size(c), M = static_cast<size_t>(m);
  const size_t qkv = static_cast<size_t>(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  const size_t sizes[TLP_WS_COUNT] = {
      M * c.hidden * 4,                                       // RES
      M * c.hidden * e,                                       // XN
      M * qkv * e,                                            // QKV
      M * static_cast<size_t>(c.n_q_heads) * c.head_dim * e,  // ATTN
      M * c.intermediate * e,                                 // ACT
      static_cast<size_t>(c.hidden) * 4,                      // HEAD
      part_elems(c, m) * 4,                                    // PART
  };
  Layout L{};
  L.part_floats = sizes[TLP_WS_PART] / 4;
  size_t o = 0;
  for (int i = 0; i < TLP_WS_COUNT; ++i) {
    L.off[i] = o;
    o += align256(sizes[i]);
  }
  L.total = o;
  return L;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

tlp_status check_weight(const tlp_config& c, const tlp_weight& w, const char* name) {
  if (!w.data) return fail(TLP_ERR_NULL, "weight %s is NULL", name);
  if (c.wformat == TLP_W_SIGN1_G128 && !w.scales)
    return fail(TLP_ERR_NULL, "1-bit weight %s has no scales", name);
  if (!aligned16(w.data))
    return fail(TLP_ERR_UNSUPPORTED, "weight %s is not 16-byte aligned", name);
  return TLP_OK;
}

tlp_status check_layer_weights(const tlp_config& c, const tlp_layer_weights* w, int idx) {
  if (!w) return fail(TLP_ERR_NULL, "layer weights are NULL");
  if (!w->attn_norm || !w->ffn_norm)
    return fail(TLP_ERR_NULL, "layer %d: a norm gain is NULL", idx);
  if (c.qk_norm && (!w->q_norm || !w->k_norm))
    return fail(TLP_ERR_NULL, "layer %d: qk_norm is on but q_norm/k_norm is NULL", idx);
  if (!aligned16(w->attn_norm) || !aligned16(w->ffn_norm) ||
      (c.qk_norm && (!aligned16(w->q_norm) || !aligned16(w->k_norm))))
    return fail(TLP_ERR_UNSUPPORTED, "layer %d: norm gains must be 16-byte aligned", idx);
  tlp_status s;
  if ((s = check_weight(c, w->w_qkv, "w_qkv")) != TLP_OK) return s;
  if ((s = check_weight(c, w->w_o, "w_o")) != TLP_OK) return s;
  if ((s = check_weight(c, w->w_gate_up, "w_gate_up")) != TLP_OK) return s;
  if ((s = check_weight(c, w->w_down, "w_down")) != TLP_OK) return s;
  return TLP_OK;
}

tlp_status check_call(const tlp_config& c, void* hidden, int n, int start, void* kc, void* vc,
                      const float* cs, const float* sn, void* ws, size_t ws_bytes, int m_ws) {
  if (!hidden || !kc || !vc || !cs || !sn || !ws)
    return fail(TLP_ERR_NULL, "hidden, caches, rope tables and workspace must be non-NULL");
  if (n <= 0) return fail(TLP_ERR_SHAPE, "n_tokens %d must be > 0", n);
  if (start < 0) return fail(TLP_ERR_POSITION, "start_position %d is negative", start);
  if (static_cast<int64_t>(start) + n > c.max_seq)
    return fail(TLP_ERR_POSITION, "start_position %d + n_tokens %d exceeds max_seq %d", start,
                n, c.max_seq);
  if (!aligned16(hidden) || !aligned16(kc) || !aligned16(vc) || !aligned16(cs) ||
      !aligned16(sn))
    return fail(TLP_ERR_UNSUPPORTED, "hidden, caches and rope tables must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return fail(TLP_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const size_t need = layout_of(c, m_ws).total;
  if (ws_bytes < need)
    return fail(TLP_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return TLP_OK;
}

// ---- per-kernel timing with HIP events (tlp_profile_begin / tlp_profile_end) --
// tlp_profile_begin creates a fixed number of event pairs for the calling
// thread; while profiling is on, every launch the thread makes is bracketed by
// the next pair, recorded on the launch's own stream (launches beyond the
// capacity are counted as not timed).  tlp_profile_end waits for the events,
// sums the elapsed times per kernel and destroys them.
struct ProfRecord {
  int kernel;
  hipEvent_t start, stop;
};
thread_local bool g_prof_on = false;
thread_local std::vector<ProfRecord> g_prof;   // created pairs; kernel < 0: not used yet
thread_local size_t g_prof_used = 0;
thread_local int32_t g_prof_dropped = 0;

struct ProfScope {
  int kernel;
  hipStream_t s;
  ProfRecord* rec = nullptr;
  hipError_t err = hipSuccess;
  ProfScope(int k, hipStream_t st) : kernel(k), s(st) {
    if (!g_prof_on) return;
    if (g_prof_used == g_prof.size()) {
      ++g_prof_dropped;
      return;
    }
    rec = &g_prof[g_prof_used++];
    rec->kernel = kernel;
    err = hipEventRecord(rec->start, s);
  }
  hipError_t finish() {
    if (!rec || err != hipSuccess) return err;
    return err = hipEventRecord(rec->stop, s);
  }
};

void prof_release() {
  for (ProfRecord& r : g_prof) {
    if (r.start) (void)hipEventDestroy(r.start);
    if (r.stop) (void)hipEventDestroy(r.stop);
  }
  g_prof.clear();
  g_prof_used = 0;
}

#define TLP_LAUNCH(kid, expr)                                                     \
  do {                                                                            \
    ProfScope ps_(kid, s);                                                        \
    hipError_t e_ = ps_.err == hipSuccess ? (expr) : ps_.err;                     \
    if (e_ == hipSuccess) e_ = ps_.finish();                                      \
    if (e_ != hipSuccess)                                                         \
      return fail(TLP_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_));           \
  } while (0)

// One layer over a micro-batch.  x_in holds the rows' input: the hidden rows
// in the activation type (x_in_f32 false) or the fp32 residual stream, to which
// the in_parts split-K slices of the previous layer's down projection are
// added.  out_act non-null: the layer's output is also rounded into out_act
// (and *out_parts = 0); otherwise the down projection's slices are left for
// the next layer (*out_parts = their count; the fp32 path never splits).
// kv_done, if not null, is recorded on s once this layer's K/V slots are in
// the cache; kv_wait, if not null, is waited for before attention reads it.
tlp_status run_layer(const tlp_config& c, const tlp_layer_weights& w, int layer, int n,
                     int start, const void* x_in, bool x_in_f32, int in_parts, void* out_act,
                     int* out_parts, char* kc, char* vc, const float* cs, const float* sn,
                     char* ws, const Layout& L, hipStream_t s, hipEvent_t kv_done = nullptr,
                     hipEvent_t kv_wait = nullptr) {
  using namespace tlp;
  const Act act = c.dtype == TLP_F32 ? Act::F32 : Act::BF16;
  const int H = c.hidden, I = c.intermediate, hd = c.head_dim;
  const int nq = c.n_q_heads, nkv = c.n_kv_heads;
  const int qkv_dim = (nq + 2 * nkv) * hd, qd = nq * hd;
  float* res = reinterpret_cast<float*>(ws + L.off[TLP_WS_RES]);
  float* part = reinterpret_cast<float*>(ws + L.off[TLP_WS_PART]);
  const size_t part_stride = static_cast<size_t>(n) * H;
  void* xn = ws + L.off[TLP_WS_XN];
  void* qkv = ws + L.off[TLP_WS_QKV];
  void* attn = ws + L.off[TLP_WS_ATTN];
  void* a = ws + L.off[TLP_WS_ACT];
  const size_t es = elt_size(c);
  const size_t layer_off = static_cast<size_t>(layer) * nkv * c.max_seq * hd * es;
  void* k_layer = kc + layer_off;
  void* v_layer = vc + layer_off;
  const bool split = act == Act::BF16;
  const bool skinny = skinny_path(c, n);
  // the weight format comes from the config: scales of dense weights are ignored
  auto scales_of = [&](const tlp_weight& wt) -> const void* {
    return c.wformat == TLP_W_SIGN1_G128 ? wt.scales : nullptr;
  };

  // 1. residual assembly + attention RMSNorm.  Rows that arrive in bf16 with
  // no slices to add need no fp32 copy yet: widening bf16 is exact, so the
  // FFN norm pass reads the same rows itself and writes the stream then.
  const bool defer_res = split && !x_in_f32 && in_parts == 0;
  // One row with dense weights: the QKV projection normalises the row itself
  // when there is nothing else for this pass to do (a bf16 row, no slices)
  const bool one_row = skinny && n == 1 && c.wformat != TLP_W_SIGN1_G128;
  const int q_splits1 = one_row ? skinny_splits(qkv_dim, H, false) : 0;
  const bool fuse_norm = one_row && defer_res && gemv_norm_ok(qkv_dim, H, q_splits1);
  RowArgs r{};
  if (!fuse_norm) {
    r.x = x_in; r.x_f32 = x_in_f32; r.ldx = H;
    r.part = part; r.n_part = in_parts; r.part_stride = part_stride;
    r.res_out = defer_res ? nullptr : res;
    r.gain = w.attn_norm; r.norm_out = xn;
    r.rows = n; r.H = H; r.eps = c.rms_eps;
    TLP_LAUNCH(TLP_K_ATTN_NORM, launch_rownorm(act, r, s));
  }
  // 2. fused QKV projection
  GemmCall g{};
  g.act = act;
  g.A = xn; g.lda = H;
  g.W = w.w_qkv.data; g.Wscale = scales_of(w.w_qkv);
  g.M = n; g.N = qkv_dim; g.K = H;
  int q_parts = 0;
  const size_t qkv_part_stride = static_cast<size_t>(n) * qkv_dim;
  if (fuse_norm) {
    q_parts = q_splits1;
    TLP_LAUNCH(TLP_K_QKV_GEMM, launch_gemv_norm(x_in, w.attn_norm, c.rms_eps, w.w_qkv.data, qkv_dim, H,
                                                part, qkv_part_stride, q_parts, s));
  } else if (skinny) {
    q_parts = skinny_splits(qkv_dim, H, c.wformat == TLP_W_SIGN1_G128);
    TLP_LAUNCH(TLP_K_QKV_GEMM, launch_gemm_skinny(xn, H, w.w_qkv.data, scales_of(w.w_qkv), n, qkv_dim, H, part,
                                                  qkv_dim, qkv_part_stride, q_parts, s));
  } else {
    // bf16 rows straight from a one-pass kernel when its tiles fill the GPU
    // (128-row tiles at 512 tokens, 256x192 at 2048), else fp32 K slices
    const bool direct = gemm_store_direct(n, qkv_dim, H, c.wformat == TLP_W_SIGN1_G128);
    if (split && !direct) {
      g.epi = Epi::Partial; g.out = part; g.ldo = qkv_dim; g.out_f32 = true;
      g.part_stride = qkv_part_stride; g.splits_out = &q_parts;
    } else {
      g.epi = Epi::Store; g.out = qkv; g.ldo = qkv_dim;
    }
    TLP_LAUNCH(TLP_K_QKV_GEMM, launch_gemm(g, s));
  }
  // 3a-3d. (slice sum,) QK-norm, RoPE, KV-cache store
  const bool kv16 = c.kv_format == TLP_KV_F16;
  TLP_LAUNCH(TLP_K_QK_ROPE_KV,
             launch_qk_rope_store(act, kv16, qkv, n, qkv_dim, part, q_parts, qkv_part_stride,
                                  w.q_norm, w.k_norm, c.qk_norm != 0, c.rms_eps, cs, sn, k_layer,
                                  v_layer, c.max_seq, start, nq, nkv, hd, s));
  if (kv_done) {
    const hipError_t e = hipEventRecord(kv_done, s);
    if (e != hipSuccess) return fail(TLP_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  }
  if (kv_wait) {
    const hipError_t e = hipStreamWaitEvent(s, kv_wait, 0);
    if (e != hipSuccess) return fail(TLP_ERR_HIP, "hipStreamWaitEvent: %s", hipGetErrorString(e));
  }
  // 3e. causal GQA attention
  // (the PART region is free here: the QKV slices have been summed)
  TLP_LAUNCH(TLP_K_ATTENTION,
             launch_attention(act, kv16, qkv, qkv_dim, k_layer, v_layer, attn, qd, n, start, nq,
                              nkv, hd, c.max_seq, split ? part : nullptr, L.part_floats, s));
  // 4. output projection: split-K slices (bf16) or a fused residual add (fp32)
  int o_parts = 0;
  g = GemmCall{};
  g.act = act;
  g.A = attn; g.lda = qd;
  g.W = w.w_o.data; g.Wscale = scales_of(w.w_o);
  g.M = n; g.N = H; g.K = qd;
  if (skinny) {
    o_parts = skinny_splits(H, qd, c.wformat == TLP_W_SIGN1_G128);
    TLP_LAUNCH(TLP_K_O_GEMM, launch_gemm_skinny(attn, qd, w.w_o.data, scales_of(w.w_o), n, H, qd, part, H,
                                                part_stride, o_parts, s));
  } else {
    if (split) {
      g.epi = Epi::Partial; g.out = part; g.ldo = H; g.out_f32 = true;
      g.part_stride = part_stride; g.splits_out = &o_parts;
    } else {
      g.epi = Epi::Resid; g.out = res; g.ldo = H; g.out_f32 = true; g.resid = res; g.ldr = H;
    }
    TLP_LAUNCH(TLP_K_O_GEMM, launch_gemm(g, s));
  }
  // 5. residual assembly + FFN RMSNorm
  r = RowArgs{};
  if (defer_res) { r.x = x_in; r.x_f32 = 0; } else { r.x = res; r.x_f32 = 1; }
  r.ldx = H;
  r.part = part; r.n_part = o_parts; r.part_stride = part_stride;
  r.res_out = res;
  r.gain = w.ffn_norm; r.norm_out = xn;
  r.rows = n; r.H = H; r.eps = c.rms_eps;
  TLP_LAUNCH(TLP_K_FFN_NORM, launch_rownorm(act, r, s));
  // 6. gate/up projection + SwiGLU
  g = GemmCall{};
  g.act = act;
  g.A = xn; g.lda = H;
  g.W = w.w_gate_up.data; g.Wscale = scales_of(w.w_gate_up);
  g.M = n; g.N = I; g.K = H;
  if (skinny) {
    // fp32 slices of [gate ; up] x_n2, then silu(gate) * up
    const int gu_parts = skinny_splits(2 * I, H, c.wformat == TLP_W_SIGN1_G128);
    const size_t gu_stride = static_cast<size_t>(n) * 2 * I;
    TLP_LAUNCH(TLP_K_GATE_UP_GEMM, launch_gemm_skinny(xn, H, w.w_gate_up.data, scales_of(w.w_gate_up), n, 2 * I, H, part,
                                                      2 * I, gu_stride, gu_parts, s));
    TLP_LAUNCH(TLP_K_SWIGLU, launch_swiglu_finish(part, gu_parts, gu_stride, n, I, a, s));
  } else {
    g.epi = Epi::SwiGLU; g.out = a; g.ldo = I;
    TLP_LAUNCH(TLP_K_GATE_UP_GEMM, launch_gemm(g, s));
  }
  // 7. down projection
  int d_parts = 0;
  g = GemmCall{};
  g.act = act;
  g.A = a; g.lda = I;
  g.W = w.w_down.data; g.Wscale = scales_of(w.w_down);
  g.M = n; g.N = H; g.K = I;
  if (skinny) {
    d_parts = skinny_splits(H, I, c.wformat == TLP_W_SIGN1_G128);
  } else if (split) {
    g.epi = Epi::Partial; g.out = part; g.ldo = H; g.out_f32 = true;
    g.part_stride = part_stride; g.splits_out = &d_parts;
  } else {
    g.epi = Epi::Resid; g.resid = res; g.ldr = H; g.ldo = H; g.out_f32 = true;
    g.out = out_act ? out_act : res;
    if (out_act) g.res_out = res;   // the output also stays in the fp32 stream
  }
  if (skinny)
    TLP_LAUNCH(TLP_K_DOWN_GEMM, launch_gemm_skinny(a, I, w.w_down.data, scales_of(w.w_down), n, H, I, part, H,
                                                   part_stride, d_parts, s));
  else
    TLP_LAUNCH(TLP_K_DOWN_GEMM, launch_gemm(g, s));
  *out_parts = 0;
  if (split) {
    if (out_act) {
      // residual assembly into the fp32 stream and the activation-type output
      r = RowArgs{};
      r.x = res; r.x_f32 = 1; r.ldx = H;
      r.part = part; r.n_part = d_parts; r.part_stride = part_stride;
      r.res_out = res; r.act_out = out_act; r.ld_act = H;
      r.rows = n; r.H = H; r.eps = c.rms_eps;
      TLP_LAUNCH(TLP_K_OUT_ROWS, launch_rownorm(act, r, s));
    } else {
      *out_parts = d_parts;
    }
  }
  return TLP_OK;
}

// Two micro-batches of a chunk in flight: the caller's pipeline handle holds a
// second stream for the odd micro-batches and, per (stream parity, layer), an
// event recorded once that micro-batch's K/V of the layer are in the cache,
// plus a start and an end event.  ChunkPipe starts the second stream behind
// the work already on the caller's stream and, when it goes out of scope,
// joins it back (all of the call's work then completes in the caller's stream
// order, also after an error).
struct ChunkPipe {
  hipStream_t main = nullptr;
  tlp_pipeline* p = nullptr;

  hipError_t init(hipStream_t s, tlp_pipeline* pipe) {
    main = s;
    p = pipe;
    hipError_t e = hipEventRecord(p->ev[2 * p->max_layers], main);
    if (e != hipSuccess) return e;
    return hipStreamWaitEvent(p->second, p->ev[2 * p->max_layers], 0);
  }
  hipEvent_t kv_event(int parity, int layer) const { return p->ev[parity * p->max_layers + layer]; }
  ~ChunkPipe() {
    if (!p) return;
    hipEvent_t end = p->ev[2 * p->max_layers + 1];
    if (hipEventRecord(end, p->second) == hipSuccess) (void)hipStreamWaitEvent(main, end, 0);
  }
};

}  // namespace

// Workspace of tlp_prefill_layer_noalloc: one static array per GPU, held by
// the loaded library until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the device
// symbol); it looks up the array's device address once per GPU and uses that.
static __device__ __align__(256) char scratch[TLP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
char* g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];

// Device address of `scratch` on GPU `dev`, looked up with that GPU current
// the first time (the caller's current device is restored).
hipError_t scratch_on_device(int dev, char** out) {
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e == hipSuccess && prev != dev) e = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (prev >= 0 && prev != dev) {
      const hipError_t e2 = hipSetDevice(prev);
      if (e == hipSuccess) e = e2;
    }
    g_scratch_err[dev] = e;
    g_scratch_ptr[dev] = e == hipSuccess ? static_cast<char*>(ptr) : nullptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace

extern "C" {

size_t tlp_workspace_bytes(const tlp_config* cfg, int32_t max_tokens) {
  if (check_config(cfg) != TLP_OK || max_tokens <= 0) return 0;
  return layout_of(*cfg, max_tokens).total;
}

tlp_status tlp_workspace_layout(const tlp_config* cfg, int32_t max_tokens, size_t* offsets) {
  tlp_status s = check_config(cfg);
  if (s != TLP_OK) return s;
  if (!offsets) return fail(TLP_ERR_NULL, "offsets is NULL");
  if (max_tokens <= 0) return fail(TLP_ERR_SHAPE, "max_tokens must be > 0");
  const Layout L = layout_of(*cfg, max_tokens);
  for (int i = 0; i < TLP_WS_COUNT; ++i) offsets[i] = L.off[i];
  return TLP_OK;
}

tlp_status tlp_rope_table(double theta, int32_t head_dim, int32_t n_pos, float* cos_host,
                          float* sin_host) {
  if (!cos_host || !sin_host) return fail(TLP_ERR_NULL, "table pointers are NULL");
  if (head_dim <= 0 || head_dim % 2 || n_pos <= 0)
    return fail(TLP_ERR_SHAPE, "head_dim must be even and positive, n_pos positive");
  if (!(theta > 0.0) || !std::isfinite(theta)) return fail(TLP_ERR_SHAPE, "theta must be > 0");
  const int half = head_dim / 2;
  for (int i = 0; i < half; ++i) {
    const double f = std::pow(theta, -2.0 * i / head_dim);
    for (int p = 0; p < n_pos; ++p) {
      const double ang = static_cast<double>(p) * f;
      cos_host[static_cast<size_t>(p) * half + i] = static_cast<float>(std::cos(ang));
      sin_host[static_cast<size_t>(p) * half + i] = static_cast<float>(std::sin(ang));
    }
  }
  return TLP_OK;
}

tlp_status tlp_prefill_layer(const tlp_config* cfg, const tlp_layer_weights* weights,
                             int32_t layer, void* hidden, int32_t n_tokens,
                             int32_t start_position, void* k_cache, void* v_cache,
                             const float* rope_cos, const float* rope_sin, void* workspace,
                             size_t workspace_bytes, void* stream) {
  tlp_status s = check_config(cfg);
  if (s != TLP_OK) return s;
  if (layer < 0 || layer >= cfg->n_layers)
    return fail(TLP_ERR_SHAPE, "layer %d outside [0, %d)", layer, cfg->n_layers);
  if ((s = check_layer_weights(*cfg, weights, layer)) != TLP_OK) return s;
  if ((s = check_call(*cfg, hidden, n_tokens, start_position, k_cache, v_cache, rope_cos,
                      rope_sin, workspace, workspace_bytes, n_tokens > 0 ? n_tokens : 1)) != TLP_OK)
    return s;
  const Layout L = layout_of(*cfg, n_tokens);
  hipStream_t st = static_cast<hipStream_t>(stream);
  g_last_error.clear();
  int parts = 0;
  return run_layer(*cfg, *weights, layer, n_tokens, start_position, hidden, false, 0, hidden,
                   &parts, static_cast<char*>(k_cache), static_cast<char*>(v_cache), rope_cos,
                   rope_sin, static_cast<char*>(workspace), L, st);
}

tlp_status tlp_prefill_layer_noalloc(const tlp_config* cfg, const tlp_layer_weights* weights,
                                     int32_t layer, void* hidden, int32_t n_tokens,
                                     int32_t start_position, void* k_cache, void* v_cache,
                                     const float* rope_cos, const float* rope_sin, void* stream) {
  tlp_status s = check_config(cfg);
  if (s != TLP_OK) return s;
  if (layer < 0 || layer >= cfg->n_layers)
    return fail(TLP_ERR_SHAPE, "layer %d outside [0, %d)", layer, cfg->n_layers);
  if ((s = check_layer_weights(*cfg, weights, layer)) != TLP_OK) return s;
  if (n_tokens <= 0) return fail(TLP_ERR_SHAPE, "n_tokens %d must be > 0", n_tokens);
  const Layout L = layout_of(*cfg, n_tokens);
  if (L.total > TLP_NOALLOC_SCRATCH_BYTES)
    return fail(TLP_ERR_WORKSPACE,
                "%d tokens need %zu bytes of workspace, above the %u-byte static scratch of "
                "tlp_prefill_layer_noalloc (use tlp_prefill_layer with a workspace)",
                n_tokens, L.total, TLP_NOALLOC_SCRATCH_BYTES);
  hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = -1;
  hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  char* ws = nullptr;
  if (e == hipSuccess) e = scratch_on_device(dev, &ws);
  if (e != hipSuccess)
    return fail(TLP_ERR_HIP, "scratch of device %d: %s", dev, hipGetErrorString(e));
  if ((s = check_call(*cfg, hidden, n_tokens, start_position, k_cache, v_cache, rope_cos,
                      rope_sin, ws, TLP_NOALLOC_SCRATCH_BYTES, n_tokens)) != TLP_OK)
    return s;
  g_last_error.clear();
  int parts = 0;
  return run_layer(*cfg, *weights, layer, n_tokens, start_position, hidden, false, 0, hidden,
                   &parts, static_cast<char*>(k_cache), static_cast<char*>(v_cache), rope_cos,
                   rope_sin, ws, L, st);
}

tlp_status tlp_prefill_chunk(const tlp_config* cfg, const tlp_layer_weights* layers,
                             void* hidden, int32_t n_tokens, int32_t start_position,
                             int32_t micro_batch, void* k_cache, void* v_cache,
                             const float* rope_cos, const float* rope_sin,
                             const void* final_norm, const void* lm_head, int32_t vocab,
                             float final_eps, float* logits, void* workspace,
                             size_t workspace_bytes, tlp_pipeline* pipeline, void* stream) {
  tlp_status s = check_config(cfg);
  if (s != TLP_OK) return s;
  if (!layers) return fail(TLP_ERR_NULL, "layers is NULL");
  for (int l = 0; l < cfg->n_layers; ++l)
    if ((s = check_layer_weights(*cfg, &layers[l], l)) != TLP_OK) return s;
  if (micro_batch <= 0) return fail(TLP_ERR_SHAPE, "micro_batch %d must be > 0", micro_batch);
  const int mb = n_tokens < micro_batch ? n_tokens : micro_batch;
  if ((s = check_call(*cfg, hidden, n_tokens, start_position, k_cache, v_cache, rope_cos,
                      rope_sin, workspace, workspace_bytes, mb > 0 ? mb : 1)) != TLP_OK)
    return s;
  if (lm_head) {
    if (!final_norm || !logits) return fail(TLP_ERR_NULL, "lm_head needs final_norm and logits");
    if (vocab <= 0) return fail(TLP_ERR_SHAPE, "vocab %d must be > 0", vocab);
    if (!aligned16(lm_head) || !aligned16(final_norm))
      return fail(TLP_ERR_UNSUPPORTED, "lm_head and final_norm must be 16-byte aligned");
    if (!(final_eps >= 0.f) || !std::isfinite(final_eps))
      return fail(TLP_ERR_SHAPE, "final_eps must be finite and >= 0");
  }
  using namespace tlp;
  const Act act = cfg->dtype == TLP_F32 ? Act::F32 : Act::BF16;
  const Layout L = layout_of(*cfg, mb);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const size_t row_bytes = static_cast<size_t>(cfg->hidden) * elt_size(*cfg);
  g_last_error.clear();
  // With room for two workspaces, micro-batch b uses half b % 2 and the odd
  // micro-batches run on a second stream, each layer's attention waiting for
  // the previous micro-batch's K/V of that layer: consecutive micro-batches
  // overlap, one layer apart.
  const int n_mb = (n_tokens + mb - 1) / mb;
  bool pipelined = pipeline && n_mb > 1 && workspace_bytes / 2 >= L.total;
  if (pipelined) {
    if (pipeline->max_layers < cfg->n_layers)
      return fail(TLP_ERR_SHAPE, "pipeline made for %d layers, the config has %d",
                  pipeline->max_layers, cfg->n_layers);
    int dev = -1;
    const hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return fail(TLP_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
    if (dev != pipeline->device)
      return fail(TLP_ERR_UNSUPPORTED, "pipeline made on device %d, the stream is on device %d",
                  pipeline->device, dev);
    // a stream being captured into a graph gets the one-stream order: the
    // call then enqueues kernels on it only
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
      pipelined = false;
  }
  {
    ChunkPipe pipe;
    if (pipelined) {
      const hipError_t e = pipe.init(st, pipeline);
      if (e != hipSuccess)
        return fail(TLP_ERR_HIP, "starting the second stream: %s", hipGetErrorString(e));
    }
    for (int b = 0; b < n_mb; ++b) {
      const int off = b * mb;
      const int m = n_tokens - off < mb ? n_tokens - off : mb;
      const int half = pipelined ? (b & 1) : 0;
      hipStream_t sb = half ? pipeline->second : st;
      char* wsb = ws + half * L.total;
      char* rows = static_cast<char*>(hidden) + static_cast<size_t>(off) * row_bytes;
      int parts = 0;
      for (int l = 0; l < cfg->n_layers; ++l) {
        const bool first = l == 0, last = l == cfg->n_layers - 1;
        s = run_layer(*cfg, layers[l], l, m, start_position + off,
                      first ? static_cast<const void*>(rows) : wsb + L.off[TLP_WS_RES], !first,
                      parts, last ? rows : nullptr, &parts, static_cast<char*>(k_cache),
                      static_cast<char*>(v_cache), rope_cos, rope_sin, wsb, L, sb,
                      pipelined ? pipe.kv_event(half, l) : nullptr,
                      pipelined && b > 0 ? pipe.kv_event(half ^ 1, l) : nullptr);
        if (s != TLP_OK) return s;
      }
    }
  }   // the second stream is joined into st here
  if (lm_head) {
    hipStream_t s = st;
    const char* last_row = static_cast<char*>(hidden) + static_cast<size_t>(n_tokens - 1) * row_bytes;
    float* xh = reinterpret_cast<float*>(ws + L.off[TLP_WS_HEAD]);
    RowArgs r{};
    r.x = last_row; r.x_f32 = 0; r.ldx = cfg->hidden;
    r.gain = final_norm; r.norm_out = xh; r.norm_f32 = 1;
    r.rows = 1; r.H = cfg->hidden; r.eps = final_eps;
    TLP_LAUNCH(TLP_K_FINAL_NORM, launch_rownorm(act, r, s));
    TLP_LAUNCH(TLP_K_LM_HEAD, launch_lm_head(act, xh, lm_head, logits, vocab, cfg->hidden, s));
  }
  return TLP_OK;
}

tlp_status tlp_pipeline_create(int32_t max_layers, tlp_pipeline** out) {
  if (!out) return fail(TLP_ERR_NULL, "out is NULL");
  *out = nullptr;
  if (max_layers <= 0) return fail(TLP_ERR_SHAPE, "max_layers %d must be > 0", max_layers);
  tlp_pipeline* p = new (std::nothrow) tlp_pipeline();
  if (!p) return fail(TLP_ERR_HIP, "out of host memory");
  p->max_layers = max_layers;
  hipError_t e = hipGetDevice(&p->device);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&p->second, hipStreamNonBlocking);
  if (e == hipSuccess) {
    p->ev.assign(2 * static_cast<size_t>(max_layers) + 2, nullptr);
    for (hipEvent_t& x : p->ev)
      if ((e = hipEventCreateWithFlags(&x, hipEventDisableTiming)) != hipSuccess) break;
  }
  if (e != hipSuccess) {
    tlp_pipeline_destroy(p);
    return fail(TLP_ERR_HIP, "pipeline resources: %s", hipGetErrorString(e));
  }
  *out = p;
  return TLP_OK;
}

tlp_status tlp_pipeline_destroy(tlp_pipeline* p) {
  if (!p) return TLP_OK;
  hipError_t first = hipSuccess;
  if (p->second) first = hipStreamSynchronize(p->second);
  for (hipEvent_t x : p->ev)
    if (x) {
      const hipError_t e = hipEventDestroy(x);
      if (first == hipSuccess) first = e;
    }
  if (p->second) {
    const hipError_t e = hipStreamDestroy(p->second);
    if (first == hipSuccess) first = e;
  }
  delete p;
  if (first != hipSuccess) return fail(TLP_ERR_HIP, "pipeline release: %s", hipGetErrorString(first));
  return TLP_OK;
}

tlp_status tlp_argmax_rows(const float* logits, int32_t rows, int32_t vocab, int64_t ld,
                           int32_t* token_ids, void* stream) {
  if (!logits || !token_ids) return fail(TLP_ERR_NULL, "logits and token_ids are required");
  if (rows <= 0 || vocab <= 0) return fail(TLP_ERR_SHAPE, "rows %d and vocab %d must be > 0",
                                           rows, vocab);
  if (ld < vocab) return fail(TLP_ERR_SHAPE, "ld %lld below vocab %d",
                              static_cast<long long>(ld), vocab);
  g_last_error.clear();
  hipStream_t s = static_cast<hipStream_t>(stream);
  TLP_LAUNCH(TLP_K_ARGMAX, tlp::launch_argmax_rows(logits, rows, vocab, static_cast<size_t>(ld),
                                                   token_ids, s));
  return TLP_OK;
}

size_t tlp_verify_workspace_bytes(const tlp_config* cfg, int32_t n_rows) {
  if (check_config(cfg) != TLP_OK || n_rows <= 0) return 0;
  return align256(static_cast<size_t>(n_rows) * cfg->hidden * elt_size(*cfg));
}

tlp_status tlp_verify_tail(const tlp_config* cfg, const void* hidden, int32_t n_rows,
                           const void* final_norm, const void* lm_head, int32_t vocab,
                           float final_eps, float* logits, int32_t* token_ids, void* workspace,
                           size_t workspace_bytes, void* stream) {
  tlp_status st = check_config(cfg);
  if (st != TLP_OK) return st;
  if (!hidden || !final_norm || !lm_head || !logits || !workspace)
    return fail(TLP_ERR_NULL, "hidden, final_norm, lm_head, logits and workspace are required");
  if (n_rows <= 0 || vocab <= 0)
    return fail(TLP_ERR_SHAPE, "n_rows %d and vocab %d must be > 0", n_rows, vocab);
  if (!(final_eps >= 0.f) || !std::isfinite(final_eps))
    return fail(TLP_ERR_SHAPE, "final_eps must be finite and >= 0");
  if (!aligned16(hidden) || !aligned16(final_norm) || !aligned16(lm_head) || !aligned16(logits))
    return fail(TLP_ERR_UNSUPPORTED, "hidden, final_norm, lm_head and logits must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(TLP_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  const size_t need = tlp_verify_workspace_bytes(cfg, n_rows);
  if (workspace_bytes < need)
    return fail(TLP_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  using namespace tlp;
  const Act act = cfg->dtype == TLP_F32 ? Act::F32 : Act::BF16;
  const int H = cfg->hidden;
  hipStream_t s = static_cast<hipStream_t>(stream);
  g_last_error.clear();
  // final RMSNorm of every row
  RowArgs r{};
  r.x = hidden; r.x_f32 = 0; r.ldx = H;
  r.gain = final_norm; r.norm_out = workspace; r.norm_f32 = 0;
  r.rows = n_rows; r.H = H; r.eps = final_eps;
  TLP_LAUNCH(TLP_K_FINAL_NORM, launch_rownorm(act, r, s));
  // LM head: fp32 logits [n_rows][vocab]
  if (act == Act::BF16 && n_rows <= kSkinnyMaxM) {
    TLP_LAUNCH(TLP_K_LM_HEAD, launch_gemm_skinny(workspace, H, lm_head, nullptr, n_rows, vocab, H, logits,
                                                 vocab, 0, 1, s));
  } else {
    GemmCall g{};
    g.act = act;
    g.A = workspace; g.lda = H;
    g.W = lm_head;
    g.M = n_rows; g.N = vocab; g.K = H;
    g.epi = Epi::StoreF32; g.out = logits; g.ldo = vocab; g.out_f32 = true;
    TLP_LAUNCH(TLP_K_LM_HEAD, launch_gemm(g, s));
  }
  if (token_ids)
    TLP_LAUNCH(TLP_K_ARGMAX, launch_argmax_rows(logits, n_rows, vocab, vocab, token_ids, s));
  return TLP_OK;
}

tlp_status tlp_profile_begin(int32_t max_launches) {
  if (max_launches <= 0) return fail(TLP_ERR_SHAPE, "max_launches %d must be > 0", max_launches);
  prof_release();
  g_prof_dropped = 0;
  g_prof.assign(static_cast<size_t>(max_launches), ProfRecord{-1, nullptr, nullptr});
  for (ProfRecord& r : g_prof) {
    hipError_t e = hipEventCreate(&r.start);
    if (e == hipSuccess) e = hipEventCreate(&r.stop);
    if (e != hipSuccess) {
      prof_release();
      return fail(TLP_ERR_HIP, "profile events: %s", hipGetErrorString(e));
    }
  }
  g_prof_on = true;
  return TLP_OK;
}

tlp_status tlp_profile_end(double* total_ms, int32_t* launches, int32_t* not_timed) {
  if (!total_ms || !launches) return fail(TLP_ERR_NULL, "output arrays are NULL");
  g_prof_on = false;
  for (int k = 0; k < TLP_K_COUNT; ++k) {
    total_ms[k] = 0.0;
    launches[k] = 0;
  }
  tlp_status st = TLP_OK;
  for (size_t i = 0; i < g_prof_used; ++i) {
    const ProfRecord& r = g_prof[i];
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess && st == TLP_OK)
      st = fail(TLP_ERR_HIP, "profile events: %s", hipGetErrorString(e));
    total_ms[r.kernel] += ms;
    launches[r.kernel] += 1;
  }
  if (not_timed) *not_timed = g_prof_dropped;
  prof_release();
  return st;
}

const char* tlp_status_string(tlp_status status) {
  switch (status) {
    case TLP_OK: return "ok";
    case TLP_ERR_NULL: return "null pointer";
    case TLP_ERR_SHAPE: return "invalid shape";
    case TLP_ERR_POSITION: return "position out of range";
    case TLP_ERR_UNSUPPORTED: return "unsupported configuration";
    case TLP_ERR_WORKSPACE: return "workspace too small or misaligned";
    case TLP_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* tlp_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
