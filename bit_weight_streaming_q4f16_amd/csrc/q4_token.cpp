// Decode tokens end to end: the decode loop of the Zero TVM documentation
// ("Decode loop") over q4f16_1 weights, with attention at a single position.
//
// One step is a fixed sequence of operations: embedding row, RMSNorm, then per
// block qkv, o (reading the value part of qkv), residual add + RMSNorm, gate/up,
// SiLU-multiply, down, residual add + RMSNorm, then the LM head and the argmax.
// Each projection is one GEMV kernel (one kernel per GEMV is the faster choice
// for a chain in which every GEMV waits for the one before it).  Where gate/up
// needs no split-K pass the glue runs inside it, and every residual add + RMSNorm
// runs inside the GEMV it feeds (q4_fused.h): four kernels per block instead of
// seven, with bitwise the same results (the separate norm kernel where a GEMV
// needs split-K or its staging does not fit LDS).  With the model option
// Q4_MODEL_FACTORED_NORM the norm is folded in factored form instead: no
// reduction before the staging, results within rounding of the defined step, not
// bitwise.  Every buffer between the kernels lives in the caller's workspace; the
// residual alternates between two buffers.  A multi-step decode keeps its tokens
// on the device: the embedding kernel takes the step's token from the caller's
// token array at a device-side counter, and the argmax kernel writes the next one
// there and advances the counter; one step is captured as a HIP graph and
// replayed: no host round trip between tokens (the pages' host-side lever is to
// submit a whole token in one command; here several tokens go per host call).
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "q4f16.h"
#include "q4_fused.h"
#include "q4_internal.h"
#include "q4_tok.h"

namespace {

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

// Byte offsets in the workspace: split-K partials first, then the activations,
// then the token bookkeeping (int32: current token, next token, counter).
struct Layout {
  q4::GemvPlan qkv, o, gate_up, down, lm_head;
  bool fuse = false;       // the glue inside the gate/up GEMV (no split-K pass in it)
  size_t res = 0, res2 = 0, h = 0, qkv_out = 0, attn = 0, gu = 0, hf = 0, dn = 0, logits = 0,
         tok = 0;
  size_t bytes = 0;
};

Layout layout_for(const q4::DeviceInfo& d, const q4_model& m) {
  Layout L;
  L.qkv = q4::plan_auto(d, 1, 3 * m.D, m.D);
  L.o = q4::plan_auto(d, 1, m.D, m.D);
  L.gate_up = q4::plan_auto(d, 1, 2 * m.F, m.D);
  L.down = q4::plan_auto(d, 1, m.D, m.F);
  L.lm_head = q4::plan_auto(d, 1, m.V, m.D);
  L.fuse = L.gate_up.splits == 1;
  size_t off = up256(std::max({L.qkv.ws_bytes, L.o.ws_bytes, L.gate_up.ws_bytes,
                               L.down.ws_bytes, L.lm_head.ws_bytes}));
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += up256(bytes);
    return o;
  };
  L.res = take(2 * m.D);
  L.res2 = take(2 * m.D);      // the residual's second buffer (it alternates)
  L.h = take(2 * m.D);
  L.qkv_out = take(2 * 3 * m.D);
  L.attn = take(2 * m.D);
  L.gu = take(2 * 2 * m.F);
  L.hf = take(2 * m.F);
  L.dn = take(2 * m.D);
  L.logits = take(2 * m.V);
  L.tok = take(16);            // int32: current token, next token, step counter
  L.bytes = off;
  return L;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_weight(const char* what, const q4_weight& w, int64_t N, int64_t K) {
  if (!w.words || !w.scales) return q4::api_fail(Q4_ERR_NULL, "%s: NULL weight pointer", what);
  if (w.N != N || w.K != K)
    return q4::api_fail(Q4_ERR_SHAPE, "%s: shape [%lld][%lld], expected [%lld][%lld]", what,
                        (long long)w.N, (long long)w.K, (long long)N, (long long)K);
  if (!aligned(w.words, 16) || !aligned(w.scales, 2))
    return q4::api_fail(Q4_ERR_ALIGN, "%s: words must be 16-byte, scales 2-byte aligned", what);
  return Q4_OK;
}

int check_gamma(const char* what, const uint16_t* g) {
  if (!g) return q4::api_fail(Q4_ERR_NULL, "%s is NULL", what);
  if (!aligned(g, 16)) return q4::api_fail(Q4_ERR_ALIGN, "%s not 16-byte aligned", what);
  return Q4_OK;
}

int check_model(const q4_model* m) {
  if (!m) return q4::api_fail(Q4_ERR_NULL, "model is NULL");
  if (m->n_blocks < 0 || (m->n_blocks > 0 && !m->blocks))
    return q4::api_fail(Q4_ERR_SHAPE, "n_blocks = %lld with blocks %p", (long long)m->n_blocks,
                        (const void*)m->blocks);
  if (m->D < 32 || m->D % 32 || m->F < 32 || m->F % 32 || m->V < 1)
    return q4::api_fail(Q4_ERR_SHAPE, "D = %lld, F = %lld, V = %lld: D and F must be positive "
                        "multiples of 32, V >= 1", (long long)m->D, (long long)m->F,
                        (long long)m->V);
  if (m->D > (1 << 20) || m->F > (1 << 20) || m->V > INT32_MAX)
    return q4::api_fail(Q4_ERR_UNSUPPORTED, "D, F or V too large");
  if (!(m->eps >= 0.f)) return q4::api_fail(Q4_ERR_SHAPE, "eps must be >= 0");
  if (m->options & ~Q4_MODEL_FACTORED_NORM)
    return q4::api_fail(Q4_ERR_SHAPE, "options = 0x%x: unknown bits", m->options);
  if (int rc = check_weight("embed", m->embed, m->V, m->D)) return rc;
  if (int rc = check_weight("lm_head", m->lm_head, m->V, m->D)) return rc;
  if (int rc = check_gamma("final_norm", m->final_norm)) return rc;
  char what[64];
  for (int64_t b = 0; b < m->n_blocks; ++b) {
    const q4_block& B = m->blocks[b];
    snprintf(what, sizeof what, "blocks[%lld].qkv", (long long)b);
    if (int rc = check_weight(what, B.qkv, 3 * m->D, m->D)) return rc;
    snprintf(what, sizeof what, "blocks[%lld].o", (long long)b);
    if (int rc = check_weight(what, B.o, m->D, m->D)) return rc;
    snprintf(what, sizeof what, "blocks[%lld].gate_up", (long long)b);
    if (int rc = check_weight(what, B.gate_up, 2 * m->F, m->D)) return rc;
    snprintf(what, sizeof what, "blocks[%lld].down", (long long)b);
    if (int rc = check_weight(what, B.down, m->D, m->F)) return rc;
    snprintf(what, sizeof what, "blocks[%lld].attn_norm", (long long)b);
    if (int rc = check_gamma(what, B.attn_norm)) return rc;
    snprintf(what, sizeof what, "blocks[%lld].ffn_norm", (long long)b);
    if (int rc = check_gamma(what, B.ffn_norm)) return rc;
  }
  return Q4_OK;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (!ws) return q4::api_fail(Q4_ERR_WORKSPACE, "needs %zu workspace bytes, ws is NULL", need);
  if (have < need)
    return q4::api_fail(Q4_ERR_WORKSPACE, "needs %zu workspace bytes, got %zu", need, have);
  if (!aligned(ws, 16)) return q4::api_fail(Q4_ERR_ALIGN, "ws not 16-byte aligned");
  return Q4_OK;
}

// Enqueue one decode step: token tok_in[0] -> tok_out[0] (and the logits).
hipError_t enqueue_step(const q4::DeviceInfo& d, const q4_model& m, const Layout& L,
                        const int32_t* tok_in, int32_t* tok_out, uint16_t* logits, uint8_t* ws,
                        hipStream_t s, int32_t* seq = nullptr, int32_t* counter = nullptr) {
  auto buf = [&](size_t off) { return reinterpret_cast<uint16_t*>(ws + off); };
  uint16_t *res = buf(L.res), *h = buf(L.h), *qkv = buf(L.qkv_out), *gu = buf(L.gu);
  uint16_t *attn = buf(L.attn), *hf = buf(L.hf), *dn = buf(L.dn);
  uint16_t* lg = logits ? logits : buf(L.logits);
  auto gemv = [&](const q4_weight& w, const q4::GemvPlan& p, const uint16_t* x, uint16_t* y) {
    const q4::GemvArgs a{w.words, w.scales, x, y, 1, w.N, w.K};
    return q4::launch_gemv(d, a, p, ws, s);
  };
#define Q4_TRY(call)                          \
  do {                                        \
    if (hipError_t e_ = (call)) return e_;    \
  } while (0)
  Q4_TRY(q4::launch_embed_rows(m.embed.words, m.embed.scales, m.V, m.D, tok_in, 1, res, s, seq,
                               counter));
  // Every residual add + RMSNorm is folded into the GEMV it feeds (q4_fused.h)
  // where that GEMV runs as one K slice: exact (the default: bitwise the norm
  // kernel followed by the GEMV) when the staging fits LDS, else as the separate
  // norm kernel; factored (Q4_MODEL_FACTORED_NORM) always.  The residual
  // alternates between two buffers (a folded GEMV's workgroups all read the old
  // one while one of them writes the new one).
  const bool factored = (m.options & Q4_MODEL_FACTORED_NORM) != 0;
  const bool exact_fits = (size_t)(m.D / 32) * 192 <= d.lds_per_block;
  uint16_t *cur = res, *other = buf(L.res2);
  q4::NormIn pend;                  // the add + norm that the next normed GEMV applies
  pend.gamma = m.n_blocks ? m.blocks[0].attn_norm : m.final_norm;
  pend.eps = m.eps;
  pend.exact = !factored;
  // y = W . RMSNorm(pending residual); glu: the gate/up GEMV with the glue (y = hf)
  auto normed = [&](const q4_weight& w, const q4::GemvPlan& p, uint16_t* y, int64_t n_out,
                    bool glu) {
    q4::NormIn a = pend;
    a.res_in = cur;
    a.res_out = pend.delta ? other : nullptr;
    hipError_t e;
    if (factored || (p.splits == 1 && exact_fits)) {
      e = q4::launch_gemv_norm_in(d, w.words, w.scales, a, y, n_out, w.K, glu, s);
    } else {
      e = q4::launch_rmsnorm(a.delta, a.res_in, a.gamma, m.eps, 1, m.D, a.res_out, h, s);
      if (e == hipSuccess && !glu) e = gemv(w, p, h, y);
      if (e == hipSuccess && glu && L.fuse)
        e = q4::launch_gemv_glu(d, w.words, w.scales, h, y, m.F, m.D, p, s);
      if (e == hipSuccess && glu && !L.fuse) {
        e = gemv(w, p, h, gu);
        if (e == hipSuccess) e = q4::launch_silu_mul(gu, y, 1, m.F, s);
      }
    }
    if (pend.delta) std::swap(cur, other);
    return e;
  };
  for (int64_t b = 0; b < m.n_blocks; ++b) {
    const q4_block& B = m.blocks[b];
    const uint16_t* next = b + 1 < m.n_blocks ? m.blocks[b + 1].attn_norm : m.final_norm;
    Q4_TRY(normed(B.qkv, L.qkv, qkv, 3 * m.D, false));
    // attention at a single position: its output is the value vector
    Q4_TRY(gemv(B.o, L.o, qkv + 2 * m.D, attn));
    pend.delta = attn;
    pend.gamma = B.ffn_norm;
    Q4_TRY(normed(B.gate_up, L.gate_up, hf, m.F, true));
    Q4_TRY(gemv(B.down, L.down, hf, dn));
    pend.delta = dn;
    pend.gamma = next;
  }
  Q4_TRY(normed(m.lm_head, L.lm_head, lg, m.V, false));
  Q4_TRY(q4::launch_argmax(lg, 1, m.V, tok_out, s, seq, counter));
#undef Q4_TRY
  return hipSuccess;
}

// ---------------------------------------------------------------- graphs

}  // namespace

// A captured decode step (the handle of include/q4f16.h): tokens[counter] ->
// tokens[counter + 1], the counter kept in the workspace.
struct q4_tokens_graph {
  hipGraphExec_t exec = nullptr;
  int device = -1;
  int32_t* counter = nullptr;        // device: the step counter in the workspace
};

namespace {

int device_error(hipError_t e, const char* what) {
  return q4::api_fail(Q4_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

size_t q4_decode_token_workspace_bytes(const q4_model* model) {
  if (check_model(model)) return 0;
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return 0;
  return layout_for(*d, *model).bytes;
}

int q4_decode_token(const q4_model* model, const int32_t* token_in, int32_t* token_out,
                    uint16_t* logits, void* ws, size_t ws_bytes, q4_stream_t stream) {
  if (int rc = check_model(model)) return q4::api_fail(rc, "q4_decode_token: %s", q4_last_error());
  if (!token_in || !token_out)
    return q4::api_fail(Q4_ERR_NULL, "q4_decode_token: token pointer is NULL");
  if (!aligned(token_in, 4) || !aligned(token_out, 4) || (logits && !aligned(logits, 2)))
    return q4::api_fail(Q4_ERR_ALIGN, "q4_decode_token: misaligned token or logits pointer");
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return q4::api_fail(Q4_ERR_DEVICE, "q4_decode_token: no HIP device");
  const Layout L = layout_for(*d, *model);
  if (int rc = check_ws(ws, ws_bytes, L.bytes))
    return q4::api_fail(rc, "q4_decode_token: %s", q4_last_error());
  hipError_t e = enqueue_step(*d, *model, L, token_in, token_out, logits,
                              static_cast<uint8_t*>(ws), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? q4::api_ok() : device_error(e, "q4_decode_token");
}

int q4_decode_tokens(const q4_model* model, int32_t* tokens, int64_t steps, void* ws,
                     size_t ws_bytes, q4_stream_t stream) {
  if (int rc = check_model(model)) return q4::api_fail(rc, "q4_decode_tokens: %s", q4_last_error());
  if (!tokens) return q4::api_fail(Q4_ERR_NULL, "q4_decode_tokens: tokens is NULL");
  if (!aligned(tokens, 4)) return q4::api_fail(Q4_ERR_ALIGN, "q4_decode_tokens: tokens misaligned");
  if (steps < 0 || steps > INT32_MAX - 1)
    return q4::api_fail(Q4_ERR_SHAPE, "q4_decode_tokens: steps = %lld", (long long)steps);
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return q4::api_fail(Q4_ERR_DEVICE, "q4_decode_tokens: no HIP device");
  const Layout L = layout_for(*d, *model);
  if (int rc = check_ws(ws, ws_bytes, L.bytes))
    return q4::api_fail(rc, "q4_decode_tokens: %s", q4_last_error());
  if (steps == 0) return q4::api_ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* w = static_cast<uint8_t*>(ws);
  int32_t* tok = reinterpret_cast<int32_t*>(w + L.tok);
  hipError_t e = q4::launch_counter_reset(tok + 2, s);
  for (int64_t i = 0; i < steps && e == hipSuccess; ++i)
    e = enqueue_step(*d, *model, L, tok, tok + 1, nullptr, w, s, tokens, tok + 2);
  return e == hipSuccess ? q4::api_ok() : device_error(e, "q4_decode_tokens");
}

int q4_tokens_graph_create(const q4_model* model, int32_t* tokens, void* ws, size_t ws_bytes,
                           q4_stream_t stream, q4_tokens_graph** out) {
  const char* what = "q4_tokens_graph_create";
  if (!out) return q4::api_fail(Q4_ERR_NULL, "%s: out is NULL", what);
  *out = nullptr;
  if (int rc = check_model(model)) return q4::api_fail(rc, "%s: %s", what, q4_last_error());
  if (!tokens) return q4::api_fail(Q4_ERR_NULL, "%s: tokens is NULL", what);
  if (!aligned(tokens, 4)) return q4::api_fail(Q4_ERR_ALIGN, "%s: tokens misaligned", what);
  if (!stream)
    return q4::api_fail(Q4_ERR_SHAPE, "%s: the null stream cannot be captured; pass a stream",
                        what);
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return q4::api_fail(Q4_ERR_DEVICE, "%s: no HIP device", what);
  const Layout L = layout_for(*d, *model);
  if (int rc = check_ws(ws, ws_bytes, L.bytes))
    return q4::api_fail(rc, "%s: %s", what, q4_last_error());
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* w = static_cast<uint8_t*>(ws);
  int32_t* tok = reinterpret_cast<int32_t*>(w + L.tok);   // cur, next, counter
  if (hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal))
    return device_error(e, what);
  hipError_t err = enqueue_step(*d, *model, L, tok, tok + 1, nullptr, w, s, tokens, tok + 2);
  hipGraph_t graph = nullptr;
  const hipError_t end = hipStreamEndCapture(s, &graph);
  if (err == hipSuccess) err = end;
  hipGraphExec_t exec = nullptr;
  if (err == hipSuccess) err = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (graph) (void)hipGraphDestroy(graph);
  if (err != hipSuccess) return device_error(err, what);
  q4_tokens_graph* g = new (std::nothrow) q4_tokens_graph;
  if (!g) {
    (void)hipGraphExecDestroy(exec);
    return q4::api_fail(Q4_ERR_DEVICE, "%s: out of host memory", what);
  }
  g->exec = exec;
  g->device = d->id;
  g->counter = tok + 2;
  *out = g;
  return q4::api_ok();
}

int q4_tokens_graph_run(q4_tokens_graph* g, int64_t steps, q4_stream_t stream) {
  const char* what = "q4_tokens_graph_run";
  if (!g || !g->exec) return q4::api_fail(Q4_ERR_NULL, "%s: graph is NULL", what);
  if (steps < 0 || steps > INT32_MAX - 1)
    return q4::api_fail(Q4_ERR_SHAPE, "%s: steps = %lld", what, (long long)steps);
  if (steps == 0) return q4::api_ok();
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = q4::launch_counter_reset(g->counter, s);
  for (int64_t i = 0; i < steps && e == hipSuccess; ++i) e = hipGraphLaunch(g->exec, s);
  return e == hipSuccess ? q4::api_ok() : device_error(e, what);
}

int q4_tokens_graph_destroy(q4_tokens_graph* g) {
  if (!g) return q4::api_ok();
  hipError_t e = g->exec ? hipGraphExecDestroy(g->exec) : hipSuccess;
  delete g;
  return e == hipSuccess ? q4::api_ok() : device_error(e, "q4_tokens_graph_destroy");
}

}  // extern "C"

// ------------------------------------------------- whole-token persistent kernel

namespace {

constexpr uint32_t kTokMagic = 0x51345431u;    // "Q4T1"
constexpr uint32_t kTokVersion = 1;
constexpr int kTokBurstItems = 2;              // items per burst (q4_tok.hip)
constexpr int64_t kTokMaxStepsPerLaunch = 4096;

// The persistent kernel's plan as it sits in the caller's buffer.
struct TokPlan {
  uint32_t magic, version;
  int32_t device, n_blocks;
  const void* ws;
  uint64_t ws_bytes, clear_bytes;
  uint64_t qk_off, logits_off, tags_off, block_stride;   // workspace layout
  uint64_t tv_off, to_off, th_off, td_off;               // within a block's tags
  int64_t D, F, V;
  q4::TokLaunch launch;
};

// Workspace layout: control block, stage table, per block the tagged outputs of
// v (qkv rows 2D..3D), o, the glue (h) and down, then the q/k rows and the logits.
struct TokLayout {
  std::vector<q4::TokStage> stages;
  q4::TokLaunch launch{};
  size_t clear_bytes = 0, qk_off = 0, logits_off = 0, tags_off = 0, block_stride = 0;
  size_t tv = 0, to = 0, th = 0, td = 0, bytes = 0;
};

int tok_lg(int64_t G) {
  int lg = 2;
  while ((4 << lg) < G && lg < 6) ++lg;
  return lg;
}

// The model's shape limits for the persistent kernel; Q4_OK or a status with the
// error text set.
int tok_supported(const char* what, const q4_model& m) {
  if (m.D > 4096 || m.F > 8192)
    return q4::api_fail(Q4_ERR_UNSUPPORTED, "%s: the whole-token kernel takes D <= 4096 and F "
                        "<= 8192 (rows of at most 4 groups per lane), got D = %lld, F = %lld",
                        what, (long long)m.D, (long long)m.F);
  if (m.V > (1 << 24))
    return q4::api_fail(Q4_ERR_UNSUPPORTED, "%s: vocabulary above 2^24", what);
  if (m.n_blocks > 4096)
    return q4::api_fail(Q4_ERR_UNSUPPORTED, "%s: more than 4096 blocks", what);
  return Q4_OK;
}

TokLayout tok_layout(const q4::DeviceInfo& d, const q4_model& m) {
  TokLayout L;
  const int64_t D = m.D, F = m.F, V = m.V, n = m.n_blocks;
  const int grid = d.cus;
  size_t off = 256;                                   // control block
  const size_t table_off = off;
  off += up256((size_t)(4 * n + 1) * sizeof(q4::TokStage));
  L.tags_off = off;
  L.tv = 0;
  L.to = L.tv + up256((size_t)4 * D);
  L.th = L.to + up256((size_t)4 * D);
  L.td = L.th + up256((size_t)4 * F);
  L.block_stride = L.td + up256((size_t)4 * D);
  off += (size_t)n * L.block_stride;
  L.clear_bytes = off;
  L.qk_off = off;
  off += up256((size_t)4 * D);
  L.logits_off = off;
  off += up256((size_t)2 * V);
  L.bytes = off;
  int maxG = 4;
  auto stage = [&](const q4_weight& w, int64_t nout, int flags, const uint16_t* gamma,
                   uint16_t* out, int64_t nplain, size_t tag_in, size_t tag_out) {
    q4::TokStage s{};
    const int64_t G = w.K / 32;
    const int lg = tok_lg(G), lpr = 1 << lg;
    s.W = reinterpret_cast<const uint4*>(w.words);
    s.S = w.scales;
    s.gamma = gamma;
    s.out = out;
    s.rows = (int)w.N;
    s.G = (int)G;
    s.lg = (int16_t)lg;
    s.C = (int16_t)((G + lpr - 1) / lpr);
    s.nout = (int)nout;
    s.flags = flags;
    s.nplain = (int)nplain;
    s.tag_in = (int)tag_in;
    s.tag_out = (int)tag_out;
    const int opb = q4::tok_outputs_per_burst(kTokBurstItems, lg, (flags & q4::kTokGlu) != 0);
    s.nburst = (int)((nout + opb - 1) / opb);
    s.sbase = s.nburst / grid;
    s.srem = s.nburst % grid;
    maxG = std::max(maxG, lpr * (int)s.C);
    L.stages.push_back(s);
  };
  auto tags = [&](int64_t b, size_t part) { return L.tags_off + (size_t)b * L.block_stride + part; };
  for (int64_t b = 0; b < n; ++b) {
    const q4_block& B = m.blocks[b];
    stage(B.qkv, 3 * D, b == 0 ? q4::kTokEmbed : q4::kTokNorm, B.attn_norm, nullptr, 2 * D,
          b == 0 ? 0 : tags(b - 1, L.td), tags(b, L.tv));
    stage(B.o, D, 0, nullptr, nullptr, 0, tags(b, L.tv), tags(b, L.to));
    stage(B.gate_up, F, q4::kTokNorm | q4::kTokGlu, B.ffn_norm, nullptr, 0, tags(b, L.to),
          tags(b, L.th));
    stage(B.down, D, 0, nullptr, nullptr, 0, tags(b, L.th), tags(b, L.td));
  }
  stage(m.lm_head, V, (n == 0 ? q4::kTokEmbed : q4::kTokNorm) | q4::kTokArgmax, m.final_norm,
        nullptr, V, n == 0 ? 0 : tags(n - 1, L.td), 0);
  q4::TokLaunch& T = L.launch;
  T.grid = grid;
  T.stages = (int)L.stages.size();
  T.maxG = maxG;
  T.D = (int)D;
  T.V = (int)V;
  T.burst = kTokBurstItems;
  T.lds_bytes = (uint32_t)q4::tok_lds_bytes(maxG, (int)D);
  T.eps = m.eps;
  T.table_off = table_off;
  T.embed_words = m.embed.words;
  T.embed_scales = m.embed.scales;
  return L;
}

int tok_layout_checked(const char* what, const q4_model* model, TokLayout* out) {
  if (int rc = check_model(model)) return q4::api_fail(rc, "%s: %s", what, q4_last_error());
  if (int rc = tok_supported(what, *model)) return rc;
  const q4::DeviceInfo* d = q4::device_info();
  if (!d) return q4::api_fail(Q4_ERR_DEVICE, "%s: no HIP device", what);
  *out = tok_layout(*d, *model);
  if (out->bytes > (size_t)INT32_MAX)
    return q4::api_fail(Q4_ERR_UNSUPPORTED, "%s: workspace above 2 GiB", what);
  if (out->launch.lds_bytes > d->lds_per_block)
    return q4::api_fail(Q4_ERR_UNSUPPORTED, "%s: needs %u bytes of LDS, the device has %zu",
                        what, out->launch.lds_bytes, d->lds_per_block);
  return Q4_OK;
}

}  // namespace

extern "C" {

size_t q4_tokens_plan_bytes(void) { return sizeof(TokPlan); }

size_t q4_tokens_workspace_bytes(const q4_model* model) {
  TokLayout L;
  if (tok_layout_checked("q4_tokens_workspace_bytes", model, &L)) return 0;
  return L.bytes;
}

int q4_tokens_plan_init(const q4_model* model, void* plan, size_t plan_bytes, void* ws,
                        size_t ws_bytes, q4_stream_t stream) {
  const char* what = "q4_tokens_plan_init";
  TokLayout L;
  if (int rc = tok_layout_checked(what, model, &L)) return rc;
  if (!plan) return q4::api_fail(Q4_ERR_NULL, "%s: plan is NULL", what);
  if (plan_bytes < sizeof(TokPlan))
    return q4::api_fail(Q4_ERR_WORKSPACE, "%s: the plan needs %zu bytes, got %zu", what,
                        sizeof(TokPlan), plan_bytes);
  if (reinterpret_cast<uintptr_t>(plan) % 8)
    return q4::api_fail(Q4_ERR_ALIGN, "%s: plan not 8-byte aligned", what);
  if (int rc = check_ws(ws, ws_bytes, L.bytes)) return q4::api_fail(rc, "%s: %s", what,
                                                                    q4_last_error());
  if (!aligned(ws, 256)) return q4::api_fail(Q4_ERR_ALIGN, "%s: ws not 256-byte aligned", what);
  uint8_t* w = static_cast<uint8_t*>(ws);
  // the q/k rows and the logits go to the workspace
  for (q4::TokStage& s : L.stages) {
    if (s.flags & q4::kTokArgmax) s.out = reinterpret_cast<uint16_t*>(w + L.logits_off);
    else if (s.nplain) s.out = reinterpret_cast<uint16_t*>(w + L.qk_off);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = q4::tok_prepare(L.launch);
  if (e == hipSuccess) e = q4::zero_words(ws, L.clear_bytes / 4, s);
  if (e == hipSuccess)
    e = q4::write_table(w + L.launch.table_off, L.stages.data(),
                        L.stages.size() * sizeof(q4::TokStage), s);
  if (e != hipSuccess) return device_error(e, what);
  TokPlan p{};
  p.magic = kTokMagic;
  p.version = kTokVersion;
  const q4::DeviceInfo* d = q4::device_info();
  p.device = d->id;
  p.n_blocks = (int32_t)model->n_blocks;
  p.ws = ws;
  p.ws_bytes = L.bytes;
  p.clear_bytes = L.clear_bytes;
  p.qk_off = L.qk_off;
  p.logits_off = L.logits_off;
  p.tags_off = L.tags_off;
  p.block_stride = L.block_stride;
  p.tv_off = L.tv;
  p.to_off = L.to;
  p.th_off = L.th;
  p.td_off = L.td;
  p.D = model->D;
  p.F = model->F;
  p.V = model->V;
  p.launch = L.launch;
  memcpy(plan, &p, sizeof p);
  return q4::api_ok();
}

int q4_tokens_run(const void* plan, int32_t* tokens, int64_t steps, uint16_t* logits,
                  q4_stream_t stream) {
  const char* what = "q4_tokens_run";
  if (!plan) return q4::api_fail(Q4_ERR_NULL, "%s: plan is NULL", what);
  TokPlan p;
  memcpy(&p, plan, sizeof p);
  if (p.magic != kTokMagic || p.version != kTokVersion)
    return q4::api_fail(Q4_ERR_SHAPE, "%s: not a plan made by q4_tokens_plan_init", what);
  if (!tokens) return q4::api_fail(Q4_ERR_NULL, "%s: tokens is NULL", what);
  if (!aligned(tokens, 4) || (logits && !aligned(logits, 2)))
    return q4::api_fail(Q4_ERR_ALIGN, "%s: misaligned tokens or logits", what);
  if (steps < 0 || steps > INT32_MAX - 1)
    return q4::api_fail(Q4_ERR_SHAPE, "%s: steps = %lld", what, (long long)steps);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != p.device)
    return q4::api_fail(Q4_ERR_DEVICE, "%s: the plan is for device %d, the current one is %d",
                        what, p.device, dev);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  // launches of at most kTokMaxStepsPerLaunch steps (the kernel's counters are
  // 32-bit); the token array chains them
  for (int64_t t0 = 0; t0 < steps && e == hipSuccess; t0 += kTokMaxStepsPerLaunch) {
    const int n = (int)std::min<int64_t>(kTokMaxStepsPerLaunch, steps - t0);
    e = q4::launch_tokens(p.launch, const_cast<void*>(p.ws), tokens + t0, n, logits, s);
  }
  return e == hipSuccess ? q4::api_ok() : device_error(e, what);
}

int64_t q4_tokens_ws_offset(const void* plan, uint32_t what, int64_t block) {
  if (!plan) return -1;
  TokPlan p;
  memcpy(&p, plan, sizeof p);
  if (p.magic != kTokMagic || p.version != kTokVersion) return -1;
  if (what == Q4_TOKENS_QK) return (int64_t)p.qk_off;
  if (what == Q4_TOKENS_LOGITS) return (int64_t)p.logits_off;
  if (block < 0 || block >= p.n_blocks) return -1;
  const uint64_t b = p.tags_off + (uint64_t)block * p.block_stride;
  switch (what) {
    case Q4_TOKENS_V: return (int64_t)(b + p.tv_off);
    case Q4_TOKENS_O: return (int64_t)(b + p.to_off);
    case Q4_TOKENS_H: return (int64_t)(b + p.th_off);
    case Q4_TOKENS_DOWN: return (int64_t)(b + p.td_off);
    default: return -1;
  }
}

}  // extern "C"
