// Host side of the libsks C ABI: argument validation (before any launch),
// workspace sizing, thread-local error text and kernel dispatch.  Every entry
// point only enqueues work on the caller's stream; nothing is allocated,
// freed or synchronised here.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>

#include "refit.h"
#include "sks_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SKS_OK;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQUIRE(cond, ...)                          \
  do {                                              \
    if (!(cond)) return fail(SKS_ERR_ARG, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(ptr, align)                                                          \
  do {                                                                                   \
    if (!(ptr)) return fail(SKS_ERR_ARG, "%s must not be NULL", #ptr);                   \
    if (!aligned((ptr), (align)))                                                        \
      return fail(SKS_ERR_ARG, "%s must be %d-byte aligned", #ptr, (int)(align));        \
  } while (0)

int hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(SKS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Shape checks shared by every call that takes the cache description.
int check_shape(const sks_kv *kv, const sks_params *p, sks::Shape &s) {
  REQUIRE(kv != nullptr, "kv must not be NULL");
  REQUIRE(p != nullptr, "params must not be NULL");
  REQUIRE(kv->D == SKS_HEAD_DIM, "D must be %d (got %d)", SKS_HEAD_DIM, kv->D);
  REQUIRE(p->rank == SKS_RANK, "rank must be %d (got %d)", SKS_RANK, p->rank);
  REQUIRE(kv->B >= 1 && kv->Hkv >= 1, "B and Hkv must be >= 1 (got %d, %d)", kv->B, kv->Hkv);
  REQUIRE(kv->dtype == SKS_KV_BF16 || kv->dtype == SKS_KV_I8 || kv->dtype == SKS_KV_I4,
          "unknown KV dtype %d", kv->dtype);
  REQUIRE(p->rows >= 1 && p->rows <= SKS_MAX_ROWS, "rows must be in [1, %d] (got %d)",
          SKS_MAX_ROWS, p->rows);
  REQUIRE(kv->T_max >= p->rows, "T_max (%d) must be >= rows (%d)", kv->T_max, p->rows);
  REQUIRE(p->pool >= 1 && p->pool <= SKS_MAX_POOL, "pool must be in [1, %d] (got %d)",
          SKS_MAX_POOL, p->pool);
  REQUIRE(kv->T_max / p->pool >= 1, "T_max / pool must be >= 1");
  REQUIRE(p->window >= 0 && p->window <= SKS_MAX_EXTENT, "window must be in [0, %d] (got %d)",
          SKS_MAX_EXTENT, p->window);
  REQUIRE(p->topk >= 1 && p->topk <= SKS_MAX_EXTENT, "topk must be in [1, %d] (got %d)",
          SKS_MAX_EXTENT, p->topk);
  REQUIRE(kv->seq_len != nullptr, "kv->seq_len must not be NULL");
  REQUIRE(aligned(kv->seq_len, 4), "kv->seq_len must be 4-byte aligned");
  const long nseg = (long)kv->B * p->rows * kv->Hkv;
  REQUIRE(nseg <= 65535, "B * rows * Hkv must be <= 65535 (got %ld)", nseg);
  if (p->pool > 1 && kv->dtype != SKS_KV_BF16)
    return fail(SKS_ERR_UNSUPPORTED, "pooling (pool > 1) needs a bf16 cache");
  if (kv->K_hot || kv->V_hot || kv->K_hot_scale || kv->V_hot_scale || kv->W_hot) {
    REQUIRE(kv->K_hot && kv->V_hot, "kv->K_hot and kv->V_hot must both be set or both NULL");
    if (p->pool > 1) return fail(SKS_ERR_UNSUPPORTED, "a hot tier needs pool == 1");
    REQUIRE(kv->W_hot >= p->window + p->rows && kv->W_hot <= kv->T_max,
            "W_hot (%d) must be in [window + rows, T_max] = [%d, %d]", kv->W_hot,
            p->window + p->rows, kv->T_max);
  }
  s.B = kv->B;
  s.R = p->rows;
  s.Hkv = kv->Hkv;
  s.T_max = kv->T_max;
  s.NB = kv->T_max / p->pool;
  s.window = p->window;
  s.topk = p->topk;
  s.pool = p->pool;
  s.dtype = kv->dtype;
  return SKS_OK;
}

int check_cache(const sks_kv *kv, bool need_v) {
  REQUIRE_PTR(kv->K, 16);
  if (need_v) REQUIRE_PTR(kv->V, 16);
  if (kv->dtype != SKS_KV_BF16) {
    REQUIRE_PTR(kv->K_scale, 2);
    if (need_v) REQUIRE_PTR(kv->V_scale, 2);
  }
  if (kv->K_hot) {
    REQUIRE_PTR(kv->K_hot, 16);
    if (need_v) REQUIRE_PTR(kv->V_hot, 16);
    if (kv->dtype != SKS_KV_BF16) {
      REQUIRE_PTR(kv->K_hot_scale, 2);
      if (need_v) REQUIRE_PTR(kv->V_hot_scale, 2);
    }
  }
  return SKS_OK;
}

int check_heads(int Hq, int Hkv) {
  REQUIRE(Hq >= 1 && Hq % Hkv == 0, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  REQUIRE(Hq / Hkv <= sks::ATTN_MAX_G, "Hq / Hkv must be <= %d (got %d)", sks::ATTN_MAX_G,
          Hq / Hkv);
  return SKS_OK;
}

#define TRY(x)                   \
  do {                           \
    int rc_ = (x);               \
    if (rc_ != SKS_OK) return rc_; \
  } while (0)

size_t ws_bytes(const sks::Shape &s, int G) {
  return sks::hist_region_bytes(s) + sks::topk_scratch_bytes(s) + sks::attn_scratch_bytes(s, G);
}

size_t topk_need(const sks::Shape &s) {
  return sks::hist_region_bytes(s) + sks::topk_scratch_bytes(s);
}

int check_ws(const void *ws, size_t given, size_t need) {
  if (!ws || given < need)
    return fail(SKS_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                ws ? given : (size_t)0);
  if (!aligned(ws, 256)) return fail(SKS_ERR_ARG, "ws must be 256-byte aligned");
  return SKS_OK;
}

// Validation of sks_decode_step's arguments (all but the workspace).
int check_step(const sks_kv *kv, const sks_params *p, const sks_step *st, int32_t flags,
               sks::Shape &s) {
  TRY(check_shape(kv, p, s));
  TRY(check_cache(kv, true));
  REQUIRE(st != nullptr, "step must not be NULL");
  REQUIRE((flags & ~(SKS_STEP_APPEND | SKS_STEP_DENSE | SKS_STEP_NO_SCORES)) == 0,
          "unknown flags 0x%x", flags);
  TRY(check_heads(st->Hq, kv->Hkv));
  REQUIRE(st->basis_per_head == 0 || st->basis_per_head == 1, "basis_per_head must be 0 or 1");
  REQUIRE_PTR(st->q, 16);
  REQUIRE_PTR(st->basis, 4);
  REQUIRE_PTR(st->key_scale, 4);
  REQUIRE_PTR(st->S, 16);
  REQUIRE_PTR(st->qsk, 16);
  REQUIRE_PTR(st->scores, 4);
  REQUIRE_PTR(st->idx, 4);
  REQUIRE_PTR(st->out, 16);
  if (st->qscale) REQUIRE(aligned(st->qscale, 4), "qscale must be 4-byte aligned");
  if (st->n_sel) REQUIRE(aligned(st->n_sel, 4), "n_sel must be 4-byte aligned");
  if (st->lse) REQUIRE(aligned(st->lse, 4), "lse must be 4-byte aligned");
  if (s.pool > 1) {
    REQUIRE_PTR(st->Kp, 16);
    REQUIRE_PTR(st->Vp, 16);
  } else {
    REQUIRE(st->Kp == nullptr && st->Vp == nullptr, "Kp and Vp must be NULL when pool == 1");
  }
  REQUIRE(st->sm_scale > 0.f && st->sm_scale < 1e30f, "sm_scale must be positive and finite");
  if (sks::ceil_div(s.NB, sks::TK_SUB) > sks::TK_MAX_SUBS)
    return fail(SKS_ERR_UNSUPPORTED, "T_max / pool above %d is not supported by the selection",
                sks::TK_MAX_SUBS * sks::TK_SUB);
  return SKS_OK;
}

// The launches of one decode step on a carved workspace: the first launch
// (query sketch, append, candidate mode's sample pass), the score pass, the
// selection, the attention and its merge.
hipError_t enqueue_step(const sks_kv &kv, const sks::Shape &s, const sks_step &st, int32_t flags,
                        const sks::TopkWs &w, hipStream_t hs) {
  const bool dense = (flags & SKS_STEP_DENSE) != 0;
  const bool cand = !dense && (flags & SKS_STEP_NO_SCORES) && sks::topk_cand_preferred(s);
  // the first launch derives the estimates itself when one workgroup samples
  // each segment; otherwise it leaves sample histograms for the score pass
  const bool est = cand && sks::topk_cand_est_early(s);
  hipError_t e = sks::launch_step_front(kv, s, st.q, st.Hq, st.basis, st.basis_per_head,
                                        st.key_scale, st.qsk, st.qscale, st.S, st.Kp, st.Vp,
                                        (flags & SKS_STEP_APPEND) != 0, cand, w, hs);
  if (!dense) {
    if (cand) {
      if (e == hipSuccess)
        e = sks::launch_score(st.qsk, st.S, kv.seq_len, s, nullptr, &w, hs, true, 0,
                              est ? w.counters : nullptr);
      // (sample histograms are cleared by the attention's merge launch, off
      // the selection's critical path)
      if (e == hipSuccess)
        e = sks::launch_topk_cand(st.qsk, st.S, st.scores, kv.seq_len, s, st.idx, st.n_sel, w, hs,
                                  false);
    } else {
      if (e == hipSuccess) e = sks::launch_score(st.qsk, st.S, kv.seq_len, s, st.scores, &w, hs);
      if (e == hipSuccess)
        e = sks::launch_topk(st.scores, kv.seq_len, s, true, st.idx, st.n_sel, w, hs);
    }
  }
  if (e == hipSuccess)
    e = sks::launch_attn(st.q, st.Hq, kv, s, st.idx, st.Kp, st.Vp, st.sm_scale, st.out, st.lse,
                         w, hs, dense, cand && !est ? w.hsamp : nullptr,
                         cand && !est ? (long)s.B * s.R * s.Hkv * sks::HIST1_BINS : 0);
  return e;
}

// ---------------------------------------------------------------- static workspace
// The workspace of sks_decode_step_static: one array per GPU, alive until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address of each
// GPU's copy comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is used.
static __device__ __align__(256) unsigned char scratch[SKS_STATIC_WORKSPACE_BYTES];

constexpr int STATIC_MAX_DEVICES = 64;
std::mutex g_static_mu;
void *g_static_ptr[STATIC_MAX_DEVICES];
bool g_static_used[STATIC_MAX_DEVICES];
sks::Shape g_static_last[STATIC_MAX_DEVICES];   // shape of the device's previous call

bool same_layout(const sks::Shape &a, const sks::Shape &b) {
  return a.B == b.B && a.R == b.R && a.Hkv == b.Hkv && a.T_max == b.T_max && a.NB == b.NB &&
         a.window == b.window && a.topk == b.topk && a.pool == b.pool && a.dtype == b.dtype;
}

// The static workspace of the device that runs `stream` (the current device
// for the null stream); `clear` is set when its selection histograms must be
// zeroed first (the device's first call, or a change of shape).
int static_workspace(hipStream_t stream, const sks::Shape &s, void *&ws, bool &clear) {
  int dev = -1;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess)
      return fail(SKS_ERR_HIP, "hipStreamGetDevice failed for the given stream");
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return fail(SKS_ERR_HIP, "hipGetDevice failed");
  }
  if (dev < 0 || dev >= STATIC_MAX_DEVICES)
    return fail(SKS_ERR_UNSUPPORTED, "device %d: the static workspace serves devices 0..%d", dev,
                STATIC_MAX_DEVICES - 1);
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return fail(SKS_ERR_HIP, "hipGetDevice failed");
    if (cur != dev && hipSetDevice(dev) != hipSuccess)
      return fail(SKS_ERR_HIP, "hipSetDevice(%d) failed", dev);
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr)
      return fail(SKS_ERR_HIP, "hipGetSymbolAddress of the static workspace on device %d: %s", dev,
                  hipGetErrorString(e));
    g_static_ptr[dev] = ptr;
  }
  ws = g_static_ptr[dev];
  clear = !g_static_used[dev] || !same_layout(g_static_last[dev], s);
  g_static_used[dev] = true;
  g_static_last[dev] = s;
  return SKS_OK;
}

}  // namespace

extern "C" {

const char *sks_last_error(void) { return g_err; }

int32_t sks_runtime_version(void) {
  int v = 0;
  if (hipRuntimeGetVersion(&v) != hipSuccess) return -1;
  return v;
}

size_t sks_workspace_bytes(const sks_kv *kv, const sks_params *p, int32_t Hq) {
  sks::Shape s;
  if (check_shape(kv, p, s) != SKS_OK) return 0;
  if (check_heads(Hq, kv->Hkv) != SKS_OK) return 0;
  return ws_bytes(s, Hq / kv->Hkv);
}

int sks_sketch_build(const sks_kv *kv, const sks_params *p, const float *basis,
                     int32_t basis_per_head, const float *key_scale, int32_t t_begin,
                     int32_t t_end, int8_t *S, uint16_t *Kp, uint16_t *Vp, sks_stream_t stream) {
  sks::Shape s;
  TRY(check_shape(kv, p, s));
  TRY(check_cache(kv, p->pool > 1));
  REQUIRE_PTR(basis, 4);
  REQUIRE_PTR(key_scale, 4);
  REQUIRE_PTR(S, 16);
  REQUIRE(basis_per_head == 0 || basis_per_head == 1, "basis_per_head must be 0 or 1");
  REQUIRE(t_begin == SKS_APPEND || (t_begin >= 0 && t_end >= t_begin),
          "position range [%d, %d) is invalid", t_begin, t_end);
  if (p->pool > 1) {
    REQUIRE_PTR(Kp, 16);
    REQUIRE_PTR(Vp, 16);
  } else {
    REQUIRE(Kp == nullptr && Vp == nullptr, "Kp and Vp must be NULL when pool == 1");
  }
  if (t_begin != SKS_APPEND) {
    t_begin = std::min(t_begin, s.T_max);
    t_end = std::min(t_end, s.T_max);
    if (t_end <= t_begin) return ok();
  }
  return hip_status(sks::launch_sketch_keys(*kv, s, basis, basis_per_head, key_scale, t_begin,
                                            t_end, S, Kp, Vp, (hipStream_t)stream),
                    "sks_sketch_build");
}

int sks_sketch_build_query(const uint16_t *q, int32_t B, int32_t R, int32_t Hq, int32_t Hkv,
                           const float *basis, int32_t basis_per_head, int8_t *qsk,
                           float *qscale, sks_stream_t stream) {
  REQUIRE(B >= 1 && R >= 1 && R <= SKS_MAX_ROWS && Hkv >= 1, "bad B/R/Hkv (%d, %d, %d)", B, R,
          Hkv);
  REQUIRE(Hq >= 1 && Hq % Hkv == 0, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  REQUIRE((long)B * R * Hkv <= 0x7fffffffL, "too many segments");
  REQUIRE(basis_per_head == 0 || basis_per_head == 1, "basis_per_head must be 0 or 1");
  REQUIRE_PTR(q, 4);
  REQUIRE_PTR(basis, 4);
  REQUIRE_PTR(qsk, 16);
  if (qscale) REQUIRE(aligned(qscale, 4), "qscale must be 4-byte aligned");
  return hip_status(sks::launch_sketch_query(q, B, R, Hq, Hkv, basis, basis_per_head, qsk, qscale,
                                             (hipStream_t)stream),
                    "sks_sketch_build_query");
}

int sks_workspace_init(void *ws, size_t ws_bytes_given, sks_stream_t stream) {
  REQUIRE(ws != nullptr, "ws must not be NULL");
  REQUIRE(aligned(ws, 256), "ws must be 256-byte aligned");
  return hip_status(sks::launch_fill(static_cast<int32_t *>(ws), ws_bytes_given / 4,
                                     (hipStream_t)stream),
                    "sks_workspace_init");
}

int sks_sketch_score(const int8_t *qsk, const int8_t *S, const sks_kv *kv, const sks_params *p,
                     int32_t *scores, void *ws, size_t ws_bytes_given, sks_stream_t stream) {
  sks::Shape s;
  TRY(check_shape(kv, p, s));
  REQUIRE_PTR(qsk, 16);
  REQUIRE_PTR(S, 16);
  REQUIRE_PTR(scores, 4);
  sks::TopkWs w{};
  if (ws) {
    TRY(check_ws(ws, ws_bytes_given, topk_need(s)));
    w = sks::topk_ws_carve(s, ws);
  }
  return hip_status(sks::launch_score(qsk, S, kv->seq_len, s, scores, ws ? &w : nullptr,
                                      (hipStream_t)stream),
                    "sks_sketch_score");
}

int sks_topk_select(const int32_t *scores, const sks_kv *kv, const sks_params *p, int32_t flags,
                    int32_t *idx, int32_t *n_sel, void *ws, size_t ws_bytes_given,
                    sks_stream_t stream) {
  sks::Shape s;
  TRY(check_shape(kv, p, s));
  REQUIRE_PTR(scores, 4);
  REQUIRE_PTR(idx, 4);
  if (n_sel) REQUIRE(aligned(n_sel, 4), "n_sel must be 4-byte aligned");
  if (sks::ceil_div(s.NB, sks::TK_SUB) > sks::TK_MAX_SUBS)
    return fail(SKS_ERR_UNSUPPORTED, "T_max / pool above %d is not supported by the selection",
                sks::TK_MAX_SUBS * sks::TK_SUB);
  REQUIRE((flags & ~SKS_TOPK_HIST_READY) == 0, "unknown flags 0x%x", flags);
  TRY(check_ws(ws, ws_bytes_given, topk_need(s)));
  const sks::TopkWs w = sks::topk_ws_carve(s, ws);
  return hip_status(sks::launch_topk(scores, kv->seq_len, s, (flags & SKS_TOPK_HIST_READY) != 0,
                                     idx, n_sel, w, (hipStream_t)stream),
                    "sks_topk_select");
}

int sks_score_candidates(const int8_t *qsk, const int8_t *S, const sks_kv *kv,
                         const sks_params *p, int32_t flags, void *ws, size_t ws_bytes_given,
                         sks_stream_t stream) {
  sks::Shape s;
  TRY(check_shape(kv, p, s));
  REQUIRE_PTR(qsk, 16);
  REQUIRE_PTR(S, 16);
  if (sks::ceil_div(s.NB, sks::TK_SUB) > sks::TK_MAX_SUBS)
    return fail(SKS_ERR_UNSUPPORTED, "T_max / pool above %d is not supported by the selection",
                sks::TK_MAX_SUBS * sks::TK_SUB);
  const int32_t known = SKS_CAND_KEEP_ESTIMATE | SKS_CAND_TEST_HIGH | SKS_CAND_TEST_ZERO;
  REQUIRE((flags & ~known) == 0, "unknown flags 0x%x", flags);
  REQUIRE((flags & (SKS_CAND_TEST_HIGH | SKS_CAND_TEST_ZERO)) !=
              (SKS_CAND_TEST_HIGH | SKS_CAND_TEST_ZERO),
          "SKS_CAND_TEST_HIGH and SKS_CAND_TEST_ZERO exclude each other");
  TRY(check_ws(ws, ws_bytes_given, topk_need(s)));
  const sks::TopkWs w = sks::topk_ws_carve(s, ws);
  const hipStream_t hs = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  const int force = (flags & SKS_CAND_TEST_HIGH) ? 1 : (flags & SKS_CAND_TEST_ZERO) ? 2 : 0;
  if (!(flags & SKS_CAND_KEEP_ESTIMATE) && !force)
    e = sks::launch_topk_sample(qsk, S, kv->seq_len, s, w, hs);
  if (e == hipSuccess)
    e = sks::launch_score(qsk, S, kv->seq_len, s, nullptr, &w, hs, true, force,
                          sks::topk_cand_est_early(s) ? w.counters : nullptr);
  return hip_status(e, "sks_score_candidates");
}

int sks_topk_select_candidates(const int8_t *qsk, const int8_t *S, const sks_kv *kv,
                               const sks_params *p, int32_t *scores, int32_t *idx,
                               int32_t *n_sel, void *ws, size_t ws_bytes_given,
                               sks_stream_t stream) {
  sks::Shape s;
  TRY(check_shape(kv, p, s));
  REQUIRE_PTR(qsk, 16);
  REQUIRE_PTR(S, 16);
  REQUIRE_PTR(scores, 4);
  REQUIRE_PTR(idx, 4);
  if (n_sel) REQUIRE(aligned(n_sel, 4), "n_sel must be 4-byte aligned");
  if (sks::ceil_div(s.NB, sks::TK_SUB) > sks::TK_MAX_SUBS)
    return fail(SKS_ERR_UNSUPPORTED, "T_max / pool above %d is not supported by the selection",
                sks::TK_MAX_SUBS * sks::TK_SUB);
  TRY(check_ws(ws, ws_bytes_given, topk_need(s)));
  const sks::TopkWs w = sks::topk_ws_carve(s, ws);
  // (sample histograms are left only where no estimate was derived at once)
  return hip_status(sks::launch_topk_cand(qsk, S, scores, kv->seq_len, s, idx, n_sel, w,
                                          (hipStream_t)stream, !sks::topk_cand_est_early(s)),
                    "sks_topk_select_candidates");
}

int sks_gather_pack(const sks_kv *kv, const sks_params *p, const int32_t *idx, const uint16_t *Kp,
                    const uint16_t *Vp, void *K_out, void *V_out, uint16_t *Ks_out,
                    uint16_t *Vs_out, int32_t *n_out, sks_stream_t stream) {
  sks::Shape s;
  TRY(check_shape(kv, p, s));
  TRY(check_cache(kv, true));
  REQUIRE_PTR(idx, 4);
  REQUIRE_PTR(K_out, 16);
  REQUIRE_PTR(V_out, 16);
  REQUIRE_PTR(n_out, 4);
  if (s.pool > 1) {
    REQUIRE_PTR(Kp, 16);
    REQUIRE_PTR(Vp, 16);
  }
  if (s.dtype != SKS_KV_BF16) {
    REQUIRE_PTR(Ks_out, 2);
    REQUIRE_PTR(Vs_out, 2);
  } else {
    REQUIRE(Ks_out == nullptr && Vs_out == nullptr, "Ks_out/Vs_out must be NULL for bf16");
  }
  return hip_status(sks::launch_gather(*kv, s, idx, Kp, Vp, K_out, V_out, Ks_out, Vs_out, n_out,
                                       (hipStream_t)stream),
                    "sks_gather_pack");
}

int sks_sparse_decode_attn(const uint16_t *q, int32_t Hq, const sks_kv *kv, const sks_params *p,
                           const int32_t *idx, const uint16_t *Kp, const uint16_t *Vp,
                           float sm_scale, float *out, float *lse, void *ws,
                           size_t ws_bytes_given, sks_stream_t stream) {
  sks::Shape s;
  TRY(check_shape(kv, p, s));
  TRY(check_cache(kv, true));
  TRY(check_heads(Hq, kv->Hkv));
  REQUIRE_PTR(q, 16);
  REQUIRE_PTR(idx, 4);
  REQUIRE_PTR(out, 16);
  if (lse) REQUIRE(aligned(lse, 4), "lse must be 4-byte aligned");
  if (s.pool > 1) {
    REQUIRE_PTR(Kp, 16);
    REQUIRE_PTR(Vp, 16);
  }
  REQUIRE(sm_scale > 0.f && sm_scale < 1e30f, "sm_scale must be positive and finite");
  TRY(check_ws(ws, ws_bytes_given,
               ws_bytes(s, Hq / kv->Hkv)));
  return hip_status(sks::launch_attn(q, Hq, *kv, s, idx, Kp, Vp, sm_scale, out, lse,
                                     sks::topk_ws_carve(s, ws), (hipStream_t)stream),
                    "sks_sparse_decode_attn");
}

int sks_decode_step(const sks_kv *kv, const sks_params *p, const sks_step *st, int32_t flags,
                    void *ws, size_t ws_bytes_given, sks_stream_t stream) {
  sks::Shape s;
  TRY(check_step(kv, p, st, flags, s));
  TRY(check_ws(ws, ws_bytes_given, ws_bytes(s, st->Hq / kv->Hkv)));
  return hip_status(enqueue_step(*kv, s, *st, flags, sks::topk_ws_carve(s, ws), (hipStream_t)stream),
                    "sks_decode_step");
}

int sks_decode_step_static(const sks_kv *kv, const sks_params *p, const sks_step *st,
                           int32_t flags, sks_stream_t stream) {
  sks::Shape s;
  TRY(check_step(kv, p, st, flags, s));
  const size_t need = ws_bytes(s, st->Hq / kv->Hkv);
  if (need > (size_t)SKS_STATIC_WORKSPACE_BYTES)
    return fail(SKS_ERR_WORKSPACE,
                "this shape needs a %zu-byte workspace, more than the %zu bytes of the static one "
                "(use sks_decode_step with a caller-provided workspace)",
                need, (size_t)SKS_STATIC_WORKSPACE_BYTES);
  const hipStream_t hs = (hipStream_t)stream;
  void *ws = nullptr;
  bool clear = false;
  TRY(static_workspace(hs, s, ws, clear));
  hipError_t e = hipSuccess;
  // the selection histograms must be zero at rest; a call of another shape
  // lays its scratch over them, so they are cleared (a fill kernel, no memset
  // node) at the device's first call and after a change of shape
  if (clear) e = sks::launch_fill(static_cast<int32_t *>(ws), sks::hist_region_bytes(s) / 4, hs);
  if (e == hipSuccess) e = enqueue_step(*kv, s, *st, flags, sks::topk_ws_carve(s, ws), hs);
  return hip_status(e, "sks_decode_step_static");
}

}  // extern "C"

// ------------------------------------------------------------ basis refit
namespace {

int check_refit_kv(const sks_kv *kv, int32_t t_begin, int32_t t_end) {
  REQUIRE(kv != nullptr, "kv must not be NULL");
  REQUIRE(kv->D == SKS_HEAD_DIM, "D must be %d (got %d)", SKS_HEAD_DIM, kv->D);
  REQUIRE(kv->B >= 1 && kv->Hkv >= 1, "B and Hkv must be >= 1 (got %d, %d)", kv->B, kv->Hkv);
  REQUIRE(kv->T_max >= 1, "T_max must be >= 1");
  REQUIRE((long)kv->B * kv->Hkv <= 65535, "B * Hkv must be <= 65535");
  REQUIRE(kv->dtype == SKS_KV_BF16 || kv->dtype == SKS_KV_I8 || kv->dtype == SKS_KV_I4,
          "unknown KV dtype %d", kv->dtype);
  if (kv->dtype != SKS_KV_BF16)
    return fail(SKS_ERR_UNSUPPORTED, "the basis refit takes bf16 keys");
  REQUIRE(t_begin >= 0 && t_begin <= t_end && t_end <= kv->T_max,
          "key range [%d, %d) must lie in [0, T_max = %d]", t_begin, t_end, kv->T_max);
  REQUIRE_PTR(kv->K, 16);
  REQUIRE(kv->seq_len != nullptr, "kv->seq_len must not be NULL");
  REQUIRE(aligned(kv->seq_len, 4), "kv->seq_len must be 4-byte aligned");
  return SKS_OK;
}

size_t refit_ws(const sks_kv *kv, int32_t t_begin, int32_t t_end) {
  const long span = (long)t_end - (long)t_begin;
  const size_t gram = sks::refit_gram_scratch_bytes(kv->B, kv->Hkv, span);
  const size_t vecs = (size_t)kv->Hkv * SKS_HEAD_DIM * SKS_HEAD_DIM * sizeof(double);
  const size_t amax = (size_t)kv->B * kv->Hkv * sks::refit_amax_chunks(span) * sizeof(float);
  return sks::align_up(std::max(gram, std::max(vecs, amax)), 256);
}

}  // namespace

extern "C" {

size_t sks_refit_workspace_bytes(const sks_kv *kv, int32_t t_begin, int32_t t_end) {
  if (check_refit_kv(kv, t_begin, t_end) != SKS_OK) return 0;
  ok();
  return refit_ws(kv, t_begin, t_end);
}

int sks_refit_gram(const sks_kv *kv, int32_t t_begin, int32_t t_end, int32_t per_head,
                   double *gram, void *ws, size_t ws_bytes_given, sks_stream_t stream) {
  TRY(check_refit_kv(kv, t_begin, t_end));
  REQUIRE_PTR(gram, 8);
  TRY(check_ws(ws, ws_bytes_given, refit_ws(kv, t_begin, t_end)));
  return hip_status(sks::launch_refit_gram(*kv, t_begin, t_end, per_head ? 1 : 0, gram, ws,
                                           (hipStream_t)stream),
                    "sks_refit_gram");
}

int sks_refit_basis(const double *gram, int32_t n, float *basis, double *eigval, void *ws,
                    size_t ws_bytes_given, sks_stream_t stream) {
  REQUIRE(n >= 1 && n <= 65535, "n must be in [1, 65535] (got %d)", n);
  REQUIRE_PTR(gram, 8);
  REQUIRE_PTR(basis, 4);
  if (eigval) REQUIRE(aligned(eigval, 8), "eigval must be 8-byte aligned");
  TRY(check_ws(ws, ws_bytes_given, (size_t)n * SKS_HEAD_DIM * SKS_HEAD_DIM * sizeof(double)));
  return hip_status(sks::launch_refit_basis(gram, n, basis, eigval, ws, (hipStream_t)stream),
                    "sks_refit_basis");
}

int sks_refit_key_scale(const sks_kv *kv, int32_t t_begin, int32_t t_end, const float *basis,
                        int32_t basis_per_head, float *key_scale, void *ws, size_t ws_bytes_given,
                        sks_stream_t stream) {
  TRY(check_refit_kv(kv, t_begin, t_end));
  REQUIRE_PTR(basis, 4);
  REQUIRE_PTR(key_scale, 4);
  TRY(check_ws(ws, ws_bytes_given, refit_ws(kv, t_begin, t_end)));
  const long span = (long)t_end - (long)t_begin;
  float *amax = static_cast<float *>(ws);
  const hipStream_t hs = (hipStream_t)stream;
  hipError_t e = sks::launch_refit_amax(*kv, t_begin, t_end, basis, basis_per_head, amax, hs);
  if (e == hipSuccess)
    e = sks::launch_refit_scale_reduce(amax, kv->B, kv->Hkv, sks::refit_amax_chunks(span),
                                       key_scale, hs);
  return hip_status(e, "sks_refit_key_scale");
}

}  // extern "C"
