// extern "C" entry points of libua.so: argument checks, workspace carving and
// kernel dispatch.  No device memory is read or allocated here.

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/ua.h"
#include "ua_kernels.hpp"

namespace {

using ua::LayerArgs;

// Workspace of ua_decode_compact_step_noalloc: one copy per GPU, loaded with
// the code object and held until the process ends.  In host code `scratch`
// only names the symbol; its device address (different on every GPU) comes
// from hipGetSymbolAddress and is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[UA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current GPU's copy of `scratch` (looked up once per GPU).
ua_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return UA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return UA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return UA_ERR_HIP;
    if (reinterpret_cast<uintptr_t>(p) % 256 != 0) return UA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return UA_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

ua_status check_dims(const ua_dims* d) {
  if (!d) return UA_ERR_INVALID_ARG;
  if (d->B < 1 || d->H_q < 1 || d->H_kv < 1 || d->d_model < 1 || d->gate_rank < 1) return UA_ERR_INVALID_ARG;
  if (d->H_q % d->H_kv != 0) return UA_ERR_INVALID_ARG;
  if (d->terms < 0 || d->terms > 7) return UA_ERR_INVALID_ARG;
  if (d->dtype != UA_F32 && d->dtype != UA_BF16) return UA_ERR_INVALID_ARG;
  if (d->y_dtype != UA_F32 && d->y_dtype != UA_BF16) return UA_ERR_INVALID_ARG;
  if (!(d->rope_base > 1.0) || !isfinite(d->rope_base)) return UA_ERR_INVALID_ARG;
  if (!(d->sm_scale >= 0.0f) || !isfinite(d->sm_scale)) return UA_ERR_INVALID_ARG;
  if (d->d_head != 64 && d->d_head != 128) return UA_ERR_UNSUPPORTED;
  const int G = d->H_q / d->H_kv;
  if (G != 1 && G != 2 && G != 3 && G != 4 && G != 8) return UA_ERR_UNSUPPORTED;
  if (d->H_kv > ua::kMaxHkv || d->gate_rank > ua::kMaxRank) return UA_ERR_UNSUPPORTED;
  if (d->d_model % 8 != 0 || d->d_model > ua::kMaxDModel) return UA_ERR_UNSUPPORTED;
  if ((int64_t)d->B * d->H_kv > ua::kMaxSeg) return UA_ERR_UNSUPPORTED;
  return UA_OK;
}

ua_status check_cache(const ua_cache* c) {
  if (!c) return UA_ERR_INVALID_ARG;
  if (!c->K || !c->V || !c->logbias || !c->kgate || !c->seg_off || !c->seg_len || !c->seg_cap || !c->next_pos ||
      !c->status)
    return UA_ERR_INVALID_ARG;
  if (!aligned(c->K, 16) || !aligned(c->V, 16) || !aligned(c->logbias, 4) || !aligned(c->kgate, 4) ||
      !aligned(c->seg_off, 8) || !aligned(c->seg_len, 4) || !aligned(c->seg_cap, 4) || !aligned(c->next_pos, 4) ||
      !aligned(c->status, 4))
    return UA_ERR_INVALID_ARG;
  if (c->total_slots < 1 || c->total_slots > ((int64_t)1 << 40)) return UA_ERR_INVALID_ARG;
  return UA_OK;
}

ua_status check_params(const ua_params* p) {
  if (!p || !p->W_dec || !p->b_dec || !p->W_dn || !p->W_up) return UA_ERR_INVALID_ARG;
  if (!aligned(p->W_dec, 16) || !aligned(p->b_dec, 4) || !aligned(p->W_dn, 16) || !aligned(p->W_up, 16) ||
      (p->b_up && !aligned(p->b_up, 4)))
    return UA_ERR_INVALID_ARG;
  return UA_OK;
}

ua_status check_tokens(const ua_tokens* t) {
  if (!t || !t->q || !t->k || !t->v || !t->x) return UA_ERR_INVALID_ARG;
  if (!aligned(t->q, 16) || !aligned(t->k, 16) || !aligned(t->v, 16) || !aligned(t->x, 16)) return UA_ERR_INVALID_ARG;
  return UA_OK;
}

bool bad_log_p(float log_p) { return isnan(log_p) || log_p > 0.0f; }

LayerArgs make_args(const ua_dims* d, const ua_params* p, const ua_cache* c, const ua_tokens* t, void* y) {
  LayerArgs a{};
  a.B = d->B;
  a.H_q = d->H_q;
  a.H_kv = d->H_kv;
  a.d = d->d_head;
  a.D_model = d->d_model;
  a.r = d->gate_rank;
  a.terms = d->terms;
  a.bf16 = d->dtype == UA_BF16;
  a.y_bf16 = d->y_dtype == UA_BF16;
  a.scale = d->sm_scale != 0.0f ? d->sm_scale : (float)(1.0 / sqrt((double)d->d_head));
  a.rope_base = d->rope_base;
  for (int i = 0; i < 64; ++i) a.inv_freq[i] = (2 * i < d->d_head) ? pow(d->rope_base, -2.0 * i / d->d_head) : 0.0;
  if (p) {
    a.W_dec = p->W_dec;
    a.b_dec = p->b_dec;
    a.W_dn = p->W_dn;
    a.W_up = p->W_up;
    a.b_up = p->b_up;
  }
  if (t) {
    a.q = t->q;
    a.k = t->k;
    a.v = t->v;
    a.x = t->x;
  }
  a.K = c->K;
  a.V = c->V;
  a.lam = c->logbias;
  a.lk = c->kgate;
  a.seg_off = c->seg_off;
  a.seg_len = c->seg_len;
  a.seg_cap = c->seg_cap;
  a.next_pos = c->next_pos;
  a.status = c->status;
  a.total_slots = c->total_slots;
  a.y = y;
  return a;
}

}  // namespace

extern "C" {

size_t ua_workspace_bytes(const ua_dims* dims, int32_t max_tokens_per_call, int64_t total_slots, int32_t max_seg_cap) {
  if (check_dims(dims) != UA_OK || total_slots < 1 || max_tokens_per_call < 1 || max_seg_cap < 1) return 0;
  ua_cache c{};
  c.total_slots = total_slots;
  LayerArgs a = make_args(dims, nullptr, &c, nullptr, nullptr);
  size_t n = ua::decode_ws_bytes(a, ua::decode_tile_entries(a.d, a.H_q / a.H_kv, a.bf16 != 0));
  const size_t np = ua::prefill_ws_bytes(a, max_tokens_per_call, max_seg_cap);
  if (np > n) n = np;
  return ua::control_bytes(a) + n + ua::control_tail_bytes(a);
}

ua_status ua_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || !aligned(ws, 256) || ws_bytes == 0) return UA_ERR_INVALID_ARG;
  const hipError_t e = ua::launch_fill_zero(ws, ws_bytes, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? UA_OK : UA_ERR_HIP;
}

static ua_status decode_common(const ua_dims* dims, const ua_params* params, const ua_cache* cache, const ua_tokens* in,
                               float log_p, void* y, bool compact, int32_t* kept_idx, void* ws, size_t ws_bytes,
                               void* stream) {
  ua_status s;
  if ((s = check_dims(dims)) != UA_OK) return s;
  if ((s = check_params(params)) != UA_OK) return s;
  if ((s = check_cache(cache)) != UA_OK) return s;
  if ((s = check_tokens(in)) != UA_OK) return s;
  if (!y || !aligned(y, 16) || bad_log_p(log_p)) return UA_ERR_INVALID_ARG;
  if (kept_idx && !aligned(kept_idx, 4)) return UA_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, 256)) return UA_ERR_INVALID_ARG;
  LayerArgs a = make_args(dims, params, cache, in, y);
  const int twg = ua::decode_tile_entries(a.d, a.H_q / a.H_kv, a.bf16 != 0);
  const size_t cb = ua::control_bytes(a);
  if (ws_bytes < cb + ua::decode_ws_bytes(a, twg) + ua::control_tail_bytes(a)) return UA_ERR_WORKSPACE;
  const ua::Control ctl = ua::control_carve(a, ws, ws_bytes);
  ua::DecodeWs w = ua::decode_ws_carve(a, ctl, reinterpret_cast<char*>(ws) + cb, twg);
  const hipError_t e = ua::launch_decode(a, w, ctl, log_p, compact, kept_idx, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? UA_OK : UA_ERR_HIP;
}

ua_status ua_decode_step(const ua_dims* dims, const ua_params* params, const ua_cache* cache, const ua_tokens* in,
                         float log_p, void* y, void* ws, size_t ws_bytes, void* stream) {
  return decode_common(dims, params, cache, in, log_p, y, false, nullptr, ws, ws_bytes, stream);
}

ua_status ua_decode_compact_step(const ua_dims* dims, const ua_params* params, const ua_cache* cache,
                                 const ua_tokens* in, float log_p, void* y, int32_t* kept_idx, void* ws,
                                 size_t ws_bytes, void* stream) {
  return decode_common(dims, params, cache, in, log_p, y, true, kept_idx, ws, ws_bytes, stream);
}

// The decode step's first launch clears every counter and look-back word the
// step uses, so the shared array needs no clearing between calls; a step whose
// workspace would not fit the array is rejected before anything is launched.
ua_status ua_decode_compact_step_noalloc(const ua_dims* dims, const ua_params* params, const ua_cache* cache,
                                         const ua_tokens* in, float log_p, void* y, int32_t* kept_idx,
                                         void* stream) {
  void* ws = nullptr;
  const ua_status s = noalloc_scratch(&ws);
  if (s != UA_OK) return s;
  return decode_common(dims, params, cache, in, log_p, y, true, kept_idx, ws, UA_NOALLOC_SCRATCH_BYTES, stream);
}

// Shared checks and workspace carving of the prefill entry points.
static ua_status prefill_setup(const ua_dims* dims, const ua_params* params, const ua_cache* cache,
                               const ua_tokens* in, void* y, void* ws, size_t ws_bytes, LayerArgs* a,
                               ua::Control* ctl, char** scratch, size_t* scratch_bytes) {
  ua_status s;
  if ((s = check_dims(dims)) != UA_OK) return s;
  if ((s = check_params(params)) != UA_OK) return s;
  if ((s = check_cache(cache)) != UA_OK) return s;
  if ((s = check_tokens(in)) != UA_OK) return s;
  if (!y || !aligned(y, 16)) return UA_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, 256)) return UA_ERR_INVALID_ARG;
  *a = make_args(dims, params, cache, in, y);
  const size_t cb = ua::control_bytes(*a);
  const size_t tb = ua::control_tail_bytes(*a);
  if (ws_bytes < cb + tb) return UA_ERR_WORKSPACE;
  *ctl = ua::control_carve(*a, ws, ws_bytes);
  // the scratch ends where the compaction flags begin
  *scratch = reinterpret_cast<char*>(ws) + cb;
  *scratch_bytes = ws_bytes / 256 * 256 - tb - cb;
  return UA_OK;
}

static ua_status prefill_status(hipError_t e) {
  if (e == hipErrorNotSupported) return UA_ERR_UNSUPPORTED;
  if (e == hipErrorOutOfMemory) return UA_ERR_WORKSPACE;
  return e == hipSuccess ? UA_OK : UA_ERR_HIP;
}

ua_status ua_prefill(const ua_dims* dims, const ua_params* params, const ua_cache* cache, const ua_tokens* in,
                     int32_t n_tokens, void* y, void* ws, size_t ws_bytes, void* stream) {
  LayerArgs a;
  ua::Control ctl;
  char* scratch;
  size_t sb;
  ua_status s;
  if (n_tokens < 1) return UA_ERR_INVALID_ARG;
  if ((s = prefill_setup(dims, params, cache, in, y, ws, ws_bytes, &a, &ctl, &scratch, &sb)) != UA_OK) return s;
  return prefill_status(ua::launch_prefill(a, ctl, n_tokens, 0, scratch, sb, reinterpret_cast<hipStream_t>(stream),
                                           -__builtin_huge_valf(), n_tokens, 0));
}

ua_status ua_prefill_pruned(const ua_dims* dims, const ua_params* params, const ua_cache* cache,
                            const ua_tokens* in, int32_t n_tokens, float log_p, void* y, int32_t* kept_idx,
                            void* ws, size_t ws_bytes, void* stream) {
  LayerArgs a;
  ua::Control ctl;
  char* scratch;
  size_t sb;
  ua_status s;
  if (n_tokens < 1 || bad_log_p(log_p)) return UA_ERR_INVALID_ARG;
  if (kept_idx && !aligned(kept_idx, 4)) return UA_ERR_INVALID_ARG;
  if ((s = prefill_setup(dims, params, cache, in, y, ws, ws_bytes, &a, &ctl, &scratch, &sb)) != UA_OK) return s;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if ((s = prefill_status(ua::launch_prefill(a, ctl, n_tokens, 0, scratch, sb, st, log_p, n_tokens, 0))) != UA_OK)
    return s;
  return ua::launch_compact(a, ctl, log_p, kept_idx, st) == hipSuccess ? UA_OK : UA_ERR_HIP;
}

ua_status ua_prefill_chunked(const ua_dims* dims, const ua_params* params, const ua_cache* cache,
                             const ua_tokens* in, int32_t n_tokens, int32_t chunk, float log_p, void* y, void* ws,
                             size_t ws_bytes, void* stream) {
  LayerArgs a;
  ua::Control ctl;
  char* scratch;
  size_t sb;
  ua_status s;
  if (n_tokens < 1 || chunk < 1 || bad_log_p(log_p)) return UA_ERR_INVALID_ARG;
  if ((s = prefill_setup(dims, params, cache, in, y, ws, ws_bytes, &a, &ctl, &scratch, &sb)) != UA_OK) return s;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  for (int32_t t0 = 0; t0 < n_tokens; t0 += chunk) {
    const int32_t nc = n_tokens - t0 < chunk ? n_tokens - t0 : chunk;
    if ((s = prefill_status(ua::launch_prefill(a, ctl, nc, 0, scratch, sb, st, -__builtin_huge_valf(), n_tokens,
                                               t0))) != UA_OK)
      return s;
    if (ua::launch_compact(a, ctl, log_p, nullptr, st) != hipSuccess) return UA_ERR_HIP;
  }
  return UA_OK;
}

ua_status ua_prefill_varlen(const ua_dims* dims, const ua_params* params, const ua_cache* cache,
                            const ua_tokens* in, const int32_t* cu_seqlens, int32_t total_tokens, int32_t max_tokens,
                            void* y, void* ws, size_t ws_bytes, void* stream) {
  LayerArgs a;
  ua::Control ctl;
  char* scratch;
  size_t sb;
  ua_status s;
  if (max_tokens < 1 || total_tokens < 1 || !cu_seqlens || !aligned(cu_seqlens, 4)) return UA_ERR_INVALID_ARG;
  if ((s = prefill_setup(dims, params, cache, in, y, ws, ws_bytes, &a, &ctl, &scratch, &sb)) != UA_OK) return s;
  return prefill_status(ua::launch_prefill(a, ctl, max_tokens, 0, scratch, sb, reinterpret_cast<hipStream_t>(stream),
                                           -__builtin_huge_valf(), 0, 0, cu_seqlens, total_tokens));
}

size_t ua_backward_workspace_bytes(const ua_dims* dims, int32_t n_tokens) {
  if (check_dims(dims) != UA_OK || n_tokens < 1) return 0;
  return ua::backward_ws_bytes(dims->B, dims->H_q, dims->H_kv, n_tokens);
}

ua_status ua_attention_backward(const ua_dims* dims, int32_t n_tokens, const ua_grad_inputs* in, const ua_grads* out,
                                void* ws, size_t ws_bytes, void* stream) {
  ua_status s;
  if ((s = check_dims(dims)) != UA_OK) return s;
  if (n_tokens < 1 || !in || !out) return UA_ERR_INVALID_ARG;
  const void* tin[3] = {in->q, in->k, in->v};
  for (const void* p : tin)
    if (!p || !aligned(p, 16)) return UA_ERR_INVALID_ARG;
  const float* fin[3] = {in->lq, in->lk, in->lb};
  for (const float* p : fin)
    if (!p || !aligned(p, 4)) return UA_ERR_INVALID_ARG;
  if (!in->dO || !aligned(in->dO, 16)) return UA_ERR_INVALID_ARG;
  float* fout[6] = {out->dq, out->dk, out->dv, out->dlq, out->dlk, out->dlb};
  for (float* p : fout)
    if (!p || !aligned(p, 16)) return UA_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, 256)) return UA_ERR_INVALID_ARG;
  if (ws_bytes < ua::backward_ws_bytes(dims->B, dims->H_q, dims->H_kv, n_tokens)) return UA_ERR_WORKSPACE;
  const float scale = dims->sm_scale > 0.0f ? dims->sm_scale : 1.0f / sqrtf((float)dims->d_head);
  const hipError_t e = ua::launch_backward(dims->B, dims->H_q, dims->H_kv, dims->d_head, n_tokens, dims->terms, scale,
                                           dims->dtype == UA_BF16, in->q, in->k, in->v, in->lq, in->lk, in->lb, in->dO,
                                           out->dq, out->dk, out->dv, out->dlq, out->dlk, out->dlb, ws,
                                           reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? UA_OK : UA_ERR_HIP;
}

ua_status ua_qk_norm(const ua_dims* dims, const float* w_q, const float* w_k, float eps, void* q, void* k,
                     int32_t n_tokens, void* stream) {
  ua_status s;
  if ((s = check_dims(dims)) != UA_OK) return s;
  if (n_tokens < 1 || !(eps >= 0.0f) || !isfinite(eps)) return UA_ERR_INVALID_ARG;
  if (w_q && (!q || !aligned(q, 16) || !aligned(w_q, 4))) return UA_ERR_INVALID_ARG;
  if (w_k && (!k || !aligned(k, 16) || !aligned(w_k, 4))) return UA_ERR_INVALID_ARG;
  const int64_t tok = (int64_t)dims->B * n_tokens;
  const int64_t nq = w_q ? tok * dims->H_q : 0;
  const int64_t nk = w_k ? tok * dims->H_kv : 0;
  const hipError_t e = ua::launch_qk_norm(dims->d_head, dims->dtype == UA_BF16, q, w_q, nq, k, w_k, nk, eps,
                                          reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? UA_OK : UA_ERR_HIP;
}

ua_status ua_compact(const ua_dims* dims, const ua_cache* cache, float log_p, int32_t* kept_idx, void* ws,
                     size_t ws_bytes, void* stream) {
  ua_status s;
  if ((s = check_dims(dims)) != UA_OK) return s;
  if ((s = check_cache(cache)) != UA_OK) return s;
  if (bad_log_p(log_p)) return UA_ERR_INVALID_ARG;
  if (kept_idx && !aligned(kept_idx, 4)) return UA_ERR_INVALID_ARG;
  if (!ws || !aligned(ws, 256)) return UA_ERR_INVALID_ARG;
  LayerArgs a = make_args(dims, nullptr, cache, nullptr, nullptr);
  if (ws_bytes < ua::control_bytes(a) + ua::control_tail_bytes(a)) return UA_ERR_WORKSPACE;
  const ua::Control ctl = ua::control_carve(a, ws, ws_bytes);
  const hipError_t e = ua::launch_compact(a, ctl, log_p, kept_idx, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? UA_OK : UA_ERR_HIP;
}

const char* ua_status_string(int32_t status) {
  switch (status) {
    case UA_OK: return "ok";
    case UA_ERR_INVALID_ARG: return "invalid argument";
    case UA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case UA_ERR_WORKSPACE: return "workspace too small";
    case UA_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int32_t ua_abi_version(void) { return UA_ABI_VERSION; }

}  // extern "C"
