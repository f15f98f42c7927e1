// C ABI of libhsa_attn: host-side validation, workspace sizing and dispatch.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing.  No C++ exception crosses the ABI.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <exception>
#include <initializer_list>
#include <mutex>

#include "../../include/hsa_attn.h"
#include "kernels.hpp"

namespace {

thread_local char g_last_error[512] = "";
thread_local void** g_events = nullptr;
thread_local int g_event_pairs = 0;
thread_local int g_event_next = 0;

void restart_timing() { g_event_next = 0; }

hsa_attn_status_t fail(hsa_attn_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

hsa_attn_status_t ok() {
  g_last_error[0] = '\0';
  return HSA_ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

enum class Call { kLandmarks, kPrefill, kDecode, kDecodeAdaptive, kPrefillAdaptive, kBackward };

// Validates the dimension block and fills a Geometry.
hsa_attn_status_t check_dims(const hsa_attn_dims_t* d, Call call, hsa_attn::Geometry* g) {
  const bool adaptive = call == Call::kDecodeAdaptive || call == Call::kPrefillAdaptive;
  if (!d) return fail(HSA_ATTN_INVALID_ARGUMENT, "dims is NULL");
  if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(HSA_ATTN_INVALID_ARGUMENT, "batch and head counts must be >= 1");
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(HSA_ATTN_INVALID_ARGUMENT, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)", d->num_q_heads,
                d->num_kv_heads);
  if (d->head_dim < 1 || d->chunk_size < 1 || d->top_k < 1)
    return fail(HSA_ATTN_INVALID_ARGUMENT, "head_dim, chunk_size and top_k must be >= 1");
  if (d->seq_len < 0) return fail(HSA_ATTN_INVALID_ARGUMENT, "seq_len must be >= 0");
  if (d->dtype != HSA_ATTN_FP32 && d->dtype != HSA_ATTN_BF16)
    return fail(HSA_ATTN_INVALID_ARGUMENT, "unknown dtype %d", d->dtype);
  if (d->reserved != 0) return fail(HSA_ATTN_INVALID_ARGUMENT, "reserved field must be 0");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(HSA_ATTN_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", d->head_dim);
  const int G = d->num_q_heads / d->num_kv_heads;
  if (call != Call::kLandmarks) {
    if (G != 1 && G != 2 && G != 4 && G != 8)
      return fail(HSA_ATTN_UNSUPPORTED, "query heads per KV head %d unsupported (1, 2, 4, 8)", G);
    if (d->chunk_size != 64) return fail(HSA_ATTN_UNSUPPORTED, "chunk_size %d unsupported (64)", d->chunk_size);
    // decode keeps one list entry per lane of a wave, prefill up to 64 per
    // row in registers; the adaptive budget doubles k; the backward's row
    // preparation spreads a row's slots over 16 lanes, two each
    const int kmax = call == Call::kBackward ? 32 : 64 / (adaptive ? 2 : 1);
    if (d->top_k > kmax) return fail(HSA_ATTN_UNSUPPORTED, "top_k %d unsupported (<= %d)", d->top_k, kmax);
    // prefill lists of more than 32 slots: the local attention's per-row
    // tables of more than four heads per KV head would not fit the LDS
    const bool prefill = call == Call::kPrefill || call == Call::kPrefillAdaptive || call == Call::kBackward;
    if (prefill && d->top_k * (adaptive ? 2 : 1) > 32 && G > 4)
      return fail(HSA_ATTN_UNSUPPORTED, "prefill with more than 32 selection slots needs num_q_heads / num_kv_heads <= 4");
  }
  if (call == Call::kDecodeAdaptive) call = Call::kDecode;
  if (call == Call::kPrefillAdaptive) call = Call::kPrefill;
  if (call == Call::kBackward) {
    if (d->dtype != HSA_ATTN_BF16) return fail(HSA_ATTN_UNSUPPORTED, "the backward pass supports bf16 storage only");
    call = Call::kPrefill;
  }
  const int64_t k_slots = (int64_t)d->top_k * (adaptive ? 2 : 1);
  const int64_t Nc = d->seq_len / d->chunk_size;
  if (call == Call::kPrefill) {
    if (Nc > 65536) return fail(HSA_ATTN_UNSUPPORTED, "prefill supports at most 65536 chunks");
    if ((d->seq_len + 63) / 64 * (int64_t)d->batch * d->num_kv_heads * 2 > 0x7fffffffLL)
      return fail(HSA_ATTN_UNSUPPORTED, "prefill grid too large");
    // remote-pair positions and row indices are int32
    if ((int64_t)d->batch * d->num_q_heads * d->seq_len * k_slots > 0x7fffffffLL)
      return fail(HSA_ATTN_UNSUPPORTED, "prefill: batch * q_heads * seq_len * top_k must stay below 2^31");
  }
  if (call == Call::kDecode && Nc > 0x7fffffffLL) return fail(HSA_ATTN_UNSUPPORTED, "cache too long");
  g->B = d->batch;
  g->Hq = d->num_q_heads;
  g->Hkv = d->num_kv_heads;
  g->G = G;
  g->D = d->head_dim;
  g->S = d->chunk_size;
  g->k = d->top_k;
  g->T = d->seq_len;
  if (adaptive) g->k = 2 * d->top_k;  // the list holds the doubled budget
  g->Nc = Nc;
  g->bf16 = d->dtype == HSA_ATTN_BF16;
  g->Tq = d->seq_len;  // every position is a query row unless a caller narrows it
  g->J0 = 0;
  return HSA_ATTN_OK;
}

hsa_attn_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(HSA_ATTN_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

// ---- debug build (HSA_ATTN_DEBUG=1): the first 256 bytes of every workspace
// hold the call's flag word; before its kernels a call clears the word and
// fills the rest of the workspace it uses and its outputs with kPoison
#ifndef HSA_ATTN_DEBUG
#define HSA_ATTN_DEBUG 0
#endif
constexpr size_t kDebugHeader = HSA_ATTN_DEBUG ? 256 : 0;
constexpr uint32_t kPoison = 0x7FC00001u;  // a quiet NaN as fp32; 2143289345 as int32

__global__ void debug_fill_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

struct Region {
  void* p;
  size_t bytes;  // a multiple of 4
};

// Debug builds: clear the flag word at `workspace` (the start of the
// caller's workspace) and poison `regions`; the flag word's device address
// for the kernels.  Release builds: nothing, and no flag word.
hsa_attn_status_t debug_prepare(void* workspace, std::initializer_list<Region> regions, hipStream_t st,
                                uint32_t** dbg) {
  *dbg = nullptr;
  if constexpr (HSA_ATTN_DEBUG) {
    hipLaunchKernelGGL(debug_fill_kernel, dim3(1), dim3(64), 0, st, static_cast<uint32_t*>(workspace),
                       (int64_t)(kDebugHeader / 4), 0u);
    for (const Region& r : regions) {
      if (!r.p || r.bytes < 4) continue;
      const int64_t n = (int64_t)(r.bytes / 4);
      hipLaunchKernelGGL(debug_fill_kernel, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 16384)), dim3(256), 0,
                         st, static_cast<uint32_t*>(r.p), n, kPoison);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e, "debug workspace fill");
    *dbg = static_cast<uint32_t*>(workspace);
  }
  return HSA_ATTN_OK;
}

}  // namespace

bool hsa_attn::next_timing_pair(hipEvent_t* start, hipEvent_t* stop) {
  if (!g_events || g_event_next + 2 > 2 * g_event_pairs) return false;
  *start = static_cast<hipEvent_t>(g_events[g_event_next]);
  *stop = static_cast<hipEvent_t>(g_events[g_event_next + 1]);
  g_event_next += 2;
  return true;
}

extern "C" {

hsa_attn_status_t hsa_attn_set_timing_events(void** events, int n_pairs) {
  if (n_pairs < 0) return fail(HSA_ATTN_INVALID_ARGUMENT, "n_pairs must be >= 0");
  if (n_pairs > 0 && !events) return fail(HSA_ATTN_INVALID_ARGUMENT, "events is NULL");
  g_events = n_pairs > 0 ? events : nullptr;
  g_event_pairs = n_pairs;
  g_event_next = 0;
  return ok();
}


const char* hsa_attn_status_string(hsa_attn_status_t s) {
  switch (s) {
    case HSA_ATTN_OK: return "ok";
    case HSA_ATTN_INVALID_ARGUMENT: return "invalid argument";
    case HSA_ATTN_UNSUPPORTED: return "unsupported shape or type";
    case HSA_ATTN_WORKSPACE_TOO_SMALL: return "workspace too small";
    case HSA_ATTN_HIP_ERROR: return "HIP error";
  }
  return "unknown status";
}

const char* hsa_attn_last_error(void) { return g_last_error; }

hsa_attn_status_t hsa_attn_workspace_size(const hsa_attn_dims_t* d, int is_decode, size_t* bytes) {
  try {
    if (!bytes) return fail(HSA_ATTN_INVALID_ARGUMENT, "bytes is NULL");
    if (is_decode < 0 || is_decode > 4) return fail(HSA_ATTN_INVALID_ARGUMENT, "kind must be 0 .. 4");
    hsa_attn::Geometry g;
    static const Call kinds[5] = {Call::kPrefill, Call::kDecode, Call::kDecodeAdaptive, Call::kPrefillAdaptive,
                                  Call::kBackward};
    const Call call = kinds[is_decode];
    const hsa_attn_status_t st = check_dims(d, call, &g);
    if (st != HSA_ATTN_OK) return st;
    if (is_decode == 4) {
      *bytes = hsa_attn::plan_backward(g).bytes + kDebugHeader;
      return ok();
    }
    // the size assumes the library keeps the selection itself (sel outputs NULL)
    const bool dec = is_decode == 1 || is_decode == 2;
    *bytes = (dec ? hsa_attn::plan_decode(g, true).bytes : hsa_attn::plan_prefill(g, true).bytes) + kDebugHeader;
    return ok();
  } catch (const std::exception& e) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error: %s", e.what());
  } catch (...) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error");
  }
}

hsa_attn_status_t hsa_attn_prefill_slab_rows(const hsa_attn_dims_t* d, int adaptive, int selection_given,
                                             size_t workspace_bytes, int64_t* slab_rows) {
  try {
    if (!slab_rows) return fail(HSA_ATTN_INVALID_ARGUMENT, "slab_rows is NULL");
    hsa_attn::Geometry g;
    const hsa_attn_status_t st = check_dims(d, adaptive ? Call::kPrefillAdaptive : Call::kPrefill, &g);
    if (st != HSA_ATTN_OK) return st;
    const size_t usable = workspace_bytes > kDebugHeader ? workspace_bytes - kDebugHeader : 0;
    *slab_rows = hsa_attn::plan_prefill_for(g, selection_given == 0, usable).slab_rows;
    return ok();
  } catch (const std::exception& e) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error: %s", e.what());
  } catch (...) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error");
  }
}

hsa_attn_status_t hsa_build_landmarks(const hsa_attn_dims_t* d, const void* k, void* landmarks, int64_t chunk_begin,
                                      int64_t chunk_end, void* stream) {
  try {
    hsa_attn::Geometry g;
    hsa_attn_status_t st = check_dims(d, Call::kLandmarks, &g);
    if (st != HSA_ATTN_OK) return st;
    if (chunk_begin < 0 || chunk_begin > chunk_end || chunk_end > g.Nc)
      return fail(HSA_ATTN_INVALID_ARGUMENT, "chunk range [%lld, %lld) outside [0, %lld]", (long long)chunk_begin,
                  (long long)chunk_end, (long long)g.Nc);
    if (chunk_begin == chunk_end) return ok();  // nothing to build; pointers may be NULL
    if (!k || !landmarks) return fail(HSA_ATTN_INVALID_ARGUMENT, "k and landmarks must be non-NULL");
    if (!aligned16(k) || !aligned16(landmarks)) return fail(HSA_ATTN_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
    restart_timing();
    hsa_attn::LandmarkArgs a{k, landmarks, (int64_t)g.B * g.Hkv, g.T, g.Nc, chunk_begin, chunk_end, g.S, g.D, g.bf16};
    return hip_status(hsa_attn::launch_landmarks(a, static_cast<hipStream_t>(stream)), "landmark launch");
  } catch (const std::exception& e) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error: %s", e.what());
  } catch (...) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error");
  }
}

// gap_tau < 0: plain top-k; otherwise the adaptive budget with threshold gap_tau
static hsa_attn_status_t forward_prefill(const hsa_attn_dims_t* d, int64_t q_offset, const void* q, const void* k,
                                         const void* v, const void* landmarks, float* out, int32_t* sel_idx,
                                         float* sel_score, void* workspace, size_t workspace_bytes, void* stream,
                                         float gap_tau = -1.0f) {
  try {
    hsa_attn::Geometry g;
    const bool adaptive = gap_tau >= 0.0f;
    hsa_attn_status_t st = check_dims(d, adaptive ? Call::kPrefillAdaptive : Call::kPrefill, &g);
    if (st != HSA_ATTN_OK) return st;
    if (q_offset < 0 || q_offset > g.T || q_offset % g.S != 0)
      return fail(HSA_ATTN_INVALID_ARGUMENT, "q_offset %lld must be a multiple of chunk_size in [0, seq_len]",
                  (long long)q_offset);
    g.Tq = g.T - q_offset;
    g.J0 = q_offset / g.S;
    // no query rows (an empty sequence, or no new tokens after the prefix):
    // nothing is read or written, so empty buffers may be NULL
    if (g.Tq == 0) return ok();
    if (!q || !k || !v || !out || (!landmarks && g.Nc > 0))
      return fail(HSA_ATTN_INVALID_ARGUMENT, "q, k, v, landmarks and out must be non-NULL");
    if ((sel_idx == nullptr) != (sel_score == nullptr))
      return fail(HSA_ATTN_INVALID_ARGUMENT, "sel_idx and sel_score must both be given or both be NULL");
    for (const void* p : {q, k, v, landmarks, (const void*)out, (const void*)sel_idx, (const void*)sel_score,
                          (const void*)workspace})
      if (p && !aligned16(p)) return fail(HSA_ATTN_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
    const bool own = sel_idx == nullptr;
    // the largest slabs of query rows the workspace holds
    const size_t usable = workspace_bytes > kDebugHeader ? workspace_bytes - kDebugHeader : 0;
    const hsa_attn::PrefillPlan plan = hsa_attn::plan_prefill_for(g, own, usable);
    if (plan.slab_rows == 0)
      return fail(HSA_ATTN_WORKSPACE_TOO_SMALL, "workspace needs at least %zu bytes (slabs of 64 query rows), got %zu",
                  plan.bytes + kDebugHeader, workspace_bytes);
    if (!workspace) return fail(HSA_ATTN_INVALID_ARGUMENT, "workspace is NULL");
    char* ws = static_cast<char*>(workspace) + kDebugHeader;
    const size_t rows_q = (size_t)g.B * g.Hq * (size_t)g.Tq;
    uint32_t* dbg = nullptr;
    st = debug_prepare(workspace,
                       {{ws, plan.bytes},
                        {out, rows_q * g.D * sizeof(float)},
                        {own ? nullptr : sel_idx, rows_q * g.k * sizeof(int32_t)},
                        {own ? nullptr : sel_score, rows_q * g.k * sizeof(float)}},
                       static_cast<hipStream_t>(stream), &dbg);
    if (st != HSA_ATTN_OK) return st;
    if (own) {
      sel_idx = reinterpret_cast<int32_t*>(ws + plan.off_sel_idx);
      sel_score = reinterpret_cast<float*>(ws + plan.off_sel_score);
    }
    restart_timing();
    hsa_attn::PrefillArgs a{g, q, k, v, landmarks, out, sel_idx, sel_score,
                            reinterpret_cast<int32_t*>(ws + plan.off_pair_pos), reinterpret_cast<int*>(ws + plan.off_cnt),
                            reinterpret_cast<int*>(ws + plan.off_off), reinterpret_cast<int32_t*>(ws + plan.off_pairs),
                            reinterpret_cast<float*>(ws + plan.off_partial), ws + plan.off_vt, plan.slab_rows,
                            plan.slab_group};
    if (adaptive) {
      a.k_base = d->top_k;
      a.gap_tau = gap_tau;
    }
    a.dbg = dbg;
    return hip_status(hsa_attn::launch_prefill(a, static_cast<hipStream_t>(stream)), "prefill launch");
  } catch (const std::exception& e) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error: %s", e.what());
  } catch (...) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error");
  }
}

hsa_attn_status_t hsa_forward_prefill(const hsa_attn_dims_t* d, const void* q, const void* k, const void* v,
                                      const void* landmarks, float* out, int32_t* sel_idx, float* sel_score,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return forward_prefill(d, 0, q, k, v, landmarks, out, sel_idx, sel_score, workspace, workspace_bytes, stream);
}

hsa_attn_status_t hsa_forward_prefill_cached(const hsa_attn_dims_t* d, int64_t q_offset, const void* q,
                                             const void* k, const void* v, const void* landmarks, float* out,
                                             int32_t* sel_idx, float* sel_score, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  return forward_prefill(d, q_offset, q, k, v, landmarks, out, sel_idx, sel_score, workspace, workspace_bytes,
                         stream);
}

// gap_tau < 0: plain top-k; otherwise the adaptive budget with threshold gap_tau
hsa_attn_status_t hsa_forward_prefill_adaptive(const hsa_attn_dims_t* d, float gap_threshold, const void* q,
                                               const void* k, const void* v, const void* landmarks, float* out,
                                               int32_t* sel_idx, float* sel_score, void* workspace,
                                               size_t workspace_bytes, void* stream) {
  if (!(gap_threshold >= 0.0f))
    return fail(HSA_ATTN_INVALID_ARGUMENT, "gap_threshold must be >= 0 (or +inf), got %g", (double)gap_threshold);
  return forward_prefill(d, 0, q, k, v, landmarks, out, sel_idx, sel_score, workspace, workspace_bytes, stream,
                         gap_threshold);
}

hsa_attn_status_t hsa_backward_prefill(const hsa_attn_dims_t* d, const void* q, const void* k, const void* v,
                                       const void* landmarks, const float* out, const float* dout,
                                       const int32_t* sel_idx, const float* sel_score, float* dq, float* dk, float* dv,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  try {
    hsa_attn::Geometry g;
    hsa_attn_status_t st = check_dims(d, Call::kBackward, &g);
    if (st != HSA_ATTN_OK) return st;
    if (g.T == 0) return ok();  // an empty sequence: nothing is read or written (empty buffers may be NULL)
    if (!q || !k || !v || !out || !dout || !sel_idx || !sel_score || !dq || !dk || !dv || (!landmarks && g.Nc > 0))
      return fail(HSA_ATTN_INVALID_ARGUMENT,
                  "q, k, v, landmarks, out, dout, sel_idx, sel_score, dq, dk and dv must be non-NULL");
    for (const void* p : {q, k, v, landmarks, (const void*)out, (const void*)dout, (const void*)sel_idx,
                          (const void*)sel_score, (const void*)dq, (const void*)dk, (const void*)dv,
                          (const void*)workspace})
      if (p && !aligned16(p)) return fail(HSA_ATTN_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
    const hsa_attn::BackwardPlan plan = hsa_attn::plan_backward(g);
    if (workspace_bytes < plan.bytes + kDebugHeader)
      return fail(HSA_ATTN_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", plan.bytes + kDebugHeader,
                  workspace_bytes);
    if (!workspace) return fail(HSA_ATTN_INVALID_ARGUMENT, "workspace is NULL");
    char* ws = static_cast<char*>(workspace) + kDebugHeader;
    const size_t qe = (size_t)g.B * g.Hq * (size_t)g.T * g.D, ke = (size_t)g.B * g.Hkv * (size_t)g.T * g.D;
    uint32_t* dbg = nullptr;
    st = debug_prepare(workspace,
                       {{ws, plan.bytes}, {dq, qe * sizeof(float)}, {dk, ke * sizeof(float)}, {dv, ke * sizeof(float)}},
                       static_cast<hipStream_t>(stream), &dbg);
    if (st != HSA_ATTN_OK) return st;
    restart_timing();
    hsa_attn::BackwardArgs a{g,  q,  k,  v,  landmarks, out, dout, sel_idx, sel_score,
                             dq, dk, dv, ws};
    a.dbg = dbg;
    return hip_status(hsa_attn::launch_backward(a, plan, static_cast<hipStream_t>(stream)), "backward launch");
  } catch (const std::exception& e) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error: %s", e.what());
  } catch (...) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error");
  }
}

static hsa_attn_status_t forward_decode(const hsa_attn_dims_t* d, const void* q, const void* k_cache,
                                        const void* v_cache, const void* landmarks, const int64_t* lens, float* out,
                                        int32_t* sel_idx, float* sel_score, void* workspace, size_t workspace_bytes,
                                        void* stream, float gap_tau = -1.0f) {
  try {
    hsa_attn::Geometry g;
    const bool adaptive = gap_tau >= 0.0f;
    hsa_attn_status_t st = check_dims(d, adaptive ? Call::kDecodeAdaptive : Call::kDecode, &g);
    if (st != HSA_ATTN_OK) return st;
    if (!q || !out || (g.Nc > 0 && (!k_cache || !v_cache || !landmarks)))
      return fail(HSA_ATTN_INVALID_ARGUMENT, "q, k_cache, v_cache, landmarks and out must be non-NULL");
    if ((sel_idx == nullptr) != (sel_score == nullptr))
      return fail(HSA_ATTN_INVALID_ARGUMENT, "sel_idx and sel_score must both be given or both be NULL");
    for (const void* p : {q, k_cache, v_cache, landmarks, (const void*)out, (const void*)sel_idx,
                          (const void*)sel_score, (const void*)workspace})
      if (p && !aligned16(p)) return fail(HSA_ATTN_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
    if (lens && (reinterpret_cast<uintptr_t>(lens) & 7u) != 0)
      return fail(HSA_ATTN_INVALID_ARGUMENT, "cache_lens must be 8-byte aligned");
    const bool own = sel_idx == nullptr;
    const hsa_attn::DecodePlan plan = hsa_attn::plan_decode(g, own);
    if (workspace_bytes < plan.bytes + kDebugHeader)
      return fail(HSA_ATTN_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", plan.bytes + kDebugHeader,
                  workspace_bytes);
    if (!workspace) return fail(HSA_ATTN_INVALID_ARGUMENT, "workspace is NULL");
    char* ws = static_cast<char*>(workspace) + kDebugHeader;
    const size_t rows_q = (size_t)g.B * g.Hq;
    uint32_t* dbg = nullptr;
    st = debug_prepare(workspace,
                       {{ws, plan.bytes},
                        {out, rows_q * g.D * sizeof(float)},
                        {own ? nullptr : sel_idx, rows_q * g.k * sizeof(int32_t)},
                        {own ? nullptr : sel_score, rows_q * g.k * sizeof(float)}},
                       static_cast<hipStream_t>(stream), &dbg);
    if (st != HSA_ATTN_OK) return st;
    if (own) {
      sel_idx = reinterpret_cast<int32_t*>(ws + plan.off_sel_idx);
      sel_score = reinterpret_cast<float*>(ws + plan.off_sel_score);
    }
    restart_timing();
    hsa_attn::DecodeArgs a{g, q, k_cache, v_cache, landmarks, out, sel_idx, sel_score, ws, lens};
    if (adaptive) {
      a.k_base = d->top_k;
      a.gap_tau = gap_tau;
    }
    a.dbg = dbg;
    return hip_status(hsa_attn::launch_decode(a, plan, static_cast<hipStream_t>(stream)), "decode launch");
  } catch (const std::exception& e) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error: %s", e.what());
  } catch (...) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error");
  }
}

hsa_attn_status_t hsa_forward_decode(const hsa_attn_dims_t* d, const void* q, const void* k_cache,
                                     const void* v_cache, const void* landmarks, float* out, int32_t* sel_idx,
                                     float* sel_score, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_decode(d, q, k_cache, v_cache, landmarks, nullptr, out, sel_idx, sel_score, workspace,
                        workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- decode without a workspace
// Device memory the no-allocation decode uses in place of a caller
// workspace: a fixed array in the library's code object, one copy per GPU,
// alive until the process ends.  Host code never passes `scratch` itself
// (its host-side name is not a device address): the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
namespace {
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's copy of `scratch`, looked up on the first call there
hsa_attn_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(HSA_ATTN_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(HSA_ATTN_HIP_ERROR, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HSA_ATTN_OK;
}
}  // namespace

extern "C" {

hsa_attn_status_t hsa_forward_decode_noalloc(const hsa_attn_dims_t* d, const void* q, const void* k_cache,
                                             const void* v_cache, const void* landmarks, float* out,
                                             int32_t* sel_idx, float* sel_score, void* stream) {
  try {
    // size the work before any HIP call: a call that does not fit is
    // rejected without touching the device
    hsa_attn::Geometry g;
    hsa_attn_status_t st = check_dims(d, Call::kDecode, &g);
    if (st != HSA_ATTN_OK) return st;
    const size_t need = hsa_attn::plan_decode(g, sel_idx == nullptr).bytes + kDebugHeader;
    if (need > kScratchBytes)
      return fail(HSA_ATTN_WORKSPACE_TOO_SMALL,
                  "decode needs %zu bytes of scratch; the no-allocation entry point holds %zu (use "
                  "hsa_forward_decode with a workspace)",
                  need, kScratchBytes);
    void* ws = nullptr;
    st = scratch_address(&ws);
    if (st != HSA_ATTN_OK) return st;
    return forward_decode(d, q, k_cache, v_cache, landmarks, nullptr, out, sel_idx, sel_score, ws, kScratchBytes,
                          stream);
  } catch (const std::exception& e) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error: %s", e.what());
  } catch (...) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error");
  }
}

hsa_attn_status_t hsa_attn_debug_flags(const void* workspace, uint32_t* flags) {
  try {
    if constexpr (!HSA_ATTN_DEBUG) {
      (void)workspace;
      (void)flags;
      return fail(HSA_ATTN_UNSUPPORTED, "this library is built without HSA_ATTN_DEBUG (libhsa_attn_debug.so has it)");
    } else {
      if (!flags) return fail(HSA_ATTN_INVALID_ARGUMENT, "flags is NULL");
      void* p = const_cast<void*>(workspace);
      if (!p) {
        const hsa_attn_status_t st = scratch_address(&p);
        if (st != HSA_ATTN_OK) return st;
      }
      hipError_t e = hipDeviceSynchronize();
      if (e != hipSuccess) return hip_status(e, "hipDeviceSynchronize");
      e = hipMemcpy(flags, p, sizeof(uint32_t), hipMemcpyDeviceToHost);
      return hip_status(e, "flag word copy");
    }
  } catch (const std::exception& e) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error: %s", e.what());
  } catch (...) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error");
  }
}

hsa_attn_status_t hsa_forward_decode_varlen(const hsa_attn_dims_t* d, const void* q, const void* k_cache,
                                            const void* v_cache, const void* landmarks, const int64_t* cache_lens,
                                            float* out, int32_t* sel_idx, float* sel_score, void* workspace,
                                            size_t workspace_bytes, void* stream) {
  if (!cache_lens) return fail(HSA_ATTN_INVALID_ARGUMENT, "cache_lens is NULL");
  return forward_decode(d, q, k_cache, v_cache, landmarks, cache_lens, out, sel_idx, sel_score, workspace,
                        workspace_bytes, stream);
}

hsa_attn_status_t hsa_forward_decode_adaptive(const hsa_attn_dims_t* d, float gap_threshold, const void* q,
                                              const void* k_cache, const void* v_cache, const void* landmarks,
                                              const int64_t* cache_lens, float* out, int32_t* sel_idx,
                                              float* sel_score, void* workspace, size_t workspace_bytes,
                                              void* stream) {
  if (!(gap_threshold >= 0.0f))
    return fail(HSA_ATTN_INVALID_ARGUMENT, "gap_threshold must be >= 0 (or +inf), got %g", (double)gap_threshold);
  return forward_decode(d, q, k_cache, v_cache, landmarks, cache_lens, out, sel_idx, sel_score, workspace,
                        workspace_bytes, stream, gap_threshold);
}

hsa_attn_status_t hsa_append_kv(const hsa_attn_dims_t* d, const void* k_new, const void* v_new, void* k_cache,
                                void* v_cache, void* landmarks, int64_t* cache_lens, void* stream) {
  try {
    hsa_attn::Geometry g;
    hsa_attn_status_t st = check_dims(d, Call::kLandmarks, &g);
    if (st != HSA_ATTN_OK) return st;
    if (!k_new || !v_new || !k_cache || !v_cache || !cache_lens || (!landmarks && g.Nc > 0))
      return fail(HSA_ATTN_INVALID_ARGUMENT, "k_new, v_new, k_cache, v_cache, landmarks and cache_lens must be non-NULL");
    for (const void* p : {k_new, v_new, (const void*)k_cache, (const void*)v_cache, (const void*)landmarks})
      if (p && !aligned16(p)) return fail(HSA_ATTN_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(cache_lens) & 7u) != 0)
      return fail(HSA_ATTN_INVALID_ARGUMENT, "cache_lens must be 8-byte aligned");
    restart_timing();
    hsa_attn::AppendArgs a{k_new, v_new, k_cache, v_cache, landmarks, cache_lens, g.B, g.Hkv, g.T, g.Nc, g.S,
                           g.D, g.bf16};
    return hip_status(hsa_attn::launch_append(a, static_cast<hipStream_t>(stream)), "append launch");
  } catch (const std::exception& e) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error: %s", e.what());
  } catch (...) {
    return fail(HSA_ATTN_HIP_ERROR, "internal error");
  }
}

}  // extern "C"
