// Host-side launch interfaces of the HSA kernels (internal to libhsa_attn).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hsa_attn {

// The next caller-provided pair of timing events when per-launch timing is
// enabled on this thread (hsa_attn_set_timing_events); false otherwise.
bool next_timing_pair(hipEvent_t* start, hipEvent_t* stop);

// Every kernel of the library is launched through this: with timing on, the
// next event pair is recorded on the stream just before and just after the
// launch.  (Handing the pair to the launch itself, hipExtLaunchKernelGGL,
// costs fewer microseconds per launch, but the runtime then holds on to the
// device memory the timed kernels touched for as long as the events live.)
template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t st, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const bool timed = next_timing_pair(&e0, &e1);
  if (timed) (void)hipEventRecord(e0, st);
  hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
  if (timed) (void)hipEventRecord(e1, st);
}

struct LandmarkArgs {
  const void* k;
  void* lm;
  int64_t bh;      // B * Hkv
  int64_t T;       // tokens per (b, g) in k
  int64_t Nc;      // landmark rows per (b, g)
  int64_t c0, c1;  // chunk range to build
  int S, D;
  bool bf16;
};
hipError_t launch_landmarks(const LandmarkArgs& a, hipStream_t st);

// one new token per sequence appended at position lens[b] of caches with
// capacity T; a chunk it completes gets its landmark; lens[b] advances
struct AppendArgs {
  const void *k_new, *v_new;
  void *k, *v, *lm;
  int64_t* lens;
  int B, Hkv;
  int64_t T, Nc;
  int S, D;
  bool bf16;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t st);

// Geometry shared by the forward passes.
struct Geometry {
  int B, Hq, Hkv, G, D, S, k;
  int64_t T;    // prefill: key length; decode: cache length (capacity)
  int64_t Nc;   // floor(T / S)
  bool bf16;
  int64_t Tq = 0;  // prefill: query rows, the last Tq of the T positions
  int64_t J0 = 0;  // prefill: (T - Tq) / S, the chunk of the first query row
};

// ---------------------------------------------------------------- decode
struct DecodePlan {
  int splits;          // landmark-scan workgroups per (b, g)
  int rows_per_split;  // landmarks per split (multiple of 64)
  size_t off_cand, off_sel_idx, off_sel_score, off_partial, off_ulist, off_ucount, bytes;
};
DecodePlan plan_decode(const Geometry& g, bool own_sel);

struct DecodeArgs {
  Geometry g;
  const void *q, *k, *v, *lm;
  float* out;
  int32_t* sel_idx;
  float* sel_score;
  void* ws;
  const int64_t* lens;  // per-sequence cache lengths (device), or null: all g.T
  // adaptive budget: 0 = plain top-g.k; otherwise g.k == 2 * k_base and a
  // head keeps g.k entries only when its k_base-th vs (k_base+1)-th score
  // gap is below gap_tau
  int k_base = 0;
  float gap_tau = 0.0f;
  uint32_t* dbg = nullptr;  // debug builds: the call's flag word
};
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t st);

// ---------------------------------------------------------------- prefill
// The query rows are processed in slabs of slab_rows rows (a multiple of 64;
// the last slab may be shorter): the chunk-major pairs of one slab and their
// outputs are all the workspace has to hold at a time, so the workspace is
// the per-call part (selection when the library keeps it, pair positions,
// bucket counts and pair lists, transposed V) plus one slab's worst case of
// chunk-major pair outputs (every pair chunk-major).
struct PrefillPlan {
  size_t off_sel_idx, off_sel_score, off_pair_pos, off_cnt, off_off, off_pairs, off_partial, off_vt, bytes;
  int64_t slab_rows;  // 0: the workspace cannot hold one slab of 64 rows
  int slab_group;     // slabs whose pairs one selection launch counts (their bucket counts side by side)
};
// at most this many slabs' bucket counts are kept at once
constexpr int kPrefillCountSlabs = 64;
// Fixed part and per-row part of the workspace (bytes).
void prefill_workspace_parts(const Geometry& g, bool own_sel, size_t* fixed, size_t* per_row);
// The plan for slabs of at most `slab_rows` rows (rounded to whole 64-row
// chunks; at least one chunk, at most the whole call).
PrefillPlan plan_prefill_slab(const Geometry& g, bool own_sel, int64_t slab_rows);
// The plan with the largest slabs a workspace of `bytes` holds (slabs of
// equal numbers of 64-row chunks; slab_rows = 0 when not even one fits).
PrefillPlan plan_prefill_for(const Geometry& g, bool own_sel, size_t bytes);
// The default plan (hsa_attn_workspace_size): one slab when its worst case
// holds at most kPrefillSlabBudget bytes of chunk-major pairs, else equal
// slabs that each stay within it.
constexpr size_t kPrefillSlabBudget = size_t(16) << 30;
PrefillPlan plan_prefill(const Geometry& g, bool own_sel);

struct PrefillArgs {
  Geometry g;
  const void *q, *k, *v, *lm;
  float* out;
  int32_t* sel_idx;
  float* sel_score;
  // workspace: remote-pair bucketing and the remote pairs' outputs
  int32_t* pair_pos;  // [B, Hq, Tq, k]
  int* cnt;           // [slab_group][B * Hkv * Nc]
  int* off;           // [slab_group][B * Hkv * Nc + 1]
  int32_t* pairs;     // [slab_group][B * Hq * slab_rows * k] (each slab's worst case)
  float* partial;     // [B * Hq * slab_rows * k, D] (one slab's worst case)
  void* vt;           // [B, Hkv, Nc, D, 64] transposed V tiles (storage dtype)
  int64_t slab_rows;  // query rows per slab (multiple of 64)
  int slab_group;     // slabs per selection launch
  // adaptive budget, as in DecodeArgs: g.k == 2 * k_base when k_base > 0
  int k_base = 0;
  float gap_tau = 0.0f;
  uint32_t* dbg = nullptr;  // debug builds: the call's flag word
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st);

// shared by the forward and backward bucketing: p[0..n) = 0; off[0..n] =
// exclusive prefix sum of cnt[0..n) (off[n] = total)
hipError_t launch_zero_ints(int* p, int64_t n, hipStream_t st);
hipError_t launch_exclusive_scan(const int* cnt, int* off, int64_t n, hipStream_t st);

// ---------------------------------------------------------------- backward
struct BackwardPlan {
  size_t off_kt, off_cnt, off_off, off_pair_pos, off_pairs, off_w, off_delta, off_dqp, bytes;
};
BackwardPlan plan_backward(const Geometry& g);

struct BackwardArgs {
  Geometry g;  // g.k = selection slots per row
  const void *q, *k, *v, *lm;
  const float *out, *dout;
  const int32_t* sel_idx;
  const float* sel_score;
  float *dq, *dk, *dv;
  void* ws;
  uint32_t* dbg = nullptr;  // debug builds: the call's flag word
};
hipError_t launch_backward(const BackwardArgs& a, const BackwardPlan& p, hipStream_t st);

}  // namespace hsa_attn
