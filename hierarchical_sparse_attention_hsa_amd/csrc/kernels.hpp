// Host-side launch interfaces of the HSA kernels (internal to libhsa_attn).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hsa_attn {

// Records the next caller-provided timing event on `st` when per-launch
// timing is enabled on this thread (hsa_attn_set_timing_events); no-op otherwise.
void mark_launch(hipStream_t st);

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
};
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t st);

// ---------------------------------------------------------------- prefill
struct PrefillPlan {
  size_t off_sel_idx, off_sel_score, off_pair_pos, off_cnt, off_off, off_pairs, off_partial, off_vt, bytes;
};
PrefillPlan plan_prefill(const Geometry& g, bool own_sel);

struct PrefillArgs {
  Geometry g;
  const void *q, *k, *v, *lm;
  float* out;
  int32_t* sel_idx;
  float* sel_score;
  // workspace: remote-pair bucketing and the remote pairs' outputs
  int32_t* pair_pos;  // [B, Hq, T, k]
  int* cnt;           // [B * Hkv * Nc]
  int* off;           // [B * Hkv * Nc + 1]
  int32_t* pairs;     // [B * Hq * T * k] (worst case)
  float* partial;     // [B * Hq * T * k, D] (worst case)
  void* vt;           // [B, Hkv, Nc, D, 64] transposed V tiles (storage dtype)
  // adaptive budget, as in DecodeArgs: g.k == 2 * k_base when k_base > 0
  int k_base = 0;
  float gap_tau = 0.0f;
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
};
hipError_t launch_backward(const BackwardArgs& a, const BackwardPlan& p, hipStream_t st);

}  // namespace hsa_attn
