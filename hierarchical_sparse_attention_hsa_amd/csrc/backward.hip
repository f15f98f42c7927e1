// HSA backward pass of the causal prefill: gradients of the layer output with
// respect to Q, K and V for an upstream gradient dOut, with the forward's
// selection held fixed (it is piecewise constant) and the landmark's
// rounding taken as the identity, so every key of a chunk receives 1/S of
// its landmark's gradient (skill card "Every Token Counts 16m Context",
// sections "Core Technique" and "Implementation"; the chain rule through its
// steps).  Per kept (row, chunk) pair, with w the fusion weight, a the
// in-chunk probabilities, g = dOut of the row and delta = g . out:
//
//   do = w g,  da_t = do . v_t,  u = sum_t a_t da_t (= do . o_c)
//   dlogit_t = a_t (da_t - u),   ds = u - w delta
//   dv_t += a_t do
//   dk_t += (dlogit_t + ds / S) q / sqrt(D)
//   dq   += (sum_t dlogit_t k_t + ds L_c) / sqrt(D)
//
// Kernels, in launch order: clear the bucket counts; bwd_prep (per row:
// delta, the fusion weights, and the bucketing of every kept pair by
// (b, g, chunk)); exclusive scan; bwd_scatter (bucket lists of pair ids);
// K^T tiles (prefill_vt_kernel on K); bwd_chunk (one workgroup per bucket:
// everything above on MFMA, dK/dV of the chunk accumulated in registers, one
// dq partial per pair); bwd_dq (sums each row's partials); zeros for the
// tokens after the last complete chunk.  Storage dtype bf16.
#include <climits>

#include "prefill_kernels.hpp"

namespace hsa_attn {

// ---------------------------------------------------------------- 1. rows
// 16 lanes per row; a workgroup takes 64 consecutive rows of the [B, Hq, T]
// order, 16 at a time (all loads issued first).  The workgroup groups its
// kept pairs by bucket in an LDS hash table, so each distinct bucket costs
// one global atomic; pair_pos gets each pair's position inside its bucket
// (-1: no pair).
constexpr int kPrepRows = 64;
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const float* __restrict__ out, const float* __restrict__ dout,
                                                       const int32_t* __restrict__ sel_idx,
                                                       const float* __restrict__ sel_score, float* __restrict__ wts,
                                                       float* __restrict__ delta, int* __restrict__ cnt,
                                                       int32_t* __restrict__ pair_pos, int64_t rows, int Hq, int G,
                                                       int64_t T_len, int64_t Nc, int k) {
  constexpr int SUB = kPrepRows / 16;    // rows per thread group of 16 lanes
  constexpr int HASH = 4096;             // >= 64 rows x 32 slots
  constexpr int DV = D / 64;             // float4 loads per lane and row
  __shared__ int hkey[HASH];
  __shared__ int hcnt[HASH];
  const int tid = threadIdx.x, j = tid & 15;
  for (int i = tid; i < HASH; i += 256) {
    hkey[i] = -1;
    hcnt[i] = 0;
  }
  int64_t row[SUB];
  bool rok[SUB];
  f32x4 xo[SUB][DV], xg[SUB][DV];
  int cc[SUB][2];
  float s[SUB][2];
#pragma unroll
  for (int u = 0; u < SUB; ++u) {
    row[u] = (int64_t)blockIdx.x * kPrepRows + 16 * u + (tid >> 4);
    rok[u] = row[u] < rows;
#pragma unroll
    for (int x = 0; x < DV; ++x) {
      const int d = 4 * j + 64 * x;
      const f32x4 z{0.f, 0.f, 0.f, 0.f};
      xo[u][x] = rok[u] ? *reinterpret_cast<const f32x4*>(out + row[u] * D + d) : z;
      xg[u][x] = rok[u] ? *reinterpret_cast<const f32x4*>(dout + row[u] * D + d) : z;
    }
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int e = j + 16 * v;
      const bool inl = rok[u] && e < k;
      cc[u][v] = inl ? sel_idx[row[u] * k + e] : -1;
      s[u][v] = inl ? sel_score[row[u] * k + e] : -__builtin_inff();
    }
  }
  __syncthreads();  // the hash table is cleared
  uint32_t slot_rank[SUB][2];
#pragma unroll
  for (int u = 0; u < SUB; ++u) {
    // delta = dout . out
    float acc = 0.0f;
#pragma unroll
    for (int x = 0; x < DV; ++x)
      acc = fmaf(xo[u][x][0], xg[u][x][0],
                 fmaf(xo[u][x][1], xg[u][x][1], fmaf(xo[u][x][2], xg[u][x][2], fmaf(xo[u][x][3], xg[u][x][3], acc))));
    acc = group_sum<16>(acc);
    if (rok[u] && j == 0) delta[row[u]] = acc;
    // fusion weights: softmax over the row's kept (and valid) scores
    const int64_t t = rok[u] ? row[u] % T_len : 0;
    const int64_t bh = rok[u] ? row[u] / T_len : 0;
    const int h = (int)(bh % Hq);
    const int64_t b = bh / Hq;
    const int64_t n = min(t / kChunk, Nc);
    bool v[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      v[x] = cc[u][x] >= 0 && cc[u][x] < n;
      if (!v[x]) s[u][x] = -__builtin_inff();
    }
    const float mx = group_max<16>(fmaxf(s[u][0], s[u][1]));
    float ex[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) ex[x] = v[x] ? expf(s[u][x] - mx) : 0.0f;
    const float den = group_sum<16>(ex[0] + ex[1]);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int e = j + 16 * x;
      if (rok[u] && e < k) wts[row[u] * k + e] = v[x] ? ex[x] / den : 0.0f;
    }
    // group the pairs by bucket
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      slot_rank[u][x] = ~0u;
      if (!v[x]) continue;
      const int key = (int)(((b * (Hq / G) + h / G) * Nc) + cc[u][x]);
      int sl = (int)(((uint32_t)key * 2654435761u) >> 8) & (HASH - 1);
      while (true) {
        const int prev = atomicCAS(&hkey[sl], -1, key);
        if (prev == -1 || prev == key) break;
        sl = (sl + 1) & (HASH - 1);
      }
      slot_rank[u][x] = ((uint32_t)sl << 16) | (uint32_t)atomicAdd(&hcnt[sl], 1);
    }
  }
  __syncthreads();
  for (int i = tid; i < HASH; i += 256) {
    const int n_i = hcnt[i];
    if (n_i > 0) hcnt[i] = atomicAdd(&cnt[hkey[i]], n_i);  // count -> first position
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < SUB; ++u)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int e = j + 16 * x;
      if (rok[u] && e < k) {
        const uint32_t sr = slot_rank[u][x];
        pair_pos[row[u] * k + e] = sr == ~0u ? -1 : hcnt[sr >> 16] + (int)(sr & 0xffffu);
      }
    }
}

// pairs[off[bucket] + pair_pos[i]] = i (the pair id: row * k + slot).  A
// thread takes V consecutive slots of one row (V divides k): their loads as
// one 16-byte load each (V = 4), the row's bucket base computed once, and
// every slot's bucket offset read at once (a slot without a pair reads the
// base's first entry).
template <int V>
__global__ void bwd_scatter_kernel(const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ pair_pos,
                                   const int* __restrict__ off, int32_t* __restrict__ pairs, int64_t total, int Hq,
                                   int G, int64_t T_len, int64_t Nc, int k, uint32_t* __restrict__ dbg) {
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * V;
  if (i0 >= total) return;
  const int64_t row = i0 / k;
  const int64_t bh = row / T_len;
  const int h = (int)(bh % Hq);
  const int64_t b = bh / Hq;
  const int* ob = off + (b * (Hq / G) + h / G) * Nc;
  int32_t pp[V], c[V];
  if constexpr (V == 4) {
    const u32x4 p4 = *reinterpret_cast<const u32x4*>(pair_pos + i0);
    const u32x4 c4 = *reinterpret_cast<const u32x4*>(sel_idx + i0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      pp[u] = (int32_t)p4[u];
      c[u] = (int32_t)c4[u];
    }
  } else {
#pragma unroll
    for (int u = 0; u < V; ++u) {
      pp[u] = pair_pos[i0 + u];
      c[u] = sel_idx[i0 + u];
    }
  }
  int o[V];
#pragma unroll
  for (int u = 0; u < V; ++u) o[u] = ob[pp[u] >= 0 && c[u] >= 0 && c[u] < Nc ? c[u] : 0];
#pragma unroll
  for (int u = 0; u < V; ++u) {
    if (pp[u] < 0) continue;
    if (!dbg_ok(dbg, c[u] >= 0 && c[u] < Nc, HSA_ATTN_DEBUG_BWD_SCATTER)) continue;
    const int64_t dst = (int64_t)o[u] + pp[u];
    if (!dbg_ok(dbg, dst >= 0 && dst < total, HSA_ATTN_DEBUG_BWD_SCATTER)) continue;
    pairs[dst] = (int32_t)(i0 + u);
  }
}

// ---------------------------------------------------------------- 2. chunks
// One workgroup (4 waves) per bucket (b, g, chunk c).  The chunk's K rows, V
// rows, K^T (tokens in vt_pos order) and landmark row are staged in LDS
// once.  The pairs are taken in rounds of four 32-pair tiles, one per wave:
//   row side (each wave, its own tile): S^T = K Q^T and the softmax, dA^T =
//     V dO^T (dO as a bf16 head + tail), u, dlogit, ds, then
//     dq^T = K^T dlogit^T (head + tail) plus ds L_c, written per pair; the
//     tile's A, dlogit + ds/S (bf16, [token][pair]), dO and Q (bf16,
//     [dim][pair]) are written to the wave's LDS slot;
//   chunk side (after a barrier, every wave over all four slots): dV += A^T dO
//     and dK += (dlogit + ds/S)^T Q on MFMA, contracting over pairs; wave w
//     owns a fixed set of 32x32 output blocks, kept in registers.
// The chunk's dK (times 1/sqrt(D)) and dV are written once at the end
// (zeros for a chunk nobody kept).
// Two fp32 values rounded to bf16 (nearest even) by one packed hardware
// conversion, the first in the low half.
__device__ __forceinline__ uint32_t bf16_pair_bits(float a, float b) {
  const bf16x2 t = __builtin_convertvector((f32x2{a, b}), bf16x2);
  uint32_t u;
  __builtin_memcpy(&u, &t, 4);
  return u;
}

template <int D>
__global__ __launch_bounds__(256) void bwd_chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kk, const uint16_t* __restrict__ vv,
    const uint16_t* __restrict__ kt_g, const uint16_t* __restrict__ lm, const float* __restrict__ dout,
    const float* __restrict__ wts, const float* __restrict__ delta, const int* __restrict__ off,
    const int32_t* __restrict__ pairs, float* __restrict__ dqp, float* __restrict__ dk, float* __restrict__ dv, int k,
    int64_t T_len, int64_t Nc, float scale, int64_t total, uint32_t* __restrict__ dbg) {
  constexpr int KCH = D / 16;            // 16-dim contraction steps
  constexpr int DM = D / 32;             // 32-dim output blocks
  constexpr int ROWB = D * 2;            // bytes of one K or V row
  constexpr int NSL = ROWB / 16;         // its 16-byte slots
  constexpr int VTB = kChunk * 2;        // bytes of one K^T row (64 tokens)
  constexpr int NSLV = VTB / 16;
  constexpr int TB = kChunk * ROWB;      // one staged tile
  constexpr int SA = kChunk * 32 * 2;    // [64 tokens][32 pairs] bf16
  constexpr int SO = D * 32 * 2;         // [D dims][32 pairs] bf16
  constexpr int SLOT = 2 * SA + 2 * SO;  // A, dlogit', dO, Q of one tile
  constexpr int NBW = DM / 2;            // output blocks per wave and matrix
  static_assert(NSL >= 8, "row swizzle needs 8 slots");
  extern __shared__ __align__(16) char smem[];
  char* ks = smem;
  char* vs = smem + TB;
  char* kts = smem + 2 * TB;
  char* stage = smem + 3 * TB;
  char* lms = stage + 4 * SLOT;  // the chunk's landmark row

  const int64_t bucket = blockIdx.x;
  const int64_t c = bucket % Nc, bg = bucket / Nc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  int begin = off[bucket], end = off[bucket + 1];
  if (!dbg_ok(dbg, begin >= 0 && begin <= end && end <= total, HSA_ATTN_DEBUG_BWD_PAIR)) begin = end = 0;
  {
    const char* kb = reinterpret_cast<const char*>(kk + (bg * T_len + c * kChunk) * D);
    const char* vb = reinterpret_cast<const char*>(vv + (bg * T_len + c * kChunk) * D);
    const char* tb = reinterpret_cast<const char*>(kt_g) + bucket * (int64_t)(D * VTB);
    constexpr int NR = kChunk * NSL / kWave;  // load instructions per row tile
    constexpr int NT = D * NSLV / kWave;      // load instructions for K^T
    for (int ii = wave; ii < 2 * NR + NT; ii += 4) {
      const char* src;
      char* dst;
      if (ii < 2 * NR) {
        const int jj = ii % NR;
        const int L = jj * kWave + lane;
        const int t = L / NSL, sp = L % NSL;
        src = (ii < NR ? kb : vb) + t * ROWB + ((sp ^ (t & 7)) * 16);
        dst = (ii < NR ? ks : vs) + jj * kWave * 16;
      } else {
        const int jj = ii - 2 * NR;
        const int L = jj * kWave + lane;
        const int d = L / NSLV, sp = L % NSLV;
        src = tb + d * VTB + ((sp ^ vt_swz(d)) * 16);
        dst = kts + jj * kWave * 16;
      }
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
    if (tid < D / 8)
      *reinterpret_cast<u32x4*>(lms + 16 * tid) = *reinterpret_cast<const u32x4*>(lm + bucket * D + 8 * tid);
    wait_loads();
    __syncthreads();
  }
  const float cexp = scale * 1.4426950408889634f;
  const int ntiles = (end - begin + 31) / 32;
  const int rounds = (ntiles + 3) / 4;
  const int pr = lane & 31;  // this lane's pair column
  char* my = stage + wave * SLOT;
  f32x16 accV[NBW], accK[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    accV[i] = f32x16{};
    accK[i] = f32x16{};
  }

  // The gathered rows of a round's tile (pair id, weight, delta, q, dOut)
  // are fetched one round ahead, while the previous round's chunk side
  // runs; the pair ids two steps ahead, while the row side runs.  Every
  // load is issued unconditionally (a lane past the bucket's end reads
  // element 0 of each array) and masked where its value is used, so the
  // compiler counts each load's completion instead of waiting for all of
  // them at the first use.
  int pid_raw = 0;     // pair id loaded for this lane's next tile
  bool pid_ok = false;
  int pid = 0;         // pair id of the tile being fetched or processed
  bool ok = false;
  float wraw = 0.0f, draw = 0.0f;
  u32x4 qraw[KCH];
  f32x4 graw[2 * KCH];
  auto fetch_id = [&](int t) {
    const int p = begin + 32 * t + pr;
    pid_ok = t < ntiles && p < end;
    pid_raw = pairs[pid_ok ? p : 0];
  };
  auto fetch_rows = [&]() {
    ok = pid_ok && dbg_ok(dbg, pid_raw >= 0 && pid_raw < total, HSA_ATTN_DEBUG_BWD_PAIR);
    pid = ok ? pid_raw : 0;
    const int64_t row = pid / k;
    wraw = wts[pid];
    draw = delta[row];
    const uint16_t* qp = q + row * D + 8 * half;
    const float* gp = dout + row * D + 8 * half;
#pragma unroll
    for (int s = 0; s < KCH; ++s) {
      qraw[s] = *reinterpret_cast<const u32x4*>(qp + 16 * s);
      graw[2 * s] = reinterpret_cast<const f32x4*>(gp + 16 * s)[0];
      graw[2 * s + 1] = reinterpret_cast<const f32x4*>(gp + 16 * s)[1];
    }
  };
  fetch_id(wave);
  fetch_rows();
  for (int r = 0; r < rounds; ++r) {
    const int ti = 4 * r + wave;
    fetch_id(ti + 4);
    if (ti < ntiles) {
      char* At = my;
      char* Lt = my + SA;
      char* Ot = my + 2 * SA;
      char* Qt = my + 2 * SA + SO;
      const float w = ok ? wraw : 0.0f, dlt = ok ? draw : 0.0f;
      // q (B operand: pair column, dims 16 s + 8 half + 0..7) and its staging
      Frag<BF16> qf[KCH];
#pragma unroll
      for (int s = 0; s < KCH; ++s) {
        const u32x4 raw = ok ? qraw[s] : u32x4{0u, 0u, 0u, 0u};
        qf[s].v = as_bf16x8(raw);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int d = 16 * s + 8 * half + i;
          *reinterpret_cast<uint16_t*>(Qt + (d * 32 + pr) * 2) = (uint16_t)(raw[i / 2] >> (16 * (i & 1)));
        }
      }
      // do = w * dout: head + tail fragments, and its bf16 staging
      Frag<BF16> dh[KCH], dtl[KCH];
#pragma unroll
      for (int s = 0; s < KCH; ++s) {
        const f32x4 z{0.f, 0.f, 0.f, 0.f};
        const f32x4 g0 = ok ? graw[2 * s] : z, g1 = ok ? graw[2 * s + 1] : z;
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = w * g0[i];
          x[4 + i] = w * g1[i];
        }
        split_bf16(x, dh[s], dtl[s]);
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const uint32_t pb = bf16_pair_bits(x[i], x[i + 1]);
          const int d = 16 * s + 8 * half + i;
          *reinterpret_cast<uint16_t*>(Ot + (d * 32 + pr) * 2) = (uint16_t)pb;
          *reinterpret_cast<uint16_t*>(Ot + ((d + 1) * 32 + pr) * 2) = (uint16_t)(pb >> 16);
        }
      }
      // S^T = K Q^T over the chunk's two 32-token blocks, softmax per pair
      f32x16 s0 = {}, s1 = {};
      {
        const char* k0 = ks + pr * ROWB;
        const char* k1 = ks + (32 + pr) * ROWB;
#pragma unroll
        for (int s = 0; s < KCH; ++s) {
          Frag<BF16> a0, a1;
          load_frag_lds<BF16>(a0, k0, lane & 7, s, half);
          load_frag_lds<BF16>(a1, k1, lane & 7, s, half);
          mfma(s0, a0, qf[s]);
          mfma(s1, a1, qf[s]);
        }
      }
      float mx = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
      mx = pair_max(mx);
      const float mb = mx * cexp;
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], cexp, -mb));
        s1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], cexp, -mb));
        sum += s0[i] + s1[i];
      }
      sum = pair_sum(sum);
      const float inv = ok ? 1.0f / sum : 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s0[i] *= inv;
        s1[i] *= inv;
      }
      // dA^T = V dO^T
      f32x16 d0 = {}, d1 = {};
      {
        const char* v0 = vs + pr * ROWB;
        const char* v1 = vs + (32 + pr) * ROWB;
#pragma unroll
        for (int s = 0; s < KCH; ++s) {
          Frag<BF16> a0, a1;
          load_frag_lds<BF16>(a0, v0, lane & 7, s, half);
          load_frag_lds<BF16>(a1, v1, lane & 7, s, half);
          mfma(d0, a0, dh[s]);
          mfma(d0, a0, dtl[s]);
          mfma(d1, a1, dh[s]);
          mfma(d1, a1, dtl[s]);
        }
      }
      float u = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) u = fmaf(s0[i], d0[i], fmaf(s1[i], d1[i], u));
      u = pair_sum(u);
      const float ds = u - w * dlt;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        d0[i] = s0[i] * (d0[i] - u);
        d1[i] = s1[i] * (d1[i] - u);
      }
      // staging of A and dlogit + ds/S: [token][pair]
      const float dss = ds * (1.0f / kChunk);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t0 = tile_row(i, half), t1 = 32 + tile_row(i, half);
        const uint32_t pa = bf16_pair_bits(s0[i], s1[i]), pl = bf16_pair_bits(d0[i] + dss, d1[i] + dss);
        *reinterpret_cast<uint16_t*>(At + (t0 * 32 + pr) * 2) = (uint16_t)pa;
        *reinterpret_cast<uint16_t*>(At + (t1 * 32 + pr) * 2) = (uint16_t)(pa >> 16);
        *reinterpret_cast<uint16_t*>(Lt + (t0 * 32 + pr) * 2) = (uint16_t)pl;
        *reinterpret_cast<uint16_t*>(Lt + (t1 * 32 + pr) * 2) = (uint16_t)(pl >> 16);
      }
      // dq^T = K^T dlogit^T + ds L_c, scaled, one fp32 row per pair
      f32x16 qa[DM];
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) qa[dm] = f32x16{};
#pragma unroll
      for (int st4 = 0; st4 < 4; ++st4) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = (st4 < 2) ? d0[8 * (st4 & 1) + e] : d1[8 * (st4 & 1) + e];
        Frag<BF16> ph, pl;
        split_bf16(pv, ph, pl);
#pragma unroll
        for (int dm = 0; dm < DM; ++dm) {
          Frag<BF16> a;
          const int d = 32 * dm + pr;
          const int slot = (2 * st4 + half) ^ vt_swz(d);
          a.load16(kts + d * VTB + slot * 16);
          mfma(qa[dm], a, ph);
          mfma(qa[dm], a, pl);
        }
      }
      if (ok) {
        float* op = dqp + (int64_t)pid * D;
#pragma unroll
        for (int dm = 0; dm < DM; ++dm)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int col = out_col(dm, q4, half);
            const u32x2 lw = *reinterpret_cast<const u32x2*>(lms + 2 * col);
            const float l0 = bf16_lo(lw[0]), l1 = bf16_hi(lw[0]), l2 = bf16_lo(lw[1]), l3 = bf16_hi(lw[1]);
            *reinterpret_cast<f32x4*>(op + col) =
                f32x4{fmaf(ds, l0, qa[dm][4 * q4]) * scale, fmaf(ds, l1, qa[dm][4 * q4 + 1]) * scale,
                      fmaf(ds, l2, qa[dm][4 * q4 + 2]) * scale, fmaf(ds, l3, qa[dm][4 * q4 + 3]) * scale};
          }
      }
    }
    __syncthreads();  // every wave's slot is written
    fetch_rows();     // the next round's tile
    // chunk side: dV += A^T dO, dK += dlogit'^T Q over the round's tiles
    for (int sl = 0; sl < 4 && 4 * r + sl < ntiles; ++sl) {
      const char* base = stage + sl * SLOT;
      const char* At = base;
      const char* Lt = base + SA;
      const char* Ot = base + 2 * SA;
      const char* Qt = base + 2 * SA + SO;
#pragma unroll
      for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
        for (int i = 0; i < NBW; ++i) {
          const int jb = wave * NBW + i;
          const int tok = 32 * (jb & 1) + pr;
          const int d = 32 * (jb >> 1) + pr;
          const int pc = 16 * kp + 8 * half;
          Frag<BF16> fa, fo, fl, fq;
          fa.load16(At + (tok * 32 + pc) * 2);
          fo.load16(Ot + (d * 32 + pc) * 2);
          fl.load16(Lt + (tok * 32 + pc) * 2);
          fq.load16(Qt + (d * 32 + pc) * 2);
          mfma(accV[i], fa, fo);
          mfma(accK[i], fl, fq);
        }
      }
    }
    __syncthreads();  // the slots are free for the next round
  }
  // write the chunk's dK and dV
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int jb = wave * NBW + i;
    const int d = 32 * (jb >> 1) + pr;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int tok = 32 * (jb & 1) + tile_row(rr, half);
      const int64_t o = (bg * T_len + c * kChunk + tok) * D + d;
      dv[o] = accV[i][rr];
      dk[o] = accK[i][rr] * scale;
    }
  }
}

// ---------------------------------------------------------------- 3. rows again
// dq of a row = the sum of its pairs' partials, in slot order; one thread per
// 4 dims of a row
template <int D>
__global__ void bwd_dq_kernel(const float* __restrict__ dqp, const int32_t* __restrict__ pair_pos,
                              float* __restrict__ dq, int64_t rows, int k) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = i / (D / 4);
  if (row >= rows) return;
  const int d = 4 * (int)(i % (D / 4));
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  // eight slots' loads in flight at a time; the sum keeps the slot order
  constexpr int U = 8;
  for (int e0 = 0; e0 < k; e0 += U) {
    bool ok[U];
    f32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ok[u] = e0 + u < k && pair_pos[row * k + e0 + u] >= 0;
#pragma unroll
    for (int u = 0; u < U; ++u)
      x[u] = ok[u] ? *reinterpret_cast<const f32x4*>(dqp + (row * k + e0 + u) * D + d) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ok[u]) {
        acc[0] += x[u][0];
        acc[1] += x[u][1];
        acc[2] += x[u][2];
        acc[3] += x[u][3];
      }
    }
  }
  *reinterpret_cast<f32x4*>(dq + row * D + d) = acc;
}

// dK = dV = 0 for the tokens after the last complete chunk of each (b, g)
__global__ void bwd_tail_kernel(float* __restrict__ dk, float* __restrict__ dv, int64_t bgs, int64_t T_len,
                                int64_t Nc, int D) {
  const int64_t tail = (T_len - Nc * kChunk) * D;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= bgs * tail) return;
  const int64_t o = (i / tail) * T_len * D + Nc * kChunk * D + i % tail;
  dk[o] = 0.0f;
  dv[o] = 0.0f;
}

// ---------------------------------------------------------------- host side
static size_t align_up_b(size_t x, size_t a) { return (x + a - 1) / a * a; }

BackwardPlan plan_backward(const Geometry& g) {
  BackwardPlan p{};
  const size_t nb = (size_t)g.B * g.Hkv * (size_t)g.Nc;
  const size_t rows = (size_t)g.B * g.Hq * (size_t)g.T;
  const size_t pairs = rows * g.k;
  size_t off = 0;
  p.off_kt = off;
  off = align_up_b(off + nb * kChunk * g.D * 2, 256);
  p.off_cnt = off;
  off = align_up_b(off + nb * sizeof(int), 256);
  p.off_off = off;
  off = align_up_b(off + (nb + 1) * sizeof(int), 256);
  p.off_pair_pos = off;
  off = align_up_b(off + pairs * sizeof(int32_t), 256);
  p.off_pairs = off;
  off = align_up_b(off + pairs * sizeof(int32_t), 256);
  p.off_w = off;
  off = align_up_b(off + pairs * sizeof(float), 256);
  p.off_delta = off;
  off = align_up_b(off + rows * sizeof(float), 256);
  p.off_dqp = off;
  off = align_up_b(off + pairs * g.D * sizeof(float), 256);
  p.bytes = off;
  return p;
}

template <int D>
static hipError_t launch_backward_d(const BackwardArgs& a, const BackwardPlan& p, hipStream_t st) {
  const Geometry& g = a.g;
  char* ws = static_cast<char*>(a.ws);
  uint16_t* kt = reinterpret_cast<uint16_t*>(ws + p.off_kt);
  int* cnt = reinterpret_cast<int*>(ws + p.off_cnt);
  int* offs = reinterpret_cast<int*>(ws + p.off_off);
  int32_t* pair_pos = reinterpret_cast<int32_t*>(ws + p.off_pair_pos);
  int32_t* pairs = reinterpret_cast<int32_t*>(ws + p.off_pairs);
  float* wts = reinterpret_cast<float*>(ws + p.off_w);
  float* delta = reinterpret_cast<float*>(ws + p.off_delta);
  float* dqp = reinterpret_cast<float*>(ws + p.off_dqp);
  const int64_t nb = (int64_t)g.B * g.Hkv * g.Nc;
  const int64_t rows = (int64_t)g.B * g.Hq * g.T;
  const int64_t total = rows * g.k;
  const float scale = 1.0f / sqrtf((float)D);
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* kk = static_cast<const uint16_t*>(a.k);
  const uint16_t* vv = static_cast<const uint16_t*>(a.v);
  hipError_t e;
  if (nb > 0 && (e = launch_zero_ints(cnt, nb, st)) != hipSuccess) return e;
  launch_kernel(bwd_prep_kernel<D>, dim3((unsigned)((rows + kPrepRows - 1) / kPrepRows)), dim3(256), 0, st,
                a.out, a.dout,
                a.sel_idx, a.sel_score, wts, delta, cnt, pair_pos, rows, g.Hq, g.G, g.T, g.Nc, g.k);
  if (nb > 0) {
    if ((e = launch_exclusive_scan(cnt, offs, nb, st)) != hipSuccess) return e;
    if (g.k % 4 == 0)
      launch_kernel(bwd_scatter_kernel<4>, dim3((unsigned)((total / 4 + 255) / 256)), dim3(256), 0, st, a.sel_idx,
                    pair_pos, offs, pairs, total, g.Hq, g.G, g.T, g.Nc, g.k, a.dbg);
    else
      launch_kernel(bwd_scatter_kernel<1>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, a.sel_idx,
                    pair_pos, offs, pairs, total, g.Hq, g.G, g.T, g.Nc, g.k, a.dbg);
    launch_kernel((prefill_vt_kernel<BF16, D>), dim3((unsigned)nb), dim3(256), 0, st, kk, kt, g.T, g.Nc);
    constexpr size_t lds = 3 * kChunk * D * 2 + 4 * (2 * kChunk * 32 * 2 + 2 * D * 32 * 2) + 2 * D;
    static_assert(lds <= 160 * 1024, "chunk kernel LDS");
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_chunk_kernel<D>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
      return e;
    launch_kernel(bwd_chunk_kernel<D>, dim3((unsigned)nb), dim3(256), lds, st, q, kk, vv, kt,
                  static_cast<const uint16_t*>(a.lm), a.dout, wts, delta, offs, pairs, dqp, a.dk, a.dv, g.k, g.T,
                  g.Nc, scale, total, a.dbg);
  }
  launch_kernel(bwd_dq_kernel<D>, dim3((unsigned)((rows * (D / 4) + 255) / 256)), dim3(256), 0, st, dqp,
                pair_pos, a.dq, rows, g.k);
  const int64_t tail = (g.T - g.Nc * kChunk) * D * (int64_t)g.B * g.Hkv;
  if (tail > 0) {
    launch_kernel(bwd_tail_kernel, dim3((unsigned)((tail + 255) / 256)), dim3(256), 0, st, a.dk, a.dv,
                  (int64_t)g.B * g.Hkv, g.T, g.Nc, D);
  }
  return hipGetLastError();
}

hipError_t launch_backward(const BackwardArgs& a, const BackwardPlan& p, hipStream_t st) {
  return a.g.D == 128 ? launch_backward_d<128>(a, p, st) : launch_backward_d<64>(a, p, st);
}

}  // namespace hsa_attn
