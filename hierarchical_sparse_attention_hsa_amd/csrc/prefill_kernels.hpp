// HSA prefill: causal HSA over a whole sequence, or over its last rows after
// a cached prefix (skill card "Every Token Counts 16m Context", sections
// "Core Technique" and "Implementation").  Kernels on one stream:
//
// prefill_select  one workgroup per (b, g, query chunk j) and group of up to
//   four query heads, one wave per head, 64 query rows per wave.  Landmark
//   tiles of 32 rows are staged in LDS (shared by the waves) and contracted
//   with the wave's queries on MFMA (bf16 in, fp32 accumulate): the
//   causal-block GEMM Q . L^T restricted to the chunks before j.  Pass 1 runs
//   the tiles from the newest chunk down and finds each row's k-th best
//   score; pass 2 recomputes the tiles that can hold a kept chunk and
//   collects the exact top-k (ties to the lower chunk index).  The scores
//   never reach memory.  The epilogue writes the selection and buckets the
//   "remote" pairs: selected chunks before the query's aligned 64-chunk
//   window, and window chunks that fewer than kLocalMinRows rows of the
//   query's 32-row block (same head) selected.
// prefill_vt      V^T tiles (tokens in the order the P.V fragments use them).
// prefill_zero / scan / scatter (prefill.hip)  counts, offsets and lists of
//   those remote pairs per (b, g, chunk).
// prefill_remote  one workgroup per remote bucket: the chunk's K and V^T are
//   staged once and its selecting rows gathered 32 at a time; writes each
//   pair's in-chunk attention output.
// prefill_local   one workgroup per (b, g, query chunk, 32-token half), one
//   wave per query head: walks the union of the rows' other ("local")
//   selected chunks (K and V^T staged in LDS), S^T = K_c Q^T and O^T += V_c^T P'^T
//   on MFMA with P' = fusion weight x in-chunk probability (0 for rows that
//   did not select the chunk, fed as a bf16 head + tail pair), then adds the
//   weighted remote outputs and writes the rows.
#pragma once

#include <algorithm>
#include <climits>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace hsa_attn {

constexpr int kChunk = 64;
// Query chunk j's aligned window: chunks [64 * floor(j / 64), j).  Selected
// chunks inside it are "local" to the attention, the others "remote".
constexpr int kLocalWindow = 64;
// A window chunk selected by fewer than this many rows of a 32-row query
// block (one head) is attended like the chunks before the window (one
// chunk-major pass over all its selecting rows) rather than by running the
// whole block through it.
#ifndef HSA_LOCAL_MIN_ROWS
#define HSA_LOCAL_MIN_ROWS 8
#endif
constexpr int kLocalMinRows = HSA_LOCAL_MIN_ROWS;

template <typename T>
__device__ __forceinline__ void load_frag_lds(Frag<T>& f, const char* row, int slot_xor, int kch, int half);

// bf16: 8 elements of one half k-chunk = one 16-byte slot (2*kch + half)
template <>
__device__ __forceinline__ void load_frag_lds<BF16>(Frag<BF16>& f, const char* row, int slot_xor, int kch,
                                                    int half) {
  const int slot = (2 * kch + half) ^ slot_xor;
  f.load16(row + slot * 16);
}
// fp32: 8 elements = two 16-byte slots (4*kch + 2*half, +1)
template <>
__device__ __forceinline__ void load_frag_lds<FP32>(Frag<FP32>& f, const char* row, int slot_xor, int kch,
                                                    int half) {
  const int s0 = (4 * kch + 2 * half) ^ slot_xor;
  const int s1 = (4 * kch + 2 * half + 1) ^ slot_xor;
  const f32x4 a = *reinterpret_cast<const f32x4*>(row + s0 * 16);
  const f32x4 b = *reinterpret_cast<const f32x4*>(row + s1 * 16);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = a[e];
    f.v[4 + e] = b[e];
  }
}

// Insert x (index xi) into a descending register list; the new element wins
// ties (callers offer candidates in descending index order).
template <int K>
__device__ __forceinline__ void list_insert(float (&s)[K], int (&id)[K], float x, int xi) {
  bool c[K];
#pragma unroll
  for (int p = 0; p < K; ++p) c[p] = x >= s[p];
#pragma unroll
  for (int p = K - 1; p >= 1; --p) {
    id[p] = c[p - 1] ? id[p - 1] : (c[p] ? xi : id[p]);
    s[p] = __builtin_amdgcn_fmed3f(s[p - 1], x, s[p]);
  }
  id[0] = c[0] ? xi : id[0];
  s[0] = c[0] ? x : s[0];
}

// Sort K (score, index) pairs in registers into the order (score
// descending, index ascending) with a bitonic network (K a power of two;
// padding entries -inf / INT_MAX sort last).
template <int K>
__device__ __forceinline__ void sort_pairs(float (&s)[K], int (&id)[K]) {
  static_assert((K & (K - 1)) == 0, "bitonic network over a power of two");
#pragma unroll
  for (int k2 = 2; k2 <= K; k2 <<= 1) {
#pragma unroll
    for (int j2 = k2 >> 1; j2 > 0; j2 >>= 1) {
#pragma unroll
      for (int i = 0; i < K; ++i) {
        const int l = i ^ j2;
        if (l > i) {
          // in ascending runs position i takes the element that comes first
          const bool l_first = s[l] > s[i] || (s[l] == s[i] && id[l] < id[i]);
          const bool swap = ((i & k2) == 0) ? l_first : !l_first;
          const float ts = s[i];
          const int ti = id[i];
          s[i] = swap ? s[l] : s[i];
          id[i] = swap ? id[l] : id[i];
          s[l] = swap ? ts : s[l];
          id[l] = swap ? ti : id[l];
        }
      }
    }
  }
}

// Insert x into a descending list of scores (ties are equal values, so no
// index is needed): one v_med3 per position.
template <int K>
__device__ __forceinline__ void score_insert(float (&s)[K], float x) {
#pragma unroll
  for (int p = K - 1; p >= 1; --p) s[p] = __builtin_amdgcn_fmed3f(s[p - 1], x, s[p]);
  s[0] = fmaxf(s[0], x);
}

// ---------------------------------------------------------------- select
//
// One workgroup per (b, g, query chunk j) and group of up to four query
// heads; one wave per head, 64 query rows per wave (lane = row).  Each wave
// streams the landmark tiles (32 chunks) of its KV head from L2 and
// contracts them with its queries on MFMA; the scores stay in registers.
//
// Pass 1 runs the tiles from the newest chunk down and keeps, per row, only
// the multiset of the k best scores (one v_med3 per list position per
// admitted candidate), which yields the row's k-th best score tau and how
// many of the k best are strictly above it.  Pass 2 recomputes the same
// tiles (bit-identical: same operands and MFMA sequence) in ascending chunk
// order and collects every candidate above tau plus the lowest-index
// candidates equal to tau until k are kept: exactly the first k in the order
// (score desc, index asc).  Tiles whose maximum cannot reach a row's
// threshold are skipped in both passes.
// Three waves per SIMD (the register budget drops to 168 at the cost of a
// few spilled values; measured faster than two waves for both list sizes).
template <typename T, int D, int G, int KSEL>
__global__ __launch_bounds__(kWave*(G < 4 ? G : 4)) __attribute__((amdgpu_waves_per_eu(3)))
void prefill_select_kernel(
    const typename T::storage* __restrict__ q, const typename T::storage* __restrict__ lm,
    int32_t* __restrict__ sel_idx, float* __restrict__ sel_score, int* __restrict__ rcnt, int32_t* __restrict__ pair_pos,
    int B, int Hkv, int64_t T_len, int64_t Nc, int nqc, int jlo, int slab_chunks, int j0, int k, float scale,
    int k_base, float gap_tau) {
  // T_len: query rows per (b, h); query row r sits at position 64*j0 + r.
  // The grid covers the query chunks [jlo, jlo + nqc) of those rows, which
  // fall in slabs of slab_chunks chunks starting at jlo; the remote pairs of
  // each slab are counted in its own block of B * Hkv * Nc bucket counts.
  // k_base > 0: adaptive budget, k == 2 * k_base (see the epilogue)
  using st = typename T::storage;
  constexpr int HPW = G < 4 ? G : 4;  // query heads (waves) per workgroup
  constexpr int HS = G / HPW;         // workgroups per (b, g, query chunk)
  constexpr int KCH = D / 16;
  constexpr int ROWB = D * T::kBytes;  // one landmark row
  constexpr int NSL = ROWB / 16;       // its 16-byte slots
  constexpr int TILE = 32 * ROWB;      // 32 landmarks
  constexpr int NI = TILE / (kWave * 16);  // direct-to-LDS loads per tile
  constexpr int PER = NI / HPW;            // of which each wave issues
  // LDS ring of NG groups of TPB tiles: one barrier per group, NG-1 groups
  // in flight.  Pass 1 uses only the ring and pass 2 only the candidate
  // store, so the two share their space.
#ifndef HSA_SEL_TPB
#define HSA_SEL_TPB 2
#endif
#ifndef HSA_SEL_NG
#define HSA_SEL_NG 3
#endif
  // (groups of one tile when the ring would hold more than 8 KiB per wave)
  constexpr int TPB = TILE * HSA_SEL_TPB <= 2 * 8192 && HPW >= 4 ? HSA_SEL_TPB : 1;
  constexpr int NG = HSA_SEL_NG;
  constexpr int NST = NG * TPB;
  constexpr int MAXT = 2048;               // Nc <= 65536
  static_assert(NI % HPW == 0 && NSL >= 8, "tile loads split evenly; row swizzle needs 8 slots");
  static_assert(NG >= 2 && (NG - 2) * TPB <= 4, "wait_tiles covers up to four later tiles");
  // ring of landmark tiles shared by the workgroup's waves: row r of a tile
  // holds its 16-byte slots XOR-swizzled by (r & 7); pass 2's kept
  // candidates: score and chunk index (Nc <= 65536)
  constexpr int RING = NST * TILE;
  constexpr int CS_BYTES = HPW * KSEL * kWave * 4;
  constexpr int STORE = CS_BYTES + HPW * KSEL * kWave * 2;
  __shared__ __align__(16) char shm[RING > STORE ? RING : STORE];
  auto ring = [&](int sg) { return shm + sg * TILE; };
  auto cs = reinterpret_cast<float(*)[KSEL][kWave]>(shm);
  auto ci = reinterpret_cast<uint16_t(*)[KSEL][kWave]>(shm + CS_BYTES);
  __shared__ uint32_t tneed[HPW][MAXT / 32];  // pass 1: tile reached a row's threshold

  const int bid = blockIdx.x;
  const int g = bid % Hkv;  // consecutive workgroups on different XCDs share nothing
  int rest = bid / Hkv;
  const int hs = rest % HS;
  rest /= HS;
  const int b = rest % B;
  const int j = jlo + nqc - 1 - rest / B;  // heaviest query chunks first
  const int tid = threadIdx.x, lane = tid & 63, hh = tid >> 6, half = lane >> 5;
  const int Hq = Hkv * G, h = g * G + hs * HPW + hh;
  const int ja = j0 + j;  // absolute query chunk
  const int64_t n = min((int64_t)ja, Nc);


  int cnt = 0;
  if (n > 0) {
    // Contraction index assignment (shared by both operands): in k-step s,
    // lane half h supplies dims 16*s + 8*h .. +8.  Query rows past the end of
    // the sequence read a valid row; their results are never used.
    Frag<T> qf[2][KCH];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int64_t tok = min((int64_t)j * kChunk + 32 * nb + (lane & 31), T_len - 1);
      const st* qp = q + (((int64_t)b * Hq + h) * T_len + tok) * D + 8 * half;
#pragma unroll
      for (int s = 0; s < KCH; ++s) load_frag_global(qf[nb][s], qp + 16 * s, true);
    }
    const char* lmg = reinterpret_cast<const char*>(lm + ((int64_t)b * Hkv + g) * Nc * D);
    const int ntiles = (int)((n + 31) / 32);
    // this wave's share of the direct-to-LDS loads of tile ti into stage sg;
    // landmark rows past the candidate range read row n-1 (masked later)
    auto issue = [&](int ti, int sg) {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int ii = hh * PER + u;
        const int L = ii * kWave + lane;
        const int r = L / NSL, sp = L % NSL;
        const int64_t c = min((int64_t)ti * 32 + r, n - 1);
        __builtin_amdgcn_global_load_lds(lmg + c * ROWB + ((sp ^ (r & 7)) * 16),
                                         (__attribute__((address_space(3))) void*)(ring(sg) + ii * kWave * 16), 16,
                                         0, 0);
      }
    };
    // wait until at most `later` tiles of this wave's loads are in flight
    auto wait_tiles = [&](int later) {
      if constexpr ((NG - 2) * TPB >= 4) {
        if (later >= 4) {
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * PER) : "memory");
          return;
        }
        if (later == 3) {
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PER) : "memory");
          return;
        }
      }
      if constexpr ((NG - 2) * TPB >= 2) {
        if (later == 2) {
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory");
          return;
        }
      }
      if constexpr ((NG - 2) * TPB >= 1) {
        if (later == 1) {
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory");
          return;
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    // Run body(i, tile, stage) over the tile sequence tile_of(0 .. count-1)
    // in groups of TPB tiles with NG-1 groups in flight and one barrier per
    // group: after the barrier of group gi every wave is done with group
    // gi-1, whose stages are refilled.
    auto pipeline = [&](int count, auto tile_of, auto body) {
      const int ngr = (count + TPB - 1) / TPB;
      for (int i = 0; i < (NG - 1) * TPB && i < count; ++i) issue(tile_of(i), i % NST);
      for (int gi = 0; gi < ngr; ++gi) {
        const int done = min(count, (gi + 1) * TPB);  // tiles needed now
        const int issued = min(count, (gi + NG - 1) * TPB);
        wait_tiles(issued - done);
        __syncthreads();
        for (int i = (gi + NG - 1) * TPB; i < (gi + NG) * TPB && i < count; ++i) issue(tile_of(i), i % NST);
        for (int i = gi * TPB; i < done; ++i) body(i, tile_of(i), ring(i % NST));
      }
      __syncthreads();  // the ring is free again
    };
    // scores of a tile: lane l gets them for query rows (l%32) and
    // 32 + (l%32) at tile rows tile_row(r, l/32)
    auto contract = [&](const char* tile, f32x16& acc0, f32x16& acc1) {
      acc0 = f32x16{};
      acc1 = f32x16{};
      const char* row = tile + (lane & 31) * ROWB;
#pragma unroll
      for (int s = 0; s < KCH; ++s) {
        Frag<T> a;
        load_frag_lds<T>(a, row, lane & 7, s, half);
        mfma(acc0, a, qf[0][s]);
        mfma(acc1, a, qf[1][s]);
      }
    };
    // per-row tile maximum: the per-lane maxima of acc0/acc1, swapped like
    // the scores, combine into the maximum over the row's 32 candidates
    auto row_max = [&](const f32x16& acc0, const f32x16& acc1) {
      float m0 = acc0[0], m1 = acc1[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        m0 = fmaxf(m0, acc0[r]);
        m1 = fmaxf(m1, acc1[r]);
      }
      const auto pm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m0), __float_as_uint(m1), false, false);
      return fmaxf(__uint_as_float(pm[0]), __uint_as_float(pm[1]));
    };
    // lane l takes query row l: lo[r] -> tile row tile_row(r, 0), hi[r] ->
    // tile_row(r, 1); rows of the top tile past the candidate range get -inf
    auto to_rows = [&](const f32x16& acc0, const f32x16& acc1, int ti, float (&lo)[16], float (&hi)[16]) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc0[r]), __float_as_uint(acc1[r]), false,
                                                        false);
        lo[r] = __uint_as_float(p[0]);
        hi[r] = __uint_as_float(p[1]);
      }
      const int cbase = ti * 32;
      if ((int64_t)cbase + 32 > n) {
        const int nv = (int)(n - cbase);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (tile_row(r, 0) >= nv) lo[r] = -__builtin_inff();
          if (tile_row(r, 1) >= nv) hi[r] = -__builtin_inff();
        }
      }
    };
    // candidate ii of the tile (chunk 32*ti + ii) in the lo/hi registers
    auto cand = [](const float (&lo)[16], const float (&hi)[16], int ii) {
      const int r = (ii / 8) * 4 + (ii % 4);
      return ((ii / 4) & 1) ? hi[r] : lo[r];
    };

    // ---- pass 1: the multiset of the k best scores.  List positions above
    // k hold +inf, so ls[KSEL-1] is the k-th best once k are seen; until
    // then the -FLT_MAX seeds keep masked (-inf) candidates out.  A tile in
    // which no row of the wave reaches its running threshold stays unmarked:
    // the threshold only grows, so pass 2 can skip it for this wave.
    for (int i = lane; i < MAXT / 32; i += kWave) tneed[hh][i] = 0u;
    float ls[KSEL];
#pragma unroll
    for (int e = 0; e < KSEL; ++e) ls[e] = (e < KSEL - k) ? __builtin_inff() : -3.402823466e38f;
    pipeline(
        ntiles, [&](int i) { return ntiles - 1 - i; },
        [&](int, int ti, const char* tile) {
          f32x16 acc0, acc1;
          contract(tile, acc0, acc1);
          const bool top = (int64_t)ti * 32 + 32 > n;
          if (!top && !__ballot(row_max(acc0, acc1) >= ls[KSEL - 1])) return;
          if (lane == 0) tneed[hh][ti >> 5] |= 1u << (ti & 31);
          float lo[16], hi[16];
          to_rows(acc0, acc1, ti, lo, hi);
          // groups of 8 candidates, skipped when no row's group maximum
          // reaches its threshold
#pragma unroll
          for (int gg = 3; gg >= 0; --gg) {
            float gm = cand(lo, hi, 8 * gg);
#pragma unroll
            for (int q = 1; q < 8; ++q) gm = fmaxf(gm, cand(lo, hi, 8 * gg + q));
            if (!__ballot(gm >= ls[KSEL - 1])) continue;
#pragma unroll
            for (int q = 7; q >= 0; --q) {
              const float x = cand(lo, hi, 8 * gg + q);
              if (x >= ls[KSEL - 1]) score_insert<KSEL>(ls, x);
            }
          }
        });

    // ---- pass 2: collect the k best in ascending chunk order.  Each wave
    // recomputes only the tiles it marked, streaming their landmark
    // fragments from L2 into registers (no barriers).
    const float tau = ls[KSEL - 1];
    int quota = KSEL;  // entries equal to tau that still fit
#pragma unroll
    for (int e = 0; e < KSEL; ++e) quota -= ls[e] > tau;
    const st* lmr = lm + ((int64_t)b * Hkv + g) * Nc * D + 8 * half;
    Frag<T> fa[KCH];
    auto fetch = [&](Frag<T>(&f)[KCH], int ti) {
      const int64_t c = min((int64_t)ti * 32 + (lane & 31), n - 1);
      const st* p = lmr + c * D;
#pragma unroll
      for (int s2 = 0; s2 < KCH; ++s2) load_frag_global(f[s2], p + 16 * s2, true);
    };
    auto marked = [&](int ti) {
      return ((__builtin_amdgcn_readfirstlane(tneed[hh][ti >> 5]) >> (ti & 31)) & 1u) != 0u;
    };
    auto next_marked = [&](int ti) {
      while (ti < ntiles && !marked(ti)) ++ti;
      return ti;
    };
    auto collect = [&](f32x16& acc0, f32x16& acc1, int ti) {
      const bool top = (int64_t)ti * 32 + 32 > n;
      if (!top && !__ballot(row_max(acc0, acc1) >= tau)) return;
      float lo[16], hi[16];
      to_rows(acc0, acc1, ti, lo, hi);
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        // skip a group of 8 in which no row reaches tau
        float gm = cand(lo, hi, 8 * gg);
#pragma unroll
        for (int q2 = 1; q2 < 8; ++q2) gm = fmaxf(gm, cand(lo, hi, 8 * gg + q2));
        if (!__ballot(gm >= tau)) continue;
#pragma unroll
        for (int q2 = 0; q2 < 8; ++q2) {
          const int ii = 8 * gg + q2;
          const float x = cand(lo, hi, ii);
          if (x >= tau) {
            const bool take = x > tau || quota > 0;
            if (x == tau) --quota;
            if (take && cnt < KSEL) {
              cs[hh][cnt][lane] = x;
              ci[hh][cnt][lane] = (uint16_t)(ti * 32 + ii);
              ++cnt;
            }
          }
        }
      }
    };
    // One register buffer: a tile's fragments are consumed by its MFMAs,
    // then the next marked tile's loads are issued (unconditionally: past
    // the last tile they re-read the last landmark) and fly while this
    // tile's candidates are collected.  (Two buffers do not fit the
    // register budget of three waves per SIMD: the spill code's reloads
    // waited for every load in flight.)
    int ti = next_marked(0);
    if (ti < ntiles) {
      fetch(fa, ti);
      while (true) {
        f32x16 acc0 = {}, acc1 = {};
#pragma unroll
        for (int s2 = 0; s2 < KCH; ++s2) {
          mfma(acc0, fa[s2], qf[0][s2]);
          mfma(acc1, fa[s2], qf[1][s2]);
        }
        const int t1 = next_marked(ti + 1);
        fetch(fa, t1);
        collect(acc0, acc1, ti);
        if (t1 >= ntiles) break;
        ti = t1;
      }
    }
  }
  const int64_t t_row = (int64_t)j * kChunk + lane;
  // order the kept set by (score desc, index asc)
  float os[KSEL];
  int oi[KSEL];
#pragma unroll
  for (int e = 0; e < KSEL; ++e) {
    os[e] = -__builtin_inff();
    oi[e] = INT_MAX;
  }
  // cs/ci hold the kept set (at most KSEL entries, distinct indices, in
  // ascending chunk order)
  if constexpr (KSEL <= 16) {
#pragma unroll
    for (int e = 0; e < KSEL; ++e) {
      if (e < cnt) {
        os[e] = cs[hh][e][lane];
        oi[e] = (int)ci[hh][e][lane];
      }
    }
    sort_pairs<KSEL>(os, oi);
  } else {
    // (a network over 32 pairs costs more registers than the kernel has)
    // list_insert lets the newest element win score ties, so the entries are
    // offered from the highest index down
    int mx = cnt;
    for (int off = 32; off >= 1; off >>= 1) mx = max(mx, __shfl_xor(mx, off));
    mx = __builtin_amdgcn_readfirstlane(mx);
    for (int e = mx - 1; e >= 0; --e) {
      if (e < cnt) list_insert<KSEL>(os, oi, cs[hh][e][lane], (int)ci[hh][e][lane]);
    }
  }
  // near-tie adaptive budget (value-of-information router abstract, k-th
  // versus (k+1)-th gap): the row keeps all k = 2 * k_base entries only when
  // its k_base-th best scaled score beats the next one by less than gap_tau
  // (the same fp32 values it stores in sel_score); otherwise entries from
  // k_base on become padding before they are written or bucketed
  if (k_base > 0) {
    float s_k = -__builtin_inff(), s_k1 = -__builtin_inff();
    bool has_k1 = false;
#pragma unroll
    for (int e = 0; e < KSEL; ++e) {
      if (e == k_base - 1) s_k = os[e] * scale + 0.0f;
      if (e == k_base) {
        s_k1 = os[e] * scale + 0.0f;
        has_k1 = oi[e] != INT_MAX;
      }
    }
    if (!(has_k1 && s_k - s_k1 < gap_tau)) {
#pragma unroll
      for (int e = 0; e < KSEL; ++e) {
        if (e >= k_base) {
          os[e] = -__builtin_inff();
          oi[e] = INT_MAX;
        }
      }
    }
  }
  // The kept set is ranked by the unscaled dot products; the stored scores
  // carry the 1/sqrt(D) factor, which can round two neighbouring dot
  // products to one value.  Slots follow the stored scores, ties by index:
  // such neighbours are swapped into index order (odd-even passes until no
  // pair is out of order; a run of equal scores is rare and short).
  float ss[KSEL];
#pragma unroll
  for (int e = 0; e < KSEL; ++e) ss[e] = oi[e] != INT_MAX ? os[e] * scale + 0.0f : -__builtin_inff();
  for (bool again = true; again;) {
    bool swapped = false;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
#pragma unroll
      for (int e = par; e + 1 < KSEL; e += 2) {
        if (ss[e] == ss[e + 1] && oi[e] > oi[e + 1]) {
          const int t = oi[e];
          oi[e] = oi[e + 1];
          oi[e + 1] = t;
          swapped = true;
        }
      }
    }
    again = __ballot(swapped) != 0;
  }
  const int64_t base = (((int64_t)b * Hq + h) * T_len + t_row) * k;
  if (t_row < T_len) {
    if (k % 4 == 0) {  // the row's slots as 16-byte stores (its row starts 16-byte aligned)
#pragma unroll
      for (int e4 = 0; e4 < KSEL / 4; ++e4) {
        if (4 * e4 < k) {
          u32x4 i4;
          f32x4 s4;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const bool ok = oi[4 * e4 + u] != INT_MAX;
            i4[u] = ok ? (uint32_t)oi[4 * e4 + u] : ~0u;
            s4[u] = ok ? ss[4 * e4 + u] : -__builtin_inff();
          }
          *reinterpret_cast<u32x4*>(sel_idx + base + 4 * e4) = i4;
          *reinterpret_cast<f32x4*>(sel_score + base + 4 * e4) = s4;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < KSEL; ++e) {
        if (e < k) {
          const bool ok = oi[e] != INT_MAX;
          sel_idx[base + e] = ok ? oi[e] : -1;
          sel_score[base + e] = ok ? ss[e] : -__builtin_inff();
        }
      }
    }
  }
  if (rcnt == nullptr) return;  // no remote bucketing (fewer than one window)

  // ---- bucket the remote selections (chunks before the query's aligned
  // window, and window chunks selected by fewer than kLocalMinRows rows of
  // the 32-row half of the wave): count them per (b, g, chunk) in rcnt and
  // give each its position
  // in its bucket.  The workgroup first groups its selections by chunk in an
  // LDS hash table in cs's space, one word per slot: chunk << 16 | count
  // (empty: all ones; counts stay below 2^16), so a chunk picked by many of
  // its rows costs one global atomic.
  constexpr int HASH = HPW * KSEL * kWave;  // >= the workgroup's selections
  constexpr uint32_t kEmpty = 0xffffffffu;
  uint32_t* hw = reinterpret_cast<uint32_t*>(&cs[0][0][0]);
  // rows of each 32-row half of the wave that selected each window chunk
  __shared__ int wcnt[HPW][2][kLocalWindow];
  for (int i = lane; i < 2 * kLocalWindow; i += kWave) (&wcnt[hh][0][0])[i] = 0;
  __syncthreads();  // every wave is done with cs and ci
  for (int i = tid; i < HASH; i += kWave * HPW) hw[i] = kEmpty;
  const int wsj = (ja / kLocalWindow) * kLocalWindow;
  const int hf = lane >> 5;
#pragma unroll
  for (int e = 0; e < KSEL; ++e)
    if (e < k && t_row < T_len && oi[e] >= wsj && oi[e] != INT_MAX) atomicAdd(&wcnt[hh][hf][oi[e] - wsj], 1);
  __syncthreads();
  uint32_t slot_rank[KSEL];  // slot << 16 | rank within the slot, or ~0
#pragma unroll
  for (int e = 0; e < KSEL; ++e) {
    slot_rank[e] = ~0u;
    const bool remote = oi[e] != INT_MAX && (oi[e] < wsj || wcnt[hh][hf][oi[e] - wsj] < kLocalMinRows);
    if (e < k && t_row < T_len && remote) {
      const int c = oi[e];
      int sl = (int)(((uint32_t)c * 2654435761u) >> 8) & (HASH - 1);
      while (true) {
        const uint32_t prev = atomicCAS(&hw[sl], kEmpty, (uint32_t)c << 16);
        if (prev == kEmpty || (prev >> 16) == (uint32_t)c) break;
        sl = (sl + 1) & (HASH - 1);
      }
      slot_rank[e] = ((uint32_t)sl << 16) | (atomicAdd(&hw[sl], 1u) & 0xffffu);
    }
  }
  __syncthreads();
  int* bucket0 = rcnt + ((int64_t)((j - jlo) / slab_chunks) * B * Hkv + (int64_t)b * Hkv + g) * Nc;
  for (int i = tid; i < HASH; i += kWave * HPW) {
    const uint32_t w = hw[i];
    if (w != kEmpty) hw[i] = (uint32_t)atomicAdd(&bucket0[w >> 16], (int)(w & 0xffffu));  // -> first position
  }
  __syncthreads();
  if (t_row < T_len) {
    auto pos_of = [&](int e) {
      const uint32_t sr = slot_rank[e];
      return sr == ~0u ? -1 : (int)hw[sr >> 16] + (int)(sr & 0xffffu);
    };
    if (k % 4 == 0) {
#pragma unroll
      for (int e4 = 0; e4 < KSEL / 4; ++e4) {
        if (4 * e4 < k) {
          u32x4 p4;
#pragma unroll
          for (int u = 0; u < 4; ++u) p4[u] = (uint32_t)pos_of(4 * e4 + u);
          *reinterpret_cast<u32x4*>(pair_pos + base + 4 * e4) = p4;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < KSEL; ++e)
        if (e < k) pair_pos[base + e] = pos_of(e);
    }
  }
}

// ---------------------------------------------------------------- attention
//
// A selected (row, chunk) pair is "local" when the chunk lies in the query's
// aligned window of kLocalWindow chunks and at least kLocalMinRows rows of
// the row's 32-row block (same head) selected it, and "remote" otherwise.
// Local pairs are shared by many rows of a query block (measured: most
// selections fall in the query's own window), so prefill_local_kernel walks
// the union of a block's local selections and runs every row of the block
// through each chunk on MFMA (rows that did not select it get weight 0): a
// chunk's cost does not depend on how many rows selected it, hence the
// minimum.  Remote pairs are scattered, so they are processed chunk-major:
// they are bucketed by
// (b, g, chunk), prefill_remote_kernel loads each chunk's K/V tile once and
// gathers its selecting rows 32 at a time into full MFMA tiles, and writes
// each pair's normalised in-chunk output; the local kernel then adds the
// weighted remote outputs of its rows.

// V^T element position of token t inside the 64-token row of column d, in
// the order the P' fragments present tokens: k-step t/16, lane half
// (t%8)/4, element 4*((t%16)/8) + t%4.
__device__ __forceinline__ int vt_pos(int t) {
  return (t / 16) * 16 + ((t % 8) / 4) * 8 + 4 * ((t % 16) / 8) + (t % 4);
}

// XOR swizzle of the 16-byte slots of V^T column d.  Reads take eight
// consecutive columns at once (d & 7 varies); stash writes take columns
// eight apart (d >> 3 varies): both sets land on distinct slots.
__device__ __forceinline__ int vt_swz(int d) { return (d & 7) ^ ((d >> 3) & 7); }

// LDS image of one chunk (both attention kernels): the K tile, 64 rows of
// D elements whose 16-byte slots are XOR-swizzled by (row & 7), then the
// V^T tile, D rows of 64 tokens in vt_pos order whose 16-byte slots are
// swizzled by vt_swz(d).  Both are filled by direct global->LDS loads
// (global_load_lds_dwordx4: lane i of an instruction writes LDS bytes
// base + 16 i), the swizzle being applied on the global side; V^T comes from
// the transposed copy written by prefill_vt_kernel.
template <typename T, int D>
struct Tile {
  static constexpr int ROWB = D * T::kBytes;       // K row bytes
  static constexpr int NSL = ROWB / 16;            // 16-byte slots per K row
  static constexpr int VTB = kChunk * T::kBytes;   // V^T row bytes
  static constexpr int NSLV = VTB / 16;            // 16-byte slots per V^T row
  static constexpr int KBYTES = kChunk * ROWB;
  static constexpr int BYTES = 2 * KBYTES;         // K tile + V^T tile
  static constexpr int NK = kChunk * NSL / kWave;  // load instructions for K
  static constexpr int NV = D * NSLV / kWave;      // load instructions for V^T
  static_assert(NSL >= 8 && NSLV >= 8, "swizzles need 8 slots per row");

  // Issue this wave's share (instructions w, w + NW, ...) of the loads of a
  // chunk: kb = the chunk's K rows, vtb = its V^T tile, lds = the buffer.
  template <int NW>
  static __device__ __forceinline__ void issue(const char* kb, const char* vtb, char* lds, int w, int lane) {
#pragma unroll
    for (int ii = 0; ii < NK + NV; ++ii) {
      if (ii % NW != w) continue;
      const char* src;
      if (ii < NK) {
        const int L = ii * kWave + lane;
        const int t = L / NSL, sp = L % NSL;
        src = kb + t * ROWB + ((sp ^ (t & 7)) * 16);
      } else {
        const int L = (ii - NK) * kWave + lane;
        const int d = L / NSLV, sp = L % NSLV;
        src = vtb + d * VTB + ((sp ^ vt_swz(d)) * 16);
      }
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds + ii * kWave * 16), 16, 0,
                                       0);
    }
  }
};

// wait for this wave's direct-to-LDS loads
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Order one wave's LDS accesses across its lanes: the hardware executes a
// wave's LDS instructions in order, so only the compiler must not move
// accesses across this point.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Transposed copy of V for the attention kernels: for every complete chunk,
// D rows of its 64 values of dimension d, tokens in vt_pos order, so that a
// chunk's V^T tile is one contiguous block.  One workgroup per chunk: a
// thread loads 16 bytes of 4 consecutive tokens, writes them transposed into
// LDS (4 tokens of one column form one contiguous piece), and the tile then
// leaves LDS in 16-byte slots.
template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_vt_kernel(const typename T::storage* __restrict__ vv,
                                                         typename T::storage* __restrict__ vt_g, int64_t T_len,
                                                         int64_t Nc) {
  using st = typename T::storage;
  using TL = Tile<T, D>;
  constexpr int EPS = 16 / T::kBytes;
  constexpr int UNITS = TL::NSL * (kChunk / 4);
  __shared__ __align__(16) char vt[D * TL::VTB];
  const int64_t bc = blockIdx.x;  // (b * Hkv + g) * Nc + c
  const int64_t c = bc % Nc, bg = bc / Nc;
  const st* vb = vv + (bg * T_len + c * kChunk) * D;
  const int tid = threadIdx.x;
  for (int u = tid; u < UNITS; u += 256) {
    const int sl = u % TL::NSL, t0 = 4 * (u / TL::NSL);
    u32x4 v4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v4[i] = *reinterpret_cast<const u32x4*>(vb + (t0 + i) * D + sl * EPS);
    const int p = vt_pos(t0);  // the four tokens sit at p .. p+3
    if constexpr (T::kBytes == 2) {
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        const int d = sl * EPS + e;
        const int w = e / 2, sh = (e & 1) * 16;
        const uint32_t lo = ((v4[0][w] >> sh) & 0xffffu) | (((v4[1][w] >> sh) & 0xffffu) << 16);
        const uint32_t hi = ((v4[2][w] >> sh) & 0xffffu) | (((v4[3][w] >> sh) & 0xffffu) << 16);
        const int pp = (((p / 8) ^ vt_swz(d)) * 8) + (p % 8);
        *reinterpret_cast<u32x2*>(vt + d * TL::VTB + pp * 2) = u32x2{lo, hi};
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        const int d = sl * EPS + e;
        const int pp = ((p / 4) ^ vt_swz(d)) * 4;
        *reinterpret_cast<u32x4*>(vt + d * TL::VTB + pp * 4) = u32x4{v4[0][e], v4[1][e], v4[2][e], v4[3][e]};
      }
    }
  }
  __syncthreads();
  char* out = reinterpret_cast<char*>(vt_g) + bc * (int64_t)(D * TL::VTB);
  for (int L = tid; L < D * TL::NSLV; L += 256) {
    const int d = L / TL::NSLV, sl = L % TL::NSLV;  // logical slot sl of row d
    *reinterpret_cast<u32x4*>(out + d * TL::VTB + sl * 16) =
        *reinterpret_cast<const u32x4*>(vt + d * TL::VTB + ((sl ^ vt_swz(d)) * 16));
  }
}

// max / sum of a value over the lane pair (l, l ^ 32)
__device__ __forceinline__ float pair_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// x = head + tail with head = x truncated to bf16 and tail = the exact
// remainder rounded to bf16 (relative error of head + tail below 2^-15)
__device__ __forceinline__ void split_bf16(const float (&x)[8], Frag<BF16>& head, Frag<BF16>& tail) {
  u32x4 hw, tw;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = __float_as_uint(x[2 * i]), b = __float_as_uint(x[2 * i + 1]);
    hw[i] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // upper halves of a (low) and b (high)
    const f32x2 r{x[2 * i] - __uint_as_float(a & 0xffff0000u), x[2 * i + 1] - __uint_as_float(b & 0xffff0000u)};
    const bf16x2 t = __builtin_convertvector(r, bf16x2);
    uint32_t tw32;
    __builtin_memcpy(&tw32, &t, 4);
    tw[i] = tw32;
  }
  head.v = as_bf16x8(hw);
  tail.v = as_bf16x8(tw);
}

// One wave, 32 query rows (B operand qf, row = lane % 32; lanes l and l^32
// hold the two halves of each row): softmax attention over the 64 tokens of
// the staged chunk, accumulated into the O^T tiles as factor * o_c.
template <typename T, int D>
__device__ __forceinline__ void attend_block(const Frag<T> (&qf)[D / 16], const char* ks, const char* vt,
                                             float factor, float cexp, f32x16 (&oacc)[D / 32], int lane) {
  constexpr int ROWB = D * T::kBytes;
  constexpr int VTB = kChunk * T::kBytes;
  constexpr int KCH = D / 16;
  constexpr int DM = D / 32;
  const int half = lane >> 5;
  // S^T = K_c Q^T: two 32-token blocks
  f32x16 s0 = {}, s1 = {};
  const char* k0 = ks + (lane & 31) * ROWB;
  const char* k1 = ks + (32 + (lane & 31)) * ROWB;
#pragma unroll
  for (int s = 0; s < KCH; ++s) {
    Frag<T> a0, a1;
    load_frag_lds<T>(a0, k0, lane & 7, s, half);
    load_frag_lds<T>(a1, k1, lane & 7, s, half);
    mfma(s0, a0, qf[s]);
    mfma(s1, a1, qf[s]);
  }
  // softmax over the row's 64 tokens; lane l and l^32 split them (the
  // permlane32 swap hands each lane its partner's value)
  float mx = -__builtin_inff();
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
  mx = pair_max(mx);
  const float mb = mx * cexp;
  float sum = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = __builtin_amdgcn_exp2f(fmaf(s0[r], cexp, -mb));
    s1[r] = __builtin_amdgcn_exp2f(fmaf(s1[r], cexp, -mb));
    sum += s0[r] + s1[r];
  }
  sum = pair_sum(sum);
  const float f = factor / sum;
  // O^T += V^T P'^T over four 16-token k-steps
#pragma unroll
  for (int ks_ = 0; ks_ < 4; ++ks_) {
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = f * ((ks_ < 2) ? s0[8 * (ks_ & 1) + e] : s1[8 * (ks_ & 1) + e]);
    if constexpr (T::kBytes == 2) {
      // P' = head + tail: the head is P' truncated to bf16 (exact upper
      // half), the tail the exact remainder rounded to bf16, so head + tail
      // carries about 16 significant bits
      Frag<BF16> phi, plo;
      split_bf16(pv, phi, plo);
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        Frag<BF16> a;
        const int d = 32 * dm + (lane & 31);
        const int slot = (2 * ks_ + half) ^ vt_swz(d);
        a.load16(vt + d * VTB + slot * 16);
        mfma(oacc[dm], a, phi);
        mfma(oacc[dm], a, plo);
      }
    } else {
      Frag<FP32> pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf.v[e] = pv[e];
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        Frag<FP32> a;
        const int d = 32 * dm + (lane & 31);
        const int s0i = (4 * ks_ + 2 * half) ^ vt_swz(d);
        const int s1i = (4 * ks_ + 2 * half + 1) ^ vt_swz(d);
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(vt + d * VTB + s0i * 16);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(vt + d * VTB + s1i * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a.v[e] = x0[e];
          a.v[4 + e] = x1[e];
        }
        mfma(oacc[dm], a, pf);
      }
    }
  }
}

// Output columns held by a lane in the O^T accumulators: for tile dm and
// register group q4, four consecutive columns starting at out_col(dm, q4).
__device__ __forceinline__ int out_col(int dm, int q4, int half) { return 32 * dm + 8 * q4 + 4 * half; }

// Remote-pair bucketing around the select kernel (prefill.hip): the bucket
// counts of a group of slabs are cleared before it (one launch); after it,
// the exclusive scans of every slab's counts give its bucket offsets (one
// launch, a workgroup per slab), and the scatter turns each pair's position
// within its bucket into its position in its slab's pair list and records
// its query row there (one launch for the group, a thread per row).
hipError_t launch_prefill_zero_counts(const PrefillArgs& a, hipStream_t st);
hipError_t launch_prefill_bucketing(const PrefillArgs& a, int nslab, int64_t r0, int64_t rn, hipStream_t st);

// ---- chunk-major attention of the remote pairs
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void prefill_remote_kernel(const typename T::storage* __restrict__ q,
                                                             const typename T::storage* __restrict__ kk,
                                                             const typename T::storage* __restrict__ vt_g,
                                                             const int* __restrict__ off,
                                                             const int32_t* __restrict__ pairs,
                                                             float* __restrict__ partial, int Hkv, int64_t T_len,
                                                             int64_t Nc, float scale, int64_t cap, int64_t qrows,
                                                             uint32_t* __restrict__ dbg) {
  using st = typename T::storage;
  using TL = Tile<T, D>;
  constexpr int KCH = D / 16;
  constexpr int DM = D / 32;
#ifndef HSA_REMOTE_STAGE_TILES
#define HSA_REMOTE_STAGE_TILES 2
#endif
  constexpr int SDM = HSA_REMOTE_STAGE_TILES;  // 32-column tiles per stage round
  static_assert(DM % SDM == 0, "rounds cover the output columns");
  // per wave: 32 rows of 32 * SDM fp32 columns, rows padded by 16 bytes so
  // that 16 rows' pieces at one column fall on distinct banks
  constexpr int kStageRow = 32 * SDM + 4;
  __shared__ __align__(16) char smem[TL::BYTES];
  __shared__ __align__(16) float stage[4][32 * kStageRow];
  char* ks = smem;
  char* vt = smem + TL::KBYTES;
  const int64_t bucket = blockIdx.x;
  const int begin = off[bucket], end = off[bucket + 1];
  if (begin == end) return;
  if (!dbg_ok(dbg, begin >= 0 && begin <= end && end <= cap, HSA_ATTN_DEBUG_REMOTE_RANGE)) return;
  const int64_t c = bucket % Nc;
  const int64_t bg = bucket / Nc;  // b * Hkv + g
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  float* stg = stage[wave];
  TL::template issue<4>(reinterpret_cast<const char*>(kk + (bg * T_len + c * kChunk) * D),
                        reinterpret_cast<const char*>(vt_g) + bucket * (int64_t)TL::KBYTES, smem, wave, lane);
  wait_loads();
  __syncthreads();
  const float cexp = scale * 1.4426950408889634f;
  // the block's query rows come into the wave's stage by direct
  // global->LDS loads, whole rows per load (row r's 16-byte slots
  // XOR-swizzled by r & 7), when 32 rows fit the stage; else as per-lane
  // MFMA fragments (which touch 32 rows per load)
  constexpr int QROWB = D * T::kBytes, QNSL = QROWB / 16, QRPI = kWave / QNSL;
  constexpr bool kQStage = 32 * QROWB <= 32 * kStageRow * 4 && QNSL >= 8 && kWave % QNSL == 0;
  // the pair ids of the wave's next block are loaded one block ahead (a
  // lane past the bucket's end reads the bucket's first pair, a valid row)
  auto pair_row = [&](int blk) {
    const int p = begin + 32 * blk + (lane & 31);
    const int32_t r = pairs[p < end ? p : begin];
    return dbg_ok(dbg, r >= 0 && r < qrows, HSA_ATTN_DEBUG_REMOTE_ROW) ? r : 0;
  };
  int32_t row_next = pair_row(wave);
  for (int blk = wave; begin + 32 * blk < end; blk += 4) {
    const bool ok = begin + 32 * blk + (lane & 31) < end;
    const int64_t row = row_next;
    row_next = pair_row(blk + 4);
    Frag<T> qf[KCH];
    if constexpr (kQStage) {
      char* qs = reinterpret_cast<char*>(stg);
      const char* qb = reinterpret_cast<const char*>(q);
#pragma unroll
      for (int ii = 0; ii < 32 / QRPI; ++ii) {
        const int r = ii * QRPI + lane / QNSL, sp = lane % QNSL;
        const int64_t rr = __shfl(row, r);  // row r's query (a valid row for past-the-end pairs)
        __builtin_amdgcn_global_load_lds(qb + rr * QROWB + ((sp ^ (r & 7)) * 16),
                                         (__attribute__((address_space(3))) void*)(qs + ii * kWave * 16), 16, 0, 0);
      }
      wait_loads();
      const char* qrow = qs + (lane & 31) * QROWB;
#pragma unroll
      for (int s = 0; s < KCH; ++s) load_frag_lds<T>(qf[s], qrow, lane & 7, s, half);
      wave_lds_fence();
    } else {
      const st* qp = q + row * D + 8 * half;
#pragma unroll
      for (int s = 0; s < KCH; ++s) load_frag_global(qf[s], qp + 16 * s, ok);
    }
    f32x16 oacc[DM];
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) oacc[dm] = f32x16{};
    attend_block<T, D>(qf, ks, vt, 1.0f, cexp, oacc, lane);
    // The block's 32 output rows leave through the wave's LDS stage, SDM
    // tiles of 32 columns at a time: a lane holds 16-byte pieces of one row,
    // which would make every store touch 32 rows; read back, each store
    // writes whole 128-byte lines.
    const int pb = begin + 32 * blk, nrow = min(end - pb, 32);
#pragma unroll
    for (int r0 = 0; r0 < DM; r0 += SDM) {
#pragma unroll
      for (int dd = 0; dd < SDM; ++dd)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(stg + (lane & 31) * kStageRow + out_col(dd, q4, half)) =
              f32x4{oacc[r0 + dd][4 * q4], oacc[r0 + dd][4 * q4 + 1], oacc[r0 + dd][4 * q4 + 2],
                    oacc[r0 + dd][4 * q4 + 3]};
      wave_lds_fence();  // the wave's LDS operations run in order; keep the compiler's too
      constexpr int LPR = 8 * SDM;   // lanes per row of the stage
      constexpr int RPI = kWave / LPR;  // rows per read
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i) {
        const int r = RPI * i + lane / LPR;
        const f32x4 x = *reinterpret_cast<const f32x4*>(stg + r * kStageRow + 4 * (lane % LPR));
        if (r < nrow) *reinterpret_cast<f32x4*>(partial + (int64_t)(pb + r) * D + 32 * r0 + 4 * (lane % LPR)) = x;
      }
      wave_lds_fence();
    }
  }
}

// ---- local pairs and fusion
#ifndef HSA_ATTN_LOCAL_WAVES_PER_EU
#define HSA_ATTN_LOCAL_WAVES_PER_EU 2
#endif
template <typename T, int D, int G, int KSEL>
__global__ __launch_bounds__(kWave* G)
    __attribute__((amdgpu_waves_per_eu(HSA_ATTN_LOCAL_WAVES_PER_EU))) void prefill_local_kernel(
    const typename T::storage* __restrict__ q, const typename T::storage* __restrict__ kk,
    const typename T::storage* __restrict__ vt_g, const int32_t* __restrict__ sel_idx,
    const float* __restrict__ sel_score, const int32_t* __restrict__ pair_pos, const float* __restrict__ partial,
    float* __restrict__ out, int B, int Hkv, int64_t T_len, int64_t T_q, int64_t Nc, int nqc, int jlo, int j0,
    int k, float scale, int nbuf, int64_t cap, uint32_t* __restrict__ dbg) {
  // the grid covers the slab of query chunks [jlo, jlo + nqc) of the T_q rows
  using st = typename T::storage;
  using TL = Tile<T, D>;
  constexpr int KCH = D / 16;
  constexpr int DM = D / 32;
  constexpr int NW = kLocalWindow / 32;  // bitmap words of one window
  // nbuf (1 or 2) chunk images, then the per-row tables: k entries per row,
  // local (chunk, weight) ascending from the front, remote (pair position,
  // weight) from the back
  extern __shared__ __align__(16) char smem[];
  int2* tab = reinterpret_cast<int2*>(smem + nbuf * TL::BYTES);
  // bitmap of the union of the workgroup's local chunks; it lives in the
  // last chunk buffer, which is first loaded after every wave holds the
  // bitmap in registers (so two workgroups of 80 KiB fit a CU)
  uint32_t* bm = reinterpret_cast<uint32_t*>(smem + (nbuf - 1) * TL::BYTES);

  const int bid = blockIdx.x;
  const int g = bid % Hkv;
  int rest = bid / Hkv;
  const int b = rest % B;
  rest /= B;
  const int hc = rest & 1;
  const int j = jlo + nqc - 1 - (rest >> 1);  // query chunk among the T_q query rows
  const int ja = j0 + j;                 // its absolute chunk (keys: T_len rows)
  const int tid = threadIdx.x, lane = tid & 63, hh = tid >> 6, half = lane >> 5;
  const int Hq = Hkv * G, h = g * G + hh;
  const int64_t n = min((int64_t)ja, Nc);
  const int ws = (ja / kLocalWindow) * kLocalWindow;  // first chunk of the query's window
  const int row = hh * 32 + (lane & 31);
  const int64_t tok = (int64_t)j * kChunk + 32 * hc + (lane & 31);
  const bool tok_ok = tok < T_q;

  if (tid < NW) bm[tid] = 0u;
  __syncthreads();

  // ---- per-row tables: fusion weights of all kept chunks, local ones in
  // ascending chunk order, remote ones with their pair positions
  int m = 0, rc = 0;
  if (lane < 32 && tok_ok && n > 0) {
    const int64_t base = (((int64_t)b * Hq + h) * T_q + tok) * k;
    int ci[KSEL];
    float sc[KSEL];
    if (k % 4 == 0) {
      // the row's slots as 16-byte loads (its row starts 16-byte aligned);
      // padding slots hold -1 / -inf
#pragma unroll
      for (int e4 = 0; e4 < KSEL / 4; ++e4) {
        const bool in = 4 * e4 < k;
        const u32x4 c4 = in ? *reinterpret_cast<const u32x4*>(sel_idx + base + 4 * e4)
                            : u32x4{~0u, ~0u, ~0u, ~0u};
        const f32x4 s4 = in ? *reinterpret_cast<const f32x4*>(sel_score + base + 4 * e4)
                            : f32x4{-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          ci[4 * e4 + u] = (int)c4[u];
          sc[4 * e4 + u] = (int)c4[u] >= 0 ? s4[u] : -__builtin_inff();
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < KSEL; ++e) {
        ci[e] = (e < k) ? sel_idx[base + e] : -1;
        sc[e] = (e < k && ci[e] >= 0) ? sel_score[base + e] : -__builtin_inff();
      }
    }
    const float smax = sc[0];
    float w[KSEL], den = 0.0f;
#pragma unroll
    for (int e = 0; e < KSEL; ++e) {
      w[e] = ci[e] >= 0 ? expf(sc[e] - smax) : 0.0f;
      den += w[e];
    }
    const float inv = 1.0f / den;
    // a pair with a bucket position (pair_pos >= 0) was attended chunk-major
    int pp[KSEL];
    if (k % 4 == 0) {
#pragma unroll
      for (int e4 = 0; e4 < KSEL / 4; ++e4) {
        const u32x4 p4 = 4 * e4 < k ? *reinterpret_cast<const u32x4*>(pair_pos + base + 4 * e4)
                                    : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < 4; ++u) pp[4 * e4 + u] = ci[4 * e4 + u] >= 0 ? (int)p4[u] : 0;
      }
    } else {
#pragma unroll
      for (int e = 0; e < KSEL; ++e) pp[e] = ci[e] >= 0 ? pair_pos[base + e] : 0;
    }
    if constexpr (HSA_ATTN_DEBUG) {
      // a local chunk must lie in the query's window and among its
      // candidates; a chunk-major pair's position inside the slab's list:
      // a pair that fails is flagged and dropped
#pragma unroll
      for (int e = 0; e < KSEL; ++e) {
        if (ci[e] < 0) continue;
        const bool good = pp[e] < 0 ? dbg_ok(dbg, ci[e] >= ws && ci[e] < ws + kLocalWindow && ci[e] < n,
                                             HSA_ATTN_DEBUG_LOCAL_CHUNK)
                                    : dbg_ok(dbg, pp[e] < cap, HSA_ATTN_DEBUG_LOCAL_POS);
        if (!good) ci[e] = -1;
      }
    }
#pragma unroll
    for (int e = 0; e < KSEL; ++e) {
      if (ci[e] >= 0 && pp[e] < 0) {
        int rank = 0;
#pragma unroll
        for (int f = 0; f < KSEL; ++f) rank += (ci[f] >= 0 && pp[f] < 0 && ci[f] < ci[e]);
        tab[row * k + rank] = make_int2(ci[e], __float_as_int(w[e] * inv));
        atomicOr(&bm[(ci[e] - ws) >> 5], 1u << ((ci[e] - ws) & 31));
        ++m;
      } else if (ci[e] >= 0) {
        ++rc;
        tab[row * k + k - rc] = make_int2(pp[e], __float_as_int(w[e] * inv));
      }
    }
  }
  m = __shfl(m, lane & 31);  // the partner lane of the row learns the counts
  rc = __shfl(rc, lane & 31);
  __syncthreads();

  Frag<T> qf[KCH];
  {
    const st* qp = q + (((int64_t)b * Hq + h) * T_q + (tok_ok ? tok : 0)) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < KCH; ++s) load_frag_global(qf[s], qp + 16 * s, tok_ok);
  }
  f32x16 oacc[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm) oacc[dm] = f32x16{};

  // walk the union of the block's local selections in ascending order
  static_assert(NW == 2, "bitmap of one 64-chunk window");
  uint32_t bw[NW];
#pragma unroll
  for (int i = 0; i < NW; ++i) bw[i] = __builtin_amdgcn_readfirstlane(bm[i]);
  int word = 0;
  uint32_t bits = bw[0];
  auto next_chunk = [&]() -> int {
    while (bits == 0u) {
      if (++word >= NW) return -1;
      bits = bw[1];
    }
    const int c = ws + word * 32 + __builtin_ctz(bits);
    bits &= bits - 1u;
    return c;
  };
  const char* kg = reinterpret_cast<const char*>(kk + ((int64_t)b * Hkv + g) * T_len * D);
  const char* vtg = reinterpret_cast<const char*>(vt_g) + ((int64_t)b * Hkv + g) * Nc * TL::KBYTES;
  auto issue = [&](int c, int buf) {
    TL::template issue<G>(kg + (int64_t)c * TL::KBYTES, vtg + (int64_t)c * TL::KBYTES, smem + buf * TL::BYTES, hh,
                          lane);
  };
  const float cexp = scale * 1.4426950408889634f;
  int ptr = 0;
  int c = next_chunk();
  if (nbuf == 1) __syncthreads();  // the bitmap shares buffer 0: all waves have read it
  if (c >= 0) issue(c, 0);
  // Chunk i sits in buffer i % nbuf.  With two buffers the loads of chunk
  // i+1 run during the computation of chunk i and one barrier per chunk
  // suffices; with one buffer (large tiles) the loads wait for it.
  for (int it = 0; c >= 0; ++it) {
    wait_loads();
    __syncthreads();  // chunk it is in LDS; every wave is done with chunk it-1
    const int cn = next_chunk();
    if (nbuf == 2 && cn >= 0) issue(cn, (it + 1) & 1);
    const char* ks = smem + (it & (nbuf - 1)) * TL::BYTES;
    const char* vt = ks + TL::KBYTES;
    float wgt = 0.0f;
    bool mine = false;
    if (ptr < m) {
      const int2 e = tab[row * k + ptr];
      mine = e.x == c;
      if (mine) {
        wgt = __int_as_float(e.y);
        ++ptr;
      }
    }
    if (__ballot(mine)) attend_block<T, D>(qf, ks, vt, wgt, cexp, oacc, lane);
    if (nbuf == 1 && cn >= 0) {
      __syncthreads();  // every wave is done with the buffer
      issue(cn, 0);
    }
    c = cn;
  }
  // add the weighted outputs of the row's remote pairs
  int rmax = rc;
  for (int off = 32; off >= 1; off >>= 1) rmax = max(rmax, __shfl_xor(rmax, off));
  for (int r = 0; r < rmax; ++r) {
    if (r < rc) {
      const int2 e = tab[row * k + k - 1 - r];
      const float w = __int_as_float(e.y);
      const float* pp = partial + (int64_t)e.x * D;
#pragma unroll
      for (int dm = 0; dm < DM; ++dm)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(pp + out_col(dm, q4, half));
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[dm][4 * q4 + i] = fmaf(w, x[i], oacc[dm][4 * q4 + i]);
        }
    }
  }
  if (tok_ok) {
    float* op = out + (((int64_t)b * Hq + h) * T_q + tok) * D;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(op + out_col(dm, q4, half)) =
            f32x4{oacc[dm][4 * q4], oacc[dm][4 * q4 + 1], oacc[dm][4 * q4 + 2], oacc[dm][4 * q4 + 3]};
  }
}

// LDS of the local kernel: nbuf chunk images and the per-row tables
size_t prefill_local_lds_bytes(const Geometry& g, int nbuf);
int prefill_local_buffers(const Geometry& g);

template <typename T, int D, int G, int KSEL>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  const Geometry& g = a.g;
  using stg = typename T::storage;
  const int nqc = (int)((g.Tq + kChunk - 1) / kChunk);  // query chunks
  const int j0 = (int)g.J0;
  const float scale = 1.0f / sqrtf((float)D);
  const stg* q = static_cast<const stg*>(a.q);
  const stg* k = static_cast<const stg*>(a.k);
  const stg* v = static_cast<const stg*>(a.v);
  constexpr int HPW = G < 4 ? G : 4;
  const int64_t nb = (int64_t)g.B * g.Hkv * g.Nc;  // chunks = remote-pair buckets
  const int cps = (int)(a.slab_rows / kChunk);      // query chunks per slab
  if (cps < 1) return hipErrorInvalidValue;
  const int nbuf = prefill_local_buffers(g);
  const size_t lds = prefill_local_lds_bytes(g, nbuf);
  auto local = prefill_local_kernel<T, D, G, KSEL>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(local),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  // Launch order per call: the transposed V tiles once; then per group of
  // up to kPrefillCountSlabs slabs of query chunks [jg, jg + ng): the
  // group's bucket counts cleared, one selection over its rows (which
  // counts each slab's remote pairs apart), one scan of every slab's counts
  // and one scatter of the group's remote pairs into each slab's list; then
  // per slab [jlo, jlo + ns): chunk-major attention, local attention and
  // fusion.
  if (nb > 0) {
    launch_kernel((prefill_vt_kernel<T, D>), dim3((unsigned)nb), dim3(256), 0, st, v, static_cast<stg*>(a.vt),
                  g.T, g.Nc);
  }
  const int sgc = cps * a.slab_group;  // query chunks per selection launch
  const int64_t cap = (int64_t)g.B * g.Hq * a.slab_rows * g.k;
  for (int jg = 0; jg < nqc; jg += sgc) {
    const int ng = std::min(sgc, nqc - jg);
    if (nb > 0) {
      hipError_t e = launch_prefill_zero_counts(a, st);
      if (e != hipSuccess) return e;
    }
    const unsigned gblocks = (unsigned)((int64_t)ng * g.B * g.Hkv);
    launch_kernel((prefill_select_kernel<T, D, G, KSEL>), dim3(gblocks * (G / HPW)), dim3(kWave * HPW), 0, st,
                  q, static_cast<const stg*>(a.lm), a.sel_idx, a.sel_score, nb > 0 ? a.cnt : nullptr,
                  a.pair_pos, g.B, g.Hkv, g.Tq, g.Nc, ng, jg, cps, j0, g.k, scale, a.k_base, a.gap_tau);
    if (nb > 0) {
      const int64_t r0 = (int64_t)jg * kChunk, rn = std::min<int64_t>((int64_t)ng * kChunk, g.Tq - r0);
      hipError_t e = launch_prefill_bucketing(a, (ng + cps - 1) / cps, r0, rn, st);
      if (e != hipSuccess) return e;
    }
    for (int jlo = jg; jlo < jg + ng; jlo += cps) {
      const int ns = std::min(cps, jg + ng - jlo);
      const int sl = (jlo - jg) / cps;
      const unsigned blocks = (unsigned)((int64_t)ns * g.B * g.Hkv);
      if (nb > 0) {
        launch_kernel((prefill_remote_kernel<T, D, G>), dim3((unsigned)nb), dim3(256), 0, st, q, k,
                      static_cast<const stg*>(a.vt), a.off + (int64_t)sl * (nb + 1), a.pairs + sl * cap,
                      a.partial, g.Hkv, g.T, g.Nc, scale, cap, (int64_t)g.B * g.Hq * g.Tq, a.dbg);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      launch_kernel(local, dim3(2 * blocks), dim3(kWave * G), lds, st, q, k, static_cast<const stg*>(a.vt),
                    a.sel_idx, a.sel_score, a.pair_pos, a.partial, a.out, g.B, g.Hkv, g.T, g.Tq, g.Nc, ns, jlo,
                    j0, g.k, scale, nbuf, cap, a.dbg);
    }
  }
  return hipGetLastError();
}

// Dispatch over the query-group size; instantiated once per (dtype, D, list
// size) in its own translation unit so the build parallelises.
template <typename T, int D, int KSEL>
hipError_t launch_prefill_g(const PrefillArgs& a, hipStream_t st) {
  switch (a.g.G) {
    case 1: return launch_prefill_t<T, D, 1, KSEL>(a, st);
    case 2: return launch_prefill_t<T, D, 2, KSEL>(a, st);
    case 4: return launch_prefill_t<T, D, 4, KSEL>(a, st);
    default:
      // 64-entry lists: the local kernel's per-row tables of eight heads
      // would not fit the LDS next to a chunk image (the host rejects it)
      if constexpr (KSEL > 32) return hipErrorNotSupported;
      else return launch_prefill_t<T, D, 8, KSEL>(a, st);
  }
}

}  // namespace hsa_attn
