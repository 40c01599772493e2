// Score every far token against the query sketch ("What it took" on the page
// "8 agents x 250K context, concurrently, on two 3090s": score every token).
//
// scores[b][i][h][t] = sum_c qsk[b][i][h][c] * S[b][h][t][c], exact int32.
//
// The pass is a pure HBM stream of 64-byte int8 rows.  Layout: a quad of
// lanes owns one token row, each lane 16 bytes, so one dwordx4 load of a wave
// covers 16 consecutive rows (1 KiB, fully coalesced).  Each lane keeps 8
// loads in flight, does v_dot4 on its 16 bytes for every query row, and the
// quad sums by DPP.  Lane p of a quad then writes the scores of unroll slots
// p and p+4, so every store instruction writes 64 consecutive int32.
//
// Optionally (HIST) the kernel also builds the level-1 selection histogram
// of each row (top 11 bits of the biased score, see k_topk.hip) in LDS while
// the scores are in registers, and adds its non-zero bins to the workspace
// histogram with integer atomics: the top-k pass then needs no extra read of
// the scores to find its threshold bin.  It also records the largest biased
// score of each row in its 1024-entry chunk (plus one; 0 for an empty
// chunk), so that the top-k filter reads only the chunks that can hold a
// candidate.
//
// In candidate mode (CAND, without HIST) no score is stored: each row keeps,
// in its chunk's candidate list of the selection workspace, the entries
// whose biased score reaches the row's estimate E, as (index, biased score)
// in index order, and the list's length.  `samp` holds the segments' sample
// histograms (built beforehand by the selection's sample pass), from which
// every workgroup derives E itself (block_estimate), so every workgroup of a
// segment finds the same E; or (EST) the segments' selection records, whose
// first int holds the estimate derived by the sample pass when one workgroup
// sampled the whole segment (a derived E is recorded there as well, for the
// final pass).  The final selection pass then needs no filter pass and
// no histogram from this pass: it counts the candidates' level-1 bins itself
// (adding a few bins per workgroup into one histogram per segment, from
// every workgroup, cost this pass 3 us at 250K in same-address atomics).
#include "sks_internal.h"

namespace sks {
namespace {

typedef int v4i_t __attribute__((ext_vector_type(4)));

// Sketch rows are read exactly once per step and the scores are consumed by
// the next kernel only: both go through nontemporal accesses so that the
// stream does not evict useful lines (measured: ~13% faster on this pass).
__device__ __forceinline__ int4 load_stream(const int4 *p) {
  const v4i_t v = __builtin_nontemporal_load(reinterpret_cast<const v4i_t *>(p));
  return make_int4(v.x, v.y, v.z, v.w);
}

constexpr int SC_THREADS = 256;
constexpr int SC_UNROLL = 8;                        // rows per lane-quad per step
constexpr int SC_WAVE_STEP = 16 * SC_UNROLL;        // 128 rows per wave step
constexpr int SC_BLOCK_STEP = SC_WAVE_STEP * (SC_THREADS / 64);   // 512

template <int R, bool HIST, bool CAND, bool EST = false>
__global__ __launch_bounds__(SC_THREADS) void score_kernel(
    const int8_t *__restrict__ qsk, const int8_t *__restrict__ S,
    const int32_t *__restrict__ seq_len, int32_t *__restrict__ scores,
    int32_t *__restrict__ hist1, int32_t *__restrict__ cmax, int n_sub_max, int Hkv, int T_max,
    int NB, int window, int pool, int topk, const int32_t *__restrict__ samp,
    int2 *__restrict__ cand, int32_t *__restrict__ cnt, int force, int32_t *__restrict__ est_out) {
  static_assert(SCORE_CHUNK == TK_SUB, "one chunk maximum per top-k sub-list");
  static_assert(SCORE_CHUNK == 4 * SC_THREADS, "candidate compaction: 4 rounds of 64 per wave");
  static_assert(!(CAND && HIST), "candidate mode builds no histogram");
  static_assert(!EST || CAND, "a given estimate is candidate mode's");
  __shared__ int lh[HIST ? R * HIST1_BINS : 1];
  __shared__ int lmax[HIST ? R * (SC_THREADS / 64) : 1];
  __shared__ int gcnt[CAND ? R * 16 : 1];                // candidates per 64-token group
  __shared__ int escan[CAND ? SC_THREADS / 64 : 1];      // estimate: the waves' bin counts
  __shared__ int e_lds[CAND ? R : 1];
  __shared__ __align__(16) int lsc[CAND ? 1 : R * SCORE_CHUNK];   // the chunk's scores, stored at the end
  const int bh = blockIdx.y, b = bh / Hkv, h = bh % Hkv;
  const int L0 = clamp_len(seq_len[b], T_max, R);
  const int Lmax = L0 + R - 1;
  const int n_far = Lmax > window ? (Lmax - window) / pool : 0;
  const int c0 = blockIdx.x * SCORE_CHUNK;
  if (c0 >= n_far) return;
  const int c1 = min(n_far, c0 + SCORE_CHUNK);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int quad = lane >> 2, part = lane & 3;
  // per-row far counts (rows differ by one token each); a row whose top-k
  // takes everything needs no histogram and no candidates
  int nf[R], ke[R];
  bool need_sel[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const RowGeom rg = row_geom(L0, i, window, pool, topk);
    nf[i] = rg.n_far;
    ke[i] = rg.k_eff;
    need_sel[i] = rg.k_eff < rg.n_far;
  }
  if (HIST) {
    for (int k = threadIdx.x; k < R * HIST1_BINS; k += SC_THREADS) lh[k] = 0;
    __syncthreads();
  }

  int4 qv[R];
#pragma unroll
  for (int i = 0; i < R; ++i)
    qv[i] = *reinterpret_cast<const int4 *>(qsk + ((size_t)(b * R + i) * Hkv + h) * RANK + part * 16);
  // candidate mode: thread t's 8 bins of each row's sample histogram, from
  // the top bin down (bins 2047 - 8t ... 2040 - 8t), loaded ahead of the
  // stream -- or (EST) the row's estimate, derived by the step's first launch.
  // Every workgroup of a segment must use the same E (the final pass relies
  // on one E per segment): block_estimate gives every workgroup reading the
  // same bins the same E, even for a workspace that held garbage.
  static_assert(HIST1_BINS == 8 * SC_THREADS, "eight sample bins per thread");
  int hsv[CAND && !EST ? R : 1][8];
  int e_pre[EST ? R : 1];
  if (EST) {
#pragma unroll
    for (int i = 0; i < R; ++i) e_pre[i] = samp[4 * ((size_t)(b * R + i) * Hkv + h)];
  } else if (CAND) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int4 *src = reinterpret_cast<const int4 *>(
          samp + ((size_t)(b * R + i) * Hkv + h) * HIST1_BINS + HIST1_BINS - 8 * (threadIdx.x + 1));
      const int4 lo4 = src[0], hi4 = src[1];     // ascending bins
      hsv[i][0] = hi4.w; hsv[i][1] = hi4.z; hsv[i][2] = hi4.y; hsv[i][3] = hi4.x;
      hsv[i][4] = lo4.w; hsv[i][5] = lo4.z; hsv[i][6] = lo4.y; hsv[i][7] = lo4.x;
    }
  }

  const int4 *Sbh = reinterpret_cast<const int4 *>(S + (size_t)bh * NB * RANK) + part;
  int32_t *out[R];
  int kmax[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    out[i] = CAND ? nullptr : scores + ((size_t)(b * R + i) * Hkv + h) * NB;
    kmax[i] = 0;
  }

  // candidate mode keeps each lane's keys and the waves' candidate ballots of
  // its (at most two) steps in registers: [step][lo, hi]
  int ck[R][4];
  unsigned long long cm[R][4];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ck[i][k] = -1;                             // no token: never a candidate
      cm[i][k] = 0ull;
    }
  static_assert(SCORE_CHUNK == 2 * SC_BLOCK_STEP, "two steps per wave and chunk");
  // A step's stream loads: every load is issued, and all of them before any
  // use (a load under a branch, or one the scheduler moves next to its use,
  // is waited for before the next one is issued).  Rows past the chunk's end
  // read its last row instead; their results are never used (keys, histogram
  // counts and stored scores all stop at the row's far count).
  auto stream = [&](int base, int4 (&sv)[SC_UNROLL]) {
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u)
      sv[u] = load_stream(&Sbh[(size_t)min(base + u * 16 + quad, c1 - 1) * 4]);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Candidate mode derives each row's estimate E (block_estimate: the lowest
  // key of the sample histogram's bin holding the rho-th largest sampled
  // key) while the first step's loads are in flight.  Its barriers stay out
  // of the loop below, whose trip count differs between waves at a row's
  // last chunk.
  int4 sv0[SC_UNROLL];
  if (CAND && !EST) {
    stream(c0 + wave * SC_WAVE_STEP, sv0);
#pragma unroll
    for (int i = 0; i < R; ++i)
      block_estimate<SC_THREADS>(hsv[i], nf[i], ke[i], SAMPLE_STRIDE, force, escan, &e_lds[i]);
  }
  int it = 0;
  for (int base = c0 + wave * SC_WAVE_STEP; base < c1; base += SC_BLOCK_STEP, ++it) {
    int4 sv[SC_UNROLL];
    if (CAND && !EST && it == 0) {
#pragma unroll
      for (int u = 0; u < SC_UNROLL; ++u) sv[u] = sv0[u];
    } else {
      stream(base, sv);
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      int acc[SC_UNROLL];
#pragma unroll
      for (int u = 0; u < SC_UNROLL; ++u) {
        int a = __builtin_amdgcn_sdot4(sv[u].x, qv[i].x, 0, false);
        a = __builtin_amdgcn_sdot4(sv[u].y, qv[i].y, a, false);
        a = __builtin_amdgcn_sdot4(sv[u].z, qv[i].z, a, false);
        a = __builtin_amdgcn_sdot4(sv[u].w, qv[i].w, a, false);
        acc[u] = quad_sum_i(a);
      }
      // lane `part` stores slots part and part + 4
      int lo = acc[0], hi = acc[4];
#pragma unroll
      for (int u = 1; u < 4; ++u) {
        lo = part == u ? acc[u] : lo;
        hi = part == u ? acc[u + 4] : hi;
      }
      const int t_lo = base + part * 16 + quad;
      const int t_hi = t_lo + 64;
      if (CAND) {
        // keys of tokens past the row's far region never become candidates
        const int klo = t_lo < nf[i] ? biased_key(lo) : -1;
        const int khi = t_hi < nf[i] ? biased_key(hi) : -1;
        if (it == 0) {
          ck[i][0] = klo;
          ck[i][1] = khi;
        } else {
          ck[i][2] = klo;
          ck[i][3] = khi;
        }
      } else {
        lsc[i * SCORE_CHUNK + (t_lo - c0)] = lo;
        lsc[i * SCORE_CHUNK + (t_hi - c0)] = hi;
      }
      if (HIST && need_sel[i]) {
        const int klo = biased_key(lo), khi = biased_key(hi);
        if (t_lo < nf[i]) {
          atomicAdd(&lh[i * HIST1_BINS + (klo >> HIST2_BITS)], 1);
          if (!CAND) kmax[i] = max(kmax[i], klo + 1);
        }
        if (t_hi < nf[i]) {
          atomicAdd(&lh[i * HIST1_BINS + (khi >> HIST2_BITS)], 1);
          if (!CAND) kmax[i] = max(kmax[i], khi + 1);
        }
      }
    }
  }
  if (HIST && !CAND) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int wm = __builtin_amdgcn_readlane(wave_incl_max(kmax[i]), 63);
      if (lane == 0) lmax[i * (SC_THREADS / 64) + wave] = wm;
    }
  }
  if (CAND) {
    if (!EST) {
      // the segment's E for the final pass, in its counters record (every
      // workgroup derived the same)
      if (est_out && blockIdx.x == 0 && threadIdx.x < R)
        est_out[4 * ((size_t)(b * R + threadIdx.x) * Hkv + h)] = e_lds[threadIdx.x];
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      // (a given estimate is clamped at 0, so that garbage in the workspace
      // can never admit the key -1 of a slot without a token)
      const int E = !EST ? e_lds[i] : force == 1 ? (1 << 30) : force == 2 ? 0 : max(e_pre[i], 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) cm[i][k] = __ballot(need_sel[i] && ck[i][k] >= E);
    }
    if (lane == 0) {
      // 64-token groups in token order: g = step * 8 + wave * 2 + (lo, hi)
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) gcnt[i * 16 + (k >> 1) * 8 + wave * 2 + (k & 1)] = __popcll(cm[i][k]);
    }
  }
  __syncthreads();
  if (CAND) {
    // Lane 4q + p holds token 16p + q of each group: its rank among the
    // group's candidates counts the set bits of parts p' < p, then those of
    // part p below quad q.  The groups' offsets in the chunk's list: lane
    // 16 (i % 4) + g of every wave scans group g of row i inside its row of
    // 16 lanes, and the offsets are read back by lane index.
    constexpr unsigned long long PART0 = 0x1111111111111111ull;
    const unsigned long long before_q = (1ull << (4 * quad)) - 1ull;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int gincl[(R + 3) / 4], gv[(R + 3) / 4];
#pragma unroll
    for (int r4 = 0; r4 < (R + 3) / 4; ++r4) {
      const int ii = 4 * r4 + (lane >> 4);
      gv[r4] = ii < R ? gcnt[ii * 16 + (lane & 15)] : 0;
      int x = gv[r4];
      x += dpp_shr<1>(x);
      x += dpp_shr<2>(x);
      x += dpp_shr<4>(x);
      x += dpp_shr<8>(x);
      gincl[r4] = x;
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (!need_sel[i]) continue;                  // uniform: the row selects everything
      const size_t seg = (size_t)(b * R + i) * Hkv + h;
      int2 *dst = cand + (seg * n_sub_max + blockIdx.x) * TK_SUB;
      const int tot = __builtin_amdgcn_readlane(gincl[i / 4], 16 * (i % 4) + 15);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int g = (k >> 1) * 8 + wv * 2 + (k & 1);
        const int off = __builtin_amdgcn_readlane(gincl[i / 4], 16 * (i % 4) + g) -
                        __builtin_amdgcn_readlane(gv[i / 4], 16 * (i % 4) + g);
        const unsigned long long M = cm[i][k];
        if ((M >> lane) & 1ull) {
          int rank = __popcll(M & (PART0 << part) & before_q);
#pragma unroll
          for (int pp = 0; pp < 3; ++pp) rank += pp < part ? __popcll(M & (PART0 << pp)) : 0;
          const int tok = c0 + (k >> 1) * SC_BLOCK_STEP + wave * SC_WAVE_STEP + (k & 1) * 64 +
                          16 * part + quad;
          dst[off + rank] = make_int2(tok, ck[i][k]);
        }
      }
      if (threadIdx.x == 0) cnt[seg * n_sub_max + blockIdx.x] = tot;
    }
  }
  // The chunk's scores leave in one burst per row: 16-byte stores when the
  // row is 16-byte aligned here, else 4-byte stores.
  const int n_chunk = c1 - c0;
#pragma unroll
  for (int i = 0; i < (CAND ? 0 : R); ++i) {
    int32_t *dst = out[i] + c0;
    if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
      for (int v = threadIdx.x; 4 * v < n_chunk; v += SC_THREADS) {
        const v4i_t w = *reinterpret_cast<const v4i_t *>(&lsc[i * SCORE_CHUNK + 4 * v]);
        if (4 * v + 4 <= n_chunk) {
          __builtin_nontemporal_store(w, reinterpret_cast<v4i_t *>(dst) + v);
        } else {
          for (int k = 0; 4 * v + k < n_chunk; ++k) dst[4 * v + k] = w[k];
        }
      }
    } else {
      for (int t = threadIdx.x; t < n_chunk; t += SC_THREADS)
        __builtin_nontemporal_store(lsc[i * SCORE_CHUNK + t], dst + t);
    }
  }
  if (HIST) {
    if (!CAND && threadIdx.x < R) {
      const int i = threadIdx.x;
      int m = 0;
#pragma unroll
      for (int w = 0; w < SC_THREADS / 64; ++w) m = max(m, lmax[i * (SC_THREADS / 64) + w]);
      cmax[((size_t)(b * R + i) * Hkv + h) * n_sub_max + blockIdx.x] = m;
    }
    for (int k = threadIdx.x; k < R * HIST1_BINS; k += SC_THREADS) {
      const int v = lh[k];
      const int i = k / HIST1_BINS;
      if (v) atomicAdd(&hist1[((size_t)(b * R + i) * Hkv + h) * HIST1_BINS + (k % HIST1_BINS)], v);
    }
  }
}

}  // namespace

hipError_t launch_score(const int8_t *qsk, const int8_t *S, const int32_t *seq_len,
                        const Shape &s, int32_t *scores, const TopkWs *w, hipStream_t st,
                        bool cand, int force, const int32_t *est) {
  if (cand && !w) return hipErrorInvalidValue;
  int32_t *hist1 = w ? w->hist1 : nullptr;
  int32_t *cmax = w ? w->cmax : nullptr;
  const int n_sub_max = w ? w->nchunk : 0;
  // the largest far count any row can have is (T_max - window) / pool <= NB
  long max_far = s.T_max > s.window ? (long)(s.T_max - s.window) / s.pool : 0;
  if (max_far <= 0) return hipSuccess;
  dim3 grid(ceil_div(max_far, SCORE_CHUNK), s.B * s.Hkv);
  switch (s.R) {
#define SKS_SCORE_CASE(RR)                                                                     \
  case RR:                                                                                     \
    if (cand && est)                                                                           \
      score_kernel<RR, false, true, true><<<grid, SC_THREADS, 0, st>>>(                        \
          qsk, S, seq_len, nullptr, nullptr, nullptr, n_sub_max, s.Hkv, s.T_max, s.NB, s.window, \
          s.pool, s.topk, est, w->cand, w->cnt, force, nullptr);                               \
    else if (cand)                                                                             \
      score_kernel<RR, false, true><<<grid, SC_THREADS, 0, st>>>(                              \
          qsk, S, seq_len, nullptr, nullptr, nullptr, n_sub_max, s.Hkv, s.T_max, s.NB, s.window, \
          s.pool, s.topk, w->hsamp, w->cand, w->cnt, force, w->counters);                      \
    else if (hist1)                                                                            \
      score_kernel<RR, true, false><<<grid, SC_THREADS, 0, st>>>(                              \
          qsk, S, seq_len, scores, hist1, cmax, n_sub_max, s.Hkv, s.T_max, s.NB, s.window,     \
          s.pool, s.topk, nullptr, nullptr, nullptr, 0, nullptr);                              \
    else                                                                                       \
      score_kernel<RR, false, false><<<grid, SC_THREADS, 0, st>>>(                             \
          qsk, S, seq_len, scores, nullptr, nullptr, 0, s.Hkv, s.T_max, s.NB, s.window,        \
          s.pool, s.topk, nullptr, nullptr, nullptr, 0, nullptr);                              \
    break;
    SKS_SCORE_CASE(1)
    SKS_SCORE_CASE(2)
    SKS_SCORE_CASE(3)
    SKS_SCORE_CASE(4)
    SKS_SCORE_CASE(5)
    SKS_SCORE_CASE(6)
    SKS_SCORE_CASE(7)
    SKS_SCORE_CASE(8)
#undef SKS_SCORE_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sks
