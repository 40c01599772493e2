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

template <int R, bool HIST>
__global__ __launch_bounds__(SC_THREADS) void score_kernel(
    const int8_t *__restrict__ qsk, const int8_t *__restrict__ S,
    const int32_t *__restrict__ seq_len, int32_t *__restrict__ scores,
    int32_t *__restrict__ hist1, int32_t *__restrict__ cmax, int n_sub_max, int Hkv, int T_max,
    int NB, int window, int pool, int topk) {
  static_assert(SCORE_CHUNK == TK_SUB, "one chunk maximum per top-k sub-list");
  __shared__ int lh[HIST ? R * HIST1_BINS : 1];
  __shared__ int lmax[HIST ? R * (SC_THREADS / 64) : 1];
  __shared__ __align__(16) int lsc[R * SCORE_CHUNK];     // this chunk's scores, written at the end
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
  // takes everything needs no histogram
  int nf[R];
  bool need_hist[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const RowGeom rg = row_geom(L0, i, window, pool, topk);
    nf[i] = rg.n_far;
    need_hist[i] = HIST && rg.k_eff < rg.n_far;
  }
  if (HIST) {
    for (int k = threadIdx.x; k < R * HIST1_BINS; k += SC_THREADS) lh[k] = 0;
    __syncthreads();
  }

  int4 qv[R];
#pragma unroll
  for (int i = 0; i < R; ++i)
    qv[i] = *reinterpret_cast<const int4 *>(qsk + ((size_t)(b * R + i) * Hkv + h) * RANK + part * 16);

  const int4 *Sbh = reinterpret_cast<const int4 *>(S + (size_t)bh * NB * RANK) + part;
  int32_t *out[R];
  int kmax[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    out[i] = scores + ((size_t)(b * R + i) * Hkv + h) * NB;
    kmax[i] = 0;
  }

  for (int base = c0 + wave * SC_WAVE_STEP; base < c1; base += SC_BLOCK_STEP) {
    int4 sv[SC_UNROLL];
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u) {
      const int t = base + u * 16 + quad;
      sv[u] = t < c1 ? load_stream(&Sbh[(size_t)t * 4]) : make_int4(0, 0, 0, 0);
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
      lsc[i * SCORE_CHUNK + (t_lo - c0)] = lo;
      lsc[i * SCORE_CHUNK + (t_hi - c0)] = hi;
      if (HIST && need_hist[i]) {
        const int klo = biased_key(lo), khi = biased_key(hi);
        if (t_lo < nf[i]) {
          atomicAdd(&lh[i * HIST1_BINS + (klo >> HIST2_BITS)], 1);
          kmax[i] = max(kmax[i], klo + 1);
        }
        if (t_hi < nf[i]) {
          atomicAdd(&lh[i * HIST1_BINS + (khi >> HIST2_BITS)], 1);
          kmax[i] = max(kmax[i], khi + 1);
        }
      }
    }
  }
  if (HIST) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int wm = __builtin_amdgcn_readlane(wave_incl_max(kmax[i]), 63);
      if (lane == 0) lmax[i * (SC_THREADS / 64) + wave] = wm;
    }
  }
  __syncthreads();
  // The chunk's scores leave in one burst per row: 16-byte stores when the
  // row is 16-byte aligned here, else 4-byte stores.
  const int n_chunk = c1 - c0;
#pragma unroll
  for (int i = 0; i < R; ++i) {
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
    if (threadIdx.x < R) {
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
                        const Shape &s, int32_t *scores, const TopkWs *w, hipStream_t st) {
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
    if (hist1)                                                                                 \
      score_kernel<RR, true><<<grid, SC_THREADS, 0, st>>>(qsk, S, seq_len, scores, hist1,      \
                                                          cmax, n_sub_max, s.Hkv, s.T_max,     \
                                                          s.NB, s.window, s.pool, s.topk);     \
    else                                                                                       \
      score_kernel<RR, false><<<grid, SC_THREADS, 0, st>>>(qsk, S, seq_len, scores, nullptr,   \
                                                           nullptr, 0, s.Hkv, s.T_max, s.NB,   \
                                                           s.window, s.pool, s.topk);          \
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
