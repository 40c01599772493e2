// Deterministic top-k selection over int32 sketch scores ("What it took" on
// the page "8 agents x 250K context, concurrently, on two 3090s": pick the
// top ~2K).  For every segment (b, i, h) it returns the k_eff far entries with
// the largest score, lower index first among equal scores, in ascending index
// order, padded with -1.
//
// Scores fit in 21 bits once biased by 2^20 (|score| <= 64*127^2).
//   level-1 histogram: 2048 bins of the top 11 bits, accumulated with integer
//     atomics (order-independent, so deterministic) into a workspace region
//     that is zero at rest.  Either the score kernel accumulates it while it
//     streams the sketches, or topk_hist_kernel does it here.
//     The same pass records the largest key of every 1024-entry sub-list.
//   filter: every workgroup first validates the segment's level-1 histogram
//     and derives the threshold bin b1 from it (the same value in every
//     workgroup; an invalid histogram makes every element a candidate), then
//     each wave skips a sub-list whose largest key lies below bin b1 and
//     otherwise compacts the candidates (bin >= b1) of its 1024-token
//     sub-chunk IN ORDER (ballot + popcount), and adds the low 10 bits of the
//     candidates inside bin b1 to the level-2 histogram (also zero at rest).
//   final (one workgroup per segment): guesses the threshold key T from the
//     level-2 histogram, loads the candidates into registers in index order
//     and counts, from the data, the candidates above T and equal to T.  When
//     those counts show that T is the k-th largest key, it emits every
//     candidate above T and the lowest-index ties at T, ascending, without a
//     sort.  Otherwise (a workspace that was not zero at rest, or more
//     candidates than the 8,192 its registers hold) it derives T from the
//     candidates themselves with an exact two-level radix select in LDS --
//     or from the raw scores, if fewer than k candidates came through.
//     The histograms are never trusted beyond what the data confirms.  It
//     returns the segment's histograms to zero.
//
// Candidate mode (the decode step when its caller does not read the scores)
// replaces the stored scores and the filter pass:
//   sample: scores every 64th far entry (512 sampled rows per workgroup)
//     into a per-segment histogram of the level-1 bins (zero at rest).
//   the score pass: every workgroup takes as the segment's estimate E the
//     lowest key of the sample bin holding the rho-th largest sampled key,
//     rho = 2 k' + 8 where k' is the expected number of sampled entries among
//     the k largest, keeps every far entry with key >= E in the candidate
//     lists (see k_score.hip) and counts those candidates (only) into the
//     level-1 histogram.  E is a heuristic: only the time depends on it.
//   final: as above, with the threshold guess taken from the candidates'
//     level-1 histogram and a level-2 histogram of the bin-b1 candidates.
//     If at least k entries reach E, the k largest are all candidates and
//     the selection is exact; otherwise E was too high and the segment's
//     scores are recomputed from the sketches and selected from in full.
#include "topk_body.h"

namespace sks {
namespace {

__global__ void fill_kernel(int32_t *p, size_t n, int32_t v) {
  for (size_t k = blockIdx.x * (size_t)blockDim.x + threadIdx.x; k < n;
       k += (size_t)gridDim.x * blockDim.x)
    p[k] = v;
}

__global__ __launch_bounds__(TK_THREADS) void topk_hist_kernel(
    const int32_t *__restrict__ scores, const int32_t *__restrict__ seq_len,
    int32_t *__restrict__ hist1, int32_t *__restrict__ cmax, int n_sub_max, int R, int Hkv,
    int T_max, int NB, int window, int pool, int topk) {
  constexpr int SUBS = TK_CHUNK / TK_SUB;          // sub-lists per workgroup
  constexpr int PER_SUB = TK_SUB / TK_THREADS;     // elements per thread and sub-list
  __shared__ int lh[HIST1_BINS];
  __shared__ int lmax[SUBS][TK_THREADS / 64];
  const int seg = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const SegGeom g = seg_geom(seg, seq_len, R, Hkv, T_max, window, pool, topk);
  if (g.k_eff >= g.n_far) return;               // everything selected: no histogram needed
  const int c0 = blockIdx.x * TK_CHUNK;
  if (c0 >= g.n_far) return;
  const int c1 = min(g.n_far, c0 + TK_CHUNK);
  for (int k = threadIdx.x; k < HIST1_BINS; k += TK_THREADS) lh[k] = 0;
  __syncthreads();
  const int32_t *row = scores + (size_t)seg * NB;
  int km[SUBS];
#pragma unroll
  for (int j = 0; j < SUBS; ++j) {
    km[j] = 0;
#pragma unroll
    for (int k = 0; k < PER_SUB; ++k) {
      const int t = c0 + j * TK_SUB + k * TK_THREADS + threadIdx.x;
      if (t < c1) {
        const int key = biased_key(row[t]);
        atomicAdd(&lh[key >> HIST2_BITS], 1);
        km[j] = max(km[j], key + 1);
      }
    }
    const int wm = __builtin_amdgcn_readlane(wave_incl_max(km[j]), 63);
    if (lane == 0) lmax[j][wave] = wm;
  }
  __syncthreads();
  if (threadIdx.x < SUBS && c0 + threadIdx.x * TK_SUB < c1) {
    int m = 0;
#pragma unroll
    for (int w = 0; w < TK_THREADS / 64; ++w) m = max(m, lmax[threadIdx.x][w]);
    cmax[(size_t)seg * n_sub_max + blockIdx.x * SUBS + threadIdx.x] = m;
  }
  int32_t *gh = hist1 + (size_t)seg * HIST1_BINS;
  for (int k = threadIdx.x; k < HIST1_BINS; k += TK_THREADS)
    if (lh[k]) atomicAdd(&gh[k], lh[k]);
}

// Level-1 threshold of one segment, computed by a whole filter workgroup
// (every workgroup of the segment computes the same value from the same
// histogram).  Thread t holds bins [8t, 8t+8).  The histogram is validated
// first (every bin in [0, n], total exactly n); an invalid one (a workspace
// that was not zero at rest) yields bin 0 -- every element a candidate.
// Returns (b1, elements in bins above b1, valid, elements in bin b1).
// Contains two __syncthreads().
constexpr int TH_PER = HIST1_BINS / TK_THREADS;
static_assert(TH_PER == 8, "two 16-byte loads of bins per thread");

__device__ int4 block_threshold(const int (&v)[TH_PER], int need, int n, int *scratch, int *res) {
  constexpr int NW = TK_THREADS / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cap = n + 1;
  int sum = 0;
  bool bad = false;
#pragma unroll
  for (int k = 0; k < TH_PER; ++k) {
    bad |= v[k] < 0 || v[k] > n;
    sum = min(sum + min(max(v[k], 0), cap), cap);
  }
  const int incl = wave_incl_add_sat(sum, cap);
  const bool wbad = __ballot(bad) != 0;
  if (lane == 63) scratch[wave] = wbad ? -1 : incl;
  __syncthreads();
  int before = 0, all = 0;
  bool invalid = false;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = scratch[w];
    invalid |= t < 0;
    before += w < wave ? t : 0;
    all = min(all + max(t, 0), cap);
  }
  if (invalid || all != n) return make_int4(0, 0, 0, 0);   // uniform
  // valid: every partial sum is exact
  int ab = n - (incl + before);                  // elements of higher threads' bins
  if (ab < need && ab + sum >= need) {           // exactly one thread
    int b = -1;
#pragma unroll
    for (int k = TH_PER - 1; k >= 0; --k) {
      if (b < 0) {
        if (ab + v[k] >= need) {
          b = threadIdx.x * TH_PER + k;
          res[0] = b;
          res[1] = ab;
          res[2] = v[k];
        } else {
          ab += v[k];
        }
      }
    }
  }
  __syncthreads();
  return make_int4(res[0], res[1], 1, res[2]);
}

__global__ __launch_bounds__(TK_THREADS) void topk_filter_kernel(
    const int32_t *__restrict__ scores, const int32_t *__restrict__ seq_len,
    const int32_t *__restrict__ hist1, const int32_t *__restrict__ cmax,
    int32_t *__restrict__ hist2, int32_t *__restrict__ thr, int32_t *__restrict__ cnt,
    int2 *__restrict__ cand, int n_sub_max, int R, int Hkv, int T_max, int NB, int window,
    int pool, int topk) {
  __shared__ int scratch[TK_THREADS / 64];
  __shared__ int res[3];
  const int seg = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = blockIdx.x * (TK_CHUNK / TK_SUB) + wave;
  const int s0 = sub * TK_SUB;
  // the histogram, this sub-list's largest key and the length, all at once
  // (the sub-list index is clamped into the array; a sub-list past the far
  // region returns below)
  const int4 *gh = reinterpret_cast<const int4 *>(hist1 + (size_t)seg * HIST1_BINS) + 2 * threadIdx.x;
  const int4 h0 = gh[0], h1v = gh[1];
  const int cm = cmax[(size_t)seg * n_sub_max + min(sub, n_sub_max - 1)];
  const SegGeom g = seg_geom(seg, seq_len, R, Hkv, T_max, window, pool, topk);
  if (g.k_eff >= g.n_far || blockIdx.x * TK_CHUNK >= g.n_far) return;   // uniform per workgroup
  const int v[TH_PER] = {h0.x, h0.y, h0.z, h0.w, h1v.x, h1v.y, h1v.z, h1v.w};
  const int4 th = block_threshold(v, g.k_eff, g.n_far, scratch, res);
  if (blockIdx.x == 0 && threadIdx.x == 0) reinterpret_cast<int4 *>(thr)[seg] = th;
  const int b1 = th.x;
  if (s0 >= g.n_far) return;                     // uniform per wave
  int32_t *cnt_out = cnt + (size_t)seg * n_sub_max + sub;
  // The histogram and the maxima come from the same pass: with a valid
  // histogram, a sub-list whose largest key lies below bin b1 holds no
  // candidate and its scores are not read.
  if (th.z && (cm == 0 || ((cm - 1) >> HIST2_BITS) < b1)) {
    if (lane == 0) *cnt_out = 0;
    return;
  }
  const bool build_h2 = th.z && th.w <= HIST2_DIRECT_MAX;
  const int s1 = min(g.n_far, s0 + TK_SUB);
  const int32_t *row = scores + (size_t)seg * NB;
  // all loads at once, the index clamped below NB (always in bounds)
  // instead of branching around the load; entries past s1 are masked below
  int raw[FILTER_ITERS];
#pragma unroll
  for (int r = 0; r < FILTER_ITERS; ++r) raw[r] = row[min(s0 + r * 64 + lane, NB - 1)];
  int2 *dst = cand + ((size_t)seg * n_sub_max + sub) * TK_SUB;
  int32_t *h2 = hist2 + (size_t)seg * HIST2_BINS;
  int n = 0;
#pragma unroll
  for (int r = 0; r < FILTER_ITERS; ++r) {
    const int t = s0 + r * 64 + lane;
    const int key = biased_key(raw[r]);
    const bool f = t < s1 && (key >> HIST2_BITS) >= b1;
    const unsigned long long m = __ballot(f);
    if (f) {
      dst[n + __popcll(m & ((1ull << lane) - 1ull))] = make_int2(t, key);
      if (build_h2 && (key >> HIST2_BITS) == b1) atomicAdd(&h2[key & (HIST2_BINS - 1)], 1);
    }
    n += __popcll(m);
  }
  if (lane == 0) *cnt_out = n;
}

constexpr int TF_THREADS = 1024;

// Sample pass: workgroup x of segment y scores sampled rows j * stride,
// j in [512x, 512x + 512), and adds their level-1 bins to the segment's
// sample histogram (`out`, zero at rest; the final pass returns it to zero).
// With EST one workgroup takes a segment's whole sample and writes the
// segment's estimate E to out[4 seg] instead (sample_estimate; `out` is the
// counters record of TopkWs then).
template <bool EST>
__global__ __launch_bounds__(SAMPLE_THREADS) void topk_sample_kernel(
    const int8_t *__restrict__ qsk, const int8_t *__restrict__ S,
    const int32_t *__restrict__ seq_len, int32_t *__restrict__ out, int R, int Hkv, int T_max,
    int NB, int window, int pool, int topk, int stride) {
  __shared__ int lh[HIST1_BINS];
  __shared__ SampleEstLds est;
  const int seg = blockIdx.y;
  const SegGeom g = seg_geom(seg, seq_len, R, Hkv, T_max, window, pool, topk);
  if (g.k_eff >= g.n_far) return;               // uniform: no selection needed
  const int m = (g.n_far + stride - 1) / stride;   // rows j * stride < n_far
  const int j0 = blockIdx.x * SAMPLE_WG_ROWS;
  if (j0 >= m) return;
  int4 sv[SAMPLE_UNROLL];
  sample_load(S, ((size_t)g.b * Hkv + g.h) * NB, j0, m, stride, sv);
  for (int k = threadIdx.x; k < HIST1_BINS; k += SAMPLE_THREADS) lh[k] = 0;
  if (EST)
    for (int k = threadIdx.x; k < HIST2_BINS; k += SAMPLE_THREADS) est.h2[k] = 0;
  const int4 qv = reinterpret_cast<const int4 *>(qsk + (size_t)seg * RANK)[threadIdx.x & 3];
  __syncthreads();
  int keys[SAMPLE_UNROLL];
  sample_bins(sv, qv, j0, m, lh, keys);
  __syncthreads();
  if (EST) {
    const int E = sample_estimate(lh, keys, g.n_far, g.k_eff, stride, est);
    if (threadIdx.x == 0) out[4 * seg] = E;
    return;
  }
  sample_flush(lh, out + (size_t)seg * HIST1_BINS);
}

__global__ __launch_bounds__(TF_THREADS) void topk_final_kernel(
    const int32_t *cnt, const int32_t *thr, const int32_t *seq_len, int32_t *hist1,
    int32_t *hist2, int n_sub_max, int R, int Hkv, FinalArgs a) {
  __shared__ FinalLds<TF_THREADS, TK_MAX_SUBS, true> lds;
  const FinalLead ld{cnt, thr, seq_len, hist1, hist2, n_sub_max, R, Hkv};
  final_body<TF_THREADS, TK_MAX_SUBS, true>(a, ld, blockIdx.x, lds);
}

void launch_final(const FinalArgs &a, int nseg, hipStream_t st) {
  topk_final_kernel<<<nseg, TF_THREADS, 0, st>>>(a.cnt, a.thr, a.seq_len, a.hist1, a.hist2,
                                                 a.n_sub_max, a.R, a.Hkv, a);
}

}  // namespace

size_t hist_region_bytes(const Shape &s) {
  const size_t nseg = (size_t)s.B * s.R * s.Hkv;
  const size_t n_sub = (size_t)ceil_div(s.NB, TK_SUB);
  return 2 * align_up(nseg * HIST1_BINS * 4, 256) + align_up(nseg * HIST2_BINS * 4, 256) +
         align_up(nseg * 16, 256) + align_up(nseg * n_sub * 4, 256);
}

size_t topk_scratch_bytes(const Shape &s) {
  const size_t nseg = (size_t)s.B * s.R * s.Hkv;
  const size_t n_sub = (size_t)ceil_div(s.NB, TK_SUB);
  return align_up(nseg * n_sub * 4, 256) + align_up(nseg * n_sub * TK_SUB * sizeof(int2), 256);
}

TopkWs topk_ws_carve(const Shape &s, void *ws) {
  const size_t nseg = (size_t)s.B * s.R * s.Hkv;
  const size_t n_sub = (size_t)ceil_div(s.NB, TK_SUB);
  char *base = static_cast<char *>(ws);
  TopkWs w{};
  char *q = base;
  w.hist1 = reinterpret_cast<int32_t *>(q);
  q += align_up(nseg * HIST1_BINS * 4, 256);
  w.hist2 = reinterpret_cast<int32_t *>(q);
  q += align_up(nseg * HIST2_BINS * 4, 256);
  w.counters = reinterpret_cast<int32_t *>(q);
  q += align_up(nseg * 16, 256);
  w.cmax = reinterpret_cast<int32_t *>(q);
  q += align_up(nseg * n_sub * 4, 256);
  w.hsamp = reinterpret_cast<int32_t *>(q);
  char *p = base + hist_region_bytes(s);
  w.scratch = p;
  w.cnt = reinterpret_cast<int32_t *>(p);
  p += align_up(nseg * n_sub * 4, 256);
  w.cand = reinterpret_cast<int2 *>(p);
  w.nchunk = (int)n_sub;
  w.attn = base + hist_region_bytes(s) + topk_scratch_bytes(s);
  return w;
}

hipError_t launch_fill(int32_t *p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  fill_kernel<<<(int)std::min<size_t>(2048, (n + 255) / 256), 256, 0, st>>>(p, n, 0);
  return hipGetLastError();
}

hipError_t launch_topk_filter(const int32_t *scores, const int32_t *seq_len, const Shape &s,
                              bool hist_ready, const TopkWs &w, hipStream_t st) {
  const int nseg = s.B * s.R * s.Hkv;
  long max_far = s.T_max > s.window ? (long)(s.T_max - s.window) / s.pool : 0;
  if (max_far > 0) {
    dim3 grid(ceil_div(max_far, TK_CHUNK), nseg);
    if (!hist_ready)
      topk_hist_kernel<<<grid, TK_THREADS, 0, st>>>(scores, seq_len, w.hist1, w.cmax, w.nchunk,
                                                    s.R, s.Hkv, s.T_max, s.NB, s.window, s.pool,
                                                    s.topk);
    topk_filter_kernel<<<grid, TK_THREADS, 0, st>>>(scores, seq_len, w.hist1, w.cmax, w.hist2,
                                                    w.counters, w.cnt, w.cand, w.nchunk, s.R,
                                                    s.Hkv, s.T_max, s.NB, s.window, s.pool,
                                                    s.topk);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const int32_t *scores, const int32_t *seq_len, const Shape &s,
                       bool hist_ready, int32_t *idx, int32_t *n_sel, const TopkWs &w,
                       hipStream_t st) {
  const int nseg = s.B * s.R * s.Hkv;
  // Far regions that fit the final pass's registers need no filter: every
  // far entry is a candidate there, and the exact select runs in LDS.
  const long max_far = s.T_max > s.window ? (long)(s.T_max - s.window) / s.pool : 0;
  FinalArgs a = final_args(scores, seq_len, s, idx, n_sel, w);
  if (max_far <= TF_REGS) {
    a.skip = 1;
    a.h1_ready = hist_ready;
  } else {
    hipError_t e = launch_topk_filter(scores, seq_len, s, hist_ready, w, st);
    if (e != hipSuccess) return e;
  }
  launch_final(a, nseg, st);
  return hipGetLastError();
}

// Candidate mode pays off where the final pass cannot simply take every far
// entry (more than TF_REGS of them), and either the sample workgroups derive
// the estimates themselves (one per segment: rows of at most 65,536 far
// entries) or single-row steps stream enough sketch rows (2^20) for the
// saved score stores to outweigh the per-workgroup estimate.  (A verify-row
// score pass that derives three rows' estimates in every workgroup measured
// slower than storing the scores.)
bool topk_cand_preferred(const Shape &s) {
  const long max_far = s.T_max > s.window ? (long)(s.T_max - s.window) / s.pool : 0;
  const long nseg = (long)s.B * s.R * s.Hkv;
  return max_far > TF_REGS && (topk_cand_est_early(s) || (s.R == 1 && nseg * max_far >= (1L << 20)));
}

bool topk_cand_est_early(const Shape &s) {
  const long max_far = s.T_max > s.window ? (long)(s.T_max - s.window) / s.pool : 0;
  return max_far <= (long)SAMPLE_WG_ROWS * SAMPLE_EST_STRIDE;
}

int topk_cand_est_stride(const Shape &s) {
  const long max_far = s.T_max > s.window ? (long)(s.T_max - s.window) / s.pool : 0;
  return max_far <= (long)SAMPLE_WG_ROWS * SAMPLE_STRIDE ? SAMPLE_STRIDE : SAMPLE_EST_STRIDE;
}

hipError_t launch_topk_sample(const int8_t *qsk, const int8_t *S, const int32_t *seq_len,
                              const Shape &s, const TopkWs &w, hipStream_t st) {
  const int nseg = s.B * s.R * s.Hkv;
  const long max_far = s.T_max > s.window ? (long)(s.T_max - s.window) / s.pool : 0;
  const long max_m = (max_far + SAMPLE_STRIDE - 1) / SAMPLE_STRIDE;
  if (max_m > 0 && topk_cand_est_early(s))
    topk_sample_kernel<true><<<dim3(1, nseg), SAMPLE_THREADS, 0, st>>>(
        qsk, S, seq_len, w.counters, s.R, s.Hkv, s.T_max, s.NB, s.window, s.pool, s.topk,
        topk_cand_est_stride(s));
  else if (max_m > 0)
    topk_sample_kernel<false><<<dim3(ceil_div(max_m, SAMPLE_WG_ROWS), nseg), SAMPLE_THREADS, 0, st>>>(
        qsk, S, seq_len, w.hsamp, s.R, s.Hkv, s.T_max, s.NB, s.window, s.pool, s.topk,
        SAMPLE_STRIDE);
  return hipGetLastError();
}

hipError_t launch_topk_cand(const int8_t *qsk, const int8_t *S, int32_t *scores,
                            const int32_t *seq_len, const Shape &s, int32_t *idx,
                            int32_t *n_sel, const TopkWs &w, hipStream_t st, bool zero_hsamp) {
  const int nseg = s.B * s.R * s.Hkv;
  FinalArgs a = final_args(scores, seq_len, s, idx, n_sel, w);
  a.cand_mode = 1;
  a.hsamp = w.hsamp;
  a.zero_hsamp = zero_hsamp ? 1 : 0;
  a.qsk = qsk;
  a.S = S;
  a.rescore = scores;
  launch_final(a, nseg, st);
  return hipGetLastError();
}

}  // namespace sks
