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
//     sort.  Otherwise (a workspace that was not zero at rest) it derives T
//     from the candidates themselves with an exact two-level radix select in
//     LDS -- or from the raw scores, if fewer than k candidates came through.
//     The histograms are never trusted beyond what the data confirms.  It
//     returns the segment's histograms to zero.
#include "sks_internal.h"

namespace sks {
namespace {

constexpr int TK_THREADS = 256;
constexpr int TF_THREADS = 1024;
constexpr int TF_WAVES = TF_THREADS / 64;
constexpr int TF_CACHE = 8192;                     // candidates held by one final workgroup
constexpr int TF_PERT = TF_CACHE / TF_THREADS;     // consecutive candidates per thread
constexpr int FILTER_ITERS = TK_SUB / 64;          // 16 loads in flight per lane
constexpr int HIST2_DIRECT_MAX = 4096;             // level-2 histogram built when bin b1 is this small
static_assert(TK_CHUNK == TK_SUB * (TK_THREADS / 64), "one sub-chunk per wave");
static_assert(TF_CACHE < 65536, "packed 16-bit counts in the emission scan");
static_assert(TF_PERT == 8, "mark padding: one int every 8 slots");

struct SegGeom {
  int b, i, h, n_far, k_eff;
};

__device__ __forceinline__ SegGeom seg_geom(int seg, const int32_t *seq_len, int R, int Hkv,
                                            int T_max, int window, int pool, int topk) {
  SegGeom g;
  g.h = seg % Hkv;
  g.i = (seg / Hkv) % R;
  g.b = seg / (Hkv * R);
  const int L0 = clamp_len(seq_len[g.b], T_max, R);
  RowGeom rg = row_geom(L0, g.i, window, pool, topk);
  g.n_far = rg.n_far;
  g.k_eff = rg.k_eff;
  return g;
}

// Inclusive block-wide prefix sum of NW waves; `tot` receives the block
// total.  `scratch` holds NW ints.  With REUSE a second barrier lets the
// caller use the same scratch again right away.
template <int NW, bool REUSE>
__device__ int block_incl_scan(int v, int *scratch, int &tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_add(v);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int before = 0;
  tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = scratch[w];
    before += w < wave ? t : 0;
    tot += t;
  }
  if (REUSE) __syncthreads();
  return incl + before;
}

// Exclusive block-wide running maximum of non-negative values (0 before the
// first thread); `scratch` holds NW ints and is not reused.
template <int NW>
__device__ int block_excl_max(int v, int *scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_max(v);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) before = max(before, w < wave ? scratch[w] : 0);
  const int prev = __builtin_amdgcn_update_dpp(0, incl, DPP_ROW_SHR + 1, 0xF, 0xF, false);
  // the lane before the first of a row is the last lane of the previous row
  const int r15 = __builtin_amdgcn_readlane(incl, 15), r31 = __builtin_amdgcn_readlane(incl, 31),
            r47 = __builtin_amdgcn_readlane(incl, 47);
  const int row = lane >> 4;
  const int prev_row = row == 0 ? 0 : (row == 1 ? r15 : (row == 2 ? r31 : r47));
  return max(before, (lane & 15) ? prev : prev_row);
}

// LDS histograms are stored padded so that 64 lanes reading their contiguous
// bins hit distinct banks.
template <int NBINS>
__device__ __forceinline__ int hpad(int b) { return b + b / (NBINS / 64); }
template <int NBINS>
constexpr int hpad_size() { return NBINS + 64; }

// Threshold search by one wave over a padded LDS histogram of NBINS bins
// (see wave_threshold_regs: an invalid histogram yields bin 0).
template <int NBINS>
__device__ int wave_threshold_bin(const int *hist, int need, int n, int &above) {
  constexpr int PER = NBINS / 64;
  const int lane = threadIdx.x & 63;
  int v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) v[k] = hist[hpad<NBINS>(lane * PER + k)];
  bool valid;
  return wave_threshold_regs<PER>(v, need, n, above, valid);
}

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

__global__ __launch_bounds__(TF_THREADS) void topk_final_kernel(
    const int32_t *__restrict__ scores, const int32_t *__restrict__ seq_len,
    int32_t *__restrict__ hist1, int32_t *__restrict__ hist2, const int32_t *__restrict__ thr,
    const int32_t *__restrict__ cnt, const int2 *__restrict__ cand, int n_sub_max, int R, int Hkv,
    int T_max, int NB, int window, int pool, int topk, int32_t *__restrict__ idx,
    int32_t *__restrict__ n_sel) {
  __shared__ int h1[hpad_size<HIST1_BINS>()];
  __shared__ int h2[hpad_size<HIST2_BINS>()];
  __shared__ int pre[TK_MAX_SUBS + 1];
  __shared__ int2 cache[TF_CACHE];
  // sub-list start marks, one int per slot padded by one every 8 so that a
  // thread's 8 consecutive slots fall in distinct banks across the wave
  __shared__ int marks[TF_CACHE + TF_CACHE / 8];
  __shared__ int sc_pre[TF_WAVES], sc_own[TF_WAVES], sc_cnt[TF_WAVES];
  __shared__ int res[6];
  const int seg = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t *gc = cnt + (size_t)seg * n_sub_max;
  int32_t *gh2 = hist2 + (size_t)seg * HIST2_BINS;
  // loads first: the first round of sub-list counts, the threshold record
  // and (wave 0) the level-2 histogram, lane l holding bins [16l, 16l+16)
  const int cv0 = threadIdx.x < n_sub_max ? gc[threadIdx.x] : 0;
  const int4 th = reinterpret_cast<const int4 *>(thr)[seg];   // (b1, above b1, valid, in b1)
  constexpr int H2_PER = HIST2_BINS / 64;
  int hv[H2_PER];
  if (wave == 0) {
#pragma unroll
    for (int k = 0; k < H2_PER / 4; ++k) {
      const int4 w = reinterpret_cast<const int4 *>(gh2 + lane * H2_PER)[k];
      hv[4 * k] = w.x;
      hv[4 * k + 1] = w.y;
      hv[4 * k + 2] = w.z;
      hv[4 * k + 3] = w.w;
    }
  }
#pragma unroll
  for (int q = 0; q < TF_PERT; ++q) marks[threadIdx.x * (TF_PERT + 1) + q] = 0;   // no mark
  const SegGeom g = seg_geom(seg, seq_len, R, Hkv, T_max, window, pool, topk);
  int32_t *out = idx + (size_t)seg * topk;
  // the filter has run: the segment's level-1 histogram returns to zero
  int32_t *gh1 = hist1 + (size_t)seg * HIST1_BINS;
  for (int k = threadIdx.x; k < HIST1_BINS; k += TF_THREADS) gh1[k] = 0;
  if (threadIdx.x == 0 && n_sel) n_sel[seg] = g.k_eff;

  // wave 0: the threshold guess T from the level-2 histogram (-1: none),
  // then that histogram returns to zero (its values are consumed)
  if (wave == 0) {
    int T = -1;
    if (g.k_eff < g.n_far && th.z && th.w >= 0 && th.w <= HIST2_DIRECT_MAX && th.x >= 0 &&
        th.x < HIST1_BINS) {
      int above;
      bool valid;
      const int b2 = wave_threshold_regs<H2_PER>(hv, g.k_eff - th.y, th.w, above, valid);
      if (valid) T = (th.x << HIST2_BITS) | b2;
    }
    if (lane == 0) res[5] = T;
#pragma unroll
    for (int k = 0; k < H2_PER / 4; ++k)
      reinterpret_cast<int4 *>(gh2 + lane * H2_PER)[k] = make_int4(0, 0, 0, 0);
  }
  if (g.k_eff >= g.n_far) {                      // every far entry is selected
    for (int j = threadIdx.x; j < topk; j += TF_THREADS) out[j] = j < g.n_far ? j : -1;
    return;
  }

  // candidate list: exclusive prefix over the sub-list counts; every
  // non-empty sub-list also marks its first slot with its number + 1
  const int n_sub = (g.n_far + TK_SUB - 1) / TK_SUB;
  int carry = 0;
  for (int base = 0; base < n_sub; base += TF_THREADS) {
    const int sidx = base + threadIdx.x;
    const int v = sidx < n_sub ? (base == 0 ? cv0 : gc[sidx]) : 0;
    int tot;
    const int incl = block_incl_scan<TF_WAVES, true>(v, sc_pre, tot);
    const int start = carry + incl - v;
    if (sidx < n_sub) {
      pre[sidx] = start;
      if (v > 0 && start < TF_CACHE) marks[start + (start >> 3)] = sidx + 1;
    }
    carry += tot;
  }
  if (threadIdx.x == 0) pre[n_sub] = carry;
  __syncthreads();
  // Fewer candidates than k means the filter's histogram was not one of these
  // scores: select from the raw scores instead.
  const bool raw = carry < g.k_eff;
  const int m = raw ? g.n_far : carry;
  const int2 *cseg = cand + (size_t)seg * n_sub_max * TK_SUB;
  const int32_t *srow = scores + (size_t)seg * NB;
  const bool cached = !raw && m <= TF_CACHE;
  const int o0 = threadIdx.x * TF_PERT;          // this thread's slots [o0, o0 + TF_PERT)

  if (cached) {
    // The sub-list holding slot o is the last mark at or before o: a running
    // maximum over the marks of this thread's slots, then across the block.
    int mk[TF_PERT];
    int run = 0;
#pragma unroll
    for (int q = 0; q < TF_PERT; ++q) {
      run = max(run, marks[threadIdx.x * (TF_PERT + 1) + q]);
      mk[q] = run;
    }
    const int before = block_excl_max<TF_WAVES>(run, sc_own);
    int2 c[TF_PERT];
#pragma unroll
    for (int q = 0; q < TF_PERT; ++q) {
      const int o = min(o0 + q, m - 1);
      const int s = min(max(max(before, mk[q]), 1) - 1, n_sub - 1);   // clamped: always in bounds
      c[q] = cseg[(size_t)s * TK_SUB + min(max(o - pre[s], 0), TK_SUB - 1)];
    }
    const int T = res[5];
    if (T >= 0) {
      // Count, from the data, the candidates above T and equal to T.  Every
      // element with key >= T is a candidate (its bin is >= b1), so T is the
      // k-th largest key exactly when above < k <= above + equal.
      int gt = 0, tie = 0;
#pragma unroll
      for (int q = 0; q < TF_PERT; ++q) {
        const bool in = o0 + q < m;
        gt += in && c[q].y > T;
        tie += in && c[q].y == T;
      }
      const int packed = gt | (tie << 16);
      int tot;
      const int ex = block_incl_scan<TF_WAVES, false>(packed, sc_cnt, tot) - packed;
      const int gt_tot = tot & 0xffff, tie_tot = tot >> 16;
      if (gt_tot < g.k_eff && gt_tot + tie_tot >= g.k_eff) {      // uniform
        const int need = g.k_eff - gt_tot;     // ties at T to take, lowest index first
        int gt_before = ex & 0xffff, tie_before = ex >> 16;
#pragma unroll
        for (int q = 0; q < TF_PERT; ++q) {
          const bool in = o0 + q < m;
          const bool is_gt = in && c[q].y > T, is_tie = in && c[q].y == T;
          const bool sel = is_gt || (is_tie && tie_before < need);
          const int pos = gt_before + min(tie_before, need);
          if (sel) out[pos] = c[q].x;
          gt_before += is_gt;
          tie_before += is_tie;
        }
        for (int j = g.k_eff + threadIdx.x; j < topk; j += TF_THREADS) out[j] = -1;
        return;
      }
    }
    // the guess did not hold: keep the candidates in LDS for the exact path
#pragma unroll
    for (int q = 0; q < TF_PERT; ++q)
      if (o0 + q < m) cache[o0 + q] = c[q];
  }

  // ---- exact path without the level-2 histogram
  auto get = [&](int o) -> int2 {                // uncached access
    if (raw) return make_int2(o, biased_key(srow[o]));
    int lo = 0, hi = n_sub;                      // last sub-list s with pre[s] <= o
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= o) lo = mid; else hi = mid;
    }
    return cseg[(size_t)lo * TK_SUB + (o - pre[lo])];
  };
  auto fetch = [&](int o) -> int2 { return cached ? cache[o] : get(o); };
  for (int k = threadIdx.x; k < hpad_size<HIST1_BINS>(); k += TF_THREADS) h1[k] = 0;
  for (int k = threadIdx.x; k < hpad_size<HIST2_BINS>(); k += TF_THREADS) h2[k] = 0;
  if (threadIdx.x == 0) res[4] = 0;
  __syncthreads();

  // Level 1 (top 11 bits): the candidates are exactly the elements of bins
  // >= thr.x.  If that bin is a legal threshold -- fewer than k candidates
  // above it, counted here from the data -- level 1 is known; otherwise it is
  // derived from the candidates' own histogram.
  bool fast = th.z && !raw && th.x >= 0 && th.x < HIST1_BINS;
  if (fast) {
    int part = 0;
    for (int o = threadIdx.x; o < m; o += TF_THREADS) part += (fetch(o).y >> HIST2_BITS) > th.x;
    part = __builtin_amdgcn_readlane(wave_incl_add(part), 63);
    if (lane == 0 && part) atomicAdd(&res[4], part);
    __syncthreads();
    const int above_data = res[4];
    fast = above_data < g.k_eff;                 // uniform
    if (fast && threadIdx.x == 0) {
      res[0] = th.x;
      res[1] = g.k_eff - above_data;             // still needed from bin b1
      h1[hpad<HIST1_BINS>(th.x)] = m - above_data;   // candidates in bin b1
    }
  }
  if (!fast) {
    for (int o = threadIdx.x; o < m; o += TF_THREADS)
      atomicAdd(&h1[hpad<HIST1_BINS>(fetch(o).y >> HIST2_BITS)], 1);
    __syncthreads();
    if (wave == 0) {
      int above;
      const int bb = wave_threshold_bin<HIST1_BINS>(h1, g.k_eff, m, above);
      if (lane == 0) {
        res[0] = bb;
        res[1] = g.k_eff - above;
      }
    }
  }
  __syncthreads();
  const int b1 = res[0], need1 = res[1];
  // level 2 (low 10 bits) over the candidates of bin b1
  for (int o = threadIdx.x; o < m; o += TF_THREADS) {
    const int2 c = fetch(o);
    if ((c.y >> HIST2_BITS) == b1) atomicAdd(&h2[hpad<HIST2_BINS>(c.y & (HIST2_BINS - 1))], 1);
  }
  __syncthreads();
  if (wave == 0) {
    int above;
    const int b2 = wave_threshold_bin<HIST2_BINS>(h2, need1, h1[hpad<HIST1_BINS>(b1)], above);
    if (lane == 0) {
      res[2] = (b1 << HIST2_BITS) | b2;
      res[3] = need1 - above;                    // ties at T to take, lowest index first
    }
  }
  __syncthreads();
  const int T = res[2], need2 = res[3];

  // ordered emission: each thread owns 4 consecutive candidates per round,
  // one block scan of packed (greater-than, tie) counts per round
  int run_gt = 0, run_tie = 0;
  for (int base = 0; base < m; base += 4 * TF_THREADS) {
    const int e0 = base + 4 * threadIdx.x;
    int2 c[4];
    int gt = 0, tie = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = e0 + q < m ? fetch(e0 + q) : make_int2(0, -1);
      gt += c[q].y > T;
      tie += c[q].y == T;
    }
    const int packed = gt | (tie << 16);
    int tot;
    const int ex = block_incl_scan<TF_WAVES, true>(packed, sc_pre, tot) - packed;
    int gt_before = run_gt + (ex & 0xffff), tie_before = run_tie + (ex >> 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool is_gt = c[q].y > T, is_tie = c[q].y == T;
      const bool sel = is_gt || (is_tie && tie_before < need2);
      const int pos = gt_before + min(tie_before, need2);
      if (sel && pos < topk) out[pos] = c[q].x;
      gt_before += is_gt;
      tie_before += is_tie;
    }
    run_gt += tot & 0xffff;
    run_tie += tot >> 16;
  }
  for (int j = g.k_eff + threadIdx.x; j < topk; j += TF_THREADS) out[j] = -1;
}

}  // namespace

size_t hist_region_bytes(const Shape &s) {
  const size_t nseg = (size_t)s.B * s.R * s.Hkv;
  const size_t n_sub = (size_t)ceil_div(s.NB, TK_SUB);
  return align_up(nseg * HIST1_BINS * 4, 256) + align_up(nseg * HIST2_BINS * 4, 256) +
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
  char *p = base + hist_region_bytes(s);
  w.scratch = p;
  w.cnt = reinterpret_cast<int32_t *>(p);
  p += align_up(nseg * n_sub * 4, 256);
  w.cand = reinterpret_cast<int2 *>(p);
  w.nchunk = (int)n_sub;
  return w;
}

hipError_t launch_fill(int32_t *p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  fill_kernel<<<(int)std::min<size_t>(2048, (n + 255) / 256), 256, 0, st>>>(p, n, 0);
  return hipGetLastError();
}

hipError_t launch_topk(const int32_t *scores, const int32_t *seq_len, const Shape &s,
                       bool hist_ready, int32_t *idx, int32_t *n_sel, const TopkWs &w,
                       hipStream_t st) {
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
  topk_final_kernel<<<nseg, TF_THREADS, 0, st>>>(scores, seq_len, w.hist1, w.hist2, w.counters,
                                                 w.cnt, w.cand, w.nchunk, s.R, s.Hkv, s.T_max,
                                                 s.NB, s.window, s.pool, s.topk, idx, n_sel);
  return hipGetLastError();
}

}  // namespace sks
