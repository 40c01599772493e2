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
//   threshold (one wave per segment): validates the histogram and derives the
//     threshold bin b1 (an invalid histogram makes every element a candidate).
//   filter: each wave compacts the candidates (bin >= b1) of its 1024-token
//     sub-chunk IN ORDER (ballot + popcount).
//   final (one workgroup per segment): caches the candidates in LDS and runs
//     an exact two-level radix select on them -- it never trusts the
//     histogram beyond the filter's pruning: if fewer than k candidates came
//     through (a histogram that was not zero at rest), it selects from the
//     raw scores instead.  One ordered pass then emits score > T plus the
//     lowest-index ties at T, ascending, without a sort.  It returns the
//     segment's histogram to zero.
#include "sks_internal.h"

namespace sks {
namespace {

constexpr int TK_THREADS = 256;
constexpr int TF_THREADS = 1024;
constexpr int TF_CACHE = 8192;                     // candidates cached in LDS
constexpr int FILTER_ITERS = TK_SUB / 64;          // 16 loads in flight per lane
static_assert(TK_CHUNK == TK_SUB * (TK_THREADS / 64), "one sub-chunk per wave");

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

// Inclusive block-wide prefix sum; `tot` receives the block total.
// `scratch` must hold blockDim.x / 64 ints.  Contains __syncthreads().
__device__ int block_incl_scan(int v, int *scratch, int &tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int n = __shfl_up(v, off);
    if (lane >= off) v += n;
  }
  if (lane == 63) scratch[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < nw ? scratch[lane] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int n = __shfl_up(w, off);
      if (lane >= off) w += n;
    }
    if (lane < nw) scratch[lane] = w;
  }
  __syncthreads();
  const int prefix = wave > 0 ? scratch[wave - 1] : 0;
  tot = scratch[nw - 1];
  __syncthreads();
  return v + prefix;
}

// Wave-level version over an LDS histogram of NBINS bins, no barriers: lane
// l owns bins [l * NBINS/64, (l+1) * NBINS/64).  The histogram is first validated (every
// bin in [0, n] and the total exactly n); an invalid one (a workspace that
// was not zero at rest) yields bin 0, i.e. every element is a candidate, so
// that all waves of all workgroups of a segment agree on the same threshold.
// Returns the threshold bin; `above` receives sum_{b' > b} hist[b'].
// LDS histograms are stored padded (see hpad) so that 64 lanes reading their
// contiguous bins hit distinct banks.
template <int NBINS>
__device__ __forceinline__ int hpad(int b) { return b + b / (NBINS / 64); }
template <int NBINS>
constexpr int hpad_size() { return NBINS + 64; }

// Same search over a padded LDS histogram of NBINS bins.  The histogram is
// validated first (every bin in [0, n], total exactly n); an invalid one (a
// workspace that was not zero at rest) yields bin 0, i.e. every element is a
// candidate, the same answer for every reader of the same histogram.
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
    int32_t *__restrict__ hist1, int R, int Hkv, int T_max, int NB, int window, int pool,
    int topk) {
  __shared__ int lh[HIST1_BINS];
  const int seg = blockIdx.y;
  const SegGeom g = seg_geom(seg, seq_len, R, Hkv, T_max, window, pool, topk);
  if (g.k_eff >= g.n_far) return;               // everything selected: no histogram needed
  const int c0 = blockIdx.x * TK_CHUNK;
  if (c0 >= g.n_far) return;
  const int c1 = min(g.n_far, c0 + TK_CHUNK);
  for (int k = threadIdx.x; k < HIST1_BINS; k += TK_THREADS) lh[k] = 0;
  __syncthreads();
  const int32_t *row = scores + (size_t)seg * NB;
  for (int t = c0 + threadIdx.x; t < c1; t += TK_THREADS)
    atomicAdd(&lh[biased_key(row[t]) >> HIST2_BITS], 1);
  __syncthreads();
  int32_t *gh = hist1 + (size_t)seg * HIST1_BINS;
  for (int k = threadIdx.x; k < HIST1_BINS; k += TK_THREADS)
    if (lh[k]) atomicAdd(&gh[k], lh[k]);
}

// One wave per segment: validate the level-1 histogram and store the
// threshold bin b1 once (0 when every element must be a candidate).  Lane l
// loads its 32 contiguous bins as 8 independent 16-byte loads.
__global__ __launch_bounds__(64) void topk_threshold_kernel(
    const int32_t *__restrict__ seq_len, const int32_t *__restrict__ hist1,
    int32_t *__restrict__ thr, int R, int Hkv, int T_max, int window, int pool, int topk) {
  constexpr int PER = HIST1_BINS / 64;
  const int seg = blockIdx.x, lane = threadIdx.x;
  const int4 *gh = reinterpret_cast<const int4 *>(hist1 + (size_t)seg * HIST1_BINS + lane * PER);
  int v[PER];
#pragma unroll
  for (int k = 0; k < PER / 4; ++k) {
    const int4 w = gh[k];
    v[4 * k] = w.x;
    v[4 * k + 1] = w.y;
    v[4 * k + 2] = w.z;
    v[4 * k + 3] = w.w;
  }
  const SegGeom g = seg_geom(seg, seq_len, R, Hkv, T_max, window, pool, topk);
  int b1 = 0, above = 0;
  bool valid = false;
  if (g.k_eff < g.n_far) b1 = wave_threshold_regs<PER>(v, g.k_eff, g.n_far, above, valid);
  if (lane == 0) reinterpret_cast<int4 *>(thr)[seg] = make_int4(b1, above, valid, 0);
}

__global__ __launch_bounds__(TK_THREADS) void topk_filter_kernel(
    const int32_t *__restrict__ scores, const int32_t *__restrict__ seq_len,
    const int32_t *__restrict__ thr, int32_t *__restrict__ cnt, int2 *__restrict__ cand,
    int n_sub_max, int R, int Hkv, int T_max, int NB, int window, int pool, int topk) {
  const int seg = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = blockIdx.x * (TK_CHUNK / TK_SUB) + wave;
  const int s0 = sub * TK_SUB;
  const int32_t *row = scores + (size_t)seg * NB;
  // Issue this wave's score loads before the length is known, all at once:
  // the index is clamped below NB (always in bounds) instead of branching
  // around the load, and entries past the far region are masked later.
  int raw[FILTER_ITERS];
#pragma unroll
  for (int r = 0; r < FILTER_ITERS; ++r) raw[r] = row[min(s0 + r * 64 + lane, NB - 1)];
  const int b1 = thr[4 * seg];
  const SegGeom g = seg_geom(seg, seq_len, R, Hkv, T_max, window, pool, topk);
  if (g.k_eff >= g.n_far || s0 >= g.n_far) return;   // uniform per wave
  const int s1 = min(g.n_far, s0 + TK_SUB);
  int2 *dst = cand + ((size_t)seg * n_sub_max + sub) * TK_SUB;
  int n = 0;
#pragma unroll
  for (int r = 0; r < FILTER_ITERS; ++r) {
    const int t = s0 + r * 64 + lane;
    const int key = biased_key(raw[r]);
    const bool f = t < s1 && (key >> HIST2_BITS) >= b1;
    const unsigned long long m = __ballot(f);
    if (f) dst[n + __popcll(m & ((1ull << lane) - 1ull))] = make_int2(t, key);
    n += __popcll(m);
  }
  if (lane == 0) cnt[(size_t)seg * n_sub_max + sub] = n;
}

__global__ __launch_bounds__(TF_THREADS) void topk_final_kernel(
    const int32_t *__restrict__ scores, const int32_t *__restrict__ seq_len,
    int32_t *__restrict__ hist1, const int32_t *__restrict__ thr, const int32_t *__restrict__ cnt,
    const int2 *__restrict__ cand, int n_sub_max, int R, int Hkv, int T_max, int NB, int window,
    int pool, int topk, int32_t *__restrict__ idx, int32_t *__restrict__ n_sel) {
  __shared__ int h1[hpad_size<HIST1_BINS>()];
  __shared__ int h2[hpad_size<HIST2_BINS>()];
  __shared__ int pre[TK_MAX_SUBS + 1];
  __shared__ int2 cache[TF_CACHE];
  __shared__ int scratch[TF_THREADS / 64];
  __shared__ int res[4];
  const int seg = blockIdx.x;
  const int32_t *gc = cnt + (size_t)seg * n_sub_max;
  // the first round of sub-list counts, loaded before the length is known
  int cv0 = threadIdx.x < n_sub_max ? gc[threadIdx.x] : 0;
  const int4 th = reinterpret_cast<const int4 *>(thr)[seg];   // (b1, above1, valid, -)
  for (int k = threadIdx.x; k < hpad_size<HIST1_BINS>(); k += TF_THREADS) h1[k] = 0;
  for (int k = threadIdx.x; k < hpad_size<HIST2_BINS>(); k += TF_THREADS) h2[k] = 0;
  const SegGeom g = seg_geom(seg, seq_len, R, Hkv, T_max, window, pool, topk);
  int32_t *out = idx + (size_t)seg * topk;
  // the filter has run: the segment's histogram returns to zero
  int32_t *gh = hist1 + (size_t)seg * HIST1_BINS;
  for (int k = threadIdx.x; k < HIST1_BINS; k += TF_THREADS) gh[k] = 0;
  if (threadIdx.x == 0 && n_sel) n_sel[seg] = g.k_eff;
  if (g.k_eff >= g.n_far) {                      // every far entry is selected
    for (int j = threadIdx.x; j < topk; j += TF_THREADS) out[j] = j < g.n_far ? j : -1;
    return;
  }

  // candidate list: exclusive prefix over the sub-list counts
  const int n_sub = (g.n_far + TK_SUB - 1) / TK_SUB;
  int carry = 0;
  for (int base = 0; base < n_sub; base += TF_THREADS) {
    const int sidx = base + threadIdx.x;
    const int v = sidx < n_sub ? (base == 0 ? cv0 : gc[sidx]) : 0;
    int tot;
    const int incl = block_incl_scan(v, scratch, tot);
    if (sidx < n_sub) pre[sidx] = carry + incl - v;
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
  auto get = [&](int o) -> int2 {
    if (raw) return make_int2(o, biased_key(srow[o]));
    int lo = 0, hi = n_sub;                      // last sub-list s with pre[s] <= o
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= o) lo = mid; else hi = mid;
    }
    return cseg[(size_t)lo * TK_SUB + (o - pre[lo])];
  };
  const bool cached = m <= TF_CACHE;
  if (cached) {
    // all lookups first, then all loads in flight together, then the stores
    constexpr int PERT = TF_CACHE / TF_THREADS;
    int2 tmp[PERT];
#pragma unroll
    for (int k = 0; k < PERT; ++k) tmp[k] = get(min(threadIdx.x + k * TF_THREADS, m - 1));
#pragma unroll
    for (int k = 0; k < PERT; ++k) {
      const int o = threadIdx.x + k * TF_THREADS;
      if (o < m) cache[o] = tmp[k];
    }
  }
  __syncthreads();
  auto fetch = [&](int o) -> int2 { return cached ? cache[o] : get(o); };

  // exact threshold key T: level 1 (top 11 bits), level 2 (low 10 bits).
  // With a valid histogram the candidates are exactly the elements of bins
  // >= b1 and level 1 is already known; otherwise derive it from the
  // candidates themselves.
  // Candidates are exactly the elements of bins >= thr.x (the filter used the
  // same value).  If that bin is a legal threshold -- the candidates above it
  // number fewer than k, counted from the data, never from the histogram --
  // level 1 is known; otherwise derive it from the candidates.
  bool fast = th.z && !raw && th.x >= 0 && th.x < HIST1_BINS;
  int above_data = 0;
  if (fast) {
    int part = 0;
    for (int o = threadIdx.x; o < m; o += TF_THREADS) part += (fetch(o).y >> HIST2_BITS) > th.x;
    block_incl_scan(part, scratch, above_data);
    fast = above_data < g.k_eff;                 // uniform: block total
  }
  if (fast) {
    if (threadIdx.x == 0) {
      res[0] = th.x;
      res[1] = g.k_eff - above_data;
      h1[hpad<HIST1_BINS>(th.x)] = m - above_data;   // candidates in bin b1
    }
  } else {
    for (int o = threadIdx.x; o < m; o += TF_THREADS)
      atomicAdd(&h1[hpad<HIST1_BINS>(fetch(o).y >> HIST2_BITS)], 1);
    __syncthreads();
    if (threadIdx.x < 64) {
      int above;
      const int bb = wave_threshold_bin<HIST1_BINS>(h1, g.k_eff, m, above);
      if (threadIdx.x == 0) {
        res[0] = bb;
        res[1] = g.k_eff - above;                // still needed from bin b1
      }
    }
  }
  __syncthreads();
  const int b1 = res[0], need1 = res[1];
  for (int o = threadIdx.x; o < m; o += TF_THREADS) {
    const int2 c = fetch(o);
    if ((c.y >> HIST2_BITS) == b1) atomicAdd(&h2[hpad<HIST2_BINS>(c.y & (HIST2_BINS - 1))], 1);
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    int above;
    const int b2 = wave_threshold_bin<HIST2_BINS>(h2, need1, h1[hpad<HIST1_BINS>(b1)], above);
    if (threadIdx.x == 0) {
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
    const int o0 = base + 4 * threadIdx.x;
    int2 c[4];
    int gt = 0, tie = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = o0 + q < m ? fetch(o0 + q) : make_int2(0, -1);
      gt += c[q].y > T;
      tie += c[q].y == T;
    }
    const int packed = gt | (tie << 16);
    int tot;
    const int ex = block_incl_scan(packed, scratch, tot) - packed;
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
  return align_up(nseg * HIST1_BINS * 4, 256) + align_up(nseg * 16, 256);
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
  TopkWs w;
  char *q = base;
  w.hist1 = reinterpret_cast<int32_t *>(q);
  q += align_up(nseg * HIST1_BINS * 4, 256);
  w.counters = reinterpret_cast<int32_t *>(q);
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
      topk_hist_kernel<<<grid, TK_THREADS, 0, st>>>(scores, seq_len, w.hist1, s.R, s.Hkv,
                                                    s.T_max, s.NB, s.window, s.pool, s.topk);
    topk_threshold_kernel<<<nseg, 64, 0, st>>>(seq_len, w.hist1, w.counters, s.R, s.Hkv,
                                               s.T_max, s.window, s.pool, s.topk);
    topk_filter_kernel<<<grid, TK_THREADS, 0, st>>>(scores, seq_len, w.counters, w.cnt, w.cand,
                                                    w.nchunk, s.R, s.Hkv, s.T_max, s.NB,
                                                    s.window, s.pool, s.topk);
  }
  topk_final_kernel<<<nseg, TF_THREADS, 0, st>>>(scores, seq_len, w.hist1, w.counters, w.cnt,
                                                 w.cand, w.nchunk, s.R, s.Hkv, s.T_max, s.NB,
                                                 s.window, s.pool, s.topk, idx, n_sel);
  return hipGetLastError();
}

}  // namespace sks
