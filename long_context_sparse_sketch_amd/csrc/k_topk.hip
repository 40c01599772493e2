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
//   filter: every workgroup derives the threshold bin b1 from the histogram;
//     each wave compacts the candidates (bin >= b1) of its 1024-token
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

// Largest bin b with sum_{b' >= b} hist[b'] >= need.  Writes b to res[0] and
// sum_{b' > b} hist[b'] to res[1]; (0, 0) if the total is below need.
__device__ void threshold_bin(const int *hist, int nbins, int need, int *scratch, int *res) {
  const int slice = nbins / blockDim.x;
  const int lo = threadIdx.x * slice;
  if (threadIdx.x == 0) {
    res[0] = 0;
    res[1] = 0;
  }
  int v = 0;
  for (int k = 0; k < slice; ++k) v += hist[lo + k];
  int tot;
  const int incl = block_incl_scan(v, scratch, tot);
  int above = tot - incl;
  if (above < need && above + v >= need) {
    for (int bb = lo + slice - 1; bb >= lo; --bb) {
      if (above + hist[bb] >= need) {
        res[0] = bb;
        res[1] = above;
        break;
      }
      above += hist[bb];
    }
  }
  __syncthreads();
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

__global__ __launch_bounds__(TK_THREADS) void topk_filter_kernel(
    const int32_t *__restrict__ scores, const int32_t *__restrict__ seq_len,
    const int32_t *__restrict__ hist1, int32_t *__restrict__ cnt, int2 *__restrict__ cand,
    int n_sub_max, int R, int Hkv, int T_max, int NB, int window, int pool, int topk) {
  __shared__ int sh[HIST1_BINS];
  __shared__ int scratch[TK_THREADS / 64];
  __shared__ int res[2];
  const int seg = blockIdx.y;
  const SegGeom g = seg_geom(seg, seq_len, R, Hkv, T_max, window, pool, topk);
  if (g.k_eff >= g.n_far) return;
  const int c0 = blockIdx.x * TK_CHUNK;
  if (c0 >= g.n_far) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = blockIdx.x * (TK_CHUNK / TK_SUB) + wave;
  const int s0 = sub * TK_SUB;
  const int s1 = min(g.n_far, s0 + TK_SUB);
  const int32_t *row = scores + (size_t)seg * NB;
  // issue this wave's score loads before waiting for the histogram
  int keys[FILTER_ITERS];
#pragma unroll
  for (int r = 0; r < FILTER_ITERS; ++r) {
    const int t = s0 + r * 64 + lane;
    keys[r] = t < s1 ? biased_key(row[t]) : -1;
  }
  const int32_t *gh = hist1 + (size_t)seg * HIST1_BINS;
  for (int k = threadIdx.x; k < HIST1_BINS; k += TK_THREADS) sh[k] = gh[k];
  __syncthreads();
  threshold_bin(sh, HIST1_BINS, g.k_eff, scratch, res);
  const int b1 = res[0];
  if (s0 >= g.n_far) return;
  int2 *dst = cand + ((size_t)seg * n_sub_max + sub) * TK_SUB;
  int n = 0;
#pragma unroll
  for (int r = 0; r < FILTER_ITERS; ++r) {
    const bool f = keys[r] >= 0 && (keys[r] >> HIST2_BITS) >= b1;
    const unsigned long long m = __ballot(f);
    if (f) dst[n + __popcll(m & ((1ull << lane) - 1ull))] = make_int2(s0 + r * 64 + lane, keys[r]);
    n += __popcll(m);
  }
  if (lane == 0) cnt[(size_t)seg * n_sub_max + sub] = n;
}

__global__ __launch_bounds__(TF_THREADS) void topk_final_kernel(
    const int32_t *__restrict__ scores, const int32_t *__restrict__ seq_len,
    int32_t *__restrict__ hist1, const int32_t *__restrict__ cnt, const int2 *__restrict__ cand,
    int n_sub_max, int R, int Hkv, int T_max, int NB, int window, int pool, int topk,
    int32_t *__restrict__ idx, int32_t *__restrict__ n_sel) {
  __shared__ int h[HIST1_BINS];
  __shared__ int pre[TK_MAX_SUBS + 1];
  __shared__ int2 cache[TF_CACHE];
  __shared__ int scratch[TF_THREADS / 64];
  __shared__ int res[2];
  const int seg = blockIdx.x;
  const SegGeom g = seg_geom(seg, seq_len, R, Hkv, T_max, window, pool, topk);
  int32_t *out = idx + (size_t)seg * topk;
  // the filter has run: the histogram has done its job and returns to zero
  int32_t *gh = hist1 + (size_t)seg * HIST1_BINS;
  for (int k = threadIdx.x; k < HIST1_BINS; k += TF_THREADS) gh[k] = 0;
  if (threadIdx.x == 0 && n_sel) n_sel[seg] = g.k_eff;
  if (g.k_eff >= g.n_far) {                      // every far entry is selected
    for (int j = threadIdx.x; j < topk; j += TF_THREADS) out[j] = j < g.n_far ? j : -1;
    return;
  }

  // candidate list: exclusive prefix over the sub-chunk counts
  const int n_sub = (g.n_far + TK_SUB - 1) / TK_SUB;
  const int32_t *gc = cnt + (size_t)seg * n_sub_max;
  int carry = 0;
  for (int base = 0; base < n_sub; base += TF_THREADS) {
    const int s = base + threadIdx.x;
    const int v = s < n_sub ? gc[s] : 0;
    int tot;
    const int incl = block_incl_scan(v, scratch, tot);
    if (s < n_sub) pre[s] = carry + incl - v;
    carry += tot;
  }
  if (threadIdx.x == 0) pre[n_sub] = carry;
  __syncthreads();
  // Fewer candidates than k means the histogram was not one of these scores
  // (the workspace was not zero at rest): select from the raw scores instead.
  const bool raw = carry < g.k_eff;
  const int m = raw ? g.n_far : carry;
  const int2 *cseg = cand + (size_t)seg * n_sub_max * TK_SUB;
  const int32_t *srow = scores + (size_t)seg * NB;
  auto get = [&](int o) -> int2 {
    if (raw) return make_int2(o, biased_key(srow[o]));
    int lo = 0, hi = n_sub;                      // last sub-chunk s with pre[s] <= o
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= o) lo = mid; else hi = mid;
    }
    return cseg[(size_t)lo * TK_SUB + (o - pre[lo])];
  };
  const bool cached = m <= TF_CACHE;
  if (cached)
    for (int o = threadIdx.x; o < m; o += TF_THREADS) cache[o] = get(o);
  __syncthreads();
  auto fetch = [&](int o) -> int2 { return cached ? cache[o] : get(o); };

  // level 1 over the candidates
  for (int k = threadIdx.x; k < HIST1_BINS; k += TF_THREADS) h[k] = 0;
  __syncthreads();
  for (int o = threadIdx.x; o < m; o += TF_THREADS) atomicAdd(&h[fetch(o).y >> HIST2_BITS], 1);
  __syncthreads();
  threshold_bin(h, HIST1_BINS, g.k_eff, scratch, res);
  const int b1 = res[0];
  const int need1 = g.k_eff - res[1];
  __syncthreads();
  // level 2: low 10 bits inside bin b1
  for (int k = threadIdx.x; k < HIST2_BINS; k += TF_THREADS) h[k] = 0;
  __syncthreads();
  for (int o = threadIdx.x; o < m; o += TF_THREADS) {
    const int2 c = fetch(o);
    if ((c.y >> HIST2_BITS) == b1) atomicAdd(&h[c.y & (HIST2_BINS - 1)], 1);
  }
  __syncthreads();
  threshold_bin(h, HIST2_BINS, need1, scratch, res);
  const int T = (b1 << HIST2_BITS) | res[0];
  const int need2 = need1 - res[1];              // ties at T to take, lowest index first

  // ordered emission: one scan of packed (greater-than, tie) counts per round
  int run_gt = 0, run_tie = 0;
  for (int base = 0; base < m; base += TF_THREADS) {
    const int o = base + threadIdx.x;
    int2 c = make_int2(0, -1);
    if (o < m) c = fetch(o);
    const int gt = (o < m && c.y > T) ? 1 : 0;
    const int tie = (o < m && c.y == T) ? 1 : 0;
    const int packed = gt | (tie << 16);
    int tot;
    const int ex = block_incl_scan(packed, scratch, tot) - packed;
    const int gt_before = run_gt + (ex & 0xffff), tie_before = run_tie + (ex >> 16);
    const int sel = gt | ((tie && tie_before < need2) ? 1 : 0);
    const int pos = gt_before + min(tie_before, need2);
    if (sel && pos < topk) out[pos] = c.x;
    run_gt += tot & 0xffff;
    run_tie += tot >> 16;
  }
  for (int j = g.k_eff + threadIdx.x; j < topk; j += TF_THREADS) out[j] = -1;
}

}  // namespace

size_t hist_region_bytes(const Shape &s) {
  const size_t nseg = (size_t)s.B * s.R * s.Hkv;
  return align_up(nseg * HIST1_BINS * 4, 256) + align_up(nseg * 4, 256);
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
  w.hist1 = reinterpret_cast<int32_t *>(base);
  w.counters = reinterpret_cast<int32_t *>(base + align_up(nseg * HIST1_BINS * 4, 256));
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
    topk_filter_kernel<<<grid, TK_THREADS, 0, st>>>(scores, seq_len, w.hist1, w.cnt, w.cand,
                                                    w.nchunk, s.R, s.Hkv, s.T_max, s.NB,
                                                    s.window, s.pool, s.topk);
  }
  topk_final_kernel<<<nseg, TF_THREADS, 0, st>>>(scores, seq_len, w.hist1, w.cnt, w.cand,
                                                 w.nchunk, s.R, s.Hkv, s.T_max, s.NB, s.window,
                                                 s.pool, s.topk, idx, n_sel);
  return hipGetLastError();
}

}  // namespace sks
