// Deterministic top-k selection over int32 sketch scores ("What it took" on
// the page "8 agents x 250K context, concurrently, on two 3090s": pick the
// top ~2K).  For every segment (b, i, h) it returns the k_eff far entries with
// the largest score, lower index first among equal scores, in ascending index
// order, padded with -1.
//
// Scores fit in 21 bits once biased by 2^20 (|score| <= 64*127^2).  Radix
// select on that key:
//   1. hist:   2048-bin histogram of the top 11 bits (LDS, then integer
//              atomics into global memory: order-independent, deterministic).
//   2. filter: every workgroup finds the threshold bin b1 from the histogram
//              and each wave compacts the candidates (bin >= b1) of its own
//              1024-token sub-chunk IN ORDER (ballot + popcount), so the
//              candidate list is index-ordered sub-chunk by sub-chunk.
//   3. final:  one workgroup per segment: exact threshold T from a second
//              1024-bin histogram over the low 10 bits of the boundary bin,
//              then one ordered pass emitting score > T, plus the first
//              (lowest-index) ties at T up to k.  Ordered block scans make the
//              output ascending without any sort.
#include "sks_internal.h"

namespace sks {
namespace {

constexpr int TK_THREADS = 256;
constexpr int TF_THREADS = 1024;
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

__device__ __forceinline__ int biased_key(int s) {
  int v = s + SCORE_BIAS;
  return v < 0 ? 0 : (v > (1 << 21) - 1 ? (1 << 21) - 1 : v);
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

// Largest bin b with sum_{b' >= b} hist[b'] >= need (requires total >= need).
// Writes b to res[0] and sum_{b' > b} hist[b'] to res[1].
__device__ void threshold_bin(const int *hist, int nbins, int need, int *scratch, int *res) {
  const int slice = nbins / blockDim.x;
  const int lo = threadIdx.x * slice;
  if (threadIdx.x == 0) {                        // defined result even if total < need
    res[0] = 0;
    res[1] = 0;
  }
  int v = 0;
  for (int k = 0; k < slice; ++k) v += hist[lo + k];
  int tot;
  const int incl = block_incl_scan(v, scratch, tot);
  int above = tot - incl;                        // bins of higher-numbered slices
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
  if (g.k_eff >= g.n_far) return;               // everything selected: no histogram
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
  const int32_t *gh = hist1 + (size_t)seg * HIST1_BINS;
  for (int k = threadIdx.x; k < HIST1_BINS; k += TK_THREADS) sh[k] = gh[k];
  __syncthreads();
  threshold_bin(sh, HIST1_BINS, g.k_eff, scratch, res);
  const int b1 = res[0];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = blockIdx.x * (TK_CHUNK / TK_SUB) + wave;
  const int s0 = sub * TK_SUB;
  if (s0 >= g.n_far) return;
  const int s1 = min(g.n_far, s0 + TK_SUB);
  const int32_t *row = scores + (size_t)seg * NB;
  int2 *dst = cand + ((size_t)seg * n_sub_max + sub) * TK_SUB;
  int n = 0;
  for (int t0 = s0; t0 < s1; t0 += 64) {
    const int t = t0 + lane;
    int key = 0;
    bool f = false;
    if (t < s1) {
      key = biased_key(row[t]);
      f = (key >> HIST2_BITS) >= b1;
    }
    const unsigned long long m = __ballot(f);
    if (f) {
      const int pos = n + __popcll(m & ((1ull << lane) - 1ull));
      dst[pos] = make_int2(t, key);
    }
    n += __popcll(m);
  }
  if (lane == 0) cnt[(size_t)seg * n_sub_max + sub] = n;
}

__global__ __launch_bounds__(TF_THREADS) void topk_final_kernel(
    const int32_t *__restrict__ seq_len, const int32_t *__restrict__ hist1,
    const int32_t *__restrict__ cnt, const int2 *__restrict__ cand, int n_sub_max, int R, int Hkv,
    int T_max, int window, int pool, int topk, int32_t *__restrict__ idx,
    int32_t *__restrict__ n_sel) {
  __shared__ int h[HIST1_BINS];
  __shared__ int pre[TK_MAX_SUBS + 1];
  __shared__ int scratch[TF_THREADS / 64];
  __shared__ int res[2];
  const int seg = blockIdx.x;
  const SegGeom g = seg_geom(seg, seq_len, R, Hkv, T_max, window, pool, topk);
  int32_t *out = idx + (size_t)seg * topk;
  if (threadIdx.x == 0 && n_sel) n_sel[seg] = g.k_eff;
  if (g.k_eff >= g.n_far) {                      // every far entry is selected
    for (int j = threadIdx.x; j < topk; j += TF_THREADS) out[j] = j < g.n_far ? j : -1;
    return;
  }
  // level 1: threshold bin and how many must come from it
  const int32_t *gh = hist1 + (size_t)seg * HIST1_BINS;
  for (int k = threadIdx.x; k < HIST1_BINS; k += TF_THREADS) h[k] = gh[k];
  __syncthreads();
  threshold_bin(h, HIST1_BINS, g.k_eff, scratch, res);
  const int b1 = res[0];
  const int need1 = g.k_eff - res[1];
  const int cnt_b1 = h[b1];
  __syncthreads();

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
  const int m = carry;
  const int2 *cseg = cand + (size_t)seg * n_sub_max * TK_SUB;
  // ordinal -> candidate: last sub-chunk s with pre[s] <= o
  auto locate = [&](int o) -> int2 {
    int lo = 0, hi = n_sub;                      // pre[lo] <= o < pre[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= o) lo = mid; else hi = mid;
    }
    return cseg[(size_t)lo * TK_SUB + (o - pre[lo])];
  };

  // level 2: exact threshold key T and the number of ties at T to take
  int T = b1 << HIST2_BITS;
  int need2 = 0x7fffffff;
  if (need1 < cnt_b1) {
    for (int k = threadIdx.x; k < HIST2_BINS; k += TF_THREADS) h[k] = 0;
    __syncthreads();
    for (int o = threadIdx.x; o < m; o += TF_THREADS) {
      const int2 c = locate(o);
      if ((c.y >> HIST2_BITS) == b1) atomicAdd(&h[c.y & (HIST2_BINS - 1)], 1);
    }
    __syncthreads();
    threshold_bin(h, HIST2_BINS, need1, scratch, res);
    T |= res[0];
    need2 = need1 - res[1];
  }

  // ordered emission
  int run_sel = 0, run_tie = 0;
  for (int base = 0; base < m; base += TF_THREADS) {
    const int o = base + threadIdx.x;
    int2 c = make_int2(0, -1);
    if (o < m) c = locate(o);
    const int tie = (o < m && c.y == T) ? 1 : 0;
    int tie_tot;
    const int tie_rank = run_tie + block_incl_scan(tie, scratch, tie_tot) - tie;
    const int sel = (o < m) && (c.y > T || (tie && tie_rank < need2)) ? 1 : 0;
    int sel_tot;
    const int pos = run_sel + block_incl_scan(sel, scratch, sel_tot) - sel;
    if (sel && pos < topk) out[pos] = c.x;
    run_tie += tie_tot;
    run_sel += sel_tot;
  }
  for (int j = g.k_eff + threadIdx.x; j < topk; j += TF_THREADS) out[j] = -1;
}

}  // namespace

size_t topk_ws_bytes(const Shape &s) {
  const size_t nseg = (size_t)s.B * s.R * s.Hkv;
  const size_t n_sub = (size_t)ceil_div(s.NB, TK_SUB);
  return align_up(nseg * HIST1_BINS * 4, 256) + align_up(nseg * n_sub * 4, 256) +
         align_up(nseg * n_sub * TK_SUB * sizeof(int2), 256);
}

TopkWs topk_ws_carve(const Shape &s, void *ws) {
  const size_t nseg = (size_t)s.B * s.R * s.Hkv;
  const size_t n_sub = (size_t)ceil_div(s.NB, TK_SUB);
  char *p = static_cast<char *>(ws);
  TopkWs w;
  w.hist1 = reinterpret_cast<int32_t *>(p);
  p += align_up(nseg * HIST1_BINS * 4, 256);
  w.cnt = reinterpret_cast<int32_t *>(p);
  p += align_up(nseg * n_sub * 4, 256);
  w.cand = reinterpret_cast<int2 *>(p);
  w.nchunk = (int)n_sub;                        // sub-chunks per segment
  return w;
}

hipError_t launch_topk(const int32_t *scores, const int32_t *seq_len, const Shape &s,
                       int32_t *idx, int32_t *n_sel, const TopkWs &w, hipStream_t st) {
  const int nseg = s.B * s.R * s.Hkv;
  const size_t nh = (size_t)nseg * HIST1_BINS;
  fill_kernel<<<(int)std::min<size_t>(1024, (nh + 255) / 256), 256, 0, st>>>(w.hist1, nh, 0);
  long max_far = s.T_max > s.window ? (long)(s.T_max - s.window) / s.pool : 0;
  if (max_far > 0) {
    dim3 grid(ceil_div(max_far, TK_CHUNK), nseg);
    topk_hist_kernel<<<grid, TK_THREADS, 0, st>>>(scores, seq_len, w.hist1, s.R, s.Hkv, s.T_max,
                                                  s.NB, s.window, s.pool, s.topk);
    topk_filter_kernel<<<grid, TK_THREADS, 0, st>>>(scores, seq_len, w.hist1, w.cnt, w.cand,
                                                    w.nchunk, s.R, s.Hkv, s.T_max, s.NB,
                                                    s.window, s.pool, s.topk);
  }
  topk_final_kernel<<<nseg, TF_THREADS, 0, st>>>(seq_len, w.hist1, w.cnt, w.cand, w.nchunk, s.R,
                                                 s.Hkv, s.T_max, s.window, s.pool, s.topk, idx,
                                                 n_sel);
  return hipGetLastError();
}

}  // namespace sks
