// Device code of the exact top-k selection: the helpers shared by its
// kernels, and the final pass as a template on the workgroup size and the
// candidate capacity.  (Selection algorithm: see k_topk.hip.)
#pragma once

#include "sks_internal.h"

namespace sks {
namespace {

constexpr int TK_THREADS = 256;
constexpr int TF_REGS = 8192;                      // candidates a final workgroup holds in registers
constexpr int TF_CACHE = 8192;                     // ... and in LDS for its exact path
constexpr int FILTER_ITERS = TK_SUB / 64;          // 16 loads in flight per lane
constexpr int HIST2_DIRECT_MAX = 4096;             // level-2 histogram built when bin b1 is this small
static_assert(TK_CHUNK == TK_SUB * (TK_THREADS / 64), "one sub-chunk per wave");
static_assert(TF_REGS < 65536 && TF_CACHE <= TF_REGS, "packed 16-bit counts in the emission scan");
// A sub-list start mark packs (sub-list + 1) << MK_SHIFT | start slot: marks
// increase with the slot, and the running maximum gives both at once.
constexpr int MK_SHIFT = 13;
static_assert(TF_REGS <= (1 << MK_SHIFT) && TK_MAX_SUBS < (1 << (30 - MK_SHIFT)), "packed marks");

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

// As wave_threshold_bin, also reporting whether the histogram's total was n.
template <int NBINS>
__device__ int wave_threshold_bin_valid(const int *hist, int need, int n, int &above, bool &valid) {
  constexpr int PER = NBINS / 64;
  const int lane = threadIdx.x & 63;
  int v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) v[k] = hist[hpad<NBINS>(lane * PER + k)];
  return wave_threshold_regs<PER>(v, need, n, above, valid);
}

// Threshold search by all NW waves of the workgroup over a padded LDS
// histogram of HIST1_BINS bins, wave w taking bins [w B, (w + 1) B), two per
// lane: the bin b holding the need-th largest of n counted keys.  Writes
// res[0] = b (-1: none, or the histogram's total is not n), res[1] = need
// minus the count above b, res[2] = the count in b.  `scratch` holds NW ints.
// Contains two __syncthreads().
template <int NW>
__device__ void block_threshold_pair(int v0, int v1, int need, int n, int *scratch, int *res);
template <int NW>
__device__ void block_threshold_bin(const int *hist, int need, int n, int *scratch, int *res) {
  const int b0 = 2 * (int)threadIdx.x;
  block_threshold_pair<NW>(hist[hpad<HIST1_BINS>(b0)], hist[hpad<HIST1_BINS>(b0 + 1)], need, n,
                           scratch, res);
}
// The same search with the lane's two bins (b0 = 2 threadIdx.x and b0 + 1)
// given as values.
template <int NW>
__device__ void block_threshold_pair(int v0, int v1, int need, int n, int *scratch, int *res) {
  constexpr int B = HIST1_BINS / NW;
  static_assert(B == 128, "two bins per lane");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b0 = wave * B + 2 * lane;            // this lane's bins b0 (lower), b0 + 1
  const bool bad = __ballot(v0 < 0 || v1 < 0 || v0 > n || v1 > n) != 0;
  const int sum = min(v0 + v1, n + 1);
  const int incl = wave_incl_add_sat(sum, n + 1);
  const int wtot = __builtin_amdgcn_readlane(incl, 63);
  if (lane == 63) scratch[wave] = bad ? n + 1 : wtot;
  if (threadIdx.x == 0) res[0] = -1;
  __syncthreads();
  int above = 0, tot = 0;                        // keys in the waves above, and in all
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = scratch[w];
    above = min(above + (w > wave ? t : 0), n + 1);
    tot = min(tot + t, n + 1);
  }
  above = min(above + (wtot - incl), n + 1);     // ... and in the lanes above this one
  if (tot == n) {
    if (above < need && above + v1 >= need) {
      res[0] = b0 + 1;
      res[1] = need - above;
      res[2] = v1;
    } else if (above + v1 < need && above + v1 + v0 >= need) {
      res[0] = b0;
      res[1] = need - above - v1;
      res[2] = v0;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------- sample pass
// Candidate mode's sample: sampled rows j * stride of a segment's far region,
// j in [j0, j0 + SAMPLE_WG_ROWS), scored against the segment's query code,
// their level-1 bins counted in an LDS histogram and then added to the
// segment's sample histogram (zero at rest), or (one workgroup per segment)
// turned into the segment's estimate at once.  A quad of lanes per sampled
// sketch row, 16 bytes each, SAMPLE_UNROLL rows per quad in flight.
constexpr int SAMPLE_THREADS = 256;
constexpr int SAMPLE_UNROLL = 8;
constexpr int SAMPLE_WG_ROWS = SAMPLE_THREADS / 4 * SAMPLE_UNROLL;   // 512 sampled rows

// Loads of this thread's sampled rows j * stride, j < m (issued before
// anything uses them); m, the cache's sampled rows, is at least 1 (a cache
// holds at least one sketch row).  The loads are unconditional, rows past m
// reading row (m - 1) * stride instead (sample_bins masks them): a load under
// a per-lane condition, or one of two definitions of sv, becomes a branch at
// whose join the compiler waits for the loads before it.
__device__ __forceinline__ void sample_load(const int8_t *__restrict__ S, size_t seg_row0, int j0,
                                            int m, int stride, int4 (&sv)[SAMPLE_UNROLL]) {
  const int part = threadIdx.x & 3, quad = threadIdx.x >> 2;
  constexpr int QUADS = SAMPLE_THREADS / 4;
  const int4 *Sseg = reinterpret_cast<const int4 *>(S + seg_row0 * RANK) + part;
  const int last = max(m - 1, 0);
#pragma unroll
  for (int u = 0; u < SAMPLE_UNROLL; ++u) {
    const int j = min(j0 + u * QUADS + quad, last);
    sv[u] = Sseg[(size_t)j * stride * 4];
  }
}

// Their scores' level-1 bins into lh (this thread's 16 bytes of the query
// code: qv); keys[u] receives the biased key of the thread's row u (lane 0 of
// each quad only; -1 for the other lanes and for rows past m).
__device__ __forceinline__ void sample_bins(const int4 (&sv)[SAMPLE_UNROLL], int4 qv, int j0, int m,
                                            int *lh, int (&keys)[SAMPLE_UNROLL]) {
  const int part = threadIdx.x & 3, quad = threadIdx.x >> 2;
  constexpr int QUADS = SAMPLE_THREADS / 4;
#pragma unroll
  for (int u = 0; u < SAMPLE_UNROLL; ++u) {
    int acc = __builtin_amdgcn_sdot4(sv[u].x, qv.x, 0, false);
    acc = __builtin_amdgcn_sdot4(sv[u].y, qv.y, acc, false);
    acc = __builtin_amdgcn_sdot4(sv[u].z, qv.z, acc, false);
    acc = __builtin_amdgcn_sdot4(sv[u].w, qv.w, acc, false);
    acc = quad_sum_i(acc);
    const int j = j0 + u * QUADS + quad;
    keys[u] = part == 0 && j < m ? biased_key(acc) : -1;
    if (keys[u] >= 0) atomicAdd(&lh[keys[u] >> HIST2_BITS], 1);
  }
}

// LDS of a sample workgroup that derives its segment's estimate itself.
struct SampleEstLds {
  int h2[HIST2_BINS];
  int escan[SAMPLE_THREADS / 64];
  int e, rank, pos;
};

// A segment's estimate E from its whole sample, held by one workgroup: the
// level-1 histogram lh (complete) and the sampled keys (sample_bins).  E is
// the rho-th largest sampled key itself (block_estimate's rule without its
// rounding down to the lower edge of that key's level-1 bin): block_estimate
// finds the bin and the key's rank in it, and a level-2 histogram of the low
// bits of the bin's sampled keys finds the key.  L.h2 must be zero on entry.
// Returns E in every thread.
__device__ int sample_estimate(const int *lh, const int (&keys)[SAMPLE_UNROLL], int n_far,
                               int k_eff, int stride, SampleEstLds &L) {
  int hv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) hv[k] = lh[HIST1_BINS - 1 - 8 * (int)threadIdx.x - k];
  block_estimate<SAMPLE_THREADS>(hv, n_far, k_eff, stride, 0, L.escan, &L.e, &L.rank);
  const int e1 = L.e, rank = L.rank;
  if (rank <= 0) return e1;                      // uniform: no sampled key to refine to
  const int b1 = e1 >> HIST2_BITS;
#pragma unroll
  for (int u = 0; u < SAMPLE_UNROLL; ++u)
    if (keys[u] >= 0 && (keys[u] >> HIST2_BITS) == b1) atomicAdd(&L.h2[keys[u] & (HIST2_BINS - 1)], 1);
  __syncthreads();
  constexpr int PER2 = HIST2_BINS / SAMPLE_THREADS;
  int v[PER2];
#pragma unroll
  for (int k = 0; k < PER2; ++k) v[k] = L.h2[HIST2_BINS - 1 - PER2 * (int)threadIdx.x - k];
  block_top_rank<SAMPLE_THREADS, PER2>(v, rank, L.escan, &L.pos);
  const int pos = L.pos;
  // (the bin holds at least `rank` sampled keys, so pos >= 0)
  return pos >= 0 ? e1 | (HIST2_BINS - 1 - pos) : e1;
}

__device__ __forceinline__ void sample_flush(const int *lh, int32_t *__restrict__ hsamp_seg) {
  for (int k = threadIdx.x; k < HIST1_BINS; k += SAMPLE_THREADS)
    if (lh[k]) atomicAdd(&hsamp_seg[k], lh[k]);
}

// Arguments of the final select pass.
struct FinalArgs {
  const int32_t *scores, *seq_len;
  int32_t *hist1, *hist2;
  const int32_t *thr, *cnt;
  const int2 *cand;
  int n_sub_max, R, Hkv, T_max, NB, window, pool, topk;
  int32_t *idx, *n_sel;
  int skip;      // no filter ran: every far entry is a candidate (n_far <= TF_REGS)
  int h1_ready;  // (with skip) the score pass built this step's level-1 histogram
  // Candidate mode: the score pass wrote the candidate lists (every far entry
  // at or above the segment's estimate) and the level-1 histogram, and no
  // scores.  A segment with fewer than k candidates is rescored from qsk and
  // S into `rescore` (the scores buffer) and selected from there.
  int cand_mode;
  int32_t *hsamp;   // candidate mode: the sample histograms, returned to zero here
  int zero_hsamp;   // ... unless 0: then a later launch of the step clears them
  const int8_t *qsk, *S;
  int32_t *rescore;
};

// LDS of the final pass for NT threads, segments of up to MAXSUB sub-lists,
// and (LDS_CACHE) the candidates cached for the exact fallback path.
template <int NT, int MAXSUB, bool LDS_CACHE>
struct FinalLds {
  int h1[hpad_size<HIST1_BINS>()];
  int h2[hpad_size<HIST2_BINS>()];
  int pre[MAXSUB + 1];
  union {
    // sub-list start marks (packed, see MK_SHIFT), one int per candidate
    // slot; read only before the candidates reach the registers
    int marks[TF_REGS];
    // the candidates for the exact path, written only after that
    int2 cache[LDS_CACHE ? TF_CACHE : 1];
  };
  int sc_pre[NT / 64], sc_own[NT / 64], sc_cnt[NT / 64];
  int res[6];
};

// The arguments of FinalArgs that the pass reads first, passed to the kernel
// as scalar arguments ahead of the struct so that they arrive preloaded in
// SGPRs and the first loads need not wait for the argument fetch.
struct FinalLead {
  const int32_t *cnt, *thr, *seq_len;
  int32_t *hist1, *hist2;
  int n_sub_max, R, Hkv;
};

// The final select pass of one segment by a workgroup of NT threads.
template <int NT, int MAXSUB, bool LDS_CACHE>
__device__ void final_body(const FinalArgs &a, const FinalLead &ld, int seg,
                           FinalLds<NT, MAXSUB, LDS_CACHE> &L) {
  constexpr int TF_THREADS = NT;
  constexpr int TF_WAVES = NT / 64;
  constexpr int TF_PERT = TF_REGS / NT;
  static_assert(TF_PERT * NT == TF_REGS, "slots per thread");
  const int32_t *scores = a.scores;           // written by this pass when rescoring
  const int32_t *__restrict__ seq_len = ld.seq_len;
  int32_t *__restrict__ hist1 = ld.hist1;
  int32_t *__restrict__ hist2 = ld.hist2;
  const int32_t *__restrict__ thr = ld.thr;
  const int32_t *__restrict__ cnt = ld.cnt;
  const int2 *__restrict__ cand = a.cand;
  const int n_sub_max = ld.n_sub_max, R = ld.R, Hkv = ld.Hkv, T_max = a.T_max, NB = a.NB,
            window = a.window, pool = a.pool, topk = a.topk;
  int32_t *__restrict__ idx = a.idx;
  int32_t *__restrict__ n_sel = a.n_sel;
  int *h1 = L.h1, *h2 = L.h2, *pre = L.pre, *marks = L.marks, *res = L.res;
  int2 *cache = L.cache;
  int *sc_pre = L.sc_pre, *sc_own = L.sc_own, *sc_cnt = L.sc_cnt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t *gc = cnt + (size_t)seg * n_sub_max;
  int32_t *gh2 = hist2 + (size_t)seg * HIST2_BINS;
  // loads first: every wave the first WL_SUBS sub-list counts (lane l those
  // of sub-lists 4l .. 4l + 3), the threshold record and (wave 0) the
  // level-2 histogram, lane l holding bins [16l, 16l+16)
  constexpr int WL_SUBS = 4 * 64;
  int cv[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) cv[u] = 4 * lane + u < n_sub_max ? gc[4 * lane + u] : 0;
  const int4 th = reinterpret_cast<const int4 *>(thr)[seg];   // (b1, above b1, valid, in b1)
  constexpr int H2_PER = HIST2_BINS / 64;
  const bool skip = a.skip, cmode = a.cand_mode;   // uniform
  // the score pass built this step's level-1 histogram
  const bool h1_ready = skip && a.h1_ready;
  int32_t *gh1 = hist1 + (size_t)seg * HIST1_BINS;
  static_assert(HIST1_BINS == 2 * TF_THREADS, "two level-1 bins per thread");
  int hv[H2_PER];
  int2 h1p = make_int2(0, 0);
  if (h1_ready) {
    // the score pass's level-1 histogram of this segment, thread t holding
    // bins 2t, 2t + 1; the same threads return them to zero afterwards
    h1p = reinterpret_cast<const int2 *>(gh1)[threadIdx.x];
#pragma unroll
    for (int k = 0; k < H2_PER; ++k) hv[k] = 0;
  } else if (wave == 0 && !cmode) {
#pragma unroll
    for (int k = 0; k < H2_PER / 4; ++k) {
      const int4 w = reinterpret_cast<const int4 *>(gh2 + lane * H2_PER)[k];
      hv[4 * k] = w.x;
      hv[4 * k + 1] = w.y;
      hv[4 * k + 2] = w.z;
      hv[4 * k + 3] = w.w;
    }
  }
  // candidate mode: the candidates' histogram, built in LDS, and the
  // estimate the candidates were kept with, from the segment's record
  // (clamped as the score pass clamps it)
  const int e_cand = cmode ? max(th.x, 0) : 0;
  if (cmode)
    for (int k = threadIdx.x; k < hpad_size<HIST1_BINS>(); k += TF_THREADS) h1[k] = 0;
  const SegGeom g = seg_geom(seg, seq_len, R, Hkv, T_max, window, pool, topk);
  int32_t *out = idx + (size_t)seg * topk;
  // The segment's histograms return to zero, and n_sel is written, on every
  // way out.  These stores come last: a wave that waits for its loads waits
  // for its earlier stores too, so stores issued here first would delay
  // every load that follows them.
  // (Candidate mode writes neither histogram: a dirty one is left as it is,
  // which costs a later storing selection time, never correctness.)
  auto finish = [&]() {
    if (h1_ready) {
      reinterpret_cast<int2 *>(gh1)[threadIdx.x] = make_int2(0, 0);   // the threads that read it
    } else if (!cmode) {
      for (int k = threadIdx.x; k < HIST1_BINS; k += TF_THREADS) gh1[k] = 0;
    }
    if (wave == 0 && !cmode) {
#pragma unroll
      for (int k = 0; k < H2_PER / 4; ++k)
        reinterpret_cast<int4 *>(gh2 + lane * H2_PER)[k] = make_int4(0, 0, 0, 0);
    }
    if (cmode && a.zero_hsamp)
      for (int k = threadIdx.x; k < HIST1_BINS; k += TF_THREADS) a.hsamp[(size_t)seg * HIST1_BINS + k] = 0;
    if (threadIdx.x == 0 && n_sel) n_sel[seg] = g.k_eff;
  };

  // wave 0: the threshold guess T from the level-2 histogram (-1: none)
  if (wave == 0) {
    int T = -1;
    if (!skip && !cmode && g.k_eff < g.n_far && th.z && th.w >= 0 && th.w <= HIST2_DIRECT_MAX &&
        th.x >= 0 && th.x < HIST1_BINS) {
      int above;
      bool valid;
      const int b2 = wave_threshold_regs<H2_PER>(hv, g.k_eff - th.y, th.w, above, valid);
      if (valid) T = (th.x << HIST2_BITS) | b2;
    }
    if (lane == 0) res[5] = T;
  }
  if (g.k_eff >= g.n_far) {                      // every far entry is selected
    for (int j = threadIdx.x; j < topk; j += TF_THREADS) out[j] = j < g.n_far ? j : -1;
    finish();
    return;
  }

  // Candidate list: sub-list s starts at slot pre[s], the exclusive prefix of
  // the counts (without a filter pass the candidates are the far entries
  // themselves).  Up to WL_SUBS sub-lists every wave computes the prefix from
  // its own registers and writes the (same) pre[] values, which it then reads
  // back itself: no workgroup barrier.  Beyond, a block-wide scan in rounds.
  const int n_sub = (g.n_far + TK_SUB - 1) / TK_SUB;
  const bool wave_local = !skip && n_sub <= WL_SUBS;   // uniform
  int carry = 0;
  int st[4];                                     // wave-local: starts of sub-lists 4 lane + u
  if (wave_local) {
    int sum = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      cv[u] = 4 * lane + u < n_sub ? cv[u] : 0;
      st[u] = sum;
      sum += cv[u];
    }
    const int incl = wave_incl_add(sum);
    carry = __builtin_amdgcn_readlane(incl, 63);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      st[u] += incl - sum;
      if (4 * lane + u < n_sub) pre[4 * lane + u] = st[u];
    }
    if (lane == 0) pre[n_sub] = carry;
  } else {
    // every non-empty sub-list marks its first slot
#pragma unroll
    for (int q = 0; q < TF_PERT; ++q) marks[q * TF_THREADS + threadIdx.x] = 0;   // no mark
    for (int base = 0; base < (skip ? 0 : n_sub); base += TF_THREADS) {
      const int sidx = base + threadIdx.x;
      const int v = sidx < n_sub ? gc[sidx] : 0;
      int tot;
      const int incl = block_incl_scan<TF_WAVES, true>(v, sc_pre, tot);
      const int start = carry + incl - v;
      if (sidx < n_sub) {
        pre[sidx] = start;
        if (v > 0 && start < TF_REGS) marks[start] = ((sidx + 1) << MK_SHIFT) | start;
      }
      carry += tot;
    }
    if (threadIdx.x == 0) pre[n_sub] = carry;
    __syncthreads();
  }
  // Fewer candidates than k means the filter's histogram was not one of these
  // scores (candidate mode: the estimate lay above the k-th largest key):
  // select from the raw scores instead.
  const bool raw = !skip && carry < g.k_eff;
  if (raw && cmode) {
    // candidate mode stored no scores: recompute this segment's, exactly as
    // the score pass does (int32 dot products of the int8 codes)
    const int4 *qrow = reinterpret_cast<const int4 *>(a.qsk + (size_t)seg * RANK);
    const int4 q0 = qrow[0], q1 = qrow[1], q2 = qrow[2], q3 = qrow[3];
    const int4 *Sseg = reinterpret_cast<const int4 *>(a.S + ((size_t)g.b * Hkv + g.h) * NB * RANK);
    int32_t *dst = a.rescore + (size_t)seg * NB;
    for (int o = threadIdx.x; o < g.n_far; o += TF_THREADS) {
      const int4 *r = Sseg + (size_t)o * 4;
      const int4 s0 = r[0], s1 = r[1], s2 = r[2], s3 = r[3];
      int acc = 0;
      acc = __builtin_amdgcn_sdot4(s0.x, q0.x, acc, false);
      acc = __builtin_amdgcn_sdot4(s0.y, q0.y, acc, false);
      acc = __builtin_amdgcn_sdot4(s0.z, q0.z, acc, false);
      acc = __builtin_amdgcn_sdot4(s0.w, q0.w, acc, false);
      acc = __builtin_amdgcn_sdot4(s1.x, q1.x, acc, false);
      acc = __builtin_amdgcn_sdot4(s1.y, q1.y, acc, false);
      acc = __builtin_amdgcn_sdot4(s1.z, q1.z, acc, false);
      acc = __builtin_amdgcn_sdot4(s1.w, q1.w, acc, false);
      acc = __builtin_amdgcn_sdot4(s2.x, q2.x, acc, false);
      acc = __builtin_amdgcn_sdot4(s2.y, q2.y, acc, false);
      acc = __builtin_amdgcn_sdot4(s2.z, q2.z, acc, false);
      acc = __builtin_amdgcn_sdot4(s2.w, q2.w, acc, false);
      acc = __builtin_amdgcn_sdot4(s3.x, q3.x, acc, false);
      acc = __builtin_amdgcn_sdot4(s3.y, q3.y, acc, false);
      acc = __builtin_amdgcn_sdot4(s3.z, q3.z, acc, false);
      acc = __builtin_amdgcn_sdot4(s3.w, q3.w, acc, false);
      dst[o] = acc;
    }
    __syncthreads();                             // the workgroup's stores are visible to it
  }
  const int m = raw || skip ? g.n_far : carry;
  const int2 *cseg = cand + (size_t)seg * n_sub_max * TK_SUB;
  const int32_t *srow = (cmode ? a.rescore : scores) + (size_t)seg * NB;
  const bool in_regs = !raw && m <= TF_REGS;    // the candidates fit the threads' registers
  const bool cached = LDS_CACHE && in_regs && m <= TF_CACHE;   // ... and the exact path's LDS
  if (in_regs) {
    // Wave-major slots: wave w holds candidates [w * 64 nq, (w + 1) * 64 nq)
    // and its register q the 64 consecutive ones from w * 64 nq + 64 q, so
    // that every load reads 64 consecutive entries.  Slots at or past m hold
    // the key -1, which no count or histogram below takes.
    const int nq = (m + 64 * TF_WAVES - 1) / (64 * TF_WAVES);   // registers in use, <= TF_PERT
    const int slot0 = wave * nq * 64 + lane;                      // slot of register 0
    int2 c[TF_PERT];
    if (skip) {
      // the far entries themselves, in index order
#pragma unroll
      for (int q = 0; q < TF_PERT; ++q) {
        const int o = slot0 + 64 * q;
        c[q] = q < nq && o < m ? make_int2(o, biased_key(srow[o])) : make_int2(0, -1);
      }
    } else {
      // The sub-list holding slot o, and its start, are those of the last
      // mark at or before o: the running maximum of the marks over the slots.
      int run = 0;                               // uniform: the last mark before
      if (wave_local) {
        // this wave's marks, written and read by it alone: those of the
        // sub-lists that start in its slot range, and as `run` the sub-list
        // holding its first slot (the last non-empty one starting at or before)
        const int begin = wave * nq * 64, end = begin + nq * 64;
#pragma unroll
        for (int q = 0; q < TF_PERT; ++q)
          if (q < nq) marks[slot0 + 64 * q] = 0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        int best = -1;                           // the last such mark
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int mark = ((4 * lane + u + 1) << MK_SHIFT) | st[u];
          if (cv[u] > 0 && st[u] >= begin && st[u] < end) marks[st[u]] = mark;
          if (cv[u] > 0 && st[u] <= begin) best = mark;
        }
        const unsigned long long bb = __ballot(best >= 0);
        if (bb) run = __builtin_amdgcn_readlane(best, 63 - __clzll((long long)bb));
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        __builtin_amdgcn_wave_barrier();
      }
      int mk[TF_PERT];
#pragma unroll
      for (int q = 0; q < TF_PERT; ++q) {
        mk[q] = run;
        if (q < nq) {                            // uniform
          mk[q] = max(wave_incl_max(marks[slot0 + 64 * q]), run);
          run = __builtin_amdgcn_readlane(mk[q], 63);
        }
      }
      int before = 0;
      if (!wave_local) {
        // the marks of the earlier waves' ranges
        if (lane == 0) sc_own[wave] = run;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < TF_WAVES; ++w) before = max(before, w < wave ? sc_own[w] : 0);
      }
#pragma unroll
      for (int q = 0; q < TF_PERT; ++q) {
        const int o = slot0 + 64 * q;
        const int pk = max(before, mk[q]);
        const int s = min(max((pk >> MK_SHIFT) - 1, 0), n_sub - 1);   // clamped: always in bounds
        const int off = min(max(o - (pk & ((1 << MK_SHIFT) - 1)), 0), TK_SUB - 1);
        c[q] = q < nq && o < m ? cseg[(size_t)s * TK_SUB + off] : make_int2(0, -1);
      }
    }
    if (!h1_ready) __syncthreads();              // res[5] (wave 0), h1 zeroed, every wave's marks read
    if (h1_ready || cmode) {
      // Guess T without a filter pass: bin b1 from a level-1 histogram (the
      // score pass's, or in candidate mode that of the candidates, counted
      // here and searched by all waves), then a level-2 histogram of the low
      // bits of the keys in bin b1, which sit in registers.  The counts below
      // check the guess against the data before it is used.
      // Candidate mode bins the keys relative to the estimate E instead, in
      // bins of 2^CAND_FINE_BITS (the top bin takes every key from
      // E + 2047 * 2^CAND_FINE_BITS up): the candidates then spread over
      // many bins instead of a few dozen, so that the histogram's atomics
      // rarely collide, and the second level is 2^CAND_FINE_BITS bins that
      // one wave searches.  A key below E (an estimate that is not the one
      // the candidates were kept with) lands in bin 0 and fails the check.
      for (int k = threadIdx.x; k < hpad_size<HIST2_BINS>(); k += TF_THREADS) h2[k] = 0;
      auto fbin = [&](int key) {
        return min(max(key - e_cand, 0) >> CAND_FINE_BITS, HIST1_BINS - 1);
      };
      if (cmode) {
#pragma unroll
        for (int q = 0; q < TF_PERT; ++q)
          if (c[q].y >= 0) atomicAdd(&h1[hpad<HIST1_BINS>(fbin(c[q].y))], 1);
        __syncthreads();
        block_threshold_bin<TF_WAVES>(h1, g.k_eff, m, sc_pre, res);   // ends with a barrier
      } else {
        block_threshold_pair<TF_WAVES>(h1p.x, h1p.y, g.k_eff, g.n_far, sc_pre, res);
      }
      const int b1 = res[0];
      constexpr int FINE = 1 << CAND_FINE_BITS;
      static_assert(FINE <= 64, "one bin per lane");
      const bool fine_ok = b1 >= 0 && b1 < HIST1_BINS - 1;   // uniform
      if (cmode) {
        if (fine_ok) {
#pragma unroll
          for (int q = 0; q < TF_PERT; ++q)
            if (c[q].y >= 0 && fbin(c[q].y) == b1) atomicAdd(&h2[(c[q].y - e_cand) & (FINE - 1)], 1);
        }
      } else if (b1 >= 0) {
#pragma unroll
        for (int q = 0; q < TF_PERT; ++q)
          if ((c[q].y >> HIST2_BITS) == b1)
            atomicAdd(&h2[hpad<HIST2_BINS>(c[q].y & (HIST2_BINS - 1))], 1);
      }
      __syncthreads();
      if (wave == 0) {
        int T = -1;
        int above;
        bool valid;
        if (cmode) {
          if (fine_ok) {
            int v[1] = {lane < FINE ? h2[lane] : 0};
            const int b2 = wave_threshold_regs<1>(v, res[1], res[2], above, valid);
            if (valid) T = e_cand + (b1 << CAND_FINE_BITS) + b2;
          }
        } else if (b1 >= 0) {
          const int b2 = wave_threshold_bin_valid<HIST2_BINS>(h2, res[1], res[2], above, valid);
          if (valid) T = (b1 << HIST2_BITS) | b2;
        }
        if (lane == 0) res[5] = T;
      }
      __syncthreads();
    }
    const int T = res[5];
    if (T >= 0) {
      // Count, from the data, the candidates above T and equal to T.  Every
      // element with key >= T is a candidate (its bin is >= b1), so T is the
      // k-th largest key exactly when above < k <= above + equal.
      int gt = 0, tie = 0;                       // this wave's, uniform
#pragma unroll
      for (int q = 0; q < TF_PERT; ++q) {
        gt += __popcll(__ballot(c[q].y > T));
        tie += __popcll(__ballot(c[q].y == T));
      }
      if (lane == 0) sc_cnt[wave] = gt | (tie << 16);
      __syncthreads();
      int gt_tot = 0, tie_tot = 0, gt_run = 0, tie_run = 0;
#pragma unroll
      for (int w = 0; w < TF_WAVES; ++w) {
        const int v = sc_cnt[w];
        gt_tot += v & 0xffff;
        tie_tot += v >> 16;
        gt_run += w < wave ? v & 0xffff : 0;
        tie_run += w < wave ? v >> 16 : 0;
      }
      if (gt_tot < g.k_eff && gt_tot + tie_tot >= g.k_eff) {      // uniform
        const int need = g.k_eff - gt_tot;     // ties at T to take, lowest index first
        const unsigned long long lt = (1ull << lane) - 1ull;
#pragma unroll
        for (int q = 0; q < TF_PERT; ++q) {
          const bool is_gt = c[q].y > T, is_tie = c[q].y == T;
          const unsigned long long gb = __ballot(is_gt), tb = __ballot(is_tie);
          const int gt_before = gt_run + __popcll(gb & lt), tie_before = tie_run + __popcll(tb & lt);
          if (is_gt || (is_tie && tie_before < need)) out[gt_before + min(tie_before, need)] = c[q].x;
          gt_run += __popcll(gb);
          tie_run += __popcll(tb);
        }
        for (int j = g.k_eff + threadIdx.x; j < topk; j += TF_THREADS) out[j] = -1;
        finish();
        return;
      }
    }
    // the guess did not hold: keep the candidates in LDS for the exact path
    // (the marks they overwrite were last read before the barrier above)
    if (cached) {
#pragma unroll
      for (int q = 0; q < TF_PERT; ++q)
        if (c[q].y >= 0) cache[slot0 + 64 * q] = c[q];
    }
  }

  // ---- exact path without the level-2 histogram
  auto get = [&](int o) -> int2 {                // uncached access
    if (raw || skip) return make_int2(o, biased_key(srow[o]));
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
  bool fast = !skip && !cmode && th.z && !raw && th.x >= 0 && th.x < HIST1_BINS;
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
  finish();
}


inline FinalArgs final_args(const int32_t *scores, const int32_t *seq_len, const Shape &s, int32_t *idx,
                     int32_t *n_sel, const TopkWs &w) {
  FinalArgs a;
  a.scores = scores;
  a.seq_len = seq_len;
  a.hist1 = w.hist1;
  a.hist2 = w.hist2;
  a.thr = w.counters;
  a.cnt = w.cnt;
  a.cand = w.cand;
  a.n_sub_max = w.nchunk;
  a.R = s.R;
  a.Hkv = s.Hkv;
  a.T_max = s.T_max;
  a.NB = s.NB;
  a.window = s.window;
  a.pool = s.pool;
  a.topk = s.topk;
  a.idx = idx;
  a.n_sel = n_sel;
  a.skip = 0;
  a.h1_ready = 0;
  a.cand_mode = 0;
  a.hsamp = nullptr;
  a.zero_hsamp = 1;
  a.qsk = nullptr;
  a.S = nullptr;
  a.rescore = nullptr;
  return a;
}

}  // namespace
}  // namespace sks
