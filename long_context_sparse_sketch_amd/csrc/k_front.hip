// The decode step's first launch: the work that comes before the score pass,
// in one grid of 256-thread workgroups ("What it took" on the page "8 agents
// x 250K context, concurrently, on two 3090s": build the sketch, score every
// token, pick the top ~2K -- graph-safe):
//
//   [0, n_samp)           candidate mode's sample pass (topk_body.h), each
//                         workgroup computing its segment's query sketch
//                         itself (the same routine and bits as below), so
//                         that it needs nothing from this launch; when one
//                         workgroup samples a whole segment (EST), it also
//                         derives the segment's estimate E for the score
//                         pass instead of publishing its histogram;
//   [.., + nq)            the query sketch of every (sequence, row, KV head);
//   [.., + n_app)         the append: the key sketch (and pooled block) of
//                         the rows' own tokens (sketch_body.h).
// The three are independent chains of a few dependent loads each, so one
// launch pays their latency once instead of three times.  The sample
// workgroups have the longest chain and come first in the grid, which is
// dispatched in order.  The append writes sketch rows of the rows' own
// tokens, which the sample pass reads only when the window is shorter than
// the rows (then a sampled row may be read while it is written: the sample
// decides only how long the selection takes, never its result).
#include "sketch_body.h"
#include "tier.h"
#include "topk_body.h"

namespace sks {
namespace {

struct FrontArgs {
  int R, Hkv, T_max, NB, window, pool, topk;
  int n_samp, samp_per_seg, samp_stride, nq, n_app, app_rows;
  const int32_t *seq_len;
  // the query sketch and the append
  const uint16_t *q;
  int Hq;
  const float *basis;
  int basis_per_head;
  const float *key_scale;
  int8_t *qsk;
  float *qscale;
  const void *K, *V;
  const uint16_t *Ks;
  const void *Kh;
  const uint16_t *Ksh;
  int W_hot;
  int8_t *S;
  uint16_t *Kp, *Vp;
  // the sample pass
  int32_t *hsamp;
  int32_t *est;   // (EST) the segments' selection records: E in the first int of each
};

struct SampleLds {
  int lh[HIST1_BINS];
  __align__(16) int8_t qcode[RANK];
  SampleEstLds est;
  SketchLds sk;
};

union FrontLds {
  SampleLds samp;
  SketchLds sk;
};

// The arguments read first (the pointers, the block counts and the shape
// numbers the block's first loads need) come as scalar arguments ahead of
// the struct, so that they arrive preloaded in SGPRs; they override the
// struct's copies.
template <int DT, bool CAND, bool EST>
__global__ __launch_bounds__(SK_THREADS) void front_kernel(const uint16_t *q, const float *basis,
                                                          const int32_t *seq_len, int8_t *S,
                                                          int nq, int n_app, int samp_per_seg,
                                                          int R, int Hkv, int Hq,
                                                          int basis_per_head, FrontArgs f) {
  static_assert(SK_THREADS == SAMPLE_THREADS, "one workgroup size");
  static_assert(!EST || CAND, "the estimate is candidate mode's");
  __shared__ FrontLds lds;
  int blk = blockIdx.x;
  if (CAND && blk < f.n_samp) {
    const int seg = blk / samp_per_seg;
    const int h = seg % Hkv, b = seg / (Hkv * R);
    const int j0 = (blk % samp_per_seg) * SAMPLE_WG_ROWS;   // EST: one workgroup per segment, 0
    // Every load is issued before the row's length is known: the sampled
    // rows j * stride < NB lie in the cache whatever the length, and those
    // past the far region are not counted.
    const int stride = f.samp_stride;
    // The query sketch's own loads go first (its chain is the longer one);
    // the sampled rows load behind them.
    int4 sv[SAMPLE_UNROLL];
    block_query_sketch(q, R, Hq, Hkv, basis, basis_per_head, seg, lds.samp.qcode, nullptr,
                       lds.samp.sk, [&] {
                         sample_load(S, ((size_t)b * Hkv + h) * f.NB, j0,
                                     (f.NB + stride - 1) / stride, stride, sv);
                         for (int k = threadIdx.x; k < HIST1_BINS; k += SAMPLE_THREADS)
                           lds.samp.lh[k] = 0;
                         if (EST)
                           for (int k = threadIdx.x; k < HIST2_BINS; k += SAMPLE_THREADS)
                             lds.samp.est.h2[k] = 0;
                       });
    const SegGeom g = seg_geom(seg, seq_len, R, Hkv, f.T_max, f.window, f.pool, f.topk);
    if (g.k_eff >= g.n_far) return;             // uniform: no selection needed
    const int m = (g.n_far + stride - 1) / stride;
    if (j0 >= m) return;
    __syncthreads();
    const int4 qv = reinterpret_cast<const int4 *>(lds.samp.qcode)[threadIdx.x & 3];
    int keys[SAMPLE_UNROLL];
    sample_bins(sv, qv, j0, m, lds.samp.lh, keys);
    __syncthreads();
    if (EST) {                                   // the whole segment's sample is here
      const int E = sample_estimate(lds.samp.lh, keys, g.n_far, g.k_eff, stride, lds.samp.est);
      if (threadIdx.x == 0) f.est[4 * seg] = E;
      return;
    }
    sample_flush(lds.samp.lh, f.hsamp + (size_t)seg * HIST1_BINS);
    return;
  }
  if (CAND) blk -= f.n_samp;
  if (blk < nq) {
    block_query_sketch(q, R, Hq, Hkv, basis, basis_per_head, blk, f.qsk + (size_t)blk * RANK,
                       f.qscale ? f.qscale + blk : nullptr, lds.sk);
    return;
  }
  blk -= nq;
  if (blk < n_app) {
    block_key_row<DT>(f.K, f.V, f.Ks, f.Kh, f.Ksh, f.W_hot, seq_len, basis, basis_per_head,
                      f.key_scale, Hkv, f.T_max, R, f.NB, f.pool, 1, 0, 0, S, f.Kp, f.Vp,
                      blk / f.app_rows, blk % f.app_rows, lds.sk);
  }
}

template <int DT>
void launch_front_t(const FrontArgs &f, bool cand, int grid, hipStream_t st) {
  if (cand && f.est)
    front_kernel<DT, true, true><<<grid, SK_THREADS, 0, st>>>(f.q, f.basis, f.seq_len, f.S, f.nq,
                                                               f.n_app, f.samp_per_seg, f.R,
                                                               f.Hkv, f.Hq, f.basis_per_head, f);
  else if (cand)
    front_kernel<DT, true, false><<<grid, SK_THREADS, 0, st>>>(f.q, f.basis, f.seq_len, f.S, f.nq,
                                                                f.n_app, f.samp_per_seg, f.R,
                                                                f.Hkv, f.Hq, f.basis_per_head, f);
  else
    front_kernel<DT, false, false><<<grid, SK_THREADS, 0, st>>>(f.q, f.basis, f.seq_len, f.S,
                                                                 f.nq, f.n_app, f.samp_per_seg,
                                                                 f.R, f.Hkv, f.Hq,
                                                                 f.basis_per_head, f);
}

}  // namespace

hipError_t launch_step_front(const sks_kv &kv, const Shape &s, const uint16_t *q, int Hq,
                             const float *basis, int basis_per_head, const float *key_scale,
                             int8_t *qsk, float *qscale, int8_t *S, uint16_t *Kp, uint16_t *Vp,
                             bool append, bool cand, const TopkWs &w, hipStream_t st) {
  FrontArgs f;
  f.R = s.R;
  f.Hkv = s.Hkv;
  f.T_max = s.T_max;
  f.NB = s.NB;
  f.window = s.window;
  f.pool = s.pool;
  f.topk = s.topk;
  f.seq_len = kv.seq_len;
  const int nseg = s.B * s.R * s.Hkv;
  f.samp_per_seg = 1;
  f.samp_stride = SAMPLE_STRIDE;
  f.n_samp = 0;
  f.est = nullptr;
  if (cand) {
    const long max_far = s.T_max > s.window ? (long)(s.T_max - s.window) / s.pool : 0;
    if (topk_cand_est_early(s)) {
      f.est = w.counters;                        // one workgroup per segment
      f.samp_stride = topk_cand_est_stride(s);
    } else {
      f.samp_per_seg = std::max(1, ceil_div((max_far + SAMPLE_STRIDE - 1) / SAMPLE_STRIDE, SAMPLE_WG_ROWS));
    }
    f.n_samp = f.samp_per_seg * nseg;
  }
  f.nq = nseg;
  // append rows per (b, h), as in launch_sketch_keys' append mode
  long app_rows = s.pool == 1 ? (long)s.R : ((long)s.R + s.pool) / s.pool + 1;
  if (app_rows > s.NB) app_rows = s.NB;
  f.app_rows = (int)app_rows;
  f.n_app = append ? f.app_rows * s.B * s.Hkv : 0;
  f.q = q;
  f.Hq = Hq;
  f.basis = basis;
  f.basis_per_head = basis_per_head;
  f.key_scale = key_scale;
  f.qsk = qsk;
  f.qscale = qscale;
  f.K = kv.K;
  f.V = kv.V;
  f.Ks = kv.K_scale;
  const HotRows hr = hot_rows(kv);
  f.Kh = hr.K;
  f.Ksh = hr.Ks;
  f.W_hot = hr.W;
  f.S = S;
  f.Kp = Kp;
  f.Vp = Vp;
  f.hsamp = w.hsamp;
  const long grid = (long)f.nq + f.n_app + f.n_samp;
  if (s.dtype == SKS_KV_I8)
    launch_front_t<SKS_KV_I8>(f, cand, (int)grid, st);
  else if (s.dtype == SKS_KV_I4)
    launch_front_t<SKS_KV_I4>(f, cand, (int)grid, st);
  else
    launch_front_t<SKS_KV_BF16>(f, cand, (int)grid, st);
  return hipGetLastError();
}

}  // namespace sks
