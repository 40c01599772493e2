// Internal declarations of libsks: device helpers, tile constants, launchers.
// gfx950 (CDNA4) only: 64-lane wavefronts, DPP row operations, v_dot4 int8.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "sks.h"

namespace sks {

// ---------------------------------------------------------------- constants
constexpr int D = SKS_HEAD_DIM;          // 128
constexpr int RANK = SKS_RANK;           // 64
constexpr int SCORE_BIAS = 1 << 20;      // |score| <= 64*127*127 < 2^20
constexpr int HIST1_BITS = 11;           // top bits of the 21-bit biased score
constexpr int HIST1_BINS = 1 << HIST1_BITS;
constexpr int HIST2_BITS = 10;           // low bits
constexpr int HIST2_BINS = 1 << HIST2_BITS;
constexpr int SCORE_CHUNK = 1024;        // tokens per score workgroup
constexpr int TK_CHUNK = 4096;           // tokens per top-k filter workgroup
constexpr int TK_SUB = 1024;             // tokens per filter wave (one candidate sub-list)
constexpr int TK_MAX_SUBS = 8192;        // sub-lists per segment the final pass can index
constexpr int ATTN_MAX_G = 8;            // query heads per KV head supported
constexpr int SAMPLE_STRIDE = 64;        // candidate mode samples one far entry in 64 ...
constexpr int SAMPLE_EST_STRIDE = 128;   // ... or in 128 where one workgroup samples a segment
constexpr int CAND_FINE_BITS = 5;        // candidate mode's final pass: bins of 32 keys above E

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// ---------------------------------------------------------------- geometry
// Per-row geometry of the step (see sks.h): clamp the device length, then
// derive far count, window start and effective k.
struct RowGeom {
  int L;      // tokens visible to the row
  int n_far;  // far tokens / blocks
  int ws;     // first exact-window token
  int k_eff;  // selected far entries
  int n_ent;  // k_eff + (L - ws): size of the attention set
};

__device__ __forceinline__ int clamp_len(int raw, int T_max, int R) {
  int hi = T_max - R + 1;
  if (hi < 0) hi = 0;
  return raw < 0 ? 0 : (raw > hi ? hi : raw);
}

__device__ __forceinline__ RowGeom row_geom(int L0, int i, int window, int pool, int topk) {
  RowGeom g;
  g.L = L0 + i;
  g.n_far = g.L > window ? (g.L - window) / pool : 0;
  g.ws = g.n_far * pool;
  g.k_eff = g.n_far < topk ? g.n_far : topk;
  g.n_ent = g.k_eff + (g.L - g.ws);
  return g;
}

// ---------------------------------------------------------------- numerics
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_bits_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Round a finite double in the normal bf16 range to bfloat16, ties to even:
// keep the top 7 explicit mantissa bits of the binary64 encoding.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const unsigned long long drop = 45;            // 52 - 7 explicit bits kept
  unsigned long long lsb = (u >> drop) & 1ull;
  u += ((1ull << (drop - 1)) - 1ull) + lsb;
  u &= ~((1ull << drop) - 1ull);
  float f = (float)__longlong_as_double((long long)u);   // exact
  return (uint16_t)(__float_as_uint(f) >> 16);
}

// Score -> unsigned 21-bit selection key (bias 2^20), clamped for safety.
__device__ __forceinline__ int biased_key(int s) {
  int v = s + SCORE_BIAS;
  return v < 0 ? 0 : (v > (1 << 21) - 1 ? (1 << 21) - 1 : v);
}

__device__ __forceinline__ int8_t quant_code(float y, float scale) {
  float v = __builtin_rintf(y / scale);
  v = fminf(fmaxf(v, -127.0f), 127.0f);
  return (int8_t)(int)v;
}

// DPP lane permutations inside a row of 16 lanes (gfx9 encodings).
constexpr int DPP_QUAD_XOR1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;  // lane i <-> 15 - i
constexpr int DPP_ROW_HMIRROR = 0x141; // lane i <-> 7 - i within each half row

template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 4 lanes of a quad; every lane gets the total.
__device__ __forceinline__ int quad_sum_i(int x) {
  x += dpp_i<DPP_QUAD_XOR1>(x);
  x += dpp_i<DPP_QUAD_XOR2>(x);
  return x;
}

// Sum over the 16 lanes of a row; every lane gets the total.  The mirror
// steps pair lanes into 4 classes {a, 7-a, 8+a, 15-a}; the quad steps then
// combine one lane of each class.
__device__ __forceinline__ float row16_sum_f(float x) {
  x += dpp_f<DPP_ROW_MIRROR>(x);
  x += dpp_f<DPP_ROW_HMIRROR>(x);
  x += dpp_f<DPP_QUAD_XOR1>(x);
  x += dpp_f<DPP_QUAD_XOR2>(x);
  return x;
}

// ---------------------------------------------------------------- wave scans
// Inclusive scans over the 64 lanes of a wave: DPP row shifts inside each row
// of 16 lanes (a lane whose source lies outside its row adds 0), then the
// totals of the lower rows, read from lanes 15, 31 and 47.
constexpr int DPP_ROW_SHR = 0x110;     // row_shr:n = 0x110 + n

template <int N>
__device__ __forceinline__ int dpp_shr(int x) {
  return __builtin_amdgcn_update_dpp(0, x, DPP_ROW_SHR + N, 0xF, 0xF, false);
}

__device__ __forceinline__ int wave_incl_add(int x) {
  x += dpp_shr<1>(x);
  x += dpp_shr<2>(x);
  x += dpp_shr<4>(x);
  x += dpp_shr<8>(x);
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Saturating version for non-negative x <= cap < 2^29: every partial sum is
// min(true sum, cap), so a total below cap is exact.
__device__ __forceinline__ int wave_incl_add_sat(int x, int cap) {
  x = min(x + dpp_shr<1>(x), cap);
  x = min(x + dpp_shr<2>(x), cap);
  x = min(x + dpp_shr<4>(x), cap);
  x = min(x + dpp_shr<8>(x), cap);
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return min(x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0), cap);
}

// Running maximum of non-negative values.
__device__ __forceinline__ int wave_incl_max(int x) {
  x = max(x, dpp_shr<1>(x));
  x = max(x, dpp_shr<2>(x));
  x = max(x, dpp_shr<4>(x));
  x = max(x, dpp_shr<8>(x));
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return max(x, max(row > 0 ? r0 : 0, max(row > 1 ? r1 : 0, row > 2 ? r2 : 0)));
}

// ---------------------------------------------------------------- candidate estimate
// Candidate mode's estimate E of a row's k-th largest biased key, from the
// row's sample histogram (every stride-th far entry scored and counted by
// level-1 bin).  With m = ceil(n_far / stride) sampled entries and
// k' = ceil(k_eff m / n_far) the expected number of them among the k largest,
// E is the lowest key of the bin holding the rho-th largest sampled key,
// rho = 2 k' + 8; E = 0 when fewer than rho entries were sampled.  force 1
// gives E above every key, 2 gives 0.  E decides only how much work the
// selection does, never its result.
//
// NT threads (8 bins each) hold the histogram, thread t bins 2047 - 8t down to
// 2040 - 8t in hv.  Bins are clamped to [0, 2^18] (a real sample never
// exceeds 2^17 per bin), so that a histogram holding garbage cannot overflow
// the sums and every workgroup reading the same bins finds the same E.
// escan holds NT / 64 ints; *e_out (LDS) receives E and, when given,
// *rank_out (LDS) the rank of the rho-th largest sampled key inside E's bin,
// counted from the top of the bin (1 ..), or 0 when E is not a bin's lower
// edge found this way.  Two barriers: the results are readable after the
// call, and escan may be used again.
template <int NT>
__device__ void block_estimate(const int (&hv)[8], int n_far, int k_eff, int stride, int force,
                               int *escan, int *e_out, int *rank_out = nullptr) {
  static_assert(NT * 8 == HIST1_BINS, "eight bins per thread");
  constexpr int HS_MAX = 1 << 18;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int sum = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) sum += min(max(hv[k], 0), HS_MAX);
  const int incl = wave_incl_add(sum);
  if (lane == 63) escan[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    before += w < wave ? escan[w] : 0;
    tot += escan[w];
  }
  const int m = (n_far + stride - 1) / stride;
  const int kp = n_far > 0 ? (int)(((long)k_eff * m + n_far - 1) / n_far) : 0;
  const int rho = 2 * kp + 8;
  int run = before + incl - sum;                 // sampled keys in higher bins
  const int top = HIST1_BINS - 1 - 8 * (int)threadIdx.x;
  if (threadIdx.x == 0 && (tot < rho || force)) {
    *e_out = force == 1 ? (1 << 30) : 0;
    if (rank_out) *rank_out = 0;
  }
  if (!force && tot >= rho && run < rho && run + sum >= rho) {
    int bin = top - 7, rank = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = min(max(hv[k], 0), HS_MAX);
      if (run < rho && run + c >= rho) {
        bin = top - k;
        rank = rho - run;
      }
      run += c;
    }
    *e_out = bin << HIST2_BITS;
    if (rank_out) *rank_out = rank;
  }
  __syncthreads();
}

// Top-down rank search over a histogram that NT threads hold PER bins each,
// thread t the bins at positions PER t .. PER t + PER - 1 counted from the
// top (position 0: the highest bin): writes *pos_out = the position at which
// the running count from the top first reaches need (1 <= need), or -1 when
// the total stays below need.  Counts are non-negative and sum below 2^31.
// Two barriers: *pos_out is readable after the call, and escan (NT / 64
// ints) may be used again.
template <int NT, int PER>
__device__ void block_top_rank(const int (&v)[PER], int need, int *escan, int *pos_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int sum = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) sum += v[k];
  const int incl = wave_incl_add(sum);
  if (lane == 63) escan[wave] = incl;
  if (threadIdx.x == 0) *pos_out = -1;
  __syncthreads();
  int run = incl - sum;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) run += w < wave ? escan[w] : 0;
  if (run < need && run + sum >= need) {
    int pos = PER * (int)threadIdx.x;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (run < need && run + v[k] >= need) pos = PER * (int)threadIdx.x + k;
      run += v[k];
    }
    *pos_out = pos;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- selection threshold
// Threshold search over a histogram held in registers, lane l holding bins
// [l*PER, (l+1)*PER) in v[].  No barriers.  The histogram is validated first
// (every bin in [0, n], total exactly n, n < 2^28); an invalid one gives
// valid = false and bin 0.  Otherwise returns the bin b with
// sum_{b' >= b} >= need > sum_{b' > b} (0 if there is none); `above` receives
// sum_{b' > b}.
template <int PER>
__device__ __forceinline__ int wave_threshold_regs(const int (&v)[PER], int need, int n, int &above,
                                                   bool &valid) {
  const int cap = n + 1;
  int sum = 0;
  bool bad = false;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    bad |= v[k] < 0 || v[k] > n;
    sum = min(sum + min(max(v[k], 0), cap), cap);
  }
  const int incl = wave_incl_add_sat(sum, cap);
  const int tot = __builtin_amdgcn_readlane(incl, 63);
  above = 0;
  valid = __ballot(bad) == 0 && tot == n;
  if (!valid) return 0;
  int ab = n - incl;                         // bins of higher lanes
  int b = -1, ab_b = 0;
  if (ab < need && ab + sum >= need) {
#pragma unroll
    for (int k = PER - 1; k >= 0; --k) {
      if (b < 0) {
        if (ab + v[k] >= need) {
          b = (int)(threadIdx.x & 63) * PER + k;
          ab_b = ab;
        } else {
          ab += v[k];
        }
      }
    }
  }
  const unsigned long long who = __ballot(b >= 0);
  if (who == 0) return 0;
  const int src = __ffsll((long long)who) - 1;
  above = __builtin_amdgcn_readlane(ab_b, src);
  return __builtin_amdgcn_readlane(b, src);
}

// ---------------------------------------------------------------- launchers
struct Shape {
  int B, R, Hkv, T_max, NB, window, topk, pool, dtype;
};

hipError_t launch_sketch_keys(const sks_kv &kv, const Shape &s, const float *basis,
                              int basis_per_head, const float *key_scale, int t_begin,
                              int t_end, int8_t *S, uint16_t *Kp, uint16_t *Vp,
                              hipStream_t st);
hipError_t launch_sketch_query(const uint16_t *q, int B, int R, int Hq, int Hkv,
                               const float *basis, int basis_per_head, int8_t *qsk,
                               float *qscale, hipStream_t st);
// Workspace layout: [hist region | selection scratch | attention partials].
// The hist region holds the level-1 and level-2 selection histograms
// [nseg][2048] and [nseg][1024], zero at rest (the calls that use them return
// them to zero), the per-segment threshold bins and the per-sub-list score
// maxima written with the level-1 histogram.  The selection scratch holds the
// candidate lists, the last region the attention partials.
// (Kernels here never communicate between workgroups inside one launch: a
// device-scope fence per workgroup costs far more on this GPU than a kernel
// boundary.)
size_t hist_region_bytes(const Shape &s);
size_t topk_scratch_bytes(const Shape &s);
size_t attn_scratch_bytes(const Shape &s, int G);

hipError_t launch_fill(int32_t *p, size_t n, hipStream_t st);
// With `w` (non-null) the score pass also builds the selection histogram;
// with `cand` it stores no scores but the selection's candidates at or above
// the estimates it derives from the sample pass's histograms (candidate
// mode; force 1: estimate above every key, 2: zero).
struct TopkWs;
hipError_t launch_score(const int8_t *qsk, const int8_t *S, const int32_t *seq_len,
                        const Shape &s, int32_t *scores, const TopkWs *w, hipStream_t st,
                        bool cand = false, int force = 0, const int32_t *est = nullptr);

struct TopkWs {
  int32_t *hist1;     // [nseg][HIST1_BINS], zero at rest
  int32_t *hist2;     // [nseg][HIST2_BINS], zero at rest
  int32_t *cmax;      // [nseg][nchunk]: largest biased score of each sub-list + 1 (0: empty)
  int32_t *hsamp;     // [nseg][HIST1_BINS]: candidate mode's sample histogram, zero at rest
  int32_t *counters;  // [nseg][4]: threshold bin b1, count above it, valid, count in b1;
                      // in candidate mode the estimate E, in the first int
  char *scratch;      // start of the selection scratch (cnt, cand)
  char *attn;         // start of the attention partials (after the selection scratch)
  int32_t *cnt;       // [nseg][nchunk]
  int2 *cand;         // [nseg][nchunk * TK_SUB]
  int nchunk;         // sub-lists per segment
};
TopkWs topk_ws_carve(const Shape &s, void *ws);
hipError_t launch_topk_filter(const int32_t *scores, const int32_t *seq_len, const Shape &s,
                              bool hist_ready, const TopkWs &w, hipStream_t st);
hipError_t launch_topk(const int32_t *scores, const int32_t *seq_len, const Shape &s,
                       bool hist_ready, int32_t *idx, int32_t *n_sel, const TopkWs &w,
                       hipStream_t st);
// Candidate mode: the sample pass (per-segment sample histograms), and the
// final pass over the score pass's candidates, which rescores a segment into
// `scores` when its estimate was too high and returns the sample histograms
// to zero (with zero_hsamp; else a later launch must).
bool topk_cand_preferred(const Shape &s);
// Whether one sample workgroup covers each segment's whole sample (at most
// SAMPLE_WG_ROWS entries at a stride of 64, or else 128), so that the sample
// pass derives the estimate E itself and the score pass reads it from the
// segment's TopkWs::counters record; and that stride.
bool topk_cand_est_early(const Shape &s);
int topk_cand_est_stride(const Shape &s);
hipError_t launch_topk_sample(const int8_t *qsk, const int8_t *S, const int32_t *seq_len,
                              const Shape &s, const TopkWs &w, hipStream_t st);
hipError_t launch_topk_cand(const int8_t *qsk, const int8_t *S, int32_t *scores,
                            const int32_t *seq_len, const Shape &s, int32_t *idx,
                            int32_t *n_sel, const TopkWs &w, hipStream_t st,
                            bool zero_hsamp = true);

// The decode step's first launch (k_front.hip): the query sketch, the append
// (append) and candidate mode's sample pass (cand) in one grid.
hipError_t launch_step_front(const sks_kv &kv, const Shape &s, const uint16_t *q, int Hq,
                             const float *basis, int basis_per_head, const float *key_scale,
                             int8_t *qsk, float *qscale, int8_t *S, uint16_t *Kp, uint16_t *Vp,
                             bool append, bool cand, const TopkWs &w, hipStream_t st);
// The attention pass and its merge; the merge also clears zero[0, nzero)
// when `zero` is given.
hipError_t launch_attn(const uint16_t *q, int Hq, const sks_kv &kv, const Shape &s,
                       const int32_t *idx, const uint16_t *Kp, const uint16_t *Vp,
                       float sm_scale, float *out, float *lse, const TopkWs &w, hipStream_t st,
                       bool dense = false, int32_t *zero = nullptr, long nzero = 0);

hipError_t launch_gather(const sks_kv &kv, const Shape &s, const int32_t *idx,
                         const uint16_t *Kp, const uint16_t *Vp, void *K_out, void *V_out,
                         uint16_t *Ks_out, uint16_t *Vs_out, int32_t *n_out, hipStream_t st);

}  // namespace sks
