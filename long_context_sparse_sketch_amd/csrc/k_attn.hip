// Sparse decode attention: one softmax over a row's selected far entries and
// its exact window ("What it adds" on the "Agens SGLang" README: sliding
// window plus mean-pooled far field merged under one softmax; "int8
// attention" over the picked rows in "What it took" on the page "8 agents x
// 250K context, concurrently, on two 3090s").
//
// Split-K flash decoding.  A workgroup takes ATTN_SPLIT (384) consecutive
// entries of one (sequence, row, KV head) attention set and all G query heads
// of that KV head; each of its 4 waves takes 96 of them as three tiles of 32
// (see attn_body.h), gathering tile t + 1 while it computes tile t.
// Attention sets under 1,536 entries take 128 entries per workgroup (one
// tile per wave), and int8 / int4 caches 256 (two tiles).
// Online softmax in the log2 domain;
// the waves' states are merged through LDS and the workgroup writes one
// partial (m, l, acc[G][128]).  A second kernel merges the partials of every
// split in split order, so results are deterministic.
#include "attn_body.h"

namespace sks {
namespace {

// One workgroup of D x merge_parts(nsplit) threads per (segment, query head
// of the group).  With `zero`, the workgroups also clear zero[0, nzero)
// between them, after their merge (stores issued before the loads would
// delay them).
__global__ __launch_bounds__(D * MP) void attn_merge_kernel(const float2 *__restrict__ part_ml,
                                                            const float *__restrict__ part_acc,
                                                            int nsplit, int G, int Hkv,
                                                            float *__restrict__ out,
                                                            float *__restrict__ lse,
                                                            int32_t *__restrict__ zero,
                                                            long nzero) {
  merge_splits(part_ml, part_acc, blockIdx.x, blockIdx.y, nsplit, G, Hkv, out, lse);
  if (zero) {
    const long nb = (long)gridDim.x * gridDim.y, blk = (long)blockIdx.y * gridDim.x + blockIdx.x;
    const long per = (nzero + nb - 1) / nb, end = min(nzero, (blk + 1) * per);
    const int nt = blockDim.x * blockDim.y, t = threadIdx.y * blockDim.x + threadIdx.x;
    for (long i = blk * per + t; i < end; i += nt) zero[i] = 0;
  }
}

template <int G, int DT, bool POOLED, int TILES>
__global__ __launch_bounds__(AT_THREADS, 2) void attn_kernel(const int32_t *idx,
                                                             const int32_t *seq_len, int topk,
                                                             int R, int Hkv, AttnArgs a,
                                                             int slot0) {
  __shared__ AttnLds<attn_kstage<DT>()> lds;
  attn_body<G, DT, POOLED, TILES>(a, idx, seq_len, topk, R, Hkv, blockIdx.y, slot0 + blockIdx.x,
                                  lds);
}

// The splits attn_split() gives: one tile per wave for small attention sets,
// else three for bf16 rows and two for int8 / int4 rows; only these kernels
// are built.
template <int G, int TILES>
hipError_t dispatch_t(dim3 grid, hipStream_t st, const AttnArgs &a, int dtype, int pool, int slot0) {
  if (dtype == SKS_KV_I8 || dtype == SKS_KV_I4) {
    if constexpr (TILES == 3) {
      return hipErrorInvalidValue;
    } else if (dtype == SKS_KV_I8) {
      attn_kernel<G, SKS_KV_I8, false, TILES><<<grid, AT_THREADS, 0, st>>>(a.idx, a.seq_len, a.topk, a.R, a.Hkv, a, slot0);
    } else {
      attn_kernel<G, SKS_KV_I4, false, TILES><<<grid, AT_THREADS, 0, st>>>(a.idx, a.seq_len, a.topk, a.R, a.Hkv, a, slot0);
    }
  } else if constexpr (TILES == 2) {
    return hipErrorInvalidValue;
  } else if (pool > 1) {
    attn_kernel<G, SKS_KV_BF16, true, TILES><<<grid, AT_THREADS, 0, st>>>(a.idx, a.seq_len, a.topk, a.R, a.Hkv, a, slot0);
  } else {
    attn_kernel<G, SKS_KV_BF16, false, TILES><<<grid, AT_THREADS, 0, st>>>(a.idx, a.seq_len, a.topk, a.R, a.Hkv, a, slot0);
  }
  return hipSuccess;
}

template <int G>
hipError_t dispatch_g(dim3 grid, hipStream_t st, const AttnArgs &a, int dtype, int pool, int slot0) {
  if (a.split == attn_split_entries<1>())
    return dispatch_t<G, 1>(grid, st, a, dtype, pool, slot0);
  else if (a.split == attn_split_entries<2>())
    return dispatch_t<G, 2>(grid, st, a, dtype, pool, slot0);
  else
    return dispatch_t<G, 3>(grid, st, a, dtype, pool, slot0);
}

}  // namespace

size_t attn_scratch_bytes(const Shape &s, int G) {
  const size_t nseg = (size_t)s.B * s.R * s.Hkv;
  const size_t n = nseg * attn_nsplit(s) * G;
  return align_up(n * sizeof(float2), 256) + align_up(n * D * sizeof(float), 256);
}

AttnArgs attn_args(const uint16_t *q, int Hq, const sks_kv &kv, const Shape &s,
                   const int32_t *idx, const uint16_t *Kp, const uint16_t *Vp, float sm_scale,
                   const TopkWs &w) {
  const int G = Hq / s.Hkv;
  const int nseg = s.B * s.R * s.Hkv;
  AttnArgs a;
  a.q = q;
  a.K = kv.K;
  a.V = kv.V;
  a.Ks = kv.K_scale;
  a.Vs = kv.V_scale;
  const HotRows hr = hot_rows(kv);
  a.Kh = hr.K;
  a.Vh = hr.V;
  a.Ksh = hr.Ks;
  a.Vsh = hr.Vs;
  a.W_hot = hr.W;
  a.seq_len = kv.seq_len;
  a.idx = idx;
  a.Kp = Kp;
  a.Vp = Vp;
  a.sm_log2 = sm_scale * 1.4426950408889634f;
  a.R = s.R;
  a.Hkv = s.Hkv;
  a.T_max = s.T_max;
  a.NB = s.NB;
  a.window = s.window;
  a.pool = s.pool;
  a.topk = s.topk;
  a.kmax = s.topk;
  a.split = attn_split(s);
  a.nsplit = attn_nsplit(s);
  const size_t n = (size_t)nseg * a.nsplit * G;
  a.part_ml = reinterpret_cast<float2 *>(w.attn);
  a.part_acc = reinterpret_cast<float *>(w.attn + align_up(n * sizeof(float2), 256));
  return a;
}

hipError_t launch_attn_slots(const AttnArgs &a, int G, int dtype, int nseg, int slot0, int nslots,
                             hipStream_t st) {
  if (nslots <= 0) return hipSuccess;
  dim3 grid(nslots, nseg);
  hipError_t e;
  switch (G) {
    case 1: e = dispatch_g<1>(grid, st, a, dtype, a.pool, slot0); break;
    case 2: e = dispatch_g<2>(grid, st, a, dtype, a.pool, slot0); break;
    case 3: e = dispatch_g<3>(grid, st, a, dtype, a.pool, slot0); break;
    case 4: e = dispatch_g<4>(grid, st, a, dtype, a.pool, slot0); break;
    case 5: e = dispatch_g<5>(grid, st, a, dtype, a.pool, slot0); break;
    case 6: e = dispatch_g<6>(grid, st, a, dtype, a.pool, slot0); break;
    case 7: e = dispatch_g<7>(grid, st, a, dtype, a.pool, slot0); break;
    case 8: e = dispatch_g<8>(grid, st, a, dtype, a.pool, slot0); break;
    default: return hipErrorInvalidValue;
  }
  return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_attn_merge(const AttnArgs &a, int G, int nseg, float *out, float *lse,
                             hipStream_t st, int32_t *zero, long nzero) {
  attn_merge_kernel<<<dim3(nseg, G), dim3(D, merge_parts(a.nsplit)), 0, st>>>(
      a.part_ml, a.part_acc, a.nsplit, G, a.Hkv, out, lse, zero, nzero);
  return hipGetLastError();
}

hipError_t launch_attn(const uint16_t *q, int Hq, const sks_kv &kv, const Shape &s,
                       const int32_t *idx, const uint16_t *Kp, const uint16_t *Vp,
                       float sm_scale, float *out, float *lse, const TopkWs &w, hipStream_t st,
                       bool dense, int32_t *zero, long nzero) {
  const int G = Hq / s.Hkv;
  const int nseg = s.B * s.R * s.Hkv;
  AttnArgs a = attn_args(q, Hq, kv, s, idx, Kp, Vp, sm_scale, w);
  if (dense) {
    // no selection: one softmax over the last window + topk tokens of each
    // row (all of them when L_i <= window + topk); the attention set is then
    // at most window + topk + pool - 1 entries, the sparse step's bound, so
    // the split count and the workspace stay those of the sparse step
    a.window = s.window + s.topk;
    a.kmax = 0;
  }
  hipError_t e = launch_attn_slots(a, G, s.dtype, nseg, 0, a.nsplit, st);
  if (e != hipSuccess) return e;
  return launch_attn_merge(a, G, nseg, out, lse, st, zero, nzero);
}

}  // namespace sks
