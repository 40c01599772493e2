// Device code of the per-step sketches, each computed by one workgroup of
// SK_THREADS threads: the query sketch of one (sequence, row, KV head) and
// the key sketch of one cached row or pooled block (the append of a step's
// own tokens, or a short range).  Key sketch: the rank-64 key sketch of the
// claims list and the "build the sketch" kernels of "What it took" on the page
// "8 agents x 250K context, concurrently, on two 3090s"; pooled blocks: the
// 4:1 mean-pooled far field of "What it adds" on the "Agens SGLang" README.
//
// The 64 x 128 products of y = P x: thread t takes basis row c = t / 4 over
// the dims 32 (t % 4) .. + 32 (its 32 basis values load first, in 8 float4,
// so they overlap the loads of x), and a quad sum adds the four parts.
#pragma once

#include "sks_internal.h"
#include "tier.h"

namespace sks {

constexpr int SK_THREADS = 256;

struct SketchLds {
  __align__(16) float x[D];             // the vector being sketched
  float red[SK_THREADS / 64];
};

namespace {

static_assert(SK_THREADS == 4 * RANK, "four threads per basis row");

// Key code from y and the reciprocal of the frozen key scale, computed once:
// a multiply instead of an IEEE division per code (equal to rne(y / scale)
// whenever 1/scale is exact, e.g. for a power-of-two scale; otherwise a code
// can differ only where y / scale lies within an ulp of a rounding boundary).
// The bulk build and the per-step append use the same form.
__device__ __forceinline__ int8_t key_code(float y, float inv_scale) {
  float v = __builtin_rintf(y * inv_scale);
  v = fminf(fmaxf(v, -127.0f), 127.0f);
  return (int8_t)(int)v;
}

// First sketch row of the range handled by this (b, h): host range or append.
__device__ __forceinline__ void sketch_range(int append, const int32_t *seq_len, int b, int T_max,
                                             int R, int pool, int NB, int t_begin, int t_end,
                                             int &j_lo, int &j_hi) {
  int lo = t_begin, hi = t_end;
  if (append) {
    int L0 = clamp_len(seq_len[b], T_max, R);
    lo = L0 - 1;
    hi = L0 - 1 + R;
    if (lo < 0) lo = 0;
  }
  lo = lo < 0 ? 0 : (lo > T_max ? T_max : lo);
  hi = hi < lo ? lo : (hi > T_max ? T_max : hi);
  j_lo = lo / pool;                       // blocks whose last token is in [lo, hi)
  j_hi = hi / pool;
  if (j_hi > NB) j_hi = NB;
}

// This thread's 32 basis values: row t / 4, dims 32 (t % 4) .. + 32 of the
// basis of the KV head (basis_h points at it).
__device__ __forceinline__ void load_basis_part(const float *__restrict__ basis_h, float4 (&pr)[8]) {
  const int t = threadIdx.x;
  const float4 *src = reinterpret_cast<const float4 *>(basis_h + (size_t)(t >> 2) * D + 32 * (t & 3));
#pragma unroll
  for (int k = 0; k < 8; ++k) pr[k] = src[k];
}

// (P x)_c for c = t / 4: this thread's 32 products in dim order, then the
// quad sum (every lane of the quad gets the same value).
__device__ __forceinline__ float dot_basis_part(const float4 (&pr)[8], const float *x) {
  const float4 *xv = reinterpret_cast<const float4 *>(x + 32 * (threadIdx.x & 3));
  float y = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float4 v = xv[k];
    y = __builtin_fmaf(pr[k].x, v.x, y);
    y = __builtin_fmaf(pr[k].y, v.y, y);
    y = __builtin_fmaf(pr[k].z, v.z, y);
    y = __builtin_fmaf(pr[k].w, v.w, y);
  }
  y += dpp_f<DPP_QUAD_XOR1>(y);
  y += dpp_f<DPP_QUAD_XOR2>(y);
  return y;
}

// Query sketch of segment seg = (b * R + i) * Hkv + h, by the whole
// workgroup: qbar = mean of the group's g query vectors (fp32, summed in head
// order), y = P_h qbar, qscale = max|y| / 127, codes = clamp(rne(y / qscale))
// (all zero, scale 0, when y == 0).  Writes the 64 codes to `codes` (global
// memory or LDS) and the scale to *qscale when qscale is not NULL.  Contains
// two __syncthreads().  `between` runs (in every thread) once the basis and
// the first eight query heads are loading and before they are used: loads it
// issues complete behind them.
template <typename F>
__device__ void block_query_sketch(const uint16_t *__restrict__ q, int R, int Hq, int Hkv,
                                   const float *__restrict__ basis, int basis_per_head, int seg,
                                   int8_t *codes, float *qscale, SketchLds &L, F &&between) {
  const int h = seg % Hkv, bi = seg / Hkv;
  const int g = Hq / Hkv;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  float4 pr[8];
  load_basis_part(basis + (basis_per_head ? (size_t)h * RANK * D : 0), pr);
  // dims 2t, 2t + 1 of the group's queries (threads t < 64), eight heads in
  // flight, loaded unconditionally (past the group: its last head again, not
  // summed)
  const uint16_t *qg = q + ((size_t)bi * Hq + (size_t)h * g) * D;
  const bool qt = t < D / 2;
  uint32_t w[8];
  if (qt) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      w[u] = *reinterpret_cast<const uint32_t *>(qg + (size_t)min(u, g - 1) * D + 2 * t);
  }
  between();
  if (qt) {
    float s0 = 0.f, s1 = 0.f;
    for (int j0 = 0; j0 < g; j0 += 8) {
      if (j0 > 0) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          w[u] = *reinterpret_cast<const uint32_t *>(qg + (size_t)min(j0 + u, g - 1) * D + 2 * t);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < g) {
          s0 += bf16_lo(w[u]);
          s1 += bf16_hi(w[u]);
        }
    }
    L.x[2 * t] = s0 / (float)g;
    L.x[2 * t + 1] = s1 / (float)g;
  }
  __syncthreads();
  const float y = dot_basis_part(pr, L.x);
  float amax = fabsf(y);
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  if (lane == 0) L.red[wave] = amax;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < SK_THREADS / 64; ++w) amax = fmaxf(amax, L.red[w]);
  const float scale = amax / 127.0f;
  if ((t & 3) == 0) codes[t >> 2] = amax > 0.f ? quant_code(y, scale) : (int8_t)0;
  if (t == 0 && qscale) *qscale = amax > 0.f ? scale : 0.f;
}
__device__ __forceinline__ void block_query_sketch(const uint16_t *__restrict__ q, int R, int Hq,
                                                   int Hkv, const float *__restrict__ basis,
                                                   int basis_per_head, int seg, int8_t *codes,
                                                   float *qscale, SketchLds &L) {
  block_query_sketch(q, R, Hq, Hkv, basis, basis_per_head, seg, codes, qscale, L, [] {});
}

// Key sketch of sketch row j_lo + jx of (b, h) = (bh / Hkv, bh % Hkv), by the
// whole workgroup (returns at once, uniformly, past the range).  pool == 1:
// the (dequantised) key of token j, read from the hot ring Kh in append mode
// (slot = position % W_hot; the full cache itself when there is no hot tier);
// pool > 1 (bf16): the fp64 mean of the block's pool K and V rows (exact
// sums, added in row order), rounded once to bf16 and stored in Kp / Vp, and
// the sketch of that stored mean.  Contains one __syncthreads().
template <int DT>
__device__ void block_key_row(const void *__restrict__ K, const void *__restrict__ V,
                              const uint16_t *__restrict__ Ks, const void *__restrict__ Kh,
                              const uint16_t *__restrict__ Ksh, int W_hot,
                              const int32_t *__restrict__ seq_len, const float *__restrict__ basis,
                              int basis_per_head, const float *__restrict__ key_scale, int Hkv,
                              int T_max, int R, int NB, int pool, int append, int t_begin,
                              int t_end, int8_t *__restrict__ S, uint16_t *__restrict__ Kp,
                              uint16_t *__restrict__ Vp, int bh, int jx, SketchLds &L) {
  const int b = bh / Hkv, h = bh % Hkv;
  int j_lo, j_hi;
  sketch_range(append, seq_len, b, T_max, R, pool, NB, t_begin, t_end, j_lo, j_hi);
  const int j = j_lo + jx;
  if (j >= j_hi) return;
  const int t = threadIdx.x;
  float4 pr[8];
  load_basis_part(basis + (basis_per_head ? (size_t)h * RANK * D : 0), pr);
  if (t < D / 2) {                       // dims 2t, 2t + 1
    if (pool == 1) {
      if (append) {
        K = Kh;
        Ks = Ksh;
      }
      const size_t row = append ? (size_t)bh * W_hot + hot_slot(j, W_hot) : (size_t)bh * T_max + j;
      float x0, x1;
      if (DT == SKS_KV_BF16) {
        const uint32_t w = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(K) + row * D)[t];
        x0 = bf16_lo(w);
        x1 = bf16_hi(w);
      } else if (DT == SKS_KV_I4) {
        const uint32_t w = (static_cast<const uint8_t *>(K) + row * (D / 2))[t];
        const float sc = f16_bits_to_float(Ks[row]);
        x0 = (float)((int32_t)(w << 28) >> 28) * sc;
        x1 = (float)((int32_t)(w << 24) >> 28) * sc;
      } else {
        const uint16_t w = reinterpret_cast<const uint16_t *>(static_cast<const int8_t *>(K) + row * D)[t];
        const float sc = f16_bits_to_float(Ks[row]);
        x0 = (float)(int8_t)(w & 0xff) * sc;
        x1 = (float)(int8_t)(w >> 8) * sc;
      }
      L.x[2 * t] = x0;
      L.x[2 * t + 1] = x1;
    } else {
      // pooled block: the K and V rows are loaded 8 at a time, all in flight
      // together, and summed in row order
      const size_t tok0 = (size_t)bh * T_max + (size_t)j * pool;
      const size_t out_row = (size_t)bh * NB + j;
      const double dpool = (double)pool;
      const uint32_t *Kw = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(K) + tok0 * D) + t;
      const uint32_t *Vw = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(V) + tok0 * D) + t;
      double k0s = 0.0, k1s = 0.0, v0s = 0.0, v1s = 0.0;
      for (int k0 = 0; k0 < pool; k0 += 8) {
        uint32_t wk[8], wv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const bool in = k0 + u < pool;
          wk[u] = in ? Kw[(size_t)(k0 + u) * (D / 2)] : 0u;
          wv[u] = in ? Vw[(size_t)(k0 + u) * (D / 2)] : 0u;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (k0 + u < pool) {
            k0s += bf16_lo(wk[u]);
            k1s += bf16_hi(wk[u]);
            v0s += bf16_lo(wv[u]);
            v1s += bf16_hi(wv[u]);
          }
      }
      const uint16_t o0 = f64_to_bf16_rne(k0s / dpool), o1 = f64_to_bf16_rne(k1s / dpool);
      const uint16_t p0 = f64_to_bf16_rne(v0s / dpool), p1 = f64_to_bf16_rne(v1s / dpool);
      reinterpret_cast<uint32_t *>(Kp + out_row * D)[t] = (uint32_t)o0 | ((uint32_t)o1 << 16);
      reinterpret_cast<uint32_t *>(Vp + out_row * D)[t] = (uint32_t)p0 | ((uint32_t)p1 << 16);
      L.x[2 * t] = __uint_as_float((uint32_t)o0 << 16);
      L.x[2 * t + 1] = __uint_as_float((uint32_t)o1 << 16);
    }
  }
  __syncthreads();
  const float y = dot_basis_part(pr, L.x);
  if ((t & 3) == 0) S[((size_t)bh * NB + j) * RANK + (t >> 2)] = key_code(y, 1.0f / key_scale[h]);
}

}  // namespace
}  // namespace sks
