// Key and query sketch kernels.
//
// Key sketch: the rank-64 "key sketch" of the claims list and the "build the
// sketch" kernel of "What it took" on the page "8 agents x 250K context,
// concurrently, on two 3090s"; the frozen basis is the "frozen sketch basis
// (one file)" of the same list.  Pooled mode: the 4:1 mean-pooled far field
// of "What it adds" on the "Agens SGLang" README.
//
// Layout: one lane per token (or pooled block).  The lane holds its key in
// 128 fp32 registers and walks the 64 basis rows; basis addresses are uniform
// across the wave, so they come through scalar loads.  The 64 int8 codes of
// a lane are staged in LDS and leave as one contiguous, coalesced block.
#include "sks_internal.h"

namespace sks {
namespace {

constexpr int KS_THREADS = 256;
constexpr int SMALL_ROWS = 64;   // up to this many rows per (b, h): wave-per-row kernel

// Project x (128 fp32 in registers) on the 64 basis rows and quantize.
// Codes are written into the LDS row `dst` (64 bytes, 16 dwords).
__device__ __forceinline__ void project_quantize(const float (&x)[D], const float *__restrict__ P,
                                                 float scale, uint32_t *dst) {
#pragma unroll 1
  for (int c4 = 0; c4 < RANK / 4; ++c4) {
    uint32_t packed = 0;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const float *row = P + (c4 * 4 + cc) * D;
      float acc = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(row[d], x[d], acc);
      packed |= (uint32_t)(uint8_t)quant_code(acc, scale) << (8 * cc);
    }
    dst[c4] = packed;
  }
}

// Load the key row of token t into fp32 registers (bf16 or int8 * fp16 scale).
template <int DT>
__device__ __forceinline__ void load_key(const void *K, const uint16_t *Ks, size_t row,
                                         float (&x)[D]) {
  if (DT == SKS_KV_BF16) {
    const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(K) + row * D);
#pragma unroll
    for (int v = 0; v < D / 8; ++v) {
      uint4 w = src[v];
      x[v * 8 + 0] = bf16_lo(w.x); x[v * 8 + 1] = bf16_hi(w.x);
      x[v * 8 + 2] = bf16_lo(w.y); x[v * 8 + 3] = bf16_hi(w.y);
      x[v * 8 + 4] = bf16_lo(w.z); x[v * 8 + 5] = bf16_hi(w.z);
      x[v * 8 + 6] = bf16_lo(w.w); x[v * 8 + 7] = bf16_hi(w.w);
    }
  } else {
    const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const int8_t *>(K) + row * D);
    float sc = f16_bits_to_float(Ks[row]);
#pragma unroll
    for (int v = 0; v < D / 16; ++v) {
      uint4 w = src[v];
      uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
          x[v * 16 + k * 4 + bb] = (float)(int8_t)(ws[k] >> (8 * bb)) * sc;   // exact
    }
  }
}

// Copy the staged code rows [0, n) of this workgroup to S rows [j0, j0 + n).
__device__ __forceinline__ void flush_codes(const uint32_t *lds, int n, int8_t *S, size_t row0) {
  uint4 *dst = reinterpret_cast<uint4 *>(S + row0 * RANK);
  const uint4 *src = reinterpret_cast<const uint4 *>(lds);
  for (int v = threadIdx.x; v < n * (RANK / 16); v += blockDim.x) dst[v] = src[v];
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

template <int DT>
__global__ __launch_bounds__(KS_THREADS) void sketch_keys_kernel(
    const void *__restrict__ K, const uint16_t *__restrict__ Ks, const int32_t *__restrict__ seq_len,
    const float *__restrict__ basis, int basis_per_head, const float *__restrict__ key_scale,
    int Hkv, int T_max, int R, int NB, int append, int t_begin, int t_end,
    int8_t *__restrict__ S) {
  __shared__ uint32_t codes[KS_THREADS * (RANK / 4)];
  const int bh = blockIdx.y, b = bh / Hkv, h = bh % Hkv;
  int j_lo, j_hi;
  sketch_range(append, seq_len, b, T_max, R, 1, NB, t_begin, t_end, j_lo, j_hi);
  const int j0 = j_lo + blockIdx.x * KS_THREADS;
  if (j0 >= j_hi) return;
  const int n = min(KS_THREADS, j_hi - j0);
  const int t = j0 + threadIdx.x;
  const float *P = basis + (basis_per_head ? (size_t)h * RANK * D : 0);
  const float scale = key_scale[h];
  if (threadIdx.x < n) {
    float x[D];
    load_key<DT>(K, Ks, (size_t)bh * T_max + t, x);
    project_quantize(x, P, scale, &codes[threadIdx.x * (RANK / 4)]);
  }
  __syncthreads();
  flush_codes(codes, n, S, (size_t)bh * NB + j0);
}

// Pooled blocks (bf16 caches): mean of `pool` consecutive K and V rows in
// fp64 (exact for bf16 inputs), rounded once to bf16; the sketch is taken of
// the stored bf16 pooled key.
__global__ __launch_bounds__(KS_THREADS) void sketch_pool_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ seq_len, const float *__restrict__ basis, int basis_per_head,
    const float *__restrict__ key_scale, int Hkv, int T_max, int R, int NB, int pool, int append,
    int t_begin, int t_end, int8_t *__restrict__ S, uint16_t *__restrict__ Kp,
    uint16_t *__restrict__ Vp) {
  __shared__ uint32_t codes[KS_THREADS * (RANK / 4)];
  const int bh = blockIdx.y, b = bh / Hkv, h = bh % Hkv;
  int j_lo, j_hi;
  sketch_range(append, seq_len, b, T_max, R, pool, NB, t_begin, t_end, j_lo, j_hi);
  const int j0 = j_lo + blockIdx.x * KS_THREADS;
  if (j0 >= j_hi) return;
  const int n = min(KS_THREADS, j_hi - j0);
  const int j = j0 + threadIdx.x;
  const float *P = basis + (basis_per_head ? (size_t)h * RANK * D : 0);
  const float scale = key_scale[h];
  if (threadIdx.x < n) {
    const size_t tok0 = (size_t)bh * T_max + (size_t)j * pool;
    const size_t out_row = (size_t)bh * NB + j;
    const double dpool = (double)pool;
    float x[D];
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const uint16_t *src = which == 0 ? K : V;
      uint16_t *dst = which == 0 ? Kp : Vp;
#pragma unroll
      for (int v = 0; v < D / 8; ++v) {
        double s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int k = 0; k < pool; ++k) {
          uint4 w = *reinterpret_cast<const uint4 *>(src + (tok0 + k) * D + v * 8);
          s[0] += bf16_lo(w.x); s[1] += bf16_hi(w.x); s[2] += bf16_lo(w.y); s[3] += bf16_hi(w.y);
          s[4] += bf16_lo(w.z); s[5] += bf16_hi(w.z); s[6] += bf16_lo(w.w); s[7] += bf16_hi(w.w);
        }
        uint16_t o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[e] = f64_to_bf16_rne(s[e] / dpool);   // exact sum, one rounding, then bf16
          if (which == 0) x[v * 8 + e] = __uint_as_float((uint32_t)o[e] << 16);
        }
        uint4 packed;
        packed.x = o[0] | ((uint32_t)o[1] << 16);
        packed.y = o[2] | ((uint32_t)o[3] << 16);
        packed.z = o[4] | ((uint32_t)o[5] << 16);
        packed.w = o[6] | ((uint32_t)o[7] << 16);
        *reinterpret_cast<uint4 *>(dst + out_row * D + v * 8) = packed;
      }
    }
    project_quantize(x, P, scale, &codes[threadIdx.x * (RANK / 4)]);
  }
  __syncthreads();
  flush_codes(codes, n, S, (size_t)bh * NB + j0);
}

// Few rows per (b, h) -- the per-step append of the rows' own tokens: one
// wave per sketch row.  The 128-element key (or pooled block) is staged in
// LDS, lane c dots basis row c with it, so the latency is that of one row
// instead of one lane walking all 64 x 128 products.
template <int DT>
__device__ void sketch_row_wave(const void *__restrict__ K, const void *__restrict__ V,
                                const uint16_t *__restrict__ Ks,
                                const int32_t *__restrict__ seq_len,
                                const float *__restrict__ basis, int basis_per_head,
                                const float *__restrict__ key_scale, int Hkv, int T_max, int R,
                                int NB, int pool, int append, int t_begin, int t_end,
                                int8_t *__restrict__ S, uint16_t *__restrict__ Kp,
                                uint16_t *__restrict__ Vp, int bh, int jx) {
  __shared__ float x[D];
  const int b = bh / Hkv, h = bh % Hkv;
  int j_lo, j_hi;
  sketch_range(append, seq_len, b, T_max, R, pool, NB, t_begin, t_end, j_lo, j_hi);
  const int j = j_lo + jx;
  if (j >= j_hi) return;
  const int lane = threadIdx.x;
  if (pool == 1) {
    const size_t row = (size_t)bh * T_max + j;
    float x0, x1;
    if (DT == SKS_KV_BF16) {
      const uint32_t w = reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(K) + row * D)[lane];
      x0 = bf16_lo(w);
      x1 = bf16_hi(w);
    } else {
      const uint16_t w = reinterpret_cast<const uint16_t *>(static_cast<const int8_t *>(K) + row * D)[lane];
      const float sc = f16_bits_to_float(Ks[row]);
      x0 = (float)(int8_t)(w & 0xff) * sc;
      x1 = (float)(int8_t)(w >> 8) * sc;
    }
    x[2 * lane] = x0;
    x[2 * lane + 1] = x1;
  } else {
    // pooled block: fp64 mean of `pool` rows (exact for bf16), rounded once to bf16
    const size_t tok0 = (size_t)bh * T_max + (size_t)j * pool;
    const size_t out_row = (size_t)bh * NB + j;
    const double dpool = (double)pool;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const uint16_t *src = static_cast<const uint16_t *>(which == 0 ? K : V);
      double s0 = 0.0, s1 = 0.0;
      for (int k = 0; k < pool; ++k) {
        const uint32_t w = reinterpret_cast<const uint32_t *>(src + (tok0 + k) * D)[lane];
        s0 += bf16_lo(w);
        s1 += bf16_hi(w);
      }
      const uint16_t o0 = f64_to_bf16_rne(s0 / dpool), o1 = f64_to_bf16_rne(s1 / dpool);
      reinterpret_cast<uint32_t *>((which == 0 ? Kp : Vp) + out_row * D)[lane] =
          (uint32_t)o0 | ((uint32_t)o1 << 16);
      if (which == 0) {
        x[2 * lane] = __uint_as_float((uint32_t)o0 << 16);
        x[2 * lane + 1] = __uint_as_float((uint32_t)o1 << 16);
      }
    }
  }
  __syncthreads();
  const float *Prow = basis + (basis_per_head ? (size_t)h * RANK * D : 0) + (size_t)lane * D;
  float y = 0.f;
#pragma unroll 8
  for (int d = 0; d < D; ++d) y = __builtin_fmaf(Prow[d], x[d], y);
  S[((size_t)bh * NB + j) * RANK + lane] = quant_code(y, key_scale[h]);
}

template <int DT>
__global__ __launch_bounds__(64) void sketch_rows_small_kernel(
    const void *__restrict__ K, const void *__restrict__ V, const uint16_t *__restrict__ Ks,
    const int32_t *__restrict__ seq_len, const float *__restrict__ basis, int basis_per_head,
    const float *__restrict__ key_scale, int Hkv, int T_max, int R, int NB, int pool, int append,
    int t_begin, int t_end, int8_t *__restrict__ S, uint16_t *__restrict__ Kp,
    uint16_t *__restrict__ Vp) {
  sketch_row_wave<DT>(K, V, Ks, seq_len, basis, basis_per_head, key_scale, Hkv, T_max, R, NB, pool,
                      append, t_begin, t_end, S, Kp, Vp, blockIdx.y, blockIdx.x);
}

// Query sketch: one wave per (b, i, h).  qbar = mean of the group's queries
// (fp32), y = P qbar by lane c, absmax over the wave, codes by lane c.
__device__ void sketch_query_wave(const uint16_t *__restrict__ q, int R, int Hq, int Hkv,
                                  const float *__restrict__ basis, int basis_per_head,
                                  int8_t *__restrict__ qsk, float *__restrict__ qscale, int seg) {
  __shared__ float qbar[D];                    // seg = (b * R + i) * Hkv + h
  const int h = seg % Hkv, bi = seg / Hkv;
  const int g = Hq / Hkv;
  const int lane = threadIdx.x;
  const uint16_t *qg = q + ((size_t)bi * Hq + (size_t)h * g) * D;
  float s0 = 0.f, s1 = 0.f;
  for (int j = 0; j < g; ++j) {
    uint32_t w = *reinterpret_cast<const uint32_t *>(qg + (size_t)j * D + 2 * lane);
    s0 += bf16_lo(w);
    s1 += bf16_hi(w);
  }
  qbar[2 * lane] = s0 / (float)g;
  qbar[2 * lane + 1] = s1 / (float)g;
  __syncthreads();
  const float *Prow = basis + (basis_per_head ? (size_t)h * RANK * D : 0) + (size_t)lane * D;
  float y = 0.f;
  for (int d = 0; d < D; ++d) y = __builtin_fmaf(Prow[d], qbar[d], y);
  float amax = fabsf(y);
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  float scale = amax / 127.0f;
  int8_t code = amax > 0.f ? quant_code(y, scale) : (int8_t)0;
  qsk[(size_t)seg * RANK + lane] = code;
  if (lane == 0 && qscale) qscale[seg] = amax > 0.f ? scale : 0.f;
}

__global__ __launch_bounds__(64) void sketch_query_kernel(
    const uint16_t *__restrict__ q, int R, int Hq, int Hkv, const float *__restrict__ basis,
    int basis_per_head, int8_t *__restrict__ qsk, float *__restrict__ qscale) {
  sketch_query_wave(q, R, Hq, Hkv, basis, basis_per_head, qsk, qscale, blockIdx.x);
}

// The step prologue in one launch: workgroups [0, nq) sketch the queries,
// the rest the rows' own tokens (append), nrows per (b, h).
template <int DT>
__global__ __launch_bounds__(64) void step_prologue_kernel(
    const uint16_t *__restrict__ q, int Hq, const void *__restrict__ K,
    const void *__restrict__ V, const uint16_t *__restrict__ Ks,
    const int32_t *__restrict__ seq_len, const float *__restrict__ basis, int basis_per_head,
    const float *__restrict__ key_scale, int Hkv, int T_max, int R, int NB, int pool, int nq,
    int nrows, int8_t *__restrict__ qsk, float *__restrict__ qscale, int8_t *__restrict__ S,
    uint16_t *__restrict__ Kp, uint16_t *__restrict__ Vp) {
  if ((int)blockIdx.x < nq) {
    sketch_query_wave(q, R, Hq, Hkv, basis, basis_per_head, qsk, qscale, blockIdx.x);
    return;
  }
  const int w = blockIdx.x - nq;
  sketch_row_wave<DT>(K, V, Ks, seq_len, basis, basis_per_head, key_scale, Hkv, T_max, R, NB, pool,
                      1, 0, 0, S, Kp, Vp, w / nrows, w % nrows);
}

}  // namespace

hipError_t launch_sketch_keys(const sks_kv &kv, const Shape &s, const float *basis,
                              int basis_per_head, const float *key_scale, int t_begin,
                              int t_end, int8_t *S, uint16_t *Kp, uint16_t *Vp,
                              hipStream_t st) {
  const int append = t_begin == SKS_APPEND;
  // rows touched per (b, h): bounded by R (+1 block) in append mode
  long span = append ? (long)s.R + s.pool : (long)t_end - (long)t_begin;
  if (span <= 0) return hipSuccess;
  long nrows = s.pool == 1 ? span : span / s.pool + 1;
  if (nrows > s.NB) nrows = s.NB;
  if (nrows <= SMALL_ROWS) {
    // few rows per (b, h): one wave per row
    dim3 g2((unsigned)nrows, s.B * s.Hkv);
    if (s.dtype == SKS_KV_BF16)
      sketch_rows_small_kernel<SKS_KV_BF16><<<g2, 64, 0, st>>>(
          kv.K, kv.V, nullptr, kv.seq_len, basis, basis_per_head, key_scale, s.Hkv, s.T_max, s.R,
          s.NB, s.pool, append, t_begin, t_end, S, Kp, Vp);
    else
      sketch_rows_small_kernel<SKS_KV_I8><<<g2, 64, 0, st>>>(
          kv.K, kv.V, kv.K_scale, kv.seq_len, basis, basis_per_head, key_scale, s.Hkv, s.T_max,
          s.R, s.NB, s.pool, append, t_begin, t_end, S, Kp, Vp);
    return hipGetLastError();
  }
  dim3 grid(ceil_div(nrows, KS_THREADS), s.B * s.Hkv);
  if (s.pool == 1) {
    if (s.dtype == SKS_KV_BF16)
      sketch_keys_kernel<SKS_KV_BF16><<<grid, KS_THREADS, 0, st>>>(
          kv.K, nullptr, kv.seq_len, basis, basis_per_head, key_scale, s.Hkv, s.T_max, s.R,
          s.NB, append, t_begin, t_end, S);
    else
      sketch_keys_kernel<SKS_KV_I8><<<grid, KS_THREADS, 0, st>>>(
          kv.K, kv.K_scale, kv.seq_len, basis, basis_per_head, key_scale, s.Hkv, s.T_max, s.R,
          s.NB, append, t_begin, t_end, S);
  } else {
    sketch_pool_kernel<<<grid, KS_THREADS, 0, st>>>(
        static_cast<const uint16_t *>(kv.K), static_cast<const uint16_t *>(kv.V), kv.seq_len,
        basis, basis_per_head, key_scale, s.Hkv, s.T_max, s.R, s.NB, s.pool, append, t_begin,
        t_end, S, Kp, Vp);
  }
  return hipGetLastError();
}

hipError_t launch_step_prologue(const uint16_t *q, int Hq, const sks_kv &kv, const Shape &s,
                                const float *basis, int basis_per_head, const float *key_scale,
                                int8_t *qsk, float *qscale, int8_t *S, uint16_t *Kp, uint16_t *Vp,
                                hipStream_t st) {
  // append rows per (b, h), as in launch_sketch_keys' append mode
  long nrows = s.pool == 1 ? (long)s.R : ((long)s.R + s.pool) / s.pool + 1;
  if (nrows > s.NB) nrows = s.NB;
  if (nrows > SMALL_ROWS) return hipErrorInvalidValue;
  const int nq = s.B * s.R * s.Hkv;
  const unsigned grid = (unsigned)(nq + nrows * s.B * s.Hkv);
  if (s.dtype == SKS_KV_BF16)
    step_prologue_kernel<SKS_KV_BF16><<<grid, 64, 0, st>>>(
        q, Hq, kv.K, kv.V, nullptr, kv.seq_len, basis, basis_per_head, key_scale, s.Hkv, s.T_max,
        s.R, s.NB, s.pool, nq, (int)nrows, qsk, qscale, S, Kp, Vp);
  else
    step_prologue_kernel<SKS_KV_I8><<<grid, 64, 0, st>>>(
        q, Hq, kv.K, kv.V, kv.K_scale, kv.seq_len, basis, basis_per_head, key_scale, s.Hkv,
        s.T_max, s.R, s.NB, s.pool, nq, (int)nrows, qsk, qscale, S, Kp, Vp);
  return hipGetLastError();
}

hipError_t launch_sketch_query(const uint16_t *q, int B, int R, int Hq, int Hkv,
                               const float *basis, int basis_per_head, int8_t *qsk,
                               float *qscale, hipStream_t st) {
  sketch_query_kernel<<<B * R * Hkv, 64, 0, st>>>(q, R, Hq, Hkv, basis, basis_per_head, qsk,
                                                  qscale);
  return hipGetLastError();
}

}  // namespace sks
