// Key and query sketch kernels.
//
// Key sketch: the rank-64 "key sketch" of the claims list and the "build the
// sketch" kernel of "What it took" on the page "8 agents x 250K context,
// concurrently, on two 3090s"; the frozen basis is the "frozen sketch basis
// (one file)" of the same list.  Pooled mode: the 4:1 mean-pooled far field
// of "What it adds" on the "Agens SGLang" README.
//
// Bulk builds run on the matrix cores (sketch_mfma_kernel, below); the few
// rows of a step's append take one workgroup per row (sketch_rows_small_kernel,
// sketch_body.h).
#include "sks_internal.h"
#include "refit.h"
#include "sketch_body.h"
#include "tier.h"

namespace sks {
namespace {

constexpr int SMALL_ROWS = 64;   // up to this many rows per (b, h): workgroup-per-row kernel

// int8 code pair (bits sh .. sh+15 of w) -> two bf16 (exact: |code| <= 127)
__device__ __forceinline__ uint32_t i8pair_bf16(uint32_t w, int sh) {
  const float a = (float)(int8_t)(w >> sh), b = (float)(int8_t)(w >> (sh + 8));
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}

// int4 codes (eight two's-complement nibbles of w, low nibble first) -> four
// bf16 pairs, exactly; out[p] holds dims 2p, 2p + 1
typedef uint32_t sk_u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ sk_u32x4_t i4x8_bf16(uint32_t w) {
  sk_u32x4_t o;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float a = (float)((int32_t)(w << (28 - 8 * p)) >> 28);
    const float b = (float)((int32_t)(w << (24 - 8 * p)) >> 28);
    o[p] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
  }
  return o;
}

// Bytes of one cached K row.
template <int DT>
constexpr int row_bytes() {
  return DT == SKS_KV_BF16 ? 2 * D : DT == SKS_KV_I8 ? D : D / 2;
}

// ---------------------------------------------------------------------------
// Bulk sketch on the matrix cores.  Per (b, h), Y[rows][64] = X[rows][128] P^T:
// v_mfma_f32_16x16x32_bf16 with A = 16 rows x 32 dims of X (lane (n, g): row
// n, dims 32c + 8g .. +8 of step c; int4 rows take dims 32g + 8c .. +8, so
// that one 16-byte load holds a lane's four steps) and B = 32 dims x 16
// basis rows (block nb, lane: basis row 4n + nb, the same dims).  X is exact
// in bf16 (bf16 rows; int8 and int4 codes, whose fp16 row scale multiplies Y
// afterwards).  The fp32 basis is split exactly into three bf16 parts, P =
// hi + mid + lo (8 + 8 + 8 significant bits), so every product is exact and
// only the fp32 accumulation rounds -- the same accuracy as an fp32 dot
// product.  The split basis sits in LDS in operand order; a lane's four
// codes of a row are staged as one word per wave and leave as 16-byte stores.
constexpr int SM_THREADS = 256;
constexpr int SM_TILE = 64;                              // rows per wave and iteration
constexpr int SM_ITERS = 16;
constexpr int SM_ROWS = SM_TILE * (SM_THREADS / 64) * SM_ITERS;   // 4096 rows per workgroup

typedef __bf16 sk_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float sk_f32x4_t __attribute__((ext_vector_type(4)));

// first of the 8 dims of MFMA step c held by lane group g
template <int DT>
__device__ __forceinline__ int sm_dim(int c, int g) {
  return DT == SKS_KV_I4 ? 32 * g + 8 * c : 32 * c + 8 * g;
}

__device__ __forceinline__ sk_f32x4_t sk_mfma(sk_u32x4_t a, sk_u32x4_t b, sk_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sk_bf16x8_t, a),
                                                 __builtin_bit_cast(sk_bf16x8_t, b), c, 0, 0, 0);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t sk_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// component `part` (0 hi, 1 mid, 2 lo) of the exact three-way bf16 split
__device__ __forceinline__ uint32_t sk_split(float p, int part) {
  const uint32_t hi = sk_bf16(p);
  if (part == 0) return hi;
  const float r1 = p - __uint_as_float(hi << 16);           // exact
  const uint32_t mid = sk_bf16(r1);
  if (part == 1) return mid;
  return sk_bf16(r1 - __uint_as_float(mid << 16));          // exact remainder, <= 8 bits
}

// AMAX: instead of codes, the largest |y| over the rows [t_begin, min(t_end,
// seq_len[b])) (the key-scale pass of a basis refit); each workgroup writes
// its maximum to amax[blockIdx.y * gridDim.x + blockIdx.x] (0 if it has no
// rows).  Rows past the range are clamped copies of its last row, which
// leave the maximum unchanged.
template <int DT, bool AMAX = false>
__global__ __launch_bounds__(SM_THREADS, 2) void sketch_mfma_kernel(
    const void *__restrict__ X, const uint16_t *__restrict__ Xs, long x_rows_per_bh,
    const int32_t *__restrict__ seq_len, const float *__restrict__ basis, int basis_per_head,
    const float *__restrict__ key_scale, int Hkv, int T_max, int R, int NB, int pool,
    int append, int t_begin, int t_end, int8_t *__restrict__ S, float *__restrict__ amax = nullptr) {
  __shared__ sk_u32x4_t bop[3][4][4][64];                   // [part][basis block][step][lane]
  __shared__ __align__(16) uint8_t stage[SM_THREADS / 64][SM_TILE * RANK];
  const int bh = blockIdx.y, b = bh / Hkv, h = bh % Hkv;
  int j_lo, j_hi;
  sketch_range(append, seq_len, b, T_max, R, pool, NB, t_begin, t_end, j_lo, j_hi);
  if constexpr (AMAX) j_hi = min(j_hi, clamp_len(seq_len[b], T_max, 1));
  const int j0 = j_lo + blockIdx.x * SM_ROWS;
  if (j0 >= j_hi) {
    if constexpr (AMAX)
      if (threadIdx.x == 0) amax[(size_t)blockIdx.y * gridDim.x + blockIdx.x] = 0.f;
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;

  // the split basis, in B-operand order
  const float *P = basis + (basis_per_head ? (size_t)h * RANK * D : 0);
  for (int e = threadIdx.x; e < 3 * 4 * 4 * 64; e += SM_THREADS) {
    const int part = e >> 10, nb = (e >> 8) & 3, c = (e >> 6) & 3, l = e & 63;
    // column n of basis block nb is basis row 4n + nb: a lane's four blocks
    // then hold four consecutive codes of a row
    const float *src = P + (size_t)(4 * (l & 15) + nb) * D + sm_dim<DT>(c, l >> 4);
    sk_u32x4_t w;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = sk_split(src[2 * k], part) | (sk_split(src[2 * k + 1], part) << 16);
    bop[part][nb][c][l] = w;
  }
  __syncthreads();

  const float kinv = AMAX ? 1.f : 1.0f / key_scale[h];
  float am = 0.f;                                           // AMAX: this lane's largest |y|
  constexpr int RB = row_bytes<DT>();
  const char *Xbh = static_cast<const char *>(X) + (size_t)bh * x_rows_per_bh * RB;
  const uint16_t *Xsbh = DT != SKS_KV_BF16 ? Xs + (size_t)bh * x_rows_per_bh : nullptr;
  uint8_t *st = stage[wave];

  // A operands of a tile: rows row0 + 16m + n (clamped into the range), 8
  // dims per step, loaded one tile ahead of their use
  auto load_tile = [&](int row0, sk_u32x4_t (&a)[4][4], float &xs) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const size_t r = (size_t)min(row0 + 16 * m + n, j_hi - 1);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (DT == SKS_KV_I4) {
          if (c == 0) {                                       // all four steps: 16 bytes
            const uint4 w = *reinterpret_cast<const uint4 *>(Xbh + r * RB + 16 * g);
            a[m][0] = sk_u32x4_t{w.x, w.y, w.z, w.w};
          }
        } else if constexpr (DT == SKS_KV_BF16) {
          const uint4 w = *reinterpret_cast<const uint4 *>(Xbh + (r * D + 32 * c + 8 * g) * 2);
          a[m][c] = sk_u32x4_t{w.x, w.y, w.z, w.w};
        } else {
          const uint2 w = *reinterpret_cast<const uint2 *>(Xbh + r * D + 32 * c + 8 * g);
          a[m][c] = sk_u32x4_t{w.x, w.y, 0u, 0u};             // converted when used
        }
      }
    }
    xs = 1.f;                                               // codes: scale of row row0 + lane
    if constexpr (DT != SKS_KV_BF16) xs = f16_bits_to_float(Xsbh[min(row0 + lane, j_hi - 1)]);
  };
  auto tile_row = [&](int it) { return j0 + it * (SM_TILE * SM_THREADS / 64) + wave * SM_TILE; };
  sk_u32x4_t cur[4][4], nxt[4][4];
  float xs_cur, xs_nxt;
  load_tile(min(tile_row(0), j_hi - 1), cur, xs_cur);
  for (int it = 0; it < SM_ITERS; ++it) {
    const int row0 = tile_row(it);
    if (row0 >= j_hi) break;                                // uniform per wave
    // the next tile's loads go out before this tile's products (a tile past
    // the range reloads the last row: in bounds, unused)
    __builtin_amdgcn_sched_barrier(0);
    load_tile(min(tile_row(it + 1), j_hi - 1), nxt, xs_nxt);
    __builtin_amdgcn_sched_barrier(0);
    sk_u32x4_t a[4][4];
    const float xs = xs_cur;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (DT == SKS_KV_BF16) {
          a[m][c] = cur[m][c];
        } else if constexpr (DT == SKS_KV_I4) {
          a[m][c] = i4x8_bf16(cur[m][0][c]);
        } else {
          const uint32_t x0 = cur[m][c][0], x1 = cur[m][c][1];
          a[m][c] = sk_u32x4_t{i8pair_bf16(x0, 0), i8pair_bf16(x0, 16), i8pair_bf16(x1, 0),
                               i8pair_bf16(x1, 16)};
        }
      }

    sk_f32x4_t acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[m][nb] = sk_f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int part = 0; part < 3; ++part) {
          const sk_u32x4_t bv = bop[part][nb][c][lane];
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[m][nb] = sk_mfma(a[m][c], bv, acc[m][nb]);
        }

    if constexpr (AMAX) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float sc = DT != SKS_KV_BF16 ? __shfl(xs, 16 * m + 4 * g + j) : 1.f;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) am = fmaxf(am, fabsf(acc[m][nb][j] * sc));
        }
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) cur[m][c] = nxt[m][c];
      xs_cur = xs_nxt;
      continue;
    }
    // codes: lane holds Y[row 16m + 4g + j][basis 4n + nb], i.e. bytes
    // 4n .. 4n + 3 of the row's code, stored as one 32-bit word
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = 16 * m + 4 * g + j;
        const float sc = DT != SKS_KV_BF16 ? __shfl(xs, rr) : 1.f;
        uint32_t word = 0;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          word |= (uint32_t)(uint8_t)key_code(acc[m][nb][j] * sc, kinv) << (8 * nb);
        *reinterpret_cast<uint32_t *>(st + rr * RANK + 4 * n) = word;
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // 64 rows x 64 B, contiguous in S: 16-byte pieces, rows past the range skipped
    uint4 *dst = reinterpret_cast<uint4 *>(S + ((size_t)bh * NB + row0) * RANK);
#pragma unroll
    for (int k = 0; k < SM_TILE * RANK / 16 / 64; ++k) {
      const int piece = k * 64 + lane;
      if (row0 + piece / (RANK / 16) < j_hi) dst[piece] = reinterpret_cast<const uint4 *>(st)[piece];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) cur[m][c] = nxt[m][c];
    xs_cur = xs_nxt;
  }
  if constexpr (AMAX) {
    // max is exact in any order: the result does not depend on the schedule
    for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
    __shared__ float wmax[SM_THREADS / 64];
    if (lane == 0) wmax[wave] = am;
    __syncthreads();
    if (threadIdx.x == 0) {
      float m = wmax[0];
      for (int w = 1; w < SM_THREADS / 64; ++w) m = fmaxf(m, wmax[w]);
      amax[(size_t)blockIdx.y * gridDim.x + blockIdx.x] = m;
    }
  }
}

// Pooled blocks (bf16 caches): mean of `pool` consecutive K and V rows in
// fp64 (exact sums of bf16 values), rounded once to bf16 and stored in Kp/Vp;
// the sketch of the stored pooled keys follows in sketch_mfma_kernel.
// Thread: one 16-byte piece (8 dims) of one block's K or V row; the 16
// threads of a row are adjacent, so every load and store is coalesced.
constexpr int PM_THREADS = 256;
constexpr int PM_BLOCKS = PM_THREADS / 32;                  // blocks per workgroup (K and V)

__global__ __launch_bounds__(PM_THREADS) void pool_mean_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V,
    const int32_t *__restrict__ seq_len, int Hkv, int T_max, int R, int NB, int pool, int append,
    int t_begin, int t_end, uint16_t *__restrict__ Kp, uint16_t *__restrict__ Vp) {
  const int bh = blockIdx.y, b = bh / Hkv;
  int j_lo, j_hi;
  sketch_range(append, seq_len, b, T_max, R, pool, NB, t_begin, t_end, j_lo, j_hi);
  const int j = j_lo + blockIdx.x * PM_BLOCKS + (threadIdx.x >> 5);
  if (j >= j_hi) return;
  const int which = (threadIdx.x >> 4) & 1, piece = threadIdx.x & 15;
  const uint16_t *src = (which == 0 ? K : V) + ((size_t)bh * T_max + (size_t)j * pool) * D + piece * 8;
  double sm[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int k = 0; k < pool; ++k) {
    const uint4 w = *reinterpret_cast<const uint4 *>(src + (size_t)k * D);
    sm[0] += bf16_lo(w.x); sm[1] += bf16_hi(w.x); sm[2] += bf16_lo(w.y); sm[3] += bf16_hi(w.y);
    sm[4] += bf16_lo(w.z); sm[5] += bf16_hi(w.z); sm[6] += bf16_lo(w.w); sm[7] += bf16_hi(w.w);
  }
  const double dpool = (double)pool;
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o[e] = f64_to_bf16_rne(sm[2 * e] / dpool) | ((uint32_t)f64_to_bf16_rne(sm[2 * e + 1] / dpool) << 16);
  *reinterpret_cast<uint4 *>((which == 0 ? Kp : Vp) + ((size_t)bh * NB + j) * D + piece * 8) =
      make_uint4(o[0], o[1], o[2], o[3]);
}

// A short range or the per-step append: one workgroup per sketch row (see
// block_key_row).
template <int DT>
__global__ __launch_bounds__(SK_THREADS) void sketch_rows_small_kernel(
    const void *__restrict__ K, const void *__restrict__ V, const uint16_t *__restrict__ Ks,
    const void *__restrict__ Kh, const uint16_t *__restrict__ Ksh, int W_hot,
    const int32_t *__restrict__ seq_len, const float *__restrict__ basis, int basis_per_head,
    const float *__restrict__ key_scale, int Hkv, int T_max, int R, int NB, int pool, int append,
    int t_begin, int t_end, int8_t *__restrict__ S, uint16_t *__restrict__ Kp,
    uint16_t *__restrict__ Vp) {
  __shared__ SketchLds lds;
  block_key_row<DT>(K, V, Ks, Kh, Ksh, W_hot, seq_len, basis, basis_per_head, key_scale, Hkv,
                    T_max, R, NB, pool, append, t_begin, t_end, S, Kp, Vp, blockIdx.y, blockIdx.x,
                    lds);
}

// Query sketch: one workgroup per (b, i, h) (see block_query_sketch).
__global__ __launch_bounds__(SK_THREADS) void sketch_query_kernel(
    const uint16_t *__restrict__ q, int R, int Hq, int Hkv, const float *__restrict__ basis,
    int basis_per_head, int8_t *__restrict__ qsk, float *__restrict__ qscale) {
  __shared__ SketchLds lds;
  const int seg = blockIdx.x;
  block_query_sketch(q, R, Hq, Hkv, basis, basis_per_head, seg, qsk + (size_t)seg * RANK,
                     qscale ? qscale + seg : nullptr, lds);
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
  if (nrows <= SMALL_ROWS || append) {
    // few rows per (b, h): one wave per row (an append is at most R + 1 rows)
    dim3 g2((unsigned)nrows, s.B * s.Hkv);
    const HotRows hr = hot_rows(kv);
#define SKS_ROWS_SMALL(DT)                                                                         \
  sketch_rows_small_kernel<DT><<<g2, SK_THREADS, 0, st>>>(kv.K, kv.V, kv.K_scale, hr.K, hr.Ks, \
                                                          hr.W,                                  \
                                                  kv.seq_len, basis, basis_per_head, key_scale,   \
                                                  s.Hkv, s.T_max, s.R, s.NB, s.pool, append,      \
                                                  t_begin, t_end, S, Kp, Vp)
    if (s.dtype == SKS_KV_BF16)
      SKS_ROWS_SMALL(SKS_KV_BF16);
    else if (s.dtype == SKS_KV_I8)
      SKS_ROWS_SMALL(SKS_KV_I8);
    else
      SKS_ROWS_SMALL(SKS_KV_I4);
#undef SKS_ROWS_SMALL
    return hipGetLastError();
  }
  dim3 grid(ceil_div(nrows, SM_ROWS), s.B * s.Hkv);
  if (s.pool == 1) {
#define SKS_MFMA(DT)                                                                              \
  sketch_mfma_kernel<DT><<<grid, SM_THREADS, 0, st>>>(kv.K, kv.K_scale, s.T_max, kv.seq_len,     \
                                                      basis, basis_per_head, key_scale, s.Hkv,   \
                                                      s.T_max, s.R, s.NB, 1, append, t_begin,    \
                                                      t_end, S)
    if (s.dtype == SKS_KV_BF16)
      SKS_MFMA(SKS_KV_BF16);
    else if (s.dtype == SKS_KV_I8)
      SKS_MFMA(SKS_KV_I8);
    else
      SKS_MFMA(SKS_KV_I4);
#undef SKS_MFMA
  } else {
    dim3 gp(ceil_div(nrows, PM_BLOCKS), s.B * s.Hkv);
    pool_mean_kernel<<<gp, PM_THREADS, 0, st>>>(
        static_cast<const uint16_t *>(kv.K), static_cast<const uint16_t *>(kv.V), kv.seq_len,
        s.Hkv, s.T_max, s.R, s.NB, s.pool, append, t_begin, t_end, Kp, Vp);
    // then the sketch of the stored pooled keys (rows of Kp, NB per (b, h))
    sketch_mfma_kernel<SKS_KV_BF16><<<grid, SM_THREADS, 0, st>>>(
        Kp, nullptr, s.NB, kv.seq_len, basis, basis_per_head, key_scale, s.Hkv, s.T_max, s.R,
        s.NB, s.pool, append, t_begin, t_end, S);
  }
  return hipGetLastError();
}

// Largest |P x| per workgroup over the keys [t_begin, min(t_end, L_b)) of
// every (b, h) (bf16 caches); amax gets grid.x * B * Hkv maxima, grid.x =
// refit_amax_chunks(...).
int refit_amax_chunks(long span) { return span <= 0 ? 1 : ceil_div(span, SM_ROWS); }

hipError_t launch_refit_amax(const sks_kv &kv, int t_begin, int t_end, const float *basis,
                             int basis_per_head, float *amax, hipStream_t st) {
  const long span = (long)t_end - (long)t_begin;
  dim3 grid(refit_amax_chunks(span), kv.B * kv.Hkv);
  sketch_mfma_kernel<SKS_KV_BF16, true><<<grid, SM_THREADS, 0, st>>>(
      kv.K, nullptr, kv.T_max, kv.seq_len, basis, basis_per_head, nullptr, kv.Hkv, kv.T_max, 1,
      kv.T_max, 1, 0, t_begin, t_end, nullptr, amax);
  return hipGetLastError();
}

hipError_t launch_sketch_query(const uint16_t *q, int B, int R, int Hq, int Hkv,
                               const float *basis, int basis_per_head, int8_t *qsk,
                               float *qscale, hipStream_t st) {
  sketch_query_kernel<<<B * R * Hkv, SK_THREADS, 0, st>>>(q, R, Hq, Hkv, basis, basis_per_head,
                                                          qsk, qscale);
  return hipGetLastError();
}

}  // namespace sks
