// Sketch-basis refit: the "frozen sketch basis (one file) plus the script to
// refit it" of "What it took" on the page "8 agents x 250K context,
// concurrently, on two 3090s".  The basis rows are the 64 leading
// eigenvectors of the Gram matrix G = sum_t x_t x_t^T of captured keys, and
// the key scale is the largest |P x| / 127 over the same keys.
//
// 1. gram_kernel: per workgroup, the Gram matrix of a chunk of one (b, h)'s
//    keys on the matrix cores (bf16 products are exact in fp32), written as
//    an fp32 partial of its 36 upper 16x16 blocks.
// 2. gram_reduce_kernel: the partials of each matrix summed in fp64, in a
//    fixed order, into the full symmetric G.
// 3. jacobi_kernel: one workgroup per matrix, cyclic two-sided Jacobi in fp64
//    with the round-robin pair order (64 disjoint rotations per round), G in
//    LDS, the eigenvectors accumulated in the workspace; then the 64 leading
//    eigenvectors, signed so that their largest-magnitude component is
//    positive, as fp32 basis rows.
// 4. the key-scale pass is the absmax mode of the matrix-core sketch kernel,
//    reduced here.
#include "refit.h"

namespace sks {
namespace {

typedef __bf16 rf_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float rf_f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t rf_u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rf_f32x4_t rf_mfma(rf_u32x4_t a, rf_u32x4_t b, rf_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(rf_bf16x8_t, a),
                                                 __builtin_bit_cast(rf_bf16x8_t, b), c, 0, 0, 0);
}

constexpr int GR_THREADS = 256;
constexpr int GR_TILE = 32;                      // keys per wave and iteration (the MFMA K)
constexpr int GR_ITERS = 64;
constexpr int GR_ROWS = GR_TILE * (GR_THREADS / 64) * GR_ITERS;   // 8192 keys per workgroup
constexpr int GR_BLOCKS = 36;                    // upper 16x16 blocks (i <= j) of 128 x 128
constexpr int GR_LROW = 132;                     // LDS row stride (bf16): conflict-free column reads
constexpr int GR_PART = GR_BLOCKS * 256;         // floats per partial

// block index of (i, j), i <= j < 8
__host__ __device__ constexpr int blk_id(int i, int j) { return i * 8 - i * (i - 1) / 2 + (j - i); }

// Gram partial of keys [lo + blockIdx.x * GR_ROWS, +GR_ROWS) of (b, h) =
// blockIdx.y, lo = max(t_begin, 0), hi = min(t_end, L_b, T_max).  Each wave
// stages 32 keys in LDS and reads them back as the MFMA operand "8 keys of one
// dim" (lane (n, g): dim 16 db + n, keys 8g .. 8g + 8), which serves as A
// (rows = dims of block i) and as B (columns = dims of block j) alike.
__global__ __launch_bounds__(GR_THREADS, 2) void gram_kernel(
    const uint16_t *__restrict__ K, const int32_t *__restrict__ seq_len, int Hkv, int T_max,
    int t_begin, int t_end, float *__restrict__ part) {
  __shared__ __align__(16) uint16_t tile[GR_THREADS / 64][GR_TILE * GR_LROW];
  __shared__ float red[GR_PART];
  const int bh = blockIdx.y, b = bh / Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int lo = max(t_begin, 0);
  const int hi = min(min(t_end, T_max), clamp_len(seq_len[b], T_max, 1));
  const int c0 = lo + blockIdx.x * GR_ROWS;
  const uint16_t *Kbh = K + (size_t)bh * T_max * D;
  uint16_t *tl = tile[wave];

  rf_f32x4_t acc[GR_BLOCKS];
#pragma unroll
  for (int k = 0; k < GR_BLOCKS; ++k) acc[k] = rf_f32x4_t{0.f, 0.f, 0.f, 0.f};

  // 32 keys x 256 B = 512 pieces of 16 B: 8 per lane; keys past hi are zero
  auto load = [&](int row0, uint4 (&w)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int x = k * 64 + lane, r = row0 + (x >> 4);
      const int rc = min(r, max(hi - 1, 0));
      w[k] = *reinterpret_cast<const uint4 *>(Kbh + (size_t)rc * D + (x & 15) * 8);
      if (r >= hi) w[k] = make_uint4(0, 0, 0, 0);
    }
  };
  auto tile_row = [&](int it) { return c0 + (it * (GR_THREADS / 64) + wave) * GR_TILE; };
  uint4 cur[8], nxt[8];
  if (hi > lo) load(tile_row(0), cur);
  for (int it = 0; it < GR_ITERS; ++it) {
    const int row0 = tile_row(it);
    if (row0 >= hi) break;                                  // uniform per wave
    __builtin_amdgcn_sched_barrier(0);
    load(tile_row(it + 1), nxt);                            // in bounds (clamped), unused past hi
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int x = k * 64 + lane;
      uint2 *dst = reinterpret_cast<uint2 *>(tl + (x >> 4) * GR_LROW + (x & 15) * 8);
      dst[0] = make_uint2(cur[k].x, cur[k].y);
      dst[1] = make_uint2(cur[k].z, cur[k].w);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    rf_u32x4_t op[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const uint16_t *col = tl + (8 * g) * GR_LROW + 16 * db + n;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        op[db][k] = (uint32_t)col[(2 * k) * GR_LROW] | ((uint32_t)col[(2 * k + 1) * GR_LROW] << 16);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = i; j < 8; ++j) acc[blk_id(i, j)] = rf_mfma(op[i], op[j], acc[blk_id(i, j)]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int k = 0; k < 8; ++k) cur[k] = nxt[k];
  }

  // the four waves' sums, in wave order, then the partial: block k element
  // (4g + r, n) at k * 256 + (4g + r) * 16 + n
  for (int w = 0; w < GR_THREADS / 64; ++w) {
    if (wave == w) {
#pragma unroll
      for (int k = 0; k < GR_BLOCKS; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int at = k * 256 + (4 * g + r) * 16 + n;
          red[at] = w == 0 ? acc[k][r] : red[at] + acc[k][r];
        }
    }
    __syncthreads();
  }
  float *dst = part + ((size_t)bh * gridDim.x + blockIdx.x) * GR_PART;
  for (int x = threadIdx.x; x < GR_PART; x += GR_THREADS) dst[x] = red[x];
}

// G[mat] = sum of the partials of matrix mat in fp64, in (b, h, chunk) order;
// per_head: mat = h, else one matrix from every head.  Thread: one element of
// the upper blocks, mirrored into the lower half.
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float *__restrict__ part, int B,
                                                          int Hkv, int nchunk, int per_head,
                                                          double *__restrict__ G) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= GR_PART) return;
  const int mat = blockIdx.y;
  // the partials of this matrix, in (b, h, chunk) order: 8 loads in flight,
  // added in order
  const int h0 = per_head ? mat : 0, nh = per_head ? 1 : Hkv;
  const int n = B * nh * nchunk;
  auto at = [&](int u) {
    const int c = u % nchunk, hb = u / nchunk, h = h0 + hb % nh, b = hb / nh;
    return (((size_t)b * Hkv + h) * nchunk + c) * GR_PART + e;
  };
  double sum = 0.0;
  for (int u0 = 0; u0 < n; u0 += 8) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = u0 + k < n ? part[at(u0 + k)] : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) sum += (double)v[k];
  }
  const int k = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
  int bi = 0;
  while (blk_id(bi, 7) < k) ++bi;                          // block row of block k
  const int bj = bi + (k - blk_id(bi, bi));
  if (bi == bj && rr > cc) return;                          // a diagonal block's lower half: mirrored
  const int row = 16 * bi + rr, col = 16 * bj + cc;
  double *Gm = G + (size_t)mat * D * D;
  Gm[(size_t)row * D + col] = sum;
  Gm[(size_t)col * D + row] = sum;
}

constexpr int JB_THREADS = 1024;
constexpr int JB_LDA = D + 1;                    // padded LDS row (fp64): column walks spread banks
constexpr int JB_MAX_SWEEPS = 60;

__global__ __launch_bounds__(JB_THREADS) void jacobi_kernel(const double *__restrict__ G,
                                                            double *__restrict__ Vws,
                                                            float *__restrict__ basis,
                                                            double *__restrict__ eigval) {
  __shared__ double A[D * JB_LDA];
  __shared__ double rc[D / 2], rs[D / 2];
  __shared__ int rp[D / 2], rq[D / 2];
  __shared__ double red[2][JB_THREADS / 64];
  __shared__ int order[D];
  __shared__ double sgn[RANK];
  __shared__ int done;
  const int mat = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const double *Gm = G + (size_t)mat * D * D;
  double *V = Vws + (size_t)mat * D * D;
  for (int x = tid; x < D * D; x += JB_THREADS) A[(x / D) * JB_LDA + x % D] = Gm[x];
  // V in registers: lane k holds, for rows i = 8 wave .. 8 wave + 7, the
  // entries of the two columns of pair k of the current round (vt: the first
  // index p, vb: the second index q).  Round r pairs (127, r) and
  // ((r + k) % 127, (r - k) % 127): from one round to the next, the first index
  // of pair k + 1 becomes that of pair k, the second of pair k - 1 that of pair
  // k (pair 0 keeps 127 and takes the first index of pair 1; pair 63 takes
  // its own second index as the first), so the columns move one lane per
  // round and V never leaves the registers until the end.
  constexpr int VR = D / (JB_THREADS / 64);      // rows per wave
  auto top_idx = [&](int r) { return lane == 0 ? D - 1 : (r + lane) % (D - 1); };
  auto bot_idx = [&](int r) { return lane == 0 ? r : (r - lane + (D - 1)) % (D - 1); };
  double vt[VR], vb[VR];
#pragma unroll
  for (int u = 0; u < VR; ++u) {
    const int i = wave * VR + u;
    vt[u] = i == top_idx(0) ? 1.0 : 0.0;
    vb[u] = i == bot_idx(0) ? 1.0 : 0.0;
  }
  __syncthreads();

  for (int sweep = 0; sweep < JB_MAX_SWEEPS; ++sweep) {
    // convergence: off-diagonal mass against the diagonal's (fixed-order sums)
    double off = 0.0, dia = 0.0;
    for (int x = tid; x < D * D; x += JB_THREADS) {
      const int i = x / D, j = x % D;
      const double a = A[i * JB_LDA + j];
      if (i == j) dia += a * a; else off += a * a;
    }
    for (int o = 32; o > 0; o >>= 1) {
      off += __shfl_xor(off, o);
      dia += __shfl_xor(dia, o);
    }
    if ((tid & 63) == 0) {
      red[0][tid >> 6] = off;
      red[1][tid >> 6] = dia;
    }
    __syncthreads();
    if (tid == 0) {
      double o = 0.0, d = 0.0;
      for (int w = 0; w < JB_THREADS / 64; ++w) {
        o += red[0][w];
        d += red[1][w];
      }
      done = !(o > 1e-30 * d);
    }
    __syncthreads();
    if (done) break;
    for (int r = 0; r < D - 1; ++r) {
      // pairs of round r: (127, r) and ((r + k) % 127, (r - k) % 127), k = 1 .. 63
      if (tid < D / 2) {
        const int p = tid == 0 ? D - 1 : (r + tid) % (D - 1);
        const int q = tid == 0 ? r : (r - tid + (D - 1)) % (D - 1);
        const double app = A[p * JB_LDA + p], aqq = A[q * JB_LDA + q], apq = A[p * JB_LDA + q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double th = (aqq - app) / (2.0 * apq);
          const double at = fabs(th);
          const double t = (th >= 0.0 ? 1.0 : -1.0) / (at + (at < 1e150 ? sqrt(th * th + 1.0) : at));
          c = 1.0 / sqrt(t * t + 1.0);
          s = t * c;
        }
        rc[tid] = c;
        rs[tid] = s;
        rp[tid] = p;
        rq[tid] = q;
      }
      __syncthreads();
      // A <- J^T A J, by 2 x 2 blocks: the block of rows (p_k, q_k) and columns
      // (p_l, q_l) depends on the rotations of pairs k and l only, so each
      // block is rotated on its rows and then on its columns in one pass
      // (the same operations per element as a pass over rows then one over
      // columns).  A diagonal block's off-diagonal pair is zero after its
      // rotation and is stored as such.  Wave w takes row pairs w, w + 16,
      // w + 32, w + 48 and lane l column pair l.
      {
        const int l = lane;
        const double cl = rc[l], sl = rs[l];
        const int pl = rp[l], ql = rq[l];
#pragma unroll
        for (int m = 0; m < D / 2 / (JB_THREADS / 64); ++m) {
          const int k = wave + m * (JB_THREADS / 64);
          const double ck = rc[k], sk = rs[k];
          double *rowp = A + rp[k] * JB_LDA, *rowq = A + rq[k] * JB_LDA;
          const double a_pp = rowp[pl], a_pq = rowp[ql], a_qp = rowq[pl], a_qq = rowq[ql];
          // rows
          const double r_pp = ck * a_pp - sk * a_qp, r_qp = sk * a_pp + ck * a_qp;
          const double r_pq = ck * a_pq - sk * a_qq, r_qq = sk * a_pq + ck * a_qq;
          // columns
          double n_pp = cl * r_pp - sl * r_pq, n_pq = sl * r_pp + cl * r_pq;
          double n_qp = cl * r_qp - sl * r_qq, n_qq = sl * r_qp + cl * r_qq;
          if (k == l && sk != 0.0) {
            n_pq = 0.0;
            n_qp = 0.0;
          }
          rowp[pl] = n_pp;
          rowp[ql] = n_pq;
          rowq[pl] = n_qp;
          rowq[ql] = n_qq;
        }
      }
      // V <- V J on this lane's pair, then the columns move to the next
      // round's lanes (see above)
      {
        const double c = rc[lane], s = rs[lane];
#pragma unroll
        for (int u = 0; u < VR; ++u) {
          const double a = vt[u], b = vb[u];
          vt[u] = c * a - s * b;
          vb[u] = s * a + c * b;
          const double from_next_top = __shfl_down(vt[u], 1);    // lane k + 1's first column
          const double from_prev_bot = __shfl_up(vb[u], 1);      // lane k - 1's second column
          const double t = lane == 0 ? vt[u] : (lane == 63 ? vb[u] : from_next_top);
          vb[u] = lane == 0 ? from_next_top : from_prev_bot;
          vt[u] = t;
        }
      }
      __syncthreads();
    }
  }

  // V to the workspace: after whole sweeps the lanes hold round 0's columns
#pragma unroll
  for (int u = 0; u < VR; ++u) {
    const int i = wave * VR + u;
    V[(size_t)i * D + top_idx(0)] = vt[u];
    V[(size_t)i * D + bot_idx(0)] = vb[u];
  }
  __syncthreads();
  // eigenvalues in descending order (equal values: lower index first)
  if (tid < D) {
    const double d = A[tid * JB_LDA + tid];
    int rank = 0;
    for (int j = 0; j < D; ++j) {
      const double e = A[j * JB_LDA + j];
      rank += (e > d) || (e == d && j < tid);
    }
    order[rank] = tid;
  }
  __syncthreads();
  if (eigval && tid < D) eigval[(size_t)mat * D + tid] = A[order[tid] * JB_LDA + order[tid]];
  // sign: the largest-magnitude component (first on ties) positive
  if (tid < RANK) {
    const int col = order[tid];
    double best = -1.0, v = 0.0;
    for (int k = 0; k < D; ++k) {
      const double x = V[(size_t)k * D + col];
      if (fabs(x) > best) {
        best = fabs(x);
        v = x;
      }
    }
    sgn[tid] = v < 0.0 ? -1.0 : 1.0;
  }
  __syncthreads();
  for (int x = tid; x < RANK * D; x += JB_THREADS) {
    const int r = x / D, k = x % D;
    basis[(size_t)mat * RANK * D + x] = (float)(sgn[r] * V[(size_t)k * D + order[r]]);
  }
}

// key_scale[h] = (max over the workgroups of (b, h) of their largest |P x|) / 127
// (1 when it is 0)
// One wave per KV head; the maximum is exact in any order.
__global__ __launch_bounds__(64) void amax_reduce_kernel(const float *__restrict__ amax, int B,
                                                         int Hkv, int nchunk,
                                                         float *__restrict__ key_scale) {
  const int h = blockIdx.x, lane = threadIdx.x;
  float m = 0.f;
  for (int u = lane; u < B * nchunk; u += 64) {
    const int b = u / nchunk, c = u % nchunk;
    m = fmaxf(m, amax[((size_t)b * Hkv + h) * nchunk + c]);
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) key_scale[h] = m > 0.f ? m / 127.0f : 1.0f;
}

}  // namespace

int refit_gram_chunks(long span) { return span <= 0 ? 1 : ceil_div(span, GR_ROWS); }

size_t refit_gram_scratch_bytes(int B, int Hkv, long span) {
  return (size_t)B * Hkv * refit_gram_chunks(span) * GR_PART * sizeof(float);
}

hipError_t launch_refit_gram(const sks_kv &kv, int t_begin, int t_end, int per_head, double *G,
                             void *ws, hipStream_t st) {
  const long span = (long)t_end - (long)t_begin;
  const int nchunk = refit_gram_chunks(span);
  float *part = static_cast<float *>(ws);
  gram_kernel<<<dim3(nchunk, kv.B * kv.Hkv), GR_THREADS, 0, st>>>(
      static_cast<const uint16_t *>(kv.K), kv.seq_len, kv.Hkv, kv.T_max, t_begin, t_end, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nmat = per_head ? kv.Hkv : 1;
  gram_reduce_kernel<<<dim3(ceil_div(GR_PART, 256), nmat), 256, 0, st>>>(part, kv.B, kv.Hkv,
                                                                         nchunk, per_head, G);
  return hipGetLastError();
}

hipError_t launch_refit_basis(const double *G, int nmat, float *basis, double *eigval, void *ws,
                              hipStream_t st) {
  jacobi_kernel<<<nmat, JB_THREADS, 0, st>>>(G, static_cast<double *>(ws), basis, eigval);
  return hipGetLastError();
}

hipError_t launch_refit_scale_reduce(const float *amax, int B, int Hkv, int nchunk,
                                     float *key_scale, hipStream_t st) {
  amax_reduce_kernel<<<Hkv, 64, 0, st>>>(amax, B, Hkv, nchunk, key_scale);
  return hipGetLastError();
}

}  // namespace sks
