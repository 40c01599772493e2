// Device code of the sparse decode attention: one attention slot of one
// segment as a template over the group size, the KV storage, pooling and the
// tiles per wave.  (Algorithm: see k_attn.hip.)
#pragma once

#include <type_traits>

#include "sks_internal.h"
#include "tier.h"

namespace sks {
namespace {

// SKS_ATTN_VALU = 1 builds the comparison variant of the attention whose Q.K
// and P.V products run on the vector ALUs (bf16 rows; everything else --
// gathers, tiles, splits, softmax, merge -- unchanged).  The library
// is built with 0; `build.py --attn-valu` builds the variant beside it.
#ifndef SKS_ATTN_VALU
#define SKS_ATTN_VALU 0
#endif

constexpr int AT_THREADS = 256;
constexpr int ATTN_SPLIT = 384;          // attention entries per workgroup, at most
constexpr long ATTN_SMALL_SET = 1536;    // smaller attention sets: 128-entry slots
constexpr float NEG_INF = -__builtin_huge_valf();

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Matrix-core version.  Per wave, tiles of 32 entries:
//   QK:  S[16 heads][16 entries] = Q x K^T with v_mfma_f32_16x16x32_bf16, two
//        sub-tiles of 16 entries (query heads padded to the 16 MFMA rows).
//        A = Q: lane (n = lane%16, g = lane/16) holds head n, dims 32i+8g..+8;
//        B = K^T: lane holds entry n, the same dims (bf16: read from the K
//        rows staged in wave-private LDS; int8 / int4: straight from the
//        gathers).
//        C: lane holds S[4g + j][n], j = 0..3.
//   softmax on that layout: each lane owns 4 heads x 1 entry; row max and
//        sums over the 16 lanes of its DPP row.  The running max is only
//        moved when a tile exceeds it by more than 2^RESCALE_SLACK (exact in
//        real arithmetic; the ratio stays far inside fp32 range).
//   PV:  O[16 heads][128] += P x V with the same MFMA, K = the 32 entries.
//        P is split into bf16 hi + lo parts (two MFMAs) so its weights keep
//        ~16 significant bits; V rows are staged row-major in wave-private
//        LDS and read back per MFMA as 8 entries x 1 dim per lane by two
//        transpose reads.
// All heads of the KV group share every gathered row; the 16-row MFMA shape
// leaves 16 - G rows idle, which costs nothing here: the pass is bound by
// the gathers.
constexpr int AM_TILE = 32;
// Entries per workgroup (the attention split): 4 waves of TILES tiles each.
// More tiles per wave keep a tile's gathers in flight while the previous one
// is consumed; fewer make more workgroups and shorter chains (see
// attn_split).
template <int TILES>
constexpr int attn_split_entries() { return (AT_THREADS / 64) * TILES * AM_TILE; }
static_assert(attn_split_entries<3>() == ATTN_SPLIT, "the largest split");
// LDS row strides in bf16: V rows of 288 B (the four rows that a lane group
// reads at once by transpose reads fall in disjoint banks), K rows of 272 B
// (the 16 rows of one 16-byte operand read fall in disjoint banks).
constexpr int VROW = 144;
constexpr int KROW = 136;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
// LDS transpose read (gfx950): within each group of 16 lanes, the 8-byte
// chunks that the lanes address form a 16 x 4 matrix M of 16-bit values
// (row = addressing lane); lane j receives M[4s + j / 4][j % 4] in slot s.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t *p) {
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t *)(p));
  return __builtin_bit_cast(uint2, r);
}
constexpr float RESCALE_SLACK = 8.0f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// LDS written by some lanes of this wave and read by others: order the
// accesses (in-order LDS queue per wave, no workgroup barrier needed).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// int8 codes -> bf16 (exact: |code| <= 127 needs 7 significant bits)
__device__ __forceinline__ uint32_t i8pair_to_bf16x2(uint32_t w, int sh) {
  const float a = (float)(int8_t)(w >> sh), b = (float)(int8_t)(w >> (sh + 8));
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}

// int4 codes (eight two's-complement nibbles of w, low nibble first: dims
// 0..7 of a group of 8) -> code + I4_BIAS as bf16, exactly: with u = nibble
// ^ 8 = code + 8 in [0, 15], the bf16 pattern 0x4300 | u is 128 + u.  The
// eight values come out in the slot order I4_ORDER = dims 0, 2, 4, 6, 1, 3,
// 5, 7, so that each bf16 pair is one byte permute of the masked low (or
// high) nibbles with the constant 0x43 bytes: about one VALU op per value.
// The bias is taken out of the products afterwards (see attn_body).
constexpr float I4_BIAS = 136.f;
__device__ __forceinline__ u32x4_t i4_biased_bf16x8(uint32_t w) {
  const uint32_t x = w ^ 0x88888888u;
  const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;   // dims 0,2,4,6 / 1,3,5,7
  const uint32_t k43 = 0x43434343u;
  // perm(S0, S1, sel): selector bytes 0-3 pick bytes of S1, 4-7 bytes of S0
  return u32x4_t{__builtin_amdgcn_perm(k43, lo, 0x04010400u), __builtin_amdgcn_perm(k43, lo, 0x04030402u),
                 __builtin_amdgcn_perm(k43, hi, 0x04010400u), __builtin_amdgcn_perm(k43, hi, 0x04030402u)};
}
// dim held by slot s (0..7) of a group of 8 in I4_ORDER
__device__ __forceinline__ int i4_slot_dim(int s) { return s < 4 ? 2 * s : 2 * (s - 4) + 1; }

// Max over the 16 lanes of each DPP row of values that are never NaN, each
// step as the median of (x, permuted x, +inf): one instruction, where fmaxf
// would first quiet the permuted operand.  `inf` must be +inf and opaque to
// the compiler (see opaque_inf), which would otherwise turn the median back
// into fmaxf.
__device__ __forceinline__ float row16_max_f(float x, float inf) {
  x = __builtin_amdgcn_fmed3f(x, dpp_f<DPP_ROW_MIRROR>(x), inf);
  x = __builtin_amdgcn_fmed3f(x, dpp_f<DPP_ROW_HMIRROR>(x), inf);
  x = __builtin_amdgcn_fmed3f(x, dpp_f<DPP_QUAD_XOR1>(x), inf);
  x = __builtin_amdgcn_fmed3f(x, dpp_f<DPP_QUAD_XOR2>(x), inf);
  return x;
}
// +inf in a register, produced by a move the compiler cannot see through
__device__ __forceinline__ float opaque_inf() {
  float v;
  asm("v_mov_b32 %0, 0x7f800000" : "=v"(v));
  return v;
}
// two floats -> bf16 pair (round to nearest even), a in the low half
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const bf16x2_t h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// Merge of the partials of one (segment, query head j, dim d) over all
// splits.  The splits are cut into merge_parts(nsplit) <= MP contiguous
// parts, merged in parallel (one group of D threads per part, MB splits'
// loads in flight at a time), and the parts' states are then combined in
// part order through LDS: the order of operations is fixed by the shape.
constexpr int MP = 4;
constexpr int MB = 16;
// one part per MB splits (one round of loads each), at most MP
inline int merge_parts(int nsplit) { return std::min(MP, std::max(1, (nsplit + MB - 1) / MB)); }

// (M, Lsum, A) over splits [s0, s1) of the segment's partials at `base`
__device__ __forceinline__ void merge_range(const float *ml, const float *part_acc, size_t base,
                                            int j, int d, int s0, int s1, int G, float &M,
                                            float &Lsum, float &A) {
  M = NEG_INF;
  Lsum = 0.f;
  A = 0.f;
  for (int c0 = s0; c0 < s1; c0 += MB) {
    float mm[MB], ll[MB], a[MB];
#pragma unroll
    for (int k = 0; k < MB; ++k) {
      const int sp = min(c0 + k, s1 - 1);
      const size_t e = (base + sp) * G + j;
      mm[k] = c0 + k < s1 ? ml[2 * e] : NEG_INF;
      ll[k] = ml[2 * e + 1];
      a[k] = part_acc[e * D + d];
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < MB; ++k) Mn = fmaxf(Mn, mm[k]);
    if (Mn == NEG_INF) continue;
    const float wa = M == NEG_INF ? 0.f : exp2_fast(M - Mn);
    Lsum *= wa;
    A *= wa;
#pragma unroll
    for (int k = 0; k < MB; ++k) {
      const float wt = mm[k] == NEG_INF ? 0.f : exp2_fast(mm[k] - Mn);
      Lsum += ll[k] * wt;
      A += a[k] * wt;
    }
    M = Mn;
  }
}

// One workgroup of D x merge_parts(nsplit) threads per (segment, query head
// j): thread (d, p) merges dim d over part p of the splits.
__device__ void merge_splits(const float2 *part_ml, const float *part_acc, int seg, int j,
                             int nsplit, int G, int Hkv, float *out, float *lse) {
  __shared__ float s_a[MP][D];
  __shared__ float s_m[MP][2];
  const int d = threadIdx.x, p = threadIdx.y, np = blockDim.y;
  const int per = (nsplit + np - 1) / np;
  const int s0 = min(p * per, nsplit), s1 = min(s0 + per, nsplit);
  float M, Lsum, A;
  merge_range(reinterpret_cast<const float *>(part_ml), part_acc, (size_t)seg * nsplit, j, d, s0,
              s1, G, M, Lsum, A);
  s_a[p][d] = A;
  if (d == 0) {
    s_m[p][0] = M;
    s_m[p][1] = Lsum;
  }
  __syncthreads();
  if (p != 0) return;
  float Mt = NEG_INF;
  for (int q = 0; q < np; ++q) Mt = fmaxf(Mt, s_m[q][0]);
  const int h = seg % Hkv, bi = seg / Hkv;
  const size_t orow = (size_t)bi * Hkv * G + (size_t)h * G + j;
  if (Mt == NEG_INF) {
    out[orow * D + d] = 0.f;
    if (d == 0 && lse) lse[orow] = NEG_INF;
    return;
  }
  float Lt = 0.f, At = 0.f;
  for (int q = 0; q < np; ++q) {
    const float mq = s_m[q][0];
    const float wt = mq == NEG_INF ? 0.f : exp2_fast(mq - Mt);
    Lt += s_m[q][1] * wt;
    At += s_a[q][d] * wt;
  }
  out[orow * D + d] = At / Lt;
  if (d == 0 && lse) lse[orow] = (Mt + __log2f(Lt)) * 0.69314718055994530942f;
}

// Arguments of the attention pass.  The partials of a segment occupy nsplit
// slots: slot s covers entries [s * split, (s + 1) * split) of the attention
// set (selected entries first, then the window), split being 128, 256 or
// 384 as chosen by attn_split(); the merge combines the slots in this order.
struct AttnArgs {
  const uint16_t *q;
  const void *K, *V;                  // full cache (selected far rows)
  const uint16_t *Ks, *Vs;
  const void *Kh, *Vh;                // window rows: hot ring of W_hot slots (or the full cache)
  const uint16_t *Ksh, *Vsh;
  int W_hot;
  const int32_t *seq_len, *idx;
  const uint16_t *Kp, *Vp;
  float sm_log2;
  int R, Hkv, T_max, NB, window, pool, topk, nsplit;
  int split;                          // entries per slot: attn_split() of the shape
  int kmax;                           // selected entries per row at most: topk, or 0 (dense step)
  float2 *part_ml;
  float *part_acc;
};

// K rows are staged in LDS for bf16 rows only (see attn_body): int8 and int4
// rows go from the loads to the products, and their workgroups, at 45 KB of
// LDS, fit three to a CU.
template <int DT>
constexpr bool attn_kstage() { return DT == SKS_KV_BF16; }
template <bool KSTAGE>
struct AttnLds {
  __align__(16) uint16_t s_v[4][AM_TILE * VROW];     // V tile per wave
  __align__(16) uint16_t s_k[KSTAGE ? 4 : 1][KSTAGE ? AM_TILE * KROW : 8];   // K tile per wave
  __align__(16) uint16_t s_p[4][2][AM_TILE * 16];    // P hi / lo [entry][head]
  float s_ml[4][16][2];
#if SKS_ATTN_VALU
  __align__(16) uint16_t s_q[16 * D];                // (VALU variant) Q, bf16 [head][dim]
  float s_alpha[4][16];                              // (VALU variant) this tile's rescale per head
#endif
};

// One attention slot (see AttnArgs) of one segment, by a workgroup of
// AT_THREADS threads, TILES tiles of AM_TILE entries per wave.
// idx, seq_len, topk, R and Hkv are those of `a`, passed separately: the
// kernel takes them as scalar arguments ahead of the struct, so that they
// arrive preloaded in SGPRs and the first loads need not wait for the
// argument fetch.
template <int G, int DT, bool POOLED, int TILES>
__device__ void attn_body(const AttnArgs &a, const int32_t *__restrict__ idx,
                          const int32_t *__restrict__ seq_len, int topk, int R, int Hkv,
                          int seg, int slot, AttnLds<attn_kstage<DT>()> &L) {
  static_assert(G >= 1 && G <= 16, "query heads per KV head");
  constexpr int WAVE_ENTRIES = TILES * AM_TILE;
  constexpr int SPLIT = attn_split_entries<TILES>();
  static_assert(WAVE_ENTRIES <= 128, "two entry descriptors per lane");
  constexpr bool TWO = WAVE_ENTRIES > 64;            // the second descriptor is used
  const uint16_t *__restrict__ q = a.q;
  const void *__restrict__ K = a.K;
  const void *__restrict__ V = a.V;
  const uint16_t *__restrict__ Ks = a.Ks;
  const uint16_t *__restrict__ Vs = a.Vs;
  const uint16_t *__restrict__ Kp = a.Kp;
  const uint16_t *__restrict__ Vp = a.Vp;
  const float sm_log2 = a.sm_log2;
  const int T_max = a.T_max, NB = a.NB, window = a.window, pool = a.pool;
  uint16_t (*s_v)[AM_TILE * VROW] = L.s_v;
  uint16_t (*s_p)[2][AM_TILE * 16] = L.s_p;
  float (*s_ml)[16][2] = L.s_ml;
  float *s_o = reinterpret_cast<float *>(&s_v[0][0]);          // reused after the loop

  const int h = seg % Hkv, bi = seg / Hkv, i = bi % R, b = bi / R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int Hq = Hkv * G;
  // The selected indices of entries e_wave + lane and e_wave + 64 + lane are
  // loaded together with the length, before it is known whether the entries
  // are selected ones (the addresses are clamped into the segment's idx row,
  // so always in bounds).
  const int e_wave = slot * SPLIT + wave * WAVE_ENTRIES;
  const int32_t *idx_row = idx + (size_t)seg * topk;
  const int sel0 = idx_row[min(e_wave + lane, topk - 1)];
  const int sel1 = TWO ? idx_row[min(e_wave + 64 + lane, topk - 1)] : -1;
  const int L0 = clamp_len(seq_len[b], T_max, R);
  const RowGeom rg = row_geom(L0, i, window, pool, a.kmax);
  const int e_hi = min((slot + 1) * SPLIT, rg.n_ent);   // end of this slot's entries

  // Descriptor of an entry: the row to gather and whether it takes part
  // (bit 0).  The row indexes the token rows of the full cache, the pooled
  // rows when bit 1 is set, or the slots of the hot ring when bit 2 is set
  // (window rows).  A window row older than the ring holds (positions below
  // ring_lo; only the dense step's longer window reaches them) comes from the
  // full cache.  Invalid entries point at ring slot 0, which always exists,
  // so the gathers below need no branches.  Lane l holds entries e_wave + l
  // (row0, flag0) and e_wave + 64 + l (row1, flag1).
  const int W_hot = a.W_hot;
  const int ring_lo = L0 + R - 1 - W_hot;
  auto describe = [&](int e, int sel, int &row, int &flag) {
    row = 0;
    flag = 4;
    if (e >= e_hi) {
      // past this slot: masked
    } else if (e < rg.k_eff) {
      if ((unsigned)sel < (unsigned)rg.n_far) {
        row = sel;
        flag = POOLED ? 3 : 1;
      }
    } else if (e < rg.n_ent) {
      // (pooled caches have no hot tier: the ring is the full cache)
      const int pos = rg.ws + (e - rg.k_eff);
      if (!POOLED && pos < ring_lo) {
        row = pos;
        flag = 1;
      } else {
        row = POOLED ? pos : hot_slot(pos, W_hot);
        flag = 5;
      }
    }
  };
  int row0, flag0, row1 = 0, flag1 = 4;
  describe(e_wave + lane, sel0, row0, flag0);
  if constexpr (TWO) describe(e_wave + 64 + lane, sel1, row1, flag1);
  // descriptor of wave entry j (a compile-time tile offset plus a lane value)
  auto desc = [&](int j, int &r, int &f) {
    if (!TWO || j < 64) {
      r = __shfl(row0, j);
      f = __shfl(flag0, j);
    } else {
      r = __shfl(row1, j - 64);
      f = __shfl(flag1, j - 64);
    }
  };

  // Q as the A operand: head n, the 8 dims of MFMA step c that lane group g
  // holds (zero rows past G).  The dot product does not depend on how the
  // 128 dims are spread over the steps, as long as Q and K use the same
  // spread: bf16 takes dims 32c + 8g .. +8; int8 takes 16 consecutive dims
  // per pair of steps, (c / 2) * 64 + 16g + (c % 2) * 8 .. +8, so that a lane
  // reads 16 bytes of an int8 row at once; int4 takes dims 32g + 8c .. +8, so
  // that the 16 bytes of a lane's int4 K load cover its four steps.
  auto qdim = [&](int c) {
    return DT == SKS_KV_I8   ? (c >> 1) * 64 + 16 * g + (c & 1) * 8
           : DT == SKS_KV_I4 ? 32 * g + 8 * c
                             : 32 * c + 8 * g;
  };
  u32x4_t qa[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    qa[c] = u32x4_t{0, 0, 0, 0};
    if (n < G) {
      const uint4 w = *reinterpret_cast<const uint4 *>(
          q + ((size_t)bi * Hq + (size_t)h * G + n) * D + qdim(c));
      if constexpr (DT == SKS_KV_I4)      // the slot order of the int4 K operand
        qa[c] = u32x4_t{(w.x & 0xffffu) | (w.y << 16), (w.z & 0xffffu) | (w.w << 16),
                        (w.x >> 16) | (w.y & 0xffff0000u), (w.z >> 16) | (w.w & 0xffff0000u)};
      else
        qa[c] = u32x4_t{w.x, w.y, w.z, w.w};
    }
  }
  constexpr bool VALU = SKS_ATTN_VALU && DT == SKS_KV_BF16;
#if SKS_ATTN_VALU
  // (VALU variant) every wave stages the group's Q in LDS (the same values:
  // each wave reads back its own writes)
  if constexpr (VALU) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (n < G)
        *reinterpret_cast<u32x4_t *>(L.s_q + n * D + qdim(c)) = qa[c];
    wave_lds_sync();
  }
  float ov[VALU ? G : 1][2];                         // (VALU variant) O[h][dims 2 lane, 2 lane + 1]
#pragma unroll
  for (int h = 0; h < (VALU ? G : 1); ++h) ov[h][0] = ov[h][1] = 0.f;
#endif
  // int8 / int4 caches: each lane's entries' row scales, with the descriptors
  float ksd0 = 1.f, vsd0 = 1.f, ksd1 = 1.f, vsd1 = 1.f;
  if constexpr (DT != SKS_KV_BF16) {
    const uint16_t *Kst = Ks + ((size_t)b * Hkv + h) * T_max;
    const uint16_t *Vst = Vs + ((size_t)b * Hkv + h) * T_max;
    const uint16_t *Ksht = a.Ksh + ((size_t)b * Hkv + h) * W_hot;
    const uint16_t *Vsht = a.Vsh + ((size_t)b * Hkv + h) * W_hot;
    ksd0 = f16_bits_to_float(((flag0 & 4) ? Ksht : Kst)[row0]);
    vsd0 = f16_bits_to_float(((flag0 & 4) ? Vsht : Vst)[row0]);
    if constexpr (TWO) {
      ksd1 = f16_bits_to_float(((flag1 & 4) ? Ksht : Kst)[row1]);
      vsd1 = f16_bits_to_float(((flag1 & 4) ? Vsht : Vst)[row1]);
    }
  }

  // int4: the K operand is code + I4_BIAS, so each logit carries
  // I4_BIAS * sum_d q_d of its head; kb4[j] is that term for head 4g + j
  // (Q times a B operand of ones: the same matrix-core arithmetic)
  float kb4[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (DT == SKS_KV_I4) {
    f32x4_t qs = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const u32x4_t ones = u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
    for (int c = 0; c < 4; ++c) qs = mfma_bf16(qa[c], ones, qs);
#pragma unroll
    for (int j = 0; j < 4; ++j) kb4[j] = I4_BIAS * qs[j];
  }
  float c4[4] = {0.f, 0.f, 0.f, 0.f};        // int4: sum of the PV weights per head (see below)

  f32x4_t o[8];
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) o[blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m4[4], l4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m4[j] = NEG_INF;
    l4[j] = 0.f;
  }

  constexpr int RB = DT == SKS_KV_BF16 ? 2 * D : DT == SKS_KV_I8 ? D : D / 2;   // row bytes
  const char *Kt = static_cast<const char *>(K) + ((size_t)b * Hkv + h) * T_max * RB;
  const char *Vt = static_cast<const char *>(V) + ((size_t)b * Hkv + h) * T_max * RB;
  const char *Kht = static_cast<const char *>(a.Kh) + ((size_t)b * Hkv + h) * W_hot * RB;
  const char *Vht = static_cast<const char *>(a.Vh) + ((size_t)b * Hkv + h) * W_hot * RB;
  const char *Kpb = reinterpret_cast<const char *>(Kp) + (POOLED ? ((size_t)b * Hkv + h) * NB * D * 2 : 0);
  const char *Vpb = reinterpret_cast<const char *>(Vp) + (POOLED ? ((size_t)b * Hkv + h) * NB * D * 2 : 0);
  uint16_t *sv = s_v[wave];

  // Raw gathered data of one tile, as loaded (staged in LDS and converted to
  // bf16 only when the tile is consumed, so that the next tile's loads stay
  // in flight meanwhile).  Load qq of a tile reads 16 bytes of chunk
  // (x & (2^VSH - 1)) of tile row (x >> VSH), x = 64 qq + lane: whole rows
  // per load.
  // bf16: V and K: 8 loads each (8 dims per chunk);
  // int8: V: 4 loads (16 dims per chunk); K is read in the operand layout,
  //       lane (n, g) of sub-tile t taking bytes 16g and 64 + 16g of entry
  //       16t + n (two loads);
  // int4: V: 2 loads (32 dims per chunk); K is read in the operand layout
  //       itself, lane (n, g) of sub-tile t taking dims 32g .. +32 of entry
  //       16t + n (16 bytes: a 64-byte row is read whole by four lanes).
  constexpr bool I8 = DT == SKS_KV_I8, I4 = DT == SKS_KV_I4, Q = I8 || I4;
  constexpr int KLD = I4 ? 1 : I8 ? 2 : 4;           // K loads per sub-tile
  constexpr int VLD = I4 ? 2 : I8 ? 4 : 8;           // V loads per tile
  constexpr int VSH = I4 ? 2 : I8 ? 3 : 4;           // log2(V loads per row)
  // bf16: K rows are gathered like V rows and staged in LDS, from where each
  // lane reads its MFMA operand (read in the operand layout, a load would
  // take 64 bytes of each of 16 rows).  int8 rows are read in the operand
  // layout (64 bytes of each of 16 rows per load): staging them too measured
  // slower, its LDS leaving room for two workgroups per CU instead of three.
  constexpr bool KLDS = attn_kstage<DT>();
  uint16_t *sk = L.s_k[KLDS ? wave : 0];
  struct Tile {
    uint4 k[2][KLD];       // bf16: K loads 0 .. 2 KLD - 1; int8 / int4: sub-tile t's operand
    uint4 v[VLD];
    int f[2];              // flags of the two K entries of this lane
    float ks[2], vs[2];    // int8 / int4 row scales of the two K entries
  };
  // K/V rows are read once per step: nontemporal loads keep them from
  // evicting lines that are reused.
  auto ld = [](const char *p) -> uint4 {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  // Every descriptor of the tile is fetched first (lane permutes through the
  // LDS unit: one round trip for all of them), then every load is issued.
  // Interleaved, each load would wait for its own permute.
  auto gather = [&](int tile, Tile &d) {
    int kr[2], kf[2], vr[VLD], vf[VLD];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = tile * AM_TILE + 16 * t + n;
      desc(j, kr[t], kf[t]);
      d.f[t] = kf[t];
      if constexpr (Q) {
        d.ks[t] = (!TWO || j < 64) ? __shfl(ksd0, j) : __shfl(ksd1, j - 64);
        d.vs[t] = (!TWO || j < 64) ? __shfl(vsd0, j) : __shfl(vsd1, j - 64);
      }
    }
#pragma unroll
    for (int qq = 0; qq < VLD; ++qq) desc(tile * AM_TILE + ((qq * 64 + lane) >> VSH), vr[qq], vf[qq]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (I4) {
#pragma unroll
      for (int t = 0; t < 2; ++t) d.k[t][0] = ld(((kf[t] & 4) ? Kht : Kt) + (size_t)kr[t] * RB + 16 * g);
    }
    if constexpr (I8) {
      // int8 rows in the operand layout (lane (n, g): bytes 16g and 64 + 16g)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const char *kb = ((kf[t] & 4) ? Kht : Kt) + (size_t)kr[t] * RB + 16 * g;
        d.k[t][0] = ld(kb);
        d.k[t][1] = ld(kb + 64);
      }
    }
#pragma unroll
    for (int qq = 0; qq < VLD; ++qq) {
      const int c = (qq * 64 + lane) & ((1 << VSH) - 1);
      const int r = vr[qq], f = vf[qq];
      const char *vbase = (POOLED && (f & 2)) ? Vpb : (!POOLED && (f & 4)) ? Vht : Vt;
      if constexpr (KLDS) {
        const char *kb = (POOLED && (f & 2)) ? Kpb : (!POOLED && (f & 4)) ? Kht : Kt;
        d.k[qq / KLD][qq % KLD] = ld(kb + (size_t)r * RB + c * 16);
      }
      d.v[qq] = ld(vbase + (size_t)r * RB + c * 16);
    }
  };
  // K operand of MFMA step c as 8 bf16 (int8 codes convert exactly; int4
  // codes as code + I4_BIAS, also exact)
  // (bf16: from the staged rows, lane (n, g) reading the 16 bytes of entry
  // 16t + n that qdim assigns to it)
  auto kop = [&](const Tile &d, int t, int c) -> u32x4_t {
    if constexpr (I4) {
      const uint4 &w = d.k[t][0];
      return i4_biased_bf16x8(c == 0 ? w.x : c == 1 ? w.y : c == 2 ? w.z : w.w);
    } else if constexpr (I8) {
      const uint4 &w = d.k[t][c >> 1];
      const uint32_t a = (c & 1) ? w.z : w.x, bb = (c & 1) ? w.w : w.y;
      return u32x4_t{i8pair_to_bf16x2(a, 0), i8pair_to_bf16x2(a, 16), i8pair_to_bf16x2(bb, 0),
                     i8pair_to_bf16x2(bb, 16)};
    } else {
      return *reinterpret_cast<const u32x4_t *>(sk + (16 * t + n) * KROW + 32 * c + 8 * g);
    }
  };

  // stage V (row-major bf16, 16-byte stores)
  auto stage_v = [&](const Tile &d) {
#pragma unroll
    for (int qq = 0; qq < VLD; ++qq) {
      const int x = qq * 64 + lane;
      const uint4 &w = d.v[qq];
      if constexpr (I4) {
        // 32 dims as code + I4_BIAS (the bias is removed from O at the end),
        // each group of 8 columns in I4_ORDER (undone when O is written)
        const int ev = x >> 2, c = x & 3;
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        uint4 *dst = reinterpret_cast<uint4 *>(sv + ev * VROW + c * 32);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const u32x4_t bv = i4_biased_bf16x8(ws[k]);
          dst[k] = make_uint4(bv[0], bv[1], bv[2], bv[3]);
        }
      } else if constexpr (I8) {
        const int ev = x >> 3, c = x & 7;
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        uint4 *dst = reinterpret_cast<uint4 *>(sv + ev * VROW + c * 16);
#pragma unroll
        for (int k = 0; k < 2; ++k)
          dst[k] = make_uint4(i8pair_to_bf16x2(ws[2 * k], 0), i8pair_to_bf16x2(ws[2 * k], 16),
                              i8pair_to_bf16x2(ws[2 * k + 1], 0), i8pair_to_bf16x2(ws[2 * k + 1], 16));
      } else {
        const int ev = x >> 4, c = x & 15;
        *reinterpret_cast<uint4 *>(sv + ev * VROW + c * 8) = w;
      }
    }
  };

  const float pinf = opaque_inf();
  auto consume = [&](const Tile &d) {
    if constexpr (KLDS) {
      // K rows as stored (16-byte stores) and V, then the operand reads
#pragma unroll
      for (int qq = 0; qq < VLD; ++qq) {
        const int x = qq * 64 + lane;
        const int ev = x >> VSH, c = x & ((1 << VSH) - 1);
        *reinterpret_cast<uint4 *>(sk + ev * KROW + c * 8) = d.k[qq / KLD][qq % KLD];
      }
      stage_v(d);
      wave_lds_sync();
    }
    // ---- QK on the matrix cores
    f32x4_t sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#if SKS_ATTN_VALU
      if constexpr (VALU) {
        // (VALU variant) this lane's 32 dims of entry 16t + n against every
        // head's Q (dot2 on bf16 pairs), then the four lane groups summed
        float part[G];
#pragma unroll
        for (int h = 0; h < G; ++h) part[h] = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4_t kv = kop(d, t, c);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const u32x4_t qv = *reinterpret_cast<const u32x4_t *>(L.s_q + h * D + qdim(c));
#pragma unroll
            for (int w = 0; w < 4; ++w) part[h] = dot2_bf16(qv[w], kv[w], part[h]);
          }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          part[h] += __shfl_xor(part[h], 16);
          part[h] += __shfl_xor(part[h], 32);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float v = 0.f;
#pragma unroll
          for (int h = 0; h < G; ++h) v = h == 4 * g + j ? part[h] : v;
          sacc[t][j] = v;
        }
      }
#endif
    }
    if constexpr (!VALU) {
      // all eight K operands first (LDS reads in flight together), then the products
      u32x4_t kb[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c) kb[t][c] = kop(d, t, c);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < 4; ++c) sacc[t] = mfma_bf16(qa[c], kb[t][c], sacc[t]);
    }

    if constexpr (!KLDS) stage_v(d);

    // ---- online softmax on the C layout (lane: heads 4g + j, entry n of each sub-tile)
    float ksc[2], vsc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      ksc[t] = Q ? d.ks[t] : 1.f;
      vsc[t] = Q ? d.vs[t] : 1.f;
    }
    float z[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        z[t][j] = (d.f[t] & 1) ? (sacc[t][j] - kb4[j]) * ksc[t] * sm_log2 : NEG_INF;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float mx = row16_max_f(fmaxf(z[0][j], z[1][j]), pinf);
      float alpha = 1.f;
      if (mx > m4[j] + RESCALE_SLACK || (m4[j] == NEG_INF && mx != NEG_INF)) {
        alpha = m4[j] == NEG_INF ? 0.f : exp2_fast(m4[j] - mx);
        l4[j] *= alpha;
        if constexpr (I4) c4[j] *= alpha;
        if constexpr (!VALU) {
#pragma unroll
          for (int blk = 0; blk < 8; ++blk) o[blk][j] *= alpha;
        }
        m4[j] = mx;
      }
#if SKS_ATTN_VALU
      if (VALU && n == 0) L.s_alpha[wave][4 * g + j] = alpha;
#endif
    }
    uint16_t *sp_hi = s_p[wave][0], *sp_lo = s_p[wave][1];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float pw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pv = (z[t][j] == NEG_INF) ? 0.f : exp2_fast(z[t][j] - m4[j]);
        l4[j] += pv;
        pw[j] = pv * vsc[t];                                // value scale folded in
#if SKS_ATTN_VALU
        // (VALU variant) P in fp32, [entry][16 heads] over the hi / lo area
        if constexpr (VALU) reinterpret_cast<float *>(sp_hi)[(16 * t + n) * 16 + 4 * g + j] = pw[j];
#endif
      }
      if constexpr (!VALU) {
        // bf16 hi + lo parts, two heads per conversion, stored as P^T
        // [entry][16 heads]: this lane's four heads of entry 16t + n
        const uint32_t h01 = bf16x2_rne(pw[0], pw[1]), h23 = bf16x2_rne(pw[2], pw[3]);
        const float hf[4] = {__uint_as_float(h01 << 16), __uint_as_float(h01 & 0xffff0000u),
                             __uint_as_float(h23 << 16), __uint_as_float(h23 & 0xffff0000u)};
        const uint32_t l01 = bf16x2_rne(pw[0] - hf[0], pw[1] - hf[1]);
        const uint32_t l23 = bf16x2_rne(pw[2] - hf[2], pw[3] - hf[3]);
        if constexpr (I4) {
          const float lf[4] = {__uint_as_float(l01 << 16), __uint_as_float(l01 & 0xffff0000u),
                               __uint_as_float(l23 << 16), __uint_as_float(l23 & 0xffff0000u)};
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) c4[jj] += hf[jj] + lf[jj];
        }
        const int at = (16 * t + n) * 16 + 4 * g;
        *reinterpret_cast<uint2 *>(sp_hi + at) = make_uint2(h01, h23);
        *reinterpret_cast<uint2 *>(sp_lo + at) = make_uint2(l01, l23);
      }
    }
    wave_lds_sync();

#if SKS_ATTN_VALU
    if constexpr (VALU) {
      // (VALU variant) this lane's two dims for every head: rescale, then
      // the 32 entries' fp32 weights times the staged bf16 V
      const float *pf = reinterpret_cast<const float *>(sp_hi);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float al = L.s_alpha[wave][h];
        ov[h][0] *= al;
        ov[h][1] *= al;
      }
#pragma unroll 8
      for (int e = 0; e < AM_TILE; ++e) {
        const uint32_t vw = *reinterpret_cast<const uint32_t *>(sv + e * VROW + 2 * lane);
        const float v0 = __uint_as_float(vw << 16), v1 = __uint_as_float(vw & 0xffff0000u);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pw = pf[e * 16 + h];
          ov[h][0] = __builtin_fmaf(pw, v0, ov[h][0]);
          ov[h][1] = __builtin_fmaf(pw, v1, ov[h][1]);
        }
      }
      wave_lds_sync();                                      // before the next tile reuses LDS
      return;
    }
#endif
    // ---- PV on the matrix cores: A = P (head n, entries 8g..8g+8), B = V
    // (P^T read back by transpose reads: lane n of group g addressing heads
    // 4 (n % 4) .. +4 of entry e0 + n / 4 ends up with head n of entries
    // e0 .. e0 + 4, and with the second read of e1 .. e1 + 4.  Lane group g
    // takes the MFMA's k-slots 8g .. 8g + 8, here entries e0 = 8g, e1 = 8g + 4
    // for even g and e0 = 8g + 4, e1 = 8g for odd g: P and V take the same
    // order, the product is the same sum, and the two lane groups of each
    // half-wave read rows 32 banks apart instead of the same banks.)
    const int e0 = 8 * g + 4 * (g & 1), e1 = 8 * g + 4 * (~g & 1);
    const int pat0 = (e0 + (n >> 2)) * 16 + 4 * (n & 3), pat1 = (e1 + (n >> 2)) * 16 + 4 * (n & 3);
    const uint2 h0 = lds_read_tr16(sp_hi + pat0), h1 = lds_read_tr16(sp_hi + pat1);
    const uint2 l0 = lds_read_tr16(sp_lo + pat0), l1 = lds_read_tr16(sp_lo + pat1);
    const u32x4_t pa_hi = u32x4_t{h0.x, h0.y, h1.x, h1.y};
    const u32x4_t pa_lo = u32x4_t{l0.x, l0.y, l1.x, l1.y};
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      // lane n of group g addresses dims 16 blk + 4 (n % 4) .. +4 of entry
      // e0 + n / 4 (and of entry e1 + n / 4); transposed, lane n holds dim
      // 16 blk + n of the entries of k-slots 8g .. 8g + 8: the MFMA's B layout
      const uint16_t *p0 = sv + (e0 + (n >> 2)) * VROW + 16 * blk + 4 * (n & 3);
      const uint16_t *p1 = sv + (e1 + (n >> 2)) * VROW + 16 * blk + 4 * (n & 3);
      const uint2 r0 = lds_read_tr16(p0), r1 = lds_read_tr16(p1);
      const u32x4_t vb = u32x4_t{r0.x, r0.y, r1.x, r1.y};
      o[blk] = mfma_bf16(pa_hi, vb, o[blk]);
      o[blk] = mfma_bf16(pa_lo, vb, o[blk]);
    }
    wave_lds_sync();                                        // before the next tile reuses LDS
  };

  // Software pipeline over the wave's tiles: the gathers of tile t + 1 are
  // issued before tile t is consumed, so that the memory system always holds
  // a tile's worth of requests per wave.
  // Straight-line code: every tile is gathered and consumed (entries past the
  // set read row 0 and are masked out), and the scheduling barriers keep each
  // tile's loads in issue order.  The wait counter is in order, so a
  // conditional or a reordered load of tile t + 1 would make tile t wait for
  // it too.
  Tile cur, nxt;
  gather(0, cur);
#pragma unroll
  for (int tile = 0; tile < TILES; ++tile) {
    __builtin_amdgcn_sched_barrier(0);
    if (tile + 1 < TILES) gather(tile + 1, nxt);
    __builtin_amdgcn_sched_barrier(0);
    consume(cur);
    cur = nxt;
  }

  // denominators: sum the lane-partials over the 16 lanes of each DPP row
#pragma unroll
  for (int j = 0; j < 4; ++j) l4[j] = row16_sum_f(l4[j]);
  // int4: O holds sum_j w_j (v_j + I4_BIAS) with w_j the bf16 weights fed to
  // the matrix cores; take out I4_BIAS * sum_j w_j
  if constexpr (I4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float cb = I4_BIAS * row16_sum_f(c4[j]);
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) o[blk][j] -= cb;
    }
  }
  __syncthreads();                                          // s_v is reused as s_o below
#if SKS_ATTN_VALU
  if constexpr (VALU) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_o[(wave * G + h) * D + 2 * lane] = ov[h][0];
      s_o[(wave * G + h) * D + 2 * lane + 1] = ov[h][1];
    }
  }
#endif
  // wave partials to LDS: O rows 4g + j < G
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int hh = 4 * g + j;
    if (hh < G) {
#pragma unroll
      for (int blk = 0; blk < (VALU ? 0 : 8); ++blk) {
        // int4: V columns are in I4_ORDER within each group of 8
        const int col = 16 * blk + n;
        const int dim = I4 ? (col & ~7) + i4_slot_dim(col & 7) : col;
        s_o[(wave * G + hh) * D + dim] = o[blk][j];
      }
      if (n == 0) {
        s_ml[wave][hh][0] = m4[j];
        s_ml[wave][hh][1] = l4[j];
      }
    }
  }
  __syncthreads();
  // merge the 4 waves and write this split's partial
  const size_t pbase = (size_t)seg * a.nsplit + slot;
  float2 *__restrict__ part_ml = a.part_ml;
  float *__restrict__ part_acc = a.part_acc;
  for (int x = threadIdx.x; x < G * D; x += AT_THREADS) {
    const int j = x / D, d = x % D;
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_ml[w][j][0]);
    float Lsum = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = s_ml[w][j][0];
      const float wt = mw == NEG_INF ? 0.f : exp2_fast(mw - M);
      Lsum += s_ml[w][j][1] * wt;
      A += s_o[(w * G + j) * D + d] * wt;
    }
    part_acc[(pbase * G + j) * D + d] = A;
    if (d == 0) part_ml[pbase * G + j] = make_float2(M, Lsum);
  }

}

// Entries per attention slot: 128 (one tile per wave) for attention sets of
// fewer than ATTN_SMALL_SET entries, which would otherwise make too few
// workgroups to fill the chip; else 384 (three tiles) for bf16 rows, whose
// gathers need the deeper pipeline, and 256 (two tiles) for int8 / int4
// rows, whose smaller gathers leave each wave's chain of dependent steps the
// longer part.  The split fixes each row's order of operations, so it is a
// function of the per-row parameters only (window, top-k, pooling, KV
// storage): never of the batch size, the rows per sequence or the heads, so
// that a row's results do not depend on what it is decoded with.
inline int attn_split(const Shape &s) {
  const long set = (long)s.topk + s.window + s.pool - 1;   // the largest attention set
  if (set < ATTN_SMALL_SET) return attn_split_entries<1>();
  return s.dtype == SKS_KV_BF16 ? attn_split_entries<3>() : attn_split_entries<2>();
}

// attention slots of a segment (the largest attention set: topk selected
// entries and a window of up to window + pool - 1 tokens)
inline int attn_nsplit(const Shape &s) {
  return ceil_div((long)s.topk + s.window + s.pool - 1, attn_split(s));
}

}  // namespace
}  // namespace sks
