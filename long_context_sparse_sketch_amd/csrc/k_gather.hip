// Gather/pack of each row's attention set ("What it took" on the page "8
// agents x 250K context, concurrently, on two 3090s": pack the picked tokens
// for the attention kernel).  Selected far entries first (ascending; pooled
// rows when pool > 1), then the exact window, into a dense per-(b, i, h)
// buffer of C = topk + window + pool - 1 row slots.  Rows move as 16-byte
// vectors, a bf16 row being 16 lanes, an int8 row 8 and an int4 row 4.
#include "sks_internal.h"
#include "tier.h"

namespace sks {
namespace {

constexpr int GP_THREADS = 256;
constexpr int GP_ROWS = 64;                        // row slots per workgroup

template <int DT, bool POOLED>
__global__ __launch_bounds__(GP_THREADS) void gather_kernel(
    const void *__restrict__ K, const void *__restrict__ V, const uint16_t *__restrict__ Ks,
    const uint16_t *__restrict__ Vs, const void *__restrict__ Kh, const void *__restrict__ Vh,
    const uint16_t *__restrict__ Ksh, const uint16_t *__restrict__ Vsh, int W_hot,
    const int32_t *__restrict__ seq_len,
    const int32_t *__restrict__ idx, const uint16_t *__restrict__ Kp,
    const uint16_t *__restrict__ Vp, int R, int Hkv, int T_max, int NB, int window, int pool,
    int topk, int C, void *__restrict__ K_out, void *__restrict__ V_out,
    uint16_t *__restrict__ Ks_out, uint16_t *__restrict__ Vs_out, int32_t *__restrict__ n_out) {
  constexpr int ROW_BYTES = DT == SKS_KV_BF16 ? D * 2 : DT == SKS_KV_I8 ? D : D / 2;
  constexpr int VECS = ROW_BYTES / 16;
  const int seg = blockIdx.y;
  const int h = seg % Hkv, bi = seg / Hkv, i = bi % R, b = bi / R;
  const RowGeom rg = row_geom(clamp_len(seq_len[b], T_max, R), i, window, pool, topk);
  if (blockIdx.x == 0 && threadIdx.x == 0) n_out[seg] = rg.n_ent;
  const int e0 = blockIdx.x * GP_ROWS;
  if (e0 >= rg.n_ent) return;
  const int32_t *idx_row = idx + (size_t)seg * topk;
  const size_t tok_base = ((size_t)b * Hkv + h) * T_max;
  const size_t hot_base = ((size_t)b * Hkv + h) * W_hot;
  const size_t blk_base = ((size_t)b * Hkv + h) * NB;
  const size_t out_base = (size_t)seg * C;

  for (int x = threadIdx.x; x < GP_ROWS * VECS; x += GP_THREADS) {
    const int e = e0 + x / VECS, v = x % VECS;
    if (e >= rg.n_ent) break;
    bool ok = true, from_pool = false, hot = false;
    size_t row;
    if (e < rg.k_eff) {
      const int sel = idx_row[e];
      ok = (unsigned)sel < (unsigned)rg.n_far;
      from_pool = POOLED;
      row = POOLED ? blk_base + (size_t)sel : tok_base + (size_t)sel;
    } else {
      hot = true;                         // window rows: hot ring (or the full cache)
      row = hot_base + (size_t)hot_slot(rg.ws + (e - rg.k_eff), W_hot);
    }
    uint4 kv4 = make_uint4(0, 0, 0, 0), vv4 = make_uint4(0, 0, 0, 0);
    if (ok) {
      const char *Kb = from_pool ? reinterpret_cast<const char *>(Kp)
                       : hot     ? static_cast<const char *>(Kh)
                                 : static_cast<const char *>(K);
      const char *Vb = from_pool ? reinterpret_cast<const char *>(Vp)
                       : hot     ? static_cast<const char *>(Vh)
                                 : static_cast<const char *>(V);
      kv4 = reinterpret_cast<const uint4 *>(Kb + row * ROW_BYTES)[v];
      vv4 = reinterpret_cast<const uint4 *>(Vb + row * ROW_BYTES)[v];
    }
    reinterpret_cast<uint4 *>(static_cast<char *>(K_out) + (out_base + e) * ROW_BYTES)[v] = kv4;
    reinterpret_cast<uint4 *>(static_cast<char *>(V_out) + (out_base + e) * ROW_BYTES)[v] = vv4;
  }
  if constexpr (DT != SKS_KV_BF16) {
    const int e = e0 + threadIdx.x;
    if (threadIdx.x < GP_ROWS && e < rg.n_ent) {
      bool ok = true, hot = false;
      size_t row;
      if (e < rg.k_eff) {
        const int sel = idx_row[e];
        ok = (unsigned)sel < (unsigned)rg.n_far;
        row = tok_base + (size_t)sel;
      } else {
        hot = true;
        row = hot_base + (size_t)hot_slot(rg.ws + (e - rg.k_eff), W_hot);
      }
      Ks_out[out_base + e] = ok ? (hot ? Ksh : Ks)[row] : (uint16_t)0;
      Vs_out[out_base + e] = ok ? (hot ? Vsh : Vs)[row] : (uint16_t)0;
    }
  }
}

}  // namespace

hipError_t launch_gather(const sks_kv &kv, const Shape &s, const int32_t *idx,
                         const uint16_t *Kp, const uint16_t *Vp, void *K_out, void *V_out,
                         uint16_t *Ks_out, uint16_t *Vs_out, int32_t *n_out, hipStream_t st) {
  const int C = s.topk + s.window + s.pool - 1;
  dim3 grid(ceil_div(C, GP_ROWS), s.B * s.R * s.Hkv);
  const HotRows hr = hot_rows(kv);
#define SKS_GATHER(DT, PO)                                                                         \
  gather_kernel<DT, PO><<<grid, GP_THREADS, 0, st>>>(kv.K, kv.V, kv.K_scale, kv.V_scale, hr.K,   \
                                                     hr.V, hr.Ks, hr.Vs, hr.W, kv.seq_len, idx,  \
                                                     Kp, Vp, s.R, s.Hkv,                         \
                                                     s.T_max, s.NB, s.window, s.pool, s.topk, C, \
                                                     K_out, V_out, Ks_out, Vs_out, n_out)
  if (s.dtype == SKS_KV_I8)
    SKS_GATHER(SKS_KV_I8, false);
  else if (s.dtype == SKS_KV_I4)
    SKS_GATHER(SKS_KV_I4, false);
  else if (s.pool > 1)
    SKS_GATHER(SKS_KV_BF16, true);
  else
    SKS_GATHER(SKS_KV_BF16, false);
#undef SKS_GATHER
  return hipGetLastError();
}

}  // namespace sks
