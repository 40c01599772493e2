// Launchers of the sketch-basis refit (k_refit.hip; the key-scale pass is the
// absmax mode of the matrix-core sketch kernel in k_sketch.hip).
#pragma once

#include "sks_internal.h"

namespace sks {

// Gram partials: workgroups per (b, h) for a key range of `span` positions,
// and the scratch they need.
int refit_gram_chunks(long span);
size_t refit_gram_scratch_bytes(int B, int Hkv, long span);
// G [per_head ? Hkv : 1][128][128] fp64 from keys [t_begin, min(t_end, L_b)).
hipError_t launch_refit_gram(const sks_kv &kv, int t_begin, int t_end, int per_head, double *G,
                             void *ws, hipStream_t st);
// basis [nmat][64][128] fp32 (and eigval [nmat][128], descending) from G;
// ws: nmat * 128 * 128 doubles.
hipError_t launch_refit_basis(const double *G, int nmat, float *basis, double *eigval, void *ws,
                              hipStream_t st);
// Key-scale pass: per-workgroup maxima of |P x| (refit_amax_chunks(span) per
// (b, h)), then key_scale[h] = max / 127.
int refit_amax_chunks(long span);
hipError_t launch_refit_amax(const sks_kv &kv, int t_begin, int t_end, const float *basis,
                             int basis_per_head, float *amax, hipStream_t st);
hipError_t launch_refit_scale_reduce(const float *amax, int B, int Hkv, int nchunk,
                                     float *key_scale, hipStream_t st);

}  // namespace sks
