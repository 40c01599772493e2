// Hot tier of the KV cache ("8 agents x 250K context, concurrently, on two
// 3090s", claims list: the full cache in host RAM, a small hot set on the
// GPU, only the picked tokens across PCIe).  Window rows and a step's own
// tokens are read from the hot ring when the cache has one, else from the
// full cache, which then acts as a "ring" of T_max slots (the identity on
// valid positions).
#pragma once

#include "sks_internal.h"

namespace sks {

struct HotRows {
  const void *K, *V;
  const uint16_t *Ks, *Vs;
  int W;
};

inline HotRows hot_rows(const sks_kv &kv) {
  if (kv.K_hot) return HotRows{kv.K_hot, kv.V_hot, kv.K_hot_scale, kv.V_hot_scale, kv.W_hot};
  return HotRows{kv.K, kv.V, kv.K_scale, kv.V_scale, kv.T_max};
}

// ring slot of position pos (0 <= pos < T_max)
__device__ __forceinline__ int hot_slot(int pos, int W) { return pos < W ? pos : pos % W; }

}  // namespace sks
