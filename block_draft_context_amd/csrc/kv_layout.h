// Layout of the per-layer context K and V in the workspace.
//
// The split-K attention streams K and V once per (sequence, head, chunk) and
// wants every wave-wide load to be one contiguous 1 KiB run, so both tensors
// are stored per (layer, K|V, head) in 64-key blocks, in the order the
// attention kernel reads them:
//
//   K: lane t of a wave owns key t of the block and reads its hd values as
//      hd/E vectors of E = 16/sizeof(S) elements:
//        [Tpad/64][hd/E][64 keys][E]
//   V: lane (kg, cp) owns columns 2cp, 2cp+1 and R = E/2 consecutive keys of
//      key group kg (KG = 128/hd groups, KG * hd/2 = 64 lanes):
//        [Tpad/64][hd/8 or hd/4 loads][KG][hd/2][R keys][2 columns]
//
// Rows T .. Tpad-1 hold zeros so that masked keys multiply finite values.
#pragma once

#include <stdint.h>

namespace dspark {

template <typename S>
struct KVLayout {
  static constexpr int E = 16 / (int)sizeof(S);   // elements per 16-byte vector
  static constexpr int R = E / 2;                 // keys per V vector

  __host__ __device__ static inline int64_t head_base(int layer, int kv, int head, int n_heads,
                                                      int64_t Tpad, int hd) {
    return ((int64_t)(layer * 2 + kv) * n_heads + head) * Tpad * hd;
  }
  // element offset of K[t][c] inside one (layer, K, head) slab
  __host__ __device__ static inline int64_t k_off(int64_t t, int c, int hd) {
    return ((t >> 6) * (hd / E) + c / E) * (64 * E) + (t & 63) * E + (c % E);
  }
  // element offset of V[t][c] inside one (layer, V, head) slab
  __host__ __device__ static inline int64_t v_off(int64_t t, int c, int hd) {
    const int KG = 128 / hd;
    const int kk = (int)(t & 63);
    const int ld = kk / (KG * R);
    const int kg = (kk / R) % KG;
    const int vec = ld * 64 + kg * (hd / 2) + c / 2;
    return (t >> 6) * 64 * (int64_t)hd + (int64_t)vec * E + (kk % R) * 2 + (c & 1);
  }
};

}  // namespace dspark
