// Eq 3 block attention over [context ++ block], split over context chunks,
// and the attention output projection.
//
// The gamma block queries of sequence b attend to its L_b context keys and
// its gamma block keys with no causal mask (module-dflash.ts, #layer). The
// context part is long and read once per layer, so it is split into chunks
// of `chunk` keys: one workgroup per (chunk, head) streams the chunk's K and
// V once and leaves an unnormalised partial (m, l, o) per query, as the
// split-chunk attention + combine kernels of dspark-runtime.js do. A second
// kernel merges those partials together with the gamma block keys by the
// log-sum-exp identity
//   M = max_c m_c,  l = sum_c l_c 2^(m_c - M),  o = sum_c o_c 2^(m_c - M) / l
// and applies W_o head by head: E = D + sum_h o_h W_o[:, h]^T (#layer's
// output projection and residual).
// Scores are kept in base 2: Q arrives pre-multiplied by hd^-1/2 * log2(e).
//
// Work split inside a chunk: each wave takes every fourth 64-key block, with
// the next block's loads in flight while the current one is computed. For
// Q.K^T lane t owns key t and reads its whole key row (hd/E 16-byte vectors,
// one 1 KiB wave-wide run each, see kv_layout.h). For P.V lane (kg, cp) owns two value
// columns and R keys per load, so each V load is again one 1 KiB run; the
// block's probabilities are broadcast through LDS. All arithmetic runs on the
// vector ALUs, accumulating in float32: with gamma <= 16 queries the
// arithmetic intensity is a few flop per byte, far below the matrix cores'.
// With bf16 storage the long-context kernel multiplies bf16 pairs
// (v_dot2_f32_bf16), Q and the probabilities rounded to bf16 once; the rest
// multiplies in float32.
#include "common.h"
#include "kernels.h"
#include "kv_layout.h"

namespace dspark {

constexpr float kNegInf = -__builtin_inff();

int64_t attention_tiles(const int32_t* cu_host, int A, int chunk) {
  int64_t n = 0;
  for (int b = 0; b < A; ++b) {
    const int64_t L = cu_host[b + 1] - cu_host[b];
    n += L > 0 ? (L + chunk - 1) / chunk : 1;
  }
  return n;
}

// Keys per chunk. Short contexts (at most ~1024 64-key blocks over all
// heads) use one block per tile and the head-split kernel, whose four waves
// share each block. Longer ones use the streaming kernel, aiming first for
// ~512 (chunk, head) workgroups of at least 256 keys. The streaming kernel
// holds one 256-thread workgroup per CU at its register use, so kAttnSlots
// workgroups run at once. Where that aim gives chunks of 1024 keys or more,
// a last partly filled round of such long chunks costs more than it saves.
// There the chunk comes from a ladder of sizes: the one with the fewest
// rounds of kAttnSlots workgroups times the keys a workgroup streams plus a
// fixed cost of about 256 keys per workgroup, the larger on ties (fewer
// partials to merge). The per-sequence rounding of ragged lengths is counted
// exactly. Shorter chunks keep the first aim, which measured faster there.
constexpr int kAttnSlots = 256;

int attention_chunk(const int32_t* cu_host, int A, int n_heads) {
  const int64_t T = cu_host[A] - cu_host[0];
  const int64_t blocks = (T + 63) / 64 + A;   // bound on sum_b ceil(L_b / 64)
  if (blocks * n_heads <= 1024) return 64;
  int64_t c = (T * n_heads + 511) / 512;
  c = ((c + 63) / 64) * 64;
  if (c < 256) c = 256;
  if (c > 16384) c = 16384;
  if (c < 1024) return (int)c;
  static const int ladder[] = {1024, 1280, 1536, 1792, 2048, 2560, 3072, 3584,
                               4096, 5120, 6144, 7168, 8192, 10240, 12288, 14336, 16384};
  int best = ladder[0];
  int64_t best_cost = -1;
  for (int lc : ladder) {
    const int64_t wg = attention_tiles(cu_host, A, lc) * n_heads;
    const int64_t cost = ((wg + kAttnSlots - 1) / kAttnSlots) * (lc + 256);
    if (best_cost < 0 || cost <= best_cost) {
      best_cost = cost;
      best = lc;
    }
  }
  return best;
}

// Sequence and key range [k0, k1) of a split-K tile; false past the plan.
// The tile prefix (device plan) is searched for the owning sequence; with one
// sequence the range follows from the tile index and the context length T1,
// so the K/V loads need no dependent memory access first. Sequence b's keys
// start at row cu[b] of the slab (a packed context) or at b * seq_stride (a
// draft cache of seq_stride rows per sequence); there are cu[b+1] - cu[b].
struct TileRange {
  int b;
  int64_t k0, k1;   // the tile's chunk of keys
  int64_t s0, s1;   // the sequence's keys
  int c, nt;        // the tile's index among its sequence's nt tiles
};
DSPARK_DEV bool tile_range(int tile, int A, int64_t T1, const int32_t* __restrict__ cu,
                           const int32_t* __restrict__ prefix, int chunk, int total_tiles,
                           int64_t seq_stride, TileRange& r) {
  if (tile >= total_tiles) return false;
  if (A == 1) {
    r.b = 0;
    r.k0 = min(T1, (int64_t)tile * chunk);
    r.k1 = min(T1, r.k0 + chunk);
    r.s0 = 0;
    r.s1 = T1;
    r.c = tile;
    r.nt = total_tiles;
    return true;
  }
  if (tile >= prefix[A]) return false;
  // sequence owning this tile: largest b with prefix[b] <= tile
  int lo = 0, hi = A - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  r.b = lo;
  const int c = tile - prefix[lo];
  const int64_t kseq0 = seq_stride > 0 ? (int64_t)lo * seq_stride : cu[lo];
  const int64_t kseq1 = kseq0 + (cu[lo + 1] - cu[lo]);
  r.k0 = min(kseq1, kseq0 + (int64_t)c * chunk);
  r.k1 = min(kseq1, r.k0 + chunk);
  r.s0 = kseq0;
  r.s1 = kseq1;
  r.c = c;
  r.nt = prefix[lo + 1] - prefix[lo];
  return true;
}

// ---------------------------------------------------------------------------
// partials: grid (total_tiles, n_heads), 256 threads (4 waves)
// part_o  [total_tiles][n_heads][G][HD]   unnormalised output
// part_ml [total_tiles][n_heads][G][2]    (max, sum) in base-2 units
// ---------------------------------------------------------------------------
template <typename S, int HD, int G>
__global__ __launch_bounds__(256) void attn_partial_kernel(
    const float* __restrict__ Q, const S* __restrict__ kv_base, int64_t Tpad, int n_heads, int n_kv, int layer,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ prefix, int A, int64_t T1, int chunk,
    int total_tiles, int64_t seq_stride, const uint8_t* __restrict__ key_mask, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  using L = KVLayout<S>;
  constexpr int E = L::E, R = L::R;
  constexpr int NKV = HD / E;            // K vectors per key row
  constexpr int KG = 128 / HD;           // key groups in the P.V lane split
  constexpr int NLD = 64 / (KG * R);     // V loads per 64-key block

  // bf16 storage multiplies bf16 pairs with v_dot2_f32_bf16 (f32
  // accumulation): Q and the block's probabilities are rounded to bf16 once,
  // K and V are used as stored, which halves the vector ALU work that bounds
  // this kernel. f32 storage keeps f32 products throughout.
  constexpr bool kDot2 = sizeof(S) == 2;
  __shared__ __attribute__((aligned(16))) float qs[kDot2 ? 1 : G][HD];
  __shared__ __attribute__((aligned(16))) float ps[kDot2 ? 1 : 4][G][64];
  __shared__ __attribute__((aligned(16))) uint32_t qb[kDot2 ? G : 1][HD / 2];   // bf16 pairs
  __shared__ __attribute__((aligned(16))) uint16_t pb[kDot2 ? 4 : 1][G][64];    // bf16 bits
  __shared__ float red_m[4][G];
  __shared__ float red_l[4][G];
  __shared__ __attribute__((aligned(16))) float red_o[4][G][HD];

  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  TileRange tr;
  if (!tile_range(tile, A, T1, cu, prefix, chunk, total_tiles, seq_stride, tr)) return;
  const int b = tr.b;
  // the sequence's keys; this tile owns every nt-th of its 64-key blocks
  const int64_t k0 = tr.s0, k1 = tr.s1;

  // query head h reads the K/V of head h / (n_heads / n_kv) (grouped K/V heads)
  const int kvh = h / (n_heads / n_kv);
  const S* __restrict__ Kh = kv_base + L::head_base(layer, 0, kvh, n_kv, Tpad, HD);
  const S* __restrict__ Vh = kv_base + L::head_base(layer, 1, kvh, n_kv, Tpad, HD);

  // The sequence's 64-key blocks blk0 .. blk1 are dealt to its nt tiles in
  // turn, and a tile's to its four waves in turn: wave w of tile c takes
  // blocks blk0 + c + (w + 4i) nt. The workgroups of one head thus read one
  // window of consecutive blocks at a time instead of nt separate streams,
  // which keeps the HBM accesses local. A block's K (NKV vectors) and V (NLD
  // vectors) live in registers; the next block's K is requested as soon as
  // the scores are done and its V as soon as P.V is done, so each load's
  // latency hides behind the other half's arithmetic. On the wave's last
  // block the "next" loads repeat that block (in bounds, unused), which keeps
  // every wait count static. The first block's loads are issued before the
  // queries are staged, so the two latencies overlap (a wave of a short
  // context has only one block).
  const int64_t blk0 = k0 >> 6, blk1 = k1 > k0 ? (k1 - 1) >> 6 : blk0 - 1;
  const int64_t bstep = 4 * (int64_t)tr.nt;
  const int64_t first = blk0 + tr.c + (int64_t)wave * tr.nt;
  const bool any = first <= blk1;
  u32x4 kreg[NKV], vreg[NLD];
  auto load_k = [&](int64_t blk) __attribute__((always_inline)) {
    const S* kp = Kh + blk * 64 * HD + lane * E;
#pragma unroll
    for (int i = 0; i < NKV; ++i) kreg[i] = ld16(kp + i * 64 * E);
  };
  // V is read once per layer: non-temporal loads (measured 5% faster per
  // forward at T = 131072 and on a ragged 16-sequence batch; marking K as
  // well was faster on the first and slower on the second)
  auto load_v = [&](int64_t blk) __attribute__((always_inline)) {
    const S* vp = Vh + blk * 64 * HD + lane * E;
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      vreg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + i * 64 * E));
  };
  if (any) {
    load_k(first);
    load_v(first);
  }
  const int d = HD * n_heads;
  if constexpr (kDot2) {
    for (int i = tid; i < G * HD / 2; i += 256) {
      const int j = i / (HD / 2), c2 = i % (HD / 2);
      const float2 q2 = *reinterpret_cast<const float2*>(Q + (int64_t)(b * G + j) * d + h * HD + 2 * c2);
      qb[j][c2] = pack_bf16x2(q2.x, q2.y);
    }
  } else {
    for (int i = tid; i < G * HD; i += 256) {
      const int j = i / HD, cc = i % HD;
      qs[j][cc] = Q[(int64_t)(b * G + j) * d + h * HD + cc];
    }
  }
  __syncthreads();

  float m_run[G], l_run[G];
  float o[G][2];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m_run[j] = kNegInf;
    l_run[j] = 0.f;
    o[j][0] = o[j][1] = 0.f;
  }
  const int kg = lane / (HD / 2), cp = lane % (HD / 2);

  if (any) {
    const int64_t last = first + ((blk1 - first) / bstep) * bstep;
    for (int64_t blk = first; blk <= last; blk += bstep) {
      const int64_t nxt = min(blk + bstep, last);
      // ---- scores: lane owns key blk*64 + lane
      const int64_t key = blk * 64 + lane;
      // padded batches: the key's mask byte, read where it is used (held
      // across the loop it pushed the kernel into register spills)
      const bool valid = key >= k0 && key < k1 && (!key_mask || key_mask[min(key, T1 - 1)] != 0);
      float s[G];
#pragma unroll
      for (int j = 0; j < G; ++j) s[j] = 0.f;
      if constexpr (kDot2) {
        // kreg[i] dword w holds dims 8i + 2w, 8i + 2w + 1 of this lane's key
#pragma unroll
        for (int i = 0; i < NKV; ++i)
#pragma unroll
          for (int j = 0; j < G; ++j) {
            const u32x4 q4 = *reinterpret_cast<const u32x4*>(&qb[j][i * 4]);
#pragma unroll
            for (int w = 0; w < 4; ++w) s[j] = dot2_bf16(kreg[i][w], q4[w], s[j]);
          }
      } else {
#pragma unroll
        for (int i = 0; i < NKV; ++i) {
          float kf[E];
          Vec16<S>::unpack(kreg[i], kf);
#pragma unroll
          for (int j = 0; j < G; ++j) {
#pragma unroll
            for (int e = 0; e < E; e += 4) {
              const f32x4 q4 = *reinterpret_cast<const f32x4*>(&qs[j][i * E + e]);
              s[j] = fmaf(q4[0], kf[e], s[j]);
              s[j] = fmaf(q4[1], kf[e + 1], s[j]);
              s[j] = fmaf(q4[2], kf[e + 2], s[j]);
              s[j] = fmaf(q4[3], kf[e + 3], s[j]);
            }
          }
        }
      }
      load_k(nxt);
      // ---- online softmax over this block (wave-uniform max; every block
      // holds at least one valid key)
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float sv = valid ? s[j] : kNegInf;
        const float bm = wave_max(sv);
        const float mn = fmaxf(m_run[j], bm);
        // a block can be fully masked (padding rows): then mn = -inf, and the
        // finite stand-in keeps alpha = 1 and p = 0 instead of NaN
        const float mf = mn == kNegInf ? 0.f : mn;
        const float alpha = exp2f(m_run[j] - mf);   // 0 when m_run = -inf
        const float p = exp2f(sv - mf);             // 0 for masked keys
        l_run[j] = l_run[j] * alpha + p;
        o[j][0] *= alpha;
        o[j][1] *= alpha;
        m_run[j] = mn;
        if constexpr (kDot2)
          pb[wave][j][lane] = __builtin_bit_cast(uint16_t, from_f32<bf16>(p));
        else
          ps[wave][j][lane] = p;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // ---- P.V: lane owns columns 2cp, 2cp+1 and R keys per vector
      if constexpr (kDot2) {
#pragma unroll
        for (int ld = 0; ld < NLD; ++ld) {
          // vreg dword r = (column 2cp, column 2cp+1) of key kb + r; regroup
          // into key pairs per column for the dot products
          const u32x4 v = vreg[ld];
          const uint32_t c0k01 = __builtin_amdgcn_perm(v[1], v[0], 0x05040100u);
          const uint32_t c1k01 = __builtin_amdgcn_perm(v[1], v[0], 0x07060302u);
          const uint32_t c0k23 = __builtin_amdgcn_perm(v[3], v[2], 0x05040100u);
          const uint32_t c1k23 = __builtin_amdgcn_perm(v[3], v[2], 0x07060302u);
          const int kb = ld * KG * R + kg * R;   // first key of this vector
#pragma unroll
          for (int j = 0; j < G; ++j) {
            const uint2 pp = *reinterpret_cast<const uint2*>(&pb[wave][j][kb]);
            o[j][0] = dot2_bf16(c0k01, pp.x, o[j][0]);
            o[j][0] = dot2_bf16(c0k23, pp.y, o[j][0]);
            o[j][1] = dot2_bf16(c1k01, pp.x, o[j][1]);
            o[j][1] = dot2_bf16(c1k23, pp.y, o[j][1]);
          }
        }
      } else {
#pragma unroll
        for (int ld = 0; ld < NLD; ++ld) {
          float vf[E];
          Vec16<S>::unpack(vreg[ld], vf);
          const int kb = ld * KG * R + kg * R;   // first key of this vector
#pragma unroll
          for (int j = 0; j < G; ++j) {
            float pr[R];
            if constexpr (R == 4) {
              const f32x4 p4 = *reinterpret_cast<const f32x4*>(&ps[wave][j][kb]);
              pr[0] = p4[0]; pr[1] = p4[1]; pr[2] = p4[2]; pr[3] = p4[3];
            } else {
#pragma unroll
              for (int r = 0; r < R; ++r) pr[r] = ps[wave][j][kb + r];
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
              o[j][0] = fmaf(pr[r], vf[2 * r], o[j][0]);
              o[j][1] = fmaf(pr[r], vf[2 * r + 1], o[j][1]);
            }
          }
        }
      }
      load_v(nxt);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }

  // ---- per-wave totals: l over lanes, o over key groups
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float lw = wave_sum(l_run[j]);
    float o0 = o[j][0], o1 = o[j][1];
#pragma unroll
    for (int off = HD / 2; off < 64; off <<= 1) {
      o0 += __shfl_xor(o0, off, kWave);
      o1 += __shfl_xor(o1, off, kWave);
    }
    if (lane == 0) {
      red_m[wave][j] = m_run[j];
      red_l[wave][j] = lw;
    }
    if (kg == 0) {
      red_o[wave][j][2 * cp] = o0;
      red_o[wave][j][2 * cp + 1] = o1;
    }
  }
  __syncthreads();

  // ---- merge the four waves and write this tile's partial
  const int64_t pbase = ((int64_t)tile * n_heads + h) * G;
  for (int i = tid; i < G * HD; i += 256) {
    const int j = i / HD, cc = i % HD;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w][j]);
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (red_m[w][j] != kNegInf) acc += red_o[w][j][cc] * exp2f(red_m[w][j] - M);
    part_o[(pbase + j) * HD + cc] = acc;
  }
  if (tid < G) {
    const int j = tid;
    float M = kNegInf;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w][j]);
    float l = 0.f;
    for (int w = 0; w < 4; ++w)
      if (red_m[w][j] != kNegInf) l += red_l[w][j] * exp2f(red_m[w][j] - M);
    part_ml[(pbase + j) * 2 + 0] = M;
    part_ml[(pbase + j) * 2 + 1] = l;
  }
}

// ---------------------------------------------------------------------------
// Head-split partials for short contexts: grid (total_tiles, n_heads), one
// 64-key chunk per tile (at most two physical 64-key blocks, since a
// sequence's keys need not start on a block boundary), 4 waves. For Q.K^T
// wave w takes a quarter of the head dimension for all 64 keys (lane = key)
// and the four partial scores are summed through LDS; every wave then runs
// the same softmax, and for P.V wave w takes a quarter of the block's keys
// for all columns. Each wave thus does a quarter of the arithmetic of a
// block, which is what bounds these launches when there are few blocks.
// ---------------------------------------------------------------------------
template <typename S, int HD, int G>
__global__ __launch_bounds__(256) void attn_hsplit_kernel(
    const float* __restrict__ Q, const S* __restrict__ kv_base, int64_t Tpad, int n_heads, int n_kv, int layer,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ prefix, int A, int64_t T1, int chunk,
    int total_tiles, int64_t seq_stride, const uint8_t* __restrict__ key_mask, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  using L = KVLayout<S>;
  constexpr int E = L::E, R = L::R;
  constexpr int NKV = HD / E;            // K vectors per key row
  constexpr int KG = 128 / HD;           // key groups in the P.V lane split
  constexpr int NLD = 64 / (KG * R);     // V loads per 64-key block
  constexpr int NKW = NKV / 4;           // K vectors per lane and wave (a quarter of the row)
  constexpr int NLW = NLD / 4;           // V loads per wave (a quarter of the keys)
  static_assert(NKV % 4 == 0 && NLD % 4 == 0, "head split");

  __shared__ __attribute__((aligned(16))) float qs[G][HD];
  __shared__ float sp[4][G][64];         // partial scores, one slice of the head per wave
  __shared__ __attribute__((aligned(16))) float ps[4][G][64];   // each wave's copy of p
  __shared__ __attribute__((aligned(16))) float red_o[4][G][HD];

  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  TileRange tr;
  if (!tile_range(tile, A, T1, cu, prefix, chunk, total_tiles, seq_stride, tr)) return;
  const int b = tr.b;
  const int64_t k0 = tr.k0, k1 = tr.k1;
  const int64_t blk0 = k0 >> 6;
  const int nblk = k1 > k0 ? (int)(((k1 - 1) >> 6) - blk0 + 1) : 0;   // 0, 1 or 2

  // both blocks' slices are requested first (the second repeats the first
  // when there is only one), then the queries are staged. A tile with no
  // keys (an empty sequence) loads nothing: its block index may lie past the
  // last block of the slab, or the K/V region may be empty altogether.
  // query head h reads the K/V of head h / (n_heads / n_kv) (grouped K/V heads)
  const int kvh = h / (n_heads / n_kv);
  const S* __restrict__ Kh = kv_base + L::head_base(layer, 0, kvh, n_kv, Tpad, HD);
  const S* __restrict__ Vh = kv_base + L::head_base(layer, 1, kvh, n_kv, Tpad, HD);
  u32x4 kreg[2][NKW], vreg[2][NLW];
  if (nblk > 0) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int64_t blk = blk0 + min(bb, nblk - 1);
      const S* kp = Kh + blk * 64 * HD + (wave * NKW) * 64 * E + lane * E;
      const S* vp = Vh + blk * 64 * HD + (wave * NLW) * 64 * E + lane * E;
#pragma unroll
      for (int i = 0; i < NKW; ++i) kreg[bb][i] = ld16(kp + i * 64 * E);
#pragma unroll
      for (int i = 0; i < NLW; ++i)   // V is read once: non-temporal, as in the streaming kernel
        vreg[bb][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + i * 64 * E));
    }
  }
  const int d = HD * n_heads;
  for (int i = tid; i < G * HD; i += 256) {
    const int j = i / HD, cc = i % HD;
    qs[j][cc] = Q[(int64_t)(b * G + j) * d + h * HD + cc];
  }
  __syncthreads();

  float m_run[G], l_run[G];
  float o[G][2];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m_run[j] = kNegInf;
    l_run[j] = 0.f;
    o[j][0] = o[j][1] = 0.f;
  }
  const int kg = lane / (HD / 2), cp = lane % (HD / 2);

#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    if (bb < nblk) {
      // ---- partial scores over this wave's quarter of the head
      float s[G];
#pragma unroll
      for (int j = 0; j < G; ++j) s[j] = 0.f;
#pragma unroll
      for (int i = 0; i < NKW; ++i) {
        float kf[E];
        Vec16<S>::unpack(kreg[bb][i], kf);
        const int c0 = (wave * NKW + i) * E;
#pragma unroll
        for (int j = 0; j < G; ++j) {
#pragma unroll
          for (int e = 0; e < E; e += 4) {
            const f32x4 q4 = *reinterpret_cast<const f32x4*>(&qs[j][c0 + e]);
            s[j] = fmaf(q4[0], kf[e], s[j]);
            s[j] = fmaf(q4[1], kf[e + 1], s[j]);
            s[j] = fmaf(q4[2], kf[e + 2], s[j]);
            s[j] = fmaf(q4[3], kf[e + 3], s[j]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < G; ++j) sp[wave][j][lane] = s[j];
      __syncthreads();
      // ---- full scores and the online softmax (the same in every wave)
      const int64_t key = (blk0 + bb) * 64 + lane;
      const bool valid = key >= k0 && key < k1 && (!key_mask || key_mask[min(key, T1 - 1)] != 0);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float sc = (sp[0][j][lane] + sp[1][j][lane]) + (sp[2][j][lane] + sp[3][j][lane]);
        const float sv = valid ? sc : kNegInf;
        const float bm = wave_max(sv);
        const float mn = fmaxf(m_run[j], bm);
        // a block can be fully masked (padding rows): then mn = -inf, and the
        // finite stand-in keeps alpha = 1 and p = 0 instead of NaN
        const float mf = mn == kNegInf ? 0.f : mn;
        const float alpha = exp2f(m_run[j] - mf);   // 0 when m_run = -inf
        const float p = exp2f(sv - mf);             // 0 for masked keys
        l_run[j] = l_run[j] * alpha + p;
        o[j][0] *= alpha;
        o[j][1] *= alpha;
        m_run[j] = mn;
        ps[wave][j][lane] = p;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // ---- P.V over this wave's quarter of the keys, all columns
#pragma unroll
      for (int i = 0; i < NLW; ++i) {
        float vf[E];
        Vec16<S>::unpack(vreg[bb][i], vf);
        const int kb = (wave * NLW + i) * KG * R + kg * R;   // first key of this vector
#pragma unroll
        for (int j = 0; j < G; ++j) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float pr = ps[wave][j][kb + r];
            o[j][0] = fmaf(pr, vf[2 * r], o[j][0]);
            o[j][1] = fmaf(pr, vf[2 * r + 1], o[j][1]);
          }
        }
      }
      __syncthreads();   // sp is rewritten by the next block
    }
  }

  // ---- o over key groups and waves (m and l are the same in every wave)
#pragma unroll
  for (int j = 0; j < G; ++j) {
    float o0 = o[j][0], o1 = o[j][1];
#pragma unroll
    for (int off = HD / 2; off < 64; off <<= 1) {
      o0 += __shfl_xor(o0, off, kWave);
      o1 += __shfl_xor(o1, off, kWave);
    }
    if (kg == 0) {
      red_o[wave][j][2 * cp] = o0;
      red_o[wave][j][2 * cp + 1] = o1;
    }
  }
  float lsum[G];
#pragma unroll
  for (int j = 0; j < G; ++j) lsum[j] = wave_sum(l_run[j]);
  __syncthreads();
  const int64_t pbase = ((int64_t)tile * n_heads + h) * G;
  for (int i = tid; i < G * HD; i += 256) {
    const int j = i / HD, cc = i % HD;
    part_o[(pbase + j) * HD + cc] = (red_o[0][j][cc] + red_o[1][j][cc]) + (red_o[2][j][cc] + red_o[3][j][cc]);
  }
  if (wave == 0 && lane < G) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (lane == j) {
        part_ml[(pbase + j) * 2 + 0] = m_run[j];
        part_ml[(pbase + j) * 2 + 1] = lsum[j];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// (m, l) combine: grid (1, n_heads, A), 256 threads. Workgroup (h, b) merges
// every context partial of sequence b and query head h with the gamma block
// keys (K_d, V_d in float32; with grouped K/V heads those of K/V head
// h / (n_heads / n_kv)) into the head's attention output o_h [gamma][hd],
// and writes it into Attn[b * gamma + j][h * hd ..] (heads concatenated).
// The output projection E = D + Attn W_o^T is a row GEMM after it: the
// heads' shares are summed in a fixed order, so the block rows are the same
// from call to call.
//
// Merge: thread (tg, c4) runs an online log-sum-exp over tiles tg, tg + TG,
// ... for four output columns of every query, with the loads of TB tiles in
// flight together; the TG groups are merged in LDS. The block rows are
// requested before the tile range is known, so the only dependent round
// trips are the tile prefix (skipped for a single sequence) and the partials.
// ---------------------------------------------------------------------------
template <int HD>
struct CombineShape {
  static constexpr int C4 = HD / 4;               // float4 columns of a head
  static constexpr int TG = 256 / C4;             // tile groups of the merge
  // LDS floats: q, k, v rows, block scores, group (o, m, l)
  static constexpr int lds_floats(int g) {
    return 3 * g * HD + ((g * g + 3) & ~3) + TG * g * HD + 2 * TG * g;
  }
};

template <int HD, int G>
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ Q, const float* __restrict__ Kd, const float* __restrict__ Vd,
    int n_heads, int n_kv, const int32_t* __restrict__ prefix, int total_tiles,
    const float* __restrict__ part_o, const float* __restrict__ part_ml, float* __restrict__ attn) {
  using Sh = CombineShape<HD>;
  constexpr int C4 = Sh::C4, TG = Sh::TG;
  constexpr int TB = G <= 5 ? 4 : (G <= 10 ? 2 : 1);   // tiles whose loads are issued together
  constexpr int QE = (G * C4 + 255) / 256;   // q / k / v float4 per thread
  extern __shared__ __attribute__((aligned(16))) float lds[];
  float* qs = lds;                        // [G][HD]
  float* ks = qs + G * HD;                // [G][HD]
  float* vs = ks + G * HD;                // [G][HD]
  float* sb = vs + G * HD;                // [G][G] block-key scores
  float* og = sb + ((G * G + 3) & ~3);    // [TG][G][HD]
  float* mg = og + TG * G * HD;           // [TG][G]
  float* lg = mg + TG * G;                // [TG][G]

  const int d = n_heads * HD;
  const int b = blockIdx.z, h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // the block rows first: this head's queries, the block keys / values of its
  // K/V head (rows of n_kv * HD)
  const int kvh = h / (n_heads / n_kv), kvd = n_kv * HD;
  f32x4 qv[QE], kv[QE], vv[QE];
#pragma unroll
  for (int u = 0; u < QE; ++u) {
    const int e = min(tid + 256 * u, G * C4 - 1);
    const int j = e / C4, c = e % C4;
    const int64_t off = (int64_t)(b * G + j) * d + h * HD + 4 * c;
    const int64_t koff = (int64_t)(b * G + j) * kvd + kvh * HD + 4 * c;
    qv[u] = *reinterpret_cast<const f32x4*>(Q + off);
    kv[u] = *reinterpret_cast<const f32x4*>(Kd + koff);
    vv[u] = *reinterpret_cast<const f32x4*>(Vd + koff);
  }

  // context partials: online merge over this thread's tiles, TB at a time
  const bool one_seq = gridDim.z == 1;
  const int t0 = one_seq ? 0 : min(prefix[b], total_tiles);
  const int t1 = one_seq ? total_tiles : min(prefix[b + 1], total_tiles);
  const int tg = tid / C4, c4 = tid % C4;
  float mrun[G], lrun[G];
  f32x4 acc[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    mrun[j] = kNegInf;
    lrun[j] = 0.f;
    acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int tb = t0 + tg; tb < t1; tb += TG * TB) {
    f32x2 ml[TB][G];
    f32x4 o[TB][G];
#pragma unroll
    for (int k = 0; k < TB; ++k) {
      const int64_t pj = ((int64_t)min(tb + k * TG, t1 - 1) * n_heads + h) * G;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        ml[k][j] = *reinterpret_cast<const f32x2*>(part_ml + (pj + j) * 2);
        o[k][j] = *reinterpret_cast<const f32x4*>(part_o + (pj + j) * HD + 4 * c4);
      }
    }
    // all of the batch's loads are issued before any is used; the merge is
    // branch-free, so no load is moved into a conditional block
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < TB; ++k) {
      const bool in = tb + k * TG < t1;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float mt = in ? ml[k][j][0] : kNegInf;   // an empty tile adds nothing
        const float mn = fmaxf(mrun[j], mt);
        const float so = mrun[j] == mn ? 1.f : exp2f(mrun[j] - mn);
        const float sn = mt == kNegInf ? 0.f : exp2f(mt - mn);
        acc[j] = acc[j] * so + o[k][j] * sn;
        lrun[j] = lrun[j] * so + ml[k][j][1] * sn;
        mrun[j] = mn;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < QE; ++u) {
    const int e = tid + 256 * u;
    if (e < G * C4) {
      const int j = e / C4, c = e % C4;
      *reinterpret_cast<f32x4*>(qs + j * HD + 4 * c) = qv[u];
      *reinterpret_cast<f32x4*>(ks + j * HD + 4 * c) = kv[u];
      *reinterpret_cast<f32x4*>(vs + j * HD + 4 * c) = vv[u];
    }
  }
#pragma unroll
  for (int j = 0; j < G; ++j) {
    *reinterpret_cast<f32x4*>(og + (tg * G + j) * HD + 4 * c4) = acc[j];
    if (c4 == 0) {
      mg[tg * G + j] = mrun[j];
      lg[tg * G + j] = lrun[j];
    }
  }
  __syncthreads();
  // block-key scores (base 2: q carries hd^-1/2 log2 e), one wave per pair
  for (int pq = wave; pq < G * G; pq += 4) {
    const int j = pq / G, jj = pq % G;
    float sc = 0.f;
#pragma unroll
    for (int c = lane; c < HD; c += 64) sc = fmaf(qs[j * HD + c], ks[jj * HD + c], sc);
    sc = wave_sum(sc);
    if (lane == 0) sb[pq] = sc;
  }
  __syncthreads();
  // o_h[j] = (sum_g o_g 2^(m_g - M) + sum_jj 2^(s_jj - M) v_jj) / l
  for (int e = tid; e < G * C4; e += 256) {
    const int j = e / C4, c = e % C4;
    float M = kNegInf;
    for (int g2 = 0; g2 < TG; ++g2) M = fmaxf(M, mg[g2 * G + j]);
#pragma unroll
    for (int jj = 0; jj < G; ++jj) M = fmaxf(M, sb[j * G + jj]);
    float l = 0.f;
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int g2 = 0; g2 < TG; ++g2) {
      const float m = mg[g2 * G + j];
      if (m != kNegInf) {
        const float w = exp2f(m - M);
        l = fmaf(lg[g2 * G + j], w, l);
        o += *reinterpret_cast<const f32x4*>(og + (g2 * G + j) * HD + 4 * c) * w;
      }
    }
#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
      const float w = exp2f(sb[j * G + jj] - M);
      l += w;
      o += *reinterpret_cast<const f32x4*>(vs + jj * HD + 4 * c) * w;
    }
    *reinterpret_cast<f32x4*>(attn + (int64_t)(b * G + j) * d + h * HD + 4 * c) = o * (1.f / l);
  }
}

template <int HD, int G>
static hipError_t launch_combine_t(const AttnArgs& a, hipStream_t s) {
  using Sh = CombineShape<HD>;
  const size_t lds = (size_t)Sh::lds_floats(G) * 4;
  auto kern = combine_kernel<HD, G>;
  if (lds > 65536) {
    static hipError_t set = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (set != hipSuccess) return set;
  }
  dim3 grid(1, a.n_heads, a.A);
  kern<<<grid, 256, lds, s>>>(a.Q, a.Kd, a.Vd, a.n_heads, a.kv.n_heads, a.prefix, a.total_tiles, a.part_o,
                              a.part_ml, a.attn);
  return hipGetLastError();
}

template <int HD>
static hipError_t combine_gamma(const AttnArgs& a, hipStream_t s) {
  switch (a.gamma) {
#define DSPARK_G(g) \
  case g: return launch_combine_t<HD, g>(a, s);
    DSPARK_G(1) DSPARK_G(2) DSPARK_G(3) DSPARK_G(4) DSPARK_G(5) DSPARK_G(6) DSPARK_G(7)
    DSPARK_G(8) DSPARK_G(9) DSPARK_G(10) DSPARK_G(11) DSPARK_G(12) DSPARK_G(13) DSPARK_G(14)
    DSPARK_G(15) DSPARK_G(16)
#undef DSPARK_G
    default: return hipErrorInvalidValue;
  }
}

template <typename S, int HD, int G>
static void launch_attn_t(dim3 grid, hipStream_t s, const AttnArgs& a) {
  if (a.chunk == 64) {
    attn_hsplit_kernel<S, HD, G><<<grid, 256, 0, s>>>(
        a.Q, static_cast<const S*>(a.kv.base), a.kv.Tpad, a.n_heads, a.kv.n_heads, a.layer, a.cu, a.prefix, a.A,
        a.kv.T, a.chunk, a.total_tiles, a.kv.seq_stride, a.kv.key_mask, a.part_o, a.part_ml);
    return;
  }
  attn_partial_kernel<S, HD, G><<<grid, 256, 0, s>>>(
      a.Q, static_cast<const S*>(a.kv.base), a.kv.Tpad, a.n_heads, a.kv.n_heads, a.layer, a.cu, a.prefix, a.A,
      a.kv.T, a.chunk, a.total_tiles, a.kv.seq_stride, a.kv.key_mask, a.part_o, a.part_ml);
}

template <typename S, int HD>
static bool dispatch_gamma(int gamma, dim3 grid, hipStream_t s, const AttnArgs& a) {
  switch (gamma) {
#define DSPARK_G(g) \
  case g: launch_attn_t<S, HD, g>(grid, s, a); return true;
    DSPARK_G(1) DSPARK_G(2) DSPARK_G(3) DSPARK_G(4) DSPARK_G(5) DSPARK_G(6) DSPARK_G(7)
    DSPARK_G(8) DSPARK_G(9) DSPARK_G(10) DSPARK_G(11) DSPARK_G(12) DSPARK_G(13) DSPARK_G(14)
    DSPARK_G(15) DSPARK_G(16)
#undef DSPARK_G
    default: return false;
  }
}

hipError_t launch_attention(int dtype, const AttnArgs& a, hipStream_t s) {
  if (a.total_tiles < a.A) return hipErrorInvalidValue;   // every sequence has a tile
  dim3 grid(a.total_tiles, a.n_heads);
  bool ok = false;
  trace_pre(K_ATTN, s);
  if (dtype == 1) {
    if (a.kv.hd == 128) ok = dispatch_gamma<bf16, 128>(a.gamma, grid, s, a);
    else if (a.kv.hd == 64) ok = dispatch_gamma<bf16, 64>(a.gamma, grid, s, a);
    else if (a.kv.hd == 32) ok = dispatch_gamma<bf16, 32>(a.gamma, grid, s, a);
  } else {
    if (a.kv.hd == 128) ok = dispatch_gamma<float, 128>(a.gamma, grid, s, a);
    else if (a.kv.hd == 64) ok = dispatch_gamma<float, 64>(a.gamma, grid, s, a);
    else if (a.kv.hd == 32) ok = dispatch_gamma<float, 32>(a.gamma, grid, s, a);
  }
  trace_post(K_ATTN, s);
  if (!ok) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  trace_pre(K_COMBINE, s);
  if (a.kv.hd == 128) e = combine_gamma<128>(a, s);
  else if (a.kv.hd == 64) e = combine_gamma<64>(a, s);
  else e = combine_gamma<32>(a, s);
  trace_post(K_COMBINE, s);
  return e;
}

}  // namespace dspark
