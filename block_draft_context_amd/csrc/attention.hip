// Eq 3 block attention over [context ++ block], split over context chunks.
//
// The gamma block queries of sequence b attend to its L_b context keys and
// its gamma block keys with no causal mask (module-dflash.ts, #layer). The
// context part is long and read once per layer, so it is split into chunks
// of `chunk` keys: one workgroup per (chunk, head) streams the chunk's K and
// V once and leaves an unnormalised partial (m, l, o) per query, as the
// split-chunk attention + combine kernels of dspark-runtime.js do. A second
// kernel, one workgroup per (sequence, head, query), merges those partials
// together with the gamma block keys by the log-sum-exp identity
//   M = max_c m_c,  l = sum_c l_c 2^(m_c - M),  o = sum_c o_c 2^(m_c - M) / l.
// Scores are kept in base 2: Q arrives pre-multiplied by hd^-1/2 * log2(e).
//
// Work split inside a chunk: each wave takes every fourth 64-key block, with
// the next block's loads in flight while the current one is computed. For
// Q.K^T lane t owns key t and reads its whole key row (hd/E 16-byte vectors,
// one 1 KiB wave-wide run each, see kv_layout.h). For P.V lane (kg, cp) owns two value
// columns and R keys per load, so each V load is again one 1 KiB run; the
// block's probabilities are broadcast through LDS. All arithmetic is float32
// on the vector ALUs: with gamma <= 16 queries the arithmetic intensity is a
// few flop per byte, far below the matrix cores'.
#include "common.h"
#include "kernels.h"
#include "kv_layout.h"

namespace dspark {

constexpr float kNegInf = -__builtin_inff();

// Keys per chunk. Short contexts (at most ~1024 64-key blocks over all
// heads) use one block per tile and the head-split kernel, whose four waves
// share each block; longer ones use chunks of >= 256 keys streamed by the
// four waves of a workgroup, aiming for ~512 (chunk, head) workgroups.
int attention_chunk(int64_t T, int n_heads, int A) {
  const int64_t blocks = (T + 63) / 64 + A;   // bound on sum_b ceil(L_b / 64)
  if (blocks * n_heads <= 1024) return 64;
  int64_t c = (T * n_heads + 511) / 512;
  c = ((c + 63) / 64) * 64;
  if (c < 256) c = 256;
  if (c > 16384) c = 16384;
  return (int)c;
}

int64_t attention_tiles(const int32_t* cu_host, int A, int chunk) {
  int64_t n = 0;
  for (int b = 0; b < A; ++b) {
    const int64_t L = cu_host[b + 1] - cu_host[b];
    n += L > 0 ? (L + chunk - 1) / chunk : 1;
  }
  return n;
}

// ---------------------------------------------------------------------------
// partials: grid (total_tiles, n_heads), 256 threads (4 waves)
// part_o  [total_tiles][n_heads][G][HD]   unnormalised output
// part_ml [total_tiles][n_heads][G][2]    (max, sum) in base-2 units
// ---------------------------------------------------------------------------
template <typename S, int HD, int G>
__global__ __launch_bounds__(256) void attn_partial_kernel(
    const float* __restrict__ Q, const S* __restrict__ kv_base, int64_t Tpad, int n_heads, int layer,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ prefix, int A, int chunk,
    int total_tiles, float* __restrict__ part_o, float* __restrict__ part_ml) {
  using L = KVLayout<S>;
  constexpr int E = L::E, R = L::R;
  constexpr int NKV = HD / E;            // K vectors per key row
  constexpr int KG = 128 / HD;           // key groups in the P.V lane split
  constexpr int NLD = 64 / (KG * R);     // V loads per 64-key block

  __shared__ __attribute__((aligned(16))) float qs[G][HD];
  __shared__ __attribute__((aligned(16))) float ps[4][G][64];
  __shared__ float red_m[4][G];
  __shared__ float red_l[4][G];
  __shared__ __attribute__((aligned(16))) float red_o[4][G][HD];

  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int dev_total = prefix[A];
  if (tile >= total_tiles || tile >= dev_total) return;

  // sequence owning this tile: largest b with prefix[b] <= tile
  int lo = 0, hi = A - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int c = tile - prefix[b];
  const int64_t kseq0 = cu[b], kseq1 = cu[b + 1];
  const int64_t k0 = min(kseq1, kseq0 + (int64_t)c * chunk);
  const int64_t k1 = min(kseq1, k0 + chunk);

  const int d = HD * n_heads;
  for (int i = tid; i < G * HD; i += 256) {
    const int j = i / HD, cc = i % HD;
    qs[j][cc] = Q[(int64_t)(b * G + j) * d + h * HD + cc];
  }
  __syncthreads();

  const S* __restrict__ Kh = kv_base + L::head_base(layer, 0, h, n_heads, Tpad, HD);
  const S* __restrict__ Vh = kv_base + L::head_base(layer, 1, h, n_heads, Tpad, HD);

  float m_run[G], l_run[G];
  float o[G][2];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m_run[j] = kNegInf;
    l_run[j] = 0.f;
    o[j][0] = o[j][1] = 0.f;
  }
  const int kg = lane / (HD / 2), cp = lane % (HD / 2);

  // The wave's 64-key blocks are blk0 + wave, +4, ... <= blk1. A block's K
  // (NKV vectors) and V (NLD vectors) live in registers; the next block's K
  // is requested as soon as the scores are done and its V as soon as P.V is
  // done, so each load's latency hides behind the other half's arithmetic.
  // On the wave's last block the "next" loads repeat that block (in bounds,
  // unused), which keeps every wait count static.
  const int64_t blk0 = k0 >> 6, blk1 = k1 > k0 ? (k1 - 1) >> 6 : blk0 - 1;
  const int64_t first = blk0 + wave;
  if (first <= blk1) {
    const int64_t last = first + ((blk1 - first) / 4) * 4;
    u32x4 kreg[NKV], vreg[NLD];
    auto load_k = [&](int64_t blk) __attribute__((always_inline)) {
      const S* kp = Kh + blk * 64 * HD + lane * E;
#pragma unroll
      for (int i = 0; i < NKV; ++i) kreg[i] = ld16(kp + i * 64 * E);
    };
    auto load_v = [&](int64_t blk) __attribute__((always_inline)) {
      const S* vp = Vh + blk * 64 * HD + lane * E;
#pragma unroll
      for (int i = 0; i < NLD; ++i) vreg[i] = ld16(vp + i * 64 * E);
    };
    load_k(first);
    load_v(first);
    for (int64_t blk = first; blk <= last; blk += 4) {
      const int64_t nxt = min(blk + 4, last);
      // ---- scores: lane owns key blk*64 + lane
      const int64_t key = blk * 64 + lane;
      const bool valid = key >= k0 && key < k1;
      float s[G];
#pragma unroll
      for (int j = 0; j < G; ++j) s[j] = 0.f;
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
      load_k(nxt);
      // ---- online softmax over this block (wave-uniform max; every block
      // holds at least one valid key)
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float sv = valid ? s[j] : kNegInf;
        const float bm = wave_max(sv);
        const float mn = fmaxf(m_run[j], bm);
        const float alpha = exp2f(m_run[j] - mn);   // 0 when m_run = -inf
        const float p = exp2f(sv - mn);             // 0 for masked keys
        l_run[j] = l_run[j] * alpha + p;
        o[j][0] *= alpha;
        o[j][1] *= alpha;
        m_run[j] = mn;
        ps[wave][j][lane] = p;
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // ---- P.V: lane owns columns 2cp, 2cp+1 and R keys per vector
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
    const float* __restrict__ Q, const S* __restrict__ kv_base, int64_t Tpad, int n_heads, int layer,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ prefix, int A, int chunk,
    int total_tiles, float* __restrict__ part_o, float* __restrict__ part_ml) {
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
  const int dev_total = prefix[A];
  if (tile >= total_tiles || tile >= dev_total) return;
  int lo = 0, hi = A - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prefix[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int c = tile - prefix[b];
  const int64_t kseq0 = cu[b], kseq1 = cu[b + 1];
  const int64_t k0 = min(kseq1, kseq0 + (int64_t)c * chunk);
  const int64_t k1 = min(kseq1, k0 + chunk);
  const int64_t blk0 = k0 >> 6;
  const int nblk = k1 > k0 ? (int)(((k1 - 1) >> 6) - blk0 + 1) : 0;   // 0, 1 or 2

  // both blocks' slices are requested first (the second repeats the first
  // when there is only one), then the queries are staged
  const S* __restrict__ Kh = kv_base + L::head_base(layer, 0, h, n_heads, Tpad, HD);
  const S* __restrict__ Vh = kv_base + L::head_base(layer, 1, h, n_heads, Tpad, HD);
  u32x4 kreg[2][NKW], vreg[2][NLW];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int64_t blk = blk0 + min(bb, max(nblk - 1, 0));
    const S* kp = Kh + blk * 64 * HD + (wave * NKW) * 64 * E + lane * E;
    const S* vp = Vh + blk * 64 * HD + (wave * NLW) * 64 * E + lane * E;
#pragma unroll
    for (int i = 0; i < NKW; ++i) kreg[bb][i] = ld16(kp + i * 64 * E);
#pragma unroll
    for (int i = 0; i < NLW; ++i) vreg[bb][i] = ld16(vp + i * 64 * E);
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
      const bool valid = key >= k0 && key < k1;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float sc = (sp[0][j][lane] + sp[1][j][lane]) + (sp[2][j][lane] + sp[3][j][lane]);
        const float sv = valid ? sc : kNegInf;
        const float bm = wave_max(sv);
        const float mn = fmaxf(m_run[j], bm);
        const float alpha = exp2f(m_run[j] - mn);   // 0 when m_run = -inf
        const float p = exp2f(sv - mn);             // 0 for masked keys
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
// combine: grid (A * n_heads, gamma), 256 threads. Query j of (sequence b,
// head h): every tile partial of b plus the gamma block keys (K_d, V_d in
// float32). Thread (tg, cc) sums tiles tg, tg + NG, ... for column cc.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ Q, const float* __restrict__ Kd, const float* __restrict__ Vd, int A,
    int gamma, int d, int n_heads, const int32_t* __restrict__ prefix, int total_tiles,
    const float* __restrict__ part_o, const float* __restrict__ part_ml, float* __restrict__ attn) {
  __shared__ float sb[kMaxGamma];
  __shared__ float redw[4];
  __shared__ float red_acc[256];
  __shared__ float Msh, Lsh;
  const int b = blockIdx.x / n_heads, h = blockIdx.x % n_heads;
  const int j = blockIdx.y;
  const int hd = d / n_heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = min(prefix[b], total_tiles), t1 = min(prefix[b + 1], total_tiles);
  const float* q = Q + (int64_t)(b * gamma + j) * d + h * hd;

  // block-key scores (one wave per key)
  for (int jj = wave; jj < gamma; jj += 4) {
    const float* kr = Kd + (int64_t)(b * gamma + jj) * d + h * hd;
    float sc = 0.f;
    for (int cc = lane; cc < hd; cc += 64) sc = fmaf(q[cc], kr[cc], sc);
    sc = wave_sum(sc);
    if (lane == 0) sb[jj] = sc;
  }
  // max over tiles
  float mloc = kNegInf;
  for (int t = t0 + tid; t < t1; t += 256)
    mloc = fmaxf(mloc, part_ml[(((int64_t)t * n_heads + h) * gamma + j) * 2]);
  mloc = wave_max(mloc);
  if (lane == 0) redw[wave] = mloc;
  __syncthreads();
  if (tid == 0) {
    float M = fmaxf(fmaxf(redw[0], redw[1]), fmaxf(redw[2], redw[3]));
    for (int jj = 0; jj < gamma; ++jj) M = fmaxf(M, sb[jj]);
    Msh = M;
  }
  __syncthreads();
  const float M = Msh;
  // l over tiles
  float lloc = 0.f;
  for (int t = t0 + tid; t < t1; t += 256) {
    const float* ml = part_ml + (((int64_t)t * n_heads + h) * gamma + j) * 2;
    if (ml[0] != kNegInf) lloc += ml[1] * exp2f(ml[0] - M);
  }
  lloc = wave_sum(lloc);
  __syncthreads();
  if (lane == 0) redw[wave] = lloc;
  __syncthreads();
  if (tid == 0) {
    float l = (redw[0] + redw[1]) + (redw[2] + redw[3]);
    for (int jj = 0; jj < gamma; ++jj) l += exp2f(sb[jj] - M);
    Lsh = l;
  }
  // weighted tile outputs: 8 tiles per batch, loads issued together
  const int ng = 256 / hd;
  const int cc = tid % hd, tg = tid / hd;
  float acc = 0.f;
  for (int tb = t0 + tg; tb < t1; tb += 8 * ng) {
    float mv[8], ov[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = min(tb + i * ng, t1 - 1);
      const int64_t pj = ((int64_t)t * n_heads + h) * gamma + j;
      mv[i] = part_ml[pj * 2];
      ov[i] = part_o[pj * hd + cc];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool in = tb + i * ng < t1 && mv[i] != kNegInf;
      acc = fmaf(in ? ov[i] : 0.f, in ? exp2f(mv[i] - M) : 0.f, acc);
    }
  }
  red_acc[tid] = acc;
  __syncthreads();
  if (tid < hd) {
    float v = 0.f;
    for (int g2 = 0; g2 < ng; ++g2) v += red_acc[g2 * hd + tid];
    for (int jj = 0; jj < gamma; ++jj)
      v = fmaf(exp2f(sb[jj] - M), Vd[(int64_t)(b * gamma + jj) * d + h * hd + tid], v);
    attn[(int64_t)(b * gamma + j) * d + h * hd + tid] = v / Lsh;
  }
}

template <typename S, int HD, int G>
static void launch_attn_t(dim3 grid, hipStream_t s, const AttnArgs& a) {
  if (a.chunk == 64) {
    attn_hsplit_kernel<S, HD, G><<<grid, 256, 0, s>>>(
        a.Q, static_cast<const S*>(a.kv.base), a.kv.Tpad, a.kv.n_heads, a.layer, a.cu, a.prefix, a.A,
        a.chunk, a.total_tiles, a.part_o, a.part_ml);
    return;
  }
  attn_partial_kernel<S, HD, G><<<grid, 256, 0, s>>>(
      a.Q, static_cast<const S*>(a.kv.base), a.kv.Tpad, a.kv.n_heads, a.layer, a.cu, a.prefix, a.A,
      a.chunk, a.total_tiles, a.part_o, a.part_ml);
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
  if (a.total_tiles == 0) return hipSuccess;
  dim3 grid(a.total_tiles, a.kv.n_heads);
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
  dim3 cgrid(a.A * a.kv.n_heads, a.gamma);
  trace_pre(K_COMBINE, s);
  combine_kernel<<<cgrid, 256, 0, s>>>(a.Q, a.Kd, a.Vd, a.A, a.gamma, a.kv.hd * a.kv.n_heads,
                                       a.kv.n_heads, a.prefix, a.total_tiles, a.part_o, a.part_ml,
                                       a.attn);
  trace_post(K_COMBINE, s);
  return hipGetLastError();
}

}  // namespace dspark
