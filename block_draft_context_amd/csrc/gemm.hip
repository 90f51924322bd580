// Context-side dense contractions for gfx950:
//   Eq 2   P = [H^{l1}; ...; H^{lm}] . W_c              (split-K fp32 partials)
//          H_ctx = RMSNorm(P; ctx_norm)                  (row pass, setup.hip)
//   Eq 3   K_c, V_c = RMSNorm(H_ctx; attn_norm_i) . W_{K,V}^i   for every layer i
//
// bf16 storage runs on the matrix cores (v_mfma_f32_32x32x16_bf16) with both
// operands staged K-contiguous in LDS. Weights are stored [out, in], which is
// already the K-contiguous B operand: W_c is used as given, and the K/V
// weights of all layers are copied into one matrix with the layer's
// attention-norm gain folded into their columns (set-up pass, setup.hip).
// The RMSNorm row factor of the context rows is applied in the K/V epilogue:
//   RMSNorm(h; g) W^T = diag(rinv) . h . (W diag(g))^T.
// float32 storage uses a plain LDS-tiled FMA GEMM.
#include "common.h"
#include "kernels.h"
#include "kv_layout.h"

#include <algorithm>
#include <type_traits>

namespace dspark {

// ---------------------------------------------------------------------------
// MFMA GEMM  C[M,N] = A[M,K] . Bt[N,K]^T  (bf16 in, fp32 accumulate)
// 256 threads = 4 waves arranged WM x WN; each wave owns a (BM/WM) x (BN/WN)
// sub-tile made of 32x32 MFMA blocks. BK = 64. LDS rows are 128 bytes with the
// 16-byte chunk index XOR-swizzled by (row & 7), so both the cooperative
// stores and the per-lane MFMA operand reads are free of bank conflicts.
// Global tiles for step k+1 are fetched into registers while step k computes.
// ---------------------------------------------------------------------------
constexpr int BK = 64;

struct EpiPartial {            // out[z][r][n] = acc, rows < M
  float* out;
  int64_t split_stride;
  DSPARK_DEV void store(int z, int r, int n, float v, int M, int N) const {
    if (r < M) out[z * split_stride + (int64_t)r * N + n] = v;
  }
};

template <typename S>
struct EpiKV {                 // K/V of every layer, row scale, tiled layout
  S* base;
  const float* rinv;
  int64_t Tpad;
  int T, d, hd, n_heads;       // d: columns of one K or V block (K/V heads * hd)
  const int32_t* dst_row;      // null: row r at r (zeros at T .. Tpad-1); else row r < T at dst_row[r]
  DSPARK_DEV void store(int /*z*/, int r, int n, float v, int /*M*/, int /*N*/) const {
    int64_t t;
    float val;
    if (dst_row) {
      if (r >= T) return;
      t = dst_row[r];
      val = v * rinv[r];
    } else {
      if (r >= Tpad) return;
      t = r;
      val = (r < T) ? v * rinv[r] : 0.f;
    }
    const int layer = n / (2 * d);
    const int kv = (n / d) & 1;
    const int w = n % d;
    const int head = w / hd, c = w % hd;
    const int64_t hb = KVLayout<S>::head_base(layer, kv, head, n_heads, Tpad, hd);
    const int64_t off = kv == 0 ? KVLayout<S>::k_off(t, c, hd) : KVLayout<S>::v_off(t, c, hd);
    base[hb + off] = from_f32<S>(val);
  }
};

DSPARK_DEV int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

// M = valid A rows (rows >= M read as zero); MR = rows covered by the grid.
template <int BM, int BN, int WM, int WN, class Epi>
__global__ __launch_bounds__(256) void gemm_bf16_nt(ASegs a, const bf16* __restrict__ Bt, int M,
                                                    int MR, int N, int K, int k_per_split,
                                                    Epi epi) {
  constexpr int FM = BM / WM / 32;
  constexpr int FN = BN / WN / 32;
  constexpr int A_CH = BM * BK / 8 / 256;   // 16-byte chunks per thread
  constexpr int B_CH = BN * BK / 8 / 256;
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) char smem[(BM + BN) * BK * 2];
  char* As = smem;
  char* Bs = smem + BM * BK * 2;

  const int tiles_m = (MR + BM - 1) / BM;
  const int tiles_n = N / BN;
  const int ntiles = tiles_m * tiles_n;
  // XCD-aware order: consecutive workgroup ids land on different XCDs; give
  // each XCD a contiguous run of tiles so its L2 sees shared panels.
  int bid = blockIdx.x;
  {
    const int per = ntiles / 8;
    if (per > 0 && bid < per * 8) bid = (bid & 7) * per + (bid >> 3);
  }
  const int tm = bid / tiles_n, tn = bid % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int z = blockIdx.z;
  const int kbeg = z * k_per_split;
  const int kend = min(K, kbeg + k_per_split);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ra[A_CH], rb[B_CH];
  auto load_tiles = [&](int k0) {
    const int sgi = k0 / a.seg_k;
    const int kin = k0 - sgi * a.seg_k;
    const bf16* __restrict__ Ap = static_cast<const bf16*>(a.seg[sgi]);
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int q = tid + 256 * i;
      const int row = q >> 3, ch = q & 7;
      const int gr = m0 + row;
      // rows past M: load a valid row, then zero it (no branch around the load)
      const u32x4 v = ld16(Ap + (int64_t)min(gr, M - 1) * a.ld + kin + ch * 8);
      ra[i] = gr < M ? v : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int q = tid + 256 * i;
      const int row = q >> 3, ch = q & 7;
      rb[i] = ld16(Bt + (int64_t)(n0 + row) * K + k0 + ch * 8);
    }
  };
  auto store_tiles = [&]() {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int q = tid + 256 * i;
      st16(As + swz(q >> 3, q & 7), ra[i]);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int q = tid + 256 * i;
      st16(Bs + swz(q >> 3, q & 7), rb[i]);
    }
  };

  if (kbeg < kend) load_tiles(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    __syncthreads();
    store_tiles();
    __syncthreads();
    if (k0 + BK < kend) load_tiles(k0 + BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int ch = ks * 2 + (lane >> 5);
      bf16x8 av[FM], bv[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * (BM / WM) + i * 32 + (lane & 31);
        av[i] = *reinterpret_cast<const bf16x8*>(As + swz(row, ch));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * (BN / WN) + j * 32 + (lane & 31);
        bv[j] = *reinterpret_cast<const bf16x8*>(Bs + swz(row, ch));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
  }

  // 32x32 accumulator layout: lane holds column (lane & 31) and rows
  // 8*(r/4) + 4*(lane/32) + (r%4) for r = 0..15.
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * (BM / WM) + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = n0 + wn * (BN / WN) + j * 32 + (lane & 31);
        epi.store(z, row, col, acc[i][j][r], M, N);
      }
}

// ---------------------------------------------------------------------------
// float32 FMA GEMM: C[M,N] = A(segments)[M,K] . B(mats)[K,N], 64x64 tiles,
// BK = 16, 4x4 outputs per thread, gain applied to B rows while staging.
// ---------------------------------------------------------------------------
template <class Epi>
__global__ __launch_bounds__(256) void gemm_f32(ASegs a, BMats b, int M, int MR, int N, int K,
                                                int k_per_split, Epi epi) {
  (void)MR;
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int tiles_n = N / 64;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * 64, n0 = tn * 64;
  const int z = blockIdx.z;
  const int kbeg = z * k_per_split, kend = min(K, kbeg + k_per_split);
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int mi = n0 / b.n_per, c0 = n0 % b.n_per;
  const float* __restrict__ W = static_cast<const float*>(b.mat[mi]);
  const float* __restrict__ g = b.gain[mi];
  float acc[4][4] = {};
  for (int k0 = kbeg; k0 < kend; k0 += 16) {
    const int sgi = k0 / a.seg_k, kin = k0 - sgi * a.seg_k;
    const float* __restrict__ Ap = static_cast<const float*>(a.seg[sgi]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;          // 64 rows x 16 k
      const int r = e >> 4, kk = e & 15;
      As[kk][r] = (m0 + r < M) ? Ap[(int64_t)(m0 + r) * a.ld + kin + kk] : 0.f;
      const int bn = e >> 4, bk = e & 15;   // 64 n x 16 k of [out, in] weights
      float v = W[(int64_t)(c0 + bn) * K + k0 + bk];
      if (g) v *= g[k0 + bk];
      Bs[bk][bn] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) epi.store(z, m0 + ty * 4 + i, n0 + tx * 4 + j, acc[i][j], M, N);
}

// ---------------------------------------------------------------------------
// Large-tile MFMA GEMM for the long context (M = T rows): 256x256 tiles, 4
// waves in 2x2, each wave a 128x128 sub-tile of 4x4 32x32 MFMA blocks (its 256
// accumulators live in the AGPR file), so each k-substep of 16 issues 16 MFMAs
// against 8 LDS operand reads and LDS bandwidth stays below the matrix-core
// rate. Operands move global -> LDS with the gfx950 direct 16-byte loads (no
// register staging) through a ring of stages of BK-deep k tiles, in 128 KiB
// of LDS either way:
//   BK = 32, 4 stages: a row's k tile is half a cache line, and a stage's
//            loads have about three steps to land;
//   BK = 64, 2 stages: a row's k tile is one whole 128-byte line, fetched by 8
//            lanes of one instruction, so the vector memory path looks up
//            half as many lines per byte; loads have about one step to land.
// The operands of the next k-substep are read while the MFMAs of the current
// one run. Lane l of a load instruction lands at LDS base + 16 l, so each lane
// fetches the global chunk that its (swizzled) LDS slot stands for.
// ---------------------------------------------------------------------------
constexpr int BG_M = 256, BG_N = 256;                 // the full tile (WT = 4)
constexpr int BG_LDS = 128 * 1024;                    // the stage ring

// BK: k depth of a stage; WT: the tile is TM = 64 WT square; NW: waves per
// workgroup, as 2 x NW/2 (rows x columns), so a wave owns a TM/2 x 2TM/NW
// sub-tile of FM x FN 32x32 MFMA blocks (WT x WT with 4 waves, one per SIMD;
// WT x WT/2 with 8 waves, two per SIMD).
template <int BK, int WT = 4, int NW = 4>
struct BigCfg {
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(WT == 2 || WT == 4, "WT");
  static_assert(NW == 4 || NW == 8, "NW");
  static constexpr int TM = 64 * WT;                  // tile rows = tile columns
  static constexpr int NWN = NW / 2;                  // waves along the columns
  static constexpr int WSM = TM / 2, WSN = TM / NWN;  // wave sub-tile
  static constexpr int FM = WSM / 32, FN = WSN / 32;  // MFMA blocks per wave
  static constexpr int ROWB = BK * 2;                 // bytes per LDS row
  static constexpr int STAGE = 2 * TM * ROWB;         // bytes per stage
  static constexpr int NST = BG_LDS / STAGE;          // stages in the ring
  static constexpr int CPR = BK / 8;                  // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;                // rows per load instruction
  static constexpr int LPO = TM / (NW * RPI);         // load instructions per operand
  static constexpr int LPS = 2 * LPO;                 // per stage
  static constexpr int SUB = BK / 16;                 // MFMA k-substeps per step
  static constexpr int NR = FM + FN;                  // operand reads per substep
  static constexpr int NM = FM * FN;                  // MFMAs per substep
  // Chunk c of row r sits in slot c ^ f(r). An MFMA operand read has lanes
  // 16g .. 16g+15 read one chunk of 16 consecutive rows; LDS serves a
  // ds_read_b128 in groups of 16 lanes over 64 four-byte banks, and row r's
  // chunk lands on bank quad (r * CPR + (c ^ f(r))) % 16, which f makes
  // distinct over the 16 rows: f(r) = (r >> 2) & 3 for 64-byte rows,
  // (r >> 1) & 7 for 128-byte rows (measured: no SQ_LDS_BANK_CONFLICT cycles
  // for the former; patterns that repeat within 16 rows cost about 4 cycles
  // per read).
  static DSPARK_DEV int swz_f(int row) { return (row / (16 / CPR)) & (CPR - 1); }
  static DSPARK_DEV int swz(int row, int chunk) { return row * ROWB + ((chunk ^ swz_f(row)) << 4); }
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One 16-byte direct global -> LDS load per lane. A plain function, so that
// kernel templates calling it with template-dependent addresses still
// instantiate in the host compilation pass, which has no such builtin.
DSPARK_DEV void lds_load16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)l, 16, 0, 0);
}

// Epilogues of the big-tile kernel (kKind): 0 float32 split-K partials,
// 1 the context K/V in the attention layout, 2 Eq 2 with its row norm
// deferred.
struct EpiPartialBig {         // out[z][r][n] = acc for r < M
  float* out;
  int64_t split_stride;
  static constexpr int kKind = 0;
  static constexpr bool kSwap = false;
};

// Eq 2 in one K split: Y = P * g (P = X W_c^T, g = ctx_norm) rounded to
// bf16, and per row and 256-column tile the sums of P^2 and of Y^2 (Y as
// stored). The row's RMS factor is then a per-row scalar: H_ctx = Y / rms(P),
// so the K/V product can take Y as its A operand and fold both norms into
// its row scale.
struct EpiNormBig {
  bf16* y;                     // [M][N]
  float* sums;                 // [M][N / 256][2]
  const float* g;              // [N]
  static constexpr int kKind = 2;
  static constexpr bool kSwap = true;     // a lane holds one row
};

template <typename S>
struct EpiKVBig {              // all layers' K/V, row scale, attention layout
  S* base;
  const float* rinv;
  int64_t Tpad;
  int T, d, hd, n_heads;       // d: columns of one K or V block (K/V heads * hd)
  int n_base;                  // column of the stacked K/V where this launch's columns start
  const int32_t* dst_row;      // null: row r at r (zeros at T .. Tpad-1); else row r < T at dst_row[r]
  static constexpr int kKind = 1;
  static constexpr bool kSwap = true;     // accumulate C^T: a lane holds one row
};

// Workgroup barrier without the release fence that __syncthreads() implies:
// that fence waits for every outstanding global load, including the direct
// LDS loads of later pipeline stages. The stage being consumed is waited for
// explicitly (wait_vmcnt); the memory clobber keeps LDS reads below it.
DSPARK_DEV void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8). The builtin, unlike inline asm, lets the compiler's
// own wait insertion see that the counters were drained.
template <int N>
DSPARK_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
DSPARK_DEV void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Each k-step is one scheduling region per k-substep (NM MFMAs). The MFMAs
// of a substep run with the NR operand reads of the next one interleaved,
// each read behind an MFMA, so that the wait for a substep's operands never
// covers a read issued just before it; in the last region, after the stage
// barrier, with the reads of the next step's first substep and the NL direct
// loads of the stage NST steps ahead. FRONT puts all the reads behind the
// first half of the MFMAs (two per MFMA where there are more reads than
// half the MFMAs), which leaves more MFMAs to cover the last read; measured
// 6% faster for the K/V product and 1.5% slower for the Eq 2 product than
// one read per MFMA.
#define DSPARK_BIG_SCHED_A(NR, NM, FRONT)                                                  \
  do {                                                                                     \
    constexpr int kHalf = (FRONT) ? ((NM) / 2 > 0 ? (NM) / 2 : 1) : (NM);                  \
    constexpr int kPer = ((NR) + kHalf - 1) / kHalf;                                       \
    constexpr int kGroups = ((NR) + kPer - 1) / kPer;                                      \
    _Pragma("unroll") for (int q = 0; q < kGroups; ++q) {                                  \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                   \
      __builtin_amdgcn_sched_group_barrier(0x100, kPer, 0);                                \
    }                                                                                      \
    _Pragma("unroll") for (int q = kGroups; q < (NM); ++q)                                 \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                   \
  } while (0)
// The first quarter of the MFMAs (at least one) with the operand reads, the
// next half (at least one) with the direct loads, then the rest.
#define DSPARK_BIG_SCHED_ISSUE(NR, NM, NL)                                                 \
  do {                                                                                     \
    constexpr int kQ1 = (NM) / 4 > 0 ? (NM) / 4 : 1;                                       \
    constexpr int kQ2 = (NM) / 2 > 0 ? (NM) / 2 : 1;                                       \
    _Pragma("unroll") for (int q = 0; q < kQ1; ++q) {                                      \
      __builtin_amdgcn_sched_group_barrier(0x100, ((NR) + kQ1 - 1) / kQ1, 0);              \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                   \
    }                                                                                      \
    _Pragma("unroll") for (int q = 0; q < kQ2; ++q) {                                      \
      __builtin_amdgcn_sched_group_barrier(0x010, ((NL) + kQ2 - 1) / kQ2, 0);              \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                   \
    }                                                                                      \
    _Pragma("unroll") for (int q = kQ1 + kQ2; q < (NM); ++q)                               \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                   \
  } while (0)

// 4x4 dword transpose among the 4 lanes of a DPP quad: afterwards a[m] of
// lane k is the a[k] that lane m held. Two exchange stages, lane ^ 2 then
// lane ^ 1, each moving two dwords per lane.
DSPARK_DEV void transpose4_quad(uint32_t (&a)[4], int k) {
  const bool lo2 = k < 2, even = (k & 1) == 0;
  const uint32_t s0 = lo2 ? a[2] : a[0], s1 = lo2 ? a[3] : a[1];
  const uint32_t r0 = __builtin_amdgcn_mov_dpp((int)s0, 0x4E, 0xf, 0xf, true);   // quad_perm 2,3,0,1
  const uint32_t r1 = __builtin_amdgcn_mov_dpp((int)s1, 0x4E, 0xf, 0xf, true);
  const uint32_t t0 = lo2 ? a[0] : r0, t1 = lo2 ? a[1] : r1;
  const uint32_t t2 = lo2 ? r0 : a[2], t3 = lo2 ? r1 : a[3];
  const uint32_t u0 = even ? t1 : t0, u1 = even ? t3 : t2;
  const uint32_t w0 = __builtin_amdgcn_mov_dpp((int)u0, 0xB1, 0xf, 0xf, true);   // quad_perm 1,0,3,2
  const uint32_t w1 = __builtin_amdgcn_mov_dpp((int)u1, 0xB1, 0xf, 0xf, true);
  a[0] = even ? t0 : w0;
  a[1] = even ? w0 : t1;
  a[2] = even ? t2 : w1;
  a[3] = even ? w1 : t3;
}

// The body of one big-tile workgroup: work item `logical` of `total` (split
// z, tile), with `smem` the stage ring followed by the tile's row scales.
template <class Epi, int HD, int BK, int WT, int NW>
DSPARK_DEV void gemm_big_body(char* smem, int logical, int total, ASegs a, const bf16* __restrict__ Bt,
                              int M, int MR, int N, int K, int k_per_split, Epi epi) {
  using C = BigCfg<BK, WT, NW>;
  constexpr int TM = C::TM, WSM = C::WSM, WSN = C::WSN, FM = C::FM, FN = C::FN;
  const int tiles_m = (MR + TM - 1) / TM;
  const int tiles_n = N / TM;
  const int ntiles = tiles_m * tiles_n;
  // Work items (split z, tile) are dealt to the 8 XCDs (workgroup i runs on
  // XCD i % 8) in contiguous runs, z-major, so an XCD owns whole K slices;
  // inside a slice, tiles go in groups of up to 4 m-tiles swept n by n, so
  // the XCD's L2 holds a few A panels while it walks the B panels (groups of
  // 4 measured 0.5-1% faster per forward than 8, and 16 5% slower).
  if (total % 8 == 0) logical = (logical % 8) * (total / 8) + logical / 8;
  const int z = logical / ntiles;
  const int t = logical % ntiles;
  const int G = min(tiles_m, 4);
  const int gsize = G * tiles_n;
  const int grp = t / gsize, first_m = grp * G;
  const int gm = min(tiles_m - first_m, G);
  const int tm = first_m + (t % gsize) % gm, tn = (t % gsize) / gm;
  const int m0 = tm * TM, n0 = tn * TM;
  const int kbeg = z * k_per_split;
  const int kend = min(K, kbeg + k_per_split);
  const int nsteps = kend > kbeg ? (kend - kbeg) / BK : 0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in a scalar register
  const int wm = wave / C::NWN, wn = wave % C::NWN;
  const int r32 = lane & 31, hi = lane >> 5;

  // lane i holds the address of A segment i; the loop reads it with a lane
  // select instead of a scalar memory load, whose wait would also drain the
  // LDS reads in flight
  uint64_t my_seg = 0;
#pragma unroll
  for (int i = 0; i < kMaxSegs; ++i)
    if (lane == i && i < a.nseg) my_seg = reinterpret_cast<uint64_t>(a.seg[i]);
  const uint32_t seg_lo = (uint32_t)my_seg, seg_hi = (uint32_t)(my_seg >> 32);

  // ---- direct global -> LDS loads of one stage (LPO for A, LPO for B per
  // thread). A wave's load instruction fills RPI LDS rows: lane l takes row
  // l / CPR and slot l % CPR. Each lane's byte offsets from the stage's scalar
  // base addresses are fixed for the whole tile, so a load is one
  // instruction on a scalar base and a 32-bit lane offset (the host
  // guarantees the offsets fit), and the LDS destinations are scalar values.
  const int rl = lane / C::CPR, slot = lane % C::CPR;
  uint32_t aoff[C::LPO], boff[C::LPO];
#pragma unroll
  for (int i = 0; i < C::LPO; ++i) {
    const int row = (i * NW + wave) * C::RPI + rl;
    const int ch = slot ^ C::swz_f(row);
    aoff[i] = (uint32_t)min(m0 + row, M - 1) * (uint32_t)(a.ld * 2) + (uint32_t)(ch * 16);
    boff[i] = (uint32_t)(n0 + row) * (uint32_t)(K * 2) + (uint32_t)(ch * 16);
  }
  auto issue = [&](int step, int stage) __attribute__((always_inline)) {
    const int k0 = kbeg + step * BK;
    const int sgi = k0 / a.seg_k;
    const int kin = k0 - sgi * a.seg_k;
    const uint64_t ap = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)seg_hi, sgi) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((int)seg_lo, sgi);
    const char* __restrict__ abase = reinterpret_cast<const char*>(ap) + (int64_t)kin * 2;
    const char* __restrict__ bbase = reinterpret_cast<const char*>(Bt) + (int64_t)k0 * 2;
    char* base = smem + stage * C::STAGE + wave * C::RPI * C::ROWB;
#pragma unroll
    for (int i = 0; i < C::LPO; ++i)
      lds_load16(abase + aoff[i], base + i * NW * C::RPI * C::ROWB);
#pragma unroll
    for (int i = 0; i < C::LPO; ++i)
      lds_load16(bbase + boff[i], base + TM * C::ROWB + i * NW * C::RPI * C::ROWB);
  };
  auto read_ops = [&](int stage, int ks, bf16x8 (&av)[FM], bf16x8 (&bv)[FN]) __attribute__((always_inline)) {
    const char* As = smem + stage * C::STAGE;
    const char* Bs = As + TM * C::ROWB;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      av[i] = *reinterpret_cast<const bf16x8*>(As + C::swz(wm * WSM + i * 32 + r32, 2 * ks + hi));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      bv[j] = *reinterpret_cast<const bf16x8*>(Bs + C::swz(wn * WSN + j * 32 + r32, 2 * ks + hi));
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  auto mfma16 = [&](const bf16x8 (&av)[FM], const bf16x8 (&bv)[FN]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = Epi::kSwap
                        ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[j], av[i], acc[i][j], 0, 0, 0)
                        : __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
  };

  // Row scales of the K/V epilogue: one direct LDS load per lane of the
  // first TM / 64 waves (the tile's TM rows), issued ahead of the stage
  // loads, so they hold no registers through the main loop and are waited
  // for with the first stage.
  // A cache target also stages each row's slab row (the row map) the same way.
  float* rsc_lds = reinterpret_cast<float*>(smem + BG_LDS);
  int32_t* dst_lds = reinterpret_cast<int32_t*>(smem + BG_LDS + TM * 4);
  if constexpr (Epi::kKind == 1) {
    if (nsteps > 0 && wave < TM / 64) {
      const int row = min(m0 + wave * 64 + lane, epi.T - 1);
      __builtin_amdgcn_global_load_lds(epi.rinv + row, (lds_ptr_t)(rsc_lds + wave * 64), 4, 0, 0);
      if (epi.dst_row)
        __builtin_amdgcn_global_load_lds(epi.dst_row + row, (lds_ptr_t)(dst_lds + wave * 64), 4, 0, 0);
    }
  }

  // Ring of NST stages of LPS direct loads per thread. Steps 0 .. NST-1 are
  // loaded up front (after the row-scale load, which the first wait covers).
  // In step s, once every wave has read its last operands of stage s % NST
  // and stage (s+1) % NST has landed (the barrier), the loads of step s+NST
  // go into stage s % NST. Near the end those loads repeat the last step
  // into the freed stage (in bounds, never read), which keeps every wait
  // count fixed.
  bf16x8 av0[FM], bv0[FN], av1[FM], bv1[FN];
  auto run_step = [&](int step, auto last) __attribute__((always_inline)) {
    const int st = step % C::NST;
#pragma unroll
    for (int ks = 1; ks < C::SUB; ++ks) {
      if (ks & 1) {
        read_ops(st, ks, av1, bv1);
        mfma16(av0, bv0);
      } else {
        read_ops(st, ks, av0, bv0);
        mfma16(av1, bv1);
      }
      DSPARK_BIG_SCHED_A(C::NR, C::NM, Epi::kKind == 1);
    }
    // SUB is even: the last substep's operands are in av1 / bv1
    if constexpr (!decltype(last)::value) {
      wait_vmcnt<C::LPS * (C::NST - 2)>();
      wait_lgkm0();
      stage_barrier();
      read_ops((step + 1) % C::NST, 0, av0, bv0);
      issue(min(step + C::NST, nsteps - 1), st);
      mfma16(av1, bv1);
      DSPARK_BIG_SCHED_ISSUE(C::NR, C::NM, C::LPS);
    } else {
      mfma16(av1, bv1);
    }
  };
  if (nsteps > 0) {
#pragma unroll
    for (int st = 0; st < C::NST; ++st) issue(min(st, nsteps - 1), st);
    wait_vmcnt<C::LPS * (C::NST - 1)>();
    stage_barrier();
    read_ops(0, 0, av0, bv0);
    for (int step = 0; step < nsteps - 1; ++step) run_step(step, std::false_type{});
    run_step(nsteps - 1, std::true_type{});
    wait_vmcnt<0>();
  }

  if constexpr (Epi::kKind == 2) {
    // Transposed accumulators, as in the K/V epilogue below: (i, j, r) of
    // this lane is tile row wm*WSM + i*32 + lane%32 and tile column
    // wn*WSN + j*32 + 8*(r/4) + 4*(lane/32) + r%4. Y leaves as 16-byte
    // vectors of 8 columns of one row (lanes l and l^32 trade halves); the
    // row sums meet in LDS past the stage ring (lanes l and l^32 first, then
    // the NWN waves of a row block), and one thread per tile row writes them.
    float* red = reinterpret_cast<float*>(smem + BG_LDS);   // [NWN][TM][2]
    const int nw = n0 + wn * WSN;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int lr = wm * WSM + i * 32 + r32;
      const int64_t row = (int64_t)m0 + lr;
      float sp = 0.f, sy = 0.f;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int cb = nw + j * 32;
        uint32_t P[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 gv = *reinterpret_cast<const f32x4*>(epi.g + cb + 8 * q + 4 * hi);
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const float p0 = acc[i][j][4 * q + 2 * x], p1 = acc[i][j][4 * q + 2 * x + 1];
            const float y0 = static_cast<float>(from_f32<bf16>(p0 * gv[2 * x]));
            const float y1 = static_cast<float>(from_f32<bf16>(p1 * gv[2 * x + 1]));
            sp += p0 * p0 + p1 * p1;
            sy += y0 * y0 + y1 * y1;
            P[q][x] = pack_bf16x2(y0, y1);   // exact: y0, y1 are bf16 values
          }
        }
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          // lanes < 32 finish column group qq of 8, lanes >= 32 group qq + 2
          const auto s0 = __builtin_amdgcn_permlane32_swap(P[qq][0], P[qq + 2][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(P[qq][1], P[qq + 2][1], false, false);
          const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
          if (row < M) st16(epi.y + row * N + cb + 8 * (qq + 2 * hi), v);
        }
      }
      sp += __shfl_xor(sp, 32, kWave);
      sy += __shfl_xor(sy, 32, kWave);
      if (hi == 0) {
        red[2 * (wn * TM + lr)] = sp;
        red[2 * (wn * TM + lr) + 1] = sy;
      }
    }
    wait_lgkm0();
    stage_barrier();
    if (tid < TM && m0 + tid < M) {
      float sp = 0.f, sy = 0.f;
#pragma unroll
      for (int w = 0; w < C::NWN; ++w) {
        sp += red[2 * (w * TM + tid)];
        sy += red[2 * (w * TM + tid) + 1];
      }
      *reinterpret_cast<f32x2*>(epi.sums + 2 * ((int64_t)(m0 + tid) * (N / TM) + tn)) = f32x2{sp, sy};
    }
  } else if constexpr (Epi::kKind == 0) {
    // accumulator (i, j, r) of this lane: tile row wm*WSM + i*32 + 8*(r/4) +
    // 4*(lane/32) + r%4, tile column wn*WSN + j*32 + lane%32
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * WSM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int col = n0 + wn * WSN + j * 32 + (lane & 31);
          if (row < M) epi.out[z * epi.split_stride + (int64_t)row * N + col] = acc[i][j][r];
        }
  } else {
    // The K/V vectors are stored non-temporally: the attention that reads
    // them later streams about 12% faster (T = 131072 and a ragged batch;
    // the forward 1-3% faster at T >= 8192, neutral at T = 2048).
    // Transposed accumulators: (i, j, r) of this lane is tile row (token)
    // wm*WSM + i*32 + lane%32 and tile column wn*WSN + j*32 + 8*(r/4) +
    // 4*(lane/32) + r%4. After the row scale and rounding, each 32x32 block
    // becomes 16-byte vectors of the attention layout with lane exchanges
    // only: K (one token x 8 columns) pairs lane l with l^32, V (4 tokens x 2
    // columns) transposes dwords among the 4 lanes of consecutive tokens.
    // With a row map (a cache target) row r < T goes to slab row dst_row[r]
    // and no padding rows are written; a V vector whose four rows land on
    // four consecutive slab rows starting at a multiple of 4 is stored
    // whole, any other as four dwords.
    using S = std::remove_pointer_t<decltype(epi.base)>;
    using L = KVLayout<S>;
    static_assert(sizeof(S) == 2 && L::R == 4, "bf16 K/V layout");
    const int nw = epi.n_base + n0 + wn * WSN;   // the wave's WSN columns lie in one K or V block
    const int layer = nw / (2 * epi.d);
    const int kv = (nw / epi.d) & 1;
    const int k4 = lane & 3;
    const bool mapped = epi.dst_row != nullptr;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t tb = (int64_t)m0 + wm * WSM + i * 32;
      const int lr = wm * WSM + i * 32;   // the block's first row within the tile
      // padding rows (T <= row < Tpad) are written as zeros
      const float rs = (nsteps > 0 && tb + r32 < epi.T) ? rsc_lds[lr + r32] : 0.f;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int w = (nw + j * 32) % epi.d;
        const int head = w / HD, c0 = w % HD;
        S* hb = epi.base + L::head_base(layer, kv, head, epi.n_heads, epi.Tpad, HD);
        // P[q][x]: columns 8q + 4*(lane/32) + 2x, +1 of token tb + lane%32
        uint32_t P[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int x = 0; x < 2; ++x)
            P[q][x] = pack_bf16x2(acc[i][j][4 * q + 2 * x] * rs, acc[i][j][4 * q + 2 * x + 1] * rs);
        if (kv == 0) {
          const int64_t t = mapped ? (int64_t)dst_lds[lr + r32] : tb + r32;
          const bool live = mapped ? tb + r32 < epi.T : t < epi.Tpad;
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            // lanes < 32 finish column group qq of 8, lanes >= 32 group qq + 2
            const auto s0 = __builtin_amdgcn_permlane32_swap(P[qq][0], P[qq + 2][0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(P[qq][1], P[qq + 2][1], false, false);
            const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
            const int g = qq + 2 * hi;
            if (live)
              __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(hb + L::k_off(t, c0 + 8 * g, HD)));
          }
        } else {
          const int64_t t0 = tb + (r32 & ~3);
          const int q0 = lr + (r32 & ~3);   // the quad's first row within the tile
#pragma unroll
          for (int set = 0; set < 2; ++set) {
            // a[c] = column pair 4*(2*set + c/2) + 2*(lane/32) + c%2 of this
            // lane's token; after the transpose lane k of the quad holds pair
            // c = k for tokens t0 .. t0+3
            uint32_t a[4] = {P[2 * set][0], P[2 * set][1], P[2 * set + 1][0], P[2 * set + 1][1]};
            transpose4_quad(a, k4);
            const int p = 4 * (2 * set + (k4 >> 1)) + 2 * hi + (k4 & 1);
            const u32x4 v = {a[0], a[1], a[2], a[3]};
            if (!mapped) {
              if (t0 < epi.Tpad)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(hb + L::v_off(t0, c0 + 2 * p, HD)));
            } else {
              const int64_t d0 = dst_lds[q0];
              const bool whole = t0 + 3 < epi.T && (d0 & 3) == 0 && dst_lds[q0 + 3] == d0 + 3;
              if (whole) {
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(hb + L::v_off(d0, c0 + 2 * p, HD)));
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (t0 + e < epi.T)
                    __builtin_nontemporal_store(
                        a[e], reinterpret_cast<uint32_t*>(hb + L::v_off(dst_lds[q0 + e], c0 + 2 * p, HD)));
              }
            }
          }
        }
      }
    }
  }
}

// The same body, persistent (one K split, an even number of k-steps): the
// workgroup goes on to items logical + stride, logical + 2 stride, ..., and
// the last k-steps of one tile load the first stages of the next, so the
// next tile's operands arrive while this tile's epilogue runs. A separate
// function: folding the tile loop into the body above changed the register
// allocation of the single-tile kernels (the K/V tail kernel spilled, the
// fuse GEMM ran 3% slower).
template <class Epi, int HD, int BK, int WT, int NW>
DSPARK_DEV void gemm_big_body_persistent(char* smem, int logical, int total, ASegs a,
                                         const bf16* __restrict__ Bt, int M, int MR, int N, int K,
                                         int k_per_split, Epi epi, int stride) {
  constexpr bool PERSIST = true;
  using C = BigCfg<BK, WT, NW>;
  constexpr int TM = C::TM, WSM = C::WSM, WSN = C::WSN, FM = C::FM, FN = C::FN;
  static_assert(C::NST == 2, "the persistent loop hands over two stages");
  const int tiles_m = (MR + TM - 1) / TM;
  const int tiles_n = N / TM;
  const int ntiles = tiles_m * tiles_n;
  // Work items (split z, tile) are dealt to the 8 XCDs (workgroup i runs on
  // XCD i % 8) in contiguous runs, z-major, so an XCD owns whole K slices;
  // inside a slice, tiles go in groups of up to 4 m-tiles swept n by n, so
  // the XCD's L2 holds a few A panels while it walks the B panels (groups of
  // 4 measured 0.5-1% faster per forward than 8, and 16 5% slower). A
  // persistent workgroup's items logical + i * stride (stride a multiple of
  // 8) stay on its XCD, and the XCD's workgroups walk its run together.
  auto decode = [&](int item, int& z_, int& m0_, int& tn_) __attribute__((always_inline)) {
    if (total % 8 == 0) item = (item % 8) * (total / 8) + item / 8;
    z_ = item / ntiles;
    const int t = item % ntiles;
    const int G = min(tiles_m, 4);
    const int gsize = G * tiles_n;
    const int grp = t / gsize, first_m = grp * G;
    const int gm = min(tiles_m - first_m, G);
    m0_ = (first_m + (t % gsize) % gm) * TM;
    tn_ = (t % gsize) / gm;
  };
  int z, m0, tn;
  decode(logical, z, m0, tn);
  int n0 = tn * TM;
  const int kbeg = z * k_per_split;   // z = 0 for every item
  const int kend = min(K, kbeg + k_per_split);
  const int nsteps = kend > kbeg ? (kend - kbeg) / BK : 0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in a scalar register
  const int wm = wave / C::NWN, wn = wave % C::NWN;
  const int r32 = lane & 31, hi = lane >> 5;

  // lane i holds the address of A segment i; the loop reads it with a lane
  // select instead of a scalar memory load, whose wait would also drain the
  // LDS reads in flight
  uint64_t my_seg = 0;
#pragma unroll
  for (int i = 0; i < kMaxSegs; ++i)
    if (lane == i && i < a.nseg) my_seg = reinterpret_cast<uint64_t>(a.seg[i]);
  const uint32_t seg_lo = (uint32_t)my_seg, seg_hi = (uint32_t)(my_seg >> 32);

  // ---- direct global -> LDS loads of one stage (LPO for A, LPO for B per
  // thread). A wave's load instruction fills RPI LDS rows: lane l takes row
  // l / CPR and slot l % CPR. Each lane's byte offsets from the stage's scalar
  // base addresses are fixed for the whole tile, so a load is one
  // instruction on a scalar base and a 32-bit lane offset (the host
  // guarantees the offsets fit), and the LDS destinations are scalar values.
  const int rl = lane / C::CPR, slot = lane % C::CPR;
  uint32_t aoff[C::LPO], boff[C::LPO];
  auto set_offsets = [&](int m0_, int n0_) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::LPO; ++i) {
      const int row = (i * NW + wave) * C::RPI + rl;
      const int ch = slot ^ C::swz_f(row);
      aoff[i] = (uint32_t)min(m0_ + row, M - 1) * (uint32_t)(a.ld * 2) + (uint32_t)(ch * 16);
      boff[i] = (uint32_t)(n0_ + row) * (uint32_t)(K * 2) + (uint32_t)(ch * 16);
    }
  };
  set_offsets(m0, n0);
  auto issue = [&](int step, int stage) __attribute__((always_inline)) {
    const int k0 = kbeg + step * BK;
    const int sgi = k0 / a.seg_k;
    const int kin = k0 - sgi * a.seg_k;
    const uint64_t ap = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)seg_hi, sgi) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((int)seg_lo, sgi);
    const char* __restrict__ abase = reinterpret_cast<const char*>(ap) + (int64_t)kin * 2;
    const char* __restrict__ bbase = reinterpret_cast<const char*>(Bt) + (int64_t)k0 * 2;
    char* base = smem + stage * C::STAGE + wave * C::RPI * C::ROWB;
#pragma unroll
    for (int i = 0; i < C::LPO; ++i)
      lds_load16(abase + aoff[i], base + i * NW * C::RPI * C::ROWB);
#pragma unroll
    for (int i = 0; i < C::LPO; ++i)
      lds_load16(bbase + boff[i], base + TM * C::ROWB + i * NW * C::RPI * C::ROWB);
  };
  auto read_ops = [&](int stage, int ks, bf16x8 (&av)[FM], bf16x8 (&bv)[FN]) __attribute__((always_inline)) {
    const char* As = smem + stage * C::STAGE;
    const char* Bs = As + TM * C::ROWB;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      av[i] = *reinterpret_cast<const bf16x8*>(As + C::swz(wm * WSM + i * 32 + r32, 2 * ks + hi));
#pragma unroll
    for (int j = 0; j < FN; ++j)
      bv[j] = *reinterpret_cast<const bf16x8*>(Bs + C::swz(wn * WSN + j * 32 + r32, 2 * ks + hi));
  };

  // A tile's first MFMAs take a zero accumulator instead of the previous
  // tile's values, so no instructions clear the accumulators between tiles.
  f32x16 acc[FM][FN];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  };
  auto mfma16 = [&](const bf16x8 (&av)[FM], const bf16x8 (&bv)[FN], auto fresh) __attribute__((always_inline)) {
    constexpr f32x16 zero = {};
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const f32x16 c = decltype(fresh)::value ? zero : acc[i][j];
        acc[i][j] = Epi::kSwap ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[j], av[i], c, 0, 0, 0)
                               : __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], c, 0, 0, 0);
      }
  };

  // Row scales of the K/V epilogue: one direct LDS load per lane of the
  // first TM / 64 waves (the tile's TM rows), issued ahead of the stage
  // loads, so they hold no registers through the main loop and are waited
  // for with the first stage.
  // A cache target also stages each row's slab row (the row map) the same way.
  // Two buffers, by tile parity: a persistent workgroup loads the next
  // tile's while this tile's epilogue reads its own.
  int par = 0;
  float* rsc_lds = reinterpret_cast<float*>(smem + BG_LDS);
  int32_t* dst_lds = reinterpret_cast<int32_t*>(smem + BG_LDS + TM * 4);
  auto load_rows = [&](int m0_, int par_) __attribute__((always_inline)) {
    if constexpr (Epi::kKind == 1) {
      if (nsteps > 0 && wave < TM / 64) {
        float* rs = reinterpret_cast<float*>(smem + BG_LDS + par_ * 2 * TM * 4);
        int32_t* ds = reinterpret_cast<int32_t*>(smem + BG_LDS + par_ * 2 * TM * 4 + TM * 4);
        const int row = min(m0_ + wave * 64 + lane, epi.T - 1);
        __builtin_amdgcn_global_load_lds(epi.rinv + row, (lds_ptr_t)(rs + wave * 64), 4, 0, 0);
        if (epi.dst_row)
          __builtin_amdgcn_global_load_lds(epi.dst_row + row, (lds_ptr_t)(ds + wave * 64), 4, 0, 0);
      }
    }
  };
  load_rows(m0, 0);

  // Ring of NST stages of LPS direct loads per thread. Steps 0 .. NST-1 are
  // loaded up front (after the row-scale load, which the first wait covers).
  // In step s, once every wave has read its last operands of stage s % NST
  // and stage (s+1) % NST has landed (the barrier), the loads of step s+NST
  // go into stage s % NST. Near the end those loads repeat the last step
  // into the freed stage (in bounds, never read), which keeps every wait
  // count fixed; a persistent workgroup with a next tile loads that tile's
  // first step there instead (its offsets replace this tile's, which no
  // later load needs).
  bool has_next = false;
  int nm0 = 0, nn0 = 0, ntn = 0;
  bf16x8 av0[FM], bv0[FN], av1[FM], bv1[FN];
  auto run_step = [&](int step, auto last, auto first) __attribute__((always_inline)) {
    const int st = step % C::NST;
#pragma unroll
    for (int ks = 1; ks < C::SUB; ++ks) {
      if (ks & 1) {
        read_ops(st, ks, av1, bv1);
        if (ks == 1 && decltype(first)::value)
          mfma16(av0, bv0, std::true_type{});
        else
          mfma16(av0, bv0, std::false_type{});
      } else {
        read_ops(st, ks, av0, bv0);
        mfma16(av1, bv1, std::false_type{});
      }
      DSPARK_BIG_SCHED_A(C::NR, C::NM, Epi::kKind == 1);
    }
    // SUB is even: the last substep's operands are in av1 / bv1
    if constexpr (!decltype(last)::value) {
      wait_vmcnt<C::LPS * (C::NST - 2)>();
      wait_lgkm0();
      stage_barrier();
      read_ops((step + 1) % C::NST, 0, av0, bv0);
      if (step + C::NST < nsteps) {
        issue(step + C::NST, st);
      } else if (PERSIST && has_next) {
        if (step + C::NST == nsteps) set_offsets(nm0, nn0);
        issue(step + C::NST - nsteps, st);
      } else {
        issue(nsteps - 1, st);
      }
      mfma16(av1, bv1, std::false_type{});
      DSPARK_BIG_SCHED_ISSUE(C::NR, C::NM, C::LPS);
    } else {
      mfma16(av1, bv1, std::false_type{});
    }
  };
  if (nsteps > 0) {
#pragma unroll
    for (int st = 0; st < C::NST; ++st) issue(min(st, nsteps - 1), st);
    wait_vmcnt<C::LPS * (C::NST - 1)>();
    stage_barrier();
    read_ops(0, 0, av0, bv0);
  }
  for (;;) {
  if constexpr (PERSIST) {
    has_next = logical + stride < total && nsteps >= 2;
    if (has_next) {
      int nz;
      decode(logical + stride, nz, nm0, ntn);
      nn0 = ntn * TM;
    }
  }
  if (nsteps > 1) {
    run_step(0, std::false_type{}, std::true_type{});
    for (int step = 1; step < nsteps - 1; ++step) run_step(step, std::false_type{}, std::false_type{});
    run_step(nsteps - 1, std::true_type{}, std::false_type{});
  } else if (nsteps == 1) {
    run_step(0, std::true_type{}, std::true_type{});
  } else {
    zero_acc();
  }
  if (nsteps > 0) {
    if (PERSIST && has_next) {
      // every wave is done with the last stage: the next tile's second step
      // goes there, and its row scales into the other buffer
      wait_lgkm0();
      stage_barrier();
      issue(1, 1);
      load_rows(nm0, par ^ 1);
    } else {
      wait_vmcnt<0>();
    }
  }

  if constexpr (Epi::kKind == 2) {
    // Transposed accumulators, as in the K/V epilogue below: (i, j, r) of
    // this lane is tile row wm*WSM + i*32 + lane%32 and tile column
    // wn*WSN + j*32 + 8*(r/4) + 4*(lane/32) + r%4. Y leaves as 16-byte
    // vectors of 8 columns of one row (lanes l and l^32 trade halves); the
    // row sums meet in LDS past the stage ring (lanes l and l^32 first, then
    // the NWN waves of a row block), and one thread per tile row writes them.
    float* red = reinterpret_cast<float*>(smem + BG_LDS);   // [NWN][TM][2]
    const int nw = n0 + wn * WSN;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int lr = wm * WSM + i * 32 + r32;
      const int64_t row = (int64_t)m0 + lr;
      float sp = 0.f, sy = 0.f;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int cb = nw + j * 32;
        uint32_t P[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 gv = *reinterpret_cast<const f32x4*>(epi.g + cb + 8 * q + 4 * hi);
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const float p0 = acc[i][j][4 * q + 2 * x], p1 = acc[i][j][4 * q + 2 * x + 1];
            const float y0 = static_cast<float>(from_f32<bf16>(p0 * gv[2 * x]));
            const float y1 = static_cast<float>(from_f32<bf16>(p1 * gv[2 * x + 1]));
            sp += p0 * p0 + p1 * p1;
            sy += y0 * y0 + y1 * y1;
            P[q][x] = pack_bf16x2(y0, y1);   // exact: y0, y1 are bf16 values
          }
        }
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          // lanes < 32 finish column group qq of 8, lanes >= 32 group qq + 2
          const auto s0 = __builtin_amdgcn_permlane32_swap(P[qq][0], P[qq + 2][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(P[qq][1], P[qq + 2][1], false, false);
          const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
          if (row < M) st16(epi.y + row * N + cb + 8 * (qq + 2 * hi), v);
        }
      }
      sp += __shfl_xor(sp, 32, kWave);
      sy += __shfl_xor(sy, 32, kWave);
      if (hi == 0) {
        red[2 * (wn * TM + lr)] = sp;
        red[2 * (wn * TM + lr) + 1] = sy;
      }
    }
    wait_lgkm0();
    stage_barrier();
    if (tid < TM && m0 + tid < M) {
      float sp = 0.f, sy = 0.f;
#pragma unroll
      for (int w = 0; w < C::NWN; ++w) {
        sp += red[2 * (w * TM + tid)];
        sy += red[2 * (w * TM + tid) + 1];
      }
      *reinterpret_cast<f32x2*>(epi.sums + 2 * ((int64_t)(m0 + tid) * (N / TM) + tn)) = f32x2{sp, sy};
    }
  } else if constexpr (Epi::kKind == 0) {
    // accumulator (i, j, r) of this lane: tile row wm*WSM + i*32 + 8*(r/4) +
    // 4*(lane/32) + r%4, tile column wn*WSN + j*32 + lane%32
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * WSM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int col = n0 + wn * WSN + j * 32 + (lane & 31);
          if (row < M) epi.out[z * epi.split_stride + (int64_t)row * N + col] = acc[i][j][r];
        }
  } else {
    // The K/V epilogue of the single-tile body (see there), with the
    // addresses of the packed (unmapped) target split into a per-lane 32-bit
    // byte offset inside a head slab, fixed per row block, and a wave-uniform
    // head base: a store then costs no 64-bit address arithmetic. A head slab
    // of the packed workspace holds Tpad * HD elements, under 4 GiB because
    // H_ctx (T * d >= Tpad * HD elements, checked on the host) is. A cache
    // target (row map) keeps the general form.
    using S = std::remove_pointer_t<decltype(epi.base)>;
    using L = KVLayout<S>;
    static_assert(sizeof(S) == 2 && L::R == 4, "bf16 K/V layout");
    const int nw = epi.n_base + n0 + wn * WSN;   // the wave's WSN columns lie in one K or V block
    const int layer = nw / (2 * epi.d);
    const int kv = (nw / epi.d) & 1;
    const int k4 = lane & 3;
    const bool mapped = epi.dst_row != nullptr;
    if (!mapped) {
      const int w0 = nw - (2 * layer + kv) * epi.d;   // the wave's first column in its K or V block
      constexpr int KG = 128 / HD;
      // lane parts of the K and V offsets (elements), independent of the row block
      const uint32_t k_lane = (uint32_t)hi * 1024u;
      const uint32_t v_lane = 32u * (uint32_t)(k4 >> 1) + 16u * (uint32_t)hi + 8u * (uint32_t)(k4 & 1);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int tb = m0 + wm * WSM + i * 32;
        const int lr = wm * WSM + i * 32;
        const float rs = (nsteps > 0 && tb + r32 < epi.T) ? rsc_lds[lr + r32] : 0.f;
        const int t = tb + r32;                 // K: this lane's token
        const int t0 = tb + (r32 & ~3);         // V: the token quad of this lane
        const int kk = t0 & 63;
        const uint32_t kofs = (uint32_t)(t >> 6) * (HD * 64u) + (uint32_t)(t & 63) * 8u + k_lane;
        const uint32_t vofs = (uint32_t)(t0 >> 6) * (HD * 64u) +
                              (uint32_t)((kk / (KG * 4)) * 64 + ((kk / 4) % KG) * (HD / 2)) * 8u + v_lane;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int w = w0 + j * 32;
          const int head = w / HD, c0 = w % HD;
          S* hb = epi.base + L::head_base(layer, kv, head, epi.n_heads, epi.Tpad, HD);
          uint32_t P[4][2];
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int x = 0; x < 2; ++x)
              P[q][x] = pack_bf16x2(acc[i][j][4 * q + 2 * x] * rs, acc[i][j][4 * q + 2 * x + 1] * rs);
          if (kv == 0) {
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
              const auto s0 = __builtin_amdgcn_permlane32_swap(P[qq][0], P[qq + 2][0], false, false);
              const auto s1 = __builtin_amdgcn_permlane32_swap(P[qq][1], P[qq + 2][1], false, false);
              const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
              S* base = hb + (c0 / 8 + qq) * 512;   // wave-uniform
              if (t < epi.Tpad)
                __builtin_nontemporal_store(
                    v, reinterpret_cast<u32x4*>(reinterpret_cast<char*>(base) + (size_t)(kofs * 2u)));
            }
          } else {
#pragma unroll
            for (int set = 0; set < 2; ++set) {
              uint32_t a[4] = {P[2 * set][0], P[2 * set][1], P[2 * set + 1][0], P[2 * set + 1][1]};
              transpose4_quad(a, k4);
              const u32x4 v = {a[0], a[1], a[2], a[3]};
              S* base = hb + c0 * 4 + 64 * set;       // wave-uniform
              if (t0 < epi.Tpad)
                __builtin_nontemporal_store(
                    v, reinterpret_cast<u32x4*>(reinterpret_cast<char*>(base) + (size_t)(vofs * 2u)));
            }
          }
        }
      }
    } else {
  #pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int64_t tb = (int64_t)m0 + wm * WSM + i * 32;
        const int lr = wm * WSM + i * 32;   // the block's first row within the tile
        // padding rows (T <= row < Tpad) are written as zeros
        const float rs = (nsteps > 0 && tb + r32 < epi.T) ? rsc_lds[lr + r32] : 0.f;
  #pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int w = (nw + j * 32) % epi.d;
          const int head = w / HD, c0 = w % HD;
          S* hb = epi.base + L::head_base(layer, kv, head, epi.n_heads, epi.Tpad, HD);
          // P[q][x]: columns 8q + 4*(lane/32) + 2x, +1 of token tb + lane%32
          uint32_t P[4][2];
  #pragma unroll
          for (int q = 0; q < 4; ++q)
  #pragma unroll
            for (int x = 0; x < 2; ++x)
              P[q][x] = pack_bf16x2(acc[i][j][4 * q + 2 * x] * rs, acc[i][j][4 * q + 2 * x + 1] * rs);
          if (kv == 0) {
            const int64_t t = mapped ? (int64_t)dst_lds[lr + r32] : tb + r32;
            const bool live = mapped ? tb + r32 < epi.T : t < epi.Tpad;
  #pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
              // lanes < 32 finish column group qq of 8, lanes >= 32 group qq + 2
              const auto s0 = __builtin_amdgcn_permlane32_swap(P[qq][0], P[qq + 2][0], false, false);
              const auto s1 = __builtin_amdgcn_permlane32_swap(P[qq][1], P[qq + 2][1], false, false);
              const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
              const int g = qq + 2 * hi;
              if (live)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(hb + L::k_off(t, c0 + 8 * g, HD)));
            }
          } else {
            const int64_t t0 = tb + (r32 & ~3);
            const int q0 = lr + (r32 & ~3);   // the quad's first row within the tile
  #pragma unroll
            for (int set = 0; set < 2; ++set) {
              // a[c] = column pair 4*(2*set + c/2) + 2*(lane/32) + c%2 of this
              // lane's token; after the transpose lane k of the quad holds pair
              // c = k for tokens t0 .. t0+3
              uint32_t a[4] = {P[2 * set][0], P[2 * set][1], P[2 * set + 1][0], P[2 * set + 1][1]};
              transpose4_quad(a, k4);
              const int p = 4 * (2 * set + (k4 >> 1)) + 2 * hi + (k4 & 1);
              const u32x4 v = {a[0], a[1], a[2], a[3]};
              if (!mapped) {
                if (t0 < epi.Tpad)
                  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(hb + L::v_off(t0, c0 + 2 * p, HD)));
              } else {
                const int64_t d0 = dst_lds[q0];
                const bool whole = t0 + 3 < epi.T && (d0 & 3) == 0 && dst_lds[q0 + 3] == d0 + 3;
                if (whole) {
                  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(hb + L::v_off(d0, c0 + 2 * p, HD)));
                } else {
  #pragma unroll
                  for (int e = 0; e < 4; ++e)
                    if (t0 + e < epi.T)
                      __builtin_nontemporal_store(
                          a[e], reinterpret_cast<uint32_t*>(hb + L::v_off(dst_lds[q0 + e], c0 + 2 * p, HD)));
                }
              }
            }
          }
        }
      }
    }
  }
  if (!(PERSIST && has_next)) break;
  // the next tile: its first two stages and row scales were requested
  // before the epilogue above
  logical += stride;
  m0 = nm0;
  n0 = nn0;
  tn = ntn;
  par ^= 1;
  rsc_lds = reinterpret_cast<float*>(smem + BG_LDS + par * 2 * TM * 4);
  dst_lds = reinterpret_cast<int32_t*>(smem + BG_LDS + par * 2 * TM * 4 + TM * 4);
  wait_vmcnt<0>();
  stage_barrier();
  read_ops(0, 0, av0, bv0);
  }
}

// the stage ring, then the epilogue's own part: the tile's row scales and
// row map (K/V) or its row sums of each column wave (Eq 2 norm); one LDS
// object, so the compiler's tracking of direct LDS loads sees a single target
template <class Epi, int WT, int NW>
constexpr int big_lds_bytes() {
  return BG_LDS + (Epi::kKind == 1 ? 4 * 64 * WT * 4 : Epi::kKind == 2 ? (NW / 2) * 64 * WT * 2 * 4 : 0);
}

template <class Epi, int HD, int BK, int WT, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_big_kernel(ASegs a, const bf16* __restrict__ Bt, int M,
                                                           int MR, int N, int K, int k_per_split, Epi epi) {
  __shared__ __attribute__((aligned(16))) char smem[big_lds_bytes<Epi, WT, NW>()];
  const int ntiles = ((MR + 64 * WT - 1) / (64 * WT)) * (N / (64 * WT));
  gemm_big_body<Epi, HD, BK, WT, NW>(smem, blockIdx.x + (int)gridDim.x * (int)blockIdx.y,
                                     ntiles * (int)gridDim.y, a, Bt, M, MR, N, K, k_per_split, epi);
}

// The K/V product in whole rounds of 256x256 tiles, persistent: one
// workgroup per CU walks tiles blockIdx.x, + gridDim.x, ..., loading each next
// tile's first two stages and row scales before the current tile's epilogue
// (a K/V tile lasts only d / 64 k-steps, so the pipeline fill of every tile
// is a visible share of its time).
template <class Epi, int HD, int BK, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_kv_persistent_kernel(ASegs a, const bf16* __restrict__ Bt, int M,
                                                                     int MR, int N, int K, Epi epi) {
  __shared__ __attribute__((aligned(16))) char smem[big_lds_bytes<Epi, 4, NW>()];
  const int ntiles = ((MR + 255) / 256) * (N / 256);
  gemm_big_body_persistent<Epi, HD, BK, 4, NW>(smem, blockIdx.x, ntiles, a, Bt, M, MR, N, K, K, epi,
                                                (int)gridDim.x);
}

// The K/V product with its partly filled last round of 256x256 tiles done as
// 128x128 tiles, in one grid: workgroups [0, nbig) take the 256x256 tiles of
// columns [0, nb), the rest the 128x128 tiles of columns [nb, N). The small
// tiles start as soon as a CU is free, with no launch boundary between.
template <class Epi, int HD, int BK, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_kv_tail_kernel(ASegs a, const bf16* __restrict__ Bt, int M,
                                                               int MR, int N, int K, int nb, int nbig,
                                                               Epi epi) {
  __shared__ __attribute__((aligned(16))) char smem[big_lds_bytes<Epi, 4, NW>()];
  const int bid = blockIdx.x;
  if (bid < nbig) {
    gemm_big_body<Epi, HD, BK, 4, NW>(smem, bid, nbig, a, Bt, M, MR, nb, K, K, epi);
  } else {
    Epi e = epi;
    e.n_base = epi.n_base + nb;
    gemm_big_body<Epi, HD, BK, 2, NW>(smem, bid - nbig, (int)gridDim.x - nbig, a, Bt + (int64_t)nb * K, M,
                                      MR, N - nb, K, K, e);
  }
}

static int pick_gemm_bm(int M) { return M >= 4096 ? 128 : 64; }
// k-tile depth of the big-tile kernel per product. Whole-line 64-deep tiles
// for both: alternating runs on one GPU measured the forward 1-2% faster at
// T = 2048 and 131072 than with 32-deep tiles (the K/V GEMM gains 3-9%; the
// fuse GEMM, which streams its taps from HBM, loses up to 4% at T = 131072
// for the shorter prefetch distance, and gains 5% at T = 2048).
constexpr int kFuseBK = 64, kKvBK = 64;
constexpr int kBigWaves = 8;   // waves per big-tile workgroup
static bool use_big_tiles(int dtype, int64_t M, int N) { return dtype == 1 && N % BG_N == 0 && M >= 512; }

// Column tiles of the K/V product done with 256x256 tiles; the rest of the
// columns go to 128x128 tiles of the same kernel body, in the same grid. With one
// 128 KiB workgroup per CU the big tiles run in rounds of kCUs; when the last
// round would be partly filled, its columns as four times as many 128x128
// tiles (each about half a big tile's time, at their lower operand reuse)
// finish sooner: at T = 2048 and 5 layers of d = 1024, 320 big tiles take
// two rounds, 256 big tiles plus 256 small ones about one and a half.
constexpr int kCUs = 256;
static int kv_big_columns(int Mrows, int N) {
  const int64_t tm = (Mrows + BG_M - 1) / BG_M, tn = N / BG_N, total = tm * tn;
  const int64_t whole = (total / kCUs) * kCUs;
  if (whole == 0 || whole == total) return (int)tn;
  const int64_t nb = whole / tm;                                  // big column tiles
  const int64_t small = ((Mrows + 127) / 128) * ((tn - nb) * 2);  // 128x128 tiles
  const int64_t cost_big = 2 * ((total + kCUs - 1) / kCUs);       // in half big-tile rounds
  const int64_t cost_split = 2 * ((tm * nb + kCUs - 1) / kCUs) + (small + kCUs - 1) / kCUs;
  return cost_split < cost_big ? (int)nb : (int)tn;
}

// K splits of the Eq 2 projection and the columns each covers. The width is
// a whole number of k tiles and the count is recomputed from it, so that
// splits * k_per_split >= K and no split is empty, whatever the sizes.
CtxSplit ctx_gemm_split(int dtype, int64_t M, int N, int K) {
  int64_t tiles, target;
  int bk;
  if (use_big_tiles(dtype, M, N)) {
    tiles = ((M + BG_M - 1) / BG_M) * (N / BG_N);
    target = 256;   // one 128 KiB-LDS workgroup per CU
    bk = kFuseBK;
  } else {
    const int bm = dtype == 1 ? pick_gemm_bm((int)std::max<int64_t>(M, 1)) : 64;
    const int bn = dtype == 1 ? 128 : 64;
    tiles = ((std::max<int64_t>(M, 1) + bm - 1) / bm) * (N / bn);
    target = 512;
    bk = dtype == 1 ? BK : 16;
  }
  int64_t sp = M <= 0 ? 1 : (target + tiles - 1) / tiles;
  const int64_t max_s = K / (4 * bk);
  if (sp > max_s) sp = max_s;
  if (sp < 1) sp = 1;
  const int64_t kps = ((K + sp * bk - 1) / (sp * bk)) * bk;   // ceil(K / sp), whole k tiles
  CtxSplit r;
  r.k_per_split = (int)kps;
  r.splits = (int)((K + kps - 1) / kps);
  r.fused = use_big_tiles(dtype, M, N) && r.splits == 1;
  r.tail_row = M;
  if (r.fused) {
    // Tiles beyond the last whole round of kCUs: if they would fill at most
    // half a round, their row tiles run as K splits of a few times as many
    // workgroups (each tile of Eq 2 lasts K / 64 k-steps, so an almost empty
    // last round costs a whole tile's time).
    const int64_t tn = N / BG_N, tm = (M + BG_M - 1) / BG_M;
    const int64_t rest = (tm * tn) % kCUs;   // a multiple of tn, since tn divides kCUs
    if (rest > 0 && 2 * rest <= kCUs) {
      int64_t ts = std::min<int64_t>(kCUs / rest, K / (4 * kFuseBK));
      if (ts >= 2) {
        const int64_t tkps = ((K + ts * kFuseBK - 1) / (ts * kFuseBK)) * kFuseBK;
        r.tail_splits = (int)((K + tkps - 1) / tkps);
        r.tail_kps = (int)tkps;
        r.tail_row = (tm - rest / tn) * BG_M;
      }
    }
  }
  return r;
}

hipError_t launch_gemm_ctx(int dtype, const ASegs& a, const BMats& b, const void* Bt, const CtxOut& o,
                           int M, int N, int K, const CtxSplit& sp, hipStream_t s) {
  const int splits = sp.splits, kps = sp.k_per_split;
  if ((int64_t)splits * kps < K || (int64_t)(splits - 1) * kps >= K) return hipErrorInvalidValue;
  if (sp.fused != (use_big_tiles(dtype, M, N) && splits == 1)) return hipErrorInvalidValue;
  float* out = o.part;
  trace_pre(K_GEMM_CTX, s);
  if (sp.fused) {
    const int M1 = (int)sp.tail_row;
    if (M1 < M && (!o.tail_part || sp.tail_splits < 2 || M1 % BG_M != 0)) return hipErrorInvalidValue;
    EpiNormBig epi{static_cast<bf16*>(o.y), o.sums, o.g};
    dim3 grid(((M1 + BG_M - 1) / BG_M) * (N / BG_N), 1, 1);
    gemm_big_kernel<EpiNormBig, 128, kFuseBK, 4, kBigWaves><<<grid, 64 * kBigWaves, 0, s>>>(
        a, static_cast<const bf16*>(Bt), M1, M1, N, K, kps, epi);
    if (M1 < M) {   // the tail rows as K splits, float32 partials
      ASegs at = a;
      for (int j = 0; j < a.nseg; ++j) at.seg[j] = static_cast<const bf16*>(a.seg[j]) + (int64_t)M1 * a.ld;
      EpiPartialBig pe{o.tail_part, (int64_t)(M - M1) * N};
      dim3 tg(((M - M1 + BG_M - 1) / BG_M) * (N / BG_N), sp.tail_splits, 1);
      gemm_big_kernel<EpiPartialBig, 128, kFuseBK, 4, kBigWaves><<<tg, 64 * kBigWaves, 0, s>>>(
          at, static_cast<const bf16*>(Bt), M - M1, M - M1, N, K, sp.tail_kps, pe);
    }
  } else if (use_big_tiles(dtype, M, N)) {
    EpiPartialBig epi{out, (int64_t)M * N};
    dim3 grid(((M + BG_M - 1) / BG_M) * (N / BG_N), splits, 1);
    gemm_big_kernel<EpiPartialBig, 128, kFuseBK, 4, kBigWaves><<<grid, 64 * kBigWaves, 0, s>>>(a, static_cast<const bf16*>(Bt),
                                                                         M, M, N, K, kps, epi);
  } else if (dtype == 1) {
    EpiPartial epi{out, (int64_t)M * N};
    const bf16* B = static_cast<const bf16*>(Bt);
    if (pick_gemm_bm(M) == 128) {
      dim3 grid(((M + 127) / 128) * (N / 128), 1, splits);
      gemm_bf16_nt<128, 128, 2, 2, EpiPartial><<<grid, 256, 0, s>>>(a, B, M, M, N, K, kps, epi);
    } else {
      dim3 grid(((M + 63) / 64) * (N / 128), 1, splits);
      gemm_bf16_nt<64, 128, 2, 2, EpiPartial><<<grid, 256, 0, s>>>(a, B, M, M, N, K, kps, epi);
    }
  } else {
    EpiPartial epi{out, (int64_t)M * N};
    dim3 grid(((M + 63) / 64) * (N / 64), 1, splits);
    gemm_f32<EpiPartial><<<grid, 256, 0, s>>>(a, b, M, M, N, K, kps, epi);
  }
  trace_post(K_GEMM_CTX, s);
  return hipGetLastError();
}

hipError_t launch_gemm_kv(int dtype, const void* h_ctx, const BMats& b, const void* Bt,
                          const float* rinv, const KVDesc& kv, int d, int kvd, int n_layers,
                          hipStream_t s) {
  ASegs a{};
  a.seg[0] = h_ctx;
  a.ld = d;
  a.seg_k = d;
  a.nseg = 1;
  // the epilogues decode a column as (layer, K or V, head, value) with kvd
  // columns per K or V block
  const int N = 2 * n_layers * kvd;
  const int M = kv.T;
  // packed: rows T..Tpad-1 are written as zeros; cache: only the T new rows
  const int Mrows = kv.dst_row ? M : (int)kv.Tpad;
  trace_pre(K_GEMM_KV, s);
  if (use_big_tiles(dtype, M, N)) {
    const bf16* B = static_cast<const bf16*>(Bt);
    const int nb = kv_big_columns(Mrows, N);
    EpiKVBig<bf16> epi{static_cast<bf16*>(kv.base), rinv, kv.Tpad, kv.T, kvd, kv.hd, kv.n_heads, 0,
                       kv.dst_row};
    const int tm = (Mrows + BG_M - 1) / BG_M;
    // 256x256 tiles only, one persistent workgroup per CU; its packed-target
    // stores take 32-bit byte offsets inside a head slab of Tpad * hd elements
    const bool slab32 = kv.dst_row || (uint64_t)kv.Tpad * kv.hd * 2 < ((uint64_t)1 << 32);
    if (nb * BG_N == N && !slab32) {
      dim3 grid(tm * (N / BG_N), 1, 1);
      if (kv.hd == 128)
        gemm_big_kernel<EpiKVBig<bf16>, 128, kKvBK, 4, kBigWaves><<<grid, 64 * kBigWaves, 0, s>>>(a, B, M, Mrows, N, d, d, epi);
      else if (kv.hd == 64)
        gemm_big_kernel<EpiKVBig<bf16>, 64, kKvBK, 4, kBigWaves><<<grid, 64 * kBigWaves, 0, s>>>(a, B, M, Mrows, N, d, d, epi);
      else
        gemm_big_kernel<EpiKVBig<bf16>, 32, kKvBK, 4, kBigWaves><<<grid, 64 * kBigWaves, 0, s>>>(a, B, M, Mrows, N, d, d, epi);
    } else if (nb * BG_N == N) {
      dim3 grid((unsigned)std::min<int64_t>((int64_t)tm * (N / BG_N), kCUs), 1, 1);
      if (kv.hd == 128)
        gemm_kv_persistent_kernel<EpiKVBig<bf16>, 128, kKvBK, kBigWaves><<<grid, 64 * kBigWaves, 0, s>>>(a, B, M, Mrows, N, d, epi);
      else if (kv.hd == 64)
        gemm_kv_persistent_kernel<EpiKVBig<bf16>, 64, kKvBK, kBigWaves><<<grid, 64 * kBigWaves, 0, s>>>(a, B, M, Mrows, N, d, epi);
      else
        gemm_kv_persistent_kernel<EpiKVBig<bf16>, 32, kKvBK, kBigWaves><<<grid, 64 * kBigWaves, 0, s>>>(a, B, M, Mrows, N, d, epi);
    } else {                // columns [0, nb * 256) in 256x256 tiles, the rest in 128x128 tiles
      const int Nb = nb * BG_N, nbig = tm * nb;
      const int nsmall = ((Mrows + 127) / 128) * ((N - Nb) / 128);
      dim3 grid(nbig + nsmall, 1, 1);
      if (kv.hd == 128)
        gemm_kv_tail_kernel<EpiKVBig<bf16>, 128, kKvBK, kBigWaves><<<grid, 64 * kBigWaves, 0, s>>>(a, B, M, Mrows, N, d, Nb, nbig,
                                                                               epi);
      else if (kv.hd == 64)
        gemm_kv_tail_kernel<EpiKVBig<bf16>, 64, kKvBK, kBigWaves><<<grid, 64 * kBigWaves, 0, s>>>(a, B, M, Mrows, N, d, Nb, nbig,
                                                                               epi);
      else
        gemm_kv_tail_kernel<EpiKVBig<bf16>, 32, kKvBK, kBigWaves><<<grid, 64 * kBigWaves, 0, s>>>(a, B, M, Mrows, N, d, Nb, nbig,
                                                                               epi);
    }
  } else if (dtype == 1) {
    EpiKV<bf16> epi{static_cast<bf16*>(kv.base), rinv, kv.Tpad, kv.T, kvd, kv.hd, kv.n_heads, kv.dst_row};
    const bf16* B = static_cast<const bf16*>(Bt);
    if (pick_gemm_bm(M) == 128) {
      dim3 grid(((Mrows + 127) / 128) * (N / 128), 1, 1);
      gemm_bf16_nt<128, 128, 2, 2, EpiKV<bf16>><<<grid, 256, 0, s>>>(a, B, M, Mrows, N, d, d, epi);
    } else {
      dim3 grid(((Mrows + 63) / 64) * (N / 128), 1, 1);
      gemm_bf16_nt<64, 128, 2, 2, EpiKV<bf16>><<<grid, 256, 0, s>>>(a, B, M, Mrows, N, d, d, epi);
    }
  } else {
    EpiKV<float> epi{static_cast<float*>(kv.base), rinv, kv.Tpad, kv.T, kvd, kv.hd, kv.n_heads, kv.dst_row};
    dim3 grid(((Mrows + 63) / 64) * (N / 64), 1, 1);
    gemm_f32<EpiKV<float>><<<grid, 256, 0, s>>>(a, b, M, Mrows, N, d, d, epi);
  }
  trace_post(K_GEMM_KV, s);
  return hipGetLastError();
}

}  // namespace dspark
