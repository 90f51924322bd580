// The Markov head, the confidence head and the greedy draft loop after the
// backbone (module-dflash.ts: #markov, #confidence, forwardInfer; the page
// "src/dspark-runtime.js" runs the same steps as markovEmbed -> markov ->
// addBias -> argmax for each drafted position).
//
// For every sequence b, starting from its anchor token, position k of the
// block takes
//   e1       = w1[prev]                       (the previous token's Markov embedding)
//   logits_k = base_logits[b, k] + e1 . w2^T  (w2 stored [vocab, rank])
//   token_k  = argmax logits_k                (the lowest index among equal maxima)
//   conf_k   = sigmoid([block[b, k], e1] . conf_w + conf_b)
// and prev = token_k. The positions depend on each other through the token,
// so the loop runs position by position, all sequences together. A position
// is two launches:
//   the logits, which stream all of w2 once: with bf16 weights and a rank up
//   to 512, markov_logits_kernel multiplies on the matrix cores and also
//   reduces its vocabulary chunk to (max, index) partials; otherwise the
//   weight-streaming row GEMM of block.hip (the base logits as its residual)
//   followed by markov_argmax_kernel;
//   markov_final_kernel, which picks the token from the partials, computes
//   the confidence and gathers the next position's embedding rows.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace dspark {

// Larger value wins; on equal values the lower index (numpy's argmax rule).
DSPARK_DEV void arg_better(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

DSPARK_DEV void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float v2 = __shfl_xor(v, off, kWave);
    const int i2 = __shfl_xor(i, off, kWave);
    arg_better(v, i, v2, i2);
  }
}

// E1[b] = w1[clamp(tok[b])] as float32; one workgroup per sequence.
template <typename S>
__global__ __launch_bounds__(256) void markov_embed_kernel(const S* __restrict__ w1, int vocab, int rank,
                                                           const int32_t* __restrict__ tok,
                                                           float* __restrict__ E1) {
  const int b = blockIdx.x;
  const int t = min(max(tok[b], 0), vocab - 1);
  for (int i = threadIdx.x; i < rank; i += 256) E1[(int64_t)b * rank + i] = to_f32(w1[(int64_t)t * rank + i]);
}

// Partials of one position: grid (P, A); workgroup (p, b) scans vocabulary
// entries [p * chunk, min(vocab, (p+1) * chunk)) of row b of the logits
// (row stride ld) and writes its best (value, index).
__global__ __launch_bounds__(256) void markov_argmax_kernel(const float* __restrict__ logits, int64_t ld,
                                                            int vocab, int chunk, float* __restrict__ pv,
                                                            int32_t* __restrict__ pi) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int p = blockIdx.x, b = blockIdx.y, P = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* row = logits + (int64_t)b * ld;
  const int v0 = p * chunk, v1 = min(vocab, v0 + chunk);
  float best = -__builtin_inff();
  int bi = vocab;
  for (int v = v0 + tid; v < v1; v += 256) arg_better(best, bi, row[v], v);
  wave_argmax(best, bi);
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) arg_better(best, bi, sv[w], si[w]);
    pv[(int64_t)b * P + p] = best;
    pi[(int64_t)b * P + p] = bi;
  }
}

// One workgroup per sequence: the token of position k from the P partials,
// the confidence of position k (with the embedding rows the position used),
// and the next position's embedding rows E1[b] = w1[token]. The loops have
// independent loads, unrolled so that a thread's loads are all in flight
// together.
template <typename S>
__global__ __launch_bounds__(256) void markov_final_kernel(
    const float* __restrict__ pv, const int32_t* __restrict__ pi, int P, int k, int gamma, int d, int vocab,
    int rank, const float* __restrict__ block, const float* __restrict__ conf_w, const float* __restrict__ conf_b,
    const S* __restrict__ w1, float* __restrict__ E1, int32_t* __restrict__ tokens, float* __restrict__ conf) {
  __shared__ float sv[4], sz[4];
  __shared__ int si[4];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float best = -__builtin_inff();
  int bi = vocab;
#pragma unroll 8
  for (int q = tid; q < P; q += 256) arg_better(best, bi, pv[(int64_t)b * P + q], pi[(int64_t)b * P + q]);
  const float* brow = block + ((int64_t)b * gamma + k) * d;
  float* e = E1 + (int64_t)b * rank;
  float z = 0.f;
#pragma unroll 8
  for (int i = tid; i < d; i += 256) z = fmaf(brow[i], conf_w[i], z);
#pragma unroll 4
  for (int i = tid; i < rank; i += 256) z = fmaf(e[i], conf_w[d + i], z);
  wave_argmax(best, bi);
  z = wave_sum(z);
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bi;
    sz[wave] = z;
  }
  __syncthreads();   // also orders every thread's reads of e before the writes below
  best = sv[0];
  bi = si[0];
  for (int w = 1; w < 4; ++w) arg_better(best, bi, sv[w], si[w]);
  const int tok = min(max(bi, 0), vocab - 1);
  if (tid == 0) {
    z = (sz[0] + sz[1]) + (sz[2] + sz[3]) + conf_b[0];
    tokens[(int64_t)b * gamma + k] = tok;
    conf[(int64_t)b * gamma + k] = 1.f / (1.f + expf(-z));
  }
#pragma unroll 4
  for (int i = tid; i < rank; i += 256) e[i] = to_f32(w1[(int64_t)tok * rank + i]);
}

// ---------------------------------------------------------------------------
// Logits and argmax partials of one position on v_mfma_f32_16x16x32_bf16.
// The A operand is 16 vocabulary rows of w2 (lane l: row l % 16, ranks
// 8 (l / 16) + 32 s .. + 8), the B operand the embeddings of 16 sequences
// (lane l: sequence l % 16, the same ranks). The embeddings are rows of the
// bf16 w1 held in float32, so their bf16 form is exact; the products are
// exact and the sums float32. The result D[4 (l / 16) + r][l % 16] is the
// logit of vocabulary row 4 (l / 16) + r for sequence l % 16: a lane holds
// four consecutive logits of one sequence, stored as one 16-byte vector.
// Grid (P, ceil(A / 16)): workgroup p owns vocabulary rows
// [p * chunk, min(vocab, (p + 1) * chunk)) for 16 sequences, so w2 is read
// once per 16 sequences. Its four waves take 16-row groups in batches of G,
// with all of a batch's weight loads in flight before the first product.
// ---------------------------------------------------------------------------
struct MarkovStep {
  const bf16* w2 = nullptr;       // [vocab][rank]
  const float* E1 = nullptr;      // [A][rank]
  const float* base = nullptr;    // base_logits + k * vocab, row stride ld
  float* logits = nullptr;        // draft logits + k * vocab, row stride ld
  float* pv = nullptr;            // [A][P]
  int32_t* pi = nullptr;
  int64_t ld = 0;
  int A = 0, vocab = 0, rank = 0, chunk = 0;
};

template <int KS> constexpr int markov_groups() { return KS <= 4 ? 4 : KS <= 8 ? 2 : 1; }

template <int KS>
__global__ __launch_bounds__(256) void markov_logits_kernel(MarkovStep a) {
  constexpr int G = markov_groups<KS>();
  __shared__ float sv[4][16];
  __shared__ int si[4][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, kg = lane >> 4;
  const int p = blockIdx.x, P = gridDim.x;
  const int b = blockIdx.y * 16 + c16;
  const bool bok = b < a.A;
  const int v_begin = p * a.chunk, v_end = min(a.vocab, v_begin + a.chunk);
  const int ng = (v_end - v_begin + 15) >> 4;    // 16-row groups of this chunk

  bf16x8 eb[KS];
  {
    const float* er = a.E1 + (int64_t)min(b, a.A - 1) * a.rank + 8 * kg;   // sequences past A: unused
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(er + 32 * s);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(er + 32 * s + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        eb[s][e] = from_f32<bf16>(x0[e]);
        eb[s][e + 4] = from_f32<bf16>(x1[e]);
      }
    }
  }
  const float* brow = a.base + (int64_t)min(b, a.A - 1) * a.ld;
  float* lrow = a.logits + (int64_t)min(b, a.A - 1) * a.ld;

  float best = -__builtin_inff();
  int bi = a.vocab;
  for (int g0 = wave * G; g0 < ng; g0 += 4 * G) {
    bf16x8 wv[G][KS];
    f32x4 bl[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int row = min(v_begin + (g0 + g) * 16 + c16, a.vocab - 1);   // past the chunk: a valid row, unused
      const bf16* wr = a.w2 + (int64_t)row * a.rank + 8 * kg;
#pragma unroll
      for (int s = 0; s < KS; ++s) wv[g][s] = *reinterpret_cast<const bf16x8*>(wr + 32 * s);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int vo = v_begin + (g0 + g) * 16 + 4 * kg;   // v_end % 4 == 0: all four or none in range
      bl[g] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (bok && g0 + g < ng && vo < v_end) bl[g] = *reinterpret_cast<const f32x4*>(brow + vo);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[g][s], eb[s], acc, 0, 0, 0);
      const int vo = v_begin + (g0 + g) * 16 + 4 * kg;
      if (g0 + g < ng && vo < v_end) {
        const f32x4 lg = acc + bl[g];
        if (bok) *reinterpret_cast<f32x4*>(lrow + vo) = lg;
#pragma unroll
        for (int r = 0; r < 4; ++r) arg_better(best, bi, lg[r], vo + r);
      }
    }
  }
  // lanes l, l + 16, l + 32, l + 48 hold the same sequence
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) {
    const float v2 = __shfl_xor(best, off, kWave);
    const int i2 = __shfl_xor(bi, off, kWave);
    arg_better(best, bi, v2, i2);
  }
  if (kg == 0) {
    sv[wave][c16] = best;
    si[wave][c16] = bi;
  }
  __syncthreads();
  if (wave == 0 && kg == 0) {
    for (int w = 1; w < 4; ++w) arg_better(best, bi, sv[w][c16], si[w][c16]);
    if (bok) {
      a.pv[(int64_t)b * P + p] = best;
      a.pi[(int64_t)b * P + p] = bi;
    }
  }
}

static bool markov_mfma(int dtype, int rank) { return dtype == 1 && rank % 64 == 0 && rank <= 512; }

static int markov_rows_per_wg(int dtype, int rank) {
  if (!markov_mfma(dtype, rank)) return 2048;
  const int ks = rank / 32;
  const int G = ks <= 4 ? 4 : ks <= 8 ? 2 : 1;
  return 64 * G;
}

MarkovGrid markov_grid(int dtype, int vocab, int rank) {
  // one chunk per workgroup; at most 2048 chunks (the partials per sequence)
  const int64_t unit = markov_rows_per_wg(dtype, rank);
  const int64_t need = (vocab + 2047) / 2048;
  const int64_t chunk = std::max(unit, (need + unit - 1) / unit * unit);
  MarkovGrid g;
  g.chunk = (int)chunk;
  g.P = (int)((vocab + chunk - 1) / chunk);
  g.mfma = markov_mfma(dtype, rank);
  return g;
}

hipError_t launch_markov(int dtype, const MarkovArgs& a, hipStream_t s) {
  const MarkovGrid mg = markov_grid(dtype, a.vocab, a.rank);
  const int P = mg.P;
  trace_pre(K_MARKOV, s);
  if (dtype == 1)
    markov_embed_kernel<bf16><<<a.A, 256, 0, s>>>(static_cast<const bf16*>(a.w1), a.vocab, a.rank, a.anchor, a.E1);
  else
    markov_embed_kernel<float><<<a.A, 256, 0, s>>>(static_cast<const float*>(a.w1), a.vocab, a.rank, a.anchor,
                                                   a.E1);
  trace_post(K_MARKOV, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ld = (int64_t)a.gamma * a.vocab;
  for (int k = 0; k < a.gamma; ++k) {
    if (mg.mfma) {
      // logits_k = base_logits[:, k] + E1 . w2^T into draft_logits[:, k], and the partials
      MarkovStep st;
      st.w2 = static_cast<const bf16*>(a.w2);
      st.E1 = a.E1;
      st.base = a.base_logits + (int64_t)k * a.vocab;
      st.logits = a.logits + (int64_t)k * a.vocab;
      st.pv = a.part_v;
      st.pi = a.part_i;
      st.ld = ld;
      st.A = a.A;
      st.vocab = a.vocab;
      st.rank = a.rank;
      st.chunk = mg.chunk;
      const dim3 grid(P, (a.A + 15) / 16);
      trace_pre(K_MARKOV, s);
      switch (a.rank / 32) {
#define DSPARK_MK(KS) \
        case KS: markov_logits_kernel<KS><<<grid, 256, 0, s>>>(st); break;
        DSPARK_MK(2) DSPARK_MK(4) DSPARK_MK(6) DSPARK_MK(8) DSPARK_MK(10) DSPARK_MK(12) DSPARK_MK(14) DSPARK_MK(16)
#undef DSPARK_MK
        default: return hipErrorInvalidValue;
      }
    } else {
      // logits_k = base_logits[:, k] + E1 . w2^T, into draft_logits[:, k]
      RowGemmArgs r{};
      r.X = a.E1;
      r.ldx = a.rank;
      r.M = a.A;
      r.K = a.rank;
      r.N = a.vocab;
      r.b.mat[0] = a.w2;
      r.b.n_per = a.vocab;
      r.b.nmat = 1;
      r.res = a.base_logits + (int64_t)k * a.vocab;
      r.out = a.logits + (int64_t)k * a.vocab;
      r.ldo = (int)ld;   // gamma * vocab < 2^31 (checked on the host)
      e = launch_rowgemm(dtype, RP_NONE, RE_RESID, r, s);
      if (e != hipSuccess) return e;
      trace_pre(K_MARKOV, s);
      markov_argmax_kernel<<<dim3(P, a.A), 256, 0, s>>>(a.logits + (int64_t)k * a.vocab, ld, a.vocab, mg.chunk,
                                                       a.part_v, a.part_i);
    }
    if (dtype == 1)
      markov_final_kernel<bf16><<<a.A, 256, 0, s>>>(a.part_v, a.part_i, P, k, a.gamma, a.d, a.vocab, a.rank,
                                                   a.block, a.conf_w, a.conf_b,
                                                   static_cast<const bf16*>(a.w1), a.E1, a.tokens, a.conf);
    else
      markov_final_kernel<float><<<a.A, 256, 0, s>>>(a.part_v, a.part_i, P, k, a.gamma, a.d, a.vocab, a.rank,
                                                    a.block, a.conf_w, a.conf_b,
                                                    static_cast<const float*>(a.w1), a.E1, a.tokens, a.conf);
    trace_post(K_MARKOV, s);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dspark
