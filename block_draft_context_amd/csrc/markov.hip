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
// so the loop runs position by position, all sequences together.
// With bf16 weights and a rank up to 512 a position is one launch,
// markov_step_kernel: every workgroup first reduces the previous position's
// (max, index) partials of its sequences to their tokens (the anchors at
// position 0); all but one then gather those tokens' rows of w1 and stream
// w2 once on the matrix cores, writing the draft logits and their own
// vocabulary chunk's partials, while the last writes the tokens and the
// position's confidences. markov_last_kernel turns the last position's
// partials into its tokens. Otherwise (float32, larger ranks) a position is the weight-
// streaming row GEMM of block.hip (the base logits as its residual),
// markov_argmax_kernel and markov_final_kernel (token, confidence, next
// embedding rows), after markov_embed_kernel.
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
// One drafted position k on v_mfma_f32_16x16x32_bf16, grid (P + 1,
// ceil(A / 16)); column y serves sequences 16 y .. 16 y + 15.
// Workgroups p < P stream the vocabulary rows [p * chunk, min(vocab, (p + 1)
// * chunk)) of w2 for those 16 sequences, so w2 is read once per 16
// sequences. The A operand is 16 rows of w2 (lane l: row l % 16, ranks
// 8 (l / 16) + 32 s .. + 8), the B operand the Markov embeddings of the 16
// sequences (lane l: sequence l % 16, the same ranks), read straight from the
// bf16 w1 rows of their previous tokens; the products are exact and the sums
// float32. D[4 (l / 16) + r][l % 16] is the logit of row 4 (l / 16) + r for
// sequence l % 16: a lane holds four consecutive logits of one sequence,
// stored as one 16-byte vector. The four waves take 16-row groups in batches
// of G; a wave's first batch of weight loads is issued before the previous
// tokens are known, so its latency overlaps theirs. Each workgroup writes
// the (max, index) of its chunk per sequence.
// Workgroup p = P writes the tokens of position k-1 and the confidences of
// position k of the column's sequences and streams nothing.
// ---------------------------------------------------------------------------
struct MarkovStep {
  const bf16* w1 = nullptr;       // [vocab][rank]
  const bf16* w2 = nullptr;       // [vocab][rank]
  const int32_t* anchor = nullptr;   // position 0: the previous tokens
  const int2* prev = nullptr;     // position k > 0: position k-1's partials [A][P] (value bits, index)
  int2* part = nullptr;           // this position's partials [A][P]
  const float* base = nullptr;    // base_logits + k * vocab, row stride ld
  float* logits = nullptr;        // draft logits + k * vocab, row stride ld
  const float* block = nullptr;   // [A][gamma][d]
  const float* conf_w = nullptr;  // [d + rank]
  const float* conf_b = nullptr;  // [1]
  int32_t* tokens = nullptr;      // [A][gamma]
  float* conf = nullptr;          // [A][gamma]
  int64_t ld = 0;
  int A = 0, vocab = 0, rank = 0, chunk = 0, P = 0, k = 0, gamma = 0, d = 0;
};

template <int KS> constexpr int markov_groups() { return KS <= 4 ? 4 : KS <= 8 ? 2 : 1; }

DSPARK_DEV int clamp_token(int t, int vocab) { return min(max(t, 0), vocab - 1); }

// tok[j] = the previous token of sequence y0 + j (j < 16): its anchor at
// position 0, else the argmax over position k-1's P partials; token 0 past
// A. A column with n sequences gives each 256 / 2^ceil(log2 n) threads.
DSPARK_DEV void markov_prev_tokens(const MarkovStep& a, int y0, int* tok, int2* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = min(16, a.A - y0);
  if (a.k == 0) {
    if (tid < 16) tok[tid] = tid < n ? clamp_token(a.anchor[y0 + tid], a.vocab) : 0;
    __syncthreads();
    return;
  }
  const int lg = n <= 1 ? 0 : n <= 2 ? 1 : n <= 4 ? 2 : n <= 8 ? 3 : 4;
  const int tps = 256 >> lg, j = tid >> (8 - lg), q = tid & (tps - 1);
  float best = -__builtin_inff();
  int bi = a.vocab;
  if (j < n) {
    // 16 loads in flight per round; indices past P repeat the last pair,
    // which cannot change the result
    const int2* pp = a.prev + (int64_t)(y0 + j) * a.P;
    for (int i0 = q; i0 < a.P; i0 += 16 * tps) {
      int2 e[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) e[u] = pp[min(i0 + u * tps, a.P - 1)];
#pragma unroll
      for (int u = 0; u < 16; ++u) arg_better(best, bi, __int_as_float(e[u].x), e[u].y);
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    if (off < tps) {   // uniform
      const float v2 = __shfl_xor(best, off, kWave);
      const int i2 = __shfl_xor(bi, off, kWave);
      arg_better(best, bi, v2, i2);
    }
  }
  if (tps <= 64) {
    if (q == 0 && j < n) tok[j] = clamp_token(bi, a.vocab);
  } else {
    // a sequence spans tps / 64 waves
    if (lane == 0) red[wave] = make_int2(__float_as_int(best), bi);
    __syncthreads();
    if (tid < n) {
      const int wpj = tps >> 6;
      best = __int_as_float(red[tid * wpj].x);
      bi = red[tid * wpj].y;
      for (int w = 1; w < wpj; ++w) arg_better(best, bi, __int_as_float(red[tid * wpj + w].x), red[tid * wpj + w].y);
      tok[tid] = clamp_token(bi, a.vocab);
    }
  }
  if (tid >= n && tid < 16) tok[tid] = 0;
  __syncthreads();
}

// Workgroup P of a column: the tokens of position k-1 and the confidences
// sigmoid([block[b, k], w1[prev]] . conf_w + conf_b) of position k; wave w
// takes sequences w, w + 4, w + 8, w + 12.
DSPARK_DEV void markov_duty(const MarkovStep& a, int y0, int* tok, int2* red) {
  markov_prev_tokens(a, y0, tok, red);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = min(16, a.A - y0);
  if (a.k > 0 && tid < n) a.tokens[(int64_t)(y0 + tid) * a.gamma + a.k - 1] = tok[tid];
  for (int j = wave; j < n; j += 4) {
    const int b = y0 + j;
    const float* brow = a.block + ((int64_t)b * a.gamma + a.k) * a.d;
    const bf16* erow = a.w1 + (int64_t)tok[j] * a.rank;
    float z = 0.f;
#pragma unroll 4
    for (int i = 4 * lane; i < a.d; i += 256) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(brow + i);
      const f32x4 c = *reinterpret_cast<const f32x4*>(a.conf_w + i);
      z = fmaf(x[0], c[0], z);
      z = fmaf(x[1], c[1], z);
      z = fmaf(x[2], c[2], z);
      z = fmaf(x[3], c[3], z);
    }
#pragma unroll 4
    for (int i = lane; i < a.rank; i += 64) z = fmaf(static_cast<float>(erow[i]), a.conf_w[a.d + i], z);
    z = wave_sum(z);
    if (lane == 0) a.conf[(int64_t)b * a.gamma + a.k] = 1.f / (1.f + expf(-(z + a.conf_b[0])));
  }
}

template <int KS>
__global__ __launch_bounds__(256) void markov_step_kernel(MarkovStep a) {
  constexpr int G = markov_groups<KS>();
  __shared__ float sv[4][16];
  __shared__ int si[4][16];
  __shared__ int tok[16];
  __shared__ int2 red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, kg = lane >> 4;
  const int p = blockIdx.x;
  const int y0 = blockIdx.y * 16;
  if (p == a.P) {   // uniform
    markov_duty(a, y0, tok, red);
    return;
  }
  const int b = y0 + c16;
  const bool bok = b < a.A;
  const int v_begin = p * a.chunk, v_end = min(a.vocab, v_begin + a.chunk);
  const int ng = (v_end - v_begin + 15) >> 4;    // 16-row groups of this chunk
  const float* brow = a.base + (int64_t)min(b, a.A - 1) * a.ld;
  float* lrow = a.logits + (int64_t)min(b, a.A - 1) * a.ld;

  // Loads past the chunk (or of sequences past A) read valid addresses and
  // their results are never stored: the weight row is clamped to the last
  // one and the logit offset to the chunk's last four (v_end % 4 == 0).
  bf16x8 wv[G][KS];
  f32x4 bl[G];
  auto load_w = [&](int g0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int row = min(v_begin + (g0 + g) * 16 + c16, a.vocab - 1);
      const bf16* wr = a.w2 + (int64_t)row * a.rank + 8 * kg;
#pragma unroll
      for (int s = 0; s < KS; ++s) wv[g][s] = *reinterpret_cast<const bf16x8*>(wr + 32 * s);
    }
  };
  auto load_base = [&](int g0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      bl[g] = *reinterpret_cast<const f32x4*>(brow + min(v_begin + (g0 + g) * 16 + 4 * kg, v_end - 4));
  };
  load_w(wave * G);
  markov_prev_tokens(a, y0, tok, red);
  bf16x8 eb[KS];
  {
    const bf16* er = a.w1 + (int64_t)tok[c16] * a.rank + 8 * kg;
#pragma unroll
    for (int s = 0; s < KS; ++s) eb[s] = *reinterpret_cast<const bf16x8*>(er + 32 * s);
  }
  load_base(wave * G);

  float best = -__builtin_inff();
  int bi = a.vocab;
  for (int g0 = wave * G; g0 < ng; g0 += 4 * G) {
    if (g0 != wave * G) {
      load_w(g0);
      load_base(g0);
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
    if (bok) a.part[(int64_t)b * a.P + p] = make_int2(__float_as_int(best), bi);
  }
}

// The last position's tokens from its partials; one workgroup per sequence.
__global__ __launch_bounds__(256) void markov_last_kernel(const int2* __restrict__ part, int P, int k, int gamma,
                                                          int vocab, int32_t* __restrict__ tokens) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float best = -__builtin_inff();
  int bi = vocab;
#pragma unroll 8
  for (int q = tid; q < P; q += 256) {
    const int2 e = part[(int64_t)b * P + q];
    arg_better(best, bi, __int_as_float(e.x), e.y);
  }
  wave_argmax(best, bi);
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) arg_better(best, bi, sv[w], si[w]);
    tokens[(int64_t)b * gamma + k] = clamp_token(bi, vocab);
  }
}

static bool markov_mfma(int dtype, int rank) { return dtype == 1 && rank % 64 == 0 && rank <= 512; }

// Vocabulary rows per workgroup. The matrix-core step kernel's workgroups
// each read the previous position's partials of up to 16 sequences, so with
// more sequences they take longer chunks (fewer partials).
static int markov_rows_per_wg(int dtype, int rank, int A) {
  if (!markov_mfma(dtype, rank)) return 2048;
  const int ks = rank / 32;
  const int G = ks <= 4 ? 4 : ks <= 8 ? 2 : 1;
  const int seqs = std::min(A, 16);
  return 64 * G * (seqs <= 2 ? 1 : seqs <= 8 ? 2 : 4);
}

MarkovGrid markov_grid(int dtype, int vocab, int rank, int A) {
  // one chunk per workgroup; at most 2048 chunks (the partials per sequence)
  const int64_t unit = markov_rows_per_wg(dtype, rank, A);
  const int64_t need = (vocab + 2047) / 2048;
  const int64_t chunk = std::max(unit, (need + unit - 1) / unit * unit);
  MarkovGrid g;
  g.chunk = (int)chunk;
  g.P = (int)((vocab + chunk - 1) / chunk);
  g.mfma = markov_mfma(dtype, rank);
  return g;
}

hipError_t launch_markov(int dtype, const MarkovArgs& a, hipStream_t s) {
  const MarkovGrid mg = markov_grid(dtype, a.vocab, a.rank, a.A);
  const int P = mg.P;
  const int64_t ld = (int64_t)a.gamma * a.vocab;
  const int64_t pstride = (int64_t)a.A * P;   // one position's partials; two buffers, by parity
  hipError_t e = hipSuccess;
  if (mg.mfma) {
    int2* part = reinterpret_cast<int2*>(a.part_v);   // [2][A][P] pairs, alternating by position
    for (int k = 0; k < a.gamma; ++k) {
      MarkovStep st;
      st.w1 = static_cast<const bf16*>(a.w1);
      st.w2 = static_cast<const bf16*>(a.w2);
      st.anchor = a.anchor;
      st.prev = part + (int64_t)((k + 1) & 1) * pstride;
      st.part = part + (int64_t)(k & 1) * pstride;
      st.base = a.base_logits + (int64_t)k * a.vocab;
      st.logits = a.logits + (int64_t)k * a.vocab;
      st.block = a.block;
      st.conf_w = a.conf_w;
      st.conf_b = a.conf_b;
      st.tokens = a.tokens;
      st.conf = a.conf;
      st.ld = ld;
      st.A = a.A;
      st.vocab = a.vocab;
      st.rank = a.rank;
      st.chunk = mg.chunk;
      st.P = P;
      st.k = k;
      st.gamma = a.gamma;
      st.d = a.d;
      const dim3 grid(P + 1, (a.A + 15) / 16);
      trace_pre(K_MARKOV, s);
      switch (a.rank / 32) {
#define DSPARK_MK(KS) \
        case KS: markov_step_kernel<KS><<<grid, 256, 0, s>>>(st); break;
        DSPARK_MK(2) DSPARK_MK(4) DSPARK_MK(6) DSPARK_MK(8) DSPARK_MK(10) DSPARK_MK(12) DSPARK_MK(14) DSPARK_MK(16)
#undef DSPARK_MK
        default: return hipErrorInvalidValue;
      }
      trace_post(K_MARKOV, s);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const int kl = a.gamma - 1;
    trace_pre(K_MARKOV, s);
    markov_last_kernel<<<a.A, 256, 0, s>>>(part + (int64_t)(kl & 1) * pstride, P, kl, a.gamma, a.vocab, a.tokens);
    trace_post(K_MARKOV, s);
    return hipGetLastError();
  }
  trace_pre(K_MARKOV, s);
  if (dtype == 1)
    markov_embed_kernel<bf16><<<a.A, 256, 0, s>>>(static_cast<const bf16*>(a.w1), a.vocab, a.rank, a.anchor, a.E1);
  else
    markov_embed_kernel<float><<<a.A, 256, 0, s>>>(static_cast<const float*>(a.w1), a.vocab, a.rank, a.anchor,
                                                   a.E1);
  trace_post(K_MARKOV, s);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int k = 0; k < a.gamma; ++k) {
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
