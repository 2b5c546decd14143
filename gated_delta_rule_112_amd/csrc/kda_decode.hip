// KDA single-token decode step: one pass over the resident float32 state.
//
// Per (b, h), with a = exp(g) (per key channel):
//   p_j = sum_i a_i k_i S_ij        (what the decayed state predicts for k)
//   r_j = sum_i a_i q_i S_ij        (decayed state read by q)
//   u_j = beta (v_j - p_j)
//   o_j = scale (r_j + (q . k) u_j)                  = scale * S_new^T q
//   S_ij <- a_i S_ij + k_i u_j                       (in place)
// "Kimi K3 Architecture Explained ...", section "Token mixing": constant
// per-token decode cost against a fixed-size state.
//
// The kernel is bound by HBM: every state element is read once and written
// once (8 bytes per element per step).  A workgroup holds a float4 column
// strip of RPT rows per thread in registers between the read and the in-place
// write, so the write never re-reads memory.  One workgroup of 1024 threads
// per (b, h) (four float4 per thread, two workgroups per compute unit):
// measured on MI355X at B = 256, H = 96 this streams 2-4 % faster than a
// persistent grid of one 256-thread workgroup per compute unit with the next
// state loading into a second register set (0.577-0.581 against
// 0.589-0.605 ms per step on one box), and than 256 or 512 threads per state;
// loading the token's vectors in the first 128 threads only (the others never
// use them) then took it to 0.566-0.571 ms.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// W: the most threads per workgroup.
template <int DK, int DV, int W = 256>
struct DecodeShape {
  static constexpr int CG = DV / 4;                                   // float4 column groups
  static constexpr int RG = (DK < W / CG) ? DK : W / CG;              // row groups
  static constexpr int RPT = DK / RG;                                 // rows per thread
  static constexpr int NT = CG * RG;                                  // threads per block
  static_assert(NT <= W && NT <= 1024 && NT % 64 == 0, "decode block must be whole wavefronts");
  static_assert(RPT * RG == DK, "rows must split evenly");
  static_assert(NT >= DK && NT >= DV, "one thread per key channel and per value column");
};

// One token's per-channel inputs for this thread (key channel tid % DK, value
// column tid % DV).
struct DecodeTok {
  float q, k, g, v, gate, beta;
};

// One (b, h): its state strip and the per-token vectors of its next token.
template <int DK, int DV, int W = 256>
struct DecodeTile {
  f32x4 s[DecodeShape<DK, DV, W>::RPT];
  DecodeTok x;
};

// Token inputs of row `row` (the (b, [t,] h) index of q, k, g [.., dk], v, gate
// [.., dv] and beta [..]).
template <int DK, int DV, typename IO>
__device__ __forceinline__ DecodeTok decode_load_tok(const IO* __restrict__ q,
                                                     const IO* __restrict__ k,
                                                     const IO* __restrict__ v,
                                                     const float* __restrict__ g,
                                                     const float* __restrict__ beta,
                                                     const IO* __restrict__ gate, int64_t row,
                                                     const IO* __restrict__ ga) {
  const int tid = threadIdx.x;
  const int ci = tid % DK, cj = tid % DV;
  DecodeTok x{};
  // only the threads of a key channel or a value column use these (the first
  // max(dk, dv)); the others load nothing (wave-uniform when dk, dv >= 64)
  if (tid >= (DK > DV ? DK : DV)) return x;
  x.q = ld_f32(q + row * DK + ci);
  x.k = ld_f32(k + row * DK + ci);
  x.v = ld_f32(v + row * DV + cj);
  x.gate = gate ? ld_f32(gate + row * DV + cj) : 0.f;
  if (ga != nullptr) {  // from logits: g = -5 sigmoid(a), beta = sigmoid(b)
    x.g = -5.f * sigmoidf_(ld_f32(ga + row * DK + ci));
    x.beta = sigmoidf_(beta[row]);
  } else {
    x.g = g[row * DK + ci];
    x.beta = beta[row];
  }
  return x;
}

// The state strip of (b, h) = bh and the inputs of token row `row`.
template <int DK, int DV, typename IO, int W = 256>
__device__ __forceinline__ void decode_load(DecodeTile<DK, DV, W>& t, const IO* __restrict__ q,
                                            const IO* __restrict__ k, const IO* __restrict__ v,
                                            const float* __restrict__ g,
                                            const float* __restrict__ beta,
                                            const float* __restrict__ state,
                                            const IO* __restrict__ gate, int64_t bh,
                                            int64_t row, const IO* __restrict__ ga) {
  using Sh = DecodeShape<DK, DV, W>;
  const int tid = threadIdx.x;
  const int cg = tid % Sh::CG, rg = tid / Sh::CG;
  const float* Sp = state + bh * (int64_t)(DK * DV);
#pragma unroll
  for (int m = 0; m < Sh::RPT; ++m)
    t.s[m] = __builtin_nontemporal_load((const f32x4*)(Sp + (rg + m * Sh::RG) * DV + 4 * cg));
  t.x = decode_load_tok<DK, DV, IO>(q, k, v, g, beta, gate, row, ga);
}

template <int DK, int DV, int W = 256>
struct DecodeSmem {
  using Sh = DecodeShape<DK, DV, W>;
  float a[DK];         // a_i = exp(g_i)
  float kk[DK];        // k_i
  float ak[DK];        // a_i * k_i
  float aq[DK];        // a_i * q_i
  float part[2][Sh::RG][DV];
  float u[DV];
  float red[Sh::NT];   // q_i k_i, then o_j^2
  float red2[Sh::NT];  // k_i^2 (with q_i^2 in red) when q and k are normalised here
  float qk, ss, nq, nk;
};

// One token against the state strip s.  The updated state is stored to Sp
// (the state of (b, h); NULL: not stored) and, with KEEP, kept in s for the
// next token; the output row goes to orow (NULL: none).
template <int DK, int DV, typename IO, bool KEEP, int W = 256>
__device__ __forceinline__ void decode_one(DecodeSmem<DK, DV, W>& sm,
                                           f32x4 (&s)[DecodeShape<DK, DV, W>::RPT],
                                           const DecodeTok& tin, float* __restrict__ Sp,
                                           IO* __restrict__ orow, bool gated, float wn,
                                           float eps, float scale, bool norm) {
  using Sh = DecodeShape<DK, DV, W>;
  constexpr int CG = Sh::CG, RG = Sh::RG, RPT = Sh::RPT, NT = Sh::NT;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  DecodeTok t = tin;

  // q and k L2-normalised over the dk channels (with the gates from logits).
  if (norm) {
    sm.red[tid] = (tid < DK) ? t.q * t.q : 0.f;
    sm.red2[tid] = (tid < DK) ? t.k * t.k : 0.f;
    __syncthreads();
    if (tid < 64) {
      float aq = 0.f, ak = 0.f;
      for (int i = tid; i < NT; i += 64) {
        aq += sm.red[i];
        ak += sm.red2[i];
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        aq += __shfl_xor(aq, off);
        ak += __shfl_xor(ak, off);
      }
      if (tid == 0) {
        sm.nq = rsqrtf(fmaxf(aq, 1e-24f));
        sm.nk = rsqrtf(fmaxf(ak, 1e-24f));
      }
    }
    __syncthreads();
    t.q *= sm.nq;
    t.k *= sm.nk;
  }

  // Per-channel factors and q . k (over the undecayed vectors).
  if (tid < DK) {
    const float a = __expf(t.g);
    sm.a[tid] = a;
    sm.kk[tid] = t.k;
    sm.ak[tid] = a * t.k;
    sm.aq[tid] = a * t.q;
  }
  sm.red[tid] = (tid < DK) ? t.q * t.k : 0.f;
  __syncthreads();
  if (tid < 64) {
    float acc = 0.f;
    for (int i = tid; i < NT; i += 64) acc += sm.red[i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (tid == 0) sm.qk = acc;
  }

  // Partial column sums over this thread's rows.
  f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + m * RG;
    p += sm.ak[i] * s[m];
    r += sm.aq[i] * s[m];
  }
  *(f32x4*)&sm.part[0][rg][4 * cg] = p;
  *(f32x4*)&sm.part[1][rg][4 * cg] = r;
  __syncthreads();

  // Column j: finish the reductions, form u_j and o_j.
  float oj = 0.f;
  if (tid < DV) {
    float pj = 0.f, rj = 0.f;
#pragma unroll 8
    for (int x = 0; x < RG; ++x) {
      pj += sm.part[0][x][tid];
      rj += sm.part[1][x][tid];
    }
    const float uj = t.beta * (t.v - pj);
    sm.u[tid] = uj;
    oj = scale * (rj + sm.qk * uj);
  }
  if (gated && orow != nullptr) sm.red[tid] = (tid < DV) ? oj * oj : 0.f;
  __syncthreads();

  // State update: S_ij <- a_i S_ij + k_i u_j (stored in place, kept for the next token).
  {
    const f32x4 u4 = *(const f32x4*)&sm.u[4 * cg];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      const int i = rg + m * RG;
      const f32x4 nv = sm.a[i] * s[m] + sm.kk[i] * u4;
      if (Sp != nullptr) __builtin_nontemporal_store(nv, (f32x4*)(Sp + i * DV + 4 * cg));
      if (KEEP) s[m] = nv;
    }
  }

  // Output, optionally through the head-wise RMSNorm x sigmoid(gate) epilogue.
  if (orow == nullptr || !gated) {
    if (orow != nullptr && tid < DV) st_f32(orow + tid, oj);
    __syncthreads();  // the shared buffers are reused by the next token
    return;
  }
  if (tid < 64) {
    float acc = 0.f;
    for (int j = tid; j < NT; j += 64) acc += sm.red[j];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (tid == 0) sm.ss = acc;
  }
  __syncthreads();
  if (tid < DV) {
    const float inv = rsqrtf(sm.ss / (float)DV + eps);
    st_f32(orow + tid, oj * inv * wn * sigmoidf_(t.gate));
  }
  __syncthreads();
}

// The single-token step: one workgroup of up to W threads per (b, h).
constexpr int kDecodeThreads = 1024;
template <int DK, int DV, typename IO, int W>
__global__ void __launch_bounds__((DecodeShape<DK, DV, W>::NT))
kda_decode_state_kernel(const IO* __restrict__ q, const IO* __restrict__ k,
                        const IO* __restrict__ v, const float* __restrict__ g,
                        const float* __restrict__ beta, float* __restrict__ state,
                        IO* __restrict__ o, const IO* __restrict__ gate,
                        const float* __restrict__ norm_w, float eps, float scale,
                        const IO* __restrict__ ga) {
  __shared__ DecodeSmem<DK, DV, W> sm;
  const int tid = threadIdx.x;
  const bool gated = gate != nullptr;
  const float wn = (gated && norm_w != nullptr && tid < DV) ? norm_w[tid] : 1.f;
  const int64_t bh = blockIdx.x;
  DecodeTile<DK, DV, W> t;
  decode_load<DK, DV, IO, W>(t, q, k, v, g, beta, state, gate, bh, bh, ga);
  decode_one<DK, DV, IO, false, W>(sm, t.s, t.x, state + bh * (int64_t)(DK * DV), o + bh * DV,
                                   gated, wn, eps, scale, ga != nullptr);
}

// K consecutive tokens of every (b, h) against its resident state: the state
// stays in registers from token to token, the outputs of all K tokens are
// written (when o is given), and the state after the first n_commit[b] tokens
// (all K when n_commit is NULL; values are clamped into [0, K]) is stored in
// place; with n_commit[b] = 0 the state is read and left as it was.  For
// speculative decoding: one call with n_commit = 0 verifies K draft tokens,
// one with the accepted counts and no output commits them (reading nothing of
// a sequence that commits 0).  The chain of K dependent token steps (each a
// few block-wide reductions) is latency-bound on one workgroup, so three
// workgroups share a compute unit (one register set each, grid of three per
// compute unit): measured on MI355X at B = 256, H = 96, K = 4 this verifies in
// 0.63 ms against 1.55 ms with one double-buffered workgroup per compute
// unit; four or more per compute unit
// were slower.  The next token's inputs load while a token is reduced.
template <int DK, int DV, typename IO, int W>
__global__ void __launch_bounds__((DecodeShape<DK, DV, W>::NT), 1)
kda_decode_multi_kernel(const IO* __restrict__ q, const IO* __restrict__ k,
                        const IO* __restrict__ v, const float* __restrict__ g,
                        const float* __restrict__ beta, float* __restrict__ state,
                        const int* __restrict__ n_commit, IO* __restrict__ o,
                        const IO* __restrict__ gate, const float* __restrict__ norm_w, float eps,
                        float scale, int64_t B, int64_t K, int64_t H, const IO* __restrict__ ga) {
  __shared__ DecodeSmem<DK, DV, W> sm;
  const int tid = threadIdx.x;
  const bool gated = gate != nullptr;
  const float wn = (gated && norm_w != nullptr && tid < DV) ? norm_w[tid] : 1.f;
  const int64_t BH = B * H, stride = gridDim.x;
  // row of token t of (b, h) = u in the [B, K, H, ..] inputs and outputs
  auto row = [&](int64_t u, int64_t t) { return ((u / H) * K + t) * H + u % H; };

  // tokens of (b, h) = u to commit, and to run (all K when there are outputs)
  auto commit = [&](int64_t u) {
    const int64_t n = n_commit != nullptr ? (int64_t)n_commit[u / H] : K;
    return n < 0 ? 0 : (n > K ? K : n);
  };
  auto runs = [&](int64_t u) { return o != nullptr ? K : commit(u); };
  // the state and first token of u, unless u has nothing to run
  auto load = [&](DecodeTile<DK, DV, W>& t, int64_t u) {
    if (runs(u) > 0)
      decode_load<DK, DV, IO, W>(t, q, k, v, g, beta, state, gate, u, row(u, 0), ga);
  };

  auto run = [&](DecodeTile<DK, DV, W>& cur, int64_t u) {
    const int64_t n = commit(u), last = runs(u);
    float* Sp = state + u * (int64_t)(DK * DV);
    DecodeTok x = cur.x;
    for (int64_t t = 0; t < last; ++t) {
      DecodeTok xn = x;
      if (t + 1 < last) xn = decode_load_tok<DK, DV, IO>(q, k, v, g, beta, gate, row(u, t + 1), ga);
      decode_one<DK, DV, IO, true, W>(sm, cur.s, x, t + 1 == n ? Sp : nullptr,
                                      o != nullptr ? o + row(u, t) * DV : nullptr, gated, wn,
                                      eps, scale, ga != nullptr);
      x = xn;
    }
  };

  for (int64_t u = blockIdx.x; u < BH; u += stride) {
    DecodeTile<DK, DV, W> t;
    load(t, u);
    run(t, u);
  }
}

// 2 <= K <= 4 tokens of every (b, h), with outputs, in the chunkwise form of
// the recurrence (the algebra of the chunked prefill, "Kimi K3: Engineering
// ...", section "Dimension 1", on one small tile): with G the cumulative
// log-decay over the tokens, Kh = k e^G, Qh = scale q e^G, Kc = k e^-G,
//   P = Kh S,  R = Qh S                      (one pass over the state)
//   A = strict_lower(Diag(beta) Kh Kc^T),  Aqk = lower(Qh Kc^T),  T = (I + A)^-1 Diag(beta)
//   D = T (V - P),  O = R + Aqk D
//   S_n = Diag(e^G_{n-1}) (S + Kc[:n]^T D[:n])   (the state after the first n tokens)
// so the K dependent token steps of kda_decode_multi_kernel become a few
// block-wide phases.  dk = dv = 128, the state in the same float4 strips as
// the single-token kernel; same contract as kda_decode_multi_kernel (with ga:
// from the raw projections, q and k normalised and g, beta from their logits).
template <typename IO, bool LOGITS>
__global__ void __launch_bounds__(256, 3)
kda_multi_chunk_kernel(const IO* __restrict__ q, const IO* __restrict__ k,
                       const IO* __restrict__ v, const float* __restrict__ g,
                       const float* __restrict__ beta, float* __restrict__ state,
                       const int* __restrict__ n_commit, IO* __restrict__ o,
                       const IO* __restrict__ gate, const float* __restrict__ norm_w, float eps,
                       float scale, int64_t B, int64_t K, int64_t H,
                       const IO* __restrict__ ga) {
  constexpr int D = 128, KM = 4, CG = D / 4, RG = 256 / CG, RPT = D / RG;
  __shared__ float kh[KM][D], qh[KM][D], kc[KM][D], ex[KM][D];
  __shared__ float vv[KM][D];            // values, then D (the deltas)
  __shared__ f32x4 part[2][KM][RG][CG];  // P, R partial sums per row group
  __shared__ float pr[2][KM][D];         // P, R
  __shared__ float am[KM][KM], aq[KM][KM], tt[KM][KM], bt[KM];
  __shared__ float rs[2][KM];            // row sums of O^2 per wave (gated epilogue)
  const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
  const int64_t BH = B * H;
  const bool gated = gate != nullptr;
  const float wn = (gated && norm_w != nullptr && tid < D) ? norm_w[tid] : 1.f;
  auto row = [&](int64_t u, int64_t t) { return ((u / H) * K + t) * H + u % H; };

  for (int64_t u = blockIdx.x; u < BH; u += gridDim.x) {
    int64_t n = n_commit != nullptr ? (int64_t)n_commit[u / H] : K;
    n = n < 0 ? 0 : (n > K ? K : n);
    const int L = (int)K;
    float* Sp = state + u * (int64_t)(D * D);
    // 1. the state strip and the tokens' inputs
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
      s[m] = __builtin_nontemporal_load((const f32x4*)(Sp + (rg + m * RG) * D + 4 * cg));
#pragma unroll 1
    for (int e = tid; e < L * D; e += 256) {
      const int t = e / D, c = e % D;
      const int64_t rw = row(u, t);
      kh[t][c] = ld_f32(k + rw * D + c);
      qh[t][c] = ld_f32(q + rw * D + c);
      kc[t][c] = LOGITS ? -5.f * sigmoidf_(ld_f32(ga + rw * D + c)) : g[rw * D + c];
      vv[t][c] = ld_f32(v + rw * D + c);
    }
    if (tid < L) {
      const float bb = beta[row(u, tid)];
      bt[tid] = LOGITS ? sigmoidf_(bb) : bb;
    }
    __syncthreads();
    if constexpr (LOGITS) {  // from raw projections: wave t L2-normalises q and k of token t
      const int t = tid / 64, l = tid % 64;
      const bool live = t < L;
      const float q0 = live ? qh[t][l] : 0.f, q1 = live ? qh[t][l + 64] : 0.f;
      const float k0 = live ? kh[t][l] : 0.f, k1 = live ? kh[t][l + 64] : 0.f;
      float nq = q0 * q0 + q1 * q1, nk = k0 * k0 + k1 * k1;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        nq += __shfl_xor(nq, off);
        nk += __shfl_xor(nk, off);
      }
      if (live) {
        const float rq = rsqrtf(fmaxf(nq, 1e-24f)), rk = rsqrtf(fmaxf(nk, 1e-24f));
        qh[t][l] = q0 * rq;
        qh[t][l + 64] = q1 * rq;
        kh[t][l] = k0 * rk;
        kh[t][l + 64] = k1 * rk;
      }
      __syncthreads();
    }
    // 2. cumulative log-decay per channel, the rescaled keys and queries
    if (tid < D) {
      float gam = 0.f;
      for (int t = 0; t < L; ++t) {
        gam += kc[t][tid];
        const float e = __expf(gam), kk = kh[t][tid];
        ex[t][tid] = e;
        kh[t][tid] = kk * e;
        qh[t][tid] = scale * qh[t][tid] * e;
        kc[t][tid] = kk * __expf(-gam);
      }
    }
    __syncthreads();
    // 3. P, R over this thread's rows; the intra-tile products
#pragma unroll 1
    for (int t = 0; t < L; ++t) {
      f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = p;
#pragma unroll
      for (int m = 0; m < RPT; ++m) {
        p += kh[t][rg + m * RG] * s[m];
        r += qh[t][rg + m * RG] * s[m];
      }
      part[0][t][rg][cg] = p;
      part[1][t][rg][cg] = r;
    }
    {  // the 16 (t, c) products, 16 lanes each over 8 channels
      const int t = tid / (16 * KM), c = (tid / 16) % KM, sub = tid % 16;
      float a = 0.f, b2 = 0.f;
#pragma unroll
      for (int m = 0; m < D / 16; ++m) {
        const int i = sub + 16 * m;
        a = fmaf(kh[t][i], kc[c][i], a);
        b2 = fmaf(qh[t][i], kc[c][i], b2);
      }
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) {
        a += __shfl_xor(a, off);
        b2 += __shfl_xor(b2, off);
      }
      if (sub == 0 && t < L && c < L) {
        am[t][c] = c < t ? bt[t] * a : 0.f;
        aq[t][c] = c <= t ? b2 : 0.f;
      }
    }
    __syncthreads();
    // 4. P and R per column; T = (I + A)^-1 Diag(beta) by forward substitution
#pragma unroll 1
    for (int e = tid; e < 2 * L * D; e += 256) {
      const int w = e / (L * D), t = (e / D) % L, j = e % D;
      float acc = 0.f;
#pragma unroll
      for (int x = 0; x < RG; ++x) acc += ((const float*)&part[w][t][x][0])[j];
      pr[w][t][j] = acc;
    }
    if (tid < L) {
      const int c = tid;
      float y[KM];
#pragma unroll
      for (int t = 0; t < KM; ++t) {
        float acc = (t == c) ? 1.f : 0.f;
        for (int m = c; m < t; ++m) acc -= am[t][m] * y[m];
        y[t] = (t < c || t >= L) ? 0.f : acc;
      }
#pragma unroll
      for (int t = 0; t < KM; ++t)
        if (t < L) tt[t][c] = y[t] * bt[c];
    }
    __syncthreads();
    // 5. D = T (V - P) and O = R + Aqk D, column j = tid (its values and
    // deltas are read and written by its thread alone)
    float ot[KM];
    if (tid < D) {
      const int j = tid;
      float dcol[KM];
#pragma unroll
      for (int t = 0; t < KM; ++t) {
        float acc = 0.f;
        if (t < L)
          for (int c = 0; c <= t; ++c) acc = fmaf(tt[t][c], vv[c][j] - pr[0][c][j], acc);
        dcol[t] = acc;
      }
#pragma unroll
      for (int t = 0; t < KM; ++t) {
        float acc = 0.f;
        if (t < L) {
          acc = pr[1][t][j];
          for (int c = 0; c <= t; ++c) acc = fmaf(aq[t][c], dcol[c], acc);
        }
        ot[t] = acc;
      }
#pragma unroll
      for (int t = 0; t < KM; ++t)
        if (t < L) vv[t][j] = dcol[t];
      if (gated) {
#pragma unroll
        for (int t = 0; t < KM; ++t) {
          float x = ot[t] * ot[t];
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
          if (tid % 64 == 0) rs[tid / 64][t] = x;
        }
      }
    }
    __syncthreads();  // D in vv; the row sums in rs
    // 6. outputs
    if (tid < D) {
      const int j = tid;
#pragma unroll
      for (int t = 0; t < KM; ++t) {
        if (t >= L) break;
        float y = ot[t];
        if (gated) {
          const float inv = rsqrtf((rs[0][t] + rs[1][t]) / (float)D + eps);
          y = y * inv * wn * sigmoidf_(ld_f32(gate + row(u, t) * D + j));
        }
        st_f32(o + row(u, t) * D + j, y);
      }
    }
    // 7. the state after n tokens
    if (n > 0) {
      const int nn = (int)n;
#pragma unroll
      for (int m = 0; m < RPT; ++m) {
        const int i = rg + m * RG;
        f32x4 acc = s[m];
        for (int t = 0; t < nn; ++t) acc += kc[t][i] * *(const f32x4*)&vv[t][4 * cg];
        __builtin_nontemporal_store(ex[nn - 1][i] * acc, (f32x4*)(Sp + i * D + 4 * cg));
      }
    }
    __syncthreads();  // the shared arrays are reused by the next (b, h)
  }
}

// The compute units of the device, at most `units`: the multi-token kernels'
// persistent grids are a multiple of it.
int decode_grid(int64_t units) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (cus < 1) cus = 256;
  return (int)(units < cus ? units : cus);
}

template <int DK, int DV, typename IO>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  const int64_t bhn = a.B * a.H;
  const int nblk = decode_grid(bhn);
  if (a.K >= 2 && a.K <= 4 && a.o != nullptr && DK == 128 && DV == 128) {
    // verify calls with few draft tokens: the chunkwise form, three workgroups per CU
    const int64_t cblk = bhn < 3 * (int64_t)nblk ? bhn : 3 * (int64_t)nblk;
    auto kern = a.ga != nullptr ? kda_multi_chunk_kernel<IO, true> : kda_multi_chunk_kernel<IO, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)cblk), dim3(256), 0, (hipStream_t)a.stream,
                       (const IO*)a.q, (const IO*)a.k, (const IO*)a.v, a.g, a.beta, a.state,
                       a.n_commit, (IO*)a.o, (const IO*)a.gate, a.norm_w, a.eps, a.scale, a.B,
                       a.K, a.H, (const IO*)a.ga);
    return hipGetLastError();
  }
  if (a.K > 0) {
    // three persistent 256-thread workgroups per CU: the chain of token steps
    // is latency-bound, and the single-token step's shape (one 1024-thread
    // workgroup per state) measured 0.81 against 0.52 ms for the commit call
    // at B = 256, H = 96, K = 4
    const int64_t mblk = bhn < 3 * (int64_t)nblk ? bhn : 3 * (int64_t)nblk;
    constexpr int MW = 256;
    using Sm = DecodeShape<DK, DV, MW>;
    hipLaunchKernelGGL((kda_decode_multi_kernel<DK, DV, IO, MW>), dim3((unsigned)mblk),
                       dim3(Sm::NT), 0, (hipStream_t)a.stream, (const IO*)a.q, (const IO*)a.k,
                       (const IO*)a.v, a.g, a.beta, a.state, a.n_commit, (IO*)a.o,
                       (const IO*)a.gate, a.norm_w, a.eps, a.scale, a.B, a.K, a.H,
                       (const IO*)a.ga);
    return hipGetLastError();
  }
  if (bhn < 1 || bhn > 0x7fffffffLL) return hipErrorInvalidValue;
  using Sw = DecodeShape<DK, DV, kDecodeThreads>;
  hipLaunchKernelGGL((kda_decode_state_kernel<DK, DV, IO, kDecodeThreads>), dim3((unsigned)bhn),
                     dim3(Sw::NT), 0, (hipStream_t)a.stream, (const IO*)a.q, (const IO*)a.k,
                     (const IO*)a.v, a.g, a.beta, a.state, (IO*)a.o, (const IO*)a.gate, a.norm_w,
                     a.eps, a.scale, (const IO*)a.ga);
  return hipGetLastError();
}

template <typename IO>
static hipError_t dispatch_dims(const DecodeArgs& a) {
#define KDA_CASE(DKV, DVV) \
  if (a.dk == DKV && a.dv == DVV) return launch_decode_t<DKV, DVV, IO>(a);
#define KDA_ROW(DKV) KDA_CASE(DKV, 16) KDA_CASE(DKV, 32) KDA_CASE(DKV, 64) KDA_CASE(DKV, 128)
  KDA_ROW(16) KDA_ROW(32) KDA_ROW(64) KDA_ROW(128)
#undef KDA_ROW
#undef KDA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a) {
  return a.io_bf16 ? dispatch_dims<bf16_t>(a) : dispatch_dims<float>(a);
}

}  // namespace kda
