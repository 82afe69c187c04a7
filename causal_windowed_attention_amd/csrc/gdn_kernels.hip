// Gated delta rule (GDN linear attention) forward for gfx950, chunkwise.
//
// SANA-Streaming ("Transformer a diffusione ibrido") runs most blocks as Gated DeltaNet
// linear attention: a fixed-size state per head carried along the stream. The pages give
// no equations; the recurrence is the published gated delta rule (Yang, Kautz and
// Hatamizadeh, "Gated Delta Networks", ICLR 2025), per token in (frame, y, x) order:
//   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
// with S of size Dv x Dk. Written as S_t = alpha_t S_{t-1} + u_t k_t^T with pseudo-values
// u_t = beta_t (v_t - alpha_t S_{t-1} k_t), a block of C = 64 tokens starting from state
// S0 (local cumulative gates gam_i = prod_{j<=i} alpha_j, kept as logs g_i) gives:
//   T  = (I + diag(beta) A)^-1 diag(beta),  A_ij = (gam_i / gam_j) k_i.k_j  (j < i)
//   U  = T V - (T diag(gam) K) S0^T = Up - W S0^T
//   O  = diag(gam) Q S0^T + ((Q K^T) o M) U,  M_ij = gam_i / gam_j  (j <= i)
//   S' = gam_C S0 + U^T Kt,  Kt = diag(gam_C / gam) K
// Three kernels: gdn_prep (every block independently: gates, T by forward substitution,
// W, Up and Kt), gdn_scan (the only sequential part: the state through the blocks, in
// row slices of S, which evolve independently; records each block's starting state and
// U), gdn_out (every block independently: the outputs). Arithmetic is fp32: register
// tiles on the VALU fed by 16-byte LDS reads (rows padded by 4 floats: aligned and
// conflict-free) in gdn_prep and gdn_out; the scan's two products on the fp32 MFMA with
// operands prefetched from global memory into registers. Inputs and outputs are bf16,
// the state fp32.
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kC = kGdnBlock;        // tokens per block
constexpr int kThr = 256;
constexpr int kCL = kC + 4;          // padded row of a 64-wide LDS tile

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ float at(const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

// acc[i][j] += sum_{k < K} A[r0 + i][k] * B(k, c0 + j), A row-major (a + r * lda + k).
// BT: B(k, c) = b[c * ldb + k] (rows of b contiguous in k); else B(k, c) = b[k * ldb + c].
// RN is a multiple of 4 when !BT; lda, ldb multiples of 4, bases 16-byte aligned.
template <int RM, int RN, int K, bool BT>
__device__ __forceinline__ void gemm(float (&acc)[RM][RN], const float* a, int lda, const float* b, int ldb, int r0,
                                     int c0) {
#pragma unroll 4
  for (int k = 0; k < K; k += 4) {
    float4 av[RM];
#pragma unroll
    for (int i = 0; i < RM; ++i) av[i] = ld4(a + (r0 + i) * lda + k);
    if constexpr (BT) {
      float4 bv[RN];
#pragma unroll
      for (int j = 0; j < RN; ++j) bv[j] = ld4(b + (c0 + j) * ldb + k);
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j) {
          acc[i][j] = fmaf(av[i].x, bv[j].x, acc[i][j]);
          acc[i][j] = fmaf(av[i].y, bv[j].y, acc[i][j]);
          acc[i][j] = fmaf(av[i].z, bv[j].z, acc[i][j]);
          acc[i][j] = fmaf(av[i].w, bv[j].w, acc[i][j]);
        }
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        float4 bv[RN / 4];
#pragma unroll
        for (int j4 = 0; j4 < RN / 4; ++j4) bv[j4] = ld4(b + (k + kk) * ldb + c0 + 4 * j4);
#pragma unroll
        for (int i = 0; i < RM; ++i) {
          const float x = at(av[i], kk);
#pragma unroll
          for (int j4 = 0; j4 < RN / 4; ++j4) {
            acc[i][4 * j4 + 0] = fmaf(x, bv[j4].x, acc[i][4 * j4 + 0]);
            acc[i][4 * j4 + 1] = fmaf(x, bv[j4].y, acc[i][4 * j4 + 1]);
            acc[i][4 * j4 + 2] = fmaf(x, bv[j4].z, acc[i][4 * j4 + 2]);
            acc[i][4 * j4 + 3] = fmaf(x, bv[j4].w, acc[i][4 * j4 + 3]);
          }
        }
      }
    }
  }
}

// Rows [0, 64) x D of a token-major [B, N, H, D] bf16 tensor into an fp32 LDS tile with
// row stride ld; tokens at or past n_valid read as zeros.
template <int D>
__device__ __forceinline__ void load_rows(float* dst, int ld, const __bf16* src, const GdnParams& p, int b, int h,
                                          int t0, int n_valid) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
#pragma unroll
  for (int e = threadIdx.x; e < kC * D / 8; e += kThr) {
    const int i = e / (D / 8), c = (e % (D / 8)) * 8;
    bf16x8 x = {};
    if (i < n_valid)
      x = *reinterpret_cast<const bf16x8*>(src + ((static_cast<size_t>(b) * p.N + t0 + i) * p.H + h) * D + c);
    st4(dst + i * ld + c, make_float4(static_cast<float>(x[0]), static_cast<float>(x[1]), static_cast<float>(x[2]),
                                      static_cast<float>(x[3])));
    st4(dst + i * ld + c + 4, make_float4(static_cast<float>(x[4]), static_cast<float>(x[5]),
                                          static_cast<float>(x[6]), static_cast<float>(x[7])));
  }
}

// Storage order of W and Kt within a block, chosen for the scan's MFMA B operands:
// W[i][k] at i * D + (k % 4) * (D / 4) + k / 4 (lane (i % 16, q = k % 4) reads its k-steps
// contiguously); Kt[i][c] at ((c / 16) * 64 + 16 (i % 4) + c % 16) * 16 + i / 4 (lane
// 16 (i % 4) + c % 16 of column tile c / 16 reads its 16 token steps contiguously).
template <int D>
__device__ __forceinline__ int wperm_index(int i, int k) { return i * D + (k & 3) * (D / 4) + (k >> 2); }
__device__ __forceinline__ int ktperm_index(int i, int c) {
  return ((c >> 4) * 64 + 16 * (i & 3) + (c & 15)) * 16 + (i >> 2);
}

// ---- gdn_prep: per block, log gates, T, W = T diag(gam) K, Up = T V, Kt ---------------------
template <int D>
__global__ __launch_bounds__(kThr) void gdn_prep(GdnParams p) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  constexpr int LD = D + 4;
  float* Ks = sm;                                // [64][LD]
  float* Vs = Ks + kC * LD;                      // [64][LD]
  float* L = Vs + kC * LD;                       // [64][kCL]: beta_i A_ij (j < i)
  float* X = L + kC * kCL;                       // [64][kCL]: T
  float* g = X + kC * kCL;                       // [64] log cumulative gates
  float* bet = g + kC;                           // [64]
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int t0 = blk * kC, n_valid = min(kC, p.N - t0);
  const size_t bh = static_cast<size_t>(b) * p.H + h;
  const size_t boff = (bh * p.nb + blk) * static_cast<size_t>(kC) * D;

  load_rows<D>(Ks, LD, static_cast<const __bf16*>(p.k), p, b, h, t0, n_valid);
  load_rows<D>(Vs, LD, static_cast<const __bf16*>(p.v), p, b, h, t0, n_valid);
  if (tid < kC) {                                // padded tokens: alpha = 1, beta = 0 (no effect)
    const bool ok = tid < n_valid;
    float s = ok ? __logf(p.alpha[bh * p.N + t0 + tid]) : 0.f;
    bet[tid] = ok ? p.beta[bh * p.N + t0 + tid] : 0.f;
#pragma unroll
    for (int o = 1; o < kC; o <<= 1) {           // prefix sum over the first wave
      const float t = __shfl_up(s, o, 64);
      if (tid >= o) s += t;
    }
    g[tid] = s;
    p.g[bh * (static_cast<size_t>(p.nb) * kC) + t0 + tid] = s;
  }
  __syncthreads();

  // L_ij = beta_i exp(g_i - g_j) k_i.k_j for j < i: a 4 x 4 tile per thread
  {
    const int r0 = (tid / 16) * 4, c0 = (tid % 16) * 4;
    float acc[4][4] = {};
    gemm<4, 4, D, true>(acc, Ks, LD, Ks, LD, r0, c0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = r0 + i, c = c0 + j;
        L[r * kCL + c] = c < r ? bet[r] * __expf(g[r] - g[c]) * acc[i][j] : 0.f;
      }
  }
  __syncthreads();
  // X = (I + L)^-1 by forward substitution. Column j depends only on itself
  // (X_jj = 1, X_ij = -sum_{k < i} L_ik X_kj), so lane j of the first wave solves it in
  // registers; L_ik is the same address for every lane (an LDS broadcast). T = X diag(beta).
  if (tid < kC) {
    const int j = tid;
    float x[kC];
#pragma unroll
    for (int i = 0; i < kC; ++i) {
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int k = 0; k + 3 < i; k += 4) {
        const float4 l = ld4(L + i * kCL + k);
        s0 = fmaf(l.x, x[k], s0);
        s1 = fmaf(l.y, x[k + 1], s1);
        s2 = fmaf(l.z, x[k + 2], s2);
        s3 = fmaf(l.w, x[k + 3], s3);
      }
#pragma unroll
      for (int k = i & ~3; k < i; ++k) s0 = fmaf(L[i * kCL + k], x[k], s0);
      x[i] = i == j ? 1.f : (i < j ? 0.f : -((s0 + s1) + (s2 + s3)));
    }
    const float bj = bet[j];
#pragma unroll
    for (int i = 0; i < kC; ++i) X[i * kCL + j] = x[i] * bj;
  }
  __syncthreads();
  // Up = T V; Kt = diag(exp(g_C - g)) K; W = T diag(exp g) K: 64 x D, 4 x RN per thread
  constexpr int RN = D / 16;
  const int r0 = (tid / 16) * 4, c0 = (tid % 16) * RN;
  {
    float acc[4][RN] = {};
    gemm<4, RN, kC, false>(acc, X, kCL, Vs, LD, r0, c0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < RN; j += 4)
        st4(p.Up + boff + (r0 + i) * D + c0 + j, make_float4(acc[i][j], acc[i][j + 1], acc[i][j + 2], acc[i][j + 3]));
  }
  const float gC = g[kC - 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {                  // this thread's Kt entries, from the unscaled K
    const float e = __expf(gC - g[r0 + i]);
#pragma unroll
    for (int j = 0; j < RN; ++j)
      p.Kt[boff + ktperm_index(r0 + i, c0 + j)] = e * Ks[(r0 + i) * LD + c0 + j];
  }
  __syncthreads();
  for (int e = tid; e < kC * D / 4; e += kThr) { // K rows scaled by gam_i, in place
    const int r = e / (D / 4), c = (e % (D / 4)) * 4;
    const float s = __expf(g[r]);
    const float4 kk = ld4(Ks + r * LD + c);
    st4(Ks + r * LD + c, make_float4(s * kk.x, s * kk.y, s * kk.z, s * kk.w));
  }
  __syncthreads();
  {
    float acc[4][RN] = {};
    gemm<4, RN, kC, false>(acc, X, kCL, Ks, LD, r0, c0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < RN; ++j) p.W[boff + wperm_index<D>(r0 + i, c0 + j)] = acc[i][j];
  }
}

// ---- gdn_scan: the state through the blocks, rows [rs, rs + 16) of S per workgroup ----------
// Per block, on the fp32 MFMA (v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16]
// and B[l / 16][l % 16] and receives C[4 (l / 16) + j][l % 16]):
//   U^T (16 x 64) = S (16 x D) W^T: wave w takes tokens [16 w, 16 w + 16), all of D;
//   S' (16 x D) = exp(g_C) S + U^T (16 x 64) Kt (64 x D): wave w takes NT column tiles.
// The state lives in registers in the C layout; U and S cross between waves through LDS
// (read back in the A layout). gdn_prep stores W and Kt in the lane order of the B
// operands (wperm_index, ktperm_index), so each lane prefetches contiguous float4s for
// the next block while the current one computes.
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(kThr) void gdn_scan(GdnParams p) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  static_assert(kGdnScanRows == 16, "one 16-row MFMA tile of the state per workgroup");
  constexpr int LD = D + 4;
  constexpr int KS = D / 4;                      // k-steps of the U product
  constexpr int NT = D / 64;                     // 16-column tiles of the state per wave
  float* Sx = sm;                                // [16][LD]  state exchange
  float* Ux = Sx + 16 * LD;                      // [64][16]  U exchange
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int l = tid & 63, w = tid >> 6, lr = l & 15, lq = l >> 4;
  const int rs = split * 16;
  const size_t bh = static_cast<size_t>(b) * p.H + h;
  auto boff = [&](int blk) { return (bh * p.nb + blk) * static_cast<size_t>(kC) * D; };

  f32x4 sc[NT];                                  // S[4 lq + j][16 (NT w + t) + lr]
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sc[t][j] = p.state_in != nullptr ? p.state_in[(bh * D + rs + 4 * lq + j) * D + 16 * (NT * w + t) + lr] : 0.f;
  float wv[KS], kv[NT][16];                      // B operands: W^T and Kt of the block
  float4 up;                                     // Up[16 w + lr][rs + 4 lq ..]
  float gC;
  auto fetch_w = [&](int blk) {
    const float* src = p.W + boff(blk) + (16 * w + lr) * D + lq * KS;
#pragma unroll
    for (int u = 0; u < KS / 4; ++u) {
      const float4 t = ld4(src + 4 * u);
      wv[4 * u] = t.x; wv[4 * u + 1] = t.y; wv[4 * u + 2] = t.z; wv[4 * u + 3] = t.w;
    }
  };
  auto fetch_rest = [&](int blk) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float* src = p.Kt + boff(blk) + ((NT * w + t) * 64 + l) * 16;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 v = ld4(src + 4 * u);
        kv[t][4 * u] = v.x; kv[t][4 * u + 1] = v.y; kv[t][4 * u + 2] = v.z; kv[t][4 * u + 3] = v.w;
      }
    }
    up = ld4(p.Up + boff(blk) + (16 * w + lr) * D + rs + 4 * lq);
    gC = p.g[bh * (static_cast<size_t>(p.nb) * kC) + blk * kC + kC - 1];
  };
  // state -> A layout (lane l: S[lr][4 s + lq]) through LDS
  float sa[KS];
  auto exchange_state = [&] {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) Sx[(4 * lq + j) * LD + 16 * (NT * w + t) + lr] = sc[t][j];
    __syncthreads();
#pragma unroll
    for (int s = 0; s < KS; ++s) sa[s] = Sx[lr * LD + 4 * s + lq];
  };
  fetch_w(0);
  fetch_rest(0);
  exchange_state();
  for (int blk = 0; blk < p.nb; ++blk) {
    float* Sst = p.Sst + (bh * p.nb + blk) * static_cast<size_t>(D) * D;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) Sst[(rs + 4 * lq + j) * D + 16 * (NT * w + t) + lr] = sc[t][j];
    // U^T tile of tokens [16 w, 16 w + 16): two accumulators over the k-steps
    f32x4 a0 = {}, a1 = {};
#pragma unroll
    for (int s = 0; s < KS; s += 2) {
      a0 = __builtin_amdgcn_mfma_f32_16x16x4f32(sa[s], wv[s], a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x4f32(sa[s + 1], wv[s + 1], a1, 0, 0, 0);
    }
    if (blk + 1 < p.nb) fetch_w(blk + 1);
    // U[16 w + lr][4 lq + j] = Up - (S W^T)^T
    const float4 u4 = make_float4(up.x - (a0[0] + a1[0]), up.y - (a0[1] + a1[1]), up.z - (a0[2] + a1[2]),
                                  up.w - (a0[3] + a1[3]));
    {                                            // U^T[c][token] for gdn_out
      float* ut = p.U + boff(blk) + static_cast<size_t>(rs + 4 * lq) * kC + 16 * w + lr;
      ut[0] = u4.x; ut[kC] = u4.y; ut[2 * kC] = u4.z; ut[3 * kC] = u4.w;
    }
    st4(Ux + (16 * w + lr) * 16 + 4 * lq, u4);
    __syncthreads();
    float ua[16];                                // A layout of U^T: U[4 s + lq][lr]
#pragma unroll
    for (int s = 0; s < 16; ++s) ua[s] = Ux[(4 * s + lq) * 16 + lr];
    const float dec = __expf(gC);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4 acc = sc[t] * dec;
#pragma unroll
      for (int s = 0; s < 16; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ua[s], kv[t][s], acc, 0, 0, 0);
      sc[t] = acc;
    }
    if (blk + 1 < p.nb) fetch_rest(blk + 1);
    exchange_state();                            // also orders this block's Ux reads before the next writes
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      p.state_out[(bh * D + rs + 4 * lq + j) * D + 16 * (NT * w + t) + lr] = sc[t][j];
}

// ---- gdn_out: the outputs of one block, transposed -------------------------------------
//   O^T = S0 Q^T diag(gam) + U^T P^T,   P^T_ji = exp(g_i - g_j) k_j.q_i  (j <= i)
// on v_mfma_f32_32x32x16_bf16 (lane l supplies A[l % 32][8 (l / 32) + e] and
// B[8 (l / 32) + e][l % 32], e < 8, and receives C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32]).
// Q and K are bf16, so P^T = K Q^T has exact products; the fp32 operands S0, U^T and P^T
// enter as bf16 pairs x = hi + lo (|x - hi - lo| <= 2^-16 |x|), S0 Q^T in two products and
// U^T P^T in three (the lo * lo term, below 2^-16 of each product, is dropped). P^T leaves
// its accumulator as the B operand in registers: the accumulator's row order within a
// 16-row step is the token order tau(e) = 8 (e / 4) + 4 (l / 32) + e % 4, so the U^T operand
// is read in that order (two 4-token runs per lane). Wave w takes query tile w % 2 and
// Dv tiles [CTW (w / 2), CTW (w / 2) + CTW) of 32 rows; every operand comes straight from
// global memory (L2), only the gates go through LDS.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ void split_bf16(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 t = static_cast<__bf16>(x[e]);
    hi[e] = t;
    lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(t));
  }
}
__device__ __forceinline__ void unpack8(const float4& a, const float4& b, float (&x)[8]) {
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(kThr) void gdn_out(GdnParams p) {
  __shared__ float gs[kC];
  constexpr int KS = D / 16;                     // k-steps over D
  constexpr int CTW = D / 64;                    // Dv tiles per wave
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int l = tid & 63, w = tid >> 6, lc = l & 31, hf = l >> 5;
  const int it = w & 1;
  const int t0 = blk * kC, n_valid = min(kC, p.N - t0);
  const size_t bh = static_cast<size_t>(b) * p.H + h;
  const size_t rs = static_cast<size_t>(p.H) * D;                  // token stride of q, k, out
  const size_t base = (static_cast<size_t>(b) * p.N + t0) * rs + static_cast<size_t>(h) * D;
  const __bf16* qb = static_cast<const __bf16*>(p.q) + base;
  const __bf16* kb = static_cast<const __bf16*>(p.k) + base;
  const size_t boff = (bh * p.nb + blk) * static_cast<size_t>(kC) * D;
  const float* S0 = p.Sst + (bh * p.nb + blk) * static_cast<size_t>(D) * D;
  const float* Ut = p.U + boff;                                     // U^T: [D][64]
  if (tid < kC) gs[tid] = p.g[bh * (static_cast<size_t>(p.nb) * kC) + t0 + tid];

  const int qi = 32 * it + lc;                                      // this lane's query (column)
  bf16x8 bq[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s)
    bq[s] = qi < n_valid ? *reinterpret_cast<const bf16x8*>(qb + qi * rs + 16 * s + 8 * hf) : bf16x8{};
  f32x16 pt[2] = {};
#pragma unroll
  for (int jt = 0; jt < 2; ++jt) {
    if (jt > it) break;
    const int kj = 32 * jt + lc;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 ak = kj < n_valid ? *reinterpret_cast<const bf16x8*>(kb + kj * rs + 16 * s + 8 * hf) : bf16x8{};
      pt[jt] = mfma_bf16(ak, bq[s], pt[jt]);
    }
  }
  __syncthreads();
  const float gi = gs[qi];
  bf16x8 pbh[2][2], pbl[2][2];                                      // [j tile][16-token step]
#pragma unroll
  for (int jt = 0; jt < 2; ++jt)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 32 * jt + 16 * s2 + 8 * (e >> 2) + 4 * hf + (e & 3);
        x[e] = (jt <= it && j <= qi) ? __expf(gi - gs[j]) * pt[jt][8 * s2 + e] : 0.f;
      }
      split_bf16(x, pbh[jt][s2], pbl[jt][s2]);
    }
  const float eg = __expf(gi);
  __bf16* ob = static_cast<__bf16*>(p.out) + base;
#pragma unroll
  for (int u = 0; u < CTW; ++u) {
    const int c = 32 * ((w >> 1) * CTW + u) + lc;                  // this lane's Dv row of O^T
    f32x16 o = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float* src = S0 + static_cast<size_t>(c) * D + 16 * s + 8 * hf;
      float x[8];
      unpack8(ld4(src), ld4(src + 4), x);
      bf16x8 ah, al;
      split_bf16(x, ah, al);
      o = mfma_bf16(ah, bq[s], o);
      o = mfma_bf16(al, bq[s], o);
    }
    o *= eg;
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      if (jt > it) break;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const float* src = Ut + c * kC + 32 * jt + 16 * s2 + 4 * hf;
        float x[8];
        unpack8(ld4(src), ld4(src + 8), x);
        bf16x8 ah, al;
        split_bf16(x, ah, al);
        o = mfma_bf16(ah, pbh[jt][s2], o);
        o = mfma_bf16(al, pbh[jt][s2], o);
        o = mfma_bf16(ah, pbl[jt][s2], o);
      }
    }
    if (qi < n_valid) {
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cr = 32 * ((w >> 1) * CTW + u) + 8 * q + 4 * hf;
        const bf16x4 v = {static_cast<__bf16>(o[4 * q]), static_cast<__bf16>(o[4 * q + 1]),
                          static_cast<__bf16>(o[4 * q + 2]), static_cast<__bf16>(o[4 * q + 3])};
        *reinterpret_cast<bf16x4*>(ob + qi * rs + cr) = v;
      }
    }
  }
}

template <int D>
constexpr size_t prep_lds() { return (2 * kC * (D + 4) + 2 * kC * kCL + 2 * kC) * sizeof(float); }
template <int D>
constexpr size_t scan_lds() { return (16 * (D + 4) + kC * 16) * sizeof(float); }

template <int D>
hipError_t launch_gdn_d(const GdnParams& p, hipStream_t st) {
  static_assert(prep_lds<D>() <= 160 * 1024 && scan_lds<D>() <= 160 * 1024,
                "LDS budget");
  static_assert(D % 64 == 0, "scan tiles");
  static bool attrs = false;                     // dynamic LDS above 64 KB, set once per process
  if (!attrs) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gdn_prep<D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(prep_lds<D>()));
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(gdn_scan<D>), hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(scan_lds<D>()));
    if (e != hipSuccess) return e;
    attrs = true;
  }
  hipLaunchKernelGGL(gdn_prep<D>, dim3(p.nb, p.H, p.B), dim3(kThr), prep_lds<D>(), st, p);
  hipLaunchKernelGGL(gdn_scan<D>, dim3(D / kGdnScanRows, p.H, p.B), dim3(kThr), scan_lds<D>(), st, p);
  hipLaunchKernelGGL(gdn_out<D>, dim3(p.nb, p.H, p.B), dim3(kThr), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn_forward(const GdnParams& p, hipStream_t st) {
  if (p.N <= 0) return hipSuccess;
  return p.D == 128 ? launch_gdn_d<128>(p, st) : launch_gdn_d<64>(p, st);
}

}  // namespace sa
