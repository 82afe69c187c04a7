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
//   S' = gam_C S0 + U^T diag(gam_C / gam) K
// Three kernels: gdn_prep (every block independently: gates, T by forward substitution,
// W and Up), gdn_scan (the only sequential part: the state through the blocks, in row
// slices of S, which evolve independently; records each block's starting state and U),
// gdn_out (every block independently: the outputs). All arithmetic is fp32 on the VALU
// through LDS tiles; inputs and outputs are bf16, the state fp32.
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kC = kGdnBlock;        // tokens per block
constexpr int kThr = 256;

__device__ __forceinline__ float bf(const __bf16 x) { return static_cast<float>(x); }

// acc[i][j] += sum_k A(r0 + i, k) * B(k, c0 + j) over k < K, with A(i, k) = a[i * ai + k * ak]
// and B(k, j) = b[k * bk + j * bj] (LDS arrays with padded strides).
template <int RM, int RN>
__device__ __forceinline__ void mm_acc(float (&acc)[RM][RN], const float* a, int ai, int ak, const float* b, int bk,
                                       int bj, int r0, int c0, int K) {
  for (int k = 0; k < K; ++k) {
    float av[RM], bv[RN];
#pragma unroll
    for (int i = 0; i < RM; ++i) av[i] = a[(r0 + i) * ai + k * ak];
#pragma unroll
    for (int j = 0; j < RN; ++j) bv[j] = b[k * bk + (c0 + j) * bj];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int j = 0; j < RN; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
  }
}

// Rows [0, 64) x D of a token-major [B, N, H, D] bf16 tensor into an fp32 LDS tile
// (stride D + 1); tokens at or past n_valid read as zeros.
template <int D>
__device__ __forceinline__ void load_rows(float* dst, const __bf16* src, const GdnParams& p, int b, int h, int t0,
                                          int n_valid) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  for (int e = threadIdx.x; e < kC * D / 8; e += kThr) {
    const int i = e / (D / 8), c = (e % (D / 8)) * 8;
    bf16x8 x = {};
    if (i < n_valid)
      x = *reinterpret_cast<const bf16x8*>(src + ((static_cast<size_t>(b) * p.N + t0 + i) * p.H + h) * D + c);
#pragma unroll
    for (int u = 0; u < 8; ++u) dst[i * (D + 1) + c + u] = bf(x[u]);
  }
}

// ---- gdn_prep: per block, log gates, T, W = T diag(gam) K and Up = T V -------------------
template <int D>
__global__ __launch_bounds__(kThr) void gdn_prep(GdnParams p) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* Ks = sm;                                // [64][D + 1]
  float* Vs = Ks + kC * (D + 1);                 // [64][D + 1]
  float* L = Vs + kC * (D + 1);                  // [64][65]: beta_i A_ij (j < i)
  float* X = L + kC * 65;                        // [64][65]: L^-1, then T
  float* g = X + kC * 65;                        // [64] log cumulative gates
  float* bet = g + kC;                           // [64]
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int t0 = blk * kC, n_valid = min(kC, p.N - t0);
  const size_t bh = static_cast<size_t>(b) * p.H + h;

  load_rows<D>(Ks, static_cast<const __bf16*>(p.k), p, b, h, t0, n_valid);
  load_rows<D>(Vs, static_cast<const __bf16*>(p.v), p, b, h, t0, n_valid);
  if (tid < kC) {                                // padded tokens: alpha = 1, beta = 0 (no effect)
    const bool ok = tid < n_valid;
    g[tid] = ok ? __logf(p.alpha[bh * p.N + t0 + tid]) : 0.f;
    bet[tid] = ok ? p.beta[bh * p.N + t0 + tid] : 0.f;
  }
  __syncthreads();
  if (tid == 0) {                                // prefix sum of 64 logs
    float s = 0.f;
    for (int i = 0; i < kC; ++i) {
      s += g[i];
      g[i] = s;
    }
  }
  __syncthreads();
  if (tid < kC) p.g[bh * (static_cast<size_t>(p.nb) * kC) + t0 + tid] = g[tid];

  // L_ij = beta_i exp(g_i - g_j) k_i.k_j for j < i: 64 x 64, a 4 x 4 tile per thread
  {
    const int r0 = (tid / 16) * 4, c0 = (tid % 16) * 4;
    float acc[4][4] = {};
    mm_acc<4, 4>(acc, Ks, D + 1, 1, Ks, 1, D + 1, r0, c0, D);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = r0 + i, c = c0 + j;
        L[r * 65 + c] = c < r ? bet[r] * __expf(g[r] - g[c]) * acc[i][j] : 0.f;
      }
  }
  __syncthreads();
  // X = (I + L)^-1 by forward substitution. Column j depends only on itself:
  // X_jj = 1, X_ij = -sum_{j <= k < i} L_ik X_kj (i > j), so thread j solves column j.
  if (tid < kC) {
    const int j = tid;
    for (int r = 0; r <= j; ++r) X[r * 65 + j] = r == j ? 1.f : 0.f;
    for (int i = j + 1; i < kC; ++i) {
      float s = 0.f;
      for (int k = j; k < i; ++k) s = fmaf(L[i * 65 + k], X[k * 65 + j], s);
      X[i * 65 + j] = -s;
    }
  }
  __syncthreads();
  // T = X diag(beta)
  for (int e = tid; e < kC * kC; e += kThr) {
    const int r = e / kC, c = e % kC;
    X[r * 65 + c] *= bet[c];
  }
  __syncthreads();
  // W = T diag(exp g) K and Up = T V: 64 x D each, rows r0..r0+3, columns c0..c0+RN-1
  constexpr int RN = D / 16;
  const int r0 = (tid / 16) * 4, c0 = (tid % 16) * RN;
  float* W = p.W + (bh * p.nb + blk) * static_cast<size_t>(kC) * D;
  float* Up = p.Up + (bh * p.nb + blk) * static_cast<size_t>(kC) * D;
  {
    float acc[4][RN] = {};
    mm_acc<4, RN>(acc, X, 65, 1, Vs, D + 1, 1, r0, c0, kC);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < RN; ++j) Up[(r0 + i) * D + c0 + j] = acc[i][j];
  }
  __syncthreads();
  for (int e = tid; e < kC * D; e += kThr) {     // K rows scaled by gam_j (in place)
    const int r = e / D, c = e % D;
    Ks[r * (D + 1) + c] *= __expf(g[r]);
  }
  __syncthreads();
  {
    float acc[4][RN] = {};
    mm_acc<4, RN>(acc, X, 65, 1, Ks, D + 1, 1, r0, c0, kC);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < RN; ++j) W[(r0 + i) * D + c0 + j] = acc[i][j];
  }
}

// ---- gdn_scan: the state through the blocks, rows [r0, r0 + 16) of S per workgroup ---------
template <int D>
__global__ __launch_bounds__(kThr) void gdn_scan(GdnParams p) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  constexpr int R = kGdnScanRows;
  float* Ss = sm;                                // [R][D + 1]   state rows
  float* Ws = Ss + R * (D + 1);                  // [64][D + 1]  W of the block
  float* Ks = Ws + kC * (D + 1);                 // [64][D + 1]  K scaled by exp(g_C - g_i)
  float* Us = Ks + kC * (D + 1);                 // [64][R + 1]  U rows of this slice
  float* g = Us + kC * (R + 1);                  // [64]
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int rs = split * R;
  const size_t bh = static_cast<size_t>(b) * p.H + h;

  for (int e = tid; e < R * D; e += kThr) {
    const int r = e / D, c = e % D;
    Ss[r * (D + 1) + c] = p.state_in != nullptr ? p.state_in[(bh * D + rs + r) * D + c] : 0.f;
  }
  for (int blk = 0; blk < p.nb; ++blk) {
    const int t0 = blk * kC, n_valid = min(kC, p.N - t0);
    __syncthreads();                             // Ss final for this block; LDS tiles free
    float* Sst = p.Sst + (bh * p.nb + blk) * static_cast<size_t>(D) * D;
    for (int e = tid; e < R * D; e += kThr) {
      const int r = e / D, c = e % D;
      Sst[(rs + r) * D + c] = Ss[r * (D + 1) + c];
    }
    const float* W = p.W + (bh * p.nb + blk) * static_cast<size_t>(kC) * D;
    for (int e = tid; e < kC * D; e += kThr) Ws[(e / D) * (D + 1) + e % D] = W[e];
    load_rows<D>(Ks, static_cast<const __bf16*>(p.k), p, b, h, t0, n_valid);
    if (tid < kC) g[tid] = p.g[bh * (static_cast<size_t>(p.nb) * kC) + t0 + tid];
    __syncthreads();
    const float gC = g[kC - 1];
    // U[i][r] = Up[i][rs + r] - sum_d W[i][d] S[r][d]: 64 x R, 4 per thread
    {
      const int i = tid / (R / 4), r0 = (tid % (R / 4)) * 4;
      float acc[1][4] = {};
      mm_acc<1, 4>(acc, Ws, D + 1, 1, Ss, 1, D + 1, i, r0, D);
      const float* Up = p.Up + (bh * p.nb + blk) * static_cast<size_t>(kC) * D;
      float* U = p.U + (bh * p.nb + blk) * static_cast<size_t>(kC) * D;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float u = Up[i * D + rs + r0 + j] - acc[0][j];
        Us[i * (R + 1) + r0 + j] = u;
        U[i * D + rs + r0 + j] = u;
      }
    }
    for (int e = tid; e < kC * D; e += kThr) {   // K rows times exp(g_C - g_i)
      const int r = e / D, c = e % D;
      Ks[r * (D + 1) + c] *= __expf(gC - g[r]);
    }
    __syncthreads();
    // S[r][c] = exp(g_C) S[r][c] + sum_i U[i][r] Ks[i][c]: R x D, R*D/256 per thread
    {
      constexpr int CN = R * D / kThr;           // columns per thread (one row each)
      const int r = tid / (D / CN), c0 = (tid % (D / CN)) * CN;
      float acc[1][CN];
      const float dec = __expf(gC);
#pragma unroll
      for (int j = 0; j < CN; ++j) acc[0][j] = dec * Ss[r * (D + 1) + c0 + j];
      mm_acc<1, CN>(acc, Us, 1, R + 1, Ks, D + 1, 1, r, c0, kC);
      __syncthreads();                           // every thread has read the old rows
#pragma unroll
      for (int j = 0; j < CN; ++j) Ss[r * (D + 1) + c0 + j] = acc[0][j];
    }
  }
  __syncthreads();
  for (int e = tid; e < R * D; e += kThr) {
    const int r = e / D, c = e % D;
    p.state_out[(bh * D + rs + r) * D + c] = Ss[r * (D + 1) + c];
  }
}

// ---- gdn_out: O = diag(exp g) Q S0^T + ((Q K^T) o M) U, one half of the Dv columns --------
template <int D>
__global__ __launch_bounds__(kThr) void gdn_out(GdnParams p) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  constexpr int DH = D / 2;
  float* Qs = sm;                                // [64][D + 1]
  float* Ks = Qs + kC * (D + 1);                 // [64][D + 1]
  float* P = Ks + kC * (D + 1);                  // [64][65]
  float* Ss = P + kC * 65;                       // [DH][D + 1]  block-start state rows of this half
  float* Us = Ss + DH * (D + 1);                 // [64][DH + 1]
  float* g = Us + kC * (DH + 1);                 // [64]
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z >> 1, half = blockIdx.z & 1, tid = threadIdx.x;
  const int t0 = blk * kC, n_valid = min(kC, p.N - t0);
  const size_t bh = static_cast<size_t>(b) * p.H + h;

  load_rows<D>(Qs, static_cast<const __bf16*>(p.q), p, b, h, t0, n_valid);
  load_rows<D>(Ks, static_cast<const __bf16*>(p.k), p, b, h, t0, n_valid);
  if (tid < kC) g[tid] = p.g[bh * (static_cast<size_t>(p.nb) * kC) + t0 + tid];
  const float* S0 = p.Sst + (bh * p.nb + blk) * static_cast<size_t>(D) * D;
  for (int e = tid; e < DH * D; e += kThr) {
    const int r = e / D, c = e % D;
    Ss[r * (D + 1) + c] = S0[(half * DH + r) * D + c];
  }
  const float* U = p.U + (bh * p.nb + blk) * static_cast<size_t>(kC) * D;
  for (int e = tid; e < kC * DH; e += kThr) {
    const int i = e / DH, c = e % DH;
    Us[i * (DH + 1) + c] = U[i * D + half * DH + c];
  }
  __syncthreads();
  {                                              // P_ij = exp(g_i - g_j) q_i.k_j for j <= i
    const int r0 = (tid / 16) * 4, c0 = (tid % 16) * 4;
    float acc[4][4] = {};
    mm_acc<4, 4>(acc, Qs, D + 1, 1, Ks, 1, D + 1, r0, c0, D);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = r0 + i, c = c0 + j;
        P[r * 65 + c] = c <= r ? __expf(g[r] - g[c]) * acc[i][j] : 0.f;
      }
  }
  __syncthreads();
  constexpr int RN = DH / 16;
  const int r0 = (tid / 16) * 4, c0 = (tid % 16) * RN;
  float acc[4][RN] = {};
  mm_acc<4, RN>(acc, Qs, D + 1, 1, Ss, 1, D + 1, r0, c0, D);       // Q S0^T
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float e = __expf(g[r0 + i]);
#pragma unroll
    for (int j = 0; j < RN; ++j) acc[i][j] *= e;
  }
  mm_acc<4, RN>(acc, P, 65, 1, Us, DH + 1, 1, r0, c0, kC);          // + P U
  __bf16* out = static_cast<__bf16*>(p.out);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + i;
    if (r >= n_valid) continue;
#pragma unroll
    for (int j = 0; j < RN; ++j)
      out[((static_cast<size_t>(b) * p.N + t0 + r) * p.H + h) * D + half * DH + c0 + j] =
          static_cast<__bf16>(acc[i][j]);
  }
}

template <int D>
constexpr size_t prep_lds() { return (2 * kC * (D + 1) + 2 * kC * 65 + 2 * kC) * sizeof(float); }
template <int D>
constexpr size_t scan_lds() {
  return (kGdnScanRows * (D + 1) + 2 * kC * (D + 1) + kC * (kGdnScanRows + 1) + kC) * sizeof(float);
}
template <int D>
constexpr size_t out_lds() {
  return (2 * kC * (D + 1) + kC * 65 + (D / 2) * (D + 1) + kC * (D / 2 + 1) + kC) * sizeof(float);
}

template <int D>
hipError_t launch_gdn_d(const GdnParams& p, hipStream_t st) {
  static_assert(prep_lds<D>() <= 160 * 1024 && scan_lds<D>() <= 160 * 1024 && out_lds<D>() <= 160 * 1024,
                "LDS budget");
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gdn_prep<D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(prep_lds<D>()));
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gdn_scan<D>), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(scan_lds<D>()));
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(gdn_out<D>), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(out_lds<D>()));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gdn_prep<D>, dim3(p.nb, p.H, p.B), dim3(kThr), prep_lds<D>(), st, p);
  hipLaunchKernelGGL(gdn_scan<D>, dim3(D / kGdnScanRows, p.H, p.B), dim3(kThr), scan_lds<D>(), st, p);
  hipLaunchKernelGGL(gdn_out<D>, dim3(p.nb, p.H, 2 * p.B), dim3(kThr), out_lds<D>(), st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn_forward(const GdnParams& p, hipStream_t st) {
  if (p.N <= 0) return hipSuccess;
  return p.D == 128 ? launch_gdn_d<128>(p, st) : launch_gdn_d<64>(p, st);
}

}  // namespace sa
