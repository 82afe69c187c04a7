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
// U), gdn_out (every block independently: the outputs). Products whose inputs are bf16
// (K K^T, Q K^T) run on the bf16 MFMA with exact products; those feeding the state
// recurrence (T V, T diag(gam) K, and the scan's two) on the fp32 MFMA; gdn_out's
// remaining products on the bf16 MFMA with fp32 operands split into bf16 hi/lo pairs
// (an output's error stays near 2^-16 of its terms and does not feed back). Inputs and
// outputs are bf16, the state fp32.
#include "sa_internal.h"

#include <mutex>

namespace sa {
namespace {

constexpr int kC = kGdnBlock;        // tokens per block
constexpr int kThr = 256;
constexpr int kCL = kC + 4;          // padded row of a 64-wide LDS tile

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

// Storage order of the scan's per-block operands: each of the scan's float4 loads reads
// 1 KB contiguously (lane l takes floats [4 l, 4 l + 4) of its load's run). Lane l = lr +
// 16 lq of wave w (columns [D/4 w, D/4 (w + 1)), NT = D / 64 tiles of 16) loads
//   W     load (mt, t): W[16 mt + lr][D/4 w + 16 t + 4 lq + e]
//   Kt^T  load (t, u):  Kt^T[D/4 w + 16 t + lr][16 lq + 4 u + e]
//   Up^T  load u of row slice r / 16: Up^T[16 (r / 16) + lr][16 lq + 4 u + e]
template <int D>
__device__ __forceinline__ int w_index(int i, int k) {      // W[i][k], i token, k column
  constexpr int NT = D / 64;
  const int w = k / (D / 4), cc = k % (D / 4);
  const int l = (i & 15) + 16 * ((cc & 15) >> 2);
  return ((((w * 4 + (i >> 4)) * NT + (cc >> 4)) * 64 + l) << 2) + (cc & 3);
}
template <int D>
__device__ __forceinline__ int kt_index(int c, int i) {     // Kt^T[c][i], c column, i token
  constexpr int NT = D / 64;
  const int w = c / (D / 4), cc = c % (D / 4);
  const int l = (cc & 15) + 16 * (i >> 4);
  return ((((w * NT + (cc >> 4)) * 4 + ((i & 15) >> 2)) * 64 + l) << 2) + (i & 3);
}
__device__ __forceinline__ int up_index(int r, int i) {     // Up^T[r][i], r row of the state, i token
  const int l = (r & 15) + 16 * (i >> 4);
  return ((((r >> 4) * 4 + ((i & 15) >> 2)) * 64 + l) << 2) + (i & 3);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void split_bf16(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 t = static_cast<__bf16>(x[e]);
    hi[e] = t;
    lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(t));
  }
}
// x = t1 + t2 + t3 to 2^-24 |x|: each part is the bf16 rounding of what the previous ones
// leave (x - t1 and x - t1 - t2 are exact in fp32)
__device__ __forceinline__ void split3_bf16(const float (&x)[8], bf16x8& t1, bf16x8& t2, bf16x8& t3) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float r = x[e];
    const __bf16 a = static_cast<__bf16>(r);
    r -= static_cast<float>(a);
    const __bf16 b = static_cast<__bf16>(r);
    r -= static_cast<float>(b);
    t1[e] = a;
    t2[e] = b;
    t3[e] = static_cast<__bf16>(r);
  }
}
__device__ __forceinline__ void unpack8(const float4& a, const float4& b, float (&x)[8]) {
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---- gdn_prep: per block, log gates, T, W = T diag(gam) K, Up = T V, Kt ---------------------
// K K^T on v_mfma_f32_32x32x16_bf16 (bf16 inputs: exact products); T by a blocked inverse
// (substitution within 16 x 16 blocks, merges on v_mfma_f32_16x16x4_f32: lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16] and receives C[4 (l / 16) + j][l % 16]); T V and
// T diag(gam) K, which feed the state recurrence, on the bf16 MFMA with T split into three
// bf16 parts (fp32 accuracy). K^T and V^T are staged transposed in LDS (rows of 64 + 8
// bf16, conflict-free).
template <int D>
__global__ __launch_bounds__(kThr) void gdn_prep(GdnParams p) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  constexpr int VL = kC + 8;                     // bf16 row of KT, VT
  float* L = sm;                                 // [64][kCL]: beta_i A_ij (j < i)
  float* X = L + kC * kCL;                       // [64][kCL]: T
  float* g = X + kC * kCL;                       // [64] log cumulative gates
  float* bet = g + kC;                           // [64]
  float* gam = bet + kC;                         // [64] cumulative gates exp(g)
  __bf16* KT = reinterpret_cast<__bf16*>(gam + kC);  // [D][VL]: K^T
  __bf16* VT = KT + D * VL;                      // [D][VL]: V^T
  float* Mb = reinterpret_cast<float*>(VT + D * VL);  // [32][36]: products of the inverse's merges
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int l = tid & 63, w = tid >> 6, lc = l & 31, hf = l >> 5;
  const int t0 = blk * kC, n_valid = min(kC, p.N - t0);
  const size_t bh = static_cast<size_t>(b) * p.H + h;
  const size_t rs = static_cast<size_t>(p.H) * D;
  const size_t base = (static_cast<size_t>(b) * p.N + t0) * rs + static_cast<size_t>(h) * D;
  const __bf16* kb = static_cast<const __bf16*>(p.k) + base;
  const __bf16* vb = static_cast<const __bf16*>(p.v) + base;
  const size_t boff = (bh * p.nb + blk) * static_cast<size_t>(kC) * D;

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
    gam[tid] = __expf(s);
    p.g[bh * (static_cast<size_t>(p.nb) * kC) + t0 + tid] = s;
  }
  for (int e = tid; e < kC * kCL / 4; e += kThr) st4(X + 4 * e, make_float4(0.f, 0.f, 0.f, 0.f));
  // K^T and V^T: a thread takes tokens (2 m, 2 m + 1) of 8 columns and writes packed pairs
#pragma unroll
  for (int e = tid; e < 32 * (D / 8); e += kThr) {
    const int m = e & 31, c = (e >> 5) * 8, i0 = 2 * m;
    bf16x8 k0 = {}, k1 = {}, v0 = {}, v1 = {};
    if (i0 < n_valid) {
      k0 = *reinterpret_cast<const bf16x8*>(kb + i0 * rs + c);
      v0 = *reinterpret_cast<const bf16x8*>(vb + i0 * rs + c);
    }
    if (i0 + 1 < n_valid) {
      k1 = *reinterpret_cast<const bf16x8*>(kb + (i0 + 1) * rs + c);
      v1 = *reinterpret_cast<const bf16x8*>(vb + (i0 + 1) * rs + c);
    }
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      *reinterpret_cast<bf16x2*>(KT + (c + u) * VL + i0) = bf16x2{k0[u], k1[u]};
      *reinterpret_cast<bf16x2*>(VT + (c + u) * VL + i0) = bf16x2{v0[u], v1[u]};
    }
  }
  // K K^T, one 32 x 32 quadrant per wave (the one above the diagonal is not needed)
  f32x16 acc = {};
  const int qr = w >> 1, qc = w & 1;
  if (w != 1) {
    const int ir = 32 * qr + lc, jr = 32 * qc + lc;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8 a = ir < n_valid ? *reinterpret_cast<const bf16x8*>(kb + ir * rs + 16 * s + 8 * hf) : bf16x8{};
      const bf16x8 bb = jr < n_valid ? *reinterpret_cast<const bf16x8*>(kb + jr * rs + 16 * s + 8 * hf) : bf16x8{};
      acc = mfma_bf16(a, bb, acc);
    }
  }
  __syncthreads();
  if (w != 1) {                                  // L_ij = beta_i exp(g_i - g_j) k_i.k_j for j < i
    const int j = 32 * qc + lc;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * qr + 8 * (r >> 2) + 4 * hf + (r & 3);
      L[i * kCL + j] = j < i ? bet[i] * __expf(g[i] - g[j]) * acc[r] : 0.f;
    }
  }
  __syncthreads();
  // X = (I + L)^-1 (T = X diag(beta)), blocked over 16 x 16 blocks. (1) Each diagonal block
  // by forward substitution: lane c < 16 of wave w solves column c of block w in registers
  // (X_ii = 1, X_ij = -sum_{j <= k < i} L_ik X_kj). (2) The lower-left block of each 32 x 32
  // diagonal block, and (3) that of the whole, as -X_B L_BA X_A for [[A, 0], [BA, B]], on
  // the fp32 MFMA through the buffer Mb. The upper blocks stay zero.
  if (l < 16) {
    const int o = 16 * w, c = l;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int k = 0; k < i; k += 2) {
        s0 = fmaf(L[(o + i) * kCL + o + k], x[k], s0);
        if (k + 1 < i) s1 = fmaf(L[(o + i) * kCL + o + k + 1], x[k + 1], s1);
      }
      x[i] = i == c ? 1.f : (i < c ? 0.f : -(s0 + s1));
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) X[(o + i) * kCL + o + c] = x[i];
  }
  const int lr = l & 15, q = l >> 4;
  // 16 x 16 x 16 product on the fp32 MFMA: C += A B with A(r, k), B(k, c) read through
  // accessors; k-step s of lane quad q is k = 4 s + q
  auto mm16 = [&](f32x4 acc, auto A, auto B, int K) {
    for (int s = 0; s < K / 4; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A(lr, 4 * s + q), B(4 * s + q, lr), acc, 0, 0, 0);
    return acc;
  };
  __syncthreads();
  if (w < 2) {                                   // (2) blocks (2w, 2w + 1)
    const int a0 = 32 * w, b0 = 32 * w + 16;
    f32x4 m = mm16(f32x4{}, [&](int r, int k) { return L[(b0 + r) * kCL + a0 + k]; },
                   [&](int k, int c) { return X[(a0 + k) * kCL + a0 + c]; }, 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) Mb[(16 * w + 4 * q + j) * 36 + lr] = m[j];
  }
  __syncthreads();
  if (w < 2) {
    const int a0 = 32 * w, b0 = 32 * w + 16;
    f32x4 x = mm16(f32x4{}, [&](int r, int k) { return X[(b0 + r) * kCL + b0 + k]; },
                   [&](int k, int c) { return Mb[(16 * w + k) * 36 + c]; }, 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) X[(b0 + 4 * q + j) * kCL + a0 + lr] = -x[j];
  }
  __syncthreads();
  const int tr = 16 * (w >> 1), tc = 16 * (w & 1);   // (3) this wave's 16 x 16 tile of 32 x 32
  {
    f32x4 m = mm16(f32x4{}, [&](int r, int k) { return L[(32 + tr + r) * kCL + k]; },
                   [&](int k, int c) { return X[k * kCL + tc + c]; }, 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) Mb[(tr + 4 * q + j) * 36 + tc + lr] = m[j];
  }
  __syncthreads();
  {
    f32x4 x = mm16(f32x4{}, [&](int r, int k) { return X[(32 + tr + r) * kCL + 32 + k]; },
                   [&](int k, int c) { return Mb[k * 36 + tc + c]; }, 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) X[(32 + tr + 4 * q + j) * kCL + tc + lr] = -x[j];
  }
  {
    // Kt^T = (diag(exp(g_C - g)) K)^T in the scan's load order (kt_index), written as
    // float4s: entries 4 f .. 4 f + 3 are load (f / 64) of their wave's run, lane f % 64,
    // i.e. four consecutive tokens of one column (one 8-byte read of K^T)
    const float gC = g[kC - 1];
    constexpr int NT = D / 64;
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    for (int f = tid; f < kC * D / 4; f += kThr) {
      const int l2 = f & 63, run = f >> 6, u = run & 3, t = (run >> 2) % NT, ww = run / (4 * NT);
      const int c = ww * (D / 4) + 16 * t + (l2 & 15), i = 16 * (l2 >> 4) + 4 * u;
      const bf16x4 kk = *reinterpret_cast<const bf16x4*>(KT + c * VL + i);
      st4(p.Kt + boff + 4 * f, make_float4(__expf(gC - g[i]) * static_cast<float>(kk[0]),
                                           __expf(gC - g[i + 1]) * static_cast<float>(kk[1]),
                                           __expf(gC - g[i + 2]) * static_cast<float>(kk[2]),
                                           __expf(gC - g[i + 3]) * static_cast<float>(kk[3])));
    }
  }
  __syncthreads();
  // Up = T V and W^T = K^T (T diag(gam))^T on v_mfma_f32_32x32x16_bf16. T enters as three
  // bf16 parts (split3: t1 + t2 + t3 = T to 2^-24), V and K are bf16: every product is exact
  // and the sums are fp32, as for an fp32 product. Tiles of 32 x 32: (token tile it, column
  // tile dt), wave w takes tiles w, w + 4, ...; the T rows this lane reads serve as the A
  // operand of Up and (scaled by gam) the B operand of W^T.
  for (int tile = w; tile < 2 * (D / 32); tile += 4) {
    const int it = tile & 1, dt = tile >> 1;
    const int ti = 32 * it + lc, dc = 32 * dt + lc;
    f32x16 au = {}, aw = {};
#pragma unroll
    for (int ks = 0; ks < kC / 16; ++ks) {
      const int j0 = 16 * ks + 8 * hf;
      const float4 x0 = ld4(X + ti * kCL + j0), x1 = ld4(X + ti * kCL + j0 + 4);
      float tb[8], tgm[8];
      unpack8(x0, x1, tb);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        tb[e] *= bet[j0 + e];
        tgm[e] = tb[e] * gam[j0 + e];
      }
      bf16x8 u1, u2, u3, g1, g2, g3;
      split3_bf16(tb, u1, u2, u3);
      split3_bf16(tgm, g1, g2, g3);
      const bf16x8 vb = *reinterpret_cast<const bf16x8*>(VT + dc * VL + j0);
      const bf16x8 kb8 = *reinterpret_cast<const bf16x8*>(KT + dc * VL + j0);
      au = mfma_bf16(u3, vb, au);
      au = mfma_bf16(u2, vb, au);
      au = mfma_bf16(u1, vb, au);
      aw = mfma_bf16(kb8, g3, aw);
      aw = mfma_bf16(kb8, g2, aw);
      aw = mfma_bf16(kb8, g1, aw);
    }
    // au: Up[32 it + 8 (r / 4) + 4 hf + r % 4][dc]; aw: W[32 it + lc][32 dt + 8 (r / 4) + 4 hf + r % 4]
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int o = 8 * r4 + 4 * hf;
      st4(p.Up + boff + up_index(dc, 32 * it + o),
          make_float4(au[4 * r4], au[4 * r4 + 1], au[4 * r4 + 2], au[4 * r4 + 3]));
      st4(p.W + boff + w_index<D>(ti, 32 * dt + o),
          make_float4(aw[4 * r4], aw[4 * r4 + 1], aw[4 * r4 + 2], aw[4 * r4 + 3]));
    }
  }
}

// ---- gdn_scan: the state through the blocks, rows [rs, rs + 16) of S per workgroup ----------
// Per block, on the fp32 MFMA (v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16]
// and B[l / 16][l % 16] and receives C[4 (l / 16) + j][l % 16]), with wave w owning the
// columns [D/4 w, D/4 (w + 1)) of the slice:
//   U (64 x 16) = Up - W S^T: wave w forms the partial over its columns (less Up on its
//     own 16 tokens), the four partials meet in LDS (double-buffered: one barrier per block);
//   S'^T = exp(g_C) S^T + Kt^T U on the wave's columns.
// The state is held as S^T in the C layout, which is also the B operand of W S^T (k-step
// (t, j) of lane quad q is column 16 t + 4 q + j): no exchange of the state between waves.
// The reduced U is read back in the B layout of Kt^T U (k-step s of quad q is token
// 16 q + s). Operands of the next block (W, Kt^T, Up^T, its gate) are fetched while the
// current one computes.
template <int D>
__global__ __launch_bounds__(kThr) void gdn_scan(GdnParams p) {
  static_assert(kGdnScanRows == 16, "one 16-row MFMA tile of the state per workgroup");
  constexpr int NT = D / 64;                     // 16-column tiles per wave
  __shared__ __attribute__((aligned(16))) float part[2][4][16][kCL];  // [buffer][wave][row][token]
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int l = tid & 63, w = tid >> 6, lr = l & 15, lq = l >> 4;
  const int rs = split * 16, cw = w * (D / 4);
  const size_t bh = static_cast<size_t>(b) * p.H + h;
  auto boff = [&](int blk) { return (bh * p.nb + blk) * static_cast<size_t>(kC) * D; };

  f32x4 sc[NT];                                  // S[rs + lr][cw + 16 t + 4 lq + j]
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p.state_in != nullptr) v = ld4(p.state_in + (bh * D + rs + lr) * D + cw + 16 * t + 4 * lq);
    sc[t] = f32x4{v.x, v.y, v.z, v.w};
  }
  struct Ops {
    float4 wa[4][NT];                            // W[16 mt + lr][cw + 16 t + 4 lq ..]     (w_index)
    float4 ka[NT][4];                            // Kt^T[cw + 16 t + lr][16 lq + 4 u ..]   (kt_index)
    float4 up;                                   // Up^T[rs + lr][16 w + 4 lq ..]          (up_index)
    float gC;
  };
  auto fetch = [&](int blk, Ops& o) {
    const size_t bo = boff(blk);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t) o.wa[mt][t] = ld4(p.W + bo + ((((w * 4 + mt) * NT + t) * 64 + l) << 2));
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < 4; ++u) o.ka[t][u] = ld4(p.Kt + bo + ((((w * NT + t) * 4 + u) * 64 + l) << 2));
    o.up = ld4(p.Up + bo + (((split * 4 + lq) * 64 + lr + 16 * w) << 2));
    o.gC = p.g[bh * (static_cast<size_t>(p.nb) * kC) + blk * kC + kC - 1];
  };
  // One block: the loads of the next block go out first, then the stores (this block's
  // starting state, later its U^T), the same number in every wave. The memory counter
  // retires in issue order, so a store issued before those loads would have to complete
  // before the current block's operands (loaded one block earlier) count as arrived.
  auto step = [&](int blk, const Ops& cur, Ops& nxt) {
    fetch(min(blk + 1, p.nb - 1), nxt);
    __builtin_amdgcn_sched_barrier(0);
    float* Sst = p.Sst + (bh * p.nb + blk) * static_cast<size_t>(D) * D;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      st4(Sst + (rs + lr) * D + cw + 16 * t + 4 * lq, make_float4(sc[t][0], sc[t][1], sc[t][2], sc[t][3]));
    __builtin_amdgcn_sched_barrier(0);
    // partial of W S^T over this wave's columns: four 16-token tiles
    f32x4 acc[4] = {};
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const float a = j == 0 ? cur.wa[mt][t].x : j == 1 ? cur.wa[mt][t].y : j == 2 ? cur.wa[mt][t].z : cur.wa[mt][t].w;
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sc[t][j], acc[mt], 0, 0, 0);
        }
    // wave w folds -Up of its own token tile into its partial: the four sum to -U
    acc[0] -= w == 0 ? f32x4{cur.up.x, cur.up.y, cur.up.z, cur.up.w} : f32x4{};
    acc[1] -= w == 1 ? f32x4{cur.up.x, cur.up.y, cur.up.z, cur.up.w} : f32x4{};
    acc[2] -= w == 2 ? f32x4{cur.up.x, cur.up.y, cur.up.z, cur.up.w} : f32x4{};
    acc[3] -= w == 3 ? f32x4{cur.up.x, cur.up.y, cur.up.z, cur.up.w} : f32x4{};
    float(*pb)[16][kCL] = part[blk & 1];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      st4(&pb[w][lr][16 * mt + 4 * lq], make_float4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]));
    __syncthreads();
    // U[16 lq + s][rs + lr] = Up - W S^T = -(sum of the partials)
    float ub[16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float4 x = ld4(&pb[v][lr][16 * lq + 4 * u]);
        sum.x -= x.x; sum.y -= x.y; sum.z -= x.z; sum.w -= x.w;
      }
      ub[4 * u] = sum.x; ub[4 * u + 1] = sum.y; ub[4 * u + 2] = sum.z; ub[4 * u + 3] = sum.w;
    }
    {                                            // U^T for gdn_out: wave w writes tokens 16 lq + 4 w ..
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = w == 0 ? ub[e] : w == 1 ? ub[4 + e] : w == 2 ? ub[8 + e] : ub[12 + e];
      st4(p.U + boff(blk) + (rs + lr) * kC + 16 * lq + 4 * w, make_float4(x[0], x[1], x[2], x[3]));
    }
    const float dec = __expf(cur.gC);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4 a = sc[t] * dec;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.ka[t][u].x, ub[4 * u], a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.ka[t][u].y, ub[4 * u + 1], a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.ka[t][u].z, ub[4 * u + 2], a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_16x16x4f32(cur.ka[t][u].w, ub[4 * u + 3], a, 0, 0, 0);
      }
      sc[t] = a;
    }
  };
  Ops opa, opb;                                  // operands of even and odd blocks
  fetch(0, opa);
  for (int blk = 0; blk < p.nb; blk += 2) {
    step(blk, opa, opb);
    if (blk + 1 >= p.nb) break;
    step(blk + 1, opb, opa);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
    st4(p.state_out + (bh * D + rs + lr) * D + cw + 16 * t + 4 * lq, make_float4(sc[t][0], sc[t][1], sc[t][2], sc[t][3]));
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
constexpr size_t prep_lds() { return (2 * kC * kCL + 3 * kC + 32 * 36) * sizeof(float) + 2 * D * (kC + 8) * sizeof(__bf16); }

template <int D>
hipError_t launch_gdn_d(const GdnParams& p, hipStream_t st) {
  static_assert(prep_lds<D>() <= 160 * 1024, "LDS budget");
  static_assert(D % 64 == 0, "scan tiles");
  // gdn_prep takes more than 64 KB of dynamic LDS. Set on every call: a host-side call, safe
  // from any thread and on whichever device is current.
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gdn_prep<D>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(prep_lds<D>()));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gdn_prep<D>, dim3(p.nb, p.H, p.B), dim3(kThr), prep_lds<D>(), st, p);
  hipLaunchKernelGGL(gdn_scan<D>, dim3(D / kGdnScanRows, p.H, p.B), dim3(kThr), 0, st, p);
  hipLaunchKernelGGL(gdn_out<D>, dim3(p.nb, p.H, p.B), dim3(kThr), 0, st, p);
  return hipGetLastError();
}

// state_out = state_in (zeros when state_in is null): the whole call when there are no
// tokens. A kernel rather than a memset or copy node, so a captured call holds kernels only.
__global__ __launch_bounds__(kThr) void gdn_state_pass(const float4* in, float4* out, size_t n4) {
  const size_t i = static_cast<size_t>(blockIdx.x) * kThr + threadIdx.x;
  if (i < n4) out[i] = in != nullptr ? in[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

hipError_t launch_gdn_state_pass(const float* in, float* out, size_t n, hipStream_t st) {
  const size_t n4 = n / 4;                        // n = B H D D, a multiple of 4096
  if (n4 == 0 || in == out) return hipSuccess;
  hipLaunchKernelGGL(gdn_state_pass, dim3(static_cast<unsigned>((n4 + kThr - 1) / kThr)), dim3(kThr), 0, st,
                     reinterpret_cast<const float4*>(in), reinterpret_cast<float4*>(out), n4);
  return hipGetLastError();
}

hipError_t launch_gdn_forward(const GdnParams& p, hipStream_t st) {
  if (p.N <= 0) return hipSuccess;
  return p.D == 128 ? launch_gdn_d<128>(p, st) : launch_gdn_d<64>(p, st);
}

// ---- scratch for the workspace-free forward ---------------------------------------------------
// A fixed device array stands in for the caller's workspace (sa_gdn_forward_noalloc). Each GPU
// the library runs on holds its own copy, placed when the code object loads there and kept
// until the process ends. Host code never uses the array's name as an address: it takes each
// device's address once from hipGetSymbolAddress and passes that to the kernels.
static_assert(kGdnScratchBytes % 256 == 0, "scratch size");
static __device__ __align__(256) char scratch[kGdnScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t gdn_scratch_address(hipStream_t st, void** out) {
  int dev = 0;
  hipError_t e = st != nullptr ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {          // first call on this device: with it current
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255u) != 0) return hipErrorInvalidValue;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace sa
