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
// W, Up and a bf16 copy of K^T), gdn_scan (the only sequential part: the state through the
// blocks, in row slices of S, which evolve independently; records each block's starting
// state and U), gdn_out (every block independently: the outputs). All products but the
// merges of T's blocked inverse (fp32 MFMA) run on the bf16 MFMA with fp32 accumulation.
// Products whose inputs are bf16 (K K^T, Q K^T) are exact;
// those feeding the state recurrence (T V, T diag(gam) K, and the scan's W S^T and
// K^T diag(gam_C / gam) U) take each fp32 operand as three bf16 parts (t1 + t2 + t3 = x to
// 2^-24 |x|) and keep every partial product down to 2^-24 of the whole, which matches an
// fp32 product; gdn_out's remaining products split fp32 operands into bf16 hi/lo pairs (an
// output's error stays near 2^-16 of its terms and does not feed back). Inputs and outputs
// are bf16, the state fp32.
#include "sa_internal.h"

#include <mutex>

namespace sa {
namespace {

constexpr int kC = kGdnBlock;        // tokens per block
constexpr int kThr = 256;
constexpr int kCL = kC + 4;          // padded row of a 64-wide LDS tile

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

// Storage order of the scan's per-block operands. The scan keeps the state slice in the
// accumulator layout of a 16 x 16 MFMA tile and feeds it back as the B operand of the next
// block's W S^T, so a lane quad q of wave w (columns [D/4 w, D/4 (w + 1)), NT = D / 64) holds
// the KQ = 4 NT consecutive columns D/4 w + KQ q + e, e < KQ; accumulator tile t, row 4 q + j
// is column D/4 w + KQ q + 4 t + j. Every operand run below is 64 lanes of contiguous
// elements, read by one load per lane.
//   W, three bf16 parts (run (w, mt, part)): lane l = r + 16 q holds W[16 mt + r][D/4 w + KQ q + e]
//   K^T, bf16 (run (w, t, s)): lane l = m + 16 q holds K^T[D/4 w + KQ (m / 4) + 4 t + m % 4][32 s + 8 q + e]
//   Up^T, fp32 (load u of row slice r / 16): Up^T[16 (r / 16) + lr][16 lq + 4 u + e]
template <int D>
__device__ __forceinline__ int w3_index(int i, int k) {     // part 0 of W[i][k]; part p at + p * 64 KQ
  constexpr int KQ = D / 16;
  const int w = k / (D / 4), cc = k % (D / 4);
  const int l = (i & 15) + 16 * (cc / KQ);
  return (((w * 4 + (i >> 4)) * 3 * 64 + l) * KQ) + cc % KQ;
}
__device__ __forceinline__ int up_index(int r, int i) {     // Up^T[r][i], r row of the state, i token
  const int l = (r & 15) + 16 * (i >> 4);
  return ((((r >> 4) * 4 + ((i & 15) >> 2)) * 64 + l) << 2) + (i & 3);
}
// Storage order of what the scan leaves for gdn_out, in gdn_out's operand order (32-row
// tiles of the 32x32x16 MFMA, lane l = lc + 32 hf takes row 32 tile + lc): every load of
// gdn_out reads 64 lanes x 16 bytes contiguously.
//   block state S0[r][k], run (tile, s, half): lane's k = 16 s + 8 hf + 4 half + e
//   U^T[r][t], run (tile, jt, s2, half):       lane's t = 32 jt + 16 s2 + 4 hf + 8 half + e
template <int D>
__device__ __forceinline__ int s0_index(int r, int k) {      // k a multiple of 4: 4 floats from here
  constexpr int KS = D / 16;
  const int l = (r & 31) + 32 * ((k >> 3) & 1);
  return ((((r >> 5) * KS + (k >> 4)) * 2 + ((k >> 2) & 1)) * 64 + l) * 4;
}
__device__ __forceinline__ int ut_index(int r, int t) {      // t a multiple of 4: 4 floats from here
  const int l = (r & 31) + 32 * ((t >> 2) & 1);
  return (((((r >> 5) * 2 + (t >> 5)) * 2 + ((t >> 4) & 1)) * 2 + ((t >> 3) & 1)) * 64 + l) * 4;
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
template <int N> struct BfVec;
template <> struct BfVec<4> { typedef __bf16 type __attribute__((ext_vector_type(4))); };
template <> struct BfVec<8> { typedef __bf16 type __attribute__((ext_vector_type(8))); };
// x = t1 + t2 + t3 to 2^-24 |x| for N values (as split3_bf16)
template <int N>
__device__ __forceinline__ void split3(const float* x, typename BfVec<N>::type& t1, typename BfVec<N>::type& t2,
                                       typename BfVec<N>::type& t3) {
#pragma unroll
  for (int e = 0; e < N; ++e) {
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
// 16 x 16 tile on the bf16 MFMA with KQ = 8 (v_mfma_f32_16x16x32_bf16) or 4
// (v_mfma_f32_16x16x16_bf16) depth values per lane: lane l supplies A[l % 16][KQ (l / 16) + e]
// and B[KQ (l / 16) + e][l % 16], e < KQ, and receives C[4 (l / 16) + j][l % 16]
template <int KQ>
__device__ __forceinline__ f32x4 mfma16(const typename BfVec<KQ>::type& a, const typename BfVec<KQ>::type& b,
                                        const f32x4& c) {
  if constexpr (KQ == 8) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  } else {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
  }
}
__device__ __forceinline__ void unpack8(const float4& a, const float4& b, float (&x)[8]) {
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---- gdn_prep: per block, log gates, T, W = T diag(gam) K, Up = T V, K^T ---------------------
// K K^T on v_mfma_f32_32x32x16_bf16 (bf16 inputs: exact products); T by a blocked inverse
// (substitution within 16 x 16 blocks, merges on v_mfma_f32_16x16x4_f32: lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16] and receives C[4 (l / 16) + j][l % 16]); T V and
// T diag(gam) K, which feed the state recurrence, on the bf16 MFMA with T split into three
// bf16 parts (fp32 accuracy); W leaves as three bf16 parts, K^T as a bf16 copy, both in the
// scan's operand order. K^T and V^T are staged transposed in LDS (rows of 64 + 8 bf16,
// conflict-free).
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
    // K^T in bf16 for the scan's state update, in its operand order: run (w, t, s) of 64
    // lanes x 8 tokens (16 bytes per lane, straight from the transposed copy in LDS)
    constexpr int NT = D / 64;
    __bf16* ktb = static_cast<__bf16*>(p.Kt) + boff;
    for (int f = tid; f < kC * D / 8; f += kThr) {
      const int l2 = f & 63, run = f >> 6, s = run & 1, t = (run >> 1) % NT, ww = run / (2 * NT);
      const int m = l2 & 15, c = ww * (D / 4) + 4 * NT * (m >> 2) + 4 * t + (m & 3);
      *reinterpret_cast<bf16x8*>(ktb + 8 * f) = *reinterpret_cast<const bf16x8*>(KT + c * VL + 32 * s + 8 * (l2 >> 4));
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
      // W in three bf16 parts (the scan's A operands): four consecutive columns, 8 bytes per part
      const float wv[4] = {aw[4 * r4], aw[4 * r4 + 1], aw[4 * r4 + 2], aw[4 * r4 + 3]};
      typename BfVec<4>::type w1, w2, w3;
      split3<4>(wv, w1, w2, w3);
      __bf16* wb = static_cast<__bf16*>(p.W) + 3 * boff + w3_index<D>(ti, 32 * dt + o);
      *reinterpret_cast<typename BfVec<4>::type*>(wb) = w1;
      *reinterpret_cast<typename BfVec<4>::type*>(wb + 64 * (D / 16)) = w2;
      *reinterpret_cast<typename BfVec<4>::type*>(wb + 128 * (D / 16)) = w3;
    }
  }
}

// ---- gdn_scan: the state through the blocks, rows [rs, rs + 16) of S per workgroup ----------
// Per block, on the bf16 MFMA (mfma16), with wave w owning the columns [D/4 w, D/4 (w + 1))
// of the slice:
//   U (64 x 16) = Up - W S^T: wave w forms the partial over its columns (less Up on its own
//     16 tokens) from W's three bf16 parts and the slice's three (t1 + t2 + t3 = x to 2^-24 |x|;
//     the six products down to 2^-24 of the whole, accumulated in fp32); the four partials
//     meet in LDS (double-buffered: one barrier per block);
//   S'^T = exp(g_C) S^T + K^T diag(exp(g_C - g)) U on the wave's columns: K is bf16 (exact
//     products) and the scaled U enters as three bf16 parts.
// The state is held as S^T in the accumulator layout, which is also the B operand of the next
// block's W S^T (lane quad q holds columns KQ q + e of the wave's range): no exchange of the
// state between waves. The reduced U is read back in the B layout of the state update (tokens
// 32 s + 8 q + e). Operands of the next block (W, K^T, Up^T, the gates) are fetched while the
// current one computes.
template <int D>
__global__ __launch_bounds__(kThr) void gdn_scan(GdnParams p) {
  static_assert(kGdnScanRows == 16, "one 16-row MFMA tile of the state per workgroup");
  constexpr int NT = D / 64;                     // 16-column accumulator tiles per wave
  constexpr int KQ = 4 * NT;                     // columns per lane quad: the depth of W S^T
  typedef typename BfVec<KQ>::type bfq;
  __shared__ __attribute__((aligned(16))) float part[2][4][16][kCL];  // [buffer][wave][row][token]
  __shared__ __attribute__((aligned(16))) float fsh[2][kC];           // [buffer][token] exp(g_C - g)
  // Workgroup -> (row slice, (b, h)). The SL = D / 16 slices of one (b, h) read the same W,
  // K^T and Up of every block. Workgroups go to the 8 XCDs (each with its own L2) in turn,
  // id mod 8, so the slices of one (b, h) take ids of one residue mod 8 and read one L2 copy
  // of those operands; the (b, h) past the last full group of 8 take consecutive ids.
  constexpr int SL = D / kGdnScanRows;
  const int id = blockIdx.x, G8 = (p.B * p.H) & ~7;
  int split, g;
  if (id < SL * G8) {
    const int r = id >> 3;
    split = r % SL;
    g = (id & 7) + 8 * (r / SL);
  } else {
    const int t = id - SL * G8;
    split = t % SL;
    g = G8 + t / SL;
  }
  const int tid = threadIdx.x;
  const int l = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), lr = l & 15, lq = l >> 4;
  const int wv = tid >> 6;                       // the wave index as a per-lane value
  const int rs = split * 16, cw = w * (D / 4);
  const size_t bh = static_cast<size_t>(g);
  auto boff = [&](int blk) { return (bh * p.nb + blk) * static_cast<size_t>(kC) * D; };
  const float* gbh = p.g + bh * (static_cast<size_t>(p.nb) * kC);
  const size_t srow = (bh * D + rs + lr) * D + cw + KQ * lq;      // this lane's run of a state row

  f32x4 sc[NT];                                  // S[rs + lr][cw + KQ lq + 4 t + j]
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p.state_in != nullptr) v = ld4(p.state_in + srow + 4 * t);
    sc[t] = f32x4{v.x, v.y, v.z, v.w};
  }
  struct Ops {
    bfq wa[4][3];                                // W parts, token tile mt
    bf16x8 ka[NT][2];                            // K^T, column tile t, 32-token step s
    float4 up;                                   // Up^T[rs + lr][16 w + 4 lq ..]   (up_index)
    float gl;                                    // g of token l (lane 63: g_C)
  };
  // The next block's operands are loaded in pieces between this block's MFMA groups: issued
  // together they would fill the CU's vector memory queue and hold the wave until the whole
  // 17 KB per wave had been accepted. For the same reason the block's starting state is
  // stored after the exchange barrier, not among the loads.
  // (in the order of use: W part 2, 1, 0 of all four token tiles; then Up^T and the gates;
  // then K^T by 32-token step)
  auto fetch_w2 = [&](int blk, Ops& o, int k) {  // loads 2 k, 2 k + 1 of fetch_w's order
    const __bf16* wsrc = static_cast<const __bf16*>(p.W) + 3 * boff(blk);
#pragma unroll
    for (int i = 2 * k; i < 2 * k + 2; ++i) {
      const int pt = 2 - i / 4, mt = i % 4;
      o.wa[mt][pt] = *reinterpret_cast<const bfq*>(wsrc + (((w * 4 + mt) * 3 + pt) * 64 + l) * KQ);
    }
  };
  auto fetch_w = [&](int blk, Ops& o, int pt) {
    const __bf16* wsrc = static_cast<const __bf16*>(p.W) + 3 * boff(blk);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      o.wa[mt][pt] = *reinterpret_cast<const bfq*>(wsrc + (((w * 4 + mt) * 3 + pt) * 64 + l) * KQ);
  };
  auto fetch_k = [&](int blk, Ops& o) {
    const size_t bo = boff(blk);
    o.up = ld4(p.Up + bo + (((split * 4 + lq) * 64 + lr + 16 * w) << 2));
    o.gl = gbh[blk * kC + l];
    const __bf16* ksrc = static_cast<const __bf16*>(p.Kt) + bo;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        o.ka[t][s2] = *reinterpret_cast<const bf16x8*>(ksrc + (((w * NT + t) * 2 + s2) * 64 + l) * 8);
  };
  auto fetch = [&](int blk, Ops& o) {
#pragma unroll
    for (int pt = 2; pt >= 0; --pt) fetch_w(blk, o, pt);
    fetch_k(blk, o);
  };
  auto step = [&](int blk, const Ops& cur, Ops& nxt) {
    const int nb1 = min(blk + 1, p.nb - 1);
    // the slice as the B operand of W S^T, in three bf16 parts
    float sv[KQ];
#pragma unroll
    for (int e = 0; e < KQ; ++e) sv[e] = sc[e >> 2][e & 3];
    bfq s1, s2, s3;
    split3<KQ>(sv, s1, s2, s3);
    __builtin_amdgcn_sched_barrier(0);
    // partial of W S^T over this wave's columns: four 16-token tiles, smallest products first,
    // the four chains interleaved; the next block's W parts load between the groups
    f32x4 acc[4] = {};
#pragma unroll
    for (int k = 0; k < 6; ++k) {
      constexpr int wp[6] = {2, 1, 0, 1, 0, 0};
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bfq& sp = k == 0 || k == 3 || k == 5 ? s1 : (k == 1 || k == 4 ? s2 : s3);
        acc[mt] = mfma16<KQ>(cur.wa[mt][wp[k]], sp, acc[mt]);
      }
      fetch_w2(nb1, nxt, k);
      __builtin_amdgcn_sched_barrier(0);
    }
    const float gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cur.gl), 63));
    const float fl = __expf(gC - cur.gl);        // exp(g_C - g_l): token l's weight in the update
    // wave w folds -Up of its own token tile into its partial: the four sum to -U
    const f32x4 up = f32x4{cur.up.x, cur.up.y, cur.up.z, cur.up.w};
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] -= (mt == w ? 1.f : 0.f) * up;
    float(*pb)[16][kCL] = part[blk & 1];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      st4(&pb[w][lr][16 * mt + 4 * lq], make_float4(acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]));
    if (wv == 0) fsh[blk & 1][l] = fl;
    __syncthreads();
    {                                            // this block's starting state, for gdn_out (s0_index)
      float* Sst = p.Sst + (bh * p.nb + blk) * static_cast<size_t>(D) * D;
#pragma unroll
      for (int t = 0; t < NT; ++t)
        st4(Sst + s0_index<D>(rs + lr, cw + KQ * lq + 4 * t), make_float4(sc[t][0], sc[t][1], sc[t][2], sc[t][3]));
    }
    // U[32 s + 8 lq + e][rs + lr] = Up - W S^T = -(sum of the partials), ub[8 s + e]
    f32x16 ub;
    float fu[16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tok = 32 * (u >> 1) + 8 * lq + 4 * (u & 1);
      float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float4 x = ld4(&pb[v][lr][tok]);
        sum.x -= x.x; sum.y -= x.y; sum.z -= x.z; sum.w -= x.w;
      }
      const float4 f4 = ld4(&fsh[blk & 1][tok]);
      ub[4 * u] = sum.x; ub[4 * u + 1] = sum.y; ub[4 * u + 2] = sum.z; ub[4 * u + 3] = sum.w;
      fu[4 * u] = f4.x; fu[4 * u + 1] = f4.y; fu[4 * u + 2] = f4.z; fu[4 * u + 3] = f4.w;
    }
    {                                            // U^T for gdn_out (ut_index): wave w writes tokens 32 (w / 2) + 8 lq + 4 (w % 2) ..
      st4(p.U + boff(blk) + ut_index(rs + lr, 32 * (w >> 1) + 8 * lq + 4 * (w & 1)),
          make_float4(ub[4 * w], ub[4 * w + 1], ub[4 * w + 2], ub[4 * w + 3]));
    }
    // the update's B operand: U scaled by exp(g_C - g) per token, in three bf16 parts
    bf16x8 u1[2], u2[2], u3[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = ub[8 * s2 + e] * fu[8 * s2 + e];
      split3<8>(x, u1[s2], u2[s2], u3[s2]);
    }
    const float dec = __expf(gC);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4 a = s2 == 0 ? sc[t] * dec : sc[t];
        a = mfma16<8>(cur.ka[t][s2], u3[s2], a);
        a = mfma16<8>(cur.ka[t][s2], u2[s2], a);
        sc[t] = mfma16<8>(cur.ka[t][s2], u1[s2], a);
      }
      if (s2 == 0) fetch_k(nb1, nxt);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  Ops opa, opb;                                  // operands of even and odd blocks
  fetch(0, opa);
  // pairs of blocks, then the odd one out: the loop is entered only from its top, so the
  // wait counts at its head see just the odd block's loads as pending
  int blk = 0;
  for (; blk + 1 < p.nb; blk += 2) {
    step(blk, opa, opb);
    step(blk + 1, opb, opa);
  }
  if (blk < p.nb) step(blk, opa, opb);
#pragma unroll
  for (int t = 0; t < NT; ++t) st4(p.state_out + srow + 4 * t, make_float4(sc[t][0], sc[t][1], sc[t][2], sc[t][3]));
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
// global memory (L2), only the gates go through LDS. The scan stores S0 and U^T in this
// kernel's operand order (s0_index, ut_index), so each of their loads is one 1 KB run.
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
  const float* Ut = p.U + boff;                                     // U^T in ut_index order
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
      const float* src = S0 + s0_index<D>(c, 16 * s + 8 * hf);   // the second half 256 floats on
      float x[8];
      unpack8(ld4(src), ld4(src + 256), x);
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
        const float* src = Ut + ut_index(c, 32 * jt + 16 * s2 + 4 * hf);   // second run 256 floats on
        float x[8];
        unpack8(ld4(src), ld4(src + 256), x);
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
  hipLaunchKernelGGL(gdn_scan<D>, dim3((D / kGdnScanRows) * p.H * p.B), dim3(kThr), 0, st, p);
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
