// RoPE-fused cache writes for streaming chunk attention (gfx950).
//
//  rope_apply      Q -> rotated Q scratch, K -> rotated staging slot, V -> transposed staging slot
//  kv_ring_append  K -> rotated cache slot, V -> transposed cache slot (a commit)
//  sink_update     same as kv_ring_append, for one sink chunk of a sink replacement
//  rope_refresh    in-place rotation of the temporal pairs of whole slots by -Delta
//
// The rotation is RoFormer's per channel pair; the pages name 3D (t, h, w) RoPE
// offsets and their periodic re-basing at chunk boundaries (StreamDiffusionV2,
// "Sommario tecnico" 2.A.2). cos/sin come from host fp64 tables rounded to
// fp32 (spatial tables in the workspace, the chunk's temporal table by value),
// so no device trigonometry runs. Arithmetic is fp32; stores round to the cache
// type (bf16: round to nearest even; fp8: E4M3 of the OCP 8-bit float format,
// clamped to +-448 and rounded to nearest even by v_cvt_pk_fp8_f32, whose
// unclamped result above 464 would be NaN). Inputs are fp32 for an fp32 cache
// and bf16 for a bf16 or fp8 cache.
//
// All four are HBM-bound streaming kernels: every input element is read once
// and every output element written once, with 16-byte vector accesses. V is
// transposed through LDS so that the cache holds V^T ([D][keys] per (b, h)),
// the operand layout the attention kernel's PV product reads; its stores are
// 16-byte vectors along the key axis when the slot offset is 16-byte aligned.
#include "sa_internal.h"

#include <type_traits>

namespace sa {
namespace {

constexpr int kTileTokens = 64;
constexpr int kThreads = 256;

template <typename T> struct alignas(16) Vec16 { T e[16 / sizeof(T)]; };
// N elements of a storage type, stored as one vector
template <typename T, int N> struct alignas(N * sizeof(T)) VecN { T e[N]; };

// One E4M3 value (OCP 8-bit float: bias 7, 3 mantissa bits, largest finite 448).
struct fp8e4m3 { uint8_t bits; };
constexpr float kE4M3Max = 448.f;

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(__bf16 x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f(fp8e4m3 x) { return __builtin_amdgcn_cvt_f32_fp8(x.bits, 0); }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f<__bf16>(float x) { return static_cast<__bf16>(x); }
template <> __device__ __forceinline__ fp8e4m3 from_f<fp8e4m3>(float x) {
  const float c = fminf(fmaxf(x, -kE4M3Max), kE4M3Max);
  return fp8e4m3{static_cast<uint8_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xff)};
}

// (cos, sin) of the pair starting at even channel ch of a token at (frame, y, x).
__device__ __forceinline__ float2 pair_cs(const float2* s_tcs, const RopeWriteParams& p, int ch,
                                          int f, int y, int x) {
  if (ch < p.dt) return s_tcs[f * (p.dt >> 1) + (ch >> 1)];
  ch -= p.dt;
  if (ch < p.dh) return p.h_cs[y * (p.dh >> 1) + (ch >> 1)];
  ch -= p.dh;
  return p.w_cs[x * (p.dw >> 1) + (ch >> 1)];
}

// Rotated pairs of one 16-byte input vector, rounded to the storage type TS. SCALED:
// the rotated values are multiplied by `post` before rounding (fp8 queries).
template <typename TI, typename TS, bool SCALED = false>
__device__ __forceinline__ VecN<TS, 16 / sizeof(TI)> rotate(const Vec16<TI>& in,
                                                           const float2 (&cs)[16 / sizeof(TI) / 2],
                                                           float post = 1.f) {
  constexpr int NP = 16 / sizeof(TI) / 2;
  VecN<TS, 2 * NP> out;
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    const float u0 = to_f(in.e[2 * e]), u1 = to_f(in.e[2 * e + 1]);
    float r0 = u0 * cs[e].x - u1 * cs[e].y, r1 = u0 * cs[e].y + u1 * cs[e].x;
    if constexpr (SCALED) {
      r0 *= post;
      r1 *= post;
    }
    out.e[2 * e] = from_f<TS>(r0);
    out.e[2 * e + 1] = from_f<TS>(r1);
  }
  return out;
}

// A 16-byte vector of input elements rounded to the storage type.
template <typename TI, typename TS>
__device__ __forceinline__ VecN<TS, 16 / sizeof(TI)> convert(const uint4& in) {
  constexpr int N = 16 / sizeof(TI);
  const TI* e = reinterpret_cast<const TI*>(&in);
  VecN<TS, N> out;
#pragma unroll
  for (int i = 0; i < N; ++i) out.e[i] = from_f<TS>(to_f(e[i]));
  return out;
}

// Transpose of a VN x VN block held as VN 16-byte vectors: in[t] = token t's VN
// channels, out[c] = channel c's VN tokens. bf16: each output dword packs the
// same-parity halves of two input dwords (v_perm_b32); fp32: register renaming.
template <typename T>
__device__ __forceinline__ void transpose_block(const uint4 (&in)[16 / sizeof(T)], uint4 (&out)[16 / sizeof(T)]) {
  constexpr int VN = 16 / sizeof(T);
  auto dw = [](const uint4& v, int k) { return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w; };
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {                // channels 2k, 2k+1
      unsigned lo[4], hi[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {           // tokens 2jj, 2jj+1
        lo[jj] = __builtin_amdgcn_perm(dw(in[2 * jj + 1], k), dw(in[2 * jj], k), 0x05040100u);
        hi[jj] = __builtin_amdgcn_perm(dw(in[2 * jj + 1], k), dw(in[2 * jj], k), 0x07060302u);
      }
      out[2 * k] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      out[2 * k + 1] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    }
  } else {
#pragma unroll
    for (int c = 0; c < VN; ++c) out[c] = make_uint4(dw(in[0], c), dw(in[1], c), dw(in[2], c), dw(in[3], c));
  }
}

// One block: 64 tokens of head blockIdx.y of stream blockIdx.z.
//  * K (and Q): thread (tid % vpt) owns one 16-byte channel vector of tokens
//    tid / vpt + j * (256 / vpt); all its loads are issued before any store.
//  * V: thread owns a VN x VN (tokens x channels) block, transposes it in
//    registers and stores VN 16-byte rows of V^T; lanes with consecutive token
//    groups of one channel group write 128 contiguous bytes per channel row.
// TI: input element type; TS: cache (storage) element type.
template <typename TI, typename TS, bool HAS_Q>
__device__ __forceinline__ void rope_write_body(const RopeWriteParams& p) {
  using T = TI;
  using VecS = VecN<TS, 16 / sizeof(TI)>;
  constexpr int VN = 16 / sizeof(T);             // elements per 16-byte input vector
  constexpr int MAXJ = 32 / VN;                  // K/Q vectors per thread (D <= 128)
  __shared__ float2 s_tcs[kMaxTemporalPairs];
  __shared__ int s_fyx[kTileTokens][3];          // (frame, y, x) of the tile's tokens

  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * kTileTokens;
  const int h = blockIdx.y, b = blockIdx.z;
  const int ntab = p.n_frames * (p.dt >> 1);
  for (int i = tid; i < ntab; i += kThreads) s_tcs[i] = p.t_cs[i];
  if (tid < kTileTokens) {
    const int n = min(n0 + tid, p.n_tokens - 1);
    const int hw = p.Hf * p.Wf;
    const int f = n / hw, rem = n - f * hw, y = rem / p.Wf;
    s_fyx[tid][0] = f;
    s_fyx[tid][1] = y;
    s_fyx[tid][2] = rem - y * p.Wf;
  }
  __syncthreads();

  const size_t bh = static_cast<size_t>(b) * p.H + h;
  const T* __restrict__ kin = static_cast<const T*>(p.k);
  const T* __restrict__ qin = static_cast<const T*>(p.q);
  const T* __restrict__ vin = static_cast<const T*>(p.v);
  TS* __restrict__ kc = static_cast<TS*>(p.kcache) + bh * p.k_bh_stride;
  TS* __restrict__ qo = static_cast<TS*>(p.qrot) + (bh * p.q_rows + p.q_row0) * p.D;
  TS* __restrict__ vt = static_cast<TS*>(p.vtcache) + bh * p.vt_bh_stride + p.row0 + n0;
  auto in_off = [&](int n, int c) {
    return ((static_cast<size_t>(b) * p.in_tokens + p.in_tok0 + n) * p.H + h) * p.D + c;
  };

  // ---- issue every load first: V blocks, then K (and Q) vectors ---------------
  constexpr int TG = kTileTokens / VN;           // token groups per tile
  constexpr int MAXB = (TG * 128 / VN + kThreads - 1) / kThreads;   // V blocks per thread (D <= 128)
  const int nblk = TG * (p.D / VN);
  const int ntok = min(kTileTokens, p.n_tokens - n0);
  uint4 vin_r[MAXB][VN];
#pragma unroll
  for (int r = 0; r < MAXB; ++r) {
    const int blk = tid + r * kThreads;
    const int t0 = (blk % TG) * VN, cb = (blk / TG) * VN;
#pragma unroll
    for (int t = 0; t < VN; ++t)
      vin_r[r][t] = blk < nblk && t0 + t < ntok ? *reinterpret_cast<const uint4*>(vin + in_off(n0 + t0 + t, cb))
                                                : make_uint4(0, 0, 0, 0);
  }
  const int vpt = p.D / VN;
  const int tpp = kThreads / vpt;                // tokens per pass
  const int passes = kTileTokens / tpp;          // <= MAXJ
  const int c0 = (tid % vpt) * VN;
  const int tl0 = tid / vpt;
  Vec16<T> kv[MAXJ], qv[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int n = n0 + tl0 + j * tpp;
    if (j < passes && n < p.n_tokens) {
      kv[j] = *reinterpret_cast<const Vec16<T>*>(kin + in_off(n, c0));
      if constexpr (HAS_Q) qv[j] = *reinterpret_cast<const Vec16<T>*>(qin + in_off(n, c0));
    }
  }

  // ---- K (and Q): rotate 16-byte channel vectors ----------------------------
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int tl = tl0 + j * tpp, n = n0 + tl;
    if (j < passes && n < p.n_tokens) {
      float2 cs[VN / 2];
#pragma unroll
      for (int e = 0; e < VN / 2; ++e) cs[e] = pair_cs(s_tcs, p, c0 + 2 * e, s_fyx[tl][0], s_fyx[tl][1], s_fyx[tl][2]);
      *reinterpret_cast<VecS*>(kc + static_cast<size_t>(p.row0 + n) * p.D + c0) = rotate<TI, TS>(kv[j], cs);
      // fp8 queries are stored times q_scale (the base-2 softmax scale brought into [1, 2))
      if constexpr (HAS_Q)
        *reinterpret_cast<VecS*>(qo + static_cast<size_t>(n) * p.D + c0) =
            rotate<TI, TS, std::is_same_v<TS, fp8e4m3>>(qv[j], cs, p.q_scale);
    }
  }

  // ---- V: VN x VN register transposes straight into V^T ---------------------
  const bool vec_ok = (p.row0 % VN) == 0;        // vector-aligned V^T rows
#pragma unroll
  for (int r = 0; r < MAXB; ++r) {
    const int blk = tid + r * kThreads;
    if (blk >= nblk) break;
    const int t0 = (blk % TG) * VN, cb = (blk / TG) * VN;
    uint4 out[VN];
    transpose_block<T>(vin_r[r], out);
    if (vec_ok && t0 + VN <= ntok) {
#pragma unroll
      for (int c = 0; c < VN; ++c)
        *reinterpret_cast<VecS*>(vt + static_cast<size_t>(cb + c) * p.key_stride + t0) = convert<TI, TS>(out[c]);
    } else {
#pragma unroll
      for (int c = 0; c < VN; ++c) {
        const VecS e = convert<TI, TS>(out[c]);
        for (int t = 0; t < VN && t0 + t < ntok; ++t) vt[static_cast<size_t>(cb + c) * p.key_stride + t0 + t] = e.e[t];
      }
    }
  }
}

template <typename TI, typename TS>
__global__ __launch_bounds__(kThreads) void rope_apply(RopeWriteParams p) {
  rope_write_body<TI, TS, true>(p);
}

template <typename TI, typename TS>
__global__ __launch_bounds__(kThreads) void kv_ring_append(RopeWriteParams p) {
  rope_write_body<TI, TS, false>(p);
}

template <typename TI, typename TS>
__global__ __launch_bounds__(kThreads) void sink_update(RopeWriteParams p) {
  rope_write_body<TI, TS, false>(p);
}

// One thread per (row, temporal pair) of one slot of one (b, h).
template <typename T>
__global__ __launch_bounds__(kThreads) void rope_refresh(RefreshParams p) {
  __shared__ float2 s_cs[kMaxRefreshPairs];
  const int np = p.dt >> 1;
  if (threadIdx.x < np) s_cs[threadIdx.x] = p.cs[threadIdx.x];
  __syncthreads();
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= static_cast<int64_t>(p.Nc) * np) return;
  const int row = static_cast<int>(i / np), j = static_cast<int>(i - static_cast<int64_t>(row) * np);
  T* e = static_cast<T*>(p.kcache) + static_cast<size_t>(blockIdx.z) * p.k_bh_stride +
         static_cast<size_t>(p.slot_row0[blockIdx.y] + row) * p.D + 2 * j;
  struct alignas(2 * sizeof(T)) Pair { T a, b; };
  const Pair in = *reinterpret_cast<const Pair*>(e);
  const float u0 = to_f(in.a), u1 = to_f(in.b);
  const float2 cs = s_cs[j];
  Pair out;
  out.a = from_f<T>(u0 * cs.x - u1 * cs.y);
  out.b = from_f<T>(u0 * cs.y + u1 * cs.x);
  *reinterpret_cast<Pair*>(e) = out;
}

}  // namespace

// dtype: 0 = fp32 in, fp32 cache; 1 = bf16 in, bf16 cache; 2 = bf16 in, fp8 cache
#define SA_WRITE_LAUNCHER(NAME, KERNEL)                                                             \
  hipError_t NAME(const RopeWriteParams& p, int dtype, hipStream_t st) {                            \
    if (p.n_tokens <= 0) return hipSuccess;                                                         \
    const dim3 grid((p.n_tokens + kTileTokens - 1) / kTileTokens, p.H, p.B);                        \
    if (dtype == 2) hipLaunchKernelGGL((KERNEL<__bf16, fp8e4m3>), grid, dim3(kThreads), 0, st, p);  \
    else if (dtype == 1) hipLaunchKernelGGL((KERNEL<__bf16, __bf16>), grid, dim3(kThreads), 0, st, p); \
    else hipLaunchKernelGGL((KERNEL<float, float>), grid, dim3(kThreads), 0, st, p);                \
    return hipGetLastError();                                                                       \
  }

SA_WRITE_LAUNCHER(launch_rope_apply, rope_apply)
SA_WRITE_LAUNCHER(launch_kv_append, kv_ring_append)
SA_WRITE_LAUNCHER(launch_sink_update, sink_update)
#undef SA_WRITE_LAUNCHER

hipError_t launch_rope_refresh(const RefreshParams& p, int dtype, hipStream_t st) {
  const int64_t items = static_cast<int64_t>(p.Nc) * (p.dt >> 1);
  if (items <= 0 || p.n_slot <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((items + kThreads - 1) / kThreads), p.n_slot, p.BH);
  if (dtype == 2) hipLaunchKernelGGL(rope_refresh<fp8e4m3>, grid, dim3(kThreads), 0, st, p);
  else if (dtype == 1) hipLaunchKernelGGL(rope_refresh<__bf16>, grid, dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL(rope_refresh<float>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace sa
