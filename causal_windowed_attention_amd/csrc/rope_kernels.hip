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
// type (bf16: round to nearest even).
//
// All four are HBM-bound streaming kernels: every input element is read once
// and every output element written once, with 16-byte vector accesses. V is
// transposed through LDS so that the cache holds V^T ([D][keys] per (b, h)),
// the operand layout the attention kernel's PV product reads; its stores are
// 16-byte vectors along the key axis when the slot offset is 16-byte aligned.
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kTileTokens = 64;
constexpr int kThreads = 256;

template <typename T> struct alignas(16) Vec16 { T e[16 / sizeof(T)]; };

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(__bf16 x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f<__bf16>(float x) { return static_cast<__bf16>(x); }

// (cos, sin) of the pair starting at even channel ch of a token at (frame, y, x).
__device__ __forceinline__ float2 pair_cs(const float2* s_tcs, const RopeWriteParams& p, int ch,
                                          int f, int y, int x) {
  if (ch < p.dt) return s_tcs[f * (p.dt >> 1) + (ch >> 1)];
  ch -= p.dt;
  if (ch < p.dh) return p.h_cs[y * (p.dh >> 1) + (ch >> 1)];
  ch -= p.dh;
  return p.w_cs[x * (p.dw >> 1) + (ch >> 1)];
}

template <typename T>
__device__ __forceinline__ Vec16<T> rotate(const Vec16<T>& in, const float2 (&cs)[16 / sizeof(T) / 2]) {
  constexpr int NP = 16 / sizeof(T) / 2;
  Vec16<T> out;
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    const float u0 = to_f(in.e[2 * e]), u1 = to_f(in.e[2 * e + 1]);
    out.e[2 * e] = from_f<T>(u0 * cs[e].x - u1 * cs[e].y);
    out.e[2 * e + 1] = from_f<T>(u0 * cs[e].y + u1 * cs[e].x);
  }
  return out;
}

// One block: 64 tokens of head blockIdx.y of stream blockIdx.z.
template <typename T, bool HAS_Q>
__device__ __forceinline__ void rope_write_body(const RopeWriteParams& p) {
  constexpr int VN = 16 / sizeof(T);             // elements per 16-byte vector
  constexpr int LDS_STRIDE = kTileTokens + VN;   // padded row of the V^T tile
  __shared__ float2 s_tcs[kMaxTemporalPairs];
  __shared__ Vec16<T> s_vraw[128 * LDS_STRIDE / VN];
  T* s_v = reinterpret_cast<T*>(s_vraw);

  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * kTileTokens;
  const int h = blockIdx.y, b = blockIdx.z;
  const int ntab = p.n_frames * (p.dt >> 1);
  for (int i = tid; i < ntab; i += kThreads) s_tcs[i] = p.t_cs[i];
  __syncthreads();

  const int vpt = p.D / VN;                      // vectors per token row of one head
  const int nvec = kTileTokens * vpt;
  const int hw = p.Hf * p.Wf;
  const size_t bh = static_cast<size_t>(b) * p.H + h;
  const T* kin = static_cast<const T*>(p.k);
  const T* vin = static_cast<const T*>(p.v);
  T* kc = static_cast<T*>(p.kcache) + bh * p.k_bh_stride;

  for (int i = tid; i < nvec; i += kThreads) {
    const int tl = i / vpt;
    const int c0 = (i - tl * vpt) * VN;
    const int n = n0 + tl;
    if (n >= p.n_tokens) continue;
    const size_t in_off =
        ((static_cast<size_t>(b) * p.in_tokens + p.in_tok0 + n) * p.H + h) * p.D + c0;
    const int f = n / hw, rem = n - f * hw, y = rem / p.Wf, x = rem - y * p.Wf;
    float2 cs[VN / 2];
#pragma unroll
    for (int e = 0; e < VN / 2; ++e) cs[e] = pair_cs(s_tcs, p, c0 + 2 * e, f, y, x);

    const Vec16<T> kv = *reinterpret_cast<const Vec16<T>*>(kin + in_off);
    *reinterpret_cast<Vec16<T>*>(kc + static_cast<size_t>(p.row0 + n) * p.D + c0) = rotate<T>(kv, cs);
    if constexpr (HAS_Q) {
      const Vec16<T> qv = *reinterpret_cast<const Vec16<T>*>(static_cast<const T*>(p.q) + in_off);
      T* qo = static_cast<T*>(p.qrot) + (bh * p.n_tokens + n) * p.D + c0;
      *reinterpret_cast<Vec16<T>*>(qo) = rotate<T>(qv, cs);
    }
    const Vec16<T> vv = *reinterpret_cast<const Vec16<T>*>(vin + in_off);
#pragma unroll
    for (int e = 0; e < VN; ++e) s_v[(c0 + e) * LDS_STRIDE + tl] = vv.e[e];
  }
  __syncthreads();

  // V^T rows: channel d holds this tile's tokens contiguously at keys row0 + n0 ...
  const int ntok = min(kTileTokens, p.n_tokens - n0);
  T* vt = static_cast<T*>(p.vtcache) + bh * p.vt_bh_stride + p.row0 + n0;
  if (ntok == kTileTokens && ((p.row0 + n0) % VN) == 0) {
    constexpr int VPR = kTileTokens / VN;        // vectors per channel row
    for (int i = tid; i < p.D * VPR; i += kThreads) {
      const int d = i / VPR, c = i - d * VPR;
      *reinterpret_cast<Vec16<T>*>(vt + static_cast<size_t>(d) * p.key_stride + c * VN) =
          *reinterpret_cast<const Vec16<T>*>(s_v + d * LDS_STRIDE + c * VN);
    }
  } else {
    for (int i = tid; i < p.D * ntok; i += kThreads) {
      const int d = i / ntok, t = i - d * ntok;
      vt[static_cast<size_t>(d) * p.key_stride + t] = s_v[d * LDS_STRIDE + t];
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void rope_apply(RopeWriteParams p) {
  rope_write_body<T, true>(p);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void kv_ring_append(RopeWriteParams p) {
  rope_write_body<T, false>(p);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void sink_update(RopeWriteParams p) {
  rope_write_body<T, false>(p);
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

hipError_t launch_rope_apply(const RopeWriteParams& p, int dtype, hipStream_t st) {
  if (p.n_tokens <= 0) return hipSuccess;
  const dim3 grid((p.n_tokens + kTileTokens - 1) / kTileTokens, p.H, p.B);
  if (dtype == 1) hipLaunchKernelGGL(rope_apply<__bf16>, grid, dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL(rope_apply<float>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_kv_append(const RopeWriteParams& p, int dtype, hipStream_t st) {
  if (p.n_tokens <= 0) return hipSuccess;
  const dim3 grid((p.n_tokens + kTileTokens - 1) / kTileTokens, p.H, p.B);
  if (dtype == 1) hipLaunchKernelGGL(kv_ring_append<__bf16>, grid, dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL(kv_ring_append<float>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_sink_update(const RopeWriteParams& p, int dtype, hipStream_t st) {
  if (p.n_tokens <= 0) return hipSuccess;
  const dim3 grid((p.n_tokens + kTileTokens - 1) / kTileTokens, p.H, p.B);
  if (dtype == 1) hipLaunchKernelGGL(sink_update<__bf16>, grid, dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL(sink_update<float>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_rope_refresh(const RefreshParams& p, int dtype, hipStream_t st) {
  const int64_t items = static_cast<int64_t>(p.Nc) * (p.dt >> 1);
  if (items <= 0 || p.n_slot <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((items + kThreads - 1) / kThreads), p.n_slot, p.BH);
  if (dtype == 1) hipLaunchKernelGGL(rope_refresh<__bf16>, grid, dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL(rope_refresh<float>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace sa
