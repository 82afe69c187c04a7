// RoPE-fused cache writes for streaming chunk attention (gfx950).
//
//  rope_apply      Q -> rotated Q scratch, K -> rotated staging slot, V -> transposed staging slot
//  kv_ring_append  K -> rotated cache slot, V -> transposed cache slot (a commit)
//  sink_update     same as kv_ring_append, for one sink chunk of a sink replacement
//  rope_refresh    in-place rotation of the temporal pairs of whole slots by -Delta
//
// The rotation is RoFormer's per channel pair; the pages name 3D (t, h, w) RoPE
// offsets and their periodic re-basing at chunk boundaries (StreamDiffusionV2,
// "Sommario tecnico" 2.A.2). cos/sin are fp64 values rounded to fp32: the
// spatial tables come from the host (in the workspace, staged in LDS by each
// block when they fit), a single launch's temporal table from the host by value,
// and a batched launch computes each entry's temporal angles in fp64 on the
// device. Arithmetic is fp32; stores round to the cache
// type (bf16: round to nearest even; fp8: E4M3 of the OCP 8-bit float format,
// clamped to +-448 and rounded to nearest even by v_cvt_pk_fp8_f32, whose
// unclamped result above 464 would be NaN). Inputs are fp32 for an fp32 cache
// and bf16 for a bf16 or fp8 cache.
//
// All four are HBM-bound streaming kernels: every input element is read once
// and every output element written once, with 16-byte vector accesses. V is
// transposed in registers and across lane pairs so that the cache holds V^T
// ([D][keys] per (b, h)), the operand layout the attention kernel's PV product
// reads; its stores are 16-byte vectors along the key axis when the slot offset
// is 16-byte aligned.
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

// Spatial (cos, sin) pairs a block stages in LDS: the h table ([Hf][d_h/2]) followed by the
// w table ([Wf][d_w/2]), when both fit and the w table follows the h table in memory.
constexpr int kMaxLdsSpatialPairs = 2048;

// (cos, sin) of the pair starting at even channel ch of a token at (frame, y, x); the spatial
// pairs come from s_hw (LDS) when hw_lds, else from the tables in global memory.
template <typename P>
__device__ __forceinline__ float2 pair_cs(const float2* s_tcs, const float2* s_hw, bool hw_lds, const P& p, int ch,
                                          int f, int y, int x) {
  if (ch < p.dt) return s_tcs[f * (p.dt >> 1) + (ch >> 1)];
  ch -= p.dt;
  const int nh = p.Hf * (p.dh >> 1);
  const int i = ch < p.dh ? y * (p.dh >> 1) + (ch >> 1) : nh + x * (p.dw >> 1) + ((ch - p.dh) >> 1);
  if (hw_lds) return s_hw[i];
  return i < nh ? p.h_cs[i] : p.w_cs[i - nh];
}

// 16 bytes per lane from the `bytes` bytes at src + voffset into LDS at lds + 16 * lane
// (buffer_load_dwordx4 ... lds: no VGPRs; lanes past the end read zeros).
__device__ __forceinline__ void lds_copy16(const void* src, int bytes, int voffset, void* lds) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), 0, bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0, 0);
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

// Transpose of a VN x VN block (VN tokens x VN channels, VN elements per 16 bytes) shared by
// lanes l and l + 32 of a wave: lane half g holds in[i] = token g VN/2 + i's VN channels and
// gets out[c] = the VN tokens of channel g VN/2 + c. Each lane transposes its half in registers
// (bf16: v_perm_b32 packs the same-parity halves of two input dwords; fp32: register renaming),
// then the two lanes exchange channel halves with v_permlane32_swap, which swaps lanes 32-63 of
// one register with lanes 0-31 of another. Every lane of the wave must run it.
template <typename T>
__device__ __forceinline__ void transpose_half_block(const uint4 (&in)[8 / sizeof(T)], uint4 (&out)[8 / sizeof(T)]) {
  constexpr int VN = 16 / sizeof(T), HV = VN / 2;
  auto dw = [](const uint4& v, int k) { return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w; };
  uint2 ch[VN];                                  // this lane's HV tokens of channel c
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {                // channels 2d, 2d+1
      ch[2 * d] = make_uint2(__builtin_amdgcn_perm(dw(in[1], d), dw(in[0], d), 0x05040100u),
                             __builtin_amdgcn_perm(dw(in[3], d), dw(in[2], d), 0x05040100u));
      ch[2 * d + 1] = make_uint2(__builtin_amdgcn_perm(dw(in[1], d), dw(in[0], d), 0x07060302u),
                                 __builtin_amdgcn_perm(dw(in[3], d), dw(in[2], d), 0x07060302u));
    }
  } else {
#pragma unroll
    for (int c = 0; c < VN; ++c) ch[c] = make_uint2(dw(in[0], c), dw(in[1], c));
  }
  // lane half 0 keeps channels [0, HV) and takes their tokens [HV, VN) from lane l + 32;
  // lane half 1 keeps channels [HV, VN) and takes their tokens [0, HV) from lane l - 32
#pragma unroll
  for (int c = 0; c < HV; ++c) {
    const auto x = __builtin_amdgcn_permlane32_swap(ch[c].x, ch[HV + c].x, false, false);
    const auto y = __builtin_amdgcn_permlane32_swap(ch[c].y, ch[HV + c].y, false, false);
    out[c] = make_uint4(x[0], y[0], x[1], y[1]);
  }
}

// One block: 64 tokens of head blockIdx.y of batch entry b.
//  * K (and Q): thread (tid % vpt) owns one 16-byte channel vector of tokens
//    tid / vpt + j * (256 / vpt); all its loads are issued before any store.
//  * V: lanes l and l + 32 share a VN x VN (tokens x channels) block, each loading
//    VN/2 of its tokens; the block is transposed in registers and across the lane
//    pair, and each lane stores VN/2 16-byte rows of V^T. Every thread loads and
//    stores as many V vectors as K vectors; the lanes of one channel group with
//    consecutive token groups write 128 contiguous bytes per channel row.
// Every global load is issued before the block sets up its position tables in LDS, so the
// table set-up and its barrier run under the load latency.
// TI: input element type; TS: cache (storage) element type. P holds the geometry (a
// RopeWriteParams or RopeBatchParams); the target pointers are passed apart; fill_tcs(i)
// gives temporal (cos, sin) entry i = frame * d_t/2 + pair.
template <typename TI, typename TS, bool HAS_Q, typename P, typename FillT>
__device__ __forceinline__ void rope_write_core(const P& p, int b, const void* q_in, const void* k_in,
                                                const void* v_in, void* qrot, void* kcache, void* vtcache,
                                                int row0, int q_row0, int in_tok0, FillT fill_tcs) {
  using T = TI;
  using VecS = VecN<TS, 16 / sizeof(TI)>;
  constexpr int VN = 16 / sizeof(T);             // elements per 16-byte input vector
  constexpr int MAXJ = 32 / VN;                  // K/Q vectors per thread (D <= 128)
  __shared__ float2 s_tcs[kMaxTemporalPairs];
  __shared__ int s_fyx[kTileTokens][3];          // (frame, y, x) of the tile's tokens
  __shared__ __attribute__((aligned(16))) float2 s_hw[kMaxLdsSpatialPairs];

  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * kTileTokens;
  const int h = blockIdx.y;

  // ---- spatial tables -> LDS, issued before the data loads -------------------------
  // The rotation's table lookups then read LDS after the barrier instead of going out to
  // memory behind this block's data loads.
  const int nh = p.Hf * (p.dh >> 1), n_hw = nh + p.Wf * (p.dw >> 1);
  const bool hw_lds = n_hw <= kMaxLdsSpatialPairs && p.w_cs == p.h_cs + nh;
  if (hw_lds) {
    // 16-byte copies: an odd pair count reads 8 bytes past the w table, inside the tables'
    // workspace region (which the host pads to 256 bytes)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), bytes = (n_hw * 8 + 15) & ~15;
    for (int c = wave; c * 1024 < bytes; c += kThreads / 64)
      lds_copy16(p.h_cs, bytes, c * 1024 + (tid & 63) * 16, reinterpret_cast<char*>(s_hw) + c * 1024);
  }

  const size_t bh = static_cast<size_t>(b) * p.H + h;
  const T* __restrict__ kin = static_cast<const T*>(k_in);
  const T* __restrict__ qin = static_cast<const T*>(q_in);
  const T* __restrict__ vin = static_cast<const T*>(v_in);
  TS* __restrict__ kc = static_cast<TS*>(kcache) + bh * p.k_bh_stride;
  TS* __restrict__ qo = static_cast<TS*>(qrot) + (bh * p.q_rows + q_row0) * p.D;
  TS* __restrict__ vt = static_cast<TS*>(vtcache) + bh * p.vt_bh_stride + row0 + n0;
  auto in_off = [&](int n, int c) {
    return ((static_cast<size_t>(b) * p.in_tokens + in_tok0 + n) * p.H + h) * p.D + c;
  };

  // ---- issue every load first: V half-blocks, then K (and Q) vectors ----------
  constexpr int TG = kTileTokens / VN;           // token groups per tile
  constexpr int HV = VN / 2;                     // tokens of a V block per lane
  constexpr int PAIRS = kThreads / 2;            // V blocks per round (one per lane pair)
  constexpr int MAXB = (TG * 128 / VN + PAIRS - 1) / PAIRS;   // rounds (D <= 128)
  // V blocks: TG * D / VN = 64 D / VN^2, a multiple of 32, so a wave's 32 pairs are all valid
  // or all invalid (the lane-pair exchange needs the whole wave)
  const int nblk = TG * (p.D / VN);
  const int ntok = min(kTileTokens, p.n_tokens - n0);
  const int vg = (tid >> 5) & 1;                 // lane half
  const int pair0 = (tid >> 6) * 32 + (tid & 31);
  uint4 vin_r[MAXB][HV];
#pragma unroll
  for (int r = 0; r < MAXB; ++r) {
    const int blk = pair0 + r * PAIRS;
    const int t0 = (blk % TG) * VN + vg * HV, cb = (blk / TG) * VN;
#pragma unroll
    for (int t = 0; t < HV; ++t)
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

  // ---- position tables (under the load latency) ------------------------------
  const int ntab = p.n_frames * (p.dt >> 1);
  for (int i = tid; i < ntab; i += kThreads) s_tcs[i] = fill_tcs(i);
  if (tid < kTileTokens) {
    const int n = min(n0 + tid, p.n_tokens - 1);
    const int hw = p.Hf * p.Wf;
    const int f = n / hw, rem = n - f * hw, y = rem / p.Wf;
    s_fyx[tid][0] = f;
    s_fyx[tid][1] = y;
    s_fyx[tid][2] = rem - y * p.Wf;
  }
  if (hw_lds) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the LDS table copies have landed
  __syncthreads();

  // ---- K (and Q): rotate 16-byte channel vectors ----------------------------
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int tl = tl0 + j * tpp, n = n0 + tl;
    if (j < passes && n < p.n_tokens) {
      float2 cs[VN / 2];
#pragma unroll
      for (int e = 0; e < VN / 2; ++e) cs[e] = pair_cs(s_tcs, s_hw, hw_lds, p, c0 + 2 * e, s_fyx[tl][0], s_fyx[tl][1], s_fyx[tl][2]);
      *reinterpret_cast<VecS*>(kc + static_cast<size_t>(row0 + n) * p.D + c0) = rotate<TI, TS>(kv[j], cs);
      // fp8 queries are stored times q_scale (the base-2 softmax scale brought into [1, 2))
      if constexpr (HAS_Q)
        *reinterpret_cast<VecS*>(qo + static_cast<size_t>(n) * p.D + c0) =
            rotate<TI, TS, std::is_same_v<TS, fp8e4m3>>(qv[j], cs, p.q_scale);
    }
  }

  // ---- V: VN x VN transposes (registers and lane pairs) straight into V^T -----
  const bool vec_ok = (row0 % VN) == 0;          // vector-aligned V^T rows
#pragma unroll
  for (int r = 0; r < MAXB; ++r) {
    const int blk = pair0 + r * PAIRS;
    if (blk >= nblk) break;                      // wave-uniform
    const int t0 = (blk % TG) * VN, cb = (blk / TG) * VN + vg * HV;   // this lane's HV channels
    uint4 out[HV];
    transpose_half_block<T>(vin_r[r], out);
    if (vec_ok && t0 + VN <= ntok) {
#pragma unroll
      for (int c = 0; c < HV; ++c)
        *reinterpret_cast<VecS*>(vt + static_cast<size_t>(cb + c) * p.key_stride + t0) = convert<TI, TS>(out[c]);
    } else {
#pragma unroll
      for (int c = 0; c < HV; ++c) {
        const VecS e = convert<TI, TS>(out[c]);
        for (int t = 0; t < VN && t0 + t < ntok; ++t) vt[static_cast<size_t>(cb + c) * p.key_stride + t0 + t] = e.e[t];
      }
    }
  }
}

// Single-stream writes: batch entry blockIdx.z, temporal table from the kernel arguments.
template <typename TI, typename TS, bool HAS_Q>
__device__ __forceinline__ void rope_write_body(const RopeWriteParams& p) {
  rope_write_core<TI, TS, HAS_Q>(p, blockIdx.z, p.q, p.k, p.v, p.qrot, p.kcache, p.vtcache, p.row0, p.q_row0,
                                 p.in_tok0, [&](int i) { return p.t_cs[i]; });
}

// Ragged batch: blockIdx.z = stream e * B + b; stream e's temporal (cos, sin) from fp64 on the
// device, (t0[e] + frame) * theta_t[pair] rounded to fp32 (the same angle the host tables use).
template <typename TI, typename TS>
__global__ __launch_bounds__(kThreads) void rope_apply_batch(RopeBatchParams p) {
  const int e = blockIdx.z / p.B, b = blockIdx.z - (blockIdx.z / p.B) * p.B;
  const int np = p.dt >> 1;
  const int t0 = p.t0[e];
  rope_write_core<TI, TS, true>(p, b, p.q[e], p.k[e], p.v[e], p.qrot[e], p.kcache[e], p.vtcache[e], p.row0[e], 0, 0,
                                [&](int i) {
                                  const int f = i / np, j = i - f * np;
                                  const double a = static_cast<double>(t0 + f) * p.theta_t[j];
                                  return make_float2(static_cast<float>(cos(a)), static_cast<float>(sin(a)));
                                });
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

// Refresh items: 16-byte vectors of the rows' temporal segments (channels [0, d_t)) of
// every target slot of one (b, h) = blockIdx.z; consecutive items cover one row's segment,
// then the next row. A thread takes kRefreshPerThread items a block apart (all loads first);
// the last vector of a segment may reach into the h channels, which are written back as read.
constexpr int kRefreshPerThread = 4;

template <typename T>
__global__ __launch_bounds__(kThreads) void rope_refresh(RefreshParams p) {
  constexpr int VN = 16 / sizeof(T);
  constexpr int R = kRefreshPerThread;
  __shared__ float2 s_cs[kMaxRefreshPairs];
  const int np = p.dt >> 1;
  const int nvec = (p.dt + VN - 1) / VN;         // vectors per row segment
  const int64_t items = static_cast<int64_t>(p.n_slot) * p.Nc * nvec;
  T* const base = static_cast<T*>(p.kcache) + static_cast<size_t>(blockIdx.z) * p.k_bh_stride;
  T* e[R];
  int vv[R];
  Vec16<T> in[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int64_t i = (static_cast<int64_t>(blockIdx.x) * R + k) * kThreads + threadIdx.x;
    e[k] = nullptr;
    vv[k] = 0;
    if (i < items) {
      const int v = static_cast<int>(i % nvec);
      const int64_t r = i / nvec;
      const int slot = static_cast<int>(r / p.Nc), row = static_cast<int>(r - static_cast<int64_t>(slot) * p.Nc);
      e[k] = base + static_cast<size_t>(p.slot_row0[slot] + row) * p.D + v * VN;
      vv[k] = v;
      in[k] = *reinterpret_cast<const Vec16<T>*>(e[k]);
    }
  }
  if (threadIdx.x < np) s_cs[threadIdx.x] = p.cs[threadIdx.x];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < R; ++k) {
    if (e[k] == nullptr) continue;
    VecN<T, VN> out;
#pragma unroll
    for (int c = 0; c < VN / 2; ++c) {
      const int j = vv[k] * (VN / 2) + c;        // temporal pair index
      const float u0 = to_f(in[k].e[2 * c]), u1 = to_f(in[k].e[2 * c + 1]);
      if (j < np) {
        const float2 cs = s_cs[j];
        out.e[2 * c] = from_f<T>(u0 * cs.x - u1 * cs.y);
        out.e[2 * c + 1] = from_f<T>(u0 * cs.y + u1 * cs.x);
      } else {
        out.e[2 * c] = in[k].e[2 * c];
        out.e[2 * c + 1] = in[k].e[2 * c + 1];
      }
    }
    *reinterpret_cast<VecN<T, VN>*>(e[k]) = out;
  }
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

hipError_t launch_rope_apply_batch(const RopeBatchParams& p, int dtype, hipStream_t st) {
  if (p.n_tokens <= 0 || p.n <= 0) return hipSuccess;
  const dim3 grid((p.n_tokens + kTileTokens - 1) / kTileTokens, p.H, p.B * p.n);
  if (dtype == 2) hipLaunchKernelGGL((rope_apply_batch<__bf16, fp8e4m3>), grid, dim3(kThreads), 0, st, p);
  else if (dtype == 1) hipLaunchKernelGGL((rope_apply_batch<__bf16, __bf16>), grid, dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL((rope_apply_batch<float, float>), grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_rope_refresh(const RefreshParams& p, int dtype, hipStream_t st) {
  const int vn = dtype == 2 ? 16 : dtype == 1 ? 8 : 4;   // elements per 16-byte vector
  const int64_t items = static_cast<int64_t>(p.n_slot) * p.Nc * ((p.dt + vn - 1) / vn);
  if (items <= 0 || p.n_slot <= 0) return hipSuccess;
  const int64_t per_block = static_cast<int64_t>(kThreads) * kRefreshPerThread;
  const dim3 grid(static_cast<unsigned>((items + per_block - 1) / per_block), 1, p.BH);
  if (dtype == 2) hipLaunchKernelGGL(rope_refresh<fp8e4m3>, grid, dim3(kThreads), 0, st, p);
  else if (dtype == 1) hipLaunchKernelGGL(rope_refresh<__bf16>, grid, dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL(rope_refresh<float>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace sa
