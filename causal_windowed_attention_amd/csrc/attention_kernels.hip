// chunk_attention: exact softmax attention of one chunk's queries over the
// visible key prefix [0, n_keys) of every (b, h): the sink, the sliding window
// of recent chunks and the chunk itself (SANA-Streaming, "Transformer a
// diffusione ibrido": softmax blocks over a sliding local window plus a
// persistent sink chunk). The cache keeps every visible key contiguous per
// (b, h), so the chunk-granular sink/window/self mask reduces to one key
// range: tiles outside it are never visited, tiles inside it need no mask, and
// only the ragged last tile masks keys >= n_keys.
//
// bf16 kernel (gfx950 MFMA), one workgroup = 4 waves = 128 query rows of one
// (b, h) and one key-range split:
//  * each wave owns 32 query rows; its rotated Q rows sit in VGPRs as the B
//    operand of v_mfma_f32_32x32x16_bf16;
//  * K tiles (64 keys x D) and V^T tiles (D x 64 keys) are staged in LDS,
//    double-buffered, with an XOR swizzle of the 16-byte chunks so the MFMA
//    operand reads of 8 consecutive rows hit distinct banks;
//  * scores are computed transposed, S^T = K Q^T: lane l holds query l % 32, so
//    the online-softmax rescale of the O^T accumulators is one scalar per lane
//    and the fp32 scores convert in registers into the B operand of
//    O^T += V^T P^T. The K rows are written into LDS with bits 2 and 3 of the
//    row index swapped, which makes the key order of the score accumulators
//    equal to the key order of the V^T operand reads;
//  * online softmax in base 2 with the scale folded into one FMA, row maxima
//    from in-lane maxima plus one cross-half exchange; the row sums stay
//    per-lane partials until the end;
//  * P is rounded to bf16 for the PV product; accumulation is fp32.
// Workgroups are mapped so that consecutive (b, h, split, q-tile) work items
// land on the same XCD (the hardware deals blocks round-robin over 8 XCDs):
// the q-tiles of one head then stream the same K/V tiles through one L2.
//
// fp32 kernel: one query row per lane, K/V tiles in LDS, FMA arithmetic (the
// small-shape fp32 path; not a throughput path).
//
// attn_combine merges key-range splits: with per-split normalised outputs O_s
// and log2-sum-exp L_s, O = sum_s 2^(L_s - L) O_s with L = log2 sum_s 2^L_s.
#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kThreads = 256;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Work item of block b for n work items in (bh, split, qt) order, qt fastest,
// with consecutive items on one XCD (blocks are dealt round-robin to 8 XCDs).
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int xcd = b & 7, idx = b >> 3;
  const int base = n >> 3, extra = n & 7;
  return xcd * base + min(xcd, extra) + idx;
}

// Swap bits 2 and 3 of a tile row index (an involution).
__device__ __forceinline__ int swap_bits23(int r) {
  return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1);
}

template <int D>
struct AttnSmem {
  __bf16 k[2][kBf16BlockN * D];
  __bf16 vt[2][D * kBf16BlockN];
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void chunk_attention_bf16(AttnParams p) {
  constexpr int BN = kBf16BlockN;
  constexpr int KC = D / 8;                      // 16-byte chunks per K row
  constexpr int VC = BN / 8;                     // 16-byte chunks per V^T row
  constexpr int KLOADS = BN * KC / kThreads;     // K chunks per thread per tile
  constexpr int VLOADS = D * VC / kThreads;      // V^T chunks per thread per tile
  constexpr int KSTEPS = D / 16;                 // MFMA k-steps of QK^T
  constexpr int MT = BN / 32;                    // 32-key score tiles per key tile
  constexpr int DT = D / 32;                     // 32-channel output tiles
  constexpr int PSTEPS = BN / 16;                // MFMA k-steps of PV
  __shared__ AttnSmem<D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;

  const int n_work = p.B * p.H * p.q_tiles * p.kv_splits;
  const int work = xcd_remap(blockIdx.x, n_work);
  const int qt = work % p.q_tiles;
  const int rest = work / p.q_tiles;
  const int split = rest % p.kv_splits;
  const int bh = rest / p.kv_splits;
  const int t_begin = static_cast<int>((static_cast<int64_t>(split) * p.key_tiles) / p.kv_splits);
  const int t_end = static_cast<int>((static_cast<int64_t>(split + 1) * p.key_tiles) / p.kv_splits);

  const __bf16* kbase = static_cast<const __bf16*>(p.kcache) + static_cast<size_t>(bh) * p.k_bh_stride;
  const __bf16* vbase = static_cast<const __bf16*>(p.vtcache) + static_cast<size_t>(bh) * p.vt_bh_stride;
  const int n_keys = p.n_keys;

  // ---- Q rows of this wave as MFMA B operands --------------------------------
  const int q = qt * kBf16BlockM + wave * 32 + l32;
  const int qrow = min(q, p.Nc - 1);
  const __bf16* qsrc = static_cast<const __bf16*>(p.q) + (static_cast<size_t>(bh) * p.Nc + qrow) * D;
  bf16x8 bq[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) bq[s] = *reinterpret_cast<const bf16x8*>(qsrc + 16 * s + 8 * g);

  // ---- tile staging: global -> registers -> LDS ------------------------------
  uint4 kreg[KLOADS], vreg[VLOADS];
  auto load_tile = [&](int t) {
    const int key0 = t * BN;
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int id = tid + i * kThreads;
      const int r = id / KC, c = id % KC;
      const int key = key0 + r;
      kreg[i] = key < n_keys ? *reinterpret_cast<const uint4*>(kbase + static_cast<size_t>(key) * D + 8 * c)
                             : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int id = tid + i * kThreads;
      const int d = id / VC, c = id % VC;
      const int k8 = key0 + 8 * c;
      uint4 v = *reinterpret_cast<const uint4*>(vbase + static_cast<size_t>(d) * p.key_stride + k8);
      if (k8 + 8 > n_keys) {                     // ragged tail: zero keys >= n_keys
        unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (k8 + e >= n_keys) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        v = make_uint4(w[0], w[1], w[2], w[3]);
      }
      vreg[i] = v;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int id = tid + i * kThreads;
      const int r = swap_bits23(id / KC), c = id % KC;
      *reinterpret_cast<uint4*>(&sm.k[buf][r * D + ((c ^ (r & 7)) * 8)]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int id = tid + i * kThreads;
      const int d = id / VC, c = id % VC;
      *reinterpret_cast<uint4*>(&sm.vt[buf][d * BN + ((c ^ (d & 7)) * 8)]) = vreg[i];
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = f32x16{};
  float m = -__builtin_inff();   // running max of scaled scores (log2 units)
  float l = 0.f;                 // per-lane partial row sum

  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    if (t + 1 < t_end) load_tile(t + 1);
    const __bf16* Ks = sm.k[buf];
    const __bf16* Vs = sm.vt[buf];
    const int key0 = t * BN;

    // S^T = K Q^T  (32 keys x 32 queries per accumulator)
    f32x16 sacc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      sacc[mt] = f32x16{};
      const int r = 32 * mt + l32;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const int c = 2 * s + g;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + r * D + ((c ^ (r & 7)) * 8));
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[s], sacc[mt], 0, 0, 0);
      }
    }
    // accumulator j of tile mt holds key key0 + 32*mt + 16*(j/8) + 8*g + j%8
    if (key0 + BN > n_keys) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (key0 + 32 * mt + 16 * (j >> 3) + 8 * g + (j & 7) >= n_keys) sacc[mt][j] = -__builtin_inff();
    }

    // online softmax (base 2)
    float mx = -__builtin_inff();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[mt][j]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx * p.scale_log2);
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
    float rs = 0.f;
    bf16x8 pb[PSTEPS];
#pragma unroll
    for (int s = 0; s < PSTEPS; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = fast_exp2(fmaf(sacc[s >> 1][8 * (s & 1) + e], p.scale_log2, -m_new));
        rs += pv;
        pb[s][e] = static_cast<__bf16>(pv);
      }
    }
    l = fmaf(l, alpha, rs);
#pragma unroll
    for (int i = 0; i < DT; ++i) o[i] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 32 * dt + l32;
#pragma unroll
      for (int s = 0; s < PSTEPS; ++s) {
        const int c = 2 * s + g;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vs + d * BN + ((c ^ (d & 7)) * 8));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s], o[dt], 0, 0, 0);
      }
    }

    if (t + 1 < t_end) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ---------------------------------------------------------------
  const float l_tot = l + __shfl_xor(l, 32);
  if (q >= p.Nc) return;
  const float inv = 1.f / l_tot;
  const float lse2 = m + __log2f(l_tot);
  const int b = bh / p.H, h = bh - b * p.H;
  if (p.kv_splits == 1) {
    __bf16* dst = static_cast<__bf16*>(p.out) + ((static_cast<size_t>(b) * p.Nc + q) * p.H + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<__bf16>(o[dt][4 * jj + e] * inv);
        *reinterpret_cast<bf16x4*>(dst + 32 * dt + 8 * jj + 4 * g) = v;
      }
    if (p.lse != nullptr && g == 0) p.lse[static_cast<size_t>(bh) * p.Nc + q] = lse2 * kLn2;
  } else {
    const size_t row = (static_cast<size_t>(split) * p.B * p.H + bh) * p.Nc + q;
    float* dst = p.part_o + row * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<float4*>(dst + 32 * dt + 8 * jj + 4 * g) =
            make_float4(o[dt][4 * jj] * inv, o[dt][4 * jj + 1] * inv, o[dt][4 * jj + 2] * inv,
                        o[dt][4 * jj + 3] * inv);
    if (g == 0) p.part_lse[row] = lse2;
  }
}

// fp32: one query row per lane, 64 rows per block, 32-key tiles through LDS.
template <int D>
__global__ __launch_bounds__(64) void chunk_attention_f32(AttnParams p) {
  constexpr int BN = kF32BlockN;
  __shared__ float sk[BN][D + 1];
  __shared__ float sv[BN][D + 1];
  const int lane = threadIdx.x;
  const int n_work = p.B * p.H * p.q_tiles * p.kv_splits;
  const int work = xcd_remap(blockIdx.x, n_work);
  const int qt = work % p.q_tiles;
  const int rest = work / p.q_tiles;
  const int split = rest % p.kv_splits;
  const int bh = rest / p.kv_splits;
  const int t_begin = static_cast<int>((static_cast<int64_t>(split) * p.key_tiles) / p.kv_splits);
  const int t_end = static_cast<int>((static_cast<int64_t>(split + 1) * p.key_tiles) / p.kv_splits);
  const float* kbase = static_cast<const float*>(p.kcache) + static_cast<size_t>(bh) * p.k_bh_stride;
  const float* vbase = static_cast<const float*>(p.vtcache) + static_cast<size_t>(bh) * p.vt_bh_stride;

  const int q = qt * kF32BlockM + lane;
  const int qrow = min(q, p.Nc - 1);
  const float* qsrc = static_cast<const float*>(p.q) + (static_cast<size_t>(bh) * p.Nc + qrow) * D;
  float qr[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = qsrc[d] * p.scale_log2;
    o[d] = 0.f;
  }
  float m = -__builtin_inff(), l = 0.f;
  for (int t = t_begin; t < t_end; ++t) {
    const int key0 = t * BN;
    const int nk = min(BN, p.n_keys - key0);
    for (int i = lane; i < BN * D; i += 64) {
      const int r = i / D, d = i - r * D;
      sk[r][d] = r < nk ? kbase[static_cast<size_t>(key0 + r) * D + d] : 0.f;
    }
    for (int i = lane; i < BN * D; i += 64) {
      const int d = i / BN, r = i - d * BN;
      sv[r][d] = r < nk ? vbase[static_cast<size_t>(d) * p.key_stride + key0 + r] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < nk; ++r) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qr[d], sk[r][d], s);
      const float m_new = fmaxf(m, s);
      const float alpha = fast_exp2(m - m_new);
      const float pw = fast_exp2(s - m_new);
      l = fmaf(l, alpha, pw);
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(o[d], alpha, pw * sv[r][d]);
      m = m_new;
    }
    __syncthreads();
  }
  if (q >= p.Nc) return;
  const float inv = 1.f / l;
  const float lse2 = m + __log2f(l);
  const int b = bh / p.H, h = bh - b * p.H;
  if (p.kv_splits == 1) {
    float* dst = static_cast<float*>(p.out) + ((static_cast<size_t>(b) * p.Nc + q) * p.H + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) dst[d] = o[d] * inv;
    if (p.lse != nullptr) p.lse[static_cast<size_t>(bh) * p.Nc + q] = lse2 * kLn2;
  } else {
    const size_t row = (static_cast<size_t>(split) * p.B * p.H + bh) * p.Nc + q;
#pragma unroll
    for (int d = 0; d < D; ++d) p.part_o[row * D + d] = o[d] * inv;
    p.part_lse[row] = lse2;
  }
}

// One thread per (b*h, query, 4-channel group).
template <typename T>
__global__ __launch_bounds__(kThreads) void attn_combine(CombineParams p) {
  const int groups = p.D / 4;
  const int64_t total = static_cast<int64_t>(p.B) * p.H * p.Nc * groups;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= total) return;
  const int g4 = static_cast<int>(i % groups);
  const int64_t rq = i / groups;                 // bh * Nc + q
  const int q = static_cast<int>(rq % p.Nc);
  const int bh = static_cast<int>(rq / p.Nc);
  const int64_t split_stride = static_cast<int64_t>(p.B) * p.H * p.Nc;
  float mx = -__builtin_inff();
  for (int s = 0; s < p.kv_splits; ++s) mx = fmaxf(mx, p.part_lse[s * split_stride + rq]);
  float wsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < p.kv_splits; ++s) {
    const float w = fast_exp2(p.part_lse[s * split_stride + rq] - mx);
    const float4 v = *reinterpret_cast<const float4*>(p.part_o + (s * split_stride + rq) * p.D + 4 * g4);
    wsum += w;
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  const float inv = 1.f / wsum;
  const int b = bh / p.H, h = bh - b * p.H;
  T* dst = static_cast<T*>(p.out) + ((static_cast<size_t>(b) * p.Nc + q) * p.H + h) * p.D + 4 * g4;
  dst[0] = static_cast<T>(acc.x * inv);
  dst[1] = static_cast<T>(acc.y * inv);
  dst[2] = static_cast<T>(acc.z * inv);
  dst[3] = static_cast<T>(acc.w * inv);
  if (p.lse != nullptr && g4 == 0) p.lse[rq] = (mx + __log2f(wsum)) * kLn2;
}

}  // namespace

hipError_t launch_chunk_attention(const AttnParams& p, int dtype, hipStream_t st) {
  const int64_t n_work = static_cast<int64_t>(p.B) * p.H * p.q_tiles * p.kv_splits;
  if (n_work <= 0) return hipSuccess;
  if (dtype == 1) {
    if (p.D == 128) hipLaunchKernelGGL(chunk_attention_bf16<128>, dim3(n_work), dim3(kThreads), 0, st, p);
    else hipLaunchKernelGGL(chunk_attention_bf16<64>, dim3(n_work), dim3(kThreads), 0, st, p);
  } else {
    if (p.D == 128) hipLaunchKernelGGL(chunk_attention_f32<128>, dim3(n_work), dim3(64), 0, st, p);
    else hipLaunchKernelGGL(chunk_attention_f32<64>, dim3(n_work), dim3(64), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine(const CombineParams& p, int dtype, hipStream_t st) {
  const int64_t total = static_cast<int64_t>(p.B) * p.H * p.Nc * (p.D / 4);
  if (total <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((total + kThreads - 1) / kThreads));
  if (dtype == 1) hipLaunchKernelGGL(attn_combine<__bf16>, grid, dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL(attn_combine<float>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace sa
