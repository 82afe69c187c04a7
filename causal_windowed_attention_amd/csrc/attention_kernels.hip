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
//  * K tiles (64 keys x D) and V^T tiles (D x 64 keys) are copied into LDS
//    through a multi-stage pipeline, with an XOR swizzle of the 16-byte chunks
//    so the MFMA operand reads are free of bank conflicts;
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

#include <type_traits>

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

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

// s_waitcnt immediate that waits for vmcnt <= n and leaves expcnt/lgkmcnt free.
__host__ __device__ constexpr int vmcnt_imm(int n) {
  return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 0x3) << 14);
}

// Swizzled position of 16-byte chunk c in LDS row r of a tile whose rows hold
// `chunks` chunks (4, 8 or 16; 4 rows of 64 bytes, 2 of 128 or 1 of 256 share a
// 256-byte bank window); an involution in c for fixed r.
__device__ __forceinline__ int swz(int c, int r, int chunks) {
  return chunks >= 16 ? (c ^ (r & 15)) : chunks == 8 ? (c ^ ((r >> 1) & 7)) : (c ^ ((r >> 2) & 3));
}

// Raw buffer resource over the `bytes` bytes at `base` (gfx9 word 3: untyped
// dwords); a lane whose offset lies past the end reads zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// 16 bytes per lane from rsrc + voffset into LDS at lds + 16 * lane
// (buffer_load_dwordx4 ... lds). The MUBUF form matters: with the FLAT-encoded
// global_load_lds in flight the compiler can only wait for lgkmcnt(0) before
// any LDS read result, which serialises the MFMA operand reads behind the
// newest one; buffer loads count in vmcnt alone.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t rsrc, int voffset, char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0, 0);
}

// Swap bits 2 and 3 of a tile row index (an involution).
__device__ __forceinline__ int swap_bits23(int r) {
  return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// bf16 tile geometry. A stage holds one K tile (64 keys x D, row-major) and
// one V^T tile (D x 64 keys) in LDS without padding. gfx950 serves a
// ds_read_b128 16 lanes (256 bytes, all 64 banks) at a time, and the MFMA
// operand reads of those 16 lanes hit 16 consecutive rows at the same logical
// 16-byte chunk; the chunks are therefore XOR-swizzled so the 16 rows land on
// 16 distinct bank groups: chunk c of a 256-byte row r sits at c ^ (r & 15),
// chunk c of a 128-byte row r (two rows per 256-byte bank window) at
// c ^ ((r >> 1) & 7). Tiles are copied global -> LDS directly
// (buffer_load_dwordx4 ... lds: lane i of a wave writes the 16 bytes at LDS base +
// 16 i), choosing each lane's source so that the chunk lands at its swizzled
// place; no VGPR staging, no LDS write instructions.
template <int D, int BN_ = kBf16BlockN>
struct Bf16Geom {
  static constexpr int BN = BN_;
  static constexpr int KROW = D * 2;          // bytes per K row
  static constexpr int VROW = BN * 2;         // bytes per V^T row
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int BUF = KBYTES + VBYTES; // one stage (K + V^T)
  static constexpr int KC = D / 8;            // 16-byte chunks per K row
  static constexpr int VC = BN / 8;           // 16-byte chunks per V^T row
  static constexpr int KCOPIES = KBYTES / 1024 / 4;   // 1 KB wave copies per wave per tile
  static constexpr int VCOPIES = VBYTES / 1024 / 4;
};

// Rescale threshold (log2 units): the running maximum used to exponentiate a
// row is only raised when a tile's maximum exceeds it by more than this, so
// un-normalised weights stay below 2^8 and the O rescale runs rarely.
constexpr float kRescaleThreshold = 8.0f;

// fp8 tile geometry: as Bf16Geom with one byte per element. A stage holds a K
// tile (64 keys x D bytes) and a V^T tile (D x 64 bytes); 128-byte K rows use
// the two-rows-per-bank-window swizzle, 64-byte V^T rows c ^ ((r >> 2) & 3).
template <int D, int BN_ = kBf16BlockN>
struct Fp8Geom {
  static constexpr int BN = BN_;
  static constexpr int KROW = D;              // bytes per K row
  static constexpr int VROW = BN;             // bytes per V^T row
  static constexpr int KBYTES = BN * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int BUF = KBYTES + VBYTES;
  static constexpr int KC = D / 16;
  static constexpr int VC = BN / 16;
};

// The fp8 PV product takes, per lane, 32 P bytes as its B operand: byte 16 a + j
// of lane half g is element j of score accumulator a. With the K tile's rows in
// natural order that element belongs to key 32 a + 8 (j / 4) + 4 g + j % 4; the
// V^T operand bytes of lane half g are keys 32 g .. 32 g + 31 in order. Storing
// key k(t) in LDS row t, with k = 32 g + 16 a + j for t = 32 a + 8 (j / 4) + 4 g
// + j % 4 (a permutation of the six index bits), makes the two orders agree, so
// V^T tiles are copied unpermuted.
__device__ __forceinline__ int fp8_key_of_row(int t) {
  return (t & 3) | (((t >> 3) & 3) << 2) | (((t >> 5) & 1) << 4) | (((t >> 2) & 1) << 5);
}

// fp8 softmax weights are formed as 2^(s - m) with m the running maximum minus
// this shift, so the largest weight of a row sits at 2^4 .. 2^8 (E4M3 holds up
// to 448) and weights down to 2^-10 of it stay in E4M3's normal range.
constexpr float kP8Shift = 4.0f;

// v_mfma_f32_32x32x64_f8f6f4 with both operands E4M3 (format 0) and unit block
// scales (E8M0 127 = 2^0).
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

#ifndef PP_READ_AHEAD
#define PP_READ_AHEAD 2
#endif

// Kernel shape parameters:
//  NW     waves per workgroup (4 or 8); each wave owns 32 * QB query rows
//  QB     32-row query blocks per wave (2: each K/V operand read feeds two MFMAs)
//  STAGES LDS stages of the tile copy pipeline: copies for tile t + STAGES - 1
//         are issued while tile t is computed, so a copy has STAGES - 1 tiles of
//         compute to land (misses to the last-level cache take microseconds)
template <int D, int NW, int QB, int STAGES>
__device__ __forceinline__ void chunk_attention_bf16_body(const AttnParams& p) {
  using G = Bf16Geom<D>;
  constexpr int BN = G::BN;
  constexpr int BM = NW * 32 * QB;               // query rows per workgroup
  constexpr int KSTEPS = D / 16;                 // MFMA k-steps of QK^T
  constexpr int MT = BN / 32;                    // 32-key score tiles per key tile
  constexpr int DT = D / 32;                     // 32-channel output tiles
  constexpr int PSTEPS = BN / 16;                // MFMA k-steps of PV
  constexpr int KCOPIES = G::KBYTES / 1024 / NW; // 1 KB copies per wave per tile
  constexpr int VCOPIES = G::VBYTES / 1024 / NW;
  static_assert(KCOPIES * NW * 1024 == G::KBYTES && VCOPIES * NW * 1024 == G::VBYTES, "copy split");
  static_assert(STAGES >= 2 && (STAGES - 2) * (KCOPIES + VCOPIES) <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * G::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  const int n_work = p.B * p.H * p.q_tiles * p.kv_splits;
  const int work = xcd_remap(blockIdx.x, n_work);
  const int qt = work % p.q_tiles;
  const int rest = work / p.q_tiles;
  const int split = rest % p.kv_splits;
  const int bh = rest / p.kv_splits;
  const int t_begin = static_cast<int>((static_cast<int64_t>(split) * p.key_tiles) / p.kv_splits);
  const int t_end = static_cast<int>((static_cast<int64_t>(split + 1) * p.key_tiles) / p.kv_splits);
  const int n_keys = p.n_keys;
  const int t_tail = (n_keys % BN) ? p.key_tiles - 1 : p.key_tiles;   // index of a ragged last tile

  const char* kbase = static_cast<const char*>(p.kcache) + static_cast<size_t>(bh) * p.k_bh_stride * 2;
  const char* vbase = static_cast<const char*>(p.vtcache) + static_cast<size_t>(bh) * p.vt_bh_stride * 2;

  // ---- Q rows of this wave as MFMA B operands --------------------------------
  const int q0 = qt * BM + wave * 32 * QB + l32;  // query of block qb: q0 + 32 * qb
  bf16x8 bq[QB][KSTEPS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = min(q0 + 32 * qb, p.Nc - 1);
    const __bf16* qsrc = static_cast<const __bf16*>(p.q) + (static_cast<size_t>(bh) * p.Nc + qrow) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) bq[qb][s] = *reinterpret_cast<const bf16x8*>(qsrc + 16 * s + 8 * g);
  }

  // ---- tile copies: lane sources for the swizzled LDS image ------------------
  // copy i of wave w fills LDS chunks P = (i * NW + w) * 64 + lane of the region
  int k_row[KCOPIES], k_src[KCOPIES], v_src[VCOPIES];
#pragma unroll
  for (int i = 0; i < KCOPIES; ++i) {
    const int P = (i * NW + wave) * 64 + lane;
    const int r = P / G::KC, c = swz(P % G::KC, r, G::KC);
    k_row[i] = swap_bits23(r);                   // key (tile-local) held by LDS row r
    k_src[i] = c * 16;
  }
#pragma unroll
  for (int i = 0; i < VCOPIES; ++i) {
    const int P = (i * NW + wave) * 64 + lane;
    const int d = P / G::VC, c = swz(P % G::VC, d, G::VC);
    v_src[i] = d * p.key_stride * 2 + c * 16;
  }
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, p.k_bh_stride * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, p.vt_bh_stride * 2);
  auto issue_tile = [&](int t, int buf) {
    const int key0 = t * BN;
    char* dst = smem + buf * G::BUF;
#pragma unroll
    for (int i = 0; i < KCOPIES; ++i) {
      const int key = min(key0 + k_row[i], n_keys - 1);   // rows past the range: any finite row
      lds_copy16(krs, key * G::KROW + k_src[i], dst + (i * NW + wave) * 1024);
    }
#pragma unroll
    for (int i = 0; i < VCOPIES; ++i)
      lds_copy16(vrs, key0 * 2 + v_src[i], dst + G::KBYTES + (i * NW + wave) * 1024);
  };

  // ---- MFMA operand read addresses -----------------------------------------
  // lane reads LDS row l32 (+ 32 per 32-row tile), logical chunk 2s + g (k-step s)
  int ka[KSTEPS], va[PSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) ka[s] = l32 * G::KROW + swz(2 * s + g, l32, G::KC) * 16;
#pragma unroll
  for (int s = 0; s < PSTEPS; ++s) va[s] = G::KBYTES + l32 * G::VROW + swz(2 * s + g, l32, G::VC) * 16;

  f32x16 o[QB][DT];
  float m[QB], l[QB];            // exponent reference (log2 units), per-lane partial row sum
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int i = 0; i < DT; ++i) o[qb][i] = f32x16{};
    m[qb] = -__builtin_inff();
    l[qb] = 0.f;
  }

  auto compute_tile = [&](int t, int buf, auto tail) {
    const char* stage = smem + buf * G::BUF;
    // S^T = K Q^T  (32 keys x 32 queries per accumulator)
    f32x16 sacc[QB][MT];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) sacc[qb][mt] = f32x16{};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(stage + ka[s] + mt * 32 * G::KROW);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sacc[qb][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[qb][s], sacc[qb][mt], 0, 0, 0);
      }
    // accumulator j of tile mt holds key t*BN + 32*mt + 16*(j/8) + 8*g + j%8
    if constexpr (decltype(tail)::value) {
      const int key0 = t * BN;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (key0 + 32 * mt + 16 * (j >> 3) + 8 * g + (j & 7) >= n_keys)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sacc[qb][mt][j] = -__builtin_inff();
    }
    bf16x8 pb[QB][PSTEPS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = sacc[qb][0][0];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[qb][mt][j]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * p.scale_log2;
      if (__any(mx > m[qb] + kRescaleThreshold)) {   // wave-uniform: raise the reference max
        const float m_new = fmaxf(m[qb], mx);
        const float alpha = fast_exp2(m[qb] - m_new);
        m[qb] = m_new;
        l[qb] *= alpha;
#pragma unroll
        for (int i = 0; i < DT; ++i) o[qb][i] *= alpha;
      }
      float rs = 0.f;
#pragma unroll
      for (int s = 0; s < PSTEPS; ++s) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = fast_exp2(fmaf(sacc[qb][s >> 1][8 * (s & 1) + e], p.scale_log2, -m[qb]));
          rs += pv;
          pb[qb][s][e] = static_cast<__bf16>(pv);
        }
      }
      l[qb] += rs;
    }
    // O^T += V^T P^T
#pragma unroll
    for (int s = 0; s < PSTEPS; ++s)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(stage + va[s] + dt * 32 * G::VROW);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb][s], o[qb][dt], 0, 0, 0);
      }
  };

  // Copy pipeline: tiles t .. t + STAGES - 2 are in flight when tile t is
  // computed. One barrier per tile publishes tile t (every wave's copies for it
  // have landed: each wave first waits until at most its copies for the
  // STAGES - 2 later tiles are outstanding) and retires tile t - 1, whose
  // buffer then receives tile t + STAGES - 1.
  constexpr int PER_TILE = KCOPIES + VCOPIES;
  const int t_stop = min(t_end, t_tail);         // full tiles [t_begin, t_stop)
#pragma unroll
  for (int i = 0; i < STAGES - 1; ++i)
    if (t_begin + i < t_end) issue_tile(t_begin + i, i);
  auto wait_tile = [&](int t) {
    const int ahead = min(t_end - 1 - t, STAGES - 2);   // later tiles already issued
    if (ahead >= STAGES - 2) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((STAGES - 2) * PER_TILE));
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
  };
  int t = t_begin;
  for (; t < t_stop; ++t) {
    const int buf = (t - t_begin) % STAGES;
    wait_tile(t);
    if (t + STAGES - 1 < t_end) issue_tile(t + STAGES - 1, (t - t_begin + STAGES - 1) % STAGES);
    compute_tile(t, buf, std::false_type{});
  }
  if (t < t_end) {                               // the ragged last tile
    wait_tile(t);
    compute_tile(t, (t - t_begin) % STAGES, std::true_type{});
  }

  // ---- epilogue ---------------------------------------------------------------
  const int b = bh / p.H, h = bh - b * p.H;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = l[qb] + __shfl_xor(l[qb], 32);
    const int q = q0 + 32 * qb;
    if (q >= p.Nc) continue;
    const float inv = 1.f / l_tot;
    const float lse2 = m[qb] + __log2f(l_tot);
    if (p.kv_splits == 1) {
      __bf16* dst = static_cast<__bf16*>(p.out) + ((static_cast<size_t>(b) * p.Nc + q) * p.H + h) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = static_cast<__bf16>(o[qb][dt][4 * jj + e] * inv);
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
              make_float4(o[qb][dt][4 * jj] * inv, o[qb][dt][4 * jj + 1] * inv,
                          o[qb][dt][4 * jj + 2] * inv, o[qb][dt][4 * jj + 3] * inv);
      if (g == 0) p.part_lse[row] = lse2;
    }
  }
}

// Value of x held by lane (l ^ 32): v_permlane32_swap exchanges the two wave halves in
// the VALU, no LDS round trip.
__device__ __forceinline__ float xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Ping-pong schedule, 8 waves x 32 query rows (BM = 256), 4 LDS stages.
// Each wave runs a sequence of blocks separated by workgroup barriers:
//   M(0) = QK(0);  V(0) = softmax(0);  M(i) = QK(i) + PV(i-1);  V(i);  ...;  M(n) = PV(n-1)
// so an M block is only MFMAs (and their LDS operand reads) and a V block only
// VALU work. Waves 4-7 run one barrier behind waves 0-3, so on every SIMD (one
// wave of each group) one wave's MFMA block overlaps the other's softmax block.
// Tile copies: tile i+2 is issued at the start of M(i); before the barrier
// that opens global slot 2i, every wave waits for its copies of tile i. A
// stage is reused 4 tiles later, after the lagging group's last PV read of it.
// Output of one ping-pong segment: the final rows, a key-range split partial,
// or a stream-K partial slot.
enum PpOut { kPpFinal = 0, kPpSplit = 1, kPpStreamK = 2 };
constexpr int kPpStages = 4;

template <int D, bool F8>
using PpGeom = std::conditional_t<F8, Fp8Geom<D>, Bf16Geom<D>>;

template <int D, bool F8>
struct PpSmem {
  static constexpr int BYTES = kPpStages * PpGeom<D, F8>::BUF;
};

// The key tiles one work item visits: up to kMaxSegs key-row ranges [lo, hi),
// each covered by tiles lo / BN .. ceil(hi / BN) - 1 and masked to its range.
// Every member is wave-uniform; the fixed-size loops keep it in scalar
// registers.
struct KeyList {
  int n, total;                                  // ranges, tiles over all ranges
  int lo[kMaxSegs], hi[kMaxSegs], t0[kMaxSegs], cum[kMaxSegs];
};

// Where one work item's operands live: rotated Q rows, K and V^T caches, output and
// LSE, with `rows` query rows per (b, h). A chunk attend or a moving buffer uses the
// kernel arguments; a ragged batch's group g uses stream g's own buffers.
struct Bases {
  const void* q;
  const void* kcache;
  const void* vtcache;
  void* out;
  float* lse;
  int rows;
};

__device__ __forceinline__ Bases bases_shared(const AttnParams& p) {
  return Bases{p.q, p.kcache, p.vtcache, p.out, p.lse, p.Nc};
}

// Values read from the argument arrays with a group index are wave-uniform, but the
// compiler cannot always prove it; without these hints a buffer resource built from
// such a pointer is wrapped in a readfirstlane loop at every copy.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* x) {
  const uint64_t u = reinterpret_cast<uint64_t>(x);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(u & 0xffffffffu)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(u >> 32)));
  return reinterpret_cast<T*>(lo | (hi << 32));
}

__device__ __forceinline__ Bases bases_group(const AttnParams& p, int g) {
  if (!p.ragged) return bases_shared(p);
  return Bases{uniform_ptr(p.g_q[g]), uniform_ptr(p.g_kc[g]), uniform_ptr(p.g_vt[g]), uniform_ptr(p.g_out[g]),
               uniform_ptr(p.g_lse[g]), p.group_rows};
}

// Key tiles [t_begin, t_end) of the single range [0, n_keys) (chunk attend, splits, stream-K).
__device__ __forceinline__ KeyList keys_single(const AttnParams& p, int t_begin, int t_end) {
  KeyList kl{};
  kl.n = 1;
  kl.total = t_end - t_begin;
  kl.lo[0] = 0;
  kl.hi[0] = p.n_keys;
  kl.t0[0] = t_begin;
  kl.cum[0] = 0;
  return kl;
}

// The key ranges of query group g (moving-buffer attend).
__device__ __forceinline__ KeyList keys_group(const AttnParams& p, int g, int BN) {
  KeyList kl{};
  kl.n = uniform(p.n_seg[g]);
  int c = 0;
#pragma unroll
  for (int k = 0; k < kMaxSegs; ++k) {
    if (k < kl.n) {
      kl.lo[k] = uniform(p.seg_lo[g][k]);
      kl.hi[k] = uniform(p.seg_hi[g][k]);
      kl.t0[k] = kl.lo[k] / BN;
      kl.cum[k] = c;
      c += (kl.hi[k] + BN - 1) / BN - kl.t0[k];
    }
  }
  kl.total = c;
  return kl;
}

// Physical key tile of visit i, with the key-row range its keys must lie in.
__device__ __forceinline__ int key_tile(const KeyList& kl, int i, int& lo, int& hi) {
  int tile = kl.t0[0] + i;
  lo = kl.lo[0];
  hi = kl.hi[0];
#pragma unroll
  for (int k = 1; k < kMaxSegs; ++k) {
    if (k < kl.n && i >= kl.cum[k]) {
      tile = kl.t0[k] + (i - kl.cum[k]);
      lo = kl.lo[k];
      hi = kl.hi[k];
    }
  }
  return tile;
}

// One ping-pong work segment: query rows [q_base, q_base + BM) of (b, h) = bh,
// valid below q_end, against key tiles [t_begin, t_end) of the range [0, n_keys)
// or, with GROUPS (a moving-buffer attend), against the key tiles of kl. The
// single-range form is a separate instantiation so the chunk attend's kernel
// carries none of the range bookkeeping. F8: E4M3 Q, K, V^T and P with the
// 32x32x64 fp8 MFMA (fp32 accumulation) instead of bf16 with 32x32x16.
template <int D, bool GROUPS, bool F8>
__device__ __forceinline__ void pp_segment(const AttnParams& p, const Bases& bs, char* smem, int bh, int q_base,
                                           int q_end, int t_begin, int t_end, const KeyList& kl, int mode,
                                           int slot) {
  using G = PpGeom<D, F8>;
  using Op = std::conditional_t<F8, i32x8, bf16x8>;   // one MFMA operand per lane
  constexpr int ES = F8 ? 1 : 2;                 // bytes per cached element
  constexpr int KK = F8 ? 64 : 16;               // MFMA reduction depth
  constexpr int NW = 8, STAGES = kPpStages;
  constexpr int BN = G::BN;
  constexpr int BM = NW * 32;
  constexpr int KSTEPS = D / KK, MT = BN / 32, DT = D / 32, PSTEPS = BN / KK;
  constexpr int KCOPIES = G::KBYTES / 1024 / NW;
  constexpr int VCOPIES = G::VBYTES / 1024 / NW;
  constexpr int PER_TILE = KCOPIES + VCOPIES;
  static_assert(KCOPIES * NW * 1024 == G::KBYTES && VCOPIES * NW * 1024 == G::VBYTES, "copy split");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lag = wave >= 4 ? 1 : 0;
  const int l32 = lane & 31, g = lane >> 5;
  const int n = GROUPS ? kl.total : t_end - t_begin;   // tiles of this work item (>= 1)
  const int n_keys = p.n_keys;
  // physical key tile of visit i and the key-row range its keys must lie in
  auto visit = [&](int i, int& lo, int& hi) {
    if constexpr (GROUPS) {
      return key_tile(kl, i, lo, hi);
    } else {
      lo = 0;
      hi = n_keys;
      return t_begin + i;
    }
  };

  const char* kbase = static_cast<const char*>(bs.kcache) + static_cast<size_t>(bh) * p.k_bh_stride * ES;
  const char* vbase = static_cast<const char*>(bs.vtcache) + static_cast<size_t>(bh) * p.vt_bh_stride * ES;

  const int q = q_base + wave * 32 + l32;
  Op bq[KSTEPS];                                 // Q^T operand: lane l holds query l % 32
  {
    const int qrow = min(q, q_end - 1);
    const char* qsrc = static_cast<const char*>(bs.q) + (static_cast<size_t>(bh) * bs.rows + qrow) * D * ES;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) bq[s] = *reinterpret_cast<const Op*>(qsrc + (KK * s + (KK / 2) * g) * ES);
  }

  // Copy sources (byte offsets) of copy c of this wave; K rows of every (b, h)
  // are padded to key_stride, so a tile never reads past the allocation.
  // Recomputed per copy (a few VALU ops) to keep registers for the pipeline.
  auto k_src = [&](int c) {
    const int P = (c * NW + wave) * 64 + lane;
    const int r = P / G::KC;
    return (F8 ? fp8_key_of_row(r) : swap_bits23(r)) * G::KROW + swz(P % G::KC, r, G::KC) * 16;
  };
  auto v_src = [&](int c) {
    const int P = (c * NW + wave) * 64 + lane;
    const int d = P / G::VC;
    return d * p.key_stride * ES + swz(P % G::VC, d, G::VC) * 16;
  };
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, p.k_bh_stride * ES);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, p.vt_bh_stride * ES);
  auto issue_tile = [&](int i) {                 // visit i into stage i % STAGES
    int lo_unused, hi_unused;
    const int key0 = visit(i, lo_unused, hi_unused) * BN;
    char* dst = smem + (i % STAGES) * G::BUF;
#pragma unroll
    for (int c = 0; c < KCOPIES; ++c) lds_copy16(krs, key0 * G::KROW + k_src(c), dst + (c * NW + wave) * 1024);
#pragma unroll
    for (int c = 0; c < VCOPIES; ++c) lds_copy16(vrs, key0 * ES + v_src(c), dst + G::KBYTES + (c * NW + wave) * 1024);
  };

  // K operand address of k-step s: row l32, swizzled chunk of logical chunk 2s + g,
  // recomputed per read (two VALU ops) rather than held in 8 registers
  // Operand reads. bf16: 16 bytes per lane, logical chunk 2 s + g of row l32.
  // fp8: 32 bytes per lane, logical chunks 4 s + 2 g and 4 s + 2 g + 1 (two reads).
  const int ka_row = l32 * G::KROW;
  auto ka = [&](int s) { return ka_row + swz(2 * s + g, l32, G::KC) * 16; };
  auto va = [&](int s) { return G::KBYTES + l32 * G::VROW + swz(2 * s + g, l32, G::VC) * 16; };
  auto k_op = [&](const char* stage, int s, int mt) -> Op {
    if constexpr (F8) {
      const char* row = stage + ka_row + mt * 32 * G::KROW;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(row + swz(4 * s + 2 * g, l32, G::KC) * 16);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(row + swz(4 * s + 2 * g + 1, l32, G::KC) * 16);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
      return *reinterpret_cast<const bf16x8*>(stage + ka(s) + mt * 32 * G::KROW);
    }
  };
  auto v_op = [&](const char* stage, int s, int dt) -> Op {
    if constexpr (F8) {                          // PSTEPS = 1: the whole 64-byte row pair
      const char* row = stage + G::KBYTES + (dt * 32 + l32) * G::VROW;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(row + swz(2 * g, l32, G::VC) * 16);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(row + swz(2 * g + 1, l32, G::VC) * 16);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
      return *reinterpret_cast<const bf16x8*>(stage + va(s) + dt * 32 * G::VROW);
    }
  };
  auto mma = [](const Op& a, const Op& b, const f32x16& c) -> f32x16 {
    if constexpr (F8) return mfma_fp8(a, b, c);
    else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  };
  // QK product. fp8: Q is stored times c * 2^k (c = softmax scale * log2 e), and the Q
  // operand's E8M0 block scale 2^-k takes the power of two back, so scores come out in
  // base-2 units; the accumulators start from -m (the C operand), so they hold s - m.
  [[maybe_unused]] const int qk_scale = uniform(p.qk_scale_e8m0);
  auto mma_qk = [&](const Op& a, const Op& b, const f32x16& c) -> f32x16 {
    if constexpr (F8) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, qk_scale);
    else return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  };

  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = f32x16{};
  f32x16 sacc[MT];
  Op pb[PSTEPS];
  // running maximum (base 2): bf16 starts from -inf; fp8 from a 0 reference that its
  // first tile moves (scores arrive already shifted by -m there)
  float m = F8 ? 0.f : -__builtin_inff(), l = 0.f;
  // fp8: the row sums of the rounded weights come from one more MFMA per tile (the
  // MFMA unit has room, the VALU does not): its A operand is a constant matrix whose
  // row 0 is all E4M3 ones (0x38), so row 0 of the product accumulates
  // sum_k P[k][query]; it lands in element 0 of lanes 0-31 (query l % 32).
  [[maybe_unused]] f32x16 osum = f32x16{};
  // fp8: -m in every element, the C operand of each tile's first QK step. m starts as a
  // 0 reference; the first tile of a segment sets it.
  [[maybe_unused]] f32x16 negm = f32x16{};
  [[maybe_unused]] const int ones4 = l32 == 0 ? 0x38383838 : 0;
  [[maybe_unused]] const i32x8 ones_row = {ones4, ones4, ones4, ones4, ones4, ones4, ones4, ones4};

  auto qk = [&](int i) {
    const char* stage = smem + (i % STAGES) * G::BUF;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sacc[mt] = F8 ? negm : f32x16{};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) sacc[mt] = mma_qk(k_op(stage, s, mt), bq[s], sacc[mt]);
  };
  auto pv = [&](int i) {
    const char* stage = smem + (i % STAGES) * G::BUF;
#pragma unroll
    for (int s = 0; s < PSTEPS; ++s)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = mma(v_op(stage, s, dt), pb[s], o[dt]);
    if constexpr (F8) osum = mfma_fp8(ones_row, pb[0], osum);
  };
  auto softmax = [&](int i) {
    int lo, hi;
    const int key0 = visit(i, lo, hi) * BN;
    if ((GROUPS && key0 < lo) || key0 + BN > hi) {   // tile cut by its range (wave-uniform branch)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = F8 ? key0 + 32 * g + 16 * mt + j : key0 + 32 * mt + 16 * (j >> 3) + 8 * g + (j & 7);
          if (key < lo || key >= hi) sacc[mt][j] = -__builtin_inff();
        }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[mt][j]);
    if constexpr (F8) {
      // scores arrive as s - m in base 2; the first tile sets m (largest weight 2^4),
      // later tiles raise it when a weight would pass 2^8
      mx = fmaxf(mx, xor32(mx));
      const bool first = i == 0;
      if (first || __any(mx > kRescaleThreshold)) {
        const float dlt = first ? mx - kP8Shift : fmaxf(0.f, mx - kP8Shift);
        m += dlt;
        if (!first) {                            // o and osum are still zero on the first tile
          const float alpha = fast_exp2(-dlt);
          osum[0] *= alpha;                      // the other elements hold zeros
#pragma unroll
          for (int d = 0; d < DT; ++d) o[d] *= alpha;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = 0; j < 16; ++j) sacc[mt][j] -= dlt;
#pragma unroll
        for (int j = 0; j < 16; ++j) negm[j] = -m;
      }
#pragma unroll
      for (int w = 0; w < 8; ++w) {              // byte 16 a + j <- element j of accumulator a
        float e4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) e4[k] = fast_exp2(sacc[w >> 2][4 * (w & 3) + k]);
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e4[0], e4[1], 0, false);
        pb[0][w] = __builtin_amdgcn_cvt_pk_fp8_f32(e4[2], e4[3], lo, true);
      }
    } else {
      mx = fmaxf(mx, xor32(mx)) * p.scale_log2;
      if (__any(mx > m + kRescaleThreshold)) {
        const float m_new = fmaxf(m, mx);
        const float alpha = fast_exp2(m - m_new);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int d = 0; d < DT; ++d) o[d] *= alpha;
      }
      float rs = 0.f;
#pragma unroll
      for (int s = 0; s < PSTEPS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pvl = fast_exp2(fmaf(sacc[s >> 1][8 * (s & 1) + e], p.scale_log2, -m));
          rs += pvl;
          pb[s][e] = static_cast<__bf16>(pvl);
        }
      l += rs;
    }
  };

  // QK(i) and PV(i-1) interleaved: step k issues the K operand read and the QK
  // MFMA of (s = k / MT, mt = k % MT) and the V operand read and the PV MFMA of
  // (s = k / DT, dt = k % DT); the scheduling barriers keep two LDS reads ahead
  // of two MFMAs so the operand registers in flight stay bounded.
  static_assert(KSTEPS * MT == PSTEPS * DT, "QK and PV have the same MFMA count");
  auto qk_pv = [&](int i) {
    const char* ks = smem + (i % STAGES) * G::BUF;
    const char* vs = smem + ((i - 1) % STAGES) * G::BUF;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sacc[mt] = F8 ? negm : f32x16{};
#pragma unroll
    for (int k = 0; k < KSTEPS * MT; ++k) {
      const int s = k / MT, mt = k % MT;
      const int sv = k / DT, dt = k % DT;
      const Op a = k_op(ks, s, mt);
      const Op v = v_op(vs, sv, dt);
      sacc[mt] = mma_qk(a, bq[s], sacc[mt]);
      o[dt] = mma(v, pb[sv], o[dt]);
    }
    if constexpr (F8) osum = mfma_fp8(ones_row, pb[0], osum);
    constexpr int AHEAD = F8 ? 1 : PP_READ_AHEAD;          // steps of operand reads in flight
    constexpr int RD = F8 ? 4 : 2;                         // LDS reads per step
    __builtin_amdgcn_sched_group_barrier(0x100, RD * AHEAD, 0);  // operands of steps 0 .. AHEAD-1
#pragma unroll
    for (int k = 0; k < KSTEPS * MT; ++k) {
      if (k + AHEAD < KSTEPS * MT) __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);  // step k+AHEAD reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // step k MFMAs
    }
    if constexpr (F8) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // the row-sum MFMA
  };
  // Both groups run the same block sequence; waves 4-7 pass one extra barrier
  // first (and waves 0-3 one at the end), which offsets them by one block.
  // Before the barrier that opens global slot 2i every wave has waited for
  // its copies of tile i: for the leading group that barrier precedes M(i),
  // for the lagging group it precedes V(i-1).
  auto wait_tile = [&](int i) {                  // tile i complete; tile i + 1 may be in flight
    if (i + 1 < n) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_TILE));
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  // MFMAs touch no memory, so the compiler may sink them past the lagging group's wait
  // branch and below the barrier that ends their block, which puts both groups' MFMAs
  // into one phase; for the fp8 blocks it does. An empty asm that takes every
  // accumulator as an operand makes the block's MFMAs issue before that branch.
  auto block_end = [&] {
    if constexpr (F8) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) asm volatile("" : "+v"(sacc[mt]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) asm volatile("" : "+v"(o[dt]));
      asm volatile("" : "+v"(osum));
      asm volatile("" : "+v"(negm));
    }
  };
  issue_tile(0);
  if (n > 1) issue_tile(1);
  if (lag) {
    wait_tile(0);
    __syncthreads();
  }
  if (!lag) wait_tile(0);
  __syncthreads();
  if (n > 2) issue_tile(2);
  qk(0);                                         // M(0)
  block_end();
  if (lag && n > 1) wait_tile(1);
  __syncthreads();
  softmax(0);                                    // V(0)
  for (int i = 1; i < n; ++i) {
    if (!lag) wait_tile(i);
    __syncthreads();
    // bf16: the wave in its MFMA block (and the copies it issues) takes priority over the
    // other group's softmax on the same SIMD (measured: 1-2 % on one chunk, 5-6 % on the
    // group kernel); the VALU-bound fp8 blocks gain nothing from it
    if constexpr (!F8) __builtin_amdgcn_s_setprio(1);
    if (i + 2 < n) issue_tile(i + 2);
    qk_pv(i);                                    // M(i)
    block_end();
    if constexpr (!F8) __builtin_amdgcn_s_setprio(0);
    if (lag && i + 1 < n) wait_tile(i + 1);
    __syncthreads();
    softmax(i);                                  // V(i)
  }
  __syncthreads();
  pv(n - 1);                                     // M(n)
  if (!lag) __syncthreads();

  // ---- epilogue ---------------------------------------------------------------
  float l_tot;
  if constexpr (F8) {
    const float t = xor32(osum[0]);
    l_tot = g ? t : osum[0];
  } else {
    l_tot = l + xor32(l);
  }
  const float inv = 1.f / l_tot;
  const float lse2 = m + __log2f(l_tot);
  if (mode == kPpStreamK) {                      // partial rows of this q-tile, all BM of them
    const size_t row = static_cast<size_t>(slot) * BM + wave * 32 + l32;
    float* dst = p.sk_part_o + row * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<float4*>(dst + 32 * dt + 8 * jj + 4 * g) =
            make_float4(o[dt][4 * jj] * inv, o[dt][4 * jj + 1] * inv, o[dt][4 * jj + 2] * inv,
                        o[dt][4 * jj + 3] * inv);
    if (g == 0) p.sk_part_lse[row] = lse2;
    return;
  }
  if (q >= q_end) return;
  const int b = bh / p.H, h = bh - b * p.H;
  if (mode == kPpFinal) {
    __bf16* dst = static_cast<__bf16*>(bs.out) + ((static_cast<size_t>(b) * bs.rows + q) * p.H + h) * D;
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
    if (bs.lse != nullptr && g == 0) bs.lse[static_cast<size_t>(bh) * bs.rows + q] = lse2 * kLn2;
  } else {
    const size_t row = (static_cast<size_t>(slot) * p.B * p.H + bh) * p.Nc + q;
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

// First iteration of stream-K workgroup w: ranges [start(w), start(w + 1)) split
// the L = q-tiles * key-tiles iterations evenly.
__device__ __forceinline__ int64_t sk_start(int w, int64_t L, int G) { return (static_cast<int64_t>(w) * L) / G; }

// Ping-pong kernel driver. Grid mode: one workgroup per (b*h, split, q-tile).
// Stream-K mode (sk_groups > 0): sk_groups persistent workgroups, each running
// its range as segments; a segment that covers a whole q-tile writes the final
// rows, a partial one writes slot 2w (the range's first segment) or 2w + 1 (its
// last), merged afterwards by attn_sk_combine.
template <int D, bool GROUPS, bool F8>
__device__ __forceinline__ void chunk_attention_pp_body(const AttnParams& p) {
  __shared__ __attribute__((aligned(1024))) char smem[PpSmem<D, F8>::BYTES];
  if constexpr (GROUPS) {                        // moving buffer: the q-tile's chunk picks the keys
    const int w = xcd_remap(blockIdx.x, p.B * p.H * p.q_tiles);
    const int qt = uniform(w % p.q_tiles), bh = uniform(w / p.q_tiles);
    const int grp = uniform(qt / p.group_qtiles);
    const int qtg = qt - grp * p.group_qtiles;
    const int row0 = p.ragged ? 0 : grp * p.group_rows;   // a ragged group has rows of its own
    pp_segment<D, true, F8>(p, bases_group(p, grp), smem, bh, row0 + qtg * (8 * 32), row0 + p.group_rows, 0, 0,
                            keys_group(p, grp, Bf16Geom<D>::BN), kPpFinal, 0);
    return;
  }
  const bool sk = p.sk_groups > 0;
  const int T = p.key_tiles;
  // grid mode: one segment, the work item's (q-tile, split); stream-K: the range of w
  const int G = sk ? p.sk_groups : p.B * p.H * p.q_tiles * p.kv_splits;
  const int w = xcd_remap(blockIdx.x, G);
  const int64_t L = static_cast<int64_t>(p.B) * p.H * p.q_tiles * T;
  const int64_t r0 = sk ? sk_start(w, L, G) : 0, r1 = sk ? sk_start(w + 1, L, G) : 1;
  const KeyList none{};
  for (int64_t it = r0; it < r1;) {
    int bh, qt, t0, t1, mode, slot;
    if (sk) {
      const int64_t u = it / T;                  // q-tile index: bh * q_tiles + qt
      bh = static_cast<int>(u / p.q_tiles);
      qt = static_cast<int>(u % p.q_tiles);
      t0 = static_cast<int>(it - u * T);
      t1 = static_cast<int>(min(static_cast<int64_t>(T), r1 - u * T));
      mode = (t0 == 0 && t1 == T) ? kPpFinal : kPpStreamK;
      slot = 2 * w + (it == r0 ? 0 : 1);
      it = u * T + t1;
    } else {
      qt = w % p.q_tiles;
      const int rest = w / p.q_tiles;
      const int split = rest % p.kv_splits;
      bh = rest / p.kv_splits;
      t0 = static_cast<int>((static_cast<int64_t>(split) * T) / p.kv_splits);
      t1 = static_cast<int>((static_cast<int64_t>(split + 1) * T) / p.kv_splits);
      mode = p.kv_splits == 1 ? kPpFinal : kPpSplit;
      slot = split;
      it = r1;
    }
    pp_segment<D, false, F8>(p, bases_shared(p), smem, bh, qt * (8 * 32), p.Nc, t0, t1, none, mode, slot);
    if (it < r1) __syncthreads();                // the next segment reuses every LDS stage
  }
}

// ---- Software-pipelined schedule ("pipe") ---------------------------------------------------
// 8 waves x 32 query rows (BM = 256), two waves per SIMD and no lag between them: every wave
// streams MFMAs and softmax VALU work at once, so both waves of a SIMD feed its matrix pipe
// and the softmax runs under the MFMAs. Iteration j of a wave issues, in one straight block,
//   first half    QK(j)   S_j = K_j Q^T              16 MFMAs, K operands read from LDS
//   second half   PV(j-2) O^T += V_{j-2}^T P_{j-2}^T 16 MFMAs, V^T operands read from LDS
//   throughout    weights of tile j-1: P = 2^(S c - m_{j-1}), rounded to bf16, row sums
//   second half   row maximum of tile j (its scores are complete after the first half)
// The VALU work is software-pipelined (scale-and-shift of pair p+2, exponentials of pair
// p+1 and packing of pair p in one step), so no instruction waits on the one before it.
// Running maximum: m_j = max_j S c if that passes m_{j-1} by more than 2^8, else m_{j-1};
// the weights of tile j use m_j, and O_j = alpha_j O_{j-1} + P_j V_j, l_j = alpha_j l_{j-1} +
// sum P_j with alpha_j = 2^(m_{j-1} - m_j): alpha_{j-1} is applied to O at the end of
// iteration j, after PV(j-2) and before PV(j-1). Scores and weights alternate between two
// register sets with the parity of j.
// K and V^T tiles sit in separate LDS rings of kPipeStages stages. Iteration j issues the
// copies of K_{j+3} and V_{j+1}, both read at iteration j + 3; one barrier per iteration
// publishes the tiles iteration j reads and retires the stages its copies overwrite.
constexpr int kPipeStages = 4;

template <int D>
struct PipeSmem {
  static constexpr int BYTES = kPipeStages * (Bf16Geom<D>::KBYTES + Bf16Geom<D>::VBYTES);
};

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, N] (the instruction takes an immediate).
template <int N>
__device__ __forceinline__ void wait_vm_at_most(int n) {
  if constexpr (N <= 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (n >= N) __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
    else wait_vm_at_most<N - 1>(n);
  }
}

template <int D>
__device__ __forceinline__ void pipe_segment(const AttnParams& p, const Bases& bs, char* smem, int bh, int q_base,
                                             int q_end, int t_begin, int t_end, int mode, int slot) {
  using G = Bf16Geom<D>;
  constexpr int NW = 8, ST = kPipeStages;
  constexpr int BN = G::BN;
  constexpr int KSTEPS = D / 16, MT = BN / 32, DT = D / 32, PSTEPS = BN / 16;
  constexpr int NQK = KSTEPS * MT, NPV = PSTEPS * DT;   // MFMAs of QK and of PV per iteration
  static_assert(NQK == NPV && NQK % 2 == 0, "QK and PV halves of equal length");
  constexpr int HALF = NQK / 2;                  // steps per half (two MFMAs a step)
  constexpr int STEPS = 2 * HALF;
  constexpr int NEL = MT * 16;                   // scores per lane per tile
  constexpr int NPAIR = NEL / 2;
  static_assert(NPAIR <= STEPS, "at most one weight pair per step");
  constexpr int KC = G::KBYTES / 1024 / NW;      // 1 KB copies per wave per K tile
  constexpr int VC = G::VBYTES / 1024 / NW;
  static_assert(KC * NW * 1024 == G::KBYTES && VC * NW * 1024 == G::VBYTES, "copy split");
  static_assert(2 * (KC + VC) <= 63, "vmcnt range");
  char* const kring = smem;
  char* const vring = smem + ST * G::KBYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int n = t_end - t_begin;                 // key tiles of this work item (>= 1)
  const int n_keys = p.n_keys;

  const char* kbase = static_cast<const char*>(bs.kcache) + static_cast<size_t>(bh) * p.k_bh_stride * 2;
  const char* vbase = static_cast<const char*>(bs.vtcache) + static_cast<size_t>(bh) * p.vt_bh_stride * 2;

  const int q = q_base + wave * 32 + l32;
  bf16x8 bq[KSTEPS];                             // Q^T operand: lane l holds query l % 32
  {
    const int qrow = min(q, q_end - 1);
    const char* qsrc = static_cast<const char*>(bs.q) + (static_cast<size_t>(bh) * bs.rows + qrow) * D * 2;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) bq[s] = *reinterpret_cast<const bf16x8*>(qsrc + (16 * s + 8 * g) * 2);
  }

  // tile copies (the ping-pong kernel's swizzled images, K and V^T in separate rings)
  auto k_src = [&](int c) {
    const int P = (c * NW + wave) * 64 + lane;
    const int r = P / G::KC;
    return swap_bits23(r) * G::KROW + swz(P % G::KC, r, G::KC) * 16;
  };
  auto v_src = [&](int c) {
    const int P = (c * NW + wave) * 64 + lane;
    const int d = P / G::VC;
    return d * p.key_stride * 2 + swz(P % G::VC, d, G::VC) * 16;
  };
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, p.k_bh_stride * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, p.vt_bh_stride * 2);
  auto issue_k = [&](int i) {
    const int key0 = (t_begin + i) * BN;
    char* dst = kring + (i % ST) * G::KBYTES;
#pragma unroll
    for (int c = 0; c < KC; ++c) lds_copy16(krs, key0 * G::KROW + k_src(c), dst + (c * NW + wave) * 1024);
  };
  auto issue_v = [&](int i) {
    const int key0 = (t_begin + i) * BN;
    char* dst = vring + (i % ST) * G::VBYTES;
#pragma unroll
    for (int c = 0; c < VC; ++c) lds_copy16(vrs, key0 * 2 + v_src(c), dst + (c * NW + wave) * 1024);
  };
  // copies issued at iteration x: a full set (K_{x+3}, V_{x+1}, or nothing useful past the
  // end) from x = 0; the prologue (x = -3, -2, -1) issues K_{x+3} and, at x = -1, V_0
  auto set_size = [&](int x) {
    if (x >= 0) return KC + VC;
    return KC * ((x + 3 < n) ? 1 : 0) + VC * (x == -1 ? 1 : 0);
  };

  const int ka_row = l32 * G::KROW;
  auto k_op = [&](const char* ks, int s, int mt) {
    return *reinterpret_cast<const bf16x8*>(ks + ka_row + swz(2 * s + g, l32, G::KC) * 16 + mt * 32 * G::KROW);
  };
  auto v_op = [&](const char* vs, int s, int dt) {
    return *reinterpret_cast<const bf16x8*>(vs + l32 * G::VROW + swz(2 * s + g, l32, G::VC) * 16 + dt * 32 * G::VROW);
  };

  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = f32x16{};
  f32x16 sc[2][MT];                              // scores of tiles of parity 0 / 1
  bf16x8 pw[2][PSTEPS];                          // their weights
  // m: reference of the latest tile whose maximum is known; the weights of the tile before
  // it use m_prev (= m except right after that maximum moved it)
  float m = -__builtin_inff(), nm_w = 0.f, l = 0.f, alpha_prev = 1.f;
  bool raise_prev = false;
  const float c2 = p.scale_log2;
  const int tail_tile = (n_keys % BN) && (t_end == p.key_tiles) ? n - 1 : -1;

  // Iteration j: QK(j) and the maximum of tile j if QK, the weights of tile j-1 if SM, PV(j-2)
  // if PV; TAIL masks tile j's keys past n_keys before its maximum. STG = j % ST when known at
  // compile time (the LDS offsets then fold into the read instructions), else -1; PAR = j % 2.
  auto iteration = [&](int j, auto stg_c, auto par_c, auto qk_c, auto sm_c, auto pv_c, auto tail_c) {
    constexpr int STG = decltype(stg_c)::value, PAR = decltype(par_c)::value;
    constexpr bool QK = decltype(qk_c)::value, SM = decltype(sm_c)::value, PV = decltype(pv_c)::value;
    constexpr bool TAIL = decltype(tail_c)::value;
    static_assert(STG < 0 || STG % 2 == PAR, "stage and parity agree");
    // K_j and V_{j-2} (the copies of iteration j - 3) have landed for this wave; the copies of
    // iterations j - 2 and j - 1 may still be in flight. The barrier makes every wave's land.
    wait_vm_at_most<2 * (KC + VC)>(set_size(j - 2) + set_size(j - 1));
    __builtin_amdgcn_s_barrier();
    // this iteration's copies (K_{j+3}, V_{j+1}) go out one at a time through the block: all
    // eight waves issuing theirs right after the barrier queue on the memory issue path. They
    // are issued unconditionally (no branch splits the block): past the last tile the source
    // offset points beyond the buffer resource, which reads zeros, into stages nothing reads.
    constexpr int kFar = 0x40000000;             // past any (b, h) region (those stay below 2^31 bytes)
    const int kofs = j + 3 < n ? (t_begin + j + 3) * BN * G::KROW : kFar;
    const int vofs = j + 1 < n ? (t_begin + j + 1) * BN * 2 : kFar;
    char* const kdst = kring + ((j + 3) % ST) * G::KBYTES;
    char* const vdst = vring + ((j + 1) % ST) * G::VBYTES;
    auto copy_at = [&](int k) {                  // copy c of KC + VC at step k = (c + 1) * CP_EVERY - 2
      constexpr int NC = KC + VC, CP_EVERY = STEPS / NC;
      static_assert(CP_EVERY >= 2 && NC * CP_EVERY <= STEPS, "copy spacing");
      if ((k + 2) % CP_EVERY == 0 && (k + 2) / CP_EVERY <= NC) {
        const int c = (k + 2) / CP_EVERY - 1;
        if (c < KC) lds_copy16(krs, kofs + k_src(c), kdst + (c * NW + wave) * 1024);
        else lds_copy16(vrs, vofs + v_src(c - KC), vdst + ((c - KC) * NW + wave) * 1024);
      }
    };
    const int kst = STG >= 0 ? STG : j % ST;
    const int vst = STG >= 0 ? (STG + 2) % ST : (j + 2) % ST;   // (j - 2) mod ST
    const char* ks = kring + kst * G::KBYTES;
    const char* vs = vring + vst * G::VBYTES;

    // MFMA x of the iteration (x < NQK: QK step, else PV step) and its operand read
    constexpr int RA = 4, RB = RA + 2;           // reads in flight ahead of their MFMA; ring size (two reads
                                                 // are issued before the two MFMAs of a step)
    [[maybe_unused]] bf16x8 op[RB];
    auto has = [&](int x) { return x < NQK ? QK : PV; };
    auto read = [&](int x) {
      if (x < NQK) {
        if constexpr (QK) op[x % RB] = k_op(ks, x / MT, x % MT);
      } else {
        if constexpr (PV) op[x % RB] = v_op(vs, (x - NQK) / DT, (x - NQK) % DT);
      }
    };
    auto mfma = [&](int x) {
      if (x < NQK) {
        if constexpr (QK) {
          const int s = x / MT, mt = x % MT;
          sc[PAR][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[x % RB], bq[s], s == 0 ? f32x16{} : sc[PAR][mt],
                                                                0, 0, 0);
        }
      } else {
        if constexpr (PV) {
          const int s = (x - NQK) / DT, dt = (x - NQK) % DT;
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[x % RB], pw[PAR][s], o[dt], 0, 0, 0);
        }
      }
    };

    // weights of tile j - 1 (scores in sc[PAR ^ 1]); pair p = elements 2p, 2p + 1; element i
    // is accumulator (i / 8) >> 1, entry 8 ((i / 8) & 1) + i % 8, and goes to pw[i / 8][i % 8]
    f32x16* const sw = sc[PAR ^ 1];
    auto el = [](int i) { return 8 * ((i / 8) & 1) + i % 8; };
    [[maybe_unused]] float rs = 0.f;
    auto w_scale = [&](int pr) {                 // s c - m
      if (pr < NPAIR) {
        const int i = 2 * pr;
        sw[(i / 8) >> 1][el(i)] = fmaf(sw[(i / 8) >> 1][el(i)], c2, nm_w);
        sw[(i / 8) >> 1][el(i + 1)] = fmaf(sw[(i / 8) >> 1][el(i + 1)], c2, nm_w);
      }
    };
    auto w_exp = [&](int pr) {
      if (pr < NPAIR) {
        const int i = 2 * pr;
        sw[(i / 8) >> 1][el(i)] = fast_exp2(sw[(i / 8) >> 1][el(i)]);
        sw[(i / 8) >> 1][el(i + 1)] = fast_exp2(sw[(i / 8) >> 1][el(i + 1)]);
      }
    };
    auto w_pack = [&](int pr) {                  // bf16 pair; the row sum adds the rounded weights
      if (pr < NPAIR) {
        const int i = 2 * pr;
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 pk = {static_cast<__bf16>(sw[(i / 8) >> 1][el(i)]),
                           static_cast<__bf16>(sw[(i / 8) >> 1][el(i + 1)])};
        const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
        rs = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, rs, false);
        pw[PAR ^ 1][i / 8][i % 8] = pk[0];
        pw[PAR ^ 1][i / 8][i % 8 + 1] = pk[1];
      }
    };

    // maximum of tile j (scores in sc[PAR], complete after the first half): four independent
    // partial maxima over MAXSTEPS steps of the second half
    constexpr int MAX0 = HALF + 1, MAXSTEPS = HALF - 2;   // leave the first step for the MFMA latency
    constexpr int NCH = 4, PER = NEL / NCH;
    static_assert(NCH * PER == NEL, "max split");
    [[maybe_unused]] float part[NCH];
    [[maybe_unused]] const int key0 = (t_begin + j) * BN;
    auto sm_max = [&](int st) {                  // st = 0 .. MAXSTEPS - 1
      f32x16* const sm = sc[PAR];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        // chain c folds its elements c*PER .. c*PER+PER-1 in groups over the steps
        const int lo = c * PER + (st * PER) / MAXSTEPS, hi = c * PER + ((st + 1) * PER) / MAXSTEPS;
#pragma unroll
        for (int i = lo; i < hi; ++i) {
          if constexpr (TAIL) {
            const int kk = key0 + 32 * (i / 16) + 16 * ((i / 8) & 1) + 8 * g + i % 8;
            if (kk >= n_keys) sm[(i / 8) >> 1][el(i)] = -__builtin_inff();
          }
          const float x = sm[(i / 8) >> 1][el(i)];
          part[c] = (i == c * PER) ? x : __builtin_fmaxf(part[c], x);
        }
      }
    };

    if constexpr (SM) { w_scale(0); w_scale(1); w_exp(0); }
#pragma unroll
    for (int x = 0; x < RA; ++x)
      if (has(x)) read(x);
#pragma unroll
    for (int k = 0; k < STEPS; ++k) {
      const int x0 = 2 * k, x1 = 2 * k + 1;
      if (x0 + RA < 2 * STEPS && has(x0 + RA)) read(x0 + RA);
      if (x1 + RA < 2 * STEPS && has(x1 + RA)) read(x1 + RA);
      if (has(x0)) mfma(x0);
      copy_at(k);
      if constexpr (SM) w_scale(k + 2);
      if constexpr (QK) {
        if (k >= MAX0 && k < MAX0 + MAXSTEPS) sm_max(k - MAX0);
      }
      if (has(x1)) mfma(x1);
      if constexpr (SM) { w_exp(k + 1); w_pack(k); }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the block's results are produced inside it (without this the compiler sinks the
    // softmax past the branches below, into the next iteration)
    if constexpr (SM) {
#pragma unroll
      for (int s2 = 0; s2 < PSTEPS; ++s2) asm volatile("" : "+v"(pw[PAR ^ 1][s2]));
      asm volatile("" : "+v"(rs));
    }
    if constexpr (QK) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) asm volatile("" : "+v"(part[c]));
    }
    if constexpr (SM) {
      l = fmaf(l, alpha_prev, rs);
      if (raise_prev) {                          // rare: tile j-1 moved the reference by more than 2^8
#pragma unroll
        for (int d = 0; d < DT; ++d) o[d] *= alpha_prev;
      }
    }
    if constexpr (QK) {
      float mx = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
      mx = fmaxf(mx, xor32(mx)) * c2;
      const float m_new = mx > m + kRescaleThreshold ? mx : m;
      raise_prev = __any(m_new != m);
      alpha_prev = fast_exp2(m - m_new);
      m = m_new;
      nm_w = -m_new;
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  using SR = std::integral_constant<int, -1>;   // stage computed at run time
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  // prologue copies: K_0 (iteration -3), K_1 (-2), K_2 and V_0 (-1)
  issue_k(0);
  if (n > 1) issue_k(1);
  if (n > 2) issue_k(2);
  issue_v(0);
  const bool tail = tail_tile == n - 1;          // the last tile is ragged
  if (n == 1) {
    if (tail) iteration(0, S0{}, P0{}, T_{}, F_{}, F_{}, T_{});
    else iteration(0, S0{}, P0{}, T_{}, F_{}, F_{}, F_{});
    iteration(1, S1{}, P1{}, F_{}, T_{}, F_{}, F_{});
    iteration(2, S2{}, P0{}, F_{}, F_{}, T_{}, F_{});
  } else {
    iteration(0, S0{}, P0{}, T_{}, F_{}, F_{}, F_{});
    int j = 1;
    if (n > 2) {
      iteration(1, S1{}, P1{}, T_{}, T_{}, F_{}, F_{});
      // full iterations j = 2 .. n - 2, four at a time (stages 2, 3, 0, 1)
      j = 2;
      for (; j + 3 < n - 1; j += 4) {
        iteration(j, S2{}, P0{}, T_{}, T_{}, T_{}, F_{});
        iteration(j + 1, S3{}, P1{}, T_{}, T_{}, T_{}, F_{});
        iteration(j + 2, S0{}, P0{}, T_{}, T_{}, T_{}, F_{});
        iteration(j + 3, S1{}, P1{}, T_{}, T_{}, T_{}, F_{});
      }
      if (j < n - 1) { iteration(j, S2{}, P0{}, T_{}, T_{}, T_{}, F_{}); ++j; }
      if (j < n - 1) { iteration(j, S3{}, P1{}, T_{}, T_{}, T_{}, F_{}); ++j; }
      if (j < n - 1) { iteration(j, S0{}, P0{}, T_{}, T_{}, T_{}, F_{}); ++j; }
    }
    // j = n - 1: the last QK (masked when ragged); j = n: weights of the last tile; j = n + 1
    const bool pv = n > 2;                       // PV(n - 3) exists at j = n - 1
    if ((n - 1) & 1) {
      if (pv) {
        if (tail) iteration(n - 1, SR{}, P1{}, T_{}, T_{}, T_{}, T_{});
        else iteration(n - 1, SR{}, P1{}, T_{}, T_{}, T_{}, F_{});
      } else {
        if (tail) iteration(n - 1, SR{}, P1{}, T_{}, T_{}, F_{}, T_{});
        else iteration(n - 1, SR{}, P1{}, T_{}, T_{}, F_{}, F_{});
      }
      iteration(n, SR{}, P0{}, F_{}, T_{}, T_{}, F_{});
      iteration(n + 1, SR{}, P1{}, F_{}, F_{}, T_{}, F_{});
    } else {
      if (tail) iteration(n - 1, SR{}, P0{}, T_{}, T_{}, T_{}, T_{});
      else iteration(n - 1, SR{}, P0{}, T_{}, T_{}, T_{}, F_{});
      iteration(n, SR{}, P1{}, F_{}, T_{}, T_{}, F_{});
      iteration(n + 1, SR{}, P0{}, F_{}, F_{}, T_{}, F_{});
    }
  }

  // ---- epilogue ---------------------------------------------------------------
  const float l_tot = l + xor32(l);
  const float inv = 1.f / l_tot;
  const float lse2 = m + __log2f(l_tot);
  if (q >= q_end) return;
  const int b = bh / p.H, h = bh - b * p.H;
  if (mode == kPpFinal) {
    __bf16* dst = static_cast<__bf16*>(bs.out) + ((static_cast<size_t>(b) * bs.rows + q) * p.H + h) * D;
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
    if (bs.lse != nullptr && g == 0) bs.lse[static_cast<size_t>(bh) * bs.rows + q] = lse2 * kLn2;
  } else {
    const size_t row = (static_cast<size_t>(slot) * p.B * p.H + bh) * p.Nc + q;
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

// Pipelined kernel driver: one workgroup per (b*h, split, q-tile).
template <int D>
__device__ __forceinline__ void chunk_attention_pipe_body(const AttnParams& p) {
  __shared__ __attribute__((aligned(1024))) char smem[PipeSmem<D>::BYTES];
  const int G = p.B * p.H * p.q_tiles * p.kv_splits;
  const int w = xcd_remap(blockIdx.x, G);
  const int T = p.key_tiles;
  const int qt = w % p.q_tiles;
  const int rest = w / p.q_tiles;
  const int split = rest % p.kv_splits;
  const int bh = rest / p.kv_splits;
  const int t0 = static_cast<int>((static_cast<int64_t>(split) * T) / p.kv_splits);
  const int t1 = static_cast<int>((static_cast<int64_t>(split + 1) * T) / p.kv_splits);
  pipe_segment<D>(p, bases_shared(p), smem, bh, qt * (8 * 32), p.Nc, t0, t1,
                  p.kv_splits == 1 ? kPpFinal : kPpSplit, split);
}

__global__ __launch_bounds__(kThreads, 2) void chunk_attention_bf16_d128(AttnParams p) {
  chunk_attention_bf16_body<128, 4, 1, 2>(p);
}

__global__ __launch_bounds__(kThreads, 2) void chunk_attention_bf16_d64(AttnParams p) {
  chunk_attention_bf16_body<64, 4, 1, 2>(p);
}

__global__ __launch_bounds__(kThreads, 1) void chunk_attention_bf16_d128_q64(AttnParams p) {
  chunk_attention_bf16_body<128, 4, 2, 2>(p);
}

__global__ __launch_bounds__(kThreads, 1) void chunk_attention_bf16_d64_q64(AttnParams p) {
  chunk_attention_bf16_body<64, 4, 2, 2>(p);
}

__global__ __launch_bounds__(2 * kThreads, 2) void chunk_attention_bf16_d128_pp(AttnParams p) {
  chunk_attention_pp_body<128, false, false>(p);
}

__global__ __launch_bounds__(2 * kThreads, 2) void chunk_attention_bf16_d64_pp(AttnParams p) {
  chunk_attention_pp_body<64, false, false>(p);
}

__global__ __launch_bounds__(2 * kThreads, 2) void chunk_attention_bf16_d128_pipe(AttnParams p) {
  chunk_attention_pipe_body<128>(p);
}

// moving-buffer attend: query groups with their own key ranges
__global__ __launch_bounds__(2 * kThreads, 2) void chunk_attention_bf16_d128_ppg(AttnParams p) {
  chunk_attention_pp_body<128, true, false>(p);
}

__global__ __launch_bounds__(2 * kThreads, 2) void chunk_attention_bf16_d64_ppg(AttnParams p) {
  chunk_attention_pp_body<64, true, false>(p);
}

// fp8 cache (E4M3 Q, K, V^T; P rounded to E4M3): the same schedule on the fp8 MFMA
__global__ __launch_bounds__(2 * kThreads, 2) void chunk_attention_fp8_d128_pp(AttnParams p) {
  chunk_attention_pp_body<128, false, true>(p);
}

__global__ __launch_bounds__(2 * kThreads, 2) void chunk_attention_fp8_d128_ppg(AttnParams p) {
  chunk_attention_pp_body<128, true, true>(p);
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
  int q_base = qt * kF32BlockM, q_end = p.Nc;
  KeyList kl;
  Bases bs = bases_shared(p);
  if (p.n_groups > 0) {                          // moving buffer or ragged batch: the q-tile's group
    const int grp = qt / p.group_qtiles;
    const int row0 = p.ragged ? 0 : grp * p.group_rows;
    q_base = row0 + (qt - grp * p.group_qtiles) * kF32BlockM;
    q_end = row0 + p.group_rows;
    kl = keys_group(p, grp, BN);
    bs = bases_group(p, grp);
  } else {
    kl = keys_single(p, t_begin, t_end);
  }
  const float* kbase = static_cast<const float*>(bs.kcache) + static_cast<size_t>(bh) * p.k_bh_stride;
  const float* vbase = static_cast<const float*>(bs.vtcache) + static_cast<size_t>(bh) * p.vt_bh_stride;
  const int q = q_base + lane;
  const int qrow = min(q, q_end - 1);
  const float* qsrc = static_cast<const float*>(bs.q) + (static_cast<size_t>(bh) * bs.rows + qrow) * D;
  float qr[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = qsrc[d] * p.scale_log2;
    o[d] = 0.f;
  }
  float m = -__builtin_inff(), l = 0.f;
  for (int t = 0; t < kl.total; ++t) {
    int lo, hi;
    const int key0 = key_tile(kl, t, lo, hi) * BN;
    const int r_lo = max(0, lo - key0), r_hi = min(BN, hi - key0);   // keys of the tile in range
    for (int i = lane; i < BN * D; i += 64) {
      const int r = i / D, d = i - r * D;
      sk[r][d] = r >= r_lo && r < r_hi ? kbase[static_cast<size_t>(key0 + r) * D + d] : 0.f;
    }
    for (int i = lane; i < BN * D; i += 64) {
      const int d = i / BN, r = i - d * BN;
      sv[r][d] = r >= r_lo && r < r_hi ? vbase[static_cast<size_t>(d) * p.key_stride + key0 + r] : 0.f;
    }
    __syncthreads();
    for (int r = r_lo; r < r_hi; ++r) {
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
  if (q >= q_end) return;
  const float inv = 1.f / l;
  const float lse2 = m + __log2f(l);
  const int b = bh / p.H, h = bh - b * p.H;
  if (p.kv_splits == 1) {
    float* dst = static_cast<float*>(bs.out) + ((static_cast<size_t>(b) * bs.rows + q) * p.H + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) dst[d] = o[d] * inv;
    if (bs.lse != nullptr) bs.lse[static_cast<size_t>(bh) * bs.rows + q] = lse2 * kLn2;
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

// Merge the stream-K partials of one q-tile (block u): slots of the workgroups
// whose ranges cut it; unsplit q-tiles were written directly and are skipped.
template <typename T>
__global__ __launch_bounds__(kThreads) void attn_sk_combine(AttnParams p) {
  constexpr int kMaxParts = 16;                  // workgroups cutting one q-tile (checked on the host)
  __shared__ int s_slot[kMaxParts];
  __shared__ int s_n;
  const int u = blockIdx.x;
  const int G = p.sk_groups, T_ = p.key_tiles, BM = p.q_rows_per_block;
  if (threadIdx.x == 0) {
    const int64_t L = static_cast<int64_t>(p.B) * p.H * p.q_tiles * T_;
    const int64_t first = static_cast<int64_t>(u) * T_, last = first + T_ - 1;
    const int w0 = static_cast<int>(((first + 1) * G + L - 1) / L - 1);   // workgroup holding iteration first
    const int w1 = static_cast<int>(((last + 1) * G + L - 1) / L - 1);
    int n = 0;
    if (w0 != w1)
      for (int w = w0; w <= w1 && n < kMaxParts; ++w) s_slot[n++] = 2 * w + (sk_start(w, L, G) < first ? 1 : 0);
    s_n = n;
  }
  __syncthreads();
  const int n = s_n;
  if (n == 0) return;                            // unsplit: written by the attention kernel
  const int bh = u / p.q_tiles, qt = u % p.q_tiles;
  const int b = bh / p.H, h = bh - b * p.H;
  const int groups = p.D / 4;
  const int rows = min(BM, p.Nc - qt * BM);
  for (int idx = threadIdx.x; idx < rows * groups; idx += kThreads) {
    const int r = idx / groups, c4 = idx - r * groups;
    const int q = qt * BM + r;
    float mx = -__builtin_inff();
    for (int j = 0; j < n; ++j) mx = fmaxf(mx, p.sk_part_lse[static_cast<size_t>(s_slot[j]) * BM + r]);
    float wsum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < n; ++j) {
      const size_t row = static_cast<size_t>(s_slot[j]) * BM + r;
      const float wt = fast_exp2(p.sk_part_lse[row] - mx);
      const float4 v = *reinterpret_cast<const float4*>(p.sk_part_o + row * p.D + 4 * c4);
      wsum += wt;
      acc.x = fmaf(wt, v.x, acc.x);
      acc.y = fmaf(wt, v.y, acc.y);
      acc.z = fmaf(wt, v.z, acc.z);
      acc.w = fmaf(wt, v.w, acc.w);
    }
    const float inv = 1.f / wsum;
    T* dst = static_cast<T*>(p.out) + ((static_cast<size_t>(b) * p.Nc + q) * p.H + h) * p.D + 4 * c4;
    dst[0] = static_cast<T>(acc.x * inv);
    dst[1] = static_cast<T>(acc.y * inv);
    dst[2] = static_cast<T>(acc.z * inv);
    dst[3] = static_cast<T>(acc.w * inv);
    if (p.lse != nullptr && c4 == 0) p.lse[static_cast<size_t>(bh) * p.Nc + q] = (mx + __log2f(wsum)) * kLn2;
  }
}

// Measurement aid, not part of the attention path: 4 waves, each issuing
// v_mfma_f32_32x32x16_bf16 on 8 independent accumulators (the issue pattern
// that keeps one wave's matrix pipe full), `iters` rounds. Operands are fixed
// per lane (benign data: few toggling bits). One launch performs
// blocks * 4 * iters * 8 * 32768 flops; every lane writes one float.
__global__ __launch_bounds__(kThreads) void mfma_probe_bf16(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(((lane * 7 + i) % 13) * 0.01f);
    b[i] = static_cast<__bf16>(((lane * 5 + i) % 11) * 0.02f);
  }
  f32x16 c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += c[j][i];
  out[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = sum;
}

// The same MFMA stream on caller data: lane l of every wave takes four A and two B operands
// (16 bytes each, run i of 64 lanes at ops[64 i + l]) and MFMA j of a round uses A[j % 4] and
// B[j % 2], so the operand values change from one MFMA to the next as in a real product.
__global__ __launch_bounds__(kThreads) void mfma_probe_bf16_data(float* out, const bf16x8* ops, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = ops[64 * i + lane];
#pragma unroll
  for (int i = 0; i < 2; ++i) b[i] = ops[64 * (4 + i) + lane];
  f32x16 c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[j & 1], c[j], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += c[j][i];
  out[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = sum;
}

}  // namespace

hipError_t launch_chunk_attention(const AttnParams& p, int dtype, hipStream_t st) {
  const int64_t n_work =
      p.sk_groups > 0 ? p.sk_groups : static_cast<int64_t>(p.B) * p.H * p.q_tiles * p.kv_splits;
  if (n_work <= 0) return hipSuccess;
  if (dtype == 2) {                              // fp8 cache: head_dim 128 only (checked by the host)
    hipLaunchKernelGGL(p.n_groups > 0 ? chunk_attention_fp8_d128_ppg : chunk_attention_fp8_d128_pp, dim3(n_work),
                       dim3(2 * kThreads), 0, st, p);
  } else if (dtype == 1) {
    if (p.n_groups > 0) {
      hipLaunchKernelGGL(p.D == 128 ? chunk_attention_bf16_d128_ppg : chunk_attention_bf16_d64_ppg, dim3(n_work),
                         dim3(2 * kThreads), 0, st, p);
    } else if (p.variant == 4 && p.D == 128) {
      hipLaunchKernelGGL(chunk_attention_bf16_d128_pipe, dim3(n_work), dim3(2 * kThreads), 0, st, p);
    } else if (p.variant == 3 || p.variant == 4) {
      hipLaunchKernelGGL(p.D == 128 ? chunk_attention_bf16_d128_pp : chunk_attention_bf16_d64_pp, dim3(n_work),
                         dim3(2 * kThreads), 0, st, p);
    } else {
      auto k = p.variant == 2 ? (p.D == 128 ? chunk_attention_bf16_d128_q64 : chunk_attention_bf16_d64_q64)
                              : (p.D == 128 ? chunk_attention_bf16_d128 : chunk_attention_bf16_d64);
      hipLaunchKernelGGL(k, dim3(n_work), dim3(kThreads), 0, st, p);
    }
  } else {
    if (p.D == 128) hipLaunchKernelGGL(chunk_attention_f32<128>, dim3(n_work), dim3(64), 0, st, p);
    else hipLaunchKernelGGL(chunk_attention_f32<64>, dim3(n_work), dim3(64), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_mfma_probe(float* out, int blocks, int iters, hipStream_t st) {
  hipLaunchKernelGGL(mfma_probe_bf16, dim3(blocks), dim3(kThreads), 0, st, out, iters);
  return hipGetLastError();
}

hipError_t launch_mfma_probe_data(float* out, const void* ops, int blocks, int iters, hipStream_t st) {
  hipLaunchKernelGGL(mfma_probe_bf16_data, dim3(blocks), dim3(kThreads), 0, st, out, static_cast<const bf16x8*>(ops),
                     iters);
  return hipGetLastError();
}

hipError_t launch_attn_sk_combine(const AttnParams& p, hipStream_t st) {
  const int n_qt = p.B * p.H * p.q_tiles;
  if (n_qt <= 0 || p.sk_groups <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_sk_combine<__bf16>, dim3(n_qt), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const CombineParams& p, int dtype, hipStream_t st) {
  const int64_t total = static_cast<int64_t>(p.B) * p.H * p.Nc * (p.D / 4);
  if (total <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((total + kThreads - 1) / kThreads));
  if (dtype == 1 || dtype == 2) hipLaunchKernelGGL(attn_combine<__bf16>, grid, dim3(kThreads), 0, st, p);
  else hipLaunchKernelGGL(attn_combine<float>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace sa
