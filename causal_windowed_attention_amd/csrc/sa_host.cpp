// Host side of the streaming chunk attention library: config validation,
// workspace layout, stream bookkeeping (sink, window ring, positions), launch
// planning and the C ABI declared in include/sa.h.
//
// Cache layout. Per (b, h) the cache has n_slots = S + W + 1 physical chunk
// slots: slots [0, S) hold the sink, slots [S, S + W + 1) are the window ring.
// The ring has one slot more than the window so the chunk being attended can
// be staged in the slot that holds no visible chunk: the r-th window commit
// lands in ring slot r mod (W + 1), and the next chunk is staged in ring slot
// ring_commits mod (W + 1) (or in the next sink slot while the sink fills).
// A commit of the staged chunk therefore needs no copy. With this assignment
// the slots the next attend sees (committed sink chunks, the last min(r, W)
// window commits and the staging slot) are always the physical prefix
// [0, visible_chunks), so the attention kernel reads one contiguous key range
// per (b, h) and skips everything else.
//
// Stream semantics follow StreamDiffusionV2 ("Sommario tecnico" 2.A.1: chunked
// B x T' x H x W processing; 2.A.2: sink updates and periodic RoPE offset
// resets at chunk boundaries) and SANA-Streaming ("Transformer a diffusione
// ibrido": softmax over a sliding local window plus a persistent sink chunk).
#include "../../include/sa.h"
#include "sa_internal.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

namespace {

using sa::AttnParams;
using sa::CombineParams;
using sa::RefreshParams;
using sa::RopeWriteParams;
static_assert(sa::kMaxBatchStreams == SA_MAX_BATCH_STREAMS, "one batched RoPE launch per sa_batch_attend");
static_assert(sa::kMaxBatchStreams >= SA_MAX_BUFFER_CHUNKS, "one batched RoPE launch per sa_buffer_attend");

constexpr size_t kAlign = 256;
constexpr int32_t kMaxPosition = 1 << 30;   // guard against int32 overflow when max_t == 0
constexpr int kSkGroups = 256;              // persistent workgroups of the stream-K schedule (one per CU)

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Derived {
  int32_t B, H, D, Hf, Wf, F, S, W, R, n_slots, NB, buf_slot0, Nc, dt, dh, dw, max_t, dtype, elem;
  int32_t key_stride, q_tiles, max_splits;
  double theta;
  float scale;
  float q_scale;             // fp8: scale * log2(e) * 2^k in [1, 2), applied to rotated Q
  int32_t qk_scale_e8m0;     // fp8: 127 - k, the E8M0 block scale that takes 2^k back
  size_t k_off, k_bytes, vt_off, vt_bytes, q_off, q_bytes, part_off, part_bytes, sk_off, sk_bytes, tab_off,
      tab_bytes, total;
};

sa_status derive(const sa_config* c, Derived* d) {
  if (c == nullptr) return SA_ERR_INVALID_ARGUMENT;
  if (c->batch < 1 || c->heads < 1 || c->frame_h < 1 || c->frame_w < 1 || c->frames_per_chunk < 1 ||
      c->sink_chunks < 0 || c->window_chunks < 0 || c->max_t < 0 || c->head_dim < 2 ||
      c->head_dim % 2 != 0)
    return SA_ERR_INVALID_ARGUMENT;
  if (c->dtype != SA_F32 && c->dtype != SA_BF16 && c->dtype != SA_FP8) return SA_ERR_INVALID_ARGUMENT;
  if (c->max_buffer_chunks < 0 || c->max_buffer_chunks > SA_MAX_BUFFER_CHUNKS || c->reserved != 0)
    return SA_ERR_INVALID_ARGUMENT;
  if (!(c->rope_theta >= 0.0) || !(c->softmax_scale >= 0.f) || !std::isfinite(c->rope_theta) ||
      !std::isfinite(c->softmax_scale))
    return SA_ERR_INVALID_ARGUMENT;
  if (c->rope_theta != 0.0 && c->rope_theta <= 1.0) return SA_ERR_INVALID_ARGUMENT;
  d->B = c->batch; d->H = c->heads; d->D = c->head_dim; d->Hf = c->frame_h; d->Wf = c->frame_w;
  d->F = c->frames_per_chunk; d->S = c->sink_chunks; d->W = c->window_chunks; d->max_t = c->max_t;
  d->dtype = c->dtype;
  d->elem = c->dtype == SA_BF16 ? 2 : c->dtype == SA_FP8 ? 1 : 4;   // cache and Q scratch element
  if (c->rope_dim_t == 0 && c->rope_dim_h == 0 && c->rope_dim_w == 0) {
    d->dh = d->dw = 2 * (d->D / 6);
    d->dt = d->D - 2 * d->dh;
  } else {
    d->dt = c->rope_dim_t; d->dh = c->rope_dim_h; d->dw = c->rope_dim_w;
    if (d->dt < 0 || d->dh < 0 || d->dw < 0 || d->dt % 2 || d->dh % 2 || d->dw % 2 ||
        d->dt + d->dh + d->dw != d->D)
      return SA_ERR_INVALID_ARGUMENT;
  }
  const int64_t nc = static_cast<int64_t>(d->F) * d->Hf * d->Wf;
  if (nc > (1 << 20)) return SA_ERR_UNSUPPORTED;
  d->Nc = static_cast<int32_t>(nc);
  if (static_cast<int64_t>(d->S) + d->W + 1 > (1 << 16)) return SA_ERR_UNSUPPORTED;
  d->R = d->W + 1;
  d->n_slots = d->S + d->R;
  d->NB = c->max_buffer_chunks;
  d->buf_slot0 = d->n_slots;                     // buffer chunk i lives in slot n_slots + i
  const int64_t keys = static_cast<int64_t>(d->n_slots + d->NB) * d->Nc;
  if (keys > (1 << 24)) return SA_ERR_UNSUPPORTED;
  if (d->D != 64 && d->D != 128) return SA_ERR_UNSUPPORTED;
  if (d->dtype == SA_FP8 && d->D != 128) return SA_ERR_UNSUPPORTED;   // one fp8 kernel: D = 128
  if (static_cast<int64_t>(d->F) * (d->dt / 2) > sa::kMaxTemporalPairs) return SA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(d->B) * d->H > 65535) return SA_ERR_UNSUPPORTED;
  if (d->max_t > 0 && static_cast<int64_t>(d->S) * d->F > d->max_t) return SA_ERR_POSITION_RANGE;
  d->theta = c->rope_theta == 0.0 ? 10000.0 : c->rope_theta;
  d->scale = c->softmax_scale == 0.f ? static_cast<float>(1.0 / std::sqrt(static_cast<double>(d->D)))
                                     : c->softmax_scale;
  d->q_scale = 1.f;
  d->qk_scale_e8m0 = 127;
  if (d->dtype == SA_FP8) {
    // scores leave the fp8 product in base-2 units: Q is stored times c * 2^k (in [1, 2))
    // and the product multiplies by 2^-k through the Q operand's E8M0 block scale
    const double c = static_cast<double>(d->scale) * 1.4426950408889634;
    const int k = -static_cast<int>(std::floor(std::log2(c)));
    if (k < -126 || k > 126) return SA_ERR_UNSUPPORTED;
    d->q_scale = static_cast<float>(c * std::ldexp(1.0, k));
    d->qk_scale_e8m0 = 127 - k;
  }
  d->key_stride = static_cast<int32_t>(align_up(static_cast<size_t>(keys), 64));
  // bf16 tile copies address one (b, h) region through a buffer resource (32-bit offsets)
  if (static_cast<int64_t>(d->key_stride) * d->D * d->elem >= (int64_t{1} << 31)) return SA_ERR_UNSUPPORTED;
  const int bm = d->dtype != SA_F32 ? sa::kBf16BlockM : sa::kF32BlockM;
  d->q_tiles = (d->Nc + bm - 1) / bm;
  // partial buffers only where splitting can help filling the chip
  const int64_t blocks = static_cast<int64_t>(d->B) * d->H * d->q_tiles;
  int64_t ms = (1024 + blocks - 1) / blocks;
  d->max_splits = static_cast<int32_t>(ms < 1 ? 1 : (ms > sa::kMaxKvSplits ? sa::kMaxKvSplits : ms));

  const size_t bh = static_cast<size_t>(d->B) * d->H;
  // K rows padded to key_stride per (b, h): a key tile never leaves the allocation
  d->k_bytes = bh * static_cast<size_t>(d->key_stride) * d->D * d->elem;
  d->vt_bytes = bh * static_cast<size_t>(d->D) * d->key_stride * d->elem;
  d->q_bytes = bh * static_cast<size_t>(d->NB > 1 ? d->NB : 1) * d->Nc * d->D * d->elem;
  d->part_bytes = d->max_splits > 1
                      ? static_cast<size_t>(d->max_splits) * bh * d->Nc * (static_cast<size_t>(d->D) + 1) * 4
                      : 0;
  // stream-K partials: 2 slots per persistent workgroup, BlockM rows of D + 1 floats
  d->sk_bytes = d->dtype != SA_F32
                    ? static_cast<size_t>(2 * kSkGroups) * sa::kBf16BlockMWide * (static_cast<size_t>(d->D) + 1) * 4
                    : 0;
  d->tab_bytes = (static_cast<size_t>(d->Hf) * (d->dh / 2) + static_cast<size_t>(d->Wf) * (d->dw / 2)) * 8;
  size_t off = 0;
  d->k_off = off; off = align_up(off + d->k_bytes, kAlign);
  d->vt_off = off; off = align_up(off + d->vt_bytes, kAlign);
  d->q_off = off; off = align_up(off + d->q_bytes, kAlign);
  d->part_off = off; off = align_up(off + d->part_bytes, kAlign);
  d->sk_off = off; off = align_up(off + d->sk_bytes, kAlign);
  d->tab_off = off; off = align_up(off + d->tab_bytes, kAlign);   // padded: the RoPE kernels copy it in 16-byte pieces
  d->total = off;
  return SA_OK;
}

struct SlotMeta {
  int32_t kind = SA_SLOT_EMPTY;
  int64_t chunk_id = 0;
  int32_t t0 = 0;
};

struct Prof {
  double total_ms = 0.0;
  int64_t launches = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> free_pairs;
};

}  // namespace

struct sa_stream {
  Derived d;
  char* ws = nullptr;          // null: planning handle
  // state (D3)
  int64_t n_appends = 0, ring_commits = 0;
  int32_t t_next = 0, sink_fill = 0;
  std::vector<SlotMeta> slots;
  bool staged_valid = false;
  int32_t staged_t = 0, staged_slot = -1;
  // last plan (D4)
  int32_t last_q_tiles = 0, last_kv_splits = 0, last_key_tiles = 0, last_delta = 0;
  int32_t kv_splits_opt = 0;
  int32_t variant_opt = 0;
  int32_t schedule_opt = 0;
  int32_t last_sk_groups = 0;
  bool profile = false;
  Prof prof[SA_K_COUNT];

  int32_t window_valid() const {
    if (sink_fill < d.S) return 0;
    return static_cast<int32_t>(ring_commits < d.W ? ring_commits : d.W);
  }
  int32_t staging_slot() const {
    if (sink_fill < d.S) return sink_fill;
    return d.S + static_cast<int32_t>(ring_commits % d.R);
  }
  int32_t visible_chunks() const { return sink_fill + window_valid() + 1; }
  bool planning() const { return ws == nullptr; }
  void* kcache() const { return ws + d.k_off; }
  void* vtcache() const { return ws + d.vt_off; }
  void* qscratch() const { return ws + d.q_off; }
  const float2* h_cs() const { return reinterpret_cast<const float2*>(ws + d.tab_off); }
  const float2* w_cs() const { return h_cs() + static_cast<size_t>(d.Hf) * (d.dh / 2); }
};

namespace {

sa_status positions_ok(const sa_stream* s, int64_t last_pos_exclusive) {
  if (s->d.max_t > 0 && last_pos_exclusive > s->d.max_t) return SA_ERR_POSITION_RANGE;
  if (last_pos_exclusive > kMaxPosition) return SA_ERR_POSITION_RANGE;
  return SA_OK;
}

double freq(const Derived& d, int seg_len, int j) {
  return std::pow(d.theta, -2.0 * j / seg_len);
}

// Temporal (cos, sin) table for frames t0 .. t0+F-1: [frame][d_t/2].
void fill_temporal(const Derived& d, int64_t t0, int n_frames, float2* out) {
  const int np = d.dt / 2;
  for (int f = 0; f < n_frames; ++f)
    for (int j = 0; j < np; ++j) {
      const double a = static_cast<double>(t0 + f) * freq(d, d.dt, j);
      out[f * np + j] = make_float2(static_cast<float>(std::cos(a)), static_cast<float>(std::sin(a)));
    }
}

void base_write_params(const sa_stream* s, RopeWriteParams* p) {
  std::memset(p, 0, sizeof(*p));
  const Derived& d = s->d;
  p->q_scale = d.q_scale;
  p->kcache = s->kcache();
  p->vtcache = s->vtcache();
  p->h_cs = s->h_cs();
  p->w_cs = s->w_cs();
  p->k_bh_stride = static_cast<int64_t>(d.key_stride) * d.D;
  p->vt_bh_stride = static_cast<int64_t>(d.D) * d.key_stride;
  p->key_stride = d.key_stride;
  p->n_tokens = d.Nc;
  p->in_tokens = d.Nc;
  p->B = d.B; p->H = d.H; p->D = d.D; p->Hf = d.Hf; p->Wf = d.Wf;
  p->dt = d.dt; p->dh = d.dh; p->dw = d.dw;
  p->n_frames = d.F;
  p->q_rows = d.Nc;
}

// The geometry of one batched rope_apply launch over n entries of stream s's configuration:
// each entry's chunk has Nc tokens, its inputs hold in_tokens tokens per batch entry and its Q
// scratch q_rows rows per (b, h). The per-entry pointers, rows and positions are the caller's.
void base_batch_params(const sa_stream* s, int32_t n, int32_t in_tokens, int32_t q_rows, sa::RopeBatchParams* p) {
  RopeWriteParams rp;
  base_write_params(s, &rp);
  const Derived& d = s->d;
  std::memset(p, 0, sizeof(*p));
  p->h_cs = rp.h_cs; p->w_cs = rp.w_cs;
  p->k_bh_stride = rp.k_bh_stride; p->vt_bh_stride = rp.vt_bh_stride;
  p->key_stride = rp.key_stride; p->n_tokens = d.Nc; p->in_tokens = in_tokens;
  p->B = rp.B; p->H = rp.H; p->D = rp.D; p->Hf = rp.Hf; p->Wf = rp.Wf;
  p->dt = rp.dt; p->dh = rp.dh; p->dw = rp.dw; p->n_frames = d.F; p->q_rows = q_rows;
  p->q_scale = rp.q_scale;
  p->n = n;
  for (int j = 0; j < d.dt / 2; ++j) p->theta_t[j] = freq(d, d.dt, j);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Launch with optional event timing on the launch stream.
template <typename F>
sa_status timed(sa_stream* s, int kid, hipStream_t st, F&& launch) {
  std::pair<hipEvent_t, hipEvent_t> ev{nullptr, nullptr};
  if (s->profile) {
    Prof& pr = s->prof[kid];
    if (!pr.free_pairs.empty()) {
      ev = pr.free_pairs.back();
      pr.free_pairs.pop_back();
    } else {
      if (hipEventCreate(&ev.first) != hipSuccess || hipEventCreate(&ev.second) != hipSuccess)
        return SA_ERR_DEVICE;
    }
    if (hipEventRecord(ev.first, st) != hipSuccess) return SA_ERR_DEVICE;
  }
  if (launch() != hipSuccess) return SA_ERR_DEVICE;
  if (s->profile) {
    if (hipEventRecord(ev.second, st) != hipSuccess) return SA_ERR_DEVICE;
    s->prof[kid].pending.push_back(ev);
  }
  return SA_OK;
}

// MFMA attention kernel variant used for this stream (automatic: the ping-pong
// kernel, variant 3; an fp8 cache has no other); 0 for the fp32 kernel.
int attn_variant(const sa_stream* s) {
  if (s->d.dtype == SA_F32) return 0;
  if (s->d.dtype == SA_FP8) return 3;
  return s->variant_opt == 0 ? 3 : s->variant_opt;
}

// Query rows per workgroup of the attention kernel used for this stream.
int attn_block_m(const sa_stream* s) {
  if (s->d.dtype == SA_F32) return sa::kF32BlockM;
  return attn_variant(s) == 1 ? sa::kBf16BlockM : sa::kBf16BlockMWide;
}

int choose_splits(const sa_stream* s, int key_tiles, int q_tiles) {
  const Derived& d = s->d;
  int splits = s->kv_splits_opt;
  if (splits <= 0) {
    // Fill the chip: 256 CUs x resident workgroups. Split the key range only
    // when the (b, h, q-tile) grid leaves more than a quarter of the slots idle.
    const int64_t blocks = static_cast<int64_t>(d.B) * d.H * q_tiles;
    const int64_t slots = attn_block_m(s) == sa::kBf16BlockMWide ? 256 : 512;   // resident workgroups
    splits = 1;
    if (blocks * 4 < slots * 3) {
      splits = static_cast<int>((slots + blocks - 1) / blocks);
      if (splits > d.max_splits) splits = d.max_splits;
    }
  }
  if (splits > key_tiles) splits = key_tiles;
  if (splits < 1) splits = 1;
  return splits;
}

// Stream-K (ping-pong kernel only): persistent workgroups sharing the
// (q-tile, key-tile) iterations evenly, when one workgroup per q-tile would
// leave part of the chip idle in the last round. 0 = grid schedule.
int choose_stream_k(const sa_stream* s, int key_tiles, int q_tiles) {
  const Derived& d = s->d;
  if (attn_variant(s) != 3 || s->kv_splits_opt > 0 || s->schedule_opt == 1) return 0;
  const int64_t n_qt = static_cast<int64_t>(d.B) * d.H * q_tiles;
  const int64_t L = n_qt * key_tiles;
  if (L < 2 * kSkGroups) return 0;               // too little work to share
  // at most 16 workgroups may cut one q-tile (the combine pass's limit)
  if (static_cast<int64_t>(key_tiles) * kSkGroups > 14 * L) return 0;
  // Only on request: measured on a power-limited part, filling the idle CUs of a ragged
  // last wave lowers the clock by about as much as it cuts cycles, and the combine pass
  // then makes the whole slower.
  return s->schedule_opt == 2 ? kSkGroups : 0;
}

// Key-row segments of a buffer attend of n chunks. Moving buffer: buffer chunk j sees
// the sink, the newest min(window_valid, W - j) committed window chunks and buffer
// chunks max(0, j - W)..j. Steps (SA_BUFFER_STEPS): the committed sink chunks, all
// window_valid committed window chunks and buffer chunk j alone. The window chunks
// are ring slots of consecutive commits, contiguous modulo R: at most two ranges.
// Ranges are sorted and adjacent ones merged.
struct BufferPlan {
  int32_t n[SA_MAX_BUFFER_CHUNKS];
  int32_t lo[SA_MAX_BUFFER_CHUNKS][SA_MAX_KEY_SEGMENTS], hi[SA_MAX_BUFFER_CHUNKS][SA_MAX_KEY_SEGMENTS];
};

sa_status plan_buffer(const sa_stream* s, int32_t n_chunks, uint32_t flags, BufferPlan* bp) {
  const Derived& d = s->d;
  if (n_chunks < 1 || n_chunks > d.NB || (flags & ~SA_BUFFER_STEPS) != 0) return SA_ERR_INVALID_ARGUMENT;
  const bool steps = (flags & SA_BUFFER_STEPS) != 0;
  if (!steps && s->sink_fill < d.S) return SA_ERR_BAD_STATE;
  const sa_status st = positions_ok(s, static_cast<int64_t>(s->t_next) + static_cast<int64_t>(n_chunks) * d.F);
  if (st != SA_OK) return st;
  const int64_t C = s->ring_commits;
  const int32_t valid = s->window_valid();
  for (int j = 0; j < n_chunks; ++j) {
    int32_t lo[SA_MAX_KEY_SEGMENTS], hi[SA_MAX_KEY_SEGMENTS];   // in slots
    int n = 0;
    if (s->sink_fill > 0) { lo[n] = 0; hi[n] = s->sink_fill; ++n; }
    // committed chunks still in chunk j's window
    const int32_t m = steps ? valid : std::max(0, std::min(valid, d.W - j));
    if (m > 0) {
      const int32_t start = static_cast<int32_t>((C - m) % d.R);
      if (start + m <= d.R) {
        lo[n] = d.S + start; hi[n] = d.S + start + m; ++n;
      } else {
        lo[n] = d.S + start; hi[n] = d.S + d.R; ++n;
        lo[n] = d.S; hi[n] = d.S + start + m - d.R; ++n;
      }
    }
    lo[n] = d.buf_slot0 + (steps ? j : std::max(0, j - d.W)); hi[n] = d.buf_slot0 + j + 1; ++n;
    for (int a = 1; a < n; ++a)                  // sort by start (n <= 4)
      for (int b = a; b > 0 && lo[b] < lo[b - 1]; --b) {
        std::swap(lo[b], lo[b - 1]);
        std::swap(hi[b], hi[b - 1]);
      }
    int out = 0;
    for (int a = 0; a < n; ++a) {
      if (out > 0 && lo[a] <= bp->hi[j][out - 1] / d.Nc) {
        bp->hi[j][out - 1] = std::max(bp->hi[j][out - 1], hi[a] * d.Nc);
      } else {
        bp->lo[j][out] = lo[a] * d.Nc;
        bp->hi[j][out] = hi[a] * d.Nc;
        ++out;
      }
    }
    bp->n[j] = out;
  }
  return SA_OK;
}

void commit_meta(sa_stream* s) {
  const int32_t slot = s->staging_slot();
  SlotMeta& m = s->slots[slot];
  m.chunk_id = s->n_appends;
  m.t0 = s->t_next;
  if (s->sink_fill < s->d.S) {
    m.kind = SA_SLOT_SINK;
    s->sink_fill += 1;
  } else {
    m.kind = SA_SLOT_WINDOW;
    s->ring_commits += 1;
    if (s->ring_commits > s->d.W) {   // the commit W+1 back leaves the window
      const int64_t evicted = s->ring_commits - 1 - s->d.W;
      s->slots[s->d.S + static_cast<int32_t>(evicted % s->d.R)].kind = SA_SLOT_EMPTY;
    }
  }
  s->t_next += s->d.F;
  s->n_appends += 1;
  s->staged_valid = false;
}

}  // namespace

extern "C" {

const char* sa_status_string(sa_status st) {
  switch (st) {
    case SA_OK: return "SA_OK";
    case SA_ERR_INVALID_ARGUMENT: return "SA_ERR_INVALID_ARGUMENT";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED";
    case SA_ERR_BAD_STATE: return "SA_ERR_BAD_STATE";
    case SA_ERR_WORKSPACE_TOO_SMALL: return "SA_ERR_WORKSPACE_TOO_SMALL";
    case SA_ERR_POSITION_RANGE: return "SA_ERR_POSITION_RANGE";
    case SA_ERR_DEVICE: return "SA_ERR_DEVICE";
  }
  return "SA_ERR_UNKNOWN";
}

sa_status sa_config_check(const sa_config* cfg) {
  Derived d;
  return derive(cfg, &d);
}

size_t sa_workspace_bytes(const sa_config* cfg) {
  Derived d;
  if (derive(cfg, &d) != SA_OK) return 0;
  return d.total;
}

sa_status sa_stream_create(const sa_config* cfg, void* d_workspace, size_t workspace_bytes, void* stream,
                           sa_stream** out) {
  if (out == nullptr) return SA_ERR_INVALID_ARGUMENT;
  Derived d;
  sa_status st = derive(cfg, &d);
  if (st != SA_OK) return st;
  if (d_workspace != nullptr) {
    if (workspace_bytes < d.total) return SA_ERR_WORKSPACE_TOO_SMALL;
    if ((reinterpret_cast<uintptr_t>(d_workspace) & (kAlign - 1)) != 0) return SA_ERR_INVALID_ARGUMENT;
  }
  sa_stream* s = new (std::nothrow) sa_stream();
  if (s == nullptr) return SA_ERR_INVALID_ARGUMENT;
  s->d = d;
  s->ws = static_cast<char*>(d_workspace);
  s->slots.assign(d.n_slots, SlotMeta());
  if (!s->planning()) {
    // spatial tables: [Hf][d_h/2] then [Wf][d_w/2], host fp64 -> fp32
    std::vector<float2> tab(static_cast<size_t>(d.Hf) * (d.dh / 2) + static_cast<size_t>(d.Wf) * (d.dw / 2));
    size_t i = 0;
    for (int y = 0; y < d.Hf; ++y)
      for (int j = 0; j < d.dh / 2; ++j) {
        const double a = y * freq(d, d.dh, j);
        tab[i++] = make_float2(static_cast<float>(std::cos(a)), static_cast<float>(std::sin(a)));
      }
    for (int x = 0; x < d.Wf; ++x)
      for (int j = 0; j < d.dw / 2; ++j) {
        const double a = x * freq(d, d.dw, j);
        tab[i++] = make_float2(static_cast<float>(std::cos(a)), static_cast<float>(std::sin(a)));
      }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    // The attention kernel's ragged last key tile reads a few K rows and V^T
    // entries past the visible keys (masked, weight 0); zeroing the caches once
    // keeps them finite.
    if (hipMemsetAsync(s->ws + d.k_off, 0, d.vt_off - d.k_off + d.vt_bytes, hs) != hipSuccess) {
      delete s;
      return SA_ERR_DEVICE;
    }
    if (!tab.empty() &&
        hipMemcpyAsync(s->ws + d.tab_off, tab.data(), tab.size() * sizeof(float2), hipMemcpyHostToDevice,
                       hs) != hipSuccess) {
      delete s;
      return SA_ERR_DEVICE;
    }
    // synchronous: the host table dies with this call
    if (hipStreamSynchronize(hs) != hipSuccess) {
      delete s;
      return SA_ERR_DEVICE;
    }
  }
  *out = s;
  return SA_OK;
}

sa_status sa_stream_destroy(sa_stream* s) {
  if (s == nullptr) return SA_OK;
  for (auto& pr : s->prof) {
    for (auto& e : pr.pending) {
      (void)hipEventSynchronize(e.second);
      (void)hipEventDestroy(e.first);
      (void)hipEventDestroy(e.second);
    }
    for (auto& e : pr.free_pairs) {
      (void)hipEventDestroy(e.first);
      (void)hipEventDestroy(e.second);
    }
  }
  delete s;
  return SA_OK;
}

sa_status sa_chunk_attend(sa_stream* s, const void* q, const void* k, const void* v, void* out, float* lse,
                          void* stream) {
  if (s == nullptr) return SA_ERR_INVALID_ARGUMENT;
  const Derived& d = s->d;
  if (!s->planning()) {
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return SA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
      return SA_ERR_INVALID_ARGUMENT;
  }
  sa_status st = positions_ok(s, static_cast<int64_t>(s->t_next) + d.F);
  if (st != SA_OK) return st;

  const int32_t slot = s->staging_slot();
  const int32_t n_keys = s->visible_chunks() * d.Nc;
  const int bn = d.dtype != SA_F32 ? sa::kBf16BlockN : sa::kF32BlockN;
  const int key_tiles = (n_keys + bn - 1) / bn;
  const int bm = attn_block_m(s);
  const int q_tiles = (d.Nc + bm - 1) / bm;
  const int sk_groups = choose_stream_k(s, key_tiles, q_tiles);
  const int splits = sk_groups > 0 ? 1 : choose_splits(s, key_tiles, q_tiles);

  if (!s->planning()) {
    hipStream_t hs = static_cast<hipStream_t>(stream);
    RopeWriteParams rp;
    base_write_params(s, &rp);
    rp.q = q; rp.k = k; rp.v = v;
    rp.qrot = s->qscratch();
    rp.row0 = slot * d.Nc;
    fill_temporal(d, s->t_next, d.F, rp.t_cs);
    st = timed(s, SA_K_ROPE_APPLY, hs, [&] { return sa::launch_rope_apply(rp, d.dtype, hs); });
    if (st != SA_OK) return st;

    AttnParams ap;
    std::memset(&ap, 0, sizeof(ap));
    ap.q = s->qscratch();
    ap.kcache = s->kcache();
    ap.vtcache = s->vtcache();
    ap.out = out;
    ap.lse = lse;
    ap.part_o = reinterpret_cast<float*>(s->ws + d.part_off);
    ap.part_lse = ap.part_o + static_cast<size_t>(d.max_splits) * d.B * d.H * d.Nc * d.D;
    ap.k_bh_stride = static_cast<int64_t>(d.key_stride) * d.D;
    ap.vt_bh_stride = static_cast<int64_t>(d.D) * d.key_stride;
    ap.key_stride = d.key_stride;
    ap.n_keys = n_keys;
    ap.Nc = d.Nc; ap.B = d.B; ap.H = d.H; ap.D = d.D;
    ap.variant = attn_variant(s);
    ap.q_rows_per_block = bm;
    ap.q_tiles = q_tiles;
    ap.kv_splits = splits;
    ap.key_tiles = key_tiles;
    ap.scale_log2 = static_cast<float>(static_cast<double>(d.scale) * 1.4426950408889634);
    ap.qk_scale_e8m0 = d.qk_scale_e8m0;
    ap.sk_groups = sk_groups;
    ap.sk_part_o = reinterpret_cast<float*>(s->ws + d.sk_off);
    ap.sk_part_lse = ap.sk_part_o + static_cast<size_t>(2 * kSkGroups) * sa::kBf16BlockMWide * d.D;
    st = timed(s, SA_K_CHUNK_ATTENTION, hs, [&] { return sa::launch_chunk_attention(ap, d.dtype, hs); });
    if (st != SA_OK) return st;
    if (sk_groups > 0) {
      st = timed(s, SA_K_ATTN_COMBINE, hs, [&] { return sa::launch_attn_sk_combine(ap, hs); });
      if (st != SA_OK) return st;
    }
    if (splits > 1) {
      CombineParams cp;
      cp.part_o = ap.part_o;
      cp.part_lse = ap.part_lse;
      cp.out = out;
      cp.lse = lse;
      cp.Nc = d.Nc; cp.B = d.B; cp.H = d.H; cp.D = d.D; cp.kv_splits = splits;
      st = timed(s, SA_K_ATTN_COMBINE, hs, [&] { return sa::launch_attn_combine(cp, d.dtype, hs); });
      if (st != SA_OK) return st;
    }
  }
  s->staged_valid = true;
  s->staged_t = s->t_next;
  s->staged_slot = slot;
  s->last_q_tiles = q_tiles;
  s->last_sk_groups = sk_groups;
  s->last_kv_splits = splits;
  s->last_key_tiles = key_tiles;
  return SA_OK;
}

sa_status sa_kv_append(sa_stream* s, const void* k, const void* v, void* stream) {
  if (s == nullptr) return SA_ERR_INVALID_ARGUMENT;
  const Derived& d = s->d;
  const bool commit_staged = (k == nullptr && v == nullptr);
  if (!commit_staged && !s->planning()) {
    if (k == nullptr || v == nullptr || !aligned16(k) || !aligned16(v)) return SA_ERR_INVALID_ARGUMENT;
  }
  sa_status st = positions_ok(s, static_cast<int64_t>(s->t_next) + d.F);
  if (st != SA_OK) return st;
  const int32_t slot = s->staging_slot();
  if (commit_staged) {
    if (!s->staged_valid || s->staged_t != s->t_next || s->staged_slot != slot) return SA_ERR_BAD_STATE;
  } else if (!s->planning()) {
    hipStream_t hs = static_cast<hipStream_t>(stream);
    RopeWriteParams rp;
    base_write_params(s, &rp);
    rp.k = k; rp.v = v;
    rp.row0 = slot * d.Nc;
    fill_temporal(d, s->t_next, d.F, rp.t_cs);
    st = timed(s, SA_K_KV_APPEND, hs, [&] { return sa::launch_kv_append(rp, d.dtype, hs); });
    if (st != SA_OK) return st;
  }
  commit_meta(s);
  return SA_OK;
}

sa_status sa_rope_refresh(sa_stream* s, int32_t new_base_t, uint32_t flags, void* stream, int32_t* delta_out) {
  if (s == nullptr) return SA_ERR_INVALID_ARGUMENT;
  if ((flags & ~SA_REFRESH_SHIFT_SINK) != 0) return SA_ERR_INVALID_ARGUMENT;
  if (new_base_t < -1) return SA_ERR_INVALID_ARGUMENT;
  const Derived& d = s->d;
  const int64_t base = new_base_t == -1 ? static_cast<int64_t>(d.S) * d.F : new_base_t;
  const int32_t wv = s->window_valid();
  std::vector<int32_t> win;                     // physical slots of visible window chunks, oldest first
  for (int64_t c = s->ring_commits - wv; c < s->ring_commits; ++c)
    win.push_back(d.S + static_cast<int32_t>(c % d.R));
  const int64_t ref = win.empty() ? s->t_next : s->slots[win[0]].t0;
  const int64_t delta = ref - base;
  const int64_t new_t_next = s->t_next - delta;
  if (new_t_next < 0 || new_t_next > kMaxPosition) return SA_ERR_POSITION_RANGE;
  std::vector<int32_t> targets = win;
  if (flags & SA_REFRESH_SHIFT_SINK) {
    for (int32_t j = 0; j < s->sink_fill; ++j) {
      const int64_t t = static_cast<int64_t>(s->slots[j].t0) - delta;
      if (t < -kMaxPosition || t > kMaxPosition) return SA_ERR_POSITION_RANGE;
      targets.push_back(j);
    }
  }
  if (!s->planning() && delta != 0 && !targets.empty()) {
    hipStream_t hs = static_cast<hipStream_t>(stream);
    RefreshParams rp;
    std::memset(&rp, 0, sizeof(rp));
    rp.kcache = s->kcache();
    rp.k_bh_stride = static_cast<int64_t>(d.key_stride) * d.D;
    rp.BH = d.B * d.H; rp.D = d.D; rp.Nc = d.Nc; rp.dt = d.dt;
    for (int j = 0; j < d.dt / 2; ++j) {
      const double a = -static_cast<double>(delta) * freq(d, d.dt, j);
      rp.cs[j] = make_float2(static_cast<float>(std::cos(a)), static_cast<float>(std::sin(a)));
    }
    for (size_t i0 = 0; i0 < targets.size(); i0 += sa::kMaxRefreshSlots) {
      rp.n_slot = 0;
      for (size_t i = i0; i < targets.size() && rp.n_slot < sa::kMaxRefreshSlots; ++i)
        rp.slot_row0[rp.n_slot++] = targets[i] * d.Nc;
      sa_status st = timed(s, SA_K_ROPE_REFRESH, hs, [&] { return sa::launch_rope_refresh(rp, d.dtype, hs); });
      if (st != SA_OK) return st;
    }
  }
  for (int32_t j : targets) s->slots[j].t0 = static_cast<int32_t>(s->slots[j].t0 - delta);
  s->t_next = static_cast<int32_t>(new_t_next);
  if (delta != 0) s->staged_valid = false;
  s->last_delta = static_cast<int32_t>(delta);
  if (delta_out != nullptr) *delta_out = static_cast<int32_t>(delta);
  return SA_OK;
}

sa_status sa_sink_update(sa_stream* s, const void* k, const void* v, void* stream) {
  if (s == nullptr) return SA_ERR_INVALID_ARGUMENT;
  const Derived& d = s->d;
  if (d.S == 0) return SA_ERR_BAD_STATE;
  if (!s->planning() && (k == nullptr || v == nullptr || !aligned16(k) || !aligned16(v)))
    return SA_ERR_INVALID_ARGUMENT;
  sa_status st = positions_ok(s, static_cast<int64_t>(d.S) * d.F);
  if (st != SA_OK) return st;
  if (!s->planning()) {
    hipStream_t hs = static_cast<hipStream_t>(stream);
    RopeWriteParams rp;
    base_write_params(s, &rp);
    rp.k = k; rp.v = v;
    rp.in_tokens = d.S * d.Nc;
    for (int32_t j = 0; j < d.S; ++j) {
      rp.row0 = j * d.Nc;
      rp.in_tok0 = j * d.Nc;
      fill_temporal(d, static_cast<int64_t>(j) * d.F, d.F, rp.t_cs);
      st = timed(s, SA_K_SINK_UPDATE, hs, [&] { return sa::launch_sink_update(rp, d.dtype, hs); });
      if (st != SA_OK) return st;
    }
  }
  for (int32_t j = 0; j < d.S; ++j) {
    s->slots[j].kind = SA_SLOT_SINK;
    s->slots[j].chunk_id = -1;
    s->slots[j].t0 = j * d.F;
  }
  s->sink_fill = d.S;
  s->staged_valid = false;
  return SA_OK;
}

sa_status sa_stream_query(const sa_stream* s, sa_state* out) {
  if (s == nullptr || out == nullptr) return SA_ERR_INVALID_ARGUMENT;
  sa_state st;
  std::memset(&st, 0, sizeof(st));
  st.n_appends = s->n_appends;
  st.ring_commits = s->ring_commits;
  st.t_next = s->t_next;
  st.sink_fill = s->sink_fill;
  st.window_valid = s->window_valid();
  st.staging_slot = s->staging_slot();
  st.n_slots = s->d.n_slots;
  st.visible_chunks = s->visible_chunks();
  st.visible_keys = st.visible_chunks * s->d.Nc;
  st.staged_valid = s->staged_valid && s->staged_t == s->t_next && s->staged_slot == st.staging_slot;
  st.last_q_tiles = s->last_q_tiles;
  st.last_kv_splits = s->last_kv_splits;
  st.last_key_tiles = s->last_key_tiles;
  st.last_delta = s->last_delta;
  st.last_sk_groups = s->last_sk_groups;
  *out = st;
  return SA_OK;
}

sa_status sa_stream_slot(const sa_stream* s, int32_t slot, sa_slot_info* out) {
  if (s == nullptr || out == nullptr || slot < 0 || slot >= s->d.n_slots) return SA_ERR_INVALID_ARGUMENT;
  const SlotMeta& m = s->slots[slot];
  sa_slot_info info;
  info.kind = m.kind;
  info.chunk_id = m.chunk_id;
  info.t0 = m.t0;
  if (slot == s->staging_slot() && m.kind != SA_SLOT_SINK) {
    info.kind = SA_SLOT_STAGING;
    info.chunk_id = s->n_appends;
    info.t0 = s->t_next;
  } else if (m.kind == SA_SLOT_EMPTY) {
    info.chunk_id = -1;
    info.t0 = 0;
  }
  *out = info;
  return SA_OK;
}

sa_status sa_stream_layout(const sa_stream* s, sa_layout* out) {
  if (s == nullptr || out == nullptr) return SA_ERR_INVALID_ARGUMENT;
  const Derived& d = s->d;
  sa_layout L;
  std::memset(&L, 0, sizeof(L));
  L.k_offset = d.k_off;
  L.k_bh_stride = static_cast<uint64_t>(d.key_stride) * d.D * d.elem;
  L.vt_offset = d.vt_off;
  L.vt_bh_stride = static_cast<uint64_t>(d.D) * d.key_stride * d.elem;
  L.q_offset = d.q_off;
  L.q_bh_stride = static_cast<uint64_t>(d.Nc) * d.D * d.elem;
  L.partial_offset = d.part_off;
  L.partial_bytes = d.part_bytes;
  L.table_offset = d.tab_off;
  L.table_bytes = d.tab_bytes;
  L.key_stride = d.key_stride;
  L.elem_bytes = d.elem;
  L.max_kv_splits = d.max_splits;
  *out = L;
  return SA_OK;
}

sa_status sa_stream_set_option(sa_stream* s, int32_t option, int64_t value) {
  if (s == nullptr) return SA_ERR_INVALID_ARGUMENT;
  switch (option) {
    case SA_OPT_KV_SPLITS:
      if (value < 0 || value > s->d.max_splits) return SA_ERR_INVALID_ARGUMENT;
      s->kv_splits_opt = static_cast<int32_t>(value);
      return SA_OK;
    case SA_OPT_ATTN_VARIANT:
      if (value < 0 || value > 4 || (s->d.dtype == SA_FP8 && value != 0 && value != 3))
        return SA_ERR_INVALID_ARGUMENT;
      s->variant_opt = static_cast<int32_t>(value);
      return SA_OK;
    case SA_OPT_SCHEDULE:
      if (value < 0 || value > 2) return SA_ERR_INVALID_ARGUMENT;
      s->schedule_opt = static_cast<int32_t>(value);
      return SA_OK;
    case SA_OPT_PROFILE:
      if (value != 0 && value != 1) return SA_ERR_INVALID_ARGUMENT;
      if (value == 1 && s->planning()) return SA_ERR_BAD_STATE;
      s->profile = value == 1;
      return SA_OK;
    default:
      return SA_ERR_INVALID_ARGUMENT;
  }
}

sa_status sa_profile_read(sa_stream* s, int32_t kernel_id, double* total_ms, int64_t* launches, int32_t reset) {
  if (s == nullptr || kernel_id < 0 || kernel_id >= SA_K_COUNT) return SA_ERR_INVALID_ARGUMENT;
  Prof& pr = s->prof[kernel_id];
  for (auto& e : pr.pending) {
    if (hipEventSynchronize(e.second) != hipSuccess) return SA_ERR_DEVICE;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e.first, e.second) != hipSuccess) return SA_ERR_DEVICE;
    pr.total_ms += ms;
    pr.launches += 1;
    pr.free_pairs.push_back(e);
  }
  pr.pending.clear();
  if (total_ms != nullptr) *total_ms = pr.total_ms;
  if (launches != nullptr) *launches = pr.launches;
  if (reset) {
    pr.total_ms = 0.0;
    pr.launches = 0;
  }
  return SA_OK;
}

sa_status sa_buffer_plan(const sa_stream* s, int32_t n_chunks, uint32_t flags, int32_t* n_seg,
                         int32_t* seg_lo, int32_t* seg_hi) {
  if (s == nullptr || n_seg == nullptr || seg_lo == nullptr || seg_hi == nullptr) return SA_ERR_INVALID_ARGUMENT;
  BufferPlan bp;
  const sa_status st = plan_buffer(s, n_chunks, flags, &bp);
  if (st != SA_OK) return st;
  for (int j = 0; j < n_chunks; ++j) {
    n_seg[j] = bp.n[j];
    for (int k = 0; k < SA_MAX_KEY_SEGMENTS; ++k) {
      seg_lo[j * SA_MAX_KEY_SEGMENTS + k] = k < bp.n[j] ? bp.lo[j][k] : 0;
      seg_hi[j * SA_MAX_KEY_SEGMENTS + k] = k < bp.n[j] ? bp.hi[j][k] : 0;
    }
  }
  return SA_OK;
}

sa_status sa_buffer_attend(sa_stream* s, const void* q, const void* k, const void* v, int32_t n_chunks,
                           uint32_t flags, void* out, float* lse, void* stream) {
  if (s == nullptr) return SA_ERR_INVALID_ARGUMENT;
  const Derived& d = s->d;
  if (!s->planning()) {
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return SA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
      return SA_ERR_INVALID_ARGUMENT;
  }
  BufferPlan bp;
  sa_status st = plan_buffer(s, n_chunks, flags, &bp);
  if (st != SA_OK) return st;
  const int bm = d.dtype != SA_F32 ? sa::kBf16BlockMWide : sa::kF32BlockM;
  const int bn = d.dtype != SA_F32 ? sa::kBf16BlockN : sa::kF32BlockN;
  const int group_qtiles = (d.Nc + bm - 1) / bm;
  int max_tiles = 0;
  for (int j = 0; j < n_chunks; ++j) {
    int t = 0;
    for (int i = 0; i < bp.n[j]; ++i) t += (bp.hi[j][i] + bn - 1) / bn - bp.lo[j][i] / bn;
    max_tiles = t > max_tiles ? t : max_tiles;
  }

  if (!s->planning()) {
    hipStream_t hs = static_cast<hipStream_t>(stream);
    // Rotate and store every buffer chunk in one launch: entry j of the batched rope_apply is
    // chunk j, with its inputs, Q scratch rows and cache slot offset to chunk j and its
    // frames at temporal positions t_next + j F on.
    {
      sa::RopeBatchParams rb;
      base_batch_params(s, n_chunks, n_chunks * d.Nc, n_chunks * d.Nc, &rb);
      const size_t in_elem = d.dtype == SA_F32 ? 4 : 2;
      const size_t chunk_in = static_cast<size_t>(d.Nc) * d.H * d.D * in_elem;    // bytes of one chunk's tokens
      const size_t chunk_q = static_cast<size_t>(d.Nc) * d.D * d.elem;             // bytes of one chunk's Q rows
      for (int j = 0; j < n_chunks; ++j) {
        rb.q[j] = static_cast<const char*>(q) + j * chunk_in;
        rb.k[j] = static_cast<const char*>(k) + j * chunk_in;
        rb.v[j] = static_cast<const char*>(v) + j * chunk_in;
        rb.qrot[j] = static_cast<char*>(s->qscratch()) + j * chunk_q;
        rb.kcache[j] = s->kcache();
        rb.vtcache[j] = s->vtcache();
        rb.row0[j] = (d.buf_slot0 + j) * d.Nc;
        rb.t0[j] = s->t_next + j * d.F;
      }
      st = timed(s, SA_K_ROPE_APPLY, hs, [&] { return sa::launch_rope_apply_batch(rb, d.dtype, hs); });
      if (st != SA_OK) return st;
    }
    AttnParams ap;
    std::memset(&ap, 0, sizeof(ap));
    ap.q = s->qscratch();
    ap.kcache = s->kcache();
    ap.vtcache = s->vtcache();
    ap.out = out;
    ap.lse = lse;
    ap.k_bh_stride = static_cast<int64_t>(d.key_stride) * d.D;
    ap.vt_bh_stride = static_cast<int64_t>(d.D) * d.key_stride;
    ap.key_stride = d.key_stride;
    ap.n_keys = (d.buf_slot0 + d.NB) * d.Nc;
    ap.Nc = n_chunks * d.Nc;                     // query rows per (b, h)
    ap.B = d.B; ap.H = d.H; ap.D = d.D;
    ap.variant = d.dtype != SA_F32 ? 3 : 0;
    ap.q_rows_per_block = bm;
    ap.q_tiles = n_chunks * group_qtiles;
    ap.kv_splits = 1;
    ap.key_tiles = max_tiles;
    ap.scale_log2 = static_cast<float>(static_cast<double>(d.scale) * 1.4426950408889634);
    ap.qk_scale_e8m0 = d.qk_scale_e8m0;
    ap.n_groups = n_chunks;
    ap.group_rows = d.Nc;
    ap.group_qtiles = group_qtiles;
    for (int j = 0; j < n_chunks; ++j) {
      ap.n_seg[j] = bp.n[j];
      for (int i = 0; i < bp.n[j]; ++i) {
        ap.seg_lo[j][i] = bp.lo[j][i];
        ap.seg_hi[j][i] = bp.hi[j][i];
      }
    }
    st = timed(s, SA_K_CHUNK_ATTENTION, hs, [&] { return sa::launch_chunk_attention(ap, d.dtype, hs); });
    if (st != SA_OK) return st;
  }
  s->staged_valid = false;
  s->last_q_tiles = n_chunks * group_qtiles;
  s->last_kv_splits = 1;
  s->last_key_tiles = max_tiles;
  s->last_sk_groups = 0;
  return SA_OK;
}

sa_status sa_batch_attend(int32_t n, sa_stream* const* streams, const void* const* q, const void* const* k,
                          const void* const* v, void* const* out, float* const* lse, void* stream) {
  if (n < 1 || n > SA_MAX_BATCH_STREAMS || streams == nullptr) return SA_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < n; ++i)
    if (streams[i] == nullptr) return SA_ERR_INVALID_ARGUMENT;
  const sa_stream* s0 = streams[0];
  const Derived& d = s0->d;
  const bool planning = s0->planning();
  for (int i = 0; i < n; ++i) {
    const sa_stream* si = streams[i];
    for (int j = 0; j < i; ++j)
      if (streams[j] == si) return SA_ERR_INVALID_ARGUMENT;     // one entry per handle
    const Derived& e = si->d;
    if (si->planning() != planning || e.B != d.B || e.H != d.H || e.D != d.D || e.Hf != d.Hf || e.Wf != d.Wf ||
        e.F != d.F || e.S != d.S || e.W != d.W || e.NB != d.NB || e.dtype != d.dtype || e.dt != d.dt ||
        e.dh != d.dh || e.dw != d.dw || e.theta != d.theta || e.scale != d.scale || e.max_t != d.max_t)
      return SA_ERR_INVALID_ARGUMENT;
    if (!planning) {
      if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return SA_ERR_INVALID_ARGUMENT;
      if (q[i] == nullptr || k[i] == nullptr || v[i] == nullptr || out[i] == nullptr) return SA_ERR_INVALID_ARGUMENT;
      if (!aligned16(q[i]) || !aligned16(k[i]) || !aligned16(v[i]) || !aligned16(out[i]) ||
          (lse != nullptr && (reinterpret_cast<uintptr_t>(lse[i]) & 3u) != 0))
        return SA_ERR_INVALID_ARGUMENT;
    }
    const sa_status st = positions_ok(si, static_cast<int64_t>(si->t_next) + e.F);
    if (st != SA_OK) return st;
  }
  const int bm = d.dtype != SA_F32 ? sa::kBf16BlockMWide : sa::kF32BlockM;
  const int bn = d.dtype != SA_F32 ? sa::kBf16BlockN : sa::kF32BlockN;
  const int group_qtiles = (d.Nc + bm - 1) / bm;
  if (!planning) {
    hipStream_t hs = static_cast<hipStream_t>(stream);
    AttnParams ap;
    std::memset(&ap, 0, sizeof(ap));
    // one launch stages every entry's chunk in its own workspace
    sa::RopeBatchParams bp;
    base_batch_params(s0, n, d.Nc, d.Nc, &bp);
    for (int i = 0; i < n; ++i) {
      sa_stream* si = streams[i];
      bp.q[i] = q[i]; bp.k[i] = k[i]; bp.v[i] = v[i];
      bp.qrot[i] = si->qscratch();
      bp.kcache[i] = si->kcache();
      bp.vtcache[i] = si->vtcache();
      bp.row0[i] = si->staging_slot() * d.Nc;
      bp.t0[i] = si->t_next;
    }
    {
      const sa_status st = timed(streams[0], SA_K_ROPE_APPLY, hs, [&] { return sa::launch_rope_apply_batch(bp, d.dtype, hs); });
      if (st != SA_OK) return st;
    }
    for (int i = 0; i < n; ++i) {
      sa_stream* si = streams[i];
      ap.g_q[i] = si->qscratch();
      ap.g_kc[i] = si->kcache();
      ap.g_vt[i] = si->vtcache();
      ap.g_out[i] = out[i];
      ap.g_lse[i] = lse != nullptr ? lse[i] : nullptr;
      ap.n_seg[i] = 1;
      ap.seg_lo[i][0] = 0;
      ap.seg_hi[i][0] = si->visible_chunks() * d.Nc;   // the physical prefix an attend reads
    }
    ap.k_bh_stride = static_cast<int64_t>(d.key_stride) * d.D;
    ap.vt_bh_stride = static_cast<int64_t>(d.D) * d.key_stride;
    ap.key_stride = d.key_stride;
    ap.n_keys = (d.buf_slot0 + d.NB) * d.Nc;
    ap.Nc = d.Nc;
    ap.B = d.B; ap.H = d.H; ap.D = d.D;
    ap.variant = d.dtype != SA_F32 ? 3 : 0;
    ap.q_rows_per_block = bm;
    ap.q_tiles = n * group_qtiles;
    ap.kv_splits = 1;
    ap.scale_log2 = static_cast<float>(static_cast<double>(d.scale) * 1.4426950408889634);
    ap.qk_scale_e8m0 = d.qk_scale_e8m0;
    ap.n_groups = n;
    ap.group_rows = d.Nc;
    ap.group_qtiles = group_qtiles;
    ap.ragged = 1;
    int max_tiles = 0;
    for (int i = 0; i < n; ++i) max_tiles = std::max(max_tiles, (ap.seg_hi[i][0] + bn - 1) / bn);
    ap.key_tiles = max_tiles;
    const sa_status st = timed(streams[0], SA_K_CHUNK_ATTENTION, hs,
                               [&] { return sa::launch_chunk_attention(ap, d.dtype, hs); });
    if (st != SA_OK) return st;
  }
  for (int i = 0; i < n; ++i) {                  // as after sa_chunk_attend
    sa_stream* si = streams[i];
    si->staged_valid = true;
    si->staged_t = si->t_next;
    si->staged_slot = si->staging_slot();
    si->last_q_tiles = group_qtiles;
    si->last_kv_splits = 1;
    si->last_key_tiles = (si->visible_chunks() * d.Nc + bn - 1) / bn;
    si->last_sk_groups = 0;
  }
  return SA_OK;
}

sa_status sa_probe_mfma_bf16(float* d_out, int32_t blocks, int32_t iters, void* stream) {
  if (d_out == nullptr || blocks < 1 || blocks > (1 << 20) || iters < 1) return SA_ERR_INVALID_ARGUMENT;
  return sa::launch_mfma_probe(d_out, blocks, iters, static_cast<hipStream_t>(stream)) == hipSuccess
             ? SA_OK : SA_ERR_DEVICE;
}

sa_status sa_probe_mfma_bf16_data(float* d_out, const void* d_operands, int32_t blocks, int32_t iters, void* stream) {
  if (d_out == nullptr || d_operands == nullptr || (reinterpret_cast<uintptr_t>(d_operands) & 15u) != 0 ||
      blocks < 1 || blocks > (1 << 20) || iters < 1)
    return SA_ERR_INVALID_ARGUMENT;
  return sa::launch_mfma_probe_data(d_out, d_operands, blocks, iters, static_cast<hipStream_t>(stream)) == hipSuccess
             ? SA_OK : SA_ERR_DEVICE;
}

}  // extern "C"

// ---- gated delta rule (GDN) forward ----------------------------------------------------------

namespace {

struct GdnLayout {
  size_t g, W, Up, Kt, U, Sst, total;
  int32_t nb;
};

sa_status gdn_layout(int32_t B, int32_t N, int32_t H, int32_t D, GdnLayout* L) {
  if (B < 1 || H < 1 || N < 0) return SA_ERR_INVALID_ARGUMENT;
  if (D != 64 && D != 128) return SA_ERR_UNSUPPORTED;
  if (B > 32767 || H > 32767 || N > (1 << 24)) return SA_ERR_UNSUPPORTED;
  const int64_t nb = (static_cast<int64_t>(N) + sa::kGdnBlock - 1) / sa::kGdnBlock;
  const size_t bhb = static_cast<size_t>(B) * H * static_cast<size_t>(nb);
  size_t off = 0;
  L->nb = static_cast<int32_t>(nb);
  L->g = off; off = align_up(off + bhb * sa::kGdnBlock * 4, kAlign);
  L->W = off; off = align_up(off + bhb * sa::kGdnBlock * D * 6, kAlign);    // three bf16 parts
  L->Up = off; off = align_up(off + bhb * sa::kGdnBlock * D * 4, kAlign);
  L->Kt = off; off = align_up(off + bhb * sa::kGdnBlock * D * 2, kAlign);   // bf16
  L->U = off; off = align_up(off + bhb * sa::kGdnBlock * D * 4, kAlign);
  L->Sst = off; off = align_up(off + bhb * static_cast<size_t>(D) * D * 4, kAlign);
  L->total = off > kAlign ? off : kAlign;        // never 0: 0 means unsupported sizes
  return SA_OK;
}

}  // namespace

size_t sa_gdn_workspace_bytes(int32_t batch, int32_t tokens, int32_t heads, int32_t head_dim) {
  GdnLayout L;
  return gdn_layout(batch, tokens, heads, head_dim, &L) == SA_OK ? L.total : 0;
}

namespace {

// The forward over a workspace of ws_bytes at ws (the caller's, or the fixed scratch).
sa_status gdn_forward_impl(const GdnLayout& L, int32_t batch, int32_t tokens, int32_t heads, int32_t head_dim,
                           const void* q, const void* k, const void* v, const float* alpha, const float* beta,
                           const float* state_in, float* state_out, void* out, void* workspace, hipStream_t hs) {
  char* ws = static_cast<char*>(workspace);
  sa::GdnParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q; p.k = k; p.v = v;
  p.alpha = alpha; p.beta = beta;
  p.state_in = state_in; p.state_out = state_out;
  p.out = out;
  p.g = reinterpret_cast<float*>(ws + L.g);
  p.W = ws + L.W;
  p.Up = reinterpret_cast<float*>(ws + L.Up);
  p.Kt = ws + L.Kt;
  p.U = reinterpret_cast<float*>(ws + L.U);
  p.Sst = reinterpret_cast<float*>(ws + L.Sst);
  p.B = batch; p.N = tokens; p.H = heads; p.D = head_dim; p.nb = L.nb;
  if (tokens == 0) {                             // no tokens: the state passes through
    const size_t n = static_cast<size_t>(batch) * heads * head_dim * head_dim;
    return sa::launch_gdn_state_pass(state_in, state_out, n, hs) == hipSuccess ? SA_OK : SA_ERR_DEVICE;
  }
  return sa::launch_gdn_forward(p, hs) == hipSuccess ? SA_OK : SA_ERR_DEVICE;
}

// Argument checks shared by both forwards (the workspace is checked by the caller).
sa_status gdn_check_args(int32_t tokens, const void* q, const void* k, const void* v, const float* alpha,
                         const float* beta, const float* state_in, const float* state_out, const void* out) {
  auto a4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
  // the states move as float4s
  if (state_out == nullptr || !aligned16(state_out) || (state_in != nullptr && !aligned16(state_in)))
    return SA_ERR_INVALID_ARGUMENT;
  if (tokens > 0) {                              // with no tokens only the state is touched
    if (q == nullptr || k == nullptr || v == nullptr || alpha == nullptr || beta == nullptr || out == nullptr)
      return SA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !a4(alpha) || !a4(beta))
      return SA_ERR_INVALID_ARGUMENT;
  }
  return SA_OK;
}

}  // namespace

sa_status sa_gdn_forward(int32_t batch, int32_t tokens, int32_t heads, int32_t head_dim, const void* q,
                         const void* k, const void* v, const float* alpha, const float* beta,
                         const float* state_in, float* state_out, void* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  GdnLayout L;
  sa_status st = gdn_layout(batch, tokens, heads, head_dim, &L);
  if (st != SA_OK) return st;
  st = gdn_check_args(tokens, q, k, v, alpha, beta, state_in, state_out, out);
  if (st != SA_OK) return st;
  if (tokens > 0) {
    if (workspace == nullptr || !aligned16(workspace)) return SA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < L.total) return SA_ERR_WORKSPACE_TOO_SMALL;
  }
  return gdn_forward_impl(L, batch, tokens, heads, head_dim, q, k, v, alpha, beta, state_in, state_out, out,
                          workspace, static_cast<hipStream_t>(stream));
}

sa_status sa_gdn_forward_noalloc(int32_t batch, int32_t tokens, int32_t heads, int32_t head_dim, const void* q,
                                 const void* k, const void* v, const float* alpha, const float* beta,
                                 const float* state_in, float* state_out, void* out, void* stream) {
  static_assert(sa::kGdnScratchBytes == SA_GDN_SCRATCH_BYTES, "scratch size in the header");
  GdnLayout L;
  sa_status st = gdn_layout(batch, tokens, heads, head_dim, &L);
  if (st != SA_OK) return st;
  if (tokens > 0 && L.total > sa::kGdnScratchBytes) return SA_ERR_WORKSPACE_TOO_SMALL;
  st = gdn_check_args(tokens, q, k, v, alpha, beta, state_in, state_out, out);
  if (st != SA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  void* scratch = nullptr;
  if (tokens > 0 && sa::gdn_scratch_address(hs, &scratch) != hipSuccess) return SA_ERR_DEVICE;
  return gdn_forward_impl(L, batch, tokens, heads, head_dim, q, k, v, alpha, beta, state_in, state_out, out,
                          scratch, hs);
}
