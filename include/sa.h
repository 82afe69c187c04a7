/*
 * sa.h -- C ABI of the streaming chunk attention library (libsa.so, gfx950).
 *
 * What it computes. Video is generated chunk by chunk; each chunk holds F latent
 * frames of Hf x Wf tokens (the B x T' x H x W input form of StreamDiffusionV2,
 * "Sommario tecnico" 2.A.1). Every query token of the current chunk gets a 3D
 * (t, h, w) rotary position embedding and attends with full softmax attention
 * to (1) a persistent sink chunk, (2) a sliding window of the most recent
 * committed chunks and (3) the current chunk itself (SANA-Streaming,
 * "Transformer a diffusione ibrido": softmax blocks with a sliding local window
 * and a persistent sink chunk). Keys are kept rotated in a bounded cache whose
 * temporal RoPE offsets can be re-based at chunk boundaries so that long
 * streams stay inside the trained position range, and the sink can be replaced
 * (StreamDiffusionV2, "Sommario tecnico" 2.A.2: sink tokens updated during the
 * stream, RoPE offsets reset periodically at block boundaries).
 *
 * Conventions fixed by this library where the pages are silent:
 *  - RoPE: head_dim D is split into contiguous segments [t | h | w] of even
 *    lengths (default d_h = d_w = 2*floor(D/6), d_t = D - 2*d_h); pair j of a
 *    segment of length d is channels (o+2j, o+2j+1) with frequency
 *    theta^(-2j/d); the rotation of a pair is RoFormer's.
 *  - Token n of a chunk sits at (t_next + n / (Hf*Wf), (n / Wf) % Hf, n % Wf).
 *  - The first S committed chunks fill the sink; later commits enter the
 *    window; W counts previous chunks (the current chunk is extra).
 *  - Softmax scale defaults to 1/sqrt(D).
 *
 * Layouts. q, k, v and out are [B, Nc, H, D] contiguous (token-major, what a
 * fused QKV projection writes), Nc = F*Hf*Wf, element type = config dtype
 * (bf16 for SA_FP8).
 * lse is [B, H, Nc] float32 (natural log). The workspace is opaque device
 * memory sized by sa_workspace_bytes(); sa_stream_layout() describes it for
 * inspection.
 *
 * Ownership. The caller owns every device buffer, including the workspace;
 * the library never allocates device memory. It owns only the host handle
 * (allocated by sa_stream_create, freed by sa_stream_destroy).
 *
 * Streams. `stream` arguments are hipStream_t values passed as void* (NULL =
 * the default stream). All device work is enqueued asynchronously on that
 * stream; calls on one handle must be ordered on one stream (the cache slot a
 * commit overwrites may still be read by an earlier attend otherwise).
 * Handles are not thread-safe; distinct handles are independent.
 *
 * Errors. Every entry point returns sa_status and never throws. Argument and
 * state errors are detected on the host before any launch and leave the state
 * unchanged; out-parameters are written only on SA_OK. A failed launch returns
 * SA_ERR_DEVICE; asynchronous device faults surface at the caller's next
 * synchronisation.
 *
 * Planning handles. A handle created with a NULL workspace runs all validation
 * and bookkeeping but never touches the device (data pointers are ignored and
 * may be NULL). It is what a scheduler (or a CPU-only test) uses to predict
 * slot assignment, positions and launch plans.
 */
#ifndef SA_H_
#define SA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sa_status {
  SA_OK = 0,
  SA_ERR_INVALID_ARGUMENT = 1,   /* bad config, NULL pointer, bad flag or base      */
  SA_ERR_UNSUPPORTED = 2,        /* shape/dtype without a kernel (see sa_config)     */
  SA_ERR_BAD_STATE = 3,          /* call not valid in the current stream state       */
  SA_ERR_WORKSPACE_TOO_SMALL = 4,
  SA_ERR_POSITION_RANGE = 5,     /* a chunk would use t >= max_t (refresh cures it)  */
  SA_ERR_DEVICE = 6              /* a HIP call failed                                */
} sa_status;

/*
 * SA_FP8: q, k, v and out are bf16; the rotated Q scratch, the K cache and the
 * V^T cache hold E4M3 values (OCP 8-bit float: 3 mantissa bits, largest finite
 * 448), each rounded to nearest even after clamping to +-448; the attention
 * products run on the fp8 MFMA with fp32 accumulation, and the softmax weights
 * are rounded to E4M3 before the PV product (weights of a row are formed
 * relative to its running maximum minus 4 in log2 units, so they stay below
 * 2^8). Outputs are normalised by the sum of the rounded weights, and lse is
 * the log of that sum (off the exact one by the weights' rounding: about
 * 1e-3 for broad attention). A lower-precision variant of the same method
 * (SANA-Streaming's mixed-precision policy quantises attention query/key
 * projections); its error bound is derived from the E4M3 rounding.
 */
typedef enum sa_dtype { SA_F32 = 0, SA_BF16 = 1, SA_FP8 = 2 } sa_dtype;

/* sa_rope_refresh flags */
#define SA_REFRESH_SHIFT_SINK 1u

/*
 * Stream configuration (72 bytes, no padding holes).
 *  batch            B >= 1 streams advancing in lockstep (same positions, own caches)
 *  heads            H >= 1
 *  head_dim         D: 64 or 128 (SA_F32, SA_BF16); 128 (SA_FP8)
 *  frame_h, frame_w latent grid of one frame, >= 1
 *  frames_per_chunk F >= 1 (one temporal RoPE unit per latent frame)
 *  sink_chunks      S >= 0 persistent sink chunks
 *  window_chunks    W >= 0 previous chunks kept in the sliding window
 *  rope_dim_t/h/w   even, summing to D; all 0 selects the default split
 *  max_t            0: unbounded; else every position used must be < max_t
 *  rope_theta       RoPE base, 0 selects 10000
 *  softmax_scale    0 selects 1/sqrt(D)
 *  dtype            SA_F32, SA_BF16 (element type of q, k, v, out and the cache)
 *                   or SA_FP8 (bf16 q, k, v, out; E4M3 cache)
 *  max_buffer_chunks NB in 0..SA_MAX_BUFFER_CHUNKS: chunks one sa_buffer_attend
 *                   may hold (NB extra cache slots per (b, h), NB*Nc Q scratch rows)
 *  reserved         must be 0
 * Limits: F * d_t / 2 <= SA_MAX_TEMPORAL_PAIRS; Nc = F*Hf*Wf <= 2^20;
 *         (S + W + 1 + NB) * Nc <= 2^24 keys, and the cache of one (b, h) (keys
 *         rounded up to 64, times D times the element size) below 2^31 bytes.
 *         A config over a limit is SA_ERR_UNSUPPORTED.
 */
typedef struct sa_config {
  int32_t batch, heads, head_dim, frame_h, frame_w, frames_per_chunk;
  int32_t sink_chunks, window_chunks;
  int32_t rope_dim_t, rope_dim_h, rope_dim_w;
  int32_t max_t;
  double rope_theta;
  float softmax_scale;
  int32_t dtype;
  int32_t max_buffer_chunks;
  int32_t reserved;
} sa_config;

#define SA_MAX_TEMPORAL_PAIRS 320
#define SA_MAX_BUFFER_CHUNKS 8
#define SA_MAX_KEY_SEGMENTS 4
#define SA_MAX_BATCH_STREAMS 8

/* Host-side stream state (D3) and the plan of the last attend (D4). */
typedef struct sa_state {
  int64_t n_appends;        /* chunks committed so far; chunk ids are 0..n_appends-1     */
  int64_t ring_commits;     /* commits that went to the window (after the sink filled)   */
  int32_t t_next;           /* temporal position of the next chunk's first frame         */
  int32_t sink_fill;        /* sink chunks holding data, 0..S                            */
  int32_t window_valid;     /* visible window chunks, 0..W                               */
  int32_t staging_slot;     /* physical slot the next chunk's own K/V are staged in      */
  int32_t n_slots;          /* physical slots per (b, h): S + W + 1                      */
  int32_t visible_chunks;   /* chunks the next attend sees, its own included             */
  int32_t visible_keys;     /* keys the next attend sees: visible_chunks * Nc            */
  int32_t staged_valid;     /* 1: the last attend's staged K/V may be committed by
                               sa_kv_append(k = v = NULL)                                */
  int32_t last_q_tiles;     /* attend launch plan: query tiles per (b, h) ...            */
  int32_t last_kv_splits;   /* ... key-range splits per query tile (1 = no combine pass) */
  int32_t last_key_tiles;   /* ... key tiles per query tile, summed over splits          */
  int32_t last_delta;       /* Delta applied by the last sa_rope_refresh                 */
  int32_t last_sk_groups;   /* attend launch plan: persistent stream-K workgroups (0: grid) */
  int32_t reserved;
} sa_state;

/* What a physical cache slot holds. */
typedef enum sa_slot_kind { SA_SLOT_EMPTY = 0, SA_SLOT_SINK = 1, SA_SLOT_WINDOW = 2,
                            SA_SLOT_STAGING = 3 } sa_slot_kind;
typedef struct sa_slot_info {
  int64_t chunk_id;   /* committed chunk id; -1 for sink chunks written by sa_sink_update */
  int32_t t0;         /* temporal position of the slot's first frame                      */
  int32_t kind;       /* sa_slot_kind                                                     */
} sa_slot_info;

/* Byte offsets of the workspace regions (for inspection and tests). Per (b, h):
 *  K cache:   [key_stride][D] rows, slot s at rows [s*Nc, (s+1)*Nc)
 *  V cache:   transposed, [D][key_stride] (keys of all slots contiguous per channel)
 *  Q scratch: [Nc][D] rotated queries of the last attend                           */
typedef struct sa_layout {
  uint64_t k_offset, k_bh_stride;      /* bytes; K row stride = D * elem_bytes          */
  uint64_t vt_offset, vt_bh_stride;    /* bytes; channel stride = key_stride * elem     */
  uint64_t q_offset, q_bh_stride;
  uint64_t partial_offset, partial_bytes;
  uint64_t table_offset, table_bytes;
  int32_t key_stride;                  /* elements per V channel row (>= n_slots*Nc)    */
  int32_t elem_bytes;
  int32_t max_kv_splits;
  int32_t reserved;
} sa_layout;

/* Kernels timed by the optional profiler. */
typedef enum sa_kernel_id {
  SA_K_ROPE_APPLY = 0, SA_K_CHUNK_ATTENTION = 1, SA_K_ATTN_COMBINE = 2,
  SA_K_KV_APPEND = 3, SA_K_ROPE_REFRESH = 4, SA_K_SINK_UPDATE = 5, SA_K_COUNT = 6
} sa_kernel_id;

/* Options for sa_stream_set_option. */
typedef enum sa_option {
  SA_OPT_KV_SPLITS = 0,     /* 0: automatic; n >= 1: force n key-range splits per query tile */
  SA_OPT_PROFILE = 1,       /* 1: record HIP events around every launch (sa_profile_read)    */
  SA_OPT_ATTN_VARIANT = 2,  /* bf16 attention kernel: 0 automatic (3), 1 = 4 waves x 32
                               query rows, 2 = 4 waves x 64 rows, 3 = 8 waves x 32 rows with
                               a ping-pong MFMA/softmax schedule, 4 = 8 waves x 32 rows, each
                               wave software-pipelining its own MFMAs and softmax (head_dim
                               128; other sizes run 3). SA_FP8: 0 or 3 only                   */
  SA_OPT_SCHEDULE = 3       /* variant 3 work distribution: 0 automatic (1), 1 = one workgroup per
                               (b, h, q-tile, split), 2 = stream-K (persistent workgroups
                               sharing the q-tile x key-tile iterations evenly, partial tiles
                               merged by a combine pass)                                     */
} sa_option;

typedef struct sa_stream sa_stream;

/* Human-readable name of a status code (static string). */
const char* sa_status_string(sa_status s);

/* Validate a config; SA_OK if a stream can be created from it. */
sa_status sa_config_check(const sa_config* cfg);

/* Workspace bytes a stream with this config needs (0 if the config is invalid). */
size_t sa_workspace_bytes(const sa_config* cfg);

/*
 * Create a stream handle. d_workspace: caller-owned device memory of at least
 * sa_workspace_bytes(cfg) bytes, 256-byte aligned, or NULL for a planning
 * handle. The RoPE spatial cos/sin tables (host fp64, rounded to fp32) are
 * uploaded into the workspace on `stream`. The stream starts empty: t_next 0,
 * no sink, empty window. *out receives the handle.
 */
sa_status sa_stream_create(const sa_config* cfg, void* d_workspace, size_t workspace_bytes,
                           void* stream, sa_stream** out);

/* Free the host handle (never the workspace). NULL is accepted. */
sa_status sa_stream_destroy(sa_stream* s);

/*
 * Attention of the current chunk (StreamDiffusionV2 2.A.1 chunked processing;
 * SANA-Streaming sink + sliding window). q, k, v: [B, Nc, H, D] inputs of the
 * current chunk; out: [B, Nc, H, D] output; lse: [B, H, Nc] float32 or NULL.
 * Rotates q and k at positions (t_next + frame, y, x), stages the rotated k
 * and v in the staging slot, then computes
 *   out_i = sum_j softmax_j(scale * <q_i, k_j>) v_j
 * over the sink, the window and the chunk itself (full, non-causal inside the
 * chunk). The stream state does not change; the call may be repeated for one
 * chunk (several denoising steps). SA_ERR_POSITION_RANGE if max_t > 0 and
 * t_next + F > max_t.
 */
sa_status sa_chunk_attend(sa_stream* s, const void* q, const void* k, const void* v,
                          void* out, float* lse, void* stream);

/* sa_buffer_attend / sa_buffer_plan flags */
#define SA_BUFFER_STEPS 1u   /* Stream-Batch over denoising steps (see below)        */

/*
 * Several chunks that follow the committed stream as the queries of one call.
 * q, k, v: [B, n*Nc, H, D] holding n consecutive chunks, 1 <= n <=
 * max_buffer_chunks; out: [B, n*Nc, H, D]; lse: [B, H, n*Nc] float32 or NULL.
 * Buffer chunk j is rotated at positions t_next + j*F.. and attends (full
 * softmax) to:
 *  flags = 0, moving buffer (StreamDiT: a buffer of consecutive chunks
 *    denoised together, with window attention): exactly what sa_chunk_attend
 *    would show it once buffer chunks 0..j-1 had been committed -- the sink,
 *    the last W chunks of (the committed window, buffer chunks 0..j-1), and
 *    itself, i.e. a block-banded chunk mask. Needs a full sink
 *    (SA_ERR_BAD_STATE otherwise: earlier buffer chunks would become sink
 *    chunks).
 *  flags = SA_BUFFER_STEPS, Stream-Batch over denoising steps
 *    (StreamDiffusionV2: chunks in flight at different denoising steps form
 *    one batch; none is committed yet): what sa_chunk_attend would show now
 *    (the committed sink chunks and window) plus itself; no buffer chunk sees
 *    another. Any sink fill.
 * The rotated buffer K/V go to the buffer slots; the stream state does not
 * change, except that nothing is staged afterwards (a following sa_kv_append
 * needs explicit k, v). Errors: SA_ERR_INVALID_ARGUMENT for n outside
 * [1, max_buffer_chunks] or unknown flags; SA_ERR_POSITION_RANGE if max_t > 0
 * and t_next + n*F > max_t. Always runs the ping-pong kernel for bf16.
 */
sa_status sa_buffer_attend(sa_stream* s, const void* q, const void* k, const void* v, int32_t n_chunks,
                           uint32_t flags, void* out, float* lse, void* stream);

/*
 * Ragged batch (StreamDiffusionV2 Stream-Batch: one launch serving several
 * streams, each at its own chunk index and position): the same as calling
 * sa_chunk_attend(streams[i], q[i], k[i], v[i], out[i], lse[i]) for i < n, but
 * with one attention launch over all entries, each with its own visible keys.
 * 1 <= n <= SA_MAX_BATCH_STREAMS distinct handles created from equal configs
 * (all planning handles or none); lse may be NULL, as may any lse[i]. Every
 * entry is validated before any launch: on an error no state changes. One
 * RoPE launch stages every entry's chunk in its own workspace, then one
 * attention launch serves all entries; both are recorded by streams[0]'s
 * profiler.
 */
sa_status sa_batch_attend(int32_t n, sa_stream* const* streams, const void* const* q, const void* const* k,
                          const void* const* v, void* const* out, float* const* lse, void* stream);

/*
 * The key segments a sa_buffer_attend of n_chunks and flags would read now (inspection,
 * planning handles included): for buffer chunk j, n_seg[j] <= SA_MAX_KEY_SEGMENTS
 * ranges [seg_lo, seg_hi) of physical key rows of one (b, h), at
 * seg_lo[j * SA_MAX_KEY_SEGMENTS + i]. Rows s*Nc.. belong to physical slot s:
 * slots 0..S-1 the sink, S..S+W the window ring, S+W+1+i buffer chunk i.
 * Segments are disjoint, sorted and not adjacent. Same errors as sa_buffer_attend.
 */
sa_status sa_buffer_plan(const sa_stream* s, int32_t n_chunks, uint32_t flags, int32_t* n_seg,
                         int32_t* seg_lo, int32_t* seg_hi);

/*
 * Commit one chunk (SANA-Streaming, "Transformer a diffusione ibrido": the
 * softmax blocks keep a persistent sink chunk and a sliding local window of the
 * most recent chunks, so the cache stays bounded as the stream grows; this call
 * is the step that slides that window). Its k, v ([B, Nc, H, D]) are rotated
 * at positions t_next.. and stored into the next sink slot while the sink is
 * not full, else into the window, evicting the oldest window chunk; then
 * t_next += F. k and v are read only; ownership stays with the caller. With k = v =
 * NULL the K/V staged by the last sa_chunk_attend are committed without any
 * device work (SA_ERR_BAD_STATE if no attend staged them since the last state
 * change).
 */
sa_status sa_kv_append(sa_stream* s, const void* k, const void* v, void* stream);

/*
 * Re-base temporal RoPE offsets at a chunk boundary (StreamDiffusionV2 2.A.2).
 * new_base_t: >= 0, or -1 for S*F (right after the pinned sink). Delta =
 * (t0 of the oldest visible window chunk, or t_next if none) - new_base_t.
 * Every visible window key is re-rotated by -Delta on the temporal pairs, the
 * window t0s and t_next move by -Delta. The sink stays pinned unless flags has
 * SA_REFRESH_SHIFT_SINK (then it moves too, and attention outputs are
 * unchanged). delta_out (nullable) receives Delta.
 */
sa_status sa_rope_refresh(sa_stream* s, int32_t new_base_t, uint32_t flags, void* stream,
                          int32_t* delta_out);

/*
 * Replace the sink (StreamDiffusionV2 2.A.2: sink tokens updated from recent
 * context; which tokens to use is the caller's policy). k, v: [B, S*Nc, H, D];
 * sink chunk j is rotated at t in [j*F, (j+1)*F). Afterwards the sink counts as
 * full. SA_ERR_BAD_STATE if S = 0.
 */
sa_status sa_sink_update(sa_stream* s, const void* k, const void* v, void* stream);

/* Current state and last launch plan. */
sa_status sa_stream_query(const sa_stream* s, sa_state* out);

/* What physical slot `slot` (0 <= slot < S + W + 1) holds; slots 0..S-1 are the sink. */
sa_status sa_stream_slot(const sa_stream* s, int32_t slot, sa_slot_info* out);

/* Workspace layout of this handle. */
sa_status sa_stream_layout(const sa_stream* s, sa_layout* out);

/* Set an sa_option. SA_ERR_INVALID_ARGUMENT for an unknown option or value. */
sa_status sa_stream_set_option(sa_stream* s, int32_t option, int64_t value);

/*
 * Profiler (SA_OPT_PROFILE = 1): total device milliseconds and launch count of
 * one kernel since the last reset, from HIP events recorded around each
 * launch on the launch stream. Synchronises on the recorded events. reset != 0
 * clears the counters after reading.
 */
sa_status sa_profile_read(sa_stream* s, int32_t kernel_id, double* total_ms, int64_t* launches,
                          int32_t reset);

/*
 * Measurement aid, not an operation of the method: launches `blocks`
 * workgroups of 4 waves that each issue v_mfma_f32_32x32x16_bf16 on 8
 * independent accumulators for `iters` rounds, i.e. blocks*4*iters*8*32768
 * flops, so a caller timing it on `stream` gets the MFMA rate the part
 * sustains (operands are fixed per lane: a benign, low-power case). d_out
 * (caller-owned device memory) receives blocks*256 floats. Asynchronous;
 * SA_ERR_INVALID_ARGUMENT for a null d_out, blocks outside [1, 2^20] or
 * iters < 1.
 */
sa_status sa_probe_mfma_bf16(float* d_out, int32_t blocks, int32_t iters, void* stream);

/*
 * The same measurement on data operands: d_operands (caller-owned device memory, 16-byte
 * aligned) holds 6 runs of 64 lanes x 8 bf16; every wave's lane l takes runs 0-3 as four A
 * operands and runs 4-5 as two B operands, and MFMA j of a round uses A[j % 4] and B[j % 2],
 * so operand values change between consecutive MFMAs as in a real product (normally
 * distributed operands make it the realistic, high-power case). Same flop count, output and
 * asynchrony as sa_probe_mfma_bf16; SA_ERR_INVALID_ARGUMENT also for a null or unaligned
 * d_operands.
 */
sa_status sa_probe_mfma_bf16_data(float* d_out, const void* d_operands, int32_t blocks, int32_t iters,
                                  void* stream);

/*
 * Gated delta rule (GDN linear attention; SANA-Streaming, "Transformer a diffusione
 * ibrido": most blocks keep a fixed-size recurrent state per head, updated as the
 * stream advances, and only the final state is kept between chunks). The pages give no
 * equations; this is the published gated delta rule (Yang, Kautz and Hatamizadeh,
 * "Gated Delta Networks", ICLR 2025), token by token in (frame, y, x) order:
 *   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t,
 * S of size D x D (value rows, key columns) per (b, h).
 *
 * sa_gdn_workspace_bytes: device workspace sa_gdn_forward needs for these sizes (0 for
 * unsupported sizes): per 64-token block of each (b, h), fp32 gates, the block's
 * products in the order the state scan reads them (T diag(gamma) K as three bf16 parts,
 * (T V)^T in fp32, K^T in bf16), the pseudo-values and the block's starting state (D x D).
 *
 * sa_gdn_forward: q, k, v: [B, N, H, D] bf16 (token-major, like sa_chunk_attend's
 * inputs; q and k as the caller prepared them, GDN normalises them to unit length);
 * alpha, beta: [B, H, N] float32 (alpha in (0, 1], beta in [0, 1]); state_in:
 * [B, H, D, D] float32 or NULL for zeros; state_out: [B, H, D, D] float32, may equal
 * state_in; out: [B, N, H, D] bf16. N may be any count >= 0 (a ragged last block is
 * padded with alpha = 1, beta = 0). Arithmetic is fp32-accurate (chunkwise: 64-token
 * blocks, a triangular solve per block, the state carried block to block; products on
 * the bf16 MFMA with fp32 operands split into three bf16 parts and fp32 accumulation). All buffers are
 * the caller's; nothing is allocated. With N = 0 only state_in / state_out are used
 * (the state passes through; the others may be NULL). Errors: SA_ERR_INVALID_ARGUMENT
 * for NULL or misaligned pointers (16 bytes for the bf16 tensors, the states and the
 * workspace, 4 for alpha and beta) or sizes < 1 (N < 0);
 * SA_ERR_UNSUPPORTED for D not 64 or 128, H or B beyond 32767, N beyond 2^24;
 * SA_ERR_WORKSPACE_TOO_SMALL; SA_ERR_DEVICE if a launch fails.
 */
size_t sa_gdn_workspace_bytes(int32_t batch, int32_t tokens, int32_t heads, int32_t head_dim);
sa_status sa_gdn_forward(int32_t batch, int32_t tokens, int32_t heads, int32_t head_dim, const void* q,
                         const void* k, const void* v, const float* alpha, const float* beta,
                         const float* state_in, float* state_out, void* out, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc: sa_gdn_forward without the workspace
 * argument. Its scratch is a fixed device array of SA_GDN_SCRATCH_BYTES inside the library;
 * each GPU the library runs on holds its own copy from the first use until the process ends.
 * The caller still passes every input and output (same meaning, layouts and errors as
 * sa_gdn_forward). Nothing is allocated: sizes whose workspace (sa_gdn_workspace_bytes)
 * exceeds SA_GDN_SCRATCH_BYTES return SA_ERR_WORKSPACE_TOO_SMALL before any device work.
 * The scratch needs no clearing (every call writes what it reads) and keeps the last call's
 * contents. All calls on one GPU share it: calls that overlap on one GPU race, so order them
 * on one stream (or synchronise between streams). The first call on a GPU looks up the
 * array's address there (SA_ERR_DEVICE if that fails); later calls only launch.
 */
#define SA_GDN_SCRATCH_BYTES 67108864
sa_status sa_gdn_forward_noalloc(int32_t batch, int32_t tokens, int32_t heads, int32_t head_dim, const void* q,
                                 const void* k, const void* v, const float* alpha, const float* beta,
                                 const float* state_in, float* state_out, void* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SA_H_ */
