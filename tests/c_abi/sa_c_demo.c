/*
 * A plain C consumer of the C ABI in include/sa.h: no Python, no torch, only the
 * HIP runtime for device memory and a stream. It runs one bf16 stream over chunk
 * files and writes each chunk's output and log-sum-exp, so that a test can hold them
 * against the oracle.
 *
 *   sa_c_demo DIR B H D FRAME_H FRAME_W F S W N_CHUNKS
 *
 * DIR/q<c>.bin, DIR/k<c>.bin, DIR/v<c>.bin: bf16 [B, Nc, H, D] of chunk c, with
 * Nc = F * FRAME_H * FRAME_W. Per chunk: sa_chunk_attend, then sa_kv_append with
 * k = v = NULL (commit the K/V the attend staged). Writes DIR/out<c>.bin (bf16
 * [B, Nc, H, D]) and DIR/lse<c>.bin (fp32 [B, H, Nc]). Exit status 0 on success,
 * 2 on a usage error (before any device call), 1 on any failed call, which is
 * printed with its status.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sa.h"

#define HIP_OK(call)                                                             \
  do {                                                                           \
    hipError_t e_ = (call);                                                      \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                 \
      return 1;                                                                  \
    }                                                                            \
  } while (0)
#define SA_OK_(call)                                                             \
  do {                                                                           \
    sa_status s_ = (call);                                                       \
    if (s_ != SA_OK) {                                                           \
      fprintf(stderr, "%s: %s\n", #call, sa_status_string(s_));                  \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

static int read_file(const char* dir, const char* name, int c, void* dst, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof(path), "%s/%s%d.bin", dir, name, c);
  FILE* f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "cannot open %s\n", path); return 1; }
  const size_t got = fread(dst, 1, bytes, f);
  fclose(f);
  if (got != bytes) { fprintf(stderr, "%s: %zu of %zu bytes\n", path, got, bytes); return 1; }
  return 0;
}

static int write_file(const char* dir, const char* name, int c, const void* src, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof(path), "%s/%s%d.bin", dir, name, c);
  FILE* f = fopen(path, "wb");
  if (!f) { fprintf(stderr, "cannot create %s\n", path); return 1; }
  const size_t put = fwrite(src, 1, bytes, f);
  fclose(f);
  return put == bytes ? 0 : 1;
}

int main(int argc, char** argv) {
  if (argc != 11) {
    fprintf(stderr, "usage: %s DIR B H D FRAME_H FRAME_W F S W N_CHUNKS\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  sa_config cfg;
  memset(&cfg, 0, sizeof(cfg));                  /* zeros select the defaults (RoPE split, base, scale) */
  cfg.batch = atoi(argv[2]);
  cfg.heads = atoi(argv[3]);
  cfg.head_dim = atoi(argv[4]);
  cfg.frame_h = atoi(argv[5]);
  cfg.frame_w = atoi(argv[6]);
  cfg.frames_per_chunk = atoi(argv[7]);
  cfg.sink_chunks = atoi(argv[8]);
  cfg.window_chunks = atoi(argv[9]);
  cfg.dtype = SA_BF16;
  const int n_chunks = atoi(argv[10]);
  if (sa_config_check(&cfg) != SA_OK || n_chunks < 1) {
    fprintf(stderr, "invalid configuration: %s\n", sa_status_string(sa_config_check(&cfg)));
    return 2;
  }
  const size_t nc = (size_t)cfg.frames_per_chunk * cfg.frame_h * cfg.frame_w;
  const size_t n = (size_t)cfg.batch * nc * cfg.heads * cfg.head_dim;
  const size_t bytes = n * 2, lse_bytes = (size_t)cfg.batch * cfg.heads * nc * 4;

  hipStream_t hs;
  HIP_OK(hipStreamCreate(&hs));
  const size_t ws_bytes = sa_workspace_bytes(&cfg);
  void *ws, *dq, *dk, *dv, *dout;
  float* dlse;
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMalloc(&dq, bytes));
  HIP_OK(hipMalloc(&dk, bytes));
  HIP_OK(hipMalloc(&dv, bytes));
  HIP_OK(hipMalloc(&dout, bytes));
  HIP_OK(hipMalloc((void**)&dlse, lse_bytes));
  uint16_t* h = (uint16_t*)malloc(bytes);
  float* hl = (float*)malloc(lse_bytes);
  if (!h || !hl) { fprintf(stderr, "host allocation failed\n"); return 1; }

  sa_stream* s = NULL;
  SA_OK_(sa_stream_create(&cfg, ws, ws_bytes, hs, &s));
  for (int c = 0; c < n_chunks; ++c) {
    if (read_file(dir, "q", c, h, bytes)) return 1;
    HIP_OK(hipMemcpy(dq, h, bytes, hipMemcpyHostToDevice));
    if (read_file(dir, "k", c, h, bytes)) return 1;
    HIP_OK(hipMemcpy(dk, h, bytes, hipMemcpyHostToDevice));
    if (read_file(dir, "v", c, h, bytes)) return 1;
    HIP_OK(hipMemcpy(dv, h, bytes, hipMemcpyHostToDevice));
    SA_OK_(sa_chunk_attend(s, dq, dk, dv, dout, dlse, hs));
    SA_OK_(sa_kv_append(s, NULL, NULL, hs));
    HIP_OK(hipStreamSynchronize(hs));
    HIP_OK(hipMemcpy(h, dout, bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hl, dlse, lse_bytes, hipMemcpyDeviceToHost));
    if (write_file(dir, "out", c, h, bytes) || write_file(dir, "lse", c, hl, lse_bytes)) return 1;
  }
  sa_state st;
  SA_OK_(sa_stream_query(s, &st));
  printf("chunks %d committed %lld t_next %d sink_fill %d window_valid %d visible_keys %d\n", n_chunks,
         (long long)st.n_appends, st.t_next, st.sink_fill, st.window_valid, st.visible_keys);
  SA_OK_(sa_stream_destroy(s));
  HIP_OK(hipFree(dlse));
  HIP_OK(hipFree(dout));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(ws));
  HIP_OK(hipStreamDestroy(hs));
  free(hl);
  free(h);
  return 0;
}
