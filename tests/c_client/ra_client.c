/*
 * A plain C client of the ring-attention C ABI (include/ra.h): no Python and no
 * torch, only the HIP runtime for device memory and a stream.  The tests build it
 * with a C compiler and drive it through files.
 *
 *   ra_client host <S> <p> <layout> <causal>
 *       The host-only entry points, for batch 1, one head, d = 64: prints
 *       "pos c pos(c,0) ... pos(c,L-1)" for every chunk c, then
 *       "pairs cq ck n" for every (query chunk, KV chunk) pair.
 *   ra_client fwd <in> <out>
 *       Reads a problem and one rank's inputs from <in>, runs ra_ring_fwd on the
 *       GPU and writes out and lse to <out>.
 *
 * <in>:  12 int64 values: B Hq Hkv d D S p layout causal dtype rank 0, then the
 *        rank's query chunk q [B, Hq, L, D] and, for c = 0 .. p-1, k_c then v_c
 *        ([B, Hkv, L, D]), as raw elements of the problem dtype (fp32, or bf16 bits).
 * <out>: out [B, Hq, L, D] in the problem dtype, then lse fp32 [B, Hq, L].
 * Exit status: 0 on success, 1 for bad usage or files, 2 for a HIP error, 3 for a
 * status other than RA_OK (the message names the call and ra_last_error()).
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ra.h"

#define HIP_CHECK(x)                                                           \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                  \
      exit(2);                                                                 \
    }                                                                          \
  } while (0)

#define RA_CHECK(x)                                                            \
  do {                                                                         \
    ra_status_t s_ = (x);                                                      \
    if (s_ != RA_OK) {                                                         \
      fprintf(stderr, "%s: %s: %s\n", #x, ra_status_str(s_), ra_last_error()); \
      exit(3);                                                                 \
    }                                                                          \
  } while (0)

/* Contiguous [B, H, L, D] tensors for q, every k/v chunk and out. */
static ra_problem_t make_problem(const int64_t h[12]) {
  ra_problem_t p;
  memset(&p, 0, sizeof p);
  p.batch = h[0];
  p.heads_q = h[1];
  p.heads_kv = h[2];
  p.head_dim = h[3];
  p.head_dim_padded = h[4];
  p.seq_total = h[5];
  p.world = (int32_t)h[6];
  p.layout = (int32_t)h[7];
  p.causal = (int32_t)h[8];
  p.dtype = (int32_t)h[9];
  const int64_t L = h[6] > 0 ? h[5] / h[6] : 0, D = h[4];
  p.q_stride[0] = p.o_stride[0] = h[1] * L * D;
  p.kv_stride[0] = h[2] * L * D;
  p.q_stride[1] = p.kv_stride[1] = p.o_stride[1] = L * D;
  p.q_stride[2] = p.kv_stride[2] = p.o_stride[2] = D;
  return p;
}

static int host_mode(int argc, char** argv) {
  if (argc != 6) return 1;
  const int64_t S = atoll(argv[2]), world = atoll(argv[3]);
  const int64_t h[12] = {1, 1, 1, 64, 64, S, world, atoll(argv[4]), atoll(argv[5]), RA_F32, 0, 0};
  const ra_problem_t p = make_problem(h);
  const int64_t L = S / world;
  int64_t* pos = (int64_t*)malloc((size_t)L * sizeof(int64_t));
  if (pos == NULL) return 1;
  for (int32_t c = 0; c < p.world; ++c) {
    RA_CHECK(ra_positions(&p, c, pos));
    printf("pos %d", c);
    for (int64_t t = 0; t < L; ++t) printf(" %lld", (long long)pos[t]);
    printf("\n");
  }
  for (int32_t cq = 0; cq < p.world; ++cq)
    for (int32_t ck = 0; ck < p.world; ++ck) {
      int64_t n = -1;
      RA_CHECK(ra_visible_pairs(&p, cq, ck, &n));
      printf("pairs %d %d %lld\n", cq, ck, (long long)n);
    }
  free(pos);
  return 0;
}

static void* read_exact(FILE* f, size_t bytes) {
  void* buf = malloc(bytes ? bytes : 1);
  if (buf == NULL || fread(buf, 1, bytes, f) != bytes) {
    fprintf(stderr, "short input file\n");
    exit(1);
  }
  return buf;
}

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  HIP_CHECK(hipMalloc(&d, bytes));
  HIP_CHECK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

static int fwd_mode(int argc, char** argv) {
  if (argc != 4) return 1;
  FILE* in = fopen(argv[2], "rb");
  if (in == NULL) return 1;
  int64_t h[12];
  if (fread(h, sizeof(int64_t), 12, in) != 12) return 1;
  const ra_problem_t p = make_problem(h);
  const int32_t rank = (int32_t)h[10];
  if (p.world < 1 || p.world > 64) return 1;
  const size_t es = p.dtype == RA_BF16 ? 2 : 4;
  const int64_t L = p.seq_total / p.world, D = p.head_dim_padded;
  const size_t nq = (size_t)(p.batch * p.heads_q * L * D);
  const size_t nkv = (size_t)(p.batch * p.heads_kv * L * D);
  const size_t nl = (size_t)(p.batch * p.heads_q * L);

  void* q_h = read_exact(in, nq * es);
  void* q_d = to_device(q_h, nq * es);
  free(q_h);
  const void* k_d[64];
  const void* v_d[64];
  for (int32_t c = 0; c < p.world; ++c) {
    void* k_h = read_exact(in, nkv * es);
    k_d[c] = to_device(k_h, nkv * es);
    free(k_h);
    void* v_h = read_exact(in, nkv * es);
    v_d[c] = to_device(v_h, nkv * es);
    free(v_h);
  }
  fclose(in);

  void *out_d = NULL, *ws_d = NULL;
  float* lse_d = NULL;
  size_t ws_bytes = 0;
  RA_CHECK(ra_ring_workspace_size(&p, &ws_bytes));
  HIP_CHECK(hipMalloc(&out_d, nq * es));
  HIP_CHECK(hipMalloc((void**)&lse_d, nl * sizeof(float)));
  HIP_CHECK(hipMalloc(&ws_d, ws_bytes));
  hipStream_t stream;
  HIP_CHECK(hipStreamCreate(&stream));
  RA_CHECK(ra_ring_fwd(&p, rank, q_d, k_d, v_d, out_d, lse_d, ws_d, ws_bytes, stream));
  HIP_CHECK(hipStreamSynchronize(stream));

  void* out_h = malloc(nq * es);
  float* lse_h = (float*)malloc(nl * sizeof(float));
  if (out_h == NULL || lse_h == NULL) return 1;
  HIP_CHECK(hipMemcpy(out_h, out_d, nq * es, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(lse_h, lse_d, nl * sizeof(float), hipMemcpyDeviceToHost));
  FILE* out = fopen(argv[3], "wb");
  if (out == NULL || fwrite(out_h, 1, nq * es, out) != nq * es ||
      fwrite(lse_h, sizeof(float), nl, out) != nl)
    return 1;
  fclose(out);

  HIP_CHECK(hipStreamDestroy(stream));
  HIP_CHECK(hipFree(q_d));
  for (int32_t c = 0; c < p.world; ++c) {
    HIP_CHECK(hipFree((void*)k_d[c]));
    HIP_CHECK(hipFree((void*)v_d[c]));
  }
  HIP_CHECK(hipFree(out_d));
  HIP_CHECK(hipFree(lse_d));
  HIP_CHECK(hipFree(ws_d));
  free(out_h);
  free(lse_h);
  return 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "host") == 0) return host_mode(argc, argv);
  if (argc >= 2 && strcmp(argv[1], "fwd") == 0) return fwd_mode(argc, argv);
  fprintf(stderr, "usage: ra_client host S p layout causal | ra_client fwd IN OUT\n");
  return 1;
}
