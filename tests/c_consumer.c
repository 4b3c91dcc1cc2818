/*
 * A plain C99 program that uses libfa.so through include/fa.h and the HIP runtime's C API only
 * (no Python, no PyTorch): the test that the boundary is usable as a C library.
 *
 *   c_consumer host
 *       argument checks, status strings, fa_fwd_plan and the empty problem; no GPU call is made.
 *   c_consumer fwd IN OUT B H T d causal scale
 *       IN holds q, k, v as bf16 bit patterns ([B,H,T,d] each, in that order). The program copies
 *       them to device memory, runs fa_fwd on a stream of its own, and writes o (bf16 bits) then
 *       lse (fp32) to OUT.
 *   c_consumer bwd IN OUT B H T d causal scale
 *       IN holds q, k, v and dO (bf16 bits, [B,H,T,d] each). The program runs fa_fwd, then fa_bwd
 *       on its outputs, and writes dq, dk, dv (bf16 bits) then delta (fp32) to OUT.
 *   c_consumer splitkv IN OUT B H T Tk d causal scale n_splits
 *       IN holds q ([B,H,T,d]) then k and v ([B,H,Tk,d]). The program allocates the workspace that
 *       fa_splitkv_workspace_bytes asks for, runs fa_fwd_splitkv and writes o then lse to OUT.
 * Exit status 0 on success; anything else prints what failed.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fa.h"

#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      fprintf(stderr, "c_consumer: ");    \
      fprintf(stderr, __VA_ARGS__);       \
      fprintf(stderr, "\n");              \
      exit(2);                            \
    }                                     \
  } while (0)

#define HIP(call)                                                                          \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    CHECK(e_ == hipSuccess, "%s failed: %s", #call, hipGetErrorString(e_));                \
  } while (0)

static int host_checks(void) {
  /* fake, aligned, distinct addresses: every call below fails validation or is empty, so none is
   * dereferenced and nothing is launched */
  char* a = (char*)(uintptr_t)0x10000;
  int codes[] = {FA_OK, FA_ERR_NULL, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED_D, FA_ERR_ALIGNMENT,
                 FA_ERR_HIP, FA_ERR_TILE, FA_ERR_SCRATCH};
  float* lse = (float*)(a + 0x40000);
  size_t ws;
  size_t i, j;
  fa_plan_info plan;

  for (i = 0; i < sizeof codes / sizeof codes[0]; ++i) {
    const char* s = fa_strerror(codes[i]);
    CHECK(s != NULL && s[0] != '\0', "fa_strerror(%d) is empty", codes[i]);
    for (j = 0; j < i; ++j) CHECK(strcmp(s, fa_strerror(codes[j])) != 0, "status strings repeat");
  }
  CHECK(fa_fwd(NULL, a + 0x10000, a + 0x20000, a + 0x30000, (float*)(a + 0x40000), 1, 1, 8, 64, 1,
               0.125f, NULL) == FA_ERR_NULL, "NULL q accepted");
  CHECK(fa_fwd(a, a + 0x10000, a + 0x20000, a + 0x30000, (float*)(a + 0x40000), 1, 1, 8, 96, 1,
               0.125f, NULL) == FA_ERR_UNSUPPORTED_D, "d = 96 accepted");
  CHECK(fa_fwd(a + 2, a + 0x10000, a + 0x20000, a + 0x30000, (float*)(a + 0x40000), 1, 1, 8, 64, 1,
               0.125f, NULL) == FA_ERR_ALIGNMENT, "misaligned q accepted");
  CHECK(fa_fwd(a, a + 0x10000, a + 0x20000, a + 0x30000, (float*)(a + 0x40000), 1, 1, 0, 64, 1,
               0.125f, NULL) == FA_OK, "empty problem rejected");
  /* the other entry points' checks (each returns before any HIP call) */
  CHECK(fa_fwd_ex(a, a + 0x10000, a + 0x20000, a + 0x30000, lse, 1, 1, 8, 64, 1, 0.125f, NULL, 96,
                  64, 3) == FA_ERR_TILE, "unknown tile accepted");
  CHECK(fa_fwd_ex(a, a + 0x10000, a + 0x20000, a + 0x30000, lse, 1, 1, 8, 64, 1, -1.0f, NULL, 128,
                  64, 4) == FA_ERR_INVALID_ARG, "negative scale accepted");
  CHECK(fa_fwd_sparse(a, a + 0x10000, a + 0x20000, a + 0x30000, lse, 2, 3, 8, 64, 1, 0.125f,
                      (const unsigned char*)(a + 0x50000), 5, NULL) == FA_ERR_INVALID_ARG,
        "mask_heads 5 accepted for B*H = 6");
  CHECK(fa_fwd_sparse(a, a + 0x10000, a + 0x20000, a + 0x30000, lse, 1, 1, FA_SPARSE_MAX_T + 1, 64, 1,
                      0.125f, (const unsigned char*)(a + 0x50000), 1, NULL) == FA_ERR_INVALID_ARG,
        "sparse T above its limit accepted");
  CHECK(fa_fwd_partial(a, a + 0x10000, a + 0x20000, (float*)(a + 0x30000), lse, 1, 1, 8, 100, 64, 1,
                       0.125f, 32, 100, NULL) == FA_ERR_INVALID_ARG, "unaligned k_begin accepted");
  CHECK(fa_merge((const float*)a, (const float*)(a + 0x10000), 0, a + 0x20000, lse, 1, 1, 8, 64,
                 NULL) == FA_ERR_INVALID_ARG, "zero parts accepted");
  ws = fa_splitkv_workspace_bytes(2, 3, 5, 64, 4);
  CHECK(ws == (size_t)4 * 2 * 3 * 5 * 65 * 4, "workspace bytes %zu", ws);
  CHECK(fa_splitkv_workspace_bytes(1, 1, 8, 64, 0) == 0, "workspace for zero splits");
  CHECK(fa_splitkv_splits(4, 12, 1, 16384, 64) >= 1, "split count");
  CHECK(fa_fwd_splitkv(a, a + 0x10000, a + 0x20000, a + 0x30000, lse, 2, 3, 5, 1000, 64, 1, 0.125f, 4,
                       a + 0x60000, ws - 1, NULL) == FA_ERR_INVALID_ARG, "small workspace accepted");
  CHECK(fa_fwd_splitkv_noalloc(a, a + 0x10000, a + 0x20000, a + 0x30000, lse, 1, 1, 1 << 22, 1 << 22,
                               128, 1, 0.0884f, 1, NULL) == FA_ERR_SCRATCH,
        "problem beyond the fixed scratch accepted");
  CHECK(fa_fwd_splitkv_noalloc(a, a + 0x10000, a + 0x20000, a + 0x30000, lse, 1, 1, 0, 100, 64, 1,
                               0.125f, 1, NULL) == FA_OK, "empty no-allocation problem rejected");
  CHECK(fa_fwd_fp8(a, a + 0x10000, a + 0x20000, a + 0x30000, lse, 1, 1, 8, 64, 1, 0.125f, 1.0f, 0.0f,
                   1.0f, NULL) == FA_ERR_INVALID_ARG, "zero descale accepted");
  CHECK(fa_bwd(a, a + 0x10000, a + 0x20000, a + 0x30000, lse, a + 0x50000, a, a + 0x60000,
               a + 0x70000, (float*)(a + 0x80000), 1, 1, 8, 64, 1, 0.125f, NULL) == FA_ERR_INVALID_ARG,
        "dq overlapping q accepted");
  CHECK(fa_fwd_plan(4, 12, 4096, 64, 1, 0, 0, 0, &plan) == FA_OK, "fa_fwd_plan failed");
  CHECK(plan.block_m > 0 && plan.block_n > 0 && plan.waves > 0 && plan.grid > 0,
        "fa_fwd_plan gave an empty launch");
  printf("plan B4 H12 T4096 d64 causal: block %dx%d, %d waves, grid %lld, key split %d\n",
         plan.block_m, plan.block_n, plan.waves, (long long)plan.grid, plan.key_split);
  printf("ok\n");
  return 0;
}

static int forward(int argc, char** argv) {
  const char *in_path, *out_path;
  int B, H, T, d, causal;
  float scale;
  size_t n, bytes_x, bytes_lse;
  uint16_t *host_qkv, *host_o;
  float* host_lse;
  void *q, *k, *v, *o;
  float* lse;
  hipStream_t stream;
  FILE* f;
  int rc;

  CHECK(argc == 10, "usage: c_consumer fwd IN OUT B H T d causal scale");
  in_path = argv[2];
  out_path = argv[3];
  B = atoi(argv[4]);
  H = atoi(argv[5]);
  T = atoi(argv[6]);
  d = atoi(argv[7]);
  causal = atoi(argv[8]);
  scale = (float)atof(argv[9]);
  CHECK(B > 0 && H > 0 && T > 0 && d > 0, "sizes must be positive");
  n = (size_t)B * H * T * d;
  bytes_x = n * sizeof(uint16_t);
  bytes_lse = (size_t)B * H * T * sizeof(float);

  host_qkv = (uint16_t*)malloc(3 * bytes_x);
  host_o = (uint16_t*)malloc(bytes_x);
  host_lse = (float*)malloc(bytes_lse);
  CHECK(host_qkv && host_o && host_lse, "out of host memory");
  f = fopen(in_path, "rb");
  CHECK(f != NULL, "cannot open %s", in_path);
  CHECK(fread(host_qkv, 1, 3 * bytes_x, f) == 3 * bytes_x, "%s is shorter than q, k, v", in_path);
  fclose(f);

  HIP(hipMalloc(&q, bytes_x));
  HIP(hipMalloc(&k, bytes_x));
  HIP(hipMalloc(&v, bytes_x));
  HIP(hipMalloc(&o, bytes_x));
  HIP(hipMalloc((void**)&lse, bytes_lse));
  HIP(hipStreamCreate(&stream));
  HIP(hipMemcpy(q, host_qkv, bytes_x, hipMemcpyHostToDevice));
  HIP(hipMemcpy(k, host_qkv + n, bytes_x, hipMemcpyHostToDevice));
  HIP(hipMemcpy(v, host_qkv + 2 * n, bytes_x, hipMemcpyHostToDevice));

  rc = fa_fwd(q, k, v, o, lse, B, H, T, d, causal, scale, (void*)stream);
  CHECK(rc == FA_OK, "fa_fwd returned %d (%s)", rc, fa_strerror(rc));
  HIP(hipStreamSynchronize(stream));
  HIP(hipMemcpy(host_o, o, bytes_x, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(host_lse, lse, bytes_lse, hipMemcpyDeviceToHost));

  f = fopen(out_path, "wb");
  CHECK(f != NULL, "cannot open %s", out_path);
  CHECK(fwrite(host_o, 1, bytes_x, f) == bytes_x && fwrite(host_lse, 1, bytes_lse, f) == bytes_lse,
        "short write to %s", out_path);
  CHECK(fclose(f) == 0, "cannot close %s", out_path);

  HIP(hipStreamDestroy(stream));
  HIP(hipFree(q));
  HIP(hipFree(k));
  HIP(hipFree(v));
  HIP(hipFree(o));
  HIP(hipFree(lse));
  free(host_qkv);
  free(host_o);
  free(host_lse);
  printf("ok\n");
  return 0;
}

/* n_in bf16 tensors of the given element counts from path, each copied to a new device buffer */
static void read_to_device(const char* path, int n_in, const size_t* counts, void** dev) {
  FILE* f = fopen(path, "rb");
  int i;
  CHECK(f != NULL, "cannot open %s", path);
  for (i = 0; i < n_in; ++i) {
    const size_t bytes = counts[i] * sizeof(uint16_t);
    void* host = malloc(bytes);
    CHECK(host != NULL, "out of host memory");
    CHECK(fread(host, 1, bytes, f) == bytes, "%s is shorter than its inputs", path);
    HIP(hipMalloc(&dev[i], bytes));
    HIP(hipMemcpy(dev[i], host, bytes, hipMemcpyHostToDevice));
    free(host);
  }
  fclose(f);
}

/* n_out device buffers of the given byte counts, in order, to path */
static void write_from_device(const char* path, int n_out, void* const* dev, const size_t* bytes) {
  FILE* f = fopen(path, "wb");
  int i;
  CHECK(f != NULL, "cannot open %s", path);
  for (i = 0; i < n_out; ++i) {
    void* host = malloc(bytes[i]);
    CHECK(host != NULL, "out of host memory");
    HIP(hipMemcpy(host, dev[i], bytes[i], hipMemcpyDeviceToHost));
    CHECK(fwrite(host, 1, bytes[i], f) == bytes[i], "short write to %s", path);
    free(host);
  }
  CHECK(fclose(f) == 0, "cannot close %s", path);
}

static int backward(int argc, char** argv) {
  int B, H, T, d, causal, rc, i;
  float scale;
  size_t n, counts[4], out_bytes[4];
  void *in[4], *o, *out[4];
  float* lse;
  hipStream_t stream;

  CHECK(argc == 10, "usage: c_consumer bwd IN OUT B H T d causal scale");
  B = atoi(argv[4]);
  H = atoi(argv[5]);
  T = atoi(argv[6]);
  d = atoi(argv[7]);
  causal = atoi(argv[8]);
  scale = (float)atof(argv[9]);
  CHECK(B > 0 && H > 0 && T > 0 && d > 0, "sizes must be positive");
  n = (size_t)B * H * T * d;
  for (i = 0; i < 4; ++i) counts[i] = n;
  read_to_device(argv[2], 4, counts, in);  /* q, k, v, dO */
  HIP(hipMalloc(&o, n * 2));
  HIP(hipMalloc((void**)&lse, (size_t)B * H * T * 4));
  for (i = 0; i < 3; ++i) {
    out_bytes[i] = n * 2;
    HIP(hipMalloc(&out[i], out_bytes[i]));
  }
  out_bytes[3] = (size_t)B * H * T * 4;
  HIP(hipMalloc(&out[3], out_bytes[3]));
  HIP(hipStreamCreate(&stream));
  rc = fa_fwd(in[0], in[1], in[2], o, lse, B, H, T, d, causal, scale, (void*)stream);
  CHECK(rc == FA_OK, "fa_fwd returned %d (%s)", rc, fa_strerror(rc));
  rc = fa_bwd(in[0], in[1], in[2], o, lse, in[3], out[0], out[1], out[2], (float*)out[3], B, H, T, d,
              causal, scale, (void*)stream);
  CHECK(rc == FA_OK, "fa_bwd returned %d (%s)", rc, fa_strerror(rc));
  HIP(hipStreamSynchronize(stream));
  write_from_device(argv[3], 4, out, out_bytes);
  HIP(hipStreamDestroy(stream));
  for (i = 0; i < 4; ++i) {
    HIP(hipFree(in[i]));
    HIP(hipFree(out[i]));
  }
  HIP(hipFree(o));
  HIP(hipFree(lse));
  printf("ok\n");
  return 0;
}

static int splitkv(int argc, char** argv) {
  int B, H, T, Tk, d, causal, n_splits, rc, i;
  float scale;
  size_t counts[3], out_bytes[2], ws_bytes;
  void *in[3], *out[2], *ws;
  hipStream_t stream;

  CHECK(argc == 12, "usage: c_consumer splitkv IN OUT B H T Tk d causal scale n_splits");
  B = atoi(argv[4]);
  H = atoi(argv[5]);
  T = atoi(argv[6]);
  Tk = atoi(argv[7]);
  d = atoi(argv[8]);
  causal = atoi(argv[9]);
  scale = (float)atof(argv[10]);
  n_splits = atoi(argv[11]);
  CHECK(B > 0 && H > 0 && T > 0 && Tk > 0 && d > 0 && n_splits > 0, "sizes must be positive");
  counts[0] = (size_t)B * H * T * d;
  counts[1] = counts[2] = (size_t)B * H * Tk * d;
  read_to_device(argv[2], 3, counts, in);  /* q, k, v */
  out_bytes[0] = counts[0] * 2;
  out_bytes[1] = (size_t)B * H * T * 4;
  for (i = 0; i < 2; ++i) HIP(hipMalloc(&out[i], out_bytes[i]));
  ws_bytes = fa_splitkv_workspace_bytes(B, H, T, d, n_splits);
  CHECK(ws_bytes > 0, "fa_splitkv_workspace_bytes returned 0");
  HIP(hipMalloc(&ws, ws_bytes));
  HIP(hipStreamCreate(&stream));
  rc = fa_fwd_splitkv(in[0], in[1], in[2], out[0], (float*)out[1], B, H, T, Tk, d, causal, scale,
                      n_splits, ws, ws_bytes, (void*)stream);
  CHECK(rc == FA_OK, "fa_fwd_splitkv returned %d (%s)", rc, fa_strerror(rc));
  HIP(hipStreamSynchronize(stream));
  write_from_device(argv[3], 2, out, out_bytes);
  HIP(hipStreamDestroy(stream));
  for (i = 0; i < 3; ++i) HIP(hipFree(in[i]));
  for (i = 0; i < 2; ++i) HIP(hipFree(out[i]));
  HIP(hipFree(ws));
  printf("ok\n");
  return 0;
}

int main(int argc, char** argv) {
  CHECK(argc >= 2, "usage: c_consumer host | fwd ... | bwd ... | splitkv ... (see the file's header)");
  if (strcmp(argv[1], "host") == 0) return host_checks();
  if (strcmp(argv[1], "fwd") == 0) return forward(argc, argv);
  if (strcmp(argv[1], "bwd") == 0) return backward(argc, argv);
  if (strcmp(argv[1], "splitkv") == 0) return splitkv(argc, argv);
  CHECK(0, "unknown mode %s", argv[1]);
  return 2;
}
