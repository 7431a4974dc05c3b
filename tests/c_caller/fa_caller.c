/* A plain C99 program that uses libfa.so through include/fa.h only: the
 * boundary as a C caller sees it (no Python, no torch).
 *
 *   fa_caller check
 *       Calls that need no GPU: version, status strings, workspace sizes and
 *       argument rejection, printed as key=value lines.  A valid call with
 *       fake pointers is also made and its status printed (FA_ERR_DEVICE
 *       where no HIP device exists); it is never made on a machine with a
 *       device (the program then stops before it).
 *   fa_caller run IN OUT
 *       Reads B, H, N, d, dtype, causal (int32), scale (float32) and the
 *       16-bit q, k, v, dO arrays ([B][H][N][d], contiguous) from IN; runs
 *       fa_fwd and fa_bwd on the current HIP device with memory it allocates
 *       itself; writes O, LSE (float32 [B][H][N]), dQ, dK, dV to OUT.
 *
 * Exit status 0 on success; 1 on a library or HIP error (printed). */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fa.h"

static int hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return 1;
  fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return 0;
}

static int fa_ok(int st, const char* what) {
  if (st == FA_OK) return 1;
  fprintf(stderr, "%s: %s (%s)\n", what, fa_status_string(st), fa_last_error_message());
  return 0;
}

static int check(void) {
  /* fake, 16-byte aligned addresses, far apart; never dereferenced */
  const uintptr_t A = (uintptr_t)1 << 20;
  void* const q = (void*)A;
  void* const k = (void*)(2 * A);
  void* const v = (void*)(3 * A);
  void* const o = (void*)(4 * A);
  float* const lse = (float*)(5 * A);
  int st, n;
  printf("version=%d\n", fa_abi_version());
  for (st = 0; st <= 4; ++st) printf("status%d=%s\n", st, fa_status_string(st));
  printf("status99=%s\n", fa_status_string(99));
  printf("bwd_workspace=%lu\n", (unsigned long)fa_bwd_workspace_bytes(2, 8, 2048, 2048, 64, FA_FP16));
  printf("bwd_ex_workspace=%lu\n", (unsigned long)fa_bwd_ex_workspace_bytes(1, 16, 2, 16384, 16384, 128, FA_BF16));
  printf("splitk_workspace=%lu\n", (unsigned long)fa_fwd_splitk_workspace_bytes(1, 2, 16384, 16384, 128, 1, -1, -1));
  st = fa_fwd(NULL, k, v, o, lse, 1, 1, 16, 16, 64, 0.125f, 0, FA_FP16, NULL);
  printf("null_q=%d message=%d\n", st, fa_last_error_message()[0] != '\0');
  printf("d96=%d\n", fa_fwd(q, k, v, o, lse, 1, 1, 16, 16, 96, 0.125f, 0, FA_FP16, NULL));
  printf("o_aliases_q=%d\n", fa_fwd(q, k, v, q, lse, 1, 1, 16, 16, 64, 0.125f, 0, FA_FP16, NULL));
  printf("empty=%d\n", fa_fwd(NULL, NULL, NULL, NULL, NULL, 0, 1, 16, 16, 64, 0.125f, 0, FA_FP16, NULL));
  if (hipGetDeviceCount(&n) == hipSuccess && n > 0) {
    printf("device=present\n");
  } else {
    (void)hipGetLastError();
    printf("valid_without_device=%d\n", fa_fwd(q, k, v, o, lse, 1, 1, 16, 16, 64, 0.125f, 0, FA_FP16, NULL));
  }
  return 0;
}

static int run(const char* in_path, const char* out_path) {
  int32_t hdr[6];
  float scale;
  FILE* f = fopen(in_path, "rb");
  if (!f || fread(hdr, sizeof(int32_t), 6, f) != 6 || fread(&scale, sizeof(float), 1, f) != 1) {
    fprintf(stderr, "cannot read the header of %s\n", in_path);
    if (f) fclose(f);
    return 1;
  }
  const int B = hdr[0], H = hdr[1], N = hdr[2], d = hdr[3], dtype = hdr[4], causal = hdr[5];
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) {
    fprintf(stderr, "bad sizes B=%d H=%d N=%d d=%d\n", B, H, N, d);
    fclose(f);
    return 1;
  }
  const size_t n = (size_t)B * H * N * d, rows = (size_t)B * H * N;
  uint16_t* host = (uint16_t*)malloc(8 * n * sizeof(uint16_t));  /* q k v dO | O dQ dK dV */
  float* host_lse = (float*)malloc(rows * sizeof(float));
  if (!host || !host_lse || fread(host, sizeof(uint16_t), 4 * n, f) != 4 * n) {
    fprintf(stderr, "cannot read the inputs of %s\n", in_path);
    fclose(f);
    free(host);
    free(host_lse);
    return 1;
  }
  fclose(f);

  void* dev[8] = {NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL}; /* q k v dO O dQ dK dV */
  float* lse = NULL;
  void* ws = NULL;
  const size_t ws_bytes = fa_bwd_workspace_bytes(B, H, N, N, d, dtype);
  int ok = 1, i;
  for (i = 0; i < 8 && ok; ++i) ok = hip_ok(hipMalloc(&dev[i], n * sizeof(uint16_t)), "hipMalloc");
  ok = ok && hip_ok(hipMalloc((void**)&lse, rows * sizeof(float)), "hipMalloc lse");
  ok = ok && hip_ok(hipMalloc(&ws, ws_bytes), "hipMalloc workspace");
  for (i = 0; i < 4 && ok; ++i)
    ok = hip_ok(hipMemcpy(dev[i], host + i * n, n * sizeof(uint16_t), hipMemcpyHostToDevice), "hipMemcpy in");
  ok = ok && fa_ok(fa_fwd(dev[0], dev[1], dev[2], dev[4], lse, B, H, N, N, d, scale, causal, dtype, NULL), "fa_fwd");
  ok = ok && fa_ok(fa_bwd(dev[0], dev[1], dev[2], dev[4], lse, dev[3], dev[5], dev[6], dev[7], B, H, N, N, d, scale,
                          causal, dtype, ws, ws_bytes, NULL),
                   "fa_bwd");
  ok = ok && hip_ok(hipDeviceSynchronize(), "kernels");
  for (i = 4; i < 8 && ok; ++i)
    ok = hip_ok(hipMemcpy(host + i * n, dev[i], n * sizeof(uint16_t), hipMemcpyDeviceToHost), "hipMemcpy out");
  ok = ok && hip_ok(hipMemcpy(host_lse, lse, rows * sizeof(float), hipMemcpyDeviceToHost), "hipMemcpy lse");
  if (ok) {
    FILE* g = fopen(out_path, "wb");
    ok = g && fwrite(host + 4 * n, sizeof(uint16_t), n, g) == n && fwrite(host_lse, sizeof(float), rows, g) == rows &&
         fwrite(host + 5 * n, sizeof(uint16_t), 3 * n, g) == 3 * n;
    if (g) ok = fclose(g) == 0 && ok;
    if (!ok) fprintf(stderr, "cannot write %s\n", out_path);
  }
  for (i = 0; i < 8; ++i) (void)hipFree(dev[i]);
  (void)hipFree(lse);
  (void)hipFree(ws);
  free(host);
  free(host_lse);
  return ok ? 0 : 1;
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "check") == 0) return check();
  if (argc == 4 && strcmp(argv[1], "run") == 0) return run(argv[2], argv[3]);
  fprintf(stderr, "usage: %s check | run IN OUT\n", argv[0]);
  return 2;
}
