/*
 * A plain C program that uses libmoba.so through include/moba.h only (no
 * Python, no C++): argument validation without a GPU, and with --gpu one
 * forward and one full attention on device buffers it allocates with the
 * HIP C API.  With every V row equal to the same vector c the softmax weights
 * of a query sum to one, so the output must be c (up to bf16 rounding),
 * whatever the selection: a check that needs no reference implementation.
 * Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moba.h"

static int failures = 0;

static void expect(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++failures;
}

/* fp32 -> bf16, round to nearest even (finite inputs) */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static float from_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint32_t lcg_state = 12345u;
static float uniform_pm1(void) {
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return (float)((lcg_state >> 8) & 0xffffff) / 8388608.0f - 1.0f;
}

static void host_checks(void) {
  expect(moba_abi_version() == MOBA_ABI_VERSION, "ABI version matches the header");
  expect(strcmp(moba_status_string(MOBA_ERR_UNSUPPORTED), "MOBA_ERR_UNSUPPORTED") == 0,
         "status strings");
  moba_status st = moba_forward(NULL, NULL, NULL, 1024, 4, 2, 128, 128, 3, NULL,
                                MOBA_DTYPE_BF16, NULL);
  expect(st == MOBA_ERR_INVALID_ARGUMENT, "NULL tensors are INVALID_ARGUMENT");
  expect(strlen(moba_last_error()) > 0, "moba_last_error explains it");
  moba_args a;
  memset(&a, 0, sizeof(a));
  a.struct_size = sizeof(a);
  a.q = a.k = a.v = (const void*)(uintptr_t)(1ull << 40); /* checked, never dereferenced */
  a.out = (void*)(uintptr_t)(1ull << 40);
  a.batch = 1; a.n_heads = 4; a.n_kv_heads = 2; a.head_dim = 96;
  a.block_size = 128; a.topk = 3; a.q_len = a.kv_len = 1024; a.dtype = MOBA_DTYPE_BF16;
  expect(moba_workspace_size(&a) == 0 && strstr(moba_last_error(), "head_dim") != NULL,
         "head_dim 96 is refused before any launch");
  a.head_dim = 128;
  expect(moba_workspace_size(&a) > 0, "workspace size of a valid problem");
}

static int gpu_checks(void) {
  const int L = 1000, H = 4, Hkv = 2, D = 128, B = 128, topk = 3;
  const size_t nq = (size_t)L * H * D, nk = (size_t)L * Hkv * D;
  uint16_t* hq = malloc(nq * 2);
  uint16_t* hk = malloc(nk * 2);
  uint16_t* hv = malloc(nk * 2);
  uint16_t* ho = malloc(nq * 2);
  float c[128];
  for (int d = 0; d < D; ++d) c[d] = from_bf16(to_bf16(sinf(0.37f * (float)d)));
  for (size_t i = 0; i < nq; ++i) hq[i] = to_bf16(uniform_pm1() * 2.0f);
  for (size_t i = 0; i < nk; ++i) hk[i] = to_bf16(uniform_pm1() * 2.0f);
  for (size_t i = 0; i < nk; ++i) hv[i] = to_bf16(c[i % D]);
  void *dq = NULL, *dk = NULL, *dv = NULL, *dout = NULL;
  if (hipMalloc(&dq, nq * 2) != hipSuccess || hipMalloc(&dk, nk * 2) != hipSuccess ||
      hipMalloc(&dv, nk * 2) != hipSuccess || hipMalloc(&dout, nq * 2) != hipSuccess) {
    printf("FAIL hipMalloc\n");
    return 1;
  }
  if (hipMemcpy(dq, hq, nq * 2, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(dk, hk, nk * 2, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(dv, hv, nk * 2, hipMemcpyHostToDevice) != hipSuccess) {
    printf("FAIL hipMemcpy to the device\n");
    return 1;
  }
  for (int pass = 0; pass < 2; ++pass) {
    moba_status st = pass == 0
        ? moba_forward(dq, dk, dv, L, H, Hkv, D, B, topk, dout, MOBA_DTYPE_BF16, NULL)
        : moba_full_attention(dq, dk, dv, L, H, Hkv, D, dout, MOBA_DTYPE_BF16, NULL);
    expect(st == MOBA_OK, pass == 0 ? "moba_forward returns MOBA_OK"
                                    : "moba_full_attention returns MOBA_OK");
    expect(hipDeviceSynchronize() == hipSuccess, "device synchronises");
    if (hipMemcpy(ho, dout, nq * 2, hipMemcpyDeviceToHost) != hipSuccess) {
      printf("FAIL hipMemcpy to the host\n");
      return 1;
    }
    double worst = 0.0;
    int nonfinite = 0;
    for (size_t i = 0; i < nq; ++i) {
      const double e = fabs((double)from_bf16(ho[i]) - (double)c[i % D]);
      if (!isfinite(e)) nonfinite = 1;
      else if (e > worst) worst = e;
    }
    printf("     max |out - c| = %.3g%s\n", worst, nonfinite ? " (and non-finite values)" : "");
    /* P enters the P.V product in bf16 (2^-9) and out is rounded (2^-9) */
    expect(!nonfinite && worst <= ldexp(1.0, -7), "every output row equals the common V row");
  }
  hipFree(dq); hipFree(dk); hipFree(dv); hipFree(dout);
  free(hq); free(hk); free(hv); free(ho);
  return 0;
}

int main(int argc, char** argv) {
  host_checks();
  if (argc > 1 && strcmp(argv[1], "--gpu") == 0 && gpu_checks() != 0) ++failures;
  printf("%s\n", failures ? "FAILED" : "passed");
  return failures ? 1 : 0;
}
