/* The whole path from C (no Python, no torch): device buffers from the HIP
 * runtime, seeded bf16 inputs from a counter-based generator, then
 * rra_estimate, rra_sparse_attn (with and without the schedule workspace) and
 * rra_dense_attn.  Checks what holds for any input:
 *   tau = 1:   every row keeps all I + 1 causal blocks, in order, and the
 *              block-sparse output is bitwise the dense one;
 *   tau = 0.9: index lists strictly ascending, 1 <= cnt <= I + 1, the mask
 *              agrees with the lists, the last row (protected) keeps all,
 *              outputs finite, and both schedules give the same bits.
 * Prints "ok" and exits 0 when every check holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "rra.h"

#define B 1
#define H 8
#define HKV 2
#define L 2048
#define D 128
#define S 16
#define BK 128
#define NB (L / BK)

static int failures = 0;
#define EXPECT(cond)                                               \
  do {                                                             \
    if (!(cond)) {                                                 \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond);   \
      ++failures;                                                  \
    }                                                              \
  } while (0)
#define HIP_OK(call)                                               \
  do {                                                             \
    hipError_t e_ = (call);                                        \
    if (e_ != hipSuccess) {                                        \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_)); \
      exit(2);                                                     \
    }                                                              \
  } while (0)

/* splitmix64 (a published counter-based generator): value n of stream `seed`. */
static uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

/* bf16 bits of a uniform value in [-1.5, 1.5) (truncated from float). */
static uint16_t bf16_uniform(uint64_t seed, uint64_t n) {
  const double u = (double)(splitmix64(seed * 0x100000001B3ull + n) >> 11) / 9007199254740992.0;
  const float f = (float)(3.0 * u - 1.5);
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  return (uint16_t)(bits >> 16);
}

static float bf16_to_float(uint16_t h) {
  const uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  HIP_OK(hipMalloc(&p, bytes));
  return p;
}

static rra_params_t params(float tau) {
  rra_params_t p;
  memset(&p, 0, sizeof p);
  p.batch = B;
  p.num_heads = H;
  p.num_kv_heads = HKV;
  p.seq_len = L;
  p.head_dim = D;
  p.stride = S;
  p.block = BK;
  p.tau = tau;
  p.causal = 1;
  p.protect_last = 1;
  return p;
}

int main(void) {
  const size_t nq = (size_t)B * H * L * D, nkv = (size_t)B * HKV * L * D;
  uint16_t* hq = malloc(nq * 2);
  uint16_t* hk = malloc(nkv * 2);
  uint16_t* hv = malloc(nkv * 2);
  for (size_t i = 0; i < nq; ++i) hq[i] = bf16_uniform(1, i);
  for (size_t i = 0; i < nkv; ++i) hk[i] = bf16_uniform(2, i);
  for (size_t i = 0; i < nkv; ++i) hv[i] = bf16_uniform(3, i);

  void* q = dev_alloc(nq * 2);
  void* k = dev_alloc(nkv * 2);
  void* v = dev_alloc(nkv * 2);
  HIP_OK(hipMemcpy(q, hq, nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk, nkv * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv, nkv * 2, hipMemcpyHostToDevice));

  const size_t nsel = (size_t)B * H * NB * NB, nrow = (size_t)B * H * NB;
  uint8_t* mask = dev_alloc(nsel);
  int32_t* idx = dev_alloc(nsel * 4);
  int32_t* cnt = dev_alloc(nrow * 4);
  void* out_sp = dev_alloc(nq * 2);
  void* out_st = dev_alloc(nq * 2);
  void* out_dn = dev_alloc(nq * 2);
  uint8_t* hmask = malloc(nsel);
  int32_t* hidx = malloc(nsel * 4);
  int32_t* hcnt = malloc(nrow * 4);
  uint16_t* hsp = malloc(nq * 2);
  uint16_t* hst = malloc(nq * 2);
  uint16_t* hdn = malloc(nq * 2);

  for (int pass = 0; pass < 2; ++pass) {
    const float tau = pass == 0 ? 1.0f : 0.9f;
    rra_params_t p = params(tau);
    size_t est_bytes = 0, attn_bytes = 0;
    EXPECT(rra_estimate_workspace_size(&p, &est_bytes) == RRA_OK);
    EXPECT(rra_attn_workspace_size(&p, &attn_bytes) == RRA_OK);
    void* est_ws = dev_alloc(est_bytes);
    void* attn_ws = dev_alloc(attn_bytes);
    HIP_OK(hipMemset(attn_ws, 0xFF, attn_bytes)); /* contents on entry do not matter */

    EXPECT(rra_estimate(&p, q, k, est_ws, est_bytes, mask, idx, cnt, NULL, NULL) == RRA_OK);
    EXPECT(rra_sparse_attn(&p, q, k, v, idx, cnt, out_sp, attn_ws, attn_bytes, NULL) == RRA_OK);
    EXPECT(rra_sparse_attn(&p, q, k, v, idx, cnt, out_st, NULL, 0, NULL) == RRA_OK);
    EXPECT(rra_dense_attn(&p, q, k, v, out_dn, attn_ws, attn_bytes, NULL) == RRA_OK);
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(hmask, mask, nsel, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hidx, idx, nsel * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hcnt, cnt, nrow * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hsp, out_sp, nq * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hst, out_st, nq * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hdn, out_dn, nq * 2, hipMemcpyDeviceToHost));

    long kept = 0;
    for (size_t r = 0; r < nrow; ++r) {
      const int I = (int)(r % NB);
      const int c = hcnt[r];
      kept += c;
      EXPECT(c >= 1 && c <= I + 1);
      if (pass == 0 || I == NB - 1) EXPECT(c == I + 1);
      int n_mask = 0;
      for (int J = 0; J < NB; ++J) n_mask += hmask[r * NB + J];
      EXPECT(n_mask == c);
      for (int j = 0; j < c; ++j) {
        const int J = hidx[r * NB + j];
        EXPECT(J >= 0 && J <= I && hmask[r * NB + J] == 1);
        if (j > 0) EXPECT(J > hidx[r * NB + j - 1]);
      }
    }
    int finite = 1;
    for (size_t i = 0; i < nq; ++i) finite &= isfinite(bf16_to_float(hsp[i])) ? 1 : 0;
    EXPECT(finite);
    EXPECT(memcmp(hsp, hst, nq * 2) == 0); /* both schedules, same bits */
    if (pass == 0) EXPECT(memcmp(hsp, hdn, nq * 2) == 0); /* tau = 1: sparse == dense, bitwise */
    printf("tau %.2f: density %.4f\n", tau, (double)kept / (double)(B * H * NB * (NB + 1) / 2));
    HIP_OK(hipFree(est_ws));
    HIP_OK(hipFree(attn_ws));
  }

  HIP_OK(hipFree(q));
  HIP_OK(hipFree(k));
  HIP_OK(hipFree(v));
  HIP_OK(hipFree(mask));
  HIP_OK(hipFree(idx));
  HIP_OK(hipFree(cnt));
  HIP_OK(hipFree(out_sp));
  HIP_OK(hipFree(out_st));
  HIP_OK(hipFree(out_dn));
  free(hq); free(hk); free(hv); free(hmask); free(hidx); free(hcnt); free(hsp); free(hst); free(hdn);
  if (failures == 0) printf("ok\n");
  return failures == 0 ? 0 : 1;
}
