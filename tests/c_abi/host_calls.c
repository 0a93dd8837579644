/* A C11 caller of librra.so (no C++, no torch): includes include/rra.h,
 * links the library and makes the host-only calls, which touch no GPU --
 * parameter validation, status strings, workspace sizes and the argument
 * checks that reject a call before anything is launched.  Prints "ok" and
 * exits 0 when every check holds. */
#include <stdio.h>
#include <string.h>

#include "rra.h"

static int failures = 0;

#define EXPECT(cond)                                           \
  do {                                                         \
    if (!(cond)) {                                             \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                              \
    }                                                          \
  } while (0)

static rra_params_t llama_8k(void) {
  rra_params_t p;
  memset(&p, 0, sizeof p); /* zero tail: head round-robin */
  p.batch = 1;
  p.num_heads = 32;
  p.num_kv_heads = 8;
  p.seq_len = 8192;
  p.head_dim = 128;
  p.stride = 16;
  p.block = 128;
  p.tau = 0.9f;
  p.causal = 1;
  p.protect_last = 1;
  return p;
}

int main(void) {
  rra_params_t p = llama_8k();
  size_t bytes = 0;

  EXPECT(rra_abi_version() == RRA_ABI_VERSION);
  EXPECT(sizeof(rra_params_t) == 56);
  EXPECT(rra_validate(&p) == RRA_OK);
  EXPECT(strlen(rra_status_str(RRA_ERR_WORKSPACE)) > 0);

  /* workspace sizes: Kagg (8 x 512 strides x 128 x 2 B) and the score matrix
   * (32 x 64 x 64 x 4 B), each rounded up to 256 B; the attention schedule 1 KB */
  EXPECT(rra_estimate_workspace_size(&p, &bytes) == RRA_OK);
  EXPECT(bytes == (size_t)8 * 512 * 128 * 2 + (size_t)32 * 64 * 64 * 4);
  EXPECT(rra_attn_workspace_size(&p, &bytes) == RRA_OK && bytes == 1024);
  EXPECT(rra_estimate_workspace_size(&p, NULL) == RRA_ERR_INVALID_ARG);

  /* invalid and unsupported parameters */
  p.head_dim = 96;
  EXPECT(rra_validate(&p) == RRA_ERR_UNSUPPORTED);
  p = llama_8k();
  p.num_kv_heads = 5; /* 32 % 5 != 0 */
  EXPECT(rra_validate(&p) != RRA_OK);
  p = llama_8k();
  p.tau = 1.5f;
  EXPECT(rra_validate(&p) == RRA_ERR_INVALID_ARG);
  p = llama_8k();
  p.rr_mode = RRA_RR_NONE;
  p.rr_offset = 16; /* must be < S */
  EXPECT(rra_validate(&p) == RRA_ERR_INVALID_ARG);
  p = llama_8k();
  p.seq_len = 8000; /* ragged: supported */
  EXPECT(rra_validate(&p) == RRA_OK);

  /* rejected before any launch: null pointers, a short workspace */
  p = llama_8k();
  {
    void* fake = (void*)(size_t)(1u << 20); /* aligned, never dereferenced */
    EXPECT(rra_sparse_attn(&p, fake, fake, fake, NULL, fake, fake, NULL, 0, NULL) == RRA_ERR_INVALID_ARG);
    EXPECT(rra_dense_attn(&p, fake, fake, fake, fake, fake, 16, NULL) == RRA_ERR_WORKSPACE);
    EXPECT(rra_estimate(&p, fake, fake, fake, 16, fake, fake, fake, NULL, NULL) == RRA_ERR_WORKSPACE);
  }

  /* an empty problem is a no-op even with null pointers */
  p.batch = 0;
  EXPECT(rra_dense_attn(&p, NULL, NULL, NULL, NULL, NULL, 0, NULL) == RRA_OK);

  if (failures == 0) printf("ok\n");
  return failures == 0 ? 0 : 1;
}
