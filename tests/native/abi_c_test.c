/* The C ABI seen from plain C (C99, no C++): the header compiles on its own,
 * the library links, and calls that the host-side checks reject or accept as
 * empty return the documented status without touching a GPU. */
#include <stdio.h>
#include <string.h>

#include "../../include/mla_attn.h"

static int fails = 0;

static void expect(int ok, const char* what) {
  if (!ok) {
    printf("FAILED: %s (last error: %s)\n", what, mla_last_error());
    ++fails;
  }
}

int main(void) {
  void* p = (void*)0x10000; /* never dereferenced: every call below stops in the checks */
  const float sc = 0.07216878f;
  const int32_t* lens = (const int32_t*)0x10000;
  const uint8_t* mask = (const uint8_t*)0x10000;

  expect(strcmp(mla_status_string(MLA_OK), "MLA_OK") == 0, "status string");
  expect(strcmp(mla_status_string((mla_status)99), "unknown status") == 0, "unknown status string");
  expect(mla_attn_decode_workspace_bytes(1, 64, 1001) > 0, "decode workspace for a part-empty grid");
  expect(mla_attn_decode_workspace_bytes(-1, 64, 1001) == 0, "decode workspace for a negative size");

  expect(mla_attn_prefill(NULL, NULL, NULL, NULL, NULL, NULL, 0, 64, 16, 16, 0, sc, NULL) == MLA_OK,
         "empty prefill");
  expect(mla_attn_prefill(p, p, p, p, p, p, 1, 4, 16, 20, 3, sc, NULL) == MLA_ERR_SHAPE,
         "prefill S != past_len + T");
  expect(strstr(mla_last_error(), "mla_attn_prefill") != NULL, "error names the entry point");
  expect(mla_attn_prefill_varlen(p, p, p, p, p, lens, lens, p, 2, 4, 33, 32, sc, NULL) ==
             MLA_ERR_SHAPE, "varlen prefill max_q_len > max_kv_len");
  expect(mla_attn_prefill_masked(p, p, p, p, p, NULL, p, 1, 4, 16, 20, 4, sc, NULL) == MLA_ERR_NULL,
         "masked prefill without a mask");
  expect(mla_attn_decode(p, p, p, p, p, p, NULL, 0, 1, 64, 1001, 1000, sc, NULL) ==
             MLA_ERR_WORKSPACE, "decode without its workspace");
  expect(mla_attn_decode_noalloc(p, p, p, p, p, NULL, 1, 64, 1001, 1000, sc, NULL) == MLA_ERR_NULL,
         "allocation-free decode without out");
  expect(mla_attn_decode_noalloc(p, p, p, p, p, p, 1, 64, 1001, 999, sc, NULL) == MLA_ERR_SHAPE,
         "allocation-free decode S != past_len + 1");
  expect(MLA_DECODE_NOALLOC_SCRATCH_BYTES >= mla_attn_decode_workspace_bytes(1, 255, 257),
         "the allocation-free scratch holds the largest decode workspace");
  expect(mla_attn_decode_masked(p, p, p, p, p, mask, p, p, 1 << 20, 1, 64, 1001, 1000, 1.0f / 0.0f, NULL) ==
             MLA_ERR_SCALE, "masked decode with an infinite scale");
  expect(mla_attn_decode_varlen(p, p, p, p, p, lens, p, p, 1 << 20, 1, 64, 1000, 1001, sc, NULL) ==
             MLA_ERR_SHAPE, "varlen decode max_seq_len > cache_len");
  expect(mla_attn_decode_paged(p, p, p, p, p, lens, lens, NULL, NULL, NULL, p, p, 1 << 20, 4, 64, 100,
                               48, 64, 1024, sc, NULL) == MLA_ERR_SHAPE,
         "paged decode block size not a multiple of 32");
  expect(mla_attn_decode_latent(p, p, p, p, p, p, p, 1 << 20, 1, 80, 11, 10, sc, NULL) == MLA_ERR_SHAPE,
         "latent decode with more than 64 heads");
  expect(mla_attn_prefill_ws(p, p, p, p, p, p, NULL, 0, 1, 2, 256, 4096, 3840, sc, NULL) ==
             MLA_ERR_WORKSPACE, "split prefill without its workspace");

  if (fails) {
    printf("%d failures\n", fails);
    return 1;
  }
  printf("abi c OK\n");
  return 0;
}
