// CPU unit test of the host-side argument checks and decode planning
// (attention_mla_causal_amd/csrc/mla_host_checks.h). Built with g++ and
// sanitizers by tests/test_host_checks.py; no HIP headers involved.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>
#include <limits>

#include "../../attention_mla_causal_amd/csrc/mla_host_checks.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);      \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

int main() {
  alignas(16) static char buf[4096];
  const void* p = buf;        // aligned
  const void* bad = buf + 2;  // misaligned
  const float sc = 0.07216878f;
  using namespace mla;

  // valid prefill
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 4, 16, 16, 0, sc, 128).status == MLA_OK);
  EXPECT(!check_prefill(p, p, p, p, p, p, 1, 4, 16, 16, 0, sc, 128).empty);
  // shapes
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 4, 16, 17, 0, sc, 128).status == MLA_ERR_SHAPE);
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 4, 16, 20, 5, sc, 128).status == MLA_ERR_SHAPE);
  EXPECT(check_prefill(p, p, p, p, p, p, -1, 4, 16, 16, 0, sc, 128).status == MLA_ERR_SHAPE);
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 4, 16, 15, -1, sc, 128).status == MLA_ERR_SHAPE);
  // S = past_len + T is formed in 64 bits; S is capped so S * 256 bytes fits 32 bits
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 4, 1, 2147483647LL + 1, 2147483647LL, sc, 128).status == MLA_ERR_SHAPE);
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 4, 1, 8388607, 8388606, sc, 128).status == MLA_OK);
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 4, 1, 8388608, 8388607, sc, 128).status == MLA_ERR_SHAPE);
  EXPECT(check_prefill(p, p, p, p, p, p, 65536, 65536, 2048, 2048, 0, sc, 128).status == MLA_ERR_SHAPE);
  // empty calls are valid no-ops, even with NULL pointers
  {
    CheckResult r = check_prefill(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 4, 16, 16, 0, sc, 128);
    EXPECT(r.status == MLA_OK && r.empty);
    r = check_prefill(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1, 4, 0, 7, 7, sc, 128);
    EXPECT(r.status == MLA_OK && r.empty);
  }
  // NULL and alignment, each argument in turn
  for (int i = 0; i < 6; ++i) {
    const void* a[6] = {p, p, p, p, p, p};
    a[i] = nullptr;
    EXPECT(check_prefill(a[0], a[1], a[2], a[3], a[4], a[5], 1, 2, 3, 3, 0, sc, 128).status == MLA_ERR_NULL);
    a[i] = bad;
    EXPECT(check_prefill(a[0], a[1], a[2], a[3], a[4], a[5], 1, 2, 3, 3, 0, sc, 128).status == MLA_ERR_ALIGN);
  }
  // scale
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 2, 3, 3, 0, NAN, 128).status == MLA_ERR_SCALE);
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 2, 3, 3, 0, INFINITY, 128).status == MLA_ERR_SCALE);
  // any finite scale is valid (zero and negative included) while scale * log2(e) stays finite
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 2, 3, 3, 0, 0.0f, 128).status == MLA_OK);
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 2, 3, 3, 0, -0.0f, 128).status == MLA_OK);
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 2, 3, 3, 0, -0.5f, 128).status == MLA_OK);
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 2, 3, 3, 0, 2.3e38f, 128).status == MLA_OK);
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 2, 3, 3, 0, -2.3e38f, 128).status == MLA_OK);
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 2, 3, 3, 0, -3.0e38f, 128).status == MLA_ERR_SCALE);
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 2, 3, 3, 0, -INFINITY, 128).status == MLA_ERR_SCALE);
  EXPECT(check_prefill(p, p, p, p, p, p, 1, 2, 3, 3, 0, 3.0e38f, 128).status == MLA_ERR_SCALE);

  // decode planning
  {
    DecodePlan pl = plan_decode(1, 64, 1001);
    EXPECT(pl.nsplit == 8 && pl.keys_per_split == 128);
    EXPECT(pl.workspace_bytes == pl.ws_o_bytes + pl.ws_ml_bytes + pl.ws_flag_bytes);
    EXPECT(pl.ws_o_bytes == size_t(64) * 8 * 128 * 4);
    EXPECT(pl.ws_ml_bytes == size_t(64) * 8 * 4 * 4);    // (max, sum, XCD id, unused) per split
    EXPECT(pl.ws_flag_bytes == size_t(64) * 8 * 8);      // one 64-bit completion flag per split
    EXPECT(pl.workspace_bytes % 256 == 0);
    pl = plan_decode(32, 64, 8192);
    EXPECT(pl.nsplit == 1 && pl.workspace_bytes == 0 && pl.keys_per_split >= 8192);
    pl = plan_decode(1, 1, 1);
    EXPECT(pl.nsplit == 1 && pl.workspace_bytes == 0);
    for (long long S : {1LL, 63LL, 64LL, 65LL, 1001LL, 4096LL, 100001LL, 2000000LL}) {
      for (long long bh : {1LL, 3LL, 64LL, 511LL, 512LL, 2048LL}) {
        pl = plan_decode(1, bh, S);
        EXPECT(pl.nsplit >= 1);
        EXPECT(pl.keys_per_split % kDecodeKeysPerTrip == 0);
        EXPECT(pl.keys_per_split * pl.nsplit >= S);               // covers every key
        EXPECT(pl.keys_per_split * (pl.nsplit - 1) < S);          // no empty split
      }
    }
    EXPECT(plan_decode(-1, 4, 10).workspace_bytes == 0);
  }
  // decode checks
  {
    DecodePlan pl;
    const size_t need = plan_decode(1, 64, 1001).workspace_bytes;
    EXPECT(check_decode(p, p, p, p, p, p, p, need, 1, 64, 1001, 1000, sc, &pl).status == MLA_OK);
    EXPECT(pl.nsplit == 8);
    EXPECT(check_decode(p, p, p, p, p, p, p, need - 1, 1, 64, 1001, 1000, sc, &pl).status == MLA_ERR_WORKSPACE);
    EXPECT(check_decode(p, p, p, p, p, p, nullptr, need, 1, 64, 1001, 1000, sc, &pl).status == MLA_ERR_WORKSPACE);
    EXPECT(check_decode(p, p, p, p, p, p, bad, need, 1, 64, 1001, 1000, sc, &pl).status == MLA_ERR_ALIGN);
    EXPECT(check_decode(p, p, p, p, p, p, p, need, 1, 64, 1001, 999, sc, &pl).status == MLA_ERR_SHAPE);
    EXPECT(check_decode(p, p, p, p, p, p, nullptr, 0, 32, 64, 8192, 8191, sc, &pl).status == MLA_OK);
    EXPECT(check_decode(p, p, p, p, p, p, nullptr, 0, 1, 64, 0, -1, sc, &pl).status == MLA_ERR_SHAPE);
    CheckResult r = check_decode(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, 64, 5, 4, sc, &pl);
    EXPECT(r.status == MLA_OK && r.empty);
  }
  // variable-length decode: pieces of at most 1024 keys (8192 from 2048 (b, h)
  // pairs on), at most 64 per (b, h)
  {
    for (long long M : {0LL, 1LL, 1000LL, 1024LL, 1025LL, 4096LL, 8192LL, 65536LL, 100000LL}) {
      for (long long bh : {1LL, 48LL, 2048LL}) {
        const DecodePlan pl = plan_decode_varlen(1, bh, M);
        const DecodePlan base = plan_decode(1, bh, M);
        EXPECT(pl.nsplit >= base.nsplit && pl.nsplit <= 64 + base.nsplit);
        if (M > 0) {
          EXPECT(pl.keys_per_split % kDecodeKeysPerTrip == 0);
          EXPECT(pl.keys_per_split * pl.nsplit >= M);
          EXPECT(pl.keys_per_split * (pl.nsplit - 1) < M);
          const long long piece = bh >= kDecodeVarlenWidePairs ? kDecodeVarlenWideKeysPerSplit : kDecodeVarlenKeysPerSplit;
          EXPECT(pl.keys_per_split <= piece || M > 64 * piece || pl.nsplit == base.nsplit);
        }
        EXPECT(pl.workspace_bytes == (pl.nsplit > 1 ? pl.ws_o_bytes + pl.ws_ml_bytes + pl.ws_flag_bytes : 0));
      }
    }
    EXPECT(plan_decode_varlen(32, 64, 8192).nsplit == 1);    // 2048 pairs: one workgroup each
    EXPECT(plan_decode_varlen(32, 64, 16384).nsplit == 2);
    EXPECT(plan_decode_varlen(16, 64, 8192).nsplit == 8);    // 1024 pairs: pieces of 1024 keys
    EXPECT(plan_decode_varlen(32, 64, 1024).nsplit == 1);
    DecodePlan pl;
    const size_t need = plan_decode_varlen(16, 64, 8192).workspace_bytes;
    EXPECT(check_decode_varlen(p, p, p, p, p, p, p, p, need, 16, 64, 8192, 8192, sc, &pl).status == MLA_OK);
    EXPECT(pl.nsplit == 8);
    EXPECT(check_decode_varlen(p, p, p, p, p, p, p, p, need, 16, 64, 8192, 8193, sc, &pl).status == MLA_ERR_SHAPE);
    EXPECT(check_decode_varlen(p, p, p, p, p, p, p, p, need - 1, 16, 64, 8192, 8192, sc, &pl).status == MLA_ERR_WORKSPACE);
    EXPECT(check_decode_varlen(p, p, nullptr, nullptr, nullptr, p, p, nullptr, 0, 2, 8, 0, 0, sc, &pl).status == MLA_OK);
    EXPECT(check_decode_varlen(p, p, nullptr, p, p, p, p, nullptr, 0, 2, 8, 16, 0, sc, &pl).status == MLA_ERR_NULL);
  }
  // prefill key-range split plan
  {
    for (long long B : {1LL, 2LL}) for (long long H : {1LL, 2LL, 8LL, 64LL})
      for (long long T : {1LL, 100LL, 256LL, 2048LL}) for (long long P : {0LL, 3840LL, 14336LL}) {
        const long long S = P + T;
        const PrefillPlan pl = plan_prefill(B, H, T, S, 128, 32);
        const long long tiles = (S + 31) / 32, wgs = B * H * ((T + 127) / 128);
        EXPECT(pl.nsplit >= 1 && pl.nsplit <= kPrefillMaxSplits);
        if (pl.nsplit > 1) {
          EXPECT(wgs < kPrefillTargetWorkgroups);
          EXPECT(pl.tiles_per_split >= kPrefillMinTilesPerSplit);
          EXPECT(pl.tiles_per_split * pl.nsplit >= tiles);          // every key covered
          EXPECT(pl.tiles_per_split * (pl.nsplit - 1) < tiles);     // every range starts inside
          EXPECT(pl.workspace_bytes == pl.ws_o_bytes + pl.ws_ml_bytes);
          EXPECT(pl.ws_o_bytes >= size_t(B * H * T) * pl.nsplit * 128 * 4);
        } else {
          EXPECT(pl.workspace_bytes == 0);
        }
      }
    EXPECT(plan_prefill(1, 8, 2048, 16384, 128, 32).nsplit == 4);   // one GPU's 8-head share
    EXPECT(plan_prefill(1, 64, 2048, 16384, 128, 32).nsplit == 1);
    PrefillPlan pl;
    const size_t need = plan_prefill(1, 8, 2048, 16384, 128, 32).workspace_bytes;
    EXPECT(check_prefill_ws(p, p, p, p, p, p, p, need, 1, 8, 2048, 16384, 14336, sc, 128, 32, &pl).status == MLA_OK);
    EXPECT(check_prefill_ws(p, p, p, p, p, p, p, need - 1, 1, 8, 2048, 16384, 14336, sc, 128, 32, &pl).status == MLA_ERR_WORKSPACE);
    EXPECT(check_prefill_ws(p, p, p, p, p, p, nullptr, 0, 1, 64, 2048, 16384, 14336, sc, 128, 32, &pl).status == MLA_OK);
  }
  // padded variable-length prefill: sizes, pointers (lengths need 4-byte
  // alignment only), scale and limits
  {
    const void* l4 = reinterpret_cast<const void*>(uintptr_t(0x10004));
    EXPECT(check_prefill_varlen(p, p, p, p, p, p, p, p, 8, 64, 2048, 16384, sc, 128).status == MLA_OK);
    EXPECT(check_prefill_varlen(p, p, p, p, p, l4, l4, p, 8, 64, 2048, 16384, sc, 128).status == MLA_OK);
    EXPECT(check_prefill_varlen(p, p, p, p, p, p, p, p, 8, 64, 2049, 2048, sc, 128).status == MLA_ERR_SHAPE);
    EXPECT(check_prefill_varlen(p, p, p, p, p, p, p, p, -1, 64, 16, 16, sc, 128).status == MLA_ERR_SHAPE);
    EXPECT(check_prefill_varlen(p, p, p, p, p, p, p, p, 1, 64, 16, 8388608, sc, 128).status == MLA_ERR_SHAPE);
    EXPECT(check_prefill_varlen(p, p, p, p, p, p, p, p, 1, 64, 16, 8388607, sc, 128).status == MLA_OK);
    EXPECT(check_prefill_varlen(p, p, p, p, p, p, p, p, 1, 64, 16, 16, 0.0f, 128).status == MLA_OK);
    EXPECT(check_prefill_varlen(p, p, p, p, p, p, p, p, 1, 64, 16, 16, -1.0f, 128).status == MLA_OK);
    EXPECT(check_prefill_varlen(p, p, p, p, p, p, p, p, 1, 64, 16, 16, NAN, 128).status == MLA_ERR_SCALE);
    const CheckResult e = check_prefill_varlen(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                               nullptr, nullptr, 4, 64, 0, 100, sc, 128);
    EXPECT(e.status == MLA_OK && e.empty);
    for (int i = 0; i < 8; ++i) {
      const void* q[8] = {p, p, p, p, p, p, p, p};
      q[i] = nullptr;
      EXPECT(check_prefill_varlen(q[0], q[1], q[2], q[3], q[4], q[5], q[6], q[7], 2, 4, 16, 32, sc, 128).status == MLA_ERR_NULL);
      q[i] = reinterpret_cast<const void*>(uintptr_t(0x10002));
      EXPECT(check_prefill_varlen(q[0], q[1], q[2], q[3], q[4], q[5], q[6], q[7], 2, 4, 16, 32, sc, 128).status == MLA_ERR_ALIGN);
    }
  }
  // latent decode: S limit (1024-byte rows in a 32-bit byte range)
  {
    LatentPlan lp;
    EXPECT(check_latent_decode(p, p, p, p, p, p, p, size_t(1) << 40, 1, 64, 2097151, 2097150, sc, &lp).status == MLA_OK);
    EXPECT(check_latent_decode(p, p, p, p, p, p, p, size_t(1) << 40, 1, 64, 2097152, 2097151, sc, &lp).status == MLA_ERR_SHAPE);
  }
  // rotary prologue: table sizes and parameters, rotation sizes and positions
  {
    EXPECT(rope_table_bytes(4096) == size_t(4096) * 256);
    EXPECT(rope_table_bytes(0) == 0 && rope_table_bytes(-1) == 0);
    EXPECT(rope_table_bytes(int64_t(1) << 24) == (size_t(1) << 24) * 256);
    EXPECT(rope_table_bytes((int64_t(1) << 24) + 1) == 0);
    EXPECT(check_rope_table(p, 4096, 50000.0, 32.0, 4096, 1.0, 1.0).status == MLA_OK);
    EXPECT(check_rope_table(nullptr, 0, 50000.0, 32.0, 4096, 1.0, 1.0).empty);
    EXPECT(check_rope_table(p, -1, 50000.0, 32.0, 4096, 1.0, 1.0).status == MLA_ERR_SHAPE);
    EXPECT(check_rope_table(p, 16, 50000.0, 32.0, 0, 1.0, 1.0).status == MLA_ERR_SHAPE);
    EXPECT(check_rope_table(p, 16, 1.0, 32.0, 4096, 1.0, 1.0).status == MLA_ERR_SCALE);
    EXPECT(check_rope_table(p, 16, NAN, 32.0, 4096, 1.0, 1.0).status == MLA_ERR_SCALE);
    EXPECT(check_rope_table(p, 16, 50000.0, 0.5, 4096, 1.0, 1.0).status == MLA_ERR_SCALE);
    EXPECT(check_rope_table(p, 16, 50000.0, 32.0, 4096, INFINITY, 1.0).status == MLA_ERR_SCALE);
    EXPECT(check_rope_table(nullptr, 16, 50000.0, 32.0, 4096, 1.0, 1.0).status == MLA_ERR_NULL);
    EXPECT(check_rope_table(bad, 16, 50000.0, 32.0, 4096, 1.0, 1.0).status == MLA_ERR_ALIGN);

    const int32_t* lens = reinterpret_cast<const int32_t*>(p);
    EXPECT(check_rope_apply(p, nullptr, p, 4096, 1, 64, 2048, 2048).status == MLA_OK);
    EXPECT(check_rope_apply(p, nullptr, p, 4096, 1, 64, 2048, 2049).status == MLA_ERR_SHAPE);  // position 4096
    EXPECT(check_rope_apply(p, lens, p, 4096, 1, 64, 2048, 2049).status == MLA_OK);  // positions from past_lens
    EXPECT(check_rope_apply(p, nullptr, p, 4096, -1, 64, 1, 0).status == MLA_ERR_SHAPE);
    EXPECT(check_rope_apply(nullptr, nullptr, nullptr, 4096, 0, 64, 5, 0).empty);
    EXPECT(check_rope_apply(p, lens, p, 0, 1, 1, 1, 0).status == MLA_ERR_SHAPE);     // empty table
    EXPECT(check_rope_apply(nullptr, nullptr, p, 16, 1, 1, 1, 0).status == MLA_ERR_NULL);
    EXPECT(check_rope_apply(p, nullptr, nullptr, 16, 1, 1, 1, 0).status == MLA_ERR_NULL);
    EXPECT(check_rope_apply(bad, nullptr, p, 16, 1, 1, 1, 0).status == MLA_ERR_ALIGN);
    EXPECT(check_rope_apply(p, nullptr, bad, 16, 1, 1, 1, 0).status == MLA_ERR_ALIGN);
    EXPECT(check_rope_apply(p, reinterpret_cast<const int32_t*>(reinterpret_cast<uintptr_t>(p) + 4), p,
                            16, 1, 1, 1, 0).status == MLA_OK);                          // lengths: 4-byte alignment
    EXPECT(check_rope_apply(p, reinterpret_cast<const int32_t*>(reinterpret_cast<uintptr_t>(p) + 2), p,
                            16, 1, 1, 1, 0).status == MLA_ERR_ALIGN);
    EXPECT(check_rope_apply(p, lens, p, 1 << 20, 65536, 64, 1024, 0).status == MLA_ERR_SHAPE);  // 2^32 rows

    // the table of a fused-prologue decode: every position below `need`, and
    // at least one row even when no sequence has a key (the kernel reads row 0)
    EXPECT(check_rope_decode_table(p, 1001, 1001).status == MLA_OK);
    EXPECT(check_rope_decode_table(p, 1000, 1001).status == MLA_ERR_SHAPE);
    EXPECT(check_rope_decode_table(p, 0, 0).status == MLA_ERR_SHAPE);
    EXPECT(check_rope_decode_table(p, 1, 0).status == MLA_OK);
    EXPECT(check_rope_decode_table(p, (int64_t(1) << 24) + 1, 16).status == MLA_ERR_SHAPE);
    EXPECT(check_rope_decode_table(nullptr, 16, 16).status == MLA_ERR_NULL);
    EXPECT(check_rope_decode_table(bad, 16, 16).status == MLA_ERR_ALIGN);
  }
  // every decode check accepts zero and negative scales and refuses non-finite ones
  {
    DecodePlan dp;
    EXPECT(check_decode(p, p, p, p, p, p, p, size_t(1) << 30, 1, 64, 1001, 1000, 0.0f, &dp).status == MLA_OK);
    EXPECT(check_decode(p, p, p, p, p, p, p, size_t(1) << 30, 1, 64, 1001, 1000, -0.07f, &dp).status == MLA_OK);
    EXPECT(check_decode(p, p, p, p, p, p, p, size_t(1) << 30, 1, 64, 1001, 1000, NAN, &dp).status == MLA_ERR_SCALE);
    EXPECT(check_decode_varlen(p, p, p, p, p, p, p, p, size_t(1) << 30, 2, 8, 64, 64, -3.0f, &dp).status == MLA_OK);
    EXPECT(check_decode_varlen(p, p, p, p, p, p, p, p, size_t(1) << 30, 2, 8, 64, 64, INFINITY, &dp).status == MLA_ERR_SCALE);
    EXPECT(check_decode_paged(p, p, p, p, p, p, p, nullptr, nullptr, nullptr, p, p, size_t(1) << 30, 2, 8, 4, 32,
                              2, 64, 0.0f, &dp).status == MLA_OK);
    EXPECT(check_decode_paged(p, p, p, p, p, p, p, nullptr, nullptr, nullptr, p, p, size_t(1) << 30, 2, 8, 4, 32,
                              2, 64, NAN, &dp).status == MLA_ERR_SCALE);
    LatentPlan lp;
    EXPECT(check_latent_decode(p, p, p, p, p, p, p, size_t(1) << 30, 1, 64, 1001, 1000, -0.07f, &lp).status == MLA_OK);
    EXPECT(check_latent_decode(p, p, p, p, p, p, p, size_t(1) << 30, 1, 64, 1001, 1000, 0.0f, &lp).status == MLA_OK);
  }
  // latent plan properties over a grid of shapes: every split holds at least
  // one key and a whole number of 32-key tiles; no more than one attention
  // workgroup per CU while B allows it; one head group per workgroup only for
  // more than 48 heads over at most 1024 sequence-tiles; the workspace holds
  // the bf16 absorbed rows, the bf16 partials and their fp32 (max, sum).
  {
    const int64_t Bs[] = {1, 2, 3, 5, 8, 12, 16, 17, 32, 64, 255, 256, 257, 1000};
    const int64_t Hs[] = {1, 8, 16, 17, 48, 49, 63, 64};
    const int64_t Ss[] = {1, 31, 32, 33, 1001, 4096, 8192, 65537, 2097151};
    for (int64_t B : Bs)
      for (int64_t H : Hs)
        for (int64_t S : Ss) {
          const LatentPlan lp = plan_latent(B, H, S);
          const int64_t tiles = (S + 31) / 32, groups = (H + 15) / 16;
          EXPECT(lp.nsplit >= 1 && lp.keys_per_split % 32 == 0 && lp.keys_per_split >= 32);
          EXPECT((lp.nsplit - 1) * lp.keys_per_split < S && S <= lp.nsplit * lp.keys_per_split);
          EXPECT(lp.head_groups == 1 || (lp.head_groups == groups && H > 48 && B * tiles <= 1024));
          if (B * lp.head_groups <= 256) EXPECT(B * lp.nsplit * lp.head_groups <= 256);
          else EXPECT(lp.nsplit == 1);
          EXPECT(lp.qt_bytes >= size_t(B * H * 576 * 2) && lp.po_bytes >= size_t(B * lp.nsplit * H * 512 * 2) &&
                 lp.pml_bytes >= size_t(B * lp.nsplit * H * 2 * 4));
          EXPECT(lp.workspace_bytes == lp.qt_bytes + lp.po_bytes + lp.pml_bytes);
          EXPECT(lp.qt_bytes % 256 == 0 && lp.po_bytes % 256 == 0 && lp.pml_bytes % 256 == 0);
        }
    EXPECT(plan_latent(0, 64, 1001).workspace_bytes == 0);
    EXPECT(plan_latent(1, 64, 1001).head_groups == 4 && plan_latent(1, 64, 1001).nsplit == 32);
    EXPECT(plan_latent(32, 64, 8192).head_groups == 1 && plan_latent(32, 64, 8192).nsplit == 8);
  }
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("host checks OK\n");
  return 0;
}
