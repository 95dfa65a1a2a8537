// Host-side argument checks and launch planning for the MLA attention core.
//
// Plain C++17, no HIP headers: the library uses it before any HIP call, and a
// g++ unit test (with sanitizers) exercises every status code on the CPU.
//
// The shape rules follow the attention-core excerpt on the Kimi K2
// "Similarities" page ("Query-key similarity"): scores must be
// (B, H, T, kv_seq_len) and the mask (B, 1, T, kv_seq_len), with
// kv_seq_len = past_len + T, else the call is rejected.
#ifndef MLA_HOST_CHECKS_H_
#define MLA_HOST_CHECKS_H_

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdio>

#include "../../include/mla_attn.h"

namespace mla {

// Decode: keys one workgroup consumes per loop trip (4 waves x 4 quarter-waves x 8 keys).
constexpr int64_t kDecodeKeysPerTrip = 128;
// Decode split heuristic: aim for this many workgroups (2 per CU on 256 CUs).
constexpr int64_t kDecodeTargetWorkgroups = 512;
constexpr int64_t kMaxGrid = 2147483647;  // grid.x limit
// The prefill and latent kernels address a sequence's keys through buffer
// resources whose 32-bit byte range must hold S rows of 256 bytes (k_nope, v)
// or 1024 bytes (latent); longer sequences are refused.
constexpr int64_t kMaxPrefillKeys = 2147483647 / 256;  // 8,388,607
constexpr int64_t kMaxLatentKeys = 2147483647 / 1024;  // 2,097,151

struct DecodePlan {
  int64_t nsplit = 1;          // workgroups per (b, h)
  int64_t keys_per_split = 0;  // multiple of kDecodeKeysPerTrip
  size_t ws_o_bytes = 0;       // fp32 [B*H, nsplit, 128]
  size_t ws_ml_bytes = 0;      // fp32 (max, sum, XCD id, unused) [B*H, nsplit]
  size_t ws_flag_bytes = 0;     // u64 completion flags [B*H, nsplit]
  size_t workspace_bytes = 0;  // total, each region 256-byte aligned
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Split the key range of each (b, h) over enough workgroups to fill the chip
// when B*H alone is too small, never making a split smaller than one trip.
inline DecodePlan plan_decode(int64_t B, int64_t H, int64_t S) {
  DecodePlan p;
  if (B <= 0 || H <= 0 || S <= 0) return p;
  const int64_t bh = B * H;
  int64_t nsplit = 1;
  if (bh < kDecodeTargetWorkgroups / 2) {
    nsplit = (kDecodeTargetWorkgroups + bh - 1) / bh;
    const int64_t max_split = (S + kDecodeKeysPerTrip - 1) / kDecodeKeysPerTrip;
    if (nsplit > max_split) nsplit = max_split;
    if (nsplit < 1) nsplit = 1;
  }
  int64_t kps = (S + nsplit - 1) / nsplit;
  kps = (kps + kDecodeKeysPerTrip - 1) / kDecodeKeysPerTrip * kDecodeKeysPerTrip;
  nsplit = (S + kps - 1) / kps;  // every split owns at least one key
  p.nsplit = nsplit;
  p.keys_per_split = kps;
  if (nsplit > 1) {
    p.ws_o_bytes = align256(size_t(bh) * size_t(nsplit) * 128 * sizeof(float));
    p.ws_ml_bytes = align256(size_t(bh) * size_t(nsplit) * 4 * sizeof(float));
    p.ws_flag_bytes = align256(size_t(bh) * size_t(nsplit) * sizeof(unsigned long long));
    p.workspace_bytes = p.ws_o_bytes + p.ws_ml_bytes + p.ws_flag_bytes;
  }
  return p;
}

// Variable-length decode: lengths differ, so a (b, h) with many keys would
// keep its workgroup running long after the short ones finished. Splitting
// every (b, h) into pieces of at most this many keys bounds that tail (the
// pieces past a short sequence's end find no key and finish at once). With
// many (b, h) pairs the GPU is full without splitting and the pieces' fixed
// costs (partials, completion flags, the merge; for a 2D mask a round trip
// for the mask bytes per piece) outweigh the tail they even out: at 32 x 64
// pairs over 8192 keys one workgroup per pair measured 0.633 against 0.648
// ms (variable lengths), 0.660 against 0.669 (paged) and 0.640 against 0.725
// (left-padding mask), so from kDecodeVarlenWidePairs pairs on the pieces
// are kDecodeVarlenWideKeysPerSplit keys long.
constexpr int64_t kDecodeVarlenKeysPerSplit = 1024;
constexpr int64_t kDecodeVarlenWidePairs = 2048;  // 8 workgroups per CU on 256 CUs
constexpr int64_t kDecodeVarlenWideKeysPerSplit = 8192;
constexpr int64_t kDecodeMaxFusedSplits = 64;

inline DecodePlan plan_decode_varlen(int64_t B, int64_t H, int64_t max_len) {
  DecodePlan p = plan_decode(B, H, max_len);
  if (B <= 0 || H <= 0 || max_len <= 0) return p;
  const int64_t piece = B * H >= kDecodeVarlenWidePairs ? kDecodeVarlenWideKeysPerSplit : kDecodeVarlenKeysPerSplit;
  int64_t want = (max_len + piece - 1) / piece;
  if (want > kDecodeMaxFusedSplits) want = kDecodeMaxFusedSplits;
  if (want <= p.nsplit) return p;
  int64_t kps = (max_len + want - 1) / want;
  kps = (kps + kDecodeKeysPerTrip - 1) / kDecodeKeysPerTrip * kDecodeKeysPerTrip;
  const int64_t nsplit = (max_len + kps - 1) / kps;
  const int64_t bh = B * H;
  p.nsplit = nsplit;
  p.keys_per_split = kps;
  p.ws_o_bytes = align256(size_t(bh) * size_t(nsplit) * 128 * sizeof(float));
  p.ws_ml_bytes = align256(size_t(bh) * size_t(nsplit) * 4 * sizeof(float));
  p.ws_flag_bytes = align256(size_t(bh) * size_t(nsplit) * sizeof(unsigned long long));
  p.workspace_bytes = p.ws_o_bytes + p.ws_ml_bytes + p.ws_flag_bytes;
  return p;
}

struct CheckResult {
  mla_status status = MLA_OK;
  bool empty = false;  // valid call with nothing to compute
  char msg[256] = {0};
};

inline CheckResult fail(mla_status s, const char* what) {
  CheckResult r;
  r.status = s;
  std::snprintf(r.msg, sizeof(r.msg), "%s", what);
  return r;
}

inline bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// softmax_scale: any finite value, of either sign or zero, whose product with
// log2(e) (the factor the kernels fold into their exponent) is a finite fp32
// (|scale| <= FLT_MAX / log2(e), about 2.36e38). Returns true, with r filled
// in, when the scale is refused.
inline bool check_scale(float scale, CheckResult* r) {
  const float c = scale * 1.4426950408889634f;
  if (std::isfinite(scale) && std::isfinite(c)) return false;
  std::snprintf(r->msg, sizeof(r->msg),
                "softmax_scale %g must be finite, with softmax_scale * log2(e) finite in fp32",
                (double)scale);
  r->status = MLA_ERR_SCALE;
  return true;
}

// Common part of both entry points. T is the number of new queries.
inline CheckResult check_common(const void* q_nope, const void* q_pe, const void* k_nope,
                                const void* k_pe, const void* v, const void* out, int64_t B,
                                int64_t H, int64_t T, int64_t S, int64_t past_len, float scale,
                                const char* const* tensor_names = nullptr) {
  CheckResult r;
  if (B < 0 || H < 0 || T < 0 || S < 0 || past_len < 0) {
    std::snprintf(r.msg, sizeof(r.msg),
                  "negative size: B=%lld H=%lld T=%lld S=%lld past_len=%lld", (long long)B,
                  (long long)H, (long long)T, (long long)S, (long long)past_len);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (S != past_len + T) {
    std::snprintf(r.msg, sizeof(r.msg),
                  "kv_seq_len S=%lld must equal past_len %lld + query length %lld", (long long)S,
                  (long long)past_len, (long long)T);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (B == 0 || H == 0 || T == 0) {
    r.empty = true;
    return r;
  }
  // every tensor is non-empty from here on (S >= T >= 1)
  const void* ptrs[6] = {q_nope, q_pe, k_nope, k_pe, v, out};
  static const char* const default_names[6] = {"q_nope", "q_pe", "k_nope", "k_pe", "v", "out"};
  const char* const* names = tensor_names ? tensor_names : default_names;
  for (int i = 0; i < 6; ++i) {
    if (ptrs[i] == nullptr) {
      std::snprintf(r.msg, sizeof(r.msg), "%s is NULL", names[i]);
      r.status = MLA_ERR_NULL;
      return r;
    }
  }
  for (int i = 0; i < 6; ++i) {
    if (misaligned(ptrs[i])) {
      std::snprintf(r.msg, sizeof(r.msg), "%s is not 16-byte aligned", names[i]);
      r.status = MLA_ERR_ALIGN;
      return r;
    }
  }
  if (check_scale(scale, &r)) return r;
  return r;
}

// Prefill key-range split: when B*H*ceil(T/block_m) workgroups would leave
// the GPU part-empty (it holds two per CU), each query tile's keys are split
// over several workgroups, each writing an fp32 partial that a second kernel
// merges. The plan fixes the number of ranges from the whole key count; the
// kernel cuts the keys each query tile sees into that many near-equal ranges
// (no longer than tiles_per_split).
constexpr int64_t kPrefillTargetWorkgroups = 512;
constexpr int64_t kPrefillMinTilesPerSplit = 16;  // 512 keys: pipeline fill and drain stay small
constexpr int64_t kPrefillMaxSplits = 16;  // the merge kernel holds at most 16 partials per row

struct PrefillPlan {
  int64_t nsplit = 1;           // key ranges per query tile
  int64_t tiles_per_split = 0;  // key tiles (kPrefillKeyTile keys) per range of the whole key count
  size_t ws_o_bytes = 0;        // fp32 [B*H*T, nsplit, 128]
  size_t ws_ml_bytes = 0;       // fp32 [B*H*T, nsplit, 2]
  size_t workspace_bytes = 0;
};

inline PrefillPlan plan_prefill(int64_t B, int64_t H, int64_t T, int64_t S, int64_t block_m,
                                int64_t key_tile) {
  PrefillPlan p;
  if (B <= 0 || H <= 0 || T <= 0 || S <= 0 || block_m <= 0 || key_tile <= 0) return p;
  const int64_t wgs = B * H * ((T + block_m - 1) / block_m);
  if (wgs >= kPrefillTargetWorkgroups) return p;
  const int64_t tiles = (S + key_tile - 1) / key_tile;
  // never past two workgroups per CU: a grid just past 512 runs a second
  // round for a few workgroups
  int64_t n = kPrefillTargetWorkgroups / wgs;
  const int64_t by_len = tiles / kPrefillMinTilesPerSplit;
  if (n > by_len) n = by_len;
  if (n > kPrefillMaxSplits) n = kPrefillMaxSplits;
  if (n <= 1) return p;
  const int64_t tps = (tiles + n - 1) / n;
  n = (tiles + tps - 1) / tps;  // every range starts inside the keys
  if (n <= 1) return p;
  const size_t rows = size_t(B) * size_t(H) * size_t(T);
  p.nsplit = n;
  p.tiles_per_split = tps;
  p.ws_o_bytes = align256(rows * size_t(n) * 128 * sizeof(float));
  p.ws_ml_bytes = align256(rows * size_t(n) * 2 * sizeof(float));
  p.workspace_bytes = p.ws_o_bytes + p.ws_ml_bytes;
  return p;
}

// block_m: queries per prefill workgroup (a property of the kernel build).
inline CheckResult check_prefill(const void* q_nope, const void* q_pe, const void* k_nope,
                                 const void* k_pe, const void* v, const void* out, int64_t B,
                                 int64_t H, int64_t T, int64_t S, int64_t past_len, float scale,
                                 int64_t block_m) {
  CheckResult r = check_common(q_nope, q_pe, k_nope, k_pe, v, out, B, H, T, S, past_len, scale);
  if (r.status != MLA_OK || r.empty) return r;
  if (S > kMaxPrefillKeys) {
    std::snprintf(r.msg, sizeof(r.msg), "S=%lld keys exceeds the prefill limit of %lld",
                  (long long)S, (long long)kMaxPrefillKeys);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  const int64_t tiles = (T + block_m - 1) / block_m;
  if (B * H > kMaxGrid / tiles) {
    std::snprintf(r.msg, sizeof(r.msg), "B*H*ceil(T/%lld) = %lld*%lld exceeds the grid limit",
                  (long long)block_m, (long long)(B * H), (long long)tiles);
    r.status = MLA_ERR_SHAPE;
  }
  return r;
}

// The prefill with a workspace: as check_prefill, plus the split plan's
// workspace and grid.
inline CheckResult check_prefill_ws(const void* q_nope, const void* q_pe, const void* k_nope,
                                    const void* k_pe, const void* v, const void* out,
                                    const void* workspace, size_t workspace_bytes, int64_t B,
                                    int64_t H, int64_t T, int64_t S, int64_t past_len,
                                    float scale, int64_t block_m, int64_t key_tile,
                                    PrefillPlan* plan_out) {
  CheckResult r = check_prefill(q_nope, q_pe, k_nope, k_pe, v, out, B, H, T, S, past_len, scale,
                                block_m);
  if (r.status != MLA_OK || r.empty) return r;
  const PrefillPlan plan = plan_prefill(B, H, T, S, block_m, key_tile);
  const int64_t tiles = (T + block_m - 1) / block_m;
  if (B * H * tiles > kMaxGrid / plan.nsplit) {
    std::snprintf(r.msg, sizeof(r.msg), "B*H*ceil(T/%lld)*nsplit exceeds the grid limit",
                  (long long)block_m);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (plan.workspace_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) {
      std::snprintf(r.msg, sizeof(r.msg), "workspace %s: %zu bytes given, %zu needed",
                    workspace == nullptr ? "is NULL" : "too small", workspace_bytes,
                    plan.workspace_bytes);
      r.status = MLA_ERR_WORKSPACE;
      return r;
    }
    if (misaligned(workspace)) {
      std::snprintf(r.msg, sizeof(r.msg), "workspace is not 16-byte aligned");
      r.status = MLA_ERR_ALIGN;
      return r;
    }
  }
  if (plan_out) *plan_out = plan;
  return r;
}

// ---- prefill of a padded, variable-length batch: sequence b has q_lens[b]
// new queries (rows [0, q_lens[b]) of its [max_q_len] query rows) over
// past_lens[b] cached keys (its keys are rows [0, past_lens[b] + q_lens[b])
// of its [max_kv_len] key rows); both arrays live in device memory.
inline CheckResult check_prefill_varlen(const void* q_nope, const void* q_pe, const void* k_nope,
                                        const void* k_pe, const void* v, const void* q_lens,
                                        const void* past_lens, const void* out, int64_t B,
                                        int64_t H, int64_t max_q, int64_t max_kv, float scale,
                                        int64_t block_m) {
  CheckResult r;
  if (B < 0 || H < 0 || max_q < 0 || max_kv < 0) {
    std::snprintf(r.msg, sizeof(r.msg),
                  "negative size: B=%lld H=%lld max_q_len=%lld max_kv_len=%lld", (long long)B,
                  (long long)H, (long long)max_q, (long long)max_kv);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (max_q > max_kv) {
    std::snprintf(r.msg, sizeof(r.msg),
                  "max_q_len %lld exceeds max_kv_len %lld (every query's own key is a key)",
                  (long long)max_q, (long long)max_kv);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (B == 0 || H == 0 || max_q == 0) {
    r.empty = true;
    return r;
  }
  const void* ptrs[8] = {q_nope, q_pe, k_nope, k_pe, v, q_lens, past_lens, out};
  static const char* const names[8] = {"q_nope", "q_pe", "k_nope", "k_pe",
                                       "v", "q_lens", "past_lens", "out"};
  for (int i = 0; i < 8; ++i) {
    if (ptrs[i] == nullptr) {
      std::snprintf(r.msg, sizeof(r.msg), "%s is NULL", names[i]);
      r.status = MLA_ERR_NULL;
      return r;
    }
    const uintptr_t align = (i == 5 || i == 6) ? 4u : 16u;
    if ((reinterpret_cast<uintptr_t>(ptrs[i]) & (align - 1)) != 0) {
      std::snprintf(r.msg, sizeof(r.msg), "%s is not %u-byte aligned", names[i], (unsigned)align);
      r.status = MLA_ERR_ALIGN;
      return r;
    }
  }
  if (check_scale(scale, &r)) return r;
  if (max_kv > kMaxPrefillKeys) {
    std::snprintf(r.msg, sizeof(r.msg), "max_kv_len=%lld keys exceeds the prefill limit of %lld",
                  (long long)max_kv, (long long)kMaxPrefillKeys);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  const int64_t tiles = (max_q + block_m - 1) / block_m;
  if (B * H > kMaxGrid / tiles) {
    std::snprintf(r.msg, sizeof(r.msg), "B*H*ceil(max_q_len/%lld) = %lld*%lld exceeds the grid limit",
                  (long long)block_m, (long long)(B * H), (long long)tiles);
    r.status = MLA_ERR_SHAPE;
  }
  return r;
}

inline CheckResult check_decode(const void* q_nope, const void* q_pe, const void* k_nope,
                                const void* k_pe, const void* v, const void* out,
                                const void* workspace, size_t workspace_bytes, int64_t B,
                                int64_t H, int64_t S, int64_t past_len, float scale,
                                DecodePlan* plan_out) {
  CheckResult r = check_common(q_nope, q_pe, k_nope, k_pe, v, out, B, H, 1, S, past_len, scale);
  if (r.status != MLA_OK || r.empty) return r;
  const DecodePlan plan = plan_decode(B, H, S);
  if (B * H > kMaxGrid / plan.nsplit) {
    std::snprintf(r.msg, sizeof(r.msg), "B*H*nsplit exceeds the grid limit");
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (plan.workspace_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) {
      std::snprintf(r.msg, sizeof(r.msg), "workspace %s: %zu bytes given, %zu needed",
                    workspace == nullptr ? "is NULL" : "too small", workspace_bytes,
                    plan.workspace_bytes);
      r.status = MLA_ERR_WORKSPACE;
      return r;
    }
    if (misaligned(workspace)) {
      std::snprintf(r.msg, sizeof(r.msg), "workspace is not 16-byte aligned");
      r.status = MLA_ERR_ALIGN;
      return r;
    }
  }
  if (plan_out) *plan_out = plan;
  return r;
}

// ---- decode over a preallocated, right-padded cache with a length per sequence
inline CheckResult check_decode_varlen(const void* q_nope, const void* q_pe, const void* k_nope,
                                       const void* k_pe, const void* v, const void* seq_lens,
                                       const void* out, const void* workspace,
                                       size_t workspace_bytes, int64_t B, int64_t H, int64_t cap,
                                       int64_t max_len, float scale, DecodePlan* plan_out) {
  CheckResult r;
  if (B < 0 || H < 0 || cap < 0 || max_len < 0) {
    std::snprintf(r.msg, sizeof(r.msg),
                  "negative size: B=%lld H=%lld cache_len=%lld max_seq_len=%lld", (long long)B,
                  (long long)H, (long long)cap, (long long)max_len);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (max_len > cap) {
    std::snprintf(r.msg, sizeof(r.msg), "max_seq_len %lld exceeds the cache length %lld",
                  (long long)max_len, (long long)cap);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (B == 0 || H == 0) {
    r.empty = true;
    return r;
  }
  const void* ptrs[7] = {q_nope, q_pe, k_nope, k_pe, v, seq_lens, out};
  static const char* const names[7] = {"q_nope", "q_pe", "k_nope_cache", "k_pe_cache",
                                       "v_cache", "seq_lens", "out"};
  for (int i = 0; i < 7; ++i) {
    const bool cache = i >= 2 && i <= 4;
    if (ptrs[i] == nullptr && !(cache && cap == 0)) {
      std::snprintf(r.msg, sizeof(r.msg), "%s is NULL", names[i]);
      r.status = MLA_ERR_NULL;
      return r;
    }
    const uintptr_t align = i == 5 ? 4u : 16u;
    if ((reinterpret_cast<uintptr_t>(ptrs[i]) & (align - 1)) != 0) {
      std::snprintf(r.msg, sizeof(r.msg), "%s is not %u-byte aligned", names[i], (unsigned)align);
      r.status = MLA_ERR_ALIGN;
      return r;
    }
  }
  if (check_scale(scale, &r)) return r;
  const DecodePlan plan = plan_decode_varlen(B, H, max_len);
  if (B * H > kMaxGrid / plan.nsplit) {
    std::snprintf(r.msg, sizeof(r.msg), "B*H*nsplit exceeds the grid limit");
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (plan.workspace_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) {
      std::snprintf(r.msg, sizeof(r.msg), "workspace %s: %zu bytes given, %zu needed",
                    workspace == nullptr ? "is NULL" : "too small", workspace_bytes,
                    plan.workspace_bytes);
      r.status = MLA_ERR_WORKSPACE;
      return r;
    }
    if (misaligned(workspace)) {
      std::snprintf(r.msg, sizeof(r.msg), "workspace is not 16-byte aligned");
      r.status = MLA_ERR_ALIGN;
      return r;
    }
  }
  if (plan_out) *plan_out = plan;
  return r;
}

// ---- decode over a paged cache, optionally appending the new token
constexpr int64_t kPagedBlockMultiple = 32;  // a wave's 32 keys of one trip share a block

inline CheckResult check_decode_paged(const void* q_nope, const void* q_pe, const void* k_nope,
                                      const void* k_pe, const void* v, const void* block_table,
                                      const void* seq_lens, const void* kn_new,
                                      const void* kp_new, const void* v_new, const void* out,
                                      const void* workspace, size_t workspace_bytes, int64_t B,
                                      int64_t H, int64_t num_blocks, int64_t block_size,
                                      int64_t max_blocks, int64_t max_len, float scale,
                                      DecodePlan* plan_out) {
  CheckResult r;
  if (B < 0 || H < 0 || num_blocks < 0 || block_size < 0 || max_blocks < 0 || max_len < 0) {
    std::snprintf(r.msg, sizeof(r.msg),
                  "negative size: B=%lld H=%lld num_blocks=%lld block_size=%lld max_blocks=%lld "
                  "max_seq_len=%lld",
                  (long long)B, (long long)H, (long long)num_blocks, (long long)block_size,
                  (long long)max_blocks, (long long)max_len);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (B == 0 || H == 0) {
    r.empty = true;
    return r;
  }
  if (block_size == 0 || block_size % kPagedBlockMultiple != 0) {
    std::snprintf(r.msg, sizeof(r.msg), "block_size %lld must be a positive multiple of %lld",
                  (long long)block_size, (long long)kPagedBlockMultiple);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (num_blocks < 1 || max_len > max_blocks * block_size) {
    std::snprintf(r.msg, sizeof(r.msg),
                  "max_seq_len %lld needs max_blocks * block_size >= it and at least one block "
                  "(max_blocks=%lld, block_size=%lld, num_blocks=%lld)",
                  (long long)max_len, (long long)max_blocks, (long long)block_size,
                  (long long)num_blocks);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  const int nnew = (kn_new != nullptr) + (kp_new != nullptr) + (v_new != nullptr);
  if (nnew != 0 && nnew != 3) {
    std::snprintf(r.msg, sizeof(r.msg),
                  "append takes all of k_nope_new, k_pe_new and v_new, or none (%d given)", nnew);
    r.status = MLA_ERR_NULL;
    return r;
  }
  const void* ptrs[11] = {q_nope, q_pe, k_nope, k_pe, v, block_table, seq_lens, out,
                          kn_new, kp_new, v_new};
  static const char* const names[11] = {"q_nope", "q_pe", "k_nope_pages", "k_pe_pages",
                                        "v_pages", "block_table", "seq_lens", "out",
                                        "k_nope_new", "k_pe_new", "v_new"};
  for (int i = 0; i < 11; ++i) {
    if (ptrs[i] == nullptr && i < 8) {
      std::snprintf(r.msg, sizeof(r.msg), "%s is NULL", names[i]);
      r.status = MLA_ERR_NULL;
      return r;
    }
    const uintptr_t align = (i == 5 || i == 6) ? 4u : 16u;
    if ((reinterpret_cast<uintptr_t>(ptrs[i]) & (align - 1)) != 0) {
      std::snprintf(r.msg, sizeof(r.msg), "%s is not %u-byte aligned", names[i], (unsigned)align);
      r.status = MLA_ERR_ALIGN;
      return r;
    }
  }
  if (check_scale(scale, &r)) return r;
  const DecodePlan plan = plan_decode_varlen(B, H, max_len);
  if (B * H > kMaxGrid / plan.nsplit) {
    std::snprintf(r.msg, sizeof(r.msg), "B*H*nsplit exceeds the grid limit");
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (plan.workspace_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) {
      std::snprintf(r.msg, sizeof(r.msg), "workspace %s: %zu bytes given, %zu needed",
                    workspace == nullptr ? "is NULL" : "too small", workspace_bytes,
                    plan.workspace_bytes);
      r.status = MLA_ERR_WORKSPACE;
      return r;
    }
    if (misaligned(workspace)) {
      std::snprintf(r.msg, sizeof(r.msg), "workspace is not 16-byte aligned");
      r.status = MLA_ERR_ALIGN;
      return r;
    }
  }
  if (plan_out) *plan_out = plan;
  return r;
}

// ---- decode over the compressed latent cache
constexpr int64_t kLatentRank = 512;             // kv_lora_rank
constexpr int64_t kLatentKeyWidth = 512 + 64;    // latent + shared rotary key, per key
constexpr int64_t kLatentKeysPerTile = 32;
constexpr int64_t kLatentTargetWorkgroups = 256; // one per CU
// Sequences x key tiles above which every attention workgroup serves all
// heads (a tile copied once for 64 heads); up to it, with more than 48
// heads, a workgroup serves one group of 16 heads: four times the workgroups
// for the same splits, each with a quarter of the queries to load, the
// output to accumulate and the partial to store (the pages' decode over the
// latent cache, 32 tiles: 20.7 -> 17.9 us; two tiles per split instead, with
// the same 64 workgroups as before, 18.7 us; four, 21.0 us). Measured
// crossover: at 1024 sequences x tiles one head group is 0-5% faster, from
// 1280 on all heads are (13-25% at 1280-1536, 2x at 8192).
constexpr int64_t kLatentAllHeadsTiles = 4 * kLatentTargetWorkgroups;

struct LatentPlan {
  int64_t nsplit = 1;          // key splits per sequence
  int64_t keys_per_split = 0;  // multiple of kLatentKeysPerTile
  int64_t head_groups = 1;     // attention workgroups per (sequence, split): 1, or ceil(H / 16)
  size_t qt_bytes = 0;         // bf16 [B, H, 576]: absorbed queries joined with q_pe
  size_t po_bytes = 0;         // bf16 [B, nsplit, H, 512]: partial latent outputs
  size_t pml_bytes = 0;        // fp32 [B, nsplit, H, 2]: partial (max, sum)
  size_t workspace_bytes = 0;  // total, each region 256-byte aligned
};

// Split each sequence's keys so about one attention workgroup per CU runs,
// never more than one per CU (the attention kernel's LDS holds one): a grid
// just past 256 would run a second round for a few workgroups (12 sequences
// of 4096 keys: 264 workgroups 58.0 us, 228 workgroups 42.7 us).
inline LatentPlan plan_latent(int64_t B, int64_t H, int64_t S) {
  LatentPlan p;
  if (B <= 0 || H <= 0 || S <= 0) return p;
  const int64_t tiles = (S + kLatentKeysPerTile - 1) / kLatentKeysPerTile;
  const int64_t groups = (H + 15) / 16;
  int64_t nsplit;
  if (groups < 4 || B * tiles > kLatentAllHeadsTiles) {
    nsplit = kLatentTargetWorkgroups / B;  // one workgroup per CU: never a second round
  } else {
    p.head_groups = groups;
    nsplit = kLatentTargetWorkgroups / (B * groups);
  }
  if (nsplit > tiles) nsplit = tiles;
  if (nsplit < 1) nsplit = 1;
  int64_t kps = (S + nsplit - 1) / nsplit;
  kps = (kps + kLatentKeysPerTile - 1) / kLatentKeysPerTile * kLatentKeysPerTile;
  nsplit = (S + kps - 1) / kps;
  p.nsplit = nsplit;
  p.keys_per_split = kps;
  p.qt_bytes = align256(size_t(B) * size_t(H) * size_t(kLatentKeyWidth) * 2);
  p.po_bytes = align256(size_t(B) * size_t(nsplit) * size_t(H) * size_t(kLatentRank) * 2);
  p.pml_bytes = align256(size_t(B) * size_t(nsplit) * size_t(H) * 2 * 4);
  p.workspace_bytes = p.qt_bytes + p.po_bytes + p.pml_bytes;
  return p;
}

inline CheckResult check_latent_decode(const void* q_nope, const void* q_pe, const void* c_kv,
                                       const void* k_pe, const void* w_kv_b, const void* out,
                                       const void* workspace, size_t workspace_bytes, int64_t B,
                                       int64_t H, int64_t S, int64_t past_len, float scale,
                                       LatentPlan* plan_out) {
  static const char* const names[6] = {"q_nope", "q_pe", "c_kv", "k_pe", "w_kv_b", "out"};
  CheckResult r =
      check_common(q_nope, q_pe, c_kv, k_pe, w_kv_b, out, B, H, 1, S, past_len, scale, names);
  if (r.status != MLA_OK || r.empty) return r;
  if (S > kMaxLatentKeys) {
    std::snprintf(r.msg, sizeof(r.msg), "S=%lld keys exceeds the latent decode limit of %lld",
                  (long long)S, (long long)kMaxLatentKeys);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (H > 64) {
    std::snprintf(r.msg, sizeof(r.msg),
                  "latent decode takes at most 64 heads (one 64-column MFMA tile), got H=%lld",
                  (long long)H);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  const LatentPlan plan = plan_latent(B, H, S);
  if (B > kMaxGrid / (plan.nsplit * plan.head_groups) || B * H > kMaxGrid) {
    std::snprintf(r.msg, sizeof(r.msg), "B*nsplit exceeds the grid limit");
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) {
    std::snprintf(r.msg, sizeof(r.msg), "workspace %s: %zu bytes given, %zu needed",
                  workspace == nullptr ? "is NULL" : "too small", workspace_bytes,
                  plan.workspace_bytes);
    r.status = MLA_ERR_WORKSPACE;
    return r;
  }
  if (misaligned(workspace)) {
    std::snprintf(r.msg, sizeof(r.msg), "workspace is not 16-byte aligned");
    r.status = MLA_ERR_ALIGN;
    return r;
  }
  if (plan_out) *plan_out = plan;
  return r;
}

// Rotary prologue. The table holds cos and sin (fp32) of every pair at every
// position 0..max_pos-1: 32 pairs x 2 floats = 256 bytes per position.
constexpr int64_t kRopePairs = 32;
constexpr int64_t kRopeTableBytesPerPos = kRopePairs * 2 * 4;
constexpr int64_t kRopeMaxPositions = int64_t(1) << 24;  // positions exact in fp32 and fp64

inline size_t rope_table_bytes(int64_t max_pos) {
  return (max_pos <= 0 || max_pos > kRopeMaxPositions) ? 0 : size_t(max_pos) * kRopeTableBytesPerPos;
}

inline CheckResult check_rope_table(const void* table, int64_t max_pos, double theta, double factor,
                                    int64_t original_max_position, double beta_fast,
                                    double beta_slow) {
  CheckResult r;
  if (max_pos < 0 || max_pos > kRopeMaxPositions) {
    std::snprintf(r.msg, sizeof(r.msg), "max_pos %lld outside [0, %lld]", (long long)max_pos,
                  (long long)kRopeMaxPositions);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (original_max_position <= 0) {
    std::snprintf(r.msg, sizeof(r.msg), "original_max_position %lld must be positive",
                  (long long)original_max_position);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (!std::isfinite(theta) || !(theta > 1.0) || !std::isfinite(factor) || !(factor >= 1.0) ||
      !std::isfinite(beta_fast) || !std::isfinite(beta_slow)) {
    std::snprintf(r.msg, sizeof(r.msg),
                  "rope parameters out of range: theta %g (> 1), factor %g (>= 1), betas %g, %g "
                  "(finite)", theta, factor, beta_fast, beta_slow);
    r.status = MLA_ERR_SCALE;
    return r;
  }
  if (max_pos == 0) {
    r.empty = true;
    return r;
  }
  if (table == nullptr) return fail(MLA_ERR_NULL, "table is NULL");
  if (misaligned(table)) return fail(MLA_ERR_ALIGN, "table is not 16-byte aligned");
  return r;
}

// The rotary table a fused-prologue decode reads: present, 16-byte aligned,
// and holding every position up to need - 1, and at least one row (the
// kernel reads the row of position S - 1, or row 0 for an empty sequence).
inline CheckResult check_rope_decode_table(const void* table, int64_t max_pos, int64_t need) {
  if (table == nullptr) return fail(MLA_ERR_NULL, "rope_table is NULL");
  if (misaligned(table)) return fail(MLA_ERR_ALIGN, "rope_table is not 16-byte aligned");
  const int64_t rows = need > 1 ? need : 1;
  if (max_pos < rows || max_pos > kRopeMaxPositions) {
    CheckResult r;
    r.status = MLA_ERR_SHAPE;
    std::snprintf(r.msg, sizeof(r.msg),
                  "rope_max_pos %lld must cover positions 0..%lld (at least one row, at most %lld)",
                  (long long)max_pos, (long long)(rows - 1), (long long)kRopeMaxPositions);
    return r;
  }
  return CheckResult{};
}

// x: [B, R, T, 64] bf16, rotated in place; row t of sequence b at position
// past_len + t (past_lens NULL) or past_lens[b] + t.
inline CheckResult check_rope_apply(const void* x, const int32_t* past_lens, const void* table,
                                    int64_t max_pos, int64_t B, int64_t R, int64_t T,
                                    int64_t past_len) {
  CheckResult r;
  if (B < 0 || R < 0 || T < 0 || past_len < 0 || max_pos < 0) {
    std::snprintf(r.msg, sizeof(r.msg), "negative size: B=%lld R=%lld T=%lld past_len=%lld max_pos=%lld",
                  (long long)B, (long long)R, (long long)T, (long long)past_len, (long long)max_pos);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (max_pos > kRopeMaxPositions) {
    std::snprintf(r.msg, sizeof(r.msg), "max_pos %lld beyond %lld", (long long)max_pos,
                  (long long)kRopeMaxPositions);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (past_lens == nullptr && past_len + T > max_pos) {
    std::snprintf(r.msg, sizeof(r.msg), "positions up to past_len %lld + T %lld - 1 need a table of "
                  "at least %lld positions, not %lld", (long long)past_len, (long long)T,
                  (long long)(past_len + T), (long long)max_pos);
    r.status = MLA_ERR_SHAPE;
    return r;
  }
  if (B == 0 || R == 0 || T == 0) {
    r.empty = true;
    return r;
  }
  if (max_pos == 0) return fail(MLA_ERR_SHAPE, "an empty table cannot rotate any row");
  if (B * R * T > kMaxGrid) return fail(MLA_ERR_SHAPE, "B * R * T rows beyond the launch limit");
  if (x == nullptr) return fail(MLA_ERR_NULL, "x is NULL");
  if (table == nullptr) return fail(MLA_ERR_NULL, "table is NULL");
  if (misaligned(x)) return fail(MLA_ERR_ALIGN, "x is not 16-byte aligned");
  if (misaligned(table)) return fail(MLA_ERR_ALIGN, "table is not 16-byte aligned");
  if (past_lens != nullptr && (reinterpret_cast<uintptr_t>(past_lens) & 3u) != 0)
    return fail(MLA_ERR_ALIGN, "past_lens is not 4-byte aligned");
  return r;
}

}  // namespace mla

#endif  // MLA_HOST_CHECKS_H_
