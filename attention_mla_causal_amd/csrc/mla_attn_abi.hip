// C ABI of the MLA attention core: argument checks on the host, then one
// kernel launch on the caller's stream. See include/mla_attn.h for the
// contract of each entry point.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <atomic>
#include <cstring>
#include <mutex>

#include "../../include/mla_attn.h"
#include "mla_host_checks.h"
#include "mla_kernels.h"

namespace {

thread_local char g_last_error[320] = {0};

void set_error(const char* where, const char* msg) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, msg);
}

mla_status report(const char* where, const mla::CheckResult& r) {
  if (r.status != MLA_OK) set_error(where, r.msg);
  return r.status;
}

mla_status device_error(const char* where, hipError_t e) {
  char msg[256];
  std::snprintf(msg, sizeof(msg), "launch failed: %s", hipGetErrorString(e));
  set_error(where, msg);
  return MLA_ERR_DEVICE;
}

constexpr float kLog2e = 1.4426950408889634f;

// XCDs of the current device (hipDeviceAttributeNumberOfXccs), looked up once
// per device; -1 when the runtime cannot tell. The decode's in-kernel merge
// relies on workgroup w running on XCD w % 8, the dispatch order of an
// 8-XCD part; on any other count the combine kernel merges instead.
constexpr int kMaxDevices = 64;
int device_xcds() {
  static std::atomic<int> cache[kMaxDevices];  // 0: not looked up yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int x = 0;
    if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || x <= 0) x = -1;
    cache[dev].store(x, std::memory_order_relaxed);
    n = x;
  }
  return n;
}

// ---- allocation-free decode: its scratch lives in the library
//
// mla_attn_decode_noalloc keeps the split partials and completion flags of
// mla_attn_decode in this file-scope array instead of a caller's workspace.
// Each device that loads the library holds its own copy until the process
// ends. In host code `scratch` names a host-side stand-in, not device memory:
// its device address is looked up once per device (with that device current)
// by hipGetSymbolAddress and only that address is ever passed to a kernel.
// Every plan_decode workspace fits: B*H*nsplit stays below 768 when the keys
// are split (nsplit <= ceil(512 / (B*H)) for B*H < 256, no split above), i.e.
// at most 410,112 bytes.
constexpr size_t kScratchBytes = MLA_DECODE_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes >= 410112, "the largest plan_decode workspace must fit");
static __device__ __align__(256) char scratch[kScratchBytes];

// Device address of `scratch` on the current device, or nullptr (with the
// HIP error in *err) when it cannot be looked up.
void* scratch_on_current_device(hipError_t* err) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

namespace {

// Optional parts of a decode call: per-sequence lengths, a paged cache, an
// appended token.
struct DecodeExtras {
  const int32_t* seq_lens = nullptr;
  const int32_t* block_table = nullptr;
  int32_t max_blocks = 0, block_size = 0, num_blocks = 0;
  const void* kn_new = nullptr;
  const void* kp_new = nullptr;
  const void* v_new = nullptr;
  const uint8_t* key_mask = nullptr;  // [B, S] 2D padding mask
  const float* rope_table = nullptr;  // fused rotary prologue: (cos, sin) [>= S positions, 32]
};

// Every decode entry point: fill the arguments from a checked plan and launch.
mla_status launch_decode_call(const char* where, const void* q_nope, const void* q_pe,
                              const void* k_nope, const void* k_pe, const void* v,
                              const DecodeExtras& x, void* out, void* workspace,
                              const mla::DecodePlan& plan, int32_t B, int32_t H, int32_t S,
                              int32_t cap, float softmax_scale, void* stream) {
  mla::DecodeArgs a{};
  const int32_t* seq_lens = x.seq_lens;
  a.seq_lens = seq_lens;
  a.block_table = x.block_table;
  a.max_blocks = x.max_blocks;
  a.block_size = x.block_size;
  a.num_blocks = x.num_blocks;
  a.kn_new = static_cast<const uint16_t*>(x.kn_new);
  a.kp_new = static_cast<const uint16_t*>(x.kp_new);
  a.v_new = static_cast<const uint16_t*>(x.v_new);
  mla::DecodeKind kind = mla::kDecodePlain;
  if (x.key_mask != nullptr) {
    a.key_mask = x.key_mask;
    kind = mla::kDecodeMasked;
  } else if (x.rope_table != nullptr) {
    a.rope_table = x.rope_table;
    kind = mla::kDecodeRope;
  }
  a.cap = cap;
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.k_nope = static_cast<const uint16_t*>(k_nope);
  a.k_pe = static_cast<const uint16_t*>(k_pe);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  char* ws = static_cast<char*>(workspace);
  a.ws_o = plan.nsplit > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  a.ws_ml = plan.nsplit > 1 ? reinterpret_cast<float*>(ws + plan.ws_o_bytes) : nullptr;
  a.ws_flag = plan.nsplit > 1
                  ? reinterpret_cast<unsigned long long*>(ws + plan.ws_o_bytes + plan.ws_ml_bytes)
                  : nullptr;
  {
    // A fresh tag per call: completion flags left by earlier calls (or any
    // garbage in the workspace) hold another value and count as not done.
    static std::atomic<unsigned long long> next_tag{0x6d6c615f00000001ull};
    a.tag = next_tag.fetch_add(1);
  }
  {
    // The split kernel merges the partials itself when every split of a
    // (b, h) runs on one XCD (on an 8-XCD part workgroup w runs on XCD w % 8,
    // and the kernel hands each XCD whole (b, h) groups); otherwise, or on a
    // part with another XCD count, a second kernel merges.
    // With a length per sequence, (b, h) pairs are dealt round-robin over
    // the XCDs when B*H is a multiple of 8, which keeps each one's splits
    // together by construction.
    const int64_t bh = (int64_t)B * H;
    const int64_t grid = bh * plan.nsplit;
    a.interleave = ((seq_lens != nullptr || x.key_mask != nullptr) && bh % 8 == 0) ? 1 : 0;
    const bool together = a.interleave || (grid % 8 == 0 && (grid / 8) % plan.nsplit == 0);
    a.fused = (plan.nsplit > 1 && plan.nsplit <= 64 && together && device_xcds() == 8) ? 1 : 0;
  }
  a.B = B;
  a.H = H;
  a.S = S;
  a.nsplit = (int32_t)plan.nsplit;
  a.keys_per_split = (int32_t)plan.keys_per_split;
  a.scale_log2 = softmax_scale * kLog2e;
  const hipError_t e = mla::launch_decode(a, kind, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(where, e);
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status mla_attn_prefill(const void* q_nope, const void* q_pe, const void* k_nope,
                            const void* k_pe, const void* v, void* out, int32_t B, int32_t H,
                            int32_t T, int32_t S, int32_t past_len, float softmax_scale,
                            void* stream) {
  const mla::CheckResult r =
      mla::check_prefill(q_nope, q_pe, k_nope, k_pe, v, out, B, H, T, S, past_len, softmax_scale,
                         mla::prefill_block_m());
  if (r.status != MLA_OK) return report("mla_attn_prefill", r);
  if (r.empty) return MLA_OK;
  mla::PrefillArgs a{};  // nsplit 0: one workgroup per query tile covers all its keys
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.k_nope = static_cast<const uint16_t*>(k_nope);
  a.k_pe = static_cast<const uint16_t*>(k_pe);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.B = B;
  a.H = H;
  a.T = T;
  a.S = S;
  a.past_len = past_len;
  a.ntiles = (int32_t)((T + mla::prefill_block_m() - 1) / mla::prefill_block_m());
  a.scale_log2 = softmax_scale * kLog2e;
  const hipError_t e = mla::launch_prefill(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error("mla_attn_prefill", e);
  return MLA_OK;
}

size_t mla_attn_prefill_workspace_bytes(int32_t B, int32_t H, int32_t T, int32_t S) {
  return mla::plan_prefill(B, H, T, S, mla::prefill_block_m(), mla::kPrefillKeyTile)
      .workspace_bytes;
}

mla_status mla_attn_prefill_ws(const void* q_nope, const void* q_pe, const void* k_nope,
                               const void* k_pe, const void* v, void* out, void* workspace,
                               size_t workspace_bytes, int32_t B, int32_t H, int32_t T, int32_t S,
                               int32_t past_len, float softmax_scale, void* stream) {
  mla::PrefillPlan plan;
  const mla::CheckResult r = mla::check_prefill_ws(
      q_nope, q_pe, k_nope, k_pe, v, out, workspace, workspace_bytes, B, H, T, S, past_len,
      softmax_scale, mla::prefill_block_m(), mla::kPrefillKeyTile, &plan);
  if (r.status != MLA_OK) return report("mla_attn_prefill_ws", r);
  if (r.empty) return MLA_OK;
  mla::PrefillArgs a{};
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.k_nope = static_cast<const uint16_t*>(k_nope);
  a.k_pe = static_cast<const uint16_t*>(k_pe);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.B = B;
  a.H = H;
  a.T = T;
  a.S = S;
  a.past_len = past_len;
  a.ntiles = (int32_t)((T + mla::prefill_block_m() - 1) / mla::prefill_block_m());
  a.scale_log2 = softmax_scale * kLog2e;
  a.nsplit = (int32_t)plan.nsplit;
  if (plan.nsplit > 1) {
    char* ws = static_cast<char*>(workspace);
    a.ws_o = reinterpret_cast<float*>(ws);
    a.ws_ml = reinterpret_cast<float*>(ws + plan.ws_o_bytes);
  }
  const hipError_t e = mla::launch_prefill(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error("mla_attn_prefill_ws", e);
  return MLA_OK;
}

mla_status mla_attn_prefill_varlen(const void* q_nope, const void* q_pe, const void* k_nope,
                                   const void* k_pe, const void* v, const int32_t* q_lens,
                                   const int32_t* past_lens, void* out, int32_t B, int32_t H,
                                   int32_t max_q_len, int32_t max_kv_len, float softmax_scale,
                                   void* stream) {
  const mla::CheckResult r = mla::check_prefill_varlen(
      q_nope, q_pe, k_nope, k_pe, v, q_lens, past_lens, out, B, H, max_q_len, max_kv_len,
      softmax_scale, mla::prefill_block_m());
  if (r.status != MLA_OK) return report("mla_attn_prefill_varlen", r);
  if (r.empty) return MLA_OK;
  mla::PrefillArgs a{};
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.k_nope = static_cast<const uint16_t*>(k_nope);
  a.k_pe = static_cast<const uint16_t*>(k_pe);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.q_lens = q_lens;
  a.past_lens = past_lens;
  a.B = B;
  a.H = H;
  a.T = max_q_len;
  a.S = max_kv_len;
  a.past_len = 0;  // the lengths stay on the device
  a.ntiles = (int32_t)((max_q_len + mla::prefill_block_m() - 1) / mla::prefill_block_m());
  a.scale_log2 = softmax_scale * kLog2e;
  const hipError_t e = mla::launch_prefill(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error("mla_attn_prefill_varlen", e);
  return MLA_OK;
}

mla_status mla_attn_prefill_masked(const void* q_nope, const void* q_pe, const void* k_nope,
                                   const void* k_pe, const void* v, const uint8_t* attn_mask,
                                   void* out, int32_t B, int32_t H, int32_t T, int32_t S,
                                   int32_t past_len, float softmax_scale, void* stream) {
  mla::CheckResult r = mla::check_prefill(q_nope, q_pe, k_nope, k_pe, v, out, B, H, T, S, past_len,
                                          softmax_scale, mla::prefill_block_m());
  if (r.status == MLA_OK && !r.empty && attn_mask == nullptr)
    r = mla::fail(MLA_ERR_NULL, "attn_mask is NULL");
  if (r.status != MLA_OK) return report("mla_attn_prefill_masked", r);
  if (r.empty) return MLA_OK;
  mla::PrefillArgs a{};  // one workgroup per query tile covers all its keys
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.k_nope = static_cast<const uint16_t*>(k_nope);
  a.k_pe = static_cast<const uint16_t*>(k_pe);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.key_mask = attn_mask;
  a.B = B;
  a.H = H;
  a.T = T;
  a.S = S;
  a.past_len = past_len;
  a.ntiles = (int32_t)((T + mla::prefill_block_m() - 1) / mla::prefill_block_m());
  a.scale_log2 = softmax_scale * kLog2e;
  const hipError_t e = mla::launch_prefill(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error("mla_attn_prefill_masked", e);
  return MLA_OK;
}

size_t mla_attn_decode_workspace_bytes(int32_t B, int32_t H, int32_t S) {
  return mla::plan_decode(B, H, S).workspace_bytes;
}

mla_status mla_attn_decode(const void* q_nope, const void* q_pe, const void* k_nope,
                           const void* k_pe, const void* v, void* out, void* workspace,
                           size_t workspace_bytes, int32_t B, int32_t H, int32_t S,
                           int32_t past_len, float softmax_scale, void* stream) {
  mla::DecodePlan plan;
  const mla::CheckResult r = mla::check_decode(q_nope, q_pe, k_nope, k_pe, v, out, workspace,
                                               workspace_bytes, B, H, S, past_len,
                                               softmax_scale, &plan);
  if (r.status != MLA_OK) return report("mla_attn_decode", r);
  if (r.empty) return MLA_OK;
  return launch_decode_call("mla_attn_decode", q_nope, q_pe, k_nope, k_pe, v, DecodeExtras{},
                            out, workspace, plan, B, H, S, S, softmax_scale, stream);
}

mla_status mla_attn_decode_noalloc(const void* q_nope, const void* q_pe, const void* k_nope,
                                   const void* k_pe, const void* v, void* out, int32_t B, int32_t H,
                                   int32_t S, int32_t past_len, float softmax_scale, void* stream) {
  const char* where = "mla_attn_decode_noalloc";
  mla::DecodePlan plan;
  // Every check runs before any HIP call, the scratch's device address
  // included: the checks see a stand-in workspace of the scratch's size (a
  // non-null, aligned value that is never dereferenced), so a plan larger
  // than the scratch is MLA_ERR_WORKSPACE.
  void* const stand_in = reinterpret_cast<void*>(uintptr_t(1) << 20);
  const mla::CheckResult r = mla::check_decode(q_nope, q_pe, k_nope, k_pe, v, out, stand_in, kScratchBytes,
                                               B, H, S, past_len, softmax_scale, &plan);
  if (r.status != MLA_OK) {
    if (r.status == MLA_ERR_WORKSPACE) {
      char msg[200];
      std::snprintf(msg, sizeof(msg), "needs %zu bytes of scratch, more than the library's %zu",
                    mla::plan_decode(B, H, S).workspace_bytes, kScratchBytes);
      set_error(where, msg);
      return MLA_ERR_WORKSPACE;
    }
    return report(where, r);
  }
  if (r.empty) return MLA_OK;
  void* ws = nullptr;
  if (plan.workspace_bytes > 0) {
    hipError_t e = hipSuccess;
    ws = scratch_on_current_device(&e);
    if (ws == nullptr) return device_error(where, e);
  }
  return launch_decode_call(where, q_nope, q_pe, k_nope, k_pe, v, DecodeExtras{}, out, ws, plan, B, H, S, S,
                            softmax_scale, stream);
}

mla_status mla_attn_decode_rope(const void* q_nope, const void* q_pe, const void* k_nope,
                                const void* k_pe, const void* v, const void* rope_table,
                                int32_t rope_max_pos, void* out, void* workspace,
                                size_t workspace_bytes, int32_t B, int32_t H, int32_t S,
                                int32_t past_len, float softmax_scale, void* stream) {
  mla::DecodePlan plan;
  mla::CheckResult r = mla::check_decode(q_nope, q_pe, k_nope, k_pe, v, out, workspace,
                                         workspace_bytes, B, H, S, past_len, softmax_scale, &plan);
  if (r.status == MLA_OK && !r.empty)
    r = mla::check_rope_decode_table(rope_table, rope_max_pos, (int64_t)past_len + 1);
  if (r.status != MLA_OK) return report("mla_attn_decode_rope", r);
  if (r.empty) return MLA_OK;
  DecodeExtras x;
  x.rope_table = static_cast<const float*>(rope_table);
  return launch_decode_call("mla_attn_decode_rope", q_nope, q_pe, k_nope, k_pe, v, x, out,
                            workspace, plan, B, H, S, S, softmax_scale, stream);
}

mla_status mla_attn_decode_masked(const void* q_nope, const void* q_pe, const void* k_nope,
                                  const void* k_pe, const void* v, const uint8_t* attn_mask,
                                  void* out, void* workspace, size_t workspace_bytes, int32_t B,
                                  int32_t H, int32_t S, int32_t past_len, float softmax_scale,
                                  void* stream) {
  // Padding differs by sequence, as lengths do: the variable-length plan
  // (pieces of at most 1024 keys) keeps long-visible sequences from trailing.
  mla::DecodePlan plan;
  mla::CheckResult r = mla::check_decode(q_nope, q_pe, k_nope, k_pe, v, out, workspace,
                                         workspace_bytes, B, H, S, past_len, softmax_scale, nullptr);
  if (r.status == MLA_OK && !r.empty) {
    plan = mla::plan_decode_varlen(B, H, S);
    if (attn_mask == nullptr) {
      r = mla::fail(MLA_ERR_NULL, "attn_mask is NULL");
    } else if (B * (int64_t)H > mla::kMaxGrid / plan.nsplit) {
      r = mla::fail(MLA_ERR_SHAPE, "B*H*nsplit exceeds the grid limit");
    } else if (plan.workspace_bytes > 0 &&
               (workspace == nullptr || workspace_bytes < plan.workspace_bytes)) {
      r = mla::fail(MLA_ERR_WORKSPACE,
                    "workspace is NULL or smaller than mla_attn_decode_varlen_workspace_bytes(B, H, S)");
    } else if (plan.workspace_bytes > 0 && mla::misaligned(workspace)) {
      r = mla::fail(MLA_ERR_ALIGN, "workspace is not 16-byte aligned");
    }
  }
  if (r.status != MLA_OK) return report("mla_attn_decode_masked", r);
  if (r.empty) return MLA_OK;
  DecodeExtras x;
  x.key_mask = attn_mask;
  return launch_decode_call("mla_attn_decode_masked", q_nope, q_pe, k_nope, k_pe, v, x, out,
                            workspace, plan, B, H, S, S, softmax_scale, stream);
}

size_t mla_attn_decode_varlen_workspace_bytes(int32_t B, int32_t H, int32_t max_seq_len) {
  return mla::plan_decode_varlen(B, H, max_seq_len).workspace_bytes;
}

mla_status mla_attn_decode_varlen(const void* q_nope, const void* q_pe, const void* k_nope_cache,
                                  const void* k_pe_cache, const void* v_cache,
                                  const int32_t* seq_lens, void* out, void* workspace,
                                  size_t workspace_bytes, int32_t B, int32_t H,
                                  int32_t cache_len, int32_t max_seq_len, float softmax_scale,
                                  void* stream) {
  mla::DecodePlan plan;
  const mla::CheckResult r = mla::check_decode_varlen(
      q_nope, q_pe, k_nope_cache, k_pe_cache, v_cache, seq_lens, out, workspace, workspace_bytes,
      B, H, cache_len, max_seq_len, softmax_scale, &plan);
  if (r.status != MLA_OK) return report("mla_attn_decode_varlen", r);
  if (r.empty) return MLA_OK;
  DecodeExtras x;
  x.seq_lens = seq_lens;
  return launch_decode_call("mla_attn_decode_varlen", q_nope, q_pe, k_nope_cache, k_pe_cache,
                            v_cache, x, out, workspace, plan, B, H, max_seq_len, cache_len,
                            softmax_scale, stream);
}

mla_status mla_attn_decode_varlen_rope(const void* q_nope, const void* q_pe,
                                       const void* k_nope_cache, const void* k_pe_cache,
                                       const void* v_cache, const int32_t* seq_lens,
                                       const void* rope_table, int32_t rope_max_pos, void* out,
                                       void* workspace, size_t workspace_bytes, int32_t B,
                                       int32_t H, int32_t cache_len, int32_t max_seq_len,
                                       float softmax_scale, void* stream) {
  mla::DecodePlan plan;
  mla::CheckResult r = mla::check_decode_varlen(
      q_nope, q_pe, k_nope_cache, k_pe_cache, v_cache, seq_lens, out, workspace, workspace_bytes,
      B, H, cache_len, max_seq_len, softmax_scale, &plan);
  if (r.status == MLA_OK && !r.empty)
    r = mla::check_rope_decode_table(rope_table, rope_max_pos, max_seq_len);
  if (r.status != MLA_OK) return report("mla_attn_decode_varlen_rope", r);
  if (r.empty) return MLA_OK;
  DecodeExtras x;
  x.seq_lens = seq_lens;
  x.rope_table = static_cast<const float*>(rope_table);
  return launch_decode_call("mla_attn_decode_varlen_rope", q_nope, q_pe, k_nope_cache, k_pe_cache,
                            v_cache, x, out, workspace, plan, B, H, max_seq_len, cache_len,
                            softmax_scale, stream);
}

size_t mla_attn_decode_paged_workspace_bytes(int32_t B, int32_t H, int32_t max_seq_len) {
  return mla::plan_decode_varlen(B, H, max_seq_len).workspace_bytes;
}

}  // extern "C"

namespace {

mla_status decode_paged_call(const char* where, const void* q_nope, const void* q_pe,
                             void* k_nope_pages, void* k_pe_pages, void* v_pages,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const void* k_nope_new, const void* k_pe_new, const void* v_new,
                             bool rope, const void* rope_table, int32_t rope_max_pos, void* out,
                             void* workspace, size_t workspace_bytes, int32_t B, int32_t H,
                             int32_t num_blocks, int32_t block_size, int32_t max_blocks,
                             int32_t max_seq_len, float softmax_scale, void* stream) {
  mla::DecodePlan plan;
  mla::CheckResult r = mla::check_decode_paged(
      q_nope, q_pe, k_nope_pages, k_pe_pages, v_pages, block_table, seq_lens, k_nope_new,
      k_pe_new, v_new, out, workspace, workspace_bytes, B, H, num_blocks, block_size, max_blocks,
      max_seq_len, softmax_scale, &plan);
  if (r.status == MLA_OK && !r.empty && rope)
    r = mla::check_rope_decode_table(rope_table, rope_max_pos, max_seq_len);
  if (r.status != MLA_OK) return report(where, r);
  if (r.empty) return MLA_OK;
  DecodeExtras x;
  x.rope_table = rope ? static_cast<const float*>(rope_table) : nullptr;
  x.seq_lens = seq_lens;
  x.block_table = block_table;
  x.max_blocks = max_blocks;
  x.block_size = block_size;
  x.num_blocks = num_blocks;
  x.kn_new = k_nope_new;
  x.kp_new = k_pe_new;
  x.v_new = v_new;
  return launch_decode_call(where, q_nope, q_pe, k_nope_pages, k_pe_pages, v_pages, x, out,
                            workspace, plan, B, H, max_seq_len, 0, softmax_scale, stream);
}

}  // namespace

extern "C" {

mla_status mla_attn_decode_paged(const void* q_nope, const void* q_pe, void* k_nope_pages,
                                 void* k_pe_pages, void* v_pages, const int32_t* block_table,
                                 const int32_t* seq_lens, const void* k_nope_new,
                                 const void* k_pe_new, const void* v_new, void* out,
                                 void* workspace, size_t workspace_bytes, int32_t B, int32_t H,
                                 int32_t num_blocks, int32_t block_size, int32_t max_blocks,
                                 int32_t max_seq_len, float softmax_scale, void* stream) {
  return decode_paged_call("mla_attn_decode_paged", q_nope, q_pe, k_nope_pages, k_pe_pages,
                           v_pages, block_table, seq_lens, k_nope_new, k_pe_new, v_new, false,
                           nullptr, 0, out, workspace, workspace_bytes, B, H, num_blocks, block_size,
                           max_blocks, max_seq_len, softmax_scale, stream);
}

mla_status mla_attn_decode_paged_rope(const void* q_nope, const void* q_pe, void* k_nope_pages,
                                      void* k_pe_pages, void* v_pages, const int32_t* block_table,
                                      const int32_t* seq_lens, const void* k_nope_new,
                                      const void* k_pe_new, const void* v_new,
                                      const void* rope_table, int32_t rope_max_pos, void* out,
                                      void* workspace, size_t workspace_bytes, int32_t B,
                                      int32_t H, int32_t num_blocks, int32_t block_size,
                                      int32_t max_blocks, int32_t max_seq_len,
                                      float softmax_scale, void* stream) {
  return decode_paged_call("mla_attn_decode_paged_rope", q_nope, q_pe, k_nope_pages, k_pe_pages,
                           v_pages, block_table, seq_lens, k_nope_new, k_pe_new, v_new, true, rope_table,
                           rope_max_pos, out, workspace, workspace_bytes, B, H, num_blocks,
                           block_size, max_blocks, max_seq_len, softmax_scale, stream);
}

size_t mla_attn_decode_latent_workspace_bytes(int32_t B, int32_t H, int32_t S) {
  return mla::plan_latent(B, H, S).workspace_bytes;
}

mla_status mla_attn_decode_latent(const void* q_nope, const void* q_pe, const void* c_kv,
                                  const void* k_pe, const void* w_kv_b, void* out,
                                  void* workspace, size_t workspace_bytes, int32_t B, int32_t H,
                                  int32_t S, int32_t past_len, float softmax_scale, void* stream) {
  mla::LatentPlan plan;
  const mla::CheckResult r =
      mla::check_latent_decode(q_nope, q_pe, c_kv, k_pe, w_kv_b, out, workspace, workspace_bytes,
                               B, H, S, past_len, softmax_scale, &plan);
  if (r.status != MLA_OK) return report("mla_attn_decode_latent", r);
  if (r.empty) return MLA_OK;
  mla::LatentArgs a;
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.c_kv = static_cast<const uint16_t*>(c_kv);
  a.k_pe = static_cast<const uint16_t*>(k_pe);
  a.w_kv_b = static_cast<const uint16_t*>(w_kv_b);
  a.out = static_cast<uint16_t*>(out);
  char* ws = static_cast<char*>(workspace);
  a.qt = reinterpret_cast<uint16_t*>(ws);
  a.po = reinterpret_cast<uint16_t*>(ws + plan.qt_bytes);
  a.pml = reinterpret_cast<float*>(ws + plan.qt_bytes + plan.po_bytes);
  a.B = B;
  a.H = H;
  a.S = S;
  a.nsplit = (int32_t)plan.nsplit;
  a.keys_per_split = (int32_t)plan.keys_per_split;
  a.head_groups = (int32_t)plan.head_groups;
  a.scale_log2 = softmax_scale * kLog2e;
  const hipError_t e = mla::launch_latent_decode(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error("mla_attn_decode_latent", e);
  return MLA_OK;
}

size_t mla_rope_table_bytes(int32_t max_pos) { return mla::rope_table_bytes(max_pos); }

mla_status mla_rope_table(void* table, int32_t max_pos, double theta, double factor,
                          int32_t original_max_position, double beta_fast, double beta_slow,
                          void* stream) {
  const mla::CheckResult r = mla::check_rope_table(table, max_pos, theta, factor,
                                                   original_max_position, beta_fast, beta_slow);
  if (r.status != MLA_OK) return report("mla_rope_table", r);
  if (r.empty) return MLA_OK;
  mla::RopeTableArgs a;
  a.table = static_cast<float*>(table);
  a.max_pos = max_pos;
  a.original_max_position = original_max_position;
  a.theta = theta;
  a.factor = factor;
  a.beta_fast = beta_fast;
  a.beta_slow = beta_slow;
  const hipError_t e = mla::launch_rope_table(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error("mla_rope_table", e);
  return MLA_OK;
}

mla_status mla_rope_apply(void* x, const int32_t* past_lens, const void* table, int32_t max_pos,
                          int32_t B, int32_t R, int32_t T, int32_t past_len, void* stream) {
  const mla::CheckResult r =
      mla::check_rope_apply(x, past_lens, table, max_pos, B, R, T, past_len);
  if (r.status != MLA_OK) return report("mla_rope_apply", r);
  if (r.empty) return MLA_OK;
  mla::RopeApplyArgs a;
  a.x = static_cast<uint16_t*>(x);
  a.x2 = nullptr;
  a.table = static_cast<const float*>(table);
  a.past_lens = past_lens;
  a.rows = (int64_t)B * R * T;
  a.rows1 = a.rows;
  a.R = R;
  a.T = T;
  a.past_len = past_len;
  a.max_pos = max_pos;
  const hipError_t e = mla::launch_rope_apply(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error("mla_rope_apply", e);
  return MLA_OK;
}

mla_status mla_rope_apply_qk(void* q_pe, void* k_pe, const int32_t* past_lens, const void* table,
                             int32_t max_pos, int32_t B, int32_t H, int32_t T, int32_t past_len,
                             void* stream) {
  // the limits of one tensor of B * (H + 1) * T rows; then the key rows' own pointer
  // (with H == 0 the query has no rows and may be NULL)
  mla::CheckResult r = mla::check_rope_apply(H > 0 ? q_pe : k_pe, past_lens, table, max_pos, B,
                                             (int64_t)H + 1, T, past_len);
  if (r.status == MLA_OK && !r.empty) {
    if (k_pe == nullptr) r = mla::fail(MLA_ERR_NULL, "k_pe is NULL");
    else if (mla::misaligned(k_pe)) r = mla::fail(MLA_ERR_ALIGN, "k_pe is not 16-byte aligned");
  }
  if (r.status != MLA_OK) return report("mla_rope_apply_qk", r);
  if (r.empty) return MLA_OK;
  mla::RopeApplyArgs a;
  a.x = static_cast<uint16_t*>(q_pe);
  a.x2 = static_cast<uint16_t*>(k_pe);
  a.table = static_cast<const float*>(table);
  a.past_lens = past_lens;
  a.rows1 = (int64_t)B * H * T;
  a.rows = a.rows1 + (int64_t)B * T;
  a.R = H;
  a.T = T;
  a.past_len = past_len;
  a.max_pos = max_pos;
  const hipError_t e = mla::launch_rope_apply(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error("mla_rope_apply_qk", e);
  return MLA_OK;
}

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN";
    case MLA_ERR_SCALE: return "MLA_ERR_SCALE";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_DEVICE: return "MLA_ERR_DEVICE";
  }
  return "unknown status";
}

const char* mla_last_error(void) { return g_last_error; }

}  // extern "C"
