// C-ABI entry points: argument checks on the host, then the gfx950 launchers.
// Nothing here allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "../../include/dakv.h"
#include "launch.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int from_hip(hipError_t e) {
  if (e == hipErrorNotSupported) return DAKV_ENOTSUP;
  return e == hipSuccess ? DAKV_OK : DAKV_EHIP;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* dakv_strerror(int code) {
  switch (code) {
    case DAKV_OK: return "ok";
    case DAKV_EINVAL: return "invalid argument (null pointer, size, alignment or workspace)";
    case DAKV_ENOTSUP: return "unsupported shape (no kernel built for it)";
    case DAKV_ERANGE: return "index content outside the contract";
    case DAKV_EHIP: return "HIP runtime error at launch";
    case DAKV_ESCRATCH:
      return "the call needs more split-partial memory than the library's fixed scratch holds";
    default: return "unknown status";
  }
}

// ------------------------------------------------------------------ kv_append
int dakv_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                   const int32_t* write_pos, int32_t* mask, int B, int H, int cap, int D,
                   int32_t* err_flag, void* stream) {
  if (B < 0 || H < 0 || cap < 0 || D <= 0) return DAKV_EINVAL;
  if (B == 0 || H == 0) return DAKV_OK;
  if (cap == 0) return DAKV_EINVAL;
  if (!k_cache || !v_cache || !k_new || !v_new || !write_pos) return DAKV_EINVAL;
  if ((D * 2) % 16 != 0) return DAKV_ENOTSUP;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return DAKV_EINVAL;
  return from_hip(dakv::launch_kv_append(k_cache, v_cache, k_new, v_new, write_pos, mask, B, H,
                                         cap, D, err_flag, as_stream(stream)));
}

// ------------------------------------------------------------------- fp8 cache
int dakv_kv_append_fp8(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                       const void* k_new, const void* v_new, const int32_t* write_pos,
                       int32_t* mask, int B, int H, int cap, int D, int32_t* err_flag,
                       void* stream) {
  if (B < 0 || H < 0 || cap <= 0 || D <= 0) return DAKV_EINVAL;
  if (B == 0 || H == 0) return DAKV_OK;
  if (D % 16 != 0 || D > 256) return DAKV_ENOTSUP;
  if (!k_codes || !v_codes || !k_scale || !v_scale || !k_new || !v_new || !write_pos)
    return DAKV_EINVAL;
  return from_hip(dakv::launch_kv_append_fp8(k_codes, v_codes, k_scale, v_scale, k_new, v_new,
                                             write_pos, mask, B, H, cap, D, err_flag,
                                             as_stream(stream)));
}

// -------------------------------------------------------------- FP4 KV cache
int dakv_kv_append_fp4(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                       const void* k_new, const void* v_new, const int32_t* write_pos,
                       int32_t* mask, int B, int H, int cap, int D, int32_t* err_flag,
                       void* stream) {
  if (B < 0 || H < 0 || cap <= 0 || D <= 0) return DAKV_EINVAL;
  if (B == 0 || H == 0) return DAKV_OK;
  if (D % 16 != 0 || D > 256) return DAKV_ENOTSUP;
  if (!k_codes || !v_codes || !k_scale || !v_scale || !k_new || !v_new || !write_pos)
    return DAKV_EINVAL;
  return from_hip(dakv::launch_kv_append_fp4(k_codes, v_codes, k_scale, v_scale, k_new, v_new,
                                             write_pos, mask, B, H, cap, D, err_flag,
                                             as_stream(stream)));
}

int dakv_decode_attn_static_fp4(const float* q, const void* k_codes, const void* v_codes,
                                const float* k_scale, const float* v_scale, const int32_t* mask,
                                const int32_t* valid_len, int B, int H, int cap, int D,
                                float scale, float* out, float* lse, void* workspace,
                                size_t workspace_bytes, int num_splits, int32_t* err_flag,
                                void* stream) {
  if (B < 0 || H < 0 || cap <= 0 || D <= 0 || num_splits < 0) return DAKV_EINVAL;
  if (B == 0 || H == 0) return DAKV_OK;
  if (D != 64 && D != 128) return DAKV_ENOTSUP;
  if (!dakv::static_supported(cap)) return DAKV_ENOTSUP;
  if (!q || !k_codes || !v_codes || !k_scale || !v_scale || !out || !workspace)
    return DAKV_EINVAL;
  if (!mask && !valid_len) return DAKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(out) ||
      !aligned16(workspace))
    return DAKV_EINVAL;
  if (workspace_bytes < dakv::static_workspace_bytes(B, H, cap, D)) return DAKV_EINVAL;
  const dakv::SplitPlan plan = dakv::plan_static(B, H, cap, D, num_splits);
  return from_hip(dakv::launch_decode_static_fp4(q, k_codes, v_codes, k_scale, v_scale, mask,
                                                 valid_len, B, H, cap, D, scale, out, lse,
                                                 workspace, plan, err_flag, as_stream(stream)));
}

size_t dakv_decode_attn_static_fp8_workspace_size(int B, int H, int cap, int D) {
  return dakv_decode_attn_static_workspace_size(B, H, cap, D);
}

int dakv_decode_attn_static_fp8(const float* q, const void* k_codes, const void* v_codes,
                                const float* k_scale, const float* v_scale, const int32_t* mask,
                                const int32_t* valid_len, int B, int H, int cap, int D,
                                float scale, float* out, float* lse, void* workspace,
                                size_t workspace_bytes, int num_splits, int32_t* err_flag,
                                void* stream) {
  if (B < 0 || H < 0 || cap <= 0 || D <= 0 || num_splits < 0) return DAKV_EINVAL;
  if (B == 0 || H == 0) return DAKV_OK;
  if (D != 64 && D != 128) return DAKV_ENOTSUP;
  if (!dakv::static_supported(cap)) return DAKV_ENOTSUP;
  if (!q || !k_codes || !v_codes || !k_scale || !v_scale || !out || !workspace)
    return DAKV_EINVAL;
  if (!mask && !valid_len) return DAKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(out) ||
      !aligned16(workspace))
    return DAKV_EINVAL;
  if (workspace_bytes < dakv::static_workspace_bytes(B, H, cap, D)) return DAKV_EINVAL;
  const dakv::SplitPlan plan = dakv::plan_static(B, H, cap, D, num_splits);
  return from_hip(dakv::launch_decode_static_fp8(
      q, const_cast<void*>(k_codes), const_cast<void*>(v_codes), const_cast<float*>(k_scale),
      const_cast<float*>(v_scale), const_cast<int32_t*>(mask), valid_len, nullptr, nullptr,
      nullptr, B, H, cap, D, scale, out, lse, workspace, plan, err_flag, as_stream(stream)));
}

int dakv_decode_step_static_fp8(const float* q, void* k_codes, void* v_codes, float* k_scale,
                                float* v_scale, const void* k_new, const void* v_new,
                                const int32_t* write_pos, int32_t* mask, const int32_t* valid_len,
                                int B, int H, int cap, int D, float scale, float* out, float* lse,
                                void* workspace, size_t workspace_bytes, int num_splits,
                                int32_t* err_flag, void* stream) {
  if (B < 0 || H < 0 || cap <= 0 || D <= 0 || num_splits < 0) return DAKV_EINVAL;
  if (B == 0 || H == 0) return DAKV_OK;
  if (D != 64 && D != 128) return DAKV_ENOTSUP;
  if (!dakv::static_supported(cap)) return DAKV_ENOTSUP;
  if (!q || !k_codes || !v_codes || !k_scale || !v_scale || !k_new || !v_new || !write_pos ||
      !out || !workspace)
    return DAKV_EINVAL;
  if (!mask && !valid_len) return DAKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_new) ||
      !aligned16(v_new) || !aligned16(out) || !aligned16(workspace))
    return DAKV_EINVAL;
  if (workspace_bytes < dakv::static_workspace_bytes(B, H, cap, D)) return DAKV_EINVAL;
  const dakv::SplitPlan plan = dakv::plan_static(B, H, cap, D, num_splits);
  return from_hip(dakv::launch_decode_static_fp8(q, k_codes, v_codes, k_scale, v_scale, mask,
                                                 valid_len, k_new, v_new, write_pos, B, H, cap, D,
                                                 scale, out, lse, workspace, plan, err_flag,
                                                 as_stream(stream)));
}

int dakv_decode_step_static_fp4(const float* q, void* k_codes, void* v_codes, float* k_scale,
                                float* v_scale, const void* k_new, const void* v_new,
                                const int32_t* write_pos, int32_t* mask, const int32_t* valid_len,
                                int B, int H, int cap, int D, float scale, float* out, float* lse,
                                void* workspace, size_t workspace_bytes, int num_splits,
                                int32_t* err_flag, void* stream) {
  if (B < 0 || H < 0 || cap <= 0 || D <= 0 || num_splits < 0) return DAKV_EINVAL;
  if (B == 0 || H == 0) return DAKV_OK;
  if (D != 64 && D != 128) return DAKV_ENOTSUP;
  if (!dakv::static_supported(cap)) return DAKV_ENOTSUP;
  if (!q || !k_codes || !v_codes || !k_scale || !v_scale || !k_new || !v_new || !write_pos ||
      !out || !workspace)
    return DAKV_EINVAL;
  if (!mask && !valid_len) return DAKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_new) ||
      !aligned16(v_new) || !aligned16(out) || !aligned16(workspace))
    return DAKV_EINVAL;
  if (workspace_bytes < dakv::static_workspace_bytes(B, H, cap, D)) return DAKV_EINVAL;
  const dakv::SplitPlan plan = dakv::plan_static(B, H, cap, D, num_splits);
  return from_hip(dakv::launch_decode_step_static_fp4(q, k_codes, v_codes, k_scale, v_scale,
                                                      mask, valid_len, k_new, v_new, write_pos,
                                                      B, H, cap, D, scale, out, lse, workspace,
                                                      plan, err_flag, as_stream(stream)));
}

// --------------------------------------------------------------- copy_kvcache
int dakv_copy_kvcache(const void* const* src, void* const* dst, int n, int B, int H,
                      int src_cap, int dst_cap, int D, const int32_t* lengths, int32_t* mask,
                      int32_t* err_flag, void* stream) {
  static_assert(dakv::kCopyMaxTensors == DAKV_COPY_MAX_TENSORS, "header and library agree");
  if (n < 1 || n > DAKV_COPY_MAX_TENSORS || B < 0 || H < 0 || src_cap <= 0 || dst_cap <= 0 ||
      D <= 0)
    return DAKV_EINVAL;
  if (B == 0) return DAKV_OK;
  if ((D * 2) % 16 != 0) return DAKV_ENOTSUP;
  if (!src || !dst || !lengths) return DAKV_EINVAL;
  for (int i = 0; i < n; ++i)
    if (!src[i] || !dst[i] || !aligned16(src[i]) || !aligned16(dst[i])) return DAKV_EINVAL;
  if (H == 0 && !mask) return DAKV_OK;
  return from_hip(dakv::launch_copy_kvcache(src, dst, n, B, H, src_cap, dst_cap, D, lengths, mask,
                                            err_flag, as_stream(stream)));
}

int dakv_trim_kvcache(int32_t* mask, const int32_t* new_len, int B, int cap, int32_t* err_flag,
                      void* stream) {
  if (B < 0 || cap <= 0) return DAKV_EINVAL;
  if (B == 0) return DAKV_OK;
  if (!mask || !new_len) return DAKV_EINVAL;
  return from_hip(dakv::launch_trim_kvcache(mask, new_len, B, cap, err_flag, as_stream(stream)));
}

// --------------------------------------------------------- decode_attn_static
size_t dakv_decode_attn_static_workspace_size(int B, int H, int cap, int D) {
  if (B <= 0 || H <= 0 || cap <= 0 || D <= 0) return 0;
  return dakv::static_workspace_bytes(B, H, cap, D);
}

int dakv_decode_attn_static_split_rows(int B, int H, int cap, int D, int num_splits) {
  if (B <= 0 || H <= 0 || num_splits < 0 || (D != 64 && D != 128)) return 0;
  if (!dakv::static_supported(cap)) return 0;
  return dakv::plan_static(B, H, cap, D, num_splits).chunk;
}

int dakv_decode_attn_static(const float* q, const void* k_cache, const void* v_cache,
                            const int32_t* mask, const int32_t* valid_len, int B, int H,
                            int cap, int D, float scale, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, int num_splits,
                            int32_t* err_flag, void* stream) {
  if (B < 0 || H < 0 || cap <= 0 || D <= 0 || num_splits < 0) return DAKV_EINVAL;
  if (B == 0 || H == 0) return DAKV_OK;
  if (D != 64 && D != 128) return DAKV_ENOTSUP;
  if (!dakv::static_supported(cap)) return DAKV_ENOTSUP;
  if (!q || !k_cache || !v_cache || !out || !workspace) return DAKV_EINVAL;
  if (!mask && !valid_len) return DAKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(workspace))
    return DAKV_EINVAL;
  if (workspace_bytes < dakv::static_workspace_bytes(B, H, cap, D)) return DAKV_EINVAL;
  const dakv::SplitPlan plan = dakv::plan_static(B, H, cap, D, num_splits);
  return from_hip(dakv::launch_decode_static(
      q, const_cast<void*>(k_cache), const_cast<void*>(v_cache), const_cast<int32_t*>(mask),
      valid_len, nullptr, nullptr, nullptr, B, H, cap, D, scale, out, lse, workspace, plan,
      err_flag, as_stream(stream)));
}

// ---------------------------------- decode_attn_static without any allocation
// The split partials of dakv_decode_attn_static_noalloc live in this fixed array
// instead of a caller workspace.  Each GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` only names the symbol: its
// device address on a device comes from hipGetSymbolAddress with that device
// current, looked up once per device and kept in g_scratch_ptr.
static __device__ __align__(256) float scratch[DAKV_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// This device's copy of scratch, or nullptr on a HIP error.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

size_t dakv_decode_attn_static_noalloc_scratch_bytes(int B, int H, int cap, int D,
                                                     int num_splits) {
  if (B <= 0 || H <= 0 || num_splits < 0 || (D != 64 && D != 128)) return 0;
  if (!dakv::static_supported(cap)) return 0;
  const dakv::SplitPlan plan = dakv::plan_static(B, H, cap, D, num_splits);
  return dakv::static_plan_workspace_bytes(B, H, D, plan);
}

int dakv_decode_attn_static_noalloc(const float* q, const void* k_cache, const void* v_cache,
                                    const int32_t* mask, const int32_t* valid_len, int B, int H,
                                    int cap, int D, float scale, float* out, float* lse,
                                    int num_splits, int32_t* err_flag, void* stream) {
  if (B < 0 || H < 0 || cap <= 0 || D <= 0 || num_splits < 0) return DAKV_EINVAL;
  if (B == 0 || H == 0) return DAKV_OK;
  if (D != 64 && D != 128) return DAKV_ENOTSUP;
  if (!dakv::static_supported(cap)) return DAKV_ENOTSUP;
  if (!q || !k_cache || !v_cache || !out) return DAKV_EINVAL;
  if (!mask && !valid_len) return DAKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return DAKV_EINVAL;
  const dakv::SplitPlan plan = dakv::plan_static(B, H, cap, D, num_splits);
  if (dakv::static_plan_workspace_bytes(B, H, D, plan) > DAKV_NOALLOC_SCRATCH_BYTES)
    return DAKV_ESCRATCH;
  void* ws = scratch_on_current_device();
  if (!ws) return DAKV_EHIP;
  return from_hip(dakv::launch_decode_static(
      q, const_cast<void*>(k_cache), const_cast<void*>(v_cache), const_cast<int32_t*>(mask),
      valid_len, nullptr, nullptr, nullptr, B, H, cap, D, scale, out, lse, ws, plan, err_flag,
      as_stream(stream)));
}

int dakv_decode_step_static(const float* q, void* k_cache, void* v_cache, const void* k_new,
                            const void* v_new, const int32_t* write_pos, int32_t* mask,
                            const int32_t* valid_len, int B, int H, int cap, int D, float scale,
                            float* out, float* lse, void* workspace, size_t workspace_bytes,
                            int num_splits, int32_t* err_flag, void* stream) {
  if (B < 0 || H < 0 || cap <= 0 || D <= 0 || num_splits < 0) return DAKV_EINVAL;
  if (B == 0 || H == 0) return DAKV_OK;
  if (D != 64 && D != 128) return DAKV_ENOTSUP;
  if (!dakv::static_supported(cap)) return DAKV_ENOTSUP;
  if (!q || !k_cache || !v_cache || !k_new || !v_new || !write_pos || !out || !workspace)
    return DAKV_EINVAL;
  if (!mask && !valid_len) return DAKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) ||
      !aligned16(v_new) || !aligned16(out) || !aligned16(workspace))
    return DAKV_EINVAL;
  if (workspace_bytes < dakv::static_workspace_bytes(B, H, cap, D)) return DAKV_EINVAL;
  const dakv::SplitPlan plan = dakv::plan_static(B, H, cap, D, num_splits);
  return from_hip(dakv::launch_decode_static(q, k_cache, v_cache, mask, valid_len, k_new, v_new,
                                             write_pos, B, H, cap, D, scale, out, lse, workspace,
                                             plan, err_flag, as_stream(stream)));
}

// --------------------------------------------------------- gather_pa_kv_cache
int dakv_gather_pa_kv_cache(const void* key_cache, const void* value_cache, int num_blocks,
                            int block_size, int Hk, int Dk, int Hv, int Dv,
                            const int32_t* block_tables, int Q, int table_cols,
                            const int32_t* seq_lens, const int32_t* seq_offset,
                            int total_tokens, void* key_out, void* value_out,
                            int32_t* err_flag, void* stream) {
  if (num_blocks <= 0 || block_size <= 0 || Hk <= 0 || Dk <= 0 || Hv <= 0 || Dv <= 0 ||
      Q < 0 || table_cols < 0 || total_tokens < 0)
    return DAKV_EINVAL;
  if (total_tokens == 0) return DAKV_OK;
  if (Q == 0 || table_cols == 0) return DAKV_EINVAL;
  if (!key_cache || !value_cache || !block_tables || !seq_lens || !key_out || !value_out)
    return DAKV_EINVAL;
  const long long kb = 2LL * Hk * Dk, vb = 2LL * Hv * Dv;
  if (kb % 16 != 0 || vb % 16 != 0) return DAKV_ENOTSUP;
  if (kb > (1 << 30) || vb > (1 << 30)) return DAKV_ENOTSUP;
  if (!aligned16(key_cache) || !aligned16(value_cache) || !aligned16(key_out) ||
      !aligned16(value_out))
    return DAKV_EINVAL;
  return from_hip(dakv::launch_gather(key_cache, value_cache, num_blocks, block_size, (int)kb,
                                      (int)vb, block_tables, Q, table_cols, seq_lens, seq_offset,
                                      total_tokens, key_out, value_out, err_flag,
                                      as_stream(stream)));
}

// ---------------------------------------------------------- decode_attn_paged
size_t dakv_decode_attn_paged_workspace_size(int B, int Hq, int D, int max_seq_len,
                                             int block_size) {
  if (B <= 0 || Hq <= 0 || D <= 0 || max_seq_len < 0 || block_size <= 0) return 0;
  return dakv::paged_workspace_bytes(B, Hq, D, max_seq_len, block_size);
}

int dakv_decode_attn_paged(const void* q, const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, int table_cols,
                           const int32_t* seq_lens, const int32_t* seq_offset, int B, int Hq,
                           int Hkv, int D, int num_blocks, int block_size, int max_seq_len,
                           float scale, float* out, float* lse, void* workspace,
                           size_t workspace_bytes, int num_splits, int32_t* err_flag,
                           void* stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || num_blocks <= 0 || block_size <= 0 ||
      max_seq_len < 0 || table_cols <= 0 || num_splits < 0)
    return DAKV_EINVAL;
  if (B == 0) return DAKV_OK;
  if (Hq % Hkv != 0) return DAKV_EINVAL;
  const int G = Hq / Hkv;
  if (D != 128) return DAKV_ENOTSUP;
  if (G != 1 && G != 2 && G != 4 && G != 8) return DAKV_ENOTSUP;
  if (block_size != 16 && block_size != 32 && block_size != 64 && block_size != 128)
    return DAKV_ENOTSUP;
  if (!dakv::paged_supported(max_seq_len, block_size)) return DAKV_ENOTSUP;
  if (!q || !key_cache || !value_cache || !block_tables || !seq_lens || !out || !workspace)
    return DAKV_EINVAL;
  if (!aligned16(q) || !aligned16(key_cache) || !aligned16(value_cache) || !aligned16(out) ||
      !aligned16(workspace))
    return DAKV_EINVAL;
  if (workspace_bytes < dakv::paged_workspace_bytes(B, Hq, D, max_seq_len, block_size))
    return DAKV_EINVAL;
  if (dakv::paged_mfma_shape(B, Hq, Hkv, D, block_size)) {
    const dakv::SplitPlan mplan =
        dakv::plan_paged_mfma(B, Hkv, max_seq_len, block_size, num_splits);
    return from_hip(dakv::launch_decode_paged_mfma(
        q, key_cache, value_cache, block_tables, table_cols, seq_lens, seq_offset, B, Hq, Hkv,
        num_blocks, block_size, max_seq_len, scale, out, lse, workspace, mplan, err_flag,
        as_stream(stream)));
  }
  const dakv::SplitPlan plan = dakv::plan_paged(B, Hkv, G, max_seq_len, block_size, num_splits);
  return from_hip(dakv::launch_decode_paged(q, key_cache, value_cache, block_tables, table_cols,
                                            seq_lens, seq_offset, B, Hq, Hkv, D, num_blocks,
                                            block_size, max_seq_len, scale, out, lse, workspace,
                                            plan, err_flag, as_stream(stream)));
}

// ------------------------------------------------------------- paged, FP8 pool
static bool paged_fp8_shape(int Hq, int Hkv, int D, int block_size) {
  if (Hkv <= 0 || Hq % Hkv != 0 || 16 % Hkv != 0) return false;
  const int G = Hq / Hkv;
  return D == 128 && (G == 1 || G == 2 || G == 4 || G == 8) &&
         (block_size == 16 || block_size == 32 || block_size == 64 || block_size == 128);
}

// Shared by the FP8 and FP4 pools (codes one byte or half a byte per element).
static int paged_append_lowbit(bool fp4, void* k_codes, void* v_codes, float* k_scale,
                               float* v_scale, const void* k_new, const void* v_new,
                               const int32_t* block_tables, int table_cols,
                               const int32_t* seq_lens, const int32_t* seq_offset, int B,
                               int Hkv, int D, int num_blocks, int block_size, int32_t* err_flag,
                               void* stream) {
  if (B < 0 || Hkv <= 0 || D <= 0 || num_blocks <= 0 || block_size <= 0 || table_cols <= 0)
    return DAKV_EINVAL;
  if (B == 0) return DAKV_OK;
  if (D > 256 || (fp4 && D % 16 != 0)) return DAKV_ENOTSUP;
  if (!k_codes || !v_codes || !k_scale || !v_scale || !k_new || !v_new || !block_tables ||
      !seq_lens)
    return DAKV_EINVAL;
  const auto launch = fp4 ? dakv::launch_paged_append_fp4 : dakv::launch_paged_append_fp8;
  return from_hip(launch(k_codes, v_codes, k_scale, v_scale, k_new, v_new, block_tables,
                         table_cols, seq_lens, seq_offset, B, Hkv, D, num_blocks, block_size,
                         err_flag, as_stream(stream)));
}

static int decode_paged_lowbit(bool fp4, const void* q, const void* k_codes,
                               const void* v_codes, const float* k_scale, const float* v_scale,
                               const int32_t* block_tables, int table_cols,
                               const int32_t* seq_lens, const int32_t* seq_offset, int B, int Hq,
                               int Hkv, int D, int num_blocks, int block_size, int max_seq_len,
                               float scale, float* out, float* lse, void* workspace,
                               size_t workspace_bytes, int num_splits, int32_t* err_flag,
                               void* stream) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || num_blocks <= 0 || block_size <= 0 ||
      max_seq_len < 0 || table_cols <= 0 || num_splits < 0)
    return DAKV_EINVAL;
  if (B == 0) return DAKV_OK;
  if (Hq % Hkv != 0) return DAKV_EINVAL;
  if (!paged_fp8_shape(Hq, Hkv, D, block_size)) return DAKV_ENOTSUP;
  if (!dakv::paged_supported(max_seq_len, block_size)) return DAKV_ENOTSUP;
  if (!q || !k_codes || !v_codes || !k_scale || !v_scale || !block_tables || !seq_lens ||
      !out || !workspace)
    return DAKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(out) ||
      !aligned16(workspace))
    return DAKV_EINVAL;
  if (workspace_bytes < dakv::paged_workspace_bytes(B, Hq, D, max_seq_len, block_size))
    return DAKV_EINVAL;
  if (dakv::paged_mfma_shape(B, Hq, Hkv, D, block_size)) {
    const dakv::SplitPlan mplan =
        dakv::plan_paged_mfma(B, Hkv, max_seq_len, block_size, num_splits);
    return from_hip(dakv::launch_decode_paged_mfma_lowbit(
        fp4, q, k_codes, v_codes, k_scale, v_scale, block_tables, table_cols, seq_lens,
        seq_offset, B, Hq, Hkv, num_blocks, block_size, max_seq_len, scale, out, lse, workspace,
        mplan, err_flag, as_stream(stream)));
  }
  const dakv::SplitPlan plan =
      dakv::plan_paged(B, Hkv, Hq / Hkv, max_seq_len, block_size, num_splits);
  const auto launch = fp4 ? dakv::launch_decode_paged_fp4 : dakv::launch_decode_paged_fp8;
  return from_hip(launch(q, k_codes, v_codes, k_scale, v_scale, block_tables, table_cols,
                         seq_lens, seq_offset, B, Hq, Hkv, num_blocks, block_size, max_seq_len,
                         scale, out, lse, workspace, plan, err_flag, as_stream(stream)));
}

int dakv_paged_append_fp8(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                          const void* k_new, const void* v_new, const int32_t* block_tables,
                          int table_cols, const int32_t* seq_lens, const int32_t* seq_offset,
                          int B, int Hkv, int D, int num_blocks, int block_size,
                          int32_t* err_flag, void* stream) {
  return paged_append_lowbit(false, k_codes, v_codes, k_scale, v_scale, k_new, v_new,
                             block_tables, table_cols, seq_lens, seq_offset, B, Hkv, D,
                             num_blocks, block_size, err_flag, stream);
}

int dakv_paged_append_fp4(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                          const void* k_new, const void* v_new, const int32_t* block_tables,
                          int table_cols, const int32_t* seq_lens, const int32_t* seq_offset,
                          int B, int Hkv, int D, int num_blocks, int block_size,
                          int32_t* err_flag, void* stream) {
  return paged_append_lowbit(true, k_codes, v_codes, k_scale, v_scale, k_new, v_new,
                             block_tables, table_cols, seq_lens, seq_offset, B, Hkv, D,
                             num_blocks, block_size, err_flag, stream);
}

int dakv_decode_attn_paged_fp8(const void* q, const void* k_codes, const void* v_codes,
                               const float* k_scale, const float* v_scale,
                               const int32_t* block_tables, int table_cols,
                               const int32_t* seq_lens, const int32_t* seq_offset, int B,
                               int Hq, int Hkv, int D, int num_blocks, int block_size,
                               int max_seq_len, float scale, float* out, float* lse,
                               void* workspace, size_t workspace_bytes, int num_splits,
                               int32_t* err_flag, void* stream) {
  return decode_paged_lowbit(false, q, k_codes, v_codes, k_scale, v_scale, block_tables,
                             table_cols, seq_lens, seq_offset, B, Hq, Hkv, D, num_blocks,
                             block_size, max_seq_len, scale, out, lse, workspace,
                             workspace_bytes, num_splits, err_flag, stream);
}

int dakv_decode_attn_paged_fp4(const void* q, const void* k_codes, const void* v_codes,
                               const float* k_scale, const float* v_scale,
                               const int32_t* block_tables, int table_cols,
                               const int32_t* seq_lens, const int32_t* seq_offset, int B,
                               int Hq, int Hkv, int D, int num_blocks, int block_size,
                               int max_seq_len, float scale, float* out, float* lse,
                               void* workspace, size_t workspace_bytes, int num_splits,
                               int32_t* err_flag, void* stream) {
  return decode_paged_lowbit(true, q, k_codes, v_codes, k_scale, v_scale, block_tables,
                             table_cols, seq_lens, seq_offset, B, Hq, Hkv, D, num_blocks,
                             block_size, max_seq_len, scale, out, lse, workspace,
                             workspace_bytes, num_splits, err_flag, stream);
}

// ---------------------------------------------------- sparse_topk_decode_attn
size_t dakv_sparse_topk_decode_attn_workspace_size(int B, int Hq, int d_qk, int d_v,
                                                   int topk) {
  if (B <= 0 || Hq <= 0 || d_qk <= 0 || d_v <= 0 || topk <= 0) return 0;
  return dakv::sparse_workspace_bytes(B, Hq, d_qk, d_v, topk);
}

// Shared by the bf16, FP8 and FP4 latent caches (format 0, 1, 2).
static int sparse_attn(const void* q, const void* kv, const float* kv_scale, int format,
                       const int32_t* indices, int B, int s_q, int Hq, int s_kv, int d_qk,
                       int d_v, int topk, float sm_scale, float* out, float* lse,
                       void* workspace, size_t workspace_bytes, int32_t* err_flag,
                       void* stream) {
  if (B < 0 || s_q < 0 || Hq <= 0 || s_kv <= 0 || d_qk <= 0 || d_v <= 0 || topk < 0)
    return DAKV_EINVAL;
  if (B == 0 || s_q == 0) return DAKV_OK;
  if ((long long)B * s_q > (1 << 24)) return DAKV_EINVAL;
  if (d_qk != 576 || d_v != 512) return DAKV_ENOTSUP;
  if (Hq % 16 != 0 || Hq > 128) return DAKV_ENOTSUP;
  // a sequence's latent rows are addressed with 32-bit byte offsets
  if ((long long)s_kv * d_qk * 2 > 0x7fffffffLL) return DAKV_ENOTSUP;
  if (!q || !kv || !out || (topk > 0 && !indices)) return DAKV_EINVAL;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(out)) return DAKV_EINVAL;
  const int pairs = B * s_q;
  const size_t need = dakv::sparse_workspace_bytes(pairs, Hq, d_qk, d_v, topk);
  if (need > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < need))
    return DAKV_EINVAL;
  return from_hip(dakv::launch_sparse(q, kv, kv_scale, format, indices, pairs, s_q, Hq, s_kv,
                                      d_qk, d_v, topk, sm_scale, out, lse, workspace, err_flag,
                                      as_stream(stream)));
}

int dakv_sparse_topk_attn(const void* q, const void* kv, const int32_t* indices, int B,
                          int s_q, int Hq, int s_kv, int d_qk, int d_v, int topk,
                          float sm_scale, float* out, float* lse, void* workspace,
                          size_t workspace_bytes, int32_t* err_flag, void* stream) {
  return sparse_attn(q, kv, nullptr, 0, indices, B, s_q, Hq, s_kv, d_qk, d_v, topk, sm_scale,
                     out, lse, workspace, workspace_bytes, err_flag, stream);
}

int dakv_sparse_topk_attn_fp8(const void* q, const void* codes, const float* scale,
                              const int32_t* indices, int B, int s_q, int Hq, int s_kv, int d_qk,
                              int d_v, int topk, float sm_scale, float* out, float* lse,
                              void* workspace, size_t workspace_bytes, int32_t* err_flag,
                              void* stream) {
  if (!scale && B > 0 && s_q > 0) return DAKV_EINVAL;
  return sparse_attn(q, codes, scale, 1, indices, B, s_q, Hq, s_kv, d_qk, d_v, topk, sm_scale,
                     out, lse, workspace, workspace_bytes, err_flag, stream);
}

int dakv_sparse_topk_attn_fp4(const void* q, const void* codes, const float* scale,
                              const int32_t* indices, int B, int s_q, int Hq, int s_kv, int d_qk,
                              int d_v, int topk, float sm_scale, float* out, float* lse,
                              void* workspace, size_t workspace_bytes, int32_t* err_flag,
                              void* stream) {
  if (!scale && B > 0 && s_q > 0) return DAKV_EINVAL;
  return sparse_attn(q, codes, scale, 2, indices, B, s_q, Hq, s_kv, d_qk, d_v, topk, sm_scale,
                     out, lse, workspace, workspace_bytes, err_flag, stream);
}

int dakv_latent_append_fp4(void* codes, float* scale, const void* new_rows,
                           const int32_t* write_pos, int B, int s_kv, int d_qk,
                           int32_t* err_flag, void* stream) {
  if (B < 0 || s_kv <= 0 || d_qk <= 0) return DAKV_EINVAL;
  if (B == 0) return DAKV_OK;
  if (d_qk > 576 || d_qk % 2 != 0) return DAKV_ENOTSUP;
  if (!codes || !scale || !new_rows || !write_pos) return DAKV_EINVAL;
  return from_hip(dakv::launch_latent_append_fp4(codes, scale, new_rows, write_pos, B, s_kv,
                                                 d_qk, err_flag, as_stream(stream)));
}

int dakv_latent_append_fp8(void* codes, float* scale, const void* new_rows,
                           const int32_t* write_pos, int B, int s_kv, int d_qk,
                           int32_t* err_flag, void* stream) {
  if (B < 0 || s_kv <= 0 || d_qk <= 0) return DAKV_EINVAL;
  if (B == 0) return DAKV_OK;
  if (d_qk > 576) return DAKV_ENOTSUP;
  if (!codes || !scale || !new_rows || !write_pos) return DAKV_EINVAL;
  return from_hip(dakv::launch_latent_append_fp8(codes, scale, new_rows, write_pos, B, s_kv,
                                                 d_qk, err_flag, as_stream(stream)));
}

int dakv_sparse_topk_decode_attn(const void* q, const void* kv, const int32_t* indices,
                                 int B, int Hq, int s_kv, int d_qk, int d_v, int topk,
                                 float sm_scale, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, int32_t* err_flag, void* stream) {
  return dakv_sparse_topk_attn(q, kv, indices, B, 1, Hq, s_kv, d_qk, d_v, topk, sm_scale, out,
                               lse, workspace, workspace_bytes, err_flag, stream);
}

// ------------------------------------------------------------ host validators
int dakv_validate_paged(const int32_t* block_tables, int Q, int table_cols,
                        const int32_t* seq_lens, const int32_t* seq_offset, int num_blocks,
                        int block_size) {
  if (Q < 0 || table_cols < 0 || num_blocks < 0 || block_size <= 0) return DAKV_EINVAL;
  if (!seq_lens) return DAKV_EINVAL;
  if (Q > 0 && table_cols > 0 && !block_tables) return DAKV_EINVAL;
  if (seq_lens[0] != 0) return DAKV_ERANGE;
  for (int q = 0; q < Q; ++q) {
    const long long len = (long long)seq_lens[q + 1] - seq_lens[q];
    if (len < 0) return DAKV_ERANGE;
    const int off = seq_offset ? seq_offset[q] : 0;
    if (off < 0 || off % block_size != 0) return DAKV_ERANGE;
    const long long first = off / block_size;
    const long long used = (len + block_size - 1) / block_size;
    if (used == 0) continue;
    if (first + used > table_cols) return DAKV_ERANGE;
    const int32_t* row = block_tables + (size_t)q * table_cols;
    for (long long c = first; c < first + used; ++c)
      if (row[c] < 0 || row[c] >= num_blocks) return DAKV_ERANGE;
  }
  return DAKV_OK;
}

int dakv_validate_sparse(const int32_t* indices, int B, int topk, int s_kv) {
  if (B < 0 || topk < 0 || s_kv < 0) return DAKV_EINVAL;
  if ((size_t)B * topk > 0 && !indices) return DAKV_EINVAL;
  const size_t n = (size_t)B * topk;
  for (size_t i = 0; i < n; ++i)
    if (indices[i] < 0 || indices[i] >= s_kv) return DAKV_ERANGE;
  return DAKV_OK;
}

int dakv_validate_range(const int32_t* values, int n, int lo, int hi) {
  if (n < 0) return DAKV_EINVAL;
  if (n > 0 && !values) return DAKV_EINVAL;
  for (int i = 0; i < n; ++i)
    if (values[i] < lo || values[i] > hi) return DAKV_ERANGE;
  return DAKV_OK;
}

}  // extern "C"
