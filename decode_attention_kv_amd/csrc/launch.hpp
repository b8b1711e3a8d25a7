// Host-side launchers of the gfx950 kernels (internal to the library).  The
// C-ABI entry points validate arguments and then call these; every launcher
// enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dakv {

constexpr int kCopyMaxTensors = 128;  // tensor pairs per copy_kvcache call
hipError_t launch_copy_kvcache(const void* const* src, void* const* dst, int n, int B, int H,
                               int src_cap, int dst_cap, int D, const int32_t* lengths,
                               int32_t* mask, int32_t* err_flag, hipStream_t stream);
hipError_t launch_trim_kvcache(int32_t* mask, const int32_t* new_len, int B, int cap,
                               int32_t* err_flag, hipStream_t stream);
hipError_t launch_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            const int32_t* write_pos, int32_t* mask, int B, int H, int cap,
                            int D, int32_t* err_flag, hipStream_t stream);

hipError_t launch_gather(const void* key_cache, const void* value_cache, int num_blocks,
                         int block_size, int k_row_bytes, int v_row_bytes,
                         const int32_t* block_tables, int Q, int table_cols,
                         const int32_t* seq_lens, const int32_t* seq_offset, int total_tokens,
                         void* key_out, void* value_out, int32_t* err_flag, hipStream_t stream);

// Split-K plan of a decode call: rows [s*chunk, (s+1)*chunk) go to split s.
struct SplitPlan {
  int chunk;       // rows per split
  int max_splits;  // splits of the longest possible sequence
};

SplitPlan plan_static(int B, int H, int cap, int D, int forced_splits);
// Whether a capacity fits the split limits of the static kernel (<= 65536 rows).
bool static_supported(int cap);
size_t static_workspace_bytes(int B, int H, int cap, int D);
// Workspace bytes a call with this plan actually writes (<= static_workspace_bytes).
size_t static_plan_workspace_bytes(int B, int H, int D, const SplitPlan& plan);
// write_pos != NULL: append k_new / v_new (bf16 [B, H, D]) first (decode_step_static_fp8)
hipError_t launch_decode_static_fp8(const float* q, void* k_codes, void* v_codes, float* k_scale,
                                    float* v_scale, int32_t* mask, const int32_t* valid_len,
                                    const void* k_new, const void* v_new,
                                    const int32_t* write_pos, int B, int H, int cap, int D,
                                    float scale, float* out, float* lse, void* ws,
                                    const SplitPlan& plan, int32_t* err_flag, hipStream_t stream);
hipError_t launch_kv_append_fp8(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                                const void* k_new, const void* v_new, const int32_t* write_pos,
                                int32_t* mask, int B, int H, int cap, int D, int32_t* err_flag,
                                hipStream_t stream);
// decode_attn_static; with write_pos != nullptr also the append of decode_step_static
hipError_t launch_decode_static(const float* q, void* k_cache, void* v_cache, int32_t* mask,
                                const int32_t* valid_len, const void* k_new, const void* v_new,
                                const int32_t* write_pos, int B, int H, int cap, int D,
                                float scale, float* out, float* lse, void* ws,
                                const SplitPlan& plan, int32_t* err_flag, hipStream_t stream);

// FP4 cache (static layout): E2M1 codes uint8 [B, H, cap, D / 2] (two per byte),
// scales fp32 [B, H, cap]
hipError_t launch_kv_append_fp4(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                                const void* k_new, const void* v_new, const int32_t* write_pos,
                                int32_t* mask, int B, int H, int cap, int D, int32_t* err_flag,
                                hipStream_t stream);
hipError_t launch_decode_static_fp4(const float* q, const void* k_codes, const void* v_codes,
                                    const float* k_scale, const float* v_scale,
                                    const int32_t* mask, const int32_t* valid_len, int B, int H,
                                    int cap, int D, float scale, float* out, float* lse, void* ws,
                                    const SplitPlan& plan, int32_t* err_flag, hipStream_t stream);
// decode_attn_static_fp4 with the quantising append of kv_append_fp4 in the same pass
hipError_t launch_decode_step_static_fp4(const float* q, void* k_codes, void* v_codes,
                                         float* k_scale, float* v_scale, int32_t* mask,
                                         const int32_t* valid_len, const void* k_new,
                                         const void* v_new, const int32_t* write_pos, int B,
                                         int H, int cap, int D, float scale, float* out,
                                         float* lse, void* ws, const SplitPlan& plan,
                                         int32_t* err_flag, hipStream_t stream);
// FP8 paged pool: codes uint8 [num_blocks, block_size, Hkv, D], scales fp32
// [num_blocks, block_size, Hkv]; D = 128, Hkv dividing 16 (the all-heads kernel).
hipError_t launch_paged_append_fp8(void* k_codes, void* v_codes, float* k_scale,
                                   float* v_scale, const void* k_new, const void* v_new,
                                   const int32_t* block_tables, int table_cols,
                                   const int32_t* seq_lens, const int32_t* seq_offset, int B,
                                   int Hkv, int D, int num_blocks, int block_size,
                                   int32_t* err_flag, hipStream_t stream);
hipError_t launch_decode_paged_fp8(const void* q, const void* k_codes, const void* v_codes,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_tables, int table_cols,
                                   const int32_t* seq_lens, const int32_t* seq_offset, int B,
                                   int Hq, int Hkv, int num_blocks, int block_size,
                                   int max_seq_len, float scale, float* out, float* lse,
                                   void* ws, const SplitPlan& plan, int32_t* err_flag,
                                   hipStream_t stream);
// FP4 paged pool: packed codes uint8 [num_blocks, block_size, Hkv, D / 2], same scales.
hipError_t launch_paged_append_fp4(void* k_codes, void* v_codes, float* k_scale,
                                   float* v_scale, const void* k_new, const void* v_new,
                                   const int32_t* block_tables, int table_cols,
                                   const int32_t* seq_lens, const int32_t* seq_offset, int B,
                                   int Hkv, int D, int num_blocks, int block_size,
                                   int32_t* err_flag, hipStream_t stream);
hipError_t launch_decode_paged_fp4(const void* q, const void* k_codes, const void* v_codes,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_tables, int table_cols,
                                   const int32_t* seq_lens, const int32_t* seq_offset, int B,
                                   int Hq, int Hkv, int num_blocks, int block_size,
                                   int max_seq_len, float scale, float* out, float* lse,
                                   void* ws, const SplitPlan& plan, int32_t* err_flag,
                                   hipStream_t stream);

SplitPlan plan_paged(int B, int Hkv, int G, int max_seq_len, int block_size,
                     int forced_splits);
// Paged decode on the matrix cores (paged_mfma.hip): Hkv in {2, 4, 8k}, G in {1, 2, 4,
// 8}, D = 128, block_size in {16, 32, 64, 128}, B <= 512; its own split plan.  The
// same kernel serves the bf16 pool and the FP8 / FP4 pools (codes dequantised with
// their row scales on the way into LDS).
bool paged_mfma_shape(int B, int Hq, int Hkv, int D, int block_size);
SplitPlan plan_paged_mfma(int B, int Hkv, int max_seq_len, int block_size, int forced_splits);
hipError_t launch_decode_paged_mfma(const void* q, const void* key_cache,
                                    const void* value_cache, const int32_t* block_tables,
                                    int table_cols, const int32_t* seq_lens,
                                    const int32_t* seq_offset, int B, int Hq, int Hkv,
                                    int num_blocks, int block_size, int max_seq_len,
                                    float scale, float* out, float* lse, void* ws,
                                    const SplitPlan& plan, int32_t* err_flag,
                                    hipStream_t stream);
hipError_t launch_decode_paged_mfma_lowbit(bool fp4, const void* q, const void* k_codes,
                                           const void* v_codes, const float* k_scale,
                                           const float* v_scale, const int32_t* block_tables,
                                           int table_cols, const int32_t* seq_lens,
                                           const int32_t* seq_offset, int B, int Hq, int Hkv,
                                           int num_blocks, int block_size, int max_seq_len,
                                           float scale, float* out, float* lse, void* ws,
                                           const SplitPlan& plan, int32_t* err_flag,
                                           hipStream_t stream);
// Whether a sequence of max_seq_len tokens fits the split limits of the paged kernel.
bool paged_supported(int max_seq_len, int block_size);
size_t paged_workspace_bytes(int B, int Hq, int D, int max_seq_len, int block_size);
hipError_t launch_decode_paged(const void* q, const void* key_cache, const void* value_cache,
                               const int32_t* block_tables, int table_cols,
                               const int32_t* seq_lens, const int32_t* seq_offset, int B,
                               int Hq, int Hkv, int D, int num_blocks, int block_size,
                               int max_seq_len, float scale, float* out, float* lse, void* ws,
                               const SplitPlan& plan, int32_t* err_flag, hipStream_t stream);

size_t sparse_workspace_bytes(int B, int Hq, int d_qk, int d_v, int topk);
// B = (sequence, q-token) pairs; the s_q tokens of sequence b / s_q share its kv rows.
// format 0: bf16 latent rows; 1: E4M3 codes, 2: E2M1 codes (two a byte), each with one
// fp32 scale per row in kv_scale.
hipError_t launch_sparse(const void* q, const void* kv, const float* kv_scale, int format,
                         const int32_t* indices, int B, int s_q, int Hq, int s_kv, int d_qk,
                         int d_v, int topk, float sm_scale, float* out, float* lse, void* ws,
                         int32_t* err_flag, hipStream_t stream);
// quantising append of one latent row (d <= 576) per sequence into [B, s_kv, d] codes
hipError_t launch_latent_append_fp8(void* codes, float* scale, const void* new_rows,
                                    const int32_t* write_pos, int B, int s_kv, int d,
                                    int32_t* err_flag, hipStream_t stream);
// the same in E2M1 (d even, d <= 640): packed codes [B, s_kv, d / 2]
hipError_t launch_latent_append_fp4(void* codes, float* scale, const void* new_rows,
                                    const int32_t* write_pos, int B, int s_kv, int d,
                                    int32_t* err_flag, hipStream_t stream);

}  // namespace dakv
