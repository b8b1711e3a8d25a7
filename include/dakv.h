/*
 * dakv.h -- decode-phase attention over a KV cache on AMD MI355X (gfx950).
 *
 * A C-ABI library: plain pointers and sizes, no framework types.  Every tensor
 * is caller-owned device memory, dense and row-major in the shape given; the
 * library never allocates, frees or synchronises.  Each call enqueues its
 * kernels on `stream` (a hipStream_t; NULL is the null stream) and returns at
 * once.  Base pointers of tensors must be 16-byte aligned.
 *
 * Return value of every entry point: DAKV_OK (0) or a negative DAKV_E* code,
 * decided on the host before anything is enqueued (DAKV_EHIP: a launch error
 * reported by the HIP runtime).  Faults that only the device can see (index
 * content of device tensors) never cause an out-of-bounds access: the kernel
 * skips the offending unit and ORs a DAKV_ERR_* bit into the optional
 * caller-owned int32 `err_flag` (pass NULL to ignore).  The host validators
 * dakv_validate_* check index content on host copies before a call.
 *
 * Sources (pages on decode attention; each entry point cites the passage that
 * defines its operation):
 *   [NPU-LLM]  OpenVINO community article on LLM inference on the Intel NPU,
 *              openvinohackathon.51openlab.com article 882, and its retelling
 *              "NPU 上的 LLM 推理：KV Cache 与软件栈" (jonathanding.github.io).
 *   [PyPTO]    "PyPTO 实现 AscendC GatherPaKvCache（Norm/ND 分支）", www.mhpn.cn.
 *   [FlashMLA] "FlashMLA на Huawei Ascend: ядро разреженного внимания изнутри",
 *              ai.flicky.cc.
 */
#ifndef DAKV_H
#define DAKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define DAKV_OK 0
#define DAKV_EINVAL (-1)  /* null pointer, bad size, misaligned pointer, short workspace */
#define DAKV_ENOTSUP (-2) /* a shape no kernel is built for (head_dim, block size, ...) */
#define DAKV_ERANGE (-3)  /* a host validator found index content outside the contract */
#define DAKV_EHIP (-4)    /* the HIP runtime reported an error at launch */
#define DAKV_ESCRATCH (-5) /* a call needs more than the fixed scratch of the no-alloc entry */

/* ---- device error-flag bits (OR-ed into *err_flag) ---------------------- */
#define DAKV_ERR_BLOCK_ID 1     /* a used block-table entry is outside [0, num_blocks) */
#define DAKV_ERR_WRITE_POS 2    /* an append position is outside [0, cap) */
#define DAKV_ERR_SPARSE_INDEX 4 /* a sparse index is outside [0, s_kv) */
#define DAKV_ERR_SEQ_LENS 8     /* cumulative seq_lens decrease, or a table offset is bad */
#define DAKV_ERR_VALID_LEN 16   /* a valid length is outside [0, cap] (clamped) */
#define DAKV_ERR_COPY_LEN 32    /* a copy or trim length is outside its buffers (clamped) */
#define DAKV_COPY_MAX_TENSORS 128 /* tensor pairs one dakv_copy_kvcache call takes */

/* Text for a status code (static storage). */
const char* dakv_strerror(int code);

/* ========================================================================
 * Static preallocated KV buffer   ([NPU-LLM] Part 1, "Solution:
 * preallocation + attention mask"; Part 2, the generate loop)
 *
 * Cache layout: k_cache, v_cache bf16 [B, H, cap, D] -- one fixed buffer per
 * layer; capacity = MAX_PROMPT_LEN + MIN_RESPONSE_LEN on the page (1024+128).
 * Row t of sequence b is attended iff t < valid_len[b] and mask[b, t] != 0.
 * ======================================================================== */

/*
 * kv_append -- write the new token's K and V into the next free row.
 * [NPU-LLM] Part 2: the cache update writes only the new row (the present
 * K/V of the new token) into the first empty slot of the past buffer and
 * increments the stored-row counter.
 *
 *   k_cache, v_cache  bf16 [B, H, cap, D], updated in place at row write_pos[b]
 *   k_new, v_new      bf16 [B, H, D]
 *   write_pos         int32 [B] device; the row to write (rows stored so far)
 *   mask              int32 [B, cap] or NULL; when given, mask[b, write_pos[b]] = 1
 *   err_flag          optional; DAKV_ERR_WRITE_POS if a position is outside
 *                     [0, cap) -- that sequence is left untouched
 * Requires D*2 to be a multiple of 16.
 */
int dakv_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                   const int32_t* write_pos, int32_t* mask, int B, int H, int cap, int D,
                   int32_t* err_flag, void* stream);

/*
 * FP8 KV cache ([FlashMLA] section on VECTOR cores per CUBE core, item 2: at
 * decode time the kernel reads the KV cache in FP8 and dequantises it; section on
 * the decoding KV-cache layout: a token's values and scale go together).  Codes
 * are OCP E4M3 (bias 7, largest finite 448), one byte per element, [B, H, cap, D];
 * every cached row has one power-of-two fp32 scale, for K in k_scale and for V in
 * v_scale, [B, H, cap]: s = 2^e, e the smallest integer with max|x| <= 448 * 2^e
 * (e = 0 for a zero row), code = x / s rounded to the nearest E4M3 value, ties to
 * the even code (zero results are the +0 code).  The cached value is
 * decode(code) * s.  (The scales live in their own arrays rather than inside the
 * row: on the GPU they are one coalesced 4-byte stream and the rows stay 16-byte
 * aligned.)
 *
 * kv_append_fp8 -- quantise the new token's K and V rows (bf16 [B, H, D], finite
 * values) and store codes and scales at row write_pos[b]; mask as kv_append.  A
 * position outside [0, cap) sets DAKV_ERR_WRITE_POS and skips that sequence.
 * D in 16 .. 256, a multiple of 16.
 */
int dakv_kv_append_fp8(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                       const void* k_new, const void* v_new, const int32_t* write_pos,
                       int32_t* mask, int B, int H, int cap, int D, int32_t* err_flag,
                       void* stream);

/* Workspace bytes dakv_decode_attn_static_fp8 needs (the same as the bf16 call's). */
size_t dakv_decode_attn_static_fp8_workspace_size(int B, int H, int cap, int D);

/*
 * decode_attn_static_fp8 -- decode_attn_static over an FP8 cache: the same query,
 * mask, valid length, scale, outputs, workspace and split rules, with row t of
 * (b, h) taken as decode(code) * scale[b, h, t] for K and for V.
 *   k_codes, v_codes  uint8 E4M3 [B, H, cap, D];  k_scale, v_scale fp32 [B, H, cap]
 * Supported: D in {64, 128}, cap <= 65536.
 */
int dakv_decode_attn_static_fp8(const float* q, const void* k_codes, const void* v_codes,
                                const float* k_scale, const float* v_scale, const int32_t* mask,
                                const int32_t* valid_len, int B, int H, int cap, int D,
                                float scale, float* out, float* lse, void* workspace,
                                size_t workspace_bytes, int num_splits, int32_t* err_flag,
                                void* stream);

/*
 * decode_step_static_fp8 -- kv_append_fp8 followed by decode_attn_static_fp8, in
 * one split pass: the split that owns write_pos[b] quantises and stores the new
 * row before attending (same results as the two calls; the new row is attended
 * whatever its mask entry says, and the mask entry is set).  Arguments as the two
 * calls; k_new, v_new bf16 [B, H, D] (finite values), write_pos int32 [B].
 */
int dakv_decode_step_static_fp8(const float* q, void* k_codes, void* v_codes, float* k_scale,
                                float* v_scale, const void* k_new, const void* v_new,
                                const int32_t* write_pos, int32_t* mask, const int32_t* valid_len,
                                int B, int H, int cap, int D, float scale, float* out, float* lse,
                                void* workspace, size_t workspace_bytes, int num_splits,
                                int32_t* err_flag, void* stream);

/*
 * copy_kvcache -- hand the prefill model's KV cache to the generate model.
 * [NPU-LLM] Part 2, step 3 of the generate flow: the prefill model's present
 * tensors (capacity 1024 there) and the generate model's past tensors (1152)
 * differ in capacity, so the valid rows [0, len) of every layer's K and V are
 * copied as a slice, all 2 x layers tensors in parallel; "Current
 * limitations": 512 MB at 7B with 1024 rows.
 *
 *   src       HOST array of n DEVICE pointers, each [B, H, src_cap, D] of 2-byte
 *             elements (bf16 or fp16: the copy moves bits)
 *   dst       HOST array of n DEVICE pointers, each [B, H, dst_cap, D]; rows
 *             [0, lengths[b]) of sequence b are overwritten, the others kept
 *   n         1 .. DAKV_COPY_MAX_TENSORS tensor pairs (pair i: src[i] -> dst[i])
 *   lengths   int32 [B] device; rows to copy per sequence, in
 *             [0, min(src_cap, dst_cap)]
 *   mask      int32 [B, dst_cap] or NULL; when given it becomes 1 for the
 *             copied rows and 0 for the rest (the stored-row count is lengths[b])
 *   err_flag  optional; a length outside the buffers is clamped into them and
 *             sets DAKV_ERR_COPY_LEN
 * Pointers 16-byte aligned; D*2 a multiple of 16.  The pointer arrays are read
 * during the call (they may be reused once it returns).
 */
int dakv_copy_kvcache(const void* const* src, void* const* dst, int n, int B, int H,
                      int src_cap, int dst_cap, int D, const int32_t* lengths,
                      int32_t* mask, int32_t* err_flag, void* stream);

/*
 * trim_kvcache -- roll each sequence's stored rows back to new_len[b].
 * [NPU-LLM] deployment features: speculative decoding cuts the cache back to
 * the last accepted position.  With the 0/1 mask, rows at and after new_len[b]
 * stop counting (mask = 0); earlier entries and the row contents are left as
 * they are.  A length of 0 resets the sequence.
 *
 *   mask      int32 [B, cap] device, updated in place
 *   new_len   int32 [B] device, in [0, cap]; outside it is clamped and sets
 *             DAKV_ERR_COPY_LEN in the optional err_flag
 */
int dakv_trim_kvcache(int32_t* mask, const int32_t* new_len, int B, int cap, int32_t* err_flag,
                      void* stream);

/*
 * Workspace bytes dakv_decode_attn_static needs (split-K partial outputs and
 * log-sum-exps).  Depends only on the sizes, so one buffer serves every call
 * of that size.
 */
size_t dakv_decode_attn_static_workspace_size(int B, int H, int cap, int D);

/*
 * Rows per split that dakv_decode_attn_static, dakv_decode_step_static and their
 * FP8 / FP4 forms use for these sizes and num_splits (0 = automatic): 64, 128 or
 * 256.  The split pass of such a call runs chunk / (rows per step) steps, so this
 * names the kernel instantiation a call reaches.  0 for sizes no kernel serves.
 * Pure host computation; no device work.
 */
int dakv_decode_attn_static_split_rows(int B, int H, int cap, int D, int num_splits);

/*
 * decode_attn_static -- one new query row per (sequence, head) attending over
 * the static buffer.  [NPU-LLM] "Attention on the NPU": decomposed SDPA
 * (Q K^T, times the scale, plus the mask, softmax, times V) and "incremental
 * SDPA" (the one-query decode case); Part 1: mask = 0 -> -inf before softmax,
 * so those rows get weight zero.  The "Flash SDPA" passage: tiles along the
 * sequence computed independently and merged exactly with a running maximum and
 * sum -- here split-K over the rows, then a log-sum-exp merge.
 *
 *   q          fp32 [B, H, D]
 *   k_cache    bf16 [B, H, cap, D];  v_cache likewise
 *   mask       int32 [B, cap] (nonzero = attend) or NULL
 *   valid_len  int32 [B] device, or NULL (= cap); at least one of mask /
 *              valid_len.  Values outside [0, cap] are clamped and flagged.
 *   scale      multiplier of q.k (1/sqrt(D) for standard attention)
 *   out        fp32 [B, H, D]: sum_t softmax(scale q.K_t) V_t over attended rows;
 *              zeros when no row is attended
 *   lse        fp32 [B, H] or NULL: natural log of sum_t exp(scale q.K_t);
 *              -inf when no row is attended
 *   workspace  device scratch of at least
 *              dakv_decode_attn_static_workspace_size(B, H, cap, D) bytes
 *   num_splits 0 = automatic; n >= 1 forces n splits of the row axis (capped at
 *              the workspace's maximum)
 * Rows not attended are never read, so NaN/Inf stored there cannot reach out.
 * Supported: D in {64, 128}; cap <= 65536.
 */
int dakv_decode_attn_static(const float* q, const void* k_cache, const void* v_cache,
                            const int32_t* mask, const int32_t* valid_len, int B, int H,
                            int cap, int D, float scale, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, int num_splits,
                            int32_t* err_flag, void* stream);

/*
 * decode_step_static -- one decode step of a layer: kv_append of the new token's
 * K/V at write_pos[b] (mask bit set when a mask is given), then
 * decode_attn_static over the updated buffer, in one pass.  [NPU-LLM] Part 2:
 * each generate step writes the new row into the next free slot, then the
 * incremental SDPA attends the whole valid buffer; the mutable command list of
 * the NPU runtime replays the same work every step.  The result is what
 * dakv_kv_append followed by dakv_decode_attn_static gives, bit for bit: the split
 * that owns position write_pos[b] stores the row and attends it from registers.
 *
 * Arguments as for the two calls; k_cache, v_cache and mask are updated in place.
 * A write position outside [0, cap) sets DAKV_ERR_WRITE_POS and that sequence is
 * attended without the new row.  Supported: D in {64, 128}.
 */
int dakv_decode_step_static(const float* q, void* k_cache, void* v_cache, const void* k_new,
                            const void* v_new, const int32_t* write_pos, int32_t* mask,
                            const int32_t* valid_len, int B, int H, int cap, int D, float scale,
                            float* out, float* lse, void* workspace, size_t workspace_bytes,
                            int num_splits, int32_t* err_flag, void* stream);

/*
 * decode_attn_static_noalloc -- dakv_decode_attn_static for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments without the workspace,
 * the same kernels and the same results bit for bit.  The split partials go to a
 * fixed device array of DAKV_NOALLOC_SCRATCH_BYTES bytes inside the library (one
 * per GPU, held from the first call on that GPU until the process ends; its
 * address is looked up on that first call, with the device current).  The call
 * itself allocates and frees nothing.
 *   Limit: a call whose partials exceed the array
 *   (dakv_decode_attn_static_noalloc_scratch_bytes(...) > DAKV_NOALLOC_SCRATCH_BYTES)
 *   returns DAKV_ESCRATCH before anything is enqueued.  16 MiB holds every call
 *   of B * H <= 256 heads at D = 128 and cap <= 4096 (the 7B-shaped layer at
 *   batch 8).
 *   Sharing: every call on one GPU uses that GPU's one array, which keeps the
 *   last call's contents; calls that overlap in time on one GPU (other streams,
 *   other threads) race on it and must be serialised by the caller.  Nothing in
 *   it needs to start at zero: each split writes its partial before the merge
 *   reads it.
 */
#define DAKV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
size_t dakv_decode_attn_static_noalloc_scratch_bytes(int B, int H, int cap, int D,
                                                     int num_splits);
int dakv_decode_attn_static_noalloc(const float* q, const void* k_cache, const void* v_cache,
                                    const int32_t* mask, const int32_t* valid_len, int B, int H,
                                    int cap, int D, float scale, float* out, float* lse,
                                    int num_splits, int32_t* err_flag, void* stream);

/* ========================================================================
 * Paged KV cache   ([PyPTO] section 3, tensor contract and gather semantics)
 *
 * key_cache bf16 [num_blocks, block_size, Hk, Dk], value_cache bf16
 * [num_blocks, block_size, Hv, Dv]; block_tables int32 [Q, table_cols];
 * seq_lens int32 [Q + 1] cumulative (seq_lens[0] = 0, non-decreasing; sequence
 * q has seq_lens[q+1] - seq_lens[q] tokens); seq_offset int32 [Q] (multiples of
 * block_size, >= 0) or NULL (all zero).  Token t of sequence q lives in
 * physical block block_tables[q, seq_offset[q]/block_size + t/block_size], slot
 * t % block_size.
 * ======================================================================== */

/*
 * gather_pa_kv_cache -- collect each sequence's paged rows into contiguous
 * outputs.  [PyPTO] 3.2: key_out[seq_lens[q] + t] = key_cache[physical block,
 * slot] and likewise for values; 3.3: shape constraints; 7: only cumulative
 * seq_lens.  A bit copy: the outputs equal the source rows bit for bit.
 *
 *   key_out    bf16 [total_tokens, Hk, Dk];  value_out bf16 [total_tokens, Hv, Dv]
 *   total_tokens  host copy of seq_lens[Q]
 *   err_flag   optional; a used block id outside [0, num_blocks) leaves that
 *              output row zero and sets DAKV_ERR_BLOCK_ID; inconsistent
 *              seq_lens set DAKV_ERR_SEQ_LENS (rows past total_tokens are never
 *              written)
 * Requires Hk*Dk*2 and Hv*Dv*2 to be multiples of 16; ENOTSUP when a token's
 * K plus V row exceeds 185344 bytes.
 */
int dakv_gather_pa_kv_cache(const void* key_cache, const void* value_cache, int num_blocks,
                            int block_size, int Hk, int Dk, int Hv, int Dv,
                            const int32_t* block_tables, int Q, int table_cols,
                            const int32_t* seq_lens, const int32_t* seq_offset,
                            int total_tokens, void* key_out, void* value_out,
                            int32_t* err_flag, void* stream);

/* Workspace bytes dakv_decode_attn_paged needs for sequences of at most
 * max_seq_len tokens. */
size_t dakv_decode_attn_paged_workspace_size(int B, int Hq, int D, int max_seq_len,
                                             int block_size);

/*
 * decode_attn_paged -- paged GQA decode attention: the masked-softmax decode of
 * decode_attn_static over the rows the block table yields (valid length = the
 * sequence length).  Query head h reads KV head h / (Hq / Hkv): several query
 * heads share one KV head ([NPU-LLM] closing part, GQA: several Q heads share
 * the same K/V tile), and its rows are read once for the whole group.
 *
 *   q            bf16 [B, Hq, D]
 *   key_cache    bf16 [num_blocks, block_size, Hkv, D]; value_cache likewise
 *   block_tables int32 [B, table_cols]; seq_lens int32 [B + 1] cumulative;
 *   seq_offset   int32 [B] or NULL
 *   max_seq_len  host upper bound of every sequence length (sizes the splits)
 *   out          fp32 [B, Hq, D];  lse fp32 [B, Hq] or NULL
 *   err_flag     optional; a bad block id excludes that block's rows and sets
 *                DAKV_ERR_BLOCK_ID; a sequence longer than max_seq_len or than
 *                its table is cut there and sets DAKV_ERR_SEQ_LENS
 * Supported: D = 128, block_size in {16, 32, 64, 128}, Hq / Hkv in {1, 2, 4, 8},
 * max_seq_len small enough for 256 splits (278528 tokens at block 16).
 */
int dakv_decode_attn_paged(const void* q, const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, int table_cols,
                           const int32_t* seq_lens, const int32_t* seq_offset, int B, int Hq,
                           int Hkv, int D, int num_blocks, int block_size, int max_seq_len,
                           float scale, float* out, float* lse, void* workspace,
                           size_t workspace_bytes, int num_splits, int32_t* err_flag,
                           void* stream);

/*
 * FP4 KV cache (static layout): the FP8 cache's scheme with E2M1 codes (OCP
 * microscaling FP4: sign, 2 exponent bits with bias 1, 1 mantissa bit;
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte with element 2i in the low
 * four bits: codes uint8 [B, H, cap, D / 2], scales fp32 [B, H, cap] per K and V;
 * a row's scale is 2^e with e the smallest integer for which max|x| <= 6 * 2^e,
 * codes round x / 2^e to the nearest value, ties to the even code, zeros to +0
 * ([FlashMLA], the decode kernel reads FP8 or FP4 and dequantises it).
 *
 * kv_append_fp4 -- as kv_append_fp8 (new rows finite; D a multiple of 16, <= 256).
 * decode_attn_static_fp4 -- as decode_attn_static_fp8 over the FP4 cache (same
 * workspace; D in {64, 128}).
 */
int dakv_kv_append_fp4(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                       const void* k_new, const void* v_new, const int32_t* write_pos,
                       int32_t* mask, int B, int H, int cap, int D, int32_t* err_flag,
                       void* stream);
int dakv_decode_attn_static_fp4(const float* q, const void* k_codes, const void* v_codes,
                                const float* k_scale, const float* v_scale, const int32_t* mask,
                                const int32_t* valid_len, int B, int H, int cap, int D,
                                float scale, float* out, float* lse, void* workspace,
                                size_t workspace_bytes, int num_splits, int32_t* err_flag,
                                void* stream);

/*
 * decode_step_static_fp4 -- kv_append_fp4 followed by decode_attn_static_fp4, in
 * one split pass, as decode_step_static_fp8 is for the FP8 cache (same results as
 * the two calls).  k_codes, v_codes uint8 [B, H, cap, D / 2]; other arguments as
 * decode_step_static_fp8.  Supported: D in {64, 128}, cap <= 65536.
 */
int dakv_decode_step_static_fp4(const float* q, void* k_codes, void* v_codes, float* k_scale,
                                float* v_scale, const void* k_new, const void* v_new,
                                const int32_t* write_pos, int32_t* mask, const int32_t* valid_len,
                                int B, int H, int cap, int D, float scale, float* out, float* lse,
                                void* workspace, size_t workspace_bytes, int num_splits,
                                int32_t* err_flag, void* stream);

/*
 * FP8 paged pool (the FP8 cache above in the paged layout): codes uint8
 * [num_blocks, block_size, Hkv, D] and one fp32 power-of-two scale per (block,
 * slot, KV head) [num_blocks, block_size, Hkv] for K and for V; values decode to
 * code * scale.
 *
 * paged_append_fp8 -- quantise each sequence's new token (k_new, v_new bf16
 * [B, Hkv, D], finite) into its last position t = len_b - 1 (len_b =
 * seq_lens[b+1] - seq_lens[b], counting the new token), at block
 * block_tables[b][seq_offset[b] / block_size + t / block_size], slot
 * t % block_size: the paged address resolution of decode_attn_paged and the
 * append-at-write-position of kv_append ([NPU-LLM] Part 1; [PyPTO] 3.2).  A
 * sequence of length 0 or an entry past its table sets DAKV_ERR_SEQ_LENS, a bad
 * block id DAKV_ERR_BLOCK_ID; that sequence is skipped.  D <= 256.
 */
int dakv_paged_append_fp8(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                          const void* k_new, const void* v_new, const int32_t* block_tables,
                          int table_cols, const int32_t* seq_lens, const int32_t* seq_offset,
                          int B, int Hkv, int D, int num_blocks, int block_size,
                          int32_t* err_flag, void* stream);

/*
 * decode_attn_paged_fp8 -- decode_attn_paged over the FP8 pool: each row's K
 * scale multiplies its scores, its V scale its weight in the output.  Arguments
 * and workspace (dakv_decode_attn_paged_workspace_size) as decode_attn_paged.
 * Supported: D = 128, Hkv dividing 16, Hq / Hkv in {1, 2, 4, 8}, block_size in
 * {16, 32, 64, 128}.
 */
int dakv_decode_attn_paged_fp8(const void* q, const void* k_codes, const void* v_codes,
                               const float* k_scale, const float* v_scale,
                               const int32_t* block_tables, int table_cols,
                               const int32_t* seq_lens, const int32_t* seq_offset, int B,
                               int Hq, int Hkv, int D, int num_blocks, int block_size,
                               int max_seq_len, float scale, float* out, float* lse,
                               void* workspace, size_t workspace_bytes, int num_splits,
                               int32_t* err_flag, void* stream);

/*
 * FP4 paged pool (the FP4 cache above in the paged layout): packed E2M1 codes
 * uint8 [num_blocks, block_size, Hkv, D / 2] (element 2i in the low four bits)
 * and the scales of the FP8 pool.
 *
 * paged_append_fp4 -- as paged_append_fp8 with E2M1 codes; D a multiple of 16,
 * up to 256.
 * decode_attn_paged_fp4 -- as decode_attn_paged_fp8 over the E2M1 codes; same
 * arguments, workspace and supported shapes.
 */
int dakv_paged_append_fp4(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                          const void* k_new, const void* v_new, const int32_t* block_tables,
                          int table_cols, const int32_t* seq_lens, const int32_t* seq_offset,
                          int B, int Hkv, int D, int num_blocks, int block_size,
                          int32_t* err_flag, void* stream);
int dakv_decode_attn_paged_fp4(const void* q, const void* k_codes, const void* v_codes,
                               const float* k_scale, const float* v_scale,
                               const int32_t* block_tables, int table_cols,
                               const int32_t* seq_lens, const int32_t* seq_offset, int B,
                               int Hq, int Hkv, int D, int num_blocks, int block_size,
                               int max_seq_len, float scale, float* out, float* lse,
                               void* workspace, size_t workspace_bytes, int num_splits,
                               int32_t* err_flag, void* stream);

/* ========================================================================
 * Top-k sparse MLA-style decode   ([FlashMLA] "Mathematical formulation")
 * ======================================================================== */

/* Workspace bytes dakv_sparse_topk_decode_attn needs. */
size_t dakv_sparse_topk_decode_attn_workspace_size(int B, int Hq, int d_qk, int d_v,
                                                   int topk);

/*
 * sparse_topk_decode_attn -- every query head of sequence b attends the topk
 * rows of its latent cache named by indices[b]:
 *   G = kv[b][indices[b]]             [topk, d_qk]   (duplicates count twice)
 *   S = softmax(sm_scale * q[b] G^T)  [Hq, topk]
 *   out[b] = S G[:, :d_v]             [Hq, d_v]
 * [FlashMLA] "Mathematical formulation"; "Course of computation": blocks of
 * the index list, online softmax with running max and sum-exp (the page rounds
 * S to bf16 before S.V; here S enters as a bf16 high part plus a bf16 low part,
 * which keeps the result within the stated tolerance).
 *
 *   q        bf16 [B, Hq, d_qk];  kv bf16 [B, s_kv, d_qk];  indices int32 [B, topk]
 *   out      fp32 [B, Hq, d_v];   lse fp32 [B, Hq] or NULL (natural log of the
 *            sum of exp(sm_scale * scores))
 *   err_flag optional; an index outside [0, s_kv) is skipped and sets
 *            DAKV_ERR_SPARSE_INDEX
 * Supported: d_qk = 576, d_v = 512, Hq a multiple of 16 up to 128, and s_kv with
 * s_kv * d_qk * 2 below 2^31 (a sequence's rows are addressed with 32-bit byte
 * offsets); otherwise DAKV_ENOTSUP.
 */
int dakv_sparse_topk_decode_attn(const void* q, const void* kv, const int32_t* indices,
                                 int B, int Hq, int s_kv, int d_qk, int d_v, int topk,
                                 float sm_scale, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, int32_t* err_flag, void* stream);

/*
 * sparse_topk_attn -- the same kernel for several q-tokens per sequence, each
 * with its own index list into the sequence's one latent cache; q-tokens are
 * computed separately ([FlashMLA] "Reminder of the algorithm": the kernel takes
 * some q-tokens and kv-tokens and an index table; "Mathematical formulation":
 * different q-tokens are always processed separately).  Token t of sequence b:
 *   out[b, t] = sparse_topk_decode_attn of q[b, t] over kv[b] with indices[b, t]
 *
 *   q        bf16 [B, s_q, Hq, d_qk];  kv bf16 [B, s_kv, d_qk];
 *   indices  int32 [B, s_q, topk]
 *   out      fp32 [B, s_q, Hq, d_v];   lse fp32 [B, s_q, Hq] or NULL
 *   workspace as dakv_sparse_topk_decode_attn_workspace_size(B * s_q, ...)
 * Supported as dakv_sparse_topk_decode_attn, and B * s_q <= 2^24.  s_q = 1 is
 * dakv_sparse_topk_decode_attn.
 */
int dakv_sparse_topk_attn(const void* q, const void* kv, const int32_t* indices, int B,
                          int s_q, int Hq, int s_kv, int d_qk, int d_v, int topk,
                          float sm_scale, float* out, float* lse, void* workspace,
                          size_t workspace_bytes, int32_t* err_flag, void* stream);

/*
 * FP8 latent cache of the sparse kernel ([FlashMLA] section on VECTOR cores per
 * CUBE core, item 2: the decode kernel reads the KV cache in FP8 and dequantises
 * it to bfloat16 for the matrix unit; section on the decoding KV-cache layout: a
 * token's values and its scale go together).  Codes uint8 [B, s_kv, d_qk] in the
 * E4M3 format and scale rule of the FP8 KV cache above, one fp32 scale per latent
 * row (all d_qk columns, value and rotary alike) in scale [B, s_kv].
 *
 * latent_append_fp8 -- quantise each sequence's new latent row (bf16 [B, d_qk],
 * finite values) and store codes and scale at row write_pos[b] (int32 [B]
 * device).  A position outside [0, s_kv) sets DAKV_ERR_WRITE_POS and skips that
 * sequence.  d_qk up to 576.
 */
int dakv_latent_append_fp8(void* codes, float* scale, const void* new_rows,
                           const int32_t* write_pos, int B, int s_kv, int d_qk,
                           int32_t* err_flag, void* stream);

/*
 * sparse_topk_attn_fp8 -- dakv_sparse_topk_attn over the FP8 latent cache: the
 * rows named by the indices are dequantised (code value times row scale, exact in
 * bf16) and attended as bf16 rows are.  Arguments as dakv_sparse_topk_attn with
 * kv replaced by codes (uint8 [B, s_kv, d_qk], 16-byte aligned) and scale (fp32
 * [B, s_kv]); same workspace size, supported shapes and error behaviour.
 */
int dakv_sparse_topk_attn_fp8(const void* q, const void* codes, const float* scale,
                              const int32_t* indices, int B, int s_q, int Hq, int s_kv, int d_qk,
                              int d_v, int topk, float sm_scale, float* out, float* lse,
                              void* workspace, size_t workspace_bytes, int32_t* err_flag,
                              void* stream);

/*
 * FP4 latent cache of the sparse kernel (same passages: the decode kernel reads
 * the KV cache in FP8 or FP4).  Codes uint8 [B, s_kv, d_qk / 2] in the E2M1
 * format, packing and scale rule of the FP4 KV cache above (element 2i in the low
 * four bits), one fp32 scale per latent row in scale [B, s_kv].
 *
 * latent_append_fp4 -- as latent_append_fp8 in E2M1; d_qk even, up to 576.
 * sparse_topk_attn_fp4 -- as sparse_topk_attn_fp8 over the E2M1 codes (uint8
 * [B, s_kv, d_qk / 2], 16-byte aligned).
 */
int dakv_latent_append_fp4(void* codes, float* scale, const void* new_rows,
                           const int32_t* write_pos, int B, int s_kv, int d_qk,
                           int32_t* err_flag, void* stream);
int dakv_sparse_topk_attn_fp4(const void* q, const void* codes, const float* scale,
                              const int32_t* indices, int B, int s_q, int Hq, int s_kv, int d_qk,
                              int d_v, int topk, float sm_scale, float* out, float* lse,
                              void* workspace, size_t workspace_bytes, int32_t* err_flag,
                              void* stream);

/* ========================================================================
 * Host validators (HOST pointers; no GPU needed).  [PyPTO] 3.3 and 5.1: the
 * index tensors are host-ready and are checked on the host before a call.
 * Return DAKV_OK, DAKV_EINVAL (null/size) or DAKV_ERANGE (bad content).
 * ======================================================================== */

/* Cumulative seq_lens [Q+1] from 0, non-decreasing; seq_offset (or NULL) >= 0
 * and divisible by block_size; every used table entry inside [0, num_blocks);
 * used columns inside the table. */
int dakv_validate_paged(const int32_t* block_tables, int Q, int table_cols,
                        const int32_t* seq_lens, const int32_t* seq_offset, int num_blocks,
                        int block_size);

/* Every index inside [0, s_kv). */
int dakv_validate_sparse(const int32_t* indices, int B, int topk, int s_kv);

/* Every value inside [lo, hi] (append positions: [0, cap-1]; valid lengths:
 * [0, cap]). */
int dakv_validate_range(const int32_t* values, int n, int lo, int hi);

#ifdef __cplusplus
}
#endif

#endif /* DAKV_H */
