// Bandwidth-bound copies: kv_append (one new row per sequence into the static
// buffer) and gather_pa_kv_cache (paged rows -> contiguous rows).  Both are bit
// copies in 16-byte units; every global access is a 128-bit load or store and
// consecutive lanes touch consecutive 16-byte pieces of a row.
#include "device.hpp"
#include "launch.hpp"

namespace dakv {

typedef uint32_t gx_u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// kv_append: the new token's K and V rows go to row write_pos[b] of every head
// (the NPU runtime's cache update writes just this row and bumps the counter).
// Grid: (B, ceil(H*D/8 / 256)); thread -> one 16-byte piece of K and of V.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
kv_append_kernel(uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                 const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                 const int32_t* __restrict__ write_pos, int32_t* __restrict__ mask, int H,
                 int cap, int D, int32_t* err_flag) {
  const int b = blockIdx.x;
  const int piece = blockIdx.y * blockDim.x + threadIdx.x;  // 8 bf16 per piece
  const int per_head = D / 8;
  const int pos = write_pos[b];
  if (pos < 0 || pos >= cap) {
    if (blockIdx.y == 0 && threadIdx.x == 0) raise_flag(err_flag, 2);
    return;
  }
  if (piece < H * per_head) {
    const int h = piece / per_head;
    const int within = piece - h * per_head;
    const size_t src = (size_t)b * H * D + (size_t)piece * 8;
    const size_t dst = (((size_t)b * H + h) * cap + pos) * D + (size_t)within * 8;
    const uint4 kv = load16(k_new + src);
    const uint4 vv = load16(v_new + src);
    store16(k_cache + dst, kv);
    store16(v_cache + dst, vv);
  }
  if (mask && blockIdx.y == 0 && threadIdx.x == 0) mask[(size_t)b * cap + pos] = 1;
}

hipError_t launch_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                            const int32_t* write_pos, int32_t* mask, int B, int H, int cap,
                            int D, int32_t* err_flag, hipStream_t stream) {
  const int pieces = H * (D / 8);
  dim3 grid(B, (pieces + 255) / 256);
  hipLaunchKernelGGL(kv_append_kernel, grid, dim3(256), 0, stream,
                     static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                     static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                     write_pos, mask, H, cap, D, err_flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// copy_kvcache: the prefill model's valid rows [0, len_b) of every (tensor,
// sequence, head) go to the same rows of the generate model's buffer.  For one
// (tensor, sequence, head) those rows are len_b * row_bytes contiguous bytes in
// both buffers (only the capacity strides differ), so the work is a batch of
// contiguous copies; a workgroup moves one kCopyBytes chunk of one of them with
// all of its loads issued before the first store (non-temporal loads; stores written
// through, kStoreThrough).
// Grid: n * B * H * chunks, chunk fastest; chunks past the copied length exit.
// ---------------------------------------------------------------------------
// 2 loads of 16 bytes per thread (8 KiB per workgroup): the 64-tensor, 1 GiB
// hand-over measured 163.9 us per call, against 163.8 / 165.4 / 170.7 us with 1 / 4 /
// 8 loads per thread (with non-temporal stores 4 loads were best: 187.8 against 190.9 /
// 189.9 / 190.1 / 192.9 us with 2 / 3 / 6 / 8).
constexpr int kCopyLoads = 2;                        // 16-byte loads per thread
constexpr int kCopyBytes = 256 * kCopyLoads * 16;    // 8 KiB per workgroup

struct CopyTable {
  const uint8_t* src[kCopyMaxTensors];
  uint8_t* dst[kCopyMaxTensors];
};

__device__ __forceinline__ int copy_len(const int32_t* lengths, int b, int lim, int32_t* err_flag,
                                        bool report) {
  int L = lengths[b];
  if (L < 0 || L > lim) {
    if (report) raise_flag(err_flag, 32);
    L = L < 0 ? 0 : lim;
  }
  return L;
}

__global__ void __launch_bounds__(256)
copy_kvcache_kernel(CopyTable t, int BH, int H, int src_cap, int dst_cap, int row_bytes,
                    int chunks, const int32_t* __restrict__ lengths, int32_t* err_flag) {
  const int c = blockIdx.x % chunks;
  const int rest = blockIdx.x / chunks;
  const int bh = rest % BH;
  const int i = rest / BH;
  const int b = bh / H;
  const int lim = min(src_cap, dst_cap);
  const int L = copy_len(lengths, b, lim, err_flag,
                         i == 0 && bh - b * H == 0 && c == 0 && threadIdx.x == 0);
  const size_t bytes = (size_t)L * row_bytes;
  const size_t start = (size_t)c * kCopyBytes;
  if (start >= bytes) return;
  const int n16 = (int)(min((size_t)kCopyBytes, bytes - start) / 16);
  const uint8_t* src = t.src[i] + (size_t)bh * src_cap * row_bytes + start;
  uint8_t* dst = t.dst[i] + (size_t)bh * dst_cap * row_bytes + start;
  const __amdgpu_buffer_rsrc_t dr = __builtin_amdgcn_make_buffer_rsrc(dst, (short)0, n16 * 16,
                                                                      0x00020000);
  gx_u32x4 v[kCopyLoads];
#pragma unroll
  for (int k = 0; k < kCopyLoads; ++k) {
    const int j = min((int)threadIdx.x + 256 * k, n16 - 1);
    v[k] = __builtin_nontemporal_load(reinterpret_cast<const gx_u32x4*>(src) + j);
  }
#pragma unroll
  for (int k = 0; k < kCopyLoads; ++k) {
    const int j = (int)threadIdx.x + 256 * k;
    if (j < n16) store16_through(dr, j * 16, make_uint4(v[k][0], v[k][1], v[k][2], v[k][3]));
  }
}

// The generate model's mask after the copy: 1 for the copied rows, 0 after.
__global__ void __launch_bounds__(256)
copy_mask_kernel(int32_t* __restrict__ mask, const int32_t* __restrict__ lengths, int cap,
                 int lim) {
  const int b = blockIdx.y;
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= cap) return;
  const int L = copy_len(lengths, b, lim, nullptr, false);
  mask[(size_t)b * cap + r] = r < L ? 1 : 0;
}

// Roll-back: rows at and after new_len[b] stop counting.
__global__ void __launch_bounds__(256)
trim_kernel(int32_t* __restrict__ mask, const int32_t* __restrict__ new_len, int cap,
            int32_t* err_flag) {
  const int b = blockIdx.y;
  const int r = blockIdx.x * 256 + threadIdx.x;
  const int L = copy_len(new_len, b, cap, err_flag, blockIdx.x == 0 && threadIdx.x == 0);
  if (r < cap && r >= L) mask[(size_t)b * cap + r] = 0;
}

hipError_t launch_copy_kvcache(const void* const* src, void* const* dst, int n, int B, int H,
                               int src_cap, int dst_cap, int D, const int32_t* lengths,
                               int32_t* mask, int32_t* err_flag, hipStream_t stream) {
  CopyTable t;
  for (int i = 0; i < n; ++i) {
    t.src[i] = static_cast<const uint8_t*>(src[i]);
    t.dst[i] = static_cast<uint8_t*>(dst[i]);
  }
  const int row_bytes = D * 2;
  const int lim = src_cap < dst_cap ? src_cap : dst_cap;
  const long long span = (long long)lim * row_bytes;
  const int chunks = (int)((span + kCopyBytes - 1) / kCopyBytes);
  const long long grid = (long long)n * B * H * chunks;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (grid > 0)
    hipLaunchKernelGGL(copy_kvcache_kernel, dim3((unsigned)grid), dim3(256), 0, stream, t, B * H,
                       H, src_cap, dst_cap, row_bytes, chunks, lengths, err_flag);
  if (mask)
    hipLaunchKernelGGL(copy_mask_kernel, dim3((dst_cap + 255) / 256, B), dim3(256), 0, stream,
                       mask, lengths, dst_cap, lim);
  return hipGetLastError();
}

hipError_t launch_trim_kvcache(int32_t* mask, const int32_t* new_len, int B, int cap,
                               int32_t* err_flag, hipStream_t stream) {
  hipLaunchKernelGGL(trim_kernel, dim3((cap + 255) / 256, B), dim3(256), 0, stream, mask, new_len,
                     cap, err_flag);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// gather_pa_kv_cache.  A workgroup owns kGatherTok consecutive OUTPUT rows, so
// every output byte is written exactly once with no atomics and the work is
// balanced whatever the sequence lengths are.  Phase 1 resolves each output row
// to its source row: a binary search of the cumulative seq_lens (staged in LDS
// when they fit) and one block-table read.  Phase 2 copies the workgroup's rows
// as one flat list of 16-byte pieces (each token's K pieces, then its V pieces):
// every thread issues kGatherSlots loads before its first store, consecutive
// threads touch consecutive pieces of a row, and there is no branch per load
// (pieces past the end re-read the last piece and are not stored; rows with a
// bad block id are written as zeros).  Loads are non-temporal (each byte moves
// once); stores are written through (kStoreThrough), so the output leaves no dirty
// lines in the L2s.
// ---------------------------------------------------------------------------
// A workgroup takes 6 tokens: at 4 KiB per token (K + V, 8 heads x 128 dims) that
// is 6 loads per thread, all in flight before the first store, in a small kernel
// that keeps several workgroups on every CU, so that the two dependent reads each
// workgroup starts with (the lengths, then the block table) overlap other
// workgroups' copies.  Measured at batch 32 x U{1..4096} (494 MB), stores written
// through: 6 tokens 76.1 us per call; 2: 84.9; 3: 77.6; 4: 77.4; 5: 76.8; 8: 77.5;
// 12: 76.9.  (With non-temporal stores 3 tokens were best: 87.0 us; 2: 90.0; 4:
// 90.6; 5: 89.6; 8: 92.9; 16: 96.7; 32 tokens, one round of 32 loads per thread,
// 294 VGPRs, one wave per SIMD: 95.1.)
constexpr int kGatherTok = 6;
constexpr int kGatherSlots = 6;
constexpr int kGatherLensLds = 4096;



__global__ void __launch_bounds__(256)
gather_kernel(const uint8_t* __restrict__ key_cache, const uint8_t* __restrict__ value_cache,
              int num_blocks, int block_size, int k_pieces, int v_pieces, uint32_t piece_magic,
              const int32_t* __restrict__ block_tables, int Q, int table_cols,
              const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ seq_offset,
              int total_tokens, uint8_t* __restrict__ key_out, uint8_t* __restrict__ value_out,
              int32_t* err_flag) {
  __shared__ long long src_row[kGatherTok];
  __shared__ int lens[kGatherLensLds];
  const int tok0 = blockIdx.x * kGatherTok;
  const int ntok = min(kGatherTok, total_tokens - tok0);
  const int tid = threadIdx.x;
  const bool staged = Q + 1 <= kGatherLensLds;
  if (staged) {
    for (int i = tid; i <= Q; i += 256) lens[i] = seq_lens[i];
    __syncthreads();
  }
  if (tid < ntok) {
    const int o = tok0 + tid;
    long long src = -1;
    // last q with seq_lens[q] <= o
    int lo = 0, hi = Q - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      const int v = staged ? lens[mid] : seq_lens[mid];
      if (v <= o) lo = mid; else hi = mid - 1;
    }
    const int q = lo;
    const int start = staged ? lens[q] : seq_lens[q];
    const int end = staged ? lens[q + 1] : seq_lens[q + 1];
    const int t = o - start;
    const int off = seq_offset ? seq_offset[q] : 0;
    if (t < 0 || t >= end - start || off < 0 || off % block_size != 0) {
      raise_flag(err_flag, 8);
    } else {
      const int col = off / block_size + t / block_size;
      if (col >= table_cols) {
        raise_flag(err_flag, 8);
      } else {
        const int phys = block_tables[(size_t)q * table_cols + col];
        if (phys < 0 || phys >= num_blocks) raise_flag(err_flag, 1);
        else src = (long long)phys * block_size + (t % block_size);
      }
    }
    src_row[tid] = src;
  }
  __syncthreads();
  const int P = k_pieces + v_pieces;
  const int N = ntok * P;
  const size_t kb = (size_t)k_pieces * 16, vb = (size_t)v_pieces * 16;
  // the workgroup's output rows of each output, stored through (sc1)
  const __amdgpu_buffer_rsrc_t rko = __builtin_amdgcn_make_buffer_rsrc(
      key_out + (size_t)tok0 * kb, (short)0, (int)(ntok * kb), 0x00020000);
  const __amdgpu_buffer_rsrc_t rvo = __builtin_amdgcn_make_buffer_rsrc(
      value_out + (size_t)tok0 * vb, (short)0, (int)(ntok * vb), 0x00020000);
  for (int base = 0; base < N; base += 256 * kGatherSlots) {
    gx_u32x4 r[kGatherSlots];
    int doff[kGatherSlots];
    bool dk[kGatherSlots];
#pragma unroll
    for (int s = 0; s < kGatherSlots; ++s) {
      const int i = min(base + s * 256 + tid, N - 1);
      const int j = (int)__umulhi((uint32_t)i, piece_magic);  // i / P
      const int pc = i - j * P;
      const long long sr = src_row[j];
      const size_t row = sr >= 0 ? (size_t)sr : 0;
      const bool is_k = pc < k_pieces;
      const uint8_t* src = is_k ? key_cache + row * kb + (size_t)pc * 16
                                : value_cache + row * vb + (size_t)(pc - k_pieces) * 16;
      dk[s] = is_k;
      doff[s] = is_k ? (int)(j * kb) + pc * 16 : (int)(j * vb) + (pc - k_pieces) * 16;
      const gx_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const gx_u32x4*>(src));
      r[s] = sr >= 0 ? v : gx_u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < kGatherSlots; ++s)
      if (base + s * 256 + tid < N) {
        const uint4 w = make_uint4(r[s][0], r[s][1], r[s][2], r[s][3]);
        if (dk[s]) store16_through(rko, doff[s], w);
        else store16_through(rvo, doff[s], w);
      }
  }
}

// Longest token row (K plus V, in 16-byte pieces) the kernel takes: the
// reciprocal multiply that splits piece indices is exact for i < kGatherTok * P
// while kGatherTok * P^2 < 2^32.
constexpr int kGatherMaxPieces = 11584;
static_assert((unsigned long long)kGatherTok * kGatherMaxPieces * kGatherMaxPieces < (1ull << 32),
              "piece split exact");

hipError_t launch_gather(const void* key_cache, const void* value_cache, int num_blocks,
                         int block_size, int k_row_bytes, int v_row_bytes,
                         const int32_t* block_tables, int Q, int table_cols,
                         const int32_t* seq_lens, const int32_t* seq_offset, int total_tokens,
                         void* key_out, void* value_out, int32_t* err_flag, hipStream_t stream) {
  if (total_tokens <= 0) return hipSuccess;
  const int kp = k_row_bytes / 16, vp = v_row_bytes / 16;
  const int P = kp + vp;
  if (P > kGatherMaxPieces) return hipErrorNotSupported;
  // ceil(2^32 / P): exact i / P for every i < kGatherTok * P when P <= kGatherMaxPieces
  const uint32_t magic = (uint32_t)(((1ull << 32) + (uint64_t)P - 1) / (uint64_t)P);
  const int grid = (total_tokens + kGatherTok - 1) / kGatherTok;
  hipLaunchKernelGGL(gather_kernel, dim3(grid), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(key_cache),
                     static_cast<const uint8_t*>(value_cache), num_blocks, block_size, kp, vp,
                     magic, block_tables, Q, table_cols, seq_lens, seq_offset, total_tokens,
                     static_cast<uint8_t*>(key_out), static_cast<uint8_t*>(value_out), err_flag);
  return hipGetLastError();
}

}  // namespace dakv
