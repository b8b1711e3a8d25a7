// Bandwidth-bound copies: kv_append (one new row per sequence into the static
// buffer) and gather_pa_kv_cache (paged rows -> contiguous rows).  Both are bit
// copies in 16-byte units; every global access is a 128-bit load or store and
// consecutive lanes touch consecutive 16-byte pieces of a row.
#include "device.hpp"
#include "launch.hpp"

namespace dakv {

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
// gather_pa_kv_cache.  A workgroup owns kGatherTok consecutive OUTPUT rows, so
// every output byte is written exactly once with no atomics and the work is
// balanced whatever the sequence lengths are.  Phase 1 resolves each output row
// to its source row (binary search of the cumulative seq_lens, then the block
// table); phase 2 streams the rows, one wave per row, 16 bytes per lane.
// ---------------------------------------------------------------------------
constexpr int kGatherTok = 32;
constexpr int kGatherUnroll = 4;

__device__ __forceinline__ void copy_rows(const uint8_t* __restrict__ ksrc,
                                          uint8_t* __restrict__ kdst, int k_pieces,
                                          const uint8_t* __restrict__ vsrc,
                                          uint8_t* __restrict__ vdst, int v_pieces,
                                          bool valid, int lane) {
  const int pieces = k_pieces > v_pieces ? k_pieces : v_pieces;
  for (int base = 0; base < pieces; base += 64 * kGatherUnroll) {
    uint4 kr[kGatherUnroll], vr[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int p = base + u * 64 + lane;
      kr[u] = make_uint4(0, 0, 0, 0);
      vr[u] = make_uint4(0, 0, 0, 0);
      if (valid && p < k_pieces) kr[u] = load16(ksrc + (size_t)p * 16);
      if (valid && p < v_pieces) vr[u] = load16(vsrc + (size_t)p * 16);
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int p = base + u * 64 + lane;
      if (p < k_pieces) store16(kdst + (size_t)p * 16, kr[u]);
      if (p < v_pieces) store16(vdst + (size_t)p * 16, vr[u]);
    }
  }
}

__global__ void __launch_bounds__(256)
gather_kernel(const uint8_t* __restrict__ key_cache, const uint8_t* __restrict__ value_cache,
              int num_blocks, int block_size, int k_row_bytes, int v_row_bytes,
              const int32_t* __restrict__ block_tables, int Q, int table_cols,
              const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ seq_offset,
              int total_tokens, uint8_t* __restrict__ key_out, uint8_t* __restrict__ value_out,
              int32_t* err_flag) {
  __shared__ long long src_row[kGatherTok];
  const int tok0 = blockIdx.x * kGatherTok;
  const int tid = threadIdx.x;
  if (tid < kGatherTok) {
    const int o = tok0 + tid;
    long long src = -1;
    if (o < total_tokens) {
      // last q with seq_lens[q] <= o
      int lo = 0, hi = Q - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seq_lens[mid] <= o) lo = mid; else hi = mid - 1;
      }
      const int q = lo;
      const int t = o - seq_lens[q];
      const int len = seq_lens[q + 1] - seq_lens[q];
      const int off = seq_offset ? seq_offset[q] : 0;
      if (t < 0 || t >= len || off < 0 || off % block_size != 0) {
        raise_flag(err_flag, 8);
      } else {
        const int col = off / block_size + t / block_size;
        if (col >= table_cols) {
          raise_flag(err_flag, 8);
        } else {
          const int phys = block_tables[(size_t)q * table_cols + col];
          if (phys < 0 || phys >= num_blocks) {
            raise_flag(err_flag, 1);
          } else {
            src = (long long)phys * block_size + (t % block_size);
          }
        }
      }
    }
    src_row[tid] = src;
  }
  __syncthreads();
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int k_pieces = k_row_bytes / 16;
  const int v_pieces = v_row_bytes / 16;
  for (int j = wave; j < kGatherTok; j += 4) {
    const int o = tok0 + j;
    if (o >= total_tokens) break;
    const long long s = src_row[j];
    const bool valid = s >= 0;
    const long long sr = valid ? s : 0;
    copy_rows(key_cache + sr * k_row_bytes, key_out + (size_t)o * k_row_bytes, k_pieces,
              value_cache + sr * v_row_bytes, value_out + (size_t)o * v_row_bytes, v_pieces,
              valid, lane);
  }
}

hipError_t launch_gather(const void* key_cache, const void* value_cache, int num_blocks,
                         int block_size, int k_row_bytes, int v_row_bytes,
                         const int32_t* block_tables, int Q, int table_cols,
                         const int32_t* seq_lens, const int32_t* seq_offset, int total_tokens,
                         void* key_out, void* value_out, int32_t* err_flag, hipStream_t stream) {
  if (total_tokens <= 0) return hipSuccess;
  const int grid = (total_tokens + kGatherTok - 1) / kGatherTok;
  hipLaunchKernelGGL(gather_kernel, dim3(grid), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(key_cache),
                     static_cast<const uint8_t*>(value_cache), num_blocks, block_size,
                     k_row_bytes, v_row_bytes, block_tables, Q, table_cols, seq_lens,
                     seq_offset, total_tokens, static_cast<uint8_t*>(key_out),
                     static_cast<uint8_t*>(value_out), err_flag);
  return hipGetLastError();
}

}  // namespace dakv
