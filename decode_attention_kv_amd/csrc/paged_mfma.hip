// Paged GQA decode on the matrix cores, for 2, 4 or a multiple of 8 KV heads.
//
// Work split: a workgroup (8 waves) works on a group of GH = min(Hkv, 8) KV heads
// of one sequence at a time; wave w serves KV head w % GH of the group and 16 GH of the 128
// output dims (part w / GH) of its G query heads.  The group's GH x 256 bytes of
// each token row (K, and likewise V) are contiguous in the pool -- a whole token
// row at Hkv <= 8, read at once, which keeps the HBM accesses of a row together
// (the same rows split over four workgroups of two heads each streamed at 3 TB/s).
// The workgroup streams 16-token tiles with coalesced 16-byte non-temporal loads
// into registers, PmShape::Ahead tiles ahead, and writes each arriving tile into one of
// two LDS tiles for the matrix cores.  The
// loads go through a buffer resource that spans exactly the tile's pool block:
// tokens past the split's end read past the resource and load zeros, and a block
// id outside the pool gives an empty resource, so no unused slot of the pool is
// ever read.
//
// Per tile and KV head (the grouped-query sharing of one K/V tile by several
// query heads, NPU article's closing section; online softmax as in its Flash SDPA
// passage):
//   * S^T[token, head] = K Q^T with v_mfma_f32_16x16x32_bf16: A = the 16 tokens'
//     K rows from LDS (lane: token lane % 16, dims 32 s + 8 (lane / 16)), B = Q^T
//     of the G query heads held in registers (columns G..15 zero), 4 k-steps.
//   * The C layout of S^T (lane: head lane % 16, tokens 4 (lane / 16) + i) is the
//     A layout of P for O = P V with v_mfma_f32_16x16x16_bf16, so each lane forms
//     its P operand from its own scores; P enters as bf16 hi + lo parts.
//   * V (the B operand: 4 tokens of one dim per lane) comes from LDS with the
//     transposing read ds_read_b64_tr_b16.
// LDS rows are 512 bytes; piece p (16 bytes) of token row t is stored at p XOR
// ((t % 16) << 1), which puts the 32 pieces of each half-wave operand read, and
// the 64 8-byte pieces of each transposing read, in distinct banks.
// The grid is persistent: as many workgroups as the device holds at once.  The
// 16-token tiles of all (sequence, head group) pairs, numbered sequence-major in
// LDS from the lengths, are cut into equal ranges, one per workgroup (a few per
// workgroup when the ranges would exceed a table span), so every workgroup streams
// about the same number of tiles and none is spent past a sequence's end.  The part
// of a range inside one (sequence, head group) is an item; the next item's table
// entries and query are loaded while the current one streams.  An item ends with
// the output (the whole of its sequence's group) or a partial, and
// piece_merge_kernel combines the partials of each query head.  A call whose
// sequences all fit one split of the plan takes whole (sequence, head group) pairs
// instead, and needs no merge.
#include "split_common.hpp"

namespace dakv {

namespace {

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

constexpr int kPmTile = 16;                           // tokens per tile
constexpr int kPmWaves = 8;
constexpr int kPmThreads = 64 * kPmWaves;
constexpr uint32_t kPmNoRow = 0x80000000u;            // a buffer offset past any block
constexpr int kPmMaxSeqs = 512;                       // sequences the split map holds
constexpr int kPmSplitsTarget = 2048;                 // splits of a call at full lengths
// The running max of a head moves only when a tile raises it by more than this
// (log2 units): the skip-scale of the FlashMLA article, so that most tiles neither
// rescale the output nor move the reference of the exponentials (which stay below
// 2^kPmRescale).
constexpr float kPmRescale = 8.0f;

// Tile geometry for a group of GH KV heads over a pool of Bits-bit elements (16:
// bf16; 8: E4M3 codes; 4: E2M1 codes, two per byte, each with a per-row scale).
// In LDS a tile is always bf16: token rows of RB bytes, K then V.  In the pool a
// token's row for the group is CRB bytes, a tile's K (or V) CH bytes, read by lane
// loads of LW bytes.
template <int GH, int Bits>
struct PmShape {
  static constexpr bool Coded = Bits < 16;
  static constexpr int RB = 256 * GH;                   // a token's K (or V) for the group
  static constexpr int Half = kPmTile * RB;             // a tile's K (or V)
  static constexpr int Buf = 2 * Half;
  static constexpr int CB = 128 * Bits / 8;             // pool bytes of one head's row
  static constexpr int CRB = GH * CB;
  static constexpr int CH = kPmTile * CRB;
  static constexpr int LW = CH / 512 >= 16 ? 16 : CH / 512;
  static constexpr int HalfLoads = CH / (512 * LW);     // lane loads of K (and V) codes
  static constexpr int Elems = LW * 8 / Bits;           // elements of one lane load
  // Scales of a coded pool: with two or more code loads per half (FP8 at 8 heads), one
  // load per half fetches the ScaleEntries (token row, head) entries the wave's code
  // loads touch and each lane takes its own with a cross-lane read; otherwise (E2M1:
  // one code load per half, where that saves no load but costs registers) every code
  // load has its own scale load.  Lane loads of a tile, per wave:
  static constexpr int ScaleEntries = HalfLoads * 64 * LW / CB;
  static constexpr bool SharedScales = Coded && HalfLoads >= 2;
  static constexpr int ScaleRegs = !Coded ? 1 : (SharedScales ? 2 : 2 * HalfLoads);
  static constexpr int Loads = 2 * HalfLoads + (!Coded ? 0 : (SharedScales ? 2 : 2 * HalfLoads));
  static constexpr int Ahead =                                  // tiles loaded ahead
      Coded ? (GH == 8 ? (Bits == 8 ? 3 : 6) : 4) : (GH == 8 ? 2 : 4);
  static constexpr int Blocks = 128 / 16 / (kPmWaves / GH);   // dim blocks of a wave
  static_assert(LW >= 4 && CH % (512 * LW) == 0, "whole lane loads per half tile");
  static_assert(CB % LW == 0, "a lane load stays inside one head's row");
  static_assert(!SharedScales || ScaleEntries <= 64, "one scale per lane");
};

typedef uint32_t pm_u32x2_t __attribute__((ext_vector_type(2)));

// one lane load of LW bytes (LW = 4, 8 or 16) into the low words of a u32x4
template <int LW>
__device__ __forceinline__ u32x4_t pm_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (LW == 16) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kLoadNonTemporal);
  } else if constexpr (LW == 8) {
    const pm_u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kLoadNonTemporal);
    return u32x4_t{v[0], v[1], 0u, 0u};
  } else {
    return u32x4_t{__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kLoadNonTemporal), 0u,
                   0u, 0u};
  }
}

// LW bytes of codes times the row's power-of-two scale -> bf16 pairs (exact: an
// E4M3 or E2M1 value times 2^e is a bf16 number); word i holds elements 2i, 2i + 1
template <int Bits, int LW>
__device__ __forceinline__ void pm_dequant(const u32x4_t& c, float sc,
                                           uint32_t (&w)[LW * 8 / Bits / 2]) {
#pragma unroll
  for (int i = 0; i < LW / 4; ++i) {
    if constexpr (Bits == 8) {
      w[2 * i] = __builtin_bit_cast(uint32_t,
                                    __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], sc, false));
      w[2 * i + 1] = __builtin_bit_cast(uint32_t,
                                        __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], sc, true));
    } else {
      w[4 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], sc, 0));
      w[4 * i + 1] =
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], sc, 1));
      w[4 * i + 2] =
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], sc, 2));
      w[4 * i + 3] =
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[i], sc, 3));
    }
  }
}

// s_waitcnt immediate waiting until at most n vector memory operations are
// outstanding (vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maximum)
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

constexpr int kWaitLgkm0Pm = 15 | (7 << 4) | (0 << 8) | (3 << 14);  // lgkmcnt(0) only

__device__ __forceinline__ int pm_slot(int p, int t) { return p ^ ((t & 15) << 1); }

__device__ __forceinline__ float pm_group4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float pm_group4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ short bf16_bits(__bf16 x) { return __builtin_bit_cast(short, x); }

}  // namespace

template <int Bits, int G, int GH>
__global__ void __launch_bounds__(kPmThreads)
paged_mfma_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ key_cache,
                  const uint8_t* __restrict__ value_cache, const float* __restrict__ k_scale,
                  const float* __restrict__ v_scale,
                  const int32_t* __restrict__ block_tables, int table_cols,
                  const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ seq_offset,
                  int B, int Hkv, int num_blocks, int block_size, int bs_log2, int max_len,
                  float scale_log2, int chunk, int max_splits, Workspace ws,
                  int32_t* __restrict__ nseg, float* __restrict__ out, float* __restrict__ lse,
                  int32_t* err_flag) {
  constexpr int D = 128;
  using S = PmShape<GH, Bits>;
  constexpr int NB = S::Blocks;
  constexpr int A = S::Ahead;
  constexpr int QB = GH * G * D * 2;             // a split's query: GH x G heads
  constexpr int QPieces = QB / 16;
  constexpr int QLoads = (QPieces + kPmThreads - 1) / kPmThreads;
  static_assert(G >= 1 && G <= 16, "query heads per KV head fit the 16 MFMA columns");
  __shared__ __attribute__((aligned(1024))) uint8_t tile0[S::Buf];
  __shared__ __attribute__((aligned(1024))) uint8_t tile1[S::Buf];
  __shared__ __attribute__((aligned(16))) uint8_t qbuf[2][QB];
  __shared__ int pref[kPmMaxSeqs + 1];   // work units (x head groups) before sequence b
  __shared__ int slen[kPmMaxSeqs];       // effective length of sequence b
  __shared__ int soff[kPmMaxSeqs];       // its table offset in blocks
  const int ngroups = Hkv / GH;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hw = wave % GH;     // KV head of the group this wave computes
  const int part = wave / GH;   // its part of the 128 output dims (NB blocks of 16)
  const int grp = lane >> 4;
  const int col16 = lane & 15;
  const int Hq = Hkv * G;
  const int bs_mask = block_size - 1;
  const uint32_t block_bytes = (uint32_t)block_size * Hkv * S::CB;   // pool bytes of a block
  const int block_rows = block_size * Hkv;                             // its (slot, head) rows
  const int W = (int)gridDim.x;

  // Work units numbered sequence-major, then head group: with ranges, the 16-token
  // tiles of every (sequence, head group) (an empty sequence counts one, so that a
  // workgroup writes its zeros); without, whole (sequence, head group) pairs.
  // Lengths, table offsets, and the prefix sum of the units.
  const bool ranged = chunk > 0;
  for (int b = threadIdx.x; b < B; b += kPmThreads) {
    int toff = 0;
    const int L = paged_len(seq_lens, seq_offset, b, block_size, table_cols, max_len, &toff,
                            err_flag, blockIdx.x == 0);
    slen[b] = L;
    soff[b] = toff;
    pref[b + 1] = ngroups * (!ranged ? 1 : (L > 0 ? (L + kPmTile - 1) / kPmTile : 1));
  }
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
      int v = b0 + lane < B ? pref[b0 + lane + 1] : 0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(v, off);
        if (lane >= off) v += u;
      }
      if (b0 + lane < B) pref[b0 + lane + 1] = carry + v;
      carry += __shfl(v, 63);
    }
    if (lane == 0) pref[0] = 0;
  }
  __syncthreads();
  const int total = pref[B];
  // Ranges: workgroup w takes the tiles [R k, R (k + 1)) for k = w, w + W, ..., with
  // R = the tiles of the call over the workgroups, so that every workgroup streams
  // about the same number of tiles whatever the mix of lengths (whole splits of a
  // fixed size left up to a split more on some workgroups: 96 against 90.4 tiles of
  // the mean at the batch-64 config).  R is at least chunk / 16 tiles, which bounds
  // the pieces of one (sequence, head group) by the splits of a chunk-sized plan
  // plus one, and at most 126 blocks, which keeps a piece's table entries within
  // two registers a lane.
  int R = 1;
  if (ranged) {
    R = (total + W - 1) / W;
    const int least = chunk / kPmTile;
    const int span = 126 * block_size / kPmTile;
    if (R < least) R = least;
    if (R > span) R = span;
  }
  if ((int)blockIdx.x * R >= total) return;

  // One item: sequence b, head group hg, rows [r0, r1), piece `split` of the n of
  // its (sequence, head group) -- with ranges the part of a range inside one
  // (sequence, head group), else a whole one (n = 1).  `next` is this workgroup's
  // next item.  Each item takes max(A, ntiles) steps (the extra ones over empty
  // tiles), so the loads run at most one item ahead of the arithmetic.
  struct Item {
    int idx, next, b, hg, split, n, r0, r1, ntiles, blk0, nblk, steps;
  };
  auto item_of = [&](int g) {
    Item it;
    it.idx = g;
    if (g >= total) {  // past the last item: no rows
      it.next = g; it.b = 0; it.hg = 0; it.split = 0; it.n = 1; it.r0 = 0; it.r1 = 0;
      it.ntiles = 0; it.blk0 = 0; it.nblk = 0; it.steps = A;
      return it;
    }
    int lo = 0, hi = B - 1;  // the sequence b with pref[b] <= g < pref[b + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pref[mid] <= g) lo = mid;
      else hi = mid - 1;
    }
    it.b = lo;
    const int L = slen[lo];
    if (ranged) {
      const int u = L > 0 ? (L + kPmTile - 1) / kPmTile : 1;  // units of a head group
      const int rel = g - pref[lo];
      it.hg = rel / u;
      const int t0 = rel - it.hg * u;
      const int first = pref[lo] + it.hg * u;                // its first unit
      const int k = g / R;
      const int rend = min((k + 1) * R, total);
      const int t1 = min(u, t0 + (rend - g));
      it.split = k - first / R;                                // range starts in (first, g]
      it.n = (first + u - 1) / R - first / R + 1;
      it.r0 = min(t0 * kPmTile, L);
      it.r1 = min(t1 * kPmTile, L);
      const int gend = g + (t1 - t0);
      it.next = gend < rend ? gend : (k + W) * R;
    } else {
      it.hg = g - pref[lo];
      it.split = 0;
      it.n = 1;
      it.r0 = 0;
      it.r1 = L;
      it.next = g + W;
    }
    it.ntiles = it.r1 > it.r0 ? (it.r1 - it.r0 + kPmTile - 1) / kPmTile : 0;
    it.blk0 = it.r0 >> bs_log2;
    it.nblk = it.r1 > it.r0 ? ((it.r1 - 1) >> bs_log2) - it.blk0 + 1 : 0;
    it.steps = it.ntiles > A ? it.ntiles : A;
    // the same in every lane (from LDS and uniform values): scalar registers
    it.next = __builtin_amdgcn_readfirstlane(it.next);
    it.b = __builtin_amdgcn_readfirstlane(it.b);
    it.hg = __builtin_amdgcn_readfirstlane(it.hg);
    it.split = __builtin_amdgcn_readfirstlane(it.split);
    it.n = __builtin_amdgcn_readfirstlane(it.n);
    it.r0 = __builtin_amdgcn_readfirstlane(it.r0);
    it.r1 = __builtin_amdgcn_readfirstlane(it.r1);
    it.ntiles = __builtin_amdgcn_readfirstlane(it.ntiles);
    it.blk0 = __builtin_amdgcn_readfirstlane(it.blk0);
    it.nblk = __builtin_amdgcn_readfirstlane(it.nblk);
    it.steps = __builtin_amdgcn_readfirstlane(it.steps);
    return it;
  };
  const int first_item = (int)blockIdx.x * R;
  int total_steps = 0;
  for (Item it = item_of(first_item); it.idx < total; it = item_of(it.next))
    total_steps += it.steps;

  // Per-item metadata: the load side reads an item's query when it reaches the item
  // and stores it to LDS one step later, after the step's wait has covered it.  The
  // block-table entries of the item the loads are in stay in registers of every
  // wave (lane l: entries l and 64 + l), and the next item's are loaded alongside
  // the query, so a tile's block id is a lane read, not an LDS round trip.
  static_assert(kMaxTableSpan <= 128, "two table registers per lane");
  u32x4_t qstage[QLoads];
  int tcur0 = -1, tcur1 = -1, tnx0 = -1, tnx1 = -1;
  auto table_load = [&](const Item& it, int& t0, int& t1) {
    const int32_t* row = block_tables + (size_t)it.b * table_cols + soff[it.b] + it.blk0;
    t0 = lane < it.nblk ? row[lane] : -1;
    t1 = 64 + lane < it.nblk ? row[64 + lane] : -1;
  };
  auto meta_load = [&](const Item& it, const Item& nx) {
    const int qhead = __builtin_amdgcn_readfirstlane(it.b * Hq + GH * it.hg * G);
    const int qrec = __builtin_amdgcn_readfirstlane(it.idx < total ? QB : 0);
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(q) + (size_t)qhead * D, (short)0, qrec, 0x00020000);
#pragma unroll
    for (int k = 0; k < QLoads; ++k) {
      const int c = (int)threadIdx.x + kPmThreads * k;
      qstage[k] = __builtin_amdgcn_raw_buffer_load_b128(qr, c < QPieces ? c * 16 : (int)kPmNoRow,
                                                        0, 0);
    }
    table_load(nx, tnx0, tnx1);
  };
  auto meta_store = [&](int parity_q) {
#pragma unroll
    for (int k = 0; k < QLoads; ++k) {
      const int c = (int)threadIdx.x + kPmThreads * k;
      if (c < QPieces) *reinterpret_cast<u32x4_t*>(&qbuf[parity_q][c * 16]) = qstage[k];
    }
  };

  Item ld = item_of(first_item);   // the item the loads are in
  table_load(ld, tcur0, tcur1);
  int ld_t = 0, ld_j = 0;          // tile of the item, ordinal of the item (LDS parity)
  bool meta_pending = false;       // the loaded query waits to be stored
  int mq = 0;                      // where it goes

  // a tile in registers: K codes, V codes (lane load k of each), and for a coded
  // pool the scales: shared, lane j holding entry j of the wave's ScaleEntries (s[0]
  // for K, s[1] for V); else the scale of each code load (s[k], s[HalfLoads + k])
  struct TileRegs {
    u32x4_t c[2 * S::HalfLoads];
    float s[S::ScaleRegs];
  };
  // Loads of the next tile on the load side: wave load I = HalfLoads wave + k of the
  // K half (and of the V half) covers pool bytes [64 LW I, 64 LW (I + 1)) of the
  // tile's group rows; lane L takes LW bytes at cb = LW (64 I + L): token row cb /
  // CRB, byte cb % CRB of it (head (cb % CRB) / CB).  A tile past the item's rows
  // gets an empty resource (zeros, no memory traffic), so every step issues the same
  // tile loads.  Returns the tile's block id (-1: none).
  auto issue = [&](TileRegs& r) -> int {
    if (ld_t == 0) {  // a new item: its query, and the next item's table
      const Item nx = item_of(ld.next);
      meta_load(ld, nx);
      meta_pending = true;
      mq = ld_j & 1;
    }
    // (the block id is made wave-uniform explicitly: a resource built from a value the
    // compiler cannot prove uniform turns every load into a loop over distinct values)
    int phys = -1;
    if (ld_t < ld.ntiles) {
      const int e = __builtin_amdgcn_readfirstlane(((ld.r0 + ld_t * kPmTile) >> bs_log2) -
                                                   ld.blk0);
      phys = e < 64 ? __builtin_amdgcn_readlane(tcur0, e) : __builtin_amdgcn_readlane(tcur1, e - 64);
    }
    const bool bad = ld_t < ld.ntiles && (phys < 0 || phys >= num_blocks);
    if (bad && threadIdx.x == 0) raise_flag(err_flag, 1);
    phys = __builtin_amdgcn_readfirstlane(bad ? -1 : phys);
    const size_t base = phys >= 0 ? (size_t)phys * block_bytes : 0;
    const int records = phys >= 0 ? (int)block_bytes : 0;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(key_cache) + base, (short)0, records, 0x00020000);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(value_cache) + base, (short)0, records, 0x00020000);
    __amdgpu_buffer_rsrc_t ksr = kr, vsr = vr;
    if constexpr (S::Coded) {
      const size_t sbase = phys >= 0 ? (size_t)phys * block_rows : 0;
      const int srecords = phys >= 0 ? block_rows * 4 : 0;
      ksr = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(k_scale) + sbase, (short)0,
                                              srecords, 0x00020000);
      vsr = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(v_scale) + sbase, (short)0,
                                              srecords, 0x00020000);
    }
    const int tok0 = ld.r0 + ld_t * kPmTile;
#pragma unroll
    for (int k = 0; k < S::HalfLoads; ++k) {
      const int cb = S::LW * (lane + 64 * (wave * S::HalfLoads + k));
      const int row = cb / S::CRB;
      const int cbr = cb % S::CRB;
      const int tok = tok0 + row;
      const int srow = (tok & bs_mask) * Hkv + GH * ld.hg;   // the group's first (slot, head)
      const bool in = tok < ld.r1;
      const uint32_t off = in ? (uint32_t)(srow * S::CB + cbr) : kPmNoRow;
      r.c[k] = pm_load<S::LW>(kr, off);
      r.c[S::HalfLoads + k] = pm_load<S::LW>(vr, off);
      if constexpr (S::Coded && !S::SharedScales) {
        const uint32_t so = in ? (uint32_t)((srow + cbr / S::CB) * 4) : kPmNoRow;
        r.s[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ksr, (int)so, 0,
                                                                      kLoadNonTemporal));
        r.s[S::HalfLoads + k] = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(vsr, (int)so, 0, kLoadNonTemporal));
      }
    }
    if constexpr (S::SharedScales) {
      // the scales: one load per half, lane j taking entry e0 + j (token row e / GH,
      // head e % GH of the group); the loads above hit ScaleEntries entries in all,
      // each shared by CB / LW lanes, so this replaces a scale load per code load
      // (measured: the per-load scale loads cost as much as the code loads)
      const int e = 64 * S::LW * wave * S::HalfLoads / S::CB + lane;
      const int tok = tok0 + e / GH;
      const bool in = lane < S::ScaleEntries && tok < ld.r1;
      const uint32_t so =
          in ? (uint32_t)((((tok & bs_mask) * Hkv + GH * ld.hg + e % GH)) * 4) : kPmNoRow;
      r.s[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ksr, (int)so, 0,
                                                                    kLoadNonTemporal));
      r.s[1] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vsr, (int)so, 0,
                                                                    kLoadNonTemporal));
    }
    if (++ld_t == ld.steps) {
      ld = item_of(ld.next);
      ld_t = 0;
      ++ld_j;
      tcur0 = tnx0;
      tcur1 = tnx1;
    }
    return phys;
  };
  // the arrived registers of a tile into an LDS tile as bf16 (codes dequantised
  // with their row's scale), pieces permuted
  auto put = [&](const TileRegs& r, uint8_t* dst) {
#pragma unroll
    for (int k = 0; k < S::HalfLoads; ++k) {
      const int cb = S::LW * (lane + 64 * (wave * S::HalfLoads + k));
      const int row = cb / S::CRB;
      const int cbr = cb % S::CRB;
      if constexpr (!S::Coded) {
        const int at = row * S::RB + pm_slot(cbr / 16, row) * 16;
        *reinterpret_cast<u32x4_t*>(dst + at) = r.c[k];
        *reinterpret_cast<u32x4_t*>(dst + S::Half + at) = r.c[S::HalfLoads + k];
      } else {
        // the load's first element as a byte offset into the bf16 row; with shared
        // scales its scale is entry (LW (lane + 64 k)) / CB of the wave's, held by
        // that lane
        const int at = (cbr / S::CB) * 256 + (cbr % S::CB) * (16 / Bits);
        const int src = (S::LW * (lane + 64 * k)) / S::CB;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t w[S::Elems / 2];
          float sc;
          if constexpr (S::SharedScales)
            sc = __int_as_float(__builtin_amdgcn_ds_bpermute(src * 4, __float_as_int(r.s[h])));
          else
            sc = r.s[h * S::HalfLoads + k];
          pm_dequant<Bits, S::LW>(r.c[h * S::HalfLoads + k], sc, w);
          uint8_t* rowp = dst + h * S::Half + row * S::RB;
          if constexpr (S::Elems >= 8) {
#pragma unroll
            for (int p = 0; p < S::Elems / 8; ++p)
              *reinterpret_cast<u32x4_t*>(rowp + pm_slot(at / 16 + p, row) * 16) =
                  u32x4_t{w[4 * p], w[4 * p + 1], w[4 * p + 2], w[4 * p + 3]};
          } else {
            *reinterpret_cast<pm_u32x2_t*>(rowp + pm_slot(at / 16, row) * 16 + at % 16) =
                pm_u32x2_t{w[0], w[1]};
          }
        }
      }
    }
  };

  // operand addresses inside a tile: A = row col16, pieces 16 hw + 4 s + grp;
  // V = row 4 grp + col16 / 4, dims 16 (NB part + jb) + 4 (col16 % 4) .. +3: piece
  // 16 hw + 2 (NB part + jb) + (col16 % 4) / 2, byte 8 (col16 % 2) of it; the
  // query operand (B: head col16 of the wave's KV head, dims 32 s + 8 grp) from
  // the item's query in LDS, zero for col16 >= G
  const int a_row = col16 * S::RB;
  int a_off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) a_off[s] = a_row + pm_slot(16 * hw + 4 * s + grp, col16) * 16;
  const int v_row_i = 4 * grp + (col16 >> 2);
  const int v_row = S::Half + v_row_i * S::RB;
  int v_off[NB];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb)
    v_off[jb] = v_row +
                pm_slot(16 * hw + 2 * (NB * part + jb) + ((col16 & 3) >> 1), v_row_i) * 16 +
                (col16 & 1) * 8;
  const int q_off = ((hw * G + (col16 < G ? col16 : 0)) * D + 8 * grp) * 2;

  // The arithmetic side: the item it works on, its tile, and the running state --
  // O of the G query heads over this wave's NB dim blocks (C layout: lane -> dim
  // 16 (NB part + jb) + col16, heads 4 grp + i; rows G..15 stay zero), the running
  // max (head col16, the same in the four lane groups) and this lane's share of
  // the sum of exponentials.
  Item ci = item_of(first_item);
  int ct = 0, cj = 0;
  f32x4_t oacc[NB];
#pragma unroll
  for (int jb = 0; jb < NB; ++jb) oacc[jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, lsum = 0.f;

  // the item's query as B operands, read from LDS at its first tile
  u32x4_t qr[4];
  auto compute = [&](const uint8_t* T, int phys) {
    const int tok0 = ci.r0 + ct * kPmTile;
    const bool block_ok = phys >= 0;
    if (ct == 0) {
      const uint8_t* qp = qbuf[cj & 1] + q_off;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        qr[s] = *reinterpret_cast<const u32x4_t*>(qp + 64 * s);
        if (col16 >= G) qr[s] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    u32x4_t a[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = *reinterpret_cast<const u32x4_t*>(T + a_off[s]);
    i16x4_t vb[NB];
#pragma unroll
    for (int jb = 0; jb < NB; ++jb)
      vb[jb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(T + v_off[jb]));
    f32x4_t st0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, st1 = st0;
    st0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[0]),
                                                  __builtin_bit_cast(bf16x8_t, qr[0]), st0, 0,
                                                  0, 0);
    st1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[1]),
                                                  __builtin_bit_cast(bf16x8_t, qr[1]), st1, 0,
                                                  0, 0);
    st0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[2]),
                                                  __builtin_bit_cast(bf16x8_t, qr[2]), st0, 0,
                                                  0, 0);
    st1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[3]),
                                                  __builtin_bit_cast(bf16x8_t, qr[3]), st1, 0,
                                                  0, 0);
    float sc[4];
    float tmax = kNegInf;
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      const bool ok = block_ok && tok0 + 4 * grp + i2 < ci.r1;
      sc[i2] = ok ? (st0[i2] + st1[i2]) * scale_log2 : kNegInf;
      tmax = fmaxf(tmax, sc[i2]);
    }
    tmax = pm_group4_max(tmax);
    // skip-scale: a wave-uniform decision; a head whose max did not move gets alpha 1
    if (__any(tmax > m + kPmRescale)) {
      const float mnew = fmaxf(m, tmax);
      const float alpha = mnew == kNegInf ? 1.f : exp2_fast(m - mnew);
      m = mnew;
      lsum *= alpha;
      // alpha of head 4 grp + i for the output rows this lane holds: heads live in
      // lanes 0..G-1 (rows G..15 belong to no head and take any finite factor)
      float a4[4];
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        const float lo = __int_as_float(
            __builtin_amdgcn_readlane(__float_as_int(alpha), i2 < G ? i2 : 0));
        if constexpr (G > 4) {
          const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 4 + i2));
          a4[i2] = grp == 1 ? hi : lo;
        } else {
          a4[i2] = lo;
        }
      }
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) oacc[jb][i2] *= a4[i2];
      }
    }
    const float ms = m == kNegInf ? 0.f : m;
    i16x4_t pa, pl;
    float psum = 0.f;
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      const float p = exp2_fast(sc[i2] - ms);
      psum += p;
      const __bf16 hi = (__bf16)p;
      pa[i2] = bf16_bits(hi);
      pl[i2] = bf16_bits((__bf16)(p - (float)hi));
    }
    lsum += psum;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
      oacc[jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb[jb], oacc[jb], 0, 0, 0);
      oacc[jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vb[jb], oacc[jb], 0, 0, 0);
    }
  };

  // End of an item: per head (lane col16) the running max and the sum of
  // exponentials, moved to the lanes that hold the head's row of O; the output
  // (an item that is its sequence's only split) or the split's partial.
  auto finish = [&]() {
    const float lhead = pm_group4_sum(lsum);
    const size_t head0 = (size_t)ci.b * Hq + (size_t)(GH * ci.hg + hw) * G;
    // the merge reads how many pieces the (sequence, head group) has
    if (ranged && ci.split == 0 && threadIdx.x == 0) nseg[ci.b * ngroups + ci.hg] = ci.n;
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      const int j = 4 * grp + i2;
      const float M = __shfl(m, j);
      const float den = __shfl(lhead, j);
      if (j < G) {
        const bool any = M != kNegInf;
        const float inv = any ? 1.f / den : 0.f;
        const float lse2 = any ? M + __log2f(den) : kNegInf;
        float* dst = ci.n == 1 ? out + (head0 + j) * D
                               : ws.o + ((head0 + j) * max_splits + ci.split) * D;
        dst += 16 * NB * part + col16;
        if (ci.n == 1) {
#pragma unroll
          for (int jb = 0; jb < NB; ++jb) dst[16 * jb] = oacc[jb][i2] * inv;
        } else {
#pragma unroll
          for (int jb = 0; jb < NB; ++jb) store_through(&dst[16 * jb], oacc[jb][i2] * inv);
        }
        if (part == 0 && col16 == 0) {
          if (ci.n == 1) {
            if (lse) lse[head0 + j] = lse2 * kLn2;
          } else {
            store_through(&ws.lse[(head0 + j) * max_splits + ci.split], lse2);
          }
        }
      }
    }
  };

  // One step s: wait for this wave's loads of tile s (the loads of the A - 1 tiles
  // issued after it may stay outstanding; anything issued before it is complete
  // too), store the item metadata loaded one step earlier and write tile s to LDS
  // tile T; the barrier then makes every wave's stores visible (one step earlier it
  // ended every wave's reads of T's previous tile, s - 2); refill the registers with
  // tile s + A (after the barrier, so that the waves' loads enter the memory
  // pipeline while other waves compute); arithmetic on tile s.  Every step issues
  // the same tile loads (the ones past the last item are empty), so one wait count
  // fits all.
  constexpr int kUnroll = A % 2 == 0 ? A : 2 * A;
  TileRegs regs[A];
  int phys_ring[A];
#pragma unroll
  for (int k = 0; k < A; ++k) phys_ring[k] = issue(regs[k]);
  auto step = [&](int s, TileRegs& r, int& phys_slot, uint8_t* T) {
    __builtin_amdgcn_s_waitcnt(wait_vm((A - 1) * S::Loads));
    if (meta_pending) {
      meta_store(mq);
      meta_pending = false;
    }
    put(r, T);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0Pm);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int phys = phys_slot;
    phys_slot = issue(r);
    if (s < total_steps) {
      if (ct < ci.ntiles) compute(T, phys);
      if (++ct == ci.steps) {
        finish();
        ci = item_of(ci.next);
        ct = 0;
        ++cj;
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) oacc[jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        m = kNegInf;
        lsum = 0.f;
      }
    }
  };
  for (int s = 0; s < total_steps; s += kUnroll) {
#pragma unroll
    for (int k = 0; k < kUnroll; ++k)
      step(s + k, regs[k % A], phys_ring[k % A], (k & 1) ? tile1 : tile0);
  }
  // the empty tiles' loads are still in flight: let them land
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
}

// ------------------------------------------------------------------- merge
// One workgroup per (sequence, query head): the pieces of its (sequence, head
// group), as many as the split kernel recorded; a head of one piece has its output.
__global__ void __launch_bounds__(kThreads)
piece_merge_kernel(Workspace ws, const int32_t* __restrict__ nseg, int heads,
                   int heads_per_group, int stride, float* __restrict__ out,
                   float* __restrict__ lse) {
  const int bh = blockIdx.x;
  const int b = bh / heads;
  const int h = bh - b * heads;
  int n = nseg[b * (heads / heads_per_group) + h / heads_per_group];
  if (n <= 1) return;
  if (n > stride) n = stride;
  merge_head<128>(ws.lse + (size_t)bh * stride, ws.o + (size_t)bh * stride * 128, n,
                  out + (size_t)bh * 128, lse ? lse + bh : nullptr);
}

static hipError_t launch_paged_piece_merge(const Workspace& w, const int32_t* nseg, int B,
                                           int Hq, int heads_per_group, int stride, float* out,
                                           float* lse, hipStream_t stream) {
  hipLaunchKernelGGL(piece_merge_kernel, dim3(B * Hq), dim3(kThreads), 0, stream, w, nseg, Hq,
                     heads_per_group, stride, out, lse);
  return hipGetLastError();
}

// ------------------------------------------------------------------- planning
static int round_up_pm(int x, int m) { return (x + m - 1) / m * m; }

bool paged_mfma_shape(int B, int Hq, int Hkv, int D, int block_size) {
  if (B > kPmMaxSeqs) return false;
  if (!(Hkv == 2 || Hkv == 4 || Hkv % 8 == 0) || Hq % Hkv != 0 || D != 128) return false;
  const int G = Hq / Hkv;
  return (G == 1 || G == 2 || G == 4 || G == 8) && block_size >= kPmTile &&
         (block_size == 16 || block_size == 32 || block_size == 64 || block_size == 128);
}

SplitPlan plan_paged_mfma(int B, int Hkv, int max_seq_len, int block_size, int forced_splits) {
  SplitPlan p;
  const int unit = block_size > kMinChunk ? block_size : kMinChunk;
  // one split may touch at most kMaxTableSpan - 2 blocks; the merge takes <= 256
  // pieces, and a (sequence, head group) has at most the plan's splits plus one
  const int most = ((kMaxTableSpan - 2) * block_size) / unit * unit;
  const int least = round_up_pm((max_seq_len + kMaxSplits - 2) / (kMaxSplits - 1), unit);
  int c;
  if (forced_splits > 0) {
    c = round_up_pm((max_seq_len + forced_splits - 1) / forced_splits, unit);
  } else {
    // about kPmSplitsTarget splits if every sequence had max_seq_len tokens.  The
    // chunk is the shortest range a workgroup takes (and bounds the pieces of a
    // sequence); each piece adds a partial output that is written, read back and
    // merged.  When the persistent workgroups took whole splits, 512-token splits
    // (the batch-64, 16384-token paged config) measured 263 us, 256-token ones
    // 287 us, 128-token ones 314 us.
    const int gh = Hkv < 8 ? Hkv : 8;
    const int groups = Hkv / gh;
    const long long want = ((long long)B * groups * max_seq_len + kPmSplitsTarget - 1) /
                           kPmSplitsTarget;
    c = round_up_pm(want < 1 ? 1 : (int)(want > 1024 ? 1024 : want), unit);
  }
  if (c < unit) c = unit;
  if (c > most) c = most;
  if (c < least) c = least;
  p.chunk = c;
  p.max_splits = max_seq_len > 0 ? (max_seq_len + c - 1) / c : 1;
  return p;
}

// Workgroups of a persistent launch: as many as the device keeps resident at once
// (occupancy per CU times the CU count, both queried once per device and kernel).
template <int Bits, int G, int GH>
static int resident_workgroups() {
  constexpr int kMaxDev = 64;
  static int cached[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  if (cached[dev] > 0) return cached[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, paged_mfma_kernel<Bits, G, GH>,
                                                   kPmThreads, 0) != hipSuccess)
    return 0;
  const int n = cus * (per_cu > 0 ? per_cu : 1);
  cached[dev] = n;  // the same value whichever thread stores it
  return n;
}

template <int Bits, int G, int GH>
static hipError_t launch_pm(const uint16_t* qb, const uint8_t* kc, const uint8_t* vc,
                            const float* ks, const float* vs, const int32_t* block_tables,
                            int table_cols,
                            const int32_t* seq_lens, const int32_t* seq_offset, int B, int Hkv,
                            int num_blocks, int block_size, int bs_log2, int max_seq_len,
                            float scale, const SplitPlan& plan, const Workspace& w,
                            int32_t* nseg, float* out, float* lse, int32_t* err_flag,
                            hipStream_t stream) {
  const int resident = resident_workgroups<Bits, G, GH>();
  if (resident <= 0) return hipErrorInvalidValue;
  // at most: a range per workgroup, or (one split) every (sequence, head group)
  const long long items = (long long)B * (Hkv / GH) * (plan.max_splits + 1);
  const unsigned grid = (unsigned)(items < resident ? items : resident);
  // ranges when a sequence may need more than one split; the piece stride of the
  // workspace is the plan's splits plus one
  const int chunk = plan.max_splits > 1 ? plan.chunk : 0;
  hipLaunchKernelGGL((paged_mfma_kernel<Bits, G, GH>), dim3(grid), dim3(kPmThreads), 0, stream,
                     qb, kc, vc, ks, vs, block_tables, table_cols, seq_lens, seq_offset, B, Hkv,
                     num_blocks, block_size, bs_log2, max_seq_len, scale * kLog2e, chunk,
                     plan.max_splits + 1, w, nseg, out, lse, err_flag);
  return hipGetLastError();
}

template <int Bits>
static hipError_t launch_paged_mfma_fmt(const void* q, const void* key_cache,
                                        const void* value_cache, const float* k_scale,
                                        const float* v_scale, const int32_t* block_tables,
                                        int table_cols, const int32_t* seq_lens,
                                        const int32_t* seq_offset, int B, int Hq, int Hkv,
                                        int num_blocks, int block_size, int max_seq_len,
                                        float scale, float* out, float* lse, void* ws,
                                        const SplitPlan& plan, int32_t* err_flag,
                                        hipStream_t stream) {
  const int stride = plan.max_splits + 1;  // pieces of a (sequence, head group), at most
  const Workspace w = carve(ws, (size_t)B * Hq, stride, 128);
  int32_t* nseg = reinterpret_cast<int32_t*>(w.lse + (size_t)B * Hq * stride);
  int bs_log2 = 0;
  while ((1 << bs_log2) < block_size) ++bs_log2;
  const auto* qb = static_cast<const uint16_t*>(q);
  const auto* kc = static_cast<const uint8_t*>(key_cache);
  const auto* vc = static_cast<const uint8_t*>(value_cache);
  // KV heads per workgroup: up to 8 (whole token rows at Hkv = 8); 4 at G = 8, whose
  // query buffers would not fit the LDS next to 8-head tiles, and over the FP4 pool,
  // where half-size tiles let two workgroups share a CU (measured at the batch-64
  // paged config: 168 us with 4 heads, 191 us with 8; the FP8 pool is faster with 8:
  // 183 us against 228 us)
  const int gh_max = (Hq / Hkv == 8 || Bits == 4) ? 4 : 8;
  const int GH = Hkv < gh_max ? Hkv : gh_max;
  hipError_t err = hipErrorInvalidValue;
#define DAKV_PM(GG, HH)                                                                       \
  err = launch_pm<Bits, GG, HH>(qb, kc, vc, k_scale, v_scale, block_tables, table_cols,       \
                                seq_lens, seq_offset, B, Hkv, num_blocks, block_size, bs_log2, \
                                max_seq_len, scale, plan, w, nseg, out, lse, err_flag, stream)
#define DAKV_PM_H(GG)                  \
  switch (GH) {                        \
    case 2: DAKV_PM(GG, 2); break;     \
    case 4: DAKV_PM(GG, 4); break;     \
    default: DAKV_PM(GG, 8); break;    \
  }
  switch (Hq / Hkv) {
    case 1: DAKV_PM_H(1); break;
    case 2: DAKV_PM_H(2); break;
    case 4: DAKV_PM_H(4); break;
    case 8:
      if (GH == 2) DAKV_PM(8, 2);
      else DAKV_PM(8, 4);
      break;
    default: return hipErrorInvalidValue;
  }
#undef DAKV_PM_H
#undef DAKV_PM
  if (err != hipSuccess || plan.max_splits <= 1) return err;
  return launch_paged_piece_merge(w, nseg, B, Hq, Hq / Hkv * GH, stride, out, lse, stream);
}

hipError_t launch_decode_paged_mfma(const void* q, const void* key_cache,
                                    const void* value_cache, const int32_t* block_tables,
                                    int table_cols, const int32_t* seq_lens,
                                    const int32_t* seq_offset, int B, int Hq, int Hkv,
                                    int num_blocks, int block_size, int max_seq_len,
                                    float scale, float* out, float* lse, void* ws,
                                    const SplitPlan& plan, int32_t* err_flag,
                                    hipStream_t stream) {
  return launch_paged_mfma_fmt<16>(q, key_cache, value_cache, nullptr, nullptr, block_tables,
                                   table_cols, seq_lens, seq_offset, B, Hq, Hkv, num_blocks,
                                   block_size, max_seq_len, scale, out, lse, ws, plan, err_flag,
                                   stream);
}

hipError_t launch_decode_paged_mfma_lowbit(bool fp4, const void* q, const void* k_codes,
                                           const void* v_codes, const float* k_scale,
                                           const float* v_scale, const int32_t* block_tables,
                                           int table_cols, const int32_t* seq_lens,
                                           const int32_t* seq_offset, int B, int Hq, int Hkv,
                                           int num_blocks, int block_size, int max_seq_len,
                                           float scale, float* out, float* lse, void* ws,
                                           const SplitPlan& plan, int32_t* err_flag,
                                           hipStream_t stream) {
  const auto launch = fp4 ? launch_paged_mfma_fmt<4> : launch_paged_mfma_fmt<8>;
  return launch(q, k_codes, v_codes, k_scale, v_scale, block_tables, table_cols, seq_lens,
                seq_offset, B, Hq, Hkv, num_blocks, block_size, max_seq_len, scale, out, lse,
                ws, plan, err_flag, stream);
}

}  // namespace dakv
