// Internal interface between the host half of libkvc (kvc_host.cpp) and its
// HIP kernels (kvc_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/kvc.h"

namespace kvc {

// One contiguous run of new rows that lands in one physical block:
// rows [row, row + count) of the append input go to slots
// [offset, offset + count) of `block`.  `offset` rows were already valid.
struct AppendSegment {
  int32_t block;
  int32_t offset;
  int32_t count;
  int32_t row;
};

struct CowPair {
  int32_t src;
  int32_t dst;
};

// Device pool description for one cache.
struct PoolDesc {
  char* k;
  char* v;
  float* k_scale;
  float* v_scale;
  int32_t num_layers;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  kvc_dtype dtype;
};

__host__ __device__ inline int dtype_bytes(kvc_dtype t) {
  switch (t) {
    case KVC_F32: return 4;
    case KVC_F16: return 2;
    case KVC_BF16: return 2;
    case KVC_FP8_E4M3: return 1;
    case KVC_INT8: return 1;
  }
  return 0;
}

// Bytes of one (block, head) tile of one pool.
__host__ __device__ inline int64_t tile_bytes(const PoolDesc& p) {
  return (int64_t)p.head_dim * p.block_size * dtype_bytes(p.dtype);
}

struct DecodePlan {
  int32_t kernel = 0;            // 1 = FMA, 2 = MFMA split-K, 3 = several tokens without a row split
  // FMA kernel: fixed partitions
  int32_t partition_tokens = 0;
  int32_t num_partitions = 0;    // ceil(max_context_len / partition_tokens)
  // MFMA kernel: even split of each KV head's blocks over work_items waves,
  // the last 1/2^pool_shift of each wave's run cut into pool_pieces pieces
  // handed out at run time (0 = static split only); partial slots per query
  // head = batch + chunk_slots()
  int32_t work_items = 0;
  int32_t pool_pieces = 0;
  int32_t pool_shift = 0;
  // several query tokens per sequence: tile_groups = 0 for decode.  Kernel 2:
  // the 16-column tiles of (query token, head) pairs are spread over
  // waves_per_group waves of a work-group and tile_groups groups (grid.z),
  // and the partial rows hold one set of slots per query token index.  Kernel
  // 3: waves_per_group 32-column tiles per work-group, tile_groups groups of
  // them per sequence (grid.z, times max_pieces).
  int32_t tile_groups = 0;
  int32_t waves_per_group = 0;
  int32_t tiles_per_wave = 0;    // kernel 2: column tiles each wave holds (1..4), reusing every K/V block it loads
  int32_t max_q = 0;
  // sliding window (every kernel): a token sees at most `window` rows ending
  // at its own; 0 = the whole history
  int32_t window = 0;
  // kernel 3: each group's steps (two blocks each) are cut into pieces of
  // split_steps steps when there are too few groups to fill the chip (0 = no
  // cut), at most max_pieces per group; partial rows
  // [batch * max_q][Hq][max_pieces]
  int32_t split_steps = 0;
  int32_t max_pieces = 0;
  // shared-prefix (cascade) decode, kernel 2: 0, or the prefix's blocks,
  // which every sequence's decode list skips; the prefix pass (kernel 3
  // without the causal mask over sequence 0's first skip_blocks blocks, the
  // batch's queries as its columns) runs pre_groups work-groups per KV head,
  // its steps cut into pre_pieces pieces of pre_split_steps (0: one piece)
  int32_t skip_blocks = 0;
  int32_t pre_groups = 0;
  int32_t pre_split_steps = 0;
  int32_t pre_pieces = 0;
  int64_t chunk_slots() const { return (int64_t)work_items * (pool_pieces + 1); }
  int64_t query_slots() const { return tile_groups ? max_q : 1; }
};

// Dynamic pool: off unless asked for (on MI355X the balance it brings gains
// next to nothing); the pool is the last eighth of each wave's run unless
// pool_shift says otherwise.
constexpr int32_t kDefaultPoolShift = 3;

// Default number of waves per launch of the MFMA decode: one per SIMD of a
// 256-CU part for 16-bit and fp8 caches (each wave's prefetch ring keeps
// enough blocks in flight to stream HBM), two per SIMD for int8, whose code
// conversion takes more vector work per block than fp8's single hardware
// convert and overlaps better with a second wave (measured on the mixed
// batch: 393 us with 1024 waves, 381 us with 2048; fp8 361 vs 371 us).
// Fixed, so results do not depend on the device's CU count.
constexpr int32_t kDefaultWaves16 = 1024;
constexpr int32_t kDefaultWavesFp8 = 1024;
constexpr int32_t kDefaultWavesInt8 = 2048;
constexpr int32_t kMaxDefaultWaves = 2048;   // the largest of the three
inline int32_t default_waves(kvc_dtype kv) {
  return kv == KVC_INT8 ? kDefaultWavesInt8 : kv == KVC_FP8_E4M3 ? kDefaultWavesFp8 : kDefaultWaves16;
}

// Byte offsets inside the decode workspace.  FMA kernel: partial rows
// [B][Hq][num_partitions] (acc, m, l).  MFMA kernel: partial rows
// [query slots][Hq][B + chunk slots] (acc, m, l) -- one query slot for decode,
// max_q with several query tokens per sequence -- then per sequence
// {first chunk, chunks},
// then one ticket counter per KV head (zeroed by the launch sequence).
struct WorkspaceLayout {
  size_t acc, m, l, seginfo, tickets, bytes;
  // shared-prefix decode: the prefix pass's partial rows [batch][Hq][pieces]
  size_t pre_acc, pre_m, pre_l;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WorkspaceLayout workspace_layout(const DecodePlan& p, int32_t batch, int32_t num_heads, int32_t num_kv_heads,
                                        int32_t head_dim) {
  WorkspaceLayout w{0, 0, 0, 0, 0, 0, 0, 0, 0};
  size_t rows;
  if (p.kernel == 3) {
    if (p.max_pieces <= 1) return w;   // every tile in one piece: outputs only
    rows = (size_t)batch * p.max_q * num_heads * p.max_pieces;
  } else if (p.kernel == 1) {
    if (p.num_partitions <= 1) return w;
    rows = (size_t)batch * num_heads * p.num_partitions;
  } else {
    rows = (size_t)p.query_slots() * num_heads * ((size_t)batch + (size_t)p.chunk_slots());
  }
  w.m = align256(rows * head_dim * sizeof(float));
  w.l = w.m + align256(rows * sizeof(float));
  w.seginfo = w.l + align256(rows * sizeof(float));
  if (p.kernel == 2) {
    w.tickets = w.seginfo + align256((size_t)batch * 2 * sizeof(int32_t));
    w.bytes = w.tickets + align256((size_t)num_kv_heads * sizeof(int32_t));
  } else {
    w.tickets = w.bytes = w.seginfo;
  }
  if (p.kernel == 2 && p.skip_blocks > 0) {
    const size_t pre_rows = (size_t)batch * num_heads * p.pre_pieces;
    w.pre_acc = w.bytes;
    w.pre_m = w.pre_acc + align256(pre_rows * head_dim * sizeof(float));
    w.pre_l = w.pre_m + align256(pre_rows * sizeof(float));
    w.bytes = w.pre_l + align256(pre_rows * sizeof(float));
  }
  return w;
}
constexpr int32_t kMaxBatch = 8192;  // the per-sequence block scan lives in LDS

// Launchers (kvc_kernels.hip).  They only launch; arguments are validated by
// the caller.  Return hipSuccess or the launch error.
hipError_t launch_copy_blocks(const PoolDesc& pool, const CowPair* pairs_dev, int32_t num_pairs,
                              hipStream_t stream);
// Appends of at most kInlineSegments segments (a decode step over up to that
// many sequences) pass their plan as a kernel argument: no upload.
constexpr int32_t kInlineSegments = 192;
struct InlineSegments {
  AppendSegment s[kInlineSegments];
};

// segs_dev (device) or segs_inline (host, copied into the kernel arguments):
// exactly one is non-NULL.
hipError_t launch_append(const PoolDesc& pool, const AppendSegment* segs_dev, const InlineSegments* segs_inline,
                         int32_t num_segments, const void* k_new, const void* v_new, kvc_dtype in_dtype,
                         int64_t total_rows, hipStream_t stream);
// Whether the decode walk writes the step's newest rows itself: the static
// matrix-core walk over a 16-bit cache (a tile's one reader writes it); other
// plans run an append kernel first.
inline bool decode_folds_append(const DecodePlan& p, kvc_dtype kv) {
  return p.kernel == 2 && p.tile_groups == 0 && p.pool_pieces == 0 && (kv == KVC_F16 || kv == KVC_BF16);
}
// q_start / total_q: several query tokens per sequence (plan.tile_groups > 0);
// NULL / ignored for decode.  k_new / v_new (decode only, NULL = none): this
// layer's new rows [batch][num_kv_heads][head_dim] in q_dtype, written to
// position context_lens[b] - 1 of every sequence before it is attended.
hipError_t launch_decode(const PoolDesc& pool, int32_t layer, const DecodePlan& plan, const void* q,
                         kvc_dtype q_dtype, const int32_t* q_start, int32_t total_q, const int32_t* block_table,
                         int32_t max_blocks, const int32_t* context_lens, int32_t max_context_len, int32_t batch,
                         int32_t num_heads, float scale, void* out, void* workspace, const void* k_new,
                         const void* v_new, hipEvent_t ev_start, hipEvent_t ev_end, hipStream_t stream);
hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, hipStream_t stream);
// Device address of the current device's static decode workspace
// (KVC_STATIC_SCRATCH_BYTES bytes), resolved on the first call per device.
hipError_t static_scratch(void** ptr);

// Shared by the host sources (defined in kvc_host.cpp).
kvc_status host_fail(kvc_status st, const char* msg);   // records msg as the thread's last error
int32_t cache_block_size(const kvc_cache* c);

}  // namespace kvc
