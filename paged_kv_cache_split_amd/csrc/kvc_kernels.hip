// HIP kernels of libkvc for CDNA4 (gfx950): append into the paged pool
// (with fp8 E4M3 or int8 quantisation), copy-on-write block copies, the
// split-K paged decode (fp32 FMA kernel; matrix-core kernel walking an even
// split of each KV head's blocks), the several-token kernels (a row split
// like decode for few new tokens per sequence; 32x32 matrix-core tiles with
// their K/V steps staged in LDS for many), their merges, and a plain
// streaming copy used for bandwidth calibration.
//
// Pool layout (one (block, KV head) tile of block_size = 16 tokens):
//   K tile: [head_dim / X][16][X] elements, X = 16 bytes / element size, so
//           a 16-byte chunk holds X consecutive dims of one token and the 16
//           tokens' chunk c are 256 contiguous bytes;
//   V tile: [head_dim][16], V transposed (token index fastest).
// Block ids index the same tile position in every layer and both pools.
//
// What the decode computes (pages cited by title and section): per query
// head, softmax(q K^T * scale) V over the sequence's cached rows including
// the one just appended ("LLM推理优化实战：从KV-Cache到Continuous Batching…" §1.1;
// "苦猿的大模型日记 · Day45 · 大模型推理加速" PART 02); query head h reads KV head
// h / G ("大模型推理加速核心KV Cache 复用机制与内存布局优化" §二); rows are reached
// through a per-sequence block table (same page §三).  The rows are consumed
// 16 (or 32) at a time with the online-softmax recurrence (running max m, sum
// l and accumulator rescaled by exp(m_old - m_new), "LLM推理优化实战…" §3.2),
// each piece of a sequence's rows leaving a (m, l, acc) triple that a second
// kernel merges exactly (the "merge between blocks" of "大模型推理加速核心KV
// Cache…" §四).  Scores are kept in the base-2 domain (scale * log2(e) folded
// in), which leaves the softmax unchanged.  Options: a sliding window (each
// token sees the window's rows ending at its own), and a shared prefix
// attended once for the whole batch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "kvc_internal.h"

namespace kvc {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
// Pointers into the constant address space: the compiler may treat memory read
// through them as unchanging for the kernel's lifetime, so a load from a
// wave-uniform address becomes a scalar load (counted on lgkmcnt, apart from
// the vector loads).  Used only for block-table rows and fp8 scales, which no
// decode kernel writes.
typedef const int32_t __attribute__((address_space(4)))* const_i32_kptr;
typedef const float __attribute__((address_space(4)))* const_f32_kptr;
// p[i] for 0 <= i < 2^30 through a 32-bit byte offset, which the scalar load
// takes as its offset register (no 64-bit index arithmetic)
__device__ __forceinline__ int32_t ld_u32_index(const_i32_kptr p, int i) {
  typedef const char __attribute__((address_space(4)))* const_c_kptr;
  return *(const_i32_kptr)((const_c_kptr)p + ((uint32_t)i << 2));
}

constexpr int kBS = 16;                       // tokens per block (device work)

// Blocks each decode wave keeps in flight (16-bit and fp8 caches).  With one
// wave per SIMD the 16-bit kernel can spend all 256 VGPRs on a deeper ring
// (measured: 4 blocks help long single-sequence runs, 5 gain nothing more);
// the fp8 kernel's ring of 3 already streams at its best.
#ifndef KVC_PREFETCH_16
#define KVC_PREFETCH_16 4
#endif
#ifndef KVC_PREFETCH_FP8
#define KVC_PREFETCH_FP8 3
#endif
// 16-bit decode with the continuous ring (its next-query registers come out
// of the ring's).
#ifndef KVC_PREFETCH_STREAM16
#define KVC_PREFETCH_STREAM16 4
#endif
// One-byte decode with the continuous ring: a block is half a 16-bit one, so
// the ring holds more of them (measured on the mixed batch, 3 / 4 / 5 / 6
// blocks: fp8 367 / 364 / 364 / 364 us, int8 412 / 406 / 405 / 396 us).
#ifndef KVC_PREFETCH_STREAM8
#define KVC_PREFETCH_STREAM8 6
#endif
// Blocks in flight for the several-token kernel with 2, 3 or 4 column tiles
// per wave (their queries and accumulators take the registers).
#ifndef KVC_PREFETCH_T2
#define KVC_PREFETCH_T2 2
#endif
#ifndef KVC_PREFETCH_T3
#define KVC_PREFETCH_T3 1
#endif
#ifndef KVC_PREFETCH_T4
#define KVC_PREFETCH_T4 1
#endif
// Decode walk: at most this many finished segments per wave kept in LDS until
// the wave's end (fewer when LDS is short; 0 writes every result at once).
#ifndef KVC_STAGE_SLOTS
#define KVC_STAGE_SLOTS 4
#endif
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// Scalar conversions
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
  return (float)h;
}

// float -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32: round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed 16-bit pair (element a in the low half), nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f16x2_t v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t packed) { return (float)__builtin_bit_cast(f16x2_t, packed)[0]; }
__device__ __forceinline__ float f16_hi(uint32_t packed) { return (float)__builtin_bit_cast(f16x2_t, packed)[1]; }

// OCP E4M3 ("FN") code -> float, from the format definition: bias 7,
// exponent field 0 subnormal (m/8 * 2^-6).  Used where the value must be exact
// and independent of hardware conversion modes (re-encoding held codes).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float mag = (e == 0) ? (float)m * 0.001953125f                       // m * 2^-9
                       : __uint_as_float(((e + 120u) << 23) | (m << 20));  // 2^(e-7) * (1 + m/8)
  return (c & 0x80u) ? -mag : mag;
}

// float -> E4M3 code, round to nearest even, saturating at +-448 (never NaN).
// Signed zero is kept.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = __builtin_fabsf(x);
  if (!(a < 448.0f)) return sign | 0x7Eu;
  if (a < 0.015625f) {                          // below 2^-6: subnormal grid m * 2^-9
    float q = __builtin_rintf(a * 512.0f);      // exact scaling, then round half to even
    return sign | (uint32_t)q;                  // q == 8 is the smallest normal code 0x08
  }
  uint32_t au = __float_as_uint(a);
  uint32_t e = (au >> 23) - 127u + 7u;          // biased E4M3 exponent, 1..15
  uint32_t mant = au & 0x7FFFFFu;
  uint32_t r = mant >> 20, rem = mant & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
  if (r == 8u) { r = 0; ++e; }
  uint32_t code = (e << 3) | r;
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

// int8 code (a two's-complement byte) -> its integer value.
__device__ __forceinline__ float int8_decode(uint32_t c) { return (float)(int8_t)(uint8_t)c; }

// float -> int8 code: nearest integer, ties to even, clamped to +-127.
__device__ __forceinline__ uint32_t int8_encode(float x) {
  const float q = fminf(fmaxf(__builtin_rintf(x), -127.0f), 127.0f);
  return (uint32_t)(uint8_t)(int8_t)(int)q;
}

// One-byte caches (fp8 E4M3 and int8): codes times a per-(block, KV head) scale.
constexpr bool is_byte_code(kvc_dtype t) { return t == KVC_FP8_E4M3 || t == KVC_INT8; }

template <kvc_dtype KV>
__device__ __forceinline__ float code_decode(uint32_t c) {
  if constexpr (KV == KVC_FP8_E4M3) return e4m3_decode(c);
  else return int8_decode(c);
}

template <kvc_dtype T>
__device__ __forceinline__ float load_elem(const void* base, int64_t i) {
  if constexpr (T == KVC_F32) return static_cast<const float*>(base)[i];
  else if constexpr (T == KVC_F16) return f16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int clamp_block(int b, int num_blocks) {
  // (num_blocks >= 1: one unsigned compare tests both ends)
  return (uint32_t)b < (uint32_t)num_blocks ? b : 0;
}
// x * y for x, y in 0 .. 2^32 - 1 (a clamped block id times the bytes of one
// block of one layer, below 4 GiB, or times the KV head count): one 32 x
// 32-bit product instead of a signed 64-bit one
__device__ __forceinline__ int64_t mul_u32(int x, int64_t y) {
  return (int64_t)((uint64_t)(uint32_t)x * (uint32_t)y);
}

// Tokens to attend for sequence b, clamped so every access stays in bounds.
__device__ __forceinline__ int attend_len(const int32_t* context_lens, int b, int max_ctx, int max_blocks) {
  int n = context_lens[b];
  n = n < max_ctx ? n : max_ctx;
  int cap = max_blocks * kBS;
  return n < cap ? n : cap;
}

// The same for a wave-uniform b, read with a scalar load: a vector load whose
// result is needed at once makes the wave wait for every vector load issued
// before it (they complete in issue order), i.e. for the tiles in flight.
__device__ __forceinline__ int attend_len_s(const int32_t* context_lens, int b, int max_ctx, int max_blocks) {
  int n = ((const_i32_kptr)context_lens)[b];
  n = n < max_ctx ? n : max_ctx;
  int cap = max_blocks * kBS;
  return n < cap ? n : cap;
}

// ---------------------------------------------------------------------------
// Copy-on-write: copy whole blocks (every layer, head, K and V, fp8 scales).
// grid (num_pairs, num_layers), 256 threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void copy_blocks_kernel(PoolDesc p, const CowPair* pairs) {
  const CowPair pr = pairs[blockIdx.x];
  const int layer = blockIdx.y;
  const int64_t block_bytes = (int64_t)p.num_kv_heads * tile_bytes(p);
  const int64_t layer_bytes = (int64_t)p.num_blocks * block_bytes;
  const int64_t src = layer * layer_bytes + (int64_t)pr.src * block_bytes;
  const int64_t dst = layer * layer_bytes + (int64_t)pr.dst * block_bytes;
  for (int64_t i = threadIdx.x * 16; i < block_bytes; i += 256 * 16) {
    *reinterpret_cast<u32x4*>(p.k + dst + i) = *reinterpret_cast<const u32x4*>(p.k + src + i);
    *reinterpret_cast<u32x4*>(p.v + dst + i) = *reinterpret_cast<const u32x4*>(p.v + src + i);
  }
  if (is_byte_code(p.dtype)) {
    const int64_t so = ((int64_t)layer * p.num_blocks + pr.src) * p.num_kv_heads;
    const int64_t dof = ((int64_t)layer * p.num_blocks + pr.dst) * p.num_kv_heads;
    for (int h = threadIdx.x; h < p.num_kv_heads; h += 256) {
      p.k_scale[dof + h] = p.k_scale[so + h];
      p.v_scale[dof + h] = p.v_scale[so + h];
    }
  }
}

// Where an append kernel finds its write plan: device memory, or its own
// kernel arguments for small plans.
struct SegFromDevice {
  const AppendSegment* p;
  __device__ __forceinline__ AppendSegment get(int i) const { return p[i]; }
};
struct SegFromArgs {
  InlineSegments v;
  __device__ __forceinline__ AppendSegment get(int i) const { return v.s[i]; }
};
// The newest row of sequence i (position context_lens[i] - 1, the one a decode
// step appends) from its block-table row: row i of the append input goes to
// that slot.  A length or block id outside the arrays gives an empty segment
// (no write).
struct SegFromTable {
  const int32_t* block_table;
  const int32_t* context_lens;
  int32_t max_blocks, num_blocks;
  __device__ __forceinline__ AppendSegment get(int i) const {
    const int n = context_lens[i];
    AppendSegment s{0, 0, 0, i};
    if (n < 1 || n > max_blocks * kBS) return s;
    const int blk = block_table[(int64_t)i * max_blocks + (n - 1) / kBS];
    if (blk < 0 || blk >= num_blocks) return s;
    s.block = blk;
    s.offset = (n - 1) % kBS;
    s.count = 1;
    return s;
  }
};

// ---------------------------------------------------------------------------
// Append (reshape-and-cache) for f32 / f16 / bf16 caches: a plain copy of
// every new row into its slot.  grid (num_segments, num_kv_heads, num_layers),
// 64 threads.
// ---------------------------------------------------------------------------
template <int EBYTES, typename SEGS>
__global__ __launch_bounds__(64) void append_copy_kernel(PoolDesc p, SEGS segs, const char* k_new,
                                                         const char* v_new, int64_t total_rows) {
  const AppendSegment sg = segs.get(blockIdx.x);
  const int h = blockIdx.y, layer = blockIdx.z;
  const int D = p.head_dim, H = p.num_kv_heads;
  constexpr int X = 16 / EBYTES;
  const int nch = D / X;
  const int64_t tb = tile_bytes(p);
  const int64_t tile_off = ((int64_t)layer * p.num_blocks + sg.block) * H * tb + (int64_t)h * tb;
  char* kt = p.k + tile_off;
  char* vt = p.v + tile_off;
  const int64_t row_bytes = (int64_t)H * D * EBYTES;
  const char* ksrc = k_new + ((int64_t)layer * total_rows + sg.row) * row_bytes + (int64_t)h * D * EBYTES;
  const char* vsrc = v_new + ((int64_t)layer * total_rows + sg.row) * row_bytes + (int64_t)h * D * EBYTES;
  // K: 16-byte chunks, chunk c of row r -> tile[c][offset + r][:]
  for (int i = threadIdx.x; i < sg.count * nch; i += 64) {
    int r = i / nch, c = i % nch;
    u32x4 val = *reinterpret_cast<const u32x4*>(ksrc + r * row_bytes + c * 16);
    *reinterpret_cast<u32x4*>(kt + ((int64_t)c * kBS + sg.offset + r) * 16) = val;
  }
  // V: element (r, d) -> tile[d][offset + r].  A whole block of 16-bit rows
  // (a prompt or a long chunk) goes one dim per lane: the lane gathers the
  // dim's 16 values (each row's values are read by consecutive lanes) and
  // writes the tile row's 32 bytes at once, so the wave's stores are 2 KiB
  // contiguous instead of 2 bytes every 32.
  if constexpr (EBYTES == 2) {
    if (sg.count == kBS && sg.offset == 0) {
      for (int d = threadIdx.x; d < D; d += 64) {
        uint32_t w[kBS / 2];
#pragma unroll
        for (int r = 0; r < kBS; r += 2) {
          const uint32_t lo = *reinterpret_cast<const uint16_t*>(vsrc + r * row_bytes + (int64_t)d * 2);
          const uint32_t hi = *reinterpret_cast<const uint16_t*>(vsrc + (r + 1) * row_bytes + (int64_t)d * 2);
          w[r / 2] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>(vt + (int64_t)d * kBS * 2) = u32x4{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4*>(vt + (int64_t)d * kBS * 2 + 16) = u32x4{w[4], w[5], w[6], w[7]};
      }
      return;
    }
  }
  for (int i = threadIdx.x; i < sg.count * D; i += 64) {
    int r = i / D, d = i % D;
    const char* s = vsrc + r * row_bytes + (int64_t)d * EBYTES;
    char* t = vt + ((int64_t)d * kBS + sg.offset + r) * EBYTES;
    if constexpr (EBYTES == 4) *reinterpret_cast<uint32_t*>(t) = *reinterpret_cast<const uint32_t*>(s);
    else *reinterpret_cast<uint16_t*>(t) = *reinterpret_cast<const uint16_t*>(s);
  }
}

// ---------------------------------------------------------------------------
// Append into a one-byte cache (fp8 E4M3, or int8): per (segment, KV head, K
// or V) apply the scale rule -- s_new = max(s_old, amax / MAXC) with MAXC =
// 448 (E4M3) or 127 (int8); re-encode held codes when the scale grows; encode
// the new rows with s_new.  grid (num_segments, num_kv_heads, 2 *
// num_layers), 64 threads (one wave).
// ---------------------------------------------------------------------------
template <kvc_dtype KV, kvc_dtype IN, typename SEGS>
__global__ __launch_bounds__(64) void append_quant_kernel(PoolDesc p, SEGS segs, const void* k_new,
                                                          const void* v_new, int64_t total_rows) {
  constexpr float kMaxCode = (KV == KVC_FP8_E4M3) ? 448.0f : 127.0f;
  auto enc = [](float x) -> uint32_t {
    if constexpr (KV == KVC_FP8_E4M3) return e4m3_encode(x);
    else return int8_encode(x);
  };
  const AppendSegment sg = segs.get(blockIdx.x);
  if (sg.count <= 0) return;
  const int h = blockIdx.y;
  const int layer = blockIdx.z >> 1;
  const bool is_v = blockIdx.z & 1;
  const int D = p.head_dim, H = p.num_kv_heads;
  const int lane = threadIdx.x;
  const int64_t tb = tile_bytes(p);  // D * 16 bytes
  uint8_t* tile = reinterpret_cast<uint8_t*>((is_v ? p.v : p.k) + ((int64_t)layer * p.num_blocks + sg.block) * H * tb +
                                             (int64_t)h * tb);
  float* scale_ptr = (is_v ? p.v_scale : p.k_scale) + ((int64_t)layer * p.num_blocks + sg.block) * H + h;
  const void* src = is_v ? v_new : k_new;
  const int64_t src_row0 = ((int64_t)layer * total_rows + sg.row) * H * D + (int64_t)h * D;
  // Position of element (slot, d) inside the tile.
  auto at = [&](int slot, int d) -> int64_t {
    return is_v ? (int64_t)d * kBS + slot : ((int64_t)(d >> 4) * kBS + slot) * 16 + (d & 15);
  };
  float amax = 0.0f;
  for (int i = lane; i < sg.count * D; i += 64) {
    int r = i / D, d = i % D;
    amax = fmaxf(amax, __builtin_fabsf(load_elem<IN>(src, src_row0 + (int64_t)r * H * D + d)));
  }
  amax = wave_max(amax);
  const float s_old = sg.offset > 0 ? *scale_ptr : 0.0f;
  const float s_new = fmaxf(s_old, amax / kMaxCode);
  if (s_new > s_old && sg.offset > 0) {
    for (int i = lane; i < sg.offset * D; i += 64) {
      int r = i / D, d = i % D;
      int64_t o = at(r, d);
      float x = code_decode<KV>(tile[o]) * s_old;
      tile[o] = (uint8_t)enc(x / s_new);
    }
  }
  for (int i = lane; i < sg.count * D; i += 64) {
    int r = i / D, d = i % D;
    float x = load_elem<IN>(src, src_row0 + (int64_t)r * H * D + d);
    tile[at(sg.offset + r, d)] = (uint8_t)enc(s_new > 0.0f ? x / s_new : x);
  }
  if (lane == 0) *scale_ptr = s_new;
}

// ---------------------------------------------------------------------------
// Decode arguments (one layer).
// ---------------------------------------------------------------------------
struct DecodeArgs {
  const void* q;
  void* out;
  const int32_t* block_table;
  const int32_t* context_lens;
  // partials: FMA kernel [B][Hq][num_parts] rows, MFMA kernel [Hq][batch + chunk_slots] rows
  float* ws_acc;   // rows x D
  float* ws_m;     // rows
  float* ws_l;     // rows
  int* ws_seginfo; // MFMA kernel: per sequence {first chunk, number of chunks}
  int* ws_ticket;  // MFMA kernel: per KV head, pool pieces handed out so far (zero at launch)
  const char* k;   // layer base of the K pool
  const char* v;   // layer base of the V pool
  const float* k_scale;  // layer base (fp8)
  const float* v_scale;
  int64_t tile_bytes;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t max_ctx;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t part_tokens;
  int32_t num_parts;
  int32_t batch;
  int32_t work_items;
  int32_t pool_pieces;   // MFMA kernel: pool pieces per wave run (0 = static split)
  int32_t pool_shift;    // MFMA kernel: pool = last 1/2^pool_shift of each run
  int32_t chunk_slots;   // MFMA kernel: bound on chunk ids, work_items * (pool_pieces + 1)
  float qk_scale;  // softmax scale * log2(e)
  // several query tokens per sequence (extend kernel; decode: NULL, 1, batch, 1)
  const int32_t* q_start;   // [batch + 1]: query rows of sequence b are q_start[b] .. q_start[b + 1] - 1
  int32_t max_q;            // bound on query tokens per sequence
  int32_t total_q;          // rows of q and out
  int32_t waves_per_group;  // waves per work-group, one column tile each
  int32_t window;           // sliding window: a token sees at most this many rows ending at its own (0 = all)
  // several tokens, one wave per 32 columns: steps per piece of a tile's rows
  // (0 = the whole range in one piece) and pieces per tile bound
  int32_t split_steps;
  int32_t max_pieces;
  // shared-prefix (cascade) decode: the decode list of every sequence starts
  // at table block skip_blocks (the prefix is attended separately); outputs
  // are then never written by the row pass itself (partials_only), and the
  // merge also folds pre_pieces partial rows per (sequence, head) from
  // pre_acc / pre_m / pre_l ([batch][Hq][pre_max_pieces]).  The prefix pass
  // runs the several-token kernel with every column seeing all rows
  // (noncausal): one sequence (batch 1) of max_ctx rows read through the
  // block table's first row, with total_q query rows; q_start and
  // context_lens are not read then.
  int32_t skip_blocks;
  int32_t partials_only;
  int32_t noncausal;
  int32_t pre_pieces;
  int32_t pre_max_pieces;
  const float* pre_acc;
  const float* pre_m;
  const float* pre_l;
  // decode with the step's append folded in (16-bit caches, static split):
  // this layer's new rows [batch][num_kv_heads][D] in the cache dtype; the row
  // of sequence b goes to position context_lens[b] - 1 before it is attended
  // (NULL: the rows are already in the pool)
  const char* k_new;
  const char* v_new;
  // decode walk: segments whose results are kept in LDS until the wave's end
  // (slots of dynamic LDS after the scan; 0 = every result written at once)
  int32_t stage_slots;
};

template <kvc_dtype QT>
__device__ __forceinline__ void store_out(void* out, int64_t i, float v) {
  if constexpr (QT == KVC_F32) static_cast<float*>(out)[i] = v;
  else if constexpr (QT == KVC_F16) static_cast<uint16_t*>(out)[i] = (uint16_t)f32_to_f16_bits(v);
  else static_cast<uint16_t*>(out)[i] = (uint16_t)f32_to_bf16_bits(v);
}

// ---------------------------------------------------------------------------
// Split-K decode, fp32 FMA (VALU) variant.  One wave per (partition, KV head,
// sequence).  Scores: lane = (token t = lane / 4, quarter j = lane % 4), each
// lane dots a quarter of head_dim against the group's queries held in LDS,
// then a quad reduction.  Values: lane owns head_dim / 64 dims and sums the
// 16 tokens' weighted rows, weights broadcast from LDS.
// ---------------------------------------------------------------------------
template <kvc_dtype KV, kvc_dtype QT, int D, int GMAX>
__global__ __launch_bounds__(64) void decode_fma_kernel(DecodeArgs a) {
  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int n = attend_len(a.context_lens, b, a.max_ctx, a.max_blocks);
  const int t0 = part * a.part_tokens;
  if (t0 >= n) return;
  const int t1 = min(n, t0 + a.part_tokens);
  const int G = a.group;
  // window: rows before lo are not seen; a partition wholly before it leaves
  // an empty partial (m = -inf, l = 0, acc = 0: weight zero in the merge)
  const int lo = a.window > 0 ? max(0, n - a.window) : 0;
  if (t1 <= lo) {
    for (int hh = 0; hh < G; ++hh) {
      const int64_t rr = ((int64_t)b * a.num_heads + g * G + hh) * a.num_parts + part;
      for (int d = lane; d < D; d += 64) a.ws_acc[rr * D + d] = 0.0f;
      if (lane == 0) {
        a.ws_m[rr] = kNegInf;
        a.ws_l[rr] = 0.0f;
      }
    }
    return;
  }
  constexpr int EB = (KV == KVC_F32) ? 4 : (is_byte_code(KV) ? 1 : 2);
  constexpr int X = 16 / EB;
  constexpr int NCH = D / X;        // 16-byte chunks per token row
  constexpr int CPL = NCH / 4;      // chunks per lane
  constexpr int DPL = D / 64;       // output dims per lane

  __shared__ float q_s[GMAX][D];
  __shared__ float p_s[GMAX][kBS];
  for (int i = lane; i < GMAX * D; i += 64) {
    int hh = i / D, d = i % D;
    float qv = 0.0f;
    if (hh < G) qv = load_elem<QT>(a.q, ((int64_t)b * a.num_heads + g * G + hh) * D + d) * a.qk_scale;
    q_s[hh][d] = qv;
  }
  __syncthreads();

  const int t = lane >> 2, j = lane & 3;
  float m[GMAX], l[GMAX], acc[GMAX][DPL];
#pragma unroll
  for (int hh = 0; hh < GMAX; ++hh) {
    m[hh] = kNegInf;
    l[hh] = 0.0f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[hh][i] = 0.0f;
  }
  const int32_t* row = a.block_table + (int64_t)b * a.max_blocks;
  for (int kb = max(t0, lo) / kBS; kb * kBS < t1; ++kb) {
    const int phys = clamp_block(row[kb], a.num_blocks);
    const int64_t toff = ((int64_t)phys * a.num_kv_heads + g) * a.tile_bytes;
    const char* kt = a.k + toff;
    const char* vt = a.v + toff;
    float ksc = 1.0f, vsc = 1.0f;
    if constexpr (is_byte_code(KV)) {
      ksc = a.k_scale[(int64_t)phys * a.num_kv_heads + g];
      vsc = a.v_scale[(int64_t)phys * a.num_kv_heads + g];
    }
    float s[GMAX];
#pragma unroll
    for (int hh = 0; hh < GMAX; ++hh) s[hh] = 0.0f;
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      const int c = cc * 4 + j;
      u32x4 raw = *reinterpret_cast<const u32x4*>(kt + ((int64_t)c * kBS + t) * 16);
      float kx[X];
      if constexpr (KV == KVC_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) kx[e] = __uint_as_float(raw[e]);
      } else if constexpr (is_byte_code(KV)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) kx[e] = code_decode<KV>((raw[e >> 2] >> (8 * (e & 3))) & 0xFFu);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t bits = (raw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          kx[e] = (KV == KVC_F16) ? f16_bits_to_f32(bits) : bf16_bits_to_f32(bits);
        }
      }
#pragma unroll
      for (int hh = 0; hh < GMAX; ++hh) {
        if (hh < G) {
#pragma unroll
          for (int e = 0; e < X; ++e) s[hh] = fmaf(q_s[hh][c * X + e], kx[e], s[hh]);
        }
      }
    }
    const bool valid = kb * kBS + t < t1 && kb * kBS + t >= lo;
    float alpha[GMAX];
#pragma unroll
    for (int hh = 0; hh < GMAX; ++hh) {
      float v = s[hh];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v = valid ? v * ksc : kNegInf;
      float mx = v;
      mx = fmaxf(mx, __shfl_xor(mx, 4));
      mx = fmaxf(mx, __shfl_xor(mx, 8));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[hh], mx);
      alpha[hh] = __builtin_amdgcn_exp2f(m[hh] - mnew);
      const float pv = __builtin_amdgcn_exp2f(v - mnew);
      l[hh] = l[hh] * alpha[hh] + (j == 0 ? pv : 0.0f);
      m[hh] = mnew;
      if (j == 0 && hh < G) p_s[hh][t] = pv * vsc;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const int d = lane + 64 * i;
      float vx[kBS];
      const char* vrow = vt + (int64_t)d * kBS * EB;
      if constexpr (KV == KVC_F32) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x4 r = *reinterpret_cast<const u32x4*>(vrow + q4 * 16);
#pragma unroll
          for (int e = 0; e < 4; ++e) vx[q4 * 4 + e] = __uint_as_float(r[e]);
        }
      } else if constexpr (is_byte_code(KV)) {
        u32x4 r = *reinterpret_cast<const u32x4*>(vrow);
#pragma unroll
        for (int e = 0; e < 16; ++e) vx[e] = code_decode<KV>((r[e >> 2] >> (8 * (e & 3))) & 0xFFu);
      } else {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          u32x4 r = *reinterpret_cast<const u32x4*>(vrow + h2 * 16);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            uint32_t bits = (r[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            vx[h2 * 8 + e] = (KV == KVC_F16) ? f16_bits_to_f32(bits) : bf16_bits_to_f32(bits);
          }
        }
      }
      // rows past the end (only in the sequence's last block) hold whatever the
      // slot held before: their weight is zero, and zeroing the values keeps a
      // NaN pattern there out of the sum
      const int vrows = t1 - kb * kBS;
      if (vrows < kBS) {
#pragma unroll
        for (int tt = 0; tt < kBS; ++tt)
          if (tt >= vrows) vx[tt] = 0.0f;
      }
#pragma unroll
      for (int hh = 0; hh < GMAX; ++hh) {
        if (hh < G) {
          float acc_h = acc[hh][i] * alpha[hh];
#pragma unroll
          for (int tt = 0; tt < kBS; ++tt) acc_h = fmaf(p_s[hh][tt], vx[tt], acc_h);
          acc[hh][i] = acc_h;
        }
      }
    }
    __syncthreads();
  }
  const int parts_b = (n + a.part_tokens - 1) / a.part_tokens;
#pragma unroll
  for (int hh = 0; hh < GMAX; ++hh) {
    if (hh >= G) continue;
    const float lt = wave_sum(l[hh]);
    const int h = g * G + hh;
    if (parts_b == 1) {
      const float inv = 1.0f / lt;
#pragma unroll
      for (int i = 0; i < DPL; ++i) store_out<QT>(a.out, ((int64_t)b * a.num_heads + h) * D + lane + 64 * i, acc[hh][i] * inv);
    } else {
      const int64_t r = ((int64_t)b * a.num_heads + h) * a.num_parts + part;
#pragma unroll
      for (int i = 0; i < DPL; ++i) a.ws_acc[r * D + lane + 64 * i] = acc[hh][i];
      if (lane == 0) {
        a.ws_m[r] = m[hh];
        a.ws_l[r] = lt;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K decode, MFMA variant (16-bit and fp8 caches).  One wave per
// (partition, KV head, sequence); the group's G <= 16 query heads are the 16
// columns of the matrix-core tiles (zero-padded).
//   scores^T [16 tokens x 16 heads] = K_tile [16 x D] * Q^T [D x 16 heads]
//       with v_mfma_f32_16x16x32_{bf16,f16}: lane (row = lane % 16, group
//       r = lane / 16) feeds the 16-byte K chunk (4 kk + r) of token lane % 16
//       straight from memory, and the same dims of query head lane % 16;
//   out^T [16 dims x 16 heads] += V^T_tile [16 dims x 16 tokens] * P^T
//       with v_mfma_f32_16x16x16: the score tile's lane layout (tokens
//       4r..4r+3 of head lane % 16) is exactly the P^T operand, and V^T rows
//       give each lane its 4 tokens as one 8-byte load.
// Softmax runs on the score tile: a lane's 4 values plus two cross-group
// shuffles give the per-head block max.
// ---------------------------------------------------------------------------
// The 16-row walks (decode, several tokens by row split) take the scores of
// int8 caches on the f16 matrix cores: a K code c becomes the f16 value
// 1152 + c with one byte permute per pair (f16 0x64XX is 1024 + XX, and
// XX = c ^ 0x80 = c + 128), and the +1152 comes back out of the scores as a
// per-column constant (1152 times the sum of the column's f16 query).  The
// products with V stay bf16: a bias there would have to come back out of a
// sum whose weights the matrix cores see rounded to 16 bits (and tiny ones as
// f16 subnormals), and 1152 times those roundings is far above the result's
// tolerance.
constexpr bool qk_f16(kvc_dtype kv) { return kv == KVC_F16 || kv == KVC_INT8; }
constexpr float kI8Bias = 1152.0f;

template <kvc_dtype KV>
__device__ __forceinline__ floatx4 mfma_qk(const u32x4& a, const u32x4& b, floatx4 c) {
  if constexpr (qk_f16(KV))
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                   0);
}

template <kvc_dtype KV>
__device__ __forceinline__ floatx4 mfma_pv(const u32x2& a, const u32x2& b, floatx4 c) {
  if constexpr (KV == KVC_F16)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c, 0, 0,
                                                     0);
}

// Two E4M3 codes (bytes 0,1 or 2,3 of w) -> two bf16 packed in a dword, with
// unit scale.  E4M3 values are exact in bf16 (3-bit mantissa, exponents
// 2^-9 .. 2^8).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Two int8 codes (bytes 0,1 or 2,3 of w) -> two bf16 packed in a dword.
// Integers up to 127 in magnitude are exact in bf16.
template <bool HI>
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w) {
  constexpr int sh = HI ? 16 : 0;
  return pack_bf16x2((float)(int8_t)(w >> sh), (float)(int8_t)(w >> (sh + 8)));
}

// Four int8 codes (x = the code dword with every sign bit flipped, c + 128 as
// unsigned bytes) -> two dwords of f16 pairs 1152 + c: byte k of the pair's
// lane goes to the low byte of its 16-bit half, 0x64 to the high byte.
__device__ __forceinline__ uint32_t i8x2_to_f16x2_biased(uint32_t x, bool hi) {
  return __builtin_amdgcn_perm(0x64646464u, x, hi ? 0x04030402u : 0x04010400u);
}

template <kvc_dtype KV, bool HI>
__device__ __forceinline__ uint32_t code2_to_bf16x2(uint32_t w) {
  if constexpr (KV == KVC_FP8_E4M3) return fp8x2_to_bf16x2<HI>(w);
  else return i8x2_to_bf16x2<HI>(w);
}

template <kvc_dtype KV, int D>
struct KvBlock {
  static constexpr int NK = is_byte_code(KV) ? D / 64 : D / 32;  // 16-byte K loads per lane
  static constexpr int NV = D / 16;                                   // V^T loads per lane
  u32x4 k[NK];
  typename std::conditional<is_byte_code(KV), uint32_t, u32x2>::type v[NV];
  float ks, vs;  // one-byte codes: the (block, head) scales, fetched with the tile
};

// K/V tiles are read once per step: non-temporal loads (streaming cache
// policy) sustain a markedly higher HBM read rate than ordinary loads.
template <typename T>
__device__ __forceinline__ T load_stream(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}

// Lane offsets inside a (block, head) tile, fixed for the kernel: with a
// wave-uniform tile base they make every tile load a scalar-base +
// 32-bit-offset load with the step folded into the immediate.
//  K tile [D/(16/E)][16][16/E]: lane (nn, r) reads 16-byte chunk r + 4*kk of
//  token nn, so its offset is lane * 16 plus kk * 1 KiB.
//  V^T tile [D][16]: lane reads tokens 4r..4r+3 of dim 16*dd + nn.
template <kvc_dtype KV>
__device__ __forceinline__ uint32_t k_lane_offset(int lane) { return (uint32_t)lane * 16u; }
template <kvc_dtype KV>
__device__ __forceinline__ uint32_t v_lane_offset(int nn, int r) {
  constexpr uint32_t E = is_byte_code(KV) ? 1u : 2u;
  return ((uint32_t)nn * kBS + 4u * (uint32_t)r) * E;
}

template <kvc_dtype KV, int D>
__device__ __forceinline__ void load_block(KvBlock<KV, D>& blk, const char* kt, const char* vt, uint32_t koff,
                                           uint32_t voff) {
  constexpr int E = is_byte_code(KV) ? 1 : 2;
#pragma unroll
  for (int kk = 0; kk < KvBlock<KV, D>::NK; ++kk) blk.k[kk] = load_stream<u32x4>(kt + koff + kk * 1024);
#pragma unroll
  for (int dd = 0; dd < KvBlock<KV, D>::NV; ++dd) {
    if constexpr (is_byte_code(KV)) blk.v[dd] = load_stream<uint32_t>(vt + voff + dd * 16 * kBS * E);
    else blk.v[dd] = load_stream<u32x2>(vt + voff + dd * 16 * kBS * E);
  }
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left at their maximum)
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// max(a, b) of raw scores, which are finite or -inf (masked), never NaN: the
// median of (a, b, +inf) is one instruction, where fmaxf adds a NaN-quieting
// instruction per operand the compiler cannot prove already quiet (matrix-core
// results, lane permutes).
// (+inf goes through an empty asm so that the compiler does not fold the
// median back into fmaxf and its quieting instructions.)
__device__ __forceinline__ float score_max(float a, float b) {
  float inf = __builtin_huge_valf();
  asm("" : "+s"(inf));
  return __builtin_amdgcn_fmed3f(a, b, inf);
}

// Max of raw scores over the lanes l, l^16, l^32, l^48 (the four row groups
// of a wave) with the gfx950 row-swap permutes: no LDS round trip.
__device__ __forceinline__ float max_over_row_groups(float x) {
  const uint32_t xb = __float_as_uint(x);
  const auto p16 = __builtin_amdgcn_permlane16_swap(xb, xb, false, false);
  const float y = score_max(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
  const uint32_t yb = __float_as_uint(y);
  const auto p32 = __builtin_amdgcn_permlane32_swap(yb, yb, false, false);
  return score_max(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}

// The P^T operand of a pair of weights as a bf16 hi part and a bf16 lo part:
// hi = the top 16 bits of each weight (truncation; one byte permute packs the
// pair), lo = the exact remainder w - hi rounded to bf16, so hi + lo is w to
// ~2^-16 relative.
__device__ __forceinline__ void split_bf16x2(float w0, float w1, uint32_t& hi, uint32_t& lo) {
  const uint32_t b0 = __float_as_uint(w0), b1 = __float_as_uint(w1);
  hi = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
  lo = pack_bf16x2(w0 - __uint_as_float(b0 & 0xFFFF0000u), w1 - __uint_as_float(b1 & 0xFFFF0000u));
}

__device__ __forceinline__ float sum_over_row_groups(float x) {
  const uint32_t xb = __float_as_uint(x);
  const auto p16 = __builtin_amdgcn_permlane16_swap(xb, xb, false, false);
  const float y = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
  const uint32_t yb = __float_as_uint(y);
  const auto p32 = __builtin_amdgcn_permlane32_swap(yb, yb, false, false);
  return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

// int8 caches on the f16 matrix cores: the query operands of N column tiles
// (q[N * NQK], bf16 as loaded) become f16 values q * 2^-e, with e >= 0 the
// smallest exponent that keeps every query value of the wave below 2^15 (0
// unless some |q| >= 2^15); kb[t] gets tile t's column bias, 1152 times the
// sum of the column's f16 values over its four lane groups.  Returns 2^e,
// which the score scale takes back.  Every lane of the wave takes part.
template <int N, int NQK>
__device__ __forceinline__ float int8_queries(u32x4* q, float* kb) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < N * NQK; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      amax = fmaxf(amax, fmaxf(__builtin_fabsf(bf16_lo(q[i][j])), __builtin_fabsf(bf16_hi(q[i][j]))));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  amax = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(amax)));
  // floor(log2(amax)) from the exponent field (amax >= 2^15 is a normal float)
  const int e = amax >= 32768.0f ? (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 - 14 : 0;
  const float down = __builtin_ldexpf(1.0f, -e);
#pragma unroll
  for (int t = 0; t < N; ++t) {
    float sum = 0.0f;
#pragma unroll
    for (int kk = 0; kk < NQK; ++kk) {
      u32x4& w = q[t * NQK + kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // values below f16's normal range become 0, so that the bias counts
        // exactly what the matrix cores multiply whether or not they keep
        // f16 subnormals
        float f0 = bf16_lo(w[j]) * down, f1 = bf16_hi(w[j]) * down;
        f0 = __builtin_fabsf(f0) < 0x1p-14f ? 0.0f : f0;
        f1 = __builtin_fabsf(f1) < 0x1p-14f ? 0.0f : f1;
        const uint32_t h = pack_f16x2(f0, f1);
        sum += f16_lo(h) + f16_hi(h);
        w[j] = h;
      }
    }
    kb[t] = kI8Bias * sum_over_row_groups(sum);
  }
  return __builtin_ldexpf(1.0f, e);
}

// The reference max only moves when a block's max exceeds it by more than
// this many log2 units, so weights stay <= 2^8 and the accumulator rescale
// (and the branch into it) is skipped for almost every block.  Any reference
// gives the same softmax; the bound only guards the float range.
constexpr float kRescaleThreshold = 8.0f;

// Query tokens of sequence b in a multi-token call: q_start[b + 1] - q_start[b],
// clamped to 0 .. min(max_q, n) so every row index stays inside the arrays.
// The loads go through the constant address space: scalar when b is uniform.
__device__ __forceinline__ int query_len(const DecodeArgs& a, int b, int n) {
  const const_i32_kptr qs = (const_i32_kptr)a.q_start;
  int ql = qs[b + 1] - qs[b];
  ql = ql < a.max_q ? ql : a.max_q;
  ql = ql < n ? ql : n;
  return ql > 0 ? ql : 0;
}

// First table block of a sequence holding a row some query token sees: with a
// window, the oldest new token (position n - ql) sees rows from
// n - ql + 1 - window on; blocks before that are never read (and may have
// been released by eviction).
__device__ __forceinline__ int first_visible_block(int n, int ql, int window) {
  const int lo = n - ql + 1 - window;
  return (window > 0 && lo > 0) ? lo / kBS : 0;
}

// First table block of a sequence's decode list: the first the window lets
// the new token see, and none of a shared prefix attended apart.
__device__ __forceinline__ int decode_first_block(const DecodeArgs& a, int n) {
  const int f = first_visible_block(n, 1, a.window);
  return f > a.skip_blocks ? f : a.skip_blocks;
}

// Exclusive scan of the sequences' block counts into LDS: seq_start[b] is the
// first block of sequence b in the batch's concatenated block list, and
// seq_start[batch] the total.  Every wave of the decode and every merge
// work-group computes the same values from context_lens.  With several query
// tokens per sequence (EXT), a sequence with no query token owns no blocks;
// with a window, a sequence's list starts at its first visible block.
template <bool EXT>
__device__ __forceinline__ int scan_block_counts(const DecodeArgs& a, int* seq_start, int lane) {
  int carry = 0;
  for (int base = 0; base < a.batch; base += 64) {
    const int bb = base + lane;
    int nb = 0;
    if (bb < a.batch) {
      const int n = attend_len(a.context_lens, bb, a.max_ctx, a.max_blocks);
      nb = n > 0 ? (n + kBS - 1) / kBS : 0;
      int ql = 1;
      if constexpr (EXT) {
        ql = query_len(a, bb, n);
        if (ql == 0) nb = 0;
      }
      if (nb > 0) nb -= EXT ? first_visible_block(n, ql, a.window) : decode_first_block(a, n);
      if (nb < 0) nb = 0;
    }
    int incl = nb;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (bb < a.batch) seq_start[bb] = carry + incl - nb;
    carry += __shfl(incl, 63);
  }
  if (lane == 0) seq_start[a.batch] = carry;
  return carry;
}

// First block of wave w when `total` blocks are split evenly over W waves;
// block x belongs to wave (x * W) / total.
__device__ __forceinline__ int wave_first_block(int64_t w, int64_t total, int64_t W) {
  return (int)((w * total + W - 1) / W);
}

// Chunks of one KV head's block list: `total` blocks split evenly over W
// waves.  With a pool (KP > 0) the last 1/2^shift of every wave's run is cut
// into KP pieces that go, at run time, to whichever wave of the head asks
// first.  Chunk ids follow the list order -- wave w's main chunk is
// w * (KP + 1), its pieces follow it -- so the chunks holding one sequence
// have consecutive ids whichever waves processed them, and the chunk bounds
// (hence the result) do not depend on who took which piece.
struct ChunkGeometry {
  int total, W, KP, shift;
  // wave ww's run is [r0, r1); its main chunk ends at rm
  __device__ void wave_range(int ww, int& r0, int& r1, int& rm) const {
    r0 = wave_first_block(ww, total, W);
    r1 = wave_first_block(ww + 1, total, W);
    rm = KP ? r1 - ((r1 - r0) >> shift) : r1;
  }
  // chunk holding list block y (piece j of a pool of len blocks starts at
  // ceil(j * len / KP), so block o of the pool is in piece o * KP / len)
  __device__ int chunk_of_block(int y) const {
    const int ww = (int)(((int64_t)y * W) / total);
    int r0, r1, rm;
    wave_range(ww, r0, r1, rm);
    if (y < rm) return ww * (KP + 1);
    return ww * (KP + 1) + 1 + (int)(((int64_t)(y - rm) * KP) / (r1 - rm));
  }
  // ticket t < W * KP: piece t % KP of wave t / KP's pool, blocks [xa, xb), id c
  __device__ void piece(int t, int& xa, int& xb, int& c) const {
    const int ww = t / KP, j = t - ww * KP;
    int r0, r1, rm;
    wave_range(ww, r0, r1, rm);
    const int64_t len = r1 - rm;
    xa = rm + (int)((j * len + KP - 1) / KP);
    xb = rm + (int)(((j + 1) * len + KP - 1) / KP);
    c = ww * (KP + 1) + 1 + j;
  }
};

// The sequence holding list block x: the last b with seq_start[b] <= x
// (an empty sequence shares its start with the next one).
__device__ __forceinline__ int seq_holding(const int* seq_start, int batch, int x) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(seq_start[mid]) <= x) lo = mid;
    else hi = mid - 1;
  }
  return __builtin_amdgcn_readfirstlane(lo);
}

// Rows past a sequence's end (only in its last block) hold whatever the slot
// held before (never written, or a previous owner's rows): their weight is
// zero, and zeroing their values keeps a NaN pattern there out of the
// accumulator (0 * NaN is NaN).  t0 = this lane's first row of the block.
template <kvc_dtype KV, int D>
__device__ __forceinline__ void zero_rows_past_end(KvBlock<KV, D>& cur, int n, int t0) {
  constexpr int NDD = D / 16;
  const int vr = n - t0;                     // rows of this lane's four inside the sequence
  if constexpr (is_byte_code(KV)) {
    const uint32_t keep = vr >= 4 ? 0xFFFFFFFFu : (vr <= 0 ? 0u : (0xFFFFFFFFu >> (32 - 8 * vr)));
#pragma unroll
    for (int dd = 0; dd < NDD; ++dd) cur.v[dd] &= keep;
  } else {
    const uint32_t keep0 = vr >= 2 ? 0xFFFFFFFFu : (vr == 1 ? 0xFFFFu : 0u);
    const uint32_t keep1 = vr >= 4 ? 0xFFFFFFFFu : (vr == 3 ? 0xFFFFu : 0u);
#pragma unroll
    for (int dd = 0; dd < NDD; ++dd) {
      cur.v[dd][0] &= keep0;
      cur.v[dd][1] &= keep1;
    }
  }
}

// Matrix-core operands of one block: the K tile (D/32 steps of 16 bytes per
// lane) and the V^T tile (D/16 dim tiles of 8 bytes per lane) as bf16 / f16.
// One-byte codes are converted here once per block; 16-bit tiles are used as
// loaded.
template <kvc_dtype KV, int D>
struct BlockOps {
  u32x4 k[D / 32];
  u32x2 v[D / 16];
};

template <kvc_dtype KV, int D>
__device__ __forceinline__ void convert_codes(const KvBlock<KV, D>& cur, BlockOps<KV, D>& ops) {
  if constexpr (KV == KVC_INT8) {
    // K: biased f16 (1152 + c), a sign flip per dword and a byte permute per
    // pair; V: bf16
#pragma unroll
    for (int c2 = 0; c2 < KvBlock<KV, D>::NK; ++c2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t x = cur.k[c2][j] ^ 0x80808080u;
        ops.k[2 * c2 + (j >> 1)][2 * (j & 1)] = i8x2_to_f16x2_biased(x, false);
        ops.k[2 * c2 + (j >> 1)][2 * (j & 1) + 1] = i8x2_to_f16x2_biased(x, true);
      }
    }
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd) {
      ops.v[dd][0] = code2_to_bf16x2<KV, false>(cur.v[dd]);
      ops.v[dd][1] = code2_to_bf16x2<KV, true>(cur.v[dd]);
    }
    return;
  }
#pragma unroll
  for (int c2 = 0; c2 < KvBlock<KV, D>::NK; ++c2) {
    ops.k[2 * c2][0] = code2_to_bf16x2<KV, false>(cur.k[c2][0]);
    ops.k[2 * c2][1] = code2_to_bf16x2<KV, true>(cur.k[c2][0]);
    ops.k[2 * c2][2] = code2_to_bf16x2<KV, false>(cur.k[c2][1]);
    ops.k[2 * c2][3] = code2_to_bf16x2<KV, true>(cur.k[c2][1]);
    ops.k[2 * c2 + 1][0] = code2_to_bf16x2<KV, false>(cur.k[c2][2]);
    ops.k[2 * c2 + 1][1] = code2_to_bf16x2<KV, true>(cur.k[c2][2]);
    ops.k[2 * c2 + 1][2] = code2_to_bf16x2<KV, false>(cur.k[c2][3]);
    ops.k[2 * c2 + 1][3] = code2_to_bf16x2<KV, true>(cur.k[c2][3]);
  }
#pragma unroll
  for (int dd = 0; dd < D / 16; ++dd) {
    ops.v[dd][0] = code2_to_bf16x2<KV, false>(cur.v[dd]);
    ops.v[dd][1] = code2_to_bf16x2<KV, true>(cur.v[dd]);
  }
}

// One block's update of one tile of 16 columns: the 16 rows' scores on the
// matrix cores, the mask (only where `edge`: rows at or past the column's
// ncol, or before its col_lo), the online-softmax step with the lazily moved
// reference max, and the PV accumulation.  kop / vop: the block's operands;
// qk: softmax scale * log2(e) (times the K scale for one-byte codes); vsc: the
// V scale (1 for 16-bit tiles).
template <kvc_dtype KV, int D>
__device__ __forceinline__ void tile_step(const u32x4* kop, const u32x2* vop, const u32x4* q, floatx4* acc,
                                          float& m, float& l, float qk, float vsc, bool edge, int t0, int ncol,
                                          int col_lo, float kb = 0.0f) {
  constexpr int NQK = D / 32, NDD = D / 16;
  floatx4 s = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < NQK; ++kk) s = mfma_qk<KV>(kop[kk], q[kk], s);
  float sv[4] = {s[0], s[1], s[2], s[3]};
  if (edge) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (t0 + e >= ncol || t0 + e < col_lo) sv[e] = kNegInf;
  }
  // the scale is positive, so the max of the raw scores, scaled, is the max
  // of the scaled scores; exp2(s * qk - m) is one fma
  // (int8: kb = the column's score bias 1152 * sum of its f16 query)
  // The column's reference max moves only when one of its 16 scores passes
  // it by the threshold, so each lane first tests its own 4: only when some
  // lane's do is the column max (over the four lanes holding the column)
  // formed.  The outcome is the same as testing the column max every block.
  float lraw = score_max(score_max(sv[0], sv[1]), score_max(sv[2], sv[3]));
  if constexpr (KV == KVC_INT8) lraw -= kb;
  if (__any(lraw * qk > m + kRescaleThreshold)) {
    float mraw = max_over_row_groups(score_max(score_max(sv[0], sv[1]), score_max(sv[2], sv[3])));
    if constexpr (KV == KVC_INT8) mraw -= kb;
    const float mx = mraw * qk;
    const bool grow = mx > m + kRescaleThreshold;
    const float mnew = grow ? mx : m;
    // (a column that has seen no row yet keeps m = -inf: alpha 1, not NaN)
    const float alpha = grow ? __builtin_amdgcn_exp2f(m - mnew) : 1.0f;
    l *= alpha;
#pragma unroll
    for (int dd = 0; dd < NDD; ++dd) acc[dd] *= alpha;
    m = mnew;
  }
  // exp2(s * qk - m), with int8's score bias taken out of the same fma
  const float moff = KV == KVC_INT8 ? __builtin_fmaf(kb, qk, m) : m;
  float pv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], qk, -moff));
  if (edge) {
    // Masked rows weigh 0 (forced: with m still -inf, or a zero one-byte
    // scale, the exponent above is NaN).  Scores of finite values are finite,
    // so -inf marks exactly the masked rows, and the index tests stay in the
    // edge path.
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (sv[e] == kNegInf) pv[e] = 0.0f;
  }
  l += (pv[0] + pv[1]) + (pv[2] + pv[3]);
  if constexpr (is_byte_code(KV)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] *= vsc;
  }
  // P^T operand as a 16-bit hi part plus a 16-bit lo part (P = hi + lo to
  // ~2^-16 relative), so rounding the weights to 16 bits costs no accuracy
  // when the weighted values cancel.
  u32x2 pb, pl;
  if constexpr (KV == KVC_F16) {
    pb[0] = pack_f16x2(pv[0], pv[1]);
    pb[1] = pack_f16x2(pv[2], pv[3]);
    pl[0] = pack_f16x2(pv[0] - f16_lo(pb[0]), pv[1] - f16_hi(pb[0]));
    pl[1] = pack_f16x2(pv[2] - f16_lo(pb[1]), pv[3] - f16_hi(pb[1]));
  } else {
    uint32_t h0, l0, h1, l1;
    split_bf16x2(pv[0], pv[1], h0, l0);
    split_bf16x2(pv[2], pv[3], h1, l1);
    pb[0] = h0; pl[0] = l0;
    pb[1] = h1; pl[1] = l1;
  }
#pragma unroll
  for (int dd = 0; dd < NDD; ++dd) {
    acc[dd] = mfma_pv<KV>(vop[dd], pb, acc[dd]);
    acc[dd] = mfma_pv<KV>(vop[dd], pl, acc[dd]);
  }
}

// Output of one column tile: the normalised rows (out, in the 16-bit dtype of
// q) or the partial (m, l, acc) at partial row rr.
template <kvc_dtype KV, int D>
__device__ __forceinline__ void write_out_row(const DecodeArgs& a, int64_t row, int r, const floatx4* acc, float lt) {
  const float inv = 1.0f / lt;
#pragma unroll
  for (int dd = 0; dd < D / 16; ++dd) {
    const int64_t o = row * D + 16 * dd + 4 * r;
    u32x2 wv;
    if constexpr (KV == KVC_F16) {
      wv[0] = pack_f16x2(acc[dd][0] * inv, acc[dd][1] * inv);
      wv[1] = pack_f16x2(acc[dd][2] * inv, acc[dd][3] * inv);
    } else {
      wv[0] = pack_bf16x2(acc[dd][0] * inv, acc[dd][1] * inv);
      wv[1] = pack_bf16x2(acc[dd][2] * inv, acc[dd][3] * inv);
    }
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + o) = wv;
  }
}

template <kvc_dtype KV, int D>
__device__ __forceinline__ void write_out(const DecodeArgs& a, int64_t out_row, int h, int r, const floatx4* acc,
                                          float lt) {
  write_out_row<KV, D>(a, out_row * a.num_heads + h, r, acc, lt);
}

template <int D>
__device__ __forceinline__ void write_partial(const DecodeArgs& a, int64_t rr, int r, const floatx4* acc, float m,
                                              float lt) {
#pragma unroll
  for (int dd = 0; dd < D / 16; ++dd) *reinterpret_cast<floatx4*>(a.ws_acc + rr * D + 16 * dd + 4 * r) = acc[dd];
  if (r == 0) {
    a.ws_m[rr] = m;
    a.ws_l[rr] = lt;
  }
}

// The split-K body for several new query tokens per sequence (q_start), each
// attending causally -- the token at position p sees rows 0..p -- so a column
// of the matrix-core tiles is a (query token, head) pair with its own count of
// visible rows.  A sequence's ceil(ql * G / 16) column tiles are spread TPW to
// a wave (the wave reuses each K/V block it loads for all of its tiles), over
// the waves of a work-group (side by side on one chunk of blocks) and over
// grid.z.  One token per sequence is decode (decode_stream, the same per-block
// arithmetic without the per-column bookkeeping).
template <kvc_dtype KV, int D, int PF, int TPW>
__device__ __forceinline__ void attend_extend(const DecodeArgs& a, int* seq_start) {
  const int w = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  // first column tile of this wave.  Tile groups run last group first: under
  // the causal mask the last tokens' tiles see the most blocks, so the longest
  // work-groups start first and the short ones fill in behind them.
  const int ct0 = __builtin_amdgcn_readfirstlane(
      ((int)(gridDim.z - 1 - blockIdx.z) * a.waves_per_group + (int)(threadIdx.x >> 6)) * TPW);
  if (threadIdx.x < 64) scan_block_counts<true>(a, seq_start, lane);
  __syncthreads();
  const int total = __builtin_amdgcn_readfirstlane(seq_start[a.batch]);
  // never more waves than blocks, so every wave that runs owns >= 1 block
  const int W = a.work_items < total ? a.work_items : total;
  if (w >= W) return;
  // chunk w: blocks [xa, xb) of this head's list (an even split)
  const ChunkGeometry geo{total, W, 0, 0};
  const int nn = lane & 15, r = lane >> 4;
  const uint32_t koff = k_lane_offset<KV>(lane), voff = v_lane_offset<KV>(nn, r);
  const int G = a.group;
  constexpr int NQK = D / 32;   // QK matrix-core steps (32 dims each)
  constexpr int NDD = D / 16;   // output dim tiles
  const int64_t head_off = (int64_t)g * a.tile_bytes;
  const int64_t block_stride = (int64_t)a.num_kv_heads * a.tile_bytes;
  const int slots = a.batch + a.chunk_slots;

  int xa, xb, rm_unused;
  geo.wave_range(w, xa, xb, rm_unused);
  const int c = w;
  // The chunk holding a sequence's first block records which chunks hold the
  // sequence (for the merge), one sequence per lane, before any tile load:
  // a store issued later would hold up the next load's wait (below).
  if (g == 0 && threadIdx.x < 64 && blockIdx.z == gridDim.z - 1) {
    int b0 = seq_holding(seq_start, a.batch, xa);
    if (seq_start[b0] < xa) ++b0;               // it began in an earlier chunk
    for (int bb = b0 + lane; bb < a.batch; bb += 64) {
      const int s0 = seq_start[bb], s1 = seq_start[bb + 1];
      if (s0 >= xb) break;
      if (s1 > s0) {
        a.ws_seginfo[2 * bb] = c;
        a.ws_seginfo[2 * bb + 1] = geo.chunk_of_block(s1 - 1) - c + 1;
      }
    }
  }
  // Results of segments before the wave's last are kept in this wave's LDS
  // slots (after the scan) and written after the walk: vector memory
  // operations complete in issue order, so a store in the middle of the walk
  // would hold up the next tile load's wait until the memory system
  // acknowledged it, which under the walk's read stream takes microseconds.
  // Per tile of a slot: the accumulator, then (m, l, destination) per lane;
  // a destination is a partial row (>= 0), an output row r as -2 - r, or -1.
  constexpr int TSLOT = NDD * 64 * 16 + 64 * 16;
  char* stage = reinterpret_cast<char*>(seq_start + a.batch + 1);
  stage += ((16 - ((uintptr_t)stage & 15)) & 15) + (threadIdx.x >> 6) * (16 + a.stage_slots * TPW * TSLOT);
  int staged = 0;
  auto flush_tile = [&](int64_t dst, const floatx4* ac, float mm, float lt) {
    if (dst >= 0) write_partial<D>(a, dst, r, ac, mm, lt);
    else if (dst <= -2) write_out_row<KV, D>(a, -2 - dst, r, ac, lt);
  };
  {
    int b = seq_holding(seq_start, a.batch, xa);
    // Everything below that indexes memory is wave-uniform (scalar registers),
    // so block ids and fp8 scales come through scalar loads, which are counted
    // apart from the vector loads of the tiles and never drain the prefetch ring.
    for (int x = xa; x < xb; ++b) {
      const int sb = __builtin_amdgcn_readfirstlane(seq_start[b]);
      const int eb = __builtin_amdgcn_readfirstlane(seq_start[b + 1]);
      if (eb <= x) continue;                      // empty sequence
      const int seg_end = eb < xb ? eb : xb;
      const int first = x - sb;                   // first block of this segment in the sequence's list
      const int count = seg_end - x;              // blocks in this segment
      const int n = __builtin_amdgcn_readfirstlane(attend_len_s(a.context_lens, b, a.max_ctx, a.max_blocks));
      const int ql = __builtin_amdgcn_readfirstlane(query_len(a, b, n));
      if (ct0 * 16 >= ql * G) {                   // no column of this sequence in the wave's tiles
        x = seg_end;
        continue;
      }
      const int q0 = __builtin_amdgcn_readfirstlane(((const_i32_kptr)a.q_start)[b]);
      const int win = a.window;
      // table index of the segment's first block
      const int tb0 = __builtin_amdgcn_readfirstlane(first_visible_block(n, ql, win)) + first;
      // Columns of this lane, one per tile: column 16 ct + nn is (query token
      // tok, head hh); the token sits at position n - ql + tok and sees rows up
      // to n - ql + tok.  With a window a column sees rows [col_lo, ncol),
      // col_lo = ncol - window.  Per tile, n_lo is the fewest rows a column
      // sees, lo_hi the highest window start, and [j0, j1) the blocks of the
      // segment some column of the tile sees; the wave walks their union.
      int hh[TPW], q_row[TPW], ncol[TPW], col_lo[TPW], n_lo[TPW], lo_hi[TPW], j0[TPW], j1[TPW];
      bool head_ok[TPW], active[TPW];
      int J0 = count, J1 = 0;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int ct = ct0 + t;
        active[t] = ct * 16 < ql * G;
        const int col = ct * 16 + nn;
        const int tok = col / G;
        hh[t] = col - tok * G;
        q_row[t] = q0 + tok;
        head_ok[t] = active[t] && tok < ql && q_row[t] >= 0 && q_row[t] < a.total_q;
        n_lo[t] = n - ql + 1 + (ct * 16) / G;
        const int n_hi = n - ql + 1 + min(ql - 1, (ct * 16 + 15) / G);
        // padding columns see all n rows, so they stay finite
        ncol[t] = head_ok[t] ? n - ql + 1 + tok : n;
        col_lo[t] = win > 0 ? max(0, ncol[t] - win) : 0;
        const int lo_lo = win > 0 ? max(0, n_lo[t] - win) : 0;
        lo_hi[t] = win > 0 ? max(0, n_hi - win) : 0;
        j0[t] = max(0, lo_lo / kBS - tb0);
        j1[t] = min(count, (n_hi + kBS - 1) / kBS - tb0);
        if (active[t] && j1[t] > j0[t]) {
          J0 = min(J0, j0[t]);
          J1 = max(J1, j1[t]);
        }
      }
      const int cnt = J1 - J0;                    // blocks the wave walks here (<= 0: none)
      const int tb = tb0 + J0;                    // table index of the first of them

      // Query operands: for step kk the lane holds 8 dims of its column's head,
      // the same dims its K operand holds for token nn.
      u32x4 qv[TPW][NQK];
      floatx4 acc[TPW][NDD];
      float m[TPW], l[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const uint16_t* qh =
            static_cast<const uint16_t*>(a.q) + ((int64_t)q_row[t] * a.num_heads + g * G + hh[t]) * D;
#pragma unroll
        for (int kk = 0; kk < NQK; ++kk) {
          int d0;
          if constexpr (is_byte_code(KV)) d0 = (r + 4 * (kk >> 1)) * 16 + (kk & 1) * 8;
          else d0 = (4 * kk + r) * 8;
          qv[t][kk] = head_ok[t] ? *reinterpret_cast<const u32x4*>(qh + d0) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int dd = 0; dd < NDD; ++dd) acc[t][dd] = floatx4{0.f, 0.f, 0.f, 0.f};
        m[t] = kNegInf;
        l[t] = 0.0f;
      }
      // int8 caches: column score biases and the score scale with the
      // queries' 2^e (see int8_queries)
      float kb[TPW];
      float qk_seg = a.qk_scale;
#pragma unroll
      for (int t = 0; t < TPW; ++t) kb[t] = 0.0f;
      if constexpr (KV == KVC_INT8) qk_seg *= int8_queries<TPW, NQK>(&qv[0][0], kb);

      if (cnt > 0) {
        // Physical block of local block j (scalar load).  Every prefetch is
        // issued, so the count of loads in flight is the same on every path;
        // past the end it re-reads the last block, which the L2 still holds.
        const const_i32_kptr row = (const_i32_kptr)(a.block_table + (int64_t)b * a.max_blocks + tb);
        auto phys_of = [&](int j) -> int {
          j = j < cnt ? j : cnt - 1;
          return clamp_block(ld_u32_index(row, j), a.num_blocks);
        };

        auto process = [&](KvBlock<KV, D>& cur, int i) {
          const int jj = J0 + i;                       // index of this block in the segment
          const int blk_row = (tb + i) * kBS;          // the block's first row
          const int t0 = blk_row + 4 * r;              // this lane's first row
          if (blk_row + kBS > n) zero_rows_past_end<KV, D>(cur, n, t0);
          float qk = qk_seg;
          float vsc = 1.0f;
          BlockOps<KV, D> conv;                        // one-byte codes: converted once, for every tile
          if constexpr (is_byte_code(KV)) {
            qk *= cur.ks;
            vsc = cur.vs;
            convert_codes<KV, D>(cur, conv);
          }
          const u32x4* kop = is_byte_code(KV) ? conv.k : cur.k;
          const u32x2* vop = is_byte_code(KV) ? conv.v : reinterpret_cast<const u32x2*>(cur.v);
#pragma unroll
          for (int t = 0; t < TPW; ++t) {
            // (wave-uniform) this tile sees no row of this block
            if (!active[t] || jj < j0[t] || jj >= j1[t]) continue;
            // Rows some column of the tile may not see exist only near the end
            // of the sequence, or before the window's start (a wave-uniform
            // test): they are masked there.
            const bool edge = blk_row + kBS > n_lo[t] || blk_row < lo_hi[t];
            tile_step<KV, D>(kop, vop, qv[t], acc[t], m[t], l[t], qk, vsc, edge, t0, ncol[t], col_lo[t], kb[t]);
          }
        };

        // Ring of PF + 1 register buffers: block i + PF is in flight while block
        // i is consumed.  The ring index is a compile-time constant after
        // unrolling.
        KvBlock<KV, D> buf[PF + 1];
        auto fetch = [&](KvBlock<KV, D>& dst, int ph) {
          const int64_t o = mul_u32(ph, block_stride) + head_off;
          load_block<KV, D>(dst, a.k + o, a.v + o, koff, voff);
          if constexpr (is_byte_code(KV)) {
            dst.ks = ((const_f32_kptr)a.k_scale)[mul_u32(ph, a.num_kv_heads) + g];
            dst.vs = ((const_f32_kptr)a.v_scale)[mul_u32(ph, a.num_kv_heads) + g];
          }
        };
#pragma unroll
        for (int j = 0; j < PF; ++j) fetch(buf[j], phys_of(j));
        int ph_next = phys_of(PF);                  // id of the next block to prefetch, one step ahead
        // Whole turns of the ring first, with no exit inside a turn: an exit that
        // led back to the loop head would leave a load in flight there and force
        // a full wait for it at the head of every turn.
        int i0 = 0;
        for (; i0 + PF + 1 <= cnt; i0 += PF + 1) {
#pragma unroll
          for (int j = 0; j <= PF; ++j) {
            const int i = i0 + j;
            const int ph = ph_next;
            ph_next = phys_of(i + PF + 1);
            fetch(buf[(j + PF) % (PF + 1)], ph);
            process(buf[j], i);
          }
        }
        // the last, partial turn
#pragma unroll
        for (int j = 0; j < PF; ++j) {
          const int i = i0 + j;
          if (i >= cnt) break;
          const int ph = ph_next;
          ph_next = phys_of(i + PF + 1);
          fetch(buf[(j + PF) % (PF + 1)], ph);
          process(buf[j], i);
        }
      }
      const bool whole = x == sb && seg_end == eb;   // the whole sequence is in this segment
      const bool stage_it = seg_end < xb && staged < a.stage_slots;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        int64_t dst = -1;
        float lt = 0.0f;
        if (active[t]) {
          // l over the head's four lane groups
          lt = sum_over_row_groups(l[t]);
          const int h = g * G + hh[t];
          // partial of (sequence b, chunk c) for this column: slot b + c is
          // unique, since every segment boundary advances the sequence, the
          // chunk, or both; one set of slots per query token index
          if (head_ok[t])
            dst = whole ? -2 - ((int64_t)q_row[t] * a.num_heads + h)
                        : ((int64_t)(q_row[t] - q0) * a.num_heads + h) * slots + b + c;
        }
        if (stage_it) {
          char* sl = stage + (staged * TPW + t) * TSLOT;
#pragma unroll
          for (int dd = 0; dd < NDD; ++dd) *reinterpret_cast<floatx4*>(sl + (dd * 64 + lane) * 16) = acc[t][dd];
          *reinterpret_cast<u32x4*>(sl + NDD * 1024 + lane * 16) =
              u32x4{__builtin_bit_cast(uint32_t, m[t]), __builtin_bit_cast(uint32_t, lt), (uint32_t)dst,
                    (uint32_t)(dst >> 32)};
        } else {
          flush_tile(dst, acc[t], m[t], lt);
        }
      }
      if (stage_it) ++staged;
      x = seg_end;
    }
  }
  // the results kept in LDS, now that no load waits behind their stores
  for (int sidx = 0; sidx < staged; ++sidx) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const char* sl = stage + (sidx * TPW + t) * TSLOT;
      floatx4 ac[NDD];
#pragma unroll
      for (int dd = 0; dd < NDD; ++dd) ac[dd] = *reinterpret_cast<const floatx4*>(sl + (dd * 64 + lane) * 16);
      const u32x4 e = *reinterpret_cast<const u32x4*>(sl + NDD * 1024 + lane * 16);
      // (the elements go through scalars: hipcc's __builtin_bit_cast of a
      // vector element reads element 0 whichever element is named)
      const uint32_t em = e[0], el = e[1], dlo = e[2], dhi = e[3];
      const int64_t dst = (int64_t)(((uint64_t)dhi << 32) | dlo);
      flush_tile(dst, ac, __builtin_bit_cast(float, em), __builtin_bit_cast(float, el));
    }
  }
}

// Decode with one continuous prefetch ring per wave.  A wave walks a sequence
// of ranges of its KV head's block list: its main chunk, then (with a pool)
// the pieces it wins.  A range is cut into segments (its runs of one
// sequence's blocks).  Two cursors walk the ranges: the prefetch cursor runs
// PF + 1 blocks ahead of the process cursor, straight across segment and
// range boundaries, so nothing in flight is drained when a segment or range
// ends; the next segment's query is loaded while the current one runs, and a
// segment change costs its output write.
//
// Pieces are claimed with a per-head ticket counter.  The ring runs in whole
// turns of PF + 1 blocks; the ticket for the range after the prefetch
// cursor's current one is requested at the head of the turn before the one in
// which that cursor reaches the range's end, and read at the next turn's head.
// A turn's worth of tile loads is issued after the request, so the wait for
// its result is a wait for the ticket alone (vector memory results return in
// issue order), not for the tiles in flight.  This needs every range to
// outlast two turns, which the pool's size test below guarantees; then the
// prefetch cursor is also never more than one range ahead of the process
// cursor, so one pending range is handed between them.
// Bytes of one LDS slot holding a finished segment of the decode walk: the
// accumulator (D/16 four-float registers per lane), m and l per lane, and the
// segment's sequence, chunk and kind.
template <int D>
constexpr int stage_slot_bytes() { return (D / 16) * 64 * 16 + 64 * 8 + 16; }

template <kvc_dtype KV, int D, int PF, bool POOL>
__device__ __forceinline__ void decode_stream(const DecodeArgs& a, int* seq_start) {
  constexpr int TURN = PF + 1;
  const int w = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x;
  const int total = __builtin_amdgcn_readfirstlane(scan_block_counts<false>(a, seq_start, lane));
  __syncthreads();
  // never more waves than blocks, so every wave that runs owns >= 1 block
  const int W = a.work_items < total ? a.work_items : total;
  if (w >= W) return;
  // The pool is used when every piece holds >= 2 turns of blocks (a wave's
  // pool is >= floor(total / W) >> shift blocks; the main chunk is at least
  // as long as the pool since shift >= 1).
  const int KP = (POOL && a.pool_pieces > 0 && a.pool_shift >= 1 &&
                  ((total / W) >> a.pool_shift) >= a.pool_pieces * 2 * TURN)
                     ? a.pool_pieces
                     : 0;
  const ChunkGeometry geo{total, W, KP, a.pool_shift};
  int xa, xb_main, r1_unused;
  geo.wave_range(w, xa, r1_unused, xb_main);
  const int nn = lane & 15, r = lane >> 4;
  const uint32_t koff = k_lane_offset<KV>(lane), voff = v_lane_offset<KV>(nn, r);
  const int G = a.group;
  constexpr int NQK = D / 32;
  constexpr int NDD = D / 16;
  const int64_t head_off = (int64_t)g * a.tile_bytes;
  const int64_t block_stride = (int64_t)a.num_kv_heads * a.tile_bytes;
  const int slots = a.batch + a.chunk_slots;
  const bool head_ok = nn < G;
  const int h = g * G + nn;
  const int win = a.window;

  auto seq_len = [&](int bb) -> int {
    return __builtin_amdgcn_readfirstlane(attend_len_s(a.context_lens, bb, a.max_ctx, a.max_blocks));
  };
  auto start_of = [&](int bb) -> int { return __builtin_amdgcn_readfirstlane(seq_start[bb]); };
  // Block-table row of sequence bb indexed by list position: entry x is the
  // physical block of list block x (the list starts at the first visible block).
  auto row_of = [&](int bb, int n_bb) -> const_i32_kptr {
    return (const_i32_kptr)(a.block_table + (int64_t)bb * a.max_blocks + decode_first_block(a, n_bb)) -
           start_of(bb);
  };
  // the first sequence after bb holding a block at or after list position x
  auto next_seq = [&](int bb, int x) -> int {
    do {
      ++bb;
    } while (start_of(bb + 1) <= x);
    return bb;
  };
  auto load_q = [&](u32x4* dst, int bq) {
    const uint16_t* qh = static_cast<const uint16_t*>(a.q) + ((int64_t)bq * a.num_heads + h) * D;
#pragma unroll
    for (int kk = 0; kk < NQK; ++kk) {
      int d0;
      if constexpr (is_byte_code(KV)) d0 = (r + 4 * (kk >> 1)) * 16 + (kk & 1) * 8;
      else d0 = (4 * kk + r) * 8;
      dst[kk] = head_ok ? *reinterpret_cast<const u32x4*>(qh + d0) : u32x4{0, 0, 0, 0};
    }
  };

  // ---- process cursor: block xp of the segment of sequence b, [x0, seg_end),
  // in the range ending at xbp with chunk id c ----
  int b = seq_holding(seq_start, a.batch, xa);
  int xp = xa, xbp = xb_main, c = w * (KP + 1);
  // (row0: the table index of list block 0 in sequence b, so list block x
  // holds rows (row0 + x) * 16 ..)
  int seg_end = 0, n = 0, row0 = 0, lo_hi = 0, nb_q = -1;
  u32x4 q[NQK], q_next[NQK];
  floatx4 acc[NDD];
  float m = kNegInf, l = 0.0f;
  // int8 caches: the column's score bias and the score scale with the
  // query's 2^e (see int8_queries)
  float kb = 0.0f, qk_seg = a.qk_scale;
  // Wave-uniform flags, one word (scalar registers are the scarce resource here).
  // The next range [na, nb) with id nc (its first block in sequence nbf) is
  // named by the prefetch cursor's ticket, entered by that cursor (F_NEXT
  // cleared, F_PEND set), then by the process cursor (F_PEND cleared); a new
  // ticket is read only after both, so the two cursors share these registers.
  constexpr int F_MORE = 1;   // a pool piece may still come
  constexpr int F_REQ = 2;    // a ticket request is in flight
  constexpr int F_NEXT = 4;   // the range after the prefetch cursor's is known
  constexpr int F_PEND = 8;   // the prefetch cursor has entered a range the process cursor has not
  constexpr int F_LAST = 16;  // the process cursor's segment is its range's last
  constexpr int F_WHOLE = 32; // the segment is its sequence's whole list
  constexpr int F_STAGED = 256; // bits 8 and up: segments kept in LDS so far
  int flags = KP != 0 ? F_MORE : 0;
  int na = 0, nb = 0, nc = 0, nbf = 0;

  // The chunk holding a sequence's first block records which chunks hold the
  // sequence (for the merge): done for a whole range when it is taken, one
  // sequence per lane.
  auto record_range = [&](int ra, int rb, int cc) {
    if (g != 0) return;
    int b0 = seq_holding(seq_start, a.batch, ra);
    if (start_of(b0) < ra) ++b0;               // it began in an earlier chunk
    for (int bb = b0 + lane; bb < a.batch; bb += 64) {
      const int s0 = seq_start[bb], s1 = seq_start[bb + 1];
      if (s0 >= rb) break;
      if (s1 > s0) {
        a.ws_seginfo[2 * bb] = cc;
        a.ws_seginfo[2 * bb + 1] = geo.chunk_of_block(s1 - 1) - cc + 1;
      }
    }
  };

  // ---- prefetch cursor: list block xf of sequence bf, in a range ending at xbf ----
  int xf = xa, xbf = xb_main, bf = b, ebf = start_of(b + 1);
  const_i32_kptr rowf = row_of(b, seq_len(b));
  int ph_last = 0;
  int left = 0;                                // blocks named by the prefetch cursor, not yet processed
  int ticket = 0;                              // lane 0: the requested ticket

  // set up the segment of sequence b starting at list block x; its query is
  // already in q.  The next segment's query (or the next range's first) is
  // requested now when known.
  auto begin = [&](int x) {
    const int sb = start_of(b), eb = start_of(b + 1);
    seg_end = eb < xbp ? eb : xbp;
    flags = (x == sb && seg_end == eb && !a.partials_only) ? (flags | F_WHOLE) : (flags & ~F_WHOLE);
    n = seq_len(b);
    row0 = decode_first_block(a, n) - sb;
    lo_hi = win > 0 ? max(0, n - win) : 0;
#pragma unroll
    for (int dd = 0; dd < NDD; ++dd) acc[dd] = floatx4{0.f, 0.f, 0.f, 0.f};
    m = kNegInf;
    l = 0.0f;
    if constexpr (KV == KVC_INT8) qk_seg = a.qk_scale * int8_queries<1, NQK>(q, &kb);
    // the query needed after this segment: the next segment's, or the next
    // range's first when that range is known
    bool want;
    if (seg_end < xbp) {
      flags &= ~F_LAST;
      nb_q = next_seq(b, seg_end);
      want = true;
    } else {
      flags |= F_LAST;
      nb_q = nbf;
      want = POOL && (flags & F_PEND);
    }
    if (want) load_q(q_next, nb_q);
  };
  // The results of segments before the wave's last go to LDS slots and are
  // written out after the walk: vector memory operations complete in issue
  // order, so a store issued in the middle of the walk would hold up every
  // later tile load's wait until the memory system acknowledged it, which
  // under the walk's own read stream takes several microseconds.
  char* stage = reinterpret_cast<char*>(seq_start + a.batch + 1);
  stage += (16 - ((uintptr_t)stage & 15)) & 15;
  constexpr int SSLOT = stage_slot_bytes<D>();
  auto write_result = [&](int bb, int cc, bool whole, const floatx4* ac, float mm, float lt) {
    if (head_ok) {
      if (whole) write_out<KV, D>(a, bb, h, r, ac, lt);
      else write_partial<D>(a, (int64_t)h * slots + bb + cc, r, ac, mm, lt);
    }
  };
  // after the segment's last block: write it out (or keep it in LDS), move
  // to the next segment
  auto finish = [&]() {
    const float lt = sum_over_row_groups(l);
    const bool final_write = (flags & F_LAST) && (!POOL || !(flags & F_PEND));
    const int ns = flags / F_STAGED;
    if (!POOL && !final_write && ns < a.stage_slots) {
      char* sl = stage + ns * SSLOT;
#pragma unroll
      for (int dd = 0; dd < NDD; ++dd) *reinterpret_cast<floatx4*>(sl + (dd * 64 + lane) * 16) = acc[dd];
      *reinterpret_cast<floatx2*>(sl + NDD * 1024 + lane * 8) = floatx2{m, lt};
      if (lane == 0)
        *reinterpret_cast<u32x4*>(sl + NDD * 1024 + 512) =
            u32x4{(uint32_t)b, (uint32_t)c, (flags & F_WHOLE) ? 1u : 0u, 0u};
      flags += F_STAGED;
    } else {
      write_result(b, c, (flags & F_WHOLE) != 0, acc, m, lt);
    }
    if (flags & F_LAST) {
      if (!POOL || !(flags & F_PEND)) return;  // the wave's last range is done
      flags &= ~F_PEND;                        // on to the next range
      nb_q = nbf;
      xp = na;
      xbp = nb;
      c = nc;
    }
    b = nb_q;
#pragma unroll
    for (int kk = 0; kk < NQK; ++kk) q[kk] = q_next[kk];
    begin(xp);
  };
  // physical id of the next block to fetch; past the last range's end the
  // last one again (the L2 still holds it), so every step issues the same loads
  auto next_phys = [&]() -> int {
    if (POOL && xf == xbf && (flags & F_NEXT)) {  // enter the next range
      flags = (flags & ~F_NEXT) | F_PEND;
      xf = na;
      xbf = nb;
      bf = nbf;
      ebf = start_of(bf + 1);
      rowf = row_of(bf, seq_len(bf));
      if (flags & F_LAST) load_q(q_next, nbf);  // the process cursor is in its range's last segment
    }
    if (xf < xbf) {
      if (xf == ebf) {
        bf = next_seq(bf, xf);
        ebf = start_of(bf + 1);
        rowf = row_of(bf, seq_len(bf));
      }
      ph_last = clamp_block(ld_u32_index(rowf, xf), a.num_blocks);
      ++xf;
      ++left;
    }
    return ph_last;
  };
  auto process = [&](KvBlock<KV, D>& cur) {
    const int blk_row = (row0 + xp) * kBS;         // the block's first row
    const int t0 = blk_row + 4 * r;               // this lane's first row
    if (blk_row + kBS > n) zero_rows_past_end<KV, D>(cur, n, t0);
    float qk = qk_seg;
    float vsc = 1.0f;
    BlockOps<KV, D> conv;
    if constexpr (is_byte_code(KV)) {
      qk *= cur.ks;
      vsc = cur.vs;
      convert_codes<KV, D>(cur, conv);
    }
    const u32x4* kop = is_byte_code(KV) ? conv.k : cur.k;
    const u32x2* vop = is_byte_code(KV) ? conv.v : reinterpret_cast<const u32x2*>(cur.v);
    const bool edge = blk_row + kBS > n || blk_row < lo_hi;
    tile_step<KV, D>(kop, vop, q, acc, m, l, qk, vsc, edge, t0, n, lo_hi, kb);
    ++xp;
    --left;
    if (xp == seg_end) finish();
  };

  // The step's append folded into the walk: the wave whose main chunk holds a
  // sequence's last block writes that sequence's newest row of this KV head
  // (each (block, head) tile is read by exactly one wave, so no other wave
  // reads it) before it loads any tile.  Its own later loads of that tile
  // then see the stores: a work-group-scope fence orders them (on gfx950
  // that takes no wait; a CU keeps one work-group's accesses in order).
  if (!POOL && a.k_new) {
    constexpr int X = 8;                          // 16-bit elements per 16-byte chunk
    bool wrote = false;
    for (int bb = b; bb < a.batch; ++bb) {
      const int sb = start_of(bb), eb = start_of(bb + 1);
      if (sb >= xb_main) break;
      if (eb <= sb || eb - 1 < xa || eb - 1 >= xb_main) continue;   // last block in another chunk
      const int pos = seq_len(bb) - 1;
      const int blk = ((const_i32_kptr)(a.block_table + (int64_t)bb * a.max_blocks))[pos / kBS];
      if (blk < 0 || blk >= a.num_blocks) continue;                 // a bad table entry: no write
      const int off = pos % kBS;
      const int64_t t = (int64_t)blk * block_stride + head_off;
      // the pools are written only here, by the tile's one reader
      char* kt = const_cast<char*>(a.k) + t;
      char* vt = const_cast<char*>(a.v) + t;
      const int64_t src = ((int64_t)bb * a.num_kv_heads + g) * D * 2;
      if (lane < D / X)
        *reinterpret_cast<u32x4*>(kt + ((int64_t)lane * kBS + off) * 16) =
            *reinterpret_cast<const u32x4*>(a.k_new + src + lane * 16);
#pragma unroll
      for (int d = lane; d < D; d += 64)
        *reinterpret_cast<uint16_t*>(vt + ((int64_t)d * kBS + off) * 2) =
            *reinterpret_cast<const uint16_t*>(a.v_new + src + d * 2);
      wrote = true;
    }
    if (wrote) __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  }
  record_range(xa, xb_main, c);
  load_q(q, b);
  begin(xa);
  KvBlock<KV, D> buf[TURN];
  auto fetch = [&](KvBlock<KV, D>& dst, int ph) {
    const int64_t o = mul_u32(ph, block_stride) + head_off;
    load_block<KV, D>(dst, a.k + o, a.v + o, koff, voff);
    if constexpr (is_byte_code(KV)) {
      dst.ks = ((const_f32_kptr)a.k_scale)[mul_u32(ph, a.num_kv_heads) + g];
      dst.vs = ((const_f32_kptr)a.v_scale)[mul_u32(ph, a.num_kv_heads) + g];
    }
  };
#pragma unroll
  for (int j = 0; j < PF; ++j) fetch(buf[j], next_phys());
  int ph_next = next_phys();                  // one step ahead
  // Whole turns while TURN named blocks wait (every block a turn processes is
  // real); fewer means the last range has been named to its end.
  while (left >= TURN) {
    // The prefetch cursor names blocks xf .. xf + PF in this turn.
    if (POOL && (flags & F_REQ) && xbf - xf <= PF) {  // it reaches its range's end: the next range is needed
      const int t = __builtin_amdgcn_readfirstlane(ticket);
      flags &= ~F_REQ;
      if (t < W * KP) {
        geo.piece(t, na, nb, nc);
        nbf = seq_holding(seq_start, a.batch, na);
        record_range(na, nb, nc);
        flags |= F_NEXT;
      } else {
        flags &= ~F_MORE;
      }
    }
    // it does so in the next turn (a request is made only then, so its answer
    // always comes in time to be used)
    if (POOL && (flags & (F_MORE | F_REQ | F_NEXT)) == F_MORE && xbf - xf > PF && xbf - xf <= PF + TURN) {
      if (lane == 0) ticket = atomicAdd(a.ws_ticket + g, 1);
      flags |= F_REQ;
    }
#pragma unroll
    for (int j = 0; j < TURN; ++j) {
      const int ph = ph_next;
      ph_next = next_phys();
      fetch(buf[(j + PF) % TURN], ph);
      process(buf[j]);
    }
  }
  const int rest = left;
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    if (j >= rest) break;
    const int ph = ph_next;
    ph_next = next_phys();
    fetch(buf[(j + PF) % TURN], ph);
    process(buf[j]);
  }
  // the results kept in LDS, now that no load waits behind their stores
  if constexpr (!POOL) {
    const int ns = flags / F_STAGED;
    for (int sidx = 0; sidx < ns; ++sidx) {
      const char* sl = stage + sidx * SSLOT;
      const u32x4 meta = *reinterpret_cast<const u32x4*>(sl + NDD * 1024 + 512);
      const int bb = __builtin_amdgcn_readfirstlane((int)meta[0]);
      const int cc = __builtin_amdgcn_readfirstlane((int)meta[1]);
      const bool whole = __builtin_amdgcn_readfirstlane((int)meta[2]) != 0;
      floatx4 ac[NDD];
#pragma unroll
      for (int dd = 0; dd < NDD; ++dd) ac[dd] = *reinterpret_cast<const floatx4*>(sl + (dd * 64 + lane) * 16);
      const floatx2 ml = *reinterpret_cast<const floatx2*>(sl + NDD * 1024 + lane * 8);
      write_result(bb, cc, whole, ac, ml[0], ml[1]);
    }
  }
}

template <kvc_dtype KV, int D, int PF, bool POOL>
__global__ __launch_bounds__(64) void decode_stream_kernel(DecodeArgs a) {
  extern __shared__ int seq_start[];   // [batch + 1]
  decode_stream<KV, D, PF, POOL>(a, seq_start);
}

// grid (work items, KV heads, tile groups), waves_per_group waves each, TPW
// column tiles per wave
template <kvc_dtype KV, int D, int PF, int TPW>
__global__ __launch_bounds__(256) void extend_mfma_kernel(DecodeArgs a) {
  extern __shared__ int seq_start[];   // [batch + 1]
  attend_extend<KV, D, PF, TPW>(a, seq_start);
}

// ---------------------------------------------------------------------------
// Several query tokens per sequence, many of them (a prompt, a long chunk):
// one wave per 32 (token, head) columns of one sequence and KV head, WT waves
// (consecutive column tiles) per work-group sharing every K/V step through
// LDS.  The work-group walks every row its columns see, 32 rows (two blocks)
// per step, on 32x32x16 matrix-core tiles, and writes the outputs itself: a
// long run of new tokens has enough column tiles to fill the chip without
// splitting the rows (with too few, each group's steps are cut into pieces).
//
// Scores: S^T[32 rows x 32 columns] = K[32 rows x D] . Q^T[D x 32 columns].
// Operand and result layouts of the 32x32x16 step: lane l holds A[l % 32][8
// (l / 32) + i] and B[8 (l / 32) + i][l % 32] (i = 0..7), and result element
// 4 g + j of lane l is C[8 g + 4 (l / 32) + j][l % 32].  The rows of a block
// enter S^T in the order rho(r) = r with bits 2 and 3 swapped, so lane l's
// results for block s (g = 2 s, 2 s + 1) are its column's weights for tokens
// 8 (l / 32) .. 8 (l / 32) + 7 of block s in order: exactly the P^T operand of
// O^T[D x 32] += V^T[D x 16] . P^T[16 x 32] for that block, whose V^T operand
// is then those 8 tokens of one dim of the transposed V tile, one load.
// ---------------------------------------------------------------------------
typedef float floatx16 __attribute__((ext_vector_type(16)));

template <kvc_dtype KV>
__device__ __forceinline__ floatx16 mfma32(const u32x4& a, const u32x4& b, floatx16 c) {
  if constexpr (KV == KVC_F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                   0);
}

// eight one-byte codes -> eight bf16 (unit scale)
template <kvc_dtype KV>
__device__ __forceinline__ u32x4 codes8_to_bf16(const u32x2& w) {
  return u32x4{code2_to_bf16x2<KV, false>(w[0]), code2_to_bf16x2<KV, true>(w[0]), code2_to_bf16x2<KV, false>(w[1]),
               code2_to_bf16x2<KV, true>(w[1])};
}

// Raw tiles of one step, as loaded: K (D/16 k-steps) and V^T (D/32 dim tiles x
// 2 blocks); 16 bytes per piece for 16-bit caches, 8 for one-byte codes.
template <kvc_dtype KV, int D>
struct FlashK {
  typename std::conditional<is_byte_code(KV), u32x2, u32x4>::type k[D / 16];
  float ks0, ks1;   // one-byte codes: the two blocks' K scales
};
template <kvc_dtype KV, int D>
struct FlashV {
  typename std::conditional<is_byte_code(KV), u32x2, u32x4>::type v[D / 32][2];
  float vs0, vs1;   // one-byte codes: the two blocks' V scales
};

// The rows that columns ct * cols .. ct * cols + cols - 1 of a sequence see
// (a 32-column tile, or a work-group's tiles): table blocks [jb0, jb1), two
// per step; n_lo / n_hi the fewest / most rows one of the columns sees, lo_lo /
// lo_hi the lowest / highest window start.
struct FlashTile {
  int n_lo, n_hi, lo_lo, lo_hi, jb0, jb1, nsteps;
};
__device__ __forceinline__ FlashTile flash_tile(int n, int ql, int G, int win, int ct, int cols, bool noncausal) {
  FlashTile t;
  const int tok_first = (ct * cols) / G;
  const int tok_last = min(ql - 1, (ct * cols + cols - 1) / G);
  t.n_lo = noncausal ? n : n - ql + 1 + tok_first;
  t.n_hi = noncausal ? n : n - ql + 1 + tok_last;
  t.lo_lo = win > 0 ? max(0, t.n_lo - win) : 0;
  t.lo_hi = win > 0 ? max(0, t.n_hi - win) : 0;
  t.jb0 = t.lo_lo / kBS;
  t.jb1 = (t.n_hi + kBS - 1) / kBS;
  t.nsteps = (t.jb1 - t.jb0 + 1) >> 1;
  return t;
}

// pieces of a tile of nsteps steps (one when its rows are not cut)
__device__ __forceinline__ int flash_pieces(int nsteps, int split_steps) {
  return split_steps > 0 ? (nsteps + split_steps - 1) / split_steps : 1;
}

// The several-token kernel's P operand: a 16-bit hi part plus a 16-bit lo
// part (1), as in decode, or the hi part alone (0).
#ifndef KVC_FLASH_P_LO
#define KVC_FLASH_P_LO 1
#endif

// 16-bit caches: each step's tiles go from HBM straight into LDS
// (global_load_lds, no registers in between), three steps deep (1), or
// through registers, two deep (0).
#ifndef KVC_FLASH_DMA
#define KVC_FLASH_DMA 1
#endif
#ifndef KVC_FLASH_STAGES
#define KVC_FLASH_STAGES 3
#endif

// One 16-byte load of every lane of the wave straight into LDS: lane i's 16
// bytes from src go to LDS byte lds_wave_base + 16 i (lds_wave_base
// wave-uniform).  The caller waits for it with vm_wait (it counts on the
// vector-memory counter like any load) and makes it visible to the other
// waves with a barrier.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(uintptr_t)lds_wave_base, 16, 0, 0);
}
// s_barrier with no fence: the callers order their own LDS and memory traffic
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// K piece r16 = 16 * dim group + score row of a block -> its piece in the
// stored tile, 16 * dim group + token (the token of score row r is rho(r))
__device__ __forceinline__ int k_piece(int r16) {
  const int r = r16 & 15;
  return (r16 & ~15) | (r & 3) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// position of K chunk j of score row r: j ^ ksw<CR>(r), CR chunks per row
template <int CR>
__device__ __forceinline__ int ksw(int r) {
  return (r / (16 / CR)) & (CR - 1);
}

template <kvc_dtype KV, int D, int WT>
__global__ __launch_bounds__(64 * WT) void extend_flash_kernel(DecodeArgs a) {
  constexpr int NK = D / 16;                  // k-steps of the score product
  constexpr int NO = D / 32;                  // 32-dim tiles of the output
  constexpr int NT = 64 * WT;                 // threads of the work-group
  // One step's tiles in LDS, as 16-bit values (one-byte codes converted on the
  // way in).  K: 32 rows (in score-tile order) x D, V^T: D rows x 32 tokens.
  // Rows are padded by 16 bytes so the 16-byte operand reads of 8 consecutive
  // lanes (8 consecutive rows) fall in 8 distinct groups of 4 banks.
  constexpr int KROW = 2 * D + 16, VROW = 2 * 32 + 16;
  constexpr int KBYTES = 32 * KROW, STAGE = KBYTES + D * VROW;
  // Loaded straight into LDS (16-bit caches) the rows cannot be padded (one
  // load instruction fills 1 KB contiguously), so the 16-byte chunks of a row
  // are permuted instead: K chunk j (dims 8j .. 8j + 7) of score row r sits at
  // position j ^ ksw(r) of its 2D-byte row, V^T chunk q (tokens 8q .. 8q + 7
  // of the step) of dim d at position q ^ ((d >> 2) & 3) of its 64-byte row;
  // either way the operand reads of 16 consecutive lanes hit 16 distinct
  // groups of banks.
  constexpr bool DMA = KVC_FLASH_DMA && !is_byte_code(KV);
  constexpr int RK = 2 * D, CR = RK / 16;             // K row bytes, 16-byte chunks per row
  constexpr int KBYTES_D = 32 * RK, STAGE_D = KBYTES_D + D * 64;
  // (eight waves: two steps per barrier, in two halves of two stages)
  constexpr int NSTAGE = DMA ? (WT == 8 ? 4 : KVC_FLASH_STAGES) : 2, SBYTES = DMA ? STAGE_D : STAGE, KOFF = DMA ? KBYTES_D : KBYTES;
  static_assert(NSTAGE == 2 || NSTAGE == 3 || NSTAGE == 4, "2 to 4 stages");
  constexpr int PERD = STAGE_D / (16 * NT);           // loads per thread and step, straight to LDS
  static_assert(STAGE_D % (16 * NT) == 0 && (32 * CR) % 64 == 0, "whole loads per stage, K and V per wave");
  __shared__ __attribute__((aligned(16))) char lds[NSTAGE * SBYTES];
  // global pieces of one step: 16 bytes each, both blocks, K then V
  constexpr int CHB = is_byte_code(KV) ? D : 2 * D;   // 16-byte pieces per (block, head) tile
  constexpr int PER = 2 * 2 * CHB / NT;               // per thread (K and V, two blocks)
  static_assert(2 * 2 * CHB % NT == 0, "pieces per thread");

  // grid (KV head, group rank and piece, sequence): in dispatch order a
  // sequence's work-groups follow each other, so the work-groups resident on
  // an XCD (all of one KV head: consecutive work-groups go to consecutive
  // XCDs) span few sequences and share their K/V rows in its L2 (chunk
  // workload: HBM bytes 1.0x the algorithmic ones, against 1.47x with the
  // sequences innermost)
  const int g = blockIdx.x, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, c32 = lane & 31;
  // Without the causal mask (a shared prefix's pass) there is one sequence of
  // max_ctx rows whose query rows are the total_q (<= max_q) rows of q.
  const bool noncausal = a.noncausal != 0;
  const int n = __builtin_amdgcn_readfirstlane(noncausal ? min(a.max_ctx, a.max_blocks * kBS)
                                                         : attend_len(a.context_lens, b, a.max_ctx, a.max_blocks));
  if (n <= 0) return;
  const int ql = __builtin_amdgcn_readfirstlane(noncausal ? min(a.max_q, a.total_q) : query_len(a, b, n));
  const int G = a.group;
  const int win = a.window;
  const int ntiles = (ql * G + 31) / 32;
  const int ngroups = (ntiles + WT - 1) / WT;
  // grid.y = (group rank, piece); rank 0 is the sequence's last group of
  // tiles: under the causal mask the last tokens see the most rows, so the
  // longest work-groups of a sequence start first
  const int rank = (int)blockIdx.y / a.max_pieces, piece = (int)blockIdx.y - rank * a.max_pieces;
  const int cg = ngroups - 1 - rank;
  if (cg < 0) return;
  // the rows the group walks: the union of its tiles' rows
  const FlashTile grp = flash_tile(n, ql, G, win, cg, 32 * WT, noncausal);
  const int npieces = flash_pieces(grp.nsteps, a.split_steps);
  if (piece >= npieces) return;
  const int jb0 = grp.jb0, jb1 = grp.jb1;
  const int s_begin = npieces > 1 ? piece * a.split_steps : 0;
  const int s_end = npieces > 1 ? min(grp.nsteps, s_begin + a.split_steps) : grp.nsteps;
  const int q0 = noncausal ? 0 : __builtin_amdgcn_readfirstlane(((const_i32_kptr)a.q_start)[b]);

  // this wave's tile and this lane's column: token tok, head hh of the group
  const int ct = cg * WT + wave;
  const bool tile_ok = ct < ntiles;
  const int col = ct * 32 + c32;
  const int tok = col / G, hh = col - tok * G;
  const int q_row = q0 + tok;
  const bool col_ok = tile_ok && tok < ql && q_row >= 0 && q_row < a.total_q;
  const int h = g * G + hh;
  // rows the column sees: [col_lo, ncol) (a padding column sees all n rows)
  const int ncol = (col_ok && !noncausal) ? n - ql + 1 + tok : n;
  const int col_lo = win > 0 ? max(0, ncol - win) : 0;
  // the wave's own rows: steps outside them are skipped, steps inside them
  // with no masked row run the plain body
  const FlashTile own = flash_tile(n, ql, G, win, tile_ok ? ct : cg * WT, 32, noncausal);
  const int w_lo = own.lo_lo, w_hi = own.n_hi, n_lo = own.n_lo, lo_hi = own.lo_hi;

  const int64_t head_off = (int64_t)g * a.tile_bytes;
  const int64_t block_stride = (int64_t)a.num_kv_heads * a.tile_bytes;
  const const_i32_kptr row = (const_i32_kptr)(a.block_table + (int64_t)b * a.max_blocks);

  // Q^T operand: dims 16 kk + 8 half .. + 7 of the lane's column
  u32x4 qv[NK];
  {
    const uint16_t* qh = static_cast<const uint16_t*>(a.q) + ((int64_t)q_row * a.num_heads + h) * D;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      qv[kk] = col_ok ? *reinterpret_cast<const u32x4*>(qh + 16 * kk + 8 * half) : u32x4{0, 0, 0, 0};
  }
  // With loads straight into LDS in flight the vector-memory counter counts
  // them too: take the queries in now, so no wait for them lands in the loop.
  if constexpr (DMA) vm_wait<0>();

  // Block ids of a step, read a step before its tiles are requested (scalar
  // loads complete out of order: their first use waits for all in flight).
  struct Ids {
    int p0, p1;
  };
  auto phys = [&](int j) -> int {   // table block j, or block jb0 past the end (its rows are all masked)
    return clamp_block(ld_u32_index(row, j < jb1 ? j : jb0), a.num_blocks);
  };
  auto ids_of = [&](int st) -> Ids {
    st = st < s_end ? st : s_end - 1;
    return Ids{phys(jb0 + 2 * st), phys(jb0 + 2 * st + 1)};
  };
  // one step's global pieces held between their load and their LDS store,
  // with the blocks' scales for one-byte codes
  struct Staged {
    u32x4 w[PER];
    float ks0, ks1, vs0, vs1;
  };
  auto load_stage = [&](Staged& r, const Ids& id) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NT;                 // piece: K pieces first, then V
      const bool is_v = c >= 2 * CHB;
      const int cc = is_v ? c - 2 * CHB : c;
      const int blk = cc / CHB, r16 = cc - blk * CHB;
      const char* base = (is_v ? a.v : a.k) + mul_u32(blk ? id.p1 : id.p0, block_stride) + head_off;
      r.w[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)(is_v ? r16 : k_piece(r16)) * 16);
    }
    if constexpr (is_byte_code(KV)) {
      r.ks0 = ((const_f32_kptr)a.k_scale)[mul_u32(id.p0, a.num_kv_heads) + g];
      r.ks1 = ((const_f32_kptr)a.k_scale)[mul_u32(id.p1, a.num_kv_heads) + g];
      r.vs0 = ((const_f32_kptr)a.v_scale)[mul_u32(id.p0, a.num_kv_heads) + g];
      r.vs1 = ((const_f32_kptr)a.v_scale)[mul_u32(id.p1, a.num_kv_heads) + g];
    }
  };
  // Store one step's pieces into LDS buffer buf.  K row of block blk, token t
  // goes to score row 16 blk + rho(t) (rho swaps bits 2 and 3 of t, its own
  // inverse); consecutive threads take consecutive score rows (k_piece), so
  // eight lanes' 16-byte stores land in eight distinct groups of banks.  V^T
  // keeps its dims as rows.  V values of rows past the
  // sequence's end (which may hold anything, NaN included) are zeroed: their
  // weight is 0, and 0 times NaN would still be NaN.
  auto store_stage = [&](const Staged& r, int buf, int k0) {
    char* kl = lds + buf * SBYTES;
    char* vl = kl + KBYTES;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NT;
      const bool is_v = c >= 2 * CHB;
      const int cc = is_v ? c - 2 * CHB : c;
      const int blk = cc / CHB, r16 = cc - blk * CHB;
      if constexpr (is_byte_code(KV)) {
        // 16 codes: K [D/16][16 tokens][16 dims], V [D][16 tokens]
        const u32x4 w = r.w[i];
        u32x4 lo = u32x4{code2_to_bf16x2<KV, false>(w[0]), code2_to_bf16x2<KV, true>(w[0]),
                         code2_to_bf16x2<KV, false>(w[1]), code2_to_bf16x2<KV, true>(w[1])};
        u32x4 hi = u32x4{code2_to_bf16x2<KV, false>(w[2]), code2_to_bf16x2<KV, true>(w[2]),
                         code2_to_bf16x2<KV, false>(w[3]), code2_to_bf16x2<KV, true>(w[3])};
        if (!is_v) {
          const int dg = r16 >> 4, rr = 16 * blk + (r16 & 15);
          *reinterpret_cast<u32x4*>(kl + rr * KROW + dg * 32) = lo;
          *reinterpret_cast<u32x4*>(kl + rr * KROW + dg * 32 + 16) = hi;
        } else {
          const int d = r16, t0 = k0 + 16 * blk;
          if (t0 + 16 > n) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              lo[e] &= ((t0 + 2 * e < n) ? 0xFFFFu : 0u) | ((t0 + 2 * e + 1 < n) ? 0xFFFF0000u : 0u);
              hi[e] &= ((t0 + 8 + 2 * e < n) ? 0xFFFFu : 0u) | ((t0 + 8 + 2 * e + 1 < n) ? 0xFFFF0000u : 0u);
            }
          }
          *reinterpret_cast<u32x4*>(vl + d * VROW + 32 * blk) = lo;
          *reinterpret_cast<u32x4*>(vl + d * VROW + 32 * blk + 16) = hi;
        }
      } else {
        // 8 values: K [D/8][16 tokens][8 dims], V [D][16 tokens] (two pieces per dim)
        u32x4 w = r.w[i];
        if (!is_v) {
          const int dg = r16 >> 4, rr = 16 * blk + (r16 & 15);
          *reinterpret_cast<u32x4*>(kl + rr * KROW + dg * 16) = w;
        } else {
          const int d = r16 >> 1, hv = r16 & 1;
          const int t0 = k0 + 16 * blk + 8 * hv;
          if (t0 + 8 > n) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              w[e] &= ((t0 + 2 * e < n) ? 0xFFFFu : 0u) | ((t0 + 2 * e + 1 < n) ? 0xFFFF0000u : 0u);
          }
          *reinterpret_cast<u32x4*>(vl + d * VROW + 32 * blk + 16 * hv) = w;
        }
      }
    }
  };

  floatx16 acc[NO];
#pragma unroll
  for (int od = 0; od < NO; ++od)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[od][e] = 0.0f;
  float m = kNegInf, l = 0.0f;

  // One step of this wave: scores from the K rows in LDS, softmax, PV with the
  // V^T rows.  EDGE (compile time): the step holds rows some column must not
  // see (the causal edge, the window's start, the sequence's end); every
  // other step is a plain one with no per-element tests.
  auto step = [&](auto edge_c, int buf, int k0, const Staged& sc) {
    constexpr bool EDGE = decltype(edge_c)::value;
    const char* kl = lds + buf * SBYTES;
    const char* vl = kl + KOFF;
    floatx16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const u32x4 kop = DMA ? *reinterpret_cast<const u32x4*>(kl + c32 * RK + 16 * ((2 * kk + half) ^ ksw<CR>(c32)))
                            : *reinterpret_cast<const u32x4*>(kl + c32 * KROW + 32 * kk + 16 * half);
      s = mfma32<KV>(kop, qv[kk], s);
    }
    bool vis[16];
    if constexpr (EDGE) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int gi = e >> 2;
        const int key = k0 + 16 * (gi >> 1) + 8 * half + 4 * (gi & 1) + (e & 3);
        vis[e] = key < ncol && key >= col_lo;
        if (!vis[e]) s[e] = kNegInf;
      }
    }
    // Scale per block (softmax scale * log2 e, times the K scale for one-byte
    // codes): both are >= 0, so a block's max of the raw scores, scaled, is
    // its max of the scaled scores, and exp2(s * qk - m) is one fma.
    float qk0 = a.qk_scale, qk1 = a.qk_scale;
    if constexpr (is_byte_code(KV)) {
      qk0 *= sc.ks0;
      qk1 *= sc.ks1;
    }
    float m0 = s[0], m1 = s[8];
#pragma unroll
    for (int e = 1; e < 8; ++e) {
      m0 = fmaxf(m0, s[e]);
      m1 = fmaxf(m1, s[8 + e]);
    }
    // (-inf * 0 is NaN: fmaxf keeps the other operand, and a column with no
    // visible row in the step keeps its reference). Both halves of the wave
    // hold the same column and reference, so the column's max exceeds the
    // reference exactly when one half's does: the swap is needed only then.
    float mx = fmaxf(m0 * qk0, m1 * qk1);
    if (__any(mx > m + kRescaleThreshold)) {
      {
        const uint32_t xb = __float_as_uint(mx);
        const auto p32 = __builtin_amdgcn_permlane32_swap(xb, xb, false, false);
        mx = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
      }
      const bool grow = mx > m + kRescaleThreshold;
      const float mnew = grow ? mx : m;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m - mnew) : 1.0f;
      l *= alpha;
#pragma unroll
      for (int od = 0; od < NO; ++od) acc[od] *= alpha;
      m = mnew;
    }
    float pv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], e < 8 ? qk0 : qk1, -m));
      if constexpr (EDGE) {
        if (!vis[e]) pv[e] = 0.0f;
      }
    }
    l += (((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]))) +
         (((pv[8] + pv[9]) + (pv[10] + pv[11])) + ((pv[12] + pv[13]) + (pv[14] + pv[15])));
    // the PV products at raised wave priority: the SIMD's other wave (another
    // work-group) does its softmax meanwhile (measured ~2% faster)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      float w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        w[i] = pv[8 * s2 + i];
        if constexpr (is_byte_code(KV)) w[i] *= (s2 == 0 ? sc.vs0 : sc.vs1);
      }
      // P^T operand as a 16-bit hi part plus (KVC_FLASH_P_LO) a 16-bit lo part
      u32x4 pb, pl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (KV == KVC_F16) {
          pb[i] = pack_f16x2(w[2 * i], w[2 * i + 1]);
          if constexpr (KVC_FLASH_P_LO) pl[i] = pack_f16x2(w[2 * i] - f16_lo(pb[i]), w[2 * i + 1] - f16_hi(pb[i]));
        } else {
          if constexpr (KVC_FLASH_P_LO) {
            uint32_t hi, lo;
            split_bf16x2(w[2 * i], w[2 * i + 1], hi, lo);
            pb[i] = hi;
            pl[i] = lo;
          } else {
            pb[i] = pack_bf16x2(w[2 * i], w[2 * i + 1]);
          }
        }
      }
#pragma unroll
      for (int od = 0; od < NO; ++od) {
        u32x4 vop;
        if constexpr (DMA) {
          vop = *reinterpret_cast<const u32x4*>(vl + (32 * od + c32) * 64 + 16 * ((2 * s2 + half) ^ ((c32 >> 2) & 3)));
          if constexpr (EDGE) {
            // rows past the sequence's end came in as they lie in the block
            // (anything, NaN included): their weight is 0, and 0 times NaN
            // would still be NaN
            const int t0 = k0 + 16 * s2 + 8 * half;
            if (t0 + 8 > n) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                vop[e] &= ((t0 + 2 * e < n) ? 0xFFFFu : 0u) | ((t0 + 2 * e + 1 < n) ? 0xFFFF0000u : 0u);
            }
          }
        } else {
          vop = *reinterpret_cast<const u32x4*>(vl + (32 * od + c32) * VROW + 32 * s2 + 16 * half);
        }
        acc[od] = mfma32<KV>(vop, pb, acc[od]);
        if constexpr (KVC_FLASH_P_LO) acc[od] = mfma32<KV>(vop, pl, acc[od]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // One step's tiles straight into LDS stage stg: load i of thread tid
  // fills stage chunk i * NT + tid (K chunks first, then V^T), so each load
  // instruction of a wave fills 64 consecutive chunks.
  auto dma_stage = [&](int stg, Ids id) {
    char* base = lds + stg * SBYTES;
    // the two blocks' tiles of this head (wave-uniform offsets)
    const int64_t o0 = mul_u32(id.p0, block_stride) + head_off, o1 = mul_u32(id.p1, block_stride) + head_off;
#pragma unroll
    for (int i = 0; i < PERD; ++i) {
      const int L = i * NT + tid;
      const char* src;
      if (L < 32 * CR) {                          // K: score row r, position pos (wave-uniform)
        const int r = L / CR, pos = L % CR;
        const int dg = pos ^ ksw<CR>(r), rr = r & 15;
        const int tkn = (rr & 3) | ((rr & 4) << 1) | ((rr & 8) >> 1);   // rho(rr)
        src = a.k + ((r >> 4) ? o1 : o0) + (int64_t)(dg * 16 + tkn) * 16;
      } else {                                    // V^T: dim d, position pos
        const int L2 = L - 32 * CR, d = L2 >> 2, pos = L2 & 3;
        const int q = pos ^ ((d >> 2) & 3);
        src = a.v + ((q >> 1) ? o1 : o0) + (int64_t)(2 * d + (q & 1)) * 16;
      }
      const uint32_t dst = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(base) +
                           (uint32_t)__builtin_amdgcn_readfirstlane((i * NT + 64 * wave) * 16);
      lds_dma16(src, dst);
    }
  };

  if constexpr (DMA && WT == 8) {
    // Eight waves wait at a barrier for the slowest of them, so they meet at
    // one every two steps (chunk workload 395-398 us against 403-407; with
    // four waves it measured the same either way): stages 0-1 and 2-3 take
    // turns, and the loads of the next two steps go out right after the
    // barrier that tells every wave is done with the two before.
    if (s_end > s_begin) {
      const Staged none{};
      dma_stage(0, ids_of(s_begin));
      if (s_begin + 1 < s_end) dma_stage(1, ids_of(s_begin + 1));
      Ids n0 = ids_of(s_begin + 2), n1 = ids_of(s_begin + 3);
      int hb = 0;   // first stage of the current two steps (0 or 2)
      for (int s0 = s_begin; s0 < s_end; s0 += 2, hb ^= 2) {
        vm_wait<0>();   // this wave's loads of steps s0 and s0 + 1
        wg_barrier();
        if (s0 + 2 < s_end) dma_stage(hb ^ 2, n0);
        if (s0 + 3 < s_end) dma_stage((hb ^ 2) + 1, n1);
        n0 = ids_of(s0 + 4);
        n1 = ids_of(s0 + 5);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int st = s0 + j;
          if (st < s_end) {
            const int k0 = (jb0 + 2 * st) * kBS;
            if (tile_ok && k0 < w_hi && k0 + 2 * kBS > w_lo) {
              if (k0 + 2 * kBS > n_lo || k0 < lo_hi) step(std::true_type{}, hb + j, k0, none);
              else step(std::false_type{}, hb + j, k0, none);
            }
          }
        }
      }
    }
  } else if constexpr (DMA) {
    // NSTAGE stages: step st's tiles were requested NSTAGE - 1 steps earlier.
    // At the head of step st every wave waits for its own loads of st (those
    // of the steps after it may stay in flight), then the barrier makes all
    // of them visible and tells that every wave is done with step st - 1,
    // whose stage then takes the loads of st + NSTAGE - 1.
    if (s_end > s_begin) {
      const Staged none{};
#pragma unroll
      for (int j = 0; j < NSTAGE - 1; ++j)
        if (s_begin + j < s_end) dma_stage(j, ids_of(s_begin + j));
      Ids idn = ids_of(s_begin + NSTAGE - 1);
      // stage of step st, and the stage that takes the loads of st + NSTAGE - 1
      int buf = 0, lbuf = NSTAGE - 1;
      for (int st = s_begin; st < s_end;
           ++st, buf = (buf + 1 == NSTAGE ? 0 : buf + 1), lbuf = (lbuf + 1 == NSTAGE ? 0 : lbuf + 1)) {
        const int ahead = min(s_end - 1 - st, NSTAGE - 2);   // later steps whose loads are in flight
        if (NSTAGE > 3 && ahead >= 2) vm_wait<(NSTAGE > 3 ? 2 : 1) * PERD>();
        else if (ahead >= 1) vm_wait<PERD>();
        else vm_wait<0>();
        wg_barrier();
        if (st + NSTAGE - 1 < s_end) dma_stage(lbuf, idn);
        idn = ids_of(st + NSTAGE);
        const int k0 = (jb0 + 2 * st) * kBS;
        if (tile_ok && k0 < w_hi && k0 + 2 * kBS > w_lo) {
          if (k0 + 2 * kBS > n_lo || k0 < lo_hi) step(std::true_type{}, buf, k0, none);
          else step(std::false_type{}, buf, k0, none);
        }
      }
    }
  } else if (s_end > s_begin) {
    Staged r;
    Ids id = ids_of(s_begin);
    load_stage(r, id);
    Ids idn = ids_of(s_begin + 1);
    store_stage(r, 0, (jb0 + 2 * s_begin) * kBS);
    Staged cur = r;   // (scales of the step being computed)
    __syncthreads();
    for (int st = s_begin; st < s_end; ++st) {
      const int buf = (st - s_begin) & 1;
      const bool more = st + 1 < s_end;
      if (more) load_stage(r, idn);              // the next step's tiles, in flight meanwhile
      idn = ids_of(st + 2);
      const int k0 = (jb0 + 2 * st) * kBS;
      // this wave's columns see some row of the step
      if (tile_ok && k0 < w_hi && k0 + 2 * kBS > w_lo) {
        if (k0 + 2 * kBS > n_lo || k0 < lo_hi) step(std::true_type{}, buf, k0, cur);
        else step(std::false_type{}, buf, k0, cur);
      }
      if (more) {
        store_stage(r, buf ^ 1, k0 + 2 * kBS);
        cur = r;
      }
      __syncthreads();
    }
  }

  // the column's sum over both halves of the wave, then its outputs
  float lt;
  {
    const uint32_t xb = __float_as_uint(l);
    const auto p32 = __builtin_amdgcn_permlane32_swap(xb, xb, false, false);
    lt = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
  }
  if (!col_ok) return;
  if (npieces > 1 || a.partials_only) {
    // this piece's partial (m, l, acc) of the column, merged by
    // merge_flash_kernel or, for a shared prefix, by the decode's merge (the
    // partial rows cover batch * max_q query rows; a malformed query_start
    // may name more, which are left unwritten)
    if ((int64_t)q_row >= (int64_t)a.batch * a.max_q) return;
    const int64_t rr = ((int64_t)q_row * a.num_heads + h) * a.max_pieces + piece;
#pragma unroll
    for (int od = 0; od < NO; ++od)
#pragma unroll
      for (int gi = 0; gi < 4; ++gi)
        *reinterpret_cast<floatx4*>(a.ws_acc + rr * D + 32 * od + 8 * gi + 4 * half) =
            floatx4{acc[od][4 * gi], acc[od][4 * gi + 1], acc[od][4 * gi + 2], acc[od][4 * gi + 3]};
    if (half == 0) {
      a.ws_m[rr] = m;
      a.ws_l[rr] = lt;
    }
    return;
  }
  const float inv = 1.0f / lt;
#pragma unroll
  for (int od = 0; od < NO; ++od)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int64_t o = ((int64_t)q_row * a.num_heads + h) * D + 32 * od + 8 * gi + 4 * half;
      u32x2 wv;
      if constexpr (KV == KVC_F16) {
        wv[0] = pack_f16x2(acc[od][4 * gi] * inv, acc[od][4 * gi + 1] * inv);
        wv[1] = pack_f16x2(acc[od][4 * gi + 2] * inv, acc[od][4 * gi + 3] * inv);
      } else {
        wv[0] = pack_bf16x2(acc[od][4 * gi] * inv, acc[od][4 * gi + 1] * inv);
        wv[1] = pack_bf16x2(acc[od][4 * gi + 2] * inv, acc[od][4 * gi + 3] * inv);
      }
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + o) = wv;
    }
}

// Merge of the pieces of the several-token kernel's cut tiles: one thread per
// (query token, query head of the group, 4 output dims), merge_tokens(G, D)
// tokens of one sequence and KV head per work-group; columns whose tile was
// not cut were written by the kernel itself.  A piece whose rows the column
// does not see left an empty partial (m = -inf, l = 0), skipped.
__host__ __device__ __forceinline__ int merge_tokens(int G, int D) {
  const int per = G * (D / 4);   // threads per query token (<= 512)
  return 512 / per;
}

template <kvc_dtype QT, int D>
__global__ __launch_bounds__(512) void merge_flash_kernel(DecodeArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  constexpr int COLS = D / 4;
  const int G = a.group;
  const int per = G * COLS;
  const int mt = merge_tokens(G, D);
  if ((int)threadIdx.x >= mt * per) return;   // (threads rounded up to whole waves)
  const int tok = (int)blockIdx.z * mt + (int)threadIdx.x / per;
  const int rem = (int)threadIdx.x % per;
  const int hh = rem / COLS, c = rem % COLS;
  if (tok >= a.max_q) return;
  const int n = attend_len(a.context_lens, b, a.max_ctx, a.max_blocks);
  if (n <= 0) return;
  const int ql = query_len(a, b, n);
  if (tok >= ql) return;
  const int q_row = a.q_start[b] + tok;
  if (q_row < 0 || q_row >= a.total_q || (int64_t)q_row >= (int64_t)a.batch * a.max_q) return;
  const int cols = 32 * a.waves_per_group;   // columns of a work-group
  const FlashTile tile = flash_tile(n, ql, G, a.window, (tok * G + hh) / cols, cols, false);
  const int np = flash_pieces(tile.nsteps, a.split_steps);
  if (np <= 1) return;
  const int h = g * G + hh;
  const int64_t row0 = ((int64_t)q_row * a.num_heads + h) * a.max_pieces;
  float M = kNegInf, L = 0.0f;
  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < np; ++p) {
    const float m = a.ws_m[row0 + p];
    if (m == kNegInf) continue;
    const float l = a.ws_l[row0 + p];
    const floatx4 v = *reinterpret_cast<const floatx4*>(a.ws_acc + (row0 + p) * D + 4 * c);
    const float Mn = fmaxf(M, m);
    const float sa = __builtin_amdgcn_exp2f(M - Mn), sb = __builtin_amdgcn_exp2f(m - Mn);
    acc = acc * sa + v * sb;
    L = L * sa + l * sb;
    M = Mn;
  }
  const float inv = 1.0f / L;
  const int64_t o = ((int64_t)q_row * a.num_heads + h) * D + 4 * c;
#pragma unroll
  for (int e = 0; e < 4; ++e) store_out<QT>(a.out, o + e, acc[e] * inv);
}

// Merge of the MFMA kernel's partials: one work-group per (KV head,
// sequence[, query token]), one thread per (query head of the group, 4 output
// dims).  The triples of chunks c_first .. c_first + np - 1 (slots b + c) are
// folded in a single pass with the online-softmax recurrence, so every load
// can be issued ahead of its use.  EXT: a chunk whose rows a query token does
// not see left an empty triple (m = -inf, l = 0), skipped.
template <kvc_dtype QT, int D, bool EXT>
__global__ __launch_bounds__(512) void merge_segments_kernel(DecodeArgs a) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int tok = EXT ? (int)blockIdx.z : 0;
  const int t = threadIdx.x;
  constexpr int COLS = D / 4;
  const int hh = t / COLS, c = t % COLS;
  // Shared-prefix decode: the prefix pass read sequence 0's first skip_blocks
  // blocks for every sequence, which is its answer only if this sequence's
  // table starts with the same blocks and it holds rows past them; otherwise
  // its outputs are NaN.  (Every thread takes part: before any return.)
  bool bad_prefix = false;
  if (!EXT && a.pre_pieces > 0) {
    bool bad = attend_len(a.context_lens, b, a.max_ctx, a.max_blocks) <= a.skip_blocks * kBS;
    const int32_t* row_b = a.block_table + (int64_t)b * a.max_blocks;
    for (int i = t; i < a.skip_blocks; i += (int)blockDim.x) bad |= row_b[i] != a.block_table[i];
    bad_prefix = __syncthreads_or(bad);
  }
  if (hh >= a.group) return;
  const int n = attend_len(a.context_lens, b, a.max_ctx, a.max_blocks);
  if (n <= 0) return;
  int q_row = b;
  if constexpr (EXT) {
    if (tok >= query_len(a, b, n)) return;
    q_row = a.q_start[b] + tok;
    if (q_row < 0 || q_row >= a.total_q) return;
  }
  // Shared-prefix decode: every sequence goes through here, with the prefix
  // pass's partials and those of its own rows past the prefix (none when the
  // prefix holds them all).
  const bool cascade = !EXT && a.pre_pieces > 0;
  int c_first = 0, np = 0;
  if (!cascade || (n + kBS - 1) / kBS > decode_first_block(a, n)) {
    c_first = a.ws_seginfo[2 * b];
    np = a.ws_seginfo[2 * b + 1];
  }
  if (!cascade && np <= 1) return;             // one chunk held the whole sequence
  if (c_first < 0 || c_first >= a.chunk_slots) np = 0;
  if (np > a.chunk_slots - c_first) np = a.chunk_slots - c_first;
  const int h = g * a.group + hh;
  const int64_t row0 = ((EXT ? (int64_t)tok * a.num_heads : 0) + h) * (a.batch + a.chunk_slots) + b + c_first;
  float M = kNegInf, L = 0.0f;
  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
  if (cascade) {
    // Every prefix piece holds rows, so its max is finite; the first step's
    // weight of the empty start (M = -inf) is a select, not a branch, so the
    // unrolled loads all issue ahead of their use.
    const int64_t pr = ((int64_t)b * a.num_heads + h) * a.pre_max_pieces;
#pragma unroll 8
    for (int p = 0; p < a.pre_pieces; ++p) {
      const float m = a.pre_m[pr + p];
      const float l = a.pre_l[pr + p];
      const floatx4 v = *reinterpret_cast<const floatx4*>(a.pre_acc + (pr + p) * D + 4 * c);
      const float Mn = fmaxf(M, m);
      const float sa = M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
      const float sb = __builtin_amdgcn_exp2f(m - Mn);
      acc = acc * sa + v * sb;
      L = L * sa + l * sb;
      M = Mn;
    }
  }
#pragma unroll 4
  for (int p = 0; p < np; ++p) {
    const float m = a.ws_m[row0 + p];
    const float l = a.ws_l[row0 + p];
    const floatx4 v = *reinterpret_cast<const floatx4*>(a.ws_acc + (row0 + p) * D + 4 * c);
    if constexpr (EXT) {
      if (m == kNegInf) continue;
    }
    const float Mn = fmaxf(M, m);
    const float sa = __builtin_amdgcn_exp2f(M - Mn), sb = __builtin_amdgcn_exp2f(m - Mn);
    acc = acc * sa + v * sb;
    L = L * sa + l * sb;
    M = Mn;
  }
  const float inv = bad_prefix ? __builtin_nanf("") : 1.0f / L;
  const int64_t o = ((int64_t)q_row * a.num_heads + h) * D + 4 * c;
#pragma unroll
  for (int e = 0; e < 4; ++e) store_out<QT>(a.out, o + e, acc[e] * inv);
}

// ---------------------------------------------------------------------------
// Merge of the FMA kernel's per-partition triples: M = max_p m_p; out = sum_p acc_p 2^(m_p - M)
// / sum_p l_p 2^(m_p - M).  One work-group of 256 threads per (head, sequence);
// D/4 threads cover one partition row with 16-byte loads, the rest stride over
// partitions, and the rows are combined through LDS.
// ---------------------------------------------------------------------------
template <kvc_dtype QT, int D>
__global__ __launch_bounds__(256) void merge_parts_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int n = attend_len(a.context_lens, b, a.max_ctx, a.max_blocks);
  const int np = (n + a.part_tokens - 1) / a.part_tokens;
  if (np <= 1) return;
  constexpr int TPR = D / 4;          // threads per partition row
  constexpr int ROWS = 256 / TPR;     // partition rows in flight
  __shared__ float red[256];
  __shared__ floatx4 part_acc[ROWS][TPR];
  __shared__ float part_l[ROWS];
  const int64_t base = ((int64_t)b * a.num_heads + h) * a.num_parts;
  float mx = kNegInf;
  for (int p = tid; p < np; p += 256) mx = fmaxf(mx, a.ws_m[base + p]);
  red[tid] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
    __syncthreads();
  }
  const float M = red[0];
  const int prow = tid / TPR, c = tid % TPR;
  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
  float L = 0.0f;
#pragma unroll 4
  for (int p = prow; p < np; p += ROWS) {
    const float w = __builtin_amdgcn_exp2f(a.ws_m[base + p] - M);
    const floatx4 v = *reinterpret_cast<const floatx4*>(a.ws_acc + (base + p) * D + 4 * c);
    acc += v * w;
    L += w * a.ws_l[base + p];
  }
  part_acc[prow][c] = acc;
  if (c == 0) part_l[prow] = L;
  __syncthreads();
  if (tid < TPR) {
    floatx4 tot = part_acc[0][tid];
    float lt = part_l[0];
#pragma unroll
    for (int rr = 1; rr < ROWS; ++rr) {
      tot += part_acc[rr][tid];
      lt += part_l[rr];
    }
    const float inv = 1.0f / lt;
    const int64_t o = ((int64_t)b * a.num_heads + h) * D + 4 * tid;
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out<QT>(a.out, o + e, tot[e] * inv);
  }
}

// ---------------------------------------------------------------------------
// Plain streaming copy (calibration).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void stream_copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                          int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// Plain streaming read (calibration): every 16-byte chunk of src read once
// with non-temporal loads.  Each wave reads its own contiguous run, eight
// 1 KiB wave loads in flight at a time (the decode's tiles are contiguous
// runs too); each wave writes the xor of its chunks to one word of sink, so
// no load is dead.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink, int64_t sink_words) {
  const int64_t waves = (int64_t)gridDim.x * 4;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // wave w's run: [r0, r1), cut in whole 64-chunk wave loads where possible
  const int64_t per = ((n16 + waves - 1) / waves + 63) / 64 * 64;
  const int64_t r0 = w * per, r1 = r0 + per < n16 ? r0 + per : n16;
  uint32_t acc = 0;
  constexpr int U = 8;
  int64_t i = r0 + lane;
  for (; i + (U - 1) * 64 < r1; i += U * 64) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 64);
    u32x4 x = v[0];
#pragma unroll
    for (int u = 1; u < U; ++u) x ^= v[u];
    acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  for (; i < r1; i += 64) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if (lane == 0) sink[w % sink_words] = acc;
}

template <kvc_dtype KV, kvc_dtype QT, int D>
hipError_t launch_fma(const DecodeArgs& a, int G, dim3 grid, hipStream_t s) {
  if (G <= 1) hipLaunchKernelGGL((decode_fma_kernel<KV, QT, D, 1>), grid, dim3(64), 0, s, a);
  else if (G <= 2) hipLaunchKernelGGL((decode_fma_kernel<KV, QT, D, 2>), grid, dim3(64), 0, s, a);
  else if (G <= 4) hipLaunchKernelGGL((decode_fma_kernel<KV, QT, D, 4>), grid, dim3(64), 0, s, a);
  else if (G <= 8) hipLaunchKernelGGL((decode_fma_kernel<KV, QT, D, 8>), grid, dim3(64), 0, s, a);
  else hipLaunchKernelGGL((decode_fma_kernel<KV, QT, D, 16>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(64) void zero_ints_kernel(int* p, int n) {
  for (int i = threadIdx.x; i < n; i += 64) p[i] = 0;
}

// tile_groups: 0 for decode; else the extend kernel's grid.z, with
// tiles_per_wave column tiles per wave
template <kvc_dtype KV, kvc_dtype QT>
hipError_t launch_decode_typed(const DecodeArgs& a, int D, int kernel, bool merge, int tile_groups,
                               int tiles_per_wave, hipEvent_t ev0, hipEvent_t ev1, hipStream_t s) {
  hipError_t e = hipSuccess;
  const size_t scan_lds = (size_t)(a.batch + 1) * sizeof(int);
  if (kernel == 1) {
    if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return e;
    dim3 grid(a.num_parts, a.num_kv_heads, a.batch);
    e = (D == 64) ? launch_fma<KV, QT, 64>(a, a.group, grid, s) : launch_fma<KV, QT, 128>(a, a.group, grid, s);
    if (e != hipSuccess) return e;
    if (ev1 && (e = hipEventRecord(ev1, s)) != hipSuccess) return e;
    if (merge) {
      dim3 mgrid(a.num_heads, a.batch);
      if (D == 64) hipLaunchKernelGGL((merge_parts_kernel<QT, 64>), mgrid, dim3(256), 0, s, a);
      else hipLaunchKernelGGL((merge_parts_kernel<QT, 128>), mgrid, dim3(256), 0, s, a);
      e = hipGetLastError();
    }
    return e;
  }
  if constexpr (KV != KVC_F32) {
    if (kernel == 3) {   // several tokens, one wave per 32 columns (and piece of their rows)
      if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return e;
      // tile_groups: work-groups of waves_per_group column tiles per sequence
      // and head; eight only for 16-bit caches at head_dim 128 (their stages
      // shared by twice the tiles, at the same two waves per SIMD)
      dim3 grid(a.num_kv_heads, tile_groups * a.max_pieces, a.batch);
      if (a.waves_per_group == 8) {
        if constexpr (is_byte_code(KV)) return hipErrorInvalidValue;
        else if (D == 128) hipLaunchKernelGGL((extend_flash_kernel<KV, 128, 8>), grid, dim3(512), 0, s, a);
        else return hipErrorInvalidValue;
      } else if (a.waves_per_group == 4) {
        if (D == 64) hipLaunchKernelGGL((extend_flash_kernel<KV, 64, 4>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((extend_flash_kernel<KV, 128, 4>), grid, dim3(256), 0, s, a);
      } else {
        return hipErrorInvalidValue;
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if (ev1 && (e = hipEventRecord(ev1, s)) != hipSuccess) return e;
      if (a.max_pieces > 1 && !a.partials_only) {
        const int mt = merge_tokens(a.group, D);
        const int threads = ((mt * a.group * (D / 4) + 63) / 64) * 64;
        dim3 mgrid(a.num_kv_heads, a.batch, (a.max_q + mt - 1) / mt);
        if (D == 64) hipLaunchKernelGGL((merge_flash_kernel<QT, 64>), mgrid, dim3(threads), 0, s, a);
        else hipLaunchKernelGGL((merge_flash_kernel<QT, 128>), mgrid, dim3(threads), 0, s, a);
        e = hipGetLastError();
      }
      return e;
    }
    constexpr int PF = is_byte_code(KV) ? KVC_PREFETCH_FP8 : KVC_PREFETCH_16;  // blocks in flight per wave
    // the continuous ring holds the next segment's query too
    constexpr int KVC_STREAM_PF = is_byte_code(KV) ? KVC_PREFETCH_STREAM8 : KVC_PREFETCH_STREAM16;
    // ticket counters start at zero (a kernel, not a memset, so the sequence
    // can be captured in a graph); without a pool no wave touches them
    if (a.pool_pieces > 0 && tile_groups == 0) {
      hipLaunchKernelGGL(zero_ints_kernel, dim3(1), dim3(64), 0, s, a.ws_ticket, a.num_kv_heads);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return e;
    const int threads = ((a.group * (D / 4) + 63) / 64) * 64;   // <= 16 heads * 32 columns = 512
    if (tile_groups == 0) {
      dim3 grid(a.work_items, a.num_kv_heads);
      // the pooled walk is a variant of its own: its bookkeeping costs scalar
      // registers the static walk needs for its loads
      if (a.pool_pieces > 0) {
        if (D == 64) hipLaunchKernelGGL((decode_stream_kernel<KV, 64, KVC_STREAM_PF, true>), grid, dim3(64), scan_lds, s, a);
        else hipLaunchKernelGGL((decode_stream_kernel<KV, 128, KVC_STREAM_PF, true>), grid, dim3(64), scan_lds, s, a);
      } else {
        // LDS slots for the walk's results before each wave's last, within
        // the share of a CU's 160 KiB that each resident work-group (one wave)
        // may take without lowering the waves resident per CU
        DecodeArgs as = a;
        const int64_t waves = (int64_t)a.work_items * a.num_kv_heads;
        const int64_t per_cu = std::max<int64_t>(4, (waves + 255) / 256);
        const int64_t budget = 163840 / per_cu - (int64_t)scan_lds - 16;
        const int sslot = D == 64 ? stage_slot_bytes<64>() : stage_slot_bytes<128>();
        as.stage_slots = (int32_t)std::max<int64_t>(0, std::min<int64_t>(KVC_STAGE_SLOTS, budget / sslot));
        const size_t lds = scan_lds + (as.stage_slots > 0 ? 16 + (size_t)as.stage_slots * sslot : 0);
        if (D == 64) hipLaunchKernelGGL((decode_stream_kernel<KV, 64, KVC_STREAM_PF, false>), grid, dim3(64), lds, s, as);
        else hipLaunchKernelGGL((decode_stream_kernel<KV, 128, KVC_STREAM_PF, false>), grid, dim3(64), lds, s, as);
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if (ev1 && (e = hipEventRecord(ev1, s)) != hipSuccess) return e;
      dim3 mgrid(a.num_kv_heads, a.batch);
      if (D == 64) hipLaunchKernelGGL((merge_segments_kernel<QT, 64, false>), mgrid, dim3(threads), 0, s, a);
      else hipLaunchKernelGGL((merge_segments_kernel<QT, 128, false>), mgrid, dim3(threads), 0, s, a);
      return hipGetLastError();
    }
    dim3 grid(a.work_items, a.num_kv_heads, tile_groups);
    dim3 block(64 * a.waves_per_group);
    // LDS slots for each wave's results before its last segment, within the
    // share of a CU's 160 KiB that each resident work-group may take (and
    // 64 KiB per work-group)
    DecodeArgs as = a;
    {
      const int tpw = std::max(1, std::min(4, tiles_per_wave));
      const int64_t wpg = std::max(1, a.waves_per_group);
      const int64_t waves = (int64_t)a.work_items * a.num_kv_heads * tile_groups * wpg;
      const int64_t per_cu = std::max<int64_t>(4, (waves + 255) / 256);
      const int64_t group = std::min<int64_t>(65536, 163840 * wpg / per_cu);
      const int64_t per_wave = (group - (int64_t)scan_lds - 16) / wpg - 16;
      const int64_t tslot = (int64_t)(D / 16) * 64 * 16 + 64 * 16;
      as.stage_slots = (int32_t)std::max<int64_t>(0, std::min<int64_t>(KVC_STAGE_SLOTS, per_wave / (tpw * tslot)));
    }
    const size_t lds = scan_lds + 16 +
                       (size_t)std::max(1, a.waves_per_group) *
                           (16 + (size_t)as.stage_slots * std::max(1, std::min(4, tiles_per_wave)) *
                                     ((size_t)(D / 16) * 64 * 16 + 64 * 16));
    // several tiles per wave leave fewer registers for the prefetch ring
    switch (tiles_per_wave) {
      case 1:
        if (D == 64) hipLaunchKernelGGL((extend_mfma_kernel<KV, 64, PF, 1>), grid, block, lds, s, as);
        else hipLaunchKernelGGL((extend_mfma_kernel<KV, 128, PF, 1>), grid, block, lds, s, as);
        break;
      case 2:
        if (D == 64) hipLaunchKernelGGL((extend_mfma_kernel<KV, 64, KVC_PREFETCH_T2, 2>), grid, block, lds, s, as);
        else hipLaunchKernelGGL((extend_mfma_kernel<KV, 128, KVC_PREFETCH_T2, 2>), grid, block, lds, s, as);
        break;
      case 3:
        if (D == 64) hipLaunchKernelGGL((extend_mfma_kernel<KV, 64, KVC_PREFETCH_T3, 3>), grid, block, lds, s, as);
        else hipLaunchKernelGGL((extend_mfma_kernel<KV, 128, KVC_PREFETCH_T3, 3>), grid, block, lds, s, as);
        break;
      default:
        if (D == 64) hipLaunchKernelGGL((extend_mfma_kernel<KV, 64, KVC_PREFETCH_T4, 4>), grid, block, lds, s, as);
        else hipLaunchKernelGGL((extend_mfma_kernel<KV, 128, KVC_PREFETCH_T4, 4>), grid, block, lds, s, as);
        break;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev1 && (e = hipEventRecord(ev1, s)) != hipSuccess) return e;
    dim3 mgrid(a.num_kv_heads, a.batch, a.max_q);
    if (D == 64) hipLaunchKernelGGL((merge_segments_kernel<QT, 64, true>), mgrid, dim3(threads), 0, s, a);
    else hipLaunchKernelGGL((merge_segments_kernel<QT, 128, true>), mgrid, dim3(threads), 0, s, a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

}  // namespace

// The decode workspace of the allocation-free entry point: one array per
// device, part of the library's code object (loaded with it, held until the
// process ends).  Host code never passes `scratch` itself to a kernel -- on
// the host the name stands for a host-side shadow -- but the device address
// hipGetSymbolAddress returns for the current device, resolved once per
// device below.
static __device__ __align__(256) char scratch[KVC_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_copy_blocks(const PoolDesc& pool, const CowPair* pairs_dev, int32_t num_pairs, hipStream_t stream) {
  if (num_pairs <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, pool.num_layers), dim3(256), 0, stream, pool, pairs_dev);
  return hipGetLastError();
}

template <kvc_dtype KV, typename SEGS>
hipError_t launch_append_quant(const PoolDesc& pool, const SEGS& segs, int32_t num_segments, const void* k_new,
                               const void* v_new, kvc_dtype in_dtype, int64_t total_rows, hipStream_t stream) {
  const dim3 g8(num_segments, pool.num_kv_heads, 2 * pool.num_layers);
  if (in_dtype == KVC_F32)
    hipLaunchKernelGGL((append_quant_kernel<KV, KVC_F32, SEGS>), g8, dim3(64), 0, stream, pool, segs, k_new, v_new,
                       total_rows);
  else if (in_dtype == KVC_F16)
    hipLaunchKernelGGL((append_quant_kernel<KV, KVC_F16, SEGS>), g8, dim3(64), 0, stream, pool, segs, k_new, v_new,
                       total_rows);
  else
    hipLaunchKernelGGL((append_quant_kernel<KV, KVC_BF16, SEGS>), g8, dim3(64), 0, stream, pool, segs, k_new, v_new,
                       total_rows);
  return hipGetLastError();
}

template <typename SEGS>
hipError_t launch_append_from(const PoolDesc& pool, const SEGS& segs, int32_t num_segments, const void* k_new,
                              const void* v_new, kvc_dtype in_dtype, int64_t total_rows, hipStream_t stream) {
  const char* kn = static_cast<const char*>(k_new);
  const char* vn = static_cast<const char*>(v_new);
  const dim3 grid(num_segments, pool.num_kv_heads, pool.num_layers);
  switch (pool.dtype) {
    case KVC_F32:
      hipLaunchKernelGGL((append_copy_kernel<4, SEGS>), grid, dim3(64), 0, stream, pool, segs, kn, vn, total_rows);
      break;
    case KVC_F16:
    case KVC_BF16:
      hipLaunchKernelGGL((append_copy_kernel<2, SEGS>), grid, dim3(64), 0, stream, pool, segs, kn, vn, total_rows);
      break;
    case KVC_FP8_E4M3:
      return launch_append_quant<KVC_FP8_E4M3>(pool, segs, num_segments, k_new, v_new, in_dtype, total_rows, stream);
    case KVC_INT8:
      return launch_append_quant<KVC_INT8>(pool, segs, num_segments, k_new, v_new, in_dtype, total_rows, stream);
  }
  return hipGetLastError();
}

// The newest row of each of `batch` sequences of one layer, read from the
// block table: the append of a decode step whose bookkeeping is already done.
hipError_t launch_append_newest(const PoolDesc& pool, int32_t layer, const int32_t* block_table, int32_t max_blocks,
                                const int32_t* context_lens, int32_t batch, const void* k_new, const void* v_new,
                                kvc_dtype in_dtype, hipStream_t stream) {
  PoolDesc one = pool;
  const int64_t layer_bytes = (int64_t)pool.num_blocks * pool.num_kv_heads * tile_bytes(pool);
  one.k = pool.k + layer * layer_bytes;
  one.v = pool.v + layer * layer_bytes;
  if (pool.k_scale) {
    one.k_scale = pool.k_scale + (int64_t)layer * pool.num_blocks * pool.num_kv_heads;
    one.v_scale = pool.v_scale + (int64_t)layer * pool.num_blocks * pool.num_kv_heads;
  }
  one.num_layers = 1;
  const SegFromTable segs{block_table, context_lens, max_blocks, pool.num_blocks};
  return launch_append_from(one, segs, batch, k_new, v_new, in_dtype, batch, stream);
}

hipError_t launch_append(const PoolDesc& pool, const AppendSegment* segs_dev, const InlineSegments* segs_inline,
                         int32_t num_segments, const void* k_new, const void* v_new, kvc_dtype in_dtype,
                         int64_t total_rows, hipStream_t stream) {
  if (num_segments <= 0) return hipSuccess;
  if (segs_inline) {
    if (num_segments > kInlineSegments) return hipErrorInvalidValue;
    SegFromArgs segs;
    segs.v = *segs_inline;
    return launch_append_from(pool, segs, num_segments, k_new, v_new, in_dtype, total_rows, stream);
  }
  return launch_append_from(pool, SegFromDevice{segs_dev}, num_segments, k_new, v_new, in_dtype, total_rows, stream);
}

// Shared-prefix decode: the prefix pass (the several-token kernel without
// the causal mask over sequence 0's first rows, partials only), then the
// decode over every sequence's rows past the prefix, whose merge folds in the
// prefix's partials.  Timing events (ev0, ev1) span both passes.  (Run on a
// second stream beside the decode, the prefix pass costs more than it hides:
// the decode's waves slow down where it lands, and the fork and join add
// their own gaps.)
template <kvc_dtype KV, kvc_dtype QT>
hipError_t launch_cascade_typed(const DecodeArgs& a, const DecodePlan& plan, int D, hipEvent_t ev0, hipEvent_t ev1,
                                hipStream_t s) {
  hipError_t e;
  const int prefix = plan.skip_blocks * kBS;
  DecodeArgs ap = a;
  ap.batch = 1;
  ap.q_start = nullptr;        // (not read without the causal mask)
  ap.total_q = a.batch;
  ap.max_q = a.batch;
  ap.context_lens = nullptr;
  ap.max_ctx = prefix;
  ap.noncausal = 1;
  ap.partials_only = 1;
  ap.ws_acc = const_cast<float*>(a.pre_acc);
  ap.ws_m = const_cast<float*>(a.pre_m);
  ap.ws_l = const_cast<float*>(a.pre_l);
  ap.max_pieces = plan.pre_pieces;
  ap.split_steps = plan.pre_split_steps;
  ap.waves_per_group = 4;
  ap.window = 0;
  ap.skip_blocks = 0;
  ap.pre_pieces = 0;
  if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return e;
  if ((e = launch_decode_typed<KV, QT>(ap, D, 3, false, plan.pre_groups, 1, nullptr, nullptr, s)) != hipSuccess)
    return e;
  return launch_decode_typed<KV, QT>(a, D, 2, true, 0, 1, nullptr, ev1, s);
}

hipError_t launch_decode(const PoolDesc& pool, int32_t layer, const DecodePlan& plan, const void* q, kvc_dtype q_dtype,
                         const int32_t* q_start, int32_t total_q, const int32_t* block_table, int32_t max_blocks,
                         const int32_t* context_lens, int32_t max_context_len, int32_t batch, int32_t num_heads,
                         float scale, void* out, void* workspace, const void* k_new, const void* v_new,
                         hipEvent_t ev_start, hipEvent_t ev_end, hipStream_t stream) {
  DecodeArgs a;
  // The step's newest rows: written by the static matrix-core walk itself
  // (16-bit caches), else by an append kernel launched first.
  a.k_new = a.v_new = nullptr;
  if (k_new) {
    if (decode_folds_append(plan, pool.dtype)) {
      a.k_new = static_cast<const char*>(k_new);
      a.v_new = static_cast<const char*>(v_new);
    } else {
      hipError_t e = launch_append_newest(pool, layer, block_table, max_blocks, context_lens, batch, k_new, v_new,
                                          q_dtype, stream);
      if (e != hipSuccess) return e;
    }
  }
  const int64_t tb = tile_bytes(pool);
  const int64_t layer_bytes = (int64_t)pool.num_blocks * pool.num_kv_heads * tb;
  a.q = q;
  a.out = out;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.k = pool.k + layer * layer_bytes;
  a.v = pool.v + layer * layer_bytes;
  a.k_scale = pool.k_scale ? pool.k_scale + (int64_t)layer * pool.num_blocks * pool.num_kv_heads : nullptr;
  a.v_scale = pool.v_scale ? pool.v_scale + (int64_t)layer * pool.num_blocks * pool.num_kv_heads : nullptr;
  a.tile_bytes = tb;
  a.num_blocks = pool.num_blocks;
  a.max_blocks = max_blocks;
  a.max_ctx = max_context_len;
  a.num_heads = num_heads;
  a.num_kv_heads = pool.num_kv_heads;
  a.group = num_heads / pool.num_kv_heads;
  a.part_tokens = plan.partition_tokens;
  a.num_parts = plan.num_partitions;
  a.batch = batch;
  a.work_items = plan.work_items;
  a.pool_pieces = plan.pool_pieces;
  a.pool_shift = plan.pool_shift;
  a.chunk_slots = (int32_t)plan.chunk_slots();
  a.qk_scale = scale * kLog2e;
  a.q_start = q_start;
  a.max_q = plan.tile_groups ? plan.max_q : 1;
  a.total_q = plan.tile_groups ? total_q : batch;
  a.waves_per_group = plan.tile_groups ? plan.waves_per_group : 1;
  a.window = plan.window;
  a.split_steps = plan.split_steps;
  a.max_pieces = plan.max_pieces;
  a.skip_blocks = plan.skip_blocks;
  a.partials_only = plan.skip_blocks > 0;
  a.noncausal = 0;
  a.pre_pieces = plan.skip_blocks > 0 ? plan.pre_pieces : 0;
  a.pre_max_pieces = plan.pre_pieces;
  a.pre_acc = a.pre_m = a.pre_l = nullptr;
  const bool merge = plan.kernel == 2 || plan.num_partitions > 1;
  const WorkspaceLayout wl = workspace_layout(plan, batch, num_heads, pool.num_kv_heads, pool.head_dim);
  char* w = static_cast<char*>(workspace);
  a.ws_acc = wl.bytes ? reinterpret_cast<float*>(w + wl.acc) : nullptr;
  a.ws_m = wl.bytes ? reinterpret_cast<float*>(w + wl.m) : nullptr;
  a.ws_l = wl.bytes ? reinterpret_cast<float*>(w + wl.l) : nullptr;
  a.ws_seginfo = (wl.bytes && plan.kernel == 2) ? reinterpret_cast<int*>(w + wl.seginfo) : nullptr;
  a.ws_ticket = (wl.bytes && plan.kernel == 2) ? reinterpret_cast<int*>(w + wl.tickets) : nullptr;
  const int D = pool.head_dim;
  if (plan.kernel == 2 && plan.skip_blocks > 0) {
    a.pre_acc = reinterpret_cast<const float*>(w + wl.pre_acc);
    a.pre_m = reinterpret_cast<const float*>(w + wl.pre_m);
    a.pre_l = reinterpret_cast<const float*>(w + wl.pre_l);
    switch (pool.dtype) {
      case KVC_F16:
        return launch_cascade_typed<KVC_F16, KVC_F16>(a, plan, D, ev_start, ev_end, stream);
      case KVC_BF16:
        return launch_cascade_typed<KVC_BF16, KVC_BF16>(a, plan, D, ev_start, ev_end, stream);
      case KVC_FP8_E4M3:
        return launch_cascade_typed<KVC_FP8_E4M3, KVC_BF16>(a, plan, D, ev_start, ev_end, stream);
      case KVC_INT8:
        return launch_cascade_typed<KVC_INT8, KVC_BF16>(a, plan, D, ev_start, ev_end, stream);
      default:
        return hipErrorInvalidValue;
    }
  }
  switch (pool.dtype) {
    case KVC_F32:
      return launch_decode_typed<KVC_F32, KVC_F32>(a, D, plan.kernel, merge, plan.tile_groups, plan.tiles_per_wave,
                                                   ev_start, ev_end, stream);
    case KVC_F16:
      return launch_decode_typed<KVC_F16, KVC_F16>(a, D, plan.kernel, merge, plan.tile_groups, plan.tiles_per_wave,
                                                   ev_start, ev_end, stream);
    case KVC_BF16:
      return launch_decode_typed<KVC_BF16, KVC_BF16>(a, D, plan.kernel, merge, plan.tile_groups, plan.tiles_per_wave,
                                                     ev_start, ev_end, stream);
    case KVC_FP8_E4M3:
      return launch_decode_typed<KVC_FP8_E4M3, KVC_BF16>(a, D, plan.kernel, merge, plan.tile_groups, plan.tiles_per_wave,
                                                         ev_start, ev_end, stream);
    case KVC_INT8:
      return launch_decode_typed<KVC_INT8, KVC_BF16>(a, D, plan.kernel, merge, plan.tile_groups, plan.tiles_per_wave,
                                                     ev_start, ev_end, stream);
  }
  (void)q_dtype;
  return hipErrorInvalidValue;
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t blocks = (n16 + 8 * 256 - 1) / (8 * 256);
  if (blocks > 256 * 8) blocks = 256 * 8;   // 8 work-groups of 4 waves per CU: one resident round
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<const u32x4*>(src),
                     n16, sink, (int64_t)sink_words);
  return hipGetLastError();
}

hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<u32x4*>(dst),
                     static_cast<const u32x4*>(src), n16);
  return hipGetLastError();
}

}  // namespace kvc
