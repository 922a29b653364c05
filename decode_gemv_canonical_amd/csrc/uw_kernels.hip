// Device kernels for gfx950 (CDNA4): on-chip exponent-Huffman decode fused
// into the decode-time product, the decompress-to-HBM alternative, the
// uncompressed bf16 products and a streaming-read probe.
//
// Method: "Unweight: how we compressed an LLM 22% without sacrificing
// quality".  The reconstructive-matmul paragraph loads compressed data,
// rebuilds bf16 weights on chip and multiplies them without writing them back
// to main memory; here the rebuild happens in registers of a wave64 and feeds
// v_dot2_f32_bf16 (batch <= 8 is a matrix-vector shape, not a dense
// contraction, so it stays on the vector ALU).  The full-decode pipeline of
// the four-pipelines paragraph is uw_decompress followed by the bf16 product.
//
// Decode scheme (one wave per block, lane l owns one code stream):
//  * the block's stream words are staged into a per-wave LDS buffer with
//    coalesced 16-byte loads; each lane's start bit is the wave's exclusive
//    prefix sum of the 64 lane bit counts;
//  * a lane keeps a 64-bit window (w0, w1) of its stream in registers and a
//    bit offset qm of (next code - 2) inside it; a peek is one v_alignbit_b32
//    and the table byte address is (peek & mask): the "-2" lands the index on
//    a 4-byte table stride for free;
//  * with code lengths <= 6 any 12-bit window starting at a code holds two
//    whole codes, so one lookup in a 4096-entry pair table returns both
//    exponents: entry = (len_a + len_b) | E_a << 7 | len_a << 16 | E_b << 23.
//    One v_bfi_b32 with the replicated sign+mantissa bytes gives two bf16
//    weights in one register, ready for v_dot2_f32_bf16.  The length sits in
//    bits 0..3 and bits 4..6 are zero, so qm += entry keeps the low 7 bits of
//    qm exact; the refill (qm &= 31) drops the exponent bits it picked up;
//  * longer codes (L > 6) use a 2^L single-code table with the same window;
//  * a raw group (exponent outside the palette) is a wave-uniform branch on a
//    bit of the block's raw bitmap, held in scalar registers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <set>
#include <string>

#include "uw_internal.h"

namespace uw {
namespace {

constexpr int kWave = 64;
constexpr int kPadWords = 4;        // words in front of each staged stream
constexpr int kTableWords = 4096;   // pair table (or 2^L single table)
constexpr int kT1Words = 64;        // single-code table for L <= 6, used to build the pair table
constexpr int kLdsLimit = 160 * 1024;
constexpr int kTransposeWords = 512;  // 16 groups x 64 lanes x bf16
constexpr int kRing = 3;              // sm tiles (1 KB each) in flight per wave
constexpr int kRingWords = kRing * 256;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ inline float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ inline uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN of the same sign.
__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = f32_bits(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return uint16_t((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Sum over the 64 lanes; every lane gets the result.  DPP inside rows of 16,
// then the four row sums are read out of lanes 0, 16, 32, 48.
__device__ inline float wave_sum(float v) {
  v += bits_f32(__builtin_amdgcn_update_dpp(0, int(f32_bits(v)), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v += bits_f32(__builtin_amdgcn_update_dpp(0, int(f32_bits(v)), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v += bits_f32(__builtin_amdgcn_update_dpp(0, int(f32_bits(v)), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += bits_f32(__builtin_amdgcn_update_dpp(0, int(f32_bits(v)), 0x140, 0xF, 0xF, false));  // row_mirror
  float a = bits_f32(__builtin_amdgcn_readlane(int(f32_bits(v)), 0));
  float b = bits_f32(__builtin_amdgcn_readlane(int(f32_bits(v)), 16));
  float c = bits_f32(__builtin_amdgcn_readlane(int(f32_bits(v)), 32));
  float d = bits_f32(__builtin_amdgcn_readlane(int(f32_bits(v)), 48));
  return (a + b) + (c + d);
}

// Exclusive prefix sum over the wave, in lane order.
__device__ inline uint32_t wave_exclusive_scan(uint32_t v, int lane) {
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    uint32_t y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  return x - v;
}

__device__ inline void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Decode tables in LDS.  T1[i] for an L-bit index i (next stream bits, first
// bit in bit 0) = len | E << 7 of the code that prefixes i.  For L <= 6 the
// pair table T2 is built from T1; for L > 6 T1 (2^L entries) is the table.
__device__ inline uint32_t single_entry(const DevMatrix& d, uint32_t idx) {
  uint32_t fallback = 1u | (uint32_t(d.sym[0] >> 24) << 7);
  for (int s = 0; s < d.n_sym; ++s) {
    const uint32_t sym = d.sym[s];
    const uint32_t len = (sym >> 16) & 0xFF;
    if (len && (idx & ((1u << len) - 1u)) == (sym & 0xFFFF)) return len | ((sym >> 24) << 7);
  }
  return fallback;  // only an incomplete (one-symbol) code leaves gaps; never met in a valid stream
}

template <bool PAIR>
__device__ void build_tables(const DevMatrix& d, uint32_t* T, uint32_t* T1) {
  const int tid = threadIdx.x, nt = blockDim.x;
  if (PAIR) {
    for (int i = tid; i < (1 << d.L); i += nt) T1[i] = single_entry(d, uint32_t(i));
    __syncthreads();
    const uint32_t m = (1u << d.L) - 1u;
    for (int i = tid; i < kTableWords; i += nt) {
      const uint32_t a = T1[uint32_t(i) & m];
      const uint32_t la = a & 0xF;
      const uint32_t b = T1[(uint32_t(i) >> la) & m];
      const uint32_t lb = b & 0xF;
      T[i] = (la + lb) | (a & 0x7F80u) | (la << 16) | ((b & 0x7F80u) << 16);
    }
  } else {
    for (int i = tid; i < (1 << d.L); i += nt) T[i] = single_entry(d, uint32_t(i));
  }
}

// ---------------------------------------------------------------------------
// LDS is addressed with absolute byte addresses: the kernels that decode use
// only dynamic LDS, which starts at address 0.  Layout (bytes):
//   [0, 16384)        decode table (pair table, or the 2^L single table)
//   [16384, 16640)    single table for L <= 6 (used to build the pair table)
//   [16640, ...)      kernel-specific area (x for products), then one stage
//                     buffer per wave: 16 pad bytes, the block's stream, 16 pad
//                     bytes, the block's raw exponent bytes.
constexpr uint32_t kT1Addr = kTableWords * 4;
constexpr uint32_t kAreaAddr = (kTableWords + kT1Words) * 4;

typedef __attribute__((address_space(3))) uint32_t lds_word;
typedef __attribute__((address_space(3))) uint8_t lds_byte;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_quad;
typedef __attribute__((address_space(3))) uint16_t lds_half;

__device__ inline uint32_t ld32(uint32_t addr) { return *reinterpret_cast<const lds_word*>(size_t(addr)); }
__device__ inline void st32(uint32_t addr, uint32_t v) { *reinterpret_cast<lds_word*>(size_t(addr)) = v; }
__device__ inline uint32_t ld8(uint32_t addr) { return *reinterpret_cast<const lds_byte*>(size_t(addr)); }
__device__ inline uint4 ld128(uint32_t addr) {
  const u32x4 v = *reinterpret_cast<const lds_quad*>(size_t(addr));
  return uint4{v.x, v.y, v.z, v.w};
}
__device__ inline void st128(uint32_t addr, uint4 v) {
  *reinterpret_cast<lds_quad*>(size_t(addr)) = u32x4{v.x, v.y, v.z, v.w};
}
__device__ inline void st16(uint32_t addr, uint32_t v) { *reinterpret_cast<lds_half*>(size_t(addr)) = uint16_t(v); }

// Per-lane cursor over the staged stream: a 64-bit window (w0, w1) plus the
// next stream word w2 (loaded one refill ahead, so a refill never waits on
// LDS), the LDS byte address of w0 and the bit offset qm of (next code - 2)
// inside the window.  Between refills qm may carry exponent bits above bit 6
// (see the pair-table layout); its low 7 bits are exact.
struct Cursor {
  uint32_t w0, w1, w2, addr, qm;
};

__device__ inline void cursor_reload(Cursor& c) {
  c.w0 = ld32(c.addr);
  c.w1 = ld32(c.addr + 4);
  c.w2 = ld32(c.addr + 8);
}

// At most 32 bits were consumed since the last refill (qm < 64): slide the
// window by one word if qm passed 32, and fetch the word after the window.
__device__ inline void cursor_refill(Cursor& c) {
  const uint32_t adv = c.qm & 32u;
  c.addr += adv >> 3;
  c.w0 = adv ? c.w1 : c.w0;
  c.w1 = adv ? c.w2 : c.w1;
  c.qm &= 31u;
  c.w2 = ld32(c.addr + 8);
}

__device__ inline uint32_t cursor_peek(const Cursor& c) { return __builtin_amdgcn_alignbit(c.w1, c.w0, c.qm); }

typedef __attribute__((address_space(1))) void global_void;
typedef __attribute__((address_space(3))) void lds_void;

// Copy n_quads 16-byte words from global memory to LDS with direct
// global->LDS loads (no registers): lane l of each 64-quad chunk writes
// dst + 16 * (chunk + l).  Completion is waited for with vmcnt.
__device__ inline void copy_to_lds_async(const uint4* src, uint32_t dst, uint32_t n_quads, int lane) {
  for (uint32_t c = 0; c < n_quads; c += kWave) {
    if (c + lane < n_quads)
      __builtin_amdgcn_global_load_lds(
          (global_void*)(const_cast<uint4*>(src + c + lane)),
          reinterpret_cast<lds_void*>(size_t(dst + 16 * c)), 16, 0, 0);
  }
}

// Issue the loads of block `blk`: its stream words and raw exponent bytes go
// into this wave's stage buffer; the lane bit count and the raw bitmap word
// of this lane come back in registers.
struct BlockHead {
  uint32_t lane_bits;
  uint32_t raw_word;  // lane w holds raw-bitmap word w of the block
};

// Block-table words read by the whole wave go through the constant address
// space so they become scalar loads (their own counter, no wait on the
// vector loads in flight).
typedef __attribute__((address_space(4))) const uint32_t const_word;
__device__ inline uint32_t scalar_word(const uint32_t* p, int64_t i) {
  return ((const const_word*)(p))[i];
}

__device__ inline BlockHead issue_head_loads(const DevMatrix& d, int blk, int lane) {
  BlockHead h;
  h.lane_bits = d.lane_bits[int64_t(blk) * kWave + lane];
  h.raw_word = lane < d.rb_words ? d.raw_bits[int64_t(blk) * d.rb_words + lane] : 0u;
  return h;
}

__device__ inline void issue_stage_loads(const DevMatrix& d, int blk, uint32_t stage, int lane) {
  const uint32_t w_begin = scalar_word(d.start_word, blk);
  const uint32_t n_quads = (scalar_word(d.start_word, blk + 1) - w_begin) / 4;
  const uint32_t r0 = scalar_word(d.first_raw, blk), r1 = scalar_word(d.first_raw, blk + 1);
  copy_to_lds_async(reinterpret_cast<const uint4*>(d.stream + w_begin), stage + 16, n_quads, lane);
  copy_to_lds_async(reinterpret_cast<const uint4*>(d.raw + int64_t(r0) * 64), stage + d.stage_raw_word * 4,
                    (r1 - r0) * 4, lane);
}

// After the block's loads: wait for them, then place the lane's cursor at the
// exclusive prefix sum of the lane bit counts.
__device__ inline void start_cursor(const BlockHead& h, uint32_t stage, int lane, Cursor& c) {
  __builtin_amdgcn_s_waitcnt(0);  // every load of the block, direct-to-LDS ones included
  const uint32_t start = wave_exclusive_scan(h.lane_bits, lane);
  wave_lds_fence();
  const uint32_t bit = 4 * 32 + start - 2;
  c.addr = stage + (bit >> 5) * 4;
  c.qm = bit & 31;
  cursor_reload(c);
}

// Replicated sign+mantissa bytes of groups (2k, 2k+1) of a 16-group tile.
__device__ inline uint32_t sm_pair(const uint4& v, int k) {
  const uint32_t w = (k >> 1) == 0 ? v.x : (k >> 1) == 1 ? v.y : (k >> 1) == 2 ? v.z : v.w;
  return __builtin_amdgcn_perm(0u, w, (k & 1) ? 0x03030202u : 0x01010000u);
}

__device__ inline uint32_t sm_byte(const uint4& v, int j) {
  const uint32_t w = (j >> 2) == 0 ? v.x : (j >> 2) == 1 ? v.y : (j >> 2) == 2 ? v.z : v.w;
  return (w >> (8 * (j & 3))) & 0xFF;
}

// Two bf16 weights in one register: sign+mantissa bits from S, exponents from E.
__device__ inline uint32_t merge_pair(uint32_t S, uint32_t E) { return (S & 0x807F807Fu) | (E & 0x7F807F80u); }

__device__ inline uint32_t merge_one(uint32_t sm, uint32_t E) {
  return ((sm & 0x80u) << 8) | (E & 0x7F80u) | (sm & 0x7Fu);
}

// sm tile t of a block (1 KB: 16 groups x 64 lanes) into ring slot `slot`.
__device__ inline void load_sm_tile_to_lds(const uint4* sm_blk, int t, uint32_t ring, int slot, int lane) {
  __builtin_amdgcn_global_load_lds((global_void*)(const_cast<uint4*>(sm_blk + t * 64 + lane)),
                                   (lds_void*)(size_t(ring + slot * 1024)), 16, 0, 0);
}

// Wait until at most kRing-1 vector-memory operations are in flight.  The
// decode loop issues no other vector-memory operation, so this means the
// oldest ring load has landed in LDS.
__device__ inline void wait_vmcnt_ring() {
  static_assert(kRing - 1 < 16, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kRing - 1) : "memory");
}

// Raw flags of the 16 groups of the tile starting at group j0 (wave-uniform).
__device__ inline uint32_t raw_mask16(uint32_t raw_word, int j0) {
  const uint32_t w = __builtin_amdgcn_readlane(raw_word, j0 >> 5);
  return (w >> (j0 & 31)) & 0xFFFFu;
}

// One code from the table: returns the entry (exponent in bits 7..14) and
// advances the cursor (qm) and the running peek p by the code's length.
template <bool PAIR>
__device__ inline uint32_t take_single(Cursor& c, uint32_t& p, uint32_t mask) {
  const uint32_t e = ld32(p & mask);
  if (PAIR) {
    const uint32_t n = (e >> 16) & 0xFu;
    p >>= n;
    c.qm += n;
  } else {
    p >>= (e & 31u);  // length in bits 0..3, bit 4 clear
    c.qm += e;        // exponent bits land above bit 6
  }
  return e;
}

// Decode a complete 16-group tile that lies inside one row and starts at an
// even column group: sink.pair(k, D) receives D = the lane's weights of
// groups (2k, 2k+1).  rmask holds the tile's raw flags, raw_rank the index
// (within the block) of its first raw group.
template <bool PAIR, class Sink>
__device__ __forceinline__ void decode_tile_pairs(Cursor& c, const uint4& cur, uint32_t rmask, uint32_t raw_area,
                                                  uint32_t raw_rank, uint32_t pmask, int lane, Sink& sink) {
  uint32_t p = cursor_peek(c);
  if (PAIR && rmask == 0) {
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
      const uint32_t e1 = ld32(p & 0x3FFCu);
      p >>= (e1 & 31u);
      const uint32_t e2 = ld32(p & 0x3FFCu);
      c.qm += e1 + e2;
      cursor_refill(c);
      p = cursor_peek(c);
      sink.pair(k, merge_pair(sm_pair(cur, k), e1));
      sink.pair(k + 1, merge_pair(sm_pair(cur, k + 1), e2));
    }
  } else {
    uint32_t rank = raw_rank;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t two = (rmask >> (2 * k)) & 3u;
      uint32_t E;
      if (PAIR && two == 0) {
        E = ld32(p & 0x3FFCu);
        p >>= (E & 31u);
        c.qm += E;
      } else {
        uint32_t ea, eb;
        if (two & 1u) ea = ld8(raw_area + (rank++) * 64 + lane) << 7;
        else ea = take_single<PAIR>(c, p, pmask) & 0x7F80u;
        if (two & 2u) eb = ld8(raw_area + (rank++) * 64 + lane) << 23;
        else eb = (take_single<PAIR>(c, p, pmask) & 0x7F80u) << 16;
        E = ea | eb;
      }
      if (!PAIR || (k & 1)) {
        cursor_refill(c);
        p = cursor_peek(c);
      }
      sink.pair(k, merge_pair(sm_pair(cur, k), E));
    }
  }
}

// Decode one block and hand the weights to `sink`:
//   sink.tile_begin(row0, c0)   before a tile that lies inside one row, starts
//                               at an even column group and is complete;
//   sink.pair(k, D)             D = weights of groups (2k, 2k+1) of that tile;
//   sink.single(jj, row, cg, w) one weight of group jj of any other tile;
//   sink.tile_end(t, nt)        after every tile.
// sm tiles stream through a kRing-slot LDS ring filled by direct-to-LDS
// loads, so kRing KB per wave are in flight and the waits are explicit.
template <bool PAIR, class Sink>
__device__ __forceinline__ void decode_block(const DevMatrix& d, int blk, uint32_t stage, uint32_t ring, int lane,
                                             Sink& sink) {
  // per-lane table words, the first sm tiles, then the stream and raw bytes;
  // one wait covers them all
  const int64_t g_first = int64_t(blk) * d.G;
  const int gb = int(std::min<int64_t>(d.G, d.n_groups - g_first));
  const int ntiles = (gb + 15) / 16;
  const BlockHead head = issue_head_loads(d, blk, lane);
  const uint4* sm_blk = reinterpret_cast<const uint4*>(d.sm + int64_t(blk) * d.G * 64);
#pragma unroll
  for (int i = 0; i < kRing; ++i) load_sm_tile_to_lds(sm_blk, std::min(i, ntiles - 1), ring, i, lane);
  issue_stage_loads(d, blk, stage, lane);
  Cursor c;
  start_cursor(head, stage, lane, c);
  const uint32_t raw_area = stage + d.stage_raw_word * 4;
  const uint32_t pmask = PAIR ? 0x3FFCu : (((1u << d.L) - 1u) << 2);
  int64_t row0 = g_first / d.gpr;
  int c0 = int(g_first - row0 * d.gpr);
  uint32_t raw_rank = 0;
  for (int t = 0; t < ntiles; ++t) {
    {
      {
        // exactly kRing-1 ring loads were issued after tile t's
        wait_vmcnt_ring();
        const int slot = t % kRing;
        const uint4 cur = ld128(ring + slot * 1024 + lane * 16);
        const int j0 = t * 16;
        const int nt = std::min(16, gb - j0);
        const uint32_t rmask = raw_mask16(head.raw_word, j0);
        if (nt == 16 && c0 + 16 <= d.gpr && (c0 & 1) == 0) {
          sink.tile_begin(row0, c0);
          decode_tile_pairs<PAIR>(c, cur, rmask, raw_area, raw_rank, pmask, lane, sink);
        } else {
          // tile crossing a row end, starting at an odd column group, or partial
          int64_t row = row0;
          int cg = c0;
          uint32_t rank = raw_rank;
          for (int jj = 0; jj < nt; ++jj, ++cg) {
            if (cg >= d.gpr) {
              cg -= d.gpr;
              ++row;
            }
            uint32_t E;
            if ((rmask >> jj) & 1u) {
              E = ld8(raw_area + (rank++) * 64 + lane) << 7;
            } else {
              uint32_t p = cursor_peek(c);
              E = take_single<PAIR>(c, p, pmask);
              cursor_refill(c);
            }
            sink.single(jj, row, cg, merge_one(sm_byte(cur, jj), E));
          }
        }
        raw_rank += __builtin_popcount(rmask);
        sink.tile_end(t, nt);
        // refill the consumed slot with tile t+kRing; one load per tile
        // (index clamped near the end) keeps the count of loads in flight fixed
        load_sm_tile_to_lds(sm_blk, std::min(t + kRing, ntiles - 1), ring, slot, lane);
        c0 += 16;
        while (c0 >= d.gpr) {
          c0 -= d.gpr;
          ++row0;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decompress: weights pass through a per-wave LDS tile [16][64] bf16 so that
// each lane stores 2 x 16 bytes of consecutive columns.
struct DecompressSink {
  const DevMatrix& d;
  uint16_t* out;
  int64_t ld_out;
  uint32_t tile;    // LDS byte address of the transpose tile
  int lane;
  int64_t trow;     // (row, col) of the current tile's first weight
  int64_t tcol;
  __device__ void tile_begin(int64_t, int) {}
  __device__ void pair(int k, uint32_t D) {
    st16(tile + ((2 * k) * kWave + lane) * 2, D);
    st16(tile + ((2 * k + 1) * kWave + lane) * 2, D >> 16);
  }
  __device__ void single(int jj, int64_t, int, uint32_t w) { st16(tile + (jj * kWave + lane) * 2, w); }
  __device__ void tile_end(int, int nt) {
    wave_lds_fence();
    if (lane * 16 < nt * 64) {
      const uint4 a = ld128(tile + lane * 32), b = ld128(tile + lane * 32 + 16);
      int64_t row = trow, col = tcol + lane * 16;
      while (col >= d.cols) {
        col -= d.cols;
        ++row;
      }
      uint4* dst = reinterpret_cast<uint4*>(out + row * ld_out + col);
      dst[0] = a;
      dst[1] = b;
    }
    wave_lds_fence();
    tcol += 1024;
    while (tcol >= d.cols) {
      tcol -= d.cols;
      ++trow;
    }
  }
};

template <bool PAIR>
__global__ __launch_bounds__(1024) void decompress_kernel(DevMatrix d, uint16_t* __restrict__ out, int64_t ld_out) {
  extern __shared__ uint32_t lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int waves = blockDim.x / kWave;
  const uint32_t stage = kAreaAddr + wave * (d.stage_words + kRingWords + kTransposeWords) * 4;
  const uint32_t ring = stage + d.stage_words * 4;
  const uint32_t tile = ring + kRingWords * 4;
  build_tables<PAIR>(d, lds, lds + kTableWords);
  __syncthreads();
  const int total_waves = gridDim.x * waves;
  for (int blk = blockIdx.x * waves + wave; blk < d.n_blocks; blk += total_waves) {
    const int64_t flat = int64_t(blk) * d.G * 64;
    DecompressSink sink{d, out, ld_out, tile, lane, flat / d.cols, flat % d.cols};
    decode_block<PAIR>(d, blk, stage, ring, lane, sink);
  }
}

// Plain-mode matrices: a strided copy of the stored bf16 bits.
__global__ void copy_plain_kernel(const uint16_t* __restrict__ src, int64_t rows, int64_t cols,
                                  uint16_t* __restrict__ out, int64_t ld_out) {
  const int64_t per_row = cols / 8;
  const int64_t n = rows * per_row;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = i / per_row, c8 = i - r * per_row;
    reinterpret_cast<uint4*>(out + r * ld_out)[c8] = reinterpret_cast<const uint4*>(src + r * cols)[c8];
  }
}

// ---------------------------------------------------------------------------
// Fused product Y[b, n] = sum_k X[b, k] W[n, k] for NBP batch columns per pass.
// X lives in LDS at kAreaAddr: bf16 as pairs, word (p*64 + l)*NBP + b =
// X[b][128p + l] | X[b][128p + 64 + l] << 16 (column groups 2p and 2p+1 at
// lane l); fp32 as word k*NBP + b = X[b][k].
template <int NBP, bool XF32>
__device__ inline void load_x(const DevMatrix& d, const void* X, int64_t ldx, int nb_valid, uint32_t* xl) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int64_t C = d.cols;
  if (XF32) {
    const float* x = static_cast<const float*>(X);
    for (uint32_t i = tid; i < uint32_t(C) * NBP; i += nt) {
      const uint32_t k = i / NBP;
      const int b = int(i % NBP);
      xl[i] = b < nb_valid ? f32_bits(x[b * ldx + k]) : 0u;
    }
  } else {
    const uint16_t* x = static_cast<const uint16_t*>(X);
    const uint32_t npairs = (uint32_t(d.gpr) + 1) / 2;
    for (uint32_t i = tid; i < npairs * 64 * NBP; i += nt) {
      const uint32_t pl = i / NBP;
      const int b = int(i % NBP);
      const uint32_t p = pl / 64, l = pl % 64;
      const int64_t k0 = 128 * int64_t(p) + l, k1 = k0 + 64;
      uint32_t v = 0;
      if (b < nb_valid) {
        v = x[b * ldx + k0];
        if (k1 < C) v |= uint32_t(x[b * ldx + k1]) << 16;
      }
      xl[i] = v;
    }
  }
}

template <int NBP, bool XF32, bool YBF16>
struct ProductSink {
  const DevMatrix& d;
  uint32_t xaddr;  // LDS byte address of x
  int lane;
  int nb_valid;
  void* Y;
  int64_t ldy;
  int64_t cur_row;
  int c0;
  uint32_t xtile;  // x address of this lane for column group c0
  float acc[NBP];
  // Finished rows are parked in registers (lane r holds the r-th finished row
  // of the unit) and written with one store after the unit, so the decode
  // loop issues no global stores.
  float rows_done[NBP];
  int64_t first_row;
  int n_done;

  __device__ void store_done() {
#pragma unroll
    for (int b = 0; b < NBP; ++b) {
      if (lane < n_done && b < nb_valid) {
        if (YBF16) static_cast<uint16_t*>(Y)[b * ldy + first_row + lane] = f32_to_bf16(rows_done[b]);
        else static_cast<float*>(Y)[b * ldy + first_row + lane] = rows_done[b];
      }
    }
    first_row += n_done;
    n_done = 0;
  }
  __device__ void flush() {
#pragma unroll
    for (int b = 0; b < NBP; ++b) {
      const float s = wave_sum(acc[b]);
      rows_done[b] = lane == n_done ? s : rows_done[b];
      acc[b] = 0.f;
    }
    ++n_done;  // a unit covers at most 64 rows (checked on the host)
  }
  __device__ void to_row(int64_t row) {
    if (row != cur_row) {
      flush();
      cur_row = row;
    }
  }
  __device__ void tile_begin(int64_t row0, int c) {
    to_row(row0);
    c0 = c;
    xtile = XF32 ? xaddr + ((uint32_t(c) * 64 + lane) * NBP) * 4 : xaddr + (((uint32_t(c) >> 1) * 64 + lane) * NBP) * 4;
  }
  // x of column group cg at this lane
  __device__ float x_at(int cg, int b) const {
    if (XF32) return bits_f32(ld32(xaddr + ((uint32_t(cg) * 64 + lane) * NBP + b) * 4));
    const uint32_t v = ld32(xaddr + (((uint32_t(cg) >> 1) * 64 + lane) * NBP + b) * 4);
    return bits_f32((cg & 1) ? (v & 0xFFFF0000u) : (v << 16));
  }
  // tile_begin() guarantees an even c0, so pair k reads x word (c0/2 + k)*64 + lane
  __device__ void pair(int k, uint32_t D) {
    if (XF32) {
      const float wa = bits_f32(D << 16), wb = bits_f32(D & 0xFFFF0000u);
      const uint32_t a = xtile + uint32_t(2 * k * 64 * NBP * 4);
#pragma unroll
      for (int b = 0; b < NBP; ++b) {
        acc[b] = __builtin_fmaf(wa, bits_f32(ld32(a + 4 * b)), acc[b]);
        acc[b] = __builtin_fmaf(wb, bits_f32(ld32(a + 64 * NBP * 4 + 4 * b)), acc[b]);
      }
    } else {
      const uint32_t a = xtile + uint32_t(k * 64 * NBP * 4);
#pragma unroll
      for (int b = 0; b < NBP; ++b) acc[b] = dot2_bf16(D, ld32(a + 4 * b), acc[b]);
    }
  }
  __device__ void single(int, int64_t row, int cg, uint32_t w) {
    to_row(row);
    const float wf = bits_f32(w << 16);
#pragma unroll
    for (int b = 0; b < NBP; ++b) acc[b] = __builtin_fmaf(wf, x_at(cg, b), acc[b]);
  }
  __device__ void tile_end(int, int) {}
};

// Wide batch chunks need more registers per lane: at most 8 waves per workgroup.
constexpr int fused_max_threads(int nbp) { return nbp >= 4 ? 512 : 1024; }

template <int NBP, bool XF32, bool PAIR, bool YBF16>
__global__ __launch_bounds__(fused_max_threads(NBP)) void fused_product_kernel(DevMatrix d, const void* __restrict__ X, int64_t ldx,
                                                             int nb_valid, void* __restrict__ Y, int64_t ldy) {
  extern __shared__ uint32_t lds[];
  const uint32_t x_words = XF32 ? uint32_t(d.cols) * NBP : ((uint32_t(d.gpr) + 1) / 2) * 64 * NBP;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int waves = blockDim.x / kWave;
  const uint32_t stage = kAreaAddr + (x_words + wave * (d.stage_words + kRingWords)) * 4;
  const uint32_t ring = stage + d.stage_words * 4;
  build_tables<PAIR>(d, lds, lds + kTableWords);
  load_x<NBP, XF32>(d, X, ldx, nb_valid, lds + kTableWords + kT1Words);
  __syncthreads();
  const int total_waves = gridDim.x * waves;
  for (int unit = blockIdx.x * waves + wave; unit < d.n_units; unit += total_waves) {
    const int blk_begin = unit * d.unit_blocks;
    const int blk_end = std::min(d.n_blocks, blk_begin + d.unit_blocks);
    const int64_t row_begin = (int64_t(blk_begin) * d.G) / d.gpr;
    ProductSink<NBP, XF32, YBF16> sink{d, kAreaAddr, lane, nb_valid, Y, ldy, row_begin, 0, 0u, {}, {}, row_begin, 0};
#pragma unroll
    for (int b = 0; b < NBP; ++b) sink.acc[b] = sink.rows_done[b] = 0.f;
    for (int blk = blk_begin; blk < blk_end; ++blk) decode_block<PAIR>(d, blk, stage, ring, lane, sink);
    sink.flush();
    sink.store_done();
  }
}

// ---------------------------------------------------------------------------
// Fused product on the matrix cores (batch >= 16): Y[b, n] = sum_k X[b, k] W[n, k].
//
// A workgroup of nw waves decodes nw blocks (or nw rows of blocks) in
// lockstep, one 16-group tile per step.  Every wave's tile lies in one row
// and covers the same 1024 columns, so after a step the workgroup holds an
// nw x 1024 bf16 slice of W in LDS (one row per wave, in natural column
// order).  That slice is the A operand of v_mfma_f32_16x16x32_bf16 (rows of
// the slice = M, padded to 16 with zeros); 16 activation rows are the B
// operand, read straight from global memory (8 consecutive bf16 per lane, so
// the k order of A and B agree).  The 32 k-steps of a slice are spread over
// the waves; each wave accumulates its share for every batch tile, and the
// partial sums are added across waves in a fixed order when the rows end.
constexpr int kMfmaRing = 2;               // sm tiles per wave in flight
constexpr uint32_t kWRowBytes = 2048 + 16;  // one row of a slice; the pad keeps the A reads conflict-free

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// How the workgroups walk the matrix (set on the host).
struct MfmaGeom {
  int nw;               // waves per workgroup = W rows per slice
  int by_block;         // 1: wave w decodes block task*nw + w (G a multiple of the groups per row)
                        // 0: wave w decodes the blocks of row task*nw + w (G divides the groups per row)
  int rows_per_block;   // by_block: G / groups per row
  int seq_blocks;       // blocks per wave and task (1, or groups per row / G)
  int tiles_per_block;  // G / 16
  int tiles_per_row;    // groups per row / 16
  int n_tasks;
};

__device__ inline floatx4 mfma_bf16(const uint4& a, const uint4& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// One wave's tile into its row of the slice: pair k holds columns 64*(2k) + lane
// and 64*(2k+1) + lane.
struct SliceSink {
  uint32_t row_addr;
  int lane;
  __device__ void pair(int k, uint32_t D) {
    st16(row_addr + ((2 * k) * kWave + lane) * 2, D);
    st16(row_addr + ((2 * k + 1) * kWave + lane) * 2, D >> 16);
  }
};

// IPW k-steps per wave and slice go with the wave count (IPW = ceil(32 / nw)):
// 16 waves (2), 11..15 (3), 8..10 (4); fewer waves leave more registers.
constexpr int mfma_max_threads(int ipw) { return ipw == 2 ? 1024 : ipw == 3 ? 960 : 640; }

template <int TB, int IPW, bool PAIR, bool YBF16>
__global__ __launch_bounds__(mfma_max_threads(IPW)) void fused_mfma_kernel(DevMatrix d, MfmaGeom g, const uint16_t* __restrict__ X,
                                                          int64_t ldx, int nb_valid, void* __restrict__ Y, int64_t ldy) {
  extern __shared__ uint32_t lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int nw = g.nw;
  const uint32_t slice = kAreaAddr;  // nw rows of kWRowBytes; also the reduction area
  const uint32_t per_wave = d.stage_words * 4 + kMfmaRing * 1024;
  const uint32_t stage = slice + uint32_t(nw) * kWRowBytes + uint32_t(wave) * per_wave;
  const uint32_t ring = stage + d.stage_words * 4;
  const uint32_t my_row = slice + uint32_t(wave) * kWRowBytes;
  const uint32_t pmask = PAIR ? 0x3FFCu : (((1u << d.L) - 1u) << 2);
  build_tables<PAIR>(d, lds, lds + kTableWords);
  __syncthreads();

  // A operand row of this lane (rows >= nw are zero padding)
  const int a_row = lane % 16, a_quad = lane / 16;
  const uint32_t a_addr = slice + uint32_t(a_row < nw ? a_row : 0) * kWRowBytes + a_quad * 16;
  // B operand: activation row b = 16 tb + lane % 16 (clamped for the address), 8 columns at 8 * (lane / 16)
  const uint16_t* xrow[TB];
  bool xvalid[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int b = 16 * tb + lane % 16;
    xvalid[tb] = b < nb_valid;
    xrow[tb] = X + int64_t(b < nb_valid ? b : 0) * ldx + 8 * a_quad;
  }
  const int seq_tiles = g.seq_blocks * g.tiles_per_block;

  for (int task = blockIdx.x; task < g.n_tasks; task += gridDim.x) {
    floatx4 acc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
    uint4 xv[IPW][TB];
    for (int sb = 0; sb < g.seq_blocks; ++sb) {
      // this wave's block
      int blk;
      bool valid;
      if (g.by_block) {
        blk = task * nw + wave;
        valid = blk < d.n_blocks;
      } else {
        const int64_t row = int64_t(task) * nw + wave;
        valid = row < d.rows;
        blk = int(row * g.seq_blocks + sb);
      }
      int ntiles = 0;
      BlockHead head{0u, 0u};
      const uint4* sm_blk = nullptr;
      // earlier ring loads (clamped repeats of the last tile) land before the slots are reused
      __builtin_amdgcn_s_waitcnt(0);
      if (valid) {
        const int64_t g_first = int64_t(blk) * d.G;
        ntiles = int((std::min<int64_t>(d.G, d.n_groups - g_first) + 15) / 16);
        head = issue_head_loads(d, blk, lane);
        sm_blk = reinterpret_cast<const uint4*>(d.sm + int64_t(blk) * d.G * 64);
#pragma unroll
        for (int i = 0; i < kMfmaRing; ++i) load_sm_tile_to_lds(sm_blk, std::min(i, ntiles - 1), ring, i, lane);
        issue_stage_loads(d, blk, stage, lane);
      }
      // activations of the first step
      {
        const int64_t col0 = int64_t(((sb * g.tiles_per_block) % g.tiles_per_row)) * 1024;
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
          const int kk = (wave + i * nw) & 31;  // distinct per i: a merged load would upset the vmcnt count
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) xv[i][tb] = *reinterpret_cast<const uint4*>(xrow[tb] + col0 + 32 * kk);
        }
      }
      Cursor c{0u, 0u, 0u, 0u, 0u};
      __builtin_amdgcn_s_waitcnt(0);
      if (valid) {
        const uint32_t start_bit = wave_exclusive_scan(head.lane_bits, lane);
        wave_lds_fence();
        const uint32_t bit = 4 * 32 + start_bit - 2;
        c.addr = stage + (bit >> 5) * 4;
        c.qm = bit & 31;
        cursor_reload(c);
      }
      const uint32_t raw_area = stage + d.stage_raw_word * 4;
      uint32_t raw_rank = 0;

      for (int t = 0; t < g.tiles_per_block; ++t) {
        const int tau = sb * g.tiles_per_block + t;
        // decode this wave's tile into its slice row
        if (valid && t < ntiles) {
          // newer than ring load t: the activations of this step and ring load t+1
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(IPW * TB + 1) : "memory");
          const uint4 cur = ld128(ring + (t % kMfmaRing) * 1024 + lane * 16);
          const uint32_t rmask = raw_mask16(head.raw_word, t * 16);
          SliceSink sink{my_row, lane};
          decode_tile_pairs<PAIR>(c, cur, rmask, raw_area, raw_rank, pmask, lane, sink);
          raw_rank += __builtin_popcount(rmask);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) st32(my_row + (i * kWave + lane) * 4, 0u);
        }
        __syncthreads();
        // matrix cores: k-steps wave, wave + nw, ... of the 32 in this slice
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
          const int kk = wave + i * nw;
          if (kk < 32) {
            uint4 a = ld128(a_addr + kk * 64);
            if (a_row >= nw) a = uint4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
              const uint4 b = xvalid[tb] ? xv[i][tb] : uint4{0u, 0u, 0u, 0u};
              acc[tb] = mfma_bf16(a, b, acc[tb]);
            }
          }
        }
        __syncthreads();
        // activations of the next step (a fixed count per step keeps the vmcnt arithmetic exact),
        // then the ring refill
        if (t + 1 < g.tiles_per_block) {
          const int64_t col0 = int64_t((tau + 1) % g.tiles_per_row) * 1024;
#pragma unroll
          for (int i = 0; i < IPW; ++i) {
            const int kk = (wave + i * nw) & 31;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) xv[i][tb] = *reinterpret_cast<const uint4*>(xrow[tb] + col0 + 32 * kk);
          }
          if (valid && t < ntiles)
            load_sm_tile_to_lds(sm_blk, std::min(t + kMfmaRing, ntiles - 1), ring, t % kMfmaRing, lane);
        }
        // the rows of this slice end here: add the partial sums of all waves
        if ((tau + 1) % g.tiles_per_row == 0) {
#pragma unroll
          for (int r = 0; r < TB; r += 2) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              if (r + q < TB) {
                const floatx4 v = acc[r + q];
                st128(slice + ((wave * 2 + q) * kWave + lane) * 16,
                      uint4{f32_bits(v.x), f32_bits(v.y), f32_bits(v.z), f32_bits(v.w)});
              }
            }
            __syncthreads();
            const int nvals = (TB - r >= 2 ? 2 : 1) * 256;
            for (int v = threadIdx.x; v < nvals; v += blockDim.x) {
              const int q = v / 256, rem = v % 256, l = rem / 4, e = rem % 4;
              float s = 0.f;
              for (int w = 0; w < nw; ++w) s += bits_f32(ld32(slice + ((w * 2 + q) * kWave + l) * 16 + e * 4));
              const int m = 4 * (l / 16) + e;  // slice row
              const int b = 16 * (r + q) + l % 16;
              int64_t row;
              bool ok;
              if (g.by_block) {
                const int64_t mb = int64_t(task) * nw + m;
                row = mb * g.rows_per_block + tau / g.tiles_per_row;
                ok = mb < d.n_blocks;
              } else {
                row = int64_t(task) * nw + m;
                ok = true;
              }
              if (m < nw && ok && row < d.rows && b < nb_valid) {
                if (YBF16) static_cast<uint16_t*>(Y)[b * ldy + row] = f32_to_bf16(s);
                else static_cast<float*>(Y)[b * ldy + row] = s;
              }
            }
            __syncthreads();
          }
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) acc[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
  }
}

// Wave-sum each accumulator and store it as row `row` of Y (lane 0 writes).
template <int NBP, bool YBF16>
__device__ inline void flush_row(float (&acc)[NBP], int64_t row, int nb_valid, void* Y, int64_t ldy, int lane) {
#pragma unroll
  for (int b = 0; b < NBP; ++b) {
    const float s = wave_sum(acc[b]);
    if (lane == 0 && b < nb_valid) {
      if (YBF16) static_cast<uint16_t*>(Y)[b * ldy + row] = f32_to_bf16(s);
      else static_cast<float*>(Y)[b * ldy + row] = s;
    }
    acc[b] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// Uncompressed bf16 product on the vector ALU (small batch): one wave per
// output row, lanes stride the row in 16-byte chunks, X in LDS as [b][k].
template <int NBP, bool XF32, bool YBF16>
__global__ __launch_bounds__(256) void bf16_gemv_kernel(const uint16_t* __restrict__ W, int64_t rows, int64_t cols,
                                                        int64_t ldw, const void* __restrict__ X, int64_t ldx, int nb_valid,
                                                        void* __restrict__ Y, int64_t ldy) {
  extern __shared__ uint32_t lds[];
  const int tid = threadIdx.x, lane = tid % kWave, wave = __builtin_amdgcn_readfirstlane(tid / kWave), waves = blockDim.x / kWave;
  // X staged as fp32 [b][k] (fp32 input) or bf16 pairs [b][k/2]
  const int64_t kp = cols / 2;
  if (XF32) {
    for (int64_t i = tid; i < cols * NBP; i += blockDim.x) {
      const int b = int(i / cols);
      const int64_t k = i - int64_t(b) * cols;
      lds[i] = b < nb_valid ? f32_bits(static_cast<const float*>(X)[b * ldx + k]) : 0u;
    }
  } else {
    for (int64_t i = tid; i < kp * NBP; i += blockDim.x) {
      const int b = int(i / kp);
      const int64_t k2 = i - int64_t(b) * kp;
      const uint16_t* xr = static_cast<const uint16_t*>(X) + b * ldx + 2 * k2;
      lds[i] = b < nb_valid ? (uint32_t(xr[0]) | (uint32_t(xr[1]) << 16)) : 0u;
    }
  }
  __syncthreads();
  const int64_t nchunks = cols / 8;
  for (int64_t row = int64_t(blockIdx.x) * waves + wave; row < rows; row += int64_t(gridDim.x) * waves) {
    const uint4* wr = reinterpret_cast<const uint4*>(W + row * ldw);
    float acc[NBP];
#pragma unroll
    for (int b = 0; b < NBP; ++b) acc[b] = 0.f;
    int64_t ch = lane;
    for (; ch + 3 * kWave < nchunks; ch += 4 * kWave) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = wr[ch + u * kWave];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t k8 = (ch + u * kWave) * 8;
        const uint32_t wv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int b = 0; b < NBP; ++b) {
          if (XF32) {
            const float* xf = reinterpret_cast<const float*>(lds) + int64_t(b) * cols + k8;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              acc[b] = __builtin_fmaf(bits_f32(wv[q] << 16), xf[2 * q], acc[b]);
              acc[b] = __builtin_fmaf(bits_f32(wv[q] & 0xFFFF0000u), xf[2 * q + 1], acc[b]);
            }
          } else {
            const uint4 xv = *reinterpret_cast<const uint4*>(lds + int64_t(b) * kp + k8 / 2);
            acc[b] = dot2_bf16(wv[0], xv.x, acc[b]);
            acc[b] = dot2_bf16(wv[1], xv.y, acc[b]);
            acc[b] = dot2_bf16(wv[2], xv.z, acc[b]);
            acc[b] = dot2_bf16(wv[3], xv.w, acc[b]);
          }
        }
      }
    }
    for (; ch < nchunks; ch += kWave) {
      const uint4 v = wr[ch];
      const int64_t k8 = ch * 8;
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int b = 0; b < NBP; ++b) {
        if (XF32) {
          const float* xf = reinterpret_cast<const float*>(lds) + int64_t(b) * cols + k8;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[b] = __builtin_fmaf(bits_f32(wv[q] << 16), xf[2 * q], acc[b]);
            acc[b] = __builtin_fmaf(bits_f32(wv[q] & 0xFFFF0000u), xf[2 * q + 1], acc[b]);
          }
        } else {
          const uint4 xv = *reinterpret_cast<const uint4*>(lds + int64_t(b) * kp + k8 / 2);
          acc[b] = dot2_bf16(wv[0], xv.x, acc[b]);
          acc[b] = dot2_bf16(wv[1], xv.y, acc[b]);
          acc[b] = dot2_bf16(wv[2], xv.z, acc[b]);
          acc[b] = dot2_bf16(wv[3], xv.w, acc[b]);
        }
      }
    }
    flush_row<NBP, YBF16>(acc, row, nb_valid, Y, ldy, lane);
  }
}

// ---------------------------------------------------------------------------
// Streaming read: every byte read once with 16-byte loads, xor-folded into
// one word per workgroup so the loads cannot be removed.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  uint32_t x = 0;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], e = src[i + 3 * stride];
    x ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ e.x ^ e.y ^ e.z ^ e.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int t = 0; t < int(blockDim.x); ++t) s ^= red[t];
    sink[blockIdx.x] = s;
  }
}

constexpr int kProbeBlocks = 2048;

// ---------------------------------------------------------------------------
// Host-side launch helpers.
int hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return UW_OK;
  return fail(UW_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool is_pair(const DevMatrix& d) { return d.L <= 6; }

// Allow the full LDS of a CU for a kernel (once per kernel).
std::mutex g_lds_mu;
std::set<const void*> g_lds_done;

template <class K>
void allow_full_lds(K kernel) {
  const void* f = reinterpret_cast<const void*>(kernel);
  std::lock_guard<std::mutex> lk(g_lds_mu);
  if (g_lds_done.insert(f).second)
    (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLimit);
}

size_t tables_bytes() { return size_t(kTableWords + kT1Words) * 4; }

size_t x_bytes(const DevMatrix& d, int nbp, bool xf32) {
  return xf32 ? size_t(d.cols) * nbp * 4 : size_t((d.gpr + 1) / 2) * 64 * nbp * 4;
}

// Waves per workgroup: as many as the work and the LDS budget allow, up to 16.
int pick_waves(int64_t units, size_t fixed, size_t per_wave) {
  int w = int(std::min<int64_t>(16, std::max<int64_t>(1, (units + 255) / 256)));
  while (w > 1 && fixed + per_wave * w > size_t(kLdsLimit)) --w;
  return w;
}

template <int NBP, bool XF32, bool PAIR, bool YBF16>
int run_fused(const uw_matrix* m, const void* X, int64_t ldx, int nb, void* Y, int64_t ldy, void* stream) {
  const DevMatrix& d = m->dev;
  const size_t fixed = tables_bytes() + x_bytes(d, NBP, XF32);
  const size_t per_wave = (size_t(d.stage_words) + kRingWords) * 4;
  if (fixed + per_wave > size_t(kLdsLimit)) return fail(UW_ERR_UNSUPPORTED, "fused product: x does not fit on chip");
  const int waves = std::min(pick_waves(d.n_units, fixed, per_wave), fused_max_threads(NBP) / kWave);
  const size_t lds = fixed + per_wave * waves;
  const int grid = int(std::max<int64_t>(1, (d.n_units + waves - 1) / waves));
  auto kern = fused_product_kernel<NBP, XF32, PAIR, YBF16>;
  allow_full_lds(kern);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(waves * kWave), lds, static_cast<hipStream_t>(stream), d, X, ldx, nb, Y, ldy);
  return hip_check(hipGetLastError(), "fused_product_kernel launch");
}

template <int NBP, bool XF32, bool PAIR>
int run_fused_y(const uw_matrix* m, const void* X, int64_t ldx, int nb, void* Y, int64_t ldy, int yt, void* stream) {
  return yt == UW_BF16 ? run_fused<NBP, XF32, PAIR, true>(m, X, ldx, nb, Y, ldy, stream)
                       : run_fused<NBP, XF32, PAIR, false>(m, X, ldx, nb, Y, ldy, stream);
}

template <int NBP, bool XF32>
int run_fused_p(const uw_matrix* m, const void* X, int64_t ldx, int nb, void* Y, int64_t ldy, int yt, void* stream) {
  return is_pair(m->dev) ? run_fused_y<NBP, XF32, true>(m, X, ldx, nb, Y, ldy, yt, stream)
                         : run_fused_y<NBP, XF32, false>(m, X, ldx, nb, Y, ldy, yt, stream);
}

template <int NBP>
int run_fused_x(const uw_matrix* m, const void* X, int64_t ldx, int xt, int nb, void* Y, int64_t ldy, int yt, void* stream) {
  return xt == UW_F32 ? run_fused_p<NBP, true>(m, X, ldx, nb, Y, ldy, yt, stream)
                      : run_fused_p<NBP, false>(m, X, ldx, nb, Y, ldy, yt, stream);
}

// Largest batch chunk (1, 2, 4 or 8) whose X copy fits next to the tables and one stage buffer per wave.
int fused_chunk(const DevMatrix& d, int64_t batch, bool xf32) {
  int nbp = 8;
  while (nbp > 1 && (nbp / 2 >= batch ||
                     tables_bytes() + x_bytes(d, nbp, xf32) + (size_t(d.stage_words) + kRingWords) * 4 * 4 >
                         size_t(kLdsLimit)))
    nbp /= 2;
  return nbp;
}

template <int NBP, bool XF32, bool YBF16>
int run_bf16(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw, const void* X, int64_t ldx, int nb, void* Y,
             int64_t ldy, void* stream) {
  const size_t lds = XF32 ? size_t(cols) * NBP * 4 : size_t(cols / 2) * NBP * 4;
  const int waves = 4;
  const int64_t grid = std::min<int64_t>((rows + waves - 1) / waves, 8192);
  auto kern = bf16_gemv_kernel<NBP, XF32, YBF16>;
  allow_full_lds(kern);
  hipLaunchKernelGGL(kern, dim3(int(grid)), dim3(waves * kWave), lds, static_cast<hipStream_t>(stream), W, rows, cols,
                     ldw, X, ldx, nb, Y, ldy);
  return hip_check(hipGetLastError(), "bf16_gemv_kernel launch");
}

template <int NBP>
int run_bf16_xy(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw, const void* X, int64_t ldx, int xt, int nb,
                void* Y, int64_t ldy, int yt, void* stream) {
  if (xt == UW_F32)
    return yt == UW_BF16 ? run_bf16<NBP, true, true>(W, rows, cols, ldw, X, ldx, nb, Y, ldy, stream)
                         : run_bf16<NBP, true, false>(W, rows, cols, ldw, X, ldx, nb, Y, ldy, stream);
  return yt == UW_BF16 ? run_bf16<NBP, false, true>(W, rows, cols, ldw, X, ldx, nb, Y, ldy, stream)
                       : run_bf16<NBP, false, false>(W, rows, cols, ldw, X, ldx, nb, Y, ldy, stream);
}

int bf16_chunk(int64_t cols, int64_t batch, bool xf32) {
  int nbp = 8;
  const size_t per = xf32 ? size_t(cols) * 4 : size_t(cols) * 2;
  while (nbp > 1 && (nbp / 2 >= batch || per * nbp > size_t(kLdsLimit))) nbp /= 2;
  return nbp;
}

size_t elem_size(int t) { return t == UW_F32 ? 4 : 2; }

}  // namespace

// ---------------------------------------------------------------------------
int launch_decompress(const uw_matrix* m, uint16_t* out, int64_t ld_out, void* stream) {
  const DevMatrix& d = m->dev;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (m->h.plain()) {
    const int64_t n = d.rows * (d.cols / 8);
    const int grid = int(std::min<int64_t>((n + 255) / 256, 8192));
    hipLaunchKernelGGL(copy_plain_kernel, dim3(grid), dim3(256), 0, s, d.plain, d.rows, d.cols, out, ld_out);
    return hip_check(hipGetLastError(), "copy_plain_kernel launch");
  }
  const size_t fixed = tables_bytes();
  const size_t per_wave = (size_t(d.stage_words) + kRingWords + kTransposeWords) * 4;
  const int waves = pick_waves(d.n_blocks, fixed, per_wave);
  const size_t lds = fixed + per_wave * waves;
  const int grid = int(std::max<int64_t>(1, (int64_t(d.n_blocks) + waves - 1) / waves));
  if (is_pair(d)) {
    allow_full_lds(decompress_kernel<true>);
    hipLaunchKernelGGL(decompress_kernel<true>, dim3(grid), dim3(waves * kWave), lds, s, d, out, ld_out);
  } else {
    allow_full_lds(decompress_kernel<false>);
    hipLaunchKernelGGL(decompress_kernel<false>, dim3(grid), dim3(waves * kWave), lds, s, d, out, ld_out);
  }
  return hip_check(hipGetLastError(), "decompress_kernel launch");
}

bool fused_supported(const uw_matrix* m, int xt, std::string* why) {
  if (m->h.plain()) return true;  // handled by the bf16 product
  const DevMatrix& d = m->dev;
  if (int64_t(d.unit_blocks) * d.G > int64_t(kWave) * d.gpr) {
    if (why) *why = "a work unit (lcm of G and the groups per row) spans more than 64 rows";
    return false;
  }
  if (tables_bytes() + x_bytes(d, 1, xt == UW_F32) + (size_t(d.stage_words) + kRingWords) * 4 > size_t(kLdsLimit)) {
    if (why) *why = "x of this width does not fit in LDS next to the decode tables";
    return false;
  }
  return true;
}

// Walk of the matrix-core kernel: waves per workgroup from the LDS budget,
// chosen so that the tasks fill whole rounds of 256 workgroups.
bool mfma_geometry(const DevMatrix& d, MfmaGeom* g, std::string* why) {
  if (d.gpr % 16) {
    if (why) *why = "the matrix-core path needs cols to be a multiple of 1024";
    return false;
  }
  if (d.G % d.gpr && d.gpr % d.G) {
    if (why) *why = "the matrix-core path needs G to divide, or be a multiple of, the groups per row";
    return false;
  }
  const size_t per_wave = kWRowBytes + size_t(d.stage_words) * 4 + kMfmaRing * 1024;
  const int nw_max = int(std::min<size_t>(16, (size_t(kLdsLimit) - tables_bytes()) / per_wave));
  if (nw_max < 8) {
    if (why) *why = "the blocks of this matrix are too large for the matrix-core path's LDS budget";
    return false;
  }
  g->by_block = d.G % d.gpr == 0;
  g->rows_per_block = g->by_block ? d.G / d.gpr : 0;
  g->seq_blocks = g->by_block ? 1 : d.gpr / d.G;
  g->tiles_per_block = d.G / 16;
  g->tiles_per_row = d.gpr / 16;
  const int64_t units = g->by_block ? int64_t(d.n_blocks) : d.rows;
  double best = -1.0;
  for (int nw = 8; nw <= nw_max; ++nw) {
    const int64_t tasks = (units + nw - 1) / nw;
    const int64_t rounds = (tasks + 255) / 256;
    const double eff = double(units) / double(rounds * 256 * nw);
    if (eff >= best - 1e-9) {
      best = eff;
      g->nw = nw;
      g->n_tasks = int(tasks);
    }
  }
  return true;
}

template <int TB, int IPW, bool PAIR>
int run_mfma(const uw_matrix* m, const MfmaGeom& g, const uint16_t* X, int64_t ldx, int nb, void* Y, int64_t ldy,
             int yt, hipStream_t s) {
  const DevMatrix& d = m->dev;
  const size_t lds = tables_bytes() + size_t(g.nw) * (kWRowBytes + size_t(d.stage_words) * 4 + kMfmaRing * 1024);
  auto kern = yt == UW_BF16 ? fused_mfma_kernel<TB, IPW, PAIR, true> : fused_mfma_kernel<TB, IPW, PAIR, false>;
  allow_full_lds(kern);
  hipLaunchKernelGGL(kern, dim3(g.n_tasks), dim3(g.nw * kWave), lds, s, d, g, X, ldx, nb, Y, ldy);
  return hip_check(hipGetLastError(), "fused_mfma_kernel launch");
}

template <int TB, bool PAIR>
int run_mfma_ipw(const uw_matrix* m, const MfmaGeom& g, const uint16_t* X, int64_t ldx, int nb, void* Y, int64_t ldy,
                 int yt, hipStream_t s) {
  if (g.nw >= 16) return run_mfma<TB, 2, PAIR>(m, g, X, ldx, nb, Y, ldy, yt, s);
  if (g.nw >= 11) return run_mfma<TB, 3, PAIR>(m, g, X, ldx, nb, Y, ldy, yt, s);
  return run_mfma<TB, 4, PAIR>(m, g, X, ldx, nb, Y, ldy, yt, s);
}

template <bool PAIR>
int run_mfma_tb(const uw_matrix* m, const MfmaGeom& g, const uint16_t* X, int64_t ldx, int nb, void* Y, int64_t ldy,
                int yt, hipStream_t s) {
  if (nb <= 16) return run_mfma_ipw<1, PAIR>(m, g, X, ldx, nb, Y, ldy, yt, s);
  if (nb <= 32) return run_mfma_ipw<2, PAIR>(m, g, X, ldx, nb, Y, ldy, yt, s);
  return run_mfma_ipw<4, PAIR>(m, g, X, ldx, nb, Y, ldy, yt, s);
}

bool fused_mfma_supported(const uw_matrix* m, int xt, std::string* why) {
  if (m->h.plain()) {
    if (why) *why = "a plain-mode matrix has nothing to decode";
    return false;
  }
  if (xt != UW_BF16) {
    if (why) *why = "the matrix-core path takes bf16 activations";
    return false;
  }
  MfmaGeom g;
  return mfma_geometry(m->dev, &g, why);
}

int launch_fused_mfma(const uw_matrix* m, const void* X, int64_t batch, int64_t ldx, void* Y, int64_t ldy, int yt,
                      void* stream) {
  const DevMatrix& d = m->dev;
  MfmaGeom g;
  std::string why;
  if (!mfma_geometry(d, &g, &why)) return fail(UW_ERR_UNSUPPORTED, "fused matrix-core product: " + why);
  if (reinterpret_cast<uintptr_t>(X) % 16 || ldx % 8)
    return fail(UW_ERR_UNSUPPORTED, "fused matrix-core product: X must be 16-byte aligned with ldx a multiple of 8");
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t b0 = 0; b0 < batch; b0 += 64) {
    const int nb = int(std::min<int64_t>(64, batch - b0));
    const uint16_t* Xb = static_cast<const uint16_t*>(X) + b0 * ldx;
    void* Yb = static_cast<char*>(Y) + b0 * ldy * elem_size(yt);
    const int rc = is_pair(d) ? run_mfma_tb<true>(m, g, Xb, ldx, nb, Yb, ldy, yt, s)
                              : run_mfma_tb<false>(m, g, Xb, ldx, nb, Yb, ldy, yt, s);
    if (rc) return rc;
  }
  return UW_OK;
}

int launch_fused(const uw_matrix* m, const void* X, int64_t batch, int64_t ldx, int xt, void* Y, int64_t ldy, int yt,
                 void* stream) {
  const DevMatrix& d = m->dev;
  if (m->h.plain()) return launch_bf16_gemm(d.plain, d.rows, d.cols, d.cols, X, batch, ldx, xt, Y, ldy, yt, stream);
  const int nbp = fused_chunk(d, batch, xt == UW_F32);
  for (int64_t b0 = 0; b0 < batch; b0 += nbp) {
    const int nb = int(std::min<int64_t>(nbp, batch - b0));
    const void* Xb = static_cast<const char*>(X) + b0 * ldx * elem_size(xt);
    void* Yb = static_cast<char*>(Y) + b0 * ldy * elem_size(yt);
    int rc;
    switch (nbp) {
      case 1: rc = run_fused_x<1>(m, Xb, ldx, xt, nb, Yb, ldy, yt, stream); break;
      case 2: rc = run_fused_x<2>(m, Xb, ldx, xt, nb, Yb, ldy, yt, stream); break;
      case 4: rc = run_fused_x<4>(m, Xb, ldx, xt, nb, Yb, ldy, yt, stream); break;
      default: rc = run_fused_x<8>(m, Xb, ldx, xt, nb, Yb, ldy, yt, stream); break;
    }
    if (rc) return rc;
  }
  return UW_OK;
}

bool bf16_gemm_supported(int64_t cols, int64_t batch, int xt, std::string* why) {
  (void)batch;
  const size_t per = xt == UW_F32 ? size_t(cols) * 4 : size_t(cols) * 2;
  if (per > size_t(kLdsLimit)) {
    if (why) *why = "x of this width does not fit in LDS";
    return false;
  }
  return true;
}

int launch_bf16_gemm(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw, const void* X, int64_t batch,
                     int64_t ldx, int xt, void* Y, int64_t ldy, int yt, void* stream) {
  const int nbp = bf16_chunk(cols, batch, xt == UW_F32);
  for (int64_t b0 = 0; b0 < batch; b0 += nbp) {
    const int nb = int(std::min<int64_t>(nbp, batch - b0));
    const void* Xb = static_cast<const char*>(X) + b0 * ldx * elem_size(xt);
    void* Yb = static_cast<char*>(Y) + b0 * ldy * elem_size(yt);
    int rc;
    switch (nbp) {
      case 1: rc = run_bf16_xy<1>(W, rows, cols, ldw, Xb, ldx, xt, nb, Yb, ldy, yt, stream); break;
      case 2: rc = run_bf16_xy<2>(W, rows, cols, ldw, Xb, ldx, xt, nb, Yb, ldy, yt, stream); break;
      case 4: rc = run_bf16_xy<4>(W, rows, cols, ldw, Xb, ldx, xt, nb, Yb, ldy, yt, stream); break;
      default: rc = run_bf16_xy<8>(W, rows, cols, ldw, Xb, ldx, xt, nb, Yb, ldy, yt, stream); break;
    }
    if (rc) return rc;
  }
  return UW_OK;
}

size_t read_probe_sink_bytes() { return size_t(kProbeBlocks) * 4; }

int launch_read_probe(const void* src, size_t bytes, void* sink, void* stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeBlocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), int64_t(bytes / 16), static_cast<uint32_t*>(sink));
  return hip_check(hipGetLastError(), "read_probe_kernel launch");
}

}  // namespace uw
