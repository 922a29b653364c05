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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ inline uint32_t lds_u32(const uint32_t* base, uint32_t byte_addr) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(base) + byte_addr);
}

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
// Per-lane cursor over the staged stream.
struct Cursor {
  uint32_t w0, w1;  // window words
  uint32_t widx;    // word index (in the wave's stage buffer) of w0
  uint32_t qm;      // bit offset of (next code - 2) in the window; bits >= 7 may hold garbage
};

__device__ inline void cursor_reload(Cursor& c, const uint32_t* stage) {
  c.w0 = stage[c.widx];
  c.w1 = stage[c.widx + 1];
}

__device__ inline void cursor_refill(Cursor& c, const uint32_t* stage) {
  c.widx += (c.qm >> 5) & 1u;
  c.qm &= 31u;
  cursor_reload(c, stage);
}

__device__ inline uint32_t cursor_peek(const Cursor& c) {
  return __builtin_amdgcn_alignbit(c.w1, c.w0, c.qm);
}

// Stage block `blk`'s stream into this wave's buffer and place the lane's cursor.
__device__ inline void stage_block(const DevMatrix& d, int blk, uint32_t* stage, int lane, Cursor& c) {
  const uint32_t w_begin = d.start_word[blk];
  const uint32_t n_words = d.start_word[blk + 1] - w_begin;
  const uint4* src = reinterpret_cast<const uint4*>(d.stream + w_begin);
  uint4* dst = reinterpret_cast<uint4*>(stage + kPadWords);
  for (uint32_t i = lane; i < n_words / 4; i += kWave) dst[i] = src[i];
  const uint32_t lb = d.lane_bits[int64_t(blk) * kWave + lane];
  const uint32_t start = wave_exclusive_scan(lb, lane);
  wave_lds_fence();
  const uint32_t bit = kPadWords * 32 + start - 2;
  c.widx = bit >> 5;
  c.qm = bit & 31;
  cursor_reload(c, stage);
}

// One code, from either table (the pair table's first half or the single table).
template <bool PAIR>
__device__ inline uint32_t decode_one(Cursor& c, const uint32_t* T, const uint32_t* stage, uint32_t idx_mask) {
  const uint32_t e = lds_u32(T, cursor_peek(c) & idx_mask);
  c.qm += PAIR ? ((e >> 16) & 0xF) : (e & 0xF);
  cursor_refill(c, stage);
  return e;  // exponent at bits 7..14
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

// Two bf16 weights in one register: bits of sign+mantissa from S, exponents from E.
__device__ inline uint32_t merge_pair(uint32_t S, uint32_t E) {
  return (S & 0x807F807Fu) | (E & 0x7F807F80u);
}

__device__ inline uint32_t merge_one(uint32_t sm, uint32_t E) {
  return ((sm & 0x80u) << 8) | (E & 0x7F80u) | (sm & 0x7Fu);
}

__device__ inline uint4 load_sm_tile(const DevMatrix& d, int blk, int t, int lane) {
  const uint8_t* p = d.sm + int64_t(blk) * d.G * 64 + int64_t(t) * 1024 + lane * 16;
  return *reinterpret_cast<const uint4*>(p);
}

__device__ inline uint32_t raw_mask16(const DevMatrix& d, int blk, int j0) {
  const uint32_t w = d.raw_bits[int64_t(blk) * d.rb_words + (j0 >> 5)];
  return (w >> (j0 & 31)) & 0xFFFFu;
}

// ---------------------------------------------------------------------------
// Decompress: every weight goes through a per-wave LDS tile [16][64] bf16 so
// that the stores are 2 x 16 bytes per lane of consecutive columns.
template <bool PAIR>
__global__ __launch_bounds__(1024) void decompress_kernel(DevMatrix d, uint16_t* __restrict__ out, int64_t ld_out) {
  extern __shared__ uint32_t lds[];
  uint32_t* T = lds;
  uint32_t* T1 = lds + kTableWords;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int waves = blockDim.x / kWave;
  uint32_t* stage = lds + kTableWords + kT1Words + wave * (d.stage_words + kTransposeWords);
  uint16_t* tileh = reinterpret_cast<uint16_t*>(stage + d.stage_words);
  build_tables<PAIR>(d, T, T1);
  __syncthreads();
  const uint32_t pair_mask = 0x3FFCu;
  const uint32_t single_mask = ((1u << d.L) - 1u) << 2;
  const int total_waves = gridDim.x * waves;
  for (int blk = blockIdx.x * waves + wave; blk < d.n_blocks; blk += total_waves) {
    Cursor c;
    stage_block(d, blk, stage, lane, c);
    const int64_t g_first = int64_t(blk) * d.G;
    const int gb = int(std::min<int64_t>(d.G, d.n_groups - g_first));
    const int ntiles = (gb + 15) / 16;
    const uint32_t first_raw = d.first_raw[blk];
    uint32_t raw_rank = 0;
    // first weight of the current tile as (row, column); advanced without divisions
    int64_t trow = (g_first * 64) / d.cols;
    int64_t tcol = g_first * 64 - trow * d.cols;
    uint4 smv = load_sm_tile(d, blk, 0, lane);
    for (int t = 0; t < ntiles; ++t) {
      const uint4 cur = smv;
      if (t + 1 < ntiles) smv = load_sm_tile(d, blk, t + 1, lane);
      const int j0 = t * 16;
      const int nt = std::min(16, gb - j0);
      const uint32_t rmask = raw_mask16(d, blk, j0);
      if (PAIR && nt == 16 && rmask == 0) {
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
          const uint32_t p = cursor_peek(c);
          const uint32_t e1 = lds_u32(T, p & pair_mask);
          const uint32_t p2 = p >> (e1 & 31u);
          const uint32_t e2 = lds_u32(T, p2 & pair_mask);
          c.qm += e1 + e2;
          cursor_refill(c, stage);
          const uint32_t D1 = merge_pair(sm_pair(cur, k), e1);
          const uint32_t D2 = merge_pair(sm_pair(cur, k + 1), e2);
          tileh[(2 * k) * kWave + lane] = uint16_t(D1);
          tileh[(2 * k + 1) * kWave + lane] = uint16_t(D1 >> 16);
          tileh[(2 * k + 2) * kWave + lane] = uint16_t(D2);
          tileh[(2 * k + 3) * kWave + lane] = uint16_t(D2 >> 16);
        }
      } else {
        for (int jj = 0; jj < nt; ++jj) {
          uint32_t E;
          if ((rmask >> jj) & 1u) {
            E = uint32_t(d.raw[int64_t(first_raw + raw_rank) * 64 + lane]) << 7;
            raw_rank++;
          } else {
            E = PAIR ? decode_one<true>(c, T, stage, pair_mask) : decode_one<false>(c, T, stage, single_mask);
          }
          tileh[jj * kWave + lane] = uint16_t(merge_one(sm_byte(cur, jj), E));
        }
      }
      wave_lds_fence();
      // lane l writes flattened weights [16 l, 16 l + 16) of the tile
      if (lane * 16 < nt * 64) {
        const uint4* src = reinterpret_cast<const uint4*>(tileh + lane * 16);
        const uint4 a = src[0], b = src[1];
        int64_t row = trow;
        int64_t col = tcol + lane * 16;
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
// X lives in LDS: bf16 as pairs xp[(p*64 + l)*NBP + b] = X[b][128p+l] | X[b][128p+64+l] << 16
// (groups 2p, 2p+1 of a row for lane l), fp32 as x[(k)*NBP + b].
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

// x value(s) for column group c (of a row) at lane l, as fp32
template <int NBP, bool XF32>
__device__ inline float x_at(const uint32_t* xl, int c, int lane, int b) {
  if (XF32) return bits_f32(xl[(int64_t(c) * 64 + lane) * NBP + b]);
  const uint32_t v = xl[((int64_t(c) >> 1) * 64 + lane) * NBP + b];
  return bits_f32((c & 1) ? (v & 0xFFFF0000u) : (v << 16));
}

template <int NBP, bool XF32>
__device__ inline void accumulate_pair(float (&acc)[NBP], uint32_t D, const uint32_t* xl, int c, int lane) {
  // D holds the weights of column groups c (low half) and c+1 (high half)
  if (XF32) {
    const float wa = bits_f32(D << 16), wb = bits_f32(D & 0xFFFF0000u);
#pragma unroll
    for (int b = 0; b < NBP; ++b) {
      acc[b] = __builtin_fmaf(wa, bits_f32(xl[(int64_t(c) * 64 + lane) * NBP + b]), acc[b]);
      acc[b] = __builtin_fmaf(wb, bits_f32(xl[(int64_t(c + 1) * 64 + lane) * NBP + b]), acc[b]);
    }
  } else {
    const uint32_t* xp = xl + ((int64_t(c) >> 1) * 64 + lane) * NBP;
#pragma unroll
    for (int b = 0; b < NBP; ++b) acc[b] = dot2_bf16(D, xp[b], acc[b]);
  }
}

template <int NBP, bool XF32, bool PAIR, bool YBF16>
__global__ __launch_bounds__(1024) void fused_product_kernel(DevMatrix d, const void* __restrict__ X, int64_t ldx,
                                                             int nb_valid, void* __restrict__ Y, int64_t ldy) {
  extern __shared__ uint32_t lds[];
  uint32_t* T = lds;
  uint32_t* T1 = lds + kTableWords;
  uint32_t* xl = lds + kTableWords + kT1Words;
  const int64_t x_words = XF32 ? d.cols * NBP : ((int64_t(d.gpr) + 1) / 2) * 64 * NBP;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int waves = blockDim.x / kWave;
  uint32_t* stage = xl + x_words + wave * d.stage_words;
  build_tables<PAIR>(d, T, T1);
  load_x<NBP, XF32>(d, X, ldx, nb_valid, xl);
  __syncthreads();
  const uint32_t pair_mask = 0x3FFCu;
  const uint32_t single_mask = ((1u << d.L) - 1u) << 2;
  const int total_waves = gridDim.x * waves;
  for (int unit = blockIdx.x * waves + wave; unit < d.n_units; unit += total_waves) {
    const int blk_begin = unit * d.unit_blocks;
    const int blk_end = std::min(d.n_blocks, blk_begin + d.unit_blocks);
    float acc[NBP];
#pragma unroll
    for (int b = 0; b < NBP; ++b) acc[b] = 0.f;
    int64_t cur_row = (int64_t(blk_begin) * d.G) / d.gpr;
    for (int blk = blk_begin; blk < blk_end; ++blk) {
      Cursor c;
      stage_block(d, blk, stage, lane, c);
      const int64_t g_first = int64_t(blk) * d.G;
      const int gb = int(std::min<int64_t>(d.G, d.n_groups - g_first));
      const int ntiles = (gb + 15) / 16;
      const uint32_t first_raw = d.first_raw[blk];
      uint32_t raw_rank = 0;
      // row and column group of the tile's first group; advanced without divisions
      int64_t row0 = g_first / d.gpr;
      int c0 = int(g_first - row0 * d.gpr);
      uint4 smv = load_sm_tile(d, blk, 0, lane);
      for (int t = 0; t < ntiles; ++t, c0 += 16) {
        while (c0 >= d.gpr) {
          c0 -= d.gpr;
          ++row0;
        }
        const uint4 cur = smv;
        if (t + 1 < ntiles) smv = load_sm_tile(d, blk, t + 1, lane);
        const int j0 = t * 16;
        const int nt = std::min(16, gb - j0);
        const uint32_t rmask = raw_mask16(d, blk, j0);
        if (PAIR && nt == 16 && rmask == 0 && c0 + 16 <= d.gpr && (c0 & 1) == 0) {
          if (row0 != cur_row) {
            flush_row<NBP, YBF16>(acc, cur_row, nb_valid, Y, ldy, lane);
            cur_row = row0;
          }
#pragma unroll
          for (int k = 0; k < 8; k += 2) {
            const uint32_t p = cursor_peek(c);
            const uint32_t e1 = lds_u32(T, p & pair_mask);
            const uint32_t p2 = p >> (e1 & 31u);
            const uint32_t e2 = lds_u32(T, p2 & pair_mask);
            c.qm += e1 + e2;
            cursor_refill(c, stage);
            accumulate_pair<NBP, XF32>(acc, merge_pair(sm_pair(cur, k), e1), xl, c0 + 2 * k, lane);
            accumulate_pair<NBP, XF32>(acc, merge_pair(sm_pair(cur, k + 1), e2), xl, c0 + 2 * k + 2, lane);
          }
        } else {
          int64_t row = row0;
          int cg = c0;
          for (int jj = 0; jj < nt; ++jj, ++cg) {
            if (cg >= d.gpr) {
              cg -= d.gpr;
              ++row;
            }
            if (row != cur_row) {
              flush_row<NBP, YBF16>(acc, cur_row, nb_valid, Y, ldy, lane);
              cur_row = row;
            }
            uint32_t E;
            if ((rmask >> jj) & 1u) {
              E = uint32_t(d.raw[int64_t(first_raw + raw_rank) * 64 + lane]) << 7;
              raw_rank++;
            } else {
              E = PAIR ? decode_one<true>(c, T, stage, pair_mask) : decode_one<false>(c, T, stage, single_mask);
            }
            const float w = bits_f32(merge_one(sm_byte(cur, jj), E) << 16);
#pragma unroll
            for (int b = 0; b < NBP; ++b) acc[b] = __builtin_fmaf(w, x_at<NBP, XF32>(xl, cg, lane, b), acc[b]);
          }
        }
      }
    }
    flush_row<NBP, YBF16>(acc, cur_row, nb_valid, Y, ldy, lane);
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
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave, waves = blockDim.x / kWave;
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
  const size_t per_wave = size_t(d.stage_words) * 4;
  if (fixed + per_wave > size_t(kLdsLimit)) return fail(UW_ERR_UNSUPPORTED, "fused product: x does not fit on chip");
  const int waves = pick_waves(d.n_units, fixed, per_wave);
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
                     tables_bytes() + x_bytes(d, nbp, xf32) + size_t(d.stage_words) * 4 * 4 > size_t(kLdsLimit)))
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
  const size_t per_wave = (size_t(d.stage_words) + kTransposeWords) * 4;
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
  if (tables_bytes() + x_bytes(d, 1, xt == UW_F32) + size_t(d.stage_words) * 4 > size_t(kLdsLimit)) {
    if (why) *why = "x of this width does not fit in LDS next to the decode tables";
    return false;
  }
  return true;
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
