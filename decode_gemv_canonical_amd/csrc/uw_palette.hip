// Direct-palette pipeline on gfx950: the batch-1 product, the small-batch
// product on the matrix cores and the decode of the UWP1 form (4-bit palette
// index + sign+mantissa byte per weight, raw 64-weight groups verbatim;
// layout in uw_palette.cpp).
//
// "Unweight: how we compressed an LLM 22% without sacrificing quality",
// section on the four execution pipelines: the direct palette skips
// preprocessing and the matmul rebuilds bf16 from the indices on the fly.
// Here there is no entropy decode at all, so the kernels are plain streams.
// GEMV and decode: lane l of a wave owns 16 consecutive weights of each 1024-weight tile, reads
// their 16 sign+mantissa bytes and 8 index bytes with one 16-byte and one
// 8-byte load (coalesced across the wave), looks up two exponents per index
// byte in a 256-entry LDS table, and multiplies with the 16 matching x values
// read as two 16-byte loads (x is small and stays in cache).
#include <algorithm>

#include "uw_device.h"

namespace uw {
namespace {

constexpr int kPalThreads = 256;  // 4 waves
constexpr int kPalChunk = 1;      // GEMV: tiles per register set
constexpr int kPalDecChunk = 4;   // decompress: tiles whose loads a wave issues together

struct DevPalette {
  const uint8_t* sm;
  const uint8_t* idx;
  const uint32_t* flags;
  const uint32_t* prefix;
  const uint8_t* raw;
  int64_t rows;
  int64_t tpr;  // 1024-weight tiles per row
  int64_t rows_per_wave;
  uint32_t pal[4];  // palette bytes, index i in byte i % 4 of word i / 4
};

__device__ inline uint32_t pal_byte(const DevPalette& p, int i) {
  const uint32_t w = i < 4 ? p.pal[0] : i < 8 ? p.pal[1] : i < 12 ? p.pal[2] : p.pal[3];
  return (w >> (8 * (i & 3))) & 0xFFu;
}

// table[b] = the exponents of index byte b: low nibble (even weight) in bits
// 7..14, high nibble (odd weight) in bits 23..30, where bf16 keeps them.
__device__ inline void build_pair_table(const DevPalette& p, uint32_t* table) {
  const int b = threadIdx.x;
  table[b] = (pal_byte(p, b & 15) << 7) | (pal_byte(p, b >> 4) << 23);
}

struct TileIn {
  uint4 sm;
  uint2 idx;
  uint32_t rmask;  // raw flags of the tile's 16 groups (wave-uniform)
  uint4 rawe;      // this lane's 16 raw exponents when its group is raw
};

// Raw flags and first raw slot of the 64 tiles from `base`: lane i holds those
// of tile base + i (tiles past the wave's last repeat the last).
struct WaveFlags {
  uint32_t flags, prefix;
  int64_t base;
};

__device__ inline void load_flags(const DevPalette& p, int64_t T, int64_t T1, int lane, WaveFlags& f) {
  const int64_t t = min(T + lane, T1 - 1);
  f.flags = (p.flags[t >> 1] >> (16 * (t & 1))) & 0xFFFFu;
  f.prefix = p.prefix[t];
  f.base = T;
}

// The loads of tile T (wave-uniform; tiles come in increasing order).  Every
// call issues the same four loads: a lane whose group is not raw, and every
// lane of a tile without raw groups, reads its own sign+mantissa bytes again
// in place of raw exponents.  So the compiler's wait before the products of
// one register set never waits for the loads of the other.
__device__ inline void load_tile(const DevPalette& p, int64_t T, int64_t T1, int lane, WaveFlags& f, TileIn& in) {
  if (T - f.base >= 64) {  // once per 64 tiles; the wait here keeps the paths after it alike
    load_flags(p, T, T1, lane, f);
    wait_vmcnt<0>();
  }
  const int k = int(T - f.base);
  in.rmask = __builtin_amdgcn_readlane(f.flags, k);
  const uint32_t pre = __builtin_amdgcn_readlane(f.prefix, k);
  const uint8_t* smp = p.sm + T * 1024 + 16 * lane;
  in.sm = *reinterpret_cast<const uint4*>(smp);
  in.idx = *reinterpret_cast<const uint2*>(p.idx + T * 512 + 8 * lane);
  const int g = lane >> 2;  // the lane's group within the tile
  const bool raw = (in.rmask >> g) & 1u;
  const uint32_t slot = pre + uint32_t(__builtin_popcount(in.rmask & ((1u << g) - 1u)));
  in.rawe = *reinterpret_cast<const uint4*>(raw ? p.raw + int64_t(slot) * 64 + 16 * (lane & 3) : smp);
}

__device__ inline uint32_t word_of(const uint4& v, int k) { return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w; }

// Weights 2k, 2k+1 of the lane's 16 as one register of two bf16.  RAW: the
// tile has raw groups (the lane's own may or may not be one).
template <bool RAW>
__device__ inline uint32_t pair_weights(const TileIn& in, const uint32_t* table, int lane, int k) {
  const uint32_t q = (k < 4 ? in.idx.x : in.idx.y) >> (8 * (k & 3));
  uint32_t E = table[q & 0xFFu];
  if (RAW && ((in.rmask >> (lane >> 2)) & 1u))
    E = __builtin_amdgcn_perm(0u, word_of(in.rawe, k >> 1), (k & 1) ? 0x0c030c02u : 0x0c010c00u) << 7;
  const uint32_t S = __builtin_amdgcn_perm(0u, word_of(in.sm, k >> 1), (k & 1) ? 0x03030202u : 0x01010000u);
  return (S & 0x807F807Fu) | (E & 0x7F807F80u);
}

template <bool XF32>
struct XTile {
  uint4 v[XF32 ? 4 : 2];
};

template <bool XF32>
__device__ inline void load_x(const void* X, int64_t t, int lane, XTile<XF32>& x) {
  const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(X) + (t * 1024 + 16 * lane) * (XF32 ? 4 : 2));
#pragma unroll
  for (int i = 0; i < (XF32 ? 4 : 2); ++i) x.v[i] = src[i];
}

template <bool XF32, bool RAW>
__device__ inline float tile_dot_as(const TileIn& in, const XTile<XF32>& x, const uint32_t* table, int lane, float acc) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t W = pair_weights<RAW>(in, table, lane, k);
    if (XF32) {
      const uint32_t x0 = word_of(x.v[k >> 1], 2 * (k & 1)), x1 = word_of(x.v[k >> 1], 2 * (k & 1) + 1);
      acc = __builtin_fmaf(bits_f32(W << 16), bits_f32(x0), acc);
      acc = __builtin_fmaf(bits_f32(W & 0xFFFF0000u), bits_f32(x1), acc);
    } else {
      acc = dot2_bf16(W, word_of(x.v[k >> 2], k & 3), acc);
    }
  }
  return acc;
}

template <bool XF32>
__device__ inline float tile_dot(const TileIn& in, const XTile<XF32>& x, const uint32_t* table, int lane, float acc) {
  return in.rmask ? tile_dot_as<XF32, true>(in, x, table, lane, acc) : tile_dot_as<XF32, false>(in, x, table, lane, acc);
}

// A wave's tiles T0 .. T1 - 1 are whole rows (tpr tiles each, row-major).
struct WaveTiles {
  int64_t T0, T1, r0;
  int tpr;
};

// The loads of tiles T .. T + kPalChunk - 1 (those past the wave's last load
// the last again, so every call issues the same loads).
template <bool XF32>
__device__ __forceinline__ void issue_set(const DevPalette& p, const void* X, const WaveTiles& w, int64_t T, int lane,
                                          WaveFlags& f, TileIn (&in)[kPalChunk], XTile<XF32> (&xs)[kPalChunk]) {
#pragma unroll
  for (int i = 0; i < kPalChunk; ++i) {
    const int64_t Ti = min(T + i, w.T1 - 1);
    load_tile(p, Ti, w.T1, lane, f, in[i]);
    load_x<XF32>(X, int(Ti - w.T0) % w.tpr, lane, xs[i]);
  }
}

// The products of tiles T .. T + kPalChunk - 1 (T < T1, so the first is
// always one of the wave's and runs without a branch that would leave its
// loads possibly pending).  A row's sum is reduced at its last tile and kept
// in lane (row - r0) of `res`: no store inside the loop (stores count with
// the loads on this chip and would perturb the waits).
template <bool XF32>
__device__ __forceinline__ void consume_set(const WaveTiles& w, int64_t T, float& acc, float& res, int lane,
                                            const uint32_t* table, const TileIn (&in)[kPalChunk],
                                            const XTile<XF32> (&xs)[kPalChunk]) {
#pragma unroll
  for (int i = 0; i < kPalChunk; ++i) {
    if (i == 0 || T + i < w.T1) {
      // the raw exponents count as read on every path, so their load is
      // waited for here and not, later, by the next load into these registers
      asm volatile("" ::"v"(in[i].rawe.x), "v"(in[i].rawe.y), "v"(in[i].rawe.z), "v"(in[i].rawe.w));
      acc = tile_dot<XF32>(in[i], xs[i], table, lane, acc);
      const int rel = int(T + i - w.T0);
      if (rel % w.tpr == w.tpr - 1) {
        const float s = wave_sum(acc);
        res = lane == rel / w.tpr ? s : res;
        acc = 0.f;
      }
    }
  }
}

// The wave's rows: rows_per_wave consecutive rows (the last wave may have fewer).
__device__ inline bool wave_tiles(const DevPalette& p, WaveTiles& w) {
  const int64_t wave = int64_t(blockIdx.x) * (kPalThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t r0 = wave * p.rows_per_wave;
  if (r0 >= p.rows) return false;
  const int64_t r1 = min(p.rows, r0 + p.rows_per_wave);
  w.r0 = r0;
  w.T0 = r0 * p.tpr;
  w.T1 = r1 * p.tpr;
  w.tpr = int(p.tpr);
  return true;
}

// One wave per rows_per_wave consecutive rows.  The wave walks their tiles in
// sets of kPalChunk with two register sets: the loads of the next set are in
// flight while the current one is multiplied.  Every path from the loads of
// one set to the products of the other issues a fixed number of loads (the
// next set's, or none after the last), so the compiler's wait before the
// products leaves the next set's loads in flight.
template <bool XF32, bool YBF16>
__global__ __launch_bounds__(kPalThreads) void palette_gemv_kernel(DevPalette p, const void* __restrict__ X,
                                                                   void* __restrict__ Y) {
  __shared__ uint32_t table[256];
  build_pair_table(p, table);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  WaveTiles w;
  if (!wave_tiles(p, w)) return;
  WaveFlags f;
  load_flags(p, w.T0, w.T1, lane, f);
  wait_vmcnt<0>();
  float acc = 0.f, res = 0.f;
  TileIn a[kPalChunk], b[kPalChunk];
  XTile<XF32> xa[kPalChunk], xb[kPalChunk];
  int64_t T = w.T0;
  issue_set<XF32>(p, X, w, T, lane, f, a, xa);
  while (true) {
    if (T + kPalChunk >= w.T1) {
      consume_set<XF32>(w, T, acc, res, lane, table, a, xa);
      break;
    }
    issue_set<XF32>(p, X, w, T + kPalChunk, lane, f, b, xb);
    consume_set<XF32>(w, T, acc, res, lane, table, a, xa);
    T += kPalChunk;
    if (T + kPalChunk >= w.T1) {
      consume_set<XF32>(w, T, acc, res, lane, table, b, xb);
      break;
    }
    issue_set<XF32>(p, X, w, T + kPalChunk, lane, f, a, xa);
    consume_set<XF32>(w, T, acc, res, lane, table, b, xb);
    T += kPalChunk;
  }
  if (lane < int(w.T1 - w.T0) / w.tpr) {
    if (YBF16) static_cast<uint16_t*>(Y)[w.r0 + lane] = f32_to_bf16(res);
    else static_cast<float*>(Y)[w.r0 + lane] = res;
  }
}

// bf16 weights to out[r * ld + c]: lane l writes its 16 weights as two
// 16-byte stores; a wave issues the loads of kPalDecChunk tiles together.
__global__ __launch_bounds__(kPalThreads) void palette_decompress_kernel(DevPalette p, uint16_t* __restrict__ out,
                                                                         int64_t ld) {
  __shared__ uint32_t table[256];
  build_pair_table(p, table);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  WaveTiles w;
  if (!wave_tiles(p, w)) return;
  WaveFlags f;
  load_flags(p, w.T0, w.T1, lane, f);
  wait_vmcnt<0>();
  for (int64_t T = w.T0; T < w.T1; T += kPalDecChunk) {
    TileIn in[kPalDecChunk];
#pragma unroll
    for (int i = 0; i < kPalDecChunk; ++i) load_tile(p, min(T + i, w.T1 - 1), w.T1, lane, f, in[i]);
#pragma unroll
    for (int i = 0; i < kPalDecChunk; ++i) {
      if (T + i < w.T1) {
        uint32_t v[8];
        if (in[i].rmask) {
#pragma unroll
          for (int k = 0; k < 8; ++k) v[k] = pair_weights<true>(in[i], table, lane, k);
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) v[k] = pair_weights<false>(in[i], table, lane, k);
        }
        const int rel = int(T + i - w.T0);
        uint4* dst = reinterpret_cast<uint4*>(out + (w.r0 + rel / w.tpr) * ld + int64_t(rel % w.tpr) * 1024 + 16 * lane);
        dst[0] = uint4{v[0], v[1], v[2], v[3]};
        dst[1] = uint4{v[4], v[5], v[6], v[7]};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Small-batch product on the matrix cores: Y[b][n] = sum_k X[b][k] W[n][k].
// A workgroup of KS waves owns 16 weight rows; wave w takes every KS-th
// 128-column block of them.  Per block, lane (r = lane % 16, j = lane / 16)
// loads 32 consecutive weights of row r (32 sm bytes, 16 index bytes) and, per
// batch tile, 32 consecutive activations of batch row 16 tb + r.  K-step s of
// the block then gives the lane weights 8s..8s+7 of its 32 as the A operand of
// v_mfma_f32_16x16x32_bf16 (row r, k = 8 j + e) and activations 8s..8s+7 as B
// (column r, k = 8 j + e): the matrix cores see k in a permuted order that A
// and B share, so every load is 32 or 64 contiguous bytes per lane.  The
// waves' partial sums meet in LDS at the end.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
constexpr int kPalMfmaMaxTB = 4;  // 64 batch rows per pass

struct BlockIn {
  uint4 sm[2];
  uint4 idx;
  uint4 rawe[2];
  bool raw;
};

// The lane's 32 weights of row `row` from column k0: sign+mantissa and index
// bytes, and the group's raw exponent bytes when it is raw.  The raw flag and
// the raw slot come from the workgroup's copy of its rows' tile flags and
// prefix counts in LDS (entry (row_local, tile) = (16-bit flags, prefix)), so
// no load waits on another; a lane whose group is not raw loads 32 bytes from
// the start of the sm section instead (FIXED), so every call issues the same
// loads and the wait for one register set can leave the other's in flight;
// else only raw lanes load them.
template <bool FIXED>
__device__ inline void load_block(const DevPalette& p, const uint2* rflags, int row_local, int64_t row, int64_t k0,
                                  BlockIn& in) {
  const int64_t i0 = row * p.tpr * 1024 + k0;  // weight index of the lane's first weight
  const uint4* s = reinterpret_cast<const uint4*>(p.sm + i0);
  in.sm[0] = s[0];
  in.sm[1] = s[1];
  in.idx = *reinterpret_cast<const uint4*>(p.idx + i0 / 2);
  const uint2 f = rflags[row_local * int(p.tpr) + int(k0 >> 10)];
  const int gi = int((k0 >> 6) & 15);
  in.raw = (f.x >> gi) & 1u;
  const uint32_t slot = f.y + uint32_t(__builtin_popcount(f.x & ((1u << gi) - 1u)));
  if (FIXED) {
    const uint4* r = in.raw ? reinterpret_cast<const uint4*>(p.raw + int64_t(slot) * 64 + (i0 & 63))
                            : reinterpret_cast<const uint4*>(p.sm);
    in.rawe[0] = r[0];
    in.rawe[1] = r[1];
  } else {
    in.rawe[0] = in.rawe[1] = uint4{0u, 0u, 0u, 0u};
    if (in.raw) {
      const uint4* r = reinterpret_cast<const uint4*>(p.raw + int64_t(slot) * 64 + (i0 & 63));
      in.rawe[0] = r[0];
      in.rawe[1] = r[1];
    }
  }
}

// Weights 8s..8s+7 of the lane's 32 as 8 bf16.
__device__ inline uint4 block_step_weights(const BlockIn& in, const uint32_t* table, int s) {
  uint32_t W[4];
  const uint32_t q = word_of(in.idx, s);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t E = table[(q >> (8 * p)) & 0xFFu];
    const uint32_t smw = word_of(in.sm[s >> 1], 2 * (s & 1) + (p >> 1));
    if (in.raw)
      E = __builtin_amdgcn_perm(0u, word_of(in.rawe[s >> 1], 2 * (s & 1) + (p >> 1)),
                                (p & 1) ? 0x0c030c02u : 0x0c010c00u) << 7;
    const uint32_t S = __builtin_amdgcn_perm(0u, smw, (p & 1) ? 0x03030202u : 0x01010000u);
    W[p] = (S & 0x807F807Fu) | (E & 0x7F807F80u);
  }
  return uint4{W[0], W[1], W[2], W[3]};
}

// The loads of one 128-column block: the activations of every batch tile
// (once, shared by the RB row blocks) and the lane's 32 weights of each of
// the RB rows.
template <int TB, int RB>
struct BlockSet {
  uint4 xv[TB][4];
  BlockIn in[RB];
};

template <int TB, int RB, bool FIXED>
__device__ __forceinline__ void load_set(const DevPalette& p, const uint2* rflags, const uint16_t* const (&xr)[TB],
                                         const int64_t (&row)[RB], int r, int64_t kb, int j, BlockSet<TB, RB>& b) {
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const uint4* xs = reinterpret_cast<const uint4*>(xr[tb] + kb * 128);
#pragma unroll
    for (int s = 0; s < 4; ++s) b.xv[tb][s] = xs[s];
  }
#pragma unroll
  for (int i = 0; i < RB; ++i) load_block<FIXED>(p, rflags, 16 * i + r, row[i], kb * 128 + 32 * j, b.in[i]);
}

// The four k-steps of a block for every row block and batch tile.
template <int TB, int RB>
__device__ __forceinline__ void mfma_set(const BlockSet<TB, RB>& b, const uint32_t* table, floatx4 (&acc)[RB][TB]) {
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 a = block_step_weights(b.in[i], table, s);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        acc[i][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                             __builtin_bit_cast(bf16x8_t, b.xv[tb][s]), acc[i][tb], 0, 0, 0);
    }
}

// Two block sets in registers (the next block's loads in flight while this
// one's products run) when they fit; else one, whose loads are all issued
// before its products.
template <int TB, int RB>
constexpr bool palette_two_sets() {
  return 2 * (16 * TB + 21 * RB) + 4 * RB * TB <= 200;
}

// SPLIT: two workgroups share each group of RB row blocks, each taking half
// of the 128-column blocks and adding its partial sums into Y (zeroed first;
// fp32 Y only).  Two partial sums added to zero give the same bits in either
// order, so the result is deterministic.  Every workgroup reads the
// activations of its part of K once, so the split lets a workgroup hold more
// rows (fewer reads of X in all) while the chip stays full.
template <int TB, int RB, bool YBF16, bool SPLIT>
__global__ __launch_bounds__(512) void palette_mfma_kernel(DevPalette p, const uint16_t* __restrict__ X, int64_t ldx,
                                                           int nb, void* __restrict__ Y, int64_t ldy) {
  static_assert(!(SPLIT && YBF16), "split partial sums are added in fp32");
  __shared__ uint32_t table[256];
  extern __shared__ float4 red[];  // [waves][TB][64] partial sums of one 16-row block, then the rows' tile flags
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, ks = blockDim.x >> 6;
  const int r = lane & 15, j = lane >> 4;
  const int tpr = int(p.tpr);
  uint2* rflags = reinterpret_cast<uint2*>(red + ks * TB * 64);  // [16 RB rows][tpr]: (flags, prefix)
  const int split = SPLIT ? int(blockIdx.x & 1) : 0;
  const int64_t base = int64_t(SPLIT ? blockIdx.x >> 1 : blockIdx.x) * 16 * RB;  // the workgroup's RB blocks of 16 rows
  for (int b = threadIdx.x; b < 256; b += blockDim.x) table[b] = (pal_byte(p, b & 15) << 7) | (pal_byte(p, b >> 4) << 23);
  for (int i = threadIdx.x; i < 16 * RB * tpr; i += blockDim.x) {
    const int64_t row = std::min<int64_t>(p.rows - 1, base + i / tpr);
    const int64_t T = row * tpr + i % tpr;
    rflags[i] = uint2{(p.flags[T >> 1] >> (16 * (T & 1))) & 0xFFFFu, p.prefix[T]};
  }
  __syncthreads();
  int64_t row[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) row[i] = std::min<int64_t>(p.rows - 1, base + 16 * i + r);  // rows past the end feed unstored outputs
  const uint16_t* xr[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) xr[tb] = X + int64_t(std::min(16 * tb + r, nb - 1)) * ldx + 32 * j;
  floatx4 acc[RB][TB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[i][tb] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int64_t n_all = p.tpr * 8;  // 128-column blocks per row
  const int64_t kb0 = SPLIT ? (split ? n_all / 2 : 0) : 0, n_blocks = SPLIT && !split ? n_all / 2 : n_all;  // its blocks
  if constexpr (palette_two_sets<TB, RB>()) {
    // Every path from the loads of one set to the products of the other
    // issues a fixed number of loads (the next set's, or none at the last
    // block), so the compiler's wait before the products leaves the next
    // set's loads in flight; a load under a condition in between would make
    // it wait for everything.
    BlockSet<TB, RB> sa, sb;
    int64_t kb = kb0 + wave;
    if (kb < n_blocks) {
      load_set<TB, RB, true>(p, rflags, xr, row, r, kb, j, sa);
      while (true) {
        if (kb + ks >= n_blocks) {
          mfma_set<TB, RB>(sa, table, acc);
          break;
        }
        load_set<TB, RB, true>(p, rflags, xr, row, r, kb + ks, j, sb);
        mfma_set<TB, RB>(sa, table, acc);
        kb += ks;
        if (kb + ks >= n_blocks) {
          mfma_set<TB, RB>(sb, table, acc);
          break;
        }
        load_set<TB, RB, true>(p, rflags, xr, row, r, kb + ks, j, sa);
        mfma_set<TB, RB>(sb, table, acc);
        kb += ks;
      }
    }
  } else {
    for (int64_t kb = kb0 + wave; kb < n_blocks; kb += ks) {
      BlockSet<TB, RB> sa;
      load_set<TB, RB, false>(p, rflags, xr, row, r, kb, j, sa);
      mfma_set<TB, RB>(sa, table, acc);
    }
  }
  // the waves' partial sums, one 16-row block at a time
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    if (i) __syncthreads();  // the previous block's sums are read
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
      red[(wave * TB + tb) * 64 + lane] = float4{acc[i][tb][0], acc[i][tb][1], acc[i][tb][2], acc[i][tb][3]};
    __syncthreads();
    // output (weight row m, batch column b) sits in lane 16 (m / 4) + b % 16, element m % 4
    for (int v = threadIdx.x; v < TB * 256; v += blockDim.x) {
      const int tb = v >> 8, m = (v >> 4) & 15, bc = v & 15;
      const int l = 16 * (m >> 2) + bc, e = m & 3;
      float sum = 0.f;
      for (int w = 0; w < ks; ++w) {
        const float4 q = red[(w * TB + tb) * 64 + l];
        sum += e == 0 ? q.x : e == 1 ? q.y : e == 2 ? q.z : q.w;
      }
      const int64_t n = base + 16 * i + m;
      const int b = 16 * tb + bc;
      if (n < p.rows && b < nb) {
        if (YBF16) static_cast<uint16_t*>(Y)[b * ldy + n] = f32_to_bf16(sum);
        else if (SPLIT) unsafeAtomicAdd(static_cast<float*>(Y) + b * ldy + n, sum);
        else static_cast<float*>(Y)[b * ldy + n] = sum;
      }
    }
  }
}

DevPalette dev_palette(const uw_palette* m) {
  const PaletteLayout& l = m->l;
  DevPalette p;
  p.sm = m->d_blob + l.off_sm;
  p.idx = m->d_blob + l.off_idx;
  p.flags = reinterpret_cast<const uint32_t*>(m->d_blob + l.off_flags);
  p.prefix = reinterpret_cast<const uint32_t*>(m->d_blob + l.off_prefix);
  p.raw = m->d_blob + l.off_raw;
  p.rows = l.rows;
  p.tpr = l.cols / 1024;
  // about 4 tiles per wave (one row of a 4096-column matrix): many short
  // waves keep the loads of many tiles in flight and shorten the tail
  p.rows_per_wave = std::max<int64_t>(1, 4 / p.tpr);
  for (int i = 0; i < 4; ++i)
    p.pal[i] = uint32_t(l.palette[4 * i]) | uint32_t(l.palette[4 * i + 1]) << 8 | uint32_t(l.palette[4 * i + 2]) << 16 |
               uint32_t(l.palette[4 * i + 3]) << 24;
  return p;
}

unsigned palette_blocks(const DevPalette& p) {
  const int64_t waves = (p.rows + p.rows_per_wave - 1) / p.rows_per_wave;
  return unsigned((waves + kPalThreads / 64 - 1) / (kPalThreads / 64));
}

int check_palette(const uw_palette* m, const char* where) {
  if (!m) return fail(UW_ERR_INVALID, std::string(where) + ": null handle");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(UW_ERR_HIP, std::string(where) + ": no current HIP device");
  if (dev != m->device) return fail(UW_ERR_INVALID, std::string(where) + ": handle belongs to another device");
  return UW_OK;
}

bool aligned_to(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

}  // namespace
}  // namespace uw

using namespace uw;

extern "C" int uw_palette_create(const void* host_blob, size_t n, const void* d_blob, uw_palette** out) {
  if (!host_blob || !d_blob || !out) return fail(UW_ERR_INVALID, "uw_palette_create: null pointer");
  if (!aligned_to(d_blob, 256)) return fail(UW_ERR_INVALID, "uw_palette_create: device blob must be 256-byte aligned");
  PaletteLayout l;
  if (int rc = palette_parse(host_blob, n, &l)) return rc;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(UW_ERR_HIP, "uw_palette_create: no current HIP device");
  uw_palette* m = new uw_palette;
  m->l = l;
  m->d_blob = static_cast<const uint8_t*>(d_blob);
  m->device = dev;
  *out = m;
  return UW_OK;
}

extern "C" void uw_palette_destroy(uw_palette* m) { delete m; }

extern "C" int uw_palette_gemv(const uw_palette* m, const void* d_x, int xt, void* d_y, int yt, void* stream) {
  if (int rc = check_palette(m, "uw_palette_gemv")) return rc;
  if ((xt != UW_F32 && xt != UW_BF16) || (yt != UW_F32 && yt != UW_BF16))
    return fail(UW_ERR_INVALID, "uw_palette_gemv: types must be UW_F32 or UW_BF16");
  if (!d_x || !aligned_to(d_x, 16)) return fail(UW_ERR_INVALID, "uw_palette_gemv: x must be non-null and 16-byte aligned");
  if (!d_y || !aligned_to(d_y, yt == UW_F32 ? 4 : 2))
    return fail(UW_ERR_INVALID, "uw_palette_gemv: y must be non-null and aligned to its element");
  const DevPalette p = dev_palette(m);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(palette_blocks(p)), block(kPalThreads);
  if (xt == UW_BF16) {
    if (yt == UW_BF16) hipLaunchKernelGGL((palette_gemv_kernel<false, true>), grid, block, 0, s, p, d_x, d_y);
    else hipLaunchKernelGGL((palette_gemv_kernel<false, false>), grid, block, 0, s, p, d_x, d_y);
  } else {
    if (yt == UW_BF16) hipLaunchKernelGGL((palette_gemv_kernel<true, true>), grid, block, 0, s, p, d_x, d_y);
    else hipLaunchKernelGGL((palette_gemv_kernel<true, false>), grid, block, 0, s, p, d_x, d_y);
  }
  return hip_check(hipGetLastError(), "palette_gemv_kernel launch");
}

extern "C" int uw_palette_decompress(const uw_palette* m, uint16_t* d_out, int64_t ld_out, void* stream) {
  if (int rc = check_palette(m, "uw_palette_decompress")) return rc;
  if (!d_out || !aligned_to(d_out, 16))
    return fail(UW_ERR_INVALID, "uw_palette_decompress: output must be non-null and 16-byte aligned");
  if (ld_out < m->l.cols || ld_out % 8)
    return fail(UW_ERR_INVALID, "uw_palette_decompress: ld_out must be >= cols and a multiple of 8");
  const DevPalette p = dev_palette(m);
  hipLaunchKernelGGL(palette_decompress_kernel, dim3(palette_blocks(p)), dim3(kPalThreads), 0,
                     static_cast<hipStream_t>(stream), p, d_out, ld_out);
  return hip_check(hipGetLastError(), "palette_decompress_kernel launch");
}

// Workgroup shape: RB blocks of 16 rows share each activation load (fewer
// re-reads of X from cache as the batch grows), and KS waves split K (at most
// 8: a 1024-column multiple splits into 8 blocks of 128).  The largest RB
// that still leaves about 1792 waves, then the fewest KS that reach it.
// Row blocks per workgroup (rb), waves splitting K within it (ks) and
// workgroups splitting K (nsplit).  rb: the largest of 4, 2, 1 that still
// gives about 224 workgroups of 8 waves.  Where that leaves one row block
// per workgroup (few rows: down_proj 4096 x 14336), Y is fp32 and there are
// two or more batch tiles, two row blocks and two workgroups per group
// instead: as many workgroups, half the reads of X (down at 32 / 64 batch
// rows: 42.7 / 69.7 -> 35.6 / 51.1 us; at 4 / 16 rows, where X is small,
// 22.7 / 29.7 -> 26.5 / 31.4, so not there).
void palette_mfma_shape(int64_t rows, int64_t kblocks, int tb, int nb, bool yf32, int* rb, int* ks, int* nsplit) {
  const int64_t blocks16 = (rows + 15) / 16;
  *rb = 1;
  *nsplit = 1;
  for (int c : {4, 2})
    if ((blocks16 + c - 1) / c * 8 >= 1792) {
      *rb = c;
      break;
    }
  if (*rb == 1 && yf32 && tb >= 2 && blocks16 >= 128 && kblocks >= 32) {
    *rb = 2;
    *nsplit = 2;
  }
  const int64_t wgs = (blocks16 + *rb - 1) / *rb * *nsplit;
  *ks = 1;
  while (*ks < 8 && wgs * *ks < 1792) *ks *= 2;
  // one batch tile over 4 row blocks: 4 waves splitting K are ahead of 8
  // (gate_proj at 1 / 4 / 16 rows, interleaved, 8 cold copies: 24.4 / 24.6 /
  // 25.5 us against 25.0 / 25.1 / 26.1); with more batch tiles 8 stay ahead.
  // Up to 4 batch rows, 2 row blocks (two register sets) with 4 waves are
  // ahead again (23.5 / 23.7 / 24.2 us at 1 / 2 / 4 rows; 29.6 at 16).
  if (tb == 1 && *rb == 4) {
    *ks = std::min(*ks, 4);
    if (nb <= 4) *rb = 2;
  }
}

// Y[b][0 .. rows) = 0 for batch row b = blockIdx.y; 16-byte stores when every
// row starts 16-byte aligned (VEC), else 4-byte ones.
template <bool VEC>
__global__ void zero_f32_rows_kernel(float* __restrict__ Y, int64_t rows, int64_t ldy) {
  float* y = Y + int64_t(blockIdx.y) * ldy;
  const int64_t i = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (VEC && i + 4 <= rows) {
    *reinterpret_cast<float4*>(y + i) = float4{0.f, 0.f, 0.f, 0.f};
  } else {
    for (int64_t j = i; j < std::min<int64_t>(i + 4, rows); ++j) y[j] = 0.f;
  }
}

template <int TB, int RB>
int launch_palette_mfma_rb(const DevPalette& p, const uint16_t* X, int64_t ldx, int nb, void* Y, int64_t ldy, int yt,
                           int ks, int nsplit, hipStream_t s) {
  // the split kernel is instantiated for 2 row blocks and 2 or more batch tiles, fp32 Y
  const bool split = RB == 2 && TB >= 2 && yt == UW_F32 && nsplit == 2;
  const size_t lds = size_t(ks) * TB * 64 * sizeof(float4) + size_t(16) * RB * size_t(p.tpr) * 8;
  const dim3 grid(unsigned((p.rows + 16 * RB - 1) / (16 * RB) * (split ? 2 : 1))), block(64 * ks);
  // the kernel also holds a 1 KiB static table
  if (lds + 1024 > size_t(kLdsLimit)) return fail(UW_ERR_UNSUPPORTED, "uw_palette_gemm: too many tiles per row");
  auto kern = yt == UW_BF16 ? palette_mfma_kernel<TB, RB, true, false> : palette_mfma_kernel<TB, RB, false, false>;
  if constexpr (RB == 2 && TB >= 2)
    if (split) kern = palette_mfma_kernel<TB, RB, false, true>;
  if (lds > 48 * 1024) {
    static std::mutex mu;
    std::lock_guard<std::mutex> lk(mu);
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              kLdsLimit - 1024);
  }
  if (split) {  // the workgroups add their partial sums into Y
    const dim3 zgrid(unsigned((p.rows + 1023) / 1024), unsigned(nb));
    if (aligned_to(Y, 16) && ldy % 4 == 0)
      hipLaunchKernelGGL(zero_f32_rows_kernel<true>, zgrid, dim3(256), 0, s, static_cast<float*>(Y), p.rows, ldy);
    else
      hipLaunchKernelGGL(zero_f32_rows_kernel<false>, zgrid, dim3(256), 0, s, static_cast<float*>(Y), p.rows, ldy);
    if (int rc = hip_check(hipGetLastError(), "zero_f32_rows_kernel launch")) return rc;
  }
  hipLaunchKernelGGL(kern, grid, block, lds, s, p, X, ldx, nb, Y, ldy);
  return hip_check(hipGetLastError(), "palette_mfma_kernel launch");
}

template <int TB>
int launch_palette_mfma(const DevPalette& p, const uint16_t* X, int64_t ldx, int nb, void* Y, int64_t ldy, int yt,
                        hipStream_t s) {
  int rb, ks, nsplit;
  palette_mfma_shape(p.rows, p.tpr * 8, TB, nb, yt == UW_F32, &rb, &ks, &nsplit);
  if (rb == 4) return launch_palette_mfma_rb<TB, 4>(p, X, ldx, nb, Y, ldy, yt, ks, nsplit, s);
  if (rb == 2) return launch_palette_mfma_rb<TB, 2>(p, X, ldx, nb, Y, ldy, yt, ks, nsplit, s);
  return launch_palette_mfma_rb<TB, 1>(p, X, ldx, nb, Y, ldy, yt, ks, nsplit, s);
}

extern "C" int uw_palette_gemm(const uw_palette* m, const void* d_X, int64_t batch, int64_t ldx, int xt, void* d_Y,
                               int64_t ldy, int yt, void* stream) {
  if (int rc = check_palette(m, "uw_palette_gemm")) return rc;
  if (xt != UW_BF16) return fail(UW_ERR_UNSUPPORTED, "uw_palette_gemm: X must be bf16 (the matrix cores take bf16)");
  if (yt != UW_F32 && yt != UW_BF16) return fail(UW_ERR_INVALID, "uw_palette_gemm: Y must be UW_F32 or UW_BF16");
  if (batch < 1 || !d_X || !d_Y) return fail(UW_ERR_INVALID, "uw_palette_gemm: batch >= 1 and non-null X, Y");
  if (!aligned_to(d_X, 16) || ldx < m->l.cols || ldx % 8)
    return fail(UW_ERR_INVALID, "uw_palette_gemm: X 16-byte aligned, ldx >= cols and a multiple of 8");
  if (ldy < m->l.rows || !aligned_to(d_Y, yt == UW_F32 ? 4 : 2))
    return fail(UW_ERR_INVALID, "uw_palette_gemm: ldy >= rows and Y aligned to its element");
  const DevPalette p = dev_palette(m);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* X = static_cast<const uint16_t*>(d_X);
  const size_t ysz = yt == UW_F32 ? 4 : 2;
  for (int64_t b0 = 0; b0 < batch; b0 += 16 * kPalMfmaMaxTB) {
    const int nb = int(std::min<int64_t>(batch - b0, 16 * kPalMfmaMaxTB));
    const uint16_t* Xp = X + b0 * ldx;
    void* Yp = static_cast<char*>(d_Y) + size_t(b0) * size_t(ldy) * ysz;
    int rc;
    if (nb <= 16) rc = launch_palette_mfma<1>(p, Xp, ldx, nb, Yp, ldy, yt, s);
    else if (nb <= 32) rc = launch_palette_mfma<2>(p, Xp, ldx, nb, Yp, ldy, yt, s);
    else rc = launch_palette_mfma<4>(p, Xp, ldx, nb, Yp, ldy, yt, s);
    if (rc) return rc;
  }
  return UW_OK;
}

extern "C" int uw_palette_info(const void* blob, size_t n, int64_t* rows, int64_t* cols, int64_t* n_raw) {
  if (!blob || !rows || !cols || !n_raw) return fail(UW_ERR_INVALID, "uw_palette_info: null pointer");
  PaletteLayout l;
  if (int rc = palette_parse(blob, n, &l)) return rc;
  *rows = l.rows;
  *cols = l.cols;
  *n_raw = l.n_raw;
  return UW_OK;
}
