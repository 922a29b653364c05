// Uncompressed bf16 product on the gfx950 matrix cores: the multiply of the
// "full decode" pipeline (decompress to HBM, then a standard matmul; the
// paragraph after the figure of the four execution pipelines in "Unweight:
// how we compressed an LLM 22% without sacrificing quality") and the product
// of plain-mode matrices.
//
// Y[b, n] = sum_k X[b, k] W[n, k]; W [rows, cols] and X [batch, cols] are
// both k-contiguous, so v_mfma_f32_16x16x32_bf16 takes its operands straight
// from global memory with no LDS staging: A = 16 weight rows, B = 16
// activation rows, D[i][j] = Y[b_j][n_i].
//
// k order.  Per k-block of 128 columns, lane (r = lane % 16, q = lane / 16)
// loads 32 consecutive values (64 bytes, four 16-byte loads) of its row at
// k = 128 kb + 32 q, for W and for X alike; k-step s (0..3) hands the lane's
// values 8 s .. 8 s + 7 to the matrix core.  MFMA element (s, q, e) is then
// column 128 kb + 32 q + 8 s + e of both operands: the hardware sees k
// permuted inside each block, identically for A and B, so the sum is the
// same.  Every lane reads 64 contiguous bytes per row and k-block.
//
// A workgroup owns RB blocks of 16 weight rows and TB tiles of 16 batch
// rows; its KS waves split the k-blocks (wave w takes kb = w, w + KS, ...)
// and their partial tiles are summed in LDS at the end.  Workgroups are
// numbered so that the batch tiles of one row group run back to back on one
// XCD (workgroups are dealt to the 8 XCDs round-robin by index): the second
// and later reads of a weight row come from that XCD's L2, not from HBM.
#include <algorithm>

#include "uw_device.h"

namespace uw {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;

__device__ __forceinline__ floatx4 mfma16(const uint4& a, const uint4& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// The lane's 32 values of one row for k-block k0 (zeros past cols; cols is a
// multiple of 8, so each 16-byte piece is wholly inside or outside).
__device__ __forceinline__ void load_row32(const uint16_t* p, int64_t k0, int64_t cols, uint4 (&v)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    v[u] = k0 + 8 * u + 8 <= cols ? *reinterpret_cast<const uint4*>(p + k0 + 8 * u) : uint4{0u, 0u, 0u, 0u};
  }
}

template <int RB, int TB>
struct Frag {
  uint4 w[RB][4];
  uint4 x[TB][4];
};

template <int RB, int TB>
__device__ __forceinline__ void load_frag(const uint16_t* const (&wr)[RB], const uint16_t* const (&xr)[TB], int64_t k0,
                                          int64_t kq, int64_t cols, Frag<RB, TB>& f) {
#pragma unroll
  for (int i = 0; i < RB; ++i) load_row32(wr[i], k0, cols - kq, f.w[i]);
#pragma unroll
  for (int t = 0; t < TB; ++t) load_row32(xr[t], k0, cols - kq, f.x[t]);
}

template <int RB, int TB>
__device__ __forceinline__ void mma_frag(const Frag<RB, TB>& f, floatx4 (&acc)[RB][TB]) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int t = 0; t < TB; ++t) acc[i][t] = mfma16(f.w[i][s], f.x[t][s], acc[i][t]);
}

// Grid: ceil(row groups / 8) * 8 * ny workgroups of KS waves (row group =
// 16 RB weight rows, ny = batch tiles of 16 TB rows).  PIPE: the next
// k-block's loads are issued before the current one is multiplied.
template <int RB, int TB, bool YBF16, bool PIPE>
__global__ __launch_bounds__(512) void bf16_mfma_kernel(const uint16_t* __restrict__ W, int64_t rows, int64_t cols,
                                                        int64_t ldw, const uint16_t* __restrict__ X, int64_t ldx,
                                                        int64_t batch, void* __restrict__ Y, int64_t ldy, int n_groups,
                                                        int ny) {
  extern __shared__ uint32_t lds[];
  const int L = blockIdx.x;
  const int grp = (L / (kXcds * ny)) * kXcds + L % kXcds;
  const int y = (L / kXcds) % ny;
  if (grp >= n_groups) return;
  const int lane = threadIdx.x % kWave, wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int ks = blockDim.x / kWave;
  const int r = lane % 16, q = lane / 16;
  const int64_t row0 = int64_t(grp) * 16 * RB, b0 = int64_t(y) * 16 * TB;
  const int64_t kq = 32 * q;
  const uint16_t* wr[RB];
  const uint16_t* xr[TB];
#pragma unroll
  for (int i = 0; i < RB; ++i) wr[i] = W + std::min<int64_t>(row0 + 16 * i + r, rows - 1) * ldw + kq;
#pragma unroll
  for (int t = 0; t < TB; ++t) xr[t] = X + std::min<int64_t>(b0 + 16 * t + r, batch - 1) * ldx + kq;
  floatx4 acc[RB][TB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int64_t nkb = (cols + 127) / 128;
  if constexpr (PIPE) {
    Frag<RB, TB> fa, fb;
    int64_t kb = wave;
    if (kb < nkb) load_frag<RB, TB>(wr, xr, 128 * kb, kq, cols, fa);
    for (; kb < nkb; kb += 2 * ks) {
      if (kb + ks < nkb) load_frag<RB, TB>(wr, xr, 128 * (kb + ks), kq, cols, fb);
      mma_frag<RB, TB>(fa, acc);
      if (kb + ks >= nkb) break;
      if (kb + 2 * ks < nkb) load_frag<RB, TB>(wr, xr, 128 * (kb + 2 * ks), kq, cols, fa);
      mma_frag<RB, TB>(fb, acc);
    }
  } else {
    for (int64_t kb = wave; kb < nkb; kb += ks) {
      Frag<RB, TB> f;
      load_frag<RB, TB>(wr, xr, 128 * kb, kq, cols, f);
      mma_frag<RB, TB>(f, acc);
    }
  }
  // partial tiles of the KS waves meet in LDS: tile (i, t) of wave w at
  // ((w * RB + i) * TB + t) * 1 KB, lane-major 16 bytes per lane
  if (ks > 1) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        const floatx4 v = acc[i][t];
        st128(uint32_t(((wave * RB + i) * TB + t) * 1024 + lane * 16),
              uint4{f32_bits(v.x), f32_bits(v.y), f32_bits(v.z), f32_bits(v.w)});
      }
    lds_barrier();
  }
  // wave w stores the tiles with (i * TB + t) % KS == w; lane (r, q) holds
  // rows 4 q .. 4 q + 3 of the tile for batch row r
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      if ((i * TB + t) % ks != wave) continue;
      floatx4 v = acc[i][t];
      if (ks > 1) {
        v = floatx4{0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < ks; ++w) {
          const uint4 p = ld128(uint32_t(((w * RB + i) * TB + t) * 1024 + lane * 16));
          v += floatx4{bits_f32(p.x), bits_f32(p.y), bits_f32(p.z), bits_f32(p.w)};
        }
      }
      const int64_t b = b0 + 16 * t + r;
      const int64_t n = row0 + 16 * i + 4 * q;
      if (b >= batch) continue;
      const float vals[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (n + e < rows) {
          if (YBF16) static_cast<uint16_t*>(Y)[b * ldy + n + e] = f32_to_bf16(vals[e]);
          else static_cast<float*>(Y)[b * ldy + n + e] = vals[e];
        }
      }
    }
}

// The large-batch form: the activations of a k-block (16 TB rows x 128
// columns) are staged once in LDS and shared by the workgroup's 4 waves,
// each of which streams its own 16 RB weight rows straight into registers.
// Two LDS buffers alternate: while the matrix cores work on block kb, the
// loads of block kb + 1 (activations and weights) are in flight; one barrier
// per block.  A staged row is 256 bytes plus 16 of padding, so the 16 rows a
// B-operand read touches start on different banks.
constexpr int kXRowBytes = 256 + 16;

template <int RB, int TB, bool YBF16>
__global__ __launch_bounds__(256) void bf16_mfma_xlds_kernel(const uint16_t* __restrict__ W, int64_t rows, int64_t cols,
                                                             int64_t ldw, const uint16_t* __restrict__ X, int64_t ldx,
                                                             int64_t batch, void* __restrict__ Y, int64_t ldy,
                                                             int n_groups, int ny) {
  constexpr int kTileBytes = 16 * TB * kXRowBytes;
  extern __shared__ uint32_t lds[];
  const int L = blockIdx.x;
  const int grp = (L / (kXcds * ny)) * kXcds + L % kXcds;
  const int y = (L / kXcds) % ny;
  if (grp >= n_groups) return;
  const int tid = threadIdx.x, lane = tid % kWave, wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int r = lane % 16, q = lane / 16;
  const int64_t row0 = int64_t(grp) * 64 * RB + int64_t(wave) * 16 * RB, b0 = int64_t(y) * 16 * TB;
  const int64_t kq = 32 * q;
  const uint16_t* wr[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) wr[i] = W + std::min<int64_t>(row0 + 16 * i + r, rows - 1) * ldw + kq;
  // staging: thread t moves 16 bytes (8 columns) of TB activation rows per block
  const int srow = tid / 16, schunk = tid % 16;
  const uint16_t* xs[TB];
#pragma unroll
  for (int u = 0; u < TB; ++u) xs[u] = X + std::min<int64_t>(b0 + 16 * u + srow, batch - 1) * ldx + 8 * schunk;
  auto stage_load = [&](int64_t kb, uint4 (&v)[TB]) {
    const int64_t k = 128 * kb + 8 * schunk;
#pragma unroll
    for (int u = 0; u < TB; ++u) v[u] = k + 8 <= cols ? *reinterpret_cast<const uint4*>(xs[u] + 128 * kb) : uint4{0u, 0u, 0u, 0u};
  };
  auto stage_store = [&](int buf, const uint4 (&v)[TB]) {
#pragma unroll
    for (int u = 0; u < TB; ++u) st128(uint32_t(buf * kTileBytes + (16 * u + srow) * kXRowBytes + 16 * schunk), v[u]);
  };
  floatx4 acc[RB][TB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int64_t nkb = (cols + 127) / 128;
  uint4 xv[TB];
  uint4 wc[RB][4], wn[RB][4];
  stage_load(0, xv);
#pragma unroll
  for (int i = 0; i < RB; ++i) load_row32(wr[i], 0, cols - kq, wc[i]);
  stage_store(0, xv);
  lds_barrier();
  // B operand of tile t, k-step s: row 16 t + r of the staged block, bytes 64 q + 16 s
  const uint32_t bq = uint32_t(r * kXRowBytes + 64 * q);
  for (int64_t kb = 0; kb < nkb; ++kb) {
    const int buf = int(kb & 1);
    const bool more = kb + 1 < nkb;
    if (more) {
      stage_load(kb + 1, xv);
#pragma unroll
      for (int i = 0; i < RB; ++i) load_row32(wr[i], 128 * (kb + 1), cols - kq, wn[i]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 xb[TB];
#pragma unroll
      for (int t = 0; t < TB; ++t) xb[t] = ld128(uint32_t(buf * kTileBytes + t * 16 * kXRowBytes) + bq + 16 * s);
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int t = 0; t < TB; ++t) acc[i][t] = mfma16(wc[i][s], xb[t], acc[i][t]);
    }
    if (more) {
      stage_store(buf ^ 1, xv);
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int u = 0; u < 4; ++u) wc[i][u] = wn[i][u];
    }
    lds_barrier();
  }
  // lane (r, q) holds rows 4 q .. 4 q + 3 of tile (i, t) for batch row r
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int64_t b = b0 + 16 * t + r;
      const int64_t n = row0 + 16 * i + 4 * q;
      if (b >= batch) continue;
      const float vals[4] = {acc[i][t].x, acc[i][t].y, acc[i][t].z, acc[i][t].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (n + e < rows) {
          if (YBF16) static_cast<uint16_t*>(Y)[b * ldy + n + e] = f32_to_bf16(vals[e]);
          else static_cast<float*>(Y)[b * ldy + n + e] = vals[e];
        }
      }
    }
}

template <int RB, int TB>
int run_xlds_gemm(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw, const uint16_t* X, int64_t batch,
                  int64_t ldx, void* Y, int64_t ldy, int yt, void* stream) {
  const int n_groups = int((rows + 64 * RB - 1) / (64 * RB));
  const int ny = int((batch + 16 * TB - 1) / (16 * TB));
  const int64_t grid = int64_t((n_groups + kXcds - 1) / kXcds) * kXcds * ny;
  const size_t lds = size_t(2) * 16 * TB * kXRowBytes;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto kern = yt == UW_BF16 ? bf16_mfma_xlds_kernel<RB, TB, true> : bf16_mfma_xlds_kernel<RB, TB, false>;
  allow_full_lds(kern);
  hipLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(256), lds, s, W, rows, cols, ldw, X, ldx, batch, Y, ldy, n_groups,
                     ny);
  return hip_check(hipGetLastError(), "bf16_mfma_xlds_kernel launch");
}

// The large-batch form with a deeper pipeline: both operands of a k-block go
// straight from global memory into LDS (buffer_load ... lds, no registers),
// into a ring of NS stages, so NS - 1 k-blocks are in flight while the
// matrix cores work on the oldest.  A workgroup of 4 waves holds 64 weight
// rows (16 per wave) and 16 TB batch rows; per k-block each wave moves its 16
// weight rows (4 KB, 4 loads) and a quarter of the activation tile (TB
// loads).  A 16-byte chunk c of staged row r sits at chunk c ^ (r % 16) of
// its 256-byte row, so the 16 rows an operand read touches hit 16 different
// bank groups.  Needs cols to be a multiple of 128 (no partial k-block to
// zero).  With nsplit = 2 the grid holds two workgroups per tile, each taking
// half of the k-blocks, and both add their partial sums into an fp32 Y that
// was zeroed first: 0 + a + b and 0 + b + a are the same float, so the
// result does not depend on their order.
constexpr int kStages = 3;

// 16 bytes per lane from the buffer resource at byte voff into LDS at m0 +
// 16 * lane (all lanes active).
__device__ __forceinline__ void stage_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t m0) {
  asm volatile(
      "s_nop 4\n"
      "s_mov_b32 m0, %[m]\n"
      "s_nop 0\n"
      "buffer_load_dwordx4 %[v], %[r], 0 offen lds"
      :
      : [m] "s"(m0), [v] "v"(voff), [r] "s"(r)
      : "memory", "m0");
}

__device__ inline __amdgpu_buffer_rsrc_t gemm_rsrc(const void* base, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), int16_t(0),
                                           int(bytes > 0x7FFFFFFFull ? 0x7FFFFFFFull : bytes), 0x00020000);
}

template <int RB, int TB, bool YBF16>
__global__ __launch_bounds__(256) void bf16_mfma_stage_kernel(const uint16_t* __restrict__ W, int64_t rows, int64_t cols,
                                                              int64_t ldw, const uint16_t* __restrict__ X, int64_t ldx,
                                                              int64_t batch, void* __restrict__ Y, int64_t ldy,
                                                              int n_groups, int ny, int nsplit) {
  constexpr uint32_t kW = uint32_t(RB) * 64 * 256;  // weight part of a stage: 64 RB rows x 256 B
  constexpr uint32_t kX = uint32_t(TB) * 16 * 256;  // activation part: 16 TB rows x 256 B
  constexpr uint32_t kStage = kW + kX;
  const int per_split = int(gridDim.x) / nsplit;
  const int split = int(blockIdx.x) / per_split;
  const int L = int(blockIdx.x) % per_split;
  const int grp = (L / (kXcds * ny)) * kXcds + L % kXcds;
  const int y = (L / kXcds) % ny;
  if (grp >= n_groups) return;
  const int tid = threadIdx.x, lane = tid % kWave, wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int r = lane % 16, q = lane / 16;
  const int64_t row0 = int64_t(grp) * 64 * RB + int64_t(wave) * 16 * RB, b0 = int64_t(y) * 16 * TB;
  const __amdgpu_buffer_rsrc_t rw = gemm_rsrc(W, uint64_t(rows - 1) * uint64_t(ldw) * 2 + uint64_t(cols) * 2);
  const __amdgpu_buffer_rsrc_t rx = gemm_rsrc(X, uint64_t(batch - 1) * uint64_t(ldx) * 2 + uint64_t(cols) * 2);
  // the lane's part of a load: 4 staged rows of 256 B per load, lane l puts
  // 16 bytes at 16 l, i.e. row 4 g + l / 16, stored chunk l % 16, which holds
  // source chunk (l % 16) ^ (row % 16)
  const int lrow = lane / 16, lchunk = lane % 16;
  uint32_t wvo[4 * RB], xvo[TB];  // byte offsets at k = 0
#pragma unroll
  for (int g = 0; g < 4 * RB; ++g) {
    const int srow = 4 * g + lrow;  // this wave's rows 16 RB w .. 16 RB (w + 1) - 1
    const int64_t n = std::min<int64_t>(row0 + srow, rows - 1);
    wvo[g] = uint32_t((n * ldw + 8 * (lchunk ^ (srow % 16))) * 2);
  }
#pragma unroll
  for (int u = 0; u < TB; ++u) {
    const int srow = 4 * (u * 4 + wave) + lrow;  // staged activation row
    const int64_t b = std::min<int64_t>(b0 + srow, batch - 1);
    xvo[u] = uint32_t((b * ldx + 8 * (lchunk ^ (srow % 16))) * 2);
  }
  const uint32_t wdst = uint32_t(wave) * 16 * RB * 256;  // this wave's weight rows in a stage
  // this workgroup's k-blocks [kb0, kb0 + nkb)
  const int64_t nkb_all = cols / 128, half = (nkb_all + nsplit - 1) / nsplit;
  const int64_t kb0 = split * half, nkb = std::max<int64_t>(0, std::min(nkb_all, kb0 + half) - kb0);
  auto issue = [&](int64_t kb, int st) {
    const uint32_t kbytes = uint32_t(kb0 + kb) * 256;
    const uint32_t base = uint32_t(st) * kStage;
#pragma unroll
    for (int g = 0; g < 4 * RB; ++g) stage_load(rw, wvo[g] + kbytes, base + wdst + uint32_t(g) * 1024);
#pragma unroll
    for (int u = 0; u < TB; ++u) stage_load(rx, xvo[u] + kbytes, base + kW + uint32_t(u * 4 + wave) * 1024);
  };
  floatx4 acc[RB][TB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[i][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  // operand reads: row r of weight block i / of activation tile t, source
  // chunk 4 q + s at stored chunk (4 q + s) ^ r
  const uint32_t arow = wdst + uint32_t(r) * 256, xrow = kW + uint32_t(r) * 256;
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (i < nkb) issue(i, i);
  for (int64_t kb = 0; kb < nkb; ++kb) {
    const int st = int(kb % kStages);
    // this wave's loads of block kb have landed once only the younger
    // blocks' (up to kStages - 2 of them, 4 RB + TB loads each) may be pending
    if (kb + kStages - 2 < nkb) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kStages - 2) * (4 * RB + TB)) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();  // every wave's loads of block kb have landed; block kb - 1 is no longer read
    if (kb + kStages - 1 < nkb) issue(kb + kStages - 1, int((kb + kStages - 1) % kStages));
    const uint32_t base = uint32_t(st) * kStage;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t ch = uint32_t(((4 * q + s) ^ r) * 16);
      uint4 a[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) a[i] = ld128(base + arow + uint32_t(i) * 16 * 256 + ch);
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        const uint4 b = ld128(base + xrow + uint32_t(t) * 16 * 256 + ch);
#pragma unroll
        for (int i = 0; i < RB; ++i) acc[i][t] = mfma16(a[i], b, acc[i][t]);
      }
    }
  }
  // lane (r, q) holds rows 4 q .. 4 q + 3 of weight block i for batch row r of tile t
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int64_t b = b0 + 16 * t + r;
      const int64_t n = row0 + 16 * i + 4 * q;
      if (b >= batch) continue;
      const float vals[4] = {acc[i][t].x, acc[i][t].y, acc[i][t].z, acc[i][t].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (n + e < rows) {
          if (YBF16) static_cast<uint16_t*>(Y)[b * ldy + n + e] = f32_to_bf16(vals[e]);
          else if (nsplit > 1) unsafeAtomicAdd(static_cast<float*>(Y) + b * ldy + n + e, vals[e]);
          else static_cast<float*>(Y)[b * ldy + n + e] = vals[e];
        }
      }
    }
}

// Y[b][n] = 0 for b < batch, n < rows (fp32), ahead of a split product.
// Y[b][0 .. rows) = 0 for batch row b = blockIdx.y; 16-byte stores when every
// row starts 16-byte aligned (VEC), else 4-byte ones.
template <bool VEC>
__global__ void zero_rows_kernel(float* __restrict__ Y, int64_t rows, int64_t ldy) {
  float* y = Y + int64_t(blockIdx.y) * ldy;
  const int64_t i = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (VEC && i + 4 <= rows) {
    *reinterpret_cast<float4*>(y + i) = float4{0.f, 0.f, 0.f, 0.f};
  } else {
    for (int64_t j = i; j < std::min<int64_t>(i + 4, rows); ++j) y[j] = 0.f;
  }
}

template <int RB, int TB>
int run_stage_gemm(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw, const uint16_t* X, int64_t batch,
                   int64_t ldx, void* Y, int64_t ldy, int yt, void* stream, int nsplit = 1) {
  const int n_groups = int((rows + 64 * RB - 1) / (64 * RB));
  const int ny = int((batch + 16 * TB - 1) / (16 * TB));
  if (yt != UW_F32 || cols / 128 < 2 * kStages) nsplit = 1;  // the split adds fp32 partial sums in place
  if (nsplit > 1) {
    const dim3 zgrid(unsigned((rows + 1023) / 1024), unsigned(batch));
    if (reinterpret_cast<uintptr_t>(Y) % 16 == 0 && ldy % 4 == 0)
      hipLaunchKernelGGL(zero_rows_kernel<true>, zgrid, dim3(256), 0, static_cast<hipStream_t>(stream),
                         static_cast<float*>(Y), rows, ldy);
    else
      hipLaunchKernelGGL(zero_rows_kernel<false>, zgrid, dim3(256), 0, static_cast<hipStream_t>(stream),
                         static_cast<float*>(Y), rows, ldy);
    if (int rc = hip_check(hipGetLastError(), "zero_rows_kernel launch")) return rc;
  }
  const int64_t grid = int64_t((n_groups + kXcds - 1) / kXcds) * kXcds * ny * nsplit;
  const size_t lds = size_t(kStages) * (size_t(RB) * 64 * 256 + size_t(TB) * 16 * 256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto kern = yt == UW_BF16 ? bf16_mfma_stage_kernel<RB, TB, true> : bf16_mfma_stage_kernel<RB, TB, false>;
  allow_full_lds(kern);
  hipLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(256), lds, s, W, rows, cols, ldw, X, ldx, batch, Y, ldy, n_groups,
                     ny, nsplit);
  return hip_check(hipGetLastError(), "bf16_mfma_stage_kernel launch");
}

template <int RB, int TB, bool PIPE>
int run_mfma_gemm(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw, const uint16_t* X, int64_t batch,
                  int64_t ldx, void* Y, int64_t ldy, int yt, int ks, void* stream) {
  const int n_groups = int((rows + 16 * RB - 1) / (16 * RB));
  const int ny = int((batch + 16 * TB - 1) / (16 * TB));
  const int64_t grid = int64_t((n_groups + kXcds - 1) / kXcds) * kXcds * ny;
  const size_t lds = ks > 1 ? size_t(ks) * RB * TB * 1024 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto kern = yt == UW_BF16 ? bf16_mfma_kernel<RB, TB, true, PIPE> : bf16_mfma_kernel<RB, TB, false, PIPE>;
  allow_full_lds(kern);
  hipLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(ks * kWave), lds, s, W, rows, cols, ldw, X, ldx, batch, Y, ldy,
                     n_groups, ny);
  return hip_check(hipGetLastError(), "bf16_mfma_kernel launch");
}

}  // namespace

// Shapes of the matrix-core product (a tuning knob: uw_bf16_gemm_config).
// id: 0 = chosen by the heuristic below; else one of the listed shapes.
// Shapes 1..9: operands straight from global memory, RB x 16 weight rows and
// TB x 16 batch rows per workgroup of KS waves splitting k.  Shapes 10..13:
// the activations staged in LDS, 4 waves of RB x 16 weight rows each (ks
// does not apply).  Shapes 14..16: both operands staged through a ring of
// LDS stages by direct loads (cols a multiple of 128 and each operand under
// 2 GiB; else the LDS-activation kernel of the same tile runs).  Shapes 17,
// 18: the staged kernel with 64 x 64 and 64 x 32 tiles and two workgroups per
// tile, each taking half of K and adding into Y (fp32 Y; with bf16 Y, or
// under 6 k-blocks, one workgroup per tile).
struct MfmaShape {
  int rb, tb, pipe, xlds;
};
constexpr MfmaShape kMfmaShapes[] = {
    {0, 0, 0, 0},  // heuristic
    {1, 1, 1, 0}, {2, 1, 1, 0}, {1, 2, 1, 0}, {2, 2, 1, 0}, {1, 4, 1, 0}, {2, 4, 0, 0}, {4, 4, 0, 0}, {4, 2, 0, 0},
    {2, 4, 1, 0}, {1, 4, 1, 1}, {2, 4, 1, 1}, {2, 2, 1, 1}, {1, 8, 1, 1},
    {1, 8, 1, 2}, {1, 4, 1, 2}, {2, 4, 1, 2},  // 14..16: both operands staged in LDS, kStages deep (cols % 128 == 0)
    {1, 4, 1, 3}, {1, 2, 1, 3},                // 17, 18: staged, two workgroups per tile splitting K (fp32 Y)
};
constexpr int kMfmaShapeCount = int(sizeof(kMfmaShapes) / sizeof(kMfmaShapes[0]));

int mfma_gemm_shape_count() { return kMfmaShapeCount; }

// The LDS-stage kernel addresses W and X with 32-bit buffer offsets and
// loads whole 128-column blocks.
static bool stage_ok(int64_t rows, int64_t cols, int64_t ldw, int64_t batch, int64_t ldx) {
  const uint64_t lim = uint64_t(1) << 31;
  return cols % 128 == 0 && uint64_t(rows) * uint64_t(ldw) * 2 < lim && uint64_t(batch) * uint64_t(ldx) * 2 < lim;
}

// The waves of a launch and the k-blocks each wave takes: KS (waves per
// workgroup, 1..8) is the smallest that gives about 4096 waves, while every
// wave keeps at least 2 k-blocks.
static int pick_ks(int64_t rows, int64_t cols, int64_t batch, int rb, int tb) {
  const int64_t groups = (rows + 16 * rb - 1) / (16 * rb);
  const int64_t ny = (batch + 16 * tb - 1) / (16 * tb);
  const int64_t nkb = (cols + 127) / 128;
  int ks = 1;
  while (ks < 8 && groups * ny * ks < 4096 && nkb / (2 * ks) >= 2) ks *= 2;
  return ks;
}

int launch_mfma_gemm(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw, const uint16_t* X, int64_t batch,
                     int64_t ldx, void* Y, int64_t ldy, int yt, int shape, int ks, void* stream) {
  if (shape <= 0 || shape >= kMfmaShapeCount) {
    // heuristic, from a sweep of every shape and ks on the MLP shapes and
    // 8192^2 (8 rotated copies of W).  9..64 batch rows: with at least 192
    // workgroups of 64 x 64, both operands staged in LDS (gate); with fewer
    // and more than 16 batch rows with fp32 Y, the staged kernel with two
    // workgroups per tile splitting K (down_proj 4096 x 14336 at 32 / 64 rows:
    // 38 / 42 us against 61 / 59; 8192^2: 38 / 45 against 52 / 53); else the
    // staged kernel from 128 workgroups, below that operands straight from
    // global memory with 4 waves splitting k.  Above 64 rows: 128 x 64 staged
    // tiles when that gives 192 workgroups.  Up to 8 batch rows (one tile of
    // 16, partly padding): 32 weight rows per workgroup and 2 waves splitting
    // k where that gives 384 workgroups (gate), else 16 rows and 4 or 8 waves
    // (down)
    const int64_t tiles64 = (batch + 63) / 64;
    const bool stage = stage_ok(rows, cols, ldw, batch, ldx);
    const int64_t g64 = (rows + 63) / 64 * tiles64;  // workgroups of 64 x 64 tiles
    if (batch > 8 && batch <= 64 && stage && g64 >= 192) {
      shape = 15;
    } else if (batch > 16 && batch <= 64 && stage && yt == UW_F32 && cols / 128 >= 6) {
      // few weight rows (down_proj, 8192^2): two workgroups per tile split K
      shape = g64 >= 96 && batch <= 32 ? 17 : 18;
    } else if (batch > 8 && batch <= 64 && stage && g64 >= 128) {
      shape = 15;
    } else if (batch > 64 && cols <= 4096 && rows >= 12288 && (batch > 128 || rows >= 24576)) {
      // tall matrices with short rows: 64 x 128 tiles with the activations in
      // LDS (14336 x 4096 at 256 rows: 75 us against 89; 28672 x 4096 at
      // 96-256 rows: 80-146 against 90-174)
      shape = 13;
    } else if (batch > 64 && stage) {
      shape = (rows + 127) / 128 * tiles64 >= 192 ? 16 : 15;
    } else if (batch <= 8 && (rows + 31) / 32 >= 384) {
      shape = 2;  // 32 weight rows per workgroup, one batch tile (gate at batch 1..8)
      if (ks <= 0) ks = 2;
    } else if (batch <= 16) {
      shape = 1;
      if (ks <= 0) ks = batch <= 2 ? 8 : 4;
    } else if (batch <= 64) {
      shape = 4;
      if (ks <= 0) ks = 4;
    } else {
      shape = 13;
    }
    // keep at least 2 k-blocks per wave
    const int64_t nkb = (cols + 127) / 128;
    while (ks > 1 && nkb / ks < 2) ks /= 2;
  }
  const MfmaShape sh = kMfmaShapes[shape];
  if (ks <= 0 && !sh.xlds) ks = pick_ks(rows, cols, batch, sh.rb, sh.tb);
  switch (shape) {
    case 1: return run_mfma_gemm<1, 1, true>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, ks, stream);
    case 2: return run_mfma_gemm<2, 1, true>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, ks, stream);
    case 3: return run_mfma_gemm<1, 2, true>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, ks, stream);
    case 4: return run_mfma_gemm<2, 2, true>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, ks, stream);
    case 5: return run_mfma_gemm<1, 4, true>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, ks, stream);
    case 6: return run_mfma_gemm<2, 4, false>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, ks, stream);
    case 7: return run_mfma_gemm<4, 4, false>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, ks, stream);
    case 8: return run_mfma_gemm<4, 2, false>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, ks, stream);
    case 9: return run_mfma_gemm<2, 4, true>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, ks, stream);
    case 10: return run_xlds_gemm<1, 4>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, stream);
    case 11: return run_xlds_gemm<2, 4>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, stream);
    case 12: return run_xlds_gemm<2, 2>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, stream);
    case 14:
      if (stage_ok(rows, cols, ldw, batch, ldx)) return run_stage_gemm<1, 8>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, stream);
      return run_xlds_gemm<1, 8>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, stream);
    case 15:
      if (stage_ok(rows, cols, ldw, batch, ldx)) return run_stage_gemm<1, 4>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, stream);
      return run_xlds_gemm<1, 4>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, stream);
    case 16:
      if (stage_ok(rows, cols, ldw, batch, ldx)) return run_stage_gemm<2, 4>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, stream);
      return run_xlds_gemm<2, 4>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, stream);
    case 17:
      if (stage_ok(rows, cols, ldw, batch, ldx))
        return run_stage_gemm<1, 4>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, stream, 2);
      return run_xlds_gemm<1, 4>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, stream);
    case 18:
      if (stage_ok(rows, cols, ldw, batch, ldx))
        return run_stage_gemm<1, 2>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, stream, 2);
      return run_xlds_gemm<2, 2>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, stream);
    default: return run_xlds_gemm<1, 8>(W, rows, cols, ldw, X, batch, ldx, Y, ldy, yt, stream);
  }
}

}  // namespace uw
