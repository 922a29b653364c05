// Exponent-only pipeline on gfx950: decode only the exponent bytes of a
// Huffman-form matrix into HBM (1 byte per weight instead of 2), then a
// reconstructive product on the matrix cores that merges them with the
// blob's own sign+mantissa bytes.
//
// "Unweight: how we compressed an LLM 22% without sacrificing quality",
// section on the four execution pipelines: one of the two middle paths
// decodes only the exponent bytes (half the preprocessing traffic) and feeds
// a reconstructive matmul that rebuilds bf16 on chip.
//
// Layout: the exponent plane uses the order of the blob's sign+mantissa
// section (flat walk: tile T = weights 1024 T .. of the row-major matrix;
// byte q of the tile is weight column 64 (q % 16) + q / 16 of the tile), so
// both planes are read with the same contiguous loads.  The activations are
// permuted into that order once per call (a small pass over X), after which
// lane (r = lane % 16, j = lane / 16) of a wave reads 32 consecutive bytes
// of each plane and 64 consecutive bytes of X' per 128-position block, and
// k-step s gives it positions 8s..8s+7 of its 32 as the A and B operands of
// v_mfma_f32_16x16x32_bf16: the same permuted k order on both sides.
#include <algorithm>

#include "uw_device.h"

namespace uw {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
constexpr int kExpMaxTB = 4;  // 64 batch rows per pass

// X'[b][1024 t + q] = X[b][1024 t + 64 (q % 16) + q / 16]
__global__ __launch_bounds__(256) void permute_x_kernel(const uint16_t* __restrict__ X, int64_t ldx, int64_t batch,
                                                        int64_t cols, uint16_t* __restrict__ Xp) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= batch * cols) return;
  const int64_t b = i / cols, c = i - b * cols;
  const int64_t t = c >> 10, q = c & 1023;
  Xp[i] = X[b * ldx + (t << 10) + 64 * (q & 15) + (q >> 4)];
}

__device__ inline uint32_t word_of(const uint4& v, int k) { return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w; }

// Positions 8s..8s+7 of the lane's 32 as 8 bf16: sign and mantissa from the
// sm bytes, exponent from the exponent bytes.
__device__ inline uint4 merge_step(const uint4 (&sm)[2], const uint4 (&ex)[2], int s) {
  uint32_t W[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int wi = 2 * (s & 1) + (p >> 1);
    const uint32_t E = __builtin_amdgcn_perm(0u, word_of(ex[s >> 1], wi), (p & 1) ? 0x0c030c02u : 0x0c010c00u) << 7;
    const uint32_t S = __builtin_amdgcn_perm(0u, word_of(sm[s >> 1], wi), (p & 1) ? 0x03030202u : 0x01010000u);
    W[p] = (S & 0x807F807Fu) | (E & 0x7F807F80u);
  }
  return uint4{W[0], W[1], W[2], W[3]};
}

// A workgroup of KS waves owns RB blocks of 16 rows; wave w takes every
// KS-th 128-position block; the partial sums meet in LDS.
template <int TB, int RB, bool YBF16>
__global__ __launch_bounds__(512) void exponent_mfma_kernel(const uint8_t* __restrict__ sm, const uint8_t* __restrict__ ex,
                                                            int64_t rows, int64_t cols, const uint16_t* __restrict__ Xp,
                                                            int nb, void* __restrict__ Y, int64_t ldy) {
  extern __shared__ float4 red[];  // [waves][TB][64]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, ks = blockDim.x >> 6;
  const int r = lane & 15, j = lane >> 4;
  const int64_t base = int64_t(blockIdx.x) * 16 * RB;
  int64_t row[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) row[i] = std::min<int64_t>(rows - 1, base + 16 * i + r);  // past the end: never stored
  const uint16_t* xr[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) xr[tb] = Xp + int64_t(std::min(16 * tb + r, nb - 1)) * cols + 32 * j;
  floatx4 acc[RB][TB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[i][tb] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int64_t n_blocks = cols / 128;
  for (int64_t kb = wave; kb < n_blocks; kb += ks) {
    uint4 xv[TB][4];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const uint4* xs = reinterpret_cast<const uint4*>(xr[tb] + kb * 128);
#pragma unroll
      for (int s = 0; s < 4; ++s) xv[tb][s] = xs[s];
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int64_t off = row[i] * cols + kb * 128 + 32 * j;  // same offset in both planes
      const uint4* ps = reinterpret_cast<const uint4*>(sm + off);
      const uint4* pe = reinterpret_cast<const uint4*>(ex + off);
      const uint4 smv[2] = {ps[0], ps[1]}, exv[2] = {pe[0], pe[1]};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 a = merge_step(smv, exv, s);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
          acc[i][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                               __builtin_bit_cast(bf16x8_t, xv[tb][s]), acc[i][tb], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    if (i) __syncthreads();
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
      if (n < rows && b < nb) {
        if (YBF16) static_cast<uint16_t*>(Y)[b * ldy + n] = f32_to_bf16(sum);
        else static_cast<float*>(Y)[b * ldy + n] = sum;
      }
    }
  }
}

// The largest RB in {4, 2, 1} leaving about 1792 waves, then the fewest KS
// (at most 8) reaching it.
void exponent_shape(int64_t rows, int* rb, int* ks) {
  const int64_t blocks16 = (rows + 15) / 16;
  *rb = 1;
  for (int c : {4, 2})
    if ((blocks16 + c - 1) / c * 8 >= 1792) {
      *rb = c;
      break;
    }
  const int64_t wgs = (blocks16 + *rb - 1) / *rb;
  *ks = 1;
  while (*ks < 8 && wgs * *ks < 1792) *ks *= 2;
}

template <int TB, int RB>
int launch_exp_rb(const uint8_t* sm, const uint8_t* ex, int64_t rows, int64_t cols, const uint16_t* Xp, int nb, void* Y,
                  int64_t ldy, int yt, int ks, hipStream_t s) {
  const size_t lds = size_t(ks) * TB * 64 * sizeof(float4);
  const dim3 grid(unsigned((rows + 16 * RB - 1) / (16 * RB))), block(64 * ks);
  if (yt == UW_BF16)
    hipLaunchKernelGGL((exponent_mfma_kernel<TB, RB, true>), grid, block, lds, s, sm, ex, rows, cols, Xp, nb, Y, ldy);
  else
    hipLaunchKernelGGL((exponent_mfma_kernel<TB, RB, false>), grid, block, lds, s, sm, ex, rows, cols, Xp, nb, Y, ldy);
  return hip_check(hipGetLastError(), "exponent_mfma_kernel launch");
}

template <int TB>
int launch_exp(const uint8_t* sm, const uint8_t* ex, int64_t rows, int64_t cols, const uint16_t* Xp, int nb, void* Y,
               int64_t ldy, int yt, hipStream_t s) {
  int rb, ks;
  exponent_shape(rows, &rb, &ks);
  if (rb == 4) return launch_exp_rb<TB, 4>(sm, ex, rows, cols, Xp, nb, Y, ldy, yt, ks, s);
  if (rb == 2) return launch_exp_rb<TB, 2>(sm, ex, rows, cols, Xp, nb, Y, ldy, yt, ks, s);
  return launch_exp_rb<TB, 1>(sm, ex, rows, cols, Xp, nb, Y, ldy, yt, ks, s);
}

bool aligned_to_elem(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

size_t exp_plane_bytes(const uw_matrix* m) { return (size_t(m->h.rows) * size_t(m->h.cols) + 255) / 256 * 256; }

}  // namespace
}  // namespace uw

using namespace uw;

extern "C" size_t uw_exponent_ws_size(const uw_matrix* m, int64_t batch) {
  if (!m || batch < 1) return 0;
  const int64_t per_pass = std::min<int64_t>(batch, 16 * kExpMaxTB);
  return exp_plane_bytes(m) + size_t(per_pass) * size_t(m->h.cols) * 2;
}

extern "C" int uw_exponent_gemm(const uw_matrix* m, const void* d_X, int64_t batch, int64_t ldx, int xt, void* d_Y,
                                int64_t ldy, int yt, void* d_ws, size_t ws_bytes, void* stream) {
  if (!m) return fail(UW_ERR_INVALID, "uw_exponent_gemm: null handle");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != m->device)
    return fail(UW_ERR_INVALID, "uw_exponent_gemm: the handle's device is not current");
  if (m->h.plain() || !m->dev.flat)
    return fail(UW_ERR_UNSUPPORTED, "uw_exponent_gemm: needs a coded blob whose tiles never cross a row "
                                    "(G and cols/64 multiples of 16)");
  if (xt != UW_BF16) return fail(UW_ERR_UNSUPPORTED, "uw_exponent_gemm: X must be bf16");
  if (yt != UW_F32 && yt != UW_BF16) return fail(UW_ERR_INVALID, "uw_exponent_gemm: Y must be UW_F32 or UW_BF16");
  if (batch < 1 || !d_X || !d_Y || !d_ws) return fail(UW_ERR_INVALID, "uw_exponent_gemm: batch >= 1, non-null X, Y, ws");
  if (ldx < m->h.cols || ldy < m->h.rows || !aligned_to_elem(d_Y, yt == UW_F32 ? 4 : 2) || !aligned_to_elem(d_X, 2))
    return fail(UW_ERR_INVALID, "uw_exponent_gemm: ldx >= cols, ldy >= rows, X and Y aligned to their element");
  if (!aligned_to_elem(d_ws, 256) || ws_bytes < uw_exponent_ws_size(m, batch))
    return fail(UW_ERR_INVALID, "uw_exponent_gemm: workspace 256-byte aligned of uw_exponent_ws_size bytes");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t rows = m->h.rows, cols = m->h.cols;
  uint8_t* ex = static_cast<uint8_t*>(d_ws);
  uint16_t* Xp = reinterpret_cast<uint16_t*>(ex + exp_plane_bytes(m));
  if (int rc = launch_decode_exponents(m, ex, stream)) return rc;
  const uint16_t* X = static_cast<const uint16_t*>(d_X);
  const size_t ysz = yt == UW_F32 ? 4 : 2;
  for (int64_t b0 = 0; b0 < batch; b0 += 16 * kExpMaxTB) {
    const int nb = int(std::min<int64_t>(batch - b0, 16 * kExpMaxTB));
    const int64_t n = int64_t(nb) * cols;
    hipLaunchKernelGGL(permute_x_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, X + b0 * ldx, ldx,
                       int64_t(nb), cols, Xp);
    if (int rc = hip_check(hipGetLastError(), "permute_x_kernel launch")) return rc;
    void* Yp = static_cast<char*>(d_Y) + size_t(b0) * size_t(ldy) * ysz;
    int rc;
    if (nb <= 16) rc = launch_exp<1>(m->dev.sm, ex, rows, cols, Xp, nb, Yp, ldy, yt, s);
    else if (nb <= 32) rc = launch_exp<2>(m->dev.sm, ex, rows, cols, Xp, nb, Yp, ldy, yt, s);
    else rc = launch_exp<4>(m->dev.sm, ex, rows, cols, Xp, nb, Yp, ldy, yt, s);
    if (rc) return rc;
  }
  return UW_OK;
}
