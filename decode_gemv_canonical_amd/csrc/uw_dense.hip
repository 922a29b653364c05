// Uncompressed kernels for gfx950: the bf16 product on the vector ALU for
// small batches (the comparator, the product half of decompress-then-multiply
// and the plain-mode path; larger batches go to the matrix-core kernel of
// uw_gemm.hip), the plain-mode copy and a streaming-read probe.
#include <algorithm>

#include "uw_device.h"

namespace uw {
namespace {

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
// Streaming read: every byte read once with 16-byte loads, xor-folded so the
// loads cannot be removed.  The launch shape comes from a sweep over
// workgroup sizes (256..1024 threads), grids (1 to 16 workgroups per compute
// unit) and loads in flight per thread (1..8), for 80 MiB and 1 GiB reads
// rotated over cold buffers: 1024 threads, 16 workgroups per compute unit,
// a grid-stride loop, 13.6-14.3 us for 80 MiB.  The closing fold is four DPP
// steps inside each row of 16 lanes and one store per row: the grid runs in 8
// rounds of resident workgroups and each round waits for its slowest wave's
// closing instructions, which with a 6-step LDS shuffle cost 4 us in all.
__device__ __forceinline__ uint32_t xor_dpp(uint32_t v, int ctrl_id) {
  int r;
  switch (ctrl_id) {
    case 0: r = __builtin_amdgcn_update_dpp(0, int(v), 0xB1, 0xF, 0xF, false); break;   // quad_perm 1,0,3,2
    case 1: r = __builtin_amdgcn_update_dpp(0, int(v), 0x4E, 0xF, 0xF, false); break;   // quad_perm 2,3,0,1
    case 2: r = __builtin_amdgcn_update_dpp(0, int(v), 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: r = __builtin_amdgcn_update_dpp(0, int(v), 0x140, 0xF, 0xF, false); break; // row_mirror
  }
  return v ^ uint32_t(r);
}

__global__ __launch_bounds__(1024) void read_probe_kernel(const uint4* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  uint32_t x = 0;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 a = src[i];
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  // every lane of a row of 16 ends with the row's xor
  x = xor_dpp(x, 0);
  x = xor_dpp(x, 1);
  x = xor_dpp(x, 2);
  x = xor_dpp(x, 3);
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (threadIdx.x % 16 == 0) sink[t / 16] = x;
}

constexpr int kProbeThreads = 1024;
constexpr int kProbeBlocksPerCu = 16;
constexpr int kProbeMaxBlocks = 16 * 256;

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

}  // namespace

int launch_copy_plain(const uint16_t* src, int64_t rows, int64_t cols, uint16_t* out, int64_t ld_out, void* stream) {
  const int64_t n = rows * (cols / 8);
  const int grid = int(std::min<int64_t>((n + 255) / 256, 8192));
  hipLaunchKernelGGL(copy_plain_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), src, rows, cols, out,
                     ld_out);
  return hip_check(hipGetLastError(), "copy_plain_kernel launch");
}

// bf16 activations that are 16-byte aligned with a row stride that is a
// multiple of 8 go to the matrix-core kernel (uw_gemm.hip), except a single
// activation row of at most kValuMaxCols columns, which the GEMV-style kernel
// (x in LDS, one wave per row) reads faster.  Measured on the MLP shapes with
// 8 rotated copies of W: gate 14336x4096 batch 1 24.5 us on the vector ALU
// against 27.8 on the matrix cores; batch 2..8 27-28 us on the matrix cores
// against 31-144 us for the vector kernel's passes over W; down 4096x14336
// batch 1 29.4 against 32.6 us.
constexpr int64_t kValuMaxCols = 8192;

bool bf16_gemm_on_mfma(const void* X, int64_t batch, int64_t cols, int64_t ldx, int xt) {
  return xt == UW_BF16 && (batch > 1 || cols > kValuMaxCols) && reinterpret_cast<uintptr_t>(X) % 16 == 0 &&
         ldx % 8 == 0;
}

bool bf16_gemm_supported(int64_t cols, int64_t batch, int xt, std::string* why) {
  if (xt == UW_BF16 && (batch > 1 || cols > kValuMaxCols)) return true;  // matrix cores, or VALU passes when X is unaligned
  const size_t per = xt == UW_F32 ? size_t(cols) * 4 : size_t(cols) * 2;
  if (per > size_t(kLdsLimit)) {
    if (why) *why = "x of this width does not fit in LDS";
    return false;
  }
  return true;
}

int launch_bf16_gemm(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw, const void* X, int64_t batch,
                     int64_t ldx, int xt, void* Y, int64_t ldy, int yt, void* stream, int shape, int ks) {
  if (bf16_gemm_on_mfma(X, batch, cols, ldx, xt))
    return launch_mfma_gemm(W, rows, cols, ldw, static_cast<const uint16_t*>(X), batch, ldx, Y, ldy, yt, shape, ks,
                            stream);
  if (xt == UW_BF16 && size_t(cols) * 2 > size_t(kLdsLimit))
    return fail(UW_ERR_UNSUPPORTED, "bf16 product: X must be 16-byte aligned with ldx a multiple of 8 for this width");
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

size_t read_probe_sink_bytes() { return size_t(kProbeMaxBlocks) * (kProbeThreads / 16) * 4; }  // a word per row of 16 lanes

int launch_read_probe(const void* src, size_t bytes, void* sink, void* stream) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const int blocks = std::min(kProbeMaxBlocks, std::max(1, cus) * kProbeBlocksPerCu);
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), int64_t(bytes / 16), static_cast<uint32_t*>(sink));
  return hip_check(hipGetLastError(), "read_probe_kernel launch");
}

}  // namespace uw
