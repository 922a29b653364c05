// Plain bf16 GEMM through rocBLAS: the product half of the
// decompress-then-multiply path once the batch makes it a real dense
// contraction.  Y[b, n] = sum_k X[b, k] W[n, k], fp32 accumulation, all
// operands row-major on the device.
//
// rocBLAS is column-major: row-major W (rows x cols, ldw) is the
// column-major cols x rows matrix A with lda = ldw, so op(A) = A^T is W;
// row-major X (batch x cols, ldx) is the column-major cols x batch matrix B;
// row-major Y (batch x rows, ldy) is the column-major rows x batch result.
#include <hip/hip_runtime_api.h>
#include <rocblas/rocblas.h>

#include <mutex>
#include <string>

#include "uw_internal.h"

namespace uw {
namespace {

constexpr int kMaxDevices = 64;

struct Handles {
  std::mutex mu;
  rocblas_handle h[kMaxDevices] = {};
};

Handles& handles() {
  static Handles s;
  return s;
}

}  // namespace

bool library_gemm_supported(int64_t rows, int64_t cols, int64_t batch, int xt) {
  const int64_t lim = int64_t(1) << 31;
  return xt == UW_BF16 && rows < lim && cols < lim && batch < lim;
}

int launch_library_gemm(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw, const void* X, int64_t batch,
                        int64_t ldx, void* Y, int64_t ldy, int yt, void* stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(UW_ERR_HIP, "library GEMM: no usable current device");
  Handles& hs = handles();
  // one handle per device; a handle is used by one call at a time
  std::lock_guard<std::mutex> lk(hs.mu);
  if (!hs.h[dev] && rocblas_create_handle(&hs.h[dev]) != rocblas_status_success) {
    hs.h[dev] = nullptr;
    return fail(UW_ERR_HIP, "library GEMM: rocblas_create_handle failed");
  }
  rocblas_handle h = hs.h[dev];
  if (rocblas_set_stream(h, static_cast<hipStream_t>(stream)) != rocblas_status_success)
    return fail(UW_ERR_HIP, "library GEMM: rocblas_set_stream failed");
  const float alpha = 1.0f, beta = 0.0f;
  const rocblas_datatype yty = yt == UW_BF16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
  const rocblas_status st =
      rocblas_gemm_ex(h, rocblas_operation_transpose, rocblas_operation_none, rocblas_int(rows), rocblas_int(batch),
                      rocblas_int(cols), &alpha, W, rocblas_datatype_bf16_r, rocblas_int(ldw), X,
                      rocblas_datatype_bf16_r, rocblas_int(ldx), &beta, Y, yty, rocblas_int(ldy), Y, yty,
                      rocblas_int(ldy), rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0,
                      rocblas_gemm_flags_none);
  if (st != rocblas_status_success)
    return fail(UW_ERR_HIP, std::string("library GEMM: rocblas_gemm_ex: ") + rocblas_status_to_string(st));
  return UW_OK;
}

}  // namespace uw
