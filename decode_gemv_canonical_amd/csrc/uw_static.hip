// uw_gemm_fused_static: uw_gemm_fused for callers that cannot allocate
// (code under graph capture, tight serving loops, harnesses that forbid
// allocation).  The decompress + GEMM variant needs R x C x 2 bytes of
// workspace for the decompressed matrix; here it runs band by band through a
// fixed scratch array that lives in the library's device image instead.
//
// scratch is a file-scope __device__ array: every GPU the library runs on
// holds its own copy (kStaticScratchBytes) until the process ends.  In host
// code the array's name is only a host-side stand-in, so the device address
// of each GPU's copy is looked up once per device with hipGetSymbolAddress
// and kept; kernels receive that address as an argument.  Calls on one GPU
// share its copy: calls that overlap on different streams of the same GPU
// race on it.  Nothing in it needs clearing: a band's decompress writes every
// element the band's product reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "uw_device.h"

namespace uw {
namespace {

constexpr size_t kStaticScratchBytes = size_t(64) << 20;  // 64 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// Device address of this GPU's scratch (looked up once per device).
int scratch_ptr(void** out) {
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(UW_ERR_HIP, "uw_gemm_fused_static: no usable current device");
  std::lock_guard<std::mutex> lk(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(UW_ERR_HIP, std::string("uw_gemm_fused_static: hipGetSymbolAddress: ") + hipGetErrorString(e));
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return UW_OK;
}

}  // namespace

size_t static_scratch_bytes() { return kStaticScratchBytes; }

// Rows of one band: whole work units (units hold whole rows; with split rows
// a unit is unit_blocks blocks), as many as fit in the scratch.
int64_t static_band_units(const uw_matrix* m) {
  const DevMatrix& d = m->dev;
  const int64_t unit_bytes = int64_t(d.rows_per_unit) * d.cols * 2;
  return unit_bytes > 0 ? int64_t(kStaticScratchBytes) / unit_bytes : 0;
}

// Decompress + GEMM through the scratch, one band of rows at a time.
int static_decompress_gemm(const uw_matrix* m, const void* X, int64_t batch, int64_t ldx, int xt, void* Y, int64_t ldy,
                           int yt, int knob, void* stream) {
  const DevMatrix& d = m->dev;
  if (m->h.plain())  // the blob holds the bf16 weights: no scratch needed
    return launch_bf16_gemm(d.plain, d.rows, d.cols, d.cols, X, batch, ldx, xt, Y, ldy, yt, stream, knob & 31, knob >> 5);
  const int64_t band = static_band_units(m);
  if (band < 1)
    return fail(UW_ERR_UNSUPPORTED, "uw_gemm_fused_static: one work unit of this matrix (" +
                                        std::to_string(d.rows_per_unit) + " rows) exceeds the " +
                                        std::to_string(kStaticScratchBytes >> 20) + " MiB scratch");
  void* ptr = nullptr;
  if (int rc = scratch_ptr(&ptr)) return rc;
  uint16_t* W = static_cast<uint16_t*>(ptr);
  const int ipu = d.flat && d.split ? d.unit_blocks : 1;  // work items per unit
  const int n_items = d.flat ? d.n_items : d.n_units;
  const size_t ysz = yt == UW_F32 ? 4 : 2;
  for (int64_t u0 = 0; u0 < d.n_units; u0 += band) {
    const int64_t u1 = std::min<int64_t>(d.n_units, u0 + band);
    const int64_t r0 = u0 * d.rows_per_unit, r1 = std::min<int64_t>(d.rows, u1 * d.rows_per_unit);
    const int i0 = int(u0 * ipu), i1 = int(std::min<int64_t>(n_items, u1 * ipu));
    if (int rc = launch_decompress_items(m, W, d.cols, i0, i1, r0, stream)) return rc;
    void* Yb = static_cast<char*>(Y) + size_t(r0) * ysz;
    if (int rc = launch_bf16_gemm(W, r1 - r0, d.cols, d.cols, X, batch, ldx, xt, Yb, ldy, yt, stream, knob & 31,
                                  knob >> 5))
      return rc;
  }
  return UW_OK;
}

}  // namespace uw
