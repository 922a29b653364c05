// The C-ABI: handles, argument checks, variant dispatch and the autotuner.
//
// "Unweight: how we compressed an LLM 22% without sacrificing quality": the
// runtime picks an execution strategy per weight matrix and batch size from
// measurements on the target hardware, not from heuristics (paragraph on the
// four pipelines; paragraph on the autotuner).  Here the candidates are the
// fused decode+product kernel and decompress-to-HBM followed by the bf16
// product; uw_autotune times both with HIP events and stores the winner.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "uw_internal.h"

using namespace uw;

namespace {

int64_t gcd64(int64_t a, int64_t b) {
  while (b) {
    int64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_matrix(const uw_matrix* m) {
  if (!m) return fail(UW_ERR_INVALID, "null matrix handle");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(UW_ERR_HIP, "hipGetDevice failed");
  if (dev != m->device) return fail(UW_ERR_INVALID, "the current device is not the handle's device");
  return UW_OK;
}

int check_dtype(int t) { return t == UW_F32 || t == UW_BF16 ? UW_OK : fail(UW_ERR_INVALID, "dtype must be UW_F32 or UW_BF16"); }

size_t esize(int t) { return t == UW_F32 ? 4 : 2; }

int check_products(const void* X, int64_t batch, int64_t ldx, int xt, const void* Y, int64_t ldy, int yt, int64_t rows,
                   int64_t cols) {
  if (batch < 0) return fail(UW_ERR_INVALID, "negative batch");
  if (check_dtype(xt) || check_dtype(yt)) return UW_ERR_INVALID;
  if (batch == 0) return UW_OK;
  if (!X || !Y) return fail(UW_ERR_INVALID, "null X or Y");
  if (!aligned(X, esize(xt)) || !aligned(Y, esize(yt))) return fail(UW_ERR_INVALID, "X or Y not aligned to its element size");
  if (ldx < cols || (batch > 1 && ldy < rows)) return fail(UW_ERR_INVALID, "ldx < cols or ldy < rows");
  return UW_OK;
}

size_t decompress_ws_bytes(const uw_matrix* m) {
  return (size_t(m->h.rows) * size_t(m->h.cols) * 2 + 255) / 256 * 256;
}

}  // namespace

extern "C" {

int uw_version(void) { return UW_VERSION; }

const char* uw_status_string(int s) {
  switch (s) {
    case UW_OK: return "ok";
    case UW_ERR_INVALID: return "invalid argument";
    case UW_ERR_FORMAT: return "invalid blob format";
    case UW_ERR_NOSPACE: return "buffer too small";
    case UW_ERR_HIP: return "HIP runtime error";
    case UW_ERR_UNSUPPORTED: return "unsupported";
    default: return "unknown status";
  }
}

const char* uw_last_error(void);

int uw_blob_info(const void* blob, size_t n, uw_info* info) {
  if (!blob || !info) return fail(UW_ERR_INVALID, "uw_blob_info: null pointer");
  BlobHeader h;
  int rc = validate_blob(static_cast<const uint8_t*>(blob), n, &h);
  if (rc) return rc;
  std::memset(info, 0, sizeof(*info));
  info->rows = h.rows;
  info->cols = h.cols;
  info->K = int32_t(h.K);
  info->L = int32_t(h.L);
  info->G = int32_t(h.G);
  info->plain = h.plain() ? 1 : 0;
  info->n_blocks = h.n_blocks;
  info->n_raw_groups = int64_t(h.n_raw_groups);
  info->total_bytes = h.total_bytes;
  info->max_segment_bytes = h.max_segment_bytes;
  std::memcpy(info->palette, h.palette, 32);
  std::memcpy(info->code_len, h.code_len, 32);
  const double w = double(h.rows) * double(h.cols);
  info->ratio = double(h.total_bytes) / (2.0 * w);
  info->bits_per_weight = 8.0 * double(h.total_bytes) / w;
  return UW_OK;
}

namespace {
// Decode tables, as the kernels hold them in LDS.  single(i): for the next
// L stream bits i (first bit in bit 0), len | exponent << 7 of the canonical
// code that prefixes i.  L <= 6: words [0, 4096) are the pair table, entry
// i = (len_a + len_b) | E_a << 7 | len_a << 16 | E_b << 23 for the two codes
// that prefix the 12 bits i, and words [4096, 4160) hold single(i) for
// i < 2^L.  L > 6: words [0, 2^L) hold single(i).
int upload_decode_tables(uw_matrix* m) {
  const BlobHeader& h = m->h;
  DevMatrix& d = m->dev;
  uint32_t code[32], rev[32];
  canonical_codes(h, code, rev);
  auto single = [&](uint32_t idx) -> uint32_t {
    for (uint32_t s = 0; s < h.K; ++s) {
      const uint32_t len = h.code_len[s];
      if (len && (idx & ((1u << len) - 1u)) == rev[s]) return len | (uint32_t(h.palette[s]) << 7);
    }
    return 1u | (uint32_t(h.palette[0]) << 7);  // gaps exist only for a one-symbol code; never met in a valid stream
  };
  std::vector<uint32_t> t(kDecodeTableWords, 0u);
  if (h.L <= 6) {
    const uint32_t mask = (1u << h.L) - 1u;
    for (uint32_t i = 0; i <= mask; ++i) t[4096 + i] = single(i);
    for (uint32_t i = 0; i < 4096; ++i) {
      const uint32_t a = t[4096 + (i & mask)], la = a & 0xF;
      const uint32_t b = t[4096 + ((i >> la) & mask)], lb = b & 0xF;
      t[i] = (la + lb) | (a & 0x7F80u) | (la << 16) | ((b & 0x7F80u) << 16);
    }
  } else {
    for (uint32_t i = 0; i < (1u << h.L); ++i) t[i] = single(i);
  }
  void* p = nullptr;
  if (hipMalloc(&p, kDecodeTableBytes) != hipSuccess) return fail(UW_ERR_HIP, "uw_matrix_create: cannot allocate the decode tables");
  if (hipMemcpy(p, t.data(), kDecodeTableBytes, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(p);
    return fail(UW_ERR_HIP, "uw_matrix_create: cannot copy the decode tables");
  }
  m->d_tables = p;
  d.tables = static_cast<const uint32_t*>(p);
  return UW_OK;
}

// Flat walk (G and the groups per row multiples of 16, so no tile crosses a
// row): one descriptor per tile for the loads of its step, two words: the
// 16-byte aligned floor of the tile's segment (byte offset in the queue) and,
// in byte i, 64 minus the lanes of the i-th of the nq 1 KB loads from that
// floor (at least one lane, so every step issues the same number of loads).  A load with nothing
// to move has lane 0 read 16 bytes at floor + 1024 i, so the blob must
// extend that far past the queue; where it does not, the walk by blocks is
// used instead.
int build_step_table(const uint8_t* hb, size_t n, uw_matrix* m) {
  const BlobHeader& h = m->h;
  DevMatrix& d = m->dev;
  d.flat = 0;
  d.steps = nullptr;
  d.n_tiles = 0;
  if (h.G % 16 || d.gpr % 16) return UW_OK;
  // the loads address the queue from 1 KB before it and the sign+mantissa
  // section with 32-bit offsets
  const uint64_t extent = 1024 + h.size_queue + 1024 * uint64_t(d.nq - 1) + 16;
  if (h.off_queue + extent - 1024 > n || extent >= (uint64_t(1) << 32) || h.size_sm >= (uint64_t(1) << 32))
    return UW_OK;
  const uint64_t nb = h.n_blocks, T = d.T;
  const int64_t n_tiles = d.n_groups / 16;
  std::vector<uint32_t> st(2 * size_t(n_tiles + 1), 0u);  // + a spare entry read past the last step
  const uint8_t* bo = hb + h.off_block;
  const uint8_t* sg = hb + h.off_seg;
  int64_t u = 0;
  for (uint64_t blk = 0; blk < nb; ++blk) {
    uint32_t b_off, start;
    std::memcpy(&b_off, bo + 4 * blk, 4);
    const uint64_t gb = std::min<uint64_t>(h.G, uint64_t(d.n_groups) - blk * h.G);
    start = b_off;
    for (uint64_t t = 0; t < gb / 16; ++t, ++u) {
      uint16_t e;
      std::memcpy(&e, sg + 2 * (blk * T + t), 2);
      const uint32_t end = b_off + 4u * e;
      const uint32_t floor16 = start & ~15u;
      const int64_t len = int64_t(end) - floor16;
      uint32_t shifts = 0;  // load i runs on lanes < n_i: its exec mask is ~0 >> (64 - n_i)
      for (int i = 0; i < d.nq; ++i) {
        const int64_t k = std::clamp<int64_t>((len - 1024 * i + 15) / 16, 1, 64);
        shifts |= uint32_t(64 - k) << (8 * i);
      }
      st[2 * u] = floor16;
      st[2 * u + 1] = shifts;
      start = end;
    }
  }
  if (u != n_tiles) return fail(UW_ERR_FORMAT, "tile count does not match the shape");
  void* p = nullptr;
  if (hipMalloc(&p, st.size() * 4) != hipSuccess) return fail(UW_ERR_HIP, "uw_matrix_create: cannot allocate the step table");
  if (hipMemcpy(p, st.data(), st.size() * 4, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(p);
    return fail(UW_ERR_HIP, "uw_matrix_create: cannot copy the step table");
  }
  m->d_steps = p;
  d.steps = static_cast<const uint32_t*>(p);
  d.n_tiles = int32_t(n_tiles);
  d.q_extent = uint32_t(extent);
  d.flat = 1;
  return UW_OK;
}
}  // namespace

int uw_matrix_create(const void* host_blob, size_t n, const void* d_blob, uw_matrix** out) {
  if (!host_blob || !d_blob || !out) return fail(UW_ERR_INVALID, "uw_matrix_create: null pointer");
  if (!aligned(d_blob, 256)) return fail(UW_ERR_INVALID, "uw_matrix_create: device blob must be 256-byte aligned");
  BlobHeader h;
  int rc = validate_blob(static_cast<const uint8_t*>(host_blob), n, &h);
  if (rc) return rc;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(UW_ERR_HIP, "uw_matrix_create: no current HIP device");
  uw_matrix* m = new uw_matrix();
  m->h = h;
  m->device = dev;
  m->d_blob = static_cast<const uint8_t*>(d_blob);
  DevMatrix& d = m->dev;
  std::memset(&d, 0, sizeof(d));
  const uint8_t* b = m->d_blob;
  d.rows = h.rows;
  d.cols = h.cols;
  d.n_groups = h.rows * (h.cols / 64);
  d.gpr = int32_t(h.cols / 64);
  if (h.plain()) {
    d.plain = reinterpret_cast<const uint16_t*>(b + h.off_plain);
  } else {
    d.block_off = reinterpret_cast<const uint32_t*>(b + h.off_block);
    d.seg = reinterpret_cast<const uint16_t*>(b + h.off_seg);
    d.queue = b + h.off_queue;
    d.sm = b + h.off_sm;
    d.G = int32_t(h.G);
    d.n_blocks = int32_t(h.n_blocks);
    d.rb_words = int32_t((h.G + 31) / 32);
    d.T = int32_t((h.G + 15) / 16);
    d.R = int32_t(h.R);
    d.L = int32_t(h.L);
    // the decode tables: built here, loaded into LDS by the kernels
    if (int rc2 = upload_decode_tables(m)) {
      uw_matrix_destroy(m);
      return rc2;
    }
    // an LDS slot holds any segment; it is filled by 1 KB direct loads
    // (a segment is loaded from its 16-byte aligned floor, up to 12 bytes
    // before it, and lanes that take no word read the word after its end)
    d.slot_bytes = int32_t((h.max_segment_bytes + 16 + 15) / 16 * 16);
    d.seg_loads = std::max(1, (d.slot_bytes + 1023) / 1024);
    // every step issues nq loads; a load with no bytes to move still has
    // lane 0 write 16 bytes at 1024 * i, which the slot must hold
    d.nq = d.seg_loads <= 2 ? 2 : 4;
    d.slot_bytes = std::max(d.slot_bytes, 1024 * (d.nq - 1) + 16);
    // a work unit covers whole rows: lcm(G, groups per row) groups
    const int64_t lcm = int64_t(h.G) / gcd64(h.G, d.gpr) * d.gpr;
    d.unit_blocks = int32_t(lcm / h.G);
    d.rows_per_unit = int32_t(lcm / d.gpr);
    d.n_units = int32_t((int64_t(h.n_blocks) + d.unit_blocks - 1) / d.unit_blocks);
    rc = build_step_table(static_cast<const uint8_t*>(host_blob), n, m);
    if (rc) {
      uw_matrix_destroy(m);
      return rc;
    }
    // one wave per block when a unit has several blocks and each block holds
    // a row end (G > groups per row): a row then spans at most two blocks,
    // and the waves of one unit share a workgroup (at most 16 waves)
    d.split = d.flat && d.unit_blocks > 1 && d.unit_blocks <= 8 && int64_t(h.G) > d.gpr;
    d.n_items = d.split ? d.n_blocks : d.n_units;
  }
  *out = m;
  return UW_OK;
}

void uw_matrix_destroy(uw_matrix* m) {
  if (!m) return;
  if (m->d_steps || m->d_tables) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != m->device) (void)hipSetDevice(m->device);
    if (m->d_steps) (void)hipFree(m->d_steps);
    if (m->d_tables) (void)hipFree(m->d_tables);
    if (cur != m->device && cur >= 0) (void)hipSetDevice(cur);
  }
  delete m;
}

int uw_decompress(const uw_matrix* m, uint16_t* d_out, int64_t ld_out, void* stream) {
  if (int rc = check_matrix(m)) return rc;
  if (!d_out || !aligned(d_out, 16)) return fail(UW_ERR_INVALID, "uw_decompress: output must be non-null and 16-byte aligned");
  if (ld_out < m->h.cols || ld_out % 8) return fail(UW_ERR_INVALID, "uw_decompress: ld_out must be >= cols and a multiple of 8");
  return launch_decompress(m, d_out, ld_out, stream);
}

int uw_gemv_fused(const uw_matrix* m, const void* d_x, int xt, void* d_y, int yt, void* stream) {
  if (int rc = check_matrix(m)) return rc;
  if (int rc = check_products(d_x, 1, m->h.cols, xt, d_y, m->h.rows, yt, m->h.rows, m->h.cols)) return rc;
  std::string why;
  if (!fused_supported(m, xt, &why)) return fail(UW_ERR_UNSUPPORTED, "uw_gemv_fused: " + why);
  if (m->h.plain() && !bf16_gemm_supported(m->h.cols, 1, xt, &why)) return fail(UW_ERR_UNSUPPORTED, "uw_gemv_fused: " + why);
  return launch_fused(m, d_x, 1, m->h.cols, xt, d_y, m->h.rows, yt, stream);
}

size_t uw_workspace_size(const uw_matrix* m, int64_t batch, int variant) {
  if (!m || batch < 0) return 0;
  if (variant == UW_VARIANT_FUSED || variant == UW_VARIANT_FUSED_MFMA) return 0;
  return decompress_ws_bytes(m);
}

int uw_set_plan(uw_matrix* m, const uw_plan* plan) {
  if (!m || !plan) return fail(UW_ERR_INVALID, "uw_set_plan: null pointer");
  if (plan->batch < 1 || plan->variant <= UW_VARIANT_AUTO || plan->variant >= UW_VARIANT_COUNT)
    return fail(UW_ERR_INVALID, "uw_set_plan: batch >= 1 and a concrete variant");
  std::lock_guard<std::mutex> lk(m->mu);
  m->plans[plan->batch] = *plan;
  return UW_OK;
}

int uw_get_plan(const uw_matrix* m, int64_t batch, uw_plan* out) {
  if (!m || !out) return fail(UW_ERR_INVALID, "uw_get_plan: null pointer");
  std::lock_guard<std::mutex> lk(m->mu);
  auto it = m->plans.find(batch);
  if (it == m->plans.end()) return fail(UW_ERR_INVALID, "uw_get_plan: no plan for this batch");
  *out = it->second;
  return UW_OK;
}

int uw_gemm_fused(const uw_matrix* m, const void* d_X, int64_t batch, int64_t ldx, int xt, void* d_Y, int64_t ldy,
                  int yt, int variant, void* d_ws, size_t ws_bytes, void* stream) {
  if (int rc = check_matrix(m)) return rc;
  if (int rc = check_products(d_X, batch, ldx, xt, d_Y, ldy, yt, m->h.rows, m->h.cols)) return rc;
  if (batch == 0) return UW_OK;
  if (variant < 0 || variant >= UW_VARIANT_COUNT) return fail(UW_ERR_INVALID, "uw_gemm_fused: unknown variant");
  std::string why, why_mfma;
  const bool fused_ok = fused_supported(m, xt, &why) && (!m->h.plain() || bf16_gemm_supported(m->h.cols, batch, xt, &why));
  const bool mfma_ok = fused_mfma_supported(m, xt, &why_mfma) && aligned(d_X, 16) && ldx % 8 == 0;
  if (!mfma_ok && why_mfma.empty()) why_mfma = "X must be 16-byte aligned with ldx a multiple of 8";
  if (variant == UW_VARIANT_AUTO) {
    uw_plan p;
    bool have = false;
    {
      std::lock_guard<std::mutex> lk(m->mu);
      auto it = m->plans.find(batch);
      if (it != m->plans.end()) {
        p = it->second;
        have = true;
      }
    }
    // Without a plan: one or two rows on VALU (when one pass takes them);
    // up to 32 rows on the matrix cores; beyond that decompress + library
    // GEMM when the workspace is given (the measured crossovers on the MLP
    // shapes: at 64 rows decompress + GEMM is ahead on down_proj).
    const bool ws_ok = d_ws && ws_bytes >= decompress_ws_bytes(m);
    if (have) variant = p.variant;
    else if (fused_ok && (batch == 1 || (batch == 2 && fused_rows_per_pass(m, batch, xt) >= 2)))
      variant = UW_VARIANT_FUSED;
    else if (mfma_ok && (batch <= 32 || (batch <= 64 && !ws_ok))) variant = UW_VARIANT_FUSED_MFMA;
    else if (ws_ok && (xt == UW_BF16 || !fused_ok)) variant = UW_VARIANT_DECOMPRESS_GEMM;
    else if (mfma_ok) variant = UW_VARIANT_FUSED_MFMA;
    else variant = fused_ok || !ws_ok ? UW_VARIANT_FUSED : UW_VARIANT_DECOMPRESS_GEMM;
  }
  if (variant == UW_VARIANT_FUSED_MFMA) {
    if (!mfma_ok) return fail(UW_ERR_UNSUPPORTED, "uw_gemm_fused: " + why_mfma);
    return launch_fused_mfma(m, d_X, batch, ldx, d_Y, ldy, yt, stream);
  }
  if (variant == UW_VARIANT_FUSED) {
    if (!fused_ok) return fail(UW_ERR_UNSUPPORTED, "uw_gemm_fused: " + why);
    return launch_fused(m, d_X, batch, ldx, xt, d_Y, ldy, yt, stream);
  }
  // decompress into the workspace, then the bf16 product
  if (!d_ws || ws_bytes < decompress_ws_bytes(m) || !aligned(d_ws, 256))
    return fail(UW_ERR_NOSPACE, "uw_gemm_fused: workspace missing, too small or not 256-byte aligned");
  if (!bf16_gemm_supported(m->h.cols, batch, xt, &why)) return fail(UW_ERR_UNSUPPORTED, "uw_gemm_fused: " + why);
  uint16_t* W = static_cast<uint16_t*>(d_ws);
  if (int rc = launch_decompress(m, W, m->h.cols, stream)) return rc;
  return launch_bf16_gemm(W, m->h.rows, m->h.cols, m->h.cols, d_X, batch, ldx, xt, d_Y, ldy, yt, stream);
}

size_t uw_autotune_scratch_size(const uw_matrix* m, int64_t batch) {
  if (!m || batch < 0) return 0;
  const size_t xb = (size_t(batch) * size_t(m->h.cols) * 2 + 255) / 256 * 256;
  const size_t yb = (size_t(batch) * size_t(m->h.rows) * 2 + 255) / 256 * 256;
  return xb + yb;
}

int uw_autotune(uw_matrix* m, int64_t batch, void* d_ws, size_t ws_bytes, void* stream, uw_plan* out) {
  if (int rc = check_matrix(m)) return rc;
  if (batch < 1) return fail(UW_ERR_INVALID, "uw_autotune: batch must be >= 1");
  const size_t need_ws = uw_workspace_size(m, batch, UW_VARIANT_AUTO);
  const size_t need = need_ws + uw_autotune_scratch_size(m, batch);
  if (!d_ws || ws_bytes < need || !aligned(d_ws, 256)) return fail(UW_ERR_NOSPACE, "uw_autotune: workspace too small");
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(d_ws);
  void* X = base + need_ws;
  void* Y = base + need_ws + (size_t(batch) * size_t(m->h.cols) * 2 + 255) / 256 * 256;
  // X = 1.0 everywhere (values do not change the work of either candidate)
  if (hipMemsetD16Async(reinterpret_cast<hipDeviceptr_t>(X), 0x3F80, size_t(batch) * size_t(m->h.cols), s) != hipSuccess)
    return fail(UW_ERR_HIP, "uw_autotune: memset failed");
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return fail(UW_ERR_HIP, "uw_autotune: event");
  uw_plan plan;
  std::memset(&plan, 0, sizeof(plan));
  plan.batch = batch;
  for (int v = 0; v < UW_VARIANT_COUNT; ++v) plan.candidate_us[v] = -1.f;
  float best = 1e30f;
  int best_v = -1;
  const int warm = 3, reps = 15;
  for (int v = UW_VARIANT_FUSED; v < UW_VARIANT_COUNT; ++v) {
    std::vector<float> t;
    int rc = UW_OK;
    for (int i = 0; i < warm + reps && rc == UW_OK; ++i) {
      hipEventRecord(e0, s);
      rc = uw_gemm_fused(m, X, batch, m->h.cols, UW_BF16, Y, m->h.rows, UW_BF16, v, d_ws, need_ws, stream);
      hipEventRecord(e1, s);
      if (rc) break;
      if (hipEventSynchronize(e1) != hipSuccess) {
        rc = UW_ERR_HIP;
        break;
      }
      float ms = 0;
      hipEventElapsedTime(&ms, e0, e1);
      if (i >= warm) t.push_back(ms * 1000.f);
    }
    if (rc == UW_ERR_HIP) {
      hipEventDestroy(e0);
      hipEventDestroy(e1);
      return rc;
    }
    if (rc || t.empty()) continue;  // not applicable to this matrix/batch
    std::sort(t.begin(), t.end());
    const float med = t[t.size() / 2];
    plan.candidate_us[v] = med;
    if (med < best) {
      best = med;
      best_v = v;
    }
  }
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  if (best_v < 0) return fail(UW_ERR_UNSUPPORTED, "uw_autotune: no candidate can run this matrix and batch");
  plan.variant = best_v;
  plan.time_us = best;
  {
    std::lock_guard<std::mutex> lk(m->mu);
    m->plans[batch] = plan;
  }
  if (out) *out = plan;
  set_error("");
  return UW_OK;
}

int uw_bf16_gemm(const uint16_t* d_W, int64_t rows, int64_t cols, int64_t ldw, const void* d_X, int64_t batch,
                 int64_t ldx, int xt, void* d_Y, int64_t ldy, int yt, void* stream) {
  if (!d_W || !aligned(d_W, 16)) return fail(UW_ERR_INVALID, "uw_bf16_gemm: W must be non-null and 16-byte aligned");
  if (rows < 1 || cols < 8 || cols % 8 || ldw < cols || ldw % 8) return fail(UW_ERR_INVALID, "uw_bf16_gemm: bad shape");
  if (int rc = check_products(d_X, batch, ldx, xt, d_Y, ldy, yt, rows, cols)) return rc;
  if (batch == 0) return UW_OK;
  std::string why;
  if (!bf16_gemm_supported(cols, batch, xt, &why)) return fail(UW_ERR_UNSUPPORTED, "uw_bf16_gemm: " + why);
  return launch_bf16_gemm(d_W, rows, cols, ldw, d_X, batch, ldx, xt, d_Y, ldy, yt, stream);
}

size_t uw_read_probe_sink_size(void) { return read_probe_sink_bytes(); }

int uw_read_probe(const void* d_src, size_t bytes, void* d_sink, void* stream) {
  if (!d_src || !d_sink || !aligned(d_src, 16) || !aligned(d_sink, 4) || bytes % 16 || bytes == 0)
    return fail(UW_ERR_INVALID, "uw_read_probe: bad arguments");
  return launch_read_probe(d_src, bytes, d_sink, stream);
}

}  // extern "C"
