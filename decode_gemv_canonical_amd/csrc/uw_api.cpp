// The C-ABI: handles, argument checks, variant dispatch, the autotuner and
// its plan files.
//
// "Unweight: how we compressed an LLM 22% without sacrificing quality": the
// runtime picks an execution strategy per weight matrix and batch size from
// measurements on the target hardware, not from heuristics (paragraph on the
// four pipelines; paragraph on the autotuner, whose result is a per-model
// configuration file).  Here the candidates are the fused decode+product on
// the vector ALU and on the matrix cores, decompress-to-HBM followed by the
// bf16 product, and an attached direct-palette copy, each with its knobs;
// uw_autotune times them cold with HIP events and stores the winner.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
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

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

constexpr size_t kFlushBytes = size_t(512) << 20;  // twice the 256 MiB last-level cache

// Whether a (variant, knob) can run a call with these operands, and why not.
struct CallShape {
  const void* X;
  int64_t batch, ldx;
  int xt;
  const void* ws;
  size_t ws_bytes;
};

bool knob_valid(int variant, int knob) {
  switch (variant) {
    case UW_VARIANT_FUSED: {
      const int rs = knob & 7, wpw = knob >> 3;
      return knob >= 0 && (rs == 0 || rs == 2 || rs == 4) && wpw <= 16;
    }
    case UW_VARIANT_FUSED_MFMA: return knob == 0 || (knob >= 8 && knob <= 16);
    case UW_VARIANT_DECOMPRESS_GEMM: {
      const int shape = knob & 31, ks = knob >> 5;
      return knob >= 0 && shape < mfma_gemm_shape_count() && (ks == 0 || ks == 1 || ks == 2 || ks == 4 || ks == 8);
    }
    case UW_VARIANT_PALETTE: return knob == 0;
    default: return false;
  }
}

bool runnable(const uw_matrix* m, int variant, int knob, const CallShape& c, std::string* why) {
  const int64_t batch = c.batch;
  switch (variant) {
    case UW_VARIANT_FUSED:
      if (!fused_supported(m, c.xt, why)) return false;
      if (m->h.plain() && !bf16_gemm_supported(m->h.cols, batch, c.xt, why)) return false;
      if ((knob & 7) && !m->h.plain() && !m->dev.flat) {
        if (why) *why = "the ring-depth knob needs the flat walk (G and cols/64 multiples of 16)";
        return false;
      }
      return true;
    case UW_VARIANT_FUSED_MFMA:
      if (!fused_mfma_supported(m, c.xt, why, knob)) return false;
      if (!aligned(c.X, 16) || c.ldx % 8) {
        if (why) *why = "X must be 16-byte aligned with ldx a multiple of 8";
        return false;
      }
      return true;
    case UW_VARIANT_DECOMPRESS_GEMM:
      if (!c.ws || c.ws_bytes < decompress_ws_bytes(m) || !aligned(c.ws, 256)) {
        if (why) *why = "workspace missing, too small or not 256-byte aligned";
        return false;
      }
      if (!bf16_gemm_supported(m->h.cols, batch, c.xt, why)) return false;
      if ((knob & 31) && !bf16_gemm_on_mfma(c.X, batch, m->h.cols, c.ldx, c.xt)) {
        if (why)
          *why = "a matrix-core GEMM shape needs bf16 X, 16-byte aligned, ldx a multiple of 8, and batch > 1 or cols > 8192";
        return false;
      }
      return true;
    case UW_VARIANT_PALETTE:
      if (!m->palette) {
        if (why) *why = "no direct-palette copy is attached";
        return false;
      }
      if (!aligned(c.X, 16) || (batch > 1 && (c.xt != UW_BF16 || c.ldx % 8))) {
        if (why) *why = "the palette path needs X 16-byte aligned (and bf16 with ldx a multiple of 8 above batch 1)";
        return false;
      }
      return true;
    default:
      if (why) *why = "unknown variant";
      return false;
  }
}

const char* variant_name(int v) {
  switch (v) {
    case UW_VARIANT_FUSED: return "fused";
    case UW_VARIANT_DECOMPRESS_GEMM: return "decompress_gemm";
    case UW_VARIANT_FUSED_MFMA: return "fused_mfma";
    case UW_VARIANT_PALETTE: return "palette";
    default: return "auto";
  }
}

uint32_t blob_crc(const uw_matrix* m) { return m->h.crc32; }

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
// L stream bits i (first bit in bit 0), len | v << 7 of the canonical code
// that prefixes i, where v is its exponent (the decode tables) or its
// palette index (the index tables, for the transcode to the direct form).
// L <= 6: words [0, 4096) are the pair table, entry i = (len_a + len_b) |
// v_a << 7 | len_a << 16 | v_b << 23 for the two codes that prefix the 12
// bits i, and words [4096, 4160) hold single(i) for i < 2^L.  L > 6: words
// [0, 2^L) hold single(i).
std::vector<uint32_t> decode_table_image(const BlobHeader& h, bool index) {
  uint32_t code[32], rev[32];
  canonical_codes(h, code, rev);
  auto value = [&](uint32_t s) { return index ? s : uint32_t(h.palette[s]); };
  auto single = [&](uint32_t idx) -> uint32_t {
    for (uint32_t s = 0; s < h.K; ++s) {
      const uint32_t len = h.code_len[s];
      if (len && (idx & ((1u << len) - 1u)) == rev[s]) return len | (value(s) << 7);
    }
    return 1u | (value(0) << 7);  // gaps exist only for a one-symbol code; never met in a valid stream
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
  return t;
}

bool flat_shape(const BlobHeader& h) { return !h.plain() && h.G % 16 == 0 && (h.cols / 64) % 16 == 0; }

// Flat walk (G and the groups per row multiples of 16, so no tile crosses a
// row): one descriptor per tile for the loads of its step, two words: the
// 16-byte aligned floor of the tile's segment (byte offset in the queue) and,
// in byte i, 64 minus the lanes of the i-th of the nq 1 KB loads from that
// floor (at least one lane, so every step issues the same number of loads).  A load with nothing
// to move has lane 0 read 16 bytes at floor + 1024 i, so the blob must
// extend that far past the queue; where it does not, the walk by blocks is
// used instead.  Returns the table (empty: no flat walk).
int build_step_table(const uint8_t* hb, size_t n, uw_matrix* m, std::vector<uint32_t>* out) {
  const BlobHeader& h = m->h;
  DevMatrix& d = m->dev;
  d.flat = 0;
  d.steps = nullptr;
  d.n_tiles = 0;
  out->clear();
  if (!flat_shape(h)) return UW_OK;
  // the loads address the queue from 1 KB before it and the sign+mantissa
  // section with 32-bit offsets
  const uint64_t extent = 1024 + h.size_queue + 1024 * uint64_t(d.nq - 1) + 16;
  if (h.off_queue + extent - 1024 > n || extent >= (uint64_t(1) << 32) || h.size_sm >= (uint64_t(1) << 32))
    return UW_OK;
  const uint64_t nb = h.n_blocks, T = d.T;
  const int64_t n_tiles = d.n_groups / 16;
  std::vector<uint32_t>& st = *out;
  st.assign(2 * size_t(n_tiles + 1), 0u);  // + a spare entry read past the last step
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
  d.n_tiles = int32_t(n_tiles);
  d.q_extent = uint32_t(extent);
  d.flat = 1;
  return UW_OK;
}
// Where uw_matrix_create puts the derived tables in the caller's device
// buffer: after the blob (256-byte aligned), the decode tables, the index
// tables, then the flat walk's step table (8 bytes per tile + a spare entry).
struct AuxLayout {
  size_t off_tables = 0, off_index_tables = 0, off_steps = 0, steps_bytes = 0, total = 0;
};

AuxLayout aux_layout(const BlobHeader& h, size_t blob_bytes) {
  AuxLayout a;
  size_t o = align256(blob_bytes);
  if (h.plain()) {
    a.off_tables = a.off_index_tables = a.off_steps = o;
    a.total = o;
    return a;
  }
  a.off_tables = o;
  o += align256(kDecodeTableBytes);
  a.off_index_tables = o;
  o += align256(kDecodeTableBytes);
  a.off_steps = o;
  a.steps_bytes = flat_shape(h) ? 8 * (size_t(h.rows) * size_t(h.cols) / 1024 + 1) : 0;
  o += align256(a.steps_bytes);
  a.total = o;
  return a;
}
}  // namespace

size_t uw_matrix_device_bytes(const void* host_blob, size_t n) {
  if (!host_blob) {
    fail(UW_ERR_INVALID, "uw_matrix_device_bytes: null blob");
    return 0;
  }
  BlobHeader h;
  if (validate_blob(static_cast<const uint8_t*>(host_blob), n, &h)) return 0;
  return aux_layout(h, n).total;
}

int uw_matrix_create(const void* host_blob, size_t n, void* d_buf, size_t d_bytes, uw_matrix** out) {
  if (!host_blob || !d_buf || !out) return fail(UW_ERR_INVALID, "uw_matrix_create: null pointer");
  if (!aligned(d_buf, 256)) return fail(UW_ERR_INVALID, "uw_matrix_create: device buffer must be 256-byte aligned");
  BlobHeader h;
  int rc = validate_blob(static_cast<const uint8_t*>(host_blob), n, &h);
  if (rc) return rc;
  const AuxLayout aux = aux_layout(h, n);
  if (d_bytes < aux.total)
    return fail(UW_ERR_INVALID, "uw_matrix_create: the device buffer is smaller than uw_matrix_device_bytes()");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(UW_ERR_HIP, "uw_matrix_create: no current HIP device");
  uw_matrix* m = new uw_matrix();
  m->h = h;
  m->device = dev;
  m->d_blob = static_cast<const uint8_t*>(d_buf);
  uint8_t* dwrite = static_cast<uint8_t*>(d_buf);
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
    const std::vector<uint32_t> tab = decode_table_image(h, false), itab = decode_table_image(h, true);
    if (hipMemcpy(dwrite + aux.off_tables, tab.data(), kDecodeTableBytes, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(dwrite + aux.off_index_tables, itab.data(), kDecodeTableBytes, hipMemcpyHostToDevice) != hipSuccess) {
      delete m;
      return fail(UW_ERR_HIP, "uw_matrix_create: cannot copy the decode tables");
    }
    d.tables = reinterpret_cast<const uint32_t*>(b + aux.off_tables);
    d.index_tables = reinterpret_cast<const uint32_t*>(b + aux.off_index_tables);
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
    std::vector<uint32_t> steps;
    rc = build_step_table(static_cast<const uint8_t*>(host_blob), n, m, &steps);
    if (rc) {
      delete m;
      return rc;
    }
    if (d.flat) {
      if (steps.size() * 4 > aux.steps_bytes ||
          hipMemcpy(dwrite + aux.off_steps, steps.data(), steps.size() * 4, hipMemcpyHostToDevice) != hipSuccess) {
        delete m;
        return fail(UW_ERR_HIP, "uw_matrix_create: cannot copy the step table");
      }
      d.steps = reinterpret_cast<const uint32_t*>(b + aux.off_steps);
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

void uw_matrix_destroy(uw_matrix* m) { delete m; }

int uw_matrix_attach_palette(uw_matrix* m, const uw_palette* p) {
  if (!m) return fail(UW_ERR_INVALID, "uw_matrix_attach_palette: null matrix handle");
  if (p && (p->l.rows != m->h.rows || p->l.cols != m->h.cols))
    return fail(UW_ERR_INVALID, "uw_matrix_attach_palette: the palette copy has another shape");
  std::lock_guard<std::mutex> lk(m->mu);
  m->palette = p;
  return UW_OK;
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
  if (variant == UW_VARIANT_FUSED || variant == UW_VARIANT_FUSED_MFMA || variant == UW_VARIANT_PALETTE) return 0;
  return decompress_ws_bytes(m);
}

int uw_set_plan(uw_matrix* m, const uw_plan* plan) {
  if (!m || !plan) return fail(UW_ERR_INVALID, "uw_set_plan: null pointer");
  if (plan->batch < 1 || plan->variant <= UW_VARIANT_AUTO || plan->variant >= UW_VARIANT_COUNT)
    return fail(UW_ERR_INVALID, "uw_set_plan: batch >= 1 and a concrete variant");
  if (!knob_valid(plan->variant, plan->knob)) return fail(UW_ERR_INVALID, "uw_set_plan: knob out of range for the variant");
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

}  // extern "C"

namespace {

// Run one (variant, knob) after the checks of runnable().  use_static:
// decompress + GEMM goes through the library's static scratch, band by band,
// instead of the workspace d_ws.
int run_variant(const uw_matrix* m, int variant, int knob, const void* d_X, int64_t batch, int64_t ldx, int xt,
                void* d_Y, int64_t ldy, int yt, void* d_ws, void* stream, bool use_static = false) {
  if (use_static && variant == UW_VARIANT_DECOMPRESS_GEMM)
    return static_decompress_gemm(m, d_X, batch, ldx, xt, d_Y, ldy, yt, knob, stream);
  switch (variant) {
    case UW_VARIANT_FUSED_MFMA: return launch_fused_mfma(m, d_X, batch, ldx, d_Y, ldy, yt, stream, knob);
    case UW_VARIANT_FUSED: return launch_fused(m, d_X, batch, ldx, xt, d_Y, ldy, yt, stream, knob);
    case UW_VARIANT_PALETTE: {
      const uw_palette* p = m->palette;
      if (batch == 1) return uw_palette_gemv(p, d_X, xt, d_Y, yt, stream);
      return uw_palette_gemm(p, d_X, batch, ldx, xt, d_Y, ldy, yt, stream);
    }
    default: {
      // decompress into the workspace, then the bf16 product
      uint16_t* W = static_cast<uint16_t*>(d_ws);
      if (int rc = launch_decompress(m, W, m->h.cols, stream)) return rc;
      return launch_bf16_gemm(W, m->h.rows, m->h.cols, m->h.cols, d_X, batch, ldx, xt, d_Y, ldy, yt, stream, knob & 31,
                              knob >> 5);
    }
  }
}

// AUTO without a usable plan: on VALU one row, and up to 8 when one pass
// takes them all with 16 waves per workgroup (gate_proj 24 / 29 / 39 us at 2
// / 4 / 8 rows against 41 on the matrix cores; 8192 x 8192 33 us at 4
// against 40; down_proj at 2 rows 31 against 39); up to 32 rows on the
// matrix cores; beyond that decompress + GEMM when the workspace is given
// (the measured crossovers on the MLP shapes: at 64 rows decompress + GEMM
// is ahead on down_proj).
int heuristic_variant(const uw_matrix* m, const CallShape& c) {
  const bool fused_ok = runnable(m, UW_VARIANT_FUSED, 0, c, nullptr);
  const bool mfma_ok = runnable(m, UW_VARIANT_FUSED_MFMA, 0, c, nullptr);
  const bool ws_ok = runnable(m, UW_VARIANT_DECOMPRESS_GEMM, 0, c, nullptr);
  const bool pal_ok = runnable(m, UW_VARIANT_PALETTE, 0, c, nullptr);
  const int64_t batch = c.batch;
  // an attached direct-palette copy: its GEMV at one batch row and its
  // matrix-core product up to 64 (MLP shapes, 8 cold copies: gate 20.3 /
  // 23.8 / 24.3 us at 1 / 2 / 4 rows against 21.0 / 24.2 / 28.2 for the fused
  // vector-ALU product, 25-45 at 8-64 against 38-87 for the fused products
  // and 56-65 for decompress + GEMM; down 20.5 / 22.3 against 23.8 / 30.9,
  // 30-70 at 16-64 against 42-77 and 65-76)
  if (pal_ok && batch <= 64) return UW_VARIANT_PALETTE;
  if (fused_ok && (batch == 1 || (batch == 2 && fused_rows_per_pass(m, batch, c.xt) >= 2) ||
                   (batch <= 8 && fused_one_full_pass(m, batch, c.xt))))
    return UW_VARIANT_FUSED;
  if (mfma_ok && (batch <= 32 || (batch <= 64 && !ws_ok))) return UW_VARIANT_FUSED_MFMA;
  if (ws_ok && (c.xt == UW_BF16 || !fused_ok)) return UW_VARIANT_DECOMPRESS_GEMM;
  if (mfma_ok) return UW_VARIANT_FUSED_MFMA;
  return fused_ok || !ws_ok ? UW_VARIANT_FUSED : UW_VARIANT_DECOMPRESS_GEMM;
}

int gemm_dispatch(const uw_matrix* m, int variant, int knob, const void* d_X, int64_t batch, int64_t ldx, int xt,
                  void* d_Y, int64_t ldy, int yt, void* d_ws, size_t ws_bytes, void* stream, const char* where,
                  bool use_static = false) {
  if (int rc = check_matrix(m)) return rc;
  if (int rc = check_products(d_X, batch, ldx, xt, d_Y, ldy, yt, m->h.rows, m->h.cols)) return rc;
  if (batch == 0) return UW_OK;
  // the static path: decompress + GEMM is runnable when a band of whole work
  // units fits in the scratch (a stand-in workspace descriptor stands for it;
  // it is never dereferenced: run_variant takes the static branch)
  alignas(256) static const uint8_t stand_in[256] = {0};
  if (use_static) {
    const bool fits = m->h.plain() || static_band_units(m) >= 1;
    d_ws = fits ? const_cast<uint8_t*>(stand_in) : nullptr;
    ws_bytes = fits ? decompress_ws_bytes(m) : 0;
  }
  const CallShape c{d_X, batch, ldx, xt, d_ws, ws_bytes};
  if (variant == UW_VARIANT_AUTO) {
    knob = 0;
    bool have = false;
    uw_plan p;
    {
      std::lock_guard<std::mutex> lk(m->mu);
      auto it = m->plans.find(batch);
      if (it != m->plans.end()) {
        p = it->second;
        have = true;
      }
    }
    // a stored plan is followed only when its variant can run this call (it
    // was tuned for bf16 X with a workspace; other operands fall back)
    if (have && runnable(m, p.variant, p.knob, c, nullptr)) {
      variant = p.variant;
      knob = p.knob;
    } else {
      variant = heuristic_variant(m, c);
    }
  }
  if (variant <= UW_VARIANT_AUTO || variant >= UW_VARIANT_COUNT)
    return fail(UW_ERR_INVALID, std::string(where) + ": unknown variant");
  if (!knob_valid(variant, knob)) return fail(UW_ERR_INVALID, std::string(where) + ": knob out of range");
  std::string why;
  if (!runnable(m, variant, knob, c, &why)) {
    if (use_static && variant == UW_VARIANT_DECOMPRESS_GEMM && why.rfind("workspace", 0) == 0)
      return fail(UW_ERR_UNSUPPORTED, std::string(where) + ": one work unit of this matrix does not fit in the " +
                                          std::to_string(static_scratch_bytes() >> 20) + " MiB scratch");
    const bool space = variant == UW_VARIANT_DECOMPRESS_GEMM && why.rfind("workspace", 0) == 0;
    return fail(space ? UW_ERR_NOSPACE : UW_ERR_UNSUPPORTED, std::string(where) + ": " + why);
  }
  return run_variant(m, variant, knob, d_X, batch, ldx, xt, d_Y, ldy, yt, d_ws, stream, use_static);
}

}  // namespace

extern "C" {

int uw_gemm_fused(const uw_matrix* m, const void* d_X, int64_t batch, int64_t ldx, int xt, void* d_Y, int64_t ldy,
                  int yt, int variant, void* d_ws, size_t ws_bytes, void* stream) {
  if (variant < 0 || variant >= UW_VARIANT_COUNT) return fail(UW_ERR_INVALID, "uw_gemm_fused: unknown variant");
  return gemm_dispatch(m, variant, 0, d_X, batch, ldx, xt, d_Y, ldy, yt, d_ws, ws_bytes, stream, "uw_gemm_fused");
}

int uw_gemm_fused_static(const uw_matrix* m, const void* d_X, int64_t batch, int64_t ldx, int xt, void* d_Y,
                         int64_t ldy, int yt, int variant, void* stream) {
  if (variant < 0 || variant >= UW_VARIANT_COUNT) return fail(UW_ERR_INVALID, "uw_gemm_fused_static: unknown variant");
  return gemm_dispatch(m, variant, 0, d_X, batch, ldx, xt, d_Y, ldy, yt, nullptr, 0, stream, "uw_gemm_fused_static",
                       true);
}

int uw_gemm_with_plan(const uw_matrix* m, const uw_plan* plan, const void* d_X, int64_t batch, int64_t ldx, int xt,
                      void* d_Y, int64_t ldy, int yt, void* d_ws, size_t ws_bytes, void* stream) {
  if (!plan) return fail(UW_ERR_INVALID, "uw_gemm_with_plan: null plan");
  if (plan->variant <= UW_VARIANT_AUTO || plan->variant >= UW_VARIANT_COUNT)
    return fail(UW_ERR_INVALID, "uw_gemm_with_plan: a concrete variant is needed");
  return gemm_dispatch(m, plan->variant, plan->knob, d_X, batch, ldx, xt, d_Y, ldy, yt, d_ws, ws_bytes, stream,
                       "uw_gemm_with_plan");
}

size_t uw_autotune_scratch_size(const uw_matrix* m, int64_t batch) {
  if (!m || batch < 0) return 0;
  const size_t xb = align256(size_t(batch) * size_t(m->h.cols) * 2);
  const size_t yb = align256(size_t(batch) * size_t(m->h.rows) * 2);
  return xb + yb + kFlushBytes;
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
  void* Y = base + need_ws + align256(size_t(batch) * size_t(m->h.cols) * 2);
  void* flush = static_cast<char*>(Y) + align256(size_t(batch) * size_t(m->h.rows) * 2);
  // X = 1.0 everywhere (values do not change the work of any candidate); the
  // probe's checksum words land in the first bytes of Y, which the timed
  // calls overwrite
  if (hipMemsetD16Async(reinterpret_cast<hipDeviceptr_t>(X), 0x3F80, size_t(batch) * size_t(m->h.cols), s) != hipSuccess)
    return fail(UW_ERR_HIP, "uw_autotune: memset failed");
  // the probe reads the region but its last sink bytes, where it writes its checksums
  const size_t flush_read = kFlushBytes - align256(read_probe_sink_bytes());
  void* sink = static_cast<char*>(flush) + flush_read;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return fail(UW_ERR_HIP, "uw_autotune: event");
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return fail(UW_ERR_HIP, "uw_autotune: event");
  }
  uw_plan plan;
  std::memset(&plan, 0, sizeof(plan));
  plan.batch = batch;
  for (int v = 0; v < UW_VARIANT_COUNT; ++v) {
    plan.candidate_us[v] = -1.f;
    plan.candidate_knob[v] = 0;
  }
  // candidates: every variant with the knobs that matter at this batch
  std::vector<std::pair<int, int>> cands;
  if (batch <= 16) {
    cands.push_back({UW_VARIANT_FUSED, 0});
    if (m->dev.flat) {
      cands.push_back({UW_VARIANT_FUSED, 2});
      cands.push_back({UW_VARIANT_FUSED, 4});
    }
  }
  for (int nw : {0, 8, 12, 16}) cands.push_back({UW_VARIANT_FUSED_MFMA, nw});
  if (batch == 1) {
    cands.push_back({UW_VARIANT_DECOMPRESS_GEMM, 0});
  } else if (batch <= 8) {
    for (int k : {0, 2 + 32 * 2, 1 + 32 * 4}) cands.push_back({UW_VARIANT_DECOMPRESS_GEMM, k});
  } else {
    // GEMM shape + 32 * waves splitting k (0 = the kernel's own pick)
    const std::vector<int> knobs = batch <= 16   ? std::vector<int>{1 + 32 * 4, 2, 15}
                                   : batch <= 32 ? std::vector<int>{4 + 32 * 4, 8, 15, 17, 18}
                                   : batch <= 64 ? std::vector<int>{4 + 32 * 4, 6, 15, 17, 18}
                                                 : std::vector<int>{16, 15, 14};
    for (int k : knobs) cands.push_back({UW_VARIANT_DECOMPRESS_GEMM, k});
  }
  cands.push_back({UW_VARIANT_PALETTE, 0});
  const CallShape c{X, batch, int64_t(m->h.cols), UW_BF16, d_ws, need_ws};
  float best = 1e30f;
  int best_v = -1, best_k = 0;
  const int warm = 3, reps = 15;
  int rc = UW_OK;
  for (const auto& [v, knob] : cands) {
    if (!runnable(m, v, knob, c, nullptr)) continue;
    std::vector<float> t;
    for (int i = 0; i < warm + reps && rc == UW_OK; ++i) {
      // evict the blob: read 512 MiB that are not the matrix
      if (i >= warm && (rc = launch_read_probe(flush, flush_read, sink, s))) break;
      if (hipEventRecord(e0, s) != hipSuccess) rc = fail(UW_ERR_HIP, "uw_autotune: event record");
      if (rc == UW_OK)
        rc = run_variant(m, v, knob, X, batch, int64_t(m->h.cols), UW_BF16, Y, int64_t(m->h.rows), UW_BF16, d_ws, stream);
      if (rc == UW_OK && hipEventRecord(e1, s) != hipSuccess) rc = fail(UW_ERR_HIP, "uw_autotune: event record");
      if (rc == UW_OK && hipEventSynchronize(e1) != hipSuccess) rc = fail(UW_ERR_HIP, "uw_autotune: synchronize");
      float ms = 0;
      if (rc == UW_OK) (void)hipEventElapsedTime(&ms, e0, e1);
      if (rc == UW_OK && i >= warm) t.push_back(ms * 1000.f);
    }
    if (rc != UW_OK) break;
    std::sort(t.begin(), t.end());
    const float med = t[t.size() / 2];
    if (plan.candidate_us[v] < 0 || med < plan.candidate_us[v]) {
      plan.candidate_us[v] = med;
      plan.candidate_knob[v] = knob;
    }
    if (med < best) {
      best = med;
      best_v = v;
      best_k = knob;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (rc != UW_OK) return rc;
  if (best_v < 0) return fail(UW_ERR_UNSUPPORTED, "uw_autotune: no candidate can run this matrix and batch");
  plan.variant = best_v;
  plan.knob = best_k;
  plan.time_us = best;
  {
    std::lock_guard<std::mutex> lk(m->mu);
    m->plans[batch] = plan;
  }
  if (out) *out = plan;
  set_error("");
  return UW_OK;
}

// ---- plan files (JSON) ------------------------------------------------------

int uw_plan_save(const uw_matrix* m, char* out, size_t* out_size) {
  if (!m || !out_size) return fail(UW_ERR_INVALID, "uw_plan_save: null pointer");
  std::string j = "{\"format\": \"uw-plan-1\", \"rows\": " + std::to_string(m->h.rows) +
                  ", \"cols\": " + std::to_string(m->h.cols) + ", \"blob_crc32\": " + std::to_string(blob_crc(m)) +
                  ", \"plans\": [";
  {
    std::lock_guard<std::mutex> lk(m->mu);
    bool first = true;
    for (const auto& [b, p] : m->plans) {
      char buf[256];
      std::snprintf(buf, sizeof buf, "%s{\"batch\": %lld, \"variant\": \"%s\", \"knob\": %d, \"time_us\": %.3f}",
                    first ? "" : ", ", static_cast<long long>(b), variant_name(p.variant), int(p.knob),
                    double(p.time_us));
      j += buf;
      first = false;
    }
  }
  j += "]}";
  const size_t need = j.size() + 1;
  if (!out) {
    *out_size = need;
    return UW_OK;
  }
  if (*out_size < need) {
    *out_size = need;
    return fail(UW_ERR_NOSPACE, "uw_plan_save: output buffer too small");
  }
  std::memcpy(out, j.c_str(), need);
  *out_size = need;
  return UW_OK;
}

}  // extern "C"

namespace {
// A reader for the JSON uw_plan_save writes (objects, arrays, strings without
// escapes, numbers); anything else is a format error.
struct Json {
  const char* p;
  bool ok = true;
  void ws() {
    while (*p == ' ' || *p == '\n' || *p == '\t' || *p == '\r') ++p;
  }
  bool eat(char c) {
    ws();
    if (*p != c) return false;
    ++p;
    return true;
  }
  std::string str() {
    ws();
    std::string r;
    if (*p != '"') {
      ok = false;
      return r;
    }
    ++p;
    while (*p && *p != '"') {
      if (*p == '\\') {
        ok = false;
        return r;
      }
      r += *p++;
    }
    if (*p != '"') ok = false;
    else ++p;
    return r;
  }
  double num() {
    ws();
    char* end = nullptr;
    const double v = std::strtod(p, &end);
    if (end == p) ok = false;
    p = end ? end : p;
    return v;
  }
};

int variant_of(const std::string& n) {
  for (int v = UW_VARIANT_FUSED; v < UW_VARIANT_COUNT; ++v)
    if (n == variant_name(v)) return v;
  return -1;
}
}  // namespace

extern "C" {

int uw_plan_load(uw_matrix* m, const char* json) {
  if (!m || !json) return fail(UW_ERR_INVALID, "uw_plan_load: null pointer");
  Json r{json};
  double rows = -1, cols = -1, crc = -1;
  std::string format;
  std::vector<uw_plan> plans;
  if (!r.eat('{')) return fail(UW_ERR_FORMAT, "uw_plan_load: not a JSON object");
  bool more = !r.eat('}');
  while (more && r.ok) {
    const std::string key = r.str();
    if (!r.ok || !r.eat(':')) return fail(UW_ERR_FORMAT, "uw_plan_load: expected a key");
    if (key == "format") format = r.str();
    else if (key == "rows") rows = r.num();
    else if (key == "cols") cols = r.num();
    else if (key == "blob_crc32") crc = r.num();
    else if (key == "plans") {
      if (!r.eat('[')) return fail(UW_ERR_FORMAT, "uw_plan_load: plans must be an array");
      bool items = !r.eat(']');
      while (items && r.ok) {
        if (!r.eat('{')) return fail(UW_ERR_FORMAT, "uw_plan_load: a plan must be an object");
        uw_plan p;
        std::memset(&p, 0, sizeof(p));
        p.batch = -1;
        p.variant = -1;
        for (int v = 0; v < UW_VARIANT_COUNT; ++v) p.candidate_us[v] = -1.f;
        bool fields = !r.eat('}');
        while (fields && r.ok) {
          const std::string k = r.str();
          if (!r.ok || !r.eat(':')) return fail(UW_ERR_FORMAT, "uw_plan_load: expected a plan field");
          if (k == "batch") p.batch = int64_t(r.num());
          else if (k == "variant") p.variant = variant_of(r.str());
          else if (k == "knob") p.knob = int32_t(r.num());
          else if (k == "time_us") p.time_us = float(r.num());
          else return fail(UW_ERR_FORMAT, "uw_plan_load: unknown plan field " + k);
          fields = r.eat(',');
          if (!fields && !r.eat('}')) return fail(UW_ERR_FORMAT, "uw_plan_load: unterminated plan");
        }
        if (!r.ok || p.batch < 1 || p.variant <= UW_VARIANT_AUTO || !knob_valid(p.variant, p.knob))
          return fail(UW_ERR_FORMAT, "uw_plan_load: invalid plan entry");
        plans.push_back(p);
        items = r.eat(',');
        if (!items && !r.eat(']')) return fail(UW_ERR_FORMAT, "uw_plan_load: unterminated plans");
      }
    } else {
      return fail(UW_ERR_FORMAT, "uw_plan_load: unknown key " + key);
    }
    more = r.eat(',');
    if (!more && !r.eat('}')) return fail(UW_ERR_FORMAT, "uw_plan_load: unterminated object");
  }
  if (!r.ok || format != "uw-plan-1") return fail(UW_ERR_FORMAT, "uw_plan_load: not a uw-plan-1 document");
  if (rows != double(m->h.rows) || cols != double(m->h.cols) || crc != double(blob_crc(m)))
    return fail(UW_ERR_FORMAT, "uw_plan_load: the plans belong to another matrix (rows, cols or blob CRC differ)");
  std::lock_guard<std::mutex> lk(m->mu);
  for (const uw_plan& p : plans) m->plans[p.batch] = p;
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

int uw_bf16_gemm_shaped(const uint16_t* d_W, int64_t rows, int64_t cols, int64_t ldw, const void* d_X, int64_t batch,
                        int64_t ldx, void* d_Y, int64_t ldy, int yt, int shape, int ks, void* stream) {
  if (!d_W || !aligned(d_W, 16)) return fail(UW_ERR_INVALID, "uw_bf16_gemm_shaped: W must be non-null and 16-byte aligned");
  if (rows < 1 || cols < 8 || cols % 8 || ldw < cols || ldw % 8)
    return fail(UW_ERR_INVALID, "uw_bf16_gemm_shaped: bad shape");
  if (int rc = check_products(d_X, batch, ldx, UW_BF16, d_Y, ldy, yt, rows, cols)) return rc;
  if (batch < 1 || !aligned(d_X, 16) || ldx % 8)
    return fail(UW_ERR_INVALID, "uw_bf16_gemm_shaped: batch >= 1, X 16-byte aligned and ldx a multiple of 8");
  if (shape < 1 || shape >= mfma_gemm_shape_count() || !(ks == 0 || ks == 1 || ks == 2 || ks == 4 || ks == 8))
    return fail(UW_ERR_INVALID, "uw_bf16_gemm_shaped: unknown shape or ks");
  return launch_mfma_gemm(d_W, rows, cols, ldw, static_cast<const uint16_t*>(d_X), batch, ldx, d_Y, ldy, yt, shape, ks,
                          stream);
}

int uw_bf16_gemm_shape_count(void) { return mfma_gemm_shape_count(); }

size_t uw_palette_transcode_size(const uw_matrix* m) {
  if (!m || !palette_transcodable(m, nullptr)) return 0;
  return transcode_layout(m).total;
}

int uw_palette_transcode(const uw_matrix* m, void* d_out, size_t out_bytes, void* stream) {
  if (int rc = check_matrix(m)) return rc;
  std::string why;
  if (!palette_transcodable(m, &why)) return fail(UW_ERR_UNSUPPORTED, "uw_palette_transcode: " + why);
  if (!d_out || !aligned(d_out, 256)) return fail(UW_ERR_INVALID, "uw_palette_transcode: output must be 256-byte aligned");
  if (out_bytes < transcode_layout(m).total) return fail(UW_ERR_NOSPACE, "uw_palette_transcode: output too small");
  return launch_palette_transcode(m, static_cast<uint8_t*>(d_out), stream);
}

int uw_palette_create_transcoded(const uw_matrix* m, const void* d_blob, uw_palette** out) {
  if (!m || !d_blob || !out) return fail(UW_ERR_INVALID, "uw_palette_create_transcoded: null pointer");
  if (!aligned(d_blob, 256)) return fail(UW_ERR_INVALID, "uw_palette_create_transcoded: blob must be 256-byte aligned");
  std::string why;
  if (!palette_transcodable(m, &why)) return fail(UW_ERR_UNSUPPORTED, "uw_palette_create_transcoded: " + why);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(UW_ERR_HIP, "uw_palette_create_transcoded: no current HIP device");
  uw_palette* p = new uw_palette;
  p->l = transcode_layout(m);
  p->d_blob = static_cast<const uint8_t*>(d_blob);
  p->device = dev;
  *out = p;
  return UW_OK;
}

size_t uw_read_probe_sink_size(void) { return read_probe_sink_bytes(); }

int uw_read_probe(const void* d_src, size_t bytes, void* d_sink, void* stream) {
  if (!d_src || !d_sink || !aligned(d_src, 16) || !aligned(d_sink, 4) || bytes % 16 || bytes == 0)
    return fail(UW_ERR_INVALID, "uw_read_probe: bad arguments");
  return launch_read_probe(d_src, bytes, d_sink, stream);
}

}  // extern "C"
