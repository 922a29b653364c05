// Host side of the direct-palette form (format UWP1): the encoder and the
// header parser.
//
// "Unweight: how we compressed an LLM 22% without sacrificing quality",
// section on the four execution pipelines: the direct-palette pipeline turns
// the weights into 4-bit palette indices when the model is loaded, and the
// matmul rebuilds bf16 from them with no preprocessing pass.  The palette is
// the 16 most frequent exponents and 64-weight groups holding any other
// exponent are kept raw (paragraph on rare exponents), the same rule as the
// Huffman form's.  Layout (little-endian, every section 256-byte aligned):
//   header 64 B: "UWP1", u32 version, u64 rows, u64 cols, u64 n_raw,
//                u8 palette[16], u32 n_pal, zeros
//   sm     1 byte per weight, (sign << 7) | mantissa, row-major
//   idx    4 bits per weight: weight i in the low nibble of byte i/2 if i is
//          even, else the high nibble; 0 inside raw groups
//   flags  1 bit per 64-weight group (bit g%32 of word g/32): raw
//   prefix u32 per 1024-weight tile: raw groups before the tile
//   raw    64 exponent bytes per raw group, in group order
#include <algorithm>
#include <cstring>
#include <vector>

#include "uw_internal.h"

namespace uw {

namespace {

inline size_t align256(size_t n) { return (n + 255) / 256 * 256; }

void put_u32(uint8_t* p, uint32_t v) { std::memcpy(p, &v, 4); }
void put_u64(uint8_t* p, uint64_t v) { std::memcpy(p, &v, 8); }
uint32_t get_u32(const uint8_t* p) {
  uint32_t v;
  std::memcpy(&v, p, 4);
  return v;
}
uint64_t get_u64(const uint8_t* p) {
  uint64_t v;
  std::memcpy(&v, p, 8);
  return v;
}

}  // namespace

PaletteLayout palette_layout(int64_t rows, int64_t cols, int64_t n_raw) {
  PaletteLayout l;
  l.rows = rows;
  l.cols = cols;
  l.n_raw = n_raw;
  const size_t n = size_t(rows) * size_t(cols);
  l.off_sm = align256(kPaletteHeaderBytes);
  l.off_idx = align256(l.off_sm + n);
  l.off_flags = align256(l.off_idx + n / 2);
  l.off_prefix = align256(l.off_flags + 4 * ((n / 64 + 31) / 32));
  l.off_raw = align256(l.off_prefix + 4 * (n / 1024));
  l.total = align256(l.off_raw + 64 * size_t(n_raw));
  return l;
}

int palette_parse(const void* blob, size_t n, PaletteLayout* out) {
  const uint8_t* b = static_cast<const uint8_t*>(blob);
  if (!blob || n < kPaletteHeaderBytes) return fail(UW_ERR_FORMAT, "palette blob: shorter than its header");
  if (std::memcmp(b, "UWP1", 4) != 0 || get_u32(b + 4) != 1) return fail(UW_ERR_FORMAT, "palette blob: bad magic");
  const int64_t rows = int64_t(get_u64(b + 8)), cols = int64_t(get_u64(b + 16));
  const int64_t n_raw = int64_t(get_u64(b + 24));
  const uint32_t n_pal = get_u32(b + 48);
  if (rows < 1 || cols < 1024 || cols % 1024 || rows > (int64_t(1) << 40) / cols || n_pal < 1 || n_pal > 16 ||
      n_raw < 0 || n_raw > rows * cols / 64)
    return fail(UW_ERR_FORMAT, "palette blob: bad header fields");
  PaletteLayout l = palette_layout(rows, cols, n_raw);
  if (l.total != n) return fail(UW_ERR_FORMAT, "palette blob: size does not match the header");
  l.n_pal = int(n_pal);
  std::memcpy(l.palette, b + 32, 16);
  // the flags must count n_raw raw groups and the prefixes must add them up
  const size_t groups = size_t(rows) * size_t(cols) / 64;
  int64_t seen = 0;
  for (size_t t = 0; t < groups / 16; ++t) {
    if (get_u32(b + l.off_prefix + 4 * t) != uint64_t(seen))
      return fail(UW_ERR_FORMAT, "palette blob: tile prefix counts disagree with the raw flags");
    const uint32_t w = get_u32(b + l.off_flags + 4 * (t / 2));
    seen += __builtin_popcount((w >> (16 * (t & 1))) & 0xFFFFu);
  }
  if (seen != n_raw) return fail(UW_ERR_FORMAT, "palette blob: raw flags disagree with the header");
  *out = l;
  return UW_OK;
}

}  // namespace uw

using namespace uw;

extern "C" int uw_palette_encode(const uint16_t* w, int64_t rows, int64_t cols, void* out, size_t* out_size) {
  if (!w || !out_size) return fail(UW_ERR_INVALID, "uw_palette_encode: null pointer");
  if (rows < 1 || cols < 1024 || cols % 1024 || rows > (int64_t(1) << 40) / cols)
    return fail(UW_ERR_INVALID, "uw_palette_encode: cols must be a positive multiple of 1024");
  const size_t n = size_t(rows) * size_t(cols);
  // exponent histogram and the top 16 (count descending, exponent ascending)
  std::vector<uint64_t> hist(256, 0);
  for (size_t i = 0; i < n; ++i) ++hist[(w[i] >> 7) & 0xFF];
  std::vector<int> present;
  for (int e = 0; e < 256; ++e)
    if (hist[e]) present.push_back(e);
  std::sort(present.begin(), present.end(), [&](int a, int b) { return hist[a] != hist[b] ? hist[a] > hist[b] : a < b; });
  const int n_pal = int(std::min<size_t>(16, present.size()));
  int index_of[256];
  std::fill(index_of, index_of + 256, -1);
  for (int i = 0; i < n_pal; ++i) index_of[present[i]] = i;
  // raw groups: any exponent outside the palette
  const size_t groups = n / 64;
  std::vector<uint8_t> raw(groups, 0);
  int64_t n_raw = 0;
  for (size_t g = 0; g < groups; ++g) {
    for (size_t k = 0; k < 64 && !raw[g]; ++k) raw[g] = index_of[(w[64 * g + k] >> 7) & 0xFF] < 0;
    n_raw += raw[g];
  }
  if (n_raw > int64_t(UINT32_MAX)) return fail(UW_ERR_INVALID, "uw_palette_encode: too many raw groups");
  const PaletteLayout l = palette_layout(rows, cols, n_raw);
  if (!out) {
    *out_size = l.total;
    return UW_OK;
  }
  if (*out_size < l.total) {
    *out_size = l.total;
    return fail(UW_ERR_NOSPACE, "uw_palette_encode: output buffer too small");
  }
  uint8_t* b = static_cast<uint8_t*>(out);
  std::memset(b, 0, l.total);
  std::memcpy(b, "UWP1", 4);
  put_u32(b + 4, 1);
  put_u64(b + 8, uint64_t(rows));
  put_u64(b + 16, uint64_t(cols));
  put_u64(b + 24, uint64_t(n_raw));
  for (int i = 0; i < n_pal; ++i) b[32 + i] = uint8_t(present[i]);
  put_u32(b + 48, uint32_t(n_pal));
  for (size_t i = 0; i < n; ++i) {
    const uint16_t v = w[i];
    b[l.off_sm + i] = uint8_t(((v >> 8) & 0x80) | (v & 0x7F));
    if (!raw[i / 64]) b[l.off_idx + i / 2] |= uint8_t(index_of[(v >> 7) & 0xFF] << (4 * (i & 1)));
  }
  int64_t k = 0;
  for (size_t g = 0; g < groups; ++g) {
    if (g % 16 == 0) put_u32(b + l.off_prefix + 4 * (g / 16), uint32_t(k));
    if (!raw[g]) continue;
    b[l.off_flags + 4 * (g / 32) + (g % 32) / 8] |= uint8_t(1u << (g % 8));
    for (size_t j = 0; j < 64; ++j) b[l.off_raw + 64 * size_t(k) + j] = uint8_t((w[64 * g + j] >> 7) & 0xFF);
    ++k;
  }
  *out_size = l.total;
  return UW_OK;
}
