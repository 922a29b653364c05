// Blob header I/O, CRC-32 and full validation of a compressed matrix.
//
// The blob carries the pieces the Unweight design needs ("Unweight: how we
// compressed an LLM 22% without sacrificing quality"): raw sign+mantissa
// bytes, Huffman-coded exponent bytes (paragraph on Huffman coding of the
// exponent byte) and raw rows of 64 for rare exponents (paragraph on rare
// exponents).  Validation runs on the host before any kernel sees the blob,
// so a corrupt or truncated blob is an error code, never a device fault.
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "uw_internal.h"

namespace uw {

namespace {
thread_local std::string g_err;

template <class T>
void put(uint8_t* dst, size_t off, T v) { std::memcpy(dst + off, &v, sizeof(T)); }
template <class T>
T get(const uint8_t* src, size_t off) { T v; std::memcpy(&v, src + off, sizeof(T)); return v; }

uint32_t g_crc_table[8][256];
std::once_flag g_crc_once;

void crc_init() {
  for (uint32_t i = 0; i < 256; ++i) {
    uint32_t c = i;
    for (int k = 0; k < 8; ++k) c = (c & 1) ? (0xEDB88320u ^ (c >> 1)) : (c >> 1);
    g_crc_table[0][i] = c;
  }
  for (uint32_t i = 0; i < 256; ++i)
    for (int t = 1; t < 8; ++t)
      g_crc_table[t][i] = (g_crc_table[t - 1][i] >> 8) ^ g_crc_table[0][g_crc_table[t - 1][i] & 0xFF];
}
}  // namespace

void set_error(const std::string& msg) { g_err = msg; }
const char* last_error_text() { return g_err.c_str(); }
int fail(int status, const std::string& msg) { g_err = msg; return status; }

uint32_t crc32(const uint8_t* p, size_t n, uint32_t crc) {
  std::call_once(g_crc_once, crc_init);
  crc = ~crc;
  // slicing by 8: eight table lookups per 8 input bytes
  while (n >= 8) {
    uint32_t a, b;
    std::memcpy(&a, p, 4);
    std::memcpy(&b, p + 4, 4);
    a ^= crc;
    crc = g_crc_table[7][a & 0xFF] ^ g_crc_table[6][(a >> 8) & 0xFF] ^ g_crc_table[5][(a >> 16) & 0xFF] ^
          g_crc_table[4][a >> 24] ^ g_crc_table[3][b & 0xFF] ^ g_crc_table[2][(b >> 8) & 0xFF] ^
          g_crc_table[1][(b >> 16) & 0xFF] ^ g_crc_table[0][b >> 24];
    p += 8;
    n -= 8;
  }
  while (n--) crc = g_crc_table[0][(crc ^ *p++) & 0xFF] ^ (crc >> 8);
  return ~crc;
}

void header_write(const BlobHeader& h, uint8_t* d) {
  std::memset(d, 0, kHeaderBytes);
  std::memcpy(d, "UWB1", 4);
  put<uint32_t>(d, 4, 1);
  put<uint32_t>(d, 8, kHeaderBytes);
  put<uint32_t>(d, 12, h.flags);
  put<int64_t>(d, 16, h.rows);
  put<int64_t>(d, 24, h.cols);
  put<uint32_t>(d, 32, h.K);
  put<uint32_t>(d, 36, h.L);
  put<uint32_t>(d, 40, h.G);
  put<uint32_t>(d, 44, h.n_blocks);
  put<uint64_t>(d, 48, h.n_raw_groups);
  put<uint64_t>(d, 56, h.total_bytes);
  put<uint32_t>(d, 64, h.crc32);
  put<uint32_t>(d, 68, h.max_block_stream_bytes);
  std::memcpy(d + 72, h.palette, 32);
  std::memcpy(d + 104, h.code_len, 32);
  const uint64_t offs[12] = {h.off_start_word, h.off_first_raw, h.off_raw_bits, h.off_lane_bits,
                             h.off_stream, h.size_stream, h.off_raw, h.size_raw,
                             h.off_sm, h.size_sm, h.off_plain, h.size_plain};
  for (int i = 0; i < 12; ++i) put<uint64_t>(d, 136 + 8 * i, offs[i]);
}

void header_read(const uint8_t* s, BlobHeader* h) {
  h->version = get<uint32_t>(s, 4);
  h->flags = get<uint32_t>(s, 12);
  h->rows = get<int64_t>(s, 16);
  h->cols = get<int64_t>(s, 24);
  h->K = get<uint32_t>(s, 32);
  h->L = get<uint32_t>(s, 36);
  h->G = get<uint32_t>(s, 40);
  h->n_blocks = get<uint32_t>(s, 44);
  h->n_raw_groups = get<uint64_t>(s, 48);
  h->total_bytes = get<uint64_t>(s, 56);
  h->crc32 = get<uint32_t>(s, 64);
  h->max_block_stream_bytes = get<uint32_t>(s, 68);
  std::memcpy(h->palette, s + 72, 32);
  std::memcpy(h->code_len, s + 104, 32);
  uint64_t* offs[12] = {&h->off_start_word, &h->off_first_raw, &h->off_raw_bits, &h->off_lane_bits,
                        &h->off_stream, &h->size_stream, &h->off_raw, &h->size_raw,
                        &h->off_sm, &h->size_sm, &h->off_plain, &h->size_plain};
  for (int i = 0; i < 12; ++i) *offs[i] = get<uint64_t>(s, 136 + 8 * i);
}

void canonical_codes(const BlobHeader& h, uint32_t code[32], uint32_t rev[32]) {
  // RFC 1951 3.2.2: count codes per length, first code of each length, then
  // hand out consecutive codes to the symbols of a length in exponent order.
  int count[kMaxL + 2] = {0};
  for (uint32_t i = 0; i < h.K; ++i) count[h.code_len[i]]++;
  count[0] = 0;
  uint32_t next[kMaxL + 2] = {0};
  uint32_t c = 0;
  for (int len = 1; len <= kMaxL; ++len) {
    c = (c + count[len - 1]) << 1;
    next[len] = c;
  }
  int order[32];
  for (uint32_t i = 0; i < h.K; ++i) order[i] = int(i);
  std::sort(order, order + h.K, [&](int a, int b) { return h.palette[a] < h.palette[b]; });
  for (uint32_t t = 0; t < h.K; ++t) {
    int i = order[t];
    int len = h.code_len[i];
    code[i] = rev[i] = 0;
    if (!len) continue;
    code[i] = next[len]++;
    uint32_t r = 0;
    for (int b = 0; b < len; ++b) r |= ((code[i] >> b) & 1u) << (len - 1 - b);
    rev[i] = r;
  }
}

namespace {
bool section_ok(uint64_t off, uint64_t size, size_t n) {
  return off % kSectionAlign == 0 && off >= kHeaderBytes && off <= n && size <= n - off;
}
}  // namespace

int validate_blob(const uint8_t* b, size_t n, BlobHeader* out) {
  if (!b) return fail(UW_ERR_INVALID, "null blob");
  if (n < kHeaderBytes) return fail(UW_ERR_FORMAT, "blob shorter than its 256-byte header");
  if (std::memcmp(b, "UWB1", 4) != 0) return fail(UW_ERR_FORMAT, "bad magic");
  BlobHeader h;
  header_read(b, &h);
  if (h.version != 1) return fail(UW_ERR_FORMAT, "unsupported version");
  if (get<uint32_t>(b, 8) != kHeaderBytes) return fail(UW_ERR_FORMAT, "bad header size");
  if (h.total_bytes != n) return fail(UW_ERR_FORMAT, "total_bytes does not match the blob size");
  if (h.flags & ~kFlagPlain) return fail(UW_ERR_FORMAT, "unknown flags");
  if (h.rows < 1 || h.cols < 64 || h.cols % 64 || h.rows > (int64_t(1) << 40) / h.cols)
    return fail(UW_ERR_FORMAT, "bad shape");
  if (crc32(b + kHeaderBytes, n - kHeaderBytes) != h.crc32) return fail(UW_ERR_FORMAT, "CRC mismatch");
  const uint64_t weights = uint64_t(h.rows) * uint64_t(h.cols);
  if (h.plain()) {
    if (h.size_plain != 2 * weights || !section_ok(h.off_plain, h.size_plain, n) || h.off_plain % 256)
      return fail(UW_ERR_FORMAT, "bad plain section");
    *out = h;
    return UW_OK;
  }
  if (h.K < 1 || h.K > kMaxK || h.L < 1 || h.L > kMaxL || h.K > (1u << h.L))
    return fail(UW_ERR_FORMAT, "bad K/L");
  if (h.G < 16 || h.G > 1024 || h.G % 16) return fail(UW_ERR_FORMAT, "bad G");
  const uint64_t n_groups = weights / 64;
  if (h.n_blocks != (n_groups + h.G - 1) / h.G) return fail(UW_ERR_FORMAT, "bad block count");
  // palette distinct; lengths form a complete prefix code (or one 1-bit code)
  uint32_t seen[8] = {0};
  int coded = 0, minlen = 99, maxlen = 0;
  uint64_t kraft = 0;  // in units of 2^-L
  for (uint32_t i = 0; i < h.K; ++i) {
    uint8_t e = h.palette[i];
    if (seen[e >> 5] & (1u << (e & 31))) return fail(UW_ERR_FORMAT, "repeated palette entry");
    seen[e >> 5] |= 1u << (e & 31);
    int len = h.code_len[i];
    if (len > int(h.L)) return fail(UW_ERR_FORMAT, "code length above L");
    if (len) {
      coded++;
      minlen = std::min(minlen, len);
      maxlen = std::max(maxlen, len);
      kraft += uint64_t(1) << (h.L - len);
    }
  }
  if (coded == 0) return fail(UW_ERR_FORMAT, "no coded symbol");
  if (coded == 1 ? (maxlen != 1) : (kraft != (uint64_t(1) << h.L)))
    return fail(UW_ERR_FORMAT, "code lengths are not a complete prefix code");
  const uint64_t nb = h.n_blocks;
  const uint64_t W = (h.G + 31) / 32;
  if (!section_ok(h.off_start_word, 4 * (nb + 1), n) || !section_ok(h.off_first_raw, 4 * (nb + 1), n) ||
      !section_ok(h.off_raw_bits, 4 * nb * W, n) || !section_ok(h.off_lane_bits, 128 * nb, n) ||
      !section_ok(h.off_stream, h.size_stream, n) || !section_ok(h.off_raw, h.size_raw, n) ||
      !section_ok(h.off_sm, h.size_sm, n) || h.size_stream % 16)
    return fail(UW_ERR_FORMAT, "section out of bounds or misaligned");
  const uint64_t g_last = n_groups - (nb - 1) * h.G;
  if (h.size_sm != (nb - 1) * uint64_t(h.G) * 64 + (g_last + 15) / 16 * 1024)
    return fail(UW_ERR_FORMAT, "bad sm section size");
  if (h.size_raw != 64 * h.n_raw_groups) return fail(UW_ERR_FORMAT, "bad raw section size");
  std::vector<uint32_t> sw(nb + 1), fr(nb + 1), rb(nb * W);
  std::memcpy(sw.data(), b + h.off_start_word, 4 * (nb + 1));
  std::memcpy(fr.data(), b + h.off_first_raw, 4 * (nb + 1));
  std::memcpy(rb.data(), b + h.off_raw_bits, 4 * nb * W);
  const uint16_t* lb = reinterpret_cast<const uint16_t*>(b + h.off_lane_bits);
  if (sw[0] != 0 || fr[0] != 0 || uint64_t(sw[nb]) * 4 != h.size_stream || fr[nb] != h.n_raw_groups)
    return fail(UW_ERR_FORMAT, "bad block table ends");
  uint32_t max_stream = 0;
  for (uint64_t blk = 0; blk < nb; ++blk) {
    const uint64_t gb = (blk + 1 == nb) ? g_last : h.G;
    if (sw[blk + 1] < sw[blk] || (sw[blk + 1] - sw[blk]) % 4) return fail(UW_ERR_FORMAT, "bad start_word");
    uint32_t nraw = 0;
    for (uint64_t w = 0; w < W; ++w) {
      uint32_t bits = rb[blk * W + w];
      const uint64_t lo = 32 * w;
      if (lo + 32 > gb) {
        uint32_t valid = gb > lo ? uint32_t(gb - lo) : 0;
        if (valid < 32 && (bits >> valid)) return fail(UW_ERR_FORMAT, "raw bit beyond the block");
      }
      nraw += __builtin_popcount(bits);
    }
    if (fr[blk + 1] != fr[blk] + nraw) return fail(UW_ERR_FORMAT, "first_raw inconsistent with raw bits");
    const uint64_t coded_groups = gb - nraw;
    uint64_t total = 0;
    for (int l = 0; l < 64; ++l) {
      uint64_t bits = lb[blk * 64 + l];
      if (bits < coded_groups * uint64_t(minlen) || bits > coded_groups * uint64_t(maxlen))
        return fail(UW_ERR_FORMAT, "lane bit count out of range");
      total += bits;
    }
    const uint64_t words = sw[blk + 1] - sw[blk];
    if (total > 32 * words || words != (total + 127) / 128 * 4)
      return fail(UW_ERR_FORMAT, "block stream size inconsistent with lane bits");
    max_stream = std::max<uint32_t>(max_stream, uint32_t(words * 4));
  }
  if (max_stream != h.max_block_stream_bytes) return fail(UW_ERR_FORMAT, "bad max block stream size");
  *out = h;
  return UW_OK;
}

}  // namespace uw

extern "C" const char* uw_last_error(void) { return uw::last_error_text(); }
