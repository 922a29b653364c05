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

// Header, 256 bytes (little-endian):
//    0 "UWB2"   4 u32 version 2   8 u32 header bytes 256   12 u32 flags (bit 0: plain)
//   16 i64 rows  24 i64 cols  32 u32 K  36 u32 L  40 u32 G  44 u32 n_blocks
//   48 u64 raw groups  56 u64 total bytes  64 u32 CRC-32 of [256, total)
//   68 u32 largest segment (bytes)  72 u8 palette[32]  104 u8 code_len[32]
//  136 u32 R (groups between refill checks)  140 u32 0
//  144 u64 off_block  152 off_seg  160 off_queue  168 size_queue  176 off_sm
//  184 size_sm  192 off_plain  200 size_plain
// Sections: block u32[n_blocks+1] (byte offset of each block's data in the
// queue), seg u16[n_blocks*T] (T = ceil(G/16): end of tile t's segment in
// words from the block start), queue (segments), sm (1 KB tiles), plain.
void header_write(const BlobHeader& h, uint8_t* d) {
  std::memset(d, 0, kHeaderBytes);
  std::memcpy(d, "UWB2", 4);
  put<uint32_t>(d, 4, 2);
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
  put<uint32_t>(d, 68, h.max_segment_bytes);
  std::memcpy(d + 72, h.palette, 32);
  std::memcpy(d + 104, h.code_len, 32);
  put<uint32_t>(d, 136, h.R);
  const uint64_t offs[8] = {h.off_block, h.off_seg, h.off_queue, h.size_queue,
                            h.off_sm, h.size_sm, h.off_plain, h.size_plain};
  for (int i = 0; i < 8; ++i) put<uint64_t>(d, 144 + 8 * i, offs[i]);
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
  h->max_segment_bytes = get<uint32_t>(s, 68);
  std::memcpy(h->palette, s + 72, 32);
  std::memcpy(h->code_len, s + 104, 32);
  h->R = get<uint32_t>(s, 136);
  uint64_t* offs[8] = {&h->off_block, &h->off_seg, &h->off_queue, &h->size_queue,
                       &h->off_sm, &h->size_sm, &h->off_plain, &h->size_plain};
  for (int i = 0; i < 8; ++i) *offs[i] = get<uint64_t>(s, 144 + 8 * i);
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
  if (std::memcmp(b, "UWB2", 4) != 0) return fail(UW_ERR_FORMAT, "bad magic");
  BlobHeader h;
  header_read(b, &h);
  if (h.version != 2) return fail(UW_ERR_FORMAT, "unsupported version");
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
  if (h.R != check_groups(h.L)) return fail(UW_ERR_FORMAT, "refill interval does not match L");
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
  const uint64_t W = (h.G + 31) / 32, T = (h.G + 15) / 16;
  if (!section_ok(h.off_block, 4 * (nb + 1), n) || !section_ok(h.off_seg, 2 * nb * T, n) ||
      !section_ok(h.off_queue, h.size_queue, n) || !section_ok(h.off_sm, h.size_sm, n) ||
      h.off_queue + h.size_queue + 16 > n)
    return fail(UW_ERR_FORMAT, "section out of bounds or misaligned");
  const uint64_t g_last = n_groups - (nb - 1) * h.G;
  if (h.size_sm != (nb - 1) * uint64_t(h.G) * 64 + (g_last + 15) / 16 * 1024)
    return fail(UW_ERR_FORMAT, "bad sm section size");
  if (h.max_segment_bytes > 4064 || h.max_segment_bytes % 4) return fail(UW_ERR_FORMAT, "bad largest segment size");
  std::vector<uint32_t> bo(nb + 1);
  std::memcpy(bo.data(), b + h.off_block, 4 * (nb + 1));
  std::vector<uint16_t> sg(nb * T);
  std::memcpy(sg.data(), b + h.off_seg, 2 * nb * T);
  if (bo[0] != 0 || bo[nb] != h.size_queue) return fail(UW_ERR_FORMAT, "bad block table ends");
  uint32_t max_seg = 0;
  uint64_t nraw_total = 0;
  const uint8_t* q = b + h.off_queue;
  for (uint64_t blk = 0; blk < nb; ++blk) {
    const uint64_t gb = (blk + 1 == nb) ? g_last : h.G;
    const uint64_t nt = (gb + 15) / 16;
    if (bo[blk + 1] < bo[blk] || bo[blk] % 4 || bo[blk + 1] - bo[blk] < 128 + 4 * W)
      return fail(UW_ERR_FORMAT, "bad block offset");
    const uint64_t words = (bo[blk + 1] - bo[blk]) / 4;
    const uint8_t* d = q + bo[blk];
    uint32_t rb[32];
    std::memcpy(rb, d + 128, 4 * W);
    // raw flags only for groups of the block; lane word counts in range; the
    // words of the segments add up to every word of every lane, once
    uint32_t nraw = 0, tile_raw[64] = {0};
    for (uint64_t w = 0; w < W; ++w) {
      const uint64_t lo = 32 * w;
      if (lo + 32 > gb) {
        const uint32_t valid = gb > lo ? uint32_t(gb - lo) : 0;
        if (valid < 32 && (rb[w] >> valid)) return fail(UW_ERR_FORMAT, "raw bit beyond the block");
      }
      nraw += __builtin_popcount(rb[w]);
      for (int k = 0; k < 32; ++k)
        if (rb[w] >> k & 1) tile_raw[(lo + k) / 16]++;
    }
    nraw_total += nraw;
    const uint64_t coded_groups = gb - nraw;
    uint64_t init = 0, later = 0;
    for (int l = 0; l < 64; ++l) {
      uint16_t nl;
      std::memcpy(&nl, d + 2 * l, 2);
      const uint64_t lo_bits = coded_groups * uint64_t(minlen), hi_bits = coded_groups * uint64_t(maxlen);
      if (nl < (lo_bits + 31) / 32 || nl > (hi_bits + 31) / 32) return fail(UW_ERR_FORMAT, "lane word count out of range");
      init += std::min<uint64_t>(nl, 2);
      later += nl > 2 ? nl - 2 : 0;
    }
    uint64_t prev = 0, taken = 0;
    for (uint64_t t = 0; t < T; ++t) {
      const uint64_t end = sg[blk * T + t];
      if (end < prev || end > words || (t >= nt && end != prev)) return fail(UW_ERR_FORMAT, "bad segment table");
      if (t < nt) {
        const uint64_t fixed = 16 * tile_raw[t] + (t == 0 ? 32 + W + init : 0);
        if (end - prev < fixed) return fail(UW_ERR_FORMAT, "segment shorter than its fixed part");
        taken += end - prev - fixed;
        max_seg = std::max<uint32_t>(max_seg, uint32_t(4 * (end - prev)));
      }
      prev = end;
    }
    if (prev != words || taken != later) return fail(UW_ERR_FORMAT, "segments inconsistent with the lane word counts");
  }
  if (nraw_total != h.n_raw_groups) return fail(UW_ERR_FORMAT, "raw group count mismatch");
  if (max_seg != h.max_segment_bytes) return fail(UW_ERR_FORMAT, "bad largest segment size");
  *out = h;
  return UW_OK;
}

}  // namespace uw

extern "C" const char* uw_last_error(void) { return uw::last_error_text(); }
