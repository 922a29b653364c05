// Host encoder: bf16 matrix -> compressed blob.
//
// "Unweight: how we compressed an LLM 22% without sacrificing quality":
//  - a bf16 is 1 sign, 8 exponent and 7 mantissa bits; sign and mantissa look
//    random and are kept as one raw byte (paragraph on the anatomy of a BF16);
//  - a handful of exponents dominate (top 16 cover >99%, ~2.6 bits of
//    entropy; paragraph on exponent redundancy), so only the exponent byte is
//    Huffman coded (paragraph on Huffman coding of the exponent byte);
//  - a row of 64 weights holding an exponent outside the top-K palette is
//    stored raw, one decision per row instead of a per-weight branch
//    (paragraph on rare exponents).
// The code is length-limited (package-merge, Larmore & Hirschberg 1990) and
// canonical (RFC 1951 3.2.2); blocks of G groups give every wavefront lane its
// own bit stream so a wave decodes a block with a prefix sum of lane lengths.
#include <algorithm>
#include <cstring>
#include <numeric>
#include <thread>
#include <atomic>
#include <functional>
#include <vector>

#include "uw_internal.h"

namespace uw {
namespace {

struct Item {
  uint64_t weight;
  uint8_t n_of[kMaxK];  // how many coins of each symbol the item holds
  bool leaf;
};

// Optimal code lengths <= max_len (coin collector / package-merge).  Leaves
// are ordered by (count, exponent); on equal weight a leaf precedes a package.
std::vector<int> limited_lengths(const std::vector<uint64_t>& counts, const std::vector<int>& key, int max_len) {
  const int n = int(counts.size());
  std::vector<int> len(n, 0);
  if (n == 1) {
    len[0] = 1;
    return len;
  }
  std::vector<int> idx(n);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) {
    return counts[a] != counts[b] ? counts[a] < counts[b] : key[a] < key[b];
  });
  std::vector<Item> leaves(n);
  for (int t = 0; t < n; ++t) {
    Item it{};
    it.weight = counts[idx[t]];
    it.n_of[idx[t]] = 1;
    it.leaf = true;
    leaves[t] = it;
  }
  std::vector<Item> list = leaves;
  for (int level = 1; level < max_len; ++level) {
    std::vector<Item> packs;
    for (size_t a = 0; a + 1 < list.size(); a += 2) {
      Item p{};
      p.weight = list[a].weight + list[a + 1].weight;
      for (int s = 0; s < n; ++s) p.n_of[s] = uint8_t(list[a].n_of[s] + list[a + 1].n_of[s]);
      p.leaf = false;
      packs.push_back(p);
    }
    std::vector<Item> merged;
    merged.reserve(leaves.size() + packs.size());
    size_t i = 0, j = 0;
    while (i < leaves.size() || j < packs.size()) {
      bool take_leaf = j == packs.size() || (i < leaves.size() && leaves[i].weight <= packs[j].weight);
      merged.push_back(take_leaf ? leaves[i++] : packs[j++]);
    }
    list.swap(merged);
  }
  for (int t = 0; t < 2 * n - 2; ++t)
    for (int s = 0; s < n; ++s) len[s] += list[t].n_of[s];
  return len;
}

int auto_groups_per_block(int64_t rows, int64_t cols) {
  const int64_t gpr = cols / 64, total = rows * gpr;
  std::vector<int> aligned, all;
  for (int g = 16; g <= 256; g += 16) {
    all.push_back(g);
    if (gpr % g == 0 || g % gpr == 0) aligned.push_back(g);
  }
  const std::vector<int>& pool = aligned.empty() ? all : aligned;
  int best = -1;
  for (int g : pool)
    if ((total + g - 1) / g >= 2048) best = std::max(best, g);
  if (best > 0) return best;
  int small = -1;
  for (int g : pool)
    if (g <= 64) small = std::max(small, g);
  return small > 0 ? small : *std::min_element(pool.begin(), pool.end());
}

uint64_t align_up(uint64_t v) { return (v + kSectionAlign - 1) / kSectionAlign * kSectionAlign; }

struct Plan {
  int64_t rows, cols, n_groups;
  int K, L, G;
  uint32_t nb, W;
  std::vector<uint8_t> pal;        // palette exponents
  std::vector<int> sym_of;         // exponent -> palette index or -1
  std::vector<uint8_t> code_len;   // per palette index
  std::vector<uint32_t> rev;       // bit-reversed code per palette index
  std::vector<uint8_t> raw;        // per group
  std::vector<uint32_t> start_word, first_raw, raw_bits;
  std::vector<uint16_t> lane_bits;
  uint32_t max_stream = 0;
  uint64_t n_raw = 0;
  uint64_t off_sw, off_fr, off_rb, off_lb, off_stream, size_stream, off_raw, size_raw, off_sm, size_sm, total;
};

void parallel_for(uint64_t n, const std::function<void(uint64_t, uint64_t)>& fn) {
  unsigned hw = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  if (n < 64 || hw == 1) {
    fn(0, n);
    return;
  }
  std::vector<std::thread> th;
  const uint64_t chunk = (n + hw - 1) / hw;
  for (unsigned t = 0; t < hw; ++t) {
    uint64_t a = t * chunk, b = std::min(n, a + chunk);
    if (a < b) th.emplace_back(fn, a, b);
  }
  for (auto& t : th) t.join();
}

uint64_t plain_size(int64_t rows, int64_t cols) { return align_up(kHeaderBytes) + 2 * uint64_t(rows) * uint64_t(cols); }

void write_plain(const uint16_t* w, int64_t rows, int64_t cols, uint8_t* out) {
  const uint64_t total = plain_size(rows, cols);
  std::memset(out, 0, total);
  const uint64_t off = align_up(kHeaderBytes);
  std::memcpy(out + off, w, 2 * uint64_t(rows) * uint64_t(cols));
  BlobHeader h;
  h.flags = kFlagPlain;
  h.rows = rows;
  h.cols = cols;
  h.total_bytes = total;
  h.off_plain = off;
  h.size_plain = 2 * uint64_t(rows) * uint64_t(cols);
  h.crc32 = crc32(out + kHeaderBytes, total - kHeaderBytes);
  header_write(h, out);
}

}  // namespace
}  // namespace uw

extern "C" int uw_encode(const uint16_t* w, int64_t rows, int64_t cols, const uw_encode_opts* opts,
                         void* out, size_t* out_size) {
  using namespace uw;
  if (!w || !out_size) return fail(UW_ERR_INVALID, "uw_encode: null pointer");
  if (rows < 1 || cols < 64 || cols % 64) return fail(UW_ERR_INVALID, "uw_encode: rows >= 1 and cols a positive multiple of 64");
  if (rows > (int64_t(1) << 40) / cols) return fail(UW_ERR_INVALID, "uw_encode: matrix too large");
  Plan p;
  p.rows = rows;
  p.cols = cols;
  p.K = opts && opts->K ? opts->K : 16;
  p.L = opts && opts->L ? opts->L : 6;
  p.G = opts && opts->G ? opts->G : auto_groups_per_block(rows, cols);
  const bool allow_plain = !(opts && (opts->flags & UW_ENC_NO_PLAIN));
  if (p.K < 1 || p.K > kMaxK || p.L < 1 || p.L > kMaxL || p.K > (1 << p.L))
    return fail(UW_ERR_INVALID, "uw_encode: need 1 <= K <= 32, 1 <= L <= 12, K <= 2^L");
  if (p.G < 16 || p.G > 1024 || p.G % 16) return fail(UW_ERR_INVALID, "uw_encode: G must be a multiple of 16 in [16, 1024]");
  const uint64_t nw = uint64_t(rows) * uint64_t(cols);
  p.n_groups = int64_t(nw / 64);

  // exponent histogram and palette (count desc, exponent asc)
  std::vector<uint64_t> hist(256, 0);
  {
    std::vector<std::vector<uint64_t>> part(16, std::vector<uint64_t>(256, 0));
    std::atomic<int> slot{0};
    parallel_for(nw, [&](uint64_t a, uint64_t b) {
      auto& h = part[slot++];
      for (uint64_t i = a; i < b; ++i) h[(w[i] >> 7) & 0xFF]++;
    });
    for (auto& h : part)
      for (int e = 0; e < 256; ++e) hist[e] += h[e];
  }
  std::vector<int> present;
  for (int e = 0; e < 256; ++e)
    if (hist[e]) present.push_back(e);
  std::sort(present.begin(), present.end(), [&](int a, int b) { return hist[a] != hist[b] ? hist[a] > hist[b] : a < b; });
  if (int(present.size()) > p.K) present.resize(p.K);
  p.pal.assign(present.begin(), present.end());
  p.sym_of.assign(256, -1);
  for (size_t i = 0; i < p.pal.size(); ++i) p.sym_of[p.pal[i]] = int(i);

  // raw groups and the histogram of coded exponents
  p.raw.assign(p.n_groups, 0);
  std::vector<uint64_t> chist(p.pal.size(), 0);
  {
    std::mutex mu;
    parallel_for(uint64_t(p.n_groups), [&](uint64_t a, uint64_t b) {
      std::vector<uint64_t> local(p.pal.size(), 0);
      for (uint64_t g = a; g < b; ++g) {
        const uint16_t* q = w + 64 * g;
        bool raw = false;
        for (int l = 0; l < 64 && !raw; ++l) raw = p.sym_of[(q[l] >> 7) & 0xFF] < 0;
        p.raw[g] = raw;
        if (!raw)
          for (int l = 0; l < 64; ++l) local[p.sym_of[(q[l] >> 7) & 0xFF]]++;
      }
      std::lock_guard<std::mutex> lk(mu);
      for (size_t i = 0; i < local.size(); ++i) chist[i] += local[i];
    });
  }
  std::vector<uint64_t> counts;
  std::vector<int> keys, which;
  for (size_t i = 0; i < p.pal.size(); ++i)
    if (chist[i]) {
      counts.push_back(chist[i]);
      keys.push_back(p.pal[i]);
      which.push_back(int(i));
    }
  if (counts.empty()) {
    // nothing can be coded: plain mode
    const uint64_t need = plain_size(rows, cols);
    if (!out) { *out_size = need; return UW_OK; }
    if (*out_size < need) { *out_size = need; return fail(UW_ERR_NOSPACE, "uw_encode: output buffer too small"); }
    write_plain(w, rows, cols, static_cast<uint8_t*>(out));
    *out_size = need;
    return UW_OK;
  }
  std::vector<int> lens = limited_lengths(counts, keys, p.L);
  p.code_len.assign(p.pal.size(), 0);
  for (size_t t = 0; t < which.size(); ++t) p.code_len[which[t]] = uint8_t(lens[t]);
  BlobHeader hc;
  hc.K = uint32_t(p.pal.size());
  hc.L = uint32_t(p.L);
  for (size_t i = 0; i < p.pal.size(); ++i) {
    hc.palette[i] = p.pal[i];
    hc.code_len[i] = p.code_len[i];
  }
  uint32_t code[32], rev[32];
  canonical_codes(hc, code, rev);
  p.rev.assign(rev, rev + p.pal.size());

  // block tables (first pass: sizes)
  p.nb = uint32_t((p.n_groups + p.G - 1) / p.G);
  p.W = uint32_t((p.G + 31) / 32);
  p.start_word.assign(p.nb + 1, 0);
  p.first_raw.assign(p.nb + 1, 0);
  p.raw_bits.assign(uint64_t(p.nb) * p.W, 0);
  p.lane_bits.assign(uint64_t(p.nb) * 64, 0);
  std::vector<uint32_t> block_words(p.nb), block_raw(p.nb);
  parallel_for(p.nb, [&](uint64_t a, uint64_t b) {
    for (uint64_t blk = a; blk < b; ++blk) {
      const int64_t g0 = int64_t(blk) * p.G, g1 = std::min<int64_t>(g0 + p.G, p.n_groups);
      uint64_t total = 0;
      uint32_t nraw = 0;
      uint32_t lanes[64] = {0};
      for (int64_t g = g0; g < g1; ++g) {
        if (p.raw[g]) {
          p.raw_bits[blk * p.W + (g - g0) / 32] |= 1u << ((g - g0) % 32);
          nraw++;
          continue;
        }
        const uint16_t* q = w + 64 * g;
        for (int l = 0; l < 64; ++l) lanes[l] += p.code_len[p.sym_of[(q[l] >> 7) & 0xFF]];
      }
      for (int l = 0; l < 64; ++l) {
        p.lane_bits[blk * 64 + l] = uint16_t(lanes[l]);
        total += lanes[l];
      }
      block_words[blk] = uint32_t((total + 127) / 128 * 4);
      block_raw[blk] = nraw;
    }
  });
  for (uint32_t blk = 0; blk < p.nb; ++blk) {
    p.start_word[blk + 1] = p.start_word[blk] + block_words[blk];
    p.first_raw[blk + 1] = p.first_raw[blk] + block_raw[blk];
    p.max_stream = std::max(p.max_stream, 4 * block_words[blk]);
  }
  p.n_raw = p.first_raw[p.nb];
  const uint64_t g_last = uint64_t(p.n_groups) - uint64_t(p.nb - 1) * p.G;
  p.size_stream = uint64_t(p.start_word[p.nb]) * 4;
  p.size_raw = 64 * p.n_raw;
  p.size_sm = uint64_t(p.nb - 1) * p.G * 64 + (g_last + 15) / 16 * 1024;
  uint64_t off = kHeaderBytes;
  off = align_up(off); p.off_sw = off; off += 4 * (uint64_t(p.nb) + 1);
  off = align_up(off); p.off_fr = off; off += 4 * (uint64_t(p.nb) + 1);
  off = align_up(off); p.off_rb = off; off += 4 * uint64_t(p.nb) * p.W;
  off = align_up(off); p.off_lb = off; off += 128 * uint64_t(p.nb);
  off = align_up(off); p.off_stream = off; off += p.size_stream;
  off = align_up(off); p.off_raw = off; off += p.size_raw;
  off = align_up(off); p.off_sm = off; off += p.size_sm;
  p.total = off;
  const bool use_plain = allow_plain && p.total - kHeaderBytes >= 2 * nw;
  const uint64_t need = use_plain ? plain_size(rows, cols) : p.total;
  if (!out) { *out_size = need; return UW_OK; }
  if (*out_size < need) { *out_size = need; return fail(UW_ERR_NOSPACE, "uw_encode: output buffer too small"); }
  uint8_t* o = static_cast<uint8_t*>(out);
  if (use_plain) {
    write_plain(w, rows, cols, o);
    *out_size = need;
    return UW_OK;
  }

  // second pass: emit
  std::memset(o, 0, p.total);
  std::memcpy(o + p.off_sw, p.start_word.data(), 4 * (uint64_t(p.nb) + 1));
  std::memcpy(o + p.off_fr, p.first_raw.data(), 4 * (uint64_t(p.nb) + 1));
  std::memcpy(o + p.off_rb, p.raw_bits.data(), 4 * uint64_t(p.nb) * p.W);
  std::memcpy(o + p.off_lb, p.lane_bits.data(), 128 * uint64_t(p.nb));
  uint32_t* stream = reinterpret_cast<uint32_t*>(o + p.off_stream);
  uint8_t* rawsec = o + p.off_raw;
  uint8_t* smsec = o + p.off_sm;
  parallel_for(p.nb, [&](uint64_t a, uint64_t b) {
    for (uint64_t blk = a; blk < b; ++blk) {
      const int64_t g0 = int64_t(blk) * p.G, g1 = std::min<int64_t>(g0 + p.G, p.n_groups);
      uint32_t* words = stream + p.start_word[blk];
      uint64_t pos = 0;  // bit position inside the block stream
      for (int l = 0; l < 64; ++l) {
        for (int64_t g = g0; g < g1; ++g) {
          if (p.raw[g]) continue;
          const int s = p.sym_of[(w[64 * g + l] >> 7) & 0xFF];
          const uint32_t c = p.rev[s], len = p.code_len[s];
          const uint32_t sh = uint32_t(pos & 31);
          words[pos >> 5] |= c << sh;
          if (sh + len > 32) words[(pos >> 5) + 1] |= c >> (32 - sh);
          pos += len;
        }
      }
      uint64_t r = p.first_raw[blk];
      uint8_t* smb = smsec + uint64_t(blk) * p.G * 64;
      for (int64_t g = g0; g < g1; ++g) {
        const uint16_t* q = w + 64 * g;
        const int64_t j = g - g0;
        if (p.raw[g]) {
          for (int l = 0; l < 64; ++l) rawsec[64 * r + l] = uint8_t((q[l] >> 7) & 0xFF);
          r++;
        }
        uint8_t* t = smb + (j >> 4) * 1024 + (j & 15);
        for (int l = 0; l < 64; ++l) t[16 * l] = uint8_t(((q[l] >> 8) & 0x80) | (q[l] & 0x7F));
      }
    }
  });
  BlobHeader h;
  h.rows = rows;
  h.cols = cols;
  h.K = uint32_t(p.pal.size());
  h.L = uint32_t(p.L);
  h.G = uint32_t(p.G);
  h.n_blocks = p.nb;
  h.n_raw_groups = p.n_raw;
  h.total_bytes = p.total;
  h.max_block_stream_bytes = p.max_stream;
  for (size_t i = 0; i < p.pal.size(); ++i) {
    h.palette[i] = p.pal[i];
    h.code_len[i] = p.code_len[i];
  }
  h.off_start_word = p.off_sw;
  h.off_first_raw = p.off_fr;
  h.off_raw_bits = p.off_rb;
  h.off_lane_bits = p.off_lb;
  h.off_stream = p.off_stream;
  h.size_stream = p.size_stream;
  h.off_raw = p.off_raw;
  h.size_raw = p.size_raw;
  h.off_sm = p.off_sm;
  h.size_sm = p.size_sm;
  h.crc32 = crc32(o + kHeaderBytes, p.total - kHeaderBytes);
  header_write(h, o);
  *out_size = p.total;
  return UW_OK;
}
