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
// canonical (RFC 1951 3.2.2).  Blocks of G groups give every wavefront lane
// its own code stream, cut into 32-bit words; the words are stored in the
// order the decoding wave takes them (refill checks every R groups, lanes in
// order), in one segment per 16-group tile, so a decoder streams a block tile
// by tile instead of holding all of it.
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

// Default G.  Candidates: multiples of 16 up to 256 that divide the groups
// per row or are a multiple of it, plus (groups per row a multiple of 16)
// any larger G whose work unit, lcm(G, groups per row), has at most 8 blocks.
// With at least 2048 blocks, pick the G that spreads one block per wave most
// evenly over the 1024 SIMDs of a 256-CU part, 4 waves per SIMD in a round:
// with b = ceil(blocks / 1024), the least ceil(b / 4) * 4 * (tiles per block
// + 1 for the block start) (a partial round costs a full one), ties to the
// larger G.  Smaller matrices: the largest aligned G <= 64.
int auto_groups_per_block(int64_t rows, int64_t cols) {
  const int64_t gpr = cols / 64, total = rows * gpr;
  std::vector<int> aligned, wide, all;
  for (int g = 16; g <= 256; g += 16) {
    all.push_back(g);
    const bool al = gpr % g == 0 || g % gpr == 0;
    if (al) aligned.push_back(g);
    if (al || (gpr % 16 == 0 && g > gpr && gpr / std::gcd<int64_t>(g, gpr) <= 8)) wide.push_back(g);
  }
  int best = -1;
  int64_t best_load = 0;
  for (int g : wide.empty() ? all : wide) {
    const int64_t nb = (total + g - 1) / g;
    if (nb < 2048) continue;
    const int64_t per_simd = (nb + 1023) / 1024;
    const int64_t load = (per_simd + 3) / 4 * 4 * (g / 16 + 1);
    if (best < 0 || load < best_load || (load == best_load && g > best)) {
      best = g;
      best_load = load;
    }
  }
  if (best > 0) return best;
  const std::vector<int>& pool = aligned.empty() ? all : aligned;
  int small = -1;
  for (int g : pool)
    if (g <= 64) small = std::max(small, g);
  return small > 0 ? small : *std::min_element(pool.begin(), pool.end());
}

uint64_t align_up(uint64_t v) { return (v + kSectionAlign - 1) / kSectionAlign * kSectionAlign; }

struct Plan {
  int64_t rows, cols, n_groups;
  int K, L, G, R;
  uint32_t nb, W, T;
  std::vector<uint8_t> pal;        // palette exponents
  std::vector<int> sym_of;         // exponent -> palette index or -1
  std::vector<uint8_t> code_len;   // per palette index
  std::vector<uint32_t> rev;       // bit-reversed code per palette index
  std::vector<uint8_t> raw;        // per group
  std::vector<std::vector<uint8_t>> data;  // per block: its segments back to back
  std::vector<uint32_t> block_off;
  std::vector<uint16_t> seg;
  uint32_t max_seg = 0;
  uint64_t n_raw = 0;
  uint64_t off_block, off_seg, off_queue, size_queue, off_sm, size_sm, total;
};

// The segments of one block (layout in uw_blob.cpp): every lane's code stream
// in words, then the refill checks of the decoder replayed to order the words.
void build_block(const Plan& p, const uint16_t* w, uint64_t blk, std::vector<uint8_t>& out, uint16_t* seg_out,
                 uint32_t& nraw_out, uint32_t& max_seg) {
  const int64_t g0 = int64_t(blk) * p.G, g1 = std::min<int64_t>(g0 + p.G, p.n_groups);
  const int gb = int(g1 - g0);
  const int ntiles = (gb + 15) / 16;
  const int cap = (gb * p.L + 31) / 32 + 1;
  std::vector<uint32_t> lw(64 * size_t(cap), 0);
  uint32_t n[64], qm[64], taken[64];
  uint32_t raw_bits[32] = {0};
  uint32_t nraw = 0;
  std::vector<uint8_t> lens(size_t(gb) * 64, 0);
  for (int j = 0; j < gb; ++j) {
    if (p.raw[g0 + j]) {
      raw_bits[j / 32] |= 1u << (j % 32);
      nraw++;
      continue;
    }
    const uint16_t* q = w + 64 * (g0 + j);
    for (int l = 0; l < 64; ++l) lens[size_t(j) * 64 + l] = p.code_len[p.sym_of[(q[l] >> 7) & 0xFF]];
  }
  for (int l = 0; l < 64; ++l) {
    uint32_t* words = lw.data() + size_t(l) * cap;
    uint64_t pos = 0;
    for (int j = 0; j < gb; ++j) {
      if (p.raw[g0 + j]) continue;
      const int s = p.sym_of[(w[64 * (g0 + j) + l] >> 7) & 0xFF];
      const uint32_t c = p.rev[s], len = p.code_len[s];
      const uint32_t sh = uint32_t(pos & 31);
      words[pos >> 5] |= c << sh;
      if (sh + len > 32) words[(pos >> 5) + 1] |= c >> (32 - sh);
      pos += len;
    }
    n[l] = uint32_t((pos + 31) / 32);
    qm[l] = 30;
    taken[l] = std::min<uint32_t>(n[l], 2);
  }
  // tile 0 starts with the lane word counts, the raw bitmap and each lane's first two words
  out.clear();
  for (int l = 0; l < 64; ++l) {
    const uint16_t v = uint16_t(n[l]);
    out.insert(out.end(), reinterpret_cast<const uint8_t*>(&v), reinterpret_cast<const uint8_t*>(&v) + 2);
  }
  auto put_word = [&](uint32_t v) {
    out.insert(out.end(), reinterpret_cast<const uint8_t*>(&v), reinterpret_cast<const uint8_t*>(&v) + 4);
  };
  for (uint32_t i = 0; i < p.W; ++i) put_word(raw_bits[i]);
  for (uint32_t i = 0; i < 2; ++i)
    for (int l = 0; l < 64; ++l)
      if (n[l] > i) put_word(lw[size_t(l) * cap + i]);
  size_t seg_start = 0;
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = 16 * t, j1 = std::min(gb, j0 + 16);
    for (int j = j0; j < j1; ++j)
      if (p.raw[g0 + j])
        for (int l = 0; l < 64; ++l) out.push_back(uint8_t((w[64 * (g0 + j) + l] >> 7) & 0xFF));
    for (int j = j0; j < j1; ++j) {
      for (int l = 0; l < 64; ++l) qm[l] += lens[size_t(j) * 64 + l];
      if ((j + 1) % p.R) continue;
      for (int l = 0; l < 64; ++l) {
        if (qm[l] < 32) continue;
        qm[l] -= 32;
        if (taken[l] < n[l]) put_word(lw[size_t(l) * cap + taken[l]++]);
      }
    }
    max_seg = std::max<uint32_t>(max_seg, uint32_t(out.size() - seg_start));
    seg_start = out.size();
    seg_out[t] = uint16_t(out.size() / 4);
  }
  for (uint32_t t = uint32_t(ntiles); t < p.T; ++t) seg_out[t] = uint16_t(out.size() / 4);
  nraw_out = nraw;
}

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

  // segments of every block (first pass), then offsets and sizes
  p.nb = uint32_t((p.n_groups + p.G - 1) / p.G);
  p.W = uint32_t((p.G + 31) / 32);
  p.T = uint32_t((p.G + 15) / 16);
  p.R = int(check_groups(uint32_t(p.L)));
  p.data.assign(p.nb, {});
  p.seg.assign(uint64_t(p.nb) * p.T, 0);
  std::vector<uint32_t> block_raw(p.nb), block_max(p.nb);
  parallel_for(p.nb, [&](uint64_t a, uint64_t b) {
    for (uint64_t blk = a; blk < b; ++blk) {
      uint32_t mx = 0;
      build_block(p, w, blk, p.data[blk], p.seg.data() + blk * p.T, block_raw[blk], mx);
      block_max[blk] = mx;
    }
  });
  p.block_off.assign(p.nb + 1, 0);
  for (uint32_t blk = 0; blk < p.nb; ++blk) {
    p.block_off[blk + 1] = p.block_off[blk] + uint32_t(p.data[blk].size());
    p.n_raw += block_raw[blk];
    p.max_seg = std::max(p.max_seg, block_max[blk]);
  }
  const uint64_t g_last = uint64_t(p.n_groups) - uint64_t(p.nb - 1) * p.G;
  p.size_queue = p.block_off[p.nb];
  p.size_sm = uint64_t(p.nb - 1) * p.G * 64 + (g_last + 15) / 16 * 1024;
  uint64_t off = kHeaderBytes;
  off = align_up(off); p.off_block = off; off += 4 * (uint64_t(p.nb) + 1);
  off = align_up(off); p.off_seg = off; off += 2 * uint64_t(p.nb) * p.T;
  off = align_up(off); p.off_queue = off; off += p.size_queue;
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
  std::memcpy(o + p.off_block, p.block_off.data(), 4 * (uint64_t(p.nb) + 1));
  std::memcpy(o + p.off_seg, p.seg.data(), 2 * uint64_t(p.nb) * p.T);
  uint8_t* smsec = o + p.off_sm;
  parallel_for(p.nb, [&](uint64_t a, uint64_t b) {
    for (uint64_t blk = a; blk < b; ++blk) {
      std::memcpy(o + p.off_queue + p.block_off[blk], p.data[blk].data(), p.data[blk].size());
      const int64_t g0 = int64_t(blk) * p.G, g1 = std::min<int64_t>(g0 + p.G, p.n_groups);
      uint8_t* smb = smsec + uint64_t(blk) * p.G * 64;
      for (int64_t g = g0; g < g1; ++g) {
        const uint16_t* q = w + 64 * g;
        const int64_t j = g - g0;
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
  h.max_segment_bytes = p.max_seg;
  h.R = uint32_t(p.R);
  for (size_t i = 0; i < p.pal.size(); ++i) {
    h.palette[i] = p.pal[i];
    h.code_len[i] = p.code_len[i];
  }
  h.off_block = p.off_block;
  h.off_seg = p.off_seg;
  h.off_queue = p.off_queue;
  h.size_queue = p.size_queue;
  h.off_sm = p.off_sm;
  h.size_sm = p.size_sm;
  h.crc32 = crc32(o + kHeaderBytes, p.total - kHeaderBytes);
  header_write(h, o);
  *out_size = p.total;
  return UW_OK;
}
