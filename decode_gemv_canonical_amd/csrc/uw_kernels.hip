// Device kernels for gfx950 (CDNA4): on-chip exponent-Huffman decode fused
// into the decode-time product (vector ALU for small batches, matrix cores
// for batches of 16 and more) and the decompress-to-HBM alternative.
//
// Method: "Unweight: how we compressed an LLM 22% without sacrificing
// quality".  The reconstructive-matmul paragraph loads compressed data,
// rebuilds bf16 weights on chip and multiplies them without writing them back
// to main memory; here the rebuild happens in registers of a wave64.  The
// full-decode pipeline of the four-pipelines paragraph is uw_decompress
// followed by the bf16 product.
//
// Decode scheme (one wave per block, lane l owns one code stream; the layout
// is described in uw_blob.cpp):
//  * a wave walks its blocks tile by tile; every tile step is one 1 KB
//    direct-to-LDS load of the tile's sign+mantissa bytes and one to four
//    1 KB loads of the tile's queue segment (raw exponent bytes and the code
//    words the lanes take during the tile), into a ring of slots with a fixed
//    number of loads per step, so an explicit vmcnt wait finds the oldest;
//  * a lane holds three words (w0, w1, w2) of its stream and qm, the bit
//    offset of (next code - 2) in w0; a peek is one v_alignbit_b32 and the
//    table byte address is (peek & mask): the "-2" lands the index on a
//    4-byte table stride for free;
//  * with code lengths <= 6 any 12-bit window starting at a code holds two
//    whole codes, so one lookup in a 4096-entry pair table returns both
//    exponents: entry = (len_a + len_b) | E_a << 7 | len_a << 16 | E_b << 23.
//    One v_bfi_b32 with the replicated sign+mantissa bytes gives two bf16
//    weights in one register.  The length sits in bits 0..3 and bits 4..6 are
//    zero, so qm += entry keeps the low 7 bits of qm exact;
//  * after every R groups the lanes with qm >= 32 shift by a word; those with
//    words left take the next one from the segment at their rank among the
//    taking lanes (ballot + mbcnt).  The read lands while the next R groups
//    decode and is merged into the window at the following check, so LDS
//    latency never sits on the decode chain;
//  * longer codes (L > 6) use a 2^L single-code table with the same window;
//  * a raw group (exponent outside the palette) is a wave-uniform branch on a
//    bit of the block's raw bitmap.
#include <algorithm>
#include <cstring>
#include <string>
#include <type_traits>

#include "uw_device.h"

namespace uw {
namespace {

constexpr int kTableWords = 4096;     // pair table (or 2^L single table)
constexpr int kT1Words = 64;          // single-code table for L <= 6 (the host builds the pair table from it)
constexpr int kTransposeWords = 512;  // 16 groups x 64 lanes x bf16

// ---------------------------------------------------------------------------
// Decode tables in LDS: the image the host built at matrix creation
// (kDecodeTableBytes: the pair table, or the 2^L single table for L > 6, then
// the single table for L <= 6), copied in with direct loads of 1 KB spread
// over the waves; the last load moves 256 B (16 lanes).  Returns the loads
// this wave issued.  Runs with all lanes active.
constexpr int kTableLoads = int((kDecodeTableBytes + 1023) / 1024);
// Buffer resource over [base, base + bytes) for raw byte-offset loads.
__device__ inline __amdgpu_buffer_rsrc_t byte_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), int16_t(0), int(bytes), 0x00020000);
}
__device__ __forceinline__ int issue_tables(const DevMatrix& d, int wave, int waves, int lane) {
  const __amdgpu_buffer_rsrc_t r = byte_rsrc(d.tables, kDecodeTableBytes);
  const uint32_t lane16 = 16u * uint32_t(lane);
  int n = 0;
  for (int i = wave; i < kTableLoads; i += waves, ++n) {
    const uint32_t off = uint32_t(i) * 1024u;
    const uint32_t lanes = std::min(64u, (kDecodeTableBytes - off) / 16u);
    const uint64_t mask = lanes == 64 ? ~0ull : ((1ull << lanes) - 1ull);
    asm volatile(
        "s_nop 4\n"
        "s_mov_b32 m0, %[m]\n"
        "s_mov_b64 exec, %[ex]\n"  // also the wait state after the M0 write
        "buffer_load_dwordx4 %[l16], %[r], %[so] offen lds\n"
        "s_mov_b64 exec, -1"
        :
        : [m] "s"(off), [ex] "s"(mask), [l16] "v"(lane16), [r] "s"(r), [so] "s"(off)
        : "memory", "m0", "exec");
  }
  return n;
}

// LDS layout (bytes): [0, 16384) decode table, [16384, 16640) single table for
// L <= 6, then the kernel's area (x for products, slices for the matrix-core
// product) and one ring per wave.
constexpr uint32_t kAreaAddr = (kTableWords + kT1Words) * 4;

// ---------------------------------------------------------------------------
// Lane decoder of one block's code streams.
struct LaneDec {
  uint32_t w0, w1, w2;  // words s-1, s, s+1 of the lane's stream
  uint32_t qm;          // bit offset of (next code - 2) in w0; its low 7 bits are exact
  uint32_t left;        // words of the lane's stream not taken yet
  uint32_t nw[2];       // word read at the latest check of each phase
  uint64_t took[2];     // lanes whose nw[phase] is their next word (wave-uniform mask)
  uint32_t raw_word;    // lane w holds raw-bitmap word w of the block
};

// Block start: the head of tile 0's segment (at LDS byte address q) holds the
// lane word counts, the raw bitmap and every lane's first two words.  Returns
// the byte offset (in the segment) of what follows the head.
__device__ inline uint32_t lane_dec_start(LaneDec& s, uint32_t q, int rb_words, int lane) {
  const uint32_t n = ld16(q + 2 * lane);
  s.raw_word = lane < rb_words ? ld32(q + 128 + 4 * lane) : 0u;
  uint32_t pos = 128 + 4 * uint32_t(rb_words);
  const uint64_t m0 = __builtin_amdgcn_ballot_w64(n >= 1);
  const uint32_t a0 = q + pos + 4 * lanes_below(m0);
  pos += 4 * uint32_t(__builtin_popcountll(m0));
  const uint64_t m1 = __builtin_amdgcn_ballot_w64(n >= 2);
  const uint32_t a1 = q + pos + 4 * lanes_below(m1);
  pos += 4 * uint32_t(__builtin_popcountll(m1));
  s.w0 = 0u;
  s.w1 = n >= 1 ? ld32(a0) : 0u;
  s.w2 = n >= 2 ? ld32(a1) : 0u;
  s.qm = 30u;
  s.left = n > 2 ? n - 2 : 0u;
  s.took[0] = s.took[1] = 0u;
  s.nw[0] = s.nw[1] = 0u;
  return pos;
}

__device__ inline uint32_t peek(const LaneDec& s) { return __builtin_amdgcn_alignbit(s.w1, s.w0, s.qm); }

// Refill check of phase PH (checks alternate phases within a block): merge the
// word read at the previous check, shift the lanes with qm >= 32 and read the
// next word of those that still have words.  q = segment base, wp = word
// offset of the next word to take (wave-uniform).  A lane that takes nothing
// reads a word inside the segment or just past its end, which the slot holds.
// left -= 1 on the lanes of mask m: one subtract with the mask as borrow
__device__ __forceinline__ uint32_t dec_masked(uint32_t left, uint64_t m) {
  uint32_t r;
  asm("v_subb_co_u32_e64 %0, vcc, %1, 0, %2" : "=v"(r) : "v"(left), "s"(m) : "vcc");
  return r;
}

template <int PH>
__device__ __forceinline__ void check(LaneDec& s, uint32_t q, uint32_t& wp) {
  const uint32_t w2 = __builtin_amdgcn_inverse_ballot_w64(s.took[PH ^ 1]) ? s.nw[PH ^ 1] : s.w2;
  const uint64_t ma = __builtin_amdgcn_ballot_w64((s.qm & 32u) != 0u);
  const uint64_t m = ma & __builtin_amdgcn_ballot_w64(s.left != 0u);
  const bool adv = __builtin_amdgcn_inverse_ballot_w64(ma);
  s.w0 = adv ? s.w1 : s.w0;
  s.w1 = adv ? w2 : s.w1;
  s.w2 = w2;
  // the segment address of word wp, kept a scalar sum (an empty asm stops
  // the compiler from folding it into the per-lane address arithmetic)
  uint32_t base;
  asm("s_lshl2_add_u32 %0, %1, %2"
      : "=s"(base)
      : "s"(__builtin_amdgcn_readfirstlane(wp)), "s"(__builtin_amdgcn_readfirstlane(q)));
  s.nw[PH] = ld32(base + 4 * lanes_below(m));
  s.took[PH] = m;
  s.left = dec_masked(s.left, m);
  s.qm &= 31u;
  wp += uint32_t(__builtin_popcountll(m));
  wp = __builtin_amdgcn_readfirstlane(wp);  // wave-uniform: keeps q + 4 wp a scalar sum
}

__device__ inline void check_rt(LaneDec& s, int ph, uint32_t q, uint32_t& wp) {
  if (ph) check<1>(s, q, wp);
  else check<0>(s, q, wp);
}

// Replicated sign+mantissa bytes of groups (2k, 2k+1) of a 16-group tile.
__device__ inline uint32_t sm_pair(const uint4& v, int k) {
  const uint32_t w = (k >> 1) == 0 ? v.x : (k >> 1) == 1 ? v.y : (k >> 1) == 2 ? v.z : v.w;
  return __builtin_amdgcn_perm(0u, w, (k & 1) ? 0x03030202u : 0x01010000u);
}

__device__ inline uint32_t sm_byte(const uint4& v, int j) {
  const uint32_t w = (j >> 2) == 0 ? v.x : (j >> 2) == 1 ? v.y : (j >> 2) == 2 ? v.z : v.w;
  return (w >> (8 * (j & 3))) & 0xFF;
}

// Two bf16 weights in one register: sign+mantissa bits from S, exponents from E.
__device__ inline uint32_t merge_pair(uint32_t S, uint32_t E) { return (S & 0x807F807Fu) | (E & 0x7F807F80u); }

__device__ inline uint32_t merge_one(uint32_t sm, uint32_t E) {
  return ((sm & 0x80u) << 8) | (E & 0x7F80u) | (sm & 0x7Fu);
}

// Raw flags of the 16 groups of the tile starting at group j0 (wave-uniform).
__device__ inline uint32_t raw_mask16(uint32_t raw_word, int j0) {
  const uint32_t w = __builtin_amdgcn_readlane(raw_word, j0 >> 5);
  return (w >> (j0 & 31)) & 0xFFFFu;
}



// One code: returns the table entry (exponent in bits 7..14) and advances qm
// and the running peek p by the code's length.
template <bool PAIR>
__device__ inline uint32_t take_single(LaneDec& s, uint32_t& p, uint32_t mask) {
  const uint32_t e = ld32(p & mask);
  if (PAIR) {
    const uint32_t n = (e >> 16) & 0xFu;
    p >>= n;
    s.qm += n;
  } else {
    p >>= (e & 31u);  // length in bits 0..3, bit 4 clear
    s.qm += e;        // exponent bits land above bit 6
  }
  return e;
}

// Decode one tile of one block.  q = LDS address of the tile's segment, rpos
// = byte offset of its raw exponent bytes (after the head on tile 0), cur =
// the lane's 16 sign+mantissa
// bytes, rmask = raw flags of the tile's groups, nt = groups in the tile.
// aligned: nt == 16 and the tile lies inside one row starting at an even
// column group; then the sink receives sink.tile_begin(row0, c0) and
// sink.pair(k, D) with D = the lane's weights of groups (2k, 2k+1); otherwise
// sink.single(jj, row, cg, w) per weight.  Returns the bytes of the segment
// it consumed (head, raw bytes and taken words), which is the segment's length.
template <bool PAIR, class Sink>
__device__ __forceinline__ uint32_t decode_tile(const DevMatrix& d, LaneDec& s, uint32_t q, uint32_t rpos,
                                            const uint4& cur, uint32_t rmask, int nt, bool aligned, int64_t row0,
                                            int c0, int lane, Sink& sink) {
  uint32_t wp = (rpos >> 2) + 16 * uint32_t(__builtin_popcount(rmask));  // words
  const uint32_t pmask = PAIR ? 0x3FFCu : (((1u << d.L) - 1u) << 2);
  if (aligned) {
    sink.tile_raw(rmask);
    sink.tile_begin(row0, c0);
    if (PAIR && rmask == 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t p = peek(s);
        const uint32_t e1 = ld32(p & 0x3FFCu);
        p >>= (e1 & 31u);
        const uint32_t e2 = ld32(p & 0x3FFCu);
        s.qm += e1 + e2;
        sink.pair(2 * c, merge_pair(sm_pair(cur, 2 * c), e1));
        sink.pair(2 * c + 1, merge_pair(sm_pair(cur, 2 * c + 1), e2));
        check_rt(s, c & 1, q, wp);
      }
    } else {
      uint32_t rp = q + rpos + lane;
      uint32_t p = peek(s);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t two = (rmask >> (2 * k)) & 3u;
        uint32_t E;
        if (PAIR && two == 0) {
          E = ld32(p & 0x3FFCu);
          p >>= (E & 31u);
          s.qm += E;
        } else {
          uint32_t ea, eb;
          if (two & 1u) {
            ea = ld8(rp) << 7;
            rp += 64;
          } else {
            ea = take_single<PAIR>(s, p, pmask) & 0x7F80u;
          }
          if (two & 2u) {
            eb = ld8(rp) << 23;
            rp += 64;
          } else {
            eb = (take_single<PAIR>(s, p, pmask) & 0x7F80u) << 16;
          }
          E = ea | eb;
        }
        sink.pair(k, merge_pair(sm_pair(cur, k), E));
        // checks after groups 4, 8, ... (R = 4) or after every pair (R = 2)
        if (PAIR || d.R == 4) {
          if (k & 1) {
            check_rt(s, ((k - 1) / 2) & 1, q, wp);
            p = peek(s);
          }
        } else {
          check_rt(s, k & 1, q, wp);
          p = peek(s);
        }
      }
    }
  } else {
    int64_t row = row0;
    int cg = c0, c = 0;
    uint32_t rp = q + rpos + lane;
    uint32_t p = peek(s);
    for (int jj = 0; jj < nt; ++jj, ++cg) {
      if (cg >= d.gpr) {
        cg -= d.gpr;
        ++row;
      }
      uint32_t E;
      if ((rmask >> jj) & 1u) {
        E = ld8(rp) << 7;
        rp += 64;
      } else {
        E = take_single<PAIR>(s, p, pmask);
      }
      sink.single(jj, row, cg, merge_one(sm_byte(cur, jj), E));
      if (((jj + 1) & (d.R - 1)) == 0) {  // R is 2 or 4
        check_rt(s, c & 1, q, wp);
        ++c;
        p = peek(s);
      }
    }
  }
  return 4 * wp;  // the segment's length in bytes: raw bytes and every word taken
}

// ---------------------------------------------------------------------------
// Tile steps through a ring of RS slots per wave: slot i = 1 KB of
// sign+mantissa bytes at sm + 1024 i and a queue slot at qs + slot_bytes i.

// What a walk needs of one block, computed once per block.
struct BlockRef {
  const uint8_t* sm;    // the block's first sign+mantissa tile
  const uint8_t* q;     // the block's data in the queue
  const uint32_t* seg;  // the 4-byte aligned word holding its first segment end
  uint32_t seg_odd;     // 1 if that end is the upper half of the word
  int gb;               // groups in the block
  int nt;               // tiles in the block
};

__device__ inline BlockRef block_ref(const DevMatrix& d, int blk) {
  BlockRef r;
  const int64_t g0 = int64_t(blk) * d.G;
  r.sm = d.sm + g0 * 64;
  r.q = d.queue + scalar_word(d.block_off, blk);
  const int64_t e = int64_t(blk) * d.T;
  r.seg = reinterpret_cast<const uint32_t*>(d.seg) + (e >> 1);
  r.seg_odd = uint32_t(e & 1);
  r.gb = int(std::min<int64_t>(d.G, d.n_groups - g0));
  r.nt = (r.gb + 15) / 16;
  return r;
}

// End (bytes from the block start) of tile t's segment.
__device__ inline uint32_t seg_end(const BlockRef& r, int t) {
  const uint32_t i = r.seg_odd + uint32_t(t);
  return 4u * ((((const const_word*)(r.seg))[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
}

// The loads of one tile step into a ring slot: 1 KB of sign+mantissa bytes
// and the queue segment [lo, hi) of the block, read from its 16-byte aligned
// floor (the slot then starts (address & 15) bytes before the segment) by NQ
// 1 KB direct loads, each with at least one active lane, so every step issues
// exactly 1 + NQ loads.
template <int NQ, bool NT = true>
__device__ inline void issue_step(const uint8_t* sm_tile, const uint8_t* q, uint32_t lo, uint32_t hi, uint32_t sm_slot,
                                  uint32_t q_slot, int lane) {
  if constexpr (NT) load_lds16_stream(sm_tile + 16 * lane, sm_slot);
  else load_lds16(sm_tile + 16 * lane, sm_slot);
  const uint8_t* a = q + lo;
  const uint32_t delta = uint32_t(reinterpret_cast<uintptr_t>(a)) & 15u;
  const uint8_t* base = a - delta;
  const uint32_t len = hi - lo + delta;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const uint32_t off = 1024u * i + 16u * uint32_t(lane);
    if (off < len || (lane == 0 && len <= 1024u * i)) load_lds16(base + (off < len ? off : 0u), q_slot + 1024u * i);
  }
}

// Wait until the oldest step in the ring has landed: each of the RS-1 younger
// steps has issued 1 + NQ loads and XTRA other vector-memory operations
// (activation loads) since.  Extra operations beyond that count (stores of a
// sink) only make the wait stricter.
template <int RS, int NQ, int XTRA>
__device__ inline void wait_oldest_step() {
  static_assert((RS - 1) * (1 + NQ + XTRA) < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((RS - 1) * (1 + NQ + XTRA)) : "memory");
}

// The table loads were issued before `issued` ring steps (1 + NQ loads
// each): wait until only those may be outstanding.
template <int RS, int NQ>
__device__ inline void wait_tables(int issued) {
  static_assert(RS * (1 + NQ) < 64, "vmcnt field");
  if (issued == RS) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(RS * (1 + NQ)) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Issue side of the ring over the tiles of blocks [b, b_end): steps run RS
// ahead of the consumer; past the end the last step is loaded again so the
// count of loads stays fixed.  The end of the next tile's segment is read one
// step early so its scalar load is back when it is needed.
template <int RS, int NQ, bool NT = true>
struct Feeder {
  BlockRef r;
  int blk, b_end, t;
  uint32_t lo, hi, next_hi;
  const uint8_t* sm_tile;
  __device__ void init(const DevMatrix& d, int b0, int b1, uint32_t sm_ring, uint32_t q_ring, int lane) {
    blk = b0;
    b_end = b1;
    t = 0;
    r = block_ref(d, b0);
    lo = hi = 0;
    next_hi = seg_end(r, 0);
    sm_tile = r.sm;
#pragma unroll
    for (int i = 0; i < RS; ++i) feed(d, sm_ring + 1024u * i, q_ring + uint32_t(d.slot_bytes) * i, lane);
  }
  __device__ void feed(const DevMatrix& d, uint32_t sm_slot, uint32_t q_slot, int lane) {
    issue_step<NQ, NT>(sm_tile, r.q, lo, next_hi, sm_slot, q_slot, lane);
    hi = next_hi;
    if (blk >= b_end) return;  // past the end: repeat the last step
    if (++t < r.nt) {
      lo = hi;
      sm_tile += 1024;
      next_hi = seg_end(r, t);
    } else if (++blk < b_end) {
      t = 0;
      r = block_ref(d, blk);
      lo = 0;
      sm_tile = r.sm;
      next_hi = seg_end(r, 0);
    } else {
      // stay on the last step
      --t;
    }
  }
};

// Consume the tiles of blocks [b0, b1) (whole rows) of one wave: every step
// waits for its slot, decodes the tile into the sink and refills the slot RS
// steps ahead.  Sink hooks: block_begin(blk), tile_end(t, nt), plus the
// per-weight calls of decode_tile.
template <int RS, int NQ, int XTRA, bool PAIR, bool NT = true, class Sink>
__device__ __forceinline__ void run_blocks(const DevMatrix& d, int b0, int b1, uint32_t sm_ring, uint32_t q_ring,
                                           int lane, Sink& sink) {
  Feeder<RS, NQ, NT> fd;
  fd.init(d, b0, b1, sm_ring, q_ring, lane);
  const int slot_bytes = d.slot_bytes, gpr = d.gpr;
  LaneDec s{};
  int slot = 0;
  for (int blk = b0; blk < b1; ++blk) {
    const BlockRef r = block_ref(d, blk);
    const int64_t g_first = int64_t(blk) * d.G;
    int64_t row0 = g_first / gpr;
    int c0 = int(g_first - row0 * gpr);
    sink.block_begin(blk);
    uint32_t pos = 0;  // bytes of the block's data consumed by earlier tiles
    const uint32_t qmis = uint32_t(reinterpret_cast<uintptr_t>(r.q));
    // tile 0: the segment starts with the block's head
    wait_oldest_step<RS, NQ, XTRA>();
    uint32_t rpos = lane_dec_start(s, q_ring + uint32_t(slot_bytes) * uint32_t(slot) + (qmis & 15u), d.rb_words, lane);
    for (int t = 0; t < r.nt; ++t) {
      const uint32_t sm_slot = sm_ring + 1024u * uint32_t(slot);
      const uint32_t q_slot = q_ring + uint32_t(slot_bytes) * uint32_t(slot);
      if (t) wait_oldest_step<RS, NQ, XTRA>();
      // a segment ends where its last word was taken, so the next one starts there
      const uint32_t q = q_slot + ((qmis + pos) & 15u);
      const uint4 cur = ld128(sm_slot + 16u * uint32_t(lane));
      const int nt = std::min(16, r.gb - 16 * t);
      const bool aligned = nt == 16 && c0 + 16 <= gpr && (c0 & 1) == 0;
      pos += decode_tile<PAIR>(d, s, q, rpos, cur, raw_mask16(s.raw_word, 16 * t), nt, aligned, row0, c0, lane, sink);
      rpos = 0;
      sink.tile_end(t, nt);
      c0 += 16;
      while (c0 >= gpr) {
        c0 -= gpr;
        ++row0;
      }
      // every LDS read of the slot is done before it is refilled
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      fd.feed(d, sm_slot, q_slot, lane);
      slot = slot + 1 == RS ? 0 : slot + 1;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // the repeated loads past the end land before the ring is reused
}

// ---------------------------------------------------------------------------
// Flat walk: when G and the groups per row are multiples of 16 no tile
// crosses a row, and the tiles of blocks [b0, b1) form one sequence of tile
// steps.  A slot is [1 KB sign+mantissa | queue part]; one M0 (the slot)
// serves all loads of a step, the queue loads reaching their part through
// the immediate offset 1024 (i + 1), which applies to both addresses.  The
// step table gives each tile's segment floor and the lanes of each load.

// The 1 + NQ loads of tile step v into a slot, from one M0 (the slot): the
// sign+mantissa tile v at offset 0 (all lanes), then the queue segment from
// its 16-byte floor at offsets 1024 (i + 1): rq starts 1 KB before the
// queue, so the immediate offset moves both addresses together.  Load i
// runs on the lanes below 64 - shift_i (byte i of `shifts`): exec =
// ~0 >> shift_i (s_lshr_b64 reads the low 6 bits of the shift).  The wave
// runs this with all lanes active.  The s_nop 4 covers a vector write of
// any of the scalar operands just before (the loads read them).  The
// sign+mantissa tile is read once and shares no cache line with another
// step, so its load is non-temporal (nt): it leaves the caches to what is
// reused (tables, x, the 16-byte floors that adjacent queue segments share)
// and, in the decompress, to the writes (gate: decompress 44.5 -> 36.0 us,
// GEMV 21.2 -> 18.9 us on one box, down 23.4 -> 22.7).  The queue loads stay
// cached: marked nt too, the line two segments share is fetched twice
// (2 % more traffic, no faster).
// The instructions of one step.  SMPOL is the cache policy of the
// sign+mantissa load ("nt " or ""); the s_lshr_b32 after the M0 write is also
// the wait state that write needs.  With NQ = 4, loads 2 and 3 run from M0 =
// slot + 2 KB and the floor + 2 KB (the immediate offset has 12 bits).
#define UW_STEP_HEAD(SMPOL)                                           \
  "s_nop 4\n"                                                         \
  "s_mov_b32 m0, %[slot]\n"                                           \
  "s_lshr_b32 %[t], %[sh], 8\n"                                       \
  "buffer_load_dwordx4 %[l16], %[rsm], %[smo] offen " SMPOL "lds\n"   \
  "s_lshr_b64 exec, -1, %[sh]\n"                                      \
  "buffer_load_dwordx4 %[l16], %[rq], %[fl] offen offset:1024 lds\n"  \
  "s_lshr_b64 exec, -1, %[t]\n"                                       \
  "buffer_load_dwordx4 %[l16], %[rq], %[fl] offen offset:2048 lds\n"
#define UW_STEP_TAIL4                                                 \
  "s_add_u32 m0, %[slot], 0x800\n"                                    \
  "s_lshr_b32 %[t], %[sh], 16\n"                                      \
  "s_add_u32 %[f2], %[fl], 0x800\n"                                   \
  "s_lshr_b64 exec, -1, %[t]\n"                                       \
  "buffer_load_dwordx4 %[l16], %[rq], %[f2] offen offset:1024 lds\n"  \
  "s_lshr_b32 %[t], %[sh], 24\n"                                      \
  "s_lshr_b64 exec, -1, %[t]\n"                                       \
  "buffer_load_dwordx4 %[l16], %[rq], %[f2] offen offset:2048 lds\n"
#define UW_STEP_IN                                                                                          \
  [slot] "s"(slot), [l16] "v"(lane16), [rsm] "s"(rsm), [smo] "s"(sm_off), [rq] "s"(rq), [fl] "s"(floor16), \
      [sh] "s"(shifts)
// NT: the sign+mantissa load is non-temporal.  A caller whose next kernel
// reads the same sign+mantissa bytes again (the exponent-plane decode) keeps
// them cached.
template <int NQ, bool NT = true>
__device__ __forceinline__ void issue_flat(__amdgpu_buffer_rsrc_t rsm, __amdgpu_buffer_rsrc_t rq, int v,
                                           uint32_t floor16, uint32_t shifts, uint32_t slot, uint32_t lane16) {
  static_assert(NQ == 2 || NQ == 4, "queue loads per step");
  const uint32_t sm_off = uint32_t(v) * 1024u;
  uint32_t t, f2;
  if constexpr (NQ == 2 && NT)
    asm volatile(UW_STEP_HEAD("nt ") "s_mov_b64 exec, -1" : [t] "=&s"(t) : UW_STEP_IN : "memory", "m0", "exec");
  else if constexpr (NQ == 2)
    asm volatile(UW_STEP_HEAD("") "s_mov_b64 exec, -1" : [t] "=&s"(t) : UW_STEP_IN : "memory", "m0", "exec");
  else if constexpr (NT)
    asm volatile(UW_STEP_HEAD("nt ") UW_STEP_TAIL4 "s_mov_b64 exec, -1"
                 : [t] "=&s"(t), [f2] "=&s"(f2)
                 : UW_STEP_IN
                 : "memory", "m0", "exec");
  else
    asm volatile(UW_STEP_HEAD("") UW_STEP_TAIL4 "s_mov_b64 exec, -1"
                 : [t] "=&s"(t), [f2] "=&s"(f2)
                 : UW_STEP_IN
                 : "memory", "m0", "exec");
  (void)f2;
}
#undef UW_STEP_HEAD
#undef UW_STEP_TAIL4
#undef UW_STEP_IN

// N loads of 16 bytes on lane 0 only (from the start of the resource) into
// the 16 bytes at dst: they keep a step's count of loads where there is
// nothing to load.  Runs with all lanes active, like issue_flat.
template <int N>
__device__ __forceinline__ void issue_dummy(__amdgpu_buffer_rsrc_t r, uint32_t dst, uint32_t lane16) {
  static_assert(N == 3 || N == 5, "loads per step");
  if constexpr (N == 3) {
    asm volatile(
        "s_nop 4\n"
        "s_mov_b32 m0, %[dst]\n"
        "s_mov_b64 exec, 1\n"  // also the wait state after the M0 write
        "buffer_load_dwordx4 %[l16], %[r], 0 offen lds\n"
        "buffer_load_dwordx4 %[l16], %[r], 0 offen lds\n"
        "buffer_load_dwordx4 %[l16], %[r], 0 offen lds\n"
        "s_mov_b64 exec, -1" ::[dst] "s"(dst),
        [l16] "v"(lane16), [r] "s"(r)
        : "memory", "m0", "exec");
  } else {
    asm volatile(
        "s_nop 4\n"
        "s_mov_b32 m0, %[dst]\n"
        "s_mov_b64 exec, 1\n"
        "buffer_load_dwordx4 %[l16], %[r], 0 offen lds\n"
        "buffer_load_dwordx4 %[l16], %[r], 0 offen lds\n"
        "buffer_load_dwordx4 %[l16], %[r], 0 offen lds\n"
        "buffer_load_dwordx4 %[l16], %[r], 0 offen lds\n"
        "buffer_load_dwordx4 %[l16], %[r], 0 offen lds\n"
        "s_mov_b64 exec, -1" ::[dst] "s"(dst),
        [l16] "v"(lane16), [r] "s"(r)
        : "memory", "m0", "exec");
  }
}

// Resources of the flat walk's loads: the sign+mantissa section, and the
// queue from 1 KB before it (so one immediate offset moves the global and
// the LDS address of a queue load together).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t flat_rsm(const DevMatrix& d) {
  return byte_rsrc(d.sm, uint32_t(d.n_tiles) * 1024u);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t flat_rq(const DevMatrix& d) { return byte_rsrc(d.queue - 1024, d.q_extent); }

// Work item u of the flat-walk VALU product and decompress: blocks [b0, b1)
// from row `row`, column group c0.  A work unit (whole rows), or with split
// rows one block, whose first tile may start mid-row.
struct WalkItem {
  int b0, b1;
  int64_t row;
  int c0;
};
__device__ __forceinline__ WalkItem walk_item(const DevMatrix& d, int u) {
  WalkItem w;
  if (d.split) {
    const int v = u * d.T, tpr = d.gpr >> 4;
    const int r = v / tpr;
    w.b0 = u;
    w.b1 = u + 1;
    w.row = r;
    w.c0 = (v - r * tpr) * 16;
  } else {
    w.b0 = u * d.unit_blocks;
    w.b1 = std::min(d.n_blocks, w.b0 + d.unit_blocks);
    w.row = int64_t(u) * d.rows_per_unit;
    w.c0 = 0;
  }
  return w;
}
// Split rows: whether the item's last row goes on in the next block.
__device__ __forceinline__ bool item_ends_mid_row(const DevMatrix& d, const WalkItem& w) {
  return std::min(w.b1 * d.T, d.n_tiles) % (d.gpr >> 4) != 0;
}

// Issue the first RS steps of the tiles of blocks [b0, b1) into the ring;
// returns the next step to issue.
template <int RS, int NQ, bool NT = true>
__device__ __forceinline__ int flat_start(const DevMatrix& d, int b0, int b1, uint32_t ring, int lane) {
  const uint32_t lane16 = 16u * uint32_t(lane);
  const uint32_t stride = 1024u + uint32_t(d.slot_bytes);
  const int u1 = std::min(b1 * d.T, d.n_tiles);
  const __amdgpu_buffer_rsrc_t rsm = flat_rsm(d), rq = flat_rq(d);
  int fv = b0 * d.T;
  const const_word* fstep = (const const_word*)(d.steps) + 2u * uint32_t(fv);
  uint32_t slot = ring;
#pragma unroll
  for (int i = 0; i < RS; ++i) {
    if (fv < u1) {
      issue_flat<NQ, NT>(rsm, rq, fv, fstep[0], fstep[1], slot, lane16);
      ++fv;
      fstep += 2;
      slot += stride;
    }
  }
  return fv;
}

// Wave priority (s_setprio takes an immediate).  A SIMD issues the ready
// wave of highest priority, the oldest first among equals; with equal
// priorities the first waves of a workgroup run ahead and the last ones end
// the kernel alone.  The walk sets its priority from the tiles it has left,
// so waves that fall behind are issued first and the waves of a SIMD finish
// together (gate GEMV -2.3 %, down -3.6 %).
__device__ __forceinline__ void set_priority(int p) {
  if (p <= 0) asm volatile("s_setprio 0");
  else if (p == 1) asm volatile("s_setprio 1");
  else if (p == 2) asm volatile("s_setprio 2");
  else asm volatile("s_setprio 3");
}

// Tiles of blocks [b0, b1), whose first tile is at row row_base, column
// group c_start (0 unless blocks split rows); flat_start has issued the
// steps before fv0.
template <int RS, int NQ, int XTRA, bool PAIR, bool NT = true, class Sink>
__device__ __forceinline__ void run_flat(const DevMatrix& d, int fv0, int b0, int b1, int64_t row_base, int c_start,
                                         uint32_t ring, int lane, Sink& sink) {
  const uint32_t lane16 = 16u * uint32_t(lane);
  const uint32_t stride = 1024u + uint32_t(d.slot_bytes);
  const uint32_t ring_last = ring + (RS - 1) * stride;
  const int T = d.T;
  const int u0 = b0 * T, u1 = std::min(b1 * T, d.n_tiles);
  const __amdgpu_buffer_rsrc_t rsm = flat_rsm(d), rq = flat_rq(d);
  // issue side: the descriptor of the next step to issue is read one step
  // ahead (the table has a spare entry at its end)
  int fv = __builtin_amdgcn_readfirstlane(fv0);
  const const_word* fstep = (const const_word*)(d.steps) + 2u * uint32_t(fv);
  uint32_t f_floor = fstep[0], f_shifts = fstep[1];
  // consume side
  uint32_t qpos = scalar_word(d.block_off, b0);  // queue offset of the next segment
  int64_t row = row_base;
  int c0 = c_start, t = 0;  // a block start
  uint32_t tile_rm = 0;  // lane t: raw flags of tile t of the current block
  uint32_t rpos = 0;     // the segment's head bytes (tile 0 of a block)
  LaneDec s{};
  uint32_t slot = ring;
  // A block start: the head of tile 0's segment starts the lane decoders.
  // It runs before the tile loop and at the end of a block's last tile (after
  // the next step's wait), so the loop itself has no block-start branch.
  auto block_start = [&]() {
    const uint32_t q = slot + 1024u + (qpos & 15u);
    rpos = lane_dec_start(s, q, d.rb_words, lane);
    tile_rm = (ld32(q + 128 + 4 * uint32_t(lane >> 1)) >> (16 * (lane & 1))) & 0xFFFFu;
  };
  // One tile step: decode the slot's tile into the sink, then (FEED) refill
  // the slot with the step RS ahead.
  auto step = [&](auto feed) {
    const uint32_t q = slot + 1024u + (qpos & 15u);
    const uint4 cur = ld128(slot + lane16);
    const uint32_t rmask = __builtin_amdgcn_readlane(tile_rm, t);
    qpos += __builtin_amdgcn_readfirstlane(decode_tile<PAIR>(d, s, q, rpos, cur, rmask, 16, true, row, c0, lane, sink));
    rpos = 0;
    sink.tile_end(t, 16);
    c0 += 16;
    if (c0 == d.gpr) {
      c0 = 0;
      ++row;
      sink.row_end();
    }
    if constexpr (decltype(feed)::value) {
      // every LDS read of the slot is done before it is refilled (the
      // builtin form, so the compiler knows the reads have completed)
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      issue_flat<NQ, NT>(rsm, rq, fv, f_floor, f_shifts, slot, lane16);
      ++fv;
      fstep += 2;
      f_floor = fstep[0];
      f_shifts = fstep[1];
    }
    slot = slot == ring_last ? ring : slot + stride;
    return ++t == T;
  };
  int v = u0;
  // steady state: RS - 1 younger steps in flight, and every step refills its
  // slot (a second wait for the same step is satisfied at once)
  if (v < u1 - RS) wait_oldest_step<RS, NQ, XTRA>();
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  block_start();
  for (; v < u1 - RS; ++v) {
    wait_oldest_step<RS, NQ, XTRA>();
    if (((u1 - v) & 3) == 0) set_priority(std::min(3, (u1 - v) >> 2));  // every 4 tiles
    if (step(std::true_type{})) {
      t = 0;
      if (v + 1 < u1 - RS) wait_oldest_step<RS, NQ, XTRA>();
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      block_start();
    }
  }
  // the last RS steps: everything has been issued
  if (v < u1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  for (; v < u1; ++v) {
    if (step(std::false_type{}) && v + 1 < u1) {
      t = 0;
      block_start();
    }
  }
}

constexpr int kRS = 4;  // tile steps in flight per wave (the flat walk may use kRSLow)
constexpr int kRSLow = 2;

__host__ __device__ inline uint32_t ring_bytes(int rs, int slot_bytes) { return uint32_t(rs) * (1024u + uint32_t(slot_bytes)); }

// ---------------------------------------------------------------------------
// Decompress.  On the flat walk each pair of weights goes straight to its
// row; on the block walk (tiles may cross rows) weights pass through a
// per-wave LDS tile [16][64] bf16 so that each lane stores 2 x 16 bytes of
// consecutive columns.
template <bool FLAT>
struct DecompressSink {
  int64_t cols, G;
  uint16_t* out;
  int64_t ld_out;
  uint32_t tile;  // LDS byte address of the transpose tile
  int lane;
  int64_t trow;   // (row, col) of the current tile's first weight
  int64_t tcol;
  uint16_t* dst;  // flat walk: this lane's column of the tile's first group
  int64_t row_base;  // output row 0 is matrix row row_base (a band of rows)
  __device__ void unit_begin(int) {}
  __device__ void unit_end() {}
  __device__ void block_begin(int blk) {
    if (FLAT) return;  // the flat walk gives each tile's place
    const int64_t flat = int64_t(blk) * G * 64;
    trow = flat / cols;
    tcol = flat - trow * cols;
  }
  __device__ void row_end() {}
  __device__ void tile_raw(uint32_t) {}
  __device__ void tile_begin(int64_t row0, int c0) {
    if (!FLAT) return;
    trow = row0;
    tcol = int64_t(c0) * 64;
    dst = out + (row0 - row_base) * ld_out + tcol + lane;
  }
  // flat walk: weight (group 2k or 2k+1, lane) straight to its row; each
  // store instruction writes 128 contiguous bytes across the wave
  __device__ void pair(int k, uint32_t D) {
    if (FLAT) {
      dst[(2 * k) * kWave] = uint16_t(D);
      dst[(2 * k + 1) * kWave] = uint16_t(D >> 16);
      return;
    }
    st16(tile + ((2 * k) * kWave + lane) * 2, D);
    st16(tile + ((2 * k + 1) * kWave + lane) * 2, D >> 16);
  }
  __device__ void single(int jj, int64_t, int, uint32_t w) { st16(tile + (jj * kWave + lane) * 2, w); }
  __device__ void tile_end(int, int nt) {
    if (FLAT) return;
    wave_lds_fence();
    if (lane * 16 < nt * 64) {
      const uint4 a = ld128(tile + lane * 32), b = ld128(tile + lane * 32 + 16);
      int64_t row = trow, col = tcol + lane * 16;
      while (!FLAT && col >= cols) {
        col -= cols;
        ++row;
      }
      uint4* dst = reinterpret_cast<uint4*>(out + (row - row_base) * ld_out + col);
      dst[0] = a;
      dst[1] = b;
    }
    wave_lds_fence();
    if (FLAT) return;
    tcol += 1024;
    while (tcol >= cols) {
      tcol -= cols;
      ++trow;
    }
  }
};

// Exponent bytes only (the exponent-only pipeline, flat walk): tile T's
// exponents go to out + 1024 T in the order of the sign+mantissa section
// (lane l's 16 bytes at 16 l, byte jj = weight l of group jj), one 16-byte
// store per lane per tile.
struct ExpSink {
  int64_t cols;
  uint8_t* out;
  int lane;
  uint8_t* dst = nullptr;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  __device__ void unit_begin(int) {}
  __device__ void unit_end() {}
  __device__ void block_begin(int) {}
  __device__ void row_end() {}
  __device__ void tile_raw(uint32_t) {}
  __device__ void tile_begin(int64_t row0, int c0) {
    dst = out + row0 * cols + int64_t(c0) * 64 + 16 * lane;
    w[0] = w[1] = w[2] = w[3] = 0u;
  }
  __device__ void pair(int k, uint32_t D) {
    w[k >> 1] |= (((D >> 7) & 0xFFu) | (((D >> 23) & 0xFFu) << 8)) << (16 * (k & 1));
  }
  __device__ void single(int, int64_t, int, uint32_t) {}  // flat-walk tiles are always whole
  __device__ void tile_end(int, int) { *reinterpret_cast<uint4*>(dst) = uint4{w[0], w[1], w[2], w[3]}; }
};

// The direct-palette form (UWP1) of the decoded tiles, for the transcode at
// load time.  The walk runs with the index tables, so a coded weight arrives
// with its palette index where the exponent would be; a raw group's weights
// arrive with their exponent bytes.  Tile T (1024 weights, flat walk: inside
// one row) holds UWP1 weights 1024 T ..: the lane's weight of group j is
// column 64 j + lane of the tile, so its sign+mantissa byte goes to sm
// + 1024 T + 64 j + lane and its index nibble to idx byte 512 T + 32 j +
// lane / 2 (even lane: low nibble; the odd neighbour's nibble comes over DPP);
// raw group j of the tile (the rank-th raw group of the matrix, rank from
// the prefix section the pre-pass wrote) puts its exponent bytes at raw +
// 64 rank.
struct PaletteOut {
  uint8_t* sm;
  uint8_t* idx;
  uint8_t* raw;
  const uint32_t* prefix;
};

struct PaletteSink {
  PaletteOut o;
  int tpr;  // tiles per row
  int lane;
  uint8_t* dsm = nullptr;
  uint8_t* didx = nullptr;
  uint8_t* draw = nullptr;
  uint32_t rmask = 0;
  __device__ void unit_begin(int) {}
  __device__ void unit_end() {}
  __device__ void block_begin(int) {}
  __device__ void row_end() {}
  __device__ void tile_raw(uint32_t r) { rmask = r; }
  __device__ void tile_begin(int64_t row0, int c0) {
    const int64_t T = row0 * tpr + (c0 >> 4);
    dsm = o.sm + T * 1024 + lane;
    didx = o.idx + T * 512 + (lane >> 1);
    draw = o.raw + int64_t(scalar_word(o.prefix, T)) * 64 + lane;
  }
  __device__ void one(int j, uint32_t h) {  // h: the weight's bf16 bits (exponent field = index or raw exponent)
    dsm[64 * j] = uint8_t(((h >> 8) & 0x80u) | (h & 0x7Fu));
    const uint32_t e = (h >> 7) & 0xFFu;
    const bool raw = (rmask >> j) & 1u;  // wave-uniform
    const uint32_t nib = raw ? 0u : e;
    const uint32_t other = uint32_t(__builtin_amdgcn_update_dpp(0, int(nib), 0xB1, 0xF, 0xF, false));  // lane ^ 1
    if (!(lane & 1)) didx[32 * j] = uint8_t(nib | (other << 4));
    if (raw) draw[64 * __builtin_popcount(rmask & ((1u << j) - 1u))] = uint8_t(e);
  }
  __device__ void pair(int k, uint32_t D) {
    one(2 * k, D & 0xFFFFu);
    one(2 * k + 1, D >> 16);
  }
  __device__ void single(int, int64_t, int, uint32_t) {}  // flat-walk tiles are always whole
  __device__ void tile_end(int, int) {}
};

// SINK: 0 = bf16 weights, 1 = exponent bytes, 2 = the direct-palette form.
template <int SINK, bool FLAT>
__device__ inline auto make_decompress_sink(const DevMatrix& d, uint16_t* out, int64_t ld_out, const PaletteOut& po,
                                            uint32_t tile, int lane) {
  if constexpr (SINK == 1) return ExpSink{d.cols, reinterpret_cast<uint8_t*>(out), lane};
  else if constexpr (SINK == 2) return PaletteSink{po, d.gpr >> 4, lane};
  else return DecompressSink<FLAT>{d.cols, d.G, out, ld_out, tile, lane, 0, 0, nullptr, 0};
}

// Work items [item0, item1) (units, or with split rows blocks, whose rows
// are whole); the bf16 sink writes matrix row r to output row r - row_base.
template <bool PAIR, int NQ, bool FLAT, int RS, int SINK = 0>
__global__ __launch_bounds__(1024) void decompress_kernel(DevMatrix d, uint16_t* __restrict__ out, int64_t ld_out,
                                                          PaletteOut po, int item0, int item1, int64_t row_base) {
  extern __shared__ uint32_t lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int waves = blockDim.x / kWave;
  const uint32_t per_wave = ring_bytes(RS, d.slot_bytes) + (FLAT ? 0u : kTransposeWords * 4);
  const uint32_t sm_ring = kAreaAddr + uint32_t(wave) * per_wave;
  const uint32_t q_ring = sm_ring + RS * 1024;
  const uint32_t tile = sm_ring + ring_bytes(RS, d.slot_bytes);
  const int u_first = item0 + blockIdx.x * waves + wave;
  const int n_items = item1;
  int fv = 0;
  // the exponent plane's product reads the sign+mantissa bytes next, so this
  // decode leaves them cached
  constexpr bool kNT = SINK != 1;
  // the decode tables, then the first unit's loads; the tables have landed
  // once only the ring's loads may be younger
  const int n_tab = issue_tables(d, wave, waves, lane);
  int issued = 0;
  if (FLAT && u_first < n_items) {
    const WalkItem it = walk_item(d, u_first);
    fv = flat_start<RS, NQ, kNT>(d, it.b0, it.b1, sm_ring, lane);
    issued = fv - it.b0 * d.T;
  }
  if (n_tab) wait_tables<RS, NQ>(issued);
  lds_barrier();
  using Sink = std::conditional_t<SINK == 1, ExpSink, std::conditional_t<SINK == 2, PaletteSink, DecompressSink<FLAT>>>;
  Sink sink = make_decompress_sink<SINK, FLAT>(d, out, ld_out, po, tile, lane);
  if constexpr (SINK == 0) sink.row_base = row_base;
  for (int u = u_first; u < n_items; u += gridDim.x * waves) {
    // the two 16-byte stores per tile only make the ring waits stricter
    if (FLAT) {
      const WalkItem it = walk_item(d, u);
      if (u != u_first) fv = flat_start<RS, NQ, kNT>(d, it.b0, it.b1, sm_ring, lane);
      run_flat<RS, NQ, 0, PAIR, kNT>(d, fv, it.b0, it.b1, it.row, it.c0, sm_ring, lane, sink);
    } else {
      const int b0 = u * d.unit_blocks, b1 = std::min(d.n_blocks, b0 + d.unit_blocks);
      run_blocks<RS, NQ, 0, PAIR, kNT>(d, b0, b1, sm_ring, q_ring, lane, sink);
    }
  }
}

// Transcode pre-pass (one workgroup): the UWP1 raw flags (16 bits per tile)
// and per-tile raw-group prefix counts from the raw bits in every block's
// head.  Thread i takes a contiguous run of blocks; the runs' counts are
// scanned in LDS.
__global__ __launch_bounds__(1024) void palette_prefix_kernel(DevMatrix d, uint16_t* __restrict__ flags,
                                                               uint32_t* __restrict__ prefix) {
  __shared__ uint32_t part[1024];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int per = (d.n_blocks + nt - 1) / nt;
  const int b0 = std::min(d.n_blocks, tid * per), b1 = std::min(d.n_blocks, b0 + per);
  auto raw_word = [&](int b, int w) {
    return *reinterpret_cast<const uint32_t*>(d.queue + d.block_off[b] + 128 + 4 * w);
  };
  uint32_t cnt = 0;
  for (int b = b0; b < b1; ++b)
    for (int w = 0; w < d.rb_words; ++w) cnt += __builtin_popcount(raw_word(b, w));
  part[tid] = cnt;
  __syncthreads();
  // exclusive scan of part[] (Hillis-Steele over the 1024 entries)
  for (int off = 1; off < nt; off <<= 1) {
    const uint32_t v = tid >= off ? part[tid - off] : 0u;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  uint32_t run = part[tid] - cnt;
  for (int b = b0; b < b1; ++b) {
    // the last block may be short: only its own tiles (flat walk: whole tiles)
    const int nt_b = int(std::min<int64_t>(d.G, d.n_groups - int64_t(b) * d.G) / 16);
    for (int t = 0; t < nt_b; ++t) {
      const int64_t T = int64_t(b) * d.T + t;
      const uint32_t f = (raw_word(b, (16 * t) >> 5) >> ((16 * t) & 31)) & 0xFFFFu;
      flags[T] = uint16_t(f);
      prefix[T] = run;
      run += __builtin_popcount(f);
    }
  }
}

// Header and the zero bytes between sections of the transcoded UWP1 blob.
struct PaletteFill {
  uint32_t head[16];        // the 64-byte header
  uint64_t gap_lo[6], gap_hi[6];  // byte ranges to clear
};
__global__ void palette_fill_kernel(uint8_t* __restrict__ out, PaletteFill f) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && tid < 16) reinterpret_cast<uint32_t*>(out)[tid] = f.head[tid];
  for (int g = 0; g < 6; ++g)
    for (uint64_t i = f.gap_lo[g] + uint64_t(blockIdx.x) * blockDim.x + tid; i < f.gap_hi[g];
         i += uint64_t(gridDim.x) * blockDim.x)
      out[i] = 0;
}

// ---------------------------------------------------------------------------
// Fused product Y[b, n] = sum_k X[b, k] W[n, k] for NBP batch columns per pass.
// X lives in LDS at kAreaAddr.  bf16 x as pairs: pair p at lane l holds
// X[b][128p + l] | X[b][128p + 64 + l] << 16 (column groups 2p and 2p+1) in
// word x_word(p, l)*NBP + b, where the 8 pairs of a 16-group tile are 8
// consecutive words of the lane (2 NBP 16-byte reads per tile); fp32 x as
// word k*NBP + b = X[b][k].  With NBP >= 2 a lane's block of 8 NBP words
// starts every 32 NBP bytes, so the lanes a read serves together would meet
// on the same banks: 16-byte chunk j of lane l's block is stored at chunk
// j ^ x_swz(l), which differs between lanes whose blocks start on the same
// bank (x_slot gives the word for pair p, lane l, batch column b).
__host__ __device__ inline uint32_t x_word(uint32_t p, uint32_t l) { return (((p >> 3) * 64 + l) << 3) + (p & 7); }
template <int NBP>
__host__ __device__ inline uint32_t x_swz(uint32_t l) {
  return NBP >= 2 ? (l * 2u * NBP / 16u) & (2u * NBP - 1u) : 0u;
}
template <int NBP>
__host__ __device__ inline uint32_t x_slot(uint32_t p, uint32_t l, uint32_t b) {
  const uint32_t w = (p & 7) * NBP + b;  // word in the lane's block
  return ((p >> 3) * 64 + l) * 8 * NBP + ((((w >> 2) ^ x_swz<NBP>(l)) << 2) | (w & 3));
}
template <int NBP, bool XF32>
__device__ inline void load_x(const DevMatrix& d, const void* X, int64_t ldx, int nb_valid, uint32_t* xl) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int64_t C = d.cols;
  if (XF32) {
    const float* x = static_cast<const float*>(X);
    for (uint32_t i = tid; i < uint32_t(C) * NBP; i += nt) {
      const uint32_t k = i / NBP;
      const int b = int(i % NBP);
      xl[i] = b < nb_valid ? f32_bits(x[b * ldx + k]) : 0u;
    }
  } else {
    const uint16_t* x = static_cast<const uint16_t*>(X);
    const uint32_t npairs = (uint32_t(d.gpr) + 15) / 16 * 8;  // whole 8-pair chunks
    for (uint32_t i = tid; i < npairs * 64 * NBP; i += nt) {
      const uint32_t pl = i / NBP;
      const int b = int(i % NBP);
      const uint32_t p = pl / 64, l = pl % 64;
      const int64_t k0 = 128 * int64_t(p) + l, k1 = k0 + 64;
      uint32_t v = 0;
      if (b < nb_valid && k0 < C) {
        v = x[b * ldx + k0];
        if (k1 < C) v |= uint32_t(x[b * ldx + k1]) << 16;
      }
      xl[x_slot<NBP>(p, l, uint32_t(b))] = v;
    }
  }
}

// One row of bf16 x, issued before the ring's first steps so that its loads
// are not queued behind them: each thread loads the two halves of up to
// kXIters words of the x_word layout into registers (asm loads, which the
// compiler does not wait for), and x_store writes them once a wait has
// covered them.  Covers cols up to 2 * 64 * kXIters * threads / 64.
constexpr int kXIters = 8;
struct XEarly {
  uint32_t lo[kXIters], hi[kXIters];
};
__device__ inline bool x_early_fits(const DevMatrix& d, int threads) {
  return ((uint32_t(d.gpr) + 15) / 16 * 8) * 64u <= uint32_t(kXIters) * uint32_t(threads);
}
__device__ __forceinline__ void x_issue(const DevMatrix& d, const uint16_t* x, XEarly& xe) {
  const uint32_t C = uint32_t(d.cols), words = ((uint32_t(d.gpr) + 15) / 16 * 8) * 64u;
#pragma unroll
  for (int j = 0; j < kXIters; ++j) {
    const uint32_t i = threadIdx.x + uint32_t(j) * blockDim.x;
    xe.lo[j] = xe.hi[j] = 0u;
    if (i < words) {
      const uint32_t k0 = 128u * (i / 64u) + i % 64u, k1 = k0 + 64u;
      asm volatile("global_load_ushort %0, %1, off" : "=v"(xe.lo[j]) : "v"(x + (k0 < C ? k0 : 0u)) : "memory");
      asm volatile("global_load_ushort %0, %1, off" : "=v"(xe.hi[j]) : "v"(x + (k1 < C ? k1 : 0u)) : "memory");
    }
  }
}
// After a wait that covers x_issue's loads.
__device__ __forceinline__ void x_store(const DevMatrix& d, XEarly& xe, uint32_t* xl) {
  const uint32_t C = uint32_t(d.cols), words = ((uint32_t(d.gpr) + 15) / 16 * 8) * 64u;
#pragma unroll
  for (int j = 0; j < kXIters; ++j) {
    asm volatile("" : "+v"(xe.lo[j]), "+v"(xe.hi[j]));
    const uint32_t i = threadIdx.x + uint32_t(j) * blockDim.x;
    if (i < words) {
      const uint32_t p = i / 64u, l = i % 64u, k0 = 128u * p + l, k1 = k0 + 64u;
      xl[x_word(p, l)] = (k0 < C ? (xe.lo[j] & 0xFFFFu) : 0u) | (k1 < C ? (xe.hi[j] << 16) : 0u);
    }
  }
}

template <int NBP, bool XF32, bool YBF16, bool FLAT>
struct ProductSink {
  const DevMatrix& d;
  uint32_t xaddr;  // LDS byte address of x
  int lane;
  int nb_valid;
  void* Y;
  int64_t ldy;
  int cur_row;  // row being accumulated, relative to first_row
  int c0;
  uint32_t xtile;  // x address of this lane for column group c0
  uint32_t xw[8 * NBP];  // flat walk, bf16 x: the tile's x words of this lane
  uint32_t xlane;        // xaddr + lane * 32 * NBP
  float acc[NBP];
  // Finished rows are parked in registers (lane r holds the r-th finished row
  // of the unit) and written with one store after the unit, so the decode
  // loop issues no global stores.
  float rows_done[NBP];
  int64_t first_row;
  int n_done;

  __device__ void store_done() {
#pragma unroll
    for (int b = 0; b < NBP; ++b) {
      if (lane < n_done && b < nb_valid) {
        if (YBF16) static_cast<uint16_t*>(Y)[b * ldy + first_row + lane] = f32_to_bf16(rows_done[b]);
        else static_cast<float*>(Y)[b * ldy + first_row + lane] = rows_done[b];
      }
    }
    first_row += n_done;
    n_done = 0;
  }
  __device__ void flush() {
#pragma unroll
    for (int b = 0; b < NBP; ++b) {
      const float s = wave_sum(acc[b]);
      rows_done[b] = lane == n_done ? s : rows_done[b];
      acc[b] = 0.f;
    }
    // every lane holds a finished row: store them.  Only the block walk
    // has units of more than 64 rows: on the flat walk (G <= 1024 and the
    // groups per row a multiple of 16) a unit spans G / gcd(G, groups per
    // row) <= 64 rows, and a split-row item at most 64 (checked on the host).
    ++n_done;
    if (!FLAT && n_done == kWave) store_done();
  }
  __device__ void to_row(int64_t row) {
    if (int(row - first_row) != cur_row) {
      flush();
      cur_row = int(row - first_row);
    }
  }
  __device__ void tile_raw(uint32_t) {}
  __device__ void tile_begin(int64_t row0, int c) {
    if (!FLAT) to_row(row0);  // the flat walk ends rows with row_end()
    c0 = c;
    if (XF32) {
      xtile = xaddr + ((uint32_t(c) * 64 + lane) * NBP) * 4;
    } else if (FLAT) {
      // c is a multiple of 16: the tile's 8 pairs are the 8 * NBP words at
      // x_word(c / 2, lane) * NBP = (c / 16 * 64 + lane) * 8 * NBP
      const uint32_t a = xlane + (uint32_t(c) >> 4) * (2048u * NBP);
      const uint32_t swz = x_swz<NBP>(uint32_t(lane));
#pragma unroll
      for (int j = 0; j < 2 * NBP; ++j) {
        const uint4 v = ld128(a + 16 * (uint32_t(j) ^ swz));
        xw[4 * j] = v.x;
        xw[4 * j + 1] = v.y;
        xw[4 * j + 2] = v.z;
        xw[4 * j + 3] = v.w;
      }
    }
  }
  // x of column group cg at this lane
  __device__ float x_at(int cg, int b) const {
    if (XF32) return bits_f32(ld32(xaddr + ((uint32_t(cg) * 64 + lane) * NBP + b) * 4));
    const uint32_t v = ld32(xaddr + x_slot<NBP>(uint32_t(cg) >> 1, uint32_t(lane), uint32_t(b)) * 4);
    return bits_f32((cg & 1) ? (v & 0xFFFF0000u) : (v << 16));
  }
  // tile_begin() guarantees an even c0: pair k is x pair c0/2 + k
  __device__ void pair(int k, uint32_t D) {
    if (XF32) {
      const float wa = bits_f32(D << 16), wb = bits_f32(D & 0xFFFF0000u);
      const uint32_t a = xtile + uint32_t(2 * k * 64 * NBP * 4);
#pragma unroll
      for (int b = 0; b < NBP; ++b) {
        acc[b] = __builtin_fmaf(wa, bits_f32(ld32(a + 4 * b)), acc[b]);
        acc[b] = __builtin_fmaf(wb, bits_f32(ld32(a + 64 * NBP * 4 + 4 * b)), acc[b]);
      }
    } else if (FLAT) {
#pragma unroll
      for (int b = 0; b < NBP; ++b) acc[b] = dot2_bf16(D, xw[k * NBP + b], acc[b]);
    } else {
      const uint32_t pk = (uint32_t(c0) >> 1) + uint32_t(k);
#pragma unroll
      for (int b = 0; b < NBP; ++b) acc[b] = dot2_bf16(D, ld32(xaddr + x_slot<NBP>(pk, uint32_t(lane), uint32_t(b)) * 4), acc[b]);
    }
  }
  __device__ void single(int, int64_t row, int cg, uint32_t w) {
    to_row(row);
    const float wf = bits_f32(w << 16);
#pragma unroll
    for (int b = 0; b < NBP; ++b) acc[b] = __builtin_fmaf(wf, x_at(cg, b), acc[b]);
  }
  __device__ void tile_end(int, int) {}
  __device__ void block_begin(int) {}
  // finished rows are stored when the work item ends
  __device__ void unit_begin(int64_t row0) {
    xlane = xaddr + uint32_t(lane) * 32u * NBP;
    first_row = row0;
    cur_row = 0;
    n_done = 0;
#pragma unroll
    for (int b = 0; b < NBP; ++b) acc[b] = rows_done[b] = 0.f;
  }
  __device__ void row_end() { flush(); }
  __device__ void unit_end() {
    if (!FLAT) flush();  // the flat walk has ended the unit's last row
    store_done();
  }
  // Split rows.  The item's last row goes on in the next block: its partial
  // sums go to LDS at `at` (NBP floats) instead of Y.
  __device__ void park_tail(uint32_t at) {
    flush();
    --n_done;
#pragma unroll
    for (int b = 0; b < NBP; ++b)
      if (lane == n_done) st32(at + 4 * b, f32_bits(rows_done[b]));
  }
  // The item's first row began in the previous block, whose wave parked that
  // part at `at`: the row is that part plus this one.
  __device__ void add_head(uint32_t at) {
#pragma unroll
    for (int b = 0; b < NBP; ++b)
      if (lane == 0) rows_done[b] = bits_f32(ld32(at + 4 * b)) + rows_done[b];
  }
};

// Up to 16 waves per workgroup (4 per SIMD, so every unit of a 4096-unit
// matrix starts in the first round); 8 batch rows of fp32 x, or on the block
// walk, need more registers per lane than 4 waves per SIMD leave: at most 8
// waves there.
constexpr int fused_max_threads(int nbp, bool xf32, bool flat) { return nbp >= 8 && (xf32 || !flat) ? 512 : 1024; }

template <int NBP, bool XF32, bool PAIR, bool YBF16, int NQ, bool FLAT, int RS>
__global__ __launch_bounds__(fused_max_threads(NBP, XF32, FLAT)) void fused_product_kernel(DevMatrix d, const void* __restrict__ X,
                                                                               int64_t ldx, int nb_valid,
                                                                               void* __restrict__ Y, int64_t ldy) {
  extern __shared__ uint32_t lds[];
  const uint32_t x_words = XF32 ? uint32_t(d.cols) * NBP : ((uint32_t(d.gpr) + 15) / 16 * 8) * 64 * NBP;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int waves = blockDim.x / kWave;
  const uint32_t sm_ring = kAreaAddr + x_words * 4 + uint32_t(wave) * ring_bytes(RS, d.slot_bytes);
  const uint32_t q_ring = sm_ring + RS * 1024;
  const int u_first = blockIdx.x * waves + wave;
  const int n_items = FLAT ? d.n_items : d.n_units;
  int fv = 0;
  // the decode tables, x (one bf16 row), then the first unit's ring steps:
  // tables and x have landed once only the ring's loads may be younger
  const int n_tab = issue_tables(d, wave, waves, lane);
  constexpr bool kEarlyX = NBP == 1 && !XF32;
  const bool early_x = kEarlyX && x_early_fits(d, blockDim.x);
  XEarly xe;
  if (kEarlyX && early_x) x_issue(d, static_cast<const uint16_t*>(X), xe);
  int issued = 0;
  if (FLAT && u_first < n_items) {
    const WalkItem it = walk_item(d, u_first);
    fv = flat_start<RS, NQ>(d, it.b0, it.b1, sm_ring, lane);
    issued = fv - it.b0 * d.T;
  }
  if (n_tab || early_x) wait_tables<RS, NQ>(issued);
  if (kEarlyX && early_x) x_store(d, xe, lds + kTableWords + kT1Words);
  else load_x<NBP, XF32>(d, X, ldx, nb_valid, lds + kTableWords + kT1Words);
  lds_barrier();
  ProductSink<NBP, XF32, YBF16, FLAT> sink{d, kAreaAddr, lane, nb_valid, Y, ldy};  // the rest set per unit
  if (FLAT && d.split) {
    // One block per wave (the grid covers every block, and a workgroup holds
    // whole units, so the wave before this one has the previous block).  A
    // row that crosses a block end is finished after one barrier: the first
    // part is parked in LDS by the wave that ends its block mid-row.
    const uint32_t parts = kAreaAddr + x_words * 4 + uint32_t(waves) * ring_bytes(RS, d.slot_bytes);
    const bool live = u_first < n_items;
    bool head = false;
    if (live) {
      const WalkItem it = walk_item(d, u_first);
      sink.unit_begin(it.row);
      run_flat<RS, NQ, 0, PAIR>(d, fv, it.b0, it.b1, it.row, it.c0, sm_ring, lane, sink);
      head = it.c0 != 0;
      if (item_ends_mid_row(d, it)) sink.park_tail(parts + uint32_t(wave) * 4u * NBP);
    }
    lds_barrier();
    if (live) {
      if (head) sink.add_head(parts + uint32_t(wave - 1) * 4u * NBP);
      sink.store_done();
    }
    return;
  }
  for (int u = u_first; u < n_items; u += gridDim.x * waves) {
    if (FLAT) {
      const WalkItem it = walk_item(d, u);
      sink.unit_begin(it.row);
      if (u != u_first) fv = flat_start<RS, NQ>(d, it.b0, it.b1, sm_ring, lane);
      run_flat<RS, NQ, 0, PAIR>(d, fv, it.b0, it.b1, it.row, it.c0, sm_ring, lane, sink);
    } else {
      sink.unit_begin(int64_t(u) * d.rows_per_unit);
      const int b0 = u * d.unit_blocks, b1 = std::min(d.n_blocks, b0 + d.unit_blocks);
      run_blocks<RS, NQ, 0, PAIR>(d, b0, b1, sm_ring, q_ring, lane, sink);
    }
    sink.unit_end();
  }
}

// ---------------------------------------------------------------------------
// Fused product on the matrix cores (batch >= 16): Y[b, n] = sum_k X[b, k] W[n, k].
//
// A workgroup of nw waves decodes nw work units (whole rows and whole
// blocks) in lockstep, one 16-group tile per step, each wave with the flat
// walk's ring of tile steps.  Every unit starts a row, so every wave's tile
// lies in one row and covers the same 1024 columns, so after a step the workgroup holds an
// nw x 1024 bf16 slice of W in LDS (one row per wave, in natural column
// order).  That slice is the A operand of v_mfma_f32_16x16x32_bf16 (rows of
// the slice = M, padded to 16 with zeros); 16 activation rows are the B
// operand, read straight from global memory (8 consecutive bf16 per lane, so
// the k order of A and B agree).  The 32 k-steps of a slice are spread over
// the waves; each wave accumulates its share for every batch tile, and the
// partial sums are added across waves in a fixed order when the rows end.
// Two slices alternate, so one barrier per step separates the decode of a
// step from the products of the previous one.
constexpr int kMfmaRS = 2;                 // tile steps per wave in flight
constexpr int kMfmaMaxRows = 64;           // batch rows per pass
constexpr uint32_t kWRowBytes = 2048 + 16;  // one row of a slice; the pad keeps the A reads conflict-free

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// How the workgroups walk the matrix (set on the host).
struct MfmaGeom {
  int nw;               // waves per workgroup = W rows per slice
  int tiles_per_block;  // G / 16
  int tiles_per_row;    // groups per row / 16
  int n_tasks;          // wave w of task k decodes work unit k * nw + w (whole rows, whole blocks)
  int split;            // 1: wave w decodes block k * nw + w instead, started late by the column
                        //    tile it begins at, so every wave's tile has the same columns
  int steps;            // split: steps per task (a multiple of tiles_per_row)
};

__device__ inline floatx4 mfma_bf16(const uint4& a, const uint4& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// One wave's tile into its row of the slice: pair k holds columns 64*(2k) + lane
// and 64*(2k+1) + lane.
struct SliceSink {
  uint32_t row_addr;
  int lane;
  __device__ void tile_raw(uint32_t) {}
  __device__ void tile_begin(int64_t, int) {}
  __device__ void pair(int k, uint32_t D) {
    st16(row_addr + ((2 * k) * kWave + lane) * 2, D);
    st16(row_addr + ((2 * k + 1) * kWave + lane) * 2, D >> 16);
  }
  __device__ void single(int jj, int64_t, int, uint32_t w) { st16(row_addr + (jj * kWave + lane) * 2, w); }
};

// s_waitcnt vmcnt(N) that also names the activation registers as read and
// written, so no use of them can be placed before it.
template <int N, int IPW, int TB>
__device__ __forceinline__ void wait_x(u32x4 (&xv)[IPW][TB]) {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
#pragma unroll
  for (int i = 0; i < IPW; ++i)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) asm volatile("" : "+v"(xv[i][tb]));
}

// IPW k-steps per wave and slice go with the wave count (IPW = ceil(32 / nw)):
// 16 waves (2), 11..15 (3), 8..10 (4); fewer waves leave more registers.
constexpr int mfma_max_threads(int ipw) { return ipw == 2 ? 1024 : ipw == 3 ? 960 : 640; }

template <int TB, int IPW, bool PAIR, bool YBF16, int NQ>
__global__ __launch_bounds__(mfma_max_threads(IPW)) void fused_mfma_kernel(DevMatrix d, MfmaGeom g, const uint16_t* __restrict__ X,
                                                                          int64_t ldx, int nb_valid, void* __restrict__ Y,
                                                                          int64_t ldy) {
  constexpr int RS = kMfmaRS;
  constexpr int XTRA = IPW * TB;  // activation loads per step
  extern __shared__ uint32_t lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int nw = g.nw;
  const uint32_t lane16 = 16u * uint32_t(lane);
  // two slices (steps alternate), then one ring per wave
  const uint32_t slice0 = kAreaAddr, slice_bytes = uint32_t(nw) * kWRowBytes;
  const uint32_t stride = 1024u + uint32_t(d.slot_bytes);
  const uint32_t ring = slice0 + 2 * slice_bytes + uint32_t(wave) * RS * stride;
  const uint32_t ring_last = ring + (RS - 1) * stride;
  const __amdgpu_buffer_rsrc_t rsm = flat_rsm(d), rq = flat_rq(d);
  const int tpt = g.tiles_per_block * (g.split ? 1 : d.unit_blocks);  // tiles per wave and task
  const int n_steps = g.split ? g.steps : tpt;
  const int n_items = g.split ? d.n_blocks : d.n_units;
  issue_tables(d, wave, nw, lane);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();

  // A operand row of this lane.  Rows >= nw and batch rows >= nb_valid read
  // real but unrelated data: they only feed output rows and columns that are
  // never stored (an MFMA output element depends on its own A row and B
  // column only).
  const int a_row = lane % 16, a_quad = lane / 16;
  const uint32_t a_off = uint32_t(a_row < nw ? a_row : 0) * kWRowBytes + a_quad * 16;
  // B operand: activation row b = 16 tb + lane % 16 (clamped for the address), 8 columns at 8 * (lane / 16)
  const uint16_t* xrow[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int b = 16 * tb + lane % 16;
    xrow[tb] = X + int64_t(b < nb_valid ? b : 0) * ldx + 8 * a_quad;
  }
  // 16 bytes per wave that take the loads of a step with no refill to issue
  const uint32_t dummy = slice0 + 2 * slice_bytes + uint32_t(nw) * RS * stride + uint32_t(wave) * 16;
  // split: the part of each slice row's first row that its block holds (a
  // row that began in the previous block), per batch row of the pass
  const uint32_t heads = dummy + uint32_t(nw - wave) * 16;

  for (int task = blockIdx.x; task < g.n_tasks; task += gridDim.x) {
    floatx4 acc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
    // this wave's tiles: the flat walk's tiles u0 .. v_end of its unit (the
    // last unit of the matrix may end early; the wave then idles in step)
    const int unit = task * nw + wave;
    const bool valid = unit < n_items;
    const int b0 = g.split ? unit : unit * d.unit_blocks;
    const int u0 = b0 * d.T;
    const int v_end = valid ? std::min(u0 + tpt, d.n_tiles) : u0;
    // split: a block that starts at column tile delta runs delta steps late
    const int delta = g.split ? u0 % g.tiles_per_row : 0;
    int fv = u0;
    uint32_t f_floor = 0, f_shifts = 0;
    const const_word* fstep = (const const_word*)(d.steps) + 2u * uint32_t(valid ? u0 : 0);
    if (valid) {
      // the first RS steps, then the descriptor of the next one (the table
      // has a spare entry after the last tile)
      uint32_t sl = ring;
#pragma unroll
      for (int i = 0; i < RS; ++i) {
        if (fv < v_end) {
          issue_flat<NQ>(rsm, rq, fv, fstep[0], fstep[1], sl, lane16);
          ++fv;
          fstep += 2;
          sl += stride;
        }
      }
      f_floor = fstep[0];
      f_shifts = fstep[1];
    }
    uint32_t qpos = valid ? scalar_word(d.block_off, b0) : 0u;
    uint32_t tile_rm = 0;
    LaneDec s{};
    uint32_t slot = ring;
    bool refill = false;  // the previous step consumed a slot that is not refilled yet
    uint32_t rf_slot = 0;
    for (int tau = 0; tau < n_steps; ++tau) {
      const int tt = tau - delta;  // this wave's tile in its unit or block
      const int t = tt % g.tiles_per_block;
      const uint32_t my_slice = slice0 + uint32_t(tau & 1) * slice_bytes;
      // This step's activations first, then the refill of the slot the
      // previous step consumed: so the wait for the activations never waits
      // for that refill.  Both are issued in asm and every wait is explicit.
      u32x4 xv[IPW][TB];
      {
        const int64_t col0 = int64_t(tau % g.tiles_per_row) * 1024;
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
          const int kk = (wave + i * nw) & 31;
#pragma unroll
          for (int tb = 0; tb < TB; ++tb)
            asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(xv[i][tb]) : "v"(xrow[tb] + col0 + 32 * kk) : "memory");
        }
      }
      // every step issues 1 + NQ loads after its activations: the refill, or
      // one-lane loads into this wave's dummy bytes
      if (refill && fv < v_end) {
        issue_flat<NQ>(rsm, rq, fv, f_floor, f_shifts, rf_slot, lane16);
        ++fv;
        fstep += 2;
        f_floor = fstep[0];
        f_shifts = fstep[1];
      } else {
        issue_dummy<1 + NQ>(rsm, dummy, lane16);
      }
      refill = false;
      const uint32_t my_row = my_slice + uint32_t(wave) * kWRowBytes;
      if (tt >= 0 && u0 + tt < v_end) {
        // loads younger than this step's: the RS - 1 steps issued after it
        // (1 + NQ each) and this step's activations; near the end, where
        // no refills follow, everything
        if (u0 + tt + RS <= v_end) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((RS - 1) * (1 + NQ) + XTRA) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const uint32_t q = slot + 1024u + (qpos & 15u);
        uint32_t rpos = 0;
        if (t == 0) {
          rpos = lane_dec_start(s, q, d.rb_words, lane);
          tile_rm = (ld32(q + 128 + 4 * uint32_t(lane >> 1)) >> (16 * (lane & 1))) & 0xFFFFu;
        }
        const uint4 cur = ld128(slot + lane16);
        SliceSink sink{my_row, lane};
        qpos += __builtin_amdgcn_readfirstlane(
            decode_tile<PAIR>(d, s, q, rpos, cur, __builtin_amdgcn_readlane(tile_rm, t), 16, true, 0, 0, lane, sink));
        refill = true;
        rf_slot = slot;
        slot = slot == ring_last ? ring : slot + stride;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) st32(my_row + (i * kWave + lane) * 4, 0u);
      }
      // the slice of this step is complete (and every wave is done with the
      // one before it, which the next step overwrites)
      lds_barrier();
      // the activations have landed once only this step's 1 + NQ loads may
      // be younger
      wait_x<1 + NQ, IPW, TB>(xv);
      // matrix cores: k-steps wave, wave + nw, ... of the 32 in this slice
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int kk = wave + i * nw;
        if (kk < 32) {
          const uint4 a = ld128(my_slice + a_off + kk * 64);
#pragma unroll
          for (int tb = 0; tb < TB; ++tb)
            acc[tb] = mfma_bf16(a, uint4{xv[i][tb].x, xv[i][tb].y, xv[i][tb].z, xv[i][tb].w}, acc[tb]);
        }
      }
      // the rows of this slice end here: add the partial sums of all waves
      // (through this step's slice, which the next step does not write)
      if ((tau + 1) % g.tiles_per_row == 0) {
#pragma unroll
        for (int r = 0; r < TB; r += 2) {
          lds_barrier();  // every wave is done reading the slice (or the previous partial sums)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            if (r + q < TB) {
              const floatx4 v = acc[r + q];
              st128(my_slice + ((wave * 2 + q) * kWave + lane) * 16,
                    uint4{f32_bits(v.x), f32_bits(v.y), f32_bits(v.z), f32_bits(v.w)});
            }
          }
          lds_barrier();
          const int nvals = (TB - r >= 2 ? 2 : 1) * 256;
          for (int v = threadIdx.x; v < nvals; v += blockDim.x) {
            const int q = v / 256, rem = v % 256, l = rem / 4, e = rem % 4;
            float sum = 0.f;
            for (int w = 0; w < nw; ++w) sum += bits_f32(ld32(my_slice + ((w * 2 + q) * kWave + l) * 16 + e * 4));
            const int m = 4 * (l / 16) + e;  // slice row
            const int b = 16 * (r + q) + l % 16;
            const int64_t mu = int64_t(task) * nw + m;  // the unit (split: block) of slice row m
            int64_t row;
            bool store = m < nw && mu < n_items && b < nb_valid;
            if (g.split && store) {
              // slice row m covers, since the last row end, the second part of
              // its first row (park it), a whole row, or the first part of its
              // last row (add the next block's parked part), else nothing
              const int tpr = g.tiles_per_row;
              const int mu0 = int(mu) * d.T, dm = mu0 % tpr, nm = std::min(d.T, d.n_tiles - mu0);
              const int last = dm + nm - 1;  // the step of its last tile
              const uint32_t hb = heads + uint32_t(m * kMfmaMaxRows + b) * 4;
              if (dm > 0 && tau == tpr - 1) {
                st32(hb, f32_bits(sum));
                store = false;
              } else if (tau - tpr >= last) {
                store = false;  // its last row was stored before
              } else {
                const int tm = std::min(tau - dm, nm - 1);
                row = (int64_t(mu0) + tm) / tpr;
                if (tau > last) sum += bits_f32(ld32(hb + kMfmaMaxRows * 4));
              }
            } else {
              row = mu * d.rows_per_unit + tau / g.tiles_per_row;
              store = store && row < d.rows;
            }
            if (store) {
              if (YBF16) static_cast<uint16_t*>(Y)[b * ldy + row] = f32_to_bf16(sum);
              else static_cast<float*>(Y)[b * ldy + row] = sum;
            }
          }
        }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
    // every load of this task has landed before the ring and slices are reused
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
  }
}

// ---------------------------------------------------------------------------
// Host-side launch helpers.
bool is_pair(const DevMatrix& d) { return d.L <= 6; }

size_t tables_bytes() { return size_t(kTableWords + kT1Words) * 4; }

size_t x_bytes(const DevMatrix& d, int nbp, bool xf32) {
  return xf32 ? size_t(d.cols) * nbp * 4 : size_t((d.gpr + 15) / 16 * 8) * 64 * nbp * 4;
}

// Compute units of the current device.
int cu_count() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Waves per workgroup (one workgroup per compute unit): enough for every
// unit to start in the first round, as far as the LDS budget and max_waves
// allow.
int pick_waves(int64_t units, size_t fixed, size_t per_wave, int max_waves = 16) {
  const int64_t cus = cu_count();
  int w = int(std::min<int64_t>(max_waves, std::max<int64_t>(1, (units + cus - 1) / cus)));
  while (w > 1 && fixed + per_wave * w > size_t(kLdsLimit)) --w;
  return w;
}

// Ring depth of the flat walk: kRS steps in flight when the waves that put
// every unit in the first round fit in LDS with it, else kRSLow (the decode,
// not the load latency, sets the pace; the units per compute unit matter more).
int flat_ring_depth(int64_t units, size_t fixed, int slot_bytes, size_t extra, int max_waves) {
  const int64_t cus = cu_count();
  const int need = int(std::min<int64_t>(max_waves, std::max<int64_t>(1, (units + cus - 1) / cus)));
  return pick_waves(units, fixed, ring_bytes(kRS, slot_bytes) + extra, max_waves) >= need ? kRS : kRSLow;
}

// knob: ring depth (0 = auto, 2 or 4) + 8 * waves per workgroup (0 = one
// workgroup per compute unit with enough waves for one round; else that many
// waves, so that smaller workgroups can share a compute unit).
template <int NBP, bool XF32, bool PAIR, bool YBF16>
int run_fused(const uw_matrix* m, const void* X, int64_t ldx, int nb, void* Y, int64_t ldy, void* stream, int knob) {
  const int rs_knob = knob & 7, wpw_knob = knob >> 3;
  DevMatrix d = m->dev;  // a copy: split rows may be turned off for this launch
  const size_t fixed = tables_bytes() + x_bytes(d, NBP, XF32);
  const int max_waves = fused_max_threads(NBP, XF32, d.flat) / kWave;
  // split rows: NBP partial sums per wave in LDS, and whole units per
  // workgroup; where a unit's waves do not fit, or a block spans more rows
  // than a wave's lanes can park (its first row waits for the previous
  // wave's part), one wave per unit
  if (d.split && (d.unit_blocks > max_waves || int64_t(d.G) > 62 * int64_t(d.gpr) ||
                  fixed + (ring_bytes(kRSLow, d.slot_bytes) + 4 * NBP) * d.unit_blocks > size_t(kLdsLimit))) {
    d.split = 0;
    d.n_items = d.n_units;
  }
  const int items = d.flat ? d.n_items : d.n_units;
  const size_t extra = d.split ? 4 * NBP : 0;
  int rs = d.flat ? flat_ring_depth(items, fixed, d.slot_bytes, extra, max_waves) : kRS;
  if (d.flat && wpw_knob) rs = kRSLow;  // several workgroups per compute unit: the short ring
  if (d.flat && rs_knob) rs = rs_knob == 4 ? kRS : kRSLow;
  if (d.split && fixed + (ring_bytes(rs, d.slot_bytes) + extra) * d.unit_blocks > size_t(kLdsLimit)) rs = kRSLow;
  const size_t per_wave = ring_bytes(rs, d.slot_bytes) + extra;
  if (fixed + per_wave * (d.split ? d.unit_blocks : 1) > size_t(kLdsLimit))
    return fail(UW_ERR_UNSUPPORTED, "fused product: x does not fit on chip");
  int waves = wpw_knob ? std::min(wpw_knob, max_waves) : pick_waves(items, fixed, per_wave, max_waves);
  if (d.split) waves = std::max(1, waves / d.unit_blocks) * d.unit_blocks;
  if (fixed + per_wave * waves > size_t(kLdsLimit))
    return fail(UW_ERR_UNSUPPORTED, "fused product: this many waves per workgroup do not fit in LDS");
  const size_t lds = fixed + per_wave * waves;
  const int grid = int(std::max<int64_t>(1, (items + waves - 1) / waves));
  auto kern = d.flat ? (rs == kRS ? (d.nq == 2 ? fused_product_kernel<NBP, XF32, PAIR, YBF16, 2, true, kRS>
                                               : fused_product_kernel<NBP, XF32, PAIR, YBF16, 4, true, kRS>)
                                  : (d.nq == 2 ? fused_product_kernel<NBP, XF32, PAIR, YBF16, 2, true, kRSLow>
                                               : fused_product_kernel<NBP, XF32, PAIR, YBF16, 4, true, kRSLow>))
                     : (d.nq == 2 ? fused_product_kernel<NBP, XF32, PAIR, YBF16, 2, false, kRS>
                                  : fused_product_kernel<NBP, XF32, PAIR, YBF16, 4, false, kRS>);
  allow_full_lds(kern);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(waves * kWave), lds, static_cast<hipStream_t>(stream), d, X, ldx, nb, Y,
                     ldy);
  return hip_check(hipGetLastError(), "fused_product_kernel launch");
}

template <int NBP, bool XF32, bool PAIR>
int run_fused_y(const uw_matrix* m, const void* X, int64_t ldx, int nb, void* Y, int64_t ldy, int yt, void* stream, int rs) {
  return yt == UW_BF16 ? run_fused<NBP, XF32, PAIR, true>(m, X, ldx, nb, Y, ldy, stream, rs)
                       : run_fused<NBP, XF32, PAIR, false>(m, X, ldx, nb, Y, ldy, stream, rs);
}

template <int NBP, bool XF32>
int run_fused_p(const uw_matrix* m, const void* X, int64_t ldx, int nb, void* Y, int64_t ldy, int yt, void* stream, int rs) {
  return is_pair(m->dev) ? run_fused_y<NBP, XF32, true>(m, X, ldx, nb, Y, ldy, yt, stream, rs)
                         : run_fused_y<NBP, XF32, false>(m, X, ldx, nb, Y, ldy, yt, stream, rs);
}

template <int NBP>
int run_fused_x(const uw_matrix* m, const void* X, int64_t ldx, int xt, int nb, void* Y, int64_t ldy, int yt, void* stream,
                int rs) {
  return xt == UW_F32 ? run_fused_p<NBP, true>(m, X, ldx, nb, Y, ldy, yt, stream, rs)
                      : run_fused_p<NBP, false>(m, X, ldx, nb, Y, ldy, yt, stream, rs);
}

// Largest batch chunk (1, 2, 4 or 8) whose X copy fits next to the tables and one stage buffer per wave.
int fused_chunk(const DevMatrix& d, int64_t batch, bool xf32) {
  int nbp = 8;
  while (nbp > 1 && (nbp / 2 >= batch ||
                     tables_bytes() + x_bytes(d, nbp, xf32) + ring_bytes(d.flat ? kRSLow : kRS, d.slot_bytes) * 4 >
                         size_t(kLdsLimit)))
    nbp /= 2;
  return nbp;
}

}  // namespace

// ---------------------------------------------------------------------------
int launch_decompress_items(const uw_matrix* m, uint16_t* out, int64_t ld_out, int item0, int item1, int64_t row_base,
                            void* stream) {
  const DevMatrix& d = m->dev;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t fixed = tables_bytes();
  const int items = item1 - item0;
  if (items <= 0) return UW_OK;
  const int rs = d.flat ? flat_ring_depth(items, fixed, d.slot_bytes, 0, 16) : kRS;
  const size_t per_wave = ring_bytes(rs, d.slot_bytes) + (d.flat ? 0 : kTransposeWords * 4);
  const int waves = pick_waves(items, fixed, per_wave);
  const size_t lds = fixed + per_wave * waves;
  const int grid = int(std::max<int64_t>(1, (int64_t(items) + waves - 1) / waves));
  auto pick = [&](auto pair) {
    constexpr bool P = decltype(pair)::value;
    return d.flat ? (rs == kRS ? (d.nq == 2 ? decompress_kernel<P, 2, true, kRS> : decompress_kernel<P, 4, true, kRS>)
                               : (d.nq == 2 ? decompress_kernel<P, 2, true, kRSLow>
                                            : decompress_kernel<P, 4, true, kRSLow>))
                  : (d.nq == 2 ? decompress_kernel<P, 2, false, kRS> : decompress_kernel<P, 4, false, kRS>);
  };
  auto kern = is_pair(d) ? pick(std::true_type{}) : pick(std::false_type{});
  allow_full_lds(kern);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(waves * kWave), lds, s, d, out, ld_out, PaletteOut{}, item0, item1, row_base);
  return hip_check(hipGetLastError(), "decompress_kernel launch");
}

int launch_decompress(const uw_matrix* m, uint16_t* out, int64_t ld_out, void* stream) {
  const DevMatrix& d = m->dev;
  if (m->h.plain()) return launch_copy_plain(d.plain, d.rows, d.cols, out, ld_out, stream);
  return launch_decompress_items(m, out, ld_out, 0, d.flat ? d.n_items : d.n_units, 0, stream);
}

// Exponent bytes of every weight, in the sign+mantissa section's tile order
// (flat walk only; the caller checks).
int launch_decode_exponents(const uw_matrix* m, uint8_t* out, void* stream) {
  const DevMatrix& d = m->dev;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t fixed = tables_bytes();
  const int items = d.n_items;
  const int rs = flat_ring_depth(items, fixed, d.slot_bytes, 0, 16);
  const size_t per_wave = ring_bytes(rs, d.slot_bytes);
  const int waves = pick_waves(items, fixed, per_wave);
  const size_t lds = fixed + per_wave * waves;
  const int grid = int(std::max<int64_t>(1, (int64_t(items) + waves - 1) / waves));
  auto pick = [&](auto pair) {
    constexpr bool P = decltype(pair)::value;
    return rs == kRS ? (d.nq == 2 ? decompress_kernel<P, 2, true, kRS, 1> : decompress_kernel<P, 4, true, kRS, 1>)
                     : (d.nq == 2 ? decompress_kernel<P, 2, true, kRSLow, 1>
                                  : decompress_kernel<P, 4, true, kRSLow, 1>);
  };
  auto kern = is_pair(d) ? pick(std::true_type{}) : pick(std::false_type{});
  allow_full_lds(kern);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(waves * kWave), lds, s, d, reinterpret_cast<uint16_t*>(out), int64_t(0),
                     PaletteOut{}, 0, items, int64_t(0));
  return hip_check(hipGetLastError(), "decompress_kernel (exponents) launch");
}

bool palette_transcodable(const uw_matrix* m, std::string* why) {
  const BlobHeader& h = m->h;
  const char* no = nullptr;
  if (h.plain()) no = "a plain-mode matrix has no palette";
  else if (!m->dev.flat) no = "the transcode needs the flat walk (G and cols/64 multiples of 16)";
  else if (h.cols % 1024) no = "the direct form needs cols to be a multiple of 1024";
  else if (h.K > 16 || (h.K < 16 && h.n_raw_groups > 0))
    no = "the palette is not the direct form's (K must be 16, or smaller with no raw group)";
  if (no && why) *why = no;
  return !no;
}

PaletteLayout transcode_layout(const uw_matrix* m) {
  PaletteLayout l = palette_layout(m->h.rows, m->h.cols, int64_t(m->h.n_raw_groups));
  l.n_pal = int(m->h.K);
  std::memset(l.palette, 0, sizeof(l.palette));
  std::memcpy(l.palette, m->h.palette, size_t(l.n_pal));
  return l;
}

int launch_palette_transcode(const uw_matrix* m, uint8_t* out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const PaletteLayout l = transcode_layout(m);
  DevMatrix d = m->dev;
  const int64_t n = d.rows * d.cols, n_tiles = n / 1024;
  // header and the gaps between sections
  PaletteFill f;
  std::memset(&f, 0, sizeof(f));
  uint8_t head[64] = {0};
  std::memcpy(head, "UWP1", 4);
  const uint32_t version = 1, n_pal = uint32_t(l.n_pal);
  const uint64_t rows = uint64_t(l.rows), cols = uint64_t(l.cols), n_raw = uint64_t(l.n_raw);
  std::memcpy(head + 4, &version, 4);
  std::memcpy(head + 8, &rows, 8);
  std::memcpy(head + 16, &cols, 8);
  std::memcpy(head + 24, &n_raw, 8);
  std::memcpy(head + 32, l.palette, 16);
  std::memcpy(head + 48, &n_pal, 4);
  std::memcpy(f.head, head, 64);
  const uint64_t lo[6] = {64, l.off_sm + uint64_t(n), l.off_idx + uint64_t(n / 2), l.off_flags + 2 * uint64_t(n_tiles),
                          l.off_prefix + 4 * uint64_t(n_tiles), l.off_raw + 64 * n_raw};
  const uint64_t hi[6] = {l.off_sm, l.off_idx, l.off_flags, l.off_prefix, l.off_raw, l.total};
  for (int i = 0; i < 6; ++i) {
    f.gap_lo[i] = lo[i];
    f.gap_hi[i] = hi[i];
  }
  hipLaunchKernelGGL(palette_fill_kernel, dim3(4), dim3(256), 0, s, out, f);
  if (int rc = hip_check(hipGetLastError(), "palette_fill_kernel launch")) return rc;
  hipLaunchKernelGGL(palette_prefix_kernel, dim3(1), dim3(1024), 0, s, d, reinterpret_cast<uint16_t*>(out + l.off_flags),
                     reinterpret_cast<uint32_t*>(out + l.off_prefix));
  if (int rc = hip_check(hipGetLastError(), "palette_prefix_kernel launch")) return rc;
  // the walk, with palette indices where the exponents would be
  d.tables = d.index_tables;
  const PaletteOut po{out + l.off_sm, out + l.off_idx, out + l.off_raw,
                      reinterpret_cast<const uint32_t*>(out + l.off_prefix)};
  const size_t fixed = tables_bytes();
  const int items = d.n_items;
  const int rs = flat_ring_depth(items, fixed, d.slot_bytes, 0, 16);
  const size_t per_wave = ring_bytes(rs, d.slot_bytes);
  const int waves = pick_waves(items, fixed, per_wave);
  const size_t lds = fixed + per_wave * waves;
  const int grid = int(std::max<int64_t>(1, (int64_t(items) + waves - 1) / waves));
  auto pick = [&](auto pair) {
    constexpr bool P = decltype(pair)::value;
    return rs == kRS ? (d.nq == 2 ? decompress_kernel<P, 2, true, kRS, 2> : decompress_kernel<P, 4, true, kRS, 2>)
                     : (d.nq == 2 ? decompress_kernel<P, 2, true, kRSLow, 2>
                                  : decompress_kernel<P, 4, true, kRSLow, 2>);
  };
  auto kern = is_pair(d) ? pick(std::true_type{}) : pick(std::false_type{});
  allow_full_lds(kern);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(waves * kWave), lds, s, d, static_cast<uint16_t*>(nullptr), int64_t(0), po, 0,
                     items, int64_t(0));
  return hip_check(hipGetLastError(), "decompress_kernel (palette transcode) launch");
}

int fused_rows_per_pass(const uw_matrix* m, int64_t batch, int xt) {
  return m->h.plain() ? int(std::min<int64_t>(batch, 8)) : fused_chunk(m->dev, batch, xt == UW_F32);
}

// Whether one pass of the vector-ALU product takes all `batch` rows with
// a full workgroup of 16 waves: x of every row next to the decode tables and
// 16 rings of the short depth.
bool fused_one_full_pass(const uw_matrix* m, int64_t batch, int xt) {
  if (m->h.plain()) return false;
  const DevMatrix& d = m->dev;
  const bool xf32 = xt == UW_F32;
  const int nbp = fused_chunk(d, batch, xf32);
  if (nbp < batch || fused_max_threads(nbp, xf32, d.flat) / kWave < 16) return false;
  const size_t per_wave = ring_bytes(d.flat ? kRSLow : kRS, d.slot_bytes) + 4 * size_t(nbp);
  return tables_bytes() + x_bytes(d, nbp, xf32) + 16 * per_wave <= size_t(kLdsLimit);
}

bool fused_supported(const uw_matrix* m, int xt, std::string* why) {
  if (m->h.plain()) return true;  // handled by the bf16 product
  const DevMatrix& d = m->dev;
  if (tables_bytes() + x_bytes(d, 1, xt == UW_F32) + ring_bytes(d.flat ? kRSLow : kRS, d.slot_bytes) >
      size_t(kLdsLimit)) {
    if (why) *why = "x of this width does not fit in LDS next to the decode tables";
    return false;
  }
  return true;
}

// Walk of the matrix-core kernel: waves per workgroup from the LDS budget,
// chosen so that the tasks fill whole rounds of 256 workgroups.
bool mfma_geometry(const DevMatrix& d, MfmaGeom* g, std::string* why, int nw_knob = 0) {
  if (d.gpr % 16) {
    if (why) *why = "the matrix-core path needs cols to be a multiple of 1024";
    return false;
  }
  if (!d.flat) {
    if (why) *why = "the matrix-core path needs the flat walk (G and cols/64 multiples of 16)";
    return false;
  }
  const size_t per_wave = 2 * kWRowBytes + ring_bytes(kMfmaRS, d.slot_bytes) + 16;
  const int nw_max = int(std::min<size_t>(16, (size_t(kLdsLimit) - tables_bytes()) / per_wave));
  if (nw_max < 8) {
    if (why) *why = "the blocks of this matrix are too large for the matrix-core path's LDS budget";
    return false;
  }
  g->tiles_per_block = d.G / 16;
  g->tiles_per_row = d.gpr / 16;
  // blocks that end mid-row: one block per wave when whole units fit in a
  // workgroup of at least 8 waves with the parked row parts
  const int nw_split = int(std::min<size_t>(16, (size_t(kLdsLimit) - tables_bytes()) / (per_wave + kMfmaMaxRows * 4)));
  g->split = d.split && nw_split / d.unit_blocks * d.unit_blocks >= 8;
  g->steps = 0;
  if (g->split) {
    int reach = 0;  // steps until the last block of a unit has its last tile
    for (int b = 0; b < d.unit_blocks; ++b) reach = std::max(reach, b * d.T % g->tiles_per_row + d.T);
    g->steps = (reach + g->tiles_per_row - 1) / g->tiles_per_row * g->tiles_per_row;
  }
  const int64_t units = g->split ? d.n_blocks : d.n_units;
  const int step_nw = g->split ? d.unit_blocks : 1;
  const int nw_top = g->split ? nw_split : nw_max;
  if (nw_knob && (nw_knob < 8 || nw_knob > nw_top || nw_knob % step_nw)) {
    if (why) *why = "this waves-per-workgroup knob does not fit the matrix's blocks";
    return false;
  }
  double best = -1.0;
  for (int nw = 8; nw <= nw_top; ++nw) {
    if (nw % step_nw || (nw_knob && nw != nw_knob)) continue;
    const int64_t tasks = (units + nw - 1) / nw;
    const int64_t rounds = (tasks + 255) / 256;
    const double eff = double(units) / double(rounds * 256 * nw);
    if (eff >= best - 1e-9) {
      best = eff;
      g->nw = nw;
      g->n_tasks = int(tasks);
    }
  }
  return true;
}

template <int TB, int IPW, bool PAIR>
int run_mfma(const uw_matrix* m, const MfmaGeom& g, const uint16_t* X, int64_t ldx, int nb, void* Y, int64_t ldy,
             int yt, hipStream_t s) {
  const DevMatrix& d = m->dev;
  const size_t lds = tables_bytes() + size_t(g.nw) * (2 * kWRowBytes + ring_bytes(kMfmaRS, d.slot_bytes) + 16 +
                                                     (g.split ? kMfmaMaxRows * 4 : 0));
  auto kern = yt == UW_BF16 ? (d.nq == 2 ? fused_mfma_kernel<TB, IPW, PAIR, true, 2> : fused_mfma_kernel<TB, IPW, PAIR, true, 4>)
                            : (d.nq == 2 ? fused_mfma_kernel<TB, IPW, PAIR, false, 2> : fused_mfma_kernel<TB, IPW, PAIR, false, 4>);
  allow_full_lds(kern);
  hipLaunchKernelGGL(kern, dim3(g.n_tasks), dim3(g.nw * kWave), lds, s, d, g, X, ldx, nb, Y, ldy);
  return hip_check(hipGetLastError(), "fused_mfma_kernel launch");
}

template <int TB, bool PAIR>
int run_mfma_ipw(const uw_matrix* m, const MfmaGeom& g, const uint16_t* X, int64_t ldx, int nb, void* Y, int64_t ldy,
                 int yt, hipStream_t s) {
  if (g.nw >= 16) return run_mfma<TB, 2, PAIR>(m, g, X, ldx, nb, Y, ldy, yt, s);
  if (g.nw >= 11) return run_mfma<TB, 3, PAIR>(m, g, X, ldx, nb, Y, ldy, yt, s);
  return run_mfma<TB, 4, PAIR>(m, g, X, ldx, nb, Y, ldy, yt, s);
}

// Up to 64 batch rows per pass (four 16-row tiles of activations and
// accumulators in registers).
template <bool PAIR>
int run_mfma_tb(const uw_matrix* m, const MfmaGeom& g, const uint16_t* X, int64_t ldx, int nb, void* Y, int64_t ldy,
                int yt, hipStream_t s) {
  if (nb <= 16) return run_mfma_ipw<1, PAIR>(m, g, X, ldx, nb, Y, ldy, yt, s);
  if (nb <= 32) return run_mfma_ipw<2, PAIR>(m, g, X, ldx, nb, Y, ldy, yt, s);
  return run_mfma_ipw<4, PAIR>(m, g, X, ldx, nb, Y, ldy, yt, s);
}

bool fused_mfma_supported(const uw_matrix* m, int xt, std::string* why, int nw) {
  if (m->h.plain()) {
    if (why) *why = "a plain-mode matrix has nothing to decode";
    return false;
  }
  if (xt != UW_BF16) {
    if (why) *why = "the matrix-core path takes bf16 activations";
    return false;
  }
  MfmaGeom g;
  return mfma_geometry(m->dev, &g, why, nw);
}

int launch_fused_mfma(const uw_matrix* m, const void* X, int64_t batch, int64_t ldx, void* Y, int64_t ldy, int yt,
                      void* stream, int nw) {
  const DevMatrix& d = m->dev;
  MfmaGeom g;
  std::string why;
  if (!mfma_geometry(d, &g, &why, nw)) return fail(UW_ERR_UNSUPPORTED, "fused matrix-core product: " + why);
  if (reinterpret_cast<uintptr_t>(X) % 16 || ldx % 8)
    return fail(UW_ERR_UNSUPPORTED, "fused matrix-core product: X must be 16-byte aligned with ldx a multiple of 8");
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t b0 = 0; b0 < batch; b0 += kMfmaMaxRows) {
    const int nb = int(std::min<int64_t>(kMfmaMaxRows, batch - b0));
    const uint16_t* Xb = static_cast<const uint16_t*>(X) + b0 * ldx;
    void* Yb = static_cast<char*>(Y) + b0 * ldy * elem_size(yt);
    const int rc = is_pair(d) ? run_mfma_tb<true>(m, g, Xb, ldx, nb, Yb, ldy, yt, s)
                              : run_mfma_tb<false>(m, g, Xb, ldx, nb, Yb, ldy, yt, s);
    if (rc) return rc;
  }
  return UW_OK;
}

int launch_fused(const uw_matrix* m, const void* X, int64_t batch, int64_t ldx, int xt, void* Y, int64_t ldy, int yt,
                 void* stream, int rs) {
  const DevMatrix& d = m->dev;
  if (m->h.plain()) return launch_bf16_gemm(d.plain, d.rows, d.cols, d.cols, X, batch, ldx, xt, Y, ldy, yt, stream);
  const int nbp = fused_chunk(d, batch, xt == UW_F32);
  for (int64_t b0 = 0; b0 < batch; b0 += nbp) {
    const int nb = int(std::min<int64_t>(nbp, batch - b0));
    const void* Xb = static_cast<const char*>(X) + b0 * ldx * elem_size(xt);
    void* Yb = static_cast<char*>(Y) + b0 * ldy * elem_size(yt);
    int rc;
    switch (nbp) {
      case 1: rc = run_fused_x<1>(m, Xb, ldx, xt, nb, Yb, ldy, yt, stream, rs); break;
      case 2: rc = run_fused_x<2>(m, Xb, ldx, xt, nb, Yb, ldy, yt, stream, rs); break;
      case 4: rc = run_fused_x<4>(m, Xb, ldx, xt, nb, Yb, ldy, yt, stream, rs); break;
      default: rc = run_fused_x<8>(m, Xb, ldx, xt, nb, Yb, ldy, yt, stream, rs); break;
    }
    if (rc) return rc;
  }
  return UW_OK;
}

}  // namespace uw
