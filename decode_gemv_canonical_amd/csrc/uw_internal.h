// Internal declarations of the uw library (host side and kernel launchers).
#pragma once

#include <cstddef>
#include <cstdint>
#include <map>
#include <mutex>
#include <string>

#include "../../include/uw.h"

namespace uw {

constexpr uint32_t kHeaderBytes = 256;
constexpr uint32_t kSectionAlign = 256;
constexpr uint32_t kFlagPlain = 1;
constexpr int kMaxK = 32;
constexpr int kMaxL = 12;
constexpr int kPairPeekBits = 12;  // two codes of <= 6 bits always fit in a 12-bit window

// Parsed header of a blob (layout in uw_blob.cpp).
struct BlobHeader {
  uint32_t version = 0, flags = 0;
  int64_t rows = 0, cols = 0;
  uint32_t K = 0, L = 0, G = 0, n_blocks = 0;
  uint64_t n_raw_groups = 0, total_bytes = 0;
  uint32_t crc32 = 0, max_segment_bytes = 0;
  uint8_t palette[32] = {0};
  uint8_t code_len[32] = {0};
  uint32_t R = 0;  // groups between two refill checks
  uint64_t off_block = 0, off_seg = 0, off_queue = 0, size_queue = 0;
  uint64_t off_sm = 0, size_sm = 0, off_plain = 0, size_plain = 0;
  bool plain() const { return flags & kFlagPlain; }
};

// Groups between refill checks for a maximum code length L: the codes decoded
// between two checks must fit in the 30 bits a lane always holds.
inline uint32_t check_groups(uint32_t L) { return L <= 7 ? 4u : 2u; }

// Serialise / parse the fixed 256-byte header (no validation in read).
void header_write(const BlobHeader& h, uint8_t* dst);
void header_read(const uint8_t* src, BlobHeader* h);

// CRC-32 (IEEE 802.3, reflected, as in zlib) of a byte range.
uint32_t crc32(const uint8_t* p, size_t n, uint32_t crc = 0);

// Full validation of a blob; on failure returns UW_ERR_FORMAT and sets the message.
int validate_blob(const uint8_t* blob, size_t n, BlobHeader* out);

// Canonical codes (RFC 1951 3.2.2) from lengths, ordered by exponent value;
// code[i] is MSB-first, rev[i] the bit-reversed pattern as stored in streams.
void canonical_codes(const BlobHeader& h, uint32_t code[32], uint32_t rev[32]);

// Per-thread error message.
void set_error(const std::string& msg);
const char* last_error_text();
int fail(int status, const std::string& msg);

// Direct-palette form (format UWP1, uw_palette.cpp): section offsets in bytes.
constexpr size_t kPaletteHeaderBytes = 64;
struct PaletteLayout {
  int64_t rows = 0, cols = 0, n_raw = 0;
  int n_pal = 0;
  uint8_t palette[16] = {0};
  size_t off_sm = 0, off_idx = 0, off_flags = 0, off_prefix = 0, off_raw = 0, total = 0;
};
PaletteLayout palette_layout(int64_t rows, int64_t cols, int64_t n_raw);
// Header fields, size and the raw flags/prefix counts; UW_ERR_FORMAT otherwise.
int palette_parse(const void* blob, size_t n, PaletteLayout* out);

// Kernel-side description of a compressed matrix, passed by value.
struct DevMatrix {
  const uint32_t* block_off;  // byte offset of each block's data in the queue
  const uint16_t* seg;        // per block, end of each tile's segment (words)
  const uint8_t* queue;
  const uint8_t* sm;
  const uint16_t* plain;
  int64_t rows, cols;
  int64_t n_groups;
  int32_t G, n_blocks, rb_words, gpr;  // gpr = groups per row = cols/64
  int32_t T;                           // tiles (segment entries) per block = ceil(G/16)
  int32_t R;                           // groups between refill checks
  int32_t L;
  int32_t slot_bytes;                  // LDS bytes of one segment slot (>= the largest segment, multiple of 16)
  int32_t seg_loads;                   // 1 KB direct loads that fill a slot
  int32_t nq;                          // 1 KB queue loads issued per tile step (2 or 4)
  int32_t flat;                        // 1: no tile crosses a row and `steps` is set
  int32_t n_tiles;                     // tiles of the matrix (flat walk)
  uint32_t q_extent;                   // flat walk: bytes readable from queue - 1 KB on
  int32_t rows_per_unit;               // rows covered by a work unit
  const uint32_t* steps;               // flat walk, per tile: {16-byte floor of its segment (queue offset),
                                       //  byte i: 64 - lanes of 1 KB queue load i (at least 1 lane)}
  int32_t unit_blocks;                 // blocks per work unit (a unit covers whole rows)
  int32_t n_units;
  int32_t split;                       // flat walk, G > gpr and not a multiple of it: the VALU product and the
                                       //  decompress give each wave one block, and a row that crosses a block
                                       //  end is summed from the two waves' parts
  int32_t n_items;                     // waves of work of those kernels: n_blocks when split, else n_units
  const uint32_t* tables;              // decode tables, built on the host (kDecodeTableBytes, the LDS image:
                                       //  pair table or 2^L single table, then the L <= 6 single table)
  const uint32_t* index_tables;        // the same image with palette indices in place of exponents
};


// Bytes of the decode-table image: 4096 words (pair table, or the 2^L
// single table for L > 6), then 64 words (the single table for L <= 6).
constexpr uint32_t kDecodeTableWords = 4096 + 64;
constexpr uint32_t kDecodeTableBytes = kDecodeTableWords * 4;

}  // namespace uw

// A direct-palette (UWP1) matrix bound to its device copy.
struct uw_palette {
  uw::PaletteLayout l;
  const uint8_t* d_blob = nullptr;
  int device = 0;
};

struct uw_matrix {
  uw::BlobHeader h;
  uw::DevMatrix dev;
  const uint8_t* d_blob = nullptr;    // the caller's device buffer: blob, then the derived tables
  int device = 0;
  const uw_palette* palette = nullptr;  // attached direct-palette copy (not owned)
  mutable std::mutex mu;
  std::map<int64_t, uw_plan> plans;
};

namespace uw {

// Launchers (uw_kernels.hip).  Shapes and pointers are checked by the caller.
int launch_decompress(const uw_matrix* m, uint16_t* out, int64_t ld_out, void* stream);
// Work items [item0, item1) of a coded matrix (units, or blocks when rows
// split across blocks; see DevMatrix::n_items), matrix row r written to
// out + (r - row_base) * ld_out.
int launch_decompress_items(const uw_matrix* m, uint16_t* out, int64_t ld_out, int item0, int item1, int64_t row_base,
                            void* stream);
// Exponent bytes (R*C, the sm section's tile order); flat walk, not plain.
int launch_decode_exponents(const uw_matrix* m, uint8_t* out, void* stream);
// rs: ring depth of the flat walk (0 = chosen from the LDS budget, else 2 or 4).
int launch_fused(const uw_matrix* m, const void* X, int64_t batch, int64_t ldx, int xt, void* Y,
                 int64_t ldy, int yt, void* stream, int rs = 0);
bool fused_supported(const uw_matrix* m, int xt, std::string* why);
// Batch rows the VALU fused product takes per pass (its x copy fits in LDS).
int fused_rows_per_pass(const uw_matrix* m, int64_t batch, int xt);
bool fused_one_full_pass(const uw_matrix* m, int64_t batch, int xt);
// nw: waves per workgroup (0 = chosen for the fewest idle waves, else 8..16).
int launch_fused_mfma(const uw_matrix* m, const void* X, int64_t batch, int64_t ldx, void* Y, int64_t ldy, int yt,
                      void* stream, int nw = 0);
bool fused_mfma_supported(const uw_matrix* m, int xt, std::string* why, int nw = 0);
// Direct-palette transcode (uw_palette_transcode): the UWP1 layout of a
// transcodable matrix, and the two kernels that write it.
bool palette_transcodable(const uw_matrix* m, std::string* why);
PaletteLayout transcode_layout(const uw_matrix* m);
int launch_palette_transcode(const uw_matrix* m, uint8_t* out, void* stream);
int launch_copy_plain(const uint16_t* src, int64_t rows, int64_t cols, uint16_t* out, int64_t ld_out, void* stream);
// bf16 product on the matrix cores (uw_gemm.hip): bf16 X, 16-byte aligned,
// ldx and ldw multiples of 8.  shape: 0 = heuristic, else an index below
// mfma_gemm_shape_count(); ks: waves per workgroup splitting k (0 = auto).
int launch_mfma_gemm(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw, const uint16_t* X, int64_t batch,
                     int64_t ldx, void* Y, int64_t ldy, int yt, int shape, int ks, void* stream);
int mfma_gemm_shape_count();
// Any bf16 product: the matrix cores for aligned bf16 X (bf16_gemm_on_mfma),
// else the vector ALU in passes of up to 8 rows.  A shape or ks applies only
// on the matrix cores.
int launch_bf16_gemm(const uint16_t* W, int64_t rows, int64_t cols, int64_t ldw, const void* X,
                     int64_t batch, int64_t ldx, int xt, void* Y, int64_t ldy, int yt, void* stream, int shape = 0,
                     int ks = 0);
bool bf16_gemm_supported(int64_t cols, int64_t batch, int xt, std::string* why);
bool bf16_gemm_on_mfma(const void* X, int64_t batch, int64_t cols, int64_t ldx, int xt);
// Cache eviction of the autotuner: read `bytes` (multiple of 16) at src.
int launch_read_probe(const void* src, size_t bytes, void* sink, void* stream);
// The allocation-free entry point's scratch (uw_static.hip): its size, the
// work units one band of rows holds (0 when one unit does not fit), and
// decompress + GEMM through it band by band.
size_t static_scratch_bytes();
int64_t static_band_units(const uw_matrix* m);
int static_decompress_gemm(const uw_matrix* m, const void* X, int64_t batch, int64_t ldx, int xt, void* Y, int64_t ldy,
                           int yt, int knob, void* stream);
size_t read_probe_sink_bytes();

}  // namespace uw
