/*
 * uw.h - lossless BF16 weight compression fused into the decode-time matmul,
 *        for AMD Instinct MI355X (gfx950).
 *
 * The method is the one of "Unweight: how we compressed an LLM 22% without
 * sacrificing quality": every bf16 weight keeps its sign and 7-bit mantissa as
 * a raw byte, its 8-bit exponent is Huffman coded (paragraph on Huffman coding
 * of the exponent byte), and a row of 64 weights holding an exponent outside
 * the top-K palette is stored raw (paragraph on rare exponents).  Decoding
 * happens on chip and feeds the multiply directly, so the reconstructed
 * weights never exist in device memory (paragraph on the reconstructive
 * matmul); a runtime chooses per matrix and batch size between the fused path
 * and decompress-then-multiply (paragraph on the four pipelines, paragraph on
 * the autotuner).
 *
 * Conventions for every entry point:
 *  - returns UW_OK (0) or a negative uw_status; nothing aborts, throws or
 *    prints across this boundary; uw_last_error() gives a message for the
 *    calling thread;
 *  - all arguments are checked on the host before anything is launched;
 *  - device entry points are asynchronous on the given stream (a hipStream_t
 *    passed as void*, NULL = the null stream) and do not synchronise, except
 *    uw_autotune, which is blocking; no entry point allocates device memory:
 *    every device buffer (blob, derived tables, inputs, outputs, workspaces)
 *    belongs to the caller;
 *  - "device pointer" means memory of the device that was current when the
 *    matrix handle was created; every device entry point runs on that device.
 *
 * Blob layout (the exchange format between uw_encode and the device kernels):
 * a 256-byte header followed by 256-byte aligned sections, all little-endian.
 *   header: "UWB2", u32 version=2, u32 header_bytes=256, u32 flags (bit 0 =
 *   plain), i64 rows, i64 cols, u32 K, u32 L, u32 G, u32 n_blocks,
 *   u64 n_raw_groups, u64 total_bytes, u32 crc32 (of bytes [256,total)),
 *   u32 largest segment bytes, u8 palette[32], u8 code_len[32], u32 R, u32 0,
 *   then u64 offsets: block, seg, queue (+size), sm (+size), plain (+size).
 *   A group is 64 consecutive weights of the row-major matrix; block b holds
 *   groups [b*G, min((b+1)*G, rows*cols/64)); tile t of a block is its groups
 *   [16t, 16t+16); lane l of a block owns weight 64*j + l of each group j.
 *   Lane l's codes (canonical, RFC 1951 3.2.2, length-limited Huffman codes
 *   over the palette, bit-reversed and packed LSB-first; raw groups skipped)
 *   form n_l 32-bit words.  A decoding lane holds three words (w0, w1, w2) =
 *   words (s-1, s, s+1) and qm, the bit offset in w0 of (next code - 2),
 *   starting at s = 0, qm = 30.  After every R-th group (R = 4 for L <= 7,
 *   else 2) each lane with qm >= 32 shifts by one word and, while it has
 *   words left, takes its next one; the words taken at one check are stored
 *   in lane order.
 *   block u32[n_blocks+1]: byte offset of each block's data in the queue;
 *   seg u16[n_blocks*ceil(G/16)]: end of tile t's segment, in words from the
 *   block start;
 *   queue: per block, tile 0's segment = u16 n_l[64], u32 raw bits
 *   [ceil(G/32)], word 0 of the lanes with n_l >= 1, word 1 of the lanes with
 *   n_l >= 2; every tile's segment then holds the 64 exponent bytes of each
 *   of its raw groups and the words taken at its checks;
 *   sm: per block ceil(G_b/16) tiles of 1024 bytes, byte (j>>4)*1024 +
 *   l*16 + (j&15) = sign+mantissa byte ((s<<7)|m) of weight 64*j + l;
 *   plain (plain mode): the bf16 bits, row-major.
 */
#ifndef UW_H
#define UW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define UW_VERSION 20000 /* 2.0.0 */

typedef enum {
  UW_OK = 0,
  UW_ERR_INVALID = -1,     /* a null/misaligned pointer, bad size or option      */
  UW_ERR_FORMAT = -2,      /* the blob is not a valid UWB2 blob                  */
  UW_ERR_NOSPACE = -3,     /* an output or workspace buffer is too small         */
  UW_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed         */
  UW_ERR_UNSUPPORTED = -5  /* valid request that this build cannot run           */
} uw_status;

typedef enum { UW_F32 = 0, UW_BF16 = 1 } uw_dtype;

/* Execution strategies for uw_gemm_fused ("four pipelines" paragraph: the
 * runtime picks one per matrix and batch size). */
typedef enum {
  UW_VARIANT_AUTO = 0,             /* the tuned plan for this batch, else a heuristic   */
  UW_VARIANT_FUSED = 1,            /* decode on chip, multiply on VALU, no bf16 in HBM  */
  UW_VARIANT_DECOMPRESS_GEMM = 2,  /* uw_decompress into the workspace, then bf16 GEMM  */
  UW_VARIANT_FUSED_MFMA = 3,       /* decode on chip, multiply on the matrix cores      */
  UW_VARIANT_PALETTE = 4,          /* the attached direct-palette copy (uw_matrix_attach_palette) */
  UW_VARIANT_COUNT = 5
} uw_variant;

#define UW_ENC_NO_PLAIN 1u /* never fall back to plain mode unless nothing can be coded */

typedef struct {
  int32_t K;      /* palette size, 1..32; 0 = 16 */
  int32_t L;      /* maximum code length, 1..12 and K <= 2^L; 0 = 6 */
  int32_t G;      /* groups of 64 weights per block: multiple of 16 in [16,1024]; 0 = automatic */
  uint32_t flags; /* UW_ENC_* */
} uw_encode_opts;

typedef struct {
  int64_t rows, cols;
  int32_t K, L, G, plain;
  int64_t n_blocks, n_raw_groups;
  uint64_t total_bytes;
  uint32_t max_segment_bytes;
  uint8_t palette[32];
  uint8_t code_len[32];
  double ratio;           /* total_bytes / (2*rows*cols) */
  double bits_per_weight; /* 8*total_bytes / (rows*cols) */
} uw_info;

/* A plan: how uw_gemm_fused runs one batch size under UW_VARIANT_AUTO.
 * knob is variant-specific (0 = the library's own choice):
 *   UW_VARIANT_FUSED            ring depth, tile steps in flight per wave (2 or 4; 0 = auto)
 *                               + 8 * waves per workgroup (1..16; 0 = one workgroup per
 *                               compute unit, sized to start every work unit at once);
 *   UW_VARIANT_FUSED_MFMA       waves per workgroup (decoded rows per slice): 8..16;
 *   UW_VARIANT_DECOMPRESS_GEMM  matrix-core GEMM shape (1..uw_bf16_gemm_shape_count()-1)
 *                               + 32 * waves splitting k (1, 2, 4 or 8; 0 = auto);
 *   UW_VARIANT_PALETTE          unused. */
typedef struct {
  int64_t batch;
  int32_t variant;                          /* the chosen uw_variant */
  int32_t knob;                             /* its knob */
  float time_us;                            /* its measured time per call */
  float candidate_us[UW_VARIANT_COUNT];     /* per variant, its best knob's time; < 0 = not measured */
  int32_t candidate_knob[UW_VARIANT_COUNT]; /* per variant, that best knob */
} uw_plan;

typedef struct uw_matrix uw_matrix;

/* Library version (UW_VERSION). */
int uw_version(void);

/* Static text for a status code. */
const char* uw_status_string(int status);

/* Message of the last failing call on this thread ("" if none). */
const char* uw_last_error(void);

/*
 * uw_encode (host) - compress a bf16 matrix into a blob.
 * Exponent histogram and top-K palette (exponent-redundancy paragraph),
 * raw 64-weight groups (rare-exponents paragraph), package-merge code
 * lengths <= L and canonical codes (Huffman paragraph), blocks of G groups
 * with one code stream per wavefront lane, stored tile by tile.
 *   w_bf16   host, rows*cols bf16 bit patterns, row-major, not modified.
 *   rows>=1, cols a positive multiple of 64.
 *   opts     may be NULL (defaults above).
 *   out      host buffer of *out_size bytes owned by the caller, or NULL to
 *            query: then *out_size receives the exact size and UW_OK returns.
 * The output is deterministic.  The coded form is replaced by plain mode when
 * it would not be smaller (unless UW_ENC_NO_PLAIN).
 * Errors: UW_ERR_INVALID (null pointers, bad shape or options),
 *         UW_ERR_NOSPACE (*out_size too small; *out_size set to the need).
 */
int uw_encode(const uint16_t* w_bf16, int64_t rows, int64_t cols, const uw_encode_opts* opts,
              void* out, size_t* out_size);

/*
 * uw_blob_info (host) - validate a blob (header, section bounds, CRC32, code
 * lengths forming a prefix code, segment tables consistent with the lane
 * word counts) and describe it.
 * Errors: UW_ERR_INVALID (null), UW_ERR_FORMAT (anything inconsistent).
 */
int uw_blob_info(const void* blob, size_t n, uw_info* info);

/*
 * uw_matrix_device_bytes (host) - bytes of the device buffer uw_matrix_create
 * takes for this blob: the blob itself (rounded up to 256 bytes), then tables
 * the kernels read that are derived from the blob and not part of it: the
 * decode tables (16640 bytes, from the code lengths; every kernel copies them
 * into LDS), the same tables with palette indices in place of exponents
 * (16640 bytes, for uw_palette_transcode) and, when G and cols/64 are
 * multiples of 16 (no 1024-weight tile crosses a row), a step table of
 * 8 bytes per tile (where each tile's segment starts and how many lanes load
 * it).  0 if the blob is invalid (uw_blob_info says why).
 */
size_t uw_matrix_device_bytes(const void* host_blob, size_t n);

/*
 * uw_matrix_create (host) - bind a handle to a blob on the current device.
 * host_blob/n is validated as by uw_blob_info.  d_buf (256-byte aligned,
 * d_bytes >= uw_matrix_device_bytes(host_blob, n)) must already hold the
 * same n bytes at its start; the call writes the derived tables after them
 * (a synchronous host-to-device copy) and allocates no device memory.  The
 * handle does not own d_buf: the caller keeps it alive and unchanged until
 * uw_matrix_destroy.  The handle keeps a copy of the header and a per-batch
 * plan cache (internally locked).
 * Errors: UW_ERR_INVALID (null, misaligned, d_bytes too small),
 *         UW_ERR_FORMAT, UW_ERR_HIP (no current device, copy failed).
 */
int uw_matrix_create(const void* host_blob, size_t n, void* d_buf, size_t d_bytes, uw_matrix** out);

/* Release a handle (NULL is ignored).  Work already queued keeps running. */
void uw_matrix_destroy(uw_matrix* m);

/*
 * uw_decompress (device) - the "full decode" pipeline's preprocessing:
 * writes the original bf16 bits, W[r][c] at d_out[r*ld_out + c].
 *   d_out   device, 16-byte aligned, rows*ld_out elements; ld_out >= cols and
 *           a multiple of 8.  Bit-exact (NaN payloads and subnormals kept).
 * Errors: UW_ERR_INVALID, UW_ERR_HIP.
 */
int uw_decompress(const uw_matrix* m, uint16_t* d_out, int64_t ld_out, void* stream);

/*
 * uw_gemv_fused (device) - y = W x with the decode fused into the product
 * (reconstructive-matmul paragraph; batch-1 decode reads every weight once).
 *   d_x  device, cols elements of xt (UW_F32 or UW_BF16), 4-byte aligned.
 *   d_y  device, rows elements of yt (UW_F32 or UW_BF16 rounded to nearest
 *        even), 4-byte aligned.  fp32 accumulation.
 * Errors: UW_ERR_INVALID, UW_ERR_UNSUPPORTED (cols too large for the on-chip
 *         copy of x: more than 32768 for bf16 x, 16384 for fp32 x), UW_ERR_HIP.
 */
int uw_gemv_fused(const uw_matrix* m, const void* d_x, int xt, void* d_y, int yt, void* stream);

/*
 * uw_gemm_fused (device) - Y = X W^T for a small batch.
 *   d_X  device, batch rows of cols elements of xt, row stride ldx >= cols.
 *   d_Y  device, batch rows of rows elements of yt, row stride ldy >= rows.
 *   variant  a uw_variant; UW_VARIANT_AUTO uses the plan stored for this
 *            batch (uw_autotune, uw_set_plan, uw_plan_load) when that plan's
 *            variant can run this call, else a heuristic (up to 64 with a
 *            direct-palette copy attached: the palette product; else batch
 *            1, batch 2 when one VALU pass takes both rows, and up to 8
 *            when one VALU pass takes them all with 16 waves per workgroup:
 *            fused on VALU; up to 32: fused on the matrix cores where supported;
 *            above: decompress + GEMM when d_ws is large enough, else the
 *            matrix cores).  An
 *            explicit variant runs with its default knob (uw_gemm_with_plan
 *            runs a given knob).
 *   d_ws/ws_bytes  caller-owned device workspace (uw_workspace_size bytes for
 *            the chosen variant; may be NULL/0 for the fused variants).
 *   UW_VARIANT_FUSED_MFMA needs bf16 X that is 16-byte aligned with ldx a
 *   multiple of 8, cols a multiple of 1024 and G a multiple of 16 (else
 *   UW_ERR_UNSUPPORTED); it runs 64 batch rows per pass.  UW_VARIANT_PALETTE
 *   needs an attached palette copy (uw_matrix_attach_palette) and bf16 X
 *   above batch 1.
 * batch == 0 is a no-op.  fp32 accumulation.
 * Errors: UW_ERR_INVALID, UW_ERR_NOSPACE (workspace), UW_ERR_UNSUPPORTED, UW_ERR_HIP.
 */
int uw_gemm_fused(const uw_matrix* m, const void* d_X, int64_t batch, int64_t ldx, int xt,
                  void* d_Y, int64_t ldy, int yt, int variant, void* d_ws, size_t ws_bytes,
                  void* stream);

/*
 * uw_gemm_fused_static (device) - uw_gemm_fused for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  It takes no workspace and allocates nothing: the
 * decompress + GEMM variant (chosen explicitly, by a stored plan, or by the
 * AUTO heuristic as if a workspace were given) runs band by band through a
 * 64 MiB scratch array in the library's device image, one band of whole rows
 * decompressed and multiplied at a time; the other variants need no scratch.
 * Each GPU the library runs on holds its own scratch until the process ends;
 * calls that overlap on one GPU (different streams) race on it, calls in one
 * stream are ordered.  Results equal uw_gemm_fused's with a workspace (the
 * same kernels; the bf16 product sees one band of rows at a time).
 * Errors: as uw_gemm_fused; UW_ERR_UNSUPPORTED when the decompress + GEMM
 *         variant is asked for and one work unit of the matrix (the rows of
 *         lcm(G, cols/64) groups) holds more than 64 MiB of bf16 weights.
 */
int uw_gemm_fused_static(const uw_matrix* m, const void* d_X, int64_t batch, int64_t ldx, int xt, void* d_Y,
                         int64_t ldy, int yt, int variant, void* stream);

/*
 * uw_gemm_with_plan (device) - as uw_gemm_fused, running exactly
 * plan->variant with plan->knob (plan->batch is not used): the form the
 * autotuner times and the tests check every knob through.
 * Errors: as uw_gemm_fused; UW_ERR_INVALID for an unknown variant or knob.
 */
int uw_gemm_with_plan(const uw_matrix* m, const uw_plan* plan, const void* d_X, int64_t batch, int64_t ldx, int xt,
                      void* d_Y, int64_t ldy, int yt, void* d_ws, size_t ws_bytes, void* stream);

/* Workspace bytes uw_gemm_fused needs for the given variant and batch
 * (UW_VARIANT_AUTO: the largest any candidate may need). */
size_t uw_workspace_size(const uw_matrix* m, int64_t batch, int variant);

/*
 * uw_autotune (device, BLOCKING) - autotuner paragraph (the runtime measures
 * real throughput on the target hardware instead of relying on heuristics):
 * time every applicable variant, each over its knobs, for this matrix and
 * batch on the given stream with HIP events (bf16 X and Y inside the
 * workspace), and store the fastest (variant, knob) in the handle's plan
 * cache; *out (may be NULL) gets a copy.  Every timed call runs cold: a read
 * of a 512 MiB region of the workspace (twice the 256 MiB last-level cache)
 * comes before it, so the blob is read from HBM as in a model's layer sweep.
 * Each candidate is warmed up 3 times and timed 15 times; its median counts.
 *   d_ws/ws_bytes  device workspace, 256-byte aligned, of at least
 *                  uw_workspace_size(m, batch, UW_VARIANT_AUTO) +
 *                  uw_autotune_scratch_size(m, batch) bytes.
 * Errors: UW_ERR_INVALID, UW_ERR_NOSPACE, UW_ERR_UNSUPPORTED (no candidate
 *         runs), UW_ERR_HIP.
 */
int uw_autotune(uw_matrix* m, int64_t batch, void* d_ws, size_t ws_bytes, void* stream, uw_plan* out);

/* Extra workspace uw_autotune uses: its own X and Y and the 512 MiB region
 * it reads to evict the blob from the caches. */
size_t uw_autotune_scratch_size(const uw_matrix* m, int64_t batch);

/* The stored plan for a batch; UW_ERR_INVALID if none. */
int uw_get_plan(const uw_matrix* m, int64_t batch, uw_plan* out);

/*
 * uw_set_plan (host) - store a plan for plan->batch (replacing any), so AUTO
 * follows a choice made elsewhere: a model-level tuning pass or a plan file
 * from an earlier run (autotuner paragraph: the tuner's result is a per-model
 * configuration file the runtime reads).  Only batch, variant and knob are
 * used by the dispatch; the times are kept for reporting.
 * Errors: UW_ERR_INVALID (null, batch < 1, variant not a concrete one, knob
 *         out of range).
 */
int uw_set_plan(uw_matrix* m, const uw_plan* plan);

/*
 * uw_plan_save (host) - the handle's plans as JSON text (NUL-terminated):
 *   {"format": "uw-plan-1", "rows": R, "cols": C, "blob_crc32": N,
 *    "plans": [{"batch": B, "variant": "fused" | "decompress_gemm" |
 *               "fused_mfma" | "palette", "knob": K, "time_us": T}, ...]}
 * in increasing batch.  out == NULL queries: *out_size gets the bytes
 * needed (with the NUL).  Errors: UW_ERR_INVALID, UW_ERR_NOSPACE.
 */
int uw_plan_save(const uw_matrix* m, char* out, size_t* out_size);

/*
 * uw_plan_load (host) - install the plans of JSON text written by
 * uw_plan_save (replacing plans of the same batch).  rows, cols and
 * blob_crc32 must match the handle's blob: a plan file belongs to one matrix.
 * Nothing is installed unless every entry is valid.
 * Errors: UW_ERR_INVALID (null), UW_ERR_FORMAT (not such JSON, or it belongs
 *         to another matrix).
 */
int uw_plan_load(uw_matrix* m, const char* json);

/*
 * uw_bf16_gemm (device) - Y = X W^T over an uncompressed bf16 matrix: the
 * multiply of the "full decode" pipeline and the uncompressed comparator.
 *   d_W  device, rows x cols bf16, row stride ldw >= cols (multiple of 8),
 *        16-byte aligned.  Other arguments as for uw_gemm_fused.
 * bf16 X that is 16-byte aligned with ldx a multiple of 8 runs on the
 * matrix cores (v_mfma_f32_16x16x32_bf16; operands straight from global
 * memory, or staged through LDS), except a single row of X with cols <= 8192,
 * and fp32 or unaligned X, which a GEMV-style kernel on the vector ALU takes
 * in passes of up to 8 rows.
 * 16, 32, 64 or 128 weight rows and 16 to 128 batch rows per workgroup; the
 * staged shapes 14..18 also need cols a multiple of 128 and each operand
 * under 2 GiB.  Shapes 17 and 18 (fp32 Y) run two workgroups per tile, each
 * over half of K, adding into Y after zeroing it; two addends keep the
 * result independent of their order, so runs are reproducible.
 * Errors: UW_ERR_INVALID, UW_ERR_UNSUPPORTED, UW_ERR_HIP.
 */
int uw_bf16_gemm(const uint16_t* d_W, int64_t rows, int64_t cols, int64_t ldw, const void* d_X,
                 int64_t batch, int64_t ldx, int xt, void* d_Y, int64_t ldy, int yt, void* stream);

/*
 * uw_bf16_gemm_shaped (device) - uw_bf16_gemm on the matrix cores with a
 * given shape: shape in [1, uw_bf16_gemm_shape_count()) picks the weight rows
 * (16 to 128) and batch rows (16 to 128) a workgroup holds and whether the
 * operands are staged in LDS, ks (1, 2, 4, 8; 0 = auto) the waves that split
 * k (for the shapes that read straight from global memory).  Needs bf16 X, 16-byte aligned,
 * ldx a multiple of 8, and batch >= 1.
 * Errors: UW_ERR_INVALID, UW_ERR_HIP.
 */
int uw_bf16_gemm_shaped(const uint16_t* d_W, int64_t rows, int64_t cols, int64_t ldw, const void* d_X,
                        int64_t batch, int64_t ldx, void* d_Y, int64_t ldy, int yt, int shape, int ks, void* stream);
/* Number of shape ids of uw_bf16_gemm_shaped (shape 0 is the automatic one). */
int uw_bf16_gemm_shape_count(void);

/*
 * uw_read_probe (device) - streaming read of `bytes` bytes (multiple of 16,
 * 16-byte aligned) that writes one checksum word per 16 threads into d_sink
 * (uw_read_probe_sink_size bytes): the fastest sustainable read rate the
 * fused kernels are measured against (the Apple-silicon page's section on
 * the limits of further optimisation measures kernels against the fastest
 * weight-read rate for their access pattern).
 * Errors: UW_ERR_INVALID, UW_ERR_HIP.
 */
int uw_read_probe(const void* d_src, size_t bytes, void* d_sink, void* stream);
size_t uw_read_probe_sink_size(void);

/*
 * uw_exponent_gemm (device) - the exponent-only pipeline (section on the four
 * execution pipelines: decode only the exponent bytes, half the preprocessing
 * traffic, then a reconstructive matmul): the exponents of every weight are
 * decoded into the workspace (1 byte per weight, in the order of the blob's
 * sign+mantissa section), X is permuted into that order, and
 * v_mfma_f32_16x16x32_bf16 multiplies bf16 rebuilt from the two byte planes,
 * 64 batch rows per pass.  Needs a coded blob whose tiles never cross a row
 * (G and cols/64 multiples of 16).
 *   d_X   device bf16 [batch, ldx], ldx >= cols.   d_Y as for uw_gemm_fused.
 *   d_ws  device, 256-byte aligned, >= uw_exponent_ws_size(m, batch) bytes.
 * Errors: UW_ERR_INVALID, UW_ERR_UNSUPPORTED (plain blob, tiles crossing rows,
 *         X not bf16), UW_ERR_HIP.
 */
int uw_exponent_gemm(const uw_matrix* m, const void* d_X, int64_t batch, int64_t ldx, int xt, void* d_Y,
                     int64_t ldy, int yt, void* d_ws, size_t ws_bytes, void* stream);
/* Workspace bytes of uw_exponent_gemm: R*C (256-rounded) + min(batch, 64)*C*2; 0 for a null handle. */
size_t uw_exponent_ws_size(const uw_matrix* m, int64_t batch);

/*
 * Direct-palette pipeline (section on the four execution pipelines: the
 * weights become 4-bit palette indices at load time and the matmul rebuilds
 * bf16 from them with no preprocessing pass).  Form UWP1: per weight one
 * sign+mantissa byte and a 4-bit index into the 16 most frequent exponents;
 * 64-weight groups holding any other exponent keep their 64 exponent bytes
 * (paragraph on rare exponents).  About 12 bits per weight plus raw groups.
 */
typedef struct uw_palette uw_palette;

/*
 * uw_palette_encode (host) - the UWP1 form of a bf16 matrix.
 *   w_bf16   host, rows*cols bf16 bit patterns, row-major, not modified.
 *   rows>=1, cols a positive multiple of 1024 (no 1024-weight tile crosses a
 *   row).  out/out_size as for uw_encode (NULL out queries the size).
 * Deterministic; the palette and the raw groups follow uw_encode's rule
 * (count descending, exponent ascending; K = 16).
 * Errors: UW_ERR_INVALID, UW_ERR_NOSPACE.
 */
int uw_palette_encode(const uint16_t* w_bf16, int64_t rows, int64_t cols, void* out, size_t* out_size);

/*
 * uw_palette_info (host) - validate a UWP1 blob (header, size, raw flags
 * against the per-tile prefix counts) and report its shape and raw groups.
 * Errors: UW_ERR_INVALID (null), UW_ERR_FORMAT.
 */
int uw_palette_info(const void* blob, size_t n, int64_t* rows, int64_t* cols, int64_t* n_raw);

/*
 * uw_palette_create (host) - bind a handle to a UWP1 blob already copied to
 * device memory (n bytes on the current device, 256-byte aligned; the caller
 * keeps it alive and unchanged until uw_palette_destroy).  host_blob/n is
 * validated as by uw_palette_info.  Allocates no device memory.
 * Errors: UW_ERR_INVALID, UW_ERR_FORMAT, UW_ERR_HIP (no current device).
 */
int uw_palette_create(const void* host_blob, size_t n, const void* d_blob, uw_palette** out);

/* Release a palette handle (NULL is ignored). */
void uw_palette_destroy(uw_palette* m);

/*
 * uw_palette_gemv (device) - y = W x over the UWP1 form, decode fused.
 *   d_x  device, cols elements of xt (UW_F32 or UW_BF16), 16-byte aligned.
 *   d_y  device, rows elements of yt (UW_F32, or UW_BF16 rounded to nearest
 *        even).  fp32 accumulation.
 * Errors: UW_ERR_INVALID (null, misaligned, wrong device), UW_ERR_HIP.
 */
int uw_palette_gemv(const uw_palette* m, const void* d_x, int xt, void* d_y, int yt, void* stream);

/*
 * uw_palette_gemm (device) - Y = X W^T over the UWP1 form on the matrix
 * cores (v_mfma_f32_16x16x32_bf16), 64 batch rows per pass; the indices are
 * rebuilt into bf16 in registers, no preprocessing pass (the pages expect this
 * pipeline to pay off at larger batches).
 *   d_X  device bf16 [batch, ldx], 16-byte aligned, ldx >= cols, multiple of 8.
 *   d_Y  device [batch, ldy] of yt (UW_F32 or UW_BF16), ldy >= rows.
 * fp32 accumulation.
 * Errors: UW_ERR_INVALID, UW_ERR_UNSUPPORTED (X not bf16), UW_ERR_HIP.
 */
int uw_palette_gemm(const uw_palette* m, const void* d_X, int64_t batch, int64_t ldx, int xt, void* d_Y,
                    int64_t ldy, int yt, void* stream);

/*
 * uw_palette_decompress (device) - the original bf16 bits of a UWP1 matrix,
 * W[r][c] at d_out[r*ld_out + c]; d_out 16-byte aligned, ld_out >= cols and a
 * multiple of 8.  Bit-exact.
 * Errors: UW_ERR_INVALID, UW_ERR_HIP.
 */
int uw_palette_decompress(const uw_palette* m, uint16_t* d_out, int64_t ld_out, void* stream);

/*
 * uw_palette_transcode_size (host) - bytes of the UWP1 form uw_palette_transcode
 * writes for a Huffman-form matrix: the same as uw_palette_encode of the
 * matrix's weights.  0 when the matrix cannot be transcoded: plain mode,
 * cols not a multiple of 1024, G not a multiple of 16, or a palette that is
 * not the direct form's (K must be 16, or smaller with no raw group).
 */
size_t uw_palette_transcode_size(const uw_matrix* m);

/*
 * uw_palette_transcode (device) - the page's "transcoded at model load"
 * step: decode the Huffman form on the device and write its UWP1 form, byte
 * for byte what uw_palette_encode produces from the original weights
 * (section on the four execution pipelines: one Huffman bundle serves both
 * distribution and inference).  Two kernels: one writes the raw flags and
 * per-tile raw counts from the blob's raw bits, the other walks the tiles
 * with a decode table that yields palette indices and writes sign+mantissa
 * bytes, index nibbles and the raw groups' exponent bytes.
 *   d_out  device, 256-byte aligned, out_bytes >= uw_palette_transcode_size(m).
 * Errors: UW_ERR_INVALID, UW_ERR_NOSPACE, UW_ERR_UNSUPPORTED, UW_ERR_HIP.
 */
int uw_palette_transcode(const uw_matrix* m, void* d_out, size_t out_bytes, void* stream);

/*
 * uw_palette_create_transcoded (host) - a palette handle over d_blob, which
 * holds (or, once the stream has run, will hold) uw_palette_transcode's
 * output for m; the layout is taken from m, so no host copy is needed.
 * Allocates no device memory.  Errors: UW_ERR_INVALID, UW_ERR_UNSUPPORTED, UW_ERR_HIP.
 */
int uw_palette_create_transcoded(const uw_matrix* m, const void* d_blob, uw_palette** out);

/*
 * uw_matrix_attach_palette (host) - make a direct-palette copy of the same
 * weights (same rows and cols; uw_palette_transcode of m, or
 * uw_palette_encode of the original weights) a candidate of m: then
 * UW_VARIANT_PALETTE runs it, uw_autotune times it, and AUTO may pick it
 * (the four-pipelines paragraph: format and pipeline are chosen per matrix
 * and batch).  p == NULL detaches.  The handle does not own p.
 * Errors: UW_ERR_INVALID (null m, shapes differ).
 */
int uw_matrix_attach_palette(uw_matrix* m, const uw_palette* p);

/*
 * Decode-ahead scheduling (the paragraph on "hard" and "easy" layers, the
 * figure caption on decoding in separate streams during initial load,
 * attention and easy MLPs, and the paragraph on splitting the compute units
 * between decode and matmul): a "hard" matrix is decompressed on a side
 * stream into one of a ring of slots while the caller's stream runs other
 * work, and its product is then a plain bf16 product from the slot.
 */
typedef struct uw_sched uw_sched;

/*
 * uw_sched_create (host) - a scheduler with n_slots (1..64) decode slots of
 * slot_bytes each at d_slots (caller-owned device memory, 256-byte aligned,
 * slot_bytes a multiple of 256 and at least rows*cols*2 of any matrix it will
 * hold) and a side stream on the current device.  decode_cus = 0 lets the
 * side stream use every compute unit; k > 0 limits it to k of them, the same
 * share on every XCD (hipExtStreamCreateWithCUMask).  Creates the stream and
 * events; allocates no device memory.
 * Errors: UW_ERR_INVALID, UW_ERR_HIP.
 */
int uw_sched_create(void* d_slots, size_t slot_bytes, int n_slots, int decode_cus, uw_sched** out);

/* Waits for the side stream and releases the scheduler (NULL is ignored). */
void uw_sched_destroy(uw_sched* s);

/* Compute units the side stream may use (0 = all); -1 for NULL. */
int uw_sched_decode_cus(const uw_sched* s);

/*
 * uw_sched_prefetch (host, enqueues device work) - decompress m into a free
 * slot on the side stream, starting once `stream` (the caller's) has reached
 * this point; *slot receives the slot.  Work the caller enqueues on `stream`
 * after this call overlaps the decode.
 * A scheduler with a compute-unit mask (decode_cus > 0) works on streams
 * that are not being captured into a graph; under capture use decode_cus = 0.
 * A scheduler is used from one host thread at a time.
 * Errors: UW_ERR_INVALID, UW_ERR_NOSPACE (no free slot: every slot holds a
 *         matrix whose uw_sched_gemm has not been called; or the matrix does
 *         not fit a slot), UW_ERR_UNSUPPORTED (a masked scheduler under graph
 *         capture), UW_ERR_HIP.
 */
int uw_sched_prefetch(uw_sched* s, const uw_matrix* m, void* stream, int* slot);

/*
 * uw_sched_gemm (host, enqueues device work) - Y = X W^T on `stream` from
 * the slot filled by uw_sched_prefetch, after its decode (uw_bf16_gemm's
 * kernels; operands as for uw_gemm_fused).  Frees the slot for the next
 * prefetch, which will wait for this product through the caller's stream.
 * Errors: UW_ERR_INVALID (no prefetched matrix in the slot, bad operands),
 *         UW_ERR_UNSUPPORTED, UW_ERR_HIP.
 */
int uw_sched_gemm(uw_sched* s, int slot, const void* d_X, int64_t batch, int64_t ldx, int xt, void* d_Y, int64_t ldy,
                  int yt, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* UW_H */
