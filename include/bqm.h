/*
 * bqm.h -- weight-only low-bit quantized matmul on MI355X (gfx950).
 *
 * C ABI of libbqm.so.  Plain pointers and sizes only.
 *
 * Conventions for every entry point:
 *   - Pointers marked [device] are HIP device memory owned by the caller (for
 *     example a torch tensor's data pointer); pointers marked [host] are host
 *     memory owned by the caller.  The library never allocates or frees
 *     memory and keeps no state beyond cached per-device properties.
 *   - Device work is enqueued asynchronously on `stream` (a hipStream_t;
 *     NULL means the default stream).  Results are valid once the stream has
 *     been synchronized.  Calls that share buffers must be ordered by the
 *     caller (same stream or events).
 *   - Every argument is validated on the host before anything is launched.
 *     The return value is BQM_OK (0) or a negative BQM_E* code; after a
 *     validation error nothing has been enqueued.  BQM_EDEVICE reports a HIP
 *     error seen while launching (hipGetLastError); a call made of several
 *     launches may then have enqueued the ones before the failing launch.
 *   - Matrices are row-major.  Weight matrices are [out, in] = [rows, cols]:
 *     every output row is contiguous along the reduction axis and quant
 *     groups run along that axis ("14MB holds 45M parameters: dissecting
 *     Needle's .cact file and W4A8 quantization", section 3).
 *   - Only gfx950 devices are accepted (BQM_ENOTSUP otherwise).
 */
#ifndef BQM_H
#define BQM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *bqm_stream_t; /* a hipStream_t */

enum {
  BQM_OK = 0,
  BQM_EINVAL = -1,  /* null pointer, bad shape, unknown bits code, bad codebook */
  BQM_EALIGN = -2,  /* a device pointer is not 16-byte aligned                 */
  BQM_ENOTSUP = -3, /* valid request the device path does not provide
                       (group != 128, a batch past the entry's limit,
                       non-gfx950 device)                                      */
  BQM_EDEVICE = -4, /* HIP reported an error while launching                   */
  BQM_ERANGE = -5   /* reported through an encoder's status word, see cq_pack  */
};

/* CQ bits codes, as the pages number them: 2/3/4 index the fitted codebooks
 * cb2/cb3/cb4 (4, 8, 16 levels); 5 is ternary {-c, 0, +c} and 1 binary
 * {-sqrt(2/pi), +sqrt(2/pi)}, both analytic and built into the library
 * ("Parse-free loading: mmap tensors and Needle's cold start", passage on
 * the CQ format).  6 is an addition: the ternary set with its indices packed
 * as base-3 digits, five to a byte (the llama.cpp TV-box / iPad page weighs
 * base-3 digits against 2-bit fields for ternary weights in its speed-up
 * table, section 18). */
enum { BQM_CQ_BINARY = 1, BQM_CQ_B2 = 2, BQM_CQ_B3 = 3, BQM_CQ_B4 = 4, BQM_CQ_TERNARY = 5,
       BQM_CQ_TERNARY_B3 = 6 };

/* Status-word bits written by the encoders (OR-ed, never cleared). */
enum { BQM_STATUS_NONFINITE = 1, BQM_STATUS_NORM_OVERFLOW = 2 };

/* Byte layout of one packed CQ matrix ("blob"):
 *   [0, idx_bytes)            index rows back to back, idx_row_bytes each; a
 *                             row is an LSB-first stream of index_bits-wide
 *                             fields (index j at bits [b*j, b*j+b)), so 8
 *                             indices fill exactly index_bits bytes and, for
 *                             4 bits, the low nibble of a byte is the even
 *                             column (Needle article, section 1);
 *   [norms_offset, +2*norms_count)  fp16 group L2 norms [rows][cols/group];
 *   total_bytes               rounded up to 64 (the .cact 64-byte blob
 *                             alignment, Needle article, section 2).
 * Ternary uses 2-bit fields holding 0/1/2 (field value 3 decodes to 0).
 * Base-3 ternary (bits 6, index_bits 0): each group is ceil(group/5) bytes
 * (26 for 128), byte j = sum_i idx[5j+i] * 3^i over the group's positions
 * 5j .. 5j+4 (the first index least significant), positions past the group
 * holding digit 1 (the zero level); a row is its groups back to back. */
typedef struct {
  int32_t rows, cols, group, bits, index_bits, levels;
  int64_t idx_row_bytes, idx_bytes, norms_offset, norms_count, total_bytes;
} bqm_cq_layout;

/* Fill `layout` [host] for a rows x cols matrix, quant group `group` (a power
 * of two >= 2 dividing cols) and bits code `bits`.  Host only, no device
 * access.  BQM_EINVAL on a bad shape, group or code. */
int cq_pack_info(int rows, int cols, int group, int bits, bqm_cq_layout *layout);

/* Built-in levels of the analytic sets: bits 1 -> 2 values, bits 5 and 6 ->
 * 3 values, ascending fp32, written to `levels` [host].  BQM_EINVAL for
 * other codes.  Host only. */
int cq_analytic_levels(int bits, float *levels);

/* Per-token symmetric int8 activations in the rotated domain
 * (Needle article, section 1: W4A8; the rotation H is orthogonal, so
 * dot(w_g, x_g) = norm_g/G * dot(cb[idx_g], H_u x_g) and only x is rotated).
 * x [device] fp32 [m, k]; q [device] int8 [m, k]; scale [device] fp32 [m].
 * Per row: u = H_u x_g for each group of `group` columns (unnormalized
 * Sylvester-order butterfly, stages of half-width 1, 2, ..., group/2),
 * s = max|u| / 127 (1 for an all-zero row), q = clip(rint(u / s), -127, 127)
 * with correctly rounded fp32 division and half-even rounding.
 * Requires k % group == 0, group == 128, k <= 65536, x and q 16-byte aligned.
 * group == 1 is the same quantizer without the rotation (a Walsh-Hadamard
 * transform of length 1 is the identity), for the Q4_0 products, whose
 * weights carry none: s = max|x| / 127 over the row, q = clip(rint(x / s),
 * -127, 127); any k <= 65536.  Other groups: BQM_ENOTSUP. */
int act_fwht_quant_a8(const float *x, int m, int k, int group, int8_t *q, float *scale,
                      bqm_stream_t stream);

/* Decode GEMV on packed CQ weights (Needle article, section 3: decode is a
 * GEMV streaming [out, in] rows; dequantization happens inside the kernel).
 *   y[b, n] = scale[b] / G * sum_g norm[n, g] * sum_{i in g} cb[idx[n, i]] * q[b, i]
 * blob [device] packed as `layout` [host] describes (16-byte aligned);
 * codebook [host] `layout->levels` fp32 values for bits 2/3/4, index order
 * (each finite and bfloat16-representable, hence exact in fp16 too;
 * BQM_EINVAL otherwise), NULL for bits 1, 5 and 6; q [device] int8 [batch, cols] from act_fwht_quant_a8;
 * scale [device] fp32 [batch]; y [device] fp32 [batch, rows].
 * 1 <= batch <= 32 and cols <= 36864 (one token's codes as fp16 fit in LDS
 * beside the level table; BQM_ENOTSUP past either).  group must be 128.  For batch >= 2
 * (>= 3 when cols > 4096) and cols <= 16384 the product runs on the matrix
 * cores in one pass over the weights for all tokens: exact fp16 levels x
 * exact fp16 codes, fp32 accumulation per group, fp32 norm per group, the
 * groups summed in a fixed order (past 16 tokens as two 16-token halves on
 * the same weight fragments).  With more than 8 tokens, at most 16 rows
 * a CU and at least 64 groups a row, the call is two launches: y is zeroed,
 * then two halves of K are summed as above and each half's scaled result is
 * added into y atomically (two addends onto zero: the same bits in either
 * order, so results stay deterministic).  Batch 1 and 2 otherwise run on the VALU
 * GEMV; for cols > 16384 batch > 4 runs on the cq_gemm kernel with that
 * kernel's arithmetic and bound (level x norm x 2^e_n rounded to fp16 once
 * per weight, see cq_gemm) and smaller batches on the VALU GEMV, 4 tokens per
 * launch.  The VALU and matrix-core routes form every product level x code
 * exactly, so each y[b, n] is within a few units of fp32 roundoff of
 * scale[b] / G * sum_g norm[n, g] * sum_i |cb[idx[n, i]]| * |q[b, i]|.
 * Base-3 ternary (bits 6): 1 <= batch <= 16 with cols <= 16384 (BQM_ENOTSUP
 * otherwise); one token on the VALU kernel (int8 dot products), 2..16 tokens
 * in one pass over the weights on the int8 matrix cores.  Either way the
 * group sums of (digit - 1) x code are exact int32 sums, scaled by the fp32
 * norm and summed over the groups in fp32 (in another order on each route,
 * so a token's y from a batched call equals its one-token y only to fp32
 * roundoff). */
int cq_gemv(const void *blob, const bqm_cq_layout *layout, const float *codebook,
            const int8_t *q, const float *scale, int batch, float *y, bqm_stream_t stream);

/* Decode GEMV from fp32 activations: act_fwht_quant_a8 then the cq_gemv
 * product.  x [device] fp32 [batch, cols], 16-byte aligned; y [device] fp32
 * [batch, rows]; q_out [device, may be NULL] int8 [batch, cols] and scale_out
 * [device, may be NULL] fp32 [batch] receive the int8 codes and scales.
 * Other arguments and limits as cq_gemv.  Where cq_gemv would leave the VALU
 * GEMV (see there), or the rows have more than 16384 columns, and both q_out
 * (16-byte aligned) and scale_out are given, the call runs as
 * act_fwht_quant_a8 into them followed by cq_gemv; rows of more than 16384
 * columns without them are BQM_ENOTSUP.  Otherwise one fused launch per 4
 * tokens: every workgroup quantizes the activations itself while its first
 * weight loads are in flight, with the VALU GEMV's arithmetic (a thread holds
 * its segments of the row in registers, hence the 16384-column bound).
 * y equals act_fwht_quant_a8 then
 * cq_gemv bit for bit for batch 1, and whenever q_out and scale_out are
 * given.  The library allocates nothing.  Base-3 ternary (bits 6): the
 * cq_gemv limits, and q_out (16-byte aligned) and scale_out are required
 * (BQM_ENOTSUP without them): act_fwht_quant_a8 into them, then the cq_gemv
 * product. */
int cq_gemv_f32(const void *blob, const bqm_cq_layout *layout, const float *codebook,
                const float *x, int batch, float *y, int8_t *q_out, float *scale_out,
                bqm_stream_t stream);

/* Lookup-table decode GEMV for the binary and ternary sets (bits 1 and 5):
 * the cq_gemv sum computed the Four-Russians / T-MAC way ("llama.cpp on a TV
 * box and a 2013 iPad Air", the kernel table's 1-bit LUT entry).  Each
 * workgroup builds, in LDS, a 16-entry table of int16 partial sums per 4
 * activations (binary: every sign pattern of 4 bits) or per 2 activations
 * (ternary: every pair of 2-bit fields), the tokens side by side in an entry;
 * each nibble of the index stream then costs one table read.  Sums are exact
 * integers per 32-index chunk, scaled by the fp32 group norm and added in
 * fp32.  blob [device] bits 1 or 5 (BQM_ENOTSUP for other codes), group 128;
 * q [device] int8 [batch, cols] (act_fwht_quant_a8); scale [device] fp32
 * [batch]; y [device] fp32 [batch, rows].  1 <= batch <= 16 (launches of up
 * to 4 tokens, fewer where their tables would pass 128 KB of LDS: 16 cols
 * bytes a token for ternary, 8 cols for binary); cols <= 8192, BQM_ENOTSUP
 * otherwise. */
int cq_gemv_lut(const void *blob, const bqm_cq_layout *layout, const int8_t *q, const float *scale, int batch,
                float *y, bqm_stream_t stream);

/* cq_gemv_f32 for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Computes exactly what cq_gemv_f32 computes with q_out and scale_out given
 * (same routes, same kernels, bit-identical y), but stages the int8 codes
 * and scales in a library-owned device scratch instead of caller buffers:
 * 256 KiB + 256 bytes per device, a static device array that each device
 * holds until the process ends (its address is looked up once per device, on
 * the first call there).  The call itself allocates nothing.  Limits: batch
 * <= 16 and cols <= 16384 (BQM_ENOTSUP past them), otherwise those of
 * cq_gemv_f32.  Every call on a device shares that device's scratch: calls
 * that may overlap on one device (different streams without ordering, or
 * host threads) race and must be serialized by the caller.  The scratch
 * needs no clearing: each call writes all it reads. */
int cq_gemv_f32_noalloc(const void *blob, const bqm_cq_layout *layout, const float *codebook,
                        const float *x, int batch, float *y, bqm_stream_t stream);

/* Prefill GEMM on packed CQ weights (Needle article, section 3: prefill is a
 * GEMM with the same layout, every row one reduction stream).  Same sum as
 * cq_gemv for m tokens: q [device] int8 [m, cols], scale [device] fp32 [m],
 * y [device] fp32 [m, rows].  The weight tile is the codebook level times
 * the group norm times 2^e_n, rounded once to fp16, where e_n is a power of
 * two per weight row chosen from the row's largest norm (level x norm x 2^e_n
 * < 2^15) and undone exactly in the fp32 epilogue.  The rounding error is at
 * most 2^-11 relative per weight for every group whose norm is at least
 * 2^-23 of its row's largest (for smaller ones the product may round to an
 * fp16 subnormal: an absolute error below 2^-39 of the row's largest
 * level x norm per weight), so each y[m, n] is within 2^-11 (plus fp32
 * roundoff) of scale[m] / G * sum_g norm[n, g] * sum_i |cb[idx[n, i]]| *
 * |q[m, i]| of the exact sum, at any scale of the row.  Activations enter as
 * exact fp16 integers; the matrix cores accumulate in fp32 and the token
 * scale is applied in fp32.  m >= 1, group must be 128.
 * Up to 32 tokens (cols <= 16384, bits 1-5) the call runs the batched
 * decode kernel of cq_gemv instead, one launch for all tokens, and up to 64
 * tokens in launches of 32 when fewer than 7/8 of the CUs would get a 64 x 64
 * tile: its products are exact (no fp16 rounding of level x norm), so the
 * bound above holds with room.
 * Base-3 ternary (bits 6): exact int32 group sums of digit minus one times
 * code on the int8 matrix cores, each scaled by the group's fp32 norm and
 * added in fp32 in group order; m <= 16 tokens (with cols <= 16384) run the
 * cq_gemv kernels, more tokens (or more columns) a GEMM that reads the
 * weights once per 128 tokens; any m, any cols.
 * Returns BQM_ENOTSUP when the packed indices or m * cols exceed 2^30 bytes
 * (the kernel addresses them with 32-bit offsets). */
int cq_gemm(const void *blob, const bqm_cq_layout *layout, const float *codebook,
            const int8_t *q, const float *scale, int m, float *y, bqm_stream_t stream);

/* Q4_0 GEMV (Minueza-32M -> KMCU v1 page, sections 2 and 3).
 * blocks [device]: rows * ceil(cols/32) blocks of 18 bytes, row-major, each
 * block = fp16 scale d (little-endian) then 16 bytes of 4-bit codes, the low
 * nibble the even element; weight = (nibble - 8) * d; rows are zero-padded to
 * a multiple of 32 so a block never straddles two rows.
 * x [device] fp32 [batch, cols] (no padding needed: columns >= cols are never
 * read); y [device] fp32 [batch, rows].  1 <= batch <= 16.  Returns
 * BQM_ENOTSUP when the blocks reach 2^31 bytes (rows * ceil(cols/32) * 18:
 * the kernel addresses them with 32-bit offsets) or batch > 16. */
int q4_0_gemv(const void *blocks, int rows, int cols, const float *x, int batch, float *y,
              bqm_stream_t stream);

/* Q4_0 prefill GEMM: the q4_0_gemv sum for m tokens (Minueza-32M -> KMCU v1
 * page, sections 2 and 3, for the blocks; Needle article, section 3: prefill
 * is a GEMM over the same [out, in] layout).
 *   y[t, r] = sum_blk sum_{j<32} ((nibble - 8) * d) * x[t, 32 blk + j]
 * blocks [device] as for q4_0_gemv (16-byte aligned); x [device] fp32
 * [m, cols], 16-byte aligned (columns >= cols are never read); y [device] fp32
 * [m, rows].  m >= 1.  Each weight (nibble - 8) * d is formed exactly in fp32
 * and the matrix cores multiply and accumulate in fp32.  Returns BQM_ENOTSUP
 * when the blocks or m * cols * 4 bytes reach 2^31 (32-bit offsets). */
int q4_0_gemm(const void *blocks, int rows, int cols, const float *x, int m, float *y,
              bqm_stream_t stream);

/* Q4_0 weights against int8 activations (A8): the Q4_0 blocks of q4_0_gemv
 * (Minueza-32M -> KMCU v1 page, sections 2-3) and the per-token codes of
 * act_fwht_quant_a8 with group 1 (8-bit activations, Needle article,
 * section 1).
 *   y[t, r] = scale[t] * sum_blk fp32(d) * sum_{j<32} (nibble - 8) * q[t, 32 blk + j]
 * Each block's sum of products is an exact int32, scaled once by the block's
 * fp32 scale; the blocks are summed in fp32.  blocks [device] as for
 * q4_0_gemv (16-byte aligned); q [device] int8 [batch or m, cols] (16-byte
 * aligned base; columns >= cols meet zero weights); scale [device] fp32
 * [batch or m]; y [device] fp32 [batch or m, rows].
 * q4_0_gemv_a8: 1 <= batch <= 16, dot products on v_dot4_i32_i8.
 * q4_0_gemm_a8: m >= 1, the int8 matrix cores, one block per instruction.
 * BQM_ENOTSUP when the blocks or the codes reach 2^31 bytes (32-bit
 * offsets), or batch > 16. */
int q4_0_gemv_a8(const void *blocks, int rows, int cols, const int8_t *q, const float *scale, int batch,
                 float *y, bqm_stream_t stream);
int q4_0_gemm_a8(const void *blocks, int rows, int cols, const int8_t *q, const float *scale, int m,
                 float *y, bqm_stream_t stream);

/* q4_0_gemv_a8 on fp32 activations, their codes formed in the same launch:
 * the per-token codes and scale of act_fwht_quant_a8 with group 1 (8-bit
 * activations, Needle article, section 1; s = RN(amax / 127), 1 for a zero
 * token; q = clamp(rint(RN(x / s)), -127, 127)), then the q4_0_gemv_a8 sum,
 * so y, q_out and scale_out equal the two-launch path's bit for bit.
 * blocks [device] as for q4_0_gemv (16-byte aligned); x [device] fp32
 * [batch, cols] (4-byte aligned); y [device] fp32 [batch, rows]; q_out
 * [device] int8 [batch, cols] and scale_out [device] fp32 [batch] receive
 * the codes and scales when non-NULL.  1 <= batch <= 16.  Every workgroup
 * holds the codes of up to 4 tokens in LDS (36 bytes a token and block):
 * BQM_ENOTSUP past 1706 blocks a row (cols > 54592), when the blocks reach
 * 2^31 bytes, or batch > 16. */
int q4_0_gemv_a8_f32(const void *blocks, int rows, int cols, const float *x, int batch, float *y,
                     int8_t *q_out, float *scale_out, bqm_stream_t stream);

/* Encode fp32 weights into a CQ blob on the device (Needle article,
 * section 1: group FWHT with the normalized Walsh-Hadamard matrix, nearest
 * Lloyd-Max level per coordinate, fp16 group L2 norm, LSB-first packing).
 * Computed in fp64 without fused multiply-adds, in the order:
 *   u = H_u w (butterfly); ss = sum_i u_i*u_i (i ascending); r = sqrt(ss);
 *   norm = fp16_rne(r / sqrt(G)); t_i = u_i * (sqrt(G) / r) (0 if r == 0);
 *   idx_i = argmin_l |t_i - cb_l| (lower l on a tie);
 * so it is bit-exact with a reference that performs the same operations.
 * w [device] fp32 [rows, cols]; codebook [host] as for cq_gemv; blob [device]
 * layout->total_bytes (16-byte aligned; padding bytes are written as zero).
 * status [device, may be NULL] int32 word OR-ed with BQM_STATUS_NONFINITE for
 * a non-finite weight and BQM_STATUS_NORM_OVERFLOW when a norm exceeds fp16;
 * the caller zeroes it beforehand and reads it after synchronizing. */
int cq_pack(const float *w, const bqm_cq_layout *layout, const float *codebook, void *blob,
            int32_t *status, bqm_stream_t stream);

/* Encode fp32 weights into Q4_0 blocks (Minueza page, sections 2 and 3):
 * pad each row to a multiple of 32, per block amax = max|w|, d = amax/8
 * (1 when amax == 0), q = clip(rint(w/d), -8, 7) with correctly rounded fp32
 * division, nibble = q + 8, block = fp16(d) then nibbles (low = even).
 * w [device] fp32 [rows, cols]; blocks [device] rows*ceil(cols/32)*18 bytes. */
int q4_0_pack(const float *w, int rows, int cols, void *blocks, bqm_stream_t stream);

/* Lloyd-Max codebook fit on the device (Needle article, section 1: 400k
 * Gaussian samples, 200 iterations; cb2/cb3/cb4).  One workgroup:
 *   fold to |z|; start the levels/2 positive levels at the interpolated order
 *   statistics (i + 1/2)/(levels/2); each iteration sets cell boundaries at
 *   midpoints of adjacent levels and moves each level to its cell mean (sums
 *   taken over blocks of 512 samples in order, then the block sums in order;
 *   an empty cell keeps its level); mirror to `levels` ascending values.
 * samples [device] fp64 [n] (2 <= n <= 524288, BQM_ENOTSUP above: one
 * workgroup of 1024 threads owns blocks of 512); levels in {2, 4, 8, 16};
 * raw [device, may be NULL] fp64 [levels] unrounded result; table [device]
 * fp32 [levels] each value rounded half-even to bfloat16 precision. */
int cq_codebook_fit(const double *samples, int64_t n, int levels, int iters, double *raw,
                    float *table, bqm_stream_t stream);

/* ---- KMCU v1 container (Minueza-32M -> KMCU v1 page, section 4) ----
 * A little-endian file: a 128-byte header (magic "KMCU", then the u32 fields
 * below in order from byte 4, rope_theta and norm_eps as f32 at bytes 64 and
 * 68, total_params at 72), n_tensors 48-byte directory records at dir_offset
 * (24-byte zero-padded name; u8 dtype at byte 24; u32 n_rows, n_cols,
 * offset, nbytes at bytes 28, 32, 36, 40), tensor data 64-byte aligned.
 * n_cols is the count before the Q4_0 rows are padded to 32.  The functions
 * read the file's bytes where the caller holds them (host memory, read or
 * mapped) and copy nothing except in kmcu_upload.  Every value handed out is
 * checked against the file first: a record's dtype is f32 or Q4_0, its nbytes
 * match its shape (f32: 4 rows cols; Q4_0: 18 rows ceil(cols/32)), its data
 * is 64-byte aligned, at or after data_offset and inside the file, and
 * data_offset itself is 64-byte aligned; BQM_EINVAL otherwise, BQM_ENOTSUP
 * for a version other than 1. */
enum { BQM_KMCU_F32 = 1, BQM_KMCU_Q4 = 2 };

typedef struct {
  uint32_t version, n_layers, dim, n_heads, n_kv_heads, head_dim, ffn_dim, vocab_size, max_seq,
      bos_id, eos_id, tied_embed, n_tensors, dir_offset, data_offset;
  float rope_theta, norm_eps;
  uint32_t total_params;
} bqm_kmcu_header;

typedef struct {
  char name[25];                  /* the record's 24 name bytes, NUL-terminated */
  uint32_t dtype;                 /* BQM_KMCU_F32 or BQM_KMCU_Q4 */
  uint32_t n_rows, n_cols, offset, nbytes;
} bqm_kmcu_tensor;

/* file [host] size bytes -> the header. */
int kmcu_header(const void *file, uint64_t size, bqm_kmcu_header *header);

/* Record `index` (0 <= index < n_tensors) of the directory. */
int kmcu_tensor(const void *file, uint64_t size, int index, bqm_kmcu_tensor *tensor);

/* The first record named `name` (BQM_EINVAL when there is none). */
int kmcu_find(const void *file, uint64_t size, const char *name, bqm_kmcu_tensor *tensor);

/* Copy the tensor's nbytes from the file [host] into dst [device, 16-byte
 * aligned, caller-owned], asynchronously on `stream` (the file memory must
 * stay valid until the copy completes).  A Q4_0 tensor lands as q4_0_gemv /
 * q4_0_gemm blocks, an f32 one as n_rows x n_cols floats. */
int kmcu_upload(const void *file, uint64_t size, const bqm_kmcu_tensor *tensor, void *dst,
                bqm_stream_t stream);

/* The whole data region in one copy: bytes [data_offset, size) of the file
 * [host] to dst [device, 16-byte aligned, dst_bytes >= size - data_offset,
 * caller-owned], asynchronously on `stream`, after every record has been
 * checked.  A tensor then starts at dst + (offset - data_offset); with dst
 * 64-byte aligned its data keeps the file's 64-byte alignment.  The file
 * memory must stay valid until the copy completes (pinned host memory makes
 * it a single DMA transfer). */
int kmcu_upload_data(const void *file, uint64_t size, void *dst, uint64_t dst_bytes,
                     bqm_stream_t stream);

/* Human-readable name of an error code (static string). */
const char *bqm_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* BQM_H */
