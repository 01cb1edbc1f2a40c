/*
 * aqd.h -- C ABI of the additive-codebook decode kernels for AMD MI355X (gfx950).
 *
 * The operation is the decode-time linear layer of Drop-by-Drop
 * ("Multi-Bitwidth Quantization for LLMs Using Additive Codebooks"):
 *
 *     y = s (.) ( What_k . xrot ),     xrot = (1/sqrt(b)) blockdiag(H_b, ..., H_b) x
 *     What_k[i][8j + t] = sum_{m < k} C_m[ codes[i][j][m] ][t]
 *
 * - section 3.2: a row of weights is cut into groups of g = 8 consecutive
 *   inputs; every group is the sum of one codeword per codebook, picked by
 *   that group's code; rows are the concatenation of their group sums.
 * - section 5: inference dequantizes from the first k <= M codebooks only
 *   (the bitwidth knob), and a block-wise Walsh-Hadamard rotation is the
 *   optional pre-processing whose counterpart is applied to the activation.
 * - section 6 "Method Definitions": K codebooks of 8 bits per 8-wide group
 *   give K bits per weight.
 * - appendix "Estimating Model Size": fp16 codebooks [M][2^B][g], B-bit codes,
 *   one fp16 scale per output row (shared by every k).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are device pointers (hipMalloc / PyTorch CUDA tensors) owned by
 *   the caller, except `layer`, which is a host pointer read during the call.
 *   The library allocates no memory and keeps no per-call state; the only
 *   global state is a per-device property cache filled on first use.
 * - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *   Work is enqueued in order on that stream; calls return before it runs.
 * - Arguments are validated on the host before anything is enqueued.  A call
 *   that returns an error has enqueued nothing and written nothing.
 *   aqd_last_error() gives a thread-local message for the last failure.
 * - fp16 and bf16 values are passed as uint16_t bit patterns.  Every
 *   conversion to fp16/bf16 rounds to nearest even.
 * - No C++ exception crosses this interface.  The library is reentrant;
 *   calls on different streams may run concurrently as long as they do not
 *   write the same buffers.
 */
#ifndef AQD_H_
#define AQD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum aqd_status {
    AQD_OK = 0,
    AQD_ERR_NULL = 1,        /* a required pointer is NULL */
    AQD_ERR_SHAPE = 2,       /* d_out/d_in/batch/M out of range or not a supported multiple */
    AQD_ERR_K = 3,           /* k outside [1, M] */
    AQD_ERR_BLOCK = 4,       /* Hadamard block not in {64,128,256} or does not divide d_in */
    AQD_ERR_DTYPE = 5,       /* unsupported dtype combination */
    AQD_ERR_ALIGN = 6,       /* a pointer is not aligned as the call requires */
    AQD_ERR_UNSUPPORTED = 7, /* group != 8 or code_bits != 8 */
    AQD_ERR_WORKSPACE = 8,   /* workspace missing or smaller than required */
    AQD_ERR_HIP = 9          /* a HIP runtime call failed; see aqd_last_error() */
} aqd_status;

typedef enum aqd_dtype {
    AQD_F16 = 0,     /* IEEE binary16 */
    AQD_BF16 = 1,    /* bfloat16 */
    AQD_F32 = 2,     /* IEEE binary32 */
    AQD_BF16X2 = 3   /* a value v stored as two bf16 planes hi, lo (hi = bf16(v),
                        lo = bf16(v - hi)); a [B][n] tensor is [2][B][n]: all hi, then all lo */
} aqd_dtype;

/* One quantized linear layer.  group and code_bits must both be 8
 * (8-wide groups, 256 codewords per codebook). */
typedef struct aqd_layer {
    int64_t d_out;      /* output rows, >= 0 */
    int64_t d_in;       /* inputs, a multiple of 8 */
    int32_t M;          /* code planes (codebooks) stored, 1..8 */
    int32_t group;      /* g, must be 8 */
    int32_t code_bits;  /* B, must be 8 */
} aqd_layer;

/* Version of this interface (incremented on any incompatible change). */
int aqd_abi_version(void);

/* Static text for a status code. */
const char* aqd_status_string(int status);

/* Thread-local text describing the last failed call on this thread ("" if none). */
const char* aqd_last_error(void);

/* ---------------------------------------------------------------------------
 * Code layout (section 5: the first k codebooks are a complete model).
 * Logical codes are [d_out][d_in/8][M] uint8, the index order of the AQLM
 * reconstruction (row i, group j, codebook m).
 *
 * The packed layout is plane-major, so the codes a k-codebook product reads
 * are exactly the first k planes.  A plane is a sequence of 1 KiB tiles, each
 * covering 16 consecutive rows and 64 consecutive groups:
 *
 *   R = ceil(d_out / 16) row tiles, T = ceil((d_in/8) / 64) group tiles,
 *   plane bytes P = R * T * 1024,
 *   packed[m*P + (jt*R + it)*1024 + l*16 + r] = codes[16*it + r][64*jt + l][m]
 *
 * with zero bytes where 16*it + r >= d_out or 64*jt + l >= d_in/8 (padding
 * that never contributes to a product).  Lane l of a 64-wide wavefront that
 * loads 16 bytes of a tile receives the codes of one group for 16 rows.
 * ------------------------------------------------------------------------- */

/* Bytes of the packed codes: M * P (see above); 0 for an invalid layer. */
size_t aqd_packed_codes_bytes(const aqd_layer* layer);

/* codes [d_out][d_in/8][M] -> packed tiles.  Byte exact; writes the padding zeros. */
aqd_status aqd_pack_codes(const uint8_t* codes, uint8_t* packed, const aqd_layer* layer, void* stream);

/* packed tiles -> codes [d_out][d_in/8][M].  Inverse of aqd_pack_codes. */
aqd_status aqd_unpack_codes(const uint8_t* packed, uint8_t* codes, const aqd_layer* layer, void* stream);

/* ---------------------------------------------------------------------------
 * Online rotation of the activation (section 5, block-wise Walsh-Hadamard
 * rotation; section 6, the rotation is applied online at inference).
 *
 * x_rot[n][beta*b + r] = (1/sqrt(b)) * sum_c H_b[r][c] * x[n][beta*b + c],
 * H_b[r][c] = (-1)^popcount(r & c) (Sylvester order), blocks of b contiguous
 * inputs starting at input 0, no sign flips (aqd_hadamard_rotate_signed adds
 * them).  Computed in fp32 by butterflies,
 * then rounded once to out_dtype.
 *
 * x:      [batch][d_in] in in_dtype (AQD_F16, AQD_BF16 or AQD_F32).
 * x_rot:  [batch][d_in] in out_dtype (AQD_F16, AQD_BF16, AQD_F32), or
 *         [2][batch][d_in] for AQD_BF16X2.  May alias x only when in_dtype and
 *         out_dtype are equal and not AQD_BF16X2.
 * block:  b in {64, 128, 256}; b must divide d_in.  batch >= 0.
 * Both pointers 16-byte aligned.
 * ------------------------------------------------------------------------- */
aqd_status aqd_hadamard_rotate(const void* x, void* x_rot, int in_dtype, int out_dtype,
                               int64_t batch, int64_t d_in, int32_t block, void* stream);

/* ---------------------------------------------------------------------------
 * Randomized block rotation R = (1/sqrt(b)) * H_b * diag(eps) per block: the
 * randomized Hadamard transform H diag(eps) named in "ApexQuant:
 * calibration-free elastic quantization", section 3 (after Eq. 2), applied
 * with the block layout of aqd_hadamard_rotate.  The weights it pairs with are
 * quantized from W R^T, so that (W R^T)(R x) = W x.
 *
 * signs:  device bit mask of d_in bits, one pattern for every batch row:
 *         eps_c = -1 when bit (c mod 8) of byte signs[c / 8] is set, else +1
 *         (the same memory read as little-endian 64-bit words: bit c mod 64 of
 *         word c / 64).  d_in / 8 bytes, 8-byte aligned, caller-owned.
 * Each input is negated (exactly) where its bit is set and the result is then
 * bit-identical to aqd_hadamard_rotate of the sign-flipped input.  Other
 * arguments, aliasing rules and errors as for aqd_hadamard_rotate, plus
 * AQD_ERR_NULL for a NULL signs and AQD_ERR_ALIGN for a misaligned one (when
 * batch * d_in > 0).
 * ------------------------------------------------------------------------- */
aqd_status aqd_hadamard_rotate_signed(const void* x, void* x_rot, int in_dtype, int out_dtype,
                                      int64_t batch, int64_t d_in, int32_t block, const uint8_t* signs,
                                      void* stream);

/* ---------------------------------------------------------------------------
 * Decode GEMV, batch 1..8 (the lookup-and-accumulate hot path).
 *
 * y[n][i] = fp16( s_i * sum_j sum_{m<k} < C_m[codes[i][j][m]], x_rot[n][8j .. 8j+8) > )
 *
 * packed_codes: plane-major codes (see above); only the first k planes are read.
 * codebooks:    fp16 [M][256][8]; only the first k codebooks are read.
 * scales:       fp16 [d_out].
 * x_rot:        fp16 [batch][d_in], the already rotated activation.
 * y:            fp16 [batch][d_out].
 * k:            1..M.  batch: 1..8.
 * workspace:    device scratch of aqd_gemv_workspace_bytes(layer, batch) bytes
 *               (NULL allowed when it is 0).  It must be zero-filled before its
 *               first use; every successful call leaves the parts that must
 *               start at zero zeroed again, so one buffer of the largest size
 *               needed serves any number of calls, at any batch, on one
 *               stream.  Calls that may overlap in time need separate
 *               workspaces.  It must not be shared with aqd_gemm_small_batch,
 *               aqd_gemm_small_batch_tiered or aqd_gemm_prefill, whose
 *               workspaces hold partial sums.
 *               A workspace whose first aqd_gemv_workspace_bytes(layer, 1)
 *               bytes are not zero when a call on a table route starts (batch
 *               1 and 2; batch 3 and 4 at k <= 2 on layers of at most 32 table
 *               slots, i.e. k * ceil(d_in / 512) <= 32) (never
 *               zero-filled, written by another entry point, or left by a call
 *               whose kernel did not complete) cannot be detected: the rows
 *               whose words are not zero get undefined outputs (a row may be
 *               left unwritten or receive a wrong value), the call still
 *               returns AQD_OK, and those words may stay non-zero for later
 *               calls.  Zero-filling the workspace again recovers.
 * Value range of the table routes (batch 1..4, above): every table entry
 * < C_m[c], x_rot[n][8j .. 8j+8) > is rounded to fp16, so its magnitude must
 * stay below 65504, and entries below 2^-14 (fp16 subnormals) carry an
 * absolute error of up to 2^-25 each; the partial row sums that travel
 * between workgroups are fixed point with 24 fraction bits (absolute error
 * up to 2^-25 per term) and saturate at 2^23.  The error therefore depends on
 * the product of the activation and codebook scales: for rotated activations
 * of RMS a and codebook entries of RMS c, the measured normwise error against
 * an exact product stays below 6e-4 for a * c / 0.05 from 2^-12 up to 2^8
 * (tested; beyond that the fp16 output of these layers overflows), is about
 * 1e-3 at 2^-13 and exceeds the 2e-3 bound near 2^-14.
 * Batch 1 and 2 read per-group tables of codeword-activation products (one
 * table per column, built on the matrix cores): one table lookup per code byte
 * (all columns' entries in one read).  Batch 3 and 4 do the same with four
 * columns per entry where k <= 2 and k * ceil(d_in / 512) <= 32.  Other calls
 * at batch 2..8 with batch * k > 4 run on the matrix cores (the fp16 operand
 * mode of aqd_gemm_small_batch, result rounded to fp16); the remaining cases use
 * codeword lookups with v_dot2 accumulation.  (Inputs too long for the tables,
 * k * ceil(d_in / 512) above 1020 at batch 1 or 510 at batch 2, take the latter
 * routes too.)
 * Accumulation is fp32; the summation order is not specified, but it is fixed:
 * repeating a call on the same inputs gives the same bits.
 * packed_codes, x_rot and workspace 16-byte aligned; codebooks 16-byte aligned.
 * ------------------------------------------------------------------------- */
size_t aqd_gemv_workspace_bytes(const aqd_layer* layer, int32_t batch);

aqd_status aqd_gemv(const uint8_t* packed_codes, const uint16_t* codebooks, const uint16_t* scales,
                    int32_t k, const uint16_t* x_rot, uint16_t* y, int32_t batch,
                    const aqd_layer* layer, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * aqd_gemv for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): no
 * workspace argument, and the call allocates nothing (no hipMalloc, no
 * allocating library routine).  Its workspace is a fixed device array inside
 * the library, AQD_NOALLOC_SCRATCH_BYTES on every GPU it runs on, held until
 * the process ends; the first call on a device looks up that device's copy.
 * Every call clears the part that must start at zero with a small fill kernel
 * on `stream` (one launch more than aqd_gemv), then runs exactly aqd_gemv's
 * kernels: outputs have aqd_gemv's bits.
 *
 * All calls on one GPU share its array: calls that may overlap in time (on
 * different streams, or from several threads) race and give undefined outputs.
 * Layers whose aqd_gemv_workspace_bytes(layer, batch) exceeds
 * AQD_NOALLOC_SCRATCH_BYTES are rejected with AQD_ERR_WORKSPACE before anything
 * is enqueued (the limit covers about 65 thousand output rows at batch 8 with
 * 14336 inputs, and about half a million at batch 1).  Other arguments and
 * errors as for aqd_gemv.
 * ------------------------------------------------------------------------- */
#define AQD_NOALLOC_SCRATCH_BYTES (16u << 20)

aqd_status aqd_gemv_noalloc(const uint8_t* packed_codes, const uint16_t* codebooks, const uint16_t* scales,
                            int32_t k, const uint16_t* x_rot, uint16_t* y, int32_t batch,
                            const aqd_layer* layer, void* stream);

/* ---------------------------------------------------------------------------
 * Grouped batch-1 GEMV: up to AQD_MAX_GROUP linears that read the same rotated
 * input (q, k and v of an attention block; gate and up of an MLP) in one
 * launch.  Each linear computes exactly what aqd_gemv computes for it at
 * batch 1 (Drop-by-Drop, sections 3.2 and 5), with the same bits.  The table
 * slots per workgroup, which decide the bits, are chosen per linear as for
 * aqd_gemv; linears that choose differently (a small linear beside a large one
 * at k = 3 or 4) are issued as one launch per choice, in the same stream.
 *
 * linears:   n_linears descriptors (host memory, read during the call only):
 *            packed codes, codebooks, scales and fp16 output y [d_out] of each
 *            linear, as for aqd_gemv; group 8 and 8-bit codes.
 * k:         codebooks used by every linear, 1..min M.
 * x_rot:     fp16 [d_in], shared.
 * workspace: aqd_gemv_grouped_workspace_bytes(linears, n_linears, d_in) bytes,
 *            zero-filled before first use and left zeroed, as for aqd_gemv.
 * Errors as for aqd_gemv; AQD_ERR_SHAPE for n_linears outside 1..AQD_MAX_GROUP;
 * AQD_ERR_UNSUPPORTED (nothing launched) when k * ceil(d_in / 512) exceeds
 * 1020: the lookup tables of one launch cannot cover the input (aqd_gemv per
 * linear still can).
 * ------------------------------------------------------------------------- */
#define AQD_MAX_GROUP 4

typedef struct {
    const uint8_t* packed_codes;
    const uint16_t* codebooks;
    const uint16_t* scales;
    uint16_t* y;
    int64_t d_out;
    int32_t M;
} aqd_linear;

size_t aqd_gemv_grouped_workspace_bytes(const aqd_linear* linears, int32_t n_linears, int64_t d_in);

aqd_status aqd_gemv_grouped(const aqd_linear* linears, int32_t n_linears, int32_t k, const uint16_t* x_rot,
                            int64_t d_in, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Rotation and grouped batch-1 GEMV in one launch.  x is the raw (unrotated)
 * fp16 activation [d_in]; every workgroup applies the block Walsh-Hadamard
 * rotation of aqd_hadamard_rotate (block 64, 128 or 256, same butterflies and
 * fp16 rounding) to the inputs it needs, then proceeds as aqd_gemv_grouped:
 * the outputs have the bits of aqd_hadamard_rotate (F16 out) followed by
 * aqd_gemv_grouped (Drop-by-Drop, section 5: the activation is rotated online).
 * AQD_ERR_BLOCK if block is not 64/128/256 or does not divide d_in; other
 * arguments, workspace and errors as for aqd_gemv_grouped.
 * ------------------------------------------------------------------------- */
aqd_status aqd_rotate_gemv_grouped(const aqd_linear* linears, int32_t n_linears, int32_t k, const uint16_t* x,
                                   int64_t d_in, int32_t block, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* ---------------------------------------------------------------------------
 * As aqd_rotate_gemv_grouped with the randomized rotation of
 * aqd_hadamard_rotate_signed: the outputs have the bits of
 * aqd_hadamard_rotate_signed (F16 out, same signs) followed by
 * aqd_gemv_grouped.  signs: d_in / 8 bytes, 8-byte aligned device memory, the
 * bit layout of aqd_hadamard_rotate_signed; AQD_ERR_NULL / AQD_ERR_ALIGN when
 * d_in > 0 and it is NULL / misaligned.  Other arguments and errors as for
 * aqd_rotate_gemv_grouped.
 * ------------------------------------------------------------------------- */
aqd_status aqd_rotate_gemv_grouped_signed(const aqd_linear* linears, int32_t n_linears, int32_t k,
                                          const uint16_t* x, int64_t d_in, int32_t block, const uint8_t* signs,
                                          void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Small-batch product, batch 1..64, on the matrix cores.  Each wave rebuilds
 * the weight slice its MFMA operand holds from the codes (codeword sums) and
 * multiplies it with 16-column tiles of the rotated activation, accumulating in
 * fp32 (v_mfma_f32_16x16x32).
 *
 * y[n][i] = s_i * sum_j sum_{m<k} < C_m[codes[i][j][m]], x_rot[n][8j .. 8j+8) >   (fp32)
 *
 * x_dtype selects the operand precision:
 *   AQD_BF16    x_rot bf16 [batch][d_in]; weights as bf16 hi + lo (2 bf16 passes)
 *   AQD_BF16X2  x_rot [2][batch][d_in] bf16 hi, lo planes; 3 bf16 passes
 *               (weights hi and lo against the activation hi, weights hi
 *               against the activation lo): close to fp32 accuracy
 *   AQD_F16     x_rot fp16 [batch][d_in]; weights as fp16 codeword sums; one
 *               fp16 pass (same MFMA rate as bf16, 2^-11 operand rounding)
 * y:      fp32 [batch][d_out], overwritten.
 * workspace: aqd_gemm_small_batch_workspace_bytes(layer, batch) bytes (split
 *         partials, fully overwritten by every call; NULL when 0).  Other
 *         arguments as for aqd_gemv.  Results are bit-reproducible.
 * ------------------------------------------------------------------------- */
size_t aqd_gemm_small_batch_workspace_bytes(const aqd_layer* layer, int32_t batch);

/* ---------------------------------------------------------------------------
 * Tiered batch: the small-batch product where column n of the batch uses its
 * own number of codebooks ks[n] (1..M), in one launch.  Each codebook plane m
 * is read once for all the columns with ks[n] > m; with the planes stored as a
 * prefix (Drop-by-Drop, section 5: any first k codebooks form a model) a batch
 * of requests at different bitwidths shares one pass over the codes.
 *
 * y[n][i] = s_i * sum_j sum_{m < ks[n]} < C_m[codes[i][j][m]], x_rot[n][8j .. 8j+8) >   (fp32)
 *
 * ks:     host array [batch], each 1..M (AQD_ERR_K otherwise), read during the call.
 * x_rot:  fp16 [batch][d_in] (already rotated).  One fp16 MFMA pass per
 *         codebook plane, fp32 accumulation.
 * y, workspace (aqd_gemm_small_batch_workspace_bytes), errors: as for
 * aqd_gemm_small_batch.
 * ------------------------------------------------------------------------- */
aqd_status aqd_gemm_small_batch_tiered(const uint8_t* packed_codes, const uint16_t* codebooks,
                                       const uint16_t* scales, const int32_t* ks, const uint16_t* x_rot,
                                       float* y, int32_t batch, const aqd_layer* layer,
                                       void* workspace, size_t workspace_bytes, void* stream);

aqd_status aqd_gemm_small_batch(const uint8_t* packed_codes, const uint16_t* codebooks,
                                const uint16_t* scales, int32_t k, const void* x_rot, int x_dtype,
                                float* y, int32_t batch, const aqd_layer* layer,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Prefill / large-batch product on the matrix cores, batch 1..32768.  The
 * compute-bound regime of the same linear (Drop-by-Drop, section 3.2: each
 * weight group is the sum of its codewords; section 5: the first k
 * codebooks).  The ApexQuant page, appendix H "Nested decoding in service",
 * notes that prefill is compute-bound and leaves it unmeasured:
 *
 *     y[n][i] = s_i * sum_c W_k[i][c] * x_rot[n][c]      (fp32 out)
 *
 * The weights are fp16 codeword sums (packed fp16 adds in plane order, as the
 * fp16 small-batch mode), multiplied with v_mfma_f32_16x16x32_f16 and
 * accumulated in fp32.  Each workgroup rebuilds its 256 weight rows from the
 * codes at k <= 2 (any batch), at k = 3, 4 up to batch 1023 and at k >= 5 up
 * to batch 511.  Otherwise the library first writes the whole fp16 weight
 * (2 * d_out * d_in bytes) into the workspace and the product reads it from
 * there.  Both forms use the same fp16 weights.  Throughput is meant for batch >= 128; any batch
 * in range is correct.
 *
 * packed_codes, codebooks, scales: as for aqd_gemv; only the first k planes
 *               and codebooks are read.
 * x_rot:        fp16 [batch][d_in], the rotated activation, 16-byte aligned.
 * y:            fp32 [batch][d_out], 4-byte aligned.
 * k:            1..M.  batch: 1..AQD_PREFILL_MAX_BATCH.
 * workspace:    aqd_gemm_prefill_workspace_bytes(layer, batch) bytes, the
 *               largest over k: the fp16 weight where it is staged (layers up
 *               to 2 GiB of fp16 weights; larger ones always rebuild in the
 *               workgroups) plus fp32 partial sums when the inputs are split.
 *               0 when neither is needed (NULL is then allowed).  16-byte
 *               aligned, fully overwritten by every call; calls that may
 *               overlap in time need separate ones.
 * The summation order is fixed (input splits are added in order by a second
 * kernel), so repeating a call gives the same bits.
 * Errors: AQD_ERR_SHAPE for batch out of range, otherwise as for
 * aqd_gemm_small_batch.
 * ------------------------------------------------------------------------- */
#define AQD_PREFILL_MAX_BATCH 32768

size_t aqd_gemm_prefill_workspace_bytes(const aqd_layer* layer, int32_t batch);

aqd_status aqd_gemm_prefill(const uint8_t* packed_codes, const uint16_t* codebooks, const uint16_t* scales,
                            int32_t k, const uint16_t* x_rot, float* y, int32_t batch, const aqd_layer* layer,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Encode side: greedy residual code assignment for fixed codebooks.
 *
 * Drop-by-Drop section 3.2 gives the decoder (a group is the sum of one
 * codeword per codebook) and section 5 the prefix order; AQLM's own code
 * search is not on the pages.  This stand-in respects the prefix order: for
 * every group of 8 targets, codebook m = 0, 1, ..., M-1 in turn takes the
 * codeword nearest (squared Euclidean distance) to the residual the earlier
 * codebooks left, and the residual loses it, so every prefix of the codes is
 * the greedy code for that many codebooks.
 *
 * The decision is taken in float32 with one fixed operation order:
 *   e_t = r_t - C[c][t];  d = fma(e_t, e_t, d) for t = 0..7 from d = 0;
 *   the smallest d wins, equal d go to the lower index;  r_t = r_t - C[c*][t].
 *
 * target:    float32 [d_out][d_in], 16-byte aligned: the weights already
 *            rotated (W Q^T, e.g. aqd_hadamard_rotate of the rows with F32
 *            in and out) and divided by their row scale.
 * codebooks: fp16 [M][256][8], 2-byte aligned.  M: 1..8.
 * codes:     uint8 [d_out][d_in/8][M] out (the logical layout aqd_pack_codes
 *            takes).  All pointers are device memory owned by the caller.
 * Errors: AQD_ERR_SHAPE for M outside 1..8, d_in not a multiple of 8 or
 * sizes out of range; AQD_ERR_NULL / AQD_ERR_ALIGN as usual.
 * ------------------------------------------------------------------------- */
aqd_status aqd_encode_greedy(const float* target, const uint16_t* codebooks, int32_t M, int64_t d_out,
                             int64_t d_in, uint8_t* codes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AQD_H_ */
