/*
 * bsl.h -- C ABI of libbsl.so: banded block-sparse attention forward on
 * MI355X (gfx950).
 *
 * The operation is the forward pass described on the NucleoByte project page
 * ("NucleoByte: GPU-Accelerated Block-Sparse Genomic Language Model"):
 *   - section 3, "Localized Block-Sparse Attention Matrix": with block size
 *     B = 32, query block i attends only to key blocks j with |i - j| <= R;
 *   - section 3, "Softmax Normalization & Online Numerical Stability": scores
 *     S = Q K^T / sqrt(d_k); a running row maximum, denominator and output are
 *     carried across the active key blocks, and the output is the softmax-
 *     weighted sum of V (divided by the denominator after the last block);
 *   - section 2, item 2, "Dynamic Ceiling Hardware Alignment": each batch is
 *     padded up to a multiple of 32; keys past a sequence's own length are
 *     masked, and blocks that hold only padding are skipped.
 * An optional causal flag additionally drops keys after the query (s > t).
 *
 * Layout.  Q, K, V and O are dense [batch][heads][n][head_dim] arrays, head_dim
 * innermost, in the plan's dtype (bf16 or fp32), on the device the plan was
 * created on.  n is the padded buffer length (a multiple of 32).  Row t of a
 * sequence with length L is real when t < L; rows t >= L are padding: their
 * Q/K/V values are never used (they may hold NaN) and their O rows are written
 * as zeros.  bsl_forward_varlen takes the packed alternative: the sequences
 * back to back in [tokens][heads][head_dim] arrays, located by offsets.
 *
 * Ownership.  The caller owns every buffer.  A plan holds only immutable
 * settings and device facts; it allocates no device memory, so one plan may be
 * used from several host threads and streams at once.
 *
 * Asynchrony.  bsl_forward, bsl_forward_traced, bsl_forward_varlen and
 * bsl_backward only enqueue work on the given stream (NULL = the default
 * stream) and never synchronise.
 *
 * Errors.  Every call returns a bsl_status.  Argument errors are reported
 * before anything is launched, and then nothing is written.  A failed launch
 * returns BSL_E_DEVICE.  bsl_last_error() gives a per-thread text for the last
 * failing call.  Nothing aborts, exits or throws across this interface.
 */
#ifndef BSL_H
#define BSL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSL_VERSION 10700 /* major * 10000 + minor * 100 + patch */

typedef enum bsl_status {
    BSL_OK = 0,
    BSL_E_INVALID = 1,     /* bad argument: nothing was launched or written */
    BSL_E_UNSUPPORTED = 2, /* well-formed but outside what this library supports */
    BSL_E_DEVICE = 3,      /* HIP runtime failure (device query or launch) */
    BSL_E_NOMEM = 4        /* host allocation of a plan failed */
} bsl_status;

typedef enum bsl_dtype {
    BSL_BF16 = 0, /* bf16 in and out; bf16 MFMA products, fp32 accumulation */
    BSL_F32 = 1   /* fp32 in and out; fp32 arithmetic throughout */
} bsl_dtype;

typedef struct bsl_desc {
    int32_t head_dim;   /* d: 32, 64 or 128 */
    int32_t heads;      /* heads per sequence, >= 1 */
    int32_t block_size; /* B: must be 32, the block size the page fixes */
    int32_t radius;     /* R >= 0: key blocks j with |i - j| <= R are scored */
    int32_t causal;     /* 0 or 1: 1 also drops keys s > t */
    int32_t dtype;      /* a bsl_dtype */
    float scale;        /* > 0: score scale; <= 0: 1 / sqrt(head_dim) */
    int32_t window;     /* 0: the block band of radius R (the page's rule).
                           W >= 1: a token window instead, the plain reading
                           of the local neighbourhood W of section 2, item 3:
                           key s is scored for query t when |t - s| <= W,
                           over the blocks within ceil(W/32) of the query
                           block.  radius is then not used (it must still be
                           >= 0).  Every call of the plan (forward, packed
                           forward, backward) uses the window. */
} bsl_desc;

typedef struct bsl_plan bsl_plan;

/* Validate *desc against the current HIP device and make a plan for it.
 * BSL_E_INVALID: desc or plan NULL, heads < 1, radius < 0, causal not 0/1,
 *   non-finite scale, window < 0.
 * BSL_E_UNSUPPORTED: head_dim not 32/64/128, block_size != 32, unknown dtype,
 *   window > 2^29, radius > 2^24, or the current device is not gfx950.
 * BSL_E_DEVICE: the device could not be queried.
 * On success *plan is set; release it with bsl_destroy. */
bsl_status bsl_create(const bsl_desc *desc, bsl_plan **plan);

/* Enqueue the forward pass.
 *   batch   >= 0 sequences; n >= 0 rows per sequence buffer, n % 32 == 0.
 *           batch == 0 or n == 0 is a no-op returning BSL_OK.
 *   q, k, v device pointers, [batch][heads][n][head_dim] in the plan's dtype.
 *   o       device pointer, same shape and dtype; every row is written.  It must
 *           not overlap q, k or v.
 *   seqlens device int32[batch] with 0 <= seqlens[b] <= n, or NULL for all n.
 *           Values outside [0, n] are clamped to it on the device.
 *   lse     device float[batch][heads][n] or NULL: natural-log log-sum-exp of
 *           each row's scaled scores over its kept keys; -inf on padded rows.
 *   stream  a hipStream_t, or NULL for the default stream.
 * q, k, v, o and lse are 16-byte aligned.  The buffers the call writes (o, lse)
 * overlap neither each other nor any buffer it reads (q, k, v, seqlens).
 * Returns BSL_E_INVALID for a NULL plan, negative sizes, n % 32 != 0, a NULL
 * q/k/v/o when batch * n > 0, a misaligned pointer, overlapping buffers, or
 * sizes whose element count does not fit in 63 bits; BSL_E_INVALID also when
 * the current device is not the plan's. */
bsl_status bsl_forward(const bsl_plan *plan, int32_t batch, int32_t n, const void *q,
                       const void *k, const void *v, void *o, const int32_t *seqlens,
                       float *lse, void *stream);

/* bsl_forward, plus a record of what the kernel did, for verification.  Below,
 * R is the plan's radius, or ceil(window / 32) for a plan with a token window.
 *   active  device int32[batch][n/32][2R+1]: for query block i of sequence b,
 *           the key blocks the kernel visited, ascending, then -1 in the unused
 *           slots (all -1 for blocks that hold only padding).
 *   masks   device uint32[batch][n/32][2R+1][32]: for slot s of query block i,
 *           word r has bit c set iff the kernel kept key c of that key block
 *           for query row r; zero for unused slots and padded query rows.
 * Both are required (non-NULL), 4-byte aligned, and are written in full; they
 * describe head 0 (the band and the masks are the same for every head).  Like
 * o and lse they overlap no other buffer of the call (BSL_E_INVALID). */
bsl_status bsl_forward_traced(const bsl_plan *plan, int32_t batch, int32_t n, const void *q,
                              const void *k, const void *v, void *o, const int32_t *seqlens,
                              float *lse, int32_t *active, uint32_t *masks, void *stream);

/* bsl_forward over a packed batch: the sequences lie back to back with no
 * padding between them (the padding the page's section 1, "Padding Waste",
 * counts as wasted memory and bandwidth), addressed by offsets.  The operation
 * per sequence is exactly bsl_forward's on that sequence alone: same band, same
 * masks, same arithmetic, so each row's output equals bit for bit the one
 * bsl_forward writes for the same data in the padded layout.
 *   batch       >= 0 sequences.
 *   tokens      >= 0 rows in the packed buffers (the sum of the lengths).
 *   max_seqlen  >= 0, a bound on every length; it sizes the launch, so the host
 *               need not read cu_seqlens.  A sequence longer than max_seqlen is
 *               treated as its first max_seqlen rows; the rest of its rows are
 *               not written.
 *   q, k, v     device pointers, [tokens][heads][head_dim] in the plan's dtype:
 *               row t of sequence b, head h, is at ((cu_seqlens[b] + t) * heads
 *               + h) * head_dim.  This is the projection's own output layout,
 *               with no transpose.
 *   o           device pointer, same shape and dtype; only the rows of the
 *               sequences are written: rows outside every [cu_seqlens[b],
 *               cu_seqlens[b+1]) are left as they were.  It must not overlap
 *               q, k or v.
 *   cu_seqlens  device int32[batch + 1], non-decreasing, cu_seqlens[0] = 0,
 *               cu_seqlens[batch] <= tokens: sequence b is rows [cu_seqlens[b],
 *               cu_seqlens[b+1]).  Values are clamped into [0, tokens] on the
 *               device (a decreasing pair gives an empty sequence), so no
 *               value can send an access outside the buffers.  Out-of-order
 *               offsets make later sequences overlap earlier ones; rows two
 *               sequences share get either's value.
 *   lse         device float[heads][tokens] or NULL: as in bsl_forward, for the
 *               sequences' rows.
 *   stream      a hipStream_t, or NULL for the default stream.
 * batch, tokens or max_seqlen == 0 is a no-op returning BSL_OK.  Returns
 * BSL_E_INVALID for a NULL plan or cu_seqlens, negative sizes, a NULL or
 * misaligned (not 16-byte) q/k/v/o, a misaligned lse, o or lse overlapping
 * each other or a buffer the call reads (q, k, v, cu_seqlens), sizes past the
 * limits of bsl_forward, or a current device that is not the plan's. */
bsl_status bsl_forward_varlen(const bsl_plan *plan, int32_t batch, int32_t tokens,
                              int32_t max_seqlen, const void *q, const void *k, const void *v,
                              void *o, const int32_t *cu_seqlens, float *lse, void *stream);

/* Host-side collation of a batch's lengths (section 2, item 2 of the page,
 * "Dynamic Ceiling Hardware Alignment"): from host int32 lengths[batch] (each
 * >= 0) write host int32 cu_seqlens[batch + 1] (exclusive prefix sums, the
 * offsets bsl_forward_varlen takes), *max_seqlen (the longest length) and
 * *ceiling (that length rounded up to the next multiple of 32: the buffer
 * length n a padded batch needs for bsl_forward).  No device work.
 * BSL_E_INVALID for batch < 0, a NULL pointer (lengths may be NULL when batch
 * is 0), a negative length, or a sum or ceiling past 2^31 - 1; nothing is
 * written then. */
bsl_status bsl_varlen_offsets(int32_t batch, const int32_t *lengths, int32_t *cu_seqlens,
                              int32_t *max_seqlen, int32_t *ceiling);

/* Enqueue the backward pass of bsl_forward (NucleoByte project page, section 3,
 * "Custom Backpropagation"): from the output gradient dO, the gradients dQ, dK,
 * dV of the same loss.  With P the forward's softmax over each row's kept keys,
 *   D_t = sum_c dO_tc O_tc,   dS_ts = P_ts (dO_t . V_s - D_t),
 *   dV = P^T dO,   dQ = scale dS K,   dK = scale dS^T Q,
 * and zero gradient on padded rows and keys.  bf16 plans at head_dim 64 and
 * 128 run on MFMA kernels; fp32 plans, and bf16 plans at head_dim 32, on
 * vector-ALU kernels (fp32 arithmetic; bf16 gradients rounded once).
 *   batch, n, seqlens, stream  as in bsl_forward (the same values it was given).
 *   q, k, v  the forward's inputs; o its output, exactly as bsl_forward wrote it.
 *   dout     device [batch][heads][n][head_dim] in the plan's dtype: the loss
 *            gradient w.r.t. o.  Rows past a sequence's length are ignored.
 *   lse      device float[batch][heads][n]: the lse bsl_forward wrote.
 *   dq, dk, dv  device, same shape and dtype as q; every element is written.
 *   delta    device float[batch][heads][n], a workspace the caller owns: the
 *            call overwrites it with D (0 on padded rows).  The library
 *            allocates nothing.
 * All tensors 16-byte aligned.  dq, dk, dv and delta must not overlap each
 * other or any input (seqlens included).  A plan with a token window differentiates the window
 * forward.  Returns BSL_E_INVALID for the argument errors bsl_forward
 * rejects, a NULL pointer, misalignment or overlap, and BSL_E_DEVICE if a
 * launch fails.
 * Nothing is written when an argument error is returned. */
bsl_status bsl_backward(const bsl_plan *plan, int32_t batch, int32_t n, const void *q,
                        const void *k, const void *v, const void *o, const void *dout,
                        const float *lse, const int32_t *seqlens, void *dq, void *dk, void *dv,
                        float *delta, void *stream);

/* bsl_backward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same gradients from the same kernels, bit for bit, with the row vector D
 * kept in a fixed workspace of the library instead of a caller's delta.
 *   Arguments as bsl_backward, without delta.
 * The workspace is one file-scope device array of 8 Mi floats (32 MiB) that
 * every device the library runs on holds until the process ends; this call
 * allocates nothing.  batch * heads * n may be at most 8,388,608 (8 Mi) rows:
 * beyond that the call returns BSL_E_UNSUPPORTED (use bsl_backward).  Every
 * call on one device uses that device's one workspace, so calls that overlap
 * in time on the same device (other streams, other threads) race and must not
 * be made; calls in order on one stream are safe.  Nothing in the workspace
 * needs to start at zero: each call writes every row it reads.  Other errors
 * as bsl_backward. */
bsl_status bsl_backward_noalloc(const bsl_plan *plan, int32_t batch, int32_t n, const void *q,
                                const void *k, const void *v, const void *o, const void *dout,
                                const float *lse, const int32_t *seqlens, void *dq, void *dk,
                                void *dv, void *stream);

/* bsl_backward over the packed layout of bsl_forward_varlen: the same
 * gradients per sequence, each sequence alone, with the rows back to back.
 *   batch, tokens, max_seqlen, cu_seqlens, stream  as in bsl_forward_varlen
 *            (the same values it was given).
 *   q, k, v, o, dout  device [tokens][heads][head_dim] in the plan's dtype: the forward's
 *            inputs and output, and the loss gradient w.r.t. o.
 *   lse      device float[heads][tokens]: the lse bsl_forward_varlen wrote.
 *   dq, dk, dv  device [tokens][heads][head_dim]: only the rows of the
 *            sequences are written; rows outside every sequence are left as
 *            they were.
 *   delta    device float[heads][tokens], the caller's workspace: D on the
 *            sequences' rows.
 * Each sequence's gradients equal, bit for bit, those bsl_backward writes for
 * the same data in the padded layout.  Errors as bsl_backward, with the size
 * limits of bsl_forward_varlen; batch, tokens or max_seqlen == 0 is a no-op. */
bsl_status bsl_backward_varlen(const bsl_plan *plan, int32_t batch, int32_t tokens,
                               int32_t max_seqlen, const void *q, const void *k, const void *v,
                               const void *o, const void *dout, const float *lse,
                               const int32_t *cu_seqlens, void *dq, void *dk, void *dv,
                               float *delta, void *stream);

/* ------------------------------------------------------------------------
 * Fused 2-bit k-mer tokenization: the step that feeds the model's token IDs
 * (NucleoByte project page, section 2, item 1, "Fused 2-Bit Tokenization"; the
 * k-mer size and vocabulary are those of section 5: 6-mers, 4096 IDs plus
 * padding and mask entries, 4100 in the usage example of section 6).
 *
 * Each base is two bits: A = 0, C = 1, G = 2, T = 3, upper or lower case (soft-
 * masked FASTA text).  Window t of a sequence covers bases t .. t+k-1 (a
 * sliding window, stride one) and its ID is the base-4 number of its codes,
 * first base most significant:  id_t = sum_p code(base[t+p]) * 4^(k-1-p)  (the
 * page prints TGGGAC = 3745, TGAAGT = 3595, GGCCCC = 2645).  A window that
 * holds any other byte ('N', IUPAC codes, line breaks) is UNK.  The special
 * IDs follow the 4^k k-mer IDs: */
#define BSL_KMER_PAD(k) (1 << (2 * (k)))        /* rows past a sequence's last window */
#define BSL_KMER_MASK(k) (BSL_KMER_PAD(k) + 1)  /* reserved for masked-token training */
#define BSL_KMER_UNK(k) (BSL_KMER_PAD(k) + 2)   /* a window holding a non-base byte */
#define BSL_KMER_VOCAB(k) (BSL_KMER_PAD(k) + 4) /* one more ID reserved: 4100 at k = 6 */

/* Enqueue the tokenization of a batch of sequences into padded rows of IDs.
 *   batch   >= 0 sequences.
 *   bases   device uint8[nbytes]: the sequences' text back to back (sequence
 *           bodies only: no FASTA headers; a line break inside a sequence is a
 *           non-base and makes its windows UNK).  Any alignment.
 *   nbytes  >= 0, the size of bases: no byte at or past it is read.
 *   starts  device int64[batch + 1]: sequence b is bytes [starts[b],
 *           starts[b+1]).  Values are clamped into [0, nbytes] on the device
 *           and a decreasing pair gives an empty sequence, so no value can send
 *           an access outside the buffer.
 *   k       1 .. 12 bases per window (6 on the page).
 *   n_out   >= 0 windows per output row (the dynamic ceiling of section 2,
 *           item 2: bsl_kmer_ceiling gives the longest window count rounded up
 *           to a multiple of 32, the n bsl_forward takes).
 *   ids     device int32[batch][n_out]: row b, column t holds window t's ID,
 *           BSL_KMER_PAD(k) for t >= ntok[b].  Every element is written.
 *   ntok    device int32[batch] or NULL: the windows written for sequence b,
 *           min(max(len_b - k + 1, 0), n_out) (the sequence lengths bsl_forward
 *           takes for the model's activations).
 *   stream  a hipStream_t, or NULL for the default stream.
 * batch == 0 is a no-op returning BSL_OK; with n_out == 0 only ntok is written
 * (ids may then be NULL).  BSL_E_INVALID for a NULL bases (when nbytes > 0),
 * starts or ids (when n_out > 0), negative sizes, k outside 1 .. 12, ids or ntok
 * overlapping the inputs or each other, or a launch of 2^31 or more
 * workgroups; BSL_E_DEVICE if the launch fails.  Nothing is written when an
 * argument error is returned. */
bsl_status bsl_kmer_tokenize(int32_t batch, const uint8_t *bases, int64_t nbytes,
                             const int64_t *starts, int32_t k, int32_t n_out, int32_t *ids,
                             int32_t *ntok, void *stream);

/* Host-side row width for bsl_kmer_tokenize: from host int64 starts[batch + 1]
 * (non-decreasing, starts[0] >= 0), *n_out = the longest sequence's window
 * count (len - k + 1, at least 0) rounded up to a multiple of 32.  No device
 * work.  BSL_E_INVALID for batch < 0, a NULL pointer, k outside 1 .. 12,
 * decreasing or negative offsets, or a result past 2^31 - 1. */
bsl_status bsl_kmer_ceiling(int32_t batch, const int64_t *starts, int32_t k, int32_t *n_out);

/* Debug validators for the device-side lengths and offsets the forward reads.
 * The forward itself clamps them (a bad value cannot cause an out-of-bounds
 * access, but it changes which rows are attended); these report them instead,
 * without a host round trip.  One small kernel is enqueued on `stream`; it
 * writes result[0] = the number of bad entries and result[1] = the index of
 * the first one, or -1 when all are valid.
 *   bsl_check_seqlens:    seqlens device int32[batch]; entry b is bad when
 *                         outside [0, n] (n as passed to bsl_forward).
 *   bsl_check_cu_seqlens: cu_seqlens device int32[batch + 1]; entry 0 is bad
 *                         when not 0, entry b > 0 when below entry b - 1 or
 *                         above tokens (as passed to bsl_forward_varlen).
 *   result                device int32[2], written in full; must not overlap
 *                         the checked array.
 * batch == 0 still writes {0, -1} (cu_seqlens then holds one entry).
 * BSL_E_INVALID for batch < 0, n or tokens < 0, a NULL pointer, or overlap;
 * BSL_E_DEVICE if the launch fails.  Nothing is written on an argument error.
 * The library allocates nothing and does not synchronise. */
bsl_status bsl_check_seqlens(int32_t batch, int32_t n, const int32_t *seqlens, int32_t *result,
                             void *stream);
bsl_status bsl_check_cu_seqlens(int32_t batch, int32_t tokens, const int32_t *cu_seqlens,
                                int32_t *result, void *stream);

/* Release a plan.  NULL is accepted and ignored.  Do not call while work
 * enqueued with the plan is being launched from another thread. */
bsl_status bsl_destroy(bsl_plan *plan);

/* Static text for a status code. */
const char *bsl_status_string(bsl_status status);

/* Text describing the last failing call on this host thread ("" if none). */
const char *bsl_last_error(void);

/* BSL_VERSION of the library actually loaded. */
int32_t bsl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSL_H */
