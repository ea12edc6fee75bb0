/*
 * pairattn.h -- C ABI of the MI355X (gfx950) pair-biased attention library.
 *
 * Three operations on the pair representation Z[I][I][c_z] of an
 * AlphaFold2-style trunk (see the page sources cited at each entry point):
 *   - triangle attention around the starting node   (orientation START)
 *   - triangle attention around the ending node     (orientation END)
 *   - MSA row attention with a bias from the pair tensor
 * plus the two halves of the starting-node call for a block of query rows
 * (pair bias from the whole Z, then attention for the rows of one block).
 *
 * Every operation computes, for its rows, gated multi-head attention with an
 * additive pair bias (c input channels, H heads of width d):
 *   x^   = LayerNorm(x) = (x - mean) / sqrt(var + eps) * gamma + beta
 *          (mean and biased variance over the channel axis)
 *   q,k,v= x^ W_q, x^ W_k, x^ W_v;   g = sigmoid(x^ W_g + b_g)
 *   B    = LayerNorm(z) W_b          (one scalar per head and pair)
 *   logit= q.k / sqrt(d) + bias[query][key], masked keys get weight 0
 *   o    = softmax-weighted sum of v (o = 0 if every key is masked)
 *   out  = (g * concat_h o_h) W_o + b_o      (the update; no residual add)
 * START (row i, query j, key k):  bias = B[j][k], key kept iff mask[i][k]
 * END   (column j, query i, key k): bias = B[k][i], key kept iff mask[k][j]
 *
 * Conventions shared by every entry point
 *   - All tensor arguments are DEVICE pointers on the current HIP device,
 *     16-byte aligned, densely packed, row-major with the last index fastest.
 *   - Element type of activations, weights and outputs is params->dtype:
 *     PAIRATTN_F32 (float) or PAIRATTN_BF16 (bfloat16 bits, uint16).  Masks
 *     are uint8 (nonzero = keep) and may be NULL (keep everything).  Pair
 *     biases handed across the boundary are float32 [H][I][I] indexed
 *     [h][query][key] in natural-log units (the value added to q.k/sqrt(d)).
 *   - The caller owns every buffer, including the workspace, whose size is
 *     given by the matching *_workspace_bytes call.  The library allocates
 *     no memory and keeps no state other than a thread-local error string
 *     and a per-device architecture check.
 *   - Outputs must not alias inputs or the workspace.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the null stream).  The return value reports argument
 *     validation and launch errors; a device fault surfaces at the caller's
 *     next synchronisation.
 *   - Arithmetic.  PAIRATTN_BF16: matrix products take fp16 operands (11
 *     significant bits) with fp32 accumulation; LayerNorm, the softmax and
 *     all sums run in fp32.  PAIRATTN_F32: fp32-accurate; every matrix
 *     product is formed from fp16 pairs (hi = fp16(x), lo = fp16(x - hi);
 *     hi.hi + hi.lo + lo.hi on the fp16 matrix cores, fp32 accumulation), so
 *     each product carries a relative error below 2^-21.  On both paths
 *     intermediate values (normalised activations, gamma o W, q, k, v, the
 *     pair bias in log2 units, the softmax weights, the gated o) must stay
 *     below 65504 in magnitude, the fp16 range; inputs in the usual ranges of
 *     these models do.  Beyond it, PAIRATTN_BF16 saturates them at +-65504:
 *     the output stays finite and the same on every call, but it is no
 *     longer the method's result, and the call still returns PAIRATTN_OK.
 *     On PAIRATTN_F32 they overflow to infinity.
 *   - Supported shapes: d = 32; H in {4, 8}; c, c_m, c_z in {64, 128, 256};
 *     any I >= 1, S >= 1, R >= 1.  Anything else returns
 *     PAIRATTN_ERR_UNSUPPORTED; there is no fallback path.
 *   - Only gfx950 devices are accepted (PAIRATTN_ERR_DEVICE otherwise).
 */
#ifndef PAIRATTN_H
#define PAIRATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pairattn_status {
  PAIRATTN_OK = 0,
  PAIRATTN_ERR_ARG = 1,          /* null pointer, bad size, misalignment, bad enum */
  PAIRATTN_ERR_UNSUPPORTED = 2,  /* valid request outside the supported shapes */
  PAIRATTN_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  PAIRATTN_ERR_DEVICE = 4,       /* current device is not gfx950 / no device */
  PAIRATTN_ERR_HIP = 5           /* a HIP runtime call or kernel launch failed */
} pairattn_status;

enum { PAIRATTN_START = 0, PAIRATTN_END = 1 };
enum { PAIRATTN_F32 = 0, PAIRATTN_BF16 = 1 };

/* Weights of one attention module.  A host struct of DEVICE pointers; it is
 * read during the call and not retained.  c = input/output channels of the
 * attended tensor, cz = channels of the pair tensor that feeds the bias
 * (cz = c for triangle attention).  Linear maps act as y = x @ W. */
typedef struct pairattn_params {
  int32_t dtype;               /* PAIRATTN_F32 or PAIRATTN_BF16 */
  const void *ln_gamma;        /* [c]     LayerNorm scale of the attended tensor */
  const void *ln_beta;         /* [c]     LayerNorm shift */
  const void *w_q;             /* [c][H*d] */
  const void *w_k;             /* [c][H*d] */
  const void *w_v;             /* [c][H*d] */
  const void *w_g;             /* [c][H*d] gate pre-activation */
  const void *b_g;             /* [H*d]   gate bias, NULL = 0 */
  const void *w_b;             /* [cz][H] pair-bias projection */
  const void *w_o;             /* [H*d][c] output projection */
  const void *b_o;             /* [c]     output bias, NULL = 0 */
  const void *lnz_gamma;       /* [cz]    MSA only: LayerNorm of the pair input */
  const void *lnz_beta;        /* [cz]    MSA only */
  float ln_eps;                /* LayerNorm epsilon (e.g. 1e-5), must be >= 0 */
  void *workspace;             /* device scratch owned by the caller */
  size_t workspace_bytes;      /* its size in bytes */
} pairattn_params;

/* Workspace sizes (bytes).  Return 0 for unsupported or invalid shapes. */
size_t pairattn_tri_workspace_bytes(int64_t I, int64_t c_z, int64_t H, int64_t d, int32_t dtype);
size_t pairattn_msa_workspace_bytes(int64_t S, int64_t I, int64_t c_m, int64_t c_z, int64_t H,
                                    int64_t d, int32_t dtype);
size_t pairattn_rows_workspace_bytes(int64_t R, int64_t I, int64_t c_z, int64_t H, int64_t d,
                                     int32_t dtype);

/* Triangle attention around the starting (orientation = PAIRATTN_START) or
 * ending (PAIRATTN_END) node of Z.
 *   z    [I][I][c_z]   pair representation
 *   mask [I][I] uint8 or NULL; START keeps key k of row i iff mask[i][k],
 *        END keeps key k of column j iff mask[k][j]
 *   out  [I][I][c_z]   attention update
 * Source: triangle self-attention over the pair representation in the
 * Evoformer (Intel AlphaFold2 page, DL-inference bullet; Dell XE8545 page,
 * EvoFormer paragraph); the bias is indexed by (query, key) only, shared by
 * every row (Intel page, Step 4 code example, nonbatched_bias); queries run
 * along one axis and keys/values along the other without forming the I x I
 * score matrix (Design-CP page, Metodologia 1). */
int pairattn_tri_fwd(const void *z, const uint8_t *mask, const pairattn_params *p, void *out,
                     int64_t I, int64_t c_z, int64_t H, int64_t d, int32_t orientation,
                     void *stream);

/* Allocation-free form of pairattn_tri_fwd, for callers that cannot allocate
 * device memory or hand over a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, layout,
 * arithmetic and result as pairattn_tri_fwd (the same kernels run); the
 * workspace and workspace_bytes fields of *p are ignored.  Its workspace is
 * a static device array of PAIRATTN_NOALLOC_SCRATCH_BYTES per GPU, held from
 * the library's first use on that GPU until the process ends.  Problems whose
 * pairattn_tri_workspace_bytes exceeds it return PAIRATTN_ERR_UNSUPPORTED
 * before any device call (I <= 507 for bf16 at H = 4, I <= 352 for fp32 at
 * H = 4 or bf16 at H = 8, I <= 252 for fp32 at H = 8).  Nothing in the
 * array needs to start at zero: each call overwrites what it reads.  Every
 * call on one GPU shares that GPU's array, so calls that overlap on one GPU
 * (other streams, other host threads) race; serialise them.  Timing marks
 * (pairattn_timing_enable) are not recorded for this call. */
#define PAIRATTN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int pairattn_tri_fwd_noalloc(const void *z, const uint8_t *mask, const pairattn_params *p,
                             void *out, int64_t I, int64_t c_z, int64_t H, int64_t d,
                             int32_t orientation, void *stream);

/* MSA row attention with pair bias.
 *   m    [S][I][c_m] MSA representation; z [I][I][c_z] pair representation
 *   mask [S][I] uint8 or NULL (key j of sequence s kept iff mask[s][j])
 *   out  [S][I][c_m]
 * bias[h][i][j] = LayerNorm_z(z[i][j]) . w_b[:, h], shared by all sequences.
 * Source: the MSA and pair tracks influence each other through attention
 * (Intel AlphaFold2 page, DL-inference bullet and the dual-track design
 * point); bias from tensor products added to the logits (Intel page,
 * Step 4). */
int pairattn_msa_row_fwd(const void *m, const void *z, const uint8_t *mask,
                         const pairattn_params *p, void *out, int64_t S, int64_t I,
                         int64_t c_m, int64_t c_z, int64_t H, int64_t d, void *stream);

/* Pair bias of triangle attention for the whole Z, in the [h][query][key]
 * layout that pairattn_tri_rows_fwd takes:
 *   START: bias[h][j][k] = LayerNorm(z[j][k]) . w_b[:, h]
 *   END:   bias[h][i][k] = LayerNorm(z[k][i]) . w_b[:, h]
 * Uses ln_gamma/ln_beta/w_b/ln_eps of p; no workspace.  bias is [H][I][I]
 * float32.  Source: Intel page, Step 4 (bias from tensor products). */
int pairattn_tri_bias(const void *z, const pairattn_params *p, float *bias, int64_t I, int64_t c_z,
                      int64_t H, int32_t orientation, void *stream);

/* Starting-node triangle attention for a block of R query rows with full-
 * length keys: one device's share when query rows are split across devices
 * and keys/values stay whole (Design-CP page, Metodologia 1, 1D row sharding:
 * self-attention recast as cross-attention), or one slice of the Intel
 * page's row slicing (Step 4).
 *   z_rows    [R][I][c_z] rows of Z
 *   bias      [H][I][I] float32 from pairattn_tri_bias over the whole Z
 *   mask_rows [R][I] uint8 or NULL
 *   out_rows  [R][I][c_z] */
int pairattn_tri_rows_fwd(const void *z_rows, const float *bias, const uint8_t *mask_rows,
                          const pairattn_params *p, void *out_rows, int64_t R, int64_t I,
                          int64_t c_z, int64_t H, int64_t d, void *stream);

/* Triangle attention of the whole Z in blocks: the low-memory form of
 * pairattn_tri_fwd, for I far above what the one-pass workspace allows.
 * The pair bias of the whole Z is computed once into the workspace; then
 * `block` rows (START) or columns (END) at a time are projected and attend
 * over all keys.  Same arguments and result as pairattn_tri_fwd (bit for bit
 * when block is even: the attention kernels pair adjacent rows), with a
 * workspace that grows with block * I instead of I * I (see
 * pairattn_tri_chunked_workspace_bytes).  block >= 1; block >= I is one
 * block.  Timing stages: "pair_bias", "blocks".
 * Source: the memory wall of the pair representation and the remedy of
 * evaluating attention in slices of rows with the bias computed once
 * (Intel page, Step 4, tensor slicing of the attention module; Design-CP
 * page, low-memory mode in its implementation details). */
size_t pairattn_tri_chunked_workspace_bytes(int64_t I, int64_t c_z, int64_t H, int64_t d,
                                            int32_t dtype, int64_t block);
int pairattn_tri_chunked_fwd(const void *z, const uint8_t *mask, const pairattn_params *p,
                             void *out, int64_t I, int64_t c_z, int64_t H, int64_t d,
                             int32_t orientation, int64_t block, void *stream);

/* One step of ring attention over a 2D device grid: starting-node attention
 * of the query pairs a device holds against one shard of key pairs of the
 * same rows, kept as a per-head output and its log-sum-exp so that shards
 * combine exactly (Design-CP page, Metodologia 1, 2D grid sharding: queries
 * split along rows, keys/values along columns and passed around a ring,
 * attention never formed as an I x I matrix).  Both paths: q_pairs and
 * kv_pairs in params->dtype (fp32, or bf16 with the bf16 path's fp16
 * operands); o, lse and bias are float either way.
 *   q_pairs  [R][Jq][c_z]  the device's query pairs (rows r, their columns)
 *   kv_pairs [R][Kn][c_z]  one shard of key pairs of the same rows
 *   bias     [H][Jq][Kn]   float, natural-log units, for these queries/keys
 *   mask     [R][Kn] uint8 or NULL (key kept iff nonzero)
 *   o        [R][Jq][H*d]  float: per head, the softmax-weighted sum of v
 *                          over the shard's kept keys (0 with none)
 *   lse      [R][H][Jq]    float: ln sum_k exp(logit_k) over those keys
 *                          (-inf with none)
 * accumulate holds bits: without PAIRATTN_PARTIAL_MERGE the call writes o
 * and lse; with it the call merges this shard into the o and lse already
 * there: lse' = ln(e^lse + e^lse_s), o' = e^(lse - lse') o + e^(lse_s -
 * lse') o_s.  PAIRATTN_PARTIAL_Q_READY states that the workspace holds what
 * the previous call with this workspace left: the packed weights and the
 * projected q of the same q_pairs, params, R, Jq, c_z, H and d (the caller
 * keeps them unchanged in between, e.g. along the shards of one ring step);
 * neither is formed again.  Other bits: PAIRATTN_ERR_ARG.  kv_pairs may be
 * q_pairs itself (Kn = Jq: the device's own shard); its k and v (and q
 * unless ready) then come from one pass over it.  Workspace:
 * pairattn_tri_partial_workspace_bytes (the q plane's place in it does not
 * depend on Kn, so shards of any size share it). */
#define PAIRATTN_PARTIAL_MERGE 1
#define PAIRATTN_PARTIAL_Q_READY 2
size_t pairattn_tri_partial_workspace_bytes(int64_t R, int64_t Jq, int64_t Kn, int64_t c_z,
                                            int64_t H, int64_t d, int32_t dtype);
int pairattn_tri_partial_fwd(const void *q_pairs, const void *kv_pairs, const float *bias,
                             const uint8_t *mask, const pairattn_params *p, float *o, float *lse,
                             int32_t accumulate, int64_t R, int64_t Jq, int64_t Kn, int64_t c_z,
                             int64_t H, int64_t d, void *stream);

/* The end of the ring: out[r][j] = (sigmoid(LN(q_pairs) W_g + b_g) * o) W_o
 * + b_o for the assembled o of pairattn_tri_partial_fwd.  out [R][Jq][c_z]
 * in params->dtype.  Workspace: pairattn_tri_partial_finish_workspace_bytes. */
size_t pairattn_tri_partial_finish_workspace_bytes(int64_t R, int64_t Jq, int64_t c_z, int64_t H,
                                                   int64_t d, int32_t dtype);
int pairattn_tri_partial_finish(const void *q_pairs, const float *o, const pairattn_params *p,
                                void *out, int64_t R, int64_t Jq, int64_t c_z, int64_t H, int64_t d,
                                void *stream);

/* Host-only argument checks with exactly the rules of the entry points
 * above (no HIP call, no device needed).  Return the status the entry point
 * would return before touching the device. */
int pairattn_validate_tri_partial(const void *q_pairs, const void *kv_pairs, const float *bias,
                                  const uint8_t *mask, const pairattn_params *p, const float *o,
                                  const float *lse, int64_t R, int64_t Jq, int64_t Kn, int64_t c_z,
                                  int64_t H, int64_t d);
int pairattn_validate_tri_partial_finish(const void *q_pairs, const float *o,
                                         const pairattn_params *p, const void *out, int64_t R,
                                         int64_t Jq, int64_t c_z, int64_t H, int64_t d);
int pairattn_validate_tri_chunked(const void *z, const uint8_t *mask, const pairattn_params *p,
                                  const void *out, int64_t I, int64_t c_z, int64_t H, int64_t d,
                                  int32_t orientation, int64_t block);
int pairattn_validate_tri(const void *z, const uint8_t *mask, const pairattn_params *p,
                          const void *out, int64_t I, int64_t c_z, int64_t H, int64_t d,
                          int32_t orientation);
int pairattn_validate_msa(const void *m, const void *z, const uint8_t *mask,
                          const pairattn_params *p, const void *out, int64_t S, int64_t I,
                          int64_t c_m, int64_t c_z, int64_t H, int64_t d);
int pairattn_validate_rows(const void *z_rows, const float *bias, const uint8_t *mask_rows,
                           const pairattn_params *p, const void *out_rows, int64_t R, int64_t I,
                           int64_t c_z, int64_t H, int64_t d);

/* Per-kernel timing of the calling thread's launches (instrumentation).
 * pairattn_timing_enable(1) makes every later entry point on this thread
 * record HIP events on its stream at its start and after each kernel it
 * launches, with no host wait (a pool of 1024 events per thread, created by
 * the enabling call; marks beyond it are dropped until the next read).  It
 * returns the previous setting, or -PAIRATTN_ERR_HIP if the events could not
 * be created.  pairattn_timing_read waits for the last event recorded and
 * writes up to `cap` stage durations in ms, of every call since the last
 * read, in launch order ("pack", "projection", "pair_bias", "mask_bits",
 * "attention", ...), with their static names; it returns the number
 * written, 0 when timing is off or nothing was recorded, or
 * -PAIRATTN_ERR_HIP on a HIP failure.  `ms` or `names` may be NULL. */
int pairattn_timing_enable(int enable);
int pairattn_timing_read(float *ms, const char **names, int cap);

/* Calibration of the softmax's second roof (instrumentation, not part of
 * the method): one launch on `stream` of 2048 x 256 threads, each running 8
 * independent chains of `iters` exp2 instructions (x <- exp2(-x)), so that
 * the issue rate of exp2 bounds it; each thread writes one float (a value
 * that keeps its chains live) to out[524288] (device, 16-byte aligned).
 * One launch evaluates 4194304 * iters exp2 per lane; timed with events on
 * `stream`, it gives this device's exp2 throughput.  iters in [1, 2^24]. */
int pairattn_calibrate_exp2(float *out, int64_t iters, void *stream);

/* Index checks of the debug build (libpairattn_debug.so, built with
 * -DPA_DEBUG; not part of the method).  There every kernel checks the
 * indices it computes (copy sources and LDS stages of the attention, its
 * q / gate tiles and staged output, the projection's stores and operand
 * copies, the keep-bits words) against the extents its shape arguments give,
 * and a failed check sets a bit in a device flag word instead of trapping.
 * This call waits for the device, then writes the OR of those bits since the
 * last call to *flags (bit 0 K/V copy source, 1 bias copy source, 2 LDS
 * stage, 3 q / gate tile, 4 projection store, 5 pair-bias store, 6 keep-bits
 * word, 7 staged output tile, 8 projection operand slice) and clears them; *checking is 1 in the debug build.
 * The release build writes 0 to both.  Either pointer may be NULL.  Returns
 * PAIRATTN_OK or PAIRATTN_ERR_HIP. */
int pairattn_debug_status(uint32_t *flags, int32_t *checking);

/* Static description of a status code. */
const char *pairattn_status_string(int status);
/* Detail of the last failure on the calling thread ("" if none). */
const char *pairattn_last_error(void);
/* Library version as major*10000 + minor*100 + patch. */
int pairattn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* PAIRATTN_H */
