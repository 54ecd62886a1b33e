/*
 * lora_fused.h -- C ABI of the MI355X (gfx950) LoRA linear layer.
 *
 * The layer (page "LoRAFusion: Efficient LoRA Fine-Tuning for LLMs", juhe.plus
 * blog, section 2, formula Y = XW + alpha*(XA)B = XW + alpha*S*B; the
 * papers.chlience.com notes, section 3, write the intermediate as S = X^ A with
 * X^ the dropped-out input):
 *
 *     keep = [u16(seed, offset + i*k + j) >= T],  T = floor(p*65536 + 0.5)
 *     S    = s * (keep (.) X) A,                  s = 1/(1-p)
 *     Y    = X W + alpha * S B
 *
 * and its backward with W frozen (no dW; juhe.plus blog, section 2):
 *
 *     dB = alpha * S^T dY      dS = alpha * dY B^T
 *     dA = s * (keep (.) X)^T dS
 *     dX = dY W^T + s * keep (.) (dS A^T)
 *
 * The multi-adapter entry points apply the same maths per token segment with
 * that segment's adapter (papers.chlience.com notes, section 5
 * "FusedMultiLoRA": every input tile carries an adapter id with its rank,
 * scaling factor and dropout ratio, and backward routes gradients to each
 * adapter).
 *
 * Shapes and layouts (all row-major, contiguous):
 *   X  m x k bf16      W  k x n bf16 (frozen)   A  k x r bf16   B  r x n bf16
 *   Y  m x n bf16      dY m x n bf16            dX m x k bf16
 *   dA k x r bf16      dB r x n bf16            (gradients are overwritten)
 *   S  m x r_s fp32    (r_s = r for the single-adapter calls, r_max for the
 *                       multi-adapter calls; columns past a row's rank are 0)
 *   keep_bits          m rows x ceil(k/32) uint32 words; element (i, j) is bit
 *                      j % 32 of word i*ceil(k/32) + j/32; bits past k are 0.
 *
 * The dropout uniform u16(seed, c) of element counter c is 16-bit half
 * (c mod 8) -- low half of the lowest word first -- of the 128-bit output of
 * Philox4x32-10 (Salmon et al., SC'11) under key (seed_lo, seed_hi) and
 * counter (b_lo, b_hi, 0, 0), b = c >> 3.  Counters use the global row index
 * of the call plus `offset`, so a call on rows [r0, r1) of a larger batch with
 * offset + r0*k reproduces those rows exactly.
 *
 * Ownership: every pointer is a caller-owned device buffer (except the few
 * host-side helpers marked "host").  The library never allocates, frees or
 * keeps a pointer past the call.  S and keep_bits are written by the forward
 * call and must stay alive and unchanged until the matching backward call.
 * Scratch space is the caller-provided `workspace`, sized by the matching
 * *_workspace_size() query; it holds nothing between calls.
 *
 * Execution: every entry point only enqueues kernels on `stream` (0 = the
 * default stream) and returns; there is no host synchronisation.  Results
 * are deterministic: the same inputs give bitwise-identical outputs.
 *
 * Errors: arguments are checked on the host before anything is enqueued; on
 * failure nothing is enqueued and a negative lora_status is returned, with
 * detail in lora_last_error_message() (thread-local).  Checks: non-NULL
 * pointers; 16-byte alignment of X, W, Y, dY, dX and the workspace; 4-byte
 * alignment of S and keep_bits; 0 <= m < 2^31; 0 < k, n < 2^31 with
 * k % 8 == 0 and n % 8 == 0; 1 <= r <= 256; 0 <= p < 1; offset % 8 == 0;
 * workspace large enough (LORA_ERR_INVALID_ARG / LORA_ERR_WORKSPACE).  The
 * layer calls (forward and backward) return LORA_ERR_UNSUPPORTED when B
 * (r or r_max by n bf16) or A (k by r or r_max bf16) exceeds 2 GiB.  When m == 0 the m-sized buffers (X, Y, S,
 * keep_bits, dY, dX) may be NULL.  The multi-adapter tables live in device memory and
 * are never read on the host: an invalid table (segments not ordered, not
 * covering [0, m), adapter index out of range, adapter rank > r_max) gives
 * undefined values in the affected rows but never an out-of-bounds access;
 * multi_lora_check_segments() validates a host copy for callers who want it.
 */
#ifndef LORA_FUSED_H
#define LORA_FUSED_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LORA_OK = 0,
    LORA_ERR_INVALID_ARG = -1,
    LORA_ERR_UNSUPPORTED = -2,
    LORA_ERR_WORKSPACE = -3,
    LORA_ERR_HIP = -4
} lora_status;

/* One adapter of the multi-adapter calls.  An array of these lives in device
 * memory (papers.chlience.com notes, section 5: the kernel looks up each
 * tile's adapter A, B, rank, scaling factor and dropout ratio from a table).
 * A: k x r, B: r x n, dA: k x r, dB: r x n, all bf16 device pointers.
 * dA/dB are only used by multi_lora_linear_bwd (may be NULL for forward). */
typedef struct {
    const void *A;
    const void *B;
    void *dA;
    void *dB;
    int32_t r;
    float alpha;
    float p;
    int32_t reserved;
} lora_adapter;

/* ---- single adapter (FusedLoRA) ---------------------------------------- */

/* Bytes of workspace lora_linear_fwd needs for this shape (may be 0). */
size_t lora_linear_fwd_workspace_size(int64_t m, int64_t k, int64_t n, int32_t r);

/* Forward: writes Y, S (m x r fp32) and keep_bits.  keep_bits may be NULL
 * only when p == 0 (then every element is kept and no mask is stored).
 * Kernel split (juhe.plus blog, section 4.1, forward items 1 and 2): one
 * kernel streams X once, generating the mask and S = s*(keep (.) X)A; one MFMA
 * GEMM computes XW and adds alpha*S*B before the single write of Y. */
lora_status lora_linear_fwd(const void *X, const void *W, const void *A, const void *B,
                            int64_t m, int64_t k, int64_t n, int32_t r, float alpha, float p,
                            uint64_t seed, uint64_t offset,
                            void *Y, float *S, uint32_t *keep_bits,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Forward at p = 0 in the concatenated form (FALQON notes, section 5.2, the
 * adapter's down-projection A stacked beside the frozen W as one operand; the
 * recompute-versus-split question of the juhe.plus blog, section 4.1):
 * Y = X W + alpha (X A) B and S = X A (fp32, m x r, row-major) in one GEMM
 * launch.  Each 256 x 256 output tile forms, inside its own K loop, the
 * 256 x r block of S its rows need (A's rows ride along with W's in every
 * stage; about 6% more matrix-core work), then adds alpha S B before the
 * single write of Y: no separate pass over X and no second pass over Y.  The
 * tiles of the first column block also write S, which lora_linear_bwd takes
 * with keep_bits = NULL and p = 0.  Needs no workspace.  r must be 8 or 16
 * and A, B and S 16-byte aligned (else LORA_ERR_UNSUPPORTED; the general
 * forward with p = 0 covers every other case).  Shapes and the other
 * pointers as for lora_linear_fwd; m == 0 returns at once. */
lora_status lora_linear_fwd_concat(const void *X, const void *W, const void *A, const void *B,
                                   int64_t m, int64_t k, int64_t n, int32_t r, float alpha,
                                   void *Y, float *S, hipStream_t stream);

/* Bytes of workspace lora_linear_bwd needs for this shape. */
size_t lora_linear_bwd_workspace_size(int64_t m, int64_t k, int64_t n, int32_t r);

/* Backward: given dY and the forward's S and keep_bits (NULL iff p == 0),
 * writes dX (m x k), dA (k x r) and dB (r x n).  Kernel split (juhe.plus
 * blog, section 4.1, backward items 3 and 5): one pass over dY yields dS and
 * dB; one pass over X and the mask yields dA; an MFMA GEMM computes dY W^T
 * and adds the masked s*(dS A^T) before the single write of dX.  m == 0
 * writes zero dA and dB.  dX may be NULL: the input gradient is then not
 * computed (its GEMM is skipped), e.g. for a layer whose input needs none. */
lora_status lora_linear_bwd(const void *dY, const void *X, const void *W, const void *A,
                            const void *B, const float *S, const uint32_t *keep_bits,
                            int64_t m, int64_t k, int64_t n, int32_t r, float alpha, float p,
                            void *dX, void *dA, void *dB,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/* The same backward for callers that cannot allocate device memory (code
 * under graph capture, tight training loops, harnesses that forbid
 * allocation): it takes no workspace and uses a scratch array of
 * lora_linear_bwd_noalloc_max_scratch() bytes (64 MiB) that the library holds
 * in static device memory, one per GPU, until the process ends.  It never
 * allocates or frees.  The scratch of the current device is used (the stream
 * must belong to it).  A shape whose workspace (lora_linear_bwd_workspace_size)
 * exceeds the scratch returns LORA_ERR_UNSUPPORTED before anything is
 * enqueued.  Every call on one GPU shares that GPU's scratch: calls that may
 * overlap in time on one GPU (different streams, different host threads
 * without ordering) race and must not be made; calls in one stream's order
 * are safe.  Outputs, checks and errors are otherwise those of
 * lora_linear_bwd, whose kernels it runs. */
size_t lora_linear_bwd_noalloc_max_scratch(void);
lora_status lora_linear_bwd_noalloc(const void *dY, const void *X, const void *W, const void *A,
                                    const void *B, const float *S, const uint32_t *keep_bits,
                                    int64_t m, int64_t k, int64_t n, int32_t r, float alpha, float p,
                                    void *dX, void *dA, void *dB, hipStream_t stream);

/* ---- mixed-adapter batch (FusedMultiLoRA) ------------------------------- */

/* Segments: rows [seg_off[s], seg_off[s+1]) use adapter seg_adapter[s];
 * seg_off (int64, num_segments+1 entries) and seg_adapter (int32) are device
 * arrays; segments must be ordered, contiguous and cover [0, m); empty
 * segments are allowed.  r_max >= every adapter's r is the row stride of S. */
size_t multi_lora_fwd_workspace_size(int64_t m, int64_t k, int64_t n, int32_t r_max,
                                     int32_t num_adapters, int32_t num_segments);

/* Forward for a mixed-adapter batch: Y (m x n), S (m x r_max; row i holds
 * its adapter's S, zero past that rank) and keep_bits (required). */
lora_status multi_lora_linear_fwd(const void *X, const void *W, const lora_adapter *adapters,
                                  int32_t num_adapters, const int64_t *seg_off,
                                  const int32_t *seg_adapter, int32_t num_segments,
                                  int64_t m, int64_t k, int64_t n, int32_t r_max,
                                  uint64_t seed, uint64_t offset,
                                  void *Y, float *S, uint32_t *keep_bits,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

size_t multi_lora_bwd_workspace_size(int64_t m, int64_t k, int64_t n, int32_t r_max,
                                     int32_t num_adapters, int32_t num_segments);

/* Backward for a mixed-adapter batch: dX, and every adapter's dA and dB
 * (through the pointers in the adapter table; summed over all of that
 * adapter's rows; zero for adapters with no rows).  dX may be NULL: the input
 * gradient is then not computed. */
lora_status multi_lora_linear_bwd(const void *dY, const void *X, const void *W,
                                  const lora_adapter *adapters, int32_t num_adapters,
                                  const int64_t *seg_off, const int32_t *seg_adapter,
                                  int32_t num_segments, const float *S,
                                  const uint32_t *keep_bits, int64_t m, int64_t k, int64_t n,
                                  int32_t r_max, void *dX,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Host: validate host copies of a segment table (0 if valid, else
 * LORA_ERR_INVALID_ARG with a message). */
lora_status multi_lora_check_segments(const int64_t *seg_off_host, const int32_t *seg_adapter_host,
                                      int32_t num_segments, int64_t m,
                                      const int32_t *adapter_r_host, int32_t num_adapters,
                                      int32_t r_max);

/* ---- mixed-adapter batching (host) ---------------------------------------
 * The step upstream of the mixed-adapter entry points: a scheduler packs the
 * samples of several adapters' global batches into microbatches of bounded
 * token count, and each microbatch's rows, grouped by adapter, become one
 * segment table (papers.chlience.com notes on LoRAFusion, section 4
 * "Multi-LoRA scheduler"; juhe.plus blog, section 4.2).  All arrays are host
 * memory owned by the caller; nothing is retained; no device work. */

/* Greedy packing of num_samples samples (lengths[i] tokens, 1 <= lengths[i]
 * <= capacity) into microbatches of at most `capacity` tokens: first-fit
 * decreasing -- samples longest first (equal lengths in index order), each
 * into the lowest-numbered microbatch with room, else into a new one (the
 * pages' greedy fallback of their MILP packer).  Writes mb_of_sample[i] (the
 * microbatch of sample i, numbered in opening order) and *num_microbatches.
 * LORA_ERR_INVALID_ARG for a length outside [1, capacity], capacity < 1,
 * num_samples < 0 or a NULL array. */
lora_status lora_pack_greedy(const int32_t *lengths, int32_t num_samples, int64_t capacity,
                             int32_t *mb_of_sample, int32_t *num_microbatches);

/* The segment table of microbatch `mb`: its samples ordered by adapter
 * (increasing id; one adapter's samples in increasing index), one segment per
 * adapter present.  Writes sample_order[0 .. *num_members) (sample indices in
 * row order; room for num_samples), seg_off[0 .. *num_segments] (token
 * offsets; room for num_adapters + 1; seg_off[*num_segments] is the
 * microbatch's row count m) and seg_adapter[0 .. *num_segments) (room for
 * num_adapters).  An empty microbatch gives zero segments and seg_off[0] = 0.
 * LORA_ERR_INVALID_ARG for an adapter id outside [0, num_adapters), a length
 * below 1 among the members, or a NULL array. */
lora_status lora_microbatch_segments(const int32_t *lengths, const int32_t *adapter_of_sample,
                                     const int32_t *mb_of_sample, int32_t num_samples,
                                     int32_t num_adapters, int32_t mb, int32_t *sample_order,
                                     int32_t *num_members, int64_t *seg_off,
                                     int32_t *seg_adapter, int32_t *num_segments);

/* Pipeline dependency check ("bubble lemma", same sections): with `stages`
 * pipeline stages, sample i sits in microbatch mb_of_sample[i] and belongs to
 * global batch batch_of_sample[i] of adapter adapter_of_sample[i].  For every
 * adapter and each of its global batches that has a later one with samples,
 * the earliest microbatch of that next batch must be at least the latest
 * microbatch of this batch plus stages - 1.  *violations = the number of
 * (adapter, batch) pairs that break it (0: the order is valid).
 * LORA_ERR_INVALID_ARG for stages < 1, an adapter id outside
 * [0, num_adapters), a negative index or a NULL array. */
lora_status lora_check_bubble_lemma(const int32_t *mb_of_sample, const int32_t *adapter_of_sample,
                                    const int32_t *batch_of_sample, int32_t num_samples,
                                    int32_t num_adapters, int32_t stages, int64_t *violations);

/* ---- DoRA norm -----------------------------------------------------------
 * DoRA rescales each output feature of the adapted weight by a learned
 * magnitude over its norm.  This computes that norm for every output feature
 * (a column here, since the layer is X W with W k x n):
 *   norm[j] = || W[:, j] + alpha * (A B)[:, j] ||_2
 * without storing the dense k x n product (page on the factored DoRA norm,
 * "core method": the norm of W + sBA per output feature, s the LoRA scale).
 * W (k x n), A (k x r) and B (r x n) are bf16 row-major device buffers,
 * 16-byte aligned; norm is n fp32 (4-byte aligned).  Sums are fp32 and
 * deterministic.  Requires 1 <= r <= 256, n % 8 == 0; the workspace holds
 * per-split partial sums (lora_dora_norm_workspace_size bytes, 16-byte
 * aligned).  LORA_ERR_UNSUPPORTED when A or B (with 32 spare rows) exceeds
 * 2 GiB. */
size_t lora_dora_norm_workspace_size(int64_t k, int64_t n, int32_t r);
lora_status lora_dora_norm(const void *W, const void *A, const void *B, int64_t k, int64_t n,
                           int32_t r, float alpha, float *norm, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* ---- pieces exposed for testing and as the frozen-layer baseline -------- */

/* The dropout mask alone (same bits the forward stores). */
lora_status lora_dropout_mask(uint64_t seed, uint64_t offset, int64_t m, int64_t k, float p,
                              uint32_t *keep_bits, hipStream_t stream);

/* Frozen linear layer, forward Y = X W and backward dX = dY W^T, on the same
 * MFMA GEMM as the LoRA path (the frozen layer the pages compare against:
 * papers.chlience.com notes, "Result 1: LoRA overhead profiling"). */
lora_status lora_frozen_fwd(const void *X, const void *W, int64_t m, int64_t k, int64_t n,
                            void *Y, hipStream_t stream);
lora_status lora_frozen_bwd(const void *dY, const void *W, int64_t m, int64_t k, int64_t n,
                            void *dX, hipStream_t stream);

/* ---- kernel timing (tracing) --------------------------------------------
 * When enabled, every kernel the library launches is bracketed by a pair of
 * HIP events recorded on the launch stream.  lora_profiling_query()
 * synchronises those events and returns, for kernels whose name contains
 * `name_substring`, the number of launches and their summed duration in
 * milliseconds since the last reset.  Event pairs come from a pool created by
 * lora_profiling_enable(1) (capacity events per kernel launch slot); launches
 * beyond the capacity are not timed. */
lora_status lora_profiling_enable(int32_t enable, int32_t capacity);
lora_status lora_profiling_reset(void);
lora_status lora_profiling_query(const char *name_substring, int64_t *launches, double *total_ms);

/* ---- status ------------------------------------------------------------ */
const char *lora_status_string(lora_status s);
const char *lora_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* LORA_FUSED_H */
