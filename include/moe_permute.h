/*
 * moe_permute.h -- C ABI of the MI355X (gfx950) MoE token permute / unpermute
 * library, libmoe_permute.so.
 *
 * What is computed (the three pages on the subject):
 *   - vLLM PR #14568, "permute/unpermute kernel for moe optimization", PR
 *     description: permute expands every token into its topk copies and
 *     orders the copies so that the tokens of each expert are contiguous, as
 *     the grouped GEMM wants them; unpermute folds the expanded grouped-GEMM
 *     output back into one row per token, weighting each copy by its
 *     topk_weight.
 *   - prhub summary of vLLM PR #43014 (preallocated MoE permute buffers),
 *     section "key code snippets", MoEPermuteScratch: the buffers and their
 *     types -- expert_first_token_offset int64 [num_experts + 1];
 *     permuted_idx and inv_permuted_idx int32 [num_tokens * topk];
 *     permuted_hidden_states [num_tokens * topk, hidden_size] of the hidden
 *     type; a sort workspace whose size is queried up front; expanded rows
 *     numbered by an arange viewed [num_tokens, topk].
 *   - same summary, sections "implementation breakdown" and "review
 *     highlights": callers preallocate every buffer once and reuse it; the
 *     library must write into the caller's buffers (never a hidden copy); the
 *     size query must be safe to call anywhere.
 *
 * Definitions used throughout (N = num_tokens, K = topk, E = num_experts):
 *   expanded row     r = t*K + k  holds topk_ids[t][k]           (0 <= r < N*K)
 *   offsets          expert_first_token_offset[e] = number of expanded rows
 *                    whose expert is < e; entry E equals N*K
 *   order            rows of one expert keep ascending r (a stable sort)
 *   permuted_idx[j]  = r, the expanded row placed at permuted position j
 *   inv_permuted_idx[r] = j, so inv[perm[j]] = j and perm[inv[r]] = r
 *   permute rows     permuted_hidden_states[j] = hidden_states[permuted_idx[j] / K]
 *   unpermute        output[t] = sum over k = 0..K-1, ascending, of
 *                    topk_weights[t][k] * expanded_output[inv_permuted_idx[t*K+k]]
 *                    accumulated in fp32 and rounded once (round to nearest even)
 *
 * Conventions for every entry point:
 *   - Stateless and reentrant.  No call allocates memory, frees memory,
 *     memsets, synchronises the host or copies host<->device.  Work is
 *     enqueued on `stream` (a hipStream_t; NULL is the null stream) and the
 *     call returns after enqueueing.  Buffers must stay valid until the
 *     stream reaches the work.
 *   - Every pointer is a device pointer owned by the caller, C-contiguous,
 *     row-major.  Outputs must not overlap inputs or each other.
 *   - Arguments are checked on the host before anything is enqueued; a
 *     failed check returns its status and leaves every buffer untouched.
 *   - Alignment: hidden / expanded / output row pointers 16 bytes, and the
 *     row length in bytes (hidden_size * element size) a multiple of 16;
 *     int32 and float arrays 4 bytes; int64 arrays (offsets, int64 ids) 8 bytes.
 *   - Limits: 1 <= num_experts <= MOE_MAX_EXPERTS; 1 <= topk <= num_experts;
 *     num_tokens >= 0; num_tokens * topk < 2^31 (int32 indices).
 */
#ifndef MOE_PERMUTE_H
#define MOE_PERMUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,         /* a size, pointer or combination is invalid */
    MOE_ERR_WORKSPACE_TOO_SMALL = 2, /* workspace_bytes < the size this call needs */
    MOE_ERR_MISALIGNED = 3,          /* pointer or row pitch breaks the alignment rules */
    MOE_ERR_UNSUPPORTED = 4,         /* element type not supported by this operation */
    MOE_ERR_HIP = 5                  /* the HIP runtime refused a launch */
} moe_status_t;

typedef enum moe_dtype {
    MOE_DTYPE_F32 = 0,      /* IEEE binary32 */
    MOE_DTYPE_BF16 = 1,     /* bfloat16 */
    MOE_DTYPE_FP8_E4M3 = 2, /* OCP fp8 E4M3FN codes (permute moves them as bytes) */
    MOE_DTYPE_INT32 = 3,    /* expert ids (topk_ids_dtype only) */
    MOE_DTYPE_INT64 = 4     /* expert ids (topk_ids_dtype only) */
} moe_dtype_t;

#define MOE_MAX_EXPERTS 1024

/*
 * moe_permute_supported -- 1 if `device` exists and is a gfx950 GPU, else 0.
 * Never fails or aborts, including on a host with no GPU or no HIP driver.
 * (Summary of vLLM PR #43014, "review highlights": the size query crashed on
 * platforms without the kernel, so callers need a guard that is always safe.)
 */
int moe_permute_supported(int device);

/*
 * moe_permute_workspace_size -- bytes of device workspace that moe_permute
 * needs for any num_tokens <= max_num_tokens with this topk and num_experts.
 * A pure host function: no HIP call, no device needed, monotone
 * non-decreasing in max_num_tokens.  Returns 0 when the arguments are outside
 * the limits above.  (Summary of vLLM PR #43014, "key code snippets": the sort
 * workspace is sized once, from the largest expanded-row count and the expert
 * count, and allocated as bytes.)
 */
size_t moe_permute_workspace_size(int64_t max_num_tokens, int32_t topk, int32_t num_experts);

/*
 * moe_permute -- expert histogram, exclusive-scan offsets, stable order of
 * the expanded rows by expert, and the gather of hidden rows into the
 * per-expert contiguous layout (vLLM PR #14568, PR description; buffers per
 * the summary of vLLM PR #43014, "key code snippets").
 *
 *   hidden_states            [N, hidden_size] of `dtype`; ignored when hidden_size == 0
 *   dtype                    MOE_DTYPE_F32 / BF16 / FP8_E4M3 (rows are moved as raw bytes)
 *   token_scale              [N] float, per-token activation scale, or NULL
 *   topk_ids                 [N, topk] of topk_ids_dtype, every value in [0, num_experts)
 *   topk_ids_dtype           MOE_DTYPE_INT32 or MOE_DTYPE_INT64.  int64 ids are read as
 *                            such and range-checked, never truncated; this removes the
 *                            separate int64 -> int32 cast pass that the summary of vLLM
 *                            PR #43014 shows in prepare_topk_ids ("key code snippets").
 *   num_tokens, hidden_size, topk, num_experts   sizes (hidden_size 0: no rows move;
 *                            the indices, and the scales when token_scale is given, do)
 *   permuted_hidden_states   [N*topk, hidden_size] of `dtype` (out); ignored when hidden_size == 0
 *   permuted_scale           [N*topk] float (out); non-NULL exactly when token_scale is
 *   expert_first_token_offset [num_experts + 1] int64 (out)
 *   permuted_idx             [N*topk] int32 (out)
 *   inv_permuted_idx         [N*topk] int32 (out)
 *   workspace                device scratch of workspace_bytes bytes (16-byte aligned);
 *                            may be NULL if moe_permute_workspace_size(N, topk, E) is 0.
 *                            Its contents on entry do not matter and are not preserved.
 *   stream                   hipStream_t
 *
 * Results never depend on earlier contents of the outputs or the workspace.
 * With num_tokens == 0 only the offsets are written (all zero).
 * An expert id outside [0, num_experts) (for int64 ids: any such int64 value)
 * is detected on the device: then every entry of expert_first_token_offset is
 * set to -1 and nothing else is written; no out-of-bounds access happens.
 */
moe_status_t moe_permute(const void *hidden_states, int32_t dtype, const float *token_scale,
                         const void *topk_ids, int32_t topk_ids_dtype, int64_t num_tokens,
                         int64_t hidden_size, int32_t topk, int32_t num_experts,
                         void *permuted_hidden_states, float *permuted_scale,
                         int64_t *expert_first_token_offset, int32_t *permuted_idx,
                         int32_t *inv_permuted_idx, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * moe_permute_static_scratch -- moe_permute for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results without `workspace` /
 * `workspace_bytes`.  The workspace is a static device array of the library,
 * MOE_STATIC_SCRATCH_BYTES bytes per GPU, held from library load until the
 * process ends; the call allocates nothing (its first call on a device looks
 * up that device's copy with hipGetSymbolAddress).
 *   - Limit: a call whose moe_permute would need more than
 *     MOE_STATIC_SCRATCH_BYTES of workspace (moe_permute_workspace_size) returns
 *     MOE_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.  Up to 16384
 *     expanded rows no workspace is used at all; up to a few hundred thousand
 *     rows (the coarse schedule) it needs at most 32 KiB.
 *   - Every call on one GPU shares that GPU's array: calls that overlap on one
 *     GPU (other streams, other threads, other processes' contexts excepted)
 *     race and must be ordered by the caller.  The kernels initialise every
 *     workspace word they read, so the contents left by an earlier call never
 *     matter.
 */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)4 << 20)
moe_status_t moe_permute_static_scratch(const void *hidden_states, int32_t dtype, const float *token_scale,
                                        const void *topk_ids, int32_t topk_ids_dtype, int64_t num_tokens,
                                        int64_t hidden_size, int32_t topk, int32_t num_experts,
                                        void *permuted_hidden_states, float *permuted_scale,
                                        int64_t *expert_first_token_offset, int32_t *permuted_idx,
                                        int32_t *inv_permuted_idx, void *stream);

/*
 * moe_permute_local_workspace_size -- as moe_permute_workspace_size, for
 * moe_permute_local with this num_local_experts.  Pure host function; returns
 * 0 outside the limits (those of moe_permute, and
 * 1 <= num_local_experts <= MOE_MAX_EXPERTS).
 */
size_t moe_permute_local_workspace_size(int64_t max_num_tokens, int32_t topk, int32_t num_experts,
                                        int32_t num_local_experts);

/*
 * moe_permute_local -- moe_permute restricted to the experts of this rank
 * (expert parallelism).  vLLM PR #14568, PR description, lists expert
 * parallelism through an expert map as not yet supported by its kernels; the
 * summary of vLLM PR #43014, "key code snippets", sizes the offsets by the
 * number of local experts.  Reading taken here:
 *
 *   expert_map        [num_experts] int32 (device): expert_map[g] is the local
 *                     id of global expert g, in [0, num_local_experts), or -1
 *                     when g lives on another rank.  Several global experts may
 *                     share a local id; their rows then share its block.
 *   num_local_experts number of local experts L (1..MOE_MAX_EXPERTS)
 *
 * A row is local when its expert's map entry is >= 0; its key is that local
 * id.  Local rows are counted, stably ordered by local id and copied exactly
 * as moe_permute does for experts; the outputs change as follows:
 *   expert_first_token_offset [L + 1]: entry l = local rows with local id < l,
 *                     entry L = number of local rows M
 *   permuted_idx, permuted_hidden_states, permuted_scale: the first M entries
 *                     / rows are written, the rest of each buffer is untouched
 *   inv_permuted_idx  [N*topk]: the slot of a local row, -1 for every other row
 * Hidden rows of tokens with no local row are not read.  moe_unpermute_local
 * (or moe_unpermute) skips the -1 entries, so its output is this rank's share
 * of each token's sum.
 * All other arguments, conventions and limits are those of moe_permute
 * (buffers are still sized for N*topk rows; workspace from
 * moe_permute_local_workspace_size).  A topk_ids value outside
 * [0, num_experts), or a map entry of a used expert outside
 * [-1, num_local_experts), is detected on the device: every entry of
 * expert_first_token_offset is set to -1 and nothing else is written.
 */
moe_status_t moe_permute_local(const void *hidden_states, int32_t dtype, const float *token_scale,
                               const void *topk_ids, int32_t topk_ids_dtype, int64_t num_tokens,
                               int64_t hidden_size, int32_t topk, int32_t num_experts,
                               const int32_t *expert_map,
                               int32_t num_local_experts, void *permuted_hidden_states,
                               float *permuted_scale, int64_t *expert_first_token_offset,
                               int32_t *permuted_idx, int32_t *inv_permuted_idx, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * moe_permute_quant_fp8 -- quantise while permuting: the permute (or, with an
 * expert map, the local-expert permute) of bf16 or f32 token rows whose
 * moved rows are fp8 E4M3FN codes with their scales, quantised on the way
 * (vLLM PR #19636 "[Kernels] MoE refactor", highlights: per-token activation
 * quantisation and block shapes; the permute per vLLM PR #14568).
 *
 * Per group of group_size consecutive elements of a token row (group_size 0:
 * the whole row, one scale per token):
 *     scale = amax / 448 as one float division (1 when amax is 0; NaN
 *             elements do not count towards amax)
 *     code  = E4M3FN(x / scale): the float quotient rounded to the nearest
 *             code, ties to even, saturated at +-448; a NaN quotient -> 0x7F
 *
 *   hidden_states     [N, hidden_size] of dtype MOE_DTYPE_BF16 or MOE_DTYPE_F32;
 *                     rows of at most 16 KiB (8192 bf16 / 4096 f32 elements)
 *   topk_ids .. num_experts   as for moe_permute
 *   expert_map, num_local_experts   NULL and 0 for the plain permute, else as
 *                     for moe_permute_local
 *   group_size        0, or a power of two dividing hidden_size, at least 8
 *                     (bf16) / 4 (f32) elements and at most 64 times that
 *   permuted_codes    [N*topk, hidden_size] bytes (out), 16-byte aligned
 *   permuted_scale    [N*topk, hidden_size / group_size] float (out; one
 *                     column for group_size 0)
 *   expert_first_token_offset, permuted_idx, inv_permuted_idx   as for
 *                     moe_permute / moe_permute_local
 *   workspace         sized by moe_permute_workspace_size, or by
 *                     moe_permute_local_workspace_size with a map
 *
 * Codes and scales of a row are written to every destination of its token
 * (only the first M rows with a map).  A bad id or map entry: offsets -1,
 * nothing else written.
 */
moe_status_t moe_permute_quant_fp8(const void *hidden_states, int32_t dtype, const void *topk_ids,
                                   int32_t topk_ids_dtype, int64_t num_tokens, int64_t hidden_size,
                                   int32_t topk, int32_t num_experts, const int32_t *expert_map,
                                   int32_t num_local_experts, int64_t group_size,
                                   uint8_t *permuted_codes, float *permuted_scale,
                                   int64_t *expert_first_token_offset, int32_t *permuted_idx,
                                   int32_t *inv_permuted_idx, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * moe_grouped_gemm_bf16 -- the expert GEMM between permute and unpermute
 * (vLLM PR #14568, PR description: the permute makes each expert's tokens
 * contiguous for a grouped GEMM, whose expanded output the unpermute then
 * reduces).  For every expert e and permuted row j in [off[e], off[e+1]):
 *     y[j][c] = sum over i of x[j][i] * w[e][c][i]
 * bf16 inputs, fp32 accumulation (on the matrix cores; at decode sizes, with
 * one or two rows per expert on average, by bf16 dot products on the vector
 * units), rounded once to bf16 (round to nearest even); the order of the fp32
 * sums is not specified.  y is in permuted order, ready for moe_unpermute.
 *
 *   x                 [max_rows, k] bf16, permuted rows (e.g. permuted_hidden_states)
 *   w                 [num_experts, n, k] bf16 (expert e: n output rows of k, a
 *                     linear layer's weight)
 *   expert_first_token_offset  [num_experts + 1] int64 on the device, as the
 *                     permute wrote it (the row counts are never read by the host)
 *   num_experts       1 .. MOE_MAX_EXPERTS
 *   max_rows          rows x and y hold; off[num_experts] must not exceed it
 *   n, k              n a multiple of 128, k a multiple of 64 and at most 2^20
 *   y                 [max_rows, n] bf16 (out); rows >= off[num_experts] untouched
 *
 * Offsets that are not a valid prefix (off[0] != 0, a decreasing entry, the
 * -1 the permute writes for a rejected id, or off[E] > max_rows) are detected
 * on the device: nothing is written.  Needs no workspace.
 */
moe_status_t moe_grouped_gemm_bf16(const void *x, const void *w, const int64_t *expert_first_token_offset,
                                   int32_t num_experts, int64_t max_rows, int64_t n, int64_t k, void *y,
                                   void *stream);

/*
 * moe_unpermute -- weighted top-k reduction of the expanded grouped-GEMM
 * output back to one row per token (vLLM PR #14568, PR description):
 *     output[t] = sum_{k=0}^{topk-1} topk_weights[t][k] * expanded_output[inv_permuted_idx[t*topk+k]]
 * accumulated in fp32 in ascending k, rounded once to `dtype`.
 *
 *   expanded_output   [N*topk, hidden_size] of `dtype`, in permuted order
 *   dtype             MOE_DTYPE_F32 or MOE_DTYPE_BF16 (else MOE_ERR_UNSUPPORTED)
 *   topk_weights      [N, topk] float
 *   inv_permuted_idx  [N*topk] int32, as written by moe_permute or
 *                     moe_permute_local
 *   output            [N, hidden_size] of `dtype` (out)
 *
 * An entry of -1 (a row of an expert on another rank, see moe_permute_local)
 * adds nothing: its row is not read and its weight not used; a token whose
 * entries are all -1 gets a zero row.  Any other entry outside [0, N*topk)
 * is detected on the device: that token's output row is filled with NaN and
 * no out-of-bounds read happens.
 * Needs no workspace.
 */
moe_status_t moe_unpermute(const void *expanded_output, int32_t dtype, const float *topk_weights,
                           const int32_t *inv_permuted_idx, int64_t num_tokens,
                           int64_t hidden_size, int32_t topk, void *output, void *stream);

/*
 * moe_unpermute_local -- moe_unpermute for the inverse index of an expert
 * split: the same reduction (vLLM PR #14568, PR description), arguments,
 * result and errors, scheduled for inverse indices written by
 * moe_permute_local, where most of a token's topk entries are -1.  With one
 * or two live entries per token the reduction is latency bound: it uses
 * every wave slot of the chip, and at topk 8 on large calls a wave sums
 * several chunks of a token row from its live entries at once.
 * moe_unpermute limits large topk-8 reductions to fewer resident waves,
 * which is faster when every entry is live.  Either entry point is correct
 * for any inverse index and gives the same bits.
 */
moe_status_t moe_unpermute_local(const void *expanded_output, int32_t dtype, const float *topk_weights,
                                 const int32_t *inv_permuted_idx, int64_t num_tokens,
                                 int64_t hidden_size, int32_t topk, void *output, void *stream);

/* Static, human-readable name of a status code. */
const char *moe_status_string(moe_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PERMUTE_H */
