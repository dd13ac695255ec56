/*
 * moe_oracle.c -- plain, slow, obviously correct CPU definition of the MoE
 * token permute / unpermute path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it.  Its users are the tests, the
 * small smoke check and the CPU-baseline leg of the benchmark.  It shares no
 * code, header, table or helper with the HIP implementation.
 *
 * Sources (the three pages on the subject):
 *   [P1] vLLM PR #14568, "permute/unpermute kernel for moe optimization",
 *        PR description: permute expands each token to its topk copies and
 *        orders them so that every expert's tokens are contiguous for the
 *        grouped GEMM; unpermute reduces the expanded grouped-GEMM output back
 *        per token, scaling by topk_weight.
 *   [P3] prhub summary of vLLM PR #43014 (preallocated MoE permute buffers),
 *        section "key code snippets", class MoEPermuteScratch: buffer names,
 *        dtypes and lengths (token_expert_indices = arange of the expanded
 *        rows viewed [n_token, topk]; expert_first_token_offset int64 of
 *        length num_local_experts+1; permuted_idx, inv_permuted_idx int32 of
 *        length max_expanded_rows; permuted_hidden_states of hidden_dtype).
 *
 * Readings taken where the pages are silent (each is listed with its reason
 * in the design notes of the repository):
 *   - expanded row r of token t, slot k is r = t*topk + k (the arange view);
 *   - rows with the same expert keep ascending r (a stable sort);
 *   - permuted_idx[j] = r, the expanded row that lands in permuted slot j;
 *     inv_permuted_idx[r] = j, its inverse;
 *   - unpermute computes out[t] = sum_k w[t,k] * Y[inv[t*topk+k]]: here the
 *     sum is formed in double precision in ascending k and rounded once to the
 *     output type (round to nearest, ties to even);
 *   - with a local-expert filter, rows of experts on other ranks are left out
 *     of the permute (inverse index -1) and add nothing in the unpermute.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -o libmoe_oracle.so moe_oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ID (-1)  /* an expert id outside [0, num_experts) */
#define ORACLE_BAD_ARG (-2) /* a size or pointer that makes no sense */
#define ORACLE_BAD_INV (-3) /* an inv_permuted_idx entry outside [0, N*topk) */

/* ------------------------------------------------------------------------ */
/* Permute, step 1 -- tokens per expert.                                      */
/* [P3] key code snippets, MoEPermuteScratch: expert_first_token_offset has   */
/* one entry per local expert plus one, so the permute needs the number of    */
/* expanded rows routed to each expert.  The expanded rows are the topk_ids   */
/* entries taken in row-major order (token_expert_indices is an arange viewed */
/* as [n_token, topk]).                                                       */
/* ------------------------------------------------------------------------ */
int oracle_expert_counts(const int32_t *topk_ids, int64_t num_tokens,
                         int32_t topk, int32_t num_experts, int64_t *counts)
{
    if (num_tokens < 0 || topk < 1 || num_experts < 1)
        return ORACLE_BAD_ARG;
    for (int32_t e = 0; e < num_experts; ++e)
        counts[e] = 0;
    for (int64_t t = 0; t < num_tokens; ++t) {
        for (int32_t k = 0; k < topk; ++k) {
            int32_t id = topk_ids[t * topk + k];
            if (id < 0 || id >= num_experts)
                return ORACLE_BAD_ID;
            counts[id] += 1;
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Permute, step 2 -- expert_first_token_offset.                              */
/* [P3] key code snippets: int64, num_experts + 1 entries.  Entry e is the    */
/* first permuted slot of expert e; the last entry is the number of expanded  */
/* rows.  This is the exclusive prefix sum of the counts.                     */
/* ------------------------------------------------------------------------ */
void oracle_expert_first_token_offset(const int64_t *counts, int32_t num_experts,
                                      int64_t *expert_first_token_offset)
{
    expert_first_token_offset[0] = 0;
    for (int32_t e = 0; e < num_experts; ++e)
        expert_first_token_offset[e + 1] = expert_first_token_offset[e] + counts[e];
}

/* ------------------------------------------------------------------------ */
/* Permute, step 3 -- stable order of the expanded rows by expert.            */
/* [P1] PR description: the expanded tokens are ordered so that each expert's */
/* tokens become contiguous.  [P3] key code snippets: permuted_idx and        */
/* inv_permuted_idx, int32, one entry per expanded row.                       */
/* A counting sort: walk the expanded rows in ascending r and hand each the   */
/* next free slot of its expert.  The ascending walk is what makes rows of    */
/* one expert keep ascending r.                                               */
/* ------------------------------------------------------------------------ */
int oracle_stable_expert_order(const int32_t *topk_ids, int64_t num_rows,
                               int32_t num_experts,
                               const int64_t *expert_first_token_offset,
                               int32_t *permuted_idx, int32_t *inv_permuted_idx)
{
    int64_t *next_slot = (int64_t *)malloc(sizeof(int64_t) * (size_t)num_experts);
    if (next_slot == NULL)
        return ORACLE_BAD_ARG;
    for (int32_t e = 0; e < num_experts; ++e)
        next_slot[e] = expert_first_token_offset[e];
    for (int64_t r = 0; r < num_rows; ++r) {
        int32_t id = topk_ids[r];
        if (id < 0 || id >= num_experts) {
            free(next_slot);
            return ORACLE_BAD_ID;
        }
        int64_t j = next_slot[id];
        next_slot[id] = j + 1;
        permuted_idx[j] = (int32_t)r;
        inv_permuted_idx[r] = (int32_t)j;
    }
    free(next_slot);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Permute, step 4 -- gather the hidden rows into the permuted layout.        */
/* [P1] PR description: the permute gathers the tokens that are not          */
/* contiguous for an expert into one contiguous block.  [P3] key code         */
/* snippets: permuted_hidden_states has max_expanded_rows * hidden_size       */
/* elements of hidden_dtype.  Expanded row r belongs to token r / topk.       */
/* The copy is of raw bytes, so any element type (fp32, bf16, fp8 codes) is   */
/* moved unchanged.  A per-token activation scale, when present, moves with   */
/* its row ([P2] vLLM PR #19636 "[Kernels] MoE refactor", highlights:         */
/* per-token activation quantisation parameters).                             */
/* ------------------------------------------------------------------------ */
void oracle_gather_rows(const uint8_t *hidden_states, int64_t row_bytes,
                        const float *token_scale, const int32_t *permuted_idx,
                        int64_t num_rows, int32_t topk,
                        uint8_t *permuted_hidden_states, float *permuted_scale)
{
    for (int64_t j = 0; j < num_rows; ++j) {
        int64_t t = permuted_idx[j] / topk;
        if (row_bytes > 0)
            memcpy(permuted_hidden_states + j * row_bytes, hidden_states + t * row_bytes,
                   (size_t)row_bytes);
        if (token_scale != NULL && permuted_scale != NULL)
            permuted_scale[j] = token_scale[t];
    }
}

/* ------------------------------------------------------------------------ */
/* Expert ids given as int64.  [P3] key code snippets, prepare_topk_ids: ids  */
/* of another integer type are cast to int32 before the permute.  The         */
/* permute depends only on the id values, so int64 ids pose the same problem  */
/* once every value is known to lie in [0, num_experts): copy them to int32,  */
/* or fail on a value outside that range (no value is ever truncated).        */
/* ------------------------------------------------------------------------ */
int oracle_ids_from_int64(const int64_t *ids64, int64_t count, int32_t num_experts, int32_t *ids32)
{
    if (count < 0 || num_experts < 1)
        return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < count; ++i) {
        if (ids64[i] < 0 || ids64[i] >= (int64_t)num_experts)
            return ORACLE_BAD_ID;
        ids32[i] = (int32_t)ids64[i];
    }
    return ORACLE_OK;
}

/* The whole permute: steps 1 to 4 in order. */
int oracle_moe_permute(const uint8_t *hidden_states, int64_t row_bytes,
                       const float *token_scale, const int32_t *topk_ids,
                       int64_t num_tokens, int32_t topk, int32_t num_experts,
                       uint8_t *permuted_hidden_states, float *permuted_scale,
                       int64_t *expert_first_token_offset, int32_t *permuted_idx,
                       int32_t *inv_permuted_idx)
{
    int64_t *counts = (int64_t *)malloc(sizeof(int64_t) * (size_t)(num_experts > 0 ? num_experts : 1));
    if (counts == NULL)
        return ORACLE_BAD_ARG;
    int status = oracle_expert_counts(topk_ids, num_tokens, topk, num_experts, counts);
    if (status == ORACLE_OK) {
        oracle_expert_first_token_offset(counts, num_experts, expert_first_token_offset);
        status = oracle_stable_expert_order(topk_ids, num_tokens * topk, num_experts,
                                            expert_first_token_offset, permuted_idx,
                                            inv_permuted_idx);
    }
    /* A token's scale moves with it to every destination, also when its row is
       zero bytes wide (a call that moves indices and scales only). */
    if (status == ORACLE_OK && (row_bytes > 0 || token_scale != NULL))
        oracle_gather_rows(hidden_states, row_bytes, token_scale, permuted_idx,
                           num_tokens * topk, topk, permuted_hidden_states,
                           permuted_scale);
    free(counts);
    return status;
}

/* ------------------------------------------------------------------------ */
/* Permute with a local-expert filter (expert parallelism).                   */
/* [P1] PR description: expert parallelism through an expert_map was not yet  */
/* supported.  [P3] key code snippets: the offsets have num_local_experts + 1 */
/* entries.  Reading taken: expert_map[g] is the local id of global expert g, */
/* or -1 when g lives elsewhere.  Only rows whose expert is local are         */
/* counted, ordered (by local id, then ascending r) and copied; such a row's  */
/* inv_permuted_idx is its slot, every other row's is -1.  permuted_idx and   */
/* the permuted rows are written for the first (number of local rows) slots.  */
/* An id outside [0, num_experts) or a map entry outside [-1, num_local)      */
/* makes the call fail.                                                       */
/* ------------------------------------------------------------------------ */
int oracle_moe_permute_local(const uint8_t *hidden_states, int64_t row_bytes,
                             const float *token_scale, const int32_t *topk_ids,
                             int64_t num_tokens, int32_t topk, int32_t num_experts,
                             const int32_t *expert_map, int32_t num_local_experts,
                             uint8_t *permuted_hidden_states, float *permuted_scale,
                             int64_t *expert_first_token_offset, int32_t *permuted_idx,
                             int32_t *inv_permuted_idx)
{
    if (num_tokens < 0 || topk < 1 || num_experts < 1 || num_local_experts < 1)
        return ORACLE_BAD_ARG;
    int64_t num_rows = num_tokens * topk;
    /* local expert of every expanded row, -1 for rows of other ranks */
    int32_t *local = (int32_t *)malloc(sizeof(int32_t) * (size_t)(num_rows > 0 ? num_rows : 1));
    int64_t *counts = (int64_t *)malloc(sizeof(int64_t) * (size_t)num_local_experts);
    int64_t *next_slot = (int64_t *)malloc(sizeof(int64_t) * (size_t)num_local_experts);
    if (local == NULL || counts == NULL || next_slot == NULL) {
        free(local);
        free(counts);
        free(next_slot);
        return ORACLE_BAD_ARG;
    }
    int status = ORACLE_OK;
    for (int32_t e = 0; e < num_local_experts; ++e)
        counts[e] = 0;
    for (int64_t r = 0; r < num_rows && status == ORACLE_OK; ++r) {
        int32_t id = topk_ids[r];
        if (id < 0 || id >= num_experts) {
            status = ORACLE_BAD_ID;
            break;
        }
        int32_t l = expert_map[id];
        if (l < -1 || l >= num_local_experts) {
            status = ORACLE_BAD_ID;
            break;
        }
        local[r] = l;
        if (l >= 0)
            counts[l] += 1;
    }
    if (status == ORACLE_OK) {
        expert_first_token_offset[0] = 0;
        for (int32_t e = 0; e < num_local_experts; ++e)
            expert_first_token_offset[e + 1] = expert_first_token_offset[e] + counts[e];
        for (int32_t e = 0; e < num_local_experts; ++e)
            next_slot[e] = expert_first_token_offset[e];
        for (int64_t r = 0; r < num_rows; ++r) {
            if (local[r] < 0) {
                inv_permuted_idx[r] = -1;
                continue;
            }
            int64_t j = next_slot[local[r]]++;
            permuted_idx[j] = (int32_t)r;
            inv_permuted_idx[r] = (int32_t)j;
        }
        if (row_bytes > 0 || token_scale != NULL)
            oracle_gather_rows(hidden_states, row_bytes, token_scale, permuted_idx,
                               expert_first_token_offset[num_local_experts], topk,
                               permuted_hidden_states, permuted_scale);
    }
    free(local);
    free(counts);
    free(next_slot);
    return status;
}

/* ------------------------------------------------------------------------ */
/* bfloat16, written from the format: 1 sign bit, 8 exponent bits (bias 127), */
/* 7 fraction bits.  Exponent field 0 holds zero and the subnormals          */
/* (fraction * 2^-133); field 255 holds infinities (fraction 0) and NaNs.    */
/* ------------------------------------------------------------------------ */
double oracle_bf16_to_double(uint16_t bits)
{
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 7) & 0xFF;
    int frac = bits & 0x7F;
    double mag;
    if (expo == 0xFF)
        mag = frac ? NAN : INFINITY;
    else if (expo == 0)
        mag = ldexp((double)frac, -133);
    else
        mag = ldexp(128.0 + (double)frac, expo - 127 - 7);
    return sign ? -mag : mag;
}

/* Round a double to the nearest bfloat16, ties to the even fraction; values */
/* whose rounded magnitude reaches 2^128 become infinity.  NaN maps to the    */
/* quiet NaN 0x7FC0 with the input's sign.                                    */
uint16_t oracle_double_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(x);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    int e2;
    frexp(a, &e2);              /* a lies in [2^(e2-1), 2^e2) */
    int p = e2 - 1;             /* binade exponent */
    if (p < -126)
        p = -126;               /* below the normal range the spacing stays 2^-133 */
    double quantum = ldexp(1.0, p - 7); /* spacing of bf16 values in this binade */
    double q = nearbyint(a / quantum);  /* a / quantum is exact; default mode is nearest-even */
    double v = q * quantum;
    if (v >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);
    if (v < ldexp(1.0, -126))  /* subnormal (or rounded up to exactly 2^-126, handled below) */
        return (uint16_t)(sign | (uint16_t)(v / ldexp(1.0, -133)));
    frexp(v, &e2);
    int expo = e2 - 1 + 127;
    int frac = (int)(v / ldexp(1.0, e2 - 1 - 7)) - 128;
    return (uint16_t)(sign | (uint16_t)(expo << 7) | (uint16_t)frac);
}

/* ------------------------------------------------------------------------ */
/* fp8 E4M3FN, written from the format (the OCP 8-bit floating-point E4M3     */
/* encoding without infinities): a sign bit, 4 exponent bits with bias 7 and  */
/* 3 fraction bits.  Exponent field 0 holds the subnormals frac * 2^-9; the   */
/* all-ones pattern S.1111.111 is NaN, so the largest finite magnitude is     */
/* 1.75 * 2^8 = 448 (S.1111.110).                                             */
/* ------------------------------------------------------------------------ */
double oracle_e4m3_to_double(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int expo = (code >> 3) & 0xF;
    int frac = code & 0x7;
    double mag;
    if (expo == 0xF && frac == 0x7)
        mag = NAN;
    else if (expo == 0)
        mag = ldexp((double)frac, -9);
    else
        mag = ldexp(8.0 + (double)frac, expo - 7 - 3);
    return sign ? -mag : mag;
}

/* Nearest E4M3FN value, ties to the even fraction, after clamping the input  */
/* to [-448, 448] (saturation, as quantisers do).  NaN maps to S.1111.111.    */
uint8_t oracle_double_to_e4m3(double x)
{
    uint8_t sign = signbit(x) ? 0x80u : 0u;
    if (isnan(x))
        return (uint8_t)(sign | 0x7Fu);
    double a = fabs(x);
    if (a > 448.0)
        a = 448.0;
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);              /* a lies in [2^(e2-1), 2^e2) */
    int p = e2 - 1;             /* binade exponent */
    if (p < -6)
        p = -6;                 /* below the normal range the spacing stays 2^-9 */
    double quantum = ldexp(1.0, p - 3);
    double v = nearbyint(a / quantum) * quantum; /* a / quantum is exact; nearest-even */
    if (v < ldexp(1.0, -6))     /* subnormal (a value rounded up to 2^-6 is handled below) */
        return (uint8_t)(sign | (uint8_t)(v / ldexp(1.0, -9)));
    frexp(v, &e2);
    int expo = e2 - 1 + 7;
    int frac = (int)(v / ldexp(1.0, e2 - 1 - 3)) - 8;
    return (uint8_t)(sign | (uint8_t)(expo << 3) | (uint8_t)frac);
}

/* ------------------------------------------------------------------------ */
/* Dynamic fp8 quantisation of activation rows.                              */
/* [P2] vLLM PR #19636 "[Kernels] MoE refactor", highlights: activations are  */
/* quantised per token (per-token activation quantisation parameters), and   */
/* the quantisation configuration carries a block shape.  Reading taken: the  */
/* row is cut into groups of `group` consecutive elements (group = h: one     */
/* scale per token); per group                                                */
/*   amax  = the largest |x| (exact),                                         */
/*   scale = amax / 448 as one float division (1 when amax is 0),             */
/*   code  = E4M3FN of the float quotient x / scale (one float division,      */
/*           then the rounding above); a NaN quotient (a NaN input, or inf /  */
/*           inf) gets the positive NaN code 0x7F, whatever its sign bit.     */
/* NaN never counts towards amax (no comparison with it holds).               */
/* x is float32 (x_is_bf16 = 0) or bfloat16 bit patterns (x_is_bf16 = 1).     */
/* scales is [rows][h / group].                                               */
/* ------------------------------------------------------------------------ */
int oracle_quantize_fp8_rows(const void *x, int x_is_bf16, int64_t rows, int64_t h, int64_t group,
                             uint8_t *codes, float *scales)
{
    if (rows < 0 || h < 1 || group < 1 || h % group != 0)
        return ORACLE_BAD_ARG;
    int64_t groups = h / group;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < groups; ++g) {
            float amax = 0.0f;
            for (int64_t i = g * group; i < (g + 1) * group; ++i) {
                float v = x_is_bf16 ? (float)oracle_bf16_to_double(((const uint16_t *)x)[r * h + i])
                                    : ((const float *)x)[r * h + i];
                if (fabsf(v) > amax)
                    amax = fabsf(v);
            }
            float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
            scales[r * groups + g] = scale;
            for (int64_t i = g * group; i < (g + 1) * group; ++i) {
                float v = x_is_bf16 ? (float)oracle_bf16_to_double(((const uint16_t *)x)[r * h + i])
                                    : ((const float *)x)[r * h + i];
                float q = v / scale;
                /* A NaN quotient (a NaN element, or an infinite one divided by an
                   infinite scale) takes the one code 0x7F.  IEEE 754 leaves the sign
                   of a NaN that arithmetic produces unspecified, and x86 (negative
                   default NaN) and the GPU (positive) differ, so a code that copied
                   it would depend on the machine.  The format codec keeps a NaN's
                   sign because it converts bits, not an arithmetic result. */
                codes[r * h + i] = isnan(q) ? 0x7Fu : oracle_double_to_e4m3((double)q);
            }
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Grouped GEMM over the permuted rows.                                       */
/* [P1] PR description: the permute makes each expert's tokens contiguous so  */
/* that a grouped GEMM can run the experts over them, and the unpermute then  */
/* reduces that GEMM's expanded output.  Reading taken: expert e's weight is  */
/* w[e] with n_out rows of k_in elements (a linear layer: y = x w[e]^T), the  */
/* rows of expert e are permuted rows [off[e], off[e+1]), and                 */
/*   y[j][n] = sum over k of x[j][k] * w[e][n][k]                             */
/* in double precision, rounded once to bfloat16.  x, w and y are bfloat16    */
/* bit patterns; y is in permuted order, as the unpermute reads it.           */
/* ------------------------------------------------------------------------ */
int oracle_grouped_gemm_bf16(const uint16_t *x, const uint16_t *w, const int64_t *off, int32_t num_experts,
                             int64_t n_out, int64_t k_in, uint16_t *y)
{
    if (num_experts < 1 || n_out < 1 || k_in < 1 || off[0] != 0)
        return ORACLE_BAD_ARG;
    for (int32_t e = 0; e < num_experts; ++e)
        if (off[e + 1] < off[e])
            return ORACLE_BAD_ARG;
    for (int32_t e = 0; e < num_experts; ++e) {
        const uint16_t *we = w + (int64_t)e * n_out * k_in;
        for (int64_t j = off[e]; j < off[e + 1]; ++j) {
            for (int64_t n = 0; n < n_out; ++n) {
                double acc = 0.0;
                for (int64_t k = 0; k < k_in; ++k)
                    acc += oracle_bf16_to_double(x[j * k_in + k]) * oracle_bf16_to_double(we[n * k_in + k]);
                y[j * n_out + n] = oracle_double_to_bf16(acc);
            }
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Unpermute.                                                                 */
/* [P1] PR description: reduce the expanded grouped-GEMM output back per      */
/* token and scale each contribution by its topk_weight:                      */
/*     out[t, h] = sum_{k=0}^{topk-1} w[t, k] * Y[inv_permuted_idx[t*topk+k], h] */
/* Y is in permuted order, so the row holding token t's slot k is             */
/* inv_permuted_idx[t*topk+k].  The sum is formed in double precision in      */
/* ascending k and rounded once to the output type.  A slot whose index is -1 */
/* (its expert lives on another rank, see the local-expert filter above)      */
/* contributes nothing.                                                       */
/* ------------------------------------------------------------------------ */
int oracle_unpermute_f32(const float *expanded_output, const float *topk_weights,
                         const int32_t *inv_permuted_idx, int64_t num_tokens,
                         int32_t topk, int64_t hidden_size, float *output)
{
    int64_t num_rows = num_tokens * topk;
    for (int64_t r = 0; r < num_rows; ++r)
        if (inv_permuted_idx[r] < -1 || inv_permuted_idx[r] >= num_rows)
            return ORACLE_BAD_INV;
    for (int64_t t = 0; t < num_tokens; ++t) {
        for (int64_t h = 0; h < hidden_size; ++h) {
            double acc = 0.0;
            for (int32_t k = 0; k < topk; ++k) {
                int64_t r = t * topk + k;
                int64_t j = inv_permuted_idx[r];
                if (j < 0)
                    continue;
                acc += (double)topk_weights[r] * (double)expanded_output[j * hidden_size + h];
            }
            output[t * hidden_size + h] = (float)acc;
        }
    }
    return ORACLE_OK;
}

int oracle_unpermute_bf16(const uint16_t *expanded_output, const float *topk_weights,
                          const int32_t *inv_permuted_idx, int64_t num_tokens,
                          int32_t topk, int64_t hidden_size, uint16_t *output)
{
    int64_t num_rows = num_tokens * topk;
    for (int64_t r = 0; r < num_rows; ++r)
        if (inv_permuted_idx[r] < -1 || inv_permuted_idx[r] >= num_rows)
            return ORACLE_BAD_INV;
    for (int64_t t = 0; t < num_tokens; ++t) {
        for (int64_t h = 0; h < hidden_size; ++h) {
            double acc = 0.0;
            for (int32_t k = 0; k < topk; ++k) {
                int64_t r = t * topk + k;
                int64_t j = inv_permuted_idx[r];
                if (j < 0)
                    continue;
                acc += (double)topk_weights[r] *
                       oracle_bf16_to_double(expanded_output[j * hidden_size + h]);
            }
            output[t * hidden_size + h] = oracle_double_to_bf16(acc);
        }
    }
    return ORACLE_OK;
}
