/*
 * oracle.h -- plain CPU oracle of the MoE re-routing operator (MoeReRoutingV2).
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The product path (the HIP library and
 * its Python binding) never calls it, and it shares no source with that path.
 *
 * Everything here is single-threaded, unblocked and written to be read against
 * the page "CANN ops-transformer MoeReRoutingV2" (nlpx.cn article), sections
 * "计算公式" (computation formulas), "参数说明" (parameter table) and
 * "约束说明" (constraints). The operator only moves bytes and computes integer
 * offsets, so there is no floating-point arithmetic and no tolerance: every
 * result is exact.
 */
#ifndef MRR_ORACLE_H
#define MRR_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes of the oracle. */
#define ORACLE_OK 0
#define ORACLE_BAD_ARGS 1   /* a NULL pointer, attr outside {0,1}, row bytes < 0 */
#define ORACLE_BAD_COUNTS 2 /* a negative count, or the counts do not sum to A   */

/*
 * SrcOffset / DstOffset of every (rank i, expert j) cell of the count matrix
 * counts[N][E] ("计算公式" section, the two double-sum formulas):
 *   src_off[i*E+j] = number of tokens in all cells before (i,j) in row-major
 *                    (rank, then expert) order  -- where segment (i,j) starts
 *                    in the rank-major input;
 *   dst_off[i*E+j] = number of tokens in all cells before (i,j) in
 *                    column-major (expert, then rank) order -- where it starts
 *                    in the expert-major output.
 * counts_is_i64 selects int64 (1) or int32 (0) elements. Outputs are [N*E]
 * int64, indexed by the row-major cell index i*E+j.
 * Returns ORACLE_BAD_COUNTS on a negative count.
 */
int oracle_offsets(const void* counts, int counts_is_i64, int64_t N, int64_t E,
                   int64_t* src_off, int64_t* dst_off);

/*
 * The whole operator on host buffers. Rows are opaque byte strings:
 *   tokens        [A][token_row_bytes]   (fp4 packs two values per byte, so
 *                                         its row bytes are H/2)
 *   scales        [A][scale_row_bytes] or NULL (absent)
 *   weight        [A] float or NULL (absent); copied as 4 raw bytes
 *   counts        [N][E] int32 or int64
 * Outputs:
 *   out_tokens    [A][token_row_bytes]
 *   out_scales    [A][scale_row_bytes]   (written only when scales != NULL)
 *   out_idx       [A] int32
 *   out_etn       [E] in the counts' dtype
 *   out_weight    [A] float              (written only when weight != NULL)
 * etn_type: 1 = per-expert counts, 0 = inclusive running sum of them.
 * idx_type: 0 = gather index (out row d came from input row idx[d]),
 *           1 = scatter index (input row s went to out row idx[s]).
 * Nothing is written unless the counts are valid (all >= 0, sum == A).
 */
int oracle_reroute(const uint8_t* tokens, int64_t A, int64_t token_row_bytes,
                   const void* counts, int counts_is_i64, int64_t N, int64_t E,
                   const uint8_t* scales, int64_t scale_row_bytes,
                   const float* weight,
                   int64_t etn_type, int64_t idx_type,
                   uint8_t* out_tokens, uint8_t* out_scales, int32_t* out_idx,
                   void* out_etn, float* out_weight);

/*
 * The inverse re-route (not on the page; the "计算公式" moves read
 * backwards): rows [A][row_bytes] in expert-major order, as the operator
 * outputs them, return to rank-major order:
 *   out_rows[SrcOffset + k] = rows[DstOffset + k]   (and scales, weight)
 * for every cell and 0 <= k < its count. idx_type 0: out_idx[s] = the input
 * (expert-major) row of output row s; 1: out_idx[d] = the output row of input
 * row d. out_etn is the forward operator's expert_token_num. Same arguments,
 * checks and return codes as oracle_reroute.
 */
int oracle_reroute_inverse(const uint8_t* rows, int64_t A, int64_t row_bytes,
                           const void* counts, int counts_is_i64, int64_t N, int64_t E,
                           const uint8_t* scales, int64_t scale_row_bytes,
                           const float* weight,
                           int64_t etn_type, int64_t idx_type,
                           uint8_t* out_rows, uint8_t* out_scales, int32_t* out_idx,
                           void* out_etn, float* out_weight);

#ifdef __cplusplus
}
#endif
#endif /* MRR_ORACLE_H */
