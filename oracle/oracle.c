/*
 * oracle.c -- plain, slow, single-threaded CPU oracle of MoeReRoutingV2.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): loaded by the tests, the smoke
 * check and the benchmark's CPU-baseline leg, never by the product path.
 *
 * Source: the page "CANN ops-transformer MoeReRoutingV2" (nlpx.cn article):
 *   - "计算公式": SrcOffset and DstOffset as double sums over the count matrix,
 *     and the three moves permute_X[DstOffset + k] = X[SrcOffset + k] for
 *     0 <= k < (tokens of the current cell), for X in tokens, per_token_scales,
 *     expert_topk_weight;
 *   - "参数说明": permute_token_idx is each token's index in the original
 *     layout (gather form for idx_type 0, scatter form for 1), and
 *     expert_token_num is the tokens per expert (count mode 1, cumsum mode 0);
 *   - "约束说明": Sum(counts) == A.
 *
 * Readings taken where the extracted text is silent or garbled:
 *   - The formulas' lower bounds lost their "=" in extraction. The double sums
 *     are read as "every cell that comes before (cur_rank, cur_expert)": in
 *     row-major (rank, expert) order for SrcOffset, because the input is laid
 *     out by source rank; in column-major (expert, rank) order for DstOffset,
 *     because the output is laid out by expert. This is the only reading under
 *     which the output is a permutation of the input.
 *   - A count of 0 is an empty segment (the page asks for counts > 0; zero is
 *     accepted because it is well defined and costs nothing). A negative count
 *     or a sum other than A is an error and nothing is written.
 *   - cumsum mode is the inclusive running sum over experts (last entry = A).
 *   - Scatter form: idx[SrcOffset + k] = DstOffset + k.
 *
 * oracle_reroute_inverse is not on the page: it is the same formulas read
 * backwards (the expert-major rows return to rank-major order, as a combine
 * step needs): out_X[SrcOffset + k] = in_X[DstOffset + k], with the same
 * offsets, the same expert_token_num, and idx in the same two forms relative
 * to its own input and output (gather: idx[out row] = in row).
 */
#include "oracle.h"

#include <stdlib.h>
#include <string.h>

static int64_t count_at(const void* counts, int counts_is_i64, int64_t cell) {
  if (counts_is_i64) return ((const int64_t*)counts)[cell];
  return (int64_t)((const int32_t*)counts)[cell];
}

/* Constraint ("约束说明"): no negative count, and the counts add up to A. */
static int counts_valid(const void* counts, int counts_is_i64, int64_t N, int64_t E, int64_t A) {
  int64_t total = 0;
  for (int64_t cell = 0; cell < N * E; ++cell) {
    int64_t c = count_at(counts, counts_is_i64, cell);
    if (c < 0) return ORACLE_BAD_COUNTS;
    total += c;
  }
  if (total != A) return ORACLE_BAD_COUNTS;
  return ORACLE_OK;
}

/* expert_token_num ("参数说明"): tokens per expert (a column sum of the count
 * matrix), or in cumsum mode the running total up to and including that
 * expert. */
static void expert_token_num(const void* counts, int counts_is_i64, int64_t N, int64_t E,
                             int64_t etn_type, void* out_etn) {
  int64_t running = 0;
  for (int64_t j = 0; j < E; ++j) {
    int64_t per_expert = 0;
    for (int64_t i = 0; i < N; ++i) per_expert += count_at(counts, counts_is_i64, i * E + j);
    running += per_expert;
    int64_t value = (etn_type == 1) ? per_expert : running;
    if (counts_is_i64)
      ((int64_t*)out_etn)[j] = value;
    else
      ((int32_t*)out_etn)[j] = (int32_t)value;
  }
}

int oracle_offsets(const void* counts, int counts_is_i64, int64_t N, int64_t E,
                   int64_t* src_off, int64_t* dst_off) {
  if (N < 0 || E < 0) return ORACLE_BAD_ARGS;
  if (N * E > 0 && (counts == NULL || src_off == NULL || dst_off == NULL)) return ORACLE_BAD_ARGS;

  for (int64_t cell = 0; cell < N * E; ++cell)
    if (count_at(counts, counts_is_i64, cell) < 0) return ORACLE_BAD_COUNTS;

  /* SrcOffset: walk the cells rank by rank, and within a rank expert by expert
   * (row-major), adding up the tokens seen so far. */
  int64_t seen = 0;
  for (int64_t i = 0; i < N; ++i) {
    for (int64_t j = 0; j < E; ++j) {
      src_off[i * E + j] = seen;
      seen += count_at(counts, counts_is_i64, i * E + j);
    }
  }

  /* DstOffset: walk the cells expert by expert, and within an expert rank by
   * rank (column-major), adding up the tokens seen so far. */
  seen = 0;
  for (int64_t j = 0; j < E; ++j) {
    for (int64_t i = 0; i < N; ++i) {
      dst_off[i * E + j] = seen;
      seen += count_at(counts, counts_is_i64, i * E + j);
    }
  }
  return ORACLE_OK;
}

int oracle_reroute(const uint8_t* tokens, int64_t A, int64_t token_row_bytes,
                   const void* counts, int counts_is_i64, int64_t N, int64_t E,
                   const uint8_t* scales, int64_t scale_row_bytes,
                   const float* weight,
                   int64_t etn_type, int64_t idx_type,
                   uint8_t* out_tokens, uint8_t* out_scales, int32_t* out_idx,
                   void* out_etn, float* out_weight) {
  if (A < 0 || N < 0 || E < 0 || token_row_bytes < 0) return ORACLE_BAD_ARGS;
  if (A > INT32_MAX) return ORACLE_BAD_ARGS; /* permute_token_idx is int32 */
  if (etn_type != 0 && etn_type != 1) return ORACLE_BAD_ARGS;
  if (idx_type != 0 && idx_type != 1) return ORACLE_BAD_ARGS;
  if (scales != NULL && (out_scales == NULL || scale_row_bytes < 0)) return ORACLE_BAD_ARGS;
  if (weight != NULL && out_weight == NULL) return ORACLE_BAD_ARGS;
  if (A > 0 && (tokens == NULL || out_tokens == NULL || out_idx == NULL)) return ORACLE_BAD_ARGS;
  if (E > 0 && out_etn == NULL) return ORACLE_BAD_ARGS;
  if (N * E > 0 && counts == NULL) return ORACLE_BAD_ARGS;

  if (counts_valid(counts, counts_is_i64, N, E, A) != ORACLE_OK) return ORACLE_BAD_COUNTS;

  /* The offsets of every cell, by the two double sums. */
  int64_t cells = N * E;
  int64_t* src_off = (int64_t*)malloc((size_t)(cells > 0 ? cells : 1) * sizeof(int64_t));
  int64_t* dst_off = (int64_t*)malloc((size_t)(cells > 0 ? cells : 1) * sizeof(int64_t));
  if (src_off == NULL || dst_off == NULL) {
    free(src_off);
    free(dst_off);
    return ORACLE_BAD_ARGS;
  }
  int rc = oracle_offsets(counts, counts_is_i64, N, E, src_off, dst_off);
  if (rc != ORACLE_OK) {
    free(src_off);
    free(dst_off);
    return rc;
  }

  /* Move every token of every cell: row SrcOffset+k of each input goes to row
   * DstOffset+k of the matching output, for k over the cell's tokens. */
  for (int64_t i = 0; i < N; ++i) {
    for (int64_t j = 0; j < E; ++j) {
      int64_t cur_tokens = count_at(counts, counts_is_i64, i * E + j);
      int64_t src = src_off[i * E + j];
      int64_t dst = dst_off[i * E + j];
      for (int64_t k = 0; k < cur_tokens; ++k) {
        memcpy(out_tokens + (dst + k) * token_row_bytes,
               tokens + (src + k) * token_row_bytes, (size_t)token_row_bytes);
        if (scales != NULL)
          memcpy(out_scales + (dst + k) * scale_row_bytes,
                 scales + (src + k) * scale_row_bytes, (size_t)scale_row_bytes);
        if (weight != NULL)
          memcpy(out_weight + (dst + k), weight + (src + k), sizeof(float));
        /* permute_token_idx: each token's index in the original layout. */
        if (idx_type == 0)
          out_idx[dst + k] = (int32_t)(src + k);  /* gather: out row -> in row */
        else
          out_idx[src + k] = (int32_t)(dst + k);  /* scatter: in row -> out row */
      }
    }
  }

  expert_token_num(counts, counts_is_i64, N, E, etn_type, out_etn);
  free(src_off);
  free(dst_off);
  return ORACLE_OK;
}

int oracle_reroute_inverse(const uint8_t* rows, int64_t A, int64_t row_bytes,
                           const void* counts, int counts_is_i64, int64_t N, int64_t E,
                           const uint8_t* scales, int64_t scale_row_bytes,
                           const float* weight,
                           int64_t etn_type, int64_t idx_type,
                           uint8_t* out_rows, uint8_t* out_scales, int32_t* out_idx,
                           void* out_etn, float* out_weight) {
  if (A < 0 || N < 0 || E < 0 || row_bytes < 0) return ORACLE_BAD_ARGS;
  if (A > INT32_MAX) return ORACLE_BAD_ARGS;
  if (etn_type != 0 && etn_type != 1) return ORACLE_BAD_ARGS;
  if (idx_type != 0 && idx_type != 1) return ORACLE_BAD_ARGS;
  if (scales != NULL && (out_scales == NULL || scale_row_bytes < 0)) return ORACLE_BAD_ARGS;
  if (weight != NULL && out_weight == NULL) return ORACLE_BAD_ARGS;
  if (A > 0 && (rows == NULL || out_rows == NULL || out_idx == NULL)) return ORACLE_BAD_ARGS;
  if (E > 0 && out_etn == NULL) return ORACLE_BAD_ARGS;
  if (N * E > 0 && counts == NULL) return ORACLE_BAD_ARGS;

  if (counts_valid(counts, counts_is_i64, N, E, A) != ORACLE_OK) return ORACLE_BAD_COUNTS;

  int64_t cells = N * E;
  int64_t* src_off = (int64_t*)malloc((size_t)(cells > 0 ? cells : 1) * sizeof(int64_t));
  int64_t* dst_off = (int64_t*)malloc((size_t)(cells > 0 ? cells : 1) * sizeof(int64_t));
  if (src_off == NULL || dst_off == NULL) {
    free(src_off);
    free(dst_off);
    return ORACLE_BAD_ARGS;
  }
  int rc = oracle_offsets(counts, counts_is_i64, N, E, src_off, dst_off);
  if (rc != ORACLE_OK) {
    free(src_off);
    free(dst_off);
    return rc;
  }

  /* Every cell's segment goes back: expert-major row DstOffset+k of the input
   * becomes rank-major row SrcOffset+k of the output. */
  for (int64_t i = 0; i < N; ++i) {
    for (int64_t j = 0; j < E; ++j) {
      int64_t cur_tokens = count_at(counts, counts_is_i64, i * E + j);
      int64_t src = src_off[i * E + j];
      int64_t dst = dst_off[i * E + j];
      for (int64_t k = 0; k < cur_tokens; ++k) {
        int64_t rank_row = src + k;    /* output row (rank-major) */
        int64_t expert_row = dst + k;  /* input row (expert-major) */
        memcpy(out_rows + rank_row * row_bytes, rows + expert_row * row_bytes, (size_t)row_bytes);
        if (scales != NULL)
          memcpy(out_scales + rank_row * scale_row_bytes,
                 scales + expert_row * scale_row_bytes, (size_t)scale_row_bytes);
        if (weight != NULL) memcpy(out_weight + rank_row, weight + expert_row, sizeof(float));
        if (idx_type == 0)
          out_idx[rank_row] = (int32_t)expert_row;  /* gather: out row -> in row */
        else
          out_idx[expert_row] = (int32_t)rank_row;  /* scatter: in row -> out row */
      }
    }
  }

  /* expert_token_num is the same as the forward operator's. */
  expert_token_num(counts, counts_is_i64, N, E, etn_type, out_etn);
  free(src_off);
  free(dst_off);
  return ORACLE_OK;
}
