/*
 * moe_rerouting_v2.h -- C ABI of the MoE re-routing operator (MoeReRoutingV2)
 * for AMD Instinct MI355X (gfx950).
 *
 * What the operator computes (page "CANN ops-transformer MoeReRoutingV2",
 * nlpx.cn article, sections "功能说明", "计算公式" and "参数说明"):
 * after the expert-parallel all-to-all a device holds tokens[A, H] ordered by
 * source rank, and within a rank by local expert. The count matrix
 * expert_token_num_per_rank[N, E] says how many of those rows came from rank
 * i for expert j. The operator reorders the rows by expert, and within an
 * expert by rank:
 *     permute_tokens[DstOffset(i,j) + k] = tokens[SrcOffset(i,j) + k],
 *     0 <= k < counts[i][j],
 * where SrcOffset(i,j) is the number of rows in the cells before (i,j) in
 * row-major (rank, expert) order and DstOffset(i,j) the number of rows in the
 * cells before (i,j) in column-major (expert, rank) order. per_token_scales
 * and expert_topk_weight rows move by the same offsets. The operator also
 * writes permute_token_idx (gather or scatter form) and expert_token_num (per
 * expert counts, or their running sum).
 *
 * With direction = MRR_INVERSE the same call runs the moves backwards, which
 * the article does not define but its formulas fix: the rows arrive in
 * expert-major order (as the forward call writes them, e.g. after the expert
 * computation) and return to rank-major order before the combine step,
 *     permute_tokens[SrcOffset(i,j) + k] = tokens[DstOffset(i,j) + k],
 * with scales and weights alike, permute_token_idx relative to this call's
 * own input and output (gather: row d of the output came from input row
 * idx[d]), and the same expert_token_num.
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a caller-owned DEVICE pointer on the current HIP
 *     device; the library never frees, keeps or allocates caller memory, and
 *     never allocates device memory of its own on the call path.
 *   - Tensors are dense, row-major, with no padding between rows.
 *   - Host-detectable errors are returned before anything is launched, and
 *     then no output is touched.
 *   - The launching calls are asynchronous and ordered on `stream` (a
 *     hipStream_t; NULL is the default stream). Errors found on the device
 *     (bad count values) are recorded in the workspace, the kernels then
 *     write no output, and mrr_get_device_status() reports them.
 *   - In-place operation is not supported: inputs, outputs and the workspace
 *     must not overlap.
 *   - Calls sharing one workspace must be ordered on one stream; distinct
 *     workspaces may be used concurrently from several threads.
 */
#ifndef MOE_REROUTING_V2_H
#define MOE_REROUTING_V2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* a hipStream_t is a struct ihipStream_t* */

/* Return codes. */
typedef enum mrr_status {
  MRR_SUCCESS = 0,
  MRR_ERROR_INVALID_VALUE = 1,      /* NULL where a pointer is required, attribute not 0/1,
                                       weight input/output not paired, overlapping buffers */
  MRR_ERROR_INVALID_SHAPE = 2,      /* A, H, N, E or a scale shape outside the contract */
  MRR_ERROR_UNSUPPORTED_DTYPE = 3,  /* a dtype code not allowed for that tensor */
  MRR_ERROR_MISALIGNED = 4,         /* a typed pointer not aligned to its element size,
                                       or a workspace not aligned to 16 bytes */
  MRR_ERROR_WORKSPACE_TOO_SMALL = 5,
  MRR_ERROR_BAD_COUNTS = 6,         /* found on the device: a negative count, a count above
                                       INT32_MAX, or counts not summing to A */
  MRR_ERROR_HIP = 7                 /* a HIP runtime call failed */
} mrr_status;

/* Element types. Token types follow the operator's prototype (REG_OP section
 * of the article); only the element width matters to the operator, which
 * moves bytes: 16 bits (F16, BF16), 8 bits (I8, F8_E5M2, F8_E4M3FN, HIF8) or
 * 4 bits (F4_E2M1, F4_E1M2, two per byte, low nibble first as stored). */
typedef enum mrr_dtype {
  MRR_F16 = 0,
  MRR_BF16 = 1,
  MRR_I8 = 2,
  MRR_F8_E5M2 = 3,
  MRR_F8_E4M3FN = 4,
  MRR_HIF8 = 5,
  MRR_F4_E2M1 = 6,
  MRR_F4_E1M2 = 7,
  MRR_I32 = 8,
  MRR_I64 = 9,
  MRR_F32 = 10,
  MRR_F8_E8M0 = 11
} mrr_dtype;

/*
 * Arguments of one call, in the order of the operator's prototype: four
 * inputs, five outputs, two attributes (REG_OP(MoeReRoutingV2) section and
 * the parameter table "参数说明" of the article).
 */
typedef struct mrr_args {
  /* tokens [A, H]: row r occupies H*bits/8 bytes (fp4: H even, H/2 bytes). */
  const void* tokens;
  int32_t tokens_dtype;            /* MRR_F16 .. MRR_F4_E1M2 */
  int64_t A;                       /* rows; 0 <= A <= INT32_MAX (the index is int32) */
  int64_t H;                       /* logical elements per row; 0 < H < 16384 */

  /* expert_token_num_per_rank [N, E]: counts[i*E + j] = rows from rank i for
   * local expert j. Values must be >= 0 (0 = empty segment) and sum to A;
   * this is checked on the device. N, E >= 0; N*E == 0 requires A == 0. */
  const void* expert_token_num_per_rank;
  int32_t counts_dtype;            /* MRR_I32 or MRR_I64 */
  int64_t N;
  int64_t E;

  /* per_token_scales, optional (NULL = absent). Shapes:
   *   MRR_F32,     ndim 1: [A]
   *   MRR_F32,     ndim 2: [A, S], S >= 1
   *   MRR_F8_E8M0, ndim 3: [A, ceil(H/64), 2]  (MX block scales of the tokens) */
  const void* per_token_scales;
  int32_t scales_dtype;
  int32_t scales_ndim;
  int64_t scales_dims[3];

  /* expert_topk_weight [A, 1] fp32, optional (NULL = absent). */
  const float* expert_topk_weight;

  /* Outputs. */
  void* permute_tokens;            /* [A, H], tokens' dtype */
  void* permute_per_token_scales;  /* scales' shape and dtype; may be NULL when the scales
                                      are absent (the output then has no meaning and is
                                      never written) */
  int32_t* permute_token_idx;      /* [A] int32 */
  void* expert_token_num;          /* [E], counts' dtype */
  float* permute_topk_weight;      /* [A, 1] fp32; must be NULL exactly when
                                      expert_topk_weight is NULL */

  /* Attributes. */
  int64_t expert_token_num_type;   /* 1 (default): rows per expert; 0: inclusive running
                                      sum of rows per expert (last entry = A) */
  int64_t idx_type;                /* 0 (default): gather, tokens[idx[d]] lands at row d;
                                      1: scatter, tokens[s] lands at row idx[s] */
  int64_t direction;               /* MRR_FORWARD (0, default): rank-major -> expert-major;
                                      MRR_INVERSE (1): expert-major -> rank-major */
} mrr_args;

/* mrr_args.direction */
enum { MRR_FORWARD = 0, MRR_INVERSE = 1 };

/*
 * Bytes of device workspace a call with A rows and an N x E count matrix
 * needs: a 256-byte header (validity status of the counts), the per-cell
 * offsets (two int32 per cell) and the source row of every output row (one
 * int32 per row), each part rounded up to 256 bytes. Returns 0 when A, N or
 * E is negative, A > INT32_MAX, or N*E is too large for 32-bit cell indices.
 * The caller allocates it (no zeroing needed); it may be reused by calls
 * ordered on one stream.
 * (A convention of this library: the article's operator keeps its offsets in
 * per-core tiling data instead. The size depends on A, not only on N and E,
 * because the gather reads the source row of every output row from the
 * workspace.)
 */
size_t mrr_workspace_size(int64_t A, int64_t N, int64_t E);

/*
 * The exact checks the launching calls make before they launch anything,
 * on the host only: no HIP call is made, so this runs without a GPU. The
 * pointers are compared and tested for alignment, never dereferenced.
 * Returns MRR_SUCCESS or the first error found.
 * The checks are the article's contract (parameter table "参数说明", the
 * constraints "约束说明" and the InferShape rules: dtypes, 0 < H < 16384,
 * shapes of the optional inputs, the pairing of the top-k weight input and
 * output) plus this library's own: pointer alignment, no overlap between any
 * output and any other buffer, and the workspace's size. The workspace
 * pointer is an argument because the alignment and overlap checks need it.
 */
mrr_status mrr_validate(const mrr_args* args, const void* workspace, size_t workspace_bytes);

/* How a call with these arguments is launched (filled by mrr_describe_plan). */
typedef struct mrr_plan_info {
  int32_t fused;                 /* what moe_rerouting_v2 launches: 1 = one kernel whose workgroups
                                    each recompute the offsets of the (small) count matrix in LDS
                                    or registers (small calls); 2 = one kernel of 64-lane
                                    workgroups (count matrices of at most 512 cells, token rows of
                                    16-byte vectors and at least 32 bytes, or of 17 bytes or more
                                    that are no multiple of 16 with both token buffers 16-byte
                                    aligned; short rows only from 2 MiB or 256 KiB of token rows
                                    where 1 applies): item waves of 256 output rows (64 with scale
                                    rows over 16 bytes), then one wave per 1 KiB of the input token
                                    rows, each computing the offsets it needs from the counts; 0 =
                                    the offsets kernel, then the gather kernel (the two-phase entry
                                    points always do that) */
  int32_t token_vec_bytes;       /* bytes per load/store of the token copy: 16, 8, 4, 2 or 1
                                    (16 also for rows that are no multiple of 16 bytes when the
                                    one-launch kernel or the stream gather moves them as aligned
                                    16-byte output blocks) */
  int32_t scale_vec_bytes;       /* the same for scale rows; 0 without scales */
  int32_t rows_per_workgroup;    /* adjacent rows per workgroup: input rows of the fused kernel,
                                    output rows of the row-workgroup gather */
  int32_t threads_per_workgroup;
  int64_t gather_workgroups;
  int64_t token_row_bytes;
  int64_t scale_row_bytes;
  int32_t scale_inline_bytes;    /* 16 or 4: scale rows move in pieces of that size together with
                                    the token rows; 0: in a separate pass after them */
  int64_t offsets_workgroups;    /* workgroups of moe_rerouting_v2_offsets(): several for larger
                                    count matrices (bands of ranks) or when the row map is
                                    written (one workgroup per 256, 512 or 1024 rows); 1 otherwise;
                                    0 when there are no cells */
  int32_t gather_kernel;         /* what moe_rerouting_v2_gather() launches: 1 = 64-lane
                                    workgroups, each moving 64 vectors of one output stream
                                    (token rows, scale rows, per-row items) with the row map
                                    the offsets phase wrote; 0 = workgroups of whole rows that
                                    search the offsets table */
  int64_t gather_launches;       /* kernel launches of the gather phase: 1, or more when its
                                    workgroups hold 2^32 or more threads in all (a launch holds
                                    at most 2^32 - 1), each piece taking the next workgroups;
                                    0 when A == 0 */
  int64_t one_launch_workgroups; /* workgroups of moe_rerouting_v2's single launch when fused is
                                    1 or 2; 0 otherwise */
} mrr_plan_info;

/*
 * Runs the same host checks as mrr_validate() and, on success, describes the
 * launch in *info. Host only, no HIP call. (A convention of this library.)
 */
mrr_status mrr_describe_plan(const mrr_args* args, const void* workspace, size_t workspace_bytes,
                             mrr_plan_info* info);

/*
 * The whole operator on `stream`, asynchronous (article "CANN ops-transformer
 * MoeReRoutingV2", section "计算公式": the two double sums and the moves of
 * tokens, per_token_scales and expert_topk_weight; section "参数说明": the
 * inputs, outputs and attributes of mrr_args, permute_token_idx in gather or
 * scatter form, expert_token_num as counts or their running sum). Depending on
 * the size of the call (see mrr_plan_info.fused) this launches either one
 * fused kernel, or moe_rerouting_v2_offsets() then moe_rerouting_v2_gather();
 * the results are identical. Host-detectable errors are returned before any
 * launch; count errors are found on the device (see mrr_get_device_status).
 */
mrr_status moe_rerouting_v2(const mrr_args* args, void* workspace, size_t workspace_bytes,
                            struct ihipStream_t* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture that may not call hipMalloc, tight serving loops, harnesses that
 * forbid allocation): moe_rerouting_v2 with no workspace argument. The library
 * uses its own scratch instead, a static device array of
 * MRR_NOALLOC_SCRATCH_BYTES on each GPU it runs on, held until the process
 * ends. Nothing is allocated or freed, by the library or by anything it calls.
 *   - A call fits when mrr_workspace_size(A, N, E) <= MRR_NOALLOC_SCRATCH_BYTES
 *     (for instance A up to about 2 million rows with a 16 x 16 count matrix,
 *     or 65536 rows with 256 x 64); larger calls return
 *     MRR_ERROR_WORKSPACE_TOO_SMALL before any launch and touch no output.
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents. Calls on one GPU must therefore be ordered (one stream,
 *     or streams synchronized with each other): calls that overlap in time on
 *     one GPU race, and their results are undefined.
 *   - The results, the checks and their error codes are moe_rerouting_v2's.
 *     Count errors found on the device leave the outputs unwritten as there;
 *     this entry point offers no status readback (a caller that needs it uses
 *     moe_rerouting_v2 with its own workspace and mrr_get_device_status).
 *   - The first call on a device looks up the scratch's address there (a HIP
 *     query, no allocation).
 */
#define MRR_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
mrr_status moe_rerouting_v2_noalloc(const mrr_args* args, struct ihipStream_t* stream);

/*
 * First phase alone (article, "计算公式": the two double sums): scans the
 * count matrix (see mrr_plan_info.offsets_workgroups) and writes into the
 * workspace the validity status and what the second phase reads: for count
 * matrices of at most 1024 cells or up to 2^17 cells with at most 1024
 * experts, the row map (the input row of every output row); otherwise the
 * SrcOffset and DstOffset table. Writes expert_token_num into
 * args->expert_token_num (only when the counts are valid).
 */
mrr_status moe_rerouting_v2_offsets(const mrr_args* args, void* workspace, size_t workspace_bytes,
                                    struct ihipStream_t* stream);

/*
 * Second phase alone (article, "计算公式": the three moves, and "参数说明":
 * permute_token_idx): moves the token rows, scale rows and weights and writes
 * permute_token_idx, from the row map or the table (mrr_plan_info.
 * gather_kernel) that a preceding moe_rerouting_v2_offsets() call with the
 * same arguments wrote into `workspace` on the same stream.
 * If that call found bad counts, or the workspace holds no row map or table
 * for this A, N, E and direction (for instance after a fused moe_rerouting_v2
 * call, which builds neither), nothing is written.
 */
mrr_status moe_rerouting_v2_gather(const mrr_args* args, void* workspace, size_t workspace_bytes,
                                   struct ihipStream_t* stream);

/*
 * Waits for `stream`, then reads the status the last call (whole or offsets
 * phase) left in `workspace`: MRR_SUCCESS (the counts were valid),
 * MRR_ERROR_BAD_COUNTS, MRR_ERROR_INVALID_VALUE if the workspace holds no
 * status (no call ran on it), or MRR_ERROR_HIP if the copy or the wait fails.
 * Synchronizing: not for use inside a hot loop. (The verdict on the article's
 * constraints of "约束说明" — counts summing to A, no negative count — which
 * only the device can check; how it is reported is this library's
 * convention.)
 */
mrr_status mrr_get_device_status(const void* workspace, struct ihipStream_t* stream);

/* A static, human-readable name of a status code. (A convention of this
 * library; the article defines no error codes.) */
const char* mrr_status_string(mrr_status status);

/* The identity of the sources this library was built from: 16 hex digits of
 * a SHA-256 over the source files, fixed at build time, in static storage.
 * (A convention of this library: loaders compare it with the sources they
 * ship with and refuse a library built from others.) */
const char* mrr_source_hash(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_REROUTING_V2_H */
