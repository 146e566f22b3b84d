/*
 * uep.h -- C-ABI of libuep.so, the MI355X (gfx950) real-time MoE expert
 * load-balancing path: load matrix -> quota solve -> local-first reroute and
 * token assignment -> permute -> redundant-slot staging, plus Waterfill
 * shared-expert placement and the LPLB min-max replica split.
 *
 * Sources (the pages the method comes from):
 *   [UEP]  "300 微秒调平 MoE 专家负载！小红书 UltraEP 逼近 94.3% 理想训推吞吐"
 *          (UltraEP technical article, m.163.com)
 *   [BLOG] "Improving DeepEP MoE Load Balance in SGLang with Waterfill and LPLB"
 *          (papercache notes of the lmsys blog)
 *
 * Conventions shared by every call
 *   - Every array argument is a DEVICE pointer owned by the caller, except where a
 *     call says "host".  The library never allocates, frees or synchronises on
 *     these calls; work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and ordered with the caller's other work on that stream.
 *   - Integer arrays are int32, row-major, with the shapes given below.
 *     bf16 data is passed as raw uint16 bits and moved bit for bit.
 *   - Geometry: R virtual EP ranks, T tokens per rank, K routing slots per token,
 *     E logical experts, home(e) = e / (E / R) for the routed experts.  A physical
 *     instance id is i = r * inst_per_rank + j (rank r, local slot j); instance
 *     tables `inst_expert[I]` give each instance's logical expert or -1.
 *   - A top-k id of -1 is an empty routing slot (a padded or absent token).  It is
 *     not counted and gets bucket position, instance and row -1.
 *   - Return value: uep_status.  Argument checks run on the host before anything
 *     is enqueued; on an error nothing is enqueued.  UEP_EHIP reports a launch
 *     failure (hipGetLastError).
 *   - Content errors (bad ids, quotas that do not match the load, ...) are found
 *     on the device and OR-ed as UEP_ERR_* bits into the optional device word
 *     `err` (may be NULL).  The caller clears it beforehand and reads it after its
 *     own synchronisation.  Outputs are unspecified when a bit is set.
 *   - Calls are stateless and re-entrant.  Calls that overlap on one stream-less
 *     set of buffers race like any other kernels writing the same memory.
 *   - Limits: R <= 64, E <= 4096, K <= 64, R*T*K < 2^31, total load < 2^31,
 *     hidden size H <= 2^29 for the row moves (a row is one store span).
 */
#ifndef UEP_H
#define UEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t uep_status;
enum {
  UEP_OK = 0,
  UEP_EINVAL = 1,      /* null pointer, negative size, r_begin/r_end out of range */
  UEP_EGEOM = 2,       /* unsupported geometry (limits above, E % R != 0, H % 8 != 0 ...) */
  UEP_EWORKSPACE = 3,  /* workspace missing or smaller than the *_workspace_size query */
  UEP_EHIP = 4         /* a kernel launch or HIP runtime call failed */
};

/* device-side content error bits */
enum {
  UEP_ERR_ID_RANGE = 1,     /* a top-k id outside [-1, E) */
  UEP_ERR_DUP_ID = 2,       /* an expert twice in one token's top-k */
  UEP_ERR_QUOTA_SUM = 4,    /* an expert's instance quotas do not sum to its load */
  UEP_ERR_INST_DUP = 8,     /* two instances of one expert on one rank */
  UEP_ERR_BAD_QUOTA = 16,   /* negative quota, or quota on an unused instance */
  UEP_ERR_COVER = 32,       /* a bucket position not covered by the transfer plan */
  UEP_ERR_LP = 64,          /* LPLB: an expert with load but no instance */
  UEP_ERR_ROW_RANGE = 128   /* a dest_row entry outside [-1, out_rows) */
};

/* Library version string and a static text for a status code (host). */
const char* uep_version(void);
const char* uep_status_string(uep_status s);

/* ------------------------------------------------------------------------- *
 * uep_device_copy -- plain device-to-device copy, the measured HBM reference line.
 * Not a step of the balancing path: it is the "achievable bandwidth" kernel against
 * which the permute and staging kernels are read, and the known-size kernel that
 * calibrates hardware byte counters.  Each workgroup copies 16 KiB with 16-byte
 * vector loads, all issued before its stores.
 *
 *   src   [bytes]  in   device memory, 16-byte aligned
 *   dst   [bytes]  out  device memory, 16-byte aligned, not overlapping src
 *   bytes               multiple of 16; 0 is a no-op
 * Returns UEP_EINVAL for null pointers or negative size, UEP_EGEOM for misaligned
 * pointers or a size that is not a multiple of 16.
 * ------------------------------------------------------------------------- */
uep_status uep_device_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * uep_device_fill -- writes a 32-bit pattern over device memory.  Not a step of the
 * balancing path: the write-only HBM reference line (the permute and staging
 * streams are mostly writes), and a fill kernel for callers that clear buffers
 * inside a captured graph and want no memset node there.  Same workgroup shape as
 * uep_device_copy (16 KiB per workgroup, 16-byte vector stores).
 *
 *   dst    [bytes]  out  device memory, 16-byte aligned
 *   bytes                multiple of 16; 0 is a no-op
 *   value                the 32-bit word written at every 4-byte offset
 * Returns UEP_EINVAL for a null pointer or negative size, UEP_EGEOM for a misaligned
 * pointer or a size that is not a multiple of 16.
 * ------------------------------------------------------------------------- */
uep_status uep_device_fill(void* dst, int64_t bytes, uint32_t value, void* stream);

/* ------------------------------------------------------------------------- *
 * uep_load_matrix -- the global load matrix of one layer.
 * [UEP] section "在 Gate 之后获取当前层真实负载" (real load after Gate): once the Gate
 * has run, every expert's exact token count for this microbatch and layer is known;
 * the routing metadata of the whole EP group forms the global load matrix.
 *
 *   topk_ids   [R][T][K]  in   expert ids in [-1, E), distinct within a token
 *   counts     [R][E]     out  counts[r][e] = number of (t, k) on rank r routed to e
 *   bucket_pos [R][T][K]  out  number of tokens t' < t on rank r whose top-k holds
 *                              the same expert (stable position in its bucket);
 *                              may be NULL: then only counts are computed (a layer
 *                              that needs the loads but no positions, e.g. the routed
 *                              loads Waterfill starts from), and duplicate ids are
 *                              not checked
 *   err                   out  optional; UEP_ERR_ID_RANGE, UEP_ERR_DUP_ID
 *   ws, ws_bytes               device workspace of uep_load_matrix_workspace_size()
 * ------------------------------------------------------------------------- */
size_t uep_load_matrix_workspace_size(int32_t R, int32_t T, int32_t K, int32_t E);
uep_status uep_load_matrix(const int32_t* topk_ids, int32_t R, int32_t T, int32_t K,
                           int32_t E, int32_t* counts, int32_t* bucket_pos, int32_t* err,
                           void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * uep_load_matrix_noalloc -- uep_load_matrix without a caller workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, outputs and errors as
 * uep_load_matrix minus ws / ws_bytes; the chunk histograms live in an 8 MiB array the
 * library holds on each GPU it runs on, until the process ends.  Geometries whose
 * uep_load_matrix_workspace_size() exceeds 8 MiB return UEP_EWORKSPACE (the layers
 * here need 0.5-5 MiB).  All calls on one GPU share that array: calls that overlap on
 * one GPU (several streams or host threads) race and must be ordered by the caller.
 * Allocates and frees nothing; the first call on a device looks up the array's device
 * address once (UEP_EHIP if that fails).
 * ------------------------------------------------------------------------- */
uep_status uep_load_matrix_noalloc(const int32_t* topk_ids, int32_t R, int32_t T, int32_t K,
                                   int32_t E, int32_t* counts, int32_t* bucket_pos,
                                   int32_t* err, void* stream);

/* ------------------------------------------------------------------------- *
 * uep_solve_quota -- joint replica placement and quota solve.
 * [UEP] section "Quota 同时决定专家副本与 token 分流": a quota is the token load an
 * expert instance receives after rerouting; each search step may instantiate a
 * replica and updates the quota distribution; at most S redundant slots per rank,
 * no logical expert twice on one rank, and a new replica gets at least q_min
 * tokens.  Section "共享冗余 slot 管理动态专家副本": mains never move.
 * Every caller with the same counts gets the same plan (deterministic, ties to
 * the lowest index).  Search ("fill to the waterline", T* = ceil(sum c / R),
 * every step opens one replica, so at most R*S steps):
 *   1. h = the most loaded rank; stop if L_h <= T*, or if L_h - T* < q_min.
 *   2. Plain step: h's mains with quota left, quota descending (id ascending on
 *      ties), each tried in turn: a new replica in the lowest free slot of the
 *      least loaded rank t with L_t < T*, a free slot and no copy of the expert,
 *      taking d = min(q_main, L_h - T*, T* - L_t) if d >= q_min.
 *   3. Relay, when no main of h can move (the quota-distribution update): for h's
 *      mains in the same order, the lowest-index rank x != h with L_x >= T*, a free
 *      slot and no copy of the donor e, one of whose mains f (quota left) has a
 *      replica on a rank y with L_y < T*.  d2 = min(q_f, T* - L_y) moves from f's
 *      main to y's replica, then e opens on x with d = min(q_e, L_h - T*,
 *      T* - (L_x - d2)) if d >= q_min.  Such an x sits exactly at T* and has one
 *      such (f, y) only (a lemma of the search), so no further order applies.
 *   4. Neither moves: stop (stats[3] = 1).
 * No rank ever rises above T*; h's excess falls every step.
 *
 *   counts      [R][E]           in   load matrix (E % R == 0, E_loc = E / R)
 *   S, q_min                          redundant slots per rank (0..8), minimum quota
 *   slot_expert [R][S]           out  expert held by each slot, -1 if empty
 *   inst_expert [R*(E_loc+S)]    out  instance table: j < E_loc main of r*E_loc + j,
 *                                     j >= E_loc slot j - E_loc
 *   inst_quota  [R*(E_loc+S)]    out  tokens each instance takes
 *   rank_load   [R]              out  load per rank after the plan
 *   stats       [4]              out  {replicas placed, steps, T*, 1 if stopped early}
 * ------------------------------------------------------------------------- */
uep_status uep_solve_quota(const int32_t* counts, int32_t R, int32_t E, int32_t S,
                           int32_t q_min, int32_t* slot_expert, int32_t* inst_expert,
                           int32_t* inst_quota, int32_t* rank_load, int32_t* stats,
                           void* stream);

/* ------------------------------------------------------------------------- *
 * uep_identity_quota -- quotas when every expert has exactly one instance
 * (used with the Waterfill layout of [BLOG] section "共享专家融合作为启用机制",
 * where each rank has one shared-expert slot next to its routed experts).
 *
 *   counts      [R][E]     in   R <= 64
 *   inst_expert [n_inst]   in   each expert at most once
 *   inst_quota  [n_inst]   out  total load of the instance's expert (0 if unused)
 * Returns UEP_EINVAL for null pointers or non-positive sizes, UEP_EGEOM for R > 64.
 * ------------------------------------------------------------------------- */
uep_status uep_identity_quota(const int32_t* counts, int32_t R, int32_t E, int32_t n_inst,
                              const int32_t* inst_expert, int32_t* inst_quota, void* stream);

/* ------------------------------------------------------------------------- *
 * uep_reroute_assign -- local-first reroute and per-token realisation.
 * [UEP] section "Quota 同时决定专家副本与 token 分流": tokens first use the instance of
 * their expert on their own rank; what the local quota cannot take goes to remote
 * instances by their remaining quota; the aggregate quotas are then realised per
 * token.  Remote fill = interval overlap: residual demands laid end to end in
 * ascending source rank against remaining capacities in ascending instance id.
 * Dispatch layout: instance blocks in instance-id order; inside a block source
 * rank ascending, then token ascending.  The tokens of (r, e) in token order fill
 * the local instance first, then the remote instances in ascending id.
 *
 *   counts, topk_ids, bucket_pos      in   from uep_load_matrix
 *   inst_per_rank, inst_expert[I],
 *   inst_quota[I]                     in   the plan; I = R * inst_per_rank
 *   r_begin, r_end                    in   per-token outputs only for sources in
 *                                          [r_begin, r_end); xfer/inst_offset always whole
 *   xfer        [R][I]                out  tokens of source r served by instance i
 *   inst_offset [I+1]                 out  first dispatch row of every instance
 *   dest_inst, dest_row [R][T][K]     out  instance and dispatch row of every pair
 *   err                               out  optional; QUOTA_SUM, INST_DUP, BAD_QUOTA, COVER
 *   ws, ws_bytes                           uep_reroute_workspace_size()
 * ------------------------------------------------------------------------- */
size_t uep_reroute_workspace_size(int32_t R, int32_t E, int32_t inst_per_rank);
uep_status uep_reroute_assign(const int32_t* counts, const int32_t* topk_ids,
                              const int32_t* bucket_pos, int32_t R, int32_t T, int32_t K,
                              int32_t E, int32_t inst_per_rank, const int32_t* inst_expert,
                              const int32_t* inst_quota, int32_t r_begin, int32_t r_end,
                              int32_t* xfer, int32_t* inst_offset, int32_t* dest_inst,
                              int32_t* dest_row, int32_t* err, void* ws, size_t ws_bytes,
                              void* stream);

/* ------------------------------------------------------------------------- *
 * uep_plan -- uep_load_matrix, uep_solve_quota and uep_reroute_assign of one layer in
 * one call ([UEP] sections "在 Gate 之后获取当前层真实负载" and "Quota 同时决定专家副本与
 * token 分流": the solve sits on the forward critical path between the Gate and the
 * dispatch).  Outputs and errors are those of the three calls, bit for bit; the solve
 * runs on the finished load matrix concurrently with the bucket-position ranking,
 * which it does not need.  Arguments are the union of the three calls' (S, q_min as
 * uep_solve_quota; r_begin / r_end restrict the assignment as in uep_reroute_assign;
 * inst_per_rank = E / R + S); ws is one workspace of uep_plan_workspace_size() bytes.
 * Geometries off the ranking fast path (E > 1024 or K > 16) run the three calls in
 * sequence.
 * ------------------------------------------------------------------------- */
size_t uep_plan_workspace_size(int32_t R, int32_t T, int32_t K, int32_t E, int32_t S);
uep_status uep_plan(const int32_t* topk_ids, int32_t R, int32_t T, int32_t K, int32_t E,
                    int32_t S, int32_t q_min, int32_t r_begin, int32_t r_end, int32_t* counts,
                    int32_t* bucket_pos, int32_t* slot_expert, int32_t* inst_expert,
                    int32_t* inst_quota, int32_t* rank_load, int32_t* stats, int32_t* xfer,
                    int32_t* inst_offset, int32_t* dest_inst, int32_t* dest_row, int32_t* err,
                    void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * uep_permute -- scatter token activations into the per-instance dispatch buffer.
 * [UEP] section "流式通信算子加速动态权重分发": once replica weights are in place,
 * token dispatch follows the reroute plan; this is its on-device permutation.
 * Each source row is read once and written to each of its K rows.
 *
 *   x        [R][T][H] bf16 bits  in   activations (H % 8 == 0, rows 16-byte aligned)
 *   dest_row [R][T][K]            in   from uep_reroute_assign (-1: no row)
 *   r_begin, r_end                     only sources in [r_begin, r_end) are moved
 *   out      [out_rows][H] bf16   out  dispatch buffer, out_rows >= the routed pairs
 *                                      (inst_offset[I] of uep_reroute_assign)
 *   row_src  [out_rows]           out  optional; (r*T + t)*K + k of the pair in each row
 *   err                           out  optional; UEP_ERR_ROW_RANGE: a dest_row entry
 *                                      outside [-1, out_rows), that pair is not moved
 * ------------------------------------------------------------------------- */
uep_status uep_permute(const uint16_t* x, const int32_t* dest_row, int32_t R, int32_t T,
                       int32_t K, int32_t H, int32_t r_begin, int32_t r_end, uint16_t* out,
                       int64_t out_rows, int32_t* row_src, int32_t* err, void* stream);

/* ------------------------------------------------------------------------- *
 * uep_combine -- expert outputs from the dispatch buffer back to token order.
 * [BLOG] section "背景知识与设计原则": DeepEP's combine brings each token's routed-
 * expert outputs back after dispatch; section "共享专家融合作为启用机制": a fused
 * shared slot is one more column of the same layout and goes through the same
 * combine.  The pages do not write it out; this is the standard MoE output with the
 * router weights as input:
 *   y[r][t] = bf16( sum_k w[r][t][k] * out[dest_row[r][t][k]] ),  slots with row -1 skipped,
 * each product and addition rounded to nearest even in fp32, k ascending from +0.0,
 * no fused multiply-add, then nearest-even rounding to bf16 (a NaN stays a NaN).
 *
 *   out      [out_rows][H] bf16   in   dispatch buffer (layout of uep_permute's out),
 *                                      16-byte aligned
 *   dest_row [R][T][K]            in   from uep_reroute_assign
 *   gate_w   [R][T][K] fp32       in   combine weights
 *   r_begin, r_end                     only tokens of ranks in [r_begin, r_end) are written
 *   y        [R][T][H] bf16 bits  out  16-byte aligned; other ranks' rows are untouched
 *   err                           out  optional; UEP_ERR_ROW_RANGE: a dest_row entry
 *                                      outside [-1, out_rows), taken as no row
 * Returns UEP_EINVAL / UEP_EGEOM like uep_permute.
 * ------------------------------------------------------------------------- */
uep_status uep_combine(const uint16_t* out, int64_t out_rows, const int32_t* dest_row,
                       const float* gate_w, int32_t R, int32_t T, int32_t K, int32_t H,
                       int32_t r_begin, int32_t r_end, uint16_t* y, int32_t* err,
                       void* stream);

/* ------------------------------------------------------------------------- *
 * uep_stage_replica_weights -- redundant-slot weight staging / gradient reduction.
 * [UEP] section "共享冗余 slot 管理动态专家副本": each rank has S fixed redundant slots
 * (weights + gradient buffer, no optimizer state) shared by every MoE layer; the
 * current layer's replica weights are written into them before dispatch.
 * Section "复用前向方案，完成权重恢复与梯度归约": backward reuses the forward plan,
 * writes the replica weights again, reduces replica gradients into the main's
 * gradient buffer and clears the redundant gradient buffer.
 * Section "流式通信算子加速动态权重分发": fixed-size tiles pulled by a persistent
 * kernel from a device-side task list derived from the plan.
 *
 *   mode = UEP_STAGE_WEIGHTS:     slot_w[r][s] = main_w[slot_expert[r][s]] (bit copy)
 *                                 for used slots of ranks in [r_begin, r_end)
 *   mode = UEP_STAGE_GRAD_REDUCE: for each expert e homed in [r_begin, r_end) with
 *                                 replicas on ranks r1 < r2 < ...:
 *                                 main_grad[e] = ((main_grad[e] + g_r1) + g_r2) + ...
 *                                 in fp32 round-to-nearest-even, then those slot
 *                                 gradients are set to +0.0
 *   slot_expert [R][S]                       in   from uep_solve_quota; entries outside
 *                                                 [0, E) are empty slots (skipped)
 *   main_w  [E][expert_elems] bf16, slot_w [R][S][expert_elems] bf16   (WEIGHTS)
 *   main_grad [E][expert_elems] f32, slot_grad [R][S][expert_elems] f32 (GRAD_REDUCE)
 *   expert_elems % 8 == 0; unused pointers of the other mode may be NULL.
 * ------------------------------------------------------------------------- */
enum { UEP_STAGE_WEIGHTS = 0, UEP_STAGE_GRAD_REDUCE = 1 };
uep_status uep_stage_replica_weights(int32_t mode, int32_t R, int32_t E, int32_t S,
                                     const int32_t* slot_expert, int32_t r_begin,
                                     int32_t r_end, const uint16_t* main_w, uint16_t* slot_w,
                                     float* main_grad, float* slot_grad,
                                     int64_t expert_elems, void* stream);

/* ------------------------------------------------------------------------- *
 * uep_waterfill -- place every token's shared-expert slot on a rank.
 * [BLOG] section "Waterfill算法执行步骤": L_r = routed load on rank r; N shared slots;
 * waterline H = ceil((sum_r L_r + N) / R); slack S_r = max(H - L_r, 0); each token's
 * shared slot goes to a candidate rank sampled in proportion to slack with a small
 * local preference; with zero slack everywhere, a clearly lighter candidate, else
 * the local rank.  Section "通信权衡与模式选择": candidates are the ranks the token
 * already visits plus its own rank (all_ranks = 0), or every rank of the EP group in
 * the all-rank mode (all_ranks != 0).
 * Constants: weights (2^p + 1) * S_r0 for the source rank r0 and 2^p * S_c for the
 * others (p = local_pref_shift, 0..8); draw = word 0 of Philox4x64-10 with counter
 * (r0*T + t, 0, 0, 0) and key (seed, layer), v = floor(draw * W / 2^64); the first
 * candidate (order: r0, then ascending rank) whose running weight exceeds v wins.
 * Zero total weight: the lightest candidate c with (2^p+1) L_c < 2^p L_r0, else r0.
 *
 *   counts     [R][E]      in   routed load matrix (E % R == 0)
 *   topk_ids   [R][T][K]   in
 *   batch_size [R]         in   live tokens per rank B_r <= T (N = sum B_r); tokens
 *                               t >= B_r get shared rank -1
 *   shared_rank[R][T]      out
 *   waterline  [1], slack [R], rank_load [R]  out  H, S_r, L_r
 *   ext_topk   [R][T][K+1] out  optional: top-k plus the column E + shared_rank
 *                               (-1 for absent tokens), i.e. the fused layout
 * ------------------------------------------------------------------------- */
uep_status uep_waterfill(const int32_t* counts, const int32_t* topk_ids,
                         const int32_t* batch_size, int32_t R, int32_t T, int32_t K,
                         int32_t E, uint64_t seed, uint64_t layer, int32_t local_pref_shift,
                         int32_t all_ranks, int32_t* shared_rank, int32_t* waterline,
                         int32_t* slack, int32_t* rank_load, int32_t* ext_topk, void* stream);

/* ------------------------------------------------------------------------- *
 * LPLB -- min-max split of replicated experts' load over their copies.
 * [BLOG] sections "线性规划（LP）公式化构建" and "决策变量与矩阵规模优化": minimise
 * the peak rank load M subject to, per rank, copy allocation + fixed single-copy
 * load + slack = M and, per replicated expert, the split summing to its true count;
 * the structural matrix depends only on the placement and is built once offline,
 * only the right-hand side changes per batch; a Big-M auxiliary column keeps the
 * system feasible and is driven to zero.  Section "从全局计数到LP求解的工程实现":
 * every rank solves the same LP on the GPU with an interior-point method into
 * preallocated buffers.  Section "从LP解决方案到Token调度": the split decides how a
 * replicated expert's tokens go to its copies (here: integer quotas by largest
 * remainder on rint(x * 256), then uep_reroute_assign).
 *
 * uep_lplb_prepare (offline): builds the LP structure from a HOST instance table
 *   inst_expert_host [R*inst_per_rank] (every expert with load needs >= 1 instance,
 *   at most one per rank) and copies it into the device buffer `lp` of
 *   uep_lplb_struct_size() bytes (synchronous copy; call outside the hot loop).
 * uep_lplb (per batch): fp32 Mehrotra predictor-corrector steps, at most `iters`.
 *   counts     [R][E]     in   load matrix
 *   iters                 in   iteration cap (0..200; the solve stops earlier once the
 *                              duality gap is at most 1e-4 of M; 30 is plenty)
 *   x          [n_copies] out  split per copy (token units, copies ordered by expert,
 *                              then instance id), normalised to sum to each count
 *   m          [1]        out  max rank load of that split
 *   inst_quota [I]        out  integer quotas for every instance
 *   stats      [4]        out  optional: {n_replicated, n_copies, iterations run, solve:
 *                              8 or 16 = block solve with lane groups of that size, 0 = dense}
 *   err                   out  optional; UEP_ERR_LP: an expert with load but no instance
 *                              or a column sum of 2^27 or more (the solve still runs), or
 *                              `lp` not a structure from uep_lplb_prepare (then nothing
 *                              else is written)
 * ------------------------------------------------------------------------- */
size_t uep_lplb_struct_size(int32_t R, int32_t E, int32_t inst_per_rank);
uep_status uep_lplb_prepare(const int32_t* inst_expert_host, int32_t R, int32_t E,
                            int32_t inst_per_rank, void* lp, size_t lp_bytes, void* stream);
uep_status uep_lplb(const int32_t* counts, const void* lp, int32_t iters, float* x, float* m,
                    int32_t* inst_quota, int32_t* stats, int32_t* err, void* stream);

/* ------------------------------------------------------------------------- *
 * uep_lplb_plan -- uep_load_matrix, uep_lplb and uep_reroute_assign of one layer in one
 * call ([BLOG] sections "从全局计数到LP求解的工程实现" and "从LP解决方案到Token调度": the LP
 * runs on the global counts, then its split decides the token dispatch).  Outputs and
 * errors are those of the three calls, bit for bit; the LP runs on the finished load
 * matrix concurrently with the bucket-position ranking, which it does not need.
 *
 *   topk_ids, R, T, K, E              in   as uep_load_matrix
 *   lp                                in   structure from uep_lplb_prepare for R, E and
 *                                          inst_per_rank; iters as uep_lplb
 *   inst_per_rank, inst_expert[I]     in   the static instance table the structure was
 *                                          built from (I = R * inst_per_rank)
 *   r_begin, r_end                    in   as uep_reroute_assign
 *   counts, bucket_pos                out  as uep_load_matrix
 *   x, m, inst_quota, stats           out  as uep_lplb
 *   xfer, inst_offset, dest_inst,
 *   dest_row                          out  as uep_reroute_assign
 *   err                               out  optional; every bit the three calls set
 *   ws, ws_bytes                           uep_lplb_plan_workspace_size()
 * Geometries off the ranking fast path (E > 1024 or K > 16) run the three calls in
 * sequence.
 * ------------------------------------------------------------------------- */
size_t uep_lplb_plan_workspace_size(int32_t R, int32_t T, int32_t K, int32_t E,
                                    int32_t inst_per_rank);
uep_status uep_lplb_plan(const int32_t* topk_ids, int32_t R, int32_t T, int32_t K, int32_t E,
                         const void* lp, int32_t inst_per_rank, const int32_t* inst_expert,
                         int32_t iters, int32_t r_begin, int32_t r_end, int32_t* counts,
                         int32_t* bucket_pos, float* x, float* m, int32_t* inst_quota,
                         int32_t* stats, int32_t* xfer, int32_t* inst_offset,
                         int32_t* dest_inst, int32_t* dest_row, int32_t* err, void* ws,
                         size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * uep_lplb_sample -- LPLB's per-token copy draw.
 * [BLOG] section "从LP解决方案到Token调度": the split, normalised per replicated expert,
 * is a probability distribution over its physical copies; every token routed to a
 * replicated expert draws one copy from it, and a single-copy expert keeps its only
 * instance.  Weights are the integers w_p = rint(max(x_p, 0) * 256) of uep_lplb's
 * quota step; the draw for slot k of global token g = r*T + t is word k mod 4 u of
 * Philox4x64-10 at counter (g, k div 4, 1, 0), key (seed, layer) (one block of the
 * generator per four slots of a token); v = floor(u * W / 2^64)
 * with W = sum w_p, and the first copy (instance order) whose running weight exceeds
 * v wins; W = 0: copy floor(u * n / 2^64) of the expert's n copies.
 * The dispatch layout then follows from uep_load_matrix on dest_inst (instances as
 * experts, E' = I), uep_identity_quota with the identity table and
 * uep_reroute_assign.
 *
 *   topk_ids  [R][T][K]   in   expert ids (-1: empty slot -> -1)
 *   lp                    in   device structure from uep_lplb_prepare (same R)
 *   x         [n_copies]  in   per-copy split (uep_lplb's x, same copy order)
 *   dest_inst [R][T][K]   out  physical instance of every pair
 *   err                   optional: UEP_ERR_ID_RANGE, UEP_ERR_LP (an expert with no
 *                         instance; or `lp` not a structure from uep_lplb_prepare for R
 *                         ranks, and then every pair is -1)
 * ------------------------------------------------------------------------- */
uep_status uep_lplb_sample(const int32_t* topk_ids, int32_t R, int32_t T, int32_t K,
                           const void* lp, const float* x, uint64_t seed, uint64_t layer,
                           int32_t* dest_inst, int32_t* err, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* UEP_H */
