/*
 * treewy.h -- C ABI for tree/chain speculative verification through one Gated
 * DeltaNet (GDN) layer on AMD Instinct MI355X (gfx950).
 *
 * Method: "TreeWY: Speculative Verification for Gated DeltaNet Hybrids".
 *   - paperpeel page, section 3 "Method: TreeWY" ("Key rewrite"): the gated
 *     delta rule is decayed additive attention with a pseudo-value,
 *       S_t = alpha_t S_{t-1} + vt_t k_t^T,
 *       vt_t = beta_t (v_t - alpha_t S_{t-1} k_t);
 *   - same page, section 2 (method summary after the prior-work list) and the
 *     mlsanity page's abstract: every draft node's pseudo-value comes from one
 *     triangular solve over the tree's strict-ancestor structure, and only the
 *     accepted state is rebuilt on commit;
 *   - review page, "Method": nodes in DFS pre-order, so the system is unit lower
 *     triangular;
 *   - paperpeel section 2, bullets on full-state snapshotting: the baseline keeps
 *     one state per draft position and rolls back by indexing.
 *
 * Per (sequence b, value head h), with Gamma_t the product of alpha over the
 * root-to-t path (inclusive):
 *   (I + A) Vt = B,   A[t,j] = beta_t (Gamma_t/Gamma_j)(k_t . k_j) for j a strict
 *                     ancestor of t,   B[t] = beta_t (v_t - Gamma_t S0 k_t)
 *   o_t  = Gamma_t S0 q_t + sum_{j ancestor-or-self of t} (Gamma_t/Gamma_j)(k_j . q_t) vt_j
 *   S_a  = Gamma_a S0 + sum_{j ancestor-or-self of a} (Gamma_a/Gamma_j) vt_j k_j^T
 * o_t equals S_t q_t for the state S_t reached at node t (no scale; fold any
 * 1/sqrt(d) into q).
 *
 * Conventions (all calls):
 *   - d_k = d_v = TREEWY_D = 128.  One query/key per value head.
 *   - Node 0 is the root: the last accepted token, whose update is NOT yet in
 *     S0.  parent[0] = -1 and every other parent[t] lies on the path from the
 *     root to node t-1 (i.e. the nodes are in DFS pre-order).  1 <= N <= 64.
 *   - Layouts are row-major and contiguous:
 *       S0, S_out     float [B][H][128 (v)][128 (k)]
 *       q, k          dtype [B][N][H][128]
 *       v             dtype [B][N][H][128]
 *       alpha, beta   dtype [B][N][H]
 *       out           float [B][N][H][128]
 *       vtilde        float [B][H][N][128]
 *       gamma         float [B][H][N]
 *       snapshots     float [B][H][N+1][128][128]  (S0, then the state after node 0..N-1)
 *       accepted      int32 [B]   (device) node index in [0, N)
 *     where dtype is TREEWY_BF16 (bf16 bit patterns) or TREEWY_F32.
 *   - Pointers named "device" must be device memory, 16-byte aligned.
 *     `parent` is a HOST array of N int32 (the topology is static per call, so
 *     the calls are capturable in a HIP graph).
 *   - The caller allocates and owns every buffer.  The library never allocates,
 *     frees, synchronises or copies device-to-host; each call only enqueues
 *     kernels on `stream` (0 = the null stream).
 *   - Aliasing: no output buffer may overlap another output or any input
 *     (as byte ranges of the sizes the layouts above give), except the
 *     in-place pairs a call names (S_out == S0 exactly, the pool, S in the
 *     prefills).  Inputs may overlap one another.  An overlap is rejected
 *     with TREEWY_ERR_ARG.
 *   - Errors: arguments are validated on the host before any HIP call; on error
 *     the call returns a negative status and enqueues nothing.  A failed launch
 *     returns TREEWY_ERR_LAUNCH.  No global mutable state (except the device
 *     scratch of treewy_prefill_chain_noalloc, see there): calls are
 *     thread-safe.  B == 0 or H == 0 is an empty batch: validated, returns
 *     TREEWY_OK, enqueues nothing.
 */
#ifndef TREEWY_H
#define TREEWY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TREEWY_D 128
#define TREEWY_MAX_NODES 64

typedef enum {
  TREEWY_OK = 0,
  TREEWY_ERR_ARG = -1,    /* null pointer, negative size, bad N */
  TREEWY_ERR_TREE = -2,   /* parent[] is not a DFS pre-order tree */
  TREEWY_ERR_ALIGN = -3,  /* a device pointer is not 16-byte aligned */
  TREEWY_ERR_DTYPE = -4,  /* unknown dtype code */
  TREEWY_ERR_LAUNCH = -5, /* the HIP launch reported an error */
  TREEWY_ERR_SIZE = -6    /* sizes overflow the supported index range */
} treewy_status;

/* Input dtype of q, k, v, alpha, beta.  The last enumerator only widens the
 * enum to the range of int, so that a code passed from another language that
 * is not one of the two (e.g. 7) is a defined value the library rejects with
 * TREEWY_ERR_DTYPE. */
typedef enum {
  TREEWY_BF16 = 0,
  TREEWY_F32 = 1,
  TREEWY_DTYPE_INT_RANGE_ = 0x7fffffff
} treewy_dtype;

/* Tree metadata (host only, no HIP call).
 * Source: review page "Method" (DFS pre-order layout) and paperpeel section 4
 * (the ancestor mask a tree needs).
 * In:  parent[N] (host).  Out: depth[N] (root 0) and anc[N], where bit j of
 * anc[t] is set iff j is a strict ancestor of t.  Either output may be NULL.
 * Returns TREEWY_OK, TREEWY_ERR_ARG (N outside 1..64 or parent NULL) or
 * TREEWY_ERR_TREE (not a DFS pre-order tree). */
int treewy_tree_meta(const int32_t* parent, int N, int32_t* depth, uint64_t* anc);

/* Verify: every node's output and pseudo-value from one solve.
 * Source: paperpeel section 3 ("Key rewrite") and section 2's method summary.
 * In (device): S0, q, k, v, alpha, beta in the layouts above; parent (host).
 * Out (device): out[B][N][H][128] = o_t, vtilde[B][H][N][128] = Vt,
 * gamma[B][H][N] = Gamma_t (kept for commit).  S0 is only read.
 * Numerics: fp32 state and outputs; S0 . [k;q] and the key/query gram run on
 * bf16 matrix cores with S0 (and fp32 q/k) split into two bf16 terms, fp32
 * accumulation (relative error ~1e-5 of |S0||k|). */
int treewy_verify(const float* S0, const void* q, const void* k, const void* v,
                  const void* alpha, const void* beta, const int32_t* parent,
                  int B, int H, int N, float* out, float* vtilde, float* gamma,
                  treewy_dtype dtype, hipStream_t stream);

/* Commit: rebuild only the accepted state.
 * Source: mlsanity abstract and review page "Method" (reconstruct the accepted
 * node's state from the same solve).
 * In (device): S0, vtilde and gamma from treewy_verify, k as given to verify,
 * accepted[B] (node index per sequence); parent (host) as given to verify.
 * Out (device): S_out[B][H][128][128] = S_a.  S_out may equal S0 (in-place
 * commit); otherwise the two must not overlap.
 * A sequence whose accepted index lies outside [0, N) gets NaN in every element
 * of its S_out blocks (no memory outside the buffers is touched).
 * Gamma ratios are formed by fp32 division; paths whose Gamma falls below the
 * fp32 normal range (~1.2e-38) are outside the supported range. */
int treewy_commit(const float* S0, const float* vtilde, const void* k, const float* gamma,
                  const int32_t* accepted, const int32_t* parent, int B, int H, int N,
                  float* S_out, treewy_dtype dtype, hipStream_t stream);

/* Commit-then-verify: the commit of the previous step fused into the verify
 * of the next one, so that the state is read once and written once per step.
 * Source: paperpeel section 6 and review page "Future work" (fusing the path
 * into one capturable kernel and deferring the state write are the next
 * steps); the arithmetic is that of treewy_commit followed by treewy_verify.
 * In (device): S0 = the state before the previous step; vtilde_prev,
 * gamma_prev (from that step's verify), k_prev (its keys) and
 * accepted_prev[B]; parent_prev (host, N_prev nodes) is its tree.  The new
 * step's q, k, v, alpha, beta, parent (host) and N as for treewy_verify.
 * Out (device): S_out[B][H][128][128] = the committed state S_a of the
 * previous step (S_out may equal S0; otherwise they must not overlap), and
 * out / vtilde / gamma of the new step verified from S_a, exactly as
 * treewy_commit(S0, ..., S_out) then treewy_verify(S_out, ...) would give (up
 * to rounding order).  vtilde and gamma must not overlap vtilde_prev and
 * gamma_prev (equal pointers are rejected with TREEWY_ERR_ARG).  A sequence
 * whose accepted_prev index lies outside [0, N_prev) gets NaN in its S_out
 * blocks and in all of its new outputs. */
int treewy_commit_verify(const float* S0, float* S_out, const float* vtilde_prev,
                         const void* k_prev, const float* gamma_prev,
                         const int32_t* accepted_prev, const int32_t* parent_prev, int N_prev,
                         const void* q, const void* k, const void* v, const void* alpha,
                         const void* beta, const int32_t* parent, int B, int H, int N,
                         float* out, float* vtilde, float* gamma, treewy_dtype dtype, hipStream_t stream);

/* Commit-then-verify over a slot-indexed state pool: the serving form, where
 * each live request owns one state block in a pool and a fixed batch bucket
 * refers to it by slot.
 * Source: as treewy_commit_verify (paperpeel section 6, review page "Future
 * work"); the pool keeps the resident state at one block per request
 * (paperpeel section 2 memory arithmetic, review page "Results").
 * In/out (device): pool[n_slots][H][128][128]; sequence b's state is
 * pool[slots[b]], read and overwritten in place with the committed state.
 * slots[B] (device int32) must be distinct (two sequences on one slot race).
 * Everything else, including vtilde_prev / gamma_prev / k_prev / out /
 * vtilde / gamma indexed by batch row b, is as for treewy_commit_verify, with
 * two differences in the per-sequence error cases:
 *   - accepted_prev[b] < 0 means "no previous step to commit" (a request that
 *     joins the batch): its state is used as it is and not rewritten;
 *     accepted_prev[b] >= N_prev still gives NaN state and outputs;
 *   - a slot outside [0, n_slots) touches no pool memory; that sequence's out
 *     and vtilde are NaN.
 * n_slots >= 1 for a non-empty batch (n_slots * H within the batch-size
 * bound). */
int treewy_commit_verify_pool(float* pool, int n_slots, const int32_t* slots,
                              const float* vtilde_prev, const void* k_prev,
                              const float* gamma_prev, const int32_t* accepted_prev,
                              const int32_t* parent_prev, int N_prev, const void* q,
                              const void* k, const void* v, const void* alpha, const void* beta,
                              const int32_t* parent, int B, int H, int N, float* out,
                              float* vtilde, float* gamma, treewy_dtype dtype, hipStream_t stream);

/* Size in bytes of one tree descriptor (the packed, validated topology of one
 * request's draft tree), for treewy_commit_verify_pool_trees. */
size_t treewy_tree_desc_size(void);

/* Validate and pack one draft tree per request (host only, no GPU call).
 * Source: the DFS pre-order parent layout (review page "Method"); as
 * treewy_tree_meta, per request.
 * In (host): parents[count][n_max] int32, request i's parent array in its
 * first counts[i] entries (1 <= counts[i] <= n_max <= 64); counts[count].
 * Out (host): desc, count descriptors of treewy_tree_desc_size() bytes each
 * (8-byte aligned); *max_depth (may be NULL) = the deepest node over all
 * requests.  On error desc is left partly written and the status names the
 * first bad request's fault (TREEWY_ERR_ARG, TREEWY_ERR_TREE). */
int treewy_tree_desc_pack(const int32_t* parents, const int32_t* counts, int count, int n_max,
                          void* desc, int* max_depth);

/* Commit-then-verify over a slot-indexed state pool with a draft tree per
 * request: treewy_commit_verify_pool where each batch row b has its own
 * tree for this step (trees[b]) and had its own tree last step
 * (trees_prev[b]).
 * Source: as treewy_commit_verify_pool, whose resident cost is one state
 * block per request whatever the tree (paperpeel section 5 "Tree width").
 * That each request drafts its own tree is this interface's reading of the
 * serving setting; the pages fix only the pre-order parent layout (review
 * page "Method").
 * trees, trees_prev (device): B descriptors each, copied from
 * treewy_tree_desc_pack's output.  N, N_prev: node-count bounds (1..64,
 * >= every request's count); every per-node array is laid out for them:
 * q, k, v [B][N][H][128], alpha, beta [B][N][H], out [B][N][H][128], vtilde
 * [B][H][N][128], gamma [B][H][N], and the previous step's k_prev,
 * vtilde_prev, gamma_prev likewise with N_prev.  depth, depth_prev: depth
 * bounds (< N, < N_prev; treewy_tree_desc_pack reports them) that pick the
 * kernel.  Rows t >= counts[b] of out / vtilde / gamma are not written.
 * Everything else (pool, slots, accepted_prev and its error cases, aliasing
 * rules) is as for treewy_commit_verify_pool.  The kernel reads each
 * descriptor from device memory and clamps every field into range, so no
 * descriptor can send an access out of bounds; a descriptor that was not
 * packed by treewy_tree_desc_pack, or a request deeper than `depth`, gives
 * undefined values in that request's outputs. */
int treewy_commit_verify_pool_trees(float* pool, int n_slots, const int32_t* slots,
                                    const float* vtilde_prev, const void* k_prev,
                                    const float* gamma_prev, const int32_t* accepted_prev,
                                    const void* trees_prev, int N_prev, int depth_prev,
                                    const void* q, const void* k, const void* v,
                                    const void* alpha, const void* beta, const void* trees,
                                    int N, int depth, int B, int H, float* out, float* vtilde,
                                    float* gamma, treewy_dtype dtype, hipStream_t stream);

/* Commit-then-verify over a bf16-stored state: treewy_commit_verify with S0
 * and S_out holding bf16 bit patterns, [B][H][128][128] (32 KiB per head
 * instead of 64).
 * Source: as treewy_commit_verify; the pages' state-memory arithmetic counts
 * a 16-bit state (paperpeel section 2).
 * The committed state is computed in fp32 from the bf16 S0 and rounded to
 * bf16 (nearest even) when stored; the new step is verified from that stored
 * value, so a later step reading S_out continues from exactly what this one
 * used.  The state needs no split on the matrix cores (it is exact in bf16).
 * Inputs must be bf16 (dtype TREEWY_BF16, else TREEWY_ERR_DTYPE).  Everything
 * else, including in-place S_out == S0 and the NaN cases, is as for
 * treewy_commit_verify.  Tolerance: the stored state carries one bf16
 * rounding (<= 2^-9 relative per element) on top of the fp32 arithmetic. */
int treewy_commit_verify_bf16state(const void* S0, void* S_out, const float* vtilde_prev,
                                   const void* k_prev, const float* gamma_prev,
                                   const int32_t* accepted_prev, const int32_t* parent_prev,
                                   int N_prev, const void* q, const void* k, const void* v,
                                   const void* alpha, const void* beta, const int32_t* parent,
                                   int B, int H, int N, float* out, float* vtilde, float* gamma,
                                   treewy_dtype dtype, hipStream_t stream);

/* Chunked prefill of a chain: run the gated delta rule over T tokens of each
 * sequence from the state S, writing every token's output and leaving the
 * state after the last token in S (in place).
 * Source: the chunkwise WY form of DeltaNet that the method extends
 * (paperpeel section 2, the chain case of the method summary; review page
 * "Method"): a chain is a width-1 tree, so each chunk of up to `chunk` tokens
 * is one chain verified from the state, and the chunk's last token is
 * committed into it before the next chunk (commit-then-verify), then after the
 * last chunk.
 * In (device): q, k, v [B][T][H][128], alpha, beta [B][T][H] (dtype), S
 * [B][H][128][128] fp32.  Out (device): out [B][T][H][128] fp32; S updated.
 * Workspace (device, caller-owned, contents undefined on return):
 * work_vtilde 2*B*H*chunk*128 floats, work_gamma 2*ceil4(B*H*chunk) floats.
 * 1 <= chunk <= 64; T >= 0 (T == 0 leaves S as it is).  Launches
 * ceil(T/chunk) + 1 kernels on `stream`. */
int treewy_prefill_chain(float* S, const void* q, const void* k, const void* v,
                         const void* alpha, const void* beta, int B, int T, int H, int chunk,
                         float* out, float* work_vtilde, float* work_gamma, treewy_dtype dtype,
                         hipStream_t stream);

/* Commit-then-verify over a slot-indexed pool of bf16-stored states: the pool
 * form (treewy_commit_verify_pool) of treewy_commit_verify_bf16state.
 * Source: as treewy_commit_verify_pool; the pages' state-memory arithmetic
 * counts a 16-bit state (paperpeel section 2), and the pool keeps it at one
 * block per request.
 * In/out (device): pool[n_slots][H][128][128] holds bf16 bit patterns (32 KiB
 * per head); sequence b's state is pool[slots[b]], committed in place and
 * rounded to bf16 (nearest even) as treewy_commit_verify_bf16state rounds it.
 * Everything else (arguments, layouts, the accepted_prev[b] < 0 and bad-slot
 * cases, aliasing) is as for treewy_commit_verify_pool; inputs must be bf16
 * (else TREEWY_ERR_DTYPE). */
int treewy_commit_verify_bf16state_pool(void* pool, int n_slots, const int32_t* slots,
                                        const float* vtilde_prev, const void* k_prev,
                                        const float* gamma_prev, const int32_t* accepted_prev,
                                        const int32_t* parent_prev, int N_prev, const void* q,
                                        const void* k, const void* v, const void* alpha,
                                        const void* beta, const int32_t* parent, int B, int H,
                                        int N, float* out, float* vtilde, float* gamma,
                                        treewy_dtype dtype, hipStream_t stream);

/* treewy_commit_verify_bf16state_pool with a draft tree per request: the
 * bf16-state pool form of treewy_commit_verify_pool_trees.
 * Source: as treewy_commit_verify_pool_trees (one state block per request
 * whatever its tree, paperpeel section 5 "Tree width") with the 16-bit state
 * of paperpeel section 2.
 * pool holds bf16 states as in treewy_commit_verify_bf16state_pool; trees,
 * trees_prev, N, N_prev, depth, depth_prev and every other argument as for
 * treewy_commit_verify_pool_trees; inputs must be bf16. */
int treewy_commit_verify_bf16state_pool_trees(void* pool, int n_slots, const int32_t* slots,
                                              const float* vtilde_prev, const void* k_prev,
                                              const float* gamma_prev,
                                              const int32_t* accepted_prev,
                                              const void* trees_prev, int N_prev, int depth_prev,
                                              const void* q, const void* k, const void* v,
                                              const void* alpha, const void* beta,
                                              const void* trees, int N, int depth, int B, int H,
                                              float* out, float* vtilde, float* gamma,
                                              treewy_dtype dtype, hipStream_t stream);

/* Size in bytes of the device scratch treewy_prefill_chain_noalloc works in
 * (one copy per GPU, held from the library's first use there until the
 * process ends). */
#define TREEWY_SCRATCH_BYTES (64u << 20)

/* treewy_prefill_chain without a workspace argument and without any device
 * allocation, for callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops that forbid allocation, harnesses that forbid
 * hipMalloc.  The pseudo-value and gate buffers between chunk launches live in
 * the library's own device scratch of TREEWY_SCRATCH_BYTES per GPU, so the
 * call is valid only while 2*B*H*chunk*128*4 + 2*ceil4(B*H*chunk)*4 bytes fit
 * in it; larger calls return TREEWY_ERR_SIZE and enqueue nothing.  Arguments,
 * results and the other errors are those of treewy_prefill_chain.  `stream`
 * must belong to the current device (else TREEWY_ERR_ARG).  The first call on
 * a device takes the scratch's device address (no allocation); a failure
 * there returns TREEWY_ERR_LAUNCH.  Every call on one GPU shares the scratch:
 * calls that overlap in time on one GPU (e.g. on two streams, or from two
 * threads) race and give undefined results.  The scratch needs no clearing:
 * each launch reads only what the launch before it wrote. */
int treewy_prefill_chain_noalloc(float* S, const void* q, const void* k, const void* v,
                                 const void* alpha, const void* beta, int B, int T, int H,
                                 int chunk, float* out, treewy_dtype dtype, hipStream_t stream);

/* Prefill of a chain in one launch: run the gated delta rule over T tokens of
 * each sequence from the state S, writing every token's output and leaving
 * the state after the last token in S (in place).  Same results as
 * treewy_prefill_chain, computed differently: one workgroup per (sequence,
 * head) holds the state on chip and takes the tokens in chunks of 16, each a
 * 16-node chain verified from the state (the chain case of the method
 * summary, paperpeel section 2; pseudo-values and outputs as in paperpeel
 * section 3 "Key rewrite"), after which the state moves to the chunk's last
 * token (the commit of the mlsanity abstract).  The state is read once and
 * written once.
 * In (device): q, k, v [B][T][H][128], alpha, beta [B][T][H] (dtype), S
 * [B][H][128][128] fp32.  Out (device): out [B][T][H][128] fp32; S updated.
 * T >= 0 (T == 0 leaves S as it is).  No workspace: every buffer is an input
 * or an output.  One kernel launch on `stream`.  The caller must not let out
 * overlap the inputs or S.
 * Errors: those of treewy_prefill_chain, and TREEWY_ERR_SIZE for H > 2^19
 * (the kernel addresses a chunk's rows with 32-bit offsets). */
int treewy_prefill(float* S, const void* q, const void* k, const void* v, const void* alpha,
                   const void* beta, int B, int T, int H, float* out, treewy_dtype dtype,
                   hipStream_t stream);

/* store_all baseline (full-state snapshotting): walk the recurrence node by
 * node, writing out[] as treewy_verify does and snapshots[b][h][0] = S0,
 * snapshots[b][h][t+1] = state after node t.
 * Source: paperpeel section 2, first bullet of the prior work (one snapshot per
 * draft position, rollback by indexing). */
int treewy_store_all(const float* S0, const void* q, const void* k, const void* v,
                     const void* alpha, const void* beta, const int32_t* parent,
                     int B, int H, int N, float* out, float* snapshots,
                     treewy_dtype dtype, hipStream_t stream);

/* store_all rollback: S_out[b][h] = snapshots[b][h][accepted[b] + 1].
 * Source: paperpeel section 2, first prior-work bullet (full-state
 * snapshotting rolls back by indexing the accepted draft position's snapshot).
 * In (device): snapshots as written by treewy_store_all, accepted[B].
 * Out (device): S_out[B][H][128][128].
 * An accepted index outside [0, N) yields NaN blocks, as in treewy_commit.
 * S_out must not overlap snapshots (TREEWY_ERR_ARG). */
int treewy_store_all_select(const float* snapshots, const int32_t* accepted,
                            int B, int H, int N, float* S_out, hipStream_t stream);

/* Static English description of a status code (never NULL). */
const char* treewy_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* TREEWY_H */
