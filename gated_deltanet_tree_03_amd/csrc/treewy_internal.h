// Internal declarations shared by the host entry points and the kernel launchers.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

#include "../../include/treewy.h"

namespace treewy {

constexpr int kD = 128;         // d_k = d_v
constexpr int kMaxNodes = 64;   // ancestor sets are 64-bit masks

// Static tree topology, passed to every kernel by value (kernel arguments), so
// a captured HIP graph replays it without any host work.
struct TreeArgs {
  uint64_t anc[kMaxNodes];   // bit j set iff j is a strict ancestor of t
  int8_t parent[kMaxNodes];  // -1 for the root
  int8_t depth[kMaxNodes];   // root = 0
  int32_t n;                 // node count
  int32_t max_depth;
};

// Validates a DFS pre-order parent array and fills `out`.  Host only.
int build_tree(const int32_t* parent, int n, TreeArgs* out);

// Residency cap by LDS: the dynamic LDS a launch reserves (unused) so that no
// more than `wg_per_cu` workgroups using `static_bytes` of LDS each fit in a
// CU's 160 KiB.  0 = no cap.
constexpr int kLdsPerCU = 160 * 1024;
constexpr int lds_cap_pad(int wg_per_cu, int static_bytes) {
  return wg_per_cu <= 0 ? 0
         : (kLdsPerCU / (wg_per_cu + 1) + 16 > static_bytes
                ? kLdsPerCU / (wg_per_cu + 1) + 16 - static_bytes
                : 0);
}

struct VerifyArgs {
  const float* S0;
  const void* q;
  const void* k;
  const void* v;
  const void* alpha;
  const void* beta;
  float* out;
  float* vtilde;
  float* gamma;
  int B, H;
  int f32_inputs;
  // commit-then-verify only: the previous step's pseudo-values, keys, gates
  // and accepted nodes; the committed state goes to S_out.
  float* S_out;
  const float* vt_prev;
  const void* k_prev;
  const float* gamma_prev;
  const int32_t* acc_prev;
  int n_prev;
  // pool form of commit-then-verify: sequence b's state is block slots[b] of
  // S0 (= S_out), n_slots blocks of H heads; nullptr = block b.
  const int32_t* slots;
  int n_slots;
  // commit-then-verify over a bf16-stored state: S0 / S_out hold bf16 bits
  int state_bf16;
  // tokens per batch row of q/k/v/alpha/beta/out (0: N) and of k_prev (0:
  // n_prev), so a chunk of a longer token-major sequence can be addressed in
  // place; acc_prev == nullptr commits the previous step's last node
  int tok_b, tok_b_prev;
  // per-sequence tree topologies (pool form): sequence b's tree is trees[b]
  // and its previous step's tree trees_prev[b] (device); tok_b and n_prev are
  // then the padded node counts, the row strides of every per-node array
  const TreeArgs* trees;
  const TreeArgs* trees_prev;
};

struct CommitArgs {
  const float* S0;
  const float* vtilde;
  const void* k;
  const float* gamma;
  const int32_t* accepted;  // nullptr: the last node
  float* S_out;
  int B, H;
  int f32_inputs;
  int tok_b;  // tokens per batch row of k (0: N)
};

struct StoreAllArgs {
  const float* S0;
  const void* q;
  const void* k;
  const void* v;
  const void* alpha;
  const void* beta;
  float* out;
  float* snapshots;
  int B, H;
  int f32_inputs;
};

struct SelectArgs {
  const float* snapshots;
  const int32_t* accepted;
  float* S_out;
  int B, H, N;
};

// one-launch prefill of a chain: S [B][H][128][128] fp32 in place; q/k/v
// [B][T][H][128], alpha/beta [B][T][H]; out [B][T][H][128] fp32; T >= 1
struct PrefillArgs {
  float* S;
  const void* q;
  const void* k;
  const void* v;
  const void* alpha;
  const void* beta;
  float* out;
  int B, H, T;
  int f32_inputs;
};

hipError_t launch_verify(const VerifyArgs& a, const TreeArgs& tree, hipStream_t s);
hipError_t launch_commit_verify(const VerifyArgs& a, const TreeArgs& tree, const TreeArgs& prev,
                                hipStream_t s);
// the commit-then-verify families (fp32 state in a batch, in a pool, bf16
// state in a batch), each in its own translation unit
hipError_t launch_commit_verify_batch(const VerifyArgs& a, const TreeArgs& tree,
                                      const TreeArgs& prev, hipStream_t s);
hipError_t launch_commit_verify_pool(const VerifyArgs& a, const TreeArgs& tree,
                                     const TreeArgs& prev, hipStream_t s);
hipError_t launch_commit_verify_s16(const VerifyArgs& a, const TreeArgs& tree,
                                    const TreeArgs& prev, hipStream_t s);
// bf16-stored states in a slot-indexed pool
hipError_t launch_commit_verify_s16_pool(const VerifyArgs& a, const TreeArgs& tree,
                                         const TreeArgs& prev, hipStream_t s);
// pool form with a tree per sequence (a.trees, a.trees_prev); bound and
// prev_bound carry only the batch's node-count and depth bounds (n, max_depth);
// a.state_bf16 picks the bf16-state pool
hipError_t launch_commit_verify_pool_trees(const VerifyArgs& a, const TreeArgs& bound,
                                           const TreeArgs& prev_bound, hipStream_t s);
hipError_t launch_commit_verify_s16_pool_trees(const VerifyArgs& a, const TreeArgs& bound,
                                               const TreeArgs& prev_bound, hipStream_t s);
hipError_t launch_commit(const CommitArgs& a, const TreeArgs& tree, hipStream_t s);
hipError_t launch_store_all(const StoreAllArgs& a, const TreeArgs& tree, hipStream_t s);
hipError_t launch_store_all_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);

// The device scratch of treewy_prefill_chain_noalloc (scratch.hip): its
// address on the current device (taken once per device) and its size.
constexpr size_t kScratchBytes = size_t(TREEWY_SCRATCH_BYTES);
hipError_t scratch_buffer(float** ptr, size_t* bytes);

}  // namespace treewy
