// C-ABI entry points: host-side validation, then one kernel launch each.
// Every check happens before the first HIP call, so a rejected call has no
// side effects.  Nothing here allocates, synchronises or keeps state.
#include <stddef.h>
#include <stdint.h>

#include <initializer_list>

#include "../../include/treewy.h"
#include "treewy_internal.h"

using namespace treewy;

namespace {

constexpr int64_t kMaxHeads = int64_t(1) << 24;  // B*H bound (grid and 32-bit tile indices)
constexpr int kPrefillMaxH = 1 << 19;  // H bound of the one-launch prefill

int check_dev(const void* p) {
  if (p == nullptr) return TREEWY_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(p) & 15u) return TREEWY_ERR_ALIGN;
  return TREEWY_OK;
}

int check_all(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs) {
    int s = check_dev(p);
    if (s != TREEWY_OK) return s;
  }
  return TREEWY_OK;
}

int check_sizes(int B, int H) {
  if (B < 0 || H < 0) return TREEWY_ERR_ARG;
  if (int64_t(B) * int64_t(H) > kMaxHeads) return TREEWY_ERR_SIZE;
  return TREEWY_OK;
}

int check_dtype(treewy_dtype dtype) {
  return (dtype == TREEWY_BF16 || dtype == TREEWY_F32) ? TREEWY_OK : TREEWY_ERR_DTYPE;
}

// One buffer's byte range, for the aliasing checks.  n == 0: nothing is
// accessed there.
struct Span {
  const void* p;
  int64_t n;
};

bool overlap(const Span& a, const Span& b) {
  if (a.n <= 0 || b.n <= 0) return false;
  using u128 = unsigned __int128;
  const u128 x = reinterpret_cast<uintptr_t>(a.p), y = reinterpret_cast<uintptr_t>(b.p);
  return x < y + static_cast<u128>(b.n) && y < x + static_cast<u128>(a.n);
}

// Outputs must not overlap one another nor any input: a kernel that writes
// one buffer while other workgroups read or write an overlapping one gives
// undefined results.  (In-place pairs the interface allows, such as
// S_out == S0, are passed as one output by the caller.)
int check_disjoint(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    for (auto o2 = o + 1; o2 != outs.end(); ++o2) {
      if (overlap(*o, *o2)) return TREEWY_ERR_ARG;
    }
    for (const Span& i : ins) {
      if (overlap(*o, i)) return TREEWY_ERR_ARG;
    }
  }
  return TREEWY_OK;
}

// Byte sizes of the per-call buffers (B*H <= 2^24, N <= 64: no overflow).
constexpr int64_t kStateBytes = int64_t(kD) * kD * 4;

int64_t in_bytes(treewy_dtype dtype) { return dtype == TREEWY_F32 ? 4 : 2; }

// Aliasing rule of the batch commit-then-verify entry points (fp32 or bf16
// state of `state_bytes` per head): S_out equal to S0 (in place) or disjoint
// from it, and every output disjoint from every input and from one another.
int check_fused_disjoint(int B, int H, int N, int N_prev, treewy_dtype dtype, const void* S0,
                         const void* S_out, int64_t state_bytes, const void* vtilde_prev,
                         const void* k_prev, const void* gamma_prev, const void* accepted_prev,
                         const void* q, const void* k, const void* v, const void* alpha,
                         const void* beta, const void* out, const void* vtilde,
                         const void* gamma) {
  const int64_t G = int64_t(B) * H, ib = in_bytes(dtype), tok = G * N * kD * ib;
  const int64_t np = N_prev;
  const bool in_place = S_out == S0;
  return check_disjoint({{S_out, G * state_bytes}, {out, G * N * kD * 4}, {vtilde, G * N * kD * 4},
                         {gamma, G * N * 4}},
                        {{S0, in_place ? 0 : G * state_bytes}, {vtilde_prev, G * np * kD * 4},
                         {k_prev, G * np * kD * ib}, {gamma_prev, G * np * 4},
                         {accepted_prev, int64_t(B) * 4}, {q, tok}, {k, tok}, {v, tok},
                         {alpha, G * N * ib}, {beta, G * N * ib}});
}

int launch_status(hipError_t e) {
  if (e != hipSuccess) return TREEWY_ERR_LAUNCH;
  return hipGetLastError() == hipSuccess ? TREEWY_OK : TREEWY_ERR_LAUNCH;
}

}  // namespace

extern "C" int treewy_tree_meta(const int32_t* parent, int N, int32_t* depth, uint64_t* anc) {
  TreeArgs tree;
  int s = build_tree(parent, N, &tree);
  if (s != TREEWY_OK) return s;
  for (int t = 0; t < N; ++t) {
    if (depth) depth[t] = tree.depth[t];
    if (anc) anc[t] = tree.anc[t];
  }
  return TREEWY_OK;
}

extern "C" int treewy_verify(const float* S0, const void* q, const void* k, const void* v,
                             const void* alpha, const void* beta, const int32_t* parent,
                             int B, int H, int N, float* out, float* vtilde, float* gamma,
                             treewy_dtype dtype, hipStream_t stream) {
  int s = check_sizes(B, H);
  if (s != TREEWY_OK) return s;
  TreeArgs tree;
  if ((s = build_tree(parent, N, &tree)) != TREEWY_OK) return s;
  if ((s = check_dtype(dtype)) != TREEWY_OK) return s;
  if (B == 0 || H == 0) return TREEWY_OK;
  if ((s = check_all({S0, q, k, v, alpha, beta, out, vtilde, gamma})) != TREEWY_OK) return s;
  {
    const int64_t G = int64_t(B) * H, tok = G * N * kD * in_bytes(dtype), gate = G * N * in_bytes(dtype);
    if ((s = check_disjoint({{out, G * N * kD * 4}, {vtilde, G * N * kD * 4}, {gamma, G * N * 4}},
                            {{S0, G * kStateBytes}, {q, tok}, {k, tok}, {v, tok}, {alpha, gate},
                             {beta, gate}})) != TREEWY_OK) {
      return s;
    }
  }
  VerifyArgs a{S0, q, k, v, alpha, beta, out, vtilde, gamma, B, H, dtype == TREEWY_F32};
  return launch_status(launch_verify(a, tree, stream));
}

extern "C" int treewy_commit_verify(const float* S0, float* S_out, const float* vtilde_prev,
                                    const void* k_prev, const float* gamma_prev,
                                    const int32_t* accepted_prev, const int32_t* parent_prev,
                                    int N_prev, const void* q, const void* k, const void* v,
                                    const void* alpha, const void* beta, const int32_t* parent,
                                    int B, int H, int N, float* out, float* vtilde, float* gamma,
                                    treewy_dtype dtype, hipStream_t stream) {
  int s = check_sizes(B, H);
  if (s != TREEWY_OK) return s;
  TreeArgs tree, prev;
  if ((s = build_tree(parent, N, &tree)) != TREEWY_OK) return s;
  if ((s = build_tree(parent_prev, N_prev, &prev)) != TREEWY_OK) return s;
  if ((s = check_dtype(dtype)) != TREEWY_OK) return s;
  if (B == 0 || H == 0) return TREEWY_OK;
  if ((s = check_all({S0, S_out, vtilde_prev, k_prev, gamma_prev, accepted_prev, q, k, v, alpha,
                      beta, out, vtilde, gamma})) != TREEWY_OK) {
    return s;
  }
  // the previous step's pseudo-values and gates are read while the new ones
  // are written: every output is disjoint from every input (S_out == S0 is
  // the in-place commit)
  if ((s = check_fused_disjoint(B, H, N, N_prev, dtype, S0, S_out, kStateBytes, vtilde_prev, k_prev,
                                gamma_prev, accepted_prev, q, k, v, alpha, beta, out, vtilde,
                                gamma)) != TREEWY_OK) {
    return s;
  }
  VerifyArgs a{S0, q, k, v, alpha, beta, out, vtilde, gamma, B, H, dtype == TREEWY_F32,
               S_out, vtilde_prev, k_prev, gamma_prev, accepted_prev, N_prev};
  return launch_status(launch_commit_verify(a, tree, prev, stream));
}

extern "C" int treewy_commit_verify_pool(float* pool, int n_slots, const int32_t* slots,
                                         const float* vtilde_prev, const void* k_prev,
                                         const float* gamma_prev, const int32_t* accepted_prev,
                                         const int32_t* parent_prev, int N_prev, const void* q,
                                         const void* k, const void* v, const void* alpha,
                                         const void* beta, const int32_t* parent, int B, int H,
                                         int N, float* out, float* vtilde, float* gamma, treewy_dtype dtype,
                                         hipStream_t stream) {
  int s = check_sizes(B, H);
  if (s != TREEWY_OK) return s;
  if (n_slots < 0) return TREEWY_ERR_ARG;
  if ((s = check_sizes(n_slots, H)) != TREEWY_OK) return s;
  TreeArgs tree, prev;
  if ((s = build_tree(parent, N, &tree)) != TREEWY_OK) return s;
  if ((s = build_tree(parent_prev, N_prev, &prev)) != TREEWY_OK) return s;
  if ((s = check_dtype(dtype)) != TREEWY_OK) return s;
  if (B == 0 || H == 0) return TREEWY_OK;
  if (n_slots < 1) return TREEWY_ERR_ARG;  // a bad slot reads slot 0 (then discards it)
  if ((s = check_all({pool, slots, vtilde_prev, k_prev, gamma_prev, accepted_prev, q, k, v, alpha,
                      beta, out, vtilde, gamma})) != TREEWY_OK) {
    return s;
  }
  {
    // the pool is read and written in place: it counts as an output
    const int64_t G = int64_t(B) * H, ib = in_bytes(dtype), tok = G * N * kD * ib;
    const int64_t np = N_prev;
    if ((s = check_disjoint({{pool, int64_t(n_slots) * H * kStateBytes}, {out, G * N * kD * 4},
                             {vtilde, G * N * kD * 4}, {gamma, G * N * 4}},
                            {{slots, int64_t(B) * 4}, {vtilde_prev, G * np * kD * 4},
                             {k_prev, G * np * kD * ib}, {gamma_prev, G * np * 4},
                             {accepted_prev, int64_t(B) * 4}, {q, tok}, {k, tok}, {v, tok},
                             {alpha, G * N * ib}, {beta, G * N * ib}})) != TREEWY_OK) {
      return s;
    }
  }
  VerifyArgs a{pool, q, k, v, alpha, beta, out, vtilde, gamma, B, H, dtype == TREEWY_F32,
               pool, vtilde_prev, k_prev, gamma_prev, accepted_prev, N_prev, slots, n_slots};
  return launch_status(launch_commit_verify(a, tree, prev, stream));
}

extern "C" size_t treewy_tree_desc_size(void) { return sizeof(TreeArgs); }

extern "C" int treewy_tree_desc_pack(const int32_t* parents, const int32_t* counts, int count,
                                     int n_max, void* desc, int* max_depth) {
  if (count < 0 || n_max < 1 || n_max > kMaxNodes) return TREEWY_ERR_ARG;
  if (count > 0 && (parents == nullptr || counts == nullptr || desc == nullptr)) {
    return TREEWY_ERR_ARG;
  }
  if (reinterpret_cast<uintptr_t>(desc) & 7u) return TREEWY_ERR_ALIGN;
  TreeArgs* out = static_cast<TreeArgs*>(desc);
  int md = 0;
  for (int i = 0; i < count; ++i) {
    const int n = counts[i];
    if (n < 1 || n > n_max) return TREEWY_ERR_ARG;
    const int s = build_tree(parents + static_cast<int64_t>(i) * n_max, n, &out[i]);
    if (s != TREEWY_OK) return s;
    if (out[i].max_depth > md) md = out[i].max_depth;
  }
  if (max_depth != nullptr) *max_depth = md;
  return TREEWY_OK;
}

extern "C" int treewy_commit_verify_pool_trees(
    float* pool, int n_slots, const int32_t* slots, const float* vtilde_prev, const void* k_prev,
    const float* gamma_prev, const int32_t* accepted_prev, const void* trees_prev, int N_prev,
    int depth_prev, const void* q, const void* k, const void* v, const void* alpha,
    const void* beta, const void* trees, int N, int depth, int B, int H, float* out, float* vtilde,
    float* gamma, treewy_dtype dtype, hipStream_t stream) {
  int s = check_sizes(B, H);
  if (s != TREEWY_OK) return s;
  if (n_slots < 0) return TREEWY_ERR_ARG;
  if ((s = check_sizes(n_slots, H)) != TREEWY_OK) return s;
  if (N < 1 || N > kMaxNodes || N_prev < 1 || N_prev > kMaxNodes) return TREEWY_ERR_ARG;
  if (depth < 0 || depth >= N || depth_prev < 0 || depth_prev >= N_prev) return TREEWY_ERR_ARG;
  if ((s = check_dtype(dtype)) != TREEWY_OK) return s;
  if (B == 0 || H == 0) return TREEWY_OK;
  if (n_slots < 1) return TREEWY_ERR_ARG;  // a bad slot reads slot 0 (then discards it)
  if ((s = check_all({pool, slots, vtilde_prev, k_prev, gamma_prev, accepted_prev, trees_prev, q,
                      k, v, alpha, beta, trees, out, vtilde, gamma})) != TREEWY_OK) {
    return s;
  }
  {
    const int64_t G = int64_t(B) * H, ib = in_bytes(dtype), tok = G * N * kD * ib;
    const int64_t np = N_prev, desc = int64_t(B) * int64_t(sizeof(TreeArgs));
    if ((s = check_disjoint({{pool, int64_t(n_slots) * H * kStateBytes}, {out, G * N * kD * 4},
                             {vtilde, G * N * kD * 4}, {gamma, G * N * 4}},
                            {{slots, int64_t(B) * 4}, {vtilde_prev, G * np * kD * 4},
                             {k_prev, G * np * kD * ib}, {gamma_prev, G * np * 4},
                             {accepted_prev, int64_t(B) * 4}, {trees_prev, desc}, {q, tok}, {k, tok},
                             {v, tok}, {alpha, G * N * ib}, {beta, G * N * ib},
                             {trees, desc}})) != TREEWY_OK) {
      return s;
    }
  }
  TreeArgs bound{}, prev_bound{};
  bound.n = N;
  bound.max_depth = depth;
  prev_bound.n = N_prev;
  prev_bound.max_depth = depth_prev;
  VerifyArgs a{pool, q, k, v, alpha, beta, out, vtilde, gamma, B, H, dtype == TREEWY_F32,
               pool, vtilde_prev, k_prev, gamma_prev, accepted_prev, N_prev, slots, n_slots};
  a.tok_b = N;
  a.tok_b_prev = N_prev;
  a.trees = static_cast<const TreeArgs*>(trees);
  a.trees_prev = static_cast<const TreeArgs*>(trees_prev);
  return launch_status(launch_commit_verify_pool_trees(a, bound, prev_bound, stream));
}

extern "C" int treewy_commit_verify_bf16state(const void* S0, void* S_out,
                                              const float* vtilde_prev, const void* k_prev,
                                              const float* gamma_prev,
                                              const int32_t* accepted_prev,
                                              const int32_t* parent_prev, int N_prev,
                                              const void* q, const void* k, const void* v,
                                              const void* alpha, const void* beta,
                                              const int32_t* parent, int B, int H, int N,
                                              float* out, float* vtilde, float* gamma, treewy_dtype dtype,
                                              hipStream_t stream) {
  int s = check_sizes(B, H);
  if (s != TREEWY_OK) return s;
  TreeArgs tree, prev;
  if ((s = build_tree(parent, N, &tree)) != TREEWY_OK) return s;
  if ((s = build_tree(parent_prev, N_prev, &prev)) != TREEWY_OK) return s;
  if (dtype != TREEWY_BF16) return TREEWY_ERR_DTYPE;  // bf16 inputs with the bf16 state
  if (B == 0 || H == 0) return TREEWY_OK;
  if ((s = check_all({S0, S_out, vtilde_prev, k_prev, gamma_prev, accepted_prev, q, k, v, alpha,
                      beta, out, vtilde, gamma})) != TREEWY_OK) {
    return s;
  }
  if ((s = check_fused_disjoint(B, H, N, N_prev, dtype, S0, S_out, kStateBytes / 2, vtilde_prev,
                                k_prev, gamma_prev, accepted_prev, q, k, v, alpha, beta, out, vtilde,
                                gamma)) != TREEWY_OK) {
    return s;
  }
  VerifyArgs a{static_cast<const float*>(S0), q, k, v, alpha, beta, out, vtilde, gamma, B, H, 0,
               static_cast<float*>(S_out), vtilde_prev, k_prev, gamma_prev, accepted_prev,
               N_prev, nullptr, 0, 1};
  return launch_status(launch_commit_verify(a, tree, prev, stream));
}

extern "C" int treewy_prefill(float* S, const void* q, const void* k, const void* v,
                              const void* alpha, const void* beta, int B, int T, int H, float* out,
                              treewy_dtype dtype, hipStream_t stream) {
  int s = check_sizes(B, H);
  if (s != TREEWY_OK) return s;
  if (H > kPrefillMaxH) return TREEWY_ERR_SIZE;  // 32-bit row offsets inside a chunk
  if (T < 0) return TREEWY_ERR_ARG;
  if ((s = check_dtype(dtype)) != TREEWY_OK) return s;
  if (B == 0 || H == 0 || T == 0) return TREEWY_OK;
  if ((s = check_all({S, q, k, v, alpha, beta, out})) != TREEWY_OK) return s;
  {
    const int64_t BT = int64_t(B) * T * H, ib = in_bytes(dtype);
    if ((s = check_disjoint({{S, int64_t(B) * H * kStateBytes}, {out, BT * kD * 4}},
                            {{q, BT * kD * ib}, {k, BT * kD * ib}, {v, BT * kD * ib},
                             {alpha, BT * ib}, {beta, BT * ib}})) != TREEWY_OK) {
      return s;
    }
  }
  PrefillArgs a{S, q, k, v, alpha, beta, out, B, H, T, dtype == TREEWY_F32};
  return launch_status(launch_prefill(a, stream));
}

extern "C" int treewy_commit_verify_bf16state_pool(
    void* pool, int n_slots, const int32_t* slots, const float* vtilde_prev, const void* k_prev,
    const float* gamma_prev, const int32_t* accepted_prev, const int32_t* parent_prev, int N_prev,
    const void* q, const void* k, const void* v, const void* alpha, const void* beta,
    const int32_t* parent, int B, int H, int N, float* out, float* vtilde, float* gamma,
    treewy_dtype dtype, hipStream_t stream) {
  int s = check_sizes(B, H);
  if (s != TREEWY_OK) return s;
  if (n_slots < 0) return TREEWY_ERR_ARG;
  if ((s = check_sizes(n_slots, H)) != TREEWY_OK) return s;
  TreeArgs tree, prev;
  if ((s = build_tree(parent, N, &tree)) != TREEWY_OK) return s;
  if ((s = build_tree(parent_prev, N_prev, &prev)) != TREEWY_OK) return s;
  if (dtype != TREEWY_BF16) return TREEWY_ERR_DTYPE;  // bf16 inputs with the bf16 state
  if (B == 0 || H == 0) return TREEWY_OK;
  if (n_slots < 1) return TREEWY_ERR_ARG;  // a bad slot reads slot 0 (then discards it)
  if ((s = check_all({pool, slots, vtilde_prev, k_prev, gamma_prev, accepted_prev, q, k, v, alpha,
                      beta, out, vtilde, gamma})) != TREEWY_OK) {
    return s;
  }
  {
    const int64_t G = int64_t(B) * H, tok = G * N * kD * 2, np = N_prev;
    if ((s = check_disjoint({{pool, int64_t(n_slots) * H * (kStateBytes / 2)},
                             {out, G * N * kD * 4}, {vtilde, G * N * kD * 4}, {gamma, G * N * 4}},
                            {{slots, int64_t(B) * 4}, {vtilde_prev, G * np * kD * 4},
                             {k_prev, G * np * kD * 2}, {gamma_prev, G * np * 4},
                             {accepted_prev, int64_t(B) * 4}, {q, tok}, {k, tok}, {v, tok},
                             {alpha, G * N * 2}, {beta, G * N * 2}})) != TREEWY_OK) {
      return s;
    }
  }
  VerifyArgs a{static_cast<const float*>(pool), q, k, v, alpha, beta, out, vtilde, gamma, B, H, 0,
               static_cast<float*>(pool), vtilde_prev, k_prev, gamma_prev, accepted_prev, N_prev,
               slots, n_slots, 1};
  return launch_status(launch_commit_verify(a, tree, prev, stream));
}

extern "C" int treewy_commit_verify_bf16state_pool_trees(
    void* pool, int n_slots, const int32_t* slots, const float* vtilde_prev, const void* k_prev,
    const float* gamma_prev, const int32_t* accepted_prev, const void* trees_prev, int N_prev,
    int depth_prev, const void* q, const void* k, const void* v, const void* alpha,
    const void* beta, const void* trees, int N, int depth, int B, int H, float* out, float* vtilde,
    float* gamma, treewy_dtype dtype, hipStream_t stream) {
  int s = check_sizes(B, H);
  if (s != TREEWY_OK) return s;
  if (n_slots < 0) return TREEWY_ERR_ARG;
  if ((s = check_sizes(n_slots, H)) != TREEWY_OK) return s;
  if (N < 1 || N > kMaxNodes || N_prev < 1 || N_prev > kMaxNodes) return TREEWY_ERR_ARG;
  if (depth < 0 || depth >= N || depth_prev < 0 || depth_prev >= N_prev) return TREEWY_ERR_ARG;
  if (dtype != TREEWY_BF16) return TREEWY_ERR_DTYPE;
  if (B == 0 || H == 0) return TREEWY_OK;
  if (n_slots < 1) return TREEWY_ERR_ARG;
  if ((s = check_all({pool, slots, vtilde_prev, k_prev, gamma_prev, accepted_prev, trees_prev, q,
                      k, v, alpha, beta, trees, out, vtilde, gamma})) != TREEWY_OK) {
    return s;
  }
  {
    const int64_t G = int64_t(B) * H, tok = G * N * kD * 2, np = N_prev;
    const int64_t desc = int64_t(B) * int64_t(sizeof(TreeArgs));
    if ((s = check_disjoint({{pool, int64_t(n_slots) * H * (kStateBytes / 2)},
                             {out, G * N * kD * 4}, {vtilde, G * N * kD * 4}, {gamma, G * N * 4}},
                            {{slots, int64_t(B) * 4}, {vtilde_prev, G * np * kD * 4},
                             {k_prev, G * np * kD * 2}, {gamma_prev, G * np * 4},
                             {accepted_prev, int64_t(B) * 4}, {trees_prev, desc}, {q, tok}, {k, tok},
                             {v, tok}, {alpha, G * N * 2}, {beta, G * N * 2},
                             {trees, desc}})) != TREEWY_OK) {
      return s;
    }
  }
  TreeArgs bound{}, prev_bound{};
  bound.n = N;
  bound.max_depth = depth;
  prev_bound.n = N_prev;
  prev_bound.max_depth = depth_prev;
  VerifyArgs a{static_cast<const float*>(pool), q, k, v, alpha, beta, out, vtilde, gamma, B, H, 0,
               static_cast<float*>(pool), vtilde_prev, k_prev, gamma_prev, accepted_prev, N_prev,
               slots, n_slots, 1};
  a.tok_b = N;
  a.tok_b_prev = N_prev;
  a.trees = static_cast<const TreeArgs*>(trees);
  a.trees_prev = static_cast<const TreeArgs*>(trees_prev);
  return launch_status(launch_commit_verify_pool_trees(a, bound, prev_bound, stream));
}

namespace {

// Checks shared by both chunked-prefill entry points (everything but the
// workspace); sets *done when the call is a valid no-op.
int prefill_chain_check(const float* S, const void* q, const void* k, const void* v,
                        const void* alpha, const void* beta, int B, int T, int H, int chunk,
                        const float* out, treewy_dtype dtype, bool* done) {
  *done = false;
  int s = check_sizes(B, H);
  if (s != TREEWY_OK) return s;
  if (T < 0 || chunk < 1 || chunk > kMaxNodes) return TREEWY_ERR_ARG;
  if ((s = check_dtype(dtype)) != TREEWY_OK) return s;
  if (B == 0 || H == 0 || T == 0) {
    *done = true;
    return TREEWY_OK;
  }
  return check_all({S, q, k, v, alpha, beta, out});
}

// Floats per pseudo-value buffer and per gate buffer (two of each).
int64_t prefill_vt_half(int B, int H, int chunk) { return int64_t(B) * H * chunk * kD; }
int64_t prefill_gm_half(int B, int H, int chunk) { return (int64_t(B) * H * chunk + 3) / 4 * 4; }

// The launches of a chunked prefill: ceil(T / chunk) commit-then-verify
// launches and a final commit, passing pseudo-values and gates between them
// in work_vtilde / work_gamma.
int prefill_chain_enqueue(float* S, const void* q, const void* k, const void* v,
                          const void* alpha, const void* beta, int B, int T, int H, int chunk,
                          float* out, float* work_vtilde, float* work_gamma, treewy_dtype dtype,
                          hipStream_t stream) {
  int s = TREEWY_OK;
  const int64_t ib = in_bytes(dtype);
  const int64_t row = int64_t(H) * kD;  // one token of q/k/v/out
  const int64_t vt_half = prefill_vt_half(B, H, chunk);
  const int64_t gm_half = prefill_gm_half(B, H, chunk);
  const char* qb = static_cast<const char*>(q);
  const char* kb = static_cast<const char*>(k);
  const char* vb = static_cast<const char*>(v);
  const char* ab = static_cast<const char*>(alpha);
  const char* bb = static_cast<const char*>(beta);
  const int nchunks = (T + chunk - 1) / chunk;
  TreeArgs tree, prev;
  int32_t par[kMaxNodes];
  for (int t = 0; t < kMaxNodes; ++t) par[t] = t - 1;
  for (int c = 0; c < nchunks; ++c) {
    const int64_t t0 = int64_t(c) * chunk;
    const int n = int(T - t0 < chunk ? T - t0 : chunk);
    if ((s = build_tree(par, n, &tree)) != TREEWY_OK) return s;
    float* vt = work_vtilde + (c & 1) * vt_half;
    float* gm = work_gamma + (c & 1) * gm_half;
    VerifyArgs a{S, qb + t0 * row * ib, kb + t0 * row * ib, vb + t0 * row * ib,
                 ab + t0 * H * ib, bb + t0 * H * ib, out + t0 * row, vt, gm, B, H,
                 dtype == TREEWY_F32};
    a.tok_b = T;
    hipError_t e;
    if (c == 0) {
      e = launch_verify(a, tree, stream);
    } else {
      // commit the previous chunk's last token into S, then verify this chunk
      a.S_out = S;
      a.vt_prev = work_vtilde + ((c - 1) & 1) * vt_half;
      a.k_prev = kb + (t0 - chunk) * row * ib;
      a.gamma_prev = work_gamma + ((c - 1) & 1) * gm_half;
      a.acc_prev = nullptr;
      a.n_prev = chunk;
      a.tok_b_prev = T;
      e = launch_commit_verify(a, tree, prev, stream);
    }
    if ((s = launch_status(e)) != TREEWY_OK) return s;
    prev = tree;
  }
  const int64_t tl = int64_t(nchunks - 1) * chunk;
  CommitArgs ca{S, work_vtilde + ((nchunks - 1) & 1) * vt_half, kb + tl * row * ib,
                work_gamma + ((nchunks - 1) & 1) * gm_half, nullptr, S, B, H,
                dtype == TREEWY_F32, T};
  return launch_status(launch_commit(ca, prev, stream));
}

// S and out (and the workspace, when the caller gives one) are disjoint from
// the token inputs and from one another.
int prefill_chain_disjoint(const float* S, const void* q, const void* k, const void* v,
                           const void* alpha, const void* beta, int B, int T, int H, int chunk,
                           const float* out, const float* work_vtilde, const float* work_gamma,
                           treewy_dtype dtype) {
  const int64_t BT = int64_t(B) * T * H, ib = in_bytes(dtype);
  const int64_t vt_bytes = work_vtilde ? 2 * prefill_vt_half(B, H, chunk) * 4 : 0;
  const int64_t gm_bytes = work_gamma ? 2 * prefill_gm_half(B, H, chunk) * 4 : 0;
  return check_disjoint({{S, int64_t(B) * H * kStateBytes}, {out, BT * kD * 4},
                         {work_vtilde, vt_bytes}, {work_gamma, gm_bytes}},
                        {{q, BT * kD * ib}, {k, BT * kD * ib}, {v, BT * kD * ib},
                         {alpha, BT * ib}, {beta, BT * ib}});
}

}  // namespace

extern "C" int treewy_prefill_chain(float* S, const void* q, const void* k, const void* v,
                                    const void* alpha, const void* beta, int B, int T, int H,
                                    int chunk, float* out, float* work_vtilde, float* work_gamma,
                                    treewy_dtype dtype, hipStream_t stream) {
  bool done = false;
  int s = prefill_chain_check(S, q, k, v, alpha, beta, B, T, H, chunk, out, dtype, &done);
  if (s != TREEWY_OK || done) return s;
  if ((s = check_all({work_vtilde, work_gamma})) != TREEWY_OK) return s;
  if ((s = prefill_chain_disjoint(S, q, k, v, alpha, beta, B, T, H, chunk, out, work_vtilde,
                                  work_gamma, dtype)) != TREEWY_OK) {
    return s;
  }
  return prefill_chain_enqueue(S, q, k, v, alpha, beta, B, T, H, chunk, out, work_vtilde,
                               work_gamma, dtype, stream);
}

extern "C" int treewy_prefill_chain_noalloc(float* S, const void* q, const void* k,
                                            const void* v, const void* alpha, const void* beta,
                                            int B, int T, int H, int chunk, float* out,
                                            treewy_dtype dtype, hipStream_t stream) {
  bool done = false;
  int s = prefill_chain_check(S, q, k, v, alpha, beta, B, T, H, chunk, out, dtype, &done);
  if (s != TREEWY_OK || done) return s;
  const int64_t vt_half = prefill_vt_half(B, H, chunk);
  const int64_t gm_half = prefill_gm_half(B, H, chunk);
  if (2 * (vt_half + gm_half) * 4 > int64_t(kScratchBytes)) return TREEWY_ERR_SIZE;
  if ((s = prefill_chain_disjoint(S, q, k, v, alpha, beta, B, T, H, chunk, out, nullptr, nullptr,
                                  dtype)) != TREEWY_OK) {
    return s;
  }
  // the scratch is taken on the current device: the stream must be one of its
  int cur = -1, sdev = -1;
  if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess) {
    return TREEWY_ERR_LAUNCH;
  }
  if (cur != sdev) return TREEWY_ERR_ARG;
  float* work = nullptr;
  size_t bytes = 0;
  if (scratch_buffer(&work, &bytes) != hipSuccess) return TREEWY_ERR_LAUNCH;
  if (2 * (vt_half + gm_half) * 4 > int64_t(bytes)) return TREEWY_ERR_SIZE;
  return prefill_chain_enqueue(S, q, k, v, alpha, beta, B, T, H, chunk, out, work,
                               work + 2 * vt_half, dtype, stream);
}

extern "C" int treewy_commit(const float* S0, const float* vtilde, const void* k,
                             const float* gamma, const int32_t* accepted, const int32_t* parent,
                             int B, int H, int N, float* S_out, treewy_dtype dtype, hipStream_t stream) {
  int s = check_sizes(B, H);
  if (s != TREEWY_OK) return s;
  TreeArgs tree;
  if ((s = build_tree(parent, N, &tree)) != TREEWY_OK) return s;
  if ((s = check_dtype(dtype)) != TREEWY_OK) return s;
  if (B == 0 || H == 0) return TREEWY_OK;
  if ((s = check_all({S0, vtilde, k, gamma, accepted, S_out})) != TREEWY_OK) return s;
  {
    const int64_t G = int64_t(B) * H;
    const bool in_place = static_cast<const void*>(S_out) == static_cast<const void*>(S0);
    if ((s = check_disjoint({{S_out, G * kStateBytes}},
                            {{S0, in_place ? 0 : G * kStateBytes}, {vtilde, G * N * kD * 4},
                             {k, G * N * kD * in_bytes(dtype)}, {gamma, G * N * 4},
                             {accepted, int64_t(B) * 4}})) != TREEWY_OK) {
      return s;
    }
  }
  CommitArgs a{S0, vtilde, k, gamma, accepted, S_out, B, H, dtype == TREEWY_F32};
  return launch_status(launch_commit(a, tree, stream));
}

extern "C" int treewy_store_all(const float* S0, const void* q, const void* k, const void* v,
                                const void* alpha, const void* beta, const int32_t* parent,
                                int B, int H, int N, float* out, float* snapshots, treewy_dtype dtype,
                                hipStream_t stream) {
  int s = check_sizes(B, H);
  if (s != TREEWY_OK) return s;
  TreeArgs tree;
  if ((s = build_tree(parent, N, &tree)) != TREEWY_OK) return s;
  if ((s = check_dtype(dtype)) != TREEWY_OK) return s;
  if (B == 0 || H == 0) return TREEWY_OK;
  if ((s = check_all({S0, q, k, v, alpha, beta, out, snapshots})) != TREEWY_OK) return s;
  {
    const int64_t G = int64_t(B) * H, tok = G * N * kD * in_bytes(dtype), gate = G * N * in_bytes(dtype);
    if ((s = check_disjoint({{out, G * N * kD * 4}, {snapshots, G * (N + 1) * kStateBytes}},
                            {{S0, G * kStateBytes}, {q, tok}, {k, tok}, {v, tok}, {alpha, gate},
                             {beta, gate}})) != TREEWY_OK) {
      return s;
    }
  }
  StoreAllArgs a{S0, q, k, v, alpha, beta, out, snapshots, B, H, dtype == TREEWY_F32};
  return launch_status(launch_store_all(a, tree, stream));
}

extern "C" int treewy_store_all_select(const float* snapshots, const int32_t* accepted, int B,
                                       int H, int N, float* S_out, hipStream_t stream) {
  int s = check_sizes(B, H);
  if (s != TREEWY_OK) return s;
  if (N < 1 || N > kMaxNodes) return TREEWY_ERR_ARG;
  if (B == 0 || H == 0) return TREEWY_OK;
  if ((s = check_all({snapshots, accepted, S_out})) != TREEWY_OK) return s;
  {
    const int64_t G = int64_t(B) * H;
    if ((s = check_disjoint({{S_out, G * kStateBytes}},
                            {{snapshots, G * (N + 1) * kStateBytes},
                             {accepted, int64_t(B) * 4}})) != TREEWY_OK) {
      return s;
    }
  }
  SelectArgs a{snapshots, accepted, S_out, B, H, N};
  return launch_status(launch_store_all_select(a, stream));
}

extern "C" const char* treewy_status_str(int status) {
  switch (status) {
    case TREEWY_OK: return "ok";
    case TREEWY_ERR_ARG: return "invalid argument (null pointer, negative size or N outside 1..64)";
    case TREEWY_ERR_TREE: return "parent[] is not a tree in DFS pre-order";
    case TREEWY_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case TREEWY_ERR_DTYPE: return "unknown dtype code";
    case TREEWY_ERR_LAUNCH: return "HIP kernel launch failed";
    case TREEWY_ERR_SIZE: return "sizes exceed the supported index range";
    default: return "unknown status";
  }
}
