// Full-state snapshotting baseline ("store_all") for gfx950.
//
// "TreeWY: Speculative Verification for Gated DeltaNet Hybrids", paperpeel
// section 2, first prior-work bullet: one recurrent-state snapshot per draft
// position, rollback by indexing the accepted one.  The walk is the gated delta
// rule in the pseudo-value form of section 3 ("Key rewrite"):
//   vt_t = beta_t (v_t - alpha_t S_p k_t),  S_t = alpha_t S_p + vt_t k_t^T,
//   o_t  = S_t q_t = alpha_t (S_p q_t) + vt_t (k_t . q_t).
//
// Rows of the state evolve independently, so a (sequence, head) is split over
// 8 workgroups of 16 rows; 16 lanes (one DPP row) share a state row, 8 columns
// each, and reduce their partial dot products with DPP.  Parent states are
// kept in registers, indexed by depth (in a pre-order the parent of t is the
// latest node at depth(t)-1); slot DS-1 holds every deeper node, and a parent
// that has been overwritten there is re-read from its own snapshot.  Each
// (N+1) x 64 KiB snapshot stream is written once with 256 B contiguous per row.
// The small rows (k, q, this workgroup's part of v, the gates) are staged in
// LDS before the walk, so the walk itself waits on no memory.
#include "../../include/treewy.h"
#include "device_common.h"
#include "treewy_internal.h"

namespace treewy {
namespace {

constexpr int kRowsPerWG = 16;
constexpr int kSaThreads = 16 * kRowsPerWG;  // 16 lanes per state row
constexpr int kGroups = kD / kRowsPerWG;      // row groups per head

// Snapshot rows and outputs are written once and only read by a later kernel
// (snapshots by the select), so they go out non-temporal (they would
// otherwise sit dirty in L2 and the Infinity Cache and drain into the
// following kernels).
__device__ __forceinline__ void st_stream(float* p, const float4& v) {
  __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4*>(p));
}

template <bool F32>
struct Raw4 {
  using T = uint2;  // 4 bf16
};
template <>
struct Raw4<true> {
  using T = float4;
};

template <bool F32>
__device__ __forceinline__ typename Raw4<F32>::T load_raw4(const void* base, int64_t idx) {
  if constexpr (F32) {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
  } else {
    return *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
  }
}

__device__ __forceinline__ void widen(const float4& r, float* x) {
  x[0] = r.x; x[1] = r.y; x[2] = r.z; x[3] = r.w;
}
__device__ __forceinline__ void widen(const uint2& r, float* x) {
  x[0] = __uint_as_float(r.x << 16);
  x[1] = __uint_as_float(r.x & 0xffff0000u);
  x[2] = __uint_as_float(r.y << 16);
  x[3] = __uint_as_float(r.y & 0xffff0000u);
}

template <bool F32>
__device__ __forceinline__ float load_raw1(const void* base, int64_t idx) {
  return load_in<F32>(base, idx);
}

// The small rows of one (sequence, head) -- k and q rows, this workgroup's
// 16 entries of each v row, the gates -- are staged into LDS up front (all
// loads issued before one wait), so the node walk runs from LDS and only the
// snapshot stream touches HBM inside it.  NMAX bounds N for the LDS layout.
template <bool F32IN, int NMAX>
struct StoreAllLayout {
  static constexpr int IB = F32IN ? 4 : 2;
  static constexpr int ROW = kD * IB;                      // bytes per k/q row
  static constexpr int OFF_Q = NMAX * ROW;
  static constexpr int OFF_V = 2 * NMAX * ROW;             // [NMAX][16] inputs
  static constexpr int OFF_AL = OFF_V + NMAX * kRowsPerWG * IB;
  static constexpr int OFF_BE = OFF_AL + NMAX * 4;
  static constexpr int OFF_O = OFF_BE + NMAX * 4;          // [NMAX][16] outputs
  static constexpr int OFF_DEPTH = OFF_O + NMAX * kRowsPerWG * 4;
  static constexpr int OFF_PARENT = OFF_DEPTH + NMAX;
  static constexpr int TOTAL = OFF_PARENT + NMAX;
};

// Workgroup -> (head, 16-row group).  The 8 row groups of a head read the
// same k and q rows, so they run on one XCD (whose L2 then serves the rows
// after the first read) and close in time.  Workgroups go to the 8 XCDs
// round-robin, block i to XCD i % 8; head h's groups are blocks
// 64 (h / 8) + 8 g + h % 8, g = 0..7, when the head count is a multiple of 8
// (otherwise the groups of a head are 8 consecutive blocks).
__device__ __forceinline__ void head_and_group(int& gh, int& grp) {
  const int bid = static_cast<int>(blockIdx.x);
  const int G = static_cast<int>(gridDim.x) / kGroups;
  if ((G & 7) == 0) {
    const int j = bid >> 3;
    gh = (j / kGroups) * 8 + (bid & 7);
    grp = j % kGroups;
  } else {
    gh = bid / kGroups;
    grp = bid % kGroups;
  }
}

// DEEP: the tree has nodes at depth >= DS - 1, whose states share the deepest
// register slot, so a parent may have to be re-read from its snapshot.  Only
// such trees compile that re-read: its loads make the compiler wait on the
// vector-memory counter in the walk, and that counter also counts the
// snapshot stores, so every node step would wait for all earlier stores.
template <bool F32IN, int DS, int NMAX, bool DEEP>
__global__ __launch_bounds__(kSaThreads) void store_all_kernel(const StoreAllArgs a, const TreeArgs tree) {
  using R4 = typename Raw4<F32IN>::T;
  using Lay = StoreAllLayout<F32IN, NMAX>;
  constexpr int IB = Lay::IB;
  __shared__ __attribute__((aligned(16))) unsigned char smem[Lay::TOTAL];
  const int N = tree.n;
  const int H = a.H;
  int gh, grp;
  head_and_group(gh, grp);
  const int b = gh / H;
  const int h = gh - b * H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j16 = lane & 15;
  const int m0 = grp * kRowsPerWG;
  const int mr = wave * 4 + (lane >> 4);  // row inside the workgroup
  const int m = m0 + mr;
  const int c0 = 4 * j16;
  const int c1 = 64 + 4 * j16;
  constexpr int64_t kBlock = kD * kD;
  const int64_t head = static_cast<int64_t>(gh) * kBlock;
  float* snap = a.snapshots + static_cast<int64_t>(gh) * (N + 1) * kBlock + m * kD;
  const int64_t tokstride = static_cast<int64_t>(H) * kD;
  const int64_t tok0 = (static_cast<int64_t>(b) * N * H + h) * kD;
  const int64_t gate0 = static_cast<int64_t>(b) * N * H + h;
  const unsigned char* kb = static_cast<const unsigned char*>(a.k);
  const unsigned char* qb = static_cast<const unsigned char*>(a.q);
  const unsigned char* vb = static_cast<const unsigned char*>(a.v);

  // ---- staging: k/q rows in 16-byte chunks, up to 8 per thread per round.
  // The chunk count per thread is a compile-time bound (NMAX rows) and every
  // lane loads (indices past the rows clamped to the last chunk), so the
  // rounds unroll and the chunks stay in registers.  (With a loop bound known
  // only at run time the chunks went through private scratch memory: one
  // load, a wait and a scratch write per chunk, and scratch writes that
  // reached HBM, 2N x 256 B per row group.)
  constexpr int CPR = kD * IB / 16;
  constexpr int PER = (2 * NMAX * CPR + kSaThreads - 1) / kSaThreads;
  constexpr int RB = PER < 8 ? PER : 8;
  const int kq_chunks = 2 * N * CPR;
#pragma unroll
  for (int base = 0; base < PER; base += RB) {
    uint4 r[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      int idx = (base + u) * kSaThreads + tid;
      idx = idx < kq_chunks ? idx : kq_chunks - 1;
      const int row = idx / CPR;
      const int j = idx - row * CPR;
      const unsigned char* src = row < N ? kb : qb;
      const int t = row < N ? row : row - N;
      r[u] = *reinterpret_cast<const uint4*>(src + (tok0 + t * tokstride) * IB + 16 * j);
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int idx = (base + u) * kSaThreads + tid;
      if (idx < kq_chunks) {
        const int row = idx / CPR;
        const int off = row < N ? row * Lay::ROW : Lay::OFF_Q + (row - N) * Lay::ROW;
        *reinterpret_cast<uint4*>(smem + off + 16 * (idx - row * CPR)) = r[u];
      }
    }
  }
  // v: this workgroup's 16 entries of each row (IB 16-byte chunks per node);
  // gates: alpha for tid < N, beta for N <= tid < 2N
  constexpr int VCH = kRowsPerWG * IB / 16;
  uint4 vr = make_uint4(0, 0, 0, 0);
  if (tid < N * VCH) {
    const int t = tid / VCH;
    const int j = tid - t * VCH;
    vr = *reinterpret_cast<const uint4*>(vb + (tok0 + t * tokstride + m0) * IB + 16 * j);
  }
  float gate = 0.f;
  if (tid < 2 * N) {
    const int t = tid < N ? tid : tid - N;
    gate = load_in<F32IN>(tid < N ? a.alpha : a.beta, gate0 + static_cast<int64_t>(t) * H);
  }

  float Sp[8];
  {
    const float4 x0 = *reinterpret_cast<const float4*>(a.S0 + head + m * kD + c0);
    const float4 x1 = *reinterpret_cast<const float4*>(a.S0 + head + m * kD + c1);
    st_stream(snap + c0, x0);
    st_stream(snap + c1, x1);
    widen(x0, Sp);
    widen(x1, Sp + 4);
  }
  // the topology to LDS: read from the kernel arguments inside the walk, a
  // node's depth and parent were vector loads whose wait also waited for every
  // snapshot store before them (the wait counter counts stores too), which
  // serialised the snapshot stream node by node
  int8_t* depth_s = reinterpret_cast<int8_t*>(smem + Lay::OFF_DEPTH);
  int8_t* parent_s = reinterpret_cast<int8_t*>(smem + Lay::OFF_PARENT);
  if (tid < N) {
    depth_s[tid] = tree.depth[tid];
    parent_s[tid] = tree.parent[tid];
  }
  if (tid < N * VCH) *reinterpret_cast<uint4*>(smem + Lay::OFF_V + 16 * tid) = vr;
  if (tid < 2 * N) reinterpret_cast<float*>(smem + (tid < N ? Lay::OFF_AL : Lay::OFF_BE))[tid < N ? tid : tid - N] = gate;
  __syncthreads();

  const float* al_s = reinterpret_cast<const float*>(smem + Lay::OFF_AL);
  const float* be_s = reinterpret_cast<const float*>(smem + Lay::OFF_BE);
  float* o_s = reinterpret_cast<float*>(smem + Lay::OFF_O);
  float slot[DS][8];
#pragma unroll
  for (int e = 0; e < DS; ++e) {
#pragma unroll
    for (int x = 0; x < 8; ++x) slot[e][x] = 0.f;
  }

  for (int t = 0; t < N; ++t) {
    const int d = depth_s[t];
    if (t > 0) {
      const int p = parent_s[t];
      const int dp = depth_s[p];
      if (dp < DS - 1) {
#pragma unroll
        for (int e = 0; e < DS - 1; ++e) {
          if (e == dp) {
#pragma unroll
            for (int x = 0; x < 8; ++x) Sp[x] = slot[e][x];
          }
        }
      } else if constexpr (DEEP) {
        if (p == t - 1) {
#pragma unroll
          for (int x = 0; x < 8; ++x) Sp[x] = slot[DS - 1][x];
        } else {
          // parent state was overwritten in the deepest slot: read back this
          // thread's own elements of the parent's snapshot
          __threadfence();
          const float* ps = snap + static_cast<int64_t>(p + 1) * kBlock;
          widen(*reinterpret_cast<const float4*>(ps + c0), Sp);
          widen(*reinterpret_cast<const float4*>(ps + c1), Sp + 4);
        }
      }
    }

    const unsigned char* krow = smem + t * Lay::ROW;
    const unsigned char* qrow = smem + Lay::OFF_Q + t * Lay::ROW;
    float kx[8], qx[8];
    widen(*reinterpret_cast<const R4*>(krow + c0 * IB), kx);
    widen(*reinterpret_cast<const R4*>(krow + c1 * IB), kx + 4);
    widen(*reinterpret_cast<const R4*>(qrow + c0 * IB), qx);
    widen(*reinterpret_cast<const R4*>(qrow + c1 * IB), qx + 4);
    float vv;
    if constexpr (F32IN) {
      vv = reinterpret_cast<const float*>(smem + Lay::OFF_V)[t * kRowsPerWG + mr];
    } else {
      vv = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(smem + Lay::OFF_V)[t * kRowsPerWG + mr]);
    }
    const float al = al_s[t];
    const float be = be_s[t];
    float pk = 0.f, pq = 0.f, kq = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      pk += Sp[x] * kx[x];
      pq += Sp[x] * qx[x];
      kq += kx[x] * qx[x];
    }
    pk = row16_sum(pk);
    pq = row16_sum(pq);
    kq = row16_sum(kq);
    const float vt = be * (vv - al * pk);
    float St[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) St[x] = al * Sp[x] + vt * kx[x];
    const float o = al * pq + vt * kq;

    float* ds = snap + static_cast<int64_t>(t + 1) * kBlock;
    st_stream(ds + c0, make_float4(St[0], St[1], St[2], St[3]));
    st_stream(ds + c1, make_float4(St[4], St[5], St[6], St[7]));
    if (j16 == 0) o_s[t * kRowsPerWG + mr] = o;

    const int sd = d < DS - 1 ? d : DS - 1;
#pragma unroll
    for (int e = 0; e < DS; ++e) {
      if (e == sd) {
#pragma unroll
        for (int x = 0; x < 8; ++x) slot[e][x] = St[x];
      }
    }
  }

  // outputs: 64 contiguous bytes per node for this workgroup's 16 rows
  // (non-temporal like the snapshots: written once, read by a later kernel)
  __syncthreads();
  constexpr int OPN = kRowsPerWG / 4;  // float4 per node
  if (tid < OPN * N) {
    const int t = tid / OPN;
    const int c = 4 * (tid - t * OPN);
    st_stream(a.out + tok0 + t * tokstride + m0 + c, *reinterpret_cast<const float4*>(o_s + t * kRowsPerWG + c));
  }
}

__global__ __launch_bounds__(256) void select_kernel(const SelectArgs a) {
  const int H = a.H;
  const int N = a.N;
  const int gh = blockIdx.x;
  const int b = gh / H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = 4 * (lane & 31);
  const int rsub = 2 * wave + (lane >> 5);
  const int rbase = blockIdx.y * 32;
  constexpr int64_t kBlock = kD * kD;
  float* dst = a.S_out + static_cast<int64_t>(gh) * kBlock;
  const int an = a.accepted[b];
  if (an < 0 || an >= N) {
    const float nan = qnan();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = rbase + 8 * i + rsub;
      *reinterpret_cast<float4*>(dst + m * kD + c) = make_float4(nan, nan, nan, nan);
    }
    return;
  }
  const float* src = a.snapshots + (static_cast<int64_t>(gh) * (N + 1) + an + 1) * kBlock;
  float4 x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = rbase + 8 * i + rsub;
    const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + m * kD + c));
    x[i] = make_float4(y.x, y.y, y.z, y.w);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = rbase + 8 * i + rsub;
    st_stream(dst + m * kD + c, x[i]);
  }
}

template <bool F32IN, int DS, bool DEEP>
hipError_t launch_sa_deep(const StoreAllArgs& a, const TreeArgs& tree, hipStream_t s) {
  static_assert(kGroups * kRowsPerWG == kD && kSaThreads <= 1024, "row groups");
  const dim3 grid(a.B * a.H * kGroups);
  // the LDS layout is sized for the node count, so that as many workgroups
  // fit on a CU as the registers allow
  if (tree.n <= 16) {
    hipLaunchKernelGGL((store_all_kernel<F32IN, DS, 16, DEEP>), grid, dim3(kSaThreads), 0, s, a, tree);
  } else if (tree.n <= 40) {
    hipLaunchKernelGGL((store_all_kernel<F32IN, DS, 40, DEEP>), grid, dim3(kSaThreads), 0, s, a, tree);
  } else {
    hipLaunchKernelGGL((store_all_kernel<F32IN, DS, kMaxNodes, DEEP>), grid, dim3(kSaThreads), 0, s, a, tree);
  }
  return hipGetLastError();
}

template <bool F32IN, int DS>
hipError_t launch_sa(const StoreAllArgs& a, const TreeArgs& tree, hipStream_t s) {
  // a tree of depth < DS has every parent at depth <= DS - 2: never in the
  // shared deepest slot
  return tree.max_depth < DS ? launch_sa_deep<F32IN, DS, false>(a, tree, s)
                             : launch_sa_deep<F32IN, DS, true>(a, tree, s);
}

}  // namespace

hipError_t launch_store_all(const StoreAllArgs& a, const TreeArgs& tree, hipStream_t s) {
  // 4 register slots cover depth <= 3 without any re-read; deeper trees fall
  // back on the snapshot re-read for parents that are not the previous node.
  return a.f32_inputs ? launch_sa<true, 4>(a, tree, s) : launch_sa<false, 4>(a, tree, s);
}

hipError_t launch_store_all_select(const SelectArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(a.B * a.H, kD / 32), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace treewy
