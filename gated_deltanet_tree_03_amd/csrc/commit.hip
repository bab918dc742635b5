// TreeWY commit kernel for gfx950: rebuild only the accepted state,
//   S_a = Gamma_a S0 + sum_{j ancestor-or-self of a} (Gamma_a / Gamma_j) vt_j k_j^T
// ("TreeWY: Speculative Verification for Gated DeltaNet Hybrids": mlsanity
// abstract and review page "Method" -- the accepted node's state is rebuilt from
// the same solve; paperpeel section 3 "Key rewrite" for the decay-weighted sum).
//
// A pure stream: 64 KiB of S0 read and 64 KiB of S_out written per (sequence,
// head), plus depth(a)+1 rows of vt and k.  Four workgroups per head, 32 rows
// each; every wave instruction touches 1 KiB contiguous (2 rows x 512 B).  S0
// is read once and S_out is not read back here, so both go non-temporal: the
// dirty state then does not linger in L2 / the Infinity Cache and drain into
// the next kernel's read stream.  Each thread reads and then writes the same
// elements, so S_out may alias S0.
#include "../../include/treewy.h"
#include "device_common.h"
#include "treewy_internal.h"

namespace treewy {
namespace {

constexpr int kRowsPerWG = 32;
constexpr int kRowIters = kRowsPerWG / 8;  // float4 per thread
constexpr int kPathChunk = 8;
static_assert(kRowsPerWG == 32 && kPathChunk * 32 == 256,
              "the path-row prefetch maps 256 threads onto 8 path nodes x 32 rows");

__device__ __forceinline__ float4 ld4(const float* p) {
  const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void st4(float* p, const float4& v) {
  const f32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}

template <bool F32IN>
__global__ __launch_bounds__(256) void commit_kernel(const CommitArgs a, const TreeArgs tree) {
  __shared__ float vt_s[kPathChunk][kRowsPerWG];
  __shared__ float kc_s[kPathChunk][kD];

  const int N = tree.n;
  const int H = a.H;
  const int gh = blockIdx.x;
  const int b = gh / H;
  const int h = gh - b * H;
  const int rbase = blockIdx.y * kRowsPerWG;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = 4 * (lane & 31);
  const int rsub = 2 * wave + (lane >> 5);  // row offset 0..7 inside each group of 8 rows
  const int64_t head = static_cast<int64_t>(gh) * (kD * kD);

  // The accepted node, its gate and the first chunk of its path rows are
  // loaded before S0: vector loads return in order, and rows loaded behind
  // the S0 block would cost a second memory round trip after it.  Lane
  // tid < 8*32 holds path node e = tid / 32: vt entry rbase + tid % 32 and
  // k columns 4*(tid % 32) .. +3.
  const int an = a.accepted ? a.accepted[b] : N - 1;  // none given: the last node
  const bool ok = an >= 0 && an < N;  // uniform per workgroup
  const float* gam = a.gamma + static_cast<int64_t>(gh) * N;
  const int64_t tokstride = static_cast<int64_t>(H) * kD;
  const int64_t tok0 = (static_cast<int64_t>(b) * (a.tok_b ? a.tok_b : N) * H + h) * kD;
  const float* vt_head = a.vtilde + static_cast<int64_t>(gh) * N * kD;
  const uint64_t path = ok ? (tree.anc[an] | (1ull << an)) : 0ull;  // the root-to-a path
  const float Ga = ok ? gam[an] : 0.f;
  float pv = 0.f, pg = 1.f;
  float4 pk = make_float4(0.f, 0.f, 0.f, 0.f);
  {
    uint64_t r = path;
    const int e = tid >> 5;
    for (int z = 0; z < e; ++z) r &= r - 1ull;
    if (r != 0ull) {  // e < 8 always: 256 threads
      const int j = __builtin_ctzll(r);
      pv = vt_head[j * kD + rbase + (tid & 31)];
      pk = load_in4<F32IN>(a.k, tok0 + j * tokstride + 4 * (tid & 31));
      pg = gam[j];
    }
  }

  float4 acc[kRowIters];
#pragma unroll
  for (int i = 0; i < kRowIters; ++i) {
    const int m = rbase + 8 * i + rsub;
    acc[i] = ld4(a.S0 + head + m * kD + c);
  }

  float* dst = a.S_out + head;
  if (!ok) {
    const float nan = qnan();
#pragma unroll
    for (int i = 0; i < kRowIters; ++i) {
      const int m = rbase + 8 * i + rsub;
      st4(dst + m * kD + c, make_float4(nan, nan, nan, nan));
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < kRowIters; ++i) {
    acc[i].x *= Ga;
    acc[i].y *= Ga;
    acc[i].z *= Ga;
    acc[i].w *= Ga;
  }

  uint64_t rest = path;
  bool first = true;
  while (rest != 0ull) {
    // next chunk of up to 8 path nodes, lowest index first
    uint64_t chunk = 0ull;
    int L = 0;
    {
      uint64_t r = rest;
      while (r != 0ull && L < kPathChunk) {
        chunk |= r & (~r + 1ull);
        r &= r - 1ull;
        ++L;
      }
      rest = r;
    }
    if (first) {
      if (tid < L * 32) {
        const int e = tid >> 5;
        const float w = Ga / pg;
        vt_s[e][tid & 31] = pv;
        *reinterpret_cast<float4*>(&kc_s[e][4 * (tid & 31)]) =
            make_float4(w * pk.x, w * pk.y, w * pk.z, w * pk.w);
      }
      first = false;
    } else {
      for (int idx = tid; idx < L * kRowsPerWG; idx += 256) {
        const int e = idx / kRowsPerWG;
        const int mm = idx - e * kRowsPerWG;
        uint64_t r = chunk;
        for (int z = 0; z < e; ++z) r &= r - 1ull;
        const int j = __builtin_ctzll(r);
        vt_s[e][mm] = vt_head[j * kD + rbase + mm];
      }
      for (int idx = tid; idx < L * kD; idx += 256) {
        const int e = idx / kD;
        const int cc = idx - e * kD;
        uint64_t r = chunk;
        for (int z = 0; z < e; ++z) r &= r - 1ull;
        const int j = __builtin_ctzll(r);
        kc_s[e][cc] = (Ga / gam[j]) * load_in<F32IN>(a.k, tok0 + j * tokstride + cc);
      }
    }
    __syncthreads();
    for (int e = 0; e < L; ++e) {
      const float4 kv = *reinterpret_cast<const float4*>(&kc_s[e][c]);
#pragma unroll
      for (int i = 0; i < kRowIters; ++i) {
        const float w = vt_s[e][8 * i + rsub];
        acc[i].x += w * kv.x;
        acc[i].y += w * kv.y;
        acc[i].z += w * kv.z;
        acc[i].w += w * kv.w;
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < kRowIters; ++i) {
    const int m = rbase + 8 * i + rsub;
    st4(dst + m * kD + c, acc[i]);
  }
}

}  // namespace

// Residency cap.  The kernel's registers allow 6 workgroups per CU, but the
// read+write stream measures ~3% faster with 4 (2 is much slower).  The
// launch reserves unused dynamic LDS so that no more than
// kWgPerCU workgroups fit in a CU's 160 KiB.
constexpr int kWgPerCU = 4;
constexpr int kStaticLds = kPathChunk * (kRowsPerWG + kD) * 4;  // vt_s + kc_s
constexpr int kPadLds = lds_cap_pad(kWgPerCU, kStaticLds);
static_assert(kWgPerCU * (kStaticLds + kPadLds) <= kLdsPerCU, "cap leaves room");

hipError_t launch_commit(const CommitArgs& a, const TreeArgs& tree, hipStream_t s) {
  const dim3 grid(a.B * a.H, kD / kRowsPerWG);
  if (a.f32_inputs) {
    hipLaunchKernelGGL(commit_kernel<true>, grid, dim3(256), kPadLds, s, a, tree);
  } else {
    hipLaunchKernelGGL(commit_kernel<false>, grid, dim3(256), kPadLds, s, a, tree);
  }
  return hipGetLastError();
}

}  // namespace treewy
