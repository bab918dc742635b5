// TreeWY verify kernel for gfx950: one workgroup per (sequence, value head).
//
// Computes, for every node t of a DFS pre-order draft tree (method of "TreeWY:
// Speculative Verification for Gated DeltaNet Hybrids": paperpeel section 3
// "Key rewrite", section 2's method summary, review page "Method"):
//   Gamma_t = alpha_t Gamma_parent(t)                     (path gate)
//   P = S0 K^T, R = S0 Q^T                               (2N mat-vecs, MFMA)
//   KK = K K^T, QK = Q K^T                                (gram, same MFMA loop)
//   (I + A) Vt = B with A[t,j] = beta_t Gamma_t/Gamma_j KK[t,j] (j strict ancestor),
//                         B[t] = beta_t (v_t - Gamma_t P[:,t])
//   o_t = Gamma_t R[:,t] + sum_{j anc-or-self} Gamma_t/Gamma_j QK[t,j] vt_j
//
// Schedule inside the workgroup (256 threads = 4 wave64):
//   0. every lane issues its share of the 64 KiB S0 block straight into VGPRs in
//      the MFMA B-operand layout (16 rows x 64 contiguous bytes per load); k and
//      q rows are staged in LDS in A-fragment order, v/alpha/beta in LDS.
//   1. lanes t < N walk their root path once: Gamma_t and the decay ratios
//      Gamma_t/Gamma_j as products of alpha (no division).
//   2. S0 is split into bf16 hi + lo; [K;Q] S0^T and [K;Q] K^T run on
//      v_mfma_f32_16x16x32_bf16 with fp32 accumulation (q, k are bf16 inputs, so
//      the only rounding is the 2^-16 split residual of S0).
//   3. accumulators go to LDS: P/R rows (aliasing the dead k/q fragments), and
//      only the gram entries on each node's path become solve/output weights,
//      indexed by ancestor depth.
//   4. 128 lanes (one per d_v column) run the forward substitution in node
//      order.  In a pre-order the strict ancestors of t are exactly the latest
//      node seen at each depth above t, so the ancestors' pseudo-values live in
//      a depth-indexed register stack and each node costs DS FMAs.
#include <type_traits>

#include "../../include/treewy.h"
#include "device_common.h"
#include "treewy_internal.h"

namespace treewy {
namespace {

constexpr int kKQStride = 136;  // bf16 per LDS fragment row: 128 + 8 pad (272 B, 16-B aligned)

template <int RT, int DS, bool F32IN>
struct VerifyLayout {
  static constexpr int NP = RT * 16;  // padded [K;Q] rows
  static constexpr int NM = RT * 8;   // largest N served by RT tiles
  static constexpr int KQ_BYTES = NP * kKQStride * 2 * (F32IN ? 2 : 1);
  static constexpr int PR_BYTES = NP * kD * 4;
  static constexpr int REGION0 = KQ_BYTES > PR_BYTES ? KQ_BYTES : PR_BYTES;
  static constexpr int V_BYTES = NM * kD * (F32IN ? 4 : 2);
  static constexpr int TAB_BYTES = NM * DS * 4;
  static constexpr int OFF_V = REGION0;
  static constexpr int OFF_RATIO = OFF_V + V_BYTES;
  static constexpr int OFF_ACOEF = OFF_RATIO + TAB_BYTES;
  static constexpr int OFF_MCOEF = OFF_ACOEF + TAB_BYTES;
  static constexpr int OFF_ALPHA = OFF_MCOEF + TAB_BYTES;
  static constexpr int OFF_BETA = OFF_ALPHA + NM * 4;
  static constexpr int OFF_GAM = OFF_BETA + NM * 4;
  static constexpr int OFF_ANC = OFF_GAM + NM * 4;
  static constexpr int OFF_DEPTH = OFF_ANC + kMaxNodes * 8;
  static constexpr int OFF_PARENT = OFF_DEPTH + kMaxNodes;
  static constexpr int TOTAL = OFF_PARENT + kMaxNodes;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int RT, int DS, bool F32IN>
__global__ __launch_bounds__(256) void verify_kernel(const VerifyArgs a, const TreeArgs tree) {
  using L = VerifyLayout<RT, DS, F32IN>;
  using VT = typename std::conditional<F32IN, float, uint16_t>::type;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  __bf16* kq_hi = reinterpret_cast<__bf16*>(smem);
  __bf16* kq_lo = kq_hi + L::NP * kKQStride;  // F32IN only
  float* pr = reinterpret_cast<float*>(smem);  // aliases kq after the MFMA phase
  VT* v_s = reinterpret_cast<VT*>(smem + L::OFF_V);
  float* ratio_s = reinterpret_cast<float*>(smem + L::OFF_RATIO);
  float* acoef_s = reinterpret_cast<float*>(smem + L::OFF_ACOEF);
  float* mcoef_s = reinterpret_cast<float*>(smem + L::OFF_MCOEF);
  float* alpha_s = reinterpret_cast<float*>(smem + L::OFF_ALPHA);
  float* beta_s = reinterpret_cast<float*>(smem + L::OFF_BETA);
  float* gam_s = reinterpret_cast<float*>(smem + L::OFF_GAM);
  uint64_t* anc_s = reinterpret_cast<uint64_t*>(smem + L::OFF_ANC);
  int8_t* depth_s = reinterpret_cast<int8_t*>(smem + L::OFF_DEPTH);
  int8_t* parent_s = reinterpret_cast<int8_t*>(smem + L::OFF_PARENT);

  const int N = tree.n;
  const int H = a.H;
  const int gh = blockIdx.x;
  const int b = gh / H;
  const int h = gh - b * H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;

  // ---- 0. loads -----------------------------------------------------------
  // S0 rows m = 32*wave + 16*ct + r16; lane group g4 takes columns
  // 32s + 4g4 + [0,4) and 32s + 16 + 4g4 + [0,4): the MFMA k-slot order.
  const float* S0h = a.S0 + static_cast<int64_t>(gh) * (kD * kD);
  float4 s0raw[2][4][2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const float* row = S0h + (wave * 32 + ct * 16 + r16) * kD + 4 * g4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      s0raw[ct][s][0] = *reinterpret_cast<const float4*>(row + 32 * s);
      s0raw[ct][s][1] = *reinterpret_cast<const float4*>(row + 32 * s + 16);
    }
  }

  if (tid < kMaxNodes) {
    anc_s[tid] = tree.anc[tid];
    depth_s[tid] = tree.depth[tid];
    parent_s[tid] = tree.parent[tid];
  }

  const int64_t tokstride = static_cast<int64_t>(H) * kD;  // t -> t+1 at fixed (b, h)
  const int64_t tok0 = (static_cast<int64_t>(b) * N * H + h) * kD;
  const int64_t gate0 = static_cast<int64_t>(b) * N * H + h;

  // k rows -> fragment rows [0, N), q rows -> [N, 2N).  Chunk j of a row holds
  // columns 4j..4j+3; within a 32-column block s it goes to slot
  // 8*(j%4) + 4*((j%8)/4), matching the S0 register layout above.
  for (int idx = tid; idx < 2 * N * 32; idx += 256) {
    const int row = idx >> 5;
    const int j = idx & 31;
    const bool is_k = row < N;
    const int t = is_k ? row : row - N;
    const void* src = is_k ? a.k : a.q;
    const int jj = j & 7;
    const int pos = row * kKQStride + 32 * (j >> 3) + 8 * (jj & 3) + 4 * (jj >> 2);
    const int64_t gidx = tok0 + t * tokstride + 4 * j;
    if constexpr (F32IN) {
      const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + gidx);
      const float xs[4] = {x.x, x.y, x.z, x.w};
      bf16x4 hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        __bf16 hh, ll;
        split_bf16(xs[e], hh, ll);
        hi[e] = hh;
        lo[e] = ll;
      }
      *reinterpret_cast<bf16x4*>(kq_hi + pos) = hi;
      *reinterpret_cast<bf16x4*>(kq_lo + pos) = lo;
    } else {
      *reinterpret_cast<uint2*>(kq_hi + pos) =
          *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + gidx);
    }
  }
  // zero the padding rows so the padded MFMA rows stay finite
  {
    const int pad_u4 = (L::NP - 2 * N) * kKQStride / 8;
    uint4* z0 = reinterpret_cast<uint4*>(kq_hi + 2 * N * kKQStride);
    uint4* z1 = reinterpret_cast<uint4*>(kq_lo + 2 * N * kKQStride);
    for (int idx = tid; idx < pad_u4; idx += 256) {
      z0[idx] = make_uint4(0, 0, 0, 0);
      if constexpr (F32IN) z1[idx] = make_uint4(0, 0, 0, 0);
    }
  }
  for (int idx = tid; idx < N * 32; idx += 256) {
    const int t = idx >> 5;
    const int j = idx & 31;
    const int64_t gidx = tok0 + t * tokstride + 4 * j;
    if constexpr (F32IN) {
      *reinterpret_cast<float4*>(v_s + t * kD + 4 * j) =
          *reinterpret_cast<const float4*>(static_cast<const float*>(a.v) + gidx);
    } else {
      *reinterpret_cast<uint2*>(v_s + t * kD + 4 * j) =
          *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.v) + gidx);
    }
  }
  if (tid < N) {
    alpha_s[tid] = load_in<F32IN>(a.alpha, gate0 + static_cast<int64_t>(tid) * H);
    beta_s[tid] = load_in<F32IN>(a.beta, gate0 + static_cast<int64_t>(tid) * H);
  }
  for (int idx = tid; idx < L::NM * DS; idx += 256) {
    acoef_s[idx] = 0.f;
    mcoef_s[idx] = 0.f;
  }
  __syncthreads();

  // ---- 1. path gates: lane t walks from t up to the root ------------------
  if (tid < N) {
    const int t = tid;
    float r = 1.f;
    int cur = t;
    for (int e = depth_s[t]; e >= 0; --e) {
      ratio_s[t * DS + e] = r;  // Gamma_t / Gamma_(ancestor at depth e)
      r *= alpha_s[cur];
      cur = parent_s[cur];
    }
    gam_s[t] = r;
    a.gamma[static_cast<int64_t>(gh) * N + t] = r;
  }

  // ---- 2. split S0 and run the contractions on MFMA ------------------------
  bf16x8 shi[2][4], slo[2][4];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float xs[8] = {s0raw[ct][s][0].x, s0raw[ct][s][0].y, s0raw[ct][s][0].z,
                           s0raw[ct][s][0].w, s0raw[ct][s][1].x, s0raw[ct][s][1].y,
                           s0raw[ct][s][1].z, s0raw[ct][s][1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 hh, ll;
        split_bf16(xs[e], hh, ll);
        shi[ct][s][e] = hh;
        slo[ct][s][e] = ll;
      }
    }
  }

  f32x4 acc[RT][2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    acc[rt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int off = (rt * 16 + r16) * kKQStride + 32 * s + 8 * g4;
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(kq_hi + off);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        acc[rt][ct] = mfma16(af, shi[ct][s], acc[rt][ct]);
        acc[rt][ct] = mfma16(af, slo[ct][s], acc[rt][ct]);
      }
      if constexpr (F32IN) {
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(kq_lo + off);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = mfma16(al, shi[ct][s], acc[rt][ct]);
      }
    }
  }

  // gram tiles (row tile rt of [K;Q]) x (column tile gt of K), spread over waves
  const int GT = (N + 15) >> 4;
  constexpr int GTM = (RT + 1) / 2;
  constexpr int MAXG = (RT * GTM + 3) / 4;
  f32x4 gacc[MAXG];
#pragma unroll
  for (int i = 0; i < MAXG; ++i) {
    gacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int tau = wave + 4 * i;
    if (tau < RT * GT) {
      const int rt = tau / GT;
      const int gt = tau - rt * GT;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int offa = (rt * 16 + r16) * kKQStride + 32 * s + 8 * g4;
        const int offb = (gt * 16 + r16) * kKQStride + 32 * s + 8 * g4;
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(kq_hi + offa);
        const bf16x8 bf = *reinterpret_cast<const bf16x8*>(kq_hi + offb);
        gacc[i] = mfma16(af, bf, gacc[i]);
        if constexpr (F32IN) {
          const bf16x8 al = *reinterpret_cast<const bf16x8*>(kq_lo + offa);
          const bf16x8 bl = *reinterpret_cast<const bf16x8*>(kq_lo + offb);
          gacc[i] = mfma16(al, bf, gacc[i]);
          gacc[i] = mfma16(af, bl, gacc[i]);
        }
      }
    }
  }
  __syncthreads();  // fragments consumed; ratios and gates visible

  // ---- 3. results to LDS ----------------------------------------------------
  // D layout of the 16x16 MFMA: lane holds rows 4*g4 + i (i < 4) of column r16.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int m = wave * 32 + ct * 16 + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rt * 16 + 4 * g4 + i;
        if (row < 2 * N) pr[row * kD + m] = acc[rt][ct][i];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < MAXG; ++i) {
    const int tau = wave + 4 * i;
    if (tau < RT * GT) {
      const int rt = tau / GT;
      const int gt = tau - rt * GT;
      const int j = gt * 16 + r16;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int row = rt * 16 + 4 * g4 + ii;
        const float val = gacc[i][ii];
        if (j < N && row < 2 * N) {
          if (row < N) {
            const int t = row;
            if ((anc_s[t] >> j) & 1ull) {
              const int e = depth_s[j];
              acoef_s[t * DS + e] = beta_s[t] * ratio_s[t * DS + e] * val;
            }
          } else {
            const int t = row - N;
            if (j == t || ((anc_s[t] >> j) & 1ull)) {
              const int e = depth_s[j];
              mcoef_s[t * DS + e] = ratio_s[t * DS + e] * val;
            }
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- 4. forward substitution and outputs, one lane per d_v column ---------
  if (tid < kD) {
    const int m = tid;
    float st[DS];
#pragma unroll
    for (int e = 0; e < DS; ++e) st[e] = 0.f;
    float* vt_out = a.vtilde + static_cast<int64_t>(gh) * N * kD + m;
    float* o_out = a.out + tok0 + m;
    for (int t = 0; t < N; ++t) {
      const int d = depth_s[t];
      const float P = pr[t * kD + m];
      const float R = pr[(N + t) * kD + m];
      float vv;
      if constexpr (F32IN) {
        vv = v_s[t * kD + m];
      } else {
        vv = bf16_bits_to_f32(v_s[t * kD + m]);
      }
      const float G = gam_s[t];
      float x = beta_s[t] * (vv - G * P);
      const float* ac = acoef_s + t * DS;
#pragma unroll
      for (int e = 0; e < DS; ++e) x -= ac[e] * st[e];
#pragma unroll
      for (int e = 0; e < DS; ++e) st[e] = (e == d) ? x : st[e];
      const float* mc = mcoef_s + t * DS;
      float o = G * R;
#pragma unroll
      for (int e = 0; e < DS; ++e) o += mc[e] * st[e];
      vt_out[t * kD] = x;
      o_out[t * tokstride] = o;
    }
  }
}

template <int RT, int DS, bool F32IN>
hipError_t launch_rt(const VerifyArgs& a, const TreeArgs& tree, hipStream_t s) {
  hipLaunchKernelGGL((verify_kernel<RT, DS, F32IN>), dim3(a.B * a.H), dim3(256), 0, s, a, tree);
  return hipGetLastError();
}

template <int DS, bool F32IN>
hipError_t launch_ds(const VerifyArgs& a, const TreeArgs& tree, int rt, hipStream_t s) {
  switch (rt) {
    case 1: return launch_rt<1, DS, F32IN>(a, tree, s);
    case 2: return launch_rt<2, DS, F32IN>(a, tree, s);
    case 3: return launch_rt<3, DS, F32IN>(a, tree, s);
    case 4: return launch_rt<4, DS, F32IN>(a, tree, s);
    case 5: return launch_rt<5, DS, F32IN>(a, tree, s);
    case 6: return launch_rt<6, DS, F32IN>(a, tree, s);
    case 7: return launch_rt<7, DS, F32IN>(a, tree, s);
    case 8: return launch_rt<8, DS, F32IN>(a, tree, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool F32IN>
hipError_t launch_dtype(const VerifyArgs& a, const TreeArgs& tree, hipStream_t s) {
  const int rt = (tree.n + 7) / 8;  // 2N rows of [K;Q] in 16-row tiles
  if (tree.max_depth < 4) return launch_ds<4, F32IN>(a, tree, rt, s);
  if (tree.max_depth < 16) return launch_ds<16, F32IN>(a, tree, rt, s);
  return launch_ds<64, F32IN>(a, tree, rt, s);
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, const TreeArgs& tree, hipStream_t s) {
  return a.f32_inputs ? launch_dtype<true>(a, tree, s) : launch_dtype<false>(a, tree, s);
}

}  // namespace treewy
