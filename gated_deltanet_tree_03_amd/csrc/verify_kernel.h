// TreeWY verify kernel for gfx950: one workgroup per (sequence, value head).
// The kernel template and its launchers; each verify*.hip file instantiates
// one family of it (split so the families compile in parallel).
//
// Computes, for every node t of a DFS pre-order draft tree (method of "TreeWY:
// Speculative Verification for Gated DeltaNet Hybrids": paperpeel section 3
// "Key rewrite", section 2's method summary, review page "Method"):
//   Gamma_t = alpha_t Gamma_parent(t)                     (path gate)
//   P = K S0^T, R = Q S0^T                                (2N mat-vecs, MFMA)
//   KK = K K^T, QK = Q K^T                                (gram, MFMA)
//   (I + A) Vt = B,  A[t,j] = beta_t Gamma_t/Gamma_j KK[t,j] for j a strict
//                    ancestor of t,  B[t] = beta_t (v_t - Gamma_t P[t])
//   o_t = Gamma_t R[t] + sum_{j anc-or-self} Gamma_t/Gamma_j QK[t,j] vt_j
//
// The solve is done in its tree-WY form.  (I + A) is unit lower triangular
// with non-zeros only on each node's root path, and so is T = (I + A)^-1 (the
// path of an ancestor is a prefix of the node's own path).  With M[t,j] =
// Gamma_t/Gamma_j QK[t,j] on the path, Vt = T B and O = Gamma R + (M T) B, so
// every output element is a sum of depth(t)+1 terms B[anc_e(t)] taken along
// the root path: per head only the small tables T and MT (N rows of
// depth+1 entries) are serial work; the 128-column part is fully parallel.
//
// Schedule inside the workgroup (kWaves wave64, 8 by default):
//   0. every global load is issued up front: the tree metadata, the small rows
//      (gates, k/q/v), for commit-then-verify the previous step's first path
//      rows, then the 64 KiB S0 block as full 128-byte lines (vector loads
//      return in order, so staging the small rows does not wait for S0);
//   1. k/q rows go to LDS in A-fragment order, v, the gates and the path rows
//      to LDS;
//   2. lanes t < N walk their root path (path list, Gamma_t and the decay
//      ratios as products of alpha); a DPP rotate turns the S0 lines into the
//      MFMA B-operand layout; commit-then-verify first commits the previous
//      step into those registers and stores the committed state; S0 is split
//      into bf16 hi + lo and [K;Q] S0^T and [K;Q] K^T run on
//      v_mfma_f32_16x16x32_bf16 with fp32 accumulation (q, k are bf16 inputs,
//      so the only rounding is the 2^-16 split residual of S0);
//   3. P/R rows go to LDS; the gram goes to LDS as a dense matrix;
//   4. one wave gathers each node's path entries of A and M and builds T and
//      MT; the other waves form B = beta (v - Gamma P);
//   5. every thread produces float4 chunks of Vt and O for (node, 4 columns).
// Template flags pick the family: FUSED (commit-then-verify), POOL (state
// blocks named by a slot per sequence), S16 (state stored as bf16: no split,
// natural k order), RAGGED (a tree per sequence, pool form); S16 combines
// with POOL and RAGGED.
#pragma once

#include <type_traits>

#include "../../include/treewy.h"
#include "device_common.h"
#include "treewy_internal.h"

namespace treewy {
namespace {

// Outputs (out, vtilde, gamma) and the committed state leave as non-temporal
// stores: written once, read by a later kernel.  Normal stores stay dirty in
// L2 and are written back when the kernel ends, a drain that nothing overlaps
// when launches run back to back (measured: (2,2,2) tree verify 72.7 -> 67.0
// us, (3,3,3) 411 -> 391 us).
// bf16 per LDS fragment row: 128 + 16 pad (288 B).  The fragment reads (16 B
// per lane, row r16, column group g4) measured conflict-free with 288-byte
// rows and at 3.6 conflict cycles per read with 272-byte rows (bank-conflict
// counter, one read instruction per pattern).
constexpr int kKQStride = 144;
constexpr int kYStride = 132;   // floats per LDS row of P / R / B: 128 + 4 pad

constexpr int kPathChunk = 8;  // commit path rows staged per round (commit-then-verify)

// Workgroup shape: kWaves = 8 wave64 per (sequence, head); each wave owns 16
// rows of S0 (kCT = 1 tile of 16), so each lane holds 8 float4 of the block.
// With 8 waves a lane moves 8 float4 of state in and (commit-then-verify) 8
// out, a burst that streams at copy speed; 16 per lane (4 waves) does not.
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kCT = 8 / kWaves;
constexpr int kS0Regs = 8 * kCT;

template <int RT, int DS, bool F32IN, bool FUSED = false>
struct VerifyLayout {
  static constexpr int NP = RT * 16;  // padded [K;Q] rows
  static constexpr int NM = RT * 8;   // largest N served by RT tiles
  static constexpr int KQ_BYTES = NP * kKQStride * 2 * (F32IN ? 2 : 1);
  static constexpr int Y_BYTES = NP * kYStride * 4;
  static constexpr int REGION0 = KQ_BYTES > Y_BYTES ? KQ_BYTES : Y_BYTES;
  static constexpr int V_BYTES = NM * kD * (F32IN ? 4 : 2);
  static constexpr int TAB_BYTES = NM * DS * 4;
  static constexpr int OFF_V = REGION0;
  static constexpr int OFF_RATIO = OFF_V + V_BYTES;
  static constexpr int OFF_TA = OFF_RATIO + TAB_BYTES;  // A, then T in place
  static constexpr int OFF_TM = OFF_TA + TAB_BYTES;     // M, then M T in place
  static constexpr int OFF_PATH = OFF_TM + TAB_BYTES;
  static constexpr int OFF_ALPHA = OFF_PATH + ((NM * DS + 15) / 16) * 16;
  static constexpr int OFF_BETA = OFF_ALPHA + NM * 4;
  static constexpr int OFF_GAM = OFF_BETA + NM * 4;
  static constexpr int OFF_DEPTH = OFF_GAM + NM * 4;
  static constexpr int OFF_PARENT = OFF_DEPTH + kMaxNodes;
  // Dense gram [K;Q] K^T, rows [0, 2N) x columns [0, N), written once after
  // the MFMA phase; before it, the same bytes stage the commit-then-verify
  // path rows (vt rows, then scaled k rows).
  // (deep trees, DS = 64, scatter the path entries straight into the tables
  // instead: their tables leave no room for a dense gram)
  static constexpr bool DENSE_GRAM = DS <= 16;
  static constexpr int GS = 16 * ((RT + 1) / 2) + 4;  // gram row stride (floats)
  static constexpr int GRAM_BYTES = DENSE_GRAM ? NP * GS * 4 : 0;
  static constexpr int FUSE_BYTES = FUSED ? 2 * kPathChunk * kD * 4 : 0;
  static constexpr int OFF_GRAM = ((OFF_PARENT + kMaxNodes + 15) / 16) * 16;
  // without a dense gram the staging shares the A/M tables (written later)
  static constexpr bool FUSE_IN_TABLES = !DENSE_GRAM && 2 * TAB_BYTES >= FUSE_BYTES;
  static constexpr int OFF_FUSE = FUSE_IN_TABLES ? OFF_TA : OFF_GRAM;
  static constexpr int UNION_BYTES = FUSE_IN_TABLES ? GRAM_BYTES
                                     : (GRAM_BYTES > FUSE_BYTES ? GRAM_BYTES : FUSE_BYTES);
  static constexpr int TOTAL = OFF_GRAM + UNION_BYTES;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Orders LDS traffic between lanes of one wave (lanes of a wave run in
// lockstep; the fences keep the compiler from moving LDS accesses across).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// T = (I + A)^-1 and M T on the root paths of a tree of depth <= 3, for node
// t by one lane on its own.  The root path p_0 (root) .. p_d = t has at most 4
// nodes, and the rows of T on it are those of the inverse of the path's own
// unit lower triangular block (the path of an ancestor is a prefix of t's
// path), so the lane forms that 4 x 4 block in registers and inverts it by
// forward substitution; no lane waits for another's rows.  With the decay
// ratio Gamma_x / Gamma_y of path nodes x, y read from row x of the ratio
// table (its entry at y's depth):
//   A_path[x][y] = beta_px (Gamma_px / Gamma_py) (k_px . k_py)   (y < x <= d)
//   M[f]        = (Gamma_t / Gamma_pf) (q_t . k_pf)              (f <= d)
//   T[t][e]     = (I + A_path)^-1 [d][e],   (M T)[t][e] = sum_{f=e..d} M[f] T_path[f][e].
// All reads are issued in two rounds (the path, then the entries it names),
// where a level-by-level walk took a dependent LDS round trip per entry and
// a wave barrier per level.  Writes T[t][e] to tabA and (M T)[t][e] to tabM
// (row stride 4), e <= d.
__device__ __forceinline__ void tables_short_paths(int t, int N, int GS, const float* gram,
                                                   const int8_t* path_s, const float* ratio_s,
                                                   const float* beta_s, const int8_t* depth_s,
                                                   float* tabA, float* tabM) {
  const int d = depth_s[t];
  const uint32_t pw = *reinterpret_cast<const uint32_t*>(path_s + 4 * t);
  const float4 rt4 = *reinterpret_cast<const float4*>(ratio_s + 4 * t);  // Gamma_t / Gamma_pf
  const float rt[4] = {rt4.x, rt4.y, rt4.z, rt4.w};
  int p[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    // entries past the path's end were never written: point them at t
    p[x] = x <= d ? static_cast<int>(static_cast<int8_t>((pw >> (8 * x)) & 0xffu)) : t;
  }
  float be[4], rat[4][4], kk[4][4], qk[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    be[x] = beta_s[p[x]];
    const float4 r = *reinterpret_cast<const float4*>(ratio_s + 4 * p[x]);
    rat[x][0] = r.x; rat[x][1] = r.y; rat[x][2] = r.z; rat[x][3] = r.w;
    qk[x] = gram[(N + t) * GS + p[x]];
#pragma unroll
    for (int y = 0; y < x; ++y) kk[x][y] = gram[p[x] * GS + p[y]];
  }
  // the path block of (I + A)^-1, rows and columns by depth (rows past d are
  // unit rows and are not used)
  float T[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      if (y > x) {
        T[x][y] = 0.f;
      } else if (y == x) {
        T[x][y] = 1.f;
      } else {
        float s = 0.f;
#pragma unroll
        for (int z = 0; z < x; ++z) {
          if (z >= y) s += (x <= d ? be[x] * rat[x][z] * kk[x][z] : 0.f) * T[z][y];
        }
        T[x][y] = -s;
      }
    }
  }
  float m[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) m[f] = f <= d ? rt[f] * qk[f] : 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (e <= d) {
      const float te = d == 0 ? T[0][e] : (d == 1 ? T[1][e] : (d == 2 ? T[2][e] : T[3][e]));
      float mt = 0.f;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        if (f >= e) mt += m[f] * T[f][e];
      }
      tabA[4 * t + e] = te;
      tabM[4 * t + e] = mt;
    }
  }
}

// Same tables for deep trees: lane e (< DS) owns column e and walks the nodes
// in pre-order, keeping column e of T for the current root path in a
// depth-indexed register stack (in a pre-order the strict ancestors of t are
// the latest nodes seen at each smaller depth).  In place: tabA holds A[t][f]
// and tabM holds M[t][f] on entry, T and M T on exit.
template <int DS>
__device__ __forceinline__ void tables_by_column(int e, int N, float* tabA, float* tabM,
                                                 const int8_t* depth_s) {
  float stk[DS];
#pragma unroll
  for (int f = 0; f < DS; ++f) stk[f] = 0.f;
  for (int t = 0; t < N; ++t) {
    const int d = depth_s[t];
    float x = (e == d) ? 1.f : 0.f;
#pragma unroll
    for (int f = 0; f < DS; ++f) {
      if (f >= e && f < d) x -= tabA[t * DS + f] * stk[f];
    }
#pragma unroll
    for (int f = 0; f < DS; ++f) stk[f] = (f == d) ? x : stk[f];
    float mt = 0.f;
#pragma unroll
    for (int f = 0; f < DS; ++f) {
      if (f >= e && f <= d) mt += tabM[t * DS + f] * stk[f];
    }
    wave_sync();  // every lane has read row t of A and M
    if (e <= d) {
      tabA[t * DS + e] = x;
      tabM[t * DS + e] = mt;
    }
    wave_sync();
  }
}

// S0 block `gh` into VGPRs.  Wave w owns rows 16*kCT*w + 16*ct + [0,16); in
// the MFMA B-operand layout lane (r16, g4) holds, for each 32-column block s,
// columns 32s + 4g4 + [0,4) ("half 0") and 32s + 16 + 4g4 + [0,4) ("half 1")
// of row r16 of the tile: the k-slot order of the A fragments.  Loading that
// layout directly makes every load instruction touch 16 rows x 64 B (half
// lines), which streams markedly slower than full lines.  So each pair
// (x[2s], x[2s+1]) is loaded as two full-line instructions -- "A" covers rows
// 0-7 of the tile, "B" rows 8-15; lanes r16 < 8 take half 0, lanes r16 >= 8
// half 1 -- and one DPP rotate by 8 inside each 16-lane row turns the pair
// into the MFMA layout (lines_to_mfma) or back (mfma_to_lines).  S0 is read
// exactly once, so the loads are non-temporal.
__device__ __forceinline__ f32x4 ror8(const f32x4& x) {
  return f32x4{dpp_mov<0x128>(x.x), dpp_mov<0x128>(x.y), dpp_mov<0x128>(x.z),
               dpp_mov<0x128>(x.w)};  // row_ror:8 -- lane i <-> lane i^8 within 16
}

// (A, B) line pair -> (half 0, half 1) of the lane's own row.
__device__ __forceinline__ void lines_to_mfma(f32x4& a, f32x4& b, bool lo) {
  const f32x4 recv = ror8(lo ? b : a);
  if (lo) {
    b = recv;
  } else {
    a = recv;
  }
}

// (half 0, half 1) of the lane's own row -> (A, B) line pair.
__device__ __forceinline__ void mfma_to_lines(f32x4& h0, f32x4& h1, bool lo) {
  const f32x4 recv = ror8(lo ? h1 : h0);
  if (lo) {
    h1 = recv;
  } else {
    h0 = recv;
  }
}

// Row and column offset (floats, inside the block) of the A and B line
// instruction of pair (ct, s) for this lane.
__device__ __forceinline__ int line_off(int wave, int ct, int s, int r16, int g4, bool second) {
  const bool lo = r16 < 8;
  const int row = wave * 16 * kCT + ct * 16 + (second ? (lo ? r16 + 8 : r16) : (lo ? r16 : r16 - 8));
  return row * kD + 32 * s + (lo ? 0 : 16) + 4 * g4;
}

__device__ __forceinline__ void load_s0(const float* S0h, int wave, int r16, int g4,
                                        f32x4 (&r)[kS0Regs]) {
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      r[ct * 8 + 2 * s] = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(S0h + line_off(wave, ct, s, r16, g4, false)));
      r[ct * 8 + 2 * s + 1] = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(S0h + line_off(wave, ct, s, r16, g4, true)));
    }
  }
}

// bf16 state (commit-then-verify over a bf16-stored state).  The state is
// exact in bf16, so S0 needs no hi/lo split and the MFMA B operand is the
// stored bits in the natural k order: lane (r16, g4) holds columns
// 32s + 8g4 + [0,8) of row r16 for block s (16 B), and the A fragments are
// staged in the same natural order.  As for fp32, a block pair (2p, 2p+1) of
// one row is 128 B, loaded as two full-line instructions ("A": rows 0-7 of the
// tile, lanes r16 < 8 taking block 2p and lanes r16 >= 8 block 2p+1 of the
// same row; "B": rows 8-15) and turned into the MFMA layout by the same DPP
// rotate by 8.  Register x[4ct + s] holds block s.
constexpr int kS16Regs = 4 * kCT;

__device__ __forceinline__ uint4 ror8u(const uint4& x) {
  return make_uint4(__float_as_uint(dpp_mov<0x128>(__uint_as_float(x.x))),
                    __float_as_uint(dpp_mov<0x128>(__uint_as_float(x.y))),
                    __float_as_uint(dpp_mov<0x128>(__uint_as_float(x.z))),
                    __float_as_uint(dpp_mov<0x128>(__uint_as_float(x.w))));
}

// (A, B) line pair <-> (block 2p, block 2p+1) of the lane's own row; the
// exchange is its own inverse.
__device__ __forceinline__ void swap_lines16(uint4& a, uint4& b, bool lo) {
  // component-wise selects: a select between the two references would make
  // the compiler address the register array through memory
  const uint4 av = a, bv = b;
  const uint4 recv = ror8u(make_uint4(lo ? bv.x : av.x, lo ? bv.y : av.y, lo ? bv.z : av.z,
                                      lo ? bv.w : av.w));
  a = make_uint4(lo ? av.x : recv.x, lo ? av.y : recv.y, lo ? av.z : recv.z, lo ? av.w : recv.w);
  b = make_uint4(lo ? recv.x : bv.x, lo ? recv.y : bv.y, lo ? recv.z : bv.z, lo ? recv.w : bv.w);
}

// Element offset (inside the block) of the A or B line load of pair (ct, p).
__device__ __forceinline__ int line_off16(int wave, int ct, int p, int r16, int g4, bool second) {
  const bool lo = r16 < 8;
  const int row = wave * 16 * kCT + ct * 16 + (second ? (lo ? r16 + 8 : r16) : (lo ? r16 : r16 - 8));
  return row * kD + 64 * p + (lo ? 0 : 32) + 8 * g4;
}

__device__ __forceinline__ void load_s0_16(const uint16_t* S0h, int wave, int r16, int g4,
                                           uint4 (&r)[kS16Regs]) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const u32x4 x = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(S0h + line_off16(wave, ct, p, r16, g4, q == 1)));
        r[ct * 4 + 2 * p + q] = make_uint4(x.x, x.y, x.z, x.w);
      }
    }
  }
}

// 8 bf16 (one block of the natural layout) <-> 2 x 4 fp32.
__device__ __forceinline__ void unpack16(const uint4& u, f32x4& lo4, f32x4& hi4) {
  lo4 = f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
              __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
  hi4 = f32x4{__uint_as_float(u.z << 16), __uint_as_float(u.z & 0xffff0000u),
              __uint_as_float(u.w << 16), __uint_as_float(u.w & 0xffff0000u)};
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const __bf16 x = to_bf16(a), y = to_bf16(b);  // round to nearest even
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, x)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, y)) << 16);
}

__device__ __forceinline__ uint4 pack16(const f32x4& lo4, const f32x4& hi4) {
  return make_uint4(pack2(lo4.x, lo4.y), pack2(lo4.z, lo4.w), pack2(hi4.x, hi4.y),
                    pack2(hi4.z, hi4.w));
}

// The small rows of one (sequence, head), held raw in VGPRs between their
// load and their staging into LDS: the two gates of lane t < N, and the k/q
// and v rows in 16-byte chunks.
template <int KQ_PER, int V_PER>
struct SmallRows {
  uint32_t ga, gb;
  uint4 kq[KQ_PER];
  uint4 v[V_PER];
};

template <int RT, bool F32IN>
struct SmallShape {
  static constexpr int IB = F32IN ? 4 : 2;             // bytes per input element
  static constexpr int CPR = kD * IB / 16;              // 16-byte chunks per 128-element row
  static constexpr int KQ_PER = (2 * RT * 8 * CPR + kThreads - 1) / kThreads;
  static constexpr int V_PER = (RT * 8 * CPR + kThreads - 1) / kThreads;
  using Rows = SmallRows<KQ_PER, V_PER>;
};

// Issues the loads of head gh's small rows.  Gates are loaded unconditionally
// from a clamped node index, as raw bits: a conversion inside a branch would
// make the compiler wait for them right away.
// One 16-byte chunk of a q/k/v row.  Large trees (RT >= 3) read them
// non-temporal: read once, and on the 40-node tree the cached loads cost ~1%
// (verify 394 -> 388 us back to back); on chains they measure the other way.
template <bool NT>
__device__ __forceinline__ uint4 ld_row16(const unsigned char* p) {
  if constexpr (NT) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}

template <int RT, bool F32IN>
__device__ __forceinline__ void load_small(const VerifyArgs& a, int N, int gh,
                                           typename SmallShape<RT, F32IN>::Rows& sr) {
  using SS = SmallShape<RT, F32IN>;
  constexpr int IB = SS::IB, CPR = SS::CPR;
  const int tid = threadIdx.x;
  const int H = a.H;
  const int b = gh / H;
  const int h = gh - b * H;
  const int64_t TB = a.tok_b ? a.tok_b : N;  // tokens per batch row
  const int64_t tokstride = static_cast<int64_t>(H) * kD;
  const int64_t tok0 = (b * TB * H + h) * kD;
  const int64_t gate0 = b * TB * H + h;
  const unsigned char* kbytes = static_cast<const unsigned char*>(a.k);
  const unsigned char* qbytes = static_cast<const unsigned char*>(a.q);
  const unsigned char* vbytes = static_cast<const unsigned char*>(a.v);
  {
    const int tn = tid < N ? tid : N - 1;
    const int64_t gi = gate0 + static_cast<int64_t>(tn) * H;
    if constexpr (F32IN) {
      sr.ga = static_cast<const uint32_t*>(a.alpha)[gi];
      sr.gb = static_cast<const uint32_t*>(a.beta)[gi];
    } else {
      sr.ga = static_cast<const uint16_t*>(a.alpha)[gi];
      sr.gb = static_cast<const uint16_t*>(a.beta)[gi];
    }
  }
#pragma unroll
  for (int i = 0; i < SS::KQ_PER; ++i) {
    const int idx = tid + kThreads * i;
    sr.kq[i] = make_uint4(0, 0, 0, 0);
    if (idx < 2 * N * CPR) {
      const int row = idx / CPR;
      const int j = idx - row * CPR;
      const bool is_k = row < N;
      const int t = is_k ? row : row - N;
      const unsigned char* src = is_k ? kbytes : qbytes;
      sr.kq[i] = ld_row16<(RT >= 3)>(src + (tok0 + t * tokstride) * IB + 16 * j);
    }
  }
#pragma unroll
  for (int i = 0; i < SS::V_PER; ++i) {
    const int idx = tid + kThreads * i;
    sr.v[i] = make_uint4(0, 0, 0, 0);
    if (idx < N * CPR) {
      const int t = idx / CPR;
      const int j = idx - t * CPR;
      sr.v[i] = ld_row16<(RT >= 3)>(vbytes + (tok0 + t * tokstride) * IB + 16 * j);
    }
  }
}

// Rows of the previous step's accepted path for commit-then-verify.  The
// first kPathChunk path nodes (lowest index first) are loaded in the kernel's
// load phase ahead of the S0 block and staged with the small rows, so the
// commit does not wait a second memory round trip after S0 arrives; lane
// tid < kPathChunk*32 holds 4 columns of row e = tid / 32 as raw bits (fp32,
// or bf16 pairs in x, y for k).
struct PathRows {
  uint64_t mask;  // accepted node and its strict ancestors; 0 if out of range
  bool keep;      // pool form, accepted index < 0: no previous step to commit
  float ga;       // Gamma of the accepted node
  uint4 vt, k;
  float g;        // Gamma of this lane's path node
};

// prev_n, prev_anc: the previous tree's node count and strict-ancestor masks.
template <bool F32IN, bool POOL>
__device__ __forceinline__ void load_path(const VerifyArgs& a, const int prev_n,
                                          const uint64_t* prev_anc, const int gh, const int b,
                                          const int h, PathRows& pr) {
  const int np = a.n_prev;
  const int acc = a.acc_prev ? a.acc_prev[b] : prev_n - 1;  // none given: the last node
  const bool ok = acc >= 0 && acc < prev_n;
  pr.keep = POOL && acc < 0;
  // (masked to the tree's nodes: a per-sequence mask is device data)
  const uint64_t live = prev_n >= 64 ? ~0ull : ((1ull << prev_n) - 1ull);
  pr.mask = ok ? ((prev_anc[acc] | (1ull << acc)) & live) : 0ull;
  pr.ga = ok ? a.gamma_prev[static_cast<int64_t>(gh) * np + acc] : 0.f;
  pr.vt = make_uint4(0, 0, 0, 0);
  pr.k = make_uint4(0, 0, 0, 0);
  pr.g = 1.f;
  const int tid = threadIdx.x;
  const int e = tid >> 5;
  const int c4 = (tid & 31) * 4;
  uint64_t r = pr.mask;
  for (int z = 0; z < e && z < kPathChunk; ++z) r &= r - 1ull;
  if (tid < kPathChunk * 32 && r != 0ull) {
    const int j = __builtin_ctzll(r);
    const int64_t tok = (static_cast<int64_t>(b) * (a.tok_b_prev ? a.tok_b_prev : np) + j) * a.H + h;
    pr.vt = *reinterpret_cast<const uint4*>(a.vt_prev + (static_cast<int64_t>(gh) * np + j) * kD + c4);
    if constexpr (F32IN) {
      pr.k = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.k_prev) + tok * kD + c4);
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.k_prev) + tok * kD + c4);
      pr.k = make_uint4(u.x, u.y, 0, 0);
    }
    pr.g = a.gamma_prev[static_cast<int64_t>(gh) * np + j];
  }
}

// Stages the first chunk of path rows: vt rows to vtp_s, k rows scaled by
// Gamma_a/Gamma_j to kp_s.
template <bool F32IN>
__device__ __forceinline__ void stage_path(const PathRows& pr, float* vtp_s, float* kp_s) {
  const int tid = threadIdx.x;
  const int L = __builtin_popcountll(pr.mask);
  if (tid < kPathChunk * 32 && tid < L * 32) {
    const int e = tid >> 5;
    const int c4 = (tid & 31) * 4;
    *reinterpret_cast<uint4*>(vtp_s + e * kD + c4) = pr.vt;
    const float w = pr.ga / pr.g;
    float4 kk;
    if constexpr (F32IN) {
      kk = make_float4(__uint_as_float(pr.k.x), __uint_as_float(pr.k.y), __uint_as_float(pr.k.z),
                       __uint_as_float(pr.k.w));
    } else {
      kk = make_float4(__uint_as_float(pr.k.x << 16), __uint_as_float(pr.k.x & 0xffff0000u),
                       __uint_as_float(pr.k.y << 16), __uint_as_float(pr.k.y & 0xffff0000u));
    }
    *reinterpret_cast<float4*>(kp_s + e * kD + c4) = make_float4(w * kk.x, w * kk.y, w * kk.z, w * kk.w);
  }
}

// The committed state of the previous step is rebuilt in the S0 registers
// before verification (commit-then-verify): S_a = Gamma_a S0 + sum over the
// root path of the previous step's accepted node a of (Gamma_a/Gamma_j) vt_j k_j^T.
// Path rows are staged through LDS, kPathChunk at a time (the first chunk is
// already staged by stage_path), the k rows already scaled by
// Gamma_a/Gamma_j; each lane updates its float4 of the block.  An empty path
// mask (accepted index out of range) makes the whole state NaN.  NATURAL: the
// lane's columns are those of the bf16-state layout (32s + 8g4 + [0,8)).
template <bool F32IN, bool NATURAL = false>
__device__ __forceinline__ void commit_in_registers(const VerifyArgs& a, const int gh, const int b,
                                                    const int h, const PathRows& pr, float* vtp_s,
                                                    float* kp_s, f32x4 (&s0)[kS0Regs]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  const int np = a.n_prev;
  const float ga = pr.ga;
  if (pr.keep) return;  // the state is already the committed one
  if (pr.mask == 0ull) {
    const float nan = qnan();
#pragma unroll
    for (int i = 0; i < kS0Regs; ++i) s0[i] = f32x4{nan, nan, nan, nan};
    return;
  }
#pragma unroll
  for (int i = 0; i < kS0Regs; ++i) s0[i] *= ga;
  const int64_t tokstride = static_cast<int64_t>(a.H) * kD;
  const int64_t tok0 =
      (static_cast<int64_t>(b) * (a.tok_b_prev ? a.tok_b_prev : np) * a.H + h) * kD;
  const float* vt_head = a.vt_prev + static_cast<int64_t>(gh) * np * kD;
  const float* gam_head = a.gamma_prev + static_cast<int64_t>(gh) * np;
  uint64_t rest = pr.mask;
  bool first = true;
  while (rest != 0ull) {
    // the next kPathChunk path nodes, lowest index first
    uint64_t chunk = 0ull;
    int L = 0;
    while (rest != 0ull && L < kPathChunk) {
      chunk |= rest & (~rest + 1ull);
      rest &= rest - 1ull;
      ++L;
    }
    if (!first) {
      __syncthreads();  // earlier readers of the staging rows are done
      for (int idx = tid; idx < L * (kD / 4); idx += kThreads) {
        const int e = idx / (kD / 4);
        const int c4 = (idx - e * (kD / 4)) * 4;
        uint64_t r = chunk;
        for (int z = 0; z < e; ++z) r &= r - 1ull;
        const int j = __builtin_ctzll(r);
        *reinterpret_cast<float4*>(vtp_s + e * kD + c4) =
            *reinterpret_cast<const float4*>(vt_head + j * kD + c4);
        const float w = ga / gam_head[j];
        const float4 kk = load_in4<F32IN>(a.k_prev, tok0 + j * tokstride + c4);
        *reinterpret_cast<float4*>(kp_s + e * kD + c4) =
            make_float4(w * kk.x, w * kk.y, w * kk.z, w * kk.w);
      }
      __syncthreads();
    }
    first = false;
    for (int e = 0; e < L; ++e) {
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        const float vm = vtp_s[e * kD + wave * 16 * kCT + ct * 16 + r16];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int ca = NATURAL ? 32 * s + 8 * g4 : 32 * s + 4 * g4;
          const int cb = NATURAL ? ca + 4 : ca + 16;
          const float4 ka = *reinterpret_cast<const float4*>(kp_s + e * kD + ca);
          const float4 kb = *reinterpret_cast<const float4*>(kp_s + e * kD + cb);
          s0[ct * 8 + 2 * s] += vm * f32x4{ka.x, ka.y, ka.z, ka.w};
          s0[ct * 8 + 2 * s + 1] += vm * f32x4{kb.x, kb.y, kb.z, kb.w};
        }
      }
    }
  }
}

// Register budget per lane, as resident waves per SIMD (workgroups per CU
// times the waves each puts on a SIMD).  The budget shapes the code; the
// hardware then fits as many workgroups as the registers actually used and
// the LDS allow.  Commit-then-verify holds the path rows and the committed
// block on top of verify's registers: at the 64-register budget of 8 waves
// per SIMD it spills.  For small trees the 128-register budget (2 resident
// workgroups per CU) is the fastest: timed interleaved on one GPU against a
// budget of 3 (85 registers, 78 used, 3 resident), the fused step took 196
// against 204 us on the 35B-like chain, 194 against 201 us on the 397B-like
// chain and 116.1 against 118.9 us on the 35B-like (2,2,2) tree.  With 3
// resident the workgroups on a CU averaged 2.47 at a time, each taking 18.6
// us; fewer resident workgroups contend less for the same bandwidth.
constexpr int kVerifyWgSmall = 4;
constexpr int kFusedWgSmall = 2;
// The bf16-state family holds half the state registers: with depth <= 3 it
// fits the 64-register budget without spilling, which measured 17% faster on
// the 35B-like chain (121 -> 100 us) and 8% on the (2,2,2) tree; deeper small
// trees would spill there and keep the fused budget.
constexpr int kS16WgSmall = 4;
template <int RT, int DS, bool FUSED, bool S16 = false, bool RAGGED = false>
constexpr int verify_waves_per_eu() {
  // deep trees (DS = 64) hold a 64-entry register stack in the table walk
  // (a bf16 state with a tree per sequence spills at the 64-register budget)
  const int small = S16 ? (DS <= 4 && !RAGGED ? kS16WgSmall : kFusedWgSmall)
                        : (FUSED ? kFusedWgSmall : kVerifyWgSmall);
  const int wg_per_cu = (RT <= 2 ? small : (RT <= 5 ? 2 : 1));
  const int w = wg_per_cu * kWaves / 4;
  return DS > 16 ? (w > 1 ? w / 2 : 1) : w;
}

// Head handled by this workgroup.  Workgroups are dispatched to the 8 XCDs
// round-robin, so consecutive block indices run on different XCDs.  For trees
// of 33+ nodes (5 row tiles) each XCD takes a contiguous range of heads
// instead (a bijection when the grid is a multiple of 8).  Measured on the
// (3,3,3) tree: commit-then-verify 619 -> 600 us, the pool form 627 -> 600 us,
// the bf16-state form 427 -> 418 us, verify alone unchanged.  On smaller trees
// it measured mixed (up to 14% slower), so they keep the plain order.
template <int RT>
__device__ __forceinline__ int head_of_block() {
  if constexpr (RT >= 5) {
    const int G = static_cast<int>(gridDim.x);
    if (G % 8 == 0) return static_cast<int>(blockIdx.x % 8) * (G / 8) + static_cast<int>(blockIdx.x / 8);
  }
  return static_cast<int>(blockIdx.x);
}

// One workgroup per (sequence, head).  With FUSED, the state is first
// committed for the previous step's accepted node (written to S_out) and the
// new step is verified from it.
template <int RT, int DS, bool F32IN, bool FUSED, bool POOL, bool S16, bool RAGGED = false>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(verify_waves_per_eu<RT, DS, FUSED, S16, RAGGED>(),
                                   verify_waves_per_eu<RT, DS, FUSED, S16, RAGGED>())))
void verify_kernel(const VerifyArgs a, const TreeArgs tree, const TreeArgs prev) {
  static_assert(!S16 || (FUSED && !F32IN), "bf16 state: commit-then-verify, bf16 inputs");
  static_assert(!RAGGED || (FUSED && POOL), "per-sequence trees: the pool form");
  using L = VerifyLayout<RT, DS, F32IN, FUSED>;
  using VT = typename std::conditional<F32IN, float, uint16_t>::type;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  __bf16* kq_hi = reinterpret_cast<__bf16*>(smem);
  __bf16* kq_lo = kq_hi + L::NP * kKQStride;  // F32IN only
  float* ys = reinterpret_cast<float*>(smem);  // P/B rows [0,N), R rows [N,2N); aliases kq
  VT* v_s = reinterpret_cast<VT*>(smem + L::OFF_V);
  float* ratio_s = reinterpret_cast<float*>(smem + L::OFF_RATIO);
  float* tabA = reinterpret_cast<float*>(smem + L::OFF_TA);
  float* tabM = reinterpret_cast<float*>(smem + L::OFF_TM);
  int8_t* path_s = reinterpret_cast<int8_t*>(smem + L::OFF_PATH);
  float* alpha_s = reinterpret_cast<float*>(smem + L::OFF_ALPHA);
  float* beta_s = reinterpret_cast<float*>(smem + L::OFF_BETA);
  float* gam_s = reinterpret_cast<float*>(smem + L::OFF_GAM);
  int8_t* depth_s = reinterpret_cast<int8_t*>(smem + L::OFF_DEPTH);
  int8_t* parent_s = reinterpret_cast<int8_t*>(smem + L::OFF_PARENT);

  const int H = a.H;
  const int gh = head_of_block<RT>();
  const int b = gh / H;
  const int h = gh - b * H;
  // Node count, and the row stride of gamma / vtilde.  With per-sequence
  // trees (RAGGED) they come from sequence b's descriptor and the padded
  // count; every field of a descriptor is clamped where it is read, so that
  // no descriptor can move an access out of bounds.
  int N = tree.n;
  int NS = tree.n;
  const TreeArgs* tdesc = nullptr;
  if constexpr (RAGGED) {
    tdesc = a.trees + b;
    const int cap = a.tok_b < L::NM ? a.tok_b : L::NM;
    const int nb = tdesc->n;
    N = nb < 1 ? 1 : (nb > cap ? cap : nb);
    NS = a.tok_b;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;

  using SS = SmallShape<RT, F32IN>;
  constexpr int CPR = SS::CPR;
  constexpr int KQ_PER = SS::KQ_PER;
  constexpr int V_PER = SS::V_PER;
  const int64_t tokstride = static_cast<int64_t>(H) * kD;  // t -> t+1 at fixed (b, h)
  const int64_t tok0 = (static_cast<int64_t>(b) * (a.tok_b ? a.tok_b : N) * H + h) * kD;

  // ---- 0. loads: every global load is issued before the first wait, small
  // rows first (with commit-then-verify, the previous step's path rows after
  // them), then the 64 KiB S0 block.  Vector-memory loads return in
  // order, so staging the small rows waits for them but not for S0.
  // the state block: the pool slot of sequence b (pool form, read first: the
  // S0 addresses wait for it), else block gh.  A slot outside the pool reads
  // slot 0 (n_slots >= 1) and turns the values to NaN where they are first
  // used: a branch around the loads would hold them back behind the small rows.
  int64_t sblk = gh;
  bool state_ok = true;
  if constexpr (POOL) {
    const int sl = a.slots[b];
    state_ok = sl >= 0 && sl < a.n_slots;
    sblk = static_cast<int64_t>(state_ok ? sl : 0) * H + h;
  }
  int m_depth = 0, m_parent = -1;
  if (tid < kMaxNodes) {
    if constexpr (RAGGED) {
      // the parent, clamped into [0, tid) (the root: -1); the depth is
      // recomputed from the parents after staging
      const int p = tdesc->parent[tid];
      m_parent = tid == 0 ? -1 : (p < 0 ? 0 : (p >= tid ? tid - 1 : p));
    } else {
      m_depth = tree.depth[tid];
      m_parent = tree.parent[tid];
    }
  }
  typename SS::Rows sr;
  load_small<RT, F32IN>(a, N, gh, sr);
  PathRows pr;
  if constexpr (FUSED) {
    if constexpr (RAGGED) {
      const TreeArgs* pdesc = a.trees_prev + b;
      const int pn = pdesc->n;
      load_path<F32IN, POOL>(a, pn < 0 ? 0 : (pn > a.n_prev ? a.n_prev : pn), pdesc->anc, gh, b, h,
                             pr);
    } else {
      load_path<F32IN, POOL>(a, prev.n, prev.anc, gh, b, h, pr);
    }
  }
  f32x4 s0[kS0Regs];
  uint4 s16[S16 ? kS16Regs : 1];
  if constexpr (S16) {
    load_s0_16(reinterpret_cast<const uint16_t*>(a.S0) + sblk * (kD * kD), wave, r16, g4, s16);
  } else {
    load_s0(a.S0 + sblk * (kD * kD), wave, r16, g4, s0);
  }

  // ---- 1. staging of the small rows into LDS --------------------------------
  if (tid < kMaxNodes) {
    depth_s[tid] = static_cast<int8_t>(m_depth);
    parent_s[tid] = static_cast<int8_t>(m_parent);
  }
  if (tid < N) {
    alpha_s[tid] = __uint_as_float(F32IN ? sr.ga : (sr.ga << 16));
    beta_s[tid] = __uint_as_float(F32IN ? sr.gb : (sr.gb << 16));
  }
  // k rows -> fragment rows [0, N), q rows -> [N, 2N).  Column c of a 32-column
  // block s sits at slot 8*(g%4) + 4*(g/4) + c%4 with g = (c%32)/4, matching
  // the S0 register layout above.
#pragma unroll
  for (int i = 0; i < KQ_PER; ++i) {
    const int idx = tid + kThreads * i;
    if (idx < 2 * N * CPR) {
      const int row = idx / CPR;
      const int j = idx - row * CPR;
      if constexpr (F32IN) {
        // 4 floats, columns 4j..4j+3: one 4-column group g = j % 8 of block j / 8
        const int g = j & 7;
        const int pos = row * kKQStride + 32 * (j >> 3) + 8 * (g & 3) + 4 * (g >> 2);
        const float xs[4] = {__uint_as_float(sr.kq[i].x), __uint_as_float(sr.kq[i].y),
                             __uint_as_float(sr.kq[i].z), __uint_as_float(sr.kq[i].w)};
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
      } else if constexpr (S16) {
        // natural k order (the bf16 state's layout): columns 8j..8j+7 in place
        *reinterpret_cast<uint4*>(kq_hi + row * kKQStride + 8 * j) = sr.kq[i];
      } else {
        // 8 bf16, columns 8j..8j+7: groups g0 = 2*(j%4) and g0+1 of block j / 4
        const int g0 = 2 * (j & 3);
        const int base = row * kKQStride + 32 * (j >> 2);
        const int pos0 = base + 8 * (g0 & 3) + 4 * (g0 >> 2);
        const int pos1 = base + 8 * ((g0 + 1) & 3) + 4 * ((g0 + 1) >> 2);
        *reinterpret_cast<uint2*>(kq_hi + pos0) = make_uint2(sr.kq[i].x, sr.kq[i].y);
        *reinterpret_cast<uint2*>(kq_hi + pos1) = make_uint2(sr.kq[i].z, sr.kq[i].w);
      }
    }
  }
  // zero the padding rows so the padded MFMA rows stay finite
  {
    const int pad_u4 = (L::NP - 2 * N) * kKQStride / 8;
    uint4* z0 = reinterpret_cast<uint4*>(kq_hi + 2 * N * kKQStride);
    uint4* z1 = reinterpret_cast<uint4*>(kq_lo + 2 * N * kKQStride);
    for (int idx = tid; idx < pad_u4; idx += kThreads) {
      z0[idx] = make_uint4(0, 0, 0, 0);
      if constexpr (F32IN) z1[idx] = make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < V_PER; ++i) {
    const int idx = tid + kThreads * i;
    if (idx < N * CPR) {
      reinterpret_cast<uint4*>(v_s)[idx] = sr.v[i];
    }
  }
  float* vtp_s = reinterpret_cast<float*>(smem + L::OFF_FUSE);
  if constexpr (FUSED) stage_path<F32IN>(pr, vtp_s, vtp_s + kPathChunk * kD);
  __syncthreads();

  // ---- 2a. root paths: lane t lists its path by depth, with the decay ratios
  // Gamma_t / Gamma_(ancestor at depth e) as products of alpha (no division),
  // and the path gate Gamma_t.
  if (tid < N) {
    const int t = tid;
    int dt;
    if constexpr (RAGGED) {
      // per-sequence trees: the depth by walking the clamped parents (a
      // tree deeper than the kernel's tables is cut there); other lanes
      // read depth_s only after the barrier that ends the MFMA phase
      int c = t, d = 0;
      while (c > 0 && d < DS - 1) {
        c = parent_s[c];
        ++d;
      }
      dt = d;
      depth_s[t] = static_cast<int8_t>(d);
    } else {
      dt = depth_s[t];
    }
    float r = 1.f;
    int cur = t;
    for (int e = dt; e >= 0; --e) {
      ratio_s[t * DS + e] = r;
      path_s[t * DS + e] = static_cast<int8_t>(cur);
      r *= alpha_s[cur];
      cur = parent_s[cur];
    }
    gam_s[t] = r;
  }

  if constexpr (FUSED) {
    // ---- 2a'. commit of the previous step into the S0 registers, then the
    // committed state goes to S_out (same layout as the loads).  Pool form: a
    // slot outside the pool read slot 0; its values turn to NaN here (and
    // nothing is written back), so every output of that sequence is NaN.
    [[maybe_unused]] const float nan = qnan();
    // (pool form: a bad slot writes nothing; "no previous step" leaves the
    // block as it is)
    const bool write_state = state_ok && !pr.keep;
    if constexpr (S16) {
      // bf16 state: widen to fp32 in the natural layout, commit, round the
      // committed state back to bf16 (the verify then runs on the stored value)
      // and store it
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
#pragma unroll
        for (int p = 0; p < 2; ++p) swap_lines16(s16[ct * 4 + 2 * p], s16[ct * 4 + 2 * p + 1], r16 < 8);
#pragma unroll
        for (int bs = 0; bs < 4; ++bs) unpack16(s16[ct * 4 + bs], s0[ct * 8 + 2 * bs], s0[ct * 8 + 2 * bs + 1]);
      }
      if constexpr (POOL) {
#pragma unroll
        for (int i = 0; i < kS0Regs; ++i) s0[i] = state_ok ? s0[i] : f32x4{nan, nan, nan, nan};
      }
      commit_in_registers<F32IN, true>(a, gh, b, h, pr, vtp_s, vtp_s + kPathChunk * kD, s0);
      uint16_t* So16 = reinterpret_cast<uint16_t*>(a.S_out) + sblk * (kD * kD);
      typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
#pragma unroll
        for (int bs = 0; bs < 4; ++bs) s16[ct * 4 + bs] = pack16(s0[ct * 8 + 2 * bs], s0[ct * 8 + 2 * bs + 1]);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          uint4 la = s16[ct * 4 + 2 * p];
          uint4 lb = s16[ct * 4 + 2 * p + 1];
          swap_lines16(la, lb, r16 < 8);
          if (write_state) {
            __builtin_nontemporal_store(u32x4{la.x, la.y, la.z, la.w},
                reinterpret_cast<u32x4*>(So16 + line_off16(wave, ct, p, r16, g4, false)));
            __builtin_nontemporal_store(u32x4{lb.x, lb.y, lb.z, lb.w},
                reinterpret_cast<u32x4*>(So16 + line_off16(wave, ct, p, r16, g4, true)));
          }
        }
      }
    } else {
    if constexpr (POOL) {
#pragma unroll
      for (int i = 0; i < kS0Regs; ++i) s0[i] = state_ok ? s0[i] : f32x4{nan, nan, nan, nan};
    }
#pragma unroll
    for (int i = 0; i < kS0Regs; i += 2) lines_to_mfma(s0[i], s0[i + 1], r16 < 8);
    commit_in_registers<F32IN>(a, gh, b, h, pr, vtp_s, vtp_s + kPathChunk * kD, s0);
    float* So = a.S_out + sblk * (kD * kD);
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f32x4 la = s0[ct * 8 + 2 * s];
        f32x4 lb = s0[ct * 8 + 2 * s + 1];
        mfma_to_lines(la, lb, r16 < 8);
        float* pa = So + line_off(wave, ct, s, r16, g4, false);
        float* pb = So + line_off(wave, ct, s, r16, g4, true);
        if (write_state) {
          __builtin_nontemporal_store(la, reinterpret_cast<f32x4*>(pa));
          __builtin_nontemporal_store(lb, reinterpret_cast<f32x4*>(pb));
        }
      }
    }
    }  // fp32 state
  } else {
#pragma unroll
    for (int i = 0; i < kS0Regs; i += 2) lines_to_mfma(s0[i], s0[i + 1], r16 < 8);
  }

  // ---- 2b. split S0 and run the contractions on MFMA ------------------------
  bf16x8 shi[kCT][4], slo[kCT][4];
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if constexpr (S16) {  // the state is exact in bf16: no residual term
        shi[ct][s] = __builtin_bit_cast(bf16x8, s16[ct * 4 + s]);
        continue;
      }
      const float xs[8] = {s0[ct * 8 + 2 * s].x, s0[ct * 8 + 2 * s].y, s0[ct * 8 + 2 * s].z,
                           s0[ct * 8 + 2 * s].w, s0[ct * 8 + 2 * s + 1].x, s0[ct * 8 + 2 * s + 1].y,
                           s0[ct * 8 + 2 * s + 1].z, s0[ct * 8 + 2 * s + 1].w};
      split_bf16x8(xs, shi[ct][s], slo[ct][s]);
    }
  }

  f32x4 acc[RT][kCT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int off = (rt * 16 + r16) * kKQStride + 32 * s + 8 * g4;
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(kq_hi + off);
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        acc[rt][ct] = mfma16(af, shi[ct][s], acc[rt][ct]);
        if constexpr (!S16) acc[rt][ct] = mfma16(af, slo[ct][s], acc[rt][ct]);
      }
      if constexpr (F32IN) {
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(kq_lo + off);
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) acc[rt][ct] = mfma16(al, shi[ct][s], acc[rt][ct]);
      }
    }
  }

  // gram tiles (row tile rt of [K;Q]) x (column tile gt of K), spread over waves
  const int GT = (N + 15) >> 4;
  constexpr int GTM = (RT + 1) / 2;
  constexpr int MAXG = (RT * GTM + kWaves - 1) / kWaves;
  f32x4 gacc[MAXG];
#pragma unroll
  for (int i = 0; i < MAXG; ++i) {
    gacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int tau = wave + kWaves * i;
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

  // ---- 3. P/R rows and the path entries of A and M to LDS -------------------
  // D layout of the 16x16 MFMA: lane holds rows 4*g4 + i (i < 4) of column r16.
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      const int m = wave * 16 * kCT + ct * 16 + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rt * 16 + 4 * g4 + i;
        if (row < 2 * N) ys[row * kYStride + m] = acc[rt][ct][i];
      }
    }
  }
  float* gram = reinterpret_cast<float*>(smem + L::OFF_GRAM);
#pragma unroll
  for (int i = 0; i < MAXG; ++i) {
    const int tau = wave + kWaves * i;
    if (tau < RT * GT) {
      const int rt = tau / GT;
      const int gt = tau - rt * GT;
      const int j = gt * 16 + r16;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int row = rt * 16 + 4 * g4 + ii;
        if constexpr (L::DENSE_GRAM) {
          gram[row * L::GS + j] = gacc[i][ii];
        } else if (j < N && row < 2 * N) {
          // j is on the root path of t iff it is t's ancestor at depth(j)
          const int t = row < N ? row : row - N;
          const int e = depth_s[j];
          const int d = depth_s[t];
          if (row < N) {
            if (e < d && path_s[t * DS + e] == j) {
              tabA[t * DS + e] = beta_s[t] * ratio_s[t * DS + e] * gacc[i][ii];
            }
          } else if (e <= d && path_s[t * DS + e] == j) {
            tabM[t * DS + e] = ratio_s[t * DS + e] * gacc[i][ii];
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- 4. tables T, M T (wave 0) and B = beta (v - Gamma P) (other waves) ---
  constexpr int OUT_PER = (L::NM * 32 + kThreads - 1) / kThreads;  // float4 chunks per thread
  if (wave == 0) {
    const float* gram = reinterpret_cast<const float*>(smem + L::OFF_GRAM);
    if constexpr (DS <= 4) {
      if (lane < N) {
        tables_short_paths(lane, N, L::GS, gram, path_s, ratio_s, beta_s, depth_s, tabA, tabM);
      }
    } else {
      // rows of A and M to LDS (already there without a dense gram), then
      // the column walk
      for (int t = lane; L::DENSE_GRAM && t < N; t += 64) {
        const int d = depth_s[t];
        const float be = beta_s[t];
        for (int e = 0; e <= d; ++e) {
          const int j = path_s[t * DS + e];
          const float r = ratio_s[t * DS + e];
          if (e < d) tabA[t * DS + e] = be * r * gram[t * L::GS + j];
          tabM[t * DS + e] = r * gram[(N + t) * L::GS + j];
        }
      }
      wave_sync();
      if (lane < DS) tables_by_column<DS>(lane, N, tabA, tabM, depth_s);
    }
  } else {
    for (int c = tid - 64; c < N * 32; c += kThreads - 64) {
      const int t = c >> 5;
      const int m4 = (c & 31) * 4;
      float vv[4];
      if constexpr (F32IN) {
        const float4 x = *reinterpret_cast<const float4*>(v_s + t * kD + m4);
        vv[0] = x.x; vv[1] = x.y; vv[2] = x.z; vv[3] = x.w;
      } else {
        const uint2 u = *reinterpret_cast<const uint2*>(v_s + t * kD + m4);
        vv[0] = __uint_as_float(u.x << 16);
        vv[1] = __uint_as_float(u.x & 0xffff0000u);
        vv[2] = __uint_as_float(u.y << 16);
        vv[3] = __uint_as_float(u.y & 0xffff0000u);
      }
      const float G = gam_s[t];
      const float be = beta_s[t];
      float4* py = reinterpret_cast<float4*>(ys + t * kYStride + m4);
      const float4 P = *py;
      *py = make_float4(be * (vv[0] - G * P.x), be * (vv[1] - G * P.y), be * (vv[2] - G * P.z),
                        be * (vv[3] - G * P.w));
    }
  }
  __syncthreads();

  // ---- 5. outputs: (node, 4 columns) chunks, sums along the root path ------
  // The gates go out here, with the other outputs: a store issued before the
  // wait for the S0 block (the wait counter counts stores too, and a store in
  // a branch makes that wait a full drain) made every workgroup wait for its
  // gate store as well as for S0.
  if (tid < N) {
    __builtin_nontemporal_store(gam_s[tid], a.gamma + static_cast<int64_t>(gh) * NS + tid);
  }
  float* vt_head = a.vtilde + static_cast<int64_t>(gh) * NS * kD;
#pragma unroll
  for (int i = 0; i < OUT_PER; ++i) {
    const int c = tid + kThreads * i;
    if (c < N * 32) {
      const int t = c >> 5;
      const int m4 = (c & 31) * 4;
      const int d = depth_s[t];
      float4 vt = make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 R = *reinterpret_cast<const float4*>(ys + (N + t) * kYStride + m4);
      const float G = gam_s[t];
      float4 o = make_float4(G * R.x, G * R.y, G * R.z, G * R.w);
      auto term = [&](int e) {
        const int p = path_s[t * DS + e];
        const float tv = tabA[t * DS + e];
        const float mv = tabM[t * DS + e];
        const float4 bb = *reinterpret_cast<const float4*>(ys + p * kYStride + m4);
        vt.x += tv * bb.x; vt.y += tv * bb.y; vt.z += tv * bb.z; vt.w += tv * bb.w;
        o.x += mv * bb.x; o.y += mv * bb.y; o.z += mv * bb.z; o.w += mv * bb.w;
      };
      if constexpr (DS <= 4) {
#pragma unroll
        for (int e = 0; e < DS; ++e) {
          if (e <= d) term(e);
        }
      } else {
        for (int e = 0; e <= d; ++e) term(e);
      }
      __builtin_nontemporal_store(f32x4{vt.x, vt.y, vt.z, vt.w},
                                  reinterpret_cast<f32x4*>(vt_head + t * kD + m4));
      __builtin_nontemporal_store(f32x4{o.x, o.y, o.z, o.w},
                                  reinterpret_cast<f32x4*>(a.out + tok0 + t * tokstride + m4));
    }
  }
}

template <int RT, int DS, bool F32IN, bool FUSED, bool POOL, bool S16, bool RAGGED>
hipError_t launch_rt(const VerifyArgs& a, const TreeArgs& tree, const TreeArgs& prev,
                     hipStream_t s) {
  hipLaunchKernelGGL((verify_kernel<RT, DS, F32IN, FUSED, POOL, S16, RAGGED>), dim3(a.B * a.H),
                     dim3(kThreads), 0, s, a, tree, prev);
  return hipGetLastError();
}

template <int DS, bool F32IN, bool FUSED, bool POOL, bool S16, bool RAGGED>
hipError_t launch_ds(const VerifyArgs& a, const TreeArgs& tree, const TreeArgs& prev, int rt,
                     hipStream_t s) {
  switch (rt) {
    case 1: return launch_rt<1, DS, F32IN, FUSED, POOL, S16, RAGGED>(a, tree, prev, s);
    case 2: return launch_rt<2, DS, F32IN, FUSED, POOL, S16, RAGGED>(a, tree, prev, s);
    case 3: return launch_rt<3, DS, F32IN, FUSED, POOL, S16, RAGGED>(a, tree, prev, s);
    case 4: return launch_rt<4, DS, F32IN, FUSED, POOL, S16, RAGGED>(a, tree, prev, s);
    case 5: return launch_rt<5, DS, F32IN, FUSED, POOL, S16, RAGGED>(a, tree, prev, s);
    case 6: return launch_rt<6, DS, F32IN, FUSED, POOL, S16, RAGGED>(a, tree, prev, s);
    case 7: return launch_rt<7, DS, F32IN, FUSED, POOL, S16, RAGGED>(a, tree, prev, s);
    case 8: return launch_rt<8, DS, F32IN, FUSED, POOL, S16, RAGGED>(a, tree, prev, s);
    default: return hipErrorInvalidValue;
  }
}

// Picks the kernel for a tree of tree.n nodes and depth tree.max_depth (with
// per-sequence trees: the bounds over the batch).
template <bool F32IN, bool FUSED, bool POOL = false, bool S16 = false, bool RAGGED = false>
hipError_t launch_dtype(const VerifyArgs& a, const TreeArgs& tree, const TreeArgs& prev,
                        hipStream_t s) {
  const int rt = (tree.n + 7) / 8;  // 2N rows of [K;Q] in 16-row tiles
  if (tree.max_depth < 4) return launch_ds<4, F32IN, FUSED, POOL, S16, RAGGED>(a, tree, prev, rt, s);
  if (tree.max_depth < 16) return launch_ds<16, F32IN, FUSED, POOL, S16, RAGGED>(a, tree, prev, rt, s);
  return launch_ds<64, F32IN, FUSED, POOL, S16, RAGGED>(a, tree, prev, rt, s);
}

}  // namespace
}  // namespace treewy
