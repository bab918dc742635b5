// Prefill of a chain in one launch: one workgroup per (sequence, head) keeps
// the 128x128 fp32 state in registers and walks the sequence in chunks of 16
// tokens, so the state crosses HBM once in and once out.
//
// A chain is a width-1 tree, so each chunk is the verification of a 16-node
// chain from the current state (method of "TreeWY: Speculative Verification
// for Gated DeltaNet Hybrids": paperpeel section 2's method summary and
// section 3 "Key rewrite"; the chunkwise WY form of DeltaNet it extends), and
// the state then moves to the chunk's last token (the commit, mlsanity
// abstract):
//   Gamma_t = prod_{i <= t} alpha_i                   (inside the chunk)
//   P = K S^T, R = Q S^T, KK = K K^T, QK = Q K^T      (MFMA)
//   (I + A) Vt = B,  A[t,j] = beta_t Gamma_t/Gamma_j KK[t,j] (j < t),
//                    B[t] = beta_t (v_t - Gamma_t P[t])
//   o_t = Gamma_t R[t] + sum_{j <= t} Gamma_t/Gamma_j QK[t,j] vt_j
//   S <- Gamma_last S + sum_j (Gamma_last/Gamma_j) vt_j k_j^T
// The last line is a rank-16 update of the state, done on MFMA: with the
// decay folded into vt (fp32, split into bf16 hi + lo) and k exact in bf16,
// the 16x16x16 MFMA's accumulator layout (lane (r16, g4) holds rows 4g4+i of
// column r16) is the state's own register layout when the product is taken
// as K'^T Vt per 16-column tile of the state, so the update accumulates into
// the state registers in place.  The factor Gamma_last on S is not applied to
// the registers: they hold S divided by a running product of the chunks'
// decays, which scales P, R and the pseudo-values instead (4 values per lane
// each, against 32 state registers).
//
// Per chunk: stage the chunk's rows (loaded during the previous chunk) into
// LDS and issue the next chunk's loads; gates; [K;Q] S^T and the gram on
// MFMA, P and R left in the accumulators; T = (I + A)^-1 by one wave, then B
// from P in registers in every wave; the pseudo-values T B and the outputs'
// M (T B) on MFMA, whose T B accumulator is the operand of both the second
// product and the state update in place; the state update.
#include "verify_kernel.h"

namespace treewy {
namespace {

constexpr int kPC = 16;           // tokens per chunk
constexpr int kPRT = 2;           // [K;Q] row tiles (2 kPC rows)
// bf16 per row of the transposed keys kt[c][t] (state column c, token t):
// 16 tokens + 8 pad, with the 4-token group of row c stored at group
// g ^ kt_swz(c >> 4) (kt_pos).  The state update reads 4 tokens of 16 rows per
// lane group (8 B per lane, one read per 16-row tile u) and the staging writes
// 8 columns of one token per lane.  Measured on this part (bank-conflict
// counter, one read instruction per pattern): reads of rows of 24 are
// conflict-free; rows of 20, 28 or 36 are not.  The swizzle differs between
// tiles u and u + 4: with equal swizzles their reads lie exactly 3072 B apart,
// the compiler pairs them into one two-address read, and both addresses of a
// lane fall in the same bank (a conflict on every such read; 1.1% of the
// prefill's time).  Rows stay 8-byte aligned for the reads.
constexpr int kKTS = kPC + 8;
__device__ __forceinline__ constexpr int kt_swz(int u) { return (u ^ (u >> 2)) & 3; }
__device__ __forceinline__ int kt_pos(int c, int t) { return c * kKTS + (t ^ (kt_swz(c >> 4) << 2)); }
constexpr int kPGS = 20;          // floats per gram row
constexpr int kPDS = kPC;         // path-table row length: a chunk is a chain of depth <= 15

template <bool F32IN>
struct PrefillLayout {
  static constexpr int NPL = F32IN ? 2 : 1;  // bf16 planes of k/q (hi, lo)
  // The staged rows of a chunk (k/q fragments, v, transposed k, gates), in
  // two copies: chunk c stages into copy c % 2, so its staging needs no
  // barrier against the previous chunk's last readers (of its k^T rows, in
  // the state update), which use the other copy.  Offsets within a copy:
  static constexpr int KQ_BYTES = 2 * kPC * kKQStride * 2 * NPL;
  static constexpr int S_V = KQ_BYTES;
  // v rows padded by 16 B: rows 4 tokens apart (one lane group each in B's
  // 2-byte reads) then fall on different banks
  static constexpr int V_ROW = kD * (F32IN ? 4 : 2) + 16;
  static constexpr int S_KT = S_V + kPC * V_ROW;
  static constexpr int S_ALPHA = S_KT + kD * kKTS * 2 * NPL;
  static constexpr int S_BETA = S_ALPHA + kPC * 4;
  static constexpr int STAGE = S_BETA + kPC * 4;
  static constexpr int OFF_GRAM = 2 * STAGE;
  static constexpr int OFF_RATIO = OFF_GRAM + 2 * kPC * kPGS * 4;
  static constexpr int OFF_TA = OFF_RATIO + kPC * kPDS * 4;  // A
  static constexpr int OFF_GAM = OFF_TA + kPC * kPDS * 4;
  // T and M as bf16 hi / lo pairs, split once by the wave that built them:
  // [4-column group][row][hi, lo] of 4 bf16 (8 B) each (the 16 lanes of a
  // group read 16 consecutive 16-byte entries: no bank conflict)
  static constexpr int OFF_TS = OFF_GAM + kPC * 4;
  static constexpr int OFF_MS = OFF_TS + kPC * 4 * 2 * 8;
  static constexpr int TOTAL = OFF_MS + kPC * 4 * 2 * 8;
  static_assert(S_V % 16 == 0 && S_KT % 16 == 0 && S_ALPHA % 16 == 0 && STAGE % 16 == 0 &&
                OFF_GRAM % 16 == 0 && OFF_RATIO % 16 == 0 && OFF_TS % 16 == 0, "16-byte rows");
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16k16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// One chunk's rows, held raw in VGPRs from their load (during the previous
// chunk) to their staging: the two gates of lane t < n, k/q and v rows in
// 16-byte chunks.  The gates stay 16-bit until staging: widened at the load,
// the widening would sit where the loop merges them and wait for the load
// right after it is issued.
template <bool F32IN>
struct ChunkRows {
  using GateT = typename std::conditional<F32IN, uint32_t, uint16_t>::type;
  GateT ga, gb;
  uint4 kq[SmallShape<kPRT, F32IN>::KQ_PER];
  uint4 v[SmallShape<kPRT, F32IN>::V_PER];
};

// Issues the loads of chunk c (n tokens) of sequence b, head h.  Every lane
// loads: indices past the chunk's rows are clamped to its last row (a branch
// around the loads would again make the loop wait for them at once).
template <bool F32IN>
__device__ __forceinline__ void load_chunk(const PrefillArgs& a, int c, int n, int b, int h,
                                           ChunkRows<F32IN>& sr) {
  using SS = SmallShape<kPRT, F32IN>;
  using GateT = typename ChunkRows<F32IN>::GateT;
  constexpr int IB = SS::IB, CPR = SS::CPR;
  const int tid = threadIdx.x;
  // Addresses: the chunk's first row (uniform, scalar arithmetic) plus a
  // 32-bit byte offset per lane (token t < 16 of the chunk: t * H rows of
  // kD inputs, below 2^32 for H <= 2^19)
  const uint32_t H = static_cast<uint32_t>(a.H);
  const int64_t row0 = (static_cast<int64_t>(b) * a.T + static_cast<int64_t>(c) * kPC) * a.H + h;
  const unsigned char* ga = static_cast<const unsigned char*>(a.alpha) + row0 * sizeof(GateT);
  const unsigned char* gb = static_cast<const unsigned char*>(a.beta) + row0 * sizeof(GateT);
  const unsigned char* kb = static_cast<const unsigned char*>(a.k) + row0 * (kD * IB);
  const unsigned char* qb = static_cast<const unsigned char*>(a.q) + row0 * (kD * IB);
  const unsigned char* vb = static_cast<const unsigned char*>(a.v) + row0 * (kD * IB);
  const uint32_t tn = static_cast<uint32_t>(tid < n ? tid : n - 1);
  const uint32_t gofs = tn * H * static_cast<uint32_t>(sizeof(GateT));
  sr.ga = *reinterpret_cast<const GateT*>(ga + gofs);
  sr.gb = *reinterpret_cast<const GateT*>(gb + gofs);
#pragma unroll
  for (int i = 0; i < SS::KQ_PER; ++i) {
    uint32_t idx = static_cast<uint32_t>(tid + kThreads * i);
    idx = idx < static_cast<uint32_t>(2 * n * CPR) ? idx : static_cast<uint32_t>(2 * n * CPR - 1);
    const uint32_t row = idx / CPR;
    const uint32_t j = idx - row * CPR;
    const bool is_k = row < static_cast<uint32_t>(n);
    const uint32_t t = is_k ? row : row - n;
    sr.kq[i] = *reinterpret_cast<const uint4*>((is_k ? kb : qb) + (t * H * (kD * IB) + 16 * j));
  }
#pragma unroll
  for (int i = 0; i < SS::V_PER; ++i) {
    uint32_t idx = static_cast<uint32_t>(tid + kThreads * i);
    idx = idx < static_cast<uint32_t>(n * CPR) ? idx : static_cast<uint32_t>(n * CPR - 1);
    const uint32_t t = idx / CPR;
    const uint32_t j = idx - t * CPR;
    sr.v[i] = *reinterpret_cast<const uint4*>(vb + (t * H * (kD * IB) + 16 * j));
  }
}

// Staging of one chunk's rows (loaded into `sr` by load_chunk):
// k rows -> fragment rows [0, n), q rows -> [kPC, kPC + n) in the A-fragment
// column order of the verify kernel (so that [K;Q] S^T leaves P in row tile 0
// and R in row tile 1 whatever n is); k also transposed into kT[c][t] (the A
// operand of the state update); v rows; the gates.  Fragment rows [n, kPC)
// and [kPC + n, 2 kPC) and columns [n, kPC) of kT are zeroed, so a short
// last chunk contributes nothing.
template <bool F32IN>
__device__ __forceinline__ void stage_chunk(const ChunkRows<F32IN>& sr, int n, unsigned char* sb) {
  using L = PrefillLayout<F32IN>;
  using SS = SmallShape<kPRT, F32IN>;
  constexpr int CPR = SS::CPR;
  const int tid = threadIdx.x;
  __bf16* kq_hi = reinterpret_cast<__bf16*>(sb);
  __bf16* kq_lo = kq_hi + 2 * kPC * kKQStride;
  __bf16* kt_hi = reinterpret_cast<__bf16*>(sb + L::S_KT);
  __bf16* kt_lo = kt_hi + kD * kKTS;
  float* alpha_s = reinterpret_cast<float*>(sb + L::S_ALPHA);
  float* beta_s = reinterpret_cast<float*>(sb + L::S_BETA);
  if (tid < n) {
    alpha_s[tid] = __uint_as_float(F32IN ? static_cast<uint32_t>(sr.ga)
                                         : (static_cast<uint32_t>(sr.ga) << 16));
    beta_s[tid] = __uint_as_float(F32IN ? static_cast<uint32_t>(sr.gb)
                                        : (static_cast<uint32_t>(sr.gb) << 16));
  }
#pragma unroll
  for (int i = 0; i < SS::KQ_PER; ++i) {
    const int idx = tid + kThreads * i;
    if (idx < 2 * n * CPR) {
      const int row = idx / CPR;
      const int j = idx - row * CPR;
      const bool is_k = row < n;
      const int frow = is_k ? row : kPC + (row - n);  // fragment row
      if constexpr (F32IN) {
        // 4 floats, columns 4j..4j+3: 4-column group g = j % 8 of block j / 8
        const int g = j & 7;
        const int pos = frow * kKQStride + 32 * (j >> 3) + 8 * (g & 3) + 4 * (g >> 2);
        const float xs[4] = {__uint_as_float(sr.kq[i].x), __uint_as_float(sr.kq[i].y),
                             __uint_as_float(sr.kq[i].z), __uint_as_float(sr.kq[i].w)};
        bf16x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          __bf16 hh, ll;
          split_bf16(xs[e], hh, ll);
          hi[e] = hh;
          lo[e] = ll;
          if (is_k) {
            kt_hi[kt_pos(4 * j + e, row)] = hh;
            kt_lo[kt_pos(4 * j + e, row)] = ll;
          }
        }
        *reinterpret_cast<bf16x4*>(kq_hi + pos) = hi;
        *reinterpret_cast<bf16x4*>(kq_lo + pos) = lo;
      } else {
        // 8 bf16, columns 8j..8j+7: groups g0 = 2*(j%4) and g0+1 of block j / 4
        const int g0 = 2 * (j & 3);
        const int base = frow * kKQStride + 32 * (j >> 2);
        const int pos0 = base + 8 * (g0 & 3) + 4 * (g0 >> 2);
        const int pos1 = base + 8 * ((g0 + 1) & 3) + 4 * ((g0 + 1) >> 2);
        *reinterpret_cast<uint2*>(kq_hi + pos0) = make_uint2(sr.kq[i].x, sr.kq[i].y);
        *reinterpret_cast<uint2*>(kq_hi + pos1) = make_uint2(sr.kq[i].z, sr.kq[i].w);
        if (is_k) {
          const uint32_t w[4] = {sr.kq[i].x, sr.kq[i].y, sr.kq[i].z, sr.kq[i].w};
          uint16_t* kt = reinterpret_cast<uint16_t*>(kt_hi);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            kt[kt_pos(8 * j + e, row)] =
                static_cast<uint16_t>((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
          }
        }
      }
    }
  }
  if (n < kPC) {
    // rows [n, kPC) of each row tile (k, then q)
    const int pad_u4 = (kPC - n) * kKQStride / 8;
    for (int idx = tid; idx < 2 * pad_u4; idx += kThreads) {
      const int tile = idx < pad_u4 ? 0 : 1;
      const int off = (tile * kPC + n) * kKQStride / 8 + (idx - tile * pad_u4);
      reinterpret_cast<uint4*>(kq_hi)[off] = make_uint4(0, 0, 0, 0);
      if constexpr (F32IN) reinterpret_cast<uint4*>(kq_lo)[off] = make_uint4(0, 0, 0, 0);
    }
    for (int idx = tid; idx < kD * kPC; idx += kThreads) {
      const int c = idx / kPC;
      const int t = idx - c * kPC;
      if (t >= n) {
        kt_hi[kt_pos(c, t)] = static_cast<__bf16>(0.f);
        if constexpr (F32IN) kt_lo[kt_pos(c, t)] = static_cast<__bf16>(0.f);
      }
    }
  }
  uint4* v_s = reinterpret_cast<uint4*>(sb + L::S_V);
#pragma unroll
  for (int i = 0; i < SS::V_PER; ++i) {
    const int idx = tid + kThreads * i;
    if (idx < n * CPR) {
      const int t = idx / CPR;
      v_s[t * (L::V_ROW / 16) + (idx - t * CPR)] = sr.v[i];
    }
  }
}

// The serial per-chunk work of one wave is written for a 16-token chain:
// rows of the small tables are read as float4 broadcasts, the loops over the
// chain are unrolled (no branch per entry, no wait per read), and entries
// past a row's end are exact zeros, so sums can run over whole rows.

// Gates of the chunk chain, lane t < n: Gamma_t / Gamma_e as the product of
// alpha over (e, t] (no division; 0 for e > t) into ratio row t, and Gamma_t.
__device__ __forceinline__ void chain_gates(int t, const float* alpha_s, float* ratio_s,
                                            float* gam_s) {
  float al[kPC];
#pragma unroll
  for (int q = 0; q < kPC / 4; ++q) {
    const float4 x = *reinterpret_cast<const float4*>(alpha_s + 4 * q);
    al[4 * q] = x.x; al[4 * q + 1] = x.y; al[4 * q + 2] = x.z; al[4 * q + 3] = x.w;
  }
  float rt[kPC];
  float r = 1.f;
#pragma unroll
  for (int e = kPC - 1; e >= 0; --e) {
    rt[e] = e <= t ? r : 0.f;
    r = e <= t ? r * al[e] : r;
  }
#pragma unroll
  for (int q = 0; q < kPC / 4; ++q) {
    *reinterpret_cast<float4*>(ratio_s + t * kPDS + 4 * q) =
        make_float4(rt[4 * q], rt[4 * q + 1], rt[4 * q + 2], rt[4 * q + 3]);
  }
  gam_s[t] = r;
}

// Rows of A and M from the gram, lane l of a wave: row t = l / 4, entries
// e = 4 (l % 4) .. +3.  A[t][e] = beta_t ratio[t][e] (k_t . k_e) for e < t,
// stored; M[t][e] = ratio[t][e] (q_t . k_e) for e <= t, returned in mv;
// zero elsewhere (rows t >= n are all zero, and so is A's diagonal).
__device__ __forceinline__ void chain_fill(int l, int n, const float* gram, const float* ratio_s,
                                           const float* beta_s, float* tabA, float (&mv)[4]) {
  const int t = l >> 2;
  const int q = l & 3;
  float av[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) mv[i] = 0.f;
  if (t < n) {
    const float4 gk = *reinterpret_cast<const float4*>(gram + t * kPGS + 4 * q);
    const float4 gq = *reinterpret_cast<const float4*>(gram + (kPC + t) * kPGS + 4 * q);
    const float4 r = *reinterpret_cast<const float4*>(ratio_s + t * kPDS + 4 * q);
    const float be = beta_s[t];
    const float kk[4] = {gk.x, gk.y, gk.z, gk.w}, qk[4] = {gq.x, gq.y, gq.z, gq.w};
    const float rr[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * q + i;
      av[i] = e < t ? be * rr[i] * kk[i] : 0.f;
      mv[i] = e <= t ? rr[i] * qk[i] : 0.f;
    }
  }
  *reinterpret_cast<float4*>(tabA + t * kPDS + 4 * q) = make_float4(av[0], av[1], av[2], av[3]);
}

// Lane 4 j + S of each quad's value, to every lane of the quad.
template <int S>
__device__ __forceinline__ float quad_bcast(float x) {
  return dpp_mov<S | (S << 2) | (S << 4) | (S << 6)>(x);  // quad_perm [S,S,S,S]
}

// T = (I + A)^-1 for the chunk chain, by the 64 lanes of one wave, as its
// transpose U = T^T = (I + A^T)^-1, column by column: lane 4 e + q keeps
// rows 4 q .. 4 q + 3 of column e of U, which are row e of T at columns
// 4 q .. 4 q + 3 -- the piece of T that lane (e, q) of the products takes as
// its operand, so T leaves the walk in registers.  U is unit upper
// triangular: U[f][e] = [f = e] - sum_{j > f} A[j][f] U[j][e], taken from the
// last row up.  Once row f of U is final (its lane broadcasts it to the
// quad), every earlier row t takes its term -A[f][t] U[f][e] at once, one FMA
// per register, from row f of A (a float4 per lane).  The serial path is one
// quad broadcast and one FMA per row; the 8 x 8 blocked inverse it replaces
// walked 8 rows of quad sums and then formed T21 = -T22 A21 T11 through LDS.
// Entries past n: A's rows f >= n are zero and so is the start of column
// e >= n, so T's rows and columns past n come out zero.
template <int F, int D>
__device__ __forceinline__ void chain_walk(float (&acc)[4], float4 (&ar)[D], const float* tabA, int q) {
  if constexpr (F >= 0) {
    const float tf = quad_bcast<F / 4>(acc[F % 4]);
    if constexpr (F > 0) {
      const float4 a4 = ar[F % D];
      // row F - D of A into the freed slot: the reads run D rows ahead of the
      // walk, which would otherwise wait on each one
      if constexpr (F - D > 0) ar[F % D] = *reinterpret_cast<const float4*>(tabA + (F - D) * kPDS + 4 * q);
      const float a[4] = {a4.x, a4.y, a4.z, a4.w};
      // the next row's register first: it is the next broadcast's input
      constexpr int k0 = (F - 1) % 4;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int k = (k0 + 4 - d) % 4;
        if (k < F) acc[k] = fmaf(-a[k], tf, acc[k]);  // rows 4 q + k < F for some q
      }
    }
    chain_walk<F - 1, D>(acc, ar, tabA, q);
  }
}

// The tables of the chunk chain by one wave: A and M from the gram, T by the
// walk, and T and M split into bf16 hi / lo pairs for every wave's products.
__device__ __forceinline__ void chain_tables(int lane, int n, const float* gram, const float* ratio_s,
                                             const float* beta_s, float* tabA, uint2* tsplit,
                                             uint2* msplit) {
  float mv[4];
  chain_fill(lane, n, gram, ratio_s, beta_s, tabA, mv);
  wave_sync();
  const int e = lane >> 2;
  const int q = lane & 3;
  float acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = (4 * q + k == e && e < n) ? 1.f : 0.f;
  constexpr int kAhead = 6;  // rows of A in flight
  float4 ar[kAhead];
#pragma unroll
  for (int d = 0; d < kAhead; ++d) {
    const int f = kPC - 1 - d;
    ar[f % kAhead] = *reinterpret_cast<const float4*>(tabA + f * kPDS + 4 * q);
  }
  chain_walk<kPC - 1, kAhead>(acc, ar, tabA, q);
  // row e of T, columns 4 q .. +3, and (fill lanes) row e of M, the same
  // columns: entry (q, e) of the [4-column group][row] split tables
  bf16x4 th, tl, mh, ml;
  split_bf16x4(acc, th, tl);
  split_bf16x4(mv, mh, ml);
  tsplit[(q * 16 + e) * 2] = __builtin_bit_cast(uint2, th);
  tsplit[(q * 16 + e) * 2 + 1] = __builtin_bit_cast(uint2, tl);
  msplit[(q * 16 + e) * 2] = __builtin_bit_cast(uint2, mh);
  msplit[(q * 16 + e) * 2 + 1] = __builtin_bit_cast(uint2, ml);
}

// Register budget as resident workgroups per CU: 2 for 16-bit inputs; fp32
// inputs hold a second plane of k/q fragments and would spill at that budget.
constexpr int kPrefillWg = 2;
template <bool F32IN>
constexpr int prefill_waves_per_eu() {
  return (F32IN ? 1 : kPrefillWg) * kWaves / 4;
}

template <bool F32IN>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(prefill_waves_per_eu<F32IN>(), prefill_waves_per_eu<F32IN>())))
void prefill_kernel(const PrefillArgs a) {
  static_assert(kWaves == 8, "one 16-row tile of the state per wave");
  using L = PrefillLayout<F32IN>;
  using SS = SmallShape<kPRT, F32IN>;
  using VT = typename std::conditional<F32IN, float, uint16_t>::type;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::TOTAL];
  float* gram = reinterpret_cast<float*>(smem + L::OFF_GRAM);
  float* ratio_s = reinterpret_cast<float*>(smem + L::OFF_RATIO);
  float* tabA = reinterpret_cast<float*>(smem + L::OFF_TA);
  float* gam_s = reinterpret_cast<float*>(smem + L::OFF_GAM);
  uint2* tsplit = reinterpret_cast<uint2*>(smem + L::OFF_TS);
  uint2* msplit = reinterpret_cast<uint2*>(smem + L::OFF_MS);

  const int T = a.T;
  const int H = a.H;
  const int gh = blockIdx.x;
  const int b = gh / H;
  const int h = gh - b * H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  const int64_t tokstride = static_cast<int64_t>(H) * kD;
  const int64_t tok0 = (static_cast<int64_t>(b) * T * H + h) * kD;

  const int nchunks = (T + kPC - 1) / kPC;

  // ---- chunk 0's rows, then the state block (returned in that order); the
  // state goes into the MFMA layout before the loop (T >= 1)
  ChunkRows<F32IN> sr;
  load_chunk<F32IN>(a, 0, T < kPC ? T : kPC, b, h, sr);
  f32x4 s0[kS0Regs];
  float* Sh = a.S + static_cast<int64_t>(gh) * (kD * kD);
  load_s0(Sh, wave, r16, g4, s0);
#pragma unroll
  for (int i = 0; i < kS0Regs; i += 2) lines_to_mfma(s0[i], s0[i + 1], r16 < 8);

  // One chunk of n tokens (FULL: n = kPC); full chunks run in a loop, a ragged
  // last chunk once after it.  A chunk's outputs are stored at the start of
  // the next chunk, right after its rows are staged, and before that chunk
  // issues the loads of the rows after it: the wait counter for vector memory
  // counts stores as well as loads, and waiting for the prefetched rows with
  // this chunk's output stores issued after them drained those stores too
  // (every chunk waited for its own output stores).  Stored a chunk later,
  // they have a whole chunk to complete before the next wait.
  float o_pend[4] = {0.f, 0.f, 0.f, 0.f};  // the previous chunk's outputs (full chunk)
  // The registers hold the state divided by a running decay g (uniform):
  // S = g * s0.  The chunk's decay Gamma_last then scales g instead of the
  // 32 state registers; P and R are scaled by g in their 4 uses per lane and
  // the update's pseudo-values by 1 / (g Gamma_last).  When g leaves
  // [2^-100, 2^100] (or is zero or not finite) it is applied to the registers
  // and restarts at 1, so s0 and the scaled pseudo-values stay far inside
  // fp32's range.
  float g = 1.f;
  auto store_outputs = [&](const int c, const int n, const bool full) {
    int lq = tid;
    asm volatile("" : "+v"(lq));
    const uint32_t m = static_cast<uint32_t>(wave * 16 + (lq & 15));
    const uint32_t ug4 = (static_cast<uint32_t>(lq) >> 4) & 3u;
    // the chunk's first output row (uniform) plus a 32-bit byte offset per
    // lane: 4 (t H kD + m) < 2^32 for t < 16 and H <= 2^19
    unsigned char* obase = reinterpret_cast<unsigned char*>(a.out + tok0 + static_cast<int64_t>(c) * kPC * tokstride);
    const uint32_t H32 = static_cast<uint32_t>(H);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t t = 4 * ug4 + i;
      if (full || t < static_cast<uint32_t>(n)) {
        __builtin_nontemporal_store(o_pend[i], reinterpret_cast<float*>(obase + 4 * (t * H32 * kD + m)));
      }
    }
  };
  auto chunk = [&](const int c, auto full) {
    constexpr bool FULL = decltype(full)::value;
    const int n = FULL ? kPC : T - c * kPC;
    // this chunk's copy of the staged rows (no barrier before the staging:
    // the previous chunk's readers after its last barrier use the other copy)
    unsigned char* sb = smem + (c & 1) * L::STAGE;
    const __bf16* kq_hi = reinterpret_cast<const __bf16*>(sb);
    const __bf16* kq_lo = kq_hi + 2 * kPC * kKQStride;
    const VT* v_s = reinterpret_cast<const VT*>(sb + L::S_V);
    const __bf16* kt_hi = reinterpret_cast<const __bf16*>(sb + L::S_KT);
    const __bf16* kt_lo = kt_hi + kD * kKTS;
    const float* alpha_s = reinterpret_cast<const float*>(sb + L::S_ALPHA);
    const float* beta_s = reinterpret_cast<const float*>(sb + L::S_BETA);
    stage_chunk<F32IN>(sr, n, sb);
    // Every lane takes its prefetched rows here, also the lanes that staged
    // none of them: a wave that skips the staging would otherwise wait for
    // those loads only where their registers are next written, after the
    // output stores below, and that wait would drain the stores too.
    asm volatile("" ::"v"(sr.ga), "v"(sr.gb));
#pragma unroll
    for (int i = 0; i < SS::KQ_PER; ++i) {
      asm volatile("" ::"v"(sr.kq[i].x), "v"(sr.kq[i].y), "v"(sr.kq[i].z), "v"(sr.kq[i].w));
    }
#pragma unroll
    for (int i = 0; i < SS::V_PER; ++i) {
      asm volatile("" ::"v"(sr.v[i].x), "v"(sr.v[i].y), "v"(sr.v[i].z), "v"(sr.v[i].w));
    }
    // The next chunk's rows (the last chunk reloads itself: no branch), as
    // soon as this chunk's are staged: they have the whole chunk to arrive.
    // Issued before the output stores, so that the wait for them at the next
    // staging leaves those stores in flight.  (Any wait on vector memory also
    // waits for loads issued before it: with register spills present, the
    // spill reloads waited for these loads, and issuing them after the
    // tables was faster, 2.55 against 2.74 ms; without spills, here is faster
    // than after the tables, 1013 against 1025 us on 256 x 256 tokens x 32
    // heads.  Staging the rows into the other LDS copy in the middle of the
    // chunk kept them live in more registers, spilled, and measured slower.)
    {
      const int cn = c + 1 < nchunks ? c + 1 : c;
      const int nn = (T - cn * kPC) < kPC ? (T - cn * kPC) : kPC;
      load_chunk<F32IN>(a, cn, nn, b, h, sr);
    }
    if (c > 0) store_outputs(c - 1, kPC, true);  // only the last chunk can be ragged
    __syncthreads();

    // gates: lane t < n of wave 2 lists Gamma_t / Gamma_e (e <= t) as
    // products of alpha over (e, t], and Gamma_t.  Not on wave 0: that wave
    // builds the tables and shares its SIMD with wave 4, and the gates on
    // another SIMD measured 2% faster.
    if (wave == 2 && lane < n) chain_gates(lane, alpha_s, ratio_s, gam_s);

    // [K;Q] S^T with S split into bf16 hi + lo (fp32 inputs: k/q split too)
    f32x4 acc[kPRT];
#pragma unroll
    for (int rt = 0; rt < kPRT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 shi, slo;
      const float xs[8] = {s0[2 * s].x, s0[2 * s].y, s0[2 * s].z, s0[2 * s].w,
                           s0[2 * s + 1].x, s0[2 * s + 1].y, s0[2 * s + 1].z, s0[2 * s + 1].w};
      split_bf16x8(xs, shi, slo);
      // the two row tiles' accumulations alternate, so that no product
      // waits on the one issued just before it
      bf16x8 af[kPRT];
#pragma unroll
      for (int rt = 0; rt < kPRT; ++rt) {
        af[rt] = *reinterpret_cast<const bf16x8*>(kq_hi + (rt * 16 + r16) * kKQStride + 32 * s + 8 * g4);
      }
#pragma unroll
      for (int rt = 0; rt < kPRT; ++rt) acc[rt] = mfma16(af[rt], shi, acc[rt]);
#pragma unroll
      for (int rt = 0; rt < kPRT; ++rt) acc[rt] = mfma16(af[rt], slo, acc[rt]);
      if constexpr (F32IN) {
#pragma unroll
        for (int rt = 0; rt < kPRT; ++rt) {
          const bf16x8 al =
              *reinterpret_cast<const bf16x8*>(kq_lo + (rt * 16 + r16) * kKQStride + 32 * s + 8 * g4);
          acc[rt] = mfma16(al, shi, acc[rt]);
        }
      }
    }
    // gram [K;Q] K^T: row tile `wave` (waves 0, 1) against the 16 key rows
    f32x4 gacc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (wave < kPRT) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int offa = (wave * 16 + r16) * kKQStride + 32 * s + 8 * g4;
        const int offb = r16 * kKQStride + 32 * s + 8 * g4;
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(kq_hi + offa);
        const bf16x8 bf = *reinterpret_cast<const bf16x8*>(kq_hi + offb);
        gacc = mfma16(af, bf, gacc);
        if constexpr (F32IN) {
          const bf16x8 al = *reinterpret_cast<const bf16x8*>(kq_lo + offa);
          const bf16x8 bl = *reinterpret_cast<const bf16x8*>(kq_lo + offb);
          gacc = mfma16(al, bf, gacc);
          gacc = mfma16(af, bl, gacc);
        }
      }
    }
    // P and R stay in the accumulators: lane (r16, g4) holds tokens 4 g4 + i
    // of state row m = 16 wave + r16, of P in acc[0] and of R in acc[1] --
    // the layout in which this lane takes B in T B and forms its outputs.
    // The gram goes to LDS for the tables.
    if (wave < kPRT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) gram[(wave * 16 + 4 * g4 + i) * kPGS + r16] = gacc[i];
    }
    __syncthreads();  // the gram and the gates visible

    // the rows of A and M and T = (I + A)^-1 (wave 0), then in every wave
    // B = beta (v - Gamma P) for its own tokens and state rows, in registers
    // (zero past n)
    if (wave == 0) {
      // the serial walk bounds the phase: its wave is issued first while it
      // shares a SIMD with the other workgroup's waves
      __builtin_amdgcn_s_setprio(3);
      chain_tables(lane, n, gram, ratio_s, beta_s, tabA, tsplit, msplit);
      __builtin_amdgcn_s_setprio(0);
    }
    float bv[4];
    float gg[4];  // g Gamma_t of this lane's tokens: the scale of P and R
    {
      const int m = wave * 16 + r16;
      const float4 be4 = *reinterpret_cast<const float4*>(beta_s + 4 * g4);
      const float4 ga4 = *reinterpret_cast<const float4*>(gam_s + 4 * g4);
      const float be[4] = {be4.x, be4.y, be4.z, be4.w};
      gg[0] = g * ga4.x; gg[1] = g * ga4.y; gg[2] = g * ga4.z; gg[3] = g * ga4.w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * g4 + i;
        float vv;
        if constexpr (F32IN) {
          vv = v_s[t * (L::V_ROW / 4) + m];
        } else {
          vv = bf16_bits_to_f32(v_s[t * (L::V_ROW / 2) + m]);
        }
        const float x = be[i] * (vv - gg[i] * acc[0][i]);
        bv[i] = (FULL || t < n) ? x : 0.f;
      }
    }
    __syncthreads();

    // Pseudo-values and outputs: wave w takes the state columns
    // m = 16 w + r16.  The T B accumulator holds tokens 4 g4 + i of column m,
    // which is this lane's B operand in the state update below, so the
    // pseudo-values stay in registers.  Lane indices come from an opaque copy
    // of tid: per-thread addresses hoisted out of the chunk loop are spilled,
    // and a reload waits for the loads issued above.
    int lq = tid;
    asm volatile("" : "+v"(lq));
    const int ur16 = lq & 15;
    const int ug4 = (lq >> 4) & 3;
    const int m = wave * 16 + ur16;
    // the decay's last gate first, then the update's k^T operands: read here,
    // they arrive during the T B and M (T B) products instead of in front of
    // the update (LDS returns in order, so the gate read waits for none of them)
    const float glast = gam_s[n - 1];
    bf16x4 kta[kS0Regs];
#pragma unroll
    for (int u = 0; u < kS0Regs; ++u) {
      // row c = 16 u + ur16: tokens 4 ug4 .. + 3 at group ug4 ^ kt_swz(u) (kt_pos)
      kta[u] = *reinterpret_cast<const bf16x4*>(kt_hi + (16 * u + ur16) * kKTS + 4 * (ug4 ^ kt_swz(u)));
    }
    // the decay after this chunk: g Gamma_last, or 1 after applying it to
    // the registers (positive floats order as unsigned integers, and
    // negatives and NaNs fall outside the range).  The test is written per
    // lane: with the decay read into a scalar register first, the compiler
    // gave the rare branch's scaled state new registers and copied the state
    // into them on the common path, every chunk.
    float inv;  // 1 / (new g): the scale of the pseudo-values in the update
    {
      const float gn = g * glast;
      constexpr uint32_t kLo = 0x0d800000u;  // 2^-100
      constexpr uint32_t kHi = 0x71800000u;  // 2^100
      const bool keep = __float_as_uint(gn) - kLo <= kHi - kLo;
      if (!keep) {
#pragma unroll
        for (int i = 0; i < kS0Regs; ++i) s0[i] *= gn;
      }
      g = keep ? gn : 1.f;
      inv = keep ? __builtin_amdgcn_rcpf(gn) : 1.f;
    }
    float vt[4];
    {
      // T B, then M (T B): 16 x 16 x 16 products on bf16 MFMA, each fp32
      // operand split into hi + lo (three passes: hi hi, hi lo, lo hi).  The
      // accumulator of T B (tokens 4 g4 + i of column m) is the B operand of
      // M (T B) in this lane, so M T is never formed.  Rows of T and M are
      // whole (zero past n); rows of B past n enter as zeros.
      const int ts = (ug4 * 16 + ur16) * 2;
      const bf16x4 tah = __builtin_bit_cast(bf16x4, tsplit[ts]);
      const bf16x4 tal = __builtin_bit_cast(bf16x4, tsplit[ts + 1]);
      const bf16x4 mah = __builtin_bit_cast(bf16x4, msplit[ts]);
      const bf16x4 mal = __builtin_bit_cast(bf16x4, msplit[ts + 1]);
      bf16x4 bbh, bbl;
      split_bf16x4(bv, bbh, bbl);
      f32x4 accT = f32x4{0.f, 0.f, 0.f, 0.f};
      accT = mfma16k16(tah, bbh, accT);
      accT = mfma16k16(tah, bbl, accT);
      accT = mfma16k16(tal, bbh, accT);
      bf16x4 vh, vl;
      {
        const float at[4] = {accT[0], accT[1], accT[2], accT[3]};
        split_bf16x4(at, vh, vl);
      }
      f32x4 accM = f32x4{0.f, 0.f, 0.f, 0.f};
      accM = mfma16k16(mah, vh, accM);
      accM = mfma16k16(mah, vl, accM);
      accM = mfma16k16(mal, vh, accM);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * ug4 + i;
        vt[i] = 0.f;
        o_pend[i] = 0.f;
        if (FULL || t < n) {
          o_pend[i] = gg[i] * acc[1][i] + accM[i];
          vt[i] = (inv * ratio_s[(n - 1) * kPDS + t]) * accT[i];  // Gamma_last / (g' Gamma_t)
        }
      }
    }

    // state update: S <- Gamma_last S + K'^T Vt per 16-column tile u of the
    // state (register u), Vt split into bf16 hi + lo; the decay is in g
    {
      bf16x4 bh, bl;
      split_bf16x4(vt, bh, bl);
#pragma unroll
      for (int u = 0; u < kS0Regs; ++u) {
        s0[u] = mfma16k16(kta[u], bh, s0[u]);
        s0[u] = mfma16k16(kta[u], bl, s0[u]);
        if constexpr (F32IN) {
          const int kto = (16 * u + ur16) * kKTS + 4 * (ug4 ^ kt_swz(u));
          const bf16x4 kl = *reinterpret_cast<const bf16x4*>(kt_lo + kto);
          s0[u] = mfma16k16(kl, bh, s0[u]);
        }
      }
    }
  };
  const int nfull = T / kPC;
  for (int c = 0; c < nfull; ++c) chunk(c, std::true_type{});
  if (nfull < nchunks) chunk(nfull, std::false_type{});
  // the last chunk's outputs
  store_outputs(nchunks - 1, T - (nchunks - 1) * kPC, nfull == nchunks);

  // ---- the state after the last token, back in place
#pragma unroll
  for (int i = 0; i < kS0Regs; ++i) s0[i] *= g;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    f32x4 la = s0[2 * s];
    f32x4 lb = s0[2 * s + 1];
    mfma_to_lines(la, lb, r16 < 8);
    __builtin_nontemporal_store(la, reinterpret_cast<f32x4*>(Sh + line_off(wave, 0, s, r16, g4, false)));
    __builtin_nontemporal_store(lb, reinterpret_cast<f32x4*>(Sh + line_off(wave, 0, s, r16, g4, true)));
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  if (a.f32_inputs) {
    hipLaunchKernelGGL(prefill_kernel<true>, dim3(a.B * a.H), dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(prefill_kernel<false>, dim3(a.B * a.H), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace treewy
