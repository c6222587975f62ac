// Forward kernel: tiled Q K^T, online safe softmax with running max and sum, optional stabilised
// shift for repeated maxima, P^ V accumulation, final normalisation and the saved logsumexp.
//
// Follows the online softmax of the BF16 Flash Attention article (ijyty.com/news/896914) §2.1 and
// the repeated-maximum shift of its §4.1, with the precision schedule of "Flash Attention低精度
// 训练稳定性优化实践" (jsqmd.com/news/761560) §3.2: Q K^T accumulated in fp32, softmax in fp32,
// P^ rounded to the 16-bit element type for the product with V.  That article names both 16-bit
// formats; the element type (bf16 or fp16) is a template parameter, and this file is compiled once
// per element type (FA_ELEM).  A third instance (FA_ELEM = 2) is the bf16 forward with the P^ V
// product in FP8 E4M3, the lower precision the article's §6.1 extends the method to, together with
// the kernel that quantises V for it (v8_pack_kernel).
//
// Work split: one workgroup of 8 waves per (query tile of 256 rows, head).  Each wave owns 32
// queries and computes S^T = K Q^T, so each lane owns one query column: its row max, repeat count
// and row sum are lane-local up to one exchange between the two 32-lane halves.  O^T is
// accumulated as V^T P^T so that the per-query rescale factor is lane-local too, and P^ goes from
// the accumulator registers straight into the next MFMA's operand without touching LDS.
//
// Ping-pong: on gfx950 a wave overlaps only a few vector instructions with its own matrix
// instructions, but two waves on one SIMD overlap almost completely when one issues MFMAs and the
// other vector work.  The 8 waves form two groups (waves 0-3 and 4-7, one of each per SIMD) that
// run in alternate phases separated by workgroup barriers:
//   matrix phase M(j): S^T of block j, then O += V^T P^T of block j-1     (MFMA)
//   vector phase V(j): mask, max/count/shift, P^ of block j, rescale O    (VALU)
// Group A runs M(0) V(0) M(1) V(1) ...; group B runs one phase behind, so in every phase one group
// works on the matrix cores while the other works on the vector ALUs.  K and V blocks (128 keys
// when causal, 64 otherwise) are double-buffered in LDS: K_{j+1} and V_j are loaded during phase
// 2j; K_j is read in phases 2j (A) and 2j+1 (B), V_j in phases 2j+2 (A) and 2j+3 (B).  Longer
// blocks halve the barriers per key; the non-causal instances run out of registers at 128.
#include <climits>
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

#ifndef FA_ELEM
#error "FA_ELEM (the element type this translation unit instantiates) must be defined"
#endif

namespace fa {

// Keys per block: 128 when causal; 64 otherwise (the non-causal instances spill at 128).  The
// FP8 P^ V instances always take 128 (their P^ packs into half the registers, and V arrives in
// 128-key blocks, each with its own scale).
template <int E, bool CAUSAL>
constexpr int fwd_bc() { return (CAUSAL || E == kElemFp8PV) ? 128 : 64; }
constexpr int kFwdBr = 256;  // queries per workgroup
constexpr int kFwdThreads = 512;

// Per-lane running state of the online softmax for one query (this lane's column).
struct RowState {
  float run_max;  // running max of the raw dot products q.k
  int run_cnt;    // how many visible keys attain it (exact count: diagnostics variant)
  float run_m2;   // second-largest raw dot product, counted with multiplicity (mode 1)
  float m2;       // current shift, in log2 units of the scaled score
  float lsum;     // this half-wave's share of the row sum
  float lcomp;    // its compensation term (compensated-sum variant): lost low-order part, negated
  float run_min;  // running min of the raw dot products over visible keys (diagnostics variant)
  int n_ones;     // exact-1.0 16-bit P^ values seen (stats variant)
  float vs;       // FP8 P^ V: scale of the V block last added (O is held in units of vs / 2^8)
};

// The shift m of the repeated-maximum rule, in log2 units of the scaled score, from the running
// state: m = beta r when the running maximum r is positive and repeats, 0 when it is negative and
// repeats, r otherwise (mode 2 takes every row as repeating).  Mode 1 knows whether r repeats from
// the two largest scores (TOP2) or from the exact count (the diagnostics variant).
template <int MODE, bool TOP2>
__device__ __forceinline__ float page_shift(const RowState& rs, float sl2, float beta) {
  const float r2 = rs.run_max * sl2;
  if (MODE == 0) return r2;
  const bool rep = (MODE == 2) || (TOP2 ? (rs.run_m2 == rs.run_max) : (rs.run_cnt > 1));
  return (rep && r2 > 0.f) ? beta * r2 : ((rep && r2 < 0.f) ? 0.f : r2);
}

// The shift the exponentials are taken against.  Under the rule's shift the largest P^ of a row is
// 2^(r - m), far below 1 when m - r is large (a large repeated maximum, or a negative one shifted
// to 0), and the 16-bit (or E4M3) rounding of P^ for the V product would go subnormal and then to
// zero, silently zeroing O.  When m - r exceeds kT, the exponent is taken against m minus a whole
// number of binades, so the largest P^ lands in (2^-(kT+1), 2^-kT]: O, l and the rescale factors
// all carry the same power of two, which cancels in O / l and is the shift's own part of the saved
// logsumexp (LSE = shift + log l).  The rounding of P^ is unchanged in relative terms, and P^ stays
// well below 1, so no exact 1.0 appears.  kT = 13 keeps 16-bit P^ in fp16's normal range (down to
// 2^-14); the FP8 variant forms 2^8 P^ and takes kT = 5 (largest value in (4, 8], E4M3 normal from
// 2^-6).  A lane that has seen no key yet (r = -inf) keeps the rule's value.
template <bool FP8>
__device__ __forceinline__ float exponent_shift(float m2, float r2) {
  constexpr float kT = FP8 ? 5.f : 13.f;
  const float gap = m2 - r2;
  const float ofs = (gap > kT && gap < 1048576.f) ? floorf(gap) - kT : 0.f;
  return m2 - ofs;
}

template <int E, int D, bool CAUSAL, int MODE, bool STATS, bool KAHAN>
__global__ __launch_bounds__(kFwdThreads, 1) void fwd_kernel(FwdArgs a) {
  constexpr int BC = fwd_bc<E, CAUSAL>(), BR = kFwdBr, KS = D / 16, DT = D / 32, KB = BC / 32;
  constexpr bool FP8 = (E == kElemFp8PV);
  static_assert(!FP8 || BC == 128, "the FP8 V blocks hold 128 keys");
  // Mode 1 needs only whether the running maximum repeats: without the diagnostics that is
  // decided by tracking the two largest scores; the diagnostics need the exact count.
  constexpr bool TOP2 = (MODE == 1) && !STATS;
  constexpr bool COUNT = STATS;
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: leads, 1: one phase behind
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  int bh, rank;
  map_block(blockIdx.x, a.BH, a.n_tiles, bh, rank);
  const int qt = CAUSAL ? a.n_tiles - 1 - rank : rank;
  const int Nq = a.Nq, Nk = a.Nk;
  const int q0 = qt * BR;
  const int64_t qoff = (int64_t)bh * Nq * D;
  const int64_t koff = (int64_t)bh * Nk * D;
  const uint16_t* Qg = a.q + qoff;
  const uint16_t* Kg = a.k + koff;
  const uint16_t* Vg = a.v + koff;

  const int qw0 = q0 + wave * 32;  // first query of this wave
  const int qrow = qw0 + l32;      // this lane's query (causal: it sees keys up to qrow + coff)

  // Q^T as the B operand: lane holds Q[qrow][16 ks + 8 hh .. + 7].
  e16x8 qf[KS];
  {
    const uint16_t* src = Qg + (int64_t)min(qrow, Nq - 1) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_e16x8(*reinterpret_cast<const i32x4*>(src + 16 * ks));
  }

  int n_kv = (Nk + BC - 1) / BC;
  if (CAUSAL) n_kv = min(n_kv, blocks_through(q0 + BR - 1 + a.coff, BC));
  // Blocks this wave has anything visible in (causal: keys up to its last query's limit).
  const int n_mine = CAUSAL ? min(n_kv, blocks_through(qw0 + 31 + a.coff, BC)) : n_kv;
  // Leading blocks visible to every query of this wave need no mask.
  const int n_plain = min(n_mine, CAUSAL ? min(blocks_within(qw0 + a.coff, BC), Nk / BC) : Nk / BC);

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = zero16();
  RowState rs{-INFINITY, 0, -INFINITY, -INFINITY, 0.f, 0.f, INFINITY, 0, 1.f};
  f32x16 s[KB];
  uint32_t pk[KB][8];
  // FP8: P^ of 64-key chunk c packed as one 8-register tuple (the MFMA's B operand): dwords 0-3
  // from 32-key sub-block 2 c, dwords 4-7 from sub-block 2 c + 1.
  i32x8 pk8[FP8 ? KB / 2 : 1];

  DirectStage<BC, D, kFwdThreads / 2> stg;  // group A's threads stage every tile
  // The FP8 instances are shorter of registers: they form the staging offsets at issue.
  if constexpr (FP8) stg.wave = __builtin_amdgcn_readfirstlane((tid & (kFwdThreads / 2 - 1)) >> 6);
  else stg.init(tid & (kFwdThreads / 2 - 1));
  // FP8 P^ V: the V block is D rows (one per head dimension) of 128 E4M3 bytes, staged like a
  // D x 64 tile of 16-bit elements.
  DirectStage<D, 64, kFwdThreads / 2> stg8;  // offsets formed at issue (no registers held)
  if constexpr (FP8) stg8.wave = __builtin_amdgcn_readfirstlane((tid & (kFwdThreads / 2 - 1)) >> 6);
  const uint16_t* V8g = FP8 ? reinterpret_cast<const uint16_t*>(a.v8 + (int64_t)bh * a.n_vblk * (D * 128)) : nullptr;
  const float* VSg = FP8 ? a.vscale + (int64_t)bh * a.n_vblk : nullptr;
  constexpr uint32_t kTileBytes = BC * D * 2;
  const uint32_t aK = lds_addr(&sK[0][0]), aV = lds_addr(&sV[0][0]);
  if (grp == 0) {
    if constexpr (FP8) stg.issue_lazy(Kg, 0, Nk, aK, lane);
    else stg.issue(Kg, 0, Nk, aK);
  }
  // Everyone waits here: the Q fragments above are then known complete, so no wait for them is
  // left inside the loop (where the tile loads would make it wait for those as well).
  wait_vm0();
  __syncthreads();

  float alpha_pending = 1.f;
  // The matrix phase is one straight-line stream of MFMA steps, each fenced: steps [0, NPV) add
  // V^T P^T of the previous block (d-tile by d-tile), steps [NPV, NPV + NSS) compute S^T of this
  // block.  The LDS operand of step k + MDEPTH is read at step k into a register ring; the
  // rescale of O by the previous block's alpha runs beside the MFMAs (d-tile 0 before the first
  // step, d-tile t + 1 during the steps of d-tile t; alpha == 1 leaves O unchanged).
  // FP8: a d-tile takes BC / 64 MFMAs of k = 64, each fed by two 16-byte reads (two steps: the
  // first only reads, the second reads and multiplies).
  constexpr int KK = FP8 ? 2 * (BC / 64) : BC / 16;
  constexpr int NPV = DT * KK, NSS = KB * KS;
  constexpr int MDEPTH = FP8 ? 2 : 4, MRING = MDEPTH + 1;
  e16x8 mring[MRING];
  // FP8 instances: step k's operand is half k & 1 of mring8[(k / 2) % 2], so the two 16-byte
  // reads of one k = 64 MFMA fill one 8-register tuple.  At step k the MFMA still uses step k - 1's
  // half while the read for step k + MDEPTH is issued: MDEPTH + 2 steps in flight, 4 positions.
  constexpr int R8 = 2;
  static_assert(!FP8 || 2 * R8 >= MDEPTH + 2, "ring positions must cover the steps in flight");
  i32x8 mring8[R8];
  auto ring_put = [&](auto kc, e16x8 x) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    if constexpr (FP8) {
      const i32x4 h = __builtin_bit_cast(i32x4, x);
      i32x8& slot = mring8[(k >> 1) % R8];
      if constexpr (k & 1)
        slot = __builtin_shufflevector(slot, __builtin_shufflevector(h, h, 0, 1, 2, 3, -1, -1, -1, -1), 0, 1, 2, 3, 8, 9, 10, 11);
      else
        slot = __builtin_shufflevector(slot, __builtin_shufflevector(h, h, 0, 1, 2, 3, -1, -1, -1, -1), 8, 9, 10, 11, 4, 5, 6, 7);
    } else {
      mring[k % MRING] = x;
    }
  };
  auto ring_get = [&](auto kc) __attribute__((always_inline)) -> e16x8 {
    constexpr int k = decltype(kc)::value;
    if constexpr (FP8) {
      const i32x8 slot = mring8[(k >> 1) % R8];
      if constexpr (k & 1)
        return __builtin_bit_cast(e16x8, __builtin_shufflevector(slot, slot, 4, 5, 6, 7));
      else
        return __builtin_bit_cast(e16x8, __builtin_shufflevector(slot, slot, 0, 1, 2, 3));
    } else {
      return mring[k % MRING];
    }
  };
  // Lane coordinates the operand reads use.  The FP8 instances re-derive them at the start of each
  // matrix phase from a value the compiler cannot see through, so the per-lane LDS addresses are
  // formed there and die with the phase instead of staying live (and spilling) across the loop.
  int mlane = lane, ml32 = l32, mhh = hh;
  auto m_read = [&](auto kc, const uint16_t* tV, const uint16_t* tK) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    const int lane = mlane, l32 = ml32, hh = mhh;
    if constexpr (k < NPV && FP8) {
      // Row 32 dt + l32 of the V block, bytes 64 ck + 32 hh + 16 part: the 32 keys of this lane
      // half, in the order P^ sits in its accumulator registers (v8_pack_kernel writes them so).
      constexpr int dt = k / KK, kk = k % KK, ck = kk >> 1, part = kk & 1;
      ring_put(kc, lds_read_row8<64>(tV, 32 * dt + l32, 32 * ck + 16 * hh + 8 * part));
    } else if constexpr (k < NPV) {
      constexpr int dt = k / KK, kk = k % KK;
      ring_put(kc, lds_read_col8_tr<D>(tV, 16 * kk, 32 * dt, lane));
    } else {
      constexpr int i = k - NPV, kb = i / KS, ks = i % KS;
      ring_put(kc, lds_read_row8<D>(tK, 32 * kb + l32, 16 * ks + 8 * hh));
    }
  };
  auto m_step = [&](auto kc) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    if constexpr (k < NPV && FP8) {
      constexpr int dt = k / KK, kk = k % KK, ck = kk >> 1;
      if constexpr (kk & 1) oacc[dt] = mfma32x32x64_fp8(mring8[(k >> 1) % R8], pk8[ck], oacc[dt]);
      if constexpr (dt + 1 < DT) {
        constexpr int per = 16 / KK;
#pragma unroll
        for (int r = per * kk; r < per * (kk + 1); ++r) oacc[dt + 1][r] *= alpha_pending;
      }
    } else if constexpr (k < NPV) {
      const e16x8 op = ring_get(kc);
      constexpr int dt = k / KK, kk = k % KK, o4 = (kk & 1) * 4;
      oacc[dt] = mfma32x32x16<E>(op, make_e16x8(pk[kk >> 1][o4], pk[kk >> 1][o4 + 1], pk[kk >> 1][o4 + 2],
                                              pk[kk >> 1][o4 + 3]), oacc[dt]);
      if constexpr (dt + 1 < DT) {
        constexpr int per = 16 / KK;
#pragma unroll
        for (int r = per * kk; r < per * (kk + 1); ++r) oacc[dt + 1][r] *= alpha_pending;
      }
    } else {
      const e16x8 op = ring_get(kc);
      constexpr int i = k - NPV, kb = i / KS, ks = i % KS;
      s[kb] = mfma32x32x16<E>(op, qf[ks], ks == 0 ? zero16() : s[kb]);
    }
  };
  auto m_stream = [&](auto k0c, auto k1c, const uint16_t* tV, const uint16_t* tK) __attribute__((always_inline)) {
    constexpr int K0 = decltype(k0c)::value, K1 = decltype(k1c)::value;
    __builtin_amdgcn_sched_barrier(0);
    static_for<K0, (K0 + MDEPTH < K1 ? K0 + MDEPTH : K1)>(
        [&](auto kc) __attribute__((always_inline)) { m_read(kc, tV, tK); });
    if constexpr (K0 == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[0][r] *= alpha_pending;
    }
    static_for<K0, K1>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (k + MDEPTH < K1) m_read(std::integral_constant<int, k + MDEPTH>{}, tV, tK);
      m_step(kc);
    });
    __builtin_amdgcn_sched_barrier(0);
  };
  using c0 = std::integral_constant<int, 0>;
  using cpv = std::integral_constant<int, NPV>;
  using cend = std::integral_constant<int, NPV + NSS>;

  // Matrix phase M(j): S^T of block j, then O = diag(alpha) O + V^T P^T for block j-1 (alpha and
  // P^ from vector phase j-1), at raised wave priority so the matrix cores are fed first when
  // both waves of a SIMD have work ready.  The two products are independent; taking S^T first
  // lets P^ and S^T share registers less (the compiler then needs no scratch in the mode-1
  // instance).  PAR = j & 1 is a compile-time constant at each call site, so the LDS buffer
  // addresses fold into instruction offsets.
  auto matrix_phase = [&](int j, auto par_tag) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_tag)::value;
    const uint16_t* tV = sV[PAR ^ 1];
    const uint16_t* tK = sK[PAR];
    const bool pv = j >= 1 && j - 1 < n_mine;
    const bool sc = j < n_mine;
    if constexpr (FP8) {
      mlane = lane;
      asm volatile("" : "+v"(mlane));
      ml32 = mlane & 31;
      mhh = mlane >> 5;
    }
    __builtin_amdgcn_s_setprio(1);
    if (sc) m_stream(cpv{}, cend{}, tV, tK);
    if (pv) m_stream(c0{}, cpv{}, tV, tK);
    __builtin_amdgcn_s_setprio(0);
  };

  // Vector phase V(j): online-softmax update for block j.
  auto vector_phase = [&](int j) __attribute__((always_inline)) {
    if (j >= n_mine) return;
    if (j >= n_plain) {
      // Element (kb, r) holds key kv0 + c + 4 hh, c = 32 kb + 8 (r / 4) + r % 4, with key indices
      // taken relative to coff (kv0 = block start - coff).  It is hidden past the last key or
      // (causal) past the lane's query, i.e. when c > lim: one compare per element against a
      // per-lane bound formed here, so nothing extra stays live across the loop.
      const int kv0 = j * BC - a.coff;
      const int lim = min(CAUSAL ? qrow - kv0 : INT_MAX, Nk - a.coff - 1 - kv0) - 4 * hh;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 32 * kb + 8 * (r >> 2) + (r & 3);
          s[kb][r] = (c > lim) ? -INFINITY : s[kb][r];
        }
    }
    if (STATS) {
      // Min over visible keys: hidden entries are exactly -inf, visible scores are finite.
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          rs.run_min = fminf(rs.run_min, s[kb][r] == -INFINITY ? INFINITY : s[kb][r]);
    }
    if constexpr (TOP2) {
      // Largest and second-largest score of the block counted with multiplicity (two chains,
      // merged), then of both halves, then with the running pair: the maximum repeats exactly
      // when the two are equal.  Max, min and med3 return one of their operands, so the
      // comparison is exact.
      float a1 = -INFINITY, a2 = -INFINITY, b1 = -INFINITY, b2 = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float x = s[kb][r], y = s[kb][r + 1];
          if (kb & 1) {
            b2 = fmaxf(b2, __builtin_amdgcn_fmed3f(b1, x, y));
            b1 = fmaxf(fmaxf(b1, x), y);
          } else {
            a2 = fmaxf(a2, __builtin_amdgcn_fmed3f(a1, x, y));
            a1 = fmaxf(fmaxf(a1, x), y);
          }
        }
      float m1 = fmaxf(a1, b1);
      float m2 = fmaxf(fminf(a1, b1), fmaxf(a2, b2));
      const auto p1 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, m1), __builtin_bit_cast(int, m1), false, false);
      const auto p2 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, m2), __builtin_bit_cast(int, m2), false, false);
      const float u1 = __builtin_bit_cast(float, (int)p1[0]), v1 = __builtin_bit_cast(float, (int)p1[1]);
      const float u2 = __builtin_bit_cast(float, (int)p2[0]), v2 = __builtin_bit_cast(float, (int)p2[1]);
      m1 = fmaxf(u1, v1);
      m2 = fmaxf(fminf(u1, v1), fmaxf(u2, v2));
      rs.run_m2 = fmaxf(fminf(rs.run_max, m1), fmaxf(rs.run_m2, m2));
      rs.run_max = fmaxf(rs.run_max, m1);
    } else {
    // Block max over both halves, and (when needed) how many visible keys attain it.
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[kb][r]);
    tmax = halves_max(tmax);
    const float new_max = fmaxf(rs.run_max, tmax);
    // The count can only change where the block reaches the running max; skip the whole count
    // when no lane of the wave does (the common case once the max has settled).
    if (COUNT && __any(tmax >= rs.run_max)) {
      int tcnt = 0;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tcnt += (s[kb][r] == tmax) ? 1 : 0;
      tcnt = halves_sum_i(tcnt);
      if (tmax == -INFINITY) tcnt = 0;
      rs.run_cnt = ((tmax == new_max) ? tcnt : 0) + ((rs.run_max == new_max) ? rs.run_cnt : 0);
    }
    rs.run_max = new_max;
    }
    // Shift for this block (log2 units).  The sign test is unchanged by the positive factor
    // scale * log2(e), and the rule is positively homogeneous, so applying it here equals
    // applying it to the natural-log scores.
    float m2_new = rs.run_max * a.sl2;
    if (MODE != 0) m2_new = exponent_shift<FP8>(page_shift<MODE, TOP2>(rs, a.sl2, a.beta), m2_new);
    const float alpha = fast_exp2(rs.m2 - m2_new);
    rs.m2 = m2_new;
    // The factor O is rescaled by.  FP8: O is held in units of this block's V scale over 2^8, so
    // it also takes the previous block's scale over this one's (block 0 starts from O = 0 and
    // rs.vs = 1); the row sum l takes alpha alone.
    float oscale = alpha;
    if constexpr (FP8) {
      const float vs = VSg[j];
      oscale = alpha * (rs.vs * __builtin_amdgcn_rcpf(vs));  // O's rescale need not be exact
      rs.vs = vs;
    }
    // FP8: P^ is formed as 2^8 P^ (exponent offset folded into the FMA) for its E4M3 rounding;
    // the row sum then carries the same factor, removed in the epilogue.
    const float m2_sub = FP8 ? m2_new - 8.f : m2_new;
    // P^ = exp2(S * scale * log2e - m), its row sum, and its 16-bit packing for the V product.
    float psum = 0.f;
    if constexpr (FP8) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          float p[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) p[u] = fast_exp2(fmaf(s[kb][r + u], a.sl2, -m2_sub));
          psum += (p[0] + p[1]) + (p[2] + p[3]);
          const uint32_t w = pack4_fp8(p[0], p[1], p[2], p[3]);
          pk8[kb >> 1][4 * (kb & 1) + (r >> 2)] = (int)w;
          if (STATS)
            rs.n_ones += ((w & 0xFFu) == kFp8OneX256) + (((w >> 8) & 0xFFu) == kFp8OneX256) +
                         (((w >> 16) & 0xFFu) == kFp8OneX256) + ((w >> 24) == kFp8OneX256);
        }
    } else {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(fmaf(s[kb][r], a.sl2, -m2_new));
        const float p1 = fast_exp2(fmaf(s[kb][r + 1], a.sl2, -m2_new));
        psum += p0 + p1;
        const uint32_t w = pack2<E>(p0, p1);
        pk[kb][r >> 1] = w;
        if (STATS) rs.n_ones += ((w & 0xFFFFu) == elem_one<E>()) + ((w >> 16) == elem_one<E>());
      }
    }
    if constexpr (KAHAN) {
      // Compensated running sum: the previous sum and its compensation scale by alpha together;
      // the low-order part lost in adding this block's sum is kept (negated) in lcomp.
      const float lprev = alpha * rs.lsum;
      const float y = psum - alpha * rs.lcomp;
      const float t = lprev + y;
      rs.lcomp = (t - lprev) - y;
      rs.lsum = t;
    } else {
      rs.lsum = alpha * rs.lsum + psum;
    }
    // O is rescaled by alpha in the next matrix phase, before this block is added.  The rescale
    // runs in every matrix phase: skipping it for a wave whose alphas are all 1 needs a second
    // copy of the P^V stream behind a branch, and with it the register allocator spills.
    alpha_pending = oscale;
  };

  // Both groups run the same sequence M(0) V(0) M(1) V(1) ... M(n_kv), each phase closed by a
  // workgroup barrier; group B passes one extra barrier first, so it runs one phase behind group
  // A (A's extra barrier at the end balances the count).  Group A alone stages the tiles: K_{j+1}
  // at the start of its M(j) (phase 2j; the buffer held K_{j-1}, last read by group B in phase
  // 2j-1) and V_j at the start of its V(j) (phase 2j+1; the buffer held V_{j-2}, last read in
  // phase 2j-1).  Splitting them keeps either phase from carrying all the load issue.  A waits
  // for both at the end of its V(j), before K_{j+1} and V_j are read in phase 2j+2.
  auto iteration = [&](int j, auto par_tag) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_tag)::value;
    if (grp == 0 && j + 1 < n_kv) {
      if constexpr (FP8) stg.issue_lazy(Kg, (j + 1) * BC, Nk, aK + (PAR ^ 1) * kTileBytes, lane);
      else stg.issue(Kg, (j + 1) * BC, Nk, aK + (PAR ^ 1) * kTileBytes);
    }
    // FP8: the V block is issued here too, so that forming its staging offsets stays out of the
    // vector phase (its buffer held V_{j-2}, last read in phase 2j - 1, as for the K buffer).
    if constexpr (FP8) {
      if (grp == 0 && j < n_kv) stg8.issue_lazy(V8g, j * D, a.n_vblk * D, aV + PAR * kTileBytes, lane);
    }
    matrix_phase(j, par_tag);
    __syncthreads();
    if constexpr (!FP8) {
      if (grp == 0 && j < n_kv) stg.issue(Vg, j * BC, Nk, aV + PAR * kTileBytes);
    }
    vector_phase(j);
    if (grp == 0) wait_vm0();
    __syncthreads();
  };
  using even = std::integral_constant<int, 0>;
  using odd = std::integral_constant<int, 1>;
  if (grp == 1) __syncthreads();
  int j = 0;
  for (; j + 1 <= n_kv; j += 2) {
    iteration(j, even{});
    iteration(j + 1, odd{});
  }
  if (j <= n_kv) iteration(j, even{});
  if (grp == 0) __syncthreads();

  // Epilogue: O = O^T / l, LSE = m + ln l, diagnostics.
  const float ltot = KAHAN ? halves_sum(rs.lsum - rs.lcomp) : halves_sum(rs.lsum);
  const float row_min = STATS ? halves_min(rs.run_min) : 0.f;
  const int ones_tot = STATS ? halves_sum_i(rs.n_ones) : 0;
  // A query that sees no key (no keys at all, or bottom-right alignment with more queries than
  // keys) has the empty sum: O = 0 and LSE = -inf.  Its lanes ran with an infinite max, so their
  // accumulators are not used.
  const bool empty = (Nk == 0) || (CAUSAL && qrow + a.coff < 0);
  // FP8: ltot is 2^8 l and O is held in units of vs / 2^8, so O = oacc vs / ltot.
  const float inv = empty ? 0.f : (FP8 ? rs.vs / ltot : 1.f / ltot);
  // O rows of this wave's 32 queries, through the tile buffers (waves 0-3 in the K buffers, 4-7 in
  // the V buffers): both groups have passed the last barrier, so no wave reads them any more, and
  // the last iterations issued no loads.
  store_rows_via_lds<E, D>(
      reinterpret_cast<uint8_t*>(wave < 4 ? &sK[0][0] : &sV[0][0]) + (wave & 3) * (64 * D), a.o + qoff + (int64_t)qw0 * D,
      Nq - qw0, lane, [&](int dt, int r) { return empty ? 0.f : oacc[dt][r] * inv; });
  if (qrow < Nq) {
    if (hh == 0) {
      const int64_t ri = (int64_t)bh * Nq + qrow;
      a.lse[ri] = empty ? -INFINITY : (rs.m2 + __log2f(ltot) - (FP8 ? 8.f : 0.f)) * kLn2;
      // The rule's shift after the last key block (natural-log units), recomputed from the final
      // running state exactly as the last vector phase formed it.
      if (a.mshift) a.mshift[ri] = empty ? -INFINITY : page_shift<MODE, TOP2>(rs, a.sl2, a.beta) * kLn2;
      if (STATS) {
        if (a.dupcnt) a.dupcnt[ri] = empty ? 0 : rs.run_cnt;
        if (a.ones) a.ones[ri] = empty ? 0 : ones_tot;
        if (a.smin) a.smin[ri] = empty ? INFINITY : row_min * a.scale;
        if (a.smax) a.smax[ri] = empty ? -INFINITY : rs.run_max * a.scale;
      }
    }
  }
}

template <int E, int D, bool CAUSAL, int MODE, bool STATS, bool KAHAN>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int grid = a.n_tiles * a.BH;
  hipLaunchKernelGGL((fwd_kernel<E, D, CAUSAL, MODE, STATS, KAHAN>), dim3(grid), dim3(kFwdThreads), 0, stream, a);
  return hipGetLastError();
}

template <int E, int D, bool CAUSAL, bool STATS, bool KAHAN>
static hipError_t launch_fwd_m(const FwdArgs& a, int mode, hipStream_t s) {
  if (mode == 0) return launch_fwd_t<E, D, CAUSAL, 0, STATS, KAHAN>(a, s);
  if (mode == 1) return launch_fwd_t<E, D, CAUSAL, 1, STATS, KAHAN>(a, s);
  return launch_fwd_t<E, D, CAUSAL, 2, STATS, KAHAN>(a, s);
}

template <int E, int D, bool CAUSAL>
static hipError_t launch_fwd_mode(const FwdArgs& a, int mode, bool stats, bool kahan, hipStream_t s) {
  if (stats)
    return kahan ? launch_fwd_m<E, D, CAUSAL, true, true>(a, mode, s) : launch_fwd_m<E, D, CAUSAL, true, false>(a, mode, s);
  return kahan ? launch_fwd_m<E, D, CAUSAL, false, true>(a, mode, s) : launch_fwd_m<E, D, CAUSAL, false, false>(a, mode, s);
}

#if FA_ELEM == 2
// V for the FP8 P^ V forward: one workgroup per (head, 128-key block).  The block's largest
// magnitude sets its scale s = amax / 448 (s = 1 for an all-zero block), and each value is stored
// as E4M3(v / s), round to nearest even.  Output per block: D rows (one per head dimension) of
// 128 bytes; byte 64 ck + 32 h + 4 sl + t of a row holds key 64 ck + 32 (sl / 4) + 8 (sl % 4) +
// 4 h + t of the block, which is the order in which the forward's P^ registers hold the keys of
// a 64-key chunk for lane half h (slot sl, byte t).  Keys past Nk are stored as 0.
template <int D>
__global__ __launch_bounds__(256) void v8_pack_kernel(const uint16_t* __restrict__ v, uint8_t* __restrict__ v8,
                                                      float* __restrict__ vscale, int Nk, int n_vblk) {
  constexpr int BK = 128;
  // Rows padded by 8 elements (16 bytes): the gather below reads 16 keys at one column, which a
  // 2D-byte stride would put in a single bank.
  constexpr int LD = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t sv[BK * LD];
  __shared__ float red[4];
  const int bh = blockIdx.x / n_vblk;
  const int jb = blockIdx.x - bh * n_vblk;
  const int tid = threadIdx.x;
  const int rows = min(BK, Nk - jb * BK);
  const uint16_t* src = v + ((int64_t)bh * Nk + (int64_t)jb * BK) * D;
  float amax = 0.f;
  for (int c = tid; c < BK * D / 8; c += 256) {
    i32x4 w = {0, 0, 0, 0};
    if (c / (D / 8) < rows) w = *reinterpret_cast<const i32x4*>(src + (int64_t)c * 8);
    *reinterpret_cast<i32x4*>(&sv[(c / (D / 8)) * LD + (c % (D / 8)) * 8]) = w;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const f32x2 f = unpack2<kElemBf16>((uint32_t)w[t]);
      amax = fmaxf(amax, fmaxf(fabsf(f[0]), fabsf(f[1])));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = amax > 0.f ? amax / 448.f : 1.f;
  const float inv = 1.f / sc;
  if (tid == 0) vscale[(int64_t)bh * n_vblk + jb] = sc;
  uint8_t* dst = v8 + ((int64_t)bh * n_vblk + jb) * (D * BK);
  for (int ch = tid; ch < D * 8; ch += 256) {
    const int d = ch >> 3, c = ch & 7;
    i32x4 out;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float x[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int pos = 16 * c + 4 * q4 + t;
        const int ck = pos >> 6, h = (pos >> 5) & 1, sl = (pos >> 2) & 7;
        const int key = 64 * ck + 32 * (sl >> 2) + 8 * (sl & 3) + 4 * h + t;
        x[t] = __builtin_bit_cast(float, (uint32_t)sv[key * LD + d] << 16) * inv;
      }
      out[q4] = (int)pack4_fp8(x[0], x[1], x[2], x[3]);
    }
    *reinterpret_cast<i32x4*>(dst + (int64_t)d * BK + 16 * c) = out;
  }
}

hipError_t launch_v8_pack(const uint16_t* v, uint8_t* v8, float* vscale, int BH, int Nk, int d, hipStream_t s) {
  const int n_vblk = (Nk + 127) / 128;
  if (BH == 0 || n_vblk == 0) return hipSuccess;
  const dim3 grid((unsigned)((int64_t)BH * n_vblk));
  if (d == 64)
    hipLaunchKernelGGL((v8_pack_kernel<64>), grid, dim3(256), 0, s, v, v8, vscale, Nk, n_vblk);
  else
    hipLaunchKernelGGL((v8_pack_kernel<128>), grid, dim3(256), 0, s, v, v8, vscale, Nk, n_vblk);
  return hipGetLastError();
}
#endif

#if FA_ELEM == 0
int fwd_kv_block(int d, bool causal) {
  if (d != 64 && d != 128) return 0;
  return causal ? fwd_bc<kElemBf16, true>() : fwd_bc<kElemBf16, false>();
}
int fwd_q_block(int d) { return (d == 64 || d == 128) ? kFwdBr : 0; }
#endif

template <int E>
hipError_t launch_fwd(FwdArgs a, int d, bool causal, int mode, bool stats, bool kahan, hipStream_t s) {
  a.n_tiles = (a.Nq + kFwdBr - 1) / kFwdBr;
  if (a.n_tiles == 0 || a.BH == 0) return hipSuccess;
  if (d == 64)
    return causal ? launch_fwd_mode<E, 64, true>(a, mode, stats, kahan, s)
                  : launch_fwd_mode<E, 64, false>(a, mode, stats, kahan, s);
  return causal ? launch_fwd_mode<E, 128, true>(a, mode, stats, kahan, s)
                : launch_fwd_mode<E, 128, false>(a, mode, stats, kahan, s);
}

template hipError_t launch_fwd<FA_ELEM>(FwdArgs, int, bool, int, bool, bool, hipStream_t);

}  // namespace fa
