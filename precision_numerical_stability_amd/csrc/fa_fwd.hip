// Forward kernel: tiled Q K^T, online safe softmax with running max and sum, optional stabilised
// shift for repeated maxima, P^ V accumulation, final normalisation and the saved logsumexp.
//
// Follows the online softmax of the BF16 Flash Attention article (ijyty.com/news/896914) §2.1 and
// the repeated-maximum shift of its §4.1, with the precision schedule of "Flash Attention低精度
// 训练稳定性优化实践" (jsqmd.com/news/761560) §3.2: Q K^T accumulated in fp32, softmax in fp32,
// P^ rounded to bf16 for the product with V.
//
// Work split: one workgroup of 4 waves per (query tile of 128 rows, head).  Each wave owns 32
// queries and computes S^T = K Q^T, so each lane owns one query column: its row max, repeat count
// and row sum are lane-local up to one exchange between the two 32-lane halves.  K and V tiles
// of 64 keys are staged through swizzled, double-buffered LDS; Q stays in registers.  O^T is
// accumulated as V^T P^T so that the per-query rescale factor is lane-local too, and P^ goes from
// the accumulator registers straight into the next MFMA's operand without touching LDS.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

constexpr int kFwdBc = 64;   // keys per step
constexpr int kFwdBr = 128;  // queries per workgroup
constexpr int kFwdThreads = 256;

template <int D, bool CAUSAL, int MODE, bool STATS>
__global__ __launch_bounds__(kFwdThreads, 2) void fwd_kernel(FwdArgs a) {
  constexpr int BC = kFwdBc, BR = kFwdBr, KS = D / 16, DT = D / 32, KB = BC / 32;
  constexpr bool COUNT = (MODE == 1) || STATS;
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  int bh, rank;
  map_block(blockIdx.x, a.BH, a.n_tiles, bh, rank);
  const int qt = CAUSAL ? a.n_tiles - 1 - rank : rank;
  const int N = a.N;
  const int q0 = qt * BR;
  const int64_t hoff = (int64_t)bh * N * D;
  const uint16_t* Qg = a.q + hoff;
  const uint16_t* Kg = a.k + hoff;
  const uint16_t* Vg = a.v + hoff;

  const int qrow = q0 + wave * 32 + l32;  // this lane's query

  // Q^T as the B operand: lane holds Q[qrow][16 ks + 8 hh .. + 7].
  bf16x8 qf[KS];
  {
    const uint16_t* src = Qg + (int64_t)min(qrow, N - 1) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8(*reinterpret_cast<const i32x4*>(src + 16 * ks));
  }

  int n_kv = (N + BC - 1) / BC;
  if (CAUSAL) n_kv = min(n_kv, (q0 + BR - 1) / BC + 1);

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = zero16();
  float run_max = -INFINITY;  // running max of the raw dot products q.k
  int run_cnt = 0;            // how many visible keys attain it
  float m2 = -INFINITY;       // current shift, in log2 units of the scaled score
  float lsum = 0.f;           // this half's share of the row sum
  int n_ones = 0;

  DirectStage<BC, D, kFwdThreads> st;
  st.init(tid);
  st.issue(Kg, 0, N, sK[0]);
  st.issue(Vg, 0, N, sV[0]);
  wait_vm0();
  __syncthreads();

  // Leading blocks visible to every query of the tile need no mask; the rest (causal diagonal,
  // ragged tail) run through the masked body after the main loop, so the loop body has a single
  // variant.
  const int n_plain = min(n_kv, CAUSAL ? q0 / BC : N / BC);
  int j = 0;
  auto step = [&](auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int buf = j & 1;
    const int kv0 = j * BC;
    if (j + 1 < n_kv) {
      st.issue(Kg, kv0 + BC, N, sK[buf ^ 1]);
      st.issue(Vg, kv0 + BC, N, sV[buf ^ 1]);
    }
    const uint16_t* tK = sK[buf];
    const uint16_t* tV = sV[buf];
    // S^T block kb: rows = keys kv0 + 32 kb + (8 (r/4) + 4 hh + r%4), column = this lane's query.
    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 kf = lds_read_row8<D>(tK, 32 * kb + l32, 16 * ks + 8 * hh);
        s[kb] = mfma32x32x16(kf, qf[ks], s[kb]);
      }
    }
    if (MASK) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool hide = (key >= N) || (CAUSAL && key > qrow);
          s[kb][r] = hide ? -INFINITY : s[kb][r];
        }
    }
    // Block max over both halves, and (when needed) how many visible keys attain it.
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[kb][r]);
    tmax = halves_max(tmax);
    const float new_max = fmaxf(run_max, tmax);
    // The count can only change where the block reaches the running max; skip the whole count
    // when no lane of the wave does (the common case once the max has settled).
    if (COUNT && __any(tmax >= run_max)) {
      int tcnt = 0;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tcnt += (s[kb][r] == tmax) ? 1 : 0;
      tcnt = halves_sum_i(tcnt);
      if (tmax == -INFINITY) tcnt = 0;
      run_cnt = ((tmax == new_max) ? tcnt : 0) + ((run_max == new_max) ? run_cnt : 0);
    }
    run_max = new_max;
    // Shift for this block (log2 units).  The sign test is unchanged by the positive factor
    // scale * log2(e), and the rule is positively homogeneous, so applying it here equals
    // applying it to the natural-log scores.
    const float r2 = run_max * a.sl2;
    float m2_new = r2;
    if (MODE != 0) {
      const bool rep = (MODE == 2) || (run_cnt > 1);
      m2_new = (rep && r2 > 0.f) ? a.beta * r2 : ((rep && r2 < 0.f) ? 0.f : r2);
    }
    const float alpha = fast_exp2(m2 - m2_new);
    m2 = m2_new;
    // P^ = exp2(S * scale * log2e - m), its row sum, and its bf16 packing for the V product.
    uint32_t pk[KB][8];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(fmaf(s[kb][r], a.sl2, -m2_new));
        const float p1 = fast_exp2(fmaf(s[kb][r + 1], a.sl2, -m2_new));
        psum += p0 + p1;
        const uint32_t w = pack_bf16x2(p0, p1);
        pk[kb][r >> 1] = w;
        if (STATS) n_ones += ((w & 0xFFFFu) == kBf16One) + ((w >> 16) == kBf16One);
      }
    lsum = alpha * lsum + psum;
    // Rescale O only if some lane's shift moved (alpha == 1 exactly leaves O unchanged).
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
    // O^T += V^T P^T over 16-key slabs.
#pragma unroll
    for (int kk = 0; kk < BC / 16; ++kk) {
      const int kb = kk >> 1;
      const int o4 = (kk & 1) * 4;
      const bf16x8 pb = make_bf16x8(pk[kb][o4], pk[kb][o4 + 1], pk[kb][o4 + 2], pk[kb][o4 + 3]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 vf = lds_read_col8_tr<D>(tV, 16 * kk, 32 * dt, lane);
        oacc[dt] = mfma32x32x16(vf, pb, oacc[dt]);
      }
    }
    wait_vm0();
    __syncthreads();
    ++j;
  };
  while (j < n_plain) step(std::integral_constant<bool, false>{});
  while (j < n_kv) step(std::integral_constant<bool, true>{});

  // Epilogue: O = O^T / l, LSE = m + ln l, diagnostics.
  const float ltot = halves_sum(lsum);
  const int ones_tot = STATS ? halves_sum_i(n_ones) : 0;
  if (qrow < N) {
    const float inv = 1.f / ltot;
    uint16_t* orow = a.o + hoff + (int64_t)qrow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * dt + 8 * rr + 4 * hh;
        i32x2 w;
        w[0] = (int)pack_bf16x2(oacc[dt][4 * rr] * inv, oacc[dt][4 * rr + 1] * inv);
        w[1] = (int)pack_bf16x2(oacc[dt][4 * rr + 2] * inv, oacc[dt][4 * rr + 3] * inv);
        *reinterpret_cast<i32x2*>(orow + d0) = w;
      }
    if (hh == 0) {
      const int64_t ri = (int64_t)bh * N + qrow;
      a.lse[ri] = (m2 + __log2f(ltot)) * kLn2;
      if (STATS) {
        if (a.dupcnt) a.dupcnt[ri] = run_cnt;
        if (a.ones) a.ones[ri] = ones_tot;
      }
    }
  }
}

template <int D, bool CAUSAL, int MODE, bool STATS>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int grid = a.n_tiles * a.BH;
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, MODE, STATS>), dim3(grid), dim3(kFwdThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_mode(const FwdArgs& a, int mode, bool stats, hipStream_t s) {
  if (stats) {
    if (mode == 0) return launch_fwd_t<D, CAUSAL, 0, true>(a, s);
    if (mode == 1) return launch_fwd_t<D, CAUSAL, 1, true>(a, s);
    return launch_fwd_t<D, CAUSAL, 2, true>(a, s);
  }
  if (mode == 0) return launch_fwd_t<D, CAUSAL, 0, false>(a, s);
  if (mode == 1) return launch_fwd_t<D, CAUSAL, 1, false>(a, s);
  return launch_fwd_t<D, CAUSAL, 2, false>(a, s);
}

int fwd_kv_block(int d) { return (d == 64 || d == 128) ? kFwdBc : 0; }
int fwd_q_block(int d) { return (d == 64 || d == 128) ? kFwdBr : 0; }

hipError_t launch_fwd(FwdArgs a, int d, bool causal, int mode, bool stats, hipStream_t s) {
  a.n_tiles = (a.N + kFwdBr - 1) / kFwdBr;
  if (d == 64) return causal ? launch_fwd_mode<64, true>(a, mode, stats, s) : launch_fwd_mode<64, false>(a, mode, stats, s);
  return causal ? launch_fwd_mode<128, true>(a, mode, stats, s) : launch_fwd_mode<128, false>(a, mode, stats, s);
}

}  // namespace fa
