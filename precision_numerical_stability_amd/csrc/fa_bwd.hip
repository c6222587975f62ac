// Backward kernels: delta = rowsum(dO o O), then dK/dV and dQ by recomputing P from the saved
// logsumexp.
//
// Follows the backward by recomputation of "FlashAttention 训练时为什么会梯度爆炸？一次拆透反向
// 传播的坑" (cnnetsun.cn/a/2497354) §2 -- keep no probability matrix, rebuild it from Q, K and the
// saved row statistics -- and the preprocessing term delta of the BF16 Flash Attention article
// (ijyty.com/news/896914) §3.1.  With S = scale Q K^T and P = exp(S - LSE):
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q.
// P does not depend on the forward's shift: LSE = m + ln l is the same for every shift.
//
// dK/dV and dQ run as two kernels with no atomics: each output tile is owned by exactly one
// workgroup, so results are deterministic.  All three run on the caller's stream in order.
//
// Tensors hold 16-bit elements (bf16 or fp16, the template parameter E; this file is compiled
// once per element type, FA_ELEM); P and dS are rounded to that type for their products, and
// every other step is fp32.
#include <type_traits>

#include <climits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

#ifndef FA_ELEM
#error "FA_ELEM (the element type this translation unit instantiates) must be defined"
#endif

namespace fa {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------------------------
// delta[row] = sum_c dO[row, c] * O[row, c], 16-bit inputs, fp32 arithmetic.  HBM-bound: one
// 16-byte load of O and of dO per thread, D / 8 threads per row.
template <int E, int D>
__global__ __launch_bounds__(kThreads) void delta_kernel(BwdArgs a) {
  constexpr int TPR = D / 8;
  constexpr int RPB = kThreads / TPR;
  const int tid = threadIdx.x;
  const int64_t total = (int64_t)a.BH * a.Nq;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;
  const int c = tid % TPR;
  float acc = 0.f;
  if (row < total) {
    const i32x4 ov = *reinterpret_cast<const i32x4*>(a.o + row * D + 8 * c);
    const i32x4 gv = *reinterpret_cast<const i32x4*>(a.dO + row * D + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 o2 = unpack2<E>((uint32_t)ov[i]);
      const f32x2 g2 = unpack2<E>((uint32_t)gv[i]);
      acc = fmaf(o2[0], g2[0], acc);
      acc = fmaf(o2[1], g2[1], acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (c == 0 && row < total) a.delta[row] = acc;
}

// ---------------------------------------------------------------------------------------------
// dQ at d = 64 (d = 128 runs dqw_kernel below): one workgroup per (128-query tile, head), 4 waves
// of 32 queries; loops over 64-key blocks.
// Lane layout as in the forward: S^T = K Q^T and dP^T = V dO^T put one query per lane, so LSE
// and delta are lane-local; dQ^T = K^T dS^T takes dS^T from the accumulator registers.  Within a
// block, the S/dP products of the second 32-key half are issued before the dS arithmetic of the
// first half and the dQ products follow, so matrix and vector work can overlap.  Blocks that need
// a mask (causal diagonal, ragged tail) run through the masked body after the main loop.
constexpr int kDqBc = 64;
constexpr int kDqBr = 128;

template <int E, int D>
__device__ __forceinline__ void dq_sdp(const uint16_t* tK, const uint16_t* tV, int kr, int l32, int hh,
                                       const e16x8 (&qf)[D / 16], const e16x8 (&gf)[D / 16], f32x16& s,
                                       f32x16& dp) {
  s = zero16();
  dp = zero16();
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const e16x8 kf = lds_read_row8<D>(tK, kr + l32, 16 * ks + 8 * hh);
    const e16x8 vf = lds_read_row8<D>(tV, kr + l32, 16 * ks + 8 * hh);
    s = mfma32x32x16<E>(kf, qf[ks], s);
    dp = mfma32x32x16<E>(vf, gf[ks], dp);
  }
}

template <int E, bool MASK, bool CAUSAL>
__device__ __forceinline__ void dq_grad(const f32x16& s, const f32x16& dp, int key0, int qrow, int nk, int hh,
                                        float sl2, float lse2, float dlt, uint32_t (&pds)[8]) {
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    float ds2[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int rr = r + u;
      float p = fast_exp2(fmaf(s[rr], sl2, -lse2));
      if (MASK) {
        // Key indices here are relative to the causal offset (key0 = block start - coff,
        // nk = Nk - coff).  Key key0 + c + 4 hh, c = 8 (rr / 4) + rr % 4, is hidden past the last
        // key or (causal) past the lane's query: c > lim.  The select also clears the infinite p
        // of a query that sees no key (LSE = -inf).
        const int lim = min(CAUSAL ? qrow - key0 - 4 * hh : INT_MAX, nk - 1 - key0 - 4 * hh);
        const int c = 8 * (rr >> 2) + (rr & 3);
        p = (c > lim) ? 0.f : p;
      }
      ds2[u] = p * (dp[rr] - dlt);
    }
    pds[r >> 1] = pack2<E>(ds2[0], ds2[1]);
  }
}

template <int E, int D>
__device__ __forceinline__ void dq_accum(const uint16_t* tK, int kr, int lane, const uint32_t (&pds)[8],
                                         f32x16 (&acc)[D / 32]) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const e16x8 db = make_e16x8(pds[4 * half], pds[4 * half + 1], pds[4 * half + 2], pds[4 * half + 3]);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const e16x8 kt = lds_read_col8_tr<D>(tK, kr + 16 * half, 32 * dt, lane);
      acc[dt] = mfma32x32x16<E>(kt, db, acc[dt]);
    }
  }
}

template <int E, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void dq_kernel(BwdArgs a) {
  constexpr int BC = kDqBc, BR = kDqBr, KS = D / 16, DT = D / 32;
  static_assert(BC == 64, "the block body handles two 32-key halves");
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
  const int Nq = a.Nq, Nk = a.Nk;
  const int q0 = qt * BR;
  const int64_t qoff = (int64_t)bh * Nq * D;
  const int64_t koff = (int64_t)bh * Nk * D;
  const uint16_t* Kg = a.k + koff;
  const uint16_t* Vg = a.v + koff;
  const int qrow = q0 + wave * 32 + l32;
  const int qsrc = min(qrow, Nq - 1);

  e16x8 qf[KS], gf[KS];
  {
    const uint16_t* qs = a.q + qoff + (int64_t)qsrc * D + 8 * hh;
    const uint16_t* gs = a.dO + qoff + (int64_t)qsrc * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = as_e16x8(*reinterpret_cast<const i32x4*>(qs + 16 * ks));
      gf[ks] = as_e16x8(*reinterpret_cast<const i32x4*>(gs + 16 * ks));
    }
  }
  const float lse2 = a.lse[(int64_t)bh * Nq + qsrc] * kLog2e;
  float dlt;
  if (a.fuse_delta) {
    // delta = sum_c dO[row, c] O[row, c] (fp32), formed here from the dO fragments already held
    // (this lane's half of the row) and the same half of O; the two halves of a row sit in lanes
    // l and l + 32.  Stored for the dK/dV kernel, which runs after this one.
    const uint16_t* os = a.o + qoff + (int64_t)qsrc * D + 8 * hh;
    float acc = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const i32x4 ov = *reinterpret_cast<const i32x4*>(os + 16 * ks);
      const i32x4 gv = __builtin_bit_cast(i32x4, gf[ks]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2 o2 = unpack2<E>((uint32_t)ov[i]);
        const f32x2 g2 = unpack2<E>((uint32_t)gv[i]);
        acc = fmaf(o2[0], g2[0], acc);
        acc = fmaf(o2[1], g2[1], acc);
      }
    }
    dlt = acc + __shfl_xor(acc, 32, 64);
    if (hh == 0 && qrow < Nq) a.delta[(int64_t)bh * Nq + qrow] = dlt;
  } else {
    dlt = a.delta[(int64_t)bh * Nq + qsrc];
  }

  int n_kv = (Nk + BC - 1) / BC;
  if (CAUSAL) n_kv = min(n_kv, blocks_through(q0 + BR - 1 + a.coff, BC));
  const int n_plain = min(n_kv, CAUSAL ? min(blocks_within(q0 + a.coff, BC), Nk / BC) : Nk / BC);

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();

  // Key block j lives in LDS buffer (j + p0) & 1 with p0 = n_plain & 1, so the masked blocks
  // after the plain loop always start in buffer 0.  Every step then knows its buffer at compile
  // time and the LDS addresses fold into instruction offsets.
  const int p0 = n_plain & 1;
  DirectStage<BC, D, kThreads> st;
  st.init(tid);
  constexpr uint32_t kTileBytes = BC * D * 2;
  const uint32_t aK = lds_addr(&sK[0][0]), aV = lds_addr(&sV[0][0]);
  st.issue(Kg, 0, Nk, aK + p0 * kTileBytes);
  st.issue(Vg, 0, Nk, aV + p0 * kTileBytes);
  wait_vm0();
  __syncthreads();

  int j = 0;
  auto step = [&](auto mask_tag, auto buf_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int buf = decltype(buf_tag)::value;
    const int kv0 = j * BC;
    if (j + 1 < n_kv) {
      st.issue(Kg, kv0 + BC, Nk, aK + (buf ^ 1) * kTileBytes);
      st.issue(Vg, kv0 + BC, Nk, aV + (buf ^ 1) * kTileBytes);
    }
    const uint16_t* tK = sK[buf];
    const uint16_t* tV = sV[buf];
    f32x16 s, dp;
    uint32_t pds0[8], pds1[8];
    f32x16 s1, dp1;
    __builtin_amdgcn_sched_barrier(0);
    dq_sdp<E, D>(tK, tV, 0, l32, hh, qf, gf, s, dp);
    sched_reads_ahead<2 * KS, 1, 4>();
    __builtin_amdgcn_sched_barrier(0);
    // dS of the first half on the vector ALUs while the second half's S/dP run on the matrix cores.
    dq_sdp<E, D>(tK, tV, 32, l32, hh, qf, gf, s1, dp1);
    dq_grad<E, MASK, CAUSAL>(s, dp, kv0 - a.coff, qrow, Nk - a.coff, hh, a.sl2, lse2, dlt, pds0);
    sched_reads_ahead_valu<2 * KS, 1, 4, 4>();
    __builtin_amdgcn_sched_barrier(0);
    dq_grad<E, MASK, CAUSAL>(s1, dp1, kv0 + 32 - a.coff, qrow, Nk - a.coff, hh, a.sl2, lse2, dlt, pds1);
    dq_accum<E, D>(tK, 0, lane, pds0, acc);
    sched_reads_ahead_valu<2 * DT, 2, 3, 8>();
    __builtin_amdgcn_sched_barrier(0);
    dq_accum<E, D>(tK, 32, lane, pds1, acc);
    sched_reads_ahead<2 * DT, 2, 3>();
    __builtin_amdgcn_sched_barrier(0);
    wait_vm0();
    __syncthreads();
    ++j;
  };
  using plain = std::integral_constant<bool, false>;
  using masked = std::integral_constant<bool, true>;
  using buf0 = std::integral_constant<int, 0>;
  using buf1 = std::integral_constant<int, 1>;
  if (p0) step(plain{}, buf1{});
  while (j < n_plain) {
    step(plain{}, buf0{});
    step(plain{}, buf1{});
  }
  while (j < n_kv) {
    step(masked{}, buf0{});
    if (j < n_kv) step(masked{}, buf1{});
  }

  // dQ rows of this wave's 32 queries, through the K buffers (the last step ended with a barrier
  // and issued no loads).
  const int qw0 = q0 + wave * 32;
  store_rows_via_lds<E, D>(reinterpret_cast<uint8_t*>(&sK[0][0]) + wave * (64 * D), a.dq + qoff + (int64_t)qw0 * D,
                           Nq - qw0, lane, [&](int dt, int r) { return acc[dt][r] * a.scale; });
}

// ---------------------------------------------------------------------------------------------
// dQ at d = 128: one workgroup per (256-query tile, head), 4 waves of 64 queries, one wave per
// SIMD.  A wave's queries form two 32-query halves, and every K or V operand it reads from LDS
// feeds the MFMAs of both halves: half the LDS operand bytes per MFMA of a 32-query wave.  The Q
// and dO fragments (B operands of S^T and dP^T, 128 registers) and the dQ^T accumulators (128)
// fill the accumulation registers; S/dP tiles, packed dS and the operand ring use the others.
//
// Keys come in 64-key blocks of two 32-key sub-blocks, staged in three LDS buffers.  The work is
// one software pipeline over the 32-key sub-blocks u of the key range: unit u issues the S/dP
// products of u + 1, runs the dS arithmetic of u beside them, and the dQ products of u - 1, so no
// MFMA waits on vector work finished just before it.  The iteration over key block j runs units
// 2j - 1 and 2j: its S/dP products read block j, its dQ products block j - 1, while block j + 1
// loads into the third buffer.  In the first iteration, units -1 and -2 run on neutral data (an
// infinite LSE makes their dS zero, and the K buffer they read is zeroed); the last block's
// remaining dS and dQ work drains after the loop.
//
// The S^T and dP^T products are VGPR-form inline-asm MFMAs (mfma32x32x16_vgpr), for which the
// compiler inserts no wait states.  Their results are read at least a few MFMAs later, and their
// B operands, the Q and dO fragments, are moved to the accumulation registers once, before the
// first iteration, so that no vector write of an operand lands just before such an MFMA.
constexpr int kDqwBc = 64;
constexpr int kDqwBr = 256;
constexpr int kDqwBuf = 3;
constexpr int kDqwIssueStep = 3;  // MFMA step of an iteration after which the next block's loads issue

template <int D>
struct DqwSched {
  static constexpr int KS = D / 16, DT = D / 32;
  static constexpr int USTEP = 6 * KS;     // MFMA steps per unit: KS groups of 6
  static constexpr int NSTEP = 2 * USTEP;  // per iteration
  static constexpr int NPAIR = NSTEP / 2;  // operand reads per iteration, one per two MFMAs
  static_assert(KS == 2 * DT, "each group of a unit carries one dQ operand");
  // Step k of an iteration: unit k / USTEP; within it group g = (k % USTEP) / 6 and slot
  // w = k % 6, of kind w / 2 (0: dQ^T += K^T dS^T, 1: S^T = K Q^T, 2: dP^T = V dO^T) for query
  // half w % 2.  The operand of steps 2p and 2p + 1 is read once (pair p).  Element e (0..31) of
  // a unit's dS arithmetic runs after step pos(uu, e) of that unit; -1 places it before the
  // unit's first step (in unit 0, beside the operand reads that start the iteration).
  static constexpr int pos(int uu, int e) { return e * USTEP / 32 - (uu == 0 ? 1 : 0); }
};

// LDS byte addresses of this lane's operand reads, relative to the first K or V buffer: rows
// (16-byte reads of row l % 32 at k-slice g) of K and of V, and the two halves of a transposed
// read of K at d-tile dt.  Every read adds a compile-time buffer and row offset, which folds into
// the instruction.  Each iteration passes the patterns through an empty asm statement, so the
// compiler keeps one copy of each instead of hoisting a sum per buffer out of the loop.
template <int D>
struct DqwAddr {
  uint32_t rk[D / 16], rv[D / 16], tk[D / 32][2];
  __device__ __forceinline__ void init(uint32_t base_k, uint32_t base_v, int lane) {
    const int l32 = lane & 31, hh = lane >> 5, s = lane & 15;
#pragma unroll
    for (int g = 0; g < D / 16; ++g) {
      const uint32_t off = 2u * (uint32_t)lds_off<D>(l32, 16 * g + 8 * hh);
      rk[g] = base_k + off;
      rv[g] = base_v + off;
    }
    const int r1 = 4 * hh + (s >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int col = 32 * dt + (((lane >> 4) & 1) << 4) + ((s & 3) << 2);
      tk[dt][0] = base_k + 2u * (uint32_t)lds_off<D>(r1, col);
      tk[dt][1] = base_k + 2u * (uint32_t)lds_off<D>(r1 + 8, col);
    }
  }
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int g = 0; g < D / 16; ++g) asm volatile("" : "+v"(rk[g]), "+v"(rv[g]));
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) asm volatile("" : "+v"(tk[dt][0]), "+v"(tk[dt][1]));
  }
};

__device__ __forceinline__ e16x8 lds_ld128(uint32_t a) {
  return as_e16x8(*reinterpret_cast<const __attribute__((address_space(3))) i32x4*>((uintptr_t)a));
}
// Transposed operand read (see lds_read_col8_tr) from the two half addresses.
__device__ __forceinline__ e16x8 lds_ld_tr(uint32_t a0, uint32_t a1) {
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((uintptr_t)a0));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((uintptr_t)a1));
  i32x2 x = __builtin_bit_cast(i32x2, lo);
  i32x2 y = __builtin_bit_cast(i32x2, hi);
  return make_e16x8((uint32_t)x[0], (uint32_t)x[1], (uint32_t)y[0], (uint32_t)y[1]);
}

template <int D>
struct DqwState {
  f32x16 s[2][2], dp[2][2];  // [set][query half]: S^T and dP^T of sub-block u live in set u & 1
  uint32_t pds[2][2][8];     // packed dS^T, [set][query half][pair of keys]
  f32x16 acc[2][D / 32];     // dQ^T, [query half][d-tile]
  e16x8 qf[2][D / 16], gf[2][D / 16];
};

// Element arithmetic of one unit's sub-block (set c): P = exp2(S scale log2e - LSE log2e),
// dS = P (dP - delta), pairs packed to the element type.  Masked: key key0 + cc + 4h (cc = 8 (r / 4)
// + r % 4, relative to the causal offset) is hidden from the half's query when cc > lim.
template <int E, int D, bool MASK, int C, int A, int R>
__device__ __forceinline__ void dqw_elem(DqwState<D>& st, float sl2, float L, float dl, int lim, float& tmp) {
  float p = fast_exp2(fmaf(st.s[C][A][R], sl2, -L));
  if (MASK) {
    constexpr int cc = 8 * (R >> 2) + (R & 3);
    p = (cc > lim) ? 0.f : p;
  }
  const float ds = p * (st.dp[C][A][R] - dl);
  if constexpr ((R & 1) == 0) tmp = ds;
  else st.pds[C][A][R >> 1] = pack2<E>(tmp, ds);
}

template <bool CAUSAL>
__device__ __forceinline__ int dqw_lim(int qrow, int key0, int nk, int hh) {
  return min(CAUSAL ? qrow - key0 - 4 * hh : INT_MAX, nk - 1 - key0 - 4 * hh);
}

// One iteration (key block j; kv0 = 64 j - coff, nk = Nk - coff): the buffer B holds block j,
// buffer (B + 2) % 3 block j - 1; issue() sends block j + 1's loads to the third buffer.  lse:
// LSE log2e of the two query halves for unit 2j; lsep the same for unit 2j - 1 (infinite in the
// first iteration).
template <int E, int D, bool CAUSAL, bool MASK, int B, typename Issue>
__device__ __forceinline__ void dqw_iter(DqwAddr<D>& ad, int kv0, int nk, const int (&qrow)[2], int lane, float sl2,
                                         const float (&lse)[2], const float (&lsep)[2], const float (&dlt)[2],
                                         DqwState<D>& st, Issue&& issue) {
  using S = DqwSched<D>;
  constexpr int DT = D / 32;
  constexpr int DP = 4;       // pairs read ahead
  constexpr int RING = DP + 1;
  constexpr uint32_t TILE = kDqwBc * D * 2;
  constexpr uint32_t OFF = B * TILE, OFFP = ((B + 2) % kDqwBuf) * TILE;  // block j, block j - 1
  const int hh = lane >> 5;
  ad.opaque();
  e16x8 ring[RING];
  int lim[2][2] = {{INT_MAX, INT_MAX}, {INT_MAX, INT_MAX}};  // [unit][query half]
  if (MASK) {
#pragma unroll
    for (int uu = 0; uu < 2; ++uu)
#pragma unroll
      for (int h = 0; h < 2; ++h) lim[uu][h] = dqw_lim<CAUSAL>(qrow[h], kv0 - 32 + 32 * uu, nk, hh);
  }
  float tmp = 0.f;

  auto read_pair = [&](auto pc) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value;
    constexpr int k = 2 * p, uu = k / S::USTEP, kk = k % S::USTEP, g = kk / 6, kind = (kk % 6) / 2;
    if constexpr (kind == 0) {
      constexpr int kh = g / DT, dt = g % DT;
      constexpr uint32_t o = OFFP + (32 * uu + 16 * kh) * 2 * D;
      ring[p % RING] = lds_ld_tr(ad.tk[dt][0] + o, ad.tk[dt][1] + o);
    } else {
      constexpr uint32_t o = OFF + 32 * uu * 2 * D;
      ring[p % RING] = lds_ld128((kind == 1 ? ad.rk[g] : ad.rv[g]) + o);
    }
  };
  auto mfma_step = [&](auto kc) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    constexpr int uu = k / S::USTEP, kk = k % S::USTEP, g = kk / 6, w = kk % 6, kind = w / 2, h = w % 2;
    const e16x8 op = ring[(k / 2) % RING];
    if constexpr (kind == 0) {
      constexpr int kh = g / DT, dt = g % DT, o = 4 * kh;
      st.acc[h][dt] = mfma32x32x16<E>(
          op, make_e16x8(st.pds[uu][h][o], st.pds[uu][h][o + 1], st.pds[uu][h][o + 2], st.pds[uu][h][o + 3]),
          st.acc[h][dt]);
    } else if constexpr (kind == 1) {
      st.s[uu][h] = mfma32x32x16_vgpr<E, g == 0>(op, st.qf[h][g], st.s[uu][h]);
    } else {
      st.dp[uu][h] = mfma32x32x16_vgpr<E, g == 0>(op, st.gf[h][g], st.dp[uu][h]);
    }
  };
  // Elements of unit uu at position kk: the sub-block in set 1 - uu.
  auto elems_at = [&](auto uc, auto kc) __attribute__((always_inline)) {
    constexpr int uu = decltype(uc)::value, kk = decltype(kc)::value;
    static_for<0, 32>([&](auto ec) __attribute__((always_inline)) {
      constexpr int e = decltype(ec)::value;
      if constexpr (S::pos(uu, e) == kk) {
        constexpr int h = e / 16, r = e % 16;
        dqw_elem<E, D, MASK, 1 - uu, h, r>(st, sl2, uu == 0 ? lsep[h] : lse[h], dlt[h], lim[uu][h], tmp);
      }
    });
  };

  __builtin_amdgcn_sched_barrier(0);
  static_for<0, DP>([&](auto pc) __attribute__((always_inline)) { read_pair(pc); });
  // The first elements read S/dP of the previous iteration's last MFMAs, issued as inline asm, for
  // which the compiler inserts no wait states: wait them out here (once per iteration).
  asm volatile("s_nop 7\n\ts_nop 3");
  __builtin_amdgcn_sched_barrier(0);
  elems_at(std::integral_constant<int, 0>{}, std::integral_constant<int, -1>{});
  static_for<0, S::NSTEP>([&](auto kc) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    constexpr int uu = k / S::USTEP, kk = k % S::USTEP;
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (k % 2 == 0 && k / 2 + DP < S::NPAIR) read_pair(std::integral_constant<int, k / 2 + DP>{});
    mfma_step(kc);
    // The next block's tile loads go out once the stream is running, so that the first MFMAs do
    // not wait behind their issue.
    if constexpr (k == kDqwIssueStep) issue();
    elems_at(std::integral_constant<int, uu>{}, std::integral_constant<int, kk>{});
    if constexpr (uu == 0 && kk == S::USTEP - 1)
      elems_at(std::integral_constant<int, 1>{}, std::integral_constant<int, -1>{});
  });
  __builtin_amdgcn_sched_barrier(0);
}

// After the last key block (at byte offset offl from the first K buffer; key0 = its second
// sub-block's first key - coff): the dS
// arithmetic of that sub-block beside the dQ products of the first, then the dQ products of the
// second.
template <int E, int D, bool CAUSAL>
__device__ __forceinline__ void dqw_drain(const DqwAddr<D>& ad, uint32_t offl, int key0, int nk, const int (&qrow)[2],
                                          int lane, float sl2, const float (&lse)[2], const float (&dlt)[2],
                                          DqwState<D>& st) {
  constexpr int DT = D / 32;
  constexpr int NP = 4 * DT;  // operand reads: 2 DT per sub-block
  const int hh = lane >> 5;
  const int lim[2] = {dqw_lim<CAUSAL>(qrow[0], key0, nk, hh), dqw_lim<CAUSAL>(qrow[1], key0, nk, hh)};
  float tmp = 0.f;
  e16x8 ring[NP];
  __builtin_amdgcn_sched_barrier(0);
  static_for<0, NP>([&](auto pc) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value;
    constexpr int sb = p / (2 * DT), kh = (p % (2 * DT)) / DT, dt = p % DT;
    const uint32_t o = offl + (32 * sb + 16 * kh) * 2 * D;
    ring[p] = lds_ld_tr(ad.tk[dt][0] + o, ad.tk[dt][1] + o);
  });
  asm volatile("s_nop 7\n\ts_nop 3");  // as at the start of an iteration
  __builtin_amdgcn_sched_barrier(0);
  static_for<0, 2 * NP>([&](auto kc) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    constexpr int p = k / 2, h = k % 2, sb = p / (2 * DT), kh = (p % (2 * DT)) / DT, dt = p % DT, o = 4 * kh;
    __builtin_amdgcn_sched_barrier(0);
    st.acc[h][dt] = mfma32x32x16<E>(
        ring[p], make_e16x8(st.pds[sb][h][o], st.pds[sb][h][o + 1], st.pds[sb][h][o + 2], st.pds[sb][h][o + 3]),
        st.acc[h][dt]);
    if constexpr (sb == 0) {
      static_for<0, 2>([&](auto ic) __attribute__((always_inline)) {
        constexpr int e = 2 * k + decltype(ic)::value;
        dqw_elem<E, D, true, 1, e / 16, e % 16>(st, sl2, lse[e / 16], dlt[e / 16], lim[e / 16], tmp);
      });
    }
  });
  __builtin_amdgcn_sched_barrier(0);
}

template <int E, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void dqw_kernel(BwdArgs a) {
  constexpr int BC = kDqwBc, BR = kDqwBr, KS = D / 16, DT = D / 32;
  constexpr int NB = kDqwBuf;
  __shared__ __attribute__((aligned(16))) uint16_t sK[NB][BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[NB][BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;

  int bh, rank;
  map_block(blockIdx.x, a.BH, a.n_tiles, bh, rank);
  const int qt = CAUSAL ? a.n_tiles - 1 - rank : rank;
  const int Nq = a.Nq, Nk = a.Nk;
  const int q0 = qt * BR;
  const int64_t qoff = (int64_t)bh * Nq * D;
  const int64_t koff = (int64_t)bh * Nk * D;
  const uint16_t* Kg = a.k + koff;
  const uint16_t* Vg = a.v + koff;
  const int qw0 = q0 + wave * 64;

  DqwState<D> st;
  int qrow[2];
  float lse[2], dlt[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    qrow[h] = qw0 + 32 * h + (lane & 31);
    const int qsrc = min(qrow[h], Nq - 1);
    const uint16_t* qs = a.q + qoff + (int64_t)qsrc * D + 8 * hh;
    const uint16_t* gs = a.dO + qoff + (int64_t)qsrc * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      st.qf[h][ks] = as_e16x8(*reinterpret_cast<const i32x4*>(qs + 16 * ks));
      st.gf[h][ks] = as_e16x8(*reinterpret_cast<const i32x4*>(gs + 16 * ks));
    }
    lse[h] = a.lse[(int64_t)bh * Nq + qsrc] * kLog2e;
    if (a.fuse_delta) {
      // delta = sum_c dO[row, c] O[row, c] (fp32) from this lane's half of the row (the other half
      // sits in lane l ^ 32), stored for the dK/dV kernel, which runs after this one.
      const uint16_t* os = a.o + qoff + (int64_t)qsrc * D + 8 * hh;
      float acc = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const i32x4 ov = *reinterpret_cast<const i32x4*>(os + 16 * ks);
        const i32x4 gv = __builtin_bit_cast(i32x4, st.gf[h][ks]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x2 o2 = unpack2<E>((uint32_t)ov[i]);
          const f32x2 g2 = unpack2<E>((uint32_t)gv[i]);
          acc = fmaf(o2[0], g2[0], acc);
          acc = fmaf(o2[1], g2[1], acc);
        }
      }
      dlt[h] = acc + __shfl_xor(acc, 32, 64);
      if (hh == 0 && qrow[h] < Nq) a.delta[(int64_t)bh * Nq + qrow[h]] = dlt[h];
    } else {
      dlt[h] = a.delta[(int64_t)bh * Nq + qsrc];
    }
  }

  // The fragments are only ever the B operand of the inline-asm MFMAs, which take it from
  // accumulation registers.  Moving them there once, here, keeps the compiler from writing them
  // just before such an MFMA, which it does not know must wait for the write.
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+a"(st.qf[h][ks]), "+a"(st.gf[h][ks]));

  int n_kv = (Nk + BC - 1) / BC;
  if (CAUSAL) n_kv = min(n_kv, blocks_through(q0 + BR - 1 + a.coff, BC));
  const int n_plain = min(n_kv, CAUSAL ? min(blocks_within(q0 + a.coff, BC), Nk / BC) : Nk / BC);

#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.acc[h][dt] = zero16();
    st.s[1][h] = zero16();
    st.dp[1][h] = zero16();
#pragma unroll
    for (int i = 0; i < 8; ++i) st.pds[0][h][i] = 0u;
  }

  // Block j lives in buffer (j + p0) % 4, p0 chosen so that the unrolled plain loop starts in
  // buffer 0 after the n_plain % 4 leading plain iterations; the masked iterations then start in
  // buffer 0 as well, and every iteration knows its buffers at compile time.
  const int rem = n_plain % NB;
  const int p0 = (NB - rem) % NB;
  DirectStage<BC, D, kThreads> stg;
  stg.init(tid);
  constexpr uint32_t kTileBytes = BC * D * 2;
  const uint32_t aK = lds_addr(&sK[0][0]), aV = lds_addr(&sV[0][0]);
  DqwAddr<D> ad;
  ad.init(aK, aV, lane);
  {
    // The K buffer of block -1, read by the first iteration's neutral dQ products.
    i32x4* z = reinterpret_cast<i32x4*>(&sK[(p0 + NB - 1) % NB][0]);
#pragma unroll
    for (int i = 0; i < BC * D * 2 / 16 / kThreads; ++i) z[i * kThreads + tid] = i32x4{0, 0, 0, 0};
  }
  if (n_kv > 0) {
    stg.issue(Kg, 0, Nk, aK + p0 * kTileBytes);
    stg.issue(Vg, 0, Nk, aV + p0 * kTileBytes);
  }
  wait_vm0();
  __syncthreads();

  float lsep[2] = {__builtin_inff(), __builtin_inff()};
  int j = 0;
  auto iter = [&](auto mask_tag, auto buf_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int B = decltype(buf_tag)::value;
    dqw_iter<E, D, CAUSAL, MASK, B>(ad, j * BC - a.coff, Nk - a.coff, qrow, lane, a.sl2, lse, lsep, dlt, st,
                                    [&]() __attribute__((always_inline)) {
                                      if (j + 1 < n_kv) {
                                        stg.issue(Kg, (j + 1) * BC, Nk, aK + ((B + 1) % NB) * kTileBytes);
                                        stg.issue(Vg, (j + 1) * BC, Nk, aV + ((B + 1) % NB) * kTileBytes);
                                      }
                                    });
    wait_vm0();
    __syncthreads();
    lsep[0] = lse[0];
    lsep[1] = lse[1];
    ++j;
  };
  using plain = std::integral_constant<bool, false>;
  using masked = std::integral_constant<bool, true>;
  using buf0 = std::integral_constant<int, 0>;
  using buf1 = std::integral_constant<int, 1>;
  using buf2 = std::integral_constant<int, 2>;
  if (rem >= 2) iter(plain{}, buf1{});
  if (rem >= 1) iter(plain{}, buf2{});
  while (j < n_plain) {
    iter(plain{}, buf0{});
    iter(plain{}, buf1{});
    iter(plain{}, buf2{});
  }
  while (j < n_kv) {
    iter(masked{}, buf0{});
    if (j < n_kv) iter(masked{}, buf1{});
    if (j < n_kv) iter(masked{}, buf2{});
  }
  if (n_kv > 0) {
    dqw_drain<E, D, CAUSAL>(ad, ((n_kv - 1 + p0) % NB) * kTileBytes, (n_kv - 1) * BC + 32 - a.coff, Nk - a.coff, qrow,
                            lane, a.sl2, lse, dlt, st);
    __syncthreads();  // the drain's reads of the K buffer are done before it becomes the stage area
  }

  // dQ rows of this wave's 64 queries, 32 at a time through a stage area in the K buffers.
#pragma unroll
  for (int h = 0; h < 2; ++h)
    store_rows_via_lds<E, D>(reinterpret_cast<uint8_t*>(&sK[0][0]) + wave * (64 * D),
                             a.dq + qoff + (int64_t)(qw0 + 32 * h) * D, Nq - (qw0 + 32 * h), lane,
                             [&](int dt, int r) { return st.acc[h][dt][r] * a.scale; });
}

// ---------------------------------------------------------------------------------------------
// dK/dV: one workgroup per (128-key tile, head), 4 waves of 32 keys; loops over 128-query blocks.
// S = Q K^T and dP = dO V^T put one key per lane (K and V stay in registers as B operands);
// dV^T = dO^T P and dK^T = Q^T dS take P and dS from the accumulator registers, with dO^T and
// Q^T read transposed from LDS.  The per-query LSE and delta come from LDS as 4-float vectors.
//
// A block is processed as four 32-query sub-blocks in one straight-line software pipeline: the
// S/dP products of sub-block t+1 are issued before the softmax-gradient arithmetic of sub-block t,
// so the matrix cores work on the next sub-block while the vector ALUs finish the current one.
//
// Registers: dK and dV accumulate in AGPRs (builtin MFMAs), S and dP are produced in VGPRs
// (VGPR-form MFMAs, mfma32x32x16_vgpr) so the gradient arithmetic reads them with no copy out of
// the accumulation registers, and the K/V fragments, used only as the B operand of those MFMAs,
// sit in AGPRs.  The gradient arithmetic reads S/dP of a sub-block whose products were issued at
// least one 16-step phase earlier, well past the MFMA's result hazard.
constexpr int kDkvBq = 128;
constexpr int kDkvBk = 128;

template <int D>
struct DkvFrags {
  e16x8 k[D / 16];
  e16x8 v[D / 16];
};

// The block's MFMA stream, in time order, is 2 SB phases of L steps (L = 2 D/16 = 4 D/32):
//   phase 0          S/dP of sub-block 0
//   phase 2t + 1     S/dP of sub-block t + 1          (t = 0 .. SB - 2)
//   phase 2t + 2     dV/dK of sub-block t             (t = 0 .. SB - 2)
//   phase 2 SB - 1   dV/dK of sub-block SB - 1
// An S/dP step is one MFMA (k-slice ks = i of S for i < D/16, then k-slice i - D/16 of dP) with
// one 16-byte operand read; the first dP step starts from -delta of the sub-block's queries (read
// from LDS as a 16-register tile at the phase's first step), so dP - delta comes out of the
// MFMAs; a dV/dK step is one MFMA (half i / (2 D/32), d-tile (i / 2) % (D/32), dV
// when i is even, dK when odd) with one transposed operand read.  The softmax-gradient arithmetic
// of half g of the block (sub-block g / 2, query rows 16 (g % 2) .. + 15 of it; 8 elements per lane)
// runs element by element beside the MFMAs: halves 0 and 1 in phase 1, half g in phase g after
// that.  Phase g reads the S/dP results of a phase that finished earlier, and the dV/dK steps of a
// half only start after its elements are packed (half 2 SB - 1 runs in the first half of the last
// phase, whose second half consumes it).
template <int D>
struct DkvSched {
  static constexpr int SB = kDkvBq / 32;
  static constexpr int L = 2 * (D / 16);
  static_assert(L == 4 * (D / 32), "S/dP and dV/dK phases have the same length");
  static constexpr int NSTEP = 2 * SB * L;
  static constexpr int phase(int k) { return k / L; }
  static constexpr bool is_sdp(int k) { return phase(k) == 0 || (phase(k) % 2 == 1 && phase(k) < 2 * SB - 1); }
  static constexpr int sub(int k) {  // sub-block the step works on
    const int p = phase(k);
    if (p == 0) return 0;
    if (p == 2 * SB - 1) return SB - 1;
    return (p % 2 == 1) ? (p + 1) / 2 : (p - 2) / 2;
  }
  // Gradient elements that run after step k's MFMA: count and the first element's flat index
  // m = 8 g + e (g = half, e = element within it).
  static constexpr int n_elem(int k) {
    const int p = phase(k), j = k % L;
    if (p == 0) return 0;
    if (p == 1) return 16 / L;
    if (p == 2 * SB - 1) return (j < L / 2) ? 16 / L : 0;
    if (p % 2 == 1) return (L == 16) ? ((j % 2 == 0) ? 1 : 0) : 1;
    return (L == 16) ? ((j % 2 == 1) ? 1 : 0) : 1;
  }
  static constexpr int first_elem(int k) {
    const int p = phase(k), j = k % L;
    if (p == 1) return j * (16 / L);
    if (p == 2 * SB - 1) return 8 * p + j * (16 / L);
    if (p % 2 == 1) return 8 * p + ((L == 16) ? j / 2 : j);
    return 8 * p + ((L == 16) ? (j - 1) / 2 : j);
  }
  // Halves whose LSE vectors are read from LDS at step k: returns a bit mask over g.  Half
  // g + 1 is read at the start of phase g, a whole phase ahead of its use (its register slot's
  // previous half, g - 1, finished in phase g - 1), except in phase 1, which runs halves 0 and 1:
  // there half 2 is read once half 0, which still uses that slot, is done (step L / 2).
  static constexpr int ld_halves(int k) {
    const int p = phase(k), j = k % L;
    if (j != (p == 1 ? L / 2 : 0) || p + 1 >= 2 * SB) return 0;
    return (p == 0) ? 0x3 : (1 << (p + 1));
  }
};

// One 128-query block: dV^T += dO^T P and dK^T += Q^T dS for this wave's 32 keys, with
// S = Q K^T and dP = dO V^T recomputed per 32-query sub-block.  Operand reads run DEPTH steps
// ahead of their MFMA through a ring of registers; every step is fenced so the order above is the
// order the instructions issue in.
template <int E, int D, bool CAUSAL, bool MASK>
__device__ __forceinline__ void dkdv_block(const uint16_t* tQ, const uint16_t* tG, const float* tL,
                                           const float* tD, int q0, int Nq, int coff, int key, int lane, float sl2,
                                           const DkvFrags<D>& f, f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32]) {
  using S = DkvSched<D>;
  constexpr int DT = D / 32;
  constexpr int DEPTH = 6;
  constexpr int RING = DEPTH + 1;  // step k's operand stays put while step k + DEPTH's is read
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  f32x16 s[2], dp[2];
  uint32_t pp[2][8], pd[2][8];
  e16x8 ring[RING];
  float4 lsl[2][2];  // [half slot][row group] LSE (log2 units)
  f32x16 nd;         // -delta tile of the sub-block whose S/dP phase runs
  float pt0 = 0.f, dt0 = 0.f;   // first element of the pair being packed

  auto read_op = [&](auto kc) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    constexpr int t = S::sub(k), i = k % S::L;
    if constexpr (S::is_sdp(k)) {
      constexpr bool is_dp = i >= D / 16;
      constexpr int ks = is_dp ? i - D / 16 : i;
      ring[k % RING] = lds_read_row8<D>(is_dp ? tG : tQ, 32 * t + l32, 16 * ks + 8 * hh);
    } else {
      constexpr int half = i / (2 * DT), dt = (i >> 1) % DT;
      ring[k % RING] = lds_read_col8_tr<D>((i & 1) ? tQ : tG, 32 * t + 16 * half, 32 * dt, lane);
    }
  };
  auto read_ld = [&](auto gc) __attribute__((always_inline)) {
    constexpr int g = decltype(gc)::value;
    constexpr int t = g >> 1, h = g & 1;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int qi = 32 * t + 8 * (2 * h + w) + 4 * hh;
      lsl[g & 1][w] = *reinterpret_cast<const float4*>(&tL[qi]);
    }
  };
  // -delta of sub-block t's queries in the accumulator layout (register r: query 32 t + 8 (r / 4)
  // + 4 h + r % 4), the C operand of its first dP MFMA.
  auto read_nd = [&](auto tc) __attribute__((always_inline)) {
    constexpr int t = decltype(tc)::value;
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const float4 v = *reinterpret_cast<const float4*>(&tD[32 * t + 8 * rq + 4 * hh]);
      nd[4 * rq] = v.x;
      nd[4 * rq + 1] = v.y;
      nd[4 * rq + 2] = v.z;
      nd[4 * rq + 3] = v.w;
    }
  };
  auto mfma_step = [&](auto kc) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    constexpr int t = S::sub(k), i = k % S::L, c = t & 1;
    const e16x8 op = ring[k % RING];
    if constexpr (S::is_sdp(k)) {
      constexpr bool is_dp = i >= D / 16;
      constexpr int ks = is_dp ? i - D / 16 : i;
      if constexpr (!is_dp) {
        s[c] = mfma32x32x16_vgpr<E, ks == 0>(op, f.k[ks], s[c]);
      } else if constexpr (ks == 0) {
        dp[c] = mfma32x32x16_vgpr_from<E>(op, f.v[0], nd);
      } else {
        dp[c] = mfma32x32x16_vgpr<E, false>(op, f.v[ks], dp[c]);
      }
    } else {
      constexpr int half = i / (2 * DT), dt = (i >> 1) % DT, o4 = 4 * half;
      if constexpr ((i & 1) == 0) {
        dv[dt] = mfma32x32x16<E>(op, make_e16x8(pp[c][o4], pp[c][o4 + 1], pp[c][o4 + 2], pp[c][o4 + 3]), dv[dt]);
      } else {
        dk[dt] = mfma32x32x16<E>(op, make_e16x8(pd[c][o4], pd[c][o4 + 1], pd[c][o4 + 2], pd[c][o4 + 3]), dk[dt]);
      }
    }
  };
  // Element e of half g: P = exp2(S scale log2e - LSE log2e), dS = P (dP - delta), masked queries
  // (past Nq, or, when causal, before key - coff, the first query that sees this lane's key)
  // give zero; pairs are packed to the element type.
  auto grad_elem = [&](auto mc) __attribute__((always_inline)) {
    constexpr int m = decltype(mc)::value;
    constexpr int g = m >> 3, e = m & 7;
    constexpr int t = g >> 1, h = g & 1, c = t & 1;
    constexpr int w = e >> 2, rq = 2 * h + w, u = e & 3, r = 4 * rq + u;
    const float4 l4 = lsl[g & 1][w];
    const float lv = u == 0 ? l4.x : u == 1 ? l4.y : u == 2 ? l4.z : l4.w;
    float p = fast_exp2(fmaf(s[c][r], sl2, -lv));
    if (MASK) {
      // Query q0 + c + 4 hh, c = 32 t + 8 rq + u, is hidden past Nq or (causal) before
      // key - coff: c > hi or c < lo.  The select also clears the infinite p of a query that sees
      // no key.
      const int hi = Nq - 1 - q0 - 4 * hh;
      const int lo = CAUSAL ? key - (q0 + coff) - 4 * hh : INT_MIN;
      constexpr int c = 32 * t + 8 * rq + u;
      p = (c > hi || c < lo) ? 0.f : p;
    }
    const float ds = p * dp[c][r];  // dP - delta
    if constexpr ((u & 1) == 0) {
      pt0 = p;
      dt0 = ds;
    } else {
      pp[c][2 * rq + (u >> 1)] = pack2<E>(pt0, p);
      pd[c][2 * rq + (u >> 1)] = pack2<E>(dt0, ds);
    }
  };

  __builtin_amdgcn_sched_barrier(0);
  static_for<0, DEPTH>([&](auto kc) __attribute__((always_inline)) { read_op(kc); });
  static_for<0, S::NSTEP>([&](auto kc) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (k + DEPTH < S::NSTEP) read_op(std::integral_constant<int, k + DEPTH>{});
    if constexpr (S::is_sdp(k) && k % S::L == 0) read_nd(std::integral_constant<int, S::sub(k)>{});
    constexpr int ldm = S::ld_halves(k);
    static_for<0, 2 * S::SB>([&](auto gc) __attribute__((always_inline)) {
      if constexpr ((ldm >> decltype(gc)::value) & 1) read_ld(gc);
    });
    mfma_step(kc);
    constexpr int m0 = S::first_elem(k), ne = S::n_elem(k);
    static_for<m0, m0 + ne>([&](auto mc) __attribute__((always_inline)) { grad_elem(mc); });
  });
  __builtin_amdgcn_sched_barrier(0);
}

template <int E, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void dkdv_kernel(BwdArgs a) {
  constexpr int BQ = kDkvBq, BK = kDkvBk, KS = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2][BQ * D];
  __shared__ __attribute__((aligned(16))) uint16_t sG[2][BQ * D];
  __shared__ __attribute__((aligned(16))) float sL[2][BQ];
  __shared__ __attribute__((aligned(16))) float sD[2][BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  int bh, rank;
  map_block(blockIdx.x, a.BH, a.n_tiles, bh, rank);
  const int kt = rank;  // causal: the first key tiles see the most queries, so they start first
  const int Nq = a.Nq, Nk = a.Nk;
  const int k0 = kt * BK;
  const int64_t qoff = (int64_t)bh * Nq * D;
  const int64_t koff = (int64_t)bh * Nk * D;
  const int64_t roff = (int64_t)bh * Nq;
  const uint16_t* Qg = a.q + qoff;
  const uint16_t* Gg = a.dO + qoff;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + l32;
  const int ksrc = min(key, Nk - 1);

  DkvFrags<D> f;
  {
    const uint16_t* ks_ = a.k + koff + (int64_t)ksrc * D + 8 * hh;
    const uint16_t* vs_ = a.v + koff + (int64_t)ksrc * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      f.k[ks] = as_e16x8(*reinterpret_cast<const i32x4*>(ks_ + 16 * ks));
      f.v[ks] = as_e16x8(*reinterpret_cast<const i32x4*>(vs_ + 16 * ks));
    }
  }

  // Query blocks visited: i_first .. n_q - 1 (causal: from the block of the first query that
  // sees key k0).  Causal blocks before i_lead hold queries that do not see every key of the
  // tile (those before k0 + BK - 1 - coff) and need the mask.
  const int n_q = (Nq + BQ - 1) / BQ;
  const int i_first = CAUSAL ? max(0, k0 - a.coff) / BQ : 0;
  const int i_lead = CAUSAL ? min(n_q, blocks_through(k0 + BK - 2 - a.coff, BQ)) : 0;

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk[dt] = zero16();
    dv[dt] = zero16();
  }

  DirectStage<BQ, D, kThreads> st;
  st.init(tid);
  constexpr uint32_t kTileBytes = BQ * D * 2;
  const uint32_t aQ = lds_addr(&sQ[0][0]), aG = lds_addr(&sG[0][0]);
  float vl = 0.f, vd = 0.f;
  auto load_rows = [&](int i) __attribute__((always_inline)) {
    if (tid < BQ) {
      const int64_t src = roff + min(i * BQ + tid, Nq - 1);
      vl = a.lse[src];  // scaled when stored: no arithmetic here, so nothing waits for the load
      vd = a.delta[src];
    }
  };
  auto store_rows = [&](int b) __attribute__((always_inline)) {
    if (tid < BQ) {
      sL[b][tid] = vl * kLog2e;
      sD[b][tid] = -vd;  // the dP products start from -delta
    }
  };

  // The masked blocks (the causal leading ones, one or two of them, and a ragged last block) run
  // through the masked body outside the main loop, so the loop body has a single variant and
  // the accumulators need no copies at branch joins.
  //
  // Query block i lives in LDS buffer (i - i_first + b0) & 1.  b0 is chosen so that the unmasked
  // loop starts in buffer 0: that loop is unrolled by two, so each of its steps knows its buffer
  // at compile time and the LDS addresses fold into instruction offsets (with a run-time buffer
  // every operand read needs its address rebuilt).  The masked steps, at most three per
  // workgroup, index the buffers at run time.
  const int n_full = Nq / BQ;  // blocks lying entirely inside the sequence
  // Leading masked blocks: at most two, since their 127 query rows span at most two 128-row blocks.
  const int n_lead = CAUSAL ? min(2, max(0, i_lead - i_first)) : 0;
  int i = i_first;
  int buf = n_lead & 1;
  auto step = [&](auto mask_tag, auto buf_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int b = buf_tag;  // a constant in the unmasked loop, a run-time value in masked steps
    const int q0 = i * BQ;
    const bool has_next = (i + 1 < n_q);
    if (has_next) {
      st.issue(Qg, q0 + BQ, Nq, aQ + (b ^ 1) * kTileBytes);
      st.issue(Gg, q0 + BQ, Nq, aG + (b ^ 1) * kTileBytes);
      load_rows(i + 1);
    }
    dkdv_block<E, D, CAUSAL, MASK>(sQ[b], sG[b], sL[b], sD[b], q0, Nq, a.coff, key, lane, a.sl2, f, dk, dv);
    if (has_next) store_rows(b ^ 1);
    wait_vm0();
    __syncthreads();
    ++i;
    buf = b ^ 1;
  };
  using masked = std::integral_constant<bool, true>;
  using plain = std::integral_constant<bool, false>;
  using buf0 = std::integral_constant<int, 0>;
  using buf1 = std::integral_constant<int, 1>;

  if (i < n_q) {
    st.issue(Qg, i * BQ, Nq, aQ + buf * kTileBytes);
    st.issue(Gg, i * BQ, Nq, aG + buf * kTileBytes);
    load_rows(i);
    store_rows(buf);
  }
  wait_vm0();
  __syncthreads();
  if (CAUSAL && i < i_lead) step(masked{}, buf);
  if (CAUSAL && i < i_lead) step(masked{}, buf);
  // buf == 0 here (n_lead steps from b0 = n_lead & 1).
  while (i + 1 < n_full) {
    step(plain{}, buf0{});
    step(plain{}, buf1{});
  }
  if (i < n_full) step(plain{}, buf0{});
  if (i < n_q) step(masked{}, buf);

  // dK and dV rows of this wave's 32 keys, through the Q and dO buffers (no wave reads them any
  // more: the last step ended with a barrier and issued no loads).
  const int rows_left = Nk - kw0;
  store_rows_via_lds<E, D>(reinterpret_cast<uint8_t*>(&sQ[0][0]) + wave * (64 * D), a.dk + koff + (int64_t)kw0 * D,
                           rows_left, lane, [&](int dt, int r) { return dk[dt][r] * a.scale; });
  store_rows_via_lds<E, D>(reinterpret_cast<uint8_t*>(&sG[0][0]) + wave * (64 * D), a.dv + koff + (int64_t)kw0 * D,
                           rows_left, lane, [&](int dt, int r) { return dv[dt][r]; });
}

// ---------------------------------------------------------------------------------------------
template <int E>
hipError_t launch_bwd_delta(BwdArgs a, int d, hipStream_t s) {
  const int64_t total = (int64_t)a.BH * a.Nq;
  if (total == 0) return hipSuccess;
  const int rpb = kThreads / (d / 8);
  const int64_t grid = (total + rpb - 1) / rpb;
  if (d == 64)
    hipLaunchKernelGGL((delta_kernel<E, 64>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((delta_kernel<E, 128>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int E>
hipError_t launch_bwd_dq(BwdArgs a, int d, bool causal, hipStream_t s) {
  a.n_tiles = (a.Nq + (d == 64 ? kDqBr : kDqwBr) - 1) / (d == 64 ? kDqBr : kDqwBr);
  if (a.n_tiles == 0 || a.BH == 0) return hipSuccess;
  const dim3 grid(a.n_tiles * a.BH);
  if (d == 64) {
    if (causal) hipLaunchKernelGGL((dq_kernel<E, 64, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((dq_kernel<E, 64, false>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (causal) hipLaunchKernelGGL((dqw_kernel<E, 128, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((dqw_kernel<E, 128, false>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <int E>
hipError_t launch_bwd_dkdv(BwdArgs a, int d, bool causal, hipStream_t s) {
  a.n_tiles = (a.Nk + kDkvBk - 1) / kDkvBk;
  if (a.n_tiles == 0 || a.BH == 0) return hipSuccess;
  const dim3 grid(a.n_tiles * a.BH);
  if (d == 64) {
    if (causal) hipLaunchKernelGGL((dkdv_kernel<E, 64, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((dkdv_kernel<E, 64, false>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (causal) hipLaunchKernelGGL((dkdv_kernel<E, 128, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((dkdv_kernel<E, 128, false>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

template hipError_t launch_bwd_delta<FA_ELEM>(BwdArgs, int, hipStream_t);
template hipError_t launch_bwd_dq<FA_ELEM>(BwdArgs, int, bool, hipStream_t);
template hipError_t launch_bwd_dkdv<FA_ELEM>(BwdArgs, int, bool, hipStream_t);

}  // namespace fa
