// Device primitives for the gfx950 attention kernels: MFMA wrappers and fp32 -> 16-bit packing for
// the two element types (bf16, fp16), swizzled LDS tiles, the LDS transpose read, and half-wave
// reductions.
//
// Register layouts (v_mfma_f32_32x32x16_bf16 and _f16 alike, one wave of 64 lanes, h = lane / 32):
//   A operand (32 x 16):  lane l holds A[l % 32][8h .. 8h + 7]
//   B operand (16 x 32):  lane l holds B[8h .. 8h + 7][l % 32]
//   C/D (32 x 32 fp32):   lane l, register r holds C[8 (r / 4) + 4 h + (r % 4)][l % 32]
// Only the pairing of A's and B's k-slots matters for a product, so an operand may carry its k
// values in any order as long as the other operand uses the same order.  The kernels use this to
// feed the C layout of one product straight into the B operand of the next: within each 16-wide
// k slab, slot t of half h holds index 4h + t (t < 4) or 8 + 4h + (t - 4) (t >= 4), which is what
// C registers 8s .. 8s + 7 of slab s hold.
//
// ds_read_b64_tr_b16: within each group of 16 lanes, lane s supplies the address of 4 consecutive
// 16-bit elements (row s / 4, columns 4 (s % 4) .. + 3 of a 4 x 16 block) and lane o receives
// column o of that block, rows 0..3.  This yields 4 consecutive k values of one output column,
// i.e. the transposed operand, from a row-major tile.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

namespace fa {

// Eight 16-bit elements: one MFMA operand per lane.  The storage is typed bf16; with fp16 elements
// the same bits are reinterpreted at the MFMA.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 e16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element type of q, k, v, o, dO and the gradients, and of the 16-bit operands the products take
// (P^ and dS are rounded to it too).  Arithmetic is fp32 for both.
constexpr int kElemBf16 = 0;
constexpr int kElemF16 = 1;
// bf16 tensors, with the P^ V product of the forward in FP8 (OCP E4M3): P^ rounded as
// e4m3(2^8 P^), V pre-rounded per 128-key block with a dynamic scale (v8_pack_kernel).  Every
// other product and every stored tensor is bf16, so the bf16 paths below serve it unchanged.
constexpr int kElemFp8PV = 2;

// Bit pattern of 1.0 in the element type.
template <int E>
constexpr uint16_t elem_one() { return E == kElemF16 ? 0x3C00 : 0x3F80; }

// C += A B, 32 x 32 x 16, fp32 accumulation, operands of element type E.
template <int E>
__device__ __forceinline__ f32x16 mfma32x32x16(e16x8 a, e16x8 b, f32x16 c) {
  if constexpr (E == kElemF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
}

// v_mfma_f32_32x32x16_{bf16,f16} in the VGPR form with the B operand read from AGPRs: the result
// (and the accumulator it continues) lives in VGPRs, where vector instructions can read it
// directly, while a loop-invariant B operand occupies accumulation registers instead.  The
// compiler's builtin picks one form for every MFMA of a kernel (the AGPR form, once a kernel needs
// more than 256 registers), so a kernel that wants both forms issues this one as inline assembly.
// ZERO: the accumulator input is the constant 0; the destination is then early-clobber, since a
// multi-pass MFMA must not write registers it is still reading A or B from.  The compiler still
// tracks the asm operands for waits on loads and for wait states after the MFMA; a vector read of
// the result must come later in the instruction stream than the hazard distance of a 32x32 MFMA.
template <int E, bool ZERO>
__device__ __forceinline__ f32x16 mfma32x32x16_vgpr(e16x8 a, e16x8 b_acc, f32x16 c) {
  f32x16 d;
  if constexpr (E == kElemF16) {
    if constexpr (ZERO) asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b_acc));
    else asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "a"(b_acc), "0"(c));
  } else {
    if constexpr (ZERO) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b_acc));
    else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=v"(d) : "v"(a), "a"(b_acc), "0"(c));
  }
  return d;
}

// As mfma32x32x16_vgpr, accumulating onto c into a distinct destination: c stays live (the
// destination is early-clobber, so it overlaps none of the inputs).
template <int E>
__device__ __forceinline__ f32x16 mfma32x32x16_vgpr_from(e16x8 a, e16x8 b_acc, f32x16 c) {
  f32x16 d;
  if constexpr (E == kElemF16) asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b_acc), "v"(c));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b_acc), "v"(c));
  return d;
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

// C += A B, 32 x 32 x 64, fp32 accumulation, E4M3 operands (32 bytes per lane: lanes 0-31 and
// 32-63 each hold one half of the k range).  A and B pair up by (lane half, byte slot), so the
// kernels may place the k values in any order that both operands share.  Unit block scales.
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Four fp32 -> four E4M3 bytes (round to nearest even), byte t = value t.
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
constexpr uint32_t kFp8OneX256 = 0x78;  // E4M3 encoding of 256 = 2^8 x 1.0

// Two fp32 -> a packed pair of the element type (round to nearest even; fp16 overflows to inf),
// low half = a.
template <int E>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (E == kElemF16) {
    f16x2 r = __builtin_convertvector((f32x2){a, b}, f16x2);
    return __builtin_bit_cast(uint32_t, r);
  } else {
    bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
  }
}

// The two elements of a packed pair as fp32 (exact): low half, high half.
template <int E>
__device__ __forceinline__ f32x2 unpack2(uint32_t w) {
  if constexpr (E == kElemF16) {
    return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
  } else {
    return (f32x2){__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xFFFF0000u)};
  }
}

__device__ __forceinline__ e16x8 as_e16x8(i32x4 v) { return __builtin_bit_cast(e16x8, v); }

__device__ __forceinline__ e16x8 make_e16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  i32x4 v = {(int)a, (int)b, (int)c, (int)d};
  return __builtin_bit_cast(e16x8, v);
}

// Reductions over the two 32-lane halves of a wave: lane l and lane l ^ 32 both receive the
// combined value.  v_permlane32_swap exchanges the first operand of the upper half with the
// second operand of the lower half, so applied to (x, x) each lane ends up holding both its own
// and its partner's x, in an order that differs by half; max and + are symmetric in it.
__device__ __forceinline__ float halves_max(float x) {
  int xi = __builtin_bit_cast(int, x);
  auto s = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return fmaxf(__builtin_bit_cast(float, (int)s[0]), __builtin_bit_cast(float, (int)s[1]));
}
__device__ __forceinline__ float halves_min(float x) {
  int xi = __builtin_bit_cast(int, x);
  auto s = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return fminf(__builtin_bit_cast(float, (int)s[0]), __builtin_bit_cast(float, (int)s[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  int xi = __builtin_bit_cast(int, x);
  auto s = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __builtin_bit_cast(float, (int)s[0]) + __builtin_bit_cast(float, (int)s[1]);
}
__device__ __forceinline__ int halves_sum_i(int x) {
  auto s = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (int)s[0] + (int)s[1];
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------------------------
// Swizzled row-major [rows][D] tiles of 16-bit elements in LDS.  The 16-byte chunk c of row r is stored at
// chunk c ^ f(r), with f an XOR-linear map of the low four bits r0..r3 of the row:
//   d = 128 (16 chunks per row):  f = 4 r0 ^ 10 r1 ^ 1 r2 ^ 8 r3
//   d = 64  ( 8 chunks per row):  f = 2 r0 ^  4 r1 ^ 1 r2 ^ 2 r3
// The two access patterns are 16-byte operand reads (lanes = consecutive rows at one logical
// chunk) and transpose reads (16-lane groups = 4 consecutive rows at an aligned chunk pair, the
// two groups of a half-wave side by side).  These maps were chosen by exhaustive search over
// XOR-linear maps so that both patterns are free of bank conflicts whether the LDS serves
// 128 bytes per cycle (32 banks: 8 / 16 lanes per cycle) or 256 bytes (64 banks: 16 / 32 lanes);
// the counters on gfx950 rule out a 32-bank-only design (a map conflict-free only for 32 banks
// doubled the measured conflict cycles).
template <int D>
__device__ __forceinline__ int swz(int row) {
  const int r0 = row & 1, r1 = (row >> 1) & 1, r2 = (row >> 2) & 1, r3 = (row >> 3) & 1;
  if constexpr (D == 128) {
    return (r0 << 2) ^ (r1 * 10) ^ r2 ^ (r3 << 3);
  } else {
    return (r0 << 1) ^ (r1 << 2) ^ r2 ^ (r3 << 1);
  }
}

// Element offset of (row, col) in a swizzled [rows][D] tile.
template <int D>
__device__ __forceinline__ int lds_off(int row, int col) {
  return row * D + ((((col >> 3) ^ swz<D>(row))) << 3) + (col & 7);
}

// 16-byte operand read: row `row`, columns col .. col + 7 (col a multiple of 8).
template <int D>
__device__ __forceinline__ e16x8 lds_read_row8(const uint16_t* tile, int row, int col) {
  return as_e16x8(*reinterpret_cast<const i32x4*>(tile + lds_off<D>(row, col)));
}

// Transposed operand read: this lane receives column (col0 + (lane % 32)) at the eight rows
// row0 + 4h + {0,1,2,3} and row0 + 8 + 4h + {0,1,2,3} (h = lane / 32), in that slot order.
template <int D>
__device__ __forceinline__ e16x8 lds_read_col8_tr(const uint16_t* tile, int row0, int col0, int lane) {
  const int s = lane & 15;
  const int g = lane >> 4;
  const int h = lane >> 5;
  const int col = col0 + ((g & 1) << 4) + ((s & 3) << 2);
  const int r1 = row0 + (h << 2) + (s >> 2);
  const uint16_t* p1 = tile + lds_off<D>(r1, col);
  const uint16_t* p2 = tile + lds_off<D>(r1 + 8, col);
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p2));
  i32x2 a = __builtin_bit_cast(i32x2, lo);
  i32x2 b = __builtin_bit_cast(i32x2, hi);
  return make_e16x8((uint32_t)a[0], (uint32_t)a[1], (uint32_t)b[0], (uint32_t)b[1]);
}

// Byte address in LDS of a __shared__ object.  Take it from the array itself (not from a pointer
// that may have passed through a select): the cast then folds to the object's LDS offset.
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) T*)p;
}

// Direct global -> LDS staging of a ROWS x D tile of 16-bit elements with buffer_load_dwordx4 ... lds: each
// lane moves 16 bytes straight into LDS (lane l of a wave writes at M0 + 16 l), so no registers
// hold the tile in flight.  The swizzle is applied on the global side: LDS chunk position p
// (row p / (D/8), physical chunk p % (D/8)) is fed from logical chunk physical ^ swz(row).  The
// buffer resource covers only rows row0 .. n_rows - 1 of the head, and the hardware returns zeros
// for rows past it (the kernels mask those keys/queries anyway).
//
// The loads are written as inline assembly.  Issued through the compiler's LDS-DMA builtin, they
// count as pending LDS writes, and the compiler then waits for them (vmcnt) before the next LDS
// read of any tile: every block would stall on the next block's memory latency.  Here the
// compiler does not see them; completion is the caller's job: wait_vm0 and then a barrier before
// the tile is read.
template <int ROWS, int D, int NT>
struct DirectStage {
  static constexpr int kChunksPerRow = D / 8;
  static constexpr int kChunks = ROWS * kChunksPerRow;
  static constexpr int kWaves = NT / 64;
  static constexpr int kPer = kChunks / NT;  // 16-byte loads per lane
  static_assert(kChunks % NT == 0, "tile must split evenly over the threads");
  int voff[kPer];  // byte offset of this lane's chunks relative to row0
  int wave;

  __device__ __forceinline__ void init(int tid) {
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int p = (wave * kPer + i) * 64 + l;
      const int r = p / kChunksPerRow;
      const int pc = p % kChunksPerRow;
      voff[i] = r * (D * 2) + ((pc ^ swz<D>(r)) << 4);
    }
  }
  // As issue, with this lane's offsets formed on the spot instead of read from voff (for kernels
  // short of registers); needs only `wave` set.  The lane index passes through an empty asm
  // statement so the compiler cannot hoist the offsets out of the caller's loop (it would keep
  // them live across the loop, which is what this variant avoids).
  __device__ __forceinline__ void issue_lazy(const uint16_t* head, int row0, int n_rows, uint32_t lds, int lane) {
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int p = (wave * kPer + i) * 64 + lane;
      const int r = p / kChunksPerRow;
      const int pc = p % kChunksPerRow;
      voff[i] = r * (D * 2) + ((pc ^ swz<D>(r)) << 4);
    }
    issue(head, row0, n_rows, lds);
  }
  // lds: byte address of the destination tile in LDS (lds_addr of the __shared__ array).
  __device__ __forceinline__ void issue(const uint16_t* head, int row0, int n_rows, uint32_t lds) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const int rows_left = n_rows - row0;
    const int nbytes = rows_left > 0 ? rows_left * (D * 2) : 0;
    const uint64_t base = (uint64_t)(uintptr_t)(head + (int64_t)row0 * D);
    // Buffer resource: 48-bit base, stride 0, num_records = bytes in range, raw-buffer flags.
    i32x4 rs;
    rs[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    rs[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(base >> 32) & 0xFFFFu));
    rs[2] = __builtin_amdgcn_readfirstlane(nbytes);
    rs[3] = 0x00020000;
    const int lds0 = (int)lds;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int m0v = __builtin_amdgcn_readfirstlane(lds0 + (wave * kPer + i) * 1024);
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
                   :
                   : "v"(voff[i]), "s"(m0v), "s"(rs)
                   : "memory", "m0");
    }
#pragma clang diagnostic pop
#else
    (void)head, (void)row0, (void)n_rows, (void)lds;
#endif
  }
};

// Store a wave's 32 output rows of D 16-bit elements held as the transposed accumulator tiles of
// 32x32 products (tile dt, register r of lane l: row l % 32, column 32 dt + 8 (r / 4) + 4 (l / 32)
// + r % 4).  Stored directly, every store instruction would put 8 bytes into each of 32 rows,
// 32 cache lines per instruction, and the vector memory pipeline takes about a line per cycle.
// Instead the rows go through LDS: each lane packs its pieces into this wave's stage area (32
// rows of 2D bytes, 16-byte chunk c of row r at chunk c ^ (r % (2D / 16)), which spreads both
// access patterns over the banks), then reads back 16-byte chunks in row order and stores them,
// so that each store instruction writes whole consecutive rows (the 32 rows are consecutive in
// memory, dst pointing at the first).  A wave reads only what it wrote itself, and one wave's LDS
// operations complete in order, so no barrier is needed; the caller makes sure no other wave still
// reads that LDS.  Rows from n_rows on are not stored.  value(dt, r) gives the element.
template <int E, int D, typename F>
__device__ __forceinline__ void store_rows_via_lds(uint8_t* stage, uint16_t* dst, int n_rows, int lane, F&& value) {
  constexpr int RB = 2 * D;     // bytes per row
  constexpr int CPR = RB / 16;  // 16-byte chunks per row
  const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      i32x2 w;
      w[0] = (int)pack2<E>(value(dt, 4 * rr), value(dt, 4 * rr + 1));
      w[1] = (int)pack2<E>(value(dt, 4 * rr + 2), value(dt, 4 * rr + 3));
      const int chunk = (4 * dt + rr) ^ (l32 % CPR);
      *reinterpret_cast<i32x2*>(stage + l32 * RB + 16 * chunk + 8 * hh) = w;
    }
#pragma unroll
  for (int i = 0; i < 32 * CPR / 64; ++i) {
    const int c = 64 * i + lane, row = c / CPR, col = c % CPR;
    const i32x4 v = *reinterpret_cast<const i32x4*>(stage + row * RB + 16 * (col ^ (row % CPR)));
    if (row < n_rows) *reinterpret_cast<i32x4*>(dst + (int64_t)row * D + 8 * col) = v;
  }
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E - 1, so that the body can
// use the index in constant expressions (register-array indices, if constexpr).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Scheduling-group masks for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedValu = 0x002;
constexpr int kSchedDsRead = 0x100;

// Ask the scheduler to run LDS operand reads DEPTH MFMAs ahead of the MFMAs that consume them:
// DEPTH reads first, then (MFMA, READS_PER reads) pairs, then the remaining MFMAs.  Applies to
// the scheduling region the call sits in (between sched_barrier fences).
template <int N_MFMA, int READS_PER, int DEPTH>
__device__ __forceinline__ void sched_reads_ahead() {
#pragma unroll
  for (int i = 0; i < DEPTH * READS_PER; ++i) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
#pragma unroll
  for (int i = 0; i < N_MFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if (i + DEPTH < N_MFMA) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, READS_PER, 0);
  }
}

// As sched_reads_ahead, with VALU_PER vector instructions placed after each MFMA as well.
template <int N_MFMA, int READS_PER, int DEPTH, int VALU_PER>
__device__ __forceinline__ void sched_reads_ahead_valu() {
#pragma unroll
  for (int i = 0; i < DEPTH * READS_PER; ++i) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
#pragma unroll
  for (int i = 0; i < N_MFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if (i + DEPTH < N_MFMA) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, READS_PER, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, VALU_PER, 0);
  }
}

// Wait until this wave's outstanding vector-memory operations (including direct LDS loads) are
// done: s_waitcnt vmcnt(0), other counters left at their maximum.
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Blocks of bc consecutive rows (from row 0) that hold any row of 0..last; 0 when last < 0.
__device__ __forceinline__ int blocks_through(int last, int bc) { return last < 0 ? 0 : last / bc + 1; }
// Blocks of bc consecutive rows (from row 0) that lie entirely within 0..last.
__device__ __forceinline__ int blocks_within(int last, int bc) { return last < 0 ? 0 : (last + 1) / bc; }

// Workgroup -> (head, tile rank).  The hardware hands consecutive workgroup ids to the 8 XCDs in
// turn, so when the head count divides by 8, id x runs on XCD x % 8 and that XCD is given the
// heads congruent to it: the concurrently running tiles of a head then share one XCD's L2.
// Ranks are walked in order within an XCD, so the longest (rank 0) tiles start first.
__device__ __forceinline__ void map_block(int x, int n_heads, int n_tiles, int& head, int& rank) {
  if ((n_heads & 7) == 0) {
    const int xcd = x & 7;
    const int slot = x >> 3;
    const int per = n_heads >> 3;
    rank = slot / per;
    head = xcd + 8 * (slot % per);
  } else {
    rank = x / n_heads;
    head = x % n_heads;
  }
  (void)n_tiles;
}

}  // namespace fa
