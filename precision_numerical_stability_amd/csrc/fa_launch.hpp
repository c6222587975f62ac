// Internal interface between the C ABI (fa_api.cpp) and the kernel translation units.
// Arguments here are already validated; these functions only launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int32_t* dupcnt;  // may be null
  int32_t* ones;    // may be null
  float* smin;      // may be null: per-row min of the scaled visible scores
  float* smax;      // may be null: per-row max of the scaled visible scores
  float* mshift;    // may be null: per-row shift of the repeated-maximum rule (natural log)
  int BH;           // B * H
  int Nq;           // queries per head
  int Nk;           // keys per head
  int coff;         // causal: key j is visible to query i iff j <= i + coff
  int n_tiles;      // query tiles per head (set by launch_fwd)
  float sl2;        // scale * log2(e)
  float scale;
  float beta;
  const uint8_t* v8;    // FP8 P^ V only: V as E4M3 blocks written by launch_v8_pack
  const float* vscale;  // FP8 P^ V only: one scale per (head, 128-key block)
  int n_vblk;           // FP8 P^ V only: 128-key blocks per head
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const float* lse;
  const uint16_t* dO;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;
  int BH;
  int Nq;       // queries per head
  int Nk;       // keys per head
  int coff;     // causal: key j is visible to query i iff j <= i + coff
  int n_tiles;  // set by each launcher
  float scale;
  float sl2;    // scale * log2(e)
  int fuse_delta;  // dQ kernel: form delta for its rows (and store it) instead of loading it
};

// Launchers per element type E (kElemBf16 = 0, kElemF16 = 1 in fa_common.hpp): the kernel
// translation units are compiled once per element type and each defines its instance.
template <int E>
hipError_t launch_fwd(FwdArgs a, int d, bool causal, int mode, bool stats, bool kahan, hipStream_t s);
template <int E>
hipError_t launch_bwd_delta(BwdArgs a, int d, hipStream_t s);
template <int E>
hipError_t launch_bwd_dkdv(BwdArgs a, int d, bool causal, hipStream_t s);
template <int E>
hipError_t launch_bwd_dq(BwdArgs a, int d, bool causal, hipStream_t s);
int fwd_kv_block(int d, bool causal);
// FP8 P^ V: quantise V ([BH, Nk, d] bf16) into v8 ([BH, ceil(Nk / 128), d, 128] bytes) and
// vscale ([BH, ceil(Nk / 128)] fp32).  Defined in the FA_ELEM = 2 instance of fa_fwd.hip.
hipError_t launch_v8_pack(const uint16_t* v, uint8_t* v8, float* vscale, int BH, int Nk, int d, hipStream_t s);
int fwd_q_block(int d);

}  // namespace fa
