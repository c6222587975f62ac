// C ABI of the attention library: argument validation (no HIP call before it passes), template
// dispatch and launches on the caller's stream.  The library allocates, frees and synchronises
// nothing and keeps no state apart from a per-thread copy of the last HIP error.
#include "../../include/fa_stable.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxElems = int64_t(1) << 40;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shared shape/parameter checks.  Returns FA_OK, or the first error found.
int check_common(int B, int H, int Nq, int Nk, int d, int causal, float scale, float beta, int stable_flag) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if (causal < FA_CAUSAL_NONE || causal > FA_CAUSAL_BOTTOM_RIGHT) return FA_ERR_PARAM;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_PARAM;
  if (!std::isfinite(beta) || !(beta >= 1.f)) return FA_ERR_PARAM;
  if (stable_flag < 0 || stable_flag > 2) return FA_ERR_PARAM;
  const int64_t bh = int64_t(B) * int64_t(H);
  if (bh == 0) return FA_OK;
  if (bh > INT32_MAX / 8) return FA_ERR_SHAPE;
  if (bh * Nq * d >= kMaxElems || bh * Nk * d >= kMaxElems) return FA_ERR_SHAPE;
  // One head's rows are addressed through 32-bit buffer ranges.
  if (int64_t(Nq) * d * 2 > int64_t(INT32_MAX) || int64_t(Nk) * d * 2 > int64_t(INT32_MAX)) return FA_ERR_SHAPE;
  return FA_OK;
}

// Key j is visible to query i iff j <= i + coff.
int causal_offset(int causal, int Nq, int Nk) { return causal == FA_CAUSAL_BOTTOM_RIGHT ? Nk - Nq : 0; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  g_last_hip_error = static_cast<int>(e);
  return FA_ERR_HIP;
}

// Bytes of the FP8 P^ V workspace: E4M3 V blocks (d rows of 128 bytes per 128-key block and head),
// then one fp32 scale per block and head.
size_t fp8pv_v8_bytes(int64_t bh, int Nk, int d) { return size_t(bh) * size_t((Nk + 127) / 128) * size_t(d) * 128; }

// The forward entry points share this body; elem is FA_ELEM_BF16, FA_ELEM_F16 or -1 for the FP8
// P^ V variant (bf16 tensors), which also takes the workspace.
int fwd_body(const void* q, const void* k, const void* v, void* o, float* lse, int32_t* dupcnt, int32_t* ones,
             float* smin, float* smax, float* mshift, void* workspace, int B, int H, int Nq, int Nk, int d, int causal,
             float scale, float beta, int stable_flag, int flags, int elem, void* stream) {
  const bool fp8pv = elem < 0;
  const int st = check_common(B, H, Nq, Nk, d, causal, scale, beta, stable_flag);
  if (st != FA_OK) return st;
  if ((flags & ~FA_FWD_COMPENSATED_SUM) != 0) return FA_ERR_PARAM;
  if (!fp8pv && elem != FA_ELEM_BF16 && elem != FA_ELEM_F16) return FA_ERR_PARAM;
  if (int64_t(B) * H == 0 || Nq == 0) return FA_OK;
  if (!q || !o || !lse) return FA_ERR_NULL;
  if (Nk > 0 && (!k || !v)) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return FA_ERR_ALIGN;
  if (!aligned(lse, 4) || (dupcnt && !aligned(dupcnt, 4)) || (ones && !aligned(ones, 4))) return FA_ERR_ALIGN;
  if ((smin && !aligned(smin, 4)) || (smax && !aligned(smax, 4)) || (mshift && !aligned(mshift, 4))) return FA_ERR_ALIGN;
  if (fp8pv && Nk > 0 && !workspace) return FA_ERR_NULL;
  if (fp8pv && !aligned(workspace, 16)) return FA_ERR_ALIGN;

  fa::FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.dupcnt = dupcnt;
  a.ones = ones;
  a.smin = smin;
  a.smax = smax;
  a.mshift = mshift;
  a.BH = B * H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.coff = causal_offset(causal, Nq, Nk);
  a.sl2 = scale * 1.4426950408889634f;
  a.scale = scale;
  a.beta = beta;
  const bool stats = dupcnt || ones || smin || smax;
  const bool kahan = (flags & FA_FWD_COMPENSATED_SUM) != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fp8pv) {
    const int64_t bh = int64_t(B) * H;
    a.n_vblk = (Nk + 127) / 128;
    a.v8 = static_cast<const uint8_t*>(workspace);
    a.vscale = reinterpret_cast<const float*>(static_cast<const uint8_t*>(workspace) + fp8pv_v8_bytes(bh, Nk, d));
    uint8_t* v8 = static_cast<uint8_t*>(workspace);
    float* vscale = reinterpret_cast<float*>(v8 + fp8pv_v8_bytes(bh, Nk, d));
    const int rc = hip_status(fa::launch_v8_pack(a.v, v8, vscale, B * H, Nk, d, s));
    if (rc != FA_OK) return rc;
    return hip_status(fa::launch_fwd<fa::kElemFp8PV>(a, d, causal != 0, stable_flag, stats, kahan, s));
  }
  return hip_status(elem == FA_ELEM_F16 ? fa::launch_fwd<fa::kElemF16>(a, d, causal != 0, stable_flag, stats, kahan, s)
                                        : fa::launch_fwd<fa::kElemBf16>(a, d, causal != 0, stable_flag, stats, kahan, s));
}

// Scratch of the no-allocation backward (fa_bwd_noalloc): delta for up to kScratchRows rows,
// one copy per GPU the library runs on, held until the process ends.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the symbol); the device
// address comes from hipGetSymbolAddress, looked up once per device with that device current.
constexpr int64_t kScratchRows = int64_t(1) << 21;  // 8 MiB of fp32
static __device__ __align__(256) float scratch[kScratchRows];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
float* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the scratch on the GPU that `stream` runs on (the current device for the
// default stream), or the HIP error of the lookup.  The kernels go to that stream, so they must
// get that GPU's copy of the array; its first lookup makes the GPU current for the call and
// restores the caller's device afterwards.
hipError_t scratch_for_stream(hipStream_t stream, float** out) {
  int dev = -1;
  hipError_t e;
  if (stream != nullptr) {
    hipDevice_t d = -1;
    e = hipStreamGetDevice(stream, &d);
    dev = static_cast<int>(d);
  } else {
    e = hipGetDevice(&dev);
  }
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    int cur = -1;
    hipError_t r = hipGetDevice(&cur);
    const bool switch_dev = (r == hipSuccess && cur != dev);
    if (switch_dev) r = hipSetDevice(dev);
    void* ptr = nullptr;
    if (r == hipSuccess) r = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (switch_dev) {
      const hipError_t back = hipSetDevice(cur);
      if (r == hipSuccess) r = back;
    }
    g_scratch_err[dev] = r;
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int fa_fwd_diag(const void* q, const void* k, const void* v, void* o, float* lse, int32_t* dupcnt,
                int32_t* ones, float* smin, float* smax, float* mshift, int B, int H, int Nq, int Nk, int d,
                int causal, float scale, float beta, int stable_flag, int flags, int elem, void* stream) {
  if (elem != FA_ELEM_BF16 && elem != FA_ELEM_F16) {
    // parameters are checked in the documented order: shapes and scalars first
    const int st = check_common(B, H, Nq, Nk, d, causal, scale, beta, stable_flag);
    return st != FA_OK ? st : FA_ERR_PARAM;
  }
  return fwd_body(q, k, v, o, lse, dupcnt, ones, smin, smax, mshift, nullptr, B, H, Nq, Nk, d, causal, scale,
                  beta, stable_flag, flags, elem, stream);
}

int fa_fwd_elem(const void* q, const void* k, const void* v, void* o, float* lse, int32_t* dupcnt,
                int32_t* ones, float* smin, float* smax, int B, int H, int Nq, int Nk, int d, int causal,
                float scale, float beta, int stable_flag, int flags, int elem, void* stream) {
  return fa_fwd_diag(q, k, v, o, lse, dupcnt, ones, smin, smax, nullptr, B, H, Nq, Nk, d, causal, scale, beta,
                     stable_flag, flags, elem, stream);
}

size_t fa_fwd_fp8pv_workspace_bytes(int B, int H, int Nk, int d) {
  if (B < 0 || H < 0 || Nk < 0 || (d != 64 && d != 128)) return 0;
  const int64_t bh = int64_t(B) * H;
  return fp8pv_v8_bytes(bh, Nk, d) + size_t(bh) * size_t((Nk + 127) / 128) * sizeof(float);
}

int fa_fwd_fp8pv(const void* q, const void* k, const void* v, void* o, float* lse, int32_t* dupcnt,
                 int32_t* ones, float* smin, float* smax, void* workspace, int B, int H, int Nq, int Nk, int d,
                 int causal, float scale, float beta, int stable_flag, int flags, void* stream) {
  return fwd_body(q, k, v, o, lse, dupcnt, ones, smin, smax, nullptr, workspace, B, H, Nq, Nk, d, causal, scale,
                  beta, stable_flag, flags, -1, stream);
}

int fa_fwd_qk(const void* q, const void* k, const void* v, void* o, float* lse, int32_t* dupcnt,
              int32_t* ones, float* smin, float* smax, int B, int H, int Nq, int Nk, int d, int causal,
              float scale, float beta, int stable_flag, int flags, void* stream) {
  return fa_fwd_elem(q, k, v, o, lse, dupcnt, ones, smin, smax, B, H, Nq, Nk, d, causal, scale, beta,
                     stable_flag, flags, FA_ELEM_BF16, stream);
}

int fa_fwd_stats(const void* q, const void* k, const void* v, void* o, float* lse, int32_t* dupcnt,
                 int32_t* ones, float* smin, float* smax, int B, int H, int N, int d, int causal,
                 float scale, float beta, int stable_flag, int flags, void* stream) {
  if (causal != 0 && causal != 1) return FA_ERR_PARAM;
  return fa_fwd_qk(q, k, v, o, lse, dupcnt, ones, smin, smax, B, H, N, N, d, causal, scale, beta,
                   stable_flag, flags, stream);
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int32_t* dupcnt,
              int32_t* ones, int B, int H, int N, int d, int causal, float scale, float beta,
              int stable_flag, void* stream) {
  return fa_fwd_stats(q, k, v, o, lse, dupcnt, ones, nullptr, nullptr, B, H, N, d, causal, scale, beta,
                      stable_flag, 0, stream);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, int causal, float scale, float beta, int stable_flag, void* stream) {
  return fa_fwd_ex(q, k, v, o, lse, nullptr, nullptr, B, H, N, d, causal, scale, beta, stable_flag,
                   stream);
}

int fa_bwd_elem(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, void* dq, void* dk, void* dv, float* delta_ws, int B, int H, int Nq, int Nk,
                int d, int causal, float scale, float beta, int stable_flag, int stages, int elem,
                void* stream) {
  const int st = check_common(B, H, Nq, Nk, d, causal, scale, beta, stable_flag);
  if (st != FA_OK) return st;
  if (stages < 1 || stages > FA_BWD_ALL) return FA_ERR_PARAM;
  if (elem != FA_ELEM_BF16 && elem != FA_ELEM_F16) return FA_ERR_PARAM;
  if (int64_t(B) * H == 0 || (Nq == 0 && Nk == 0)) return FA_OK;
  if (Nq > 0 && (!q || !o || !lse || !dO || !dq || !delta_ws)) return FA_ERR_NULL;
  if (Nk > 0 && (!k || !v || !dk || !dv)) return FA_ERR_NULL;
  // dK and dV read Q, dO, LSE and delta whenever there are queries at all.
  if (Nq > 0 && Nk > 0 && (!q || !dO)) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dO, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return FA_ERR_ALIGN;
  if (!aligned(lse, 4) || !aligned(delta_ws, 4)) return FA_ERR_ALIGN;

  fa::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.lse = lse;
  a.dO = static_cast<const uint16_t*>(dO);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.delta = delta_ws;
  a.BH = B * H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.coff = causal_offset(causal, Nq, Nk);
  a.scale = scale;
  a.sl2 = scale * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f16 = elem == FA_ELEM_F16;
  int rc = FA_OK;
  auto run_dq = [&]() {
    return hip_status(f16 ? fa::launch_bwd_dq<fa::kElemF16>(a, d, causal != 0, s)
                          : fa::launch_bwd_dq<fa::kElemBf16>(a, d, causal != 0, s));
  };
  // With both delta and dQ requested, the dQ kernel forms delta for its rows (it holds dO already)
  // and runs first, so the delta kernel and one kernel boundary drop out; dK/dV follows.
  const bool fuse = (stages & FA_BWD_DELTA) && (stages & FA_BWD_DQ);
  if (fuse) {
    a.fuse_delta = 1;
    rc = run_dq();
    a.fuse_delta = 0;
    if (rc != FA_OK) return rc;
  } else if (stages & FA_BWD_DELTA) {
    rc = hip_status(f16 ? fa::launch_bwd_delta<fa::kElemF16>(a, d, s) : fa::launch_bwd_delta<fa::kElemBf16>(a, d, s));
    if (rc != FA_OK) return rc;
  }
  if (stages & FA_BWD_DKDV) {
    rc = hip_status(f16 ? fa::launch_bwd_dkdv<fa::kElemF16>(a, d, causal != 0, s)
                        : fa::launch_bwd_dkdv<fa::kElemBf16>(a, d, causal != 0, s));
    if (rc != FA_OK) return rc;
  }
  if ((stages & FA_BWD_DQ) && !fuse) rc = run_dq();
  return rc;
}

int fa_bwd_qk(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dO, void* dq, void* dk, void* dv, float* delta_ws, int B, int H, int Nq, int Nk,
              int d, int causal, float scale, float beta, int stable_flag, int stages, void* stream) {
  return fa_bwd_elem(q, k, v, o, lse, dO, dq, dk, dv, delta_ws, B, H, Nq, Nk, d, causal, scale, beta,
                     stable_flag, stages, FA_ELEM_BF16, stream);
}

int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dO, void* dq, void* dk, void* dv, float* delta_ws, int B, int H, int N,
              int d, int causal, float scale, float beta, int stable_flag, int stages, void* stream) {
  if (causal != 0 && causal != 1) return FA_ERR_PARAM;
  return fa_bwd_qk(q, k, v, o, lse, dO, dq, dk, dv, delta_ws, B, H, N, N, d, causal, scale, beta,
                   stable_flag, stages, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dO, void* dq, void* dk, void* dv, float* delta_ws, int B, int H, int N, int d,
           int causal, float scale, float beta, int stable_flag, void* stream) {
  return fa_bwd_ex(q, k, v, o, lse, dO, dq, dk, dv, delta_ws, B, H, N, d, causal, scale, beta,
                   stable_flag, FA_BWD_ALL, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal,
                   float scale, float beta, int stable_flag, void* stream) {
  // fa_bwd's checks (less the workspace), then the size, all before any HIP call.
  if (causal != 0 && causal != 1) return FA_ERR_PARAM;
  const int st = check_common(B, H, N, N, d, causal, scale, beta, stable_flag);
  if (st != FA_OK) return st;
  const int64_t rows = int64_t(B) * H * N;
  if (rows == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dO, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  if (rows > kScratchRows) return FA_ERR_SCRATCH;
  float* ws = nullptr;
  const int rc = hip_status(scratch_for_stream(static_cast<hipStream_t>(stream), &ws));
  if (rc != FA_OK) return rc;
  return fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, ws, B, H, N, d, causal, scale, beta, stable_flag, stream);
}

size_t fa_bwd_noalloc_max_rows(void) { return size_t(kScratchRows); }

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (B < 0 || H < 0 || N < 0 || (d != 64 && d != 128)) return 0;
  return size_t(B) * size_t(H) * size_t(N) * sizeof(float);
}

int fa_fwd_kv_block(int d, int causal) { return fa::fwd_kv_block(d, causal != 0); }

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: B, H or a sequence length negative, or the problem is too large";
    case FA_ERR_HEADDIM: return "FA_ERR_HEADDIM: d must be 64 or 128";
    case FA_ERR_PARAM: return "FA_ERR_PARAM: causal, scale, beta, stable_flag, flags, stages or elem out of range";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: tensor pointers must be 16-byte aligned, vectors 4-byte";
    case FA_ERR_HIP: return "FA_ERR_HIP: a HIP call failed (see fa_last_hip_error)";
    case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH: B*H*N exceeds the rows the no-allocation backward holds (fa_bwd_noalloc_max_rows)";
    default: return "unknown fa_status";
  }
}

int fa_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
