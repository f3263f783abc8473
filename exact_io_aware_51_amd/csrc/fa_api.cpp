// fa_api.cpp -- the C ABI of libfa (declared in include/fa.h).
//
// Every argument is validated here, before any HIP call, so an invalid call
// queues nothing and can be tested on a machine without a GPU.  Valid calls
// pick the kernel instantiation for (dtype, d, causal) and queue it on the
// caller's stream.  No device memory is allocated, freed or cached here.
#include <cmath>
#include <cstdint>

#include "fa.h"
#include "fa_launch.h"

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
  const void* p;
  size_t bytes;
};

bool overlap(Range a, Range b) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

size_t elem_bytes(int dtype) { return dtype == FA_F32 ? 4 : 2; }

// Shape / dtype / scale checks shared by both passes.
int check_common(int B, int H, int N, int d, float scale, int causal, int dtype) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if ((long long)B * H * N >= (1LL << 31)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || !std::isfinite(scale * 1.4426950408889634f)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

}  // namespace

extern "C" {

int fa_version(void) { return kVersion; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument (NULL or misaligned pointer, bad size, non-finite scale, causal not 0/1, or outputs aliasing inputs)";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension or dtype (d must be 64 or 128; dtype fp32, fp16 or bf16)";
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than fa_bwd_workspace_bytes()";
    case FA_ERR_HIP: return "the HIP runtime refused the launch (no device, invalid stream, or an earlier error)";
    default: return "unknown status";
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, fa_dtype dtype, void* stream) {
  int st = check_common(B, H, N, d, scale, causal, (int)dtype);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return FA_ERR_INVALID_ARG;
  if (lse && !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  const size_t tb = (size_t)B * H * N * d * elem_bytes(dtype);
  const size_t lb = (size_t)B * H * N * sizeof(float);
  const Range ins[3] = {{q, tb}, {k, tb}, {v, tb}};
  for (const Range& r : ins) {
    if (overlap({o, tb}, r)) return FA_ERR_INVALID_ARG;
    if (lse && overlap({lse, lb}, r)) return FA_ERR_INVALID_ARG;
  }
  if (lse && overlap({o, tb}, {lse, lb})) return FA_ERR_INVALID_ARG;

  fa::FwdProblem p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.H = H; p.N = N; p.d = d;
  p.scale = scale; p.causal = causal; p.dtype = (int)dtype;
  (void)hipGetLastError();  // report only this launch's error
  return hip_status(fa::launch_fwd(p, reinterpret_cast<hipStream_t>(stream)));
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, fa_dtype dtype) {
  if (check_common(B, H, N, d, 1.0f, 0, (int)dtype) != FA_OK) return 0;
  const size_t need = (size_t)B * H * N * sizeof(float);
  return (need + 255) & ~(size_t)255;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
           float scale, int causal, fa_dtype dtype, void* stream) {
  int st = check_common(B, H, N, d, scale, causal, (int)dtype);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  const void* p16[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : p16)
    if (!aligned(p, 16)) return FA_ERR_INVALID_ARG;
  if (!aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  const size_t need = fa_bwd_workspace_bytes(B, H, N, d, dtype);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return FA_ERR_WORKSPACE;
  const size_t tb = (size_t)B * H * N * d * elem_bytes(dtype);
  const size_t lb = (size_t)B * H * N * sizeof(float);
  const Range ins[6] = {{q, tb}, {k, tb}, {v, tb}, {o, tb}, {dout, tb}, {lse, lb}};
  const Range outs[4] = {{dq, tb}, {dk, tb}, {dv, tb}, {workspace, need}};
  for (int i = 0; i < 4; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return i == 3 ? FA_ERR_WORKSPACE : FA_ERR_INVALID_ARG;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return j == 3 ? FA_ERR_WORKSPACE : FA_ERR_INVALID_ARG;
  }

  fa::BwdProblem p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv; p.dvec = static_cast<float*>(workspace);
  p.B = B; p.H = H; p.N = N; p.d = d;
  p.scale = scale; p.causal = causal; p.dtype = (int)dtype;
  (void)hipGetLastError();
  return hip_status(fa::launch_bwd(p, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
