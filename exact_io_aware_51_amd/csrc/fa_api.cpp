// fa_api.cpp -- the C ABI of libfa (declared in include/fa.h).
//
// Every argument is validated here, before any HIP call, so an invalid call
// queues nothing and can be tested on a machine without a GPU.  Valid calls
// pick the kernel instantiation for (dtype, d, causal) and queue it on the
// caller's stream.  No device memory is allocated, freed or cached here.
#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "fa.h"
#include "fa_launch.h"

namespace {

constexpr int kVersion = 10100;  // 1.1.0: dropout, 8-bit forward, split-key forward
// Block-sparse kernels keep one mask row or column as bits in LDS: at most
// 64 x 64 blocks of 128.
constexpr int kMaxSparseN = 64 * 64 * 128;
// Key ranges a split-key forward may use.
constexpr int kMaxSplits = 256;

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
int check_shape(int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if ((long long)B * H * Nq >= (1LL << 31) || (long long)B * H * Nk >= (1LL << 31)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || !std::isfinite(scale * 1.4426950408889634f)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

int check_common(int B, int H, int N, int d, float scale, int causal, int dtype) {
  return check_shape(B, H, N, N, d, scale, causal, dtype);
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Bytes of a block-sparse mask: one byte per (128-query block, 128-key block) pair per (batch, head).
size_t mask_bytes(int B, int H, int Nq, int Nk) {
  const size_t bq = (size_t)(Nq + fa::kMaskBlock - 1) / fa::kMaskBlock, bk = (size_t)(Nk + fa::kMaskBlock - 1) / fa::kMaskBlock;
  return (size_t)B * H * bq * bk;
}

// Dropout settings of one call (on = 0: none).  A weight is kept when its
// 32-bit Philox word is >= threshold = floor(p * 2^32), so it is dropped with
// probability threshold / 2^32 (p up to 2^-32); kept weights are scaled by
// 1 / (1 - p).
struct DropSpec {
  int on;
  unsigned threshold, seed_lo, seed_hi, offset;
  float scale;
};
constexpr DropSpec kNoDrop{0, 0u, 0u, 0u, 0u, 1.0f};

int drop_spec(float p, unsigned long long seed, unsigned offset, DropSpec* out) {
  if (!(p >= 0.0f && p < 1.0f)) return FA_ERR_INVALID_ARG;  // also rejects NaN
  const double t = std::floor((double)p * 4294967296.0);    // < 2^32 since p < 1
  *out = DropSpec{p > 0.0f ? 1 : 0, (unsigned)t, (unsigned)(seed & 0xFFFFFFFFull), (unsigned)(seed >> 32), offset,
                  (float)(1.0 / (1.0 - (double)p))};
  return FA_OK;
}

// Forward validation and launch for q/o of Nq rows and k/v of Nk rows per
// (batch, head), with optional device arrays of per-sequence lengths.
int run_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk, int d,
            const int* seqlens_q, const int* seqlens_k, const unsigned char* block_mask, float scale, int causal,
            int dtype, void* stream, const DropSpec& drop = kNoDrop, int splits = 1, void* part = nullptr) {
  int st = check_shape(B, H, Nq, Nk, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return FA_ERR_INVALID_ARG;
  if (lse && !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  if ((seqlens_q && !aligned(seqlens_q, 4)) || (seqlens_k && !aligned(seqlens_k, 4))) return FA_ERR_INVALID_ARG;
  const size_t tq = (size_t)B * H * Nq * d * elem_bytes(dtype);
  const size_t tk = (size_t)B * H * Nk * d * elem_bytes(dtype);
  const size_t lb = (size_t)B * H * Nq * sizeof(float);
  const size_t sb = (size_t)B * sizeof(int);
  const Range ins[6] = {{q, tq}, {k, tk}, {v, tk}, {seqlens_q, seqlens_q ? sb : 0}, {seqlens_k, seqlens_k ? sb : 0},
                        {block_mask, block_mask ? mask_bytes(B, H, Nq, Nk) : 0}};
  for (const Range& r : ins) {
    if (overlap({o, tq}, r)) return FA_ERR_INVALID_ARG;
    if (lse && overlap({lse, lb}, r)) return FA_ERR_INVALID_ARG;
  }
  if (lse && overlap({o, tq}, {lse, lb})) return FA_ERR_INVALID_ARG;

  fa::FwdProblem p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.H = H; p.Nq = Nq; p.Nk = Nk; p.d = d;
  p.seqlens_q = seqlens_q; p.seqlens_k = seqlens_k;
  p.block_mask = block_mask;
  p.drop_on = drop.on; p.drop_threshold = drop.threshold; p.drop_seed_lo = drop.seed_lo;
  p.drop_seed_hi = drop.seed_hi; p.drop_offset = drop.offset; p.drop_scale = drop.scale;
  p.scale = scale; p.causal = causal; p.dtype = dtype;
  p.splits = splits; p.part = static_cast<float*>(part);
  (void)hipGetLastError();  // report only this launch's error
  return hip_status(fa::launch_fwd(p, reinterpret_cast<hipStream_t>(stream)));
}

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
    case FA_ERR_TOO_LARGE: return "B * H * N exceeds the static scratch of fa_bwd_static (FA_STATIC_SCRATCH_ROWS rows); use fa_bwd";
    default: return "unknown status";
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, fa_dtype dtype, void* stream) {
  return run_fwd(q, k, v, o, lse, B, H, N, N, d, nullptr, nullptr, nullptr, scale, causal, (int)dtype, stream);
}

int fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk, int d,
              const int* seqlens_q, const int* seqlens_k, float scale, int causal, fa_dtype dtype, void* stream) {
  return run_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, seqlens_q, seqlens_k, nullptr, scale, causal, (int)dtype, stream);
}

size_t fa_fwd_kv_split_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits) {
  if (check_shape(B, H, Nq, Nk, d, 1.0f, 0, FA_BF16) != FA_OK) return 0;
  if (num_splits < 1 || num_splits > kMaxSplits) return 0;
  if (num_splits == 1) return 0;
  const size_t need = (size_t)num_splits * B * H * Nq * (d + 1) * sizeof(float);
  return (need + 255) & ~(size_t)255;
}

int fa_fwd_kv_split_hint(int B, int H, int Nq, int Nk, int d) {
  if (check_shape(B, H, Nq, Nk, d, 1.0f, 0, FA_BF16) != FA_OK) return 1;
  const long long wgs = (long long)B * H * ((Nq + 127) / 128);
  const long long tiles = (Nk + 63) / 64;
  long long s = (2 * 256 + wgs - 1) / wgs;  // about two workgroups per CU
  const long long by_len = tiles / 16;      // each split at least 16 key tiles (1024 keys)
  if (s > by_len) s = by_len;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : (int)s;
}

int fa_fwd_kv_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                    int d, const int* seqlens_q, const int* seqlens_k, float scale, int causal, int num_splits,
                    void* workspace, size_t workspace_bytes, fa_dtype dtype, void* stream) {
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_INVALID_ARG;
  if (num_splits == 1)
    return run_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, seqlens_q, seqlens_k, nullptr, scale, causal, (int)dtype, stream);
  const int st = check_shape(B, H, Nq, Nk, d, scale, causal, (int)dtype);
  if (st != FA_OK) return st;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if ((long long)B * H * ((Nq + 127) / 128) * num_splits >= (1LL << 31)) return FA_ERR_INVALID_ARG;  // grid size
  const size_t need = fa_fwd_kv_split_workspace_bytes(B, H, Nq, Nk, d, num_splits);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return FA_ERR_WORKSPACE;
  const size_t tq = (size_t)B * H * Nq * d * elem_bytes(dtype), tk = (size_t)B * H * Nk * d * elem_bytes(dtype);
  const size_t sb = (size_t)B * sizeof(int);
  const Range others[7] = {{q, tq}, {k, tk}, {v, tk}, {o, tq}, {lse, lse ? (size_t)B * H * Nq * sizeof(float) : 0},
                           {seqlens_q, seqlens_q ? sb : 0}, {seqlens_k, seqlens_k ? sb : 0}};
  for (const Range& r : others)
    if (r.p && overlap({workspace, need}, r)) return FA_ERR_WORKSPACE;
  return run_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, seqlens_q, seqlens_k, nullptr, scale, causal, (int)dtype, stream,
                 kNoDrop, num_splits, workspace);
}

int fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                  const unsigned char* block_mask, float scale, int causal, fa_dtype dtype, void* stream) {
  if (!block_mask) return FA_ERR_INVALID_ARG;
  if (N > kMaxSparseN) return FA_ERR_UNSUPPORTED;
  return run_fwd(q, k, v, o, lse, B, H, N, N, d, nullptr, nullptr, block_mask, scale, causal, (int)dtype, stream);
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, float dropout_p, unsigned long long seed, unsigned offset, fa_dtype dtype,
                   void* stream) {
  DropSpec drop;
  int st = drop_spec(dropout_p, seed, offset, &drop);
  if (st != FA_OK) return st;
  return run_fwd(q, k, v, o, lse, B, H, N, N, d, nullptr, nullptr, nullptr, scale, causal, (int)dtype, stream, drop);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, float descale_q, float descale_k, float descale_v, void* stream) {
  return fa_fwd_fp8_fmt(q, k, v, o, lse, B, H, N, d, scale, causal, descale_q, descale_k, descale_v, FA_FP8_E4M3,
                        stream);
}

int fa_fwd_fp8_fmt(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, float descale_q, float descale_k, float descale_v, fa_fp8_format fmt,
                   void* stream) {
  const int f = static_cast<int>(fmt);
  if (f != FA_FP8_E4M3 && f != FA_FP8_E5M2) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if ((long long)B * H * N >= (1LL << 31)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !std::isfinite(descale_q) || !std::isfinite(descale_k) || !std::isfinite(descale_v))
    return FA_ERR_INVALID_ARG;
  const double eff = (double)scale * descale_q * descale_k;  // scale of the raw code products
  if (!std::isfinite((float)eff) || !std::isfinite((float)eff * 1.4426950408889634f)) return FA_ERR_INVALID_ARG;
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return FA_ERR_INVALID_ARG;
  if (lse && !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  const size_t ti = (size_t)B * H * N * d, to = 2 * ti, lb = (size_t)B * H * N * sizeof(float);
  const Range ins[3] = {{q, ti}, {k, ti}, {v, ti}};
  for (const Range& r : ins) {
    if (overlap({o, to}, r)) return FA_ERR_INVALID_ARG;
    if (lse && overlap({lse, lb}, r)) return FA_ERR_INVALID_ARG;
  }
  if (lse && overlap({o, to}, {lse, lb})) return FA_ERR_INVALID_ARG;
  fa::FwdProblem p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.B = B; p.H = H; p.Nq = N; p.Nk = N; p.d = d;
  p.scale = (float)eff; p.causal = causal; p.descale_v = descale_v;
  p.fp8_format = f == FA_FP8_E5M2 ? 1 : 0;
  (void)hipGetLastError();  // report only this launch's error
  return hip_status(fa::launch_fwd8(p, reinterpret_cast<hipStream_t>(stream)));
}

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, fa_dtype dtype) {
  if (check_common(B, H, N, d, 1.0f, 0, (int)dtype) != FA_OK) return 0;
  const size_t need = (size_t)B * H * N * sizeof(float);
  return (need + 255) & ~(size_t)255;
}

}  // extern "C"

namespace {

// Validation of a backward call (or one stage of it).  A slot the stage does
// not use holds kUnused (the address of a private host object, which no caller
// can pass by accident); every other pointer is checked.
struct BwdPtrs {
  const void *q, *k, *v, *o, *dout, *lse;
  void *dq, *dk, *dv, *ws;
};

const char kUnusedTag = 0;
const void* const kUnused = &kUnusedTag;

int check_bwd(const BwdPtrs& p, size_t workspace_bytes, int B, int H, int Nq, int Nk, int d, const int* seqlens_q,
              const int* seqlens_k, const unsigned char* block_mask, float scale, int causal, int dtype) {
  int st = check_shape(B, H, Nq, Nk, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  if ((seqlens_q && !aligned(seqlens_q, 4)) || (seqlens_k && !aligned(seqlens_k, 4))) return FA_ERR_INVALID_ARG;
  const void* p16[] = {p.q, p.k, p.v, p.o, p.dout, p.dq, p.dk, p.dv};
  for (const void* x : p16) {
    if (x == kUnused) continue;
    if (!x || !aligned(x, 16)) return FA_ERR_INVALID_ARG;
  }
  if (p.lse != kUnused && (!p.lse || !aligned(p.lse, 4))) return FA_ERR_INVALID_ARG;
  const size_t need = fa_bwd_workspace_bytes(B, H, Nq, d, (fa_dtype)dtype);
  if (p.ws != kUnused && (!p.ws || workspace_bytes < need || !aligned(p.ws, 16))) return FA_ERR_WORKSPACE;
  const size_t tq = (size_t)B * H * Nq * d * elem_bytes(dtype);
  const size_t tk = (size_t)B * H * Nk * d * elem_bytes(dtype);
  const size_t lb = (size_t)B * H * Nq * sizeof(float);
  const size_t sb = (size_t)B * sizeof(int);
  const Range ins[9] = {{p.q, tq},    {p.k, tk},   {p.v, tk}, {p.o, tq}, {p.dout, tq}, {p.lse, lb},
                        {seqlens_q ? seqlens_q : kUnused, sb}, {seqlens_k ? seqlens_k : kUnused, sb},
                        {block_mask ? static_cast<const void*>(block_mask) : kUnused, mask_bytes(B, H, Nq, Nk)}};
  const Range outs[4] = {{p.dq, tq}, {p.dk, tk}, {p.dv, tk}, {p.ws, need}};
  for (int i = 0; i < 4; ++i) {
    if (outs[i].p == kUnused) continue;
    for (const Range& r : ins)
      if (r.p != kUnused && overlap(outs[i], r)) return i == 3 ? FA_ERR_WORKSPACE : FA_ERR_INVALID_ARG;
    for (int j = i + 1; j < 4; ++j)
      if (outs[j].p != kUnused && overlap(outs[i], outs[j])) return j == 3 ? FA_ERR_WORKSPACE : FA_ERR_INVALID_ARG;
  }
  return FA_OK;
}

fa::BwdProblem bwd_problem(const BwdPtrs& p, int B, int H, int Nq, int Nk, int d, const int* seqlens_q,
                          const int* seqlens_k, const unsigned char* block_mask, float scale, int causal,
                          int dtype, const DropSpec& drop = kNoDrop) {
  fa::BwdProblem b;
  auto use = [](const void* x) { return x == kUnused ? nullptr : x; };
  b.q = use(p.q); b.k = use(p.k); b.v = use(p.v); b.o = use(p.o); b.dout = use(p.dout);
  b.lse = static_cast<const float*>(use(p.lse));
  b.dq = const_cast<void*>(use(p.dq)); b.dk = const_cast<void*>(use(p.dk)); b.dv = const_cast<void*>(use(p.dv));
  b.dvec = static_cast<float*>(const_cast<void*>(use(p.ws)));
  b.B = B; b.H = H; b.Nq = Nq; b.Nk = Nk; b.d = d;
  b.seqlens_q = seqlens_q; b.seqlens_k = seqlens_k;
  b.block_mask = block_mask;
  b.drop_on = drop.on; b.drop_threshold = drop.threshold; b.drop_seed_lo = drop.seed_lo;
  b.drop_seed_hi = drop.seed_hi; b.drop_offset = drop.offset; b.drop_scale = drop.scale;
  b.scale = scale; b.causal = causal; b.dtype = dtype;
  b.dq_rowsum = 0;
  return b;
}

int run_stages(const fa::BwdProblem& b, std::initializer_list<int> stages, void* stream) {
  (void)hipGetLastError();  // report only these launches' errors
  hipError_t e = hipSuccess;
  for (int s : stages) {
    e = fa::launch_bwd_stage(b, s, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) break;
  }
  return hip_status(e);
}

// A whole backward pass: dQ with the row sums D formed on the way, then dK/dV.
int run_bwd(const fa::BwdProblem& b, void* stream) { return run_stages(b, {3, 1}, stream); }

}  // namespace

extern "C" {

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
           float scale, int causal, fa_dtype dtype, void* stream) {
  const BwdPtrs p{q, k, v, o, dout, lse, dq, dk, dv, workspace};
  int st = check_bwd(p, workspace_bytes, B, H, N, N, d, nullptr, nullptr, nullptr, scale, causal, (int)dtype);
  if (st != FA_OK) return st;
  return run_bwd(bwd_problem(p, B, H, N, N, d, nullptr, nullptr, nullptr, scale, causal, (int)dtype), stream);
}

int fa_bwd_kv(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
              void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk,
              int d, const int* seqlens_q, const int* seqlens_k, float scale, int causal, fa_dtype dtype,
              void* stream) {
  const BwdPtrs p{q, k, v, o, dout, lse, dq, dk, dv, workspace};
  int st = check_bwd(p, workspace_bytes, B, H, Nq, Nk, d, seqlens_q, seqlens_k, nullptr, scale, causal, (int)dtype);
  if (st != FA_OK) return st;
  return run_bwd(bwd_problem(p, B, H, Nq, Nk, d, seqlens_q, seqlens_k, nullptr, scale, causal, (int)dtype), stream);
}

int fa_bwd_sparse(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                  const unsigned char* block_mask, float scale, int causal, fa_dtype dtype, void* stream) {
  if (!block_mask) return FA_ERR_INVALID_ARG;
  if (N > kMaxSparseN) return FA_ERR_UNSUPPORTED;
  const BwdPtrs p{q, k, v, o, dout, lse, dq, dk, dv, workspace};
  int st = check_bwd(p, workspace_bytes, B, H, N, N, d, nullptr, nullptr, block_mask, scale, causal, (int)dtype);
  if (st != FA_OK) return st;
  return run_bwd(bwd_problem(p, B, H, N, N, d, nullptr, nullptr, block_mask, scale, causal, (int)dtype), stream);
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                   float scale, int causal, float dropout_p, unsigned long long seed, unsigned offset, fa_dtype dtype,
                   void* stream) {
  DropSpec drop;
  int st = drop_spec(dropout_p, seed, offset, &drop);
  if (st != FA_OK) return st;
  const BwdPtrs p{q, k, v, o, dout, lse, dq, dk, dv, workspace};
  st = check_bwd(p, workspace_bytes, B, H, N, N, d, nullptr, nullptr, nullptr, scale, causal, (int)dtype);
  if (st != FA_OK) return st;
  return run_bwd(bwd_problem(p, B, H, N, N, d, nullptr, nullptr, nullptr, scale, causal, (int)dtype, drop), stream);
}

int fa_bwd_static(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, fa_dtype dtype,
                  void* stream) {
  const BwdPtrs p{q, k, v, o, dout, lse, dq, dk, dv, const_cast<void*>(kUnused)};
  int st = check_bwd(p, 0, B, H, N, N, d, nullptr, nullptr, nullptr, scale, causal, (int)dtype);
  if (st != FA_OK) return st;
  if ((long long)B * H * N > fa::kStaticScratchRows) return FA_ERR_TOO_LARGE;
  static_assert(fa::kStaticScratchRows == FA_STATIC_SCRATCH_ROWS, "fa.h states the scratch capacity");
  float* dvec = nullptr;
  if (fa::static_scratch(reinterpret_cast<hipStream_t>(stream), &dvec) != hipSuccess) return FA_ERR_HIP;
  fa::BwdProblem b = bwd_problem(p, B, H, N, N, d, nullptr, nullptr, nullptr, scale, causal, (int)dtype);
  b.dvec = dvec;
  return run_bwd(b, stream);
}

int fa_bwd_rowsum(const void* o, const void* dout, void* workspace, size_t workspace_bytes, int B, int H, int N,
                  int d, fa_dtype dtype, void* stream) {
  void* un = const_cast<void*>(kUnused);
  const BwdPtrs p{kUnused, kUnused, kUnused, o, dout, kUnused, un, un, un, workspace};
  int st = check_bwd(p, workspace_bytes, B, H, N, N, d, nullptr, nullptr, nullptr, 1.0f, 0, (int)dtype);
  if (st != FA_OK) return st;
  return run_stages(bwd_problem(p, B, H, N, N, d, nullptr, nullptr, nullptr, 1.0f, 0, (int)dtype), {0}, stream);
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                const void* workspace, size_t workspace_bytes, void* dk, void* dv, int B, int H, int N, int d,
                float scale, int causal, fa_dtype dtype, void* stream) {
  void* un = const_cast<void*>(kUnused);
  const BwdPtrs p{q, k, v, kUnused, dout, lse, un, dk, dv, const_cast<void*>(workspace)};
  int st = check_bwd(p, workspace_bytes, B, H, N, N, d, nullptr, nullptr, nullptr, scale, causal, (int)dtype);
  if (st != FA_OK) return st;
  return run_stages(bwd_problem(p, B, H, N, N, d, nullptr, nullptr, nullptr, scale, causal, (int)dtype), {1}, stream);
}

int fa_bwd_dq_rowsum(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     void* workspace, size_t workspace_bytes, void* dq, int B, int H, int N, int d, float scale,
                     int causal, fa_dtype dtype, void* stream) {
  void* un = const_cast<void*>(kUnused);
  const BwdPtrs p{q, k, v, o, dout, lse, dq, un, un, workspace};
  int st = check_bwd(p, workspace_bytes, B, H, N, N, d, nullptr, nullptr, nullptr, scale, causal, (int)dtype);
  if (st != FA_OK) return st;
  return run_stages(bwd_problem(p, B, H, N, N, d, nullptr, nullptr, nullptr, scale, causal, (int)dtype), {3}, stream);
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse, const void* workspace,
              size_t workspace_bytes, void* dq, int B, int H, int N, int d, float scale, int causal, fa_dtype dtype,
              void* stream) {
  void* un = const_cast<void*>(kUnused);
  const BwdPtrs p{q, k, v, kUnused, dout, lse, dq, un, un, const_cast<void*>(workspace)};
  int st = check_bwd(p, workspace_bytes, B, H, N, N, d, nullptr, nullptr, nullptr, scale, causal, (int)dtype);
  if (st != FA_OK) return st;
  return run_stages(bwd_problem(p, B, H, N, N, d, nullptr, nullptr, nullptr, scale, causal, (int)dtype), {2}, stream);
}

}  // extern "C"
