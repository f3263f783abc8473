// fa_launch.h -- internal interface between the C ABI and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// q, o: [B, H, Nq, d]; k, v: [B, H, Nk, d]; lse: [B, H, Nq].  seqlens_q /
// seqlens_k: optional device int32[B] sequence lengths (nullptr: Nq / Nk).
constexpr int kMaskBlock = 128;  // rows and keys per block of a block-sparse mask

struct FwdProblem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, Nq, Nk, d;
  const int* seqlens_q;
  const int* seqlens_k;
  // optional device uint8 [B, H, ceil(Nq/128), ceil(Nk/128)]: 0 removes the
  // scores of that (128-query block, 128-key block) pair (nullptr: dense)
  const unsigned char* block_mask;
  // dropout on the attention weights (drop_on = 0: none): keep when Philox
  // word >= drop_threshold, kept weights scaled by drop_scale = 1 / (1 - p)
  int drop_on;
  unsigned drop_threshold, drop_seed_lo, drop_seed_hi, drop_offset;
  float drop_scale;
  float scale;
  int causal;
  int dtype;  // 0 = fp32, 1 = fp16, 2 = bf16 (launch_fwd8: 8-bit inputs, bf16 o)
  float descale_v;  // launch_fwd8 only: o = (P v) * descale_v; scale already holds descale_q * descale_k
  int fp8_format;   // launch_fwd8 only: q, k, v codes are 0 = E4M3, 1 = E5M2
  // key splitting (16-bit only; splits <= 1: none): split s handles key tiles
  // [s * ceil(tiles / splits), ...) and writes fp32 partials into `part`
  // ([splits][B*H*Nq][d] outputs, then [splits][B*H*Nq] LSEs); a merge pass writes o / lse
  int splits;
  float* part;
};

struct BwdProblem {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;  // workspace: fp32 [B*H*Nq] row sums D_i
  int B, H, Nq, Nk, d;
  const int* seqlens_q;
  const int* seqlens_k;
  const unsigned char* block_mask;  // as in FwdProblem
  int drop_on;                      // as in FwdProblem
  unsigned drop_threshold, drop_seed_lo, drop_seed_hi, drop_offset;
  float drop_scale;
  float scale;
  int causal;
  int dtype;
  // launch_dq16 only: the dQ kernel also forms D from o and dout and writes it
  // to dvec, for the dK/dV stage that runs after it (no row-sum stage)
  int dq_rowsum;
};

hipError_t launch_fwd(const FwdProblem& p, hipStream_t s);
hipError_t launch_fwd16(const FwdProblem& p, hipStream_t s);  // bf16 / fp16 only
hipError_t launch_fwd16_128(const FwdProblem& p, hipStream_t s);  // d = 128 (fa_fwd16_d128.hip)
hipError_t launch_fwd8(const FwdProblem& p, hipStream_t s);   // E4M3 or E5M2 q, k, v; bf16 o; Nq = Nk, dense
// split keys (p.splits > 1, 16-bit): partials into p.part, then the merge into o / lse
hipError_t launch_decode(const FwdProblem& p, hipStream_t s);       // Nq == 1
hipError_t launch_split_merge(const FwdProblem& p, hipStream_t s);
// Capacity of the static device scratch that holds fa_bwd_static's row sums
// D (one fp32 per query row: B * H * N at most this).
constexpr long long kStaticScratchRows = 1LL << 22;
// That scratch's address on the device `stream` runs on (looked up once per
// device; allocates nothing).
hipError_t static_scratch(hipStream_t stream, float** out);
// stage: 0 = row sums D, 1 = dK/dV (reads D), 2 = dQ (reads D), 3 = dQ that
// forms and writes D itself (so the sequence 3, 1 is a whole backward pass)
hipError_t launch_bwd_stage(const BwdProblem& p, int stage, hipStream_t s);
hipError_t launch_dq16(const BwdProblem& p, hipStream_t s);    // bf16 / fp16 only
hipError_t launch_dkdv16(const BwdProblem& p, hipStream_t s);  // bf16 / fp16 only
// the dropout instantiations (fa_bwd16_drop.hip, a separate compilation unit)
hipError_t launch_dq16_drop(const BwdProblem& p, hipStream_t s);
hipError_t launch_dkdv16_drop(const BwdProblem& p, hipStream_t s);

}  // namespace fa
