// fa_bwd16.hip -- backward kernels for 16-bit I/O (bf16, fp16) on gfx950.
//
// Same algorithm and outputs as the generic backward (fa_bwd.hip): the score
// tiles are recomputed from Q, K and the forward's log-sum-exp, never stored
// ("How Flash Attention Works: Tiling, Softmax, GPU I/O", section "The
// Backward Pass: Recomputation Instead of Stored Activations"), and
//   P = exp(scale S - LSE), dP = dO V^T, dS = P (dP - D),
//   dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
// The 16-bit kernels use the machinery of the pipelined forward
// (fa_fwd16.hip): streamed tiles go straight from device memory into LDS with
// buffer loads, rows packed and chunk-permuted by Tile16::sw so row reads and
// transposing reads avoid bank conflicts, and the products of one tile are
// software-pipelined against the element-wise work of the next.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tile16.h"

namespace fa {

struct Bwd16Args {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;
  const float* dvec;
  const void* o;     // dQ kernel: non-null = form D from o and dout and write it to dvec_out
  float* dvec_out;
  void* dq;
  void* dk;
  void* dv;
  const int* seqlens_q;  // optional per-sequence lengths (device int32[B])
  const int* seqlens_k;
  const unsigned char* block_mask;  // block-sparse: [B, H, nbq, nbk] (SPARSE kernels only)
  int nbq, nbk;
  Dropout drop;                     // DROP kernels only
  int Nq, Nk, H;
  int nblk;
  int total;
  float c;      // scale * log2(e), signed
  float scale;
};

// Row-fragment reads kept in flight ahead of the S / dP products in the dQ
// kernels that carry dS into the next step (d = 64; d = 128 with dropout or a
// block mask: twelve of a 32-key half's sixteen) and in the d = 64 dK/dV
// kernel (all eight of a 32-query half).
constexpr int kBwdReadAhead = 12;

// Scheduling hint: NM matrix ops with R LDS reads each, the reads issued P
// matrix ops ahead of their use.
template <int NM, int R, int P>
__device__ inline void reads_ahead() {
  __builtin_amdgcn_sched_group_barrier(0x100, R * P, 0);
#pragma unroll
  for (int i = 0; i < NM - P; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, P, 0);
}

// --------------------------------------------------------------------------
// dQ: a workgroup owns 128 queries (32 per wave, Q and dO rows in VGPRs) and
// streams 64-key K/V tiles.  Step j computes S^T_j = K_j Q^T and
// dP^T_j = V_j dO^T, then forms dS^T_j while the matrix cores accumulate
// dQ^T += K_{j-1}^T dS^T_{j-1}.  LDS: K in three stages (K_{j-1}, K_j and the
// one being loaded), V in two.  Launched as the first backward stage, the
// kernel also forms the row sums D of its queries (it holds their dO rows
// already) and writes them for the dK/dV kernel.
// dQ kernel, dense d = 128 (no dropout, no block mask): two waves per SIMD
// (256 VGPRs each) with each tile's dQ products issued in its own step and no
// extra read-ahead schedule.  Carrying dS into the next step (the schedule of
// d = 64 and of the dropout / block-sparse kernels) needs ~300 VGPRs and so
// one wave per SIMD, which measured 9% slower on the c5 backward.
template <int D, bool SPARSE, bool DROP>
struct DqShape {
  static constexpr bool TWO = D == 128 && !SPARSE && !DROP;
  static constexpr int OCC = D == 64 || TWO ? 2 : 1;
  static constexpr int AHEAD = TWO ? 0 : kBwdReadAhead;
};

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
__global__ __launch_bounds__(256, (DqShape<D, SPARSE, DROP>::OCC)) void dq16_kernel(Bwd16Args a) {
  using M = Mma<T>;
  constexpr bool NOPIPE = DqShape<D, SPARSE, DROP>::TWO;
  constexpr int AHEAD = DqShape<D, SPARSE, DROP>::AHEAD;
  using TL = Tile16<D>;
  using Frag = typename M::Frag;
  constexpr int KSTEPS = D / 16;
  constexpr int MB = D / 32;
  // K stages: three when tile j-1's dQ products run in step j (K_{j-1}, K_j
  // and the one being loaded), two when each tile's dQ products finish in its
  // own step; V always two.  With two K stages every LDS offset of a step fits
  // a read instruction's 16-bit immediate at d = 128, which saves the address
  // registers that V's second stage would otherwise need.
  constexpr int KST = NOPIPE ? 2 : 3;
  constexpr int KREG = 0;                // [K0 K1 (K2) V0 V1]
  constexpr int VREG = KST * TL::BYTES;

  __shared__ __attribute__((aligned(1024))) char smem[(KST + 2) * TL::BYTES];

  const int tid = thread_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int Nq = a.Nq, Nk = a.Nk;

  int bh, qb;
  block_order<32 * DqShape<D, SPARSE, DROP>::OCC>(block_id(), a.total, a.nblk, CAUSAL, &bh, &qb);
  if (CAUSAL) qb = a.nblk - 1 - qb;
  const int q0 = qb * 128;
  const int qw = q0 + wave * 32;
  const Seq sq = seq_of(a.seqlens_q, a.seqlens_k, bh / a.H, Nq, Nk);
  const size_t headq = (size_t)bh * (size_t)Nq * D, headk = (size_t)bh * (size_t)Nk * D;
  const T* __restrict__ Q = reinterpret_cast<const T*>(a.q) + headq;
  const T* __restrict__ dO = reinterpret_cast<const T*>(a.dout) + headq;
  const char* Kg = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.k) + headk);
  const char* Vg = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.v) + headk);

  const int myq = qw + col;
  Frag qf[KSTEPS], dof[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    qf[ks] = myq < sq.lq ? row_frag<T>(Q + (size_t)myq * D + ks * 16, h) : zero_frag<T>();
    dof[ks] = myq < sq.lq ? row_frag<T>(dO + (size_t)myq * D + ks * 16, h) : zero_frag<T>();
  }
  const float lse2 = myq < sq.lq ? a.lse[(size_t)bh * Nq + myq] * kLog2e : 0.0f;
  float dd;
  if (a.o != nullptr) {
    // D = rowsum(dO o O) of the lane's query from its dO fragments and the
    // matching halves of its O row (the two half-waves hold the two halves),
    // written for the dK/dV kernel that runs after this one
    float part = 0.0f;
    if (myq < sq.lq) {
      const T* O = reinterpret_cast<const T*>(a.o) + headq + (size_t)myq * D;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const Frag of = row_frag<T>(O + ks * 16, h);
#pragma unroll
        for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)of[e], (float)dof[ks][e], part);
      }
    }
    dd = halves_sum(part);
    if (h == 0 && myq < Nq) a.dvec_out[(size_t)bh * Nq + myq] = dd;
  } else {
    dd = myq < sq.lq ? a.dvec[(size_t)bh * Nq + myq] : 0.0f;
  }

  // key tiles this block visits, and how many leading ones no real row sees masked
  int nt, nt_full;
  query_block_tiles<CAUSAL, 64>(sq, q0, 128, &nt, &nt_full);
  const int lim = key_limit<CAUSAL>(sq, myq);
  const int wlast = qw + 31 + sq.off;  // causal: the last key any row of this wave may see
  // block-sparse: this query block's mask row, packed into bits in LDS; a key
  // tile is live unless its 128-key block is masked out
  __shared__ uint64_t mwords[SPARSE ? kMaxMaskWords : 1];
  if constexpr (SPARSE) {
    pack_mask_words(mwords, a.block_mask + ((size_t)bh * a.nbq + qb) * a.nbk, a.nbk, 1, lane, wave, 4);
    __syncthreads();
  }

  uint32_t goff[TL::ROUNDS];
  tile16_load_offsets<D>(goff, wave, lane);
  auto dma = [&](const char* g, int row0, int region) __attribute__((always_inline)) {
    const auto rs = buffer_rsrc(g + (size_t)row0 * TL::ROWB, tile_bytes(sq.lk - row0, 64, TL::ROWB));
#pragma unroll
    for (int i = 0; i < TL::ROUNDS; ++i) lds_load16(rs, smem + region + (i * 4 + wave) * 1024, goff[i]);
  };

  uint32_t krow[KSTEPS], vrow[KSTEPS], ktr[MB][2];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    krow[ks] = KREG + tile16_row_addr<D>(col, ks, h);
    vrow[ks] = VREG + tile16_row_addr<D>(col, ks, h);
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) ktr[mb][hf] = KREG + tile16_tr_addr<D>(lane, mb, hf);

  f32x16 dqacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) dqacc[mb] = f32x16{};
  Frag dsf[2][2];  // dS^T of the previous tile, [32-key block][k-step]
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t) dsf[kb][t] = zero_frag<T>();
  const float c = a.c;

  auto dq_prev = [&](auto kps) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          dqacc[mb] = M::mma(tile16_tr_frag<T, D>(smem, ktr[mb][0], ktr[mb][1], kps * TL::BYTES + (32 * kb + 16 * t) * TL::ROWB),
                             dsf[kb][t], dqacc[mb]);
  };

  // Step j (jp: the tile visited before it, jn: the one after; j - 1 and j + 1
  // unless block sparsity skips tiles): K_j in K stage ks3, V_j in V stage vs2,
  // K_jp in the K stage before ks3.  Stages advance by one per step.
  auto step = [&](int j, int jn, int jp, auto ks3, auto vs2, auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int kps = ks3 == 0 ? KST - 1 : ks3 - 1;
    wait_vmem();
    __builtin_amdgcn_s_barrier();
    if (jn < nt) {
      const int kn = ks3 == KST - 1 ? 0 : ks3 + 1;
      dma(Kg, 64 * jn, KREG + kn * TL::BYTES);
      dma(Vg, 64 * jn, VREG + (vs2 ^ 1) * TL::BYTES);
    }
    const int k0 = 64 * j;
    const bool act = FULL || !CAUSAL || k0 <= wlast;
    const bool prev = FULL || (jp >= 0 && (!CAUSAL || 64 * jp <= wlast));
    if (act) {
      const int t0 = lim - k0 - 4 * h;
      // the two 32-key halves one after the other keeps two accumulators live, not four
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        __builtin_amdgcn_s_setprio(1);
        f32x16 s = f32x16{}, p = f32x16{};
        const int ko = ks3 * TL::BYTES + kb * 32 * TL::ROWB, vo = vs2 * TL::BYTES + kb * 32 * TL::ROWB;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          s = M::mma(tile16_row_frag<T>(smem, krow[ks] + ko), qf[ks], s);
          p = M::mma(tile16_row_frag<T>(smem, vrow[ks] + vo), dof[ks], p);
        }
        if constexpr (AHEAD > 0) reads_ahead<2 * KSTEPS, 1, (AHEAD > 0 ? AHEAD : 1)>();
        __builtin_amdgcn_s_setprio(0);
        if (!NOPIPE && kb == 0 && prev) dq_prev(kps);
        const int tk = t0 - 32 * kb;
        // dropout: dP of a dropped weight is 0, of a kept one dP / (1 - p)
        u32x4v w[4];
        if constexpr (DROP) {
#pragma unroll
          for (int g = 0; g < 4; ++g) w[g] = a.drop.words((k0 + 32 * kb + 8 * g + 4 * h) >> 2, myq, bh);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = fast_exp2(__builtin_fmaf(s[r], c, -lse2));
          if constexpr (!FULL) {
            const int ro = 8 * (r >> 2) + (r & 3);
            e = ro <= tk ? e : 0.0f;
          }
          if constexpr (DROP)
            p[r] = e * ((w[r >> 2][r & 3] >= a.drop.threshold ? p[r] * a.drop.scale : 0.0f) - dd);
          else
            p[r] = e * (p[r] - dd);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) dsf[kb][t] = acc_frag<T>(p, t);
      }
      if (NOPIPE) dq_prev(ks3);
    } else if (!NOPIPE && prev) {
      dq_prev(kps);
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if constexpr (!SPARSE) {
    if (nt > 0) {  // (nt is block-uniform: every wave takes the same barriers)
      dma(Kg, 0, KREG);
      dma(Vg, 0, VREG);
      // tile 0 owes no dQ product yet: generic step
      step(0, 1, -1, 0, 0, std::false_type{});
      int j = 1;
      // mask-free steps, six at a time so that every LDS offset is a constant.
      // Only where two waves share a SIMD (256 VGPRs): with the offsets as
      // runtime values those kernels spill.  One-wave kernels (d = 128 with
      // dropout) take the runtime-stage loop below, which keeps one register
      // assignment for the accumulators and lets the LDS reads run ahead.
      constexpr bool UNROLL6 = DqShape<D, SPARSE, DROP>::OCC == 2;
      // (j starts at 1: K stages j % KST = 1, 2, 0, 1, 2, 0 or 1, 0, 1, 0, 1, 0)
      using K2 = std::conditional_t<KST == 2, I0, I2>;
      using K0 = std::conditional_t<KST == 2, I1, I0>;
      using K1 = std::conditional_t<KST == 2, I0, I1>;
      using K2b = std::conditional_t<KST == 2, I1, I2>;
      for (; UNROLL6 && j + 5 < nt_full; j += 6) {
        step(j, j + 1, j - 1, I1{}, I1{}, std::true_type{});
        step(j + 1, j + 2, j, K2{}, I0{}, std::true_type{});
        step(j + 2, j + 3, j + 1, K0{}, I1{}, std::true_type{});
        step(j + 3, j + 4, j + 2, K1{}, I0{}, std::true_type{});
        step(j + 4, j + 5, j + 3, K2b{}, I1{}, std::true_type{});
        step(j + 5, j + 6, j + 4, I0{}, I0{}, std::true_type{});
      }
      // the rest (up to five mask-free tiles, then the masked ones): runtime stages
      for (; j < nt; ++j) {
        if (j < nt_full)
          step(j, j + 1, j - 1, j % KST, j & 1, std::true_type{});
        else
          step(j, j + 1, j - 1, j % KST, j & 1, std::false_type{});
      }
      wait_vmem();
      __builtin_amdgcn_s_barrier();
      if (!NOPIPE && (!CAUSAL || 64 * (nt - 1) <= wlast)) dq_prev((nt - 1) % KST);
    }
  } else {
    // Only live tiles are visited, in increasing order; step t uses K stage
    // t % KST and V stage t % 2, and is unmasked when its tile lies below nt_full.
    auto next = [&](int j) __attribute__((always_inline)) { return next_live_tile(mwords, j, 2, a.nbk, nt); };
    int j = next(-1);
    if (j < nt) {
      dma(Kg, 64 * j, KREG);
      dma(Vg, 64 * j, VREG);
      int jn = next(j);
      step(j, jn, -1, 0, 0, std::false_type{});
      int jp = j, t = 1;
      j = jn;
      // unmasked tiles (below nt_full) come first in the walk: two loops, so
      // that no loop holds both step bodies
      for (; j < nt_full; ++t) {
        jn = next(j);
        step(j, jn, jp, t % KST, t & 1, std::true_type{});
        jp = j;
        j = jn;
      }
      for (; j < nt; ++t) {
        jn = next(j);
        step(j, jn, jp, t % KST, t & 1, std::false_type{});
        jp = j;
        j = jn;
      }
      wait_vmem();
      __builtin_amdgcn_s_barrier();
      if (!NOPIPE && (!CAUSAL || 64 * jp <= wlast)) dq_prev((t - 1) % KST);
    }
  }

  if (myq < Nq) {  // padding rows store zeros
    T* row = reinterpret_cast<T*>(a.dq) + headq + (size_t)myq * D;
    const bool real = myq < sq.lq;
    const float sc = a.scale;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mb + 8 * g + 4 * h;
        float q4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) q4[u] = real ? dqacc[mb][4 * g + u] * sc : 0.0f;
        store4<T>(row + d0, q4[0], q4[1], q4[2], q4[3]);
      }
  }
}

// --------------------------------------------------------------------------
// dK, dV at d = 64 (d = 128: dkdv16n_kernel, dkdv32s_kernel): a workgroup owns 128
// keys (32 per wave; K and V rows in VGPRs as the stationary B operands) and
// streams 64-query tiles of Q and dO, with the query rows' LSE (pre-scaled to
// log2 units) and D, through LDS.  Per 32-query half: S = Q K^T and
// dP = dO V^T, then P and dS element-wise, then dV^T += dO^T P and
// dK^T += Q^T dS with the transposing reads of dO and Q.  Without dropout the
// kernel fits 256 VGPRs with no spills, so two waves share each SIMD
// (measured 1.5x faster than one); the dropout instantiations would spill at
// 256 and run one wave per SIMD.
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
__global__ __launch_bounds__(256, DROP ? 1 : 2) void dkdv16_kernel(Bwd16Args a) {
  static_assert(D == 64, "d = 128 has its own kernel");
  using M = Mma<T>;
  using TL = Tile16<D>;
  using Frag = typename M::Frag;
  constexpr int KSTEPS = D / 16;
  constexpr int MB = D / 32;
  constexpr int QREG = 0;                  // [Q0 Q1 dO0 dO1 lse0 lse1 D0 D1]
  constexpr int OREG = 2 * TL::BYTES;
  constexpr int LREG = 4 * TL::BYTES;      // 2 x 64 floats of -LSE * log2(e)
  constexpr int DREG = LREG + 512;         // 2 x 64 floats of D

  __shared__ __attribute__((aligned(1024))) char smem[4 * TL::BYTES + 1024];

  const int tid = thread_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int Nq = a.Nq, Nk = a.Nk;

  int bh, kblk;  // under the causal mask key block 0 is seen by the most query tiles
  block_order<(DROP ? 32 : 64)>(block_id(), a.total, a.nblk, CAUSAL, &bh, &kblk);
  const int kb0 = kblk * 128;
  const int kw = kb0 + 32 * wave;
  const Seq sq = seq_of(a.seqlens_q, a.seqlens_k, bh / a.H, Nq, Nk);
  const size_t headq = (size_t)bh * (size_t)Nq * D, headk = (size_t)bh * (size_t)Nk * D;
  const char* Qg = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.q) + headq);
  const char* Og = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.dout) + headq);
  const float* lse = a.lse + (size_t)bh * Nq;
  const float* dvec = a.dvec + (size_t)bh * Nq;

  const int mykey = kw + col;
  Frag kf[KSTEPS], vf[KSTEPS];
  {
    const T* Kp = reinterpret_cast<const T*>(a.k) + headk;
    const T* Vp = reinterpret_cast<const T*>(a.v) + headk;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      kf[ks] = mykey < sq.lk ? row_frag<T>(Kp + (size_t)mykey * D + ks * 16, h) : zero_frag<T>();
      vf[ks] = mykey < sq.lk ? row_frag<T>(Vp + (size_t)mykey * D + ks * 16, h) : zero_frag<T>();
    }
  }

  // query tiles of real queries; under the causal mask key j is first seen by
  // query j - off.  A block of padding keys visits none.
  const int nt = kb0 < sq.lk ? (sq.lq + 63) / 64 : 0;
  int first = 0, full0 = 0;
  if (CAUSAL) {
    const int f = floor_div(kb0 - sq.off, 64);
    first = f > 0 ? f : 0;
    // query tiles every wave sees unmasked: [full0, full1); the block's last
    // key kb0 + 127 is seen by every query from kb0 + 127 - off on
    const int g = floor_div(kb0 + 127 - sq.off + 63, 64);
    full0 = g > first ? g : first;
  }
  const int full1 = sq.lq / 64;
  // block-sparse: this key block's mask column, packed into bits in LDS; a
  // query tile is live unless its 128-row block is masked out
  __shared__ uint64_t mwords[SPARSE ? kMaxMaskWords : 1];
  if constexpr (SPARSE) {
    pack_mask_words(mwords, a.block_mask + (size_t)bh * a.nbq * a.nbk + kblk, a.nbq, a.nbk, lane, wave, 4);
    __syncthreads();
  }

  uint32_t goff[TL::ROUNDS];
  tile16_load_offsets<D>(goff, wave, lane);
  float lse_next = 0.0f, d_next = 0.0f;  // wave 0 stages the next tile's per-row values
  auto fetch = [&](int i, int stage) __attribute__((always_inline)) {
    const int row0 = 64 * i;
    const auto rq = buffer_rsrc(Qg + (size_t)row0 * TL::ROWB, tile_bytes(sq.lq - row0, 64, TL::ROWB));
    const auto ro = buffer_rsrc(Og + (size_t)row0 * TL::ROWB, tile_bytes(sq.lq - row0, 64, TL::ROWB));
#pragma unroll
    for (int r = 0; r < TL::ROUNDS; ++r) {
      lds_load16(rq, smem + QREG + stage * TL::BYTES + (r * 4 + wave) * 1024, goff[r]);
      lds_load16(ro, smem + OREG + stage * TL::BYTES + (r * 4 + wave) * 1024, goff[r]);
    }
    if (wave == 0) {
      const int qi = row0 + lane;
      lse_next = qi < sq.lq ? -lse[qi] * kLog2e : 0.0f;
      d_next = qi < sq.lq ? dvec[qi] : 0.0f;
    }
  };
  auto publish = [&](int stage) __attribute__((always_inline)) {  // wave 0 writes the staged per-row values
    if (wave == 0) {
      reinterpret_cast<float*>(smem + LREG)[stage * 64 + lane] = lse_next;
      reinterpret_cast<float*>(smem + DREG)[stage * 64 + lane] = d_next;
    }
  };

  uint32_t qrow[KSTEPS], qtr[MB][2];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) qrow[ks] = tile16_row_addr<D>(col, ks, h);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) qtr[mb][hf] = tile16_tr_addr<D>(lane, mb, hf);

  f32x16 dkacc[MB], dvacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    dkacc[mb] = f32x16{};
    dvacc[mb] = f32x16{};
  }
  const float c = a.c;

  // Step i: query tile i in stage st; the next tile to visit, in (i + 1 unless
  // block sparsity skips tiles), is fetched into st ^ 1.
  auto step = [&](int i, int in, auto st, auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    wait_vmem();
    publish(st);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // LDS writes done (lgkmcnt(0))
    __builtin_amdgcn_s_barrier();
    if (in < nt) fetch(in, st ^ 1);
    const int i0 = 64 * i;
    if (!FULL && CAUSAL && i0 + 63 + sq.off < kw) return;  // no query of the tile sees this wave's keys
    const int qo = QREG + st * TL::BYTES, oo = OREG + st * TL::BYTES;
    const float* lt = reinterpret_cast<const float*>(smem + LREG) + st * 64;
    const float* dt = reinterpret_cast<const float*>(smem + DREG) + st * 64;
    Frag pf[2][2], sf[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        s = M::mma(tile16_row_frag<T>(smem, qrow[ks] + qo + 32 * qb * TL::ROWB), kf[ks], s);
        dp = M::mma(tile16_row_frag<T>(smem, qrow[ks] + oo + 32 * qb * TL::ROWB), vf[ks], dp);
      }
      reads_ahead<2 * KSTEPS, 1, kBwdReadAhead>();
      // rows of s / dp: queries i0 + 32 qb + acc_row(r, h); column: key mykey
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int rr = 32 * qb + 8 * g + 4 * h;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lt + rr);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dt + rr);
        // dropout keep bits of queries i0 + rr .. + 3 against this lane's key
        const uint32_t kbits = DROP ? a.drop.quad_keep(mykey >> 2, i0 + rr, bh, col & 3) : 0u;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * g + u;
          float p = fast_exp2(__builtin_fmaf(s[r], c, l4[u]));
          if constexpr (!FULL) {
            const int qi = i0 + rr + u;
            p = (qi < sq.lq && (!CAUSAL || mykey <= qi + sq.off)) ? p : 0.0f;
          }
          if constexpr (DROP) {
            // dropout: dV takes the kept weights (1 / (1 - p) applied at the
            // store); dP of a dropped weight is 0, of a kept one dP / (1 - p)
            const bool kp = (kbits >> (4 * u)) & 1u;
            s[r] = kp ? p : 0.0f;
            dp[r] = p * ((kp ? dp[r] * a.drop.scale : 0.0f) - d4[u]);
          } else {
            s[r] = p;
            dp[r] = p * (dp[r] - d4[u]);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        pf[qb][t] = acc_frag<T>(s, t);
        sf[qb][t] = acc_frag<T>(dp, t);
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int off = (32 * qb + 16 * t) * TL::ROWB;
          dvacc[mb] = M::mma(tile16_tr_frag<T, D>(smem, qtr[mb][0] + oo, qtr[mb][1] + oo, off), pf[qb][t], dvacc[mb]);
          dkacc[mb] = M::mma(tile16_tr_frag<T, D>(smem, qtr[mb][0] + qo, qtr[mb][1] + qo, off), sf[qb][t], dkacc[mb]);
        }
  };

  if constexpr (!SPARSE) {
    if (first < nt) {
      fetch(first, 0);
      // The LDS stage alternates with the tile; it is a runtime value here.
      // With compile-time stages (two steps per iteration) the compiler kept
      // the dK/dV accumulators in two alternating register sets and, short of
      // registers, issued every LDS read just before its product; one step
      // per iteration keeps one assignment and lets the reads run ahead.
      int i = first;
      for (; i < nt && i < full0; ++i) step(i, i + 1, (i - first) & 1, std::false_type{});
      for (; i < full1; ++i) step(i, i + 1, (i - first) & 1, std::true_type{});
      for (; i < nt; ++i) step(i, i + 1, (i - first) & 1, std::false_type{});
    }
  } else {
    // Only live query tiles are visited, in increasing order, alternating
    // stages; a step is unmasked when its tile lies in [full0, full1).  As in
    // the dense loops, the stage is a runtime value and masked and unmasked
    // tiles run in loops of their own (one loop holding both step bodies
    // made the compiler shuffle the accumulators between register sets).
    auto next = [&](int i) __attribute__((always_inline)) { return next_live_tile(mwords, i, 2, a.nbq, nt); };
    int i = live_tile_from(mwords, first, 2, a.nbq, nt);
    if (i < nt) {
      fetch(i, 0);
      int st = 0;
      for (; i < nt && i < full0; st ^= 1) {
        const int in = next(i);
        step(i, in, st, std::false_type{});
        i = in;
      }
      for (; i < full1; st ^= 1) {
        const int in = next(i);
        step(i, in, st, std::true_type{});
        i = in;
      }
      for (; i < nt; st ^= 1) {
        const int in = next(i);
        step(i, in, st, std::false_type{});
        i = in;
      }
    }
  }

  if (mykey < Nk) {  // padding keys store zeros
    T* dkrow = reinterpret_cast<T*>(a.dk) + headk + (size_t)mykey * D;
    T* dvrow = reinterpret_cast<T*>(a.dv) + headk + (size_t)mykey * D;
    const bool real = mykey < sq.lk;
    const float sc = a.scale;
    const float sv = DROP ? a.drop.scale : 1.0f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mb + 8 * g + 4 * h;
        float k4[4], v4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          k4[u] = real ? dkacc[mb][4 * g + u] * sc : 0.0f;
          v4[u] = real ? dvacc[mb][4 * g + u] * sv : 0.0f;
        }
        store4<T>(dkrow + d0, k4[0], k4[1], k4[2], k4[3]);
        store4<T>(dvrow + d0, v4[0], v4[1], v4[2], v4[3]);
      }
  }
}

// --------------------------------------------------------------------------
// dK, dV at d = 128 with a block mask or dropout (without either,
// dkdv32s_kernel below): each wave owns 16 keys, so that two waves share each
// SIMD.  With 32 keys per wave (the layout of
// dkdv16_kernel) the d = 128 dK/dV accumulators and stationary K/V fragments
// alone would take 192 registers, leaving one wave per SIMD; with 16 keys
// they take 96.
// WAVES = 8 (no causal mask): one workgroup of 128 keys per CU.  WAVES = 4
// (causal mask): two workgroups of 64 keys per CU, whose waves pair up on the
// SIMDs out of step with each other, so one's element-wise work meets the
// other's products; that measured 3-10% faster under the mask (the causal
// grid's many short blocks) and 2.4% slower without it (each Q/dO tile is
// streamed by twice as many workgroups).  The products run on the 16x16x32
// instruction (the same rate per flop).  Per 32-query half and wave:
// S = Q K^T and dP = dO V^T (two 16-query blocks, four 32-channel steps),
// then dV^T += dO^T P and dK^T += Q^T dS (eight 16-channel blocks, the 32
// queries as one contraction step).  P and dS go from the accumulators
// straight into the B operand: a lane holds its key's weights for queries
// 16 b + 4 g + r (g = lane / 16, b = query block, r = register), which become
// contraction slot 8 g + 4 b + r, and the transposing reads of dO and Q hand
// the A operand the same queries in the same slots.  The Q and dO tiles keep
// their 16-byte chunks permuted by Tile16n::sw, under which both read
// patterns are conflict-free on gfx950, where a 16-byte read is served in
// four passes of the 16 lanes that agree in lane bits 2 and 4, and an 8-byte
// read in two passes of 32 consecutive lanes (inferred from bank-conflict
// counts of isolated read patterns): the row fragments (one chunk of 16
// consecutive rows per 16 lanes) and the transposing reads (two adjacent
// chunks of 8 consecutive rows per 32 lanes).
// Operand reads kept in flight ahead of the 16x16x32 products: row fragments
// of S / dP, and transposing pairs of dV / dK.
constexpr int kNarrowRowAhead = 8;
constexpr int kNarrowTrAhead = 4;

struct Tile16n {
  static constexpr int ROWB = 256;    // one row of 128 16-bit values
  static constexpr int BYTES = 64 * ROWB;
  __device__ static constexpr int sw(int r) { return (r ^ (r << 1)) & 15; }
  __device__ static constexpr int phys(int r, int chunk) { return r * ROWB + ((chunk ^ sw(r)) << 4); }
};

template <typename T, bool CAUSAL, bool SPARSE, bool DROP, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void dkdv16n_kernel(Bwd16Args a) {
  using M = Mma16<T>;
  using Frag = typename M::Frag;
  using TL = Tile16n;
  constexpr int D = 128;
  constexpr int KEYS = 16 * WAVES;       // keys per workgroup
  constexpr int ROUNDS = TL::BYTES / (1024 * WAVES);  // direct loads per tile and wave
  constexpr int KS = D / 32;             // contraction steps of S and dP
  constexpr int NB = D / 16;             // 16-channel blocks of dK^T and dV^T
  constexpr int QREG = 0;                // [Q0 Q1 dO0 dO1 lse0 lse1 D0 D1]
  constexpr int OREG = 2 * TL::BYTES;
  constexpr int LREG = 4 * TL::BYTES;    // 2 x 64 floats of -LSE * log2(e)
  constexpr int DREG = LREG + 512;       // 2 x 64 floats of D

  __shared__ __attribute__((aligned(1024))) char smem[4 * TL::BYTES + 1024];

  const int tid = thread_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, col = lane & 15;
  const int Nq = a.Nq, Nk = a.Nk;

  int bh, kblk;  // under the causal mask key block 0 is seen by the most query tiles
  block_order<32 * (8 / WAVES)>(block_id(), a.total, a.nblk, CAUSAL, &bh, &kblk);
  const int kb0 = kblk * KEYS;
  const int kw = kb0 + 16 * wave;
  const Seq sq = seq_of(a.seqlens_q, a.seqlens_k, bh / a.H, Nq, Nk);
  const size_t headq = (size_t)bh * (size_t)Nq * D, headk = (size_t)bh * (size_t)Nk * D;
  const char* Qg = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.q) + headq);
  const char* Og = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.dout) + headq);
  const float* lse = a.lse + (size_t)bh * Nq;
  const float* dvec = a.dvec + (size_t)bh * Nq;

  // B operands of S and dP: the lane's key, channels 32 ks + 8 g .. + 7
  const int mykey = kw + col;
  Frag kf[KS], vf[KS];
  {
    const T* Kp = reinterpret_cast<const T*>(a.k) + headk + (size_t)mykey * D + 8 * g;
    const T* Vp = reinterpret_cast<const T*>(a.v) + headk + (size_t)mykey * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = mykey < sq.lk ? __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(Kp + 32 * ks)) : zero_frag<T>();
      vf[ks] = mykey < sq.lk ? __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(Vp + 32 * ks)) : zero_frag<T>();
    }
  }

  // query tiles of real queries (a block of padding keys visits none), as in
  // dkdv16_kernel: under the causal mask key kb0 is first seen by query
  // kb0 - off, and every query from kb0 + KEYS - 1 - off on sees all keys
  const int nt = kb0 < sq.lk ? (sq.lq + 63) / 64 : 0;
  int first = 0, full0 = 0;
  if (CAUSAL) {
    const int f = floor_div(kb0 - sq.off, 64);
    first = f > 0 ? f : 0;
    const int gq = floor_div(kb0 + KEYS - 1 - sq.off + 63, 64);
    full0 = gq > first ? gq : first;
  }
  const int full1 = sq.lq / 64;
  // block-sparse: the 128-key mask column of this workgroup's keys, packed
  // into bits in LDS; a query tile is live unless its 128-row block is masked out
  __shared__ uint64_t mwords[SPARSE ? kMaxMaskWords : 1];
  if constexpr (SPARSE) {
    pack_mask_words(mwords, a.block_mask + (size_t)bh * a.nbq * a.nbk + (kb0 >> 7), a.nbq, a.nbk, lane, wave, WAVES);
    __syncthreads();
  }

  // direct loads: slot s = (WAVES r + wave) * 64 + lane, 16 bytes at LDS byte
  // 16 s, holds logical chunk (s % 16) ^ sw(row) of row s / 16
  uint32_t goff[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int sl = (r * WAVES + wave) * 64 + lane;
    const int row = sl >> 4, pc = sl & 15;
    goff[r] = row * TL::ROWB + ((pc ^ TL::sw(row)) << 4);
  }
  float lse_next = 0.0f, d_next = 0.0f;  // wave 0 stages the next tile's per-row values
  auto fetch = [&](int i, int stage) __attribute__((always_inline)) {
    const int row0 = 64 * i;
    const auto rq = buffer_rsrc(Qg + (size_t)row0 * TL::ROWB, tile_bytes(sq.lq - row0, 64, TL::ROWB));
    const auto ro = buffer_rsrc(Og + (size_t)row0 * TL::ROWB, tile_bytes(sq.lq - row0, 64, TL::ROWB));
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      lds_load16(rq, smem + QREG + stage * TL::BYTES + (r * WAVES + wave) * 1024, goff[r]);
      lds_load16(ro, smem + OREG + stage * TL::BYTES + (r * WAVES + wave) * 1024, goff[r]);
    }
    if (wave == 0) {
      const int qi = row0 + lane;
      lse_next = qi < sq.lq ? -lse[qi] * kLog2e : 0.0f;
      d_next = qi < sq.lq ? dvec[qi] : 0.0f;
    }
  };
  auto publish = [&](int stage) __attribute__((always_inline)) {
    if (wave == 0) {
      reinterpret_cast<float*>(smem + LREG)[stage * 64 + lane] = lse_next;
      reinterpret_cast<float*>(smem + DREG)[stage * 64 + lane] = d_next;
    }
  };

  // A operands.  Row fragments of S and dP: query 16 b + col, chunk 4 ks + g.
  // Transposing reads of dV^T and dK^T: lane (g, col) points at query row
  // 4 g + col / 4 (+ 16 for slots 4 .. 7), channels 16 nb + 4 (col % 4) .. + 3,
  // and receives channel 16 nb + col of queries 4 g + e.
  uint32_t qrow[KS], qtr[NB];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qrow[ks] = TL::phys(col, 4 * ks + g);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) qtr[nb] = TL::phys(4 * g + (col >> 2), 2 * nb + ((col & 3) >> 1)) + 8 * (col & 1);
  auto rowf = [&](uint32_t addr) __attribute__((always_inline)) {
    return __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(smem + addr));
  };
  auto trf = [&](uint32_t addr) __attribute__((always_inline)) {
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x4 lo = lds_tr16(smem + addr);
    const i16x4 hi = lds_tr16(smem + addr + 16 * TL::ROWB);
    const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(Frag, both);
  };

  f32x4 dkacc[NB], dvacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    dkacc[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    dvacc[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const float c = a.c;

  // Step i: query tile i in stage st; tile i + 1 is fetched into st ^ 1.
  auto step = [&](int i, int in, int st, auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    wait_vmem();
    publish(st);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // LDS writes done (lgkmcnt(0))
    __builtin_amdgcn_s_barrier();
    if (in < nt) fetch(in, st ^ 1);
    const int i0 = 64 * i;
    if (!FULL && CAUSAL && i0 + 63 + sq.off < kw) return;  // no query of the tile sees this wave's keys
    const int qo = QREG + st * TL::BYTES, oo = OREG + st * TL::BYTES;
    const float* lt = reinterpret_cast<const float*>(smem + LREG) + st * 64;
    const float* dt = reinterpret_cast<const float*>(smem + DREG) + st * 64;
#pragma unroll
    for (int hq = 0; hq < 2; ++hq) {
      f32x4 s[2], dp[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        s[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        dp[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const uint32_t ro = qrow[ks] + (32 * hq + 16 * b) * TL::ROWB;
          s[b] = M::mma(rowf(ro + qo), kf[ks], s[b]);
          dp[b] = M::mma(rowf(ro + oo), vf[ks], dp[b]);
        }
      // a 16-cycle product cannot hide an LDS read issued just before it
      reads_ahead<4 * KS, 1, kNarrowRowAhead>();
      // element-wise work at the higher issue priority: of the two waves on a
      // SIMD, the one in its product phase needs a slot once per product
      __builtin_amdgcn_s_setprio(1);
      Frag pf, sf;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int rr = 32 * hq + 16 * b + 4 * g;  // queries i0 + rr .. + 3 against this lane's key
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lt + rr);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dt + rr);
        // dropout keep bits of queries i0 + rr .. + 3 against this lane's key: a
        // DPP quad holds four consecutive keys against the same four queries
        const uint32_t kbits = DROP ? a.drop.quad_keep(mykey >> 2, i0 + rr, bh, col & 3) : 0u;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[b][r], c, l4[r]));
          if constexpr (!FULL) {
            const int qi = i0 + rr + r;
            p = (qi < sq.lq && (!CAUSAL || mykey <= qi + sq.off)) ? p : 0.0f;
          }
          if constexpr (DROP) {
            // dV takes the kept weights (1 / (1 - p) applied at the store); dP of
            // a dropped weight is 0, of a kept one dP / (1 - p)
            const bool kp = (kbits >> (4 * r)) & 1u;
            pf[4 * b + r] = (T)(kp ? p : 0.0f);
            sf[4 * b + r] = (T)(p * ((kp ? dp[b][r] * a.drop.scale : 0.0f) - d4[r]));
          } else {
            pf[4 * b + r] = (T)p;
            sf[4 * b + r] = (T)(p * (dp[b][r] - d4[r]));
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const uint32_t to = qtr[nb] + 32 * hq * TL::ROWB;
        dvacc[nb] = M::mma(trf(to + oo), pf, dvacc[nb]);
        dkacc[nb] = M::mma(trf(to + qo), sf, dkacc[nb]);
      }
      reads_ahead<2 * NB, 2, kNarrowTrAhead>();
    }
  };

  if constexpr (!SPARSE) {
    if (first < nt) {
      fetch(first, 0);
      int i = first;
      for (; i < nt && i < full0; ++i) step(i, i + 1, (i - first) & 1, std::false_type{});
      for (; i < full1; ++i) step(i, i + 1, (i - first) & 1, std::true_type{});
      for (; i < nt; ++i) step(i, i + 1, (i - first) & 1, std::false_type{});
    }
  } else {
    // only live query tiles, in increasing order, alternating stages; masked
    // and unmasked tiles in loops of their own, as in dkdv16_kernel
    auto next = [&](int i) __attribute__((always_inline)) { return next_live_tile(mwords, i, 2, a.nbq, nt); };
    int i = live_tile_from(mwords, first, 2, a.nbq, nt);
    if (i < nt) {
      fetch(i, 0);
      int st = 0;
      for (; i < nt && i < full0; st ^= 1) {
        const int in = next(i);
        step(i, in, st, std::false_type{});
        i = in;
      }
      for (; i < full1; st ^= 1) {
        const int in = next(i);
        step(i, in, st, std::true_type{});
        i = in;
      }
      for (; i < nt; st ^= 1) {
        const int in = next(i);
        step(i, in, st, std::false_type{});
        i = in;
      }
    }
  }

  if (mykey < Nk) {  // padding keys store zeros
    T* dkrow = reinterpret_cast<T*>(a.dk) + headk + (size_t)mykey * D;
    T* dvrow = reinterpret_cast<T*>(a.dv) + headk + (size_t)mykey * D;
    const bool real = mykey < sq.lk;
    const float sc = a.scale;
    const float sv = DROP ? a.drop.scale : 1.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int d0 = 16 * nb + 4 * g;  // rows 4 g .. + 3 of channel block nb
      float k4[4], v4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        k4[r] = real ? dkacc[nb][r] * sc : 0.0f;
        v4[r] = real ? dvacc[nb][r] * sv : 0.0f;
      }
      store4<T>(dkrow + d0, k4[0], k4[1], k4[2], k4[3]);
      store4<T>(dvrow + d0, v4[0], v4[1], v4[2], v4[3]);
    }
  }
}

// --------------------------------------------------------------------------
// dK, dV at d = 128 without block mask or dropout, with K and V resident in
// LDS: eight waves own 128 keys; wave w takes keys 32 (w % 4) .. + 31 against
// queries 32 (w / 4) .. + 31 of every 64-query tile, so each Q / dO row read
// serves the wave's two 16-key blocks and each K / V row read its two
// 16-query blocks.  Per wave and tile: 32 row reads and 32 transposing reads
// for 64 products, where the 16-key kernel needs 32 and 64: the LDS time per
// CU and tile falls from about 2650 to 1840 cycles (reads at 256 B/clk for
// 16-byte rows and 191 B/clk transposed, plus the tiles' direct writes)
// against 2048 matrix cycles per SIMD.  128 + 128 key rows and two Q / dO
// stages take 129 KiB, so one workgroup runs per CU, two waves per SIMD.  The
// two waves of a key group (w, w + 4) hold partial dK / dV over their query
// halves; at the end the second adds its partials into the first through LDS
// (a fixed order), and the first stores.  Measured against the 16-key kernel
// (best of 5, interleaved): c5 dK/dV 2-4% faster, B=1 H=8 N=32768 causal 8-9%,
// B=1 H=16 N=8192 non-causal 5%.  With a block mask (c5 shape, 50% kept) the
// whole backward ran 5% and with dropout 4% slower, so those keep the 16-key
// kernel: two workgroups per CU balance uneven blocks better and overlap the
// dropout generator's VALU work with the other workgroup's products.
template <typename T, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void dkdv32s_kernel(Bwd16Args a) {
  using M = Mma16<T>;
  using Frag = typename M::Frag;
  using TL = Tile16n;
  constexpr int D = 128;
  constexpr int WAVES = 8;
  constexpr int KEYS = 128;
  constexpr int KS = D / 32;
  constexpr int NB = D / 16;
  constexpr int KREG = 0;                 // K: 128 rows
  constexpr int VREG = 2 * TL::BYTES;     // V: 128 rows
  constexpr int QREG = 4 * TL::BYTES;     // Q0 Q1
  constexpr int OREG = 6 * TL::BYTES;     // dO0 dO1
  constexpr int LREG = 8 * TL::BYTES;     // 2 x 64 floats of -LSE * log2(e)
  constexpr int DREG = LREG + 512;        // 2 x 64 floats of D
  constexpr int QROUNDS = TL::BYTES / (1024 * WAVES);   // direct loads per 64-row tile and wave

  __shared__ __attribute__((aligned(1024))) char smem[8 * TL::BYTES + 1024];

  const int tid = thread_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3, qh = wave >> 2;
  const int g = lane >> 4, col = lane & 15;
  const int Nq = a.Nq, Nk = a.Nk;

  // Heads grouped for 128 workgroups per XCD although an XCD holds 32 of
  // these: with one workgroup per CU, a group sized to the XCD is one round of
  // the grid (c5: 8 heads x 32 blocks on 256 CUs), so each round mixed long
  // and short blocks and the next group's longest ones started late; wider
  // groups keep the longest-first order across rounds.  Measured (best of 7,
  // interleaved): c5 dK/dV +3.7 to +4.4%, B=1 H=16 N=8192 causal +1.6%, the
  // c2 shape +0.3 to +1.2%, long sequences unchanged.  (The two-workgroup
  // forward and dQ kernels gained nothing from wider groups.)
  int bh, kblk;
  block_order<128>(block_id(), a.total, a.nblk, CAUSAL, &bh, &kblk);
  const int kb0 = kblk * KEYS;
  const int kw = kb0 + 32 * kg;
  const Seq sq = seq_of(a.seqlens_q, a.seqlens_k, bh / a.H, Nq, Nk);
  const size_t headq = (size_t)bh * (size_t)Nq * D, headk = (size_t)bh * (size_t)Nk * D;
  const char* Qg = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.q) + headq);
  const char* Og = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.dout) + headq);
  const char* Kg = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.k) + headk);
  const char* Vg = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.v) + headk);
  const float* lse = a.lse + (size_t)bh * Nq;
  const float* dvec = a.dvec + (size_t)bh * Nq;

  const int nt = kb0 < sq.lk ? (sq.lq + 63) / 64 : 0;
  int first = 0, full0 = 0;
  if (CAUSAL) {
    const int f = floor_div(kb0 - sq.off, 64);
    first = f > 0 ? f : 0;
    const int gq = floor_div(kb0 + KEYS - 1 - sq.off + 63, 64);
    full0 = gq > first ? gq : first;
  }
  const int full1 = sq.lq / 64;

  // direct loads: slot s = (WAVES r + wave) * 64 + lane, 16 bytes at LDS byte
  // 16 s, holds logical chunk (s % 16) ^ sw(row) of row s / 16
  auto slot_off = [&](int r) __attribute__((always_inline)) {
    const int sl = (r * WAVES + wave) * 64 + lane;
    const int row = sl >> 4, pc = sl & 15;
    return (uint32_t)(row * TL::ROWB + ((pc ^ TL::sw(row)) << 4));
  };
  uint32_t goff[QROUNDS];
#pragma unroll
  for (int r = 0; r < QROUNDS; ++r) goff[r] = slot_off(r);
  if (first < nt) {  // K and V of the block's 128 keys, once
    const auto rk = buffer_rsrc(Kg + (size_t)kb0 * TL::ROWB, tile_bytes(sq.lk - kb0, KEYS, TL::ROWB));
    const auto rv = buffer_rsrc(Vg + (size_t)kb0 * TL::ROWB, tile_bytes(sq.lk - kb0, KEYS, TL::ROWB));
#pragma unroll
    for (int r = 0; r < 2 * QROUNDS; ++r) {
      lds_load16(rk, smem + KREG + (r * WAVES + wave) * 1024, slot_off(r));
      lds_load16(rv, smem + VREG + (r * WAVES + wave) * 1024, slot_off(r));
    }
  }
  float lse_next = 0.0f, d_next = 0.0f;  // wave 0 stages the next tile's per-row values
  auto fetch = [&](int i, int stage) __attribute__((always_inline)) {
    const int row0 = 64 * i;
    const auto rq = buffer_rsrc(Qg + (size_t)row0 * TL::ROWB, tile_bytes(sq.lq - row0, 64, TL::ROWB));
    const auto ro = buffer_rsrc(Og + (size_t)row0 * TL::ROWB, tile_bytes(sq.lq - row0, 64, TL::ROWB));
#pragma unroll
    for (int r = 0; r < QROUNDS; ++r) {
      lds_load16(rq, smem + QREG + stage * TL::BYTES + (r * WAVES + wave) * 1024, goff[r]);
      lds_load16(ro, smem + OREG + stage * TL::BYTES + (r * WAVES + wave) * 1024, goff[r]);
    }
    if (wave == 0) {
      const int qi = row0 + lane;
      lse_next = qi < sq.lq ? -lse[qi] * kLog2e : 0.0f;
      d_next = qi < sq.lq ? dvec[qi] : 0.0f;
    }
  };
  auto publish = [&](int stage) __attribute__((always_inline)) {
    if (wave == 0) {
      reinterpret_cast<float*>(smem + LREG)[stage * 64 + lane] = lse_next;
      reinterpret_cast<float*>(smem + DREG)[stage * 64 + lane] = d_next;
    }
  };

  // Row fragments: lane (g, col) reads row 16 blk + col, chunk 4 ks + g, of
  // the Q / dO tile (queries 32 qh + 16 b + col) or the K / V rows (keys
  // 32 kg + 16 kb + col).  Transposing reads of dO and Q as in dkdv16n_kernel.
  uint32_t qrow[KS], krow[KS], qtr[NB];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qrow[ks] = TL::phys(32 * qh + col, 4 * ks + g);
    krow[ks] = TL::phys(32 * kg + col, 4 * ks + g);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    qtr[nb] = TL::phys(32 * qh + 4 * g + (col >> 2), 2 * nb + ((col & 3) >> 1)) + 8 * (col & 1);
  auto rowf = [&](uint32_t addr) __attribute__((always_inline)) {
    return __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(smem + addr));
  };
  auto trf = [&](uint32_t addr) __attribute__((always_inline)) {
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x4 lo = lds_tr16(smem + addr);
    const i16x4 hi = lds_tr16(smem + addr + 16 * TL::ROWB);
    const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(Frag, both);
  };

  f32x4 dkacc[NB][2], dvacc[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      dkacc[nb][kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      dvacc[nb][kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  const float c = a.c;

  auto step = [&](int i, int in, int st, auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    wait_vmem();
    publish(st);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // LDS writes done (lgkmcnt(0))
    __builtin_amdgcn_s_barrier();
    if (in < nt) fetch(in, st ^ 1);
    const int i0 = 64 * i;
    const int qw0 = i0 + 32 * qh;  // this wave's first query of the tile
    if (!FULL && CAUSAL && qw0 + 31 + sq.off < kw) return;  // no query of this half sees the wave's keys
    const int qo = QREG + st * TL::BYTES, oo = OREG + st * TL::BYTES;
    const float* lt = reinterpret_cast<const float*>(smem + LREG) + st * 64;
    const float* dt = reinterpret_cast<const float*>(smem + DREG) + st * 64;
    f32x4 s[2][2], dp[2][2];  // [query block b][key block kb]
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[b][kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        dp[b][kb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      Frag qa[2], oa[2], kbf[2], vbf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        qa[u] = rowf(qrow[ks] + 16 * u * TL::ROWB + qo);
        oa[u] = rowf(qrow[ks] + 16 * u * TL::ROWB + oo);
        kbf[u] = rowf(krow[ks] + 16 * u * TL::ROWB + KREG);
        vbf[u] = rowf(krow[ks] + 16 * u * TL::ROWB + VREG);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[b][kb] = M::mma(qa[b], kbf[kb], s[b][kb]);
          dp[b][kb] = M::mma(oa[b], vbf[kb], dp[b][kb]);
        }
    }
    // reads 8 ahead of the S / dP products; the element-wise work at the
    // higher issue priority, as in dkdv16n_kernel
    reads_ahead<8 * KS, 1, 8>();
    __builtin_amdgcn_s_setprio(1);
    Frag pf[2], sf[2];  // [key block]
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int rr = 32 * qh + 16 * b + 4 * g;  // queries i0 + rr .. + 3
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(lt + rr);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(dt + rr);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = kw + 16 * kb + col;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[b][kb][r], c, l4[r]));
          if constexpr (!FULL) {
            const int qi = i0 + rr + r;
            p = (qi < sq.lq && (!CAUSAL || key <= qi + sq.off)) ? p : 0.0f;
          }
          pf[kb][4 * b + r] = (T)p;
          sf[kb][4 * b + r] = (T)(p * (dp[b][kb][r] - d4[r]));
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const Frag ot = trf(qtr[nb] + oo);
      const Frag qt = trf(qtr[nb] + qo);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        dvacc[nb][kb] = M::mma(ot, pf[kb], dvacc[nb][kb]);
        dkacc[nb][kb] = M::mma(qt, sf[kb], dkacc[nb][kb]);
      }
    }
    reads_ahead<4 * NB, 1, 8>();  // transposing reads 8 ahead (4: 1% slower)
  };

  if (first < nt) {
    fetch(first, 0);
    int i = first;
    for (; i < nt && i < full0; ++i) step(i, i + 1, (i - first) & 1, std::false_type{});
    for (; i < full1; ++i) step(i, i + 1, (i - first) & 1, std::true_type{});
    for (; i < nt; ++i) step(i, i + 1, (i - first) & 1, std::false_type{});
  }

  // the query-half-1 waves hand their partial sums to the half-0 waves of the
  // same keys through LDS (64 KiB per accumulator kind, reusing the tiles)
  wait_vmem();
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [kg][nb][kb][4 regs][64 lanes] x (dK, dV)
  constexpr int RED = 4 * NB * 2 * 4 * 64;      // floats per accumulator kind
  if (qh == 1) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int o = (((kg * NB + nb) * 2 + kb) * 4 + r) * 64 + lane;
          red[o] = dkacc[nb][kb][r];
          red[RED + o] = dvacc[nb][kb][r];
        }
  }
  __syncthreads();
  if (qh == 0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = kw + 16 * kb + col;
      if (key < Nk) {  // padding keys store zeros
        T* dkrow = reinterpret_cast<T*>(a.dk) + headk + (size_t)key * D;
        T* dvrow = reinterpret_cast<T*>(a.dv) + headk + (size_t)key * D;
        const bool real = key < sq.lk;
        const float sc = a.scale;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int d0 = 16 * nb + 4 * g;
          float k4[4], v4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int o = (((kg * NB + nb) * 2 + kb) * 4 + r) * 64 + lane;
            k4[r] = real ? (dkacc[nb][kb][r] + red[o]) * sc : 0.0f;
            v4[r] = real ? (dvacc[nb][kb][r] + red[RED + o]) : 0.0f;
          }
          store4<T>(dkrow + d0, k4[0], k4[1], k4[2], k4[3]);
          store4<T>(dvrow + d0, v4[0], v4[1], v4[2], v4[3]);
        }
      }
    }
  }
}

// Fill the kernel arguments shared by the dK/dV and dQ kernels; nblk is the
// number of owned 128-row blocks per (batch, head).
static Bwd16Args bwd16_args(const BwdProblem& p, int nblk) {
  Bwd16Args a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.dout = p.dout; a.lse = p.lse; a.dvec = p.dvec;
  a.o = p.dq_rowsum ? p.o : nullptr;
  a.dvec_out = p.dq_rowsum ? p.dvec : nullptr;
  a.dq = p.dq; a.dk = p.dk; a.dv = p.dv;
  a.seqlens_q = p.seqlens_q; a.seqlens_k = p.seqlens_k;
  a.block_mask = p.block_mask;
  a.nbq = (p.Nq + kMaskBlock - 1) / kMaskBlock;
  a.nbk = (p.Nk + kMaskBlock - 1) / kMaskBlock;
  a.drop = Dropout{p.drop_threshold, p.drop_seed_lo, p.drop_seed_hi, p.drop_offset, p.drop_scale};
  a.Nq = p.Nq; a.Nk = p.Nk; a.H = p.H;
  a.scale = p.scale;
  a.c = p.scale * kLog2e;
  a.nblk = nblk;
  a.total = a.nblk * p.B * p.H;
  return a;
}
static_assert(kMaskBlock == 128, "a dK/dV workgroup's 128 keys are one mask block column");

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
static hipError_t launch_dkdv16_t(const BwdProblem& p, hipStream_t stream) {
  if constexpr (D == 128 && !SPARSE && !DROP) {  // 32 keys per wave, K and V in LDS
    const Bwd16Args a = bwd16_args(p, (p.Nk + 127) / 128);
    hipLaunchKernelGGL((dkdv32s_kernel<T, CAUSAL>), dim3(a.total), dim3(512), 0, stream, a);
  } else if constexpr (D == 128) {  // 16 keys per wave
    constexpr int WAVES = CAUSAL ? 4 : 8;
    const Bwd16Args a = bwd16_args(p, (p.Nk + 16 * WAVES - 1) / (16 * WAVES));
    hipLaunchKernelGGL((dkdv16n_kernel<T, CAUSAL, SPARSE, DROP, WAVES>), dim3(a.total), dim3(64 * WAVES), 0, stream, a);
  } else {
    const Bwd16Args a = bwd16_args(p, (p.Nk + 127) / 128);
    hipLaunchKernelGGL((dkdv16_kernel<T, D, CAUSAL, SPARSE, DROP>), dim3(a.total), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

template <typename T, bool SPARSE, bool DROP>
static hipError_t launch_dkdv16_s(const BwdProblem& p, hipStream_t s) {
  if (p.d == 64)
    return p.causal ? launch_dkdv16_t<T, 64, true, SPARSE, DROP>(p, s) : launch_dkdv16_t<T, 64, false, SPARSE, DROP>(p, s);
  return p.causal ? launch_dkdv16_t<T, 128, true, SPARSE, DROP>(p, s)
                  : launch_dkdv16_t<T, 128, false, SPARSE, DROP>(p, s);
}

#ifndef FA_BWD16_DROPOUT_UNIT
// (block sparsity and dropout are not combined: the API rejects that)
template <typename T>
static hipError_t launch_dkdv16_d(const BwdProblem& p, hipStream_t s) {
  if (p.drop_on) return launch_dkdv16_drop(p, s);
  return p.block_mask ? launch_dkdv16_s<T, true, false>(p, s) : launch_dkdv16_s<T, false, false>(p, s);
}

hipError_t launch_dkdv16(const BwdProblem& p, hipStream_t s) {
  return p.dtype == 1 ? launch_dkdv16_d<_Float16>(p, s) : launch_dkdv16_d<__bf16>(p, s);
}
#else
hipError_t launch_dkdv16_drop(const BwdProblem& p, hipStream_t s) {
  return p.dtype == 1 ? launch_dkdv16_s<_Float16, false, true>(p, s) : launch_dkdv16_s<__bf16, false, true>(p, s);
}
#endif

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
static hipError_t launch_dq16_t(const BwdProblem& p, hipStream_t stream) {
  const Bwd16Args a = bwd16_args(p, (p.Nq + 127) / 128);
  hipLaunchKernelGGL((dq16_kernel<T, D, CAUSAL, SPARSE, DROP>), dim3(a.total), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename T, bool SPARSE, bool DROP>
static hipError_t launch_dq16_s(const BwdProblem& p, hipStream_t s) {
  if (p.d == 64)
    return p.causal ? launch_dq16_t<T, 64, true, SPARSE, DROP>(p, s) : launch_dq16_t<T, 64, false, SPARSE, DROP>(p, s);
  return p.causal ? launch_dq16_t<T, 128, true, SPARSE, DROP>(p, s) : launch_dq16_t<T, 128, false, SPARSE, DROP>(p, s);
}

#ifndef FA_BWD16_DROPOUT_UNIT
template <typename T>
static hipError_t launch_dq16_d(const BwdProblem& p, hipStream_t s) {
  if (p.drop_on) return launch_dq16_drop(p, s);
  return p.block_mask ? launch_dq16_s<T, true, false>(p, s) : launch_dq16_s<T, false, false>(p, s);
}

hipError_t launch_dq16(const BwdProblem& p, hipStream_t s) {
  return p.dtype == 1 ? launch_dq16_d<_Float16>(p, s) : launch_dq16_d<__bf16>(p, s);
}
#else
hipError_t launch_dq16_drop(const BwdProblem& p, hipStream_t s) {
  return p.dtype == 1 ? launch_dq16_s<_Float16, false, true>(p, s) : launch_dq16_s<__bf16, false, true>(p, s);
}
#endif

}  // namespace fa
