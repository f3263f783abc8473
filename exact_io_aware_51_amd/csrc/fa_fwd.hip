// fa_fwd.hip -- fused exact-attention forward pass for fp32 I/O on gfx950
// (16-bit I/O runs the pipelined kernels of fa_fwd16.hip).
//
// One workgroup owns a block of BM = 128 query rows of one (batch, head) and
// streams the key/value tiles of that head past it ("How Flash Attention
// Works: Tiling, Softmax, GPU I/O", section "Tiling Q, K, and V for Fast
// On-Chip Memory").  Each of its four waves owns 32 query rows:
//   * its Q rows live in VGPRs for the whole loop (the B operand of S^T = K Q^T);
//   * K and V tiles of BN = 64 keys are staged in LDS, double-buffered through
//     registers so the global loads of tile j+1 overlap the matrix work on j;
//   * S^T = K Q^T and O^T += V^T P^T run on the matrix cores with fp32
//     accumulation; with S^T, each lane owns one query column, so the running
//     row max / normaliser of the online softmax ("Online Softmax Without the
//     Full Score Matrix") are per-lane scalars plus one half-wave swap;
//   * P^T is fed back from the accumulator registers as the next B operand
//     and V^T comes from LDS with the transposing read, so P never leaves
//     registers ("Kernel Fusion and Incremental Output Accumulation");
//   * under the causal mask, tiles wholly above the diagonal are skipped and
//     only diagonal/edge tiles evaluate the mask (FlashAttention-2's trimming of
//     non-matmul work, same page, section "FlashAttention 1 vs 2 vs 3").
// Only O and one log-sum-exp per row are written to device memory.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int* seqlens_q;  // optional per-sequence lengths (device int32[B])
  const int* seqlens_k;
  const unsigned char* block_mask;  // block-sparse: [B, H, nqb, nbk] (SPARSE kernels only)
  int nbk;
  Dropout drop;                     // DROP kernels only
  int Nq, Nk, H;
  int nqb;     // query blocks per head
  int total;   // workgroups in the grid
  float c;     // |scale| * log2(e)
  int negate;  // scale < 0: Q enters with its sign flipped (exact), c = |scale| log2 e
};

constexpr int kFwdBM = 128;
constexpr int kFwdBN = 64;
constexpr int kFwdThreads = 256;

template <typename T, int D>
struct FwdLayout {
  static constexpr int ROWB = D * (int)sizeof(T);
  // LDS row strides (elements).  K is read as rows (16 B per lane, 32 rows at
  // one column); V is read through the transposing read (4 rows x 32 B per
  // 16 lanes).  The pads spread those accesses over the banks.
  static constexpr int KSTR = D + (sizeof(T) == 2 ? 8 : 2);
  static constexpr int VSTR = D + (sizeof(T) == 2 ? 32 : 2);
  static constexpr int KTILE = kFwdBN * KSTR;  // elements
  static constexpr int VTILE = kFwdBN * VSTR;
  static constexpr int CPR = ROWB / 16;                        // 16-byte chunks per row
  static constexpr int PER_THREAD = kFwdBN * CPR / kFwdThreads;  // chunks per thread per tile
  static constexpr int LDS_BYTES = 2 * (KTILE + VTILE) * (int)sizeof(T);
  static_assert(kFwdBN * CPR % kFwdThreads == 0, "tile chunks must split evenly");
};

// Rescale the running output only when some row's max has grown by more than
// 2^kTau since the reference max was last moved.  O and l are always scaled
// against the same reference, so the final O = acc / l is unchanged; the
// weights 2^(c s - m) stay below 2^kTau, far inside fp32 and bf16 range.
constexpr float kTau = 8.0f;

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
__global__ __launch_bounds__(kFwdThreads, (sizeof(T) == 2 || D == 64) ? 2 : 1) void fwd_kernel(FwdArgs a) {
  using M = Mma<T>;
  using L = FwdLayout<T, D>;
  using Frag = typename M::Frag;
  constexpr int KSTEPS = D / M::KS;
  constexpr int MB = D / 32;           // 32-column blocks of the output
  constexpr int PSTEPS = 32 / M::KS;   // k-steps per 32-key block in P*V

  __shared__ __attribute__((aligned(16))) T smem[L::LDS_BYTES / sizeof(T)];
  T* lds_k = smem;                 // [2][KTILE]
  T* lds_v = smem + 2 * L::KTILE;  // [2][VTILE]

  const int tid = thread_id();
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int Nq = a.Nq, Nk = a.Nk;

  // block coordinates are wave-uniform; keep them (and every address built
  // from them) in scalar registers
  const int bid = xcd_remap(block_id(), a.total);
  const int bh = __builtin_amdgcn_readfirstlane(bid / a.nqb);
  int qb = __builtin_amdgcn_readfirstlane(bid - bh * a.nqb);
  if (CAUSAL) qb = a.nqb - 1 - qb;  // the longest causal rows start first
  const int q0 = qb * kFwdBM;
  const int qw = q0 + wave * 32;
  const Seq sq = seq_of(a.seqlens_q, a.seqlens_k, bh / a.H, Nq, Nk);
  const T* __restrict__ Q = reinterpret_cast<const T*>(a.q) + (size_t)bh * (size_t)Nq * D;
  const char* Kb = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.k) + (size_t)bh * (size_t)Nk * D);
  const char* Vb = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.v) + (size_t)bh * (size_t)Nk * D);

  // Q rows of this lane's query column, as B fragments (k = d).
  const int myq = qw + col;
  Frag qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    qf[ks] = myq < sq.lq ? row_frag<T>(Q + (size_t)myq * D + ks * M::KS, h) : zero_frag<T>();
    if (a.negate) qf[ks] = neg_frag<T>(qf[ks]);
  }

  int ntiles, nfull;
  query_block_tiles<CAUSAL, kFwdBN>(sq, q0, kFwdBM, &ntiles, &nfull);
  // largest key this lane's query may see (negative: none)
  const int lim = key_limit<CAUSAL>(sq, myq);
  const int wlast = qw + 31 + sq.off;  // causal: the last key any row of this wave may see
  // block-sparse: a key tile is live unless its 128-key block is masked out for this query block
  const unsigned char* mrow = SPARSE ? a.block_mask + ((size_t)bh * a.nqb + qb) * a.nbk : nullptr;
  auto live = [&](int j) {
    if constexpr (SPARSE)
      return mrow[(j * kFwdBN) / kMaskBlock] != 0;
    else
      return true;
  };

  // Global -> register staging of one K/V tile: 16-byte chunks, coalesced.
  // The buffer view of the tile ends at the sequence's last key, so reads
  // past it return zeros.
  uint32_t goff[L::PER_THREAD], soff[L::PER_THREAD], voff[L::PER_THREAD];
#pragma unroll
  for (int i = 0; i < L::PER_THREAD; ++i) {
    const int c = tid + i * kFwdThreads;
    const int row = c / L::CPR, cc = c - row * L::CPR;
    goff[i] = row * L::ROWB + cc * 16;
    soff[i] = (row * L::KSTR + cc * (16 / sizeof(T))) * sizeof(T);
    voff[i] = (row * L::VSTR + cc * (16 / sizeof(T))) * sizeof(T);
  }
  u32x4 kreg[L::PER_THREAD], vreg[L::PER_THREAD];
  auto load_tile = [&](int j) {
    const size_t base = (size_t)j * kFwdBN * L::ROWB;
    const uint32_t left = tile_bytes(sq.lk - j * kFwdBN, kFwdBN, L::ROWB);
    const auto rk = buffer_rsrc(Kb + base, left);
    const auto rv = buffer_rsrc(Vb + base, left);
#pragma unroll
    for (int i = 0; i < L::PER_THREAD; ++i) {
      kreg[i] = buffer_load16(rk, goff[i]);
      vreg[i] = buffer_load16(rv, goff[i]);
    }
  };
  auto store_tile = [&](int buf) {
    char* kd = reinterpret_cast<char*>(lds_k + buf * L::KTILE);
    char* vd = reinterpret_cast<char*>(lds_v + buf * L::VTILE);
#pragma unroll
    for (int i = 0; i < L::PER_THREAD; ++i) {
      *reinterpret_cast<u32x4*>(kd + soff[i]) = kreg[i];
      *reinterpret_cast<u32x4*>(vd + voff[i]) = vreg[i];
    }
  };

  f32x16 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) oacc[mb] = f32x16{};
  float m = kMaxFloor;  // reference max of c * s (log2 units), same in both half-waves
  float l = 0.0f;       // this half-wave's share of sum 2^(c s - m)
  const float c = a.c;

  // One 64-key tile: S^T = K Q^T, online softmax, O^T += V^T P^T.
  auto tile = [&](const T* kt, const T* vt, int k0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    const T* kr0 = kt + col * L::KSTR;
    const T* kr1 = kt + (32 + col) * L::KSTR;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      s0 = M::mma(row_frag<T>(kr0 + ks * M::KS, h), qf[ks], s0);
      s1 = M::mma(row_frag<T>(kr1 + ks * M::KS, h), qf[ks], s1);
    }
    // key of register r in block kb is k0 + 32 kb + acc_row(r, h); allowed iff <= lim
    const int t0 = lim - k0 - 4 * h, t1 = t0 - 32;
    float mx = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ro = 8 * (r >> 2) + (r & 3);
      float x0 = s0[r], x1 = s1[r];
      if constexpr (MASK) {
        x0 = ro <= t0 ? x0 : -__builtin_inff();
        x1 = ro <= t1 ? x1 : -__builtin_inff();
      }
      mx = __builtin_fmaxf(mx, __builtin_fmaxf(x0, x1));
    }
    mx = halves_max(mx);
    float mt = mx * c;
    if constexpr (MASK) mt = mx > -__builtin_inff() ? mt : -__builtin_inff();
    if (any_lane(mt > m + kTau)) {
      const float mnew = __builtin_fmaxf(m, mt);
      const float alpha = fast_exp2(m - mnew);
      l *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;
      m = mnew;
    }
    const float negm = -m;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p0 = fast_exp2(__builtin_fmaf(s0[r], c, negm));
      float p1 = fast_exp2(__builtin_fmaf(s1[r], c, negm));
      if constexpr (MASK) {
        const int ro = 8 * (r >> 2) + (r & 3);
        p0 = ro <= t0 ? p0 : 0.0f;
        p1 = ro <= t1 ? p1 : 0.0f;
      }
      s0[r] = p0;
      s1[r] = p1;
      l += p0 + p1;
    }
    // dropout: zero the weights of dropped keys (1 / (1 - p) goes with 1 / l)
    if constexpr (DROP) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x4v w0 = a.drop.words((k0 + 8 * g + 4 * h) >> 2, myq, bh);
        const u32x4v w1 = a.drop.words((k0 + 32 + 8 * g + 4 * h) >> 2, myq, bh);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          s0[4 * g + u] = w0[u] >= a.drop.threshold ? s0[4 * g + u] : 0.0f;
          s1[4 * g + u] = w1[u] >= a.drop.threshold ? s1[4 * g + u] : 0.0f;
        }
      }
    }
    // O^T += V^T P^T over the tile's 64 keys
#pragma unroll
    for (int t = 0; t < PSTEPS; ++t) {
      const Frag pf0 = acc_frag<T>(s0, t);
      const Frag pf1 = acc_frag<T>(s1, t);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        oacc[mb] = M::mma(trans_frag<T>(vt, L::VSTR, 0, t, 32 * mb, lane), pf0, oacc[mb]);
        oacc[mb] = M::mma(trans_frag<T>(vt, L::VSTR, 32, t, 32 * mb, lane), pf1, oacc[mb]);
      }
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles && live(j + 1)) load_tile(j + 1);
    const int k0 = j * kFwdBN;
    // waves whose rows all precede this tile's first key have nothing to do,
    // and neither does anyone for a tile block sparsity removed
    if ((!CAUSAL || k0 <= wlast) && live(j)) {
      const T* kt = lds_k + buf * L::KTILE;
      const T* vt = lds_v + buf * L::VTILE;
      // a tile is unmasked for the wave when every row of it may see every key
      const bool edge = j >= nfull && ((k0 + kFwdBN > sq.lk) || (CAUSAL && k0 + kFwdBN - 1 > qw + sq.off) ||
                                       qw + 31 >= sq.lq);
      if (edge)
        tile(kt, vt, k0, std::true_type{});
      else
        tile(kt, vt, k0, std::false_type{});
    }
    if (j + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: O = O_acc / l, LSE = ln(2^m * l); padding rows and rows that
  // see no key store O = 0, LSE = -inf.
  l = halves_sum(l);
  if (myq < Nq) {
    const bool real = myq < sq.lq && l > 0.0f;
    const float inv = real ? (DROP ? a.drop.scale : 1.0f) / l : 0.0f;
    T* orow = reinterpret_cast<T*>(a.o) + (size_t)bh * (size_t)Nq * D + (size_t)myq * D;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mb + 8 * g + 4 * h;
        float o4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) o4[u] = real ? oacc[mb][4 * g + u] * inv : 0.0f;
        store4<T>(orow + d0, o4[0], o4[1], o4[2], o4[3]);
      }
    if (a.lse != nullptr && h == 0)
      a.lse[(size_t)bh * Nq + myq] = real ? (m + __builtin_log2f(l)) * kLn2 : -__builtin_inff();
  }
}

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
static hipError_t launch_fwd_t(const FwdProblem& p, hipStream_t stream) {
  FwdArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o; a.lse = p.lse;
  a.seqlens_q = p.seqlens_q; a.seqlens_k = p.seqlens_k;
  a.Nq = p.Nq; a.Nk = p.Nk; a.H = p.H;
  a.block_mask = p.block_mask;
  a.nbk = (p.Nk + kMaskBlock - 1) / kMaskBlock;
  a.drop = Dropout{p.drop_threshold, p.drop_seed_lo, p.drop_seed_hi, p.drop_offset, p.drop_scale};
  a.nqb = (p.Nq + kFwdBM - 1) / kFwdBM;
  static_assert(kFwdBM == kMaskBlock, "one workgroup's query rows are one mask block row");
  a.total = a.nqb * p.B * p.H;
  const float sc = p.scale;
  a.negate = sc < 0.0f;
  a.c = (sc < 0.0f ? -sc : sc) * kLog2e;
  hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL, SPARSE, DROP>), dim3(a.total), dim3(kFwdThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, bool SPARSE, bool DROP>
static hipError_t launch_fwd_s(const FwdProblem& p, hipStream_t s) {
  if (p.d == 64)
    return p.causal ? launch_fwd_t<T, 64, true, SPARSE, DROP>(p, s) : launch_fwd_t<T, 64, false, SPARSE, DROP>(p, s);
  return p.causal ? launch_fwd_t<T, 128, true, SPARSE, DROP>(p, s) : launch_fwd_t<T, 128, false, SPARSE, DROP>(p, s);
}

// fp32 I/O runs this kernel; 16-bit I/O runs the pipelined kernels of
// fa_fwd16.hip.  (Block sparsity and dropout are not combined: the API
// rejects that.)
hipError_t launch_fwd(const FwdProblem& p, hipStream_t s) {
  if (p.dtype != 0) return launch_fwd16(p, s);
  if (p.drop_on) return launch_fwd_s<float, false, true>(p, s);
  return p.block_mask != nullptr ? launch_fwd_s<float, true, false>(p, s) : launch_fwd_s<float, false, false>(p, s);
}

}  // namespace fa
