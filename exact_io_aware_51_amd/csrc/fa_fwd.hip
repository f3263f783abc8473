// fa_fwd.hip -- fused exact-attention forward pass for gfx950.
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
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int N;
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

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads, 2) void fwd_kernel(FwdArgs a) {
  using M = Mma<T>;
  using L = FwdLayout<T, D>;
  using Frag = typename M::Frag;
  constexpr int KSTEPS = D / M::KS;
  constexpr int MB = D / 32;           // 32-column blocks of the output
  constexpr int PSTEPS = 32 / M::KS;   // k-steps per 32-key block in P*V

  __shared__ __attribute__((aligned(16))) T smem[L::LDS_BYTES / sizeof(T)];
  T* lds_k = smem;                 // [2][KTILE]
  T* lds_v = smem + 2 * L::KTILE;  // [2][VTILE]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int N = a.N;

  const int bid = xcd_remap(blockIdx.x, a.total);
  const int bh = bid / a.nqb;
  int qb = bid - bh * a.nqb;
  if (CAUSAL) qb = a.nqb - 1 - qb;  // the longest causal rows start first
  const int q0 = qb * kFwdBM;
  const int qw = q0 + wave * 32;
  const size_t head = (size_t)bh * (size_t)N * D;
  const T* __restrict__ Q = reinterpret_cast<const T*>(a.q) + head;
  const T* __restrict__ K = reinterpret_cast<const T*>(a.k) + head;
  const T* __restrict__ V = reinterpret_cast<const T*>(a.v) + head;

  // Q rows of this lane's query column, as B fragments (k = d).
  Frag qf[KSTEPS];
  {
    const int qrow = qw + col;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      qf[ks] = qrow < N ? row_frag<T>(Q + (size_t)qrow * D + ks * M::KS, h) : zero_frag<T>();
      if (a.negate) qf[ks] = neg_frag<T>(qf[ks]);
    }
  }

  const int ntiles_all = (N + kFwdBN - 1) / kFwdBN;
  int ntiles = ntiles_all;
  if (CAUSAL) {
    const int last = (q0 + kFwdBM - 1) / kFwdBN + 1;
    ntiles = last < ntiles_all ? last : ntiles_all;
  }

  // Global -> register staging of one K/V tile (16-byte chunks, coalesced).
  u32x4 kreg[L::PER_THREAD], vreg[L::PER_THREAD];
  auto load_tile = [&](int j) {
    const int k0 = j * kFwdBN;
#pragma unroll
    for (int i = 0; i < L::PER_THREAD; ++i) {
      const int c = tid + i * kFwdThreads;
      const int row = c / L::CPR, cc = c - row * L::CPR;
      const int key = k0 + row;
      if (key < N) {
        const size_t off = (size_t)key * D + cc * (16 / sizeof(T));
        kreg[i] = *reinterpret_cast<const u32x4*>(K + off);
        vreg[i] = *reinterpret_cast<const u32x4*>(V + off);
      } else {
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
        vreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < L::PER_THREAD; ++i) {
      const int c = tid + i * kFwdThreads;
      const int row = c / L::CPR, cc = c - row * L::CPR;
      const int e = cc * (16 / sizeof(T));
      *reinterpret_cast<u32x4*>(lds_k + buf * L::KTILE + row * L::KSTR + e) = kreg[i];
      *reinterpret_cast<u32x4*>(lds_v + buf * L::VTILE + row * L::VSTR + e) = vreg[i];
    }
  };

  f32x16 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) oacc[mb] = f32x16{};
  float m = kMaxFloor;  // running max of c * s over the keys seen so far (log2 units)
  float l = 0.0f;       // running normaliser sum 2^(c s - m)
  const float c = a.c;
  const int myq = qw + col;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) load_tile(j + 1);
    const int k0 = j * kFwdBN;
    // waves whose rows all precede this tile's first key have nothing to do
    if (!CAUSAL || k0 <= qw + 31) {
      const T* kt = lds_k + buf * L::KTILE;
      const T* vt = lds_v + buf * L::VTILE;
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const T* krow = kt + (32 * kb + col) * L::KSTR;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
          s[kb] = M::mma(row_frag<T>(krow + ks * M::KS, h), qf[ks], s[kb]);
      }
      // mask: keys past the end, and (causal) keys after the lane's query
      const bool edge = (k0 + kFwdBN > N) || (CAUSAL && k0 + kFwdBN - 1 > qw);
      uint32_t live[2] = {0xffffffffu, 0xffffffffu};
      if (edge) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + acc_row(r, h);
            const bool ok = key < N && (!CAUSAL || key <= myq);
            if (!ok) live[kb] &= ~(1u << r);
          }
        }
      }
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = (live[kb] >> r) & 1u ? s[kb][r] : -__builtin_inff();
          mx = __builtin_fmaxf(mx, x);
        }
      mx = halves_max(mx);
      const float mt = mx > -__builtin_inff() ? mx * c : kMaxFloor;
      const float mnew = __builtin_fmaxf(m, mt);
      const float alpha = fast_exp2(m - mnew);
      float rs = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[kb][r], c, -mnew));
          p = (live[kb] >> r) & 1u ? p : 0.0f;
          s[kb][r] = p;
          rs += p;
        }
      rs = halves_sum(rs);
      l = __builtin_fmaf(l, alpha, rs);
      m = mnew;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;
      // O^T += V^T P^T over the tile's 64 keys
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < PSTEPS; ++t) {
          const Frag pf = acc_frag<T>(s[kb], t);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            oacc[mb] = M::mma(trans_frag<T>(vt, L::VSTR, 32 * kb, t, 32 * mb, lane), pf, oacc[mb]);
        }
    }
    if (j + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: O = O_acc / l, LSE = ln(2^m * l).
  if (myq < N) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    T* orow = reinterpret_cast<T*>(a.o) + head + (size_t)myq * D;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mb + 8 * g + 4 * h;
        store4<T>(orow + d0, oacc[mb][4 * g] * inv, oacc[mb][4 * g + 1] * inv,
                  oacc[mb][4 * g + 2] * inv, oacc[mb][4 * g + 3] * inv);
      }
    if (a.lse != nullptr && h == 0)
      a.lse[(size_t)bh * N + myq] = l > 0.0f ? (m + __builtin_log2f(l)) * kLn2 : -__builtin_inff();
  }
}

template <typename T, int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdProblem& p, hipStream_t stream) {
  FwdArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o; a.lse = p.lse;
  a.N = p.N;
  a.nqb = (p.N + kFwdBM - 1) / kFwdBM;
  a.total = a.nqb * p.B * p.H;
  const float sc = p.scale;
  a.negate = sc < 0.0f;
  a.c = (sc < 0.0f ? -sc : sc) * kLog2e;
  hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL>), dim3(a.total), dim3(kFwdThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_fwd_d(const FwdProblem& p, hipStream_t s) {
  if (p.d == 64) return p.causal ? launch_fwd_t<T, 64, true>(p, s) : launch_fwd_t<T, 64, false>(p, s);
  return p.causal ? launch_fwd_t<T, 128, true>(p, s) : launch_fwd_t<T, 128, false>(p, s);
}

hipError_t launch_fwd(const FwdProblem& p, hipStream_t s) {
  switch (p.dtype) {
    case 0: return launch_fwd_d<float>(p, s);
    case 1: return launch_fwd_d<_Float16>(p, s);
    default: return launch_fwd_d<__bf16>(p, s);
  }
}

}  // namespace fa
