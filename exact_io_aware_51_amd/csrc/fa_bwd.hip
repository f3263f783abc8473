// fa_bwd.hip -- backward pass of fused exact attention for gfx950: the row
// sums D for every dtype, dK/dV and dQ for fp32 I/O (16-bit I/O runs the
// kernels of fa_bwd16.hip).
//
// Only O and the per-row log-sum-exp were kept by the forward pass; the score
// tiles are recomputed here tile by tile from Q, K and LSE, never read from
// device memory ("How Flash Attention Works: Tiling, Softmax, GPU I/O",
// section "The Backward Pass: Recomputation Instead of Stored Activations").
// The gradient formulas are the chain rule on O = softmax(scale Q K^T) V:
//   P = exp(scale S - LSE),  dV = P^T dO,  dP = dO V^T,
//   D_i = sum_c dO_ic O_ic (= sum_j P_ij dP_ij),  dS = P (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
// Three kernels, all deterministic (no atomics):
//   bwd_pre  : D_i, one pass over dO and O (bound by device memory);
//   bwd_dkdv : a workgroup owns 128 keys (32 per wave, K and V rows in VGPRs)
//              and streams query tiles (Q, dO, LSE, D) through LDS,
//              accumulating dK^T and dV^T on the matrix cores;
//   bwd_dq   : a workgroup owns 128 queries (Q and dO rows in VGPRs) and
//              streams key tiles (K, V) through LDS, accumulating dQ^T.
// Every product keeps the owned rows as the accumulator's lane column, feeds
// the recomputed P or dS back from registers as a B operand, and reads the
// other operand transposed out of LDS (see fa_device.h).
#include <mutex>

#include "fa_device.h"
#include "fa_launch.h"

// Row sums D of fa_bwd_static, which takes no workspace: kStaticScratchRows
// fp32 values (16 MiB) of device memory that every GPU the library runs on
// holds from its first fa_bwd_static call until the process ends.
static __device__ __align__(256) float scratch[fa::kStaticScratchRows];

namespace fa {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {};  // scratch's address on each device, once looked up
}  // namespace

// In host code `scratch` names a host-side stand-in, not device memory: the
// array's address on a device comes from hipGetSymbolAddress with that device
// current, looked up once per device and kept.
hipError_t static_scratch(hipStream_t stream, float** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);  // the device the launches will run on
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    g_scratch[dev] = static_cast<float*>(p);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;
  const int* seqlens_q;  // optional per-sequence lengths (device int32[B])
  const int* seqlens_k;
  const unsigned char* block_mask;  // block-sparse: [B, H, nbq, nbk] (SPARSE kernels only)
  int nbq, nbk;
  Dropout drop;                     // DROP kernels only
  int Nq, Nk, H;
  int nblk;    // blocks per head along the owned dimension
  int total;   // workgroups in the grid
  float c;     // scale * log2(e), signed
  float scale;
};

constexpr int kBwdThreads = 256;
constexpr int kBwdOwn = 128;   // owned rows per workgroup (32 per wave)
static_assert(kBwdOwn == kMaskBlock, "a workgroup's owned rows are one block-sparse mask block");
constexpr int kBwdTile = 64;   // streamed rows per tile

// --------------------------------------------------------------------------
// D_i = sum_c dO_ic * O_ic, fp32.  LPR lanes cooperate on one row.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                      float* __restrict__ dvec, long long rows) {
  constexpr int EPL = 16 / sizeof(T);  // elements per lane (one 16-byte chunk)
  constexpr int LPR = D / EPL;         // lanes per row
  constexpr int RPB = 256 / LPR;       // rows per block
  const int tid = thread_id();
  const long long row = (long long)block_id() * RPB + tid / LPR;
  const int part = tid % LPR;
  float acc = 0.0f;
  if (row < rows) {
    const size_t off = (size_t)row * D + part * EPL;
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + off);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dout + off);
    typedef T TV __attribute__((ext_vector_type(EPL)));
    const TV av = __builtin_bit_cast(TV, a), bv = __builtin_bit_cast(TV, b);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc = __builtin_fmaf((float)av[e], (float)bv[e], acc);
  }
#pragma unroll
  for (int w = LPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, LPR);
  if (row < rows && part == 0) dvec[row] = acc;
}

template <typename T, int D>
struct BwdLayout {
  static constexpr int ROWB = D * (int)sizeof(T);
  static constexpr int STR = D + (sizeof(T) == 2 ? 8 : 2);  // LDS row stride, elements
  static constexpr int TILE = kBwdTile * STR;
  static constexpr int CPR = ROWB / 16;
  static constexpr int PER_THREAD = kBwdTile * CPR / kBwdThreads;
  static_assert(kBwdTile * CPR % kBwdThreads == 0, "tile chunks must split evenly");
  static constexpr int LDS_BYTES = 2 * 2 * TILE * (int)sizeof(T) + 2 * 2 * kBwdTile * 4;
};

// --------------------------------------------------------------------------
// dK, dV for 128 keys per workgroup.
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using M = Mma<T>;
  using L = BwdLayout<T, D>;
  using Frag = typename M::Frag;
  constexpr int KSTEPS = D / M::KS;
  constexpr int MB = D / 32;
  constexpr int PSTEPS = 32 / M::KS;

  __shared__ __attribute__((aligned(16))) char smem[L::LDS_BYTES];
  T* lds_q = reinterpret_cast<T*>(smem);          // [2][TILE]
  T* lds_do = lds_q + 2 * L::TILE;                 // [2][TILE]
  float* lds_lse = reinterpret_cast<float*>(lds_do + 2 * L::TILE);  // [2][64], log2 units
  float* lds_d = lds_lse + 2 * kBwdTile;                            // [2][64]

  const int tid = thread_id();
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int Nq = a.Nq, Nk = a.Nk;

  const int bid = xcd_remap(block_id(), a.total);
  const int bh = __builtin_amdgcn_readfirstlane(bid / a.nblk);  // wave-uniform: keep scalar
  const int kblk = __builtin_amdgcn_readfirstlane(bid - bh * a.nblk);
  const int kb0 = kblk * kBwdOwn;
  const int kw = kb0 + 32 * wave;
  const Seq sq = seq_of(a.seqlens_q, a.seqlens_k, bh / a.H, Nq, Nk);
  const size_t headq = (size_t)bh * (size_t)Nq * D, headk = (size_t)bh * (size_t)Nk * D;
  const T* __restrict__ Q = reinterpret_cast<const T*>(a.q) + headq;
  const T* __restrict__ Kp = reinterpret_cast<const T*>(a.k) + headk;
  const T* __restrict__ Vp = reinterpret_cast<const T*>(a.v) + headk;
  const T* __restrict__ dO = reinterpret_cast<const T*>(a.dout) + headq;
  const float* __restrict__ lse = a.lse + (size_t)bh * Nq;
  const float* __restrict__ dvec = a.dvec + (size_t)bh * Nq;

  // K and V rows of this lane's key column, as B fragments (k = d).
  Frag kf[KSTEPS], vf[KSTEPS];
  {
    const int key = kw + col;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      kf[ks] = key < sq.lk ? row_frag<T>(Kp + (size_t)key * D + ks * M::KS, h) : zero_frag<T>();
      vf[ks] = key < sq.lk ? row_frag<T>(Vp + (size_t)key * D + ks * M::KS, h) : zero_frag<T>();
    }
  }

  // query tiles: real queries only; under the causal mask key j is first seen
  // by query j - off.  A block of padding keys visits none.
  const int ntiles = kb0 < sq.lk ? (sq.lq + kBwdTile - 1) / kBwdTile : 0;
  int first = 0;
  if (CAUSAL) {
    const int f = floor_div(kb0 - sq.off, kBwdTile);
    first = f > 0 ? f : 0;
  }
  // block-sparse: a query tile is live unless its 128-row block is masked out for this key block
  const unsigned char* mcol = SPARSE ? a.block_mask + (size_t)bh * a.nbq * a.nbk + kblk : nullptr;
  auto live = [&](int j) {
    if constexpr (SPARSE)
      return mcol[(size_t)((j * kBwdTile) / kMaskBlock) * a.nbk] != 0;
    else
      return true;
  };

  u32x4 qreg[L::PER_THREAD], doreg[L::PER_THREAD];
  float lse_r = 0.0f, d_r = 0.0f;
  auto load_tile = [&](int j) {
    const int i0 = j * kBwdTile;
#pragma unroll
    for (int i = 0; i < L::PER_THREAD; ++i) {
      const int c = tid + i * kBwdThreads;
      const int row = c / L::CPR, cc = c - row * L::CPR;
      const int qi = i0 + row;
      if (qi < sq.lq) {
        const size_t off = (size_t)qi * D + cc * (16 / sizeof(T));
        qreg[i] = *reinterpret_cast<const u32x4*>(Q + off);
        doreg[i] = *reinterpret_cast<const u32x4*>(dO + off);
      } else {
        qreg[i] = u32x4{0u, 0u, 0u, 0u};
        doreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < kBwdTile) {
      const int qi = i0 + tid;
      lse_r = qi < sq.lq ? lse[qi] * kLog2e : 0.0f;
      d_r = qi < sq.lq ? dvec[qi] : 0.0f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < L::PER_THREAD; ++i) {
      const int c = tid + i * kBwdThreads;
      const int row = c / L::CPR, cc = c - row * L::CPR;
      const int e = cc * (16 / sizeof(T));
      *reinterpret_cast<u32x4*>(lds_q + buf * L::TILE + row * L::STR + e) = qreg[i];
      *reinterpret_cast<u32x4*>(lds_do + buf * L::TILE + row * L::STR + e) = doreg[i];
    }
    if (tid < kBwdTile) {
      lds_lse[buf * kBwdTile + tid] = lse_r;
      lds_d[buf * kBwdTile + tid] = d_r;
    }
  };

  f32x16 dkacc[MB], dvacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    dkacc[mb] = f32x16{};
    dvacc[mb] = f32x16{};
  }
  const float c = a.c;
  const int mykey = kw + col;

  if (first < ntiles) {
    load_tile(first);
    store_tile(0);
  }
  __syncthreads();

  for (int j = first; j < ntiles; ++j) {
    const int buf = (j - first) & 1;
    if (j + 1 < ntiles && live(j + 1)) load_tile(j + 1);
    const int i0 = j * kBwdTile;
    // waves whose keys all follow this tile's last query have nothing to do,
    // and neither does anyone for a tile block sparsity removed
    if ((!CAUSAL || i0 + kBwdTile - 1 + sq.off >= kw) && live(j)) {
      const T* qt = lds_q + buf * L::TILE;
      const T* dot = lds_do + buf * L::TILE;
      const float* lt = lds_lse + buf * kBwdTile;
      const float* dt = lds_d + buf * kBwdTile;
      const bool edge = (i0 + kBwdTile > sq.lq) || (CAUSAL && i0 + sq.off < kw + 31);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 s = f32x16{}, dp = f32x16{};
        const T* qrow = qt + (32 * qb + col) * L::STR;
        const T* dorow = dot + (32 * qb + col) * L::STR;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          s = M::mma(row_frag<T>(qrow + ks * M::KS, h), kf[ks], s);
          dp = M::mma(row_frag<T>(dorow + ks * M::KS, h), vf[ks], dp);
        }
        // s: rows = queries i0 + 32 qb + acc_row(r, h), column = key mykey
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int rr = 32 * qb + 8 * g + 4 * h;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(lt + rr);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dt + rr);
          const uint32_t kbits = DROP ? a.drop.quad_keep(mykey >> 2, i0 + rr, bh, col & 3) : 0u;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = 4 * g + u;
            float p = fast_exp2(__builtin_fmaf(s[r], c, -l4[u]));
            if (edge) {
              const int qi = i0 + rr + u;
              const bool ok = qi < sq.lq && (!CAUSAL || mykey <= qi + sq.off);
              p = ok ? p : 0.0f;
            }
            if constexpr (DROP) {
              // dV takes the kept weights (1 / (1 - p) at the store); dP of a
              // dropped weight is 0, of a kept one dP / (1 - p)
              const bool kp = (kbits >> (4 * u)) & 1u;
              s[r] = kp ? p : 0.0f;
              dp[r] = p * ((kp ? dp[r] * a.drop.scale : 0.0f) - d4[u]);
            } else {
              s[r] = p;
              dp[r] = p * (dp[r] - d4[u]);
            }
          }
        }
        // dV^T += dO^T P,  dK^T += Q^T dS   (contraction over this block's 32 queries)
#pragma unroll
        for (int t = 0; t < PSTEPS; ++t) {
          const Frag pf = acc_frag<T>(s, t);
          const Frag sf = acc_frag<T>(dp, t);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            dvacc[mb] = M::mma(trans_frag<T>(dot, L::STR, 32 * qb, t, 32 * mb, lane), pf, dvacc[mb]);
            dkacc[mb] = M::mma(trans_frag<T>(qt, L::STR, 32 * qb, t, 32 * mb, lane), sf, dkacc[mb]);
          }
        }
      }
    }
    if (j + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (mykey < Nk) {  // padding keys store zeros
    T* dkrow = reinterpret_cast<T*>(a.dk) + headk + (size_t)mykey * D;
    T* dvrow = reinterpret_cast<T*>(a.dv) + headk + (size_t)mykey * D;
    const bool real = mykey < sq.lk;
    const float sc = a.scale;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mb + 8 * g + 4 * h;
        float k4[4], v4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          k4[u] = real ? dkacc[mb][4 * g + u] * sc : 0.0f;
          v4[u] = real ? dvacc[mb][4 * g + u] * (DROP ? a.drop.scale : 1.0f) : 0.0f;
        }
        store4<T>(dkrow + d0, k4[0], k4[1], k4[2], k4[3]);
        store4<T>(dvrow + d0, v4[0], v4[1], v4[2], v4[3]);
      }
  }
}

// --------------------------------------------------------------------------
// dQ for 128 queries per workgroup.
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dq_kernel(BwdArgs a) {
  using M = Mma<T>;
  using L = BwdLayout<T, D>;
  using Frag = typename M::Frag;
  constexpr int KSTEPS = D / M::KS;
  constexpr int MB = D / 32;
  constexpr int PSTEPS = 32 / M::KS;

  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * L::TILE * sizeof(T)];
  T* lds_k = reinterpret_cast<T*>(smem);  // [2][TILE]
  T* lds_v = lds_k + 2 * L::TILE;          // [2][TILE]

  const int tid = thread_id();
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int Nq = a.Nq, Nk = a.Nk;

  const int bid = xcd_remap(block_id(), a.total);
  const int bh = __builtin_amdgcn_readfirstlane(bid / a.nblk);  // wave-uniform: keep scalar
  int qb = __builtin_amdgcn_readfirstlane(bid - bh * a.nblk);
  if (CAUSAL) qb = a.nblk - 1 - qb;
  const int q0 = qb * kBwdOwn;
  const int qw = q0 + 32 * wave;
  const Seq sq = seq_of(a.seqlens_q, a.seqlens_k, bh / a.H, Nq, Nk);
  const size_t headq = (size_t)bh * (size_t)Nq * D, headk = (size_t)bh * (size_t)Nk * D;
  const T* __restrict__ Q = reinterpret_cast<const T*>(a.q) + headq;
  const T* __restrict__ Kp = reinterpret_cast<const T*>(a.k) + headk;
  const T* __restrict__ Vp = reinterpret_cast<const T*>(a.v) + headk;
  const T* __restrict__ dO = reinterpret_cast<const T*>(a.dout) + headq;

  const int myq = qw + col;
  Frag qf[KSTEPS], dof[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    qf[ks] = myq < sq.lq ? row_frag<T>(Q + (size_t)myq * D + ks * M::KS, h) : zero_frag<T>();
    dof[ks] = myq < sq.lq ? row_frag<T>(dO + (size_t)myq * D + ks * M::KS, h) : zero_frag<T>();
  }
  const float lse2 = myq < sq.lq ? a.lse[(size_t)bh * Nq + myq] * kLog2e : 0.0f;
  const float dq_d = myq < sq.lq ? a.dvec[(size_t)bh * Nq + myq] : 0.0f;

  int ntiles, nfull;
  query_block_tiles<CAUSAL, kBwdTile>(sq, q0, kBwdOwn, &ntiles, &nfull);
  const int lim = key_limit<CAUSAL>(sq, myq);
  const int wlast = qw + 31 + sq.off;  // causal: the last key any row of this wave may see
  // block-sparse: a key tile is live unless its 128-key block is masked out for this query block
  const unsigned char* mrow = SPARSE ? a.block_mask + ((size_t)bh * a.nbq + qb) * a.nbk : nullptr;
  auto live = [&](int j) {
    if constexpr (SPARSE)
      return mrow[(j * kBwdTile) / kMaskBlock] != 0;
    else
      return true;
  };

  u32x4 kreg[L::PER_THREAD], vreg[L::PER_THREAD];
  auto load_tile = [&](int j) {
    const int k0 = j * kBwdTile;
#pragma unroll
    for (int i = 0; i < L::PER_THREAD; ++i) {
      const int c = tid + i * kBwdThreads;
      const int row = c / L::CPR, cc = c - row * L::CPR;
      const int key = k0 + row;
      if (key < sq.lk) {
        const size_t off = (size_t)key * D + cc * (16 / sizeof(T));
        kreg[i] = *reinterpret_cast<const u32x4*>(Kp + off);
        vreg[i] = *reinterpret_cast<const u32x4*>(Vp + off);
      } else {
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
        vreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < L::PER_THREAD; ++i) {
      const int c = tid + i * kBwdThreads;
      const int row = c / L::CPR, cc = c - row * L::CPR;
      const int e = cc * (16 / sizeof(T));
      *reinterpret_cast<u32x4*>(lds_k + buf * L::TILE + row * L::STR + e) = kreg[i];
      *reinterpret_cast<u32x4*>(lds_v + buf * L::TILE + row * L::STR + e) = vreg[i];
    }
  };

  f32x16 dqacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) dqacc[mb] = f32x16{};
  const float c = a.c;

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles && live(j + 1)) load_tile(j + 1);
    const int k0 = j * kBwdTile;
    if ((!CAUSAL || k0 <= wlast) && live(j)) {
      const T* kt = lds_k + buf * L::TILE;
      const T* vt = lds_v + buf * L::TILE;
      // unmasked when every row of the wave may see every key of the tile
      const bool edge = j >= nfull && ((k0 + kBwdTile > sq.lk) || (CAUSAL && k0 + kBwdTile - 1 > qw + sq.off) ||
                                       qw + 31 >= sq.lq);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 s = f32x16{}, dp = f32x16{};
        const T* krow = kt + (32 * kb + col) * L::STR;
        const T* vrow = vt + (32 * kb + col) * L::STR;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          s = M::mma(row_frag<T>(krow + ks * M::KS, h), qf[ks], s);
          dp = M::mma(row_frag<T>(vrow + ks * M::KS, h), dof[ks], dp);
        }
        // s^T: rows = keys k0 + 32 kb + acc_row(r, h), column = query myq
        u32x4v w[4];  // dropout words of the four 4-key groups
        if constexpr (DROP) {
#pragma unroll
          for (int g = 0; g < 4; ++g) w[g] = a.drop.words((k0 + 32 * kb + 8 * g + 4 * h) >> 2, myq, bh);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(__builtin_fmaf(s[r], c, -lse2));
          if (edge) {
            const int key = k0 + 32 * kb + acc_row(r, h);
            p = key <= lim ? p : 0.0f;
          }
          if constexpr (DROP)
            dp[r] = p * ((w[r >> 2][r & 3] >= a.drop.threshold ? dp[r] * a.drop.scale : 0.0f) - dq_d);
          else
            dp[r] = p * (dp[r] - dq_d);
        }
        // dQ^T += K^T dS^T  (contraction over this block's 32 keys)
#pragma unroll
        for (int t = 0; t < PSTEPS; ++t) {
          const Frag sf = acc_frag<T>(dp, t);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            dqacc[mb] = M::mma(trans_frag<T>(kt, L::STR, 32 * kb, t, 32 * mb, lane), sf, dqacc[mb]);
        }
      }
    }
    if (j + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (myq < Nq) {  // padding rows store zeros
    T* dqrow = reinterpret_cast<T*>(a.dq) + headq + (size_t)myq * D;
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
        store4<T>(dqrow + d0, q4[0], q4[1], q4[2], q4[3]);
      }
  }
}

// --------------------------------------------------------------------------
// Row sums D (every dtype and head size).
template <typename T, int D>
static hipError_t launch_pre_t(const BwdProblem& p, hipStream_t stream) {
  const long long rows = (long long)p.B * p.H * p.Nq;
  constexpr int LPR = D / (16 / sizeof(T));
  constexpr int RPB = 256 / LPR;
  const long long blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const T*>(p.o), reinterpret_cast<const T*>(p.dout), p.dvec, rows);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_pre_d(const BwdProblem& p, hipStream_t s) {
  return p.d == 64 ? launch_pre_t<T, 64>(p, s) : launch_pre_t<T, 128>(p, s);
}

static hipError_t launch_pre(const BwdProblem& p, hipStream_t s) {
  switch (p.dtype) {
    case 0: return launch_pre_d<float>(p, s);
    case 1: return launch_pre_d<_Float16>(p, s);
    default: return launch_pre_d<__bf16>(p, s);
  }
}

// dK/dV (stage 1) or dQ (stage 2) for fp32 I/O.
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
static hipError_t launch_bwd_t(const BwdProblem& p, int stage, hipStream_t stream) {
  BwdArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o; a.dout = p.dout; a.lse = p.lse;
  a.dq = p.dq; a.dk = p.dk; a.dv = p.dv; a.dvec = p.dvec;
  a.seqlens_q = p.seqlens_q; a.seqlens_k = p.seqlens_k;
  a.block_mask = p.block_mask;
  a.drop = Dropout{p.drop_threshold, p.drop_seed_lo, p.drop_seed_hi, p.drop_offset, p.drop_scale};
  a.nbq = (p.Nq + kMaskBlock - 1) / kMaskBlock;
  a.nbk = (p.Nk + kMaskBlock - 1) / kMaskBlock;
  a.Nq = p.Nq; a.Nk = p.Nk; a.H = p.H;
  a.scale = p.scale;
  a.c = p.scale * kLog2e;
  a.nblk = ((stage == 1 ? p.Nk : p.Nq) + kBwdOwn - 1) / kBwdOwn;
  a.total = a.nblk * p.B * p.H;
  if (stage == 1)
    hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL, SPARSE, DROP>), dim3(a.total), dim3(kBwdThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, SPARSE, DROP>), dim3(a.total), dim3(kBwdThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, bool SPARSE, bool DROP>
static hipError_t launch_bwd_s(const BwdProblem& p, int stage, hipStream_t s) {
  if (p.d == 64)
    return p.causal ? launch_bwd_t<T, 64, true, SPARSE, DROP>(p, stage, s)
                    : launch_bwd_t<T, 64, false, SPARSE, DROP>(p, stage, s);
  return p.causal ? launch_bwd_t<T, 128, true, SPARSE, DROP>(p, stage, s)
                  : launch_bwd_t<T, 128, false, SPARSE, DROP>(p, stage, s);
}

// The dK/dV and dQ kernels above serve fp32 I/O; 16-bit I/O runs the kernels
// of fa_bwd16.hip.  (Block sparsity and dropout are not combined: the API
// rejects that.)
hipError_t launch_bwd_stage(const BwdProblem& p, int stage, hipStream_t s) {
  if (stage == 0) return launch_pre(p, s);
  if (stage == 3) {
    if (p.dtype != 0) {  // the 16-bit dQ kernel forms D from its own dO rows and the O rows
      BwdProblem f = p;
      f.dq_rowsum = 1;
      return launch_dq16(f, s);
    }
    const hipError_t e = launch_pre(p, s);
    return e != hipSuccess ? e : launch_bwd_stage(p, 2, s);
  }
  if (p.dtype != 0) return stage == 1 ? launch_dkdv16(p, s) : launch_dq16(p, s);
  if (p.drop_on) return launch_bwd_s<float, false, true>(p, stage, s);
  return p.block_mask != nullptr ? launch_bwd_s<float, true, false>(p, stage, s)
                                 : launch_bwd_s<float, false, false>(p, stage, s);
}

}  // namespace fa
