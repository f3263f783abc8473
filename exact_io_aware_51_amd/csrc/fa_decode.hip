// fa_decode.hip -- split-key forward for one query row per (batch, head):
// decoding against a key cache.
//
// With a single query there is nothing to share a key tile with, so the
// tiled kernel's LDS staging, its 128-row query blocks (127 of them padding)
// and its per-tile barrier are pure overhead, and one tile in flight per
// workgroup leaves HBM latency exposed.  Here every wave streams its own keys
// from device memory straight into registers.  D / 8 consecutive lanes hold
// one key row, 8 channels (16 bytes) each, so one load instruction reads whole
// consecutive rows (1 KiB contiguous), and a lane keeps only its 8 output
// channels.  Each lane group keeps the online softmax state of the keys it saw
// ("How Flash Attention Works: Tiling, Softmax, GPU I/O", section "Online
// Softmax Without the Full Score Matrix"): a running maximum m, the normaliser
// l and its slice of the output, rescaled lazily (only when the maximum grows
// by more than 2^8, as in the tiled kernels).  At the end the groups and waves
// are merged with the same rescale and the workgroup writes its key range's
// normalised fp32 output and LSE; split_merge_kernel combines the ranges.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int* seqlens_q;
  const int* seqlens_k;
  int Nk, H, splits, split_keys;  // split s covers keys [s * split_keys, (s + 1) * split_keys)
  int rows;                       // B * H
  float c;                        // |scale| * log2(e)
  uint32_t flip;                  // sign bits of both halves when the scale is negative
  float* part_o;                  // [splits][rows][D]
  float* part_lse;                // [splits][rows]
};

template <typename T> struct Half2;
template <> struct Half2<__bf16> {
  typedef __bf16 V __attribute__((ext_vector_type(2)));
  __device__ static inline float dot(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(V, a), __builtin_bit_cast(V, b), c, false);
  }
  __device__ static inline float lo(uint32_t x) { return __uint_as_float(x << 16); }
  __device__ static inline float hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }
};
template <> struct Half2<_Float16> {
  typedef _Float16 V __attribute__((ext_vector_type(2)));
  __device__ static inline float dot(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(V, a), __builtin_bit_cast(V, b), c, false);
  }
  __device__ static inline float lo(uint32_t x) { return (float)__builtin_bit_cast(V, x)[0]; }
  __device__ static inline float hi(uint32_t x) { return (float)__builtin_bit_cast(V, x)[1]; }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  using P = Half2<T>;
  constexpr int LPK = D / 8;       // lanes per key row (8 channels, 16 bytes each)
  constexpr int KPI = 64 / LPK;    // keys per load instruction: 4 (d = 128) or 8 (d = 64)
  constexpr int U = 4;  // key slots per lane and iteration
  constexpr int STEP = U * KPI;    // keys per wave and iteration
  __shared__ float red[4][D + 2];

  const int lane = thread_id() & 63;
  const int wave = __builtin_amdgcn_readfirstlane(thread_id() >> 6);
  const int bid = block_id();
  const int split = __builtin_amdgcn_readfirstlane(bid % a.splits);
  const int bh = __builtin_amdgcn_readfirstlane(bid / a.splits);
  const Seq sq = seq_of(a.seqlens_q, a.seqlens_k, bh / a.H, 1, a.Nk);
  const int grp = lane / LPK, chunk = lane % LPK;
  const int kbeg = split * a.split_keys;
  const int kend = sq.lk < kbeg + a.split_keys ? sq.lk : kbeg + a.split_keys;

  uint32_t q2[4];
  {
    const u32x4 x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(a.q) + (size_t)bh * D + 8 * chunk);
#pragma unroll
    for (int e = 0; e < 4; ++e) q2[e] = x[e] ^ a.flip;
  }
  const T* kbase = reinterpret_cast<const T*>(a.k) + (size_t)bh * a.Nk * D + 8 * chunk;
  const T* vbase = reinterpret_cast<const T*>(a.v) + (size_t)bh * a.Nk * D + 8 * chunk;

  float m = kMaxFloor, l = 0.0f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.0f;
  const float c = a.c;

  if (sq.lq > 0) {
    for (int base = kbeg + STEP * wave; base < kend; base += 4 * STEP) {  // wave-uniform trip count
      u32x4 k4[U], v4[U];
      bool valid[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int key = base + KPI * u + grp;
        valid[u] = key < kend;
        k4[u] = u32x4{0u, 0u, 0u, 0u};
        v4[u] = u32x4{0u, 0u, 0u, 0u};
        if (valid[u]) {
          k4[u] = *reinterpret_cast<const u32x4*>(kbase + (size_t)key * D);
          v4[u] = *reinterpret_cast<const u32x4*>(vbase + (size_t)key * D);
        }
      }
      float s[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float x = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) x = P::dot(q2[e], k4[u][e], x);
#pragma unroll
        for (int w = 1; w < LPK; w <<= 1) x += __shfl_xor(x, w);  // the row's other channels
        s[u] = valid[u] ? x * c : -__builtin_inff();
      }
      float smax = s[0];
#pragma unroll
      for (int u = 1; u < U; ++u) smax = __builtin_fmaxf(smax, s[u]);
      if (any_lane(smax > m + 8.0f)) {
        const float mnew = smax > m + 8.0f ? smax : m;
        const float alpha = fast_exp2(m - mnew);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= alpha;
        m = mnew;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = fast_exp2(s[u] - m);
        l += p;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[2 * e] = __builtin_fmaf(p, P::lo(v4[u][e]), o[2 * e]);
          o[2 * e + 1] = __builtin_fmaf(p, P::hi(v4[u][e]), o[2 * e + 1]);
        }
      }
    }
  }

  // merge the KPI lane groups (same chunk, different keys): common maximum, then sums
  float mx = m;
#pragma unroll
  for (int x = LPK; x < 64; x <<= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, x));
  const float w = fast_exp2(m - mx);
  l *= w;
#pragma unroll
  for (int x = LPK; x < 64; x <<= 1) l += __shfl_xor(l, x);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float y = o[e] * w;
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) y += __shfl_xor(y, x);
    o[e] = y;
  }
  if (grp == 0) {  // lanes 0 .. LPK - 1 hold the wave's channels
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][8 * chunk + e] = o[e];
    if (chunk == 0) {
      red[wave][D] = mx;
      red[wave][D + 1] = l;
    }
  }
  __syncthreads();
  if (wave == 0) {
    float mw[4], lw[4], big = red[0][D];
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      mw[ww] = red[ww][D];
      lw[ww] = red[ww][D + 1];
      big = __builtin_fmaxf(big, mw[ww]);
    }
    float L = 0.0f, e[4];
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      e[ww] = fast_exp2(mw[ww] - big);
      L += e[ww] * lw[ww];
    }
    const bool real = L > 0.0f;
    const float inv = real ? 1.0f / L : 0.0f;
    const size_t row = (size_t)split * a.rows + bh;
#pragma unroll
    for (int t = 0; t < D / 64; ++t) {
      const int ch = lane + 64 * t;
      float y = 0.0f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) y += e[ww] * red[ww][ch];
      a.part_o[row * D + ch] = y * inv;
    }
    if (lane == 0) a.part_lse[row] = real ? (big + __builtin_log2f(L)) * kLn2 : -__builtin_inff();
  }
}

template <typename T, int D>
static hipError_t launch_decode_t(const FwdProblem& p, hipStream_t stream) {
  DecodeArgs a;
  a.q = p.q; a.k = p.k; a.v = p.v;
  a.seqlens_q = p.seqlens_q; a.seqlens_k = p.seqlens_k;
  a.Nk = p.Nk; a.H = p.H; a.splits = p.splits;
  const int per = (p.Nk + p.splits - 1) / p.splits;
  a.split_keys = (per + 127) / 128 * 128;
  a.rows = p.B * p.H;
  const float sc = p.scale;
  a.c = (sc < 0.0f ? -sc : sc) * kLog2e;
  a.flip = sc < 0.0f ? 0x80008000u : 0u;
  a.part_o = p.part;
  a.part_lse = p.part + (size_t)p.splits * a.rows * D;
  hipLaunchKernelGGL((decode_kernel<T, D>), dim3(a.rows * p.splits), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_split_merge(p, stream);
}

hipError_t launch_decode(const FwdProblem& p, hipStream_t s) {
  if (p.dtype == 1) return p.d == 64 ? launch_decode_t<_Float16, 64>(p, s) : launch_decode_t<_Float16, 128>(p, s);
  return p.d == 64 ? launch_decode_t<__bf16, 64>(p, s) : launch_decode_t<__bf16, 128>(p, s);
}

}  // namespace fa
