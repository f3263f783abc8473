// fa_fwd8.hip -- forward pass for OCP E4M3 or E5M2 (8-bit) inputs on the gfx950 matrix cores.
//
// The schedule is the 16-bit forward's (fa_fwd16.hip): a workgroup of four
// waves owns 128 query rows of one (batch, head), 64-key K/V tiles stream
// through LDS by direct loads, S^T = K Q^T keeps the query as the accumulator's
// lane column, the softmax is online with the speculative exponentials, and
// the P V products of tile j-1 are issued beside the softmax of tile j ("How
// Flash Attention Works: Tiling, Softmax, GPU I/O", sections "Tiling Q, K, and
// V for Fast On-Chip Memory" and "Online Softmax Without the Full Score
// Matrix").  What differs is the operand format, the lower-precision path the
// same page attributes to FlashAttention 3 ("FlashAttention 1 vs 2 vs 3"):
//
//  * Both products run on v_mfma_scale_f32_32x32x64_f8f6f4 with unit block
//    scales: 64 contraction elements per instruction at twice the 16-bit rate.
//    The instruction takes each operand's format separately, so q, k and v
//    may be E4M3 or E5M2 (FMT) while P, packed here, is always E4M3.  A lane supplies 32 bytes per operand, and the hardware
//    pairs operand slots by (half-wave, byte), so the contraction index may be
//    assigned to slots freely as long as both operands agree.
//  * For P V the slot (h, e = 16 kb + 4 g + u) holds key 32 kb + 8 g + 4 h + u:
//    exactly the keys the score accumulators leave in a lane, so P is packed
//    from registers (v_cvt_pk_fp8_f32, round to nearest even) without moving.
//    The lazy rescale keeps every p <= 2^8, inside E4M3's range of 448.
//  * V^T fragments come from ds_read_b64_tr_b8: within 16 lanes, lane i
//    receives byte i mod 8 of the 8-byte rows addressed by lanes 2 e + i / 8,
//    so each lane gathers one channel of 8 keys per read.
//  * The dequantisation factors of q and k fold into the exponent scale, that
//    of v into the final 1 / l; O is written in bf16.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tile16.h"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// Transposing 8-bit LDS read.  Like lds_tr16 (fa_tile16.h), the pointer is
// restrict-qualified so the read is not ordered behind the direct loads in
// flight into other LDS stages; each step waits for those loads explicitly
// before any wave reads the stage they fill.
__device__ __attribute__((always_inline)) inline i32x2 lds_tr8(const char* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p);
}

struct Fwd8Args {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int N, nqb, total;
  float c;          // |scale * descale_q * descale_k| * log2(e)
  int negate;       // that product is negative: flip the sign bit of q
  float descale_v;
};

// A tile of 64 rows of D bytes, filled by direct loads that write 1 KiB per
// wave instruction contiguously; the 16-byte chunks of row r sit XOR-permuted
// by sw(r).  With 64 banks of 4 bytes, sw makes both read patterns
// conflict-free: 16 lanes reading the same chunk of 16 consecutive rows (K
// fragments, ds_read_b128), and 32 lanes reading 8 bytes each from two
// adjacent chunks of the 8 rows {b .. b+3, b+8 .. b+11} (V^T fragments,
// ds_read_b64_tr_b8, b a multiple of 4).
template <int D>
struct Tile8 {
  static constexpr int ROWS = 64;
  static constexpr int ROWB = D;
  static constexpr int CPR = D / 16;          // 16-byte chunks per row: 8 or 4
  static constexpr int BYTES = ROWS * ROWB;   // 8 or 4 KiB
  static constexpr int ROUNDS = BYTES / 4096; // direct loads per tile per wave (4 waves)
  __device__ static constexpr int sw(int r) {
    return CPR == 8 ? (((r >> 2) & 1) | (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2)) : ((r >> 2) & 3);
  }
  __device__ static constexpr int phys(int r, int chunk) { return r * ROWB + ((chunk ^ sw(r)) << 4); }
};

// Operand format codes of the instruction: 0 = E4M3, 1 = E5M2.
constexpr int kE4M3 = 0;
constexpr int kE5M2 = 1;

template <int FA, int FB>
__device__ inline f32x16 mma8(i32x8 a, i32x8 b, f32x16 c) {
  // formats of A and B; block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 127, 0, 127);
}

// Four floats to four E4M3 bytes (round to nearest even), first in the low byte.
__device__ inline int pack_e4m3(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

template <int D, bool CAUSAL, int FMT>
__global__ __launch_bounds__(256, 2) void fwd8_kernel(Fwd8Args a) {
  constexpr int BN = 64;  // keys per tile
  constexpr int KB = 2;   // 32-key blocks per tile
  using TL = Tile8<D>;
  constexpr int KSTEPS = D / 64;  // S products per 32-key block
  constexpr int MB = D / 32;      // 32-channel blocks of O
  constexpr int KREG = 0;         // LDS regions: [K0 K1 V0 V1]
  constexpr int VREG = 2 * TL::BYTES;

  __shared__ __attribute__((aligned(1024))) char smem[4 * TL::BYTES];

  const int tid = thread_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int N = a.N;

  int bh, qb;
  block_order<64>(block_id(), a.total, a.nqb, CAUSAL, &bh, &qb);
  if (CAUSAL) qb = a.nqb - 1 - qb;
  const int q0 = qb * 128;
  const int qw = q0 + wave * 32;
  const Seq sq{N, N, 0};
  const size_t head = (size_t)bh * (size_t)N * D;
  const unsigned char* Q = reinterpret_cast<const unsigned char*>(a.q) + head;
  const char* Kg = reinterpret_cast<const char*>(a.k) + head;
  const char* Vg = reinterpret_cast<const char*>(a.v) + head;

  // Q^T operand: lane (query myq, half h) holds bytes [64 ks + 32 h, + 32) of its row
  const int myq = qw + col;
  i32x8 qf[KSTEPS];
  const uint32_t flip = a.negate ? 0x80808080u : 0u;
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    u32x4 lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
    if (myq < N) {
      const u32x4* p = reinterpret_cast<const u32x4*>(Q + (size_t)myq * D + 64 * ks + 32 * h);
      lo = p[0] ^ flip;
      hi = p[1] ^ flip;
    }
    qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }

  int nt, nt_full;
  query_block_tiles<CAUSAL, BN>(sq, q0, 128, &nt, &nt_full);
  const int lim = key_limit<CAUSAL>(sq, myq);
  const int wlast = qw + 31;  // causal: the last key any row of this wave may see

  // ---- direct loads: lane's source offset inside a tile, per round
  uint32_t goff[TL::ROUNDS];
#pragma unroll
  for (int i = 0; i < TL::ROUNDS; ++i) {
    const int s = (i * 4 + wave) * 64 + lane;
    const int r = s / TL::CPR, pc = s % TL::CPR;
    goff[i] = r * TL::ROWB + ((pc ^ TL::sw(r)) << 4);
  }
  auto dma = [&](const char* g, int row0, int region) __attribute__((always_inline)) {
    const auto rs = buffer_rsrc(g + (size_t)row0 * TL::ROWB, tile_bytes(sq.lk - row0, BN, TL::ROWB));
#pragma unroll
    for (int i = 0; i < TL::ROUNDS; ++i) lds_load16(rs, smem + region + (i * 4 + wave) * 1024, goff[i]);
  };

  // ---- LDS read addresses (per lane), relative to smem
  // K operand: key col of the 32-key block, bytes [64 ks + 32 h, + 32) = chunks 4 ks + 2 h, + 1
  uint32_t kaddr[KSTEPS][2];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
    for (int j = 0; j < 2; ++j) kaddr[ks][j] = KREG + TL::phys(col, 4 * ks + 2 * h + j);
  // V^T operand, read t (bytes 8 t .. 8 t + 7 of the lane's 32): this lane
  // addresses row 2 e + par of its 16-lane group's read, i.e. key
  // 16 t + 8 (e / 4) + 4 h + e % 4, channels 32 mb + 16 (group & 1) + 8 par + 0..7
  uint32_t vaddr[MB];
  {
    const int rho = lane & 15, e = rho >> 1, par = rho & 1;
    const int key = 8 * (e >> 2) + 4 * h + (e & 3);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) vaddr[mb] = VREG + TL::phys(key, 2 * mb + ((lane >> 4) & 1)) + 8 * par;
  }
  auto kfrag = [&](int stage, int kb, int ks) __attribute__((always_inline)) {
    const int off = stage * TL::BYTES + kb * 32 * TL::ROWB;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(smem + kaddr[ks][0] + off);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(smem + kaddr[ks][1] + off);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto vfrag = [&](int stage, int mb) __attribute__((always_inline)) {
    i32x2 r[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      r[t] = lds_tr8(smem + vaddr[mb] + stage * TL::BYTES + 16 * t * TL::ROWB);
    return i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
  };

  f32x16 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) oacc[mb] = f32x16{};
  i32x8 pf = i32x8{0, 0, 0, 0, 0, 0, 0, 0};  // P of the previous tile, waiting for its V
  float m = kMaxFloor;
  float l = 0.0f;
  const float c = a.c;

  auto pv = [&](int vstage) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) oacc[mb] = mma8<FMT, kE4M3>(vfrag(vstage, mb), pf, oacc[mb]);
  };
  // registers 8 t .. 8 t + 7 of block kb (keys 32 kb + 8 g + 4 h + u, g = 2 t, 2 t + 1)
  // are P slots 16 kb + 8 t .. + 7, i.e. dwords 4 kb + 2 t and 4 kb + 2 t + 1
  auto pack_half = [&](const f32x16& x, int kb, int t) __attribute__((always_inline)) {
    pf[4 * kb + 2 * t] = pack_e4m3(x[8 * t], x[8 * t + 1], x[8 * t + 2], x[8 * t + 3]);
    pf[4 * kb + 2 * t + 1] = pack_e4m3(x[8 * t + 4], x[8 * t + 5], x[8 * t + 6], x[8 * t + 7]);
  };

  // One pipeline step: S_j, softmax_j, and (if owed) O += P_{j-1} V_{j-1}.
  // KST alternates: K_j sits in K stage KST, V_{j-1} in V stage KST ^ 1.
  auto step = [&](int j, auto kst_tag, auto full_tag) __attribute__((always_inline)) {
    constexpr int KST = decltype(kst_tag)::value;
    constexpr bool FULL = decltype(full_tag)::value;  // unmasked, and tile j-1 was done
    wait_vmem();
    __builtin_amdgcn_s_barrier();
    if (j + 1 < nt) dma(Kg, BN * (j + 1), KREG + (KST ^ 1) * TL::BYTES);
    dma(Vg, BN * j, VREG + KST * TL::BYTES);

    const int k0 = BN * j;
    const bool act = FULL || !CAUSAL || k0 <= wlast;
    const bool prev = FULL || (j > 0 && (!CAUSAL || BN * (j - 1) <= wlast));
    if (act) {
      __builtin_amdgcn_s_setprio(1);
      f32x16 sc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sc[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sc[kb] = mma8<FMT, FMT>(kfrag(KST, kb, ks), qf[ks], sc[kb]);
      __builtin_amdgcn_s_setprio(0);
      if constexpr (FULL) {
        // unmasked tile: exponentiate against the running maximum first; a
        // lane row sum <= 2^8 bounds every p by 2^8, else redo with the new maximum
        pv(KST ^ 1);
        const float negm = -m;
        float rs = 0.0f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            f32x16 p8;
#pragma unroll
            for (int e = 0; e < 8; ++e) p8[8 * t + e] = fast_exp2(__builtin_fmaf(sc[kb][8 * t + e], c, negm));
            const float s8 = sum8(p8, 8 * t);
            rs = (kb == 0 && t == 0) ? s8 : rs + s8;
            pack_half(p8, kb, t);
          }
        if (any_lane(rs > 256.0f)) {
          float mx = sc[0][0];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, sc[kb][r]);
          const float mnew = __builtin_fmaxf(m, halves_max(mx) * c);
          const float alpha = fast_exp2(m - mnew);
          rs = 0.0f;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              f32x16 p8;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                p8[8 * t + e] = fast_exp2(__builtin_fmaf(sc[kb][8 * t + e], c, -mnew));
                rs += p8[8 * t + e];
              }
              pack_half(p8, kb, t);
            }
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;
          l *= alpha;
          m = mnew;
        }
        l += rs;
        return;
      }
      // key of register r in block kb is k0 + 32 kb + acc_row(r, h); allowed iff <= lim
      const int t0 = lim - k0 - 4 * h;
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ro = 8 * (r >> 2) + (r & 3);
          mx = __builtin_fmaxf(mx, ro <= t0 - 32 * kb ? sc[kb][r] : -__builtin_inff());
        }
      mx = halves_max(mx);
      const float mt = mx > -__builtin_inff() ? mx * c : -__builtin_inff();
      const bool need = any_lane(mt > m + 8.0f);
      const float mnew = need ? __builtin_fmaxf(m, mt) : m;
      const float alpha = fast_exp2(m - mnew);
      const float negm = -mnew;
      if (prev) pv(KST ^ 1);
      float rs = 0.0f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ro = 8 * (r >> 2) + (r & 3);
          const float p = fast_exp2(__builtin_fmaf(sc[kb][r], c, negm));
          sc[kb][r] = ro <= t0 - 32 * kb ? p : 0.0f;
        }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) rs += sum8(sc[kb], 0) + sum8(sc[kb], 8);
      if (need) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;
        l *= alpha;
      }
      l += rs;
      m = mnew;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) pack_half(sc[kb], kb, t);
    } else if (prev) {
      pv(KST ^ 1);
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if (nt > 0) {  // (nt is block-uniform: every wave takes the same barriers)
    dma(Kg, 0, KREG);
    step(0, I0{}, std::false_type{});
    int j = 1;
    for (; j + 1 < nt_full; j += 2) {
      step(j, I1{}, std::true_type{});
      step(j + 1, I0{}, std::true_type{});
    }
    if (j < nt_full) {
      step(j, I1{}, std::true_type{});
      ++j;
    }
    for (; j < nt; ++j) {
      if (j & 1)
        step(j, I1{}, std::false_type{});
      else
        step(j, I0{}, std::false_type{});
    }
    // the last tile's P still owes its V product
    wait_vmem();
    __builtin_amdgcn_s_barrier();
    if (!CAUSAL || BN * (nt - 1) <= wlast) {
      if ((nt - 1) & 1)
        pv(1);
      else
        pv(0);
    }
  }

  l = halves_sum(l);
  if (myq < N) {
    const bool real = l > 0.0f;
    const float inv = real ? a.descale_v / l : 0.0f;
    __bf16* orow = reinterpret_cast<__bf16*>(a.o) + head + (size_t)myq * D;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * mb + 8 * g + 4 * h;
        store4<__bf16>(orow + d0, oacc[mb][4 * g] * inv, oacc[mb][4 * g + 1] * inv, oacc[mb][4 * g + 2] * inv,
                       oacc[mb][4 * g + 3] * inv);
      }
    if (a.lse != nullptr && h == 0)
      a.lse[(size_t)bh * N + myq] = real ? (m + __builtin_log2f(l)) * kLn2 : -__builtin_inff();
  }
}

template <int D, bool CAUSAL, int FMT>
static hipError_t launch_fwd8_t(const FwdProblem& p, hipStream_t stream) {
  Fwd8Args a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o; a.lse = p.lse;
  a.N = p.Nq;
  a.nqb = (p.Nq + 127) / 128;
  a.total = a.nqb * p.B * p.H;
  const float sc = p.scale;
  a.negate = sc < 0.0f;
  a.c = (sc < 0.0f ? -sc : sc) * kLog2e;
  a.descale_v = p.descale_v;
  hipLaunchKernelGGL((fwd8_kernel<D, CAUSAL, FMT>), dim3(a.total), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_fwd8_f(const FwdProblem& p, hipStream_t s) {
  if (p.d == 64) return p.causal ? launch_fwd8_t<64, true, FMT>(p, s) : launch_fwd8_t<64, false, FMT>(p, s);
  return p.causal ? launch_fwd8_t<128, true, FMT>(p, s) : launch_fwd8_t<128, false, FMT>(p, s);
}

hipError_t launch_fwd8(const FwdProblem& p, hipStream_t s) {
  return p.fp8_format == kE5M2 ? launch_fwd8_f<kE5M2>(p, s) : launch_fwd8_f<kE4M3>(p, s);
}

}  // namespace fa
