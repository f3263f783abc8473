// fa_fwd16.hip -- software-pipelined forward pass for 16-bit I/O (bf16, fp16) on gfx950.
//
// Same tiling as the generic forward (fa_fwd.hip): a workgroup of four waves
// owns 128 query rows of one (batch, head); each wave keeps its 32 Q rows in
// VGPRs and streams 64-key K/V tiles past them ("How Flash Attention Works:
// Tiling, Softmax, GPU I/O", sections "Tiling Q, K, and V for Fast On-Chip
// Memory" and "Online Softmax Without the Full Score Matrix").  What differs:
//
//  * K and V tiles go from device memory straight into LDS (buffer loads with
//    the LDS destination), two stages each, so no VGPRs or LDS-write
//    instructions are spent on staging.  Rows are packed back to back and the
//    16-byte chunks of row r are permuted by XOR with sw(r), which keeps both
//    the row-fragment reads of K and the transposing reads of V free of bank
//    conflicts.
//  * The work of tile j is software-pipelined against tile j-1 inside each
//    wave: after S_j = K_j Q^T, the exponentials of tile j are issued together
//    with the P_{j-1} V_{j-1} products, so the matrix cores run while the
//    vector ALUs evaluate the softmax (the overlap FlashAttention-3 gets from
//    warp specialisation on Hopper, "FlashAttention 1 vs 2 vs 3", done here
//    within one wave).
//  * Tiles that need no mask run a mask-free body whose LDS addresses are
//    compile-time offsets from a handful of per-lane base registers.
//  * In that body the exponentials are taken against the running maximum
//    before this tile's maximum is known; the row sums they produce bound
//    every p, so the maximum (a 30-instruction tree per lane) is only formed
//    when a sum shows that some p may exceed 2^8, and the tile is then redone
//    against the new maximum.  Either way each p is exp2 of its score minus a
//    maximum that is at most 8 below the true running one, as in the lazy
//    rescale of the generic kernel, and the result is the same softmax.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"
#include "fa_tile16.h"

namespace fa {

struct Fwd16Args {
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
  int nqb;
  int total;
  float c;
  int negate;
  // SPLIT kernels: key range split s covers tiles [s * split_tiles, (s + 1) * split_tiles)
  // and writes fp32 partial O [splits][B*H*Nq][D] and LSE [splits][B*H*Nq] instead of o / lse
  int splits, split_tiles;
  int rows;  // B * H * Nq
  float* part_o;
  float* part_lse;
};

// K-fragment reads kept in flight ahead of the score products (measured: 4
// and 8 within 1%, 12 slower)
constexpr int kFwdReadAhead = 4;

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP, bool SPLIT = false>
__global__ __launch_bounds__(256, 2) void fwd16_kernel(Fwd16Args a) {
  constexpr int BN = 64;  // keys per tile
  constexpr int KB = BN / 32;                      // 32-key blocks per tile
  using M = Mma<T>;
  using TL = Tile16<D, BN>;
  using Frag = typename M::Frag;
  constexpr int KSTEPS = D / 16;
  constexpr int MB = D / 32;
  constexpr int KREG = 0;               // LDS regions: [K0 K1 V0 V1]
  constexpr int VREG = 2 * TL::BYTES;

  __shared__ __attribute__((aligned(1024))) char smem[4 * TL::BYTES];

  const int tid = thread_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, col = lane & 31;
  const int Nq = a.Nq, Nk = a.Nk;

  int split = 0, bh, qb;
  if constexpr (SPLIT) {
    int bid = xcd_remap(block_id(), a.total);
    split = __builtin_amdgcn_readfirstlane(bid % a.splits);
    bid = __builtin_amdgcn_readfirstlane(bid / a.splits);
    bh = __builtin_amdgcn_readfirstlane(bid / a.nqb);
    qb = __builtin_amdgcn_readfirstlane(bid - bh * a.nqb);
  } else {
    block_order<(D == 64 ? 96 : 64)>(block_id(), a.total, a.nqb, CAUSAL, &bh, &qb);  // 3 (d = 64) or 2 workgroups per CU
  }
  if (CAUSAL) qb = a.nqb - 1 - qb;
  const int q0 = qb * 128;
  const int qw = q0 + wave * 32;
  const Seq sq = seq_of(a.seqlens_q, a.seqlens_k, bh / a.H, Nq, Nk);
  const T* __restrict__ Q = reinterpret_cast<const T*>(a.q) + (size_t)bh * (size_t)Nq * D;
  const char* Kg = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.k) + (size_t)bh * (size_t)Nk * D);
  const char* Vg = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.v) + (size_t)bh * (size_t)Nk * D);

  const int myq = qw + col;
  Frag qf[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    qf[ks] = myq < sq.lq ? row_frag<T>(Q + (size_t)myq * D + ks * 16, h) : zero_frag<T>();
    if (a.negate) qf[ks] = neg_frag<T>(qf[ks]);
  }

  // key tiles this block visits, and how many leading ones no real row sees masked
  int nt, nt_full;
  query_block_tiles<CAUSAL, BN>(sq, q0, 128, &nt, &nt_full);
  // split-key kernels visit tiles [tlo, nt) of their own range only
  int tlo = 0;
  if constexpr (SPLIT) {
    tlo = split * a.split_tiles;
    nt = __builtin_amdgcn_readfirstlane(nt < tlo + a.split_tiles ? nt : tlo + a.split_tiles);
    nt_full = nt_full < nt ? nt_full : nt;
  }
  const int lim = key_limit<CAUSAL>(sq, myq);
  const int wlast = qw + 31 + sq.off;  // causal: the last key any row of this wave may see
  // block-sparse: this query block's mask row, packed into bits in LDS; a key
  // tile is live unless its 128-key block is masked out
  constexpr int TPB = kMaskBlock / BN;  // key tiles per mask block
  __shared__ uint64_t mwords[SPARSE ? kMaxMaskWords : 1];
  if constexpr (SPARSE) {
    pack_mask_words(mwords, a.block_mask + ((size_t)bh * a.nqb + qb) * a.nbk, a.nbk, 1, lane, wave, 4);
    __syncthreads();
  }

  // ---- direct loads: lane's source offset inside a tile, per round
  uint32_t goff[TL::ROUNDS];
  tile16_load_offsets<D, BN>(goff, wave, lane);
  auto dma = [&](const char* g, int row0, int region) __attribute__((always_inline)) {
    const auto rs = buffer_rsrc(g + (size_t)row0 * TL::ROWB, tile_bytes(sq.lk - row0, BN, TL::ROWB));
#pragma unroll
    for (int i = 0; i < TL::ROUNDS; ++i)
      lds_load16(rs, smem + region + (i * 4 + wave) * 1024, goff[i]);
  };

  // ---- LDS read addresses (per lane), relative to smem
  uint32_t kaddr[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) kaddr[ks] = KREG + tile16_row_addr<D>(col, ks, h);
  uint32_t vaddr[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) vaddr[mb][hf] = VREG + tile16_tr_addr<D>(lane, mb, hf);
  auto kfrag = [&](int stage, int kb, int ks) __attribute__((always_inline)) {
    return tile16_row_frag<T>(smem, kaddr[ks] + stage * TL::BYTES + kb * 32 * TL::ROWB);
  };
  auto vfrag = [&](int stage, int kb, int t, int mb) __attribute__((always_inline)) {
    return tile16_tr_frag<T, D>(smem, vaddr[mb][0], vaddr[mb][1], stage * TL::BYTES + (32 * kb + 16 * t) * TL::ROWB);
  };

  f32x16 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) oacc[mb] = f32x16{};
  Frag pf[KB][2];  // P of the previous tile, [32-key block][k-step], waiting for its V
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t) pf[kb][t] = zero_frag<T>();
  float m = kMaxFloor;
  float l = 0.0f;
  const float c = a.c;

  // dropout: zero the weights of dropped keys in x (registers 8 t .. 8 t + 7
  // of 32-key block kb, keys k0 + 32 kb + acc_row(r, h)); 1 / (1 - p) is
  // applied with the final 1 / l
  auto drop_mask = [&](f32x16& x, int kb, int t, int k0) __attribute__((always_inline)) {
    if constexpr (DROP) {
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        const int j0 = k0 + 32 * kb + 8 * (2 * t + gg) + 4 * h;
        const u32x4v w = a.drop.words(j0 >> 2, myq, bh);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 8 * t + 4 * gg + u;
          x[r] = w[u] >= a.drop.threshold ? x[r] : 0.0f;
        }
      }
    }
  };

  auto pv = [&](int vstage) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) oacc[mb] = M::mma(vfrag(vstage, kb, t, mb), pf[kb][t], oacc[mb]);
  };

  // One pipeline step: S_j, softmax_j, and (if owed) O += P_jp V_jp, where jp is
  // the tile visited before j and jn the one visited after it (j - 1 and j + 1
  // unless block sparsity skips tiles).  KST alternates from step to step: K_j
  // sits in K stage KST, V_jp in V stage KST ^ 1.
  auto step = [&](int j, int jn, int jp, auto kst_tag, auto full_tag) __attribute__((always_inline)) {
    constexpr int KST = decltype(kst_tag)::value;
    // mode 1: unmasked, and tile jp was done (speculative exponentials);
    // mode 2: unmasked first tile (maximum first, nothing owed); mode 0: masked
    constexpr int MODE = decltype(full_tag)::value;
    constexpr bool FULL = MODE == 1;
    constexpr bool NOMASK = MODE != 0;
    wait_vmem();
    __builtin_amdgcn_s_barrier();
    if (jn < nt) dma(Kg, BN * jn, KREG + (KST ^ 1) * TL::BYTES);
    dma(Vg, BN * j, VREG + KST * TL::BYTES);

    const int k0 = BN * j;
    const bool act = NOMASK || !CAUSAL || k0 <= wlast;
    const bool prev = FULL || (jp >= 0 && (!CAUSAL || BN * jp <= wlast));
    if (act) {
      // Wave priority: low for the score products, raised again for the
      // element-wise phase.  The two waves of a SIMD alternate between these
      // phases; the products are long and independent (one issue per 32
      // cycles keeps the matrix core busy), while the softmax is a chain of
      // dependent VALU instructions whose issue delays stall its wave.
      // Measured against the opposite assignment: c4 +4.5%, c5 +5.7%.
      __builtin_amdgcn_s_setprio(0);
      f32x16 sc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sc[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sc[kb] = M::mma(kfrag(KST, kb, ks), qf[ks], sc[kb]);
      // keep kFwdReadAhead K-fragment reads in flight ahead of the matrix ops
      __builtin_amdgcn_sched_group_barrier(0x100, kFwdReadAhead, 0);
#pragma unroll
      for (int i = 0; i < KB * KSTEPS - kFwdReadAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kFwdReadAhead, 0);
      __builtin_amdgcn_s_setprio(1);
      if constexpr (FULL) {
        // Unmasked tile: exponentiate against the running maximum m without
        // looking for this tile's maximum first. If a lane's partial row sum
        // stays <= 2^8, every p is <= 2^8, which is the bound the lazy rescale
        // keeps anyway. Otherwise (rare) redo the tile against the new maximum.
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
            const float s8 = sum8(p8, 8 * t);  // pairwise: dependency depth 3, not a chain of 8
            rs = (kb == 0 && t == 0) ? s8 : rs + s8;
            drop_mask(p8, kb, t, k0);
            pf[kb][t] = acc_frag<T>(p8, t);
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
              drop_mask(p8, kb, t, k0);
              pf[kb][t] = acc_frag<T>(p8, t);
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
      float xs[KB * 16];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ro = 8 * (r >> 2) + (r & 3);
          float x = sc[kb][r];
          if constexpr (!NOMASK) x = ro <= t0 - 32 * kb ? x : -__builtin_inff();
          xs[16 * kb + r] = x;
        }
      // 3-input max tree over the lane's scores
      float mx = __builtin_fmaxf(xs[0], __builtin_fmaxf(xs[1], xs[2]));
#pragma unroll
      for (int r = 3; r + 1 < KB * 16; r += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(xs[r], xs[r + 1]));
      mx = __builtin_fmaxf(mx, xs[KB * 16 - 1]);
      mx = halves_max(mx);
      float mt = mx * c;
      if constexpr (!NOMASK) mt = mx > -__builtin_inff() ? mt : -__builtin_inff();
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
          float p = fast_exp2(__builtin_fmaf(sc[kb][r], c, negm));
          if constexpr (!NOMASK) {
            const int ro = 8 * (r >> 2) + (r & 3);
            p = ro <= t0 - 32 * kb ? p : 0.0f;
          }
          sc[kb][r] = p;
        }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) rs += sum8(sc[kb], 0) + sum8(sc[kb], 8);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) drop_mask(sc[kb], kb, t, k0);
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
        for (int t = 0; t < 2; ++t) pf[kb][t] = acc_frag<T>(sc[kb], t);
    } else if (prev) {
      pv(KST ^ 1);
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  if constexpr (!SPARSE) {
    // tile j sits in stage (j - tlo) & 1; tlo = 0 except in split-key kernels
    if (nt > tlo) {  // (nt and tlo are block-uniform: every wave takes the same barriers)
      dma(Kg, BN * tlo, KREG);
      if (tlo < nt_full)
        step(tlo, tlo + 1, -1, I0{}, I2{});
      else
        step(tlo, tlo + 1, -1, I0{}, I0{});
      int j = tlo + 1;
      for (; j + 1 < nt_full; j += 2) {
        step(j, j + 1, j - 1, I1{}, I1{});
        step(j + 1, j + 2, j, I0{}, I1{});
      }
      if (j < nt_full) {
        step(j, j + 1, j - 1, I1{}, I1{});
        ++j;
      }
      for (; j < nt; ++j) {
        if ((j - tlo) & 1)
          step(j, j + 1, j - 1, I1{}, I0{});
        else
          step(j, j + 1, j - 1, I0{}, I0{});
      }
      // the last tile's P still owes its V product
      wait_vmem();
      __builtin_amdgcn_s_barrier();
      if (!CAUSAL || BN * (nt - 1) <= wlast) {
        if ((nt - 1 - tlo) & 1)
          pv(1);
        else
          pv(0);
      }
    }
  } else {
    // Only live tiles are visited; steps alternate stages as in the dense
    // loop, and a step is unmasked when its tile (and so the previous one,
    // visited in increasing order) lies below nt_full.
    auto next = [&](int j) __attribute__((always_inline)) { return next_live_tile(mwords, j, TPB, a.nbk, nt); };
    int j = next(-1);
    if (j < nt) {
      dma(Kg, BN * j, KREG);
      int jp = -1, jn = next(j);
      if (j < nt_full)
        step(j, jn, jp, I0{}, I2{});
      else
        step(j, jn, jp, I0{}, I0{});
      jp = j; j = jn;
      int par = 1;  // stage parity of the next step
      while (j < nt_full) {
        jn = next(j);
        step(j, jn, jp, I1{}, I1{});
        jp = j; j = jn;
        if (j >= nt_full) {
          par = 0;
          break;
        }
        jn = next(j);
        step(j, jn, jp, I0{}, I1{});
        jp = j; j = jn;
      }
      for (; j < nt; par ^= 1) {
        jn = next(j);
        if (par)
          step(j, jn, jp, I1{}, I0{});
        else
          step(j, jn, jp, I0{}, I0{});
        jp = j; j = jn;
      }
      // the last visited tile's P still owes its V product (stage par ^ 1)
      wait_vmem();
      __builtin_amdgcn_s_barrier();
      if (!CAUSAL || BN * jp <= wlast) {
        if (par ^ 1)
          pv(1);
        else
          pv(0);
      }
    }
  }

  // padding rows and rows that see no key store O = 0, LSE = -inf
  l = halves_sum(l);
  if constexpr (SPLIT) {
    // this key range's normalised partial output and its LSE, both fp32
    if (myq < Nq) {
      const bool real = myq < sq.lq && l > 0.0f;
      const float inv = real ? 1.0f / l : 0.0f;
      const size_t row = (size_t)split * a.rows + (size_t)bh * Nq + myq;
      float* prow = a.part_o + row * D;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = 32 * mb + 8 * g + 4 * h;
          f32x4 o4;
#pragma unroll
          for (int u = 0; u < 4; ++u) o4[u] = real ? oacc[mb][4 * g + u] * inv : 0.0f;
          *reinterpret_cast<f32x4*>(prow + d0) = o4;
        }
      if (h == 0) a.part_lse[row] = real ? (m + __builtin_log2f(l)) * kLn2 : -__builtin_inff();
    }
    return;
  }
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

// Merge of split-key partials: one wave per row.  With M = max_s LSE_s and
// w_s = exp(LSE_s - M): LSE = M + ln sum_s w_s and O = sum_s w_s O_s / sum_s w_s,
// the same rescale the online softmax applies tile by tile.
template <typename T, int D>
__global__ __launch_bounds__(256) void split_merge_kernel(const float* part_o, const float* part_lse, int splits,
                                                          int rows, T* o, float* lse) {
  constexpr int PER = D / 64;  // channels per lane
  const int lane = thread_id() & 63;
  const int row = __builtin_amdgcn_readfirstlane(block_id() * 4 + (thread_id() >> 6));
  if (row >= rows) return;
  float mx = -__builtin_inff();
  for (int sp = 0; sp < splits; ++sp) mx = __builtin_fmaxf(mx, part_lse[(size_t)sp * rows + row]);
  float acc[PER] = {}, wsum = 0.0f;
  if (mx > -__builtin_inff()) {
    for (int sp = 0; sp < splits; ++sp) {
      const float ls = part_lse[(size_t)sp * rows + row];
      const float w = ls > -__builtin_inff() ? fast_exp2((ls - mx) * kLog2e) : 0.0f;
      wsum += w;
      const float* po = part_o + ((size_t)sp * rows + row) * D + lane * PER;
#pragma unroll
      for (int u = 0; u < PER; ++u) acc[u] += w * po[u];
    }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  T* orow = o + (size_t)row * D + lane * PER;
#pragma unroll
  for (int u = 0; u < PER; ++u) orow[u] = (T)(acc[u] * inv);
  if (lse != nullptr && lane == 0) lse[row] = wsum > 0.0f ? mx + __builtin_log2f(wsum) * kLn2 : -__builtin_inff();
}

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP, bool SPLIT = false>
static hipError_t launch_fwd16_t(const FwdProblem& p, hipStream_t stream) {
  Fwd16Args a;
  a.q = p.q; a.k = p.k; a.v = p.v; a.o = p.o; a.lse = p.lse;
  a.seqlens_q = p.seqlens_q; a.seqlens_k = p.seqlens_k;
  a.Nq = p.Nq; a.Nk = p.Nk; a.H = p.H;
  a.block_mask = p.block_mask;
  a.nbk = (p.Nk + kMaskBlock - 1) / kMaskBlock;
  a.drop = Dropout{p.drop_threshold, p.drop_seed_lo, p.drop_seed_hi, p.drop_offset, p.drop_scale};
  a.nqb = (p.Nq + 127) / 128;
  static_assert(kMaskBlock == 128, "one workgroup's 128 query rows are one mask block row");
  a.total = a.nqb * p.B * p.H;
  const float sc = p.scale;
  a.negate = sc < 0.0f;
  a.c = (sc < 0.0f ? -sc : sc) * kLog2e;
  a.splits = 1; a.split_tiles = 0; a.rows = p.B * p.H * p.Nq; a.part_o = nullptr; a.part_lse = nullptr;
  if constexpr (SPLIT) {
    a.splits = p.splits;
    const int tiles = (p.Nk + 63) / 64;
    a.split_tiles = (tiles + p.splits - 1) / p.splits;
    a.part_o = p.part;
    a.part_lse = p.part + (size_t)p.splits * a.rows * D;
    a.total *= p.splits;
    hipLaunchKernelGGL((fwd16_kernel<T, D, CAUSAL, false, false, true>), dim3(a.total), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_split_merge(p, stream);
  }
  hipLaunchKernelGGL((fwd16_kernel<T, D, CAUSAL, SPARSE, DROP>), dim3(a.total), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Every 16-bit forward variant for one head size D.  (Block sparsity,
// dropout and key splitting are not combined: the API rejects that.)
template <typename T, int D>
static hipError_t launch_fwd16_dd(const FwdProblem& p, hipStream_t s) {
  const bool c = p.causal;
  if (p.splits > 1)
    return c ? launch_fwd16_t<T, D, true, false, false, true>(p, s) : launch_fwd16_t<T, D, false, false, false, true>(p, s);
  if (p.drop_on) return c ? launch_fwd16_t<T, D, true, false, true>(p, s) : launch_fwd16_t<T, D, false, false, true>(p, s);
  if (p.block_mask != nullptr)
    return c ? launch_fwd16_t<T, D, true, true, false>(p, s) : launch_fwd16_t<T, D, false, true, false>(p, s);
  return c ? launch_fwd16_t<T, D, true, false, false>(p, s) : launch_fwd16_t<T, D, false, false, false>(p, s);
}

#ifndef FA_FWD16_D128_UNIT
template <typename T, int D>
static hipError_t launch_split_merge_t(const FwdProblem& p, hipStream_t s) {
  const int rows = p.B * p.H * p.Nq;
  const float* po = p.part;
  const float* pl = p.part + (size_t)p.splits * rows * D;
  hipLaunchKernelGGL((split_merge_kernel<T, D>), dim3((rows + 3) / 4), dim3(256), 0, s, po, pl, p.splits, rows,
                     reinterpret_cast<T*>(p.o), p.lse);
  return hipGetLastError();
}

hipError_t launch_split_merge(const FwdProblem& p, hipStream_t s) {
  if (p.dtype == 1) return p.d == 64 ? launch_split_merge_t<_Float16, 64>(p, s) : launch_split_merge_t<_Float16, 128>(p, s);
  return p.d == 64 ? launch_split_merge_t<__bf16, 64>(p, s) : launch_split_merge_t<__bf16, 128>(p, s);
}

// d = 128 is instantiated in fa_fwd16_d128.hip, a unit compiled with other
// scheduling; this unit holds d = 64 and the split-key merge.
hipError_t launch_fwd16(const FwdProblem& p, hipStream_t s) {
  if (p.splits > 1 && p.Nq == 1) return launch_decode(p, s);  // one query row per head
  if (p.d == 128) return launch_fwd16_128(p, s);
  return p.dtype == 1 ? launch_fwd16_dd<_Float16, 64>(p, s) : launch_fwd16_dd<__bf16, 64>(p, s);
}
#else
hipError_t launch_fwd16_128(const FwdProblem& p, hipStream_t s) {
  return p.dtype == 1 ? launch_fwd16_dd<_Float16, 128>(p, s) : launch_fwd16_dd<__bf16, 128>(p, s);
}
#endif

}  // namespace fa
