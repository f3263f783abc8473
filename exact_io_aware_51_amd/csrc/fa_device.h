// fa_device.h -- device-side building blocks for the gfx950 attention kernels.
//
// Matrix-core conventions (CDNA4, wave64), checked lane by lane on gfx950:
//   v_mfma_f32_32x32x16_{bf16,f16}: C[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[l%32][8*(l/32) + e], e = 0..7
//     B: lane l holds B[8*(l/32) + e][l%32]
//     C: lane l, register r holds C[8*(r/4) + 4*(l/32) + r%4][l%32]
//   v_mfma_f32_32x32x2_f32: the same with one element per lane (k = l/32).
// So a 32x32 accumulator gives each lane one column j = l%32 and 16 rows.
// Every kernel here computes products with that column standing for the
// query (or key) the lane owns, so row reductions stay inside a lane plus
// one swap between the two half-waves.
//
// The contraction index of a second product can be permuted freely as long
// as both operands use the same permutation.  Feeding a 32x32 accumulator
// (converted to the I/O type) straight in as the B operand uses the
// permutation "logical k = 8h + e  <->  physical index 8*(r/4) + 4h + r%4"
// (r = 8t + e for k-step t), which the transposed A operand then reads with
// ds_read_b64_tr_b16.  Semantics of that instruction on gfx950, per group of
// 16 lanes: if lane j's address points at four 16-bit values M[j][0..3], lane
// i receives M[4e + i/4][i%4] in element e.  Pointing lane j at row
// (base + j/4), columns (c0 + 4*(j%4) .. +3) therefore hands lane i the four
// rows base..base+3 of column c0 + i: a 4x16 transpose for free.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running-max floor: finite, so that exp2(m_old - m_new) never sees inf - inf.
constexpr float kMaxFloor = -1.0e30f;

// ---------------------------------------------------------------------------
// Matrix-core traits per element type.  KS = contraction elements per MFMA;
// each lane supplies KS/2 consecutive contraction elements.
template <typename T> struct Mma;

template <> struct Mma<__bf16> {
  static constexpr int KS = 16;
  using Frag = bf16x8;
  __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<_Float16> {
  static constexpr int KS = 16;
  using Frag = f16x8;
  __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int KS = 2;
  using Frag = float;
  __device__ static inline f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// The 16x16x32 instruction for 16-bit operands (same rate per flop), checked
// lane by lane on gfx950:
//   A: lane l holds A[l%16][8*(l/16) + e], B: lane l holds B[8*(l/16) + e][l%16],
//   C: lane l, register r holds C[4*(l/16) + r][l%16].
template <typename T> struct Mma16;

template <> struct Mma16<__bf16> {
  using Frag = bf16x8;
  __device__ static inline f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma16<_Float16> {
  using Frag = f16x8;
  __device__ static inline f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// Fragment loads.

// "Row" fragment: the KS/2 contraction elements lane l supplies, taken from a
// row stored contiguously (global or LDS).  p points at element (row, k0) of
// the lane's own row; the lane's half h = l/32 selects the sub-chunk.
template <typename T>
__device__ inline typename Mma<T>::Frag row_frag(const T* p, int h) {
  if constexpr (sizeof(T) == 2) {
    u32x4 raw = *reinterpret_cast<const u32x4*>(p + 8 * h);
    return __builtin_bit_cast(typename Mma<T>::Frag, raw);
  } else {
    return p[h];
  }
}

template <typename T>
__device__ inline typename Mma<T>::Frag zero_frag() {
  if constexpr (sizeof(T) == 2) {
    u32x4 z = {0u, 0u, 0u, 0u};
    return __builtin_bit_cast(typename Mma<T>::Frag, z);
  } else {
    return 0.0f;
  }
}

template <typename T>
__device__ inline typename Mma<T>::Frag neg_frag(typename Mma<T>::Frag f) {
  if constexpr (sizeof(T) == 2) {
    u32x4 raw = __builtin_bit_cast(u32x4, f);
    raw ^= 0x80008000u;  // exact sign flip of every 16-bit element
    return __builtin_bit_cast(typename Mma<T>::Frag, raw);
  } else {
    return -f;
  }
}

// Transposed A fragment for a product whose contraction runs over the rows of
// a row-major LDS tile (V in P*V, dO in dO^T*P, Q in Q^T*dS, K in K^T*dS).
//   tile    : LDS tile base, row stride `stride` elements
//   row0    : first row of the 32-row block being contracted
//   t       : k-step inside the block (16-bit: 0..1, fp32: 0..15)
//   col0    : first column of the 32-column output block (M index)
// Row order follows the accumulator permutation described at the top.
template <typename T>
__device__ inline typename Mma<T>::Frag trans_frag(const T* tile, int stride, int row0, int t,
                                                   int col0, int lane) {
  const int h = lane >> 5;
  if constexpr (sizeof(T) == 2) {
    const int i = lane & 15;
    const int cb = col0 + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
    const int rb = row0 + 16 * t + 4 * h + (i >> 2);
    const T* p0 = tile + rb * stride + cb;
    const T* p1 = p0 + 8 * stride;
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(typename Mma<T>::Frag, both);
  } else {
    const int row = row0 + 8 * (t >> 2) + 4 * h + (t & 3);
    return tile[row * stride + col0 + (lane & 31)];
  }
}

// B fragment from a 32x32 fp32 accumulator (k-step t), rounded to T.
template <typename T>
__device__ inline typename Mma<T>::Frag acc_frag(const f32x16& c, int t) {
  if constexpr (sizeof(T) == 2) {
    typename Mma<T>::Frag f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (T)c[8 * t + e];
    return f;
  } else {
    return c[t];
  }
}

// Row (within a 32-row accumulator block) held in register r by half h.
__device__ constexpr inline int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Combine a value with its copy in lane l ^ 32 (the other half-wave) without
// touching LDS.  v_permlane32_swap exchanges one half of each operand with the
// other, so of the two results one is x and the other is the partner's x;
// max and sum of the pair are therefore the same in every lane.
__device__ inline float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum of registers o .. o + 7 of an accumulator, pairwise (dependency depth 3).
__device__ inline float sum8(const f32x16& x, int o) {
  return ((x[o] + x[o + 1]) + (x[o + 2] + x[o + 3])) + ((x[o + 4] + x[o + 5]) + (x[o + 6] + x[o + 7]));
}

// Blocks are dispatched round-robin over the 8 XCDs (blockIdx % 8 = XCD).
// Renumber them so that consecutive logical indices share an XCD (and so its
// L2): XCD x receives logical blocks [x*q + min(x, r), ...) in order.
// Work-item and work-group ids straight from the hardware registers.  The
// kernels are built with IEEE mode off, which the device library is not, and
// LLVM does not inline across that difference: threadIdx / blockIdx (and
// __umulhi) would become real calls, turning every kernel into a non-leaf
// function.
__device__ __attribute__((always_inline)) inline int thread_id() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __attribute__((always_inline)) inline int block_id() { return (int)__builtin_amdgcn_workgroup_id_x(); }

__device__ inline int xcd_remap(int bid, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = bid & 7, local = bid >> 3;
  return x * q + (x < r ? x : r) + local;
}

// Head and rank of a workgroup in a grid of nblk blocks per head over
// total / nblk heads.  Rank 0 is the block with the most tiles under the
// causal mask; a kernel maps it to its own block index.
//  * equal-cost blocks (no causal mask): xcd_remap order, so each XCD's L2
//    serves few heads;
//  * causal: heads in groups, ranks in order across the heads of a group
//    (longest first), groups one after another.  Workgroups are dispatched
//    round-robin over the 8 XCDs (bid % 8), so a group of 8 g heads gives each
//    XCD g heads, and g = ceil(SLOTS / nblk) (SLOTS: workgroups one XCD runs
//    at once) is the fewest that still fills an XCD with blocks in
//    longest-first order.  Ordering each head on its own instead left an XCD
//    with its first heads' short blocks in the early slots and its last
//    heads' longest blocks running last (c5-shape forward: makespan 102
//    tile-times vs 70 in a list-scheduling model of one XCD); ordering by rank
//    across all heads fixed that but kept every head of an XCD active at once,
//    and the L2 then missed on 25-43% more bytes.
template <int SLOTS>
__device__ inline void block_order(int bid, int total, int nblk, bool by_rank, int* bh, int* rank) {
  if (by_rank) {
    const int heads = total / nblk;
    int g = 8 * ((SLOTS + nblk - 1) / nblk);
    g = g < heads ? g : heads;
    const int grp = bid / (g * nblk);
    const int rest = heads - grp * g;
    const int gh = rest < g ? rest : g;  // heads in this group (the last may be partial)
    const int t = bid - grp * g * nblk;
    *rank = __builtin_amdgcn_readfirstlane(t / gh);
    *bh = __builtin_amdgcn_readfirstlane(grp * g + (t - (t / gh) * gh));
  } else {
    const int b = xcd_remap(bid, total);
    *bh = __builtin_amdgcn_readfirstlane(b / nblk);
    *rank = __builtin_amdgcn_readfirstlane(b - *bh * nblk);
  }
}

// Buffer resource over `bytes` bytes starting at `base`: raw buffer loads at
// offsets at or beyond `bytes` return zeros, which pads ragged tiles for free.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Byte count for the descriptor of one tile of `tile_rows` rows when
// `rows_left` rows remain before the end of the sequence: loads past it return
// zeros.  Clamped to the tile, so the 32-bit count cannot wrap however long
// the sequence is (the tile's base address is formed in 64 bits by the caller).
__device__ inline uint32_t tile_bytes(int rows_left, int tile_rows, int row_bytes) {
  return (uint32_t)(rows_left < tile_rows ? rows_left : tile_rows) * (uint32_t)row_bytes;
}

__device__ inline u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// 16 bytes per lane from a buffer straight into LDS: lane i's bytes land at
// lds + 16 i (the LDS address must be wave-uniform).  The host pass of the
// compiler does not know this builtin and would silently drop the kernel's host
// stub, so only the device pass sees it.
__device__ inline void lds_load16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
#else
  (void)r; (void)lds; (void)off;
#endif
}

// Wave-uniform "does any lane want this".
__device__ inline bool any_lane(bool x) { return __builtin_amdgcn_ballot_w64(x) != 0; }

// Counter-based random words: Philox4x32 with 10 rounds (Salmon, Moraes, Dror
// and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011).  One round
// multiplies counter words 0 and 2 by the two round constants (64-bit
// products), then c <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key gains
// the two Weyl increments between rounds.
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

__device__ inline u32x4v philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    c0 = hi1 ^ c1 ^ (k0 + r * W0);
    c1 = lo1;
    c2 = hi0 ^ c3 ^ (k1 + r * W1);
    c3 = lo0;
  }
  return u32x4v{c0, c1, c2, c3};
}

// Dropout on the attention weights of one (batch, head): keep_ij when word
// j & 3 of Philox(counter (j >> 2, i, bh, offset), key = seed) is at least the
// threshold floor(p 2^32).  Kept weights are scaled by 1 / (1 - p) (`scale`),
// which the kernels fold into their final normalisation.
struct Dropout {
  uint32_t threshold;
  uint32_t seed_lo, seed_hi;
  uint32_t offset;
  float scale;
  // the four random words of keys 4 g .. 4 g + 3 (g = j >> 2) for query i
  __device__ inline u32x4v words(int g, int i, int bh) const {
    return philox4x32_10((uint32_t)g, (uint32_t)i, (uint32_t)bh, offset, seed_lo, seed_hi);
  }
  // Keep bits for a lane that holds one key (4 g + c, c = lane & 3, the same g
  // across its DPP quad of four lanes) against queries i0 .. i0 + 3.  Each lane
  // draws the words of one query (i0 + c), which cover the quad's four keys;
  // the four 4-bit keep rows are gathered across the quad, so one draw serves
  // four weights instead of one.  Bit 4 u of the result keeps query i0 + u.
  // Needs all four lanes of the quad active.
  __device__ __attribute__((always_inline)) inline uint32_t quad_keep(int g, int i0, int bh, int c) const {
    const u32x4v w = words(g, i0 + c, bh);
    uint32_t m = (w[0] >= threshold ? 1u : 0u) | (w[1] >= threshold ? 2u : 0u) | (w[2] >= threshold ? 4u : 0u) |
                 (w[3] >= threshold ? 8u : 0u);
    m <<= 4 * c;                                                               // row c of the 4 x 4 keep block
    m |= (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false);   // quad_perm [1, 0, 3, 2]
    m |= (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false);   // quad_perm [2, 3, 0, 1]
    return m >> c;                                                             // column c: this lane's key
  }
};

// Floor of a / b for b > 0 and any sign of a.
__device__ inline int floor_div(int a, int b) { return a >= 0 ? a / b : -((b - 1 - a) / b); }

// Geometry of one sequence of a batch: lq real queries of Nq rows, lk real
// keys of Nk rows (lengths from the optional device arrays, clamped into
// [0, Nq] / [0, Nk]).  The queries are the last lq positions of the key
// sequence, so under the causal mask query i may see key j iff j <= i + off,
// off = lk - lq; with equal counts and no lengths this is j <= i.
struct Seq {
  int lq, lk, off;
};

__device__ inline Seq seq_of(const int* seqlens_q, const int* seqlens_k, int b, int Nq, int Nk) {
  int lq = Nq, lk = Nk;
  if (seqlens_q != nullptr) {
    const int x = seqlens_q[b];
    lq = x < 0 ? 0 : (x > Nq ? Nq : x);
  }
  if (seqlens_k != nullptr) {
    const int x = seqlens_k[b];
    lk = x < 0 ? 0 : (x > Nk ? Nk : x);
  }
  lq = __builtin_amdgcn_readfirstlane(lq);
  lk = __builtin_amdgcn_readfirstlane(lk);
  return {lq, lk, lk - lq};
}

// Block-sparse masks: one row (or column) of a [nbq, nbk] byte mask packed into
// 64-bit words in LDS, bit b of word w standing for block 64 w + b.  Up to
// kMaxMaskWords words, i.e. 4096 blocks per row or column.
constexpr int kMaxMaskWords = 64;

// Every wave of the workgroup packs words wave, wave + nwaves, ...: lane l of
// word w reads mask[(64 w + l) * stride].  A barrier must follow before the
// words are read.
__device__ inline void pack_mask_words(uint64_t* words, const unsigned char* mask, int nb, int stride, int lane,
                                       int wave, int nwaves) {
  const int nw = (nb + 63) >> 6;
  for (int w = wave; w < nw; w += nwaves) {
    const int b = 64 * w + lane;
    const bool on = b < nb && mask[(size_t)b * stride] != 0;
    const uint64_t bits = __builtin_amdgcn_ballot_w64(on);
    if (lane == 0) words[w] = bits;
  }
}

// The first kept block at or after b (nb when there is none); wave-uniform.
__device__ inline int next_kept(const uint64_t* words, int b, int nb) {
  while (b < nb) {
    const int w = b >> 6;
    const uint64_t word = words[w];
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)word);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(word >> 32));
    const uint64_t bits = ((((uint64_t)hi) << 32) | lo) >> (b & 63);
    if (bits != 0) {
      const int r = b + __builtin_ctzll(bits);
      return r < nb ? r : nb;
    }
    b = (w + 1) << 6;
  }
  return nb;
}

// Tiles of kMaskBlock / tpb rows, n of them: a tile is live when its mask
// block is kept.  The first live tile at or after t (n when there is none).
__device__ inline int live_tile_from(const uint64_t* words, int t, int tpb, int nb, int n) {
  if (t >= n) return n;
  const int b = t / tpb;
  const int kb = next_kept(words, b, nb);
  if (kb == b) return t;
  const int u = kb * tpb;
  return u < n ? u : n;
}

// The live tile after the live tile t (or the first one, t = -1): the tiles of
// one block are consecutive, so the next tile is live too unless it starts a
// new block.
__device__ inline int next_live_tile(const uint64_t* words, int t, int tpb, int nb, int n) {
  const int u = t + 1;
  if (u >= n) return n;
  if (t >= 0 && u % tpb != 0) return u;
  return live_tile_from(words, u, tpb, nb, n);
}

// Largest key query row i may see; negative when it sees none (a padding row,
// or a causal row that starts before the first key).
template <bool CAUSAL>
__device__ inline int key_limit(const Seq& s, int i) {
  if (i >= s.lq) return -1;
  const int lim = CAUSAL ? i + s.off : s.lk - 1;
  return lim < s.lk - 1 ? lim : s.lk - 1;
}

// Key tiles of width BN that a block of query rows [q0, q0 + rows) visits
// (*nt), and how many leading ones no real row of the block sees masked (*nfull).
template <bool CAUSAL, int BN>
__device__ inline void query_block_tiles(const Seq& s, int q0, int rows, int* nt, int* nfull) {
  const int last = (q0 + rows - 1 < s.lq - 1 ? q0 + rows - 1 : s.lq - 1);  // last real row
  if (last < q0) {
    *nt = 0;
    *nfull = 0;
    return;
  }
  const int kmax = key_limit<CAUSAL>(s, last);
  const int kmin = key_limit<CAUSAL>(s, q0);  // the limit only grows with the row
  const int n = kmax < 0 ? 0 : kmax / BN + 1;
  const int f = kmin < 0 ? 0 : (kmin + 1) / BN;
  *nt = n;
  *nfull = f < n ? f : n;
}

// Store 4 consecutive elements (fp32 in) as T.
template <typename T>
__device__ inline void store4(T* p, float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    typedef T T4 __attribute__((ext_vector_type(4)));
    T4 v = {(T)a, (T)b, (T)c, (T)d};
    *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, v);
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
  }
}

}  // namespace fa
