// fa_tile16.h -- LDS tiles of 16-bit rows filled by direct (buffer -> LDS) loads.
//
// A tile is ROWS (64 by default) rows of D 16-bit elements, rows packed back to back.  Direct
// loads write 1 KiB per wave instruction, contiguously, so rows cannot be
// padded; instead the 16-byte chunks of row r are stored XOR-permuted by
// sw(r).  With sw chosen per row length (checked with a 64-bank model), the
// two read patterns of the matrix-core operands are conflict-free:
//   * row fragments: 32 lanes read 16 B each from 32 different rows at the
//     same logical chunk (A/B operands whose contraction runs along the row);
//   * transposing reads (ds_read_b64_tr_b16): each 16-lane group reads 8 B
//     from 4 consecutive rows x 4 chunks (operands contracted over rows).
#pragma once

#include "fa_device.h"

namespace fa {

template <int D, int ROWS = 64>
struct Tile16 {
  static constexpr int ROWB = 2 * D;
  static constexpr int CPR = ROWB / 16;            // 16-byte chunks per row: 8 or 16
  static constexpr int BYTES = ROWS * ROWB;        // 8, 16 or 32 KiB
  static constexpr int ROUNDS = ROWS * CPR / 256;  // direct loads per tile per wave (4 waves)
  __device__ static constexpr int sw(int r) {
    return CPR == 16 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
  __device__ static constexpr int phys(int r, int chunk) { return r * ROWB + ((chunk ^ sw(r)) << 4); }
};

// s_waitcnt vmcnt(0) with the other counters left alone.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Source offset (bytes inside a tile) each lane loads in direct-load round i,
// for a 4-wave workgroup: slot s = (4 i + wave) * 64 + lane holds logical
// chunk (s % CPR) ^ sw(row) of row s / CPR.
template <int D, int ROWS = 64>
__device__ inline void tile16_load_offsets(uint32_t* goff, int wave, int lane) {
  using TL = Tile16<D, ROWS>;
#pragma unroll
  for (int i = 0; i < TL::ROUNDS; ++i) {
    const int s = (i * 4 + wave) * 64 + lane;
    const int r = s / TL::CPR, pc = s % TL::CPR;
    goff[i] = r * TL::ROWB + ((pc ^ TL::sw(r)) << 4);
  }
}

// Byte address of the row fragment of `row` for k-step ks (16 elements per
// step, 8 per half-wave h).
template <int D>
__device__ constexpr inline uint32_t tile16_row_addr(int row, int ks, int h) {
  return Tile16<D>::phys(row, 2 * ks + h);
}

// Byte addresses of the two transposing reads (rows +0..3 and +8..11 of a
// 16-row step) for output column block mb, as trans_frag in fa_device.h lays
// them out; add (first row) * ROWB for the rows being contracted.
template <int D>
__device__ inline uint32_t tile16_tr_addr(int lane, int mb, int hf) {
  const int i = lane & 15, g = (lane >> 4) & 1, h = lane >> 5;
  const int row = 4 * h + (i >> 2) + 8 * hf;
  const int chunk = 4 * mb + 2 * g + ((i & 3) >> 1);
  return Tile16<D>::phys(row, chunk) + 8 * (i & 1);
}

template <typename T>
__device__ inline typename Mma<T>::Frag tile16_row_frag(const char* smem, uint32_t addr) {
  return __builtin_bit_cast(typename Mma<T>::Frag, *reinterpret_cast<const u32x4*>(smem + addr));
}

// Transposing 16-bit LDS read.  The compiler cannot tell an LDS read from the
// direct (buffer -> LDS) loads still in flight into other stages, and without
// alias information it waits for all of them (vmcnt(0)) before the read, which
// stalls each pipeline step on the loads it has just issued for the next tile.
// The restrict-qualified pointer gives the read that information.  Every kernel
// waits for its direct loads explicitly (vmcnt(0), then a barrier, since other
// waves read what each wave loads) before reading the stage they filled.
__device__ __attribute__((always_inline)) inline i16x4 lds_tr16(const char* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}

template <typename T, int D>
__device__ inline typename Mma<T>::Frag tile16_tr_frag(const char* smem, uint32_t a0, uint32_t a1, int off) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x4 lo = lds_tr16(smem + a0 + off);
  const i16x4 hi = lds_tr16(smem + a1 + off);
  const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(typename Mma<T>::Frag, both);
}

}  // namespace fa
