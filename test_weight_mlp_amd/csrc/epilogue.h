// Epilogue of the Z, V_hat and apply kernels: a finished output tile is staged
// in LDS (row = token, column = feature) and written row-major to
// out [tokens, F] in 16-byte stores along F.
#pragma once

#include "common.h"

namespace ipttt {

// Row-major store of a staged tile lC [BM][LDC] of the general kernels.
template <typename T, int BM, int BN, int LDC>
__device__ __forceinline__ void store_tile_rows(const T* lC, T* __restrict__ out, int64_t m0, int mrows, int n0,
                                                int nrows, int F, int tid) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int VPR = BN / VE;  // vectors per tile row
  for (int v = tid; v < BM * VPR; v += kThreads) {
    const int r = v / VPR, cv = (v - r * VPR) * VE;
    if (r < mrows && cv < nrows)
      *reinterpret_cast<u32x4*>(out + (m0 + r) * (int64_t)F + n0 + cv) =
          *reinterpret_cast<const u32x4*>(lC + r * LDC + cv);
  }
}

// Transposed store of a staged tile lC [BM][LDC] (rows r < nrows, columns
// c < ncols): out[(c0 + c) * ld + r0 + r] = lC[r][c], 16 bytes along r per
// store.  nrows must be a multiple of the vector length.
template <typename T, int BM, int BN, int LDC>
__device__ __forceinline__ void store_tile_cols(const T* lC, T* __restrict__ out, int64_t ld, int64_t r0, int nrows,
                                                int64_t c0, int ncols, int tid) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int VPC = BM / VE;  // vectors per output row (one tile column)
  for (int v = tid; v < BN * VPC; v += kThreads) {
    const int c = v / VPC, rv = (v - c * VPC) * VE;
    if (c < ncols && rv < nrows) {
      u32x4 x;
      T* e = reinterpret_cast<T*>(&x);
#pragma unroll
      for (int q = 0; q < VE; ++q) e[q] = lC[(rv + q) * LDC + c];
      *reinterpret_cast<u32x4*>(out + (c0 + c) * ld + r0 + rv) = x;
    }
  }
}

// Writes one wave's 32x32 accumulator block (fp32, MFMA layout: element j of
// lane l is row 8*(j/4) + 4*(l/32) + j%4, column l%32, relative to
// (row0, col0)) into the row-major LDS tile rowT [.][LDR], rounded to bf16.
// Lane pairs swap halves through a DPP quad permute so that each lane stores
// two adjacent columns of two rows as two 4-byte words.
template <int LDR>
__device__ __forceinline__ void stage_block_rows(const float (&v)[16], bf16* rowT, int row0, int col0, int lane) {
  const int c = col0 + (lane & 31);
  const bool odd = lane & 1;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = row0 + 8 * g + 4 * (lane >> 5);
    const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[4 * g]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[4 * g + 1]) << 16);
    const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[4 * g + 2]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[4 * g + 3]) << 16);
    // The even lane keeps rows r, r+1 and takes its odd partner's values of
    // those rows; the odd lane keeps rows r+2, r+3.
    const uint32_t give = odd ? lo : hi;
    const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)give, 0xB1, 0xF, 0xF, false);
    const uint32_t mine = odd ? hi : lo;
    // even lane (column c): mine = (r, r+1) at c, got = (r, r+1) at c+1;
    // odd lane (column c): mine = (r+2, r+3) at c, got = (r+2, r+3) at c-1.
    const uint32_t w0 = odd ? ((got & 0xFFFFu) | (mine << 16)) : ((mine & 0xFFFFu) | (got << 16));
    const uint32_t w1 = odd ? ((got >> 16) | (mine & 0xFFFF0000u)) : ((mine >> 16) | (got & 0xFFFF0000u));
    const int rr = odd ? r + 2 : r;
    const int cc = odd ? c - 1 : c;
    *reinterpret_cast<uint32_t*>(rowT + rr * LDR + cc) = w0;
    *reinterpret_cast<uint32_t*>(rowT + (rr + 1) * LDR + cc) = w1;
  }
}

// Row-major store of a staged bf16 tile: rows [lo, hi) of the tile go to
// out[(m0 + r) * F + n0 + c].  STREAM selects non-temporal stores, for
// outputs that no kernel reads again soon (they would otherwise push the
// operands of the running GEMM out of the caches).
template <int BM, int BN, int LDR, int NT, bool STREAM = false>
__device__ __forceinline__ void store_rows(const bf16* rowT, bf16* __restrict__ out, int64_t m0, int lo, int hi,
                                           int n0, int nrows, int F, int tid) {
  constexpr int VPR = BN / 8;
  for (int v = tid; v < BM * VPR; v += NT) {
    const int r = v / VPR, cv = (v - r * VPR) * 8;
    if (r >= lo && r < hi && cv < nrows) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(rowT + r * LDR + cv);
      u32x4* dst = reinterpret_cast<u32x4*>(out + (m0 + r) * (int64_t)F + n0 + cv);
      if constexpr (STREAM)
        __builtin_nontemporal_store(x, dst);
      else
        *dst = x;
    }
  }
}

// Unpadded staging tile [.][LDR] (LDR a multiple of 128 elements) whose
// 16-byte column chunks are XOR-swizzled by bits 1-2 of the row: the 4-byte
// writes of stage_block_rows_swz (rows r, r+2, r+4, r+6 of one instruction)
// then fall on distinct banks, and a 16-lane read of one row stays a
// permutation of its 256 bytes.
template <int LDR>
__device__ __forceinline__ int swz_elem(int r, int c) {
  static_assert(LDR % 128 == 0, "staging pitch");
  return r * LDR + (c ^ (((r >> 1) & 3) << 5));
}

template <int LDR>
__device__ __forceinline__ void stage_block_rows_swz(const float (&v)[16], bf16* rowT, int row0, int col0,
                                                     int lane) {
  const int c = col0 + (lane & 31);
  const bool odd = lane & 1;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = row0 + 8 * g + 4 * (lane >> 5);
    const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[4 * g]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[4 * g + 1]) << 16);
    const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[4 * g + 2]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[4 * g + 3]) << 16);
    const uint32_t give = odd ? lo : hi;
    const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)give, 0xB1, 0xF, 0xF, false);
    const uint32_t mine = odd ? hi : lo;
    const uint32_t w0 = odd ? ((got & 0xFFFFu) | (mine << 16)) : ((mine & 0xFFFFu) | (got << 16));
    const uint32_t w1 = odd ? ((got >> 16) | (mine & 0xFFFF0000u)) : ((mine >> 16) | (got & 0xFFFF0000u));
    const int rr = odd ? r + 2 : r;
    const int cc = odd ? c - 1 : c;
    *reinterpret_cast<uint32_t*>(rowT + swz_elem<LDR>(rr, cc)) = w0;
    *reinterpret_cast<uint32_t*>(rowT + swz_elem<LDR>(rr + 1, cc)) = w1;
  }
}

// Row-major store of a swizzled staging tile (see swz_elem); STREAM as in
// store_rows.
template <int BM, int BN, int LDR, int NT, bool STREAM = false>
__device__ __forceinline__ void store_rows_swz(const bf16* rowT, bf16* __restrict__ out, int64_t m0, int lo, int hi,
                                               int n0, int nrows, int F, int tid) {
  constexpr int VPR = BN / 8;
  for (int v = tid; v < BM * VPR; v += NT) {
    const int r = v / VPR, cv = (v - r * VPR) * 8;
    if (r >= lo && r < hi && cv < nrows) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(rowT + swz_elem<LDR>(r, cv));
      u32x4* dst = reinterpret_cast<u32x4*>(out + (m0 + r) * (int64_t)F + n0 + cv);
      if constexpr (STREAM)
        __builtin_nontemporal_store(x, dst);
      else
        *dst = x;
    }
  }
}

}  // namespace ipttt
