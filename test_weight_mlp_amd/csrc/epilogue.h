// Epilogue shared by the Z and V_hat kernels: a finished BM x BN output tile
// sits in LDS (row = token, column = feature) and is written twice:
//   row-major        out [tokens, F]                 (16-byte stores along F)
//   chunk-transposed outT[(row*N + chunk)*F + j][Cp] (16-byte stores along tokens)
// The second copy is what the token-axis contractions (V_hat^T Z) read, so
// their MFMA operands arrive K-contiguous.
#pragma once

#include "common.h"

namespace ipttt {

struct ChunkGrid {
  int64_t T;  // tokens per row
  int C, N, Cp;
};

// Row, chunk and in-chunk offset of the tokens of one tile.  The tile's first
// token is split once (a uniform 64-bit division); the rest is 32-bit
// unsigned arithmetic (rows hold fewer than 2^31 tokens).
struct TilePos {
  int64_t b0;    // row of the tile's first token
  uint32_t t0;   // its position in that row
  uint32_t T, C;
  __device__ __forceinline__ TilePos(int64_t m0, const ChunkGrid& g) {
    b0 = m0 / g.T;
    t0 = (uint32_t)(m0 - b0 * g.T);
    T = (uint32_t)g.T;
    C = (uint32_t)g.C;
  }
  // token r of the tile -> (row, chunk, offset)
  __device__ __forceinline__ void at(int r, int64_t& b, int& i, int& c) const {
    uint32_t t = t0 + (uint32_t)r;
    b = b0;
    while (t >= T) { t -= T; ++b; }
    const uint32_t q = t / C;
    i = (int)q;
    c = (int)(t - q * C);
  }
};

// Chunk-transposed store of a staged column-major tile colT [BN][LDCOL]
// (column = feature, 8 consecutive tokens per 16-byte piece): token r of the
// tile, feature j goes to outT[((b*N + i)*F + n0 + j)*Cp + c].  Pieces that
// would straddle a chunk or row end are written element by element.
template <int BM, int BN, int LDCOL, int NT>
__device__ __forceinline__ void store_chunk_t(const bf16* colT, bf16* __restrict__ outT, int64_t m0, int mrows,
                                              int n0, int nrows, int F, const ChunkGrid& g, int tid) {
  constexpr int GPC = BM / 8;
  const TilePos pos(m0, g);
  for (int v = tid; v < BN * GPC; v += NT) {
    const int col = v / GPC, r0 = (v - col * GPC) * 8;
    if (col >= nrows || r0 >= mrows) continue;
    int64_t b;
    int i, c;
    pos.at(r0, b, i, c);
    const int L = (int)min((uint32_t)g.C, pos.T - (uint32_t)i * (uint32_t)g.C);
    if ((c & 7) == 0 && r0 + 8 <= mrows && c + 8 <= L) {
      *reinterpret_cast<u32x4*>(outT + ((b * g.N + i) * (int64_t)F + n0 + col) * g.Cp + c) =
          *reinterpret_cast<const u32x4*>(colT + col * LDCOL + r0);
    } else {
      for (int q = 0; q < 8 && r0 + q < mrows; ++q) {
        int64_t bq;
        int iq, cq;
        pos.at(r0 + q, bq, iq, cq);
        outT[((bq * g.N + iq) * (int64_t)F + n0 + col) * g.Cp + cq] = colT[col * LDCOL + r0 + q];
      }
    }
  }
}

template <typename T, int BM, int BN, int LDC>
__device__ __forceinline__ void store_rows_and_chunk_t(const T* lC, T* __restrict__ out, T* __restrict__ outT,
                                                       int64_t m0, int mrows, int n0, int nrows, int F,
                                                       const ChunkGrid& g, int tid) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int VPR = BN / VE;  // vectors per tile row
  for (int v = tid; v < BM * VPR; v += kThreads) {
    const int r = v / VPR, cv = (v - r * VPR) * VE;
    if (r < mrows && cv < nrows)
      *reinterpret_cast<u32x4*>(out + (m0 + r) * (int64_t)F + n0 + cv) =
          *reinterpret_cast<const u32x4*>(lC + r * LDC + cv);
  }
  if (outT == nullptr) return;
  constexpr int GPC = BM / VE;  // token groups per tile column
  for (int v = tid; v < BN * GPC; v += kThreads) {
    const int col = v / GPC, r0 = (v - col * GPC) * VE;
    if (col >= nrows || r0 >= mrows) continue;
    const int64_t tok = m0 + r0;
    const int64_t b = tok / g.T, tt = tok - b * g.T;
    const int i = (int)(tt / g.C), c = (int)(tt - (int64_t)i * g.C);
    const int L = (int)min((int64_t)g.C, g.T - (int64_t)i * g.C);
    if ((c % VE) == 0 && r0 + VE <= mrows && c + VE <= L) {
      u32x4 x;
      T* e = reinterpret_cast<T*>(&x);
#pragma unroll
      for (int q = 0; q < VE; ++q) e[q] = lC[(r0 + q) * LDC + col];
      *reinterpret_cast<u32x4*>(outT + ((b * g.N + i) * (int64_t)F + n0 + col) * g.Cp + c) = x;
    } else {
      for (int q = 0; q < VE && r0 + q < mrows; ++q) {
        const int64_t tq = m0 + r0 + q;
        const int64_t bq = tq / g.T, ttq = tq - bq * g.T;
        const int iq = (int)(ttq / g.C), cq = (int)(ttq - (int64_t)iq * g.C);
        outT[((bq * g.N + iq) * (int64_t)F + n0 + col) * g.Cp + cq] = lC[(r0 + q) * LDC + col];
      }
    }
  }
}

}  // namespace ipttt

namespace ipttt {

// Writes one wave's 32x32 accumulator block values (fp32, MFMA layout:
// element j of lane l is row 8*(j/4) + 4*(l/32) + j%4, column l%32, relative to
// (row0, col0)) into two LDS staging tiles, rounded to bf16:
//   rowT [BM][BN + 8]  row-major: lane pairs swap halves through a DPP quad
//                      permute so that each lane stores two adjacent columns of
//                      two rows as two 4-byte words;
//   colT [BN][BM + 8]  column-major: each lane's 4 consecutive rows are 8
//                      contiguous bytes.
template <int BM, int BN>
__device__ __forceinline__ void stage_block_dual(const float (&v)[16], bf16* rowT, bf16* colT, int row0, int col0,
                                                 int lane) {
  constexpr int LDR = BN + 8, LDCOL = BM + 8;
  const int c = col0 + (lane & 31);
  const bool odd = lane & 1;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = row0 + 8 * g + 4 * (lane >> 5);
    bf16 q[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) q[t] = (bf16)v[4 * g + t];
    // column-major: rows r..r+3 of column c
    uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, q[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, q[1]) << 16);
    uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, q[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, q[3]) << 16);
    *reinterpret_cast<uint2*>(colT + c * LDCOL + r) = make_uint2(lo, hi);
    // row-major: even lane keeps rows r, r+1 and takes its odd partner's
    // values of those rows; the odd lane keeps rows r+2, r+3.
    const uint32_t give = odd ? lo : hi;
    const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)give, 0xB1, 0xF, 0xF, false);
    const uint32_t mine = odd ? hi : lo;
    // For the even lane (column c): mine = (r, r+1) at c, got = (r, r+1) at c+1.
    // For the odd lane (column c): mine = (r+2, r+3) at c, got = (r+2, r+3) at c-1.
    const uint32_t w0 = odd ? ((got & 0xFFFFu) | (mine << 16)) : ((mine & 0xFFFFu) | (got << 16));
    const uint32_t w1 = odd ? ((got >> 16) | (mine & 0xFFFF0000u)) : ((mine >> 16) | (got & 0xFFFF0000u));
    const int rr = odd ? r + 2 : r;
    const int cc = odd ? c - 1 : c;
    *reinterpret_cast<uint32_t*>(rowT + rr * LDR + cc) = w0;
    *reinterpret_cast<uint32_t*>(rowT + (rr + 1) * LDR + cc) = w1;
  }
}

// Stores a staged BM x BN tile: row-major out [tokens, F] from rowT, and the
// chunk-transposed copy outT from colT (16-byte pieces along tokens).
template <int BM, int BN, int NT = kThreads>
__device__ __forceinline__ void store_dual(const bf16* rowT, const bf16* colT, bf16* __restrict__ out,
                                           bf16* __restrict__ outT, int64_t m0, int mrows, int n0, int nrows, int F,
                                           const ChunkGrid& g, int tid) {
  constexpr int LDR = BN + 8, LDCOL = BM + 8;
  constexpr int VPR = BN / 8;
  for (int v = tid; v < BM * VPR; v += NT) {
    const int r = v / VPR, cv = (v - r * VPR) * 8;
    if (r < mrows && cv < nrows)
      *reinterpret_cast<u32x4*>(out + (m0 + r) * (int64_t)F + n0 + cv) =
          *reinterpret_cast<const u32x4*>(rowT + r * LDR + cv);
  }
  if (outT == nullptr) return;
  store_chunk_t<BM, BN, LDCOL, NT>(colT, outT, m0, mrows, n0, nrows, F, g, tid);
}

}  // namespace ipttt

namespace ipttt {

// Row-major staging only (see stage_block_dual): tile rowT [.][LDR].
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
    const uint32_t give = odd ? lo : hi;
    const uint32_t got = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)give, 0xB1, 0xF, 0xF, false);
    const uint32_t mine = odd ? hi : lo;
    const uint32_t w0 = odd ? ((got & 0xFFFFu) | (mine << 16)) : ((mine & 0xFFFFu) | (got << 16));
    const uint32_t w1 = odd ? ((got >> 16) | (mine & 0xFFFF0000u)) : ((mine >> 16) | (got & 0xFFFF0000u));
    const int rr = odd ? r + 2 : r;
    const int cc = odd ? c - 1 : c;
    *reinterpret_cast<uint32_t*>(rowT + rr * LDR + cc) = w0;
    *reinterpret_cast<uint32_t*>(rowT + (rr + 1) * LDR + cc) = w1;
  }
}

// Column-major staging only: tile colT [.][LDCOL], 4 consecutive rows per lane.
template <int LDCOL>
__device__ __forceinline__ void stage_block_cols(const float (&v)[16], bf16* colT, int row0, int col0, int lane) {
  const int c = col0 + (lane & 31);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = row0 + 8 * g + 4 * (lane >> 5);
    const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[4 * g]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[4 * g + 1]) << 16);
    const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[4 * g + 2]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)v[4 * g + 3]) << 16);
    *reinterpret_cast<uint2*>(colT + c * LDCOL + r) = make_uint2(lo, hi);
  }
}

// Row-major store of a staged tile: rows [lo, hi) of the tile go to
// out[(m0 + r) * F + n0 + c].
template <int BM, int BN, int LDR, int NT>
__device__ __forceinline__ void store_rows(const bf16* rowT, bf16* __restrict__ out, int64_t m0, int lo, int hi,
                                           int n0, int nrows, int F, int tid) {
  constexpr int VPR = BN / 8;
  for (int v = tid; v < BM * VPR; v += NT) {
    const int r = v / VPR, cv = (v - r * VPR) * 8;
    if (r >= lo && r < hi && cv < nrows)
      *reinterpret_cast<u32x4*>(out + (m0 + r) * (int64_t)F + n0 + cv) =
          *reinterpret_cast<const u32x4*>(rowT + r * LDR + cv);
  }
}

}  // namespace ipttt
