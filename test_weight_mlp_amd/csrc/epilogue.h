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
