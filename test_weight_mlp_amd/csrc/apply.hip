// Apply: O_[i] = Z_[i] W^T with each token's document state
// (lijianxiong.blog "In-Place Test-Time Training", 高效的块状更新机制, 步骤一).
// Tokens of chunk i before its first document start use the chunk's effective
// weight W_down + S_i written by the scan; tokens from that start on belong to
// a document that began inside the chunk and use W_down
// (iplexlaw.co.kr review, section 6: reset at document boundaries).
//
// One workgroup = one token tile x output tile of one chunk, K = d_ff (bf16 with
// d_model, d_ff multiples of 64: 256 x 256 on the 8-wave core, the weights
// read as ready-made MFMA B fragments; otherwise 128 x 128 from row-major
// weights).  A tile that straddles the first document start runs the K loop
// once per weight and keeps the rows each weight owns.
#include "launch.h"
#include "common.h"
#include "epilogue.h"
#include "mfma_core.h"

namespace ipttt {

template <typename T>
__global__ __launch_bounds__(kThreads) void apply_kernel(const T* __restrict__ Z, const T* __restrict__ Wbuf,
                                                         const T* __restrict__ Wd, const int32_t* __restrict__ table,
                                                         T* __restrict__ O, int64_t Tn, int C, int N, int d, int f,
                                                         int tiles_m, int tiles_n) {
  typedef Geo<T, 128, 128> G;
  constexpr int VE = G::VE;
  constexpr int LDC = G::BN + VE;
  constexpr int kStage = (G::BM + G::BN) * G::LDK;
  constexpr int kEpi = G::BM * LDC;
  __shared__ __attribute__((aligned(16))) T lds[kStage > kEpi ? kStage : kEpi];
  T* lA = lds;
  T* lB = lds + G::BM * G::LDK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Logical order: chunk-major, then output tile, then token tile, so the
  // workgroups sharing one chunk's weight run next to each other.
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int per_chunk = tiles_m * tiles_n;
  const int bc = t / per_chunk;
  const int rem = t - bc * per_chunk;
  const int tn = rem / tiles_m, tm = rem - tn * tiles_m;
  const int b = bc / N, i = bc - b * N;
  const int L = (int)min((int64_t)C, Tn - (int64_t)i * C);
  const int m0 = tm * G::BM;
  if (m0 >= L) return;
  const int mrows = min(G::BM, L - m0);
  const int n0 = tn * G::BN, nrows = min(G::BN, d - n0);
  const int r0 = table[bc * 3 + 0];
  const int64_t tok0 = (int64_t)b * Tn + (int64_t)i * C + m0;
  const T* A = Z + tok0 * f;

  for (int pass = 0; pass < 2; ++pass) {
    // pass 0: rows [m0, min(r0, m0+mrows)) with the chunk's weight
    // pass 1: rows [max(r0, m0), m0+mrows) with W_down
    const int lo = pass == 0 ? 0 : max(r0 - m0, 0);
    const int hi = pass == 0 ? min(r0 - m0, mrows) : mrows;
    if (lo >= hi) continue;
    const T* W = (pass == 0 ? Wbuf + (int64_t)bc * d * f : Wd) + (int64_t)n0 * f;
    floatx16 acc[G::MB][G::NB];
    zero_acc<G>(acc);
    TileLoad<T, G::BM> la;
    TileLoad<T, G::BN> lb;
    la.load(A, f, mrows, 0, f, tid);
    lb.load(W, f, nrows, 0, f, tid);
    for (int k0 = 0; k0 < f; k0 += G::BK) {
      la.template store<G::LDK>(lA, tid);
      lb.template store<G::LDK>(lB, tid);
      __syncthreads();
      if (k0 + G::BK < f) {
        la.load(A, f, mrows, k0 + G::BK, f, tid);
        lb.load(W, f, nrows, k0 + G::BK, f, tid);
      }
      stage_mma<T, G>(lA, lB, acc, wm, wn, lane);
      __syncthreads();
    }
    T* lC = lds;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = wm * G::WM + mb * 32 + acc_row(j, lane);
          const int c = wn * G::WN + nb * 32 + (lane & 31);
          lC[r * LDC + c] = from_f32<T>(acc[mb][nb][j]);
        }
    __syncthreads();
    constexpr int VPR = G::BN / VE;
    for (int v = tid; v < G::BM * VPR; v += kThreads) {
      const int r = v / VPR, cv = (v - r * VPR) * VE;
      if (r >= lo && r < hi && cv < nrows)
        *reinterpret_cast<u32x4*>(O + (tok0 + r) * d + n0 + cv) = *reinterpret_cast<const u32x4*>(lC + r * LDC + cv);
    }
    __syncthreads();
  }
}

// bf16 fast path (d_model, d_ff multiples of 64): 256 tokens x 256 outputs
// per workgroup of 8 waves (core::Tile8H, the half-stage ring: the weights
// stream from HBM), K = d_ff.  The weights (each chunk's W_down + S_i, and
// W_down) come fragment-major from the scan: 1 KB per (32 outputs, 16 of K)
// block, (d/32) * (f/16) blocks per matrix.
typedef core::Tile8H<256, 256, 1, 2, 4, 1> OTile;

__global__ __launch_bounds__(OTile::NT) void apply_fast_kernel(const bf16* __restrict__ Z, const bf16* __restrict__ Wbuf,
                                                              const bf16* __restrict__ Wdfrag,
                                                              const int32_t* __restrict__ table, bf16* __restrict__ O,
                                                              int64_t Tn, int C, int N, int d, int f, int tiles_m,
                                                              int tiles_n, int row0, int i0, int nw) {
  constexpr int BM = 256, BN = 256, LD = 264;
  constexpr int LDS = OTile::LDS_ELEMS > BM * LD ? OTile::LDS_ELEMS : BM * LD;
  __shared__ __attribute__((aligned(1024))) bf16 lds[LDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // chunk-major, then output tile, then token tile: workgroups that share a
  // chunk's weight run next to each other
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int per_chunk = tiles_m * tiles_n;
  // bl: the row within this pass, whose window of nw per-chunk weights
  // (chunks i0 ..) starts at Wbuf + bl * nw * d * f; b = row0 + bl: the row of
  // the problem
  const int bcl = t / per_chunk;
  const int rem = t - bcl * per_chunk;
  const int tn = rem / tiles_m, tm = rem - tn * tiles_m;
  const int bl = bcl / nw, i = i0 + bcl - bl * nw;
  const int b = row0 + bl, bc = b * N + i;
  const int L = (int)min((int64_t)C, Tn - (int64_t)i * C);
  const int m0 = tm * BM;
  if (m0 >= L) return;
  const int mrows = min(BM, L - m0);
  const int n0 = tn * BN, nrows = min(BN, d - n0);
  const int r0 = table[bc * 3 + 0];
  const int64_t tok0 = (int64_t)b * Tn + (int64_t)i * C + m0;
  const core::Operand oa = core::make_operand(Z + tok0 * f, (int64_t)f * 2, (int64_t)mrows * f * 2);
  for (int pass = 0; pass < 2; ++pass) {
    // pass 0: rows before the chunk's first document start, chunk weight;
    // pass 1: rows from that start on, W_down
    const int lo = pass == 0 ? 0 : max(r0 - m0, 0);
    const int hi = pass == 0 ? min(r0 - m0, mrows) : mrows;
    if (lo >= hi) continue;
    // fragment rows of this tile's 256 outputs: (n0/32 ..) * (f/16) fragments
    const bf16* W = (pass == 0 ? Wbuf + (int64_t)bcl * d * f : Wdfrag) + (int64_t)(n0 / 32) * (f / 16) * 512;
    const core::Operand ob[1] = {core::make_operand(W, (int64_t)f * 64, (int64_t)(d - n0) * f * 2)};
    floatx16 acc[1][2][4];
    core::zero(acc);
    OTile::run(oa, ob, f, lds, acc, wave, lane);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = acc[0][mb][nb][j];
        stage_block_rows<LD>(v, lds, wm * 64 + mb * 32, wn * 128 + nb * 32, lane);
      }
    __syncthreads();
    store_rows<BM, BN, LD, OTile::NT, true>(lds, O, tok0, lo, hi, n0, nrows, d, tid);
    __syncthreads();
  }
}

hipError_t launch_apply(const Prob& p, const void* Z, const void* Wbuf, const void* Wd, const void* Wdfrag,
                        const int32_t* table, void* O, hipStream_t st, int row0, int nrows, int i0, int i1) {
  note_launch("apply", st);
  if (i1 < 0) i1 = (int)p.N;
  if (fast_scan(p)) {
    if (i0 < 0 || i0 >= i1 || i1 > p.N) return hipErrorInvalidValue;
    const int nb = nrows < 0 ? (int)p.B : nrows, nw = i1 - i0;
    const int tm = (p.C + 255) / 256, tn = (p.d + 255) / 256;
    const int64_t fb = (int64_t)nb * nw * tm * tn;
    apply_fast_kernel<<<(unsigned)fb, OTile::NT, 0, st>>>((const bf16*)Z, (const bf16*)Wbuf, (const bf16*)Wdfrag, table,
                                                          (bf16*)O, p.T, p.C, p.N, p.d, p.f, tm, tn, row0, i0, nw);
    return hipGetLastError();
  }
  if (row0 != 0 || (nrows >= 0 && nrows != p.B) || i0 != 0 || i1 != p.N) return hipErrorInvalidValue;
  const int tiles_m = (p.C + 127) / 128, tiles_n = (p.d + 127) / 128;
  const int64_t blocks = p.B * p.N * (int64_t)tiles_m * tiles_n;
  if (p.dtype == 1)
    apply_kernel<bf16><<<(unsigned)blocks, kThreads, 0, st>>>((const bf16*)Z, (const bf16*)Wbuf, (const bf16*)Wd,
                                                              table, (bf16*)O, p.T, p.C, p.N, p.d, p.f, tiles_m,
                                                              tiles_n);
  else
    apply_kernel<float><<<(unsigned)blocks, kThreads, 0, st>>>((const float*)Z, (const float*)Wbuf,
                                                               (const float*)Wd, table, (float*)O, p.T, p.C, p.N,
                                                               p.d, p.f, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace ipttt
