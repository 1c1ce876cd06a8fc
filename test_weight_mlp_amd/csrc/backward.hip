// Backward pass of the layer: the gradients of <O, dO> with respect to H,
// X0, W_gate, W_up, W_down, the conv weights and W_target.  The reverse of
// lijianxiong.blog "In-Place Test-Time Training" (方法 > 原地自适应, 高效的块状更新机制,
// 对齐语言模型的目标函数, 工程实现) and of the clip and reset of the iplexlaw.co.kr
// review, section 6: the plain chain rule through each forward step.
//
// The contractions run on one batched product, C[m, n] = sum over up to
// three operand pairs of sum_k A[m, k] B[n, k], both operands K-contiguous:
// nt_fast_kernel on the forward's 8-wave core (256 x 256 tiles) for bf16
// with K a multiple of 64, nt_kernel on the general 4-wave 128 x 128 tiles
// otherwise.  A batch is either one (row, chunk) of the problem, whose rows,
// output columns and K range can be restricted to the chunk's segments, or a
// plain matrix.  Operands whose K axis is not contiguous are transposed first.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "epilogue.h"
#include "launch.h"
#include "mfma_core.h"

namespace ipttt {

// ---------------------------------------------------------------- nt_kernel

template <typename T>
__global__ __launch_bounds__(kThreads) void nt_kernel(NTArgs a, const int32_t* __restrict__ table, int64_t Tn,
                                                      int C, int Nch) {
  typedef Geo<T, 128, 128> G;
  __shared__ __attribute__((aligned(16))) T lds[(G::BM + G::BN) * G::LDK];
  T* lA = lds;
  T* lB = lds + G::BM * G::LDK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int z = blockIdx.y;
  int64_t tok0 = 0;
  int mlo = 0, mhi = a.M, klo = 0, khi = 0, nlo = 0, nhi = a.N;
  bool kseg = false;
  if (a.chunked) {
    const int b = z / Nch, i = z - b * Nch;
    const int L = (int)min((int64_t)C, Tn - (int64_t)i * C);
    tok0 = (int64_t)b * Tn + (int64_t)i * C;
    const int r0 = table[z * 3 + 0], l0 = table[z * 3 + 1], carry = table[z * 3 + 2];
    switch (a.rows) {
      case NT_ROWS_ALL: mlo = 0; mhi = L; break;
      case NT_ROWS_HEAD: mlo = 0; mhi = r0; break;
      case NT_ROWS_TAIL: mlo = r0; mhi = L; break;
      default: mlo = l0; mhi = carry ? L : l0; break;  // the carried segment
    }
    if (a.kseg) { klo = l0; khi = L; kseg = true; }
    if (a.nseg) { nlo = l0; nhi = L; }
  }
  const int tiles_n = (a.N + G::BN - 1) / G::BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int m0 = tm * G::BM, n0 = tn * G::BN;
  if (mlo >= mhi || nlo >= nhi || m0 >= mhi || m0 + G::BM <= mlo || n0 >= nhi || n0 + G::BN <= nlo) return;

  floatx16 acc[G::MB][G::NB];
  zero_acc<G>(acc);
  for (int q = 0; q < a.npairs; ++q) {
    const NTPair& pq = a.pr[q];
    const int k_lo = kseg ? klo : 0, k_hi = kseg ? khi : pq.K;
    if (k_lo >= k_hi) continue;
    const T* Ab = static_cast<const T*>(pq.A);
    const T* Bb = static_cast<const T*>(pq.B);
    const T* Ap = pq.a_tok ? Ab + (tok0 + m0) * pq.lda : Ab + z * pq.sa + (int64_t)m0 * pq.lda;
    const T* Bp = pq.b_tok ? Bb + (tok0 + n0) * pq.ldb : Bb + z * pq.sb + (int64_t)n0 * pq.ldb;
    const int arows = mhi - m0, brows = nhi - n0;
    TileLoad<T, G::BM> la;
    TileLoad<T, G::BN> lb;
    const int kbeg = (k_lo / G::BK) * G::BK;
    la.load_kmask(Ap, pq.lda, arows, kbeg, k_lo, k_hi, tid);
    lb.load_kmask(Bp, pq.ldb, brows, kbeg, k_lo, k_hi, tid);
    for (int k0 = kbeg; k0 < k_hi; k0 += G::BK) {
      la.template store<G::LDK>(lA, tid);
      lb.template store<G::LDK>(lB, tid);
      __syncthreads();
      if (k0 + G::BK < k_hi) {
        la.load_kmask(Ap, pq.lda, arows, k0 + G::BK, k_lo, k_hi, tid);
        lb.load_kmask(Bp, pq.ldb, brows, k0 + G::BK, k_lo, k_hi, tid);
      }
      stage_mma<T, G>(lA, lB, acc, wm, wn, lane);
      __syncthreads();
    }
  }
  const float sa = a.a0 * (a.ca != nullptr ? a.ca[z] : 1.0f);
  const float sx = a.x0 * (a.cx != nullptr ? a.cx[z] : 1.0f);
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = m0 + wm * G::WM + mb * 32 + acc_row(j, lane);
        const int c = n0 + wn * G::WN + nb * 32 + (lane & 31);
        if (r >= mlo && r < mhi && c >= nlo && c < nhi) {
          const int64_t idx = a.c_tok ? (tok0 + r) * a.ldc + c : z * a.sc + (int64_t)r * a.ldc + c;
          float v = sa * acc[mb][nb][j];
          if (a.X != nullptr) v += sx * a.X[idx];
          if (a.c_f32)
            static_cast<float*>(a.C)[idx] = v;
          else
            static_cast<T*>(a.C)[idx] = from_f32<T>(v);
        }
      }
}

// bf16 products with K a multiple of 64 and no K restriction run on the
// 8-wave core of the forward (256 x 256 tiles, direct-to-LDS loads through
// buffer resources that end at the last valid row, so rows past the range
// read as zero), on its half-stage ring: the chunk weights and their
// adjoints stream from HBM; same batches, ranges and epilogue as nt_kernel.
typedef core::Tile8H<256, 256, 1, 2, 4> NTFast;
typedef core::Tile8H<256, 256, 1, 2, 4, 1> NTFastFrag;   // B fragment-major
typedef core::Tile8H<256, 256, 1, 2, 4, 2> NTFastFragT;  // B transposed fragment-major
typedef core::Tile8H<256, 256, 1, 2, 4, 3> NTFastKmaj;   // B = X^T, X row-major [K, N]

// One operand pair's K loop.  The operands are restrict parameters of this
// inlined function: the compiler then tells the core's LDS reads apart from
// its direct-to-LDS operand loads, and inserts no wait for those loads in
// front of the (transposing) reads; the core's own stage waits order them.
template <class TILE>
__device__ __forceinline__ void nt_pair_run(const bf16* __restrict__ Ap, int64_t astride, int64_t abytes,
                                            const bf16* __restrict__ Bp, int64_t bstride, int64_t bbytes, int K,
                                            bf16* lds, floatx16 (&acc)[1][2][4], int wave, int lane) {
  const core::Operand oa = core::make_operand(Ap, astride, abytes);
  const core::Operand ob[1] = {core::make_operand(Bp, bstride, bbytes)};
  TILE::run(oa, ob, K, lds, acc, wave, lane);
}

// Pair q's B layout is (MODES >> 2q) & 3: 0 rows, 1 fragment-major (the
// forward's chunk weights W [d, f] as B = W, K = f), 2 the same layout used
// transposed (B = W^T, K = d), 3 K-major rows (B = X^T for X [K, N]
// row-major: the chunk's token rows, K = token, rows past the chunk read as
// zero; or a plain matrix such as W_gate [f, d] in dH = dG W_gate).
//
// Workgroups are numbered 1-D.  When xcd_batches is set (the batch count is
// then a multiple of 8), each XCD (workgroup id mod 8) takes whole batches, and walks a batch's
// tiles with the token tiles of one column tile next to each other: the
// chunk's per-batch operands (up to 100 MB of weights and their adjoints)
// then stream through that XCD's L2 once, each column tile of B read by its
// token tiles back to back, and the token tiles of A stay resident for every
// column tile.  Otherwise tiles go row-major, batch by batch (so that the few
// busy batches of a product restricted to the chunks' tails spread over every
// XCD).
template <int MODES>
__global__ __launch_bounds__(NTFast::NT) void nt_fast_kernel(NTArgs a, const int32_t* __restrict__ table,
                                                             int64_t Tn, int C, int Nch, bool xcd_batches,
                                                             int tiles_m) {
  constexpr int BM = 256, BN = 256;
  __shared__ __attribute__((aligned(1024))) bf16 lds[NTFast::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (a.N + BN - 1) / BN, tiles = tiles_m * tiles_n;
  int z, tm, tn;
  if (xcd_batches) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int t = slot % tiles;
    z = xcd + 8 * (slot / tiles);
    tm = t % tiles_m;
    tn = t / tiles_m;
  } else {
    const int t = blockIdx.x % tiles;
    z = blockIdx.x / tiles;
    tm = t / tiles_n;
    tn = t - tm * tiles_n;
  }
  int64_t tok0 = 0;
  int mlo = 0, mhi = a.M, nlo = 0, nhi = a.N, L = 0;
  bool alt0 = false;  // pair 0 reads a.tail_B
  if (a.chunked) {
    const int b = z / Nch, i = z - b * Nch;
    L = (int)min((int64_t)C, Tn - (int64_t)i * C);
    tok0 = (int64_t)b * Tn + (int64_t)i * C;
    const int r0 = table[z * 3 + 0], l0 = table[z * 3 + 1], carry = table[z * 3 + 2];
    switch (a.rows) {
      case NT_ROWS_ALL: mlo = 0; mhi = L; break;
      case NT_ROWS_HEAD: mlo = 0; mhi = r0; break;
      case NT_ROWS_TAIL: mlo = r0; mhi = L; break;
      case NT_ROWS_HEADZ: mlo = 0; mhi = r0 == 0 ? L : r0; alt0 = r0 == 0; break;
      case NT_ROWS_TAILNZ: mlo = r0; mhi = r0 == 0 ? 0 : L; break;
      default: mlo = l0; mhi = carry ? L : l0; break;
    }
    if (a.nseg) { nlo = l0; nhi = L; }
  }
  const int m0 = tm * BM, n0 = tn * BN;
  if (mlo >= mhi || nlo >= nhi || m0 >= mhi || m0 + BM <= mlo || n0 >= nhi || n0 + BN <= nlo) return;
  floatx16 acc[1][2][4];
  core::zero(acc);
  // constant pair indices keep each pair's fields in scalar registers
  auto pair = [&](auto qc) {
    constexpr int q = decltype(qc)::value, mode = (MODES >> (2 * q)) & 3;
    if (q >= a.npairs) return false;
    const NTPair& pq = a.pr[q];
    const bf16* Ab = static_cast<const bf16*>(pq.A);
    const bool alt = q == 0 && alt0;
    const bf16* Bb = static_cast<const bf16*>(alt ? a.tail_B : pq.B);
    const int64_t sbq = alt ? 0 : pq.sb;
    const bf16* Ap = pq.a_tok ? Ab + (tok0 + m0) * pq.lda : Ab + z * pq.sa + (int64_t)m0 * pq.lda;
    const int64_t abytes = (int64_t)(mhi - m0) * pq.lda * 2;
    if constexpr (mode == 1) {
      // 32-row blocks of K/16 fragments of 1 KB each
      const bf16* Bp = Bb + z * sbq + (int64_t)(n0 / 32) * (pq.K / 16) * 512;
      nt_pair_run<NTFastFrag>(Ap, pq.lda * 2, abytes, Bp, (int64_t)pq.K * 64, (int64_t)(nhi - n0) * pq.K * 2, pq.K,
                              lds, acc, wave, lane);
    } else if constexpr (mode == 2) {
      // K/32 blocks of ldb/16 fragments; this tile's columns start at
      // fragment n0/16 of every block
      const bf16* Bp = Bb + z * sbq + (int64_t)(n0 / 16) * 512;
      nt_pair_run<NTFastFragT>(Ap, pq.lda * 2, abytes, Bp, pq.ldb * 64,
                               (int64_t)pq.K * pq.ldb * 2 - (int64_t)(n0 / 16) * 1024, pq.K, lds, acc, wave, lane);
    } else if constexpr (mode == 3) {
      // X's rows from column n0 on: the chunk's token rows (rows past L read
      // as zero) or the batch's K rows
      const bf16* Bp = (pq.b_tok ? Bb + tok0 * pq.ldb : Bb + z * sbq) + n0;
      const int64_t rows = pq.b_tok ? L : pq.K;
      nt_pair_run<NTFastKmaj>(Ap, pq.lda * 2, abytes, Bp, pq.ldb * 2, rows * pq.ldb * 2 - (int64_t)n0 * 2, pq.K, lds,
                              acc, wave, lane);
    } else {
      const bf16* Bp = pq.b_tok ? Bb + (tok0 + n0) * pq.ldb : Bb + z * sbq + (int64_t)n0 * pq.ldb;
      nt_pair_run<NTFast>(Ap, pq.lda * 2, abytes, Bp, pq.ldb * 2, (int64_t)(nhi - n0) * pq.ldb * 2, pq.K, lds, acc,
                          wave, lane);
    }
    return true;
  };
  if (pair(std::integral_constant<int, 0>{}) && pair(std::integral_constant<int, 1>{}))
    pair(std::integral_constant<int, 2>{});
  const float sa = a.a0 * (a.ca != nullptr ? a.ca[z] : 1.0f);
  const float sx = a.x0 * (a.cx != nullptr ? a.cx[z] : 1.0f);
  const bool staged = !a.c_f32 && !a.nseg && (a.ldc & 7) == 0 && (a.N & 7) == 0 && (a.c_tok || (a.sc & 7) == 0);
  if (staged) {
    // bf16 output over whole rows: the tile goes through LDS (the stage
    // buffers, free after the K loop) and out in 16-byte row stores; X, if
    // any, is read in the accumulator layout (32 consecutive floats a row)
    constexpr int LDR = BN;
    static_assert(BM * LDR <= NTFast::LDS_ELEMS, "staging tile");
    // X through a buffer resource that ends at row mhi: rows outside
    // [mlo, mhi) and columns past nhi read as zero, with no branches, so
    // that the loads of a block issue back to back
    const float* Xb = a.X != nullptr ? a.X + (a.c_tok ? tok0 * a.ldc : z * a.sc) : nullptr;
    const int64_t xbytes = (int64_t)mhi * a.ldc * 4;
    const bool xin = Xb != nullptr && xbytes < 0x7FFFFF00LL;
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(Xb), (short)0, xin ? (int)xbytes : 0, 0x00020000);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = sa * acc[0][mb][nb][j];
        if (Xb != nullptr) {
          const int c = n0 + wn * 128 + nb * 32 + (lane & 31);
          if (xin) {
            float x[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int r = m0 + wm * 64 + mb * 32 + acc_row(j, lane);
              const uint32_t off = (r >= mlo && c < nhi) ? ((uint32_t)r * (uint32_t)a.ldc + (uint32_t)c) * 4u
                                                         : 0x7FFFFF00u;
              x[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(xr, (int)off, 0, 0));
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] += sx * x[j];
          } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int r = m0 + wm * 64 + mb * 32 + acc_row(j, lane);
              if (r >= mlo && r < mhi && c < nhi) v[j] += sx * Xb[(int64_t)r * a.ldc + c];
            }
          }
        }
        stage_block_rows_swz<LDR>(v, lds, wm * 64 + mb * 32, wn * 128 + nb * 32, lane);
      }
    core::lds_barrier();
    bf16* out = static_cast<bf16*>(a.C) + (a.c_tok ? tok0 * a.ldc : z * a.sc);
    store_rows_swz<BM, BN, LDR, NTFast::NT>(lds, out, m0, max(mlo - m0, 0), min(mhi - m0, BM), n0, nhi - n0,
                                            (int)a.ldc, tid);
    return;
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = m0 + wm * 64 + mb * 32 + acc_row(j, lane);
        const int c = n0 + wn * 128 + nb * 32 + (lane & 31);
        if (r >= mlo && r < mhi && c >= nlo && c < nhi) {
          const int64_t idx = a.c_tok ? (tok0 + r) * a.ldc + c : z * a.sc + (int64_t)r * a.ldc + c;
          float v = sa * acc[0][mb][nb][j];
          if (a.X != nullptr) v += sx * a.X[idx];
          if (a.c_f32)
            static_cast<float*>(a.C)[idx] = v;
          else
            static_cast<bf16*>(a.C)[idx] = (bf16)v;
        }
      }
}

static bool nt_fast_ok(const Prob& p, const NTArgs& a) {
  if (p.dtype != 1 || (a.kseg && !a.kzero) || a.npairs < 1 || a.npairs > 3) return false;
  auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  if (a.chunked && a.rows == NT_ROWS_HEADZ && (a.tail_B == nullptr || !al16(a.tail_B))) return false;
  // the loads address a tile's 256 rows with 32-bit offsets
  const int64_t lim = (int64_t(1) << 32) - 4096;
  for (int q = 0; q < a.npairs; ++q) {
    const NTPair& pq = a.pr[q];
    if (pq.A == nullptr || pq.B == nullptr || !al16(pq.A) || !al16(pq.B)) return false;
    if (pq.K % NTFast::KS != 0 || pq.lda % 8 != 0) return false;
    if (pq.lda * 2 * 256 + (int64_t)pq.K * 2 >= lim) return false;
    if (pq.b_frag) {
      if (pq.b_tok || (int64_t)pq.K * 2 * 256 >= lim) return false;
    } else if (pq.b_fragt) {
      // the fragments' row blocks are whole 16-column steps
      if (pq.b_tok || pq.ldb % 16 != 0 || pq.K * pq.ldb * 2 >= lim) return false;
    } else if (pq.b_kmaj) {
      if ((pq.b_tok && !a.chunked) || pq.ldb % 8 != 0 || (int64_t)(pq.K + 64) * pq.ldb * 2 >= lim) return false;
    } else if (pq.ldb % 8 != 0 || pq.ldb * 2 * 256 + (int64_t)pq.K * 2 >= lim) {
      return false;
    }
  }
  return true;
}

hipError_t launch_nt(const Prob& p, const NTArgs& a, int batches, const int32_t* table, hipStream_t st) {
  note_launch("nt", st);
  const int rows = a.chunked ? p.C : a.M;
  const int nb = a.chunked ? (int)(p.B * p.N) : batches;
  if (rows <= 0 || a.N <= 0 || nb <= 0) return hipSuccess;
  const bool fast = nt_fast_ok(p, a);
  int modes = 0;
  for (int q = 0; q < a.npairs && q < 3; ++q) {
    if (a.pr[q].b_frag + a.pr[q].b_fragt + a.pr[q].b_kmaj > 1) return hipErrorInvalidValue;
    modes |= (a.pr[q].b_frag ? 1 : a.pr[q].b_fragt ? 2 : a.pr[q].b_kmaj ? 3 : 0) << (2 * q);
  }
  // fragment-major B and the HEADZ/TAILNZ rows need the 8-wave path
  const bool zrows = a.chunked && (a.rows == NT_ROWS_HEADZ || a.rows == NT_ROWS_TAILNZ);
  if ((modes != 0 || zrows) && !fast) return hipErrorInvalidValue;
  if (fast) {
    const int tiles_m = (rows + 255) / 256;
    const int64_t wgs = (int64_t)tiles_m * ((a.N + 255) / 256) * nb;
    if (wgs >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    const dim3 g((unsigned)wgs);
    const bool xb = nb % 8 == 0 && !(a.chunked && (a.rows == NT_ROWS_TAIL || a.rows == NT_ROWS_TAILNZ));
    switch (modes) {
      case 0: nt_fast_kernel<0><<<g, NTFast::NT, 0, st>>>(a, table, p.T, p.C, p.N, xb, tiles_m); break;
      case 1: nt_fast_kernel<1><<<g, NTFast::NT, 0, st>>>(a, table, p.T, p.C, p.N, xb, tiles_m); break;
      case 2 | (2 << 2):
        nt_fast_kernel<2 | (2 << 2)><<<g, NTFast::NT, 0, st>>>(a, table, p.T, p.C, p.N, xb, tiles_m);
        break;
      case 3: nt_fast_kernel<3><<<g, NTFast::NT, 0, st>>>(a, table, p.T, p.C, p.N, xb, tiles_m); break;
      case 3 | (3 << 2):
        nt_fast_kernel<3 | (3 << 2)><<<g, NTFast::NT, 0, st>>>(a, table, p.T, p.C, p.N, xb, tiles_m);
        break;
      case 2 | (2 << 2) | (3 << 4):
        nt_fast_kernel<2 | (2 << 2) | (3 << 4)><<<g, NTFast::NT, 0, st>>>(a, table, p.T, p.C, p.N, xb, tiles_m);
        break;
      default: return hipErrorInvalidValue;  // a combination no caller uses
    }
    return hipGetLastError();
  }
  const int64_t tiles = (int64_t)((rows + 127) / 128) * ((a.N + 127) / 128);
  dim3 g((unsigned)tiles, (unsigned)nb);
  if (p.dtype == 1)
    nt_kernel<bf16><<<g, kThreads, 0, st>>>(a, table, p.T, p.C, p.N);
  else
    nt_kernel<float><<<g, kThreads, 0, st>>>(a, table, p.T, p.C, p.N);
  return hipGetLastError();
}

// ------------------------------------------------------------ small kernels

// 8 consecutive elements to or from fp32 registers (16- or 32-byte accesses).
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<bf16>(const bf16* p, float (&v)[8]) {
  const bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)x[i];
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const float4_t a = *reinterpret_cast<const float4_t*>(p), b = *reinterpret_cast<const float4_t*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = a[i], v[4 + i] = b[i];
}
__device__ __forceinline__ void store8(bf16* p, const float (&v)[8]) {
  bf16x8 x;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (bf16)v[i];
  *reinterpret_cast<bf16x8*>(p) = x;
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4_t*>(p) = float4_t{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<float4_t*>(p + 4) = float4_t{v[4], v[5], v[6], v[7]};
}


// out[c * Rp + r] = in[r * Cc + c] for r < R, zero for R <= r < Rp.
template <typename T>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const T* __restrict__ in, T* __restrict__ out, int64_t R,
                                                            int Cc, int64_t Rp) {
  __shared__ T tile[32][33];
  const int64_t r0 = (int64_t)blockIdx.x * 32;
  const int c0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int k = ty; k < 32; k += 8) {
    const int64_t r = r0 + k;
    const int c = c0 + tx;
    tile[k][tx] = (r < R && c < Cc) ? in[r * Cc + c] : from_f32<T>(0.0f);
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int c = c0 + k;
    const int64_t r = r0 + tx;
    if (c < Cc && r < Rp) out[(int64_t)c * Rp + r] = tile[tx][k];
  }
}

hipError_t launch_transpose_pad(const Prob& p, const void* in, int64_t R, int Cc, int64_t Rp, void* out,
                                hipStream_t st) {
  note_launch("transpose_pad", st);
  dim3 g((unsigned)((Rp + 31) / 32), (unsigned)((Cc + 31) / 32));
  if (p.dtype == 1)
    transpose_pad_kernel<bf16><<<g, 256, 0, st>>>((const bf16*)in, (bf16*)out, R, Cc, Rp);
  else
    transpose_pad_kernel<float><<<g, 256, 0, st>>>((const float*)in, (float*)out, R, Cc, Rp);
  return hipGetLastError();
}

// out[e] = sum_{q < P} part[q * n + e], in the order q = 0, 1, ...
__global__ __launch_bounds__(256) void sum_parts_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                        int64_t n, int P) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  float s = 0.0f;
  for (int q = 0; q < P; ++q) s += part[(int64_t)q * n + e];
  out[e] = s;
}

// Sums of a group of consecutive parts, left in place in the group's first
// part (group g: parts [g * per, min(P, (g + 1) * per)), in order).
__global__ __launch_bounds__(256) void sum_groups_kernel(float* __restrict__ part, int64_t n, int P, int per) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  const int q0 = blockIdx.y * per, q1 = min(P, q0 + per);
  float s = 0.0f;
  for (int q = q0; q < q1; ++q) s += part[(int64_t)q * n + e];
  part[(int64_t)q0 * n + e] = s;
}

// out[e] = sum of the group sums, in group order.
__global__ __launch_bounds__(256) void sum_strided_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                          int64_t n, int G, int64_t stride) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= n) return;
  float s = 0.0f;
  for (int g = 0; g < G; ++g) s += part[(int64_t)g * stride + e];
  out[e] = s;
}

hipError_t launch_sum_parts(float* part, float* out, int64_t n, int P, hipStream_t st) {
  note_launch("sum_parts", st);
  const unsigned gx = (unsigned)((n + 255) / 256);
  if (P >= 64 && n < (int64_t(1) << 22)) {
    // many parts of a short vector: first sum groups of parts in parallel
    const int G = 32, per = (P + G - 1) / G, groups = (P + per - 1) / per;
    sum_groups_kernel<<<dim3(gx, (unsigned)groups), 256, 0, st>>>(part, n, P, per);
    sum_strided_kernel<<<gx, 256, 0, st>>>(part, out, n, groups, (int64_t)per * n);
    return hipGetLastError();
  }
  sum_parts_kernel<<<gx, 256, 0, st>>>(part, out, n, P);
  return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ in, T* __restrict__ out, int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n) out[e] = from_f32<T>(in[e]);
}

template <typename T>
__global__ __launch_bounds__(256) void widen_kernel(const T* __restrict__ in, float* __restrict__ out, int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n) out[e] = to_f32(in[e]);
}

// fp32 -> dtype (to_dtype) or dtype -> fp32.
hipError_t launch_convert(const Prob& p, const void* in, void* out, int64_t n, bool to_dtype, hipStream_t st) {
  note_launch("convert", st);
  const unsigned g = (unsigned)((n + 255) / 256);
  if (to_dtype) {
    if (p.dtype == 1) convert_kernel<bf16><<<g, 256, 0, st>>>((const float*)in, (bf16*)out, n);
    else convert_kernel<float><<<g, 256, 0, st>>>((const float*)in, (float*)out, n);
  } else {
    if (p.dtype == 1) widen_kernel<bf16><<<g, 256, 0, st>>>((const bf16*)in, (float*)out, n);
    else widen_kernel<float><<<g, 256, 0, st>>>((const float*)in, (float*)out, n);
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n_words) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n_words) p[e] = 0u;
}

hipError_t launch_zero(void* ptr, size_t bytes, hipStream_t st) {
  note_launch("zero", st);
  const int64_t n = (int64_t)(bytes / 4);
  if (n > 0) fill_zero_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>((uint32_t*)ptr, n);
  return hipGetLastError();
}

// One pass over each chunk's tokens, kDotParts workgroups per chunk: on the
// carried segment [l0, L) of a carrying chunk, the partial sums of
// <V_hat, A> (A = Z dDW^T, fp32), summed in order by coef_kernel, and
// Vc = cpos V_hat with cpos = eta alpha (the coefficient coef_kernel gives
// such a chunk); Vc = 0 on every other token.  8 features per thread.
template <typename T>
__global__ __launch_bounds__(256) void seg_dot_scale_kernel(const T* __restrict__ V, const float* __restrict__ A,
                                                            const int32_t* __restrict__ table,
                                                            const float* __restrict__ alpha, float eta,
                                                            float* __restrict__ dots, T* __restrict__ Vc, int64_t Tn,
                                                            int C, int N, int d) {
  const int z = blockIdx.y, part = blockIdx.x;
  const int b = z / N, i = z - b * N;
  const int L = (int)min((int64_t)C, Tn - (int64_t)i * C);
  const int l0 = table[z * 3 + 1], carry = table[z * 3 + 2];
  const float cz = carry ? eta * alpha[z] : 0.0f;
  const int64_t tok0 = (int64_t)b * Tn + (int64_t)i * C;
  const int vpr = d >> 3;
  const int64_t nv = (int64_t)L * vpr;
  float s = 0.0f;
  for (int64_t v = (int64_t)part * blockDim.x + threadIdx.x; v < nv; v += (int64_t)kDotParts * blockDim.x) {
    const int t = (int)(v / vpr), c = (int)(v - (int64_t)t * vpr) * 8;
    const int64_t off = (tok0 + t) * d + c;
    float x[8], y[8];
    if (carry && t >= l0) {
      float a[8];
      load8(V + off, x);
      load8(A + off, a);
#pragma unroll
      for (int q = 0; q < 8; ++q) s += x[q] * a[q], y[q] = cz * x[q];
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) y[q] = 0.0f;
    }
    store8(Vc + off, y);
  }
  __shared__ float red[256];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) dots[(int64_t)z * kDotParts + part] = red[0];
}

hipError_t launch_seg_dot_scale(const Prob& p, const void* V, const float* A, const int32_t* table,
                                const float* alpha, float eta, float* dots, void* Vc, hipStream_t st) {
  note_launch("seg_dot_scale", st);
  dim3 g(kDotParts, (unsigned)(p.B * p.N));
  if (p.dtype == 1)
    seg_dot_scale_kernel<bf16><<<g, 256, 0, st>>>((const bf16*)V, A, table, alpha, eta, dots, (bf16*)Vc, p.T, p.C,
                                                  p.N, p.d);
  else
    seg_dot_scale_kernel<float><<<g, 256, 0, st>>>((const float*)V, A, table, alpha, eta, dots, (float*)Vc, p.T,
                                                   p.C, p.N, p.d);
  return hipGetLastError();
}

// Per (row, chunk): the coefficients of the delta's adjoint,
// dD = eta alpha (dDW - kappa D) with kappa = <dDW, D> / |D|^2 when the chunk
// was clipped (the derivative of tau D / |D|), else 0:
//   cpos = eta alpha (carrying chunks; 0 otherwise), cneg = -cpos kappa.
// |D|^2 is the sum of the Gram partials of the forward's clip (or, with gram
// NULL, follows from the clip scale itself), <dDW, D> the sum of the seg_dot
// partials; both in fp64 in a fixed order.
__global__ __launch_bounds__(256) void coef_kernel(const float* __restrict__ alpha, const float* __restrict__ gram,
                                                   int npairs, const float* __restrict__ dots,
                                                   const int32_t* __restrict__ table, float eta, float tau,
                                                   float* __restrict__ cpos, float* __restrict__ cneg, int nchunks) {
  const int z = blockIdx.x * blockDim.x + threadIdx.x;
  if (z >= nchunks) return;
  const bool carry = table[z * 3 + 2] != 0;
  const float c = carry ? eta * alpha[z] : 0.0f;
  double kappa = 0.0;
  if (carry && tau > 0.0f && alpha[z] < 1.0f) {
    double n2 = 0.0, dot = 0.0;
    if (gram != nullptr) {
      for (int k = 0; k < npairs; ++k) n2 += (double)gram[(int64_t)z * npairs + k];
    } else {
      // the clip acted: alpha = tau / (|eta| |D|), so |D|^2 = (tau / (|eta| alpha))^2
      const double nd = (double)tau / (fabs((double)eta) * (double)alpha[z]);
      n2 = nd * nd;
    }
    for (int k = 0; k < kDotParts; ++k) dot += (double)dots[(int64_t)z * kDotParts + k];
    if (n2 > 0.0) kappa = dot / n2;
  }
  cpos[z] = c;
  cneg[z] = (float)(-(double)c * kappa);
}

hipError_t launch_coef(const Prob& p, const float* alpha, const float* gram, int npairs, const float* dots,
                       const int32_t* table, float eta, float tau, float* cpos, float* cneg, hipStream_t st) {
  note_launch("coef", st);
  const int n = (int)(p.B * p.N);
  coef_kernel<<<(n + 255) / 256, 256, 0, st>>>(alpha, gram, npairs, dots, table, eta, tau, cpos, cneg, n);
  return hipGetLastError();
}

// ------------------------------------------------------------ gated MLP

// dG = dZ * U * SiLU'(G), dU = dZ * SiLU(G) with G = H W_gate^T and
// U = H W_up^T recomputed on the matrix cores (the dual product of the
// forward's Z kernel, general tiles), written in dtype.
// SiLU'(x) = s (1 + x (1 - s)) with s the logistic function.
template <typename T>
__global__ __launch_bounds__(kThreads) void gated_z_bwd_kernel(const T* __restrict__ H, const T* __restrict__ Wg,
                                                               const T* __restrict__ Wu, const T* __restrict__ dZ,
                                                               T* __restrict__ dG, T* __restrict__ dU, int64_t M,
                                                               int d, int f) {
  typedef Geo<T, 128, 128> G;
  __shared__ __attribute__((aligned(16))) T lds[(G::BM + 2 * G::BN) * G::LDK];
  T* lA = lds;
  T* lB0 = lds + G::BM * G::LDK;
  T* lB1 = lB0 + G::BN * G::LDK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (f + G::BN - 1) / G::BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int64_t m0 = (int64_t)tm * G::BM;
  const int n0 = tn * G::BN;
  const int mrows = (int)min((int64_t)G::BM, M - m0), nrows = min(G::BN, f - n0);
  const T* A = H + m0 * d;
  const T* B0 = Wg + (int64_t)n0 * d;
  const T* B1 = Wu + (int64_t)n0 * d;
  floatx16 ag[G::MB][G::NB], au[G::MB][G::NB];
  zero_acc<G>(ag);
  zero_acc<G>(au);
  TileLoad<T, G::BM> la;
  TileLoad<T, G::BN> lb0, lb1;
  la.load(A, d, mrows, 0, d, tid);
  lb0.load(B0, d, nrows, 0, d, tid);
  lb1.load(B1, d, nrows, 0, d, tid);
  for (int k0 = 0; k0 < d; k0 += G::BK) {
    la.template store<G::LDK>(lA, tid);
    lb0.template store<G::LDK>(lB0, tid);
    lb1.template store<G::LDK>(lB1, tid);
    __syncthreads();
    if (k0 + G::BK < d) {
      la.load(A, d, mrows, k0 + G::BK, d, tid);
      lb0.load(B0, d, nrows, k0 + G::BK, d, tid);
      lb1.load(B1, d, nrows, k0 + G::BK, d, tid);
    }
    stage_mma<T, G>(lA, lB0, ag, wm, wn, lane);
    stage_mma<T, G>(lA, lB1, au, wm, wn, lane);
    __syncthreads();
  }
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = wm * G::WM + mb * 32 + acc_row(j, lane);
        const int c = wn * G::WN + nb * 32 + (lane & 31);
        if (r < mrows && c < nrows) {
          const int64_t idx = (m0 + r) * f + n0 + c;
          const float g = ag[mb][nb][j], u = au[mb][nb][j], dz = to_f32(dZ[idx]);
          const float s = 1.0f / (1.0f + __expf(-g));
          dG[idx] = from_f32<T>(dz * u * (s * (1.0f + g * (1.0f - s))));
          dU[idx] = from_f32<T>(dz * g * s);
        }
      }
}

// bf16, d_model a multiple of 64: the same on the forward Z kernel's 8-wave
// core (256 tokens x 128 features of both products per workgroup).
typedef core::Tile8<256, 128, 2, 2, 2> ZBTile;

__global__ __launch_bounds__(ZBTile::NT) void gated_z_bwd_fast_kernel(const bf16* __restrict__ H,
                                                                     const bf16* __restrict__ Wg,
                                                                     const bf16* __restrict__ Wu,
                                                                     const bf16* __restrict__ dZ,
                                                                     bf16* __restrict__ dG, bf16* __restrict__ dU,
                                                                     int64_t M, int d, int f) {
  constexpr int BM = 256, BN = 128;
  __shared__ __attribute__((aligned(1024))) bf16 lds[ZBTile::LDS_ELEMS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (f + BN - 1) / BN;
  int tm, tn;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, 8, tm, tn);
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  const core::Operand oa = core::make_operand(H + m0 * d, (int64_t)d * 2, (M - m0) * d * 2);
  const core::Operand ob[2] = {core::make_operand(Wg + (int64_t)n0 * d, (int64_t)d * 2, (int64_t)(f - n0) * d * 2),
                               core::make_operand(Wu + (int64_t)n0 * d, (int64_t)d * 2, (int64_t)(f - n0) * d * 2)};
  floatx16 acc[2][2][2];
  core::zero(acc);
  ZBTile::run(oa, ob, d, lds, acc, wave, lane);
  // Epilogue through LDS (both stage buffers are free now): the dZ tile is
  // read in 16-byte rows into buffer 0, dG is staged in buffer 1 and stored
  // in rows, then dU takes buffer 0 (the same swizzled staging as the
  // forward Z kernel).
  const int tid = threadIdx.x;
  const int mrows = (int)min((int64_t)BM, M - m0), nrows = min(BN, f - n0);
  bf16* zt = lds;                        // [BM][BN] dZ, row-major
  bf16* stg = lds + ZBTile::STAGE;       // staging of dG
  for (int v = tid; v < BM * (BN / 8); v += ZBTile::NT) {
    const int r = v / (BN / 8), c = (v % (BN / 8)) * 8;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (r < mrows && c < nrows) x = *reinterpret_cast<const u32x4*>(dZ + (m0 + r) * f + n0 + c);
    *reinterpret_cast<u32x4*>(zt + r * BN + c) = x;
  }
  core::lds_barrier();
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float g[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = wm * 64 + mb * 32 + acc_row(j, lane), c = wn * 64 + nb * 32 + (lane & 31);
        const float x = acc[0][mb][nb][j], u = acc[1][mb][nb][j], dz = (float)zt[r * BN + c];
        const float s = 1.0f / (1.0f + __expf(-x));
        g[j] = dz * u * (s * (1.0f + x * (1.0f - s)));
        acc[1][mb][nb][j] = dz * x * s;  // dU, kept until buffer 0 is free
      }
      stage_block_rows_swz<BN>(g, stg, wm * 64 + mb * 32, wn * 64 + nb * 32, lane);
    }
  core::lds_barrier();
  store_rows_swz<BM, BN, BN, ZBTile::NT, true>(stg, dG, m0, 0, mrows, n0, nrows, f, tid);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float u[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) u[j] = acc[1][mb][nb][j];
      stage_block_rows_swz<BN>(u, zt, wm * 64 + mb * 32, wn * 64 + nb * 32, lane);
    }
  core::lds_barrier();
  store_rows_swz<BM, BN, BN, ZBTile::NT, true>(zt, dU, m0, 0, mrows, n0, nrows, f, tid);
}

hipError_t launch_gated_z_bwd(const Prob& p, const void* H, const void* Wg, const void* Wu, const void* dZ, void* dG,
                              void* dU, hipStream_t st) {
  note_launch("gated_z_bwd", st);
  if (p.dtype == 1 && p.d % 64 == 0) {
    const int64_t tiles = ((p.M + 255) / 256) * ((p.f + 127) / 128);
    gated_z_bwd_fast_kernel<<<(unsigned)tiles, ZBTile::NT, 0, st>>>((const bf16*)H, (const bf16*)Wg,
                                                                    (const bf16*)Wu, (const bf16*)dZ, (bf16*)dG,
                                                                    (bf16*)dU, p.M, p.d, p.f);
    return hipGetLastError();
  }
  const int64_t tiles = ((p.M + 127) / 128) * ((p.f + 127) / 128);
  if (p.dtype == 1)
    gated_z_bwd_kernel<bf16><<<(unsigned)tiles, kThreads, 0, st>>>((const bf16*)H, (const bf16*)Wg, (const bf16*)Wu,
                                                                   (const bf16*)dZ, (bf16*)dG, (bf16*)dU, p.M, p.d,
                                                                   p.f);
  else
    gated_z_bwd_kernel<float><<<(unsigned)tiles, kThreads, 0, st>>>((const float*)H, (const float*)Wg,
                                                                    (const float*)Wu, (const float*)dZ, (float*)dG,
                                                                    (float*)dU, p.M, p.d, p.f);
  return hipGetLastError();
}

// dG = dZ * U * SiLU'(G), dU = dZ * SiLU(G) from the G and U the forward
// saved (the same formulas as the recomputing kernels), 8 elements a thread.
template <typename T>
__global__ __launch_bounds__(256) void gated_grad_kernel(const T* __restrict__ Gs, const T* __restrict__ Us,
                                                         const T* __restrict__ dZ, T* __restrict__ dG,
                                                         T* __restrict__ dU, int64_t n8) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= n8) return;
  float g[8], u[8], dz[8], a[8], b[8];
  load8(Gs + v * 8, g);
  load8(Us + v * 8, u);
  load8(dZ + v * 8, dz);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float s = 1.0f / (1.0f + __expf(-g[q]));
    a[q] = dz[q] * u[q] * (s * (1.0f + g[q] * (1.0f - s)));
    b[q] = dz[q] * g[q] * s;
  }
  store8(dG + v * 8, a);
  store8(dU + v * 8, b);
}

hipError_t launch_gated_grad(const Prob& p, const void* GU, const void* dZ, void* dG, void* dU, hipStream_t st) {
  note_launch("gated_grad", st);
  const int64_t n = p.M * p.f, n8 = n / 8;  // f is a multiple of 8
  const unsigned g = (unsigned)((n8 + 255) / 256);
  if (p.dtype == 1)
    gated_grad_kernel<bf16><<<g, 256, 0, st>>>((const bf16*)GU, (const bf16*)GU + n, (const bf16*)dZ, (bf16*)dG,
                                               (bf16*)dU, n8);
  else
    gated_grad_kernel<float><<<g, 256, 0, st>>>((const float*)GU, (const float*)GU + n, (const float*)dZ, (float*)dG,
                                                (float*)dU, n8);
  return hipGetLastError();
}

// ------------------------------------------------------------------ conv

// Both conv gradients in one pass (d is a multiple of 8): a thread owns 8
// channels and a run of R consecutive tokens, and slides two 5-row windows
// down the run, dY[s-4 .. s] for dX0[s] and X0[s .. s+4] for the weight
// gradient of token s, so that dY and X0 are each read once (the rows the
// windows reach beyond the run come from the neighbouring runs, mostly out
// of L2).  Run q writes its weight-gradient partial sums to part[q][c][k];
// runs past the last token write zeros.
template <typename T>
__global__ __launch_bounds__(256) void conv_bwd_fused_kernel(const float* __restrict__ dY, const T* __restrict__ X0,
                                                             const T* __restrict__ convw,
                                                             const uint8_t* __restrict__ segs, T* __restrict__ dX0,
                                                             float* __restrict__ part, int64_t M, int d, int R) {
  const int groups = d >> 3;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)groups * kConvParts) return;
  const int q = (int)(idx / groups), c0 = (int)(idx - (int64_t)q * groups) * 8;
  const int64_t t0 = (int64_t)q * R, t1 = min(M, t0 + R);
  float w[5][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int k = 0; k < 5; ++k) w[k][i] = to_f32(convw[(c0 + i) * 5 + k]);
  // dyw[k] = dY[s - k] with its window's tap count tw[k]; xw[k] = X0[s + k]
  float dyw[5][8], xw[5][8], acc[5][8];
  int tw[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    tw[k] = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) dyw[k][i] = xw[k][i] = acc[k][i] = 0.0f;
  }
  if (t0 < t1) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t tp = t0 - 1 - k, tx = t0 + k;
      if (tp >= 0) {
        tw[k] = segs[tp] & 7;
        load8(dY + tp * d + c0, dyw[k]);
      }
      if (tx < M) load8(X0 + tx * d + c0, xw[k + 1]);
    }
  }
  for (int64_t s = t0; s < t1; ++s) {
#pragma unroll
    for (int k = 4; k > 0; --k) {
      tw[k] = tw[k - 1];
#pragma unroll
      for (int i = 0; i < 8; ++i) dyw[k][i] = dyw[k - 1][i];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) xw[k][i] = xw[k + 1][i];
    tw[0] = segs[s] & 7;
    load8(dY + s * d + c0, dyw[0]);
    if (s + 4 < M) load8(X0 + (s + 4) * d + c0, xw[4]);
    else
#pragma unroll
      for (int i = 0; i < 8; ++i) xw[4][i] = 0.0f;
    float dx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) dx[i] = 0.0f;
#pragma unroll
    for (int k = 0; k < 5; ++k)
      if (k < tw[k])
#pragma unroll
        for (int i = 0; i < 8; ++i) dx[i] += w[k][i] * dyw[k][i];
    store8(dX0 + s * d + c0, dx);
#pragma unroll
    for (int k = 0; k < 5; ++k)
      if (k < tw[0])
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[k][i] += dyw[0][i] * xw[k][i];
  }
  float* out = part + ((int64_t)q * d + c0) * 5;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int k = 0; k < 5; ++k) out[i * 5 + k] = acc[k][i];
}

hipError_t launch_conv_bwd(const Prob& p, const float* dY, const void* X0, const void* convw, const uint8_t* segs,
                           void* dX0, float* part, hipStream_t st) {
  note_launch("conv_bwd", st);
  if (p.d % 8 != 0) return hipErrorInvalidValue;
  const int R = (int)((p.M + kConvParts - 1) / kConvParts);
  const unsigned g = (unsigned)(((int64_t)(p.d / 8) * kConvParts + 255) / 256);
  if (p.dtype == 1)
    conv_bwd_fused_kernel<bf16><<<g, 256, 0, st>>>(dY, (const bf16*)X0, (const bf16*)convw, segs, (bf16*)dX0, part,
                                                   p.M, p.d, R);
  else
    conv_bwd_fused_kernel<float><<<g, 256, 0, st>>>(dY, (const float*)X0, (const float*)convw, segs, (float*)dX0,
                                                    part, p.M, p.d, R);
  return hipGetLastError();
}

}  // namespace ipttt
