// Chunk deltas and the fused scan of the fast-weight state.
//
// The update of chunk i is dW_i = eta V_hat_[i]^T Z_[i] (lijianxiong.blog
// "In-Place Test-Time Training", 对齐语言模型的目标函数: the gradient step of the
// negative inner-product loss), rescaled to Frobenius norm tau when larger
// (tencent article "榨干MLP的剩余价值", 详细步骤 4 note; iplexlaw.co.kr review,
// section 6).  Chunk i applies W_down plus the deltas of the chunks before it
// only: an exclusive prefix sum (lijianxiong.blog, 工程实现; iplexlaw review,
// sections 3 and 6), restarted at every document start.
//
// Kernels:
//   gram_kernel   per (row, chunk, token-tile pair): the masked contraction
//                 sum_{s,t} (V V^T)[s,t] (Z Z^T)[s,t] = ||V^T Z||_F^2 over the
//                 chunk's carried segment, without forming the d x f delta.
//   alpha_kernel  sums the partials in a fixed order (fp64) -> clip scale.
//   scan_kernel   one workgroup per 128 x 128 tile of the d x f state, resident
//                 in fp32 registers while it walks the chunks of one row: emit
//                 the chunk's effective weight W_down + S_i, then add
//                 alpha_i eta V_hat^T Z (token-axis MFMA contraction on the
//                 chunk-transposed copies).
//   dw_kernel     diagnostic: the carried delta of every chunk, materialised.
#include <algorithm>
#include <cstdlib>

#include "launch.h"
#include "common.h"
#include "mfma_core.h"
#include "epilogue.h"
#include "pingpong.h"

namespace ipttt {

constexpr int kGramTile = 128;

// The 8-wave Gram path (the shapes of the 8-wave scan): 256-token tile pairs
// (p <= q) of a chunk, the Z Z^T product split over d_ff into `gram_splits`
// ranges of whole 64-column stages so that the launch fills the CUs (the
// V V^T tile of each pair is formed once and stored).
constexpr int kGramFastTile = 256;
static int gram_tile_pairs(const Prob& p) {
  const int nt = (p.C + kGramFastTile - 1) / kGramFastTile;
  return nt * (nt + 1) / 2;
}
static int gram_splits(const Prob& p) {
  const int64_t wg = p.B * p.N * (int64_t)gram_tile_pairs(p);
  const int64_t want = (3 * 256 + wg - 1) / wg;  // about three rounds on 256 CUs
  return (int)std::max<int64_t>(1, std::min<int64_t>({want, 8, (int64_t)p.f / 64}));
}

int gram_pairs(const Prob& p) {
  if (fast_scan(p)) return gram_tile_pairs(p) * gram_splits(p);
  const int nt = (p.C + kGramTile - 1) / kGramTile;
  return nt * (nt + 1) / 2;
}

size_t gram_scratch_bytes(const Prob& p, int64_t chunks) {
  return fast_scan(p) ? (size_t)chunks * gram_tile_pairs(p) * kGramFastTile * kGramFastTile * sizeof(float) : 0;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void gram_kernel(const T* __restrict__ V, const T* __restrict__ Z,
                                                        const int32_t* __restrict__ table, float* __restrict__ partials,
                                                        int64_t Tn, int C, int N, int d, int f, int npairs) {
  typedef Geo<T, kGramTile, kGramTile> G;
  __shared__ __attribute__((aligned(16))) T lds[(G::BM + G::BN) * G::LDK];
  __shared__ float red[kThreads / 64];
  T* lA = lds;
  T* lB = lds + G::BM * G::LDK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // The tile pairs of one chunk share their Z and V_hat rows: consecutive
  // logical ids (same chunk) run on one XCD and meet in its L2.
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int bc = t / npairs, pair = t - bc * npairs;
  int p = 0, rem = pair;
  const int nt = (C + kGramTile - 1) / kGramTile;
  while (rem >= nt - p) { rem -= nt - p; ++p; }
  const int q = p + rem;  // p <= q
  const int b = bc / N, i = bc - b * N;
  const int L = (int)min((int64_t)C, Tn - (int64_t)i * C);
  const int l0 = table[bc * 3 + 1];
  const int s0 = p * kGramTile, t0 = q * kGramTile;
  float part = 0.0f;
  if (s0 < L && t0 < L && s0 + kGramTile > l0 && t0 + kGramTile > l0) {
    const int srows = min(kGramTile, L - s0), trows = min(kGramTile, L - t0);
    const int64_t tok = (int64_t)b * Tn + (int64_t)i * C;
    floatx16 gz[G::MB][G::NB], gv[G::MB][G::NB];
    zero_acc<G>(gz);
    zero_acc<G>(gv);
    // Two contractions with the same tile pair: over d_ff for Z, over d_model for V.
    for (int which = 0; which < 2; ++which) {
      const T* X = which == 0 ? Z : V;
      const int K = which == 0 ? f : d;
      const T* As = X + (tok + s0) * K;
      const T* Bs = X + (tok + t0) * K;
      TileLoad<T, G::BM> la;
      TileLoad<T, G::BN> lb;
      la.load(As, K, srows, 0, K, tid);
      lb.load(Bs, K, trows, 0, K, tid);
      for (int k0 = 0; k0 < K; k0 += G::BK) {
        la.template store<G::LDK>(lA, tid);
        lb.template store<G::LDK>(lB, tid);
        __syncthreads();
        if (k0 + G::BK < K) {
          la.load(As, K, srows, k0 + G::BK, K, tid);
          lb.load(Bs, K, trows, k0 + G::BK, K, tid);
        }
        if (which == 0)
          stage_mma<T, G>(lA, lB, gz, wm, wn, lane);
        else
          stage_mma<T, G>(lA, lB, gv, wm, wn, lane);
        __syncthreads();
      }
    }
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int s = s0 + wm * G::WM + mb * 32 + acc_row(j, lane);
          const int t = t0 + wn * G::WN + nb * 32 + (lane & 31);
          const bool in = s >= l0 && s < L && t >= l0 && t < L;
          part += in ? gz[mb][nb][j] * gv[mb][nb][j] : 0.0f;
        }
    if (p != q) part *= 2.0f;  // the (q, p) tile of both symmetric Grams
  }
  for (int off = 32; off > 0; off >>= 1) part += __shfl_down(part, off, 64);
  if (lane == 0) red[wave] = part;
  __syncthreads();
  if (tid == 0) partials[(int64_t)bc * npairs + pair] = (red[0] + red[1]) + (red[2] + red[3]);
}

// Tile pair (p <= q) number `pair` of nt tiles, in the order (0,0), (0,1),
// .., (0,nt-1), (1,1), ..
__device__ __forceinline__ void gram_pair(int pair, int nt, int& p, int& q) {
  p = 0;
  int rem = pair;
  while (rem >= nt - p) { rem -= nt - p; ++p; }
  q = p + rem;
}

// Gram tiles on the persistent ping-pong core (pingpong.h): tile pair (p, q)
// of a chunk multiplies rows [tok0 + 256p, +256) of X [tokens, ldx] (A)
// against rows [tok0 + 256q, +256) (the two 128-row B operands) over K
// columns [k0, k0 + 64 S); rows at or past the chunk's end L read as zero,
// and a pair on the diagonal loads its rows once.
__device__ __forceinline__ void gram_operands(const bf16* __restrict__ X, int64_t ldx, int64_t tok0, int L, int p,
                                              int q, int k0, core::Operand& oa, core::Operand (&ob)[2]) {
  const int rp = min(kGramFastTile, L - kGramFastTile * p), rq = min(kGramFastTile, L - kGramFastTile * q);
  oa = core::make_operand(X + (tok0 + kGramFastTile * p) * ldx + k0, ldx * 2, (int64_t)rp * ldx * 2 - (int64_t)k0 * 2);
#pragma unroll
  for (int o = 0; o < 2; ++o)
    ob[o] = core::make_operand(X + (tok0 + kGramFastTile * q + pingpong::BN * o) * ldx + k0, ldx * 2,
                               (int64_t)(rq - pingpong::BN * o) * ldx * 2 - (int64_t)k0 * 2);
}

// Element j of block (o, mb, nb) of a lane of a wave of the ping-pong core:
// its index in a stored 256 x 256 fp32 tile (accumulator order, so that the
// 64 lanes of one register write 256 consecutive bytes), and its row and
// column in the tile.
__device__ __forceinline__ int gram_slot(int wave, int o, int mb, int nb, int j, int lane) {
  return ((((wave * 2 + o) * 2 + mb) * 2 + nb) * 16 + j) * 64 + lane;
}

// Whether tile pair (p, q) of a chunk of length L whose carried segment
// starts at l0 holds any token pair of that segment.
__device__ __forceinline__ bool gram_pair_live(int p, int q, int L, int l0) {
  return kGramFastTile * q < L && kGramFastTile * (p + 1) > l0 && kGramFastTile * (q + 1) > l0;
}

// Gv[(bc, pair)] = V V^T of the pair's tiles (fp32, in accumulator order, see
// gram_slot) for the chunks [c0, c0 + n): tiles (chunk, pair), the pairs of
// a chunk next to each other.  Pairs with no token pair of the carried
// segment are not stored (gram_z_fast_kernel skips them).
__global__ __launch_bounds__(512) void gram_v_fast_kernel(const bf16* __restrict__ V, const int32_t* __restrict__ table,
                                                        float* __restrict__ Gv, int64_t Tn, int C, int N, int d, int np,
                                                        int nt, int64_t c0, int n) {
  __shared__ __attribute__((aligned(1024))) bf16 lds[pingpong::LDS_ELEMS];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  auto where = [&](int tt, int64_t& bc, int& p, int& q, int& L, int& l0) {
    bc = c0 + tt / np;
    gram_pair(tt % np, nt, p, q);
    const int64_t i = bc % N;
    L = (int)min((int64_t)C, Tn - i * C);
    l0 = table[bc * 3 + 1];
  };
  auto operands = [&](int tt, core::Operand& oa, core::Operand (&ob)[2], bool& shared, int& S) {
    int64_t bc;
    int p, q, L, l0;
    where(tt, bc, p, q, L, l0);
    const int64_t b = bc / N, i = bc - b * N;
    gram_operands(V, d, b * Tn + i * C, L, p, q, 0, oa, ob);
    shared = p == q;
    S = d / pingpong::KS;
  };
  auto epilogue = [&](int tt, floatx16 (&acc)[2][2][2], bf16*) {
    int64_t bc;
    int p, q, L, l0;
    where(tt, bc, p, q, L, l0);
    if (!gram_pair_live(p, q, L, l0)) return;
    float* g = Gv + (int64_t)tt * (kGramFastTile * kGramFastTile);
#pragma unroll
    for (int o = 0; o < 2; ++o)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int j = 0; j < 16; ++j) g[gram_slot(wave, o, mb, nb, j, lane)] = acc[o][mb][nb][j];
  };
  pingpong::run<true>(lds, n * np, operands, epilogue);
}

// partials[(bc * np + pair) * ks + k] = the masked sum over the pair's tile of
// Gv * (Z Z^T over the k-th of ks ranges of d_ff stages), doubled for p < q
// (the (q, p) tile is the transpose): summed over pairs and ranges, the
// squared norm of V_seg^T Z_seg.  Tiles (chunk, range, pair), so that the
// pairs of one (chunk, range) share Z rows; every slot is written.
__global__ __launch_bounds__(512) void gram_z_fast_kernel(const bf16* __restrict__ Z, const int32_t* __restrict__ table,
                                                        const float* __restrict__ Gv, float* __restrict__ partials,
                                                        int64_t Tn, int C, int N, int f, int np, int nt, int ks,
                                                        int64_t c0, int n) {
  __shared__ __attribute__((aligned(1024))) bf16 lds[pingpong::LDS_ELEMS];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int SF = f / pingpong::KS;
  auto where = [&](int tt, int64_t& bc, int& pair, int& k, int& p, int& q, int& L, int& l0) {
    pair = tt % np;
    k = (tt / np) % ks;
    bc = c0 + tt / (np * ks);
    gram_pair(pair, nt, p, q);
    const int64_t i = bc % N;
    L = (int)min((int64_t)C, Tn - i * C);
    l0 = table[bc * 3 + 1];
  };
  auto operands = [&](int tt, core::Operand& oa, core::Operand (&ob)[2], bool& shared, int& S) {
    int64_t bc;
    int pair, k, p, q, L, l0;
    where(tt, bc, pair, k, p, q, L, l0);
    const int64_t b = bc / N, i = bc - b * N;
    const int s0 = k * SF / ks, s1 = (k + 1) * SF / ks;
    gram_operands(Z, f, b * Tn + i * C, L, p, q, s0 * pingpong::KS, oa, ob);
    shared = p == q;
    S = s1 - s0;
  };
  auto epilogue = [&](int tt, floatx16 (&acc)[2][2][2], bf16* stg) {
    int64_t bc;
    int pair, k, p, q, L, l0;
    where(tt, bc, pair, k, p, q, L, l0);
    float part = 0.0f;
    if (gram_pair_live(p, q, L, l0)) {
      const float* g = Gv + ((bc - c0) * np + pair) * (int64_t)(kGramFastTile * kGramFastTile);
#pragma unroll
      for (int o = 0; o < 2; ++o)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int sr = kGramFastTile * p + wm * 64 + mb * 32 + acc_row(j, lane);
              const int tc = kGramFastTile * q + o * pingpong::BN + wn * 64 + nb * 32 + (lane & 31);
              const bool in = sr >= l0 && sr < L && tc >= l0 && tc < L;
              const float v = g[gram_slot(wave, o, mb, nb, j, lane)];
              part += in ? acc[o][mb][nb][j] * v : 0.0f;
            }
      if (p != q) part *= 2.0f;
    }
    for (int off = 32; off > 0; off >>= 1) part += __shfl_down(part, off, 64);
    float* red = reinterpret_cast<float*>(stg);
    if (lane == 0) red[wave] = part;
    core::lds_barrier();
    if (threadIdx.x == 0)
      partials[(bc * np + pair) * ks + k] =
          ((red[0] + red[1]) + (red[2] + red[3])) + ((red[4] + red[5]) + (red[6] + red[7]));
    core::lds_barrier();
  };
  pingpong::run<true>(lds, n * np * ks, operands, epilogue);
}

__global__ __launch_bounds__(256) void alpha_kernel(const float* __restrict__ partials, float* __restrict__ alpha,
                                                    int nchunks, int npairs, float eta, float tau) {
  const int bc = blockIdx.x * blockDim.x + threadIdx.x;
  if (bc >= nchunks) return;
  double s = 0.0;
  for (int k = 0; k < npairs; ++k) s += (double)partials[(int64_t)bc * npairs + k];
  const double n = fabs((double)eta) * sqrt(fmax(s, 0.0));
  alpha[bc] = (tau > 0.0f && n > (double)tau) ? (float)((double)tau / n) : 1.0f;
}

hipError_t launch_gram_fast(const Prob& p, const void* V, const void* Z, const int32_t* table, float* partials,
                            float* Gv, int64_t c0, int64_t c1, hipStream_t st) {
  const int np = gram_tile_pairs(p), nt = (p.C + kGramFastTile - 1) / kGramFastTile, ks = gram_splits(p);
  const int n = (int)(c1 - c0);
  // one persistent workgroup per CU at most (the tile walk needs a multiple of 8)
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  auto grid = [&](int64_t tiles) {
    return (unsigned)std::min<int64_t>(std::max(8, cus / 8 * 8), (tiles + 7) / 8 * 8);
  };
  note_launch("gram_v", st);
  gram_v_fast_kernel<<<grid((int64_t)n * np), 512, 0, st>>>((const bf16*)V, table, Gv, p.T, p.C, p.N, p.d, np, nt, c0,
                                                           n);
  note_launch("gram", st);
  gram_z_fast_kernel<<<grid((int64_t)n * np * ks), 512, 0, st>>>((const bf16*)Z, table, Gv, partials, p.T, p.C, p.N,
                                                                p.f, np, nt, ks, c0, n);
  return hipGetLastError();
}

hipError_t launch_alpha_only(const Prob& p, const float* partials, float eta, float tau, float* alpha,
                             hipStream_t st) {
  const int nchunks = (int)(p.B * p.N);
  note_launch("alpha", st);
  alpha_kernel<<<(nchunks + 255) / 256, 256, 0, st>>>(partials, alpha, nchunks, tau > 0.0f ? gram_pairs(p) : 0,
                                                      eta, tau);
  return hipGetLastError();
}

hipError_t launch_alpha(const Prob& p, const void* V, const void* Z, const int32_t* table,
                        float eta, float tau, float* alpha, float* partials, void* scratch, hipStream_t st) {
  const int nchunks = (int)(p.B * p.N);
  const int npairs = gram_pairs(p);
  if (tau > 0.0f && fast_scan(p)) {
    const hipError_t e = launch_gram_fast(p, V, Z, table, partials, static_cast<float*>(scratch), 0, p.B * p.N, st);
    if (e != hipSuccess) return e;
  } else if (tau > 0.0f) {
    const int64_t blocks = (int64_t)nchunks * npairs;
    note_launch("gram", st);
    if (p.dtype == 1)
      gram_kernel<bf16><<<(unsigned)blocks, kThreads, 0, st>>>((const bf16*)V, (const bf16*)Z, table, partials,
                                                               p.T, p.C, p.N, p.d, p.f, npairs);
    else
      gram_kernel<float><<<(unsigned)blocks, kThreads, 0, st>>>((const float*)V, (const float*)Z, table,
                                                                partials, p.T, p.C, p.N, p.d, p.f, npairs);
  }
  note_launch("alpha", st);
  alpha_kernel<<<(nchunks + 255) / 256, 256, 0, st>>>(partials, alpha, nchunks, tau > 0.0f ? npairs : 0,
                                                      eta, tau);
  return hipGetLastError();
}

// D += V_hat_seg^T Z_seg for this tile: A rows = d features (V_t), B rows =
// f features (Z_t), K = tokens of the chunk restricted to [l0, L).
template <typename T, class G>
__device__ __forceinline__ void chunk_delta_tile(const T* Vt_rows, const T* Zt_rows, int Cp, int nd, int nf,
                                                 int l0, int L, T* lA, T* lB, floatx16 (&D)[G::MB][G::NB],
                                                 int tid, int wm, int wn, int lane) {
  TileLoad<T, G::BM> la;
  TileLoad<T, G::BN> lb;
  const int kbeg = (l0 / G::BK) * G::BK;
  la.load_kmask(Vt_rows, Cp, nd, kbeg, l0, L, tid);
  lb.load_kmask(Zt_rows, Cp, nf, kbeg, l0, L, tid);
  for (int k0 = kbeg; k0 < L; k0 += G::BK) {
    la.template store<G::LDK>(lA, tid);
    lb.template store<G::LDK>(lB, tid);
    __syncthreads();
    if (k0 + G::BK < L) {
      la.load_kmask(Vt_rows, Cp, nd, k0 + G::BK, l0, L, tid);
      lb.load_kmask(Zt_rows, Cp, nf, k0 + G::BK, l0, L, tid);
    }
    stage_mma<T, G>(lA, lB, D, wm, wn, lane);
    __syncthreads();
  }
}

// CARRY: R holds S alone (started from Sin in a continuing row), each
// emitted weight is W_down + S rounded once, the last chunk's delta is added
// too when Sout is given, and Sout receives the final R.  Otherwise R holds
// W_down + S.  TOUT: the weights are written transposed, [f, d] per chunk
// (the operand layout of the backward's dO W products).
template <typename T, bool CARRY, bool TOUT = false>
__global__ __launch_bounds__(kThreads) void scan_kernel(const T* __restrict__ Zt, const T* __restrict__ Vt,
                                                        const T* __restrict__ Wd, const int32_t* __restrict__ table,
                                                        const float* __restrict__ alpha, float eta,
                                                        T* __restrict__ Wbuf, const float* Sin, float* Sout,
                                                        int64_t Tn, int C, int N, int Cp, int d, int f) {
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

  const int tiles_f = (f + G::BN - 1) / G::BN;
  const int tile = blockIdx.x, b = blockIdx.y;
  const int td = tile / tiles_f, tf = tile - td * tiles_f;
  const int d0 = td * G::BM, f0 = tf * G::BN;
  const int nd = min(G::BM, d - d0), nf = min(G::BN, f - f0);

  // R = W_down + S, or S alone (CARRY), fp32, in the accumulator layout of
  // this wave's block.  src = W_down, Sin or nothing (zeros).
  floatx16 R[G::MB][G::NB];
  auto load_state = [&](int src) {
    const float* Sb = CARRY && Sin != nullptr ? Sin + (int64_t)b * d * f : nullptr;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = wm * G::WM + mb * 32 + acc_row(j, lane);
          const int c = wn * G::WN + nb * 32 + (lane & 31);
          const int64_t e = (int64_t)(d0 + r) * f + f0 + c;
          float v = 0.0f;
          if (r < nd && c < nf) {
            if (src == 0) v = to_f32(Wd[e]);
            else if (src == 1 && Sb != nullptr) v = Sb[e];
          }
          R[mb][nb][j] = v;
        }
  };
  // reset state: W_down, or zero
  const int reset = CARRY ? 2 : 0;
  // A continuing row (its chunk 0 starts no document) starts from Sin.
  load_state(CARRY && table[(b * N) * 3 + 0] > 0 ? 1 : reset);

  for (int i = 0; i < N; ++i) {
    const int bc = b * N + i;
    const int L = (int)min((int64_t)C, Tn - (int64_t)i * C);
    const int r0 = table[bc * 3 + 0], l0 = table[bc * 3 + 1];
    // the last chunk's delta only matters to the carried-out state
    const bool carry = table[bc * 3 + 2] != 0 || (CARRY && i == N - 1 && Sout != nullptr);
    if (r0 > 0) {
      // Effective weight of chunk i (pre-update state): rows [0, r0) apply it.
      T* lC = lds;
#pragma unroll
      for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int r = wm * G::WM + mb * 32 + acc_row(j, lane);
            const int c = wn * G::WN + nb * 32 + (lane & 31);
            float w = R[mb][nb][j];
            if (CARRY && r < nd && c < nf) w += to_f32(Wd[(int64_t)(d0 + r) * f + f0 + c]);
            lC[r * LDC + c] = from_f32<T>(w);
          }
      __syncthreads();
      T* W = Wbuf + (int64_t)bc * d * f;
      if constexpr (TOUT) {
        store_tile_cols<T, G::BM, G::BN, LDC>(lC, W, d, d0, nd, f0, nf, tid);
      } else {
        constexpr int VPR = G::BN / VE;
        for (int v = tid; v < G::BM * VPR; v += kThreads) {
          const int r = v / VPR, cv = (v - r * VPR) * VE;
          if (r < nd && cv < nf)
            *reinterpret_cast<u32x4*>(W + (int64_t)(d0 + r) * f + f0 + cv) =
                *reinterpret_cast<const u32x4*>(lC + r * LDC + cv);
        }
      }
      __syncthreads();
    }
    if (carry && r0 < L) load_state(reset);  // a document starts inside this chunk
    if (carry) {
      floatx16 D[G::MB][G::NB];
      zero_acc<G>(D);
      const T* Va = Vt + ((int64_t)bc * d + d0) * Cp;
      const T* Zb = Zt + ((int64_t)bc * f + f0) * Cp;
      chunk_delta_tile<T, G>(Va, Zb, Cp, nd, nf, l0, L, lA, lB, D, tid, wm, wn, lane);
      const float s = alpha[bc] * eta;
#pragma unroll
      for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
          for (int j = 0; j < 16; ++j) R[mb][nb][j] = fmaf(s, D[mb][nb][j], R[mb][nb][j]);
    }
  }
  if (CARRY && Sout != nullptr) {
    float* So = Sout + (int64_t)b * d * f;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = wm * G::WM + mb * 32 + acc_row(j, lane);
          const int c = wn * G::WN + nb * 32 + (lane & 31);
          if (r < nd && c < nf) So[(int64_t)(d0 + r) * f + f0 + c] = R[mb][nb][j];
        }
  }
}

// Reverse scan of the backward pass.  With P_i = dO_[i][0:r0]^T Z_[i][0:r0],
// the gradient with respect to the state S_i that chunk i applies, the
// adjoints run backwards through the chunks:
//   G_i = P_i + (r0_i == L_i && carry_i ? G_{i+1} : 0),   G_N = 0,
// and the delta of chunk i receives dDW_i = carry_i * G_{i+1}.  One
// workgroup per 128 x 128 tile of the d x f state and per row, walking the
// chunks from the last; G stays in fp32 registers.  dDW_i is written in both
// layouts ([d, f] and [f, d]) for every chunk (zero where it does not carry), and the tile's sum
// of dO^T Z over every token of the row (the W_down gradient of that row) is
// written to Wpart[b].  dOt and Zt are chunk-transposed copies.
template <typename T>
__global__ __launch_bounds__(kThreads) void rscan_kernel(const T* __restrict__ dOt, const T* __restrict__ Zt,
                                                         const int32_t* __restrict__ table, T* __restrict__ dDW,
                                                         T* __restrict__ dDWt, float* __restrict__ Wpart, int64_t Tn,
                                                         int C, int N, int Cp, int d, int f) {
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
  const int tiles_f = (f + G::BN - 1) / G::BN;
  const int tile = blockIdx.x, b = blockIdx.y;
  const int td = tile / tiles_f, tf = tile - td * tiles_f;
  const int d0 = td * G::BM, f0 = tf * G::BN;
  const int nd = min(G::BM, d - d0), nf = min(G::BN, f - f0);

  floatx16 R[G::MB][G::NB], Wacc[G::MB][G::NB], D[G::MB][G::NB];
  zero_acc<G>(R);
  zero_acc<G>(Wacc);
  for (int i = N - 1; i >= 0; --i) {
    const int bc = b * N + i;
    const int L = (int)min((int64_t)C, Tn - (int64_t)i * C);
    const int r0 = table[bc * 3 + 0];
    const bool carry = table[bc * 3 + 2] != 0;
    {
      // every chunk gets its dDW, zero where the chunk does not carry, so
      // that products over all of a chunk's rows read defined values
      T* lC = lds;
#pragma unroll
      for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int r = wm * G::WM + mb * 32 + acc_row(j, lane);
            const int c = wn * G::WN + nb * 32 + (lane & 31);
            lC[r * LDC + c] = from_f32<T>(carry ? R[mb][nb][j] : 0.0f);
          }
      __syncthreads();
      store_tile_rows<T, G::BM, G::BN, LDC>(lC, dDW + (int64_t)bc * d * f, d0, nd, f0, nf, f, tid);
      store_tile_cols<T, G::BM, G::BN, LDC>(lC, dDWt + (int64_t)bc * d * f, d, d0, nd, f0, nf, tid);
      __syncthreads();
    }
    const T* Va = dOt + ((int64_t)bc * d + d0) * Cp;
    const T* Zb = Zt + ((int64_t)bc * f + f0) * Cp;
    // head [0, r0): the tokens that apply S_i
    zero_acc<G>(D);
    if (r0 > 0) chunk_delta_tile<T, G>(Va, Zb, Cp, nd, nf, 0, r0, lA, lB, D, tid, wm, wn, lane);
    const bool keep = r0 == L && carry;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          Wacc[mb][nb][j] += D[mb][nb][j];
          R[mb][nb][j] = keep ? R[mb][nb][j] + D[mb][nb][j] : D[mb][nb][j];
        }
    // tail [r0, L): these tokens apply W_down only
    if (r0 < L) {
      zero_acc<G>(D);
      chunk_delta_tile<T, G>(Va, Zb, Cp, nd, nf, r0, L, lA, lB, D, tid, wm, wn, lane);
#pragma unroll
      for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
          for (int j = 0; j < 16; ++j) Wacc[mb][nb][j] += D[mb][nb][j];
    }
  }
  float* Wp = Wpart + (int64_t)b * d * f;
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = wm * G::WM + mb * 32 + acc_row(j, lane);
        const int c = wn * G::WN + nb * 32 + (lane & 31);
        if (r < nd && c < nf) Wp[(int64_t)(d0 + r) * f + f0 + c] = Wacc[mb][nb][j];
      }
}

hipError_t launch_rscan(const Prob& p, const void* dOt, const void* Zt, const int32_t* table, void* dDW, void* dDWt,
                        float* Wpart, hipStream_t st) {
  note_launch("rscan", st);
  dim3 grid((unsigned)(((p.d + 127) / 128) * ((p.f + 127) / 128)), (unsigned)p.B);
  if (p.dtype == 1)
    rscan_kernel<bf16><<<grid, kThreads, 0, st>>>((const bf16*)dOt, (const bf16*)Zt, table, (bf16*)dDW, (bf16*)dDWt,
                                                  Wpart, p.T, p.C, p.N, p.Cp, p.d, p.f);
  else
    rscan_kernel<float><<<grid, kThreads, 0, st>>>((const float*)dOt, (const float*)Zt, table, (float*)dDW,
                                                   (float*)dDWt, Wpart, p.T, p.C, p.N, p.Cp, p.d, p.f);
  return hipGetLastError();
}

// bf16 fast path (d_model, d_ff multiples of 64).
//
// One workgroup of 8 waves per 256 (f) x 256 (d) tile of the state and per
// row, walking the chunks in order.  Each wave owns a 64 (f) x 128 (d) block
// (2 x 4 MFMA tiles of 32x32) of R = W_down + S in fp32 registers, and the
// MFMAs accumulate straight into it: their V_hat operand comes pre-scaled by
// the chunk's alpha * eta (scale_rows_kernel), so R += (a eta V_hat_seg)^T
// Z_seg needs no separate delta registers.  R's fp32 rounding, about 1e-7
// relative, is far below that of the bf16 weight it emits.
//
// Operands are read in their row layouts, Z [tokens, f] and V_s [tokens, d]:
// stages of 64 tokens go HBM -> LDS with direct-to-LDS buffer loads (row r of
// a stage = token l0 + 64 st + r of the chunk's carried segment; the buffer
// resource ends at the chunk end, so tokens past it read as zero and the
// segment needs no mask), and the MFMA fragments, K = token, come out of LDS
// with transposing reads: ds_read_b64_tr_b16 gives each lane 4 consecutive
// tokens of one feature column, two of them one 32x32x16 operand fragment.
// LDS rows keep their 64-byte units XOR-swizzled by (row & 3), so that the 4
// rows x 64 bytes a half-wave reads fall on distinct banks.
//
// The emitted weight of chunk i (the state before its update) is written
// straight from the R registers, before the chunk's first MFMA, in the
// layout the apply kernel loads as MFMA B fragments: 1 KB fragment
// (d block of 32, f k-step of 16) at ((d/32) * (f/16) + f/16) KB, lane a's 16
// bytes at 16 a holding d = 32 (d/32) + a % 32, f = 16 (f/16) + 8 (a/32) .. +7.
// The accumulator group q (4 rows of f at one d column) of lane l is exactly
// half of such a lane slot, so each 8-byte store of a wave covers 512
// contiguous bytes.
namespace scanrow {
constexpr int kStoreNT = 2;  // buffer store cache policy: non-temporal
constexpr int NT = 512, TF = 256, KS = 64, MB = 2;

// Tile geometry with NB 32-column d blocks per wave: 256 f x 64*NB d.
template <int NB>
struct ScanGeo {
  static constexpr int TD = 2 * NB * 32;
  static constexpr int PZ = TF * 2, PV = TD * 2;                  // LDS row pitch, bytes
  static constexpr int ZB = KS * PZ, VB = KS * PV;
  static constexpr int NIZ = ZB / 1024, NIV = VB / 1024;          // 1 KB load instructions per stage
  static constexpr int NIW = (NIZ + NIV) / 8;                     // per wave
  static constexpr int NIZW = NIZ / 8;                            // of which Z
  static_assert((NIZ % 8) == 0 && (NIV % 8) == 0, "equal load counts per wave");
  static_assert(TF == 4 * MB * 32, "wave grid");
};
// The forward scan's ring: five slots of half a stage (the Z part or the V
// part of a 256 x 256 tile's stage), the whole LDS.
constexpr int SLOT = ScanGeo<4>::ZB, NSLOT = 5, RING_BYTES = NSLOT * SLOT;
static_assert(ScanGeo<4>::VB == SLOT && ScanGeo<2>::ZB == SLOT && RING_BYTES <= 160 * 1024, "half-stage slots");
}  // namespace scanrow

// The state tiles of one row: nbig "big" 256 x 256 tiles covering f-tiles
// [0, nbf) x all d (as many as the CUs run at once), then 256 x 128 tiles
// for the remaining f rows, which fill the next round of CUs.  (380 big
// tiles alone would leave half the CUs idle in their second round.)
struct ScanTiles {
  int nbf, tiles_d;   // big tiles: nbf x tiles_d
  int nbig;           // nbf * tiles_d
  int small_d;        // 128-wide d tiles per f row of the small part
  int total;          // workgroups per row
};

// Vs[t] = alpha[chunk(t)] * eta * V_hat[t], rounded to bf16: the scan's
// pre-scaled operand (8 features per thread).
__global__ __launch_bounds__(256) void scale_rows_kernel(const bf16* __restrict__ V, const float* __restrict__ alpha,
                                                         float eta, bf16* __restrict__ Vs, int64_t M, int64_t Tn,
                                                         int C, int N, int d) {
  const int vpr = d / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= M * vpr) return;
  const int64_t t = idx / vpr;
  const int c = (int)(idx - t * vpr) * 8;
  const int64_t b = t / Tn;
  const int i = (int)((t - b * Tn) / C);
  const float s = alpha[b * N + i] * eta;
  const u32x4 x = *reinterpret_cast<const u32x4*>(V + t * d + c);
  u32x4 y;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float lo = __uint_as_float(x[q] << 16) * s, hi = __uint_as_float(x[q] & 0xFFFF0000u) * s;
    y[q] = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)hi) << 16);
  }
  *reinterpret_cast<u32x4*>(Vs + t * d + c) = y;
}

// Per-lane offsets of a row-layout scan tile (256 f x 64 NB d, see above):
// the byte offsets of this wave's stage loads, relative to the stage's first
// token row (instruction k < NIZW fills Z bytes [1024 q, +1024) of the stage,
// the others bytes of the second operand, q = wave + 8 k), and the LDS byte
// offsets of the transposing fragment reads (k-step 0, first half; k-step kk
// adds 16 rows, the second half 4 rows).  Lane l addresses row 8 (l/32) +
// (l%16)/4 and the 8 bytes 4 (l%4) .. of the 16-column half (l/16)%2 of its
// 32-column block; (row & 3) = (l/4) & 3.
template <int NB>
struct ScanLanes {
  uint32_t voff[scanrow::ScanGeo<NB>::NIW];
  int za[scanrow::MB], va[NB];
  __device__ __forceinline__ ScanLanes(int wave, int lane, int f, int d, int f0, int d0) {
    using namespace scanrow;
    typedef ScanGeo<NB> G;
#pragma unroll
    for (int k = 0; k < G::NIW; ++k) {
      const int q = wave + 8 * k;
      if (k < G::NIZW) {
        const int o = q * 1024 + 16 * lane, r = o / G::PZ, w = o % G::PZ;
        const int u = (w >> 6) ^ (r & 3);
        voff[k] = (uint32_t)r * (uint32_t)(f * 2) + (uint32_t)(f0 * 2 + u * 64 + (w & 63));
      } else {
        const int o = (q - G::NIZ) * 1024 + 16 * lane, r = o / G::PV, w = o % G::PV;
        const int u = (w >> 6) ^ (r & 3);
        voff[k] = (uint32_t)r * (uint32_t)(d * 2) + (uint32_t)(d0 * 2 + u * 64 + (w & 63));
      }
    }
    const int wm = wave >> 1, wn = wave & 1;
    const int sw = (lane >> 2) & 3;
    const int rbase = 8 * (lane >> 5) + ((lane & 15) >> 2);
    const int inu = 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
#pragma unroll
    for (int x = 0; x < MB; ++x) za[x] = rbase * G::PZ + 64 * ((MB * wm + x) ^ sw) + inu;
#pragma unroll
    for (int x = 0; x < NB; ++x) va[x] = G::ZB + rbase * G::PV + 64 * ((NB * wn + x) ^ sw) + inu;
  }
};

// R += Z_stage^T X_stage (K = token) for the stage whose Z part sits in the
// LDS slot at byte sb and X part in the slot at byte vb.  Fragments of
// k-step kk+1 are read while the MFMAs of k-step kk run; the scheduling
// barriers keep the compiler from hoisting every read of the stage (that
// would need more registers than the wave has).  mid() runs once the first
// k-step's MFMAs are issued, so that whatever it does (the scalar work and
// loads of later stages) overlaps the matrix core's work instead of delaying
// the stage's first MFMA.
template <int NB, class Mid>
__device__ __forceinline__ void scan_stage_mma(const ScanLanes<NB>& ln, const char* lds, int sb,
                                               floatx16 (&R)[scanrow::MB][NB], int vb, Mid mid) {
  using namespace scanrow;
  typedef ScanGeo<NB> G;
  typedef __attribute__((address_space(3))) short4_t* lp;
  bf16x8 a[2][MB], v[2][NB];
  auto fetch = [&](int kk, int slot) {
#pragma unroll
    for (int x = 0; x < MB; ++x) {
      const int zo = sb + ln.za[x] + kk * 16 * G::PZ;
      const short4_t z0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(lds + zo));
      const short4_t z1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(lds + zo + 4 * G::PZ));
      a[slot][x] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(z0, z1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int x = 0; x < NB; ++x) {
      const int vo = vb - G::ZB + ln.va[x] + kk * 16 * G::PV;  // va counts from the Z part's start
      const short4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(lds + vo));
      const short4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(lds + vo + 4 * G::PV));
      v[slot][x] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  fetch(0, 0);
#pragma unroll
  for (int kk = 0; kk < KS / 16; ++kk) {
    const int cur = kk & 1;
    if (kk + 1 < KS / 16) fetch(kk + 1, cur ^ 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        R[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][mb], v[cur][nb], R[mb][nb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (kk == 0) {
      mid();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// CARRY: R holds S alone, as in scan_kernel; Sin and Sout point at row b's
// d x f fp32 state (or are NULL).
//
// Chunk window [i0, i1): the tile walks only those chunks and emits their
// weights at Wbuf + (bl * (i1 - i0) + i - i0) * d * f.  A window that starts
// past chunk 0 takes R from Rst (row b's d x f fp32 buffer), and one that ends
// before chunk N stores R there after its last chunk's update, so that a row
// walked in windows computes exactly what one walk over all its chunks does.
template <int NB, bool CARRY>
__device__ __forceinline__ void scan_tile(const bf16* __restrict__ Z, const bf16* __restrict__ Vs,
                                          const bf16* __restrict__ Wd, const int32_t* __restrict__ table,
                                          bf16* __restrict__ Wbuf, bf16* __restrict__ Wdfrag, const float* Sin,
                                          float* Sout, int64_t Tn, int C, int N, int d, int f, int b, int bl,
                                          int f0, int d0, char* lds, int i0, int i1, float* Rst) {
  using namespace scanrow;
  constexpr int NIW = ScanGeo<NB>::NIW, NIZW = ScanGeo<NB>::NIZW, NIZ = ScanGeo<NB>::NIZ;
  // The wave index goes through readfirstlane so that everything derived
  // from it (tile offsets, fragment block addresses) is known wave-uniform
  // and lives in scalar registers.
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  const ScanLanes<NB> ln(wave, lane, f, d, f0, d0);

  floatx16 R[MB][NB];
  // W_down and the emitted weights go through buffer resources of exactly
  // d*f*2 bytes: the blocks of a ragged edge tile get an offset past the end,
  // where loads read zero and stores are dropped, so there is no branch.
  const int wbytes = d * f * 2;
  const __amdgpu_buffer_rsrc_t wd_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(Wd), (short)0, wbytes, 0x00020000);
  auto load_wdown = [&]() {
    // An opaque copy of the lane index keeps the compiler from hoisting the
    // element offsets of this rarely repeated reload out of the chunk loop.
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int fb = f0 + wm * MB * 32 + mb * 32, db = d0 + wn * NB * 32 + nb * 32;
        const bool in = fb < f && db < d;
        const int dc = db + (ln & 31), fr = fb + 4 * (ln >> 5);
        const int off = in ? (dc * f + fr) * 2 : 0x7FFFFFF0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(wd_rsrc, off + 16 * q, 0, 0));
          R[mb][nb][4 * q + 0] = __uint_as_float(w.x << 16);
          R[mb][nb][4 * q + 1] = __uint_as_float(w.x & 0xFFFF0000u);
          R[mb][nb][4 * q + 2] = __uint_as_float(w.y << 16);
          R[mb][nb][4 * q + 3] = __uint_as_float(w.y & 0xFFFF0000u);
        }
        // one block's loads at a time (all at once would need 64 registers)
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  // The fp32 state S (CARRY) through a resource of d*f*4 bytes, the same
  // lane mapping as W_down: 16 bytes = 4 rows of f per accumulator group.
  auto state_io = [&](float* S, bool store) {
    const __amdgpu_buffer_rsrc_t s_rsrc = __builtin_amdgcn_make_buffer_rsrc(S, (short)0, wbytes * 2, 0x00020000);
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int fb = f0 + wm * MB * 32 + mb * 32, db = d0 + wn * NB * 32 + nb * 32;
        const bool in = fb < f && db < d;
        const int off = in ? ((db + (ln & 31)) * f + fb + 4 * (ln >> 5)) * 4 : 0x7FFFFF00;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (store) {
            const float4_t v = {R[mb][nb][4 * q], R[mb][nb][4 * q + 1], R[mb][nb][4 * q + 2], R[mb][nb][4 * q + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), s_rsrc, off + 32 * q, 0, 0);
          } else {
            const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(s_rsrc, off + 32 * q, 0, 0);
            R[mb][nb][4 * q + 0] = __uint_as_float(w[0]);
            R[mb][nb][4 * q + 1] = __uint_as_float(w[1]);
            R[mb][nb][4 * q + 2] = __uint_as_float(w[2]);
            R[mb][nb][4 * q + 3] = __uint_as_float(w[3]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  auto zero_state = [&]() {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) R[mb][nb][j] = 0.0f;
  };
  // bf16(R) (CARRY: bf16(W_down + R)) -> fragment-major weight W: NG stores
  // of 8 bytes per lane, each wave store covering 512 contiguous bytes.
  const int elane = 16 * (lane & 31) + 8 * (lane >> 5);  // lane's bytes in a half fragment
  auto emit = [&](bf16* W) {
    const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(W, (short)0, wbytes, 0x00020000);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int fb = f0 + wm * MB * 32 + mb * 32, db = d0 + wn * NB * 32 + nb * 32;
        const bool in = fb < f && db < d;
        const int blk = in ? ((db >> 5) * (f >> 4) + (fb >> 4)) * 1024 : 0x7FFFF000;
        float wv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) wv[j] = R[mb][nb][j];
        if constexpr (CARRY) {
          const int off = in ? ((db + (lane & 31)) * f + fb + 4 * (lane >> 5)) * 2 : 0x7FFFFFF0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(wd_rsrc, off + 16 * q, 0, 0));
            wv[4 * q + 0] += __uint_as_float(w.x << 16);
            wv[4 * q + 1] += __uint_as_float(w.x & 0xFFFF0000u);
            wv[4 * q + 2] += __uint_as_float(w.y << 16);
            wv[4 * q + 3] += __uint_as_float(w.y & 0xFFFF0000u);
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x2 lo = __builtin_convertvector((float2_t){wv[4 * q], wv[4 * q + 1]}, bf16x2);
          const bf16x2 hi = __builtin_convertvector((float2_t){wv[4 * q + 2], wv[4 * q + 3]}, bf16x2);
          // streaming store (nt): the weight is read back by the apply, much later
          __builtin_amdgcn_raw_buffer_store_b64(
              __builtin_bit_cast(u32x2, (bf16x4){lo[0], lo[1], hi[0], hi[1]}), w_rsrc,
              elane + (q >> 1) * 1024 + (q & 1) * 512, blk, kStoreNT);
        }
      }
  };

  if constexpr (CARRY) {
    zero_state();
    if (b == 0 && i0 == 0) emit(Wdfrag);  // W_down itself, for the tokens after a document start
    if (i0 > 0) {
      state_io(Rst, false);
    } else if (Sin != nullptr && table[(b * N) * 3 + 0] > 0) {
      // A continuing row (its chunk 0 starts no document) starts from Sin.
      state_io(const_cast<float*>(Sin), false);
    }
  } else {
    if (i0 > 0) {
      state_io(Rst, false);
    } else {
      load_wdown();
      if (b == 0) emit(Wdfrag);
    }
  }

  // With a state to hand out, the last chunk's delta is formed as well.
  const bool last_too = CARRY && Sout != nullptr;
  // (table indices through readfirstlane: known wave-uniform, the reads are
  // scalar loads, which do not wait on the vector memory operations in flight)
  auto seg_lo = [&](int i) { return table[__builtin_amdgcn_readfirstlane((b * N + i) * 3 + 1)]; };
  auto len_of = [&](int i) { return (int)min((int64_t)C, Tn - (int64_t)i * C); };
  auto carries = [&](int i) {
    return table[__builtin_amdgcn_readfirstlane((b * N + i) * 3 + 2)] != 0 || (last_too && i == N - 1);
  };
  // A load cursor: the stage `st` of chunk i's carried segment (rows tokens
  // from its start), and the buffer resource over that segment's rows of Z
  // (part 0) or V_s (part 1).  The table is read and the resource built only
  // when the cursor enters a chunk, not at every stage.
  struct Cur {
    int i, st, rows;
    __amdgpu_buffer_rsrc_t rs;
  };
  auto open = [&](Cur& c, int part) {
    const int l0 = seg_lo(c.i);
    c.rows = len_of(c.i) - l0;
    if (part == 0) {
      const int64_t tok = (int64_t)b * Tn + (int64_t)c.i * C + l0;
      c.rs = core::make_operand(Z + tok * f, (int64_t)f * 2, (int64_t)c.rows * f * 2).rsrc;
    } else {
      // V_s holds the window's tokens of each row (all of them without windows)
      const int64_t tokv = (int64_t)bl * Tn + (int64_t)(c.i - i0) * C + l0;
      c.rs = core::make_operand(Vs + tokv * d, (int64_t)d * 2, (int64_t)c.rows * d * 2).rsrc;
    }
  };
  // Next stage in processing order; i = i1: none.
  auto advance = [&](Cur& c, int part) {
    if ((c.st + 1) * KS < c.rows) {
      ++c.st;
      return;
    }
    c.st = 0;
    for (int j = c.i + 1; j < i1; ++j)
      if (carries(j)) {
        c.i = j;
        open(c, part);
        return;
      }
    c.i = i1;
  };
  // The loads of one part of the cursor's stage into the LDS slot at byte `at`.
  auto issue_part = [&](const Cur& c, int part, int at) {
    char* base = lds + at;
    if (part == 0) {
      const int sz = c.st * KS * f * 2;
#pragma unroll
      for (int k = 0; k < NIZW; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rs, (core::lds_ptr_t)(base + (wave + 8 * k) * 1024), 16,
                                                 ln.voff[k], sz, 0, core::kLoadAux);
    } else {
      const int sv = c.st * KS * d * 2;
#pragma unroll
      for (int k = NIZW; k < NIW; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rs, (core::lds_ptr_t)(base + (wave + 8 * k - NIZ) * 1024), 16,
                                                 ln.voff[k], sv, 0, core::kLoadAux);
    }
  };

  // Ring of five half-stage slots: the stages are numbered q = 0, 1, ... in
  // processing order; the Z tile of stage q sits in slot 2q % 5 and its V_s
  // tile in slot (2q + 1) % 5.  While stage q is multiplied, the V_s tile of
  // stage q+1 and the Z tile of stage q+2 are loaded into the slots stage q-1
  // freed (the barrier at the top of stage q ends every read of them), so a
  // Z tile (streamed from HBM) has two stages to arrive and a V_s tile one.
  // `pend` counts this wave's memory operations issued after the V_s tile
  // issued last (the next stage's Z tile, and the stores and W_down loads of
  // a chunk boundary): at the top of stage q at most that many may still be
  // outstanding, which leaves stage q's own tiles complete (vector memory
  // operations retire in issue order).
  constexpr int NBLK = MB * NB;
  auto m5 = [](int x) { return x >= NSLOT ? x - NSLOT : x; };  // x < 10
  Cur cv, cz;
  cv.i = i1;
  cv.st = 0;
  cv.rows = 0;
  cv.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(Z), (short)0, 0, 0x00020000);
  for (int j = i0; j < i1; ++j)
    if (carries(j)) {
      cv.i = j;
      open(cv, 1);
      break;
    }
  cz = cv;
  int pend = 0;
  if (cz.i < i1) {
    open(cz, 0);
    issue_part(cz, 0, 0);
    advance(cz, 0);
    issue_part(cv, 1, SLOT);
    advance(cv, 1);
    if (cz.i < i1) {
      issue_part(cz, 0, 2 * SLOT);
      advance(cz, 0);
      pend = NIZW;
    }
  }

  int h = 0;  // 2q % 5 for the stage q about to be multiplied
  for (int i = i0; i < i1; ++i) {
    const int64_t bc = (int64_t)b * N + i;
    const int L = len_of(i);
    const int r0 = table[bc * 3 + 0], l0 = table[bc * 3 + 1];
    const bool carry = carries(i);
    bf16* W = Wbuf + ((int64_t)bl * (i1 - i0) + i - i0) * d * f;
    // Rows [0, r0) of chunk i apply its effective weight: the state before the
    // chunk's update, written before its first MFMA changes R.
    if (r0 > 0) {
      emit(W);
      pend += CARRY ? 8 * NBLK : 4 * NBLK;
    }
    // A document starts inside the chunk: the carried segment starts from the
    // reset state.
    if (carry && r0 < L) {
      if constexpr (CARRY) {
        zero_state();
      } else {
        load_wdown();
        pend += 4 * NBLK;
      }
    }
    const int nst = carry ? (L - l0 + KS - 1) / KS : 0;
    for (int st = 0; st < nst; ++st) {
      // in the steady state only the Z tile issued last may be outstanding
      if (pend == NIZW)
        core::wait_vmcnt<NIZW>();
      else
        core::wait_vmcnt_at_most(pend);
      core::lds_barrier();
      const int hv = m5(h + 3), hz = m5(h + 4);
      // the loads of later stages go out once this stage's first MFMAs are issued
      auto issue_next = [&]() {
        if (cv.i < i1) {
          issue_part(cv, 1, hv * SLOT);
          advance(cv, 1);
          pend = 0;
        }
        if (cz.i < i1) {
          issue_part(cz, 0, hz * SLOT);
          advance(cz, 0);
          pend += NIZW;
        }
      };
      scan_stage_mma<NB>(ln, lds, h * SLOT, R, m5(h + 1) * SLOT, issue_next);
      h = m5(h + 2);
    }
  }
  if (i1 < N) state_io(Rst, true);
  else if (last_too) state_io(Sout, true);
}

template <bool CARRY>
__global__ __launch_bounds__(512) void scan_fast_kernel(const bf16* __restrict__ Z, const bf16* __restrict__ Vs,
                                                        const bf16* __restrict__ Wd,
                                                        const int32_t* __restrict__ table,
                                                        bf16* __restrict__ Wbuf, bf16* __restrict__ Wdfrag,
                                                        const float* Sin, float* Sout, int64_t Tn, int C, int N,
                                                        int d, int f, ScanTiles st, int row0, int i0, int i1,
                                                        float* Rst) {
  __shared__ __attribute__((aligned(1024))) char lds[scanrow::RING_BYTES];
  // row b of the problem; the pass's per-chunk weights and scaled V_hat
  // start at its first row, row0 (local row bl)
  const int bl = blockIdx.y, b = row0 + bl;
  const int64_t srow = (int64_t)b * d * f;
  const float* sin_b = CARRY && Sin != nullptr ? Sin + srow : nullptr;
  float* sout_b = CARRY && Sout != nullptr ? Sout + srow : nullptr;
  float* rst_b = Rst != nullptr ? Rst + (int64_t)bl * d * f : nullptr;
  // The hardware hands consecutive workgroups to the 8 XCDs in turn.  Each
  // XCD takes an even share of the big tiles first (they fill the first
  // round on every XCD), then its share of the small ones; within each kind
  // its tiles are a contiguous range (big ones in groups of 6 f-tiles, d
  // fastest), so the ~32 workgroups an XCD runs at once share their Z and
  // V_s rows in its L2.
  const int total = st.total, xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  const int bq = st.nbig >> 3, br = st.nbig & 7;
  const int big_share = bq + (xcd < br ? 1 : 0);
  if (idx < big_share) {
    const int tb = xcd * bq + min(xcd, br) + idx;
    int tf, td;
    grouped_tile(tb, st.nbf, st.tiles_d, 6, tf, td);
    scan_tile<4, CARRY>(Z, Vs, Wd, table, Wbuf, Wdfrag, sin_b, sout_b, Tn, C, N, d, f, b, bl, tf * scanrow::TF,
                        td * 256, lds, i0, i1, rst_b);
  } else {
    int u = idx - big_share;  // small tiles of the XCDs before this one come first
    for (int y = 0; y < xcd; ++y) u += (total - y + 7) / 8 - (bq + (y < br ? 1 : 0));
    const int tf = st.nbf + u / st.small_d, td = u % st.small_d;
    scan_tile<2, CARRY>(Z, Vs, Wd, table, Wbuf, Wdfrag, sin_b, sout_b, Tn, C, N, d, f, b, bl, tf * scanrow::TF,
                        td * 128, lds, i0, i1, rst_b);
  }
}

// The reverse scan of the backward (see rscan_kernel) on the 8-wave
// row-layout core of the forward scan: the state adjoint G of one 256 f x
// 64 NB d tile in fp32 registers, the second operand dO in place of V_s.
// Per chunk, walking from the last:
//   emit    dDW_i = carry_i G_{i+1} (fragment-major like the forward's
//           weights; zeros where the chunk does not carry);
//   tail    R += dO_tail^T Z_tail, tokens [r0, L), which apply W_down only;
//   reset   unless r0 == L and carry_i, R (which then holds whole runs of
//           contributions) is added to the row's W_down gradient and zeroed;
//   head    R += dO_head^T Z_head, tokens [0, r0): now R = G_i.
// Every token's dO^T Z reaches the W_down gradient exactly once: the tail
// and the head of a chunk through R, in the flush that ends their run.
// Wpart is this row's fp32 row-major d x f W_down gradient (written, not
// accumulated into).
template <int NB>
__device__ __forceinline__ void rscan_tile(const bf16* __restrict__ Z, const bf16* __restrict__ dO,
                                           const int32_t* __restrict__ table, bf16* __restrict__ dDW,
                                           float* __restrict__ Wpart, int64_t Tn, int C, int N, int d, int f, int b,
                                           int f0, int d0, char* lds) {
  using namespace scanrow;
  constexpr int NIW = ScanGeo<NB>::NIW, NIZW = ScanGeo<NB>::NIZW, NIZ = ScanGeo<NB>::NIZ;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const ScanLanes<NB> ln(wave, lane, f, d, f0, d0);

  floatx16 R[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) R[mb][nb][j] = 0.0f;

  // Ragged edge blocks get offsets past the resources' ends (dropped stores,
  // zero loads), as in scan_tile.
  const int wbytes = d * f * 2;
  const int elane = 16 * (lane & 31) + 8 * (lane >> 5);
  auto emit = [&](bf16* W, bool zero) {
    const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(W, (short)0, wbytes, 0x00020000);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int fb = f0 + wm * MB * 32 + mb * 32, db = d0 + wn * NB * 32 + nb * 32;
        const bool in = fb < f && db < d;
        const int blk = in ? ((db >> 5) * (f >> 4) + (fb >> 4)) * 1024 : 0x7FFFF000;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u32x2 w = {0u, 0u};
          if (!zero) {
            const bf16x2 lo = __builtin_convertvector((float2_t){R[mb][nb][4 * q], R[mb][nb][4 * q + 1]}, bf16x2);
            const bf16x2 hi = __builtin_convertvector((float2_t){R[mb][nb][4 * q + 2], R[mb][nb][4 * q + 3]}, bf16x2);
            w = __builtin_bit_cast(u32x2, (bf16x4){lo[0], lo[1], hi[0], hi[1]});
          }
          __builtin_amdgcn_raw_buffer_store_b64(w, w_rsrc, elane + (q >> 1) * 1024 + (q & 1) * 512, blk, kStoreNT);
        }
      }
  };
  // Wpart[tile] += R, then R = 0.  The first flush stores (Wpart needs no
  // clearing); later ones, one per further document boundary, load, add and
  // store back 16 bytes at a time (each element belongs to this lane alone,
  // so the sum order stays fixed; the stage pipeline's fragment registers
  // are free here and hold the loaded values).
  // A flush with nothing accumulated since the last one is skipped, except
  // the final one of a tile that stored nothing yet (then it stores zeros):
  // a row of one document thus stores its tile once and adds nothing.
  // Returns the memory operations it issued per accumulator block.
  bool first = true, dirty = false;
  const __amdgpu_buffer_rsrc_t p_rsrc = __builtin_amdgcn_make_buffer_rsrc(Wpart, (short)0, wbytes * 2, 0x00020000);
  auto flush = [&](bool last) -> int {
    if (!dirty && !(last && first)) return 0;
    const int ops = first ? 4 : 8;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int fb = f0 + wm * MB * 32 + mb * 32, db = d0 + wn * NB * 32 + nb * 32;
        const bool in = fb < f && db < d;
        const int off = in ? ((db + (lane & 31)) * f + fb + 4 * (lane >> 5)) * 4 : 0x7FFFFF00;
        float4_t old[4] = {};
        if (!first) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            old[q] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(p_rsrc, off + 32 * q, 0, 0));
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4_t v = {old[q][0] + R[mb][nb][4 * q], old[q][1] + R[mb][nb][4 * q + 1],
                              old[q][2] + R[mb][nb][4 * q + 2], old[q][3] + R[mb][nb][4 * q + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), p_rsrc, off + 32 * q, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) R[mb][nb][j] = 0.0f;
      }
    first = false;
    dirty = false;
    return ops;
  };

  // Segments in processing order: s = 2 k + part for chunk i = N - 1 - k,
  // part 0 = the tail [r0, L), part 1 = the head [0, r0).  (Table indices
  // through readfirstlane: known wave-uniform, the reads are scalar loads.)
  auto len_of = [&](int i) { return (int)min((int64_t)C, Tn - (int64_t)i * C); };
  auto seg = [&](int s, int& i, int& lo, int& hi) {
    i = N - 1 - (s >> 1);
    const int r0 = table[__builtin_amdgcn_readfirstlane((b * N + i) * 3 + 0)];
    if (s & 1) { lo = 0; hi = r0; }
    else { lo = r0; hi = len_of(i); }
  };
  // A load cursor, as in scan_tile: stage st of segment s (rows tokens), and
  // the buffer resource over the segment's rows of Z (part 0) or dO (part 1),
  // built only when the cursor enters a segment.
  struct Cur {
    int s, st, rows;
    __amdgpu_buffer_rsrc_t rs;
  };
  auto open = [&](Cur& c, int part) {
    int i, lo, hi;
    seg(c.s, i, lo, hi);
    c.rows = hi - lo;
    const int64_t tok = (int64_t)b * Tn + (int64_t)i * C + lo;
    if (part == 0)
      c.rs = core::make_operand(Z + tok * f, (int64_t)f * 2, (int64_t)c.rows * f * 2).rsrc;
    else
      c.rs = core::make_operand(dO + tok * d, (int64_t)d * 2, (int64_t)c.rows * d * 2).rsrc;
  };
  // Next stage in processing order; s = 2N: none.
  auto advance = [&](Cur& c, int part) {
    if ((c.st + 1) * KS < c.rows) {
      ++c.st;
      return;
    }
    c.st = 0;
    for (int t = c.s + 1; t < 2 * N; ++t) {
      int i, lo, hi;
      seg(t, i, lo, hi);
      if (hi > lo) {
        c.s = t;
        open(c, part);
        return;
      }
    }
    c.s = 2 * N;
  };
  auto issue_part = [&](const Cur& c, int part, int at) {
    char* base = lds + at;
    if (part == 0) {
      const int sz = c.st * KS * f * 2;
#pragma unroll
      for (int k = 0; k < NIZW; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rs, (core::lds_ptr_t)(base + (wave + 8 * k) * 1024), 16,
                                                 ln.voff[k], sz, 0, core::kLoadAux);
    } else {
      const int sv = c.st * KS * d * 2;
#pragma unroll
      for (int k = NIZW; k < NIW; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rs, (core::lds_ptr_t)(base + (wave + 8 * k - NIZ) * 1024), 16,
                                                 ln.voff[k], sv, 0, core::kLoadAux);
    }
  };

  // The forward scan's ring of five half-stage slots (see scan_tile): the Z
  // tile of stage q in slot 2q % 5, its dO tile in slot (2q + 1) % 5; while
  // stage q is multiplied, the dO tile of stage q+1 and the Z tile of stage
  // q+2 go into the slots of stage q-1, issued once the stage's first k-step
  // of MFMAs is under way.  pend counts this wave's memory operations issued
  // after the dO tile issued last; at the top of a stage at most that many may
  // be outstanding (they retire in issue order).
  constexpr int NBLK = MB * NB;
  auto m5 = [](int x) { return x >= NSLOT ? x - NSLOT : x; };  // x < 10
  Cur cv, cz;
  cv.s = 2 * N;
  cv.st = 0;
  cv.rows = 0;
  cv.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(Z), (short)0, 0, 0x00020000);
  for (int t = 0; t < 2 * N; ++t) {
    int i, lo, hi;
    seg(t, i, lo, hi);
    if (hi > lo) {
      cv.s = t;
      open(cv, 1);
      break;
    }
  }
  cz = cv;
  int pend = 0;
  if (cz.s < 2 * N) {
    open(cz, 0);
    issue_part(cz, 0, 0);
    advance(cz, 0);
    issue_part(cv, 1, SLOT);
    advance(cv, 1);
    if (cz.s < 2 * N) {
      issue_part(cz, 0, 2 * SLOT);
      advance(cz, 0);
      pend = NIZW;
    }
  }
  int h = 0;  // 2q % 5 for the stage q about to be multiplied

  // Stages of `rows` tokens, the next ones in processing order.
  auto run_stages = [&](int rows) {
    const int nst = (rows + KS - 1) / KS;
    dirty = dirty || nst > 0;
    for (int st = 0; st < nst; ++st) {
      if (pend == NIZW)
        core::wait_vmcnt<NIZW>();
      else
        core::wait_vmcnt_at_most(pend);
      core::lds_barrier();
      const int hv = m5(h + 3), hz = m5(h + 4);
      auto issue_next = [&]() {
        if (cv.s < 2 * N) {
          issue_part(cv, 1, hv * SLOT);
          advance(cv, 1);
          pend = 0;
        }
        if (cz.s < 2 * N) {
          issue_part(cz, 0, hz * SLOT);
          advance(cz, 0);
          pend += NIZW;
        }
      };
      scan_stage_mma<NB>(ln, lds, h * SLOT, R, m5(h + 1) * SLOT, issue_next);
      h = m5(h + 2);
    }
  };
  for (int i = N - 1; i >= 0; --i) {
    const int64_t bc = (int64_t)b * N + i;
    const int L = len_of(i), r0 = table[bc * 3 + 0];
    const bool carry = table[bc * 3 + 2] != 0;
    emit(dDW + bc * (int64_t)d * f, !carry);
    pend += 4 * NBLK;
    run_stages(L - r0);                                     // tail
    if (!(r0 == L && carry)) pend += flush(false) * NBLK;  // the run ends here
    run_stages(r0);                                         // head
  }
  flush(true);
}

// One row per blockIdx.y; the tile assignment of scan_fast_kernel.
__global__ __launch_bounds__(512) void rscan_fast_kernel(const bf16* __restrict__ Z, const bf16* __restrict__ dO,
                                                         const int32_t* __restrict__ table, bf16* __restrict__ dDW,
                                                         float* __restrict__ Wpart, int64_t Tn, int C, int N, int d,
                                                         int f, ScanTiles st) {
  __shared__ __attribute__((aligned(1024))) char lds[scanrow::RING_BYTES];
  const int b = blockIdx.y;
  float* wp = Wpart + (int64_t)b * d * f;
  const int total = st.total, xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
  const int bq = st.nbig >> 3, br = st.nbig & 7;
  const int big_share = bq + (xcd < br ? 1 : 0);
  if (idx < big_share) {
    const int tb = xcd * bq + min(xcd, br) + idx;
    int tf, td;
    grouped_tile(tb, st.nbf, st.tiles_d, 6, tf, td);
    rscan_tile<4>(Z, dO, table, dDW, wp, Tn, C, N, d, f, b, tf * scanrow::TF, td * 256, lds);
  } else {
    int u = idx - big_share;
    for (int y = 0; y < xcd; ++y) u += (total - y + 7) / 8 - (bq + (y < br ? 1 : 0));
    const int tf = st.nbf + u / st.small_d, td = u % st.small_d;
    rscan_tile<2>(Z, dO, table, dDW, wp, Tn, C, N, d, f, b, tf * scanrow::TF, td * 128, lds);
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void dw_kernel(const T* __restrict__ Vt, const T* __restrict__ Zt,
                                                      const int32_t* __restrict__ table, const float* __restrict__ alpha,
                                                      float eta, float* __restrict__ dW, int64_t Tn, int C, int N,
                                                      int Cp, int d, int f) {
  typedef Geo<T, 128, 128> G;
  __shared__ __attribute__((aligned(16))) T lds[(G::BM + G::BN) * G::LDK];
  T* lA = lds;
  T* lB = lds + G::BM * G::LDK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_f = (f + G::BN - 1) / G::BN;
  const int tile = blockIdx.x, bc = blockIdx.y;
  const int td = tile / tiles_f, tf = tile - td * tiles_f;
  const int d0 = td * G::BM, f0 = tf * G::BN;
  const int nd = min(G::BM, d - d0), nf = min(G::BN, f - f0);
  const int i = bc % N;
  const int L = (int)min((int64_t)C, Tn - (int64_t)i * C);
  const int l0 = table[bc * 3 + 1];
  floatx16 D[G::MB][G::NB];
  zero_acc<G>(D);
  chunk_delta_tile<T, G>(Vt + ((int64_t)bc * d + d0) * Cp, Zt + ((int64_t)bc * f + f0) * Cp, Cp, nd, nf, l0, L,
                         lA, lB, D, tid, wm, wn, lane);
  const float s = alpha[bc] * eta;
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = wm * G::WM + mb * 32 + acc_row(j, lane);
        const int c = wn * G::WN + nb * 32 + (lane & 31);
        if (r < nd && c < nf) dW[((int64_t)bc * d + d0 + r) * f + f0 + c] = s * D[mb][nb][j];
      }
}

hipError_t launch_dw(const Prob& p, const void* Vt, const void* Zt, const int32_t* table,
                     const float* alpha, float eta, float* dW, hipStream_t st) {
  note_launch("dw", st);
  dim3 grid((unsigned)(((p.d + 127) / 128) * ((p.f + 127) / 128)), (unsigned)(p.B * p.N));
  if (p.dtype == 1)
    dw_kernel<bf16><<<grid, kThreads, 0, st>>>((const bf16*)Vt, (const bf16*)Zt, table, alpha, eta, dW, p.T,
                                               p.C, p.N, p.Cp, p.d, p.f);
  else
    dw_kernel<float><<<grid, kThreads, 0, st>>>((const float*)Vt, (const float*)Zt, table, alpha, eta, dW, p.T,
                                                p.C, p.N, p.Cp, p.d, p.f);
  return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(256) void chunk_transpose_kernel(const T* __restrict__ in, T* __restrict__ out, int64_t Tn,
                                                              int C, int N, int Cp, int F, int ftiles, int ctiles) {
  __shared__ T tile[32][33];
  const int64_t blk = blockIdx.x;
  const int ft = (int)(blk % ftiles);
  const int64_t rest = blk / ftiles;
  const int ct = (int)(rest % ctiles);
  const int64_t bc = rest / ctiles;
  const int b = (int)(bc / N), i = (int)(bc - (int64_t)b * N);
  const int L = (int)min((int64_t)C, Tn - (int64_t)i * C);
  const int j0 = ft * 32, c0 = ct * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t tok0 = (int64_t)b * Tn + (int64_t)i * C;
  for (int y = ty; y < 32; y += 8) {
    const int c = c0 + y, j = j0 + tx;
    if (c < L && j < F) tile[y][tx] = in[(tok0 + c) * F + j];
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    const int j = j0 + y, c = c0 + tx;
    if (c < L && j < F) out[(bc * F + j) * Cp + c] = tile[tx][y];
  }
}

hipError_t launch_chunk_transpose(const Prob& p, const void* in, int F, void* out, hipStream_t st) {
  note_launch("chunk_transpose", st);
  const int ftiles = (F + 31) / 32, ctiles = (p.C + 31) / 32;
  const int64_t blocks = p.B * p.N * (int64_t)ctiles * ftiles;
  if (p.dtype == 1)
    chunk_transpose_kernel<bf16><<<(unsigned)blocks, 256, 0, st>>>((const bf16*)in, (bf16*)out, p.T, p.C, p.N, p.Cp, F,
                                                                   ftiles, ctiles);
  else
    chunk_transpose_kernel<float><<<(unsigned)blocks, 256, 0, st>>>((const float*)in, (float*)out, p.T, p.C, p.N, p.Cp,
                                                                    F, ftiles, ctiles);
  return hipGetLastError();
}

// Token-axis products on the row-layout core: C_p[m, n] = sum_t A_p[t, m]
// B_p[t, n] over all M tokens, for up to two products p = blockIdx.y that
// share their shapes (the weight gradients dW_gate = dG^T H and dW_up =
// dU^T H, or dW_target = Y^T dV).  One 256 x 256 output tile per workgroup,
// in fp32 registers; the tokens stream through in 64-token stages, the
// operands re-based every kTnBlock tokens so that the buffer offsets stay
// 32-bit.  A, B and C are row-major ([M, ma], [M, nb], [ma, nb]); ma and nb
// multiples of 64.  With gridDim.z > 1 the tokens are split into slices of
// `per`, and slice z writes its partial product to C_p + z * ma * nb.
constexpr int kTnBlock = 16384;

// The operands come in as restrict parameters of this inlined tile function:
// the compiler then tells the tile's LDS reads apart from its direct-to-LDS
// operand loads and inserts no wait for those loads before the reads (the
// kernel's own stage waits order them).
__device__ __forceinline__ void tn_tile(const bf16* __restrict__ A, const bf16* __restrict__ B,
                                        float* __restrict__ Cp, int64_t M, int ma, int nb, char* lds) {
  using namespace scanrow;
  constexpr int NB = 4;
  typedef ScanGeo<NB> G;
  constexpr int NIW = G::NIW, NIZW = G::NIZW, NIZ = G::NIZ;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_n = (nb + 255) / 256;
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int m0 = (t / tiles_n) * TF, n0 = (t % tiles_n) * 256;
  const ScanLanes<NB> ln(wave, lane, ma, nb, m0, n0);
  floatx16 R[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int x = 0; x < NB; ++x)
#pragma unroll
      for (int j = 0; j < 16; ++j) R[mb][x][j] = 0.0f;

  const int64_t nblk = (M + kTnBlock - 1) / kTnBlock;
  auto rows_of = [&](int64_t blk) { return (int)min((int64_t)kTnBlock, M - blk * kTnBlock); };
  // Load cursors as in scan_tile: stage st of token block blk, and the
  // buffer resource over that block's rows of A (part 0) or B (part 1),
  // built once per block.
  struct Cur {
    int64_t blk;
    int st;
    __amdgpu_buffer_rsrc_t rs;
  };
  auto open = [&](Cur& c, int part) {
    const int64_t tok = c.blk * kTnBlock;
    const int rows = rows_of(c.blk);
    if (part == 0)
      c.rs = core::make_operand(A + tok * ma, (int64_t)ma * 2, (int64_t)rows * ma * 2).rsrc;
    else
      c.rs = core::make_operand(B + tok * nb, (int64_t)nb * 2, (int64_t)rows * nb * 2).rsrc;
  };
  auto advance = [&](Cur& c, int part) {
    if ((c.st + 1) * KS < rows_of(c.blk)) {
      ++c.st;
      return;
    }
    c.st = 0;
    if (++c.blk < nblk) open(c, part);
  };
  auto issue_part = [&](const Cur& c, int part, int at) {
    char* base = lds + at;
    if (part == 0) {
      const int sz = c.st * KS * ma * 2;
#pragma unroll
      for (int k = 0; k < NIZW; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rs, (core::lds_ptr_t)(base + (wave + 8 * k) * 1024), 16,
                                                 ln.voff[k], sz, 0, core::kLoadAux);
    } else {
      const int sv = c.st * KS * nb * 2;
#pragma unroll
      for (int k = NIZW; k < NIW; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rs, (core::lds_ptr_t)(base + (wave + 8 * k - NIZ) * 1024), 16,
                                                 ln.voff[k], sv, 0, core::kLoadAux);
    }
  };
  // The forward scan's ring of five half-stage slots (see scan_tile): A
  // tiles two stages ahead, B tiles one, issued once a stage's first k-step
  // of MFMAs is under way; pend counts this wave's loads issued after the B
  // tile issued last.
  auto m5 = [](int x) { return x >= NSLOT ? x - NSLOT : x; };  // x < 10
  Cur cv;
  cv.blk = 0;
  cv.st = 0;
  open(cv, 1);
  Cur cz = cv;
  open(cz, 0);
  issue_part(cz, 0, 0);
  advance(cz, 0);
  issue_part(cv, 1, SLOT);
  advance(cv, 1);
  int pend = 0;
  if (cz.blk < nblk) {
    issue_part(cz, 0, 2 * SLOT);
    advance(cz, 0);
    pend = NIZW;
  }
  int h = 0;  // 2q % 5 for the stage q about to be multiplied
  for (int64_t blk = 0; blk < nblk; ++blk) {
    const int nst = (rows_of(blk) + KS - 1) / KS;
    for (int st = 0; st < nst; ++st) {
      if (pend == NIZW)
        core::wait_vmcnt<NIZW>();
      else
        core::wait_vmcnt_at_most(pend);
      core::lds_barrier();
      const int hv = m5(h + 3), hz = m5(h + 4);
      auto issue_next = [&]() {
        if (cv.blk < nblk) {
          issue_part(cv, 1, hv * SLOT);
          advance(cv, 1);
          pend = 0;
        }
        if (cz.blk < nblk) {
          issue_part(cz, 0, hz * SLOT);
          advance(cz, 0);
          pend += NIZW;
        }
      };
      scan_stage_mma<NB>(ln, lds, h * SLOT, R, m5(h + 1) * SLOT, issue_next);
      h = m5(h + 2);
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int x = 0; x < NB; ++x)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = m0 + wm * MB * 32 + mb * 32 + acc_row(j, lane);
        const int c = n0 + wn * NB * 32 + x * 32 + (lane & 31);
        if (r < ma && c < nb) Cp[(int64_t)r * nb + c] = R[mb][x][j];
      }
}

__global__ __launch_bounds__(512) void tn_fast_kernel(const bf16* A0, const bf16* A1, const bf16* B0, const bf16* B1,
                                                      float* C0, float* C1, int64_t Mall, int64_t per, int ma, int nb) {
  __shared__ __attribute__((aligned(1024))) char lds[scanrow::RING_BYTES];
  const int p = blockIdx.y;
  const int64_t tb = (int64_t)blockIdx.z * per;
  tn_tile((p ? A1 : A0) + tb * ma, (p ? B1 : B0) + tb * nb, (p ? C1 : C0) + (int64_t)blockIdx.z * ma * nb,
          min(per, Mall - tb), ma, nb, lds);
}

hipError_t launch_tn_fast(int nprod, const void* const* A, const void* const* B, float* const* C, int64_t M,
                          int ma, int nb, int splits, hipStream_t st) {
  note_launch("tn_fast", st);
  const int k1 = nprod > 1 ? 1 : 0;
  const int tiles = ((ma + scanrow::TF - 1) / scanrow::TF) * ((nb + 255) / 256);
  const int64_t per = (M + splits - 1) / splits;
  // every slice holds at least one token
  if (splits < 1 || (int64_t)(splits - 1) * per >= M) return hipErrorInvalidValue;
  dim3 g((unsigned)tiles, (unsigned)nprod, (unsigned)splits);
  tn_fast_kernel<<<g, scanrow::NT, 0, st>>>((const bf16*)A[0], (const bf16*)A[k1], (const bf16*)B[0],
                                            (const bf16*)B[k1], C[0], C[k1], M, per, ma, nb);
  return hipGetLastError();
}

int tn_fast_splits(int nprod, int64_t M, int ma, int nb, int cap) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t tiles = (int64_t)nprod * ((ma + scanrow::TF - 1) / scanrow::TF) * ((nb + 255) / 256);
  int best = 1;
  double bt = 1e300;
  for (int s = 1; s <= 8 && s <= cap; ++s) {
    if (s > 1 && M / s < 1024) break;
    // rounds of one workgroup per CU, each slice 1/s of the tokens
    const double t = (double)((tiles * s + cus - 1) / cus) / s;
    if (t < bt * 0.999) bt = t, best = s;
  }
  return best;
}

// The state tiles of one row for the device's CU count (see ScanTiles).
// The tile plan of the forward and reverse scans: as many 256 x 256 tiles as
// there are CUs, the rest of the f rows as 256 x 128 tiles.  IPTTT_SCAN_CUS (a
// positive integer, read at each call) replaces the device's CU count, so
// that small problems can run on the 256 x 128 tiles too; every state element
// is accumulated in the same order on both kinds, so the results are the same.
static int scan_plan_cus() {
  if (const char* e = std::getenv("IPTTT_SCAN_CUS")) {
    char* end = nullptr;
    const long v = std::strtol(e, &end, 10);
    if (end != e && *end == '\0' && v > 0 && v <= (1 << 20)) return (int)v;
  }
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return cus;
}

static ScanTiles scan_tiles(const Prob& p) {
  ScanTiles tl;
  const int cus = scan_plan_cus();
  const int tiles_f = (p.f + scanrow::TF - 1) / scanrow::TF;
  tl.tiles_d = (p.d + 255) / 256;
  tl.nbf = std::min(tiles_f, std::max(1, cus / tl.tiles_d));
  tl.nbig = tl.nbf * tl.tiles_d;
  tl.small_d = (p.d + 127) / 128;
  tl.total = tl.nbig + (tiles_f - tl.nbf) * tl.small_d;
  return tl;
}

hipError_t launch_rscan_fast(const Prob& p, const void* Z, const void* dO, const int32_t* table, void* dDW,
                             float* Wpart, hipStream_t st) {
  note_launch("rscan_fast", st);
  const ScanTiles tl = scan_tiles(p);
  dim3 g((unsigned)tl.total, (unsigned)p.B);
  rscan_fast_kernel<<<g, scanrow::NT, 0, st>>>((const bf16*)Z, (const bf16*)dO, table, (bf16*)dDW, Wpart, p.T, p.C,
                                               p.N, p.d, p.f, tl);
  return hipGetLastError();
}

hipError_t launch_scan_transposed(const Prob& p, const void* Zt, const void* Vt, const void* Wd,
                                  const int32_t* table, const float* alpha, float eta, void* WbufT, hipStream_t st) {
  note_launch("scan_transposed", st);
  dim3 grid((unsigned)(((p.d + 127) / 128) * ((p.f + 127) / 128)), (unsigned)p.B);
  if (p.dtype == 1)
    scan_kernel<bf16, false, true><<<grid, kThreads, 0, st>>>((const bf16*)Zt, (const bf16*)Vt, (const bf16*)Wd,
                                                              table, alpha, eta, (bf16*)WbufT, nullptr, nullptr, p.T,
                                                              p.C, p.N, p.Cp, p.d, p.f);
  else
    scan_kernel<float, false, true><<<grid, kThreads, 0, st>>>((const float*)Zt, (const float*)Vt, (const float*)Wd,
                                                               table, alpha, eta, (float*)WbufT, nullptr, nullptr,
                                                               p.T, p.C, p.N, p.Cp, p.d, p.f);
  return hipGetLastError();
}

hipError_t launch_scan(const Prob& p, const void* Z, const void* V, const void* Zt, const void* Vt,
                       const void* Wd, const int32_t* table, const float* alpha, float eta, void* Wbuf,
                       void* Wdfrag, void* Vs, bool carry, const float* Sin, float* Sout, hipStream_t st, int row0,
                       int nrows, int i0, int i1, float* Rst) {
  if (fast_scan(p)) {
    const int nb = nrows < 0 ? (int)p.B : nrows;
    if (i1 < 0) i1 = (int)p.N;
    const bool win = i0 > 0 || i1 < p.N;
    if (i0 < 0 || i0 >= i1 || i1 > p.N || (win && (Rst == nullptr || nb != 1))) return hipErrorInvalidValue;
    // the pass's scaled V_hat: each row's tokens, or a window's tokens of its
    // one row
    const int64_t t0 = (int64_t)i0 * p.C, wt = win ? std::min<int64_t>((int64_t)i1 * p.C, p.T) - t0 : p.T;
    const int64_t nv = (int64_t)nb * wt * (p.d / 8);
    note_launch("scale_rows", st);
    scale_rows_kernel<<<(unsigned)((nv + 255) / 256), 256, 0, st>>>(
        (const bf16*)V + ((int64_t)row0 * p.T + t0) * p.d, alpha + (int64_t)row0 * p.N + i0, eta, (bf16*)Vs,
        (int64_t)nb * wt, wt, p.C, p.N, p.d);
    const ScanTiles tl = scan_tiles(p);
    dim3 g((unsigned)tl.total, (unsigned)nb);
    note_launch("scan", st);
    if (carry)
      scan_fast_kernel<true><<<g, scanrow::NT, 0, st>>>((const bf16*)Z, (const bf16*)Vs, (const bf16*)Wd, table,
                                                        (bf16*)Wbuf, (bf16*)Wdfrag, Sin, Sout, p.T, p.C, p.N, p.d,
                                                        p.f, tl, row0, i0, i1, Rst);
    else
      scan_fast_kernel<false><<<g, scanrow::NT, 0, st>>>((const bf16*)Z, (const bf16*)Vs, (const bf16*)Wd, table,
                                                         (bf16*)Wbuf, (bf16*)Wdfrag, nullptr, nullptr, p.T, p.C,
                                                         p.N, p.d, p.f, tl, row0, i0, i1, Rst);
    return hipGetLastError();
  }
  if (row0 != 0 || (nrows >= 0 && nrows != p.B) || i0 != 0 || (i1 >= 0 && i1 != p.N)) return hipErrorInvalidValue;
  dim3 grid((unsigned)(((p.d + 127) / 128) * ((p.f + 127) / 128)), (unsigned)p.B);
  note_launch("scan", st);
  if (p.dtype == 1) {
    if (carry)
      scan_kernel<bf16, true><<<grid, kThreads, 0, st>>>((const bf16*)Zt, (const bf16*)Vt, (const bf16*)Wd, table,
                                                         alpha, eta, (bf16*)Wbuf, Sin, Sout, p.T, p.C, p.N, p.Cp,
                                                         p.d, p.f);
    else
      scan_kernel<bf16, false><<<grid, kThreads, 0, st>>>((const bf16*)Zt, (const bf16*)Vt, (const bf16*)Wd, table,
                                                          alpha, eta, (bf16*)Wbuf, nullptr, nullptr, p.T, p.C, p.N,
                                                          p.Cp, p.d, p.f);
  } else {
    if (carry)
      scan_kernel<float, true><<<grid, kThreads, 0, st>>>((const float*)Zt, (const float*)Vt, (const float*)Wd,
                                                          table, alpha, eta, (float*)Wbuf, Sin, Sout, p.T, p.C, p.N,
                                                          p.Cp, p.d, p.f);
    else
      scan_kernel<float, false><<<grid, kThreads, 0, st>>>((const float*)Zt, (const float*)Vt, (const float*)Wd,
                                                           table, alpha, eta, (float*)Wbuf, nullptr, nullptr, p.T,
                                                           p.C, p.N, p.Cp, p.d, p.f);
  }
  return hipGetLastError();
}

}  // namespace ipttt
