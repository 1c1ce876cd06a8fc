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
#include "launch.h"
#include "common.h"
#include "mfma_core.h"
#include "epilogue.h"

namespace ipttt {

constexpr int kGramTile = 128;

int gram_pairs(const Prob& p) {
  const int nt = (p.C + kGramTile - 1) / kGramTile;
  return nt * (nt + 1) / 2;
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

  const int bc = blockIdx.x / npairs, pair = blockIdx.x - bc * npairs;
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

__global__ __launch_bounds__(256) void alpha_kernel(const float* __restrict__ partials, float* __restrict__ alpha,
                                                    int nchunks, int npairs, float eta, float tau) {
  const int bc = blockIdx.x * blockDim.x + threadIdx.x;
  if (bc >= nchunks) return;
  double s = 0.0;
  for (int k = 0; k < npairs; ++k) s += (double)partials[(int64_t)bc * npairs + k];
  const double n = fabs((double)eta) * sqrt(fmax(s, 0.0));
  alpha[bc] = (tau > 0.0f && n > (double)tau) ? (float)((double)tau / n) : 1.0f;
}

hipError_t launch_alpha(const Prob& p, const void* V, const void* Z, const int32_t* table,
                        float eta, float tau, float* alpha, float* partials, hipStream_t st) {
  const int nchunks = (int)(p.B * p.N);
  const int npairs = gram_pairs(p);
  if (tau > 0.0f) {
    const int64_t blocks = (int64_t)nchunks * npairs;
    if (p.dtype == 1)
      gram_kernel<bf16><<<(unsigned)blocks, kThreads, 0, st>>>((const bf16*)V, (const bf16*)Z, table, partials,
                                                               p.T, p.C, p.N, p.d, p.f, npairs);
    else
      gram_kernel<float><<<(unsigned)blocks, kThreads, 0, st>>>((const float*)V, (const float*)Z, table,
                                                                partials, p.T, p.C, p.N, p.d, p.f, npairs);
  }
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

template <typename T>
__global__ __launch_bounds__(kThreads) void scan_kernel(const T* __restrict__ Zt, const T* __restrict__ Vt,
                                                        const T* __restrict__ Wd, const int32_t* __restrict__ table,
                                                        const float* __restrict__ alpha, float eta,
                                                        T* __restrict__ Wbuf, int64_t Tn, int C, int N, int Cp,
                                                        int d, int f) {
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

  // R = W_down + S (fp32), in the accumulator layout of this wave's block.
  floatx16 R[G::MB][G::NB];
  auto load_wdown = [&]() {
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = wm * G::WM + mb * 32 + acc_row(j, lane);
          const int c = wn * G::WN + nb * 32 + (lane & 31);
          R[mb][nb][j] = (r < nd && c < nf) ? to_f32(Wd[(int64_t)(d0 + r) * f + f0 + c]) : 0.0f;
        }
  };
  load_wdown();

  for (int i = 0; i < N; ++i) {
    const int bc = b * N + i;
    const int L = (int)min((int64_t)C, Tn - (int64_t)i * C);
    const int r0 = table[bc * 3 + 0], l0 = table[bc * 3 + 1], carry = table[bc * 3 + 2];
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
            lC[r * LDC + c] = from_f32<T>(R[mb][nb][j]);
          }
      __syncthreads();
      T* W = Wbuf + (int64_t)bc * d * f;
      constexpr int VPR = G::BN / VE;
      for (int v = tid; v < G::BM * VPR; v += kThreads) {
        const int r = v / VPR, cv = (v - r * VPR) * VE;
        if (r < nd && cv < nf)
          *reinterpret_cast<u32x4*>(W + (int64_t)(d0 + r) * f + f0 + cv) =
              *reinterpret_cast<const u32x4*>(lC + r * LDC + cv);
      }
      __syncthreads();
    }
    if (r0 < L) load_wdown();  // a document starts inside this chunk
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
}

// bf16 fast path (d_model, d_ff multiples of 64).  One workgroup of 8 waves
// per 256 (d) x 128 (f) tile of the state and per row; wave w owns d rows
// 64*(w/2).. and f columns 64*(w%2).. (2 x 2 blocks of 32x32).  Registers hold
// R = W_down + S (fp32; its rounding, about 1e-7 relative, is far below that
// of the bf16 weight it emits) and the chunk's delta D.  A document start
// reloads R from W_down.
//
// Token stages run back to back across chunks with the later stages' loads in
// flight; partial stages (a document start inside the chunk, a short
// last chunk) have the out-of-segment tokens zeroed in LDS before their MFMAs.
// The waves split the memory work: waves 0-3 issue every operand load, so
// their vector-memory counter only ever holds loads; waves 4-7 stream the
// chunk's effective weight (staged once per chunk in LDS as bf16) to memory
// in 16-byte stores spread over the chunk's stages and never wait for them.
// Each SIMD runs one wave of each kind.
__global__ __launch_bounds__(512) void scan_fast_kernel(const bf16* __restrict__ Zt, const bf16* __restrict__ Vt,
                                                        const bf16* __restrict__ Wd,
                                                        const int32_t* __restrict__ table,
                                                        const float* __restrict__ alpha, float eta,
                                                        bf16* __restrict__ Wbuf, int64_t Tn, int C, int N, int Cp,
                                                        int d, int f) {
  // Token stages of 64 (128-byte LDS rows) in a ring of NBUF buffers: up to
  // NBUF - 1 stages' loads are in flight while one is multiplied (the ring
  // also works with 4 buffers of 32 tokens, which measured no faster).
  constexpr int NT = 512, BM = 256, BN = 128, KS = 64, ROWB = 128, NBUF = 2;
  constexpr int SA = BM * KS, SB = BN * KS, STAGE = SA + SB;
  constexpr int NLW = 4;                                      // loading waves
  constexpr int RPI = 1024 / ROWB;                            // rows per load instruction
  constexpr int NA = BM / (NLW * RPI), NBI = BN / (NLW * RPI), NLOAD = NA + NBI;
  constexpr int KSTEPS = ROWB / 32;
  __shared__ __attribute__((aligned(1024))) bf16 lds[NBUF * STAGE + BM * BN];
  bf16* stg = lds + NBUF * STAGE;  // [BM][BN] bf16 copy of the chunk's effective weight
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const bool loader = wave < NLW;
  const int tiles_f = (f + BN - 1) / BN, tiles_d = (d + BM - 1) / BM;
  const int b = blockIdx.y;
  // Each XCD walks a contiguous range of tiles in groups of 5 d-tiles, so the
  // ~32 workgroups it runs at once share their V_t and Z_t slices in its L2.
  int td, tf;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), tiles_d, tiles_f, 5, td, tf);
  const int d0 = td * BM, f0 = tf * BN;
  const int nd = min(BM, d - d0), nf = min(BN, f - f0);

  floatx16 R[1][2][2], D[1][2][2];
  auto load_wdown = [&]() {
    // An opaque copy of the lane index keeps the compiler from hoisting the 64
    // element addresses of this (rarely repeated) reload out of the chunk loop,
    // where they would stay live and spill.
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int rb = wm * 64 + mb * 32 + 4 * (ln >> 5);
        const int c = wn * 64 + nb * 32 + (ln & 31);
        const bf16* base = Wd + (int64_t)(d0 + rb) * f + f0 + c;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int ro = ((j >> 2) << 3) + (j & 3);  // row of element j relative to rb
          R[0][mb][nb][j] = (rb + ro < nd && c < nf) ? (float)base[(int64_t)ro * f] : 0.0f;
        }
      }
  };
  load_wdown();

  auto kbeg_of = [&](int i) { return (table[(b * N + i) * 3 + 1] / KS) * KS; };
  auto len_of = [&](int i) { return (int)min((int64_t)C, Tn - (int64_t)i * C); };
  // Advance (i, k0) to the next stage in processing order (i = N: none).
  auto advance = [&](int& i, int& k0) {
    if (k0 + KS < len_of(i)) { k0 += KS; return; }
    for (int j = i + 1; j < N; ++j)
      if (table[(b * N + j) * 3 + 2]) { i = j; k0 = kbeg_of(j); return; }
    i = N;
    k0 = 0;
  };
  auto issue = [&](int i, int k0, bf16* buf, int q0, int q1) {
    const int64_t bc = (int64_t)b * N + i;
    const core::Operand oa = core::make_operand(Vt + (bc * d + d0) * Cp, (int64_t)Cp * 2, (int64_t)nd * Cp * 2);
    const core::Operand ob = core::make_operand(Zt + (bc * f + f0) * Cp, (int64_t)Cp * 2, (int64_t)nf * Cp * 2);
#pragma unroll
    for (int q = 0; q < NLOAD; ++q) {
      if (q < q0 || q >= q1) continue;
      if (q < NA) core::load_tile_part<BM, ROWB, NLW>(oa, k0, buf, wave, lane, q, 1);
      else core::load_tile_part<BN, ROWB, NLW>(ob, k0, buf + SA, wave, lane, q - NA, 1);
    }
  };
  // Store rows [r0, r1) of the staged weight (the storing waves' share).
  auto emit_rows = [&](bf16* W, int r0, int r1) {
    const int st = tid - NLW * 64;
    for (int v = st; v < (r1 - r0) * (BN / 8); v += NT - NLW * 64) {
      const int r = r0 + v / (BN / 8), c = (v % (BN / 8)) * 8;
      if (r < nd && c < nf)  // streaming store: the weight is read back much later, by the apply
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(stg + r * BN + c),
                                    reinterpret_cast<u32x4*>(W + (int64_t)(d0 + r) * f + f0 + c));
    }
  };

  // Ring of issued stages: buffers cbuf .. cbuf+ahead-1 (mod NBUF) hold them;
  // (fi, fk) is the next stage to issue.
  int cbuf = 0, ahead = 0, fi = N, fk = 0;
  for (int j = 0; j < N; ++j)
    if (table[(b * N + j) * 3 + 2]) { fi = j; fk = kbeg_of(j); break; }
  for (int a = 0; a < NBUF - 1 && fi < N; ++a) {
    if (loader) issue(fi, fk, lds + ((cbuf + ahead) % NBUF) * STAGE, 0, NLOAD);
    ++ahead;
    advance(fi, fk);
  }

  for (int i = 0; i < N; ++i) {
    const int64_t bc = (int64_t)b * N + i;
    const int L = len_of(i);
    const int r0 = table[bc * 3 + 0], l0 = table[bc * 3 + 1], carry = table[bc * 3 + 2];
    const bool emit = r0 > 0;  // rows [0, r0) of chunk i apply its effective weight
    bf16* W = Wbuf + bc * d * f;
    const int kb = (l0 / KS) * KS;
    const int nst = carry ? (L - kb + KS - 1) / KS : 0;  // stages of this chunk
    const int erows = nst > 0 ? ((BM + nst - 1) / nst + 7) / 8 * 8 : BM;
    int emitted = 0;
    if (emit) {
      // Stage R = W_down + S_i (the pre-update state) as bf16 for the storing waves.
      core::lds_barrier();  // the previous chunk's staged rows have all been read
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          float v[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) v[j] = R[0][mb][nb][j];
          stage_block_rows<BN>(v, stg, wm * 64 + mb * 32, wn * 64 + nb * 32, lane);
        }
      core::lds_barrier();
    }
    if (r0 < L) load_wdown();  // a document starts inside this chunk
    if (carry) {
      core::zero(D);
      for (int k0 = kb; k0 < L; k0 += KS) {
        // this stage is the oldest of `ahead` issued ones
        if (loader) {
          if (ahead >= 3) core::wait_vmcnt<2 * NLOAD>();
          else if (ahead == 2) core::wait_vmcnt<NLOAD>();
          else core::wait_vmcnt<0>();
        }
        core::lds_barrier();
        bf16* buf = lds + cbuf * STAGE;
        if (k0 < l0 || k0 + KS > L) {
          core::mask_tile_k<BM, ROWB, NT>(buf, l0 - k0, L - k0, tid);
          core::mask_tile_k<BN, ROWB, NT>(buf + SA, l0 - k0, L - k0, tid);
          core::lds_barrier();
        }
        const bool more = fi < N;
        const int ii = fi, ik = fk;
        bf16* nbuf = lds + ((cbuf + ahead) % NBUF) * STAGE;
        const bool emit_now = emit && emitted < BM;
        const int e0 = emitted;
        emitted = emit_now ? min(BM, emitted + erows) : emitted;
        const int e1 = emitted;
        const bf16* const lB[1] = {buf + SA};
        core::mma_stage<2, 2, 1, ROWB>(buf, lB, D, wm * 64, wn * 64, lane, [&](int kk) {
          if (loader) {
            if (more) issue(ii, ik, nbuf, (kk * NLOAD) / KSTEPS, ((kk + 1) * NLOAD) / KSTEPS);
          } else if (kk == 0 && emit_now) {
            emit_rows(W, e0, e1);
          }
        });
        if (more) {
          ++ahead;
          advance(fi, fk);
        }
        --ahead;
        cbuf = (cbuf + 1) % NBUF;
      }
    }
    if (emit && emitted < BM && !loader) emit_rows(W, emitted, BM);  // rows the stages did not cover
    if (carry) {
      const float sc = alpha[bc] * eta;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int j = 0; j < 16; ++j) R[0][mb][nb][j] = fmaf(sc, D[0][mb][nb][j], R[0][mb][nb][j]);
    }
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
  dim3 grid((unsigned)(((p.d + 127) / 128) * ((p.f + 127) / 128)), (unsigned)(p.B * p.N));
  if (p.dtype == 1)
    dw_kernel<bf16><<<grid, kThreads, 0, st>>>((const bf16*)Vt, (const bf16*)Zt, table, alpha, eta, dW, p.T,
                                               p.C, p.N, p.Cp, p.d, p.f);
  else
    dw_kernel<float><<<grid, kThreads, 0, st>>>((const float*)Vt, (const float*)Zt, table, alpha, eta, dW, p.T,
                                                p.C, p.N, p.Cp, p.d, p.f);
  return hipGetLastError();
}

hipError_t launch_scan(const Prob& p, const void* Zt, const void* Vt, const void* Wd,
                       const int32_t* table, const float* alpha, float eta, void* Wbuf,
                       hipStream_t st) {
  if (p.dtype == 1 && p.d % 64 == 0 && p.f % 64 == 0) {
    dim3 g((unsigned)(((p.d + 255) / 256) * ((p.f + 127) / 128)), (unsigned)p.B);
    scan_fast_kernel<<<g, 512, 0, st>>>((const bf16*)Zt, (const bf16*)Vt, (const bf16*)Wd, table, alpha, eta,
                                        (bf16*)Wbuf, p.T, p.C, p.N, p.Cp, p.d, p.f);
    return hipGetLastError();
  }
  dim3 grid((unsigned)(((p.d + 127) / 128) * ((p.f + 127) / 128)), (unsigned)p.B);
  if (p.dtype == 1)
    scan_kernel<bf16><<<grid, kThreads, 0, st>>>((const bf16*)Zt, (const bf16*)Vt, (const bf16*)Wd, table, alpha,
                                                 eta, (bf16*)Wbuf, p.T, p.C, p.N, p.Cp, p.d, p.f);
  else
    scan_kernel<float><<<grid, kThreads, 0, st>>>((const float*)Zt, (const float*)Vt, (const float*)Wd, table,
                                                  alpha, eta, (float*)Wbuf, p.T, p.C, p.N, p.Cp, p.d, p.f);
  return hipGetLastError();
}

}  // namespace ipttt
