// V_hat = Conv1D(X0) W_target: the LM-aligned target (lijianxiong.blog
// "In-Place Test-Time Training", 对齐语言模型的目标函数; tencent article
// "榨干MLP的剩余价值", 详细步骤 3; iplexlaw.co.kr review, section 6).
//
// W_target is stored [d_in, d_out]; the B operand wants d_in contiguous, so a
// small kernel first writes its transpose (and the conv weights tap-major)
// into the workspace.  Each token reads as many of its five X0 rows as its
// window allows (padding at chunk ends and document starts).
//   bf16, d_model a multiple of 64: an elementwise pass writes the conv output
//     Y (bf16) to the workspace, then target_fast_kernel multiplies it by
//     W_target on the matrix cores (256 x 256 tiles, 8 waves, persistent);
//   otherwise: the conv is folded into the staging of the A operand of a
//     128 x 128 tile product (target_kernel).
#include <algorithm>

#include "epilogue.h"
#include "launch.h"
#include "mfma_core.h"
#include "pingpong.h"

namespace ipttt {

// out[c][r] = in[r][c] for a rows x cols matrix, through a 32x33 LDS tile.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, T* __restrict__ out, int rows,
                                                        int cols) {
  __shared__ T tile[32][33];
  const int bx = blockIdx.x * 32, by = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int y = ty; y < 32; y += 8) {
    const int r = by + y, c = bx + tx;
    if (r < rows && c < cols) tile[y][tx] = in[(int64_t)r * cols + c];
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    const int c = bx + y, r = by + tx;
    if (r < rows && c < cols) out[(int64_t)c * rows + r] = tile[tx][y];
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void target_kernel(const T* __restrict__ X0, const T* __restrict__ convT,
                                                          const T* __restrict__ WtT, const uint8_t* __restrict__ segs,
                                                          T* __restrict__ V, int64_t M, int d) {
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
  const int tiles_m = (int)((M + G::BM - 1) / G::BM), tiles_n = (d + G::BN - 1) / G::BN;
  int tm, tn;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, 16, tm, tn);
  const int64_t m0 = (int64_t)tm * G::BM;
  const int n0 = tn * G::BN;
  const int mrows = (int)min((int64_t)G::BM, M - m0), nrows = min(G::BN, d - n0);
  const T* B = WtT + (int64_t)n0 * d;

  // A staging: the conv output for this thread's vectors, computed in fp32
  // and rounded once.
  constexpr int NVA = G::BM * 8 / kThreads;
  u32x4 av[NVA];
  uint8_t taps[NVA];
#pragma unroll
  for (int j = 0; j < NVA; ++j) {
    const int r = (tid + j * kThreads) >> 3;
    taps[j] = r < mrows ? (segs[m0 + r] & 7) : 0;
  }
  auto load_a = [&](int k0) {
#pragma unroll
    for (int j = 0; j < NVA; ++j) {
      const int idx = tid + j * kThreads;
      const int r = idx >> 3, k = k0 + (idx & 7) * VE;
      float y[VE];
#pragma unroll
      for (int q = 0; q < VE; ++q) y[q] = 0.0f;
      if (k < d) {
        for (int s = 0; s < taps[j]; ++s) {
          u32x4 xv = *reinterpret_cast<const u32x4*>(X0 + (m0 + r + s) * d + k);
          u32x4 wv = *reinterpret_cast<const u32x4*>(convT + (int64_t)s * d + k);
          const T* xe = reinterpret_cast<const T*>(&xv);
          const T* we = reinterpret_cast<const T*>(&wv);
#pragma unroll
          for (int q = 0; q < VE; ++q) y[q] = fmaf(to_f32(we[q]), to_f32(xe[q]), y[q]);
        }
      }
      T* e = reinterpret_cast<T*>(&av[j]);
#pragma unroll
      for (int q = 0; q < VE; ++q) e[q] = from_f32<T>(y[q]);
    }
  };
  auto store_a = [&]() {
#pragma unroll
    for (int j = 0; j < NVA; ++j) {
      const int idx = tid + j * kThreads;
      *reinterpret_cast<u32x4*>(lA + (idx >> 3) * G::LDK + (idx & 7) * VE) = av[j];
    }
  };

  floatx16 acc[G::MB][G::NB];
  zero_acc<G>(acc);
  TileLoad<T, G::BN> lb;
  load_a(0);
  lb.load(B, d, nrows, 0, d, tid);
  for (int k0 = 0; k0 < d; k0 += G::BK) {
    store_a();
    lb.template store<G::LDK>(lB, tid);
    __syncthreads();
    if (k0 + G::BK < d) {
      load_a(k0 + G::BK);
      lb.load(B, d, nrows, k0 + G::BK, d, tid);
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
  store_tile_rows<T, G::BM, G::BN, LDC>(lC, V, m0, mrows, n0, nrows, d, tid);
}

// Y[t, c] = sum over the token's taps of convw[c, k] * X0[t+k, c], rounded once
// to the data type.  A thread owns 16 bytes of channels over a run of
// kConvRun consecutive tokens and slides a five-row window of X0 down the run
// (rows past the last token clamped to it), so each X0 row and each tap's
// weights are loaded once per run; taps beyond a token's count are dropped.
// The weights are read in their own [d, 5] layout: a thread's channels own 5
// VE consecutive elements, 16-byte aligned (80 bytes per 16-byte channel group).
constexpr int kConvRun = 8;
template <typename T>
__global__ __launch_bounds__(256) void conv_kernel(const T* __restrict__ X0, const T* __restrict__ convw,
                                                   const uint8_t* __restrict__ segs, T* __restrict__ Y, int64_t M,
                                                   int d) {
  constexpr int VE = 16 / sizeof(T);
  const int vpr = d / VE;
  const int64_t runs = (M + kConvRun - 1) / kConvRun;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= runs * vpr) return;
  const int64_t run = idx / vpr;
  const int c = (int)(idx - run * vpr) * VE;
  const int64_t t0 = run * kConvRun;
  u32x4 xv[kConvRun + 4], wv[5];
#pragma unroll
  for (int s = 0; s < kConvRun + 4; ++s) xv[s] = *reinterpret_cast<const u32x4*>(X0 + min(t0 + s, M - 1) * d + c);
#pragma unroll
  for (int s = 0; s < 5; ++s) wv[s] = *reinterpret_cast<const u32x4*>(convw + (int64_t)c * 5 + s * VE);
  const T* wa = reinterpret_cast<const T*>(wv);  // channel c + q, tap s at wa[5 q + s]
#pragma unroll
  for (int k = 0; k < kConvRun; ++k) {
    const int64_t t = t0 + k;
    if (t >= M) break;
    const int taps = segs[t] & 7;
    float y[VE];
#pragma unroll
    for (int q = 0; q < VE; ++q) y[q] = 0.0f;
#pragma unroll
    for (int s = 0; s < 5; ++s) {
      const T* xe = reinterpret_cast<const T*>(&xv[k + s]);
#pragma unroll
      for (int q = 0; q < VE; ++q) y[q] = s < taps ? fmaf(to_f32(wa[5 * q + s]), to_f32(xe[q]), y[q]) : y[q];
    }
    u32x4 out;
    T* oe = reinterpret_cast<T*>(&out);
#pragma unroll
    for (int q = 0; q < VE; ++q) oe[q] = from_f32<T>(y[q]);
    *reinterpret_cast<u32x4*>(Y + t * d + c) = out;
  }
}

// Threads of conv_kernel.
template <typename T>
static int64_t conv_threads(const Prob& p) {
  return (p.M + kConvRun - 1) / kConvRun * (p.d / (16 / (int)sizeof(T)));
}

// Tap-major identity conv weights (tap 0 = 1, the others 0): the target
// without Conv1D on the general kernels, whose conv is fused into the GEMM.
template <typename T>
__global__ __launch_bounds__(256) void identity_taps_kernel(T* __restrict__ convT, int d) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < 5 * d; i += gridDim.x * blockDim.x)
    convT[i] = from_f32<T>(i < d ? 1.0f : 0.0f);
}

// V_hat = Y W_target on the matrix cores: 256 tokens x 256 outputs per tile on
// the persistent ping-pong core (pingpong.h), whose two 128-row B operands are
// the two halves of the tile's 256 rows of W_target^T (WtT[n, k], transposed
// once per call, so both operands are read as rows); each half is staged
// through LDS and written as row-major V.  (Reading W_target K-major in place,
// with transposing fragment reads, took 0.52 ms instead of 0.39 at the 4B
// shape on the non-persistent core: more than the 0.02 ms transpose.)
__global__ __launch_bounds__(512) void target_fast_kernel(const bf16* __restrict__ Y, const bf16* __restrict__ WtT,
                                                        bf16* __restrict__ V, int64_t M, int d) {
  using namespace pingpong;
  constexpr int BW = 2 * BN;  // output columns per tile
  __shared__ __attribute__((aligned(1024))) bf16 lds[LDS_ELEMS];
  const int tid = threadIdx.x;
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (d + BW - 1) / BW;
  auto origin = [&](int tt, int64_t& m0, int& n0) {
    int tm, tn;
    grouped_tile(tt, tiles_m, tiles_n, 8, tm, tn);
    m0 = (int64_t)tm * BM;
    n0 = tn * BW;
  };
  auto operands = [&](int tt, core::Operand& oa, core::Operand (&ob)[2], bool&, int& S) {
    int64_t m0;
    int n0;
    origin(tt, m0, n0);
    S = d / KS;
    oa = core::make_operand(Y + m0 * d, (int64_t)d * 2, (M - m0) * d * 2);
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const int r0 = n0 + o * BN;  // rows past d read as zero (valid bytes clamp at 0)
      ob[o] = core::make_operand(WtT + (int64_t)r0 * d, (int64_t)d * 2, (int64_t)(d - r0) * d * 2);
    }
  };
  auto epilogue = [&](int tt, floatx16 (&acc)[2][2][2], bf16* stg) {
    int64_t mt;
    int nt;
    origin(tt, mt, nt);
    const int mrows = (int)min((int64_t)BM, M - mt);
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      stage_wave(stg, [&](int mb, int nb, int j) { return acc[o][mb][nb][j]; });
      core::lds_barrier();
      store_rows_swz<BM, BN, LDR, 512, false>(stg, V, mt, 0, mrows, nt + o * BN, min(BN, d - nt - o * BN), d, tid);
      core::lds_barrier();
    }
  };
  pingpong::run(lds, tiles_m * tiles_n, operands, epilogue);
}

template <typename T>
static void launch_target_t(const Prob& p, const T* X0, const T* convw, const T* Wt, const uint8_t* segs,
                            T* V, T* scratch, hipStream_t st) {
  T* WtT = scratch;
  T* convT = scratch + (int64_t)p.d * p.d;
  T* Y = convT + (int64_t)5 * p.d;
  const int64_t nv = conv_threads<T>(p);
  if (p.target == 2) {  // no W_target: V_hat is the conv output itself
    note_launch("conv", st);
    conv_kernel<T><<<(unsigned)((nv + 255) / 256), 256, 0, st>>>(X0, convw, segs, V, p.M, p.d);
    return;
  }
  // both GEMMs take W_target transposed
  note_launch("target_prep", st);
  dim3 tg((p.d + 31) / 32, (p.d + 31) / 32);
  transpose_kernel<T><<<tg, 256, 0, st>>>(Wt, WtT, p.d, p.d);
  if constexpr (sizeof(T) == 2) {
    if (p.d % 64 == 0) {
      const T* A = X0;  // no Conv1D: the GEMM reads X0 directly
      if (p.target == 0) {
        note_launch("conv", st);
        conv_kernel<T><<<(unsigned)((nv + 255) / 256), 256, 0, st>>>(X0, convw, segs, Y, p.M, p.d);
        A = Y;
      }
      // one persistent workgroup per CU (the tile walk needs a multiple of 8)
      int dev = 0, cus = 256;
      if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      const int64_t tiles = ((p.M + 255) / 256) * ((p.d + 255) / 256);
      const int64_t g = std::min<int64_t>(std::max(8, cus / 8 * 8), (tiles + 7) / 8 * 8);
      note_launch("target_gemm", st);
      target_fast_kernel<<<(unsigned)g, 512, 0, st>>>(A, WtT, V, p.M, p.d);
      return;
    }
  }
  // the general kernel fuses the conv and takes its taps tap-major
  if (p.target == 1) {
    identity_taps_kernel<T><<<(5 * p.d + 255) / 256, 256, 0, st>>>(convT, p.d);
  } else {
    dim3 cgd(1, (p.d + 31) / 32);
    transpose_kernel<T><<<cgd, 256, 0, st>>>(convw, convT, p.d, 5);
  }
  const int64_t tiles = ((p.M + 127) / 128) * ((p.d + 127) / 128);
  note_launch("target_gemm", st);
  target_kernel<T><<<(unsigned)tiles, kThreads, 0, st>>>(X0, convT, WtT, segs, V, p.M, p.d);
}

// The conv alone, Y (dtype) = Conv1D(X0).
template <typename T>
static void launch_conv_only_t(const Prob& p, const T* X0, const T* convw, const uint8_t* segs, T* Y,
                               hipStream_t st) {
  const int64_t nv = conv_threads<T>(p);
  note_launch("conv", st);
  conv_kernel<T><<<(unsigned)((nv + 255) / 256), 256, 0, st>>>(X0, convw, segs, Y, p.M, p.d);
}

hipError_t launch_conv_only(const Prob& p, const void* X0, const void* convw, const uint8_t* segs, void* Y,
                            void* scratch, hipStream_t st) {
  (void)scratch;
  if (p.dtype == 1)
    launch_conv_only_t<bf16>(p, (const bf16*)X0, (const bf16*)convw, segs, (bf16*)Y, st);
  else
    launch_conv_only_t<float>(p, (const float*)X0, (const float*)convw, segs, (float*)Y, st);
  return hipGetLastError();
}

hipError_t launch_target(const Prob& p, const void* X0, const void* convw, const void* Wt,
                         const uint8_t* segs, void* V, void* scratch, hipStream_t st) {
  if (p.dtype == 1)
    launch_target_t<bf16>(p, (const bf16*)X0, (const bf16*)convw, (const bf16*)Wt, segs, (bf16*)V,
                          (bf16*)scratch, st);
  else
    launch_target_t<float>(p, (const float*)X0, (const float*)convw, (const float*)Wt, segs,
                           (float*)V, (float*)scratch, st);
  return hipGetLastError();
}

}  // namespace ipttt
