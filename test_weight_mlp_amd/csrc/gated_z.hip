// Z = SiLU(H W_gate^T) * (H W_up^T): the intermediate activation of the gated
// MLP (lijianxiong.blog "In-Place Test-Time Training", 方法 > 原地自适应 and
// 高效的块状更新机制; phi = SiLU).
//
// One workgroup computes a 128-token x 128-feature tile of Z: the same H tile
// is multiplied by the gate and the up tiles (a dual GEMM, K = d_model), both
// products stay in fp32 registers, and the epilogue applies SiLU(g) * u before
// rounding once to the output type.  Z is written row-major.
#include <algorithm>

#include "epilogue.h"
#include "launch.h"
#include "mfma_core.h"
#include "pingpong.h"

namespace ipttt {

// SAVE: also write G = H W_gate^T and U = H W_up^T (dtype) for the backward.
template <typename T, bool SAVE>
__global__ __launch_bounds__(kThreads) void gated_z_kernel(const T* __restrict__ H, const T* __restrict__ Wg,
                                                           const T* __restrict__ Wu, T* __restrict__ Z,
                                                           T* __restrict__ Gs, T* __restrict__ Us, int64_t M, int d,
                                                           int f) {
  typedef Geo<T, 128, 128> G;
  constexpr int LDC = G::BN + G::VE;
  constexpr int kStage = (G::BM + 2 * G::BN) * G::LDK;
  constexpr int kEpi = G::BM * LDC;
  __shared__ __attribute__((aligned(16))) T lds[kStage > kEpi ? kStage : kEpi];
  T* lA = lds;
  T* lB0 = lds + G::BM * G::LDK;
  T* lB1 = lB0 + G::BN * G::LDK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tiles_m = (int)((M + G::BM - 1) / G::BM), tiles_n = (f + G::BN - 1) / G::BN;
  int tm, tn;
  grouped_tile(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, 16, tm, tn);
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

  T* lC = lds;
  // which = 0: Z, 1: G, 2: U
  auto emit = [&](int which, T* out) {
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = wm * G::WM + mb * 32 + acc_row(j, lane);
          const int c = wn * G::WN + nb * 32 + (lane & 31);
          const float g = ag[mb][nb][j], u = au[mb][nb][j];
          lC[r * LDC + c] = from_f32<T>(which == 0 ? silu_f32(g) * u : which == 1 ? g : u);
        }
    __syncthreads();
    store_tile_rows<T, G::BM, G::BN, LDC>(lC, out, m0, mrows, n0, nrows, f, tid);
  };
  emit(0, Z);
  if constexpr (SAVE) {
    __syncthreads();
    emit(1, Gs);
    __syncthreads();
    emit(2, Us);
  }
}

// bf16 fast path (d_model a multiple of 64): 256 tokens x 128 features per
// tile on the persistent ping-pong core (pingpong.h), the gate and up tiles
// of W against the same H tile; the epilogue forms SiLU(g) * u in fp32,
// stages it through LDS and writes Z rows with non-temporal stores.  The
// tiles are grouped 4 token tiles at a time so that an XCD's workgroups share
// H and weight panels in its L2.
template <bool SAVE>
__global__ __launch_bounds__(512) void gated_z_fast_kernel(const bf16* __restrict__ H, const bf16* __restrict__ Wg,
                                                         const bf16* __restrict__ Wu, bf16* __restrict__ Z,
                                                         bf16* __restrict__ Gs, bf16* __restrict__ Us, int64_t M, int d,
                                                         int f) {
  using namespace pingpong;
  __shared__ __attribute__((aligned(1024))) bf16 lds[LDS_ELEMS];
  const int tid = threadIdx.x;
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (f + BN - 1) / BN;
  auto origin = [&](int tt, int64_t& m0, int& n0) {
    int tm, tn;
    grouped_tile(tt, tiles_m, tiles_n, 4, tm, tn);
    m0 = (int64_t)tm * BM;
    n0 = tn * BN;
  };
  auto operands = [&](int tt, core::Operand& oa, core::Operand (&ob)[2], bool&, int& S) {
    int64_t m0;
    int n0;
    origin(tt, m0, n0);
    S = d / KS;
    oa = core::make_operand(H + m0 * d, (int64_t)d * 2, (M - m0) * d * 2);
    ob[0] = core::make_operand(Wg + (int64_t)n0 * d, (int64_t)d * 2, (int64_t)(f - n0) * d * 2);
    ob[1] = core::make_operand(Wu + (int64_t)n0 * d, (int64_t)d * 2, (int64_t)(f - n0) * d * 2);
  };
  auto epilogue = [&](int tt, floatx16 (&acc)[2][2][2], bf16* stg) {
    int64_t mt;
    int nt;
    origin(tt, mt, nt);
    const int mrows = (int)min((int64_t)BM, M - mt), nrows = min(BN, f - nt);
    stage_wave(stg, [&](int mb, int nb, int j) { return silu_f32(acc[0][mb][nb][j]) * acc[1][mb][nb][j]; });
    core::lds_barrier();
    store_rows_swz<BM, BN, LDR, 512, true>(stg, Z, mt, 0, mrows, nt, nrows, f, tid);
    core::lds_barrier();
    if constexpr (SAVE) {
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        stage_wave(stg, [&](int mb, int nb, int j) { return acc[o][mb][nb][j]; });
        core::lds_barrier();
        store_rows_swz<BM, BN, LDR, 512, true>(stg, o == 0 ? Gs : Us, mt, 0, mrows, nt, nrows, f, tid);
        core::lds_barrier();
      }
    }
  };
  pingpong::run(lds, tiles_m * tiles_n, operands, epilogue);
}

hipError_t launch_gated_z(const Prob& p, const void* H, const void* Wg, const void* Wu, void* Z, void* GU,
                          hipStream_t st) {
  const size_t e = p.dtype == 1 ? 2 : 4;
  void* Gs = GU;
  void* Us = GU != nullptr ? static_cast<char*>(GU) + (size_t)p.M * p.f * e : nullptr;
  const bool save = GU != nullptr;
  const int64_t tiles = ((p.M + 127) / 128) * ((p.f + 127) / 128);
  note_launch("gated_z", st);
  if (p.dtype == 1 && p.d % 64 == 0) {
    // one persistent workgroup per CU (the mapping needs a multiple of 8)
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
      (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t fast_tiles = ((p.M + 255) / 256) * ((p.f + 127) / 128);
    const int64_t g = std::min<int64_t>(std::max(8, cus / 8 * 8), (fast_tiles + 7) / 8 * 8);
    if (save)
      gated_z_fast_kernel<true><<<(unsigned)g, 512, 0, st>>>((const bf16*)H, (const bf16*)Wg, (const bf16*)Wu,
                                                          (bf16*)Z, (bf16*)Gs, (bf16*)Us, p.M, p.d, p.f);
    else
      gated_z_fast_kernel<false><<<(unsigned)g, 512, 0, st>>>((const bf16*)H, (const bf16*)Wg, (const bf16*)Wu,
                                                           (bf16*)Z, nullptr, nullptr, p.M, p.d, p.f);
  } else if (p.dtype == 1) {
    if (save)
      gated_z_kernel<bf16, true><<<(unsigned)tiles, kThreads, 0, st>>>(
          (const bf16*)H, (const bf16*)Wg, (const bf16*)Wu, (bf16*)Z, (bf16*)Gs, (bf16*)Us, p.M, p.d, p.f);
    else
      gated_z_kernel<bf16, false><<<(unsigned)tiles, kThreads, 0, st>>>(
          (const bf16*)H, (const bf16*)Wg, (const bf16*)Wu, (bf16*)Z, nullptr, nullptr, p.M, p.d, p.f);
  } else {
    if (save)
      gated_z_kernel<float, true><<<(unsigned)tiles, kThreads, 0, st>>>(
          (const float*)H, (const float*)Wg, (const float*)Wu, (float*)Z, (float*)Gs, (float*)Us, p.M, p.d, p.f);
    else
      gated_z_kernel<float, false><<<(unsigned)tiles, kThreads, 0, st>>>(
          (const float*)H, (const float*)Wg, (const float*)Wu, (float*)Z, nullptr, nullptr, p.M, p.d, p.f);
  }
  return hipGetLastError();
}

}  // namespace ipttt
