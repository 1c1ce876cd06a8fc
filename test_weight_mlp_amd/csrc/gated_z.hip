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
// tile, gate and up tiles against the same H tile, 8 waves (two per SIMD), a
// wave holding 64 x 64 of both products.  Operands move HBM/L2 -> LDS with
// direct-to-LDS loads into two stage buffers of 64 K columns.
//
// Persistent: one workgroup per CU walks its tiles, and before writing out a
// finished tile it issues the first stage of its next one, so that load
// latency and the epilogue overlap.  Workgroup w runs on XCD w % 8 (the
// hardware hands out consecutive workgroups to the XCDs in turn); the 32 of
// an XCD walk a contiguous range of logical tiles together, 32 at a time,
// grouped 4 token tiles at a time so that they share H and weight panels in
// the XCD's L2.
//
// Ping-pong schedule: waves 0-3 and 4-7 are two groups with one wave of each
// on every SIMD.  A tile's K loop is cut into clusters of two k-steps (32 of
// K); every wave alternates a memory
// phase (the LDS fragment reads of its next cluster, and once per stage its
// share of the direct-to-LDS loads of the next stage) and a compute phase
// (the cluster's 16 MFMAs on fragments already in registers), and group 1 runs
// one phase behind group 0.  A workgroup barrier ends every phase, so at any
// time one wave of each SIMD multiplies while the other reads: the matrix
// core does not wait for the fragment reads that follow each barrier.
// A wave's phases per stage s (S stages of 64 K): memory (half 0), compute,
// memory (half 1), compute.  Barriers count arrivals, not code positions:
// group 1 meets one extra barrier before its first phase, so every barrier
// sits between phase k of group 0 and phase k-1 of group 1.  Stage s+1 goes
// into the buffer of stage s-1 once the barrier after the last read of
// stage s-1 (group 1, half 1) has passed, and every wave's loads of it are
// done before the barrier after which group 0 first reads it.
template <bool SAVE>
__global__ __launch_bounds__(512) void gated_z_fast_kernel(const bf16* __restrict__ H, const bf16* __restrict__ Wg,
                                                         const bf16* __restrict__ Wu, bf16* __restrict__ Z,
                                                         bf16* __restrict__ Gs, bf16* __restrict__ Us, int64_t M, int d,
                                                         int f) {
  constexpr int BM = 256, BN = 128, LDR = BN, KS = 64;
  constexpr int SA = BM * KS, SB = BN * KS, STAGE = SA + 2 * SB;  // bf16 elements
  static_assert(BM * LDR <= STAGE, "the staging tile reuses one stage buffer");
  __shared__ __attribute__((aligned(1024))) bf16 lds[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, hi = lane >> 5;
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (f + BN - 1) / BN;
  const int ntiles = tiles_m * tiles_n;
  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int range = (ntiles + 7) >> 3;
  const int t_end = min(ntiles, (xcd + 1) * range);
  int t = xcd * range + slot;
  if (t >= t_end) return;

  auto operands = [&](int tt, int64_t& m0, int& n0, core::Operand& oa, core::Operand (&ob)[2]) {
    int tm, tn;
    grouped_tile(tt, tiles_m, tiles_n, 4, tm, tn);
    m0 = (int64_t)tm * BM;
    n0 = tn * BN;
    oa = core::make_operand(H + m0 * d, (int64_t)d * 2, (M - m0) * d * 2);
    ob[0] = core::make_operand(Wg + (int64_t)n0 * d, (int64_t)d * 2, (int64_t)(f - n0) * d * 2);
    ob[1] = core::make_operand(Wu + (int64_t)n0 * d, (int64_t)d * 2, (int64_t)(f - n0) * d * 2);
  };
  // this wave's 8 direct-to-LDS loads of stage s (4 of the H tile, 2 of each weight tile)
  auto issue_stage = [&](const core::Operand& oa, const core::Operand (&ob)[2], int s, int buf) {
    bf16* b = lds + buf * STAGE;
    const int k0 = s * KS;
    core::load_tile_part<BM, 128, 8>(oa, k0, b, wave, lane, 0, 4);
    core::load_tile_part<BN, 128, 8>(ob[0], k0, b + SA, wave, lane, 0, 2);
    core::load_tile_part<BN, 128, 8>(ob[1], k0, b + SA + SB, wave, lane, 0, 2);
  };
  const int S = d / KS;
  int base = 0;
  int64_t m0;
  int n0;
  core::Operand oa, ob[2];
  operands(t, m0, n0, oa, ob);
  bool pre = false;
  for (; t < t_end; t += per_xcd) {
    floatx16 acc[2][2][2];
    core::zero(acc);
    bf16x8 fa[2][2], fb[2][2][2];  // [k-step][block], [k-step][gate/up][block]
    if (!pre) issue_stage(oa, ob, 0, base);
    core::wait_vmcnt<0>();
    core::lds_barrier();
    // memory phase of half h (k-steps 2h, 2h+1) of stage s
    auto mem = [&](int s, int h) {
      if (h == 0 && s + 1 < S) issue_stage(oa, ob, s + 1, (base + s + 1) & 1);
      const bf16* b = lds + ((base + s) & 1) * STAGE;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int c = (2 * h + kk) * 2 + hi;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) fa[kk][mb] = core::ld_frag<128>(b, wm * 64 + mb * 32 + lr, c);
#pragma unroll
        for (int o = 0; o < 2; ++o)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) fb[kk][o][nb] = core::ld_frag<128>(b + SA + o * SB, wn * 64 + nb * 32 + lr, c);
      }
    };
    auto compute = [&]() {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int o = 0; o < 2; ++o)
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
              acc[o][mb][nb] =
                  __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk][mb], fb[kk][o][nb], acc[o][mb][nb], 0, 0, 0);
    };
    auto phase_end = [&](bool wait_loads) {
      __builtin_amdgcn_sched_barrier(0);
      if (wait_loads) core::wait_vmcnt<0>();
      core::lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // Both groups run the same phases; group 1 meets one extra barrier before
    // them and group 0 one after, so group 1 is one phase behind throughout.
    // Each wave issues its loads of stage s+1 in its memory phase of half 0
    // of stage s, and waits for them before the barrier ahead of group 0's
    // first read of stage s+1 (group 0: after its compute phase of half 1 of
    // stage s; group 1: after its memory phase of half 1).
    if (grp == 1) phase_end(false);
    for (int s = 0; s < S; ++s) {
      mem(s, 0);
      phase_end(false);
      compute();
      phase_end(false);
      mem(s, 1);
      phase_end(grp == 1);
      compute();
      phase_end(grp == 0);
    }
    if (grp == 0) phase_end(false);
    const int64_t mt = m0;
    const int nt = n0;
    const int mrows = (int)min((int64_t)BM, M - mt), nrows = min(BN, f - nt);
    bf16* stg = lds + ((base + S - 1) & 1) * STAGE;  // the stage buffer read last
    base = (base + S) & 1;
    pre = t + per_xcd < t_end;
    if (pre) {
      operands(t + per_xcd, m0, n0, oa, ob);
      issue_stage(oa, ob, 0, base);
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float z[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) z[j] = silu_f32(acc[0][mb][nb][j]) * acc[1][mb][nb][j];
        stage_block_rows_swz<LDR>(z, stg, wm * 64 + mb * 32, wn * 64 + nb * 32, lane);
      }
    core::lds_barrier();
    store_rows_swz<BM, BN, LDR, 512, true>(stg, Z, mt, 0, mrows, nt, nrows, f, tid);
    core::lds_barrier();
    if constexpr (SAVE) {
#pragma unroll
      for (int o = 0; o < 2; ++o) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            float v[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = acc[o][mb][nb][j];
            stage_block_rows_swz<LDR>(v, stg, wm * 64 + mb * 32, wn * 64 + nb * 32, lane);
          }
        core::lds_barrier();
        store_rows_swz<BM, BN, LDR, 512, true>(stg, o == 0 ? Gs : Us, mt, 0, mrows, nt, nrows, f, tid);
        core::lds_barrier();
      }
    }
  }
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
