// Persistent ping-pong product core for gfx950: per tile, two NT products
// that share their A operand, acc[o] = A[256 rows, K] * B_o[128 rows, K]^T
// (o = 0, 1), with direct-to-LDS operand loads, 32x32x16 bf16 MFMAs and an
// epilogue supplied by the kernel that uses it.  The gated MLP's Z kernel
// takes B_0 = W_gate and B_1 = W_up rows of one 128-feature tile; the LM
// target's GEMM takes the two 128-row halves of one 256-column tile of
// W_target^T.
//
// 256 rows x (128 + 128) columns per tile, 8 waves (two per SIMD), a wave
// holding 64 x 64 of both products.  Operands move HBM/L2 -> LDS with
// direct-to-LDS loads into two stage buffers of 64 K columns.
//
// Persistent: one workgroup per CU walks its tiles, and before writing out a
// finished tile it issues the first stage of its next one, so that load
// latency and the epilogue overlap.  Workgroup w runs on XCD w % 8 (the
// hardware hands out consecutive workgroups to the XCDs in turn); the 32 of
// an XCD walk a contiguous range of logical tiles together, 32 at a time, so
// that tiles next to each other in the caller's order share operand panels
// in the XCD's L2.
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
#pragma once

#include "common.h"
#include "epilogue.h"
#include "mfma_core.h"

namespace ipttt {
namespace pingpong {

constexpr int BM = 256, BN = 128, KS = 64, LDR = BN;
constexpr int SA = BM * KS, SB = BN * KS, STAGE = SA + 2 * SB;  // bf16 elements
static_assert(BM * LDR <= STAGE, "the staging tile reuses one stage buffer");
constexpr int LDS_ELEMS = 2 * STAGE;

// Walk tiles [0, ntiles) with the workgroups of the launch (a multiple of 8,
// one per CU).  operands(t, oa, ob, shared, S) sets tile t's operand
// resources (A rows [256], B_0 and B_1 rows [128], K-contiguous) and its K
// length in 64-column stages S; with SHARE, `shared` says that B_0 and B_1
// are rows [0, 128) and [128, 256) of A itself (a Gram tile on the diagonal),
// so that only A is loaded.  epilogue(t, acc, stg) consumes the finished
// accumulators, with the 64 KB stage buffer `stg` free for staging (the next
// tile's first stage is already in flight in the other buffer); it must end
// with an LDS barrier if it wrote `stg`.
template <bool SHARE = false, class Operands, class Epilogue>
__device__ __forceinline__ void run(bf16* lds, int ntiles, Operands&& operands, Epilogue&& epilogue) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, hi = lane >> 5;
  const int per_xcd = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int range = (ntiles + 7) >> 3;
  const int t_end = min(ntiles, (xcd + 1) * range);
  int t = xcd * range + slot;
  if (t >= t_end) return;

  // this wave's 8 direct-to-LDS loads of stage s (4 of the A tile, 2 of each B tile)
  auto issue_stage = [&](const core::Operand& oa, const core::Operand (&ob)[2], bool sh, int s, int buf) {
    bf16* b = lds + buf * STAGE;
    const int k0 = s * KS;
    core::load_tile_part<BM, 128, 8>(oa, k0, b, wave, lane, 0, 4);
    if (!SHARE || !sh) {
      core::load_tile_part<BN, 128, 8>(ob[0], k0, b + SA, wave, lane, 0, 2);
      core::load_tile_part<BN, 128, 8>(ob[1], k0, b + SA + SB, wave, lane, 0, 2);
    }
  };
  int base = 0;
  core::Operand oa, ob[2];
  bool shared = false;
  int S_next = 0;
  operands(t, oa, ob, shared, S_next);
  bool pre = false;
  for (; t < t_end; t += per_xcd) {
    const int S = S_next;
    const bool sh = SHARE && shared;
    // B_o's rows relative to the stage buffer: after A, or A's own rows
    const int brow = sh ? 0 : BM;
    floatx16 acc[2][2][2];
    core::zero(acc);
    bf16x8 fa[2][2], fb[2][2][2];  // [k-step][block], [k-step][B operand][block]
    if (!pre) issue_stage(oa, ob, sh, 0, base);
    core::wait_vmcnt<0>();
    core::lds_barrier();
    // memory phase of half h (k-steps 2h, 2h+1) of stage s
    auto mem = [&](int s, int h) {
      if (h == 0 && s + 1 < S) issue_stage(oa, ob, sh, s + 1, (base + s + 1) & 1);
      const bf16* b = lds + ((base + s) & 1) * STAGE;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int c = (2 * h + kk) * 2 + hi;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) fa[kk][mb] = core::ld_frag<128>(b, wm * 64 + mb * 32 + lr, c);
#pragma unroll
        for (int o = 0; o < 2; ++o)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) fb[kk][o][nb] = core::ld_frag<128>(b, brow + o * BN + wn * 64 + nb * 32 + lr, c);
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
    bf16* stg = lds + ((base + S - 1) & 1) * STAGE;  // the stage buffer read last
    base = (base + S) & 1;
    pre = t + per_xcd < t_end;
    if (pre) {
      operands(t + per_xcd, oa, ob, shared, S_next);
      issue_stage(oa, ob, SHARE && shared, 0, base);
    }
    epilogue(t, acc, stg);
  }
}

// Stage a wave's 64 x 64 block of product o (values v(o, mb, nb, j)) into the
// swizzled 256 x 128 staging tile.
template <class Value>
__device__ __forceinline__ void stage_wave(bf16* stg, Value&& v) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float z[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) z[j] = v(mb, nb, j);
      stage_block_rows_swz<LDR>(z, stg, wm * 64 + mb * 32, wn * 64 + nb * 32, lane);
    }
}

}  // namespace pingpong
}  // namespace ipttt
