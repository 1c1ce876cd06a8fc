// bf16 tile-product core for gfx950: direct-to-LDS operand loads, XOR-swizzled
// LDS tiles, double buffering (or a ring of half stages), 32x32x16 MFMA with
// (MB*32) x (NB*32) wave tiles.
//
// Operands are K-contiguous rows ("NT" products).  A K stage holds ROWB bytes
// per row (128: 64 bf16, or 64: 32 bf16).  A wave-wide buffer_load_dwordx4 ...
// lds writes its 64 lanes' 16-byte pieces to 1 KB of consecutive LDS, lane i at
// offset 16*i, so lane i fetches row i / (ROWB/16) of its 1 KB block and
// whichever 16-byte column chunk belongs in slot i % (ROWB/16) of that row.
// LDS row r holds logical chunk c at slot c ^ ((r / RPL) % SLOTS), RPL = 256 /
// ROWB rows per 256 bytes, SLOTS = ROWB / 16: the LDS has 64 four-byte banks and
// serves a ds_read_b128 16 lanes at a time, and the 16 rows that 16
// neighbouring lanes read (one chunk each) then land on 16 distinct bank quads.
// Loads go through buffer resources: bytes past the resource's end read as
// zero, which covers ragged matrix edges.
#pragma once

#include "common.h"

namespace ipttt {
namespace core {

constexpr int BK = 64;        // bf16 K elements of a 128-byte stage row

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Cache-policy bits of the operand loads (buffer instruction aux operand).
#ifndef IPTTT_LOAD_AUX
#define IPTTT_LOAD_AUX 0
#endif
constexpr int kLoadAux = IPTTT_LOAD_AUX;

struct Operand {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t row_stride;  // bytes between consecutive rows
};

// Resource covering [base, base + valid_bytes); reads beyond return zero.
__device__ __forceinline__ Operand make_operand(const void* base, int64_t row_stride_bytes, int64_t valid_bytes) {
  Operand op;
  const int64_t lim = valid_bytes < 0 ? 0 : (valid_bytes > 0xFFFFFFF0LL ? 0xFFFFFFF0LL : valid_bytes);
  op.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)lim, 0x00020000);
  op.row_stride = (uint32_t)row_stride_bytes;
  return op;
}

// Byte offset of (row r, logical 16-byte chunk c) inside an LDS tile.
template <int ROWB = 128>
__device__ __forceinline__ int swz(int r, int c) {
  constexpr int RPL = 256 / ROWB, SLOTS = ROWB / 16;
  return r * ROWB + ((c ^ ((r / RPL) & (SLOTS - 1))) << 4);
}

// Issue the loads of an R x (ROWB/2) tile (K columns [k0, k0 + ROWB/2)) into
// `tile`, shared by the NW waves of the workgroup.
template <int R, int ROWB = 128, int NW = 4>
__device__ __forceinline__ void load_tile(const Operand& op, int k0, bf16* tile, int wave, int lane) {
  constexpr int LPR = ROWB / 16;        // lanes per row
  constexpr int RPI = 64 / LPR;         // rows per wave instruction (1 KB)
  constexpr int PER_WAVE = R / (NW * RPI);
  static_assert(R % (NW * RPI) == 0, "tile rows");
  const int rr = lane / LPR;
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int blk = wave * PER_WAVE + j;
    const int r = blk * RPI + rr;
    const int c = (lane % LPR) ^ ((r / (256 / ROWB)) & (LPR - 1));  // chunk that belongs in this slot
    const uint32_t voff = (uint32_t)r * op.row_stride + (uint32_t)k0 * 2u + (uint32_t)c * 16u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(op.rsrc, (lds_ptr_t)(tile + blk * RPI * (ROWB / 2)), 16, voff, 0, 0,
                                             kLoadAux);
  }
}

// The wave-instructions [j0, j0 + jn) of load_tile, so that a stage's loads
// can be spread between the MFMAs of the previous stage.
template <int R, int ROWB = 128, int NW = 4>
__device__ __forceinline__ void load_tile_part(const Operand& op, int k0, bf16* tile, int wave, int lane, int j0,
                                               int jn) {
  constexpr int LPR = ROWB / 16, RPI = 64 / LPR, PER_WAVE = R / (NW * RPI);
  static_assert(R % (NW * RPI) == 0, "tile rows");
  const int rr = lane / LPR;
#pragma unroll
  for (int j = j0; j < j0 + jn && j < PER_WAVE; ++j) {
    const int blk = wave * PER_WAVE + j;
    const int r = blk * RPI + rr;
    const int c = (lane % LPR) ^ ((r / (256 / ROWB)) & (LPR - 1));
    const uint32_t voff = (uint32_t)r * op.row_stride + (uint32_t)k0 * 2u + (uint32_t)c * 16u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(op.rsrc, (lds_ptr_t)(tile + blk * RPI * (ROWB / 2)), 16, voff, 0, 0,
                                             kLoadAux);
  }
}

// Fragment-major operand: the matrix is stored as 1 KB MFMA B fragments,
// fragment (block n32 of 32 rows, k-step k16 of 16 K columns) at byte
// (n32 * row_stride) + k16 * 1024, lane l's 16 bytes at 16 * l (row l % 32,
// K columns 8 * (l / 32) .. +7 of the k-step).  A stage's B tile is then
// R/32 row blocks of ROWB/32 consecutive fragments; wave-instruction q of a
// stage copies fragment (q / KSTEPS, q % KSTEPS) to LDS byte 1024 * q, and the
// MFMA reads it back at 16 * lane, conflict-free and without a swizzle.
template <int R, int ROWB = 128, int NW = 4>
__device__ __forceinline__ void load_frag_part(const Operand& op, int k0, bf16* tile, int wave, int lane, int j0,
                                               int jn) {
  constexpr int KSTEPS = ROWB / 32, NI = R / 32 * KSTEPS, PER_WAVE = NI / NW;
  static_assert(NI % NW == 0, "fragment split");
#pragma unroll
  for (int j = j0; j < j0 + jn && j < PER_WAVE; ++j) {
    const int q = wave * PER_WAVE + j;
    const uint32_t voff = (uint32_t)(q / KSTEPS) * op.row_stride + (uint32_t)(k0 / 16 + q % KSTEPS) * 1024u +
                          (uint32_t)lane * 16u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(op.rsrc, (lds_ptr_t)(tile + q * 512), 16, voff, 0, 0, kLoadAux);
  }
}

// Fragment-major operand used transposed: a matrix W [K, N] stored in the
// fragment-major layout above with its K rows as the 32-row blocks (fragment
// (K/32, N/16) at (K/32) * row_stride + (N/16) KB, unit u = the 16 bytes at
// 16 u: row u % 32, columns 8 (u/32) .. +7), in a product that contracts over
// K.  A stage (KS = ROWB/2 rows of K, R columns of N) is 2 x R/16 fragments;
// wave-instruction q of a stage copies fragment (row block q % 2, column step
// s = q / 2) to LDS byte 1024 q with its units permuted: unit (row r, half h)
// goes to position (r ^ 4h ^ 8 (s & 1)) + 32 h, so that the transposing reads
// of 32 lanes (4 rows x 16 columns of two neighbouring column steps) fall on
// 32 distinct 8-byte bank pairs.
template <int R, int NW = 4>
__device__ __forceinline__ void load_fragT_part(const Operand& op, int k0, bf16* tile, int wave, int lane, int j0,
                                                int jn) {
  constexpr int NI = 2 * R / 16, PER_WAVE = NI / NW;
  static_assert(NI % NW == 0, "fragment split");
  const int h = lane >> 5;
#pragma unroll
  for (int j = j0; j < j0 + jn && j < PER_WAVE; ++j) {
    const int q = wave * PER_WAVE + j;
    const int s = q >> 1, b = q & 1;
    const int r = (lane & 31) ^ (4 * h) ^ (8 * (s & 1));
    const uint32_t voff = (uint32_t)(k0 / 32 + b) * op.row_stride + (uint32_t)s * 1024u + (uint32_t)(r + 32 * h) * 16u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(op.rsrc, (lds_ptr_t)(tile + q * 512), 16, voff, 0, 0, kLoadAux);
  }
}

// K-major operand: B[n, k] = X[k, n] for X row-major [K, ldx] (a product that
// contracts over X's rows, such as tokens).  A stage is KS = 64 rows of X by
// R = 256 columns, 512 bytes per LDS row, its 64-byte units XOR-swizzled by
// (row & 3); wave-instruction q of a stage fills LDS rows 2q and 2q + 1.
template <int R, int NW = 4>
__device__ __forceinline__ void load_kmaj_part(const Operand& op, int k0, bf16* tile, int wave, int lane, int j0,
                                               int jn) {
  static_assert(R == 256, "one 512-byte LDS row per K row");
  constexpr int NI = 64 * R * 2 / 1024, PER_WAVE = NI / NW;
  static_assert(NI % NW == 0, "load split");
#pragma unroll
  for (int j = j0; j < j0 + jn && j < PER_WAVE; ++j) {
    const int q = wave * PER_WAVE + j;
    const int r = 2 * q + (lane >> 5), u = ((lane & 31) >> 2) ^ (r & 3);
    const uint32_t voff = (uint32_t)(k0 + r) * op.row_stride + (uint32_t)(u * 64 + 16 * (lane & 3));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(op.rsrc, (lds_ptr_t)(tile + q * 512), 16, voff, 0, 0, kLoadAux);
  }
}

// Workgroup barrier that orders LDS only: waits for this wave's own LDS
// operations and meets the other waves, without draining its outstanding
// global stores or loads (the __syncthreads() fences would wait for both).
// Waves whose direct-to-LDS loads must be visible wait for them first.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most n (a run-time count) vector-memory operations of this
// wave are outstanding: the largest of a few fixed counts not above n (a
// smaller count only waits longer).
__device__ __forceinline__ void wait_vmcnt_at_most(int n) {
  if (n >= 63) wait_vmcnt<63>();
  else if (n >= 48) wait_vmcnt<48>();
  else if (n >= 36) wait_vmcnt<36>();
  else if (n >= 32) wait_vmcnt<32>();
  else if (n >= 24) wait_vmcnt<24>();
  else if (n >= 20) wait_vmcnt<20>();
  else if (n >= 16) wait_vmcnt<16>();
  else if (n >= 12) wait_vmcnt<12>();
  else if (n >= 8) wait_vmcnt<8>();
  else if (n >= 4) wait_vmcnt<4>();
  else wait_vmcnt<0>();
}

template <int ROWB = 128>
__device__ __forceinline__ bf16x8 ld_frag(const bf16* tile, int r, int c) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + swz<ROWB>(r, c));
}

// The fragment reads of one k-step of a stage in LDS: A rows arow0 + 32 mb
// + .., B_op rows (or columns) brow0 + 32 nb + .., for MB x NB blocks of
// 32x32 per operand.  BMODE: how B sits in LDS: 0 swizzled rows
// (load_tile), 1 fragment-major (load_frag_part), 2 transposed
// fragment-major (load_fragT_part, ROWB 128), 3 K-major rows
// (load_kmaj_part, ROWB 128, 256 columns).
template <int MB, int NB, int NOPS, int ROWB = 128, int BMODE = 0>
struct Frags {
  int t0 = 0, t1 = 0;  // BMODE 2: byte offsets within a stage's B tile
  int k3[NB];          // BMODE 3: byte offsets of each column block
  __device__ __forceinline__ Frags(int lane, int brow0) {
    static_assert(BMODE < 2 || ROWB == 128, "transposed operands: 64-row stages");
    const int hi = lane >> 5;
    // BMODE 2: lane (half h, group g = column step parity, row r, column
    // quarter cp) reads rows 8h + r (+4) of k-step kk, columns 4 cp .. +3 of
    // column step brow0/16 + 2 nb + g
    if constexpr (BMODE == 2) {
      const int g = (lane >> 4) & 1, r = (lane >> 2) & 3, cp = lane & 3, fh = cp >> 1;
      t0 = (brow0 / 16 + g) * 2048 + 16 * (8 * (hi ^ g) + r + 4 * fh + 32 * fh) + 8 * (cp & 1);
      t1 = t0 + 64 - 128 * fh;
    }
    // BMODE 3: lane reads rows 8h + (lane & 15) / 4 (+4) of k-step kk, the 8
    // bytes 8 (lane & 3) of 16-column half g of its 64-byte unit, that unit
    // stored at slot unit ^ (row & 3)
    if constexpr (BMODE == 3) {
      const int r = (lane >> 2) & 3, g = (lane >> 4) & 1;
      const int base = (8 * hi + r) * 512 + 32 * g + 8 * (lane & 3) + 2 * brow0;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) k3[nb] = base + 64 * (nb ^ r);
    }
  }
  // The A and B fragments of k-step kk of a stage in LDS.
  __device__ __forceinline__ void read(const bf16* lA, const bf16* const (&lB)[NOPS], int arow0, int brow0, int lane,
                                       int kk, bf16x8 (&a)[MB], bf16x8 (&b)[NOPS][NB]) const {
    typedef __attribute__((address_space(3))) short4_t* lp4;
    constexpr int KSTEPS = ROWB / 32;
    const int lr = lane & 31, c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) a[mb] = ld_frag<ROWB>(lA, arow0 + mb * 32 + lr, c);
#pragma unroll
    for (int o = 0; o < NOPS; ++o)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (BMODE == 1) {
          b[o][nb] = *reinterpret_cast<const bf16x8*>(lB[o] + ((brow0 / 32 + nb) * KSTEPS + kk) * 512 + lane * 8);
        } else if constexpr (BMODE == 2) {
          const char* tb = reinterpret_cast<const char*>(lB[o]) + nb * 4096 + (kk >> 1) * 1024 + (kk & 1) * 256;
          const short4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp4)(tb + t0));
          const short4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp4)(tb + t1));
          b[o][nb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
        } else if constexpr (BMODE == 3) {
          const char* tb = reinterpret_cast<const char*>(lB[o]) + kk * 16 * 512 + k3[nb];
          const short4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp4)tb);
          const short4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp4)(tb + 4 * 512));
          b[o][nb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          b[o][nb] = ld_frag<ROWB>(lB[o], brow0 + nb * 32 + lr, c);
        }
      }
  }
};

// acc[op][mb][nb] += A[arow0 + 32mb + .., :] * B_op[brow0 + 32nb + .., :]^T over one
// K stage.  MB x NB blocks of 32x32 per operand.  The fragments of k-step
// kk+1 are read from LDS while the MFMAs of k-step kk run, and hook(kk) (for
// instance a slice of the next stage's global loads) is issued before them.
// BMODE: how B sits in LDS: 0 swizzled rows (load_tile), 1 fragment-major
// (load_frag_part), 2 transposed fragment-major (load_fragT_part, ROWB 128),
// 3 K-major rows (load_kmaj_part, ROWB 128, 256 columns).
template <int MB, int NB, int NOPS, int ROWB = 128, int BMODE = 0, class Hook>
__device__ __forceinline__ void mma_stage(const bf16* lA, const bf16* const (&lB)[NOPS],
                                          floatx16 (&acc)[NOPS][MB][NB], int arow0, int brow0, int lane,
                                          Hook&& hook) {
  constexpr int KSTEPS = ROWB / 32;
  const Frags<MB, NB, NOPS, ROWB, BMODE> fr(lane, brow0);
  bf16x8 a[2][MB];
  bf16x8 b[2][NOPS][NB];
  fr.read(lA, lB, arow0, brow0, lane, 0, a[0], b[0]);
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    const int cur = kk & 1;
    hook(kk);
    if (kk + 1 < KSTEPS) fr.read(lA, lB, arow0, brow0, lane, kk + 1, a[cur ^ 1], b[cur ^ 1]);
    // Keep the compiler from sinking the reads of k-step kk+1 below the
    // MFMAs of k-step kk (it otherwise reuses one fragment set and waits on
    // every read right before its use).
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int o = 0; o < NOPS; ++o)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[o][mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[cur][mb], b[cur][o][nb], acc[o][mb][nb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int MB, int NB, int NOPS, int ROWB = 128>
__device__ __forceinline__ void mma_stage(const bf16* lA, const bf16* const (&lB)[NOPS],
                                          floatx16 (&acc)[NOPS][MB][NB], int arow0, int brow0, int lane) {
  mma_stage<MB, NB, NOPS, ROWB, 0>(lA, lB, acc, arow0, brow0, lane, [](int) {});
}

// Zero the K columns of an LDS tile (rows [0, R)) outside [klo, khi), both
// relative to the stage start.  Used for partial token stages.
template <int R, int ROWB = 128, int NT = kThreads>
__device__ __forceinline__ void mask_tile_k(bf16* tile, int klo, int khi, int tid) {
  constexpr int KS = ROWB / 2;
  for (int e = tid; e < R * KS; e += NT) {
    const int r = e / KS, k = e - r * KS;
    if (k < klo || k >= khi) {
      bf16* p = reinterpret_cast<bf16*>(reinterpret_cast<char*>(tile) + swz<ROWB>(r, k >> 3)) + (k & 7);
      *p = (bf16)0.0f;
    }
  }
}

template <int NOPS, int MB, int NB>
__device__ __forceinline__ void zero(floatx16 (&acc)[NOPS][MB][NB]) {
#pragma unroll
  for (int o = 0; o < NOPS; ++o)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[o][mb][nb][j] = 0.0f;
}

}  // namespace core
}  // namespace ipttt

namespace ipttt {
namespace core {

// One workgroup tile C[BM x BN] (per B operand) += A[BM x K] B_o[BN x K]^T for
// K a multiple of KS = ROWB/2, with NW waves (8, or 4 for one wave per SIMD)
// in an (NW/2) x 2 grid: wave w owns rows (w/2)*MB*32 .. +MB*32 and columns
// (w%2)*NB*32 .. +NB*32 of every product.  NBUF LDS buffers form a ring: up to
// NBUF-1 stages' loads are in flight while one stage is multiplied, and the
// loads of each new stage are spread over the k-steps of the current one.
template <int BM, int BN, int NOPS, int MB, int NB, int ROWB = 128, int NBUF = 2, int BMODE = 0, int NW_ = 8>
struct Tile8 {
  static constexpr int NW = NW_, NT = NW * 64;
  static constexpr int KS = ROWB / 2, RPI = 1024 / ROWB, KSTEPS = ROWB / 32;
  static constexpr int SA = BM * KS, SB = BN * KS, STAGE = SA + NOPS * SB;
  static constexpr int LDS_ELEMS = NBUF * STAGE;
  static constexpr int NA = BM / (NW * RPI), NBI = BN / (NW * RPI);  // load instructions per wave
  static constexpr int NLOAD = NA + NOPS * NBI;
  static_assert(NW == 8 || NW == 4, "wave count");
  static_assert(BM == (NW / 2) * MB * 32 && BN == 2 * NB * 32, "wave grid");
  static_assert(BM % (NW * RPI) == 0 && BN % (NW * RPI) == 0, "load split");
  static_assert(NBUF >= 2 && NBUF <= 4, "ring depth: the waits cover at most two later stages");

  // Issue load instructions [q0, q1) of this wave's list for stage s, into
  // ring buffer (s + base) % NBUF.
  static __device__ __forceinline__ void issue(const Operand& oa, const Operand (&ob)[NOPS], bf16* lds, int s,
                                               int q0, int q1, int wave, int lane, int base = 0) {
    bf16* buf = lds + ((s + base) % NBUF) * STAGE;
    const int k0 = s * KS;
#pragma unroll
    for (int q = 0; q < NLOAD; ++q) {
      if (q < q0 || q >= q1) continue;
      if (q < NA) {
        load_tile_part<BM, ROWB, NW>(oa, k0, buf, wave, lane, q, 1);
      } else {
        const int o = (q - NA) / NBI, j = (q - NA) % NBI;
        if constexpr (BMODE == 1)
          load_frag_part<BN, ROWB, NW>(ob[o], k0, buf + SA + o * SB, wave, lane, j, 1);
        else if constexpr (BMODE == 2)
          load_fragT_part<BN, NW>(ob[o], k0, buf + SA + o * SB, wave, lane, j, 1);
        else if constexpr (BMODE == 3)
          load_kmaj_part<BN, NW>(ob[o], k0, buf + SA + o * SB, wave, lane, j, 1);
        else
          load_tile_part<BN, ROWB, NW>(ob[o], k0, buf + SA + o * SB, wave, lane, j, 1);
      }
    }
  }

  // The first NBUF-1 stages of a product, issued ahead (a persistent kernel
  // calls this for its next tile before writing out the current one).
  static __device__ __forceinline__ void prefetch(const Operand& oa, const Operand (&ob)[NOPS], int K, bf16* lds,
                                                  int wave, int lane, int base) {
    const int S = K / KS;
    for (int s = 0; s < NBUF - 1 && s < S; ++s) issue(oa, ob, lds, s, 0, NLOAD, wave, lane, base);
  }

  // acc += the whole K loop.  Stage s lives in ring buffer (s + base) % NBUF;
  // with pre, the first NBUF-1 stages were already issued by prefetch().  The
  // next product's base is (base + K/KS) % NBUF, and buffer
  // (base + K/KS - 1) % NBUF, the last one read, is free once this returns.
  static __device__ __forceinline__ void run(const Operand& oa, const Operand (&ob)[NOPS], int K, bf16* lds,
                                             floatx16 (&acc)[NOPS][MB][NB], int wave, int lane, int base = 0,
                                             bool pre = false) {
    const int wm = wave >> 1, wn = wave & 1;
    const int S = K / KS;
    if (!pre) prefetch(oa, ob, K, lds, wave, lane, base);
    for (int s = 0; s < S; ++s) {
      // stage s has landed once at most the later issued stages are pending
      const int later = min(NBUF - 2, S - 1 - s);
      if (later >= 2) wait_vmcnt<2 * NLOAD>();
      else if (later == 1) wait_vmcnt<NLOAD>();
      else wait_vmcnt<0>();
      __syncthreads();
      const bf16* buf = lds + ((s + base) % NBUF) * STAGE;
      const bf16* lB[NOPS];
#pragma unroll
      for (int o = 0; o < NOPS; ++o) lB[o] = buf + SA + o * SB;
      const int sn = s + NBUF - 1;  // the stage whose buffer was freed by this barrier
      const bool more = sn < S;
      mma_stage<MB, NB, NOPS, ROWB, BMODE>(buf, reinterpret_cast<const bf16* const(&)[NOPS]>(lB), acc, wm * MB * 32,
                                    wn * NB * 32, lane, [&](int kk) {
                                      if (more)
                                        issue(oa, ob, lds, sn, (kk * NLOAD) / KSTEPS,
                                              ((kk + 1) * NLOAD) / KSTEPS, wave, lane, base);
                                    });
    }
    __syncthreads();
  }
};


// The Tile8 product on a ring of five half-stage slots instead of two whole
// stages, for products whose operands stream from HBM.  A stage's B part
// (its NOPS B tiles) and its A part each fill one slot of SA elements (SA ==
// NOPS * SB); half h of the sequence B0 A0 B1 A1 B2 ... (stage h / 2, B when
// h is even) lives in slot h % 5.  While stage s is multiplied, stage s+1 and
// the B part of stage s+2 are in flight: the barrier at the top of stage s
// frees the slots of stage s-1, which then take A of stage s+1 (during
// k-steps 0 and 1) and B of stage s+2 (k-steps 2 and 3).  A B tile thus has
// two stages to arrive and an A tile one, in 160 KB of LDS, where two whole
// stages give every tile one.  Non-persistent: the ring starts empty and is
// drained when run() returns.
template <int BM, int BN, int NOPS, int MB, int NB, int BMODE = 0>
struct Tile8H {
  typedef Tile8<BM, BN, NOPS, MB, NB, 128, 2, BMODE> Base;
  static constexpr int NW = 8, NT = NW * 64, KS = 64;
  static constexpr int SA = Base::SA, SB = Base::SB, SLOT = SA, NSLOT = 5;
  static constexpr int LDS_ELEMS = NSLOT * SLOT;
  static constexpr int NA = Base::NA, NBL = NOPS * Base::NBI;  // load instructions per wave: A part, B part
  static_assert(SA == NOPS * SB, "equal half-stage slots");
  static_assert(Base::KSTEPS == 4 && NA % 2 == 0 && NBL % 2 == 0, "two k-steps per part");

  // Load instructions [q0, q1) of this wave's list for half h, if its stage
  // exists (same: the A halves are not loaded).
  static __device__ __forceinline__ void issue_half(const Operand& oa, const Operand (&ob)[NOPS], bf16* lds, int h,
                                                    int S, int q0, int q1, int wave, int lane, bool same) {
    const int s = h >> 1;
    if (s >= S || ((h & 1) && same)) return;
    bf16* slot = lds + (h % NSLOT) * SLOT;
    const int k0 = s * KS;
    if (h & 1) {
#pragma unroll
      for (int q = 0; q < NA; ++q)
        if (q >= q0 && q < q1) load_tile_part<BM, 128, NW>(oa, k0, slot, wave, lane, q, 1);
    } else {
#pragma unroll
      for (int q = 0; q < NBL; ++q) {
        if (q < q0 || q >= q1) continue;
        const int o = q / Base::NBI, j = q % Base::NBI;
        if constexpr (BMODE == 1)
          load_frag_part<BN, 128, NW>(ob[o], k0, slot + o * SB, wave, lane, j, 1);
        else if constexpr (BMODE == 2)
          load_fragT_part<BN, NW>(ob[o], k0, slot + o * SB, wave, lane, j, 1);
        else if constexpr (BMODE == 3)
          load_kmaj_part<BN, NW>(ob[o], k0, slot + o * SB, wave, lane, j, 1);
        else
          load_tile_part<BN, 128, NW>(ob[o], k0, slot + o * SB, wave, lane, j, 1);
      }
    }
  }

  // acc += the whole K loop (K a multiple of 64); the LDS is free again on
  // return.  same (one B operand, in A's row layout: BM == BN, BMODE 0): A
  // is that operand too, so only the B halves are loaded and the A fragments
  // are read from them; the waits are unchanged, since a stage's B half was
  // the part that arrived last.
  static __device__ __forceinline__ void run(const Operand& oa, const Operand (&ob)[NOPS], int K, bf16* lds,
                                             floatx16 (&acc)[NOPS][MB][NB], int wave, int lane, bool same = false) {
    const int wm = wave >> 1, wn = wave & 1;
    const int S = K / KS;
    for (int h = 0; h < 3; ++h) issue_half(oa, ob, lds, h, S, 0, NA + NBL, wave, lane, same);
    for (int s = 0; s < S; ++s) {
      // Halves 2s and 2s+1 have landed once at most half 2s+2 (B of stage
      // s+1) is pending: the counter retires this wave's loads in order.
      if (s + 1 < S) wait_vmcnt<NBL>();
      else wait_vmcnt<0>();
      // LDS-only barrier: __syncthreads() would also wait for the loads
      // left in flight on purpose
      lds_barrier();
      const bf16* lb = lds + ((2 * s) % NSLOT) * SLOT;
      const bf16* la = same ? lb : lds + ((2 * s + 1) % NSLOT) * SLOT;
      const bf16* lB[NOPS];
#pragma unroll
      for (int o = 0; o < NOPS; ++o) lB[o] = lb + o * SB;
      mma_stage<MB, NB, NOPS, 128, BMODE>(la, reinterpret_cast<const bf16* const(&)[NOPS]>(lB), acc, wm * MB * 32,
                                          wn * NB * 32, lane, [&](int kk) {
                                            if (kk < 2)
                                              issue_half(oa, ob, lds, 2 * s + 3, S, kk * NA / 2, (kk + 1) * NA / 2,
                                                         wave, lane, same);
                                            else
                                              issue_half(oa, ob, lds, 2 * s + 4, S, (kk - 2) * NBL / 2,
                                                         (kk - 1) * NBL / 2, wave, lane, same);
                                          });
    }
    __syncthreads();
  }
};

}  // namespace core
}  // namespace ipttt
