// Shared device helpers of the In-Place TTT kernels (gfx950 / CDNA4).
//
// Every contraction of the layer is run as an "NT" product on the matrix
// cores: both operands are stored K-contiguous (row-major A[M][K], B[N][K]),
// staged through LDS in 128-byte K slices, and multiplied with
//   bf16: v_mfma_f32_32x32x16_bf16 (8 bf16 of K per lane and operand)
//   fp32: v_mfma_f32_32x32x2_f32   (1 fp32 of K per lane and operand; exact
//         fp32 products, no reduced-precision inputs)
// A workgroup has 4 wave64s in a 2x2 arrangement; each wave owns a
// (BM/2) x (BN/2) block of 32x32 MFMA tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ipttt {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves of 64 lanes

template <typename T> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int KG = 16;   // K consumed by one MFMA
  static constexpr int EPL = 8;   // K elements each lane supplies per operand
  typedef bf16x8 frag;
  static __device__ __forceinline__ frag ld(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
  static __device__ __forceinline__ floatx16 mma(frag a, frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int KG = 2;
  static constexpr int EPL = 1;
  typedef float frag;
  static __device__ __forceinline__ frag ld(const float* p) { return *p; }
  static __device__ __forceinline__ floatx16 mma(frag a, frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }

// Geometry of one NT tile product.
template <typename T, int BM_, int BN_>
struct Geo {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int VE = 16 / sizeof(T);       // elements per 16-byte vector
  static constexpr int BK = 128 / sizeof(T);      // K per LDS stage (128 bytes/row)
  static constexpr int LDK = BK + VE;             // LDS row pitch, one vector of padding
  static constexpr int WM = BM / 2, WN = BN / 2;  // wave tile
  static constexpr int MB = WM / 32, NB = WN / 32;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tiles are multiples of 64");
};

// Row of 32x32 accumulator element j held by `lane`:
// row = 8*(j/4) + 4*(lane/32) + j%4, column = lane%32.
__device__ __forceinline__ int acc_row(int j, int lane) { return ((j >> 2) << 3) + ((lane >> 5) << 2) + (j & 3); }

// A [R x BK] slice of a K-contiguous matrix, moved global -> registers -> LDS
// in 16-byte vectors.  Rows >= nrows and K columns >= kend read as zero, so
// ragged edges need no special casing; kend must be a multiple of VE.
template <typename T, int R>
struct TileLoad {
  static constexpr int VE = 16 / sizeof(T);
  static constexpr int NV = R * 8 / kThreads;  // 8 vectors per 128-byte row
  static_assert(NV >= 1 && (R * 8) % kThreads == 0, "tile rows");
  u32x4 v[NV];

  __device__ __forceinline__ void load(const T* __restrict__ base, int64_t ld, int nrows, int k0,
                                       int kend, int tid) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int idx = tid + j * kThreads;
      const int r = idx >> 3, k = k0 + (idx & 7) * VE;
      if (r < nrows && k < kend)
        v[j] = *reinterpret_cast<const u32x4*>(base + (int64_t)r * ld + k);
      else
        v[j] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // Same, but K positions outside [klo, khi) read as zero element by element
  // (a select, so whatever the buffer holds there never reaches the product).
  __device__ __forceinline__ void load_kmask(const T* __restrict__ base, int64_t ld, int nrows,
                                             int k0, int klo, int khi, int tid) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int idx = tid + j * kThreads;
      const int r = idx >> 3, k = k0 + (idx & 7) * VE;
      u32x4 x = u32x4{0u, 0u, 0u, 0u};
      if (r < nrows && k < khi && k + VE > klo) {
        x = *reinterpret_cast<const u32x4*>(base + (int64_t)r * ld + k);
        if (k < klo || k + VE > khi) {
          T* e = reinterpret_cast<T*>(&x);
#pragma unroll
          for (int q = 0; q < VE; ++q)
            if (k + q < klo || k + q >= khi) e[q] = from_f32<T>(0.0f);
        }
      }
      v[j] = x;
    }
  }

  template <int LDK>
  __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int idx = tid + j * kThreads;
      const int r = idx >> 3, c = (idx & 7) * VE;
      *reinterpret_cast<u32x4*>(lds + r * LDK + c) = v[j];
    }
  }
};

// One LDS stage of C += A B^T for this wave's block.
template <typename T, class G>
__device__ __forceinline__ void stage_mma(const T* lA, const T* lB, floatx16 (&acc)[G::MB][G::NB],
                                          int wm, int wn, int lane) {
  typedef Mma<T> M;
  const int lr = lane & 31, lk = (lane >> 5) * M::EPL;
#pragma unroll
  for (int kk = 0; kk < G::BK / M::KG; ++kk) {
    typename M::frag a[G::MB], b[G::NB];
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
      a[mb] = M::ld(lA + (wm * G::WM + mb * 32 + lr) * G::LDK + kk * M::KG + lk);
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb)
      b[nb] = M::ld(lB + (wn * G::WN + nb * 32 + lr) * G::LDK + kk * M::KG + lk);
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) acc[mb][nb] = M::mma(a[mb], b[nb], acc[mb][nb]);
  }
}

template <class G>
__device__ __forceinline__ void zero_acc(floatx16 (&acc)[G::MB][G::NB]) {
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[mb][nb][j] = 0.0f;
}

// The hardware hands consecutive workgroup ids to the 8 XCDs in turn.  This
// maps them so that each XCD works on one contiguous range of logical tiles,
// which then share operands in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int pid, int G) {
  const int xcd = pid & 7, idx = pid >> 3;
  const int q = G >> 3, r = G & 7;
  const int base = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
  return base + idx;
}

// Logical tile id -> (tile_m, tile_n), walking GM rows of M tiles together so
// that neighbouring tiles reuse both operands.
__device__ __forceinline__ void grouped_tile(int t, int tiles_m, int tiles_n, int GM, int& tm, int& tn) {
  const int per_group = GM * tiles_n;
  const int g = t / per_group;
  const int first_m = g * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in = t - g * per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

// SiLU(x) = x * sigmoid(x) with the hardware reciprocal (about 1 ulp); for
// x -> -inf, exp(-x) overflows to +inf and the result goes to -0.
__device__ __forceinline__ float silu_f32(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

}  // namespace ipttt
