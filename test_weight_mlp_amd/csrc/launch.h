// Internal launchers of the In-Place TTT kernels, called by the C ABI layer.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace ipttt {

// Calls the caller's launch hook, if one is set (ipttt_set_launch_hook),
// with the name of the kernel (or group of small kernels) enqueued next.
void note_launch(const char* kernel, hipStream_t st);

// A validated problem in the form the kernels use.
struct Prob {
  int64_t B, T, M;  // rows, tokens per row, B*T
  int d, f;         // d_model, d_ff
  int C;            // chunk length, min(C, T)
  int N;            // chunks per row
  int Cp;           // pitch of the chunk-transposed copies: C rounded up to 8
  int dtype;        // 0 = fp32, 1 = bf16
  int target;       // 0: Conv1D(X0) W_target, 1: X0 W_target, 2: Conv1D(X0)
};

// bf16 with d_model and d_ff multiples of 64 runs the 8-wave kernels: the
// scan reads Z and V_hat in their row layouts and hands the apply its
// per-chunk weights as MFMA fragments.  Everything else runs the general
// kernels, whose scan reads chunk-transposed copies of Z and V_hat and
// writes row-major weights.
// The 8-wave kernels address through 32-bit buffer offsets: one row's d x f
// state (fp32), and the rows of one chunk of Z and V_hat (a chunk's operand
// resource starts at its first token, and a stage's offset runs up to
// (C + 64) rows of max(d, f) bf16).  Larger shapes take the general kernels,
// which index in 64 bits.
inline bool fast_scan(const Prob& p) {
  const int64_t w = p.d > p.f ? p.d : p.f;
  return p.dtype == 1 && p.d % 64 == 0 && p.f % 64 == 0 && (int64_t)p.d * p.f * 4 < (int64_t(1) << 31) &&
         ((int64_t)p.C + 64) * w * 2 < (int64_t(1) << 31);
}

// Document starts passed by value (kernel arguments), so that building the
// descriptors needs no host-to-device copy.
struct StartBatch {
  static constexpr int kMax = 384;
  int n;
  int64_t v[kMax];
};

// continues: host flags per row, or NULL (see ipttt_problem).
hipError_t launch_segments(const Prob& p, const int64_t* starts, int64_t n_starts, const uint8_t* continues,
                           uint8_t* segs, int32_t* table, hipStream_t st);
// GU: NULL, or [2, M, f] dtype receiving G = H W_gate^T then U = H W_up^T.
hipError_t launch_gated_z(const Prob& p, const void* H, const void* Wg, const void* Wu, void* Z, void* GU,
                          hipStream_t st);
// scratch: d*d + 5*d elements (transposed W_target and conv weights)
hipError_t launch_target(const Prob& p, const void* X0, const void* convw, const void* Wt,
                         const uint8_t* segs, void* V, void* scratch, hipStream_t st);
// Clip scales.  partials: B*N*gram_pairs(p) floats (every one written);
// scratch: gram_scratch_bytes(p, B*N) bytes (the stored V V^T tiles of the
// 8-wave Gram path; none on the general path).
int gram_pairs(const Prob& p);
size_t gram_scratch_bytes(const Prob& p, int64_t chunks);
hipError_t launch_alpha(const Prob& p, const void* V, const void* Z, const int32_t* table,
                        float eta, float tau, float* alpha, float* partials, void* scratch, hipStream_t st);
// fast_scan(p) only: the Gram partial sums of chunks [c0, c1) (flat row-major
// chunk indices), with Gv holding gram_scratch_bytes(p, c1 - c0) bytes; then
// launch_alpha_only turns the partials of every chunk into clip scales.
hipError_t launch_gram_fast(const Prob& p, const void* V, const void* Z, const int32_t* table, float* partials,
                            float* Gv, int64_t c0, int64_t c1, hipStream_t st);
hipError_t launch_alpha_only(const Prob& p, const float* partials, float eta, float tau, float* alpha,
                             hipStream_t st);
// Chunk-transposed copy of a [B*T, F] tensor: out[((b*N + i)*F + j)*Cp + c]
// = in[(b*T + i*C + c)*F + j]; offsets c >= the chunk's length are not written.
hipError_t launch_chunk_transpose(const Prob& p, const void* in, int F, void* out, hipStream_t st);
hipError_t launch_dw(const Prob& p, const void* Vt, const void* Zt, const int32_t* table,
                     const float* alpha, float eta, float* dW, hipStream_t st);
// fast_scan(p): Z, V row-major; Vs (B*T*d scratch) receives alpha * eta * V,
// Wbuf B*N fragment-major weights and Wdfrag W_down in the same layout (Zt,
// Vt unused).  Otherwise: Zt, Vt are chunk-transposed copies and Wbuf
// receives B*N row-major weights (Wdfrag, Vs unused).
// carry: the state is S alone (fp32, [B, d, f] row-major like Sin and Sout),
// started from Sin[b] in rows whose chunk 0 has r0 > 0 (Sin may be NULL:
// zeros), and each emitted weight is W_down + S rounded once; Sout (or NULL)
// receives each row's final state, the last chunk's update included.
// Otherwise the registers hold W_down + S and Sin, Sout are unused.
// fast_scan(p) only: row0 and nrows (< 0: every row) restrict the launch to
// rows [row0, row0 + nrows) of the problem; Wbuf and Vs then hold those rows
// only (row row0 first), while the table, Z, V, alpha, Sin, Sout and O keep
// every row.  i0 and i1 (< 0: N) restrict it to the chunk window [i0, i1):
// Wbuf and Vs then hold those chunks of the launch's one row (nrows = 1 is
// required), chunk i0 first; a window that starts after chunk 0 or ends
// before chunk N carries the row's fp32 state through Rst ([d, f], required
// then, ignored otherwise).
hipError_t launch_scan(const Prob& p, const void* Z, const void* V, const void* Zt, const void* Vt,
                       const void* Wd, const int32_t* table, const float* alpha, float eta, void* Wbuf,
                       void* Wdfrag, void* Vs, bool carry, const float* Sin, float* Sout, hipStream_t st,
                       int row0 = 0, int nrows = -1, int i0 = 0, int i1 = -1, float* Rst = nullptr);
// Rows and chunk window as for launch_scan (fast_scan(p) only), with Wbuf the
// window's weights as that launch wrote them.
hipError_t launch_apply(const Prob& p, const void* Z, const void* Wbuf, const void* Wd, const void* Wdfrag,
                        const int32_t* table, void* O, hipStream_t st, int row0 = 0, int nrows = -1, int i0 = 0,
                        int i1 = -1);

// The allocation-free call's static scratch on the current device (its
// address there, looked up on the device's first use; noalloc.hip).
hipError_t noalloc_scratch(void** ptr);

// ---- backward

// General scan of the forward (R = W_down + S) writing the per-chunk weights
// transposed, [f, d] per chunk, from chunk-transposed Zt and Vt.
hipError_t launch_scan_transposed(const Prob& p, const void* Zt, const void* Vt, const void* Wd,
                                  const int32_t* table, const float* alpha, float eta, void* WbufT, hipStream_t st);
// Reverse scan: dDW ([d, f] per chunk) and dDWt ([f, d]) for carrying chunks,
// Wpart [B, d, f] fp32 the per-row W_down gradient.
hipError_t launch_rscan(const Prob& p, const void* dOt, const void* Zt, const int32_t* table, void* dDW, void* dDWt,
                        float* Wpart, hipStream_t st);

// fast_scan(p): the reverse scan on the 8-wave core from row-layout Z and
// dO: dDW fragment-major per chunk (the layout of the forward's weights) and
// Wpart [B, d, f] fp32, the per-row W_down gradients (overwritten).
hipError_t launch_rscan_fast(const Prob& p, const void* Z, const void* dO, const int32_t* table, void* dDW,
                             float* Wpart, hipStream_t st);

// C_q[m, n] = sum_t A_q[t, m] B_q[t, n] over M tokens, fp32 out, for nprod
// (1 or 2) products of the same shapes; bf16, A [M, ma], B [M, nb] row-major,
// ma and nb multiples of 64.  With splits > 1 the tokens are cut into that
// many slices and C_q receives splits consecutive [ma, nb] partial products
// (each slice must hold a token: hipErrorInvalidValue otherwise).
hipError_t launch_tn_fast(int nprod, const void* const* A, const void* const* B, float* const* C, int64_t M,
                          int ma, int nb, int splits, hipStream_t st);
// The token slices in [1, min(8, cap)] that finish such a product soonest
// on this device (one workgroup per CU; at least 1024 tokens a slice).
int tn_fast_splits(int nprod, int64_t M, int ma, int nb, int cap);

// Rows of a chunk a batched product covers (NTArgs::rows).
// HEADZ (8-wave path only): as HEAD, but a chunk whose first document starts
// at its first token (r0 = 0) runs all its rows, pair 0 reading
// NTArgs::tail_B; TAILNZ: as TAIL for the other chunks only.
enum { NT_ROWS_ALL = 0, NT_ROWS_HEAD = 1, NT_ROWS_TAIL = 2, NT_ROWS_SEG = 3, NT_ROWS_HEADZ = 4, NT_ROWS_TAILNZ = 5 };

// One operand pair of a batched product: A [m, k] and B [n, k], dtype,
// K-contiguous rows.  tok: the operand is a [tokens, ld] matrix and row m of
// batch z is token tok0(z) + m (chunked products only); otherwise row m of
// batch z is at z * stride + m * ld.
struct NTPair {
  const void *A = nullptr, *B = nullptr;
  int64_t lda = 0, ldb = 0, sa = 0, sb = 0;
  int a_tok = 0, b_tok = 0;
  // B in the fragment-major layout of the forward's chunk weights (rows n,
  // K-steps of 16): a per-batch matrix of N rows (8-wave path only)
  int b_frag = 0;
  // B = W^T for W [K, ldb] in that fragment-major layout (K/32 blocks of
  // ldb/16 fragments), per batch: the product contracts over W's rows
  // (8-wave path only)
  int b_fragt = 0;
  // B = X^T for X [K, ldb] row-major, contracting over X's rows: with b_tok
  // the batch's chunk rows of a token-addressed X (rows past the chunk read
  // as zero; chunked products), else the batch's matrix at z * sb (8-wave
  // path only)
  int b_kmaj = 0;
  int K = 0;
};

// C[m, n] = a0 ca[z] sum_pairs sum_k A[m, k] B[n, k] + x0 cx[z] X[m, n].
// chunked: batch z is (row, chunk) z of the problem, m a chunk-relative
//   token; rows restricts m (NT_ROWS_*; SEG = [l0, L) of carrying chunks),
//   kseg restricts K to [l0, L), nseg restricts n to [l0, L).
// Otherwise batch z has M rows.  The output C (and X) is addressed like a
// tok or per-batch operand by c_tok, ldc, sc; c_f32 selects float output.
struct NTArgs {
  NTPair pr[3];
  int npairs = 1;
  void* C = nullptr;
  int64_t ldc = 0, sc = 0;
  int c_tok = 0, c_f32 = 0;
  const float* X = nullptr;
  const float *ca = nullptr, *cx = nullptr;
  // NT_ROWS_HEADZ: pair 0's B for chunks with r0 = 0, one matrix for every
  // batch (stride 0), laid out like pair 0's B
  const void* tail_B = nullptr;
  float a0 = 1.0f, x0 = 1.0f;
  int M = 0, N = 0;
  int chunked = 0, rows = NT_ROWS_ALL, kseg = 0, nseg = 0;
  // With kseg: the operands hold zeros at every K position outside
  // [l0, L), so the product may run over all of K.
  int kzero = 0;
};
hipError_t launch_nt(const Prob& p, const NTArgs& a, int batches, const int32_t* table, hipStream_t st);

constexpr int kDotParts = 8;    // partial sums per chunk of seg_dot_scale_kernel
constexpr int kConvParts = 1024; // token slices of the conv weight gradient

// out[c * Rp + r] = in[r * Cc + c], zero rows R <= r < Rp.
hipError_t launch_transpose_pad(const Prob& p, const void* in, int64_t R, int Cc, int64_t Rp, void* out,
                                hipStream_t st);
// out[e] = sum_{q < P} part[q * n + e]; part may be overwritten.
hipError_t launch_sum_parts(float* part, float* out, int64_t n, int P, hipStream_t st);
hipError_t launch_convert(const Prob& p, const void* in, void* out, int64_t n, bool to_dtype, hipStream_t st);
hipError_t launch_zero(void* ptr, size_t bytes, hipStream_t st);
// dots: kDotParts partial sums of <V, A> per chunk over its carried segment;
// Vc = eta alpha V there (carrying chunks), 0 on every other token (dtype).
hipError_t launch_seg_dot_scale(const Prob& p, const void* V, const float* A, const int32_t* table,
                                const float* alpha, float eta, float* dots, void* Vc, hipStream_t st);
hipError_t launch_coef(const Prob& p, const float* alpha, const float* gram, int npairs, const float* dots,
                       const int32_t* table, float eta, float tau, float* cpos, float* cneg, hipStream_t st);
hipError_t launch_gated_z_bwd(const Prob& p, const void* H, const void* Wg, const void* Wu, const void* dZ, void* dG,
                              void* dU, hipStream_t st);
// dG, dU from the saved G and U (GU as written by launch_gated_z), elementwise.
hipError_t launch_gated_grad(const Prob& p, const void* GU, const void* dZ, void* dG, void* dU, hipStream_t st);
// dX0 and the conv weight-gradient partials (part: kConvParts * d * 5 floats)
hipError_t launch_conv_bwd(const Prob& p, const float* dY, const void* X0, const void* convw, const uint8_t* segs,
                           void* dX0, float* part, hipStream_t st);
// Y = the conv of the target (tap counts from segs), dtype, [B*T, d];
// scratch as for launch_target.
hipError_t launch_conv_only(const Prob& p, const void* X0, const void* convw, const uint8_t* segs, void* Y,
                            void* scratch, hipStream_t st);

}  // namespace ipttt
