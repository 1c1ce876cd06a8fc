// Document/chunk descriptors on the device (integer, bit-exact).
//
// One byte per token: bit 7 = the token starts a document (every row start
// does, unless the row continues a document of the previous call), bits 0-2 = number of conv taps it reads, min(5, end(t) - t), where
// end(t) = min(chunk end, next document start, T).  Plus, per (row, chunk),
// the triple (r0, l0, carry) that drives the reset in the scan: resets at
// document boundaries (iplexlaw.co.kr In-Place TTT review, section 6) on the
// fixed chunk grid of lijianxiong.blog "In-Place Test-Time Training",
// 高效的块状更新机制.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace ipttt {

__global__ __launch_bounds__(256) void seg_init_kernel(uint8_t* __restrict__ segs, int64_t n, int64_t T) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) segs[t] = (t % T == 0) ? 0x80 : 0;
}

__global__ __launch_bounds__(64) void seg_mark_kernel(uint8_t* __restrict__ segs, StartBatch s, uint8_t value) {
  for (int k = threadIdx.x; k < s.n; k += blockDim.x) segs[s.v[k]] = value;
}

// One block per (row, chunk).  Only bit 7 of neighbouring bytes is read while
// other blocks rewrite their low bits, and every writer keeps bit 7, so the
// reads are stable.
__global__ __launch_bounds__(256) void seg_finish_kernel(uint8_t* __restrict__ segs, int32_t* __restrict__ table,
                                                         int64_t T, int C, int N) {
  const int bc = blockIdx.x;
  const int b = bc / N, i = bc - b * N;
  const int64_t lo = (int64_t)b * T + (int64_t)i * C;
  const int L = (int)min((int64_t)C, T - (int64_t)i * C);
  __shared__ int s_first, s_last;
  if (threadIdx.x == 0) { s_first = L; s_last = 0; }
  __syncthreads();
  int first = L, last = 0;
  for (int c = threadIdx.x; c < L; c += blockDim.x) {
    const uint8_t me = segs[lo + c];
    if (me & 0x80) { first = min(first, c); last = max(last, c); }
    int n = 1;
    while (n < 5 && c + n < L && !(segs[lo + c + n] & 0x80)) ++n;
    segs[lo + c] = (uint8_t)((me & 0x80) | n);
  }
  atomicMin(&s_first, first);
  atomicMax(&s_last, last);
  __syncthreads();
  if (threadIdx.x == 0 && table != nullptr) {
    const bool has_next = i + 1 < N;
    const int carry = has_next ? !(segs[lo + L] & 0x80) : 0;
    table[bc * 3 + 0] = s_first;
    table[bc * 3 + 1] = s_last;
    table[bc * 3 + 2] = carry;
  }
}

// The same descriptors in one launch, when the listed tokens fit in one
// batch: entry v >= 0 is a document start at token v, entry v < 0 says that
// row start -v-1 continues a document (starts nothing unless also listed as
// a start).  One block per (row, chunk) writes only its chunk's bytes: the
// row-start flag, then the listed starts inside the chunk (each entry looked
// at once per block), then the tap counts; whether the next chunk's first
// token starts a document (carry) is read off the list, not from memory
// another block writes.
__global__ __launch_bounds__(256) void seg_build_kernel(uint8_t* __restrict__ segs, int32_t* __restrict__ table,
                                                        StartBatch s, int64_t T, int C, int N) {
  const int bc = blockIdx.x;
  const int b = bc / N, i = bc - b * N;
  const int64_t lo = (int64_t)b * T + (int64_t)i * C;
  const int L = (int)min((int64_t)C, T - (int64_t)i * C);
  __shared__ int s_cont, s_next, s_first, s_last;
  if (threadIdx.x == 0) { s_cont = 0; s_next = 0; s_first = L; s_last = 0; }
  __syncthreads();
  for (int k = threadIdx.x; k < s.n; k += blockDim.x) {
    const int64_t v = s.v[k];
    if (i == 0 && v == -lo - 1) s_cont = 1;  // this row continues a document
    if (v == lo + L) s_next = 1;             // the next chunk starts with a listed start
  }
  __syncthreads();
  const bool row_start = i == 0 && !s_cont;
  for (int c = threadIdx.x; c < L; c += blockDim.x) segs[lo + c] = (c == 0 && row_start) ? 0x80 : 0;
  __syncthreads();
  for (int k = threadIdx.x; k < s.n; k += blockDim.x) {
    const int64_t v = s.v[k];
    if (v >= lo && v < lo + L) segs[v] = 0x80;
  }
  __syncthreads();
  // only bit 7 of neighbouring bytes is read while their low bits are
  // rewritten, and every writer keeps bit 7
  int first = L, last = 0;
  for (int c = threadIdx.x; c < L; c += blockDim.x) {
    const uint8_t me = segs[lo + c];
    if (me & 0x80) { first = min(first, c); last = max(last, c); }
    int n = 1;
    while (n < 5 && c + n < L && !(segs[lo + c + n] & 0x80)) ++n;
    segs[lo + c] = (uint8_t)((me & 0x80) | n);
  }
  atomicMin(&s_first, first);
  atomicMax(&s_last, last);
  __syncthreads();
  if (threadIdx.x == 0 && table != nullptr) {
    table[bc * 3 + 0] = s_first;
    table[bc * 3 + 1] = s_last;
    // a chunk that is not its row's last ends before the next row start
    table[bc * 3 + 2] = i + 1 < N ? !s_next : 0;
  }
}

hipError_t launch_segments(const Prob& p, const int64_t* starts, int64_t n_starts, const uint8_t* continues,
                           uint8_t* segs, int32_t* table, hipStream_t st) {
  const int64_t n = p.M;
  note_launch("segments", st);
  int64_t n_cont = 0;
  if (continues != nullptr)
    for (int64_t b = 0; b < p.B; ++b) n_cont += continues[b] ? 1 : 0;
  if (n_starts + n_cont <= StartBatch::kMax) {
    StartBatch s;
    s.n = 0;
    if (continues != nullptr)
      for (int64_t b = 0; b < p.B; ++b)
        if (continues[b]) s.v[s.n++] = -(b * p.T) - 1;
    for (int64_t k = 0; k < n_starts; ++k) s.v[s.n++] = starts[k];
    seg_build_kernel<<<(unsigned)(p.B * p.N), 256, 0, st>>>(segs, table, s, p.T, p.C, p.N);
    return hipGetLastError();
  }
  seg_init_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(segs, n, p.T);
  // Rows that continue a document of the previous call: their first token
  // starts nothing (unless listed below).
  if (continues != nullptr) {
    StartBatch s;
    s.n = 0;
    for (int64_t b = 0; b < p.B; ++b) {
      if (continues[b]) s.v[s.n++] = b * p.T;
      if (s.n == StartBatch::kMax || (b + 1 == p.B && s.n > 0)) {
        seg_mark_kernel<<<1, 64, 0, st>>>(segs, s, 0);
        s.n = 0;
      }
    }
  }
  for (int64_t k = 0; k < n_starts; k += StartBatch::kMax) {
    StartBatch s;
    s.n = (int)min((int64_t)StartBatch::kMax, n_starts - k);
    for (int q = 0; q < s.n; ++q) s.v[q] = starts[k + q];
    seg_mark_kernel<<<1, 64, 0, st>>>(segs, s, 0x80);
  }
  seg_finish_kernel<<<(unsigned)(p.B * p.N), 256, 0, st>>>(segs, table, p.T, p.C, p.N);
  return hipGetLastError();
}

}  // namespace ipttt
