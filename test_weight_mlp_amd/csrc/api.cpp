// C ABI of the In-Place TTT layer forward: argument validation, the host
// segment table, workspace layout and the launch sequences.  Nothing is
// launched and nothing is written unless every argument checks out.
#include <cmath>
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "../../include/ipttt.h"
#include "launch.h"

using ipttt::Prob;

namespace {
// The caller's launch hook (a measurement aid), process-wide.
ipttt_launch_hook g_hook = nullptr;
void* g_hook_user = nullptr;
}  // namespace

namespace ipttt {
void note_launch(const char* kernel, hipStream_t st) {
  const ipttt_launch_hook h = g_hook;
  if (h != nullptr) h(kernel, static_cast<void*>(st), g_hook_user);
}
}  // namespace ipttt

namespace {

constexpr int64_t kMaxTokens = (int64_t(1) << 31) - 1;  // B*T fits a signed 32-bit grid index
constexpr int64_t kMaxDim = int64_t(1) << 20;
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;
// Launch grids carry rows, or (row, chunk) pairs, in their y dimension, which
// the device caps at 65536 blocks.
constexpr int64_t kMaxGridY = 65535;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

size_t elt_bytes(const Prob& p) { return p.dtype == IPTTT_BF16 ? 2 : 4; }

// Validates everything about the problem, fills the kernel view.
ipttt_status check_problem(const ipttt_problem* q, Prob* p) {
  if (q == nullptr) return IPTTT_ERR_NULL;
  if (q->dtype != IPTTT_F32 && q->dtype != IPTTT_BF16) return IPTTT_ERR_DTYPE;
  if (q->target < IPTTT_TARGET_LM || q->target > IPTTT_TARGET_NO_PROJ) return IPTTT_ERR_ARG;
  if (q->rows < 1 || q->seq_len < 1 || q->d_model < 1 || q->d_ff < 1 || q->chunk < 1)
    return IPTTT_ERR_SHAPE;
  if (q->d_model % 8 != 0 || q->d_ff % 8 != 0) return IPTTT_ERR_SHAPE;
  if (q->d_model > kMaxDim || q->d_ff > kMaxDim) return IPTTT_ERR_SHAPE;
  if (q->rows > kMaxTokens / q->seq_len) return IPTTT_ERR_SHAPE;
  Prob r;
  r.B = q->rows;
  r.T = q->seq_len;
  r.M = q->rows * q->seq_len;
  r.d = (int)q->d_model;
  r.f = (int)q->d_ff;
  r.C = (int)(q->chunk < q->seq_len ? q->chunk : q->seq_len);
  r.N = (int)((r.T + r.C - 1) / r.C);
  r.Cp = (r.C + 7) / 8 * 8;
  r.dtype = q->dtype;
  r.target = q->target;
  // Every grid must fit; the largest are the apply (per chunk x tile) and
  // the Gram (per chunk x tile pair) launches.
  const int64_t chunks = r.B * r.N;
  if (r.B > kMaxGridY || chunks > kMaxGridY) return IPTTT_ERR_SHAPE;
  const int64_t tm = (r.C + 127) / 128, tn_d = (r.d + 127) / 128, tn_f = (r.f + 127) / 128;
  if (chunks > kMaxGrid / (tm * tn_d)) return IPTTT_ERR_SHAPE;
  if (chunks > kMaxGrid / (tm * (tm + 1) / 2)) return IPTTT_ERR_SHAPE;
  if (((r.M + 127) / 128) > kMaxGrid / (tn_f > tn_d ? tn_f : tn_d)) return IPTTT_ERR_SHAPE;
  // chunk-transposed copies (general kernels, diagnostic dW): 32 x 32 tiles
  const int64_t ct = (r.C + 31) / 32, ft = ((r.d > r.f ? r.d : r.f) + 31) / 32;
  if (chunks > kMaxGrid / (ct * ft)) return IPTTT_ERR_SHAPE;
  // Per-chunk weights of the scan, B*N*d*f elements, must be addressable.
  const int64_t df = (int64_t)r.d * r.f;
  if (chunks > (int64_t(1) << 62) / (df * 4)) return IPTTT_ERR_SHAPE;
  if ((q->seg_table == nullptr) != (q->seg_bytes == nullptr)) return IPTTT_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(q->seg_table) & 3) != 0) return IPTTT_ERR_ALIGN;
  if (q->n_doc_starts < 0) return IPTTT_ERR_SEGMENTS;
  if (q->n_doc_starts > 0 && q->doc_starts == nullptr) return IPTTT_ERR_NULL;
  for (int64_t k = 0; k < q->n_doc_starts; ++k) {
    const int64_t s = q->doc_starts[k];
    if (s < 0 || s >= r.M) return IPTTT_ERR_SEGMENTS;
    if (k > 0 && s <= q->doc_starts[k - 1]) return IPTTT_ERR_SEGMENTS;
  }
  *p = r;
  return IPTTT_OK;
}

// Workspace: per-token segment bytes | segment table | one region that each
// call uses for itself:
//   ipttt_target       W_target^T, tap-major conv weights, conv output Y
//   ipttt_chunk_delta  Gram partials | chunk-transposed V_hat, Z (dW only)
//   ipttt_scan_apply   per-chunk weights | fragment-major W_down | scaled V_hat
//                      (bf16 fast path) or per-chunk weights | chunk-transposed
//                      V_hat, Z (general path)
struct Layout {
  size_t segs, table, call, total;
  size_t vt_bytes;      // chunk-transposed V_hat; the Z copy follows it
  size_t wbuf, wdfrag;  // offsets of the scan's weights inside the call region
  size_t vs;            // offset of the scaled V_hat (fast path)
  size_t rst;           // offset of the state carried between chunk windows
};

// Passes of the 8-wave scan and apply.  Their per-chunk weights take B*N*d*f
// elements for all rows at once; passes reuse one pass's worth of weights and
// of scaled V_hat, kept with W_down's fragments within the pass budget: whole
// rows while a row fits, else windows of whole chunks of one row, each window
// handing the fp32 state after its last chunk to the next (d*f*4 bytes, also
// counted).  Rows are independent and the state goes through the buffer bit
// for bit, so the passes compute exactly what one pass over everything would.
constexpr size_t kPassBytes = size_t(4) << 30;
size_t pass_budget() {
  // IPTTT_PASS_BYTES (bytes) overrides the default budget of 4 GiB
  if (const char* e = std::getenv("IPTTT_PASS_BYTES")) {
    char* end = nullptr;
    const unsigned long long v = std::strtoull(e, &end, 10);
    if (end != e && *end == '\0' && v > 0) return (size_t)v;
  }
  return kPassBytes;
}
struct Passes {
  int64_t rows;  // rows per pass
  int64_t chunks;  // chunks per window (N: whole rows)
};
Passes min_passes(const Prob& p) {
  if (!ipttt::fast_scan(p)) return {p.B, p.N};
  const size_t e = elt_bytes(p), wd = (size_t)p.d * p.f * e, budget = pass_budget();
  const size_t per_row = (size_t)p.N * wd + (size_t)p.T * p.d * e;
  if (wd + per_row <= budget) return {std::min<int64_t>(p.B, (int64_t)((budget - wd) / per_row)), p.N};
  const size_t fixed = wd + (size_t)p.d * p.f * sizeof(float), per_chunk = wd + (size_t)p.C * p.d * e;
  const int64_t n = budget > fixed ? (int64_t)((budget - fixed) / per_chunk) : 0;
  return {1, std::max<int64_t>(1, std::min<int64_t>(n, p.N - 1))};
}

// Passes of the diagnostic delta output, whose chunk-transposed copies of
// V_hat and Z take B*N*Cp*(d+f) elements for all rows: whole rows, or windows
// of a row's chunks, within a quarter of the pass budget, so that this path
// never sets the workspace size.
Passes dw_passes(const Prob& p) {
  const size_t per_chunk = (size_t)p.Cp * ((size_t)p.d + p.f) * elt_bytes(p), budget = pass_budget() / 4;
  if ((size_t)p.N * per_chunk <= budget)
    return {std::min<int64_t>(p.B, (int64_t)(budget / ((size_t)p.N * per_chunk))), p.N};
  return {1, std::max<int64_t>(1, (int64_t)(budget / per_chunk))};
}

// ps.rows > 0: the scan's regions for those passes (the minimal workspace
// uses min_passes(p)).
Layout layout(const Prob& p, Passes ps = {0, 0}) {
  Layout l;
  const int64_t chunks = p.B * p.N;
  l.segs = 0;
  l.table = align256((size_t)p.M);
  l.call = l.table + align256((size_t)chunks * 3 * sizeof(int32_t));
  const size_t e = elt_bytes(p);
  const size_t target = ((size_t)p.d * p.d + 5 * (size_t)p.d + (size_t)p.M * p.d) * e;
  const size_t vt_bytes = align256((size_t)chunks * p.Cp * (size_t)p.d * e);
  const size_t zt_bytes = align256((size_t)chunks * p.Cp * (size_t)p.f * e);
  const size_t partials = align256((size_t)chunks * ipttt::gram_pairs(p) * sizeof(float));
  const size_t weights = align256((size_t)chunks * p.d * (size_t)p.f * e);
  l.wbuf = 0;
  const Passes dwp = dw_passes(p);
  const size_t dwr = (size_t)dwp.rows * dwp.chunks;  // chunks of one pass
  const size_t gscr = align256(ipttt::gram_scratch_bytes(p, chunks));
  const size_t delta = partials + gscr + align256(dwr * p.Cp * (size_t)p.d * e) +
                       align256(dwr * p.Cp * (size_t)p.f * e);
  size_t scan;
  if (ipttt::fast_scan(p)) {
    if (ps.rows <= 0) ps = min_passes(p);
    const size_t rpp = (size_t)ps.rows;
    l.wdfrag = align256(rpp * (size_t)ps.chunks * p.d * (size_t)p.f * e);
    l.vs = l.wdfrag + align256((size_t)p.d * p.f * e);
    const size_t vrow = ps.chunks < p.N ? (size_t)ps.chunks * p.C : (size_t)p.T;  // V_s tokens per row
    l.rst = l.vs + align256(rpp * vrow * p.d * e);
    scan = l.rst + (ps.chunks < p.N ? align256(rpp * p.d * (size_t)p.f * sizeof(float)) : 0);
  } else {
    l.wdfrag = l.vs = l.rst = 0;
    scan = weights + vt_bytes + zt_bytes;
  }
  size_t m = target > delta ? target : delta;
  m = m > scan ? m : scan;
  l.vt_bytes = vt_bytes;
  l.total = l.call + align256(m);
  return l;
}

// Backward workspace: segment bytes | table | one region per call.
//   scan_apply_backward: alpha, Gram partials, dot partials, coefficients |
//     chunk-transposed V_hat, Z, dO | per-chunk weights [f, d] | delta
//     adjoints [f, d] and [d, f] | W_down^T | per-row W_down gradients |
//     A = Z dDW^T (fp32) | chunk Grams Z Z^T, V V^T (dtype) | scaled V_hat
//     (the 8-wave path uses no transposed copies: the weights region holds
//     the recomputed fragment-major chunk weights when none are saved, the
//     W_down^T region W_down in that layout, the delta adjoints [d, f] theirs)
//   target_backward: tap-major conv weights | Y | dY (fp32) | Y^T, dV^T | conv
//     partials (the 8-wave path keeps dW_target's token-slice partials in Y^T, dV^T)
//   z_backward: dG, dU | W_gate^T, W_up^T | dG^T, dU^T, H^T
struct BwdLayout {
  size_t table, call, total;
  // scan_apply_backward
  size_t alpha, gram, gscr, dots, cpos, cneg, vt, zt, dot, w1, w2, w3, wdt, wpart, abuf, gz, gv, vc;
  // target_backward
  size_t convt, y, dy, yt, dvt, cpart;
  // z_backward
  size_t dg, du, wgt, wut, dgt, dut, ht;
  int64_t Mp;
};

// Pitch of the backward's chunk Grams (Z_seg Z_seg^T and V_seg V_seg^T, one
// per chunk, zero outside the carried segment).  The 8-wave products that
// contract over them run whole 64-token K stages, so there the pitch is C
// rounded up to 64 and the zeros fill the last stage; the general products
// take C rounded up to 8, like the chunk-transposed copies.
int gram_pitch(const Prob& p) { return ipttt::fast_scan(p) ? (p.C + 63) / 64 * 64 : p.Cp; }

BwdLayout bwd_layout(const Prob& p) {
  BwdLayout l;
  const int64_t chunks = p.B * p.N;
  const size_t e = elt_bytes(p);
  l.table = align256((size_t)p.M);
  l.call = l.table + align256((size_t)chunks * 3 * sizeof(int32_t));
  l.Mp = (p.M + 63) / 64 * 64;  // token-axis pitch of the transposed copies: whole 64-token K stages
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
  const size_t df = (size_t)p.d * p.f;
  l.alpha = take((size_t)chunks * 4);
  l.gram = take((size_t)chunks * ipttt::gram_pairs(p) * 4);
  l.gscr = take(ipttt::gram_scratch_bytes(p, chunks));
  l.dots = take((size_t)chunks * ipttt::kDotParts * 4);
  l.cpos = take((size_t)chunks * 4);
  l.cneg = take((size_t)chunks * 4);
  // regions only the general path uses take no room on the 8-wave path
  const bool fast = ipttt::fast_scan(p);
  const bool tnfast = fast && p.d < 65536 && p.f < 65536;
  l.vt = take(fast ? 0 : (size_t)chunks * p.Cp * (size_t)p.d * e);
  l.zt = take(fast ? 0 : (size_t)chunks * p.Cp * (size_t)p.f * e);
  l.dot = take(fast ? 0 : (size_t)chunks * p.Cp * (size_t)p.d * e);
  l.w1 = take((size_t)chunks * df * e);
  l.w2 = take(fast ? 0 : (size_t)chunks * df * e);
  l.w3 = take((size_t)chunks * df * e);
  l.wdt = take(df * e);
  l.wpart = take((size_t)p.B * df * 4);
  l.abuf = take((size_t)p.M * p.d * 4);
  const size_t gp = (size_t)gram_pitch(p);
  l.gz = take((size_t)chunks * gp * gp * e);
  l.gv = take((size_t)chunks * gp * gp * e);
  l.vc = take((size_t)p.M * p.d * e);
  const size_t sa = o;
  o = 0;
  l.convt = take((size_t)5 * p.d * e);
  l.y = take((size_t)p.M * p.d * e);
  l.dy = take((size_t)p.M * p.d * 4);
  l.yt = take((size_t)l.Mp * p.d * e);
  l.dvt = take((size_t)l.Mp * p.d * e);
  l.cpart = take((size_t)ipttt::kConvParts * p.d * 5 * 4);
  const size_t tg = o;
  o = 0;
  l.dg = take((size_t)p.M * p.f * e);
  l.du = take((size_t)p.M * p.f * e);
  l.wgt = take(fast ? 0 : df * e);
  l.wut = take(fast ? 0 : df * e);
  l.dgt = take(tnfast ? 0 : (size_t)l.Mp * p.f * e);
  l.dut = take(tnfast ? 0 : (size_t)l.Mp * p.f * e);
  l.ht = take(tnfast ? 0 : (size_t)l.Mp * p.d * e);
  const size_t zb = o;
  l.total = l.call + std::max(sa, std::max(tg, zb));
  return l;
}

// The largest passes of the 8-wave scan and apply that a workspace of
// ws_bytes holds (at least the minimal layout's): more rows per pass, or,
// where rows are cut into chunk windows, longer windows.
Passes passes_for_workspace(const Prob& p, size_t ws_bytes) {
  Passes ps = min_passes(p);
  if (!ipttt::fast_scan(p)) return ps;
  if (ps.chunks == p.N) {
    int64_t lo = ps.rows, hi = p.B;
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) / 2;
      if (layout(p, {mid, p.N}).total <= ws_bytes) lo = mid;
      else hi = mid - 1;
    }
    ps.rows = lo;
    return ps;
  }
  // a whole row drops the state buffer, so it is tried first
  if (layout(p, {1, p.N}).total <= ws_bytes) return {1, p.N};
  int64_t lo = ps.chunks, hi = p.N - 1;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    if (layout(p, {1, mid}).total <= ws_bytes) lo = mid;
    else hi = mid - 1;
  }
  ps.chunks = lo;
  return ps;
}

ipttt_status check_ws(const Prob& p, void* ws, size_t ws_bytes, Layout* l) {
  *l = layout(p);
  if (ws == nullptr || ws_bytes < l->total) return IPTTT_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return IPTTT_ERR_ALIGN;
  return IPTTT_OK;
}

// Saved forward state (fast path only): the per-chunk weights W_down + S_i
// in the scan's fragment-major layout, then W_down in the same layout.
size_t saved_bytes(const Prob& p) {
  if (!ipttt::fast_scan(p)) return 0;
  const size_t e = elt_bytes(p);
  return align256((size_t)p.B * p.N * p.d * (size_t)p.f * e) + align256((size_t)p.d * p.f * e);
}
size_t saved_wdfrag(const Prob& p) { return align256((size_t)p.B * p.N * p.d * (size_t)p.f * elt_bytes(p)); }

ipttt_status hip_status(hipError_t e) { return e == hipSuccess ? IPTTT_OK : IPTTT_ERR_HIP; }

template <class... P>
bool all_aligned(P... ptrs) {
  return (aligned16(ptrs) && ...);
}

template <class... P>
bool any_null(P... ptrs) {
  return ((ptrs == nullptr) || ...);
}

ipttt_status build_segments(const ipttt_problem* q, const Prob& p, void* ws, const Layout& l,
                            hipStream_t st, uint8_t** segs, int32_t** table) {
  if (q->seg_table != nullptr) {  // prepared by the caller (ipttt_segments_device)
    *segs = const_cast<uint8_t*>(q->seg_bytes);
    *table = const_cast<int32_t*>(q->seg_table);
    return IPTTT_OK;
  }
  *segs = static_cast<uint8_t*>(ws) + l.segs;
  *table = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + l.table);
  return hip_status(ipttt::launch_segments(p, q->doc_starts, q->n_doc_starts, q->continues, *segs, *table, st));
}

// Shared prologue of the backward calls: validation of the problem and the
// workspace, then the segment descriptors.
ipttt_status bwd_begin(const ipttt_problem* q, Prob* p, void* ws, size_t ws_bytes, BwdLayout* l) {
  ipttt_status s = check_problem(q, p);
  if (s != IPTTT_OK) return s;
  *l = bwd_layout(*p);
  if (ws == nullptr || ws_bytes < l->total) return IPTTT_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return IPTTT_ERR_ALIGN;
  return IPTTT_OK;
}

ipttt_status bwd_segments(const ipttt_problem* q, const Prob& p, void* ws, const BwdLayout& l, hipStream_t st,
                          uint8_t** segs, int32_t** table, char** call) {
  *call = static_cast<char*>(ws) + l.call;
  if (q->seg_table != nullptr) {  // prepared by the caller (ipttt_segments_device)
    *segs = const_cast<uint8_t*>(q->seg_bytes);
    *table = const_cast<int32_t*>(q->seg_table);
    return IPTTT_OK;
  }
  *segs = static_cast<uint8_t*>(ws);
  *table = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + l.table);
  return hip_status(ipttt::launch_segments(p, q->doc_starts, q->n_doc_starts, q->continues, *segs, *table, st));
}

}  // namespace

extern "C" {

int ipttt_abi_version(void) { return IPTTT_ABI_VERSION; }

void ipttt_set_launch_hook(ipttt_launch_hook hook, void* user) {
  g_hook = nullptr;
  g_hook_user = user;
  g_hook = hook;
}

const char* ipttt_status_string(int status) {
  switch (status) {
    case IPTTT_OK: return "ok";
    case IPTTT_ERR_NULL: return "a required pointer is NULL";
    case IPTTT_ERR_SHAPE: return "invalid or unsupported sizes";
    case IPTTT_ERR_DTYPE: return "unsupported dtype";
    case IPTTT_ERR_ALIGN: return "pointer not aligned (tensors: 16 bytes, workspace: 256 bytes)";
    case IPTTT_ERR_SEGMENTS: return "doc_starts not strictly increasing within [0, rows*seq_len)";
    case IPTTT_ERR_WORKSPACE: return "workspace missing or too small";
    case IPTTT_ERR_HIP: return "HIP runtime error";
    case IPTTT_ERR_ARG: return "invalid scalar argument, target kind, or S_out partly overlapping S_in";
    case IPTTT_ERR_SCRATCH: return "problem too large for the allocation-free call's static scratch";
    default: return "unknown status";
  }
}

ipttt_status ipttt_validate(const ipttt_problem* q) {
  Prob p;
  return check_problem(q, &p);
}

size_t ipttt_workspace_bytes(const ipttt_problem* q) {
  Prob p;
  if (check_problem(q, &p) != IPTTT_OK) return 0;
  return layout(p).total;
}

ipttt_status ipttt_segment_table(const ipttt_problem* q, int32_t* table) {
  Prob p;
  ipttt_status s = check_problem(q, &p);
  if (s != IPTTT_OK) return s;
  if (table == nullptr) return IPTTT_ERR_NULL;
  // Walk the chunks of each row with a cursor into the sorted start list.
  int64_t k = 0;
  for (int64_t b = 0; b < p.B; ++b) {
    const int64_t row0 = b * p.T;
    while (k < q->n_doc_starts && q->doc_starts[k] < row0) ++k;
    for (int64_t i = 0; i < p.N; ++i) {
      const int64_t lo = row0 + i * p.C;
      const int64_t hi = std::min(lo + p.C, row0 + p.T);
      int32_t first = -1, last = 0;
      // a row start is a document start, unless the row continues one
      if (i == 0 && !(q->continues != nullptr && q->continues[b])) first = 0;
      while (k < q->n_doc_starts && q->doc_starts[k] < hi) {
        const int32_t off = (int32_t)(q->doc_starts[k] - lo);
        if (first < 0) first = off;
        last = off;
        ++k;
      }
      int32_t* e = table + (b * p.N + i) * 3;
      e[0] = first < 0 ? (int32_t)(hi - lo) : first;
      e[1] = last;
      const bool next_starts = (i + 1 < p.N) && k < q->n_doc_starts && q->doc_starts[k] == hi;
      e[2] = (i + 1 < p.N && !next_starts) ? 1 : 0;
    }
  }
  return IPTTT_OK;
}

ipttt_status ipttt_segments_device(const ipttt_problem* q, int32_t* table, uint8_t* segs,
                                   void* stream) {
  Prob p;
  ipttt_status s = check_problem(q, &p);
  if (s != IPTTT_OK) return s;
  if (segs == nullptr) return IPTTT_ERR_NULL;
  if (table != nullptr && (reinterpret_cast<uintptr_t>(table) & 3) != 0) return IPTTT_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(ipttt::launch_segments(p, q->doc_starts, q->n_doc_starts, q->continues, segs, table,
                                           static_cast<hipStream_t>(stream)));
}

ipttt_status ipttt_z(const ipttt_problem* q, const void* H, const void* W_gate, const void* W_up,
                     void* Z, void* stream) {
  Prob p;
  ipttt_status s = check_problem(q, &p);
  if (s != IPTTT_OK) return s;
  if (any_null(H, W_gate, W_up, Z)) return IPTTT_ERR_NULL;
  if (!all_aligned(H, W_gate, W_up, Z)) return IPTTT_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(ipttt::launch_gated_z(p, H, W_gate, W_up, Z, nullptr, static_cast<hipStream_t>(stream)));
}

ipttt_status ipttt_z_save(const ipttt_problem* q, const void* H, const void* W_gate, const void* W_up, void* Z,
                          void* GU, void* stream) {
  Prob p;
  ipttt_status s = check_problem(q, &p);
  if (s != IPTTT_OK) return s;
  if (any_null(H, W_gate, W_up, Z, GU)) return IPTTT_ERR_NULL;
  if (!all_aligned(H, W_gate, W_up, Z, GU)) return IPTTT_ERR_ALIGN;
  (void)hipGetLastError();
  return hip_status(ipttt::launch_gated_z(p, H, W_gate, W_up, Z, GU, static_cast<hipStream_t>(stream)));
}

ipttt_status ipttt_target(const ipttt_problem* q, const void* X0, const void* conv_w,
                          const void* W_target, void* V, void* ws, size_t ws_bytes, void* stream) {
  Prob p;
  ipttt_status s = check_problem(q, &p);
  if (s != IPTTT_OK) return s;
  if (any_null(X0, V)) return IPTTT_ERR_NULL;
  if (conv_w == nullptr && p.target != IPTTT_TARGET_NO_CONV) return IPTTT_ERR_NULL;
  if (W_target == nullptr && p.target != IPTTT_TARGET_NO_PROJ) return IPTTT_ERR_NULL;
  if (!all_aligned(X0, conv_w, W_target, V)) return IPTTT_ERR_ALIGN;
  Layout l;
  if ((s = check_ws(p, ws, ws_bytes, &l)) != IPTTT_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  uint8_t* segs;
  int32_t* table;
  if ((s = build_segments(q, p, ws, l, st, &segs, &table)) != IPTTT_OK) return s;
  void* scratch = static_cast<char*>(ws) + l.call;
  return hip_status(ipttt::launch_target(p, X0, conv_w, W_target, segs, V, scratch, st));
}

ipttt_status ipttt_chunk_delta(const ipttt_problem* q, const void* V, const void* Z, float eta, float tau,
                               float* alpha, float* dW, void* ws, size_t ws_bytes, void* stream) {
  Prob p;
  ipttt_status s = check_problem(q, &p);
  if (s != IPTTT_OK) return s;
  if (any_null(V, Z, alpha)) return IPTTT_ERR_NULL;
  if (!all_aligned(V, Z, alpha, dW)) return IPTTT_ERR_ALIGN;
  if (!std::isfinite(eta) || !std::isfinite(tau)) return IPTTT_ERR_ARG;
  Layout l;
  if ((s = check_ws(p, ws, ws_bytes, &l)) != IPTTT_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  uint8_t* segs;
  int32_t* table;
  if ((s = build_segments(q, p, ws, l, st, &segs, &table)) != IPTTT_OK) return s;
  char* call = static_cast<char*>(ws) + l.call;
  float* partials = reinterpret_cast<float*>(call);
  char* gscr = call + align256((size_t)p.B * p.N * ipttt::gram_pairs(p) * sizeof(float));
  if ((s = hip_status(ipttt::launch_alpha(p, V, Z, table, eta, tau, alpha, partials, gscr, st))) != IPTTT_OK)
    return s;
  if (dW == nullptr) return IPTTT_OK;
  // The materialised deltas contract over tokens: chunk-transposed copies,
  // made and used in passes of whole rows or of windows of one row's chunks
  // (each pass as a problem of its own: rows are independent, and so is each
  // chunk's delta given its segment-table entry and clip scale).
  const Passes dwp = dw_passes(p);
  const size_t e = elt_bytes(p);
  char* vt = gscr + align256(ipttt::gram_scratch_bytes(p, p.B * p.N));
  char* zt = vt + align256((size_t)dwp.rows * dwp.chunks * p.Cp * (size_t)p.d * e);
  for (int64_t b0 = 0; b0 < p.B; b0 += dwp.rows) {
    for (int64_t i0 = 0; i0 < p.N; i0 += dwp.chunks) {
      Prob q = p;
      q.B = std::min(dwp.rows, p.B - b0);
      q.N = (int)std::min<int64_t>(dwp.chunks, p.N - i0);
      q.T = dwp.chunks < p.N ? std::min<int64_t>(p.T - i0 * p.C, q.N * p.C) : p.T;
      q.M = q.B * q.T;
      const size_t t0 = (size_t)b0 * p.T + (size_t)i0 * p.C;
      const char* Vb = static_cast<const char*>(V) + t0 * p.d * e;
      const char* Zb = static_cast<const char*>(Z) + t0 * p.f * e;
      const int64_t c0 = b0 * p.N + i0;
      if ((s = hip_status(ipttt::launch_chunk_transpose(q, Vb, p.d, vt, st))) != IPTTT_OK) return s;
      if ((s = hip_status(ipttt::launch_chunk_transpose(q, Zb, p.f, zt, st))) != IPTTT_OK) return s;
      if ((s = hip_status(ipttt::launch_dw(q, vt, zt, table + c0 * 3, alpha + c0, eta, dW + (size_t)c0 * p.d * p.f,
                                           st))) != IPTTT_OK)
        return s;
    }
  }
  return IPTTT_OK;
}

ipttt_status ipttt_chunk_delta_noalloc(const ipttt_problem* q, const void* V, const void* Z, float eta, float tau,
                                       float* alpha, void* stream) {
  Prob p;
  ipttt_status s = check_problem(q, &p);
  if (s != IPTTT_OK) return s;
  if (any_null(V, Z, alpha)) return IPTTT_ERR_NULL;
  if (!all_aligned(V, Z, alpha)) return IPTTT_ERR_ALIGN;
  if (!std::isfinite(eta) || !std::isfinite(tau)) return IPTTT_ERR_ARG;
  // The scratch regions of ipttt_chunk_delta (dW = NULL), in the same order:
  // segment bytes | segment table | Gram partials | stored V V^T tiles, the
  // last for a window of chunks at a time (at least one) when the 8-wave
  // Gram path runs.
  Layout l;
  l.segs = 0;
  l.table = align256((size_t)p.M);
  const int64_t chunks = p.B * p.N;
  const size_t partials = l.table + align256((size_t)chunks * 3 * sizeof(int32_t));
  const size_t gscr = partials + align256((size_t)chunks * ipttt::gram_pairs(p) * sizeof(float));
  const size_t per_chunk = ipttt::gram_scratch_bytes(p, 1);
  const bool windows = per_chunk > 0 && tau > 0.0f;
  if (gscr + (windows ? per_chunk : 0) > (size_t)IPTTT_NOALLOC_SCRATCH_BYTES) return IPTTT_ERR_SCRATCH;
  const int64_t window = windows ? std::min<int64_t>(chunks, ((size_t)IPTTT_NOALLOC_SCRATCH_BYTES - gscr) / per_chunk)
                                 : chunks;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  void* scratch = nullptr;
  if ((s = hip_status(ipttt::noalloc_scratch(&scratch))) != IPTTT_OK) return s;
  uint8_t* segs;
  int32_t* table;
  if ((s = build_segments(q, p, scratch, l, st, &segs, &table)) != IPTTT_OK) return s;
  float* part = reinterpret_cast<float*>(static_cast<char*>(scratch) + partials);
  if (!windows) return hip_status(ipttt::launch_alpha(p, V, Z, table, eta, tau, alpha, part, nullptr, st));
  float* gv = reinterpret_cast<float*>(static_cast<char*>(scratch) + gscr);
  for (int64_t c0 = 0; c0 < chunks; c0 += window)
    if ((s = hip_status(ipttt::launch_gram_fast(p, V, Z, table, part, gv, c0, std::min(chunks, c0 + window), st))) !=
        IPTTT_OK)
      return s;
  return hip_status(ipttt::launch_alpha_only(p, part, eta, tau, alpha, st));
}

}  // extern "C"

namespace {

ipttt_status scan_apply(const ipttt_problem* q, const void* Z, const void* V, const void* W_down, const float* alpha,
                        float eta, bool carry, const float* S_in, float* S_out, void* O, void* saved,
                        size_t saved_size, void* ws, size_t ws_bytes, void* stream) {
  Prob p;
  ipttt_status s = check_problem(q, &p);
  if (s != IPTTT_OK) return s;
  if (any_null(Z, V, W_down, alpha, O)) return IPTTT_ERR_NULL;
  if (!all_aligned(Z, V, W_down, alpha, O, S_in, S_out)) return IPTTT_ERR_ALIGN;
  const size_t need = saved_bytes(p);
  if (need > 0 && saved != nullptr) {
    if (saved_size < need) return IPTTT_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(saved) & 255) != 0) return IPTTT_ERR_ALIGN;
  } else {
    saved = nullptr;
  }
  if (!std::isfinite(eta)) return IPTTT_ERR_ARG;
  if (S_in != nullptr && S_out != nullptr && S_in != S_out) {
    // S_out is either S_in itself or disjoint from it
    const size_t bytes = (size_t)p.B * p.d * (size_t)p.f * sizeof(float);
    const uintptr_t a = reinterpret_cast<uintptr_t>(S_in), b = reinterpret_cast<uintptr_t>(S_out);
    if (a < b + bytes && b < a + bytes) return IPTTT_ERR_ARG;
  }
  Layout l;
  if ((s = check_ws(p, ws, ws_bytes, &l)) != IPTTT_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  uint8_t* segs;
  int32_t* table;
  if ((s = build_segments(q, p, ws, l, st, &segs, &table)) != IPTTT_OK) return s;
  char* call = static_cast<char*>(ws) + l.call;
  void* Wbuf = saved != nullptr ? saved : call + l.wbuf;
  void* Wdfrag = saved != nullptr ? static_cast<char*>(saved) + saved_wdfrag(p)
                                  : ipttt::fast_scan(p) ? call + l.wdfrag : nullptr;
  void* Vs = ipttt::fast_scan(p) ? call + l.vs : nullptr;
  void* vt = nullptr;
  void* zt = nullptr;
  if (!ipttt::fast_scan(p)) {
    vt = call + align256((size_t)p.B * p.N * p.d * (size_t)p.f * elt_bytes(p));
    zt = static_cast<char*>(vt) + l.vt_bytes;
    if ((s = hip_status(ipttt::launch_chunk_transpose(p, V, p.d, vt, st))) != IPTTT_OK) return s;
    if ((s = hip_status(ipttt::launch_chunk_transpose(p, Z, p.f, zt, st))) != IPTTT_OK) return s;
  }
  if (ipttt::fast_scan(p)) {
    // passes of as many whole rows as the workspace holds (one pass when
    // every row's weights fit), or of windows of a row's chunks; the saved
    // state holds every chunk's weights at its own offset
    const Passes ps = passes_for_workspace(p, ws_bytes);
    const Layout lp = layout(p, ps);
    Wbuf = call + lp.wbuf;
    Wdfrag = saved != nullptr ? Wdfrag : call + lp.wdfrag;
    Vs = call + lp.vs;
    float* Rst = ps.chunks < p.N ? reinterpret_cast<float*>(call + lp.rst) : nullptr;
    const size_t chunk_bytes = (size_t)p.d * p.f * elt_bytes(p);
    for (int64_t b0 = 0; b0 < p.B; b0 += ps.rows) {
      const int nb = (int)std::min(ps.rows, p.B - b0);
      for (int64_t i0 = 0; i0 < p.N; i0 += ps.chunks) {
        const int i1 = (int)std::min<int64_t>(p.N, i0 + ps.chunks);
        void* wb = saved != nullptr ? static_cast<char*>(saved) + ((size_t)b0 * p.N + i0) * chunk_bytes : Wbuf;
        if ((s = hip_status(ipttt::launch_scan(p, Z, V, nullptr, nullptr, W_down, table, alpha, eta, wb, Wdfrag, Vs,
                                               carry, S_in, S_out, st, (int)b0, nb, (int)i0, i1, Rst))) != IPTTT_OK)
          return s;
        if ((s = hip_status(ipttt::launch_apply(p, Z, wb, W_down, Wdfrag, table, O, st, (int)b0, nb, (int)i0,
                                                i1))) != IPTTT_OK)
          return s;
      }
    }
    return IPTTT_OK;
  }
  if ((s = hip_status(ipttt::launch_scan(p, Z, V, zt, vt, W_down, table, alpha, eta, Wbuf, Wdfrag, Vs, carry, S_in,
                                         S_out, st))) != IPTTT_OK)
    return s;
  return hip_status(ipttt::launch_apply(p, Z, Wbuf, W_down, Wdfrag, table, O, st));
}

}  // namespace

extern "C" {

ipttt_status ipttt_scan_apply(const ipttt_problem* q, const void* Z, const void* V, const void* W_down,
                              const float* alpha, float eta, void* O, void* ws, size_t ws_bytes,
                              void* stream) {
  return scan_apply(q, Z, V, W_down, alpha, eta, false, nullptr, nullptr, O, nullptr, 0, ws, ws_bytes, stream);
}

size_t ipttt_saved_bytes(const ipttt_problem* q) {
  Prob p;
  if (check_problem(q, &p) != IPTTT_OK) return 0;
  return saved_bytes(p);
}

ipttt_status ipttt_scan_apply_save(const ipttt_problem* q, const void* Z, const void* V, const void* W_down,
                                   const float* alpha, float eta, void* O, void* saved, size_t saved_size, void* ws,
                                   size_t ws_bytes, void* stream) {
  Prob p;
  const ipttt_status s = check_problem(q, &p);
  if (s != IPTTT_OK) return s;
  if (saved_bytes(p) > 0 && saved == nullptr) return IPTTT_ERR_NULL;
  return scan_apply(q, Z, V, W_down, alpha, eta, false, nullptr, nullptr, O, saved, saved_size, ws, ws_bytes, stream);
}

ipttt_status ipttt_scan_apply_carry(const ipttt_problem* q, const void* Z, const void* V, const void* W_down,
                                    const float* alpha, float eta, const float* S_in, float* S_out, void* O,
                                    void* ws, size_t ws_bytes, void* stream) {
  return scan_apply(q, Z, V, W_down, alpha, eta, true, S_in, S_out, O, nullptr, 0, ws, ws_bytes, stream);
}

size_t ipttt_backward_workspace_bytes(const ipttt_problem* q) {
  Prob p;
  if (check_problem(q, &p) != IPTTT_OK) return 0;
  return bwd_layout(p).total;
}

}  // extern "C"

namespace {

// alpha_in: the forward's clip scales (else recomputed); saved: the forward's
// saved state (else its chunk weights are recomputed).
ipttt_status scan_apply_backward(const ipttt_problem* q, const void* Z, const void* V, const void* W_down, float eta,
                                 float tau, const float* alpha_in, const void* saved, size_t saved_size,
                                 const void* dO, void* dZ, void* dV, float* dW_down, void* ws, size_t ws_bytes,
                                 void* stream) {
  Prob p;
  BwdLayout l;
  ipttt_status s;
  if ((s = bwd_begin(q, &p, ws, ws_bytes, &l)) != IPTTT_OK) return s;
  if (any_null(Z, V, W_down, dO, dZ, dV, dW_down)) return IPTTT_ERR_NULL;
  if (!all_aligned(Z, V, W_down, dO, dZ, dV, dW_down, alpha_in)) return IPTTT_ERR_ALIGN;
  if (!std::isfinite(eta) || !std::isfinite(tau)) return IPTTT_ERR_ARG;
  if (saved_bytes(p) > 0 && saved != nullptr) {
    if (saved_size < saved_bytes(p)) return IPTTT_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(saved) & 255) != 0) return IPTTT_ERR_ALIGN;
  } else {
    saved = nullptr;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  uint8_t* segs;
  int32_t* table;
  char* c;
  if ((s = bwd_segments(q, p, ws, l, st, &segs, &table, &c)) != IPTTT_OK) return s;
  const size_t e = elt_bytes(p);
  const int gp = gram_pitch(p);
  const int64_t df = (int64_t)p.d * p.f, cp2 = (int64_t)gp * gp;
  float* alpha_ws = reinterpret_cast<float*>(c + l.alpha);
  const float* alpha = alpha_in != nullptr ? alpha_in : alpha_ws;
  float* gram = reinterpret_cast<float*>(c + l.gram);
  float* dots = reinterpret_cast<float*>(c + l.dots);
  float* cpos = reinterpret_cast<float*>(c + l.cpos);
  float* cneg = reinterpret_cast<float*>(c + l.cneg);
  void *Vt = c + l.vt, *Zt = c + l.zt, *dOt = c + l.dot, *WT = c + l.w1, *dDWt = c + l.w2, *dDW = c + l.w3;
  void *WdT = c + l.wdt, *Gz = c + l.gz, *Gv = c + l.gv, *Vc = c + l.vc;
  float* Wpart = reinterpret_cast<float*>(c + l.wpart);
  float* Abuf = reinterpret_cast<float*>(c + l.abuf);
  const bool clip = tau > 0.0f;
#define IPTTT_TRY(x)                                   \
  do {                                                 \
    if ((s = hip_status(x)) != IPTTT_OK) return s;     \
  } while (0)
  // With the clip, the chunk Grams are zeroed first: the clip's products then
  // run over whole chunks, zeros standing in for everything outside the
  // carried segment.  The 8-wave products read V_hat and Z in their row
  // layout (rows past a chunk read as zero); the general ones take
  // chunk-transposed copies, their padding past a short last chunk zeroed.
  const bool fast = ipttt::fast_scan(p);
  if (clip) {
    if (!fast) {
      IPTTT_TRY(ipttt::launch_zero(Vt, (size_t)p.B * p.N * p.Cp * (size_t)p.d * e, st));
      IPTTT_TRY(ipttt::launch_zero(Zt, (size_t)p.B * p.N * p.Cp * (size_t)p.f * e, st));
    }
    IPTTT_TRY(ipttt::launch_zero(Gz, (size_t)p.B * p.N * cp2 * e, st));
    IPTTT_TRY(ipttt::launch_zero(Gv, (size_t)p.B * p.N * cp2 * e, st));
  }
  if (!fast) {
    IPTTT_TRY(ipttt::launch_chunk_transpose(p, V, p.d, Vt, st));
    IPTTT_TRY(ipttt::launch_chunk_transpose(p, Z, p.f, Zt, st));
    IPTTT_TRY(ipttt::launch_chunk_transpose(p, dO, p.d, dOt, st));
  }
  // the forward's clip scales and norms (the norms follow from the scales
  // where the clip acts), and its per-chunk weights
  if (alpha_in == nullptr) IPTTT_TRY(ipttt::launch_alpha(p, V, Z, table, eta, tau, alpha_ws, gram, c + l.gscr, st));
  if (saved != nullptr) {
    WT = const_cast<void*>(saved);
    WdT = static_cast<char*>(const_cast<void*>(saved)) + saved_wdfrag(p);
  } else if (fast) {
    // the forward's own scan: its fragment-major chunk weights, and W_down in
    // the same layout (the scaled V_hat goes to Vc, which is written later);
    // the dZ products read both transposed straight from that layout
    IPTTT_TRY(ipttt::launch_scan(p, Z, V, nullptr, nullptr, W_down, table, alpha, eta, WT, WdT, Vc, false, nullptr,
                                 nullptr, st));
  } else {
    IPTTT_TRY(ipttt::launch_scan_transposed(p, Zt, Vt, W_down, table, alpha, eta, WT, st));
    IPTTT_TRY(ipttt::launch_transpose_pad(p, W_down, p.d, p.f, p.d, WdT, st));
  }
  // reverse scan: the delta adjoints dDW_i, and dW_down
  if (fast) {
    // dDW fragment-major (like the forward's weights)
    IPTTT_TRY(ipttt::launch_rscan_fast(p, Z, dO, table, dDW, Wpart, st));
  } else {
    IPTTT_TRY(ipttt::launch_rscan(p, dOt, Zt, table, dDW, dDWt, Wpart, st));
  }
  IPTTT_TRY(ipttt::launch_sum_parts(Wpart, dW_down, df, (int)p.B, st));
  // A = Z_seg dDW^T on each carrying segment
  ipttt::NTArgs b;
  b.chunked = 1; b.rows = ipttt::NT_ROWS_SEG;
  b.pr[0].A = Z; b.pr[0].a_tok = 1; b.pr[0].lda = p.f;
  b.pr[0].B = dDW; b.pr[0].sb = df; b.pr[0].ldb = p.f; b.pr[0].K = p.f; b.pr[0].b_frag = fast;
  b.C = Abuf; b.c_tok = 1; b.ldc = p.d; b.c_f32 = 1;
  b.N = p.d;
  IPTTT_TRY(ipttt::launch_nt(p, b, 0, table, st));
  // the clip's adjoint coefficients: cpos = eta alpha, cneg = -eta alpha kappa
  // (with Vc = eta alpha V_seg, an operand of dZ)
  IPTTT_TRY(ipttt::launch_seg_dot_scale(p, V, Abuf, table, alpha, eta, dots, Vc, st));
  IPTTT_TRY(ipttt::launch_coef(p, alpha, alpha_in != nullptr ? nullptr : gram, ipttt::gram_pairs(p), dots, table, eta,
                               tau, cpos, cneg, st));
  if (clip) {
    // chunk Grams on the carried segments: Z_seg Z_seg^T and cneg V_seg V_seg^T
    ipttt::NTArgs g;
    g.chunked = 1; g.rows = ipttt::NT_ROWS_SEG; g.nseg = 1;
    g.pr[0].A = Z; g.pr[0].a_tok = 1; g.pr[0].lda = p.f;
    g.pr[0].B = Z; g.pr[0].b_tok = 1; g.pr[0].ldb = p.f; g.pr[0].K = p.f;
    g.C = Gz; g.sc = cp2; g.ldc = gp;  // dtype: an operand of the next products
    g.N = p.C;
    IPTTT_TRY(ipttt::launch_nt(p, g, 0, table, st));
    g.pr[0].A = V; g.pr[0].lda = p.d; g.pr[0].B = V; g.pr[0].ldb = p.d; g.pr[0].K = p.d;
    g.C = Gv; g.ca = cneg;
    IPTTT_TRY(ipttt::launch_nt(p, g, 0, table, st));
  }
  // dV = eta alpha (A - kappa Z_seg Z_seg^T V_seg) on carrying segments, 0 elsewhere
  IPTTT_TRY(ipttt::launch_zero(dV, (size_t)p.M * p.d * e, st));
  ipttt::NTArgs v;
  v.chunked = 1; v.rows = ipttt::NT_ROWS_SEG; v.kseg = 1; v.kzero = 1;
  if (clip) {
    v.pr[0].A = Gz; v.pr[0].sa = cp2; v.pr[0].lda = gp;
    v.pr[0].B = Vt; v.pr[0].sb = (int64_t)p.d * p.Cp; v.pr[0].ldb = p.Cp; v.pr[0].K = gp;
    if (fast) { v.pr[0].B = V; v.pr[0].sb = 0; v.pr[0].ldb = p.d; v.pr[0].b_kmaj = 1; v.pr[0].b_tok = 1; }
  } else {
    v.npairs = 0;
  }
  v.C = dV; v.c_tok = 1; v.ldc = p.d;
  v.ca = cneg; v.X = Abuf; v.cx = cpos;
  v.N = p.d;
  IPTTT_TRY(ipttt::launch_nt(p, v, 0, table, st));
  // dZ = dO (W_down + S_i) + eta alpha (V_seg dDW - kappa V_seg V_seg^T Z_seg):
  // one product per chunk part with up to three operand pairs, the scales
  // folded into the operands (Vc = eta alpha V_seg, Gv = cneg V V^T)
  ipttt::NTArgs z;
  z.chunked = 1;
  z.npairs = clip ? 3 : 2;
  z.pr[0].A = dO; z.pr[0].a_tok = 1; z.pr[0].lda = p.d;
  z.pr[0].B = WT; z.pr[0].sb = df; z.pr[0].ldb = p.d; z.pr[0].K = p.d;
  z.pr[1].A = Vc; z.pr[1].a_tok = 1; z.pr[1].lda = p.d;
  z.pr[1].B = dDWt; z.pr[1].sb = df; z.pr[1].ldb = p.d; z.pr[1].K = p.d;
  if (fast) {
    // W_i and dDW_i [d, f] fragment-major, read as B = W^T
    z.pr[0].ldb = p.f; z.pr[0].b_fragt = 1;
    z.pr[1].B = dDW; z.pr[1].ldb = p.f; z.pr[1].b_fragt = 1;
  }
  z.pr[2].A = Gv; z.pr[2].sa = cp2; z.pr[2].lda = gp;
  z.pr[2].B = Zt; z.pr[2].sb = (int64_t)p.f * p.Cp; z.pr[2].ldb = p.Cp; z.pr[2].K = gp;
  if (fast) { z.pr[2].B = Z; z.pr[2].sb = 0; z.pr[2].ldb = p.f; z.pr[2].b_kmaj = 1; z.pr[2].b_tok = 1; }
  z.C = dZ; z.c_tok = 1; z.ldc = p.f;
  z.N = p.f;
  // Rows before the chunk's first document start apply W_down + S_i, rows
  // from it on W_down.  On the 8-wave path a chunk whose document starts at
  // its first row (all of it W_down) runs in the first launch, so the
  // second only has the chunks split by a document start.
  z.rows = fast ? ipttt::NT_ROWS_HEADZ : ipttt::NT_ROWS_HEAD;
  z.tail_B = WdT;
  IPTTT_TRY(ipttt::launch_nt(p, z, 0, table, st));
  z.pr[0].B = WdT; z.pr[0].sb = 0;
  z.rows = fast ? ipttt::NT_ROWS_TAILNZ : ipttt::NT_ROWS_TAIL;
  IPTTT_TRY(ipttt::launch_nt(p, z, 0, table, st));
  return IPTTT_OK;
}

}  // namespace

extern "C" {

ipttt_status ipttt_scan_apply_backward(const ipttt_problem* q, const void* Z, const void* V, const void* W_down,
                                       float eta, float tau, const void* dO, void* dZ, void* dV, float* dW_down,
                                       void* ws, size_t ws_bytes, void* stream) {
  return scan_apply_backward(q, Z, V, W_down, eta, tau, nullptr, nullptr, 0, dO, dZ, dV, dW_down, ws, ws_bytes,
                             stream);
}

ipttt_status ipttt_scan_apply_backward_saved(const ipttt_problem* q, const void* Z, const void* V, const void* W_down,
                                             float eta, float tau, const float* alpha, const void* saved,
                                             size_t saved_size, const void* dO, void* dZ, void* dV, float* dW_down,
                                             void* ws, size_t ws_bytes, void* stream) {
  if (alpha == nullptr) return IPTTT_ERR_NULL;
  return scan_apply_backward(q, Z, V, W_down, eta, tau, alpha, saved, saved_size, dO, dZ, dV, dW_down, ws, ws_bytes,
                             stream);
}

ipttt_status ipttt_target_backward(const ipttt_problem* q, const void* X0, const void* conv_w, const void* W_target,
                                   const void* dV, void* dX0, float* dconv_w, float* dW_target, void* ws,
                                   size_t ws_bytes, void* stream) {
  Prob p;
  BwdLayout l;
  ipttt_status s;
  if ((s = bwd_begin(q, &p, ws, ws_bytes, &l)) != IPTTT_OK) return s;
  const bool conv = p.target != IPTTT_TARGET_NO_CONV, proj = p.target != IPTTT_TARGET_NO_PROJ;
  if (any_null(X0, dV, dX0)) return IPTTT_ERR_NULL;
  if (conv && (conv_w == nullptr || dconv_w == nullptr)) return IPTTT_ERR_NULL;
  if (proj && (W_target == nullptr || dW_target == nullptr)) return IPTTT_ERR_NULL;
  if (!all_aligned(X0, conv_w, W_target, dV, dX0, dconv_w, dW_target)) return IPTTT_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  uint8_t* segs;
  int32_t* table;
  char* c;
  if ((s = bwd_segments(q, p, ws, l, st, &segs, &table, &c)) != IPTTT_OK) return s;
  float* dY = reinterpret_cast<float*>(c + l.dy);
  // dY = dV W_target^T (or dV itself without the projection)
  if (proj) {
    ipttt::NTArgs a;
    a.chunked = 1;
    a.pr[0].A = dV; a.pr[0].a_tok = 1; a.pr[0].lda = p.d;
    a.pr[0].B = W_target; a.pr[0].ldb = p.d; a.pr[0].K = p.d;
    a.C = dY; a.c_tok = 1; a.ldc = p.d; a.c_f32 = 1;
    a.N = p.d;
    IPTTT_TRY(ipttt::launch_nt(p, a, 0, table, st));
    // dW_target = Y^T dV over every token
    const void* Y = X0;
    if (conv) {
      IPTTT_TRY(ipttt::launch_conv_only(p, X0, conv_w, segs, c + l.y, c + l.convt, st));
      Y = c + l.y;
    }
    if (p.dtype == 1 && p.d % 64 == 0 && p.d < 65536) {
      // contracted along the token axis in place; token slices write partial
      // products over the (here unused) transposed-copy regions
      const int cap = (int)((l.cpart - l.yt) / ((size_t)p.d * p.d * 4));
      const int sp = ipttt::tn_fast_splits(1, p.M, p.d, p.d, cap);
      float* dst = sp > 1 ? reinterpret_cast<float*>(c + l.yt) : dW_target;
      const void* A[1] = {Y};
      const void* Bm[1] = {dV};
      float* Cw[1] = {dst};
      IPTTT_TRY(ipttt::launch_tn_fast(1, A, Bm, Cw, p.M, p.d, p.d, sp, st));
      if (sp > 1) IPTTT_TRY(ipttt::launch_sum_parts(dst, dW_target, (int64_t)p.d * p.d, sp, st));
    } else {
      IPTTT_TRY(ipttt::launch_transpose_pad(p, Y, p.M, p.d, l.Mp, c + l.yt, st));
      IPTTT_TRY(ipttt::launch_transpose_pad(p, dV, p.M, p.d, l.Mp, c + l.dvt, st));
      ipttt::NTArgs w;
      w.pr[0].A = c + l.yt; w.pr[0].lda = l.Mp;
      w.pr[0].B = c + l.dvt; w.pr[0].ldb = l.Mp; w.pr[0].K = (int)l.Mp;
      w.C = dW_target; w.ldc = p.d; w.c_f32 = 1;
      w.M = p.d; w.N = p.d;
      IPTTT_TRY(ipttt::launch_nt(p, w, 1, table, st));
    }
  } else {
    IPTTT_TRY(ipttt::launch_convert(p, dV, dY, p.M * p.d, false, st));
  }
  if (!conv) {
    IPTTT_TRY(ipttt::launch_convert(p, dY, dX0, p.M * p.d, true, st));
    return IPTTT_OK;
  }
  float* part = reinterpret_cast<float*>(c + l.cpart);
  IPTTT_TRY(ipttt::launch_conv_bwd(p, dY, X0, conv_w, segs, dX0, part, st));
  IPTTT_TRY(ipttt::launch_sum_parts(part, dconv_w, (int64_t)p.d * 5, ipttt::kConvParts, st));
  return IPTTT_OK;
}

}  // extern "C"

namespace {

// GU: the G and U the forward saved (ipttt_z_save), or NULL (recomputed).
ipttt_status z_backward(const ipttt_problem* q, const void* H, const void* W_gate, const void* W_up, const void* GU,
                        const void* dZ, void* dH, float* dW_gate, float* dW_up, void* ws, size_t ws_bytes,
                        void* stream) {
  Prob p;
  BwdLayout l;
  ipttt_status s;
  if ((s = bwd_begin(q, &p, ws, ws_bytes, &l)) != IPTTT_OK) return s;
  if (any_null(H, W_gate, W_up, dZ, dH, dW_gate, dW_up)) return IPTTT_ERR_NULL;
  if (!all_aligned(H, W_gate, W_up, dZ, dH, dW_gate, dW_up, GU)) return IPTTT_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  uint8_t* segs;
  int32_t* table;
  char* c;
  if ((s = bwd_segments(q, p, ws, l, st, &segs, &table, &c)) != IPTTT_OK) return s;
  void *dG = c + l.dg, *dU = c + l.du;
  if (GU != nullptr) {
    IPTTT_TRY(ipttt::launch_gated_grad(p, GU, dZ, dG, dU, st));
  } else {
    IPTTT_TRY(ipttt::launch_gated_z_bwd(p, H, W_gate, W_up, dZ, dG, dU, st));
  }
  // dH = dG W_gate + dU W_up (the 8-wave path reads W_gate and W_up
  // K-major in place; the general one takes transposed copies)
  const bool fast = ipttt::fast_scan(p);
  ipttt::NTArgs a;
  a.chunked = 1;
  a.npairs = 2;
  a.pr[0].A = dG; a.pr[0].a_tok = 1; a.pr[0].lda = p.f;
  if (fast) {
    a.pr[0].B = W_gate; a.pr[0].ldb = p.d; a.pr[0].K = p.f; a.pr[0].b_kmaj = 1;
  } else {
    IPTTT_TRY(ipttt::launch_transpose_pad(p, W_gate, p.f, p.d, p.f, c + l.wgt, st));
    IPTTT_TRY(ipttt::launch_transpose_pad(p, W_up, p.f, p.d, p.f, c + l.wut, st));
    a.pr[0].B = c + l.wgt; a.pr[0].ldb = p.f; a.pr[0].K = p.f;
  }
  a.pr[1] = a.pr[0];
  a.pr[1].A = dU; a.pr[1].B = fast ? W_up : static_cast<const void*>(c + l.wut);
  a.C = dH; a.c_tok = 1; a.ldc = p.d;
  a.N = p.d;
  IPTTT_TRY(ipttt::launch_nt(p, a, 0, table, st));
  // dW_gate = dG^T H, dW_up = dU^T H over every token: contracted along the
  // token axis in place (bf16 fast shapes), else from transposed copies
  if (ipttt::fast_scan(p) && p.d < 65536 && p.f < 65536) {
    const void* A[2] = {dG, dU};
    const void* Bm[2] = {H, H};
    float* Cw[2] = {dW_gate, dW_up};
    IPTTT_TRY(ipttt::launch_tn_fast(2, A, Bm, Cw, p.M, p.f, p.d, 1, st));
    return IPTTT_OK;
  }
  IPTTT_TRY(ipttt::launch_transpose_pad(p, H, p.M, p.d, l.Mp, c + l.ht, st));
  IPTTT_TRY(ipttt::launch_transpose_pad(p, dG, p.M, p.f, l.Mp, c + l.dgt, st));
  IPTTT_TRY(ipttt::launch_transpose_pad(p, dU, p.M, p.f, l.Mp, c + l.dut, st));
  ipttt::NTArgs w;
  w.pr[0].A = c + l.dgt; w.pr[0].lda = l.Mp;
  w.pr[0].B = c + l.ht; w.pr[0].ldb = l.Mp; w.pr[0].K = (int)l.Mp;
  w.C = dW_gate; w.ldc = p.d; w.c_f32 = 1;
  w.M = p.f; w.N = p.d;
  IPTTT_TRY(ipttt::launch_nt(p, w, 1, table, st));
  w.pr[0].A = c + l.dut; w.C = dW_up;
  IPTTT_TRY(ipttt::launch_nt(p, w, 1, table, st));
  return IPTTT_OK;
#undef IPTTT_TRY
}

}  // namespace

extern "C" {

ipttt_status ipttt_z_backward(const ipttt_problem* q, const void* H, const void* W_gate, const void* W_up,
                              const void* dZ, void* dH, float* dW_gate, float* dW_up, void* ws, size_t ws_bytes,
                              void* stream) {
  return z_backward(q, H, W_gate, W_up, nullptr, dZ, dH, dW_gate, dW_up, ws, ws_bytes, stream);
}

ipttt_status ipttt_z_backward_saved(const ipttt_problem* q, const void* H, const void* W_gate, const void* W_up,
                                    const void* GU, const void* dZ, void* dH, float* dW_gate, float* dW_up, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (GU == nullptr) return IPTTT_ERR_NULL;
  return z_backward(q, H, W_gate, W_up, GU, dZ, dH, dW_gate, dW_up, ws, ws_bytes, stream);
}

}  // extern "C"
