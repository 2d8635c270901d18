// C ABI of the deterministic ragged BF16 grouped GEMM (include/moe_ragged_bf16.h).
//
// Host side only: argument validation (before anything is enqueued, as the
// accumulate description of flashinfer PR #8924 requires of its checks), the
// sizing rules of the wgrad row split, and the kernel launches.  The host never
// reads offs, never allocates and never synchronises.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>

#include "grouped_gemm.h"
#include "moe_ragged_bf16.h"

namespace mdg {

// ----------------------------------------------------------------- sizing rules
// Rows per chunk of the wgrad row split.  A pure function of the sizes, so the
// chunking (and with it every bit of dW) never depends on the device, timing or
// the workspace handed in.  It aims at >= kSplitTargetUnits work units even when
// one expert holds all rows, and never splits below kMinChunkRows rows.
constexpr int64_t kSplitTargetUnits = 512;
constexpr int64_t kMinChunkRows = 256;

int64_t wgrad_chunk_rows(int64_t m_rows, int64_t n, int64_t k, int32_t num_groups) {
  (void)num_groups;
  const int64_t tiles = ((n + kTileI - 1) / kTileI) * ((k + kTileJ - 1) / kTileJ);
  const int64_t want_chunks = (kSplitTargetUnits + tiles - 1) / tiles;
  int64_t r = (m_rows + want_chunks - 1) / want_chunks;
  r = (r + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
  return r < kMinChunkRows ? kMinChunkRows : r;
}

// Upper bound on the number of experts with more than R rows.
int64_t wgrad_max_split_groups(int64_t m_rows, int64_t chunk_rows, int32_t num_groups) {
  const int64_t big = m_rows / (chunk_rows + 1);
  return big < num_groups ? big : num_groups;
}

// Upper bound on sum over split experts of ceil(m_e / R):
// sum ceil(m_e/R) <= sum floor(m_e/R) + #split <= floor(M/R) + #split.
int64_t wgrad_max_partial_slots(int64_t m_rows, int64_t chunk_rows, int32_t num_groups) {
  const int64_t big = wgrad_max_split_groups(m_rows, chunk_rows, num_groups);
  return big == 0 ? 0 : m_rows / chunk_rows + big;
}

// fwd/dgrad: units of the persistent schedule (an upper bound: row tiles of
// every group, each group's last one possibly partial, times column tiles).
int64_t fwd_dgrad_units_ub(Op op, int64_t m_rows, int64_t n, int64_t k, int32_t num_groups) {
  const int64_t n_j = (op == kFwd) ? (n + kTileJ - 1) / kTileJ : (k + kTileJ - 1) / kTileJ;
  const int64_t row_tiles_ub = (m_rows + kTileI - 1) / kTileI + num_groups;
  return row_tiles_ub * n_j;
}

// fwd/dgrad: fp32 partial tiles of the tail split.  The tail holds fewer than
// kBalanceSlots units, each cut into at most kMaxSplit pieces, and the plan
// never uses more pieces than kBalanceSlots (nor than this bound).
int64_t tail_slots(int64_t units_ub) {
  const int64_t s = units_ub * kMaxSplit;
  return s < kBalanceSlots ? s : kBalanceSlots;
}

size_t fwd_dgrad_workspace(Op op, int64_t m_rows, int64_t n, int64_t k, int32_t num_groups) {
  const int64_t slots = tail_slots(fwd_dgrad_units_ub(op, m_rows, n, k, num_groups));
  return (size_t)kTailHeadBytes + (size_t)slots * kTileI * kTileJ * sizeof(float);
}

namespace {

constexpr size_t kTableBytes = 4096;  // reserved head of the workspace

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Workspace regions of wgrad, in order: reserved head, fp32 partial tiles of
// split experts.
struct WgradWorkspace {
  size_t partial_off, total;
};

WgradWorkspace wgrad_workspace(int64_t m_rows, int64_t n, int64_t k, int32_t num_groups) {
  WgradWorkspace w;
  const int64_t r = wgrad_chunk_rows(m_rows, n, k, num_groups);
  const int64_t slots = wgrad_max_partial_slots(m_rows, r, num_groups);
  w.partial_off = kTableBytes;
  w.total = align256(w.partial_off + (size_t)slots * (size_t)n * (size_t)k * sizeof(float));
  return w;
}

struct DeviceInfo {
  bool ok = false;
  bool gfx950 = false;
  int cus = 0;
};

DeviceInfo g_dev[64];
std::once_flag g_dev_once[64];

int query_device(DeviceInfo* out, int* device) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MDG_EHIP;
  *device = dev;
  std::call_once(g_dev_once[dev], [dev]() {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
    g_dev[dev].gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev[dev].cus = prop.multiProcessorCount;
    g_dev[dev].ok = true;
  });
  if (!g_dev[dev].ok) return MDG_EHIP;
  *out = g_dev[dev];
  return MDG_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlaps(Range a, Range b) {
  if (a.hi == a.lo || b.hi == b.lo) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// Shared size checks.  Sizes are kept small enough for the kernels' 32-bit
// in-tile arithmetic: rows < 2^31, n and k < 2^20, and per-expert n*k < 2^31.
int check_sizes(int64_t m_rows, int64_t n, int64_t k, int32_t num_groups) {
  if (m_rows < 0 || n <= 0 || k <= 0 || num_groups <= 0) return MDG_EINVAL;
  if (num_groups > kMaxGroups) return MDG_EUNSUPPORTED;
  if (n % kNAlign != 0 || k % kKAlign != 0) return MDG_EUNSUPPORTED;
  if (m_rows > kMaxRows || n > (1 << 20) || k > (1 << 20) || n * k > INT32_MAX)
    return MDG_EUNSUPPORTED;
  return MDG_OK;
}

int persistent_grid(int64_t units_upper_bound, int cus) {
  int64_t g = cus > 0 ? cus : 256;
  if (units_upper_bound < g) g = units_upper_bound;
  if (g >= 8) g -= g % 8;
  return g < 1 ? 1 : (int)g;
}

}  // namespace
}  // namespace mdg

// A prepared launch: every argument validated, every kernel parameter and grid
// computed.  Enqueueing it only launches kernels (no checks, no allocation, no
// synchronisation, no memset), so it can be recorded into a HIP graph.
struct mdg_launch {
  int op;                 // mdg::Op
  int device;             // HIP device current at preparation
  int dw_dtype, accumulate;
  mdg::GemmParams p;
  int gemm_grid;          // 0: nothing to enqueue at all
  int tail_gx, tail_gy;   // fwd/dgrad tail reduce grid (0: none)
  int red_gx, red_gy;     // wgrad chunk reduce (0: none)
  int64_t workspace_bytes;
};

namespace mdg {
namespace {

// The checks of fwd/dgrad that need neither the workspace nor the device.
int check_fwd_dgrad(const void* a, const void* w, const int32_t* offs, void* out, int64_t m_rows, int64_t n,
                    int64_t k, int32_t num_groups) {
  int st = check_sizes(m_rows, n, k, num_groups);
  if (st != MDG_OK) return st;
  // Row-indexed tensors may be NULL when there are no rows (never dereferenced).
  if (!w || !offs || (m_rows > 0 && (!a || !out))) return MDG_EINVAL;
  if (!aligned16(a) || !aligned16(w) || !aligned4(offs) || !aligned16(out)) return MDG_EINVAL;
  return MDG_OK;
}

int prepare_fwd_dgrad(Op op, const void* a, const void* w, const int32_t* offs, void* out, int64_t m_rows,
                      int64_t n, int64_t k, int32_t num_groups, void* workspace, size_t workspace_bytes,
                      mdg_launch* l) {
  int st = check_fwd_dgrad(a, w, offs, out, m_rows, n, k, num_groups);
  if (st != MDG_OK) return st;
  const size_t need = fwd_dgrad_workspace(op, m_rows, n, k, num_groups);
  if (!workspace || workspace_bytes < need) return MDG_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MDG_EINVAL;
  const int64_t a_cols = (op == kFwd) ? k : n;
  const int64_t o_cols = (op == kFwd) ? n : k;
  const Range ra = range_of(a, m_rows * a_cols * 2);
  const Range rw = range_of(w, (int64_t)num_groups * n * k * 2);
  const Range ro = range_of(offs, (int64_t)num_groups * 4);
  const Range ry = range_of(out, m_rows * o_cols * 2);
  const Range rws = range_of(workspace, (int64_t)need);
  if (overlaps(ry, ra) || overlaps(ry, rw) || overlaps(ry, ro) || overlaps(ry, rws)) return MDG_EOVERLAP;
  if (overlaps(rws, ra) || overlaps(rws, rw) || overlaps(rws, ro)) return MDG_EOVERLAP;

  *l = mdg_launch{};
  l->op = op;
  l->device = -1;
  l->workspace_bytes = (int64_t)need;
  if (m_rows == 0) return MDG_OK;  // nothing to enqueue

  DeviceInfo dev;
  st = query_device(&dev, &l->device);
  if (st != MDG_OK) return st;
  if (!dev.gfx950) return MDG_EUNSUPPORTED;

  GemmParams& p = l->p;
  p.a = static_cast<const uint16_t*>(a);
  p.b = static_cast<const uint16_t*>(w);
  p.offs = offs;
  p.out = out;
  p.m_rows = m_rows;
  p.n = (int32_t)n;
  p.k = (int32_t)k;
  p.num_groups = num_groups;
  const int64_t units_ub = fwd_dgrad_units_ub(op, m_rows, n, k, num_groups);
  const int64_t slots = tail_slots(units_ub);
  char* ws = static_cast<char*>(workspace);
  p.tail_head = reinterpret_cast<int32_t*>(ws);
  p.partial = reinterpret_cast<float*>(ws + kTailHeadBytes);
  p.tail_slots = (int32_t)slots;
  l->gemm_grid = persistent_grid(units_ub + slots, dev.cus);
  // Split tail units (at most kBalanceSlots / 2 of them, as each has >= 2
  // pieces): the reduce kernel reads the plan the GEMM kernel wrote and exits
  // at once when there is none.
  if (slots >= 2) {
    l->tail_gx = 8;
    l->tail_gy = (int)std::min<int64_t>(kBalanceSlots / 2, slots / 2);
  }
  return MDG_OK;
}

int prepare_wgrad(const void* g, const void* x, const int32_t* offs, void* dw, int dw_dtype, int accumulate,
                  int64_t m_rows, int64_t n, int64_t k, int32_t num_groups, void* workspace,
                  size_t workspace_bytes, mdg_launch* l) {
  int st = check_sizes(m_rows, n, k, num_groups);
  if (st != MDG_OK) return st;
  if (dw_dtype != MDG_BF16 && dw_dtype != MDG_FP32) return MDG_EINVAL;
  if (!offs || !dw || (m_rows > 0 && (!g || !x))) return MDG_EINVAL;
  if (!aligned16(g) || !aligned16(x) || !aligned4(offs) || !aligned16(dw)) return MDG_EINVAL;
  const WgradWorkspace wl = wgrad_workspace(m_rows, n, k, num_groups);
  const size_t need = wl.total;
  if (!workspace || workspace_bytes < need) return MDG_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MDG_EINVAL;
  const int64_t esz = dw_dtype == MDG_FP32 ? 4 : 2;
  const Range rg = range_of(g, m_rows * n * 2);
  const Range rx = range_of(x, m_rows * k * 2);
  const Range ro = range_of(offs, (int64_t)num_groups * 4);
  const Range rd = range_of(dw, (int64_t)num_groups * n * k * esz);
  const Range rws = range_of(workspace, (int64_t)need);
  if (overlaps(rd, rg) || overlaps(rd, rx) || overlaps(rd, ro) || overlaps(rd, rws)) return MDG_EOVERLAP;
  if (overlaps(rws, rg) || overlaps(rws, rx) || overlaps(rws, ro)) return MDG_EOVERLAP;

  *l = mdg_launch{};
  l->op = kWgrad;
  l->device = -1;
  l->dw_dtype = dw_dtype;
  l->accumulate = accumulate != 0;
  l->workspace_bytes = (int64_t)need;
  // An accumulate over zero rows launches nothing and leaves dw unchanged.
  if (m_rows == 0 && accumulate) return MDG_OK;

  DeviceInfo dev;
  st = query_device(&dev, &l->device);
  if (st != MDG_OK) return st;
  if (!dev.gfx950) return MDG_EUNSUPPORTED;

  const int64_t r = wgrad_chunk_rows(m_rows, n, k, num_groups);
  char* ws = static_cast<char*>(workspace);
  GemmParams& p = l->p;
  p.a = static_cast<const uint16_t*>(g);
  p.b = static_cast<const uint16_t*>(x);
  p.offs = offs;
  p.out = dw;
  p.partial = reinterpret_cast<float*>(ws + wl.partial_off);
  p.m_rows = m_rows;
  p.n = (int32_t)n;
  p.k = (int32_t)k;
  p.num_groups = num_groups;
  p.chunk_rows = (int32_t)r;
  p.out_fp32 = dw_dtype == MDG_FP32;
  p.accumulate = accumulate != 0;

  const int64_t tiles = ((n + kTileI - 1) / kTileI) * ((k + kTileJ - 1) / kTileJ);
  const int64_t units_ub = tiles * (num_groups + m_rows / r);
  if (units_ub > INT32_MAX) return MDG_EUNSUPPORTED;
  const int64_t split_ub = wgrad_max_split_groups(m_rows, r, num_groups);
  if (split_ub > 65535) return MDG_EUNSUPPORTED;
  const int64_t cus = dev.cus > 0 ? dev.cus : 256;
  l->gemm_grid = persistent_grid(units_ub, dev.cus);
  if (split_ub > 0) {
    const int64_t nk4 = n * k / 4;
    int64_t gx = (nk4 + kThreads * 4 - 1) / (kThreads * 4);
    const int64_t cap = (4 * cus + split_ub - 1) / split_ub;
    if (gx > cap) gx = cap;
    if (gx < 1) gx = 1;
    l->red_gx = (int)gx;
    l->red_gy = (int)split_ub;
  }
  return MDG_OK;
}

// Enqueues a prepared launch: nothing but kernel launches.
int enqueue(const mdg_launch& l, hipStream_t s) {
  if (l.gemm_grid == 0) return MDG_OK;
  if (launch_gemm(static_cast<Op>(l.op), l.p, l.gemm_grid, s) != hipSuccess) return MDG_EHIP;
  if (l.tail_gy > 0 && launch_tail_reduce(l.p, l.tail_gx, l.tail_gy, s) != hipSuccess) return MDG_EHIP;
  if (l.red_gy > 0 && launch_wgrad_reduce(l.p, l.red_gx, l.red_gy, s) != hipSuccess) return MDG_EHIP;
  return MDG_OK;
}

int publish(int st, const mdg_launch& l, mdg_launch** out) {
  if (st != MDG_OK) return st;
  mdg_launch* h = new (std::nothrow) mdg_launch(l);
  if (!h) return MDG_ENOMEM;
  *out = h;
  return MDG_OK;
}

mdg_status status(int st) { return static_cast<mdg_status>(st); }

int kernels_of(const mdg_launch& l) {
  if (l.gemm_grid == 0) return 0;
  return 1 + (l.tail_gy > 0) + (l.red_gy > 0);
}

}  // namespace
}  // namespace mdg

using namespace mdg;

extern "C" {

MDG_API int grouped_det_gemm_abi_version(void) { return MDG_ABI_VERSION; }

MDG_API const char* grouped_det_gemm_status_string(int s) {
  switch (s) {
    case MDG_OK: return "ok";
    case MDG_EINVAL: return "invalid argument (null or misaligned pointer, negative size or bad enum)";
    case MDG_EUNSUPPORTED: return "unsupported shape or device (needs gfx950, n % 8 == 0, k % 8 == 0, 1 <= groups <= 1024)";
    case MDG_EOVERLAP: return "an output overlaps an input, the offsets or the workspace";
    case MDG_EWORKSPACE: return "workspace missing or too small";
    case MDG_EHIP: return "HIP runtime error";
    case MDG_ENOMEM: return "host memory allocation failed";
    default: return "unknown status";
  }
}

MDG_API size_t grouped_det_gemm_fwd_workspace_bytes(int64_t m_rows, int64_t n, int64_t k, int32_t num_groups) {
  if (check_sizes(m_rows, n, k, num_groups) != MDG_OK) return 0;
  return fwd_dgrad_workspace(kFwd, m_rows, n, k, num_groups);
}

MDG_API size_t grouped_det_gemm_dgrad_workspace_bytes(int64_t m_rows, int64_t n, int64_t k, int32_t num_groups) {
  if (check_sizes(m_rows, n, k, num_groups) != MDG_OK) return 0;
  return fwd_dgrad_workspace(kDgrad, m_rows, n, k, num_groups);
}

MDG_API mdg_status grouped_det_gemm_fwd(const void* x, const void* w, const int32_t* offs, void* y, int64_t m_rows,
                         int64_t n, int64_t k, int32_t num_groups, void* workspace, size_t workspace_bytes,
                         void* stream) {
  mdg_launch l;
  const int st = prepare_fwd_dgrad(kFwd, x, w, offs, y, m_rows, n, k, num_groups, workspace, workspace_bytes, &l);
  return status(st != MDG_OK ? st : enqueue(l, static_cast<hipStream_t>(stream)));
}

MDG_API mdg_status grouped_det_gemm_fwd_noalloc(const void* x, const void* w, const int32_t* offs, void* y,
                                                int64_t m_rows, int64_t n, int64_t k, int32_t num_groups,
                                                void* stream) {
  int st = check_fwd_dgrad(x, w, offs, y, m_rows, n, k, num_groups);
  if (st != MDG_OK) return status(st);
  if (m_rows == 0) return status(MDG_OK);  // nothing to enqueue (as grouped_det_gemm_fwd)
  // the static array holds the largest fwd workspace, so no valid size is refused here
  if (fwd_dgrad_workspace(kFwd, m_rows, n, k, num_groups) > kFwdScratchBytes) return status(MDG_EWORKSPACE);
  DeviceInfo dev;
  int device = -1;
  st = query_device(&dev, &device);
  if (st != MDG_OK) return status(st);
  if (!dev.gfx950) return status(MDG_EUNSUPPORTED);
  void* ws = nullptr;
  if (fwd_scratch_address(device, &ws) != hipSuccess) return status(MDG_EHIP);
  mdg_launch l;
  st = prepare_fwd_dgrad(kFwd, x, w, offs, y, m_rows, n, k, num_groups, ws, kFwdScratchBytes, &l);
  return status(st != MDG_OK ? st : enqueue(l, static_cast<hipStream_t>(stream)));
}

MDG_API mdg_status grouped_det_gemm_dgrad(const void* g, const void* w, const int32_t* offs, void* dx, int64_t m_rows,
                           int64_t n, int64_t k, int32_t num_groups, void* workspace, size_t workspace_bytes,
                           void* stream) {
  mdg_launch l;
  const int st = prepare_fwd_dgrad(kDgrad, g, w, offs, dx, m_rows, n, k, num_groups, workspace, workspace_bytes, &l);
  return status(st != MDG_OK ? st : enqueue(l, static_cast<hipStream_t>(stream)));
}

MDG_API int64_t grouped_det_gemm_wgrad_chunk_rows(int64_t m_rows, int64_t n, int64_t k, int32_t num_groups) {
  if (check_sizes(m_rows, n, k, num_groups) != MDG_OK) return 0;
  return wgrad_chunk_rows(m_rows, n, k, num_groups);
}

MDG_API size_t grouped_det_gemm_wgrad_workspace_bytes(int64_t m_rows, int64_t n, int64_t k, int32_t num_groups) {
  if (check_sizes(m_rows, n, k, num_groups) != MDG_OK) return 0;
  return wgrad_workspace(m_rows, n, k, num_groups).total;
}

MDG_API mdg_status grouped_det_gemm_wgrad(const void* g, const void* x, const int32_t* offs, void* dw, int dw_dtype,
                           int accumulate, int64_t m_rows, int64_t n, int64_t k, int32_t num_groups,
                           void* workspace, size_t workspace_bytes, void* stream) {
  mdg_launch l;
  const int st = prepare_wgrad(g, x, offs, dw, dw_dtype, accumulate, m_rows, n, k, num_groups, workspace,
                               workspace_bytes, &l);
  return status(st != MDG_OK ? st : enqueue(l, static_cast<hipStream_t>(stream)));
}

MDG_API mdg_status grouped_det_gemm_prepare_fwd(const void* x, const void* w, const int32_t* offs, void* y, int64_t m_rows,
                                 int64_t n, int64_t k, int32_t num_groups, void* workspace,
                                 size_t workspace_bytes, mdg_launch** launch) {
  if (!launch) return status(MDG_EINVAL);
  *launch = nullptr;
  mdg_launch l;
  return status(publish(prepare_fwd_dgrad(kFwd, x, w, offs, y, m_rows, n, k, num_groups, workspace, workspace_bytes, &l),
                 l, launch));
}

MDG_API mdg_status grouped_det_gemm_prepare_dgrad(const void* g, const void* w, const int32_t* offs, void* dx, int64_t m_rows,
                                   int64_t n, int64_t k, int32_t num_groups, void* workspace,
                                   size_t workspace_bytes, mdg_launch** launch) {
  if (!launch) return status(MDG_EINVAL);
  *launch = nullptr;
  mdg_launch l;
  return status(publish(prepare_fwd_dgrad(kDgrad, g, w, offs, dx, m_rows, n, k, num_groups, workspace, workspace_bytes,
                                   &l),
                 l, launch));
}

MDG_API mdg_status grouped_det_gemm_prepare_wgrad(const void* g, const void* x, const int32_t* offs, void* dw, int dw_dtype,
                                   int accumulate, int64_t m_rows, int64_t n, int64_t k, int32_t num_groups,
                                   void* workspace, size_t workspace_bytes, mdg_launch** launch) {
  if (!launch) return status(MDG_EINVAL);
  *launch = nullptr;
  mdg_launch l;
  return status(publish(prepare_wgrad(g, x, offs, dw, dw_dtype, accumulate, m_rows, n, k, num_groups, workspace,
                               workspace_bytes, &l),
                 l, launch));
}

MDG_API mdg_status grouped_det_gemm_launch(const mdg_launch* launch, void* stream) {
  if (!launch) return status(MDG_EINVAL);
  if (launch->gemm_grid == 0) return status(MDG_OK);  // nothing to enqueue
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return status(MDG_EHIP);
  if (dev != launch->device) return status(MDG_EINVAL);
  return status(enqueue(*launch, static_cast<hipStream_t>(stream)));
}

MDG_API mdg_status grouped_det_gemm_launch_info(const mdg_launch* launch, mdg_launch_info* info) {
  if (!launch || !info) return status(MDG_EINVAL);
  mdg_launch_info r;
  memset(&r, 0, sizeof(r));
  r.op = launch->op;
  r.device = launch->device;
  r.kernels = kernels_of(*launch);
  r.gemm_grid = launch->gemm_grid;
  r.dw_dtype = launch->dw_dtype;
  r.accumulate = launch->accumulate;
  r.chunk_rows = launch->op == kWgrad ? launch->p.chunk_rows : 0;
  r.tail_slots = launch->op == kWgrad ? 0 : launch->p.tail_slots;
  r.workspace_bytes = launch->workspace_bytes;
  *info = r;
  return status(MDG_OK);
}

MDG_API void grouped_det_gemm_launch_free(mdg_launch* launch) { delete launch; }

MDG_API mdg_status grouped_det_gemm_zero_pad_rows(void* out, const int32_t* offs, int64_t m_rows, int64_t row_bytes,
                                   int32_t num_groups, void* stream) {
  if (m_rows < 0 || row_bytes <= 0 || num_groups <= 0) return status(MDG_EINVAL);
  if (num_groups > kMaxGroups) return status(MDG_EUNSUPPORTED);
  if (row_bytes % 16 != 0 || m_rows > kMaxRows || row_bytes > (int64_t)1 << 24) return status(MDG_EUNSUPPORTED);
  if (!offs || (m_rows > 0 && !out)) return status(MDG_EINVAL);
  if (!aligned16(out) || !aligned4(offs)) return status(MDG_EINVAL);
  if (overlaps(range_of(out, m_rows * row_bytes), range_of(offs, (int64_t)num_groups * 4))) return status(MDG_EOVERLAP);
  if (m_rows == 0) return status(MDG_OK);

  DeviceInfo dev;
  int device = -1;
  const int st = query_device(&dev, &device);
  if (st != MDG_OK) return status(st);
  if (!dev.gfx950) return status(MDG_EUNSUPPORTED);
  const int64_t vecs = m_rows * (row_bytes / 16);
  const int64_t cap = 2 * (int64_t)(dev.cus > 0 ? dev.cus : 256);
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(cap, (vecs + kThreads - 1) / kThreads));
  if (launch_zero_rows(out, offs, num_groups, m_rows, row_bytes, grid, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return status(MDG_EHIP);
  return status(MDG_OK);
}

}  // extern "C"
