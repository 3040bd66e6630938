// C ABI of the MoE gate / dispatch / combine library: host-side argument checks,
// layout workspace carving and kernel launches. Every check runs before anything is
// enqueued; the library allocates no memory and keeps no device state between calls.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/moe_gate.h"
#include "internal.h"
#include "moe_device.h"

namespace {

constexpr uint64_t kLayoutMagic = 0x4d4f454c41594f54ull;  // "MOELAYOT"
constexpr size_t kAlign = 256;

thread_local std::string g_last_error;

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status_t hip_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: HIP error %d (%s)", what, static_cast<int>(err),
              hipGetErrorString(err));
}

size_t elem_bytes(moe_dtype_t dt) {
  switch (dt) {
    case MOE_F32: return 4;
    case MOE_BF16: return 2;
    case MOE_F16: return 2;
    default: return 0;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Sizes of a layout, and where each of its arrays sits in the workspace.
// The handle's arrays come first; the tile tables, which only the layout build itself
// uses, last, so that `handle_bytes` is the share a handle needs once it is built.
struct Plan {
  int64_t rows = 0;
  int32_t ntiles = 0;
  size_t off_counts = 0, off_kept = 0, off_offsets = 0, off_dst = 0, off_src = 0,
         off_route = 0, off_checksum = 0, off_flags = 0, off_tile_counts = 0,
         off_tile_checksum = 0, off_tile_flags = 0, handle_bytes = 0, bytes = 0;
};

size_t take(size_t& cursor, size_t nbytes) {
  cursor = (cursor + kAlign - 1) / kAlign * kAlign;
  const size_t at = cursor;
  cursor += nbytes;
  return at;
}

moe_status_t check_sizes(int32_t s, int32_t e, int32_t k, int32_t capacity) {
  if (s < 0) return fail(MOE_ERR_INVALID_ARG, "s must be >= 0 (got %d)", s);
  if (e < 1) return fail(MOE_ERR_INVALID_ARG, "e must be >= 1 (got %d)", e);
  if (k < 1 || k > e) return fail(MOE_ERR_INVALID_ARG, "k must be in [1, e] (got k=%d, e=%d)", k, e);
  if (e > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "e=%d exceeds MOE_MAX_EXPERTS=%d", e, MOE_MAX_EXPERTS);
  if (k > MOE_MAX_TOPK)
    return fail(MOE_ERR_UNSUPPORTED, "k=%d exceeds MOE_MAX_TOPK=%d", k, MOE_MAX_TOPK);
  if (s > INT32_MAX - 65536)
    return fail(MOE_ERR_UNSUPPORTED, "s=%d exceeds the supported token count", s);
  if (static_cast<int64_t>(s) * k > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "s*k=%lld exceeds 32-bit route ids",
                static_cast<long long>(s) * k);
  if (capacity > 0 && static_cast<int64_t>(e) * capacity > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "e*capacity=%lld exceeds 32-bit row ids",
                static_cast<long long>(e) * capacity);
  return MOE_OK;
}

struct Options {
  int32_t route_major = 0;
  int32_t pad_multiple = 1;
};

moe_status_t read_options(const moe_layout_options_t* o, int32_t s, int32_t e, int32_t k,
                          int32_t capacity, Options* out) {
  Options opt;
  if (o != nullptr) {
    opt.route_major = o->route_major;
    opt.pad_multiple = o->pad_multiple;
  }
  if (opt.route_major != 0 && opt.route_major != 1)
    return fail(MOE_ERR_INVALID_ARG, "route_major must be 0 or 1 (got %d)", opt.route_major);
  if (opt.pad_multiple < 1)
    return fail(MOE_ERR_INVALID_ARG, "pad_multiple must be >= 1 (got %d)", opt.pad_multiple);
  if (opt.pad_multiple > 1 && capacity > 0)
    return fail(MOE_ERR_INVALID_ARG, "pad_multiple applies to dropless layouts only");
  if (static_cast<int64_t>(s) * k + static_cast<int64_t>(e) * (opt.pad_multiple - 1) > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "padded row count exceeds 32-bit row ids");
  *out = opt;
  return MOE_OK;
}

Plan make_plan(int32_t s, int32_t e, int32_t k, int32_t capacity, const Options& opt) {
  Plan p;
  p.rows = capacity > 0 ? static_cast<int64_t>(e) * capacity
                        : static_cast<int64_t>(s) * k + static_cast<int64_t>(e) * (opt.pad_multiple - 1);
  const int64_t items = opt.route_major ? static_cast<int64_t>(s) * k : s;
  p.ntiles = static_cast<int32_t>((items + moe::kTileTokens - 1) / moe::kTileTokens);
  const size_t routes = static_cast<size_t>(s) * k;
  size_t cur = 0;
  p.off_counts = take(cur, sizeof(int32_t) * e);
  p.off_kept = take(cur, sizeof(int32_t) * e);
  p.off_offsets = take(cur, sizeof(int32_t) * (e + 1));
  p.off_dst = take(cur, sizeof(int32_t) * routes);
  p.off_src = take(cur, sizeof(int32_t) * static_cast<size_t>(p.rows));
  p.off_route = take(cur, sizeof(int32_t) * routes);
  p.off_checksum = take(cur, sizeof(uint64_t));
  p.off_flags = take(cur, sizeof(int32_t));
  p.handle_bytes = (cur + kAlign - 1) / kAlign * kAlign;
  p.off_tile_counts = take(cur, sizeof(int32_t) * static_cast<size_t>(moe::tile_row_length(p.ntiles)) * e);
  p.off_tile_checksum = take(cur, sizeof(uint64_t) * static_cast<size_t>(p.ntiles));
  p.off_tile_flags = take(cur, sizeof(int32_t) * static_cast<size_t>(p.ntiles));
  p.bytes = (cur + kAlign - 1) / kAlign * kAlign;
  return p;
}

// Rebuild the device view of a handle, checking that it is one of ours and consistent.
moe_status_t view_of(const moe_layout_t* h, moe::LayoutView* v) {
  if (h == nullptr) return fail(MOE_ERR_INVALID_ARG, "layout is NULL");
  if (h->magic != kLayoutMagic)
    return fail(MOE_ERR_HANDLE_MISMATCH, "layout was not filled by moe_dispatch_layout");
  moe_status_t st = check_sizes(h->s, h->e, h->k, h->capacity);
  if (st != MOE_OK) return fail(MOE_ERR_HANDLE_MISMATCH, "layout sizes invalid: %s", g_last_error.c_str());
  moe_layout_options_t o{h->route_major, h->pad_multiple};
  Options opt;
  st = read_options(&o, h->s, h->e, h->k, h->capacity, &opt);
  if (st != MOE_OK) return fail(MOE_ERR_HANDLE_MISMATCH, "layout options invalid: %s", g_last_error.c_str());
  const Plan p = make_plan(h->s, h->e, h->k, h->capacity, opt);
  if (h->rows != p.rows || h->workspace == nullptr || h->workspace_bytes < p.handle_bytes)
    return fail(MOE_ERR_HANDLE_MISMATCH, "layout fields are inconsistent with its sizes");
  char* ws = static_cast<char*>(h->workspace);
  if (reinterpret_cast<char*>(h->dst) != ws + p.off_dst ||
      reinterpret_cast<char*>(h->src) != ws + p.off_src ||
      reinterpret_cast<char*>(h->counts) != ws + p.off_counts)
    return fail(MOE_ERR_HANDLE_MISMATCH, "layout arrays do not point into its workspace");
  v->s = h->s;
  v->e = h->e;
  v->k = h->k;
  v->capacity = h->capacity > 0 ? h->capacity : 0;
  v->route_major = opt.route_major;
  v->pad_multiple = opt.pad_multiple;
  v->rows = p.rows;
  v->ntiles = p.ntiles;
  v->counts = reinterpret_cast<int32_t*>(ws + p.off_counts);
  v->kept = reinterpret_cast<int32_t*>(ws + p.off_kept);
  v->offsets = reinterpret_cast<int32_t*>(ws + p.off_offsets);
  v->dst = reinterpret_cast<int32_t*>(ws + p.off_dst);
  v->src = reinterpret_cast<int32_t*>(ws + p.off_src);
  v->route_idx = reinterpret_cast<int32_t*>(ws + p.off_route);
  v->checksum = reinterpret_cast<uint64_t*>(ws + p.off_checksum);
  v->flags = reinterpret_cast<int32_t*>(ws + p.off_flags);
  // the tile tables are in the workspace only if it was sized for them (a layout built
  // with moe_dispatch_layout_static_scratch had them elsewhere); only a build uses them
  const bool tables = h->workspace_bytes >= p.bytes;
  v->tile_counts = tables ? reinterpret_cast<int32_t*>(ws + p.off_tile_counts) : nullptr;
  v->tile_checksum = tables ? reinterpret_cast<uint64_t*>(ws + p.off_tile_checksum) : nullptr;
  v->tile_flags = tables ? reinterpret_cast<int32_t*>(ws + p.off_tile_flags) : nullptr;
  return MOE_OK;
}

// Checks shared by the row calls: element type, row length and alignment, and that a
// non-empty array is not NULL.
moe_status_t check_rows(int32_t m, moe_dtype_t dtype, int64_t* row_chunks) {
  const size_t eb = elem_bytes(dtype);
  if (eb == 0) return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", static_cast<int>(dtype));
  if (m < 1) return fail(MOE_ERR_INVALID_ARG, "m must be >= 1 (got %d)", m);
  const size_t row_bytes = eb * static_cast<size_t>(m);
  if (row_bytes % 16 != 0)
    return fail(MOE_ERR_MISALIGNED, "row length m*%zu = %zu bytes is not a multiple of 16", eb,
                row_bytes);
  *row_chunks = static_cast<int64_t>(row_bytes / 16);
  return MOE_OK;
}

moe_status_t check_array(const void* p, int64_t n_rows, const char* name, bool rows16) {
  if (n_rows == 0) return MOE_OK;
  if (p == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);
  if (rows16 && !aligned16(p)) return fail(MOE_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

#define MOE_TRY(expr)                      \
  do {                                     \
    const moe_status_t st_ = (expr);       \
    if (st_ != MOE_OK) return st_;         \
  } while (0)

// ---------------------------------------------------------------------------------
// Static scratch for moe_dispatch_layout_static_scratch: the layout's tile tables in a
// device array of the library's own, for callers that cannot allocate.

constexpr size_t kStaticScratchBytes = static_cast<size_t>(2) << 20;  // 2 MiB per GPU
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

}  // namespace

// One copy per GPU the library's code is loaded on, held until the process ends. On the
// host, `scratch` names only a stand-in: host code uses the device address that
// scratch_address() looks up, never the name.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

// The address of `scratch` on the device the stream belongs to (the current device for
// the null stream), looked up once per device with that device current (each GPU holds
// its own copy at its own address; the caller's current device is restored), then kept.
moe_status_t scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t err = hipSuccess;
  if (stream == nullptr) {
    err = hipGetDevice(&dev);
  } else {
    hipDevice_t sdev = 0;
    err = hipStreamGetDevice(stream, &sdev);
    dev = static_cast<int>(sdev);
  }
  if (err != hipSuccess) return hip_status(err, "moe_dispatch_layout_static_scratch: the stream's device");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d is beyond the %d devices the static scratch tracks",
                dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    int cur = -1;
    err = hipGetDevice(&cur);
    if (err != hipSuccess) return hip_status(err, "moe_dispatch_layout_static_scratch: hipGetDevice");
    if (cur != dev && (err = hipSetDevice(dev)) != hipSuccess)
      return hip_status(err, "moe_dispatch_layout_static_scratch: hipSetDevice");
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t restore = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (err != hipSuccess)
      return hip_status(err, "moe_dispatch_layout_static_scratch: hipGetSymbolAddress(scratch)");
    if (restore != hipSuccess)
      return hip_status(restore, "moe_dispatch_layout_static_scratch: restoring the current device");
    if (p == nullptr)
      return fail(MOE_ERR_HIP, "moe_dispatch_layout_static_scratch: hipGetSymbolAddress gave NULL");
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_last_error.c_str(); }

const char* moe_status_string(moe_status_t status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HANDLE_MISMATCH: return "MOE_ERR_HANDLE_MISMATCH";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_STATUS_UNKNOWN";
  }
}

size_t moe_layout_workspace_bytes_ex(int32_t s, int32_t e, int32_t k, int32_t capacity,
                                     const moe_layout_options_t* options) {
  const std::string saved = g_last_error;
  if (capacity < 0) capacity = 0;
  Options opt;
  if (check_sizes(s, e, k, capacity) != MOE_OK ||
      read_options(options, s, e, k, capacity, &opt) != MOE_OK) {
    g_last_error = saved;
    return 0;
  }
  return make_plan(s, e, k, capacity, opt).bytes;
}

size_t moe_layout_workspace_bytes(int32_t s, int32_t e, int32_t k, int32_t capacity) {
  return moe_layout_workspace_bytes_ex(s, e, k, capacity, nullptr);
}

moe_status_t moe_gate_topk(const float* logits, int32_t s, int32_t e, int32_t k,
                           int32_t* topk_idx, float* topk_w, void* stream) {
  MOE_TRY(check_sizes(s, e, k, 0));
  MOE_TRY(check_array(logits, s, "logits", false));
  MOE_TRY(check_array(topk_idx, s, "topk_idx", false));
  MOE_TRY(check_array(topk_w, s, "topk_w", false));
  return hip_status(moe::launch_gate_topk(logits, s, e, k, topk_idx, topk_w,
                                          static_cast<hipStream_t>(stream)),
                    "moe_gate_topk");
}

moe_status_t moe_gate_topk_backward(const int32_t* topk_idx, const float* topk_w,
                                    const float* grad_w, int32_t s, int32_t e, int32_t k,
                                    float* grad_logits, void* stream) {
  MOE_TRY(check_sizes(s, e, k, 0));
  MOE_TRY(check_array(topk_idx, s, "topk_idx", false));
  MOE_TRY(check_array(topk_w, s, "topk_w", false));
  MOE_TRY(check_array(grad_w, s, "grad_w", false));
  MOE_TRY(check_array(grad_logits, s, "grad_logits", false));
  return hip_status(moe::launch_gate_topk_backward(topk_idx, topk_w, grad_w, s, e, k,
                                                   grad_logits, static_cast<hipStream_t>(stream)),
                    "moe_gate_topk_backward");
}

moe_status_t moe_dispatch_layout(const int32_t* topk_idx, int32_t s, int32_t e, int32_t k,
                                 int32_t capacity, void* workspace, size_t workspace_bytes,
                                 moe_layout_t* layout, void* stream) {
  return moe_dispatch_layout_ex(topk_idx, s, e, k, capacity, nullptr, workspace, workspace_bytes,
                                layout, stream);
}

// Checks, fills the handle and launches the layout build. The tile tables go to
// `tables` if given (the static scratch array: the workspace then needs only the
// handle's share), else to the workspace's own tile region.
static moe_status_t build_layout(const int32_t* topk_idx, int32_t s, int32_t e, int32_t k,
                                 int32_t capacity, const moe_layout_options_t* options,
                                 void* workspace, size_t workspace_bytes, moe_layout_t* layout,
                                 void* stream, bool static_tables, const char* what) {
  if (capacity < 0) capacity = 0;
  MOE_TRY(check_sizes(s, e, k, capacity));
  Options opt;
  MOE_TRY(read_options(options, s, e, k, capacity, &opt));
  if (layout == nullptr) return fail(MOE_ERR_INVALID_ARG, "layout is NULL");
  MOE_TRY(check_array(topk_idx, s, "topk_idx", false));
  if (workspace == nullptr) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return fail(MOE_ERR_MISALIGNED, "workspace is not %zu-byte aligned", kAlign);
  const Plan p = make_plan(s, e, k, capacity, opt);
  const size_t need = static_tables ? p.handle_bytes : p.bytes;
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, the layout needs %zu", workspace_bytes, need);
  char* tables = nullptr;
  if (static_tables) {
    const size_t table_bytes = p.bytes - p.handle_bytes;
    if (table_bytes > kStaticScratchBytes)
      return fail(MOE_ERR_UNSUPPORTED,
                  "%s: the layout's tile tables need %zu bytes, more than the %zu of the static "
                  "scratch array (fewer tokens or experts per call, or moe_dispatch_layout_ex)",
                  what, table_bytes, kStaticScratchBytes);
    void* base = nullptr;
    MOE_TRY(scratch_address(static_cast<hipStream_t>(stream), &base));
    tables = static_cast<char*>(base);
  }

  char* ws = static_cast<char*>(workspace);
  moe_layout_t h;
  std::memset(&h, 0, sizeof(h));
  h.magic = kLayoutMagic;
  h.s = s;
  h.e = e;
  h.k = k;
  h.capacity = capacity;
  h.route_major = opt.route_major;
  h.pad_multiple = opt.pad_multiple;
  h.rows = p.rows;
  h.counts = reinterpret_cast<int32_t*>(ws + p.off_counts);
  h.kept = reinterpret_cast<int32_t*>(ws + p.off_kept);
  h.offsets = reinterpret_cast<int32_t*>(ws + p.off_offsets);
  h.dst = reinterpret_cast<int32_t*>(ws + p.off_dst);
  h.src = reinterpret_cast<int32_t*>(ws + p.off_src);
  h.route_idx = reinterpret_cast<int32_t*>(ws + p.off_route);
  h.checksum = reinterpret_cast<uint64_t*>(ws + p.off_checksum);
  h.flags = reinterpret_cast<int32_t*>(ws + p.off_flags);
  h.scratch = static_tables ? nullptr : ws + p.off_tile_counts;
  h.workspace = workspace;
  h.workspace_bytes = workspace_bytes;

  moe::LayoutView v;
  MOE_TRY(view_of(&h, &v));
  if (static_tables) {  // same offsets within the tables as in a full workspace
    v.tile_counts = reinterpret_cast<int32_t*>(tables + (p.off_tile_counts - p.handle_bytes));
    v.tile_checksum = reinterpret_cast<uint64_t*>(tables + (p.off_tile_checksum - p.handle_bytes));
    v.tile_flags = reinterpret_cast<int32_t*>(tables + (p.off_tile_flags - p.handle_bytes));
  }
  const moe_status_t st =
      hip_status(moe::launch_layout(topk_idx, v, static_cast<hipStream_t>(stream)), what);
  if (st == MOE_OK) *layout = h;
  return st;
}

moe_status_t moe_dispatch_layout_ex(const int32_t* topk_idx, int32_t s, int32_t e, int32_t k,
                                    int32_t capacity, const moe_layout_options_t* options,
                                    void* workspace, size_t workspace_bytes,
                                    moe_layout_t* layout, void* stream) {
  return build_layout(topk_idx, s, e, k, capacity, options, workspace, workspace_bytes, layout,
                      stream, false, "moe_dispatch_layout");
}

moe_status_t moe_dispatch_layout_static_scratch(const int32_t* topk_idx, int32_t s, int32_t e,
                                                int32_t k, int32_t capacity,
                                                const moe_layout_options_t* options,
                                                void* workspace, size_t workspace_bytes,
                                                moe_layout_t* layout, void* stream) {
  return build_layout(topk_idx, s, e, k, capacity, options, workspace, workspace_bytes, layout,
                      stream, true, "moe_dispatch_layout_static_scratch");
}

static moe_status_t dispatch_common(const moe_layout_t* layout, const int32_t* verify_idx,
                                    const void* x, int32_t m, moe_dtype_t dtype, void* out,
                                    void* stream, const char* what) {
  moe::LayoutView v;
  MOE_TRY(view_of(layout, &v));
  int64_t rc = 0;
  MOE_TRY(check_rows(m, dtype, &rc));
  MOE_TRY(check_array(x, v.s, "x", true));
  MOE_TRY(check_array(out, v.rows, "out", true));
  return hip_status(moe::launch_dispatch(v, verify_idx, x, rc, out, static_cast<hipStream_t>(stream)),
                    what);
}

moe_status_t moe_dispatch(const moe_layout_t* layout, const void* x, int32_t m,
                          moe_dtype_t dtype, void* out, void* stream) {
  return dispatch_common(layout, nullptr, x, m, dtype, out, stream, "moe_dispatch");
}

moe_status_t moe_dispatch_replay(const moe_layout_t* layout, const int32_t* topk_idx,
                                 const void* x, int32_t m, moe_dtype_t dtype, void* out,
                                 void* stream) {
  return dispatch_common(layout, topk_idx, x, m, dtype, out, stream, "moe_dispatch_replay");
}

moe_status_t moe_combine(const moe_layout_t* layout, const void* expert_out,
                         const float* topk_w, int32_t m, moe_dtype_t dtype, void* y,
                         void* stream) {
  moe::LayoutView v;
  MOE_TRY(view_of(layout, &v));
  int64_t rc = 0;
  MOE_TRY(check_rows(m, dtype, &rc));
  MOE_TRY(check_array(expert_out, v.s > 0 ? v.rows : 0, "expert_out", true));
  MOE_TRY(check_array(y, v.s, "y", true));
  return hip_status(moe::launch_combine(v, expert_out, topk_w, rc, static_cast<int>(dtype), y,
                                        static_cast<hipStream_t>(stream)),
                    "moe_combine");
}

moe_status_t moe_dispatch_weighted(const moe_layout_t* layout, const void* x,
                                   const float* topk_w, int32_t m, moe_dtype_t dtype, void* out,
                                   void* stream) {
  moe::LayoutView v;
  MOE_TRY(view_of(layout, &v));
  int64_t rc = 0;
  MOE_TRY(check_rows(m, dtype, &rc));
  MOE_TRY(check_array(x, v.s, "x", true));
  MOE_TRY(check_array(topk_w, v.s, "topk_w", false));
  MOE_TRY(check_array(out, v.rows, "out", true));
  return hip_status(moe::launch_dispatch_weighted(v, x, topk_w, rc, static_cast<int>(dtype), out,
                                                  static_cast<hipStream_t>(stream)),
                    "moe_dispatch_weighted");
}

moe_status_t moe_dispatch_weighted_backward(const moe_layout_t* layout, const void* grad_out,
                                            const void* x, const float* topk_w, int32_t m,
                                            moe_dtype_t dtype, void* grad_x, float* grad_w,
                                            void* stream) {
  moe::LayoutView v;
  MOE_TRY(view_of(layout, &v));
  int64_t rc = 0;
  MOE_TRY(check_rows(m, dtype, &rc));
  MOE_TRY(check_array(grad_out, v.s > 0 ? v.rows : 0, "grad_out", true));
  MOE_TRY(check_array(x, v.s, "x", true));
  MOE_TRY(check_array(topk_w, v.s, "topk_w", false));
  MOE_TRY(check_array(grad_x, v.s, "grad_x", true));
  MOE_TRY(check_array(grad_w, v.s, "grad_w", false));
  return hip_status(moe::launch_dispatch_weighted_backward(v, grad_out, x, topk_w, rc,
                                                           static_cast<int>(dtype), grad_x, grad_w,
                                                           static_cast<hipStream_t>(stream)),
                    "moe_dispatch_weighted_backward");
}

moe_status_t moe_expert_gemm(const moe_layout_t* layout, const void* a, int32_t gather,
                             const void* weights, int32_t m, int32_t n, moe_dtype_t dtype,
                             const float* topk_w, void* out, void* stream) {
  moe::LayoutView v;
  MOE_TRY(view_of(layout, &v));
  if (dtype != MOE_BF16 && dtype != MOE_F16)
    return fail(MOE_ERR_UNSUPPORTED, "moe_expert_gemm supports bf16 and f16 only (got dtype %d)",
                static_cast<int>(dtype));
  if (gather != 0 && gather != 1)
    return fail(MOE_ERR_INVALID_ARG, "gather must be 0 or 1 (got %d)", gather);
  int64_t rc_in = 0, rc_out = 0;
  MOE_TRY(check_rows(m, dtype, &rc_in));
  MOE_TRY(check_rows(n, dtype, &rc_out));
  if (v.s > 0 && moe::expert_gemm_grid(v, n) > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "rows x n too large for one grouped GEMM launch");
  const int64_t a_rows = gather ? v.s : v.rows;
  MOE_TRY(check_array(a, v.s > 0 ? a_rows : 0, "a", true));
  MOE_TRY(check_array(weights, v.s > 0 ? v.e : 0, "weights", true));
  MOE_TRY(check_array(topk_w, topk_w != nullptr ? v.s : 0, "topk_w", false));
  MOE_TRY(check_array(out, v.rows, "out", true));
  if (v.rows > 0 && a_rows > 0) {
    const char* ob = static_cast<const char*>(out);
    const char* ab = static_cast<const char*>(a);
    const size_t eb = elem_bytes(dtype);
    if (ob < ab + a_rows * m * eb && ab < ob + v.rows * n * eb)
      return fail(MOE_ERR_INVALID_ARG, "a and out may not overlap");
  }
  return hip_status(moe::launch_expert_gemm(v, a, gather != 0, weights, topk_w, m, n,
                                            static_cast<int>(dtype), out,
                                            static_cast<hipStream_t>(stream)),
                    "moe_expert_gemm");
}

moe_status_t moe_expert_gemm_wgrad(const moe_layout_t* layout, const void* a, int32_t gather,
                                   const void* grad_out, int32_t m, int32_t n, moe_dtype_t dtype,
                                   moe_dtype_t grad_w_dtype, void* grad_w, void* stream) {
  moe::LayoutView v;
  MOE_TRY(view_of(layout, &v));
  if (dtype != MOE_BF16 && dtype != MOE_F16)
    return fail(MOE_ERR_UNSUPPORTED, "moe_expert_gemm_wgrad supports bf16 and f16 only (got dtype %d)",
                static_cast<int>(dtype));
  if (grad_w_dtype != MOE_F32 && grad_w_dtype != dtype)
    return fail(MOE_ERR_UNSUPPORTED, "grad_w_dtype must be float32 or dtype (got %d, dtype %d)",
                static_cast<int>(grad_w_dtype), static_cast<int>(dtype));
  if (gather != 0 && gather != 1)
    return fail(MOE_ERR_INVALID_ARG, "gather must be 0 or 1 (got %d)", gather);
  int64_t rc_in = 0, rc_out = 0;
  MOE_TRY(check_rows(m, dtype, &rc_in));
  MOE_TRY(check_rows(n, dtype, &rc_out));
  const int64_t tiles = static_cast<int64_t>((n + 255) / 256) * ((m + 255) / 256) * v.e;
  if (tiles > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "e x n x m too large for one weight-gradient launch");
  const int64_t a_rows = gather ? v.s : v.rows;
  MOE_TRY(check_array(a, v.s > 0 ? a_rows : 0, "a", true));
  MOE_TRY(check_array(grad_out, v.s > 0 ? v.rows : 0, "grad_out", true));
  MOE_TRY(check_array(grad_w, v.e, "grad_w", true));
  const char* wb = static_cast<const char*>(grad_w);
  const size_t w_bytes = static_cast<size_t>(v.e) * n * m * elem_bytes(grad_w_dtype);
  const size_t eb = elem_bytes(dtype);
  const struct {
    const void* p;
    size_t bytes;
  } inputs[2] = {{a, static_cast<size_t>(a_rows) * m * eb}, {grad_out, static_cast<size_t>(v.rows) * n * eb}};
  for (const auto& in : inputs) {
    const char* ib = static_cast<const char*>(in.p);
    if (v.s > 0 && in.bytes > 0 && wb < ib + in.bytes && ib < wb + w_bytes)
      return fail(MOE_ERR_INVALID_ARG, "grad_w may not overlap a or grad_out");
  }
  return hip_status(moe::launch_expert_gemm_wgrad(v, a, gather != 0, grad_out, m, n,
                                                  static_cast<int>(dtype), grad_w_dtype == MOE_F32,
                                                  grad_w, static_cast<hipStream_t>(stream)),
                    "moe_expert_gemm_wgrad");
}

moe_status_t moe_expert_gemm_dgrad(const moe_layout_t* layout, const void* grad_out,
                                   const void* weights, int32_t m, int32_t n, moe_dtype_t dtype,
                                   void* grad_a, void* stream) {
  moe::LayoutView v;
  MOE_TRY(view_of(layout, &v));
  if (dtype != MOE_BF16 && dtype != MOE_F16)
    return fail(MOE_ERR_UNSUPPORTED, "moe_expert_gemm_dgrad supports bf16 and f16 only (got dtype %d)",
                static_cast<int>(dtype));
  int64_t rc_in = 0, rc_out = 0;
  MOE_TRY(check_rows(m, dtype, &rc_in));
  MOE_TRY(check_rows(n, dtype, &rc_out));
  if (v.s > 0 && moe::expert_gemm_kn_grid(v, m) > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "rows x m too large for one input-gradient launch");
  MOE_TRY(check_array(grad_out, v.s > 0 ? v.rows : 0, "grad_out", true));
  MOE_TRY(check_array(weights, v.s > 0 ? v.e : 0, "weights", true));
  MOE_TRY(check_array(grad_a, v.rows, "grad_a", true));
  if (v.rows > 0) {
    const char* ob = static_cast<const char*>(grad_a);
    const char* gb = static_cast<const char*>(grad_out);
    const size_t eb = elem_bytes(dtype);
    if (ob < gb + v.rows * n * eb && gb < ob + v.rows * m * eb)
      return fail(MOE_ERR_INVALID_ARG, "grad_out and grad_a may not overlap");
  }
  // grad_a = grad_out @ W[x]: the grouped GEMM with K = n, N = m, the weights read [K][N]
  return hip_status(moe::launch_expert_gemm_kn(v, grad_out, weights, n, m, static_cast<int>(dtype), grad_a,
                                               static_cast<hipStream_t>(stream)),
                    "moe_expert_gemm_dgrad");
}

moe_status_t moe_renormalize_kept(const moe_layout_t* layout, const float* topk_w, float* w_out,
                                  void* stream) {
  moe::LayoutView v;
  MOE_TRY(view_of(layout, &v));
  MOE_TRY(check_array(topk_w, v.s, "topk_w", false));
  MOE_TRY(check_array(w_out, v.s, "w_out", false));
  if (v.s > 0 && topk_w == w_out) return fail(MOE_ERR_INVALID_ARG, "topk_w and w_out may not overlap");
  return hip_status(moe::launch_renormalize_kept(v, topk_w, w_out, static_cast<hipStream_t>(stream)),
                    "moe_renormalize_kept");
}

moe_status_t moe_renormalize_kept_backward(const moe_layout_t* layout, const float* topk_w,
                                           const float* grad_out, float* grad_w, void* stream) {
  moe::LayoutView v;
  MOE_TRY(view_of(layout, &v));
  MOE_TRY(check_array(topk_w, v.s, "topk_w", false));
  MOE_TRY(check_array(grad_out, v.s, "grad_out", false));
  MOE_TRY(check_array(grad_w, v.s, "grad_w", false));
  return hip_status(moe::launch_renormalize_kept_backward(v, topk_w, grad_out, grad_w,
                                                          static_cast<hipStream_t>(stream)),
                    "moe_renormalize_kept_backward");
}

moe_status_t moe_combine_backward(const moe_layout_t* layout, const void* grad_y,
                                  const void* expert_out, const float* topk_w, int32_t m,
                                  moe_dtype_t dtype, void* grad_expert_out, float* grad_w,
                                  void* stream) {
  moe::LayoutView v;
  MOE_TRY(view_of(layout, &v));
  int64_t rc = 0;
  MOE_TRY(check_rows(m, dtype, &rc));
  MOE_TRY(check_array(grad_y, v.s, "grad_y", true));
  MOE_TRY(check_array(expert_out, v.s > 0 ? v.rows : 0, "expert_out", true));
  MOE_TRY(check_array(topk_w, v.s, "topk_w", false));
  MOE_TRY(check_array(grad_expert_out, v.rows, "grad_expert_out", true));
  MOE_TRY(check_array(grad_w, v.s, "grad_w", false));
  return hip_status(moe::launch_combine_backward(v, grad_y, expert_out, topk_w, rc,
                                                 static_cast<int>(dtype), grad_expert_out, grad_w,
                                                 static_cast<hipStream_t>(stream)),
                    "moe_combine_backward");
}

moe_status_t moe_dispatch_backward(const moe_layout_t* layout, const void* grad_out,
                                   int32_t m, moe_dtype_t dtype, void* grad_x, void* stream) {
  moe::LayoutView v;
  MOE_TRY(view_of(layout, &v));
  int64_t rc = 0;
  MOE_TRY(check_rows(m, dtype, &rc));
  MOE_TRY(check_array(grad_out, v.s > 0 ? v.rows : 0, "grad_out", true));
  MOE_TRY(check_array(grad_x, v.s, "grad_x", true));
  return hip_status(moe::launch_combine(v, grad_out, nullptr, rc, static_cast<int>(dtype), grad_x,
                                        static_cast<hipStream_t>(stream)),
                    "moe_dispatch_backward");
}

moe_status_t moe_layout_read(const moe_layout_t* layout, int32_t* flags_host,
                             uint64_t* checksum_host, void* stream) {
  moe::LayoutView v;
  MOE_TRY(view_of(layout, &v));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (flags_host != nullptr)
    MOE_TRY(hip_status(hipMemcpyAsync(flags_host, v.flags, sizeof(int32_t), hipMemcpyDeviceToHost, st),
                       "moe_layout_read"));
  if (checksum_host != nullptr)
    MOE_TRY(hip_status(hipMemcpyAsync(checksum_host, v.checksum, sizeof(uint64_t),
                                      hipMemcpyDeviceToHost, st),
                       "moe_layout_read"));
  return hip_status(hipStreamSynchronize(st), "moe_layout_read");
}

}  // extern "C"
