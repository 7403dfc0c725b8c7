// bsa_api.cpp -- the C ABI declared in include/bsa.h: argument validation,
// the per-handle workspace, the order of the kernel launches, per-stage
// timing.  Every step of the computation runs in the gfx950 kernels; this
// file only checks, allocates and enqueues.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "bsa.h"
#include "bsa_launch.hpp"

#define BSA_API extern "C" __attribute__((visibility("default")))

struct bsa_handle_s {
  int device = 0;
  void* noalloc = nullptr;  // device address of the fixed workspace on this device
  char err[512] = {0};
  // workspace
  float* repr = nullptr;
  size_t repr_bytes = 0;
  uint16_t* split = nullptr;  // bf16 three-term split of repr, for the fused selection
  size_t split_bytes = 0;
  float* panel = nullptr;
  size_t panel_bytes = 0;
  int32_t* idx = nullptr;
  size_t idx_bytes = 0;
  int64_t panel_chunk_bytes = int64_t(128) << 20;
  int select_strategy = BSA_SELECT_FUSED;
  // block-gather workspace
  int fine_strategy = BSA_FINE_BLOCK_GATHER;
  int64_t fine_chunk_bytes = int64_t(1) << 30;
  struct Buf {
    void* p = nullptr;
    size_t bytes = 0;
  };
  Buf g_count, g_offsets, g_items, g_item_rec, g_rank, g_rec, g_wgv, g_list, g_po;
  // backward: per-row (lse, delta), per-pair dq, per-item dk/dv, bf16 dout
  Buf b_ld, b_dq, b_dkv, b_dob;
  bool counts_zero = false;  // g_count holds zeros (the bucketing's scan leaves it so)
  Buf r_q, r_k, r_v, r_o, r_do, r_lse, r_idx, r_dq, r_dk, r_dv;  // padded copies (ragged lengths)
  // block table of sequences padded to whole blocks: device copy, pinned
  // staging copy, and an event on the last upload from the staging copy
  Buf tab;
  void* tab_host = nullptr;
  size_t tab_host_bytes = 0;
  hipEvent_t tab_ev = nullptr;
  bool tab_ev_live = false;
  Buf s_part, s_lse;  // static mode: partial rows of split query tiles and their log-sum-exp
  int64_t static_item_tiles = 0;  // 0: chosen per call; else the most key tiles per work item
  int union_rows = 64;            // query-tile rows of the query-tile union fine stage
  int32_t* fallbacks = nullptr;   // device counters [4]: fused-selection second walks, exact fallbacks,
                                  // and the repair list's counters (one per call parity)
  int repair_parity = 0;          // parity of the next call of the selection's split instance
  Buf sel_repair;                 // the split instance's repair list, one int per select workgroup
  // timing
  bool profiling = false;
  struct Rec {
    int stage;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> free_events;
};

// A validated static tile list in device memory (bsa_tiles_create), with the
// work-item schedules made from it so far (one per item size).
struct bsa_tiles_s {
  int device = 0;
  int n = 0, nt = 0;
  int64_t nnz = 0;
  std::vector<int32_t> row_ptr;   // host copy [nt + 1]
  int32_t* col = nullptr;         // device [nnz]
  uint64_t* rowmask = nullptr;    // device [nnz][64], or NULL
  struct Schedule {
    int64_t S = 0;                // most key tiles per item
    std::vector<int4> items, split;  // host copies (kept while the device copies may be read)
    int nslots = 0;
    int4* d_items = nullptr;
    int4* d_split = nullptr;
  };
  std::vector<Schedule> schedules;
};

namespace bsa {
bsa_status tiles_check(const int32_t* row_ptr, const int32_t* col, const uint64_t* rowmask, int64_t nnz,
                       int n, int tile, char* why, size_t why_len);
}

namespace {

thread_local char g_err[512] = {0};

bsa_status fail(bsa_handle h, bsa_status s, const char* fmt, ...) {
  char* buf = h ? h->err : g_err;
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, 512, fmt, ap);
  va_end(ap);
  return s;
}

class DeviceGuard {
 public:
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev_) != hipSuccess) prev_ = -1;
    if (prev_ != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev_ >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev_) (void)hipSetDevice(prev_);
  }

 private:
  int prev_ = -1;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bsa_status grow(bsa_handle h, void** ptr, size_t* have, size_t need, const char* what) {
  if (*have >= need) return BSA_OK;
  if (*ptr) {
    (void)hipFree(*ptr);
    *ptr = nullptr;
    *have = 0;
  }
  if (getenv("BSA_TEST_FAIL_ALLOC") && std::strcmp(getenv("BSA_TEST_FAIL_ALLOC"), "1") == 0)
    return fail(h, BSA_ERR_OUT_OF_MEMORY, "%s: allocation of %zu bytes refused (BSA_TEST_FAIL_ALLOC)",
                what, need);
  if (hipMalloc(ptr, need) != hipSuccess) {
    (void)hipGetLastError();
    *ptr = nullptr;
    return fail(h, BSA_ERR_OUT_OF_MEMORY, "%s: hipMalloc(%zu) failed", what, need);
  }
  *have = need;
  return BSA_OK;
}

hipEvent_t take_event(bsa_handle h) {
  if (!h->free_events.empty()) {
    hipEvent_t e = h->free_events.back();
    h->free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Launch `fn` (returning hipError_t) for `stage`, bracketed by events when
// timing is on.
template <typename F>
bsa_status timed_launch(bsa_handle h, int stage, hipStream_t s, const char* what, F&& fn) {
  hipEvent_t a = nullptr, b = nullptr;
  if (h->profiling) {
    a = take_event(h);
    b = take_event(h);
    if (!a || !b || hipEventRecord(a, s) != hipSuccess)
      return fail(h, BSA_ERR_LAUNCH, "%s: could not record a timing event", what);
  }
  const hipError_t e = fn();
  if (e != hipSuccess)
    return fail(h, BSA_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  if (h->profiling) {
    if (hipEventRecord(b, s) != hipSuccess)
      return fail(h, BSA_ERR_LAUNCH, "%s: could not record a timing event", what);
    h->recs.push_back({stage, a, b});
  }
  return BSA_OK;
}

struct Shape {
  int batch, heads, n, d;
  int64_t bh() const { return int64_t(batch) * heads; }
  int64_t elems() const { return bh() * n * d; }
  // The same problem with n rounded up to whole 64-key blocks.
  Shape padded() const { return Shape{batch, heads, (n + 63) / 64 * 64, d}; }
};

bsa_status check_shape(bsa_handle h, const char* fn, const Shape& s, bsa_dtype dtype, int block,
                       bool ragged_ok = false) {
  if (s.batch < 1 || s.heads < 1 || s.n < 1 || s.d < 1)
    return fail(h, BSA_ERR_INVALID_ARG, "%s: batch, heads, n and d must be >= 1 (got %d, %d, %d, %d)",
                fn, s.batch, s.heads, s.n, s.d);
  if (dtype != BSA_FP32 && dtype != BSA_BF16)
    return fail(h, BSA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, int(dtype));
  if (block != 64)
    return fail(h, BSA_ERR_UNSUPPORTED, "%s: block must be 64 (got %d)", fn, block);
  if (s.d != 64 && s.d != 128)
    return fail(h, BSA_ERR_UNSUPPORTED, "%s: d must be 64 or 128 (got %d)", fn, s.d);
  if (s.n % 64 != 0 && !ragged_ok)
    return fail(h, BSA_ERR_UNSUPPORTED, "%s: n must be a multiple of 64 (got %d)", fn, s.n);
  if (s.bh() * s.n > (int64_t(1) << 31) / 1 || s.elems() > (int64_t(1) << 40))
    return fail(h, BSA_ERR_UNSUPPORTED, "%s: problem too large (batch*heads*n = %lld)", fn,
                (long long)(s.bh() * s.n));
  return BSA_OK;
}

bsa_status check_ptr(bsa_handle h, const char* fn, const char* name, const void* p) {
  if (!p) return fail(h, BSA_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
  if (!aligned16(p)) return fail(h, BSA_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, name);
  return BSA_OK;
}

bsa_status check_scale(bsa_handle h, const char* fn, float scale) {
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(h, BSA_ERR_INVALID_ARG, "%s: scale must be finite and > 0 (got %g)", fn, double(scale));
  return BSA_OK;
}

bsa_status check_dynamic(bsa_handle h, const char* fn, const Shape& s, int topk, int causal) {
  if (topk < 1) return fail(h, BSA_ERR_INVALID_ARG, "%s: topk must be >= 1 (got %d)", fn, topk);
  if (causal != 0 && causal != 1)
    return fail(h, BSA_ERR_INVALID_ARG, "%s: causal must be 0 or 1 (got %d)", fn, causal);
  if ((s.n + 63) / 64 > 2048)
    return fail(h, BSA_ERR_UNSUPPORTED, "%s: ceil(n/64) must be <= 2048 (got %d)", fn, (s.n + 63) / 64);
  return BSA_OK;
}

#define TRY(expr)                     \
  do {                                \
    const bsa_status _st = (expr);    \
    if (_st != BSA_OK) return _st;    \
  } while (0)

}  // namespace

// ------------------------------------------------------------- lifetime --

BSA_API const char* bsa_status_string(bsa_status s) {
  switch (s) {
    case BSA_OK: return "ok";
    case BSA_ERR_INVALID_ARG: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported";
    case BSA_ERR_NO_DEVICE: return "no gfx950 device";
    case BSA_ERR_OUT_OF_MEMORY: return "out of device memory";
    case BSA_ERR_LAUNCH: return "launch failed";
  }
  return "unknown status";
}

BSA_API const char* bsa_last_error(bsa_handle h) { return h ? h->err : g_err; }

BSA_API bsa_status bsa_create(int device, bsa_handle* out) {
  if (!out) return fail(nullptr, BSA_ERR_INVALID_ARG, "bsa_create: out is NULL");
  *out = nullptr;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
    (void)hipGetLastError();
    return fail(nullptr, BSA_ERR_NO_DEVICE, "bsa_create: no HIP device");
  }
  if (device < 0 || device >= count)
    return fail(nullptr, BSA_ERR_NO_DEVICE, "bsa_create: device %d out of range (count %d)", device, count);
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess)
    return fail(nullptr, BSA_ERR_NO_DEVICE, "bsa_create: cannot query device %d", device);
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(nullptr, BSA_ERR_NO_DEVICE, "bsa_create: device %d is %s, not gfx950", device,
                prop.gcnArchName);
  void* arena = nullptr;
  {
    DeviceGuard dg(device);
    const hipError_t e = bsa::noalloc_scratch(device, &arena);
    if (e != hipSuccess)
      return fail(nullptr, BSA_ERR_NO_DEVICE, "bsa_create: cannot locate the fixed workspace on device %d: %s",
                  device, hipGetErrorString(e));
  }
  bsa_handle h = new (std::nothrow) bsa_handle_s();
  if (!h) return fail(nullptr, BSA_ERR_OUT_OF_MEMORY, "bsa_create: host allocation failed");
  h->device = device;
  h->noalloc = arena;
  {
    DeviceGuard dg(device);
    if (hipMalloc(reinterpret_cast<void**>(&h->fallbacks), 4 * sizeof(int32_t)) != hipSuccess ||
        hipMemset(h->fallbacks, 0, 4 * sizeof(int32_t)) != hipSuccess) {
      (void)hipGetLastError();
      if (h->fallbacks) (void)hipFree(h->fallbacks);
      delete h;
      return fail(nullptr, BSA_ERR_OUT_OF_MEMORY, "bsa_create: cannot allocate the handle's counter");
    }
  }
  *out = h;
  return BSA_OK;
}

BSA_API bsa_status bsa_destroy(bsa_handle h) {
  if (!h) return BSA_OK;
  DeviceGuard dg(h->device);
  for (auto& r : h->recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (auto e : h->free_events) (void)hipEventDestroy(e);
  if (h->tab_ev) (void)hipEventDestroy(h->tab_ev);
  if (h->tab_host) (void)hipHostFree(h->tab_host);
  if (h->fallbacks) (void)hipFree(h->fallbacks);
  if (h->repr) (void)hipFree(h->repr);
  if (h->split) (void)hipFree(h->split);
  if (h->panel) (void)hipFree(h->panel);
  if (h->idx) (void)hipFree(h->idx);
  for (auto* b : {&h->g_count, &h->g_offsets, &h->g_items, &h->g_item_rec, &h->g_rank, &h->g_rec, &h->g_wgv, &h->g_list, &h->g_po,
                 &h->b_ld, &h->b_dq, &h->b_dkv, &h->b_dob, &h->r_q, &h->r_k, &h->r_v, &h->r_o, &h->r_do, &h->r_lse,
                 &h->r_idx, &h->r_dq, &h->r_dk, &h->r_dv, &h->s_part, &h->s_lse, &h->tab, &h->sel_repair})
    if (b->p) (void)hipFree(b->p);
  delete h;
  return BSA_OK;
}

BSA_API bsa_status bsa_set_option(bsa_handle h, int option, int64_t value) {
  if (!h) return fail(nullptr, BSA_ERR_INVALID_ARG, "bsa_set_option: handle is NULL");
  switch (option) {
    case BSA_OPT_PANEL_CHUNK_BYTES:
      if (value < 1) return fail(h, BSA_ERR_INVALID_ARG, "bsa_set_option: panel chunk must be > 0");
      h->panel_chunk_bytes = value;
      return BSA_OK;
    case BSA_OPT_FINE_STRATEGY:
      if (value != BSA_FINE_BLOCK_GATHER && value != BSA_FINE_QUERY_TILE && value != BSA_FINE_PER_QUERY)
        return fail(h, BSA_ERR_INVALID_ARG, "bsa_set_option: unknown fine strategy %lld", (long long)value);
      h->fine_strategy = static_cast<int>(value);
      return BSA_OK;
    case BSA_OPT_SELECT_STRATEGY:
      if (value != BSA_SELECT_FUSED && value != BSA_SELECT_PANEL)
        return fail(h, BSA_ERR_INVALID_ARG, "bsa_set_option: unknown select strategy %lld", (long long)value);
      h->select_strategy = static_cast<int>(value);
      return BSA_OK;
    case BSA_OPT_FINE_CHUNK_BYTES:
      if (value < 1) return fail(h, BSA_ERR_INVALID_ARG, "bsa_set_option: fine chunk must be > 0");
      h->fine_chunk_bytes = value;
      return BSA_OK;
    case BSA_OPT_STATIC_ITEM_TILES:
      if (value < 0) return fail(h, BSA_ERR_INVALID_ARG, "bsa_set_option: static item tiles must be >= 0");
      h->static_item_tiles = value;
      return BSA_OK;
    case BSA_OPT_UNION_ROWS:
      if (value != 16 && value != 32 && value != 64)
        return fail(h, BSA_ERR_INVALID_ARG, "bsa_set_option: union rows must be 16, 32 or 64 (got %lld)",
                    (long long)value);
      h->union_rows = static_cast<int>(value);
      return BSA_OK;
    default:
      return fail(h, BSA_ERR_INVALID_ARG, "bsa_set_option: unknown option %d", option);
  }
}

BSA_API bsa_status bsa_workspace_bytes(bsa_handle h, size_t* bytes) {
  if (!h || !bytes) return fail(h, BSA_ERR_INVALID_ARG, "bsa_workspace_bytes: NULL argument");
  *bytes = h->repr_bytes + h->split_bytes + h->panel_bytes + h->idx_bytes;
  for (auto* b : {&h->g_count, &h->g_offsets, &h->g_items, &h->g_item_rec, &h->g_rank, &h->g_rec, &h->g_wgv, &h->g_list, &h->g_po,
                 &h->b_ld, &h->b_dq, &h->b_dkv, &h->b_dob, &h->r_q, &h->r_k, &h->r_v, &h->r_o, &h->r_do, &h->r_lse,
                 &h->r_idx, &h->r_dq, &h->r_dk, &h->r_dv, &h->s_part, &h->s_lse, &h->tab, &h->sel_repair})
    *bytes += b->bytes;
  return BSA_OK;
}

// ----------------------------------------------------------- stage 1 ----

namespace {

bsa_status run_pool(bsa_handle h, const void* k, float* repr, uint16_t* split, const Shape& s,
                    bsa_dtype dt, hipStream_t st, const int4* tab = nullptr) {
  return timed_launch(h, BSA_STAGE_POOL, st, "block_pool", [&] {
    return bsa::launch_block_pool(k, repr, split, s.bh(), s.n, s.d, dt, st, tab);
  });
}

// The layout the kernels run on: ks.bh() slices (batch x heads, or heads for
// a variable-length batch) of ks.n rows, ks.n a multiple of 64, every
// sequence starting on a block boundary.  tab: the block table when a slice
// is not one sequence of whole blocks (empty otherwise).  copy: the caller's
// rows (src_rows per slice) must be copied into that layout, some sequence
// not being whole blocks, and the results copied back.
struct Plan {
  Shape ks;
  int src_rows = 0;
  bool copy = false;
  std::vector<int4> tab;
};

// One sequence of s.n rows per (batch, head).
Plan plan_dense(const Shape& s) {
  Plan p;
  p.ks = s.padded();
  p.src_rows = s.n;
  p.copy = p.ks.n != s.n;
  if (p.copy) {
    const int nb = p.ks.n / 64;
    p.tab.resize(size_t(nb));
    for (int b = 0; b < nb; ++b) p.tab[size_t(b)] = make_int4(0, nb, std::min(64, s.n - 64 * b), 64 * b);
  }
  return p;
}

// Sequences cu[i] .. cu[i + 1] - 1 of the caller's rows of every head.
bsa_status plan_varlen(bsa_handle h, const char* fn, const int32_t* cu, int nseq, int heads, int d, Plan* p) {
  if (!cu) return fail(h, BSA_ERR_INVALID_ARG, "%s: cu_seqlens is NULL", fn);
  if (nseq < 1 || heads < 1)
    return fail(h, BSA_ERR_INVALID_ARG, "%s: nseq and heads must be >= 1 (got %d, %d)", fn, nseq, heads);
  if (cu[0] != 0) return fail(h, BSA_ERR_INVALID_ARG, "%s: cu_seqlens[0] must be 0 (got %d)", fn, cu[0]);
  int64_t blocks = 0;
  for (int i = 0; i < nseq; ++i) {
    if (cu[i + 1] < cu[i])
      return fail(h, BSA_ERR_INVALID_ARG, "%s: cu_seqlens decreases at %d (%d -> %d)", fn, i, cu[i], cu[i + 1]);
    blocks += (int64_t(cu[i + 1]) - cu[i] + 63) / 64;
  }
  if (cu[nseq] < 1) return fail(h, BSA_ERR_INVALID_ARG, "%s: the batch has no rows", fn);
  if (blocks > 2048)
    return fail(h, BSA_ERR_UNSUPPORTED, "%s: the sequences take %lld blocks of 64 rows per head; at most 2048",
                fn, (long long)blocks);
  p->ks = Shape{1, heads, int(blocks * 64), d};
  p->src_rows = cu[nseq];
  p->copy = false;
  p->tab.assign(size_t(blocks), make_int4(0, 0, 0, 0));
  int b0 = 0;
  for (int i = 0; i < nseq; ++i) {
    const int len = cu[i + 1] - cu[i], nbs = (len + 63) / 64;
    if (len % 64 != 0) p->copy = true;
    for (int j = 0; j < nbs; ++j)
      p->tab[size_t(b0 + j)] = make_int4(b0, b0 + nbs, std::min(64, len - 64 * j), cu[i] + 64 * j);
    b0 += nbs;
  }
  return BSA_OK;
}

// The plan's block table on the device (NULL when it has none), copied on
// the stream from a pinned staging buffer; the staging buffer is rewritten
// only once the previous copy from it has finished.
bsa_status upload_tab(bsa_handle h, const Plan& p, hipStream_t st, const int4** out) {
  *out = nullptr;
  if (p.tab.empty()) return BSA_OK;
  const size_t bytes = p.tab.size() * sizeof(int4);
  TRY(grow(h, &h->tab.p, &h->tab.bytes, bytes, "block table"));
  if (h->tab_ev_live && hipEventSynchronize(h->tab_ev) != hipSuccess)
    return fail(h, BSA_ERR_LAUNCH, "block table: waiting for the previous upload failed");
  h->tab_ev_live = false;
  if (h->tab_host_bytes < bytes) {
    if (h->tab_host) (void)hipHostFree(h->tab_host);
    h->tab_host = nullptr;
    h->tab_host_bytes = 0;
    if (hipHostMalloc(&h->tab_host, bytes, hipHostMallocDefault) != hipSuccess) {
      (void)hipGetLastError();
      h->tab_host = nullptr;
      return fail(h, BSA_ERR_OUT_OF_MEMORY, "block table: pinned host allocation of %zu bytes failed", bytes);
    }
    h->tab_host_bytes = bytes;
  }
  std::memcpy(h->tab_host, p.tab.data(), bytes);
  if (!h->tab_ev && hipEventCreateWithFlags(&h->tab_ev, hipEventDisableTiming) != hipSuccess) {
    h->tab_ev = nullptr;
    return fail(h, BSA_ERR_LAUNCH, "block table: could not create an event");
  }
  if (hipMemcpyAsync(h->tab.p, h->tab_host, bytes, hipMemcpyHostToDevice, st) != hipSuccess ||
      hipEventRecord(h->tab_ev, st) != hipSuccess) {
    (void)hipGetLastError();
    return fail(h, BSA_ERR_LAUNCH, "block table: upload failed");
  }
  h->tab_ev_live = true;
  *out = static_cast<const int4*>(h->tab.p);
  return BSA_OK;
}

// Copies of caller rows into the plan's layout and back.
bsa_status pad_rows(bsa_handle h, const void* src, void* dst, const Plan& p, const int4* tab, int words,
                    uint32_t fill, hipStream_t st) {
  return timed_launch(h, BSA_STAGE_RAGGED_COPY, st, "padding copy", [&] {
    return bsa::launch_pad_rows(src, dst, p.ks.bh(), p.src_rows, p.ks.n, words, fill, tab, st);
  });
}

bsa_status unpad_rows(bsa_handle h, const void* src, void* dst, const Plan& p, const int4* tab, int words,
                      hipStream_t st) {
  return timed_launch(h, BSA_STAGE_RAGGED_COPY, st, "copy back", [&] {
    return bsa::launch_unpad_rows(src, dst, p.ks.bh(), p.src_rows, p.ks.n, words, tab, st);
  });
}

int elem_bytes(bsa_dtype dt) { return dt == BSA_BF16 ? 2 : 4; }

bool fused_select(bsa_handle h, int topk) {
  return h->select_strategy == BSA_SELECT_FUSED && topk <= bsa::kFusedSelectMaxK;
}

bsa::HeadBudget uniform_budget(int topk) {
  bsa::HeadBudget hb;
  hb.heads = 1;
  hb.k[0] = topk;
  return hb;
}

// A fixed region of device memory handed out front to back (256-byte
// aligned pieces); the workspace of the no-allocation entry point.
struct Arena {
  unsigned char* base = nullptr;
  size_t cap = 0, used = 0;
  size_t avail() const { return cap > align(used) ? cap - align(used) : 0; }
  static size_t align(size_t x) { return (x + 255) & ~size_t(255); }
  void* take(size_t bytes) {
    const size_t off = align(used);
    if (off + bytes > cap) return nullptr;
    used = off + bytes;
    return base + off;
  }
};

bsa_status take(bsa_handle h, Arena* arena, void** out, size_t bytes, const char* what) {
  *out = arena->take(bytes);
  if (!*out)
    return fail(h, BSA_ERR_UNSUPPORTED, "%s: %zu bytes do not fit the %zu bytes left of the fixed workspace",
                what, bytes, arena->avail());
  return BSA_OK;
}

// Stage 1 selection over all rows: one fused coarse_score + topk_select
// kernel (k <= 32, fused strategy), else coarse_score and topk_select through
// a panel, in chunks of at most panel_chunk_bytes of panel (with an arena: of
// what is left of it).  v (nullable): the V the fine stage will read, which
// the fused kernel may read ahead (launch_coarse_select).
bsa_status run_select(bsa_handle h, const void* q, const float* repr, const uint16_t* split,
                      int32_t* idx, const Shape& s, bsa_dtype dt, int topk,
                      const bsa::HeadBudget& hb, int causal, hipStream_t st, Arena* arena = nullptr,
                      const int4* tab = nullptr, const void* v = nullptr) {
  const int64_t nb = s.n / 64;
  const int64_t total = s.bh() * s.n;
  if (fused_select(h, topk)) {
    int32_t* repair_list = nullptr;
    const bool repair = bsa::select_uses_repair(s.d, dt, topk);
    if (repair) {
      const size_t bytes = size_t(total / 64) * sizeof(int32_t);
      if (arena) {
        TRY(take(h, arena, reinterpret_cast<void**>(&repair_list), bytes, "selection repair list"));
      } else {
        TRY(grow(h, &h->sel_repair.p, &h->sel_repair.bytes, bytes, "selection repair list"));
        repair_list = static_cast<int32_t*>(h->sel_repair.p);
      }
    }
    const int parity = h->repair_parity;
    TRY(timed_launch(h, BSA_STAGE_COARSE_TOPK, st, "coarse_select", [&] {
      return bsa::launch_coarse_select(q, repr, split, idx, total, s.n, s.d, dt, topk, hb, causal, st, tab,
                                       h->fallbacks, h->fallbacks + 2, repair_list, parity, v);
    }));
    if (repair) h->repair_parity ^= 1;  // the next such call lists at the counter this one cleared
    return BSA_OK;
  }
  int64_t chunk = h->panel_chunk_bytes / (nb * 4) / 64 * 64;
  if (arena) {
    const int64_t fit = int64_t(arena->avail() / size_t(nb * 4)) / 64 * 64;
    if (fit < 64) return fail(h, BSA_ERR_UNSUPPORTED, "score panel: one 64-row chunk does not fit the fixed workspace");
    if (chunk > fit) chunk = fit;
  }
  if (chunk < 64) chunk = 64;
  if (chunk > total) chunk = total;
  float* panel = nullptr;
  if (arena) {
    TRY(take(h, arena, reinterpret_cast<void**>(&panel), size_t(chunk) * nb * 4, "score panel"));
  } else {
    TRY(grow(h, reinterpret_cast<void**>(&h->panel), &h->panel_bytes, size_t(chunk) * nb * 4,
             "panel workspace"));
    panel = h->panel;
  }
  for (int64_t r0 = 0; r0 < total; r0 += chunk) {
    const int64_t rows = (total - r0) < chunk ? (total - r0) : chunk;
    TRY(timed_launch(h, BSA_STAGE_COARSE, st, "coarse_score", [&] {
      return bsa::launch_coarse_score(q, repr, panel, r0, rows, s.n, s.d, dt, causal, st);
    }));
    TRY(timed_launch(h, BSA_STAGE_TOPK, st, "topk_select", [&] {
      return bsa::launch_topk_select(panel, idx, r0, rows, s.n, topk, hb, causal, st, tab);
    }));
  }
  return BSA_OK;
}

bsa_status grow_buf(bsa_handle h, bsa_handle_s::Buf& b, size_t need, const char* what) {
  return grow(h, &b.p, &b.bytes, need, what);
}

// The bucket counts must be zero when a bucketing starts; the scan kernel
// clears them after use, so only a new buffer or a failed launch needs a
// clearing kernel.  Returns the words to clear (0 if none) and assumes the
// bucketing about to be enqueued succeeds; run_gather_index undoes that on
// failure.
// A buffer that has to grow is new memory whatever its address (a free
// followed by an allocation can return the same pointer), so growth itself
// marks the counts as not known to be zero.
bsa_status grow_counts(bsa_handle h, size_t buckets, int64_t* clear_words) {
  if (h->g_count.bytes < buckets * 4) h->counts_zero = false;
  TRY(grow_buf(h, h->g_count, buckets * 4, "bucket counts"));
  *clear_words = h->counts_zero ? 0 : int64_t(h->g_count.bytes / 4);
  return BSA_OK;
}

bsa_status run_gather_index(bsa_handle h, bsa::GatherArgs& a, int64_t r0, int64_t rows, int stage,
                            const char* what, hipStream_t st, bool handle_counts = true) {
  const bsa_status r = timed_launch(h, stage, st, what, [&] { return bsa::launch_gather_index(a, r0, rows, st); });
  if (handle_counts) h->counts_zero = r == BSA_OK;
  a.ws.count_words = 0;  // cleared by the first bucketing of this call
  return r;
}

// Device bytes the block-gather fine stage needs for a chunk of `chunk`
// query rows (each piece 256-byte aligned, as an Arena hands them out).
struct FineGeom {
  int64_t chunk, pairs, buckets, slots;
  int qsegs;
  size_t bytes;
};
FineGeom fine_geom(const Shape& s, bsa_dtype dt, int topk, int64_t chunk) {
  FineGeom g;
  g.chunk = chunk;
  g.pairs = chunk * topk;
  g.qsegs = bsa::gather_segments(s.n, s.d, topk, dt);
  const int64_t nb = s.n / 64;
  const int64_t heads_spanned = s.bh() < (chunk + s.n - 1) / s.n + 1 ? s.bh() : (chunk + s.n - 1) / s.n + 1;
  g.buckets = heads_spanned * g.qsegs * nb;
  g.slots = bsa::gather_grid(chunk, topk, g.buckets, bsa::gather_item_pairs(s.d, dt));
  const size_t pieces[] = {size_t(g.buckets) * 4, size_t(g.buckets + 1) * 4, size_t(g.buckets + 1) * 4,
                           size_t(g.slots) * 16, size_t(g.pairs) * 4, size_t(g.pairs) * 4,
                           size_t(g.pairs) * s.d * (dt == BSA_BF16 ? 2 : 4), size_t(g.pairs) * 8,
                           size_t(chunk / 64 + 1) * 4};
  g.bytes = 0;
  for (size_t b : pieces) g.bytes += Arena::align(b);
  return g;
}

// The block-gather fine stage with every buffer carved from `arena`: the
// largest row chunk whose buffers fit is used; the bucket counts are cleared
// by a kernel at the start of every call (the arena keeps what the last call
// left).
bsa_status run_fine_arena(bsa_handle h, const void* q, const void* k, const void* v, float* out, float* lse,
                          const int32_t* idx, const Shape& s, bsa_dtype dt, int topk, float scale, int causal,
                          hipStream_t st, Arena& arena) {
  const int64_t total = s.bh() * s.n;
  const int64_t align = (s.n % 256 == 0) ? 256 : 64;
  int64_t chunk = (total + align - 1) / align * align;
  while (chunk > align && fine_geom(s, dt, topk, chunk).bytes > arena.avail())
    chunk = (chunk / 2 + align - 1) / align * align;
  if (chunk > total) chunk = total;
  const FineGeom g = fine_geom(s, dt, topk, chunk);
  if (g.bytes > arena.avail())
    return fail(h, BSA_ERR_UNSUPPORTED, "fine stage: one chunk of %lld rows needs %zu bytes, the fixed workspace "
                "has %zu left", (long long)chunk, g.bytes, arena.avail());
  bsa::GatherArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.idx = idx;
  a.n = s.n;
  a.d = s.d;
  a.topk = topk;
  a.causal = causal;
  a.scale = scale;
  a.dtype = dt;
  a.qsegs = g.qsegs;
  a.item_pairs = bsa::gather_item_pairs(s.d, dt);
  void* p[9];
  const size_t sizes[] = {size_t(g.buckets) * 4, size_t(g.buckets + 1) * 4, size_t(g.buckets + 1) * 4,
                          size_t(g.slots) * 16, size_t(g.pairs) * 4, size_t(g.pairs) * 4,
                          size_t(g.pairs) * s.d * (dt == BSA_BF16 ? 2 : 4), size_t(g.pairs) * 8,
                          size_t(chunk / 64 + 1) * 4};
  for (int i = 0; i < 9; ++i) TRY(take(h, &arena, &p[i], sizes[i], "fine-stage workspace"));
  a.ws.count = static_cast<int32_t*>(p[0]);
  a.ws.count_words = g.buckets;
  a.ws.offsets = static_cast<int32_t*>(p[1]);
  a.ws.items = static_cast<int32_t*>(p[2]);
  a.ws.item_rec = static_cast<int4*>(p[3]);
  a.ws.rank = static_cast<int32_t*>(p[4]);
  a.ws.list = static_cast<int32_t*>(p[5]);
  a.ws.partial_o = p[6];
  a.ws.rec = static_cast<int2*>(p[7]);
  a.ws.wg_valid = static_cast<int32_t*>(p[8]);
  for (int64_t r0 = 0; r0 < total; r0 += chunk) {
    const int64_t rows = (total - r0) < chunk ? (total - r0) : chunk;
    TRY(run_gather_index(h, a, r0, rows, BSA_STAGE_GATHER_INDEX, "block-gather bucketing", st, false));
    TRY(timed_launch(h, BSA_STAGE_FINE, st, "sparse_flash_fwd",
                     [&] { return bsa::launch_gather_partial(a, r0, rows, st); }));
    TRY(timed_launch(h, BSA_STAGE_GATHER_COMBINE, st, "block-gather combine",
                     [&] { return bsa::launch_gather_combine(a, r0, rows, st); }));
  }
  return BSA_OK;
}

// Stage 2 for the dynamic path, with the handle's fine strategy.
bsa_status run_fine(bsa_handle h, const void* q, const void* k, const void* v, float* out,
                    float* lse, const int32_t* idx, const Shape& s, bsa_dtype dt, int topk,
                    float scale, int causal, hipStream_t st, const int4* tab = nullptr, Arena* arena = nullptr) {
  if (arena && h->fine_strategy == BSA_FINE_BLOCK_GATHER)  // whole-block sequences only (no table)
    return run_fine_arena(h, q, k, v, out, lse, idx, s, dt, topk, scale, causal, st, *arena);
  if (h->fine_strategy == BSA_FINE_QUERY_TILE)
    return timed_launch(h, BSA_STAGE_FINE, st, "sparse_flash_fwd", [&] {
      return bsa::launch_sparse_flash_dynamic(q, k, v, out, lse, idx, s.bh(), s.n, s.d, topk, scale,
                                              causal, dt, st, tab, h->union_rows);
    });
  if (h->fine_strategy == BSA_FINE_PER_QUERY)
    return timed_launch(h, BSA_STAGE_FINE, st, "sparse_flash_fwd", [&] {
      return bsa::launch_sparse_flash_per_query(q, k, v, out, lse, idx, s.bh() * s.n, s.n, s.d, topk, scale,
                                                causal, dt, st, tab);
    });
  const int64_t total = s.bh() * s.n;
  const size_t per_row = bsa::gather_pair_bytes(s.d, dt) * size_t(topk);
  const int64_t align = (s.n % 256 == 0) ? 256 : 64;  // keeps bucketing workgroups inside one head
  int64_t chunk = h->fine_chunk_bytes / int64_t(per_row) / align * align;
  if (chunk < align) chunk = align;
  if (chunk > total) chunk = total;
  const int64_t pairs = chunk * topk;
  const int64_t nb = s.n / 64;
  const int qsegs = bsa::gather_segments(s.n, s.d, topk, dt);
  const int64_t heads_spanned = s.bh() < (chunk + s.n - 1) / s.n + 1 ? s.bh() : (chunk + s.n - 1) / s.n + 1;
  const int64_t buckets = heads_spanned * qsegs * nb;
  int64_t clear_words = 0;
  TRY(grow_counts(h, size_t(buckets), &clear_words));
  TRY(grow_buf(h, h->g_offsets, size_t(buckets + 1) * 4, "bucket offsets"));
  TRY(grow_buf(h, h->g_items, size_t(buckets + 1) * 4, "bucket work items"));
  const int item_pairs = bsa::gather_item_pairs(s.d, dt);
  TRY(grow_buf(h, h->g_item_rec, size_t(bsa::gather_grid(chunk, topk, buckets, item_pairs)) * 16,
               "work-item records"));
  TRY(grow_buf(h, h->g_rank, size_t(pairs) * 4, "pair ranks"));
  TRY(grow_buf(h, h->g_list, size_t(pairs) * 4, "pair lists"));
  TRY(grow_buf(h, h->g_po, size_t(pairs) * s.d * (dt == BSA_BF16 ? 2 : 4), "partial outputs"));
  TRY(grow_buf(h, h->g_rec, size_t(pairs) * 8, "block-ordered pair records"));
  TRY(grow_buf(h, h->g_wgv, size_t(chunk / 64 + 1) * 4, "pairs per bucketing workgroup"));
  bsa::GatherArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.idx = idx;
  a.n = s.n;
  a.d = s.d;
  a.topk = topk;
  a.causal = causal;
  a.scale = scale;
  a.dtype = dt;
  a.qsegs = qsegs;
  a.item_pairs = item_pairs;
  a.seqtab = tab;
  a.ws.count = static_cast<int32_t*>(h->g_count.p);
  a.ws.count_words = clear_words;
  a.ws.offsets = static_cast<int32_t*>(h->g_offsets.p);
  a.ws.items = static_cast<int32_t*>(h->g_items.p);
  a.ws.item_rec = static_cast<int4*>(h->g_item_rec.p);
  a.ws.rank = static_cast<int32_t*>(h->g_rank.p);
  a.ws.rec = static_cast<int2*>(h->g_rec.p);
  a.ws.wg_valid = static_cast<int32_t*>(h->g_wgv.p);
  a.ws.list = static_cast<int32_t*>(h->g_list.p);
  a.ws.partial_o = h->g_po.p;
  for (int64_t r0 = 0; r0 < total; r0 += chunk) {
    const int64_t rows = (total - r0) < chunk ? (total - r0) : chunk;
    TRY(run_gather_index(h, a, r0, rows, BSA_STAGE_GATHER_INDEX, "block-gather bucketing", st));
    TRY(timed_launch(h, BSA_STAGE_FINE, st, "sparse_flash_fwd",
                     [&] { return bsa::launch_gather_partial(a, r0, rows, st); }));
    TRY(timed_launch(h, BSA_STAGE_GATHER_COMBINE, st, "block-gather combine",
                     [&] { return bsa::launch_gather_combine(a, r0, rows, st); }));
  }
  return BSA_OK;
}

}  // namespace

BSA_API bsa_status bsa_block_pool(bsa_handle h, const void* k, float* repr_out, int batch,
                                  int heads, int n, int d, bsa_dtype dtype, int block,
                                  void* stream) {
  const char* fn = "bsa_block_pool";
  if (!h) return fail(nullptr, BSA_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  const Shape s{batch, heads, n, d};
  TRY(check_shape(h, fn, s, dtype, block));
  TRY(check_ptr(h, fn, "k", k));
  TRY(check_ptr(h, fn, "repr_out", repr_out));
  DeviceGuard dg(h->device);
  return run_pool(h, k, repr_out, nullptr, s, dtype, static_cast<hipStream_t>(stream));
}

BSA_API bsa_status bsa_coarse_score(bsa_handle h, const void* q, const float* repr,
                                    float* panel_out, int batch, int heads, int n, int d,
                                    bsa_dtype dtype, int block, int causal, void* stream) {
  const char* fn = "bsa_coarse_score";
  if (!h) return fail(nullptr, BSA_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  const Shape s{batch, heads, n, d};
  TRY(check_shape(h, fn, s, dtype, block));
  TRY(check_dynamic(h, fn, s, 1, causal));
  TRY(check_ptr(h, fn, "q", q));
  TRY(check_ptr(h, fn, "repr", repr));
  TRY(check_ptr(h, fn, "panel_out", panel_out));
  DeviceGuard dg(h->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return timed_launch(h, BSA_STAGE_COARSE, st, "coarse_score", [&] {
    return bsa::launch_coarse_score(q, repr, panel_out, 0, s.bh() * s.n, s.n, s.d, dtype, causal,
                                    st);
  });
}

BSA_API bsa_status bsa_topk_select(bsa_handle h, const float* panel, int32_t* block_idx_out,
                                   int batch, int heads, int n, int block, int topk, int causal,
                                   void* stream) {
  const char* fn = "bsa_topk_select";
  if (!h) return fail(nullptr, BSA_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  const Shape s{batch, heads, n, 64};
  TRY(check_shape(h, fn, s, BSA_FP32, block));
  TRY(check_dynamic(h, fn, s, topk, causal));
  TRY(check_ptr(h, fn, "panel", panel));
  if (!block_idx_out) return fail(h, BSA_ERR_INVALID_ARG, "%s: block_idx_out is NULL", fn);
  DeviceGuard dg(h->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return timed_launch(h, BSA_STAGE_TOPK, st, "topk_select", [&] {
    return bsa::launch_topk_select(panel, block_idx_out, 0, s.bh() * s.n, s.n, topk,
                                   uniform_budget(topk), causal, st);
  });
}

// ----------------------------------------------------------- stage 2 ----

BSA_API bsa_status bsa_fine_forward(bsa_handle h, const void* q, const void* k, const void* v,
                                    float* out, const int32_t* block_idx, int batch, int heads,
                                    int n, int d, bsa_dtype dtype, int block, int topk,
                                    float scale, int causal, void* stream) {
  const char* fn = "bsa_fine_forward";
  if (!h) return fail(nullptr, BSA_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  const Shape s{batch, heads, n, d};
  TRY(check_shape(h, fn, s, dtype, block, true));
  TRY(check_dynamic(h, fn, s, topk, causal));
  TRY(check_scale(h, fn, scale));
  TRY(check_ptr(h, fn, "q", q));
  TRY(check_ptr(h, fn, "k", k));
  TRY(check_ptr(h, fn, "v", v));
  TRY(check_ptr(h, fn, "out", out));
  if (!block_idx) return fail(h, BSA_ERR_INVALID_ARG, "%s: block_idx is NULL", fn);
  DeviceGuard dg(h->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s.n % 64 == 0) return run_fine(h, q, k, v, out, nullptr, block_idx, s, dtype, topk, scale, causal, st);
  // ragged n: whole-block copies; the padding rows select nothing
  const Plan p = plan_dense(s);
  const Shape& sp = p.ks;
  const int4* tab = nullptr;
  TRY(upload_tab(h, p, st, &tab));
  const size_t in_bytes = size_t(sp.elems()) * elem_bytes(dtype);
  const int w = s.d * elem_bytes(dtype) / 4;
  TRY(grow_buf(h, h->r_q, in_bytes, "padded q"));
  TRY(grow_buf(h, h->r_k, in_bytes, "padded k"));
  TRY(grow_buf(h, h->r_v, in_bytes, "padded v"));
  TRY(grow_buf(h, h->r_o, size_t(sp.elems()) * 4, "padded out"));
  TRY(grow_buf(h, h->r_idx, size_t(sp.bh() * sp.n * topk) * 4, "padded indices"));
  TRY(pad_rows(h, q, h->r_q.p, p, tab, w, 0u, st));
  TRY(pad_rows(h, k, h->r_k.p, p, tab, w, 0u, st));
  TRY(pad_rows(h, v, h->r_v.p, p, tab, w, 0u, st));
  TRY(pad_rows(h, block_idx, h->r_idx.p, p, tab, topk, 0xFFFFFFFFu, st));
  TRY(run_fine(h, h->r_q.p, h->r_k.p, h->r_v.p, static_cast<float*>(h->r_o.p), nullptr,
               static_cast<const int32_t*>(h->r_idx.p), sp, dtype, topk, scale, causal, st, tab));
  return unpad_rows(h, h->r_o.p, out, p, tab, s.d, st);
}

namespace {
// The forward entry points after their own argument checks, on the layout
// of plan p; topk = index row length (the largest budget).
bsa_status forward_impl(bsa_handle h, const char* fn, const void* q, const void* k, const void* v,
                        float* out, int32_t* block_idx_out, float* lse_out, const Plan& p,
                        bsa_dtype dtype, int topk, const bsa::HeadBudget& hb, float scale,
                        int causal, void* stream) {
  TRY(check_scale(h, fn, scale));
  TRY(check_ptr(h, fn, "q", q));
  TRY(check_ptr(h, fn, "k", k));
  TRY(check_ptr(h, fn, "v", v));
  TRY(check_ptr(h, fn, "out", out));
  if (block_idx_out && (reinterpret_cast<uintptr_t>(block_idx_out) & 3u))
    return fail(h, BSA_ERR_INVALID_ARG, "%s: block_idx_out is not 4-byte aligned", fn);
  DeviceGuard dg(h->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // Sequences that are not whole blocks run on copies padded to whole blocks
  // (sp); the padding keys are masked, the padding rows' results dropped.
  const Shape& sp = p.ks;
  const int4* tab = nullptr;
  TRY(upload_tab(h, p, st, &tab));
  const void *pq = q, *pk = k, *pv = v;
  float* pout = out;
  float* plse = lse_out;
  int32_t* idx = block_idx_out;
  if (p.copy) {
    const size_t in_bytes = size_t(sp.elems()) * elem_bytes(dtype);
    const int w = sp.d * elem_bytes(dtype) / 4;
    TRY(grow_buf(h, h->r_q, in_bytes, "padded q"));
    TRY(grow_buf(h, h->r_k, in_bytes, "padded k"));
    TRY(grow_buf(h, h->r_v, in_bytes, "padded v"));
    TRY(grow_buf(h, h->r_o, size_t(sp.elems()) * 4, "padded out"));
    if (lse_out) TRY(grow_buf(h, h->r_lse, size_t(sp.bh() * sp.n) * 4, "padded lse"));
    TRY(pad_rows(h, q, h->r_q.p, p, tab, w, 0u, st));
    TRY(pad_rows(h, k, h->r_k.p, p, tab, w, 0u, st));
    TRY(pad_rows(h, v, h->r_v.p, p, tab, w, 0u, st));
    pq = h->r_q.p;
    pk = h->r_k.p;
    pv = h->r_v.p;
    pout = static_cast<float*>(h->r_o.p);
    plse = lse_out ? static_cast<float*>(h->r_lse.p) : nullptr;
    idx = nullptr;
  }
  const int64_t nb = sp.n / 64;
  // The fused bf16 selection reads the split representatives only.
  const bool want_split = fused_select(h, topk) && dtype == BSA_BF16;
  if (want_split)
    TRY(grow(h, reinterpret_cast<void**>(&h->split), &h->split_bytes, bsa::split_buffer_bytes(sp.bh(), int(nb), sp.d),
             "split repr workspace"));
  else
    TRY(grow(h, reinterpret_cast<void**>(&h->repr), &h->repr_bytes, size_t(sp.bh() * nb * sp.d) * 4,
             "repr workspace"));
  float* repr = want_split ? nullptr : h->repr;
  uint16_t* split = want_split ? h->split : nullptr;
  if (!idx) {
    TRY(grow(h, reinterpret_cast<void**>(&h->idx), &h->idx_bytes, size_t(sp.bh() * sp.n * topk) * 4,
             "index workspace"));
    idx = h->idx;
  }
  TRY(run_pool(h, pk, repr, split, sp, dtype, st, tab));
  TRY(run_select(h, pq, repr, split, idx, sp, dtype, topk, hb, causal, st, nullptr, tab, pv));
  TRY(run_fine(h, pq, pk, pv, pout, plse, idx, sp, dtype, topk, scale, causal, st, tab));
  if (p.copy) {
    TRY(unpad_rows(h, pout, out, p, tab, sp.d, st));
    if (block_idx_out) TRY(unpad_rows(h, idx, block_idx_out, p, tab, topk, st));
    if (lse_out) TRY(unpad_rows(h, plse, lse_out, p, tab, 1, st));
  }
  return BSA_OK;
}

// Per-head budgets from a host array (heads entries, each in [1, topk_max]).
bsa_status read_budgets(bsa_handle h, const char* fn, const int32_t* head_topk, int heads,
                        int topk_max, bsa::HeadBudget* hb) {
  if (heads > bsa::kMaxBudgetHeads)
    return fail(h, BSA_ERR_UNSUPPORTED, "%s: at most %d heads with per-head budgets (got %d)", fn,
                bsa::kMaxBudgetHeads, heads);
  hb->heads = heads;
  for (int i = 0; i < heads; ++i) {
    if (head_topk[i] < 1 || head_topk[i] > topk_max)
      return fail(h, BSA_ERR_INVALID_ARG, "%s: head_topk[%d] = %d is outside [1, topk_max = %d]", fn, i,
                  head_topk[i], topk_max);
    hb->k[i] = head_topk[i];
  }
  return BSA_OK;
}
}  // namespace

BSA_API bsa_status bsa_forward(bsa_handle h, const void* q, const void* k, const void* v,
                               float* out, int32_t* block_idx_out, int batch, int heads, int n,
                               int d, bsa_dtype dtype, int block, int topk, float scale,
                               int causal, void* stream) {
  const char* fn = "bsa_forward";
  if (!h) return fail(nullptr, BSA_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  const Shape s{batch, heads, n, d};
  TRY(check_shape(h, fn, s, dtype, block, true));
  TRY(check_dynamic(h, fn, s, topk, causal));
  return forward_impl(h, fn, q, k, v, out, block_idx_out, nullptr, plan_dense(s), dtype, topk,
                      uniform_budget(topk), scale, causal, stream);
}

BSA_API bsa_status bsa_forward_noalloc(bsa_handle h, const void* q, const void* k, const void* v,
                                       float* out, int32_t* block_idx_out, int batch, int heads, int n,
                                       int d, bsa_dtype dtype, int block, int topk, float scale,
                                       int causal, void* stream) {
  const char* fn = "bsa_forward_noalloc";
  if (!h) return fail(nullptr, BSA_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  const Shape s{batch, heads, n, d};
  TRY(check_shape(h, fn, s, dtype, block));
  TRY(check_dynamic(h, fn, s, topk, causal));
  TRY(check_scale(h, fn, scale));
  TRY(check_ptr(h, fn, "q", q));
  TRY(check_ptr(h, fn, "k", k));
  TRY(check_ptr(h, fn, "v", v));
  TRY(check_ptr(h, fn, "out", out));
  if (!block_idx_out || (reinterpret_cast<uintptr_t>(block_idx_out) & 3u))
    return fail(h, BSA_ERR_INVALID_ARG, "%s: block_idx_out is NULL or not 4-byte aligned", fn);
  if (!h->noalloc) return fail(h, BSA_ERR_NO_DEVICE, "%s: no fixed workspace on device %d", fn, h->device);
  DeviceGuard dg(h->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  Arena arena;
  arena.base = static_cast<unsigned char*>(h->noalloc);
  arena.cap = bsa::kNoAllocScratchBytes;
  const int64_t nb = s.n / 64;
  const bool want_split = fused_select(h, topk) && dtype == BSA_BF16;
  float* repr = nullptr;
  uint16_t* split = nullptr;
  if (want_split)
    TRY(take(h, &arena, reinterpret_cast<void**>(&split), bsa::split_buffer_bytes(s.bh(), int(nb), s.d),
             "split representatives"));
  else
    TRY(take(h, &arena, reinterpret_cast<void**>(&repr), size_t(s.bh() * nb * s.d) * 4, "representatives"));
  // no events either: per-stage timing is off for this call
  const bool profiling = h->profiling;
  h->profiling = false;
  bsa_status r = run_pool(h, k, repr, split, s, dtype, st);
  if (r == BSA_OK)
    r = run_select(h, q, repr, split, block_idx_out, s, dtype, topk, uniform_budget(topk), causal, st, &arena,
                   nullptr, v);
  if (r == BSA_OK)
    r = run_fine(h, q, k, v, out, nullptr, block_idx_out, s, dtype, topk, scale, causal, st, nullptr, &arena);
  h->profiling = profiling;
  return r;
}

BSA_API bsa_status bsa_forward_budgets(bsa_handle h, const void* q, const void* k, const void* v,
                                       float* out, int32_t* block_idx_out, int batch, int heads,
                                       int n, int d, bsa_dtype dtype, int block,
                                       const int32_t* head_topk, int topk_max, float scale,
                                       int causal, void* stream) {
  const char* fn = "bsa_forward_budgets";
  if (!h) return fail(nullptr, BSA_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  const Shape s{batch, heads, n, d};
  TRY(check_shape(h, fn, s, dtype, block, true));
  TRY(check_dynamic(h, fn, s, topk_max, causal));
  if (!head_topk) return fail(h, BSA_ERR_INVALID_ARG, "%s: head_topk is NULL", fn);
  bsa::HeadBudget hb;
  TRY(read_budgets(h, fn, head_topk, heads, topk_max, &hb));
  return forward_impl(h, fn, q, k, v, out, block_idx_out, nullptr, plan_dense(s), dtype, topk_max, hb, scale,
                      causal, stream);
}

BSA_API bsa_status bsa_forward_train(bsa_handle h, const void* q, const void* k, const void* v,
                                     float* out, int32_t* block_idx_out, float* lse_out, int batch,
                                     int heads, int n, int d, bsa_dtype dtype, int block,
                                     const int32_t* head_topk, int topk, float scale, int causal,
                                     void* stream) {
  const char* fn = "bsa_forward_train";
  if (!h) return fail(nullptr, BSA_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  const Shape s{batch, heads, n, d};
  TRY(check_shape(h, fn, s, dtype, block, true));
  TRY(check_dynamic(h, fn, s, topk, causal));
  if (!block_idx_out) return fail(h, BSA_ERR_INVALID_ARG, "%s: block_idx_out is NULL", fn);
  if (!lse_out) return fail(h, BSA_ERR_INVALID_ARG, "%s: lse_out is NULL", fn);
  if (reinterpret_cast<uintptr_t>(lse_out) & 3u)
    return fail(h, BSA_ERR_INVALID_ARG, "%s: lse_out is not 4-byte aligned", fn);
  bsa::HeadBudget hb = uniform_budget(topk);
  if (head_topk) TRY(read_budgets(h, fn, head_topk, heads, topk, &hb));
  return forward_impl(h, fn, q, k, v, out, block_idx_out, lse_out, plan_dense(s), dtype, topk, hb, scale,
                      causal, stream);
}

namespace {
// The backward entry points after their shape checks, on the layout of plan p.
bsa_status backward_impl(bsa_handle h, const char* fn, const void* q, const void* k, const void* v,
                         const float* out, const float* dout, const int32_t* block_idx, const float* lse,
                         float* dq, float* dk, float* dv, const Plan& p, bsa_dtype dtype, int topk,
                         float scale, int causal, void* stream) {
  TRY(check_scale(h, fn, scale));
  TRY(check_ptr(h, fn, "q", q));
  TRY(check_ptr(h, fn, "k", k));
  TRY(check_ptr(h, fn, "v", v));
  TRY(check_ptr(h, fn, "out", out));
  TRY(check_ptr(h, fn, "dout", dout));
  TRY(check_ptr(h, fn, "dq", dq));
  TRY(check_ptr(h, fn, "dk", dk));
  TRY(check_ptr(h, fn, "dv", dv));
  if (!block_idx || (reinterpret_cast<uintptr_t>(block_idx) & 3u))
    return fail(h, BSA_ERR_INVALID_ARG, "%s: block_idx is NULL or not 4-byte aligned", fn);
  if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(h, BSA_ERR_INVALID_ARG, "%s: lse is NULL or not 4-byte aligned", fn);
  DeviceGuard dg(h->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // Sequences that are not whole blocks run on copies padded to whole
  // blocks (the padding rows select nothing, the padding keys are masked),
  // and dq, dk, dv are copied back.
  const Shape& sp = p.ks;
  const int4* tab = nullptr;
  TRY(upload_tab(h, p, st, &tab));
  float *gq = dq, *gk = dk, *gv = dv;
  if (p.copy) {
    const size_t in_bytes = size_t(sp.elems()) * elem_bytes(dtype);
    const size_t f_bytes = size_t(sp.elems()) * 4;
    const int w = sp.d * elem_bytes(dtype) / 4;
    TRY(grow_buf(h, h->r_q, in_bytes, "padded q"));
    TRY(grow_buf(h, h->r_k, in_bytes, "padded k"));
    TRY(grow_buf(h, h->r_v, in_bytes, "padded v"));
    TRY(grow_buf(h, h->r_o, f_bytes, "padded out"));
    TRY(grow_buf(h, h->r_do, f_bytes, "padded dout"));
    TRY(grow_buf(h, h->r_lse, size_t(sp.bh() * sp.n) * 4, "padded lse"));
    TRY(grow_buf(h, h->r_idx, size_t(sp.bh() * sp.n * topk) * 4, "padded indices"));
    TRY(grow_buf(h, h->r_dq, f_bytes, "padded dq"));
    TRY(grow_buf(h, h->r_dk, f_bytes, "padded dk"));
    TRY(grow_buf(h, h->r_dv, f_bytes, "padded dv"));
    TRY(pad_rows(h, q, h->r_q.p, p, tab, w, 0u, st));
    TRY(pad_rows(h, k, h->r_k.p, p, tab, w, 0u, st));
    TRY(pad_rows(h, v, h->r_v.p, p, tab, w, 0u, st));
    TRY(pad_rows(h, out, h->r_o.p, p, tab, sp.d, 0u, st));
    TRY(pad_rows(h, dout, h->r_do.p, p, tab, sp.d, 0u, st));
    TRY(pad_rows(h, lse, h->r_lse.p, p, tab, 1, 0u, st));
    TRY(pad_rows(h, block_idx, h->r_idx.p, p, tab, topk, 0xFFFFFFFFu, st));
    q = h->r_q.p;
    k = h->r_k.p;
    v = h->r_v.p;
    out = static_cast<const float*>(h->r_o.p);
    dout = static_cast<const float*>(h->r_do.p);
    lse = static_cast<const float*>(h->r_lse.p);
    block_idx = static_cast<const int32_t*>(h->r_idx.p);
    gq = static_cast<float*>(h->r_dq.p);
    gk = static_cast<float*>(h->r_dk.p);
    gv = static_cast<float*>(h->r_dv.p);
  }
  const int64_t total = sp.bh() * sp.n;
  const int64_t align = (sp.n % 256 == 0) ? 256 : 64;  // keeps bucketing workgroups inside one head
  const size_t per_row = size_t(topk) * size_t(sp.d) * elem_bytes(dtype);  // the per-pair dq rows
  int64_t chunk = h->fine_chunk_bytes / int64_t(per_row) / align * align;
  if (chunk < align) chunk = align;
  if (chunk > total) chunk = total;
  const int64_t pairs = chunk * topk;
  const int64_t nb = sp.n / 64;
  // One query segment per head: the backward's gathered rows (Q and dO) get
  // little L2 reuse at any segment size, and fewer segments mean fewer
  // per-item dk, dv partials to write and sum.
  const int qsegs = 1;
  const int64_t heads_spanned = sp.bh() < (chunk + sp.n - 1) / sp.n + 1 ? sp.bh() : (chunk + sp.n - 1) / sp.n + 1;
  const int64_t buckets = heads_spanned * qsegs * nb;
  const int64_t slots = bsa::gather_grid(chunk, topk, buckets, bsa::bwd_item_pairs(sp.d));
  int64_t clear_words = 0;
  TRY(grow_counts(h, size_t(buckets), &clear_words));
  TRY(grow_buf(h, h->g_offsets, size_t(buckets + 1) * 4, "bucket offsets"));
  TRY(grow_buf(h, h->g_items, size_t(buckets + 1) * 4, "bucket work items"));
  TRY(grow_buf(h, h->g_item_rec, size_t(slots) * 16, "work-item records"));
  TRY(grow_buf(h, h->g_rank, size_t(pairs) * 4, "pair ranks"));
  TRY(grow_buf(h, h->g_rec, size_t(pairs) * 8, "block-ordered pair records"));
  TRY(grow_buf(h, h->g_wgv, size_t(chunk / 64 + 1) * 4, "pairs per bucketing workgroup"));
  TRY(grow_buf(h, h->g_list, size_t(pairs) * 4, "pair lists"));
  TRY(grow_buf(h, h->b_ld, size_t(total) * 8, "backward row statistics"));
  if (dtype == BSA_BF16) TRY(grow_buf(h, h->b_dob, size_t(total) * sp.d * 2, "backward bf16 dout"));
  TRY(grow_buf(h, h->b_dq, size_t(pairs) * sp.d * elem_bytes(dtype), "backward dq contributions"));
  TRY(grow_buf(h, h->b_dkv, size_t(slots) * 2 * 64 * sp.d * 4, "backward dk/dv contributions"));
  bsa::BackwardArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.idx = block_idx;
  a.dq = gq;
  a.dk = gk;
  a.dv = gv;
  a.n = sp.n;
  a.seqtab = tab;
  a.d = sp.d;
  a.topk = topk;
  a.causal = causal;
  a.scale = scale;
  a.dtype = dtype;
  a.qsegs = qsegs;
  a.ld = static_cast<float2*>(h->b_ld.p);
  a.dout_b = dtype == BSA_BF16 ? static_cast<uint16_t*>(h->b_dob.p) : nullptr;
  a.dq_part = static_cast<float*>(h->b_dq.p);
  a.dkv_part = static_cast<float*>(h->b_dkv.p);
  a.ws.count = static_cast<int32_t*>(h->g_count.p);
  a.ws.count_words = clear_words;
  a.ws.offsets = static_cast<int32_t*>(h->g_offsets.p);
  a.ws.items = static_cast<int32_t*>(h->g_items.p);
  a.ws.item_rec = static_cast<int4*>(h->g_item_rec.p);
  a.ws.rank = static_cast<int32_t*>(h->g_rank.p);
  a.ws.rec = static_cast<int2*>(h->g_rec.p);
  a.ws.wg_valid = static_cast<int32_t*>(h->g_wgv.p);
  a.ws.list = static_cast<int32_t*>(h->g_list.p);
  bsa::GatherArgs gi;  // the bucketing of the forward, with backward-sized work items
  gi.q = q;
  gi.idx = block_idx;
  gi.n = sp.n;
  gi.seqtab = tab;
  gi.d = sp.d;
  gi.topk = topk;
  gi.causal = causal;
  gi.dtype = dtype;
  gi.qsegs = qsegs;
  gi.item_pairs = bsa::bwd_item_pairs(sp.d);
  gi.ws = a.ws;
  TRY(timed_launch(h, BSA_STAGE_BWD_PREP, st, "backward row statistics",
                   [&] { return bsa::launch_bwd_prep(a, total, st); }));
  for (int64_t r0 = 0; r0 < total; r0 += chunk) {
    const int64_t rows = (total - r0) < chunk ? (total - r0) : chunk;
    TRY(run_gather_index(h, gi, r0, rows, BSA_STAGE_BWD_INDEX, "backward bucketing", st));
    TRY(timed_launch(h, BSA_STAGE_BWD_PAIRS, st, "backward pair kernel",
                     [&] { return bsa::launch_bwd_pairs(a, r0, rows, st); }));
    TRY(timed_launch(h, BSA_STAGE_BWD_REDUCE, st, "backward dq reduction",
                     [&] { return bsa::launch_bwd_dq(a, r0, rows, st); }));
    TRY(timed_launch(h, BSA_STAGE_BWD_REDUCE, st, "backward dk/dv reduction",
                     [&] { return bsa::launch_bwd_dkv(a, r0, rows, st); }));
  }
  if (p.copy) {
    TRY(unpad_rows(h, gq, dq, p, tab, sp.d, st));
    TRY(unpad_rows(h, gk, dk, p, tab, sp.d, st));
    TRY(unpad_rows(h, gv, dv, p, tab, sp.d, st));
  }
  return BSA_OK;
}
}  // namespace

BSA_API bsa_status bsa_backward(bsa_handle h, const void* q, const void* k, const void* v,
                                const float* out, const float* dout, const int32_t* block_idx,
                                const float* lse, float* dq, float* dk, float* dv, int batch,
                                int heads, int n, int d, bsa_dtype dtype, int block, int topk,
                                float scale, int causal, void* stream) {
  const char* fn = "bsa_backward";
  if (!h) return fail(nullptr, BSA_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  const Shape s{batch, heads, n, d};
  TRY(check_shape(h, fn, s, dtype, block, true));
  TRY(check_dynamic(h, fn, s, topk, causal));
  return backward_impl(h, fn, q, k, v, out, dout, block_idx, lse, dq, dk, dv, plan_dense(s), dtype, topk,
                       scale, causal, stream);
}



// ------------------------------------------------- variable lengths --

namespace {
bsa_status check_varlen(bsa_handle h, const char* fn, int heads, int d, bsa_dtype dtype, int block, int topk,
                        int causal) {
  if (dtype != BSA_FP32 && dtype != BSA_BF16)
    return fail(h, BSA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, int(dtype));
  if (block != 64) return fail(h, BSA_ERR_UNSUPPORTED, "%s: block must be 64 (got %d)", fn, block);
  if (d != 64 && d != 128) return fail(h, BSA_ERR_UNSUPPORTED, "%s: d must be 64 or 128 (got %d)", fn, d);
  if (heads < 1) return fail(h, BSA_ERR_INVALID_ARG, "%s: heads must be >= 1 (got %d)", fn, heads);
  if (topk < 1) return fail(h, BSA_ERR_INVALID_ARG, "%s: topk must be >= 1 (got %d)", fn, topk);
  if (causal != 0 && causal != 1)
    return fail(h, BSA_ERR_INVALID_ARG, "%s: causal must be 0 or 1 (got %d)", fn, causal);
  return BSA_OK;
}

bsa_status check_plan_size(bsa_handle h, const char* fn, const Plan& p) {
  if (p.ks.bh() * p.ks.n > (int64_t(1) << 31))
    return fail(h, BSA_ERR_UNSUPPORTED, "%s: problem too large (heads * padded rows = %lld)", fn,
                (long long)(p.ks.bh() * p.ks.n));
  return BSA_OK;
}
}  // namespace

BSA_API bsa_status bsa_forward_varlen(bsa_handle h, const void* q, const void* k, const void* v, float* out,
                                      int32_t* block_idx_out, float* lse_out, const int32_t* cu_seqlens,
                                      int nseq, int heads, int d, bsa_dtype dtype, int block,
                                      const int32_t* head_topk, int topk, float scale, int causal,
                                      void* stream) {
  const char* fn = "bsa_forward_varlen";
  if (!h) return fail(nullptr, BSA_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  TRY(check_varlen(h, fn, heads, d, dtype, block, topk, causal));
  Plan p;
  TRY(plan_varlen(h, fn, cu_seqlens, nseq, heads, d, &p));
  TRY(check_plan_size(h, fn, p));
  if (lse_out && (reinterpret_cast<uintptr_t>(lse_out) & 3u))
    return fail(h, BSA_ERR_INVALID_ARG, "%s: lse_out is not 4-byte aligned", fn);
  bsa::HeadBudget hb = uniform_budget(topk);
  if (head_topk) TRY(read_budgets(h, fn, head_topk, heads, topk, &hb));
  return forward_impl(h, fn, q, k, v, out, block_idx_out, lse_out, p, dtype, topk, hb, scale, causal, stream);
}

BSA_API bsa_status bsa_backward_varlen(bsa_handle h, const void* q, const void* k, const void* v,
                                       const float* out, const float* dout, const int32_t* block_idx,
                                       const float* lse, float* dq, float* dk, float* dv,
                                       const int32_t* cu_seqlens, int nseq, int heads, int d, bsa_dtype dtype,
                                       int block, int topk, float scale, int causal, void* stream) {
  const char* fn = "bsa_backward_varlen";
  if (!h) return fail(nullptr, BSA_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  TRY(check_varlen(h, fn, heads, d, dtype, block, topk, causal));
  Plan p;
  TRY(plan_varlen(h, fn, cu_seqlens, nseq, heads, d, &p));
  TRY(check_plan_size(h, fn, p));
  return backward_impl(h, fn, q, k, v, out, dout, block_idx, lse, dq, dk, dv, p, dtype, topk, scale, causal,
                       stream);
}

// ------------------------------------------------------ static forward --

BSA_API bsa_status bsa_tiles_create(bsa_handle h, int n, int tile, const int32_t* row_ptr,
                                    const int32_t* col, const uint64_t* rowmask, int64_t nnz,
                                    bsa_tiles* out) {
  const char* fn = "bsa_tiles_create";
  if (!h) return fail(nullptr, BSA_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  if (!out) return fail(h, BSA_ERR_INVALID_ARG, "%s: out is NULL", fn);
  *out = nullptr;
  char why[256] = {0};
  const bsa_status st = bsa::tiles_check(row_ptr, col, rowmask, nnz, n, tile, why, sizeof why);
  if (st != BSA_OK) return fail(h, st, "%s: %s", fn, why);
  if (nnz > (int64_t(1) << 31) - 1)
    return fail(h, BSA_ERR_UNSUPPORTED, "%s: at most 2^31 - 1 list entries (got %lld)", fn, (long long)nnz);
  DeviceGuard dg(h->device);
  bsa_tiles t = new (std::nothrow) bsa_tiles_s();
  if (!t) return fail(h, BSA_ERR_OUT_OF_MEMORY, "%s: host allocation failed", fn);
  t->device = h->device;
  t->n = n;
  t->nt = (n + 63) / 64;
  t->nnz = nnz;
  t->row_ptr.assign(row_ptr, row_ptr + t->nt + 1);
  size_t have = 0;
  bsa_status r = BSA_OK;
  if (nnz > 0) {
    r = grow(h, reinterpret_cast<void**>(&t->col), &have, size_t(nnz) * 4, "tile list");
    if (r == BSA_OK && hipMemcpy(t->col, col, size_t(nnz) * 4, hipMemcpyHostToDevice) != hipSuccess)
      r = fail(h, BSA_ERR_LAUNCH, "%s: copy of the tile list failed", fn);
    if (r == BSA_OK && rowmask) {
      have = 0;
      r = grow(h, reinterpret_cast<void**>(&t->rowmask), &have, size_t(nnz) * 64 * 8, "tile row masks");
      if (r == BSA_OK &&
          hipMemcpy(t->rowmask, rowmask, size_t(nnz) * 64 * 8, hipMemcpyHostToDevice) != hipSuccess)
        r = fail(h, BSA_ERR_LAUNCH, "%s: copy of the row masks failed", fn);
    }
  }
  if (r != BSA_OK) {
    (void)bsa_tiles_destroy(t);
    return r;
  }
  *out = t;
  return BSA_OK;
}

BSA_API bsa_status bsa_tiles_destroy(bsa_tiles t) {
  if (!t) return BSA_OK;
  DeviceGuard dg(t->device);
  if (t->col) (void)hipFree(t->col);
  if (t->rowmask) (void)hipFree(t->rowmask);
  for (auto& sc : t->schedules) {
    if (sc.d_items) (void)hipFree(sc.d_items);
    if (sc.d_split) (void)hipFree(sc.d_split);
  }
  delete t;
  return BSA_OK;
}

namespace {

// Work items of at most S key tiles (a longer query-tile list is cut into
// ceil(count / S) items of near-equal length that write partials), ordered
// heaviest first; empty query tiles get an item of length 0 (it writes zeros).
bsa_status tiles_schedule(bsa_handle h, bsa_tiles t, int64_t S, const bsa_tiles_s::Schedule** out) {
  for (const auto& sc : t->schedules)
    if (sc.S == S) {
      *out = &sc;
      return BSA_OK;
    }
  bsa_tiles_s::Schedule sc;
  sc.S = S;
  for (int q = 0; q < t->nt; ++q) {
    const int p0 = t->row_ptr[q], c = t->row_ptr[q + 1] - p0;
    if (c <= S) {
      sc.items.push_back(make_int4(q, p0, c, -1));
      continue;
    }
    const int m = static_cast<int>((c + S - 1) / S);
    sc.split.push_back(make_int4(q, sc.nslots, m, 0));
    for (int j = 0, p = p0; j < m; ++j) {
      const int len = c / m + (j < c % m ? 1 : 0);
      sc.items.push_back(make_int4(q, p, len, sc.nslots + j));
      p += len;
    }
    sc.nslots += m;
  }
  std::stable_sort(sc.items.begin(), sc.items.end(), [](const int4& a, const int4& b) { return a.z > b.z; });
  size_t have = 0;
  TRY(grow(h, reinterpret_cast<void**>(&sc.d_items), &have, sc.items.size() * sizeof(int4), "static work items"));
  if (!sc.split.empty()) {
    have = 0;
    const bsa_status r = grow(h, reinterpret_cast<void**>(&sc.d_split), &have, sc.split.size() * sizeof(int4),
                              "static split list");
    if (r != BSA_OK) {
      (void)hipFree(sc.d_items);
      return r;
    }
  }
  if (hipMemcpy(sc.d_items, sc.items.data(), sc.items.size() * sizeof(int4), hipMemcpyHostToDevice) != hipSuccess ||
      (!sc.split.empty() &&
       hipMemcpy(sc.d_split, sc.split.data(), sc.split.size() * sizeof(int4), hipMemcpyHostToDevice) != hipSuccess)) {
    (void)hipFree(sc.d_items);
    if (sc.d_split) (void)hipFree(sc.d_split);
    return fail(h, BSA_ERR_LAUNCH, "bsa_forward_static: copy of the work-item schedule failed");
  }
  t->schedules.push_back(std::move(sc));
  *out = &t->schedules.back();
  return BSA_OK;
}

// Item size: enough items for about four workgroups per CU (halving from one
// item per query tile), and no item longer than about twice the mean list.
int64_t pick_item_tiles(const bsa_tiles_s& t, int64_t bh) {
  int64_t maxc = 1, total = 0;
  for (int q = 0; q < t.nt; ++q) {
    const int64_t c = t.row_ptr[q + 1] - t.row_ptr[q];
    maxc = c > maxc ? c : maxc;
    total += c;
  }
  // About two work items per compute unit (256 CUs): cut each query tile's
  // list into `per` items when there are too few query tiles for that (at
  // N = 8k, one head, S = 5: 0.040 ms against 0.043 at S = 4 and 0.059 at one
  // item per tile); and no item longer than about twice the mean list, so a
  // skewed list is spread over several items whatever the problem size.
  const int64_t tiles = bh * t.nt;
  const int64_t per = tiles >= 512 ? 1 : (512 + tiles - 1) / tiles;
  const int64_t S = (maxc + per - 1) / per;
  int64_t bal = (2 * total + t.nt - 1) / t.nt;
  if (bal < 4) bal = 4;
  return S < bal ? S : bal;
}

}  // namespace

BSA_API bsa_status bsa_forward_static(bsa_handle h, const void* q, const void* k, const void* v,
                                      float* out, int batch, int heads, int n, int d,
                                      bsa_dtype dtype, int tile, bsa_tiles tiles, float scale,
                                      void* stream) {
  const char* fn = "bsa_forward_static";
  if (!h) return fail(nullptr, BSA_ERR_INVALID_ARG, "%s: handle is NULL", fn);
  const Shape s{batch, heads, n, d};
  TRY(check_shape(h, fn, s, dtype, tile, true));
  TRY(check_scale(h, fn, scale));
  TRY(check_ptr(h, fn, "q", q));
  TRY(check_ptr(h, fn, "k", k));
  TRY(check_ptr(h, fn, "v", v));
  TRY(check_ptr(h, fn, "out", out));
  if (!tiles) return fail(h, BSA_ERR_INVALID_ARG, "%s: tiles is NULL", fn);
  if (tiles->n != n)
    return fail(h, BSA_ERR_INVALID_ARG, "%s: the tile list was made for n = %d, not %d", fn, tiles->n, n);
  if (tiles->device != h->device)
    return fail(h, BSA_ERR_INVALID_ARG, "%s: the tile list lives on device %d, the handle on %d", fn,
                tiles->device, h->device);
  DeviceGuard dg(h->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t S = h->static_item_tiles > 0 ? h->static_item_tiles : pick_item_tiles(*tiles, s.bh());
  const bsa_tiles_s::Schedule* sc = nullptr;
  TRY(tiles_schedule(h, tiles, S, &sc));
  bsa::StaticLaunch a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.bh = s.bh();
  a.n = n;
  a.d = d;
  a.dtype = dtype;
  a.scale = scale;
  a.col = tiles->col;
  a.rowmask = tiles->rowmask;
  a.items = sc->d_items;
  a.nitems = int64_t(sc->items.size());
  a.split = sc->d_split;
  a.nsplit = int64_t(sc->split.size());
  a.nslots = sc->nslots;
  if (sc->nslots > 0) {
    const size_t rows = size_t(s.bh()) * sc->nslots * 64;
    TRY(grow_buf(h, h->s_part, rows * d * 4, "static partial rows"));
    TRY(grow_buf(h, h->s_lse, rows * 4, "static partial log-sum-exp"));
    a.part = static_cast<float*>(h->s_part.p);
    a.part_lse = static_cast<float*>(h->s_lse.p);
  }
  TRY(timed_launch(h, BSA_STAGE_FINE, st, "sparse_flash_fwd (static)",
                   [&] { return bsa::launch_sparse_flash_static(a, st); }));
  if (a.nsplit == 0) return BSA_OK;
  return timed_launch(h, BSA_STAGE_STATIC_COMBINE, st, "static partial merge",
                      [&] { return bsa::launch_static_combine(a, st); });
}

// ------------------------------------------------------------- timing ---

BSA_API bsa_status bsa_profile_enable(bsa_handle h, int on) {
  if (!h) return fail(nullptr, BSA_ERR_INVALID_ARG, "bsa_profile_enable: handle is NULL");
  h->profiling = on != 0;
  return BSA_OK;
}

BSA_API bsa_status bsa_profile_read(bsa_handle h, double* ms, int64_t* launches, int reset) {
  if (!h || !ms) return fail(h, BSA_ERR_INVALID_ARG, "bsa_profile_read: NULL argument");
  DeviceGuard dg(h->device);
  for (int i = 0; i < BSA_NUM_STAGES; ++i) {
    ms[i] = 0.0;
    if (launches) launches[i] = 0;
  }
  for (auto& r : h->recs) {
    if (hipEventSynchronize(r.b) != hipSuccess)
      return fail(h, BSA_ERR_LAUNCH, "bsa_profile_read: event wait failed");
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
      return fail(h, BSA_ERR_LAUNCH, "bsa_profile_read: elapsed-time query failed");
    ms[r.stage] += t;
    if (launches) launches[r.stage] += 1;
  }
  if (reset) {
    for (auto& r : h->recs) {
      h->free_events.push_back(r.a);
      h->free_events.push_back(r.b);
    }
    h->recs.clear();
  }
  return BSA_OK;
}

BSA_API bsa_status bsa_select_fallbacks(bsa_handle h, int64_t* counts, int reset) {
  if (!h || !counts) return fail(h, BSA_ERR_INVALID_ARG, "bsa_select_fallbacks: NULL argument");
  DeviceGuard dg(h->device);
  int32_t c[2] = {0, 0};
  if (hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(c, h->fallbacks, sizeof(c), hipMemcpyDeviceToHost) != hipSuccess ||
      (reset && hipMemset(h->fallbacks, 0, sizeof(c)) != hipSuccess)) {
    (void)hipGetLastError();
    return fail(h, BSA_ERR_LAUNCH, "bsa_select_fallbacks: reading the counters failed");
  }
  counts[0] = c[0];
  counts[1] = c[1];
  return BSA_OK;
}
