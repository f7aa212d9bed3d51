// saf_api.cpp -- the C ABI of libsaf.so (declared in include/saf.h): argument checks, workspace
// layout and kernel launch order.  Every check runs before the first HIP call, so a rejected call
// enqueues nothing.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include <initializer_list>

#include "../../include/saf.h"
#include "saf_internal.h"

namespace {

thread_local char g_err[512] = "";

saf_status fail(saf_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

saf_status hip_fail(hipError_t e, const char* where) {
  return fail(SAF_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
constexpr int kMaxT = 65536;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape checks common to the layer calls.  Returns SAF_OK or the status to report.
saf_status check_shape(int B, int H, int T, int d) {
  if (B < 0 || H < 1 || T < 0) return fail(SAF_ERR_INVALID_ARG, "need B >= 0, H >= 1, T >= 0 (got B=%d H=%d T=%d)", B, H, T);
  if (H > saf::kMaxHeads) return fail(SAF_ERR_UNSUPPORTED, "H=%d exceeds the supported %d heads", H, saf::kMaxHeads);
  if (T > kMaxT) return fail(SAF_ERR_UNSUPPORTED, "T=%d exceeds the supported %d", T, kMaxT);
  if (d != 64 && d != 128) return fail(SAF_ERR_UNSUPPORTED, "head width d=%d is not supported (64 or 128)", d);
  return SAF_OK;
}

saf_status check_groups(int H, int Hkv) {
  if (Hkv < 1 || Hkv > H || H % Hkv != 0)
    return fail(SAF_ERR_INVALID_ARG, "Hkv=%d must divide H=%d (query heads per key/value head)", Hkv, H);
  return SAF_OK;
}

bool sizes_ok(int B, int H, int T, int d) {
  return B >= 0 && H >= 1 && H <= saf::kMaxHeads && T >= 0 && T <= kMaxT && (d == 64 || d == 128);
}

struct Need {
  const void* p;
  const char* name;
};

saf_status check_ptrs(std::initializer_list<Need> ptrs) {
  for (const Need& n : ptrs) {
    if (!n.p) return fail(SAF_ERR_INVALID_ARG, "%s is NULL", n.name);
    if (!aligned16(n.p)) return fail(SAF_ERR_INVALID_ARG, "%s is not 16-byte aligned", n.name);
  }
  return SAF_OK;
}

saf_status check_scale(float scale, int d, float* out) {
  if (isnan(scale) || isinf(scale)) return fail(SAF_ERR_INVALID_ARG, "scale must be finite");
  *out = scale > 0.f ? scale : 1.0f / sqrtf((float)d);
  return SAF_OK;
}

saf_status fill_mask(const uint8_t* replaced, int H, uint64_t* rep, bool* any_rep) {
  memset(rep, 0, sizeof(uint64_t) * (saf::kMaxHeads / 64));
  if (!replaced) return fail(SAF_ERR_INVALID_ARG, "replaced (host mask) is NULL");
  *any_rep = false;
  for (int h = 0; h < H; ++h)
    if (replaced[h]) {
      rep[h >> 6] |= 1ull << (h & 63);
      *any_rep = true;
    }
  return SAF_OK;
}

// Slice order of the work items (LayerArgs::qord, kvord; SlotOrder describes why).  cost[h] is a
// head's class key (larger = more expensive); heads are listed by descending key, ties in index
// order.  More distinct keys than kMaxClasses collapse into one class (order kept).
static void fill_slot_order(saf::SlotOrder& o, const int* cost, int n) {
  int m = 0, ncls = 0;
  int keys[saf::kMaxHeads + 1];
  for (int h = 0; h < n; ++h) keys[h] = cost[h];
  int prev = INT32_MAX;
  o.cls[0] = 0;
  while (m < n) {
    int best = INT32_MIN;
    for (int h = 0; h < n; ++h)
      if (keys[h] < prev && keys[h] > best) best = keys[h];
    for (int h = 0; h < n; ++h)
      if (keys[h] == best) o.head[m++] = (uint8_t)h;
    if (ncls < saf::kMaxClasses) ++ncls;
    o.cls[ncls] = (int16_t)m;
    prev = best;
  }
  o.ncls = ncls;
}

void fill_order(saf::LayerArgs& la, const uint8_t* replaced) {
  int cost[saf::kMaxHeads];
  la.n_ord = 0;
  for (int h = 0; h < la.H; ++h) {
    cost[h] = replaced[h] ? 0 : 1;
    la.n_ord += cost[h];
  }
  fill_slot_order(la.qord, cost, la.H);
  const int G = la.H / la.Hkv;
  la.n_kv_ord = 0;
  for (int hk = 0; hk < la.Hkv; ++hk) {
    cost[hk] = 0;
    for (int m = 0; m < G; ++m) cost[hk] += !replaced[hk * G + m];
    la.n_kv_ord += cost[hk] > 0;
  }
  fill_slot_order(la.kvord, cost, la.Hkv);
}

// ---- optional per-kernel event tracing (saf_trace_begin / saf_trace_end)
struct Trace {
  saf_kernel_event* ev = nullptr;
  int cap = 0;
  int n = 0;
};
thread_local Trace g_trace;

// Launch one kernel through `fn`, bracketed by the caller's trace events when tracing is on.
template <typename F>
hipError_t traced(const char* name, hipStream_t s, F&& fn) {
  Trace& t = g_trace;
  const bool rec = t.ev && t.n < t.cap;
  if (rec) {
    hipError_t e = hipEventRecord(t.ev[t.n].start, s);
    if (e != hipSuccess) return e;
  }
  hipError_t e = fn();
  if (e != hipSuccess) return e;
  if (rec) {
    t.ev[t.n].name = name;
    e = hipEventRecord(t.ev[t.n].stop, s);
    if (e != hipSuccess) return e;
    ++t.n;
  }
  return hipSuccess;
}

// A second stream per (host thread, device), created on first use and kept, on which the
// backward's query-block kernel runs beside the key-block kernel: both depend only on the
// preprocess and write disjoint outputs, so the hardware can fill one kernel's tail with the other's
// blocks.  The fork and join are event record / wait pairs on the caller's stream, which a graph
// capture of that stream records as dependencies.  Default stream priority.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
thread_local SideStream g_side[kMaxDevices];
thread_local bool g_overlap = false;  // saf_set_backward_overlap

// The side stream of the current device, or nullptr (then everything runs on the caller's stream).
SideStream* side_stream() {
  if (!g_overlap) return nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  SideStream& ss = g_side[dev];
  if (!ss.s) {
    hipStream_t s = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
      if (f) hipEventDestroy(f);
      hipStreamDestroy(s);
      return nullptr;
    }
    ss.s = s;
    ss.fork = f;
    ss.join = j;
  }
  return &ss;
}

// ---- Library-owned workspace of saf_attn_bwd_noalloc (for callers that cannot allocate) ----------
// One array per device (each GPU the library runs on holds its own copy until the process ends).
// Host code never uses the array's name as an address: on the host it is only a stand-in for the
// symbol, and a kernel given it would fault.  The device address is looked up once per device
// with hipGetSymbolAddress (the device current) and kept.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` in *out (looked up on the first call on a device).
saf_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "no-allocation backward: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SAF_ERR_UNSUPPORTED, "device %d is beyond the %d devices this library serves", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "no-allocation backward: hipGetSymbolAddress");
    if (!ptr) return fail(SAF_ERR_HIP, "no-allocation backward: hipGetSymbolAddress gave no address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SAF_OK;
}

size_t pattern_bytes(int H, int P) {
  return align_up(sizeof(float) * (size_t)saf::pattern_stride(P) * H);
}
size_t fwd_ws(int B, int H, int T, int d) {
  (void)B; (void)d;
  return pattern_bytes(H, T);  // the prepared pattern, when the caller passes none
}
size_t bwd_ws(int B, int H, int T, int d) {
  (void)d;
  return pattern_bytes(H, T) + align_up(sizeof(float) * (size_t)B * H * T);  // pattern, delta
}

// The backward keeps the ordinary heads' dS between its two kernels (bwd_kv stores it, bwd_dq_ds
// reads it) for bf16 at d = 128 without grouped key/value heads, when the workspace has room.
bool ds_path(saf_dtype dt, int d, int H, int Hkv, int n_ord) {
  return dt == SAF_BF16 && d == 128 && Hkv == H && n_ord > 0;
}

size_t pgrad_ws(int B, int H, int T, int d) {
  (void)d;
  const size_t nkb = (size_t)(T + saf::pattern_grad_sub_block() - 1) / saf::pattern_grad_sub_block();
  return pattern_bytes(H, T) + 2 * align_up(sizeof(float) * (size_t)B * H * T) +
         align_up(sizeof(float) * (size_t)B * H * nkb * T) +  // pattern, delta, da / dr partials
         align_up(sizeof(double) * (size_t)B * H * saf::pattern_grad_chunks(T) * T);
}

struct FitLayout {
  size_t colp, rowp, diagp, entp, state, zpart, gpart, bmax, total;
};
FitLayout fit_layout(int H, int T) {
  const size_t nrt = (T + saf::fit_row_tile() - 1) / saf::fit_row_tile();
  const size_t nct = (T + saf::fit_col_tile() - 1) / saf::fit_col_tile();
  FitLayout L;
  L.colp = 0;
  L.rowp = L.colp + align_up(sizeof(double) * H * nrt * T);
  L.diagp = L.rowp + align_up(sizeof(double) * H * nct * T);
  L.entp = L.diagp + align_up(sizeof(double) * H * nrt * nct * saf::fit_tile_distances());
  L.state = L.entp + align_up(sizeof(double) * H * nrt * nct);
  const size_t ncb = (T + saf::fit_conv_block() - 1) / saf::fit_conv_block();
  L.zpart = L.state + align_up(sizeof(double) * H * saf::fit_state_stride(T));
  L.gpart = L.zpart + align_up(sizeof(double) * H * ncb * T);
  L.bmax = L.gpart + align_up(sizeof(double) * H * ncb * 2 * T);
  L.total = L.bmax + align_up(sizeof(double) * H * saf::fit_adam_blocks(T) * 2);
  return L;
}

// Point la.pat at the caller's prepared pattern, or prepare one for length T at ws.
saf_status setup_pattern(saf::LayerArgs& la, bool any_rep, const void* pattern, int T, void* ws,
                         hipStream_t stream, const char* what) {
  if (!any_rep) return SAF_OK;
  if (pattern) {
    la.pat.base = const_cast<float*>(reinterpret_cast<const float*>(pattern));
    la.pat.P = la.pat_len;
  } else {
    la.pat.base = reinterpret_cast<float*>(ws);
    la.pat.P = T;
  }
  la.pat.stride = saf::pattern_stride(la.pat.P);
  if (!pattern) {
    hipError_t e = traced("pattern_prepare", stream, [&] { return saf::launch_pattern_prepare(la, stream); });
    if (e != hipSuccess) return hip_fail(e, what);
  }
  return SAF_OK;
}
size_t calib_tiles(int T, int* nqt, int* nkt) {
  *nqt = (T + saf::kCalibQTile - 1) / saf::kCalibQTile;
  *nkt = (T + saf::kCalibKTile - 1) / saf::kCalibKTile;
  return (size_t)(*nqt) * (*nkt);
}
// bf16 queries in fragment order (CalibArgs::qfrag): 2 bytes per element of the padded rows
size_t calib_qfrag_bytes(int N, int H, int nqt, int d) {
  return align_up(2 * (size_t)N * H * nqt * saf::kCalibQTile * d);
}
size_t calib_ws(int N, int H, int T, int d) {
  int nqt, nkt;
  const size_t tiles = calib_tiles(T, &nqt, &nkt);
  return align_up(sizeof(float) * (size_t)N * H * T) + 2 * align_up(sizeof(double) * (size_t)H * tiles) +
         calib_qfrag_bytes(N, H, nqt, d);
}

}  // namespace

extern "C" {

size_t saf_attn_fwd_workspace_size(int B, int H, int T, int d) {
  if (!sizes_ok(B, H, T, d)) return SIZE_MAX;
  return fwd_ws(B, H, T, d);
}

size_t saf_attn_bwd_workspace_size(int B, int H, int T, int d) {
  if (!sizes_ok(B, H, T, d)) return SIZE_MAX;
  if (B == 0 || T == 0) return 0;
  return bwd_ws(B, H, T, d);
}

size_t saf_attn_bwd_ds_workspace_size(saf_dtype dt, int B, int H, int Hkv, int T, int d, int n_replaced) {
  if ((dt != SAF_F32 && dt != SAF_BF16) || !sizes_ok(B, H, T, d) || Hkv < 1 || Hkv > H ||
      H % Hkv != 0 || n_replaced < 0 || n_replaced > H)
    return SIZE_MAX;
  if (B == 0 || T == 0) return 0;
  const size_t base = bwd_ws(B, H, T, d);
  if (!ds_path(dt, d, H, Hkv, H - n_replaced)) return base;
  return base + align_up(saf::ds_bytes(B, H - n_replaced, T));
}

static saf_status fwd_impl(saf_dtype dt, int B, int H, int Hkv, int T, int d, const void* q,
                           const void* k, const void* v, const uint8_t* replaced, const float* a,
                           const float* r, int pat_len, const void* pattern, float scale, void* o,
                           float* lse, void* ws, size_t ws_bytes, hipStream_t stream);
static saf_status bwd_impl(saf_dtype dt, int B, int H, int Hkv, int T, int d, const void* q,
                           const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, const uint8_t* replaced, const float* a,
                           const float* r, int pat_len, const void* pattern, float scale, void* dq,
                           void* dk, void* dv, void* ws, size_t ws_bytes, hipStream_t stream,
                           bool allow_side = true, bool lib_ws = false);

saf_status saf_attn_fwd(saf_dtype dt, int B, int H, int T, int d, const void* q, const void* k,
                        const void* v, const uint8_t* replaced, const float* a, const float* r,
                        int pat_len, const void* pattern, float scale, void* o, float* lse,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  return fwd_impl(dt, B, H, H, T, d, q, k, v, replaced, a, r, pat_len, pattern, scale, o, lse, ws,
                  ws_bytes, stream);
}

saf_status saf_attn_fwd_gqa(saf_dtype dt, int B, int H, int Hkv, int T, int d, const void* q,
                            const void* k, const void* v, const uint8_t* replaced, const float* a,
                            const float* r, int pat_len, const void* pattern, float scale, void* o,
                            float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return fwd_impl(dt, B, H, Hkv, T, d, q, k, v, replaced, a, r, pat_len, pattern, scale, o, lse, ws,
                  ws_bytes, stream);
}

saf_status saf_attn_bwd(saf_dtype dt, int B, int H, int T, int d, const void* q, const void* k,
                        const void* v, const void* o, const void* dout, const float* lse,
                        const uint8_t* replaced, const float* a, const float* r, int pat_len,
                        const void* pattern, float scale, void* dq, void* dk, void* dv, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  return bwd_impl(dt, B, H, H, T, d, q, k, v, o, dout, lse, replaced, a, r, pat_len, pattern, scale,
                  dq, dk, dv, ws, ws_bytes, stream);
}

saf_status saf_attn_bwd_gqa(saf_dtype dt, int B, int H, int Hkv, int T, int d, const void* q,
                            const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, const uint8_t* replaced, const float* a,
                            const float* r, int pat_len, const void* pattern, float scale, void* dq,
                            void* dk, void* dv, void* ws, size_t ws_bytes, hipStream_t stream) {
  return bwd_impl(dt, B, H, Hkv, T, d, q, k, v, o, dout, lse, replaced, a, r, pat_len, pattern,
                  scale, dq, dk, dv, ws, ws_bytes, stream);
}

saf_status saf_attn_bwd_noalloc(saf_dtype dt, int B, int H, int T, int d, const void* q,
                                const void* k, const void* v, const void* o, const void* dout,
                                const float* lse, const uint8_t* replaced, const float* a,
                                const float* r, int pat_len, const void* pattern, float scale,
                                void* dq, void* dk, void* dv, hipStream_t stream) {
  // the library's device array as the workspace; no side stream (it would be created on first use)
  return bwd_impl(dt, B, H, H, T, d, q, k, v, o, dout, lse, replaced, a, r, pat_len, pattern, scale,
                  dq, dk, dv, nullptr, 0, stream, /*allow_side=*/false, /*lib_ws=*/true);
}

size_t saf_attn_bwd_pattern_workspace_size(int B, int H, int T, int d) {
  if (!sizes_ok(B, H, T, d)) return SIZE_MAX;
  if (B == 0 || T == 0) return 0;
  return pgrad_ws(B, H, T, d);
}

size_t saf_calibrate_workspace_size(int N, int H, int T, int d) {
  if (N < 2 || !sizes_ok(1, H, T, d)) return SIZE_MAX;
  if (T == 0) return 0;
  return calib_ws(N, H, T, d);
}

const char* saf_last_error(void) { return g_err; }

size_t saf_pattern_size(int H, int pat_len) {
  if (H < 1 || H > saf::kMaxHeads || pat_len < 0 || pat_len > kMaxT) return SIZE_MAX;
  return pattern_bytes(H, pat_len);
}

saf_status saf_pattern_prepare(int H, const uint8_t* replaced, const float* a, const float* r,
                               int pat_len, void* pattern, size_t pattern_bytes_given,
                               hipStream_t stream) {
  g_err[0] = 0;
  if (H < 1) return fail(SAF_ERR_INVALID_ARG, "need H >= 1 (got %d)", H);
  if (H > saf::kMaxHeads) return fail(SAF_ERR_UNSUPPORTED, "H=%d exceeds the supported %d heads", H, saf::kMaxHeads);
  if (pat_len < 0) return fail(SAF_ERR_INVALID_ARG, "pat_len=%d is negative", pat_len);
  if (pat_len > kMaxT) return fail(SAF_ERR_UNSUPPORTED, "pat_len=%d exceeds the supported %d", pat_len, kMaxT);
  saf::LayerArgs la;
  memset(&la, 0, sizeof(la));
  bool any_rep = false;
  saf_status st = fill_mask(replaced, H, la.rep, &any_rep);
  if (st != SAF_OK) return st;
  if (!any_rep || pat_len == 0) return SAF_OK;
  if (!a || !r) return fail(SAF_ERR_INVALID_ARG, "a and r are required when a head is replaced");
  if (!pattern) return fail(SAF_ERR_INVALID_ARG, "pattern is NULL");
  if (((uintptr_t)pattern & (kAlign - 1)) != 0) return fail(SAF_ERR_INVALID_ARG, "pattern is not 256-byte aligned");
  if (pattern_bytes_given < pattern_bytes(H, pat_len))
    return fail(SAF_ERR_INVALID_ARG, "pattern buffer too small (%zu < %zu bytes)", pattern_bytes_given, pattern_bytes(H, pat_len));
  la.H = H; la.Hkv = H; la.T = pat_len; la.pat_len = pat_len;
  la.a = a; la.r = r;
  return setup_pattern(la, true, nullptr, pat_len, pattern, stream, "pattern preparation");
}

saf_status saf_set_backward_overlap(int enable) {
  g_err[0] = 0;
  g_overlap = enable != 0;
  return SAF_OK;
}

saf_status saf_trace_begin(saf_kernel_event* ev, int capacity) {
  g_err[0] = 0;
  if (!ev || capacity < 1) return fail(SAF_ERR_INVALID_ARG, "trace needs an event array and capacity >= 1");
  g_trace.ev = ev;
  g_trace.cap = capacity;
  g_trace.n = 0;
  return SAF_OK;
}

int saf_trace_end(void) {
  const int n = g_trace.n;
  g_trace = Trace();
  return n;
}

static saf_status fwd_impl(saf_dtype dt, int B, int H, int Hkv, int T, int d, const void* q,
                    const void* k, const void* v, const uint8_t* replaced, const float* a,
                    const float* r, int pat_len, const void* pattern, float scale, void* o,
                    float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (dt != SAF_F32 && dt != SAF_BF16) return fail(SAF_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  saf_status st = check_shape(B, H, T, d);
  if (st != SAF_OK) return st;
  if ((st = check_groups(H, Hkv)) != SAF_OK) return st;
  if (B == 0 || T == 0) return SAF_OK;
  saf::LayerArgs la;
  memset(&la, 0, sizeof(la));
  bool any_rep = false;
  if ((st = fill_mask(replaced, H, la.rep, &any_rep)) != SAF_OK) return st;
  bool any_ord = false;
  for (int h = 0; h < H; ++h) any_ord |= !replaced[h];
  if (any_ord && (st = check_ptrs({{q, "q"}, {k, "k"}})) != SAF_OK) return st;
  if ((st = check_ptrs({{v, "v"}, {o, "o"}})) != SAF_OK) return st;
  if (!lse) return fail(SAF_ERR_INVALID_ARG, "lse is NULL");
  if (any_rep) {
    if (!a || !r) return fail(SAF_ERR_INVALID_ARG, "a and r are required when a head is replaced");
    if (pat_len < T) return fail(SAF_ERR_INVALID_ARG, "pat_len=%d is shorter than T=%d", pat_len, T);
  }
  if (any_rep && pattern && ((uintptr_t)pattern & (kAlign - 1)) != 0)
    return fail(SAF_ERR_INVALID_ARG, "pattern is not 256-byte aligned");
  if (any_rep && !pattern) {
    const size_t need = fwd_ws(B, H, T, d);
    if (!ws) return fail(SAF_ERR_INVALID_ARG, "ws is NULL (needed to prepare the pattern)");
    if (((uintptr_t)ws & (kAlign - 1)) != 0) return fail(SAF_ERR_INVALID_ARG, "ws is not 256-byte aligned");
    if (ws_bytes < need) return fail(SAF_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", ws_bytes, need);
  }
  float s;
  if ((st = check_scale(scale, d, &s)) != SAF_OK) return st;

  la.B = B; la.H = H; la.T = T; la.d = d;
  la.Hkv = Hkv;
  fill_order(la, replaced);
  la.pat_len = pat_len;
  la.scale = s;
  la.scale_log2 = s * 1.4426950408889634f;
  la.q = q; la.k = k; la.v = v;
  la.a = a; la.r = r;
  la.lse = lse;
  la.out = o;
  if ((st = setup_pattern(la, any_rep, pattern, T, ws, stream, "pattern preparation")) != SAF_OK) return st;
  const bool bf = dt == SAF_BF16;
  hipError_t e = traced("mixed_fwd", stream, [&] { return saf::launch_mixed_fwd(la, bf, stream); });
  if (e != hipSuccess) return hip_fail(e, "mixed forward launch");
  return SAF_OK;
}

static saf_status bwd_impl(saf_dtype dt, int B, int H, int Hkv, int T, int d, const void* q,
                    const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    const uint8_t* replaced, const float* a, const float* r, int pat_len,
                    const void* pattern, float scale, void* dq, void* dk, void* dv, void* ws,
                    size_t ws_bytes, hipStream_t stream, bool allow_side, bool lib_ws) {
  g_err[0] = 0;
  if (dt != SAF_F32 && dt != SAF_BF16) return fail(SAF_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  saf_status st = check_shape(B, H, T, d);
  if (st != SAF_OK) return st;
  if ((st = check_groups(H, Hkv)) != SAF_OK) return st;
  if (B == 0 || T == 0) return SAF_OK;
  saf::LayerArgs la;
  memset(&la, 0, sizeof(la));
  bool any_rep = false;
  if ((st = fill_mask(replaced, H, la.rep, &any_rep)) != SAF_OK) return st;
  bool any_ord = false;
  for (int h = 0; h < H; ++h) any_ord |= !replaced[h];
  if (any_ord && (st = check_ptrs({{q, "q"}, {k, "k"}, {o, "o"}})) != SAF_OK) return st;
  if ((st = check_ptrs({{v, "v"}, {dout, "dout"}, {dq, "dq"}, {dk, "dk"}, {dv, "dv"}})) != SAF_OK)
    return st;
  if (!lse) return fail(SAF_ERR_INVALID_ARG, "lse is NULL");
  if (any_rep) {
    if (!a || !r) return fail(SAF_ERR_INVALID_ARG, "a and r are required when a head is replaced");
    if (pat_len < T) return fail(SAF_ERR_INVALID_ARG, "pat_len=%d is shorter than T=%d", pat_len, T);
  }
  if (any_rep && pattern && ((uintptr_t)pattern & (kAlign - 1)) != 0)
    return fail(SAF_ERR_INVALID_ARG, "pattern is not 256-byte aligned");
  const size_t need = bwd_ws(B, H, T, d);
  if (lib_ws) {  // saf_attn_bwd_noalloc: the library's device array
    if (need > kScratchBytes)
      return fail(SAF_ERR_UNSUPPORTED,
                  "saf_attn_bwd_noalloc: B=%d H=%d T=%d needs %zu workspace bytes, more than its "
                  "%zu-byte device array (call saf_attn_bwd with a workspace instead)",
                  B, H, T, need, kScratchBytes);
  } else {
    if (!ws) return fail(SAF_ERR_INVALID_ARG, "ws is NULL");
    if (((uintptr_t)ws & (kAlign - 1)) != 0) return fail(SAF_ERR_INVALID_ARG, "ws is not 256-byte aligned");
    if (ws_bytes < need) return fail(SAF_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", ws_bytes, need);
  }
  float s;
  if ((st = check_scale(scale, d, &s)) != SAF_OK) return st;
  if (lib_ws) {  // every argument checked: look up this device's array
    if ((st = scratch_address(&ws)) != SAF_OK) return st;
    ws_bytes = kScratchBytes;
  }

  la.B = B; la.H = H; la.T = T; la.d = d;
  la.Hkv = Hkv;
  fill_order(la, replaced);
  la.pat_len = pat_len;
  la.scale = s;
  la.scale_log2 = s * 1.4426950408889634f;
  la.q = q; la.k = k; la.v = v; la.o = o; la.dout = dout;
  la.a = a; la.r = r;
  la.lse = const_cast<float*>(lse);
  la.delta = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + pattern_bytes(H, T));
  la.dq = dq; la.dk = dk; la.dv = dv;
  if ((st = setup_pattern(la, any_rep, pattern, T, ws, stream, "pattern preparation")) != SAF_OK) return st;
  const bool bf = dt == SAF_BF16;
  SideStream* side = (any_ord && allow_side) ? side_stream() : nullptr;
  int n_ord = 0;
  for (int h = 0; h < H; ++h) n_ord += !replaced[h];
  // dS kept in the workspace (its room after the pattern and delta): one stream, the key-block
  // kernel first
  const bool keep_ds = !lib_ws && !side && ds_path(dt, d, H, Hkv, n_ord) &&
                       ws_bytes - need >= saf::ds_bytes(B, n_ord, T);
  if (keep_ds) {
    la.dsw = reinterpret_cast<char*>(ws) + need;
    const long long n32 = (T + 31) / 32;
    la.ds_ntri = n32 * (n32 + 1) / 2;
  }
  hipError_t e = traced("bwd_pre", stream, [&] { return saf::launch_bwd_pre(la, bf, stream); });
  if (e != hipSuccess) return hip_fail(e, "backward preprocess launch");
  if (keep_ds) {
    e = traced("bwd_kv", stream, [&] { return saf::launch_bwd_kv(la, bf, stream); });
    if (e != hipSuccess) return hip_fail(e, "backward key-block launch");
    e = traced("bwd_dq_ds", stream, [&] { return saf::launch_bwd_dq_ds(la, stream); });
    if (e != hipSuccess) return hip_fail(e, "backward query-block launch");
    return SAF_OK;
  }
  if (side) {  // fork: the query-block kernel on the side stream after the preprocess
    if ((e = hipEventRecord(side->fork, stream)) != hipSuccess) return hip_fail(e, "backward fork");
    if ((e = hipStreamWaitEvent(side->s, side->fork, 0)) != hipSuccess) return hip_fail(e, "backward fork");
    e = traced("bwd_dq", side->s, [&] { return saf::launch_bwd_dq(la, bf, side->s); });
    if (e != hipSuccess) return hip_fail(e, "backward query-block launch");
  } else if (any_ord) {
    // one stream: the query-block kernel first; the key-block kernel then finds the Q, K, V and dO
    // tiles it shares with it in the caches (1B-shaped layer: step -0.3 to -0.6%)
    e = traced("bwd_dq", stream, [&] { return saf::launch_bwd_dq(la, bf, stream); });
    if (e != hipSuccess) return hip_fail(e, "backward query-block launch");
  }
  e = traced("bwd_kv", stream, [&] { return saf::launch_bwd_kv(la, bf, stream); });
  if (e != hipSuccess) return hip_fail(e, "backward key-block launch");
  if (side) {  // join
    if ((e = hipEventRecord(side->join, side->s)) != hipSuccess) return hip_fail(e, "backward join");
    if ((e = hipStreamWaitEvent(stream, side->join, 0)) != hipSuccess) return hip_fail(e, "backward join");
  }
  return SAF_OK;
}

saf_status saf_attn_bwd_pattern(saf_dtype dt, int B, int H, int T, int d, const void* v,
                                const void* o, const void* dout, const float* lse,
                                const uint8_t* replaced, const float* a, const float* r, int pat_len,
                                const void* pattern, float* da, float* dr, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (dt != SAF_F32 && dt != SAF_BF16) return fail(SAF_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  saf_status st = check_shape(B, H, T, d);
  if (st != SAF_OK) return st;
  saf::LayerArgs la;
  memset(&la, 0, sizeof(la));
  bool any_rep = false;
  if ((st = fill_mask(replaced, H, la.rep, &any_rep)) != SAF_OK) return st;
  if (!any_rep) return SAF_OK;  // no replaced head: nothing to write
  if (!a || !r) return fail(SAF_ERR_INVALID_ARG, "a and r are required when a head is replaced");
  if (pat_len < T) return fail(SAF_ERR_INVALID_ARG, "pat_len=%d is shorter than T=%d", pat_len, T);
  if (!da || !dr) return fail(SAF_ERR_INVALID_ARG, "da and dr are required");
  if (((uintptr_t)da & 3u) || ((uintptr_t)dr & 3u)) return fail(SAF_ERR_INVALID_ARG, "da or dr is not 4-byte aligned");
  saf::HeadList rl;
  rl.n = 0;
  for (int h = 0; h < H; ++h)
    if (replaced[h]) rl.h[rl.n++] = (uint8_t)h;
  if (B == 0 || T == 0) {
    // an empty batch or sequence: the gradient is zero; clear the rows with the reduce kernel
    if (pat_len == 0) return SAF_OK;
    la.B = 0; la.H = H; la.Hkv = H; la.T = 0; la.pat_len = pat_len;
    la.da = da; la.dr = dr;
    hipError_t e = traced("pattern_grad_reduce", stream, [&] { return saf::launch_pattern_grad_reduce(la, rl, stream); });
    return e == hipSuccess ? SAF_OK : hip_fail(e, "pattern gradient reduction launch");
  }
  if ((st = check_ptrs({{v, "v"}, {o, "o"}, {dout, "dout"}})) != SAF_OK) return st;
  if (!lse) return fail(SAF_ERR_INVALID_ARG, "lse is NULL");
  if (pattern && ((uintptr_t)pattern & (kAlign - 1)) != 0)
    return fail(SAF_ERR_INVALID_ARG, "pattern is not 256-byte aligned");
  const size_t need = pgrad_ws(B, H, T, d);
  if (!ws) return fail(SAF_ERR_INVALID_ARG, "ws is NULL");
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return fail(SAF_ERR_INVALID_ARG, "ws is not 256-byte aligned");
  if (ws_bytes < need) return fail(SAF_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", ws_bytes, need);

  la.B = B; la.H = H; la.T = T; la.d = d;
  la.Hkv = H;
  fill_order(la, replaced);  // the preprocess takes the replaced slices from the query order
  la.pat_len = pat_len;
  la.v = v; la.o = o; la.dout = dout;
  la.a = a; la.r = r;
  la.lse = const_cast<float*>(lse);
  char* base = reinterpret_cast<char*>(ws) + pattern_bytes(H, T);
  const size_t slab = align_up(sizeof(float) * (size_t)B * H * T);
  la.delta = reinterpret_cast<float*>(base);
  la.delta_rep = 1;
  la.dap = reinterpret_cast<float*>(base + slab);
  la.drp = reinterpret_cast<float*>(base + 2 * slab);
  {
    const size_t nsb = (size_t)(T + saf::pattern_grad_sub_block() - 1) / saf::pattern_grad_sub_block();
    la.drc = reinterpret_cast<double*>(base + 2 * slab + align_up(sizeof(float) * (size_t)B * H * nsb * T));
  }
  la.da = da; la.dr = dr;
  if ((st = setup_pattern(la, true, pattern, T, ws, stream, "pattern preparation")) != SAF_OK) return st;
  const bool bf = dt == SAF_BF16;
  hipError_t e = traced("bwd_pre", stream, [&] { return saf::launch_bwd_pre(la, bf, stream); });
  if (e != hipSuccess) return hip_fail(e, "backward preprocess launch");
  e = traced("bwd_pattern", stream, [&] { return saf::launch_bwd_pattern(la, rl, bf, stream); });
  if (e != hipSuccess) return hip_fail(e, "pattern gradient launch");
  e = traced("pattern_grad_reduce", stream, [&] { return saf::launch_pattern_grad_reduce(la, rl, stream); });
  if (e != hipSuccess) return hip_fail(e, "pattern gradient reduction launch");
  return SAF_OK;
}

size_t saf_fit_pattern_workspace_size(int H, int T) {
  if (H < 1 || H > saf::kMaxHeads || T < 0 || T > kMaxT) return SIZE_MAX;
  if (T == 0) return 0;
  return fit_layout(H, T).total;
}

saf_status saf_fit_pattern(int H, int T, const float* ahat, int steps, double lr, float* a,
                           float* r, double* kl, double* loss, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  g_err[0] = 0;
  if (H < 1 || T < 0) return fail(SAF_ERR_INVALID_ARG, "need H >= 1 and T >= 0 (got H=%d T=%d)", H, T);
  if (H > saf::kMaxHeads) return fail(SAF_ERR_UNSUPPORTED, "H=%d exceeds the supported %d heads", H, saf::kMaxHeads);
  if (T > kMaxT) return fail(SAF_ERR_UNSUPPORTED, "T=%d exceeds the supported %d", T, kMaxT);
  if (steps < 0 || steps > 1000000) return fail(SAF_ERR_INVALID_ARG, "steps=%d is not in [0, 10^6]", steps);
  if (!(lr > 0.0) || std::isinf(lr)) return fail(SAF_ERR_INVALID_ARG, "lr must be positive and finite");
  if (T == 0) return SAF_OK;
  if (!ahat || !a || !r || !kl) return fail(SAF_ERR_INVALID_ARG, "ahat, a, r and kl are required");
  if (((uintptr_t)ahat & 3u) || ((uintptr_t)a & 3u) || ((uintptr_t)r & 3u) || ((uintptr_t)kl & 7u) ||
      ((uintptr_t)loss & 7u))
    return fail(SAF_ERR_INVALID_ARG, "misaligned pointer");
  const FitLayout L = fit_layout(H, T);
  if (!ws) return fail(SAF_ERR_INVALID_ARG, "ws is NULL");
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return fail(SAF_ERR_INVALID_ARG, "ws is not 256-byte aligned");
  if (ws_bytes < L.total) return fail(SAF_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", ws_bytes, L.total);

  saf::FitArgs fa;
  memset(&fa, 0, sizeof(fa));
  char* base = reinterpret_cast<char*>(ws);
  fa.H = H; fa.T = T;
  fa.ahat = ahat;
  fa.nrt = (T + saf::fit_row_tile() - 1) / saf::fit_row_tile();
  fa.nct = (T + saf::fit_col_tile() - 1) / saf::fit_col_tile();
  fa.colp = reinterpret_cast<double*>(base + L.colp);
  fa.rowp = reinterpret_cast<double*>(base + L.rowp);
  fa.diagp = reinterpret_cast<double*>(base + L.diagp);
  fa.entp = reinterpret_cast<double*>(base + L.entp);
  fa.state = reinterpret_cast<double*>(base + L.state);
  fa.stride = saf::fit_state_stride(T);
  fa.ncb = (T + saf::fit_conv_block() - 1) / saf::fit_conv_block();
  fa.zpart = reinterpret_cast<double*>(base + L.zpart);
  fa.gpart = reinterpret_cast<double*>(base + L.gpart);
  fa.bmax = reinterpret_cast<double*>(base + L.bmax);
  fa.a_out = a; fa.r_out = r; fa.kl = kl; fa.loss = loss;
  hipError_t e = traced("fit_marginals", stream, [&] { return saf::launch_fit_marginals(fa, stream); });
  if (e != hipSuccess) return hip_fail(e, "fit marginals launch");
  e = traced("fit_init", stream, [&] { return saf::launch_fit_init(fa, stream); });
  if (e != hipSuccess) return hip_fail(e, "fit init launch");
  for (int s = 1; s <= steps; ++s) {
    // Adam's bias corrections for step s (beta1 = 0.9, beta2 = 0.999)
    const double c1 = 1.0 - pow(0.9, (double)s), c2 = 1.0 - pow(0.999, (double)s);
    e = traced("fit_z", stream, [&] { return saf::launch_fit_z(fa, stream); });
    if (e != hipSuccess) return hip_fail(e, "fit normaliser launch");
    e = traced("fit_step", stream, [&] { return saf::launch_fit_step(fa, lr, c1, c2, stream); });
    if (e != hipSuccess) return hip_fail(e, "fit step launch");
  }
  e = traced("fit_z", stream, [&] { return saf::launch_fit_z(fa, stream); });
  if (e != hipSuccess) return hip_fail(e, "fit normaliser launch");
  e = traced("fit_final", stream, [&] { return saf::launch_fit_final(fa, stream); });
  if (e != hipSuccess) return hip_fail(e, "fit final launch");
  return SAF_OK;
}

saf_status saf_calibrate(saf_dtype dt, int N, int H, int T, int d, const void* q, const void* k,
                         float scale, float* ahat, double* svar, double* skl, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (dt != SAF_F32 && dt != SAF_BF16) return fail(SAF_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (N < 2) return fail(SAF_ERR_INVALID_ARG, "N=%d: the variance score needs N >= 2", N);
  saf_status st = check_shape(1, H, T, d);
  if (st != SAF_OK) return st;
  if (T == 0) return SAF_OK;
  if ((st = check_ptrs({{q, "q"}, {k, "k"}, {ahat, "ahat"}})) != SAF_OK) return st;
  if (!svar) return fail(SAF_ERR_INVALID_ARG, "svar is NULL");
  if ((uintptr_t)svar & 7u) return fail(SAF_ERR_INVALID_ARG, "svar is not 8-byte aligned");
  if ((uintptr_t)skl & 7u) return fail(SAF_ERR_INVALID_ARG, "skl is not 8-byte aligned");
  const size_t need = calib_ws(N, H, T, d);
  if (!ws) return fail(SAF_ERR_INVALID_ARG, "ws is NULL");
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return fail(SAF_ERR_INVALID_ARG, "ws is not 256-byte aligned");
  if (ws_bytes < need) return fail(SAF_ERR_INVALID_ARG, "workspace too small (%zu < %zu bytes)", ws_bytes, need);
  float s;
  if ((st = check_scale(scale, d, &s)) != SAF_OK) return st;

  saf::CalibArgs ca;
  memset(&ca, 0, sizeof(ca));
  ca.N = N; ca.H = H; ca.T = T; ca.d = d;
  ca.scale_log2 = s * 1.4426950408889634f;
  ca.q = q; ca.k = k;
  ca.lse2 = reinterpret_cast<float*>(ws);
  ca.m2 = reinterpret_cast<double*>(reinterpret_cast<char*>(ws) + align_up(sizeof(float) * (size_t)N * H * T));
  ca.ahat = ahat;
  ca.svar = svar;
  ca.skl = skl;
  const size_t tiles = calib_tiles(T, &ca.n_qt, &ca.n_kt);
  ca.n_ag = saf::calib_groups(ca.n_qt);
  ca.klp = reinterpret_cast<double*>(reinterpret_cast<char*>(ca.m2) + align_up(sizeof(double) * (size_t)H * tiles));
  const bool bf = dt == SAF_BF16;
  ca.qfrag = bf ? reinterpret_cast<char*>(ca.klp) + align_up(sizeof(double) * (size_t)H * tiles) : nullptr;
  hipError_t e = traced("calib_lse", stream, [&] { return saf::launch_calib_lse(ca, bf, stream); });
  if (e != hipSuccess) return hip_fail(e, "calibration statistics launch");
  e = traced("calib_stats", stream, [&] { return saf::launch_calib_stats(ca, bf, stream); });
  if (e != hipSuccess) return hip_fail(e, "calibration tile launch");
  e = traced("calib_zero", stream, [&] { return saf::launch_calib_zero(ca, stream); });
  if (e != hipSuccess) return hip_fail(e, "calibration zero-fill launch");
  e = traced("calib_reduce", stream, [&] { return saf::launch_calib_reduce(ca, stream); });
  if (e != hipSuccess) return hip_fail(e, "calibration reduction launch");
  return SAF_OK;
}

saf_status saf_select_heads(int L, int H, const double* score, const uint8_t* accepted,
                            double ratio, uint8_t* replaced, int* n_selected) {
  g_err[0] = 0;
  if (L < 1 || H < 1 || (long long)L * H > (1LL << 24))
    return fail(SAF_ERR_INVALID_ARG, "L=%d, H=%d: need L, H >= 1 and L*H <= 2^24", L, H);
  if (!score || !replaced || !n_selected) return fail(SAF_ERR_INVALID_ARG, "score, replaced or n_selected is NULL");
  if (!(ratio >= 0.0 && ratio <= 1.0)) return fail(SAF_ERR_INVALID_ARG, "ratio %g is not in [0, 1]", ratio);
  const int n = L * H;
  for (int x = 0; x < n; ++x)
    if (std::isnan(score[x])) return fail(SAF_ERR_INVALID_ARG, "score of layer %d head %d is NaN", x / H, x % H);
  // k = round(ratio * L * H), halves to even
  const double want = ratio * (double)n, fl = std::floor(want);
  int k = (int)fl;
  if (want - fl > 0.5 || (want - fl == 0.5 && (k & 1))) ++k;
  std::vector<int> order(n);
  for (int x = 0; x < n; ++x) order[x] = x;
  // ascending score; equal scores keep (layer, head) order, which is the index order
  std::stable_sort(order.begin(), order.end(), [&](int u, int v) { return score[u] < score[v]; });
  memset(replaced, 0, (size_t)n);
  int taken = 0;
  for (int x = 0; x < n && taken < k; ++x) {
    const int idx = order[x];
    if (accepted && !accepted[idx]) continue;
    replaced[idx] = 1;
    ++taken;
  }
  *n_selected = taken;
  return SAF_OK;
}

}  // extern "C"
