// la_api.hip -- C-ABI front end: argument validation, device check, dispatch, status codes.
// The operation and the contract of every entry point are documented in lightning_attn.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "la_internal.h"
#include "lightning_attn.h"

namespace {

thread_local char g_err[512] = "";

la_status fail(la_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
la_status fail(la_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Whether the byte ranges [a, a + na) and [b, b + nb) intersect (empty ranges never do).
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t elem_bytes(la_dtype dtype) { return dtype == LA_BF16 ? 2 : 4; }

// Callers may pass any int as a dtype; reading a value outside the enumerators through the enum
// type is undefined in C++, so every entry point checks the argument's bytes first and only
// then uses it as an la_dtype.
int dtype_code(const la_dtype &d) {
  int v;
  std::memcpy(&v, &d, sizeof v);
  return v;
}
bool valid_dtype(const la_dtype &d) {
  const int v = dtype_code(d);
  return v == LA_F32 || v == LA_BF16;
}
#define LA_CHECK_DTYPE(d)                                                                  \
  do {                                                                                     \
    if (!valid_dtype(d)) return fail(LA_ERR_UNSUPPORTED, "unknown dtype %d", dtype_code(d)); \
  } while (0)

// A buffer argument of a call: its byte range and its name for the error message.
struct Buf {
  const void *p;
  size_t n;
  const char *name;
};

// Every buffer a call writes must be disjoint from every other buffer of the call, read or
// written (a kernel that writes one while another workgroup still reads or writes it would
// give wrong results with no error); buffers that are only read may share memory.
la_status check_disjoint(std::initializer_list<Buf> written, std::initializer_list<Buf> read) {
  for (const Buf *w = written.begin(); w != written.end(); ++w) {
    for (const Buf *w2 = w + 1; w2 != written.end(); ++w2)
      if (overlaps(w->p, w->n, w2->p, w2->n))
        return fail(LA_ERR_INVALID_ARG, "%s overlaps %s", w->name, w2->name);
    for (const Buf &r : read)
      if (overlaps(w->p, w->n, r.p, r.n))
        return fail(LA_ERR_INVALID_ARG, "%s overlaps %s", w->name, r.name);
  }
  return LA_OK;
}

// Byte sizes of the argument kinds.
size_t act_bytes(int64_t n, int32_t H, int32_t D, la_dtype dtype) {
  return (size_t)n * H * D * elem_bytes(dtype);
}
size_t state_bytes(int64_t n, int32_t H, int32_t D) { return (size_t)n * H * D * D * sizeof(float); }
size_t cu_bytes(const int32_t *cu, int32_t S) { return cu ? (size_t)(S + 1) * sizeof(int32_t) : 0; }

// The prefill's buffers (plus the split workspace, when given): out and final_state are written.
la_status check_prefill_buffers(const void *q, const void *k, const void *v, const float *decay,
                                const int32_t *cu, const float *init, const void *out,
                                const float *fs, const void *ws, size_t ws_bytes, int64_t T,
                                int32_t S, int32_t H, int32_t D, la_dtype dtype) {
  const size_t act = act_bytes(T, H, D, dtype), st = state_bytes(S, H, D);
  return check_disjoint({{out, act, "out"}, {fs, st, "final_state"}, {ws, ws_bytes, "workspace"}},
                        {{q, act, "q"}, {k, act, "k"}, {v, act, "v"},
                         {decay, (size_t)H * sizeof(float), "decay"},
                         {cu, cu_bytes(cu, S), "cu_seqlens"}, {init, st, "initial_state"}});
}

// Default block size of the bf16 prefill from the environment variable LA_BLOCK (read once):
// 0 when unset, 64 or 128, -1 for any other value.  Meant for running a test suite at either
// block size without changing its calls.
int env_block() {
  static std::once_flag once;
  static int value = 0;
  std::call_once(once, [] {
    const char *e = std::getenv("LA_BLOCK");
    if (e == nullptr || *e == '\0') value = 0;
    else if (std::strcmp(e, "64") == 0) value = 64;
    else if (std::strcmp(e, "128") == 0) value = 128;
    else value = -1;
  });
  return value;
}

constexpr int kMaxDevices = 64;
// Size of the static scratch of la_prefill_split_static (per device).
constexpr size_t kScratchBytes = LA_SPLIT_STATIC_SCRATCH_BYTES;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];   // 1 = gfx950, 0 = other arch
int g_dev_cus[kMaxDevices];  // compute units

// Checks that the current device exists and is a gfx950; cached per device.  *cus (optional)
// receives its number of compute units.
la_status check_device(int *cus = nullptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(LA_ERR_HIP, "device index %d out of range", dev);
  hipError_t perr = hipSuccess;
  std::call_once(g_dev_once[dev], [&]() {
    hipDeviceProp_t prop;
    perr = hipGetDeviceProperties(&prop, dev);
    g_dev_ok[dev] = (perr == hipSuccess && std::strncmp(prop.gcnArchName, "gfx950", 6) == 0);
    g_dev_cus[dev] = perr == hipSuccess ? prop.multiProcessorCount : 0;
  });
  if (perr != hipSuccess)
    return fail(LA_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(perr));
  if (!g_dev_ok[dev]) return fail(LA_ERR_UNSUPPORTED, "device %d is not a gfx950", dev);
  if (cus) *cus = g_dev_cus[dev];
  return LA_OK;
}

la_status check_common(const void *q, const void *k, const void *v, const float *decay,
                       const void *out, int64_t ntok, int32_t H, int32_t D, la_dtype dtype) {
  if (D != 64 && D != 128) return fail(LA_ERR_UNSUPPORTED, "head dimension %d not in {64,128}", D);
  if (H < 1) return fail(LA_ERR_INVALID_ARG, "H = %d < 1", H);
  if (H > 65536) return fail(LA_ERR_INVALID_ARG, "H = %d > 65536", H);
  if (ntok < 0) return fail(LA_ERR_INVALID_ARG, "negative token count %lld", (long long)ntok);
  if (decay == nullptr) return fail(LA_ERR_INVALID_ARG, "decay is NULL");
  if (ntok > 0) {
    if (!q || !k || !v || !out) return fail(LA_ERR_INVALID_ARG, "q, k, v or out is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
      return fail(LA_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
    if (ntok > (int64_t(1) << 40) / ((int64_t)H * D))
      return fail(LA_ERR_INVALID_ARG, "tensor too large");
  }
  return LA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Largest number of segments valid cu_seqlens can produce: sum over sequences of
// ceil(n_s / L) <= ceil(T / L) + S - 1.
int64_t split_capacity(int64_t T, int32_t S, int64_t seg_len) {
  return T <= 0 ? 0 : (T + seg_len - 1) / seg_len + S - 1;
}

struct SplitLayout {
  int64_t cap;
  int32_t sub;  // state slots per segment slot
  size_t states, seg_cu, seq_seg0, seg_rfirst, bytes;  // byte offsets and total size
};

// Most segments per sequence for which the bf16 split forms incoming states in the segment
// prefill's prologue instead of a separate combine launch.
constexpr int64_t kFusedMaxSegments = 16;

// Whether the bf16 split runs as two launches (segment states found on the device, incoming
// states formed in the segment prefill's prologue): while each segment's 32-bit byte offsets
// hold and no sequence can have more than kFusedMaxSegments segments.
bool split_fused(int64_t T, int32_t H, int32_t D, int64_t seg_len) {
  return (seg_len + 64) * (int64_t)H * D * 2 < (int64_t(1) << 31) &&
         (T + seg_len - 1) / seg_len <= kFusedMaxSegments;
}

// Sub-segments per segment of the two-launch form's state pass.  Only the segments before the
// last of each sequence need a state; when they are too few to fill the device (one
// sequence cut in two: a workgroup per head and 32 columns), their states are computed in
// sub-segments of seg_len / sub tokens by sub times as many, shorter workgroups (the segment
// prefill adds sub states per earlier segment).  Doubled while the state pass stays within one
// round of workgroups on 256 compute units (one workgroup per CU at d = 128, two at d = 64: its
// LDS), sub-segments keep at least 2,048 tokens, and a segment's prologue adds at most 16
// states.  A function of the sizes only, so the workspace size needs no device.
int32_t split_sub(int64_t T, int32_t S, int32_t H, int32_t D, int64_t seg_len) {
  const int64_t segs = (T + seg_len - 1) / seg_len;  // segments of all sequences (at most)
  if (segs <= S) return 1;  // few sequences, if any, are cut: nothing to spread
  const int64_t need = segs - S;                      // segments before a sequence's last
  const int64_t wgs = need * H * (D / 32), round = D == 64 ? 512 : 256;
  int32_t sub = 1;
  while (sub < 8 && wgs * sub * 2 <= round && seg_len % (sub * 2) == 0 &&
         seg_len / (sub * 2) >= 2048 && (segs - 1) * sub * 2 <= 16)
    sub *= 2;
  return sub;
}

SplitLayout split_layout(int64_t T, int32_t S, int32_t H, int32_t D, int32_t seg_blocks,
                         int32_t sub = 1) {
  SplitLayout l;
  l.cap = split_capacity(T, S, (int64_t)seg_blocks * 64);
  l.sub = sub;
  l.states = 0;
  l.seg_cu = align256((size_t)l.cap * sub * H * D * D * sizeof(float));
  l.seq_seg0 = l.seg_cu + align256((size_t)(l.cap + 1) * sizeof(int32_t));
  l.seg_rfirst = l.seq_seg0 + align256((size_t)(S + 1) * sizeof(int32_t));
  l.bytes = l.seg_rfirst + align256((size_t)l.cap * sizeof(int32_t));
  return l;
}


// Piecewise-linear cost (microseconds) of one 64-token block step of a workgroup, as a function
// of how many workgroups run at once (first column).  bf16 has two tables: inputs that stay in
// the 256 MB last-level cache between passes, and inputs that stream from HBM.
struct CostPt { double w, us; };
constexpr CostPt kBf16D128Cached[] = {{1, 0.71}, {32, 0.70}, {128, 0.75}, {256, 0.87}};
constexpr CostPt kBf16D128Hbm[] = {{1, 0.71}, {32, 0.865}, {128, 0.92}, {256, 1.06}};
constexpr CostPt kBf16D64Cached[] = {{1, 0.51}, {16, 0.61}, {64, 0.63}, {128, 0.64}, {256, 0.66}};
constexpr CostPt kBf16D64Hbm[] = {{1, 0.51}, {16, 0.60}, {64, 0.87}, {128, 0.91}, {256, 0.97}};

double cost_at(const CostPt *t, int n, double w) {
  if (w <= t[0].w) return t[0].us;
  for (int i = 1; i < n; ++i)
    if (w <= t[i].w) return t[i - 1].us + (t[i].us - t[i - 1].us) * (w - t[i - 1].w) /
                                             (t[i].w - t[i - 1].w);
  return t[n - 1].us;
}
#define LA_COST_AT(table, w) cost_at(table, (int)(sizeof(table) / sizeof(table[0])), w)

// Block-step cost for `w` concurrent workgroups over `bytes` of q, k, v and out.  fp32 is bound
// by its matrix products and costs the same at any load; bf16 blends its cached and streaming
// tables as the working set grows from 256 MiB to 512 MiB.
double block_cost(la_dtype dtype, int32_t D, double w, double bytes) {
  if (dtype == LA_F32) return D == 64 ? 2.7 : 4.4;
  const double mib = 1024.0 * 1024.0;
  double f = (bytes - 256 * mib) / (256 * mib);
  f = f < 0 ? 0 : (f > 1 ? 1 : f);
  const double c = D == 64 ? LA_COST_AT(kBf16D64Cached, w) : LA_COST_AT(kBf16D128Cached, w);
  const double h = D == 64 ? LA_COST_AT(kBf16D64Hbm, w) : LA_COST_AT(kBf16D128Hbm, w);
  return (1 - f) * c + f * h;
}
}  // namespace

// Scratch of the allocation-free split prefill (la_prefill_split_static): the segment states and
// segment table that la_prefill_split keeps in the caller's workspace.  Every device the library
// runs on holds its own copy from module load until the process ends.  In host code the name is
// only a host-side stand-in; kernels get the device address from scratch_address().
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of the current device's scratch, looked up once per device with that device
// current.
la_status scratch_address(void **p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(LA_ERR_HIP, "device index %d out of range", dev);
  std::call_once(g_scratch_once[dev], [&]() {
    g_scratch_ptr[dev] = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr)
    return fail(LA_ERR_HIP, "hipGetSymbolAddress(scratch): %s",
                hipGetErrorString(g_scratch_err[dev]));
  *p = g_scratch_ptr[dev];
  return LA_OK;
}

// The split prefill behind la_prefill_split (the caller's workspace) and
// la_prefill_split_static (the library's static scratch, static_scratch = true: workspace and
// workspace_bytes are ignored).  The dtype has been checked.
la_status prefill_split_impl(const void *q, const void *k, const void *v, const float *decay,
                             const int32_t *cu_seqlens, const float *initial_state, void *out,
                             float *final_state, int64_t T, int32_t S, int32_t H, int32_t D,
                             la_dtype dtype, int32_t seg_blocks, void *workspace,
                             size_t workspace_bytes, bool static_scratch, void *stream) {
  la_status st = check_common(q, k, v, decay, out, T, H, D, dtype);
  if (st != LA_OK) return st;
  if (S < 1) return fail(LA_ERR_INVALID_ARG, "S = %d < 1", S);
  if (cu_seqlens == nullptr && S != 1)
    return fail(LA_ERR_INVALID_ARG, "cu_seqlens is NULL but S = %d (must be 1)", S);
  if (seg_blocks < 1) return fail(LA_ERR_INVALID_ARG, "seg_blocks = %d < 1", seg_blocks);
  st = check_prefill_buffers(q, k, v, decay, cu_seqlens, initial_state, out, final_state, nullptr,
                             0, T, S, H, D, dtype);
  if (st != LA_OK) return st;
  if (T > 0x7fffffffLL) return fail(LA_ERR_INVALID_ARG, "split prefill needs T < 2^31");
  if (T == 0)  // no segments: final states are the initial states (or zeros)
    return la_prefill_ex(q, k, v, decay, cu_seqlens, initial_state, out, final_state, T, S, H,
                         D, dtype, stream);
  const int64_t seg_len = (int64_t)seg_blocks * 64;
  const bool fused = dtype == LA_BF16 && split_fused(T, H, D, seg_len);
  SplitLayout lay =
      split_layout(T, S, H, D, seg_blocks, fused ? split_sub(T, S, H, D, seg_len) : 1);
  // the static scratch takes the sub-segment states only when they fit
  if (static_scratch && lay.bytes > kScratchBytes) lay = split_layout(T, S, H, D, seg_blocks, 1);
  if (lay.cap * lay.sub * H * (D / 32) > 0x7fffffffLL ||
      (long long)S * H * (D * D / 256) > 0x7fffffffLL)
    return fail(LA_ERR_INVALID_ARG, "too many segments");
  if (static_scratch) {
    if (lay.bytes > kScratchBytes)
      return fail(LA_ERR_INVALID_ARG,
                  "these sizes need %zu bytes of split workspace; the static scratch holds %zu "
                  "(use la_prefill_split with a caller workspace, or longer segments)",
                  lay.bytes, kScratchBytes);
    st = check_device();
    if (st != LA_OK) return st;
    st = scratch_address(&workspace);
    if (st != LA_OK) return st;
  } else {
    if (workspace == nullptr) return fail(LA_ERR_INVALID_ARG, "workspace is NULL");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(LA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (workspace_bytes < lay.bytes)
      return fail(LA_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes,
                  lay.bytes);
    st = check_prefill_buffers(q, k, v, decay, cu_seqlens, initial_state, out, final_state,
                               workspace, lay.bytes, T, S, H, D, dtype);
    if (st != LA_OK) return st;
    st = check_device();
    if (st != LA_OK) return st;
  }

  char *ws = static_cast<char *>(workspace);
  float *states = reinterpret_cast<float *>(ws + lay.states);
  int32_t *seg_cu = reinterpret_cast<int32_t *>(ws + lay.seg_cu);
  int32_t *seq_seg0 = reinterpret_cast<int32_t *>(ws + lay.seq_seg0);
  const int32_t cap = (int32_t)lay.cap;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto prefill = dtype == LA_BF16 ? la_launch_prefill_bf16 : la_launch_prefill_f32;

  // bf16, two launches: the segment states (each workgroup finds its segment in cu_seqlens),
  // then every segment from the incoming state its workgroup forms from the earlier segments'
  // states (no table, no combine launch; a segment's prologue reads every earlier segment's
  // states of its sequence).
  if (fused) {
    hipError_t e = la_launch_segment_states_fused_bf16(cu_seqlens, T, S, seg_len, lay.sub, cap,
                                                       k, v, decay, H, D, states, initial_state,
                                                       final_state, s);
    if (e != hipSuccess) return fail(LA_ERR_HIP, "segment state launch: %s", hipGetErrorString(e));
    LaPrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.decay = decay;
    a.cu_seqlens = cu_seqlens;
    a.initial_state = initial_state;
    a.out = out;
    a.final_state = final_state;
    a.T = T;
    a.S = S;
    a.H = H;
    a.D = D;
    // Long segments run the 128-token kernel (measured: 8,192-token segments 2.6% faster);
    // short ones the 64-token kernel (1,024-token segments: 5% faster than 128).
    e = seg_len % 128 == 0 && seg_len >= 4096
            ? la_launch_prefill_split_bf16_b128(a, seg_len, states, cap, lay.sub, s)
            : la_launch_prefill_split_bf16(a, seg_len, states, cap, lay.sub, s);
    if (e != hipSuccess)
      return fail(LA_ERR_HIP, "segment prefill launch: %s", hipGetErrorString(e));
    return LA_OK;
  }

  hipError_t e = la_launch_seg_table(cu_seqlens, T, S, (int64_t)seg_blocks * 64, cap, seg_cu,
                                     seq_seg0, nullptr, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "segment table launch: %s", hipGetErrorString(e));
  // Segment states from zero: only k and v are read.
  LaPrefillArgs a{};
  a.k = k;
  a.v = v;
  a.decay = decay;
  a.cu_seqlens = seg_cu;
  a.final_state = states;
  a.T = T;
  a.S = cap;
  a.H = H;
  a.D = D;
  a.state_only = true;
  e = dtype == LA_BF16 ? la_launch_segment_states_bf16(a, (int64_t)seg_blocks * 64, s) : prefill(a, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "segment state launch: %s", hipGetErrorString(e));
  e = la_launch_combine(decay, seg_cu, seq_seg0, S, H, D, initial_state, states, final_state,
                        false, false, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "combine launch: %s", hipGetErrorString(e));
  // Every segment from its incoming state.
  a.q = q;
  a.out = out;
  a.initial_state = states;
  a.final_state = nullptr;
  a.state_only = false;
  e = prefill(a, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "segment prefill launch: %s", hipGetErrorString(e));
  return LA_OK;
}

}  // namespace

extern "C" {

int32_t la_abi_version(void) { return LA_ABI_VERSION; }

const char *la_status_str(la_status s) {
  // Callers may pass any int; reading a value outside the enumerators through the enum type is
  // undefined in C++, so the argument's bytes are read as an int.
  int v;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case LA_OK: return "LA_OK";
    case LA_ERR_INVALID_ARG: return "LA_ERR_INVALID_ARG";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
    case LA_ERR_HIP: return "LA_ERR_HIP";
  }
  return "LA_ERR_UNKNOWN";
}

const char *la_last_error(void) { return g_err; }

la_status la_prefill_with_block_size(const void *q, const void *k, const void *v,
                                     const float *decay, const int32_t *cu_seqlens,
                                     const float *initial_state, void *out, float *final_state,
                                     int64_t T, int32_t S, int32_t H, int32_t D, la_dtype dtype,
                                     int32_t block_size, void *stream) {
  g_err[0] = '\0';
  LA_CHECK_DTYPE(dtype);
  if (block_size == 0 && dtype == LA_BF16) {
    block_size = env_block();
    if (block_size < 0) return fail(LA_ERR_INVALID_ARG, "LA_BLOCK must be 64 or 128");
    // 128-token blocks measured as fast or faster than 64 on every MI355X shape timed
    // (65,536 tokens: 0.9% at 64 heads, 6-11% at 8-32 heads and at d = 64)
    if (block_size == 0) block_size = 128;
  }
  if (block_size == 0) block_size = 64;
  if (block_size != 64 && block_size != 128)
    return fail(LA_ERR_INVALID_ARG, "block_size = %d not in {0, 64, 128}", block_size);
  if (block_size == 128 && dtype != LA_BF16)
    return fail(LA_ERR_UNSUPPORTED, "128-token blocks are built for bf16 storage only");
  la_status st = check_common(q, k, v, decay, out, T, H, D, dtype);
  if (st != LA_OK) return st;
  if (S < 1) return fail(LA_ERR_INVALID_ARG, "S = %d < 1", S);
  if (cu_seqlens == nullptr && S != 1)
    return fail(LA_ERR_INVALID_ARG, "cu_seqlens is NULL but S = %d (must be 1)", S);
  if ((long long)S * H * (D / 32) > 0x7fffffffLL) return fail(LA_ERR_INVALID_ARG, "S*H too large");
  st = check_prefill_buffers(q, k, v, decay, cu_seqlens, initial_state, out, final_state, nullptr,
                             0, T, S, H, D, dtype);
  if (st != LA_OK) return st;
  if (final_state == nullptr && (T == 0)) return LA_OK;  // nothing to compute or write
  st = check_device();
  if (st != LA_OK) return st;

  LaPrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.decay = decay;
  a.cu_seqlens = cu_seqlens;
  a.initial_state = initial_state;
  a.out = out;
  a.final_state = final_state;
  a.T = T;
  a.S = S;
  a.H = H;
  a.D = D;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = dtype == LA_F32        ? la_launch_prefill_f32(a, s)
                 : block_size == 128 ? la_launch_prefill_bf16_b128(a, s)
                                     : la_launch_prefill_bf16(a, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "prefill launch: %s", hipGetErrorString(e));
  return LA_OK;
}

la_status la_prefill_ex(const void *q, const void *k, const void *v, const float *decay,
                        const int32_t *cu_seqlens, const float *initial_state, void *out,
                        float *final_state, int64_t T, int32_t S, int32_t H, int32_t D,
                        la_dtype dtype, void *stream) {
  g_err[0] = '\0';
  LA_CHECK_DTYPE(dtype);
  return la_prefill_with_block_size(q, k, v, decay, cu_seqlens, initial_state, out, final_state,
                                    T, S, H, D, dtype, 0, stream);
}

la_status la_prefill(const void *q, const void *k, const void *v, const float *decay,
                     const int32_t *cu_seqlens, void *out, float *final_state, int64_t T,
                     int32_t S, int32_t H, int32_t D, la_dtype dtype, void *stream) {
  g_err[0] = '\0';
  LA_CHECK_DTYPE(dtype);
  return la_prefill_ex(q, k, v, decay, cu_seqlens, nullptr, out, final_state, T, S, H, D, dtype,
                       stream);
}

size_t la_prefill_split_workspace_size(int64_t T, int32_t S, int32_t H, int32_t D,
                                       int32_t seg_blocks) {
  if (T < 0 || S < 1 || H < 1 || (D != 64 && D != 128) || seg_blocks < 1) return 0;
  const int64_t seg_len = (int64_t)seg_blocks * 64;
  // the larger of the two forms: the bf16 two-launch one may keep sub-segment states
  const int32_t sub = T > 0 && split_fused(T, H, D, seg_len) ? split_sub(T, S, H, D, seg_len) : 1;
  return split_layout(T, S, H, D, seg_blocks, sub).bytes;
}

int32_t la_prefill_split_blocks_for(int64_t T, int32_t S, int32_t H, int32_t D, la_dtype dtype,
                                    int32_t compute_units) {
  if (!valid_dtype(dtype)) return 0;
  if (T <= 0 || S < 1 || H < 1 || (D != 64 && D != 128) || compute_units < 1) return 0;
  const int64_t slices = D / 32;
  if ((int64_t)S * H * slices >= compute_units) return 0;  // the plain launch fills the device
  const int64_t blocks = (T + 63) / 64;
  int64_t seg = (blocks * H * slices + compute_units - 1) / compute_units;  // ~1 WG per CU
  if (seg < 4) seg = 4;                               // keep segments a few blocks long
  if (seg >= blocks || seg > 0x7fffffff) return 0;    // no sequence would be cut
  // Cost model in microseconds, fitted to MI355X timings of both paths over T = 512 .. 65,536,
  // H = 1 .. 64, both head sizes and both dtypes.  The plain scan is ~6 us of launch plus one
  // block step per block of a sequence (the mean length T / S stands in for the longest) with
  // S * H * slices workgroups in flight.  The split is ~17 us of launches, the segment pass (one
  // block step per block of a segment, the device full), the segment-state pass (0.55 of that
  // for bf16, whose state pass runs token-parallel; 0.75 for fp32) and ~0.5 us per segment of a
  // sequence in the serial combine.  Split only when it saves at least 5%.
  const double bytes = (double)T * H * D * elem_bytes(dtype) * 4.0;
  const int64_t nb = (blocks + S - 1) / S;                // blocks of a (mean) sequence
  const double w_plain = (double)S * H * slices;
  double w_split = (double)((blocks + seg - 1) / seg + S - 1) * H * slices;  // all segments
  if (w_split > compute_units) w_split = compute_units;
  const double plain = 6.0 + (double)nb * block_cost(dtype, D, w_plain, bytes);
  double so = dtype == LA_F32 ? 0.75 : 0.55;
  const int64_t count = (nb + seg - 1) / seg;  // segments of a (mean) sequence
  // The two-launch bf16 form computes no state for the last segment of a sequence; its state
  // pass then runs fewer workgroups (measured: two segments per sequence save about a quarter
  // of the pass, eight about 6%).
  if (dtype == LA_BF16 && split_fused(T, H, D, seg * 64))
    so *= ((double)count - 0.5) / (double)count;
  const double split = 17.0 + (double)seg * block_cost(dtype, D, w_split, bytes) * (1.0 + so) +
                       0.5 * (double)count;
  if (split >= 0.95 * plain) return 0;
  return (int32_t)seg;
}

int32_t la_prefill_split_blocks(int64_t T, int32_t S, int32_t H, int32_t D, la_dtype dtype) {
  if (!valid_dtype(dtype)) return 0;
  int cus = 0;
  if (check_device(&cus) != LA_OK || cus <= 0) return 0;
  return la_prefill_split_blocks_for(T, S, H, D, dtype, cus);
}

la_status la_prefill_split(const void *q, const void *k, const void *v, const float *decay,
                           const int32_t *cu_seqlens, const float *initial_state, void *out,
                           float *final_state, int64_t T, int32_t S, int32_t H, int32_t D,
                           la_dtype dtype, int32_t seg_blocks, void *workspace,
                           size_t workspace_bytes, void *stream) {
  g_err[0] = '\0';
  LA_CHECK_DTYPE(dtype);
  return prefill_split_impl(q, k, v, decay, cu_seqlens, initial_state, out, final_state, T, S, H,
                            D, dtype, seg_blocks, workspace, workspace_bytes, false, stream);
}

la_status la_prefill_split_static(const void *q, const void *k, const void *v,
                                  const float *decay, const int32_t *cu_seqlens,
                                  const float *initial_state, void *out, float *final_state,
                                  int64_t T, int32_t S, int32_t H, int32_t D, la_dtype dtype,
                                  int32_t seg_blocks, void *stream) {
  g_err[0] = '\0';
  LA_CHECK_DTYPE(dtype);
  return prefill_split_impl(q, k, v, decay, cu_seqlens, initial_state, out, final_state, T, S, H,
                            D, dtype, seg_blocks, nullptr, 0, true, stream);
}

}  // extern "C"

namespace {
// Argument checks shared by the backward entry points (no device access).
la_status check_backward(const void *q, const void *k, const void *v, const float *decay,
                         const int32_t *cu_seqlens, const float *initial_state,
                         const void *d_out, const float *d_final_state, const void *dq,
                         const void *dk, const void *dv, const float *d_initial_state,
                         const void *ws, size_t ws_bytes, int64_t T, int32_t S, int32_t H,
                         int32_t D, la_dtype dtype) {
  la_status st = check_common(q, k, v, decay, d_out, T, H, D, dtype);
  if (st != LA_OK) return st;
  if (T > 0) {
    if (!dq || !dk || !dv) return fail(LA_ERR_INVALID_ARG, "dq, dk or dv is NULL");
    if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv))
      return fail(LA_ERR_INVALID_ARG, "dq, dk and dv must be 16-byte aligned");
  }
  if (S < 1) return fail(LA_ERR_INVALID_ARG, "S = %d < 1", S);
  if (cu_seqlens == nullptr && S != 1)
    return fail(LA_ERR_INVALID_ARG, "cu_seqlens is NULL but S = %d (must be 1)", S);
  if ((long long)S * H * (D / 32) > 0x7fffffffLL) return fail(LA_ERR_INVALID_ARG, "S*H too large");
  const size_t act = act_bytes(T, H, D, dtype), stb = state_bytes(S, H, D);
  return check_disjoint({{dq, act, "dq"}, {dk, act, "dk"}, {dv, act, "dv"},
                         {d_initial_state, stb, "d_initial_state"}, {ws, ws_bytes, "workspace"}},
                        {{q, act, "q"}, {k, act, "k"}, {v, act, "v"}, {d_out, act, "d_out"},
                         {decay, (size_t)H * sizeof(float), "decay"},
                         {cu_seqlens, cu_bytes(cu_seqlens, S), "cu_seqlens"},
                         {initial_state, stb, "initial_state"},
                         {d_final_state, stb, "d_final_state"}});
}
}  // namespace

extern "C" {

la_status la_backward(const void *q, const void *k, const void *v, const float *decay,
                      const int32_t *cu_seqlens, const float *initial_state, const void *d_out,
                      const float *d_final_state, void *dq, void *dk, void *dv,
                      float *d_initial_state, int64_t T, int32_t S, int32_t H, int32_t D,
                      la_dtype dtype, void *stream) {
  g_err[0] = '\0';
  LA_CHECK_DTYPE(dtype);
  la_status st = check_backward(q, k, v, decay, cu_seqlens, initial_state, d_out, d_final_state,
                                dq, dk, dv, d_initial_state, nullptr, 0, T, S, H, D, dtype);
  if (st != LA_OK) return st;
  if (T == 0 && d_initial_state == nullptr) return LA_OK;
  // bf16: the three scans use the prefill's default block size (128, or LA_BLOCK)
  const int block = dtype == LA_BF16 ? env_block() : 64;
  if (block < 0) return fail(LA_ERR_INVALID_ARG, "LA_BLOCK must be 64 or 128");
  st = check_device();
  if (st != LA_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto scan = dtype == LA_F32 ? la_launch_prefill_f32
              : block == 64   ? la_launch_prefill_bf16
                              : la_launch_prefill_bf16_b128;

  LaPrefillArgs a{};
  a.decay = decay;
  a.cu_seqlens = cu_seqlens;
  a.T = T;
  a.S = S;
  a.H = H;
  a.D = D;
  hipError_t e;
  if (T > 0) {
    // dq_t = sum_{s<=t} lambda^(t-s) (do_t . v_s) k_s + lambda^(t+1) S0 do_t: the forward scan
    // with (query, key, value) = (do, v, k) and the initial state transposed.
    a.q = d_out;
    a.k = v;
    a.v = k;
    a.initial_state = initial_state;
    a.init_transposed = true;
    a.out = dq;
    e = scan(a, s);
    if (e != hipSuccess) return fail(LA_ERR_HIP, "dq launch: %s", hipGetErrorString(e));
    // dk_s = sum_{t>=s} lambda^(t-s) (v_s . do_t) q_t + lambda^(n-1-s) dSn v_s: the reversed
    // scan with (v, do, q), dSn transposed as an initial state weighted lambda^t.
    a.q = v;
    a.k = d_out;
    a.v = q;
    a.initial_state = d_final_state;
    a.reverse = true;
    a.init_inclusive = true;
    a.out = dk;
    e = scan(a, s);
    if (e != hipSuccess) return fail(LA_ERR_HIP, "dk launch: %s", hipGetErrorString(e));
  }
  // dv_s = sum_{t>=s} lambda^(t-s) (k_s . q_t) do_t + lambda^(n-1-s) dSn^T k_s: the reversed
  // scan with (k, q, do) and dSn as is; its final state times lambda is
  // dS0 = sum_t lambda^(t+1) q_t^T do_t + lambda^n dSn (dSn itself for an empty sequence).
  a.q = k;
  a.k = q;
  a.v = d_out;
  a.initial_state = d_final_state;
  a.reverse = true;
  a.init_inclusive = true;
  a.init_transposed = false;
  a.out = dv;
  a.final_state = d_initial_state;
  e = scan(a, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "dv launch: %s", hipGetErrorString(e));
  return LA_OK;
}

la_status la_backward_split(const void *q, const void *k, const void *v, const float *decay,
                            const int32_t *cu_seqlens, const float *initial_state,
                            const void *d_out, const float *d_final_state, void *dq, void *dk,
                            void *dv, float *d_initial_state, int64_t T, int32_t S, int32_t H,
                            int32_t D, la_dtype dtype, int32_t seg_blocks, void *workspace,
                            size_t workspace_bytes, void *stream) {
  g_err[0] = '\0';
  LA_CHECK_DTYPE(dtype);
  la_status st = check_backward(q, k, v, decay, cu_seqlens, initial_state, d_out, d_final_state,
                                dq, dk, dv, d_initial_state, nullptr, 0, T, S, H, D, dtype);
  if (st != LA_OK) return st;
  if (seg_blocks < 1) return fail(LA_ERR_INVALID_ARG, "seg_blocks = %d < 1", seg_blocks);
  if (T > 0x7fffffffLL) return fail(LA_ERR_INVALID_ARG, "split backward needs T < 2^31");
  if (T == 0)  // no segments
    return la_backward(q, k, v, decay, cu_seqlens, initial_state, d_out, d_final_state, dq, dk,
                       dv, d_initial_state, T, S, H, D, dtype, stream);
  const SplitLayout lay = split_layout(T, S, H, D, seg_blocks);
  if (lay.cap * H * (D / 32) > 0x7fffffffLL || (long long)S * H * (D * D / 256) > 0x7fffffffLL)
    return fail(LA_ERR_INVALID_ARG, "too many segments");
  if (workspace == nullptr) return fail(LA_ERR_INVALID_ARG, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(LA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < lay.bytes)
    return fail(LA_ERR_INVALID_ARG, "workspace of %zu bytes, %zu needed", workspace_bytes,
                lay.bytes);
  st = check_backward(q, k, v, decay, cu_seqlens, initial_state, d_out, d_final_state, dq, dk, dv,
                      d_initial_state, workspace, lay.bytes, T, S, H, D, dtype);
  if (st != LA_OK) return st;
  st = check_device();
  if (st != LA_OK) return st;

  char *ws = static_cast<char *>(workspace);
  float *states = reinterpret_cast<float *>(ws + lay.states);
  int32_t *seg_cu = reinterpret_cast<int32_t *>(ws + lay.seg_cu);
  int32_t *seq_seg0 = reinterpret_cast<int32_t *>(ws + lay.seq_seg0);
  int32_t *seg_rfirst = reinterpret_cast<int32_t *>(ws + lay.seg_rfirst);
  const int32_t cap = (int32_t)lay.cap;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto scan = dtype == LA_BF16 ? la_launch_prefill_bf16 : la_launch_prefill_f32;
  // The segment scans of long segments (>= 4,096 tokens, whole 128-token blocks) use the
  // 128-token kernel, as the split prefill does; the state-only passes stay as they are.
  const int64_t seg_len = (int64_t)seg_blocks * 64;
  auto seg_scan = dtype == LA_BF16 && seg_len % 128 == 0 && seg_len >= 4096
                      ? la_launch_prefill_bf16_b128
                      : scan;

  hipError_t e = la_launch_seg_table(cu_seqlens, T, S, (int64_t)seg_blocks * 64, cap, seg_cu,
                                     seq_seg0, seg_rfirst, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "segment table launch: %s", hipGetErrorString(e));

  // dq: the forward scan (query, key, value) = (do, v, k) from S0^T, split like the prefill.
  LaPrefillArgs a{};
  a.k = v;
  a.v = k;
  a.decay = decay;
  a.cu_seqlens = seg_cu;
  a.final_state = states;
  a.T = T;
  a.S = cap;
  a.H = H;
  a.D = D;
  a.state_only = true;
  e = dtype == LA_BF16 ? la_launch_segment_states_bf16(a, (int64_t)seg_blocks * 64, s) : scan(a, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "dq segment states: %s", hipGetErrorString(e));
  e = la_launch_combine(decay, seg_cu, seq_seg0, S, H, D, initial_state, states, nullptr, true,
                        false, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "dq combine: %s", hipGetErrorString(e));
  a.q = d_out;
  a.out = dq;
  a.initial_state = states;
  a.final_state = nullptr;
  a.state_only = false;
  e = seg_scan(a, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "dq segments: %s", hipGetErrorString(e));

  // dv and dk: reversed scans (k, q, do) and (v, do, q) whose states are transposes of each
  // other, so one set of segment states serves both: states of (key, value) = (q, do) from
  // zero, combined from dSn in reversed segment order (dSn inclusive), which also gives dS0.
  LaPrefillArgs b{};
  b.k = q;
  b.v = d_out;
  b.decay = decay;
  b.cu_seqlens = seg_cu;
  b.final_state = states;
  b.T = T;
  b.S = cap;
  b.H = H;
  b.D = D;
  b.reverse = true;
  b.state_only = true;
  e = dtype == LA_BF16 ? la_launch_segment_states_bf16(b, (int64_t)seg_blocks * 64, s) : scan(b, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "dv/dk segment states: %s", hipGetErrorString(e));
  e = la_launch_combine(decay, seg_cu, seq_seg0, S, H, D, d_final_state, states, d_initial_state,
                        false, true, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "dv/dk combine: %s", hipGetErrorString(e));
  // Each segment from its incoming state; the last segment of a sequence (met first by the
  // reversed scan) starts from dSn, which counts as inclusive.
  b.q = k;
  b.k = q;
  b.v = d_out;
  b.out = dv;
  b.initial_state = states;
  b.final_state = nullptr;
  b.state_only = false;
  b.init_inclusive = true;
  b.seq_incl = seg_rfirst;
  e = seg_scan(b, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "dv segments: %s", hipGetErrorString(e));
  b.q = v;
  b.k = d_out;
  b.v = q;
  b.out = dk;
  b.init_transposed = true;
  e = seg_scan(b, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "dk segments: %s", hipGetErrorString(e));
  return LA_OK;
}

la_status la_decode_step(const void *q, const void *k, const void *v, const float *decay,
                         float *state, void *out, int32_t Bt, int32_t H, int32_t D,
                         la_dtype dtype, void *stream) {
  g_err[0] = '\0';
  LA_CHECK_DTYPE(dtype);
  la_status st = check_common(q, k, v, decay, out, Bt, H, D, dtype);
  if (st != LA_OK) return st;
  if (Bt == 0) return LA_OK;
  if (state == nullptr) return fail(LA_ERR_INVALID_ARG, "state is NULL");
  if (!aligned16(state)) return fail(LA_ERR_INVALID_ARG, "state must be 16-byte aligned");
  if ((long long)Bt * H > 0x7fffffffLL) return fail(LA_ERR_INVALID_ARG, "Bt*H too large");
  {
    const size_t act = act_bytes(Bt, H, D, dtype);
    st = check_disjoint({{state, state_bytes(Bt, H, D), "state"}, {out, act, "out"}},
                        {{q, act, "q"}, {k, act, "k"}, {v, act, "v"},
                         {decay, (size_t)H * sizeof(float), "decay"}});
    if (st != LA_OK) return st;
  }
  st = check_device();
  if (st != LA_OK) return st;
  LaDecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.decay = decay;
  a.state = state;
  a.out = out;
  a.Bt = Bt;
  a.H = H;
  a.D = D;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = dtype == LA_BF16 ? la_launch_decode_bf16(a, s) : la_launch_decode_f32(a, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return LA_OK;
}

la_status la_decode_tokens(const void *q, const void *k, const void *v, const float *decay,
                           float *state, void *out, int32_t Bt, int32_t m, int32_t H, int32_t D,
                           la_dtype dtype, void *stream) {
  g_err[0] = '\0';
  LA_CHECK_DTYPE(dtype);
  if (m < 1) return fail(LA_ERR_INVALID_ARG, "m = %d < 1 tokens per sequence", m);
  if (Bt < 0) return fail(LA_ERR_INVALID_ARG, "negative batch %d", Bt);
  la_status st = check_common(q, k, v, decay, out, (int64_t)Bt * m, H, D, dtype);
  if (st != LA_OK) return st;
  if (Bt == 0) return LA_OK;
  if (state == nullptr) return fail(LA_ERR_INVALID_ARG, "state is NULL");
  if (!aligned16(state)) return fail(LA_ERR_INVALID_ARG, "state must be 16-byte aligned");
  if ((long long)Bt * H > 0x7fffffffLL) return fail(LA_ERR_INVALID_ARG, "Bt*H too large");
  {
    const size_t act = act_bytes((int64_t)Bt * m, H, D, dtype);
    st = check_disjoint({{state, state_bytes(Bt, H, D), "state"}, {out, act, "out"}},
                        {{q, act, "q"}, {k, act, "k"}, {v, act, "v"},
                         {decay, (size_t)H * sizeof(float), "decay"}});
    if (st != LA_OK) return st;
  }
  st = check_device();
  if (st != LA_OK) return st;
  LaDecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.decay = decay;
  a.state = state;
  a.out = out;
  a.Bt = Bt;
  a.H = H;
  a.D = D;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = dtype == LA_BF16 ? la_launch_decode_multi_bf16(a, m, s)
                                  : la_launch_decode_multi_f32(a, m, s);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return LA_OK;
}

}  // extern "C"
