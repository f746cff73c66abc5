// C ABI of the Wan attention library: argument checks, dispatch, scratch memory.
// The contract of every entry point is documented in include/wan_attn.h.

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "wan_attn.h"
#include "wan_attn_internal.h"

namespace {

bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("WAN_ATTN_LOG");
    return e != nullptr && e[0] == '1';
  }();
  return on;
}

#define WAN_LOG(...)                          \
  do {                                        \
    if (log_enabled()) {                      \
      std::fprintf(stderr, "[wan_attn] " __VA_ARGS__); \
      std::fputc('\n', stderr);               \
    }                                         \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// Shape checks shared by every entry point.  Sizes must be positive, the head dimension 128, and
// every index the kernels form must fit their 32-bit counters (tokens, tiles) and 64-bit offsets.
int check_shape(int64_t batch, int64_t heads, int64_t s_q, int64_t s_kv, int64_t head_dim) {
  if (batch < 1 || heads < 1 || s_q < 1 || s_kv < 1 || head_dim < 1) return WAN_ATTN_EINVAL;
  if (head_dim != wan::kHeadDim) return WAN_ATTN_EUNSUPPORTED;
  const int64_t kMax32 = 0x7fffffffLL;
  if (batch > kMax32 || heads > 65536 || s_q > kMax32 - 256 || s_kv > kMax32 - 256)
    return WAN_ATTN_EINVAL;   // heads: 64 token rows of one tile stay within a 32-bit byte offset
  // workgroup count (256-row query tiles) must fit in int; element counts in 2^60
  const long double tiles = (long double)wan::ceil_div(s_q, 64) * (long double)batch * heads;
  if (tiles > (long double)kMax32 - 8) return WAN_ATTN_EINVAL;
  const long double elems = (long double)batch * heads * (long double)(s_q > s_kv ? s_q : s_kv) * head_dim;
  if (elems > (long double)(1LL << 60)) return WAN_ATTN_EINVAL;
  return WAN_ATTN_OK;
}

// The first n_out buffers are outputs: none may overlap another output or any input.
bool outputs_overlap(const void* const* ptrs, const int64_t* bytes, int n_out, int n) {
  for (int a = 0; a < n_out; ++a)
    for (int b = 0; b < n; ++b)
      if (b != a && overlaps(ptrs[a], bytes[a], ptrs[b], bytes[b])) return true;
  return false;
}

// The 8-bit kernel addresses a head's pre-transposed V codes (128 rows of s_kv_pad bytes) through
// one buffer descriptor with a 32-bit byte range: 128 * s_kv_pad must stay below 2^31.
int check_attn8_size(int64_t s_kv) {
  const int64_t s_pad = wan::ceil_div(s_kv, wan::kQuantBlock) * wan::kQuantBlock;
  return (int64_t)wan::kHeadDim * s_pad >= (1LL << 31) ? WAN_ATTN_EUNSUPPORTED : WAN_ATTN_OK;
}

int check_qkvo(const void* q, const void* k, const void* v, const void* o, int64_t batch,
               int64_t heads, int64_t s_q, int64_t s_kv) {
  if (!q || !k || !v || !o) return WAN_ATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return WAN_ATTN_EALIGN;
  const int64_t qb = batch * s_q * heads * wan::kHeadDim * 2;
  const int64_t kb = batch * s_kv * heads * wan::kHeadDim * 2;
  if (overlaps(o, qb, q, qb) || overlaps(o, qb, k, kb) || overlaps(o, qb, v, kb)) return WAN_ATTN_EINVAL;
  return WAN_ATTN_OK;
}

int from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return WAN_ATTN_OK;
  WAN_LOG("%s failed: %s", what, hipGetErrorString(e));
  return e == hipErrorOutOfMemory ? WAN_ATTN_ENOMEM : WAN_ATTN_ELAUNCH;
}

// Per-device stream-ordered pool for the 8-bit path's scratch; memory freed on a stream returns
// to the pool and is reused by later calls instead of going back to the driver.
std::mutex g_pool_mu;
hipMemPool_t g_pools[64] = {};

int pool_for_current_device(hipMemPool_t* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return WAN_ATTN_ELAUNCH;
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if (!g_pools[dev]) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool;
    if (hipMemPoolCreate(&pool, &props) != hipSuccess) return WAN_ATTN_ELAUNCH;
    uint64_t keep = UINT64_MAX;
    (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    g_pools[dev] = pool;
  }
  *out = g_pools[dev];
  return WAN_ATTN_OK;
}

struct Attn8Layout {
  size_t q_codes, k_codes, q_scale, k_scale, v_codes, v_scale, smooth, chan_max, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Test hook: with WAN_ATTN_TEST_FAIL_ALLOC=1 in the environment when the library first allocates
// scratch, every scratch allocation of the process fails (WAN_ATTN_ENOMEM), so that callers can test
// their handling of it.  Read once, like WAN_ATTN_LOG.
bool fail_alloc_hook() {
  static const bool on = [] {
    const char* e = std::getenv("WAN_ATTN_TEST_FAIL_ALLOC");
    return e != nullptr && e[0] == '1';
  }();
  return on;
}

// Stream-ordered scratch from the device's pool (nullptr on failure).
void* scratch_alloc(size_t bytes, hipStream_t st, int* rc) {
  hipMemPool_t pool;
  *rc = pool_for_current_device(&pool);
  if (*rc) return nullptr;
  if (fail_alloc_hook()) {
    *rc = WAN_ATTN_ENOMEM;
    return nullptr;
  }
  void* ws = nullptr;
  hipError_t e = hipMallocFromPoolAsync(&ws, bytes, pool, st);
  if (e != hipSuccess || ws == nullptr) {
    WAN_LOG("scratch allocation of %zu bytes failed", bytes);
    *rc = WAN_ATTN_ENOMEM;
    return nullptr;
  }
  return ws;
}

// bf16 forward (lse optional).  Too few query tiles to fill the GPU: key ranges in parallel,
// partial results in stream-ordered scratch, combined into o, scratch released on the stream.
int fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, const wan::AttnShape& sh,
             hipStream_t st) {
  const int split = wan::attn_bf16_split(sh);
  if (split == 1) return from_hip(wan::launch_attn_bf16(q, k, v, o, lse, sh, st), "bf16 attention launch");
  int rc = WAN_ATTN_OK;
  void* ws = scratch_alloc(wan::attn_bf16_split_bytes(sh, split), st, &rc);
  if (!ws) return rc;
  rc = from_hip(wan::launch_attn_bf16_split(q, k, v, o, lse, sh, split, ws, st), "bf16 split attention launch");
  hipError_t fe = hipFreeAsync(ws, st);
  if (!rc && fe != hipSuccess) rc = from_hip(fe, "scratch release");
  return rc;
}

Attn8Layout attn8_layout(int64_t b, int64_t H, int64_t s_q, int64_t s_kv) {
  Attn8Layout L;
  const size_t nbq = (size_t)wan::ceil_div(s_q, wan::kQuantBlock);
  const size_t nbk = (size_t)wan::ceil_div(s_kv, wan::kQuantBlock);
  const size_t skv_pad = nbk * wan::kQuantBlock;
  size_t off = 0;
  L.q_codes = off; off = align256(off + (size_t)b * s_q * H * wan::kHeadDim);
  L.k_codes = off; off = align256(off + (size_t)b * s_kv * H * wan::kHeadDim);
  L.v_codes = off; off = align256(off + (size_t)b * H * wan::kHeadDim * skv_pad);
  L.q_scale = off; off = align256(off + (size_t)b * H * nbq * 4);
  L.k_scale = off; off = align256(off + (size_t)b * H * nbk * 4);
  L.v_scale = off; off = align256(off + (size_t)b * H * wan::kHeadDim * 4);
  L.smooth = off;  off = align256(off + (size_t)b * H * wan::kHeadDim * 4);
  L.chan_max = off; off = align256(off + (size_t)b * H * 3 * wan::kHeadDim * 4);
  L.total = off;
  return L;
}

// FP8 GEMM sizes: rows >= 1; the reduced dimension a positive multiple of 64 (one MFMA step) of
// at most 2^20 (32-bit tile offsets; and the products stay exactly summable in float64 for the
// tests); the work-item count of the GEMM within 32 bits.
int check_fp8_dims(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 1) return WAN_ATTN_EINVAL;
  if (cols % 64 != 0 || cols > (1LL << 20)) return WAN_ATTN_EUNSUPPORTED;
  if (rows > (1LL << 40)) return WAN_ATTN_EINVAL;
  return WAN_ATTN_OK;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// VSA sizes: the key-block count within the selection sort's LDS, keep within [1, n_kb], and the
// coarse stage's one-dimensional grids (2 * batch * heads * blocks workgroups) within 31 bits.
int check_vsa(int64_t batch, int64_t heads, int64_t s_q, int64_t s_kv, int64_t keep) {
  const int64_t n_qb = wan::ceil_div(s_q, 64), n_kb = wan::ceil_div(s_kv, 64);
  if (n_kb > wan::vsa_max_key_blocks()) return WAN_ATTN_EUNSUPPORTED;
  if (keep < 1 || keep > n_kb) return WAN_ATTN_EINVAL;
  if ((long double)2 * batch * heads * (n_qb > n_kb ? n_qb : n_kb) > 2147483000.0L) return WAN_ATTN_EINVAL;
  return WAN_ATTN_OK;
}

// Argument checks of the backward entry points: sizes, null and alignment, and no output overlapping
// an input or another output.
int check_bwd(const void* q, const void* k, const void* v, const void* o, const void* d_o, const void* lse,
              const void* dq, const void* dk, const void* dv, int64_t batch, int64_t heads, int64_t s_q,
              int64_t s_kv, int64_t head_dim) {
  int rc = check_shape(batch, heads, s_q, s_kv, head_dim);
  if (rc) return rc;
  const void* ptrs[] = {dq, dk, dv, q, k, v, o, d_o, lse};
  for (const void* p : ptrs)
    if (!p) return WAN_ATTN_EINVAL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return WAN_ATTN_EALIGN;
  const int64_t qb = batch * s_q * heads * wan::kHeadDim * 2;
  const int64_t kb = batch * s_kv * heads * wan::kHeadDim * 2;
  const int64_t lb = batch * heads * s_q * 4;
  const int64_t bytes[] = {qb, kb, kb, qb, kb, kb, qb, qb, lb};
  if (outputs_overlap(ptrs, bytes, 3, 9)) return WAN_ATTN_EINVAL;
  return WAN_ATTN_OK;
}

// Scratch of wan_attn_bwd_noalloc, for callers that cannot allocate: the backward's per-row
// statistics (lse * log2(e) and D, 8 bytes per query row padded to 64) in a file-scope device array.
// Every GPU the library runs on holds its own copy until the process ends.  In host code the array's
// name is only a host-side stand-in: the kernels get the address that hipGetSymbolAddress returns for
// the current device, looked up once per device on that device's first call.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::mutex g_noalloc_mu;
void* g_noalloc_ptr[64] = {};

int noalloc_scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return WAN_ATTN_ELAUNCH;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      WAN_LOG("hipGetSymbolAddress of the no-allocation scratch failed: %s", hipGetErrorString(e));
      return WAN_ATTN_ELAUNCH;
    }
    g_noalloc_ptr[dev] = ptr;
  }
  *out = g_noalloc_ptr[dev];
  return WAN_ATTN_OK;
}

}  // namespace


extern "C" {

int wan_attn_version(void) { return WAN_ATTN_VERSION; }

int wan_attn_release_scratch(void) {
  std::lock_guard<std::mutex> lock(g_pool_mu);
  int rc = WAN_ATTN_OK;
  for (hipMemPool_t pool : g_pools)
    if (pool && hipMemPoolTrimTo(pool, 0) != hipSuccess) rc = WAN_ATTN_ELAUNCH;
  return rc;
}

const char* wan_attn_strerror(int code) {
  switch (code) {
    case WAN_ATTN_OK: return "success";
    case WAN_ATTN_EINVAL: return "invalid argument (null pointer, bad size, unknown dtype or overlapping output)";
    case WAN_ATTN_EALIGN: return "pointer not 16-byte aligned";
    case WAN_ATTN_ENOMEM: return "out of device memory for scratch";
    case WAN_ATTN_ELAUNCH: return "HIP runtime error while launching";
    case WAN_ATTN_EUNSUPPORTED: return "unsupported size (head_dim other than 128, or an FP8 GEMM or VSA size outside its limits)";
    default: return "unknown status code";
  }
}

size_t wan_attn8_quantize_scratch_bytes(int64_t batch, int64_t heads) {
  if (batch < 1 || heads < 1) return 0;
  return (size_t)batch * heads * 3 * wan::kHeadDim * sizeof(float);
}

int wan_attn8_quantize(const void* q, const void* k, const void* v, int64_t batch, int64_t heads,
                       int64_t s_q, int64_t s_kv, int64_t head_dim, void* q_codes, void* q_scale,
                       void* k_codes, void* k_scale, void* v_codes, void* v_scale, void* smooth,
                       void* scratch, void* stream) {
  int rc = check_shape(batch, heads, s_q, s_kv, head_dim);
  if (rc) return rc;
  if (!q || !k || !v || !q_codes || !q_scale || !k_codes || !k_scale || !v_codes || !v_scale ||
      !smooth || !scratch)
    return WAN_ATTN_EINVAL;
  const void* ptrs[] = {q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, smooth, scratch, q, k, v};
  for (const void* p : ptrs)
    if (!aligned16(p)) return WAN_ATTN_EALIGN;
  {
    const int64_t bh = batch * heads, d = wan::kHeadDim;
    const int64_t nbq = wan::ceil_div(s_q, wan::kQuantBlock), nbk = wan::ceil_div(s_kv, wan::kQuantBlock);
    const int64_t bytes[] = {bh * s_q * d, bh * nbq * 4, bh * s_kv * d, bh * nbk * 4, bh * d * nbk * wan::kQuantBlock,
                             bh * d * 4, bh * d * 4, (int64_t)wan_attn8_quantize_scratch_bytes(batch, heads),
                             bh * s_q * d * 2, bh * s_kv * d * 2, bh * s_kv * d * 2};
    if (outputs_overlap(ptrs, bytes, 8, 11)) return WAN_ATTN_EINVAL;
  }
  const wan::AttnShape sh{batch, heads, s_q, s_kv};
  WAN_LOG("quantize b=%lld H=%lld s_q=%lld s_kv=%lld", (long long)batch, (long long)heads,
          (long long)s_q, (long long)s_kv);
  return from_hip(wan::launch_attn8_quantize(
                      q, k, v, sh, static_cast<int8_t*>(q_codes), static_cast<float*>(q_scale),
                      static_cast<int8_t*>(k_codes), static_cast<float*>(k_scale),
                      static_cast<uint8_t*>(v_codes), static_cast<float*>(v_scale),
                      static_cast<float*>(smooth), static_cast<float*>(scratch),
                      static_cast<hipStream_t>(stream)),
                  "quantize launch");
}

int wan_attn8_fwd_quantized(const void* q_codes, const void* q_scale, const void* k_codes,
                            const void* k_scale, const void* v_codes, const void* v_scale, void* o,
                            int64_t batch, int64_t heads, int64_t s_q, int64_t s_kv,
                            int64_t head_dim, void* stream) {
  int rc = check_shape(batch, heads, s_q, s_kv, head_dim);
  if (rc) return rc;
  rc = check_attn8_size(s_kv);
  if (rc) return rc;
  if (!q_codes || !q_scale || !k_codes || !k_scale || !v_codes || !v_scale || !o) return WAN_ATTN_EINVAL;
  const void* ptrs[] = {o, q_codes, q_scale, k_codes, k_scale, v_codes, v_scale};
  for (const void* p : ptrs)
    if (!aligned16(p)) return WAN_ATTN_EALIGN;
  {
    const int64_t bh = batch * heads, d = wan::kHeadDim;
    const int64_t nbq = wan::ceil_div(s_q, wan::kQuantBlock), nbk = wan::ceil_div(s_kv, wan::kQuantBlock);
    const int64_t bytes[] = {bh * s_q * d * 2, bh * s_q * d, bh * nbq * 4, bh * s_kv * d, bh * nbk * 4,
                             bh * d * nbk * wan::kQuantBlock, bh * d * 4};
    if (outputs_overlap(ptrs, bytes, 1, 7)) return WAN_ATTN_EINVAL;
  }
  const wan::AttnShape sh{batch, heads, s_q, s_kv};
  return from_hip(wan::launch_attn8_fwd(static_cast<const int8_t*>(q_codes),
                                        static_cast<const float*>(q_scale),
                                        static_cast<const int8_t*>(k_codes),
                                        static_cast<const float*>(k_scale),
                                        static_cast<const uint8_t*>(v_codes),
                                        static_cast<const float*>(v_scale), o, sh,
                                        static_cast<hipStream_t>(stream)),
                  "8-bit attention launch");
}

int wan_attn_fwd(const void* q, const void* k, const void* v, void* o, int64_t batch,
                 int64_t heads, int64_t s_q, int64_t s_kv, int64_t head_dim, int dtype,
                 void* stream) {
  int rc = check_shape(batch, heads, s_q, s_kv, head_dim);
  if (rc) return rc;
  if (dtype != WAN_ATTN_BF16 && dtype != WAN_ATTN_INT8_FP8) return WAN_ATTN_EINVAL;
  if (dtype == WAN_ATTN_INT8_FP8) {
    rc = check_attn8_size(s_kv);
    if (rc) return rc;
  }
  rc = check_qkvo(q, k, v, o, batch, heads, s_q, s_kv);
  if (rc) return rc;
  const wan::AttnShape sh{batch, heads, s_q, s_kv};
  hipStream_t st = static_cast<hipStream_t>(stream);
  WAN_LOG("fwd dtype=%d b=%lld H=%lld s_q=%lld s_kv=%lld", dtype, (long long)batch,
          (long long)heads, (long long)s_q, (long long)s_kv);
  if (dtype == WAN_ATTN_BF16) return fwd_bf16(q, k, v, o, nullptr, sh, st);

  // 8-bit: quantise into stream-ordered scratch, attend, release the scratch on the stream.
  const Attn8Layout L = attn8_layout(batch, heads, s_q, s_kv);
  void* ws = scratch_alloc(L.total, st, &rc);
  if (!ws) return rc;
  unsigned char* base = static_cast<unsigned char*>(ws);
  int8_t* qc = reinterpret_cast<int8_t*>(base + L.q_codes);
  int8_t* kc = reinterpret_cast<int8_t*>(base + L.k_codes);
  uint8_t* vc = base + L.v_codes;
  float* qs = reinterpret_cast<float*>(base + L.q_scale);
  float* kscale = reinterpret_cast<float*>(base + L.k_scale);
  float* vscale = reinterpret_cast<float*>(base + L.v_scale);
  float* sm = reinterpret_cast<float*>(base + L.smooth);
  float* cm = reinterpret_cast<float*>(base + L.chan_max);
  rc = from_hip(wan::launch_attn8_quantize(q, k, v, sh, qc, qs, kc, kscale, vc, vscale, sm, cm, st),
                "quantize launch");
  if (!rc)
    rc = from_hip(wan::launch_attn8_fwd(qc, qs, kc, kscale, vc, vscale, o, sh, st),
                  "8-bit attention launch");
  hipError_t fe = hipFreeAsync(ws, st);
  if (!rc && fe != hipSuccess) rc = from_hip(fe, "scratch release");
  return rc;
}

int wan_attn_fwd_lse(const void* q, const void* k, const void* v, void* o, void* lse, int64_t batch,
                     int64_t heads, int64_t s_q, int64_t s_kv, int64_t head_dim, void* stream) {
  int rc = check_shape(batch, heads, s_q, s_kv, head_dim);
  if (rc) return rc;
  rc = check_qkvo(q, k, v, o, batch, heads, s_q, s_kv);
  if (rc) return rc;
  if (!lse) return WAN_ATTN_EINVAL;
  if (!aligned16(lse)) return WAN_ATTN_EALIGN;
  const int64_t lb = batch * heads * s_q * 4;
  const int64_t qb = batch * s_q * heads * wan::kHeadDim * 2;
  const int64_t kb = batch * s_kv * heads * wan::kHeadDim * 2;
  if (overlaps(lse, lb, q, qb) || overlaps(lse, lb, k, kb) || overlaps(lse, lb, v, kb) || overlaps(lse, lb, o, qb))
    return WAN_ATTN_EINVAL;
  const wan::AttnShape sh{batch, heads, s_q, s_kv};
  WAN_LOG("fwd_lse b=%lld H=%lld s_q=%lld s_kv=%lld", (long long)batch, (long long)heads, (long long)s_q,
          (long long)s_kv);
  return fwd_bf16(q, k, v, o, static_cast<float*>(lse), sh, static_cast<hipStream_t>(stream));
}

int wan_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                 const void* lse, void* dq, void* dk, void* dv, int64_t batch, int64_t heads,
                 int64_t s_q, int64_t s_kv, int64_t head_dim, void* stream) {
  int rc = check_bwd(q, k, v, o, d_o, lse, dq, dk, dv, batch, heads, s_q, s_kv, head_dim);
  if (rc) return rc;
  const wan::AttnShape sh{batch, heads, s_q, s_kv};
  hipStream_t st = static_cast<hipStream_t>(stream);
  WAN_LOG("bwd b=%lld H=%lld s_q=%lld s_kv=%lld", (long long)batch, (long long)heads, (long long)s_q,
          (long long)s_kv);
  void* ws = scratch_alloc(wan::attn_bwd_scratch_bytes(sh), st, &rc);
  if (!ws) return rc;
  rc = from_hip(wan::launch_attn_bwd(q, k, v, o, d_o, static_cast<const float*>(lse), dq, dk, dv, sh, ws, st),
                "backward launch");
  hipError_t fe = hipFreeAsync(ws, st);
  if (!rc && fe != hipSuccess) rc = from_hip(fe, "scratch release");
  return rc;
}

int wan_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                         const void* lse, void* dq, void* dk, void* dv, int64_t batch, int64_t heads,
                         int64_t s_q, int64_t s_kv, int64_t head_dim, void* stream) {
  int rc = check_bwd(q, k, v, o, d_o, lse, dq, dk, dv, batch, heads, s_q, s_kv, head_dim);
  if (rc) return rc;
  const wan::AttnShape sh{batch, heads, s_q, s_kv};
  if (wan::attn_bwd_scratch_bytes(sh) > kNoallocScratchBytes) {
    WAN_LOG("bwd_noalloc: %zu bytes of row statistics exceed the %zu-byte static scratch",
            wan::attn_bwd_scratch_bytes(sh), kNoallocScratchBytes);
    return WAN_ATTN_EUNSUPPORTED;
  }
  void* ws = nullptr;
  rc = noalloc_scratch_for_current_device(&ws);
  if (rc) return rc;
  WAN_LOG("bwd_noalloc b=%lld H=%lld s_q=%lld s_kv=%lld", (long long)batch, (long long)heads, (long long)s_q,
          (long long)s_kv);
  return from_hip(wan::launch_attn_bwd(q, k, v, o, d_o, static_cast<const float*>(lse), dq, dk, dv, sh, ws,
                                       static_cast<hipStream_t>(stream)),
                  "backward launch");
}

int wan_fp8_quantize_rows(const void* x, int64_t rows, int64_t cols, void* codes, void* scales, void* stream) {
  int rc = check_fp8_dims(rows, cols);
  if (rc) return rc;
  if (!x || !codes || !scales) return WAN_ATTN_EINVAL;
  if (!aligned16(x) || !aligned16(codes) || !aligned4(scales)) return WAN_ATTN_EALIGN;
  const int64_t xb = rows * cols * 2, cb = rows * cols, sb = rows * 4;
  if (overlaps(codes, cb, x, xb) || overlaps(scales, sb, x, xb) || overlaps(scales, sb, codes, cb))
    return WAN_ATTN_EINVAL;
  WAN_LOG("fp8_quantize_rows rows=%lld cols=%lld", (long long)rows, (long long)cols);
  return from_hip(wan::launch_fp8_quantize_rows(x, rows, cols, codes, static_cast<float*>(scales),
                                                static_cast<hipStream_t>(stream)),
                  "fp8 row quantisation launch");
}

int wan_fp8_quantize_tensor(const void* w, int64_t rows, int64_t cols, void* codes, void* scale, void* stream) {
  int rc = check_fp8_dims(rows, cols);
  if (rc) return rc;
  if (!w || !codes || !scale) return WAN_ATTN_EINVAL;
  if (!aligned16(w) || !aligned16(codes) || !aligned4(scale)) return WAN_ATTN_EALIGN;
  const int64_t wb = rows * cols * 2, cb = rows * cols;
  if (overlaps(codes, cb, w, wb) || overlaps(scale, 4, w, wb) || overlaps(scale, 4, codes, cb))
    return WAN_ATTN_EINVAL;
  WAN_LOG("fp8_quantize_tensor rows=%lld cols=%lld", (long long)rows, (long long)cols);
  return from_hip(wan::launch_fp8_quantize_tensor(w, rows, cols, codes, static_cast<float*>(scale),
                                                  static_cast<hipStream_t>(stream)),
                  "fp8 tensor quantisation launch");
}

int wan_fp8_gemm(const void* x_codes, const void* x_scales, const void* w_codes, const void* w_scale, void* y,
                 int64_t m, int64_t n, int64_t k, void* stream) {
  int rc = check_fp8_dims(m, k);
  if (rc) return rc;
  rc = check_fp8_dims(n, k);
  if (rc) return rc;
  if (n % 4 != 0) return WAN_ATTN_EUNSUPPORTED;
  if ((long double)wan::ceil_div(m, 256) * (long double)wan::ceil_div(n, 256) > 2147483000.0L)
    return WAN_ATTN_EINVAL;
  if (!x_codes || !x_scales || !w_codes || !w_scale || !y) return WAN_ATTN_EINVAL;
  if (!aligned16(x_codes) || !aligned16(w_codes) || !aligned16(y) || !aligned4(x_scales) || !aligned4(w_scale))
    return WAN_ATTN_EALIGN;
  const int64_t yb = m * n * 2;
  if (overlaps(y, yb, x_codes, m * k) || overlaps(y, yb, w_codes, n * k) || overlaps(y, yb, x_scales, m * 4) ||
      overlaps(y, yb, w_scale, 4))
    return WAN_ATTN_EINVAL;
  WAN_LOG("fp8_gemm m=%lld n=%lld k=%lld", (long long)m, (long long)n, (long long)k);
  return from_hip(wan::launch_fp8_gemm(x_codes, static_cast<const float*>(x_scales), w_codes,
                                       static_cast<const float*>(w_scale), y, m, n, k,
                                       static_cast<hipStream_t>(stream)),
                  "fp8 gemm launch");
}

size_t wan_vsa_select_scratch_bytes(int64_t batch, int64_t heads, int64_t s_q, int64_t s_kv) {
  if (check_shape(batch, heads, s_q, s_kv, wan::kHeadDim)) return 0;
  return wan::vsa_select_scratch_bytes(wan::AttnShape{batch, heads, s_q, s_kv});
}

int wan_vsa_select(const void* q, const void* k, int64_t batch, int64_t heads, int64_t s_q, int64_t s_kv,
                   int64_t head_dim, int64_t keep, void* block_idx, void* scratch, void* stream) {
  int rc = check_shape(batch, heads, s_q, s_kv, head_dim);
  if (rc) return rc;
  rc = check_vsa(batch, heads, s_q, s_kv, keep);
  if (rc) return rc;
  if (!q || !k || !block_idx || !scratch) return WAN_ATTN_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(block_idx) || !aligned16(scratch)) return WAN_ATTN_EALIGN;
  const wan::AttnShape sh{batch, heads, s_q, s_kv};
  const int64_t qb = batch * s_q * heads * wan::kHeadDim * 2, kb = batch * s_kv * heads * wan::kHeadDim * 2;
  const int64_t ib = batch * heads * wan::ceil_div(s_q, 64) * keep * 4;
  const int64_t sb = (int64_t)wan::vsa_select_scratch_bytes(sh);
  if (overlaps(block_idx, ib, q, qb) || overlaps(block_idx, ib, k, kb) || overlaps(block_idx, ib, scratch, sb) ||
      overlaps(scratch, sb, q, qb) || overlaps(scratch, sb, k, kb))
    return WAN_ATTN_EINVAL;
  WAN_LOG("vsa_select b=%lld H=%lld s_q=%lld s_kv=%lld keep=%lld", (long long)batch, (long long)heads,
          (long long)s_q, (long long)s_kv, (long long)keep);
  return from_hip(wan::launch_vsa_select(q, k, sh, (int)keep, static_cast<int*>(block_idx), scratch,
                                         static_cast<hipStream_t>(stream)),
                  "vsa select launch");
}

int wan_vsa_attn(const void* q, const void* k, const void* v, const void* block_idx, void* o, int64_t batch,
                 int64_t heads, int64_t s_q, int64_t s_kv, int64_t head_dim, int64_t keep, void* stream) {
  int rc = check_shape(batch, heads, s_q, s_kv, head_dim);
  if (rc) return rc;
  rc = check_vsa(batch, heads, s_q, s_kv, keep);
  if (rc) return rc;
  rc = check_qkvo(q, k, v, o, batch, heads, s_q, s_kv);
  if (rc) return rc;
  if (!block_idx) return WAN_ATTN_EINVAL;
  if (!aligned16(block_idx)) return WAN_ATTN_EALIGN;
  const int64_t qb = batch * s_q * heads * wan::kHeadDim * 2;
  const int64_t ib = batch * heads * wan::ceil_div(s_q, 64) * keep * 4;
  if (overlaps(o, qb, block_idx, ib)) return WAN_ATTN_EINVAL;
  const wan::AttnShape sh{batch, heads, s_q, s_kv};
  WAN_LOG("vsa_attn b=%lld H=%lld s_q=%lld s_kv=%lld keep=%lld", (long long)batch, (long long)heads,
          (long long)s_q, (long long)s_kv, (long long)keep);
  return from_hip(wan::launch_vsa_attn(q, k, v, static_cast<const int*>(block_idx), (int)keep, o, sh,
                                       static_cast<hipStream_t>(stream)),
                  "vsa attention launch");
}

int wan_vsa_fwd(const void* q, const void* k, const void* v, void* o, int64_t batch, int64_t heads, int64_t s_q,
                int64_t s_kv, int64_t head_dim, int64_t keep, void* stream) {
  int rc = check_shape(batch, heads, s_q, s_kv, head_dim);
  if (rc) return rc;
  if (keep <= 0) keep = (wan::ceil_div(s_kv, 64) + 7) / 8;
  rc = check_vsa(batch, heads, s_q, s_kv, keep);
  if (rc) return rc;
  rc = check_qkvo(q, k, v, o, batch, heads, s_q, s_kv);
  if (rc) return rc;
  const wan::AttnShape sh{batch, heads, s_q, s_kv};
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t idx_bytes = align256((size_t)(batch * heads * wan::ceil_div(s_q, 64) * keep) * 4);
  void* ws = scratch_alloc(idx_bytes + wan::vsa_select_scratch_bytes(sh), st, &rc);
  if (!ws) return rc;
  int* idx = static_cast<int*>(ws);
  WAN_LOG("vsa_fwd b=%lld H=%lld s_q=%lld s_kv=%lld keep=%lld", (long long)batch, (long long)heads,
          (long long)s_q, (long long)s_kv, (long long)keep);
  rc = from_hip(wan::launch_vsa_select(q, k, sh, (int)keep, idx, static_cast<unsigned char*>(ws) + idx_bytes, st),
                "vsa select launch");
  if (!rc) rc = from_hip(wan::launch_vsa_attn(q, k, v, idx, (int)keep, o, sh, st), "vsa attention launch");
  hipError_t fe = hipFreeAsync(ws, st);
  if (!rc && fe != hipSuccess) rc = from_hip(fe, "scratch release");
  return rc;
}

}  // extern "C"
