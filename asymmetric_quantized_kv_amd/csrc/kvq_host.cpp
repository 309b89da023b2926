// Host side of the C ABI: argument checks, cache bookkeeping, split planning and
// kernel launches.  Every check runs before the first HIP call of an entry point.
#include "../../include/kvq.h"
#include "kvq_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <mutex>
#include <utility>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <string>
#include <vector>

using namespace kvq;

// One layer's storage: its layout (K and V bits may differ from layer to layer), plane
// geometry and byte offset in the arena.
struct LayerGeom {
  int layout, kbits, vbits;
  Geom g;
  int64_t base;
};

struct kv_cache {
  int n_layers, hkv, d;
  int64_t max_tokens;
  std::vector<LayerGeom> lg;
  uint8_t* arena;
  int64_t bytes;          // the planes (the footprint)
  int64_t counter_off;    // then kMaxHeadSplit uint32 split counters per (layer, KV head), zero between calls
  int64_t guard_off;      // then kGuardBytes guard bytes
  std::vector<int64_t> len;
  int device;
  bool poisoned;
};

namespace {

thread_local char g_err[512] = "";
thread_local int g_status = KV_OK;

int fail(int code, const char* fmt, ...) {
  g_status = code;
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_err() {
  g_err[0] = '\0';
  g_status = KV_OK;
}

bool layout_bits(int layout, int* kb, int* vb) {
  static const int tab[6][2] = {{16, 16}, {8, 8}, {8, 4}, {4, 8}, {4, 4}, {kF8, 4}};
  if (layout < 0 || layout > 5) return false;
  *kb = tab[layout][0];
  *vb = tab[layout][1];
  return true;
}

// Guard bytes after the planes of every arena: a fixed pattern that no kernel writes, checked by
// kv_cache_check_guard (a write past the last plane would land there first).
constexpr int64_t kGuardBytes = 256;
constexpr int kGuardByte = 0xA5;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
int64_t ceil_div(int64_t x, int64_t m) { return (x + m - 1) / m; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape check shared by kv_cache_create and kv_layout_footprint_bytes.
int check_shape(int layout, int n_layers, int n_kv_heads, int head_dim, int64_t max_tokens) {
  int kb, vb;
  if (!layout_bits(layout, &kb, &vb)) return fail(KV_EINVAL, "layout %d is not one of 0..5", layout);
  if (n_layers < 1) return fail(KV_EINVAL, "n_layers must be >= 1 (got %d)", n_layers);
  if (n_kv_heads < 1) return fail(KV_EINVAL, "n_kv_heads must be >= 1 (got %d)", n_kv_heads);
  if (head_dim < 32 || head_dim % 32 || head_dim > (1 << 16))
    return fail(KV_EINVAL, "head_dim must be a multiple of 32 in [32, 65536] (got %d)", head_dim);
  if (max_tokens < 1 || max_tokens > (int64_t(1) << 31) - kGranule)
    return fail(KV_EINVAL, "max_tokens out of range (got %lld)", (long long)max_tokens);
  // the arena size must not overflow: layers x heads x cap x (at most 4 D bytes per token)
  const __int128 worst = (__int128)n_layers * n_kv_heads * round_up(max_tokens, kGranule) * (4 * (__int128)head_dim);
  if (worst > ((__int128)1 << 50))
    return fail(KV_EINVAL, "a cache of %d layers x %d KV heads x %lld tokens x head_dim %d is too large", n_layers,
                n_kv_heads, (long long)max_tokens, head_dim);
  return KV_OK;
}

Geom make_geom(int kb, int vb, int d, int64_t max_tokens) {
  Geom g;
  g.cap = round_up(max_tokens, kGranule);
  g.kc = code_row_bytes(kb, d);
  g.ks = scale_row_bytes(kb, d);
  g.vc = code_row_bytes(vb, d);
  g.vs = scale_row_bytes(vb, d);
  return g;
}

uint8_t* layer_base(const kv_cache* c, int layer) { return c->arena + c->lg[layer].base; }

bool uniform_layout(const kv_cache* c) {
  for (const LayerGeom& l : c->lg)
    if (l.layout != c->lg[0].layout) return false;
  return true;
}

int check_cache(const kv_cache* c) {
  if (!c) return fail(KV_EINVAL, "cache is NULL");
  if (c->poisoned) return fail(KV_EHIP, "cache is poisoned by an earlier HIP error");
  return KV_OK;
}

int hip_fail(kv_cache* c, hipError_t e, const char* what) {
  if (c) c->poisoned = true;
  return fail(KV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(int dt) { return dt == KV_F32 || dt == KV_BF16 || dt == KV_F16; }

// Decode group sizes are padded to one of the instantiated widths.
int decode_group_pad(int g) {
  if (g <= 1) return 1;
  if (g <= 2) return 2;
  if (g <= 4) return 4;
  if (g <= 8) return 8;
  if (g <= 16) return 16;
  return -1;
}

// Split plan.  A launch is cut along the context into n splits so that its
// workgroups fill the device in as few rounds as possible: with `base` workgroups per
// split and `slots` resident workgroups, the time is ~ ceil(base * n / slots) rounds
// of (tokens per split).  The workspace bound depends only on shapes and the device,
// not on lengths, so a workspace sized once keeps fitting while the caches grow.
constexpr int64_t kChunkMinKeysPerSplit = 1024;
constexpr int kMaxSplitsChunk = 64;

std::mutex g_plan_mu;

// resident workgroups of `kernel` (`threads` per workgroup) on `device`; 0 if unknown
int g_cus[64];   // compute units per device, 0 until asked, -1 when the query failed

int device_cus_locked(int device) {
  if (device < 0 || device >= 64) return 0;
  if (g_cus[device] == 0 && hipDeviceGetAttribute(&g_cus[device], hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) {
    (void)hipGetLastError();
    g_cus[device] = -1;
  }
  return std::max(g_cus[device], 0);
}

int device_cus(int device) {
  std::lock_guard<std::mutex> lk(g_plan_mu);
  return device_cus_locked(device);
}

int64_t resident_slots(int device, const void* kernel, int threads = 256) {
  static std::vector<std::pair<const void*, int>> per_cu;
  std::lock_guard<std::mutex> lk(g_plan_mu);
  const int cus = device_cus_locked(device);
  if (cus <= 0) return 0;
  int n = -1;
  for (auto& e : per_cu)
    if (e.first == kernel) n = e.second;
  if (n < 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess) {
      (void)hipGetLastError();
      n = 1;
    }
    per_cu.emplace_back(kernel, std::max(n, 1));
    n = std::max(n, 1);
  }
  return (int64_t)cus * n;
}

int64_t split_cap(int64_t base, int64_t slots, int64_t hard_cap) {
  if (slots <= 0) slots = 1024;
  return std::max<int64_t>(1, std::min<int64_t>(hard_cap, ceil_div(2 * slots, base)));
}

// Pick the split count; `gran` is the split granularity in tokens.
void plan_splits(int64_t base, int64_t slots, int64_t cap, int64_t len, int64_t gran, int64_t min_tokens,
                 int* n_splits, int64_t* tps) {
  if (slots <= 0) slots = 1024;
  double best = 0;
  *n_splits = 1;
  *tps = round_up(std::max<int64_t>(len, 1), gran);
  for (int64_t s = 1; s <= cap; ++s) {
    const int64_t t = std::max(round_up(min_tokens, gran), round_up(ceil_div(len, s), gran));
    const int64_t n = ceil_div(len, t);
    if (n != s && s > 1) continue;
    const double cost = (double)ceil_div(base * n, slots) * (double)t;
    if (s == 1 || cost < best * 0.98) {
      best = cost;
      *n_splits = (int)n;
      *tps = t;
    }
  }
}

int check_sessions(kv_cache* const* sessions, int n_sessions, int layer) {
  if (!sessions) return fail(KV_EINVAL, "sessions is NULL");
  if (n_sessions < 1) return fail(KV_EINVAL, "n_sessions must be >= 1 (got %d)", n_sessions);
  const kv_cache* s0 = sessions[0];
  for (int i = 0; i < n_sessions; ++i) {
    const kv_cache* c = sessions[i];
    if (!c) return fail(KV_EINVAL, "session %d is NULL", i);
    if (c->poisoned) return fail(KV_EHIP, "session %d is poisoned by an earlier HIP error", i);
    if (c->n_layers != s0->n_layers || c->hkv != s0->hkv || c->d != s0->d)
      return fail(KV_EINVAL, "session %d does not share (n_layers, n_kv_heads, head_dim) with session 0", i);
    if (c->device != s0->device) return fail(KV_EINVAL, "session %d lives on another device", i);
  }
  if (layer < 0 || layer >= s0->n_layers) return fail(KV_EINVAL, "layer %d out of range [0, %d)", layer, s0->n_layers);
  for (int i = 1; i < n_sessions; ++i)
    if (sessions[i]->lg[layer].layout != s0->lg[layer].layout)
      return fail(KV_EINVAL, "session %d stores layer %d in another layout than session 0", i, layer);
  return KV_OK;
}

}  // namespace

extern "C" {

const char* kv_last_error(void) { return g_err; }

int kv_last_status(void) { return g_status; }

int64_t kv_layout_footprint_bytes(int layout, int n_layers, int n_kv_heads, int head_dim,
                                  int64_t max_tokens) {
  clear_err();
  int rc = check_shape(layout, n_layers, n_kv_heads, head_dim, max_tokens);
  if (rc) return rc;
  int kb, vb;
  layout_bits(layout, &kb, &vb);
  Geom g = make_geom(kb, vb, head_dim, max_tokens);
  return (int64_t)n_layers * n_kv_heads * g.region();
}

int64_t kv_layered_footprint_bytes(const int* layouts, int n_layers, int n_kv_heads, int head_dim,
                                   int64_t max_tokens) {
  clear_err();
  if (!layouts) return fail(KV_EINVAL, "layouts is NULL");
  if (n_layers < 1) return fail(KV_EINVAL, "n_layers must be >= 1 (got %d)", n_layers);
  for (int l = 0; l < n_layers; ++l)   // the bound on the whole arena, per layout
    if (int rc = check_shape(layouts[l], n_layers, n_kv_heads, head_dim, max_tokens)) return rc;
  int64_t total = 0;
  for (int l = 0; l < n_layers; ++l) {
    const int64_t b = kv_layout_footprint_bytes(layouts[l], 1, n_kv_heads, head_dim, max_tokens);
    if (b < 0) return b;
    total += b;
  }
  return total;
}

kv_cache* kv_cache_create_layered(const int* layouts, int n_layers, int n_kv_heads, int head_dim,
                                  int64_t max_tokens) {
  clear_err();
  if (!layouts) {
    fail(KV_EINVAL, "layouts is NULL");
    return nullptr;
  }
  if (n_layers < 1) {
    fail(KV_EINVAL, "n_layers must be >= 1 (got %d)", n_layers);
    return nullptr;
  }
  for (int l = 0; l < n_layers; ++l)
    if (check_shape(layouts[l], n_layers, n_kv_heads, head_dim, max_tokens)) return nullptr;
  if (head_dim != 64 && head_dim != 128) {
    fail(KV_EUNSUPPORTED, "head_dim %d is valid but only 64 and 128 are built", head_dim);
    return nullptr;
  }
  std::vector<LayerGeom> lg(n_layers);
  int64_t bytes = 0;
  for (int l = 0; l < n_layers; ++l) {
    LayerGeom& x = lg[l];
    x.layout = layouts[l];
    layout_bits(x.layout, &x.kbits, &x.vbits);
    x.g = make_geom(x.kbits, x.vbits, head_dim, max_tokens);
    x.base = bytes;
    bytes += (int64_t)n_kv_heads * x.g.region();
  }
  const char* fault = getenv("KVQ_FAULT");
  if (fault && strcmp(fault, "alloc") == 0) {
    fail(KV_ENOMEM, "hipMalloc of %lld bytes failed (forced by KVQ_FAULT=alloc)", (long long)bytes);
    return nullptr;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(KV_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  const int64_t counter_off = round_up(bytes, 256);
  const int64_t guard_off = counter_off + round_up(4 * (int64_t)n_layers * n_kv_heads * kMaxHeadSplit, 256);
  void* p = nullptr;
  e = hipMalloc(&p, (size_t)(guard_off + kGuardBytes));
  if (e != hipSuccess || !p) {
    (void)hipGetLastError();
    fail(KV_ENOMEM, "hipMalloc of %lld bytes failed: %s", (long long)(guard_off + kGuardBytes), hipGetErrorString(e));
    return nullptr;
  }
  e = hipMemset(p, 0, (size_t)guard_off);
  if (e == hipSuccess) e = hipMemset(static_cast<uint8_t*>(p) + guard_off, kGuardByte, kGuardBytes);
  if (e != hipSuccess) {
    (void)hipFree(p);
    fail(KV_EHIP, "hipMemset: %s", hipGetErrorString(e));
    return nullptr;
  }
  kv_cache* c = new kv_cache;
  c->n_layers = n_layers;
  c->hkv = n_kv_heads;
  c->d = head_dim;
  c->max_tokens = max_tokens;
  c->lg = std::move(lg);
  c->arena = static_cast<uint8_t*>(p);
  c->bytes = bytes;
  c->counter_off = counter_off;
  c->guard_off = guard_off;
  c->len.assign(n_layers, 0);
  c->device = dev;
  c->poisoned = false;
  return c;
}

kv_cache* kv_cache_create(int layout, int n_layers, int n_kv_heads, int head_dim,
                          int64_t max_tokens) {
  clear_err();
  if (check_shape(layout, n_layers, n_kv_heads, head_dim, max_tokens)) return nullptr;
  std::vector<int> layouts(n_layers, layout);
  return kv_cache_create_layered(layouts.data(), n_layers, n_kv_heads, head_dim, max_tokens);
}

int kv_cache_layout(const kv_cache* cache, int layer) {
  clear_err();
  if (!cache) return fail(KV_EINVAL, "cache is NULL");
  if (layer < 0 || layer >= cache->n_layers) return fail(KV_EINVAL, "layer %d out of range", layer);
  return cache->lg[layer].layout;
}

int kv_cache_shape(const kv_cache* cache, int* n_layers, int* n_kv_heads, int* head_dim, int64_t* max_tokens) {
  clear_err();
  if (!cache) return fail(KV_EINVAL, "cache is NULL");
  if (n_layers) *n_layers = cache->n_layers;
  if (n_kv_heads) *n_kv_heads = cache->hkv;
  if (head_dim) *head_dim = cache->d;
  if (max_tokens) *max_tokens = cache->max_tokens;
  return KV_OK;
}

int kv_cache_check_guard(const kv_cache* cache) {
  clear_err();
  int rc = check_cache(cache);
  if (rc) return rc;
  uint8_t g[kGuardBytes];
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(g, cache->arena + cache->guard_off, (size_t)kGuardBytes, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(const_cast<kv_cache*>(cache), e, "guard read");
  for (int64_t i = 0; i < kGuardBytes; ++i)
    if (g[i] != kGuardByte)
      return fail(KV_EINVAL, "guard byte %lld after the arena reads 0x%02x, not 0x%02x: something wrote past the planes",
                  (long long)i, g[i], kGuardByte);
  return KV_OK;
}

void kv_cache_destroy(kv_cache* cache) {
  if (!cache) return;
  if (cache->arena) (void)hipFree(cache->arena);
  delete cache;
}

int64_t kv_footprint_bytes(const kv_cache* cache) {
  clear_err();
  if (!cache) return fail(KV_EINVAL, "cache is NULL");
  return cache->bytes;
}

int64_t kv_cache_len(const kv_cache* cache, int layer) {
  clear_err();
  if (!cache) return fail(KV_EINVAL, "cache is NULL");
  if (layer < 0 || layer >= cache->n_layers) return fail(KV_EINVAL, "layer %d out of range", layer);
  return cache->len[layer];
}

int kv_cache_reset(kv_cache* cache) {
  clear_err();
  if (!cache) return fail(KV_EINVAL, "cache is NULL");
  std::fill(cache->len.begin(), cache->len.end(), 0);
  return KV_OK;
}

int kv_cache_truncate(kv_cache* cache, int layer, int64_t new_len) {
  clear_err();
  if (!cache) return fail(KV_EINVAL, "cache is NULL");
  if (layer < 0 || layer >= cache->n_layers) return fail(KV_EINVAL, "layer %d out of range", layer);
  if (new_len < 0 || new_len > cache->len[layer])
    return fail(KV_EINVAL, "new_len %lld outside [0, len = %lld]", (long long)new_len, (long long)cache->len[layer]);
  cache->len[layer] = new_len;
  return KV_OK;
}

int kv_cache_plane(const kv_cache* cache, int layer, int kv_head, int plane, const void** ptr,
                   int64_t* row_bytes) {
  clear_err();
  if (!cache) return fail(KV_EINVAL, "cache is NULL");
  if (!ptr || !row_bytes) return fail(KV_EINVAL, "ptr and row_bytes must not be NULL");
  if (layer < 0 || layer >= cache->n_layers) return fail(KV_EINVAL, "layer %d out of range", layer);
  if (kv_head < 0 || kv_head >= cache->hkv) return fail(KV_EINVAL, "kv_head %d out of range", kv_head);
  const Geom& g = cache->lg[layer].g;
  const uint8_t* region = layer_base(cache, layer) + (int64_t)kv_head * g.region();
  int64_t off, rb;
  switch (plane) {
    case KV_PLANE_KC: off = g.off_kc(); rb = g.kc; break;
    case KV_PLANE_KS: off = g.off_ks(); rb = g.ks; break;
    case KV_PLANE_VC: off = g.off_vc(); rb = g.vc; break;
    case KV_PLANE_VS: off = g.off_vs(); rb = g.vs; break;
    default: return fail(KV_EINVAL, "plane %d is not one of 0..3", plane);
  }
  *ptr = rb ? region + off : nullptr;
  *row_bytes = rb;
  return KV_OK;
}

// ---- session offload and restore ------------------------------------------------------
// Saved form: a header (magic, version, layout or -1 when layers differ, n_layers,
// n_kv_heads, head_dim), one int64 length and one int32 layout per layer, padded to 64
// bytes, then for every (layer, KV head) the first len[layer] rows of its planes KC, KS,
// VC, VS in that order.
namespace {
constexpr uint32_t kSessionMagic = 0x5351564bu;   // "KVQS"
constexpr uint32_t kSessionVersion = 2;
struct SessionHeader {
  uint32_t magic, version;
  int32_t layout, n_layers, n_kv_heads, head_dim;
  int64_t reserved;
};
static_assert(sizeof(SessionHeader) == 32, "header layout");
static_assert(sizeof(DecodeArgs) <= 4096, "decode kernel arguments");

int64_t session_data_offset(int n_layers) {
  return round_up((int64_t)sizeof(SessionHeader) + 12 * (int64_t)n_layers, 64);
}

int64_t session_bytes(const kv_cache* c, const int64_t* lens) {
  int64_t b = session_data_offset(c->n_layers);
  for (int l = 0; l < c->n_layers; ++l) {
    const Geom& g = c->lg[l].g;
    b += lens[l] * c->hkv * ((int64_t)g.kc + g.ks + g.vc + g.vs);
  }
  return b;
}

// one asynchronous copy per (layer, KV head, plane); to_host: cache -> buf, else buf -> cache
hipError_t session_copy(const kv_cache* c, uint8_t* buf, const int64_t* lens, bool to_host, hipStream_t st) {
  int64_t off = session_data_offset(c->n_layers);
  for (int l = 0; l < c->n_layers; ++l) {
    const Geom& g = c->lg[l].g;
    const int64_t pl_off[4] = {g.off_kc(), g.off_ks(), g.off_vc(), g.off_vs()};
    const int64_t pl_row[4] = {g.kc, g.ks, g.vc, g.vs};
    for (int h = 0; h < c->hkv; ++h) {
      uint8_t* region = layer_base(c, l) + (int64_t)h * g.region();
      for (int p = 0; p < 4; ++p) {
        const int64_t n = lens[l] * pl_row[p];
        if (n == 0) continue;
        hipError_t e = to_host ? hipMemcpyAsync(buf + off, region + pl_off[p], (size_t)n, hipMemcpyDefault, st)
                               : hipMemcpyAsync(region + pl_off[p], buf + off, (size_t)n, hipMemcpyDefault, st);
        if (e != hipSuccess) return e;
        off += n;
      }
    }
  }
  return hipSuccess;
}
}  // namespace

int64_t kv_session_bytes(const kv_cache* cache) {
  clear_err();
  if (!cache) return fail(KV_EINVAL, "cache is NULL");
  return session_bytes(cache, cache->len.data());
}

int kv_session_save(const kv_cache* cache, void* dst, size_t dst_bytes, void* stream) {
  clear_err();
  int rc = check_cache(cache);
  if (rc) return rc;
  if (!dst) return fail(KV_EINVAL, "dst is NULL");
  const int64_t need = session_bytes(cache, cache->len.data());
  if ((int64_t)dst_bytes < need)
    return fail(KV_EINVAL, "buffer of %zu bytes is smaller than the %lld the session needs", dst_bytes, (long long)need);
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, dst) == hipSuccess && attr.type == hipMemoryTypeDevice)
    return fail(KV_EINVAL, "dst must be host memory (the header is written by the host)");
  (void)hipGetLastError();
  const int32_t layout = uniform_layout(cache) ? cache->lg[0].layout : -1;
  SessionHeader hd{kSessionMagic, kSessionVersion, layout, cache->n_layers, cache->hkv, cache->d, 0};
  uint8_t* out = static_cast<uint8_t*>(dst);
  const int64_t data = session_data_offset(cache->n_layers);
  memset(out, 0, (size_t)data);
  memcpy(out, &hd, sizeof(hd));
  memcpy(out + sizeof(hd), cache->len.data(), 8 * (size_t)cache->n_layers);
  for (int l = 0; l < cache->n_layers; ++l) {
    const int32_t lay = cache->lg[l].layout;
    memcpy(out + sizeof(hd) + 8 * (size_t)cache->n_layers + 4 * (size_t)l, &lay, 4);
  }
  hipError_t e = session_copy(cache, out, cache->len.data(), true, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(const_cast<kv_cache*>(cache), e, "session save copy");
  return KV_OK;
}

int kv_session_load(kv_cache* cache, const void* src, size_t src_bytes, void* stream) {
  clear_err();
  int rc = check_cache(cache);
  if (rc) return rc;
  if (!src) return fail(KV_EINVAL, "src is NULL");
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, src) == hipSuccess && attr.type == hipMemoryTypeDevice)
    return fail(KV_EINVAL, "src must be host memory (the header is read by the host)");
  (void)hipGetLastError();
  if (src_bytes < sizeof(SessionHeader)) return fail(KV_EINVAL, "buffer of %zu bytes holds no session header", src_bytes);
  SessionHeader hd;
  memcpy(&hd, src, sizeof(hd));
  if (hd.magic != kSessionMagic || hd.version != kSessionVersion)
    return fail(KV_EINVAL, "not a saved session (magic %08x, version %u)", hd.magic, hd.version);
  if (hd.n_layers != cache->n_layers || hd.n_kv_heads != cache->hkv || hd.head_dim != cache->d)
    return fail(KV_EINVAL, "saved session (%d layers, %d KV heads, head_dim %d) does not match the cache",
                hd.n_layers, hd.n_kv_heads, hd.head_dim);
  if ((int64_t)src_bytes < session_data_offset(cache->n_layers))
    return fail(KV_EINVAL, "buffer of %zu bytes is shorter than the session header", src_bytes);
  const uint8_t* in = static_cast<const uint8_t*>(src);
  std::vector<int64_t> lens(cache->n_layers);
  memcpy(lens.data(), in + sizeof(hd), 8 * lens.size());
  for (int l = 0; l < cache->n_layers; ++l) {
    int32_t lay;
    memcpy(&lay, in + sizeof(hd) + 8 * lens.size() + 4 * (size_t)l, 4);
    if (lay != cache->lg[l].layout)
      return fail(KV_EINVAL, "layer %d was saved in layout %d, the cache stores layout %d", l, lay, cache->lg[l].layout);
    if (lens[l] < 0) return fail(KV_EINVAL, "saved length %lld of layer %d is negative", (long long)lens[l], l);
    if (lens[l] > cache->max_tokens)
      return fail(KV_ECAPACITY, "saved length %lld of layer %d exceeds max_tokens %lld", (long long)lens[l], l,
                  (long long)cache->max_tokens);
  }
  const int64_t need = session_bytes(cache, lens.data());
  if ((int64_t)src_bytes < need)
    return fail(KV_EINVAL, "buffer of %zu bytes is shorter than the %lld the saved session needs", src_bytes, (long long)need);
  hipError_t e = session_copy(cache, const_cast<uint8_t*>(in), lens.data(), false, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(cache, e, "session load copy");
  cache->len = lens;
  return KV_OK;
}

int kv_cache_copy_plane(const kv_cache* cache, int layer, int kv_head, int plane, int64_t row0,
                        int64_t n_rows, void* dst, void* stream) {
  const void* p = nullptr;
  int64_t rb = 0;
  int rc = kv_cache_plane(cache, layer, kv_head, plane, &p, &rb);
  if (rc) return rc;
  if (!dst) return fail(KV_EINVAL, "dst is NULL");
  if (row0 < 0 || n_rows < 0 || row0 > cache->lg[layer].g.cap || n_rows > cache->lg[layer].g.cap - row0)
    return fail(KV_EINVAL, "rows [%lld, %lld) outside the plane", (long long)row0, (long long)(row0 + n_rows));
  if (cache->poisoned) return fail(KV_EHIP, "cache is poisoned by an earlier HIP error");
  if (rb == 0 || n_rows == 0) return KV_OK;
  hipError_t e = hipMemcpyAsync(dst, static_cast<const uint8_t*>(p) + row0 * rb, (size_t)(n_rows * rb),
                                hipMemcpyDefault, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(const_cast<kv_cache*>(cache), e, "hipMemcpyAsync");
  return KV_OK;
}

int kv_append_quant(kv_cache* cache, int layer, const void* k, const void* v, int dtype,
                    int64_t n_new, void* stream) {
  clear_err();
  int rc = check_cache(cache);
  if (rc) return rc;
  if (layer < 0 || layer >= cache->n_layers) return fail(KV_EINVAL, "layer %d out of range [0, %d)", layer, cache->n_layers);
  if (n_new < 0) return fail(KV_EINVAL, "n_new must be >= 0 (got %lld)", (long long)n_new);
  if (!dtype_ok(dtype)) return fail(KV_EINVAL, "dtype %d is not one of KV_F32/KV_BF16/KV_F16", dtype);
  if (n_new > cache->max_tokens - cache->len[layer])
    return fail(KV_ECAPACITY, "append of %lld tokens to layer %d (len %lld) exceeds max_tokens %lld",
                (long long)n_new, layer, (long long)cache->len[layer], (long long)cache->max_tokens);
  if (n_new == 0) return KV_OK;
  if (!k || !v) return fail(KV_EINVAL, "k and v must not be NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(KV_EINVAL, "k and v must be 16-byte aligned");
  AppendArgs a;
  a.src[0] = k;
  a.src[1] = v;
  const LayerGeom& L = cache->lg[layer];
  a.layer_base = layer_base(cache, layer);
  a.g = L.g;
  a.t0 = cache->len[layer];
  a.n = n_new;
  a.hkv = cache->hkv;
  hipError_t e = launch_append(a, L.kbits, L.vbits, dtype, cache->d, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(cache, e, "append launch");
  cache->len[layer] += n_new;
  return KV_OK;
}

}  // extern "C"

namespace {

constexpr int64_t kMaxSplitsDecode = 65535;   // the split is the decode grid's z dimension

int64_t partial_bytes(int64_t rows, int n_splits, int d) {
  return rows * n_splits * (int64_t)(d + 2) * (int64_t)sizeof(float);
}

int check_q_out(const void* q, int q_dtype, const void* out, const char* out_name) {
  if (!dtype_ok(q_dtype)) return fail(KV_EINVAL, "q_dtype %d is not one of KV_F32/KV_BF16/KV_F16", q_dtype);
  if (!q || !out) return fail(KV_EINVAL, "q and %s must not be NULL", out_name);
  if (!aligned16(q) || !aligned16(out)) return fail(KV_EINVAL, "q and %s must be 16-byte aligned", out_name);
  return KV_OK;
}

int check_workspace(const void* ws, size_t ws_bytes, int64_t need) {
  if ((int64_t)ws_bytes < need)
    return fail(KV_EINVAL, "workspace of %zu bytes is smaller than the %lld needed", ws_bytes, (long long)need);
  if (need && (!ws || !aligned16(ws))) return fail(KV_EINVAL, "workspace must be a 16-byte aligned device pointer");
  return KV_OK;
}

// A caller-chosen split: n_splits ranges of `per` tokens (a multiple of `gran`) that
// together cover `len` tokens.
int check_split(int n_splits, int64_t per, int64_t gran, int64_t len, const char* what) {
  if (n_splits < 1 || n_splits > 65535) return fail(KV_EINVAL, "n_splits must be in [1, 65535] (got %d)", n_splits);
  if (per < 1 || per % gran || per > (int64_t(1) << 40))
    return fail(KV_EINVAL, "%s must be a positive multiple of %lld (got %lld)", what, (long long)gran, (long long)per);
  if ((int64_t)n_splits * per < len)
    return fail(KV_EINVAL, "%d splits of %lld do not cover %lld cached tokens", n_splits, (long long)per, (long long)len);
  return KV_OK;
}

// What a decode call checks and derives before its first launch.
struct DecodePrep {
  int hkv, d, group, gp, kbits, vbits, device;
  int64_t max_len, base, slots;
  std::vector<int64_t> lens;   // cached tokens of each session in the layer
};

int decode_prepare(kv_cache* const* sessions, int n_sessions, int layer, int n_q_heads, bool need_tokens,
                   DecodePrep* p) {
  int rc = check_sessions(sessions, n_sessions, layer);
  if (rc) return rc;
  const kv_cache* s0 = sessions[0];
  if (n_q_heads < 1 || n_q_heads % s0->hkv)
    return fail(KV_EINVAL, "n_q_heads %d is not a positive multiple of n_kv_heads %d", n_q_heads, s0->hkv);
  if (s0->hkv > 65535) return fail(KV_EUNSUPPORTED, "n_kv_heads %d exceeds one launch (65535)", s0->hkv);
  p->hkv = s0->hkv;
  p->d = s0->d;
  p->kbits = s0->lg[layer].kbits;
  p->vbits = s0->lg[layer].vbits;
  p->device = s0->device;
  p->group = n_q_heads / s0->hkv;
  p->gp = decode_group_pad(p->group);
  if (p->gp < 0) return fail(KV_EUNSUPPORTED, "decode group size %d > 16 is not built", p->group);
  p->max_len = 0;
  p->lens.resize(n_sessions);
  for (int i = 0; i < n_sessions; ++i) {
    if (need_tokens && sessions[i]->len[layer] == 0)
      return fail(KV_EEMPTY, "session %d has no cached token in layer %d", i, layer);
    p->lens[i] = sessions[i]->len[layer];
    p->max_len = std::max(p->max_len, sessions[i]->len[layer]);
  }
  p->base = (int64_t)n_sessions * p->hkv;
  p->slots = resident_slots(p->device, decode_kernel_for(p->kbits, p->vbits, p->d, p->gp));
  return KV_OK;
}

// Splits per session for a decode call: every session is cut at the same tokens_per_split,
// so a session of len tokens keeps ceil(len / tps) workgroups per KV head busy and the
// splits past its end exit at once.  With lengths that differ a lot, many splits let the
// long sessions spread over the device while short ones take one workgroup each.
constexpr int64_t kDecodeWgFixedTokens = 256;   // per-workgroup overhead, in streamed tokens
// The latency of merging the splits inside the launch (each partial written through to memory,
// the split counter, the last workgroup's coherent reads), in streamed tokens.  Measured on a
// 22-layer step (4 KV heads x 64, one session): a layer of 512 tokens takes 6.3 us in one split;
// 1,024 tokens take 7.75 us in one split against 8.6 in two; from 1,536 tokens on the split
// plan wins (9.1 us at 1,536 in three splits against 10.0 in one).
constexpr int64_t kDecodeMergeTokens = 768;
constexpr int kMinSplitGroup = 2;               // query heads a workgroup keeps when a head's group is split

int64_t decode_split_cap(const DecodePrep& p) {
  const int64_t slots = p.slots > 0 ? p.slots : 1024;
  return std::max<int64_t>(1, std::min<int64_t>(kMaxSplitsDecode, ceil_div(2 * slots, p.hkv)));
}

void decode_plan(const DecodePrep& p, int* n_splits, int64_t* tps) {
  const int64_t slots = p.slots > 0 ? p.slots : 1024;
  const int64_t gran = kDecodeWaveTokens;
  const int64_t cap = decode_split_cap(p);
  double best = 0;
  *n_splits = 1;
  *tps = round_up(std::max<int64_t>(p.max_len, 1), gran);
  for (int64_t s = 1; s <= cap; ++s) {
    const int64_t t = round_up(ceil_div(p.max_len, s), gran);
    const int64_t n = ceil_div(p.max_len, t);
    if (n != s && s > 1) continue;
    int64_t busy = 0;   // workgroups per KV head that hold tokens
    for (int64_t len : p.lens) busy += std::max<int64_t>(1, ceil_div(len, t));
    // rounds of the busy workgroups times (the tokens each one streams + a fixed cost of
    // kDecodeWgFixedTokens for its query preparation and epilogue), a small charge for the
    // empty workgroups, and for a split plan the merge: its latency and its read of n partials
    // per row
    const int64_t rows = (int64_t)p.lens.size() * p.hkv * p.group;
    const double cost = (double)ceil_div(busy * p.hkv, slots) * (double)(t + kDecodeWgFixedTokens) +
                        0.02 * (double)gran * (double)((n * (int64_t)p.lens.size() - busy) * p.hkv) / (double)slots +
                        (n > 1 ? (double)kDecodeMergeTokens + (double)rows * n * (p.d + 2) * 4.0 / (double)(208 * slots)
                               : 0.0);
    if (s == 1 || cost < best * 0.98) {
      best = cost;
      *n_splits = (int)n;
      *tps = t;
    }
    if (t == gran) break;
  }
}

// Whether a split decode call launches only its busy workgroups (see DecodeArgs::compact):
// then the splits past a session's end write nothing, and the merge reads each session's
// first n_valid = ceil(len / tps) splits.  The library's own calls do it when one launch
// holds every session and some session is shorter than the split range (otherwise there is
// no empty workgroup to drop, and the workgroups' split lookup would only add latency);
// kv_attend_decode_partial always writes every split.
bool decode_compact(int n_sessions, int n_splits, const int32_t* n_valid) {
  if (n_splits <= 1 || n_sessions > kMaxSessions) return false;
  int64_t pieces = 0;   // the grid's second dimension
  bool empty = false;
  for (int i = 0; i < n_sessions; ++i) {
    pieces += n_valid[i];
    empty |= n_valid[i] < n_splits;
  }
  return empty && pieces <= 65535;
}

// Sessions longest first (stable): workgroups are dispatched in launch order, so the long
// sessions' work starts early and the short ones fill the tail.
std::vector<int> longest_first(const std::vector<int64_t>& lens) {
  std::vector<int> order(lens.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return lens[x] > lens[y]; });
  return order;
}

// A streamed launch (DecodeArgs::stream): the sessions' blocks of kDecodeWaveTokens tokens,
// longest session first and laid end to end, are cut into n_wg ranges per KV head, one
// workgroup each and all resident at once, so no workgroup waits for a second round or
// streams alone at the end.  A session overlapped by several ranges leaves one partial per
// range, merged in the launch.  Each part of a session a workgroup takes costs it the
// session's query preparation and an epilogue besides its blocks, so the cut balances blocks
// plus kStreamPartTokens per part: a range over many short sessions holds fewer blocks.
// (768 tokens per part measured best for 64 sessions of 512..32,768 tokens, K8V4, Hkv 8,
// D 128: 178-180 us a call against 181 at 256 and 186-187 at 1,024, same box.)
constexpr int64_t kStreamPartTokens = 768;
struct StreamPlan {
  int n_wg = 0;
  int max_seg = 0;                             // partials per row the workspace must hold
  std::vector<int32_t> wg_block0;              // n_wg + 1 range bounds
  std::vector<int32_t> block0, wfirst, nseg;   // per session, in longest-first order
};

StreamPlan stream_plan(const DecodePrep& p, const std::vector<int>& order, int n_wg) {
  StreamPlan sp;
  const int n = (int)order.size();
  std::vector<int64_t> nb(n);
  int64_t total = 0;
  sp.block0.resize(n);
  for (int i = 0; i < n; ++i) {
    sp.block0[i] = (int32_t)total;
    nb[i] = ceil_div(std::max<int64_t>(p.lens[order[i]], 1), kDecodeWaveTokens);
    total += nb[i];
  }
  sp.n_wg = (int)std::max<int64_t>(1, std::min<int64_t>(n_wg, total));
  const double part = (double)kStreamPartTokens / kDecodeWaveTokens;   // a part's fixed cost, in blocks
  const double target = ((double)total + part * (double)(n + sp.n_wg - 1)) / sp.n_wg;
  sp.wg_block0.assign(sp.n_wg + 1, (int32_t)total);
  sp.wg_block0[0] = 0;
  int w = 0;
  double cum = 0;
  int64_t b = 0;
  for (int i = 0; i < n; ++i) {
    cum += part;                         // the session's first part
    for (int64_t j = 0; j < nb[i]; ++j) {
      cum += 1.0;
      ++b;
      if (cum >= target * (w + 1) && w + 1 < sp.n_wg && b < total) {
        sp.wg_block0[++w] = (int32_t)b;   // the next workgroup starts at block b
        if (j + 1 < nb[i]) cum += part;   // and takes the rest of this session as a new part
      }
    }
  }
  // the workgroup of block x: the last range starting at or before it (ranges past the last
  // cut are empty and start at `total`, beyond every block)
  auto range_of = [&](int64_t x) {
    return (int)(std::upper_bound(sp.wg_block0.begin(), sp.wg_block0.begin() + sp.n_wg, (int32_t)x) -
                 sp.wg_block0.begin()) - 1;
  };
  sp.wfirst.resize(n);
  sp.nseg.resize(n);
  for (int i = 0; i < n; ++i) {
    const int w0 = range_of(sp.block0[i]), w1 = range_of(sp.block0[i] + nb[i] - 1);
    sp.wfirst[i] = w0;
    sp.nseg[i] = w1 - w0 + 1;
    sp.max_seg = std::max(sp.max_seg, sp.nseg[i]);
  }
  return sp;
}

int decode_launch(kv_cache* const* sessions, int n_sessions, int layer, const DecodePrep& p, const void* q,
                  int q_dtype, int n_q_heads, float sm_scale, int n_splits, int64_t tps, bool partial, float* ws,
                  float* out, hipStream_t st, bool compact = false, bool fused = false,
                  const StreamPlan* stream = nullptr) {
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.hkv = p.hkv;
  a.hq = n_q_heads;
  a.group = p.group;
  a.n_splits = n_splits;
  a.partial = partial ? 1 : 0;
  a.fused = partial && fused ? 1 : 0;
  a.tps = tps;
  a.q = q;
  a.q_dtype = q_dtype;
  a.qk_scale = sm_scale * 1.4426950408889634f;
  a.ws = ws;
  a.out = out;
  const std::vector<int> order = longest_first(p.lens);
  if (stream) {   // one launch of every session (the caller checked n_sessions <= kMaxSessions)
    a.n_splits = stream->max_seg;
    a.partial = 1;
    a.fused = 1;
    a.stream = 1;
    a.n_wg = stream->n_wg;
    for (int w = 0; w <= stream->n_wg; ++w) a.wg_block0[w] = stream->wg_block0[w];
    a.n_sess = n_sessions;
    for (int i = 0; i < n_sessions; ++i) {
      const kv_cache* c = sessions[order[i]];
      a.sess[i].base = layer_base(c, layer);
      a.sess[i].counters = reinterpret_cast<uint32_t*>(c->arena + c->counter_off) + (int64_t)layer * c->hkv * kMaxHeadSplit;
      a.sess[i].cap = c->lg[layer].g.cap;
      a.sess[i].len = c->len[layer];
      a.sess[i].row = (int32_t)order[i];
      a.sess[i].piece0 = stream->block0[i];
      a.sess[i].wfirst = stream->wfirst[i];
      a.sess[i].nseg = stream->nseg[i];
    }
    a.hsplit = 1;
    a.one_chunk = 0;
    hipError_t e = launch_decode(a, p.kbits, p.vbits, p.d, decode_group_pad(a.group), st);
    if (e != hipSuccess) {
      for (int i = 0; i < n_sessions; ++i) sessions[i]->poisoned = true;
      return fail(KV_EHIP, "decode launch: %s", hipGetErrorString(e));
    }
    return KV_OK;
  }
  for (int b0 = 0; b0 < n_sessions; b0 += kMaxSessions) {
    const int nb = std::min(kMaxSessions, n_sessions - b0);
    a.n_sess = nb;
    for (int i = 0; i < nb; ++i) {
      const int r = order[b0 + i];
      const kv_cache* c = sessions[r];
      a.sess[i].base = layer_base(c, layer);
      a.sess[i].counters = reinterpret_cast<uint32_t*>(c->arena + c->counter_off) + (int64_t)layer * c->hkv * kMaxHeadSplit;
      a.sess[i].cap = c->lg[layer].g.cap;
      a.sess[i].len = c->len[layer];
      a.sess[i].row = (int32_t)r;
    }
    a.compact = compact ? 1 : 0;
    a.n_pieces = 0;
    for (int i = 0; i < nb; ++i) {   // each session's busy splits, one after the other
      a.sess[i].piece0 = a.n_pieces;
      a.n_pieces += (int32_t)ceil_div(std::max<int64_t>(a.sess[i].len, 1), tps);
    }
    // A launch of one round (a workgroup per compute unit at most) is latency-bound: it splits
    // each KV head's query group over up to kMaxHeadSplit workgroups while they still fit (each
    // reads the head's codes; the chain of work per workgroup shrinks), and if its waves hold a
    // single chunk each, takes the variant that requests all codes up front.
    const int64_t wgs = (int64_t)a.hkv * (compact ? a.n_pieces : (int64_t)nb * n_splits);
    const int64_t cus = device_cus(p.device);
    a.hsplit = 1;
    for (int hs = kMaxHeadSplit; hs > 1; hs /= 2)
      if (p.group % hs == 0 && p.group / hs >= kMinSplitGroup && wgs * hs <= cus) {
        a.hsplit = hs;
        break;
      }
    a.group = p.group / a.hsplit;
    a.one_chunk = tps <= kDecodeWaveTokens && wgs * a.hsplit <= cus ? 1 : 0;
    hipError_t e = launch_decode(a, p.kbits, p.vbits, p.d, decode_group_pad(a.group), st);
    if (e != hipSuccess) {
      for (int i = 0; i < n_sessions; ++i) sessions[i]->poisoned = true;
      return fail(KV_EHIP, "decode launch: %s", hipGetErrorString(e));
    }
  }
  return KV_OK;
}

// n_valid (optional): per session of rows_per_sess rows, how many of its splits hold partials
hipError_t merge_launch(const float* ws, int64_t rows, int n_splits, int d, float* out, hipStream_t st,
                        int rows_per_sess = 0, const int32_t* n_valid = nullptr) {
  MergeArgs m;
  memset(&m, 0, sizeof(m));
  m.ws = ws;
  m.out = out;
  m.rows = rows;
  m.n_splits = n_splits;
  m.d = d;
  if (rows_per_sess > 0 && n_valid) {
    m.rows_per_sess = rows_per_sess;
    for (int64_t i = 0; i < rows / rows_per_sess && i < kMaxSessions; ++i) m.n_valid[i] = n_valid[i];
  }
  return launch_merge(m, st);
}

// What a chunk call checks and derives before its first launch.
struct ChunkPrep {
  int group;
  int64_t len, rows, mtiles, base, slots;
};

int chunk_prepare(const kv_cache* cache, int layer, int n_q_heads, int64_t n_new, bool need_tokens, ChunkPrep* p) {
  int rc = check_cache(cache);
  if (rc) return rc;
  if (layer < 0 || layer >= cache->n_layers) return fail(KV_EINVAL, "layer %d out of range [0, %d)", layer, cache->n_layers);
  if (n_q_heads < 1 || n_q_heads % cache->hkv)
    return fail(KV_EINVAL, "n_q_heads %d is not a positive multiple of n_kv_heads %d", n_q_heads, cache->hkv);
  if (cache->hkv > 65535) return fail(KV_EUNSUPPORTED, "n_kv_heads %d exceeds one launch (65535)", cache->hkv);
  p->len = cache->len[layer];
  if (need_tokens) {
    if (p->len == 0) return fail(KV_EEMPTY, "layer %d has no cached token", layer);
    if (n_new < 1 || n_new > p->len)
      return fail(KV_EINVAL, "n_new %lld must be in [1, len = %lld] (append the chunk first)", (long long)n_new,
                  (long long)p->len);
  } else if (n_new < 1) {
    return fail(KV_EINVAL, "n_new must be >= 1");
  }
  p->group = n_q_heads / cache->hkv;
  p->rows = n_new * p->group;
  p->mtiles = ceil_div(p->rows, kChunkRows);
  if (p->mtiles > 0x7fffffff) return fail(KV_EUNSUPPORTED, "chunk of %lld rows is too large", (long long)p->rows);
  p->base = p->mtiles * cache->hkv;
  p->slots = resident_slots(cache->device, chunk_kernel_for(cache->lg[layer].kbits, cache->lg[layer].vbits, cache->d, false),
                            kChunkThreads);
  return KV_OK;
}

// Splits considered for a chunk.  At least 2 even when the row tiles alone exceed the
// resident workgroups: 640 tiles on 256 slots run 2.5 rounds (the last one half idle) at one
// split, but 5 full rounds of half-length work at two.
int64_t chunk_split_cap(const ChunkPrep& p) {
  return std::max<int64_t>(2, split_cap(p.base, p.slots, kMaxSplitsChunk));
}

// Estimated duration of a chunk launch under the split (n, t), in units of one 64-key tile of
// one workgroup.  Each workgroup costs its causal key-tile count plus a fixed start-up and
// epilogue charge; the workgroups of each XCD are list-scheduled over that die's resident
// slots in the order the kernel hands them out (die x takes t = x * per + i, i = 0, 1, ...,
// as row tile t % mtiles of split t / (mtiles * hkv)).  More than one split adds the merge's
// traffic (partials written and read back) at a nominal bandwidth.
double chunk_cost(const ChunkPrep& p, int d, int n, int64_t t, std::vector<double>& heap) {
  constexpr double kWgFixedTiles = 2.0;
  constexpr double kMergeBytesPerSec = 5e12, kCuFlopsPerSec = 2.9e12;
  const int64_t slots = p.slots > 0 ? p.slots : 1024;
  const int64_t die_slots = std::max<int64_t>(1, slots / kXcds);
  const int64_t hkv = p.base / p.mtiles, n_new = p.rows / p.group, base_pos = p.len - n_new;
  const int64_t total = p.base * n, per = total / kXcds, rem = total % kXcds;
  double makespan = 0;
  for (int64_t x = 0; x < (int64_t)kXcds; ++x) {
    const int64_t cnt = per + (x < rem ? 1 : 0), first = x * per + std::min(x, rem);
    if (cnt == 0) continue;
    heap.assign((size_t)std::min(die_slots, cnt), 0.0);
    for (int64_t i = 0; i < cnt; ++i) {
      const int64_t wg = first + i, mt = wg % p.mtiles, sp = wg / (p.mtiles * hkv);
      const int64_t last_row = std::min((mt + 1) * kChunkRows, p.rows) - 1;
      const int64_t k_lo = sp * t, k_hi = std::min({k_lo + t, p.len, base_pos + last_row / p.group + 1});
      const double w = kWgFixedTiles + (k_hi > k_lo ? (double)ceil_div(k_hi - k_lo, kChunkKeys) : 0.0);
      std::pop_heap(heap.begin(), heap.end(), std::greater<double>());
      heap.back() += w;
      std::push_heap(heap.begin(), heap.end(), std::greater<double>());
    }
    makespan = std::max(makespan, *std::max_element(heap.begin(), heap.end()));
  }
  if (n > 1) {
    const double bytes = 2.0 * (double)(p.rows * hkv) * n * (d + 2) * sizeof(float);
    const double tile_sec = (double)kChunkRows * kChunkKeys * 4.0 * d / kCuFlopsPerSec;
    makespan += bytes / kMergeBytesPerSec / tile_sec;
  }
  return makespan;
}

void chunk_plan(const ChunkPrep& p, int d, int* n_splits, int64_t* tps) {
  const int64_t cap = chunk_split_cap(p);
  if (p.base * cap > (int64_t(1) << 20)) {   // very large launches: the round-count model
    plan_splits(p.base, p.slots, cap, p.len, kChunkKeys, kChunkMinKeysPerSplit, n_splits, tps);
    return;
  }
  std::vector<double> heap;
  double best = 0;
  *n_splits = 1;
  *tps = round_up(std::max<int64_t>(p.len, 1), kChunkKeys);
  for (int64_t s = 1; s <= cap; ++s) {
    const int64_t t = std::max(round_up(kChunkMinKeysPerSplit, kChunkKeys), round_up(ceil_div(p.len, s), kChunkKeys));
    const int64_t n = ceil_div(p.len, t);
    if (n != s && s > 1) continue;
    const double cost = chunk_cost(p, d, (int)n, s == 1 ? *tps : t, heap);
    if (s == 1 || cost < best * 0.98) {
      best = cost;
      *n_splits = (int)n;
      *tps = s == 1 ? *tps : t;
    }
  }
}

int chunk_launch(kv_cache* cache, int layer, const ChunkPrep& p, const void* q, int q_dtype, int n_q_heads,
                 int64_t n_new, float sm_scale, int n_splits, int64_t tps, bool partial, float* ws, float* out,
                 hipStream_t st) {
  ChunkArgs a;
  memset(&a, 0, sizeof(a));
  a.base = layer_base(cache, layer);
  a.g = cache->lg[layer].g;
  a.len = p.len;
  a.n_new = n_new;
  a.hkv = cache->hkv;
  a.hq = n_q_heads;
  a.group = p.group;
  a.n_splits = n_splits;
  a.partial = partial ? 1 : 0;
  a.tps = tps;
  a.q = q;
  a.q_dtype = q_dtype;
  a.qk_scale = sm_scale * 1.4426950408889634f;
  a.ws = ws;
  a.out = out;
  hipError_t e = launch_chunk(a, cache->lg[layer].kbits, cache->lg[layer].vbits, cache->d, st);
  if (e != hipSuccess) return hip_fail(cache, e, "chunk launch");
  return KV_OK;
}

// Split partials and their merge in one launch: the last workgroup of each (session, KV head)
// to finish merges.  Its split counters live in the session's arena, so launches of more than
// kMaxSessions sessions stay independent; a cache passed twice in one call would share its
// counters between two rows and takes the separate merge instead.
bool repeated_cache(kv_cache* const* sessions, int n_sessions) {
  std::vector<const kv_cache*> seen(sessions, sessions + n_sessions);
  std::sort(seen.begin(), seen.end());
  return std::adjacent_find(seen.begin(), seen.end()) != seen.end();
}

void decode_valid(const DecodePrep& p, int n_sessions, int64_t tps, int32_t* n_valid) {
  for (int i = 0; i < n_sessions && i < kMaxSessions; ++i) n_valid[i] = (int32_t)ceil_div(std::max<int64_t>(p.lens[i], 1), tps);
}

// Where the split plan would launch only the busy workgroups of uneven sessions (one launch,
// fused merge), a streamed launch takes its place when the device's resident workgroups per KV
// head fit the range table and the workspace (ws_bytes) holds its partials.
bool decode_stream(kv_cache* const* sessions, int n_sessions, const DecodePrep& p, int q_dtype, int n_q_heads,
                   int n_splits, int64_t tps, int64_t ws_bytes, StreamPlan* sp) {
  if (n_sessions < 2 || n_sessions > kMaxSessions || n_splits <= 1) return false;
  int32_t n_valid[kMaxSessions];
  decode_valid(p, n_sessions, tps, n_valid);
  if (!decode_compact(n_sessions, n_splits, n_valid) || repeated_cache(sessions, n_sessions)) return false;
  const int64_t slots = resident_slots(p.device, decode_kernel_for(p.kbits, p.vbits, p.d, p.gp, true, q_dtype == KV_F32));
  const int64_t n_wg = std::min<int64_t>(slots > 0 ? slots / p.hkv : 0, decode_split_cap(p));
  if (n_wg < 2 || n_wg > kMaxStreamWg) return false;
  *sp = stream_plan(p, longest_first(p.lens), (int)n_wg);
  return partial_bytes(n_sessions * (int64_t)n_q_heads, sp->max_seg, p.d) <= ws_bytes;
}

// kv_attend_decode's work once its arguments are checked and planned: the streamed launch, or
// the partial pass (or the whole attention for one split) and the merge, with the partials in ws.
int decode_run(kv_cache* const* sessions, int n_sessions, int layer, const DecodePrep& p, const void* q, int q_dtype,
               int n_q_heads, float sm_scale, float* out, int n_splits, int64_t tps, float* ws, hipStream_t st,
               const StreamPlan* stream = nullptr) {
  if (stream)
    return decode_launch(sessions, n_sessions, layer, p, q, q_dtype, n_q_heads, sm_scale, n_splits, tps, true, ws, out,
                         st, false, true, stream);
  int32_t n_valid[kMaxSessions];
  decode_valid(p, n_sessions, tps, n_valid);
  const bool compact = decode_compact(n_sessions, n_splits, n_valid);
  const bool repeated = n_splits > 1 && repeated_cache(sessions, n_sessions);
  int rc = decode_launch(sessions, n_sessions, layer, p, q, q_dtype, n_q_heads, sm_scale, n_splits, tps, n_splits > 1,
                         ws, out, st, compact, /*fused=*/!repeated);
  if (rc || !repeated) return rc;
  hipError_t e = merge_launch(ws, (int64_t)n_sessions * n_q_heads, n_splits, p.d, out, st,
                              compact ? n_q_heads : 0, compact ? n_valid : nullptr);
  if (e != hipSuccess) {
    for (int i = 0; i < n_sessions; ++i) sessions[i]->poisoned = true;
    return fail(KV_EHIP, "merge launch: %s", hipGetErrorString(e));
  }
  return KV_OK;
}

}  // namespace

extern "C" {

int64_t kv_decode_workspace_bytes(kv_cache* const* sessions, int n_sessions, int layer, int n_q_heads) {
  clear_err();
  DecodePrep p;
  int rc = decode_prepare(sessions, n_sessions, layer, n_q_heads, false, &p);
  if (rc) return rc;
  // no plan splits a context finer than kDecodeWaveTokens, so the splits are also bounded by
  // the sessions' capacities (still a function of shapes only: a workspace sized once keeps
  // fitting as the caches grow)
  int64_t by_capacity = 1;
  for (int i = 0; i < n_sessions; ++i)
    by_capacity = std::max(by_capacity, ceil_div(sessions[i]->max_tokens, kDecodeWaveTokens));
  const int64_t cap = std::min(decode_split_cap(p), by_capacity);
  if (cap <= 1) return 0;
  return (int64_t)n_sessions * n_q_heads * cap * (p.d + 2) * (int64_t)sizeof(float);
}

int kv_decode_plan(kv_cache* const* sessions, int n_sessions, int layer, int n_q_heads, int* n_splits,
                   int64_t* tokens_per_split) {
  clear_err();
  if (!n_splits || !tokens_per_split) return fail(KV_EINVAL, "n_splits and tokens_per_split must not be NULL");
  DecodePrep p;
  int rc = decode_prepare(sessions, n_sessions, layer, n_q_heads, true, &p);
  if (rc) return rc;
  decode_plan(p, n_splits, tokens_per_split);
  return KV_OK;
}

int kv_attend_decode(kv_cache* const* sessions, int n_sessions, int layer, const void* q,
                     int q_dtype, int n_q_heads, float sm_scale, float* out, void* workspace,
                     size_t ws_bytes, void* stream) {
  clear_err();
  DecodePrep p;
  int rc = decode_prepare(sessions, n_sessions, layer, n_q_heads, true, &p);
  if (rc) return rc;
  if ((rc = check_q_out(q, q_dtype, out, "out"))) return rc;
  int n_splits;
  int64_t tps;
  decode_plan(p, &n_splits, &tps);
  StreamPlan sp;
  const bool streamed = workspace && decode_stream(sessions, n_sessions, p, q_dtype, n_q_heads, n_splits, tps, (int64_t)ws_bytes, &sp);
  const int64_t need = n_splits > 1 ? partial_bytes(n_sessions * (int64_t)n_q_heads, streamed ? sp.max_seg : n_splits, p.d) : 0;
  if ((rc = check_workspace(workspace, ws_bytes, need))) return rc;
  return decode_run(sessions, n_sessions, layer, p, q, q_dtype, n_q_heads, sm_scale, out, n_splits, tps,
                    static_cast<float*>(workspace), static_cast<hipStream_t>(stream), streamed ? &sp : nullptr);
}

int kv_decode_launch_kind(kv_cache* const* sessions, int n_sessions, int layer, int q_dtype, int n_q_heads,
                          size_t ws_bytes) {
  clear_err();
  DecodePrep p;
  int rc = decode_prepare(sessions, n_sessions, layer, n_q_heads, true, &p);
  if (rc) return rc;
  if (!dtype_ok(q_dtype)) return fail(KV_EINVAL, "q_dtype %d is not one of KV_F32/KV_BF16/KV_F16", q_dtype);
  int n_splits;
  int64_t tps;
  decode_plan(p, &n_splits, &tps);
  StreamPlan sp;
  return decode_stream(sessions, n_sessions, p, q_dtype, n_q_heads, n_splits, tps, (int64_t)ws_bytes, &sp) ? 1 : 0;
}

int kv_attend_decode_static(kv_cache* const* sessions, int n_sessions, int layer, const void* q,
                            int q_dtype, int n_q_heads, float sm_scale, float* out, void* stream) {
  clear_err();
  DecodePrep p;
  int rc = decode_prepare(sessions, n_sessions, layer, n_q_heads, true, &p);
  if (rc) return rc;
  if ((rc = check_q_out(q, q_dtype, out, "out"))) return rc;
  int n_splits;
  int64_t tps;
  decode_plan(p, &n_splits, &tps);
  StreamPlan sp;
  const bool streamed = decode_stream(sessions, n_sessions, p, q_dtype, n_q_heads, n_splits, tps, (int64_t)kStaticScratchBytes, &sp);
  const int64_t need = n_splits > 1 ? partial_bytes(n_sessions * (int64_t)n_q_heads, streamed ? sp.max_seg : n_splits, p.d) : 0;
  if (need > (int64_t)kStaticScratchBytes)
    return fail(KV_EINVAL,
                "the split plan of this call (%d splits x %lld rows) needs %lld bytes of partials, more than the %lld "
                "bytes of static scratch; use kv_attend_decode with a workspace",
                n_splits, (long long)n_sessions * n_q_heads, (long long)need, (long long)kStaticScratchBytes);
  float* ws = nullptr;
  if (need > 0) {
    hipError_t e = static_scratch(p.device, &ws);
    if (e != hipSuccess) return fail(KV_EHIP, "static scratch lookup: %s", hipGetErrorString(e));
  }
  return decode_run(sessions, n_sessions, layer, p, q, q_dtype, n_q_heads, sm_scale, out, n_splits, tps, ws,
                    static_cast<hipStream_t>(stream), streamed ? &sp : nullptr);
}

int kv_attend_decode_partial(kv_cache* const* sessions, int n_sessions, int layer, const void* q,
                             int q_dtype, int n_q_heads, float sm_scale, int n_splits,
                             int64_t tokens_per_split, float* partials, size_t partials_bytes,
                             void* stream) {
  clear_err();
  DecodePrep p;
  int rc = decode_prepare(sessions, n_sessions, layer, n_q_heads, true, &p);
  if (rc) return rc;
  if ((rc = check_q_out(q, q_dtype, partials, "partials"))) return rc;
  if ((rc = check_split(n_splits, tokens_per_split, kDecodeWaveTokens, p.max_len, "tokens_per_split"))) return rc;
  const int64_t need = partial_bytes(n_sessions * (int64_t)n_q_heads, n_splits, p.d);
  if ((int64_t)partials_bytes < need)
    return fail(KV_EINVAL, "partials buffer of %zu bytes is smaller than the %lld needed", partials_bytes, (long long)need);
  return decode_launch(sessions, n_sessions, layer, p, q, q_dtype, n_q_heads, sm_scale, n_splits,
                       tokens_per_split, true, partials, nullptr, static_cast<hipStream_t>(stream));
}

int kv_merge_partials(const float* partials, int64_t rows, int n_splits, int head_dim, float* out,
                      void* stream) {
  clear_err();
  if (rows < 0) return fail(KV_EINVAL, "rows must be >= 0 (got %lld)", (long long)rows);
  if (n_splits < 1) return fail(KV_EINVAL, "n_splits must be >= 1 (got %d)", n_splits);
  if (head_dim < 1 || head_dim > (1 << 20)) return fail(KV_EINVAL, "head_dim %d out of range", head_dim);
  if (rows > (int64_t)4 * 0x7fffffff) return fail(KV_EUNSUPPORTED, "%lld rows exceed one launch", (long long)rows);
  if (rows == 0) return KV_OK;
  if (!partials || !out) return fail(KV_EINVAL, "partials and out must not be NULL");
  if (!aligned16(partials) || !aligned16(out)) return fail(KV_EINVAL, "partials and out must be 16-byte aligned");
  hipError_t e = merge_launch(partials, rows, n_splits, head_dim, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KV_EHIP, "merge launch: %s", hipGetErrorString(e));
  return KV_OK;
}

int64_t kv_chunk_workspace_bytes(const kv_cache* cache, int layer, int n_q_heads, int64_t n_new) {
  clear_err();
  ChunkPrep p;
  int rc = chunk_prepare(cache, layer, n_q_heads, n_new, false, &p);
  if (rc) return rc;
  return partial_bytes(n_new * n_q_heads, (int)chunk_split_cap(p), cache->d);
}

int kv_chunk_plan(const kv_cache* cache, int layer, int n_q_heads, int64_t n_new, int* n_splits,
                  int64_t* keys_per_split) {
  clear_err();
  if (!n_splits || !keys_per_split) return fail(KV_EINVAL, "n_splits and keys_per_split must not be NULL");
  ChunkPrep p;
  int rc = chunk_prepare(cache, layer, n_q_heads, n_new, true, &p);
  if (rc) return rc;
  chunk_plan(p, cache->d, n_splits, keys_per_split);
  return KV_OK;
}

int kv_attend_chunk(kv_cache* cache, int layer, const void* q, int q_dtype, int n_q_heads,
                    int64_t n_new, float sm_scale, float* out, void* workspace, size_t ws_bytes,
                    void* stream) {
  clear_err();
  ChunkPrep p;
  int rc = chunk_prepare(cache, layer, n_q_heads, n_new, true, &p);
  if (rc) return rc;
  if ((rc = check_q_out(q, q_dtype, out, "out"))) return rc;
  int n_splits;
  int64_t tps;
  chunk_plan(p, cache->d, &n_splits, &tps);
  const int64_t need = n_splits > 1 ? partial_bytes(n_new * n_q_heads, n_splits, cache->d) : 0;
  if ((rc = check_workspace(workspace, ws_bytes, need))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* ws = static_cast<float*>(workspace);
  if ((rc = chunk_launch(cache, layer, p, q, q_dtype, n_q_heads, n_new, sm_scale, n_splits, tps, n_splits > 1, ws,
                         out, st)))
    return rc;
  if (n_splits > 1) {
    hipError_t e = merge_launch(ws, n_new * n_q_heads, n_splits, cache->d, out, st);
    if (e != hipSuccess) return hip_fail(cache, e, "merge launch");
  }
  return KV_OK;
}

int kv_attend_chunk_partial(kv_cache* cache, int layer, const void* q, int q_dtype, int n_q_heads,
                            int64_t n_new, float sm_scale, int n_splits, int64_t keys_per_split,
                            float* partials, size_t partials_bytes, void* stream) {
  clear_err();
  ChunkPrep p;
  int rc = chunk_prepare(cache, layer, n_q_heads, n_new, true, &p);
  if (rc) return rc;
  if ((rc = check_q_out(q, q_dtype, partials, "partials"))) return rc;
  if ((rc = check_split(n_splits, keys_per_split, kChunkKeys, p.len, "keys_per_split"))) return rc;
  if (n_splits > 65535) return fail(KV_EUNSUPPORTED, "n_splits %d exceeds one launch (65535)", n_splits);
  const int64_t need = partial_bytes(n_new * n_q_heads, n_splits, cache->d);
  if ((int64_t)partials_bytes < need)
    return fail(KV_EINVAL, "partials buffer of %zu bytes is smaller than the %lld needed", partials_bytes, (long long)need);
  return chunk_launch(cache, layer, p, q, q_dtype, n_q_heads, n_new, sm_scale, n_splits, keys_per_split, true,
                      partials, nullptr, static_cast<hipStream_t>(stream));
}

}  // extern "C"
