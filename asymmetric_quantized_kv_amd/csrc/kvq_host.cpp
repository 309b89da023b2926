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
#include <string>
#include <vector>

using namespace kvq;

struct kv_cache {
  int layout, n_layers, hkv, d;
  int64_t max_tokens;
  int kbits, vbits;
  Geom g;
  uint8_t* arena;
  int64_t bytes;
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
  static const int tab[5][2] = {{16, 16}, {8, 8}, {8, 4}, {4, 8}, {4, 4}};
  if (layout < 0 || layout > 4) return false;
  *kb = tab[layout][0];
  *vb = tab[layout][1];
  return true;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
int64_t ceil_div(int64_t x, int64_t m) { return (x + m - 1) / m; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape check shared by kv_cache_create and kv_layout_footprint_bytes.
int check_shape(int layout, int n_layers, int n_kv_heads, int head_dim, int64_t max_tokens) {
  int kb, vb;
  if (!layout_bits(layout, &kb, &vb)) return fail(KV_EINVAL, "layout %d is not one of 0..4", layout);
  if (n_layers < 1) return fail(KV_EINVAL, "n_layers must be >= 1 (got %d)", n_layers);
  if (n_kv_heads < 1) return fail(KV_EINVAL, "n_kv_heads must be >= 1 (got %d)", n_kv_heads);
  if (head_dim < 32 || head_dim % 32) return fail(KV_EINVAL, "head_dim must be a positive multiple of 32 (got %d)", head_dim);
  if (max_tokens < 1 || max_tokens > (int64_t(1) << 31) - kGranule)
    return fail(KV_EINVAL, "max_tokens out of range (got %lld)", (long long)max_tokens);
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
int64_t resident_slots(int device, const void* kernel, int threads = 256) {
  static int cus[64];
  static std::vector<std::pair<const void*, int>> per_cu;
  std::lock_guard<std::mutex> lk(g_plan_mu);
  if (device < 0 || device >= 64) return 0;
  if (cus[device] == 0 && hipDeviceGetAttribute(&cus[device], hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) {
    (void)hipGetLastError();
    cus[device] = -1;
  }
  if (cus[device] <= 0) return 0;
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
  return (int64_t)cus[device] * n;
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
    if (c->layout != s0->layout || c->n_layers != s0->n_layers || c->hkv != s0->hkv || c->d != s0->d)
      return fail(KV_EINVAL, "session %d does not share (layout, n_layers, n_kv_heads, head_dim) with session 0", i);
    if (c->device != s0->device) return fail(KV_EINVAL, "session %d lives on another device", i);
  }
  if (layer < 0 || layer >= s0->n_layers) return fail(KV_EINVAL, "layer %d out of range [0, %d)", layer, s0->n_layers);
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

kv_cache* kv_cache_create(int layout, int n_layers, int n_kv_heads, int head_dim,
                          int64_t max_tokens) {
  clear_err();
  if (check_shape(layout, n_layers, n_kv_heads, head_dim, max_tokens)) return nullptr;
  if (head_dim != 64 && head_dim != 128) {
    fail(KV_EUNSUPPORTED, "head_dim %d is valid but only 64 and 128 are built", head_dim);
    return nullptr;
  }
  int kb, vb;
  layout_bits(layout, &kb, &vb);
  Geom g = make_geom(kb, vb, head_dim, max_tokens);
  int64_t bytes = (int64_t)n_layers * n_kv_heads * g.region();
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
  void* p = nullptr;
  e = hipMalloc(&p, (size_t)bytes);
  if (e != hipSuccess || !p) {
    (void)hipGetLastError();
    fail(KV_ENOMEM, "hipMalloc of %lld bytes failed: %s", (long long)bytes, hipGetErrorString(e));
    return nullptr;
  }
  e = hipMemset(p, 0, (size_t)bytes);
  if (e != hipSuccess) {
    (void)hipFree(p);
    fail(KV_EHIP, "hipMemset: %s", hipGetErrorString(e));
    return nullptr;
  }
  kv_cache* c = new kv_cache;
  c->layout = layout;
  c->n_layers = n_layers;
  c->hkv = n_kv_heads;
  c->d = head_dim;
  c->max_tokens = max_tokens;
  c->kbits = kb;
  c->vbits = vb;
  c->g = g;
  c->arena = static_cast<uint8_t*>(p);
  c->bytes = bytes;
  c->len.assign(n_layers, 0);
  c->device = dev;
  c->poisoned = false;
  return c;
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
  const Geom& g = cache->g;
  const uint8_t* region = cache->arena + ((int64_t)layer * cache->hkv + kv_head) * g.region();
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

int kv_cache_copy_plane(const kv_cache* cache, int layer, int kv_head, int plane, int64_t row0,
                        int64_t n_rows, void* dst, void* stream) {
  const void* p = nullptr;
  int64_t rb = 0;
  int rc = kv_cache_plane(cache, layer, kv_head, plane, &p, &rb);
  if (rc) return rc;
  if (!dst) return fail(KV_EINVAL, "dst is NULL");
  if (row0 < 0 || n_rows < 0 || row0 + n_rows > cache->g.cap)
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
  if (cache->len[layer] + n_new > cache->max_tokens)
    return fail(KV_ECAPACITY, "append of %lld tokens to layer %d (len %lld) exceeds max_tokens %lld",
                (long long)n_new, layer, (long long)cache->len[layer], (long long)cache->max_tokens);
  if (n_new == 0) return KV_OK;
  if (!k || !v) return fail(KV_EINVAL, "k and v must not be NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(KV_EINVAL, "k and v must be 16-byte aligned");
  AppendArgs a;
  a.src[0] = k;
  a.src[1] = v;
  a.layer_base = cache->arena + (int64_t)layer * cache->hkv * cache->g.region();
  a.g = cache->g;
  a.t0 = cache->len[layer];
  a.n = n_new;
  a.hkv = cache->hkv;
  hipError_t e = launch_append(a, cache->kbits, cache->vbits, dtype, cache->d, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(cache, e, "append launch");
  cache->len[layer] += n_new;
  return KV_OK;
}

int64_t kv_decode_workspace_bytes(kv_cache* const* sessions, int n_sessions, int layer, int n_q_heads) {
  clear_err();
  int rc = check_sessions(sessions, n_sessions, layer);
  if (rc) return rc;
  const kv_cache* s0 = sessions[0];
  if (n_q_heads < 1 || n_q_heads % s0->hkv)
    return fail(KV_EINVAL, "n_q_heads %d is not a positive multiple of n_kv_heads %d", n_q_heads, s0->hkv);
  const int gp = decode_group_pad(n_q_heads / s0->hkv);
  if (gp < 0) return fail(KV_EUNSUPPORTED, "decode group size %d > 16 is not built", n_q_heads / s0->hkv);
  const int64_t base = (int64_t)n_sessions * s0->hkv;
  const int64_t slots = resident_slots(s0->device, decode_kernel_for(s0->kbits, s0->vbits, s0->d, gp));
  const int64_t cap = split_cap(base, slots, 1 << 20);
  if (cap <= 1) return 0;
  return (int64_t)n_sessions * n_q_heads * cap * (s0->d + 2) * (int64_t)sizeof(float);
}

int kv_attend_decode(kv_cache* const* sessions, int n_sessions, int layer, const void* q,
                     int q_dtype, int n_q_heads, float sm_scale, float* out, void* workspace,
                     size_t ws_bytes, void* stream) {
  clear_err();
  int rc = check_sessions(sessions, n_sessions, layer);
  if (rc) return rc;
  const kv_cache* s0 = sessions[0];
  const int hkv = s0->hkv, d = s0->d;
  if (n_q_heads < 1 || n_q_heads % hkv)
    return fail(KV_EINVAL, "n_q_heads %d is not a positive multiple of n_kv_heads %d", n_q_heads, hkv);
  const int group = n_q_heads / hkv;
  const int gp = decode_group_pad(group);
  if (gp < 0) return fail(KV_EUNSUPPORTED, "decode group size %d > 16 is not built", group);
  if (!dtype_ok(q_dtype)) return fail(KV_EINVAL, "q_dtype %d is not one of KV_F32/KV_BF16/KV_F16", q_dtype);
  if (!q || !out) return fail(KV_EINVAL, "q and out must not be NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(KV_EINVAL, "q and out must be 16-byte aligned");
  int64_t max_len = 0;
  for (int i = 0; i < n_sessions; ++i) {
    if (sessions[i]->len[layer] == 0) return fail(KV_EEMPTY, "session %d has no cached token in layer %d", i, layer);
    max_len = std::max(max_len, sessions[i]->len[layer]);
  }
  const int64_t base = (int64_t)n_sessions * hkv;
  const int64_t slots = resident_slots(s0->device, decode_kernel_for(s0->kbits, s0->vbits, d, gp));
  int n_splits;
  int64_t tps;
  plan_splits(base, slots, split_cap(base, slots, 1 << 20), max_len, kDecodeWaveTokens, kDecodeWaveTokens,
              &n_splits, &tps);
  int64_t need = n_splits > 1 ? (int64_t)n_sessions * n_q_heads * n_splits * (d + 2) * (int64_t)sizeof(float) : 0;
  if ((int64_t)ws_bytes < need) return fail(KV_EINVAL, "workspace of %zu bytes is smaller than the %lld needed", ws_bytes, (long long)need);
  if (need && (!workspace || !aligned16(workspace))) return fail(KV_EINVAL, "workspace must be a 16-byte aligned device pointer");

  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.hkv = hkv;
  a.hq = n_q_heads;
  a.group = group;
  a.n_splits = n_splits;
  a.tps = tps;
  a.q = q;
  a.q_dtype = q_dtype;
  a.qk_scale = sm_scale * 1.4426950408889634f;
  a.ws = static_cast<float*>(workspace);
  a.out = out;
  a.kc = s0->g.kc;
  a.ks = s0->g.ks;
  a.vc = s0->g.vc;
  a.vs = s0->g.vs;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int b0 = 0; b0 < n_sessions; b0 += kMaxSessions) {
    int nb = std::min(kMaxSessions, n_sessions - b0);
    a.n_sess = nb;
    a.sess0 = b0;
    for (int i = 0; i < nb; ++i) {
      const kv_cache* c = sessions[b0 + i];
      a.sess[i].base = c->arena + (int64_t)layer * hkv * c->g.region();
      a.sess[i].cap = c->g.cap;
      a.sess[i].len = c->len[layer];
    }
    hipError_t e = launch_decode(a, s0->kbits, s0->vbits, d, gp, st);
    if (e != hipSuccess) {
      for (int i = 0; i < n_sessions; ++i) sessions[i]->poisoned = true;
      return fail(KV_EHIP, "decode launch: %s", hipGetErrorString(e));
    }
  }
  if (n_splits > 1) {
    MergeArgs m;
    m.ws = a.ws;
    m.out = out;
    m.rows = (int64_t)n_sessions * n_q_heads;
    m.n_splits = n_splits;
    m.d = d;
    hipError_t e = launch_merge(m, st);
    if (e != hipSuccess) {
      for (int i = 0; i < n_sessions; ++i) sessions[i]->poisoned = true;
      return fail(KV_EHIP, "merge launch: %s", hipGetErrorString(e));
    }
  }
  return KV_OK;
}

int64_t kv_chunk_workspace_bytes(const kv_cache* cache, int layer, int n_q_heads, int64_t n_new) {
  clear_err();
  int rc = check_cache(cache);
  if (rc) return rc;
  if (layer < 0 || layer >= cache->n_layers) return fail(KV_EINVAL, "layer %d out of range", layer);
  if (n_q_heads < 1 || n_q_heads % cache->hkv)
    return fail(KV_EINVAL, "n_q_heads %d is not a positive multiple of n_kv_heads %d", n_q_heads, cache->hkv);
  if (n_new < 1) return fail(KV_EINVAL, "n_new must be >= 1");
  int64_t rows = n_new * (n_q_heads / cache->hkv);
  int64_t base = ceil_div(rows, kChunkRows) * cache->hkv;
  const int64_t slots = resident_slots(cache->device, chunk_kernel_for(cache->kbits, cache->vbits, cache->d, false),
                                       kChunkThreads);
  int64_t cap = split_cap(base, slots, kMaxSplitsChunk);
  if (cap <= 1) return 0;
  return n_new * n_q_heads * cap * (cache->d + 2) * (int64_t)sizeof(float);
}

int kv_attend_chunk(kv_cache* cache, int layer, const void* q, int q_dtype, int n_q_heads,
                    int64_t n_new, float sm_scale, float* out, void* workspace, size_t ws_bytes,
                    void* stream) {
  clear_err();
  int rc = check_cache(cache);
  if (rc) return rc;
  if (layer < 0 || layer >= cache->n_layers) return fail(KV_EINVAL, "layer %d out of range [0, %d)", layer, cache->n_layers);
  if (n_q_heads < 1 || n_q_heads % cache->hkv)
    return fail(KV_EINVAL, "n_q_heads %d is not a positive multiple of n_kv_heads %d", n_q_heads, cache->hkv);
  if (!dtype_ok(q_dtype)) return fail(KV_EINVAL, "q_dtype %d is not one of KV_F32/KV_BF16/KV_F16", q_dtype);
  const int64_t len = cache->len[layer];
  if (len == 0) return fail(KV_EEMPTY, "layer %d has no cached token", layer);
  if (n_new < 1 || n_new > len)
    return fail(KV_EINVAL, "n_new %lld must be in [1, len = %lld] (append the chunk first)", (long long)n_new, (long long)len);
  if (!q || !out) return fail(KV_EINVAL, "q and out must not be NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(KV_EINVAL, "q and out must be 16-byte aligned");
  const int group = n_q_heads / cache->hkv;
  const int64_t rows = n_new * group;
  const int64_t mtiles = ceil_div(rows, kChunkRows);
  if (mtiles > 0x7fffffff) return fail(KV_EUNSUPPORTED, "chunk of %lld rows is too large", (long long)rows);
  const int64_t base = mtiles * cache->hkv;
  const int64_t slots = resident_slots(cache->device, chunk_kernel_for(cache->kbits, cache->vbits, cache->d, false),
                                       kChunkThreads);
  int n_splits;
  int64_t tps;
  plan_splits(base, slots, split_cap(base, slots, kMaxSplitsChunk), len, kChunkKeys, kChunkMinKeysPerSplit,
              &n_splits, &tps);
  int64_t need = n_splits > 1 ? n_new * n_q_heads * n_splits * (cache->d + 2) * (int64_t)sizeof(float) : 0;
  if ((int64_t)ws_bytes < need) return fail(KV_EINVAL, "workspace of %zu bytes is smaller than the %lld needed", ws_bytes, (long long)need);
  if (need && (!workspace || !aligned16(workspace))) return fail(KV_EINVAL, "workspace must be a 16-byte aligned device pointer");

  ChunkArgs a;
  a.base = cache->arena + (int64_t)layer * cache->hkv * cache->g.region();
  a.g = cache->g;
  a.len = len;
  a.n_new = n_new;
  a.hkv = cache->hkv;
  a.hq = n_q_heads;
  a.group = group;
  a.n_splits = n_splits;
  a.tps = tps;
  a.q = q;
  a.q_dtype = q_dtype;
  a.qk_scale = sm_scale * 1.4426950408889634f;
  a.ws = static_cast<float*>(workspace);
  a.out = out;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_chunk(a, cache->kbits, cache->vbits, cache->d, st);
  if (e != hipSuccess) return hip_fail(cache, e, "chunk launch");
  if (n_splits > 1) {
    MergeArgs m;
    m.ws = a.ws;
    m.out = out;
    m.rows = n_new * n_q_heads;
    m.n_splits = n_splits;
    m.d = cache->d;
    e = launch_merge(m, st);
    if (e != hipSuccess) return hip_fail(cache, e, "merge launch");
  }
  return KV_OK;
}

}  // extern "C"
