/*
 * kvq.h -- C ABI of the asymmetric quantized session KV cache for gfx950 (MI355X).
 *
 * A session cache keeps every token's keys and values between turns so that a new
 * turn only processes its new tokens ("Reutilizacao de Cache KV para Conversas Longas
 * no Apple Silicon Oferece Aceleracao de 200x", openclawradar.com, section "Principais
 * Descobertas e Benchmarks").  Keys and values are stored with different bit widths
 * ("KVSplit -- contexto 2 a 3 vezes mais longo em Apple Silicon", pt.news.hada.io
 * topic 20969, sections "Principais resultados de benchmark" and "Assimetria entre key
 * e value"), quantized when the tokens are written, independently of the model weights
 * (same page, section "Opinioes no Hacker News").
 *
 * Storage format (the pages print footprints, not a format; this one reproduces every
 * footprint the KVSplit page prints, section "Uso de memoria conforme o comprimento da
 * sequencia"):
 *   - per (token, KV head), head_dim is cut into blocks of 32 consecutive elements;
 *   - 8-bit and 4-bit blocks carry one fp16 scale d = fp16_rne(fp32(amax / qmax)),
 *     qmax = 127 or 7, saturated at 65504; codes q = clamp(round_half_away(fp32(x / d)),
 *     -qmax, qmax), all zero when d == 0;
 *   - 8-bit codes are int8 (two's complement); 4-bit codes are nibbles u = q + 8, byte j
 *     of a block = u[2j] | u[2j+1] << 4; the FP16 layout stores fp16_rne(x), no scale;
 *   - fp8 keys (KV_KF8V4) are OCP "MX" blocks: the offloading page ("KV Cache
 *     Offloading for Context-Intensive Tasks", section "2. Metodologia", its fourth item)
 *     names FP8 KV storage without fixing a format, and gfx950 converts OCP E4M3 in
 *     hardware.  Per 32-element block one exponent byte s = e + 127 with
 *     e = clamp(floor(log2(amax)) - 8, -127, 127) (-127 for an all-zero block), and per
 *     element the E4M3 code (bias 7, largest 448, no infinities) of x * 2^-e rounded to
 *     nearest, ties to even, saturated at +-448; a result of zero is stored as +0.
 *     x_hat = E4M3 value * 2^(s - 127).  Decode, and the chunk path with fp16 or fp32
 *     queries, widen these keys to fp16 (exactly while |x| < 65536: the fp16 control
 *     layout's range); the chunk path with bf16 queries multiplies them as they are, on
 *     the MX-fp8 matrix instructions;
 *   - planes per (layer, KV head), token-major: KC [cap][code bytes], KS [cap][scale
 *     bytes] (2*D/32 for fp16 scales, D/32 for exponent bytes), VC, VS; cap = max_tokens
 *     rounded up to 256 tokens (the KVSplit page's remark on 256-byte alignment, section
 *     "Otimizacao para Apple Silicon e limitacoes").
 *
 * Conventions for every entry point:
 *   - status: 0 (KV_OK) or a negative KV_E* code; kv_last_error() then holds a message
 *     (thread-local).  All argument checks happen on the host before any launch; on a
 *     check failure the cache is unchanged.  After a HIP error the cache is poisoned and
 *     every later call on it returns KV_EHIP until kv_cache_destroy.
 *   - device pointers (k, v, q, out, workspace) belong to the caller, must be 16-byte
 *     aligned, and must stay valid until the stream has passed the call.  The library
 *     owns the cache arena.
 *   - every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *     The cached length of a layer advances when kv_append_quant is enqueued.
 *   - a handle must not be used from two threads at once; handles are independent.
 *
 * Numerics of the attention calls (outputs are fp32, within 5e-3 of exact attention over
 * the dequantized cache on the tested workloads):
 *   - queries of any finite magnitude.  Decode with 8- and 4-bit keys carries each query
 *     head as q ~ s (256 hi + lo), s = max|q| / 32512 (integer digits): an absolute error
 *     of at most max|q| / 65024 per element, so a channel far larger than the rest leaves
 *     the rest that much resolution.  Decode with fp8 or fp16 keys and the chunk path
 *     scale the query by a power of two that puts its largest element (per head in
 *     decode, per 32 query rows in the chunk path) in [2^14, 2^15) and carry it in fp16:
 *     16-bit queries exactly, fp32 queries as an fp16 high and low part.  The chunk path
 *     with fp8 keys and bf16 queries splits each query element into two E4M3 parts with a
 *     power-of-two scale per 32-element block (exact but for elements below 2^-13 of their
 *     block's largest); its block-scaled products were measured less accurate than the
 *     fp16 ones: on the same inputs, 1.1 to 2.7 times the widened path's output error
 *     (worst tested 3.9e-3 against 1.5e-3, a softmax made peaked by keys growing 70-fold
 *     along the context; 0.7-1.8e-3 against 0.4-1.0e-3 on the other cases): the
 *     instruction keeps each product only down to 2^-14 of the largest one in its
 *     32-element block.
 *   - the chunk path carries dequantized keys and values in fp16 (keys as an fp16 high
 *     part plus a scaled 6- or 8-bit low part): their magnitudes must stay below 65504,
 *     or the outputs are not finite.  Decode takes 8- and 4-bit keys exactly (integer dot
 *     products, then the block scale) and applies value scales to fp16 weights p * d.
 *   - a NaN input element gives unspecified codes; an infinity saturates its block's scale
 *     at 65504 and takes the clamped code, as the format above gives.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define KV_OK            0
#define KV_EINVAL       -1   /* bad argument (null, range, alignment, shape mismatch)   */
#define KV_ECAPACITY    -2   /* append past max_tokens                                   */
#define KV_ENOMEM       -3   /* device allocation failed                                 */
#define KV_EUNSUPPORTED -4   /* valid but not built (head_dim other than 64/128, ...)    */
#define KV_EEMPTY       -5   /* attention over a layer with no cached token              */
#define KV_EHIP         -6   /* a HIP call failed; the cache is poisoned                 */

/* layouts: key bits x value bits (0..4: the five configurations the KVSplit page
 * compares; 5: fp8 keys, the FP8 alternative of the offloading page, with 4-bit values) */
#define KV_FP16  0
#define KV_K8V8  1
#define KV_K8V4  2
#define KV_K4V8  3
#define KV_K4V4  4
#define KV_KF8V4 5

/* element types of k, v, q */
#define KV_F32  0
#define KV_BF16 1
#define KV_F16  2

/* planes of one (layer, KV head) */
#define KV_PLANE_KC 0   /* key codes    */
#define KV_PLANE_KS 1   /* key scales   */
#define KV_PLANE_VC 2   /* value codes  */
#define KV_PLANE_VS 3   /* value scales */

typedef struct kv_cache kv_cache;

/* Create an empty session cache on the current HIP device.
 * layout: KV_FP16..KV_KF8V4.  n_layers >= 1, n_kv_heads >= 1, head_dim in {64, 128}
 * (other multiples of 32 up to 65536 -> KV_EUNSUPPORTED), 1 <= max_tokens <= 2^31 - 256,
 * and n_layers * n_kv_heads * round_up(max_tokens, 256) * 4 * head_dim <= 2^50 (KV_EINVAL
 * beyond: the arena size stays far from int64 overflow).
 * Allocates n_layers * n_kv_heads * round_up(max_tokens, 256) token rows, zero-filled.
 * Returns NULL on error (kv_last_error() says why; KV_ENOMEM if hipMalloc failed). */
kv_cache* kv_cache_create(int layout, int n_layers, int n_kv_heads, int head_dim,
                          int64_t max_tokens);

/* The same with a layout per layer: layer l stores its keys and values as layouts[l]
 * (layer-specific quantization, planned in the KVSplit page, section "Configuracao
 * recomendada e roadmap").
 * layouts: host array of n_layers layout codes.  Every entry point then works per layer
 * in that layer's layout; a decode call over several sessions needs them to share the
 * layer's layout.  Errors as kv_cache_create. */
kv_cache* kv_cache_create_layered(const int* layouts, int n_layers, int n_kv_heads, int head_dim,
                                  int64_t max_tokens);

/* Layout code of one layer; < 0 on bad arguments. */
int kv_cache_layout(const kv_cache* cache, int layer);

/* Shape of a cache as created: any of the out pointers may be NULL.  KV_EINVAL for a NULL
 * cache.  (Lets a binding check k, v, q and out against the cache before a call.) */
int kv_cache_shape(const kv_cache* cache, int* n_layers, int* n_kv_heads, int* head_dim,
                   int64_t* max_tokens);

/* Debugging aid: the arena carries 256 guard bytes of a fixed pattern after its planes, which
 * no kernel writes.  Waits for the device to finish all queued work, reads them back and
 * returns KV_OK if they are intact, KV_EINVAL (with the first changed byte in
 * kv_last_error) if something wrote past the planes, KV_EHIP if the read failed. */
int kv_cache_check_guard(const kv_cache* cache);

/* Free the arena.  The caller ensures no queued work still uses the cache.  NULL is a no-op. */
void kv_cache_destroy(kv_cache* cache);

/* Quantize n_new tokens and write them at rows [len, len + n_new) of `layer`
 * (quantize-on-append; the KVSplit page, section "Opinioes no Hacker News").
 * k, v: device, [n_new][n_kv_heads][head_dim] contiguous, element type `dtype`.
 * Errors: KV_EINVAL (null cache/pointer, layer out of range, n_new < 0, bad dtype,
 * misaligned pointer), KV_ECAPACITY (len + n_new > max_tokens), KV_EHIP.
 * n_new == 0 is a no-op. */
int kv_append_quant(kv_cache* cache, int layer, const void* k, const void* v, int dtype,
                    int64_t n_new, void* stream);

/* Single-query attention for each of n_sessions caches over all of their cached tokens
 * of `layer`: out[s][h] = softmax(sm_scale * q[s][h] . K_s^T) V_s, with q head h reading
 * KV head h / (n_q_heads / n_kv_heads).  The dense definition of attention over the
 * dequantized cache; the pages discuss where it is bound (KVSplit page, "Opinioes no
 * Hacker News": the gain comes from memory traffic).
 * sessions: host array of n_sessions handles sharing (layout, n_layers, n_kv_heads,
 * head_dim); their lengths may differ.  q: device [n_sessions][n_q_heads][head_dim] of
 * q_dtype.  out: device fp32, same shape.  workspace: device scratch of at least
 * kv_decode_workspace_bytes(...) bytes (may be NULL when that is 0).
 * Launch: the split plan of kv_decode_plan, its partials merged in the same launch (in a
 * second launch when a cache is passed twice); or, for
 * 2..64 sessions of uneven lengths (the plan would leave some session's later splits empty),
 * no cache passed twice, at most 128 resident workgroups per KV head (4 or more KV heads at
 * two workgroups per compute unit) and a workspace that holds its partials, a
 * streamed launch: the sessions' 512-token blocks, longest session first and laid end to
 * end, are cut into one range per resident workgroup of each KV head (balancing blocks plus a
 * fixed cost per session part), and a session that several ranges overlap is merged from
 * their partials.  Both compute the same attention to within rounding; each is deterministic.
 * Errors: KV_EINVAL (mismatched sessions, n_q_heads % n_kv_heads, group size > 16,
 * small workspace, null/misaligned pointers), KV_EEMPTY (a session with len == 0),
 * KV_EHIP. */
int kv_attend_decode(kv_cache* const* sessions, int n_sessions, int layer, const void* q,
                     int q_dtype, int n_q_heads, float sm_scale, float* out,
                     void* workspace, size_t ws_bytes, void* stream);

/* kv_attend_decode without a workspace and without any allocation, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  The split partials live in a static device array of the library
 * (16 MiB per device, held from module load until the process ends).  Same arguments,
 * launch and results as kv_attend_decode (bit for bit), except that a streamed launch whose
 * partials exceed 16 MiB gives way to the split plan here.  Errors as kv_attend_decode,
 * plus KV_EINVAL when the split plan's partials (n_splits * n_sessions * n_q_heads *
 * (head_dim + 2) * 4 bytes, see kv_decode_plan) exceed 16 MiB; a one-split plan needs none.
 * Every call on a device shares that device's array: calls that overlap on one device (on
 * different streams, or from different threads) race for it and must not be issued. */
int kv_attend_decode_static(kv_cache* const* sessions, int n_sessions, int layer, const void* q,
                            int q_dtype, int n_q_heads, float sm_scale, float* out, void* stream);

/* Which launch kv_attend_decode takes for these sessions, queries of q_dtype and a workspace
 * of ws_bytes: 0 = the split plan of kv_decode_plan, 1 = the streamed launch (see
 * kv_attend_decode); < 0 on bad arguments (as kv_attend_decode).  Host-only, no device work. */
int kv_decode_launch_kind(kv_cache* const* sessions, int n_sessions, int layer, int q_dtype,
                          int n_q_heads, size_t ws_bytes);

/* Workspace bytes kv_attend_decode needs for these sessions; < 0 on bad arguments.  It
 * depends only on shapes (n_sessions, n_q_heads, head_dim, the sessions' max_tokens, the
 * device), so a workspace sized once fits every later call on the same caches. */
int64_t kv_decode_workspace_bytes(kv_cache* const* sessions, int n_sessions, int layer,
                                  int n_q_heads);

/* The two passes of kv_attend_decode, callable one by one (to time or overlap them, or to
 * merge partials computed elsewhere, e.g. on several devices).
 *
 * kv_decode_plan: the split kv_attend_decode uses for these sessions (unless it takes the
 * streamed launch) -- the context is cut into *n_splits ranges of *tokens_per_split tokens
 * (a multiple of 512) covering the longest session.  Errors as kv_attend_decode (KV_EEMPTY
 * for an empty session).
 *
 * kv_attend_decode_partial: the first pass alone, with a split of the caller's choice
 * (1 <= n_splits <= 65535; tokens_per_split a positive multiple of 512 with n_splits *
 * tokens_per_split >= the longest session).  Split s of session b covers tokens
 * [s * tokens_per_split, min((s + 1) * tokens_per_split, len_b)).  Writes, per row
 * r = b * n_q_heads + h and split s, partials[(r * n_splits + s) * (head_dim + 2) + i]:
 *   i <  head_dim:  o_i = sum_t 2^(x_t - m) v_t,i   (not normalized)
 *   i == head_dim:  m,  the running max, max_t x_t - 8 <= m <= max_t x_t
 *   i == head_dim+1: l = sum_t 2^(x_t - m)
 * with x_t = sm_scale * log2(e) * q . k_t (base-2 units).  (o, m, l) is unique only up to
 * the common rescale m -> m', o, l -> o, l * 2^(m - m'); o / l and m + log2(l) are not.
 * A split with no token has m = -inf, l = 0, o = 0.  partials: device fp32 of at least
 * n_sessions * n_q_heads * n_splits * (head_dim + 2) * 4 bytes (partials_bytes).
 * The merge (below) of these partials is the attention of kv_attend_decode.
 * (The log-sum-exp recombination of softmax sums over disjoint key ranges; the pages
 * do not discuss splitting, which is an implementation choice for long contexts.) */
int kv_decode_plan(kv_cache* const* sessions, int n_sessions, int layer, int n_q_heads,
                   int* n_splits, int64_t* tokens_per_split);
int kv_attend_decode_partial(kv_cache* const* sessions, int n_sessions, int layer,
                             const void* q, int q_dtype, int n_q_heads, float sm_scale,
                             int n_splits, int64_t tokens_per_split, float* partials,
                             size_t partials_bytes, void* stream);

/* Second pass: out[r][i] = sum_s 2^(m_s - M) o_s,i / sum_s 2^(m_s - M) l_s with
 * M = max_s m_s over the n_splits partials of row r (layout as above); splits with
 * m = -inf drop out.  partials: device fp32 [rows][n_splits][head_dim + 2]; out: device
 * fp32 [rows][head_dim].  rows == 0 is a no-op.  The weights 2^(m_s - M) are fp32: a
 * split with m_s < M - 126 weighs nothing, which is exact to fp32 rounding for partials
 * as the partial passes write them (l >= 2^-8, |o_i| <= l max|v|).  Errors: KV_EINVAL
 * (null or misaligned pointers, n_splits < 1, head_dim out of range), KV_EHIP. */
int kv_merge_partials(const float* partials, int64_t rows, int n_splits, int head_dim,
                      float* out, void* stream);

/* Causal attention of the last n_new cached positions of `layer` (the turn just
 * appended) against everything cached so far: only the new tokens are processed
 * (openclawradar.com page, section "Principais Descobertas e Benchmarks").
 * Query row j sits at absolute position len - n_new + j and sees keys [0, that position],
 * its own chunk read back quantized from the cache.
 * q: device [n_new][n_q_heads][head_dim] of q_dtype; out: device fp32, same shape.
 * workspace: at least kv_chunk_workspace_bytes(...) bytes.
 * Errors: KV_EINVAL (n_new < 1 or > len, n_q_heads % n_kv_heads, small workspace,
 * null/misaligned pointers), KV_EEMPTY (len == 0), KV_EHIP. */
int kv_attend_chunk(kv_cache* cache, int layer, const void* q, int q_dtype, int n_q_heads,
                    int64_t n_new, float sm_scale, float* out, void* workspace,
                    size_t ws_bytes, void* stream);

/* Workspace bytes kv_attend_chunk needs; < 0 on bad arguments. */
int64_t kv_chunk_workspace_bytes(const kv_cache* cache, int layer, int n_q_heads,
                                 int64_t n_new);

/* The two passes of kv_attend_chunk, callable one by one.
 * kv_chunk_plan: the split kv_attend_chunk uses -- the cached keys [0, len) are cut into
 * *n_splits ranges of *keys_per_split keys (a multiple of 64).
 * kv_attend_chunk_partial: the first pass with a split of the caller's choice
 * (1 <= n_splits <= 65535; keys_per_split a positive multiple of 64 with n_splits *
 * keys_per_split >= len).  Query row j sees the keys of split s that are also in
 * [0, len - n_new + j].  Partials as for kv_attend_decode_partial with rows
 * r = j * n_q_heads + h; a row that sees no key of a split gets m = -inf, l = 0, o = 0.
 * kv_merge_partials turns them into the output of kv_attend_chunk. */
int kv_chunk_plan(const kv_cache* cache, int layer, int n_q_heads, int64_t n_new,
                  int* n_splits, int64_t* keys_per_split);
int kv_attend_chunk_partial(kv_cache* cache, int layer, const void* q, int q_dtype,
                            int n_q_heads, int64_t n_new, float sm_scale, int n_splits,
                            int64_t keys_per_split, float* partials, size_t partials_bytes,
                            void* stream);

/* Device bytes of all planes: n_layers * n_kv_heads * cap * (K row + V row), the footprint
 * the KVSplit page tabulates (section "Uso de memoria conforme o comprimento da sequencia").
 * < 0 for a NULL cache. */
int64_t kv_footprint_bytes(const kv_cache* cache);

/* The same footprint for a shape, without allocating (pure host arithmetic). < 0 if invalid
 * (the shape rules of kv_cache_create, except that any multiple of 32 up to 65536 is a
 * valid head_dim here). */
int64_t kv_layout_footprint_bytes(int layout, int n_layers, int n_kv_heads, int head_dim,
                                  int64_t max_tokens);

/* The footprint of a cache with a layout per layer: the sum of the layers' footprints. */
int64_t kv_layered_footprint_bytes(const int* layouts, int n_layers, int n_kv_heads, int head_dim,
                                   int64_t max_tokens);

/* Cached tokens of `layer` (as enqueued); < 0 on bad arguments. */
int64_t kv_cache_len(const kv_cache* cache, int layer);

/* Forget every cached token (lengths to 0; bytes are left as they are), for a full
 * rebuild after a cache miss (openclawradar.com page, "Principais Descobertas e
 * Benchmarks": a miss re-processes the whole context). */
int kv_cache_reset(kv_cache* cache);

/* Forget the tokens of `layer` at positions >= new_len (lengths only; bytes are left as
 * they are and are overwritten by the next append).  Rolls a session back to an earlier
 * turn, e.g. to re-run or discard the last turn.  KV_EINVAL if new_len is negative or
 * larger than the cached length. */
int kv_cache_truncate(kv_cache* cache, int layer, int64_t new_len);

/* Device address and row pitch of one plane of (layer, kv_head).  *ptr is NULL and
 * *row_bytes 0 for the scale planes of the FP16 layout. */
int kv_cache_plane(const kv_cache* cache, int layer, int kv_head, int plane,
                   const void** ptr, int64_t* row_bytes);

/* Copy rows [row0, row0 + n_rows) of a plane to dst (device or host memory, packed with
 * row pitch = row_bytes) on `stream`; synchronous when dst is pageable host memory. */
int kv_cache_copy_plane(const kv_cache* cache, int layer, int kv_head, int plane,
                        int64_t row0, int64_t n_rows, void* dst, void* stream);

/* Session offload and restore: the packed cache of a session leaves the GPU between turns
 * and comes back for the next one, so a cache hit costs a host-link transfer of the
 * quantized bytes instead of a re-prefill of the context (openclawradar.com page, "Principais
 * Descobertas e Benchmarks": sessions are kept between turns; "KV Cache Offloading for
 * Context-Intensive Tasks", gist.science: KV moved to host memory and reloaded on demand).
 *
 * Saved form: a 32-byte header (magic "KVQS", version 2, the layout of every layer or -1
 * when layers differ, n_layers, n_kv_heads, head_dim as 32-bit integers, 8 zero bytes), one
 * int64 cached length per layer, one int32 layout per layer, zero padding to a multiple of
 * 64 bytes, then for every layer and KV head the first len[layer] rows of the planes KC,
 * KS, VC, VS in that order (row bytes as kv_cache_plane reports).
 *
 * kv_session_bytes: size of that form for the cache as it stands; < 0 for a NULL cache.
 * kv_session_save: writes it to dst, which must be host memory (pinned memory from
 *   hipHostMalloc gives the full host-link rate; pageable memory makes the copies
 *   synchronous).  The header is written by the host during the call; the plane bytes
 *   land when `stream` passes the call.  The cache is unchanged.
 *   Errors: KV_EINVAL (NULL or device dst, dst_bytes too small), KV_EHIP.
 * kv_session_load: replaces the contents of `cache` with a saved session read from host
 *   memory src.  The header must match the cache's (n_layers, n_kv_heads, head_dim and
 *   every layer's layout).  Lengths take the saved values when the call is enqueued; rows past them
 *   are left as they are.
 *   Errors: KV_EINVAL (NULL or device src, bad magic or version, shape mismatch, src_bytes
 *   too small), KV_ECAPACITY (a saved length above max_tokens), KV_EHIP.  On an error
 *   the cache is unchanged. */
int64_t kv_session_bytes(const kv_cache* cache);
int kv_session_save(const kv_cache* cache, void* dst, size_t dst_bytes, void* stream);
int kv_session_load(kv_cache* cache, const void* src, size_t src_bytes, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* kv_last_error(void);

/* Status code of the last failed call on this thread (KV_OK if none); the way to get
 * the reason a kv_cache_create returned NULL. */
int kv_last_status(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
