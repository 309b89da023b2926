// Internal declarations shared by the host side of the C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace kvq {

constexpr int kBlock = 32;          // elements per quantization block
constexpr int kGranule = 256;       // capacity granule (tokens)
constexpr int kMaxSessions = 64;    // sessions per decode launch (kernel-argument table)
constexpr int kDecodeChunk = 128;   // tokens one wave scores before its softmax update
constexpr int kDecodeWaveTokens = 4 * kDecodeChunk;  // split granularity of decode
constexpr int kMaxHeadSplit = 2;    // decode workgroups per KV head at most (see DecodeArgs::hsplit)
constexpr int kMaxStreamWg = 128;   // workgroups per KV head of a streamed decode launch at most
constexpr int kChunkThreads = 768;  // threads per chunk-prefill workgroup: 8 consumer + 4 producer waves
constexpr int kChunkRows = 256;     // query rows per chunk-prefill workgroup (32 per consumer wave)
constexpr int kChunkKeys = 64;      // keys per chunk-prefill tile
constexpr uint32_t kXcds = 8;       // accelerator dies of an MI355X; workgroups are dealt round-robin

constexpr size_t kStaticScratchBytes = size_t(16) << 20;   // device scratch of kv_attend_decode_static

constexpr int kF8 = 9;              // "bits" marker of fp8 (E4M3) codes with power-of-two block scales

__host__ __device__ constexpr int code_row_bytes(int bits, int d) {
  return bits == 16 ? 2 * d : (bits == 8 || bits == kF8 ? d : d / 2);
}
__host__ __device__ constexpr int scale_row_bytes(int bits, int d) {
  return bits == 16 ? 0 : (bits == kF8 ? d / kBlock : 2 * (d / kBlock));
}

// Planes of one (layer, KV head) region, token-major, in this order: KC, KS, VC, VS.
struct Geom {
  int64_t cap;      // tokens per plane
  int32_t kc, ks, vc, vs;  // row bytes
  __host__ __device__ int64_t region() const { return cap * (int64_t)(kc + ks + vc + vs); }
  __host__ __device__ int64_t off_kc() const { return 0; }
  __host__ __device__ int64_t off_ks() const { return cap * (int64_t)kc; }
  __host__ __device__ int64_t off_vc() const { return cap * (int64_t)(kc + ks); }
  __host__ __device__ int64_t off_vs() const { return cap * (int64_t)(kc + ks + vc); }
};

struct AppendArgs {
  const void* src[2];     // k, v: [n][Hkv][D]
  uint8_t* layer_base;    // arena + layer * Hkv * region
  Geom g;
  int64_t t0;             // first row written
  int64_t n;              // tokens
  int hkv;
};

struct SessionRef {
  const uint8_t* base;    // arena + layer * Hkv * region of this session
  uint32_t* counters;     // fused launches: the session's split counters of the layer, kMaxHeadSplit per KV head
  int64_t cap;
  int64_t len;
  int32_t row;            // index of the session in the call (rows of q / out / workspace)
  int32_t piece0;         // compact launches: index of its first busy split among all sessions;
                          // streamed launches: index of its first token block among all sessions
  int32_t wfirst, nseg;   // streamed launches: the first workgroup (per KV head) whose block range
                          // overlaps the session, and how many do (its partials; 1: no merge)
};

struct DecodeArgs {
  // the scalars first: a workgroup's first kernel-argument loads then share one cache line
  int n_sess;             // sessions in this launch
  int hkv, hq, group;
  int n_splits;
  int partial;            // 1: write (o, m, l) partials to ws; 0: normalized out (n_splits == 1)
  // compact != 0: the grid holds only the workgroups with tokens, session by session: session
  // i's busy splits are pieces sess[i].piece0 .. + ceil(len / tps) - 1 of n_pieces; a split
  // past a session's end then has no workgroup and no partial
  int compact, n_pieces;
  // fused != 0 (with partial): the last workgroup of each (session, KV head) to finish merges
  // that head's partials into out, found with the session's split counter for the head (left
  // at zero between calls)
  int fused;
  // hsplit: workgroups per KV head (1 or kMaxHeadSplit = 2); workgroup part j of KV head h takes query
  // heads j * group .. (j + 1) * group - 1 of the head's group (group = the KV head's group /
  // hsplit), and grid x = hkv * hsplit
  int hsplit;
  // one_chunk != 0: tps <= kDecodeWaveTokens (each wave holds at most one chunk) and the grid
  // fits the device at one workgroup per compute unit
  int one_chunk;
  // stream != 0 (fused, one launch): the sessions' token blocks of kDecodeWaveTokens, laid end
  // to end in session order, are cut into n_wg ranges, one per workgroup of each KV head (grid
  // y): workgroup w takes blocks [wg_block0[w], wg_block0[w + 1]), the part of every session
  // that range overlaps, all workgroups in one round
  int stream, n_wg;
  int q_dtype;
  int64_t tps;            // tokens per split, multiple of kDecodeWaveTokens
  const void* q;
  float qk_scale;         // sm_scale * log2(e)
  float* ws;              // [S][Hq][n_splits][D + 2] partials when partial
  float* out;             // [S][Hq][D] otherwise
  SessionRef sess[kMaxSessions];
  int32_t wg_block0[kMaxStreamWg + 1];
};

struct ChunkArgs {
  const uint8_t* base;    // arena + layer * Hkv * region
  Geom g;
  int64_t len;            // cached tokens (the chunk is the last n_new of them)
  int64_t n_new;
  int hkv, hq, group;
  int n_splits;
  int partial;            // 1: write (o, m, l) partials to ws; 0: normalized out (n_splits == 1)
  int64_t tps;            // keys per split, multiple of kChunkKeys
  const void* q;
  int q_dtype;
  float qk_scale;
  float* ws;              // [n_new][Hq][n_splits][D + 2] partials when partial
  float* out;             // [n_new][Hq][D] otherwise
};

struct MergeArgs {
  const float* ws;        // [rows][n_splits][D + 2]: o (unnormalized), m (log2 units), l
  float* out;             // [rows][D]
  int64_t rows;
  int n_splits;
  int d;
  // rows_per_sess > 0: row r belongs to session r / rows_per_sess, whose partials are its first
  // n_valid[session] splits only (the others were never written)
  int rows_per_sess;
  int32_t n_valid[kMaxSessions];
};

// Launchers (one per translation unit).  They return hipErrorInvalidValue for a
// combination that is not instantiated.
hipError_t launch_append(const AppendArgs& a, int kbits, int vbits, int dtype, int d,
                         hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int kbits, int vbits, int d, int gp,
                         hipStream_t s);
hipError_t launch_chunk(const ChunkArgs& a, int kbits, int vbits, int d, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);

// Device address of the library's static scratch (kStaticScratchBytes) on `device`, looked up
// once per device and kept.
hipError_t static_scratch(int device, float** ptr);

// Kernel symbols, for occupancy queries by the split planner.
// stream: the streamed variant; q_fp32: with fp32 queries (which carry a low part for fp16 and
// fp8 keys in that variant)
const void* decode_kernel_for(int kbits, int vbits, int d, int gp, bool stream = false, bool q_fp32 = false);
const void* chunk_kernel_for(int kbits, int vbits, int d, bool q_fp32);

}  // namespace kvq
