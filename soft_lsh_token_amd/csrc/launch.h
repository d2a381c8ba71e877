// Host-side launchers of the SOCKET kernels.  Arguments have been validated
// by the C ABI layer before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace socketlsh {

// Query heads per scorer (and dense) pass: the largest of 4, 2 and 1 that
// divides G = Hq / Hkv.  A KV row with more query heads is taken in
// G / pass_heads(G) passes ("sub-rows"): sub-row v of the B*Hkv*sub rows
// serves query heads b*Hq + (v % (Hkv*sub)) * pass_heads(G) + [0, pass_heads(G))
// and reads KV row v / sub.
inline int pass_heads(int G) { return G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1; }
inline int pass_subs(int G) { return G / pass_heads(G); }

hipError_t launch_hash_keys(const void* K, const void* V, int dtype, int B, int Hkv,
                            int64_t n_cap, const int32_t* pos0, int count, const void* W, int L,
                            int P, uint8_t* ids, float* vnorm, hipStream_t s);

struct ScoreWs {
  float* img;           // [B*Hkv][img_floats]  LDS images of the soft tables (soft mode)
  uint32_t* qcodes;     // [B*Hq][words per code]  query codes (hard mode; same region)
  int img_floats;
  uint32_t* hist;       // [B*Hq][kHistBins]
  uint32_t* counters;   // [B*Hq]  candidates gathered by the top-k scan
  uint32_t* bitmap;     // [B*Hq][words]  selection bitmap, words = ceil(n_cap/8192)*256
  uint2* cand;          // [B*Hq][n_cap]  top-k candidates (score bits, key)
  float* scores;        // [B*Hq][ns]  when the caller passes no score buffer
  float* usum;          // [B*Hq]  sums of the soft counts (sampling estimator)
  float* gsum;          // [B*Hq][ceil(n_cap/64)]  score sums of 64-key groups (estimator)
  float* epart;         // [B*Hq][kEstSlices][kHead]  estimator partial sums
  float* esz;           // [B*Hq][2]  estimator totals: score sum S, soft-count sum Z
  int64_t words;
  int64_t groups;       // ceil(n_cap / 64)
};

constexpr int kEstSlices = 32;  // at most 32 slices of 256 draws (8192 draws a head)

size_t score_ws_layout(int B, int Hq, int Hkv, int64_t n_cap, int L, ScoreWs* ws, void* base);

// The selection workspace behind a first region of first_bytes (table images
// or query codes): histograms, counters, bitmaps, candidates, scores.
size_t select_ws_layout(size_t first_bytes, int B, int Hq, int64_t n_cap, ScoreWs* ws,
                        void* base);

// A key to hash while the tables are built: position lens[b] - 1 of every KV
// row (K == nullptr: none).
struct AppendKey {
  const void* K = nullptr;
  const void* V = nullptr;
  const int32_t* lens = nullptr;
  uint8_t* ids = nullptr;
  float* vnorm = nullptr;
  int64_t n_cap = 0;
};

// Algorithm 2, part 1: the soft tables of every query head, written as the
// scorer's LDS images; clears the selection histograms and counters.
// Optionally hashes the key appended at lens[b] - 1 (Algorithm 1 for one key).
hipError_t launch_soft_tables(const void* q, int dtype, int B, int Hq, int Hkv, const void* W,
                              int L, int P, float tau, const ScoreWs& ws, hipStream_t s,
                              AppendKey ak = AppendKey{});

// Keys always selected besides the top-k: the first `sink` and the last
// `window` keys of each sequence.
struct SinkWindow {
  int sink, window;
};

// Algorithm 2, part 2: scores of every key plus the first-digit histogram of
// the keys that compete for the top-k.
hipError_t launch_score(int B, int Hq, int Hkv, int L, int P, const uint8_t* ids,
                        const float* vnorm, const int32_t* lens, int64_t n_cap, SinkWindow sw,
                        float* scores, bool soft_sums, const ScoreWs& ws, hipStream_t s);

// The value-aware sampling estimator T(q) from the scores and soft-count sums
// left in the workspace by launch_score(..., soft_sums = true).
hipError_t launch_estimate(const float* scores, const float* vnorm, const void* V, int dtype,
                           int B, int Hq, int Hkv, const int32_t* lens, int64_t n_cap,
                           const float* u, int M, float* out, int32_t* draws, const ScoreWs& ws,
                           hipStream_t s);

// The attention a selection may be followed by (socket_decode_step): query,
// K and V of the step, their dtype, KV heads, scale and output.
struct AttendSpec {
  const void* q;
  const void* K;
  const void* V;
  int dtype;
  int Hkv;
  float scale;
  float* out;
};

// Algorithm 3: top-k selection from the scores and their histogram, united
// with the sink and window keys.  With att, the selecting workgroups also run
// each head's attention over its selection when the sizes allow it; then
// *attended is set and no separate attention launch is needed.
hipError_t launch_topk(int B, int Hq, const float* scores, const int32_t* lens, int64_t n_cap,
                       const int32_t* ks, int k_max, SinkWindow sw, int32_t* idx,
                       const ScoreWs& ws, hipStream_t s, const AttendSpec* att = nullptr,
                       bool* attended = nullptr, float* part = nullptr, int part_splits = 0);

// Key ranges of the decode step's selection + attention by range: 256-key
// blocks a range, and ranges (attention splits) a row of n_cap keys.
int range_blocks(int64_t n_cap);
int range_splits(int64_t n_cap);

// Hard-LSH comparison mode: packed sign codes of the L*P planes per key,
// stored word-major: codes[(b*Hkv + h) * words + w][n_cap].
int codes_words(int L, int P);  // 32-bit words per code: ceil(L*P / 32)

hipError_t launch_hash_codes_mfma(const uint16_t* K, const uint16_t* V, int B, int Hkv,
                                  int64_t n_cap, const int32_t* pos0, int count,
                                  const uint16_t* W, int LP, int WPK, uint32_t* codes,
                                  float* vnorm, hipStream_t s);
hipError_t launch_hash_codes(const void* K, const void* V, int dtype, int B, int Hkv,
                             int64_t n_cap, const int32_t* pos0, int count, const void* W, int L,
                             int P, uint32_t* codes, float* vnorm, hipStream_t s);

hipError_t launch_hard_score(const void* q, int dtype, int B, int Hq, int Hkv, const void* W,
                             int L, int P, const uint32_t* codes, const float* vnorm,
                             const int32_t* lens, int64_t n_cap, SinkWindow sw, float* scores,
                             const ScoreWs& ws, hipStream_t s);

struct DecodeWs {
  float* part;          // [B*Hq][splits][kHead + 2]
  int splits;
};

// min_splits: partials reserved per head beyond ceil(k_max / kSplitKeys).
size_t decode_ws_layout(int B, int Hq, int k_max, DecodeWs* ws, void* base, int min_splits = 0);

hipError_t launch_sparse_decode(const void* q, const void* K, const void* V, int dtype, int B,
                                int Hq, int Hkv, int64_t n_cap, const int32_t* idx, int k_max,
                                float scale, float* out, const DecodeWs& ws, hipStream_t s);

// Merge per-split partials [heads][splits][kHead + 2] (o, m, l) into out.
hipError_t launch_decode_combine(const float* part, int heads, int splits, float* out,
                                 hipStream_t s);

struct DenseWs {
  float* part;          // [B*Hq][splits][kHead + 2]
  int splits, chunk;    // splits of `chunk` keys each
};

size_t dense_ws_layout(int B, int Hq, int Hkv, int64_t n_cap, DenseWs* ws, void* base);

// Full attention over keys [0, lens[b]) of every query head (GQA groups of
// 1, 2 or 4 query heads per KV head).
hipError_t launch_dense_decode(const void* q, const void* K, const void* V, int dtype, int B,
                               int Hq, int Hkv, int64_t n_cap, const int32_t* lens, float scale,
                               float* out, const DenseWs& ws, hipStream_t s);

}  // namespace socketlsh
