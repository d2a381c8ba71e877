// C ABI of the SOCKET decode path: argument checks, workspace sizing and
// dispatch to the kernels.  Every check happens before anything is enqueued.
#include "../../include/socket_lsh.h"
#include "common.h"
#include "launch.h"

using namespace socketlsh;

namespace {

constexpr int kMaxL = 128;       // 16 ID words of at most 8 tables each
constexpr int kMaxScoreL = 128;
constexpr int kMaxKmax = 1 << 16;  // 1024 attention splits of 64 keys
constexpr int kMaxRangeSplits = 1024;  // key ranges a row at most (the merge's limit)
constexpr int kMaxCodeBits = 4096;  // hard-LSH mode: L * P
constexpr int kMaxGroup = 64;       // query heads per KV head
constexpr int kMaxDraws = 8192;     // sampling estimator: draws per query head

// Table shapes with an ID layout: one-byte IDs (P <= 8) for up to 128
// tables, two-byte IDs (P = 9 or 10) for up to 64.
static bool tables_ok(int L, int P) {
  return P <= 8 ? L <= kMaxL : P <= 10 && L <= 64;
}

// Any whole number of query heads per KV head (G > 4 runs G / 4 passes of
// four heads, or of two or one when 4 does not divide G).
bool group_ok(int Hq, int Hkv) {
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv) return false;
  return Hq / Hkv <= kMaxGroup;
}

int from_hip(hipError_t e) { return e == hipSuccess ? SOCKET_OK : SOCKET_EHIP; }

}  // namespace

extern "C" {

const char* socket_status_string(int status) {
  switch (status) {
    case SOCKET_OK: return "ok";
    case SOCKET_EINVAL: return "invalid argument";
    case SOCKET_EUNSUPPORTED: return "unsupported configuration";
    case SOCKET_ENOSPC: return "workspace too small";
    case SOCKET_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int socket_version(void) { return 100; }

int socket_hash_keys(const void* K, const void* V, int dtype, int B, int Hkv, int d,
                     int64_t n_cap, const int32_t* pos0, int count, const void* W, int L, int P,
                     uint8_t* ids, float* vnorm, void* stream) {
  // IDs need K and W, norms need V; at least one of the two outputs
  if (!pos0 || (!ids && !vnorm)) return SOCKET_EINVAL;
  if (ids && (!K || !W)) return SOCKET_EINVAL;
  if (!V != !vnorm) return SOCKET_EINVAL;
  if (dtype != SOCKET_F32 && dtype != SOCKET_BF16) return SOCKET_EINVAL;
  if (B <= 0 || Hkv <= 0 || n_cap <= 0 || count < 0 || L <= 0 || P <= 0) return SOCKET_EINVAL;
  if (n_cap >= ((int64_t)1 << 31)) return SOCKET_EUNSUPPORTED;
  if (d != kHead || !tables_ok(L, P)) return SOCKET_EUNSUPPORTED;
  if ((int64_t)B * Hkv * count >= ((int64_t)1 << 31)) return SOCKET_EUNSUPPORTED;
  if (count == 0) return SOCKET_OK;
  return from_hip(launch_hash_keys(K, V, dtype, B, Hkv, n_cap, pos0, count, W, L, P, ids, vnorm,
                                   static_cast<hipStream_t>(stream)));
}

size_t socket_ids_bytes(int B, int Hkv, int64_t n_cap, int L, int P) {
  if (B <= 0 || Hkv <= 0 || n_cap <= 0 || L <= 0 || P <= 0 || !tables_ok(L, P)) return 0;
  return (size_t)B * Hkv * ids_groups(n_cap) * 64 * ids_key_bytes(L, P);
}

size_t socket_score_topk_workspace(int B, int Hq, int Hkv, int64_t n_cap, int L, int P,
                                   int k_max) {
  (void)k_max;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_cap <= 0 || L <= 0 || L > kMaxScoreL || P <= 0 ||
      !tables_ok(L, P) || !group_ok(Hq, Hkv))
    return 0;
  return score_ws_layout(B, Hq, Hkv, n_cap, L, nullptr, nullptr);
}

static int score_ws(int B, int Hq, int Hkv, int64_t n_cap, int L, void* ws, size_t ws_bytes,
                    ScoreWs* w) {
  if (!ws) return SOCKET_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return SOCKET_EINVAL;
  const size_t need = score_ws_layout(B, Hq, Hkv, n_cap, L, w, ws);
  return ws_bytes < need ? SOCKET_ENOSPC : SOCKET_OK;
}

static int check_sizes(int B, int Hq, int Hkv, int L, int P, int64_t n_cap) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_cap <= 0 || L <= 0 || P <= 0) return SOCKET_EINVAL;
  if (Hq % Hkv) return SOCKET_EINVAL;
  if (!group_ok(Hq, Hkv)) return SOCKET_EUNSUPPORTED;
  if (!tables_ok(L, P) || L > kMaxScoreL) return SOCKET_EUNSUPPORTED;
  if (n_cap >= ((int64_t)1 << 31) || (int64_t)B * Hq * n_cap >= ((int64_t)1 << 40))
    return SOCKET_EUNSUPPORTED;
  return SOCKET_OK;
}

int socket_soft_tables(const void* q, int dtype, int B, int Hq, int Hkv, int d, const void* W,
                       int L, int P, float tau, int64_t n_cap, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!q || !W) return SOCKET_EINVAL;
  if (dtype != SOCKET_F32 && dtype != SOCKET_BF16) return SOCKET_EINVAL;
  if (!(tau > 0.f) || !(tau < INFINITY)) return SOCKET_EINVAL;
  int rc = check_sizes(B, Hq, Hkv, L, P, n_cap);
  if (rc) return rc;
  if (d != kHead) return SOCKET_EUNSUPPORTED;
  ScoreWs w;
  if ((rc = score_ws(B, Hq, Hkv, n_cap, L, ws, ws_bytes, &w))) return rc;
  return from_hip(launch_soft_tables(q, dtype, B, Hq, Hkv, W, L, P, tau, w,
                                     static_cast<hipStream_t>(stream)));
}

// Sink and window sizes: non-negative, and (with k_max > 0) their sum fits in
// an index row.
static bool sink_window_ok(int sink, int window, int k_max) {
  if (sink < 0 || window < 0 || sink > (1 << 30) || window > (1 << 30)) return false;
  return k_max <= 0 || sink + window <= k_max;
}

int socket_score(int B, int Hq, int Hkv, int L, int P, const uint8_t* ids, const float* vnorm,
                 const int32_t* lens, int64_t n_cap, int sink, int window, float* scores,
                 void* ws, size_t ws_bytes, void* stream) {
  if (!ids || !vnorm || !lens) return SOCKET_EINVAL;
  if (!sink_window_ok(sink, window, 0)) return SOCKET_EINVAL;
  int rc = check_sizes(B, Hq, Hkv, L, P, n_cap);
  if (rc) return rc;
  ScoreWs w;
  if ((rc = score_ws(B, Hq, Hkv, n_cap, L, ws, ws_bytes, &w))) return rc;
  return from_hip(launch_score(B, Hq, Hkv, L, P, ids, vnorm, lens, n_cap, SinkWindow{sink, window},
                               scores ? scores : w.scores, false, w,
                               static_cast<hipStream_t>(stream)));
}

int socket_topk(int B, int Hq, int Hkv, int L, const float* scores, const int32_t* lens,
                int64_t n_cap, const int32_t* ks, int k_max, int sink, int window, int32_t* idx,
                void* ws, size_t ws_bytes, void* stream) {
  if (!lens || !ks || !idx) return SOCKET_EINVAL;
  if (k_max <= 0 || !sink_window_ok(sink, window, k_max)) return SOCKET_EINVAL;
  if (k_max > kMaxKmax) return SOCKET_EUNSUPPORTED;
  int rc = check_sizes(B, Hq, Hkv, L, 1, n_cap);
  if (rc) return rc;
  ScoreWs w;
  if ((rc = score_ws(B, Hq, Hkv, n_cap, L, ws, ws_bytes, &w))) return rc;
  return from_hip(launch_topk(B, Hq, scores ? scores : w.scores, lens, n_cap, ks, k_max,
                              SinkWindow{sink, window}, idx, w,
                              static_cast<hipStream_t>(stream)));
}

int socket_score_topk(const void* q, int dtype, int B, int Hq, int Hkv, int d, const void* W,
                      int L, int P, float tau, const uint8_t* ids, const float* vnorm,
                      const int32_t* lens, int64_t n_cap, const int32_t* ks, int k_max, int sink,
                      int window, int32_t* idx, float* scores, void* ws, size_t ws_bytes,
                      void* stream) {
  if (!q || !W || !ids || !vnorm || !lens || !ks || !idx || !ws) return SOCKET_EINVAL;
  if (dtype != SOCKET_F32 && dtype != SOCKET_BF16) return SOCKET_EINVAL;
  if (k_max <= 0 || !sink_window_ok(sink, window, k_max)) return SOCKET_EINVAL;
  if (!(tau > 0.f) || !(tau < INFINITY)) return SOCKET_EINVAL;
  int rc = check_sizes(B, Hq, Hkv, L, P, n_cap);
  if (rc) return rc;
  if (d != kHead || k_max > kMaxKmax) return SOCKET_EUNSUPPORTED;
  ScoreWs w;
  if ((rc = score_ws(B, Hq, Hkv, n_cap, L, ws, ws_bytes, &w))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* sc = scores ? scores : w.scores;
  hipError_t e = launch_soft_tables(q, dtype, B, Hq, Hkv, W, L, P, tau, w, s);
  const SinkWindow sw{sink, window};
  if (e == hipSuccess)
    e = launch_score(B, Hq, Hkv, L, P, ids, vnorm, lens, n_cap, sw, sc, false, w, s);
  if (e == hipSuccess) e = launch_topk(B, Hq, sc, lens, n_cap, ks, k_max, sw, idx, w, s);
  return from_hip(e);
}

// The fused step's workspace: the selection workspace, then the attention's.
static size_t step_ws(int B, int Hq, int Hkv, int64_t n_cap, int L, int k_max, ScoreWs* sw,
                      DecodeWs* dw, void* base) {
  const size_t a = (score_ws_layout(B, Hq, Hkv, n_cap, L, nullptr, nullptr) + 255) & ~(size_t)255;
  if (base) score_ws_layout(B, Hq, Hkv, n_cap, L, sw, base);
  // room for one partial per key range (the selection + attention by range)
  const int rs = range_splits(n_cap);
  const size_t d = decode_ws_layout(B, Hq, k_max, dw, base ? static_cast<char*>(base) + a : nullptr,
                                    rs <= kMaxRangeSplits ? rs : 0);
  return a + d;
}

size_t socket_decode_step_workspace(int B, int Hq, int Hkv, int64_t n_cap, int L, int P,
                                    int k_max) {
  if (socket_score_topk_workspace(B, Hq, Hkv, n_cap, L, P, k_max) == 0 || k_max <= 0 ||
      k_max > kMaxKmax)
    return 0;
  return step_ws(B, Hq, Hkv, n_cap, L, k_max, nullptr, nullptr, nullptr);
}

int socket_decode_step(const void* q, const void* K, const void* V, int dtype, int B, int Hq,
                       int Hkv, int d, const void* W, int L, int P, float tau, uint8_t* ids,
                       float* vnorm, const int32_t* lens, int64_t n_cap, const int32_t* ks,
                       int k_max, int sink, int window, float scale, int32_t* idx, float* scores,
                       float* out, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !K || !V || !W || !ids || !vnorm || !lens || !ks || !idx || !out || !ws)
    return SOCKET_EINVAL;
  if (dtype != SOCKET_F32 && dtype != SOCKET_BF16) return SOCKET_EINVAL;
  if (k_max <= 0 || !sink_window_ok(sink, window, k_max)) return SOCKET_EINVAL;
  if (!(tau > 0.f) || !(tau < INFINITY)) return SOCKET_EINVAL;
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return SOCKET_EINVAL;
  int rc = check_sizes(B, Hq, Hkv, L, P, n_cap);
  if (rc) return rc;
  if (d != kHead || k_max > kMaxKmax) return SOCKET_EUNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return SOCKET_EINVAL;
  ScoreWs w;
  DecodeWs dw;
  if (ws_bytes < step_ws(B, Hq, Hkv, n_cap, L, k_max, nullptr, nullptr, nullptr))
    return SOCKET_ENOSPC;
  step_ws(B, Hq, Hkv, n_cap, L, k_max, &w, &dw, ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* sc = scores ? scores : w.scores;
  AppendKey ak;
  ak.K = K;
  ak.V = V;
  ak.lens = lens;
  ak.ids = ids;
  ak.vnorm = vnorm;
  ak.n_cap = n_cap;
  const SinkWindow sw{sink, window};
  hipError_t e = launch_soft_tables(q, dtype, B, Hq, Hkv, W, L, P, tau, w, s, ak);
  if (e == hipSuccess)
    e = launch_score(B, Hq, Hkv, L, P, ids, vnorm, lens, n_cap, sw, sc, false, w, s);
  // the selecting workgroups attend too when the sizes allow it
  const AttendSpec att{q, K, V, dtype, Hkv, scale, out};
  bool attended = false;
  if (e == hipSuccess)
    e = launch_topk(B, Hq, sc, lens, n_cap, ks, k_max, sw, idx, w, s, &att, &attended, dw.part,
                    dw.splits);
  if (e == hipSuccess && !attended)
    e = launch_sparse_decode(q, K, V, dtype, B, Hq, Hkv, n_cap, idx, k_max, scale, out, dw, s);
  return from_hip(e);
}

size_t socket_sparse_decode_workspace(int B, int Hq, int d, int k_max) {
  if (B <= 0 || Hq <= 0 || d != kHead || k_max <= 0) return 0;
  return decode_ws_layout(B, Hq, k_max, nullptr, nullptr);
}

int socket_sparse_decode(const void* q, const void* K, const void* V, int dtype, int B, int Hq,
                         int Hkv, int d, int64_t n_cap, const int32_t* idx, int k_max,
                         float scale, float* out, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !K || !V || !idx || !out || !ws) return SOCKET_EINVAL;
  if (dtype != SOCKET_F32 && dtype != SOCKET_BF16) return SOCKET_EINVAL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_cap <= 0 || k_max <= 0) return SOCKET_EINVAL;
  if (Hq % Hkv) return SOCKET_EINVAL;
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return SOCKET_EINVAL;
  if (d != kHead || k_max > kMaxKmax) return SOCKET_EUNSUPPORTED;
  if (n_cap >= ((int64_t)1 << 31)) return SOCKET_EUNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return SOCKET_EINVAL;
  DecodeWs w;
  const size_t need = decode_ws_layout(B, Hq, k_max, &w, ws);
  if (ws_bytes < need) return SOCKET_ENOSPC;
  return from_hip(launch_sparse_decode(q, K, V, dtype, B, Hq, Hkv, n_cap, idx, k_max, scale, out,
                                       w, static_cast<hipStream_t>(stream)));
}

// Hard-LSH comparison mode: P divides 32 (no table straddles a code word).
static bool hard_ok(int L, int P) {
  return L >= 1 && (P == 1 || P == 2 || P == 4 || P == 8 || P == 16) && L * P <= kMaxCodeBits;
}

size_t socket_codes_bytes(int B, int Hkv, int64_t n_cap, int L, int P) {
  if (B <= 0 || Hkv <= 0 || n_cap <= 0 || !hard_ok(L, P)) return 0;
  return (size_t)B * Hkv * codes_words(L, P) * n_cap * sizeof(uint32_t);
}

int socket_hash_codes(const void* K, const void* V, int dtype, int B, int Hkv, int d,
                      int64_t n_cap, const int32_t* pos0, int count, const void* W, int L, int P,
                      uint32_t* codes, float* vnorm, void* stream) {
  if (!K || !V || !pos0 || !W || !codes || !vnorm) return SOCKET_EINVAL;
  if (dtype != SOCKET_F32 && dtype != SOCKET_BF16) return SOCKET_EINVAL;
  if (B <= 0 || Hkv <= 0 || n_cap <= 0 || count < 0 || L <= 0 || P <= 0) return SOCKET_EINVAL;
  if (d != kHead || !hard_ok(L, P)) return SOCKET_EUNSUPPORTED;
  if (n_cap >= ((int64_t)1 << 31)) return SOCKET_EUNSUPPORTED;
  const int64_t blocks = (int64_t)B * Hkv * count * ((L * P + 63) / 64);
  if (blocks >= ((int64_t)1 << 31)) return SOCKET_EUNSUPPORTED;
  if (count == 0) return SOCKET_OK;
  return from_hip(launch_hash_codes(K, V, dtype, B, Hkv, n_cap, pos0, count, W, L, P, codes,
                                    vnorm, static_cast<hipStream_t>(stream)));
}

size_t socket_hard_score_topk_workspace(int B, int Hq, int Hkv, int64_t n_cap, int L, int P,
                                        int k_max) {
  (void)k_max;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_cap <= 0 || !hard_ok(L, P) || !group_ok(Hq, Hkv) ||
      n_cap >= ((int64_t)1 << 31))
    return 0;
  return select_ws_layout((size_t)B * Hq * codes_words(L, P) * sizeof(uint32_t), B, Hq, n_cap,
                          nullptr, nullptr);
}

int socket_hard_score_topk(const void* q, int dtype, int B, int Hq, int Hkv, int d, const void* W,
                           int L, int P, const uint32_t* codes, const float* vnorm,
                           const int32_t* lens, int64_t n_cap, const int32_t* ks, int k_max,
                           int sink, int window, int32_t* idx, float* scores, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!q || !W || !codes || !vnorm || !lens || !ks || !idx || !ws) return SOCKET_EINVAL;
  if (dtype != SOCKET_F32 && dtype != SOCKET_BF16) return SOCKET_EINVAL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_cap <= 0 || L <= 0 || P <= 0) return SOCKET_EINVAL;
  if (Hq % Hkv) return SOCKET_EINVAL;
  if (k_max <= 0 || !sink_window_ok(sink, window, k_max)) return SOCKET_EINVAL;
  if (d != kHead || k_max > kMaxKmax || !group_ok(Hq, Hkv) || !hard_ok(L, P))
    return SOCKET_EUNSUPPORTED;
  if (n_cap >= ((int64_t)1 << 31) || (int64_t)B * Hq * n_cap >= ((int64_t)1 << 40))
    return SOCKET_EUNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return SOCKET_EINVAL;
  ScoreWs w;
  const size_t need = select_ws_layout((size_t)B * Hq * codes_words(L, P) * sizeof(uint32_t), B,
                                       Hq, n_cap, &w, ws);
  if (ws_bytes < need) return SOCKET_ENOSPC;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* sc = scores ? scores : w.scores;
  const SinkWindow sw{sink, window};
  hipError_t e = launch_hard_score(q, dtype, B, Hq, Hkv, W, L, P, codes, vnorm, lens, n_cap, sw,
                                   sc, w, s);
  if (e == hipSuccess) e = launch_topk(B, Hq, sc, lens, n_cap, ks, k_max, sw, idx, w, s);
  return from_hip(e);
}

int socket_sample_estimate(const void* q, int dtype, int B, int Hq, int Hkv, int d, const void* W,
                           int L, int P, float tau, const uint8_t* ids, const float* vnorm,
                           const void* V, const int32_t* lens, int64_t n_cap, const float* u,
                           int M, float* out, int32_t* draws, float* scores, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!q || !W || !ids || !vnorm || !V || !lens || !u || !out || !ws) return SOCKET_EINVAL;
  if (dtype != SOCKET_F32 && dtype != SOCKET_BF16) return SOCKET_EINVAL;
  if (M <= 0) return SOCKET_EINVAL;
  if (!(tau > 0.f) || !(tau < INFINITY)) return SOCKET_EINVAL;
  int rc = check_sizes(B, Hq, Hkv, L, P, n_cap);
  if (rc) return rc;
  if (d != kHead || M > kMaxDraws) return SOCKET_EUNSUPPORTED;
  ScoreWs w;
  if ((rc = score_ws(B, Hq, Hkv, n_cap, L, ws, ws_bytes, &w))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* sc = scores ? scores : w.scores;
  hipError_t e = launch_soft_tables(q, dtype, B, Hq, Hkv, W, L, P, tau, w, s);
  if (e == hipSuccess)
    e = launch_score(B, Hq, Hkv, L, P, ids, vnorm, lens, n_cap, SinkWindow{0, 0}, sc, true, w, s);
  if (e == hipSuccess)
    e = launch_estimate(sc, vnorm, V, dtype, B, Hq, Hkv, lens, n_cap, u, M, out, draws, w, s);
  return from_hip(e);
}

size_t socket_dense_decode_workspace(int B, int Hq, int Hkv, int d, int64_t n_cap) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d != kHead || n_cap <= 0 ||
      n_cap >= ((int64_t)1 << 31))
    return 0;
  return dense_ws_layout(B, Hq, Hkv, n_cap, nullptr, nullptr);
}

int socket_dense_decode(const void* q, const void* K, const void* V, int dtype, int B, int Hq,
                        int Hkv, int d, int64_t n_cap, const int32_t* lens, float scale,
                        float* out, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !K || !V || !lens || !out || !ws) return SOCKET_EINVAL;
  if (dtype != SOCKET_F32 && dtype != SOCKET_BF16) return SOCKET_EINVAL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n_cap <= 0) return SOCKET_EINVAL;
  if (Hq % Hkv) return SOCKET_EINVAL;
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return SOCKET_EINVAL;
  if (d != kHead || !group_ok(Hq, Hkv)) return SOCKET_EUNSUPPORTED;
  if (n_cap >= ((int64_t)1 << 31)) return SOCKET_EUNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(ws) & 255) return SOCKET_EINVAL;
  DenseWs w;
  const size_t need = dense_ws_layout(B, Hq, Hkv, n_cap, &w, ws);
  if (ws_bytes < need) return SOCKET_ENOSPC;
  return from_hip(launch_dense_decode(q, K, V, dtype, B, Hq, Hkv, n_cap, lens, scale, out, w,
                                      static_cast<hipStream_t>(stream)));
}

}  // extern "C"
