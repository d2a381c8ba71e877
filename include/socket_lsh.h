/*
 * socket_lsh.h -- C ABI of the SOCKET sparse-attention decode path for
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the one of "SOCKET: SOft Collision Kernel EsTimator for
 * Sparse Attention" (paperpeel.com/paper/2602.06283), Section 4.1 "The Final
 * Algorithm": keys are hashed into L tables at prefill and their bucket IDs
 * are cached with the value-vector norms (Algorithm 1); at decode the query
 * induces a probability distribution over the buckets of each table and each
 * key is scored by the probability mass of its own buckets, weighted by its
 * value norm (Algorithm 2, Section 1 "Key Idea"); the top-k keys are selected
 * and exact attention runs over that subset only (Algorithm 3, Section 2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor arguments are DEVICE pointers owned by the caller; the library
 *   never allocates, frees or retains them.  Work is enqueued on `stream`
 *   (a hipStream_t, passed as void*; NULL means the default stream) and the
 *   call returns right after enqueueing.  Nothing is synchronised.
 * - No global state is kept between calls; calls on different streams with
 *   disjoint outputs and workspaces may run concurrently.
 * - Layouts are dense, row-major, with the last index contiguous:
 *     K, V      [B][Hkv][n_cap][d]      dtype SOCKET_BF16 or SOCKET_F32
 *     q         [B][Hq][d]              same dtype as K
 *     W         [L*P][d]                same dtype as K; rows l*P..l*P+P-1 are
 *                                       the P hyperplanes of table l
 *     ids       bucket-ID cache, socket_ids_bytes() bytes, tiled (below)
 *     vnorm     [B][Hkv][n_cap]         float32
 *     lens, ks  [B]                     int32, device
 *     idx       [B][Hq][k_max]          int32
 *     scores    [B][Hq][ns]             float32, ns = n_cap rounded up to 64
 *     out       [B][Hq][d]              float32
 * - Query head g reads KV head g / (Hq / Hkv) (grouped-query attention).
 *   Hq must be a multiple of Hkv, with G = Hq / Hkv <= 64.  The scorer and
 *   the dense kernel take the query heads of a KV row four at a time (two
 *   or one when 4 does not divide G), so with G > 4 a KV row's IDs (or K
 *   and V) are read G / 4 times per step.
 * - d must be 128.  Either 1 <= P <= 8 and 1 <= L <= 128, or P in {9, 10}
 *   and 1 <= L <= 64.  1 <= k_max <= 65536.
 *
 * Bucket-ID cache layout
 * ----------------------
 * The bucket ID of table l (bit j = sign of plane j) is a cell of C bytes:
 * C = 1 for P <= 8, C = 2 (little-endian) for P = 9 or 10 and L <= 32
 * (packed ten-bit cells for larger L, below).  The IDs of a key
 * are cut into 16 words of TL tables, TL = 1, 2, 4 or 8 the smallest power of
 * two with 16*TL >= L; word w holds tables w*TL .. w*TL+TL-1 (cell b of the
 * word = table w*TL + b; tables >= L read as 0) and is WB = TL*C bytes long.
 * Keys are tiled in groups of 64: key i of KV row r = b*Hkv + h lies in group
 * i/64 at t = i%64, t = 16*kg + x; with u = (x - w) mod 16 and R = 16/WB its
 * word w is stored at byte offset
 *   ((r * ceil(n_cap/64) + i/64) * 1024 + (u/R)*64*R + (16*kg + w)*R + u%R) * WB.
 * This order lets the scorer read its words with 16-byte loads, 1 KiB per
 * wave and load.
 * Packed words (P = 9 or 10 with 33 <= L <= 64, TL = 4): the four IDs of a
 * word are ten-bit fields, table w*4 + m at bits 10m .. 10m+9 of a 40-bit
 * value, and a key takes 80 bytes (SOCKET Sec. 1 puts the footprint at about
 * 600 bits a token with P = 10 and L = 60).  With the same t, kg, x, u and
 * lane c = 16*kg + w, the low 32 bits (little-endian) of word w start at
 *   (r * ceil(n_cap/64) + i/64) * 5120 + (u/4)*1024 + 16*c + 4*(u%4)
 * and its high byte lies at
 *   (r * ceil(n_cap/64) + i/64) * 5120 + 4096 + 16*c + u.
 * - Errors are reported as negative return codes before anything is
 *   enqueued (argument checks), or as SOCKET_EHIP when a launch fails.
 *   Nothing throws or aborts.  socket_status_string() names a code.
 */
#ifndef SOCKET_LSH_H
#define SOCKET_LSH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SOCKET_OK = 0,
  SOCKET_EINVAL = -1,       /* null pointer, bad size, bad shape            */
  SOCKET_EUNSUPPORTED = -2, /* valid but not implemented (d != 128, P > 10) */
  SOCKET_ENOSPC = -3,       /* workspace smaller than the *_workspace size  */
  SOCKET_EHIP = -4          /* a HIP launch failed                          */
};

enum { SOCKET_F32 = 0, SOCKET_BF16 = 1 };

/* Name of a status code (static string). */
const char* socket_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int socket_version(void);

/* Size in bytes of the bucket-ID cache for B x Hkv rows of n_cap keys and L
 * tables of P planes (0 for invalid or unsupported sizes). */
size_t socket_ids_bytes(int B, int Hkv, int64_t n_cap, int L, int P);

/*
 * socket_hash_keys -- Algorithm 1 (SOCKET Sec. 4.1; bucket ID = sign pattern
 * of W^(l) k, Appendix B.2) plus the value-norm cache (Sec. 1 "Key Idea").
 *
 * For every sequence b, KV head h and position i in [pos0[b], pos0[b]+count):
 *   ID of table l of key i = sum_j [ <W[l*P+j], K[b][h][i]> > 0 ] << j
 *   vnorm[b][h][i]         = || V[b][h][i] ||_2
 * The projection is accumulated in float32 (bf16 products are exact in
 * float32).  A projection of exactly zero gives bit 0.  Positions at or past
 * n_cap are skipped.  Prefill passes pos0 = 0 and count = n; the decode-time
 * append passes pos0 = current length and count = 1 after the caller has
 * written the new row of K and V.
 *
 * pos0 is a device int32 array [B].  ids (socket_ids_bytes(B, Hkv, n_cap, L, P)
 * bytes) receives all 16 words of every hashed key in the tiled layout;
 * other keys and other rows of vnorm are untouched.
 *
 * Either output may be left out: ids = NULL computes the value norms only
 * (K and W may then be NULL), V = vnorm = NULL computes the bucket IDs only.
 * A V without a vnorm (or the reverse), or neither output, is SOCKET_EINVAL.
 * The results do not depend on which outputs are asked for.
 */
int socket_hash_keys(const void* K, const void* V, int dtype, int B, int Hkv, int d,
                     int64_t n_cap, const int32_t* pos0, int count, const void* W, int L,
                     int P, uint8_t* ids, float* vnorm, void* stream);

/* Workspace bytes needed by socket_score_topk for these sizes (0 if unsupported). */
size_t socket_score_topk_workspace(int B, int Hq, int Hkv, int64_t n_cap, int L, int P,
                                   int k_max);

/*
 * socket_score_topk -- Algorithms 2 and 3 of SOCKET Sec. 4.1.
 *
 * For each sequence b and query head g (KV head h = g / (Hq/Hkv)):
 *   u[l][j]   = <W[l*P+j], q[b][g]>                         (float64)
 *   p_l(c)    = softmax over buckets c of (sum_j s_j(c) u[l][j]) / tau,
 *               s_j(c) = +1 if bit j of c is set else -1
 *               (equivalently prod_j sigmoid(2 s_j(c) u[l][j] / tau))
 *   s_i       = vnorm[b][h][i] * sum_l p_l(ID of table l of key i)   for i < lens[b]
 *   F_b       = { i < n : i < sink or i >= n - window },  n = lens[b]
 *               (sink and local-window keys, always attended; SOCKET Sec. 6
 *               setup includes 64 or 128 of them)
 *   idx[b][g] = F_b united with the min(ks[b], n - |F_b|) keys outside F_b
 *               with the largest s_i; among equal scores the lower index
 *               wins.  The indices are written in ascending order and the
 *               row is padded with -1 up to k_max.  sink = window = 0 gives
 *               plain top-k.
 * Scores are float32, score row stride ns = n_cap rounded up to a multiple of
 * 64 (rows start 256-byte aligned).  A table entry is either the float32 rounding of the
 * float64 p_l(c), or the float32 product lo * hi of the float32 roundings of
 * its two factors (added with one fused multiply-add).  If `scores` is not NULL the scores of every i < lens[b] are
 * written there (entries i >= lens[b] are left untouched).
 *
 * lens and ks are device int32 arrays [B] with 0 <= lens[b] <= n_cap and
 * ks[b] + sink + window <= k_max (a negative ks[b] is treated as 0; a larger
 * one is cut to k_max - |F_b|).  sink, window >= 0 with sink + window <=
 * k_max, else SOCKET_EINVAL.  tau > 0.
 * ws must hold socket_score_topk_workspace(B, Hq, Hkv, n_cap, L, P, k_max) bytes
 * and be 256-byte aligned; its contents need not be initialised.
 */
int socket_score_topk(const void* q, int dtype, int B, int Hq, int Hkv, int d, const void* W,
                      int L, int P, float tau, const uint8_t* ids, const float* vnorm,
                      const int32_t* lens, int64_t n_cap, const int32_t* ks, int k_max, int sink,
                      int window, int32_t* idx, float* scores, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * The three stages of socket_score_topk, for callers that schedule or time
 * them separately.  All three take the same workspace (sized by
 * socket_score_topk_workspace for the same B, Hq, Hkv, n_cap, L) and must be
 * enqueued in this order on one stream for one query batch:
 *
 * socket_soft_tables -- Algorithm 2, first half: the float64 projections of
 *   q[b][g] and the bucket distribution of every table, stored in the
 *   workspace either as the full table p_l(c) or as its two factors, each
 *   value rounded once to float32: lo_l(c & 15) (planes 0..3) and
 *   hi_l(c >> 4) (planes 4..P-1) for P <= 8, lo_l(c & 31) (planes 0..4) and
 *   hi_l(c >> 5) (planes 5..P-1) for P = 9 or 10.  Also clears the selection histograms and
 *   counters held in the workspace.
 * socket_score -- Algorithm 2, second half: s_i for every i < lens[b] of every
 *   query head, written to `scores` (or into the workspace when scores is
 *   NULL), plus a histogram of the top bits of the scores of the keys
 *   outside F_b in the workspace.
 * socket_topk -- Algorithm 3: the top-k indices per query head, from the same
 *   `scores` pointer (NULL = workspace) and the histogram left by
 *   socket_score, which must have been given the same sink and window.
 *   Output as in socket_score_topk.
 */
int socket_soft_tables(const void* q, int dtype, int B, int Hq, int Hkv, int d, const void* W,
                       int L, int P, float tau, int64_t n_cap, void* ws, size_t ws_bytes,
                       void* stream);
int socket_score(int B, int Hq, int Hkv, int L, int P, const uint8_t* ids, const float* vnorm,
                 const int32_t* lens, int64_t n_cap, int sink, int window, float* scores,
                 void* ws, size_t ws_bytes, void* stream);
int socket_topk(int B, int Hq, int Hkv, int L, const float* scores, const int32_t* lens,
                int64_t n_cap, const int32_t* ks, int k_max, int sink, int window, int32_t* idx,
                void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes needed by socket_decode_step (0 if unsupported). */
size_t socket_decode_step_workspace(int B, int Hq, int Hkv, int64_t n_cap, int L, int P,
                                    int k_max);

/*
 * socket_decode_step -- one whole decode step for callers that have written
 * the new token's key and value at position lens[b] - 1 of K and V (lens
 * counts the new token): hashes that key and stores its value norm (as
 * socket_hash_keys with pos0 = lens - 1 and count = 1), then selects as
 * socket_score_topk (with sink and window) and attends as
 * socket_sparse_decode, writing idx, scores (may be NULL) and out.  The key is
 * hashed inside the table kernel, and when the query heads do not outnumber
 * the GPU's compute units the selection ends in a kernel that also attends,
 * one workgroup per (query head, range of keys), so the step takes one launch
 * fewer than the three calls.  IDs, norms, scores and idx equal the three
 * calls' bit for bit; out agrees with theirs to rounding (its partial sums
 * are taken over key ranges instead of runs of 64 selected keys).  ws must
 * hold socket_decode_step_workspace(...) bytes, 256-byte aligned.
 */
int socket_decode_step(const void* q, const void* K, const void* V, int dtype, int B, int Hq,
                       int Hkv, int d, const void* W, int L, int P, float tau, uint8_t* ids,
                       float* vnorm, const int32_t* lens, int64_t n_cap, const int32_t* ks,
                       int k_max, int sink, int window, float scale, int32_t* idx, float* scores,
                       float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * socket_decode_step_noalloc -- socket_decode_step without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * allocates nothing and calls no allocating routine; its scratch memory is
 * one static device array of SOCKET_NOALLOC_SCRATCH_BYTES per GPU, held from
 * the first call on that GPU until the process ends.
 *
 * Arguments, results and status codes are those of socket_decode_step.
 * Sizes whose socket_decode_step_workspace() exceeds
 * SOCKET_NOALLOC_SCRATCH_BYTES are rejected with SOCKET_ENOSPC before
 * anything is enqueued (the 32K and 128K single-sequence steps fit; a batch
 * of 16 sequences of 32K keys does not).  Every call on one GPU shares that
 * GPU's array, and the array keeps the last call's contents (each call
 * clears what it needs cleared inside its own kernels): calls that can
 * overlap on one GPU -- on different streams, or from different host
 * threads without ordering -- race on it and must not be issued.
 */
#define SOCKET_NOALLOC_SCRATCH_BYTES (64u << 20)

int socket_decode_step_noalloc(const void* q, const void* K, const void* V, int dtype, int B,
                               int Hq, int Hkv, int d, const void* W, int L, int P, float tau,
                               uint8_t* ids, float* vnorm, const int32_t* lens, int64_t n_cap,
                               const int32_t* ks, int k_max, int sink, int window, float scale,
                               int32_t* idx, float* scores, float* out, void* stream);

/* Workspace bytes needed by socket_sparse_decode for these sizes. */
size_t socket_sparse_decode_workspace(int B, int Hq, int d, int k_max);

/*
 * socket_sparse_decode -- exact softmax attention over the selected keys
 * (SOCKET Sec. 2 and Sec. 4.1, Algorithm 3):
 *   a_i = exp(scale * <q, K_i>) / sum_{i' in S} exp(scale * <q, K_i'>)
 *   out[b][g] = sum_{i in S} a_i V_i,   S = { idx[b][g][t] : t < k_max, idx >= 0 }
 * with K, V of KV head g / (Hq/Hkv).  Accumulation is float32.  Entries of
 * idx equal to -1 are skipped; every other entry must lie in [0, n_cap).
 * A row with no selected key produces zeros.  `scale` is usually 1/sqrt(d).
 * ws must hold socket_sparse_decode_workspace(B, Hq, d, k_max) bytes,
 * 256-byte aligned; its contents need not be initialised.
 */
int socket_sparse_decode(const void* q, const void* K, const void* V, int dtype, int B, int Hq,
                         int Hkv, int d, int64_t n_cap, const int32_t* idx, int k_max,
                         float scale, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * socket_sample_estimate -- the value-aware sampling estimator T(q) of the
 * SOCKET analysis (Sec. 5.1, Theorem 3; Appendix B.2), an unbiased Monte
 * Carlo estimate of the soft-attention output y(q) = sum_j a~_j v_j:
 *   s~_j = sum_l p_l(ID_l(K_j)), a~_j = s~_j / sum_i s~_i   (i, j < lens[b])
 *   p_j  = a~_j ||v_j|| / S_1,  S_1 = sum_j a~_j ||v_j||
 *   J_m  = the first j whose running sum of s_j exceeds u[b][g][m] * sum_i s_i
 *          (s_j = vnorm_j * s~_j, the score of socket_score_topk; so J_m ~ p)
 *   out[b][g] = (S_1 / M) * sum_{m < M} V_{J_m} / vnorm_{J_m}
 * The M uniforms u (device float32 [B][Hq][M], values in [0, 1)) are
 * inputs; draws (device int32 [B][Hq][M], may be NULL) receives J_m.  A head
 * with no key of positive score gives zeros (and draws of -1).  Arguments
 * otherwise as in socket_score_topk (same workspace size, tables and IDs);
 * V is the value cache [B][Hkv][n_cap][d]; 1 <= M <= 8192.
 */
int socket_sample_estimate(const void* q, int dtype, int B, int Hq, int Hkv, int d, const void* W,
                           int L, int P, float tau, const uint8_t* ids, const float* vnorm,
                           const void* V, const int32_t* lens, int64_t n_cap, const float* u,
                           int M, float* out, int32_t* draws, float* scores, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * Hard-LSH comparison mode -- the estimator SOCKET is compared with (SOCKET
 * Sec. 3.1, Sec. 5.3; Appendix A.2, Table 9: best at P = 2 with L = 300 or
 * 500 tables): the score of key i is
 *   s_i = vnorm[b][h][i] * #{ l : ID_l(K_i) == ID_l(q) },
 * IDs as in socket_hash_keys, the query's IDs from the same float32
 * projections.  P must divide 32 (1, 2, 4, 8 or 16) and L*P <= 4096.
 *
 * Codes: the L*P sign bits of a key, bit p = l*P + j = [<W[p], K_i> > 0],
 * 32 bits per word (bit p in word p/32 at bit p%32), cw = ceil(L*P/32)
 * words, stored word-major as uint32 codes[B][Hkv][cw][n_cap]; bits at or
 * past L*P are 0.  socket_codes_bytes() gives the size (0 if unsupported).
 */
size_t socket_codes_bytes(int B, int Hkv, int64_t n_cap, int L, int P);

/* Hashing for the hard mode: like socket_hash_keys (same projections,
 * positions and value norms), writing codes instead of tiled IDs. */
int socket_hash_codes(const void* K, const void* V, int dtype, int B, int Hkv, int d,
                      int64_t n_cap, const int32_t* pos0, int count, const void* W, int L, int P,
                      uint32_t* codes, float* vnorm, void* stream);

/* Workspace bytes needed by socket_hard_score_topk (0 if unsupported). */
size_t socket_hard_score_topk_workspace(int B, int Hq, int Hkv, int64_t n_cap, int L, int P,
                                        int k_max);

/*
 * socket_hard_score_topk -- hard collision-count scores of every key and the
 * selection of socket_score_topk (sink and window keys, then the top-k of
 * the rest, ties to the lower index, ascending, padded with -1) from them.
 * Arguments as in socket_score_topk with codes in place of ids; ws must hold
 * socket_hard_score_topk_workspace(B, Hq, Hkv, n_cap, L, P, k_max) bytes,
 * 256-byte aligned.
 */
int socket_hard_score_topk(const void* q, int dtype, int B, int Hq, int Hkv, int d, const void* W,
                           int L, int P, const uint32_t* codes, const float* vnorm,
                           const int32_t* lens, int64_t n_cap, const int32_t* ks, int k_max,
                           int sink, int window, int32_t* idx, float* scores, void* ws,
                           size_t ws_bytes, void* stream);

/* Workspace bytes needed by socket_dense_decode for these sizes (0 if unsupported). */
size_t socket_dense_decode_workspace(int B, int Hq, int Hkv, int d, int64_t n_cap);

/*
 * socket_dense_decode -- full softmax attention of each decode query over
 * every key of its sequence: the dense (FlashAttention-style) reference point
 * against which the SOCKET paper quotes its decode speedups (Sec. 1,
 * contributions; Sec. 6), computed at the same shapes as the sparse path.
 *   out[b][g] = sum_{i < lens[b]} a_i V_i,
 *   a_i = exp(scale * <q, K_i>) / sum_{i' < lens[b]} exp(scale * <q, K_i'>)
 * with K, V of KV head g / (Hq/Hkv).  Accumulation is
 * float32.  lens is a device int32 array [B], 0 <= lens[b] <= n_cap; an
 * empty sequence produces zeros.  ws must hold
 * socket_dense_decode_workspace(B, Hq, Hkv, d, n_cap) bytes, 256-byte aligned;
 * its contents need not be initialised.
 */
int socket_dense_decode(const void* q, const void* K, const void* V, int dtype, int B, int Hq,
                        int Hkv, int d, int64_t n_cap, const int32_t* lens, float scale,
                        float* out, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SOCKET_LSH_H */
