// Exact softmax attention of one decode query over its selected keys
// (SOCKET Sec. 2 and Sec. 4.1, Algorithm 3: exact attention over the
// retrieved subset).
//
// Split-k gather flash-decode: workgroup (b, g, s) gathers the K and V rows of
// entries [s*KS, (s+1)*KS) of idx[b][g], keeps the split's logits in LDS,
// and writes the unnormalised partial (o_s, m_s, l_s) with
//   m_s = max logit, l_s = sum exp(logit - m_s), o_s = sum exp(logit - m_s) v.
// A second kernel merges the splits of each (b, g) in a fixed order.
// A 16-lane row owns one key row at a time (16 B per lane for bf16), so the
// gathers are 256-B contiguous reads and the dot products reduce with DPP.
#include "common.h"
#include "launch.h"

namespace socketlsh {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;

static inline size_t align256d(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_ws_layout(int B, int Hq, int k_max, DecodeWs* ws, void* base, int min_splits) {
  int splits = (k_max + kSplitKeys - 1) / kSplitKeys;
  if (splits < min_splits) splits = min_splits;
  const size_t heads = (size_t)B * Hq;
  size_t off = 0;
  const size_t o_part = off; off = align256d(off + heads * splits * kPartStride * sizeof(float));
  if (ws) {
    char* p = static_cast<char*>(base);
    ws->part = reinterpret_cast<float*>(p + o_part);
    ws->splits = splits;
  }
  return off;
}

// grid: B*Hq*splits blocks of kDecThreads.
template <typename T>
__global__ __launch_bounds__(kDecThreads) void decode_partial_kernel(
    const T* __restrict__ q, const T* __restrict__ K, const T* __restrict__ V, int Hq, int Hkv,
    int64_t n_cap, const int32_t* __restrict__ idx, int k_max, float scale, int splits,
    float* __restrict__ part) {
  const int bg = blockIdx.x / splits;
  const int sp = blockIdx.x % splits;
  const int b = bg / Hq, g = bg % Hq;
  const int h = g / (Hq / Hkv);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, kg = lane >> 4, j = lane & 15;
  const int t0 = sp * kSplitKeys;
  int t1 = t0 + kSplitKeys;
  if (t1 > k_max) t1 = k_max;
  const int nt = t1 - t0;

  __shared__ float logit[kSplitKeys];
  __shared__ float red[kDecWaves * 4][kHead];
  __shared__ float sh_m, sh_l;

  float qf[8];
  load_row8<T>(q + (int64_t)bg * kHead, j, qf);
  const int32_t* irow = idx + (int64_t)bg * k_max;
  const int64_t kvbase = ((int64_t)b * Hkv + h) * n_cap;

  // row (wave, kg) owns entries t = wave*4 + kg + 16*r, r < kRounds; every
  // index, K row and V row it needs is requested before any is used
  constexpr int kRounds = kSplitKeys / (kDecWaves * 4);
  int32_t ii[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int t = wave * 4 + kg + 16 * r;
    int32_t i = t < nt ? irow[t0 + t] : -1;
    if (i >= n_cap) i = -1;  // out-of-range entries are skipped like padding
    ii[r] = i;
  }
  float kf[kRounds][8], vf[kRounds][8];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t row = kvbase + (ii[r] >= 0 ? ii[r] : 0);
    load_row8<T>(K + row * kHead, j, kf[r]);
    load_row8<T>(V + row * kHead, j, vf[r]);
  }
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int t = wave * 4 + kg + 16 * r;
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = fmaf(qf[e], kf[r][e], dot);
    dot = row16_sum(dot);
    if (j == 0 && t < nt) logit[t] = ii[r] >= 0 ? dot * scale : -INFINITY;
  }
  __syncthreads();
  if (wave == 0) {
    float m = -INFINITY;
    for (int t = lane; t < nt; t += 64) m = fmaxf(m, logit[t]);
    m = wave_max(m);
    float l = 0.f;
    for (int t = lane; t < nt; t += 64) {
      const float p = logit[t] == -INFINITY ? 0.f : __expf(logit[t] - m);
      logit[t] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) { sh_m = m; sh_l = l; }
  }
  __syncthreads();
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int t = wave * 4 + kg + 16 * r;
    if (t < nt && ii[r] >= 0) {
      const float p = logit[t];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(p, vf[r][e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[wave * 4 + kg][8 * j + e] = acc[e];
  __syncthreads();
  float* out = part + ((int64_t)bg * splits + sp) * kPartStride;
  if (tid < kHead) {
    float o = 0.f;
#pragma unroll
    for (int r = 0; r < kDecWaves * 4; ++r) o += red[r][tid];
    out[tid] = o;
  }
  if (tid == 0) {
    out[kHead] = sh_m;
    out[kHead + 1] = sh_l;
  }
}

// grid: B*Hq blocks of kHead threads.  Merges the splits of one query head:
// M = max_s m_s, w_s = exp(m_s - M), out = sum_s w_s o_s / sum_s w_s l_s,
// with the sums taken in split order.
constexpr int kMaxSplits = 1024;

__global__ __launch_bounds__(kHead) void decode_combine_kernel(const float* __restrict__ part,
                                                               int splits,
                                                               float* __restrict__ out) {
  const int bg = blockIdx.x;
  const int d = threadIdx.x;
  const float* p = part + (int64_t)bg * splits * kPartStride;
  __shared__ float wsh[kMaxSplits], lsh[kMaxSplits];
  __shared__ float red[kHead / 64];
  __shared__ float sh_M, sh_L;
  float m = -INFINITY;
  for (int s = d; s < splits; s += kHead) {
    const float* ps = p + (int64_t)s * kPartStride;
    const float ms = ps[kHead], ls = ps[kHead + 1];
    wsh[s] = ls > 0.f ? ms : -INFINITY;
    lsh[s] = ls;
    m = fmaxf(m, wsh[s]);
  }
  m = wave_max(m);
  if ((d & 63) == 0) red[d >> 6] = m;
  __syncthreads();
  if (d == 0) {
    float M = red[0];
    for (int w = 1; w < kHead / 64; ++w) M = fmaxf(M, red[w]);
    sh_M = M;
  }
  __syncthreads();
  const float M = sh_M;
  for (int s = d; s < splits; s += kHead)
    wsh[s] = wsh[s] == -INFINITY ? 0.f : __expf(wsh[s] - M);
  __syncthreads();
  if (d == 0) {
    float L = 0.f;
    for (int s = 0; s < splits; ++s) L = fmaf(lsh[s], wsh[s], L);
    sh_L = L;
  }
  float o = 0.f;
  int s = 0;
  for (; s + 8 <= splits; s += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(int64_t)(s + u) * kPartStride + d];
#pragma unroll
    for (int u = 0; u < 8; ++u) o = fmaf(v[u], wsh[s + u], o);
  }
  for (; s < splits; ++s) o = fmaf(p[(int64_t)s * kPartStride + d], wsh[s], o);
  __syncthreads();
  const float L = sh_L;
  out[(int64_t)bg * kHead + d] = L > 0.f ? o / L : 0.f;
}

hipError_t launch_sparse_decode(const void* q, const void* K, const void* V, int dtype, int B,
                                int Hq, int Hkv, int64_t n_cap, const int32_t* idx, int k_max,
                                float scale, float* out, const DecodeWs& ws, hipStream_t s) {
  const int heads = B * Hq;
  const unsigned nblk = (unsigned)(heads * ws.splits);
  if (dtype == 1)
    decode_partial_kernel<uint16_t><<<nblk, kDecThreads, 0, s>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(K),
        static_cast<const uint16_t*>(V), Hq, Hkv, n_cap, idx, k_max, scale, ws.splits, ws.part);
  else
    decode_partial_kernel<float><<<nblk, kDecThreads, 0, s>>>(
        static_cast<const float*>(q), static_cast<const float*>(K), static_cast<const float*>(V),
        Hq, Hkv, n_cap, idx, k_max, scale, ws.splits, ws.part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine(ws.part, heads, ws.splits, out, s);
}

// The same merge for at most kFewSplits splits in one round trip: thread d
// loads every split's (m, l) and its own o values at once and merges them in
// registers, in split order, with no LDS and no barrier.
constexpr int kFewSplits = 32;

// grid: B*Hq blocks rounded up to a multiple of kXcds; head bg = logical block
// (blockIdx mod 8) * (grid / 8) + blockIdx / 8, so a head is merged on the XCD
// that ran its splits when the split kernel remaps its blocks the same way
// (the decode step's range kernel does).
template <int NS>
__global__ __launch_bounds__(kHead) void decode_combine_few_kernel(const float* __restrict__ part,
                                                                   int splits,
                                                                   float* __restrict__ out,
                                                                   int heads) {
  const int bg = (int)(blockIdx.x % kXcds) * (int)(gridDim.x / kXcds) + (int)(blockIdx.x / kXcds);
  if (bg >= heads) return;
  const int d = threadIdx.x;
  const float* p = part + (int64_t)bg * splits * kPartStride;
  float o[NS], m[NS], l[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int sc = s < splits ? s : splits - 1;  // past the last split: re-read it, weight 0
    o[s] = p[(int64_t)sc * kPartStride + d];
    m[s] = p[(int64_t)sc * kPartStride + kHead];
    l[s] = p[(int64_t)sc * kPartStride + kHead + 1];
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < splits && l[s] > 0.f) M = fmaxf(M, m[s]);
  float L = 0.f, acc = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float w = (s < splits && l[s] > 0.f) ? __expf(m[s] - M) : 0.f;
    L = fmaf(l[s], w, L);
    acc = fmaf(o[s], w, acc);
  }
  out[(int64_t)bg * kHead + d] = L > 0.f ? acc / L : 0.f;
}

// The merge for up to NG*kFewSplits splits: group x (kHead threads) merges
// splits [x*per, (x+1)*per) as decode_combine_few_kernel does, in one round
// trip, and group 0 then merges the NG group results in group order.
template <int NG>
__global__ __launch_bounds__(NG * kHead) void decode_combine_wide_kernel(
    const float* __restrict__ part, int splits, float* __restrict__ out) {
  const int bg = blockIdx.x;
  const int x = threadIdx.x / kHead, d = threadIdx.x % kHead;
  const int per = (splits + NG - 1) / NG;
  const int s0 = x * per;
  const int s1 = s0 + per < splits ? s0 + per : splits;
  const float* p = part + (int64_t)bg * splits * kPartStride;
  __shared__ float gm[NG], gl[NG], go[NG][kHead];
  float o[kFewSplits], m[kFewSplits], l[kFewSplits];
#pragma unroll
  for (int t = 0; t < kFewSplits; ++t) {
    int sc = s0 + t < s1 ? s0 + t : s1 - 1;  // past the group's last split: re-read it, weight 0
    if (sc < 0) sc = 0;
    o[t] = p[(int64_t)sc * kPartStride + d];
    m[t] = p[(int64_t)sc * kPartStride + kHead];
    l[t] = p[(int64_t)sc * kPartStride + kHead + 1];
  }
  float M = -INFINITY;
#pragma unroll
  for (int t = 0; t < kFewSplits; ++t)
    if (s0 + t < s1 && l[t] > 0.f) M = fmaxf(M, m[t]);
  float L = 0.f, acc = 0.f;
#pragma unroll
  for (int t = 0; t < kFewSplits; ++t) {
    const float w = (s0 + t < s1 && l[t] > 0.f) ? __expf(m[t] - M) : 0.f;
    L = fmaf(l[t], w, L);
    acc = fmaf(o[t], w, acc);
  }
  go[x][d] = acc;
  if (d == 0) {
    gm[x] = M;
    gl[x] = L;
  }
  __syncthreads();
  if (x == 0) {
    float MM = -INFINITY;
#pragma unroll
    for (int y = 0; y < NG; ++y)
      if (gl[y] > 0.f) MM = fmaxf(MM, gm[y]);
    float LL = 0.f, oo = 0.f;
#pragma unroll
    for (int y = 0; y < NG; ++y) {
      const float w = gl[y] > 0.f ? __expf(gm[y] - MM) : 0.f;
      LL = fmaf(gl[y], w, LL);
      oo = fmaf(go[y][d], w, oo);
    }
    out[(int64_t)bg * kHead + d] = LL > 0.f ? oo / LL : 0.f;
  }
}

hipError_t launch_decode_combine(const float* part, int heads, int splits, float* out,
                                 hipStream_t s) {
  if (splits > kMaxSplits) return hipErrorInvalidValue;
  const unsigned g8 = (unsigned)((heads + kXcds - 1) / kXcds * kXcds);
  if (splits <= 8) decode_combine_few_kernel<8><<<g8, kHead, 0, s>>>(part, splits, out, heads);
  else if (splits <= 16)
    decode_combine_few_kernel<16><<<g8, kHead, 0, s>>>(part, splits, out, heads);
  else if (splits <= kFewSplits)
    decode_combine_few_kernel<kFewSplits><<<g8, kHead, 0, s>>>(part, splits, out, heads);
  else if (splits <= 4 * kFewSplits)
    decode_combine_wide_kernel<4><<<heads, 4 * kHead, 0, s>>>(part, splits, out);
  else if (splits <= 8 * kFewSplits)
    decode_combine_wide_kernel<8><<<heads, 8 * kHead, 0, s>>>(part, splits, out);
  else decode_combine_kernel<<<heads, kHead, 0, s>>>(part, splits, out);
  return hipGetLastError();
}

}  // namespace socketlsh
