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
constexpr int kSplitKeys = 64;  // entries of idx per workgroup
constexpr int kPartStride = kHead + 2;

static inline size_t align256d(size_t x) { return (x + 255) & ~(size_t)255; }

size_t decode_ws_layout(int B, int Hq, int k_max, DecodeWs* ws, void* base) {
  const int splits = (k_max + kSplitKeys - 1) / kSplitKeys;
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

// Load 8 consecutive head elements [8*j, 8*j+8) of a row as floats.
template <typename T>
__device__ __forceinline__ void load_row8(const T* row, int j, float* f);
template <>
__device__ __forceinline__ void load_row8<uint16_t>(const uint16_t* row, int j, float* f) {
  const uint4 v = reinterpret_cast<const uint4*>(row)[j];
  unpack_bf16x8(v, f);
}
template <>
__device__ __forceinline__ void load_row8<float>(const float* row, int j, float* f) {
  const float4 a = reinterpret_cast<const float4*>(row)[2 * j];
  const float4 b = reinterpret_cast<const float4*>(row)[2 * j + 1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
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
  __shared__ int32_t rows[kSplitKeys];
  __shared__ float red[kDecWaves * 4][kHead];
  __shared__ float sh_m, sh_l;

  float qf[8];
  load_row8<T>(q + (int64_t)bg * kHead, j, qf);
  const int32_t* irow = idx + (int64_t)bg * k_max;
  const int64_t kvbase = ((int64_t)b * Hkv + h) * n_cap;

  // logits: row (wave, kg) takes entries t0 + wave*4 + kg, +16, ...
  for (int t = wave * 4 + kg; t < nt; t += kDecWaves * 4) {
    int32_t i = irow[t0 + t];
    if (i >= n_cap) i = -1;  // out-of-range entries are skipped like padding
    float dot = 0.f;
    if (i >= 0) {
      float kf[8];
      load_row8<T>(K + (kvbase + i) * kHead, j, kf);
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(qf[e], kf[e], dot);
    }
    dot = row16_sum(dot);
    if (j == 0) {
      logit[t] = i >= 0 ? dot * scale : -INFINITY;
      rows[t] = i;
    }
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
  for (int t = wave * 4 + kg; t < nt; t += kDecWaves * 4) {
    const int32_t i = rows[t];
    if (i >= 0) {
      const float p = logit[t];
      float vf[8];
      load_row8<T>(V + (kvbase + i) * kHead, j, vf);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(p, vf[e], acc[e]);
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

// grid: B*Hq blocks of 128 threads.  Merges the splits in index order.
__global__ __launch_bounds__(kHead) void decode_combine_kernel(const float* __restrict__ part,
                                                               int splits,
                                                               float* __restrict__ out) {
  const int bg = blockIdx.x;
  const int d = threadIdx.x;
  const float* p = part + (int64_t)bg * splits * kPartStride;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) {
    const float* ps = p + (int64_t)s * kPartStride;
    if (ps[kHead + 1] > 0.f) M = fmaxf(M, ps[kHead]);
  }
  float L = 0.f, o = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float* ps = p + (int64_t)s * kPartStride;
    const float ls = ps[kHead + 1];
    if (ls > 0.f) {
      const float w = __expf(ps[kHead] - M);
      L = fmaf(ls, w, L);
      o = fmaf(ps[d], w, o);
    }
  }
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
  decode_combine_kernel<<<heads, kHead, 0, s>>>(ws.part, ws.splits, out);
  return hipGetLastError();
}

}  // namespace socketlsh
