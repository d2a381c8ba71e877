// The value-aware sampling estimator T(q) of the SOCKET analysis (Sec. 5.1
// "Sampling-based Estimator", Theorem 3; Appendix B.2): with soft counts
// s~_j = sum_l p_l(b_l(k_j) | q), soft attention weights a~_j = s~_j / Z~,
// Z~ = sum_j s~_j, draw M keys J_m with probability
//   p_j = a~_j ||v_j|| / S_1,   S_1 = sum_j a~_j ||v_j||,
// and average X_m = a~_J v_J / p_J = S_1 v_J / ||v_J||:
//   T(q) = (S_1 / M) sum_m v_J / ||v_J||,
// an unbiased estimate of the soft-attention output sum_j a~_j v_j.  Since
// a~_j ||v_j|| = s_j / Z~ with s_j the SOCKET score (value norm times soft
// count), p_j is proportional to s_j and S_1 = (sum_j s_j) / Z~.
//
// The random numbers are inputs: draw m of head (b, g) uses the uniform
// u[b][g][m] in [0, 1) and takes the first key whose running score sum
// exceeds u * sum_j s_j (keys without mass are never drawn).
//
// One workgroup per query head: thread t sums the scores of keys
// [t*C, (t+1)*C) in key order, a block scan turns those into chunk starts,
// and each draw finds its chunk by binary search over the starts and its key
// by walking the chunk in order.  The drawn value rows are then summed in a
// fixed order: 16 lanes per row, 64 row slots (slot r takes draws r, r + 64,
// ...), the slots added up in LDS.
#include "common.h"
#include "launch.h"

namespace socketlsh {

constexpr int kEstThreads = 1024;
constexpr int kEstWaves = kEstThreads / 64;
constexpr int kEstMaxDraws = 8192;
constexpr int kEstSlots = kEstThreads / 16;  // value rows gathered at once (16 lanes a row)
constexpr int kEstBatch = 8;   // scores loaded together along a chunk
constexpr int kEstRowBatch = 4;  // value rows per lane in flight

// Elements 8j .. 8j+7 of a value row as float32.
template <typename T>
__device__ __forceinline__ void elems8(const T* row, int j, float* f);
template <>
__device__ __forceinline__ void elems8<uint16_t>(const uint16_t* row, int j, float* f) {
  unpack_bf16x8(reinterpret_cast<const uint4*>(row)[j], f);
}
template <>
__device__ __forceinline__ void elems8<float>(const float* row, int j, float* f) {
  const float4 a = reinterpret_cast<const float4*>(row)[2 * j];
  const float4 b = reinterpret_cast<const float4*>(row)[2 * j + 1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// grid: B*Hq blocks of kEstThreads.
template <typename T>
__global__ __launch_bounds__(kEstThreads) void estimate_kernel(
    const float* __restrict__ scores, int64_t sstride, const float* __restrict__ vnorm,
    const T* __restrict__ V, const int32_t* __restrict__ lens, int Hq, int Hkv, int64_t n_cap,
    const float* __restrict__ usum, const float* __restrict__ u, int M, float* __restrict__ out,
    int32_t* __restrict__ draws) {
  const int bg = blockIdx.x;
  const int b = bg / Hq, h = (bg % Hq) / (Hq / Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t n = lens[b];
  if (n < 0) n = 0;
  if (n > n_cap) n = n_cap;
  __shared__ float cstart[kEstThreads + 1];
  __shared__ float wtot[kEstWaves];
  __shared__ int32_t J[kEstMaxDraws];
  __shared__ float part[kEstSlots][kHead];

  // chunk sums in key order, then an exclusive scan of them
  const float* srow = scores + (int64_t)bg * sstride;
  const int64_t C = (n + kEstThreads - 1) / kEstThreads;
  const int64_t j0 = (int64_t)tid * C;
  const int64_t j1 = j0 + C < n ? j0 + C : n;
  float cs = 0.f;
  for (int64_t j = j0; j < j1; j += kEstBatch) {
    float v[kEstBatch];
#pragma unroll
    for (int i = 0; i < kEstBatch; ++i) v[i] = srow[j + i < j1 ? j + i : j1 - 1];
#pragma unroll
    for (int i = 0; i < kEstBatch; ++i) cs += j + i < j1 ? v[i] : 0.f;
  }
  float inc = cs;
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wtot[wave] = inc;
  __syncthreads();
  float before = 0.f;
  for (int w = 0; w < wave; ++w) before += wtot[w];
  cstart[tid] = before + inc - cs;
  if (tid == kEstThreads - 1) cstart[kEstThreads] = before + inc;
  __syncthreads();
  const float S = cstart[kEstThreads];
  const float Z = usum[bg];
  float* o = out + (int64_t)bg * kHead;
  if (n == 0 || !(S > 0.f) || !(Z > 0.f)) {
    if (tid < kHead) o[tid] = 0.f;
    if (draws)
      for (int m = tid; m < M; m += kEstThreads) draws[(int64_t)bg * M + m] = -1;
    return;
  }

  // draws
  const float top = __uint_as_float(__float_as_uint(S) - 1u);  // the float below S (> 0)
  for (int m = tid; m < M; m += kEstThreads) {
    float t = u[(int64_t)bg * M + m] * S;
    if (t > top) t = top;
    int lo = 0, hi = kEstThreads - 1;  // last chunk whose start is <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cstart[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    int64_t pick = -1, last = -1;
    float acc = cstart[lo];
    const int64_t c1 = (int64_t)(lo + 1) * C < n ? (int64_t)(lo + 1) * C : n;
    for (int64_t j = (int64_t)lo * C; j < c1 && pick < 0; j += kEstBatch) {
      float v[kEstBatch];
#pragma unroll
      for (int i = 0; i < kEstBatch; ++i) v[i] = srow[j + i < c1 ? j + i : c1 - 1];
#pragma unroll
      for (int i = 0; i < kEstBatch; ++i) {
        if (pick < 0 && j + i < c1) {
          if (v[i] > 0.f) last = j + i;
          acc += v[i];
          if (acc > t) pick = j + i;
        }
      }
    }
    // rounding between the scan and the walk: take the last key with mass
    // at or before the chunk end (some key has mass, since S > 0)
    if (pick < 0 || !(srow[pick] > 0.f)) {
      pick = last;
      const int64_t from = (int64_t)lo * C < n ? (int64_t)lo * C : n;
      for (int64_t j = from - 1; pick < 0 && j >= 0; --j)
        if (srow[j] > 0.f) pick = j;
      for (int64_t j = from; pick < 0 && j < n; ++j)
        if (srow[j] > 0.f) pick = j;
    }
    J[m] = (int32_t)pick;
    if (draws) draws[(int64_t)bg * M + m] = (int32_t)pick;
  }
  __syncthreads();

  // sum of v_J / ||v_J||: slot r takes draws r, r + 64, ...; lane j of the
  // slot's 16 owns elements 8j .. 8j+7
  const int r = tid >> 4, j = tid & 15;
  const int64_t rowbase = ((int64_t)b * Hkv + h) * n_cap;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int m0 = r; m0 < M; m0 += kEstSlots * kEstRowBatch) {
    float x[kEstRowBatch][8], nv[kEstRowBatch];
#pragma unroll
    for (int i = 0; i < kEstRowBatch; ++i) {  // past the last draw: re-read it, add nothing
      const int m = m0 + i * kEstSlots;
      const int64_t row = rowbase + J[m < M ? m : r];
      elems8<T>(V + row * kHead, j, x[i]);
      nv[i] = vnorm[row];
    }
#pragma unroll
    for (int i = 0; i < kEstRowBatch; ++i) {
      if (m0 + i * kEstSlots < M) {
        const float inv = 1.f / nv[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(x[i][e], inv, acc[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[r][8 * j + e] = acc[e];
  __syncthreads();
  if (tid < kHead) {
    float t = 0.f;
    for (int g = 0; g < kEstSlots; ++g) t += part[g][tid];
    o[tid] = (S / Z) / (float)M * t;
  }
}

hipError_t launch_estimate(const float* scores, const float* vnorm, const void* V, int dtype,
                           int B, int Hq, int Hkv, const int32_t* lens, int64_t n_cap,
                           const float* u, int M, float* out, int32_t* draws, const ScoreWs& ws,
                           hipStream_t s) {
  if (M > kEstMaxDraws) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(B * Hq);
  if (dtype == 1)
    estimate_kernel<uint16_t><<<grid, kEstThreads, 0, s>>>(
        scores, score_stride(n_cap), vnorm, static_cast<const uint16_t*>(V), lens, Hq, Hkv, n_cap,
        ws.usum, u, M, out, draws);
  else
    estimate_kernel<float><<<grid, kEstThreads, 0, s>>>(
        scores, score_stride(n_cap), vnorm, static_cast<const float*>(V), lens, Hq, Hkv, n_cap,
        ws.usum, u, M, out, draws);
  return hipGetLastError();
}

}  // namespace socketlsh
