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
// Spread over the chip: the scorer leaves, besides the scores, each head's
// score sum over every 64-key group.  Workgroup (head, slice) of
// estimate_draw_kernel takes draws [256*slice, 256*slice + 256):
//  * thread t sums the groups of its run [t*R, (t+1)*R) (R = ceil(groups /
//    256)) in group order, and a block scan of the run totals gives the run
//    starts (the same in every slice of the head);
//  * thread t's draw finds its run by binary search over the run starts, its
//    group by walking the run's group sums, its key by walking the group's
//    64 scores in key order;
//  * the slice's drawn value rows are summed in a fixed order (16 lanes per
//    row, 16 row slots, slot r taking draws r, r + 16, ...).
// estimate_merge_kernel adds the slices of each head in slice order.  The
// fp32 group sums and the in-group walk need not agree to the last bit: a
// draw whose running sum falls in the rounding gap at the end of a group takes
// the group's last key with mass.
#include "common.h"
#include "launch.h"

namespace socketlsh {

constexpr int kDrawThreads = 256;  // draws per slice, one a thread
constexpr int kEstMaxDraws = kEstSlices * kDrawThreads;
constexpr int kEstRowSlots = kDrawThreads / 16;

// grid: B*Hq*slices blocks of kDrawThreads, slices = ceil(M / kDrawThreads).
template <typename T>
__global__ __launch_bounds__(kDrawThreads) void estimate_draw_kernel(
    const float* __restrict__ scores, int64_t sstride, const float* __restrict__ gsum,
    int64_t gstride, const float* __restrict__ vnorm, const T* __restrict__ V,
    const int32_t* __restrict__ lens, int Hq, int Hkv, int64_t n_cap,
    const float* __restrict__ usum, const float* __restrict__ u, int M, int slices,
    float* __restrict__ epart, float* __restrict__ esz, int32_t* __restrict__ draws) {
  const int bg = blockIdx.x / slices, sl = blockIdx.x % slices;
  const int b = bg / Hq, h = (bg % Hq) / (Hq / Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t n = lens[b];
  if (n < 0) n = 0;
  if (n > n_cap) n = n_cap;
  const int64_t G = (n + 63) >> 6;
  const int64_t R = (G + kDrawThreads - 1) / kDrawThreads;
  __shared__ float rstart[kDrawThreads + 1];
  __shared__ float wtot[kDrawThreads / 64];
  __shared__ int32_t J[kDrawThreads];
  __shared__ float part[kEstRowSlots][kHead];
  const float* gs = gsum + (int64_t)bg * gstride;
  const float* srow = scores + (int64_t)bg * sstride;

  // run totals in group order (four group sums requested at a time), then
  // their exclusive scan
  const int64_t g0 = (int64_t)tid * R;
  const int64_t g1 = g0 + R < G ? g0 + R : G;
  float tot = 0.f;
  for (int64_t g = g0; g < g1; g += 4) {
    float x[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = gs[g + q < g1 ? g + q : g1 - 1];
#pragma unroll
    for (int q = 0; q < 4; ++q) tot = g + q < g1 ? tot + x[q] : tot;
  }
  float inc = tot;
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wtot[wave] = inc;
  __syncthreads();
  float before = 0.f;
  for (int w = 0; w < wave; ++w) before += wtot[w];
  rstart[tid] = before + inc - tot;
  if (tid == kDrawThreads - 1) rstart[kDrawThreads] = before + inc;
  __syncthreads();
  const float S = rstart[kDrawThreads];
  const float Z = usum[bg];
  if (sl == 0 && tid == 0) {
    esz[2 * bg] = S;
    esz[2 * bg + 1] = Z;
  }
  float* pout = epart + ((int64_t)bg * kEstSlices + sl) * kHead;
  const int m = sl * kDrawThreads + tid;
  if (n == 0 || !(S > 0.f) || !(Z > 0.f)) {  // uniform: nothing to draw
    if (draws && m < M) draws[(int64_t)bg * M + m] = -1;
    if (tid < kHead) pout[tid] = 0.f;
    return;
  }

  // this thread's draw: run, then group, then key
  int32_t pick = -1;
  if (m < M) {
    const float top = __uint_as_float(__float_as_uint(S) - 1u);  // the float below S (> 0)
    float t = u[(int64_t)bg * M + m] * S;
    if (t > top) t = top;
    int lo = 0, hi = kDrawThreads - 1;  // last run whose start is <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (rstart[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    const int64_t r0 = (int64_t)lo * R;
    const int64_t r1 = r0 + R < G ? r0 + R : G;
    float acc = rstart[lo];
    int64_t g = r1 - 1;  // rounding past the run's end: its last group
    bool found = false;
    for (int64_t x0 = r0; x0 < r1 && !found; x0 += 4) {  // four group sums a step
      float gv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) gv[q] = gs[x0 + q < r1 ? x0 + q : r1 - 1];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool ok = !found && x0 + q < r1;
        const bool hit = ok && acc + gv[q] > t;
        g = hit ? x0 + q : g;
        acc = ok && !hit ? acc + gv[q] : acc;
        found = found || hit;
      }
    }
    // the group's keys in order
    const int64_t k0 = g * 64;
    float v[64];
    const uint4* src = reinterpret_cast<const uint4*>(srow + k0);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint4 w4 = src[q];  // the score row is padded to whole groups
      v[4 * q] = __uint_as_float(w4.x); v[4 * q + 1] = __uint_as_float(w4.y);
      v[4 * q + 2] = __uint_as_float(w4.z); v[4 * q + 3] = __uint_as_float(w4.w);
    }
    // branch-free: the running sum over the group's valid keys in key order;
    // the first key with mass whose running sum exceeds t, and the last key
    // with mass
    const int lim = n - k0 < 64 ? (int)(n - k0) : 64;
    int first = -1, lastm = -1;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const float vi = i < lim ? v[i] : 0.f;
      acc += vi;
      const bool mass = vi > 0.f;
      lastm = mass ? i : lastm;
      first = first < 0 && mass && acc > t ? i : first;
    }
    if (first >= 0) pick = (int32_t)(k0 + first);
    const int64_t last = lastm >= 0 ? k0 + lastm : -1;
    // rounding between the sums and the walk: the group's last key with mass,
    // else the nearest key with mass before the group, else after it
    if (pick < 0) pick = (int32_t)last;
    for (int64_t j = k0 - 1; pick < 0 && j >= 0; --j)
      if (srow[j] > 0.f) pick = (int32_t)j;
    for (int64_t j = k0 + 64; pick < 0 && j < n; ++j)
      if (srow[j] > 0.f) pick = (int32_t)j;
    if (draws) draws[(int64_t)bg * M + m] = pick;
  }
  J[tid] = pick;
  __syncthreads();

  // sum of v_J / ||v_J|| over the slice's draws: slot r takes draws r, r + 16, ...;
  // lane j of the slot's 16 owns elements 8j .. 8j+7
  const int nd = M - sl * kDrawThreads < kDrawThreads ? M - sl * kDrawThreads : kDrawThreads;
  const int r = tid >> 4, j = tid & 15;
  const int64_t rowbase = ((int64_t)b * Hkv + h) * n_cap;
  float a8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) a8[e] = 0.f;
  // value rows in flight per lane: a slot's whole share of a full slice for bf16
  constexpr int RB = sizeof(T) == 2 ? kDrawThreads / kEstRowSlots : kDrawThreads / kEstRowSlots / 2;
  for (int d0 = r; d0 < nd; d0 += kEstRowSlots * RB) {
    Row8<T> x[RB];
    float nv[RB];
    bool use[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {  // past the last draw: read row 0, add nothing
      const int d = d0 + i * kEstRowSlots;
      const int32_t jd = d < nd ? J[d] : -1;
      use[i] = jd >= 0;
      const int64_t row = rowbase + (jd >= 0 ? jd : 0);
      x[i] = fetch_row8<T>(V + row * kHead, j);
      nv[i] = vnorm[row];
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (use[i]) {
        float f[8];
        unpack_row8<T>(x[i], f);
        const float inv = 1.f / nv[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) a8[e] = fmaf(f[e], inv, a8[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[r][8 * j + e] = a8[e];
  __syncthreads();
  if (tid < kHead) {
    float t = 0.f;
    for (int g = 0; g < kEstRowSlots; ++g) t += part[g][tid];
    pout[tid] = t;
  }
}

// grid: B*Hq blocks of kHead threads: out = (S / Z) / M * (sum of the slices).
__global__ __launch_bounds__(kHead) void estimate_merge_kernel(
    const float* __restrict__ epart, const float* __restrict__ esz, int M, int slices,
    float* __restrict__ out) {
  const int bg = blockIdx.x, d = threadIdx.x;
  const float S = esz[2 * bg], Z = esz[2 * bg + 1];
  float t = 0.f;
  for (int sl = 0; sl < slices; ++sl) t += epart[((int64_t)bg * kEstSlices + sl) * kHead + d];
  out[(int64_t)bg * kHead + d] = (S > 0.f && Z > 0.f) ? (S / Z) / (float)M * t : 0.f;
}

hipError_t launch_estimate(const float* scores, const float* vnorm, const void* V, int dtype,
                           int B, int Hq, int Hkv, const int32_t* lens, int64_t n_cap,
                           const float* u, int M, float* out, int32_t* draws, const ScoreWs& ws,
                           hipStream_t s) {
  if (M <= 0 || M > kEstMaxDraws) return hipErrorInvalidValue;
  const int slices = (M + kDrawThreads - 1) / kDrawThreads;
  const unsigned grid = (unsigned)(B * Hq * slices);
  if (dtype == 1)
    estimate_draw_kernel<uint16_t><<<grid, kDrawThreads, 0, s>>>(
        scores, score_stride(n_cap), ws.gsum, ws.groups, vnorm, static_cast<const uint16_t*>(V),
        lens, Hq, Hkv, n_cap, ws.usum, u, M, slices, ws.epart, ws.esz, draws);
  else
    estimate_draw_kernel<float><<<grid, kDrawThreads, 0, s>>>(
        scores, score_stride(n_cap), ws.gsum, ws.groups, vnorm, static_cast<const float*>(V),
        lens, Hq, Hkv, n_cap, ws.usum, u, M, slices, ws.epart, ws.esz, draws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  estimate_merge_kernel<<<(unsigned)(B * Hq), kHead, 0, s>>>(ws.epart, ws.esz, M, slices, out);
  return hipGetLastError();
}

}  // namespace socketlsh
