// Hard-LSH comparison mode: the estimator SOCKET is compared with (SOCKET
// Sec. 3.1 and Sec. 5.3; Appendix A.2 "Ablations for Hard LSH Estimator",
// where hard LSH does best at P = 2 with L = 300 or 500 tables): a key
// scores its value norm times the number of tables in which it falls into
// the query's own bucket,
//   s_i = ||v_i|| * #{ l : b_l(k_i) == b_l(q) },
// the tau -> 0 limit of the soft score.
//
// A key's bucket IDs are kept as one packed sign code: bit p = l*P + j is the
// sign of plane j of table l (the order of the rows of W), 32 bits a word,
// ceil(L*P/32) words, stored word-major so that a wave reading word w of 64
// consecutive keys reads 256 contiguous bytes.  With P dividing 32 no table
// straddles two words: a table matches when its P-bit group of
// (key code XOR query code) is zero, which the scorer finds by OR-folding
// each group into its lowest bit and counting with one popcount per word.
// The scores (and a first-digit histogram of those that compete) go through
// the same top-k kernels as the soft scores.
#include "common.h"
#include "launch.h"

namespace socketlsh {

int codes_words(int L, int P) { return (L * P + 31) / 32; }

template <typename T>
__device__ __forceinline__ void row8(const T* p, float* f);
template <>
__device__ __forceinline__ void row8<uint16_t>(const uint16_t* p, float* f) {
  unpack_bf16x8(*reinterpret_cast<const uint4*>(p), f);
}
template <>
__device__ __forceinline__ void row8<float>(const float* p, float* f) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// ---------------------------------------------------------------- codes

// grid: rows*S one-wave blocks, S = ceil(L*P/64).  Block (row, s) projects
// key row `row` (position pos0[b] + c; pos0 == nullptr means 0) on planes
// 64s .. 64s+63, one per lane, in float32 (bf16 products are exact), and
// stores the two code words the wave ballot gives.  Slice 0 also stores the
// value norm when V is given.  When hist is given (query codes), the blocks
// of a row also clear its selection histogram and candidate counter.
template <typename T>
__global__ __launch_bounds__(64) void hash_codes_kernel(
    const T* __restrict__ K, const T* __restrict__ V, int Hkv, int64_t n_cap,
    const int32_t* __restrict__ pos0, int count, const T* __restrict__ W, int LP, int WPK, int S,
    uint32_t* __restrict__ codes, float* __restrict__ vnorm, uint32_t* __restrict__ hist,
    uint32_t* __restrict__ counters) {
  constexpr int NV = kHead * (int)sizeof(T) / 16;
  const int s = blockIdx.x % S;
  const int rc = blockIdx.x / S;
  const int c = rc % count;
  const int bh = rc / count;
  const int b = bh / Hkv;
  const int lane = threadIdx.x;
  const int p = s * 64 + lane;
  const bool live = p < LP;
  if (hist) {
    for (int i = s * 64 + lane; i < kHistBins; i += S * 64) hist[(int64_t)bh * kHistBins + i] = 0u;
    if (s == 0 && lane == 0) counters[bh] = 0u;
  }
  uint4 wv[NV];
  if (live) {
    const uint4* wr = reinterpret_cast<const uint4*>(W + (int64_t)p * kHead);
#pragma unroll
    for (int v = 0; v < NV; ++v) wv[v] = wr[v];
  }
  const int64_t pos = (pos0 ? (int64_t)pos0[b] : 0) + c;
  if (pos < 0 || pos >= n_cap) return;
  __shared__ float kf[kHead];
  float vf[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) vf[i] = 0.f;
  const int64_t row = (int64_t)bh * n_cap + pos;
  if (lane < 16) row8<T>(K + row * kHead + 8 * lane, kf + 8 * lane);
  const bool norm = V != nullptr && s == 0;
  if (norm && lane >= 16 && lane < 32) row8<T>(V + row * kHead + 8 * (lane - 16), vf);
  __syncthreads();
  float z = 0.f;
  if (live) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      float f[8];
      int cnt;
      if constexpr (sizeof(T) == 2) {
        unpack_bf16x8(wv[v], f);
        cnt = 8;
      } else {
        f[0] = __uint_as_float(wv[v].x); f[1] = __uint_as_float(wv[v].y);
        f[2] = __uint_as_float(wv[v].z); f[3] = __uint_as_float(wv[v].w);
        cnt = 4;
      }
#pragma unroll
      for (int e = 0; e < cnt; ++e) z = fmaf(f[e], kf[v * cnt + e], z);
    }
  }
  const uint64_t m = __ballot(live && z > 0.f);  // z == 0 gives bit 0
  if (norm) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(vf[i], vf[i], ss);
    ss = row16_sum(ss);
    if (lane == 16) vnorm[row] = sqrtf(ss);
  }
  const int w = 2 * s + lane;  // lanes 0 and 1 store the slice's two words
  if (lane < 2 && w < WPK)
    codes[((int64_t)bh * WPK + w) * n_cap + pos] = lane ? (uint32_t)(m >> 32) : (uint32_t)m;
}

hipError_t launch_hash_codes(const void* K, const void* V, int dtype, int B, int Hkv,
                             int64_t n_cap, const int32_t* pos0, int count, const void* W, int L,
                             int P, uint32_t* codes, float* vnorm, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const int LP = L * P, WPK = codes_words(L, P), S = (LP + 63) / 64;
  if (dtype == 1 && pos0 && V && vnorm && count >= 64)  // bf16 prefill: the MFMA GEMM
    return launch_hash_codes_mfma(static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V),
                                  B, Hkv, n_cap, pos0, count, static_cast<const uint16_t*>(W), LP,
                                  WPK, codes, vnorm, s);
  const dim3 grid((unsigned)((int64_t)B * Hkv * count * S));
  if (dtype == 1)
    hash_codes_kernel<uint16_t><<<grid, 64, 0, s>>>(
        static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V), Hkv, n_cap, pos0, count,
        static_cast<const uint16_t*>(W), LP, WPK, S, codes, vnorm, nullptr, nullptr);
  else
    hash_codes_kernel<float><<<grid, 64, 0, s>>>(
        static_cast<const float*>(K), static_cast<const float*>(V), Hkv, n_cap, pos0, count,
        static_cast<const float*>(W), LP, WPK, S, codes, vnorm, nullptr, nullptr);
  return hipGetLastError();
}

// ---------------------------------------------------------------- scorer

constexpr int kHardThreads = 256;
constexpr int kHardUnroll = 8;  // code words loaded together per key

// Matching tables of one code word: after folding, bit P*t of y is set when
// any bit of group t of x is; `low` has bit P*t set for the valid groups.
template <int P>
__device__ __forceinline__ uint32_t group_matches(uint32_t x, uint32_t low) {
  if constexpr (P >= 2) x |= x >> 1;
  if constexpr (P >= 4) x |= x >> 2;
  if constexpr (P >= 8) x |= x >> 4;
  if constexpr (P >= 16) x |= x >> 8;
  return (uint32_t)__popc(~x & low);
}

// grid: a multiple of kXcds blocks, at least rows*nblk; logical block lid
// (XCD-local as in the soft scorer) takes keys [blk*kpb, (blk+1)*kpb) of
// sub-row lid / nblk, one key per thread at a time, for its G query heads.
// Sub-rows as in the soft scorer: Hkv of them per sequence, sub-row bh reading
// the codes and norms of KV row bh / sub.
template <int G, int P>
__global__ __launch_bounds__(kHardThreads) void hard_scorer_kernel(
    const uint32_t* __restrict__ qcodes, const uint32_t* __restrict__ codes,
    const float* __restrict__ vnorm, const int32_t* __restrict__ lens, int Hq, int Hkv, int sub,
    int LP, int WPK, int64_t n_cap, int sink, int window, int rows, int nblk, int kpb,
    float* __restrict__ scores, uint32_t* __restrict__ hist) {
  const int lid = (int)(blockIdx.x % kXcds) * (int)(gridDim.x / kXcds) + (int)(blockIdx.x / kXcds);
  if (lid >= rows * nblk) return;
  const int blk = lid % nblk, bh = lid / nblk;
  const int b = bh / Hkv, h = bh % Hkv;
  int64_t n = lens[b];
  if (n < 0) n = 0;
  if (n > n_cap) n = n_cap;
  const int64_t f_lo = sink < n ? sink : n;
  const int64_t f_hi = n - window > 0 ? n - window : 0;
  const int64_t k0 = (int64_t)blk * kpb;
  const int64_t k1 = k0 + kpb < n ? k0 + kpb : n;
  if (k0 >= k1) return;
  const int tid = threadIdx.x;
  const int bg0 = b * Hq + h * G;
  const int64_t sst = score_stride(n_cap);
  __shared__ uint32_t lhist[G * kHistBins];
  for (int i = tid; i < G * kHistBins; i += kHardThreads) lhist[i] = 0u;
  __syncthreads();

  // low bit of every valid P-bit group of word w
  uint32_t lowpat = 0u;
  for (int t = 0; t < 32; t += P) lowpat |= 1u << t;
  const int kv = bh / sub;  // the KV row of this sub-row
  const uint32_t* crow = codes + (int64_t)kv * WPK * n_cap;
  const uint32_t* qrow = qcodes + (int64_t)bg0 * WPK;  // uniform: scalar loads
  for (int64_t key = k0 + tid; key < k1; key += kHardThreads) {
    uint32_t cnt[G];
#pragma unroll
    for (int g = 0; g < G; ++g) cnt[g] = 0u;
    for (int w0 = 0; w0 < WPK; w0 += kHardUnroll) {
      uint32_t kw[kHardUnroll];
#pragma unroll
      for (int i = 0; i < kHardUnroll; ++i) {
        const int w = w0 + i < WPK ? w0 + i : WPK - 1;  // past the code: re-read, masked below
        kw[i] = crow[(int64_t)w * n_cap + key];
      }
#pragma unroll
      for (int i = 0; i < kHardUnroll; ++i) {
        const int w = w0 + i;
        const int rem = LP - 32 * w;
        const uint32_t low = w >= WPK ? 0u : rem >= 32 ? lowpat : lowpat & ((1u << rem) - 1u);
        const int wq = w < WPK ? w : WPK - 1;
#pragma unroll
        for (int g = 0; g < G; ++g) cnt[g] += group_matches<P>(kw[i] ^ qrow[g * WPK + wq], low);
      }
    }
    const float vn = vnorm[(int64_t)kv * n_cap + key];
    const bool ranked = key >= f_lo && key < f_hi;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sv = vn * (float)cnt[g];
      scores[(int64_t)(bg0 + g) * sst + key] = sv;
      uint32_t dg = __float_as_uint(sv) >> kHistShift;
      if (dg > kHistBins - 1) dg = kHistBins - 1;
      if (ranked) atomicAdd(&lhist[g * kHistBins + dg], 1u);
    }
  }
  __syncthreads();
  for (int i = tid; i < G * kHistBins; i += kHardThreads) {
    const uint32_t v = lhist[i];
    if (v) atomicAdd(&hist[(int64_t)(bg0 + i / kHistBins) * kHistBins + (i % kHistBins)], v);
  }
}

static int device_cu_count() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
      cus = prop.multiProcessorCount;
    if (cus <= 0) cus = 256;
  }
  return cus;
}

hipError_t launch_hard_score(const void* q, int dtype, int B, int Hq, int Hkv, const void* W,
                             int L, int P, const uint32_t* codes, const float* vnorm,
                             const int32_t* lens, int64_t n_cap, SinkWindow sw, float* scores,
                             const ScoreWs& ws, hipStream_t s) {
  const int LP = L * P, WPK = codes_words(L, P), S = (LP + 63) / 64;
  // the query codes (each query head as a one-key row), clearing the histograms
  const dim3 qgrid((unsigned)((int64_t)B * Hq * S));
  if (dtype == 1)
    hash_codes_kernel<uint16_t><<<qgrid, 64, 0, s>>>(
        static_cast<const uint16_t*>(q), nullptr, Hq, 1, nullptr, 1,
        static_cast<const uint16_t*>(W), LP, WPK, S, ws.qcodes, nullptr, ws.hist, ws.counters);
  else
    hash_codes_kernel<float><<<qgrid, 64, 0, s>>>(
        static_cast<const float*>(q), nullptr, Hq, 1, nullptr, 1, static_cast<const float*>(W), LP,
        WPK, S, ws.qcodes, nullptr, ws.hist, ws.counters);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // about four blocks per CU over the sub-rows
  const int G = Hq / Hkv, GK = pass_heads(G), sub = pass_subs(G);
  const int Hv = Hkv * sub;
  const int64_t rows = (int64_t)B * Hv;
  int64_t nblk = (4 * device_cu_count() + rows - 1) / rows;
  int64_t kpb = (n_cap + nblk - 1) / nblk;
  kpb = (kpb + kHardThreads - 1) / kHardThreads * kHardThreads;
  nblk = (n_cap + kpb - 1) / kpb;
  const int64_t grid = (rows * nblk + kXcds - 1) / kXcds * kXcds;
  auto go = [&](auto gt, auto pt) {
    constexpr int GG = decltype(gt)::value, PP = decltype(pt)::value;
    hard_scorer_kernel<GG, PP><<<(unsigned)grid, kHardThreads, 0, s>>>(
        ws.qcodes, codes, vnorm, lens, Hq, Hv, sub, LP, WPK, n_cap, sw.sink, sw.window,
        (int)rows, (int)nblk, (int)kpb, scores, ws.hist);
  };
  auto by_p = [&](auto gt) {
    switch (P) {
      case 1: go(gt, std::integral_constant<int, 1>{}); break;
      case 2: go(gt, std::integral_constant<int, 2>{}); break;
      case 4: go(gt, std::integral_constant<int, 4>{}); break;
      case 8: go(gt, std::integral_constant<int, 8>{}); break;
      default: go(gt, std::integral_constant<int, 16>{}); break;
    }
  };
  if (GK == 1) by_p(std::integral_constant<int, 1>{});
  else if (GK == 2) by_p(std::integral_constant<int, 2>{});
  else by_p(std::integral_constant<int, 4>{});
  return hipGetLastError();
}

}  // namespace socketlsh
