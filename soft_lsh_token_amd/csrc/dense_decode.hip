// Dense flash-decode: exact softmax attention of each decode query over every
// key of its sequence.  This is the full-attention reference point that the
// SOCKET paper (Sec. 1, contributions; Sec. 6 "Experiments") measures its
// decode speedups against (FlashAttention), at the same shapes as the sparse
// path.
//
// Split-k over the sequence: workgroup (b, h, s) streams keys
// [s*chunk, (s+1)*chunk) of KV row (b, h) once for all G query heads of that
// KV head (grouped-query attention).  A 16-lane row owns one key at a time
// (16 B of K and of V per lane for bf16); the 16 rows of the workgroup take
// consecutive keys, so a wave's loads cover 1 KiB of K and 1 KiB of V
// contiguously.  Each row keeps an online softmax per head (running max m,
// sum l, unnormalised output o) over batches of kDenseU keys whose loads are
// issued one batch ahead.  For bf16 the query-key dot products run on
// v_dot2c_f32_bf16 (two bf16 products per instruction, float32
// accumulation), straight from the loaded words.  The rows are merged in LDS
// and the workgroup writes the same unnormalised partial (o, m, l) per query
// head as the sparse decode, merged by its combine kernel.
#include "common.h"
#include "launch.h"

namespace socketlsh {

constexpr int kDenseThreads = 256;
constexpr int kDenseRows = kDenseThreads / 16;  // keys per workgroup step
constexpr int kDenseU = 4;                      // keys per row per batch
constexpr int kDenseBlocks = 512;               // workgroups aimed for (2 per CU)
constexpr int kDenseMaxSplits = 1024;           // the combine kernel's limit
constexpr int kDensePart = kHead + 2;

static inline size_t align256x(size_t x) { return (x + 255) & ~(size_t)255; }

// Keys per split: about kDenseBlocks workgroups over the B*Hkv KV rows (a
// workgroup's stream must be long enough to keep its loads in flight; with
// fewer, longer splits the chip is not filled), a multiple of
// kDenseRows*kDenseU, and few enough splits for the combine kernel.
int dense_chunk(int B, int Hkv, int64_t n_cap) {
  int64_t c = ((int64_t)B * Hkv * n_cap + kDenseBlocks - 1) / kDenseBlocks;
  const int64_t lo = (n_cap + kDenseMaxSplits - 1) / kDenseMaxSplits;
  if (c < lo) c = lo;
  constexpr int step = kDenseRows * kDenseU;
  return (int)((c + step - 1) / step * step);
}

size_t dense_ws_layout(int B, int Hq, int Hkv, int64_t n_cap, DenseWs* ws, void* base) {
  const int chunk = dense_chunk(B, Hkv * pass_subs(Hq / Hkv), n_cap);  // over the sub-rows
  const int splits = (int)((n_cap + chunk - 1) / chunk);
  const size_t off = align256x((size_t)B * Hq * splits * kDensePart * sizeof(float));
  if (ws) {
    ws->part = static_cast<float*>(base);
    ws->splits = splits;
    ws->chunk = chunk;
  }
  return off;
}

template <typename T>
__device__ __forceinline__ uint4 load16(const T* row, int j, int half);
// bf16: one 16-byte vector = elements 8j .. 8j+7
template <>
__device__ __forceinline__ uint4 load16<uint16_t>(const uint16_t* row, int j, int half) {
  (void)half;
  return reinterpret_cast<const uint4*>(row)[j];
}
// float32: two vectors per lane, elements 8j .. 8j+3 (half 0) and 8j+4 .. 8j+7 (half 1)
template <>
__device__ __forceinline__ uint4 load16<float>(const float* row, int j, int half) {
  return reinterpret_cast<const uint4*>(row)[2 * j + half];
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// c plus the dot product of the 8 bf16 values packed in a and in b
__device__ __forceinline__ float dot8_bf16(const uint4 a, const uint4 b, float c) {
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x),
                                      __builtin_bit_cast(bf16x2_t, b.x), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y),
                                      __builtin_bit_cast(bf16x2_t, b.y), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z),
                                      __builtin_bit_cast(bf16x2_t, b.z), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w),
                                      __builtin_bit_cast(bf16x2_t, b.w), c, false);
  return c;
}

template <typename T>
struct KeyRegs {
  static constexpr int NV = sizeof(T) == 2 ? 1 : 2;  // 16-byte vectors per lane per row
  uint4 k[kDenseU][NV], v[kDenseU][NV];
};

template <typename T>
__device__ __forceinline__ void widen(const uint4 (&r)[KeyRegs<T>::NV], float* f) {
  if constexpr (sizeof(T) == 2) {
    unpack_bf16x8(r[0], f);
  } else {
    f[0] = __uint_as_float(r[0].x); f[1] = __uint_as_float(r[0].y);
    f[2] = __uint_as_float(r[0].z); f[3] = __uint_as_float(r[0].w);
    f[4] = __uint_as_float(r[1].x); f[5] = __uint_as_float(r[1].y);
    f[6] = __uint_as_float(r[1].z); f[7] = __uint_as_float(r[1].w);
  }
}

// grid: B*Hkv*splits blocks of kDenseThreads, Hkv sub-rows per sequence:
// sub-row bh serves query heads b*Hq + (bh % Hkv)*G + [0, G) and reads the K
// and V rows of KV row bh / sub.
template <typename T, int G>
__global__ __launch_bounds__(kDenseThreads) void dense_partial_kernel(
    const T* __restrict__ q, const T* __restrict__ K, const T* __restrict__ V, int Hq, int Hkv,
    int sub, int64_t n_cap, const int32_t* __restrict__ lens, float scale, int splits, int chunk,
    float* __restrict__ part) {
  using Regs = KeyRegs<T>;
  constexpr int NV = Regs::NV;
  const int sp = blockIdx.x % splits;
  const int bh = blockIdx.x / splits;
  const int b = bh / Hkv, h = bh % Hkv;
  const int kv = bh / sub;  // the KV row of this sub-row
  const int tid = threadIdx.x, row = tid >> 4, j = tid & 15;
  int64_t n = lens[b];
  if (n < 0) n = 0;
  if (n > n_cap) n = n_cap;
  const int64_t c0 = (int64_t)sp * chunk;
  const int64_t c1 = c0 + chunk < n ? c0 + chunk : n;
  const int bg0 = b * Hq + h * G;

  // this lane's 8 query elements of each head: packed bf16 (dot2 path) or float32
  constexpr bool kDot2 = sizeof(T) == 2;
  uint4 qp[G];
  float qf[kDot2 ? 1 : G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    uint4 r[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) r[u] = load16<T>(q + (int64_t)(bg0 + g) * kHead, j, u);
    if constexpr (kDot2) qp[g] = r[0];
    else widen<T>(r, qf[g]);
  }
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }

  // batch t: keys c0 + (t*kDenseU + u)*kDenseRows + row, u < kDenseU; loads
  // past the split re-read its first key (always present when the split is
  // not empty) and are masked out of the softmax
  const T* Kr = K + (int64_t)kv * n_cap * kHead;
  const T* Vr = V + (int64_t)kv * n_cap * kHead;
  const int64_t nk = c1 - c0;
  const int nbatch = nk > 0 ? (int)((nk + kDenseRows * kDenseU - 1) / (kDenseRows * kDenseU)) : 0;
  auto issue = [&](int t, Regs& r) {
#pragma unroll
    for (int u = 0; u < kDenseU; ++u) {
      int64_t key = c0 + (int64_t)(t * kDenseU + u) * kDenseRows + row;
      if (key >= c1) key = c0;
#pragma unroll
      for (int x = 0; x < NV; ++x) {
        r.k[u][x] = load16<T>(Kr + key * kHead, j, x);
        r.v[u][x] = load16<T>(Vr + key * kHead, j, x);
      }
    }
  };
  auto consume = [&](int t, const Regs& r) {
    float s[kDenseU][G];
#pragma unroll
    for (int u = 0; u < kDenseU; ++u) {
      const int64_t key = c0 + (int64_t)(t * kDenseU + u) * kDenseRows + row;
      float kf[8];
      if constexpr (!kDot2) widen<T>(r.k[u], kf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
        if constexpr (kDot2) {
          d = dot8_bf16(qp[g], r.k[u][0], 0.f);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) d = fmaf(qf[g][e], kf[e], d);
        }
        d = row16_sum(d);
        s[u][g] = key < c1 ? d * scale : -INFINITY;
      }
    }
    float p[kDenseU][G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = m[g];
#pragma unroll
      for (int u = 0; u < kDenseU; ++u) mx = fmaxf(mx, s[u][g]);
      // mx == -inf only while every key so far was masked: nothing to add
      const float alpha = m[g] == -INFINITY ? 0.f : __expf(m[g] - mx);
      float add = 0.f;
#pragma unroll
      for (int u = 0; u < kDenseU; ++u) {
        p[u][g] = s[u][g] == -INFINITY ? 0.f : __expf(s[u][g] - mx);
        add += p[u][g];
      }
      l[g] = fmaf(l[g], alpha, add);
      m[g] = mx;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < kDenseU; ++u) {
      float vf[8];
      widen<T>(r.v[u], vf);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(p[u][g], vf[e], acc[g][e]);
    }
  };

  Regs ra, rb;
  if (nbatch > 0) issue(0, ra);
  for (int t = 0; t < nbatch; t += 2) {
    if (t + 1 < nbatch) issue(t + 1, rb);
    consume(t, ra);
    if (t + 1 < nbatch) {
      if (t + 2 < nbatch) issue(t + 2, ra);
      consume(t + 1, rb);
    }
  }

  // merge the 16 rows: M = max m_r, o = sum_r o_r e^(m_r - M), L likewise
  __shared__ float red[kDenseRows][G][kHead];
  __shared__ float rm[kDenseRows][G], rl[kDenseRows][G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[row][g][8 * j + e] = acc[g][e];
    if (j == 0) {
      rm[row][g] = m[g];
      rl[row][g] = l[g];
    }
  }
  __syncthreads();
  for (int i = tid; i < G * kHead; i += kDenseThreads) {
    const int g = i / kHead, e = i % kHead;
    float M = -INFINITY;
#pragma unroll
    for (int r = 0; r < kDenseRows; ++r) M = fmaxf(M, rm[r][g]);
    float o = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int r = 0; r < kDenseRows; ++r) {
        const float w = rm[r][g] == -INFINITY ? 0.f : __expf(rm[r][g] - M);
        o = fmaf(red[r][g][e], w, o);
        L = fmaf(rl[r][g], w, L);
      }
    }
    float* out = part + ((int64_t)(bg0 + g) * splits + sp) * kDensePart;
    out[e] = o;
    if (e == 0) {
      out[kHead] = M;
      out[kHead + 1] = L;
    }
  }
}

hipError_t launch_dense_decode(const void* q, const void* K, const void* V, int dtype, int B,
                               int Hq, int Hkv, int64_t n_cap, const int32_t* lens, float scale,
                               float* out, const DenseWs& ws, hipStream_t s) {
  const int G = Hq / Hkv, GK = pass_heads(G), sub = pass_subs(G);
  const unsigned grid = (unsigned)((int64_t)B * Hkv * sub * ws.splits);
  auto go = [&](auto tag, auto gtag) {
    using T = decltype(tag);
    constexpr int GG = decltype(gtag)::value;
    dense_partial_kernel<T, GG><<<grid, kDenseThreads, 0, s>>>(
        static_cast<const T*>(q), static_cast<const T*>(K), static_cast<const T*>(V), Hq,
        Hkv * sub, sub, n_cap, lens, scale, ws.splits, ws.chunk, ws.part);
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  if (dtype == 1) {
    if (GK == 1) go(uint16_t{}, I1{});
    else if (GK == 2) go(uint16_t{}, I2{});
    else go(uint16_t{}, I4{});
  } else {
    if (GK == 1) go(float{}, I1{});
    else if (GK == 2) go(float{}, I2{});
    else go(float{}, I4{});
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine(ws.part, B * Hq, ws.splits, out, s);
}

}  // namespace socketlsh
