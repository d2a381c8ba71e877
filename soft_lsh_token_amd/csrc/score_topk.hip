// Query soft hashing, soft-count scoring and top-k selection
// (SOCKET Sec. 4.1, Algorithms 2 and 3).
//
// Soft hashing: table l gives bucket c the probability
//   p_l(c) = softmax_c( sum_j s_j(c) u_lj / tau ),  s_j(c) = +1 if bit j of c else -1,
// which factorises over the planes as prod_j sigmoid(2 s_j(c) u_lj / tau), so
// p_l(c) = lo_l(c & 15) * hi_l(c >> 4) with 16-entry halves over planes 0..3
// and 4..P-1.  The projections u = W q are taken in float64.
//
// The soft-tables kernel writes, per KV head, an image of the tables of its G
// query heads laid out for the scorer's LDS: as many tables as fit kept in
// full (one lookup per key), the rest as their two halves (two lookups and a
// multiply).  One image slot holds the G heads' values of one entry, so one
// 16-byte LDS read serves all G query heads.
//
// Scorer (one pass per KV head for all of its GQA query heads): lane j of a
// 16-lane row owns TL consecutive tables (j*TL .. j*TL+TL-1) and reads their
// bucket IDs as TL-byte words out of the 16-byte per-lane vectors of the
// tiled ID cache.  Each of the 16 rounds of a 64-key group gives lane j key
// (j + x) mod 16 of its row, and the image slots of lane j sit in bank group
// j, so the 16 lookups of a row never collide whatever the bucket IDs are
// (gfx950 serves 16 lanes of a ds_read_b128 per cycle).  A rotated
// reduce-scatter over the row (DPP row_ror) leaves each lane the full sum of
// its own key.  Blocks of one KV head are placed on one XCD so that its image
// is fetched from HBM into one L2 only.
//
// Top-k: the scorer also builds, per query head, a histogram of the top
// digit of the float32 score bits (scores are non-negative, so their bit
// patterns order like the values).  A scan kernel spread over many workgroups
// per query head finds the bin holding the k-th largest score, marks every
// key above it in a bitmap and collects the keys of that bin as candidates;
// one resolve workgroup per head settles them exactly (radix select on the
// remaining score bits, then on the index so that the lower index wins a tie)
// and turns the bitmap into ascending indices.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace socketlsh {

// ---------------------------------------------------------------- table images

// LDS image of the tables of one KV row (its G query heads).  Lane j of a
// 16-lane scorer row owns tables j*TL .. j*TL+TL-1; the first NF of them are
// kept as full tables, the other NS = TL - NF as their two factors:
//   full slot (m*256 + e)*16 + j                      e < 2^P, m < NF
//   half slot FULL + ((hf*HE + c)*NS + m)*16 + j      hf = 0 (low planes) or
//                                                      1 (high planes), c < HE, m < NS
// one slot = G floats (the G query heads).  Bank group of a slot = j, so the
// 16 lookups of a row never collide.  For P <= 8 the halves have HE = 16
// entries (planes 0..3 and 4..P-1) and NF is the largest count whose image
// fits in the 160 KiB of LDS next to the G-head score histogram; for
// 8 < P <= 10 (WIDE) a full table would not fit, NF = 0 and the halves have
// HE = 32 entries (planes 0..4 and 5..P-1).
template <int G, int TL, bool WIDE>
struct ImageShape {
  static constexpr int HE = WIDE ? 32 : 16;
  static constexpr bool fit(int nf) {
    return 256 * nf * 16 * G + 2 * HE * (TL - nf) * 16 * G <= 40960 - G * kHistBins;
  }
  static constexpr int pick() {
    if (WIDE) return 0;
    int nf = 0;
    for (int c = 0; c <= TL; ++c)
      if (fit(c)) nf = c;
    return nf;
  }
  static constexpr int NF = pick();
  static constexpr int NS = TL - NF;
  static constexpr int FULL = 256 * NF * 16 * G;   // floats
  static constexpr int HALF = 2 * HE * NS * 16 * G;
  static constexpr int FLOATS = FULL + HALF;
};

struct ImageDims {
  int G, TL, NF, NS, HE, full, floats;
};

// Shape of the image for G query heads per KV head, L tables of P planes.
static ImageDims image_dims(int G, int L, int P) {
  const int TL = ids_tables_per_word(L);
  auto make = [](auto g, auto tl, auto wide) {
    using S = ImageShape<decltype(g)::value, decltype(tl)::value, decltype(wide)::value>;
    return ImageDims{decltype(g)::value, decltype(tl)::value, S::NF, S::NS, S::HE, S::FULL,
                     S::FLOATS};
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  using N = std::false_type;
  using Y = std::true_type;
  if (P > 8) {  // L <= 64
    switch (G * 16 + TL) {
      case 17: return make(I1{}, I1{}, Y{});
      case 18: return make(I1{}, I2{}, Y{});
      case 20: return make(I1{}, I4{}, Y{});
      case 33: return make(I2{}, I1{}, Y{});
      case 34: return make(I2{}, I2{}, Y{});
      case 36: return make(I2{}, I4{}, Y{});
      case 65: return make(I4{}, I1{}, Y{});
      case 66: return make(I4{}, I2{}, Y{});
      default: return make(I4{}, I4{}, Y{});
    }
  }
  switch (G * 16 + TL) {
    case 17: return make(I1{}, I1{}, N{});
    case 18: return make(I1{}, I2{}, N{});
    case 20: return make(I1{}, I4{}, N{});
    case 24: return make(I1{}, I8{}, N{});
    case 33: return make(I2{}, I1{}, N{});
    case 34: return make(I2{}, I2{}, N{});
    case 36: return make(I2{}, I4{}, N{});
    case 40: return make(I2{}, I8{}, N{});
    case 65: return make(I4{}, I1{}, N{});
    case 66: return make(I4{}, I2{}, N{});
    case 68: return make(I4{}, I4{}, N{});
    default: return make(I4{}, I8{}, N{});
  }
}

// Floats reserved per KV row for its image: enough for either ID width.
static int image_stride(int G, int L) {
  const int a = image_dims(G, L, 8).floats;
  const int b = L <= 64 ? image_dims(G, L, 10).floats : 0;
  return a > b ? a : b;
}

// ---------------------------------------------------------------- workspace

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Keys per top-k scan workgroup (the bitmap covers whole ones).  Its LDS
// (one candidate slot per key, 72 KiB) lets two workgroups share a CU, 512
// over the chip; 9216 rather than 8192 keeps a 32K or 128K row plus its
// appended keys in 4 or 15 workgroups instead of adding a one-key fifth or
// seventeenth, which at 32 heads would not fit in one wave of residency.
constexpr int kScanKeys = 9216;

size_t score_ws_layout(int B, int Hq, int Hkv, int64_t n_cap, int L, ScoreWs* ws, void* base) {
  const int G = Hq / Hkv;
  const int img_floats = image_stride(G == 1 || G == 2 ? G : 4, L);
  const size_t n = select_ws_layout((size_t)B * Hkv * img_floats * sizeof(float), B, Hq, n_cap,
                                    ws, base);
  if (ws) ws->img_floats = img_floats;
  return n;
}

size_t select_ws_layout(size_t first_bytes, int B, int Hq, int64_t n_cap, ScoreWs* ws,
                        void* base) {
  const size_t heads = (size_t)B * Hq;
  const int64_t words = (n_cap + kScanKeys - 1) / kScanKeys * (kScanKeys / 32);
  size_t off = 0;
  const size_t o_img = off; off = align256(off + first_bytes);
  const size_t o_hist = off; off = align256(off + heads * kHistBins * sizeof(uint32_t));
  const size_t o_cnt = off; off = align256(off + heads * sizeof(uint32_t));
  const size_t o_bm = off; off = align256(off + heads * words * sizeof(uint32_t));
  const size_t o_cand = off; off = align256(off + heads * (size_t)n_cap * sizeof(uint2));
  const size_t o_sc = off; off = align256(off + heads * (size_t)score_stride(n_cap) * sizeof(float));
  const size_t o_us = off; off = align256(off + heads * sizeof(float));
  if (ws) {
    char* p = static_cast<char*>(base);
    ws->img = reinterpret_cast<float*>(p + o_img);
    ws->qcodes = reinterpret_cast<uint32_t*>(p + o_img);
    ws->img_floats = 0;
    ws->hist = reinterpret_cast<uint32_t*>(p + o_hist);
    ws->counters = reinterpret_cast<uint32_t*>(p + o_cnt);
    ws->bitmap = reinterpret_cast<uint32_t*>(p + o_bm);
    ws->cand = reinterpret_cast<uint2*>(p + o_cand);
    ws->scores = reinterpret_cast<float*>(p + o_sc);
    ws->usum = reinterpret_cast<float*>(p + o_us);
    ws->words = words;
  }
  return off;
}

// ---------------------------------------------------------------- soft tables

constexpr int kTabThreads = 256;  // >= TL * P * G projections (8 * 8 * 4)

template <int G>
__device__ __forceinline__ void store_slot(float* dst, const float* v) {
  if constexpr (G == 4) *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  else if constexpr (G == 2) *reinterpret_cast<float2*>(dst) = make_float2(v[0], v[1]);
  else dst[0] = v[0];
}

// grid: B*Hkv*16 blocks of kTabThreads.  Block (bh, j) computes the tables
// j*TL .. j*TL+TL-1 (the tables of scorer lane j) for the G query heads of KV
// row bh and writes their image slots whole (one slot = the G heads' values
// of one entry).  It also clears a 1/16 share of those heads' histograms
// (block j = 0: their candidate counters and soft-count sums).
// Tables l >= L (padding of the last lane word) get all-zero entries.
// With ak.K set, blocks past the first B*Hkv*16 hash the key appended at
// position lens[b] - 1 of each KV row (append_block below) alongside.
template <typename T>
__device__ void append_block(const T* __restrict__ W, int Hkv, int L, int P, int TL, int nab,
                             int rows, const AppendKey& ak);

template <typename T, int G>
__global__ __launch_bounds__(kTabThreads) void soft_tables_kernel(
    const T* __restrict__ q, const T* __restrict__ W, int Hq, int Hkv, int L, int P, float tau,
    int TL, int NF, int NS, int HE, int FULL, int img_floats, float* __restrict__ img,
    uint32_t* __restrict__ hist, uint32_t* __restrict__ counters, float* __restrict__ usum,
    AppendKey ak, int rows, int nab) {
  if ((int)blockIdx.x >= rows * 16) {  // uniform
    append_block<T>(W, Hkv, L, P, TL, nab, rows, ak);
    return;
  }
  // Logical table block lid = (blockIdx mod 8) * (2 rows) + blockIdx / 8: the
  // 16 blocks of a KV row share an XCD (blocks go to the XCDs round robin),
  // so the 16-byte slots they write into each image line meet in one L2.
  const int lid = (int)(blockIdx.x % kXcds) * (rows * 16 / kXcds) + (int)(blockIdx.x / kXcds);
  const int bh = lid >> 4, j = lid & 15;
  const int b = bh / Hkv, h = bh % Hkv;
  const int bg0 = b * Hq + h * G;
  const int tid = threadIdx.x;
  float* im = img + (int64_t)bh * img_floats;
  __shared__ float qf[G][kHead];         // the queries (exact in float32)
  __shared__ double sig[kTabThreads][2];  // [(m*P + plane)*G + g][bit] = sigmoid(+-2u/tau)
  __shared__ double half[8][G][64];       // [m][g][hf*HE + c]

  constexpr int kHistShare = G * kHistBins / 16;
  for (int i = tid; i < kHistShare; i += kTabThreads)
    hist[(int64_t)bg0 * kHistBins + j * kHistShare + i] = 0u;
  if (j == 0 && tid < G) {
    counters[bg0 + tid] = 0u;
    usum[bg0 + tid] = 0.f;
  }
  for (int i = tid; i < G * kHead; i += kTabThreads) {
    const int64_t src = (int64_t)(bg0 + i / kHead) * kHead + i % kHead;
    if constexpr (sizeof(T) == 2) qf[i / kHead][i % kHead] = __uint_as_float((uint32_t)q[src] << 16);
    else qf[i / kHead][i % kHead] = q[src];
  }
  // projections: two threads (lanes 2p, 2p+1) per (table member m, plane
  // pl, head g), each taking half of the 128-element dot product
  constexpr int NV = kHead * (int)sizeof(T) / 32;  // 16-byte vectors per half row
  const int nproj = TL * P * G;
  const int hv = tid & 1;
  uint4 raw[2][NV];
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int pr = (tid >> 1) + it * (kTabThreads / 2);
    const int m = pr / (P * G), pl = (pr / G) % P;
    const int l = j * TL + m;
    if (pr < nproj && l < L) {
      const uint4* wr = reinterpret_cast<const uint4*>(W + (int64_t)(l * P + pl) * kHead) + hv * NV;
#pragma unroll
      for (int v = 0; v < NV; ++v) raw[it][v] = wr[v];
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int pr = (tid >> 1) + it * (kTabThreads / 2);
    if (it * (kTabThreads / 2) >= nproj) break;  // uniform
    const int m = pr / (P * G), pl = (pr / G) % P, g = pr % G;
    const int l = j * TL + m;
    const bool live = pr < nproj && l < L;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    if (live) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        float f[8];
        int cnt;
        if constexpr (sizeof(T) == 2) {
          unpack_bf16x8(raw[it][v], f);
          cnt = 8;
        } else {
          f[0] = __uint_as_float(raw[it][v].x); f[1] = __uint_as_float(raw[it][v].y);
          f[2] = __uint_as_float(raw[it][v].z); f[3] = __uint_as_float(raw[it][v].w);
          cnt = 4;
        }
        const int base = hv * (kHead / 2) + v * cnt;
#pragma unroll
        for (int e = 0; e < cnt; ++e)
          acc[e & 3] = fma((double)f[e], (double)qf[g][base + e], acc[e & 3]);
      }
    }
    double u = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    u += __shfl_xor(u, 1, 64);  // the partner lane's half
    if (pr < nproj && hv == 0) {
      // sigmoid(x) and sigmoid(-x) from one exponential of -|x|
      const double x = 2.0 * u / (double)tau;
      const double e = exp(-fabs(x));
      const double big = 1.0 / (1.0 + e), small = e * big;
      sig[pr][1] = x >= 0.0 ? big : small;  // bit set: corner sign +1
      sig[pr][0] = x >= 0.0 ? small : big;  // bit clear: corner sign -1
    }
  }
  __syncthreads();
  // halves: planes 0 .. plo-1 and plo .. P-1, HE entries each
  const int plo = HE == 32 ? 5 : (P < 4 ? P : 4);
  const int phi = P - plo;
  for (int i = tid; i < TL * G * 2 * HE; i += kTabThreads) {
    const int mm = i / (G * 2 * HE), gg = (i / (2 * HE)) % G, r = i % (2 * HE);
    const int hf = r / HE, c = r % HE;
    const int nb = hf ? phi : plo;
    double prod = 0.0;
    if (c < (1 << nb) && j * TL + mm < L) {
      prod = 1.0;
      const int p0 = hf ? plo : 0;
      for (int jj = 0; jj < nb; ++jj) prod *= sig[(mm * P + p0 + jj) * G + gg][(c >> jj) & 1];
    }
    half[mm][gg][r] = prod;
  }
  __syncthreads();
  // full tables, table-major: slot (m*256 + e)*16 + j for entries e < 2^P
  const int nent = 1 << P;
  const int lomask = (1 << plo) - 1;
  for (int i = tid; i < NF * nent; i += kTabThreads) {
    const int e = i / NF, mm = i % NF;
    float v[G];
#pragma unroll
    for (int gg = 0; gg < G; ++gg)
      v[gg] = (float)(half[mm][gg][e & lomask] * half[mm][gg][HE + (e >> plo)]);
    store_slot<G>(im + ((int64_t)(mm * 256 + e) * 16 + j) * G, v);
  }
  // factored tables: slot FULL/G + ((hc*NS + m - NF)*16 + j), hc = hf*HE + c
  for (int i = tid; i < 2 * HE * NS; i += kTabThreads) {
    const int hc = i / NS, mm = NF + i % NS;
    float v[G];
#pragma unroll
    for (int gg = 0; gg < G; ++gg) v[gg] = (float)half[mm][gg][hc];
    store_slot<G>(im + FULL + ((int64_t)i * 16 + j) * G, v);
  }
}

// Append blocks: block a of KV row bh (a < nab) projects the new key at
// lens[b] - 1 on the planes of ID words a*WPB .. a*WPB+WPB-1, one plane per
// thread, in float32 with the accumulation order of the hashing kernels, and
// stores those words; block 0 also stores the value norm.  WPB = the whole
// words of TL*P planes that fit in kTabThreads threads.
template <typename T>
__device__ void append_block(const T* __restrict__ W, int Hkv, int L, int P, int TL, int nab,
                             int rows, const AppendKey& ak) {
  const int ag = (int)blockIdx.x - rows * 16;
  const int bh = ag / nab, a = ag % nab;
  const int b = bh / Hkv;
  const int tid = threadIdx.x;
  const int WP = TL * P;              // planes per ID word (<= 64)
  const int WPB = kTabThreads / WP;   // whole words per block
  const int w0 = a * WPB;
  const int word = w0 + tid / WP, qq = tid % WP;
  const int m = qq / P, pl = qq % P, l = word * TL + m;
  const bool live = tid < WPB * WP && word < 16 && l < L;
  // the plane's W row first: it does not depend on the key position
  constexpr int NV = kHead * (int)sizeof(T) / 16;
  uint4 wv[NV];
  if (live) {
    const uint4* wr = reinterpret_cast<const uint4*>(W + (int64_t)(l * P + pl) * kHead);
#pragma unroll
    for (int v = 0; v < NV; ++v) wv[v] = wr[v];
  }
  const int64_t pos = (int64_t)ak.lens[b] - 1;
  if (pos < 0 || pos >= ak.n_cap) return;  // uniform: no key to append
  const int64_t row = (int64_t)bh * ak.n_cap + pos;
  const T* K = static_cast<const T*>(ak.K);
  const T* V = static_cast<const T*>(ak.V);
  __shared__ float kf[kHead];
  __shared__ uint32_t kbit[kTabThreads];
  if (tid < kHead) {
    if constexpr (sizeof(T) == 2) kf[tid] = __uint_as_float((uint32_t)K[row * kHead + tid] << 16);
    else kf[tid] = K[row * kHead + tid];
  }
  const bool norm = a == 0 && tid < 16;  // lanes 0..15 of wave 0: the value norm
  float vf[8];
  if (norm) {
    if constexpr (sizeof(T) == 2) {
      unpack_bf16x8(reinterpret_cast<const uint4*>(V + row * kHead)[tid], vf);
    } else {
      const float4 x = reinterpret_cast<const float4*>(V + row * kHead)[2 * tid];
      const float4 y = reinterpret_cast<const float4*>(V + row * kHead)[2 * tid + 1];
      vf[0] = x.x; vf[1] = x.y; vf[2] = x.z; vf[3] = x.w;
      vf[4] = y.x; vf[5] = y.y; vf[6] = y.z; vf[7] = y.w;
    }
  }
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
  kbit[tid] = live && z > 0.f ? 1u : 0u;  // z == 0 gives bit 0
  if (a == 0 && tid < 64) {  // the whole row of 16 lanes joins the DPP sum
    float ss = 0.f;
    if (norm) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(vf[i], vf[i], ss);
    }
    ss = row16_sum(ss);
    if (tid == 0) ak.vnorm[row] = sqrtf(ss);
  }
  __syncthreads();
  if (tid < WPB && w0 + tid < 16) {
    const int wd = w0 + tid;
    const int C = P > 8 ? 2 : 1, WB = TL * C;
    uint64_t w[2] = {0ull, 0ull};
    for (int mm = 0; mm < TL; ++mm) {
      uint64_t id = 0ull;
      if (wd * TL + mm < L)
        for (int p2 = 0; p2 < P; ++p2) id |= (uint64_t)kbit[tid * WP + mm * P + p2] << p2;
      const int bit = 8 * C * mm;
      w[bit >> 6] |= id << (bit & 63);
    }
    uint8_t* dst = ak.ids + ids_word_offset(bh, ak.n_cap, WB, pos, wd);
    if (WB == 1) *dst = (uint8_t)w[0];
    else if (WB == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w[0];
    else if (WB == 4) *reinterpret_cast<uint32_t*>(dst) = (uint32_t)w[0];
    else if (WB == 8) *reinterpret_cast<uint2*>(dst) = make_uint2((uint32_t)w[0], (uint32_t)(w[0] >> 32));
    else *reinterpret_cast<uint4*>(dst) = make_uint4((uint32_t)w[0], (uint32_t)(w[0] >> 32),
                                                     (uint32_t)w[1], (uint32_t)(w[1] >> 32));
  }
}
// ---------------------------------------------------------------- scorer

template <int G>
__device__ __forceinline__ void lds_get(const float* lds, int slot, float* v) {
  if constexpr (G == 1) {
    v[0] = lds[slot];
  } else if constexpr (G == 2) {
    const float2 t = reinterpret_cast<const float2*>(lds)[slot];
    v[0] = t.x; v[1] = t.y;
  } else {
    const float4 t = reinterpret_cast<const float4*>(lds)[slot];
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  }
}

constexpr int kScoreThreads = 512;
constexpr int kScoreWaves = kScoreThreads / 64;

// Reduce-scatter over a 16-lane row (see score_group): on entry lane j holds
// in u[x] its contribution to key (j + x) mod 16 of the row; on exit u[0] of
// lane j is the sum over the 16 lanes for key j.  Stage d adds, for x < d,
// the value lane j - d holds for the same key (its slot x + d); row_ror:d
// gives lane j the register of lane (j - d) mod 16.

// The WB-byte ID word of round x from the lane's WB 16-byte vectors.
template <int WB>
__device__ __forceinline__ uint2 round_word(const uint4 (&v)[WB], int x) {
  constexpr int R = 16 / WB;
  const uint4 q = v[x / R];
  const int k = x % R;  // word index inside the vector
  if constexpr (WB == 8) {
    return k == 0 ? make_uint2(q.x, q.y) : make_uint2(q.z, q.w);
  } else {
    const int byte = k * WB;
    const uint32_t d = byte < 4 ? q.x : byte < 8 ? q.y : byte < 12 ? q.z : q.w;
    return make_uint2(WB == 4 ? d : (d >> (8 * (byte & 3))) & (WB == 2 ? 0xFFFFu : 0xFFu), 0u);
  }
}

// Cell M of a word of C-byte cells.
template <int C, int M>
__device__ __forceinline__ uint32_t word_cell(uint2 w) {
  if constexpr (C == 1) return ((M < 4 ? w.x : w.y) >> (8 * (M & 3))) & 255u;
  else return ((M < 2 ? w.x : w.y) >> (16 * (M & 1))) & 0xFFFFu;
}

constexpr int kPrefetch = 1;  // 64-key groups of IDs each wave keeps in flight

// The lookups of one round: NF full-table slots and NS lo/hi half slots.
template <int NF, int NS, int G>
struct RoundVals {
  float f[NF > 0 ? NF : 1][G];
  float lo[NS > 0 ? NS : 1][G];
  float hi[NS > 0 ? NS : 1][G];
};

// Full tables are stored table-major: slot (M*256 + cell)*16 + j.  For G = 4
// a slot is 16 bytes, so the byte address M*65536 + cell*256 + 16*j is one
// byte permute of the ID word (cell -> byte 1) and jw = 16*j | 1 << 8 (16*j
// -> byte 0, and table M = 1 -> byte 2); NF <= 2 at G = 4.
template <int NF, int NS, int G, int M = 0>
__device__ __forceinline__ void issue_full(const float* lds, uint2 w, int j, uint32_t jw,
                                           RoundVals<NF, NS, G>& r) {
  if constexpr (M < NF) {
    if constexpr (G == 4) {
      static_assert(NF <= 2, "a byte permute addresses two full tables");
      constexpr uint32_t sel = 0x0c000000u | ((M ? 0x01u : 0x0cu) << 16) | ((4u + M) << 8);
      const uint32_t a = __builtin_amdgcn_perm(w.x, jw, sel);
      const float4 t = *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(lds) + a);
      r.f[M][0] = t.x; r.f[M][1] = t.y; r.f[M][2] = t.z; r.f[M][3] = t.w;
    } else {
      lds_get<G>(lds, (M * 256 + (int)word_cell<1, M>(w)) * 16 + j, r.f[M]);
    }
    issue_full<NF, NS, G, M + 1>(lds, w, j, jw, r);
  }
}

// Half-table lookups of tables NF .. NF+NS-1 (C-byte cells, HE-entry halves).
template <int NF, int NS, int G, int C, int HE, int M = 0>
__device__ __forceinline__ void issue_half(const float* lds, uint2 w, int j, int plo,
                                           RoundVals<NF, NS, G>& r) {
  if constexpr (M < NS) {
    // the two factors' entries as bit fields of the word (one extract each)
    constexpr int T = NF + M, PER = 4 / C;  // cells per 32-bit half of the word
    const uint32_t src = T < PER ? w.x : w.y;
    constexpr uint32_t off = 8 * C * (T % PER);
    const uint32_t lo = __builtin_amdgcn_ubfe(src, off, (uint32_t)plo);
    const uint32_t hi = __builtin_amdgcn_ubfe(src, off + (uint32_t)plo, 8 * C - (uint32_t)plo);
    lds_get<G>(lds, ((int)lo * NS + M) * 16 + j, r.lo[M]);
    lds_get<G>(lds, ((HE + (int)hi) * NS + M) * 16 + j, r.hi[M]);
    issue_half<NF, NS, G, C, HE, M + 1>(lds, w, j, plo, r);
  }
}

template <int NF, int NS, int G>
__device__ __forceinline__ void round_sum(const RoundVals<NF, NS, G>& r, float (&acc)[G]) {
#pragma unroll
  for (int gg = 0; gg < G; ++gg) {
    float a = NF > 0 ? r.f[0][gg] : r.lo[0][gg] * r.hi[0][gg];
#pragma unroll
    for (int m = 1; m < NF; ++m) a += r.f[m][gg];
#pragma unroll
    for (int m = NF > 0 ? 0 : 1; m < NS; ++m) a = fmaf(r.lo[m][gg], r.hi[m][gg], a);
    acc[gg] = a;
  }
}

// Soft-count sums of one 64-key group: 16 rounds, round x giving lane j its
// tables' share of key (j + x) mod 16 of its row; the LDS lookups of round
// x + 1 are issued before round x is summed.  The first reduce-scatter stage
// (row_ror 8) is applied as soon as round x + 8 is summed, so only 8 rounds of
// partial sums stay live.  On exit u[0] of lane j holds the sums of its key.
template <int NF, int NS, int G, int C, int HE, int WB>
__device__ __forceinline__ void score_group(const float* lds, const uint4 (&ids)[WB], int j,
                                            int plo, float (&u)[8][G]) {
  constexpr int FULL = 256 * NF * 16 * G;
  const uint32_t jw = ((uint32_t)j << 4) | 0x100u;
  RoundVals<NF, NS, G> cur, nxt;
  {
    const uint2 w = round_word<WB>(ids, 0);
    issue_full<NF, NS, G>(lds, w, j, jw, cur);
    issue_half<NF, NS, G, C, HE>(lds + FULL, w, j, plo, cur);
  }
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    if (x < 15) {
      const uint2 w = round_word<WB>(ids, x + 1);
      issue_full<NF, NS, G>(lds, w, j, jw, nxt);
      issue_half<NF, NS, G, C, HE>(lds + FULL, w, j, plo, nxt);
    }
    float acc[G];
    round_sum<NF, NS, G>(cur, acc);
    if (x < 8) {
#pragma unroll
      for (int gg = 0; gg < G; ++gg) u[x][gg] = acc[gg];
    } else {
#pragma unroll
      for (int gg = 0; gg < G; ++gg) u[x - 8][gg] += dpp_f32<0x128>(acc[gg]);
    }
    cur = nxt;
  }
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int g = 0; g < G; ++g) u[x][g] += dpp_f32<0x124>(u[x + 4][g]);
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int g = 0; g < G; ++g) u[x][g] += dpp_f32<0x122>(u[x + 2][g]);
#pragma unroll
  for (int g = 0; g < G; ++g) u[0][g] += dpp_f32<0x121>(u[1][g]);
}

// grid: a multiple of kXcds blocks of kScoreThreads, at least B*Hkv*nblk.
// Logical block lid = (blockIdx mod 8) * (grid / 8) + blockIdx / 8 keeps
// consecutive logical blocks -- the blocks of one KV row -- on one XCD.
// When every sequence has the same length, logical block blk of KV row bh
// owns the 64-key groups [blk*gpb, (blk+1)*gpb) of that row.  With ragged
// lengths a row-aligned split would leave the blocks of short rows idle while
// those of the longest rows set the time, so the valid groups of all rows
// (in row order) are cut into rows*nblk equal shares instead; a share may
// span rows, and the block scores it row by row, loading each row's table
// image and merging each row's histogram in turn.  Within a row segment the
// waves take the groups round robin, each keeping the IDs of its next
// kPrefetch groups in flight (a ring of registers, indexed by compile-time
// constants so no copy waits on a load).  Each score also goes into an LDS
// histogram of its top digit, merged into the head's global histogram at the
// end of the segment.  Scores do not depend on the split.
template <int G, int TL, bool WIDE>
__global__ __launch_bounds__(kScoreThreads) void scorer_kernel(
    const float* __restrict__ img, int img_floats, const uint8_t* __restrict__ ids,
    const float* __restrict__ vnorm, const int32_t* __restrict__ lens, int Hq, int Hkv, int P,
    int64_t n_cap, int sink, int window, int rows, int nblk, int gpb, float* __restrict__ scores,
    uint32_t* __restrict__ hist, float* __restrict__ usum) {
  using Sh = ImageShape<G, TL, WIDE>;
  constexpr int NF = Sh::NF, NS = Sh::NS, HE = Sh::HE;
  constexpr int C = WIDE ? 2 : 1;  // bytes per ID
  constexpr int WB = TL * C;       // bytes per ID word
  constexpr int D = kPrefetch;
  __shared__ __attribute__((aligned(16))) float lds[Sh::FLOATS];
  __shared__ uint32_t lhist[G * kHistBins];
  const int lid = (int)(blockIdx.x % kXcds) * (int)(gridDim.x / kXcds) + (int)(blockIdx.x / kXcds);
  if (lid >= rows * nblk) return;
  const int tid = threadIdx.x, lane = tid & 63, j = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t sst = score_stride(n_cap);
  const int plo = WIDE ? 5 : (P < 4 ? P : 4);
  auto seq_len = [&](int b) {
    int64_t n = lens[b];
    if (n > n_cap) n = n_cap;
    if (n < 0) n = 0;
    return n;
  };

  // Score groups [g_begin, g_end) (g_begin < g_end) of KV row bh; every wave
  // of the block calls it.
  auto segment = [&](int bh, int64_t g_begin, int64_t g_end) {
    const int b = bh / Hkv;
    const int h = bh % Hkv;
    const int64_t n = seq_len(b);
    // sink and window keys [0, f_lo) and [f_hi, n) are always selected:
    // scored, but kept out of the selection histogram
    const int64_t f_lo = sink < n ? sink : n;
    const int64_t f_hi = n - window > 0 ? n - window : 0;
    const int bg0 = b * Hq + h * G;

    // The first D groups' IDs and norms, then the table image.  Group loads
    // are issued unconditionally (a group past the segment re-reads its last
    // group, keys past n_cap re-read the last norm) so that no branch sits
    // between a load and its use and each wait covers only the group needed.
    const uint8_t* idg = ids + (int64_t)bh * ids_groups(n_cap) * 1024 * WB;
    const float* vrow = vnorm + (int64_t)bh * n_cap;
    auto load_group = [&](int64_t gi, uint4 (&v)[WB], float& vn) {
      const int64_t gl = gi < g_end ? gi : g_end - 1;
      const uint4* src = reinterpret_cast<const uint4*>(idg + gl * 1024 * WB) + lane;
#pragma unroll
      for (int qv = 0; qv < WB; ++qv) v[qv] = src[qv * 64];
      const int64_t key = gl * 64 + lane;
      vn = vrow[key < n_cap ? key : n_cap - 1];
    };
    uint4 buf[D + 1][WB];
    float vb[D + 1];
    int64_t gi = g_begin + wave;
#pragma unroll
    for (int d = 0; d < D; ++d) load_group(gi + (int64_t)d * kScoreWaves, buf[d], vb[d]);
    {
      // The image goes straight from global memory into LDS (16 bytes per
      // lane, no registers), every load of the block in flight at once.
      const uint4* src = reinterpret_cast<const uint4*>(img + (int64_t)bh * img_floats);
      uint4* dst = reinterpret_cast<uint4*>(lds);
      constexpr int NV = Sh::FLOATS / 4;
      constexpr int PER = (NV + kScoreThreads - 1) / kScoreThreads;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int base = k * kScoreThreads + wave * 64;  // this wave's 64 vectors
        if (NV % kScoreThreads == 0 || base + lane < NV)
          __builtin_amdgcn_global_load_lds(src + base + lane, dst + base, 16, 0, 0);
      }
      for (int i = tid; i < G * kHistBins; i += kScoreThreads) lhist[i] = 0u;
      __builtin_amdgcn_s_waitcnt(0);  // the LDS writes of those loads have landed
    }
    __syncthreads();

    float us[G];  // this lane's soft counts (before the value norm), summed when usum is set
#pragma unroll
    for (int gg = 0; gg < G; ++gg) us[gg] = 0.f;
    bool more = gi < g_end;
    while (more) {
#pragma unroll
      for (int s = 0; s <= D; ++s) {
        if (more) {
          load_group(gi + (int64_t)D * kScoreWaves, buf[(s + D) % (D + 1)], vb[(s + D) % (D + 1)]);
          float u[8][G];
          score_group<NF, NS, G, C, HE, WB>(lds, buf[s], j, plo, u);
          const int64_t key = gi * 64 + lane;
          const bool valid = key < n;
          const uint32_t ranked = valid && key >= f_lo && key < f_hi ? 1u : 0u;
#pragma unroll
          for (int gg = 0; gg < G; ++gg) {
            const float sv = vb[s] * u[0][gg];
            uint32_t dg = __float_as_uint(sv) >> kHistShift;
            if (dg > kHistBins - 1) dg = kHistBins - 1;
            atomicAdd(&lhist[gg * kHistBins + dg], ranked);
          }
          if (valid) {
#pragma unroll
            for (int gg = 0; gg < G; ++gg) {
              scores[(int64_t)(bg0 + gg) * sst + key] = vb[s] * u[0][gg];
              us[gg] += u[0][gg];
            }
          }
          gi += kScoreWaves;
          more = gi < g_end;
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < G * kHistBins; i += kScoreThreads) {
      const uint32_t v = lhist[i];
      if (v) atomicAdd(&hist[(int64_t)(bg0 + i / kHistBins) * kHistBins + (i % kHistBins)], v);
    }
    if (usum) {  // per-head sums of the soft counts, for the sampling estimator
      __syncthreads();  // the merge above has read the histogram: reuse its LDS
      float* red = reinterpret_cast<float*>(lhist);  // [kScoreWaves][G]
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        const float t = wave_sum(us[gg]);
        if (lane == 0) red[wave * G + gg] = t;
      }
      __syncthreads();
      if (tid < G) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < kScoreWaves; ++w) t += red[w * G + tid];
        atomicAdd(&usum[bg0 + tid], t);
      }
    }
    __syncthreads();  // a following segment reuses the image and histogram LDS
  };

  // Whether the sequence lengths differ (in groups), the same in every wave:
  // scalar loads for up to 64 sequences, else 64 a step across the lanes.
  // Uniform lengths take the row-aligned split.
  const int B = rows / Hkv;
  const uint32_t ng0 = (uint32_t)((seq_len(0) + 63) >> 6);
  bool ragged = false;
  if (B <= 64) {
    for (int b = 1; b < B; ++b) ragged |= (uint32_t)((seq_len(b) + 63) >> 6) != ng0;
  } else {
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int b = b0 + lane;
      const uint32_t ng = b < B ? (uint32_t)((seq_len(b) + 63) >> 6) : ng0;
      ragged |= __ballot(ng != ng0) != 0ull;
    }
  }
  if (!ragged) {
    const int blk = lid % nblk;
    const int64_t gb = (int64_t)blk * gpb;
    int64_t ge = (int64_t)ng0;
    if (ge > gb + gpb) ge = gb + gpb;
    if (gb < ge) segment(lid / nblk, gb, ge);
    return;
  }
  // Ragged lengths: share lid of the row-ordered valid groups, row by row.
  // The totals and offsets are wave-uniform and kept in scalar registers.
  uint32_t total = 0u;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const uint32_t ng = b < B ? (uint32_t)((seq_len(b) + 63) >> 6) : 0u;
    total += (uint32_t)__builtin_amdgcn_readfirstlane((int)__shfl(wave_incl_scan(ng), 63, 64)) *
             (uint32_t)Hkv;
  }
  const uint32_t shares = (uint32_t)(rows * nblk);
  const uint32_t per = (total + shares - 1) / shares;
  uint32_t G0 = (uint32_t)lid * per;
  const uint32_t G1 = G0 + per < total ? G0 + per : total;
  int bcur = 0;
  uint32_t base = 0u;  // groups of the sequences before bcur (all KV heads)
  while (G0 < G1) {
    // the sequence whose groups hold G0, by a wave scan over 64 sequences at a time
    for (;;) {
      const int b = bcur + lane;
      const uint32_t ng = b < B ? (uint32_t)((seq_len(b) + 63) >> 6) * (uint32_t)Hkv : 0u;
      const uint32_t inc = wave_incl_scan(ng);
      const uint64_t past = __ballot(b < B && base + inc <= G0);  // sequences ending by G0
      const int skip = __popcll(past);  // a prefix of the lanes
      if (skip < 64) {
        base += skip ? (uint32_t)__builtin_amdgcn_readfirstlane((int)__shfl(inc, skip - 1, 64)) : 0u;
        bcur += skip;
        break;
      }
      base += (uint32_t)__builtin_amdgcn_readfirstlane((int)__shfl(inc, 63, 64));
      bcur += 64;
    }
    const uint32_t ngb = (uint32_t)((seq_len(bcur) + 63) >> 6);
    const uint32_t h = (G0 - base) / ngb;
    const uint32_t row0 = base + h * ngb;  // first group of KV row (bcur, h)
    const uint32_t row1 = row0 + ngb;
    const uint32_t s1 = G1 < row1 ? G1 : row1;
    segment(bcur * Hkv + (int)h, (int64_t)(G0 - row0), (int64_t)(s1 - row0));
    G0 = s1;
  }
}

// ---------------------------------------------------------------- top-k

// Two kernels per call:
//  scan    (kScanKeys keys per workgroup, many per query head): from the
//          head's first-digit histogram (built by the scorer) find the bin d1
//          holding the k-th largest score; write a bitmap of the keys in
//          higher bins and append the keys of bin d1 to the head's candidate
//          list (one counter per head).
//  resolve (one workgroup per query head): radix select on the remaining 21
//          score bits, then on the key index (the lower index wins a tie),
//          picks the candidates that complete the top-k; the bitmap plus
//          those candidates become ascending indices.
// Bitmap layout: 256-key block j (keys 256j + 4i + e, i < 64, e < 4) is 8
// words; words 8j + 2e and 8j + 2e + 1 hold bit i = key 256j + 4i + e (the
// ballot, over a wave that loaded 4 consecutive keys per lane, of the lanes'
// e-th keys).
// 12 waves, each taking three rounds of 256 keys: every wave runs a short
// serial chain of ballots and LDS appends, and with two workgroups a CU each
// SIMD has six waves to issue from.
constexpr int kScanThreads = 768;
constexpr int kResThreads = 1024;
constexpr int kResWaves = kResThreads / 64;
constexpr int kCandCap = 6144;                     // candidates resolved in LDS

// The 8 bits of b moved to bits 0, 4, ..., 28.
__device__ __forceinline__ uint32_t spread4(uint32_t b) {
  b = (b | (b << 12)) & 0x000F000Fu;
  b = (b | (b << 6)) & 0x03030303u;
  b = (b | (b << 3)) & 0x11111111u;
  return b;
}

// Block-wide inclusive scan of one value per thread (NT threads).
template <int NT>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_incl_scan(v);
  __syncthreads();
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  uint32_t off = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) off += w < wave ? wsum[w] : 0u;
  return v + off;
}

struct Boundary {
  uint32_t d1, above;
};

struct Pick {
  uint32_t digit, before, inbin;
};

// Selection sizes of one sequence: n keys; the sink and window keys
// [0, f_lo) and [f_hi, n) (nf of them) are always selected; k of the other
// n - nf keys are chosen by score; total = k + nf <= k_max indices out.
struct SelSizes {
  int64_t n, k, total, f_lo, f_hi;
};

__device__ __forceinline__ SelSizes sel_sizes(int64_t n_cap, int32_t len, int32_t kk, int k_max,
                                              int sink, int window) {
  SelSizes z;
  int64_t nn = len;
  if (nn < 0) nn = 0;
  if (nn > n_cap) nn = n_cap;
  z.n = nn;
  z.f_lo = sink < nn ? sink : nn;
  z.f_hi = nn - window > 0 ? nn - window : 0;
  const int64_t nf = z.f_lo + (nn - (z.f_hi > z.f_lo ? z.f_hi : z.f_lo));
  int64_t k2 = kk;
  if (k2 < 0) k2 = 0;
  if (k2 > nn - nf) k2 = nn - nf;
  if (k2 > k_max - nf) k2 = k_max - nf > 0 ? k_max - nf : 0;
  z.k = k2;
  z.total = k2 + nf;
  return z;
}

// Bin of the first digit that holds the k-th largest score, and how many keys
// lie in higher bins, from the head's histogram.  Thread t of NT takes the
// KPT = ceil(1024/NT) bins counted down from 1023 - KPT*t (none past bin 0):
// load_hist_slice reads them (issued before a kernel's bulk loads, so the
// boundary does not wait behind those), boundary_of finds the bin.  All
// threads must call boundary_of.
template <int NT>
struct HistSlice {
  static constexpr int KPT = (kHistBins + NT - 1) / NT;
  uint32_t c[KPT];
};

template <int NT>
__device__ __forceinline__ HistSlice<NT> load_hist_slice(const uint32_t* hh) {
  HistSlice<NT> h;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < HistSlice<NT>::KPT; ++i) {
    const int bin = kHistBins - 1 - HistSlice<NT>::KPT * tid - i;
    h.c[i] = bin >= 0 ? hh[bin] : 0u;
  }
  return h;
}

template <int NT>
__device__ Boundary boundary_of(const HistSlice<NT>& h, uint32_t k, uint32_t* wsum, Boundary* sh) {
  constexpr int KPT = HistSlice<NT>::KPT;
  const int tid = threadIdx.x;
  uint32_t sum = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) sum += h.c[i];
  if (tid == 0) *sh = Boundary{0u, 0u};
  const uint32_t inc = block_incl_scan<NT>(sum, wsum);
  uint32_t prev = inc - sum;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int bin = kHistBins - 1 - KPT * tid - i;
    if (bin >= 0 && prev < k && k <= prev + h.c[i]) *sh = Boundary{(uint32_t)bin, prev};
    prev += h.c[i];
  }
  __syncthreads();
  const Boundary r = *sh;
  __syncthreads();
  return r;
}

template <int NT>
__device__ Boundary find_boundary(const uint32_t* hh, uint32_t k, uint32_t* wsum, Boundary* sh) {
  const HistSlice<NT> h = load_hist_slice<NT>(hh);
  return boundary_of<NT>(h, k, wsum, sh);
}

// grid: B*Hq*CH blocks of NT threads (rounded up to a multiple of kXcds),
// CH = ceil(n_cap / kScanKeys).  Logical block lid (remapped as in the
// scorer, so a KV row's query heads are scanned on the XCD whose L2 received
// their scores) covers keys [c*kScanKeys, (c+1)*kScanKeys) of head lid / CH.
// Each wave gathers its candidates in an LDS region of R slots; when a ballot
// would overflow it, that ballot's candidates go straight to the global list
// under a reservation of their own.  NT = kScanThreads with R = the keys a
// wave meets (no overflow) suits a few workgroups a CU; NT = 256 with
// R = 256 uses a ninth of the LDS and a third of the waves, so that large
// batches keep eight workgroups a CU instead of two.
template <int NT, int R>
__global__ __launch_bounds__(NT) void topk_scan_kernel(
    const float* __restrict__ scores, int64_t n_cap, int64_t sstride,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ ks, int k_max, int sink,
    int window, int Hq, int CH, int heads, const uint32_t* __restrict__ hist,
    uint32_t* __restrict__ counters, uint32_t* __restrict__ bitmap, int64_t words,
    uint2* __restrict__ cand) {
  const int lid = (int)(blockIdx.x % kXcds) * (int)(gridDim.x / kXcds) + (int)(blockIdx.x / kXcds);
  if (lid >= heads * CH) return;
  const int bg = lid / CH;
  const int c = lid % CH;
  const int b = bg / Hq;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SelSizes z = sel_sizes(n_cap, lens[b], ks[b], k_max, sink, window);
  const int64_t n = z.n, k = z.k;
  if (z.total == 0) return;
  const int64_t c0 = (int64_t)c * kScanKeys;
  if (c0 >= n) return;

  // the head's histogram slice, then every score of this workgroup: load r
  // covers keys c0 + r*4*NT + 256*wave + 4*lane .. +3
  constexpr int NW = NT / 64;                  // waves
  constexpr int NL = kScanKeys / (NT * 4);     // 16-byte loads per thread
  static_assert(kScanKeys % (NT * 4) == 0, "whole load rounds of four keys a thread");
  constexpr bool kNoOverflow = R >= NL * 256;  // a wave meets NL*256 keys
  const HistSlice<NT> hs = load_hist_slice<NT>(hist + (int64_t)bg * kHistBins);
  const uint32_t* srow = reinterpret_cast<const uint32_t*>(scores) + (int64_t)bg * sstride;
  uint4 v[NL];
#pragma unroll
  for (int r = 0; r < NL; ++r) {
    int64_t key = c0 + r * (NT * 4) + tid * 4;
    if (key > sstride - 4) key = sstride - 4;  // past the row: re-read its end
    v[r] = *reinterpret_cast<const uint4*>(srow + key);
  }
  __shared__ uint32_t wsum[NW];
  __shared__ Boundary shb;
  const Boundary bd = boundary_of<NT>(hs, (uint32_t)k, wsum, &shb);
  // above d1: bits > thr_sel; in d1: bits >= thr_lo and not above (the top
  // digit is clamped to kHistBins - 1 here as in the histogram).  Sink and
  // window keys are selected whatever their score and never candidates.
  const uint32_t thr_lo = bd.d1 << kHistShift;
  const uint32_t thr_sel = bd.d1 < (uint32_t)(kHistBins - 1) ? ((bd.d1 + 1) << kHistShift) - 1u
                                                            : 0xFFFFFFFFu;
  const bool by_score = k > 0;
  uint32_t* bm = bitmap + (int64_t)bg * words;
  const uint64_t lt = lanemask_lt64();
  // candidates gather in LDS, wave w in its own region [w*R, (w+1)*R); one
  // global reservation per workgroup at the end
  __shared__ uint2 lc[NW * R];
  __shared__ uint32_t wcnt[NW], gbase;
  uint2* gc = cand + (int64_t)bg * n_cap;
  uint32_t wpos = 0u;  // uniform per wave
  // 32-bit key arithmetic (n_cap < 2^31); per-lane pointers computed once so
  // the unrolled rounds keep few scalar registers live
  const uint32_t n32 = (uint32_t)n, flo = (uint32_t)z.f_lo, fhi = (uint32_t)z.f_hi;
  const uint32_t lo = by_score ? thr_lo : 0xFFFFFFFFu;  // k == 0: no candidates
  const uint32_t hi = by_score ? thr_sel : 0xFFFFFFFFu;  // k == 0: nothing above
  const uint32_t key0 = (uint32_t)c0 + (uint32_t)(wave * 256 + 4 * lane);
  uint32_t* bml = bm + (((uint32_t)c0 + (uint32_t)wave * 256u) >> 5) + (lane & 7);
  const uint32_t bsel = (uint32_t)((lane >> 1) & 3);
#pragma unroll
  for (int r = 0; r < NL; ++r) {
    const uint32_t kr = key0 + (uint32_t)(r * NT * 4);
    const uint32_t sb[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
    uint64_t ms[4], mc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = kr + (uint32_t)e;
      const bool valid = key < n32;
      const bool forced = key < flo || key >= fhi;
      const bool above = by_score && sb[e] > hi;
      ms[e] = __ballot(valid && (forced || above));
      mc[e] = __ballot(valid && !forced && !above && by_score && sb[e] >= lo);
    }
    // lane l < 8 stores word l of the block (words 2e, 2e+1 = ballot e)
    {
      const uint64_t a = bsel == 0 ? ms[0] : bsel == 1 ? ms[1] : bsel == 2 ? ms[2] : ms[3];
      if (lane < 8) bml[r * (NT * 4 / 32)] = (lane & 1) ? (uint32_t)(a >> 32) : (uint32_t)a;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t pc = (uint32_t)__popcll(mc[e]);
      const uint32_t rank = (uint32_t)__popcll(mc[e] & lt);
      if (kNoOverflow || wpos + pc <= (uint32_t)R) {  // uniform per wave
        if ((mc[e] >> lane) & 1ull) lc[wave * R + wpos + rank] = make_uint2(sb[e], kr + e);
        wpos += pc;
      } else {  // this ballot's candidates straight to the global list
        uint32_t base = 0u;
        if (lane == 0) base = atomicAdd(&counters[bg], pc);
        base = __shfl(base, 0, 64);
        if (((mc[e] >> lane) & 1ull) && base + rank < n32) gc[base + rank] = make_uint2(sb[e], kr + e);
      }
    }
  }
  if (lane == 0) wcnt[wave] = wpos;
  __syncthreads();
  uint32_t pre[NW], cnt = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    pre[w] = cnt;
    cnt += wcnt[w];
  }
  if (cnt == 0) return;  // uniform
  if (tid == 0) gbase = atomicAdd(&counters[bg], cnt);
  __syncthreads();
  const uint32_t g0 = gbase;
  for (uint32_t t = tid; t < cnt; t += NT) {
    int w = 0;
#pragma unroll
    for (int x = 1; x < NW; ++x) w += t >= pre[x] ? 1 : 0;
    if (g0 + t < (uint32_t)n) gc[g0 + t] = lc[w * R + (t - pre[w])];
  }
}

// Among candidates whose low 21 score bits match (vmask, vval) -- and, when
// BY_INDEX, whose index matches (imask, ival) -- histogram the 7-bit digit at
// `shift` of the score bits (or of the index) and return the digit holding
// the `need`-th entry: counted from the top for scores, from the bottom for
// indices (the lower index wins a tie).
template <bool BY_INDEX, int NT = kResThreads>
__device__ Pick radix_pick(const uint2* cands, uint32_t C, uint32_t vmask, uint32_t vval,
                           uint32_t imask, uint32_t ival, int shift, uint32_t need,
                           uint32_t* h128, Pick* shpick) {
  const int tid = threadIdx.x;
  if (tid < 128) h128[tid] = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < C; i += NT) {
    const uint2 e = cands[i];
    const uint32_t v = e.x & 0x1FFFFFu;
    if ((v & vmask) != vval) continue;
    if (BY_INDEX && ((e.y & imask) != ival)) continue;
    const uint32_t x = BY_INDEX ? e.y : v;
    atomicAdd(&h128[(x >> shift) & 127u], 1u);
  }
  __syncthreads();
  if (tid < 64) {
    const int b0 = BY_INDEX ? 2 * tid : 127 - 2 * tid;
    const int b1 = BY_INDEX ? 2 * tid + 1 : 126 - 2 * tid;
    const uint32_t c0 = h128[b0], c1 = h128[b1];
    const uint32_t inc = wave_incl_scan(c0 + c1);
    const uint32_t prev = inc - c0 - c1;
    if (prev < need && need <= prev + c0) *shpick = Pick{(uint32_t)b0, prev, c0};
    else if (prev + c0 < need && need <= inc) *shpick = Pick{(uint32_t)b1, prev + c0, c1};
  }
  __syncthreads();
  const Pick r = *shpick;
  __syncthreads();
  return r;
}

// LDS of one resolve by NT threads.
template <int NT>
struct ResolveSmem {
  uint32_t wsum[NT / 64];
  Boundary shb;
  uint32_t h128[128];
  Pick shpick;
  uint32_t seg_total;
  uint2 lcand[kCandCap];
  uint32_t lbm[NT * 8];  // NT 256-key bitmap blocks: one segment
};

// The resolve of head bg (all threads of an NT-thread workgroup): radix
// select of the candidates that complete the top-k, then every selected key
// handed to emit(position, key), positions ascending with the key.
template <int NT, typename Emit>
__device__ __forceinline__ void resolve_head(int bg, int64_t n_cap, const SelSizes& z,
                                             const uint32_t* __restrict__ hist,
                                             const uint32_t* __restrict__ counters,
                                             const uint32_t* __restrict__ bitmap, int64_t words,
                                             const uint2* __restrict__ cand, ResolveSmem<NT>& sm,
                                             Emit emit) {
  const int tid = threadIdx.x;
  const int64_t n = z.n, k = z.k;

  // every independent load at once: candidate count, the first kCandCap
  // candidates (whatever their count), this thread's first bitmap block,
  // its histogram bin (inside find_boundary)
  const HistSlice<NT> hs = load_hist_slice<NT>(hist + (int64_t)bg * kHistBins);
  const uint2* gc = cand + (int64_t)bg * n_cap;
  const uint32_t* bm = bitmap + (int64_t)bg * words;
  const uint32_t Cg = counters[bg];
  uint2 cv[(kCandCap / NT)];
#pragma unroll
  for (int i = 0; i < (kCandCap / NT); ++i) {
    int64_t ci = (int64_t)i * NT + tid;
    if (ci >= n_cap) ci = n_cap - 1;
    cv[i] = gc[ci];
  }
  const int64_t nblocks = (n + 255) >> 8;
  const int64_t bl0 = tid < nblocks ? tid : 0;
  const uint4 bw0 = reinterpret_cast<const uint4*>(bm)[bl0 * 2];
  const uint4 bw1 = reinterpret_cast<const uint4*>(bm)[bl0 * 2 + 1];
  const Boundary bd = boundary_of<NT>(hs, (uint32_t)k, sm.wsum, &sm.shb);
  const uint32_t C = Cg < (uint32_t)n ? Cg : (uint32_t)n;
  const bool in_lds = C <= (uint32_t)kCandCap;
  if (in_lds) {
#pragma unroll
    for (int i = 0; i < (kCandCap / NT); ++i) {
      const uint32_t ci = (uint32_t)(i * NT + tid);
      if (ci < C) sm.lcand[ci] = cv[i];
    }
  }
  // the first segment's bitmap blocks go to LDS now, while their loads are
  // certainly in (the radix passes below do not touch lbm)
  {
    const bool mine = tid < nblocks;
    uint4* lb = reinterpret_cast<uint4*>(sm.lbm);
    lb[tid * 2] = mine ? bw0 : make_uint4(0u, 0u, 0u, 0u);
    lb[tid * 2 + 1] = mine ? bw1 : make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  const uint2* lc = in_lds ? sm.lcand : gc;

  // the candidates that complete the top-k
  uint32_t need = (uint32_t)k - bd.above;  // 1 <= need <= C when k > 0
  uint32_t vmask = 0u, vval = 0u, imax = 0xFFFFFFFFu;
  if (k > 0 && need < C) {
    uint32_t ties = 0u;
    for (int shift = 14; shift >= 0; shift -= 7) {
      const Pick pk = radix_pick<false, NT>(lc, C, vmask, vval, 0u, 0u, shift, need, sm.h128, &sm.shpick);
      need -= pk.before;
      vval |= pk.digit << shift;
      vmask |= 127u << shift;
      ties = pk.inbin;
    }
    if (ties > need) {  // among keys with exactly that score, the lower indices win
      uint32_t imask = 0u, ival = 0u;
      int top = 0;
      while (((uint64_t)1 << top) < (uint64_t)n) ++top;
      int shift = top > 7 ? top - 7 : 0;
      for (;;) {
        const Pick pk = radix_pick<true, NT>(lc, C, vmask, vval, imask, ival, shift, need, sm.h128, &sm.shpick);
        need -= pk.before;
        ival |= pk.digit << shift;
        imask |= 127u << shift;
        if (shift == 0) break;
        shift = shift > 7 ? shift - 7 : 0;
      }
      imax = ival;
    }
  }

  // bitmap + chosen candidates -> ascending indices, NT 256-key
  // blocks at a time (thread t owns block t of the segment)
  uint32_t written = 0;
  for (int64_t b0 = 0; b0 < nblocks; b0 += NT) {
    const int64_t segb = (nblocks - b0) < NT ? (nblocks - b0) : NT;
    if (b0 > 0) {  // later segments: their bitmap blocks now (segment 0 is in LDS already)
      const int64_t bl = tid < segb ? b0 + tid : b0;
      const uint4 w0 = reinterpret_cast<const uint4*>(bm)[bl * 2];
      const uint4 w1 = reinterpret_cast<const uint4*>(bm)[bl * 2 + 1];
      const bool mine = tid < segb;
      uint4* lb = reinterpret_cast<uint4*>(sm.lbm);
      lb[tid * 2] = mine ? w0 : make_uint4(0u, 0u, 0u, 0u);
      lb[tid * 2 + 1] = mine ? w1 : make_uint4(0u, 0u, 0u, 0u);
      __syncthreads();
    }
    for (uint32_t i = tid; i < C; i += NT) {
      const uint2 e = lc[i];
      const uint32_t v = e.x & 0x1FFFFFu;
      const int64_t blk = (int64_t)(e.y >> 8) - b0;
      if (blk >= 0 && blk < segb && (v > vval || (v == vval && e.y <= imax))) {
        const uint32_t i4 = (e.y >> 2) & 63u, ee = e.y & 3u;
        atomicOr(&sm.lbm[blk * 8 + ee * 2 + (i4 >> 5)], 1u << (i4 & 31));
      }
    }
    __syncthreads();
    // thread t takes WPT consecutive 32-key words of the segment, each
    // rebuilt in key order from the 8-bit slices of the block's 4 masks
    const int64_t segw = ((n - b0 * 256) + 31) >> 5 < (int64_t)NT * 8
                             ? ((n - b0 * 256) + 31) >> 5 : (int64_t)NT * 8;
    const int WPT = (int)((segw + NT - 1) / NT);  // <= 8
    uint32_t kw[8];
    uint32_t cnt = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int64_t wi = (int64_t)tid * WPT + q;
      uint32_t x = 0u;
      if (q < WPT && wi < segw) {
        const int blk = (int)(wi >> 3), sub = (int)(wi & 7);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t b8 = (sm.lbm[blk * 8 + 2 * e + (sub >> 2)] >> ((sub & 3) * 8)) & 255u;
          x |= spread4(b8) << e;  // key 4i + e of the word at bit 4i + e
        }
      }
      kw[q] = x;
      cnt += __popc(x);
    }
    const uint32_t incw = block_incl_scan<NT>(cnt, sm.wsum);
    uint32_t pos = written + incw - cnt;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t x = kw[q];
      const int64_t kbase = b0 * 256 + ((int64_t)tid * WPT + q) * 32;
      while (x) {
        const int bit = __ffs(x) - 1;
        x &= x - 1;
        emit(pos, (int32_t)(kbase + bit));
        ++pos;
      }
    }
    if (tid == NT - 1) sm.seg_total = incw;
    __syncthreads();
    written += sm.seg_total;
    __syncthreads();
  }
}

// grid: B*Hq blocks of NT threads (1024; 512 for batches of more heads than
// CUs, whose 16-wave workgroups took the dispatcher about 8 us to start).
template <int NT>
__global__ __launch_bounds__(NT) void topk_resolve_kernel(
    int64_t n_cap, const int32_t* __restrict__ lens, const int32_t* __restrict__ ks, int k_max,
    int sink, int window, int Hq, const uint32_t* __restrict__ hist,
    const uint32_t* __restrict__ counters,
    const uint32_t* __restrict__ bitmap, int64_t words, const uint2* __restrict__ cand,
    int32_t* __restrict__ idx) {
  const int bg = blockIdx.x;
  const int b = bg / Hq;
  const int tid = threadIdx.x;
  const SelSizes z = sel_sizes(n_cap, lens[b], ks[b], k_max, sink, window);
  int32_t* out = idx + (int64_t)bg * k_max;
  if (z.total == 0) {
    for (int t = tid; t < k_max; t += NT) out[t] = -1;
    return;
  }
  __shared__ ResolveSmem<NT> sm;
  resolve_head<NT>(bg, n_cap, z, hist, counters, bitmap, words, cand, sm,
               [&](uint32_t pos, int32_t key) {
                 if (pos < (uint32_t)k_max) out[pos] = key;
               });
  for (int64_t t = z.total + tid; t < k_max; t += NT) out[t] = -1;
}

// ---------------------------------------------------------------- one-pass top-k

// For n_cap <= kResThreads * 4 * kOneMaxRounds: one workgroup per query head
// does the scan and the resolve above on its own, with the head's scores in
// registers and the selection bitmap and candidates in LDS.  This saves the
// second launch for short rows; for longer ones the per-key passes of a single
// CU per head cost more than the launch, and the scan spreads them over
// several workgroups per head.  Round r of
// thread t holds keys r*4096 + 4t .. +3 (coalesced 16-byte loads); the
// bitmap has the global bitmap's layout (wave ballots per 256-key block).
// Candidates beyond the LDS capacity are settled from the registers instead.
// Workgroups are remapped as in the scorer (logical head lid = (blockIdx mod
// 8) * (grid / 8) + blockIdx / 8), so a head is selected on the XCD whose L2
// received its scores.
constexpr int kOneMaxRounds = 2;
constexpr int kOneKeys = kResThreads * 4;  // keys per round

// The boundary-bin candidates of this thread's keys in round r (4 bits).
template <int NR>
__device__ __forceinline__ uint32_t cand_bits(const uint4 (&v)[NR], int r, uint32_t key,
                                              uint32_t n, uint32_t flo, uint32_t fhi,
                                              uint32_t lo, uint32_t hi) {
  const uint32_t sb[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
  uint32_t m = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t kk = key + (uint32_t)e;
    m |= (uint32_t)(kk < n && kk >= flo && kk < fhi && sb[e] <= hi && sb[e] >= lo) << e;
  }
  return m;
}

// radix_pick over the candidates held in registers (overflow path).
template <int NR, bool BY_INDEX>
__device__ Pick radix_regs(const uint4 (&v)[NR], uint32_t n, uint32_t flo, uint32_t fhi,
                           uint32_t lo, uint32_t hi, uint32_t vmask, uint32_t vval,
                           uint32_t imask, uint32_t ival, int shift, uint32_t need,
                           uint32_t* h128, Pick* shpick) {
  const int tid = threadIdx.x;
  if (tid < 128) h128[tid] = 0u;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const uint32_t key = (uint32_t)(r * kOneKeys + 4 * tid);
    const uint32_t m = cand_bits<NR>(v, r, key, n, flo, fhi, lo, hi);
    const uint32_t sb[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t low = sb[e] & 0x1FFFFFu, kk = key + (uint32_t)e;
      if (((m >> e) & 1u) && (low & vmask) == vval && (!BY_INDEX || (kk & imask) == ival))
        atomicAdd(&h128[((BY_INDEX ? kk : low) >> shift) & 127u], 1u);
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int b0 = BY_INDEX ? 2 * tid : 127 - 2 * tid;
    const int b1 = BY_INDEX ? 2 * tid + 1 : 126 - 2 * tid;
    const uint32_t c0 = h128[b0], c1 = h128[b1];
    const uint32_t inc = wave_incl_scan(c0 + c1);
    const uint32_t prev = inc - c0 - c1;
    if (prev < need && need <= prev + c0) *shpick = Pick{(uint32_t)b0, prev, c0};
    else if (prev + c0 < need && need <= inc) *shpick = Pick{(uint32_t)b1, prev + c0, c1};
  }
  __syncthreads();
  const Pick r = *shpick;
  __syncthreads();
  return r;
}

// grid: B*Hq blocks of kResThreads.
template <int NR>
__global__ __launch_bounds__(kResThreads) void topk_onepass_kernel(
    const float* __restrict__ scores, int64_t n_cap, int64_t sstride,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ ks, int k_max, int sink,
    int window, int Hq, int heads, const uint32_t* __restrict__ hist,
    int32_t* __restrict__ idx) {
  const int bg = (int)(blockIdx.x % kXcds) * (int)(gridDim.x / kXcds) + (int)(blockIdx.x / kXcds);
  if (bg >= heads) return;
  const int b = bg / Hq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const SelSizes z = sel_sizes(n_cap, lens[b], ks[b], k_max, sink, window);
  const int64_t k = z.k;
  int32_t* out = idx + (int64_t)bg * k_max;
  if (z.total == 0) {
    for (int t = tid; t < k_max; t += kResThreads) out[t] = -1;
    return;
  }
  // every score load first (past the row: re-read its end, masked below)
  const uint32_t* srow = reinterpret_cast<const uint32_t*>(scores) + (int64_t)bg * sstride;
  uint4 v[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    int64_t kk = (int64_t)r * kOneKeys + 4 * tid;
    if (kk > sstride - 4) kk = sstride - 4;
    v[r] = *reinterpret_cast<const uint4*>(srow + kk);
  }
  __shared__ uint32_t wsum[kResWaves];
  __shared__ Boundary shb;
  __shared__ uint32_t h128[128];
  __shared__ Pick shpick;
  __shared__ uint32_t wcount[kResWaves];
  __shared__ uint2 lcand[kCandCap];
  __shared__ uint32_t lbm[NR * kOneKeys / 32];
  Boundary bd{0u, 0u};
  if (k > 0)  // uniform
    bd = find_boundary<kResThreads>(hist + (int64_t)bg * kHistBins, (uint32_t)k, wsum, &shb);
  const uint32_t n = (uint32_t)z.n, flo = (uint32_t)z.f_lo, fhi = (uint32_t)z.f_hi;
  // candidates: lo <= bits <= hi; selected outright: bits > hi (nothing when k == 0)
  const uint32_t lo = k > 0 ? bd.d1 << kHistShift : 1u;
  const uint32_t hi = k > 0 ? (bd.d1 < (uint32_t)(kHistBins - 1)
                                   ? ((bd.d1 + 1) << kHistShift) - 1u : 0xFFFFFFFFu)
                            : 0u;
  const bool above_ok = k > 0 && hi != 0xFFFFFFFFu;
  // pass 1: selection ballots into the bitmap, candidates counted per wave
  const uint64_t lt = lanemask_lt64();
  uint32_t wc = 0u;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const uint32_t base = (uint32_t)(r * kOneKeys + wave * 256);  // this wave's 256-key block
    const uint32_t sb[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
    uint64_t ms[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = base + 4 * lane + e;
      const bool valid = key < n;
      const bool forced = key < flo || key >= fhi;
      ms[e] = __ballot(valid && (forced || (above_ok && sb[e] > hi)));
      wc += (uint32_t)__popcll(__ballot(valid && !forced && sb[e] <= hi && sb[e] >= lo));
    }
    // block j = base / 256: words 8j + 2e (+1) = the ballot of the lanes' e-th keys
    if (lane < 8) {
      const uint64_t a = ms[lane >> 1];
      lbm[(base >> 5) + lane] = (lane & 1) ? (uint32_t)(a >> 32) : (uint32_t)a;
    }
  }
  if (lane == 0) wcount[wave] = wc;
  __syncthreads();
  uint32_t cpos = 0u, C = 0u;
#pragma unroll
  for (int w = 0; w < kResWaves; ++w) {
    const uint32_t c = wcount[w];
    cpos += w < wave ? c : 0u;
    C += c;
  }
  const bool in_lds = C <= (uint32_t)kCandCap;
  // pass 2: this wave's candidates in key order from its base position
  if (in_lds && wc) {  // uniform per wave
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint32_t base = (uint32_t)(r * kOneKeys + wave * 256);
      const uint32_t sb[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = base + 4 * lane + e;
        const bool c = key < n && key >= flo && key < fhi && sb[e] <= hi && sb[e] >= lo;
        const uint64_t mc = __ballot(c);
        if (c) lcand[cpos + (uint32_t)__popcll(mc & lt)] = make_uint2(sb[e], key);
        cpos += (uint32_t)__popcll(mc);
      }
    }
  }
  __syncthreads();

  // the candidates that complete the top-k
  uint32_t need = k > 0 ? (uint32_t)k - bd.above : 0u;  // 1 <= need <= C when k > 0
  uint32_t vmask = 0u, vval = 0u, imax = 0xFFFFFFFFu;
  if (k > 0 && need < C) {  // uniform
    uint32_t ties = 0u;
    for (int shift = 14; shift >= 0; shift -= 7) {
      const Pick pk = in_lds
          ? radix_pick<false>(lcand, C, vmask, vval, 0u, 0u, shift, need, h128, &shpick)
          : radix_regs<NR, false>(v, n, flo, fhi, lo, hi, vmask, vval, 0u, 0u, shift, need,
                                  h128, &shpick);
      need -= pk.before;
      vval |= pk.digit << shift;
      vmask |= 127u << shift;
      ties = pk.inbin;
    }
    if (ties > need) {  // among keys with exactly that score, the lower indices win
      uint32_t imask = 0u, ival = 0u;
      int top = 0;
      while (((uint64_t)1 << top) < (uint64_t)n) ++top;
      int shift = top > 7 ? top - 7 : 0;
      for (;;) {
        const Pick pk = in_lds
            ? radix_pick<true>(lcand, C, vmask, vval, imask, ival, shift, need, h128, &shpick)
            : radix_regs<NR, true>(v, n, flo, fhi, lo, hi, vmask, vval, imask, ival, shift,
                                   need, h128, &shpick);
        need -= pk.before;
        ival |= pk.digit << shift;
        imask |= 127u << shift;
        if (shift == 0) break;
        shift = shift > 7 ? shift - 7 : 0;
      }
      imax = ival;
    }
  }
  // the chosen candidates join the bitmap
  if (in_lds) {
    for (uint32_t i = tid; i < C; i += kResThreads) {
      const uint2 e = lcand[i];
      const uint32_t low = e.x & 0x1FFFFFu;
      if (low > vval || (low == vval && e.y <= imax)) {
        const uint32_t i4 = (e.y >> 2) & 63u, ee = e.y & 3u;
        atomicOr(&lbm[(e.y >> 8) * 8 + ee * 2 + (i4 >> 5)], 1u << (i4 & 31));
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint32_t key = (uint32_t)(r * kOneKeys + 4 * tid);
      const uint32_t m = cand_bits<NR>(v, r, key, n, flo, fhi, lo, hi);
      const uint32_t sb[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t low = sb[e] & 0x1FFFFFu, kk = key + (uint32_t)e;
        if (((m >> e) & 1u) && (low > vval || (low == vval && kk <= imax))) {
          const uint32_t i4 = (kk >> 2) & 63u;
          atomicOr(&lbm[(kk >> 8) * 8 + (uint32_t)e * 2 + (i4 >> 5)], 1u << (i4 & 31));
        }
      }
    }
  }
  __syncthreads();
  // key-order 32-bit words from the block masks (W consecutive words a thread)
  constexpr int W = (NR * kOneKeys / 32 + kResThreads - 1) / kResThreads;
  const int64_t segw = ((int64_t)n + 31) >> 5;
  uint32_t kw[W];
  uint32_t cnt = 0u;
#pragma unroll
  for (int q = 0; q < W; ++q) {
    const int64_t wi = (int64_t)tid * W + q;
    uint32_t x = 0u;
    if (wi < segw) {
      const int blk = (int)(wi >> 3), sub = (int)(wi & 7);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t b8 = (lbm[blk * 8 + 2 * e + (sub >> 2)] >> ((sub & 3) * 8)) & 255u;
        x |= spread4(b8) << e;  // key 4i + e of the word at bit 4i + e
      }
    }
    kw[q] = x;
    cnt += __popc(x);
  }
  const uint32_t incw = block_incl_scan<kResThreads>(cnt, wsum);
  uint32_t pos = incw - cnt;
#pragma unroll
  for (int q = 0; q < W; ++q) {
    uint32_t x = kw[q];
    const uint32_t kbase = (uint32_t)(((int64_t)tid * W + q) * 32);
    while (x) {
      const int bit = __ffs(x) - 1;
      x &= x - 1;
      if (pos < (uint32_t)k_max) out[pos] = (int32_t)(kbase + bit);
      ++pos;
    }
  }
  for (int64_t t = z.total + tid; t < k_max; t += kResThreads) out[t] = -1;
}

// ---------------------------------------------------------------- launchers

static int device_cus() {
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

template <int G, int TL, bool WIDE>
static void launch_scorer(int B, int Hkv, int Hq, int P, int64_t n_cap, SinkWindow sw,
                          float* usum, const ScoreWs& ws,
                          const uint8_t* ids, const float* vnorm, const int32_t* lens,
                          float* scores, hipStream_t s) {
  // one block per CU: the 64-key groups of every KV row are split evenly
  const int64_t ng = ids_groups(n_cap);
  const int64_t rows = (int64_t)B * Hkv;
  int64_t nblk = (device_cus() + rows - 1) / rows;
  if (nblk > ng) nblk = ng;
  const int64_t gpb = (ng + nblk - 1) / nblk;
  nblk = (ng + gpb - 1) / gpb;
  const int64_t grid = (rows * nblk + kXcds - 1) / kXcds * kXcds;
  scorer_kernel<G, TL, WIDE><<<(unsigned)grid, kScoreThreads, 0, s>>>(
      ws.img, ws.img_floats, ids, vnorm, lens, Hq, Hkv, P, n_cap, sw.sink, sw.window, (int)rows,
      (int)nblk, (int)gpb, scores, ws.hist, usum);
}

template <int G>
static void launch_scorer_g(int B, int Hkv, int Hq, int L, int P, int64_t n_cap, SinkWindow sw,
                            float* usum,
                            const ScoreWs& ws, const uint8_t* ids, const float* vnorm,
                            const int32_t* lens, float* scores, hipStream_t s) {
  if (P > 8) {  // two-byte IDs, L <= 64
    switch (ids_tables_per_word(L)) {
      case 1: launch_scorer<G, 1, true>(B, Hkv, Hq, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
      case 2: launch_scorer<G, 2, true>(B, Hkv, Hq, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
      default: launch_scorer<G, 4, true>(B, Hkv, Hq, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
    }
    return;
  }
  switch (ids_tables_per_word(L)) {
    case 1: launch_scorer<G, 1, false>(B, Hkv, Hq, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
    case 2: launch_scorer<G, 2, false>(B, Hkv, Hq, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
    case 4: launch_scorer<G, 4, false>(B, Hkv, Hq, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
    default: launch_scorer<G, 8, false>(B, Hkv, Hq, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
  }
}

hipError_t launch_soft_tables(const void* q, int dtype, int B, int Hq, int Hkv, const void* W,
                              int L, int P, float tau, const ScoreWs& ws, hipStream_t s,
                              AppendKey ak) {
  const int G = Hq / Hkv;
  const ImageDims im = image_dims(G == 1 || G == 2 ? G : 4, L, P);
  const int rows = B * Hkv;
  const int TLw = ids_tables_per_word(L);
  const int nab = ak.K ? (16 + kTabThreads / (TLw * P) - 1) / (kTabThreads / (TLw * P)) : 0;
  const unsigned grid = (unsigned)(rows * (16 + nab));
  auto go = [&](auto tag, auto gtag) {
    using T = decltype(tag);
    constexpr int GG = decltype(gtag)::value;
    soft_tables_kernel<T, GG><<<grid, kTabThreads, 0, s>>>(
        static_cast<const T*>(q), static_cast<const T*>(W), Hq, Hkv, L, P, tau, im.TL, im.NF,
        im.NS, im.HE, im.full, ws.img_floats, ws.img, ws.hist, ws.counters, ws.usum, ak, rows,
        nab);
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  if (dtype == 1) {
    if (G == 1) go(uint16_t{}, I1{});
    else if (G == 2) go(uint16_t{}, I2{});
    else go(uint16_t{}, I4{});
  } else {
    if (G == 1) go(float{}, I1{});
    else if (G == 2) go(float{}, I2{});
    else go(float{}, I4{});
  }
  return hipGetLastError();
}

hipError_t launch_score(int B, int Hq, int Hkv, int L, int P, const uint8_t* ids,
                        const float* vnorm, const int32_t* lens, int64_t n_cap, SinkWindow sw,
                        float* scores, bool soft_sums,
                        const ScoreWs& ws, hipStream_t s) {
  float* usum = soft_sums ? ws.usum : nullptr;
  switch (Hq / Hkv) {
    case 1: launch_scorer_g<1>(B, Hkv, Hq, L, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
    case 2: launch_scorer_g<2>(B, Hkv, Hq, L, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
    default: launch_scorer_g<4>(B, Hkv, Hq, L, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_topk(int B, int Hq, const float* scores, const int32_t* lens, int64_t n_cap,
                       const int32_t* ks, int k_max, SinkWindow sw, int32_t* idx, const ScoreWs& ws,
                       hipStream_t s) {
  if (n_cap <= (int64_t)kOneKeys * kOneMaxRounds) {  // every score of a head in one workgroup
    const int rounds = (int)((n_cap + kOneKeys - 1) / kOneKeys);
    auto go = [&](auto rt) {
      constexpr int NR = decltype(rt)::value;
      topk_onepass_kernel<NR><<<(unsigned)((B * Hq + kXcds - 1) / kXcds * kXcds), kResThreads, 0,
                                s>>>(scores, n_cap, score_stride(n_cap), lens, ks, k_max,
                                     sw.sink, sw.window, Hq, B * Hq, ws.hist, idx);
    };
    if (rounds <= 1) go(std::integral_constant<int, 1>{});
    else go(std::integral_constant<int, 2>{});
    return hipGetLastError();
  }
  const int CH = (int)((n_cap + kScanKeys - 1) / kScanKeys);
  const int64_t nscan = (int64_t)B * Hq * CH;
  const unsigned sgrid = (unsigned)((nscan + kXcds - 1) / kXcds * kXcds);
  // two kScanThreads workgroups fit a CU; beyond that, the small ones
  if (nscan <= 2 * (int64_t)device_cus())
    topk_scan_kernel<kScanThreads, kScanKeys / (kScanThreads / 64)><<<sgrid, kScanThreads, 0, s>>>(
        scores, n_cap, score_stride(n_cap), lens, ks, k_max, sw.sink, sw.window, Hq, CH, B * Hq,
        ws.hist, ws.counters, ws.bitmap, ws.words, ws.cand);
  else
    topk_scan_kernel<256, 256><<<sgrid, 256, 0, s>>>(
        scores, n_cap, score_stride(n_cap), lens, ks, k_max, sw.sink, sw.window, Hq, CH, B * Hq,
        ws.hist, ws.counters, ws.bitmap, ws.words, ws.cand);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (B * Hq <= device_cus())
    topk_resolve_kernel<kResThreads><<<(unsigned)(B * Hq), kResThreads, 0, s>>>(
        n_cap, lens, ks, k_max, sw.sink, sw.window, Hq, ws.hist, ws.counters, ws.bitmap, ws.words,
        ws.cand, idx);
  else
    topk_resolve_kernel<512><<<(unsigned)(B * Hq), 512, 0, s>>>(
        n_cap, lens, ks, k_max, sw.sink, sw.window, Hq, ws.hist, ws.counters, ws.bitmap, ws.words,
        ws.cand, idx);
  return hipGetLastError();
}

}  // namespace socketlsh
