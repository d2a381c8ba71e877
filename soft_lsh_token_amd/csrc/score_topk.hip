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
  const int img_floats = image_stride(pass_heads(G), L);
  const size_t rows = (size_t)B * Hkv * pass_subs(G);  // one image per sub-row
  const size_t n = select_ws_layout(rows * img_floats * sizeof(float), B, Hq, n_cap, ws, base);
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
  const size_t o_gs = off; off = align256(off + heads * (size_t)ids_groups(n_cap) * sizeof(float));
  const size_t o_ep = off; off = align256(off + heads * kEstSlices * kHead * sizeof(float));
  const size_t o_ez = off; off = align256(off + heads * 2 * sizeof(float));
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
    ws->gsum = reinterpret_cast<float*>(p + o_gs);
    ws->epart = reinterpret_cast<float*>(p + o_ep);
    ws->esz = reinterpret_cast<float*>(p + o_ez);
    ws->groups = ids_groups(n_cap);
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

// grid: rows*16 blocks of kTabThreads, rows = B*Hkv*sub sub-rows of G query
// heads each.  Block (bh, j) computes the tables j*TL .. j*TL+TL-1 (the
// tables of scorer lane j) for the G query heads of sub-row bh and writes
// their image slots whole (one slot = the G heads' values of one entry).  It
// also clears a 1/16 share of those heads' histograms (block j = 0: their
// candidate counters and soft-count sums).
// Tables l >= L (padding of the last lane word) get all-zero entries.
// With ak.K set, blocks past the first rows*16 hash the key appended at
// position lens[b] - 1 of each of the B*Hkv KV rows (append_block below).
template <typename T>
__device__ void append_block(const T* __restrict__ W, int Hkv, int L, int P, int TL, int nab,
                             int rows, const AppendKey& ak);

template <typename T, int G, bool TWO>
__global__ __launch_bounds__(kTabThreads) void soft_tables_kernel(
    const T* __restrict__ q, const T* __restrict__ W, int Hq, int Hkv, int L, int P, float tau,
    int TL, int NF, int NS, int HE, int FULL, int img_floats, float* __restrict__ img,
    uint32_t* __restrict__ hist, uint32_t* __restrict__ counters, float* __restrict__ usum,
    AppendKey ak, int rows, int nab, int sub) {
  if ((int)blockIdx.x >= rows * 16) {  // uniform
    append_block<T>(W, Hkv, L, P, TL, nab, rows, ak);
    return;
  }
  const int Hv = Hkv * sub;  // sub-rows per sequence (rows = B * Hv)
  // Logical table block lid = (blockIdx mod 8) * (2 rows) + blockIdx / 8: the
  // 16 blocks of a KV row share an XCD (blocks go to the XCDs round robin),
  // so the 16-byte slots they write into each image line meet in one L2.
  const int lid = (int)(blockIdx.x % kXcds) * (rows * 16 / kXcds) + (int)(blockIdx.x / kXcds);
  const int bh = lid >> 4, j = lid & 15;
  const int b = bh / Hv, h = bh % Hv;
  const int bg0 = b * Hq + h * G;
  const int tid = threadIdx.x;
  float* im = img + (int64_t)bh * img_floats;
  // the queries (exact in float32), row 2g + h = half h of head g, rows
  // padded to 68 floats so the 2G rows the lanes of a wave read at one time
  // sit in different bank groups
  constexpr int kQRow = kHead / 2 + 4;
  __shared__ float qf[2 * G][kQRow];
  __shared__ double sig[kTabThreads][2];  // [(m*P + plane)*G + g][bit] = sigmoid(+-2u/tau)
  // [(m*G + g)*2HE + hf*HE + c]: TL*G*2*HE <= 256*G entries (TL <= 8 with
  // HE = 16, TL <= 4 with HE = 32)
  __shared__ double half[256 * G];

  constexpr int kHistShare = G * kHistBins / 16;
  for (int i = tid; i < kHistShare; i += kTabThreads)
    hist[(int64_t)bg0 * kHistBins + j * kHistShare + i] = 0u;
  if (j == 0 && tid < G) {
    counters[bg0 + tid] = 0u;
    usum[bg0 + tid] = 0.f;
  }
  for (int i = tid; i < G * kHead; i += kTabThreads) {
    const int64_t src = (int64_t)(bg0 + i / kHead) * kHead + i % kHead;
    float* dst = &qf[2 * (i / kHead) + (i % kHead) / (kHead / 2)][(i % kHead) % (kHead / 2)];
    if constexpr (sizeof(T) == 2) *dst = __uint_as_float((uint32_t)q[src] << 16);
    else *dst = q[src];
  }
  // projections: eight threads per W row (table member m, plane pl); thread
  // s of the eight takes elements 16s .. 16s+15 of the row's dot products
  // with all G queries, so each row is read once, and three butterfly steps
  // add the eight partial sums
  constexpr int EPT = kHead / 8;                  // elements a thread
  constexpr int NV = EPT * (int)sizeof(T) / 16;   // 16-byte vectors a thread
  const int nrows = TL * P;                       // TWO: more than kTabThreads / 8
  const int s8 = tid & 7;
  constexpr int NIT = TWO ? 2 : 1;  // rounds of rows
  uint4 raw[NIT][NV];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int row = (tid >> 3) + it * (kTabThreads / 8);
    const int l = j * TL + row / P;
    if (row < nrows && l < L) {
      const uint4* wr = reinterpret_cast<const uint4*>(W + (int64_t)(l * P + row % P) * kHead +
                                                       s8 * EPT);
#pragma unroll
      for (int v = 0; v < NV; ++v) raw[it][v] = wr[v];
    }
  }
  lds_barrier();  // the queries (the W loads and histogram clears stay in flight)
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int row = (tid >> 3) + it * (kTabThreads / 8);
    if (it * (kTabThreads / 8) >= nrows) break;  // uniform
    const int l = j * TL + row / P;
    const bool live = row < nrows && l < L;
    const float* qrow = &qf[s8 / 4][(s8 % 4) * EPT];  // this slice of head 0's query
    double acc[G][4];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g][0] = acc[g][1] = acc[g][2] = acc[g][3] = 0.0;
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
#pragma unroll
        for (int e = 0; e < cnt; ++e)
#pragma unroll
          for (int g = 0; g < G; ++g)
            acc[g][e & 3] = fma((double)f[e], (double)qrow[2 * g * kQRow + v * cnt + e],
                                acc[g][e & 3]);
      }
    }
    // every lane of the eight gets every head's sum; lane g of them takes
    // head g's sigmoid, so the G exponentials run side by side
    double ug = 0.0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      double u = (acc[g][0] + acc[g][1]) + (acc[g][2] + acc[g][3]);
      u += __shfl_xor(u, 1, 64);
      u += __shfl_xor(u, 2, 64);
      u += __shfl_xor(u, 4, 64);
      if (s8 == g) ug = u;
    }
    if (row < nrows && s8 < G) {
      // sigmoid(x) and sigmoid(-x) from one exponential of -|x|
      const double x = 2.0 * ug / (double)tau;
      const double e = exp(-fabs(x));
      const double big = 1.0 / (1.0 + e), small = e * big;
      sig[row * G + s8][1] = x >= 0.0 ? big : small;  // bit set: corner sign +1
      sig[row * G + s8][0] = x >= 0.0 ? small : big;  // bit clear: corner sign -1
    }
  }
  lds_barrier();  // the sigmoids (global stores and loads stay in flight)
  // halves: planes 0 .. plo-1 and plo .. P-1, HE entries each
  const int plo = HE == 32 ? 5 : (P < 4 ? P : 4);
  const int phi = P - plo;
  const int hs = HE == 32 ? 5 : 4;  // log2 HE (16 or 32): shifts, not divisions
  for (int i = tid; i < TL * G * 2 * HE; i += kTabThreads) {
    const int pair = i >> (hs + 1), mm = pair / G, gg = pair % G, r = i & (2 * HE - 1);
    const int hf = r >> hs, c = r & (HE - 1);
    const int nb = hf ? phi : plo;
    double prod = 0.0;
    if (c < (1 << nb) && j * TL + mm < L) {
      // at most 5 planes a half: all of its sigmoids requested at once (rows
      // past nb, clamped inside sig, are not multiplied in)
      const int p0 = hf ? plo : 0;
      double sv[5];
#pragma unroll
      for (int jj = 0; jj < 5; ++jj) {
        const int row = (mm * P + p0 + jj) * G + gg;
        sv[jj] = sig[row < kTabThreads ? row : kTabThreads - 1][(c >> jj) & 1];
      }
      prod = 1.0;
#pragma unroll
      for (int jj = 0; jj < 5; ++jj)
        if (jj < nb) prod *= sv[jj];
    }
    half[(mm * G + gg) * 2 * HE + r] = prod;
  }
  lds_barrier();  // the halves
  // full tables, table-major: slot (m*256 + e)*16 + j for entries e < 2^P
  const int nent = 1 << P;
  const int lomask = (1 << plo) - 1;
  for (int mm = 0; mm < NF; ++mm) {
    for (int e = tid; e < nent; e += kTabThreads) {
      float v[G];
#pragma unroll
      for (int gg = 0; gg < G; ++gg)
        v[gg] = (float)(half[(mm * G + gg) * 2 * HE + (e & lomask)] *
                        half[(mm * G + gg) * 2 * HE + HE + (e >> plo)]);
      store_slot<G>(im + ((int64_t)(mm * 256 + e) * 16 + j) * G, v);
    }
  }
  // factored tables: slot FULL/G + ((hc*NS + m - NF)*16 + j), hc = hf*HE + c
  for (int ms = 0; ms < NS; ++ms) {
    for (int hc = tid; hc < 2 * HE; hc += kTabThreads) {
      const int mm = NF + ms, i = hc * NS + ms;
      float v[G];
#pragma unroll
      for (int gg = 0; gg < G; ++gg) v[gg] = (float)half[(mm * G + gg) * 2 * HE + hc];
      store_slot<G>(im + FULL + ((int64_t)i * 16 + j) * G, v);
    }
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
  // the first half of the plane's W row first: it does not depend on the key
  // position (the second half comes after it is used, so that the append
  // path needs no more registers than the table blocks of the same launch)
  constexpr int NV = kHead * (int)sizeof(T) / 16;
  constexpr int NH = NV / 2;
  const uint4* wr = reinterpret_cast<const uint4*>(W + (int64_t)(live ? l * P + pl : 0) * kHead);
  uint4 wv[NH];
  if (live) {
#pragma unroll
    for (int v = 0; v < NH; ++v) wv[v] = wr[v];
  }
  const int64_t pos = (int64_t)ak.lens[b] - 1;
  if (pos < 0 || pos >= ak.n_cap) return;  // uniform: no key to append
  const int64_t row = (int64_t)bh * ak.n_cap + pos;
  const T* K = static_cast<const T*>(ak.K);
  const T* V = static_cast<const T*>(ak.V);
  __shared__ float kf[kHead];
  __shared__ uint32_t kbit[kTabThreads];
  // the key's elements and the value row's slices requested together, every
  // thread from an in-range address (one round trip, not two)
  const T kraw = K[row * kHead + (tid < kHead ? tid : 0)];
  const int vs = tid & 15;
  Row8<T> vraw = fetch_row8<T>(V + row * kHead, vs);
  if (tid < kHead) {
    if constexpr (sizeof(T) == 2) kf[tid] = __uint_as_float((uint32_t)kraw << 16);
    else kf[tid] = kraw;
  }
  const bool norm = a == 0 && tid < 16;  // lanes 0..15 of wave 0: the value norm
  float vf[8];
  unpack_row8<T>(vraw, vf);
  __syncthreads();
  float z = 0.f;
  if (live) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (hh == 1) {
#pragma unroll
        for (int v = 0; v < NH; ++v) wv[v] = wr[NH + v];
      }
#pragma unroll
      for (int v = 0; v < NH; ++v) {
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
        for (int e = 0; e < cnt; ++e) z = fmaf(f[e], kf[(hh * NH + v) * cnt + e], z);
      }
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
    const int CB = ids_cell_bits(L, P);
    uint64_t w = 0ull;
    for (int mm = 0; mm < TL; ++mm) {
      uint64_t id = 0ull;
      if (wd * TL + mm < L)
        for (int p2 = 0; p2 < P; ++p2) id |= (uint64_t)kbit[tid * WP + mm * P + p2] << p2;
      w |= id << (CB * mm);
    }
    ids_store_word(ak.ids, bh, ak.n_cap, L, P, pos, wd, w);
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

// The ID word of round x from the lane's NV 16-byte vectors: WB = NV bytes
// (w.x, and w.y for WB = 8), or, packed (PK, five vectors), the low 32 bits
// in w.x and the high byte in w.y.
template <int NV, bool PK>
__device__ __forceinline__ uint2 round_word(const uint4 (&v)[NV], int x) {
  if constexpr (PK) {
    static_assert(NV == 5, "packed words: four vectors of low words and one of high bytes");
    const uint4 q = v[x >> 2];
    const uint32_t lo = (x & 3) == 0 ? q.x : (x & 3) == 1 ? q.y : (x & 3) == 2 ? q.z : q.w;
    const uint4 h = v[4];
    const uint32_t hd = (x >> 2) == 0 ? h.x : (x >> 2) == 1 ? h.y : (x >> 2) == 2 ? h.z : h.w;
    return make_uint2(lo, hd >> (8 * (x & 3)));
  } else {
    constexpr int WB = NV;
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
}

// Cell M of a word of C-byte cells.
template <int C, int M>
__device__ __forceinline__ uint32_t word_cell(uint2 w) {
  if constexpr (C == 1) return ((M < 4 ? w.x : w.y) >> (8 * (M & 3))) & 255u;
  else return ((M < 2 ? w.x : w.y) >> (16 * (M & 1))) & 0xFFFFu;
}

constexpr int kPrefetch = 1;  // 64-key groups of IDs each wave keeps in flight
// The fixed cost of a scorer row segment (its image load, barrier and
// histogram merge, about 4.7 us) in 64-key groups of a 512-thread block
// (about 0.32 us each), for splitting ragged batches.
constexpr int kSegGroups = 15;

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

// Half-table lookups of tables NF .. NF+NS-1 (C-byte cells, HE-entry halves;
// PK: ten-bit cells at bit 10*T of the 40-bit word, five-bit halves).
template <int NF, int NS, int G, int C, int HE, bool PK, int M = 0>
__device__ __forceinline__ void issue_half(const float* lds, uint2 w, int j, int plo,
                                           RoundVals<NF, NS, G>& r) {
  if constexpr (M < NS) {
    // the two factors' entries as bit fields of the word (one extract each)
    constexpr int T = NF + M;
    uint32_t lo, hi;
    if constexpr (PK) {
      static_assert(NF == 0 && NS == 4, "packed words hold four factored tables");
      if constexpr (T < 3) {
        lo = __builtin_amdgcn_ubfe(w.x, 10 * T, 5);
        hi = __builtin_amdgcn_ubfe(w.x, 10 * T + 5, 5);
      } else {  // bits 30 .. 39 straddle the low word and the high byte
        lo = __builtin_amdgcn_alignbit(w.y, w.x, 30) & 31u;
        hi = __builtin_amdgcn_ubfe(w.y, 3, 5);
      }
    } else {
      constexpr int PER = 4 / C;  // cells per 32-bit half of the word
      const uint32_t src = T < PER ? w.x : w.y;
      constexpr uint32_t off = 8 * C * (T % PER);
      lo = __builtin_amdgcn_ubfe(src, off, (uint32_t)plo);
      hi = __builtin_amdgcn_ubfe(src, off + (uint32_t)plo, 8 * C - (uint32_t)plo);
    }
    lds_get<G>(lds, ((int)lo * NS + M) * 16 + j, r.lo[M]);
    lds_get<G>(lds, ((HE + (int)hi) * NS + M) * 16 + j, r.hi[M]);
    issue_half<NF, NS, G, C, HE, PK, M + 1>(lds, w, j, plo, r);
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
template <int NF, int NS, int G, int C, int HE, int NV, bool PK>
__device__ __forceinline__ void score_group(const float* lds, const uint4 (&ids)[NV], int j,
                                            int plo, float (&u)[8][G]) {
  constexpr int FULL = 256 * NF * 16 * G;
  const uint32_t jw = ((uint32_t)j << 4) | 0x100u;
  RoundVals<NF, NS, G> cur, nxt;
  {
    const uint2 w = round_word<NV, PK>(ids, 0);
    issue_full<NF, NS, G>(lds, w, j, jw, cur);
    issue_half<NF, NS, G, C, HE, PK>(lds + FULL, w, j, plo, cur);
  }
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    if (x < 15) {
      const uint2 w = round_word<NV, PK>(ids, x + 1);
      issue_full<NF, NS, G>(lds, w, j, jw, nxt);
      issue_half<NF, NS, G, C, HE, PK>(lds + FULL, w, j, plo, nxt);
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

// grid: a multiple of kXcds blocks of kScoreThreads, at least rows*nblk.
// Rows are sub-rows (Hkv of them per sequence): sub-row bh serves the G query
// heads b*Hq + (bh % Hkv)*G + [0, G) and reads the IDs and norms of KV row
// bh / sub (sub = 1 when a KV row has at most 4 query heads).
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
    const float* __restrict__ vnorm, const int32_t* __restrict__ lens, int Hq, int Hkv, int sub,
    int P, int64_t n_cap, int sink, int window, int rows, int nblk, int gpb,
    float* __restrict__ scores,
    uint32_t* __restrict__ hist, float* __restrict__ usum, float* __restrict__ gsum) {
  using Sh = ImageShape<G, TL, WIDE>;
  constexpr int NF = Sh::NF, NS = Sh::NS, HE = Sh::HE;
  constexpr int C = WIDE ? 2 : 1;  // bytes per ID
  constexpr int WB = TL * C;       // bytes per ID word (unpacked)
  constexpr bool PK = WIDE && TL == 4;      // packed ten-bit cells
  constexpr int NV = PK ? 5 : WB;           // 16-byte ID vectors per lane and group
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

  // Score groups [g_begin, g_end) (g_begin < g_end) of sub-row bh; every wave
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
    const int kv = bh / sub;  // the KV row of this sub-row
    const uint8_t* idg = ids + (int64_t)kv * ids_groups(n_cap) * 1024 * NV;
    const float* vrow = vnorm + (int64_t)kv * n_cap;
    auto load_group = [&](int64_t gi, uint4 (&v)[NV], float& vn) {
      const int64_t gl = gi < g_end ? gi : g_end - 1;
      const uint4* src = reinterpret_cast<const uint4*>(idg + gl * 1024 * NV) + lane;
#pragma unroll
      for (int qv = 0; qv < NV; ++qv) v[qv] = src[qv * 64];
      const int64_t key = gl * 64 + lane;
      vn = vrow[key < n_cap ? key : n_cap - 1];
    };
    uint4 buf[D + 1][NV];
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
          score_group<NF, NS, G, C, HE, NV, PK>(lds, buf[s], j, plo, u);
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
          if (gsum) {  // uniform: each head's score sum over the group (estimator)
#pragma unroll
            for (int gg = 0; gg < G; ++gg) {
              const float t = wave_incl_scan_f32(valid ? vb[s] * u[0][gg] : 0.f);
              if (lane == 63) gsum[(int64_t)(bg0 + gg) * ids_groups(n_cap) + gi] = t;
            }
          }
          gi += kScoreWaves;
          more = gi < g_end;
        }
      }
    }
    lds_barrier();  // the LDS histogram is complete (the score stores stay in flight)
    for (int i = tid; i < G * kHistBins; i += kScoreThreads) {
      const uint32_t v = lhist[i];
      if (v) atomicAdd(&hist[(int64_t)(bg0 + i / kHistBins) * kHistBins + (i % kHistBins)], v);
    }
    if (usum) {  // per-head sums of the soft counts, for the sampling estimator
      lds_barrier();  // the merge above has read the histogram: reuse its LDS
      float* red = reinterpret_cast<float*>(lhist);  // [kScoreWaves][G]
#pragma unroll
      for (int gg = 0; gg < G; ++gg) {
        const float t = wave_sum(us[gg]);
        if (lane == 0) red[wave * G + gg] = t;
      }
      lds_barrier();
      if (tid < G) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < kScoreWaves; ++w) t += red[w * G + tid];
        atomicAdd(&usum[bg0 + tid], t);
      }
    }
    lds_barrier();  // a following segment reuses the image and histogram LDS
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
  // Each non-empty row counts kSegGroups groups more than it holds (a row
  // segment's image load and histogram merge cost about that much), so a
  // share that spans row starts takes fewer keys; a share inside a row's
  // extra groups scores nothing there.  The totals and offsets are
  // wave-uniform and kept in scalar registers.
  auto padded = [&](int b) {  // a row's groups plus its fixed cost, 0 for an empty row
    const uint32_t ng = (uint32_t)((seq_len(b) + 63) >> 6);
    return ng ? ng + (uint32_t)kSegGroups : 0u;
  };
  uint32_t total = 0u;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const uint32_t ng = b < B ? padded(b) : 0u;
    total += (uint32_t)__builtin_amdgcn_readfirstlane((int)__shfl(wave_incl_scan(ng), 63, 64)) *
             (uint32_t)Hkv;
  }
  const uint32_t shares = (uint32_t)(rows * nblk);
  const uint32_t per = (total + shares - 1) / shares;
  uint32_t G0 = (uint32_t)lid * per;
  const uint32_t G1 = G0 + per < total ? G0 + per : total;
  int bcur = 0;
  uint32_t base = 0u;  // padded groups of the sequences before bcur (all KV heads)
  while (G0 < G1) {
    // the sequence whose padded groups hold G0, by a wave scan over 64 sequences at a time
    for (;;) {
      const int b = bcur + lane;
      const uint32_t ng = b < B ? padded(b) * (uint32_t)Hkv : 0u;
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
    const uint32_t ngp = padded(bcur);  // > 0: G0 lies in this sequence's rows
    const uint32_t h = (G0 - base) / ngp;
    const uint32_t row0 = base + h * ngp;  // padded start of KV row (bcur, h)
    const uint32_t row1 = row0 + ngp;
    const uint32_t s1 = G1 < row1 ? G1 : row1;
    const uint32_t k = (uint32_t)kSegGroups;  // the row's groups start after its fixed cost
    const uint32_t a = G0 - row0 > k ? G0 - row0 - k : 0u;
    const uint32_t e = s1 - row0 > k ? s1 - row0 - k : 0u;
    if (a < e) segment(bcur * Hkv + (int)h, (int64_t)a, (int64_t)e);
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

// Block-wide inclusive scan of one value per thread (NT threads).  Its
// barriers order LDS only: global loads and stores in flight stay in flight.
template <int NT>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_incl_scan(v);
  lds_barrier();
  if (lane == 63) wsum[wave] = v;
  lds_barrier();
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
  lds_barrier();  // LDS only: the caller's bulk loads stay in flight
  const Boundary r = *sh;
  lds_barrier();
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

// ---------------------------------------------------------------- attention in the selecting workgroup

// Exact softmax attention (SOCKET Sec. 2 and Sec. 4.1, Algorithm 3) of one
// query over the S keys listed in LDS `sel`, run by the NT threads of the
// workgroup that selected them, so a decode step needs no separate attention
// launches.  16 lanes share a key row (8 head elements each); the R = NT/16
// rows take keys t = row, row + R, ... in batches of AB, every K and V load of
// a batch issued before any is used, and keep an online softmax (m, l, o).
// The R rows are then merged in row order (fixed order, so results repeat bit
// for bit): M = max m_r, w_r = exp(m_r - M), out = sum w_r o_r / sum w_r l_r.
// mo: R*kHead floats of LDS, mml: 2*R floats of LDS.
template <typename T, int NT, int AB>
__device__ __forceinline__ void attend_selected(const T* __restrict__ qrow, const T* __restrict__ Kh,
                                const T* __restrict__ Vh, const int32_t* sel, int S, float scale,
                                float* mo, float* mml, float* __restrict__ out) {
  constexpr int R = NT / 16;
  const int tid = threadIdx.x, j = tid & 15, row = tid >> 4;
  float qf[8];
  load_row8<T>(qrow, j, qf);
  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  for (int t0 = row; t0 < S; t0 += R * AB) {  // the 16 lanes of a row agree
    int32_t ki[AB];
#pragma unroll
    for (int a = 0; a < AB; ++a) {
      const int t = t0 + a * R;
      ki[a] = t < S ? sel[t] : -1;
    }
    Row8<T> kr[AB], vr[AB];
#pragma unroll
    for (int a = 0; a < AB; ++a) {
      const int64_t r = ki[a] >= 0 ? ki[a] : 0;
      kr[a] = fetch_row8<T>(Kh + r * kHead, j);
      vr[a] = fetch_row8<T>(Vh + r * kHead, j);
    }
    float lg[AB], mx = m;
#pragma unroll
    for (int a = 0; a < AB; ++a) {
      float kf[8];
      unpack_row8<T>(kr[a], kf);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(qf[e], kf[e], dot);
      dot = row16_sum(dot);
      lg[a] = ki[a] >= 0 ? dot * scale : -INFINITY;
      mx = fmaxf(mx, lg[a]);
    }
    // t0 < S, so the batch's first key is a real one and mx is finite
    const float c = m == -INFINITY ? 0.f : __expf(m - mx);
    l *= c;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= c;
#pragma unroll
    for (int a = 0; a < AB; ++a) {
      const float p = lg[a] == -INFINITY ? 0.f : __expf(lg[a] - mx);
      float vf[8];
      unpack_row8<T>(vr[a], vf);
      l += p;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(p, vf[e], o[e]);
    }
    m = mx;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) mo[row * kHead + 8 * j + e] = o[e];
  if (j == 0) {
    mml[2 * row] = m;
    mml[2 * row + 1] = l;
  }
  __syncthreads();
  if (tid < kHead) {
    float M = -INFINITY;
    for (int r = 0; r < R; ++r)
      if (mml[2 * r + 1] > 0.f) M = fmaxf(M, mml[2 * r]);
    float L = 0.f, O = 0.f;
    for (int r = 0; r < R; ++r) {
      const float lr = mml[2 * r + 1];
      const float w = lr > 0.f ? __expf(mml[2 * r] - M) : 0.f;
      L = fmaf(lr, w, L);
      O = fmaf(mo[r * kHead + tid], w, O);
    }
    out[tid] = L > 0.f ? O / L : 0.f;
  }
}

// Where a selecting workgroup attends: its query row, the K and V rows of its
// KV head, the scale, and its output row.
template <typename T>
struct AttendArgs {
  const T* q;
  const T* K;
  const T* V;
  float* out;
  int Hkv;
  float scale;
};

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

  // every independent load at once: candidate count, the first NT
  // candidates (one a thread, whatever their count), this thread's first
  // bitmap block, its histogram bin (inside find_boundary)
  const HistSlice<NT> hs = load_hist_slice<NT>(hist + (int64_t)bg * kHistBins);
  const uint2* gc = cand + (int64_t)bg * n_cap;
  const uint32_t* bm = bitmap + (int64_t)bg * words;
  const uint32_t Cg = counters[bg];
  const uint2 cv = gc[(int64_t)tid < n_cap ? (int64_t)tid : n_cap - 1];
  const int64_t nblocks = (n + 255) >> 8;
  const int64_t bl0 = tid < nblocks ? tid : 0;
  const uint4 bw0 = reinterpret_cast<const uint4*>(bm)[bl0 * 2];
  const uint4 bw1 = reinterpret_cast<const uint4*>(bm)[bl0 * 2 + 1];
  const Boundary bd = boundary_of<NT>(hs, (uint32_t)k, sm.wsum, &sm.shb);
  const uint32_t C = Cg < (uint32_t)n ? Cg : (uint32_t)n;
  const bool in_lds = C <= (uint32_t)kCandCap;
  if (in_lds) {
    if ((uint32_t)tid < C) sm.lcand[tid] = cv;
    // more than NT candidates (rare): the rest in a second round trip
    for (uint32_t ci = (uint32_t)(NT + tid); ci < C; ci += NT) sm.lcand[ci] = gc[ci];
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
    lds_barrier();  // the index stores stay in flight
    written += sm.seg_total;
    lds_barrier();
  }
}

// grid: B*Hq blocks of NT threads (1024; 512 for batches of more heads than
// CUs, whose 16-wave workgroups took the dispatcher about 8 us to start).
// With ATT the workgroup then runs the head's attention over its selection
// (attend_selected), which it keeps in the candidate list's LDS: rows of at
// most one emit segment (NT 256-key blocks) and k_max <= 2*kCandCap.
template <int NT, bool ATT, typename T>
__global__ __launch_bounds__(NT) void topk_resolve_kernel(
    int64_t n_cap, const int32_t* __restrict__ lens, const int32_t* __restrict__ ks, int k_max,
    int sink, int window, int Hq, const uint32_t* __restrict__ hist,
    const uint32_t* __restrict__ counters,
    const uint32_t* __restrict__ bitmap, int64_t words, const uint2* __restrict__ cand,
    int32_t* __restrict__ idx, AttendArgs<T> at) {
  const int bg = blockIdx.x;
  const int b = bg / Hq;
  const int tid = threadIdx.x;
  const SelSizes z = sel_sizes(n_cap, lens[b], ks[b], k_max, sink, window);
  int32_t* out = idx + (int64_t)bg * k_max;
  if (z.total == 0) {
    for (int t = tid; t < k_max; t += NT) out[t] = -1;
    if (ATT && tid < kHead) at.out[(int64_t)bg * kHead + tid] = 0.f;
    return;
  }
  __shared__ ResolveSmem<NT> sm;
  __shared__ float mml[ATT ? 2 * (NT / 16) : 1];
  static_assert(NT * 8 >= (NT / 16) * kHead, "the segment bitmap LDS holds the attention merge");
  int32_t* lsel = reinterpret_cast<int32_t*>(sm.lcand);
  resolve_head<NT>(bg, n_cap, z, hist, counters, bitmap, words, cand, sm,
               [&](uint32_t pos, int32_t key) {
                 if (pos < (uint32_t)k_max) {
                   out[pos] = key;
                   if (ATT) lsel[pos] = key;
                 }
               });
  for (int64_t t = z.total + tid; t < k_max; t += NT) out[t] = -1;
  if constexpr (ATT) {
    const int g = bg % Hq, h = g / (Hq / at.Hkv);
    const int64_t kv = ((int64_t)b * at.Hkv + h) * n_cap * kHead;
    const int S = (int)(z.total < k_max ? z.total : k_max);
    attend_selected<T, NT, 4>(
        at.q + (int64_t)bg * kHead, at.K + kv, at.V + kv, lsel, S, at.scale,
        reinterpret_cast<float*>(sm.lbm), mml, at.out + (int64_t)bg * kHead);
  }
}

// ---------------------------------------------------------------- streaming top-k

// The score-bit threshold vval and key threshold imax that complete a top-k
// of `need` among C candidates (all with the same top digit): a candidate is
// chosen iff its low 21 bits exceed vval, or equal it with key <= imax.
// All NT threads call it.
template <int NT>
__device__ void settle_candidates(const uint2* cl, uint32_t C, uint32_t need, uint32_t n,
                                  uint32_t* h128, Pick* shpick, uint32_t& vval, uint32_t& imax) {
  auto pick = [&](auto by_index, uint32_t vm, uint32_t vv, uint32_t im, uint32_t iv, int shift) {
    constexpr bool BI = decltype(by_index)::value;
    return radix_pick<BI, NT>(cl, C, vm, vv, im, iv, shift, need, h128, shpick);
  };
  uint32_t vmask = 0u, ties = 0u;
  vval = 0u;
  imax = 0xFFFFFFFFu;
  for (int shift = 14; shift >= 0; shift -= 7) {
    const Pick pk = pick(std::false_type{}, vmask, vval, 0u, 0u, shift);
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
      const Pick pk = pick(std::true_type{}, vmask, vval, imask, ival, shift);
      need -= pk.before;
      ival |= pk.digit << shift;
      imask |= 127u << shift;
      if (shift == 0) break;
      shift = shift > 7 ? shift - 7 : 0;
    }
    imax = ival;
  }
}

// One workgroup of NT threads per query head does the whole selection in one
// launch and one read of the head's scores (rows of up to 32*BMW keys):
//  1. the bin d1 of the first digit that holds the k-th largest score, from
//     the head's histogram (built by the scorer);
//  2. one pass over the score row, D loads of 16 bytes per thread in flight:
//     wave ballots of "above d1" (and of the sink and window keys) go to an
//     LDS bitmap, and the keys of bin d1 are gathered as candidates (score
//     bits, key) in LDS;
//  3. the candidates that complete the top-k are settled by radix select on
//     the remaining 21 score bits, then on the key (the lower index wins a
//     tie), and join the bitmap;
//  4. the bitmap becomes ascending indices (a block scan of word counts).
// Bitmap layout: 256-key block j (keys 256j + 4i + e, lane i < 64, e < 4) is
// 8 words; words 8j + 2e and 8j + 2e + 1 hold bit i = key 256j + 4i + e, the
// ballot over the wave that loaded 4 consecutive keys per lane.  Blocks
// clear of the row's ends (no sink, window or past-the-end key) cost two
// compares and two ballots per key.
// More candidates than the LDS holds (many equal scores) take a second pass
// that writes them all to the workspace's global list, and step 3 reads them
// there.  Workgroups are remapped as in the scorer
// (logical head (blockIdx mod 8) * (grid / 8) + blockIdx / 8), so a head is
// selected on the XCD whose L2 received its scores.
// With ATT the workgroup then runs the head's attention over its selection
// (attend_selected; the selection is kept in the candidate list's LDS, so
// k_max <= 2*CAP).
template <int NT, int BMW, int CAP, int D, bool ATT, typename T>
__global__ __launch_bounds__(NT) void topk_stream_kernel(
    const float* __restrict__ scores, int64_t n_cap, int64_t sstride,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ ks, int k_max, int sink,
    int window, int Hq, int heads, const uint32_t* __restrict__ hist, uint2* __restrict__ cand,
    int32_t* __restrict__ idx, AttendArgs<T> at) {
  constexpr int NW = NT / 64;
  constexpr int RK = 4 * NT;  // keys per round (one 16-byte load per thread)
  const int bg = (int)(blockIdx.x % kXcds) * (int)(gridDim.x / kXcds) + (int)(blockIdx.x / kXcds);
  if (bg >= heads) return;
  const int b = bg / Hq;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SelSizes z = sel_sizes(n_cap, lens[b], ks[b], k_max, sink, window);
  const int64_t k = z.k;
  int32_t* out = idx + (int64_t)bg * k_max;
  if (z.total == 0) {
    for (int t = tid; t < k_max; t += NT) out[t] = -1;
    if (ATT && tid < kHead) at.out[(int64_t)bg * kHead + tid] = 0.f;
    return;
  }
  static_assert(!ATT || BMW >= (NT / 16) * kHead, "the bitmap LDS holds the attention merge");
  __shared__ uint32_t bm[BMW];
  __shared__ uint2 lc[CAP];
  __shared__ float mml[ATT ? 2 * (NT / 16) : 1];
  int32_t* lsel = reinterpret_cast<int32_t*>(lc);  // the selection, once lc is free
  __shared__ uint32_t wsum[NW];
  __shared__ Boundary shb;
  __shared__ uint32_t h128[128];
  __shared__ Pick shpick;
  __shared__ uint32_t ccount, seg_total;

  // 1. the histogram slice (one bin a thread) and the first D rounds of
  // scores, then the boundary while the scores are in flight
  const uint32_t n = (uint32_t)z.n, flo = (uint32_t)z.f_lo, fhi = (uint32_t)z.f_hi;
  const int rounds = (int)((n + RK - 1) / RK);
  const bool by_score = k > 0;
  const HistSlice<NT> hs = load_hist_slice<NT>(hist + (int64_t)bg * kHistBins);
  const uint32_t* srow = reinterpret_cast<const uint32_t*>(scores) + (int64_t)bg * sstride;
  const uint32_t last = (uint32_t)sstride - 4u;
  const uint32_t lkey = (uint32_t)wave * 256u + 4u * (uint32_t)lane;  // this lane's first key in a round
  auto load = [&](int r) {
    uint32_t key = (uint32_t)r * RK + lkey;
    if (key > last) key = last;  // past the row: re-read its end (masked below)
    return *reinterpret_cast<const uint4*>(srow + key);
  };
  uint4 ring[D];
#pragma unroll
  for (int d = 0; d < D; ++d) ring[d] = load(d);
  if (tid == 0) ccount = 0u;
  Boundary bd{0u, 0u};
  if (by_score) bd = boundary_of<NT>(hs, (uint32_t)k, wsum, &shb);  // uniform; has barriers
  else __syncthreads();  // ccount
  // candidates: lo <= bits <= hi; selected outright: bits > hi.  Without a
  // top-k part (k = 0) nothing is above and nothing is a candidate.
  const uint32_t lo = by_score ? bd.d1 << kHistShift : 0xFFFFFFFFu;
  const uint32_t hi = by_score ? (bd.d1 < (uint32_t)(kHistBins - 1)
                                      ? ((bd.d1 + 1) << kHistShift) - 1u : 0xFFFFFFFFu)
                               : 0xFFFFFFFFu;

  // Ballots of round r: sel[e] (selected outright) and cnd[e] (candidates),
  // bit i = key r*RK + 256*wave + 4i + e; c[e]: this lane's key e is one.
  auto classify = [&](const uint4& v, int r, uint64_t (&sel)[4], uint64_t (&cnd)[4],
                      bool (&c)[4]) {
    const uint32_t sb[4] = {v.x, v.y, v.z, v.w};
    const uint32_t kb = (uint32_t)r * RK + (uint32_t)wave * 256u;  // the wave's block
    if (kb >= flo && kb + 256u <= fhi) {  // uniform: every key valid, none forced
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool above = sb[e] > hi;
        c[e] = by_score && !above && sb[e] >= lo;
        sel[e] = __ballot(above);
        cnd[e] = __ballot(c[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = kb + 4u * (uint32_t)lane + (uint32_t)e;
        const bool valid = key < n;
        const bool forced = key < flo || key >= fhi;
        const bool above = sb[e] > hi;
        c[e] = valid && !forced && by_score && !above && sb[e] >= lo;
        sel[e] = __ballot(valid && (forced || above));
        cnd[e] = __ballot(c[e]);
      }
    }
  };
  // This wave's candidates of round r from position base on: LDS slots below
  // CAP (dst == nullptr), or the global list (dst).
  auto place = [&](auto to_global, const uint4& v, int r, const uint64_t (&cnd)[4],
                   const bool (&c)[4], uint32_t base, uint2* dst) {
    const uint32_t sb[4] = {v.x, v.y, v.z, v.w};
    const uint32_t key0 = (uint32_t)r * RK + lkey;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (cnd[e]) {  // uniform
        const uint32_t pos = base + __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(cnd[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)cnd[e], 0u));
        if (c[e]) {
          const uint2 ent = make_uint2(sb[e], key0 + (uint32_t)e);
          if constexpr (decltype(to_global)::value) dst[pos] = ent;
          else lc[pos] = ent;
        }
        base += (uint32_t)__popcll(cnd[e]);
      }
    }
  };

  // 2. the streaming pass.  Whole blocks of D rounds run unconditionally, each
  // round refilling its ring slot, once used, with the round D ahead (clamped
  // loads), so no branch sits between a load and its use and every slot is
  // reloaded in place; the last rounds, already in the ring, are then
  // processed without further loads.
  auto process = [&](const uint4& v, int r) {
    uint64_t sel[4], cnd[4];
    bool c[4];
    classify(v, r, sel, cnd, c);
    const uint32_t j = (uint32_t)r * NW + (uint32_t)wave;  // 256-key block
    if (lane == 0) {
      uint4* dst = reinterpret_cast<uint4*>(bm + j * 8);
      dst[0] = make_uint4((uint32_t)sel[0], (uint32_t)(sel[0] >> 32), (uint32_t)sel[1],
                          (uint32_t)(sel[1] >> 32));
      dst[1] = make_uint4((uint32_t)sel[2], (uint32_t)(sel[2] >> 32), (uint32_t)sel[3],
                          (uint32_t)(sel[3] >> 32));
    }
    const uint32_t cnt =
        (uint32_t)(__popcll(cnd[0]) + __popcll(cnd[1]) + __popcll(cnd[2]) + __popcll(cnd[3]));
    if (cnt) {  // uniform per wave
      uint32_t base = 0u;
      if (lane == 0) base = atomicAdd(&ccount, cnt);
      base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
      // past the LDS list: counted only (the overflow pass rewrites them all)
      if (base + cnt <= (uint32_t)CAP) place(std::false_type{}, v, r, cnd, c, base, nullptr);
    }
  };
  int r0 = 0;
  for (; r0 + D <= rounds; r0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      process(ring[d], r0 + d);
      ring[d] = load(r0 + d + D);
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (r0 + d < rounds) process(ring[d], r0 + d);  // uniform
  __syncthreads();
  const uint32_t C = ccount;
  const uint32_t need = by_score ? (uint32_t)k - bd.above : 0u;  // 1 <= need <= C when k > 0

  // 3. the candidates that complete the top-k join the bitmap
  auto mark = [&](const uint2* cl, uint32_t i0, uint32_t step, uint32_t vval, uint32_t imax) {
    for (uint32_t i = i0; i < C; i += step) {
      const uint2 e = cl[i];
      const uint32_t v = e.x & 0x1FFFFFu;
      if (v > vval || (v == vval && e.y <= imax)) {
        const uint32_t t = e.y & 255u, ln = t >> 2;
        atomicOr(&bm[(e.y >> 8) * 8 + (t & 3u) * 2 + (ln >> 5)], 1u << (ln & 31));
      }
    }
  };
  if (C <= (uint32_t)CAP) {  // uniform
    uint32_t vval = 0u, imax = 0xFFFFFFFFu;
    if (by_score && need < C) settle_candidates<NT>(lc, C, need, n, h128, &shpick, vval, imax);
    mark(lc, (uint32_t)tid, (uint32_t)NT, vval, imax);
  } else {  // all candidates to the global list (a second pass), settled by the workgroup
    uint2* gc = cand + (int64_t)bg * n_cap;
    __syncthreads();  // every thread has read ccount
    if (tid == 0) ccount = 0u;
    __syncthreads();
    for (int r = 0; r < rounds; ++r) {
      const uint4 v = load(r);
      uint64_t sel[4], cnd[4];
      bool c[4];
      classify(v, r, sel, cnd, c);
      const uint32_t cnt = (uint32_t)(__popcll(cnd[0]) + __popcll(cnd[1]) + __popcll(cnd[2]) +
                                      __popcll(cnd[3]));
      if (cnt) {
        uint32_t base = 0u;
        if (lane == 0) base = atomicAdd(&ccount, cnt);
        base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
        place(std::true_type{}, v, r, cnd, c, base, gc);
      }
    }
    __syncthreads();  // the list is complete and visible to the workgroup
    uint32_t vval = 0u, imax = 0xFFFFFFFFu;
    if (by_score && need < C) settle_candidates<NT>(gc, C, need, n, h128, &shpick, vval, imax);
    mark(gc, (uint32_t)tid, (uint32_t)NT, vval, imax);
  }
  __syncthreads();

  // 4. ascending indices: segments of NT*SW key-order words (SW consecutive
  // words a thread), each rebuilt from the 8-bit slices of its block's four
  // ballots
  constexpr int SW = 4;
  const uint32_t nwords = (n + 31) >> 5;
  uint32_t written = 0u;
  for (uint32_t w0 = 0; w0 < nwords; w0 += NT * SW) {
    uint32_t kw[SW], cnt = 0u;
#pragma unroll
    for (int q = 0; q < SW; ++q) {
      const uint32_t wi = w0 + (uint32_t)tid * SW + q;
      uint32_t x = 0u;
      if (wi < nwords) {
        const uint32_t blk = wi >> 3, sub = wi & 7;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t b8 = (bm[blk * 8 + 2 * e + (sub >> 2)] >> ((sub & 3) * 8)) & 255u;
          x |= spread4(b8) << e;  // key 4i + e of the word at bit 4i + e
        }
      }
      kw[q] = x;
      cnt += (uint32_t)__popc(x);
    }
    const uint32_t inc = block_incl_scan<NT>(cnt, wsum);
    uint32_t pos = written + inc - cnt;
#pragma unroll
    for (int q = 0; q < SW; ++q) {
      uint32_t x = kw[q];
      const uint32_t kbase = (w0 + (uint32_t)tid * SW + q) * 32u;
      while (x) {
        const int bit = __ffs(x) - 1;
        x &= x - 1;
        if (pos < (uint32_t)k_max) {
          out[pos] = (int32_t)(kbase + bit);
          if (ATT) lsel[pos] = (int32_t)(kbase + bit);
        }
        ++pos;
      }
    }
    if (tid == NT - 1) seg_total = inc;
    lds_barrier();  // the index stores stay in flight
    written += seg_total;
    lds_barrier();
  }
  for (int64_t t = z.total + tid; t < k_max; t += NT) out[t] = -1;
  if constexpr (ATT) {
    const int g = bg % Hq, h = g / (Hq / at.Hkv);
    const int64_t kv = ((int64_t)b * at.Hkv + h) * n_cap * kHead;
    const int S = (int)(z.total < k_max ? z.total : k_max);
    attend_selected<T, NT, 4>(at.q + (int64_t)bg * kHead, at.K + kv, at.V + kv, lsel, S,
                              at.scale, reinterpret_cast<float*>(bm), mml,
                              at.out + (int64_t)bg * kHead);
  }
}

// ---------------------------------------------------------------- selection + attention by key range

// The decode step's selection and attention when its query heads do not
// outnumber the CUs: after the scan, one workgroup per (query head, key range) settles
// the head's boundary-bin candidates itself (each range's workgroup repeats
// the same radix select, which reads a few hundred candidates), lists the
// selected keys of its range in ascending order, writes them at their place
// in the head's index row, and runs split-k attention over them (SOCKET
// Sec. 4.1, Algorithm 3, exact attention over the retrieved subset).  The
// partials (o, m, l) go to the split-k merge, one split per range.  This
// takes the place of the per-head resolve and of the split-k partial launch.
// A range is RB whole 256-key bitmap blocks (at least 8, at most
// kRangeBlocksMax).  Rows of up to kShortRowBlocks blocks (64K keys) take
// about 8 ranges of 512-thread workgroups, longer rows about 16 ranges of
// 256-thread workgroups: in alternating runs these beat 12, 16 and 32 ranges
// of 256 threads at 32K keys, and 8 ranges of 512 threads at 128K.
constexpr int kRangeBlocksMax = 31;
constexpr int kShortRowBlocks = 256;
constexpr int kSelAttCandCap = 2048;  // candidates settled in LDS (more: read in place)

int range_blocks(int64_t n_cap) {
  const int64_t nb = (n_cap + 255) / 256;
  const bool short_row = nb <= kShortRowBlocks;
  int64_t rb = short_row ? (nb + 7) / 8 : (nb + 15) / 16;
  if (rb < 8) rb = 8;
  const int64_t cap = short_row ? kRangeBlocksMax : 24;  // 24: measured best for long rows
  if (rb > cap) rb = cap;
  return (int)rb;
}

int range_splits(int64_t n_cap) {
  const int64_t nb = (n_cap + 255) / 256;
  const int rb = range_blocks(n_cap);
  return (int)((nb + rb - 1) / rb);
}

// Attention of one query over the S keys key0 + sel[t] (t < S, ascending) by
// the NT threads of a workgroup, written as an unnormalised split-k partial
// pp = (o, m, l) with m the largest logit, l = sum exp(logit - m) and
// o = sum exp(logit - m) v.  16 lanes share a key row; the R = NT/16 rows take
// keys t = row, row + R, ... in batches of AB (every K and V load of a batch
// issued before any is used) with an online softmax, then merge in row order.
// No key: o = 0, m = -inf, l = 0 (a split the merge skips).
template <typename T, int NT, int AB>
__device__ __forceinline__ void attend_partial(const T* __restrict__ qrow,
                                               const T* __restrict__ Kh,
                                               const T* __restrict__ Vh, const uint16_t* sel,
                                               int64_t key0, int S, float scale, float* mo,
                                               float* mml, float* __restrict__ pp) {
  constexpr int R = NT / 16;
  const int tid = threadIdx.x, j = tid & 15, row = tid >> 4;
  float qf[8];
  load_row8<T>(qrow, j, qf);
  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  for (int t0 = row; t0 < S; t0 += R * AB) {  // the 16 lanes of a row agree
    int64_t ki[AB];
    bool live[AB];
#pragma unroll
    for (int a = 0; a < AB; ++a) {
      const int t = t0 + a * R;
      live[a] = t < S;
      ki[a] = key0 + (live[a] ? (int64_t)sel[t] : 0);
    }
    Row8<T> kr[AB], vr[AB];
#pragma unroll
    for (int a = 0; a < AB; ++a) {
      kr[a] = fetch_row8<T>(Kh + ki[a] * kHead, j);
      vr[a] = fetch_row8<T>(Vh + ki[a] * kHead, j);
    }
    float lg[AB], mx = m;
#pragma unroll
    for (int a = 0; a < AB; ++a) {
      float kf[8];
      unpack_row8<T>(kr[a], kf);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = fmaf(qf[e], kf[e], dot);
      dot = row16_sum(dot);
      lg[a] = live[a] ? dot * scale : -INFINITY;
      mx = fmaxf(mx, lg[a]);
    }
    // t0 < S, so the batch's first key is a real one and mx is finite
    const float c = m == -INFINITY ? 0.f : __expf(m - mx);
    l *= c;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= c;
#pragma unroll
    for (int a = 0; a < AB; ++a) {
      const float p = lg[a] == -INFINITY ? 0.f : __expf(lg[a] - mx);
      float vf[8];
      unpack_row8<T>(vr[a], vf);
      l += p;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(p, vf[e], o[e]);
    }
    m = mx;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) mo[row * kHead + 8 * j + e] = o[e];
  if (j == 0) {
    mml[2 * row] = m;
    mml[2 * row + 1] = l;
  }
  __syncthreads();
  if (tid < kHead) {
    float M = -INFINITY;
    for (int r = 0; r < R; ++r)
      if (mml[2 * r + 1] > 0.f) M = fmaxf(M, mml[2 * r]);
    float L = 0.f, O = 0.f;
    for (int r = 0; r < R; ++r) {
      const float lr = mml[2 * r + 1];
      const float w = lr > 0.f ? __expf(mml[2 * r] - M) : 0.f;
      L = fmaf(lr, w, L);
      O = fmaf(mo[r * kHead + tid], w, O);
    }
    pp[tid] = O;
    if (tid == 0) {
      pp[kHead] = M;
      pp[kHead + 1] = L;
    }
  }
}

// grid: B*Hq*S blocks of NT threads (rounded up to a multiple of kXcds);
// logical block bg*S + s takes bitmap blocks [s*RB, (s+1)*RB) of head bg.
template <int NT, typename T>
__global__ __launch_bounds__(NT) void select_attend_kernel(
    int64_t n_cap, const int32_t* __restrict__ lens, const int32_t* __restrict__ ks, int k_max,
    int sink, int window, int Hq, int heads, int S, int RB, const uint32_t* __restrict__ hist,
    const uint32_t* __restrict__ counters, const uint32_t* __restrict__ bitmap, int64_t words,
    const uint2* __restrict__ cand, int32_t* __restrict__ idx, AttendArgs<T> at,
    float* __restrict__ part) {
  constexpr int NW = NT / 64;
  constexpr int CPT = 1024 / NT;  // candidates a thread requests with the first loads
  static_assert(kSelAttCandCap >= CPT * NT, "the first loads fit the LDS list");
  static_assert(kRangeBlocksMax * 8 <= NT, "one key-order word of the range a thread");
  // logical block (blockIdx mod 8) * (grid / 8) + blockIdx / 8, remapped as
  // in the scan, so a head's ranges run on the XCD that scanned it
  const int lid = (int)(blockIdx.x % kXcds) * (int)(gridDim.x / kXcds) + (int)(blockIdx.x / kXcds);
  const int bg = lid / S, s = lid % S;
  if (bg >= heads) return;
  const int b = bg / Hq;
  const int tid = threadIdx.x;
  const SelSizes z = sel_sizes(n_cap, lens[b], ks[b], k_max, sink, window);
  const int64_t n = z.n, k = z.k;
  int32_t* out = idx + (int64_t)bg * k_max;
  float* pp = part + ((int64_t)bg * S + s) * kPartStride;
  if (s == 0)
    for (int64_t t = z.total + tid; t < k_max; t += NT) out[t] = -1;
  const int64_t nblocks = (n + 255) >> 8;
  const int64_t blk0 = (int64_t)s * RB;
  const int64_t blk1 = blk0 + RB < nblocks ? blk0 + RB : nblocks;
  if (z.total == 0 || blk0 >= nblocks) {  // uniform: an empty split
    if (tid < kHead) pp[tid] = 0.f;
    if (tid == 0) {
      pp[kHead] = -INFINITY;
      pp[kHead + 1] = 0.f;
    }
    return;
  }

  __shared__ uint32_t wsum[NW];
  __shared__ Boundary shb;
  __shared__ uint32_t h128[128];
  __shared__ Pick shpick;
  __shared__ uint32_t lbm[kRangeBlocksMax * 8];
  __shared__ uint16_t lsel[kRangeBlocksMax * 256];
  __shared__ float mml[2 * (NT / 16)];
  __shared__ uint2 lcand[kSelAttCandCap];  // later the attention's row partials
  static_assert(kSelAttCandCap * 2 >= (NT / 16) * kHead, "the candidate LDS holds the merge");

  // every independent load at once: the histogram slice, the candidate
  // count, the first CPT*NT candidates, the range's bitmap words and the
  // bitmap before the range (for the number of selected keys ahead of it)
  const HistSlice<NT> hs = load_hist_slice<NT>(hist + (int64_t)bg * kHistBins);
  const uint2* gc = cand + (int64_t)bg * n_cap;
  const uint32_t* bm = bitmap + (int64_t)bg * words;
  const uint32_t Cg = counters[bg];
  uint2 cv[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int64_t ci = (int64_t)tid + i * NT;
    cv[i] = gc[ci < n_cap ? ci : n_cap - 1];
  }
  const int nw = (int)(blk1 - blk0) * 8;  // words of the range
  const uint32_t rw = bm[blk0 * 8 + (tid < nw ? tid : 0)];
  const uint4* bm4 = reinterpret_cast<const uint4*>(bm);
  const int64_t nv = blk0 * 2;  // 16-byte vectors before the range
  uint32_t pre = 0u;
  for (int64_t v0 = 0; v0 < nv; v0 += 4 * NT) {
    uint4 w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t vi = v0 + tid + i * NT;
      w4[i] = bm4[vi < nv ? vi : 0];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (v0 + tid + i * NT < nv)
        pre += __popc(w4[i].x) + __popc(w4[i].y) + __popc(w4[i].z) + __popc(w4[i].w);
  }
  const Boundary bd = boundary_of<NT>(hs, (uint32_t)k, wsum, &shb);
  const uint32_t C = Cg < (uint32_t)n ? Cg : (uint32_t)n;
  const bool in_lds = C <= (uint32_t)kSelAttCandCap;
  if (in_lds) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      if ((uint32_t)(tid + i * NT) < C) lcand[tid + i * NT] = cv[i];
    for (uint32_t ci = (uint32_t)(CPT * NT + tid); ci < C; ci += NT) lcand[ci] = gc[ci];
  }
  if (tid < nw) lbm[tid] = rw;
  __syncthreads();
  const uint2* lc = in_lds ? lcand : gc;

  // the candidates that complete the top-k: a candidate is chosen iff its
  // low 21 score bits exceed vval, or equal it with key <= imax
  uint32_t vval = 0u, imax = 0xFFFFFFFFu;
  const uint32_t need = (uint32_t)k - bd.above;  // 1 <= need <= C when k > 0
  if (k > 0 && need < C) settle_candidates<NT>(lc, C, need, (uint32_t)n, h128, &shpick, vval, imax);

  // chosen candidates: counted when ahead of the range, marked when in it
  const uint32_t r0 = (uint32_t)(blk0 * 256), r1 = (uint32_t)(blk1 * 256);
  for (uint32_t i = tid; i < C; i += NT) {
    const uint2 e = lc[i];
    const uint32_t v = e.x & 0x1FFFFFu;
    if (v > vval || (v == vval && e.y <= imax)) {
      if (e.y < r0) {
        ++pre;
      } else if (e.y < r1) {
        const uint32_t blk = (e.y - r0) >> 8, i4 = (e.y >> 2) & 63u, ee = e.y & 3u;
        atomicOr(&lbm[blk * 8 + ee * 2 + (i4 >> 5)], 1u << (i4 & 31));
      }
    }
  }
  __syncthreads();
  // key-order word t of the range (keys r0 + 32t .. +31), rebuilt from the
  // 8-bit slices of its block's four ballot masks
  uint32_t x = 0u;
  if (tid < nw) {
    const int blk = tid >> 3, sub = tid & 7;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t b8 = (lbm[blk * 8 + 2 * e + (sub >> 2)] >> ((sub & 3) * 8)) & 255u;
      x |= spread4(b8) << e;
    }
  }
  const uint32_t cnt = (uint32_t)__popc(x);
  // one scan gives both the selected keys ahead of the range (the sum of
  // pre, at most k_max <= 2^16) and this word's place in the range (a range
  // holds at most kRangeBlocksMax*256 < 2^13 keys): pre above bit 13
  static_assert(kRangeBlocksMax * 256 < (1 << 13), "range counts fit 13 bits");
  const uint32_t inc = block_incl_scan<NT>((pre << 13) | cnt, wsum);
  __shared__ uint32_t sh_all;
  if (tid == NT - 1) sh_all = inc;
  lds_barrier();
  const uint32_t all = sh_all;
  const uint32_t ahead = all >> 13;          // selected keys before the range
  const uint32_t S_cnt = all & 0x1FFFu;      // selected keys in the range
  uint32_t p = (inc & 0x1FFFu) - cnt;
  while (x) {
    const int bit = __ffs(x) - 1;
    x &= x - 1;
    const uint32_t off = (uint32_t)tid * 32u + (uint32_t)bit;
    lsel[p] = (uint16_t)off;
    const uint32_t gp = ahead + p;
    if (gp < (uint32_t)k_max) out[gp] = (int32_t)(r0 + off);
    ++p;
  }
  __syncthreads();
  const int g = bg % Hq, h = g / (Hq / at.Hkv);
  const int64_t kv = ((int64_t)b * at.Hkv + h) * n_cap * kHead;
  attend_partial<T, NT, 4>(at.q + (int64_t)bg * kHead, at.K + kv, at.V + kv, lsel, (int64_t)r0,
                           (int)S_cnt, at.scale, reinterpret_cast<float*>(lcand), mml, pp);
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
static void launch_scorer(int B, int Hkv, int sub, int Hq, int P, int64_t n_cap, SinkWindow sw,
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
      ws.img, ws.img_floats, ids, vnorm, lens, Hq, Hkv, sub, P, n_cap, sw.sink, sw.window,
      (int)rows, (int)nblk, (int)gpb, scores, ws.hist, usum, usum ? ws.gsum : nullptr);
}

template <int G>
static void launch_scorer_g(int B, int Hkv, int sub, int Hq, int L, int P, int64_t n_cap,
                            SinkWindow sw, float* usum,
                            const ScoreWs& ws, const uint8_t* ids, const float* vnorm,
                            const int32_t* lens, float* scores, hipStream_t s) {
  if (P > 8) {  // two-byte IDs, L <= 64
    switch (ids_tables_per_word(L)) {
      case 1: launch_scorer<G, 1, true>(B, Hkv, sub, Hq, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
      case 2: launch_scorer<G, 2, true>(B, Hkv, sub, Hq, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
      default: launch_scorer<G, 4, true>(B, Hkv, sub, Hq, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
    }
    return;
  }
  switch (ids_tables_per_word(L)) {
    case 1: launch_scorer<G, 1, false>(B, Hkv, sub, Hq, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
    case 2: launch_scorer<G, 2, false>(B, Hkv, sub, Hq, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
    case 4: launch_scorer<G, 4, false>(B, Hkv, sub, Hq, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
    default: launch_scorer<G, 8, false>(B, Hkv, sub, Hq, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
  }
}

hipError_t launch_soft_tables(const void* q, int dtype, int B, int Hq, int Hkv, const void* W,
                              int L, int P, float tau, const ScoreWs& ws, hipStream_t s,
                              AppendKey ak) {
  const int G = Hq / Hkv, GK = pass_heads(G), sub = pass_subs(G);
  const ImageDims im = image_dims(GK, L, P);
  const int rows = B * Hkv * sub;  // table blocks: 16 per sub-row
  const int TLw = ids_tables_per_word(L);
  const int nab = ak.K ? (16 + kTabThreads / (TLw * P) - 1) / (kTabThreads / (TLw * P)) : 0;
  const unsigned grid = (unsigned)(rows * 16 + B * Hkv * nab);
  const bool two = im.TL * P > kTabThreads / 8;  // W rows past one round of eight threads each
  auto go = [&](auto tag, auto gtag) {
    using T = decltype(tag);
    constexpr int GG = decltype(gtag)::value;
    if (two)
      soft_tables_kernel<T, GG, true><<<grid, kTabThreads, 0, s>>>(
          static_cast<const T*>(q), static_cast<const T*>(W), Hq, Hkv, L, P, tau, im.TL, im.NF,
          im.NS, im.HE, im.full, ws.img_floats, ws.img, ws.hist, ws.counters, ws.usum, ak, rows,
          nab, sub);
    else
      soft_tables_kernel<T, GG, false><<<grid, kTabThreads, 0, s>>>(
          static_cast<const T*>(q), static_cast<const T*>(W), Hq, Hkv, L, P, tau, im.TL, im.NF,
          im.NS, im.HE, im.full, ws.img_floats, ws.img, ws.hist, ws.counters, ws.usum, ak, rows,
          nab, sub);
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
  return hipGetLastError();
}

hipError_t launch_score(int B, int Hq, int Hkv, int L, int P, const uint8_t* ids,
                        const float* vnorm, const int32_t* lens, int64_t n_cap, SinkWindow sw,
                        float* scores, bool soft_sums,
                        const ScoreWs& ws, hipStream_t s) {
  float* usum = soft_sums ? ws.usum : nullptr;
  const int G = Hq / Hkv, sub = pass_subs(G);
  const int Hv = Hkv * sub;  // sub-rows per sequence
  switch (pass_heads(G)) {
    case 1: launch_scorer_g<1>(B, Hv, sub, Hq, L, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
    case 2: launch_scorer_g<2>(B, Hv, sub, Hq, L, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
    default: launch_scorer_g<4>(B, Hv, sub, Hq, L, P, n_cap, sw, usum, ws, ids, vnorm, lens, scores, s); break;
  }
  return hipGetLastError();
}

// Rows of up to kStreamKeys keys take the streaming top-k (one workgroup per
// head); longer rows spread the classification over many scan workgroups per
// head before one resolve workgroup per head (a single workgroup's compare
// and ballot work grows with the row: at 128K keys it cost 29 us against
// 18 us for scan + resolve).
constexpr int64_t kStreamKeys = 40960;

hipError_t launch_topk(int B, int Hq, const float* scores, const int32_t* lens, int64_t n_cap,
                       const int32_t* ks, int k_max, SinkWindow sw, int32_t* idx, const ScoreWs& ws,
                       hipStream_t s, const AttendSpec* att, bool* attended, float* part,
                       int part_splits) {
  if (attended) *attended = false;
  const int64_t heads = (int64_t)B * Hq;
  const bool many = heads > device_cus();
  const int64_t sst = score_stride(n_cap);
  // the attention arguments of the fused kernels, in K's element type
  auto with_att = [&](auto tag, auto&& go) {
    using T = decltype(tag);
    AttendArgs<T> a{static_cast<const T*>(att->q), static_cast<const T*>(att->K),
                    static_cast<const T*>(att->V), att->out, att->Hkv, att->scale};
    go(a);
  };
  const AttendArgs<uint16_t> none{};
  // the scan: bitmap of the keys above the boundary bin, candidates of that bin
  auto scan = [&]() {
    const int CH = (int)((n_cap + kScanKeys - 1) / kScanKeys);
    const int64_t nscan = heads * CH;
    const unsigned sgrid = (unsigned)((nscan + kXcds - 1) / kXcds * kXcds);
    // two kScanThreads workgroups fit a CU; beyond that, the small ones
    if (nscan <= 2 * (int64_t)device_cus())
      topk_scan_kernel<kScanThreads, kScanKeys / (kScanThreads / 64)><<<sgrid, kScanThreads, 0, s>>>(
          scores, n_cap, sst, lens, ks, k_max, sw.sink, sw.window, Hq, CH, (int)heads,
          ws.hist, ws.counters, ws.bitmap, ws.words, ws.cand);
    else
      topk_scan_kernel<256, 256><<<sgrid, 256, 0, s>>>(
          scores, n_cap, sst, lens, ks, k_max, sw.sink, sw.window, Hq, CH, (int)heads,
          ws.hist, ws.counters, ws.bitmap, ws.words, ws.cand);
    return hipGetLastError();
  };
  // A decode step whose heads do not outnumber the CUs: the scan, then the
  // selection and attention by key range (many workgroups a head instead of
  // one CU selecting a head), then the split-k merge of the ranges.
  const int S = range_splits(n_cap);
  if (att && !many && part && S <= part_splits) {
    hipError_t e = scan();
    if (e != hipSuccess) return e;
    const int RB = range_blocks(n_cap);
    const bool short_row = (n_cap + 255) / 256 <= kShortRowBlocks;
    auto go = [&](auto a) {
      using T = typename std::remove_const<typename std::remove_pointer<decltype(a.q)>::type>::type;
      const unsigned grid = (unsigned)((heads * S + kXcds - 1) / kXcds * kXcds);
      if (short_row)
        select_attend_kernel<512, T><<<grid, 512, 0, s>>>(
            n_cap, lens, ks, k_max, sw.sink, sw.window, Hq, (int)heads, S, RB, ws.hist, ws.counters,
            ws.bitmap, ws.words, ws.cand, idx, a, part);
      else
        select_attend_kernel<256, T><<<grid, 256, 0, s>>>(
            n_cap, lens, ks, k_max, sw.sink, sw.window, Hq, (int)heads, S, RB, ws.hist, ws.counters,
            ws.bitmap, ws.words, ws.cand, idx, a, part);
    };
    if (att->dtype == 1) with_att(uint16_t{}, go);
    else with_att(float{}, go);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (attended) *attended = true;
    return launch_decode_combine(part, (int)heads, S, att->out, s);
  }
  if (n_cap <= kStreamKeys) {
    // 512-thread form (33 KiB of LDS, several a CU) for batches with more
    // heads than CUs, else the 1024-thread form (one a CU)
    const unsigned hgrid = (unsigned)((heads + kXcds - 1) / kXcds * kXcds);
    constexpr int kSmallCap = 2048, kBigCap = 8192;
    // Attending in the selecting workgroup (one CU per head) pays only when
    // there are more heads than CUs: with 32 heads one CU gathering a head's
    // 656 K and V rows took ~15 us, against ~10 us for the split-k kernels.
    const bool fuse = att && many && k_max <= 2 * kSmallCap;
    auto run = [&](auto ntag, auto atag, auto a) {
      constexpr int NT = decltype(ntag)::value;
      constexpr bool ATT = decltype(atag)::value;
      using T = typename std::remove_pointer<decltype(a.q)>::type;
      using TT = typename std::remove_const<T>::type;
      if constexpr (NT == 512)
        topk_stream_kernel<512, 4096, kSmallCap, 8, ATT, TT><<<hgrid, 512, 0, s>>>(
            scores, n_cap, sst, lens, ks, k_max, sw.sink, sw.window, Hq, (int)heads, ws.hist,
            ws.cand, idx, a);
      else
        topk_stream_kernel<1024, 16384, kBigCap, 8, ATT, TT><<<hgrid, 1024, 0, s>>>(
            scores, n_cap, sst, lens, ks, k_max, sw.sink, sw.window, Hq, (int)heads, ws.hist,
            ws.cand, idx, a);
    };
    using N5 = std::integral_constant<int, 512>;
    using N10 = std::integral_constant<int, 1024>;
    if (fuse) {
      auto go = [&](auto a) {
        if (many) run(N5{}, std::true_type{}, a);
        else run(N10{}, std::true_type{}, a);
      };
      if (att->dtype == 1) with_att(uint16_t{}, go);
      else with_att(float{}, go);
      if (attended) *attended = true;
    } else if (many) {
      run(N5{}, std::false_type{}, none);
    } else {
      run(N10{}, std::false_type{}, none);
    }
    return hipGetLastError();
  }
  hipError_t e = scan();
  if (e != hipSuccess) return e;
  const int rnt = many ? 512 : kResThreads;
  const bool fuse = att && many && (n_cap + 255) / 256 <= rnt && k_max <= 2 * kCandCap;
  auto run = [&](auto ntag, auto atag, auto a) {
    constexpr int NT = decltype(ntag)::value;
    constexpr bool ATT = decltype(atag)::value;
    using T = typename std::remove_const<typename std::remove_pointer<decltype(a.q)>::type>::type;
    topk_resolve_kernel<NT, ATT, T><<<(unsigned)heads, NT, 0, s>>>(
        n_cap, lens, ks, k_max, sw.sink, sw.window, Hq, ws.hist, ws.counters, ws.bitmap, ws.words,
        ws.cand, idx, a);
  };
  using R5 = std::integral_constant<int, 512>;
  using R10 = std::integral_constant<int, kResThreads>;
  if (fuse) {
    auto go = [&](auto a) {
      if (many) run(R5{}, std::true_type{}, a);
      else run(R10{}, std::true_type{}, a);
    };
    if (att->dtype == 1) with_att(uint16_t{}, go);
    else with_att(float{}, go);
    if (attended) *attended = true;
  } else if (many) {
    run(R5{}, std::false_type{}, none);
  } else {
    run(R10{}, std::false_type{}, none);
  }
  return hipGetLastError();
}

}  // namespace socketlsh
