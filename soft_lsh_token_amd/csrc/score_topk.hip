// Query soft hashing, soft-count scoring and top-k selection
// (SOCKET Sec. 4.1, Algorithms 2 and 3).
//
// Soft hashing: table l gives bucket c the probability
//   p_l(c) = softmax_c( sum_j s_j(c) u_lj / tau ),  s_j(c) = +1 if bit j of c else -1,
// which factorises over the planes as prod_j sigmoid(2 s_j(c) u_lj / tau).
// Every table is therefore split into a low half (planes 0..3) and a high
// half (planes 4..P-1) of at most 16 entries each; the scorer rebuilds
// p_l(c) = lo_l(c & 15) * hi_l(c >> 4) in LDS.  The projections u = W q are
// taken in float64.
//
// Scorer (one pass per KV head for all of its GQA query heads): lane j of a
// 16-lane row owns TL consecutive tables (j*TL .. j*TL+TL-1), so it reads one
// TL-byte word of bucket IDs per key.  The tables of the G query heads are
// interleaved in LDS as
//   slot(c, m, j) = (c * MC + m) * 16 + j,   one slot = G floats,
// for member m of the MC tables per lane held in LDS at a time.  A row works
// on one key at a time, so its 16 lookups fall into 16 different 16-byte
// bank groups whatever the bucket IDs are (gfx950 serves 16 lanes of a
// ds_read_b128 per cycle).  Per-lane partial sums are reduced across the row
// with DPP.  When the tables of the G heads do not fit in 128 KiB at once
// (G = 4: 64 tables x 256 entries x 16 B = 256 KiB) they are rebuilt in
// chunks; the IDs and value norms of all the workgroup's keys are loaded
// into registers before the first chunk, so their HBM latency hides behind
// the table build and no ID byte is read twice.
//
// Top-k: the scorer also builds, per query head, a histogram of the top
// digit of the float32 score bits (scores are non-negative, so their bit
// patterns order like the values).  The scan kernel finds the bin holding
// the k-th largest score, marks every key above it in a bitmap and collects
// the keys of that bin as candidates; the resolve kernel settles the
// candidates exactly (radix select on the remaining score bits, then on the
// index so that the lower index wins a tie) and turns the bitmap into
// ascending indices.
#include "common.h"
#include "launch.h"

namespace socketlsh {

// ---------------------------------------------------------------- workspace

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t score_ws_layout(int B, int Hq, int64_t n_cap, int L, ScoreWs* ws, void* base) {
  const size_t heads = (size_t)B * Hq;
  const int64_t words = ((n_cap + 63) / 64) * 2;
  size_t off = 0;
  const size_t o_sub = off; off = align256(off + heads * L * 32 * sizeof(float));
  const size_t o_hist = off; off = align256(off + heads * kHistBins * sizeof(uint32_t));
  const size_t o_cnt = off; off = align256(off + heads * 4 * sizeof(uint32_t));
  const size_t o_bm = off; off = align256(off + heads * words * sizeof(uint32_t));
  const size_t o_cand = off; off = align256(off + heads * (size_t)n_cap * sizeof(uint2));
  const size_t o_sc = off; off = align256(off + heads * (size_t)n_cap * sizeof(float));
  if (ws) {
    char* p = static_cast<char*>(base);
    ws->sub = reinterpret_cast<float*>(p + o_sub);
    ws->hist = reinterpret_cast<uint32_t*>(p + o_hist);
    ws->counters = reinterpret_cast<uint32_t*>(p + o_cnt);
    ws->bitmap = reinterpret_cast<uint32_t*>(p + o_bm);
    ws->cand = reinterpret_cast<uint2*>(p + o_cand);
    ws->scores = reinterpret_cast<float*>(p + o_sc);
    ws->words = words;
  }
  return off;
}

// ---------------------------------------------------------------- soft tables

template <typename T>
__device__ __forceinline__ void load_w8(const T* p, float* f);
template <>
__device__ __forceinline__ void load_w8<uint16_t>(const uint16_t* p, float* f) {
  unpack_bf16x8(*reinterpret_cast<const uint4*>(p), f);
}
template <>
__device__ __forceinline__ void load_w8<float>(const float* p, float* f) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// grid: B*Hq blocks, 256 threads.  Also clears the head's histogram and counters.
template <typename T>
__global__ __launch_bounds__(256) void soft_tables_kernel(const T* __restrict__ q,
                                                          const T* __restrict__ W, int L, int P,
                                                          float tau, float* __restrict__ sub,
                                                          uint32_t* __restrict__ hist,
                                                          uint32_t* __restrict__ counters) {
  const int bg = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ double qd[kHead];
  __shared__ double sig[2048][2];  // [plane][bit] = sigmoid(-+2u/tau)
  if (tid < kHead) {
    if constexpr (sizeof(T) == 2)
      qd[tid] = (double)__uint_as_float((uint32_t)q[(int64_t)bg * kHead + tid] << 16);
    else
      qd[tid] = (double)q[(int64_t)bg * kHead + tid];
  }
  for (int i = tid; i < kHistBins; i += blockDim.x) hist[(int64_t)bg * kHistBins + i] = 0u;
  if (tid < 4) counters[bg * 4 + tid] = 0u;
  __syncthreads();
  const int planes = L * P;
  const double inv_tau = 1.0 / (double)tau;
  for (int pl = tid; pl < planes; pl += blockDim.x) {
    const T* wr = W + (int64_t)pl * kHead;
    float wf[kHead];
#pragma unroll
    for (int t = 0; t < kHead; t += 8) load_w8<T>(wr + t, wf + t);
    double u = 0.0;
#pragma unroll
    for (int t = 0; t < kHead; ++t) u = fma((double)wf[t], qd[t], u);
    const double x = 2.0 * u * inv_tau;
    sig[pl][1] = 1.0 / (1.0 + exp(-x));  // bit set: corner sign +1
    sig[pl][0] = 1.0 / (1.0 + exp(x));   // bit clear: corner sign -1
  }
  __syncthreads();
  const int plo = P < 4 ? P : 4;
  const int phi = P - plo;
  for (int e = tid; e < L * 32; e += blockDim.x) {
    const int l = e >> 5, r = e & 31, hf = r >> 4, c = r & 15;
    const int nb = hf ? phi : plo;
    double prod = 0.0;
    if (c < (1 << nb)) {
      prod = 1.0;
      const int p0 = l * P + (hf ? plo : 0);
      for (int j = 0; j < nb; ++j) prod *= sig[p0 + j][(c >> j) & 1];
    }
    sub[((int64_t)bg * L + l) * 32 + r] = (float)prod;
  }
}

// ---------------------------------------------------------------- scorer

template <int G>
__device__ __forceinline__ void lds_add(const float* lds, int slot, float* acc) {
  if constexpr (G == 1) {
    acc[0] += lds[slot];
  } else if constexpr (G == 2) {
    const float2 v = reinterpret_cast<const float2*>(lds)[slot];
    acc[0] += v.x; acc[1] += v.y;
  } else {
    const float4 v = reinterpret_cast<const float4*>(lds)[slot];
    acc[0] += v.x; acc[1] += v.y; acc[2] += v.z; acc[3] += v.w;
  }
}

// One TL-byte word of bucket IDs (TL <= 8) as two dwords.
template <int TL>
__device__ __forceinline__ uint2 load_ids(const uint8_t* p) {
  uint2 w = make_uint2(0u, 0u);
  if constexpr (TL == 1) w.x = p[0];
  else if constexpr (TL == 2) w.x = *reinterpret_cast<const uint16_t*>(p);
  else if constexpr (TL == 4) w.x = *reinterpret_cast<const uint32_t*>(p);
  else w = *reinterpret_cast<const uint2*>(p);
  return w;
}

template <int B8>
__device__ __forceinline__ uint32_t id_byte(uint2 w) {
  return ((B8 < 4 ? w.x : w.y) >> (8 * (B8 & 3))) & 255u;
}

constexpr int kScoreThreads = 512;
constexpr int kScoreWaves = kScoreThreads / 64;
constexpr int kTableFloats = 32768;  // 128 KiB of tables in LDS at a time
// Half-tables of one chunk, one padded row of G*32 + 2 floats per table, so
// that the 32 tables a wave reads from in the table build sit in distinct
// LDS banks; later reused for the histogram (G*1024 <= 4096 words).
constexpr int kStageFloats = 4352;
template <int G>
struct StageRow {
  static constexpr int value = G * 32 + 2;
};

// Compile-time shape of the scorer.  G: query heads per KV head; TL: tables
// (= ID bytes) per lane per key; S: 64-key groups per wave.
template <int G, int TL, int S>
struct ScorerShape {
  static constexpr int MC = (TL < 8 / G) ? TL : 8 / G;  // tables per lane in LDS at a time
  static constexpr int NCH = TL / MC;                    // chunks
};

// Reduce-scatter over a 16-lane row.  On entry lane j holds in u[x] its
// contribution to key (j + x) mod 16 of the row; on exit u[0] of lane j is
// the sum over the 16 lanes for key j.  Stage d adds, for x < d, the value
// lane j - d holds for the same key (its slot x + d); row_ror:d gives lane j
// the register of lane (j - d) mod 16.
template <int G>
__device__ __forceinline__ void row16_reduce_scatter(float (&u)[16][G]) {
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int g = 0; g < G; ++g) u[x][g] += dpp_f32<0x128>(u[x + 8][g]);
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

// grid: B*Hkv*nblk, block = kScoreThreads threads.  Block blk of (b, h) owns
// the 64-key groups [blk*gpb, (blk+1)*gpb) (gpb <= kScoreWaves*S); wave w
// takes groups blk*gpb + w + kScoreWaves*s, s < S.
template <int G, int TL, int S>
__global__ __launch_bounds__(kScoreThreads) void scorer_kernel(
    const float* __restrict__ sub, const uint8_t* __restrict__ ids,
    const float* __restrict__ vnorm, const int32_t* __restrict__ lens, int Hq, int Hkv, int L,
    int P, int64_t n_cap, int nblk, int gpb, float* __restrict__ scores,
    uint32_t* __restrict__ hist) {
  using Sh = ScorerShape<G, TL, S>;
  constexpr int MC = Sh::MC, NCH = Sh::NCH;
  __shared__ __attribute__((aligned(16))) float tab[kTableFloats];
  __shared__ __attribute__((aligned(16))) float stage[kStageFloats];
  const int blk = blockIdx.x % nblk;
  const int bh = blockIdx.x / nblk;
  const int b = bh / Hkv;
  const int h = bh % Hkv;
  int64_t n = lens[b];
  if (n > n_cap) n = n_cap;
  const int64_t g_begin = (int64_t)blk * gpb;
  int64_t g_end = (n + 63) >> 6;
  if (g_end > g_begin + gpb) g_end = g_begin + gpb;
  if (g_begin >= g_end) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, kg = lane >> 4, j = lane & 15;
  const int bg0 = b * Hq + h * G;
  const int plo = P < 4 ? P : 4;
  const int lomask = (1 << plo) - 1;
  const int nent = 1 << P;
  // first key of this wave's group s (groups past g_end hold no keys)
  auto gkey = [&](int s) -> int64_t {
    const int64_t gi = g_begin + wave + (int64_t)kScoreWaves * s;
    return gi < g_end ? gi * 64 : n;
  };

  // Row kg of the wave owns keys kg*16 .. kg*16+15 of each 64-key group; in
  // round x lane j takes its ID word j of key kg*16 + (j + x) mod 16, which the
  // tiled ID layout stores at word slot x*64 + lane of the group, so every
  // load of the wave reads 64 consecutive words.  All bucket IDs, norms and
  // half-tables this lane will need are requested before any table work.
  const uint8_t* idg = ids + (int64_t)bh * ids_groups(n_cap) * 1024 * TL;
  uint2 idw[S][16];
  float vnv[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t k0 = gkey(s);
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      idw[s][x] = make_uint2(0u, 0u);
      if (k0 < n) idw[s][x] = load_ids<TL>(idg + ((k0 >> 6) * 1024 + x * 64 + lane) * TL);
    }
    const int64_t key = k0 + lane;  // the key this lane finishes
    vnv[s] = key < n ? vnorm[(int64_t)bh * n_cap + key] : 0.f;
  }
  constexpr int ROW = StageRow<G>::value;
  constexpr int NSTAGE = 16 * MC * G * 32;             // half-table floats per chunk
  constexpr int SPT = (NSTAGE + kScoreThreads - 1) / kScoreThreads;
  float stv[NCH][SPT];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
#pragma unroll
    for (int q = 0; q < SPT; ++q) {
      const int i = tid + q * kScoreThreads;
      const int r = i & 31, rest = i >> 5;
      const int g = rest % G, m = (rest / G) % MC, jj = rest / (G * MC);
      const int l = jj * TL + c * MC + m;
      stv[c][q] = (i < NSTAGE && l < L) ? sub[((int64_t)(bg0 + g) * L + l) * 32 + r] : 0.f;
    }

  float part[S][G];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int g = 0; g < G; ++g) part[s][g] = 0.f;

#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    __syncthreads();
    // half-tables of this chunk: stage[(jj*MC + m)*ROW + g*32 + r] for table jj*TL + c*MC + m
#pragma unroll
    for (int q = 0; q < SPT; ++q) {
      const int i = tid + q * kScoreThreads;
      if (i < NSTAGE) {
        const int r = i & 31, rest = i >> 5;
        const int g = rest % G, t = rest / G;
        stage[t * ROW + g * 32 + r] = stv[c][q];
      }
    }
    __syncthreads();
    // full tables: slot (e*MC + m)*16 + jj holds p_l(e) of the G heads
    const int nslots = nent * MC * 16;
    for (int slot = tid; slot < nslots; slot += kScoreThreads) {
      const int jj = slot & 15;
      const int m = (slot >> 4) % MC;
      const int e = slot / (16 * MC);
      const float* st = stage + (jj * MC + m) * ROW;
      float v[G];
#pragma unroll
      for (int g = 0; g < G; ++g) v[g] = st[g * 32 + (e & lomask)] * st[g * 32 + 16 + (e >> plo)];
      if constexpr (G == 4) {
        reinterpret_cast<float4*>(tab)[slot] = make_float4(v[0], v[1], v[2], v[3]);
      } else if constexpr (G == 2) {
        reinterpret_cast<float2*>(tab)[slot] = make_float2(v[0], v[1]);
      } else {
        tab[slot] = v[0];
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < S; ++s) {
      float u[16][G];
#pragma unroll
      for (int x = 0; x < 16; ++x) {
#pragma unroll
        for (int g = 0; g < G; ++g) u[x][g] = 0.f;
#pragma unroll
        for (int m = 0; m < MC; ++m) {
          uint32_t e;
          switch (c * MC + m) {
            case 0: e = id_byte<0>(idw[s][x]); break;
            case 1: e = id_byte<1>(idw[s][x]); break;
            case 2: e = id_byte<2>(idw[s][x]); break;
            case 3: e = id_byte<3>(idw[s][x]); break;
            case 4: e = id_byte<4>(idw[s][x]); break;
            case 5: e = id_byte<5>(idw[s][x]); break;
            case 6: e = id_byte<6>(idw[s][x]); break;
            default: e = id_byte<7>(idw[s][x]); break;
          }
          lds_add<G>(tab, ((int)e * MC + m) * 16 + j, u[x]);
        }
      }
      row16_reduce_scatter<G>(u);
#pragma unroll
      for (int g = 0; g < G; ++g) part[s][g] += u[0][g];
    }
  }

  // scores and the first-digit histogram (in the staging buffer)
  __syncthreads();
  uint32_t* lhist = reinterpret_cast<uint32_t*>(stage);
  for (int i = tid; i < G * kHistBins; i += kScoreThreads) lhist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t key = gkey(s) + lane;
    if (key < n) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float sc = vnv[s] * part[s][g];
        scores[(int64_t)(bg0 + g) * n_cap + key] = sc;
        uint32_t dg = __float_as_uint(sc) >> kHistShift;
        if (dg > kHistBins - 1) dg = kHistBins - 1;
        atomicAdd(&lhist[g * kHistBins + dg], 1u);
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < G * kHistBins; i += kScoreThreads) {
    const uint32_t v = lhist[i];
    if (v) atomicAdd(&hist[(int64_t)(bg0 + i / kHistBins) * kHistBins + (i % kHistBins)], v);
  }
}

// ---------------------------------------------------------------- top-k: scan

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelGroups = 16;                             // 64-key groups per wave
constexpr int kSelChunk = kSelWaves * kSelGroups * 64;     // keys per scan workgroup (8192)
constexpr int kCandLds = 4096;                             // candidates resolved in LDS

// Block-wide inclusive scan of one value per thread (kSelThreads threads).
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  uint32_t off = 0;
  for (int w = 0; w < wave; ++w) off += wsum[w];
  return v + off;
}

struct Boundary {
  uint32_t d1, above;
};

// Bin of the first digit that holds the k-th largest score, and how many keys
// lie in higher bins.  Every thread of the block must call it.
__device__ Boundary find_boundary(const uint32_t* hh, uint32_t k, uint32_t* wsum, Boundary* sh) {
  const int tid = threadIdx.x;
  const uint32_t c_hi = hh[kHistBins - 1 - 2 * tid];
  const uint32_t c_lo = hh[kHistBins - 2 - 2 * tid];
  const uint32_t inc = block_incl_scan(c_hi + c_lo, wsum);
  const uint32_t prev = inc - c_hi - c_lo;
  if (prev < k && k <= prev + c_hi) *sh = Boundary{(uint32_t)(kHistBins - 1 - 2 * tid), prev};
  else if (prev + c_hi < k && k <= inc) *sh = Boundary{(uint32_t)(kHistBins - 2 - 2 * tid), prev + c_hi};
  __syncthreads();
  const Boundary r = *sh;
  __syncthreads();
  return r;
}

__device__ __forceinline__ void clamp_nk(int64_t n_cap, int32_t len, int32_t kk, int k_max,
                                         int64_t* n, int64_t* k) {
  int64_t nn = len;
  if (nn < 0) nn = 0;
  if (nn > n_cap) nn = n_cap;
  int64_t k2 = kk;
  if (k2 < 0) k2 = 0;
  if (k2 > nn) k2 = nn;
  if (k2 > k_max) k2 = k_max;
  *n = nn;
  *k = k2;
}

// grid: B*Hq*CH blocks of kSelThreads, CH = ceil(n_cap / kSelChunk).
__global__ __launch_bounds__(kSelThreads) void topk_scan_kernel(
    const float* __restrict__ scores, int64_t n_cap, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ ks, int k_max, int Hq, int CH, const uint32_t* __restrict__ hist,
    uint32_t* __restrict__ counters, uint32_t* __restrict__ bitmap, int64_t words,
    uint2* __restrict__ cand) {
  const int bg = blockIdx.x / CH;
  const int c = blockIdx.x % CH;
  const int b = bg / Hq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t n, k;
  clamp_nk(n_cap, lens[b], ks[b], k_max, &n, &k);
  if (k == 0) return;
  const int64_t n64 = (n + 63) & ~(int64_t)63;
  const int64_t c0 = (int64_t)c * kSelChunk;
  if (c0 >= n64) return;

  // this lane's scores first (16 keys, one per 64-key group of the wave)
  const float* srow = scores + (int64_t)bg * n_cap;
  uint32_t bits[kSelGroups];
#pragma unroll
  for (int i = 0; i < kSelGroups; ++i) {
    const int64_t key = c0 + ((int64_t)i * kSelWaves + wave) * 64 + lane;
    bits[i] = key < n ? __float_as_uint(srow[key]) : 0u;
  }
  __shared__ uint32_t wsum[kSelWaves];
  __shared__ Boundary shb;
  const Boundary bd = find_boundary(hist + (int64_t)bg * kHistBins, (uint32_t)k, wsum, &shb);

  // candidates gather in LDS first; one global reservation per workgroup
  __shared__ uint2 lc[kSelChunk];
  __shared__ uint32_t lcount, gbase;
  if (tid == 0) lcount = 0u;
  __syncthreads();
  uint32_t* bm = bitmap + (int64_t)bg * words;
#pragma unroll
  for (int i = 0; i < kSelGroups; ++i) {
    const int64_t base = c0 + ((int64_t)i * kSelWaves + wave) * 64;
    if (base >= n64) break;
    const int64_t key = base + lane;
    const bool valid = key < n;
    uint32_t dg = bits[i] >> kHistShift;
    if (dg > kHistBins - 1) dg = kHistBins - 1;
    const bool sel = valid && dg > bd.d1;
    const bool cnd = valid && dg == bd.d1;
    const uint64_t smask = __ballot(sel);
    const uint64_t cmask = __ballot(cnd);
    if (lane == 0) *reinterpret_cast<uint2*>(bm + (base >> 5)) =
        make_uint2((uint32_t)smask, (uint32_t)(smask >> 32));
    if (cmask) {
      uint32_t pos0 = 0;
      if (lane == 0) pos0 = atomicAdd(&lcount, (uint32_t)__popcll(cmask));
      pos0 = __shfl(pos0, 0, 64);
      if (cnd) lc[pos0 + __popcll(cmask & lanemask_lt64())] = make_uint2(bits[i], (uint32_t)key);
    }
  }
  __syncthreads();
  const uint32_t cnt = lcount;
  if (cnt == 0) return;
  if (tid == 0) gbase = atomicAdd(&counters[bg * 4 + 0], cnt);
  __syncthreads();
  uint2* crow = cand + (int64_t)bg * n_cap + gbase;
  for (uint32_t t = tid; t < cnt; t += kSelThreads) crow[t] = lc[t];
}

// ---------------------------------------------------------------- top-k: resolve

struct Pick {
  uint32_t digit, before, inbin;
};

// Among candidates whose low 21 score bits match (vmask, vval) -- and, when
// BY_INDEX, whose index matches (imask, ival) -- histogram the 7-bit digit at
// `shift` of the score bits (or of the index) and return the digit holding
// the `need`-th entry: counted from the top for scores, from the bottom for
// indices (the lower index wins a tie).
template <bool BY_INDEX>
__device__ Pick radix_pick(const uint2* cand, uint32_t C, uint32_t vmask, uint32_t vval,
                           uint32_t imask, uint32_t ival, int shift, uint32_t need,
                           uint32_t* h128, Pick* shpick) {
  const int tid = threadIdx.x;
  if (tid < 128) h128[tid] = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < C; i += kSelThreads) {
    const uint2 e = cand[i];
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
    uint32_t inc = c0 + c1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = __shfl_up(inc, o, 64);
      if (tid >= o) inc += t;
    }
    const uint32_t prev = inc - c0 - c1;
    if (prev < need && need <= prev + c0) *shpick = Pick{(uint32_t)b0, prev, c0};
    else if (prev + c0 < need && need <= inc) *shpick = Pick{(uint32_t)b1, prev + c0, c1};
  }
  __syncthreads();
  const Pick r = *shpick;
  __syncthreads();
  return r;
}

constexpr int kSegWords = kSelThreads * 8;  // bitmap words turned into indices per pass

// grid: B*Hq blocks of kSelThreads.
__global__ __launch_bounds__(kSelThreads) void topk_resolve_kernel(
    int64_t n_cap, const int32_t* __restrict__ lens, const int32_t* __restrict__ ks, int k_max,
    int Hq, const uint32_t* __restrict__ hist, const uint32_t* __restrict__ counters,
    const uint32_t* __restrict__ bitmap, int64_t words, const uint2* __restrict__ cand,
    int32_t* __restrict__ idx) {
  const int bg = blockIdx.x;
  const int b = bg / Hq;
  const int tid = threadIdx.x;
  int64_t n, k;
  clamp_nk(n_cap, lens[b], ks[b], k_max, &n, &k);
  int32_t* out = idx + (int64_t)bg * k_max;
  if (k == 0) {
    for (int t = tid; t < k_max; t += kSelThreads) out[t] = -1;
    return;
  }
  __shared__ uint32_t wsum[kSelWaves];
  __shared__ Boundary shb;
  __shared__ uint32_t h128[128];
  __shared__ Pick shpick;
  __shared__ uint2 lcand[kCandLds];
  __shared__ uint32_t lbm[kSegWords];
  __shared__ uint32_t seg_total;

  const Boundary bd = find_boundary(hist + (int64_t)bg * kHistBins, (uint32_t)k, wsum, &shb);
  const uint32_t C = counters[bg * 4 + 0];
  uint32_t need = (uint32_t)k - bd.above;  // 1 <= need <= C
  const uint2* crow = cand + (int64_t)bg * n_cap;
  const uint2* cp = crow;
  if (C <= (uint32_t)kCandLds) {
    for (uint32_t i = tid; i < C; i += kSelThreads) lcand[i] = crow[i];
    __syncthreads();
    cp = lcand;
  }
  // low 21 bits of the score (the boundary bin fixes the rest)
  uint32_t vmask = 0u, vval = 0u, ties = 0u;
  for (int shift = 14; shift >= 0; shift -= 7) {
    const Pick pk = radix_pick<false>(cp, C, vmask, vval, 0u, 0u, shift, need, h128, &shpick);
    need -= pk.before;
    vval |= pk.digit << shift;
    vmask |= 127u << shift;
    ties = pk.inbin;
  }
  // among keys with exactly that score, the lower indices win
  uint32_t imax = 0xFFFFFFFFu;
  if (ties > need) {
    uint32_t imask = 0u, ival = 0u;
    int top = 0;
    while (((uint64_t)1 << top) < (uint64_t)n) ++top;
    int shift = top > 7 ? top - 7 : 0;
    for (;;) {
      const Pick pk = radix_pick<true>(cp, C, vmask, vval, imask, ival, shift, need, h128, &shpick);
      need -= pk.before;
      ival |= pk.digit << shift;
      imask |= 127u << shift;
      if (shift == 0) break;
      shift = shift > 7 ? shift - 7 : 0;
    }
    imax = ival;
  }
  // bitmap (+ the chosen candidates) -> ascending indices, one segment at a time
  const uint32_t* bm = bitmap + (int64_t)bg * words;
  const int64_t nwords = (n + 31) >> 5;
  uint32_t written = 0;
  for (int64_t w0 = 0; w0 < nwords; w0 += kSegWords) {
    const int64_t segn = (nwords - w0) < kSegWords ? (nwords - w0) : kSegWords;
    for (int i = tid; i < kSegWords; i += kSelThreads) lbm[i] = i < segn ? bm[w0 + i] : 0u;
    __syncthreads();
    for (uint32_t i = tid; i < C; i += kSelThreads) {
      const uint2 e = cp[i];
      const uint32_t v = e.x & 0x1FFFFFu;
      const int64_t wi = (int64_t)(e.y >> 5) - w0;
      if (wi >= 0 && wi < segn && (v > vval || (v == vval && e.y <= imax)))
        atomicOr(&lbm[wi], 1u << (e.y & 31));
    }
    __syncthreads();
    uint32_t wv[8];
    uint32_t cnt = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      wv[t] = lbm[tid * 8 + t];
      cnt += __popc(wv[t]);
    }
    const uint32_t inc = block_incl_scan(cnt, wsum);
    uint32_t pos = written + inc - cnt;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      uint32_t x = wv[t];
      const int64_t wi = w0 + tid * 8 + t;
      while (x) {
        const int bit = __ffs(x) - 1;
        x &= x - 1;
        if (pos < (uint32_t)k_max) out[pos] = (int32_t)(wi * 32 + bit);
        ++pos;
      }
    }
    if (tid == kSelThreads - 1) seg_total = inc;
    __syncthreads();
    written += seg_total;
    __syncthreads();
  }
  for (int64_t t = (int64_t)k + tid; t < k_max; t += kSelThreads) out[t] = -1;
}

// ---------------------------------------------------------------- launchers

template <int G, int TL, int S>
static void launch_scorer(int B, int Hkv, int Hq, int L, int P, int64_t n_cap, int nblk, int gpb,
                          const ScoreWs& ws, const uint8_t* ids, const float* vnorm,
                          const int32_t* lens, float* scores, hipStream_t s) {
  scorer_kernel<G, TL, S><<<(unsigned)(B * Hkv * nblk), kScoreThreads, 0, s>>>(
      ws.sub, ids, vnorm, lens, Hq, Hkv, L, P, n_cap, nblk, gpb, scores, ws.hist);
}

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

// Split the 64-key groups of every (b, h) over blocks so that the grid fills
// the CUs once (one scorer block fits per CU), within the S groups per wave
// that the register budget allows.
template <int G, int TL>
static void launch_scorer_s(int B, int Hkv, int Hq, int L, int P, int64_t n_cap,
                            const ScoreWs& ws, const uint8_t* ids, const float* vnorm,
                            const int32_t* lens, float* scores, hipStream_t s) {
  constexpr int SMAX = G == 4 ? (TL == 8 ? 1 : 4) : (TL == 8 ? 2 : (G == 2 ? 4 : 8));
  const int64_t ng = (n_cap + 63) / 64;
  const int64_t heads = (int64_t)B * Hkv;
  int64_t nblk = (device_cus() + heads - 1) / heads;
  if (nblk > ng) nblk = ng;
  int64_t gpb = (ng + nblk - 1) / nblk;
  if (gpb > (int64_t)kScoreWaves * SMAX) {
    gpb = (int64_t)kScoreWaves * SMAX;
    nblk = (ng + gpb - 1) / gpb;
  }
  const int need = (int)((gpb + kScoreWaves - 1) / kScoreWaves);
  const int nb = (int)nblk, gp = (int)gpb;
  if constexpr (SMAX >= 8) {
    if (need > 4) return launch_scorer<G, TL, 8>(B, Hkv, Hq, L, P, n_cap, nb, gp, ws, ids, vnorm, lens, scores, s);
  }
  if constexpr (SMAX >= 4) {
    if (need > 2) return launch_scorer<G, TL, 4>(B, Hkv, Hq, L, P, n_cap, nb, gp, ws, ids, vnorm, lens, scores, s);
  }
  if constexpr (SMAX >= 2) {
    if (need > 1) return launch_scorer<G, TL, 2>(B, Hkv, Hq, L, P, n_cap, nb, gp, ws, ids, vnorm, lens, scores, s);
  }
  launch_scorer<G, TL, 1>(B, Hkv, Hq, L, P, n_cap, nb, gp, ws, ids, vnorm, lens, scores, s);
}

template <int G>
static void launch_scorer_g(int B, int Hkv, int Hq, int L, int P, int64_t n_cap,
                            const ScoreWs& ws, const uint8_t* ids, const float* vnorm,
                            const int32_t* lens, float* scores, hipStream_t s) {
  const int per_lane = ids_word_bytes(L);  // tables per lane
  if (per_lane <= 1) launch_scorer_s<G, 1>(B, Hkv, Hq, L, P, n_cap, ws, ids, vnorm, lens, scores, s);
  else if (per_lane <= 2) launch_scorer_s<G, 2>(B, Hkv, Hq, L, P, n_cap, ws, ids, vnorm, lens, scores, s);
  else if (per_lane <= 4) launch_scorer_s<G, 4>(B, Hkv, Hq, L, P, n_cap, ws, ids, vnorm, lens, scores, s);
  else launch_scorer_s<G, 8>(B, Hkv, Hq, L, P, n_cap, ws, ids, vnorm, lens, scores, s);
}

hipError_t launch_soft_tables(const void* q, int dtype, int B, int Hq, const void* W, int L,
                              int P, float tau, const ScoreWs& ws, hipStream_t s) {
  const int heads = B * Hq;
  if (dtype == 1)
    soft_tables_kernel<uint16_t><<<heads, 256, 0, s>>>(static_cast<const uint16_t*>(q),
                                                       static_cast<const uint16_t*>(W), L, P,
                                                       tau, ws.sub, ws.hist, ws.counters);
  else
    soft_tables_kernel<float><<<heads, 256, 0, s>>>(static_cast<const float*>(q),
                                                    static_cast<const float*>(W), L, P, tau,
                                                    ws.sub, ws.hist, ws.counters);
  return hipGetLastError();
}

hipError_t launch_score(int B, int Hq, int Hkv, int L, int P, const uint8_t* ids,
                        const float* vnorm, const int32_t* lens, int64_t n_cap, float* scores,
                        const ScoreWs& ws, hipStream_t s) {
  switch (Hq / Hkv) {
    case 1: launch_scorer_g<1>(B, Hkv, Hq, L, P, n_cap, ws, ids, vnorm, lens, scores, s); break;
    case 2: launch_scorer_g<2>(B, Hkv, Hq, L, P, n_cap, ws, ids, vnorm, lens, scores, s); break;
    default: launch_scorer_g<4>(B, Hkv, Hq, L, P, n_cap, ws, ids, vnorm, lens, scores, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_topk(int B, int Hq, const float* scores, const int32_t* lens, int64_t n_cap,
                       const int32_t* ks, int k_max, int32_t* idx, const ScoreWs& ws,
                       hipStream_t s) {
  const int CH = (int)((n_cap + kSelChunk - 1) / kSelChunk);
  topk_scan_kernel<<<(unsigned)(B * Hq * CH), kSelThreads, 0, s>>>(
      scores, n_cap, lens, ks, k_max, Hq, CH, ws.hist, ws.counters, ws.bitmap, ws.words, ws.cand);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  topk_resolve_kernel<<<(unsigned)(B * Hq), kSelThreads, 0, s>>>(
      n_cap, lens, ks, k_max, Hq, ws.hist, ws.counters, ws.bitmap, ws.words, ws.cand, idx);
  return hipGetLastError();
}

}  // namespace socketlsh
