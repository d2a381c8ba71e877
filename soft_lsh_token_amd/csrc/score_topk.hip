// Query soft hashing, soft-count scoring and top-k selection
// (SOCKET Sec. 4.1, Algorithms 2 and 3).
//
// Soft hashing: table l gives bucket c the probability
//   p_l(c) = softmax_c( sum_j s_j(c) u_lj / tau ),  s_j(c) = +1 if bit j of c else -1,
// which factorises over the planes as prod_j sigmoid(2 s_j(c) u_lj / tau).
// The factorisation splits every table into a low half (planes 0..3) and a
// high half (planes 4..7) of at most 16 entries each; the scorer rebuilds
// p_l(c) = lo_l(c & 15) * hi_l(c >> 4) in LDS.  The projections u = W q are
// taken in float64.
//
// Scorer (one pass per KV head for all of its GQA query heads): the tables
// of the G query heads of one KV head are interleaved in LDS as
//   slot(c, m, j) = (c * M + m) * 16 + j,   one slot = G floats,
// where lane j of a 16-lane row owns tables j*M .. j*M+M-1 of the current
// chunk.  A 16-lane row works on one key at a time, so its 16 lookups fall
// into 16 different 16-byte bank groups whatever the bucket IDs are (gfx950
// serves 16 lanes of a ds_read_b128 per cycle).  The per-lane partial sums
// are reduced across the row with DPP.  When the tables of all G heads do
// not fit in 128 KiB the tables are processed in chunks.
//
// Top-k: the scorer also builds, per query head, a histogram of the top
// digit of the float32 score bits (scores are non-negative, so their bit
// patterns order like the values).  The select kernel finds the bin that
// holds the k-th largest score, marks every key above it in a bitmap, and
// collects the keys of the boundary bin as candidates.  The last workgroup
// of each head resolves the candidates exactly by radix select on (score
// bits, lower index first) and turns the bitmap into ascending indices.
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
    double u = 0.0;
    for (int t = 0; t < kHead; ++t) {
      double w;
      if constexpr (sizeof(T) == 2)
        w = (double)__uint_as_float((uint32_t)W[(int64_t)pl * kHead + t] << 16);
      else
        w = (double)W[(int64_t)pl * kHead + t];
      u = fma(w, qd[t], u);
    }
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
struct VecG;
template <> struct VecG<1> { typedef float type; };
template <> struct VecG<2> { typedef float2 type; };
template <> struct VecG<4> { typedef float4 type; };

template <int G>
__device__ __forceinline__ void lds_add(const float* lds, int slot, float* acc) {
  if constexpr (G == 1) {
    acc[0] += lds[slot];
  } else if constexpr (G == 2) {
    const float2 v = reinterpret_cast<const float2*>(lds)[slot];
    acc[0] += v.x; acc[1] += v.y;
  } else if constexpr (G == 4) {
    const float4 v = reinterpret_cast<const float4*>(lds)[slot];
    acc[0] += v.x; acc[1] += v.y; acc[2] += v.z; acc[3] += v.w;
  } else {
    const float4 v0 = reinterpret_cast<const float4*>(lds)[2 * slot];
    const float4 v1 = reinterpret_cast<const float4*>(lds)[2 * slot + 1];
    acc[0] += v0.x; acc[1] += v0.y; acc[2] += v0.z; acc[3] += v0.w;
    acc[4] += v1.x; acc[5] += v1.y; acc[6] += v1.z; acc[7] += v1.w;
  }
}

constexpr int kScoreThreads = 1024;
constexpr int kScoreWaves = kScoreThreads / 64;
constexpr int kTableFloats = 32768;  // 128 KiB of tables per chunk

// G: query heads per KV head; M: tables per lane per chunk (16*M tables per
// chunk); S: 64-key groups per wave.  grid: B*Hkv*nblk, block = 1024 threads.
template <int G, int M, int S>
__global__ __launch_bounds__(kScoreThreads) void scorer_kernel(
    const float* __restrict__ sub, const uint8_t* __restrict__ ids,
    const float* __restrict__ vnorm, const int32_t* __restrict__ lens, int Hq, int Hkv, int L,
    int P, int64_t n_cap, int nblk, float* __restrict__ scores, uint32_t* __restrict__ hist) {
  __shared__ __attribute__((aligned(16))) float tab[kTableFloats];
  __shared__ uint32_t lhist[G * kHistBins];
  constexpr int TC = 16 * M;
  constexpr int KPB = kScoreWaves * S * 64;
  const int blk = blockIdx.x % nblk;
  const int bh = blockIdx.x / nblk;
  const int b = bh / Hkv;
  const int h = bh % Hkv;
  int64_t n = lens[b];
  if (n > n_cap) n = n_cap;
  const int64_t kb0 = (int64_t)blk * KPB;
  if (kb0 >= n) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, kg = lane >> 4, j = lane & 15;
  const int bg0 = b * Hq + h * G;
  const int plo = P < 4 ? P : 4;
  const int lomask = (1 << plo) - 1;
  const int nent = 1 << P;
  for (int i = tid; i < G * kHistBins; i += kScoreThreads) lhist[i] = 0u;

  const int64_t wbase = kb0 + (int64_t)wave * S * 64;
  const uint8_t* idrow = ids + ((int64_t)bh * n_cap) * L;
  float part[S][G];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int g = 0; g < G; ++g) part[s][g] = 0.f;

  const int nchunks = (L + TC - 1) / TC;
  for (int c = 0; c < nchunks; ++c) {
    __syncthreads();
    // rebuild the chunk's tables: slot = (e*M + m)*16 + jj holds table c*TC + jj*M + m
    const int nslots = nent * TC;
    for (int slot = tid; slot < nslots; slot += kScoreThreads) {
      const int jj = slot & 15;
      const int m = (slot >> 4) % M;
      const int e = slot / (16 * M);
      const int l = c * TC + jj * M + m;
      float v[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        v[g] = 0.f;
        if (l < L) {
          const float* st = sub + ((int64_t)(bg0 + g) * L + l) * 32;
          v[g] = st[e & lomask] * st[16 + (e >> plo)];
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) tab[slot * G + g] = v[g];
    }
    __syncthreads();
    const int l0 = c * TC + j * M;  // first table of this lane in the chunk
#pragma unroll
    for (int s = 0; s < S; ++s) {
      for (int rr = 0; rr < 16; ++rr) {
        const int64_t key = wbase + s * 64 + kg * 16 + rr;
        float acc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = 0.f;
        if (key < n) {
          const uint8_t* p = idrow + key * L + l0;
          uint32_t e8[M];
          if ((L % M) == 0 && l0 + M <= L) {
            if constexpr (M == 1) {
              e8[0] = p[0];
            } else if constexpr (M == 2) {
              const uint32_t w = *reinterpret_cast<const uint16_t*>(p);
              e8[0] = w & 255u; e8[1] = w >> 8;
            } else if constexpr (M == 4) {
              const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
#pragma unroll
              for (int m = 0; m < 4; ++m) e8[m] = (w >> (8 * m)) & 255u;
            } else {
              const uint2 w = *reinterpret_cast<const uint2*>(p);
#pragma unroll
              for (int m = 0; m < 4; ++m) e8[m] = (w.x >> (8 * m)) & 255u;
#pragma unroll
              for (int m = 0; m < 4; ++m) e8[4 + m] = (w.y >> (8 * m)) & 255u;
            }
          } else {
#pragma unroll
            for (int m = 0; m < M; ++m) e8[m] = (l0 + m < L) ? (uint32_t)p[m] : 0u;
          }
#pragma unroll
          for (int m = 0; m < M; ++m) lds_add<G>(tab, ((int)e8[m] * M + m) * 16 + j, acc);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = row16_sum(acc[g]);
        if (j == rr) {
#pragma unroll
          for (int g = 0; g < G; ++g) part[s][g] += acc[g];
        }
      }
    }
  }
  // lane (kg, j) now holds key wbase + s*64 + lane
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int64_t key = wbase + s * 64 + lane;
    if (key < n) {
      const float vn = vnorm[(int64_t)bh * n_cap + key];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float sc = vn * part[s][g];
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

// ---------------------------------------------------------------- top-k select

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelChunk = 8192;   // keys per select workgroup (multiple of 64)
constexpr int kCandLds = 4096;    // candidates resolved from LDS when they fit

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

// Among entries of `cand` (count C) whose bits satisfy (bits & mask) == val,
// histogram the 7-bit digit (x >> shift) & 127 of x = key(entry) and return,
// through `out`, the largest digit whose suffix count reaches `need` (or the
// smallest digit whose prefix count reaches it when `ascending`).
struct Pick {
  uint32_t digit, before, inbin;
};

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
    // value digits: scan from the top bin down; index digits: from bin 0 up
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

// grid: B*Hq*CH blocks of kSelThreads.  CH = ceil(n_cap / kSelChunk).
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(
    const float* __restrict__ scores, int64_t n_cap, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ ks, int k_max, int Hq, int CH, const uint32_t* __restrict__ hist,
    uint32_t* __restrict__ counters, uint32_t* __restrict__ bitmap, int64_t words,
    uint2* __restrict__ cand, int32_t* __restrict__ idx) {
  const int bg = blockIdx.x / CH;
  const int c = blockIdx.x % CH;
  const int b = bg / Hq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t n = lens[b];
  if (n < 0) n = 0;
  if (n > n_cap) n = n_cap;
  int64_t k = ks[b];
  if (k < 0) k = 0;
  if (k > n) k = n;
  if (k > k_max) k = k_max;
  int32_t* out = idx + (int64_t)bg * k_max;
  if (k == 0) {
    if (c == 0)
      for (int t = tid; t < k_max; t += kSelThreads) out[t] = -1;
    return;
  }
  const int64_t n64 = (n + 63) & ~(int64_t)63;
  const int64_t c0 = (int64_t)c * kSelChunk;
  if (c0 >= n64) return;
  const int nch = (int)((n64 + kSelChunk - 1) / kSelChunk);

  __shared__ uint32_t wsum[kSelWaves];
  __shared__ uint32_t sh_d1, sh_above, sh_last;
  __shared__ uint32_t h128[128];
  __shared__ Pick shpick;
  __shared__ uint2 lcand[kCandLds];
  __shared__ uint32_t seg[kSelThreads];

  // 1. boundary bin of the first digit (histogram built by the scorer)
  {
    const uint32_t* hh = hist + (int64_t)bg * kHistBins;
    const uint32_t c_hi = hh[kHistBins - 1 - 2 * tid];
    const uint32_t c_lo = hh[kHistBins - 2 - 2 * tid];
    const uint32_t inc = block_incl_scan(c_hi + c_lo, wsum);
    const uint32_t prev = inc - c_hi - c_lo;
    const uint32_t kk = (uint32_t)k;
    if (prev < kk && kk <= prev + c_hi) { sh_d1 = kHistBins - 1 - 2 * tid; sh_above = prev; }
    else if (prev + c_hi < kk && kk <= inc) { sh_d1 = kHistBins - 2 - 2 * tid; sh_above = prev + c_hi; }
    __syncthreads();
  }
  const uint32_t d1 = sh_d1;
  const uint32_t above = sh_above;

  // 2. scan this chunk: keys above the boundary bin go to the bitmap, keys in it are candidates
  const float* srow = scores + (int64_t)bg * n_cap;
  uint32_t* bm = bitmap + (int64_t)bg * words;
  uint2* crow = cand + (int64_t)bg * n_cap;
  int64_t c1 = c0 + kSelChunk;
  if (c1 > n64) c1 = n64;
  for (int64_t base = c0 + (int64_t)wave * 64; base < c1; base += kSelThreads) {
    const int64_t key = base + lane;
    uint32_t bits = 0u;
    const bool valid = key < n;
    if (valid) bits = __float_as_uint(srow[key]);
    uint32_t dg = bits >> kHistShift;
    if (dg > kHistBins - 1) dg = kHistBins - 1;
    const bool sel = valid && dg > d1;
    const bool cnd = valid && dg == d1;
    const uint64_t smask = __ballot(sel);
    const uint64_t cmask = __ballot(cnd);
    if (lane == 0) {
      bm[base >> 5] = (uint32_t)smask;
      bm[(base >> 5) + 1] = (uint32_t)(smask >> 32);
    }
    if (cmask) {
      uint32_t pos0 = 0;
      if (lane == 0) pos0 = atomicAdd(&counters[bg * 4 + 0], (uint32_t)__popcll(cmask));
      pos0 = __shfl(pos0, 0, 64);
      if (cnd) crow[pos0 + __popcll(cmask & lanemask_lt64())] = make_uint2(bits, (uint32_t)key);
    }
  }

  // 3. the last workgroup of this head finishes the selection
  __threadfence();
  __syncthreads();
  if (tid == 0) sh_last = (atomicAdd(&counters[bg * 4 + 1], 1u) == (uint32_t)(nch - 1)) ? 1u : 0u;
  __syncthreads();
  if (!sh_last) return;
  __threadfence();

  const uint32_t C = __atomic_load_n(&counters[bg * 4 + 0], __ATOMIC_RELAXED);
  uint32_t need = (uint32_t)k - above;  // 1 <= need <= C
  const uint2* cp = crow;
  if (C <= (uint32_t)kCandLds) {
    for (uint32_t i = tid; i < C; i += kSelThreads) lcand[i] = crow[i];
    __syncthreads();
    cp = lcand;
  }
  // 3a. low 21 bits of the score (the boundary bin fixes the rest)
  uint32_t vmask = 0u, vval = 0u, ties = 0u;
  for (int shift = 14; shift >= 0; shift -= 7) {
    const Pick pk = radix_pick<false>(cp, C, vmask, vval, 0u, 0u, shift, need, h128, &shpick);
    need -= pk.before;
    vval |= pk.digit << shift;
    vmask |= 127u << shift;
    ties = pk.inbin;
  }
  // 3b. among keys with exactly that score, the lower indices win
  uint32_t imax = 0xFFFFFFFFu;
  if (ties > need) {
    uint32_t imask = 0u, ival = 0u;
    int top = 0;
    while (((uint64_t)1 << top) < (uint64_t)n) ++top;  // indices fit in `top` bits
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
  for (uint32_t i = tid; i < C; i += kSelThreads) {
    const uint2 e = cp[i];
    const uint32_t v = e.x & 0x1FFFFFu;
    if (v > vval || (v == vval && e.y <= imax)) atomicOr(&bm[e.y >> 5], 1u << (e.y & 31));
  }
  __threadfence();
  __syncthreads();
  // 4. bitmap -> ascending indices
  const int64_t nwords = (n + 31) >> 5;
  constexpr int WPT = 8;
  uint32_t written = 0;
  for (int64_t w0 = 0; w0 < nwords; w0 += (int64_t)kSelThreads * WPT) {
    uint32_t wv[WPT];
    uint32_t cnt = 0;
#pragma unroll
    for (int t = 0; t < WPT; ++t) {
      const int64_t wi = w0 + (int64_t)tid * WPT + t;
      wv[t] = wi < nwords ? bm[wi] : 0u;
      if (wi == nwords - 1 && (n & 31)) wv[t] &= (1u << (n & 31)) - 1u;
      cnt += __popc(wv[t]);
    }
    const uint32_t inc = block_incl_scan(cnt, wsum);
    uint32_t pos = written + inc - cnt;
#pragma unroll
    for (int t = 0; t < WPT; ++t) {
      uint32_t x = wv[t];
      const int64_t wi = w0 + (int64_t)tid * WPT + t;
      while (x) {
        const int bit = __ffs(x) - 1;
        x &= x - 1;
        if (pos < (uint32_t)k_max) out[pos] = (int32_t)(wi * 32 + bit);
        ++pos;
      }
    }
    if (tid == kSelThreads - 1) seg[0] = inc;
    __syncthreads();
    written += seg[0];
    __syncthreads();
  }
  for (int64_t t = (int64_t)k + tid; t < k_max; t += kSelThreads) out[t] = -1;
}

// ---------------------------------------------------------------- launcher

template <int G, int M, int S>
static void launch_scorer(int B, int Hkv, int Hq, int L, int P, int64_t n_cap,
                          const ScoreWs& ws, const uint8_t* ids, const float* vnorm,
                          const int32_t* lens, float* scores, hipStream_t s) {
  constexpr int KPB = kScoreWaves * S * 64;
  const int nblk = (int)((n_cap + KPB - 1) / KPB);
  scorer_kernel<G, M, S><<<(unsigned)(B * Hkv * nblk), kScoreThreads, 0, s>>>(
      ws.sub, ids, vnorm, lens, Hq, Hkv, L, P, n_cap, nblk, scores, ws.hist);
}

template <int G, int M>
static void launch_scorer_s(int S, int B, int Hkv, int Hq, int L, int P, int64_t n_cap,
                            const ScoreWs& ws, const uint8_t* ids, const float* vnorm,
                            const int32_t* lens, float* scores, hipStream_t s) {
  switch (S) {
    case 1: launch_scorer<G, M, 1>(B, Hkv, Hq, L, P, n_cap, ws, ids, vnorm, lens, scores, s); break;
    case 2: launch_scorer<G, M, 2>(B, Hkv, Hq, L, P, n_cap, ws, ids, vnorm, lens, scores, s); break;
    case 4: launch_scorer<G, M, 4>(B, Hkv, Hq, L, P, n_cap, ws, ids, vnorm, lens, scores, s); break;
    default: launch_scorer<G, M, 8>(B, Hkv, Hq, L, P, n_cap, ws, ids, vnorm, lens, scores, s); break;
  }
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
  // 64-key groups per wave: aim for about one workgroup per CU
  const int64_t total = (int64_t)B * Hkv * n_cap;
  int S = 1;
  while (S < 8 && total > (int64_t)256 * kScoreThreads * S * 3 / 2) S *= 2;
  const int G = Hq / Hkv;
  switch (G) {
    case 1: launch_scorer_s<1, 8>(S, B, Hkv, Hq, L, P, n_cap, ws, ids, vnorm, lens, scores, s); break;
    case 2: launch_scorer_s<2, 4>(S, B, Hkv, Hq, L, P, n_cap, ws, ids, vnorm, lens, scores, s); break;
    default: launch_scorer_s<4, 2>(S, B, Hkv, Hq, L, P, n_cap, ws, ids, vnorm, lens, scores, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_topk(int B, int Hq, const float* scores, const int32_t* lens, int64_t n_cap,
                       const int32_t* ks, int k_max, int32_t* idx, const ScoreWs& ws,
                       hipStream_t s) {
  const int CH = (int)((n_cap + kSelChunk - 1) / kSelChunk);
  topk_select_kernel<<<(unsigned)(B * Hq * CH), kSelThreads, 0, s>>>(
      scores, n_cap, lens, ks, k_max, Hq, CH, ws.hist, ws.counters, ws.bitmap, ws.words, ws.cand,
      idx);
  return hipGetLastError();
}

}  // namespace socketlsh
