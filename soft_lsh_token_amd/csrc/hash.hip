// Key hashing and value norms (SOCKET Sec. 4.1, Algorithm 1: one bucket per
// table per key from L random projections, cached with the value norms;
// Appendix B.2: the bucket ID is the sign pattern of W^(l) k).
//
// Two projection paths:
//  * hash_mfma_kernel: bf16 keys, P = 8 with L in {16, 32, 64}, or P = 10
//    with any L <= 64.  The projection Z = W K^T is a bf16 MFMA GEMM
//    (v_mfma_f32_32x32x16_bf16, fp32 accumulation).  W stays in registers
//    for the whole workgroup (each consumer wave owns two 32-row MFMA tiles
//    of planes: 8 tables of 8 planes, or 6 tables of 10 planes plus 4 zero
//    rows); producer waves stream 128-key tiles of K through two LDS buffers
//    (and the value rows of the same keys to their norms) while the
//    consumers multiply the previous tile.  The planes of each tile are
//    ordered so that every lane's accumulators hold complete tables, which
//    turns the sign test + bit packing into lane-local work.
//    The same kernel also writes the packed sign codes of the hard-LSH mode
//    (any number of planes L*P): every 32-plane A tile pair of a consumer
//    wave then gives one 32-bit code word per key half-wave, and workgroups
//    split the planes into chunks of at most 16 words.
//  * hash_generic_kernel: any dtype, P <= 10, any L; one-wave workgroups,
//    each projecting one slice of a key's planes, one plane per lane.  Used
//    for float32 keys, for odd shapes and for the decode-time append of a
//    few keys.
#include "common.h"
#include "launch.h"

namespace socketlsh {

// ---------------------------------------------------------------- generic path

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* f);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* f) {
  unpack_bf16x8(*reinterpret_cast<const uint4*>(p), f);
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* f) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// grid: B*Hkv*count*S one-wave blocks.  The 16 ID words of a key (word w =
// tables w*TL .. w*TL+TL-1) are split into S slices of WPB words; block
// (key, s) projects the planes of slice s, one plane per lane, so a block
// reads only its slice of W.  The plane row is requested before the key
// position and the K (and, in slice 0, V) row right after it: two dependent
// global round trips per key.  The signs come out of one wave ballot, whose
// bit t*P + j is plane j of the slice's table t.
constexpr int kGenThreads = 64;

template <typename T>
__global__ __launch_bounds__(kGenThreads) void hash_generic_kernel(
    const T* __restrict__ K, const T* __restrict__ V, int Hkv, int64_t n_cap,
    const int32_t* __restrict__ pos0, int count, const T* __restrict__ W, int L, int P, int TL,
    int C, int WPB, int S, uint8_t* __restrict__ ids, float* __restrict__ vnorm) {
  constexpr int NV = kHead * (int)sizeof(T) / 16;  // 16-byte vectors per row
  const int s = blockIdx.x % S;
  const int rc = blockIdx.x / S;
  const int c = rc % count;
  const int bh = rc / count;
  const int b = bh / Hkv;
  const int lane = threadIdx.x;
  const int wpl = TL * P;               // planes per ID word
  const int pl = s * WPB * wpl + lane;  // this lane's plane
  const bool live = lane < WPB * wpl && pl / P < L;
  uint4 wv[NV];
  if (live) {
    const uint4* wr = reinterpret_cast<const uint4*>(W + (int64_t)pl * kHead);
#pragma unroll
    for (int v = 0; v < NV; ++v) wv[v] = wr[v];
  }
  const int64_t pos = (int64_t)pos0[b] + c;
  if (pos < 0 || pos >= n_cap) return;
  const int64_t row = (int64_t)bh * n_cap + pos;
  __shared__ float kf[kHead];
  float vf[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) vf[i] = 0.f;
  const bool norms = vnorm != nullptr;  // uniform: IDs only when there is no norm cache
  if (lane < 16) load8<T>(K + row * kHead + 8 * lane, kf + 8 * lane);
  if (norms && s == 0 && lane >= 16 && lane < 32) load8<T>(V + row * kHead + 8 * (lane - 16), vf);
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
  const uint64_t m = __ballot(live && z > 0.f);
  if (norms && s == 0) {  // value norm: lanes 16..31 form one DPP row
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(vf[i], vf[i], ss);
    ss = row16_sum(ss);
    if (lane == 16) vnorm[row] = sqrtf(ss);
  }
  if (lane < WPB) {
    // word = TL tables, cell b8 at bit b8 * CB (at most 64 bits)
    const int word = s * WPB + lane;
    const int CB = ids_cell_bits(L, P);
    uint64_t w = 0ull;
    for (int b8 = 0; b8 < TL; ++b8) {
      const int t = word * TL + b8;  // table
      if (t < L) {
        const uint64_t id = (m >> ((lane * TL + b8) * P)) & ((1ull << P) - 1ull);
        w |= id << (CB * b8);
      }
    }
    ids_store_word(ids, bh, n_cap, L, P, pos, word, w);
  }
}

// ---------------------------------------------------------------- norms only

// The value norms of rows [pos0[b], pos0[b]+count) without hashing: 16 lanes
// per row, 8 elements each, summed in the order of the hashing kernels
// (per-lane fused multiply-adds, then a DPP butterfly over the row), so the
// norms equal theirs bit for bit.  grid: ceil(B*Hkv*count / 16) blocks of
// kNormThreads; row r of the launch is position r % count of KV row r / count.
constexpr int kNormThreads = 256;

template <typename T>
__global__ __launch_bounds__(kNormThreads) void value_norms_kernel(
    const T* __restrict__ V, int Hkv, int64_t n_cap, const int32_t* __restrict__ pos0, int count,
    int64_t rows, float* __restrict__ vnorm) {
  int64_t r = (int64_t)blockIdx.x * (kNormThreads / 16) + (threadIdx.x >> 4);
  const bool live = r < rows;
  if (!live) r = rows - 1;  // the row's 16 lanes agree; re-read the last row, store nothing
  const int j = threadIdx.x & 15;
  const int64_t bh = r / count;
  const int64_t pos = (int64_t)pos0[bh / Hkv] + r % count;
  const bool in = live && pos >= 0 && pos < n_cap;
  float f[8];
  load_row8<T>(V + (bh * n_cap + (in ? pos : 0)) * kHead, j, f);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss);
  ss = row16_sum(ss);
  if (in && j == 0) vnorm[bh * n_cap + pos] = sqrtf(ss);
}

// ---------------------------------------------------------------- MFMA path

constexpr int kBTile = 32;     // keys per MFMA B tile
constexpr int kTK = 128;       // keys per LDS tile
constexpr int kProd = 4;       // producer waves
constexpr int kRowU4 = 17;     // K rows in LDS padded to 272 B: 16 consecutive keys hit 16 bank groups
constexpr int kProdU4 = kTK * 16 / (kProd * 64);  // K (and V) vectors per producer thread per tile (8)
constexpr int kStageRow = 68;  // two-byte IDs staged per key (64 tables + pad: 8-byte rows, 2-bank skew)

// Two-byte IDs of tables t0, t0+1, t0+2 of key pos (those < L), in the tiled
// layout of L tables (TL per word, 2*TL-byte words).  The lane holding table
// L - 1 also clears the rest of its word, and `pad` lanes clear the words
// past the last table, so that tables >= L read as 0.
__device__ __forceinline__ void store_wide(uint8_t* ids, int64_t bh, int64_t n_cap, int64_t pos,
                                           int L, int t0, uint32_t id0, uint32_t id1,
                                           uint32_t id2, bool pad) {
  const int TL = ids_tables_per_word(L), WB = 2 * TL;
  const uint32_t v[3] = {id0, id1, id2};
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int t = t0 + k;
    if (t < L) {
      *reinterpret_cast<uint16_t*>(ids + ids_word_offset(bh, n_cap, WB, pos, t / TL) +
                                   2 * (t % TL)) = (uint16_t)v[k];
      if (t == L - 1)
        for (int z = L; z % TL; ++z)
          *reinterpret_cast<uint16_t*>(ids + ids_word_offset(bh, n_cap, WB, pos, z / TL) +
                                       2 * (z % TL)) = (uint16_t)0;
    }
  }
  if (pad) {
    for (int w = (L + TL - 1) / TL; w < 16; ++w) {
      uint8_t* dst = ids + ids_word_offset(bh, n_cap, WB, pos, w);
      if (WB == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(0u, 0u);
      else if (WB == 4) *reinterpret_cast<uint32_t*>(dst) = 0u;
      else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)0;
    }
  }
}

// Block = NW consumer waves + kProd producer waves.  With one-byte IDs
// (WIDE false, P = 8, L = 8*NW) consumer wave w owns tables [8w, 8w+8) = two
// 32-plane MFMA A tiles, held in registers; with two-byte IDs (WIDE, P = 10,
// L <= 6*NW) it owns tables [6w, 6w+6).  Consumers only run MFMAs, pack sign
// bits and store IDs.  The producers load the next 128-key
// tile of K and V, write K into the other of two LDS buffers and store the
// value norms, while the consumers work on the current tile: one block
// barrier per tile, passed by every wave the same number of times.  MFMA
// k-slot (8*half + i) of step kk is head element 64*half + 8*kk + i for both
// operands.  Row R of A tile tt is plane r&7 of table
// 8w + 4*((R>>2)&1) + 2*tt + (r>>3), r = ((R>>3)<<2)|(R&3), so with the
// 32x32 accumulator layout (register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4) lane l holds whole tables.  WIDE: register r of
// tile tt in lane half h is accumulator c = 16*tt + r of that half; c < 30
// is plane c % 10 of table 6w + 3h + c / 10, and c = 30, 31 are zero rows.
// CODES (hard-LSH sign codes, LP = L*P planes, WPK words a key): the
// one-byte pipeline with plane 64*(NW*chunk + w) + 32*h + c as accumulator c
// of lane half h, so that the lane's packed word is code word
// 2*(NW*chunk + w) + h, bit c; planes >= LP are zero rows and masked out.
// grid: chunks*B*Hkv*nblk blocks; block blk hashes keys [pos0 + blk*kpb,
// +kpb) of (b, h) (for plane chunk `chunk` in CODES mode, the norms with
// chunk 0).  NRM false: no V loads, no norms.
constexpr int kModeIds8 = 0;    // one-byte IDs, P = 8
constexpr int kModeIds10 = 1;   // two-byte IDs, P = 10, L <= 32
constexpr int kModeCodes = 2;   // packed sign codes
constexpr int kModeIds10P = 3;  // packed ten-bit IDs, P = 10, 32 < L <= 64
template <int NW, int MODE, bool NRM>
__global__ __launch_bounds__((NW + kProd) * 64) void hash_mfma_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V, int Hkv, int64_t n_cap,
    const int32_t* __restrict__ pos0, int count, const uint16_t* __restrict__ W, int Lw,
    uint8_t* __restrict__ ids, float* __restrict__ vnorm, int kpb, int nblk,
    uint32_t* __restrict__ codes, int LP, int WPK, int chunks) {
  constexpr bool WIDE = MODE == kModeIds10 || MODE == kModeIds10P;
  constexpr bool PACKED = MODE == kModeIds10P;
  constexpr int L8 = NW * 8;  // tables of the one-byte layout
  constexpr int NB = kTK / kBTile;
  const int per_chunk = (int)(gridDim.x / (unsigned)chunks);
  const int chunk = (int)blockIdx.x / per_chunk;
  const int blk = ((int)blockIdx.x % per_chunk) % nblk;
  const int bh = ((int)blockIdx.x % per_chunk) / nblk;
  const bool nrm = NRM && chunk == 0;  // uniform
  const int b = bh / Hkv;
  const int64_t first = (int64_t)pos0[b];
  const int64_t start = first + (int64_t)blk * kpb;
  int64_t end = first + count;
  if (end > n_cap) end = n_cap;
  if (end > start + kpb) end = start + kpb;
  if (start >= end || start < 0) return;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const bool producer = wave >= NW;
  const int64_t rowbase = (int64_t)bh * n_cap;
  const int ntiles = (int)((end - start + kTK - 1) / kTK);
  __shared__ uint4 ktile[2][kTK * kRowU4];
  // two-byte IDs of the last two tiles, for packed words (WIDE with L > 32)
  __shared__ __attribute__((aligned(16))) uint16_t stage[PACKED ? 2 * kTK * kStageRow : 2];

  if (producer) {
    // The next tile's K and V wait in registers (8 named vectors each, one
    // per load u).  Loads use a uniform base of this workgroup's key range
    // plus a 32-bit byte offset (at most kpb rows of 256 bytes), clamped to
    // the range so every load is issued; K goes to LDS before any norm is
    // stored.
    static_assert(kProdU4 == 8, "eight vectors per producer thread");
    const char* kbase = reinterpret_cast<const char*>(K + (rowbase + start) * kHead);
    const char* vbase = nrm ? reinterpret_cast<const char*>(V + (rowbase + start) * kHead) : nullptr;
    const uint32_t last = (uint32_t)(end - start - 1);
    const int pt = tid - NW * 64;  // 0 .. kProd*64-1
    auto off_of = [&](int t, int u) -> uint32_t {
      const int e = pt + u * kProd * 64;
      uint32_t r = (uint32_t)(t * kTK + (e >> 4));
      if (r > last) r = last;  // past the range: re-read its last key
      return r * (kHead * 2) + (uint32_t)(e & 15) * 16u;
    };
#define SOCKET_LD(u) \
    k##u = *reinterpret_cast<const uint4*>(kbase + off_of(tl, u)); \
    if (nrm) v##u = *reinterpret_cast<const uint4*>(vbase + off_of(tl, u));
#define SOCKET_ST(u) kt[((pt + u * kProd * 64) >> 4) * kRowU4 + (pt & 15)] = k##u;
#define SOCKET_NRM(u) \
    { float f[8]; unpack_bf16x8(v##u, f); float ss = 0.f; \
      for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss); n##u = sqrtf(row16_sum(ss)); }
#define SOCKET_VN(u) \
    { const int64_t pos = start + (int64_t)ts * kTK + ((pt + u * kProd * 64) >> 4); \
      if (pos < end) vnorm[rowbase + pos] = n##u; }
    uint4 k0, k1, k2, k3, k4, k5, k6, k7, v0, v1, v2, v3, v4, v5, v6, v7;
    {
      const int tl = 0;
      SOCKET_LD(0) SOCKET_LD(1) SOCKET_LD(2) SOCKET_LD(3)
      SOCKET_LD(4) SOCKET_LD(5) SOCKET_LD(6) SOCKET_LD(7)
    }
    for (int ts = 0; ts <= ntiles; ++ts) {
      // stage tile ts (its loads were issued one step earlier), then load ts + 1
      if (ts < ntiles) {
        uint4* kt = ktile[ts & 1];
        SOCKET_ST(0) SOCKET_ST(1) SOCKET_ST(2) SOCKET_ST(3)
        SOCKET_ST(4) SOCKET_ST(5) SOCKET_ST(6) SOCKET_ST(7)
        if (nrm) {
          float n0, n1, n2, n3, n4, n5, n6, n7;
          SOCKET_NRM(0) SOCKET_NRM(1) SOCKET_NRM(2) SOCKET_NRM(3)
          SOCKET_NRM(4) SOCKET_NRM(5) SOCKET_NRM(6) SOCKET_NRM(7)
          if ((pt & 15) == 0) {
            SOCKET_VN(0) SOCKET_VN(1) SOCKET_VN(2) SOCKET_VN(3)
            SOCKET_VN(4) SOCKET_VN(5) SOCKET_VN(6) SOCKET_VN(7)
          }
        }
        const int tl = ts + 1;
        SOCKET_LD(0) SOCKET_LD(1) SOCKET_LD(2) SOCKET_LD(3)
        SOCKET_LD(4) SOCKET_LD(5) SOCKET_LD(6) SOCKET_LD(7)
      }
      lds_barrier();  // the next tile's loads stay in flight
    }
#undef SOCKET_LD
#undef SOCKET_ST
#undef SOCKET_NRM
#undef SOCKET_VN
    return;
  }

  // consumers: W-stationary A operands
  const int half = lane >> 5;
  const int col = lane & 31;
  bf16x8_t a[2][8];
  {
    const int R = col;
    const int hout = (R >> 2) & 1;
    const int r = ((R >> 3) << 2) | (R & 3);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if constexpr (WIDE) {
        const int c = 16 * tt + r;
        const int table = 6 * wave + 3 * hout + c / 10;
        const bool live = c < 30 && table < Lw;
        const uint16_t* wr = W + (int64_t)(live ? table * 10 + c % 10 : 0) * kHead + 64 * half;
        const bf16x8_t zero = {};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(wr + 8 * kk);
          a[tt][kk] = live ? v : zero;
        }
      } else {
        // stored negated: the accumulator of a plane is then -(W k), rounded as
        // W k with the sign flipped, so the plane's bit (W k > 0) is its sign
        // bit (an exact zero sums to +0 from the +0 start and gives 0)
        // plane 64*wave + 32*hout + 16*tt + r (of the chunk, for codes)
        int plane = 64 * wave + 32 * hout + 16 * tt + r;
        bool live = true;
        if constexpr (MODE == kModeCodes) {
          plane += 64 * NW * chunk;
          live = plane < LP;
        }
        const uint16_t* wr = W + (int64_t)(live ? plane : 0) * kHead + 64 * half;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const uint4 v = *reinterpret_cast<const uint4*>(wr + 8 * kk);
          a[tt][kk] = live ? __builtin_bit_cast(
                                 bf16x8_t, make_uint4(v.x ^ 0x80008000u, v.y ^ 0x80008000u,
                                                      v.z ^ 0x80008000u, v.w ^ 0x80008000u))
                           : bf16x8_t{};
        }
      }
    }
  }
  if constexpr (PACKED) {  // tables no wave projects stay 0
    uint32_t* z = reinterpret_cast<uint32_t*>(stage);
    for (int i = tid; i < kTK * kStageRow; i += NW * 64) z[i] = 0u;
  }
  lds_barrier();
  if constexpr (!WIDE) {
    // One-byte IDs: a software pipeline over the tile's four 32-key blocks.
    // Block bt runs the tile-0 chain, then the tile-1 chain; the tile-0
    // accumulators are packed while the tile-1 chain runs, and the tile-1
    // accumulators while the next block's tile-0 chain runs, so the sign
    // packing and the ID stores overlap MFMAs.  The B operands of the next
    // block are read from LDS once the current tile-1 chain has taken them.
    // Bit c of a block's word = accumulator c (register c of tile 0, then of
    // tile 1); one funnel shift takes in each sign bit.
    constexpr int TL = ids_word_bytes(L8, 8);     // P = 8: one byte per table
    const int t0w = (8 * wave + 4 * half) / TL;   // first ID word of the lane's 4 tables
    auto pack16 = [](const f32x16_t& x) {
      uint32_t w = 0u;
#pragma unroll
      for (int r = 15; r >= 0; --r) w = __builtin_amdgcn_alignbit(w, __float_as_uint(x[r]), 31u);
      return w;
    };
    // register r of tile tt = plane r & 7 of table 8w + 4*half + 2*tt + (r >> 3):
    // the word holds the 4 tables 8w + 4*half .. +3 as ID bytes of the tiled layout
    // code word of the lane (CODES): its index, and the mask of its planes < LP
    const int cw = 2 * (NW * chunk + wave) + half;
    const int cbits = LP - 32 * cw;
    const uint32_t cmask = cbits >= 32 ? ~0u : cbits > 0 ? (1u << cbits) - 1u : 0u;
    uint32_t* crow = codes + ((int64_t)bh * WPK + (cw < WPK ? cw : 0)) * n_cap;
    auto store = [&](int64_t pos, uint32_t word) {
      if constexpr (MODE == kModeCodes) {
        if (cw < WPK) crow[pos] = word & cmask;
      } else if constexpr (TL == 4) {
        *reinterpret_cast<uint32_t*>(ids + ids_word_offset(bh, n_cap, TL, pos, t0w)) = word;
      } else if constexpr (TL == 2) {
        *reinterpret_cast<uint16_t*>(ids + ids_word_offset(bh, n_cap, TL, pos, t0w)) =
            (uint16_t)word;
        *reinterpret_cast<uint16_t*>(ids + ids_word_offset(bh, n_cap, TL, pos, t0w + 1)) =
            (uint16_t)(word >> 16);
      } else {
#pragma unroll
        for (int b8 = 0; b8 < 4; ++b8)
          ids[ids_word_offset(bh, n_cap, TL, pos, t0w + b8)] = (uint8_t)(word >> (8 * b8));
      }
    };
    // a codes wave whose planes are all past LP only keeps the barriers
    const bool idle = MODE == kModeCodes && 2 * (NW * chunk + wave) >= WPK;
    for (int t = 0; t < ntiles; ++t) {
      if (idle) {
        lds_barrier();
        continue;
      }
      const int64_t t0 = start + (int64_t)t * kTK;
      const uint4* kt = ktile[t & 1] + col * kRowU4 + 8 * half;
      const bool full = t0 + kTK <= end;
      bf16x8_t b[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) b[kk] = __builtin_bit_cast(bf16x8_t, kt[kk]);
      f32x16_t x0, x1;
      uint32_t lo = 0u;
#pragma unroll
      for (int bt = 0; bt < NB; ++bt) {
        x0 = f32x16_t{0};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
          x0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][kk], b[kk], x0, 0, 0, 0);
        if (bt > 0) {  // the previous block's tile-1 half, then its word
          uint32_t w = (pack16(x1) << 16) | lo;
          asm volatile("" : "+v"(w));  // pack here, not inside the predicated store
          const int64_t pos = t0 + (bt - 1) * kBTile + col;
          if (full || pos < end) store(pos, w);
        }
        x1 = f32x16_t{0};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
          x1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][kk], b[kk], x1, 0, 0, 0);
        lo = pack16(x0);
        if (bt + 1 < NB) {
#pragma unroll
          for (int kk = 0; kk < 8; ++kk)
            b[kk] = __builtin_bit_cast(bf16x8_t, kt[(bt + 1) * kBTile * kRowU4 + kk]);
        }
      }
      {
        uint32_t w = (pack16(x1) << 16) | lo;
        asm volatile("" : "+v"(w));
        const int64_t pos = t0 + (NB - 1) * kBTile + col;
        if (full || pos < end) store(pos, w);
      }
      lds_barrier();  // the ID stores stay in flight
    }
    return;
  }
  // Packed words: the consumers write their IDs into the tile's stage, and
  // after the tile's barrier turn the previous tile's stage into whole words
  // (one word a thread: key kl = i / 16, word j = i % 16).
  auto pack_tile = [&](int tp) {
    const uint16_t* st = stage + (tp & 1) * kTK * kStageRow;
    const int64_t t0p = start + (int64_t)tp * kTK;
    for (int i = wave * 64 + lane; i < kTK * 16; i += NW * 64) {
      const int kl = i >> 4, j = i & 15;
      const int64_t pos = t0p + kl;
      if (pos < end) {
        const uint2 c = *reinterpret_cast<const uint2*>(st + kl * kStageRow + 4 * j);
        const uint64_t w = (uint64_t)(c.x & 0xFFFFu) | ((uint64_t)(c.x >> 16) << 10) |
                           ((uint64_t)(c.y & 0xFFFFu) << 20) | ((uint64_t)(c.y >> 16) << 30);
        ids_store_word(ids, bh, n_cap, Lw, 10, pos, j, w);
      }
    }
  };
  for (int t = 0; t < ntiles; ++t) {
    const int64_t t0 = start + (int64_t)t * kTK;
    const uint4* kt = ktile[t & 1];
    if constexpr (PACKED) {
      if (t > 0) pack_tile(t - 1);
    }
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) {
      f32x16_t acc0 = {0}, acc1 = {0};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const uint4 bv = kt[(bt * kBTile + col) * kRowU4 + 8 * half + kk];
        const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, bv);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][kk], bop, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][kk], bop, acc1, 0, 0, 0);
      }
      const int64_t pos = t0 + bt * kBTile + col;
      // a plane is set when its float bits, read as an int, clamp to 1 in [0, 1]
      uint32_t id0 = 0u, id1 = 0u, id2 = 0u;
#pragma unroll
      for (int c = 0; c < 30; ++c) {
        const float v = c < 16 ? acc0[c] : acc1[c - 16];
        const uint32_t bit = (uint32_t)min(max(__float_as_int(v), 0), 1) << (c % 10);
        if (c < 10) id0 |= bit;
        else if (c < 20) id1 |= bit;
        else id2 |= bit;
      }
      if constexpr (PACKED) {
        uint16_t* st = stage + (t & 1) * kTK * kStageRow + (bt * kBTile + col) * kStageRow;
        const int tb = 6 * wave + 3 * half;
        if (tb < 64) st[tb] = (uint16_t)id0;
        if (tb + 1 < 64) st[tb + 1] = (uint16_t)id1;
        if (tb + 2 < 64) st[tb + 2] = (uint16_t)id2;
      } else if (pos < end) {
        store_wide(ids, bh, n_cap, pos, Lw, 6 * wave + 3 * half, id0, id1, id2,
                   wave == 0 && half == 0);
      }
    }
    lds_barrier();  // the ID stores stay in flight
  }
  if constexpr (PACKED) pack_tile(ntiles - 1);  // complete: the loop ended on a barrier
}

// ---------------------------------------------------------------- launcher

hipError_t launch_hash_keys(const void* K, const void* V, int dtype, int B, int Hkv,
                            int64_t n_cap, const int32_t* pos0, int count, const void* W, int L,
                            int P, uint8_t* ids, float* vnorm, hipStream_t s) {
  if (count <= 0 || B <= 0 || Hkv <= 0) return hipSuccess;
  const int64_t rows = (int64_t)B * Hkv * count;
  const bool bf16 = dtype == 1;
  if (!ids) {  // value norms only
    const unsigned grid = (unsigned)((rows + kNormThreads / 16 - 1) / (kNormThreads / 16));
    if (bf16)
      value_norms_kernel<uint16_t><<<grid, kNormThreads, 0, s>>>(
          static_cast<const uint16_t*>(V), Hkv, n_cap, pos0, count, rows, vnorm);
    else
      value_norms_kernel<float><<<grid, kNormThreads, 0, s>>>(
          static_cast<const float*>(V), Hkv, n_cap, pos0, count, rows, vnorm);
    return hipGetLastError();
  }
  // the MFMA path covers every ID word when L is 16, 32 or 64
  const bool mfma_ok = bf16 && P == 8 && (L == 16 || L == 32 || L == 64) && count >= 64;
  const bool wide_ok = bf16 && P == 10 && L <= 64 && count >= 64;
  if (mfma_ok || wide_ok) {
    // about one workgroup per CU, each streaming a contiguous key range
    int64_t nblk = (256 + (int64_t)B * Hkv - 1) / ((int64_t)B * Hkv);
    int64_t kpb = ((count + nblk - 1) / nblk + 127) / 128 * 128;
    nblk = (count + kpb - 1) / kpb;
    const dim3 grid((unsigned)(B * Hkv * nblk));
    const uint16_t* Kb = static_cast<const uint16_t*>(K);
    const uint16_t* Vb = static_cast<const uint16_t*>(V);
    const uint16_t* Wb = static_cast<const uint16_t*>(W);
    auto go = [&](auto nw, auto wide) {
      constexpr int NW = decltype(nw)::value;
      constexpr int MODE = decltype(wide)::value == 2 ? kModeIds10P
                           : decltype(wide)::value == 1 ? kModeIds10 : kModeIds8;
      if (vnorm)
        hash_mfma_kernel<NW, MODE, true><<<grid, (NW + kProd) * 64, 0, s>>>(
            Kb, Vb, Hkv, n_cap, pos0, count, Wb, L, ids, vnorm, (int)kpb, (int)nblk, nullptr, 0,
            0, 1);
      else
        hash_mfma_kernel<NW, MODE, false><<<grid, (NW + kProd) * 64, 0, s>>>(
            Kb, Vb, Hkv, n_cap, pos0, count, Wb, L, ids, vnorm, (int)kpb, (int)nblk, nullptr, 0,
            0, 1);
    };
    using N = std::integral_constant<int, 0>;  // one-byte IDs
    using Y = std::integral_constant<int, 1>;  // two-byte IDs
    using Q = std::integral_constant<int, 2>;  // packed ten-bit IDs
    if (mfma_ok) {
      switch (L) {
        case 16: go(std::integral_constant<int, 2>{}, N{}); break;
        case 32: go(std::integral_constant<int, 4>{}, N{}); break;
        default: go(std::integral_constant<int, 8>{}, N{}); break;
      }
    } else if (!ids_packed(L, P)) {  // six 10-plane tables per consumer wave
      const int nw = (L + 5) / 6;
      if (nw <= 2) go(std::integral_constant<int, 2>{}, Y{});
      else if (nw <= 4) go(std::integral_constant<int, 4>{}, Y{});
      else go(std::integral_constant<int, 6>{}, Y{});
    } else {
      const int nw = (L + 5) / 6;  // 6 .. 11
      if (nw <= 6) go(std::integral_constant<int, 6>{}, Q{});
      else if (nw <= 8) go(std::integral_constant<int, 8>{}, Q{});
      else if (nw <= 10) go(std::integral_constant<int, 10>{}, Q{});
      else go(std::integral_constant<int, 11>{}, Q{});
    }
    return hipGetLastError();
  }
  // words per slice: the largest power of two with WPB * TL * P <= 64 planes
  const int TL = ids_tables_per_word(L);
  const int C = ids_cell_bytes(P);
  int WPB = 16;
  while (WPB > 1 && WPB * TL * P > kGenThreads) WPB >>= 1;
  const int S = 16 / WPB;
  const dim3 grid((unsigned)(rows * S));
  if (bf16)
    hash_generic_kernel<uint16_t><<<grid, kGenThreads, 0, s>>>(
        static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V), Hkv, n_cap, pos0, count,
        static_cast<const uint16_t*>(W), L, P, TL, C, WPB, S, ids, vnorm);
  else
    hash_generic_kernel<float><<<grid, kGenThreads, 0, s>>>(
        static_cast<const float*>(K), static_cast<const float*>(V), Hkv, n_cap, pos0, count,
        static_cast<const float*>(W), L, P, TL, C, WPB, S, ids, vnorm);
  return hipGetLastError();
}

// Hard-LSH sign codes of bf16 keys on the MFMA path: plane chunks of at most
// 16 code words (8 consumer waves), about one workgroup per CU in all.
hipError_t launch_hash_codes_mfma(const uint16_t* K, const uint16_t* V, int B, int Hkv,
                                  int64_t n_cap, const int32_t* pos0, int count,
                                  const uint16_t* W, int LP, int WPK, uint32_t* codes,
                                  float* vnorm, hipStream_t s) {
  const int waves = (WPK + 1) / 2;  // consumer waves over all chunks
  const int chunks = (waves + 7) / 8;
  const int per = (waves + chunks - 1) / chunks;
  const int64_t heads = (int64_t)B * Hkv;
  int64_t nblk = (256 + heads * chunks - 1) / (heads * chunks);
  int64_t kpb = ((count + nblk - 1) / nblk + 127) / 128 * 128;
  nblk = (count + kpb - 1) / kpb;
  const dim3 grid((unsigned)(chunks * heads * nblk));
  auto go = [&](auto nw) {
    constexpr int NW = decltype(nw)::value;
    hash_mfma_kernel<NW, kModeCodes, true><<<grid, (NW + kProd) * 64, 0, s>>>(
        K, V, Hkv, n_cap, pos0, count, W, 0, nullptr, vnorm, (int)kpb, (int)nblk, codes, LP, WPK,
        chunks);
  };
  if (per <= 2) go(std::integral_constant<int, 2>{});
  else if (per <= 4) go(std::integral_constant<int, 4>{});
  else if (per <= 5) go(std::integral_constant<int, 5>{});
  else if (per <= 6) go(std::integral_constant<int, 6>{});
  else go(std::integral_constant<int, 8>{});
  return hipGetLastError();
}

}  // namespace socketlsh
