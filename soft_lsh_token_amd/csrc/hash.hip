// Key hashing and value norms (SOCKET Sec. 4.1, Algorithm 1: one bucket per
// table per key from L random projections, cached with the value norms;
// Appendix B.2: the bucket ID is the sign pattern of W^(l) k).
//
// Two projection paths:
//  * hash_mfma_kernel: bf16 keys, P = 8, L in {16, 32, 64}.  The projection
//    Z = W K^T is a bf16 MFMA GEMM (v_mfma_f32_32x32x16_bf16, fp32
//    accumulation).  W stays in registers for the whole workgroup (each wave
//    owns 8 tables = 64 planes = two 32-row MFMA tiles); 32-key tiles of K
//    pass through LDS.  The planes of each 32-row tile are ordered so that
//    every lane's accumulators hold complete tables, which turns the sign
//    test + bit packing into lane-local work and one 32-bit store.  The value
//    rows of the same keys stream through the tile loop for their norms.
//  * hash_generic_kernel: any dtype, P <= 8, any L; one-wave workgroups,
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
    int WPB, int S, uint8_t* __restrict__ ids, float* __restrict__ vnorm) {
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
  if (lane < 16) load8<T>(K + row * kHead + 8 * lane, kf + 8 * lane);
  if (s == 0 && lane >= 16 && lane < 32) load8<T>(V + row * kHead + 8 * (lane - 16), vf);
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
  if (s == 0) {  // value norm: lanes 16..31 form one DPP row
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(vf[i], vf[i], ss);
    ss = row16_sum(ss);
    if (lane == 16) vnorm[row] = sqrtf(ss);
  }
  if (lane < WPB) {
    const int word = s * WPB + lane;
    uint64_t w = 0;
    for (int b8 = 0; b8 < TL; ++b8) {
      const int t = word * TL + b8;  // table
      if (t < L) w |= ((m >> ((lane * TL + b8) * P)) & ((1ull << P) - 1ull)) << (8 * b8);
    }
    uint8_t* dst = ids + ids_word_offset(bh, n_cap, L, pos, word);
    if (TL == 1) *dst = (uint8_t)w;
    else if (TL == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w;
    else if (TL == 4) *reinterpret_cast<uint32_t*>(dst) = (uint32_t)w;
    else *reinterpret_cast<uint2*>(dst) = make_uint2((uint32_t)w, (uint32_t)(w >> 32));
  }
}

// ---------------------------------------------------------------- MFMA path

constexpr int kTileKeys = 32;
constexpr int kRowU4 = 17;  // K rows in LDS padded to 272 B: 16 consecutive keys hit 16 bank groups

// Block = NW waves, NW = L / 8; wave w owns tables [8w, 8w+8).
// grid: B*Hkv*nblk blocks; block blk hashes keys [pos0 + blk*kpb, +kpb) of (b, h).
template <int NW>
__global__ __launch_bounds__(NW * 64) void hash_mfma_kernel(const uint16_t* __restrict__ K,
                                                            const uint16_t* __restrict__ V,
                                                            int Hkv, int64_t n_cap,
                                                            const int32_t* __restrict__ pos0,
                                                            int count,
                                                            const uint16_t* __restrict__ W,
                                                            uint8_t* __restrict__ ids,
                                                            float* __restrict__ vnorm, int kpb,
                                                            int nblk) {
  constexpr int L = NW * 8;
  const int blk = blockIdx.x % nblk;
  const int bh = blockIdx.x / nblk;
  const int b = bh / Hkv;
  const int64_t first = (int64_t)pos0[b];
  const int64_t start = first + (int64_t)blk * kpb;
  int64_t end = first + count;
  if (end > n_cap) end = n_cap;
  if (end > start + kpb) end = start + kpb;
  if (start >= end || start < 0) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int half = lane >> 5;  // A/B operand: which 8 k-slots; C: which row quartet
  const int col = lane & 31;

  // W-stationary A operands.  MFMA k-slot (8*half + i) of step kk is element
  // d = 64*half + 8*kk + i (the same map is used for K below).
  bf16x8_t a[2][8];
  {
    const int R = col;  // A row held by this lane
    const int hout = (R >> 2) & 1;
    const int r = ((R >> 3) << 2) | (R & 3);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int table = 8 * wave + 4 * hout + 2 * tt + (r >> 3);
      const int plane = r & 7;
      const uint16_t* wr = W + ((int64_t)(table * 8 + plane)) * kHead + 64 * half;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) a[tt][kk] = *reinterpret_cast<const bf16x8_t*>(wr + 8 * kk);
    }
  }

  __shared__ uint4 ktile[kTileKeys * kRowU4];
  const uint4* K4 = reinterpret_cast<const uint4*>(K);
  const uint4* V4 = reinterpret_cast<const uint4*>(V);
  const int64_t rowbase = (int64_t)bh * n_cap;

  for (int64_t t0 = start; t0 < end; t0 += kTileKeys) {
    // K rows into LDS; V rows straight to their norms (16 lanes per row)
    for (int e = tid; e < kTileKeys * 16; e += NW * 64) {
      const int key = e >> 4, part = e & 15;
      const int64_t pos = t0 + key;
      uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = kv;
      if (pos < end) {
        kv = K4[(rowbase + pos) * 16 + part];
        vv = V4[(rowbase + pos) * 16 + part];
      }
      ktile[key * kRowU4 + part] = kv;
      float f[8];
      unpack_bf16x8(vv, f);
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss);
      ss = row16_sum(ss);
      if (part == 0 && pos < end) vnorm[rowbase + pos] = sqrtf(ss);
    }
    __syncthreads();
    f32x16_t acc0 = {0}, acc1 = {0};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const uint4 bv = ktile[col * kRowU4 + 8 * half + kk];
      const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, bv);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][kk], bop, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][kk], bop, acc1, 0, 0, 0);
    }
    __syncthreads();
    // accumulator r of tile tt holds plane (r & 7) of table 8w + 4*half + 2*tt + (r >> 3)
    uint32_t word = 0u;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      word |= (acc0[r] > 0.f ? 1u : 0u) << ((r >> 3) * 8 + (r & 7));
      word |= (acc1[r] > 0.f ? 1u : 0u) << (16 + (r >> 3) * 8 + (r & 7));
    }
    // the 4 tables 8w + 4*half .. +3 of key pos, as IDs words of the tiled layout
    const int64_t pos = t0 + col;
    if (pos < end) {
      constexpr int TL = ids_word_bytes(L);
      const int t0w = (8 * wave + 4 * half) / TL;  // first word index
      if constexpr (TL == 4) {
        *reinterpret_cast<uint32_t*>(ids + ids_word_offset(bh, n_cap, L, pos, t0w)) = word;
      } else if constexpr (TL == 2) {
        *reinterpret_cast<uint16_t*>(ids + ids_word_offset(bh, n_cap, L, pos, t0w)) =
            (uint16_t)word;
        *reinterpret_cast<uint16_t*>(ids + ids_word_offset(bh, n_cap, L, pos, t0w + 1)) =
            (uint16_t)(word >> 16);
      } else {
#pragma unroll
        for (int b8 = 0; b8 < 4; ++b8)
          ids[ids_word_offset(bh, n_cap, L, pos, t0w + b8)] = (uint8_t)(word >> (8 * b8));
      }
    }
  }
}

// ---------------------------------------------------------------- launcher

hipError_t launch_hash_keys(const void* K, const void* V, int dtype, int B, int Hkv,
                            int64_t n_cap, const int32_t* pos0, int count, const void* W, int L,
                            int P, uint8_t* ids, float* vnorm, hipStream_t s) {
  if (count <= 0 || B <= 0 || Hkv <= 0) return hipSuccess;
  const int64_t rows = (int64_t)B * Hkv * count;
  const bool bf16 = dtype == 1;
  // the MFMA path covers every ID word when L is 16, 32 or 64
  const bool mfma_ok = bf16 && P == 8 && (L == 16 || L == 32 || L == 64) && count >= 64;
  if (mfma_ok) {
    const int kpb = 1024;
    const int nblk = (count + kpb - 1) / kpb;
    const dim3 grid((unsigned)(B * Hkv * nblk));
    const uint16_t* Kb = static_cast<const uint16_t*>(K);
    const uint16_t* Vb = static_cast<const uint16_t*>(V);
    const uint16_t* Wb = static_cast<const uint16_t*>(W);
    switch (L) {
      case 16: hash_mfma_kernel<2><<<grid, 128, 0, s>>>(Kb, Vb, Hkv, n_cap, pos0, count, Wb, ids, vnorm, kpb, nblk); break;
      case 32: hash_mfma_kernel<4><<<grid, 256, 0, s>>>(Kb, Vb, Hkv, n_cap, pos0, count, Wb, ids, vnorm, kpb, nblk); break;
      default: hash_mfma_kernel<8><<<grid, 512, 0, s>>>(Kb, Vb, Hkv, n_cap, pos0, count, Wb, ids, vnorm, kpb, nblk); break;
    }
    return hipGetLastError();
  }
  // words per slice: the largest power of two with WPB * TL * P <= 64 planes
  const int TL = ids_word_bytes(L);
  int WPB = 16;
  while (WPB > 1 && WPB * TL * P > kGenThreads) WPB >>= 1;
  const int S = 16 / WPB;
  const dim3 grid((unsigned)(rows * S));
  if (bf16)
    hash_generic_kernel<uint16_t><<<grid, kGenThreads, 0, s>>>(
        static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V), Hkv, n_cap, pos0, count,
        static_cast<const uint16_t*>(W), L, P, TL, WPB, S, ids, vnorm);
  else
    hash_generic_kernel<float><<<grid, kGenThreads, 0, s>>>(
        static_cast<const float*>(K), static_cast<const float*>(V), Hkv, n_cap, pos0, count,
        static_cast<const float*>(W), L, P, TL, WPB, S, ids, vnorm);
  return hipGetLastError();
}

}  // namespace socketlsh
