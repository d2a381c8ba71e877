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
//  * hash_generic_kernel: any dtype, P <= 8, any L; one workgroup per key,
//    one thread per plane.  Used for float32 keys, for odd shapes and for
//    the decode-time append of a few keys.
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

// grid: B*Hkv*count blocks (block = one key), kGenThreads threads; thread t
// projects planes t, t + kGenThreads, ...  The 128-element plane row is read
// with vector loads, all issued before the dot product.
constexpr int kGenThreads = 512;

template <typename T>
__global__ __launch_bounds__(kGenThreads) void hash_generic_kernel(
    const T* __restrict__ K, const T* __restrict__ V, int Hkv, int64_t n_cap,
    const int32_t* __restrict__ pos0, int count, const T* __restrict__ W, int L, int P,
    uint8_t* __restrict__ ids, float* __restrict__ vnorm) {
  const int c = blockIdx.x % count;
  const int bh = blockIdx.x / count;
  const int b = bh / Hkv;
  const int64_t pos = (int64_t)pos0[b] + c;
  if (pos < 0 || pos >= n_cap) return;
  const int64_t row = (int64_t)bh * n_cap + pos;
  __shared__ float kf[kHead];
  __shared__ uint32_t bits[256];
  const int tid = threadIdx.x;
  if (tid < kHead / 8) load8<T>(K + row * kHead + 8 * tid, kf + 8 * tid);
  if (tid < 256) bits[tid] = 0u;
  __syncthreads();
  const int planes = L * P;
  for (int pl = tid; pl < planes; pl += kGenThreads) {
    const T* wr = W + (int64_t)pl * kHead;
    float z = 0.f;
#pragma unroll
    for (int h0 = 0; h0 < kHead; h0 += kHead / 2) {
      float wf[kHead / 2];
#pragma unroll
      for (int t = 0; t < kHead / 2; t += 8) load8<T>(wr + h0 + t, wf + t);
#pragma unroll
      for (int t = 0; t < kHead / 2; ++t) z = fmaf(wf[t], kf[h0 + t], z);
    }
    if (z > 0.f) atomicOr(&bits[pl / P], 1u << (pl % P));
  }
  if (tid < 16) {
    float f[8];
    load8<T>(V + row * kHead + 8 * tid, f);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(f[i], f[i], ss);
    ss = row16_sum(ss);
    if (tid == 0) vnorm[row] = sqrtf(ss);
  }
  __syncthreads();
  // word j of this key: tables j*TL .. j*TL+TL-1 (0 past L), in the tiled layout
  const int TL = ids_word_bytes(L);
  if (tid < 16) {
    uint64_t w = 0;
    for (int b8 = 0; b8 < TL; ++b8) {
      const int l = tid * TL + b8;
      if (l < L) w |= (uint64_t)(bits[l] & 255u) << (8 * b8);
    }
    uint8_t* dst = ids + ids_word_offset(bh, n_cap, L, pos, tid);
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
  const dim3 grid((unsigned)rows);
  if (bf16)
    hash_generic_kernel<uint16_t><<<grid, kGenThreads, 0, s>>>(
        static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V), Hkv, n_cap, pos0, count,
        static_cast<const uint16_t*>(W), L, P, ids, vnorm);
  else
    hash_generic_kernel<float><<<grid, kGenThreads, 0, s>>>(
        static_cast<const float*>(K), static_cast<const float*>(V), Hkv, n_cap, pos0, count,
        static_cast<const float*>(W), L, P, ids, vnorm);
  return hipGetLastError();
}

}  // namespace socketlsh
