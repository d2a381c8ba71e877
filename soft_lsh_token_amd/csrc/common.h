// Device helpers shared by the SOCKET kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace socketlsh {

constexpr int kHead = 128;       // supported head dimension
constexpr int kHistBins = 1024;  // first top-k digit: float bits >> 21 (non-negative floats)
constexpr int kHistShift = 21;
constexpr int kXcds = 8;         // workgroup i of a dispatch runs on XCD i mod 8
constexpr int kSplitKeys = 64;   // idx entries per split of the split-k attention
constexpr int kPartStride = kHead + 2;  // a split's partial: o[kHead], m, l

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Bucket-ID cache layout.  Each table's ID is a cell of C bytes (C = 1 for
// P <= 8, 2 for P <= 10).  The IDs of one key are cut into 16 words of T
// tables (word j = tables j*T .. j*T+T-1; tables >= L read as 0), T the
// smallest power of two with 16*T >= L, so a word is WB = T*C bytes.  Keys
// are tiled in groups of 64.  Inside a group, word j of key t = 16*kg + x
// belongs to scorer lane 16*kg + j in round r = (x - j) mod 16 and is stored
// at word slot
//   (r / R) * 64 * R + (16*kg + j) * R + r % R,   R = 16 / WB,
// so that a lane's words of R consecutive rounds form one 16-byte vector and
// a wave's 16-byte loads read 1 KiB contiguously.
//
// Packed words (P = 9 or 10 with 33 <= L <= 64, so T = 4): ten-bit cells,
// cell m of word j at bits 10m .. 10m+9 of a 40-bit value, 80 bytes a key.
// A lane's 16 words are five 16-byte vectors of the group's 5 KiB slab,
// vector v at byte v*1024 + 16*lane: vectors 0..3 hold the low 32 bits of
// rounds 4v .. 4v+3, vector 4 the high byte of round r at byte r.
__host__ __device__ constexpr int ids_tables_per_word(int L) {
  return L <= 16 ? 1 : L <= 32 ? 2 : L <= 64 ? 4 : 8;
}
__host__ __device__ constexpr int ids_cell_bytes(int P) { return P > 8 ? 2 : 1; }
__host__ __device__ constexpr int ids_word_bytes(int L, int P) {
  return ids_tables_per_word(L) * ids_cell_bytes(P);
}
__host__ __device__ constexpr bool ids_packed(int L, int P) {
  return P > 8 && ids_tables_per_word(L) == 4;
}
// bit offset of cell m inside a word is m * ids_cell_bits
__host__ __device__ constexpr int ids_cell_bits(int L, int P) {
  return ids_packed(L, P) ? 10 : 8 * ids_cell_bytes(P);
}
__host__ __device__ constexpr int ids_key_bytes(int L, int P) {
  return ids_packed(L, P) ? 80 : 16 * ids_word_bytes(L, P);
}
// 16-byte vectors of one scorer lane per 64-key group (the group's slab is
// 1024 * this many bytes)
__host__ __device__ constexpr int ids_lane_vectors(int L, int P) { return ids_key_bytes(L, P) / 16; }
__host__ __device__ inline int64_t ids_groups(int64_t n_cap) { return (n_cap + 63) / 64; }

// Byte offset of word j of key `key` of KV row bh, for WB-byte words.
__host__ __device__ inline int64_t ids_word_offset(int64_t bh, int64_t n_cap, int WB, int64_t key,
                                                   int j) {
  const int R = 16 / WB;
  const int64_t gi = key >> 6;
  const int t = (int)(key & 63), kg = t >> 4, x = t & 15;
  const int r = (x - j) & 15;
  const int slot = (r / R) * 64 * R + ((kg << 4) | j) * R + (r % R);
  return ((bh * ids_groups(n_cap) + gi) * 1024 + slot) * WB;
}

// Packed words: byte offsets of the low 32 bits and of the high byte of word
// j of key `key` of KV row bh.
__host__ __device__ inline void ids_packed_offsets(int64_t bh, int64_t n_cap, int64_t key, int j,
                                                   int64_t* lo, int64_t* hi) {
  const int64_t base = (bh * ids_groups(n_cap) + (key >> 6)) * 5120;
  const int t = (int)(key & 63), kg = t >> 4, x = t & 15;
  const int r = (x - j) & 15;
  const int lane = (kg << 4) | j;
  *lo = base + (r >> 2) * 1024 + lane * 16 + (r & 3) * 4;
  *hi = base + 4096 + lane * 16 + r;
}

// Stores word j of key `key` of KV row bh: cell m of the word at bits
// m * ids_cell_bits(L, P) of w.
__device__ inline void ids_store_word(uint8_t* ids, int64_t bh, int64_t n_cap, int L, int P,
                                      int64_t key, int j, uint64_t w) {
  if (ids_packed(L, P)) {
    int64_t lo, hi;
    ids_packed_offsets(bh, n_cap, key, j, &lo, &hi);
    *reinterpret_cast<uint32_t*>(ids + lo) = (uint32_t)w;
    ids[hi] = (uint8_t)(w >> 32);
    return;
  }
  const int WB = ids_word_bytes(L, P);  // at most 8 (T = 8 only with one-byte cells)
  uint8_t* dst = ids + ids_word_offset(bh, n_cap, WB, key, j);
  if (WB == 1) *dst = (uint8_t)w;
  else if (WB == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w;
  else if (WB == 4) *reinterpret_cast<uint32_t*>(dst) = (uint32_t)w;
  else *reinterpret_cast<uint2*>(dst) = make_uint2((uint32_t)w, (uint32_t)(w >> 32));
}

// Row stride (floats) of the per-head score rows: n_cap rounded up to 64, so
// every row starts 256-byte aligned.
__host__ __device__ inline int64_t score_stride(int64_t n_cap) { return (n_cap + 63) & ~(int64_t)63; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 bf16 packed in a uint4 -> 8 floats (exact widening).
__device__ __forceinline__ void unpack_bf16x8(const uint4 v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// Load 8 consecutive head elements [8*j, 8*j+8) of a row as floats (bf16
// rows are passed as uint16_t).
template <typename T>
__device__ __forceinline__ void load_row8(const T* row, int j, float* f);
template <>
__device__ __forceinline__ void load_row8<uint16_t>(const uint16_t* row, int j, float* f) {
  const uint4 v = reinterpret_cast<const uint4*>(row)[j];
  unpack_bf16x8(v, f);
}
template <>
__device__ __forceinline__ void load_row8<float>(const float* row, int j, float* f) {
  const float4 a = reinterpret_cast<const float4*>(row)[2 * j];
  const float4 b = reinterpret_cast<const float4*>(row)[2 * j + 1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// The same 8 elements kept packed (bf16: one 16-byte vector; fp32: two) so
// that many rows can be in flight in few registers; unpack when used.
template <typename T>
struct Row8 {
  uint4 a, b;  // fp32: a, b = elements 0..3, 4..7
};
template <>
struct Row8<uint16_t> {
  uint4 a;
};
template <typename T>
__device__ __forceinline__ Row8<T> fetch_row8(const T* row, int j) {
  Row8<T> r;
  if constexpr (sizeof(T) == 2) {
    r.a = reinterpret_cast<const uint4*>(row)[j];
  } else {
    r.a = reinterpret_cast<const uint4*>(row)[2 * j];
    r.b = reinterpret_cast<const uint4*>(row)[2 * j + 1];
  }
  return r;
}
template <typename T>
__device__ __forceinline__ void unpack_row8(const Row8<T>& r, float* f) {
  if constexpr (sizeof(T) == 2) {
    unpack_bf16x8(r.a, f);
  } else {
    f[0] = __uint_as_float(r.a.x); f[1] = __uint_as_float(r.a.y);
    f[2] = __uint_as_float(r.a.z); f[3] = __uint_as_float(r.a.w);
    f[4] = __uint_as_float(r.b.x); f[5] = __uint_as_float(r.b.y);
    f[6] = __uint_as_float(r.b.z); f[7] = __uint_as_float(r.b.w);
  }
}

// DPP move within rows of 16 lanes (row_ror:n is control 0x120 + n).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// Workgroup barrier that orders LDS only: waits for this wave's own LDS
// operations, then s_barrier.  Unlike __syncthreads() it does not wait for
// outstanding global loads and stores, so prefetches stay in flight across
// it.  Use only where the barrier protects LDS data.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP only: shifts by
// 1, 2, 4, 8 inside each 16-lane row, then row_bcast:15 adds row r's total to
// rows 1 and 3 and row_bcast:31 adds rows 0-1's total to rows 2 and 3.
// Lanes without a source read 0 (`old`).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// The same inclusive prefix sum for floats, in the same fixed order (so any
// two waves that scan the same values get the same sums bit for bit).
__device__ __forceinline__ float wave_incl_scan_f32(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xA, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xC, 0xF, false));
  return x;
}

// OR over each group of 8 lanes (quad swaps, then the mirror inside each
// half row, which pairs lane i with lane 7 - i of the other quad).
__device__ __forceinline__ uint32_t or8_lanes(uint32_t x) {
  x |= dpp_u32<0xB1>(x);   // quad_perm [1,0,3,2]
  x |= dpp_u32<0x4E>(x);   // quad_perm [2,3,0,1]
  x |= dpp_u32<0x141>(x);  // row_half_mirror
  return x;
}

// Butterfly sum over each row of 16 lanes; every lane of the row gets the
// same total (each level adds the same two operands in every lane).
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0x128>(x);
  x += dpp_f32<0x124>(x);
  x += dpp_f32<0x122>(x);
  x += dpp_f32<0x121>(x);
  return x;
}

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f32<0x128>(x));
  x = fmaxf(x, dpp_f32<0x124>(x));
  x = fmaxf(x, dpp_f32<0x122>(x));
  x = fmaxf(x, dpp_f32<0x121>(x));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ uint64_t lanemask_lt64() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace socketlsh
