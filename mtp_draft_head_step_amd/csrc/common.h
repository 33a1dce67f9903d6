// Device helpers shared by the gfx950 kernels: bf16 conversion, wave64
// reductions, orderable argmax keys, the RoPE angle.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

constexpr int kWave = 64;
constexpr int MTP_MAX_DRAFT_DEV = 16;  // drafts per verify (host bound in the ABI)

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Round to nearest, ties to even (NaN -> quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum(v, kWave); }
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// DPP move of v (lanes without a source read 0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xF, false));
}

// Sum over aligned groups of `width` lanes (8, 16, 32 or 64) with DPP row
// operations; the group's total is valid in its LAST lane only.
__device__ __forceinline__ float group_sum_last(float v, int width) {
  v += dpp_mov<0xB1, 0xF>(v);                      // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E, 0xF>(v);                      // quad_perm [2,3,0,1]
  v += dpp_mov<0x114, 0xF>(v);                     // row_shr:4
  if (width >= 16) v += dpp_mov<0x118, 0xF>(v);    // row_shr:8
  if (width >= 32) v += dpp_mov<0x142, 0xA>(v);    // row_bcast:15 into rows 1, 3
  if (width >= 64) v += dpp_mov<0x143, 0xC>(v);    // row_bcast:31 into rows 2, 3
  return v;
}

// Sum over aligned groups of `width` lanes (8, 16, 32 or 64), valid in EVERY
// lane of the group, bit-identical across the group (each step adds a lane's
// value to its partner's, whose own step adds the same two numbers): xor 1 and
// xor 2 by quad permutes, then the 8- and 16-lane mirrors (DPP, no LDS
// traffic), then xor 16 by a swizzle and xor 32 by a lane permute.
template <int CTRL>
__device__ __forceinline__ float dpp_all(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// The value of lane ^ O (O = 1, 2, 4, 8, 16 by a bit-mode swizzle within each
// 32 lanes; O = 32 by a lane permute).
template <int O>
__device__ __forceinline__ float xor_lane(float v) {
  if constexpr (O == 32) {
    return __shfl_xor(v, 32, kWave);
  } else {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x1F | (O << 10)));
  }
}

__device__ __forceinline__ float group_sum_all(float v, int width) {
  v += dpp_all<0xB1>(v);                           // quad_perm [1,0,3,2]
  v += dpp_all<0x4E>(v);                           // quad_perm [2,3,0,1]
  v += dpp_all<0x141>(v);                          // row_half_mirror: the other quad of the 8
  if (width >= 16) v += dpp_all<0x140>(v);         // row_mirror: the other 8 of the 16
  if (width >= 32)                                 // xor 16 within each 32 (bit-mode swizzle)
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  if (width >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// 16-byte streaming load: a non-temporal hint for data read once (weights), so
// it does not displace reusable lines from the caches.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// cos and sin of the RoPE angle pos * theta^(-2i/D): the angle is formed and
// reduced to [-pi, pi] in fp64 (positions reach 2^20), then fp32 sincos.
// l2t = log2(theta) in fp64.
__device__ __forceinline__ void rope_cs(int pos, int i, int D, double l2t, float& c, float& s) {
  const double inv_freq = exp2(-2.0 * static_cast<double>(i) / static_cast<double>(D) * l2t);
  const double ang = static_cast<double>(pos) * inv_freq;
  const double two_pi = 6.283185307179586476925286766559;
  const double r = fma(-rint(ang * (1.0 / two_pi)), two_pi, ang);
  sincosf(static_cast<float>(r), &s, &c);
}

// Monotone map float -> uint32 (larger float, larger key); -0 is folded into +0.
__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// Argmax key: maximum value first, then the LOWEST index.
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t idx) {
  return (static_cast<unsigned long long>(ord_key(v)) << 32) | (0xFFFFFFFFu - idx);
}
__device__ __forceinline__ int argmax_index(unsigned long long key) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
}
__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int o) {
  uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o, kWave);
  uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o, kWave);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}
// The value of lane ^ o for o in {1, 2, 4, 8, 16, 32}, 32-bit: xor 1 and 2 by
// quad permutes, xor 4 and 8 by DPP row shifts (lane i reads i + o in the lower
// half of each o-pair block, i - o in the upper), xor 16 by a bit-mode swizzle,
// xor 32 by a lane permute.  o must fold to a constant.
__device__ __forceinline__ uint32_t xor_lane_u32(uint32_t v, int o, int lane) {
  const int x = static_cast<int>(v);
  switch (o) {
    case 1: return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
    case 2: return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
    case 4: {
      const int up = __builtin_amdgcn_update_dpp(0, x, 0x104, 0xF, 0xF, false);     // row_shl:4
      const int dn = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);     // row_shr:4
      return static_cast<uint32_t>((lane & 4) ? dn : up);
    }
    case 8: {
      const int up = __builtin_amdgcn_update_dpp(0, x, 0x108, 0xF, 0xF, false);     // row_shl:8
      const int dn = __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);     // row_shr:8
      return static_cast<uint32_t>((lane & 8) ? dn : up);
    }
    case 16: return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(x, 0x401F));
    default: return static_cast<uint32_t>(__shfl_xor(x, 32, kWave));
  }
}
__device__ __forceinline__ unsigned long long xor_lane_u64(unsigned long long v, int o, int lane) {
  const uint32_t lo = xor_lane_u32(static_cast<uint32_t>(v), o, lane);
  const uint32_t hi = xor_lane_u32(static_cast<uint32_t>(v >> 32), o, lane);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long w = shfl_xor_u64(v, o);
    v = w > v ? w : v;
  }
  return v;
}

// Largest key of n partial argmax keys, reduced by one workgroup (blockDim 256).
// The same maximum in two parts, so a caller can issue the key loads with its
// other entry loads: _first loads up to 4 keys per thread (strided by the block)
// and keeps their maximum; _rest adds the remaining keys and reduces over the
// block (every thread must call it).
__device__ __forceinline__ unsigned long long block_max_u64_first(const unsigned long long* parts, int n) {
  unsigned long long v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = threadIdx.x + u * static_cast<int>(blockDim.x);
    v[u] = i < n ? parts[i] : 0ull;
  }
  unsigned long long b = v[0];
#pragma unroll
  for (int u = 1; u < 4; ++u) b = v[u] > b ? v[u] : b;
  return b;
}
__device__ __forceinline__ unsigned long long block_max_u64_rest(const unsigned long long* parts, int n,
                                                                 unsigned long long b) {
  __shared__ unsigned long long s_part[4];
  for (int i = threadIdx.x + 4 * static_cast<int>(blockDim.x); i < n; i += blockDim.x) b = parts[i] > b ? parts[i] : b;
  b = wave_max_u64(b);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = b;
  __syncthreads();
  b = s_part[0];
  for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) b = s_part[w] > b ? s_part[w] : b;
  __syncthreads();
  return b;
}

__device__ __forceinline__ unsigned long long block_max_u64(const unsigned long long* parts, int n) {
  __shared__ unsigned long long s_part[4];
  unsigned long long b = 0ull;
  for (int i = threadIdx.x; i < n; i += blockDim.x) b = parts[i] > b ? parts[i] : b;
  b = wave_max_u64(b);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = b;
  __syncthreads();
  b = s_part[0];
  for (int w = 1; w < static_cast<int>(blockDim.x >> 6); ++w) b = s_part[w] > b ? s_part[w] : b;
  __syncthreads();
  return b;
}

// Draft-KV rollback of one session's state words {length, round base, -,
// error}: the new length (to_len >= 0, else the round base, plus min(k,
// n_draft - 1) accepted chained entries when `keep`), or -1 when that passes
// the current length (the caller then stores error 2).
__device__ __forceinline__ int rollback_length(int to_len, int len, int base, int k, bool keep, int n_draft) {
  int to = to_len;
  if (to_len < 0) {
    to = base;
    if (keep) {
      const int keep_max = n_draft > 0 ? n_draft - 1 : 0;
      const int kk = k < 0 ? 0 : k;
      to += kk < keep_max ? kk : keep_max;
    }
  }
  return (to < 0 || to > len) ? -1 : to;
}

}  // namespace mtp
