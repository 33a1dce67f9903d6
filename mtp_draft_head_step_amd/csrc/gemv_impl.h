// Weight-streaming GEMV for gfx950 (batch-1 and few-row draft steps): the
// kernel template and its launch shape.  Each gemv_*.hip file instantiates the
// launches of one weight type (and a few row counts), so the instantiations
// compile in parallel; gemv.hip holds the dispatch and the launch facts.
//
// The draft-head step reads every weight once per call (about 1 flop per byte),
// so these kernels are bound by HBM bandwidth.  Layout of the work:
//  * each weight row is split over `lpr` lanes; every lane issues 16-byte loads
//    (8 bf16 / 4 fp32 / 16 int8) and a wave keeps RPW rows x UNROLL loads in
//    flight before consuming them;
//  * the activation rows (1..16) are staged once per workgroup in LDS (fp32; bf16
//    for few-row flushes with bf16 weights, which halves LDS and raises occupancy),
//    with the producer's RMSNorm (or the embedding gather + twin RMSNorm of the
//    pair) folded into the staging, so no separate norm kernel runs;
//  * lanes of a row are reduced with xor shuffles, in a fixed order (no float
//    atomics: results are bit-identical run to run);
//  * epilogues fuse the residual add, SwiGLU (gate and up rows of the same index
//    are paired in one wave) and the logits argmax (packed 64-bit key: max value
//    then lowest index; one key per workgroup, merged by the finishing kernel).
//  * no workgroup waits for or signals another: on gfx950 a device-scope fence
//    writes back and invalidates the XCD's L2, which costs far more than the
//    extra one-workgroup kernel that merges the partial keys.
#pragma once
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mtp {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 4;   // 16-byte loads per slot in flight
constexpr int kMaxLds = 144 * 1024;   // dynamic LDS a GEMV may ask for

template <int WT> struct WTraits;
template <> struct WTraits<W_F32> { static constexpr int EPC = 4; };
template <> struct WTraits<W_BF16> { static constexpr int EPC = 8; };
template <> struct WTraits<W_I8> { static constexpr int EPC = 16; };

__device__ __forceinline__ float load_val(const void* p, size_t i, int bf16) {
  return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

template <int WT>
__device__ __forceinline__ float dot_chunk(const uint4& w, const float* __restrict__ xp) {
  float s = 0.f;
  if constexpr (WT == W_F32) {
    const float4 x = *reinterpret_cast<const float4*>(xp);
    s = __uint_as_float(w.x) * x.x + __uint_as_float(w.y) * x.y + __uint_as_float(w.z) * x.z +
        __uint_as_float(w.w) * x.w;
  } else if constexpr (WT == W_BF16) {
    const float4 x0 = *reinterpret_cast<const float4*>(xp);
    const float4 x1 = *reinterpret_cast<const float4*>(xp + 4);
    s = __uint_as_float(w.x << 16) * x0.x + __uint_as_float(w.x & 0xFFFF0000u) * x0.y +
        __uint_as_float(w.y << 16) * x0.z + __uint_as_float(w.y & 0xFFFF0000u) * x0.w +
        __uint_as_float(w.z << 16) * x1.x + __uint_as_float(w.z & 0xFFFF0000u) * x1.y +
        __uint_as_float(w.w << 16) * x1.z + __uint_as_float(w.w & 0xFFFF0000u) * x1.w;
  } else {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 x = *reinterpret_cast<const float4*>(xp + 4 * q);
      const int32_t v = static_cast<int32_t>(ws[q]);
      s += static_cast<float>((v << 24) >> 24) * x.x + static_cast<float>((v << 16) >> 24) * x.y +
           static_cast<float>((v << 8) >> 24) * x.z + static_cast<float>(v >> 24) * x.w;
    }
  }
  return s;
}

// 16 bytes of bf16 weights times 8 bf16 inputs staged in LDS: four packed
// bf16 dot products (v_dot2_f32_bf16, fp32 accumulation).
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot_chunk_bb(const uint4& w, const uint16_t* __restrict__ xp) {
  const uint4 x = *reinterpret_cast<const uint4*>(xp);
  float d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, x.x),
                                            0.f, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, x.y), d, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, x.z), d, false);
  d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, x.w), d, false);
  return d;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// 4 consecutive elements (bf16 or fp32) as fp32.
__device__ __forceinline__ float4 load4(const void* p, size_t i, int bf16) {
  if (bf16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
  }
  return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
}

// Stage dst[k - k0] = src[off + k] * nw[noff + k] (nw may be null: factor 1)
// for k in [kb, ke), 4 values per thread per step and up to 8 steps of loads in
// flight, and add the sum of squares of the src values to ss.
template <bool XB>
__device__ __forceinline__ void stage_range(void* dst, const void* src, long long off, int src_bf16,
                                            const void* nw, long long noff, int nw_bf16, int kb, int ke,
                                            int k0, float& ss) {
  constexpr int kB = 8;
  for (int base = kb + threadIdx.x * 4; base < ke; base += kB * kThreads * 4) {
    float4 xv[kB], wv[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int k = base + u * kThreads * 4;
      if (k < ke) {
        xv[u] = load4(src, static_cast<size_t>(off + k), src_bf16);
        wv[u] = nw ? load4(nw, static_cast<size_t>(noff + k), nw_bf16) : make_float4(1.f, 1.f, 1.f, 1.f);
      }
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int k = base + u * kThreads * 4;
      if (k < ke) {
        const float4 x = xv[u], w = wv[u];
        ss += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
        if constexpr (XB) {
          const uint32_t lo = f32_to_bf16(x.x * w.x) | (static_cast<uint32_t>(f32_to_bf16(x.y * w.y)) << 16);
          const uint32_t hi = f32_to_bf16(x.z * w.z) | (static_cast<uint32_t>(f32_to_bf16(x.w * w.w)) << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(dst) + (k - k0)) = make_uint2(lo, hi);
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(dst) + (k - k0)) =
              make_float4(x.x * w.x, x.y * w.y, x.z * w.z, x.w * w.w);
        }
      }
    }
  }
}

// One segment of a staged input row: dst[k - k0] = src[off + k] * nw[noff + k]
// for k in [kb, ke) (nw null: factor 1).
struct StageSeg {
  const void* src;
  long long off;
  const void* nw;
  long long noff;
  int kb, ke;
};

// 8 consecutive values from raw 16-byte pieces (bf16: piece 0; fp32: pieces 0, 1).
template <bool BF>
__device__ __forceinline__ void unpack8(const uint4 (&r)[2], float (&v)[8]) {
  if constexpr (BF) {
    const uint32_t w[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  } else {
    v[0] = __uint_as_float(r[0].x); v[1] = __uint_as_float(r[0].y);
    v[2] = __uint_as_float(r[0].z); v[3] = __uint_as_float(r[0].w);
    v[4] = __uint_as_float(r[1].x); v[5] = __uint_as_float(r[1].y);
    v[6] = __uint_as_float(r[1].z); v[7] = __uint_as_float(r[1].w);
  }
}

template <bool BF>
__device__ __forceinline__ void load8raw(const void* p, long long i, uint4 (&r)[2]) {
  if constexpr (BF) {
    r[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
  } else {
    r[0] = *reinterpret_cast<const uint4*>(static_cast<const float*>(p) + i);
    r[1] = *reinterpret_cast<const uint4*>(static_cast<const float*>(p) + i + 4);
  }
}

// Staging of one or two adjacent segments (A then B, B possibly empty) in one
// pass: 8 values per thread per step in 16-byte loads, KB steps of loads in
// flight.  Every workgroup of a launch stages the same row, so the launch's
// staging time follows its count of cache requests; wide loads and a single
// pass over both halves of the fc input keep that count low.  Adds the sums of
// squares of the src values of A and B to sa and sb.
template <bool XB, bool SBF, int NWK, int KB>   // NWK: 0 no norm weight, 1 bf16, 2 fp32
__device__ __forceinline__ void stage_segs(void* dst, const StageSeg& A, const StageSeg& B, int k0,
                                           float& sa, float& sb) {
  const int kb = A.kb < A.ke ? A.kb : B.kb;
  const int ke = B.kb < B.ke ? B.ke : A.ke;
  for (int base = kb + threadIdx.x * 8; base < ke; base += KB * kThreads * 8) {
    uint4 xr[KB][2], wr[KB][2];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int k = base + u * kThreads * 8;
      if (k < ke) {
        const StageSeg& S = k < A.ke ? A : B;
        load8raw<SBF>(S.src, S.off + k, xr[u]);
        if constexpr (NWK == 1) load8raw<true>(S.nw, S.noff + k, wr[u]);
        if constexpr (NWK == 2) load8raw<false>(S.nw, S.noff + k, wr[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int k = base + u * kThreads * 8;
      if (k < ke) {
        float x[8], w[8];
        unpack8<SBF>(xr[u], x);
        if constexpr (NWK == 1) unpack8<true>(wr[u], w);
        if constexpr (NWK == 2) unpack8<false>(wr[u], w);
        if constexpr (NWK == 0)
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = 1.f;
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) t += x[e] * x[e];
        if (k < A.ke) sa += t; else sb += t;
        if constexpr (XB) {
          uint32_t o[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            o[q] = f32_to_bf16(x[2 * q] * w[2 * q]) | (static_cast<uint32_t>(f32_to_bf16(x[2 * q + 1] * w[2 * q + 1])) << 16);
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(dst) + (k - k0)) = make_uint4(o[0], o[1], o[2], o[3]);
        } else {
          float* d = static_cast<float*>(dst) + (k - k0);
          *reinterpret_cast<float4*>(d) = make_float4(x[0] * w[0], x[1] * w[1], x[2] * w[2], x[3] * w[3]);
          *reinterpret_cast<float4*>(d + 4) = make_float4(x[4] * w[4], x[5] * w[5], x[6] * w[6], x[7] * w[7]);
        }
      }
    }
  }
}

// The 16-byte staging for the source / norm-weight types of a launch; false if
// the segments are not in whole, aligned 8-value groups (the caller then stages
// 4 values at a time).
template <bool XB>
__device__ __forceinline__ bool stage_wide(void* dst, const StageSeg& A, const StageSeg& B, int src_bf16,
                                           int nw_bf16, int k0, float& sa, float& sb) {
  const bool has_nw = A.nw != nullptr;
  long long al = A.off | A.kb | A.ke | k0;                       // whole 8-value groups
  uintptr_t ap = reinterpret_cast<uintptr_t>(A.src);             // 16-byte aligned bases
  if (has_nw) {
    al |= A.noff;
    ap |= reinterpret_cast<uintptr_t>(A.nw);
  }
  if (B.kb < B.ke) {
    al |= B.off | B.kb | B.ke;
    ap |= reinterpret_cast<uintptr_t>(B.src);
    if (has_nw) {
      al |= B.noff;
      ap |= reinterpret_cast<uintptr_t>(B.nw);
    }
  }
  if ((al & 7) || (ap & 15)) return false;
  if (src_bf16) {
    if (!has_nw) stage_segs<XB, true, 0, 8>(dst, A, B, k0, sa, sb);
    else if (nw_bf16) stage_segs<XB, true, 1, 8>(dst, A, B, k0, sa, sb);
    else stage_segs<XB, true, 2, 4>(dst, A, B, k0, sa, sb);
  } else {
    if (!has_nw) stage_segs<XB, false, 0, 8>(dst, A, B, k0, sa, sb);
    else if (nw_bf16) stage_segs<XB, false, 1, 6>(dst, A, B, k0, sa, sb);
    else return false;   // fp32 rows and weights: 16 bytes per request already
  }
  return true;
}

__device__ __forceinline__ float4 mul4(float4 a, float4 b, float s) {
  return make_float4(a.x * b.x * s, a.y * b.y * s, a.z * b.z * s, a.w * b.w * s);
}

// U chunks of every row slot: all loads first (unconditional, wave-uniform
// trip count), then the FMAs.  lane_row[s] points at this lane's first chunk of
// row slot s; consecutive chunks of a lane are `stride` bytes apart.
template <int RPW, int U>
__device__ __forceinline__ void gemv_load(uint4 (&w)[RPW][U], const char* const (&lane_row)[RPW], int j,
                                          int lpr) {
  const size_t stride = static_cast<size_t>(lpr) * 16;
#pragma unroll
  for (int s = 0; s < RPW; ++s)
#pragma unroll
    for (int u = 0; u < U; ++u)
      w[s][u] = load_stream16(lane_row[s] + static_cast<size_t>(j + u) * stride);
}

template <int WT, int NR, int RPW, int U, bool TWO, bool XB>
__device__ __forceinline__ void gemv_fma(float (&acc)[RPW][NR], float (&acc2)[RPW][NR],
                                         const uint4 (&w)[RPW][U], int j, int lpr,
                                         const void* __restrict__ xl, int kp,
                                         const uint16_t* const (&srow)[RPW], int g0, int split) {
  constexpr int EPC = WTraits<WT>::EPC;
  float scl[RPW][U];
  if constexpr (WT == W_I8) {
#pragma unroll
    for (int s = 0; s < RPW; ++s)
#pragma unroll
      for (int u = 0; u < U; ++u) scl[s][u] = f16_to_f32(srow[s][(g0 + (j + u) * lpr) >> 3]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    // chunks at or past `split` (in chunk units of this lane's sequence) feed acc2
    const bool second = TWO && g0 + (j + u) * lpr >= split;
#pragma unroll
    for (int s = 0; s < RPW; ++s)
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float d;
        if constexpr (XB)
          d = dot_chunk_bb(w[s][u], static_cast<const uint16_t*>(xl) + r * kp + (j + u) * lpr * EPC);
        else
          d = dot_chunk<WT>(w[s][u], static_cast<const float*>(xl) + r * kp + (j + u) * lpr * EPC);
        if constexpr (WT == W_I8) d *= scl[s][u];
        if constexpr (TWO) {          // value selects: both arrays stay in registers
          acc[s][r] += second ? 0.f : d;
          acc2[s][r] += second ? d : 0.f;
        } else {
          acc[s][r] += d;
        }
      }
  }
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at dst + 16 l (dst wave-uniform).
__device__ __forceinline__ void lds_direct16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// The prefetched chunks j .. j + pf - 1 of every row slot, read back from this
// wave's LDS region (slot (s, u) at byte 1024 (s pf + u), each lane its own 16
// bytes), in the same accumulation order as the streamed path.
template <int WT, int NR, int RPW, bool TWO, bool XB>
__device__ __forceinline__ void gemv_fma_lds(float (&acc)[RPW][NR], float (&acc2)[RPW][NR], const char* pfw,
                                             int pf, int lane, int j, int lpr, const void* __restrict__ xl, int kp,
                                             const uint16_t* const (&srow)[RPW], int g0, int split) {
  for (int u = 0; u < pf; ++u) {
    uint4 w[RPW][1];
#pragma unroll
    for (int s = 0; s < RPW; ++s)
      w[s][0] = *reinterpret_cast<const uint4*>(pfw + (s * pf + u) * 1024 + lane * 16);
    gemv_fma<WT, NR, RPW, 1, TWO, XB>(acc, acc2, w, j + u, lpr, xl, kp, srow, g0, split);
  }
}

template <int WT, int NR, int RPW, int U, bool TWO, bool XB>
__device__ __forceinline__ void gemv_body(float (&acc)[RPW][NR], float (&acc2)[RPW][NR],
                                          const char* const (&lane_row)[RPW], int j, int lpr,
                                          const void* __restrict__ xl, int kp,
                                          const uint16_t* const (&srow)[RPW], int g0, int split) {
  uint4 w[RPW][U];
  gemv_load<RPW, U>(w, lane_row, j, lpr);
  gemv_fma<WT, NR, RPW, U, TWO, XB>(acc, acc2, w, j, lpr, xl, kp, srow, g0, split);
}

// Row slot s of row block blk: the weight row pointer (rows past the end read
// row 0, a valid address, and are discarded), its index in its matrix, the
// int8 scale row, and whether it is valid.
template <int WT, int RPW>
__device__ __forceinline__ void gemv_rows(const GemvArgs& a, int blk, int rows_per_wg, int wave, int rps,
                                          int sub, bool swiglu, const char* (&rowp)[RPW],
                                          const uint16_t* (&srow)[RPW], int (&rowid)[RPW],
                                          bool (&valid)[RPW]) {
  constexpr int WBYTES = WT == W_F32 ? 4 : (WT == W_BF16 ? 2 : 1);
  const size_t row_bytes = static_cast<size_t>(a.K) * WBYTES;
#pragma unroll
  for (int s = 0; s < RPW; ++s) {
    int r, mat = 0;
    if (swiglu) {
      r = blk * rows_per_wg + (wave * (RPW / 2) + s / 2) * rps + sub;
      mat = s & 1;
      valid[s] = r < a.M;
    } else {
      r = blk * rows_per_wg + (wave * RPW + s) * rps + sub;
      valid[s] = r < a.M;
      if (r >= a.m[0]) { r -= a.m[0]; mat = 1; if (r >= a.m[1]) { r -= a.m[1]; mat = 2; } }
    }
    if (!valid[s]) { r = 0; mat = 0; }
    rowid[s] = r;
    rowp[s] = static_cast<const char*>(a.w[mat]) + static_cast<size_t>(r) * row_bytes;
    srow[s] = (WT == W_I8) ? a.scales + static_cast<size_t>(r) * (a.K >> 7) : nullptr;
  }
}

// WSK: the four waves of a workgroup share its rows and split each row's
// chunks between them (partial dot products summed through LDS in wave
// order), so a workgroup's row block is RPW rows and a persistent grid divides
// the rows evenly over the CUs.
template <int WT, int NR, int RPW, bool TWO, bool XB, bool WSK>
__global__ __launch_bounds__(kThreads) void k_gemv(GemvArgs a) {
  // staged inputs [NR][kp]: fp32, or bf16 when XB (few-row flushes with bf16 weights)
  extern __shared__ __attribute__((aligned(16))) float xs_f[];
  using XT = typename std::conditional<XB, uint16_t, float>::type;
  XT* xs = reinterpret_cast<XT*>(xs_f);
  __shared__ float s_red[kWaves][2 * NR];
  __shared__ float s_inv[2 * NR];
  __shared__ unsigned long long s_best[kWaves][NR];
  __shared__ float s_wsk[WSK ? kWaves : 1][WSK ? RPW * 8 * NR : 1][2];
  constexpr int EPC = WTraits<WT>::EPC;

  if (a.batch <= 1 && a.kv_state && a.kv_state[3] != 0) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;

  // the previous step's argmax merge, in every workgroup; its stores (the
  // token and the append commit, workgroup 0) wait for the kernel's end, since
  // a store this early would keep the compiler from loading the launch's
  // uniform inputs through the scalar cache
  int ftok = -1, flen = 0, fn = 0;
  if (TWO && NR == 1 && a.fin_parts) {
    flen = a.fin_state[0];
    const int nd0 = a.fin_ndev ? *a.fin_ndev : a.fin_nmax;
    unsigned long long b = block_max_u64_first(a.fin_parts, a.fin_nparts);
    b = block_max_u64_rest(a.fin_parts, a.fin_nparts, b);
    fn = min(max(nd0, 0), a.fin_nmax);
    // the same in every lane: read out as a scalar so the staging branches and
    // the embedding row address stay uniform
    if (fn > 0) ftok = __builtin_amdgcn_readfirstlane(argmax_index(b));
  }
  auto fin_commit = [&]() {
    if (TWO && NR == 1 && a.fin_parts && blockIdx.x == 0 && tid == 0) {
      if (fn > 0 && a.fin_amax) *a.fin_amax = ftok;
      a.fin_state[0] = flen + fn;
      if (a.fin_set_base) a.fin_state[1] = flen + fn;
    }
  };

  // ---- activation rows handled by this launch.  Slot r (of NR) reads
  // workspace row jr[r], token tr[r] and hidden row hr[r]; ROW_LAST outputs of
  // the hidden copy and the logits go to row orw[r]; vr[r] tells whether the
  // slot holds a row at all.  One session: rows j < n (device count), ROW_LAST
  // the row n - 1.  Several sessions: flattened rows b * n_max + j, valid when j
  // is below session b's count and its error word is clear; ROW_LAST slot r is
  // session row_base + r's last row.
  int jr[NR], tr[NR], hr[NR], orw[NR];
  bool vr[NR];
  int32_t* er[NR];
  bool any = false;
  if (a.batch <= 1) {
    int n = a.n_max;
    if (a.n_dev) n = min(max(*a.n_dev, 0), a.n_max);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int j = (a.row_sel == ROW_LAST) ? n - 1 : a.row_base + r;
      vr[r] = (a.row_sel == ROW_LAST) ? (r == 0 && n > 0) : (j < n);
      jr[r] = tr[r] = hr[r] = vr[r] ? j : 0;
      orw[r] = (a.row_sel == ROW_LAST) ? 0 : jr[r];
      er[r] = a.err;
      any = any || vr[r];
    }
  } else {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int b = (a.row_sel == ROW_LAST) ? a.row_base + r : (a.row_base + r) / a.n_max;
      int nb = 0;
      if (b < a.batch) {
        const int32_t* sb = a.kv_state + 4 * b;
        nb = sb[3] != 0 ? 0 : (a.n_dev ? min(max(a.n_dev[b * a.ndev_sb], 0), a.n_max) : a.n_max);
      }
      const int jj = (a.row_sel == ROW_LAST) ? nb - 1 : (a.row_base + r) - b * a.n_max;
      vr[r] = b < a.batch && jj >= 0 && jj < nb;
      jr[r] = vr[r] ? b * a.n_max + jj : 0;
      tr[r] = vr[r] ? b * a.tok_sb + jj : 0;
      hr[r] = vr[r] ? b * a.hid_sb + jj : 0;
      orw[r] = vr[r] ? b * a.out_sb : 0;
      er[r] = (b < a.batch) ? const_cast<int32_t*>(a.kv_state) + 4 * b + 3 : nullptr;   // the state is writable
      any = any || vr[r];
    }
  }
  if (!any) {
    if (a.out_mode == OUT_LOGITS && threadIdx.x < NR) a.amax_part[threadIdx.x * gridDim.x + blockIdx.x] = 0ull;
    fin_commit();
    return;
  }
  const int K = a.K;
  const int half = (a.in_mode == IN_EMBED) ? K / 2 : K;
  const int lpr = a.lpr;
  const int rps = kWave / lpr;          // rows per slot
  const int sub = lane / lpr;           // row within the slot
  const int li = lane % lpr;            // lane within the row
  const bool swiglu = (a.out_mode == OUT_SWIGLU);
  const int rows_per_wg = (WSK ? 1 : kWaves) * (swiglu ? RPW / 2 : RPW) * rps;
  const int nblocks = (a.M + rows_per_wg - 1) / rows_per_wg;
  const int nphase = (K + a.kp - 1) / a.kp;
  const int wrow = WSK ? 0 : wave;      // the wave's place in the row block

  // Inputs are staged as x * w_norm; the scalar 1 / rms(x) of each activation
  // row is applied to the finished dot products (it factors out), so the sum of
  // squares is reduced after the weights have been streamed, not before.  The
  // embedding-cat input has two halves with their own scales: chunks of the
  // hidden half accumulate separately (acc2).
  float ss[2 * NR];
#pragma unroll
  for (int i = 0; i < 2 * NR; ++i) ss[i] = 0.f;
  const int split_chunk = TWO ? half / EPC : 0x7FFFFFFF;
  bool have_inv = (a.in_mode == IN_F32);
  if (have_inv && tid < 2 * NR) s_inv[tid] = (tid & 1) ? 0.f : 1.f;

  unsigned long long best[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) best[r] = 0ull;

  for (int blk = blockIdx.x; blk < nblocks; blk += (a.grid_stride ? gridDim.x : nblocks)) {
    // row slots: plain mode slot s -> its row; swiglu slot pair (2p, 2p+1) -> (gate r, up r)
    const char* rowp[RPW];
    const uint16_t* srow[RPW];
    int rowid[RPW];
    bool valid[RPW];
    gemv_rows<WT, RPW>(a, blk, rows_per_wg, wrow, rps, sub, swiglu, rowp, srow, rowid, valid);

    float acc[RPW][NR], acc2[RPW][NR];   // acc2: hidden half of the embedding-cat input
#pragma unroll
    for (int s = 0; s < RPW; ++s)
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[s][r] = acc2[s][r] = 0.f;

    for (int ph = 0; ph < nphase; ++ph) {
      const int k0 = ph * a.kp;
      const int klen = min(a.kp, K - k0);
      // ---- stage this phase's inputs in LDS; a single-phase grid-stride loop
      // stages once, a multi-phase loop restages per phase
      if (blk == static_cast<int>(blockIdx.x) || nphase > 1) {
        __syncthreads();
        if constexpr (NR <= 4) {
          // the first chunks of this wave's rows go to LDS while the input is staged
          if (a.pf > 0 && blk == static_cast<int>(blockIdx.x) && nphase == 1) {
            const int cpl0 = (K / EPC) / lpr;
            const int jb = WSK ? wave * cpl0 / kWaves : 0;
            const size_t stride = static_cast<size_t>(lpr) * 16;
            char* pfw = reinterpret_cast<char*>(xs_f) + a.pf_off + wave * (RPW * a.pf * 1024);
#pragma unroll
            for (int s = 0; s < RPW; ++s) {
              const char* lr = rowp[s] + static_cast<size_t>(li) * 16;
              for (int u = 0; u < a.pf; ++u)
                lds_direct16(lr + static_cast<size_t>(jb + u) * stride, pfw + (s * a.pf + u) * 1024);
            }
          }
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          XT* dst = xs + r * a.kp;
          float se = 0.f, sh = 0.f;   // sums of squares: whole input / hidden half
          if (vr[r]) {
            if (a.in_mode != IN_EMBED) {
              const StageSeg A{a.x, static_cast<long long>(jr[r]) * a.ldx, (a.in_mode == IN_RMS) ? a.nw : nullptr,
                               0, k0, k0 + klen};
              const StageSeg B{nullptr, 0, nullptr, 0, 0, 0};
              if (WT == W_F32 || !stage_wide<XB>(dst, A, B, 0, a.nw_bf16, k0, se, sh))
                stage_range<XB>(dst, a.x, static_cast<long long>(jr[r]) * a.ldx, 0,
                            (a.in_mode == IN_RMS) ? a.nw : nullptr, 0, a.nw_bf16, k0, k0 + klen, k0, se);
            } else if (WT != W_F32 && a.embed_bf16 == a.hid_bf16 && (ftok >= 0 ? ftok : a.tok[tr[r]]) >= 0 &&
                       (ftok >= 0 ? ftok : a.tok[tr[r]]) < a.vocab_tok) {
              // both halves in one pass (the embedding and hidden rows share a type)
              const int tk = ftok >= 0 ? ftok : a.tok[tr[r]];
              const int ea = k0, eb = min(k0 + klen, half), ha = max(k0, half), hb = k0 + klen;
              const StageSeg A{a.embed, static_cast<long long>(tk) * half, a.nw, 0, ea, ea < eb ? eb : ea};
              const StageSeg B{a.hid, static_cast<long long>(hr[r]) * a.ld_hid - half, a.nw2,
                               -static_cast<long long>(half), ha, ha < hb ? hb : ha};
              if (!stage_wide<XB>(dst, A, B, a.embed_bf16, a.nw_bf16, k0, se, sh)) {
                if (ea < eb)
                  stage_range<XB>(dst, a.embed, static_cast<long long>(tk) * half, a.embed_bf16, a.nw, 0,
                              a.nw_bf16, ea, eb, k0, se);
                if (ha < hb)
                  stage_range<XB>(dst, a.hid, static_cast<long long>(hr[r]) * a.ld_hid - half, a.hid_bf16, a.nw2,
                              -static_cast<long long>(half), a.nw_bf16, ha, hb, k0, sh);
              }
            } else {
              const int ea = k0, eb = min(k0 + klen, half);
              const int tk = ftok >= 0 ? ftok : a.tok[tr[r]];
              if (tk >= 0 && tk < a.vocab_tok) {
                if (ea < eb)
                  stage_range<XB>(dst, a.embed, static_cast<long long>(tk) * half, a.embed_bf16, a.nw, 0,
                              a.nw_bf16, ea, eb, k0, se);
              } else {
                // a token outside the vocabulary: its embedding half stays zero and
                // the KV error word is set (every later kernel is then a no-op)
                for (int k = ea + tid; k < eb; k += kThreads) dst[k - k0] = XT(0);
                if (er[r] && blockIdx.x == 0 && tid == 0) *er[r] = 4;
              }
              const int ha = max(k0, half), hb = k0 + klen;
              if (ha < hb)
                stage_range<XB>(dst, a.hid, static_cast<long long>(hr[r]) * a.ld_hid - half, a.hid_bf16, a.nw2,
                            -static_cast<long long>(half), a.nw_bf16, ha, hb, k0, sh);
            }
          } else {
            for (int k = tid; k < klen; k += kThreads) dst[k] = XT(0);
          }
          ss[2 * r] += se;
          ss[2 * r + 1] += sh;
        }
        __syncthreads();
      }

      // ---- stream the weights of this phase: cpl chunks per lane (wave-uniform)
      const int cpl = (klen / EPC) / lpr;
      const char* lane_row[RPW];
#pragma unroll
      for (int s = 0; s < RPW; ++s) lane_row[s] = rowp[s] + (static_cast<size_t>(k0 / EPC) + li) * 16;
      const XT* xl = xs + li * EPC;
      const int g0 = (k0 / EPC) + li;   // chunk index of j = 0 (int8 scale groups)
      int j = WSK ? wave * cpl / kWaves : 0;
      const int je = WSK ? (wave + 1) * cpl / kWaves : cpl;
      // few-row passes keep twice the loads in flight (their staged rows cap
      // the workgroups per CU)
      constexpr int kU = NR > 1 ? 2 * kUnroll : kUnroll;
      if constexpr (NR <= 4) {
        if (a.pf > 0 && blk == static_cast<int>(blockIdx.x) && nphase == 1) {
          // the prefetched chunks; the next batch's loads go out first
          const char* pfw = reinterpret_cast<const char*>(xs_f) + a.pf_off + wave * (RPW * a.pf * 1024);
          const int jp = j + a.pf;
          if (jp + kU <= je) {
            uint4 wn[RPW][kU];
            gemv_load<RPW, kU>(wn, lane_row, jp, lpr);
            gemv_fma_lds<WT, NR, RPW, TWO, XB>(acc, acc2, pfw, a.pf, lane, j, lpr, xl, a.kp, srow, g0, split_chunk);
            gemv_fma<WT, NR, RPW, kU, TWO, XB>(acc, acc2, wn, jp, lpr, xl, a.kp, srow, g0, split_chunk);
            j = jp + kU;
          } else {
            gemv_fma_lds<WT, NR, RPW, TWO, XB>(acc, acc2, pfw, a.pf, lane, j, lpr, xl, a.kp, srow, g0, split_chunk);
            j = jp;
          }
        }
      }
      for (; j + kU <= je; j += kU)
        gemv_body<WT, NR, RPW, kU, TWO, XB>(acc, acc2, lane_row, j, lpr, xl, a.kp, srow, g0, split_chunk);
      if constexpr (kU > kUnroll)
        for (; j + kUnroll <= je; j += kUnroll)
          gemv_body<WT, NR, RPW, kUnroll, TWO, XB>(acc, acc2, lane_row, j, lpr, xl, a.kp, srow, g0, split_chunk);
      for (; j + 2 <= je; j += 2)
        gemv_body<WT, NR, RPW, 2, TWO, XB>(acc, acc2, lane_row, j, lpr, xl, a.kp, srow, g0, split_chunk);
      for (; j < je; ++j)
        gemv_body<WT, NR, RPW, 1, TWO, XB>(acc, acc2, lane_row, j, lpr, xl, a.kp, srow, g0, split_chunk);
    }

    // ---- the inverse RMS of each activation row (once, after the first block)
    if (!have_inv) {
#pragma unroll
      for (int i = 0; i < 2 * NR; ++i) {
        const float v = wave_sum(ss[i]);
        if (lane == 0) s_red[wave][i] = v;
      }
      __syncthreads();
      if (tid < 2 * NR) {
        float v = 0.f;
        for (int w = 0; w < kWaves; ++w) v += s_red[w][tid];
        // odd entries scale the hidden half, which only the embedding-cat input has
        s_inv[tid] = ((tid & 1) && a.in_mode != IN_EMBED) ? 0.f
                                                          : rsqrtf(v / static_cast<float>(half) + a.eps);
      }
      __syncthreads();
      have_inv = true;
    }

    // ---- reduce each row over its lanes (total in the row's last lane), apply
    // 1/rms, run the epilogue
#pragma unroll
    for (int s = 0; s < RPW; ++s)
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        acc[s][r] = group_sum_last(acc[s][r], lpr);
        if constexpr (TWO) acc2[s][r] = group_sum_last(acc2[s][r], lpr);
      }
    if constexpr (WSK) {
      // the waves' partial sums of each row, added in wave order
      if (li == lpr - 1) {
#pragma unroll
        for (int s = 0; s < RPW; ++s)
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            s_wsk[wave][(s * 8 + sub) * NR + r][0] = acc[s][r];
            if constexpr (TWO) s_wsk[wave][(s * 8 + sub) * NR + r][1] = acc2[s][r];
          }
      }
      __syncthreads();
      if (wave == 0 && li == lpr - 1) {
#pragma unroll
        for (int s = 0; s < RPW; ++s)
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            float v = 0.f, v2 = 0.f;
            for (int w = 0; w < kWaves; ++w) {
              v += s_wsk[w][(s * 8 + sub) * NR + r][0];
              if constexpr (TWO) v2 += s_wsk[w][(s * 8 + sub) * NR + r][1];
            }
            acc[s][r] = v;
            if constexpr (TWO) acc2[s][r] = v2;
          }
      }
      __syncthreads();   // s_wsk is rewritten by the next row block
    }
#pragma unroll
    for (int s = 0; s < RPW; ++s)
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float v = acc[s][r] * s_inv[2 * r];
        if constexpr (TWO) v += acc2[s][r] * s_inv[2 * r + 1];
        acc[s][r] = v;
      }

    if (li == lpr - 1 && (!WSK || wave == 0)) {
      if (swiglu) {
#pragma unroll
        for (int s = 0; s < RPW; s += 2) {
          if (!valid[s]) continue;
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            if (!vr[r]) continue;
            a.y[static_cast<size_t>(jr[r]) * a.ldy + rowid[s]] = silu(acc[s][r]) * acc[s + 1][r];
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < RPW; ++s) {
          if (!valid[s]) continue;
          const int row = blk * rows_per_wg + (wrow * RPW + s) * rps + sub;
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            if (!vr[r]) continue;
            const int j = jr[r];
            float v = acc[s][r];
            if (a.out_mode == OUT_LOGITS) {
              if (a.logits) a.logits[static_cast<size_t>(orw[r]) * a.M + row] = v;
              const unsigned long long key = argmax_key(v, static_cast<uint32_t>(row));
              best[r] = key > best[r] ? key : best[r];
              continue;
            }
            if (a.out_mode == OUT_RESID) v += a.res[static_cast<size_t>(j) * a.ldres + row];
            a.y[static_cast<size_t>(j) * a.ldy + row] = v;
            if (a.y2) {
              const size_t o = static_cast<size_t>(orw[r]) * a.ldy2 + row;
              if (a.y2_bf16) static_cast<uint16_t*>(a.y2)[o] = f32_to_bf16(v);
              else static_cast<float*>(a.y2)[o] = v;
            }
          }
        }
      }
    }
  }

  if (a.out_mode == OUT_LOGITS) {
    // one key per (slot, workgroup), merged per slot by the finishing kernel
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const unsigned long long b = wave_max_u64(best[r]);
      if (lane == 0) s_best[wave][r] = b;
    }
    __syncthreads();
    if (tid < NR) {
      unsigned long long b = s_best[0][tid];
      for (int w = 1; w < kWaves; ++w) b = s_best[w][tid] > b ? s_best[w][tid] : b;
      a.amax_part[tid * gridDim.x + blockIdx.x] = b;
    }
  }
  fin_commit();
}

// Launch shape.  Single-phase launches are persistent: the grid is sized by
// how many workgroups fit per CU (LDS bound) and balanced so every workgroup
// gets the same number of row blocks (+-1); each stages its input once.
struct GemvTuning {
  // measured on MI355X (rows per slot, workgroups per CU, waves splitting each
  // row) for the 27B-shaped head, with the first-chunk prefetch
  int rpw_large = 2, wg_per_cu_large = 2, wsk_large = 0;    // unembedding (>= large_rows rows)
  int rpw_swiglu = 2, wg_per_cu_swiglu = 2, wsk_swiglu = 0; // gate/up pairs
  int rpw_small = 2, wg_per_cu_small = 3, wsk_small = 0;    // 6K..64K-row projections
  int rpw_few = 2, wg_per_cu_few = 8, wsk_few = 0;          // projections of < few_rows rows
  int rpw_long = 2, wg_per_cu_long = 2, wsk_long = 1;       // the same with rows of >= long_k columns
  int rpw_embed = 2, wg_per_cu_embed = 6, wsk_embed = 0;    // the fc projection
  int wg_per_cu_rows = 6, wsk_rows = 0, rpw_rows = 2;       // few-row (NR > 1) flush passes
  long large_rows = 65536;
  int few_rows = 6144;
  int long_k = 12288;
};
constexpr GemvTuning kGemvTuning{};

// Occupancy of `fn` at `lds` bytes of dynamic LDS on the current device and the
// device's compute units; raising a kernel's dynamic LDS limit (gemv.hip).
hipError_t occupancy_of(const void* fn, size_t lds, int* per_cu, int* cus);
hipError_t raise_lds_limit(const void* fn);

// XB1: stage one bf16 row (the long-K projection: half the LDS, which leaves
// room for the first-chunk prefetch; the input rounded to bf16 as the matrix-core
// products round theirs)
template <int WT, int NR, int RPW, bool TWO, bool WSK = false, bool XB1 = false>
hipError_t launch_t(const GemvArgs& a0, hipStream_t s, int* grid_out, int max_per_cu) {
  constexpr bool XB = (NR > 1 || XB1) && WT == W_BF16;
  GemvArgs a = a0;
  if (a.out_mode == OUT_SWIGLU && RPW < 2) return hipErrorInvalidValue;
  const int rps = kWave / a.lpr;
  const int rows_per_wg = (WSK ? 1 : kWaves) * ((a.out_mode == OUT_SWIGLU) ? RPW / 2 : RPW) * rps;
  const int nblocks = (a.M + rows_per_wg - 1) / rows_per_wg;
  size_t lds = static_cast<size_t>(NR) * a.kp * (XB ? 2 : 4);
  int grid = nblocks;
  const void* fn = reinterpret_cast<const void*>(&k_gemv<WT, NR, RPW, TWO, XB, WSK>);
  a.pf = 0;
  a.pf_off = 0;
  if (a.grid_stride) {
    // workgroups per CU: the kernel's real occupancy (registers and LDS) at this
    // LDS size, capped by the tuning
    int occ = 1, cus = 1;
    hipError_t e = occupancy_of(fn, lds, &occ, &cus);
    if (e != hipSuccess) return e;
    occ = occ < 1 ? 1 : (occ > max_per_cu ? max_per_cu : occ);
    const int cap = cus * occ;
    const int per = (nblocks + cap - 1) / cap;          // row blocks per workgroup
    grid = (nblocks + per - 1) / per;
    // few-row passes (2-4 rows) over small matrices skip it: those stay
    // cache-resident between launches, so the prefetch only adds an LDS pass
    constexpr size_t kWBytes = WT == W_F32 ? 4 : (WT == W_BF16 ? 2 : 1);
    const bool big = static_cast<size_t>(a.M) * a.K * kWBytes >= (static_cast<size_t>(4) << 20);
    if ((NR == 1 || (NR <= 4 && big)) && a.kp >= a.K) {
      // the first-chunk prefetch: as many chunks per lane (up to one streamed
      // batch) as fit beside the staged row(s) without lowering the occupancy
      const int cpl = (a.K / WTraits<WT>::EPC) / a.lpr;
      const int per_wave = WSK ? cpl / kWaves : cpl;
      const size_t off = (lds + 15) & ~static_cast<size_t>(15);
      for (int pf = per_wave < kUnroll ? per_wave : kUnroll; pf >= 1; --pf) {
        const size_t tot = off + static_cast<size_t>(kWaves) * RPW * pf * 1024;
        if (tot > kMaxLds) continue;
        int occ1 = 1, cus1 = 1;
        e = occupancy_of(fn, tot, &occ1, &cus1);
        if (e != hipSuccess) return e;
        if ((occ1 > max_per_cu ? max_per_cu : occ1) >= occ) {
          a.pf = pf;
          a.pf_off = static_cast<int>(off);
          lds = tot;
          break;
        }
      }
    }
  }
  if (grid_out) *grid_out = grid;
  if (a.dry_run) return hipSuccess;
  if (lds > 64 * 1024) {   // gfx950 gives a workgroup up to 160 KB of LDS on request
    const hipError_t e = raise_lds_limit(fn);
    if (e != hipSuccess) return e;
  }
  (void)hipGetLastError();
  hipLaunchKernelGGL((k_gemv<WT, NR, RPW, TWO, XB, WSK>), dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int WT, int NR>
hipError_t launch_r(const GemvArgs& a, hipStream_t s, int* g) {
  const GemvTuning& t = kGemvTuning;
  const bool swiglu = a.out_mode == OUT_SWIGLU;
  int rpw, per_cu, wsk;
  if (a.in_mode == IN_EMBED) { rpw = t.rpw_embed; per_cu = t.wg_per_cu_embed; wsk = t.wsk_embed; }
  else if (swiglu) { rpw = t.rpw_swiglu; per_cu = t.wg_per_cu_swiglu; wsk = t.wsk_swiglu; }
  else if (a.M >= t.large_rows) { rpw = t.rpw_large; per_cu = t.wg_per_cu_large; wsk = t.wsk_large; }
  else if (a.K >= t.long_k) { rpw = t.rpw_long; per_cu = t.wg_per_cu_long; wsk = t.wsk_long; }
  else if (a.M < t.few_rows) { rpw = t.rpw_few; per_cu = t.wg_per_cu_few; wsk = t.wsk_few; }
  else { rpw = t.rpw_small; per_cu = t.wg_per_cu_small; wsk = t.wsk_small; }
  if (swiglu && rpw < 2) rpw = 2;
  // the wave-split rows: launches of bf16 weights
  constexpr bool kWsk = WT == W_BF16;
  if (NR > 1) { per_cu = t.wg_per_cu_rows; wsk = t.wsk_rows; }
  if (a.in_mode == IN_EMBED) {
    if constexpr (WT == W_I8) return hipErrorInvalidValue;
    else if constexpr (kWsk) {
      if (wsk) return launch_t<WT, NR, 2, true, true>(a, s, g, per_cu);
    }
    if constexpr (WT != W_I8) {   // the fc projection
      if (NR > 1 && t.rpw_rows == 1) return launch_t<WT, NR, 1, true>(a, s, g, per_cu);
      return launch_t<WT, NR, 2, true>(a, s, g, per_cu);
    }
  }
  if constexpr (NR > 1) {
    if constexpr (kWsk) {
      if (wsk) return launch_t<WT, NR, 2, false, true>(a, s, g, per_cu);
    }
    if (t.rpw_rows == 1) return launch_t<WT, NR, 1, false>(a, s, g, per_cu);
    return launch_t<WT, NR, 2, false>(a, s, g, per_cu);   // few-row flushes
  } else {
    if constexpr (kWsk) {
      if (wsk) {
        switch (rpw) {
          case 1: return launch_t<WT, NR, 1, false, true>(a, s, g, per_cu);
          case 2:
            if (a.K >= t.long_k && a.in_mode == IN_F32) return launch_t<WT, NR, 2, false, true, true>(a, s, g, per_cu);
            return launch_t<WT, NR, 2, false, true>(a, s, g, per_cu);
          default:
            if (a.K >= t.long_k && a.in_mode == IN_F32) return launch_t<WT, NR, 4, false, true, true>(a, s, g, per_cu);
            return launch_t<WT, NR, 4, false, true>(a, s, g, per_cu);
        }
      }
    }
    switch (rpw) {
      case 1: return launch_t<WT, NR, 1, false>(a, s, g, per_cu);
      case 2: return launch_t<WT, NR, 2, false>(a, s, g, per_cu);
      default: return launch_t<WT, NR, 4, false>(a, s, g, per_cu);
    }
  }
}

}  // namespace mtp
