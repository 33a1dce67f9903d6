// Weight-streaming GEMV for gfx950 (batch-1 and few-row draft steps).
//
// The draft-head step reads every weight once per call (about 1 flop per byte),
// so these kernels are bound by HBM bandwidth.  Layout of the work:
//  * each weight row is split over `lpr` lanes; every lane issues 16-byte loads
//    (8 bf16 / 4 fp32 / 16 int8) and a wave keeps RPW rows x UNROLL loads in
//    flight before consuming them;
//  * the activation rows (1..16) are staged once per workgroup in LDS as fp32,
//    with the producer's RMSNorm (or the embedding gather + twin RMSNorm of the
//    pair) folded into the staging, so no separate norm kernel runs;
//  * lanes of a row are reduced with xor shuffles, in a fixed order (no float
//    atomics: results are bit-identical run to run);
//  * epilogues fuse the residual add, SwiGLU (gate and up rows of the same index
//    are paired in one wave) and the logits argmax (packed 64-bit key, max value
//    then lowest index, one atomicMax per workgroup, the last workgroup writes
//    the int32 result and re-arms the slot).
#include "common.h"
#include "kernels.h"

namespace mtp {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kRPW = 4;      // row slots per wave
constexpr int kUnroll = 4;   // 16-byte loads per slot in flight
constexpr int kLdsBytes = 64 * 1024;

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

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

template <int WT, int NR>
__global__ __launch_bounds__(kThreads) void k_gemv(GemvArgs a) {
  extern __shared__ float xs[];  // [NR][kp]
  __shared__ float s_red[kWaves][2 * NR];
  __shared__ float s_inv[2 * NR];
  __shared__ unsigned long long s_best[kWaves];
  constexpr int EPC = WTraits<WT>::EPC;

  if (a.kv_state && a.kv_state[3] != 0) return;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;

  // ---- activation rows handled by this launch
  int n = a.n_max;
  if (a.n_dev) n = min(max(*a.n_dev, 0), a.n_max);
  int j0, nrows;
  if (a.row_sel == ROW_LAST) {
    j0 = n - 1;
    nrows = n > 0 ? 1 : 0;
  } else {
    j0 = a.row_base;
    nrows = min(NR, n - a.row_base);
  }
  if (nrows <= 0) {
    if (a.out_mode == OUT_LOGITS && last_block_ticket(a.counter, gridDim.x)) {
      atomicExch(a.amax_slot, 0ull);
    }
    return;
  }
  const int K = a.K;

  // ---- per-row inverse RMS of the input (recomputed per workgroup from L2)
  if (a.in_mode != IN_F32) {
    const int half = (a.in_mode == IN_EMBED) ? K / 2 : K;
    float ss[2 * NR];
#pragma unroll
    for (int i = 0; i < 2 * NR; ++i) ss[i] = 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      if (r < nrows) {
        const int j = j0 + r;
        if (a.in_mode == IN_RMS) {
          const float* xr = a.x + static_cast<size_t>(j) * a.ldx;
          for (int k = tid * 4; k < K; k += kThreads * 4) {
            const float4 v = *reinterpret_cast<const float4*>(xr + k);
            ss[2 * r] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
          }
        } else {
          const int t = a.tok[j];
          for (int k = tid; k < half; k += kThreads) {
            const float e = load_val(a.embed, static_cast<size_t>(t) * half + k, a.embed_bf16);
            const float h = load_val(a.hid, j * a.ld_hid + k, a.hid_bf16);
            ss[2 * r] += e * e;
            ss[2 * r + 1] += h * h;
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 2 * NR; ++i) {
      float v = wave_sum(ss[i]);
      if (lane == 0) s_red[wave][i] = v;
    }
    __syncthreads();
    if (tid < 2 * NR) {
      float v = 0.f;
      for (int w = 0; w < kWaves; ++w) v += s_red[w][tid];
      s_inv[tid] = rsqrtf(v / static_cast<float>(half) + a.eps);
    }
    __syncthreads();
  }

  const int lpr = a.lpr;
  const int rps = kWave / lpr;          // rows per slot
  const int sub = lane / lpr;           // row within the slot
  const int li = lane % lpr;            // lane within the row
  const bool swiglu = (a.out_mode == OUT_SWIGLU);
  const int rows_per_wg = kWaves * (swiglu ? kRPW / 2 : kRPW) * rps;
  const int nblocks = (a.M + rows_per_wg - 1) / rows_per_wg;
  const int nphase = (K + a.kp - 1) / a.kp;

  unsigned long long best = 0ull;

  for (int blk = blockIdx.x; blk < nblocks; blk += (a.grid_stride ? gridDim.x : nblocks)) {
    // rows of the slots: plain mode slot s -> row; swiglu slot pair (2p, 2p+1) -> (gate r, up r)
    const char* rowp[kRPW];
    int rowid[kRPW];
    bool valid[kRPW];
#pragma unroll
    for (int s = 0; s < kRPW; ++s) {
      int r, mat;
      if (swiglu) {
        r = blk * rows_per_wg + (wave * (kRPW / 2) + s / 2) * rps + sub;
        mat = s & 1;
        valid[s] = r < a.M;
      } else {
        r = blk * rows_per_wg + (wave * kRPW + s) * rps + sub;
        valid[s] = r < a.M;
        mat = 0;
        int rr = r;
        if (rr >= a.m[0]) { rr -= a.m[0]; mat = 1; if (rr >= a.m[1]) { rr -= a.m[1]; mat = 2; } }
        if (valid[s]) r = rr;
      }
      rowid[s] = r;
      const size_t row_bytes = static_cast<size_t>(K) * (WT == W_F32 ? 4 : (WT == W_BF16 ? 2 : 1));
      rowp[s] = valid[s] ? static_cast<const char*>(a.w[mat]) + static_cast<size_t>(r) * row_bytes
                         : static_cast<const char*>(a.w[0]);
    }

    float acc[kRPW][NR];
#pragma unroll
    for (int s = 0; s < kRPW; ++s)
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[s][r] = 0.f;

    for (int ph = 0; ph < nphase; ++ph) {
      const int k0 = ph * a.kp;
      const int klen = min(a.kp, K - k0);
      // ---- stage the (normalised) inputs of this phase in LDS
      // a single-phase grid-stride loop stages once; multi-phase restages per phase
      const bool need_stage = (blk == static_cast<int>(blockIdx.x)) || nphase > 1;
      if (need_stage) {
        __syncthreads();
        const int q4 = klen / 4;
        for (int idx = tid; idx < NR * q4; idx += kThreads) {
          const int r = idx / q4;
          const int k = k0 + (idx - r * q4) * 4;
          float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
          if (r < nrows) {
            const int j = j0 + r;
            if (a.in_mode == IN_F32) {
              v = *reinterpret_cast<const float4*>(a.x + static_cast<size_t>(j) * a.ldx + k);
            } else if (a.in_mode == IN_RMS) {
              v = *reinterpret_cast<const float4*>(a.x + static_cast<size_t>(j) * a.ldx + k);
              const float inv = s_inv[2 * r];
              v.x *= inv * load_val(a.nw, k, a.nw_bf16);
              v.y *= inv * load_val(a.nw, k + 1, a.nw_bf16);
              v.z *= inv * load_val(a.nw, k + 2, a.nw_bf16);
              v.w *= inv * load_val(a.nw, k + 3, a.nw_bf16);
            } else {
              const int half = K / 2;
              float t[4];
              for (int e = 0; e < 4; ++e) {
                const int kk = k + e;
                if (kk < half) {
                  t[e] = load_val(a.embed, static_cast<size_t>(a.tok[j]) * half + kk, a.embed_bf16) * s_inv[2 * r] *
                         load_val(a.nw, kk, a.nw_bf16);
                } else {
                  t[e] = load_val(a.hid, j * a.ld_hid + kk - half, a.hid_bf16) * s_inv[2 * r + 1] *
                         load_val(a.nw2, kk - half, a.nw_bf16);
                }
              }
              v = make_float4(t[0], t[1], t[2], t[3]);
            }
          }
          *reinterpret_cast<float4*>(xs + r * a.kp + (k - k0)) = v;
        }
        __syncthreads();
      }

      // ---- stream the weights of this phase
      const int nch = klen / EPC;
      const int c_base = k0 / EPC;
      for (int c = li; c < nch; c += lpr * kUnroll) {
        uint4 wv[kRPW][kUnroll];
#pragma unroll
        for (int s = 0; s < kRPW; ++s)
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            const int cc = c + u * lpr;
            if (valid[s] && cc < nch)
              wv[s][u] = *reinterpret_cast<const uint4*>(rowp[s] + static_cast<size_t>(c_base + cc) * 16);
            else
              wv[s][u] = make_uint4(0u, 0u, 0u, 0u);
          }
#pragma unroll
        for (int s = 0; s < kRPW; ++s)
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            const int cc = c + u * lpr;
            if (cc < nch) {
              float scale = 1.f;
              if constexpr (WT == W_I8) {
                if (valid[s]) {
                  const int grp = (k0 + cc * EPC) >> 7;
                  scale = f16_to_f32(a.scales[static_cast<size_t>(rowid[s]) * (K >> 7) + grp]);
                }
              }
#pragma unroll
              for (int r = 0; r < NR; ++r) {
                const float d = dot_chunk<WT>(wv[s][u], xs + r * a.kp + cc * EPC);
                if constexpr (WT == W_I8) acc[s][r] += d * scale; else acc[s][r] += d;
              }
            }
          }
      }
    }

    // ---- reduce each row over its lanes and run the epilogue
#pragma unroll
    for (int s = 0; s < kRPW; ++s)
#pragma unroll
      for (int r = 0; r < NR; ++r) acc[s][r] = group_sum(acc[s][r], lpr);

    if (li == 0) {
      if (swiglu) {
#pragma unroll
        for (int s = 0; s < kRPW; s += 2) {
          if (!valid[s]) continue;
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            if (r >= nrows) continue;
            const int j = j0 + r;
            a.y[static_cast<size_t>(j) * a.ldy + rowid[s]] = silu(acc[s][r]) * acc[s + 1][r];
          }
        }
      } else {
#pragma unroll
        for (int s = 0; s < kRPW; ++s) {
          if (!valid[s]) continue;
          const int row = blk * rows_per_wg + (wave * kRPW + s) * rps + sub;
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            if (r >= nrows) continue;
            const int j = j0 + r;
            float v = acc[s][r];
            if (a.out_mode == OUT_LOGITS) {
              if (a.logits) a.logits[row] = v;
              const unsigned long long key = argmax_key(v, static_cast<uint32_t>(row));
              best = key > best ? key : best;
              continue;
            }
            if (a.out_mode == OUT_RESID) v += a.res[static_cast<size_t>(j) * a.ldres + row];
            a.y[static_cast<size_t>(j) * a.ldy + row] = v;
            if (a.y2) {
              const size_t o = (a.row_sel == ROW_LAST) ? row : static_cast<size_t>(j) * a.ldy2 + row;
              if (a.y2_bf16) static_cast<uint16_t*>(a.y2)[o] = f32_to_bf16(v);
              else static_cast<float*>(a.y2)[o] = v;
            }
          }
        }
      }
    }
  }

  if (a.out_mode == OUT_LOGITS) {
    best = wave_max_u64(best);
    if (lane == 0) s_best[wave] = best;
    __syncthreads();
    if (tid == 0) {
      unsigned long long b = s_best[0];
      for (int w = 1; w < kWaves; ++w) b = s_best[w] > b ? s_best[w] : b;
      atomicMax(a.amax_slot, b);
    }
    if (last_block_ticket(a.counter, gridDim.x) && tid == 0) {
      const unsigned long long b = atomicExch(a.amax_slot, 0ull);
      if (a.amax_out) *a.amax_out = argmax_index(b);
    }
  }
}

template <int WT, int NR>
static hipError_t launch_t(const GemvArgs& a, hipStream_t s) {
  const int rps = kWave / a.lpr;
  const int rows_per_wg = kWaves * ((a.out_mode == OUT_SWIGLU) ? kRPW / 2 : kRPW) * rps;
  const int nblocks = (a.M + rows_per_wg - 1) / rows_per_wg;
  int grid = nblocks;
  if (a.grid_stride) grid = nblocks < 2048 ? nblocks : 2048;
  const size_t lds = static_cast<size_t>(NR) * a.kp * sizeof(float);
  (void)hipGetLastError();
  hipLaunchKernelGGL((k_gemv<WT, NR>), dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int WT>
static hipError_t launch_w(const GemvArgs& a, int nr, hipStream_t s) {
  switch (nr) {
    case 1: return launch_t<WT, 1>(a, s);
    case 2: return launch_t<WT, 2>(a, s);
    case 4: return launch_t<WT, 4>(a, s);
    case 8: return launch_t<WT, 8>(a, s);
    case 16: return launch_t<WT, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv(const GemvArgs& a, int wtype, int nr, hipStream_t s) {
  switch (wtype) {
    case W_F32: return launch_w<W_F32>(a, nr, s);
    case W_BF16: return launch_w<W_BF16>(a, nr, s);
    case W_I8: return launch_w<W_I8>(a, nr, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtp
