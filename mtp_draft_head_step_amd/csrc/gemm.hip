// Many-row projections of the pending-pair flush on the gfx950 matrix cores.
//
// A flush of n pairs runs every projection of the head over n activation rows
// (the pages' pending-pair flush: "Ollama qwen3_5 MTP loader and SelfDraft
// path", Facts, MTP drafting).  Past a few rows the weight-streaming GEMV turns
// compute-bound, so these rows go through bf16 MFMA tiles instead:
//
//   k_rows_prep  one workgroup per activation row: the normalised input row in
//                bf16, RMSNorm(x; w) or [RMSNorm(E[t]; w_pe) | RMSNorm(h; w_ph)]
//                (the fused input of the head's fc), or plain x (IN_F32), fp32
//                arithmetic, one rounding to bf16 per element; 16-byte loads,
//                four per thread in flight.
//   k_gemm       Y[j, c] = sum_k A[j, k] W[c, k] for a 64 x 64 tile of (row j,
//                output c) per workgroup; four waves each own a 32 x 32 block
//                computed with v_mfma_f32_32x32x16_bf16 from 64-column slices
//                of A and W staged in LDS; fp32 accumulation; epilogues: plain
//                store, residual add (with an optional act-dtype copy), and the
//                SwiGLU product silu(gate) * up of two weight matrices.
#include "common.h"
#include "kernels.h"

namespace mtp {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kTM = 64;            // activation rows per tile
constexpr int kTN = 64;            // output columns per tile
constexpr int kTK = 64;            // reduction slice staged per step
constexpr int kLdsRow = kTK + 8;   // bf16 per LDS row (16 B pad against bank conflicts)

// ---------------------------------------------------------------------------
// row preparation
// ---------------------------------------------------------------------------
// 8 consecutive elements (bf16 or fp32) as fp32.
__device__ __forceinline__ void load8f(const void* p, long long i, int bf16, float (&v)[8]) {
  if (bf16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  } else {
    const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    const float4 y = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i + 4);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  }
}

__device__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < static_cast<int>(blockDim.x) / kWave; ++w) t += red[w];
  return t;
}

// One row: source segment(s) of 8-element jobs.  IN_EMBED: jobs k < half read
// the embedding row, the rest the hidden row.
struct PrepRow {
  const void* src0;  long long off0;  int bf0;   // embedding row / x row
  const void* src1;  long long off1;  int bf1;   // hidden row (IN_EMBED)
  int half;
};

constexpr int kPrepU = 4;   // jobs in flight per thread

__device__ __forceinline__ void prep_load(const PrepRow& r, int k, float (&v)[8]) {
  if (k < r.half) {
    if (r.src0) load8f(r.src0, r.off0 + k, r.bf0, v);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
  } else {
    load8f(r.src1, r.off1 + (k - r.half), r.bf1, v);
  }
}

__global__ __launch_bounds__(256) void k_rows_prep(PrepArgs a) {
  __shared__ float red[4];
  if (a.kv_state && a.kv_state[3] != 0) return;
  int n = a.n_max;
  if (a.n_dev) n = min(max(*a.n_dev, 0), a.n_max);
  const int j = blockIdx.x;
  if (j >= n) return;
  uint16_t* out = a.out + static_cast<long long>(j) * a.ld_out;
  const int K = a.K;
  PrepRow r;
  if (a.in_mode == IN_EMBED) {
    const int tk = a.tok[j];
    const bool ok = tk >= 0 && tk < a.vocab_tok;
    if (!ok && a.err && threadIdx.x == 0) *a.err = 4;   // token outside the vocabulary
    r.half = K / 2;
    r.src0 = ok ? a.embed : nullptr; r.off0 = static_cast<long long>(ok ? tk : 0) * r.half; r.bf0 = a.embed_bf16;
    r.src1 = a.hid; r.off1 = static_cast<long long>(j) * a.ld_hid; r.bf1 = a.hid_bf16;
  } else {
    r.half = K;
    r.src0 = a.x; r.off0 = static_cast<long long>(j) * a.ldx; r.bf0 = 0;
    r.src1 = nullptr; r.off1 = 0; r.bf1 = 0;
  }
  const int njobs = K / 8;
  // pass 1: sums of squares (first part / second part)
  float se = 0.f, sh = 0.f;
  if (a.in_mode != IN_F32) {
    for (int f0 = threadIdx.x; f0 < njobs; f0 += 256 * kPrepU) {
      float v[kPrepU][8];
#pragma unroll
      for (int u = 0; u < kPrepU; ++u)
        if (f0 + u * 256 < njobs) prep_load(r, (f0 + u * 256) * 8, v[u]);
#pragma unroll
      for (int u = 0; u < kPrepU; ++u) {
        const int k = (f0 + u * 256) * 8;
        if (k >= K) continue;
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) t += v[u][e] * v[u][e];
        if (k < r.half) se += t; else sh += t;
      }
    }
  }
  float inv0 = 1.f, inv1 = 1.f;
  if (a.in_mode == IN_RMS) {
    inv0 = 1.0f / sqrtf(block_sum(se, red) / static_cast<float>(K) + a.eps);
  } else if (a.in_mode == IN_EMBED) {
    inv0 = 1.0f / sqrtf(block_sum(se, red) / static_cast<float>(r.half) + a.eps);
    inv1 = 1.0f / sqrtf(block_sum(sh, red) / static_cast<float>(r.half) + a.eps);
  }
  // pass 2: bf16(x * w * inv) (IN_F32: bf16(x))
  for (int f0 = threadIdx.x; f0 < njobs; f0 += 256 * kPrepU) {
    float v[kPrepU][8], w[kPrepU][8];
#pragma unroll
    for (int u = 0; u < kPrepU; ++u) {
      const int k = (f0 + u * 256) * 8;
      if (k >= K) continue;
      prep_load(r, k, v[u]);
      if (a.in_mode == IN_F32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[u][e] = 1.f;
      } else if (k < r.half) {
        load8f(a.nw, k, a.nw_bf16, w[u]);
      } else {
        load8f(a.nw2, k - r.half, a.nw_bf16, w[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kPrepU; ++u) {
      const int k = (f0 + u * 256) * 8;
      if (k >= K) continue;
      const float inv = k < r.half ? inv0 : inv1;
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = f32_to_bf16(v[u][2 * q] * w[u][2 * q] * inv) |
               (static_cast<uint32_t>(f32_to_bf16(v[u][2 * q + 1] * w[u][2 * q + 1] * inv)) << 16);
      *reinterpret_cast<uint4*>(out + k) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

hipError_t launch_rows_prep(const PrepArgs& a, hipStream_t s) {
  if (a.n_max <= 0) return hipSuccess;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_rows_prep, dim3(a.n_max), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// the tiled MFMA product
// ---------------------------------------------------------------------------
// 16 consecutive bf16 of one A row starting at column k (bf16 rows, or fp32
// rows rounded to bf16 on the way in).
__device__ __forceinline__ void load_a16(const GemmArgs& a, int row, int k, uint4& lo, uint4& hi) {
  if (a.a_f32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.a) +
                                                      static_cast<long long>(row) * a.lda + k);
    float4 f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = p[i];
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[2 * i] = f32_to_bf16(f[i].x) | (static_cast<uint32_t>(f32_to_bf16(f[i].y)) << 16);
      w[2 * i + 1] = f32_to_bf16(f[i].z) | (static_cast<uint32_t>(f32_to_bf16(f[i].w)) << 16);
    }
    lo = make_uint4(w[0], w[1], w[2], w[3]);
    hi = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.a) +
                                                    static_cast<long long>(row) * a.lda + k);
    lo = p[0];
    hi = p[1];
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

template <bool SWIGLU>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kTM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kTN * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t Us[SWIGLU ? kTN * kLdsRow : 8];
  if (a.kv_state && a.kv_state[3] != 0) return;
  int n = a.n_max;
  if (a.n_dev) n = min(max(*a.n_dev, 0), a.n_max);
  const int r0 = blockIdx.y * kTM;
  if (r0 >= n) return;
  const int c0 = blockIdx.x * kTN;
  // the stacked matrix holding output columns [c0, c0 + 64) (tiles never straddle)
  const uint16_t* W = a.w[0];
  int cl = c0;
  if (!SWIGLU) {
    if (cl >= a.m[0]) {
      cl -= a.m[0];
      W = a.w[1];
      if (cl >= a.m[1]) {
        cl -= a.m[1];
        W = a.w[2];
      }
    }
  }
  const uint16_t* U = a.w[1];   // SWIGLU: up rows beside the gate rows

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;          // this wave's 32 x 32 block
  // staging: thread t moves 16 bf16 of row t / 4 at column (t % 4) * 16
  const int sr = tid >> 2, sk = (tid & 3) * 16;
  const int arow = min(r0 + sr, a.n_max - 1);       // rows past n are computed, not stored
  const long long wrow = static_cast<long long>(cl + sr) * a.K;

  f32x16_t acc = {};
  f32x16_t accu = {};
  uint4 pa0, pa1, pb0, pb1, pu0 = {}, pu1 = {};
  load_a16(a, arow, sk, pa0, pa1);
  {
    const uint4* p = reinterpret_cast<const uint4*>(W + wrow + sk);
    pb0 = p[0];
    pb1 = p[1];
    if (SWIGLU) {
      const uint4* q = reinterpret_cast<const uint4*>(U + wrow + sk);
      pu0 = q[0];
      pu1 = q[1];
    }
  }
  for (int k0 = 0; k0 < a.K; k0 += kTK) {
    __syncthreads();
    *reinterpret_cast<uint4*>(As + sr * kLdsRow + sk) = pa0;
    *reinterpret_cast<uint4*>(As + sr * kLdsRow + sk + 8) = pa1;
    *reinterpret_cast<uint4*>(Bs + sr * kLdsRow + sk) = pb0;
    *reinterpret_cast<uint4*>(Bs + sr * kLdsRow + sk + 8) = pb1;
    if (SWIGLU) {
      *reinterpret_cast<uint4*>(Us + sr * kLdsRow + sk) = pu0;
      *reinterpret_cast<uint4*>(Us + sr * kLdsRow + sk + 8) = pu1;
    }
    __syncthreads();
    // prefetch the next slice while this one is multiplied
    const int kn = k0 + kTK;
    if (kn < a.K) {
      load_a16(a, arow, kn + sk, pa0, pa1);
      const uint4* p = reinterpret_cast<const uint4*>(W + wrow + kn + sk);
      pb0 = p[0];
      pb1 = p[1];
      if (SWIGLU) {
        const uint4* q = reinterpret_cast<const uint4*>(U + wrow + kn + sk);
        pu0 = q[0];
        pu1 = q[1];
      }
    }
#pragma unroll
    for (int ks = 0; ks < kTK / 16; ++ks) {
      const int kk = ks * 16 + (lane >> 5) * 8;
      const bf16x8_t af = __builtin_bit_cast(bf16x8_t,
          *reinterpret_cast<const uint4*>(As + (wr * 32 + (lane & 31)) * kLdsRow + kk));
      const bf16x8_t bf = __builtin_bit_cast(bf16x8_t,
          *reinterpret_cast<const uint4*>(Bs + (wc * 32 + (lane & 31)) * kLdsRow + kk));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
      if (SWIGLU) {
        const bf16x8_t uf = __builtin_bit_cast(bf16x8_t,
            *reinterpret_cast<const uint4*>(Us + (wc * 32 + (lane & 31)) * kLdsRow + kk));
        accu = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, uf, accu, 0, 0, 0);
      }
    }
  }

  // epilogue: element i of the accumulator is (row (i/4)*8 + (lane/32)*4 + i%4,
  // column lane % 32) of this wave's block
  const int col = c0 + wc * 32 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + wr * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
    if (r >= n) continue;
    float v = acc[i];
    if (SWIGLU) v = silu(v) * accu[i];
    if (a.out_mode == OUT_RESID) v += a.res[static_cast<long long>(r) * a.ldres + col];
    a.y[static_cast<long long>(r) * a.ldy + col] = v;
    if (a.y2) {
      if (a.y2_bf16)
        static_cast<uint16_t*>(a.y2)[static_cast<long long>(r) * a.ldy2 + col] = f32_to_bf16(v);
      else
        static_cast<float*>(a.y2)[static_cast<long long>(r) * a.ldy2 + col] = v;
    }
  }
}

bool gemm_supported(int M, int K, const int* m, int nmat) {
  if (M <= 0 || K <= 0 || M % kTN || K % kTK) return false;
  for (int i = 0; i < nmat; ++i)
    if (m[i] % kTN) return false;
  return true;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.n_max <= 0) return hipSuccess;
  const dim3 grid(a.M / kTN, (a.n_max + kTM - 1) / kTM);
  (void)hipGetLastError();
  if (a.out_mode == OUT_SWIGLU)
    hipLaunchKernelGGL(k_gemm<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_gemm<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mtp
