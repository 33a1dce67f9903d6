// Many-row projections of the pending-pair flush on the gfx950 matrix cores.
//
// A flush of n pairs runs every projection of the head over n activation rows
// (the pages' pending-pair flush: "Ollama qwen3_5 MTP loader and SelfDraft
// path", Facts, MTP drafting).  Past a few rows the weight-streaming GEMV turns
// compute-bound, so these rows go through bf16 MFMA tiles instead:
//
//   k_rows_prep  one workgroup per activation row: the normalised input row in
//                bf16, RMSNorm(x; w) or [RMSNorm(E[t]; w_pe) | RMSNorm(h; w_ph)]
//                (the fused input of the head's fc), fp32 arithmetic, one
//                rounding to bf16 per element.
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
__device__ __forceinline__ float load1(const void* p, long long i, int bf16) {
  return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
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

__global__ __launch_bounds__(256) void k_rows_prep(PrepArgs a) {
  __shared__ float red[4];
  if (a.kv_state && a.kv_state[3] != 0) return;
  int n = a.n_max;
  if (a.n_dev) n = min(max(*a.n_dev, 0), a.n_max);
  const int j = blockIdx.x;
  if (j >= n) return;
  uint16_t* out = a.out + static_cast<long long>(j) * a.ld_out;
  if (a.in_mode == IN_RMS) {
    const float* x = a.x + static_cast<long long>(j) * a.ldx;
    float ss = 0.f;
    for (int k = threadIdx.x; k < a.K; k += blockDim.x) ss += x[k] * x[k];
    const float inv = 1.0f / sqrtf(block_sum(ss, red) / static_cast<float>(a.K) + a.eps);
    for (int k = threadIdx.x; k < a.K; k += blockDim.x)
      out[k] = f32_to_bf16(x[k] * load1(a.nw, k, a.nw_bf16) * inv);
    return;
  }
  // IN_EMBED: [RMSNorm(E[tok]; nw) | RMSNorm(hid; nw2)], each half `half` wide
  const int half = a.K / 2;
  const int tk = a.tok[j];
  const bool ok = tk >= 0 && tk < a.vocab_tok;
  if (!ok && a.err && threadIdx.x == 0) *a.err = 4;   // token outside the vocabulary
  const long long eoff = static_cast<long long>(ok ? tk : 0) * half;
  const long long hoff = static_cast<long long>(j) * a.ld_hid;
  float se = 0.f, sh = 0.f;
  for (int k = threadIdx.x; k < half; k += blockDim.x) {
    const float e = ok ? load1(a.embed, eoff + k, a.embed_bf16) : 0.f;
    const float h = load1(a.hid, hoff + k, a.hid_bf16);
    se += e * e;
    sh += h * h;
  }
  const float inv_e = 1.0f / sqrtf(block_sum(se, red) / static_cast<float>(half) + a.eps);
  const float inv_h = 1.0f / sqrtf(block_sum(sh, red) / static_cast<float>(half) + a.eps);
  for (int k = threadIdx.x; k < half; k += blockDim.x) {
    const float e = ok ? load1(a.embed, eoff + k, a.embed_bf16) : 0.f;
    const float h = load1(a.hid, hoff + k, a.hid_bf16);
    out[k] = f32_to_bf16(e * load1(a.nw, k, a.nw_bf16) * inv_e);
    out[half + k] = f32_to_bf16(h * load1(a.nw2, k, a.nw_bf16) * inv_h);
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
