// Few-row projections (2..16 activation rows) with bf16 weights on the matrix
// cores: the in-round flush of the k + 1 completed pairs ("Ollama qwen3_5 MTP
// loader and SelfDraft path", Facts, MTP drafting) streams every weight once
// for all its rows.  A plain GEMV spends 8 conversions and 8 x rows FMAs of
// vector ALU per 16 bytes of weights; here one v_mfma_f32_16x16x32_bf16 per 16
// bytes does the work, so the pass stays bound by HBM.
//
// A workgroup owns 16 output columns at a time; its four waves split the
// reduction into four contiguous ranges and stream them with eight 16-byte
// loads in flight per lane.  The MFMA A operand is the bf16 input rows staged
// in LDS as x * w_norm (rows past the count read as zero), B is the weight tile
// (lane l: row l % 16, eight columns at 8 (l / 16) of each 32-column step).
// The waves' 16 x 16 partial tiles are added in wave order through LDS, then
// 1 / rms of each row (deferred: it factors out of the dot products) and the
// epilogue (plain, residual, SwiGLU pair) are applied.
#include "common.h"
#include "kernels.h"

namespace mtp {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8s;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4s;

constexpr int kSkU = 8;                        // 32-column steps in flight per wave
constexpr int kSkMaxLds = 128 * 1024;          // staged rows (bf16) per workgroup
constexpr int kSkCUs = 256;

__device__ __forceinline__ float sk_silu(float z) { return z / (1.0f + __expf(-z)); }

// 8 consecutive elements (bf16 or fp32) as fp32.
__device__ __forceinline__ void sk_load8(const void* p, long long i, int bf16, float (&v)[8]) {
  if (bf16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = __uint_as_float(w[q] << 16);
      v[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// dst[k] = bf16(src[off + k] * nw[k]) for k in [0, len) (nw null: factor 1), 8
// elements per thread per step and four steps of loads in flight; returns the
// thread's share of the sum of squares of the src values.  len % 8 == 0.
__device__ __forceinline__ float sk_stage(uint16_t* dst, const void* src, long long off, int src_bf16,
                                          const void* nw, int nw_bf16, int len) {
  float ss = 0.f;
  for (int base = threadIdx.x * 8; base < len; base += 256 * 8 * 4) {
    float v[4][8], w[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = base + u * 256 * 8;
      if (k < len) {
        sk_load8(src, off + k, src_bf16, v[u]);
        if (nw) sk_load8(nw, k, nw_bf16, w[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = base + u * 256 * 8;
      if (k < len) {
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float a = v[u][2 * q], b = v[u][2 * q + 1];
          ss += a * a + b * b;
          const float wa = nw ? w[u][2 * q] : 1.f, wb = nw ? w[u][2 * q + 1] : 1.f;
          o[q] = f32_to_bf16(a * wa) | (static_cast<uint32_t>(f32_to_bf16(b * wb)) << 16);
        }
        *reinterpret_cast<uint4*>(dst + k) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
  return ss;
}

template <bool TWO, bool SWIGLU>
__global__ __launch_bounds__(256) void k_skinny(GemvArgs a, int nr) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // [nr][K] bf16
  __shared__ float s_part[4][64][8];
  __shared__ float s_ss[4][32];
  __shared__ float s_inv[32];
  if (a.kv_state && a.kv_state[3] != 0) return;
  int n = a.n_max;
  if (a.n_dev) n = min(max(*a.n_dev, 0), a.n_max);
  const int j0 = a.row_base;
  const int nrows = min(nr, n - j0);
  if (nrows <= 0) return;
  const int K = a.K;
  const int half = TWO ? K / 2 : K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- stage x * w_norm (bf16) of every row, and each row's sum(s) of squares
  for (int r = 0; r < nr; ++r) {
    float se = 0.f, sh = 0.f;
    uint16_t* dst = xs + static_cast<long long>(r) * K;
    if (r < nrows) {
      const int jr = j0 + r;
      if (a.in_mode == IN_EMBED) {
        const int tk = a.tok[jr];
        const bool ok = tk >= 0 && tk < a.vocab_tok;
        if (!ok && a.err && blockIdx.x == 0 && tid == 0) *a.err = 4;   // token outside the vocabulary
        if (ok)
          se = sk_stage(dst, a.embed, static_cast<long long>(tk) * half, a.embed_bf16, a.nw, a.nw_bf16, half);
        else
          for (int k = tid; k < half; k += 256) dst[k] = 0;
        sh = sk_stage(dst + half, a.hid, static_cast<long long>(jr) * a.ld_hid, a.hid_bf16, a.nw2, a.nw_bf16,
                      half);
      } else {
        se = sk_stage(dst, a.x, static_cast<long long>(jr) * a.ldx, 0, a.in_mode == IN_RMS ? a.nw : nullptr,
                      a.nw_bf16, K);
      }
    } else {
      for (int k = tid * 8; k < K; k += 256 * 8) *reinterpret_cast<uint4*>(dst + k) = make_uint4(0u, 0u, 0u, 0u);
    }
    se = wave_sum(se);
    sh = wave_sum(sh);
    if (lane == 0) {
      s_ss[wave][2 * r] = se;
      s_ss[wave][2 * r + 1] = sh;
    }
  }
  __syncthreads();
  if (tid < 2 * nr) {
    const float v = s_ss[0][tid] + s_ss[1][tid] + s_ss[2][tid] + s_ss[3][tid];
    float inv;
    if (a.in_mode == IN_F32) inv = (tid & 1) ? 0.f : 1.f;
    else if (a.in_mode == IN_RMS) inv = (tid & 1) ? 0.f : rsqrtf(v / static_cast<float>(K) + a.eps);
    else inv = rsqrtf(v / static_cast<float>(half) + a.eps);
    s_inv[tid] = inv;
  }
  __syncthreads();

  const int ntiles = a.M / 16;
  const int nk = K / 32;                                   // 32-column steps
  const int kb = wave * nk / 4, ke = (wave + 1) * nk / 4;  // this wave's steps
  const int kh = half / 32;                                // first step of the second half
  const int ar = lane & 15;                                // A row / B column of this lane
  const bool arow_ok = ar < nrows;
  const uint16_t* xrow = xs + static_cast<long long>(ar) * K + (lane >> 4) * 8;

  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int c0 = tile * 16;
    const uint16_t* W = static_cast<const uint16_t*>(a.w[0]);
    int cl = c0;
    if (!SWIGLU) {
      if (cl >= a.m[0]) {
        cl -= a.m[0];
        W = static_cast<const uint16_t*>(a.w[1]);
        if (cl >= a.m[1]) {
          cl -= a.m[1];
          W = static_cast<const uint16_t*>(a.w[2]);
        }
      }
    }
    const long long roff = static_cast<long long>(cl + ar) * K + (lane >> 4) * 8;
    const uint16_t* wrow = W + roff;
    const uint16_t* urow = SWIGLU ? static_cast<const uint16_t*>(a.w[1]) + roff : nullptr;
    f32x4s acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};

    for (int kk = kb; kk < ke; kk += kSkU) {
      const int cnt = min(kSkU, ke - kk);
      uint4 b[kSkU], u[kSkU];
#pragma unroll
      for (int i = 0; i < kSkU; ++i)
        if (i < cnt) {
          b[i] = load_stream16(wrow + static_cast<long long>(kk + i) * 32);
          if (SWIGLU) u[i] = load_stream16(urow + static_cast<long long>(kk + i) * 32);
        }
#pragma unroll
      for (int i = 0; i < kSkU; ++i)
        if (i < cnt) {
          uint4 xa = make_uint4(0u, 0u, 0u, 0u);
          if (arow_ok) xa = *reinterpret_cast<const uint4*>(xrow + (kk + i) * 32);
          const bf16x8s af = __builtin_bit_cast(bf16x8s, xa);
          const bf16x8s bf = __builtin_bit_cast(bf16x8s, b[i]);
          if (SWIGLU) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8s, u[i]), acc2, 0, 0, 0);
          } else if (TWO && kk + i >= kh) {
            acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc2, 0, 0, 0);
          } else {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc, 0, 0, 0);
          }
        }
    }

    // the four waves' partial tiles, added in wave order
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s_part[wave][lane][i] = acc[i];
      s_part[wave][lane][4 + i] = acc2[i];
    }
    __syncthreads();
    if (wave == 0) {
      const int col = c0 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = (lane >> 4) * 4 + i;          // activation row of this element
        if (rr >= nrows) continue;
        float v = 0.f, v2 = 0.f;
        for (int w = 0; w < 4; ++w) {
          v += s_part[w][lane][i];
          v2 += s_part[w][lane][4 + i];
        }
        const int j = j0 + rr;
        float out;
        if (SWIGLU) {
          out = sk_silu(v * s_inv[2 * rr]) * (v2 * s_inv[2 * rr]);
        } else {
          out = v * s_inv[2 * rr];
          if (TWO) out += v2 * s_inv[2 * rr + 1];
          if (a.out_mode == OUT_RESID) out += a.res[static_cast<long long>(j) * a.ldres + col];
        }
        a.y[static_cast<long long>(j) * a.ldy + col] = out;
        if (!SWIGLU && a.y2) {
          if (a.y2_bf16)
            static_cast<uint16_t*>(a.y2)[static_cast<long long>(j) * a.ldy2 + col] = f32_to_bf16(out);
          else
            static_cast<float*>(a.y2)[static_cast<long long>(j) * a.ldy2 + col] = out;
        }
      }
    }
    __syncthreads();   // s_part is rewritten by the next tile
  }
}

bool skinny_supported(const GemvArgs& a, int nr) {
  if (nr < 2 || nr > 16) return false;
  if (a.M % 16 || a.K % 64) return false;
  if (a.out_mode != OUT_F32 && a.out_mode != OUT_RESID && a.out_mode != OUT_SWIGLU) return false;
  for (int i = 0; i < 3; ++i)
    if (a.m[i] % 16) return false;
  return static_cast<long long>(nr) * a.K * 2 <= kSkMaxLds;
}

template <bool TWO, bool SWIGLU>
static hipError_t launch_sk(const GemvArgs& a, int nr, hipStream_t s) {
  const size_t lds = static_cast<size_t>(nr) * a.K * 2;
  static bool raised = false;
  if (!raised) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_skinny<TWO, SWIGLU>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kSkMaxLds);
    if (e != hipSuccess) return e;
    raised = true;
  }
  const int ntiles = a.M / 16;
  int occ = static_cast<int>((160 * 1024) / (lds + 12 * 1024));
  occ = occ < 1 ? 1 : (occ > 4 ? 4 : occ);
  const int grid = ntiles < kSkCUs * occ ? ntiles : kSkCUs * occ;
  (void)hipGetLastError();
  hipLaunchKernelGGL((k_skinny<TWO, SWIGLU>), dim3(grid), dim3(256), lds, s, a, nr);
  return hipGetLastError();
}

hipError_t launch_skinny(const GemvArgs& a, int nr, hipStream_t s) {
  if (a.out_mode == OUT_SWIGLU) return launch_sk<false, true>(a, nr, s);
  if (a.in_mode == IN_EMBED) return launch_sk<true, false>(a, nr, s);
  return launch_sk<false, false>(a, nr, s);
}

}  // namespace mtp
