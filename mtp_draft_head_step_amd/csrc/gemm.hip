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

constexpr int kPrepU = 4;          // jobs in flight per thread
constexpr int kPrepThreads = 1024; // a row's jobs in one pass up to 4096 jobs (32768 columns)
// split reduces (k_gemm_reduce, k_gemm_reduce_norm)
constexpr int kNormThreads = 1024;
constexpr int kNormPer = 2;        // float4 columns per thread: rows of up to 8192
constexpr int kNormMaxSplit = 8;   // splits whose loads are issued together (more: a plain loop)

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

__global__ __launch_bounds__(kPrepThreads) void k_rows_prep(PrepArgs a) {
  __shared__ float red[kPrepThreads / kWave];
  const int j = blockIdx.x;
  const int K = a.K;
  uint16_t* out = a.out + static_cast<long long>(j) * a.ld_out;
  int tj = j, hj = j;           // token index and hidden row of this row
  int32_t* err = a.err;
  if (a.batch <= 1) {
    const int err0 = a.kv_state ? a.kv_state[3] : 0;   // both words in one round trip
    const int nd0 = a.n_dev ? *a.n_dev : a.n_max;
    if (err0 != 0) return;
    const int n = min(max(nd0, 0), a.n_max);
    if (j >= n) return;
  } else {
    // session b's pair jj; rows past its count (or of a session in error) are zeros
    const int b = j / a.n_max, jj = j - b * a.n_max;
    const int32_t* sb = a.kv_state + 4 * b;
    const int nb = sb[3] != 0 ? 0 : (a.n_dev ? min(max(a.n_dev[b * a.ndev_sb], 0), a.n_max) : a.n_max);
    if (jj >= nb) {
      for (int k = threadIdx.x; k < K; k += kPrepThreads) out[k] = 0;
      return;
    }
    tj = b * a.tok_sb + jj;
    hj = b * a.hid_sb + jj;
    err = const_cast<int32_t*>(a.kv_state) + 4 * b + 3;   // the state words are writable
  }
  PrepRow r;
  if (a.in_mode == IN_EMBED) {
    const int tk = a.tok[tj];
    const bool ok = tk >= 0 && tk < a.vocab_tok;
    if (!ok && err && threadIdx.x == 0) *err = 4;   // token outside the vocabulary
    r.half = K / 2;
    r.src0 = ok ? a.embed : nullptr; r.off0 = static_cast<long long>(ok ? tk : 0) * r.half; r.bf0 = a.embed_bf16;
    r.src1 = a.hid; r.off1 = static_cast<long long>(hj) * a.ld_hid; r.bf1 = a.hid_bf16;
  } else {
    r.half = K;
    r.src0 = a.x; r.off0 = static_cast<long long>(j) * a.ldx; r.bf0 = 0;
    r.src1 = nullptr; r.off1 = 0; r.bf1 = 0;
  }
  const int njobs = K / 8;
  // pass 1: sums of squares (first part / second part)
  float se = 0.f, sh = 0.f;
  if (a.in_mode != IN_F32) {
    for (int f0 = threadIdx.x; f0 < njobs; f0 += kPrepThreads * kPrepU) {
      float v[kPrepU][8];
#pragma unroll
      for (int u = 0; u < kPrepU; ++u)
        if (f0 + u * kPrepThreads < njobs) prep_load(r, (f0 + u * kPrepThreads) * 8, v[u]);
#pragma unroll
      for (int u = 0; u < kPrepU; ++u) {
        const int k = (f0 + u * kPrepThreads) * 8;
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
  for (int f0 = threadIdx.x; f0 < njobs; f0 += kPrepThreads * kPrepU) {
    float v[kPrepU][8], w[kPrepU][8];
#pragma unroll
    for (int u = 0; u < kPrepU; ++u) {
      const int k = (f0 + u * kPrepThreads) * 8;
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
      const int k = (f0 + u * kPrepThreads) * 8;
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

// ---------------------------------------------------------------------------
// Several sessions' last rows as matrix-core products (o_proj, the MLP and the
// unembedding): k_last_rows_norm writes row b = bf16(x * w * inv) of session
// b's last row (zeros for a session with no row or a set error word), the
// products run over those rows, and k_argmax_rows turns each 4096-logit chunk
// of a logits row into one argmax key (the finishing kernel merges them as it
// merges the GEMV's).
__device__ __forceinline__ int last_row_of(const int32_t* state, const int32_t* n_dev, int ndev_sb, int n_max,
                                           int batch, int b) {
  if (b >= batch || state[4 * b + 3] != 0) return -1;
  const int n = n_dev ? min(max(n_dev[b * ndev_sb], 0), n_max) : n_max;
  return n > 0 ? n - 1 : -1;
}

__global__ __launch_bounds__(kPrepThreads) void k_last_rows_norm(LastRowsArgs a) {
  __shared__ float red[kPrepThreads / kWave];
  const int b = blockIdx.x;
  const int j = last_row_of(a.state, a.n_dev, a.ndev_sb, a.n_max, a.batch, b);
  uint16_t* out = a.out + static_cast<size_t>(b) * a.K;
  if (j < 0) {
    for (int k = threadIdx.x; k < a.K; k += kPrepThreads) out[k] = 0;
    return;
  }
  const float* x = a.x + (a.compact_in ? static_cast<size_t>(b) : static_cast<size_t>(b) * a.n_max + j) * a.K;
  float se = 0.f;
  for (int k = threadIdx.x; k < a.K; k += kPrepThreads) se += x[k] * x[k];
  const float inv = 1.0f / sqrtf(block_sum(se, red) / static_cast<float>(a.K) + a.eps);
  for (int k = threadIdx.x; k < a.K; k += kPrepThreads) {
    const float v = x[k];
    if (a.copy) {
      const size_t o = static_cast<size_t>(b) * a.copy_ld + k;
      if (a.copy_bf16) static_cast<uint16_t*>(a.copy)[o] = f32_to_bf16(v);
      else static_cast<float*>(a.copy)[o] = v;
    }
    const float w = a.nw_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(a.nw)[k]) : static_cast<const float*>(a.nw)[k];
    out[k] = f32_to_bf16(v * w * inv);
  }
}

hipError_t launch_last_rows_norm(const LastRowsArgs& a, hipStream_t s) {
  if (a.rows < 1 || a.K < 1 || a.rows < a.batch) return hipErrorInvalidValue;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_last_rows_norm, dim3(a.rows), dim3(kPrepThreads), 0, s, a);
  return hipGetLastError();
}

constexpr int kArgmaxChunk = 4096;

__global__ __launch_bounds__(256) void k_argmax_rows(ArgmaxRowsArgs a) {
  __shared__ unsigned long long s_best[4];
  const int c = blockIdx.x, b = blockIdx.y;
  const int lo = c * kArgmaxChunk, hi = min(a.V, lo + kArgmaxChunk);
  const bool valid = last_row_of(a.state, a.n_dev, a.ndev_sb, a.n_max, a.batch, b) >= 0;
  const float* row = a.logits + static_cast<size_t>(b) * a.ld;
  float* out = (valid && a.logits_out) ? a.logits_out + static_cast<size_t>(b) * a.out_sb * a.V : nullptr;
  unsigned long long best = 0ull;
  if (valid && a.copy) {
    const int per = (a.K + gridDim.x - 1) / gridDim.x;
    const int k1 = min(a.K, (c + 1) * per);
    const float* src = a.copy_src + static_cast<size_t>(b) * a.K;
    for (int k = c * per + threadIdx.x; k < k1; k += 256) {
      const size_t o = static_cast<size_t>(b) * a.copy_ld + k;
      if (a.copy_bf16) static_cast<uint16_t*>(a.copy)[o] = f32_to_bf16(src[k]);
      else static_cast<float*>(a.copy)[o] = src[k];
    }
  }
  if (valid) {
    for (int i = lo + threadIdx.x; i < hi; i += 256) {
      const float v = row[i];
      const unsigned long long key = argmax_key(v, static_cast<uint32_t>(i));
      best = key > best ? key : best;
      if (out) out[i] = v;
    }
  }
  best = wave_max_u64(best);
  if ((threadIdx.x & 63) == 0) s_best[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long m = s_best[0];
    for (int w = 1; w < 4; ++w) m = s_best[w] > m ? s_best[w] : m;
    a.parts[static_cast<size_t>(b) * a.nparts + c] = m;
  }
}

int argmax_rows_parts(int V) { return (V + kArgmaxChunk - 1) / kArgmaxChunk; }

hipError_t launch_argmax_rows(const ArgmaxRowsArgs& a, hipStream_t s) {
  if (a.batch < 1 || a.nparts != argmax_rows_parts(a.V)) return hipErrorInvalidValue;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_argmax_rows, dim3(a.nparts, a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rows_prep(const PrepArgs& a, hipStream_t s) {
  if (a.n_max <= 0) return hipSuccess;
  const int rows = a.batch > 1 ? a.batch * a.n_max : a.n_max;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_rows_prep, dim3(rows), dim3(kPrepThreads), 0, s, a);
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
    if (SWIGLU) {
      v = silu(v) * accu[i];
      if (a.y_bf16) {
        static_cast<uint16_t*>(static_cast<void*>(a.y))[static_cast<long long>(r) * a.ldy + col] = f32_to_bf16(v);
        continue;
      }
    }
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

// ---------------------------------------------------------------------------
// the weight-streaming product: every flush row in one workgroup
// ---------------------------------------------------------------------------
// A workgroup takes up to 256 activation rows and 128 weight rows (SwiGLU: 64
// gate and the matching 64 up rows) over one range of 64-column reduction
// steps, with two kinds of wave:
//
//   waves 0-3 (products): each owns 32 weight rows.  Its loads are coalesced:
//     load q of a step brings rows 8q .. 8q + 7, eight lanes per row's
//     128-byte slice (eight whole cache lines per instruction), issued three
//     steps ahead into a ring of three register slots; every weight byte is
//     loaded once, by one wave.  At its step the wave passes the slice through
//     a private padded LDS tile into the layout of the B operand of
//     v_mfma_f32_32x32x16_bf16: lane l takes weight row l % 32 at columns
//     k0 + 32 (l / 32) + 8 q + [0, 8) for reduction slice q.  The contraction
//     pairs A and B by position only, so the A operand of slice q is read from
//     LDS at the same columns.  (Loading straight into the B layout puts 32
//     rows, 32 bytes each, in every instruction; at the 27B shape that pattern
//     moved about a third of the bytes per second.)
//   waves 4-7 (staging): the activation rows of each step into a three-stage
//     LDS ring (rows padded by 16 bytes: conflict-free 16-byte reads), eight
//     lanes per row's slice, loads issued two steps ahead.
//
// The split keeps each kind's memory counter to its own loads (the counter
// completes in issue order, so one kind's waits never cover the other's
// younger loads).  Both kinds pass the same barriers: one per step.  The step
// loop has no early exit (exits in the middle of the three-step body cost the
// accumulators a second register set): the step count is rounded up to a
// multiple of three and the staging waves write zero activations for the
// extra steps, which then add exactly nothing.  With few
// output tiles the reduction range is split over workgroups; the partial sums
// go to a workspace and k_gemm_reduce adds them in split order and applies the
// epilogue.
constexpr int kSM = 256;          // activation rows per workgroup
constexpr int kSN = 128;          // weight rows per workgroup
constexpr int kSK = 64;           // reduction columns per step
constexpr int kSLd = kSK + 8;     // bf16 per LDS row
constexpr int kSWgs = 256;        // workgroups a split aims for (one per compute unit)
constexpr int kSMinSteps = 4;     // fewest steps a split takes
// Below this many weights the pipeline's fill and drain outweigh its streaming
// (the 64 x 64 tiles, many small workgroups, finish first).
constexpr long long kSMinWeights = 1LL << 22;

bool gemm_stream_supported(int M, int K, const int* m, int nmat, bool swiglu) {
  if (M <= 0 || K <= 0 || K % kSK) return false;
  if (static_cast<long long>(M) * K * (swiglu ? 2 : 1) < kSMinWeights) return false;
  if (swiglu) return M % (kSN / 2) == 0;
  if (M % kSN) return false;
  for (int i = 0; i < nmat; ++i)
    if (m[i] % kSN) return false;
  return true;
}

// tiles (workgroup column blocks) of a streaming product
static int stream_tiles(int M, bool swiglu) { return M / (swiglu ? kSN / 2 : kSN); }

// More tiles than workgroups in one round: stream-K (each workgroup an equal
// share of the (tile, step) units) instead of a second, mostly idle round.
static bool stream_k(int M, bool swiglu) { return stream_tiles(M, swiglu) > kSWgs; }

int gemm_split(int M, int K, bool swiglu) {
  if (swiglu || stream_k(M, swiglu)) return 1;
  const int tiles = M / kSN;
  int s = kSWgs / (tiles > 0 ? tiles : 1);
  const int cap = (K / kSK) / kSMinSteps;
  if (s > cap) s = cap;
  return s < 1 ? 1 : s;
}

size_t gemm_part_floats(int rows, int M, int K, const int* m, int nmat, bool swiglu) {
  if (!gemm_stream_supported(M, K, m, nmat, swiglu)) return 0;
  if (stream_k(M, swiglu)) return 2 * static_cast<size_t>(stream_tiles(M, swiglu)) * rows * kSN;   // head + tail
  const int s = gemm_split(M, K, swiglu);
  return s > 1 ? static_cast<size_t>(s) * rows * M : 0;
}

// residual add, store, optional act-dtype copy of four consecutive columns
__device__ __forceinline__ void gemm_put4(const GemmArgs& a, long long row, int col, float4 v) {
  if (a.out_mode == OUT_RESID) {
    const float4 q = *reinterpret_cast<const float4*>(a.res + row * a.ldres + col);
    v.x += q.x; v.y += q.y; v.z += q.z; v.w += q.w;
  }
  *reinterpret_cast<float4*>(a.y + row * a.ldy + col) = v;
  if (a.y2) {
    if (a.y2_bf16)
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.y2) + row * a.ldy2 + col) =
          make_uint2(f32_to_bf16(v.x) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16),
                     f32_to_bf16(v.z) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16));
    else
      *reinterpret_cast<float4*>(static_cast<float*>(a.y2) + row * a.ldy2 + col) = v;
  }
}

__device__ __forceinline__ void gemm_put(const GemmArgs& a, int r, int col, float v) {
  if (a.out_mode == OUT_RESID) v += a.res[static_cast<long long>(r) * a.ldres + col];
  a.y[static_cast<long long>(r) * a.ldy + col] = v;
  if (a.y2) {
    if (a.y2_bf16)
      static_cast<uint16_t*>(a.y2)[static_cast<long long>(r) * a.ldy2 + col] = f32_to_bf16(v);
    else
      static_cast<float*>(a.y2)[static_cast<long long>(r) * a.ldy2 + col] = v;
  }
}

// The product waves of k_gemm_stream: weights three steps ahead in registers,
// 32 weight rows a wave, all activation rows from LDS; the sums end in LDS as
// a row-major fp32 tile (column = wave * 32 + lane % 32).
template <bool SWIGLU, int NT>
__device__ __forceinline__ void gemm_stream_products(const GemmArgs& a, uint16_t* As, int kStage, int kTLd,
                                                     int r0, int tile, int sb, int nst, int nst3, int lane,
                                                     int wave, uint16_t* Wl) {
  // ---- product waves: this wave's 32 weight rows and their output columns
  const uint16_t* W;
  int wrow;
  if (SWIGLU) {
    W = wave < 2 ? a.w[0] : a.w[1];
    wrow = tile * (kSN / 2) + (wave & 1) * 32;
  } else {
    int cl = tile * kSN + wave * 32;
    W = a.w[0];
    if (cl >= a.m[0]) {
      cl -= a.m[0];
      W = a.w[1];
      if (cl >= a.m[1]) {
        cl -= a.m[1];
        W = a.w[2];
      }
    }
    wrow = cl;
  }
  // load q: row wrow + 8q + lane / 8, the 16 bytes at step column (lane % 8) * 8
  const char* bp = reinterpret_cast<const char*>(W + static_cast<long long>(wrow + (lane >> 3)) * a.K +
                                                 static_cast<long long>(sb) * kSK + (lane & 7) * 8);
  const long long qstride = static_cast<long long>(a.K) * 16;   // 8 rows, in bytes
  auto issue = [&](uint4 (&b)[4], int st) {
    st = min(st, nst - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) b[q] = load_stream16(bp + static_cast<long long>(st) * kSK * 2 + q * qstride);
  };
  f32x16_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16_t{};
  const int aoff = (lane & 31) * kSLd + (lane >> 5) * 32;
  uint16_t* wput = Wl + (lane >> 3) * kSLd + (lane & 7) * 8;
  auto compute = [&](int stage, const uint4 (&b)[4]) {
    const uint16_t* base = As + stage * kStage + aoff;
    // the step's 32 x 64 weight slice through the wave's LDS tile (only this
    // wave touches it; its LDS operations complete in issue order)
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<uint4*>(wput + q * 8 * kSLd) = b[q];
    __builtin_amdgcn_wave_barrier();
    // The operands of the next unit (a slice's A fragments for HT row blocks
    // and its B fragment) are read while the products of this unit run: two
    // register sets, so the LDS latency hides behind the matrix cores.  At 8
    // row blocks a unit is half a slice (a whole slice twice over would spill).
    constexpr int HT = NT > 4 ? NT / 2 : NT;    // row blocks per unit
    constexpr int UPQ = NT / HT;                // units per reduction slice
    uint4 av[2][HT], bv[2];
    auto fetch = [&](int u, uint4 (&ar)[HT], uint4& br) {
      const int q = u / UPQ, t0 = (u % UPQ) * HT;
      br = *reinterpret_cast<const uint4*>(Wl + aoff + q * 8);
#pragma unroll
      for (int t = 0; t < HT; ++t) ar[t] = *reinterpret_cast<const uint4*>(base + (t0 + t) * 32 * kSLd + q * 8);
    };
    fetch(0, av[0], bv[0]);
#pragma unroll
    for (int u = 0; u < 4 * UPQ; ++u) {
      if (u + 1 < 4 * UPQ) fetch(u + 1, av[(u + 1) & 1], bv[(u + 1) & 1]);
      const int t0 = (u % UPQ) * HT;
      const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, bv[u & 1]);
#pragma unroll
      for (int t = 0; t < HT; ++t)
        acc[t0 + t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av[u & 1][t]), bf,
                                                              acc[t0 + t], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_wave_barrier();   // the next step's writes follow these reads
  };
  uint4 b0[4], b1[4], b2[4];
  issue(b0, 0);
  issue(b1, 1);
  issue(b2, 2);
  __syncthreads();
  for (int s = 0; s < nst3; s += 3) {
    compute(0, b0);
    issue(b0, s + 3);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    compute(1, b1);
    issue(b1, s + 4);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    compute(2, b2);
    issue(b2, s + 5);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  }

  // accumulator element i of block t: row t * 32 + (i / 4) * 8 + (lane / 32) * 4
  // + i % 4, column lane % 32 of the wave's 32 (the staging ring is free after
  // the last step's barrier)
  float* T = reinterpret_cast<float*>(As);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = t * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
      T[r * kTLd + wave * 32 + (lane & 31)] = acc[t][i];
    }
}

// NT: 32-row blocks of activations computed (NT * 32 >= the rows a launch sees)
template <bool SWIGLU, int NT>
__global__ __launch_bounds__(512) void k_gemm_stream(GemmArgs a) {
  constexpr int kRows = NT * 32;
  constexpr int kStage = kSM * kSLd;                  // bf16 per LDS stage (256 rows)
  constexpr int kTLd = kSN + 4;                       // floats per row of the epilogue tile
  constexpr int kWTile = 32 * kSLd;                    // bf16 per product wave's weight tile
  constexpr int kLoop = (3 * kStage + 4 * kWTile) * 2;  // bytes: staging ring + weight tiles
  constexpr int kLds = kLoop > kRows * kTLd * 4 ? kLoop : kRows * kTLd * 4;
  __shared__ __attribute__((aligned(16))) uint16_t As[kLds / 2];
  if (a.kv_state && a.kv_state[3] != 0) return;
  int n = a.n_max;
  if (a.n_dev) n = min(max(*a.n_dev, 0), a.n_max);
  const int r0 = blockIdx.z * kSM;
  if (r0 >= n) return;
  const int rows = min(n - r0, kRows);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // this workgroup's work: one tile over one range of steps (split K), or with
  // stream-K a contiguous range of (tile, step) units that may end one tile
  // and begin the next
  const int steps = a.K / kSK;
  const int sp = blockIdx.y, nsp = gridDim.y;
  int u0, u1;
  if (a.sk_units) {
    const long long tot = static_cast<long long>(a.M / (SWIGLU ? kSN / 2 : kSN)) * steps;
    u0 = blockIdx.x * a.sk_units;
    u1 = static_cast<int>(min(tot, static_cast<long long>(u0) + a.sk_units));
  } else {
    u0 = blockIdx.x * steps + static_cast<int>(static_cast<long long>(steps) * sp / nsp);
    u1 = blockIdx.x * steps + static_cast<int>(static_cast<long long>(steps) * (sp + 1) / nsp);
  }
  for (int u = u0; u < u1;) {
    const int tile = u / steps;
    const int sb = u % steps;
    const int nst = min(steps - sb, u1 - u);
    const int nst3 = (nst + 2) / 3 * 3;             // steps run (the extra ones add zeros)
    // a stream-K piece of a tile: its sums go to the tile's head or tail slot
    const bool piece = a.sk_units && nst < steps;
    u += nst;

    if (wave >= 4) {
      // ---- staging waves: the step's slice of the NT * 32 activation rows into
      // LDS stage (step % 3).  Piece i of thread t is 16 bytes of row i * 32 +
      // t / 8 at column (t % 8) * 8, so eight neighbouring lanes read one row's
      // whole 128-byte slice (8 cache lines an instruction, not 64).  Rows past
      // n_max clamp (computed, never stored).
      const int t = tid - 256;
      const uint4* ap[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const int row = min(r0 + i * 32 + (t >> 3), a.n_max - 1);
        ap[i] = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.a) + static_cast<long long>(row) * a.lda +
                                               static_cast<long long>(sb) * kSK + (t & 7) * 8);
      }
      uint4 p0[NT], p1[NT], p2[NT];
      auto load = [&](uint4 (&p)[NT], int st) {
        st = min(st, nst - 1);
#pragma unroll
        for (int i = 0; i < NT; ++i) p[i] = ap[i][static_cast<long long>(st) * (kSK / 8)];
      };
      auto store = [&](const uint4 (&p)[NT], int stage, int st) {
        const uint32_t keep = st < nst ? 0xFFFFFFFFu : 0u;
        uint16_t* dst = As + stage * kStage + (t >> 3) * kSLd + (t & 7) * 8;
#pragma unroll
        for (int i = 0; i < NT; ++i)
          *reinterpret_cast<uint4*>(dst + i * 32 * kSLd) =
              make_uint4(p[i].x & keep, p[i].y & keep, p[i].z & keep, p[i].w & keep);
      };
      load(p0, 0);
      load(p1, 1);
      load(p2, 2);
      store(p0, 0, 0);
      __syncthreads();
      // during step s: store step s + 1 (issued two steps back), then issue
      // step s + 3 into the slot step s used
      // (the scheduling fences keep each step's register work on its side of
      // the barrier, so a wait for a slot never moves ahead of its step)
      for (int s = 0; s < nst3; s += 3) {
        store(p1, 1, s + 1);
        load(p0, s + 3);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        store(p2, 2, s + 2);
        load(p1, s + 4);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        store(p0, 0, s + 3);
        load(p2, s + 5);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      gemm_stream_products<SWIGLU, NT>(a, As, kStage, kTLd, r0, tile, sb, nst, nst3, lane, wave,
                                       As + 3 * kStage + wave * kWTile);
    }
    __syncthreads();   // the products' sums are in LDS (row-major, kTLd floats a row)

    // ---- epilogue: every thread, 16-byte pieces of whole rows
    const float* T = reinterpret_cast<const float*>(As);
    if (piece) {
      // all 128 columns of the tile (SwiGLU: gate, then up) into its head
      // (pieces starting at step 0) or tail slot; k_gemm_fixup adds them
      float* slot = a.part + (static_cast<long long>(tile) * 2 + (sb == 0 ? 0 : 1)) * a.n_max * kSN;
      for (int e = tid; e < rows * 32; e += 512) {
        const int r = e >> 5, c = (e & 31) * 4;
        *reinterpret_cast<float4*>(slot + static_cast<long long>(r0 + r) * kSN + c) =
            *reinterpret_cast<const float4*>(T + r * kTLd + c);
      }
    } else if (SWIGLU) {
      // columns [0, 64) hold the gate sums, [64, 128) the up sums of the same outputs
      for (int e = tid; e < rows * 16; e += 512) {
        const int r = e >> 4, c = (e & 15) * 4;
        const float4 g = *reinterpret_cast<const float4*>(T + r * kTLd + c);
        const float4 uu = *reinterpret_cast<const float4*>(T + r * kTLd + 64 + c);
        const float4 v = make_float4(silu(g.x) * uu.x, silu(g.y) * uu.y, silu(g.z) * uu.z, silu(g.w) * uu.w);
        const long long o = static_cast<long long>(r0 + r) * a.ldy + tile * (kSN / 2) + c;
        if (a.y_bf16) {
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(static_cast<void*>(a.y)) + o) =
              make_uint2(f32_to_bf16(v.x) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16),
                         f32_to_bf16(v.z) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16));
        } else {
          *reinterpret_cast<float4*>(a.y + o) = v;
        }
      }
    } else {
      for (int e = tid; e < rows * 32; e += 512) {
        const int r = e >> 5, c = (e & 31) * 4;
        float4 v = *reinterpret_cast<const float4*>(T + r * kTLd + c);
        const long long row = r0 + r;
        const int col = tile * kSN + c;
        if (nsp > 1) {
          *reinterpret_cast<float4*>(a.part + (static_cast<long long>(sp) * a.n_max + row) * a.M + col) = v;
          continue;
        }
        gemm_put4(a, row, col, v);
      }
    }
    __syncthreads();   // LDS is reused by the next piece
  }
}

// Stream-K tiles cut between two workgroups: head + tail (in that order), then
// the epilogue; a thread per four output columns of one row.
template <bool SWIGLU>
__global__ __launch_bounds__(256) void k_gemm_fixup(GemmArgs a, int steps) {
  if (a.kv_state && a.kv_state[3] != 0) return;
  int n = a.n_max;
  if (a.n_dev) n = min(max(*a.n_dev, 0), a.n_max);
  constexpr int kOut = SWIGLU ? kSN / 2 : kSN;        // output columns per tile
  const int tiles = a.M / kOut;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const int per_row = tiles * (kOut / 4);
  const int r = static_cast<int>(idx / per_row);
  const int q = static_cast<int>(idx % per_row);
  const int tile = q / (kOut / 4), c = (q % (kOut / 4)) * 4;
  if (r >= n) return;
  const long long first = static_cast<long long>(tile) * steps, last = first + steps - 1;
  if (first / a.sk_units == last / a.sk_units) return;   // one workgroup finished it
  const float* h = a.part + (static_cast<long long>(tile) * 2 * a.n_max + r) * kSN;
  const float* t = h + static_cast<long long>(a.n_max) * kSN;
  auto sum4 = [&](int col) {
    const float4 x = *reinterpret_cast<const float4*>(h + col), y = *reinterpret_cast<const float4*>(t + col);
    return make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
  };
  if (SWIGLU) {
    const float4 g = sum4(c), u = sum4(64 + c);
    const float4 v = make_float4(silu(g.x) * u.x, silu(g.y) * u.y, silu(g.z) * u.z, silu(g.w) * u.w);
    const long long o = static_cast<long long>(r) * a.ldy + tile * kOut + c;
    if (a.y_bf16) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(static_cast<void*>(a.y)) + o) =
          make_uint2(f32_to_bf16(v.x) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16),
                     f32_to_bf16(v.z) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16));
    } else {
      *reinterpret_cast<float4*>(a.y + o) = v;
    }
  } else {
    gemm_put4(a, r, tile * kOut + c, sum4(c));
  }
}

// Sum of the split partials in split order, then the epilogue; a thread per
// four consecutive output columns of one row.
__global__ __launch_bounds__(256) void k_gemm_reduce(GemmArgs a, int nsp) {
  const int per_row = a.M / 4;
  const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  const int r = static_cast<int>(idx / per_row);
  const int c = static_cast<int>(idx % per_row) * 4;
  if (r >= a.n_max) return;
  // the entry words and this thread's split partials in one memory round trip
  // (rows past the device count are read, not written)
  const int err0 = a.kv_state ? a.kv_state[3] : 0;
  const int nd0 = a.n_dev ? *a.n_dev : a.n_max;
  const long long stride = static_cast<long long>(a.n_max) * a.M;
  const float* p = a.part + static_cast<long long>(r) * a.M + c;
  float4 v = *reinterpret_cast<const float4*>(p);
  float4 pv[kNormMaxSplit];
  if (nsp <= kNormMaxSplit) {
#pragma unroll
    for (int q = 1; q < kNormMaxSplit; ++q)
      if (q < nsp) pv[q] = *reinterpret_cast<const float4*>(p + q * stride);
  }
  if (err0 != 0) return;
  const int n = min(max(nd0, 0), a.n_max);
  if (r >= n) return;
  if (nsp <= kNormMaxSplit) {
    // added in split order
#pragma unroll
    for (int q = 1; q < kNormMaxSplit; ++q)
      if (q < nsp) {
        v.x += pv[q].x; v.y += pv[q].y; v.z += pv[q].z; v.w += pv[q].w;
      }
  } else {
    for (int q = 1; q < nsp; ++q) {
      const float4 w = *reinterpret_cast<const float4*>(p + q * stride);
      v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
    }
  }
  gemm_put(a, r, c, v.x);
  gemm_put(a, r, c + 1, v.y);
  gemm_put(a, r, c + 2, v.z);
  gemm_put(a, r, c + 3, v.w);
}

// The split reduce of a product whose output feeds a normalised row: one
// workgroup of 1024 threads per row sums the partials in split order (all of a
// column's split loads issued together), applies the epilogue (residual,
// act-dtype copy), keeps the row in registers and writes bf16(y * w * (1 /
// rms(y))) -- the row preparation the next product reads.
__global__ __launch_bounds__(kNormThreads) void k_gemm_reduce_norm(GemmArgs a, int nsp, RowNorm rn) {
  __shared__ float red[kNormThreads / kWave];
  const int r = blockIdx.x;
  const int per = a.M / 4;
  const long long stride = static_cast<long long>(a.n_max) * a.M;
  // every load first (one memory round trip): the entry words, the split
  // partials, the residual and the norm weight of this thread's columns (rows
  // past the device count are read, not written)
  const int err0 = a.kv_state ? a.kv_state[3] : 0;
  const int nd0 = a.n_dev ? *a.n_dev : a.n_max;
  float4 pv[kNormPer][kNormMaxSplit], rv[kNormPer];
  uint2 wb[kNormPer];
  float4 wf[kNormPer];
#pragma unroll
  for (int i = 0; i < kNormPer; ++i) {
    const int c4 = threadIdx.x + i * kNormThreads;
    if (c4 >= per) continue;
    const int c = c4 * 4;
    const float* p = a.part + static_cast<long long>(r) * a.M + c;
#pragma unroll
    for (int q = 0; q < kNormMaxSplit; ++q)
      if (q < nsp) pv[i][q] = *reinterpret_cast<const float4*>(p + q * stride);
    if (a.out_mode == OUT_RESID) rv[i] = *reinterpret_cast<const float4*>(a.res + static_cast<long long>(r) * a.ldres + c);
    if (rn.nw_bf16) wb[i] = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(rn.nw) + c);
    else wf[i] = *reinterpret_cast<const float4*>(static_cast<const float*>(rn.nw) + c);
  }
  if (err0 != 0) return;
  const int n = min(max(nd0, 0), a.n_max);
  if (r >= n) return;
  float4 v[kNormPer];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kNormPer; ++i) {
    const int c4 = threadIdx.x + i * kNormThreads;
    if (c4 >= per) continue;
    const int c = c4 * 4;
    float4 t = pv[i][0];
#pragma unroll
    for (int q = 1; q < kNormMaxSplit; ++q)
      if (q < nsp) {
        t.x += pv[i][q].x; t.y += pv[i][q].y; t.z += pv[i][q].z; t.w += pv[i][q].w;
      }
    if (a.out_mode == OUT_RESID) {
      t.x += rv[i].x; t.y += rv[i].y; t.z += rv[i].z; t.w += rv[i].w;
    }
    *reinterpret_cast<float4*>(a.y + static_cast<long long>(r) * a.ldy + c) = t;
    if (a.y2) {
      if (a.y2_bf16)
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.y2) + static_cast<long long>(r) * a.ldy2 + c) =
            make_uint2(f32_to_bf16(t.x) | (static_cast<uint32_t>(f32_to_bf16(t.y)) << 16),
                       f32_to_bf16(t.z) | (static_cast<uint32_t>(f32_to_bf16(t.w)) << 16));
      else
        *reinterpret_cast<float4*>(static_cast<float*>(a.y2) + static_cast<long long>(r) * a.ldy2 + c) = t;
    }
    v[i] = t;
    ss += t.x * t.x + t.y * t.y + t.z * t.z + t.w * t.w;
  }
  const float inv = 1.0f / sqrtf(block_sum(ss, red) / static_cast<float>(a.M) + rn.eps);
  uint16_t* out = rn.out + static_cast<long long>(r) * rn.ld_out;
#pragma unroll
  for (int i = 0; i < kNormPer; ++i) {
    const int c4 = threadIdx.x + i * kNormThreads;
    if (c4 >= per) continue;
    const int c = c4 * 4;
    float w[4];
    if (rn.nw_bf16) {
      const uint2 u = wb[i];
      w[0] = __uint_as_float(u.x << 16); w[1] = __uint_as_float(u.x & 0xFFFF0000u);
      w[2] = __uint_as_float(u.y << 16); w[3] = __uint_as_float(u.y & 0xFFFF0000u);
    } else {
      const float4 f = wf[i];
      w[0] = f.x; w[1] = f.y; w[2] = f.z; w[3] = f.w;
    }
    *reinterpret_cast<uint2*>(out + c) =
        make_uint2(f32_to_bf16(v[i].x * w[0] * inv) | (static_cast<uint32_t>(f32_to_bf16(v[i].y * w[1] * inv)) << 16),
                   f32_to_bf16(v[i].z * w[2] * inv) | (static_cast<uint32_t>(f32_to_bf16(v[i].w * w[3] * inv)) << 16));
  }
}

bool gemm_supported(int M, int K, const int* m, int nmat) {
  if (M <= 0 || K <= 0 || M % kTN || K % kTK) return false;
  for (int i = 0; i < nmat; ++i)
    if (m[i] % kTN) return false;
  return true;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s, const RowNorm* rn, bool* normed, int* split_left) {
  if (normed) *normed = false;
  if (split_left) *split_left = 1;
  if (a.n_max <= 0) return hipSuccess;
  const bool swiglu = a.out_mode == OUT_SWIGLU;
  (void)hipGetLastError();
  // the streaming epilogue moves 16-byte pieces: leading dimensions in whole
  // pieces, buffers aligned to them
  auto al = [](const void* p, int b) { return (reinterpret_cast<uintptr_t>(p) & (b - 1)) == 0; };
  const bool pieces = a.ldy % 4 == 0 && al(a.y, 16) && al(a.part, 16) &&
                      (a.out_mode != OUT_RESID || (a.ldres % 4 == 0 && al(a.res, 16))) &&
                      (!a.y2 || (a.ldy2 % 4 == 0 && al(a.y2, 16)));
  if (gemm_stream_supported(a.M, a.K, a.m, swiglu ? 2 : 3, swiglu) && !a.a_f32 && pieces) {
    const int nsp = gemm_split(a.M, a.K, swiglu);
    const bool sk = stream_k(a.M, swiglu);
    if ((nsp > 1 || sk) && !a.part) return hipErrorInvalidValue;
    GemmArgs b = a;
    const int tiles = stream_tiles(a.M, swiglu), steps = a.K / kSK;
    const long long units = static_cast<long long>(tiles) * steps;
    b.sk_units = sk ? static_cast<int>((units + kSWgs - 1) / kSWgs) : 0;
    const int gx = sk ? static_cast<int>((units + b.sk_units - 1) / b.sk_units) : tiles;
    const dim3 grid(gx, nsp, (a.n_max + kSM - 1) / kSM);
    // 32-row blocks computed: enough for every row a launch can see
    const int nt = a.n_max > 128 ? 8 : (a.n_max > 64 ? 4 : 2);
#define MTP_STREAM(SW, NT) hipLaunchKernelGGL((k_gemm_stream<SW, NT>), grid, dim3(512), 0, s, b)
    if (swiglu) {
      if (nt == 8) MTP_STREAM(true, 8); else if (nt == 4) MTP_STREAM(true, 4); else MTP_STREAM(true, 2);
    } else {
      if (nt == 8) MTP_STREAM(false, 8); else if (nt == 4) MTP_STREAM(false, 4); else MTP_STREAM(false, 2);
    }
#undef MTP_STREAM
    if (nsp > 1 && split_left && !rn && a.out_mode == OUT_F32) {
      *split_left = nsp;                       // the caller's next kernel reduces
    } else if (nsp > 1) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (rn && a.out_mode != OUT_SWIGLU && a.M <= kNormThreads * 4 * kNormPer && a.M % 4 == 0 &&
          nsp <= kNormMaxSplit && rn->ld_out % 4 == 0 && al(rn->out, 8)) {
        hipLaunchKernelGGL(k_gemm_reduce_norm, dim3(static_cast<unsigned>(a.n_max)), dim3(kNormThreads), 0, s, a,
                           nsp, *rn);
        if (normed) *normed = true;
      } else {
        const long long threads = static_cast<long long>(a.n_max) * (a.M / 4);
        hipLaunchKernelGGL(k_gemm_reduce, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, s, a,
                           nsp);
      }
    }
    if (sk) {
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const long long threads = static_cast<long long>(a.n_max) * (a.M / 4);
      const dim3 fg(static_cast<unsigned>((threads + 255) / 256));
      if (swiglu) hipLaunchKernelGGL(k_gemm_fixup<true>, fg, dim3(256), 0, s, b, steps);
      else hipLaunchKernelGGL(k_gemm_fixup<false>, fg, dim3(256), 0, s, b, steps);
    }
    return hipGetLastError();
  }
  const dim3 grid(a.M / kTN, (a.n_max + kTM - 1) / kTM);
  if (swiglu)
    hipLaunchKernelGGL(k_gemm<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_gemm<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mtp
