// Draft-KV append and attention over the draft KV for few query rows (the
// batch-1 step and small in-round flushes).
//
// k_rope_append: per (row, head) wave: per-head RMSNorm of q or k over head_dim,
//   rotate-half RoPE at position state[0] + row (angle computed in fp64), k and v
//   appended to the cache in the KV dtype, roped q kept in fp32.  Capacity and
//   count checks set the sticky error word; the last workgroup advances the
//   length (and the round base when asked).
// k_attn: split-K attention.  Workgroup (chunk, kv head, row) covers a
//   contiguous key range; lanes are laid along head_dim so each K/V row is read
//   with coalesced 16-byte loads, and the GQA group's query heads share every
//   key load.  Scores, then exp, then P.V; unnormalised partials (o, max, sum).
// k_attn_merge: fixed-order log-sum-exp merge of the chunk partials.
#include "common.h"
#include "kernels.h"

namespace mtp {

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_rope_append(RopeArgs a) {
  __shared__ float sv[256];
  int32_t* st = a.state;
  if (st[3] != 0) return;
  const int ndev = a.n_dev ? *a.n_dev : a.n_max;
  const int len0 = st[0];
  const bool bad_count = ndev < 0 || ndev > a.n_max;
  const int n = bad_count ? 0 : ndev;
  if (bad_count || len0 + n > a.capacity) {
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
      st[3] = bad_count ? 3 : 1;
    return;
  }
  const int j = blockIdx.x;
  const int lane = threadIdx.x;
  if (j < n) {
    const int h = blockIdx.y;
    const int D = a.d;
    const int half = D / 2;
    const int pos = len0 + j;
    const bool is_q = h < a.hq;
    const int kvh = h - a.hq;
    const float* row = a.qkv + static_cast<size_t>(j) * a.ld_qkv;
    const float* src = is_q ? row + h * D : row + a.hq * D + kvh * D;
    const void* nw = is_q ? a.q_norm : a.k_norm;
    float ss = 0.f;
    for (int d = lane; d < D; d += 64) ss += src[d] * src[d];
    ss = wave_sum(ss);
    const float inv = rsqrtf(ss / static_cast<float>(D) + a.eps);
    for (int d = lane; d < D; d += 64) {
      const float w = a.nw_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(nw)[d])
                                : static_cast<const float*>(nw)[d];
      sv[d] = src[d] * inv * w;
    }
    __syncthreads();
    for (int i = lane; i < half; i += 64) {
      const double invf = pow(static_cast<double>(a.theta), -2.0 * i / D);
      const double ang = static_cast<double>(pos) * invf;
      const float c = static_cast<float>(cos(ang));
      const float s = static_cast<float>(sin(ang));
      const float x1 = sv[i], x2 = sv[i + half];
      const float o1 = x1 * c - x2 * s;
      const float o2 = x1 * s + x2 * c;
      if (is_q) {
        float* q = a.q_out + static_cast<size_t>(j) * a.hq * D + h * D;
        q[i] = o1;
        q[i + half] = o2;
      } else {
        const size_t off = (static_cast<size_t>(kvh) * a.capacity + pos) * D;
        if (a.kv_bf16) {
          static_cast<uint16_t*>(a.kc)[off + i] = f32_to_bf16(o1);
          static_cast<uint16_t*>(a.kc)[off + i + half] = f32_to_bf16(o2);
        } else {
          static_cast<float*>(a.kc)[off + i] = o1;
          static_cast<float*>(a.kc)[off + i + half] = o2;
        }
      }
    }
    if (!is_q) {
      const float* vsrc = row + (a.hq + a.hkv) * D + kvh * D;
      const size_t off = (static_cast<size_t>(kvh) * a.capacity + pos) * D;
      for (int d = lane; d < D; d += 64) {
        if (a.kv_bf16) static_cast<uint16_t*>(a.vc)[off + d] = f32_to_bf16(vsrc[d]);
        else static_cast<float*>(a.vc)[off + d] = vsrc[d];
      }
    }
  }
  // all workgroups have read state[0]; the last one advances it
  const bool last = last_block_ticket(a.counter, gridDim.x * gridDim.y);
  if (last && threadIdx.x == 0) {
    st[0] = len0 + n;
    if (a.set_base) st[1] = len0 + n;
  }
}

hipError_t launch_rope_append(const RopeArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_rope_append, dim3(a.n_max, a.hq + a.hkv), dim3(64), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kMaxChunk = 512;

template <bool KVB, int D, int G>
__global__ __launch_bounds__(kAttnThreads) void k_attn(AttnArgs a) {
  constexpr int EPL = KVB ? 8 : 4;   // elements per lane (16 bytes)
  constexpr int LPK = D / EPL;       // lanes per key row
  constexpr int KPI = 64 / LPK;      // keys per wave instruction
  __shared__ float qs[G][D];
  __shared__ float sc[kMaxChunk][G];
  __shared__ float red[kAttnWaves][G];
  __shared__ float stat[2][G];
  __shared__ float oacc[kAttnWaves][G][D];

  const int32_t* st = a.state;
  if (st[3] != 0) return;
  int n = a.n_max;
  if (a.n_dev) n = min(max(*a.n_dev, 0), a.n_max);
  const int j = (a.row_sel == ROW_LAST) ? n - 1 : static_cast<int>(blockIdx.z);
  if (j < 0 || j >= n) return;
  const int off = st[0] - n;        // the rows' K/V are already appended
  const int L = off + j + 1;        // keys visible to row j
  const int h = blockIdx.y;
  const int c = blockIdx.x;
  int ck = (L + a.nchunk - 1) / a.nchunk;
  ck = (ck + 15) & ~15;
  const int k0 = c * ck;
  const int k1 = min(L, k0 + ck);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t pbase = (static_cast<size_t>(j) * a.hq + h * G) * a.nchunk + c;

  if (k0 >= k1) {
    for (int idx = tid; idx < G * D; idx += kAttnThreads) {
      const int g = idx / D, d = idx - g * D;
      a.part_o[(pbase + static_cast<size_t>(g) * a.nchunk) * D + d] = 0.f;
    }
    if (tid < G) {
      a.part_ml[(pbase + static_cast<size_t>(tid) * a.nchunk) * 2] = -INFINITY;
      a.part_ml[(pbase + static_cast<size_t>(tid) * a.nchunk) * 2 + 1] = 0.f;
    }
    return;
  }

  const float scale = rsqrtf(static_cast<float>(D));
  for (int idx = tid; idx < G * D; idx += kAttnThreads) {
    const int g = idx / D, d = idx - g * D;
    qs[g][d] = a.q[static_cast<size_t>(j) * a.hq * D + (h * G + g) * D + d] * scale;
  }
  __syncthreads();

  const int grp = lane / LPK;
  const int li = lane % LPK;
  const int d0 = li * EPL;
  float qr[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) qr[g][e] = qs[g][d0 + e];

  const size_t head_off = static_cast<size_t>(h) * a.capacity * D;
  const char* kbase = static_cast<const char*>(a.kc) + head_off * (KVB ? 2 : 4);
  const char* vbase = static_cast<const char*>(a.vc) + head_off * (KVB ? 2 : 4);
  constexpr int row_bytes = D * (KVB ? 2 : 4);

  // scores
  // wave-uniform trip count so every lane takes part in the group reductions
  for (int base = k0 + wave * KPI; base < k1; base += KPI * kAttnWaves) {
    const int kk = base + grp;
    const bool ok = kk < k1;
    uint4 kv = make_uint4(0u, 0u, 0u, 0u);
    if (ok) kv = *reinterpret_cast<const uint4*>(kbase + static_cast<size_t>(kk) * row_bytes + d0 * (KVB ? 2 : 4));
    float kf[EPL];
    if constexpr (KVB) {
      const uint32_t w[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) { kf[2 * q] = __uint_as_float(w[q] << 16); kf[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u); }
    } else {
      kf[0] = __uint_as_float(kv.x); kf[1] = __uint_as_float(kv.y); kf[2] = __uint_as_float(kv.z); kf[3] = __uint_as_float(kv.w);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) p += qr[g][e] * kf[e];
      p = group_sum(p, LPK);
      if (ok && li == 0) sc[kk - k0][g] = p;
    }
  }
  __syncthreads();

  // max and exp-sum per query head
  const int cn = k1 - k0;
  {
    float m[G];
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = -INFINITY;
    for (int i = tid; i < cn; i += kAttnThreads)
#pragma unroll
      for (int g = 0; g < G; ++g) m[g] = fmaxf(m[g], sc[i][g]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float v = wave_max(m[g]);
      if (lane == 0) red[wave][g] = v;
    }
    __syncthreads();
    if (tid < G) {
      float v = red[0][tid];
      for (int w = 1; w < kAttnWaves; ++w) v = fmaxf(v, red[w][tid]);
      stat[0][tid] = v;
    }
    __syncthreads();
    float l[G];
#pragma unroll
    for (int g = 0; g < G; ++g) l[g] = 0.f;
    for (int i = tid; i < cn; i += kAttnThreads)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = __expf(sc[i][g] - stat[0][g]);
        sc[i][g] = p;
        l[g] += p;
      }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float v = wave_sum(l[g]);
      if (lane == 0) red[wave][g] = v;
    }
    __syncthreads();
    if (tid < G) {
      float v = 0.f;
      for (int w = 0; w < kAttnWaves; ++w) v += red[w][tid];
      stat[1][tid] = v;
    }
    __syncthreads();
  }

  // P . V
  float acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  for (int kk = k0 + wave * KPI + grp; kk < k1; kk += KPI * kAttnWaves) {
    const uint4 vv = *reinterpret_cast<const uint4*>(vbase + static_cast<size_t>(kk) * row_bytes + d0 * (KVB ? 2 : 4));
    float vf[EPL];
    if constexpr (KVB) {
      const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) { vf[2 * q] = __uint_as_float(w[q] << 16); vf[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u); }
    } else {
      vf[0] = __uint_as_float(vv.x); vf[1] = __uint_as_float(vv.y); vf[2] = __uint_as_float(vv.z); vf[3] = __uint_as_float(vv.w);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float p = sc[kk - k0][g];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] += p * vf[e];
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float v = acc[g][e];
      for (int o = LPK; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
      acc[g][e] = v;
    }
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) oacc[wave][g][d0 + e] = acc[g][e];
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kAttnThreads) {
    const int g = idx / D, d = idx - g * D;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) v += oacc[w][g][d];
    a.part_o[(pbase + static_cast<size_t>(g) * a.nchunk) * D + d] = v;
  }
  if (tid < G) {
    a.part_ml[(pbase + static_cast<size_t>(tid) * a.nchunk) * 2] = stat[0][tid];
    a.part_ml[(pbase + static_cast<size_t>(tid) * a.nchunk) * 2 + 1] = stat[1][tid];
  }
}

__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  const int32_t* st = a.state;
  if (st[3] != 0) return;
  int n = a.n_max;
  if (a.n_dev) n = min(max(*a.n_dev, 0), a.n_max);
  const int j = (a.row_sel == ROW_LAST) ? n - 1 : static_cast<int>(blockIdx.y);
  if (j < 0 || j >= n) return;
  const int hq = blockIdx.x;
  const int D = a.d;
  const size_t base = (static_cast<size_t>(j) * a.hq + hq) * a.nchunk;
  float M = -INFINITY;
  for (int c = 0; c < a.nchunk; ++c) M = fmaxf(M, a.part_ml[(base + c) * 2]);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float num = 0.f, den = 0.f;
    for (int c = 0; c < a.nchunk; ++c) {
      const float mc = a.part_ml[(base + c) * 2];
      if (mc == -INFINITY) continue;
      const float w = __expf(mc - M);
      num += w * a.part_o[(base + c) * D + d];
      den += w * a.part_ml[(base + c) * 2 + 1];
    }
    a.o[static_cast<size_t>(j) * a.hq * D + hq * D + d] = num / den;
  }
}

template <bool KVB, int D>
static hipError_t attn_d(const AttnArgs& a, dim3 grid, hipStream_t s) {
  const int g = a.hq / a.hkv;
  (void)hipGetLastError();
  switch (g) {
    case 1: hipLaunchKernelGGL((k_attn<KVB, D, 1>), grid, dim3(kAttnThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_attn<KVB, D, 2>), grid, dim3(kAttnThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_attn<KVB, D, 3>), grid, dim3(kAttnThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_attn<KVB, D, 4>), grid, dim3(kAttnThreads), 0, s, a); break;
    case 6: hipLaunchKernelGGL((k_attn<KVB, D, 6>), grid, dim3(kAttnThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_attn<KVB, D, 8>), grid, dim3(kAttnThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int rows = (a.row_sel == ROW_LAST) ? 1 : a.n_max;
  const dim3 grid(a.nchunk, a.hkv, rows);
  hipError_t e;
  if (a.kv_bf16) {
    switch (a.d) {
      case 64: e = attn_d<true, 64>(a, grid, s); break;
      case 128: e = attn_d<true, 128>(a, grid, s); break;
      case 256: e = attn_d<true, 256>(a, grid, s); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.d) {
      case 64: e = attn_d<false, 64>(a, grid, s); break;
      case 128: e = attn_d<false, 128>(a, grid, s); break;
      case 256: e = attn_d<false, 256>(a, grid, s); break;
      default: return hipErrorInvalidValue;
    }
  }
  if (e != hipSuccess) return e;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_attn_merge, dim3(a.hq, rows), dim3(a.d < 256 ? a.d : 256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mtp
