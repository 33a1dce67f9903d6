// Causal attention of the many-row pending-pair flush on the gfx950 matrix
// cores (bf16 draft KV).
//
// Flush row j (slot off + j) attends over keys [0, off + j] of its kv head
// (the head's own draft cache; "feat(inference): support the qwen3_5_mtp
// drafter ...", section "Upstream contract to port": one full-attention layer).
// The query vectors of a kv head are the (row, grouped head) pairs, taken 64 at
// a time by a workgroup (16 per wave) over one key chunk; chunks are merged by
// the log-sum-exp merge of the split-K decode path, so the partial (o, m, l)
// layout is the same.
//
// Per 64-key block a wave computes its 16 x 64 scores transposed, S^T = K Q^T,
// with v_mfma_f32_16x16x32_bf16 (K rows straight from LDS as the A operand, the
// wave's bf16 queries held in registers as B), runs the online softmax per
// query (a query's 64 scores sit in the four lanes that share lane % 16), and
// accumulates O^T += V^T P^T: the probabilities never leave registers, because
// the B operand of that product takes each lane's own score values (keys
// 32s + 4 (lane/16) + {0..3} and 32s + 16 + 4 (lane/16) + {0..3}) and the A
// operand reads V^T (staged transposed in LDS) at the same keys.
//
// Scores are kept in the exp2 domain (log2 e is folded into the query scale),
// so each probability is one v_exp_f32; the causal and chunk-end masks are
// applied only to the blocks that reach them.  The chunks of the many-row flush
// are merged by k_attn_merge_rows, one wave per (row, head).
#include "common.h"
#include "kernels.h"

namespace mtp {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8v;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4v;

constexpr int kFKeys = 64;     // keys per block
constexpr int kFQ = 64;        // query vectors per workgroup (16 per wave)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Two floats as packed bf16 (low half first), rounded to nearest even by the
// gfx950 conversion instruction.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v;
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2v v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_attn_flush(AttnArgs a) {
  constexpr int KLD = D + 8;          // bf16 per LDS K row
  constexpr int VLD = kFKeys + 4;     // bf16 per LDS V^T row (34 words: 16 rows hit distinct banks)
  constexpr int DK = D / 32;          // 32-wide head_dim steps of S^T
  constexpr int DT = D / 16;          // 16-row head_dim tiles of O^T
  constexpr float kNeg = -INFINITY;
  // S register stages of K/V loads in flight and NB LDS buffers: head_dim
  // 64 and 128 keep two blocks in flight and double-buffer LDS (one barrier
  // per block); head_dim 256 needs its registers for the accumulators
  constexpr int S = D <= 128 ? 2 : 1;
  constexpr int NB = D <= 128 ? 2 : 1;
  constexpr int KSZ = kFKeys * KLD, VSZ = D * VLD;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[NB * KSZ];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[NB * VSZ];

  const int32_t* st = a.state;
  if (st[3] != 0) return;
  int n = a.n_max;
  if (a.n_dev) n = min(max(*a.n_dev, 0), a.n_max);
  const int G = a.hq / a.hkv;
  const int nq = n * G;
  const int qb = blockIdx.y * kFQ;
  if (qb >= nq) return;
  const int kvh = blockIdx.z;
  const int c = blockIdx.x;
  const int off = st[0];                    // pre-append length (committed by k_finish)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // the key chunk, and the keys this workgroup's rows can see
  int ck = (off + n + a.nchunk - 1) / a.nchunk;
  ck = (ck + kFKeys - 1) / kFKeys * kFKeys;
  const int jmax = min(n, (qb + kFQ - 1) / G + 1) - 1;      // last row in this workgroup
  const int k0 = c * ck;
  const int k1 = min(k0 + ck, off + jmax + 1);

  // this lane's query vector (column lane % 16 of the wave's S^T tiles)
  const int qv = qb + wave * 16 + (lane & 15);
  const bool qok = qv < nq;
  const int jq = qok ? qv / G : 0;
  const int head = kvh * G + (qok ? qv % G : 0);
  const int kmax = off + jq;                                 // last key row jq sees
  const int kmax_wave = off + (qb + wave * 16) / G;          // the same for the wave's first row
  const float scale = rsqrtf(static_cast<float>(D)) * kLog2e;   // scores in the exp2 domain
  bf16x8v qf[DK];
  {
    // (jq, head) is a valid row for every lane, so all loads are issued
    // unconditionally and at once; lanes past the last query take zeros
    const float* qp = a.q + (static_cast<size_t>(jq) * a.hq + head) * D + (lane >> 4) * 8;
    const float qs = qok ? scale : 0.f;
    float4 qv[DK][2];
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      qv[dk][0] = *reinterpret_cast<const float4*>(qp + dk * 32);
      qv[dk][1] = *reinterpret_cast<const float4*>(qp + dk * 32 + 4);
    }
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) {
      const float x[8] = {qv[dk][0].x, qv[dk][0].y, qv[dk][0].z, qv[dk][0].w,
                          qv[dk][1].x, qv[dk][1].y, qv[dk][1].z, qv[dk][1].w};
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i] * qs, x[2 * i + 1] * qs);
      qf[dk] = __builtin_bit_cast(bf16x8v, make_uint4(w[0], w[1], w[2], w[3]));
    }
  }

  f32x4v acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = f32x4v{0.f, 0.f, 0.f, 0.f};
  float m = kNeg, l = 0.f;

  const uint16_t* kc = static_cast<const uint16_t*>(a.kc) + static_cast<size_t>(kvh) * a.capacity * D;
  const uint16_t* vc = static_cast<const uint16_t*>(a.vc) + static_cast<size_t>(kvh) * a.capacity * D;
  // staging of a 64-key block (keys past k1 read the last key: their scores are
  // masked, so their V rows meet zero probabilities):
  //   K rows  thread t moves 16-byte pieces t, t + 256, ... (row-major)
  //   V^T     thread t takes KB = D / 32 keys KB (t % NG) + [0, KB) at dims
  //           8 (t / NG) + [0, 8), transposes the KB x 8 block in registers and
  //           writes 8 rows of KB keys of V^T (consecutive lanes write
  //           consecutive words of a row: conflict-free)
  constexpr int kKPer = kFKeys * D / 8 / 256;                // K pieces per thread
  constexpr int KB = D / 32;                                 // V keys per thread
  constexpr int NG = kFKeys / KB;                            // V key groups
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  u32x4v kpf[S][kKPer], vpf[S][KB];   // native vectors: kept in registers across the loop
  const int vg = tid % NG, vd = (tid / NG) * 8;
  // the loads of the block at kb into stage q (written out, not in a lambda:
  // the arrays must stay in registers)
#define MTP_FLUSH_LOAD(q, kb)                                                              \
  {                                                                                        \
    _Pragma("unroll") for (int u = 0; u < kKPer; ++u) {                                    \
      const int e = tid + 256 * u;                                                         \
      const int key = min((kb) + e / (D / 8), k1 - 1), d8 = (e % (D / 8)) * 8;             \
      kpf[q][u] = *reinterpret_cast<const u32x4v*>(kc + static_cast<size_t>(key) * D + d8); \
    }                                                                                      \
    _Pragma("unroll") for (int j = 0; j < KB; ++j) {                                       \
      const int key = min((kb) + vg * KB + j, k1 - 1);                                     \
      vpf[q][j] = *reinterpret_cast<const u32x4v*>(vc + static_cast<size_t>(key) * D + vd); \
    }                                                                                      \
  }

  if (k0 < k1) {
#pragma unroll
    for (int q = 0; q < S; ++q) MTP_FLUSH_LOAD(q, k0 + q * kFKeys);
  }
  for (int kb0 = k0; kb0 < k1; kb0 += S * kFKeys) {
#pragma unroll
  for (int q = 0; q < S; ++q) {
    const int kb = kb0 + q * kFKeys;
    if (kb >= k1) break;   // uniform over the workgroup
    uint16_t* const Kb = Ks + (q % NB) * KSZ;
    uint16_t* const Vb = Vt + (q % NB) * VSZ;
    // one LDS buffer: wait until the previous block's operand reads are done;
    // two: the barrier of the previous block already ordered the reads of this
    // buffer (two blocks back) before these writes
    if (NB == 1) __syncthreads();
#pragma unroll
    for (int u = 0; u < kKPer; ++u) {
      const int e = tid + 256 * u;
      *reinterpret_cast<u32x4v*>(Kb + (e / (D / 8)) * KLD + (e % (D / 8)) * 8) = kpf[q][u];
    }
    {
      // word w of a piece holds dims 2w (low half) and 2w + 1 (high half)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t o[KB / 2];
#pragma unroll
        for (int p = 0; p < KB / 2; ++p) {
          const uint32_t lo = vpf[q][2 * p][i >> 1], hi = vpf[q][2 * p + 1][i >> 1];
          o[p] = (i & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
        uint16_t* dst = Vb + (vd + i) * VLD + vg * KB;
        if constexpr (KB == 2) {
          *reinterpret_cast<uint32_t*>(dst) = o[0];
        } else {
#pragma unroll
          for (int p = 0; p < KB / 2; p += 2)
            *reinterpret_cast<uint2*>(dst + 2 * p) = make_uint2(o[p], o[p + 1]);
        }
      }
    }
    __syncthreads();
    // the loads S blocks ahead fly during the products (unconditional: past
    // the last block they reload the clamped last key, unused; a conditional
    // load would keep the arrays out of registers)
    MTP_FLUSH_LOAD(q, kb + S * kFKeys);

    // S^T for four 16-key tiles
    f32x4v s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dk = 0; dk < DK; ++dk) {
        const bf16x8v kf = __builtin_bit_cast(bf16x8v,
            *reinterpret_cast<const uint4*>(Kb + (kt * 16 + (lane & 15)) * KLD + dk * 32 + (lane >> 4) * 8));
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[dk], s[kt], 0, 0, 0);
      }
    }
    // causal and chunk-end masks (only where the block reaches them: the
    // wave's first query row sees the fewest keys) and the online softmax of
    // query lane % 16, in the exp2 domain (exp2(-inf) = 0)
    if (kb + kFKeys > k1 || kb + kFKeys - 1 > kmax_wave) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + kt * 16 + (lane >> 4) * 4 + i;
          if (key >= k1 || key > kmax) s[kt][i] = kNeg;
        }
    }
    float bmax = kNeg;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) bmax = fmaxf(bmax, s[kt][i]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    const float mnew = fmaxf(m, bmax);
    const float msub = (mnew == kNeg) ? 0.f : mnew;   // a fully masked query keeps p = 0
    const float r = __builtin_amdgcn_exp2f(m - msub);
    m = mnew;
    l *= r;
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[t] *= r;
    uint32_t pw[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(s[kt][i] - msub);
        l += p[i];
      }
      pw[kt][0] = pack_bf16x2(p[0], p[1]);
      pw[kt][1] = pack_bf16x2(p[2], p[3]);
    }
    // O^T += V^T P^T over two 32-key steps
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8v pf = __builtin_bit_cast(bf16x8v,
          make_uint4(pw[2 * ks][0], pw[2 * ks][1], pw[2 * ks + 1][0], pw[2 * ks + 1][1]));
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const uint16_t* vrow = Vb + (t * 16 + (lane & 15)) * VLD + ks * 32 + (lane >> 4) * 4;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
        const bf16x8v vf = __builtin_bit_cast(bf16x8v, make_uint4(lo.x, lo.y, hi.x, hi.y));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc[t], 0, 0, 0);
      }
    }
  }
  }
#undef MTP_FLUSH_LOAD

  // the chunk's partial: o (unnormalised), m, l for each query vector
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (!qok) return;
  const size_t pidx = (static_cast<size_t>(jq) * a.hq + head) * a.nchunk + c;
  float* po = a.part_o + pidx * D;
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    const int d = t * 16 + (lane >> 4) * 4;
    *reinterpret_cast<float4*>(po + d) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
  }
  if ((lane >> 4) == 0) {
    a.part_ml[pidx * 2] = m * kLn2;   // the natural-log maximum the merge expects
    a.part_ml[pidx * 2 + 1] = l;
  }
}

// The chunks of the flush rows merged by log-sum-exp: one wave per (row, query
// head).  Lane c holds chunk c (and c + 64) for the weights exp(m_c - M); lane
// d then sums head_dim columns d * D / 64 + [0, D / 64) over the chunks in
// increasing order.
template <int D>
__global__ __launch_bounds__(256) void k_attn_merge_rows(AttnArgs a) {
  constexpr int DPL = D / 64;
  __shared__ float wts[4][kFlushMaxChunks];
  if (a.state[3] != 0) return;
  int n = a.n_max;
  if (a.n_dev) n = min(max(*a.n_dev, 0), a.n_max);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pr = blockIdx.x * 4 + wave;
  const int j = pr / a.hq, h = pr % a.hq;
  const bool ok = j < n;
  const int nc = a.nchunk;
  const size_t base = (static_cast<size_t>(ok ? j : 0) * a.hq + h) * nc;
  const float* po = a.part_o + base * D + lane * DPL;
  // the column loads of the first kPre chunks go out with the (m, l) loads
  constexpr int kPre = 32 / DPL;
  const int npre = nc < kPre ? nc : kPre;
  float vp[kPre][DPL];
#pragma unroll
  for (int u = 0; u < kPre; ++u)
    if (u < npre)
#pragma unroll
      for (int q = 0; q < DPL; ++q) vp[u][q] = po[static_cast<size_t>(u) * D + q];
  float mc0 = -INFINITY, mc1 = -INFINITY, lc0 = 0.f, lc1 = 0.f;
  if (lane < nc) {
    mc0 = a.part_ml[(base + lane) * 2];
    lc0 = a.part_ml[(base + lane) * 2 + 1];
  }
  if (lane + 64 < nc) {
    mc1 = a.part_ml[(base + lane + 64) * 2];
    lc1 = a.part_ml[(base + lane + 64) * 2 + 1];
  }
  const float M = wave_max(fmaxf(mc0, mc1));
  const float w0 = (mc0 == -INFINITY) ? 0.f : __expf(mc0 - M);
  const float w1 = (mc1 == -INFINITY) ? 0.f : __expf(mc1 - M);
  const float den = wave_sum(w0 * lc0 + w1 * lc1);
  wts[wave][lane] = w0;
  wts[wave][lane + 64] = w1;
  __syncthreads();
  if (!ok) return;
  float num[DPL];
#pragma unroll
  for (int q = 0; q < DPL; ++q) num[q] = 0.f;
#pragma unroll
  for (int u = 0; u < kPre; ++u)
    if (u < npre)
#pragma unroll
      for (int q = 0; q < DPL; ++q) num[q] += wts[wave][u] * vp[u][q];
  constexpr int kIn = 8;   // chunk loads in flight per round trip
  int c = npre;
  for (; c + kIn <= nc; c += kIn) {
    float v[kIn][DPL];
#pragma unroll
    for (int u = 0; u < kIn; ++u)
#pragma unroll
      for (int q = 0; q < DPL; ++q) v[u][q] = po[static_cast<size_t>(c + u) * D + q];
#pragma unroll
    for (int u = 0; u < kIn; ++u)
#pragma unroll
      for (int q = 0; q < DPL; ++q) num[q] += wts[wave][c + u] * v[u][q];
  }
  for (; c < nc; ++c)
#pragma unroll
    for (int q = 0; q < DPL; ++q) num[q] += wts[wave][c] * po[static_cast<size_t>(c) * D + q];
  const float inv = 1.0f / den;
  const size_t oi = (static_cast<size_t>(j) * a.hq + h) * D + lane * DPL;
#pragma unroll
  for (int q = 0; q < DPL; ++q) {
    if (a.o_bf16) reinterpret_cast<uint16_t*>(a.o)[oi + q] = f32_to_bf16(num[q] * inv);
    else a.o[oi + q] = num[q] * inv;
  }
}

hipError_t launch_attention_flush(const AttnArgs& a, hipStream_t s) {
  if (a.nchunk < 1 || a.nchunk > kFlushMaxChunks) return hipErrorInvalidValue;
  const int G = a.hq / a.hkv;
  const dim3 grid(a.nchunk, (a.n_max * G + kFQ - 1) / kFQ, a.hkv);
  const dim3 mgrid((a.n_max * a.hq + 3) / 4);
  int slot = -1;
  time_mark(TIME_ATTENTION, true, s, &slot);
  (void)hipGetLastError();
  switch (a.d) {
    case 64: hipLaunchKernelGGL(k_attn_flush<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(k_attn_flush<128>, grid, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(k_attn_flush<256>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  time_mark(TIME_ATTENTION, false, s, &slot);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (a.d) {
    case 64: hipLaunchKernelGGL(k_attn_merge_rows<64>, mgrid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(k_attn_merge_rows<128>, mgrid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(k_attn_merge_rows<256>, mgrid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace mtp
