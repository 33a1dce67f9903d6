// Draft-KV append and attention over the draft KV for few query rows (the
// batch-1 step and small in-round flushes).
//
// k_rope_append: per (row, head) wave: per-head RMSNorm of q or k over head_dim,
//   rotate-half RoPE at position state[0] + row (angle reduced in fp64), k and v
//   appended to the cache in the KV dtype, roped q kept in fp32.  Capacity and
//   count checks set the sticky error word.  The length itself is advanced by
//   the finishing kernel, so every kernel of the step reads the same state[0].
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
  // every entry word in one memory round trip
  const int err0 = st[3];
  const int ndev = a.n_dev ? *a.n_dev : a.n_max;
  const int len0 = st[0];
  if (err0 != 0) return;
  const bool bad_count = ndev < a.n_min || ndev < 0 || ndev > a.n_max;
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
    const double l2t = log2(static_cast<double>(a.theta));
    for (int i = lane; i < half; i += 64) {
      float c, s;
      rope_cs(pos, i, D, l2t, c, s);
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
}

hipError_t launch_rope_append(const RopeArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_rope_append, dim3(a.n_max, a.hq + a.hkv), dim3(64), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / 64;
constexpr int kMaxChunks = 4096;  // chunks per (row, head): capacity <= 2^20

template <bool KVB>
__device__ __forceinline__ void unpack16(const uint4& v, float (&f)[KVB ? 8 : 4]) {
  if constexpr (KVB) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = __uint_as_float(w[q] << 16);
      f[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  } else {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
}

// Split-K attention for one (key chunk, kv head, query row).  Lanes are laid
// along head_dim (LPK lanes hold one 16-byte slice each of a K or V row), so a
// wave covers KPI keys per load; each lane group keeps its own online-softmax
// state (running max m, sum l, unnormalised o) over the keys it visits, KB keys
// (2 KB loads) in flight per step.  Groups merge with xor shuffles, waves
// through LDS; the chunk's (o, m, l) partial goes to the merge kernel.
// RMSNorm over head_dim of one head (src, D fp32 values) times the norm weight,
// then rotate-half RoPE at `pos` (one wave): put(d, value) for every d < D, each
// value by the lane that computed it.
// Element d of a projection row held as nsp split-K partials ps floats apart,
// summed in split order (nsp <= 1: the row itself).  The first kSplitLoads
// partials are loaded together (one memory round trip); offsets are 32-bit
// element indices from one base, so every split shares one scalar address.
// Compiled for head_dim >= kSplitMinHeadDim only (SPLIT; the host defers no
// reduce below it).
constexpr int kSplitLoads = 4;
template <int NE, bool SPLIT>
__device__ __forceinline__ void load_split_row(const float* src, int ps, int nsp, int lane, float (&x)[NE]) {
  if (!SPLIT || nsp <= 1) {
#pragma unroll
    for (int k = 0; k < NE; ++k) x[k] = src[lane + 64 * k];
    return;
  }
  float y[kSplitLoads][NE];
#pragma unroll
  for (int q = 0; q < kSplitLoads; ++q)
    if (q == 0 || q < nsp)
#pragma unroll
      for (int k = 0; k < NE; ++k) y[q][k] = src[q * ps + lane + 64 * k];
#pragma unroll
  for (int k = 0; k < NE; ++k) x[k] = y[0][k];
#pragma unroll
  for (int q = 1; q < kSplitLoads; ++q)
    if (q < nsp)
#pragma unroll
      for (int k = 0; k < NE; ++k) x[k] += y[q][k];
  for (int q = kSplitLoads; q < nsp; ++q)
#pragma unroll
    for (int k = 0; k < NE; ++k) x[k] += src[q * ps + lane + 64 * k];
}

template <int D, typename Put>
__device__ __forceinline__ void norm_rope_head(const float* src, const void* nw, int nw_bf16, float eps,
                                               int pos, double l2t, int lane, Put put,
                                               const float2* cs = nullptr, int ps = 0, int nsp = 1) {
  // cs: (cos, sin) of every rotation pair at `pos`, if the caller has them;
  // ps, nsp: the row as split-K partials (load_split_row)
  // every load first (one memory round trip), then the arithmetic in the same
  // per-lane order as an element-at-a-time loop: lane holds d = lane + 64 k
  constexpr int NE = D / 64;                 // elements per lane (D >= 64)
  constexpr int NP = (D / 2 + 63) / 64;      // rotation pairs per lane
  float x[NE];
  load_split_row<NE, (D >= kSplitMinHeadDim)>(src, ps, nsp, lane, x);
  // weights as raw bits (bf16 in the high half once converted); the
  // conversion waits until after both load forms join
  uint32_t b1[NP], b2[NP];
  if (nw_bf16) {
#pragma unroll
    for (int r = 0; r < NP; ++r) {
      const int i = (lane + 64 * r) % (D / 2);   // lanes past D / 2 (D = 64) load a valid weight, unused
      b1[r] = static_cast<const uint16_t*>(nw)[i];
      b2[r] = static_cast<const uint16_t*>(nw)[i + D / 2];
    }
  } else {
#pragma unroll
    for (int r = 0; r < NP; ++r) {
      const int i = (lane + 64 * r) % (D / 2);
      b1[r] = static_cast<const uint32_t*>(nw)[i];
      b2[r] = static_cast<const uint32_t*>(nw)[i + D / 2];
    }
  }
  const int wsh = nw_bf16 ? 16 : 0;
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < NE; ++k) ss += x[k] * x[k];
  ss = group_sum_all(ss, 64);
  const float inv = rsqrtf(ss / static_cast<float>(D) + eps);
  // element i + D / 2 of pair r: with D >= 128 it is this lane's x[r + NE / 2];
  // with D = 64 it sits in lane + 32
  const float up = __shfl_down(x[0], 32, 64);
#pragma unroll
  for (int r = 0; r < NP; ++r) {
    const int i = lane + 64 * r;
    if (i < D / 2) {
      const float xa = x[r];
      const float xb = (D >= 128) ? x[(r + NE / 2) % NE] : up;
      const float x1 = xa * inv * __uint_as_float(b1[r] << wsh), x2 = xb * inv * __uint_as_float(b2[r] << wsh);
      float c, sn;
      if (cs) {
        c = cs[i].x;
        sn = cs[i].y;
      } else {
        rope_cs(pos, i, D, l2t, c, sn);
      }
      put(i, x1 * c - x2 * sn);
      put(i + D / 2, x1 * sn + x2 * c);
    }
  }
}

// NW waves per workgroup (8 for heavy one-row decode launches: two waves per
// SIMD hide part of the latency of the per-key reductions)
template <bool KVB, int D, int G, bool FUSE, int NW>
__global__ __launch_bounds__(NW * 64) void k_attn(AttnArgs a) {
  constexpr int kAttnWaves = NW, kAttnThreads = NW * 64;
  constexpr int EPL = KVB ? 8 : 4;   // elements per lane (16 bytes)
  constexpr int LPK = D / EPL;       // lanes per key row
  constexpr int KPI = 64 / LPK;      // keys per wave instruction
  constexpr int KB = 4;              // keys per lane group per step
  constexpr float kNeg = -1e30f;
  __shared__ float s_m[kAttnWaves][G], s_l[kAttnWaves][G];
  __shared__ float s_o[kAttnWaves][G][D];
  __shared__ float s_q[FUSE ? G : 1][FUSE ? D : 1];
  __shared__ float2 s_cs[FUSE ? D / 2 : 1];   // RoPE (cos, sin) at the query's position

  // several sessions (ROW_LAST with the fused append only): blockIdx.z is the
  // session, with its own state words, K/V and workspace rows
  const bool multi = FUSE && a.batch > 1;
  const int sess = multi ? static_cast<int>(blockIdx.z) : 0;
  int32_t* st = a.state + 4 * sess;
  constexpr int ebytes = KVB ? 2 : 4;
  void* kcs = static_cast<char*>(a.kc) + (multi ? sess * a.kv_sb * ebytes : 0ll);
  void* vcs = static_cast<char*>(a.vc) + (multi ? sess * a.kv_sb * ebytes : 0ll);
  const int rb = sess * a.n_max;    // the session's first workspace row
  // every entry word in one memory round trip
  const int err0 = st[3];
  const int off = st[0];            // pre-append length (committed by k_finish)
  const int nd0 = a.n_dev ? a.n_dev[multi ? sess * a.ndev_sb : 0] : a.n_max;
  if (err0 != 0) return;
  int n = a.n_max;
  if constexpr (FUSE) {
    // the append's checks (once per launch and session, by its first workgroup)
    const int ndev = nd0;
    const bool bad_count = ndev < a.n_min || ndev < 0 || ndev > a.n_max;
    if (bad_count || off + ndev > a.capacity) {
      if (blockIdx.x == 0 && blockIdx.y == 0 && (multi || blockIdx.z == 0) && threadIdx.x == 0)
        st[3] = bad_count ? 3 : 1;
      return;
    }
    n = ndev;
  } else if (a.n_dev) {
    n = min(max(nd0, 0), a.n_max);
  }
  const int j = (a.row_sel == ROW_LAST) ? n - 1 : static_cast<int>(blockIdx.z);
  if (j < 0 || j >= n) return;
  const int jf = rb + j;            // workspace row
  const int L = off + j + 1;        // keys visible to row j
  const int h = blockIdx.y;
  const int c = blockIdx.x;
  int ck = (L + a.nchunk - 1) / a.nchunk;
  ck = (ck + 15) & ~15;
  const int k0 = c * ck;
  const int k1 = min(L, k0 + ck);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t pbase = (static_cast<size_t>(jf) * a.hq + h * G) * a.nchunk + c;

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

  const int grp = lane / LPK;
  const int li = lane % LPK;
  const int d0 = li * EPL;
  const float scale = rsqrtf(static_cast<float>(D));

  // The first step's K and V rows are loaded before anything else: they do not
  // depend on the query, so their memory latency overlaps the fused norm / RoPE
  // prologue.  Rows of slots appended by this launch (>= off) are read again
  // after the prologue's barrier.
  const size_t head_off = static_cast<size_t>(h) * a.capacity * D;
  const char* kbase = static_cast<const char*>(kcs) + (head_off + d0) * ebytes;
  const char* vbase = static_cast<const char*>(vcs) + (head_off + d0) * ebytes;
  constexpr int row_bytes = D * ebytes;
  constexpr int kstride = KPI * kAttnWaves;   // keys between a group's consecutive keys
  const int base0 = k0 + wave * KPI;
  uint4 kv[KB], vv[KB];
#pragma unroll
  for (int b = 0; b < KB; ++b) {
    const int kk = base0 + grp + b * kstride;
    const int kc = kk < k1 ? kk : k0;           // a valid row; result masked below
    kv[b] = *reinterpret_cast<const uint4*>(kbase + static_cast<size_t>(kc) * row_bytes);
    vv[b] = *reinterpret_cast<const uint4*>(vbase + static_cast<size_t>(kc) * row_bytes);
  }

  float qr[G][EPL];
  if constexpr (FUSE) {
    const double l2t = log2(static_cast<double>(a.theta));
    // the rotation of the query position, once per workgroup for all its heads
    if (tid < D / 2) {
      float c, sn;
      rope_cs(off + j, tid, D, l2t, c, sn);
      s_cs[tid] = make_float2(c, sn);
    }
    // new slots in this chunk: k normed and roped, k and v appended (a wave per slot)
    const int s0 = max(off, k0), s1 = min(off + n, k1);
    for (int sl = s0 + wave; sl < s1; sl += kAttnWaves) {
      const float* row = a.qkv + static_cast<size_t>(rb + sl - off) * a.ld_qkv;
      const size_t o = (static_cast<size_t>(h) * a.capacity + sl) * D;
      norm_rope_head<D>(row + (a.hq + h) * D, a.k_norm, a.nw_bf16, a.eps, sl, l2t, lane, [&](int d, float v) {
        if constexpr (KVB) static_cast<uint16_t*>(kcs)[o + d] = f32_to_bf16(v);
        else static_cast<float*>(kcs)[o + d] = v;
      }, nullptr, a.qkv_pstride, a.qkv_nsp);
      const float* vsrc = row + (a.hq + a.hkv + h) * D;
      float vv[D / 64];
      load_split_row<D / 64, (D >= kSplitMinHeadDim)>(vsrc, a.qkv_pstride, a.qkv_nsp, lane, vv);
#pragma unroll
      for (int k = 0; k < D / 64; ++k) {
        if constexpr (KVB) static_cast<uint16_t*>(vcs)[o + lane + 64 * k] = f32_to_bf16(vv[k]);
        else static_cast<float*>(vcs)[o + lane + 64 * k] = vv[k];
      }
    }
    // the query heads of this kv head, row j, normed and roped
    __syncthreads();   // the rotation table is complete
    const float* qrow = a.qkv + static_cast<size_t>(jf) * a.ld_qkv;
    for (int g = wave; g < G; g += kAttnWaves) {
      float* qd = s_q[g];
      norm_rope_head<D>(qrow + (h * G + g) * D, a.q_norm, a.nw_bf16, a.eps, off + j, l2t, lane,
                        [&](int d, float v) { qd[d] = v; }, s_cs, a.qkv_pstride, a.qkv_nsp);
    }
    __syncthreads();   // the appended rows and the queries are visible to the whole workgroup
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) qr[g][e] = s_q[g][d0 + e] * scale;
    if (k1 > off) {   // this chunk holds appended slots: their rows again
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        const int kk = base0 + grp + b * kstride;
        if (kk >= off && kk < k1) {
          kv[b] = *reinterpret_cast<const uint4*>(kbase + static_cast<size_t>(kk) * row_bytes);
          vv[b] = *reinterpret_cast<const uint4*>(vbase + static_cast<size_t>(kk) * row_bytes);
        }
      }
    }
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float* qp = a.q + (static_cast<size_t>(j) * a.hq + h * G + g) * D + d0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) qr[g][e] = qp[e] * scale;
    }
  }

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNeg;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  // wave-uniform trip count so every lane takes part in the group reductions;
  // the next step's rows are loaded while this step's are used
  for (int base = base0; base < k1; base += KB * kstride) {
    bool ok[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) ok[b] = base + grp + b * kstride < k1;
    uint4 kn[KB], vn[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const int kk = base + KB * kstride + grp + b * kstride;
      const int kc = kk < k1 ? kk : k0;         // past the chunk: a valid row, unused
      kn[b] = *reinterpret_cast<const uint4*>(kbase + static_cast<size_t>(kc) * row_bytes);
      vn[b] = *reinterpret_cast<const uint4*>(vbase + static_cast<size_t>(kc) * row_bytes);
    }
    float sc[KB][G];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      float kf[EPL];
      unpack16<KVB>(kv[b], kf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) p += qr[g][e] * kf[e];
        p = group_sum_all(p, LPK);
        sc[b][g] = ok[b] ? p : kNeg;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mb = sc[0][g];
#pragma unroll
      for (int b = 1; b < KB; ++b) mb = fmaxf(mb, sc[b][g]);
      const float mnew = fmaxf(m[g], mb);
      const float r = __expf(m[g] - mnew);
      l[g] *= r;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= r;
      m[g] = mnew;
    }
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      float vf[EPL];
      unpack16<KVB>(vv[b], vf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = ok[b] ? __expf(sc[b][g] - m[g]) : 0.f;
        l[g] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] += p * vf[e];
      }
    }
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      kv[b] = kn[b];
      vv[b] = vn[b];
    }
  }

  // merge the wave's lane groups (same head_dim slice, different keys): the
  // partner of a lane is lane ^ o, o = LPK, 2 LPK, .., 32
#define MTP_ATTN_MERGE(O)                                                                  \
  if constexpr (LPK <= (O)) {                                                              \
    _Pragma("unroll") for (int g = 0; g < G; ++g) {                                        \
      const float mo = xor_lane<O>(m[g]);                                                  \
      const float lo = xor_lane<O>(l[g]);                                                  \
      const float mnew = fmaxf(m[g], mo);                                                  \
      const float ra = __expf(m[g] - mnew), rb = __expf(mo - mnew);                        \
      l[g] = l[g] * ra + lo * rb;                                                          \
      _Pragma("unroll") for (int e = 0; e < EPL; ++e)                                      \
        acc[g][e] = acc[g][e] * ra + xor_lane<O>(acc[g][e]) * rb;                          \
      m[g] = mnew;                                                                         \
    }                                                                                      \
  }
  MTP_ATTN_MERGE(8)
  MTP_ATTN_MERGE(16)
  MTP_ATTN_MERGE(32)
#undef MTP_ATTN_MERGE
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[wave][g][d0 + e] = acc[g][e];
      if (li == 0) { s_m[wave][g] = m[g]; s_l[wave][g] = l[g]; }
    }
  }
  __syncthreads();
  // merge the waves
  for (int idx = tid; idx < G * D; idx += kAttnThreads) {
    const int g = idx / D, d = idx - g * D;
    float M = s_m[0][g];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) M = fmaxf(M, s_m[w][g]);
    float o = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float r = __expf(s_m[w][g] - M);
      o += r * s_o[w][g][d];
      lsum += r * s_l[w][g];
    }
    a.part_o[(pbase + static_cast<size_t>(g) * a.nchunk) * D + d] = o;
    if (d == 0) {
      a.part_ml[(pbase + static_cast<size_t>(g) * a.nchunk) * 2] = M;
      a.part_ml[(pbase + static_cast<size_t>(g) * a.nchunk) * 2 + 1] = lsum;
    }
  }
}

// One workgroup per (row, query head): chunk weights exp(m_c - M) in LDS, then
// every thread sums its head_dim column over the chunks.  The column loads of
// the first kMergePre chunks are issued with the (m, l) loads, before the
// weights are known, so the merge costs about one memory round trip.
constexpr int kMergePre = 64;

__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  __shared__ float wts[kMaxChunks];
  __shared__ float red[4];
  __shared__ float s_m, s_den;
  // several sessions (ROW_LAST): blockIdx.y is the session
  const bool multi = a.batch > 1 && a.row_sel == ROW_LAST;
  const int sess = multi ? static_cast<int>(blockIdx.y) : 0;
  const int32_t* st = a.state + 4 * sess;
  const int err0 = st[3];
  const int nd0 = a.n_dev ? a.n_dev[multi ? sess * a.ndev_sb : 0] : a.n_max;
  const int n = min(max(nd0, 0), a.n_max);
  const int jl = (a.row_sel == ROW_LAST) ? n - 1 : static_cast<int>(blockIdx.y);
  const bool valid = err0 == 0 && jl >= 0 && jl < n;
  if (a.o_compact) {
    // gathered rows for products over the sessions' last rows: o at row sess
    // (bf16) and the residual row, spread over the session's head blocks;
    // zeros for a session without a row
    if (a.xg_out) {
      float* xo = a.xg_out + static_cast<size_t>(sess) * a.ld_xg;
      const float* xs = valid ? a.xg + (static_cast<size_t>(sess) * a.n_max + jl) * a.ld_xg : nullptr;
      for (int k = blockIdx.x * 256 + threadIdx.x; k < a.ld_xg; k += gridDim.x * 256) xo[k] = valid ? xs[k] : 0.f;
    }
    if (!valid) {
      if (static_cast<int>(threadIdx.x) < a.d)
        reinterpret_cast<uint16_t*>(a.o)[(static_cast<size_t>(sess) * a.hq + blockIdx.x) * a.d + threadIdx.x] = 0;
      return;
    }
  }
  if (!valid) return;
  const int j = sess * a.n_max + jl;   // workspace row
  const int hq = blockIdx.x;
  const int D = a.d;
  const int nc = a.nchunk;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t base = (static_cast<size_t>(j) * a.hq + hq) * nc;
  const float* po = a.part_o + base * D;
  const int d = tid;                   // this thread's column (D <= 256)
  const int npre = nc < kMergePre ? nc : kMergePre;
  float v[kMergePre];
  if (d < D) {
#pragma unroll
    for (int u = 0; u < kMergePre; ++u)
      if (u < npre) v[u] = po[static_cast<size_t>(u) * D + d];
  }
  float m = -INFINITY;
  for (int c = tid; c < nc; c += 256) m = fmaxf(m, a.part_ml[(base + c) * 2]);
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (tid == 0) s_m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  const float M = s_m;
  float den = 0.f;
  for (int c = tid; c < nc; c += 256) {
    const float mc = a.part_ml[(base + c) * 2];
    const float w = (mc == -INFINITY) ? 0.f : __expf(mc - M);
    wts[c] = w;
    den += w * a.part_ml[(base + c) * 2 + 1];
  }
  den = wave_sum(den);
  __syncthreads();
  if (lane == 0) red[wave] = den;
  __syncthreads();
  if (tid == 0) s_den = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  if (d >= D) return;
  const float inv = 1.0f / s_den;
  // accumulator k takes the chunks c = k (mod 4) in increasing order
  float num0 = 0.f, num1 = 0.f, num2 = 0.f, num3 = 0.f;
#pragma unroll
  for (int u = 0; u < kMergePre; u += 4) {
    if (u < npre) num0 += wts[u] * v[u];
    if (u + 1 < npre) num1 += wts[u + 1] * v[u + 1];
    if (u + 2 < npre) num2 += wts[u + 2] * v[u + 2];
    if (u + 3 < npre) num3 += wts[u + 3] * v[u + 3];
  }
  int c = npre;
  // the rest: sixteen chunk loads in flight per round trip
  for (; c + 16 <= nc; c += 16) {
    float w16[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) w16[u] = po[static_cast<size_t>(c + u) * D + d];
#pragma unroll
    for (int u = 0; u < 16; u += 4) {
      num0 += wts[c + u] * w16[u];
      num1 += wts[c + u + 1] * w16[u + 1];
      num2 += wts[c + u + 2] * w16[u + 2];
      num3 += wts[c + u + 3] * w16[u + 3];
    }
  }
  for (; c < nc; ++c) {
    const float x = wts[c] * po[static_cast<size_t>(c) * D + d];
    switch (c & 3) {
      case 0: num0 += x; break;
      case 1: num1 += x; break;
      case 2: num2 += x; break;
      default: num3 += x; break;
    }
  }
  const float out = ((num0 + num1) + (num2 + num3)) * inv;
  const size_t oi = static_cast<size_t>(a.o_compact ? sess : j) * a.hq * D + hq * D + d;
  if (a.o_bf16) reinterpret_cast<uint16_t*>(a.o)[oi] = f32_to_bf16(out);
  else a.o[oi] = out;
}

template <bool KVB, int D, bool FUSE, int NW>
static hipError_t attn_dgw(const AttnArgs& a, dim3 grid, hipStream_t s) {
  const int g = a.hq / a.hkv;
  (void)hipGetLastError();
  switch (g) {
    case 1: hipLaunchKernelGGL((k_attn<KVB, D, 1, FUSE, NW>), grid, dim3(NW * 64), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_attn<KVB, D, 2, FUSE, NW>), grid, dim3(NW * 64), 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_attn<KVB, D, 3, FUSE, NW>), grid, dim3(NW * 64), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_attn<KVB, D, 4, FUSE, NW>), grid, dim3(NW * 64), 0, s, a); break;
    case 6: hipLaunchKernelGGL((k_attn<KVB, D, 6, FUSE, NW>), grid, dim3(NW * 64), 0, s, a); break;
    case 8:
      if constexpr (NW == 4) hipLaunchKernelGGL((k_attn<KVB, D, 8, FUSE, NW>), grid, dim3(NW * 64), 0, s, a);
      else return hipErrorInvalidValue;   // eight heads a group keep four waves (register room)
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool KVB, int D, bool FUSE>
static hipError_t attn_dg(const AttnArgs& a, dim3 grid, hipStream_t s) {
  // one-row launches over bf16 K/V with many products per key (grouped heads x
  // head_dim >= 1024, up to six heads a group): eight waves per workgroup (on
  // the 27B shape 1 us less per launch; the tiny head's two grouped heads of 64
  // measured 0.2 us slower)
  const int g = a.hq / a.hkv;
  if (KVB && a.row_sel == ROW_LAST && g <= 6 && g * D >= 1024)
    return attn_dgw<KVB, D, FUSE, KVB ? 8 : 4>(a, grid, s);
  return attn_dgw<KVB, D, FUSE, 4>(a, grid, s);
}

template <bool KVB, int D>
static hipError_t attn_d(const AttnArgs& a, dim3 grid, hipStream_t s) {
  return (a.fuse_rope && a.row_sel == ROW_LAST) ? attn_dg<KVB, D, true>(a, grid, s)
                                                : attn_dg<KVB, D, false>(a, grid, s);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.batch > 1 && !(a.row_sel == ROW_LAST && a.fuse_rope)) return hipErrorNotSupported;
  const int rows = (a.row_sel == ROW_LAST) ? (a.batch > 1 ? a.batch : 1) : a.n_max;
  const dim3 grid(a.nchunk, a.hkv, rows);
  // the matrix-core flush attention launches its own merge
  if (a.mfma && a.kv_bf16 && a.row_sel == ROWS_RANGE) return launch_attention_flush(a, s);
  hipError_t e;
  int slot = -1;
  time_mark(TIME_ATTENTION, true, s, &slot);
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
  time_mark(TIME_ATTENTION, false, s, &slot);
  if (e != hipSuccess) return e;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_attn_merge, dim3(a.hq, rows), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mtp

namespace mtp {

__global__ __launch_bounds__(256) void k_finish(FinishArgs a) {
  const int sess = a.batch > 1 ? static_cast<int>(blockIdx.x) : 0;   // one workgroup per session
  int32_t* st = a.state + 4 * sess;
  // every load first (one memory round trip): the entry words and this
  // thread's first argmax keys
  const int err0 = st[3];
  const int len0 = st[0];
  const int nd0 = a.n_dev ? a.n_dev[sess * a.ndev_sb] : a.n_max;
  const unsigned long long* parts = a.parts ? a.parts + static_cast<size_t>(sess) * a.nparts : nullptr;
  unsigned long long b0 = 0ull;
  if (parts) b0 = block_max_u64_first(parts, a.nparts);
  if (err0 != 0) return;
  const int n = min(max(nd0, 0), a.n_max);
  if (parts) {
    const unsigned long long b = block_max_u64_rest(parts, a.nparts, b0);
    if (threadIdx.x == 0 && a.amax_out && n > 0) a.amax_out[sess * a.out_sb] = argmax_index(b);
  }
  if (threadIdx.x == 0) {
    const int len = len0 + n;
    st[0] = len;
    if (a.set_base) st[1] = len;
  }
}

hipError_t launch_finish(const FinishArgs& a, hipStream_t s) {
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_finish, dim3(a.batch > 1 ? a.batch : 1), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mtp
