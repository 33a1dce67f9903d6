// Dispatch of the weight-streaming GEMV launches (the kernel and its launch
// shape are in gemv_impl.h, instantiated per weight type in gemv_*.hip) and the
// per-device launch facts they share.
#include <map>
#include <mutex>
#include <set>
#include <tuple>

#include "kernels.h"

namespace mtp {

constexpr int kThreads = 256;
constexpr int kMaxLds = 144 * 1024;   // dynamic LDS a GEMV may ask for

// instantiated in gemv_f32.hip, gemv_bf16_*.hip, gemv_i8.hip
template <int WT, int NR>
hipError_t launch_r(const GemvArgs& a, hipStream_t s, int* g);

// Launch facts per device, behind one lock: the compute-unit count, a kernel's
// occupancy at a dynamic LDS size, and whether its dynamic LDS limit was raised.
struct LaunchFacts {
  std::mutex mu;
  std::map<int, int> cus;
  std::map<std::tuple<int, const void*, size_t>, int> occ;
  std::set<std::pair<int, const void*>> raised;
};
static LaunchFacts& launch_facts() {
  static LaunchFacts f;
  return f;
}

// Workgroups of `fn` (256 threads, `lds` bytes of dynamic LDS) that fit on one
// compute unit of the current device, and that device's compute units.
hipError_t occupancy_of(const void* fn, size_t lds, int* per_cu, int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  LaunchFacts& f = launch_facts();
  std::lock_guard<std::mutex> lk(f.mu);
  auto c = f.cus.find(dev);
  if (c == f.cus.end()) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    c = f.cus.emplace(dev, n > 0 ? n : 1).first;
  }
  *cus = c->second;
  const auto key = std::make_tuple(dev, fn, lds);
  auto o = f.occ.find(key);
  if (o == f.occ.end()) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, lds) != hipSuccess || n < 1)
      n = static_cast<int>((160 * 1024) / (lds + 2048));
    o = f.occ.emplace(key, n < 1 ? 1 : n).first;
  }
  *per_cu = o->second;
  return hipSuccess;
}

// Allow `fn` up to kMaxLds of dynamic LDS on the current device (once).
hipError_t raise_lds_limit(const void* fn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  LaunchFacts& f = launch_facts();
  std::lock_guard<std::mutex> lk(f.mu);
  if (f.raised.count({dev, fn})) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
  if (e == hipSuccess) f.raised.insert({dev, fn});
  return e;
}

template <int WT>
static hipError_t launch_w(const GemvArgs& a, int nr, hipStream_t s, int* g) {
  if (WT == W_I8 && a.out_mode != OUT_LOGITS) return hipErrorInvalidValue;   // unembedding only
  {
    switch (nr) {
      case 1: return launch_r<WT, 1>(a, s, g);
      case 2: return launch_r<WT, 2>(a, s, g);
      case 3: return launch_r<WT, 3>(a, s, g);
      case 4: return launch_r<WT, 4>(a, s, g);
      case 8: return launch_r<WT, 8>(a, s, g);
      case 16: return launch_r<WT, 16>(a, s, g);
      default: return hipErrorInvalidValue;
    }
  }
}

hipError_t launch_gemv(const GemvArgs& a, int wtype, int nr, hipStream_t s, int* grid_out) {
  switch (wtype) {
    case W_F32: return launch_w<W_F32>(a, nr, s, grid_out);
    case W_BF16: return launch_w<W_BF16>(a, nr, s, grid_out);
    case W_I8: return launch_w<W_I8>(a, nr, s, grid_out);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtp
