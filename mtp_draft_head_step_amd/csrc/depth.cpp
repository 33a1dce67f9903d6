// Draft-depth controller (host code): picks how many tokens the head drafts in
// each round so that committed tokens per unit of round time are maximal.
//
// The pages ("Ollama qwen3_5 MTP loader and SelfDraft path", Facts on depth
// control; the Ollama x/mlxrunner commit that chooses the draft length to
// maximise throughput) fix the rule: draft argmax_N committed(N) / cost(N)
// from live per-position acceptance and a per-width round cost, N from 0
// (plain decode) up to one past the deepest position drafted so far, a probe
// one deeper than the choice every 4 rounds backing off to every 512, and the
// state kept across requests.  Where they leave a step open this follows one
// plain reading: Laplace estimates (accepts + 1) / (attempts + 2) per
// position, committed(N) = 1 + sum_i prod_{j<=i} a_j, the caller seeds the
// cost of every depth and reported round times move it by an exponential
// average with weight 1/4, ties go to the smaller depth, and the probe
// interval doubles at each probe and returns to 4 when the choice changes.
//
// Arithmetic is fp64 in a fixed order with contraction off, so the decisions
// are reproducible bit for bit.
#pragma clang fp contract(off)

#include <new>
#include <vector>

#include "mtp.h"

namespace {
constexpr int kProbeFirst = 4;
constexpr int kProbeMax = 512;
constexpr double kCostWeight = 0.25;
}  // namespace

struct mtp_depth_ctl {
  int max_depth = 0;
  std::vector<double> cost;          // [0, max_depth]: round cost at each depth
  std::vector<long long> attempts;   // [1, max_depth]: rounds that reached position i
  std::vector<long long> accepts;    // [1, max_depth]: ... and accepted its draft
  int choice = 0;
  int interval = kProbeFirst;
  int since_probe = 0;

  double rate(int i) const {
    return (static_cast<double>(accepts[i]) + 1.0) / (static_cast<double>(attempts[i]) + 2.0);
  }
  int frontier() const {
    int f = 0;
    for (int i = 1; i <= max_depth; ++i)
      if (attempts[i] > 0) f = i;
    return f;
  }
  int argmax() const {
    const int top = frontier() + 1 < max_depth ? frontier() + 1 : max_depth;
    double total = 1.0, run = 1.0;
    double best = total / cost[0];
    int best_n = 0;
    for (int n = 1; n <= top; ++n) {
      run = run * rate(n);
      total = total + run;
      const double v = total / cost[n];
      if (v > best) {
        best = v;
        best_n = n;
      }
    }
    return best_n;
  }
};

extern "C" {

int mtp_depth_ctl_create(int32_t max_depth, const double* cost, mtp_depth_ctl** out) {
  if (!out) return MTP_E_INVALID_ARG;
  *out = nullptr;
  if (max_depth < 0 || max_depth > MTP_MAX_DRAFT || !cost) return MTP_E_INVALID_ARG;
  for (int i = 0; i <= max_depth; ++i)
    if (!(cost[i] > 0.0)) return MTP_E_INVALID_ARG;   // also rejects NaN
  mtp_depth_ctl* c = new (std::nothrow) mtp_depth_ctl;
  if (!c) return MTP_E_INVALID_ARG;
  c->max_depth = max_depth;
  c->cost.assign(cost, cost + max_depth + 1);
  c->attempts.assign(max_depth + 1, 0);
  c->accepts.assign(max_depth + 1, 0);
  c->choice = c->argmax();
  *out = c;
  return MTP_OK;
}

void mtp_depth_ctl_destroy(mtp_depth_ctl* c) { delete c; }

int32_t mtp_depth_ctl_next(mtp_depth_ctl* c) {
  if (!c) return MTP_E_INVALID_ARG;
  if (++c->since_probe >= c->interval) {
    c->since_probe = 0;
    c->interval = 2 * c->interval < kProbeMax ? 2 * c->interval : kProbeMax;
    return c->choice + 1 < c->max_depth ? c->choice + 1 : c->max_depth;
  }
  return c->choice;
}

int mtp_depth_ctl_report(mtp_depth_ctl* c, int32_t depth, int32_t accepted, double round_cost) {
  if (!c || depth < 0 || depth > c->max_depth || accepted < 0 || accepted > depth || !(round_cost > 0.0))
    return MTP_E_INVALID_ARG;
  // positions 1..accepted were accepted; position accepted + 1 (if drafted) was tried and rejected
  const int reached = accepted + 1 < depth ? accepted + 1 : depth;
  for (int i = 1; i <= reached; ++i) {
    ++c->attempts[i];
    if (i <= accepted) ++c->accepts[i];
  }
  c->cost[depth] = (1.0 - kCostWeight) * c->cost[depth] + kCostWeight * round_cost;
  const int n = c->argmax();
  if (n != c->choice) {
    c->choice = n;
    c->interval = kProbeFirst;
    c->since_probe = 0;
  }
  return MTP_OK;
}

int mtp_depth_ctl_state(const mtp_depth_ctl* c, int32_t* choice, int32_t* interval, double* cost) {
  if (!c) return MTP_E_INVALID_ARG;
  if (choice) *choice = c->choice;
  if (interval) *interval = c->interval;
  if (cost)
    for (int i = 0; i <= c->max_depth; ++i) cost[i] = c->cost[i];
  return MTP_OK;
}

}  // extern "C"
