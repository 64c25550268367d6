// Optional per-kernel timing of the library's own launches with HIP events
// recorded on the caller's stream (used by measurement tools; off by default).
#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "launch.h"
#include "mla.h"

namespace mla {
namespace {

struct Rec {
  const char* name;
  hipEvent_t start, stop;
};

std::mutex g_mu;
bool g_on = false;
std::string g_only;  // when set, only launches of this name are timed
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t s) : name_(name), s_(s), start_(nullptr) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || (!g_only.empty() && g_only != name_)) return;
  start_ = take_event();
  if (start_ && hipEventRecord((hipEvent_t)start_, s_) != hipSuccess) {
    g_pool.push_back((hipEvent_t)start_);
    start_ = nullptr;
  }
}

ProfScope::~ProfScope() {
  if (!start_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t stop = take_event();
  if (!stop) {
    g_pool.push_back((hipEvent_t)start_);
    return;
  }
  if (hipEventRecord(stop, s_) != hipSuccess) {
    g_pool.push_back((hipEvent_t)start_);
    g_pool.push_back(stop);
    return;
  }
  g_recs.push_back(Rec{name_, (hipEvent_t)start_, stop});
}

}  // namespace mla

using mla::g_mu;
using mla::g_on;
using mla::g_only;
using mla::g_pool;
using mla::g_recs;

extern "C" {

mla_status mla_profile_only(const char* kernel_name) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_only = kernel_name ? kernel_name : "";
  return MLA_OK;
}

mla_status mla_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& r : g_recs) {
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_recs.clear();
  g_on = true;
  return MLA_OK;
}

mla_status mla_profile_end(int32_t max_kernels, char* names, int32_t name_len, double* total_ms,
                           int32_t* launches, int32_t* n_kernels) {
  if (!n_kernels || (max_kernels > 0 && (!names || !total_ms || !launches))) return MLA_ERR_NULL_ARG;
  if (max_kernels < 0 || name_len < 2) return MLA_ERR_BAD_SHAPE;
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = false;
  std::vector<std::string> keys;
  std::vector<double> sums;
  std::vector<int> counts;
  mla_status st = MLA_OK;
  for (auto& r : g_recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) {
      st = MLA_ERR_HIP;
      continue;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      st = MLA_ERR_HIP;
      continue;
    }
    size_t k = 0;
    while (k < keys.size() && keys[k] != r.name) ++k;
    if (k == keys.size()) {
      keys.push_back(r.name);
      sums.push_back(0.0);
      counts.push_back(0);
    }
    sums[k] += ms;
    counts[k] += 1;
  }
  for (auto& r : g_recs) {
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_recs.clear();
  *n_kernels = (int32_t)keys.size();
  for (int32_t i = 0; i < (int32_t)keys.size() && i < max_kernels; ++i) {
    strncpy(names + (size_t)i * name_len, keys[i].c_str(), name_len - 1);
    names[(size_t)i * name_len + name_len - 1] = 0;
    total_ms[i] = sums[i];
    launches[i] = counts[i];
  }
  return st;
}

}  // extern "C"
