// Kernel timing records for benchmarks (spec_profile_enable / spec_profile_read).
#include <mutex>
#include <string>
#include <vector>

#include "profile.hpp"
#include "specdec.h"

namespace specdec {
namespace {

struct Record {
    hipEvent_t start;
    hipEvent_t stop;
};

std::mutex g_mu;
std::string g_target;          // kernel being timed ("" = none, "*" = all)
std::vector<Record> g_records; // records of the current session
std::vector<Record> g_pool;    // events kept for reuse

bool matches(const char* kernel) {
    return !g_target.empty() && (g_target == "*" || g_target == kernel);
}

}  // namespace

void* prof_begin(const char* kernel, hipStream_t s) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!matches(kernel)) return nullptr;
    Record r;
    if (!g_pool.empty()) {
        r = g_pool.back();
        g_pool.pop_back();
    } else if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.stop) != hipSuccess) {
        return nullptr;
    }
    hipEventRecord(r.start, s);
    g_records.push_back(r);
    return reinterpret_cast<void*>(g_records.size());   // 1-based index
}

void prof_end(void* token, hipStream_t s) {
    if (!token) return;
    std::lock_guard<std::mutex> lk(g_mu);
    const size_t i = reinterpret_cast<size_t>(token) - 1;
    if (i < g_records.size()) hipEventRecord(g_records[i].stop, s);
}

}  // namespace specdec

using namespace specdec;

extern "C" {

spec_status_t spec_profile_enable(const char* kernel) {
    std::lock_guard<std::mutex> lk(g_mu);
    for (auto& r : g_records) g_pool.push_back(r);
    g_records.clear();
    g_target = kernel ? kernel : "";
    return SPEC_OK;
}

spec_status_t spec_profile_read(int* launches, double* total_ms) {
    std::lock_guard<std::mutex> lk(g_mu);
    double sum = 0.0;
    for (auto& r : g_records) {
        if (hipEventSynchronize(r.stop) != hipSuccess) return SPEC_ERR_HIP;
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return SPEC_ERR_HIP;
        sum += ms;
    }
    if (launches) *launches = (int)g_records.size();
    if (total_ms) *total_ms = sum;
    return SPEC_OK;
}

}  // extern "C"
