// Optional per-kernel-class timing with HIP events (see li_timing_enable).
#include "li_timing.hpp"

#include <mutex>
#include <vector>

namespace li {
namespace {

struct Pair {
    hipEvent_t a, b;
};

struct Registry {
    std::mutex m;
    bool on = false;
    std::vector<Pair> pending[LI_KERNEL_CLASSES];
    std::vector<hipEvent_t> spare;
};

Registry &reg()
{
    static Registry r;
    return r;
}

hipEvent_t take_event(Registry &r)
{
    if (!r.spare.empty()) {
        hipEvent_t e = r.spare.back();
        r.spare.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

} // namespace

static thread_local TimedScope *t_current = nullptr;

TimedScope::TimedScope(int cls, hipStream_t s, bool one_kernel)
    : cls_(cls), s_(s), a_(nullptr), b_(nullptr), one_(one_kernel), taken_(false), prev_(nullptr)
{
    Registry &r = reg();
    std::lock_guard<std::mutex> g(r.m);
    if (!r.on || cls < 0 || cls >= LI_KERNEL_CLASSES) return;
    a_ = take_event(r);
    b_ = take_event(r);
    if (!a_ || !b_ || (!one_ && hipEventRecord(a_, s_) != hipSuccess)) {
        if (a_) r.spare.push_back(a_);
        if (b_) r.spare.push_back(b_);
        a_ = b_ = nullptr;
        return;
    }
    if (one_) {
        prev_ = t_current;
        t_current = this;
    }
}

TimedScope::~TimedScope()
{
    if (!a_) return;
    if (one_) t_current = prev_;
    Registry &r = reg();
    std::lock_guard<std::mutex> g(r.m);
    const bool ok = one_ ? taken_ : hipEventRecord(b_, s_) == hipSuccess;
    if (ok) {
        r.pending[cls_].push_back(Pair{a_, b_});
    } else {
        r.spare.push_back(a_);
        r.spare.push_back(b_);
    }
}

void kernel_events(hipEvent_t *start, hipEvent_t *stop)
{
    TimedScope *t = t_current;
    if (!t || t->taken_) {
        *start = *stop = nullptr;
        return;
    }
    t->taken_ = true;
    *start = t->a_;
    *stop = t->b_;
}

void timing_enable(bool on)
{
    Registry &r = reg();
    std::lock_guard<std::mutex> g(r.m);
    r.on = on;
}

hipError_t timing_read(int cls, double *total_ms, int64_t *launches)
{
    Registry &r = reg();
    std::vector<Pair> mine;
    {
        std::lock_guard<std::mutex> g(r.m);
        mine.swap(r.pending[cls]);
    }
    double tot = 0.0;
    hipError_t err = hipSuccess;
    for (const Pair &p : mine) {
        float ms = 0.0f;
        hipError_t e = hipEventSynchronize(p.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.a, p.b);
        if (e != hipSuccess && err == hipSuccess) err = e;
        tot += ms;
    }
    {
        std::lock_guard<std::mutex> g(r.m);
        for (const Pair &p : mine) {
            r.spare.push_back(p.a);
            r.spare.push_back(p.b);
        }
    }
    *total_ms = tot;
    *launches = (int64_t)mine.size();
    return err;
}

} // namespace li
