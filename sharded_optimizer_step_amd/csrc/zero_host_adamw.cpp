// zero_host_adamw.cpp -- the optimizer half of the CPU-offloaded shard step
// (ZeRO-Offload: "第2章 软件程序与专用硬件的结合", section 2.3.4, keeps the
// optimizer state in CPU memory; gsyq.cn/news/457874 section 4.2 configures
// it as offload_optimizer on the cpu with pinned memory).
//
// The update is the AdamW step of the GPU kernels (bias-corrected, eps outside
// the root, decay decoupled and scaled by lr), evaluated in binary64 from the
// fp32 state and rounded once on store. Build with -ffp-contract=off and
// -fno-math-errno: no fused multiply-adds, and the square root may vectorize
// (IEEE division and square root are correctly rounded in every vector width,
// so the result does not depend on how the loop is vectorized).
#include "zero_host.h"

#include <sched.h>

#include <algorithm>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>

namespace zero {

namespace {

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN with its sign.
inline uint16_t to_bf16(float x)
{
    uint32_t u;
    std::memcpy(&u, &x, sizeof u);
    const uint32_t rne = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const uint32_t qnan = (u >> 16) | 0x40u;
    return static_cast<uint16_t>((u & 0x7FFFFFFFu) > 0x7F800000u ? qnan : rne);  // a select, no branch
}

}  // namespace

namespace {

// UNIT_BC: both bias corrections are exactly 1.0 (late steps: beta^t below
// half an ulp of 1), where x / 1.0 == x for every x, so skipping the two
// divisions changes no bit of the result.
// SCALED: the staged g is the unscaled fold, multiplied here in binary32 by
// gscale (the product the GPU's fold pass stores), before anything else.
template <bool UNIT_BC, bool SCALED>
void adamw_loop(float* __restrict__ w, float* __restrict__ m, float* __restrict__ v, const float* __restrict__ g,
                uint16_t* __restrict__ out, int64_t n, const HostAdamScalars& c)
{
    const double b1 = c.b1, omb1 = c.omb1, b2 = c.b2, omb2 = c.omb2, decay = c.decay, lr = c.lr, bc1 = c.bc1,
                 bc2 = c.bc2, eps = c.eps, coef = c.coef;
    const float gscale = c.gscale;
    for (int64_t i = 0; i < n; ++i) {
        const float g32 = SCALED ? g[i] * gscale : g[i];
        const double gi = static_cast<double>(g32) * coef;
        const double mn = b1 * static_cast<double>(m[i]) + omb1 * gi;
        const double vn = b2 * static_cast<double>(v[i]) + omb2 * gi * gi;
        const double m_hat = UNIT_BC ? mn : mn / bc1;
        const double v_hat = UNIT_BC ? vn : vn / bc2;
        const double wn = static_cast<double>(w[i]) * decay - lr * m_hat / (std::sqrt(v_hat) + eps);
        const float wf = static_cast<float>(wn);
        m[i] = static_cast<float>(mn);
        v[i] = static_cast<float>(vn);
        w[i] = wf;
        out[i] = to_bf16(wf);
    }
}

}  // namespace

void host_adamw_range(float* w, float* m, float* v, const float* g, uint16_t* out, int64_t n,
                      const HostAdamScalars& c)
{
    const bool unit = c.bc1 == 1.0 && c.bc2 == 1.0;
    if (c.gscale == 1.0f)
        unit ? adamw_loop<true, false>(w, m, v, g, out, n, c) : adamw_loop<false, false>(w, m, v, g, out, n, c);
    else
        unit ? adamw_loop<true, true>(w, m, v, g, out, n, c) : adamw_loop<false, true>(w, m, v, g, out, n, c);
}

struct ThreadTeam::Impl {
    std::mutex mu;
    std::condition_variable go, done;
    std::vector<std::thread> threads;
    const std::function<void(int, int)>* fn = nullptr;
    uint64_t generation = 0;
    int pending = 0;
    bool stop = false;
};

ThreadTeam::ThreadTeam(int n) : impl_(new Impl), n_(n < 1 ? 1 : n)
{
    for (int member = 1; member < n_; ++member) {
        impl_->threads.emplace_back([this, member] {
            Impl& s = *impl_;
            uint64_t seen = 0;
            for (;;) {
                const std::function<void(int, int)>* fn;
                {
                    std::unique_lock<std::mutex> lk(s.mu);
                    s.go.wait(lk, [&] { return s.stop || s.generation != seen; });
                    if (s.stop) return;
                    seen = s.generation;
                    fn = s.fn;
                }
                (*fn)(member, n_);
                std::lock_guard<std::mutex> lk(s.mu);
                if (--s.pending == 0) s.done.notify_one();
            }
        });
    }
}

ThreadTeam::~ThreadTeam()
{
    {
        std::lock_guard<std::mutex> lk(impl_->mu);
        impl_->stop = true;
    }
    impl_->go.notify_all();
    for (std::thread& t : impl_->threads) t.join();
    delete impl_;
}

void ThreadTeam::run(const std::function<void(int, int)>& fn)
{
    Impl& s = *impl_;
    {
        std::lock_guard<std::mutex> lk(s.mu);
        s.fn = &fn;
        s.pending = n_ - 1;
        ++s.generation;
    }
    s.go.notify_all();
    fn(0, n_);
    std::unique_lock<std::mutex> lk(s.mu);
    s.done.wait(lk, [&] { return s.pending == 0; });
}

int host_threads_available()
{
    cpu_set_t set;
    CPU_ZERO(&set);
    if (sched_getaffinity(0, sizeof set, &set) == 0) {
        const int k = CPU_COUNT(&set);
        if (k > 0) return k;
    }
    const unsigned h = std::thread::hardware_concurrency();
    return h > 0 ? static_cast<int>(h) : 1;
}

void host_adamw_parallel(ThreadTeam& team, float* w, float* m, float* v, const float* g, uint16_t* out, int64_t n,
                         const HostAdamScalars& c)
{
    if (n <= 0) return;
    team.run([&](int member, int members) {
        // contiguous slices, 64-element aligned so that no two members share
        // a cache line of any array
        const int64_t per = ((n + members - 1) / members + 63) / 64 * 64;
        const int64_t b = std::min<int64_t>(n, per * member);
        const int64_t e = std::min<int64_t>(n, b + per);
        if (e > b) host_adamw_range(w + b, m + b, v + b, g + b, out + b, e - b, c);
    });
}

}  // namespace zero
