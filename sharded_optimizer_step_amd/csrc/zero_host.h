// zero_host.h -- the host half of the CPU-offloaded shard step: AdamW on
// host-resident fp32 state, run by a team of host threads. Plain C++ (no HIP
// headers): compiled by the host compiler with contraction off, so every
// binary64 operation rounds as written. Not part of the public C ABI.
#pragma once

#include <cstdint>
#include <functional>

namespace zero {

// binary64 scalars of one host AdamW step (the clip coefficient included).
struct HostAdamScalars {
    double b1, omb1, b2, omb2;  // beta1, 1-beta1, beta2, 1-beta2
    double decay;               // 1 - lr*weight_decay
    double lr;
    double bc1, bc2;            // 1 - beta1^t, 1 - beta2^t
    double eps;
    double coef;                // clip coefficient applied to g
    float gscale = 1.0f;        // binary32 multiplier of the staged g, applied
                                // first (g = fl32(g * gscale)), as the GPU fold does
};

// Elements [0, n): AdamW on w, m, v (fp32, in place) from the fp32 gradient
// g, evaluated in binary64 and rounded once; out = bf16 round-to-nearest-even
// of the new w. The five arrays must not overlap.
void host_adamw_range(float* w, float* m, float* v, const float* g, uint16_t* out, int64_t n,
                      const HostAdamScalars& c);

// A fixed team of host threads that runs one function on every member and
// returns when all are done. Member 0 is the calling thread.
class ThreadTeam {
public:
    explicit ThreadTeam(int n);
    ~ThreadTeam();
    ThreadTeam(const ThreadTeam&) = delete;
    ThreadTeam& operator=(const ThreadTeam&) = delete;
    int size() const { return n_; }
    void run(const std::function<void(int member, int members)>& fn);

private:
    struct Impl;
    Impl* impl_;
    int n_;
};

// Host threads the process may use: the size of its affinity mask (>= 1).
int host_threads_available();

// host_adamw_range over [0, n) split across the team in 64-element-aligned
// slices.
void host_adamw_parallel(ThreadTeam& team, float* w, float* m, float* v, const float* g, uint16_t* out, int64_t n,
                         const HostAdamScalars& c);

}  // namespace zero
