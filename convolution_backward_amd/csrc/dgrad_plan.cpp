#include "dgrad_plan.h"

#include <algorithm>

namespace cbw {

int out_extent(int in, int filt, int stride, int pad)
{
    if (stride < 1 || pad < 0)
        return 0;
    const long span = (long)in + 2L * pad - filt;
    if (span < 0)
        return 0;
    return (int)(span / stride + 1);
}

namespace {

struct AxisPhase {
    int extent;  // lattice size along this axis
    int first;   // first tap
    int count;   // number of taps
    int d0;      // dy offset of the first tap
};

// One spatial axis: dx extent `in`, filter extent `filt`.
AxisPhase axis_phase(int offset, int in, int filt, int stride, int pad)
{
    AxisPhase a{};
    a.extent = offset < in ? (in - offset + stride - 1) / stride : 0;
    a.first = (offset + pad) % stride;
    a.count = a.first < filt ? (filt - 1 - a.first) / stride + 1 : 0;
    a.d0 = (offset + pad - a.first) / stride;  // exact: offset + pad - first is a multiple of stride
    return a;
}

}  // namespace

bool make_plan(int N, int H, int W, int K, int R, int S, int stride, int pad, Plan& plan)
{
    plan = Plan{};
    plan.P = out_extent(H, R, stride, pad);
    plan.Q = out_extent(W, S, stride, pad);
    if (plan.P < 1 || plan.Q < 1 || N < 1 || K < 1)
        return false;
    for (int ph = 0; ph < stride; ++ph) {
        const AxisPhase ah = axis_phase(ph, H, R, stride, pad);
        if (ah.extent == 0)
            continue;
        for (int pw = 0; pw < stride; ++pw) {
            const AxisPhase aw = axis_phase(pw, W, S, stride, pad);
            if (aw.extent == 0)
                continue;
            Phase p{};
            p.ph = ph;
            p.pw = pw;
            p.Hp = ah.extent;
            p.Wp = aw.extent;
            p.r0 = ah.first;
            p.t0 = aw.first;
            p.nr = ah.count;
            p.nt = aw.count;
            p.dr0 = ah.d0;
            p.dt0 = aw.d0;
            p.M = (int64_t)N * p.Hp * p.Wp;
            p.Kg = (int64_t)K * p.nr * p.nt;
            plan.phases.push_back(p);
        }
    }
    std::stable_sort(plan.phases.begin(), plan.phases.end(),
                     [](const Phase& a, const Phase& b) { return a.nr * a.nt > b.nr * b.nt; });
    return true;
}

}  // namespace cbw
