// Stride-phase planner for conv2d dgrad (host only, integer arithmetic).
//
// With stride s, output row h = ph + s*i receives only the filter rows r with
// h + pad - r divisible by s, i.e. r = r0 + a*s with r0 = (ph + pad) mod s,
// from dy row p = (h + pad - r)/s = i + dr0 - a, dr0 = (ph + pad - r0)/s.
// Splitting dx into the s*s lattices (ph, pw) therefore turns the strided
// dgrad into s*s dense sub-GEMMs with no inserted zeros (the strided case the
// tvm PR "[CUTLASS] Conv2d dgrad" singles out as needing its own kernel).
#pragma once

#include <cstdint>
#include <vector>

namespace cbw {

struct Phase {
    int ph, pw;      // lattice offsets
    int Hp, Wp;      // lattice extents in dx
    int r0, t0;      // first row / column tap
    int nr, nt;      // tap counts
    int dr0, dt0;    // dy offsets of the first taps
    int64_t M;       // N*Hp*Wp
    int64_t Kg;      // K*nr*nt
};

struct Plan {
    int P = 0, Q = 0;
    std::vector<Phase> phases;  // heaviest first, empty lattices omitted
};

int out_extent(int in, int filt, int stride, int pad);

// Fills `plan`; returns false if the shape has no valid forward output.
bool make_plan(int N, int H, int W, int K, int R, int S, int stride, int pad, Plan& plan);

}  // namespace cbw
