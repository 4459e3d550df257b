// Launcher of the whole-triangle Gram kernel (kernels_gram_tri.hip).
#pragma once

#include "muon_internal.h"

namespace muon {

// Padded short side of the problems the whole-triangle Gram takes (bf16 X).
constexpr int kTriRows = 384;

// A = s^2 X X^T (s = the Frobenius scale in round 0, else 1) of bf16 problems
// whose padded short side rp is kTriRows: one workgroup per listed problem
// (items[b].ns; ti and tj unused) computes all of A, both triangles, and the
// fp32 diagonal adiag, exactly what the tiled Gram writes.  List the
// problems with the largest cp first: the hardware hands workgroups out in
// index order, so the longest start first.
hipError_t launch_ns_gram_tri(hipStream_t s, const NsDev* ns, const GemmItem* items,
                              int64_t nitems, int iter);

}  // namespace muon
