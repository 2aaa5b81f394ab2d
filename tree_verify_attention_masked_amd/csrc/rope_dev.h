// Rotary position embedding of the tree's rows (RoFormer's rotary position
// embedding in the half-split layout): for j < D/2 the pair (x_j, x_{j + D/2})
// of a row at position p turns by the angle p * theta^(-2j/D).  Angles, their
// cosines and sines are taken in fp64, each rotated value in fp64 with one
// fused multiply-add, rounded once to fp32 (the caller rounds to the storage
// type), so every kernel that rotates a row gets the same bits.
#pragma once

#include <math.h>

namespace spectree {

__device__ __forceinline__ double rope_angle(int pos, int j, int D, double log2_theta) {
  return static_cast<double>(pos) * exp2(-(2.0 * j / D) * log2_theta);
}

// Cosine and sine of the angle of pair j at position p (one shared argument reduction).
__device__ __forceinline__ void rope_cos_sin(int pos, int j, int D, double log2_theta, double* c, double* s) {
  sincos(rope_angle(pos, j, D, log2_theta), s, c);
}

__device__ __forceinline__ void rope_turn(float x0, float x1, double c, double s, float* y0, float* y1) {
  *y0 = static_cast<float>(fma(static_cast<double>(x0), c, -(static_cast<double>(x1) * s)));
  *y1 = static_cast<float>(fma(static_cast<double>(x1), c, static_cast<double>(x0) * s));
}

}  // namespace spectree
