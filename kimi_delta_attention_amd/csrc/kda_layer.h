// kda_layer.h -- the steps on either side of the recurrence in a KDA layer, one
// token row at a time, shared by the standalone prologue / epilogue kernels and
// the fused decode kernel so that both round identically.
//
// Prologue ("Kimi Delta Attention 完全拆解", section "一次 KDA 前向究竟发生了什么";
// "从线性注意力到 KDA", the ShortConv and L2Norm bullets):
//     q, k = L2Norm(Swish(ShortConv(x_q / x_k))),  v = Swish(ShortConv(x_v))
// ShortConv is depthwise and causal with kernel 4: tap 3 weights the current
// token, tap j the token 3 - j before it; before a sequence's first token the
// inputs come from the conv state (the last 3 inputs, oldest first) or are 0.
// L2Norm: x / sqrt(sum x^2 + eps).
// Epilogue ("从线性注意力到 KDA", the per-head output norm and gate):
//     y = o / sqrt(mean o^2 + eps) * w * Sigmoid(g)   over the head's Dv channels
//
// A row of D channels is handled by one wave: lane l holds channels 2l, 2l + 1
// (D = 128) or channel l (D = 64); row sums use one fixed xor butterfly, so
// every lane holds bitwise the same sum.
#pragma once

#include "kda_common.h"

namespace kda {

struct ConvArgs {
  const float* w[3];  // [H, D, 4] taps of q, k, v
  float eps;          // L2Norm epsilon
};

struct OutGateArgs {
  const void* g;  // [rows, H, Dv] gate logits (the token inputs' dtype)
  const float* w; // [Dv] RMSNorm weight
  float eps;
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ float swish(float a) { return a / (1.f + expf(-a)); }

template <typename T>
__device__ __forceinline__ float to_f(T x) { return (float)x; }

// CPL channels of one lane: loads and stores of a row
template <typename T, int CPL>
__device__ __forceinline__ void row_load(const T* row, int lane, float (&x)[CPL]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) x[c] = to_f(row[CPL * lane + c]);
}
template <typename T, int CPL>
__device__ __forceinline__ void row_store(T* row, int lane, const float (&x)[CPL]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) row[CPL * lane + c] = (T)x[c];
}

// One token row of one tensor: conv over (h[0], h[1], h[2], x), Swish, and for
// q and k the L2Norm.  Products are summed oldest tap first with explicit fmas.
template <int CPL, bool NORM>
__device__ __forceinline__ void prologue_row(const float (&h)[3][CPL], const float (&x)[CPL],
                                             const float (&w)[CPL][4], float eps,
                                             float (&y)[CPL]) {
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float a = w[c][0] * h[0][c];
    a = __builtin_fmaf(w[c][1], h[1][c], a);
    a = __builtin_fmaf(w[c][2], h[2][c], a);
    a = __builtin_fmaf(w[c][3], x[c], a);
    y[c] = swish(a);
    ss = __builtin_fmaf(y[c], y[c], ss);
  }
  if constexpr (NORM) {
    const float r = 1.f / sqrtf(wave_sum(ss) + eps);
#pragma unroll
    for (int c = 0; c < CPL; ++c) y[c] *= r;
  }
}

// One output row: RMSNorm over the row (D = 64 * CPL channels), weight, gate.
template <int CPL>
__device__ __forceinline__ void epilogue_row(const float (&o)[CPL], const float (&g)[CPL],
                                             const float (&w)[CPL], float eps,
                                             float (&y)[CPL]) {
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) ss = __builtin_fmaf(o[c], o[c], ss);
  const float r = 1.f / sqrtf(wave_sum(ss) * (1.f / (64 * CPL)) + eps);
#pragma unroll
  for (int c = 0; c < CPL; ++c) y[c] = o[c] * r * w[c] / (1.f + expf(-g[c]));
}

}  // namespace kda
