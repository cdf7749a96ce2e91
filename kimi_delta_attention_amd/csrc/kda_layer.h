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
// (D = 128) or channel l (D = 64).  Row sums pair lanes with DPP row rotations
// by 8, 4, 2 and 1 and then the permlane16 / permlane32 swaps: each step adds
// the same pairs in every lane, so every lane holds bitwise the same sum.
// Transcendentals use the hardware units (exp2, reciprocal, reciprocal square
// root, each about 1 ulp): Swish(a) = a / (1 + 2^(-a log2 e)).
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

// The fused layer decode step's extra operands: the projections' outputs of the
// call's tokens ([B, N, H, D], the token dtype), the conv taps and state
// ([B, 3, H, 2 Dk + Dv] fp32), and the output gate.
struct LayerIO {
  const void *xq, *xk, *xv;
  ConvArgs conv;
  float* conv_state;
  OutGateArgs out;
};

template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float wave_sum(float x) {
  x = dpp_add<0x128>(x);  // row_ror:8
  x = dpp_add<0x124>(x);  // row_ror:4
  x = dpp_add<0x122>(x);  // row_ror:2
  x = dpp_add<0x121>(x);  // row_ror:1
  const unsigned xb = __float_as_uint(x);
  const auto h = __builtin_amdgcn_permlane16_swap(xb, xb, false, false);
  x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  const unsigned yb = __float_as_uint(x);
  const auto w = __builtin_amdgcn_permlane32_swap(yb, yb, false, false);
  return __uint_as_float(w[0]) + __uint_as_float(w[1]);
}

// Sum over the four 16-lane rows at the same position (lanes l, l ^ 16,
// l ^ 32, l ^ 48): the permlane16 and permlane32 swaps, each adding the same
// pair in both lanes, so the four lanes hold bitwise the same sum.
__device__ __forceinline__ float rows4_sum(float x) {
  const unsigned xb = __float_as_uint(x);
  const auto h = __builtin_amdgcn_permlane16_swap(xb, xb, false, false);
  x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  const unsigned yb = __float_as_uint(x);
  const auto w = __builtin_amdgcn_permlane32_swap(yb, yb, false, false);
  return __uint_as_float(w[0]) + __uint_as_float(w[1]);
}

// Sigmoid(a) = 1 / (1 + 2^(-a log2 e)) on the hardware units
__device__ __forceinline__ float sigmoid_hw(float a) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-a * 1.44269504088896341f));
}

__device__ __forceinline__ float swish(float a) { return a * sigmoid_hw(a); }

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

// ShortConv of one channel over (h0, h1, h2, x) (oldest first; taps t[0..3],
// t[3] on the current token), then Swish; products summed oldest tap first
// with explicit fmas.
__device__ __forceinline__ float conv_swish(const floatx4& t, float h0, float h1, float h2,
                                            float x) {
  float a = t[0] * h0;
  a = __builtin_fmaf(t[1], h1, a);
  a = __builtin_fmaf(t[2], h2, a);
  a = __builtin_fmaf(t[3], x, a);
  return swish(a);
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
    const float r = __builtin_amdgcn_rsqf(wave_sum(ss) + eps);
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
  const float r = __builtin_amdgcn_rsqf(wave_sum(ss) * (1.f / (64 * CPL)) + eps);
#pragma unroll
  for (int c = 0; c < CPL; ++c) y[c] = o[c] * r * w[c] * sigmoid_hw(g[c]);
}

}  // namespace kda
