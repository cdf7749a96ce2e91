// kda_internal.h -- launch interface between the C-ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
  const void *q, *k, *v;
  const float *alpha, *beta;
  float* state;
  void* o;
  bool qkv_bf16, o_bf16;
  int B, H, Dk, Dv;
  void* stream;
};

struct PrefillArgs {
  const void *q, *k, *v;
  const float *alpha, *beta;
  const float* initial_state;
  float* final_state;
  void* o;
  bool qkv_bf16, o_bf16;
  // Sequences: either n_seq dense sequences of T tokens (cu_seqlens == NULL),
  // or n_seq packed sequences delimited by the device array cu_seqlens.
  const int32_t* cu_seqlens;
  int n_seq, T, H, Dk, Dv;
  void* stream;
};

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_prefill(const PrefillArgs& a);      // dispatch (kda_prefill.hip)
hipError_t launch_prefill_f32(const PrefillArgs& a);  // fp32 inputs (kda_prefill_f32.hip)
bool prefill_supported(bool qkv_bf16, int Dk, int Dv);

}  // namespace kda
