// kda_internal.h -- launch interface between the C-ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda_common.h"
#include "kda_layer.h"

namespace kda {

enum DecodeMode { DECODE_STEP = 0, DECODE_VERIFY = 1, DECODE_COMMIT = 2 };
constexpr int kMaxDraft = 16;  // tokens per session of one verify / commit call

struct DecodeArgs {
  const void *q, *k, *v;
  Gate gate;
  const float* beta;
  float* state;
  void* o;
  bool qkv_bf16, o_bf16;
  int B, H, Dk, Dv;
  void* stream;
  int mode = DECODE_STEP;
  int N = 1;                          // tokens per session (verify, commit)
  const int32_t* n_accept = nullptr;  // commit: accepted tokens per session
  bool layer = false;                 // the fused layer step (io below; o receives y)
  LayerIO io{};
};

// The layer prefill: the first pass reads the projections' outputs (q, k, v
// of PrefillArgs) and applies the prologue; after the recurrence the conv
// state is handed on and the epilogue turns o into y.
struct LayerPro {
  ConvArgs conv;
  const float* st_in;   // [n_seq, 3, H, 2 Dk + Dv] fp32 or null (zeros)
  float* st_out;        // same shape or null; not aliasing st_in
  OutGateArgs out;      // g [tokens, H, Dv] (bf16), w [Dv], eps
  void* y;              // [tokens, H, Dv]
  bool y_bf16;
};

struct PrefillArgs {
  const void *q, *k, *v;
  Gate gate;
  const float* beta;
  const float* initial_state;
  float* final_state;
  void* o;
  bool qkv_bf16, o_bf16;
  // Sequences: either n_seq dense sequences of T tokens (cu_seqlens == NULL),
  // or n_seq packed sequences delimited by the device array cu_seqlens.
  const int32_t* cu_seqlens;
  int n_seq, T, H, Dk, Dv;
  // Optional device scratch; with at least prefill_two_pass_bytes(...) bytes
  // the two-pass schedule runs, otherwise the fused kernel.
  void* workspace;
  size_t workspace_bytes;
  void* stream;
  // Segments per window and sequence of the two-pass state recurrence (1: one
  // workgroup walks all of a window's chunks); above 1 the workspace must hold
  // prefill_segmented_bytes(...).
  int nseg = 1;
  const LayerPro* pro = nullptr;  // the layer prefill (two-pass only)
};

hipError_t launch_decode(const DecodeArgs& a);

// The layer's prologue and epilogue as standalone passes (kda_layer.hip).
struct PrologueArgs {
  const void *xq, *xk, *xv;        // [tokens, H, D] the projections' outputs
  bool bf16;                       // token tensors bf16 (else fp32)
  ConvArgs conv;
  const float* st_in;              // [n_seq, 3, H, 2 Dk + Dv] or null (zeros)
  float* st_out;                   // same shape or null; not aliasing st_in
  const int32_t* cu_seqlens;       // packed: [n_seq + 1]; dense: null
  int n_seq;
  long long Tseq;                  // dense: tokens per sequence
  long long total;                 // tokens in all
  int H, Dk, Dv;
  void *q, *k, *v;                 // outputs, the token dtype
  void* stream;
};
struct EpilogueArgs {
  const void* o;                   // [rows, H, Dv]
  bool o_bf16;
  const void* g;                   // [rows, H, Dv]
  bool g_bf16;
  const float* w;                  // [Dv]
  float eps;
  void* y;                         // [rows, H, Dv]
  bool y_bf16;
  long long rows;                  // tokens
  int H, Dv;
  void* stream;
};
hipError_t launch_prologue(const PrologueArgs& a);
hipError_t launch_epilogue(const EpilogueArgs& a);
// The conv state after each sequence (its last three inputs, or the state
// handed in for a sequence shorter than three), without the prologue's rows.
hipError_t launch_conv_state(const PrologueArgs& a);
hipError_t launch_prefill(const PrefillArgs& a);      // dispatch (kda_prefill.hip)
// (kda_noalloc.hip) the device scratch of the entry point that allocates
// nothing: 128 MiB per device, its address on the current device
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_prefill_f32(const PrefillArgs& a);  // fp32 inputs, Dk = 64 (kda_prefill_f32.hip)
hipError_t launch_prefill_recurrent(const PrefillArgs& a);  // fp32 inputs, Dk = 128 (kda_decode.hip)
bool prefill_supported(bool qkv_bf16, int Dk, int Dv);

// Two-pass bf16 prefill.  Workspace bytes it needs (0 if unavailable for the
// shape; independent of the sequence length), and whether it is expected to
// beat the fused kernel on the current device (`tokens`: packed total).
size_t prefill_two_pass_bytes(int n_seq, int H, int Dk, int Dv);
bool prefill_two_pass_preferred(int n_seq, long long tokens, int H, int Dk, int Dv);
constexpr int kMaxSegments = 16;  // segments per window and sequence
size_t prefill_segmented_bytes(int n_seq, int H, int Dk, int Dv, int nseg);
int prefill_segments_preferred(int n_seq, long long tokens, int H, int Dk, int Dv);
// (kda_prefill_state.hip) operand-image bytes per (chunk, head); the state
// pass over one window of packed tokens [tok_lo, tok_hi) (state read from the
// initial state for a sequence's first chunk, else from `carry`, and written
// to `carry`); the chunk table of packed sequences (clamped to `cap` chunks).
size_t prefill_image_bytes(int Dk, int Dv);
// Segments of a window processed side by side (nseg > 1): the summaries
// [nseg - 1][n_seq][H][Dk][Dk + Dv] and the entry states [nseg][n_seq][H][Dk][Dv]
// (entry 0 a copy of the state entering the window, so that no workgroup reads
// the carried state that another one writes) live in the caller's workspace.
struct SegmentArgs {
  int nseg = 1;
  float* seg_in = nullptr;
  float* summ = nullptr;
};
hipError_t launch_prefill_state(const PrefillArgs& a, const unsigned char* img,
                                const int32_t* chunk_off, float* carry, long long tok_lo,
                                long long tok_hi, int cap, const SegmentArgs& sg = SegmentArgs{});
hipError_t launch_chunk_table(const int32_t* cu_seqlens, int n_seq, int cap, int32_t* chunk_off,
                              void* stream);
// (kda_prefill_prep.hip) the first pass over one window: operand images of the
// (chunk, head) items of the chunks starting in [tok_lo, tok_hi) (at most `cap`
// chunks), item (chunk - first chunk of the window) * H + head, on a persistent
// grid of `grid` workgroups (prefill_prep_per_cu() of them fit a compute unit).
int prefill_prep_per_cu();
hipError_t launch_prefill_prep(const PrefillArgs& a, unsigned char* img, const int32_t* chunk_off,
                               long long tok_lo, long long tok_hi, int cap, int grid);

}  // namespace kda
