// kda_api.cpp -- the C ABI declared in include/kda.h: argument validation on the
// host (before any HIP call), dispatch to the kernels, status strings.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kda_internal.h"

namespace {

thread_local char g_msg[512] = "";

kda_status fail(kda_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kda_status fail(kda_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return s;
}

kda_status ok() {
  g_msg[0] = '\0';
  return KDA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A byte range of a caller's tensor; overlap checks between the outputs an
// entry point writes and the tensors it reads (an empty or absent range
// overlaps nothing).
struct Range {
  const void* p;
  size_t n;
};
bool overlaps(Range a, Range b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a.p), y = reinterpret_cast<uintptr_t>(b.p);
  return x < y + b.n && y < x + a.n;
}
// The first output of `outs` that overlaps an input of `ins`, as "out / in"
// names, or nullptr.
template <size_t NO, size_t NI>
bool any_overlap(const Range (&outs)[NO], const char* const (&on)[NO], const Range (&ins)[NI],
                 const char* const (&in)[NI], const char** a, const char** b) {
  for (size_t i = 0; i < NO; ++i)
    for (size_t j = 0; j < NI; ++j)
      if (overlaps(outs[i], ins[j])) {
        *a = on[i];
        *b = in[j];
        return true;
      }
  return false;
}
size_t esize(kda_dtype d) { return d == KDA_BF16 ? 2 : 4; }
// bytes of a gate tensor over `rows` (token, head) rows
size_t gate_bytes(const kda_gate* g, size_t rows, int Dk) {
  if (!g || g->kind == KDA_GATE_NONE) return 0;
  return g->kind == KDA_GATE_SCALAR ? rows * 4 : rows * (size_t)Dk * 4;
}

kda_status check_common(const void* q, const void* k, const void* v, kda_dtype qkv,
                        const float* beta, const void* o, kda_dtype od, int H, int Dk, int Dv) {
  if (!q || !k || !v || !beta || !o)
    return fail(KDA_ERR_INVALID_ARGUMENT, "q, k, v, beta and o must be non-null");
  if (qkv != KDA_F32 && qkv != KDA_BF16) return fail(KDA_ERR_INVALID_ARGUMENT, "bad qkv_dtype");
  if (od != KDA_F32 && od != KDA_BF16) return fail(KDA_ERR_INVALID_ARGUMENT, "bad o_dtype");
  if (H <= 0 || Dk <= 0 || Dv <= 0)
    return fail(KDA_ERR_INVALID_ARGUMENT, "H, Dk and Dv must be positive");
  // token tensors are read and written element by element: natural alignment suffices
  const uintptr_t m_in = qkv == KDA_BF16 ? 1u : 3u, m_out = od == KDA_BF16 ? 1u : 3u;
  if (((uintptr_t)q & m_in) || ((uintptr_t)k & m_in) || ((uintptr_t)v & m_in) ||
      ((uintptr_t)beta & 3u) || ((uintptr_t)o & m_out))
    return fail(KDA_ERR_INVALID_ARGUMENT, "tensor pointers must be aligned to their element size");
  return KDA_OK;
}

// The gate descriptor: kind, tensors, bound.  `vec16`: the caller's kernels read
// a per-channel gate with 16-byte loads.
kda_status check_gate(const kda_gate* g, bool vec16, kda::Gate* out) {
  if (!g) return fail(KDA_ERR_INVALID_ARGUMENT, "gate descriptor must be non-null");
  if (g->kind < KDA_GATE_ALPHA || g->kind > KDA_GATE_NONE)
    return fail(KDA_ERR_INVALID_ARGUMENT, "unknown gate kind %d", (int)g->kind);
  const bool per_channel = g->kind == KDA_GATE_ALPHA || g->kind == KDA_GATE_LOG ||
                           g->kind == KDA_GATE_BOUNDED;
  if (g->kind != KDA_GATE_NONE) {
    if (!g->gate) return fail(KDA_ERR_INVALID_ARGUMENT, "gate tensor (alpha) must be non-null");
    const uintptr_t m = (vec16 && per_channel) ? 15u : 3u;
    if ((uintptr_t)g->gate & m)
      return fail(KDA_ERR_INVALID_ARGUMENT, "gate tensor (alpha) must be %d-byte aligned",
                  (int)m + 1);
  }
  if (g->kind == KDA_GATE_BOUNDED) {
    if (!g->a_log || ((uintptr_t)g->a_log & 3u))
      return fail(KDA_ERR_INVALID_ARGUMENT, "bounded gate needs a non-null, aligned a_log");
    if (!(g->g_min >= -5.f && g->g_min < 0.f))
      return fail(KDA_ERR_INVALID_ARGUMENT, "bounded gate g_min must lie in [-5, 0) (got %g)",
                  (double)g->g_min);
  }
  out->kind = (int)g->kind;
  out->g = g->kind == KDA_GATE_NONE ? nullptr : g->gate;
  out->a_log = g->kind == KDA_GATE_BOUNDED ? g->a_log : nullptr;
  out->g_min = g->kind == KDA_GATE_BOUNDED ? g->g_min : 0.f;
  return KDA_OK;
}

kda_status hip_status(hipError_t e) {
  if (e == hipSuccess) return ok();
  return fail(KDA_ERR_HIP, "HIP error %d: %s", (int)e, hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
  }
  return "KDA_ERR_UNKNOWN";
}

const char* kda_last_error_message(void) { return g_msg; }

size_t kda_prefill_workspace_size(int B, int T, int H, int Dk, int Dv, int chunk) {
  if (B < 0 || T < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || chunk != 64) return (size_t)-1;
  return kda::prefill_two_pass_bytes(B, H, Dk, Dv);
}

size_t kda_prefill_varlen_workspace_size(int N, int total_tokens, int H, int Dk, int Dv,
                                         int chunk) {
  if (N < 0 || total_tokens < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || chunk != 64) return (size_t)-1;
  return kda::prefill_two_pass_bytes(N, H, Dk, Dv);
}

int kda_prefill_two_pass_preferred(kda_dtype qkv_dtype, int n_seq, int total_tokens, int H, int Dk,
                                   int Dv) {
  if (qkv_dtype != KDA_BF16) return 0;
  return kda::prefill_two_pass_preferred(n_seq, total_tokens, H, Dk, Dv) ? 1 : 0;
}

size_t kda_prefill_segmented_workspace_size(int n_seq, int H, int Dk, int Dv, int chunk,
                                            int n_segments) {
  if (n_seq < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || chunk != 64 || n_segments < 1 ||
      n_segments > kda::kMaxSegments)
    return (size_t)-1;
  return kda::prefill_segmented_bytes(n_seq, H, Dk, Dv, n_segments);
}

int kda_prefill_segments_preferred(kda_dtype qkv_dtype, int n_seq, int total_tokens, int H, int Dk,
                                   int Dv) {
  if (qkv_dtype != KDA_BF16) return 1;
  return kda::prefill_segments_preferred(n_seq, total_tokens, H, Dk, Dv);
}

static kda_status prefill_common(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                                 const kda_gate* gate, const float* beta,
                                 const int32_t* cu_seqlens, int n_seq, int T,
                                 const float* initial_state, float* final_state, void* o,
                                 kda_dtype o_dtype, int H, int Dk, int Dv, int chunk,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 int nseg = 1, const kda::LayerPro* pro = nullptr) {
  if (n_seq < 0 || T < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "negative batch or length");
  if (n_seq == 0) return ok();
  kda::Gate g = {KDA_GATE_NONE, nullptr, nullptr, 0.f};
  const bool vec16 = qkv_dtype == KDA_BF16 || Dk == 128;  // 16-byte input loads
  if (T > 0 || cu_seqlens) {
    kda_status s = check_common(q, k, v, qkv_dtype, beta, o, o_dtype, H, Dk, Dv);
    if (s != KDA_OK) return s;
    s = check_gate(gate, vec16, &g);
    if (s != KDA_OK) return s;
  } else if (H <= 0 || Dk <= 0 || Dv <= 0) {
    // T == 0: no token tensor is read; the kernel only hands the state through
    return fail(KDA_ERR_INVALID_ARGUMENT, "H, Dk and Dv must be positive");
  }
  if (chunk != 64) return fail(KDA_ERR_UNSUPPORTED, "chunk must be 64 (got %d)", chunk);
  // the bf16 kernels and the fp32 token recurrence (Dk = 128) read q, k, v
  // (and a per-channel gate, checked above) with 8- and 16-byte vector loads
  if (vec16 && (T > 0 || cu_seqlens) && (!aligned16(q) || !aligned16(k) || !aligned16(v)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "this prefill needs 16-byte aligned q, k, v and alpha");
  if ((initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "state pointers must be 16-byte aligned");
  if (!kda::prefill_supported(qkv_dtype == KDA_BF16, Dk, Dv))
    return fail(KDA_ERR_UNSUPPORTED,
                "unsupported head dims Dk=%d Dv=%d (Dk, Dv in {64, 128})", Dk, Dv);
  // token offsets are 64-bit in the kernels; the head / row counts must fit int32
  if ((long long)n_seq * H * (Dv / 64) > 0x7fffffffLL)
    return fail(KDA_ERR_INVALID_ARGUMENT, "too many (sequence, head) work items");
  if (T == 0 && !cu_seqlens && !final_state) return ok();
  {
    // outputs against inputs (final_state may be initial_state itself: in place)
    const size_t tok = cu_seqlens ? (size_t)T : (size_t)n_seq * T;
    const size_t rows = tok * H, st = (size_t)n_seq * H * Dk * Dv * 4;
    const size_t xe = pro ? 2 : esize(qkv_dtype);
    const Range ins[] = {{q, rows * Dk * xe}, {k, rows * Dk * xe}, {v, rows * Dv * xe},
                         {beta, rows * 4}, {gate ? gate->gate : nullptr, gate_bytes(gate, rows, Dk)},
                         {cu_seqlens, cu_seqlens ? (size_t)(n_seq + 1) * 4 : 0},
                         {initial_state == final_state ? nullptr : initial_state, st},
                         {workspace, workspace ? workspace_bytes : 0}};
    const char* const in[] = {"q", "k", "v", "beta", "the gate tensor", "cu_seqlens",
                              "initial_state", "workspace"};
    const Range outs[] = {{o, rows * Dv * esize(o_dtype)}, {final_state, st}};
    const char* const on[] = {"o", "final_state"};
    const char *a = nullptr, *b = nullptr;
    if (any_overlap(outs, on, ins, in, &a, &b))
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s must not overlap %s", a, b);
    if (overlaps(outs[0], outs[1]))
      return fail(KDA_ERR_INVALID_ARGUMENT, "o must not overlap final_state");
  }
  if (workspace && ((uintptr_t)workspace & 255u))
    return fail(KDA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (nseg > 1) {
    if (qkv_dtype != KDA_BF16)
      return fail(KDA_ERR_UNSUPPORTED, "the segmented schedule needs bf16 q, k, v");
    const size_t need = kda::prefill_segmented_bytes(n_seq, H, Dk, Dv, nseg);
    if (!workspace || workspace_bytes < need)
      return fail(KDA_ERR_INVALID_ARGUMENT,
                  "the segmented schedule needs a workspace of %zu bytes (got %zu)", need,
                  workspace ? workspace_bytes : (size_t)0);
    if ((long long)nseg * n_seq * H * ((Dk + Dv) / 64) > 0x7fffffffLL)
      return fail(KDA_ERR_INVALID_ARGUMENT, "too many (segment, sequence, head) work items");
  }
  kda::PrefillArgs a;
  a.q = q; a.k = k; a.v = v; a.gate = g; a.beta = beta;
  a.initial_state = initial_state; a.final_state = final_state; a.o = o;
  a.qkv_bf16 = qkv_dtype == KDA_BF16; a.o_bf16 = o_dtype == KDA_BF16;
  a.cu_seqlens = cu_seqlens; a.n_seq = n_seq; a.T = T; a.H = H; a.Dk = Dk; a.Dv = Dv;
  a.workspace = workspace; a.workspace_bytes = workspace ? workspace_bytes : 0;
  a.stream = stream;
  a.nseg = nseg;
  a.pro = pro;
  return hip_status(kda::launch_prefill(a));
}

kda_status kda_prefill_segmented(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                                 const kda_gate* gate, const float* beta,
                                 const int32_t* cu_seqlens, int n_seq, int T,
                                 const float* initial_state, float* final_state, void* o,
                                 kda_dtype o_dtype, int H, int Dk, int Dv, int chunk,
                                 int n_segments, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (n_seq < 0 || T < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "n_seq and T must be >= 0");
  if (n_segments < 1 || n_segments > kda::kMaxSegments)
    return fail(KDA_ERR_INVALID_ARGUMENT, "n_segments must lie in [1, %d] (got %d)",
                kda::kMaxSegments, n_segments);
  if (cu_seqlens && ((uintptr_t)cu_seqlens & 3u))
    return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens must be 4-byte aligned");
  if (n_seq > 0 && qkv_dtype != KDA_BF16)
    return fail(KDA_ERR_UNSUPPORTED, "the segmented schedule needs bf16 q, k, v");
  if (n_seq > 0 && (T > 0 || cu_seqlens)) {  // without tokens only the states are handed on
    const size_t need = kda::prefill_segmented_bytes(n_seq, H, Dk, Dv, n_segments);
    if (need == 0 && kda::prefill_supported(true, Dk, Dv) && H > 0)
      return fail(KDA_ERR_INVALID_ARGUMENT, "sizes too large for the segmented schedule");
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(KDA_ERR_INVALID_ARGUMENT,
                  "the segmented schedule needs a workspace of %zu bytes (got %zu)", need,
                  workspace ? workspace_bytes : (size_t)0);
  }
  return prefill_common(q, k, v, qkv_dtype, gate, beta, cu_seqlens, n_seq, T, initial_state,
                        final_state, o, o_dtype, H, Dk, Dv, chunk, workspace, workspace_bytes,
                        stream, n_segments);
}

kda_status kda_prefill_chunked_gated(const void* q, const void* k, const void* v,
                                     kda_dtype qkv_dtype, const kda_gate* gate,
                                     const float* beta, const float* initial_state,
                                     float* final_state, void* o, kda_dtype o_dtype, int B, int T,
                                     int H, int Dk, int Dv, int chunk, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (B < 0 || T < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "B and T must be >= 0");
  return prefill_common(q, k, v, qkv_dtype, gate, beta, nullptr, B, T, initial_state,
                        final_state, o, o_dtype, H, Dk, Dv, chunk, workspace, workspace_bytes,
                        stream);
}

kda_status kda_prefill_chunked(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                               const float* alpha, const float* beta,
                               const float* initial_state, float* final_state, void* o,
                               kda_dtype o_dtype, int B, int T, int H, int Dk, int Dv, int chunk,
                               void* workspace, size_t workspace_bytes, void* stream) {
  const kda_gate g = {KDA_GATE_ALPHA, alpha, nullptr, 0.f};
  return kda_prefill_chunked_gated(q, k, v, qkv_dtype, &g, beta, initial_state, final_state, o,
                                   o_dtype, B, T, H, Dk, Dv, chunk, workspace, workspace_bytes,
                                   stream);
}

kda_status kda_prefill_chunked_noalloc(const void* q, const void* k, const void* v,
                                       kda_dtype qkv_dtype, const float* alpha, const float* beta,
                                       const float* initial_state, float* final_state, void* o,
                                       kda_dtype o_dtype, int B, int T, int H, int Dk, int Dv,
                                       int chunk, void* stream) {
  if (B < 0 || T < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "B and T must be >= 0");
  if (B == 0) return ok();
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (qkv_dtype == KDA_BF16 && T > 0) {  // the two-pass schedule and its workspace
    if (chunk != 64) return fail(KDA_ERR_UNSUPPORTED, "chunk must be 64 (got %d)", chunk);
    if (H <= 0 || Dk <= 0 || Dv <= 0)
      return fail(KDA_ERR_INVALID_ARGUMENT, "H, Dk and Dv must be positive");
    const size_t need = kda::prefill_two_pass_bytes(B, H, Dk, Dv);
    if (need == 0)
      return fail(KDA_ERR_UNSUPPORTED, "unsupported head dims Dk=%d Dv=%d", Dk, Dv);
    if (need > kda::kNoAllocScratchBytes)
      return fail(KDA_ERR_INVALID_ARGUMENT,
                  "B=%d, H=%d, Dk=%d, Dv=%d need %zu bytes of workspace, more than the %zu "
                  "bytes of device scratch this entry point has",
                  B, H, Dk, Dv, need, kda::kNoAllocScratchBytes);
    if (hipError_t e = kda::noalloc_scratch(&ws); e != hipSuccess) return hip_status(e);
    ws_bytes = kda::kNoAllocScratchBytes;
  }
  const kda_gate g = {KDA_GATE_ALPHA, alpha, nullptr, 0.f};
  return prefill_common(q, k, v, qkv_dtype, &g, beta, nullptr, B, T, initial_state, final_state,
                        o, o_dtype, H, Dk, Dv, chunk, ws, ws_bytes, stream);
}

kda_status kda_prefill_varlen_gated(const void* q, const void* k, const void* v,
                                    kda_dtype qkv_dtype, const kda_gate* gate, const float* beta,
                                    const int32_t* cu_seqlens, int N, int total_tokens,
                                    const float* initial_state, float* final_state, void* o,
                                    kda_dtype o_dtype, int H, int Dk, int Dv, int chunk,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (N < 0 || total_tokens < 0)
    return fail(KDA_ERR_INVALID_ARGUMENT, "N and total_tokens must be >= 0");
  if (N > 0 && !cu_seqlens) return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens must be non-null");
  if (N > 0 && ((uintptr_t)cu_seqlens & 3u))
    return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens must be 4-byte aligned");
  return prefill_common(q, k, v, qkv_dtype, gate, beta, cu_seqlens, N, total_tokens,
                        initial_state, final_state, o, o_dtype, H, Dk, Dv, chunk, workspace,
                        workspace_bytes, stream);
}

kda_status kda_prefill_varlen(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                              const float* alpha, const float* beta, const int32_t* cu_seqlens,
                              int N, int total_tokens, const float* initial_state,
                              float* final_state, void* o, kda_dtype o_dtype, int H, int Dk,
                              int Dv, int chunk, void* workspace, size_t workspace_bytes,
                              void* stream) {
  const kda_gate g = {KDA_GATE_ALPHA, alpha, nullptr, 0.f};
  return kda_prefill_varlen_gated(q, k, v, qkv_dtype, &g, beta, cu_seqlens, N, total_tokens,
                                  initial_state, final_state, o, o_dtype, H, Dk, Dv, chunk,
                                  workspace, workspace_bytes, stream);
}

kda_status kda_decode_step_gated(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                                 const kda_gate* gate, const float* beta, float* state, void* o,
                                 kda_dtype o_dtype, int B, int H, int Dk, int Dv, void* stream) {
  if (B < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "B must be >= 0");
  if (B == 0) return ok();
  kda_status s = check_common(q, k, v, qkv_dtype, beta, o, o_dtype, H, Dk, Dv);
  if (s != KDA_OK) return s;
  kda::Gate g;
  s = check_gate(gate, true, &g);
  if (s != KDA_OK) return s;
  if (!state) return fail(KDA_ERR_INVALID_ARGUMENT, "state must be non-null");
  if (!aligned16(state) || !aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(KDA_ERR_INVALID_ARGUMENT, "q, k, v and state must be 16-byte aligned");
  if (!((Dk == 64 || Dk == 128) && (Dv == 64 || Dv == 128)))
    return fail(KDA_ERR_UNSUPPORTED, "Dk and Dv must be 64 or 128 (got %d, %d)", Dk, Dv);
  if ((long long)B * H > 0x7fffffffLL) return fail(KDA_ERR_INVALID_ARGUMENT, "B*H too large");
  kda::DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.gate = g; a.beta = beta; a.state = state; a.o = o;
  a.qkv_bf16 = qkv_dtype == KDA_BF16; a.o_bf16 = o_dtype == KDA_BF16;
  a.B = B; a.H = H; a.Dk = Dk; a.Dv = Dv; a.stream = stream;
  return hip_status(kda::launch_decode(a));
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                           const float* alpha, const float* beta, float* state, void* o,
                           kda_dtype o_dtype, int B, int H, int Dk, int Dv, void* stream) {
  const kda_gate g = {KDA_GATE_ALPHA, alpha, nullptr, 0.f};
  return kda_decode_step_gated(q, k, v, qkv_dtype, &g, beta, state, o, o_dtype, B, H, Dk, Dv,
                               stream);
}

static bool dtype_ok(kda_dtype d) { return d == KDA_F32 || d == KDA_BF16; }
static bool eps_ok(float e) { return e > 0.f && e < 3.0e38f; }

static kda_status check_conv(const kda_conv* c, kda::ConvArgs* out) {
  if (!c) return fail(KDA_ERR_INVALID_ARGUMENT, "conv descriptor must be non-null");
  if (!c->w_q || !c->w_k || !c->w_v)
    return fail(KDA_ERR_INVALID_ARGUMENT, "conv taps w_q, w_k, w_v must be non-null");
  if (((uintptr_t)c->w_q | (uintptr_t)c->w_k | (uintptr_t)c->w_v) & 3u)
    return fail(KDA_ERR_INVALID_ARGUMENT, "conv taps must be 4-byte aligned");
  if (!eps_ok(c->eps)) return fail(KDA_ERR_INVALID_ARGUMENT, "L2Norm eps must be finite and > 0");
  out->w[0] = c->w_q; out->w[1] = c->w_k; out->w[2] = c->w_v; out->eps = c->eps;
  return KDA_OK;
}

kda_status kda_prologue(const void* xq, const void* xk, const void* xv, kda_dtype dtype,
                        const kda_conv* conv, const float* conv_state_in,
                        float* conv_state_out, const int32_t* cu_seqlens, int N, int T,
                        int H, int Dk, int Dv, void* q, void* k, void* v, void* stream) {
  if (N < 0 || T < 0 || H <= 0) return fail(KDA_ERR_INVALID_ARGUMENT, "need N, T >= 0 and H > 0");
  if (N == 0) return ok();
  if (!dtype_ok(dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "bad dtype");
  kda::ConvArgs ca;
  kda_status s = check_conv(conv, &ca);
  if (s != KDA_OK) return s;
  if (!((Dk == 64 || Dk == 128) && (Dv == 64 || Dv == 128)))
    return fail(KDA_ERR_UNSUPPORTED, "Dk and Dv must be 64 or 128 (got %d, %d)", Dk, Dv);
  const long long total = cu_seqlens ? (long long)T : (long long)N * T;
  if (total > 0) {
    if (!xq || !xk || !xv || !q || !k || !v)
      return fail(KDA_ERR_INVALID_ARGUMENT, "x_q, x_k, x_v, q, k and v must be non-null");
    if (!aligned16(xq) || !aligned16(xk) || !aligned16(xv) || !aligned16(q) || !aligned16(k) ||
        !aligned16(v))
      return fail(KDA_ERR_INVALID_ARGUMENT, "token tensors must be 16-byte aligned");
    const size_t e = esize(dtype), rows = (size_t)total * H;
    const size_t sw = (size_t)N * 3 * H * (2 * Dk + Dv) * 4;
    const Range ins[] = {{xq, rows * Dk * e}, {xk, rows * Dk * e}, {xv, rows * Dv * e},
                         {conv->w_q, (size_t)H * Dk * 16}, {conv->w_k, (size_t)H * Dk * 16},
                         {conv->w_v, (size_t)H * Dv * 16}, {conv_state_in, conv_state_in ? sw : 0},
                         {cu_seqlens, cu_seqlens ? (size_t)(N + 1) * 4 : 0}};
    const char* const in[] = {"x_q", "x_k", "x_v", "w_q", "w_k", "w_v", "conv_state_in",
                              "cu_seqlens"};
    const Range outs[] = {{q, rows * Dk * e}, {k, rows * Dk * e}, {v, rows * Dv * e},
                          {conv_state_out, conv_state_out ? sw : 0}};
    const char* const on[] = {"q", "k", "v", "conv_state_out"};
    const char *a = nullptr, *b = nullptr;
    if (any_overlap(outs, on, ins, in, &a, &b))
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s must not overlap %s", a, b);
    for (int i = 0; i < 4; ++i)
      for (int j = i + 1; j < 4; ++j)
        if (overlaps(outs[i], outs[j]))
          return fail(KDA_ERR_INVALID_ARGUMENT, "%s must not overlap %s", on[i], on[j]);
  }
  if ((conv_state_in && !aligned16(conv_state_in)) || (conv_state_out && !aligned16(conv_state_out)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "conv states must be 16-byte aligned");
  if (conv_state_out && conv_state_out == conv_state_in)
    return fail(KDA_ERR_INVALID_ARGUMENT, "conv_state_out must not alias conv_state_in");
  if (cu_seqlens && ((uintptr_t)cu_seqlens & 3u))
    return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens must be 4-byte aligned");
  kda::PrologueArgs a;
  a.xq = xq; a.xk = xk; a.xv = xv; a.bf16 = dtype == KDA_BF16; a.conv = ca;
  a.st_in = conv_state_in; a.st_out = conv_state_out; a.cu_seqlens = cu_seqlens; a.n_seq = N;
  a.Tseq = T; a.total = total; a.H = H; a.Dk = Dk; a.Dv = Dv; a.q = q; a.k = k; a.v = v;
  a.stream = stream;
  return hip_status(kda::launch_prologue(a));
}

kda_status kda_epilogue(const void* o, kda_dtype o_dtype, const void* g, kda_dtype g_dtype,
                        const float* w, float eps, void* y, kda_dtype y_dtype,
                        long long tokens, int H, int Dv, void* stream) {
  if (tokens < 0 || H <= 0) return fail(KDA_ERR_INVALID_ARGUMENT, "need tokens >= 0 and H > 0");
  if (!dtype_ok(o_dtype) || !dtype_ok(g_dtype) || !dtype_ok(y_dtype))
    return fail(KDA_ERR_INVALID_ARGUMENT, "bad dtype");
  if (!eps_ok(eps)) return fail(KDA_ERR_INVALID_ARGUMENT, "RMSNorm eps must be finite and > 0");
  if (Dv != 64 && Dv != 128) return fail(KDA_ERR_UNSUPPORTED, "Dv must be 64 or 128 (got %d)", Dv);
  if (tokens == 0) return ok();
  if (!o || !g || !w || !y) return fail(KDA_ERR_INVALID_ARGUMENT, "o, g, w and y must be non-null");
  if (!aligned16(o) || !aligned16(g) || !aligned16(y) || ((uintptr_t)w & 3u))
    return fail(KDA_ERR_INVALID_ARGUMENT, "o, g, y must be 16-byte aligned, w 4-byte");
  if (y == o && y_dtype != o_dtype)
    return fail(KDA_ERR_INVALID_ARGUMENT, "y may alias o only with the same dtype");
  kda::EpilogueArgs a;
  a.o = o; a.o_bf16 = o_dtype == KDA_BF16; a.g = g; a.g_bf16 = g_dtype == KDA_BF16; a.w = w;
  a.eps = eps; a.y = y; a.y_bf16 = y_dtype == KDA_BF16; a.rows = tokens; a.H = H; a.Dv = Dv;
  a.stream = stream;
  return hip_status(kda::launch_epilogue(a));
}

// Shape and pointer checks shared by verify and commit (q and o are checked by
// the caller where they exist).
static kda_status multi_common(const void* k, const void* v, kda_dtype qkv_dtype,
                               const kda_gate* gate, const float* beta, const float* state,
                               int B, int N, int H, int Dk, int Dv, kda::Gate* g) {
  if (!k || !v || !beta || !state)
    return fail(KDA_ERR_INVALID_ARGUMENT, "k, v, beta and state must be non-null");
  if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16)
    return fail(KDA_ERR_INVALID_ARGUMENT, "bad qkv_dtype");
  if (H <= 0 || Dk <= 0 || Dv <= 0)
    return fail(KDA_ERR_INVALID_ARGUMENT, "H, Dk and Dv must be positive");
  if (!aligned16(k) || !aligned16(v) || !aligned16(state) || ((uintptr_t)beta & 3u))
    return fail(KDA_ERR_INVALID_ARGUMENT,
                "k, v and state must be 16-byte aligned, beta 4-byte aligned");
  kda_status s = check_gate(gate, true, g);
  if (s != KDA_OK) return s;
  if (!((Dk == 64 || Dk == 128) && (Dv == 64 || Dv == 128)))
    return fail(KDA_ERR_UNSUPPORTED, "Dk and Dv must be 64 or 128 (got %d, %d)", Dk, Dv);
  if (N > kda::kMaxDraft)
    return fail(KDA_ERR_UNSUPPORTED, "at most %d tokens per session (got %d)", kda::kMaxDraft, N);
  if ((long long)B * H > 0x7fffffffLL) return fail(KDA_ERR_INVALID_ARGUMENT, "B*H too large");
  return KDA_OK;
}

kda_status kda_decode_verify(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                             const kda_gate* gate, const float* beta, const float* state,
                             void* o, kda_dtype o_dtype, int B, int N, int H, int Dk, int Dv,
                             void* stream) {
  if (B < 0 || N < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "B and N must be >= 0");
  if (B == 0 || N == 0) return ok();
  if (!q || !o) return fail(KDA_ERR_INVALID_ARGUMENT, "q and o must be non-null");
  if (o_dtype != KDA_F32 && o_dtype != KDA_BF16)
    return fail(KDA_ERR_INVALID_ARGUMENT, "bad o_dtype");
  if (!aligned16(q) || ((uintptr_t)o & (o_dtype == KDA_BF16 ? 1u : 3u)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "q must be 16-byte aligned, o element-aligned");
  kda::Gate g;
  kda_status s = multi_common(k, v, qkv_dtype, gate, beta, state, B, N, H, Dk, Dv, &g);
  if (s != KDA_OK) return s;
  kda::DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.gate = g; a.beta = beta; a.state = const_cast<float*>(state);
  a.o = o; a.qkv_bf16 = qkv_dtype == KDA_BF16; a.o_bf16 = o_dtype == KDA_BF16;
  a.B = B; a.H = H; a.Dk = Dk; a.Dv = Dv; a.stream = stream;
  a.mode = kda::DECODE_VERIFY; a.N = N;
  return hip_status(kda::launch_decode(a));
}

kda_status kda_decode_commit(const void* k, const void* v, kda_dtype qkv_dtype,
                             const kda_gate* gate, const float* beta, const int32_t* n_accept,
                             float* state, int B, int N, int H, int Dk, int Dv, void* stream) {
  if (B < 0 || N < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "B and N must be >= 0");
  if (B == 0 || N == 0) return ok();
  if (!n_accept || ((uintptr_t)n_accept & 3u))
    return fail(KDA_ERR_INVALID_ARGUMENT, "n_accept must be non-null and 4-byte aligned");
  kda::Gate g;
  kda_status s = multi_common(k, v, qkv_dtype, gate, beta, state, B, N, H, Dk, Dv, &g);
  if (s != KDA_OK) return s;
  kda::DecodeArgs a;
  a.q = nullptr; a.k = k; a.v = v; a.gate = g; a.beta = beta; a.state = state; a.o = nullptr;
  a.qkv_bf16 = qkv_dtype == KDA_BF16; a.o_bf16 = false;
  a.B = B; a.H = H; a.Dk = Dk; a.Dv = Dv; a.stream = stream;
  a.mode = kda::DECODE_COMMIT; a.N = N; a.n_accept = n_accept;
  return hip_status(kda::launch_decode(a));
}

kda_status kda_decode_layer(kda_decode_mode mode, const void* xq, const void* xk, const void* xv,
                            kda_dtype x_dtype, const kda_conv* conv, float* conv_state,
                            const kda_gate* gate, const float* beta, float* state,
                            const kda_out_gate* out, void* y, kda_dtype y_dtype,
                            const int32_t* n_accept, int B, int N, int H, int Dk, int Dv,
                            void* stream) {
  if (mode != KDA_DECODE_STEP && mode != KDA_DECODE_VERIFY && mode != KDA_DECODE_COMMIT)
    return fail(KDA_ERR_INVALID_ARGUMENT, "unknown decode mode %d", (int)mode);
  if (B < 0 || N < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "B and N must be >= 0");
  if (mode == KDA_DECODE_STEP && N != 1 && B > 0)
    return fail(KDA_ERR_INVALID_ARGUMENT, "a step takes N == 1 token per session");
  if (B == 0 || N == 0) return ok();
  kda::Gate g;
  kda_status s = multi_common(xk, xv, x_dtype, gate, beta, state, B, N, H, Dk, Dv, &g);
  if (s != KDA_OK) return s;
  kda::ConvArgs ca;
  if ((s = check_conv(conv, &ca)) != KDA_OK) return s;
  if (!xq || !aligned16(xq)) return fail(KDA_ERR_INVALID_ARGUMENT, "x_q must be non-null and 16-byte aligned");
  if (!conv_state || !aligned16(conv_state))
    return fail(KDA_ERR_INVALID_ARGUMENT, "conv_state must be non-null and 16-byte aligned");
  kda::OutGateArgs og = {nullptr, nullptr, 1.f};
  if (mode != KDA_DECODE_COMMIT) {
    if (!out || !out->g || !out->w || !y)
      return fail(KDA_ERR_INVALID_ARGUMENT, "the output gate (g, w) and y must be non-null");
    if (!aligned16(out->g) || ((uintptr_t)out->w & 3u) || !aligned16(y))
      return fail(KDA_ERR_INVALID_ARGUMENT, "g and y must be 16-byte aligned, w 4-byte");
    if (!eps_ok(out->eps)) return fail(KDA_ERR_INVALID_ARGUMENT, "RMSNorm eps must be finite and > 0");
    if (!dtype_ok(y_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "bad y_dtype");
    og.g = out->g; og.w = out->w; og.eps = out->eps;
  } else if (!n_accept || ((uintptr_t)n_accept & 3u)) {
    return fail(KDA_ERR_INVALID_ARGUMENT, "n_accept must be non-null and 4-byte aligned");
  }
  kda::DecodeArgs a;
  a.q = nullptr; a.k = nullptr; a.v = nullptr; a.gate = g; a.beta = beta; a.state = state;
  a.o = mode == KDA_DECODE_COMMIT ? nullptr : y;
  a.qkv_bf16 = x_dtype == KDA_BF16; a.o_bf16 = mode != KDA_DECODE_COMMIT && y_dtype == KDA_BF16;
  a.B = B; a.H = H; a.Dk = Dk; a.Dv = Dv; a.stream = stream;
  a.mode = mode == KDA_DECODE_STEP ? kda::DECODE_STEP
         : mode == KDA_DECODE_VERIFY ? kda::DECODE_VERIFY : kda::DECODE_COMMIT;
  a.N = N; a.n_accept = n_accept;
  a.layer = true;
  a.io.xq = xq; a.io.xk = xk; a.io.xv = xv; a.io.conv = ca; a.io.conv_state = conv_state;
  a.io.out = og;
  return hip_status(kda::launch_decode(a));
}

kda_status kda_prefill_layer(const void* xq, const void* xk, const void* xv, kda_dtype x_dtype,
                             const kda_conv* conv, const float* conv_state_in,
                             float* conv_state_out, const kda_gate* gate, const float* beta,
                             const int32_t* cu_seqlens, int n_seq, int T,
                             const float* initial_state, float* final_state, float* o,
                             const kda_out_gate* out, void* y, kda_dtype y_dtype, int H, int Dk,
                             int Dv, int chunk, int n_segments, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (n_seq < 0 || T < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "n_seq and T must be >= 0");
  if (n_seq == 0) return ok();
  if (x_dtype != KDA_BF16) {
    if (!dtype_ok(x_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "bad x_dtype");
    return fail(KDA_ERR_UNSUPPORTED, "the layer prefill takes bf16 projections");
  }
  if (!dtype_ok(y_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "bad y_dtype");
  if (n_segments < 1 || n_segments > kda::kMaxSegments)
    return fail(KDA_ERR_INVALID_ARGUMENT, "n_segments must lie in [1, %d] (got %d)",
                kda::kMaxSegments, n_segments);
  kda::LayerPro pro{};
  kda_status s = check_conv(conv, &pro.conv);
  if (s != KDA_OK) return s;
  if (((uintptr_t)conv->w_q | (uintptr_t)conv->w_k | (uintptr_t)conv->w_v) & 15u)
    return fail(KDA_ERR_INVALID_ARGUMENT, "conv taps must be 16-byte aligned");
  if ((conv_state_in && !aligned16(conv_state_in)) || (conv_state_out && !aligned16(conv_state_out)))
    return fail(KDA_ERR_INVALID_ARGUMENT, "conv states must be 16-byte aligned");
  if (conv_state_out && conv_state_out == conv_state_in)
    return fail(KDA_ERR_INVALID_ARGUMENT, "conv_state_out must not alias conv_state_in");
  if (!out || !out->w || !eps_ok(out->eps))
    return fail(KDA_ERR_INVALID_ARGUMENT, "output gate: w non-null and eps finite and > 0");
  const bool tokens = T > 0;
  if (tokens) {
    if (!out->g || !y || !o)
      return fail(KDA_ERR_INVALID_ARGUMENT, "o, y and the output gate g must be non-null");
    if (!aligned16(out->g) || !aligned16(y) || !aligned16(o) || ((uintptr_t)out->w & 3u))
      return fail(KDA_ERR_INVALID_ARGUMENT, "o, y, g must be 16-byte aligned, w 4-byte");
    if ((void*)o == y && y_dtype != KDA_F32)
      return fail(KDA_ERR_INVALID_ARGUMENT, "y may alias o only as fp32");
    if (cu_seqlens && ((uintptr_t)cu_seqlens & 3u))
      return fail(KDA_ERR_INVALID_ARGUMENT, "cu_seqlens must be 4-byte aligned");
    if (kda::prefill_supported(true, Dk, Dv) && H > 0) {
      const size_t need = kda::prefill_segmented_bytes(n_seq, H, Dk, Dv, n_segments);
      if (need == 0) return fail(KDA_ERR_INVALID_ARGUMENT, "sizes too large for the layer prefill");
      if (!workspace || workspace_bytes < need)
        return fail(KDA_ERR_INVALID_ARGUMENT,
                    "the layer prefill needs a workspace of %zu bytes (got %zu)", need,
                    workspace ? workspace_bytes : (size_t)0);
    }
  }
  if (tokens) {
    const size_t tok = cu_seqlens ? (size_t)T : (size_t)n_seq * T;
    const size_t rows = tok * H, sw = (size_t)n_seq * 3 * H * (2 * Dk + Dv) * 4;
    const Range ins[] = {{xq, rows * Dk * 2}, {xk, rows * Dk * 2}, {xv, rows * Dv * 2},
                         {out->g, rows * Dv * 2}, {beta, rows * 4},
                         {gate ? gate->gate : nullptr, gate_bytes(gate, rows, Dk)},
                         {conv->w_q, (size_t)H * Dk * 16}, {conv->w_k, (size_t)H * Dk * 16},
                         {conv->w_v, (size_t)H * Dv * 16}, {conv_state_in, conv_state_in ? sw : 0},
                         {cu_seqlens, cu_seqlens ? (size_t)(n_seq + 1) * 4 : 0}};
    const char* const in[] = {"x_q", "x_k", "x_v", "g", "beta", "the gate tensor", "w_q", "w_k",
                              "w_v", "conv_state_in", "cu_seqlens"};
    // y may be o itself (fp32), checked above; otherwise the three are apart
    const Range outs[] = {{o, rows * Dv * 4}, {(void*)y == (void*)o ? nullptr : y, rows * Dv * esize(y_dtype)},
                          {conv_state_out, conv_state_out ? sw : 0}};
    const char* const on[] = {"o", "y", "conv_state_out"};
    const char *a = nullptr, *b = nullptr;
    if (any_overlap(outs, on, ins, in, &a, &b))
      return fail(KDA_ERR_INVALID_ARGUMENT, "%s must not overlap %s", a, b);
    for (int i = 0; i < 3; ++i)
      for (int j = i + 1; j < 3; ++j)
        if (overlaps(outs[i], outs[j]))
          return fail(KDA_ERR_INVALID_ARGUMENT, "%s must not overlap %s", on[i], on[j]);
  }
  pro.st_in = conv_state_in;
  pro.st_out = conv_state_out;
  pro.out.g = out->g;
  pro.out.w = out->w;
  pro.out.eps = out->eps;
  pro.y = y;
  pro.y_bf16 = y_dtype == KDA_BF16;
  return prefill_common(xq, xk, xv, x_dtype, gate, beta, cu_seqlens, n_seq, T, initial_state,
                        final_state, o, KDA_F32, H, Dk, Dv, chunk, workspace, workspace_bytes,
                        stream, n_segments, &pro);
}

}  // extern "C"
