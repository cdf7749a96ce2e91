/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward operator.
 *
 * The operator, per (sequence, head), with S in R^{Dk x Dv} (rows = key
 * channels, columns = value channels):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                      (read-out from the UPDATED state)
 *
 * alpha_t in (0,1]^Dk decays each key channel (row) of the state first; the
 * delta-rule erase and the write then act on the decayed state.  Sources:
 * "Kimi Delta Attention 完全拆解" (pinghaoyang.com.cn), section "KDA 的核心：让遗忘从
 * 一个标量细化为逐通道向量"; "Kimi K3模型架构详解" (gentlecold.top), section 3.2
 * "KDA的递推式"; "从线性注意力到 KDA" (blog.javazero.top), sections "一步在线学习" and
 * "衰减为什么要按行做".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller, dense and
 *    row-major in the shapes given, aligned to their element size; state
 *    pointers (initial_state, final_state, state), the decode entry points'
 *    q, k, v and per-channel gate, and, for the bf16 prefill entry points, q,
 *    k, v and alpha 16-byte aligned; a prefill workspace 256-byte aligned.  The library never allocates device memory and keeps
 *    no state besides cached device properties.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls enqueue work asynchronously on it; a kernel fault surfaces at the
 *    caller's next synchronisation.
 *  - Argument errors are detected on the host and returned BEFORE anything is
 *    launched (KDA_ERR_INVALID_ARGUMENT / KDA_ERR_UNSUPPORTED);
 *    kda_last_error_message() then gives the detail (thread-local).  A failed
 *    launch returns KDA_ERR_HIP.  No exception or abort crosses the ABI.
 *  - Supported shapes: Dk, Dv in {64, 128}; chunk == 64.  q/k/v dtype KDA_BF16
 *    or KDA_F32 (all three the same); alpha, beta and the state are fp32; the
 *    output o is KDA_F32 or KDA_BF16.  The prefill entry points compute fp32
 *    q/k/v in fp32 arithmetic: with Dk == 64 in the chunk form, with Dk == 128
 *    as the token recurrence (one workgroup per sequence and head stepping
 *    its tokens; the same function, slower); fp32 q, k, v and a per-channel
 *    gate 16-byte aligned at Dk == 128.  The layer prefill and the segmented
 *    schedule take bf16 only (as stated with them).
 *  - Documented, not checked: alpha in (0, 1] (any value in it, however fast
 *    the decay: a 16-token tile whose decay product leaves the range of the
 *    chunked kernels' factored form is computed by exact running products
 *    instead); finite beta; monotone cu_seqlens.  Checked: no output's byte
 *    range overlaps an input's (except final_state == initial_state, in place,
 *    and y == o where documented).
 *  - Results are deterministic (no floating-point atomics): the same call on
 *    the same inputs gives bitwise-identical results, and a sequence of a
 *    packed batch gives bitwise the result it gives when run alone.  Both
 *    prefill schedules (below) compute the same products in the same order and
 *    give bitwise-identical results.
 *
 * Prefill schedules (bf16 inputs)
 * -------------------------------
 * The chunk form splits every 64-token chunk into work that does not depend on
 * the entry state (decays, A and its UT inverse, W, U, the intra-chunk q.k
 * matrix) and a short state-dependent remainder ("Kimi Delta Attention 完全拆解",
 * section "chunk 内并行、chunk 间递推").  Fused: one kernel, one workgroup per
 * (sequence, head, 64-wide value slice) walks its chunks and does both.
 * Two-pass: the packed token axis is cut into windows of 8192 tokens; for each
 * window a first kernel does the state-independent work of the chunks starting
 * in it, once per (chunk, head) over the whole device, and leaves per-chunk
 * operands in the caller's workspace, and a second kernel runs the recurrence
 * over those chunks, carrying the state from window to window.  The two-pass
 * schedule runs when the call passes a workspace of at least
 * kda_prefill_workspace_size / kda_prefill_varlen_workspace_size bytes (a
 * non-zero value); otherwise the fused kernel runs.  Like the state, the
 * workspace does not grow with the sequence length (about 16.3 MiB per head for
 * one sequence at Dk = Dv = 128); its contents on return are unspecified.
 * kda_prefill_two_pass_preferred says which schedule is expected to be faster
 * on the current device.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad alignment      */
    KDA_ERR_UNSUPPORTED = 2,      /* valid but not built (head dim, chunk, dtype) */
    KDA_ERR_HIP = 3               /* the HIP runtime reported an error            */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/*
 * The decay gate, for the *_gated entry points.  The recurrence always uses a
 * per-key-channel alpha_t in (0, 1]^Dk; the gate hands it over in one of the
 * parametrizations the pages describe, and the kernels form alpha (in fp32) as
 * they load it:
 *
 *   KDA_GATE_ALPHA    gate [.., H, Dk] fp32 = alpha itself (what the plain
 *                     entry points take)
 *   KDA_GATE_LOG      gate [.., H, Dk] fp32 = g = log alpha <= 0, alpha = exp(g):
 *                     the gate kept in log space ("Kimi Delta Attention 完全拆解",
 *                     section "KDA 的核心：让遗忘从一个标量细化为逐通道向量")
 *   KDA_GATE_BOUNDED  gate [.., H, Dk] fp32 = logits z, a_log [H] fp32 = A;
 *                     g = g_min * Sigmoid(exp(A_h) z), alpha = exp(g): K3's
 *                     lower-bounded gate with g_min = -5 on the pages ("Kimi K3 的
 *                     KDA" section 6; "Kimi K3模型架构详解" section 3.4).  g_min must
 *                     lie in [-5, 0): every token then decays by at most e^-5,
 *                     which keeps the 16-token tile factors of the chunked paths
 *                     in fp32 range
 *   KDA_GATE_SCALAR   gate [.., H] fp32 = one alpha per token and head, applied
 *                     to every key channel: gated DeltaNet, the vector gate with
 *                     equal components (same section of "Kimi Delta Attention
 *                     完全拆解")
 *   KDA_GATE_NONE     no decay, alpha = 1: DeltaNet; `gate` is ignored
 *
 * ".." stands for the leading token dimensions of the entry point: [B, T] for
 * the dense prefill, [1, total_tokens] for the packed prefill, [B] for decode.
 * Pointers are device pointers aligned like alpha (16 bytes for the bf16
 * prefill paths with a per-channel gate, 4 bytes otherwise).
 */
typedef enum {
    KDA_GATE_ALPHA = 0,
    KDA_GATE_LOG = 1,
    KDA_GATE_BOUNDED = 2,
    KDA_GATE_SCALAR = 3,
    KDA_GATE_NONE = 4
} kda_gate_kind;

typedef struct {
    kda_gate_kind kind;
    const float* gate;   /* per kind above; may be NULL for KDA_GATE_NONE        */
    const float* a_log;  /* [H] per-head log scale A, KDA_GATE_BOUNDED only      */
    float g_min;         /* KDA_GATE_BOUNDED only, in [-5, 0)                   */
} kda_gate;

/*
 * kda_prefill_chunked -- dense prefill over B sequences of T tokens each.
 * The chunkwise form of the recurrence: inside each 64-token chunk the
 * cumulative decay, the strictly lower-triangular beta-weighted decayed k k^T
 * matrix A, its unit-triangular inverse (I + A)^{-1} (the UT transform), the
 * intra-chunk q.k matrix and the pseudo-values U - W S are formed, and the state
 * is handed from chunk to chunk ("Kimi Delta Attention 完全拆解", section
 * "chunk 内并行、chunk 间递推"; "Kimi K3 的 KDA" section 5; "Kimi K3模型架构详解"
 * section 3.5).  Equal to the token recurrence up to rounding.
 *
 *   q, k          [B, T, H, Dk]  qkv_dtype
 *   v             [B, T, H, Dv]  qkv_dtype
 *   alpha         [B, T, H, Dk]  fp32, per-key-channel decay
 *   beta          [B, T, H]      fp32, write strength
 *   initial_state [B, H, Dk, Dv] fp32, or NULL for zeros
 *   final_state   [B, H, Dk, Dv] fp32, or NULL to skip; may equal initial_state
 *                 (updated in place)
 *   o             [B, T, H, Dv]  o_dtype
 *   chunk         must be 64
 *   workspace     NULL (fused schedule) or device scratch of workspace_bytes
 *                 bytes, 256-byte aligned, not aliasing any tensor; with at
 *                 least kda_prefill_workspace_size(B, T, H, Dk, Dv, chunk)
 *                 bytes (bf16 inputs) the two-pass schedule runs
 * T == 0 or B == 0 is allowed (then only final_state = initial_state is written).
 */
kda_status kda_prefill_chunked(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                               const float* alpha, const float* beta,
                               const float* initial_state, float* final_state,
                               void* o, kda_dtype o_dtype,
                               int B, int T, int H, int Dk, int Dv, int chunk,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_prefill_chunked_noalloc -- kda_prefill_chunked for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The same arguments without a workspace;
 * bf16 inputs run the two-pass schedule with its workspace in a device array
 * of the library (128 MiB, one per device, held until the process ends; its
 * address is looked up on the first call on a device), so the results are
 * bitwise those of kda_prefill_chunked with a workspace.  fp32 inputs need no
 * workspace.  Calls neither hipMalloc nor hipFree.
 *   Sizes whose kda_prefill_workspace_size exceeds 128 MiB (at Dk = Dv = 128:
 *   more than 7 heads of one sequence) return KDA_ERR_INVALID_ARGUMENT.
 *   Every call on a device shares that device's array: calls that overlap on
 *   one device (other streams, other threads) race and must be serialised by
 *   the caller.  Nothing in the array needs clearing between calls.
 */
kda_status kda_prefill_chunked_noalloc(const void* q, const void* k, const void* v,
                                       kda_dtype qkv_dtype, const float* alpha, const float* beta,
                                       const float* initial_state, float* final_state,
                                       void* o, kda_dtype o_dtype,
                                       int B, int T, int H, int Dk, int Dv, int chunk,
                                       void* stream);

/*
 * kda_prefill_varlen -- packed variable-length prefill.  N sequences are
 * concatenated along the token axis (B = 1); sequence i occupies tokens
 * cu_seqlens[i] .. cu_seqlens[i+1]-1, has its own initial state and final state,
 * and its chunks start at its own first token (the last chunk may be partial).
 * A sequence's results do not depend on its neighbours ("Kimi Delta Attention
 * 完全拆解", section "数值路径必须以 recurrent 版本为基准校验").
 *
 *   q, k, alpha   [1, total_tokens, H, Dk];  v, o [1, total_tokens, H, Dv]
 *   beta          [1, total_tokens, H]
 *   cu_seqlens    DEVICE int32 [N + 1], cu_seqlens[0] = 0,
 *                 cu_seqlens[N] = total_tokens, non-decreasing (read on the
 *                 device; not checked)
 *   initial_state [N, H, Dk, Dv] or NULL;  final_state [N, H, Dk, Dv] or NULL
 *   workspace     as for kda_prefill_chunked, sized by
 *                 kda_prefill_varlen_workspace_size(N, total_tokens, ...)
 * Other arguments as for kda_prefill_chunked.
 */
kda_status kda_prefill_varlen(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                              const float* alpha, const float* beta,
                              const int32_t* cu_seqlens, int N, int total_tokens,
                              const float* initial_state, float* final_state,
                              void* o, kda_dtype o_dtype,
                              int H, int Dk, int Dv, int chunk,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_decode_step -- one token for each of B sessions, the fused recurrent
 * form: decay the state, read the decayed state's answer for k, write the
 * corrected value along k, read out with q ("Kimi Delta Attention 完全拆解",
 * section "一次 KDA 前向究竟发生了什么", the decode sequence; section "Prefill 与
 * decode 必须走不同 Kernel").  The state is read once and written once.
 *
 *   q, k   [B, H, Dk] qkv_dtype;  v [B, H, Dv] qkv_dtype
 *   alpha  [B, H, Dk] fp32;       beta [B, H] fp32
 *   state  [B, H, Dk, Dv] fp32, updated IN PLACE
 *   o      [B, H, Dv] o_dtype
 * q, k, v, alpha and state 16-byte aligned.
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                           const float* alpha, const float* beta, float* state,
                           void* o, kda_dtype o_dtype, int B, int H, int Dk, int Dv,
                           void* stream);

/*
 * kda_prefill_chunked_gated, kda_prefill_varlen_gated, kda_decode_step_gated --
 * the same operations with the decay given as a kda_gate (`gate` a HOST
 * pointer to the descriptor, read during the call; the tensors it names are
 * device tensors) instead of an alpha tensor.  The plain entry points are
 * these with {KDA_GATE_ALPHA, alpha}.  An unknown kind, a NULL gate tensor (for
 * a kind that reads one), a NULL a_log or a g_min outside [-5, 0) for
 * KDA_GATE_BOUNDED return KDA_ERR_INVALID_ARGUMENT.
 */
kda_status kda_prefill_chunked_gated(const void* q, const void* k, const void* v,
                                     kda_dtype qkv_dtype, const kda_gate* gate,
                                     const float* beta, const float* initial_state,
                                     float* final_state, void* o, kda_dtype o_dtype,
                                     int B, int T, int H, int Dk, int Dv, int chunk,
                                     void* workspace, size_t workspace_bytes, void* stream);

kda_status kda_prefill_varlen_gated(const void* q, const void* k, const void* v,
                                    kda_dtype qkv_dtype, const kda_gate* gate,
                                    const float* beta, const int32_t* cu_seqlens, int N,
                                    int total_tokens, const float* initial_state,
                                    float* final_state, void* o, kda_dtype o_dtype,
                                    int H, int Dk, int Dv, int chunk,
                                    void* workspace, size_t workspace_bytes, void* stream);

kda_status kda_decode_step_gated(const void* q, const void* k, const void* v,
                                 kda_dtype qkv_dtype, const kda_gate* gate, const float* beta,
                                 float* state, void* o, kda_dtype o_dtype, int B, int H, int Dk,
                                 int Dv, void* stream);

/*
 * kda_decode_verify, kda_decode_commit -- speculative decoding with replay.
 * The state is updated in place, so tokens a verifier rejects cannot be taken
 * back once stepped; following "Kimi K3模型架构详解" (section 9.2, the inference
 * kernel; section 10.1, rollback by replay; section 11.1, the decode /
 * spec-decode regime), no state copy is
 * kept per draft position: the caller keeps the draft tokens' inputs, verify
 * computes their outputs without touching the state, and commit replays the
 * accepted ones into it.
 *
 * kda_decode_verify: for each of B sessions, N tokens (1 <= N <= 16) stepped
 * in order from `state`; o[b, t] is the output of token t after tokens
 * 0..t.  `state` is READ ONLY.
 *   q, k   [B, N, H, Dk] qkv_dtype;  v [B, N, H, Dv] qkv_dtype
 *   gate   kda_gate over [B, N, H, Dk] ([B, N, H] for KDA_GATE_SCALAR)
 *   beta   [B, N, H] fp32
 *   state  [B, H, Dk, Dv] fp32, not written
 *   o      [B, N, H, Dv] o_dtype
 *
 * kda_decode_commit: for each session b, tokens 0..n_accept[b]-1 of the same
 * k, v, gate and beta tensors folded into `state` (IN PLACE).
 *   n_accept  DEVICE int32 [B], read on the device and clamped to [0, N];
 *             a session with 0 is left untouched
 *
 * Arithmetic: below 6 drafts for verify and below 12 for commit, the tokens
 * are stepped with exactly the arithmetic of kda_decode_step, so verify's
 * outputs are bitwise the steps' outputs and commit leaves bitwise the state
 * that n_accept[b] steps would leave.  From 6 (verify) and 12 (commit) drafts
 * on, the drafts are one chunk of the chunk form ("Kimi Delta Attention 完全拆解",
 * section "chunk 内并行、chunk 间递推"), evaluated in fp32 on the matrix cores:
 * equal to the steps up to fp32 rounding (about 1e-6 relative), not bitwise.
 *
 * Both: q, k, v, state and a per-channel gate 16-byte aligned, beta and
 * n_accept 4-byte aligned, o element-aligned; Dk, Dv in {64, 128}.  B == 0 or
 * N == 0 is a no-op; N > 16 returns KDA_ERR_UNSUPPORTED.
 */
kda_status kda_decode_verify(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                             const kda_gate* gate, const float* beta, const float* state,
                             void* o, kda_dtype o_dtype, int B, int N, int H, int Dk, int Dv,
                             void* stream);

kda_status kda_decode_commit(const void* k, const void* v, kda_dtype qkv_dtype,
                             const kda_gate* gate, const float* beta, const int32_t* n_accept,
                             float* state, int B, int N, int H, int Dk, int Dv, void* stream);

/*
 * The layer's steps on either side of the recurrence ("Kimi Delta Attention
 * 完全拆解", section "一次 KDA 前向究竟发生了什么", the formulas for q, k, v and the
 * layer output; "从线性注意力到 KDA", the ShortConv / L2Norm bullets and the
 * per-head output norm and gate):
 *   prologue  q, k = L2Norm(Swish(ShortConv(x_q / x_k))), v = Swish(ShortConv(x_v))
 *   epilogue  y = RMSNorm(o) * w * Sigmoid(g), per head over its Dv channels
 * x_q, x_k, x_v and g are the outputs of the layer's projections (not part of
 * this library).  ShortConv is depthwise and causal with kernel size 4: per
 * channel, y_t = w[0] x_{t-3} + w[1] x_{t-2} + w[2] x_{t-1} + w[3] x_t, no bias.
 * Its state is the last 3 inputs of q | k | v of every head, the only state of
 * the layer besides S: conv state [sessions, 3, H, 2 Dk + Dv] fp32, oldest row
 * first.  L2Norm: x / sqrt(sum x^2 + eps).  RMSNorm: o / sqrt(mean o^2 + eps).
 */
typedef struct {
    const float* w_q;  /* [H, Dk, 4] taps (tap 3 weights the current token) */
    const float* w_k;  /* [H, Dk, 4] */
    const float* w_v;  /* [H, Dv, 4] */
    float eps;         /* L2Norm epsilon, finite and > 0 (e.g. 1e-6) */
} kda_conv;

/*
 * kda_prologue -- the prologue over a prefill, dense (cu_seqlens NULL: N
 * sequences of T tokens, tensors [N, T, H, .]) or packed (cu_seqlens DEVICE
 * int32 [N + 1], T = total tokens, tensors [1, T, H, .]).
 *   xq, xk [.., H, Dk], xv [.., H, Dv]  dtype;  q, k, v outputs of the same
 *                      shapes and dtype (rounded once), not aliasing the inputs
 *   conv_state_in      [N, 3, H, 2 Dk + Dv] fp32 or NULL (zeros): the inputs
 *                      before each sequence's first token
 *   conv_state_out     same shape or NULL (not written): the last 3 inputs of
 *                      each sequence (an empty sequence's is copied through);
 *                      must not alias conv_state_in
 * All tensors 16-byte aligned; Dk, Dv in {64, 128}.
 */
kda_status kda_prologue(const void* xq, const void* xk, const void* xv, kda_dtype dtype,
                        const kda_conv* conv, const float* conv_state_in,
                        float* conv_state_out, const int32_t* cu_seqlens, int N, int T,
                        int H, int Dk, int Dv, void* q, void* k, void* v, void* stream);

/*
 * kda_epilogue -- y = RMSNorm(o) * w * Sigmoid(g) for `tokens` x H rows of Dv.
 *   o [tokens, H, Dv] o_dtype;  g [tokens, H, Dv] g_dtype;  w [Dv] fp32
 *   y [tokens, H, Dv] y_dtype (may alias o when the dtypes match)
 * eps finite and > 0 (e.g. 1e-5); all tensors 16-byte aligned; Dv in {64, 128}.
 */
kda_status kda_epilogue(const void* o, kda_dtype o_dtype, const void* g, kda_dtype g_dtype,
                        const float* w, float eps, void* y, kda_dtype y_dtype,
                        long long tokens, int H, int Dv, void* stream);

/*
 * kda_decode_layer -- the whole recurrent layer step in one kernel, as K3's
 * inference kernel fuses it ("Kimi K3模型架构详解" section 9.2: short conv, input
 * norm, gate, recurrence and output norm): the prologue from the projections'
 * outputs and the conv state, the decode call of `mode`, the epilogue.
 *   KDA_DECODE_STEP    N must be 1: y written; state and conv_state advanced
 *   KDA_DECODE_VERIFY  y of the N tokens; state and conv_state only read
 *   KDA_DECODE_COMMIT  the first n_accept[b] tokens replayed from their cached
 *                      projections: state and conv_state advanced; no y
 *   xq, xk [B, N, H, Dk], xv [B, N, H, Dv]  x_dtype (xq is needed by commit too:
 *                      the conv state of q advances)
 *   conv, conv_state   as for kda_prologue, conv_state [B, 3, H, 2 Dk + Dv]
 *   gate, beta         as for kda_decode_verify ([B, N, H, Dk] / [B, N, H])
 *   state              [B, H, Dk, Dv] fp32
 *   out                output gate: g [B, N, H, Dv] x_dtype, w [Dv], eps
 *   y                  [B, N, H, Dv] y_dtype (not for commit)
 * The fused verify and commit take the plain calls' forms (the token loop
 * below 6 / 12 drafts, the chunk form from there on): with the standalone
 * kda_prologue before and kda_epilogue after the plain call (its o in fp32),
 * the results are bitwise the same, conv state included.
 * Time for memory: the fused call needs no intermediate q, k, v or o; on
 * MI355X it is faster than the three calls at every draft count.
 * Alignment and limits as for kda_decode_verify.
 */
typedef enum { KDA_DECODE_STEP = 0, KDA_DECODE_VERIFY = 1, KDA_DECODE_COMMIT = 2 } kda_decode_mode;

typedef struct {
    const void* g;     /* [B, N, H, Dv] output-gate logits, the token dtype */
    const float* w;    /* [Dv] RMSNorm weight */
    float eps;         /* finite and > 0 (e.g. 1e-5) */
} kda_out_gate;

kda_status kda_decode_layer(kda_decode_mode mode, const void* xq, const void* xk, const void* xv,
                            kda_dtype x_dtype, const kda_conv* conv, float* conv_state,
                            const kda_gate* gate, const float* beta, float* state,
                            const kda_out_gate* out, void* y, kda_dtype y_dtype,
                            const int32_t* n_accept, int B, int N, int H, int Dk, int Dv,
                            void* stream);

/*
 * kda_prefill_layer -- the recurrent layer over a prefill, from the
 * projections' outputs to the gated output: the prologue, the two-pass
 * (optionally segmented) recurrence and the epilogue ("Kimi Delta Attention
 * 完全拆解", section "一次 KDA 前向究竟发生了什么"; "从线性注意力到 KDA", the
 * ShortConv / L2Norm bullets and the output norm and gate).  The prologue runs
 * inside the first pass as it loads each chunk, so q, k and v are never
 * stored; the conv state is handed on after the recurrence and the epilogue
 * turns o into y.
 *   xq, xk [.., H, Dk], xv [.., H, Dv]  bf16 (x_dtype must be KDA_BF16)
 *   conv, conv_state_in, conv_state_out  as for kda_prologue (taps 16-byte
 *                      aligned; conv_state_out may be NULL)
 *   gate, beta, cu_seqlens, n_seq, T, initial_state, final_state  as for
 *                      kda_prefill_segmented (dense when cu_seqlens is NULL)
 *   o                  [.., H, Dv] fp32: the recurrence's output, before the
 *                      epilogue (caller-owned scratch or result)
 *   out                output gate: g [.., H, Dv] bf16, w [Dv], eps
 *   y                  [.., H, Dv] y_dtype (may alias o as fp32)
 *   n_segments, workspace  as for kda_prefill_segmented (workspace required
 *                      when there are tokens; 1 segment is the two-pass
 *                      schedule)
 * Equal to kda_prologue, the recurrence and kda_epilogue up to rounding (the
 * L2Norm's sum of squares is associated differently; q, k, v are rounded to
 * bf16 as the standalone prologue stores them).  The one call trades time for
 * memory: it needs no q, k, v buffers (3 x tokens x H x Dk bf16 values), but
 * where they fit, kda_prologue + kda_prefill_chunked (two-pass) + kda_epilogue
 * run faster (on MI355X, for 8192 tokens and 96 heads of 128 channels, about
 * 1.27 ms against 1.42 ms).
 */
kda_status kda_prefill_layer(const void* xq, const void* xk, const void* xv, kda_dtype x_dtype,
                             const kda_conv* conv, const float* conv_state_in,
                             float* conv_state_out, const kda_gate* gate, const float* beta,
                             const int32_t* cu_seqlens, int n_seq, int T,
                             const float* initial_state, float* final_state, float* o,
                             const kda_out_gate* out, void* y, kda_dtype y_dtype, int H, int Dk,
                             int Dv, int chunk, int n_segments, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * kda_prefill_workspace_size -- workspace bytes that enable the two-pass
 * schedule of kda_prefill_chunked for these sizes, independent of T (the state
 * is fixed-size, "Kimi K3 混合线性注意力": the per-session state does not grow
 * with length): a chunk table of B + 1 int32, one carried state per
 * (sequence, head) and the operand blocks of one window, (128 + B) * H of them
 * (131,584 B each at Dk = Dv = 128).  0 when the schedule does not exist for
 * the shape (head dims outside {64, 128}, or B <= 0).  (size_t)-1 for invalid
 * sizes.  Only bf16 inputs use it.
 */
size_t kda_prefill_workspace_size(int B, int T, int H, int Dk, int Dv, int chunk);

/*
 * kda_prefill_varlen_workspace_size -- as above for kda_prefill_varlen with N
 * packed sequences (any total_tokens, any split of them): the same layout
 * with B = N.
 */
size_t kda_prefill_varlen_workspace_size(int N, int total_tokens, int H, int Dk, int Dv,
                                         int chunk);

/*
 * kda_prefill_two_pass_preferred -- 1 if the two-pass schedule is expected to
 * be faster than the fused kernel on the current device for n_seq sequences of
 * total_tokens tokens in all, else 0.  The fused kernel fills the device with
 * n_seq * H * Dv / 64 workgroups and repeats the state-independent work for
 * each 64-wide value slice; the two-pass schedule wins when that grid is below
 * about twice the compute-unit count and the sequences are at least 4 chunks
 * long on average, and only while its workspace is at most 1/16 of device
 * memory and 16 GiB.
 */
int kda_prefill_two_pass_preferred(kda_dtype qkv_dtype, int n_seq, int total_tokens, int H, int Dk,
                                   int Dv);

/*
 * kda_prefill_segmented -- the two-pass prefill with the recurrence of each
 * window cut along the chunk axis, for calls with few (sequence, head) pairs
 * (few heads per device), where one workgroup per (sequence, head, 64 values)
 * walking a window's 64 chunks in order leaves most compute units idle.  A
 * segment of consecutive chunks acts on its entry state as the affine map
 * S -> M S + b, and maps compose associatively, (M2, b2) o (M1, b1) =
 * (M2 M1, M2 b1 + b2) ("Kimi K3模型架构详解", section 3.6, the segment summary
 * of context parallelism, here between segments of one device instead of
 * ranks).  Per window: a summary kernel carries [M | b] from [I | 0] through
 * each segment but the last (all segments at once), a combine kernel chains
 * the summaries into each segment's entry state (the split-bf16 MFMA product
 * of the state pass, in fp32), and the state pass runs all segments at once
 * from their entry states.  Each sequence uses min(n_segments, its chunks in
 * the window) segments; with one segment it runs exactly the two-pass schedule.
 *
 *   cu_seqlens    NULL: n_seq dense sequences of T tokens, tensors as for
 *                 kda_prefill_chunked with B = n_seq; else DEVICE int32
 *                 [n_seq + 1] delimiting packed sequences, T = total_tokens,
 *                 tensors as for kda_prefill_varlen with N = n_seq
 *   n_segments    in [1, 16] (kda_prefill_segments_preferred suggests one)
 *   workspace     required: at least kda_prefill_segmented_workspace_size(
 *                 n_seq, H, Dk, Dv, chunk, n_segments) bytes, 256-byte aligned
 * bf16 q, k, v only (KDA_ERR_UNSUPPORTED otherwise); other arguments as for
 * kda_prefill_chunked_gated.  Equal to the token recurrence up to rounding;
 * deterministic, but with n_segments > 1 not bitwise equal to the other
 * schedules (the products are associated differently), and a packed
 * sequence's segment boundaries depend on where its windows fall.
 */
kda_status kda_prefill_segmented(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                                 const kda_gate* gate, const float* beta,
                                 const int32_t* cu_seqlens, int n_seq, int T,
                                 const float* initial_state, float* final_state, void* o,
                                 kda_dtype o_dtype, int H, int Dk, int Dv, int chunk,
                                 int n_segments, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * kda_prefill_segmented_workspace_size -- the two-pass workspace plus the
 * segments' entry states (n_segments * n_seq * H * Dk * Dv fp32) and summaries
 * ((n_segments - 1) * n_seq * H * Dk * (Dk + Dv) fp32); 0 for unsupported head
 * dims, (size_t)-1 for invalid sizes or n_segments outside [1, 16].
 */
size_t kda_prefill_segmented_workspace_size(int n_seq, int H, int Dk, int Dv, int chunk,
                                            int n_segments);

/*
 * kda_prefill_segments_preferred -- a segment count expected to be fastest on
 * the current device (1: do not segment): the largest whose summary pass,
 * (n_segments - 1) * n_seq * H * (Dk + Dv) / 64 workgroups, fits one per
 * compute unit, at most 8, and at least 4 chunks per segment; 1 where the
 * two-pass schedule itself is not preferred or the inputs are not bf16.
 */
int kda_prefill_segments_preferred(kda_dtype qkv_dtype, int n_seq, int total_tokens, int H, int Dk,
                                   int Dv);

/* Static string naming a status code. */
const char* kda_status_string(kda_status s);

/* Thread-local detail of the last error returned on this thread ("" if none). */
const char* kda_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
