// kda_decode.hip -- decode kernels for B sessions x H heads (gfx950): the
// one-token step, and the multi-token verify / commit pair of speculative
// decoding.
//
// Fused recurrent form ("Kimi Delta Attention 完全拆解", section "一次 KDA 前向究竟
// 发生了什么": decay, the decayed state's answer for k, the corrected write along
// k, read-out with q; "Kimi K3模型架构详解" section 3.2):
//     Sbar = Diag(alpha) S,  u = beta (v - Sbar^T k),  S' = Sbar + k u^T,
//     o = S'^T q = Sbar^T q + (q.k) u
// The last identity lets both reductions (Sbar^T k and Sbar^T q) run in the same
// pass over the state, so each fp32 state tile is read once and written once:
// the step is HBM-bound (about 1 FLOP per byte), no MFMA.
//
// Mapping: one workgroup (4 waves) per (session, head) tile of Dk x Dv fp32.
// Wave w owns the value columns [w*Dv/4, (w+1)*Dv/4); a lane holds float4
// column groups of a set of rows, so every global access is a 16-byte vector
// and a wave touches whole 64..128-byte row segments; the state write uses
// non-temporal stores.  The column sums over
// the key axis are finished inside the wave with DPP row rotations and the
// permlane swaps (no LDS, no barrier).
//
// Speculative decoding ("Kimi K3模型架构详解" sections 9.2, 10.1 and 11.1): the state is
// updated in place, so a rejected draft token cannot simply be dropped.  Verify
// runs N draft tokens per session from the state kept in registers and writes
// their outputs, but not the state; commit replays the first n_accept[b] of
// those tokens from their cached inputs (k, v, gate, beta) and writes the
// state once.  A round moves three state tiles (read, read, write) where N
// single steps move 2N, and rejected tokens cost nothing to undo.  Both stage
// the session's N tokens in LDS once (alpha formed there), with the key-side
// vectors permuted so each lane reads its rows as contiguous 16-byte words.
#include "kda_common.h"
#include "kda_frag.h"
#include "kda_internal.h"
#include "kda_layer.h"

// Every product and sum is rounded on its own (no fused multiply-add
// contraction): the one-token step and the multi-token kernels evaluate the
// same per-token expressions in different code shapes, and uncontracted they
// agree bitwise (N single steps = verify + commit of N tokens).
#pragma clang fp contract(off)

namespace kda {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// four consecutive elements as fp32 (8- or 16-byte aligned)
template <typename TIn>
__device__ __forceinline__ floatx4 ld4(const TIn* p);
template <>
__device__ __forceinline__ floatx4 ld4<float>(const float* p) {
  return *reinterpret_cast<const floatx4*>(p);
}
template <>
__device__ __forceinline__ floatx4 ld4<bf16>(const bf16* p) {
  const u32x2 x = *reinterpret_cast<const u32x2*>(p);
  return floatx4{__uint_as_float(x[0] << 16), __uint_as_float(x[0] & 0xffff0000u),
                 __uint_as_float(x[1] << 16), __uint_as_float(x[1] & 0xffff0000u)};
}

// the same four elements as loaded (ld; gld through a pointer whose address
// space the compiler cannot see), widened to fp32 where they are used
// (cvt): the wait for a load goes where its first use is, so the use of a
// load that should not hold back the loads issued after it comes after them
// a load from device memory through a pointer whose address space the
// compiler cannot see (a global load, not a flat one, which is waited for
// with every other load in flight)
template <typename T>
__device__ __forceinline__ T gload(const void* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}
template <typename TIn>
struct Raw4;
template <>
struct Raw4<float> {
  typedef floatx4 T;
  static __device__ __forceinline__ T ld(const float* p) { return *reinterpret_cast<const T*>(p); }
  static __device__ __forceinline__ T gld(const float* p) { return gload<T>(p); }
  static __device__ __forceinline__ floatx4 cvt(const T& x) { return x; }
};
template <>
struct Raw4<bf16> {
  typedef u32x2 T;
  static __device__ __forceinline__ T ld(const bf16* p) { return *reinterpret_cast<const T*>(p); }
  static __device__ __forceinline__ T gld(const bf16* p) { return gload<T>(p); }
  static __device__ __forceinline__ floatx4 cvt(const T& x) {
    return floatx4{__uint_as_float(x[0] << 16), __uint_as_float(x[0] & 0xffff0000u),
                   __uint_as_float(x[1] << 16), __uint_as_float(x[1] & 0xffff0000u)};
  }
};

// Lane geometry of a Dk x Dv tile on 4 waves: wave w owns CW value columns;
// LPR lanes share a row set, a lane holds float4 columns of the NP rows
// ro + RPP i.
template <int DK, int DV>
struct Geo {
  static constexpr int CW = DV / 4;
  static constexpr int LPR = CW / 4;
  static constexpr int RPP = 64 / LPR;
  static constexpr int NP = DK / RPP;
  static_assert(NP * RPP == DK, "row split");
};

// Sum of x over the lanes of the wave that share lane % LPR (LPR = 4 or 8: the
// lanes holding the same value columns), in every such lane, without LDS: a DPP
// row rotation by 8 (and by 4) pairs the lanes inside a 16-lane row, and the
// gfx950 permlane16 / permlane32 swaps bring the other row / half-wave next to
// it (swapping a register with itself leaves x and its partner's x in the two
// results, so their sum is x + x[lane ^ 16] or x + x[lane ^ 32]).  Every lane
// adds the same pairs, so all of them hold bitwise the same sum.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPR == 4 || LPR == 8, "lane groups of 4 or 8");
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  if constexpr (LPR == 4)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
  const unsigned xb = __float_as_uint(x);
  const auto h = __builtin_amdgcn_permlane16_swap(xb, xb, false, false);
  x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  const unsigned yb = __float_as_uint(x);
  const auto w = __builtin_amdgcn_permlane32_swap(yb, yb, false, false);
  return __uint_as_float(w[0]) + __uint_as_float(w[1]);
}

// q.k over the rows a lane holds (x, y), finished across the lane group
template <int NP, int LPR>
__device__ __forceinline__ float dot_rows(const float (&x)[NP], const float (&y)[NP]) {
  float d = 0.f;
#pragma unroll
  for (int i = 0; i < NP; ++i) d = __builtin_fmaf(x[i], y[i], d);
  return group_sum<LPR>(d);
}

// One token on the state rows a lane holds (kr = k, ak = alpha k, aq = alpha q,
// al = alpha at those rows; qk = q.k; vv = v at the lane's 4 columns).  The
// decayed state's sums come from the stored state and the alpha-scaled vectors,
// (Diag(alpha) S)^T k = S^T (alpha k), so the decay folds into the update:
//     u = beta (v - S^T (alpha k)),  o = S^T (alpha q) + (q.k) u,
//     S' = Diag(alpha) S + k u^T   (a multiply and an fma per element)
// s is replaced by S'; returns o for the lane's 4 columns.  Explicit fmas only,
// so every kernel that calls this rounds identically.
template <int NP, int LPR>
__device__ __forceinline__ floatx4 token_step(floatx4 (&s)[NP], const float (&kr)[NP],
                                              const float (&ak)[NP], const float (&aq)[NP],
                                              const float (&al)[NP], float qk, float b,
                                              floatx4 vv) {
  floatx4 old = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NP; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      old[j] = __builtin_fmaf(s[i][j], ak[i], old[j]);  // S^T (alpha k), this lane's rows
      p[j] = __builtin_fmaf(s[i][j], aq[i], p[j]);      // S^T (alpha q)
    }
  // finish the sums over the lanes that share these columns
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    old[j] = group_sum<LPR>(old[j]);
    p[j] = group_sum<LPR>(p[j]);
  }
  floatx4 u, o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u[j] = b * (vv[j] - old[j]);
    o[j] = __builtin_fmaf(qk, u[j], p[j]);
  }
  // decay in place, then the rank-one write accumulated into the same register
#pragma unroll
  for (int i = 0; i < NP; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) s[i][j] = __builtin_fmaf(kr[i], u[j], s[i][j] * al[i]);
  return o;
}

// alpha of key channels c..c+3 of one token row, correctly rounded library
// exponentials as in the one-token step (same values bit for bit)
template <int KIND>
__device__ __forceinline__ floatx4 alpha4_exact(const Gate& G, size_t row, int Dk, int c,
                                                float sc) {
  floatx4 x = gate_load4<KIND>(G, true, row, Dk, c);
  if constexpr (KIND == GATE_LOG) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = expf(x[e]);
  } else if constexpr (KIND == GATE_BOUNDED) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = gate_bounded(x[e], sc, G.g_min);
  }
  return x;
}

// Per-token LDS record, fp32: k, alpha k, alpha and (with outputs) q, alpha q,
// each permuted to [ro][i] (row ro + RPP i at ro * NP + i); v; beta; q.k.
template <int DK, int DV, bool VERIFY>
struct Rec {
  static constexpr int K = 0;
  static constexpr int AK = DK;
  static constexpr int AL = 2 * DK;
  static constexpr int Q = 3 * DK;                // verify only
  static constexpr int AQ = 4 * DK;               // verify only
  static constexpr int V = VERIFY ? 5 * DK : 3 * DK;
  static constexpr int Bt = V + DV;
  static constexpr int QK = Bt + 1;               // verify only
  static constexpr int stride = Bt + 4;           // floats, keeps 16-byte alignment
};

template <int NP>
__device__ __forceinline__ void ld_rows(const float* p, float (&x)[NP]) {
#pragma unroll
  for (int i = 0; i < NP; i += 4) {
    const floatx4 t = *reinterpret_cast<const floatx4*>(p + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[i + e] = t[e];
  }
}

// Prologue of token t's row of one tensor for the fused layer, from the raw
// rows staged in LDS (xr: [3 + n][2 Dk + Dv], the conv state's three rows and
// then the tokens') and the head's taps of the tensor staged in LDS ([D][4]),
// rounded to the token dtype as the standalone prologue stores it, into the
// token's record: k (with alpha k), q (with alpha q) or v.
template <typename TIn, int CPL, bool NORM, int NP, int RPP>
__device__ __forceinline__ void layer_row(const float* xr, const float* taps, float eps, int t,
                                          int off, int SW, int lane, float* dst, float* adst,
                                          const float* al) {
  float hist[3][CPL], xc[CPL], w[CPL][4], y[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int ch = CPL * lane + c;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[c][j] = taps[ch * 4 + j];
#pragma unroll
    for (int j = 0; j < 3; ++j) hist[j][c] = xr[(t + j) * SW + off + ch];
    xc[c] = xr[(t + 3) * SW + off + ch];
  }
  prologue_row<CPL, NORM>(hist, xc, w, eps, y);
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int ch = CPL * lane + c;
    const float yr = (float)(TIn)y[c];
    if (adst) {  // key-side vectors: permuted record rows, alpha-scaled copy
      const int pos = (ch % RPP) * NP + ch / RPP;
      dst[pos] = yr;
      adst[pos] = al[pos] * yr;
    } else {
      dst[ch] = yr;
    }
  }
}

// The fused layer's prologue rows of tokens t0 .. t0 + cnt - 1 (cnt <= 4) of
// one tensor, straight from memory.  pro_load fetches the head's taps and the
// cnt + 3 raw rows of the lane's channels (raw row r < 3 is conv-state row r,
// fp32, row stride csr; row r >= 3 is token r - 3 of x, row stride xr);
// pro_rows slides the conv window over them -- the arithmetic of layer_row --
// and writes each row, rounded to the token dtype as the standalone prologue
// stores it, to dst + t * ldd.  Split so that a wave issues the loads of all
// its blocks ahead of its other loads.  The loads take no branches (a load
// under a branch is waited for inside it): rows outside the tokens re-read a
// token row in range and are not used, and where the block may be the first
// (MAYBE_FIRST) the conv-state rows are read too and chosen when t0 = 0.
template <int CPL>
struct ProBlock {
  float w[CPL][4], raw[7][CPL];
};
template <typename TIn, int CPL, bool MAYBE_FIRST, int CPLM>
__device__ __forceinline__ void pro_load(ProBlock<CPLM>& b, const float* cs, const TIn* x,
                                         size_t xr, int csr, const float* taps, int t0, int n,
                                         int lane) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const floatx4 t4 = *reinterpret_cast<const floatx4*>(taps + (CPL * lane + c) * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) b.w[c][j] = t4[j];
  }
#pragma unroll
  for (int r = 0; r < 7; ++r) {
    const int tk = max(0, min(t0 + r - 3, n - 1));
    float x4[CPL];
    row_load<TIn, CPL>(x + (size_t)tk * xr, lane, x4);
    if (MAYBE_FIRST && r < 3) {
      float c4[CPL];
      row_load<float, CPL>(cs + (size_t)r * csr, lane, c4);
#pragma unroll
      for (int c = 0; c < CPL; ++c) x4[c] = t0 == 0 ? c4[c] : x4[c];
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) b.raw[r][c] = x4[c];
  }
}
template <typename TIn, int CPL, bool NORM, int CPLM>
__device__ __forceinline__ void pro_rows(const ProBlock<CPLM>& b, float eps, int t0, int cnt,
                                         int lane, float* dst, int ldd) {
  float w[CPL][4];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) w[c][j] = b.w[c][j];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < cnt) {
      float hist[3][CPL], xc[CPL], y[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
#pragma unroll
        for (int j = 0; j < 3; ++j) hist[j][c] = b.raw[i + j][c];
        xc[c] = b.raw[i + 3][c];
      }
      prologue_row<CPL, NORM>(hist, xc, w, eps, y);
#pragma unroll
      for (int c = 0; c < CPL; ++c) dst[(t0 + i) * ldd + CPL * lane + c] = (float)(TIn)y[c];
    }
  }
}

// One kernel for the three decode calls, by MODE:
//   DECODE_STEP    one token (N = 1): output written, state written in place
//   DECODE_VERIFY  tokens 0..N-1: outputs written, state untouched
//   DECODE_COMMIT  tokens 0..n_accept[b]-1 (clamped to [0, N]) replayed into the
//                  state, written in place; no outputs
// All of them stage the tokens' inputs in LDS (one coalesced pass, alpha and the
// alpha-scaled vectors formed once) and step the state held in registers with
// token_step, so the three calls agree bitwise.
// LAYER: the whole recurrent layer step of "Kimi K3模型架构详解" section 9.2 in one
// kernel -- q, k, v come from the projections' outputs through the prologue
// (the conv state read, and advanced by step and commit), and the outputs leave
// through the epilogue (RMSNorm and gate) as y; with the standalone prologue and
// epilogue around the plain call the results are bitwise the same.
template <int DK, int DV, typename TIn, typename TOut, int KIND, int MODE, bool LAYER>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(MODE == DECODE_VERIFY ? 4 : 1))) void decode_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    Gate gate, const float* __restrict__ beta, float* __restrict__ state, TOut* __restrict__ o,
    const int32_t* __restrict__ n_accept, int N, int H, LayerIO io) {
  constexpr bool VERIFY = MODE != DECODE_COMMIT;  // outputs (and q) needed
  constexpr bool WRITE = MODE != DECODE_VERIFY;   // state written back
  using G = Geo<DK, DV>;
  using R = Rec<DK, DV, VERIFY>;
  constexpr int NP = G::NP, LPR = G::LPR, RPP = G::RPP;
  extern __shared__ __align__(16) float rec[];

  const int tile = blockIdx.x;  // (session, head) flattened
  const int sb = tile / H, h = tile - sb * H;
  int n = N;
  if constexpr (MODE == DECODE_COMMIT) {
    const int na = n_accept[sb];
    n = na < 0 ? 0 : (na > N ? N : na);
    if (n == 0) return;  // nothing accepted: the state stays as it is
  }
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int cg = lane % LPR;
  const int ro = lane / LPR;
  const int col = w * G::CW + 4 * cg;

  float* S = state + (size_t)tile * DK * DV;
  floatx4 s[NP];
  auto load_state = [&]() {
#pragma unroll
    for (int i = 0; i < NP; ++i)
      s[i] = MODE == DECODE_VERIFY  // (see the chunk kernel's state loads)
                 ? __builtin_nontemporal_load(
                       reinterpret_cast<const floatx4*>(S + (size_t)(ro + RPP * i) * DV + col))
                 : *reinterpret_cast<const floatx4*>(S + (size_t)(ro + RPP * i) * DV + col);
  };
  // The (smaller) staging loads are issued before the state's, so that the
  // staging -- and the layer's prologue rows -- which wait for them, and with
  // them for every load issued earlier, run while the state is still arriving.
  constexpr int SW = 2 * DK + DV;                  // conv-state row: q | k | v
  // LAYER: the raw rows [3 + n][SW] (conv state, then the tokens' projections),
  // the gate logits [n][Dv] and the head's conv taps [SW][4]; the raw rows'
  // space later holds o [n][Dv]
  float* xr = rec + R::stride * N;
  float* gs = xr + (N + 3) * SW;
  float* tp = gs + N * DV;
  constexpr int CPLV = DV / 64;
  float wn[CPLV];  // RMSNorm weight of the lane's channels (layer epilogue)
  const float sc = KIND == GATE_BOUNDED ? expf(gate.a_log[h]) : 1.f;
  if constexpr (LAYER) {
    // Every staging load is issued first, at clamped indices and without
    // branches (a load under a branch or inside a loop is waited for there,
    // which would put each group of them on the workgroup's chain), then the
    // state's, then the stores.  Unrolled for up to MAXN tokens, the most this
    // mode takes before the chunk form; loops take any beyond.
    constexpr int MAXN = MODE == DECODE_STEP ? 1 : MODE == DECODE_VERIFY ? 5 : 11;
    constexpr int TPT = (SW + 255) / 256, CRT = (3 * SW / 4 + 255) / 256;
    constexpr int XRT = (MAXN * SW / 4 + 255) / 256, ALT = (MAXN * DK / 4 + 255) / 256;
    constexpr int GST = VERIFY ? (MAXN * DV / 4 + 255) / 256 : 1;
    const float* cs = io.conv_state + ((size_t)sb * 3 * H + h) * SW;
    const size_t row0 = (size_t)sb * N * H + h;  // (token 0, head h)
    // the per-tensor pointers held as scalars (behind empty asm), so that the
    // per-lane choice among them stays a select and does not become a load
    // of the pointer from the argument block, waited for before the taps'; the
    // asm hides their address space, so their loads go through gload
    const float *w0 = io.conv.w[0], *w1 = io.conv.w[1], *w2 = io.conv.w[2];
    const TIn *pq = (const TIn*)io.xq, *pk = (const TIn*)io.xk, *pv = (const TIn*)io.xv;
    __asm__ volatile("" : "+s"(w0), "+s"(w1), "+s"(w2));
    __asm__ volatile("" : "+s"(pq), "+s"(pk), "+s"(pv));
    auto tap_src = [&](int idx) {
      const int ten = idx < DK ? 0 : idx < 2 * DK ? 1 : 2;
      const int ch = idx - (ten == 0 ? 0 : ten == 1 ? DK : 2 * DK), D = ten == 2 ? DV : DK;
      const float* wt = ten == 0 ? w0 : ten == 1 ? w1 : w2;
      return wt + ((size_t)h * D + ch) * 4;
    };
    auto x_src = [&](int idx) {  // raw row item idx of the tokens: 4 values
      const int t = idx / (SW / 4), c = 4 * (idx % (SW / 4));
      const size_t row = row0 + (size_t)t * H;
      const TIn* xp = c < DK ? pq + row * DK + c
                             : c < 2 * DK ? pk + row * DK + c - DK : pv + row * DV + c - 2 * DK;
      return Raw4<TIn>::gld(xp);
    };
    // (token-dtype values stay as loaded until their stores, after the state's loads)
    floatx4 tv[TPT], cv[CRT], av[ALT];
    typename Raw4<TIn>::T xv[XRT], gv[GST];
#pragma unroll
    for (int i = 0; i < TPT; ++i) tv[i] = gload<floatx4>(tap_src(min(tid + 256 * i, SW - 1)));
    if constexpr (VERIFY) {
#pragma unroll
      for (int c = 0; c < CPLV; ++c) wn[c] = io.out.w[CPLV * lane + c];
    }
#pragma unroll
    for (int i = 0; i < CRT; ++i) {
      const int idx = min(tid + 256 * i, 3 * (SW / 4) - 1);
      cv[i] = *reinterpret_cast<const floatx4*>(cs + (size_t)(idx / (SW / 4)) * H * SW +
                                                4 * (idx % (SW / 4)));
    }
#pragma unroll
    for (int i = 0; i < XRT; ++i) xv[i] = x_src(min(tid + 256 * i, n * (SW / 4) - 1));
    if constexpr (VERIFY) {
#pragma unroll
      for (int i = 0; i < GST; ++i) {
        const int idx = min(tid + 256 * i, n * (DV / 4) - 1);
        gv[i] = Raw4<TIn>::ld((const TIn*)io.out.g + (row0 + (size_t)(idx / (DV / 4)) * H) * DV +
                              4 * (idx % (DV / 4)));
      }
    }
#pragma unroll
    for (int i = 0; i < ALT; ++i) {
      const int idx = min(tid + 256 * i, n * (DK / 4) - 1);
      av[i] = gate_load4<KIND>(gate, true, row0 + (size_t)(idx / (DK / 4)) * H, DK,
                               4 * (idx % (DK / 4)));
    }
    const float btv = beta[row0 + (size_t)min(tid, n - 1) * H];
    // (the state's loads stay after the staging loads, and the stores after them)
    __builtin_amdgcn_sched_barrier(0);
    load_state();
    __builtin_amdgcn_sched_barrier(0);
    // the stores (alpha formed as alpha4_exact forms it).  The first round
    // stores at the same clamped indices -- the threads past an item count
    // store the last item again, the same values to the same place -- so that
    // its stores sit under no branch the compiler would move their loads
    // into; later rounds (rarely partly used) keep the guard, as repeated
    // stores to one address from a whole wave serialize
    auto put_alpha = [&](int idx, floatx4 a4) {
      const int t = idx / (DK / 4), c = 4 * (idx % (DK / 4));
      if constexpr (KIND == GATE_LOG) {
#pragma unroll
        for (int e = 0; e < 4; ++e) a4[e] = expf(a4[e]);
      } else if constexpr (KIND == GATE_BOUNDED) {
#pragma unroll
        for (int e = 0; e < 4; ++e) a4[e] = gate_bounded(a4[e], sc, gate.g_min);
      }
      float* rt = rec + t * R::stride;
#pragma unroll
      for (int e = 0; e < 4; ++e) rt[R::AL + ((c + e) % RPP) * NP + (c + e) / RPP] = a4[e];
    };
#pragma unroll
    for (int i = 0; i < TPT; ++i)
      if (i == 0 || tid + 256 * i < SW)
        *reinterpret_cast<floatx4*>(tp + 4 * min(tid + 256 * i, SW - 1)) = tv[i];
#pragma unroll
    for (int i = 0; i < CRT; ++i) {
      const int idx = min(tid + 256 * i, 3 * (SW / 4) - 1);
      if (i == 0 || tid + 256 * i < 3 * (SW / 4))
        *reinterpret_cast<floatx4*>(xr + (idx / (SW / 4)) * SW + 4 * (idx % (SW / 4))) = cv[i];
    }
#pragma unroll
    for (int i = 0; i < XRT; ++i) {
      const int idx = min(tid + 256 * i, n * (SW / 4) - 1);
      if (i == 0 || tid + 256 * i < n * (SW / 4))
        *reinterpret_cast<floatx4*>(xr + (3 + idx / (SW / 4)) * SW + 4 * (idx % (SW / 4))) =
            Raw4<TIn>::cvt(xv[i]);
    }
    for (int idx = tid + 256 * XRT; idx < n * (SW / 4); idx += 256)
      *reinterpret_cast<floatx4*>(xr + (3 + idx / (SW / 4)) * SW + 4 * (idx % (SW / 4))) =
          Raw4<TIn>::cvt(x_src(idx));
    if constexpr (VERIFY) {
#pragma unroll
      for (int i = 0; i < GST; ++i) {
        const int idx = min(tid + 256 * i, n * (DV / 4) - 1);
        if (i == 0 || tid + 256 * i < n * (DV / 4))
          *reinterpret_cast<floatx4*>(gs + (idx / (DV / 4)) * DV + 4 * (idx % (DV / 4))) =
              Raw4<TIn>::cvt(gv[i]);
      }
      for (int idx = tid + 256 * GST; idx < n * (DV / 4); idx += 256)
        *reinterpret_cast<floatx4*>(gs + (idx / (DV / 4)) * DV + 4 * (idx % (DV / 4))) =
            ld4<TIn>((const TIn*)io.out.g + (row0 + (size_t)(idx / (DV / 4)) * H) * DV +
                     4 * (idx % (DV / 4)));
    }
#pragma unroll
    for (int i = 0; i < ALT; ++i)
      if (i == 0 || tid + 256 * i < n * (DK / 4))
        put_alpha(min(tid + 256 * i, n * (DK / 4) - 1), av[i]);
    for (int idx = tid + 256 * ALT; idx < n * (DK / 4); idx += 256)
      put_alpha(idx, gate_load4<KIND>(gate, true, row0 + (size_t)(idx / (DK / 4)) * H, DK,
                                      4 * (idx % (DK / 4))));
    if (tid < n) rec[tid * R::stride + R::Bt] = btv;
  } else {
    // stage the n tokens' inputs (alpha and the alpha-scaled vectors formed
    // once): as above, every load first, then the state's, then the stores
    constexpr int MAXN = MODE == DECODE_STEP ? 1 : MODE == DECODE_VERIFY ? 5 : 11;
    constexpr int KT = (MAXN * DK / 4 + 255) / 256, VT = (MAXN * DV / 4 + 255) / 256;
    floatx4 aa[KT];
    typename Raw4<TIn>::T ka[KT], qa[KT], va[VT];  // as loaded (widened at their stores)
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      const int idx = min(tid + 256 * i, n * (DK / 4) - 1);
      const size_t row = ((size_t)sb * N + idx / (DK / 4)) * H + h;
      const int c = 4 * (idx % (DK / 4));
      ka[i] = Raw4<TIn>::ld(k + row * DK + c);
      qa[i] = ka[i];
      if constexpr (VERIFY) qa[i] = Raw4<TIn>::ld(q + row * DK + c);
      aa[i] = gate_load4<KIND>(gate, true, row, DK, c);
    }
#pragma unroll
    for (int i = 0; i < VT; ++i) {
      const int idx = min(tid + 256 * i, n * (DV / 4) - 1);
      va[i] = Raw4<TIn>::ld(v + (((size_t)sb * N + idx / (DV / 4)) * H + h) * DV + 4 * (idx % (DV / 4)));
    }
    const float btv = beta[((size_t)sb * N + min(tid, n - 1)) * H + h];
    // (the state's loads stay after the staging loads, and the stores after them)
    __builtin_amdgcn_sched_barrier(0);
    load_state();
    __builtin_amdgcn_sched_barrier(0);
    auto put_k = [&](int idx, floatx4 a4, const floatx4& k4, const floatx4& q4) {
      const int t = idx / (DK / 4), c = 4 * (idx % (DK / 4));
      if constexpr (KIND == GATE_LOG) {
#pragma unroll
        for (int e = 0; e < 4; ++e) a4[e] = expf(a4[e]);
      } else if constexpr (KIND == GATE_BOUNDED) {
#pragma unroll
        for (int e = 0; e < 4; ++e) a4[e] = gate_bounded(a4[e], sc, gate.g_min);
      }
      float* rt = rec + t * R::stride;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = ((c + e) % RPP) * NP + (c + e) / RPP;
        rt[R::K + pos] = k4[e];
        rt[R::AK + pos] = a4[e] * k4[e];
        rt[R::AL + pos] = a4[e];
        if constexpr (VERIFY) {
          rt[R::Q + pos] = q4[e];
          rt[R::AQ + pos] = a4[e] * q4[e];
        }
      }
    };
#pragma unroll
    for (int i = 0; i < KT; ++i)  // (the first round clamped, as above)
      if (i == 0 || tid + 256 * i < n * (DK / 4))
        put_k(min(tid + 256 * i, n * (DK / 4) - 1), aa[i], Raw4<TIn>::cvt(ka[i]),
              Raw4<TIn>::cvt(qa[i]));
    for (int idx = tid + 256 * KT; idx < n * (DK / 4); idx += 256) {
      const size_t row = ((size_t)sb * N + idx / (DK / 4)) * H + h;
      const int c = 4 * (idx % (DK / 4));
      floatx4 q4 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (VERIFY) q4 = ld4<TIn>(q + row * DK + c);
      put_k(idx, gate_load4<KIND>(gate, true, row, DK, c), ld4<TIn>(k + row * DK + c), q4);
    }
#pragma unroll
    for (int i = 0; i < VT; ++i) {
      const int idx = min(tid + 256 * i, n * (DV / 4) - 1);
      if (i == 0 || tid + 256 * i < n * (DV / 4))
        *reinterpret_cast<floatx4*>(rec + (idx / (DV / 4)) * R::stride + R::V +
                                    4 * (idx % (DV / 4))) = Raw4<TIn>::cvt(va[i]);
    }
    for (int idx = tid + 256 * VT; idx < n * (DV / 4); idx += 256) {
      const int t = idx / (DV / 4), c = 4 * (idx % (DV / 4));
      const size_t row = ((size_t)sb * N + t) * H + h;
      *reinterpret_cast<floatx4*>(rec + t * R::stride + R::V + c) = ld4<TIn>(v + row * DV + c);
    }
    if (tid < n) rec[tid * R::stride + R::Bt] = btv;
  }
  __syncthreads();
  if constexpr (LAYER) {
    // prologue rows into the records, one wave per (token, tensor); commit
    // needs no q
    for (int r = w; r < 3 * n; r += 4) {
      const int t = r / 3, ten = r - 3 * (r / 3);
      float* rt = rec + t * R::stride;
      if (ten == 0) {
        if constexpr (VERIFY)
          layer_row<TIn, DK / 64, true, NP, RPP>(xr, tp, io.conv.eps, t, 0, SW, lane, rt + R::Q,
                                                 rt + R::AQ, rt + R::AL);
      } else if (ten == 1) {
        layer_row<TIn, DK / 64, true, NP, RPP>(xr, tp + 4 * DK, io.conv.eps, t, DK, SW, lane,
                                               rt + R::K, rt + R::AK, rt + R::AL);
      } else {
        layer_row<TIn, DV / 64, false, NP, RPP>(xr, tp + 8 * DK, io.conv.eps, t, 2 * DK, SW,
                                                lane, rt + R::V, nullptr, nullptr);
      }
    }
    if constexpr (MODE != DECODE_VERIFY) {
      // the conv state advances past the n tokens: its new rows are the last
      // three of the raw rows
      float* cs = io.conv_state + ((size_t)sb * 3 * H + h) * SW;
      for (int idx = tid; idx < 3 * (SW / 4); idx += 256) {
        const int j = idx / (SW / 4), c = 4 * (idx % (SW / 4));
        *reinterpret_cast<floatx4*>(cs + (size_t)j * H * SW + c) =
            *reinterpret_cast<const floatx4*>(xr + (n + j) * SW + c);
      }
    }
    __syncthreads();
  }
  if constexpr (MODE == DECODE_VERIFY) {
    // q.k of each token (the loop below computes it in place for a single step)
    for (int t = w; t < n; t += 4) {
      float kr[NP], qr[NP];
      ld_rows<NP>(rec + t * R::stride + R::K + ro * NP, kr);
      ld_rows<NP>(rec + t * R::stride + R::Q + ro * NP, qr);
      const float qk = dot_rows<NP, LPR>(kr, qr);
      if (lane == 0) rec[t * R::stride + R::QK] = qk;
    }
    __syncthreads();
  }

  for (int t = 0; t < n; ++t) {
    const float* rt = rec + t * R::stride;
    float kr[NP], ak[NP], aq[NP], al[NP];
    ld_rows<NP>(rt + R::K + ro * NP, kr);
    ld_rows<NP>(rt + R::AK + ro * NP, ak);
    ld_rows<NP>(rt + R::AL + ro * NP, al);
    float qk = 0.f;
    if constexpr (MODE == DECODE_VERIFY) {
      ld_rows<NP>(rt + R::AQ + ro * NP, aq);
      qk = rt[R::QK];
    } else if constexpr (MODE == DECODE_STEP) {
      float qr[NP];
      ld_rows<NP>(rt + R::AQ + ro * NP, aq);
      ld_rows<NP>(rt + R::Q + ro * NP, qr);
      qk = dot_rows<NP, LPR>(kr, qr);
    } else {
#pragma unroll
      for (int i = 0; i < NP; ++i) aq[i] = 0.f;
    }
    const floatx4 vv = *reinterpret_cast<const floatx4*>(rt + R::V + col);
    const floatx4 ov = token_step<NP, LPR>(s, kr, ak, aq, al, qk, rt[R::Bt], vv);
    if constexpr (VERIFY) {
      if (ro == 0) {
        if constexpr (LAYER) {
          // to the epilogue, through LDS (the raw rows are consumed)
          *reinterpret_cast<floatx4*>(xr + t * DV + col) = ov;
        } else {
          TOut* ot = o + (((size_t)sb * N + t) * H + h) * DV + col;
#pragma unroll
          for (int j = 0; j < 4; ++j) ot[j] = (TOut)ov[j];
        }
      }
    }
  }
  if constexpr (LAYER && VERIFY) {
    // epilogue rows, one wave per token: y = RMSNorm(o) w Sigmoid(g)
    __syncthreads();
    constexpr int CPL = CPLV;
    for (int t = w; t < n; t += 4) {
      float ov[CPL], gv[CPL], y[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        ov[c] = xr[t * DV + CPL * lane + c];
        gv[c] = gs[t * DV + CPL * lane + c];
      }
      const size_t row = (((size_t)sb * N + t) * H + h) * DV;
      epilogue_row<CPL>(ov, gv, wn, io.out.eps, y);
      row_store<TOut, CPL>(o + row, lane, y);
    }
  }
  if constexpr (WRITE) {
    // streaming (non-temporal) stores: the state is written once and not re-read
    // by this launch; on gfx950 this write path sustains close to HBM peak where
    // ordinary stores of the same pattern stall on the cache write-back path
#pragma unroll
    for (int i = 0; i < NP; ++i)
      __builtin_nontemporal_store(s[i],
                                  reinterpret_cast<floatx4*>(S + (size_t)(ro + RPP * i) * DV + col));
  }
}

// The prefill as the token recurrence, for fp32 q, k, v where the chunked
// fp32 kernel's LDS plan does not fit (Dk = 128): one workgroup per
// (sequence, head) holds the state tile in registers, as the decode kernel
// does, and steps the sequence's tokens in blocks of NBLK staged in LDS
// (records as for verify), writing o per token and the state once at the end
// ("Kimi Delta Attention 完全拆解", section "一次 KDA 前向究竟发生了什么": the
// recurrent form, which the chunk form equals up to rounding).  Empty
// sequences hand their state through.
constexpr int NBLK = 16;
template <int DK, int DV, typename TIn, typename TOut, int KIND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void recurrent_prefill_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v, Gate gate,
    const float* __restrict__ beta, const float* s_init, float* s_final, TOut* __restrict__ o,
    const int32_t* __restrict__ cu_seqlens, int n_seq, int T, int H) {
  using G = Geo<DK, DV>;
  using R = Rec<DK, DV, true>;
  constexpr int NP = G::NP, LPR = G::LPR, RPP = G::RPP;
  extern __shared__ __align__(16) float rec[];
  const int tile = blockIdx.x;  // (sequence, head)
  const int seq = tile / H, h = tile - seq * H;
  long long start, len;
  if (cu_seqlens) {
    start = cu_seqlens[seq];
    len = (long long)cu_seqlens[seq + 1] - start;
  } else {
    start = (long long)seq * T;
    len = T;
  }
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int cg = lane % LPR, ro = lane / LPR, col = w * G::CW + 4 * cg;
  floatx4 s[NP];
  {
    const float* S = s_init ? s_init + (size_t)tile * DK * DV : nullptr;
#pragma unroll
    for (int i = 0; i < NP; ++i)
      s[i] = S ? *reinterpret_cast<const floatx4*>(S + (size_t)(ro + RPP * i) * DV + col)
               : floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const float sc = KIND == GATE_BOUNDED ? expf(gate.a_log[h]) : 1.f;
  for (long long t0 = 0; t0 < len; t0 += NBLK) {
    const int n = (int)(len - t0 < NBLK ? len - t0 : NBLK);
    __syncthreads();  // the block before is done with the records
    for (int idx = tid; idx < n * (DK / 4); idx += 256) {
      const int t = idx / (DK / 4), c = 4 * (idx % (DK / 4));
      const size_t row = (size_t)(start + t0 + t) * H + h;
      const floatx4 a4 = alpha4_exact<KIND>(gate, row, DK, c, sc);
      const floatx4 k4 = ld4<TIn>(k + row * DK + c);
      const floatx4 q4 = ld4<TIn>(q + row * DK + c);
      float* rt = rec + t * R::stride;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int pos = ((c + e) % RPP) * NP + (c + e) / RPP;
        rt[R::K + pos] = k4[e];
        rt[R::AK + pos] = a4[e] * k4[e];
        rt[R::AL + pos] = a4[e];
        rt[R::Q + pos] = q4[e];
        rt[R::AQ + pos] = a4[e] * q4[e];
      }
    }
    for (int idx = tid; idx < n * (DV / 4); idx += 256) {
      const int t = idx / (DV / 4), c = 4 * (idx % (DV / 4));
      const size_t row = (size_t)(start + t0 + t) * H + h;
      *reinterpret_cast<floatx4*>(rec + t * R::stride + R::V + c) = ld4<TIn>(v + row * DV + c);
    }
    if (tid < n) rec[tid * R::stride + R::Bt] = beta[(size_t)(start + t0 + tid) * H + h];
    __syncthreads();
    for (int t = w; t < n; t += 4) {  // q.k of each token
      float kr[NP], qr[NP];
      ld_rows<NP>(rec + t * R::stride + R::K + ro * NP, kr);
      ld_rows<NP>(rec + t * R::stride + R::Q + ro * NP, qr);
      const float qk = dot_rows<NP, LPR>(kr, qr);
      if (lane == 0) rec[t * R::stride + R::QK] = qk;
    }
    __syncthreads();
    for (int t = 0; t < n; ++t) {
      const float* rt = rec + t * R::stride;
      float kr[NP], ak[NP], aq[NP], al[NP];
      ld_rows<NP>(rt + R::K + ro * NP, kr);
      ld_rows<NP>(rt + R::AK + ro * NP, ak);
      ld_rows<NP>(rt + R::AL + ro * NP, al);
      ld_rows<NP>(rt + R::AQ + ro * NP, aq);
      const floatx4 vv = *reinterpret_cast<const floatx4*>(rt + R::V + col);
      const floatx4 ov = token_step<NP, LPR>(s, kr, ak, aq, al, rt[R::QK], rt[R::Bt], vv);
      if (ro == 0) {
        TOut* ot = o + ((size_t)(start + t0 + t) * H + h) * DV + col;
#pragma unroll
        for (int j = 0; j < 4; ++j) ot[j] = (TOut)ov[j];
      }
    }
  }
  if (s_final) {
    float* S = s_final + (size_t)tile * DK * DV;
#pragma unroll
    for (int i = 0; i < NP; ++i)
      __builtin_nontemporal_store(s[i], reinterpret_cast<floatx4*>(S + (size_t)(ro + RPP * i) * DV + col));
  }
}

// ---- Speculative verify / commit as one chunk -------------------------------
// The n <= 16 draft tokens of a session are one chunk of the chunk form ("Kimi
// Delta Attention 完全拆解", section "chunk 内并行、chunk 间递推"; the prefill's
// algebra with the chunk starting at the first draft), evaluated in fp32 on the
// fp32 matrix cores (v_mfma_f32_16x16x4_f32).  With Gamma_t = alpha_1 ... alpha_t
// per key channel (from the first draft token) and S the state read:
//   A_tj   = beta_t sum_c k_tc k_jc Gamma_tc / Gamma_jc  (j < t),  T = (I + A)^{-1}
//   P      = T Diag(beta) (V - (Gamma*K) S)       (the corrected writes u_t)
//   verify: o = (Gamma*Q) S + Mqk P,   Mqk_tj = sum_c q_tc k_jc Gamma_tc / Gamma_jc  (j <= t)
//   commit: S' = Diag(Gamma_n) S + Ktil^T P,   Ktil_j = (Gamma_n / Gamma_j) k_j
// The state tile is read once (and written once by commit) and the work on it is
// two products (three for verify's o) on the matrix cores, where the token loop
// spends four VALU operations per state element and token.  The results agree
// with the token loop up to fp32 rounding, not bitwise.
//
// Mapping: one workgroup (4 waves) per (session, head).  Wave w owns the value
// columns [w CW, (w + 1) CW); lane (g = l / 16, tr = l % 16) holds, for each
// k-step s of 4 key channels, S[4s + g][w CW + E tr + e] (e < E = CW / 16) -- the
// B operand of the fp32 MFMA with the tile's columns taken E apart -- loaded as
// E consecutive floats, so a row segment of the wave's columns is one
// contiguous 64..128-byte access.  The token-side operands (Gamma*K, k / Gamma,
// Gamma*Q) sit in LDS as [token][channel]; A and Mqk are summed over the key
// channels by the four waves in parts; T is formed by every wave for itself
// (N^16 = 0 for the strictly lower 16 x 16 A: (I + N)^{-1} = (I - N)(I + N^2)
// (I + N^4)(I + N^8)).  Ktil^T for commit is stored with its rows permuted so
// that the product's accumulator rows are the state rows each lane holds.
// The decay ratios are factored as (Gamma_t k_t) . (k_j / Gamma_j) while every
// channel's Gamma_n stays at or above kTileMin; otherwise A and Mqk come from
// running products of the decays between the two tokens (exact, slower).
template <int DK, int DV, bool COMMIT>
struct SpecGeo {
  static constexpr int CW = DV / 4;   // value columns per wave
  static constexpr int E = CW / 16;   // columns per lane (1 or 2)
  static constexpr int KS = DK / 4;   // k-steps over the key channels
  static constexpr int KW = KS / 4;   // k-steps per wave of the A / Mqk sums
  static constexpr int ld = DK + 4;   // [16][DK] token arrays (conflict-free reads)
  static constexpr int ldT = 20;      // the 16 x 16 scratch
  static constexpr int ldKt = 16;     // commit's Ktil^T [DK][16]
  static constexpr int oK = 0;              // k, then Gamma*k
  static constexpr int oA = oK + 16 * ld;   // alpha, then k / Gamma
  static constexpr int oQ = oA + 16 * ld;   // verify: q, then Gamma*q; commit: Ktil^T
  static constexpr int szQ = COMMIT ? DK * ldKt : 16 * ld;
  static constexpr int oB = oQ + szQ;       // beta [16]
  static constexpr int oG = oB + 16;        // commit: Gamma_n [DK]
  static constexpr int oF = oG + DK;        // exact-path flags, one per scanning wave
  static constexpr int oP = oF + 4;         // partial A / Mqk sums [4][2][256]
  static constexpr int oW = oP + 4 * 2 * 256;  // per-wave 16 x 16 scratch [4][16 * ldT]
  static constexpr int total = oW + 4 * 16 * ldT;
  static_assert(oP % 4 == 0 && oW % 4 == 0 && oQ % 4 == 0, "16-byte LDS rows");
};

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// M X for a 16 x 16 M whose row this lane read as a = M[tr][4g .. 4g + 3] and
// X in the accumulator layout (lane holds X[4g + i][tr]): MFMA i takes k-slot g
// as k = 4g + i.  The result is in the accumulator layout.
__device__ __forceinline__ floatx4 mm16(const floatx4& a, const floatx4& x) {
  floatx4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) y = mfma4(a[i], x[i], y);
  return y;
}
__device__ __forceinline__ void lds_sync() { __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int E>
struct SpecVec;
// ld: plain loads; ldnt: non-temporal loads, for a state that is only read
// (verify: 3-9 % faster on MI355X; where the state is written back as well,
// non-temporal loads made the step and the token-loop commit 7-24 % slower)
template <>
struct SpecVec<1> {
  typedef float F;
  static __device__ __forceinline__ void ld(const float* p, float (&x)[1]) { x[0] = *p; }
  static __device__ __forceinline__ void ldnt(const float* p, float (&x)[1]) {
    x[0] = __builtin_nontemporal_load(p);
  }
  static __device__ __forceinline__ void st(float* p, const float (&x)[1]) {
    __builtin_nontemporal_store(x[0], p);
  }
};
template <>
struct SpecVec<2> {
  typedef float F __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ void ld(const float* p, float (&x)[2]) {
    const F t = *reinterpret_cast<const F*>(p);
    x[0] = t[0];
    x[1] = t[1];
  }
  static __device__ __forceinline__ void ldnt(const float* p, float (&x)[2]) {
    const F t = __builtin_nontemporal_load(reinterpret_cast<const F*>(p));
    x[0] = t[0];
    x[1] = t[1];
  }
  static __device__ __forceinline__ void st(float* p, const float (&x)[2]) {
    __builtin_nontemporal_store(F{x[0], x[1]}, reinterpret_cast<F*>(p));
  }
};
template <typename T, int E>
__device__ __forceinline__ void ld_elems(const T* p, float (&x)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = (float)p[e];
}
template <typename T, int E>
__device__ __forceinline__ void st_elems(T* p, const float (&x)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e) p[e] = (T)x[e];
}

// FORM: SPEC_VERIFY, SPEC_VERIFY8 (at most 8 drafts: Gamma*K and Gamma*Q
// stacked into one 16-row operand, so one pass of products with the state
// gives both), SPEC_COMMIT.
enum SpecForm { SPEC_VERIFY = 0, SPEC_VERIFY8 = 1, SPEC_COMMIT = 2 };

// LAYER: the fused layer's verify and commit in the chunk form -- q, k, v
// (commit: k, v) from the projections' outputs through the prologue rows (each
// wave reads the raw rows of its blocks of tokens straight from the conv state
// and the projections); verify's o through the epilogue rows into y; commit
// advances the conv state past the accepted tokens.  With the standalone
// prologue and epilogue around the plain call the results are bitwise the
// same.  The LDS leaves room for three workgroups per CU with 2-byte tokens,
// two with 4-byte ones (which then take the registers of two waves per SIMD).
template <int DK, int DV, typename TIn, typename TOut, int KIND, int FORM, bool LAYER = false,
          bool COMMIT = FORM == SPEC_COMMIT, bool STACK = FORM == SPEC_VERIFY8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(LAYER && sizeof(TIn) == 4 ? 2 : COMMIT || LAYER || sizeof(TIn) == 4 ? 3 : 4))) void spec_chunk_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v, Gate gate,
    const float* __restrict__ beta, float* __restrict__ state, TOut* __restrict__ o,
    const int32_t* __restrict__ n_accept, int N, int H, LayerIO io) {
  using G = SpecGeo<DK, DV, COMMIT>;
  constexpr int CW = G::CW, E = G::E, KS = G::KS, ld = G::ld, ldT = G::ldT, ldKt = G::ldKt;
  __shared__ __align__(16) float sm[G::total];
  float* sK = sm + G::oK;
  float* sA = sm + G::oA;
  float* sQ = sm + G::oQ;
  float* sB = sm + G::oB;
  float* part = sm + G::oP;

  const int tile = blockIdx.x;  // (session, head) flattened
  const int sb = tile / H, h = tile - sb * H;
  int n = N;
  if constexpr (COMMIT) {
    const int na = n_accept[sb];
    n = na < 0 ? 0 : (na > N ? N : na);
    if (n == 0) return;  // nothing accepted: the state stays as it is
  }
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int tr = lane & 15, g = lane >> 4;
  const int col0 = w * CW + E * tr;  // this lane's first value column

  // the layer's dynamic LDS: the prologue's v rows [N][Dv] (then o [N][Dv] for
  // the epilogue) and, for 4-byte tokens, the exact path's copies of the
  // prologue's k and q [2][N][Dk]; 2-byte tokens keep those copies in the
  // partial sums' space (free until the sums are written)
  constexpr int SW = 2 * DK + DV, CPLK = DK / 64, CPLV = DV / 64;
  static_assert(sizeof(TIn) == 4 || 2 * 16 * DK * sizeof(TIn) <= 4 * 2 * 256 * sizeof(float),
                "k and q copies in the partial sums' space");
  extern __shared__ __align__(16) float dyn[];
  float* sV = dyn;
  TIn* cpy = sizeof(TIn) == 2 ? reinterpret_cast<TIn*>(part) : reinterpret_cast<TIn*>(dyn + N * DV);

  // The tokens' inputs are issued first and the state tile after them: loads
  // complete in order, so the token work below waits only for its own loads
  // while the state is still arriving.  Rows n..15 are alpha = 1, k = q = 0,
  // beta = 0.
  constexpr int SIT = 16 * (DK / 4) / 256;  // staging items per thread
  floatx4 ga[SIT], k4[SIT], q4[SIT];
  typename Raw4<TIn>::T kr[SIT], qr[SIT];  // k and q as loaded (widened after the state's loads)
#pragma unroll
  for (int it = 0; it < SIT; ++it) {
    const int idx = tid + 256 * it, t = idx / (DK / 4), c = 4 * (idx % (DK / 4));
    const bool ok = t < n;
    const size_t row = ((size_t)sb * N + (ok ? t : 0)) * H + h;
    ga[it] = gate_load4<KIND>(gate, ok, row, DK, c);
    k4[it] = floatx4{0.f, 0.f, 0.f, 0.f};
    q4[it] = k4[it];
    if constexpr (!LAYER) {  // (the layer's k and q come from the prologue rows)
      // loaded unconditionally (row 0 stands in past the drafts) and chosen
      // where used: a load under a branch is waited for inside it
      kr[it] = Raw4<TIn>::ld(k + row * DK + c);
      if constexpr (!COMMIT) qr[it] = Raw4<TIn>::ld(q + row * DK + c);
    }
  }
  const float bt = tid < n ? beta[((size_t)sb * N + tid) * H + h] : 0.f;
  float vv[4][E];  // v of rows 4g + i at this lane's columns
  TIn vr[4][E];    // ... as loaded (widened with k and q, after the state's loads)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 4 * g + i;
#pragma unroll
    for (int e = 0; e < E; ++e) vv[i][e] = 0.f;
    if constexpr (!LAYER) {
      const TIn* vp = v + (((size_t)sb * N + (t < n ? t : 0)) * H + h) * DV + col0;
#pragma unroll
      for (int e = 0; e < E; ++e) vr[i][e] = vp[e];
    }
  }
  // the layer's prologue: one wave per (block of 4 tokens, tensor), job
  // jb = NT block + tensor over the NT tensors the call needs (commit: k and
  // v), at most three per wave (jobs w, w + 4, w + 8), so that the first
  // blocks are jobs 0..NT-1; their loads go out ahead of the state's (a wave's
  // slot past the last job loads the rows of job 0 and computes nothing)
  static_assert(kMaxDraft <= 16, "three prologue blocks per wave");
  constexpr int CPLM = CPLK > CPLV ? CPLK : CPLV, NT = COMMIT ? 2 : 3;
  ProBlock<CPLM> pb[3];
  const int nb = (n + 3) >> 2;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  float* cs = io.conv_state + ((size_t)sb * 3 * H + h) * SW;
  const size_t xs = (size_t)sb * N * H + h;  // row of (token 0, head h)
  // commit: the conv state's new rows, raw rows n .. n + 2 of (its three rows,
  // then the tokens'), read here and written once every wave is past its
  // prologue rows (the reads of the old rows are then done); each source row
  // is read from both places in range and chosen, without branches
  constexpr int CIT = (3 * SW / 4 + 255) / 256;
  floatx4 cn[CIT];
  if constexpr (LAYER && COMMIT) {
#pragma unroll
    for (int it = 0; it < CIT; ++it) {
      const int idx = min(tid + 256 * it, 3 * SW / 4 - 1);
      const int j = idx / (SW / 4), c = 4 * (idx % (SW / 4)), r = n + j;
      const int tk = max(r - 3, 0), ten = c < DK ? 0 : c < 2 * DK ? 1 : 2;
      const int cc = c - (ten == 0 ? 0 : ten == 1 ? DK : 2 * DK), D = ten == 2 ? DV : DK;
      const TIn* x = (const TIn*)(ten == 0 ? io.xq : ten == 1 ? io.xk : io.xv);
      const floatx4 fx = ld4<TIn>(x + (xs + (size_t)tk * H) * D + cc);
      const floatx4 fc = *reinterpret_cast<const floatx4*>(cs + (size_t)min(r, 2) * H * SW + c);
      cn[it] = r < 3 ? fc : fx;
    }
  }
  if constexpr (LAYER) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int jb = wu + 4 * i < NT * nb ? wu + 4 * i : 0;
      const int ten = (3 - NT) + jb % NT, t0 = 4 * (jb / NT);
      const TIn* x = (const TIn*)(ten == 0 ? io.xq : ten == 1 ? io.xk : io.xv);
      const float* tp = ten == 0 ? io.conv.w[0] : ten == 1 ? io.conv.w[1] : io.conv.w[2];
      if constexpr (DK == DV) {
        if (i == 0)
          pro_load<TIn, CPLK, true>(pb[i], cs + ten * DK, x + xs * DK, (size_t)H * DK, H * SW,
                                    tp + (size_t)h * DK * 4, t0, n, lane);
        else
          pro_load<TIn, CPLK, false>(pb[i], cs, x + xs * DK, (size_t)H * DK, H * SW,
                                     tp + (size_t)h * DK * 4, t0, n, lane);
      } else if (ten == 2) {  // (Dk != Dv: the loads under the branch wait there)
        pro_load<TIn, CPLV, true>(pb[i], cs + 2 * DK, x + xs * DV, (size_t)H * DV, H * SW,
                                  tp + (size_t)h * DV * 4, t0, n, lane);
      } else {
        pro_load<TIn, CPLK, true>(pb[i], cs + ten * DK, x + xs * DK, (size_t)H * DK, H * SW,
                                  tp + (size_t)h * DK * 4, t0, n, lane);
      }
    }
  }
  // alpha, and the zero rows of k and q, into the token arrays (the layer does
  // this ahead of the state loads, which frees the gate's registers there)
#define KDA_SPEC_STAGE()                                                                    \
  {                                                                                         \
    const float sc = KIND == GATE_BOUNDED ? expf(gate.a_log[h]) : 1.f;                      \
    _Pragma("unroll") for (int it = 0; it < SIT; ++it) {                                    \
      const int idx = tid + 256 * it, t = idx / (DK / 4), c = 4 * (idx % (DK / 4));        \
      floatx4 a4 = ga[it];                                                                  \
      if constexpr (KIND == GATE_LOG) {                                                     \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) a4[e] = expf(a4[e]);                  \
      } else if constexpr (KIND == GATE_BOUNDED) {                                          \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) a4[e] =                               \
            gate_bounded(a4[e], sc, gate.g_min);                                            \
      }                                                                                     \
      *reinterpret_cast<floatx4*>(sA + t * ld + c) = a4;                                    \
      if (!LAYER || t >= n) { /* the layer's rows below n are the prologue's */             \
        *reinterpret_cast<floatx4*>(sK + t * ld + c) = k4[it];                              \
        if constexpr (!COMMIT) *reinterpret_cast<floatx4*>(sQ + t * ld + c) = q4[it];       \
      }                                                                                     \
    }                                                                                       \
    if (tid < 16) sB[tid] = bt;                                                             \
  }
  if constexpr (LAYER) KDA_SPEC_STAGE()
  // the state tile: k-step s holds row 4s + g
  float* S = state + (size_t)tile * DK * DV;
  float sr[KS][E];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if constexpr (COMMIT) SpecVec<E>::ld(S + (size_t)(4 * s + g) * DV + col0, sr[s]);
    else SpecVec<E>::ldnt(S + (size_t)(4 * s + g) * DV + col0, sr[s]);
  }
  // (nothing below is moved above the state's loads)
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!LAYER) {
#pragma unroll
    for (int it = 0; it < SIT; ++it) {
      const bool ok = (tid + 256 * it) / (DK / 4) < n;
      k4[it] = ok ? Raw4<TIn>::cvt(kr[it]) : k4[it];
      if constexpr (!COMMIT) q4[it] = ok ? Raw4<TIn>::cvt(qr[it]) : q4[it];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < E; ++e) vv[i][e] = 4 * g + i < n ? (float)vr[i][e] : 0.f;
  }
  if constexpr (LAYER) {
    // the prologue rows into the token arrays (rows n..15 stay zero)
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int jb = wu + 4 * i, ten = (3 - NT) + jb % NT, t0 = 4 * (jb / NT);
      const int cnt = min(4, n - t0);
      if (jb >= NT * nb) continue;
      if (ten == 0) pro_rows<TIn, CPLK, true>(pb[i], io.conv.eps, t0, cnt, lane, sQ, ld);
      else if (ten == 1) pro_rows<TIn, CPLK, true>(pb[i], io.conv.eps, t0, cnt, lane, sK, ld);
      else pro_rows<TIn, CPLV, false>(pb[i], io.conv.eps, t0, cnt, lane, sV, DV);
    }
  }

  const float scl = KIND == GATE_BOUNDED ? expf(gate.a_log[h]) : 1.f;
  if constexpr (!LAYER) KDA_SPEC_STAGE()
#undef KDA_SPEC_STAGE
  __syncthreads();
  if constexpr (LAYER) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * g + i;
#pragma unroll
      for (int e = 0; e < E; ++e) vv[i][e] = t < n ? sV[t * DV + col0 + e] : 0.f;
    }
    if constexpr (COMMIT) {  // the conv state advances past the n tokens
#pragma unroll
      for (int it = 0; it < CIT; ++it) {
        const int idx = tid + 256 * it;
        if (idx < 3 * SW / 4)
          *reinterpret_cast<floatx4*>(cs + (size_t)(idx / (SW / 4)) * H * SW + 4 * (idx % (SW / 4))) =
              cn[it];
      }
    }
  }

  // per key channel: Gamma_t by a running product; Gamma*k, k / Gamma (and
  // Gamma*q) in place; commit: Ktil by a suffix product (no division), and
  // Gamma_n (each block of four tokens read ahead of its products)
  if (tid < DK) {
    const int c = tid;
    if constexpr (COMMIT) {
      const int p = (c & ~15) + 4 * (c & 3) + ((c & 15) >> 2);  // Ktil^T row of channel c
      float sfx = 1.f;
#pragma unroll
      for (int t0 = 12; t0 >= 0; t0 -= 4) {
        float al[4], kc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          al[u] = sA[(t0 + u) * ld + c];
          kc[u] = sK[(t0 + u) * ld + c];
        }
#pragma unroll
        for (int u = 3; u >= 0; --u) {
          sQ[p * ldKt + t0 + u] = sfx * kc[u];
          sfx *= al[u];
        }
      }
    }
    float gm = 1.f;
#pragma unroll
    for (int t0 = 0; t0 < 16; t0 += 4) {
      float al[4], kc[4], qc[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        al[u] = sA[(t0 + u) * ld + c];
        kc[u] = sK[(t0 + u) * ld + c];
        if constexpr (!COMMIT) qc[u] = sQ[(t0 + u) * ld + c];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + u;
        if (LAYER && t < n) {  // the prologue's k and q (token-dtype values), for the exact path
          cpy[t * DK + c] = (TIn)kc[u];
          if constexpr (!COMMIT) cpy[(n + t) * DK + c] = (TIn)qc[u];
        }
        gm *= al[u];
        sK[t * ld + c] = gm * kc[u];
        // k / Gamma: read only while every channel stays in the factored range
        sA[t * ld + c] = kc[u] * __builtin_amdgcn_rcpf(gm);
        if constexpr (!COMMIT) sQ[t * ld + c] = gm * qc[u];
      }
    }
    if constexpr (COMMIT) sm[G::oG + c] = gm;
    const bool low = __builtin_amdgcn_ballot_w64(gm < frag::kTileMin) != 0;
    if (lane == 0) sm[G::oF + w] = low ? 1.f : 0.f;
  }
  __syncthreads();
  bool exact = sm[G::oF] != 0.f;
  if constexpr (DK == 128) exact = exact || sm[G::oF + 1] != 0.f;

  // ---- A (unscaled) and Mqk: rows t, columns j, parts over the key channels
  if (!exact) {
    floatx4 pa = {0.f, 0.f, 0.f, 0.f}, pm = pa;
#pragma unroll
    for (int s = w * G::KW; s < (w + 1) * G::KW; ++s) {
      const int c = 4 * s + g;
      const float kg = sA[tr * ld + c];
      pa = mfma4(sK[tr * ld + c], kg, pa);
      if constexpr (!COMMIT) pm = mfma4(sQ[tr * ld + c], kg, pm);
    }
    *reinterpret_cast<floatx4*>(part + (2 * w) * 256 + 4 * lane) = pa;
    *reinterpret_cast<floatx4*>(part + (2 * w + 1) * 256 + 4 * lane) = pm;
  } else {
    // thread (t, j): the decays between the two tokens as a running product
    const int t = tid >> 4, j = tid & 15;
    float a = 0.f, m = 0.f;
    if (j <= t && t < n) {
      const size_t rt = ((size_t)sb * N + t) * H + h, rj = ((size_t)sb * N + j) * H + h;
#pragma unroll 1
      for (int c = 0; c < DK; c += 4) {
        floatx4 r = {1.f, 1.f, 1.f, 1.f};
        for (int u = j + 1; u <= t; ++u) {
          const floatx4 a4 = alpha4_exact<KIND>(gate, ((size_t)sb * N + u) * H + h, DK, c, scl);
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = r[e] * a4[e];
        }
        floatx4 kt, kj, qt = {0.f, 0.f, 0.f, 0.f};
        if constexpr (LAYER) {
          kt = ld4<TIn>(cpy + t * DK + c);
          kj = ld4<TIn>(cpy + j * DK + c);
          if constexpr (!COMMIT) qt = ld4<TIn>(cpy + (n + t) * DK + c);
        } else {
          kt = ld4<TIn>(k + rt * DK + c);
          kj = ld4<TIn>(k + rj * DK + c);
          if constexpr (!COMMIT) qt = ld4<TIn>(q + rt * DK + c);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float kr = kj[e] * r[e];
          a = a + kt[e] * kr;
          m = m + qt[e] * kr;
        }
      }
    }
    if constexpr (LAYER) __syncthreads();  // (the copies may sit in the sums' space)
    // (t, j) sits at lane 16 (t / 4) + j, entry t % 4 of the accumulator layout
    const int pos = 4 * (16 * (t >> 2) + j) + (t & 3);
    part[pos] = a;
    part[256 + pos] = m;
    for (int idx = tid; idx < 3 * 2 * 256; idx += 256) part[2 * 256 + idx] = 0.f;
  }
  __syncthreads();
  floatx4 am = {0.f, 0.f, 0.f, 0.f}, mm = am;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    am += *reinterpret_cast<const floatx4*>(part + (2 * u) * 256 + 4 * lane);
    if constexpr (!COMMIT) mm += *reinterpret_cast<const floatx4*>(part + (2 * u + 1) * 256 + 4 * lane);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 4 * g + i;
    am[i] = tr < t ? sB[t] * am[i] : 0.f;
    mm[i] = tr <= t ? mm[i] : 0.f;
  }

  // ---- T Diag(beta) (and Mqk) as row reads of this wave's scratch
  float* buf = sm + G::oW + w * 16 * ldT;
  auto put = [&](const floatx4& x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) buf[(4 * g + i) * ldT + tr] = x[i];
    lds_sync();
  };
  auto row = [&]() -> floatx4 {
    const floatx4 r = *reinterpret_cast<const floatx4*>(buf + tr * ldT + 4 * g);
    lds_sync();
    return r;
  };
  put(am);
  const floatx4 aN = row();
  const floatx4 n2 = mm16(aN, am);
  put(n2);
  const floatx4 a2 = row();
  const floatx4 n4 = mm16(a2, n2);
  put(n4);
  const floatx4 a4r = row();
  floatx4 X = mm16(a4r, n4);  // N^8
#pragma unroll
  for (int i = 0; i < 4; ++i) X[i] += (4 * g + i == tr) ? 1.f : 0.f;
  X += mm16(a4r, X);
  X += mm16(a2, X);
  X -= mm16(aN, X);
  const float bj = sB[tr];
#pragma unroll
  for (int i = 0; i < 4; ++i) X[i] = X[i] * bj;
  put(X);
  const floatx4 aT = row();
  floatx4 aM = {0.f, 0.f, 0.f, 0.f};
  if constexpr (STACK) {
    // Mqk shifted down by 8 rows: its product with P lands on the rows that
    // hold (Gamma*Q) S below
#pragma unroll
    for (int i = 0; i < 4; ++i) buf[((4 * g + i + 8) & 15) * ldT + tr] = g < 2 ? mm[i] : 0.f;
    lds_sync();
    aM = row();
  } else if constexpr (!COMMIT) {
    put(mm);
    aM = row();
  }

  // the epilogue's weight and gate logits (tokens w + 4 r), ahead of the
  // products: loaded at a clamped token (no branch, which would wait for each
  // load in turn) and kept in the token dtype until the epilogue uses them
  float wn[CPLV];
  TIn gv[4][CPLV];
  if constexpr (LAYER) {
    ld_elems<float, CPLV>(io.out.w + CPLV * lane, wn);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = min(w + 4 * r, n - 1);
      const TIn* gp = (const TIn*)io.out.g + (((size_t)sb * N + t) * H + h) * DV + CPLV * lane;
#pragma unroll
      for (int c = 0; c < CPLV; ++c) gv[r][c] = gp[c];
    }
  }

  // ---- (Gamma*K) S and (Gamma*Q) S on this wave's columns
  floatx4 R[E], Y[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    R[e] = floatx4{0.f, 0.f, 0.f, 0.f};
    Y[e] = R[e];
  }
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    // stacked: rows 0..7 take Gamma*K, rows 8..15 Gamma*Q of tokens 0..7
    const float gk = STACK && tr >= 8 ? sQ[(tr - 8) * ld + 4 * s + g] : sK[tr * ld + 4 * s + g];
#pragma unroll
    for (int e = 0; e < E; ++e) R[e] = mfma4(gk, sr[s][e], R[e]);
    if constexpr (!COMMIT && !STACK) {
      const float gq = sQ[tr * ld + 4 * s + g];
#pragma unroll
      for (int e = 0; e < E; ++e) Y[e] = mfma4(gq, sr[s][e], Y[e]);
    }
  }

  // ---- P = T Diag(beta) (V - (Gamma*K) S): rows t = 4g + i, columns col0 + e
  floatx4 P[E];
  {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      floatx4 d;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = STACK && g >= 2 ? 0.f : vv[i][e] - R[e][i];
      P[e] = mm16(aT, d);
    }
  }

  if constexpr (!COMMIT) {
    float ov[4][E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const floatx4 x = (STACK ? R[e] : Y[e]) + mm16(aM, P[e]);
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i][e] = x[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = STACK ? 4 * (g - 2) + i : 4 * g + i;
      if ((!STACK || g >= 2) && t < n) {
        if constexpr (LAYER) {  // to the epilogue, through LDS (the v rows are consumed)
#pragma unroll
          for (int e = 0; e < E; ++e) sV[t * DV + col0 + e] = ov[i][e];
        } else {
          st_elems<TOut, E>(o + (((size_t)sb * N + t) * H + h) * DV + col0, ov[i]);
        }
      }
    }
    if constexpr (LAYER) {
      // epilogue rows, one wave per token (t = w + 4 r): y = RMSNorm(o) w Sigmoid(g)
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = w + 4 * r;
        if (t < n) {
          float ovr[CPLV], gr[CPLV], y[CPLV];
#pragma unroll
          for (int c = 0; c < CPLV; ++c) {
            ovr[c] = sV[t * DV + CPLV * lane + c];
            gr[c] = (float)gv[r][c];
          }
          epilogue_row<CPLV>(ovr, gr, wn, io.out.eps, y);
          row_store<TOut, CPLV>(o + (((size_t)sb * N + t) * H + h) * DV, lane, y);
        }
      }
    }
  } else {
    // S' = Diag(Gamma_n) S + Ktil^T P: row tile rt of the permuted Ktil^T gives
    // accumulator row 4g + i = state row 16 rt + 4i + g = k-step 4 rt + i
    const float* gn = sm + G::oG;
#pragma unroll
    for (int rt = 0; rt < DK / 16; ++rt) {
      const floatx4 ak = *reinterpret_cast<const floatx4*>(sQ + (16 * rt + tr) * ldKt + 4 * g);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const floatx4 acc = mm16(ak, P[e]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 4 * rt + i;
          sr[s][e] = gn[4 * s + g] * sr[s][e] + acc[i];
        }
      }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) SpecVec<E>::st(S + (size_t)(4 * s + g) * DV + col0, sr[s]);
  }
}

// LDS of one workgroup: N token records; with the layer, the raw rows
// [3 + N][2 Dk + Dv], the gate logits [N][Dv] and the conv taps [2 Dk + Dv][4]
template <int DK, int DV, bool VERIFY>
constexpr int multi_lds_bytes(int N, bool layer = false) {
  return (int)sizeof(float) * (Rec<DK, DV, VERIFY>::stride * N +
                               (layer ? (N + 7) * (2 * DK + DV) + N * DV : 0));
}

// the largest LDS a mode's instantiation may ask for (N up to kMaxDraft),
// granted once per instantiation before its first launch
template <typename K>
static hipError_t allow_lds(K kern, int bytes, bool& done, int below = 65536) {
  if (done || bytes <= below) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     bytes);
  if (e == hipSuccess) done = true;
  return e;
}

// Verify and commit of at least this many draft tokens run as one chunk
// (spec_chunk_kernel), the fused layer's calls too; fewer step the tokens.
// The token loop's cost grows with N and the chunk form's hardly does; on
// MI355X at 64 sessions x 96 heads x 128 x 128 they cross near 5 tokens for
// verify (stacked form, 6: 115 against about 120 us; 8: 115 against 147 us)
// and near 12 for commit (16: 178 against 201 us; 8: 162 against 153 us).
constexpr int kSpecVerifyChunkMin = 6;
constexpr int kSpecCommitChunkMin = 12;

// the layer's calls: v (then o) rows [N][Dv]; for 4-byte tokens also the
// copies of k and q [2][N][Dk]
template <int DK, int DV, typename TIn>
constexpr int spec_layer_lds_bytes(int N) {
  return (int)sizeof(float) * N * (DV + (sizeof(TIn) == 4 ? 2 * DK : 0));
}

template <int DK, int DV, typename TIn, typename TOut, int KIND, bool LAYER>
static hipError_t launch_spec_chunk(const DecodeArgs& a) {
  const dim3 grid(a.B * a.H);
  // with the layer, static and dynamic LDS together pass 64 KiB: the larger
  // size is granted once per instantiation (idempotent if raced)
  const int lds = LAYER ? spec_layer_lds_bytes<DK, DV, TIn>(a.N) : 0;
  const int mx = LAYER ? spec_layer_lds_bytes<DK, DV, TIn>(kMaxDraft) : 0;
  static bool lds8 = false, lds16 = false, ldsc = false;
  if (a.mode == DECODE_VERIFY && a.N <= 8) {
    if (hipError_t e = allow_lds(spec_chunk_kernel<DK, DV, TIn, TOut, KIND, SPEC_VERIFY8, LAYER>,
                                 mx, lds8, 0);
        e != hipSuccess)
      return e;
    hipLaunchKernelGGL((spec_chunk_kernel<DK, DV, TIn, TOut, KIND, SPEC_VERIFY8, LAYER>), grid,
                       dim3(256), lds, (hipStream_t)a.stream, (const TIn*)a.q, (const TIn*)a.k,
                       (const TIn*)a.v, a.gate, a.beta, a.state, (TOut*)a.o,
                       (const int32_t*)nullptr, a.N, a.H, a.io);
  } else if (a.mode == DECODE_VERIFY) {
    if (hipError_t e = allow_lds(spec_chunk_kernel<DK, DV, TIn, TOut, KIND, SPEC_VERIFY, LAYER>,
                                 mx, lds16, 0);
        e != hipSuccess)
      return e;
    hipLaunchKernelGGL((spec_chunk_kernel<DK, DV, TIn, TOut, KIND, SPEC_VERIFY, LAYER>), grid,
                       dim3(256), lds, (hipStream_t)a.stream, (const TIn*)a.q, (const TIn*)a.k,
                       (const TIn*)a.v, a.gate, a.beta, a.state, (TOut*)a.o,
                       (const int32_t*)nullptr, a.N, a.H, a.io);
  } else {
    if (hipError_t e = allow_lds(spec_chunk_kernel<DK, DV, TIn, float, KIND, SPEC_COMMIT, LAYER>,
                                 mx, ldsc, 0);
        e != hipSuccess)
      return e;
    hipLaunchKernelGGL((spec_chunk_kernel<DK, DV, TIn, float, KIND, SPEC_COMMIT, LAYER>), grid,
                       dim3(256), lds, (hipStream_t)a.stream, (const TIn*)nullptr,
                       (const TIn*)a.k, (const TIn*)a.v, a.gate, a.beta, a.state,
                       (float*)nullptr, a.n_accept, a.N, a.H, a.io);
  }
  return hipGetLastError();
}

template <int DK, int DV, typename TIn, typename TOut, int KIND, bool LAYER>
static hipError_t launch_decode_l(const DecodeArgs& a) {
  const dim3 grid(a.B * a.H);
  if (a.mode == DECODE_VERIFY && a.N >= kSpecVerifyChunkMin)
    return launch_spec_chunk<DK, DV, TIn, TOut, KIND, LAYER>(a);
  if (a.mode == DECODE_COMMIT && a.N >= kSpecCommitChunkMin)
    return launch_spec_chunk<DK, DV, TIn, TOut, KIND, LAYER>(a);
  static bool lds_v = false, lds_c = false;  // per instantiation; idempotent if raced
  if (a.mode == DECODE_VERIFY) {
    if (hipError_t e = allow_lds(decode_kernel<DK, DV, TIn, TOut, KIND, DECODE_VERIFY, LAYER>,
                                 multi_lds_bytes<DK, DV, true>(kMaxDraft, LAYER), lds_v);
        e != hipSuccess)
      return e;
  } else if (a.mode == DECODE_COMMIT) {
    if (hipError_t e = allow_lds(decode_kernel<DK, DV, TIn, float, KIND, DECODE_COMMIT, LAYER>,
                                 multi_lds_bytes<DK, DV, false>(kMaxDraft, LAYER), lds_c);
        e != hipSuccess)
      return e;
  }
  if (a.mode == DECODE_STEP) {
    hipLaunchKernelGGL((decode_kernel<DK, DV, TIn, TOut, KIND, DECODE_STEP, LAYER>), grid,
                       dim3(256), (multi_lds_bytes<DK, DV, true>(1, LAYER)), (hipStream_t)a.stream,
                       (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, a.gate, a.beta, a.state,
                       (TOut*)a.o, (const int32_t*)nullptr, 1, a.H, a.io);
  } else if (a.mode == DECODE_VERIFY) {
    hipLaunchKernelGGL((decode_kernel<DK, DV, TIn, TOut, KIND, DECODE_VERIFY, LAYER>), grid,
                       dim3(256), (multi_lds_bytes<DK, DV, true>(a.N, LAYER)),
                       (hipStream_t)a.stream, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v,
                       a.gate, a.beta, a.state, (TOut*)a.o, (const int32_t*)nullptr, a.N, a.H,
                       a.io);
  } else {
    hipLaunchKernelGGL((decode_kernel<DK, DV, TIn, float, KIND, DECODE_COMMIT, LAYER>), grid,
                       dim3(256), (multi_lds_bytes<DK, DV, false>(a.N, LAYER)),
                       (hipStream_t)a.stream, (const TIn*)nullptr, (const TIn*)a.k,
                       (const TIn*)a.v, a.gate, a.beta, a.state, (float*)nullptr, a.n_accept, a.N,
                       a.H, a.io);
  }
  return hipGetLastError();
}

template <int DK, int DV, typename TIn, typename TOut, int KIND>
static hipError_t launch_decode_k(const DecodeArgs& a) {
  return a.layer ? launch_decode_l<DK, DV, TIn, TOut, KIND, true>(a)
                 : launch_decode_l<DK, DV, TIn, TOut, KIND, false>(a);
}

// one instantiation per gate kind: the per-row decay is a straight-line loop
template <int DK, int DV, typename TIn, typename TOut>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  switch (a.gate.kind) {
    case GATE_LOG: return launch_decode_k<DK, DV, TIn, TOut, GATE_LOG>(a);
    case GATE_BOUNDED: return launch_decode_k<DK, DV, TIn, TOut, GATE_BOUNDED>(a);
    case GATE_SCALAR: return launch_decode_k<DK, DV, TIn, TOut, GATE_SCALAR>(a);
    case GATE_NONE: return launch_decode_k<DK, DV, TIn, TOut, GATE_NONE>(a);
    default: return launch_decode_k<DK, DV, TIn, TOut, GATE_ALPHA>(a);
  }
}

template <int DK, int DV>
static hipError_t launch_decode_d(const DecodeArgs& a) {
  if (a.qkv_bf16) {
    return a.o_bf16 ? launch_decode_t<DK, DV, bf16, bf16>(a) : launch_decode_t<DK, DV, bf16, float>(a);
  }
  return a.o_bf16 ? launch_decode_t<DK, DV, float, bf16>(a) : launch_decode_t<DK, DV, float, float>(a);
}

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.Dk == 128 && a.Dv == 128) return launch_decode_d<128, 128>(a);
  if (a.Dk == 128 && a.Dv == 64) return launch_decode_d<128, 64>(a);
  if (a.Dk == 64 && a.Dv == 128) return launch_decode_d<64, 128>(a);
  return launch_decode_d<64, 64>(a);
}

template <int DK, int DV, typename TOut, int KIND>
static hipError_t launch_rec_k(const PrefillArgs& a) {
  const int grid = a.n_seq * a.H;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((recurrent_prefill_kernel<DK, DV, float, TOut, KIND>), dim3(grid), dim3(256),
                     ((int)sizeof(float) * Rec<DK, DV, true>::stride * NBLK), (hipStream_t)a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, a.gate, a.beta,
                     a.initial_state, a.final_state, (TOut*)a.o, a.cu_seqlens, a.n_seq, a.T, a.H);
  return hipGetLastError();
}
template <int DK, int DV, typename TOut>
static hipError_t launch_rec_t(const PrefillArgs& a) {
  switch (a.gate.kind) {
    case GATE_LOG: return launch_rec_k<DK, DV, TOut, GATE_LOG>(a);
    case GATE_BOUNDED: return launch_rec_k<DK, DV, TOut, GATE_BOUNDED>(a);
    case GATE_SCALAR: return launch_rec_k<DK, DV, TOut, GATE_SCALAR>(a);
    case GATE_NONE: return launch_rec_k<DK, DV, TOut, GATE_NONE>(a);
    default: return launch_rec_k<DK, DV, TOut, GATE_ALPHA>(a);
  }
}

// fp32 q, k, v with Dk = 128 (the fp32 chunked kernel serves Dk = 64)
hipError_t launch_prefill_recurrent(const PrefillArgs& a) {
  if (a.Dv == 128) return a.o_bf16 ? launch_rec_t<128, 128, bf16>(a) : launch_rec_t<128, 128, float>(a);
  return a.o_bf16 ? launch_rec_t<128, 64, bf16>(a) : launch_rec_t<128, 64, float>(a);
}

}  // namespace kda
