// kda_decode.hip -- one-token KDA step for B sessions x H heads (gfx950).
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
// the key axis are finished with cross-lane xor shuffles inside the wave (no
// LDS, no barrier).
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

template <typename TIn>
__device__ __forceinline__ float ld_in(const TIn* p, size_t i);
template <>
__device__ __forceinline__ float ld_in<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_in<bf16>(const bf16* p, size_t i) { return (float)p[i]; }

template <int DK, int DV, typename TIn, typename TOut, int KIND>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    Gate gate, const float* __restrict__ beta, float* __restrict__ state, TOut* __restrict__ o,
    int H) {
  constexpr int CW = DV / 4;       // value columns per wave
  constexpr int LPR = CW / 4;      // lanes sharing one row (float4 each)
  constexpr int RPP = 64 / LPR;    // rows covered per pass
  constexpr int NP = DK / RPP;     // passes (rows per lane)
  static_assert(NP * RPP == DK, "row split");

  const int tile = blockIdx.x;     // (session, head) flattened
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int cg = lane % LPR;
  const int ro = lane / LPR;
  const int col = w * CW + 4 * cg;

  float* S = state + (size_t)tile * DK * DV;
  const TIn* qt = q + (size_t)tile * DK;
  const TIn* kt = k + (size_t)tile * DK;

  floatx4 s[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i)
    s[i] = *reinterpret_cast<const floatx4*>(S + (size_t)(ro + RPP * i) * DV + col);

  float kr[NP], qr[NP], al[NP];
  if constexpr (KIND == GATE_BOUNDED) {
    // the LPR lanes that hold the same rows each evaluate NP / LPR of the gates
    // (two exponentials each) and read the others' across the group
    constexpr int PER = NP / LPR;
    static_assert(PER * LPR == NP, "rows per lane split");
    float mine[PER];
    const float sc = expf(gate.a_log[tile % H]);
#pragma unroll
    for (int j = 0; j < PER; ++j)
      mine[j] = gate_bounded(gate.g[(size_t)tile * DK + ro + RPP * (PER * cg + j)], sc,
                             gate.g_min);
    const int base = lane - cg;
#pragma unroll
    for (int i = 0; i < NP; ++i) al[i] = __shfl(mine[i % PER], base + i / PER, 64);
  } else {
    gate_alpha_rows<KIND, NP, RPP>(gate, tile, DK, ro, 0, al);
  }
  floatx4 old = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
  float qk = 0.f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int r = ro + RPP * i;
    const float a = al[i];
    kr[i] = ld_in(kt, r);
    qr[i] = ld_in(qt, r);
    s[i] *= a;                     // Sbar = Diag(alpha) S
    old += s[i] * kr[i];           // Sbar^T k (partial over this lane's rows)
    p += s[i] * qr[i];             // Sbar^T q
    qk += kr[i] * qr[i];
  }
  // finish the sums over the lanes that share these columns
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      old[j] += __shfl_xor(old[j], m);
      p[j] += __shfl_xor(p[j], m);
    }
    qk += __shfl_xor(qk, m);
  }
  const float b = beta[tile];
  floatx4 u;
#pragma unroll
  for (int j = 0; j < 4; ++j) u[j] = b * (ld_in(v + (size_t)tile * DV, col + j) - old[j]);

  // streaming (non-temporal) stores: the state is written once and not re-read
  // by this launch; on gfx950 this write path sustains close to HBM peak where
  // ordinary stores of the same pattern stall on the cache write-back path
#pragma unroll
  for (int i = 0; i < NP; ++i)
    __builtin_nontemporal_store(s[i] + kr[i] * u,
                                reinterpret_cast<floatx4*>(S + (size_t)(ro + RPP * i) * DV + col));

  if (ro == 0) {
    TOut* ot = o + (size_t)tile * DV + col;
#pragma unroll
    for (int j = 0; j < 4; ++j) ot[j] = (TOut)(p[j] + qk * u[j]);
  }
}

template <int DK, int DV, typename TIn, typename TOut, int KIND>
static hipError_t launch_decode_k(const DecodeArgs& a) {
  hipLaunchKernelGGL((decode_step_kernel<DK, DV, TIn, TOut, KIND>), dim3(a.B * a.H), dim3(256), 0,
                     (hipStream_t)a.stream, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v,
                     a.gate, a.beta, a.state, (TOut*)a.o, a.H);
  return hipGetLastError();
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

}  // namespace kda
