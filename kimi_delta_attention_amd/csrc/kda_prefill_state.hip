// kda_prefill_state.hip -- second pass of the two-pass chunked prefill (gfx950):
// the chunk-to-chunk state recurrence, and the chunk table of packed sequences.
//
// The chunk form splits each 64-token chunk into work that does not depend on
// the entry state S (decays, the UT transform T, W, U, Mqk, Gamma*Q, Ktil; done
// by the first pass for every (chunk, head) at once, "Kimi Delta Attention
// 完全拆解", section "chunk 内并行、chunk 间递推") and the part that does:
//
//   P  = U - W S,   O = (Gamma*Q) S + Mqk P,   S' = Diag(Gamma_C) S + Ktil^T P
//
// This kernel runs that part.  One workgroup owns (sequence, head, 64-wide
// value slice) and walks the chunks in order with the state slice in MFMA
// accumulators, exactly as the fused kernel does, but its per-chunk operands
// arrive as register images (Images<DK, DV>) that are fetched with coalesced
// 16-byte loads one chunk ahead.  Eight waves: wave (w, hh) takes token tile w
// (tokens 16w..16w+15) and value half hh for P and O, and state rows
// [w*DK/4, (w+1)*DK/4) x the same value half for the update.  The products and
// their order are those of the fused kernel, so both schedules give bitwise
// the same results.
#include "kda_common.h"
#include "kda_frag.h"
#include "kda_internal.h"

namespace kda {
namespace {

using namespace frag;

constexpr int NTH_S = 512;

template <int DK>
struct StatePlan {
  static constexpr int ldS = DK + 8, ldP = CH + 8;
  static constexpr int ST = BV * ldS * 2 * 2, PT = BV * ldP * 2 * 2;
  static constexpr int oST = 0, oPT = ST, total = ST + PT;
};

template <int DK, int DV, typename TOut>
__global__ __launch_bounds__(NTH_S) void prefill_state_kernel(
    const unsigned char* __restrict__ img, const int32_t* __restrict__ chunk_off,
    const int32_t* __restrict__ cu_seqlens, const float* __restrict__ s_init,
    float* __restrict__ s_final, TOut* __restrict__ o, int n_seq, int T, int H) {
  using L = StatePlan<DK>;
  using IM = Images<DK, DV>;
  constexpr int NKB = DK / 32;
  constexpr int RPW = DK / 4;
  constexpr int RTW = RPW / 16;
  constexpr int NCH = BV / 32;
  constexpr int ldS = L::ldS, ldP = L::ldP;
  constexpr int loS = BV * ldS, loP = BV * ldP;

  extern __shared__ __align__(16) unsigned char smem[];
  bf16* ST = reinterpret_cast<bf16*>(smem + L::oST);
  bf16* PT = reinterpret_cast<bf16*>(smem + L::oPT);

  const int tid = threadIdx.x;
  const int w8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = w8 >> 2;
  const int w = w8 & 3;
  const int lane = tid & 63;

  constexpr int nsl = DV / BV;
  const int total = n_seq * H * nsl;
  int wid = blockIdx.x;
  if ((total & 7) == 0) wid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int sl = wid % nsl;
  const int h = (wid / nsl) % H;
  const int seq = wid / (nsl * H);
  long long start, len;
  int ci0;  // global index of the sequence's first chunk
  if (cu_seqlens) {
    start = cu_seqlens[seq];
    len = (long long)cu_seqlens[seq + 1] - start;
    ci0 = chunk_off[seq];
    // the table's chunk count (equal to ceil(len / 64) for monotone offsets)
    const long long tab = (long long)(chunk_off[seq + 1] - ci0) * CH;
    if (len > tab) len = tab;
  } else {
    start = (long long)seq * T;
    len = T;
    ci0 = seq * ((T + CH - 1) / CH);
  }
  const int vcol0 = sl * BV;
  const int vh0 = 32 * hh;
  const int vt0 = (vcol0 + vh0) / 16;  // first U tile of this wave

  floatx4 Sacc[RTW][NCH];
  {
    const int tr = lane & 15, g = lane >> 4;
    const float* si = s_init ? s_init + ((size_t)seq * H + h) * DK * DV : nullptr;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = w * RPW + rt * 16 + 4 * g + i;
          Sacc[rt][c][i] = si ? si[(size_t)row * DV + vcol0 + vh0 + c * 16 + tr] : 0.f;
        }
  }

  // Operands of one chunk, loaded one chunk ahead into a single register set:
  // the W, (Gamma*Q) and U parts right after W S and (Gamma*Q) S have used
  // them, the Mqk, Ktil and Gamma_C parts after the state update.
  struct Ops {
    bf16x8 wh[NKB], wl[NKB], qf[NKB], mh[2], ml[2], kh[RTW][2], kl[RTW][2];
    floatx4 u[NCH], gc[RTW];
  };
  auto item_base = [&](int c) -> const unsigned char* {
    return img + ((size_t)(ci0 + c) * H + h) * IM::bytes;
  };
  auto load_a = [&](int c, Ops& op) {
    const unsigned char* b = item_base(c);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      op.wh[kb] = *frame_ptr<bf16x8>(b, IM::w_frame(w, kb, 0), lane);
      op.wl[kb] = *frame_ptr<bf16x8>(b, IM::w_frame(w, kb, 1), lane);
      op.qf[kb] = *frame_ptr<bf16x8>(b, IM::q_frame(w, kb), lane);
    }
#pragma unroll
    for (int c2 = 0; c2 < NCH; ++c2) op.u[c2] = *frame_ptr<floatx4>(b, IM::u_frame(w, vt0 + c2), lane);
  };
  auto load_b = [&](int c, Ops& op) {
    const unsigned char* b = item_base(c);
    const int g = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      op.mh[kb] = *frame_ptr<bf16x8>(b, IM::m_frame(w, kb, 0), lane);
      op.ml[kb] = *frame_ptr<bf16x8>(b, IM::m_frame(w, kb, 1), lane);
    }
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        op.kh[rt][kb] = *frame_ptr<bf16x8>(b, IM::k_frame(RTW * w + rt, kb, 0), lane);
        op.kl[rt][kb] = *frame_ptr<bf16x8>(b, IM::k_frame(RTW * w + rt, kb, 1), lane);
      }
      op.gc[rt] = *reinterpret_cast<const floatx4*>(b + IM::g_off +
                                                    4 * (w * RPW + rt * 16 + 4 * g));
    }
  };

  const int nch = (int)((len + CH - 1) / CH);
  Ops op;
  if (nch > 0) {
    load_a(0, op);
    load_b(0, op);
  }
  for (int c = 0; c < nch; ++c) {
    int lane_x = lane;
    __asm__ volatile("" : "+v"(lane_x));
    const int tr = lane_x & 15;
    const int g = lane_x >> 4;
    const long long tok0 = start + (long long)c * CH;
    const int nv = (int)(len - (long long)c * CH < CH ? len - (long long)c * CH : CH);
    const bool more = c + 1 < nch;

    // ---- the state as the B operand of W S and (Gamma*Q) S: [value][channel
    // position], position 32kb + 8g + 4h + i holds channel 32kb + 16h + 4g + i
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int c0r = w * RPW + rt * 16;
      const int pos = 32 * (c0r >> 5) + 8 * g + 4 * ((c0r >> 4) & 1);
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
        float x4[4] = {Sacc[rt][cc][0], Sacc[rt][cc][1], Sacc[rt][cc][2], Sacc[rt][cc][3]};
        st_split4(ST + (vh0 + 16 * cc + tr) * ldS + pos, loS, x4);
      }
    }
    __syncthreads();

    // ---- P = U - W S and O = (Gamma*Q) S for tile w, this wave's columns
    floatx4 accO[NCH];
    {
      floatx4 accW[NCH];
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
        accW[cc] = floatx4{0.f, 0.f, 0.f, 0.f};
        accO[cc] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) {
          const bf16x8 bh = frag_ld(ST, ldS, vh0 + 16 * cc + tr, 32 * kb, g);
          const bf16x8 bl = frag_ld(ST + loS, ldS, vh0 + 16 * cc + tr, 32 * kb, g);
          accW[cc] = mma_ab(op.wh[kb], op.wl[kb], bh, bl, accW[cc]);
          accO[cc] = mfma_bf16(op.qf[kb], bh, accO[cc]);
          accO[cc] = mfma_bf16(op.qf[kb], bl, accO[cc]);
        }
      }
      float pv[NCH][4];
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc)
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[cc][i] = op.u[cc][i] - accW[cc][i];
      if (more) load_a(c + 1, op);
      // P to LDS as [value][token position]; token 32kb + 16h + 4g + i sits at
      // position 32kb + 8g + 4h + i (the order of the Mqk^T operand)
      const int pos = 32 * (w >> 1) + 8 * g + 4 * (w & 1);
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) st_split4(PT + (vh0 + 16 * cc + tr) * ldP + pos, loP, pv[cc]);
    }
    __syncthreads();

    // ---- O += Mqk P; store o
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb > (w >> 1)) continue;
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
        const bf16x8 bh = frag_ld(PT, ldP, vh0 + 16 * cc + tr, 32 * kb, g);
        const bf16x8 bl = frag_ld(PT + loP, ldP, vh0 + 16 * cc + tr, 32 * kb, g);
        accO[cc] = mma_ab(op.mh[kb], op.ml[kb], bh, bl, accO[cc]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 16 * w + 4 * g + i;
      if (rr < nv) {
        TOut* orow = o + ((size_t)(tok0 + rr) * H + h) * DV + vcol0 + vh0 + tr;
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) __builtin_nontemporal_store((TOut)accO[cc][i], orow + 16 * cc);
      }
    }

    // ---- S = Diag(Gamma_C) S + Ktil^T P
    {
      bf16x8 bph[2][NCH], bpl[2][NCH];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc) {
          bph[kb][cc] = frag_ld(PT, ldP, vh0 + 16 * cc + tr, 32 * kb, g);
          bpl[kb][cc] = frag_ld(PT + loP, ldP, vh0 + 16 * cc + tr, 32 * kb, g);
        }
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) {
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc)
#pragma unroll
          for (int i = 0; i < 4; ++i) Sacc[rt][cc][i] *= op.gc[rt][i];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int cc = 0; cc < NCH; ++cc)
            Sacc[rt][cc] = mma_ab(op.kh[rt][kb], op.kl[rt][kb], bph[kb][cc], bpl[kb][cc], Sacc[rt][cc]);
      }
    }
    if (more) load_b(c + 1, op);
    __syncthreads();  // PT and ST reads done before the next chunk overwrites them
  }

  if (s_final) {
    const int tr = lane & 15, g = lane >> 4;
    float* sf = s_final + ((size_t)seq * H + h) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = w * RPW + rt * 16 + 4 * g + i;
          sf[(size_t)row * DV + vcol0 + vh0 + cc * 16 + tr] = Sacc[rt][cc][i];
        }
  }
}

// chunk_off[s] = number of 64-token chunks of the sequences before s
// (s = 0..n_seq), clamped to the `cap` chunks the workspace holds (reached only
// if cu_seqlens is not monotone); one workgroup, blocked prefix sum.
__device__ __forceinline__ int chunks_of(const int32_t* cu, int s) {
  const int len = cu[s + 1] - cu[s];
  return len > 0 ? (len + CH - 1) / CH : 0;
}

__global__ __launch_bounds__(256) void chunk_table_kernel(const int32_t* __restrict__ cu_seqlens,
                                                          int n_seq, int cap,
                                                          int32_t* __restrict__ chunk_off) {
  __shared__ int part[256];
  const int t = threadIdx.x;
  const int per = (n_seq + 255) / 256;
  const int s0 = t * per, s1 = s0 + per < n_seq ? s0 + per : n_seq;
  int sum = 0;
  for (int s = s0; s < s1; ++s) sum += chunks_of(cu_seqlens, s);
  part[t] = sum;
  __syncthreads();
  if (t == 0) {
    int acc = 0;
    for (int i = 0; i < 256; ++i) {
      const int x = part[i];
      part[i] = acc;
      acc += x;
    }
    chunk_off[n_seq] = acc < cap ? acc : cap;
  }
  __syncthreads();
  int acc = part[t];
  for (int s = s0; s < s1; ++s) {
    chunk_off[s] = acc < cap ? acc : cap;
    acc += chunks_of(cu_seqlens, s);
  }
}

template <int DK, int DV, typename TOut>
hipError_t launch_state_t(const PrefillArgs& a, const unsigned char* img, const int32_t* chunk_off) {
  using L = StatePlan<DK>;
  auto kern = prefill_state_kernel<DK, DV, TOut>;
  const int grid = a.n_seq * a.H * (DV / BV);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTH_S), L::total, (hipStream_t)a.stream, img, chunk_off,
                     a.cu_seqlens, a.initial_state, a.final_state, (TOut*)a.o, a.n_seq, a.T, a.H);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_state_d(const PrefillArgs& a, const unsigned char* img, const int32_t* chunk_off) {
  return a.o_bf16 ? launch_state_t<DK, DV, bf16>(a, img, chunk_off)
                  : launch_state_t<DK, DV, float>(a, img, chunk_off);
}

}  // namespace

hipError_t launch_prefill_state(const PrefillArgs& a, const unsigned char* img,
                                const int32_t* chunk_off) {
  if (a.Dk == 128) {
    return a.Dv == 128 ? launch_state_d<128, 128>(a, img, chunk_off)
                       : launch_state_d<128, 64>(a, img, chunk_off);
  }
  return a.Dv == 128 ? launch_state_d<64, 128>(a, img, chunk_off)
                     : launch_state_d<64, 64>(a, img, chunk_off);
}

hipError_t launch_chunk_table(const int32_t* cu_seqlens, int n_seq, int cap, int32_t* chunk_off,
                              void* stream) {
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, cu_seqlens,
                     n_seq, cap, chunk_off);
  return hipGetLastError();
}

size_t prefill_image_bytes(int Dk, int Dv) {
  if (Dk == 128) return Dv == 128 ? Images<128, 128>::bytes : Images<128, 64>::bytes;
  return Dv == 128 ? Images<64, 128>::bytes : Images<64, 64>::bytes;
}

}  // namespace kda
