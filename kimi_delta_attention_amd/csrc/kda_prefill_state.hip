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
// This kernel runs that part for one window of packed tokens (the chunks that
// start in it).  One workgroup owns (sequence, head, 64-wide value slice) and
// walks its chunks of the window in order with the state slice in MFMA
// accumulators, entering from the initial state (at the sequence's first chunk)
// or from the carry buffer, and leaving the state in the carry buffer (the
// caller's final state or workspace); its per-chunk operands arrive as register images
// (Images<DK, DV>) fetched with coalesced 16-byte loads.  Eight waves; wave
// (w, hh) fetches only operands no other wave of the workgroup fetches (the
// per-compute-unit load path, not HBM, limits this pass):
//   W S and (Gamma*Q) S   token tile w, all 64 values, channel half hh; the
//                         two halves are added through LDS, each wave keeping
//                         the sum for its value half hh
//   P, Mqk P, o           token tile w, value half hh
//   state update          Dk = 128: state rows 16(2w + hh).., all 64 values;
//                         Dk = 64: rows 16w.., value half hh
// The fused kernel computes the same products with the same accumulation
// order (the two channel halves as separate chains, low half first), so both
// schedules give bitwise the same results.
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
  // partial sums handed between the two waves of a tile: [w][from hh][tile j][W, O] frames
  static constexpr int XC = 4 * 2 * 2 * 2 * 1024;
  static constexpr int oST = 0, oPT = ST, oXC = ST + PT, total = ST + PT + XC;
  static_assert(total <= 163840, "LDS budget");
};

template <int DK, int DV, typename TOut>
__global__ __launch_bounds__(NTH_S) void prefill_state_kernel(
    const unsigned char* __restrict__ img, const int32_t* __restrict__ chunk_off,
    const int32_t* __restrict__ cu_seqlens, const float* s_init, float* carry,
    TOut* __restrict__ o, int n_seq, int T, int H, long long tok_lo, long long tok_hi, int cap) {
  using L = StatePlan<DK>;
  using IM = Images<DK, DV>;
  constexpr int NKB = DK / 32;
  constexpr int NKH = NKB / 2;                   // 32-channel blocks per channel half
  constexpr int NVT = BV / 16;                   // value tiles of the slice
  constexpr int KVT = DK == 128 ? NVT : NVT / 2;  // value tiles of this wave's state rows
  constexpr int ldS = L::ldS, ldP = L::ldP;
  constexpr int loS = BV * ldS, loP = BV * ldP;

  extern __shared__ __align__(16) unsigned char smem[];
  bf16* ST = reinterpret_cast<bf16*>(smem + L::oST);
  bf16* PT = reinterpret_cast<bf16*>(smem + L::oPT);
  unsigned char* XC = smem + L::oXC;

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
  int ci0, nch_seq;  // global index of the sequence's first chunk, its chunk count
  if (cu_seqlens) {
    start = cu_seqlens[seq];
    len = (long long)cu_seqlens[seq + 1] - start;
    ci0 = chunk_off[seq];
    nch_seq = chunk_off[seq + 1] - ci0;  // ceil(len / 64) for monotone offsets
  } else {
    start = (long long)seq * T;
    len = T;
    nch_seq = (T + CH - 1) / CH;
    ci0 = seq * nch_seq;
  }
  if (len > (long long)nch_seq * CH) len = (long long)nch_seq * CH;
  // this window's chunks of the sequence, [c_lo, c_hi); item slot of chunk c
  // is ci0 + c - ci_lo, below cap
  const int ci_lo = chunks_before(tok_lo, cu_seqlens, chunk_off, n_seq, T);
  auto first_from = [&](long long tok) {
    long long c = (tok - start + CH - 1) / CH;
    if (c < 0) c = 0;
    return (int)(c < nch_seq ? c : nch_seq);
  };
  int c_lo = first_from(tok_lo), c_hi = first_from(tok_hi);
  if (c_lo < ci_lo - ci0) c_lo = ci_lo - ci0;          // reached only for
  if (c_hi > cap + ci_lo - ci0) c_hi = cap + ci_lo - ci0;  // non-monotone cu_seqlens
  // an empty sequence hands its initial state through in the first window
  if (!(c_lo < c_hi || (nch_seq == 0 && tok_lo == 0))) return;
  const int vcol0 = sl * BV;
  const int vh0 = 32 * hh;             // value half of P and o
  const int vt0 = (vcol0 + vh0) / 16;  // its first U tile
  // state rows and value tiles of the update
  const int srt = DK == 128 ? 2 * w + hh : w;  // 16-row tile
  const int sv0 = DK == 128 ? 0 : 2 * hh;      // first value tile (within the slice)

  floatx4 Sacc[KVT];
  {
    const int tr = lane & 15, g = lane >> 4;
    const float* src = c_lo == 0 ? s_init : carry;
    const float* si = src ? src + ((size_t)seq * H + h) * DK * DV : nullptr;
#pragma unroll
    for (int j = 0; j < KVT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * srt + 4 * g + i;
        Sacc[j][i] = si ? si[(size_t)row * DV + vcol0 + 16 * (sv0 + j) + tr] : 0.f;
      }
  }

  // Operands of one chunk: OpsA (W and Gamma*Q of this wave's channel half, U
  // of its value half; needed first) and OpsB (Mqk of tile w, Ktil of the state
  // rows, Gamma_C; needed last).  Both are fetched one chunk ahead into second
  // register sets, OpsB at the start of a chunk and OpsA after its first
  // barrier.  Every fetch is unconditional (the last chunk refetches itself) so
  // that the compiler's waits for one group never have to cover the other.
  struct OpsA {
    bf16x8 wh[NKH], wl[NKH], qf[NKH];
    floatx4 u[2];
  };
  struct OpsB {
    bf16x8 mh[2], ml[2], kh[2], kl[2];
    floatx4 gc;
  };
  auto item_base = [&](int c) -> const unsigned char* {
    return img + ((size_t)(ci0 + c - ci_lo) * H + h) * IM::bytes;
  };
  auto load_a = [&](int c, OpsA& op) {
    const unsigned char* b = item_base(c);
#pragma unroll
    for (int kk = 0; kk < NKH; ++kk) {
      op.wh[kk] = *frame_ptr<bf16x8>(b, IM::w_frame(w, NKH * hh + kk, 0), lane);
      op.wl[kk] = *frame_ptr<bf16x8>(b, IM::w_frame(w, NKH * hh + kk, 1), lane);
      op.qf[kk] = *frame_ptr<bf16x8>(b, IM::q_frame(w, NKH * hh + kk), lane);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) op.u[j] = *frame_ptr<floatx4>(b, IM::u_frame(w, vt0 + j), lane);
  };
  auto load_b = [&](int c, OpsB& op) {
    const unsigned char* b = item_base(c);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      op.mh[kb] = *frame_ptr<bf16x8>(b, IM::m_frame(w, kb, 0), lane);
      op.ml[kb] = *frame_ptr<bf16x8>(b, IM::m_frame(w, kb, 1), lane);
      op.kh[kb] = *frame_ptr<bf16x8>(b, IM::k_frame(srt, kb, 0), lane);
      op.kl[kb] = *frame_ptr<bf16x8>(b, IM::k_frame(srt, kb, 1), lane);
    }
    op.gc = *reinterpret_cast<const floatx4*>(b + IM::g_off + 4 * (16 * srt + 4 * (lane >> 4)));
  };
  // partial-sum frames: [w][from hh][tile j][W, O]
  auto xc = [&](int from, int j, int part, int ln) {
    return reinterpret_cast<floatx4*>(XC + ((((w * 2 + from) * 2 + j) * 2 + part) * 1024) + 16 * ln);
  };

  OpsA op;
  OpsB ob;
  if (c_lo < c_hi) {
    load_a(c_lo, op);
    load_b(c_lo, ob);
  }
  for (int c = c_lo; c < c_hi; ++c) {
    OpsB nb;
    load_b(c + 1 < c_hi ? c + 1 : c, nb);
    int lane_x = lane;
    __asm__ volatile("" : "+v"(lane_x));
    const int tr = lane_x & 15;
    const int g = lane_x >> 4;
    const long long tok0 = start + (long long)c * CH;
    const int nv = (int)(len - (long long)c * CH < CH ? len - (long long)c * CH : CH);

    // ---- the state as the B operand of W S and (Gamma*Q) S: [value][channel
    // position], position 32kb + 8g + 4h + i holds channel 32kb + 16h + 4g + i
    {
      const int c0r = 16 * srt;
      const int pos = 32 * (c0r >> 5) + 8 * g + 4 * ((c0r >> 4) & 1);
#pragma unroll
      for (int j = 0; j < KVT; ++j) {
        float x4[4] = {Sacc[j][0], Sacc[j][1], Sacc[j][2], Sacc[j][3]};
        st_split4(ST + (16 * (sv0 + j) + tr) * ldS + pos, loS, x4);
      }
    }
    __syncthreads();
    OpsA nx;
    load_a(c + 1 < c_hi ? c + 1 : c, nx);

    // ---- W S and (Gamma*Q) S over this wave's channel half, all 64 values
    floatx4 accW[NVT], accO[NVT];
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) {
      accW[vt] = floatx4{0.f, 0.f, 0.f, 0.f};
      accO[vt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kk = 0; kk < NKH; ++kk) {
      const int kb = NKH * hh + kk;
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const bf16x8 bh = frag_ld(ST, ldS, 16 * vt + tr, 32 * kb, g);
        const bf16x8 bl = frag_ld(ST + loS, ldS, 16 * vt + tr, 32 * kb, g);
        accW[vt] = mma_ab(op.wh[kk], op.wl[kk], bh, bl, accW[vt]);
        accO[vt] = mfma_bf16(op.qf[kk], bh, accO[vt]);
        accO[vt] = mfma_bf16(op.qf[kk], bl, accO[vt]);
      }
    }
    // hand the partner's value half over, take its partial sums for ours
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      *xc(hh, j, 0, lane_x) = accW[2 * (1 - hh) + j];
      *xc(hh, j, 1, lane_x) = accO[2 * (1 - hh) + j];
    }
    __syncthreads();
    floatx4 accP[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const floatx4 pw = *xc(1 - hh, j, 0, lane_x), po = *xc(1 - hh, j, 1, lane_x);
      const floatx4 mw = accW[2 * hh + j], mo = accO[2 * hh + j];
      const floatx4 wsum = hh ? pw + mw : mw + pw;  // low channel half first
      accP[j] = hh ? po + mo : mo + po;             // (Gamma*Q) S, then Mqk P below
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = op.u[j][i] - wsum[i];
      // P to LDS as [value][token position]; token 32kb + 16h + 4g + i sits at
      // position 32kb + 8g + 4h + i (the order of the Mqk^T operand)
      const int pos = 32 * (w >> 1) + 8 * g + 4 * (w & 1);
      st_split4(PT + (vh0 + 16 * j + tr) * ldP + pos, loP, pv);
    }
    op = nx;
    __syncthreads();

    // ---- O += Mqk P; store o.  Both token blocks for every tile: the Mqk
    // frames of blocks after the tile are zero, and a branch here would let the
    // compiler move their fetch next to this use.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 bh = frag_ld(PT, ldP, vh0 + 16 * j + tr, 32 * kb, g);
        const bf16x8 bl = frag_ld(PT + loP, ldP, vh0 + 16 * j + tr, 32 * kb, g);
        accP[j] = mma_ab(ob.mh[kb], ob.ml[kb], bh, bl, accP[j]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 16 * w + 4 * g + i;
      if (rr < nv) {
        TOut* orow = o + ((size_t)(tok0 + rr) * H + h) * DV + vcol0 + vh0 + tr;
#pragma unroll
        for (int j = 0; j < 2; ++j) __builtin_nontemporal_store((TOut)accP[j][i], orow + 16 * j);
      }
    }

    // ---- S = Diag(Gamma_C) S + Ktil^T P
#pragma unroll
    for (int j = 0; j < KVT; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Sacc[j][i] *= ob.gc[i];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 bh = frag_ld(PT, ldP, 16 * (sv0 + j) + tr, 32 * kb, g);
        const bf16x8 bl = frag_ld(PT + loP, ldP, 16 * (sv0 + j) + tr, 32 * kb, g);
        Sacc[j] = mma_ab(ob.kh[kb], ob.kl[kb], bh, bl, Sacc[j]);
      }
    }
    ob = nb;
    __syncthreads();  // PT, ST and the partial sums are read before the next chunk rewrites them
  }

  {
    const int tr = lane & 15, g = lane >> 4;
    float* sf = carry + ((size_t)seq * H + h) * DK * DV;
#pragma unroll
    for (int j = 0; j < KVT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * srt + 4 * g + i;
        sf[(size_t)row * DV + vcol0 + 16 * (sv0 + j) + tr] = Sacc[j][i];
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
hipError_t launch_state_t(const PrefillArgs& a, const unsigned char* img, const int32_t* chunk_off,
                          float* carry, long long tok_lo, long long tok_hi, int cap) {
  using L = StatePlan<DK>;
  auto kern = prefill_state_kernel<DK, DV, TOut>;
  static bool attr_set = false;  // per instantiation; idempotent if raced
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, L::total);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int grid = a.n_seq * a.H * (DV / BV);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTH_S), L::total, (hipStream_t)a.stream, img, chunk_off,
                     a.cu_seqlens, a.initial_state, carry, (TOut*)a.o, a.n_seq, a.T, a.H, tok_lo,
                     tok_hi, cap);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_state_d(const PrefillArgs& a, const unsigned char* img, const int32_t* chunk_off,
                          float* carry, long long tok_lo, long long tok_hi, int cap) {
  return a.o_bf16 ? launch_state_t<DK, DV, bf16>(a, img, chunk_off, carry, tok_lo, tok_hi, cap)
                  : launch_state_t<DK, DV, float>(a, img, chunk_off, carry, tok_lo, tok_hi, cap);
}

}  // namespace

hipError_t launch_prefill_state(const PrefillArgs& a, const unsigned char* img,
                                const int32_t* chunk_off, float* carry, long long tok_lo,
                                long long tok_hi, int cap) {
  if (a.Dk == 128) {
    return a.Dv == 128 ? launch_state_d<128, 128>(a, img, chunk_off, carry, tok_lo, tok_hi, cap)
                       : launch_state_d<128, 64>(a, img, chunk_off, carry, tok_lo, tok_hi, cap);
  }
  return a.Dv == 128 ? launch_state_d<64, 128>(a, img, chunk_off, carry, tok_lo, tok_hi, cap)
                     : launch_state_d<64, 64>(a, img, chunk_off, carry, tok_lo, tok_hi, cap);
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
