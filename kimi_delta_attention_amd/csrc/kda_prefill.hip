// kda_prefill.hip -- chunked KDA prefill for bf16 inputs on gfx950 (dense and
// packed varlen), plus the dispatch of both prefill kernels.
//
// Chunk form of S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,
// o_t = S_t^T q_t ("Kimi Delta Attention 完全拆解", section "chunk 内并行、chunk 间
// 递推"; "Kimi K3 的 KDA" section 5; "Kimi K3模型架构详解" sections 3.4-3.5).  For a
// 64-token chunk with entry state S and in-chunk cumulative decay
// Gamma_r = prod_{s<=r} a_s (per key channel):
//
//   A_rj   = b_r sum_c k_rc k_jc Gamma_rc / Gamma_jc      (j < r)
//   T      = (I + A)^{-1}                                  (UT transform)
//   W      = T Diag(b) (Gamma * K),   U = T Diag(b) V
//   P      = U - W S                                       (per-token corrections)
//   Mqk_rj = sum_c q_rc k_jc Gamma_rc / Gamma_jc          (j <= r)
//   O      = (Gamma * Q) S + Mqk P
//   S'     = Diag(Gamma_C) S + Ktil^T P,   Ktil_j = (Gamma_C / Gamma_j) * k_j
//
// Decay ratios inside A and Mqk are factored over 16-token tiles: with P_r the
// product of a from the start of r's tile up to r and E_n the whole-tile
// product, a pair (r in tile m, j in tile n < m) uses P_r and
// (E_n / P_j) * prod_{n<i<m} E_i, both <= 1; the diagonal tile uses P_r and
// 1 / P_j, bounded by one tile's decay (the tiling the bounded gate of
// "Kimi K3 的 KDA" section 6 is made for).
//
// Work decomposition.  One workgroup (8 waves, two per SIMD) owns (sequence,
// head, 64-wide value slice) and walks the chunks in order; the state slice
// stays in MFMA accumulators for the whole sequence.  Token tile w (tokens
// 16w..16w+15 of the chunk) belongs to a pair of waves: during operand build
// and the A / Mqk products each wave of the pair takes one half of the key
// channels (the halves are summed through LDS), afterwards each takes one
// 32-column half of the value slice.  A lane holds token 16w + l%16 and, per
// 32-channel block kb, the 8 channels 32kb + 4g + {0..3} and
// 32kb + 16 + 4g + {0..3} (g = l/16).  That set is exactly the k range an MFMA
// 16x16x32 output tile of a transposed product delivers to a lane, so outputs
// chain into the next product's operands in registers: (Gamma*K)^T T^T gives W
// in the operand layout of W S, and Mqk^T tiles give the operand of Mqk P.
// Products contracted over the token axis read row-major [token][channel] LDS
// tiles through the gfx950 transpose read (ds_read_b64_tr_b16).  The
// within-tile decay products are a 16-lane DPP scan; T comes from a blockwise
// solve on fp32 MFMA whose diagonal 16x16 blocks use the nilpotent product
// (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8).
//
// Precision: bf16 MFMA with split-bf16 operands (x = hi + lo, product
// hi*hi + hi*lo + lo*hi) everywhere except A (single pass); U and (Gamma*Q) S
// split only the side that is not exact in bf16, W only the T Diag(b) side
// (an emulation of every per-product choice against the fp64 recurrence, over
// the gate regimes of the tests, set this policy).
#include "kda_common.h"
#include "kda_frag.h"
#include "kda_internal.h"

// Every product is rounded on its own (no fused multiply-add contraction):
// the fused kernel and the two-pass kernels evaluate the same expressions in
// different code shapes, and only uncontracted arithmetic gives them bitwise
// the same results whatever the compiler's scheduling.
#pragma clang fp contract(off)

namespace kda {
namespace {

constexpr int NTH = 512;  // 8 waves
// two-pass window: 128 chunks (8192 packed tokens).  Larger windows mean fewer
// launches and, for the segmented schedule, longer segments per summary and
// combine: against 64 chunks, 1.051 vs 1.061 ms on the 96-head 8K layer and
// 0.227 vs 0.260 ms on its 12-head share (6 segments); 32 and 16 chunks were
// slower (1.092, 1.145 ms).  The workspace holds one window's operands.
constexpr int WIN_CHUNKS = 128;

using namespace frag;

// LDS plan (bytes).  R0 is reused phase by phase:
//   A / Mqk:      RT (right operands of every row tile, position order)
//   partials:     AF, AF2 (the two channel halves of beta*A), MQ0, MQ1 (of Mqk), TF
//   solve:        AF, AF2, TF, and the per-wave scratch SCR in the MQ0 region
//   T*b, V:       TB (T Diag(b), split) and VS (V slice) over MQ0 / MQ1
//   serial:       ST (state, split), PT (P, split), KT (Ktil, split)
// GK ((Gamma*K), bf16, [token][channel]) and QT ((Gamma*Q), [token][position])
// live from operand build to their last product; ES / GC / BS are small.  VW is
// the width of the staged V block (the 64-wide value slice).
template <int DK, int VW>
struct Plan {
  static constexpr int ldR = DK + 8, ldG = DK + 8, ldQ = DK + 8, ldA = CH + 4, ldT = CH + 8,
                       ldV = VW + 8, ldS = DK + 8, ldP = CH + 8;
  static constexpr int RT = 160 * ldR * 2 * 2;
  static constexpr int AF = CH * ldA * 4, TB = CH * ldT * 2 * 2, VS = CH * ldV * 2;
  static constexpr int ST = BV * ldS * 2 * 2, PT = BV * ldP * 2 * 2, KT = CH * ldG * 2 * 2;
  static constexpr int oRT = 0;
  static constexpr int oAF = 0, oAF2 = AF, oTF = 2 * AF, oMQ0 = 3 * AF, oMQ1 = 4 * AF,
                       oSCR = 3 * AF, oTB = 3 * AF, oVS = 3 * AF + TB, endB = oVS + VS;
  static constexpr int oST = 0, oPT = ST, oKT = ST + PT, endC = ST + PT + KT;
  static constexpr int m1 = RT > 5 * AF ? RT : 5 * AF;
  static constexpr int m2 = endB > endC ? endB : endC;
  static constexpr int R0 = m1 > m2 ? m1 : m2;
  static constexpr int GK = CH * ldG * 2, QT = CH * ldQ * 2, QTL = 16 * ldQ * 2;
  static constexpr int oGK = R0, oQT = oGK + GK, oQTL = oQT + QT, oES = oQTL + QTL,
                       oGC = oES + 4 * DK * 4,
                       oBS = oGC + DK * 4, total = oBS + CH * 4;
  static_assert(total <= 163840, "LDS budget (160 KiB)");
  static_assert(4 * 2048 <= AF, "T-solve scratch fits in the MQ0 region");
  static_assert(oTB >= oTF + AF, "TB is built from TF and must not overlap it");
  static_assert((oGK | oQT | oQTL | oES | oGC | oBS | oTF | oTB | oVS | oPT | oKT | oAF2 | oMQ1) % 16 == 0,
                "alignment");
};

// One workgroup per (sequence, head, 64-wide value slice), state carried
// across the sequence's chunks.
template <int DK, typename TOut, int KIND>
__global__ __launch_bounds__(NTH) void prefill_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    Gate gate, const float* __restrict__ beta,
    const float* __restrict__ s_init, float* __restrict__ s_final, TOut* __restrict__ o,
    const int32_t* __restrict__ cu_seqlens, int n_seq, int T, int H, int DV) {
  using L = Plan<DK, BV>;
  constexpr int NKB = DK / 32;   // 32-channel blocks
  constexpr int NKH = NKB / 2;   // blocks of one channel half
  constexpr int NCHT = DK / 16;  // 16-channel tiles
  constexpr int RPW = DK / 4;    // state rows per token-tile wave pair
  constexpr int RTW = RPW / 16;  // state row tiles per wave
  constexpr int NCH = BV / 32;   // value tiles per wave (its 32-column half)
  constexpr int ldR = L::ldR, ldG = L::ldG, ldQ = L::ldQ, ldA = L::ldA, ldT = L::ldT,
                ldV = L::ldV, ldS = L::ldS, ldP = L::ldP;
  constexpr int loR = 160 * ldR, loG = CH * ldG, loT = CH * ldT, loS = BV * ldS, loP = BV * ldP;

  extern __shared__ __align__(16) unsigned char smem[];
  bf16* RT = reinterpret_cast<bf16*>(smem + L::oRT);
  float* AF = reinterpret_cast<float*>(smem + L::oAF);
  float* AF2 = reinterpret_cast<float*>(smem + L::oAF2);
  float* TF = reinterpret_cast<float*>(smem + L::oTF);
  float* MQ0 = reinterpret_cast<float*>(smem + L::oMQ0);
  float* MQ1 = reinterpret_cast<float*>(smem + L::oMQ1);
  float* SCR = reinterpret_cast<float*>(smem + L::oSCR);
  bf16* TB = reinterpret_cast<bf16*>(smem + L::oTB);
  bf16* VS = reinterpret_cast<bf16*>(smem + L::oVS);
  bf16* ST = reinterpret_cast<bf16*>(smem + L::oST);
  bf16* PT = reinterpret_cast<bf16*>(smem + L::oPT);
  bf16* KT = reinterpret_cast<bf16*>(smem + L::oKT);
  bf16* GK = reinterpret_cast<bf16*>(smem + L::oGK);
  bf16* QT = reinterpret_cast<bf16*>(smem + L::oQT);
  bf16* QTL = reinterpret_cast<bf16*>(smem + L::oQTL);  // low halves of tile 0's rows
  float* ES = reinterpret_cast<float*>(smem + L::oES);  // [4][DK] tile decays
  float* GC = reinterpret_cast<float*>(smem + L::oGC);  // [DK] chunk decay
  float* BS = reinterpret_cast<float*>(smem + L::oBS);  // [64] beta

  const int tid = threadIdx.x;
  // Eight waves: wave pair (w, hh) with hh = 0, 1 shares token tile w.  Waves
  // are dealt to the 4 SIMDs round-robin, so pairing tile s with tile 3 - s
  // on one SIMD evens out the per-tile work (low tiles build more decay
  // variants, high tiles compute more A / Mqk pairs).
  const int w8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = w8 >> 2;                       // channel half (prep) / value half (serial)
  const int w = hh ? 3 - (w8 & 3) : (w8 & 3);   // token tile
  const int lane = tid & 63;
  const int tr = lane & 15;
  const int g = lane >> 4;

  const int nsl = DV / BV;
  int sl, h, seq;
  long long start, len;
  {
    const int total = n_seq * H * nsl;
    int wid = blockIdx.x;
    if ((total & 7) == 0) wid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    sl = wid % nsl;
    h = (wid / nsl) % H;
    seq = wid / (nsl * H);
    if (cu_seqlens) {
      start = cu_seqlens[seq];
      len = (long long)cu_seqlens[seq + 1] - start;
    } else {
      start = (long long)seq * T;
      len = T;
    }
  }
  const int vcol0 = sl * BV;
  const int vh0 = 32 * hh;  // this wave's value columns within the slice
  // per-head logit scale exp(A_h) of the bounded gate
  const float gsc = KIND == GATE_BOUNDED ? expf(gate.a_log[h]) : 1.f;

  // state: wave (w, hh) owns key rows [w*RPW, (w+1)*RPW) x value columns vh0..vh0+31
  floatx4 Sacc[RTW][NCH];
  {
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

  // One chunk: first token (global index), valid tokens, head, offset in the
  // sequence.
  struct Desc {
    long long tok0;
    int nv, hd;
    long long c0;
  };

  const int r = 16 * w + tr;  // this lane's token within the chunk

  // Global loads of one chunk for this lane's token and channel half (k, q,
  // alpha), 8 values of the V slice and beta.  One register set: each part is
  // refetched for the next chunk right after its last use in the current one
  // (alpha after the scan, k and q after the operand build, v and beta after
  // the V slice is staged), so no copies are needed and the loads have most of
  // a chunk to arrive.
  struct ChunkIn {
    uint2v k[NKH][2], q[NKH][2];
    floatx4 a[NKH][2];
    uint4v v;
    float b;
  };
  // V columns this lane stages: 8 of the slice
  const int vld0 = vcol0 + vh0 + 8 * g;
  auto load_part = [&](const Desc& d, ChunkIn& in, int part) {
    const bool okc = r < d.nv;
    const size_t thc = (size_t)(d.tok0 + r) * H + d.hd;
    if (part == 3) {
      in.v = okc ? *reinterpret_cast<const uint4v*>(v + thc * DV + vld0) : uint4v{0u, 0u, 0u, 0u};
      in.b = okc ? beta[thc] : 0.f;
      return;
    }
#pragma unroll
    for (int kk = 0; kk < NKH; ++kk)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int c = 32 * (NKH * hh + kk) + 16 * hf + 4 * g;
        if (part == 0) in.k[kk][hf] = okc ? *reinterpret_cast<const uint2v*>(k + thc * DK + c)
                                          : uint2v{0u, 0u};
        if (part == 1) in.q[kk][hf] = okc ? *reinterpret_cast<const uint2v*>(q + thc * DK + c)
                                          : uint2v{0u, 0u};
        if (part == 2) in.a[kk][hf] = gate_load4<KIND>(gate, okc, thc, DK, c);
      }
  };
  Desc cur = Desc{start, (int)(len < CH ? len : CH), h, 0};
  bool have = len > 0;
  ChunkIn in;
  if (have) {
    for (int part = 0; part < 4; ++part) load_part(cur, in, part);
    gate_finish_blocks<KIND, NKH>(gate, gsc, in.a);
  }

  while (have) {
    const long long c1 = cur.c0 + CH;
    const bool more = c1 < len;
    const Desc nxt = Desc{start + c1, (int)(len - c1 < CH ? len - c1 : CH), h, c1};
    // Lane indices, re-derived each chunk behind an empty asm so that the
    // compiler recomputes the many per-lane LDS addresses inside the loop
    // instead of keeping them all live across it (which exhausts the 256
    // registers a wave has at two waves per SIMD).
    int lane_x = lane;
    __asm__ volatile("" : "+v"(lane_x));
    const int tr = lane_x & 15;
    const int g = lane_x >> 4;
    const int r = 16 * w + tr;
    const int tid = 64 * w8 + lane_x;
    const int nv = cur.nv;
    const long long tok0 = cur.tok0;
    __syncthreads();  // the previous chunk is done with LDS

    const float bt = in.b;

    // ---- within-tile decay products P (inclusive scan over the 16 tokens)
    float Pv[NKH][8];
#pragma unroll
    for (int kk = 0; kk < NKH; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) Pv[kk][e] = in.a[kk][e >> 2][e & 3];
    row_scan_mul<8 * NKH>(&Pv[0][0]);
    if (more) load_part(nxt, in, 2);
    if (tr == 15) {  // whole-tile decay E_w of this wave's channels
#pragma unroll
      for (int kk = 0; kk < NKH; ++kk)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          *reinterpret_cast<floatx4*>(ES + w * DK + 32 * (NKH * hh + kk) + 16 * hf + 4 * g) =
              floatx4{Pv[kk][4 * hf], Pv[kk][4 * hf + 1], Pv[kk][4 * hf + 2], Pv[kk][4 * hf + 3]};
    }
    if (g == 0 && hh == 0) BS[r] = bt;
    __syncthreads();

    // A tile whose decay product leaves the range of the factored form takes
    // the exact path (the first pass does the same, in the same order): the
    // diagonal tile's A and Mqk sums of this wave's channel half by running
    // products, and suffix products in place of E / P below.  The decays are
    // loaded again (the scan overwrote them, and the next chunk's are in flight).
    const bool exact = tile_flagged<DK>(ES + w * DK, lane_x);
    auto alpha_of = [&](int kb, float* al) {
      floatx4 a4[1][2];
      const bool okc = r < nv;
      const size_t thc = (size_t)(tok0 + r) * H + h;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) a4[0][hf] = gate_load4<KIND>(gate, okc, thc, DK, 32 * kb + 16 * hf + 4 * g);
      gate_finish_blocks<KIND, 1>(gate, gsc, a4);
#pragma unroll
      for (int e = 0; e < 8; ++e) al[e] = a4[0][e >> 2][e & 3];
    };
    float dA[4] = {}, dM[4] = {};
    if (exact) {
      float al[NKH][8];
#pragma unroll
      for (int kk = 0; kk < NKH; ++kk) alpha_of(NKH * hh + kk, al[kk]);
      tile_exact_sums<NKH>(al, in.k, in.q, tr, g, dA, dM);
    }

    // ---- operands for this wave's channels.  Registers: KL = k*P and QL = q*P
    // (split), the B operands of A^T and Mqk^T; Ktil (split) until it is stored.
    // LDS: RT rows of this tile for row tiles mm >= w, GK = k*Gamma (bf16,
    // [token][channel]), QT = q*Gamma ([token][position]).
    bf16x8 kl[NKH], qlh[NKH], qll[NKH], kth[NKH], ktl[NKH];
#pragma unroll
    for (int kk = 0; kk < NKH; ++kk) {
      const int kb = NKH * hh + kk;
      auto ld_e = [&](int i, float* out) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const floatx4 e4 = *reinterpret_cast<const floatx4*>(ES + i * DK + 32 * kb + 16 * hf + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) out[4 * hf + e] = e4[e];
        }
      };
      float kk8[8], qq[8], pre[8], post[8], Ew[8], tmp[8];
      ld_e(w, Ew);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pre[e] = 1.f;
        post[e] = 1.f;
        kk8[e] = bfv(in.k[kk][e >> 2][(e & 3) >> 1], e & 1);
        qq[e] = bfv(in.q[kk][e >> 2][(e & 3) >> 1], e & 1);
      }
      for (int i = 0; i < w; ++i) {
        ld_e(i, tmp);
#pragma unroll
        for (int e = 0; e < 8; ++e) pre[e] *= tmp[e];
      }
      for (int i = w + 1; i < 4; ++i) {
        ld_e(i, tmp);
#pragma unroll
        for (int e = 0; e < 8; ++e) post[e] *= tmp[e];
      }
      float y[8], gk[8], kt[8], rd[8], re[8], sfx[8];
      bf16x8 qt8;
      if (exact) {  // decay from after this token to the tile's end, as a product
        alpha_of(kb, sfx);
        row_rscan_excl<8>(sfx);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kl[kk][e] = (bf16)(kk8[e] * Pv[kk][e]);
        y[e] = qq[e] * Pv[kk][e];
        const float gam = pre[e] * Pv[kk][e];
        qt8[e] = (bf16)(qq[e] * gam);
        gk[e] = kk8[e] * gam;
        const float ip = __builtin_amdgcn_rcpf(Pv[kk][e]);
        const float ew = exact ? sfx[e] : Ew[e] * ip;
        kt[e] = kk8[e] * (ew * post[e]);
        rd[e] = kk8[e] * ip;  // (not used in an exact tile)
        re[e] = kk8[e] * ew;
      }
      split8(y, qlh[kk], qll[kk]);
      split8(kt, kth[kk], ktl[kk]);
      // (Gamma*Q) at operand positions 32kb + 8g.. of token r
      *reinterpret_cast<bf16x8*>(QT + r * ldQ + 32 * kb + 8 * g) = qt8;
      // tile 0 of a sequence's first chunk keeps Gamma*Q split (its read-out
      // of the entry state is the least decayed, and a short sequence is
      // nothing else); there Gamma = P, so Gamma*Q is q P and its low half is
      // qll
      if (w == 0 && cur.c0 == 0)
        *reinterpret_cast<bf16x8*>(QTL + r * ldQ + 32 * kb + 8 * g) = qll[kk];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        st_bf16x4(GK + r * ldG + 32 * kb + 16 * hf + 4 * g, gk + 4 * hf);
      if (w == 0 && tr == 0) {
        float gc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) gc[e] = Ew[e] * post[e];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          *reinterpret_cast<floatx4*>(GC + 32 * kb + 16 * hf + 4 * g) =
              floatx4{gc[4 * hf], gc[4 * hf + 1], gc[4 * hf + 2], gc[4 * hf + 3]};
      }
      {
        const int row = 8 * w * (w + 1) + r;  // 16 * w(w+1)/2 rows precede row tile w
        bf16x8 hi, lo;
        split8(rd, hi, lo);
        *reinterpret_cast<bf16x8*>(RT + row * ldR + 32 * kb + 8 * g) = hi;
        *reinterpret_cast<bf16x8*>(RT + row * ldR + 32 * kb + 8 * g + loR) = lo;
      }
      for (int mm = w + 1; mm < 4; ++mm) {
        const int row = 8 * mm * (mm + 1) + r;
        bf16x8 hi, lo;
        split8(re, hi, lo);
        *reinterpret_cast<bf16x8*>(RT + row * ldR + 32 * kb + 8 * g) = hi;
        *reinterpret_cast<bf16x8*>(RT + row * ldR + 32 * kb + 8 * g + loR) = lo;
        if (mm < 3) {
          ld_e(mm, tmp);
#pragma unroll
          for (int e = 0; e < 8; ++e) re[e] *= tmp[e];
        }
      }
    }
    __syncthreads();
    if (more) {
      load_part(nxt, in, 0);
      load_part(nxt, in, 1);
    }

    // ---- A^T and Mqk^T tiles (j in tile n, r in tile w), n = 0..w, over this
    // wave's channel half; the two halves are summed through LDS
    floatx4 accA[4], accM[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      accA[n] = floatx4{0.f, 0.f, 0.f, 0.f};
      accM[n] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (n > w) continue;
      const int row = 8 * w * (w + 1) + 16 * n + tr;
#pragma unroll
      for (int kk = 0; kk < NKH; ++kk) {
        const int kb = NKH * hh + kk;
        const bf16x8 ah = frag_ld(RT, ldR, row, 32 * kb, g);
        const bf16x8 al = frag_ld(RT + loR, ldR, row, 32 * kb, g);
        accA[n] = mfma_bf16(ah, kl[kk], accA[n]);
        accM[n] = mma_ab(ah, al, qlh[kk], qll[kk], accM[n]);
      }
      if (n == w && exact) {  // the diagonal tile from the exact sums
        accA[n] = floatx4{dA[0], dA[1], dA[2], dA[3]};
        accM[n] = floatx4{dM[0], dM[1], dM[2], dM[3]};
      }
    }
    __syncthreads();  // RT reads done; the partials overwrite it
    {
      float* AFh = hh ? AF2 : AF;
      float* MQh = hh ? MQ1 : MQ0;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        if (n > w) continue;
        float a4[4], m4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 16 * n + 4 * g + i;
          a4[i] = (j < r) ? bt * accA[n][i] : 0.f;
          m4[i] = (j <= r) ? accM[n][i] : 0.f;
        }
        *reinterpret_cast<floatx4*>(AFh + r * ldA + 16 * n + 4 * g) = floatx4{a4[0], a4[1], a4[2], a4[3]};
        *reinterpret_cast<floatx4*>(MQh + r * ldA + 16 * n + 4 * g) = floatx4{m4[0], m4[1], m4[2], m4[3]};
      }
    }
    __syncthreads();
    // Mqk^T into operand fragments of Mqk P (token k-slots in the swizzled order)
    bf16x8 mqh[2], mql[2];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      floatx4 m4 = {0.f, 0.f, 0.f, 0.f};
      if (n <= w)
        m4 = *reinterpret_cast<const floatx4*>(MQ0 + r * ldA + 16 * n + 4 * g) +
             *reinterpret_cast<const floatx4*>(MQ1 + r * ldA + 16 * n + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16 hv = (bf16)m4[i];
        mqh[n >> 1][4 * (n & 1) + i] = hv;
        mql[n >> 1][4 * (n & 1) + i] = (bf16)(m4[i] - (float)hv);
      }
    }
    __syncthreads();  // MQ0 / MQ1 reads done; the solve's scratch reuses them

    // ---- T = (I + A)^{-1} (A = AF + AF2), blockwise over 16x16 tiles on fp32
    // MFMA 16x16x4 by waves 0..3.  Every product is (LDS matrix, row-major, read
    // 16 bytes per lane as the A operand) x (register matrix in the accumulator
    // layout, which is the B operand layout): lane l supplies k = 4g + s in MFMA s.
    {
      auto arow = [&](const float* M, int ld) -> floatx4 {
        return *reinterpret_cast<const floatx4*>(M + tr * ld + 4 * g);
      };
      auto mm16 = [&](const floatx4& a, const floatx4& x) -> floatx4 {
        floatx4 yv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) yv = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], x[s], yv, 0, 0, 0);
        return yv;
      };
      if (hh == 0) {
        // diagonal block of tile w: N = A_ww strictly lower, N^16 = 0, so
        // (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8)
        const int b0 = 16 * w;
        float* S2 = SCR + w * 512;
        float* S4 = S2 + 256;
        floatx4 nB;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          nB[i] = AF[(b0 + 4 * g + i) * ldA + b0 + tr] + AF2[(b0 + 4 * g + i) * ldA + b0 + tr];
        const floatx4 aN = arow(AF + b0 * ldA + b0, ldA) + arow(AF2 + b0 * ldA + b0, ldA);
        const floatx4 n2 = mm16(aN, nB);
#pragma unroll
        for (int i = 0; i < 4; ++i) S2[(4 * g + i) * 16 + tr] = n2[i];
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const floatx4 a2 = arow(S2, 16);
        const floatx4 n4 = mm16(a2, n2);
#pragma unroll
        for (int i = 0; i < 4; ++i) S4[(4 * g + i) * 16 + tr] = n4[i];
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const floatx4 a4 = arow(S4, 16);
        floatx4 X = mm16(a4, n4);  // N^8
#pragma unroll
        for (int i = 0; i < 4; ++i) X[i] += (4 * g + i == tr) ? 1.f : 0.f;
        X += mm16(a4, X);
        X += mm16(a2, X);
        X -= mm16(aN, X);
#pragma unroll
        for (int i = 0; i < 4; ++i) TF[(b0 + 4 * g + i) * ldA + b0 + tr] = X[i];
      }
      __syncthreads();
      // below the diagonal by distance d: T_mn = -T_mm sum_{j=n}^{m-1} A_mj T_jn
#pragma unroll
      for (int d = 1; d < 4; ++d) {
        const int m = w, n = w - d;
        if (hh == 0 && n >= 0) {
          floatx4 Xs = {0.f, 0.f, 0.f, 0.f};
          for (int j = n; j < m; ++j) {
            floatx4 tB;
#pragma unroll
            for (int i = 0; i < 4; ++i) tB[i] = TF[(16 * j + 4 * g + i) * ldA + 16 * n + tr];
            Xs += mm16(arow(AF + 16 * m * ldA + 16 * j, ldA) + arow(AF2 + 16 * m * ldA + 16 * j, ldA), tB);
          }
          const floatx4 Y = mm16(arow(TF + 16 * m * ldA + 16 * m, ldA), Xs);
#pragma unroll
          for (int i = 0; i < 4; ++i) TF[(16 * m + 4 * g + i) * ldA + 16 * n + tr] = -Y[i];
        }
        __syncthreads();
      }
    }

    // ---- TB = T Diag(beta) (split, [r][j]) and the V slice ([token][value])
#pragma unroll
    for (int it = 0; it < CH * CH / 4 / NTH; ++it) {
      const int idx = tid + NTH * it;
      const int rr = idx >> 4, j0 = 4 * (idx & 15);
      const floatx4 t4 = *reinterpret_cast<const floatx4*>(TF + rr * ldA + j0);
      const floatx4 b4 = *reinterpret_cast<const floatx4*>(BS + j0);
      float x4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x4[e] = (j0 + e <= rr) ? t4[e] * b4[e] : 0.f;
      st_split4(TB + rr * ldT + j0, loT, x4);
    }
    // the next chunk's gate values (fetched after the scan; only k and q were
    // fetched after them) become alpha here, off the scan's dependency chain
    if (more) gate_finish_blocks<KIND, NKH>(gate, gsc, in.a);
    *reinterpret_cast<uint4v*>(VS + r * ldV + vh0 + 8 * g) = in.v;
    if (more) load_part(nxt, in, 3);
    __syncthreads();

    // ---- W^T = (Gamma*K)^T (T Diag b)^T for this tile's tokens, kept as the
    // split operand of W S: all channels, computed by both waves of the pair.
    // U = T Diag(b) V for this wave's 32 value columns.
    bf16x8 wh[NCHT / 2], wl[NCHT / 2];
    floatx4 accU[NCH];
    {
      bf16x8 tbh[2], tbl[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        tbh[kb] = frag_ld(TB, ldT, r, 32 * kb, g);
        tbl[kb] = frag_ld(TB + loT, ldT, r, 32 * kb, g);
      }
#pragma unroll
      for (int ct = 0; ct < NCHT; ++ct) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb > (w >> 1)) continue;
          // split T Diag(b) only: (Gamma*K) single-rounded is within the error
          // budget of this product, the T side is not
          const bf16x8 ah = frag_tr(GK, ldG, 16 * ct, 32 * kb + 8 * g, 32 * kb + 8 * g + 4, tr);
          acc = mfma_bf16(ah, tbh[kb], acc);
          acc = mfma_bf16(ah, tbl[kb], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16 hv = (bf16)acc[i];
          wh[ct >> 1][4 * (ct & 1) + i] = hv;
          wl[ct >> 1][4 * (ct & 1) + i] = (bf16)(acc[i] - (float)hv);
        }
      }
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int vc = vh0 + 16 * c;
        accU[c] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (kb > (w >> 1)) continue;
          const bf16x8 b = frag_tr(VS, ldV, vc, 32 * kb + 8 * g, 32 * kb + 8 * g + 4, tr);
          accU[c] = mfma_bf16(tbh[kb], b, accU[c]);
          accU[c] = mfma_bf16(tbl[kb], b, accU[c]);
        }
      }
    }
    __syncthreads();  // TB / VS / GK reads done; ST, PT and KT overwrite the region

    // ---- Ktil ([token][channel], split) and the state as the B operand of W S
    // and (Gamma*Q) S: [value][channel position], position 32kb + 8g + 4h + i
    // holds channel 32kb + 16h + 4g + i
#pragma unroll
    for (int kk = 0; kk < NKH; ++kk) {
      const int kb = NKH * hh + kk;
      // whole 32-bit words (element pairs) of the packed registers
      const uint4v uh = __builtin_bit_cast(uint4v, kth[kk]);
      const uint4v ul = __builtin_bit_cast(uint4v, ktl[kk]);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        *reinterpret_cast<uint2v*>(KT + r * ldG + 32 * kb + 16 * hf + 4 * g) =
            uint2v{uh[2 * hf], uh[2 * hf + 1]};
        *reinterpret_cast<uint2v*>(KT + r * ldG + 32 * kb + 16 * hf + 4 * g + loG) =
            uint2v{ul[2 * hf], ul[2 * hf + 1]};
      }
    }
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
      const int c0r = w * RPW + rt * 16;
      const int pos = 32 * (c0r >> 5) + 8 * g + 4 * ((c0r >> 4) & 1);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        float x4[4] = {Sacc[rt][c][0], Sacc[rt][c][1], Sacc[rt][c][2], Sacc[rt][c][3]};
        st_split4(ST + (vh0 + 16 * c + tr) * ldS + pos, loS, x4);
      }
    }
    __syncthreads();

    // ---- P = U - W S and O = (Gamma*Q) S for this tile's tokens, this wave's
    // columns; each product is accumulated as two chains, the low and the high
    // channel half, added at the end (the order the state pass uses)
    floatx4 accO[NCH];
    {
      const bool wsplit = w_split_chunk<DK>(GC, lane_x);
      floatx4 accW[NCH], accW2[NCH], accO2[NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        accW[c] = floatx4{0.f, 0.f, 0.f, 0.f};
        accO[c] = floatx4{0.f, 0.f, 0.f, 0.f};
        accW2[c] = floatx4{0.f, 0.f, 0.f, 0.f};
        accO2[c] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 aq = frag_ld(QT, ldQ, r, 32 * kb, g);
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const bf16x8 bh = frag_ld(ST, ldS, vh0 + 16 * c + tr, 32 * kb, g);
          const bf16x8 bl = frag_ld(ST + loS, ldS, vh0 + 16 * c + tr, 32 * kb, g);
          floatx4& aw = kb < NKH ? accW[c] : accW2[c];
          floatx4& ao = kb < NKH ? accO[c] : accO2[c];
          aw = mma_w(wsplit, wh[kb], wl[kb], bh, bl, aw);
          ao = mfma_bf16(aq, bh, ao);
          ao = mfma_bf16(aq, bl, ao);
        }
      }
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        accW[c] = accW[c] + accW2[c];
        accO[c] = accO[c] + accO2[c];
      }
      // P to LDS as [value][token position]; token 32kb + 16h + 4g + i sits at
      // position 32kb + 8g + 4h + i (the order of the Mqk^T operand)
      const int pos = 32 * (w >> 1) + 8 * g + 4 * (w & 1);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        float x4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x4[i] = accU[c][i] - accW[c][i];
        st_split4(PT + (vh0 + 16 * c + tr) * ldP + pos, loP, x4);
      }
    }
    __syncthreads();

    // ---- tile 0 of the first chunk keeps Gamma*Q split: its low halves times
    // the state's high halves (as the two-pass state pass adds them, before
    // Mqk P)
    if (w == 0 && cur.c0 == 0) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 aql = frag_ld(QTL, ldQ, r, 32 * kb, g);
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          accO[c] = mfma_bf16(aql, frag_ld(ST, ldS, vh0 + 16 * c + tr, 32 * kb, g), accO[c]);
      }
    }
    // ---- O += Mqk P; store o
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb > (w >> 1)) continue;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const bf16x8 bh = frag_ld(PT, ldP, vh0 + 16 * c + tr, 32 * kb, g);
        const bf16x8 bl = frag_ld(PT + loP, ldP, vh0 + 16 * c + tr, 32 * kb, g);
        accO[c] = mma_ab(mqh[kb], mql[kb], bh, bl, accO[c]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 16 * w + 4 * g + i;
      if (rr < nv) {
        TOut* orow = o + ((size_t)(tok0 + rr) * H + h) * DV + vcol0 + vh0 + tr;
#pragma unroll
        for (int c = 0; c < NCH; ++c) __builtin_nontemporal_store((TOut)accO[c][i], orow + 16 * c);
      }
    }

    // ---- S = Diag(Gamma_C) S + Ktil^T P
    {
      bf16x8 bph[2][NCH], bpl[2][NCH];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          bph[kb][c] = frag_ld(PT, ldP, vh0 + 16 * c + tr, 32 * kb, g);
          bpl[kb][c] = frag_ld(PT + loP, ldP, vh0 + 16 * c + tr, 32 * kb, g);
        }
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) {
        const int c0r = w * RPW + rt * 16;
        const floatx4 gc = *reinterpret_cast<const floatx4*>(GC + c0r + 4 * g);
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) Sacc[rt][c][i] *= gc[i];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          // Ktil^T rows c0r.., token k-slots in the same order as P's positions
          const bf16x8 ah = frag_tr(KT, ldG, c0r, 32 * kb + 4 * g, 32 * kb + 16 + 4 * g, tr);
          const bf16x8 al = frag_tr(KT + loG, ldG, c0r, 32 * kb + 4 * g, 32 * kb + 16 + 4 * g, tr);
#pragma unroll
          for (int c = 0; c < NCH; ++c)
            Sacc[rt][c] = mma_ab(ah, al, bph[kb][c], bpl[kb][c], Sacc[rt][c]);
        }
      }
    }
    cur = nxt;
    have = more;
  }

  if (s_final) {
    float* sf = s_final + ((size_t)seq * H + h) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = w * RPW + rt * 16 + 4 * g + i;
          sf[(size_t)row * DV + vcol0 + vh0 + c * 16 + tr] = Sacc[rt][c][i];
        }
  }
}

template <typename K>
hipError_t set_lds(K kern, int bytes) {
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

// one instantiation per gate kind: the alpha path carries no gate code, and the
// transforms of the other kinds run where their values are used
template <int DK, typename TOut, int KIND>
hipError_t launch_fused_k(const PrefillArgs& a) {
  using L = Plan<DK, BV>;
  auto kern = prefill_bf16_kernel<DK, TOut, KIND>;
  static bool attr_set = false;  // per instantiation; idempotent if raced
  if (!attr_set) {
    if (hipError_t e = set_lds(kern, L::total); e != hipSuccess) return e;
    attr_set = true;
  }
  const int grid = a.n_seq * a.H * (a.Dv / BV);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTH), L::total, (hipStream_t)a.stream,
                     (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.gate, a.beta,
                     a.initial_state, a.final_state, (TOut*)a.o, a.cu_seqlens, a.n_seq, a.T, a.H,
                     a.Dv);
  return hipGetLastError();
}

template <int DK, typename TOut>
hipError_t launch_fused(const PrefillArgs& a) {
  switch (a.gate.kind) {
    case GATE_LOG: return launch_fused_k<DK, TOut, GATE_LOG>(a);
    case GATE_BOUNDED: return launch_fused_k<DK, TOut, GATE_BOUNDED>(a);
    case GATE_SCALAR: return launch_fused_k<DK, TOut, GATE_SCALAR>(a);
    case GATE_NONE: return launch_fused_k<DK, TOut, GATE_NONE>(a);
    default: return launch_fused_k<DK, TOut, GATE_ALPHA>(a);
  }
}

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

size_t table_bytes(int n_seq) { return ((size_t)(n_seq + 1) * 4 + 255) / 256 * 256; }
size_t carry_bytes(int n_seq, int H, int Dk, int Dv) {
  return ((size_t)n_seq * H * Dk * Dv * 4 + 255) / 256 * 256;
}

}  // namespace

bool prefill_supported(bool qkv_bf16, int Dk, int Dv) {
  if (!(Dv == 64 || Dv == 128)) return false;
  if (qkv_bf16) return Dk == 64 || Dk == 128;
  return Dk == 64 || Dk == 128;  // fp32 inputs: the fp32-MFMA chunk kernel (Dk = 64) or the
                                // token recurrence (Dk = 128)
}

// Workspace of the two-pass schedule: the chunk table (packed calls), a state
// carried from window to window when the caller passes no final_state, and the
// operand blocks of one window -- at most WIN_CHUNKS + n_seq chunks start in a
// window of WIN_CHUNKS * 64 packed tokens (one partial chunk per sequence).
// Independent of the sequence length.
size_t prefill_two_pass_bytes(int n_seq, int H, int Dk, int Dv) {
  if (n_seq <= 0 || H <= 0 || !prefill_supported(true, Dk, Dv)) return 0;
  const long long items = (long long)(WIN_CHUNKS + n_seq) * H;
  if (items > 0x7fffffffLL) return 0;
  return table_bytes(n_seq) + carry_bytes(n_seq, H, Dk, Dv) +
         (size_t)items * prefill_image_bytes(Dk, Dv);
}

// The segmented schedule adds, after the two-pass workspace, the segments'
// entry states [nseg][n_seq][H][Dk][Dv] and the summaries [M | b]
// [nseg - 1][n_seq][H][Dk][Dk + Dv], fp32.
size_t seg_in_bytes(int n_seq, int H, int Dk, int Dv, int nseg) {
  return ((size_t)nseg * n_seq * H * Dk * Dv * 4 + 255) / 256 * 256;
}

size_t prefill_segmented_bytes(int n_seq, int H, int Dk, int Dv, int nseg) {
  const size_t base = prefill_two_pass_bytes(n_seq, H, Dk, Dv);
  if (base == 0 || nseg < 1 || nseg > kMaxSegments) return 0;
  if (nseg == 1) return base;
  return base + seg_in_bytes(n_seq, H, Dk, Dv, nseg) +
         (size_t)(nseg - 1) * n_seq * H * Dk * (Dk + Dv) * 4;
}

size_t device_mem() {
  static size_t mem[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (mem[dev] == 0) {
    size_t b = 0;
    if (hipDeviceTotalMem(&b, dev) != hipSuccess) b = 0;
    mem[dev] = b;
  }
  return mem[dev];
}

bool prefill_two_pass_preferred(int n_seq, long long tokens, int H, int Dk, int Dv) {
  if (n_seq <= 0 || H <= 0 || !prefill_supported(true, Dk, Dv)) return false;
  // The fused kernel runs one workgroup per (sequence, head, 64-wide value
  // slice) and repeats the state-independent work once per slice; the two-pass
  // schedule does that work once per (chunk, head) on every compute unit.  It
  // pays off when the fused grid leaves the device under-filled and the
  // sequences are several chunks long, and is chosen only while its workspace
  // stays within 1/16 of device memory (and 16 GiB).
  const long long grid = (long long)n_seq * H * (Dv / BV);
  if (!(grid < 2LL * device_cus() && tokens / n_seq >= 4 * CH)) return false;
  const size_t need = prefill_two_pass_bytes(n_seq, H, Dk, Dv);
  size_t cap = device_mem() / 16;
  if (cap == 0 || cap > (size_t(16) << 30)) cap = size_t(16) << 30;
  return need > 0 && need <= cap;
}

int prefill_segments_preferred(int n_seq, long long tokens, int H, int Dk, int Dv) {
  if (!prefill_two_pass_preferred(n_seq, tokens, H, Dk, Dv)) return 1;
  // The state pass runs n_seq * H * Dv / 64 workgroups per window, each walking
  // up to 64 chunks in order; with few of them most compute units idle.
  // Segments multiply the workgroups: the summary pass runs (nseg - 1) * grid *
  // (Dk + Dv) / Dv of them (one per compute unit fits), the state pass nseg *
  // grid.  The largest nseg whose summary pass fits the device in one round was
  // the fastest on MI355X at 12, 24, 48 and 96 heads (within 2%), and only
  // while a sequence has at least 4 chunks per segment in a window.
  const long long grid = (long long)n_seq * H * (Dv / BV);
  long long ns = 1 + (long long)device_cus() * Dv / (grid * (Dk + Dv));
  const long long per_seq = tokens / n_seq / CH;  // chunks per sequence
  const long long win = per_seq < WIN_CHUNKS ? per_seq : WIN_CHUNKS;
  if (ns > win / 4) ns = win / 4;
  if (ns > 8) ns = 8;
  return ns < 2 ? 1 : (int)ns;
}

// The layer prefill after the recurrence: the conv state handed on, and the
// epilogue over o.
hipError_t layer_tail(const PrefillArgs& a, long long total) {
  const LayerPro& p = *a.pro;
  PrologueArgs c{};
  c.xq = a.q; c.xk = a.k; c.xv = a.v; c.bf16 = a.qkv_bf16;
  c.st_in = p.st_in; c.st_out = p.st_out; c.cu_seqlens = a.cu_seqlens; c.n_seq = a.n_seq;
  c.Tseq = a.T; c.total = total; c.H = a.H; c.Dk = a.Dk; c.Dv = a.Dv; c.stream = a.stream;
  if (hipError_t e = launch_conv_state(c); e != hipSuccess) return e;
  EpilogueArgs ep{};
  ep.o = a.o; ep.o_bf16 = a.o_bf16; ep.g = p.out.g; ep.g_bf16 = a.qkv_bf16; ep.w = p.out.w;
  ep.eps = p.out.eps; ep.y = p.y; ep.y_bf16 = p.y_bf16; ep.rows = total; ep.H = a.H;
  ep.Dv = a.Dv; ep.stream = a.stream;
  return launch_epilogue(ep);
}

hipError_t launch_prefill(const PrefillArgs& a) {
  if (!a.qkv_bf16) return a.Dk == 64 ? launch_prefill_f32(a) : launch_prefill_recurrent(a);
  const bool varlen = a.cu_seqlens != nullptr;
  // packed tokens in all (dense: n_seq sequences of T tokens back to back)
  const long long total = varlen ? (long long)a.T : (long long)a.n_seq * a.T;
  const size_t need = prefill_two_pass_bytes(a.n_seq, a.H, a.Dk, a.Dv);
  SegmentArgs sg;
  if (a.nseg > 1) {  // the caller checked the workspace size
    if (a.workspace_bytes < prefill_segmented_bytes(a.n_seq, a.H, a.Dk, a.Dv, a.nseg))
      return hipErrorInvalidValue;
    sg.nseg = a.nseg;
    sg.seg_in = reinterpret_cast<float*>(static_cast<unsigned char*>(a.workspace) + need);
    sg.summ = reinterpret_cast<float*>(static_cast<unsigned char*>(a.workspace) + need +
                                       seg_in_bytes(a.n_seq, a.H, a.Dk, a.Dv, a.nseg));
  }
  if (need == 0 || !a.workspace || a.workspace_bytes < need || total == 0) {
    // the layer prefill's prologue lives in the two-pass first pass: without
    // tokens only the states are handed through
    if (a.pro && total > 0) return hipErrorInvalidValue;
    hipError_t e = a.Dk == 128 ? (a.o_bf16 ? launch_fused<128, bf16>(a) : launch_fused<128, float>(a))
                               : (a.o_bf16 ? launch_fused<64, bf16>(a) : launch_fused<64, float>(a));
    if (e == hipSuccess && a.pro) e = layer_tail(a, total);
    return e;
  }
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  int32_t* chunk_off = varlen ? reinterpret_cast<int32_t*>(ws) : nullptr;
  float* scratch = reinterpret_cast<float*>(ws + table_bytes(a.n_seq));
  unsigned char* img = ws + table_bytes(a.n_seq) + carry_bytes(a.n_seq, a.H, a.Dk, a.Dv);
  float* carry = a.final_state ? a.final_state : scratch;
  const int cap = WIN_CHUNKS + a.n_seq;
  if (varlen) {
    const long long all = (total + CH - 1) / CH + a.n_seq;
    if (hipError_t e = launch_chunk_table(a.cu_seqlens, a.n_seq,
                                          (int)(all < 0x7fffffffLL ? all : 0x7fffffffLL),
                                          chunk_off, a.stream);
        e != hipSuccess)
      return e;
  }
  int grid = device_cus() * prefill_prep_per_cu();
  if ((long long)cap * a.H < grid) grid = cap * a.H;
  const long long win = (long long)WIN_CHUNKS * CH;
  for (long long t0 = 0; t0 < total; t0 += win) {
    hipError_t e = launch_prefill_prep(a, img, chunk_off, t0, t0 + win, cap, grid);
    if (e != hipSuccess) return e;
    e = launch_prefill_state(a, img, chunk_off, carry, t0, t0 + win, cap, sg);
    if (e != hipSuccess) return e;
  }
  if (a.pro) return layer_tail(a, total);
  return hipSuccess;
}

}  // namespace kda
