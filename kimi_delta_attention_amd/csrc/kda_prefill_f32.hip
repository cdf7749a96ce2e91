// kda_prefill_f32.hip -- chunked KDA prefill for fp32 inputs (gfx950, fp32 MFMA).
//
// The chunk form of the recurrence S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1}
// + b_t k_t v_t^T, o_t = S_t^T q_t ("Kimi Delta Attention 完全拆解", section
// "chunk 内并行、chunk 间递推"; "Kimi K3 的 KDA" section 5; "Kimi K3模型架构详解"
// sections 3.4-3.5).  For a 64-token chunk with entry state S and in-chunk
// cumulative decay Gamma_r = prod_{s<=r} a_s (per key channel):
//
//   A_rj  = b_r sum_c k_rc k_jc Gamma_rc / Gamma_jc           (j < r)
//   T     = (I + A)^{-1}                                       (UT transform)
//   W     = T Diag(b) (Gamma * K),   U = T Diag(b) V
//   P     = U - W S                                            (pseudo-values)
//   Mqk_rj = sum_c q_rc k_jc Gamma_rc / Gamma_jc              (j <= r)
//   O     = (Gamma * Q) S + Mqk P
//   S'    = Diag(Gamma_C) S + Ktil^T P,  Ktil_j = (Gamma_C / Gamma_j) * k_j
//
// (P's rows are the per-token corrections u_r = b_r (v_r - Sbar_r^T k_r).)
// The decay ratios inside A and Mqk are split over 16-token tiles: with
// P_r = product of a from the start of r's tile up to r, a pair (r in tile m,
// j in tile n) uses left factor P_r (<= 1) and right factor (E_n / P_j) times
// the whole-tile decays E_i of the tiles strictly between (all <= 1), and the
// diagonal tile uses 1 / P_j, bounded by the decay of one 16-token tile (the
// tiling the bounded gate of "Kimi K3 的 KDA" section 6 is made for).
//
// One workgroup (4 waves) owns (sequence, head, 64-wide value slice) and walks
// the chunks in order; the state slice lives in MFMA accumulators for the
// whole sequence.  This instantiation serves fp32 inputs (Dk = 64): every
// product runs on fp32 MFMA 16x16x4 with operands staged in LDS, so results
// stay within fp32 rounding of the recurrence.  (The template still carries the
// split-bf16 operand machinery; bf16 inputs use the kernel in kda_prefill.hip.)
#include "kda_common.h"
#include "kda_internal.h"
#include "kda_layer.h"

namespace kda {
namespace f32path {

constexpr int CH = 64;   // chunk length
constexpr int NTH = 256; // threads per workgroup

// LDS layout.  Arrays are MFMA operands stored k-contiguous ([M][K] for A
// operands, [N][K] for B operands); a split array is its hi part followed by
// its lo part.  Arrays of different phases share space; the static_asserts
// check that arrays alive at the same time do not overlap.
template <int DK, int BV, bool F32OPS>
struct Layout {
  static constexpr int ES = F32OPS ? 4 : 2;
  static constexpr bool LO = !F32OPS;
  static constexpr int ldK = DK + 8;   // rows indexed by token, DK channels
  static constexpr int ldC = CH + 8;   // rows of 64 tokens
  static constexpr int ldA = CH + 4;   // fp32 A and T
  static constexpr int sz(int rows, int ld, bool lo) { return rows * ld * ES * (lo ? 2 : 1); }
  static constexpr int KL = sz(CH, ldK, false);
  static constexpr int QL = sz(CH, ldK, LO);
  static constexpr int RT = sz(160, ldK, LO);
  static constexpr int VT = sz(BV, ldC, false);
  static constexpr int AF = CH * ldA * 4;
  static constexpr int TF = CH * ldA * 4;
  static constexpr int MQ = sz(CH, ldC, LO);
  static constexpr int WO = sz(CH, ldK, LO);
  static constexpr int TB = sz(CH, ldC, LO);
  static constexpr int GK = sz(DK, ldC, LO);
  static constexpr int QT = sz(CH, ldK, false);
  static constexpr int KT = sz(DK, ldC, LO);
  static constexpr int ST = sz(BV, ldK, LO);
  static constexpr int PT = sz(BV, ldC, LO);
  // serial phase: MQ | WO | QT | KT | ST | PT
  static constexpr int oMQ = 0, oWO = oMQ + MQ, oQT = oWO + WO, oKT = oQT + QT, oST = oKT + KT,
                       oPT = oST + ST, endSerial = oPT + PT;
  // A / Mqk phase: KL | QL | RT ; V is parked in the P region
  static constexpr int oKL = 0, oQL = oKL + KL, oRT = oQL + QL, endA = oRT + RT;
  static constexpr int oVT = oPT;
  // triangular solve: T in the W region, A in the S region
  static constexpr int oTF = oWO, oAF = oST;
  // W / U phase: TB | GK from the Q region on
  static constexpr int oTB = oQT, oGK = oTB + TB;
  // fixed tail: per-tile decays E[4][DK], chunk decay gC[DK], beta[64]
  static constexpr int oES = endSerial > oVT + VT ? endSerial : oVT + VT;
  static constexpr int oGC = oES + 4 * DK * 4;
  static constexpr int oBS = oGC + DK * 4;
  static constexpr int total = oBS + CH * 4;
  static_assert(endA <= oVT, "phase-A operands overlap V");
  static_assert(TF <= WO && AF <= ST, "A/T placement");
  static_assert(oTB >= oTF + TF, "TB overlaps T");
  static_assert(oGK + GK <= oVT, "W-phase operands overlap V");
  static_assert(total <= 163840, "LDS budget (160 KiB)");
};

// Precision policy per product (bf16 path).  A is single-pass; U splits only
// the T side because V is exact in bf16; (Gamma*Q) S splits only S; every other
// product splits both operands.
struct Pol {
  static constexpr int A = P_SINGLE, M = P_SPLIT_AB, W = P_SPLIT_AB, U = P_SPLIT_A,
                       WS = P_SPLIT_AB, QS = P_SPLIT_B, MP = P_SPLIT_AB, KP = P_SPLIT_AB;
};

template <typename TIn>
__device__ __forceinline__ float ldf(const TIn* p, size_t i);
template <>
__device__ __forceinline__ float ldf<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ldf<bf16>(const bf16* p, size_t i) { return (float)p[i]; }

// Pairs of 16-token tiles (row tile, column tile) of A / Mqk computed by each
// wave; n < 0 marks an upper block the wave zeroes in Mqk instead.
__device__ __forceinline__ void pair_of(int w, int p, int& mm, int& n) {
  const int tab[4][3][2] = {{{0, 0}, {3, 0}, {3, 1}},
                            {{1, 0}, {1, 1}, {3, 2}},
                            {{2, 0}, {2, 1}, {0, -1}},
                            {{2, 2}, {3, 3}, {2, -3}}};
  mm = tab[w][p][0];
  n = tab[w][p][1];
}

template <int DK, int BV, bool F32OPS, typename TIn, typename TOut>
__global__ __launch_bounds__(NTH) void prefill_f32_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    Gate gate, const float* __restrict__ beta,
    const float* __restrict__ s_init, float* __restrict__ s_final, TOut* __restrict__ o,
    const int32_t* __restrict__ cu_seqlens, int n_seq, int T, int H, int DV) {
  using L = Layout<DK, BV, F32OPS>;
  using Ld = Lds<F32OPS>;
  using E = typename Ld::T;
  constexpr int NSEG = DK / 64;        // (tile, channel) segments per thread
  constexpr int TPC = NTH / DK;        // tiles covered by one pass of the threads
  constexpr int RPW = DK / 4;          // state rows per wave
  constexpr int RTW = RPW / 16;        // state row tiles per wave
  constexpr int NCT = BV / 16;         // value column tiles
  constexpr int NKB = DK / 32;         // k-blocks over the key axis
  constexpr int ldK = L::ldK, ldC = L::ldC, ldA = L::ldA;
  constexpr int loQL = CH * ldK, loRT = 160 * ldK, loMQ = CH * ldC, loWO = CH * ldK,
                loTB = CH * ldC, loGK = DK * ldC, loKT = DK * ldC, loST = BV * ldK,
                loPT = BV * ldC;

  extern __shared__ __align__(16) unsigned char smem[];
  E* KL = reinterpret_cast<E*>(smem + L::oKL);
  E* QL = reinterpret_cast<E*>(smem + L::oQL);
  E* RT = reinterpret_cast<E*>(smem + L::oRT);
  E* VT = reinterpret_cast<E*>(smem + L::oVT);
  float* AF = reinterpret_cast<float*>(smem + L::oAF);
  float* TF = reinterpret_cast<float*>(smem + L::oTF);
  E* MQ = reinterpret_cast<E*>(smem + L::oMQ);
  E* WO = reinterpret_cast<E*>(smem + L::oWO);
  E* TB = reinterpret_cast<E*>(smem + L::oTB);
  E* GK = reinterpret_cast<E*>(smem + L::oGK);
  E* QT = reinterpret_cast<E*>(smem + L::oQT);
  E* KT = reinterpret_cast<E*>(smem + L::oKT);
  E* ST = reinterpret_cast<E*>(smem + L::oST);
  E* PT = reinterpret_cast<E*>(smem + L::oPT);
  float* ESd = reinterpret_cast<float*>(smem + L::oES);  // [4][DK]
  float* GC = reinterpret_cast<float*>(smem + L::oGC);   // [DK]
  float* BS = reinterpret_cast<float*>(smem + L::oBS);   // [64]

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  // ---- work item: (sequence, head, value slice); the slices of one head are
  // placed on the same XCD (block ids are dealt round-robin over 8 XCDs).
  const int nsl = DV / BV;
  const int total = n_seq * H * nsl;
  int wid = blockIdx.x;
  if ((total & 7) == 0) wid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int sl = wid % nsl;
  const int h = (wid / nsl) % H;
  const int seq = wid / (nsl * H);
  long long start, len;
  if (cu_seqlens) {
    start = cu_seqlens[seq];
    len = (long long)cu_seqlens[seq + 1] - start;
  } else {
    start = (long long)seq * T;
    len = T;
  }
  const int vcol0 = sl * BV;

  // ---- state slice in accumulators: wave w owns key rows [w*RPW, (w+1)*RPW)
  floatx4 Sacc[RTW][NCT];
  {
    const float* si = s_init ? s_init + ((size_t)seq * H + h) * DK * DV : nullptr;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = w * RPW + rt * 16 + 4 * g4 + i;
          const int col = vcol0 + ct * 16 + l16;
          Sacc[rt][ct][i] = si ? si[(size_t)row * DV + col] : 0.f;
        }
  }

  const int ch = tid % DK;
  for (long long c0 = 0; c0 < len; c0 += CH) {
    const int nv = (int)(len - c0 < CH ? len - c0 : CH);
    const long long tok0 = start + c0;
    __syncthreads();  // previous chunk's serial phase is done with LDS

    // ---- load: k, q, alpha for this thread's (tile, channel) segments;
    // P = running product of alpha from the tile start.
    TIn kf[NSEG][16], qf[NSEG][16];  // exact input values (bf16 stays bf16)
    float Pf[NSEG][16], af[NSEG][16];
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      const int m = tid / DK + s * TPC;
      float run = 1.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = 16 * m + j;
        const bool ok = r < nv;
        const size_t off = ((size_t)(tok0 + r) * H + h) * DK + ch;
        kf[s][j] = ok ? k[off] : (TIn)0.f;
        qf[s][j] = ok ? q[off] : (TIn)0.f;
        const float a = ok ? gate_alpha1(gate, (size_t)(tok0 + r) * H + h, DK, ch, h) : 1.f;
        run = (j == 0) ? a : run * a;
        Pf[s][j] = run;
        af[s][j] = a;
      }
      ESd[m * DK + ch] = run;
    }
    if (tid < CH) BS[tid] = tid < nv ? beta[(size_t)(tok0 + tid) * H + h] : 0.f;
    {
      // V slice, transposed to [value][token] (B operand of U = T Diag(b) V)
      const int vv = tid & 63;
#pragma unroll 4
      for (int i = 0; i < CH / 4; ++i) {
        const int r = (tid >> 6) + 4 * i;
        const float x = (r < nv && vv < BV)
                            ? ldf(v, ((size_t)(tok0 + r) * H + h) * DV + vcol0 + vv) : 0.f;
        if (vv < BV) Ld::store_hi(VT, vv * ldC + r, x);
      }
    }
    __syncthreads();

    // ---- build the A / Mqk operands
    float pre[NSEG], post[NSEG], Em[NSEG];
    float Et[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) Et[i] = ESd[i * DK + ch];
    if (tid < DK) GC[ch] = Et[0] * Et[1] * Et[2] * Et[3];
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      const int m = tid / DK + s * TPC;
      float p = 1.f, po = 1.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < m) p *= Et[i];
        if (i > m) po *= Et[i];
      }
      pre[s] = p;
      post[s] = po;
      Em[s] = Et[m];
      // decay from after token j to the end of tile m, a product of decays
      // (no division by P, so nothing overflows however fast the decay)
      float sf[16];
      {
        float run = 1.f;
#pragma unroll
        for (int j = 15; j >= 0; --j) {
          sf[j] = run;
          run *= af[s][j];
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = 16 * m + j;
        const float kv = (float)kf[s][j];
        Ld::store_hi(KL, r * ldK + ch, kv * Pf[s][j]);
        Ld::store(QL, r * ldK + ch, loQL, (float)qf[s][j] * Pf[s][j]);
        // right operand rows for row tiles mm > m (the diagonal tile is summed
        // exactly below)
        float ke = kv * sf[j];                            // decayed to the end of tile m
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          if (mm <= m) continue;
          const int base = 8 * mm * (mm + 1);            // 16 * mm(mm+1)/2
          Ld::store(RT, (base + r) * ldK + ch, loRT, ke);
          ke *= Et[mm];
        }
      }
    }
    __syncthreads();

    // ---- A and Mqk: 16x16 tile pairs, K = DK
    floatx4 accA[3], accM[3];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      accA[p] = floatx4{0.f, 0.f, 0.f, 0.f};
      accM[p] = floatx4{0.f, 0.f, 0.f, 0.f};
      int mm, n;
      pair_of(w, p, mm, n);
      if (n < 0 || n == mm) continue;  // diagonal tiles: exact sums below
      const int base = 8 * mm * (mm + 1);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const auto ak = Ld::load(KL, ldK, 16 * mm + l16, 32 * kb, 0, false);
        const auto aq = Ld::load(QL, ldK, 16 * mm + l16, 32 * kb, loQL, wants_lo_a(Pol::M));
        const auto b = Ld::load(RT, ldK, base + 16 * n + l16, 32 * kb, loRT, true);
        accA[p] = mma<Pol::A>(ak, b, accA[p]);
        accM[p] = mma<Pol::M>(aq, b, accM[p]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      int mm, n;
      pair_of(w, p, mm, n);
      if (n < 0) {  // zero an upper block of Mqk that the output product reads
        const int nn = -n;
#pragma unroll
        for (int i = 0; i < 4; ++i) Ld::store(MQ, (16 * mm + 4 * g4 + i) * ldC + 16 * nn + l16, loMQ, 0.f);
        continue;
      }
      if (n == mm) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mm + 4 * g4 + i, j = 16 * n + l16;
        AF[r * ldA + j] = (j < r) ? BS[r] * accA[p][i] : 0.f;
        Ld::store(MQ, r * ldC + j, loMQ, (j <= r) ? accM[p][i] : 0.f);
      }
    }
    // ---- the diagonal tile of wave w's token tile, exactly: for tokens
    // j <= r of the tile, sum_c k_rc k_jc R and sum_c q_rc k_jc R with
    // R = alpha_{j+1} ... alpha_r of channel c, a running product (every factor
    // <= 1); lane c holds channel c of the tile (Dk = 64: one channel a lane)
    // and the wave sums over the channels.
    static_assert(NSEG == 1 && TPC == 4, "one (tile, channel) segment per thread");
    {
      const int m = w;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float kr = (float)kf[0][r], qr = (float)qf[0][r];
        float ca[16], cm[16];
        float R = 1.f;
#pragma unroll
        for (int j = r; j >= 0; --j) {
          const float t = (float)kf[0][j] * R;
          ca[j] = kr * t;
          cm[j] = qr * t;
          R *= af[0][j];
        }
        float av = 0.f, mv = 0.f;
#pragma unroll
        for (int j = 0; j <= r; ++j) {
          const float sa = wave_sum(ca[j]), sm = wave_sum(cm[j]);
          av = lane == j ? sa : av;
          mv = lane == 16 + j ? sm : mv;
        }
        const int rr = 16 * m + r;
        if (lane < 16) AF[rr * ldA + 16 * m + lane] = lane < r ? BS[rr] * av : 0.f;
        else if (lane < 32) Ld::store(MQ, rr * ldC + 16 * m + lane - 16, loMQ, lane - 16 <= r ? mv : 0.f);
      }
    }
    __syncthreads();

    // ---- T = (I + A)^{-1}: diagonal 16x16 blocks by substitution (fp32) ...
    if (lane < 16) {
      const int c = lane, b0 = 16 * w;
      float t[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) t[i] = (i == c) ? 1.f : 0.f;
#pragma unroll
      for (int jj = 0; jj < 15; ++jj)
#pragma unroll
        for (int i = jj + 1; i < 16; ++i) t[i] -= AF[(b0 + i) * ldA + b0 + jj] * t[jj];
#pragma unroll
      for (int i = 0; i < 16; ++i) TF[(b0 + i) * ldA + b0 + c] = t[i];
    }
    __syncthreads();
    // ... then blocks below the diagonal, by distance d from it:
    // T_mn = -T_mm sum_{j=n}^{m-1} A_mj T_jn  (fp32 MFMA 16x16x4)
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      const int m = w, n = w - d;
      if (n >= 0) {
        floatx4 X = {0.f, 0.f, 0.f, 0.f};
        for (int j = n; j < m; ++j)
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const float a = AF[(16 * m + l16) * ldA + 16 * j + 4 * g4 + s];
            const float b = TF[(16 * j + 4 * g4 + s) * ldA + 16 * n + l16];
            X = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, X, 0, 0, 0);
          }
        floatx4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float a = TF[(16 * m + l16) * ldA + 16 * m + 4 * g4 + s];
          Y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, X[s], Y, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) TF[(16 * m + 4 * g4 + i) * ldA + 16 * n + l16] = -Y[i];
      }
      __syncthreads();
    }

    // ---- TB = T Diag(b) (A operand of W and U) and (Gamma * K) as B operand
    for (int idx = tid; idx < CH * CH; idx += NTH) {
      const int r = idx >> 6, j = idx & 63;
      Ld::store(TB, r * ldC + j, loTB, (j <= r) ? TF[r * ldA + j] * BS[j] : 0.f);
    }
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      const int m = tid / DK + s * TPC;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        Ld::store(GK, ch * ldC + 16 * m + j, loGK, (float)kf[s][j] * (pre[s] * Pf[s][j]));
    }
    __syncthreads();

    // ---- W = TB (Gamma*K)  [64 x DK] and U = TB V [64 x BV]; wave w: row tile w
    floatx4 accU[NCT];
    {
      floatx4 accW[DK / 16];
#pragma unroll
      for (int ct = 0; ct < DK / 16; ++ct) accW[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) accU[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
      for (int kb = 0; kb <= (w >> 1); ++kb) {
        const auto a = Ld::load(TB, ldC, 16 * w + l16, 32 * kb, loTB, true);
#pragma unroll
        for (int ct = 0; ct < DK / 16; ++ct) {
          const auto b = Ld::load(GK, ldC, 16 * ct + l16, 32 * kb, loGK, wants_lo_b(Pol::W));
          accW[ct] = mma<Pol::W>(a, b, accW[ct]);
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const auto b = Ld::load(VT, ldC, 16 * ct + l16, 32 * kb, 0, false);
          accU[ct] = mma<Pol::U>(a, b, accU[ct]);
        }
      }
      __syncthreads();  // TB / GK / V reads done before the regions are reused
#pragma unroll
      for (int ct = 0; ct < DK / 16; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Ld::store(WO, (16 * w + 4 * g4 + i) * ldK + 16 * ct + l16, loWO, accW[ct][i]);
    }

    // ---- (Gamma * Q) and Ktil^T operands, and the state as B operand
#pragma unroll
    for (int s = 0; s < NSEG; ++s) {
      const int m = tid / DK + s * TPC;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = 16 * m + j;
        Ld::store_hi(QT, r * ldK + ch, (float)qf[s][j] * (pre[s] * Pf[s][j]));
        float sfx = 1.f;  // decay from after token j to the end of tile m
#pragma unroll
        for (int i = j + 1; i < 16; ++i) sfx *= af[s][i];
        Ld::store(KT, ch * ldC + r, loKT, (float)kf[s][j] * (sfx * post[s]));
      }
    }
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Ld::store(ST, (16 * ct + l16) * ldK + w * RPW + rt * 16 + 4 * g4 + i, loST, Sacc[rt][ct][i]);
    __syncthreads();

    // ---- serial part.  P = U - W S and O = (Gamma*Q) S  (wave w: token tile w)
    floatx4 accO[NCT];
    {
      floatx4 accWS[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        accWS[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
        accO[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const auto aw = Ld::load(WO, ldK, 16 * w + l16, 32 * kb, loWO, true);
        const auto aq = Ld::load(QT, ldK, 16 * w + l16, 32 * kb, 0, false);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const auto b = Ld::load(ST, ldK, 16 * ct + l16, 32 * kb, loST, true);
          accWS[ct] = mma<Pol::WS>(aw, b, accWS[ct]);
          accO[ct] = mma<Pol::QS>(aq, b, accO[ct]);
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          Ld::store(PT, (16 * ct + l16) * ldC + 16 * w + 4 * g4 + i, loPT, accU[ct][i] - accWS[ct][i]);
    }
    __syncthreads();

    // ---- O += Mqk P, store o
    for (int kb = 0; kb <= (w >> 1); ++kb) {
      const auto a = Ld::load(MQ, ldC, 16 * w + l16, 32 * kb, loMQ, true);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const auto b = Ld::load(PT, ldC, 16 * ct + l16, 32 * kb, loPT, true);
        accO[ct] = mma<Pol::MP>(a, b, accO[ct]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * g4 + i;
      if (r < nv) {
        TOut* orow = o + ((size_t)(tok0 + r) * H + h) * DV + vcol0 + l16;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) orow[16 * ct] = (TOut)accO[ct][i];
      }
    }

    // ---- S = Diag(Gamma_C) S + Ktil^T P
    {
      decltype(Ld::load(PT, ldC, 0, 0, loPT, true)) bp[2][NCT];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) bp[kb][ct] = Ld::load(PT, ldC, 16 * ct + l16, 32 * kb, loPT, true);
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) {
        float gc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) gc[i] = GC[w * RPW + rt * 16 + 4 * g4 + i];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i) Sacc[rt][ct][i] *= gc[i];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const auto a = Ld::load(KT, ldC, w * RPW + rt * 16 + l16, 32 * kb, loKT, true);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) Sacc[rt][ct] = mma<Pol::KP>(a, bp[kb][ct], Sacc[rt][ct]);
        }
      }
    }
  }

  if (s_final) {
    float* sf = s_final + ((size_t)seq * H + h) * DK * DV;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = w * RPW + rt * 16 + 4 * g4 + i;
          const int col = vcol0 + ct * 16 + l16;
          sf[(size_t)row * DV + col] = Sacc[rt][ct][i];
        }
  }
}

template <int DK, bool F32OPS, typename TIn, typename TOut>
static hipError_t launch_t(const PrefillArgs& a) {
  constexpr int BV = 64;
  using L = Layout<DK, BV, F32OPS>;
  auto kern = prefill_f32_kernel<DK, BV, F32OPS, TIn, TOut>;
  static bool attr_set = false;  // per instantiation; benign if raced (idempotent)
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, L::total);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int grid = a.n_seq * a.H * (a.Dv / BV);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTH), L::total, (hipStream_t)a.stream,
                     (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v, a.gate, a.beta,
                     a.initial_state, a.final_state, (TOut*)a.o, a.cu_seqlens, a.n_seq, a.T, a.H,
                     a.Dv);
  return hipGetLastError();
}

}  // namespace f32path

hipError_t launch_prefill_f32(const PrefillArgs& a) {
  using namespace f32path;
  return a.o_bf16 ? launch_t<64, true, float, bf16>(a) : launch_t<64, true, float, float>(a);
}

}  // namespace kda
