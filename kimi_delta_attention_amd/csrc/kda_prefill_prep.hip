// kda_prefill_prep.hip -- first pass of the two-pass chunked prefill (gfx950):
// everything of a 64-token chunk that does not depend on the entry state,
// written as the per-(chunk, head) operand images (Images<DK, DV>) that the
// state pass (kda_prefill_state.hip) reads.
//
// Chunk form ("Kimi Delta Attention 完全拆解", section "chunk 内并行、chunk 间
// 递推"; "Kimi K3 的 KDA" section 5): with Gamma_r the in-chunk cumulative decay
// of token r (per key channel),
//
//   A_rj   = b_r sum_c k_rc k_jc Gamma_rc / Gamma_jc   (j < r),   T = (I + A)^{-1}
//   W      = T Diag(b) (Gamma * K),   U = T Diag(b) V
//   Mqk_rj = sum_c q_rc k_jc Gamma_rc / Gamma_jc       (j <= r)
//   Ktil_j = (Gamma_C / Gamma_j) * k_j,  and Gamma * Q, Gamma_C
//
// with the decay ratios factored over 16-token tiles (P_r: product of a from
// the start of r's tile to r; E_n: whole-tile product), so that no factor
// exceeds one tile's decay.
//
// Work decomposition.  A workgroup of four waves owns one (chunk, head) item at
// a time and walks the window's items (a persistent grid, two workgroups per
// compute unit so that one item's barrier and memory stalls overlap the
// other's work).  Wave w takes token tile w of the item (tiles rotate with the
// item so that the heavy low tiles spread over the SIMDs); a lane holds token
// 16w + l%16 and, per 32-channel block kb, the 8 channels 32kb + 4g + {0..3}
// and 32kb + 16 + 4g + {0..3} (g = l/16), i.e. operand position 8g + 4h + i
// holds channel 16h + 4g + i.  The phases:
//   1. within-tile decay scan (16-lane DPP scan), tile decays E to LDS
//   2. operands: k P and (q P split) to LDS (A operands of A and Mqk, rows =
//      tokens), Gamma*K to LDS, Gamma*Q straight into the image, Ktil kept
//      in registers
//   3. A and Mqk for key tile n = w against query tiles m >= w: the key side
//      (k scaled by the ratio of tile decays, one variant per m) is the
//      register A operand, the query side the B operand read from LDS
//   4. Mqk image, T = (I + A)^{-1} (blockwise, fp32 MFMA)
//   5. T Diag(b) (split) and V to LDS; W^T and U images
//   6. Ktil through LDS into the transposed operand images
// Precision as in the fused kernel (kda_prefill.hip): every product and every
// rounding step is the same, in the same order, so both schedules give
// bitwise the same images and results.
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

using namespace frag;

constexpr int NTH_P = 256;  // four waves, one per token tile

// LDS plan (bytes).  Region R is reused phase by phase:
//   operands (2-3):  KL (k P, bf16), QLh / QLl (q P, split)      [token][position]
//   A, Mqk   (3-4):  AF (b A), MQ (Mqk)                           [token][token] fp32
//   solve    (4):    TF (T; its unused upper blocks hold the diagonal solve's
//                    N^2 / N^4 scratch)
//   T b      (5):    TB (T Diag(b), split); VS (V) is no longer staged
//   Ktil     (6):    KT (split)                                   [token][channel]
// GK (Gamma*K, [token][channel]) lives from phase 2 to 5; ES / GC / BS are small.
template <int DK, int DV>
struct PrepPlan {
  static constexpr int ldK = DK + 8, ldA = CH + 4, ldT = CH + 8, ldV = DV + 8;
  static constexpr int TILE = CH * ldK * 2;         // one [64][DK + 8] bf16 tile
  static constexpr int F32T = CH * ldA * 4;         // one [64][68] fp32 tile
  static constexpr int TBsz = CH * ldT * 2 * 2, VSsz = CH * ldV * 2;
  static constexpr int oKL = 0, oQLh = TILE, oQLl = 2 * TILE;
  static constexpr int oAF = 0, oMQ = F32T;
  static constexpr int oTB = 0, oVS = TBsz;
  static constexpr int oTF = (oVS + VSsz > 2 * F32T) ? oVS + VSsz : 2 * F32T;
  static constexpr int oKT = 0;
  static constexpr int m1 = 3 * TILE > oTF + F32T ? 3 * TILE : oTF + F32T;
  static constexpr int R = m1 > 2 * TILE ? m1 : 2 * TILE;
  static constexpr int oR0 = 0;
  static constexpr int oGK = R, oES = oGK + TILE, oGC = oES + 4 * DK * 4, oBS = oGC + DK * 4,
                       total = oBS + CH * 4;
  static_assert(total <= 81920, "two workgroups per compute unit");
  // With the layer prologue, at the start of an item: the chunk's raw inputs
  // XR ([64][SWP + 8] bf16, then the results) in R, and in GK the three
  // inputs before the chunk ([3][SWP] fp32) and the partial sums of squares
  // of the L2Norm ([4][64] fp32).
  static constexpr int SWP = 2 * DK + DV, ldX = SWP + 8;
  // and the item's conv taps ([SWP][4] fp32) after the plan
  static constexpr int oTP = total, totalP = oTP + SWP * 16;
  static_assert(totalP <= 81920, "two workgroups per compute unit with the prologue");
  static_assert(CH * ldX * 2 <= R && (3 * SWP + 4 * CH) * 4 <= TILE, "prologue staging");
  static_assert(oTB + TBsz <= oTF && oMQ + F32T <= oTF, "TF is read while TB, VS are written");
  static_assert((oQLh | oQLl | oMQ | oTF | oVS | oGK | oES | oGC | oBS) % 16 == 0, "alignment");
};

// The layer prologue in front of the first pass ("Kimi Delta Attention
// 完全拆解", section "一次 KDA 前向究竟发生了什么"): q, k = L2Norm(Swish(ShortConv
// (x))), v = Swish(ShortConv(x)), computed from the projections' outputs as
// the chunk is loaded, so that q, k and v never reach memory.  The raw rows
// go through LDS for the convolution's three previous inputs (the rows before
// the chunk from the sequence's previous chunk or its conv state); the
// results are rounded to bf16, as the standalone prologue stores them.
struct ProArgs {
  ConvArgs conv;
  const float* st_in;  // [n_seq, 3, H, 2 Dk + Dv] fp32 or null (zeros)
};

// b x + b y with both products rounded: the fused kernel scales each channel
// half separately and adds them later
__device__ __forceinline__ float scaled_sum(float b, float x, float y) { return b * x + b * y; }

template <int DK, int DV, int KIND, bool PRO>
__global__ __launch_bounds__(NTH_P, 2) void prefill_prep_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    Gate gate, const float* __restrict__ beta,
    const int32_t* __restrict__ cu_seqlens, int n_seq, int T, int H, unsigned char* __restrict__ img,
    const int32_t* __restrict__ chunk_off, long long tok_lo, long long tok_hi, int cap, ProArgs pa) {
  using L = PrepPlan<DK, DV>;
  using IM = Images<DK, DV>;
  constexpr int NKB = DK / 32;   // 32-channel blocks
  constexpr int NKH = NKB / 2;   // blocks of one channel half
  constexpr int NCHT = DK / 16;  // 16-channel tiles
  constexpr int NVT = DV / 16;   // 16-value tiles
  constexpr int NVL = DV / 32;   // 16-byte v loads per lane
  constexpr int ldK = L::ldK, ldA = L::ldA, ldT = L::ldT;
  constexpr int loK = CH * ldK, loT = CH * ldT;

  extern __shared__ __align__(16) unsigned char smem[];
  bf16* KL = reinterpret_cast<bf16*>(smem + L::oKL);
  bf16* QLh = reinterpret_cast<bf16*>(smem + L::oQLh);
  bf16* QLl = reinterpret_cast<bf16*>(smem + L::oQLl);
  float* AF = reinterpret_cast<float*>(smem + L::oAF);
  float* MQ = reinterpret_cast<float*>(smem + L::oMQ);
  float* TF = reinterpret_cast<float*>(smem + L::oTF);
  bf16* TB = reinterpret_cast<bf16*>(smem + L::oTB);
  bf16* KT = reinterpret_cast<bf16*>(smem + L::oKT);
  bf16* GK = reinterpret_cast<bf16*>(smem + L::oGK);
  float* ES = reinterpret_cast<float*>(smem + L::oES);  // [4][DK] tile decays
  float* GC = reinterpret_cast<float*>(smem + L::oGC);  // [DK] chunk decay
  float* BS = reinterpret_cast<float*>(smem + L::oBS);  // [64] beta
  bf16* XR = reinterpret_cast<bf16*>(smem + L::oR0);    // prologue raw rows [64][ldX]
  float* HI = reinterpret_cast<float*>(smem + L::oGK);  // prologue HIST [3][SWP]
  float* TP = reinterpret_cast<float*>(smem + L::oTP);  // prologue taps [SWP][4]
  constexpr int SWP = L::SWP, ldX = L::ldX;

  const int w4 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // items of this window: chunks that start in [tok_lo, tok_hi), head-minor
  const int ci_lo = chunks_before(tok_lo, cu_seqlens, chunk_off, n_seq, T);
  int nc = chunks_before(tok_hi, cu_seqlens, chunk_off, n_seq, T) - ci_lo;
  if (nc > cap) nc = cap;  // reached only if cu_seqlens is not monotone
  const int n_items = nc > 0 ? nc * H : 0;

  // One item: chunk ci of head hd; its first token and valid tokens.
  struct Item {
    long long tok0, start;  // first token of the chunk, of its sequence
    int nv, hd, seq;
  };
  auto locate = [&](int item) {
    const int ci = ci_lo + item / H;
    Item d;
    d.hd = item - (ci - ci_lo) * H;
    long long st, ln, cc;
    if (chunk_off) {
      int lo = 0, hi = n_seq - 1;  // last sequence whose first chunk is <= ci
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunk_off[mid] <= ci) lo = mid;
        else hi = mid - 1;
      }
      st = cu_seqlens[lo];
      ln = (long long)cu_seqlens[lo + 1] - st;
      cc = (long long)(ci - chunk_off[lo]) * CH;
      d.seq = lo;
    } else {
      const int nch = (T + CH - 1) / CH;
      const int sq = ci / nch;
      st = (long long)sq * T;
      ln = T;
      cc = (long long)(ci - sq * nch) * CH;
      d.seq = sq;
    }
    d.start = st;
    d.tok0 = st + cc;
    d.nv = (int)(ln - cc < CH ? ln - cc : CH);
    return d;
  };
  // k, q, gate values (as stored) of this lane's token and channels, and beta;
  // token tile (w4 + item) & 3.  Loads only, straight into the registers that
  // hold them until the item starts (order_in and finish_in use them there),
  // so that a prefetch waits for nothing: buffer loads through descriptors
  // that span the chunk's nv tokens read zero past them, with no select.
  uint4v kr[NKB], qr[NKB];  // raw 16-byte pieces (order_in)
  floatx4 ain[NKB][2];      // gate values as stored (finish_in)
  float bt = 0.f;
  auto rsrc = [](const void* base, long long bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
  };
  auto load_in = [&](int item, const Item& d, int ln) {
    const int gl = ln >> 4;
    const int r = 16 * ((w4 + item) & 3) + (ln & 15);
    const size_t row0 = (size_t)d.tok0 * H + d.hd;  // (first token, head)
    const long long rows = (long long)d.nv * H;    // rows the chunk's tokens span
    const int ro = r * H;                           // this lane's row after row0
    const auto rk = rsrc(k + row0 * DK, rows * DK * 2);
    const auto rq = rsrc(q + row0 * DK, rows * DK * 2);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      // k and q in 16 bytes per lane: row gl of the wave reads channels
      // 8 (gl >> 1) + 16 (gl & 1) .. + 8 of the block, so a token's 32
      // channels come in one 64-byte piece (order_in puts them in place)
      const int c8 = 32 * kb + 8 * (gl >> 1) + 16 * (gl & 1);
      kr[kb] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(rk, (ro * DK + c8) * 2, 0, 0));
      qr[kb] = __builtin_bit_cast(uint4v, __builtin_amdgcn_raw_buffer_load_b128(rq, (ro * DK + c8) * 2, 0, 0));
    }
    if constexpr (KIND == GATE_SCALAR) {
      const auto rg = rsrc(gate.g + row0, rows * 4);
      ain[0][0][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, ro * 4, 0, 0));
    } else if constexpr (KIND != GATE_NONE) {
      const auto rg = rsrc(gate.g + row0 * DK, rows * DK * 4);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          ain[kb][hf] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        rg, (ro * DK + 32 * kb + 16 * hf + 4 * gl) * 4, 0, 0));
    }
    bt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(beta + row0, rows * 4), ro * 4, 0, 0));
  };
  // alpha of this lane's token and channels (rows past the chunk's end: the
  // gate value whose alpha is 1)
  float Pv[NKB][8];
  auto finish_in = [&](int hd, bool okc) {
    if constexpr (KIND == GATE_SCALAR) {
      const float x = okc ? ain[0][0][0] : 1.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) ain[kb][hf] = floatx4{x, x, x, x};
    } else if constexpr (KIND == GATE_NONE) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) ain[kb][hf] = floatx4{1.f, 1.f, 1.f, 1.f};
    } else {
      constexpr float f = KIND == GATE_LOG ? 0.f : KIND == GATE_BOUNDED ? -INFINITY : 1.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          if (!okc) ain[kb][hf] = floatx4{f, f, f, f};
    }
    gate_finish_blocks<KIND, NKB>(gate, KIND == GATE_BOUNDED ? expf(gate.a_log[hd]) : 1.f, ain);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) Pv[kb][i] = ain[kb][i >> 2][i & 3];
  };
  uint2v kin[NKB][2], qin[NKB][2];  // k, q of the operand layout (order_in)
  // A permlane16 swap of the middle halves of the loaded pieces between rows
  // 0 / 1 and 2 / 3 leaves each lane its 4-channel groups 4 gl and 16 + 4 gl.
  // Done after every load of the item has been issued: its wait for the k and
  // q loads then holds back no other load.
  auto order_in = [&]() {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const auto sk = __builtin_amdgcn_permlane16_swap(kr[kb][a], kr[kb][2 + a], false, false);
        const auto sq = __builtin_amdgcn_permlane16_swap(qr[kb][a], qr[kb][2 + a], false, false);
        kin[kb][0][a] = sk[0];
        kin[kb][1][a] = sk[1];
        qin[kb][0][a] = sq[0];
        qin[kb][1][a] = sq[1];
      }
  };
  // The inputs of an item are loaded while the item before runs its phases
  // 4 to 6 (they are dead after its phase 3; issued after phase 4's Mqk
  // stores, which would otherwise queue behind them): otherwise every item
  // waits for its own loads, and all workgroups read at the same time.  (With the layer
  // prologue the registers do not allow it: its items load at their start.)
  Item pre{};
  if constexpr (!PRO) {
    if ((int)blockIdx.x < n_items) {
      pre = locate(blockIdx.x);
      load_in(blockIdx.x, pre, threadIdx.x & 63);
    }
  }
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    // Lane index behind an empty asm, so that the per-lane addresses are
    // recomputed per item rather than held (or spilled) across the loop.
    int lane_x = threadIdx.x & 63;
    __asm__ volatile("" : "+v"(lane_x));
    int tid_x = threadIdx.x;  // the same for the workgroup-wide prologue staging
    __asm__ volatile("" : "+v"(tid_x));
    const Item cur = PRO ? locate(item) : pre;
    const bool first = cur.tok0 == cur.start;  // the sequence's first chunk
    if constexpr (PRO) load_in(item, cur, lane_x);
    const long long tok0 = cur.tok0;
    const int nv = cur.nv, hd = cur.hd;
    unsigned char* im = img + (size_t)item * IM::bytes;
    const int tr = lane_x & 15;
    const int g = lane_x >> 4;
    const int w = (w4 + item) & 3;  // token tile of this wave
    // issue priority by the tile's share of the item's work (tile 0 takes four
    // of the ten A / Mqk blocks, tile 3 one): on a SIMD shared with the other
    // workgroup's wave, the wave the next barrier waits for goes first.  The
    // layer prologue deals its work by wave, not by tile, so with it the
    // priorities are level until the prologue is done (set by tile from its
    // start, they made that pass 10 % slower).
    if constexpr (!PRO) {
      if (w == 0) __builtin_amdgcn_s_setprio(3);
      else if (w == 1) __builtin_amdgcn_s_setprio(2);
      else if (w == 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    } else {
      __builtin_amdgcn_s_setprio(0);
    }
    const int r = 16 * w + tr;      // this lane's token within the chunk
    const bool okc = r < nv;
    const size_t thc = (size_t)(tok0 + r) * H + hd;

    // (layer prologue) the raw v rows of the wave's token tile: load j covers
    // whole rows (DV / 8 lanes of 16 bytes per row, rows 16 w + VRJ j +
    // lane / (DV / 8)), so that each row is read in one coalesced piece.  The
    // prologue's v goes into the operand block for the state pass; without the
    // prologue the state pass reads v itself.
    constexpr int VLR = DV / 8, VRJ = 64 / VLR;
    const int vrow = 16 * w + lane_x / VLR, vcol = 8 * (lane_x % VLR);
    uint4v vin[NVL];
    if constexpr (PRO) {
#pragma unroll
      for (int j = 0; j < NVL; ++j) {
        const int rv = vrow + VRJ * j;
        vin[j] = rv < nv ? *reinterpret_cast<const uint4v*>(v + ((size_t)(tok0 + rv) * H + hd) * DV + vcol)
                         : uint4v{0u, 0u, 0u, 0u};
      }
    }

    // prologue: the three inputs before the chunk (fp32).  Each is read from
    // both places without a branch (a load under a branch is waited for
    // inside it, which held every item's start for five serial loads): the
    // token row when it lies in the sequence (else the sequence's first row,
    // not used) and the conv-state row through a buffer descriptor that reads
    // zero where there is no conv state; the choice is made where they are
    // stored, after the barrier below.
    constexpr int HPT = (3 * SWP + NTH_P - 1) / NTH_P, TPT = (SWP + NTH_P - 1) / NTH_P;
    bf16 hx[HPT];
    float hs[HPT];
    floatx4 tpv[TPT];
    if constexpr (PRO) {
      const auto rs = rsrc(pa.st_in ? (const void*)(pa.st_in + (size_t)cur.seq * 3 * H * SWP)
                                    : (const void*)q,
                           pa.st_in ? 3LL * H * SWP * 4 : 0);
#pragma unroll
      for (int i = 0; i < HPT; ++i) {
        const int idx = min(tid_x + NTH_P * i, 3 * SWP - 1);
        const int j = idx / SWP, c = idx % SWP;
        const int ten = c < DK ? 0 : c < 2 * DK ? 1 : 2;
        const int cc = c - (ten == 0 ? 0 : ten == 1 ? DK : 2 * DK);
        const int D = ten < 2 ? DK : DV;
        const long long p = tok0 - 3 + j, pc = p >= cur.start ? p : cur.start;
        const int jj = (int)(p - cur.start + 3) < 2 ? (int)(p - cur.start + 3) : 2;
        const bf16* xt = ten == 0 ? q : ten == 1 ? k : v;
        hx[i] = xt[((size_t)pc * H + hd) * D + cc];
        hs[i] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rs, ((jj * H + hd) * SWP + c) * 4, 0, 0));
      }
      // the head's taps, to LDS with the rows below (read as broadcasts, they
      // cost no memory wait per group); loaded like the inputs above, with
      // the tensor's pointer chosen by selects rather than an indexed load
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        const int c = min(tid_x + NTH_P * i, SWP - 1);
        const int ten = c < DK ? 0 : c < 2 * DK ? 1 : 2;
        const int cc = c - (ten == 0 ? 0 : ten == 1 ? DK : 2 * DK);
        const int D = ten < 2 ? DK : DV;
        const float* wt = ten == 0 ? pa.conv.w[0] : ten == 1 ? pa.conv.w[1] : pa.conv.w[2];
        tpv[i] = *reinterpret_cast<const floatx4*>(wt + ((size_t)hd * D + cc) * 4);
      }
    }

    if constexpr (!PRO) order_in();  // the prologue reads the rows back in place
    finish_in(hd, okc);

    // ---- prologue (layer prefill): ShortConv over the three previous
    // inputs, Swish, and the L2Norm of q and k.  The raw rows go to LDS; then
    // lane l of every wave takes token l of the chunk over a range of
    // channels (waves 0 / 1: the two halves of q, waves 2 / 3: the halves of
    // k, each wave a quarter of v), so that the taps are the same in every
    // lane and the previous inputs come from the lanes below (a wave-wide
    // DPP shift by one lane; lane 0 takes the input before the chunk).  The
    // two halves of a row's sum of squares meet through LDS; the results,
    // rounded to bf16, replace the raw values in LDS and are read back in the
    // operand layout.  Phase 1's barrier ends these LDS reads before phase 2
    // reuses the region.
    if constexpr (PRO) {
      __syncthreads();  // the item before is done with R and GK
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {  // the pieces as loaded (8 channels from c8)
        const int c8 = 32 * kb + 8 * (g >> 1) + 16 * (g & 1);
        *reinterpret_cast<uint4v*>(XR + r * ldX + c8) = qr[kb];
        *reinterpret_cast<uint4v*>(XR + r * ldX + DK + c8) = kr[kb];
      }
#pragma unroll
      for (int j = 0; j < NVL; ++j)
        *reinterpret_cast<uint4v*>(XR + (vrow + VRJ * j) * ldX + 2 * DK + vcol) = vin[j];
#pragma unroll
      for (int i = 0; i < HPT; ++i) {
        const int idx = tid_x + NTH_P * i;
        if (idx < 3 * SWP) HI[idx] = tok0 - 3 + idx / SWP >= cur.start ? (float)hx[i] : hs[i];
      }
#pragma unroll
      for (int i = 0; i < TPT; ++i) {
        const int c = tid_x + NTH_P * i;
        if (c < SWP) *reinterpret_cast<floatx4*>(TP + 4 * c) = tpv[i];
      }
      __syncthreads();
      const int row = lane_x;             // token of the chunk
      const bool okr = row < nv;
      float* SS = HI + 3 * SWP;           // [4 waves][64 rows] partial sums of squares
      // one group of 8 channels c0.. of the [q | k | v] row for this lane's
      // token: ShortConv + Swish into y
      auto group8 = [&](int c0, float* y) {
        const uint4v u = *reinterpret_cast<const uint4v*>(XR + row * ldX + c0);
        const floatx4 o0 = *reinterpret_cast<const floatx4*>(HI + 0 * SWP + c0);
        const floatx4 o1 = *reinterpret_cast<const floatx4*>(HI + 0 * SWP + c0 + 4);
        const floatx4 p0 = *reinterpret_cast<const floatx4*>(HI + 1 * SWP + c0);
        const floatx4 p1 = *reinterpret_cast<const floatx4*>(HI + 1 * SWP + c0 + 4);
        const floatx4 q0 = *reinterpret_cast<const floatx4*>(HI + 2 * SWP + c0);
        const floatx4 q1 = *reinterpret_cast<const floatx4*>(HI + 2 * SWP + c0 + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = bfv(u[e >> 1], e & 1);
          // inputs 1, 2, 3 tokens back: lane l - 1's, or before the chunk
          const float h1 = __int_as_float(__builtin_amdgcn_update_dpp(
              __float_as_int(e < 4 ? q0[e] : q1[e - 4]), __float_as_int(x), 0x138, 0xf, 0xf, false));
          const float h2 = __int_as_float(__builtin_amdgcn_update_dpp(
              __float_as_int(e < 4 ? p0[e] : p1[e - 4]), __float_as_int(h1), 0x138, 0xf, 0xf, false));
          const float h3 = __int_as_float(__builtin_amdgcn_update_dpp(
              __float_as_int(e < 4 ? o0[e] : o1[e - 4]), __float_as_int(h2), 0x138, 0xf, 0xf, false));
          const floatx4 t = *reinterpret_cast<const floatx4*>(TP + 4 * (c0 + e));
          y[e] = conv_swish(t, h3, h2, h1, x);
        }
      };
      auto store8 = [&](int c0, const float* z) {
        uint4v u;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          u[e] = (unsigned)__builtin_bit_cast(unsigned short, (bf16)(okr ? z[2 * e] : 0.f)) |
                 ((unsigned)__builtin_bit_cast(unsigned short, (bf16)(okr ? z[2 * e + 1] : 0.f)) << 16);
        *reinterpret_cast<uint4v*>(XR + row * ldX + c0) = u;
      };
      // q or k half of this wave
      {
        const int ten = w4 >> 1, half = w4 & 1;
        const int cc0 = half * (DK / 2);
        const int off = ten * DK + cc0;
        float ss = 0.f;
        for (int gi = 0; gi < DK / 16; ++gi) {
          float y[8];
          group8(off + 8 * gi, y);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(y[e], y[e], ss);
        }
        SS[w4 * 64 + row] = ss;
        __syncthreads();
        // the two halves in a fixed order, so both waves form the same norm
        const float tot = SS[(w4 & 2) * 64 + row] + SS[((w4 & 2) + 1) * 64 + row];
        const float rn = __builtin_amdgcn_rsqf(tot + pa.conv.eps);
        for (int gi = 0; gi < DK / 16; ++gi) {
          float y[8];
          group8(off + 8 * gi, y);
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] *= rn;
          store8(off + 8 * gi, y);
        }
      }
      // v quarter of this wave
      {
        const int cc0 = w4 * (DV / 4);
        for (int gi = 0; gi < DV / 32; ++gi) {
          float y[8];
          group8(2 * DK + cc0 + 8 * gi, y);
          store8(2 * DK + cc0 + 8 * gi, y);
        }
      }
      __syncthreads();
      // the results in the operand layout
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int c = 32 * kb + 16 * hf + 4 * g;
          qin[kb][hf] = *reinterpret_cast<const uint2v*>(XR + r * ldX + c);
          kin[kb][hf] = *reinterpret_cast<const uint2v*>(XR + r * ldX + DK + c);
        }
#pragma unroll
      for (int j = 0; j < NVL; ++j)
        vin[j] = *reinterpret_cast<const uint4v*>(XR + (vrow + VRJ * j) * ldX + 2 * DK + vcol);
    }

    if constexpr (PRO) {  // the prologue is done: priority by tile (see above)
      if (w == 0) __builtin_amdgcn_s_setprio(3);
      else if (w == 1) __builtin_amdgcn_s_setprio(2);
      else if (w == 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    // ---- 1. within-tile decay products P (inclusive scan over the 16 tokens)
#pragma unroll
    for (int kb = 0; kb < NKB; kb += 2) row_scan_mul<16>(&Pv[kb][0]);
    if (tr == 15) {  // whole-tile decay E_w
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          *reinterpret_cast<floatx4*>(ES + w * DK + 32 * kb + 16 * hf + 4 * g) =
              floatx4{Pv[kb][4 * hf], Pv[kb][4 * hf + 1], Pv[kb][4 * hf + 2], Pv[kb][4 * hf + 3]};
    }
    if (g == 0) BS[r] = bt;
    __syncthreads();

    // A tile whose decay product leaves the range of the factored form takes
    // the exact path: the diagonal tile's A and Mqk by running products (per
    // channel half, as the fused kernel's waves form them; parked in this
    // wave's first T frames, which phase 5 writes later, so that nothing extra
    // stays in registers through phase 2), and, after phase 2, suffix products in
    // place of E / P.  The decays are loaded again (the scan overwrote them).
    const bool exact = tile_flagged<DK>(ES + w * DK, lane_x);
    const float gsc = KIND == GATE_BOUNDED ? expf(gate.a_log[hd]) : 1.f;
    auto alpha_of = [&](int kb, float* al) {
      floatx4 a4[1][2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) a4[0][hf] = gate_load4<KIND>(gate, okc, thc, DK, 32 * kb + 16 * hf + 4 * g);
      gate_finish_blocks<KIND, 1>(gate, gsc, a4);
#pragma unroll
      for (int e = 0; e < 8; ++e) al[e] = a4[0][e >> 2][e & 3];
    };
    if (exact) {
      float dA[2][4], dM[2][4];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float al[NKH][8];
#pragma unroll
        for (int kk = 0; kk < NKH; ++kk) alpha_of(NKH * hh + kk, al[kk]);
        tile_exact_sums<NKH>(al, kin + NKH * hh, qin + NKH * hh, tr, g, dA[hh], dM[hh]);
      }
      floatx4 ra, rm;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * w + 4 * g + i;
        ra[i] = (j < r) ? scaled_sum(bt, dA[0][i], dA[1][i]) : 0.f;
        rm[i] = (j <= r) ? dM[0][i] + dM[1][i] : 0.f;
      }
      *frame_ptr<floatx4>(im, IM::tb_frame(w, 0, 0), lane_x) = ra;
      *frame_ptr<floatx4>(im, IM::tb_frame(w, 0, 1), lane_x) = rm;
    }

    // ---- 2. operands of this lane's token, per 32-channel block
    bf16x8 kth[NKB], ktl[NKB];  // Ktil (split), kept until phase 6
    float vd[NKB][8], vn[NKB][8];  // key-side variants: k / P and k E_w / P
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
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
        kk8[e] = bfv(kin[kb][e >> 2][(e & 3) >> 1], e & 1);
        qq[e] = bfv(qin[kb][e >> 2][(e & 3) >> 1], e & 1);
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
      float y[8], gk[8], kt[8];
      bf16x8 kl8, qt8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kl8[e] = (bf16)(kk8[e] * Pv[kb][e]);
        y[e] = qq[e] * Pv[kb][e];
        const float gam = pre[e] * Pv[kb][e];
        qt8[e] = (bf16)(qq[e] * gam);
        gk[e] = kk8[e] * gam;
        const float ip = __builtin_amdgcn_rcpf(Pv[kb][e]);
        const float ew = Ew[e] * ip;  // (an exact tile replaces it below)
        kt[e] = kk8[e] * (ew * post[e]);
        vd[kb][e] = kk8[e] * ip;
        vn[kb][e] = kk8[e] * ew;
      }
      bf16x8 yh, yl;
      split8(y, yh, yl);
      split8(kt, kth[kb], ktl[kb]);
      *reinterpret_cast<bf16x8*>(KL + r * ldK + 32 * kb + 8 * g) = kl8;
      *reinterpret_cast<bf16x8*>(QLh + r * ldK + 32 * kb + 8 * g) = yh;
      *reinterpret_cast<bf16x8*>(QLl + r * ldK + 32 * kb + 8 * g) = yl;
      put_frame(im, IM::q_frame(w, kb), lane_x, qt8);
      // tile 0 of a sequence's first chunk keeps Gamma*Q split (its read-out
      // of the entry state is the least decayed, and a short sequence is
      // nothing else); there Gamma = P, so Gamma*Q is q P and its low half is yl
      if (w == 0 && first) put_frame(im, IM::ql_frame(kb), lane_x, yl);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) st_bf16x4(GK + r * ldK + 32 * kb + 16 * hf + 4 * g, gk + 4 * hf);
      if (w == 0 && tr == 0) {
        float gc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) gc[e] = Ew[e] * post[e];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          *reinterpret_cast<floatx4*>(GC + 32 * kb + 16 * hf + 4 * g) =
              floatx4{gc[4 * hf], gc[4 * hf + 1], gc[4 * hf + 2], gc[4 * hf + 3]};
      }
    }
    if (exact) {
      // E / P_j of an exact tile as the product of the decays after token j
      // (no factor above 1): Ktil and the key side of the later tiles again
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float sfx[8], post[8], kk8[8], kt[8];
        alpha_of(kb, sfx);
        row_rscan_excl<8>(sfx);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          post[e] = 1.f;
          kk8[e] = bfv(kin[kb][e >> 2][(e & 3) >> 1], e & 1);
        }
        for (int i = w + 1; i < 4; ++i)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const floatx4 e4 = *reinterpret_cast<const floatx4*>(ES + i * DK + 32 * kb + 16 * hf + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) post[4 * hf + e] *= e4[e];
          }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kt[e] = kk8[e] * (sfx[e] * post[e]);
          vn[kb][e] = kk8[e] * sfx[e];
        }
        split8(kt, kth[kb], ktl[kb]);
      }
    }
    __syncthreads();
    if (threadIdx.x < DK)
      __builtin_nontemporal_store(GC[threadIdx.x], reinterpret_cast<float*>(im + IM::g_off) + threadIdx.x);
    const bool wsplit = w_split_chunk<DK>(GC, lane_x);  // W's low part kept for this chunk
    if (threadIdx.x == 0)
      __builtin_nontemporal_store(wsplit ? 1 : 0, reinterpret_cast<int*>(im + IM::f_off));

    // ---- 3. A and Mqk blocks (query tile m >= n, key tile n = w): the key
    // side k * (Gamma_r / Gamma_j restricted to the key) is this lane's
    // register operand, one variant per m; two chains over the channel halves
    floatx4 rA[4], rM[4];
    {
      const int n = w;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        rA[m] = floatx4{0.f, 0.f, 0.f, 0.f};
        rM[m] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (m < n) continue;
        if (m > n + 1) {  // variant of tile m: the one of m - 1 times E_{m-1}
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              const floatx4 e4 =
                  *reinterpret_cast<const floatx4*>(ES + (m - 1) * DK + 32 * kb + 16 * hf + 4 * g);
#pragma unroll
              for (int e = 0; e < 4; ++e) vn[kb][4 * hf + e] *= e4[e];
            }
        }
        floatx4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, m0 = a0, m1 = a0;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          float vs[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) vs[e] = m == n ? vd[kb][e] : vn[kb][e];
          bf16x8 vh, vl;
          split8(vs, vh, vl);
          const bf16x8 akl = frag_ld(KL, ldK, 16 * m + tr, 32 * kb, g);
          const bf16x8 aqh = frag_ld(QLh, ldK, 16 * m + tr, 32 * kb, g);
          const bf16x8 aql = frag_ld(QLl, ldK, 16 * m + tr, 32 * kb, g);
          floatx4& aa = kb < NKH ? a0 : a1;
          floatx4& mm = kb < NKH ? m0 : m1;
          // key side as the A operand (rows j), query side as B (columns r)
          aa = mfma_bf16(vh, akl, aa);
          mm = mfma_bf16(vh, aqh, mm);
          mm = mfma_bf16(vh, aql, mm);
          mm = mfma_bf16(vl, aqh, mm);
        }
        // b_r A_rj (j < r) and Mqk_rj (j <= r) for rows j = 16n + 4g + i of
        // key tile n, column r = 16m + tr; each channel half is scaled and
        // masked, then summed
        const float br = BS[16 * m + tr];
        const int rq = 16 * m + tr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 16 * n + 4 * g + i;
          rA[m][i] = (j < rq) ? scaled_sum(br, a0[i], a1[i]) : 0.f;
          rM[m][i] = (j <= rq) ? m0[i] + m1[i] : 0.f;
        }
        if (m == n && exact) {  // the diagonal tile from the exact sums
          rA[m] = *frame_ptr<floatx4>(im, IM::tb_frame(w, 0, 0), lane_x);
          rM[m] = *frame_ptr<floatx4>(im, IM::tb_frame(w, 0, 1), lane_x);
        }
      }
    }
    __syncthreads();  // KL / QL reads done; AF and MQ overwrite them
    {
      const int n = w;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (m < n) continue;
        *reinterpret_cast<floatx4*>(AF + (16 * m + tr) * ldA + 16 * n + 4 * g) = rA[m];
        *reinterpret_cast<floatx4*>(MQ + (16 * m + tr) * ldA + 16 * n + 4 * g) = rM[m];
      }
    }
    __syncthreads();

    // ---- 4. Mqk image of this tile's queries (token k-slots in the swizzled
    // order), then T = (I + A)^{-1}, blockwise over 16x16 tiles on fp32 MFMA
    // 16x16x4: every product is (LDS matrix, row-major, read 16 bytes per lane
    // as the A operand) x (register matrix in the accumulator layout, which is
    // the B operand layout)
    {
      bf16x8 mqh[2], mql[2];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        floatx4 m4 = {0.f, 0.f, 0.f, 0.f};
        if (n <= w) m4 = *reinterpret_cast<const floatx4*>(MQ + r * ldA + 16 * n + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16 hv = (bf16)m4[i];
          mqh[n >> 1][4 * (n & 1) + i] = hv;
          mql[n >> 1][4 * (n & 1) + i] = (bf16)(m4[i] - (float)hv);
        }
      }
      // (the frames of key blocks after the tile, all zero, are not written)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb > (w >> 1)) continue;
        put_frame(im, IM::m_frame(w, kb, 0), lane_x, mqh[kb]);
        put_frame(im, IM::m_frame(w, kb, 1), lane_x, mql[kb]);
      }
    }
    if constexpr (!PRO) {  // the next item's inputs (see above)
      const int nxt = item + (int)gridDim.x;
      if (nxt < n_items) {
        pre = locate(nxt);
        load_in(nxt, pre, lane_x);
      }
    }
    {
      auto arow = [&](const float* M) -> floatx4 {
        return *reinterpret_cast<const floatx4*>(M + tr * ldA + 4 * g);
      };
      auto mm16 = [&](const floatx4& a, const floatx4& x) -> floatx4 {
        floatx4 yv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) yv = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], x[s], yv, 0, 0, 0);
        return yv;
      };
      {
        // diagonal block of tile w: N = A_ww strictly lower, N^16 = 0, so
        // (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8).  N^2 is staged in
        // the block itself, N^4 in the unused upper block (w, w + 1 mod 4), or
        // for w = 3 in block (3, 0), which the last round writes later.
        const int b0 = 16 * w;
        float* S2 = TF + b0 * ldA + b0;
        float* S4 = TF + b0 * ldA + 16 * ((w + 1) & 3);
        floatx4 nB;
#pragma unroll
        for (int i = 0; i < 4; ++i) nB[i] = AF[(b0 + 4 * g + i) * ldA + b0 + tr];
        const floatx4 aN = arow(AF + b0 * ldA + b0);
        const floatx4 n2 = mm16(aN, nB);
#pragma unroll
        for (int i = 0; i < 4; ++i) S2[(4 * g + i) * ldA + tr] = n2[i];
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const floatx4 a2 = arow(S2);
        const floatx4 n4 = mm16(a2, n2);
#pragma unroll
        for (int i = 0; i < 4; ++i) S4[(4 * g + i) * ldA + tr] = n4[i];
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const floatx4 a4 = arow(S4);
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
        if (n >= 0) {
          floatx4 Xs = {0.f, 0.f, 0.f, 0.f};
          for (int j = n; j < m; ++j) {
            floatx4 tB;
#pragma unroll
            for (int i = 0; i < 4; ++i) tB[i] = TF[(16 * j + 4 * g + i) * ldA + 16 * n + tr];
            Xs += mm16(arow(AF + 16 * m * ldA + 16 * j), tB);
          }
          const floatx4 Y = mm16(arow(TF + 16 * m * ldA + 16 * m), Xs);
#pragma unroll
          for (int i = 0; i < 4; ++i) TF[(16 * m + 4 * g + i) * ldA + 16 * n + tr] = -Y[i];
        }
        __syncthreads();
      }
    }

    // ---- 5. TB = T Diag(beta) (split, [r][j]); then W^T = (Gamma*K)^T
    // (T Diag b)^T for this tile's tokens, all channels, as the operand image
    // of W S, and T Diag(b) as the operand image of U
#pragma unroll
    for (int it = 0; it < CH * CH / 4 / NTH_P; ++it) {
      const int idx = 64 * w4 + lane_x + NTH_P * it;
      const int rr = idx >> 4, j0 = 4 * (idx & 15);
      const floatx4 t4 = *reinterpret_cast<const floatx4*>(TF + rr * ldA + j0);
      const floatx4 b4 = *reinterpret_cast<const floatx4*>(BS + j0);
      float x4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x4[e] = (j0 + e <= rr) ? t4[e] * b4[e] : 0.f;
      st_split4(TB + rr * ldT + j0, loT, x4);
    }
    if constexpr (PRO) {  // the prologue's v rows (zero past the chunk's end)
#pragma unroll
      for (int j = 0; j < NVL; ++j)
        __builtin_nontemporal_store(
            vin[j], reinterpret_cast<uint4v*>(im + IM::v_off + ((size_t)(vrow + VRJ * j) * DV + vcol) * 2));
    }
    __syncthreads();
    {
      bf16x8 tbh[2], tbl[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        tbh[kb] = frag_ld(TB, ldT, r, 32 * kb, g);
        tbl[kb] = frag_ld(TB + loT, ldT, r, 32 * kb, g);
      }
#pragma unroll
      for (int kp = 0; kp < NCHT / 2; ++kp) {
        bf16x8 wh, wl;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int ct = 2 * kp + h2;
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            if (kb > (w >> 1)) continue;
            // split T Diag(b) only: (Gamma*K) single-rounded is within the
            // error budget of this product, the T side is not
            const bf16x8 ah = frag_tr(GK, ldK, 16 * ct, 32 * kb + 8 * g, 32 * kb + 8 * g + 4, tr);
            acc = mfma_bf16(ah, tbh[kb], acc);
            acc = mfma_bf16(ah, tbl[kb], acc);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bf16 hv = (bf16)acc[i];
            wh[4 * h2 + i] = hv;
            wl[4 * h2 + i] = (bf16)(acc[i] - (float)hv);
          }
        }
        put_frame(im, IM::w_frame(w, kp, 0), lane_x, wh);
        if (wsplit) put_frame(im, IM::w_frame(w, kp, 1), lane_x, wl);
      }
      // T Diag(b) as the A operand of U = T Diag(b) V, which the state pass
      // forms (the frames of key blocks after the tile are zero, not stored)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb > (w >> 1)) continue;
        put_frame(im, IM::tb_frame(w, kb, 0), lane_x, tbh[kb]);
        put_frame(im, IM::tb_frame(w, kb, 1), lane_x, tbl[kb]);
      }
    }
    __syncthreads();  // TB / GK reads done; KT overwrites the region

    // ---- 6. Ktil ([token][channel], split) into the A operand images of
    // Ktil^T P, 16 state rows per frame
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      // whole 32-bit words (element pairs) of the packed registers
      const uint4v uh = __builtin_bit_cast(uint4v, kth[kb]);
      const uint4v ul = __builtin_bit_cast(uint4v, ktl[kb]);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        *reinterpret_cast<uint2v*>(KT + r * ldK + 32 * kb + 16 * hf + 4 * g) = uint2v{uh[2 * hf], uh[2 * hf + 1]};
        *reinterpret_cast<uint2v*>(KT + loK + r * ldK + 32 * kb + 16 * hf + 4 * g) =
            uint2v{ul[2 * hf], ul[2 * hf + 1]};
      }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NCHT / 4; ++s) {
      const int rt = w4 + 4 * s;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        put_frame(im, IM::k_frame(rt, kb, 0), lane_x,
                  frag_tr(KT, ldK, 16 * rt, 32 * kb + 4 * g, 32 * kb + 16 + 4 * g, tr));
        put_frame(im, IM::k_frame(rt, kb, 1), lane_x,
                  frag_tr(KT + loK, ldK, 16 * rt, 32 * kb + 4 * g, 32 * kb + 16 + 4 * g, tr));
      }
    }
  }
}

template <int DK, int DV, int KIND, bool PRO>
hipError_t launch_kp(const PrefillArgs& a, unsigned char* img, const int32_t* chunk_off,
                     long long tok_lo, long long tok_hi, int cap, int grid) {
  using L = PrepPlan<DK, DV>;
  constexpr int lds = PRO ? L::totalP : L::total;
  auto kern = prefill_prep_kernel<DK, DV, KIND, PRO>;
  static bool attr_set = false;  // per instantiation; idempotent if raced
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  ProArgs pa{};
  if (PRO) pa = ProArgs{a.pro->conv, a.pro->st_in};
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTH_P), lds, (hipStream_t)a.stream, (const bf16*)a.q,
                     (const bf16*)a.k, (const bf16*)a.v, a.gate, a.beta, a.cu_seqlens, a.n_seq, a.T, a.H,
                     img, chunk_off, tok_lo, tok_hi, cap, pa);
  return hipGetLastError();
}

template <int DK, int DV, int KIND>
hipError_t launch_k(const PrefillArgs& a, unsigned char* img, const int32_t* chunk_off,
                    long long tok_lo, long long tok_hi, int cap, int grid) {
  return a.pro ? launch_kp<DK, DV, KIND, true>(a, img, chunk_off, tok_lo, tok_hi, cap, grid)
               : launch_kp<DK, DV, KIND, false>(a, img, chunk_off, tok_lo, tok_hi, cap, grid);
}

// one instantiation per gate kind, as for the fused kernel
template <int DK, int DV>
hipError_t launch_t(const PrefillArgs& a, unsigned char* img, const int32_t* chunk_off,
                    long long tok_lo, long long tok_hi, int cap, int grid) {
  switch (a.gate.kind) {
    case GATE_LOG: return launch_k<DK, DV, GATE_LOG>(a, img, chunk_off, tok_lo, tok_hi, cap, grid);
    case GATE_BOUNDED:
      return launch_k<DK, DV, GATE_BOUNDED>(a, img, chunk_off, tok_lo, tok_hi, cap, grid);
    case GATE_SCALAR:
      return launch_k<DK, DV, GATE_SCALAR>(a, img, chunk_off, tok_lo, tok_hi, cap, grid);
    case GATE_NONE: return launch_k<DK, DV, GATE_NONE>(a, img, chunk_off, tok_lo, tok_hi, cap, grid);
    default: return launch_k<DK, DV, GATE_ALPHA>(a, img, chunk_off, tok_lo, tok_hi, cap, grid);
  }
}

}  // namespace

int prefill_prep_per_cu() { return 2; }

hipError_t launch_prefill_prep(const PrefillArgs& a, unsigned char* img, const int32_t* chunk_off,
                               long long tok_lo, long long tok_hi, int cap, int grid) {
  if (a.Dk == 128)
    return a.Dv == 128 ? launch_t<128, 128>(a, img, chunk_off, tok_lo, tok_hi, cap, grid)
                       : launch_t<128, 64>(a, img, chunk_off, tok_lo, tok_hi, cap, grid);
  return a.Dv == 128 ? launch_t<64, 128>(a, img, chunk_off, tok_lo, tok_hi, cap, grid)
                     : launch_t<64, 64>(a, img, chunk_off, tok_lo, tok_hi, cap, grid);
}

}  // namespace kda
