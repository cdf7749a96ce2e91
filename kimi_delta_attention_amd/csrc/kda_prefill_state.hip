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
// caller's final state or workspace); its per-chunk operands arrive as register
// images (Images<DK, DV>) fetched with coalesced 16-byte loads, one chunk ahead.
//
// Eight waves in two roles, one wave of each role per SIMD.  Token tile w
// (tokens 16w..16w+15 of the chunk) has a chain wave (waves 0..3), which
// computes W S and P = U - W S for the tile's 16 tokens, and an output wave
// (waves 4..7), which computes (Gamma*Q) S and Mqk P and stores o.  Both update
// a share of the state: Dk = 128, state rows 16(2w + role).., all 64 values;
// Dk = 64, rows 16w.., value tiles 2 role, 2 role + 1.  Per chunk:
//   1. every wave writes its state tiles to LDS as the split B operand of
//      W S and (Gamma*Q) S                                        -- barrier
//   2. chain: W S (two channel-half chains), P, P to LDS (split);
//      output: (Gamma*Q) S (two channel-half chains)               -- barrier
//   3. chain: S = Diag(Gamma_C) S + Ktil^T P on its tiles;
//      output: o = (Gamma*Q) S + Mqk P, stored; the same state update
// so the state's dependency chain (W S -> P -> Ktil^T P) shares each SIMD's
// matrix pipe with independent output work and a chunk costs two barriers.
// Every wave fetches only the operand frames it uses, and no frame is fetched
// twice in a workgroup.  The fused kernel computes the same products with the
// same accumulation order (the two channel halves as separate chains, low half
// first), so both schedules give bitwise the same results.
#include <type_traits>

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

constexpr int NTH_S = 512;

template <int DK, int BV>
struct StatePlan {
  // Row strides of 8 (mod 16) dwords, and in ST and PT the 16-byte chunks of
  // a row swapped in pairs on rows with bit 2 set (chunk c at c ^ ((row >> 2)
  // & 1)): measured on gfx950, the 16-byte operand reads (row = lane % 16,
  // chunk = lane / 16) and 16-byte writes then take no bank conflicts, where a
  // stride of 4 (mod 8) dwords doubles the reads.  The 8-byte writes of the
  // split halves keep a 2-way conflict.
  static constexpr int ldS = DK + 16, ldP = CH + 16;
  // o staging of each output wave: 16 rows x BV values fp32
  static constexpr int ldO = BV + 8;
  // v rows of a chunk, [token][value] bf16, two buffers (the chunk after the
  // current one is staged while U of the current one is formed)
  static constexpr int ldV = BV + 8;
  static constexpr int ST = BV * ldS * 2 * 2, PT = BV * ldP * 2 * 2, OS = 4 * 16 * ldO * 4,
                       VS = CH * ldV * 2;
  static constexpr int oST = 0, oPT = ST, oOS = ST + PT, oVS = oOS + OS, total = oVS + 2 * VS;
  static_assert(total <= 163840, "LDS budget");
  static_assert(oOS % 16 == 0 && oVS % 16 == 0 && VS % 16 == 0, "alignment");
};

// Lane quad transpose: lane b of each group of four lanes holds x[i] = element
// (i, b) of a 4x4 block and receives element (b, i).  Two exchange steps, over
// lane bit 0 / element bit 0 and then lane bit 1 / element bit 1, each a DPP
// quad permutation and a per-lane select.
template <int CTRL>
__device__ __forceinline__ float quad_perm(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ floatx4 quad_transpose(const floatx4& x, int b) {
  floatx4 z, y;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float t = quad_perm<0xB1>(x[i ^ 1]);  // lanes [1, 0, 3, 2]
    z[i] = ((b ^ i) & 1) ? t : x[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float t = quad_perm<0x4E>(z[i ^ 2]);  // lanes [2, 3, 0, 1]
    y[i] = ((b ^ i) & 2) ? t : z[i];
  }
  return y;
}

// Four consecutive o values of one row through a buffer descriptor: a store
// whose byte offset lies beyond the descriptor's range is dropped by the
// hardware, which masks the rows past the end of a partial chunk without a
// branch (non-temporal: o is written once).
template <typename TOut>
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t rs, int off, const floatx4& y);
template <>
__device__ __forceinline__ void store4<float>(__amdgpu_buffer_rsrc_t rs, int off, const floatx4& y) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint4v, y), rs, off, 0, 2);
}
template <>
__device__ __forceinline__ void store4<bf16>(__amdgpu_buffer_rsrc_t rs, int off, const floatx4& y) {
  uint2v u;
  u[0] = (unsigned)__builtin_bit_cast(unsigned short, (bf16)y[0]) |
         ((unsigned)__builtin_bit_cast(unsigned short, (bf16)y[1]) << 16);
  u[1] = (unsigned)__builtin_bit_cast(unsigned short, (bf16)y[2]) |
         ((unsigned)__builtin_bit_cast(unsigned short, (bf16)y[3]) << 16);
  __builtin_amdgcn_raw_buffer_store_b64(u, rs, off, 0, 2);
}

// Waits for every outstanding vector memory access of the wave.  Placed after
// the fetch in front of a chunk loop, so that the loop is entered with nothing
// in flight but what the loop body itself issues (the wait counts the compiler
// derives for the loop then hold on every iteration).
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The chunks of one sequence that start in the window [tok_lo, tok_hi): chunk
// c of the sequence (c_lo <= c < c_hi) has item slot ci0 + c - ci_lo (below cap).
struct SeqWindow {
  long long start, len;
  int ci0, ci_lo, nch_seq, c_lo, c_hi;
};
__device__ __forceinline__ SeqWindow seq_window(const int32_t* cu_seqlens, const int32_t* chunk_off,
                                                int n_seq, int T, int seq, long long tok_lo,
                                                long long tok_hi, int cap) {
  SeqWindow sw;
  if (cu_seqlens) {
    sw.start = cu_seqlens[seq];
    sw.len = (long long)cu_seqlens[seq + 1] - sw.start;
    sw.ci0 = chunk_off[seq];
    sw.nch_seq = chunk_off[seq + 1] - sw.ci0;  // ceil(len / 64) for monotone offsets
  } else {
    sw.start = (long long)seq * T;
    sw.len = T;
    sw.nch_seq = (T + CH - 1) / CH;
    sw.ci0 = seq * sw.nch_seq;
  }
  if (sw.len > (long long)sw.nch_seq * CH) sw.len = (long long)sw.nch_seq * CH;
  sw.ci_lo = chunks_before(tok_lo, cu_seqlens, chunk_off, n_seq, T);
  auto first_from = [&](long long tok) {
    long long c = (tok - sw.start + CH - 1) / CH;
    if (c < 0) c = 0;
    return (int)(c < sw.nch_seq ? c : sw.nch_seq);
  };
  sw.c_lo = first_from(tok_lo);
  sw.c_hi = first_from(tok_hi);
  if (sw.c_lo < sw.ci_lo - sw.ci0) sw.c_lo = sw.ci_lo - sw.ci0;            // reached only for
  if (sw.c_hi > cap + sw.ci_lo - sw.ci0) sw.c_hi = cap + sw.ci_lo - sw.ci0;  // non-monotone cu_seqlens
  return sw;
}

// Segments of a sequence's chunks in a window: nseg, but no more than its
// chunk count (so that no segment is empty), and 1 when it has none.
__device__ __forceinline__ int seg_count(int nseg, int c_lo, int c_hi) {
  const int n = c_hi - c_lo;
  return n <= 1 ? 1 : (nseg < n ? nseg : n);
}

// SUMMARY: instead of the state, the workgroup carries a 64-column slice of
// [M | b] (Dk + Dv columns, from [I | 0]) through its segment of the window's
// chunks -- the segment's affine map S -> M S + b ("Kimi K3模型架构详解"
// section 3.6): the M columns see U = 0, no output is formed, and the result
// goes to `summ`.  With nseg > 1 the window's chunks of a sequence are cut
// into ns = seg_count(nseg, ..) segments of consecutive chunks; when ns > 1,
// the normal workgroup of segment s enters from seg_in[s] (the combine
// kernel's entry states) and only the last segment writes the carried state.
// With ns = 1, segment 0 runs exactly as the unsegmented pass.
template <int DK, int DV, int BV, typename TOut, bool SUMMARY>
__global__ __launch_bounds__(NTH_S) void prefill_state_kernel(
    const unsigned char* __restrict__ img, const int32_t* __restrict__ chunk_off,
    const int32_t* __restrict__ cu_seqlens, const float* s_init, float* carry,
    TOut* __restrict__ o, const bf16* __restrict__ v, int n_seq, int T, int H, long long tok_lo,
    long long tok_hi, int cap, int nseg, const float* __restrict__ seg_in,
    float* __restrict__ summ) {
  static_assert(BV == 32 || BV == 64, "value slice of 32 or 64 columns");
  constexpr int SWC = SUMMARY ? DK + DV : DV;  // columns the workgroups carry
  using L = StatePlan<DK, BV>;
  using IM = Images<DK, DV>;
  constexpr int NKB = DK / 32;
  constexpr int NKH = NKB / 2;                   // 32-channel blocks per channel half
  constexpr int NVT = BV / 16;                   // value tiles of the slice
  constexpr int KVT = DK == 128 ? NVT : NVT / 2;  // value tiles of this wave's state rows
  constexpr int ldS = L::ldS, ldP = L::ldP, ldO = L::ldO, ldV = L::ldV;
  constexpr int loS = BV * ldS, loP = BV * ldP;

  extern __shared__ __align__(16) unsigned char smem[];
  bf16* ST = reinterpret_cast<bf16*>(smem + L::oST);
  bf16* PT = reinterpret_cast<bf16*>(smem + L::oPT);
  float* OS = reinterpret_cast<float*>(smem + L::oOS);
  bf16* VS0 = reinterpret_cast<bf16*>(smem + L::oVS);  // v rows, buffers 0 and 1

  const int tid = threadIdx.x;
  const int w8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = w8 >> 2;  // 0: chain wave, 1: output wave
  const int w = w8 & 3;      // token tile
  const int lane = tid & 63;

  constexpr int nsl = SWC / BV;
  const int nsg = SUMMARY ? nseg - 1 : nseg;  // segments with a workgroup each
  const int total = nsg * n_seq * H * nsl;
  // Workgroups are dealt round-robin over the 8 XCDs.  The nsl slices of one
  // (segment, sequence, head) stay on one XCD (they fetch the same operand
  // frames, so all but the first hit that XCD's L2), and consecutive
  // (segment, sequence, head) pairs go to different XCDs: a window of a packed
  // batch often holds chunks of only one or two sequences, whose pairs are
  // consecutive, and they should spread over the whole device.
  int wid = blockIdx.x;
  const int npair = total / nsl;
  if ((npair & 7) == 0) {
    const int x = blockIdx.x & 7, r = blockIdx.x >> 3;
    wid = ((r / nsl) * 8 + x) * nsl + r % nsl;
  }
  const int sl = wid % nsl;
  const int h = (wid / nsl) % H;
  const int seq = (wid / (nsl * H)) % n_seq;
  const int seg = wid / (nsl * H * n_seq);
  const SeqWindow sw = seq_window(cu_seqlens, chunk_off, n_seq, T, seq, tok_lo, tok_hi, cap);
  const long long start = sw.start, len = sw.len;
  const int ci0 = sw.ci0, ci_lo = sw.ci_lo, nch_seq = sw.nch_seq;
  const bool window_first = sw.c_lo == 0;  // the window starts the sequence
  const int ns = seg_count(nseg, sw.c_lo, sw.c_hi);
  // a summary only for segments before the last
  if (seg >= (SUMMARY ? ns - 1 : ns)) return;
  // this workgroup's segment of the window's chunks
  const int n_ch = sw.c_hi > sw.c_lo ? sw.c_hi - sw.c_lo : 0;
  const int c_lo = sw.c_lo + n_ch * seg / ns, c_hi = sw.c_lo + n_ch * (seg + 1) / ns;
  // an empty sequence hands its initial state through in the first window
  if (!(c_lo < c_hi || (nch_seq == 0 && tok_lo == 0))) return;
  const int vcol0 = sl * BV;
  // the U tiles of the slice: b's columns map to v's; M's columns see U = 0
  const bool u_zero = SUMMARY && vcol0 < DK;
  const int vt0 = (SUMMARY ? (u_zero ? 0 : vcol0 - DK) : vcol0) / 16;
  // state tiles of this wave
  const int srt = DK == 128 ? 2 * w + role : w;  // 16-row tile
  const int sv0 = DK == 128 ? 0 : KVT * role;    // first value tile (within the slice)

  floatx4 Sacc[KVT];
  {
    const int tr = lane & 15, g = lane >> 4;
    const float* src = ns > 1 ? seg_in + (size_t)seg * n_seq * H * DK * DV
                              : window_first ? s_init : carry;
    const float* si = src ? src + ((size_t)seq * H + h) * DK * DV : nullptr;
#pragma unroll
    for (int j = 0; j < KVT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * srt + 4 * g + i;
        const int col = vcol0 + 16 * (sv0 + j) + tr;
        if constexpr (SUMMARY)
          Sacc[j][i] = col == row ? 1.f : 0.f;  // [I | 0]
        else
          Sacc[j][i] = si ? si[(size_t)row * DV + col] : 0.f;
      }
  }

  auto item_base = [&](int c) -> const unsigned char* {
    return img + ((size_t)(ci0 + c - ci_lo) * H + h) * IM::bytes;
  };
  // the state as the B operand of W S and (Gamma*Q) S: [value][channel
  // position], position 32kb + 8g + 4h + i holds channel 32kb + 16h + 4g + i
  // (gs: the lane's chunk g after the swizzle of its row 16 j + tr)
  auto put_state = [&](int gs, int tr) {
    const int c0r = 16 * srt;
    const int pos = 32 * (c0r >> 5) + 8 * gs + 4 * ((c0r >> 4) & 1);
#pragma unroll
    for (int j = 0; j < KVT; ++j) {
      float x4[4] = {Sacc[j][0], Sacc[j][1], Sacc[j][2], Sacc[j][3]};
      st_split4(ST + (16 * (sv0 + j) + tr) * ldS + pos, loS, x4);
    }
  };
  // the fetch index of the chunk after c: the last chunk fetches itself again,
  // so that every fetch is unconditional
  auto next_of = [&](int c) { return c + 1 < c_hi ? c + 1 : c; };

  if (role == 0) {
    // ---- chain waves: they carry the state's dependency chain, so they take
    // the issue priority over the output wave of their SIMD (whose work has
    // slack until the chunk's barriers)
    __builtin_amdgcn_s_setprio(2);
    static_assert(BV == 64, "v rows staged by the 256 chain threads, 32 bytes each");
    struct Ops {
      bf16x8 wh[NKB], wl[NKB];
      bf16x8 th[2], tl[2];   // T Diag(b) of the tile's rows (A operand of U)
      floatx4 u[NVT];        // U of the tile, formed during the chunk before
      bf16x8 kh[2], kl[2];
      floatx4 gc;
      uint4v vr[2];          // this thread's v rows of the chunk after
      int ws;       // this chunk keeps W split (its low frames were fetched)
      int ws_next;  // the next chunk's flag, read one chunk ahead of its W frames
    };
    // the chunk's W split flag (written by the first pass)
    auto flag_of = [&](int c) -> int {
      return *reinterpret_cast<const int*>(item_base(c) + IM::f_off);
    };
    // the operands of W S and of U (fetched during the W S of the chunk before;
    // W's low frames only for a split chunk) and the rest (fetched during its
    // state update, with the flag of the chunk after)
    auto fetch_w = [&](int c, int ws, Ops& op) {
      const unsigned char* b = item_base(c);
      op.ws = ws;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        op.wh[kb] = *frame_ptr<bf16x8>(b, IM::w_frame(w, kb, 0), lane);
        if (ws) op.wl[kb] = *frame_ptr<bf16x8>(b, IM::w_frame(w, kb, 1), lane);
      }
      if (!u_zero) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          // key block 1 of tiles 0 and 1 lies after the tile: its frames are
          // not stored and its products are not formed
          const int kbt = kb > (w >> 1) ? 0 : kb;
          op.th[kb] = *frame_ptr<bf16x8>(b, IM::tb_frame(w, kbt, 0), lane);
          op.tl[kb] = *frame_ptr<bf16x8>(b, IM::tb_frame(w, kbt, 1), lane);
        }
      }
    };
    // v rows of chunk c for this thread: row tid / 4, columns 16 (tid % 4) and
    // + 8 of the slice (zero past the chunk's end); from v, or from the
    // operand block where the first pass formed v (the layer prologue)
    const int vrow = tid >> 2, vcol = 16 * (tid & 3);
    auto load_v = [&](int c, uint4v (&vr)[2]) {
      if (u_zero) return;
      const long long c0 = (long long)c * CH;
      const int nvc = (int)(len - c0 < CH ? len - c0 : CH);
      const int col = 16 * vt0 + vcol;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (vrow >= nvc) {
          vr[j] = uint4v{0u, 0u, 0u, 0u};
        } else if (v) {
          vr[j] = *reinterpret_cast<const uint4v*>(v + ((size_t)(start + c0 + vrow) * H + h) * DV +
                                                   col + 8 * j);
        } else {
          vr[j] = *reinterpret_cast<const uint4v*>(item_base(c) + IM::v_off +
                                                   ((size_t)vrow * DV + col + 8 * j) * 2);
        }
      }
    };
    auto put_v = [&](int c, const uint4v (&vr)[2]) {
      if (u_zero) return;
      bf16* VS = VS0 + (c & 1) * (CH * ldV);
#pragma unroll
      for (int j = 0; j < 2; ++j) *reinterpret_cast<uint4v*>(VS + vrow * ldV + vcol + 8 * j) = vr[j];
    };
    // U = T Diag(b) V of the tile, every value of the slice (the first pass's
    // products, in its order); zero for M's columns of a summary
    auto form_u = [&](int c, Ops& op) {
      const int tr = lane & 15, g = lane >> 4;
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) op.u[vt] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (u_zero) return;
      const bf16* VS = VS0 + (c & 1) * (CH * ldV);
      // one loop per number of key blocks (1 for tiles 0, 1; 2 for tiles 2,
      // 3), so that no branch cuts it (see W S)
      auto u_loop = [&](auto nkb) {
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
          for (int kb = 0; kb < decltype(nkb)::value; ++kb) {
            const bf16x8 bv = frag_tr(VS, ldV, 16 * vt, 32 * kb + 8 * g, 32 * kb + 8 * g + 4, tr);
            op.u[vt] = mfma_bf16(op.th[kb], bv, op.u[vt]);
            op.u[vt] = mfma_bf16(op.tl[kb], bv, op.u[vt]);
          }
      };
      if (w >> 1)
        u_loop(std::integral_constant<int, 2>{});
      else
        u_loop(std::integral_constant<int, 1>{});
    };
    auto fetch_r = [&](int c, Ops& op) {
      const unsigned char* b = item_base(c);
      op.ws_next = flag_of(next_of(c));
      op.gc = *reinterpret_cast<const floatx4*>(b + IM::g_off + 4 * (16 * srt + 4 * (lane >> 4)));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        op.kh[kb] = *frame_ptr<bf16x8>(b, IM::k_frame(srt, kb, 0), lane);
        op.kl[kb] = *frame_ptr<bf16x8>(b, IM::k_frame(srt, kb, 1), lane);
      }
      load_v(next_of(c), op.vr);
    };
    auto chunk = [&](int c, const Ops& op, Ops& nx) {
      int lane_x = lane;
      __asm__ volatile("" : "+v"(lane_x));
      const int tr = lane_x & 15;
      const int g = lane_x >> 4;
      const int gs = g ^ ((tr >> 2) & 1);  // swizzled chunk of ST / PT rows
      put_v(next_of(c), op.vr);  // read after the barrier below, by the U of the next chunk
      __syncthreads();
      const int ws_next = __builtin_amdgcn_readfirstlane(op.ws_next);
      fetch_w(next_of(c), ws_next, nx);
      const bool ws = op.ws != 0;
      // ---- W S over both channel halves (separate chains, low half first)
      // and P = U - W S, to LDS as [value][token position]: token
      // 32kb + 16h + 4g + i sits at position 32kb + 8g + 4h + i (the order of
      // the Mqk^T operand)
      floatx4 a0[NVT], a1[NVT];
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        a0[vt] = floatx4{0.f, 0.f, 0.f, 0.f};
        a1[vt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      // one loop per value of the (wave-uniform) split flag: a branch inside
      // the loop would cut it into blocks that each wait for their own LDS
      // reads, with no read issued ahead of the products
      auto ws_loop = [&](auto split) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int vt = 0; vt < NVT; ++vt) {
            const bf16x8 bh = frag_ld(ST, ldS, 16 * vt + tr, 32 * kb, gs);
            const bf16x8 bl = frag_ld(ST + loS, ldS, 16 * vt + tr, 32 * kb, gs);
            floatx4& acc = kb < NKH ? a0[vt] : a1[vt];
            acc = mma_w(decltype(split)::value, op.wh[kb], op.wl[kb], bh, bl, acc);
          }
      };
      if (ws)
        ws_loop(std::true_type{});
      else
        ws_loop(std::false_type{});
      const int pos = 32 * (w >> 1) + 8 * gs + 4 * (w & 1);
#pragma unroll
      for (int vt = 0; vt < NVT; ++vt) {
        const floatx4 wsv = a0[vt] + a1[vt];
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = op.u[vt][i] - wsv[i];
        st_split4(PT + (16 * vt + tr) * ldP + pos, loP, pv);
      }
      __syncthreads();
      fetch_r(next_of(c), nx);
      // ---- S = Diag(Gamma_C) S + Ktil^T P on this wave's tiles
#pragma unroll
      for (int j = 0; j < KVT; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) Sacc[j][i] *= op.gc[i];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 bh = frag_ld(PT, ldP, 16 * (sv0 + j) + tr, 32 * kb, gs);
          const bf16x8 bl = frag_ld(PT + loP, ldP, 16 * (sv0 + j) + tr, 32 * kb, gs);
          Sacc[j] = mma_ab(op.kh[kb], op.kl[kb], bh, bl, Sacc[j]);
        }
      }
      // the updated state as the next chunk's operand (ST is not read after
      // the second barrier), then U of the next chunk (its v rows were staged
      // before the first barrier of this chunk), off the state's dependency
      // chain
      put_state(gs, tr);
      form_u(next_of(c), nx);
    };
    if (c_lo < c_hi) {
      Ops X, Y;
      fetch_w(c_lo, __builtin_amdgcn_readfirstlane(flag_of(c_lo)), X);
      load_v(c_lo, X.vr);
      put_v(c_lo, X.vr);
      {
        const int tr = lane & 15, g = lane >> 4;
        put_state(g ^ ((tr >> 2) & 1), tr);  // the entry state as the first chunk's operand
      }
      __syncthreads();  // (matched by the output waves)
      form_u(c_lo, X);
      fetch_r(c_lo, X);
      wait_vm0();
      for (int c = c_lo; c < c_hi; c += 2) {
        chunk(c, X, Y);
        if (c + 1 >= c_hi) break;
        chunk(c + 1, Y, X);
      }
    }
  } else {
    // ---- output waves
    constexpr int OSV = DK == 128 ? 0 : NVT / 2;  // first value tile of the state update
    struct Ops {
      bf16x8 qf[NKB];
      bf16x8 mh[2], ml[2];
      bf16x8 kh[2], kl[2];
      floatx4 gc;
    };
    // (Gamma*Q) and Mqk frames (fetched during the (Gamma*Q) S of the chunk
    // before) and the state-update operands (fetched during its update)
    auto fetch_w = [&](int c, Ops& op) {
      if constexpr (SUMMARY) return;  // no output: only the state update
      const unsigned char* b = item_base(c);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) op.qf[kb] = *frame_ptr<bf16x8>(b, IM::q_frame(w, kb), lane);

#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // key block 1 of tiles 0 and 1 lies after the tile: its frames are
        // zero and not stored; block 0 is fetched again in their place (the
        // fetch stays unconditional) and zeroed when used
        const int kbm = kb > (w >> 1) ? 0 : kb;
        op.mh[kb] = *frame_ptr<bf16x8>(b, IM::m_frame(w, kbm, 0), lane);
        op.ml[kb] = *frame_ptr<bf16x8>(b, IM::m_frame(w, kbm, 1), lane);
      }
    };
    auto fetch_r = [&](int c, Ops& op) {
      const unsigned char* b = item_base(c);
      op.gc = *reinterpret_cast<const floatx4*>(b + IM::g_off + 4 * (16 * srt + 4 * (lane >> 4)));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        op.kh[kb] = *frame_ptr<bf16x8>(b, IM::k_frame(srt, kb, 0), lane);
        op.kl[kb] = *frame_ptr<bf16x8>(b, IM::k_frame(srt, kb, 1), lane);
      }
    };
    // o of chunk c through this wave's LDS staging area: a quad transpose
    // gives each lane four consecutive values of row 4g + (tr & 3), stored as
    // one 16-byte word; read back, each store instruction covers whole rows of
    // the slice (64 / (BV / 4) of them).  The descriptor spans the chunk's nv
    // rows.
    auto store_o = [&](int c, const floatx4 (&ov)[NVT], int tr, int g, int lane_x) {
      if constexpr (!SUMMARY) {
        const long long tok0 = start + (long long)c * CH;
        const int nv = (int)(len - (long long)c * CH < CH ? len - (long long)c * CH : CH);
        float* os = OS + w * 16 * ldO;
        const int b = tr & 3;
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
          *reinterpret_cast<floatx4*>(os + (4 * g + b) * ldO + 16 * vt + 4 * (tr >> 2)) =
              quad_transpose(ov[vt], b);
        const size_t rowel = (size_t)H * DV;  // elements from one token to the next
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            o + ((size_t)tok0 * H + h) * DV + vcol0, 0, (int)((size_t)nv * rowel * sizeof(TOut)),
            0x00020000);
        constexpr int LPO = BV / 4;    // lanes per o row
        constexpr int RPI = 64 / LPO;  // rows per store instruction
#pragma unroll
        for (int q4 = 0; q4 < 16 / RPI; ++q4) {
          const int row = RPI * q4 + lane_x / LPO;
          const int cq = 4 * (lane_x % LPO);
          const floatx4 y = *reinterpret_cast<const floatx4*>(os + row * ldO + cq);
          store4<TOut>(rs, (int)(((size_t)(16 * w + row) * rowel + cq) * sizeof(TOut)), y);
        }
      }
    };
    // One chunk.  The o of the chunk before is stored during this chunk's
    // (Gamma*Q) S, where the output waves wait for the chain's W S anyway, and
    // the updated state goes to LDS right after the update: neither holds up
    // the next chunk's first barrier.
    floatx4 ovp[NVT];  // o of the chunk before
    // the low halves of Gamma*Q of tile 0 of the sequence's first chunk (wave
    // 0 only), fetched with the first chunk's other operands
    bf16x8 qlb[NKB];
    auto fetch_ql = [&](int c) {
      if constexpr (!SUMMARY) {
        if (w == 0) {
          const unsigned char* b = item_base(c);
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) qlb[kb] = *frame_ptr<bf16x8>(b, IM::ql_frame(kb), lane);
        }
      }
    };
    auto chunk = [&](int c, const Ops& op, Ops& nx) {
      int lane_x = lane;
      __asm__ volatile("" : "+v"(lane_x));
      const int tr = lane_x & 15;
      const int g = lane_x >> 4;
      const int gs = g ^ ((tr >> 2) & 1);
      __syncthreads();
      fetch_w(next_of(c), nx);
      // ---- (Gamma*Q) S over both channel halves (separate chains, low half first)
      floatx4 ov[NVT];
      if constexpr (!SUMMARY) {
        floatx4 a0[NVT], a1[NVT];
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
          a0[vt] = floatx4{0.f, 0.f, 0.f, 0.f};
          a1[vt] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int vt = 0; vt < NVT; ++vt) {
            const bf16x8 bh = frag_ld(ST, ldS, 16 * vt + tr, 32 * kb, gs);
            const bf16x8 bl = frag_ld(ST + loS, ldS, 16 * vt + tr, 32 * kb, gs);
            floatx4& acc = kb < NKH ? a0[vt] : a1[vt];
            acc = mfma_bf16(op.qf[kb], bh, acc);
            acc = mfma_bf16(op.qf[kb], bl, acc);
          }
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) ov[vt] = a0[vt] + a1[vt];
        if (c > c_lo) store_o(c - 1, ovp, tr, g, lane_x);
        // tile 0 of the sequence's first chunk keeps Gamma*Q split: its low
        // halves times the state's high halves join o before the second
        // barrier (after it the chain waves overwrite ST with the updated
        // state)
        if (w == 0 && c == 0) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt)
              ov[vt] = mfma_bf16(qlb[kb], frag_ld(ST, ldS, 16 * vt + tr, 32 * kb, gs), ov[vt]);
        }
      }
      __syncthreads();
      fetch_r(next_of(c), nx);
      // ---- O += Mqk P and the state update of this wave's tiles, from the
      // same P fragments (the Mqk block after the tile enters as zeros)
      bf16x8 mh1{}, ml1{};  // (no output in the summary mode: its frames are not fetched)
      if (!SUMMARY && w >= 2) {
        mh1 = op.mh[1];
        ml1 = op.ml[1];
      }
#pragma unroll
      for (int j = 0; j < KVT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) Sacc[j][i] *= op.gc[i];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
          const bf16x8 bh = frag_ld(PT, ldP, 16 * vt + tr, 32 * kb, gs);
          const bf16x8 bl = frag_ld(PT + loP, ldP, 16 * vt + tr, 32 * kb, gs);
          if constexpr (!SUMMARY)
            ov[vt] = mma_ab(kb ? mh1 : op.mh[0], kb ? ml1 : op.ml[0], bh, bl, ov[vt]);
          if (vt >= OSV && vt < OSV + KVT)
            Sacc[vt - OSV] = mma_ab(op.kh[kb], op.kl[kb], bh, bl, Sacc[vt - OSV]);
        }
      put_state(gs, tr);  // ST is not read after the second barrier
      if constexpr (!SUMMARY) {
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) ovp[vt] = ov[vt];
      }
    };
    if (c_lo < c_hi) {
      Ops X, Y;
      fetch_w(c_lo, X);
      fetch_r(c_lo, X);
      if (c_lo == 0) fetch_ql(c_lo);
      {
        const int tr = lane & 15, g = lane >> 4;
        put_state(g ^ ((tr >> 2) & 1), tr);
      }
      __syncthreads();  // the chain waves' staging of the first chunk's v rows
      wait_vm0();
      for (int c = c_lo; c < c_hi; c += 2) {
        chunk(c, X, Y);
        if (c + 1 >= c_hi) break;
        chunk(c + 1, Y, X);
      }
      {
        int lane_x = lane;
        __asm__ volatile("" : "+v"(lane_x));
        store_o(c_hi - 1, ovp, lane_x & 15, lane_x >> 4, lane_x);
      }
    }
  }

  if (SUMMARY || seg == ns - 1) {
    const int tr = lane & 15, g = lane >> 4;
    float* sf = SUMMARY ? summ + (((size_t)seg * n_seq + seq) * H + h) * DK * SWC
                        : carry + ((size_t)seq * H + h) * DK * DV;
#pragma unroll
    for (int j = 0; j < KVT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * srt + 4 * g + i;
        sf[(size_t)row * SWC + vcol0 + 16 * (sv0 + j) + tr] = Sacc[j][i];
      }
  }
}

// Entry states of the segments of one window, for a sequence with ns > 1
// segments: E_0 is the state entering the window (the initial state in the
// sequence's first window, else the carried one) and E_{s+1} = M_s E_s + b_s,
// the composition of the segment maps ("Kimi K3模型架构详解" section 3.6).
// One workgroup of 8 waves per (sequence, head, 32-column slice of the state);
// wave w owns row tile w % (Dk / 16) and Dk / 64 of the two column tiles.  The
// slice of E_s sits in LDS as the split (high, low bf16) B operand,
// [column][row], in one of two buffers (one barrier per step); rows of M_s are
// the split A fragments; each product is the three-term split-bf16 MFMA
// product of the state pass, added to b_s in fp32.  A step's M_s rows and b_s
// are fetched three steps ahead: one step's work is shorter than a memory
// access.  A step costs about 3 us on MI355X (the chain of barrier, LDS reads,
// MFMAs and LDS writes of few waves), so the combine grows with the segment
// count; more independent MFMA chains per step did not shorten it.
template <int DK, int DV>
__global__ __launch_bounds__(512) void segment_combine_kernel(
    const float* __restrict__ summ, float* __restrict__ seg_in,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ chunk_off,
    const float* s_init, const float* carry, int n_seq, int T, int H, long long tok_lo,
    long long tok_hi, int cap, int nseg) {
  constexpr int SC = 32, SWC = DK + DV, ld = DK + 8, NKB = DK / 32;
  constexpr int NRT = DK / 16, CTW = NRT / 4;  // row tiles; column tiles per wave
  constexpr int BUF = 2 * SC * ld;             // one buffer: high parts, then low parts
  __shared__ __align__(16) bf16 EB[2 * BUF];
  constexpr int nsl = DV / SC;
  const int sl = blockIdx.x % nsl, h = (blockIdx.x / nsl) % H, seq = blockIdx.x / (nsl * H);
  const SeqWindow sw = seq_window(cu_seqlens, chunk_off, n_seq, T, seq, tok_lo, tok_hi, cap);
  const int ns = seg_count(nseg, sw.c_lo, sw.c_hi);
  if (ns <= 1) return;  // the state pass enters from the state itself
  const float* src = sw.c_lo == 0 ? s_init : carry;
  const float* si = src ? src + ((size_t)seq * H + h) * DK * DV : nullptr;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, tr = lane & 15, g = lane >> 4;
  const int rt = w % NRT, ct0 = (w / NRT) * CTW;
  const int col0 = sl * SC;
  const size_t head = ((size_t)seq * H + h) * DK * DV;
  const size_t seg_stride = (size_t)n_seq * H * DK * DV;
  struct Step {
    floatx4 m[NKB][2];  // M_s row 16 rt + tr, columns 32 kb + 8 g ..
    floatx4 b[CTW];     // b_s rows 16 rt + 4 g + i, this lane's column of tile j
  };
  auto fetch = [&](int s, Step& st) {
    const float* ms = summ + (((size_t)s * n_seq + seq) * H + h) * DK * SWC;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const float* mr = ms + (size_t)(16 * rt + tr) * SWC + 32 * kb + 8 * g;
      st.m[kb][0] = *reinterpret_cast<const floatx4*>(mr);
      st.m[kb][1] = *reinterpret_cast<const floatx4*>(mr + 4);
    }
#pragma unroll
    for (int j = 0; j < CTW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st.b[j][i] = ms[(size_t)(16 * rt + 4 * g + i) * SWC + DK + col0 + 16 * (ct0 + j) + tr];
  };
  floatx4 acc[CTW];
  auto put = [&](bf16* E) {
#pragma unroll
    for (int j = 0; j < CTW; ++j) {
      float x4[4] = {acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
      st_split4(E + (16 * (ct0 + j) + tr) * ld + 16 * rt + 4 * g, SC * ld, x4);
    }
  };
  // a ring of three steps' operands, fetched three steps ahead (the chain is
  // unrolled over its at most kMaxSegments - 1 steps, so every ring index is a
  // constant)
  constexpr int RING = 3;
  Step ring[RING];
#pragma unroll
  for (int s = 0; s < RING; ++s)
    if (s + 1 < ns) fetch(s, ring[s]);
  if (si) {
#pragma unroll
    for (int j = 0; j < CTW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[j][i] = si[(size_t)(16 * rt + 4 * g + i) * DV + col0 + 16 * (ct0 + j) + tr];
  } else {
#pragma unroll
    for (int j = 0; j < CTW; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int j = 0; j < CTW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      seg_in[head + (size_t)(16 * rt + 4 * g + i) * DV + col0 + 16 * (ct0 + j) + tr] = acc[j][i];
  put(EB);
  __syncthreads();
#pragma unroll
  for (int s = 0; s < kMaxSegments - 1; ++s) {
    if (s + 1 >= ns) break;
    Step& cur = ring[s % RING];
    const bf16* E = EB + (s & 1) * BUF;
#pragma unroll
    for (int j = 0; j < CTW; ++j) acc[j] = cur.b[j];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const float x8[8] = {cur.m[kb][0][0], cur.m[kb][0][1], cur.m[kb][0][2], cur.m[kb][0][3],
                           cur.m[kb][1][0], cur.m[kb][1][1], cur.m[kb][1][2], cur.m[kb][1][3]};
      bf16x8 ah, al;
      split8(x8, ah, al);
#pragma unroll
      for (int j = 0; j < CTW; ++j) {
        const bf16x8 bh = frag_ld(E, ld, 16 * (ct0 + j) + tr, 32 * kb, g);
        const bf16x8 bl = frag_ld(E + SC * ld, ld, 16 * (ct0 + j) + tr, 32 * kb, g);
        acc[j] = mma_ab(ah, al, bh, bl, acc[j]);
      }
    }
    // the ring slot just used takes the step RING ahead
    if (s + RING + 1 < ns) fetch(s + RING, cur);
    float* out = seg_in + (size_t)(s + 1) * seg_stride + head;
#pragma unroll
    for (int j = 0; j < CTW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[(size_t)(16 * rt + 4 * g + i) * DV + col0 + 16 * (ct0 + j) + tr] = acc[j][i];
    if (s + 2 < ns) {
      // the other buffer was last read in the step before, ahead of its barrier
      put(EB + ((s + 1) & 1) * BUF);
      __syncthreads();
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

// value slice of one state-pass workgroup: 64 columns.  32 (twice the
// workgroups, every frame fetched by four instead of two) is slower: the pass
// is bound by frame fetches per compute unit, not by idle compute units.
constexpr int BV_STATE = 64;

template <int DK, int DV, typename TOut, bool SUMMARY>
hipError_t launch_state_t(const PrefillArgs& a, const unsigned char* img, const int32_t* chunk_off,
                          float* carry, long long tok_lo, long long tok_hi, int cap,
                          const SegmentArgs& sg) {
  constexpr int BV = BV_STATE;
  using L = StatePlan<DK, BV>;
  auto kern = prefill_state_kernel<DK, DV, BV, TOut, SUMMARY>;
  static bool attr_set = false;  // per instantiation; idempotent if raced
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, L::total);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int cols = SUMMARY ? DK + DV : DV;
  const int grid = (SUMMARY ? sg.nseg - 1 : sg.nseg) * a.n_seq * a.H * (cols / BV);
  if (grid <= 0) return hipSuccess;
  // the layer prefill's v exists only in the operand blocks (the first pass's
  // prologue formed it); otherwise the state pass reads the caller's v
  const bf16* v = a.pro ? nullptr : static_cast<const bf16*>(a.v);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTH_S), L::total, (hipStream_t)a.stream, img, chunk_off,
                     a.cu_seqlens, a.initial_state, carry, (TOut*)a.o, v, a.n_seq, a.T, a.H,
                     tok_lo, tok_hi, cap, sg.nseg, sg.seg_in, sg.summ);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_state_d(const PrefillArgs& a, const unsigned char* img, const int32_t* chunk_off,
                          float* carry, long long tok_lo, long long tok_hi, int cap,
                          const SegmentArgs& sg, bool summary) {
  if (summary)  // no output: one instantiation
    return launch_state_t<DK, DV, float, true>(a, img, chunk_off, carry, tok_lo, tok_hi, cap, sg);
  return a.o_bf16
             ? launch_state_t<DK, DV, bf16, false>(a, img, chunk_off, carry, tok_lo, tok_hi, cap, sg)
             : launch_state_t<DK, DV, float, false>(a, img, chunk_off, carry, tok_lo, tok_hi, cap, sg);
}

template <int DK, int DV>
hipError_t launch_combine_t(const PrefillArgs& a, const int32_t* chunk_off, float* carry,
                            long long tok_lo, long long tok_hi, int cap, const SegmentArgs& sg) {
  const int grid = a.n_seq * a.H * (DV / 32);
  hipLaunchKernelGGL((segment_combine_kernel<DK, DV>), dim3(grid), dim3(512), 0,
                     (hipStream_t)a.stream, sg.summ, sg.seg_in, a.cu_seqlens, chunk_off,
                     a.initial_state, carry, a.n_seq, a.T, a.H, tok_lo, tok_hi, cap, sg.nseg);
  return hipGetLastError();
}

hipError_t state_dispatch(const PrefillArgs& a, const unsigned char* img, const int32_t* chunk_off,
                          float* carry, long long tok_lo, long long tok_hi, int cap,
                          const SegmentArgs& sg, bool summary) {
  if (a.Dk == 128)
    return a.Dv == 128 ? launch_state_d<128, 128>(a, img, chunk_off, carry, tok_lo, tok_hi, cap, sg, summary)
                       : launch_state_d<128, 64>(a, img, chunk_off, carry, tok_lo, tok_hi, cap, sg, summary);
  return a.Dv == 128 ? launch_state_d<64, 128>(a, img, chunk_off, carry, tok_lo, tok_hi, cap, sg, summary)
                     : launch_state_d<64, 64>(a, img, chunk_off, carry, tok_lo, tok_hi, cap, sg, summary);
}

}  // namespace

hipError_t launch_prefill_state(const PrefillArgs& a, const unsigned char* img,
                                const int32_t* chunk_off, float* carry, long long tok_lo,
                                long long tok_hi, int cap, const SegmentArgs& sg) {
  if (sg.nseg > 1) {
    if (hipError_t e = state_dispatch(a, img, chunk_off, carry, tok_lo, tok_hi, cap, sg, true);
        e != hipSuccess)
      return e;
    hipError_t e;
    if (a.Dk == 128)
      e = a.Dv == 128 ? launch_combine_t<128, 128>(a, chunk_off, carry, tok_lo, tok_hi, cap, sg)
                      : launch_combine_t<128, 64>(a, chunk_off, carry, tok_lo, tok_hi, cap, sg);
    else
      e = a.Dv == 128 ? launch_combine_t<64, 128>(a, chunk_off, carry, tok_lo, tok_hi, cap, sg)
                      : launch_combine_t<64, 64>(a, chunk_off, carry, tok_lo, tok_hi, cap, sg);
    if (e != hipSuccess) return e;
  }
  return state_dispatch(a, img, chunk_off, carry, tok_lo, tok_hi, cap, sg, false);
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
