// State pass of the matrix-core chunked prefill: walks the pairs of 16-token
// tiles of one head in order with the float32 state resident in matrix-core
// accumulators, consuming the per-pair records of the tile builder
// (kda_chunk_rec.h):
//   D_a = T_a V_a - W_a S                 O_a = Qh_a S + Aqk_a D_a
//   D_b = T_b V_b - W_b' S + P D_a        O_b = Qh_b' S + Q_ba D_a + Aqk_b D_b
//   S  <- Diag(E_a E_b) S + [Kb_a' | Kb_b]^T [D_a ; D_b]
// ("Kimi K3: Engineering a 2.8 Trillion Parameter Frontier", section
// "Dimension 1"), and, when a gate is given, the head-wise RMSNorm x
// sigmoid(gate) epilogue ("Kimi K3 Architecture Explained ...", section
// "Token mixing").
//
// One launch per segment of pairs.  The first workgroups of the launch run
// the state pass over the segment; the remaining ones build the records of
// the next segment (kda_chunk_tile.h) into the other half of the workspace.
//
// A state workgroup owns one (b, h) and DVW of its value columns (all 128, or
// 64 when two workgroups share a head).  It has two kinds of wavefronts:
//   state waves (DVW / CPW): each keeps CPW state columns x 128 rows in 16x16
//     accumulators, rows in the permuted channel order of the record, so that
//     the state is the k-operand of its own products without moving between
//     lanes:
//       D   (lane (c, g): D[4 g + r][c])         16x16x32 products over slabs
//       O^T (lane (t, g): O[t][4 g + r])         transposed: each lane holds 4
//                                                consecutive output columns of one token
//       S_b <- E * S_b + Kb^T_b [D_a ; D_b]      one 16x16x32 product per block
//     V is moved from its token-major rows into the k-operand layout by a bf16
//     product with a 0/1 selection matrix (exact).
//   loader waves (kLoaders): copy each pair's record and v rows into an LDS
//     ring slot, and its gate rows into a slot of a second ring, from memory
//     with direct-to-LDS loads, kLead pairs ahead of the state waves, and wait
//     for the next pair's copies before the barrier that ends a step; with
//     the gate they also turn the gate rows of the pair being consumed into
//     w * sigmoid(gate) (float16) in place.
// One barrier per step (pair).  The output of pair x is normalised and
// written during step x + 1, once the row sums of squares of all state waves
// are in LDS, so its arithmetic fills the matrix-core chains of the next
// pair; its gate rows outlive its record slot by a step, hence the second
// ring.  Each accumulation chain uses a single matrix instruction shape.
//
// LDS ring slot: [record][v rows]; gate slot: [gate rows].  The v and gate
// areas hold 32 rows of DVW bf16 columns with the 16-byte chunk u of row t
// stored at chunk position swz(t, u), so that the 8-byte reads of the state
// waves (one token per lane, 4 columns) fall in distinct banks.
//
// Precision: the state and every accumulation are float32; the state, V and
// D enter the products as float16 (11-bit significand).  Float16's range is
// kept out of the way by a power-of-two scale per state wavefront: the method
// is linear in (V, S) for fixed q, k, g, beta, so each wavefront runs on
// sigma V and sigma S (its own value columns; columns are independent) and
// divides its outputs and stored states by sigma, all exactly.  Before each
// pair it takes the largest magnitude m of its scaled state and values; when
// m leaves [2^2, 2^11) it rescales the accumulators so that m lands in
// [2^9, 2^10) (then |D| < 2^15 with unit keys), which keeps every float16
// operand normal and finite for any float32 state or bfloat16 values.
#include <stdlib.h>

#include <type_traits>

#include "kda_chunk_rec.h"
#include "kda_chunk_tile.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kLoaders = 4;  // loader wavefronts, one per SIMD

// s_waitcnt with vmcnt = N and the other counters left alone (gfx9 encoding).
constexpr unsigned vmcnt_imm(int n) {
  return (unsigned)((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt with vmcnt = N and lgkmcnt = 0.
constexpr unsigned vmcnt_lgkm0_imm(int n) { return vmcnt_imm(n) & ~(0xFu << 8); }

// x with its k-values 0..3 replaced by lo (4..7 kept).
__device__ __forceinline__ f16x8 with_low(f16x8 x, f16x4 lo) {
  const f16x8 l8 = __builtin_shufflevector(lo, lo, 0, 1, 2, 3, -1, -1, -1, -1);
  return __builtin_shufflevector(l8, x, 0, 1, 2, 3, 12, 13, 14, 15);
}

// Elements 4 h .. 4 h + 3 of x (h = 0 or 1).
__device__ __forceinline__ bf16x4 half4(bf16x8 x, int h) {
  return h == 0 ? __builtin_shufflevector(x, x, 0, 1, 2, 3) : __builtin_shufflevector(x, x, 4, 5, 6, 7);
}

// A slot is a whole number of 1 KB blocks (one direct-to-LDS load of a wave
// each); every block holds only record bytes or only v / gate bytes.
template <int DVW, bool GATE>
struct SlotCfg {
  static constexpr int kRowB = DVW * 2;                  // bytes per v / gate row
  static constexpr int kCpr = DVW / 8;                   // 16-byte chunks per row
  static constexpr int kRowsB = rec::kP * kRowB;         // bytes of a pair's v (or gate) rows
  static constexpr int kRecBlocks = (rec::kBytes + 1023) / 1024;
  static constexpr int kV = kRecBlocks * 1024;           // v rows offset in a slot
  static constexpr int kData = kV + kRowsB;
  static constexpr int kInstr = kLoaders * 1024;         // bytes per loader round
  static constexpr int kSlot = (kData + kInstr - 1) / kInstr * kInstr;
  static constexpr int kGSlot = GATE ? kRowsB : 0;       // gate slot
  static constexpr int kPer = (kSlot + kGSlot) / kInstr; // loads per loader wave per pair
  // Ring: the pair being consumed and kLead pairs in flight, within 150 KB
  // with the gate ring (kLead + 2 slots: the gate of the pair before is read
  // by the epilogue of the step, that of the pair consumed is converted).
  static constexpr int kRing = (150 * 1024 / (kSlot + kGSlot)) < 4
                                   ? (150 * 1024 / (kSlot + kGSlot)) : 4;
  static constexpr int kLead = kRing - 1;
  static constexpr int kGRing = GATE ? kLead + 2 : 0;
  static_assert(kRowsB % 1024 == 0 && kGSlot % kInstr == 0, "v and gate rows must be whole rounds");
  static_assert(kLead >= 1, "the ring needs a slot in flight");
  static constexpr int kRowsPerBankLine = 256 / kRowB;   // rows sharing the 64 banks
  // Chunk position of chunk u of row t (an involution in u for fixed t).
  static __device__ __forceinline__ int swz(int t, int u) {
    return u ^ ((t / kRowsPerBankLine) % kCpr);
  }
};

template <int DVW, int CPW, bool GATE, bool WO, bool PACKED, bool LOGITS>
__global__ void __launch_bounds__(64 * (DVW / CPW + kLoaders), 1)
kda_state_kernel(const unsigned char* __restrict__ recs, const bf16_t* __restrict__ v,
                 const float* __restrict__ s_in, float* __restrict__ s_next,
                 bf16_t* __restrict__ o, const bf16_t* __restrict__ gate,
                 const float* __restrict__ norm_w, float eps, Seqs<PACKED> seqs, int64_t H,
                 int64_t BH,
                 int64_t x0, int64_t nseg, int64_t n_state_wg, float* __restrict__ ckpt,
                 int64_t ckpt_every, bool ckpt_frag, float scale,
                 tile::Args<PACKED, LOGITS> next) {
  using SC = SlotCfg<DVW, GATE>;
  constexpr int kRing = SC::kRing, kLead = SC::kLead;
  constexpr int NSW = DVW / CPW;   // state wavefronts
  constexpr int NCB = CPW / 16;    // 16-column blocks per state wavefront
  static_assert(NCB == 2, "a lane's output columns are one 16-byte run of both column blocks");
  constexpr int NSPLIT = rec::kDV / DVW;
  static_assert(CPW % 16 == 0 && DVW % CPW == 0 && rec::kDV % DVW == 0, "bad column split");
  static_assert(!GATE || NSPLIT == 1, "the gated RMSNorm needs a head's full dv row");
  static_assert(!GATE || WO, "the gated epilogue only shapes the output");
  static_assert(kLead * SC::kPer <= 63, "outstanding loads per loader wave exceed vmcnt");

  constexpr int NW = NSW + kLoaders;  // wavefronts per workgroup
  constexpr int kRingB = kRing * SC::kSlot;
  constexpr int kGRingB = SC::kGRing * SC::kGSlot;
  constexpr int kRsB = 2 * rec::kP * NSW * 4;
  constexpr int kStateB = kRingB + kGRingB + kRsB;
  constexpr int kTileB = NW * (int)sizeof(tile::Scratch);
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kStateB > kTileB ? kStateB : kTileB];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // wave-uniform
  const int lane = tid % 64;
  const int lc = lane % 16, lg = lane / 16;

  if ((int64_t)blockIdx.x >= n_state_wg) {
    // ======================== tile workgroups: records of the next segment
    tile::Scratch* scratch = (tile::Scratch*)lds;
    const int64_t first = ((int64_t)blockIdx.x - n_state_wg) * NW + wave;
    const int64_t stride = ((int64_t)gridDim.x - n_state_wg) * NW;
    tile::build_range(next, first, stride, &scratch[wave], lane);
    return;
  }

  // ======================= state workgroups: the pairs of this segment
  unsigned char (*ring)[SC::kSlot] = (unsigned char (*)[SC::kSlot])lds;
  unsigned char* gring = lds + kRingB;  // gate slots of kGSlot bytes
  // row sums of O^2, [pair & 1][token of pair][wave]
  float (*rs)[rec::kP][NSW] = (float (*)[rec::kP][NSW])(lds + kRingB + kGRingB);

  // Keep the NSPLIT workgroups of one head on one XCD (workgroups are dealt
  // round-robin over the 8 XCDs) so that they share its records in L2.
  int64_t wg = blockIdx.x;
  const int64_t total = n_state_wg;  // BH * NSPLIT
  if (NSPLIT > 1 && total % 8 == 0) wg = (wg % 8) * (total / 8) + wg / 8;
  const int64_t bh = wg / NSPLIT;
  const int col0 = (int)(wg % NSPLIT) * DVW;  // first value column of the workgroup
  const int64_t b = bh / H, h = bh % H;
  // This head's sequence: T tokens from row t0.  Only its live pairs (those
  // with a token of the sequence) are walked; past them the state is carried
  // unchanged (the tile workgroups build no records for them either).
  const int64_t T = seqs.len(b), t0 = seqs.start(b);
  int64_t live = (T + rec::kP - 1) / rec::kP - x0;
  live = live < 0 ? 0 : (live > nseg ? nseg : live);

  const int64_t rstride = H * rec::kDV;  // elements between consecutive tokens of a head

  if (wave >= NSW) {
    // ========================================================== loader waves
    const int lw = wave - NSW;
    const unsigned char* R0 = recs + bh * nseg * (int64_t)rec::kBytes;
    // Block i kLoaders + lw of a pair (its slot's blocks, then its gate
    // slot's) is this wave's i-th load.  Its kind and this lane's source
    // offset are fixed; a pair only moves the base.
    //   record block j:  R0 + x * kBytes + 16 (64 j + lane)   (the padding of the
    //                    last record block re-reads record chunks)
    //   v / gate block:  row t (of 32), column chunk u of the pair:
    //                    base_x + t * row stride + 2 (col0 + 8 u)
    int kind[SC::kPer];        // 0 record, 1 v, 2 gate (wave-uniform)
    unsigned loff[SC::kPer];   // byte offset from the pair base (full pairs)
    int lrow[SC::kPer], lcol[SC::kPer];
#pragma unroll
    for (int i = 0; i < SC::kPer; ++i) {
      const int blk = i * kLoaders + lw;
      const int c = blk * 64 + lane;
      if (blk < SC::kRecBlocks) {
        kind[i] = 0;
        // record bytes to copy: the norm area only when q and k are normalised here
        constexpr int kRead = LOGITS ? rec::kBytes : rec::kNorm;
        loff[i] = 16u * (unsigned)(c < kRead / 16 ? c : c - 64);
        lrow[i] = lcol[i] = 0;
      } else {
        int q = (blk < SC::kSlot / 1024 ? blk - SC::kRecBlocks : blk - SC::kSlot / 1024) * 64 + lane;
        kind[i] = blk < SC::kSlot / 1024 ? 1 : 2;  // v rows (and the slot's padding) or gate rows
        q %= SC::kRowsB / 16;  // the padding re-reads v rows
        const int t = q / SC::kCpr, u = SC::swz(t, q % SC::kCpr);
        lrow[i] = t;
        lcol[i] = col0 + 8 * u;
        loff[i] = (unsigned)(2 * (t * rstride + lcol[i]));
      }
    }
    // Copy pair xt (< live) into ring slot `slot` and gate slot `gslot`.
    const bf16_t* vg = GATE ? gate : v;
    auto issue = [&](int64_t xt, int slot, int gslot) {
      const int64_t row0 = (x0 + xt) * rec::kP;               // first token of the pair
      const bool full = row0 + rec::kP <= T;
      const unsigned char* base_r = R0 + xt * rec::kBytes;
      const int64_t pair0 = ((t0 + row0) * H + h) * rec::kDV;  // element offset of row 0 (full)
      const unsigned char* base_v = (const unsigned char*)(v + pair0);
      const unsigned char* base_g = (const unsigned char*)(vg + pair0);
#pragma unroll
      for (int i = 0; i < SC::kPer; ++i) {
        const unsigned char* src =
            (kind[i] == 0 ? base_r : (kind[i] == 2 ? base_g : base_v)) + loff[i];
        if (kind[i] != 0 && !full) {
          // a pair at or past the sequence's end: rows clamped into the sequence
          // (their tokens are identity tokens; the values read do not matter)
          const int64_t r = seqs.row(b, row0 + lrow[i]);
          src = (const unsigned char*)((kind[i] == 2 ? vg : v) + (r * H + h) * rec::kDV +
                                       lcol[i]);
        }
        const int blk = i * kLoaders + lw;
        unsigned char* dst = blk < SC::kSlot / 1024
                                 ? ring[slot] + blk * 1024
                                 : gring + gslot * SC::kGSlot + (blk - SC::kSlot / 1024) * 1024;
        // Records keep the default cache policy (they were just written and
        // are read once from the memory-side cache); v and gate rows are read
        // once from HBM and are loaded non-temporal (cache-policy bit nt).
        if (kind[i] == 0)
          __builtin_amdgcn_global_load_lds(
              (const __attribute__((address_space(1))) void*)src,
              (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        else
          __builtin_amdgcn_global_load_lds(
              (const __attribute__((address_space(1))) void*)src,
              (__attribute__((address_space(3))) void*)dst, 16, 0, 2);
      }
    };
    // Gate chunks of this lane (GATE: the pair's 32 gate rows are
    // kGateChunks 16-byte chunks, kGatePer per loader lane): replaced in place
    // by w * sigmoid(gate) in float16 before the barrier after which the
    // state waves read them.
    constexpr int kGateChunks = SC::kRowsB / 16;
    constexpr int kGatePer = kGateChunks / (kLoaders * 64);
    static_assert(!GATE || kGatePer * kLoaders * 64 == kGateChunks, "whole gate chunks per lane");
    // Gate chunk gp sits in the pair's block kSlot / 1024 + gp / 64, loaded
    // by loader wave (that block) % kLoaders = lw: each loader wave converts
    // only blocks that its own vmcnt wait has seen complete.
    static_assert((SC::kSlot / 1024) % kLoaders == 0,
                  "gate blocks must be converted by the wave that loaded them");
    float gw[kGatePer > 0 ? kGatePer : 1][8];
#pragma unroll
    for (int j = 0; j < kGatePer; ++j) {
      const int gp = (j * kLoaders + lw) * 64 + lane;             // chunk position in the rows
      const int gu = SC::swz(gp / SC::kCpr, gp % SC::kCpr);       // its column chunk
#pragma unroll
      for (int e = 0; e < 8; ++e)
        gw[j][e] = (GATE && norm_w != nullptr) ? norm_w[col0 + 8 * gu + e] : 1.f;
    }
    // The chunks were completed before the last barrier; the direct-to-LDS
    // loads still in flight target other slots.  Plain loads and stores here
    // would make the compiler wait for all of those loads first, so the LDS
    // accesses are issued directly.
    auto convert_gate = [&](int gslot) {
#pragma unroll
      for (int j = 0; j < kGatePer; ++j) {
        const int gp = (j * kLoaders + lw) * 64 + lane;
        const unsigned addr = lds_addr(gring + gslot * SC::kGSlot + 16 * gp);
        const bf16x8 x = __builtin_bit_cast(bf16x8, ds_read16(addr));
        f16x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          y[e] = (f16)(gw[j][e] * __builtin_amdgcn_rcpf(
                                      1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * (float)x[e])));
        ds_write16(addr, as_f4(y));
      }
    };
    // No loads past the segment's last pair: the waits below count the loads
    // in flight, so near the end (fewer pairs in flight) they wait for all.
#pragma unroll
    for (int y = 0; y < kLead; ++y)
      if (y < live) issue(y, y, y);
    if (kLead <= live)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((kLead - 1) * SC::kPer));  // pair 0 is in LDS
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_barrier();
    // Ring slot of pair x: x % kRing; gate slot: x % kGRing.
    int slot_issue = kLead, gslot_issue = kLead, gslot_cur = 0;
    for (int64_t xl = 0; xl < live; ++xl) {
      // the slot of pair xl - 1 (free since the last barrier) and the gate
      // slot of pair xl - 2 (read by the epilogue of the last step)
      const bool more = xl + kLead < live;  // a pair to issue (uniform)
      if (more) issue(xl + kLead, slot_issue, gslot_issue);
      slot_issue = slot_issue == kRing - 1 ? 0 : slot_issue + 1;
      if constexpr (GATE) {
        gslot_issue = gslot_issue == SC::kGRing - 1 ? 0 : gslot_issue + 1;
        convert_gate(gslot_cur);  // read by the epilogue of the next step
        gslot_cur = gslot_cur == SC::kGRing - 1 ? 0 : gslot_cur + 1;
      }
      // pair xl + 1 is in LDS; the converted gate is written
      if (more)
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm((kLead - 1) * SC::kPer));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
      __builtin_amdgcn_s_barrier();
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    return;
  }

  // ============================================================ state waves
  const int wl = wave * CPW;  // first column of this wave, in the workgroup
  // Value column of index c in column block cb (a relabelling within the
  // wave's 32 columns): each lane's output elements, rows 4 g + r of both
  // blocks' O^T, are then 8 adjacent columns, wl + 8 g + [0, 8).
  auto vcol = [&](int cb, int c) { return wl + 8 * (c / 4) + 4 * cb + c % 4; };

  // State: block kb of column block cb, lane (c, g), r = row chan(kb, 4 g + r),
  // column vcol(cb, c).
  // It holds sigma S with sigma = 2^sh (wave-uniform), see the precision note.
  f32x4 S[NCB][8];
  int sh = 0;
  float sig = 1.f, isig = 1.f;  // 2^sh, 2^-sh
  // This wave's columns of the state, to a [dk, dv] row-major float32 state at p.
  auto store_state = [&](float* p) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        float* pc = p + col0 + vcol(cb, lc);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          pc[rec::chan(kb, 4 * lg + r) * rec::kDV] = S[cb][kb][r] * isig;
      }
  };
  // The same in accumulator order (16-column group 2 (col0 + wl) / 32 + cb).
  auto store_state_frag = [&](float* p) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      float* pw = p + 2048 * (2 * ((col0 + wl) / 32) + cb) + 4 * lane;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) *(f32x4*)(pw + 256 * kb) = S[cb][kb] * isig;
    }
  };
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      f32x4 x = zero4();
      if (s_in != nullptr) {
        const float* p = s_in + bh * rec::kDK * rec::kDV + col0 + vcol(cb, lc);
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = p[rec::chan(kb, 4 * lg + r) * rec::kDV];
      }
      S[cb][kb] = x;
    }
  // Selection matrix for the v transpose: B[k = 4 g + e][c] = (k == c).
  bf16x4 ident;
#pragma unroll
  for (int e = 0; e < 4; ++e) ident[e] = (bf16_t)((4 * lg + e == lc) ? 1.f : 0.f);
  // LDS byte offset, within the v / gate rows, of this lane's 8 columns
  // vcol(cb, 4 lg + e) (one 16-byte chunk) of token lc (tile a); tile b's
  // token lc is 16 rows further, with the same swizzle (rows 16 apart permute
  // their chunks alike).
  static_assert(16 % SC::kRowsPerBankLine == 0 && (16 / SC::kRowsPerBankLine) % SC::kCpr == 0,
                "rows 16 apart must swizzle alike");
  const int tile_off = lc * SC::kRowB + 16 * SC::swz(lc, (wl + 8 * lg) / 8);

  // Output of pair x: this lane writes tokens lc and 16 + lc, columns
  // col0 + wl + 8 lg + [0, 8).
  const int64_t o_lane = lc * rstride + col0 + wl + 8 * lg;
  auto o_pair = [&](int64_t x) { return o + ((t0 + (x0 + x) * rec::kP) * H + h) * rec::kDV; };
  __syncthreads();  // pair 0 is in LDS

  // Epilogue of pair x: y = O / rms(O) * w * sigmoid(gate), tokens lc and
  // 16 + lc, from the row sums of every state wave and the gate rows that the
  // loader waves converted.
  auto epilogue = [&](int64_t x, const f32x4 (&Pa)[NCB], const f32x4 (&Pb)[NCB]) {
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int w = 0; w < NSW; ++w) {
      sa += rs[x & 1][lc][w];
      sb += rs[x & 1][16 + lc][w];
    }
    const float inva = rsqrtf(sa * (1.f / (float)rec::kDV) + eps);
    const float invb = rsqrtf(sb * (1.f / (float)rec::kDV) + eps);
    const int64_t tok = (x0 + x) * rec::kP + lc;
    const unsigned char* G = gring + (SC::kGRing > 0 ? (int)(x % SC::kGRing) : 0) * SC::kGSlot;
    bf16_t* op = o_pair(x) + o_lane;
    const f16x8 swa = *(const f16x8*)(G + tile_off);
    const f16x8 swb = *(const f16x8*)(G + 16 * SC::kRowB + tile_off);
    bf16x8 ya, yb;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ya[4 * cb + r] = (bf16_t)(Pa[cb][r] * inva * (float)swa[4 * cb + r]);
        yb[4 * cb + r] = (bf16_t)(Pb[cb][r] * invb * (float)swb[4 * cb + r]);
      }
    if (tok < T) __builtin_nontemporal_store(ya, (bf16x8*)op);
    if (tok + rec::kC < T) __builtin_nontemporal_store(yb, (bf16x8*)(op + rec::kC * rstride));
  };

  f32x4 Pa[NCB], Pb[NCB];  // outputs of the previous pair, normalised one step later
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) Pa[cb] = Pb[cb] = zero4();
  // T_a and Aqk_a as 8-wide operands whose k-values 4..7 stay zero: the
  // 16-deep products T_a V_a and D_a^T Aqk_a^T run as 16x16x32 products (one
  // instruction shape per accumulation chain) whatever the other operand
  // holds in those k-values.
  f16x8 ta8 = {}, aa8 = {};
  int slot = 0;  // ring slot of pair xl
  for (int64_t xl = 0; xl < live; ++xl) {
    const bool pfull = (x0 + xl + 1) * rec::kP <= T;  // every token of the pair is in the sequence
    const unsigned char* Rs = ring[slot];

    // The LDS operands are read in batches (those of the D products, those of
    // the O products, those of the state update), each issued before the
    // products that precede its use, so that the step waits for LDS a few
    // times rather than once per product.
    ta8 = with_low(ta8, *(const f16x4*)(Rs + rec::kTa + lane * 8));
    const f16x8 tbp = *(const f16x8*)(Rs + rec::kTbP + lane * 16);
    // lane (t, g), column block cb: V[t][vcol(cb, 4 g + e)], elements 4 cb + e
    const bf16x8 vna = *(const bf16x8*)(Rs + SC::kV + tile_off);
    const bf16x8 vnb = *(const bf16x8*)(Rs + SC::kV + 16 * SC::kRowB + tile_off);
    f16x8 wa[4], wb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      wa[s] = *(const f16x8*)(Rs + rec::kWa + s * 1024 + lane * 16);
      wb[s] = *(const f16x8*)(Rs + rec::kWb + s * 1024 + lane * 16);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (GATE) {
      if (xl > 0) epilogue(xl - 1, Pa, Pb);
    }

    // ---- D_a, D_b.  Every accumulation chain uses one instruction shape,
    // 16x16x32 (a 16x16x16 result fed straight into a 16x16x32 accumulator
    // read stale values on gfx950).
    // V in the k-operand layout, float32 (exact): lane (c, g): V_a[4 g + e][vcol(cb, c)]
    f32x4 vf[NCB][2];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      vf[cb][0] = mma16b(half4(vna, cb), ident, zero4());
      vf[cb][1] = mma16b(half4(vnb, cb), ident, zero4());
    }
    // The scale: the largest magnitude m of sigma S and sigma V, one
    // reduction over the wave.  When m leaves the window (rare) it is taken
    // again with V unscaled (sigma V may have overflowed), and the state and
    // sigma V are moved.
    f32x4 vs[NCB][2];  // sigma V
    {
      float m0 = 0.f, m1 = 0.f;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        vs[cb][0] = vf[cb][0] * sig;
        vs[cb][1] = vf[cb][1] * sig;
#pragma unroll
        for (int r = 0; r < 4; ++r) m0 = fmaxf(m0, fmaxf(fabsf(vs[cb][0][r]), fabsf(vs[cb][1][r])));
#pragma unroll
        for (int kb = 0; kb < 8; kb += 2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            m0 = fmaxf(m0, fabsf(S[cb][kb][r]));
            m1 = fmaxf(m1, fabsf(S[cb][kb + 1][r]));
          }
      }
      // raw keys: D' = Diag(1/|k|) D exceeds D by up to the pair's largest 1/|k|
      int ek = 0;
      if constexpr (LOGITS) {
        ek = exp_of(((const float*)(Rs + rec::kNorm))[32]);
        ek = ek > 0 ? ek : 0;
      }
      // The scale stays when the largest magnitude times 2^ek lies in
      // [2^kLoExp, 2^(kHiExp + 1)) or every value is zero: three lane votes;
      // the reduction across lanes only when it moves.
      const float mm = fmaxf(m0, m1), fk = exp2i(-ek);
      const bool kept =
          __builtin_amdgcn_ballot_w64(mm >= (float)(1 << (kHiExp + 1)) * fk) == 0 &&
          (__builtin_amdgcn_ballot_w64(mm >= (float)(1 << kLoExp) * fk) != 0 ||
           __builtin_amdgcn_ballot_w64(mm > 0.f) == 0);
      int em = kept ? kNoExp : exp_of(wave_max_nonneg(mm));
      if (em != kNoExp) em += ek;
      if (!kept && scale_shift(em, sh) != 0) {  // wave-uniform
        float ms = 0.f, mv = 0.f;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
          for (int r = 0; r < 4; ++r) mv = fmaxf(mv, fmaxf(fabsf(vf[cb][0][r]), fabsf(vf[cb][1][r])));
#pragma unroll
          for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) ms = fmaxf(ms, fabsf(S[cb][kb][r]));
        }
        const int es = exp_of(wave_max_nonneg(ms));
        int ev = exp_of(wave_max_nonneg(mv));
        ev = ev == kNoExp ? kNoExp : ev + sh;
        em = es > ev ? es : ev;
        if (em != kNoExp) em += ek;
        const int d = scale_shift(em, sh);
        if (d != 0) {
          const float f = exp2i(d);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) S[cb][kb] *= f;
          sh += d;
          sig = exp2i(sh);
          isig = exp2i(-sh);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            vs[cb][0] = vf[cb][0] * sig;
            vs[cb][1] = vf[cb][1] * sig;
          }
        }
      }
    }
    f16x8 sop[NCB][4];
    f16x8 dab[NCB];  // [D_a ; D_b] in k-operand order (lane (c, g): D[4 g + e][c])
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
      for (int s = 0; s < 4; ++s) sop[cb][s] = cat8(to_h4(S[cb][2 * s]), to_h4(S[cb][2 * s + 1]));
      const f16x4 va = to_h4(vs[cb][0]);
      const f16x4 vb = to_h4(vs[cb][1]);
      f32x4 d = mma32h(ta8, cat8(va, vb), zero4());  // k-values 4..7 of ta8 are zero
#pragma unroll
      for (int s = 0; s < 4; ++s) d = mma32h(wa[s], sop[cb][s], d);
      const f16x4 da16 = to_h4(d);
      f32x4 e = mma32h(tbp, cat8(vb, da16), zero4());  // T_b V_b + P D_a
#pragma unroll
      for (int s = 0; s < 4; ++s) e = mma32h(wb[s], sop[cb][s], e);
      dab[cb] = cat8(da16, to_h4(e));
    }
    __builtin_amdgcn_sched_barrier(0);
    aa8 = with_low(aa8, *(const f16x4*)(Rs + rec::kAa + lane * 8));
    const f16x8 qbaab = *(const f16x8*)(Rs + rec::kQbaAb + lane * 16);
    f16x8 qa[4], qb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qa[s] = *(const f16x8*)(Rs + rec::kQa + s * 1024 + lane * 16);
      qb[s] = *(const f16x8*)(Rs + rec::kQb + s * 1024 + lane * 16);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- O_a^T, O_b^T (lane (t, g): O[t][4 g + r])
    // With q and k normalised in the kernels, D above is D' = Diag(1/|k|) D
    // (the record's T, W and P rows carry 1/|k|), which is what the raw-key
    // factors Kb, Aqk and Q_ba take, and each output row takes 1/|q| of its token.
    // Every output row is also multiplied by scale / sigma (the records hold
    // the unscaled queries; the state and D are sigma times theirs).
    float rqa = scale * isig, rqb = scale * isig;
    if constexpr (LOGITS) {
      rqa *= ((const float*)(Rs + rec::kNorm))[lc];
      rqb *= ((const float*)(Rs + rec::kNorm))[16 + lc];
    }
    f32x4 Oa[NCB], Ob[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      f32x4 x = zero4(), y = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        x = mma32h(sop[cb][s], qa[s], x);
        y = mma32h(sop[cb][s], qb[s], y);
      }
      Oa[cb] = mma32h(dab[cb], aa8, x) * rqa;    // + D_a^T Aqk_a^T (k-values 4..7 of aa8 are zero)
      Ob[cb] = mma32h(dab[cb], qbaab, y) * rqb;  // + D_a^T Q_ba^T + D_b^T Aqk_b^T
    }
    if constexpr (GATE) {
      float pa = 0.f, pb = 0.f;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pa = fmaf(Oa[cb][r], Oa[cb][r], pa);
          pb = fmaf(Ob[cb][r], Ob[cb][r], pb);
        }
      pa += __shfl_xor(pa, 16);
      pa += __shfl_xor(pa, 32);
      pb += __shfl_xor(pb, 16);
      pb += __shfl_xor(pb, 32);
      if (lg == 0) {
        rs[xl & 1][lc][wave] = pa;
        rs[xl & 1][16 + lc][wave] = pb;
      }
    } else if constexpr (WO) {
      const int64_t tok = (x0 + xl) * rec::kP + lc;
      bf16_t* op = o_pair(xl) + o_lane;
      bf16x8 ya, yb;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ya[4 * cb + r] = (bf16_t)Oa[cb][r];
          yb[4 * cb + r] = (bf16_t)Ob[cb][r];
        }
      if (pfull || tok < T) __builtin_nontemporal_store(ya, (bf16x8*)op);
      if (pfull || tok + rec::kC < T)
        __builtin_nontemporal_store(yb, (bf16x8*)(op + rec::kC * rstride));
    }

    // ---- S <- Diag(E_a E_b) S + [Kb_a' | Kb_b]^T [D_a ; D_b]
    __builtin_amdgcn_sched_barrier(0);
    f16x8 kb8[8];
    f32x4 e4[8];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      kb8[kb] = *(const f16x8*)(Rs + rec::kKb + kb * 1024 + lane * 16);
      e4[kb] = *(const f32x4*)(Rs + rec::kEn + 4 * (32 * (kb / 2) + 8 * lg + 4 * (kb % 2)));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        S[cb][kb] = mma32h(kb8[kb], dab[cb], S[cb][kb] * e4[kb]);

    // State checkpoint after every ckpt_every tokens (a multiple of a pair's 32).
    if (ckpt != nullptr) {
      const int64_t done = (x0 + xl + 1) * rec::kP;  // tokens consumed (uniform)
      if (done % ckpt_every == 0 && done <= T) {
        const int64_t nck = seqs.T / ckpt_every, ic = done / ckpt_every - 1;
        float* pk = ckpt + ((b * nck + ic) * H + h) * (int64_t)(rec::kDK * rec::kDV);
        if (ckpt_frag)
          store_state_frag(pk);
        else
          store_state(pk);
      }
    }
    if constexpr (GATE) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        Pa[cb] = Oa[cb];
        Pb[cb] = Ob[cb];
      }
    }
    __syncthreads();  // pair xl + 1 is in LDS; the slot of pair xl may be refilled
    slot = slot == kRing - 1 ? 0 : slot + 1;
  }
  if constexpr (GATE) {
    if (live > 0) epilogue(live - 1, Pa, Pb);  // its row sums are in LDS since the last barrier
  }

  if (s_next != nullptr) store_state(s_next + bh * rec::kDK * rec::kDV);
}

// One launch: the state workgroups (first) walk segment `cur` of every head
// while the remaining workgroups build the records of segment `nxt`.
struct Seg {
  int64_t x0 = 0, n = 0;  // first pair, pair count (n = 0: none)
  unsigned char* recs = nullptr;
};

int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return cus > 0 ? cus : 256;
}

template <int DVW, int CPW, bool GATE, bool WO, bool PACKED, bool LOGITS>
hipError_t launch_state_t(const ChunkArgs& a, Seg cur, const float* s_in, float* s_next,
                          const ChunkArgs& ab, Seg nxt, int cus) {
  constexpr int NW = DVW / CPW + kLoaders;
  const int64_t BH = a.B * a.H, BHb = ab.B * ab.H;
  const int64_t n_state = cur.n > 0 ? BH * (rec::kDV / DVW) : 0;
  int64_t n_tile = 0;
  if (nxt.n > 0) {
    const int64_t want = (BHb * nxt.n + NW - 1) / NW;  // one pair per wavefront at most
    int64_t avail = cus - n_state;
    if (avail < cus / 4) avail = cus / 4;              // always make progress
    n_tile = want < avail ? want : avail;
  }
  const int64_t nblk = n_state + n_tile;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  const Seqs<PACKED> seqs{a.cu, a.T, PACKED ? a.total : a.B * a.T};
  const Seqs<PACKED> seqb{ab.cu, ab.T, PACKED ? ab.total : ab.B * ab.T};
  tile::Args<PACKED, LOGITS> tb{(const bf16_t*)ab.q, (const bf16_t*)ab.k, ab.g, ab.beta,
                                (const bf16_t*)ab.ga, nxt.recs, seqb, ab.H, BHb, nxt.x0,
                                nxt.n > 0 ? nxt.n : 1};
  hipLaunchKernelGGL((kda_state_kernel<DVW, CPW, GATE, WO, PACKED, LOGITS>),
                     dim3((unsigned)nblk), dim3(64 * NW),
                     0, (hipStream_t)a.stream, cur.recs, (const bf16_t*)a.v, s_in, s_next,
                     (bf16_t*)a.o, (const bf16_t*)a.gate, a.norm_w, a.eps, seqs, a.H, BH, cur.x0,
                     cur.n > 0 ? cur.n : 1, n_state, a.ckpt, a.ckpt_every, a.ckpt_frag, a.scale, tb);
  return hipGetLastError();
}

// Columns per workgroup: a head's whole dv row when the gated norm is fused
// (it needs the row); otherwise half of it when the state workgroups of the
// split still leave half of the compute units to the tile workgroups.
int split_for(const ChunkArgs& a, int cus) {
  if (a.gate != nullptr && a.o != nullptr) return 1;
  if (const char* e = getenv("KDA_CHUNK_SPLIT")) {
    const int s = atoi(e);
    if (s == 1 || s == 2) return s;
  }
  return (2 * a.B * a.H <= cus / 2) ? 2 : 1;
}

// Pairs per segment.  One launch per segment, and the records of the segment
// being consumed are read back while the next segment's are written: two
// segments of about 96 MiB of records each stay within the 256 MB
// memory-side cache (v and gate rows and outputs bypass it), which makes the
// read-back cheap.  The length is the whole number of
// builder rounds (one pair per tile wavefront of the launch) nearest to that
// size: a launch lasts until its slowest tile wavefront is done, so a
// segment one pair over a round costs a whole round more.  At most 256 MiB
// per record buffer.  Long sequences take more launches of the same length
// (about 60 us each at 96 heads, far above the launch overhead).
int64_t seg_pairs(int64_t BH, int64_t npairs, int cus, int split) {
  int64_t seg = 0;
  if (const char* e = getenv("KDA_SEG_PAIRS")) seg = atoll(e);
  if (seg <= 0) {
    const int64_t per_row = BH * (int64_t)rec::kBytes;  // record bytes of one pair of every head
    const int64_t want = (int64_t(96) << 20) / per_row;
    const int64_t cap = (int64_t(256) << 20) / per_row;
    // pairs per builder round: tile wavefronts of a launch / heads
    const int64_t nw = rec::kDV / split / 32 + kLoaders;
    int64_t avail = cus - BH * split;
    if (avail < cus / 4) avail = cus / 4;
    int64_t round = nw * avail / BH;
    if (round < 1) round = 1;
    int64_t k = (want + round / 2) / round;  // nearest whole number of rounds
    if (k < 1) k = 1;
    seg = k * round < cap ? k * round : cap;
  }
  if (seg < 1) seg = 1;
  return seg < npairs ? seg : npairs;
}

int64_t pairs_of(int64_t T) { return (T + rec::kP - 1) / rec::kP; }

// The kernel instance for the call's workgroup layout.
template <bool PACKED, bool LOGITS>
hipError_t launch_layout(const ChunkArgs& a, int split, Seg cur, const float* s_in,
                         float* s_next, const ChunkArgs& ab, Seg nxt, int cus) {
#define KDA_LAUNCH(DVW, GATE, WO) \
  launch_state_t<DVW, 32, GATE, WO, PACKED, LOGITS>(a, cur, s_in, s_next, ab, nxt, cus)
  if (a.o == nullptr)
    return split == 2 ? KDA_LAUNCH(64, false, false) : KDA_LAUNCH(128, false, false);
  if (a.gate != nullptr) return KDA_LAUNCH(128, true, true);
  return split == 2 ? KDA_LAUNCH(64, false, true) : KDA_LAUNCH(128, false, true);
#undef KDA_LAUNCH
}

}  // namespace

bool chunk_mfma_supports(int dk, int dv, bool io_bf16) {
  return io_bf16 && dk == rec::kDK && dv == rec::kDV;
}

// Sequences per launch group.  The state workgroups of a group take about
// 3/8 of the compute units (96 of 256: the layout the segment length and the
// builder rounds are tuned for, with the other 5/8 building records); a larger
// batch runs group after group, each through the whole segment pipeline,
// rather than state and tile workgroups taking turns on the compute units.
int64_t group_seqs(int64_t B, int64_t H, int cus) {
  int64_t g = (3 * (int64_t)cus / 8) / H;
  if (const char* e = getenv("KDA_GROUP_SEQS")) g = atoll(e);  // tests and tuning
  if (g < 1) g = 1;
  return g < B ? g : B;
}

size_t chunk_mfma_workspace(int64_t B, int64_t T, int64_t H) {
  const int cus = device_cus();
  const int64_t BH = group_seqs(B, H, cus) * H, np = pairs_of(T);
  // either workgroup layout (it depends on the gate, unknown here)
  const int64_t s1 = seg_pairs(BH, np, cus, 1), s2 = seg_pairs(BH, np, cus, 2);
  const int64_t seg = s1 > s2 ? s1 : s2;
  // two record buffers (the segment being consumed and the one being built),
  // then a carried state for when s_out is absent
  return (size_t)(2 * BH * seg * rec::kBytes) + (size_t)(BH * rec::kDK * rec::kDV * 4);
}

size_t chunk_mfma_workspace_min(int64_t B, int64_t H) {
  const int64_t BH = group_seqs(B, H, device_cus()) * H;
  // one pair of every head of a launch group in each record buffer, and the carried state
  return (size_t)(2 * BH * rec::kBytes) + (size_t)(BH * rec::kDK * rec::kDV * 4);
}

namespace {

// One group of sequences as the state pass and the tile builder see it: the
// call's arguments offset to the group, its workgroup layout and segments.
struct Group {
  ChunkArgs a;
  int split = 1;
  int64_t seg = 1, nsegs = 0;
};

// Group gi of a call (sequences gi * gB .. of gB per group; the last may be
// smaller).  ws_half is the size of one record buffer (the workspace holds two
// and a carried state): a group's segments are capped so that its records fit.
Group group_at(const ChunkArgs& a, int cus, int64_t ws_half, int64_t gi) {
  const int64_t gB = group_seqs(a.B, a.H, cus), np = pairs_of(a.T);
  const int64_t sd = a.H * rec::kDK * rec::kDV;  // state elements per sequence
  const int64_t b0 = gi * gB;
  Group gr;
  ChunkArgs& g = gr.a;
  g = a;
  g.B = (a.B - b0) < gB ? (a.B - b0) : gB;
  if (a.cu != nullptr) {
    g.cu = a.cu + b0;  // packed rows stay absolute
  } else {
    const int64_t rows = b0 * a.T * a.H;  // token rows of the sequences before the group
    g.q = (const bf16_t*)a.q + rows * rec::kDK;
    g.k = (const bf16_t*)a.k + rows * rec::kDK;
    g.v = (const bf16_t*)a.v + rows * rec::kDV;
    if (a.g != nullptr) g.g = a.g + rows * rec::kDK;
    if (a.ga != nullptr) g.ga = (const bf16_t*)a.ga + rows * rec::kDK;
    g.beta = a.beta + rows;
    if (a.o != nullptr) g.o = (bf16_t*)a.o + rows * rec::kDV;
    if (a.gate != nullptr) g.gate = (const bf16_t*)a.gate + rows * rec::kDV;
  }
  if (a.s0 != nullptr) g.s0 = a.s0 + b0 * sd;
  if (a.s_out != nullptr) g.s_out = a.s_out + b0 * sd;
  if (a.ckpt != nullptr) g.ckpt = a.ckpt + b0 * (a.T / a.ckpt_every) * sd;
  const int64_t BH = g.B * g.H;
  gr.split = split_for(g, cus);
  gr.seg = seg_pairs(BH, np, cus, gr.split);
  const int64_t fit = ws_half / (BH * (int64_t)rec::kBytes);
  if (gr.seg > fit) gr.seg = fit;
  if (gr.seg < 1) gr.seg = 1;
  gr.nsegs = (np + gr.seg - 1) / gr.seg;
  return gr;
}

int64_t n_groups(const ChunkArgs& a, int cus) {
  const int64_t gB = group_seqs(a.B, a.H, cus);
  return (a.B + gB - 1) / gB;
}

int64_t record_half(int64_t B, int64_t T, int64_t H, int cus) {
  const int64_t BH = group_seqs(B, H, cus) * H;
  return ((int64_t)chunk_mfma_workspace(B, T, H) - BH * rec::kDK * rec::kDV * 4) / 2;
}

// One record buffer of a call's workspace: the default size, or less when the
// call brings a smaller workspace (ws_bytes; the segments are then shorter).
int64_t record_half_of(const ChunkArgs& a, int cus) {
  const int64_t half = record_half(a.B, a.T, a.H, cus);
  if (a.ws_bytes <= 0) return half;
  const int64_t BH = group_seqs(a.B, a.H, cus) * a.H;
  const int64_t fit = ((a.ws_bytes - BH * rec::kDK * rec::kDV * 4) / 2) & ~int64_t(255);
  return fit < half ? fit : half;
}

}  // namespace

int64_t chunk_mfma_launches(int64_t B, int64_t T, int64_t H) {
  const int cus = device_cus();
  ChunkArgs a{};
  a.B = B;
  a.T = T;
  a.H = H;
  const int64_t half = record_half(B, T, H, cus), ng = n_groups(a, cus);
  int64_t n = 1;  // the first segment's records
  // every group but the last has the same shape
  if (ng > 1) n += (ng - 1) * group_at(a, cus, half, 0).nsegs;
  n += group_at(a, cus, half, ng - 1).nsegs;
  return n;
}

hipError_t launch_chunk_mfma(const ChunkArgs& a) {
  if (!chunk_mfma_supports(a.dk, a.dv, a.io_bf16)) return hipErrorNotSupported;
  const int cus = device_cus();
  const int64_t half = record_half_of(a, cus);
  const int64_t np = pairs_of(a.T);
  // Every segment of every group, in order, as one pipeline: launch i runs
  // the state pass over item i and builds the records of item i + 1, also
  // when that item starts the next group.  Records alternate between the two
  // halves of the workspace; the carried state follows them.  Items are
  // walked with a cursor (group index, segment index), nothing is stored.
  const int64_t ng = n_groups(a, cus);
  struct Item {
    Group g;
    int64_t gi = -1, j = 0;  // gi < 0: no item
  };
  auto next_item = [&](const Item& it) {
    Item n;
    if (it.gi < 0) return n;
    if (it.j + 1 < it.g.nsegs) {
      n = it;
      ++n.j;
    } else if (it.gi + 1 < ng) {
      n.g = group_at(a, cus, half, it.gi + 1);
      n.gi = it.gi + 1;
    }
    return n;
  };
  unsigned char* buf[2] = {(unsigned char*)a.workspace, (unsigned char*)a.workspace + half};
  float* carry_ws = (float*)((unsigned char*)a.workspace + 2 * half);
  auto seg_of = [&](const Item& it, int64_t i) {
    Seg sg;
    if (it.gi >= 0) {
      sg.x0 = it.j * it.g.seg;
      sg.n = (np - sg.x0) < it.g.seg ? (np - sg.x0) : it.g.seg;
      sg.recs = buf[i & 1];
    }
    return sg;
  };
  Item cur, nxt;  // items i and i + 1
  nxt.g = group_at(a, cus, half, 0);
  nxt.gi = 0;
  for (int64_t i = -1; i < 0 || cur.gi >= 0; ++i) {
    const Seg scur = seg_of(cur, i), snxt = seg_of(nxt, i + 1);
    const Group& gs = cur.gi >= 0 ? cur.g : nxt.g;  // state pass
    const Group& gb = nxt.gi >= 0 ? nxt.g : cur.g;  // tile builder
    const ChunkArgs& as = gs.a;
    float* carry = as.s_out != nullptr ? as.s_out : carry_ws;
    const int64_t j = cur.gi >= 0 ? cur.j : 0;
    const float* s_in = j == 0 ? as.s0 : carry;
    float* s_next = j == gs.nsegs - 1 ? as.s_out : carry;
    // 32 state columns per state wavefront: one state and one loader
    // wavefront per SIMD, each with up to 256 registers (the tile builder
    // running in the same launch needs them).
    hipError_t e;
    if (a.cu != nullptr && a.ga != nullptr)
      e = launch_layout<true, true>(as, gs.split, scur, s_in, s_next, gb.a, snxt, cus);
    else if (a.cu != nullptr)
      e = launch_layout<true, false>(as, gs.split, scur, s_in, s_next, gb.a, snxt, cus);
    else if (a.ga != nullptr)
      e = launch_layout<false, true>(as, gs.split, scur, s_in, s_next, gb.a, snxt, cus);
    else
      e = launch_layout<false, false>(as, gs.split, scur, s_in, s_next, gb.a, snxt, cus);
    if (e != hipSuccess) return e;
    cur = nxt;
    nxt = next_item(nxt);
  }
  return hipSuccess;
}

}  // namespace kda
