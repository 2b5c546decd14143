// State kernel of the matrix-core chunked prefill: walks the tiles of one
// head in order with the float32 state resident in matrix-core accumulators,
// consuming the per-tile records of the tile kernel (kda_chunk_rec.h):
//   D = T V - W S,   O = Qh S + Aqk D,   S <- Diag(e^G_15) S + Kb^T D
// ("Kimi K3: Engineering a 2.8 Trillion Parameter Frontier", section
// "Dimension 1"), and, when a gate is given, the head-wise RMSNorm x
// sigmoid(gate) epilogue ("Kimi K3 Architecture Explained ...", section
// "Token mixing").
//
// One workgroup owns one (b, h) and DVW of its value columns (all 128, or 64
// when two workgroups share a head).  It has two kinds of wavefronts:
//   state waves (DVW / CPW): each keeps CPW state columns x 128 rows in 16x16
//     accumulators, rows in the permuted channel order of the record, so that
//     the state is the k-operand of its own products without moving between
//     lanes:
//       D   (lane (c, g): D[4 g + r][c]) = T V + sum_s (-W)_s S_s          (16x16x32)
//       O^T (lane (t, g): O[t][4 g + r]) = sum_s S_s^T Qh_s^T + D^T Aqk^T (transposed:
//            each lane holds 4 consecutive output columns of one token)
//       S_b <- e^G_15 * S_b + Kb^T_b D                                     (16x16x16)
//     V is moved from its token-major tile into the k-operand layout by a
//     bf16 product with a 0/1 selection matrix (exact).  The output of tile x
//     is normalised and written in iteration x + 1, once the row sums of
//     squares of all state waves are in LDS.
//   loader waves (kLoaders): copy each tile's record, v tile and gate tile
//     from memory straight into an LDS ring slot with direct-to-LDS loads,
//     kLead tiles ahead of the state waves, and wait for the next tile's
//     copies before every workgroup barrier.  The state waves issue no
//     global loads inside the loop.
// One workgroup barrier per tile.  Each accumulation chain uses a single
// matrix instruction shape.
//
// LDS ring slot: [record][v tile][gate tile][pad].  The v and gate tiles hold
// 16 rows of DVW bf16 columns with the 16-byte chunk u of row t stored at
// chunk position swz(t, u), so that the 8-byte reads of the state waves (one
// token per lane, 4 columns) fall in distinct banks.
//
// Precision: the state and every accumulation are float32; the state and D
// enter the products as float16 (11-bit significand), which requires the
// state, the values and D to stay below 65504 in magnitude.
#include <stdlib.h>

#include <type_traits>

#include "kda_chunk_rec.h"
#include "kda_chunk_tile.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kLoaders = 4;       // loader wavefronts, one per SIMD
constexpr int kLead = 4;          // tiles in flight ahead of the one being consumed
constexpr int kRing = kLead + 2;  // + the tile being consumed + the one being finished

// s_waitcnt with vmcnt = N and the other counters left alone (gfx9 encoding).
constexpr unsigned vmcnt_imm(int n) {
  return (unsigned)((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt with vmcnt = N and lgkmcnt = 0.
constexpr unsigned vmcnt_lgkm0_imm(int n) { return vmcnt_imm(n) & ~(0xFu << 8); }

// A slot is a whole number of 1 KB blocks (one direct-to-LDS load of a wave
// each); every block holds only record bytes or only v / gate bytes.
template <int DVW, bool GATE>
struct SlotCfg {
  static constexpr int kRowB = DVW * 2;                  // bytes per v / gate row
  static constexpr int kCpr = DVW / 8;                   // 16-byte chunks per row
  static constexpr int kTileB = rec::kC * kRowB;         // bytes per v / gate tile
  static constexpr int kRecBlocks = (rec::kBytes + 1023) / 1024;
  static constexpr int kTileBlocks = kTileB / 1024;
  static constexpr int kV = kRecBlocks * 1024;           // v tile offset in a slot
  static constexpr int kG = kV + kTileB;                 // gate tile offset
  static constexpr int kData = kG + (GATE ? kTileB : 0);
  static constexpr int kInstr = kLoaders * 1024;         // bytes per loader round
  static constexpr int kSlot = (kData + kInstr - 1) / kInstr * kInstr;
  static constexpr int kPer = kSlot / kInstr;            // loads per loader wave per tile
  static_assert(kTileB % 1024 == 0, "v tiles must be whole blocks");
  static constexpr int kRowsPerBankLine = 256 / kRowB;   // rows sharing the 64 banks
  // Chunk position of chunk u of row t (an involution in u for fixed t).
  static __device__ __forceinline__ int swz(int t, int u) {
    return u ^ ((t / kRowsPerBankLine) % kCpr);
  }
};

template <int DVW, int CPW, bool GATE, bool WO>
__global__ void __launch_bounds__(64 * (DVW / CPW + kLoaders), 1)
kda_state_kernel(const unsigned char* __restrict__ recs, const bf16_t* __restrict__ v,
                 const float* __restrict__ s_in, float* __restrict__ s_next,
                 bf16_t* __restrict__ o, const bf16_t* __restrict__ gate,
                 const float* __restrict__ norm_w, float eps, int64_t T, int64_t H, int64_t BH,
                 int64_t x0, int64_t nseg, int64_t n_state_wg, tile::Args next) {
  using SC = SlotCfg<DVW, GATE>;
  constexpr int NSW = DVW / CPW;   // state wavefronts
  constexpr int NCB = CPW / 16;    // 16-column blocks per state wavefront
  constexpr int NSPLIT = rec::kDV / DVW;
  static_assert(CPW % 16 == 0 && DVW % CPW == 0 && rec::kDV % DVW == 0, "bad column split");
  static_assert(!GATE || NSPLIT == 1, "the gated RMSNorm needs a head's full dv row");
  static_assert(!GATE || WO, "the gated epilogue only shapes the output");
  static_assert(kLead * SC::kPer <= 63, "outstanding loads per loader wave exceed vmcnt");

  constexpr int NW = NSW + kLoaders;  // wavefronts per workgroup
  constexpr int kRingB = kRing * SC::kSlot;
  constexpr int kRsB = 2 * rec::kC * NSW * 4;
  constexpr int kStateB = kRingB + kRsB;
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
    tile::build_range<(NW <= 8)>(next, first, stride, &scratch[wave], lane);
    return;
  }

  // ======================= state workgroups: the tiles of this segment
  unsigned char (*ring)[SC::kSlot] = (unsigned char (*)[SC::kSlot])lds;
  float (*rs)[rec::kC][NSW] = (float (*)[rec::kC][NSW])(lds + kRingB);  // row sums of O^2

  // Keep the NSPLIT workgroups of one head on one XCD (workgroups are dealt
  // round-robin over the 8 XCDs) so that they share its records in L2.
  int64_t wg = blockIdx.x;
  const int64_t total = n_state_wg;  // BH * NSPLIT
  if (NSPLIT > 1 && total % 8 == 0) wg = (wg % 8) * (total / 8) + wg / 8;
  const int64_t bh = wg / NSPLIT;
  const int col0 = (int)(wg % NSPLIT) * DVW;  // first value column of the workgroup
  const int64_t b = bh / H, h = bh % H;

  const int64_t rstride = H * rec::kDV;  // elements between consecutive tokens of a head

  if (wave >= NSW) {
    // ========================================================== loader waves
    const int lw = wave - NSW;
    const unsigned char* R0 = recs + bh * nseg * (int64_t)rec::kBytes;
    // Block i kLoaders + lw of a slot is this wave's i-th load.  Its kind and
    // this lane's source offset are fixed; a tile only moves the base.
    //   record block j:  R0 + x * kBytes + 16 (64 j + lane)   (the padding of the
    //                    last record block re-reads record chunks)
    //   v / gate block:  row t, column chunk u of the tile:
    //                    base_x + t * row stride + 2 (col0 + 8 u)
    int kind[SC::kPer];        // 0 record, 1 v, 2 gate (wave-uniform)
    unsigned loff[SC::kPer];   // byte offset from the tile base (full tiles)
    int lrow[SC::kPer], lcol[SC::kPer];
#pragma unroll
    for (int i = 0; i < SC::kPer; ++i) {
      const int blk = i * kLoaders + lw;
      const int c = blk * 64 + lane;
      if (blk < SC::kRecBlocks) {
        kind[i] = 0;
        loff[i] = 16u * (unsigned)(c < rec::kBytes / 16 ? c : c - 64);
        lrow[i] = lcol[i] = 0;
      } else {
        int q = (blk - SC::kRecBlocks) * 64 + lane;
        const int which = q / (SC::kTileB / 16);
        kind[i] = (GATE && which == 1) ? 2 : 1;  // past the gate tile: padding, re-reads v
        q %= SC::kTileB / 16;
        const int t = q / SC::kCpr, u = SC::swz(t, q % SC::kCpr);
        lrow[i] = t;
        lcol[i] = col0 + 8 * u;
        loff[i] = (unsigned)(2 * (t * rstride + lcol[i]));
      }
    }
    // Copy tile xt (clamped into the segment) into ring slot `slot`.
    auto issue = [&](int64_t xt, int slot) {
      xt = xt < nseg ? xt : nseg - 1;
      const int64_t row0 = (x0 + xt) * rec::kC;               // first token of the tile
      const bool full = row0 + rec::kC <= T;
      const unsigned char* base_r = R0 + xt * rec::kBytes;
      const int64_t tile0 = ((b * T + row0) * H + h) * rec::kDV;  // element offset of row 0
      const unsigned char* base_v = (const unsigned char*)(v + tile0);
      const unsigned char* base_g = (const unsigned char*)((GATE ? gate : v) + tile0);
#pragma unroll
      for (int i = 0; i < SC::kPer; ++i) {
        const unsigned char* bt = kind[i] == 0 ? base_r : (kind[i] == 2 ? base_g : base_v);
        unsigned off = loff[i];
        if (kind[i] != 0 && !full) {  // the sequence's last, partial tile: clamp rows into it
          const int64_t t = row0 + lrow[i] < T ? lrow[i] : T - 1 - row0;
          off = (unsigned)(2 * (t * rstride + lcol[i]));
        }
        const unsigned char* src = bt + off;
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)src,
            (__attribute__((address_space(3))) void*)(ring[slot] + (i * kLoaders + lw) * 1024), 16,
            0, 0);
      }
    };
    // Gate chunk of this lane (GATE: kLoaders x 64 lanes cover the tile): it is
    // replaced in place by w * sigmoid(gate) in float16 one iteration before
    // the state waves read it.
    static_assert(!GATE || kLoaders * 64 == SC::kTileB / 16, "one gate chunk per loader lane");
    const int gp = lw * 64 + lane;                       // chunk position in the tile
    const int gu = SC::swz(gp / SC::kCpr, gp % SC::kCpr);  // its column chunk
    float gw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      gw[e] = (GATE && norm_w != nullptr) ? norm_w[col0 + 8 * gu + e] : 1.f;
    // The chunk was completed before the last barrier; the direct-to-LDS loads
    // still in flight target other slots.  Plain loads and stores here would
    // make the compiler wait for all of those loads first, so the two LDS
    // accesses are issued directly.
    auto convert_gate = [&](int slot) {
      const unsigned addr = (unsigned)(uintptr_t)(
          (__attribute__((address_space(3))) unsigned char*)(ring[slot] + SC::kG + 16 * gp));
      i16x8 raw;
      asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(raw) : "v"(addr));
      const bf16x8 x = __builtin_bit_cast(bf16x8, raw);
      f16x8 y;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        y[e] = (f16)(gw[e] * __builtin_amdgcn_rcpf(
                                 1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * (float)x[e])));
      asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(__builtin_bit_cast(i16x8, y))
                   : "memory");
    };
#pragma unroll
    for (int y = 0; y < kLead; ++y) issue(y, y);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((kLead - 1) * SC::kPer));  // tile 0 is in LDS
    __builtin_amdgcn_s_barrier();
    int slot_issue = kLead, slot_cur = 0;
    for (int64_t xl = 0; xl <= nseg; ++xl) {
      issue(xl + kLead, slot_issue);
      slot_issue = slot_issue == kRing - 1 ? 0 : slot_issue + 1;
      if (GATE && xl < nseg) convert_gate(slot_cur);
      slot_cur = slot_cur == kRing - 1 ? 0 : slot_cur + 1;
      // tile xl + 1 is in LDS and the converted gate is written
      __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm((kLead - 1) * SC::kPer));
      __builtin_amdgcn_s_barrier();
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    return;
  }

  // ============================================================ state waves
  const int wl = wave * CPW;  // first column of this wave, in the workgroup

  // State: block kb of column block cb, lane (c, g), r = row chan(kb, 4 g + r).
  f32x4 S[NCB][8];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      f32x4 x = zero4();
      if (s_in != nullptr) {
        const float* p = s_in + bh * rec::kDK * rec::kDV + col0 + wl + 16 * cb + lc;
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = p[rec::chan(kb, 4 * lg + r) * rec::kDV];
      }
      S[cb][kb] = x;
    }
  // Selection matrix for the v transpose: B[k = 4 g + e][c] = (k == c).
  bf16x4 ident;
#pragma unroll
  for (int e = 0; e < 4; ++e) ident[e] = (bf16_t)((4 * lg + e == lc) ? 1.f : 0.f);
  // LDS byte offset, within a v / gate tile, of this lane's 4 columns of token lc.
  int tile_off[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int col = wl + 16 * cb + 4 * lg;
    tile_off[cb] = lc * SC::kRowB + 16 * SC::swz(lc, col / 8) + 2 * (col % 8);
  }

  f32x4 Oa[NCB], Ob[NCB];  // outputs of even / odd tiles (finished one tile later)
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) Oa[cb] = Ob[cb] = zero4();
  // Output of tile x: this lane writes token lc, columns col0 + wl + 16 cb + 4 lg.
  const int64_t o_lane = lc * rstride + col0 + wl + 4 * lg;
  auto o_tile = [&](int64_t x) { return o + ((b * T + (x0 + x) * rec::kC) * H + h) * rec::kDV; };
  __syncthreads();  // tile 0 is in LDS

  int slot = 0;  // ring slot of tile xl
  // One tile per call: the epilogue of tile xl - 1 and the state step of tile
  // xl.  The first and last calls are peeled, so that the steady state is one
  // basic block and the epilogue's arithmetic can fill the matrix-core chain.
  // Only the sequence's last tile can be partial (`tail`).
  auto step = [&](int64_t xl, auto EPI, auto CHAIN, bool tail, f32x4 (&Oprev)[NCB],
                  f32x4 (&O)[NCB]) {
    constexpr bool kEpi = decltype(EPI)::value && GATE;
    constexpr bool kChain = decltype(CHAIN)::value;
    const int slot_prev = slot == 0 ? kRing - 1 : slot - 1;
    const unsigned char* Rs = ring[slot];

    // The LDS operands are read in two batches (those of the D and O products
    // first, those of the state update once the products are issued), so
    // that the step waits for LDS twice rather than once per product.
    float rsum[NSW];
    f16x4 sw[NCB];
    if constexpr (kEpi) {
#pragma unroll
      for (int w = 0; w < NSW; ++w) rsum[w] = rs[(xl - 1) & 1][lc][w];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        sw[cb] = *(const f16x4*)(ring[slot_prev] + SC::kG + tile_off[cb]);
    }
    f16x4 t_op, aqk_op, ka[8];
    f16x8 w_op[4], q_op[4];
    bf16x4 vn[NCB];
    f32x4 e4[8];
    if constexpr (kChain) {
      t_op = *(const f16x4*)(Rs + rec::kT + lane * 8);
      aqk_op = *(const f16x4*)(Rs + rec::kAqk + lane * 8);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) vn[cb] = *(const bf16x4*)(Rs + SC::kV + tile_off[cb]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        w_op[s] = *(const f16x8*)(Rs + rec::kW + s * 1024 + lane * 16);
        q_op[s] = *(const f16x8*)(Rs + rec::kQh + s * 1024 + lane * 16);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- epilogue of tile xl - 1: y = O / rms(O) * w * sigmoid(gate)
    if constexpr (kEpi) {
      float ss = 0.f;
#pragma unroll
      for (int w = 0; w < NSW; ++w) ss += rsum[w];
      const float inv = rsqrtf(ss * (1.f / (float)rec::kDV) + eps);
      const int64_t tok = (x0 + xl - 1) * rec::kC + lc;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        bf16x4 y;
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = (bf16_t)(Oprev[cb][r] * inv * (float)sw[cb][r]);
        if (!tail || tok < T) *(bf16x4*)(o_tile(xl - 1) + o_lane + 16 * cb) = y;
      }
    }

    // ---- state step of tile xl
    if constexpr (kChain) {
      f16x4 d16[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f16x8 sop[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) sop[s] = cat8(to_h4(S[cb][2 * s]), to_h4(S[cb][2 * s + 1]));
        const f16x4 vop = to_h4(mma16b(vn[cb], ident, zero4()));  // lane (c, g): V[4 g + e][c]
        // T V and D^T Aqk^T are 16x16x32 products with k-values 4..7 of each
        // lane zero: every accumulation chain uses one instruction shape (a
        // 16x16x16 result fed straight into a 16x16x32 accumulator read stale
        // values on gfx950).
        f32x4 d = mma32h(cat8(t_op, f16x4{}), cat8(vop, f16x4{}), zero4());
        f32x4 oc = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          d = mma32h(w_op[s], sop[s], d);
          oc = mma32h(sop[s], q_op[s], oc);
        }
        d16[cb] = to_h4(d);
        O[cb] = mma32h(cat8(d16[cb], f16x4{}), cat8(aqk_op, f16x4{}), oc);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        ka[kb] = *(const f16x4*)(Rs + rec::kKb + kb * 512 + lane * 8);
        e4[kb] = *(const f32x4*)(Rs + rec::kEn + 4 * (32 * (kb / 2) + 8 * lg + 4 * (kb % 2)));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) S[cb][kb] = mma16h(ka[kb], d16[cb], S[cb][kb] * e4[kb]);
      if constexpr (GATE) {
        float p = 0.f;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) p = fmaf(O[cb][r], O[cb][r], p);
        p += __shfl_xor(p, 16);
        p += __shfl_xor(p, 32);
        if (lg == 0) rs[xl & 1][lc][wave] = p;
      } else if constexpr (WO) {
        const int64_t tok = (x0 + xl) * rec::kC + lc;
        if (!tail || tok < T) {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const bf16x4 y = {(bf16_t)O[cb][0], (bf16_t)O[cb][1], (bf16_t)O[cb][2],
                              (bf16_t)O[cb][3]};
            *(bf16x4*)(o_tile(xl) + o_lane + 16 * cb) = y;
          }
        }
      }
    }
    __syncthreads();  // tile xl + 1 is in LDS; the slot of tile xl - 1 may be refilled
    slot = slot == kRing - 1 ? 0 : slot + 1;
  };
  using yes = std::true_type;
  using no = std::false_type;
  // Tile xl keeps its output in Oa (xl even) or Ob (xl odd).
  step(0, no{}, yes{}, nseg == 1, Ob, Oa);
  int64_t xl = 1;
  for (; xl + 2 < nseg; xl += 2) {
    step(xl, yes{}, yes{}, false, Oa, Ob);
    step(xl + 1, yes{}, yes{}, false, Ob, Oa);
  }
  for (; xl < nseg; ++xl) {  // the last one or two tiles (the last may be partial)
    if (xl & 1)
      step(xl, yes{}, yes{}, xl == nseg - 1, Oa, Ob);
    else
      step(xl, yes{}, yes{}, xl == nseg - 1, Ob, Oa);
  }
  if (nseg & 1)
    step(nseg, yes{}, no{}, true, Oa, Ob);
  else
    step(nseg, yes{}, no{}, true, Ob, Oa);

  if (s_next != nullptr) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        float* p = s_next + bh * rec::kDK * rec::kDV + col0 + wl + 16 * cb + lc;
#pragma unroll
        for (int r = 0; r < 4; ++r) p[rec::chan(kb, 4 * lg + r) * rec::kDV] = S[cb][kb][r];
      }
  }
}

// One launch: the state workgroups (first) walk segment `cur` of every head
// while the remaining workgroups build the records of segment `nxt`.
struct Seg {
  int64_t x0 = 0, n = 0;  // first tile, tile count (n = 0: none)
  unsigned char* recs = nullptr;
};

int device_cus() {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return cus > 0 ? cus : 256;
}

template <int DVW, int CPW, bool GATE, bool WO>
hipError_t launch_state_t(const ChunkArgs& a, Seg cur, const float* s_in, float* s_next, Seg nxt,
                          int cus) {
  constexpr int NW = DVW / CPW + kLoaders;
  const int64_t BH = a.B * a.H;
  const int64_t n_state = cur.n > 0 ? BH * (rec::kDV / DVW) : 0;
  int64_t n_tile = 0;
  if (nxt.n > 0) {
    const int64_t want = (BH * nxt.n + NW - 1) / NW;  // one tile per wavefront at most
    int64_t avail = cus - n_state;
    if (avail < cus / 4) avail = cus / 4;              // always make progress
    n_tile = want < avail ? want : avail;
  }
  const int64_t nblk = n_state + n_tile;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  tile::Args tb{(const bf16_t*)a.q, (const bf16_t*)a.k, a.g, a.beta, nxt.recs,
                a.T, a.H, BH, nxt.x0, nxt.n > 0 ? nxt.n : 1, a.scale};
  hipLaunchKernelGGL((kda_state_kernel<DVW, CPW, GATE, WO>), dim3((unsigned)nblk), dim3(64 * NW),
                     0, (hipStream_t)a.stream, cur.recs, (const bf16_t*)a.v, s_in, s_next,
                     (bf16_t*)a.o, (const bf16_t*)a.gate, a.norm_w, a.eps, a.T, a.H, BH, cur.x0,
                     cur.n > 0 ? cur.n : 1, n_state, tb);
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

// Tiles per segment.  One launch per segment, and the records of the
// segment being consumed are read back while the next segment's are written:
// a segment of about 64 MiB of records stays within the 256 MB memory-side
// cache with the rest of a launch's traffic, which makes the read-back
// cheaper; longer sequences use longer segments (at most about 64 launches,
// at most 256 MiB per record buffer) so that the per-launch cost (state load
// and store, pipeline fill) stays small.
int64_t seg_tiles(int64_t BH, int64_t nchunks) {
  int64_t seg = 0;
  if (const char* e = getenv("KDA_SEG_TILES")) seg = atoll(e);
  if (seg <= 0) {
    const int64_t per_row = BH * (int64_t)rec::kBytes;  // record bytes of one tile of every head
    seg = (int64_t(64) << 20) / per_row;
    const int64_t min_seg = (nchunks + 63) / 64;
    if (seg < min_seg) seg = min_seg;
    const int64_t cap = (int64_t(256) << 20) / per_row;
    if (seg > cap) seg = cap;
  }
  if (seg < 1) seg = 1;
  return seg < nchunks ? seg : nchunks;
}

}  // namespace

bool chunk_mfma_supports(int dk, int dv, bool io_bf16) {
  return io_bf16 && dk == rec::kDK && dv == rec::kDV;
}

size_t chunk_mfma_workspace(int64_t B, int64_t T, int64_t H) {
  const int64_t BH = B * H, nch = (T + rec::kC - 1) / rec::kC;
  const int64_t seg = seg_tiles(BH, nch);
  // two record buffers (the segment being consumed and the one being built),
  // then a carried state for when s_out is absent
  return (size_t)(2 * BH * seg * rec::kBytes) + (size_t)(BH * rec::kDK * rec::kDV * 4);
}

int64_t chunk_mfma_launches(int64_t B, int64_t T, int64_t H) {
  const int64_t nch = (T + rec::kC - 1) / rec::kC;
  const int64_t seg = seg_tiles(B * H, nch);
  return (nch + seg - 1) / seg + 1;  // one per segment, plus the first segment's records
}

hipError_t launch_chunk_mfma(const ChunkArgs& a) {
  if (!chunk_mfma_supports(a.dk, a.dv, a.io_bf16)) return hipErrorNotSupported;
  const int64_t BH = a.B * a.H, nch = (a.T + rec::kC - 1) / rec::kC;
  const int64_t seg = seg_tiles(BH, nch);
  const int64_t nsegs = (nch + seg - 1) / seg;
  unsigned char* buf[2] = {(unsigned char*)a.workspace,
                           (unsigned char*)a.workspace + BH * seg * rec::kBytes};
  float* carry = a.s_out != nullptr ? a.s_out : (float*)(buf[1] + BH * seg * rec::kBytes);
  const int cus = device_cus();
  const int split = split_for(a, cus);
  // State columns per state wavefront: 16 (two state wavefronts per SIMD, so
  // that one's matrix-core and LDS latencies are covered by the other's work)
  // unless KDA_CPW=32 asks for one wavefront of 32 columns per SIMD.
  int cpw = 16;
  if (const char* e = getenv("KDA_CPW")) cpw = atoi(e) == 32 ? 32 : 16;
  auto segment = [&](int64_t j) {
    Seg sg;
    if (j >= 0 && j < nsegs) {
      sg.x0 = j * seg;
      sg.n = (nch - sg.x0) < seg ? (nch - sg.x0) : seg;
      sg.recs = buf[j & 1];
    }
    return sg;
  };
  // Launch j: state pass over segment j, records of segment j + 1.
  for (int64_t j = -1; j < nsegs; ++j) {
    const Seg cur = segment(j), nxt = segment(j + 1);
    const float* s_in = (j <= 0) ? a.s0 : carry;
    float* s_next = (j == nsegs - 1) ? a.s_out : carry;
    hipError_t e;
    if (a.o == nullptr)
      e = split == 2 ? launch_state_t<64, 32, false, false>(a, cur, s_in, s_next, nxt, cus)
          : cpw == 16 ? launch_state_t<128, 16, false, false>(a, cur, s_in, s_next, nxt, cus)
                      : launch_state_t<128, 32, false, false>(a, cur, s_in, s_next, nxt, cus);
    else if (a.gate != nullptr)
      e = cpw == 16 ? launch_state_t<128, 16, true, true>(a, cur, s_in, s_next, nxt, cus)
                    : launch_state_t<128, 32, true, true>(a, cur, s_in, s_next, nxt, cus);
    else if (split == 2)
      e = launch_state_t<64, 32, false, true>(a, cur, s_in, s_next, nxt, cus);
    else
      e = cpw == 16 ? launch_state_t<128, 16, false, true>(a, cur, s_in, s_next, nxt, cus)
                    : launch_state_t<128, 32, false, true>(a, cur, s_in, s_next, nxt, cus);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kda
