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

#include "kda_chunk_rec.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kLoaders = 2;       // loader wavefronts
constexpr int kLead = 4;          // tiles in flight ahead of the one being consumed
constexpr int kRing = kLead + 2;  // + the tile being consumed + the one being finished

// s_waitcnt with vmcnt = N and the other counters left alone (gfx9 encoding).
constexpr unsigned vmcnt_imm(int n) {
  return (unsigned)((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int DVW, bool GATE>
struct SlotCfg {
  static constexpr int kRowB = DVW * 2;                  // bytes per v / gate row
  static constexpr int kCpr = DVW / 8;                   // 16-byte chunks per row
  static constexpr int kTileB = rec::kC * kRowB;         // bytes per v / gate tile
  static constexpr int kV = rec::kBytes;                 // v tile offset in a slot
  static constexpr int kG = kV + kTileB;                 // gate tile offset
  static constexpr int kData = kG + (GATE ? kTileB : 0);
  static constexpr int kInstr = kLoaders * 1024;         // bytes per loader round
  static constexpr int kSlot = (kData + kInstr - 1) / kInstr * kInstr;
  static constexpr int kPer = kSlot / kInstr;            // loads per loader wave per tile
  static constexpr int kRowsPerBankLine = 256 / kRowB;   // rows sharing the 64 banks
  // Chunk position of chunk u of row t (an involution in u for fixed t).
  static __device__ __forceinline__ int swz(int t, int u) {
    return u ^ ((t / kRowsPerBankLine) % kCpr);
  }
};

template <int DVW, int CPW, bool GATE>
__global__ void __launch_bounds__(64 * (DVW / CPW + kLoaders), 1)
kda_state_kernel(const unsigned char* __restrict__ recs, const bf16_t* __restrict__ v,
                 const float* __restrict__ s_in, float* __restrict__ s_next,
                 bf16_t* __restrict__ o, const bf16_t* __restrict__ gate,
                 const float* __restrict__ norm_w, float eps, int64_t T, int64_t H, int64_t BH,
                 int64_t x0, int64_t nseg) {
  using SC = SlotCfg<DVW, GATE>;
  constexpr int NSW = DVW / CPW;   // state wavefronts
  constexpr int NCB = CPW / 16;    // 16-column blocks per state wavefront
  constexpr int NSPLIT = rec::kDV / DVW;
  static_assert(CPW % 16 == 0 && DVW % CPW == 0 && rec::kDV % DVW == 0, "bad column split");
  static_assert(!GATE || NSPLIT == 1, "the gated RMSNorm needs a head's full dv row");
  static_assert(kLead * SC::kPer <= 63, "outstanding loads per loader wave exceed vmcnt");

  __shared__ __attribute__((aligned(1024))) unsigned char ring[kRing][SC::kSlot];
  __shared__ __attribute__((aligned(16))) float rs[2][rec::kC][NSW];  // row sums of O^2

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int lc = lane % 16, lg = lane / 16;

  // Keep the NSPLIT workgroups of one head on one XCD (workgroups are dealt
  // round-robin over the 8 XCDs) so that they share its records in L2.
  int64_t wg = blockIdx.x;
  const int64_t total = BH * NSPLIT;
  if (NSPLIT > 1 && total % 8 == 0) wg = (wg % 8) * (total / 8) + wg / 8;
  const int64_t bh = wg / NSPLIT;
  const int col0 = (int)(wg % NSPLIT) * DVW;  // first value column of the workgroup
  const int64_t b = bh / H, h = bh % H;

  auto rowoff = [&](int64_t xl, int r) {  // element offset of a [B, T, H, dv] row, clamped
    int64_t tok = (x0 + xl) * rec::kC + r;
    tok = tok < T ? tok : T - 1;
    return ((b * T + tok) * H + h) * rec::kDV;
  };

  if (wave >= NSW) {
    // ========================================================== loader waves
    const int lw = wave - NSW;
    const unsigned char* R0 = recs + bh * nseg * (int64_t)rec::kBytes;
    // Copy tile xt (clamped into the segment) into ring slot `slot`: round i
    // of this wave moves the 64 chunks [(i kLoaders + lw) 64, + 64) of the slot.
    auto issue = [&](int64_t xt, int slot) {
      xt = xt < nseg ? xt : nseg - 1;
#pragma unroll
      for (int i = 0; i < SC::kPer; ++i) {
        const int base = (i * kLoaders + lw) * 64;  // first chunk of the round
        const int c = base + lane;                  // chunk of this lane (a round may
        const bool is_rec = c < SC::kV / 16;        // straddle the record's end)
        // v or gate chunk; chunks of the padding re-read a v chunk
        int q = is_rec ? 0 : c - SC::kV / 16;
        const bool is_gate = GATE && q >= SC::kTileB / 16 && q < 2 * SC::kTileB / 16;
        q = q % (SC::kTileB / 16);
        const int t = q / SC::kCpr, u = SC::swz(t, q % SC::kCpr);
        const unsigned char* src_rec = R0 + xt * rec::kBytes + (is_rec ? c * 16 : 0);
        const unsigned char* src_tile =
            (const unsigned char*)((is_gate ? gate : v) + rowoff(xt, t) + col0 + 8 * u);
        const unsigned char* src = is_rec ? src_rec : src_tile;
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)src,
            (__attribute__((address_space(3))) void*)(ring[slot] + base * 16), 16, 0, 0);
      }
    };
#pragma unroll
    for (int y = 0; y < kLead; ++y) issue(y, y);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((kLead - 1) * SC::kPer));  // tile 0 is in LDS
    __builtin_amdgcn_s_barrier();
    int slot_issue = kLead;
    for (int64_t xl = 0; xl <= nseg; ++xl) {
      issue(xl + kLead, slot_issue);
      slot_issue = slot_issue == kRing - 1 ? 0 : slot_issue + 1;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((kLead - 1) * SC::kPer));  // tile xl + 1 is in LDS
      __builtin_amdgcn_s_barrier();
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    return;
  }

  // ============================================================ state waves
  const int wl = wave * CPW;  // first column of this wave, in the workgroup
  const bool write_o = o != nullptr;

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
  f32x4 wn[NCB];  // norm weight of this lane's 4 output columns (4-byte aligned pointer)
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      wn[cb][r] = (GATE && norm_w != nullptr) ? norm_w[col0 + wl + 16 * cb + 4 * lg + r] : 1.f;
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

  f32x4 Oprev[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) Oprev[cb] = zero4();
  __syncthreads();  // tile 0 is in LDS

  int slot = 0;  // ring slot of tile xl
  for (int64_t xl = 0; xl <= nseg; ++xl) {
    const int slot_prev = slot == 0 ? kRing - 1 : slot - 1;

    // ---- epilogue of tile xl - 1: y = O / rms(O) * w * sigmoid(gate)
    if (GATE && write_o && xl >= 1) {
      float ss = 0.f;
#pragma unroll
      for (int w = 0; w < NSW; ++w) ss += rs[(xl - 1) & 1][lc][w];
      const float inv = rsqrtf(ss * (1.f / (float)rec::kDV) + eps);
      const int64_t tok = (x0 + xl - 1) * rec::kC + lc;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const bf16x4 g4 = *(const bf16x4*)(ring[slot_prev] + SC::kG + tile_off[cb]);
        bf16x4 y;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sg = __builtin_amdgcn_rcpf(
              1.f + __builtin_amdgcn_exp2f(-1.4426950408889634f * (float)g4[r]));
          y[r] = (bf16_t)(Oprev[cb][r] * inv * wn[cb][r] * sg);
        }
        if (tok < T) *(bf16x4*)(o + rowoff(xl - 1, lc) + col0 + wl + 16 * cb + 4 * lg) = y;
      }
    }

    // ---- state step of tile xl
    if (xl < nseg) {
      const unsigned char* Rs = ring[slot];
      const f16x4 t_op = *(const f16x4*)(Rs + rec::kT + lane * 8);
      const f16x4 aqk_op = *(const f16x4*)(Rs + rec::kAqk + lane * 8);
      f16x8 w_op[4], q_op[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        w_op[s] = *(const f16x8*)(Rs + rec::kW + s * 1024 + lane * 16);
        q_op[s] = *(const f16x8*)(Rs + rec::kQh + s * 1024 + lane * 16);
      }
      f16x4 d16[NCB];
      f32x4 O[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        f16x8 sop[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) sop[s] = cat8(to_h4(S[cb][2 * s]), to_h4(S[cb][2 * s + 1]));
        const bf16x4 vn = *(const bf16x4*)(Rs + SC::kV + tile_off[cb]);
        const f16x4 vop = to_h4(mma16b(vn, ident, zero4()));  // lane (c, g): V[4 g + e][c]
        // T V as a 16x16x32 product with k-values 4..7 of each lane zero: every
        // accumulation chain uses one instruction shape (a 16x16x16 result fed
        // straight into a 16x16x32 accumulator read stale values on gfx950).
        f32x4 d0 = mma32h(cat8(t_op, f16x4{}), cat8(vop, f16x4{}), zero4()), d1 = zero4();
        f32x4 o0 = zero4(), o1 = zero4();
#pragma unroll
        for (int s = 0; s < 4; s += 2) {
          d0 = mma32h(w_op[s], sop[s], d0);
          d1 = mma32h(w_op[s + 1], sop[s + 1], d1);
          o0 = mma32h(sop[s], q_op[s], o0);
          o1 = mma32h(sop[s + 1], q_op[s + 1], o1);
        }
        d16[cb] = to_h4(d0 + d1);
        O[cb] = mma16h(d16[cb], aqk_op, o0 + o1);
      }
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const f16x4 ka = *(const f16x4*)(Rs + rec::kKb + kb * 512 + lane * 8);
        const f32x4 e4 =
            *(const f32x4*)(Rs + rec::kEn + 4 * (32 * (kb / 2) + 8 * lg + 4 * (kb % 2)));
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) S[cb][kb] = mma16h(ka, d16[cb], S[cb][kb] * e4);
      }
      if (GATE) {
        float p = 0.f;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int r = 0; r < 4; ++r) p = fmaf(O[cb][r], O[cb][r], p);
        p += __shfl_xor(p, 16);
        p += __shfl_xor(p, 32);
        if (lg == 0) rs[xl & 1][lc][wave] = p;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) Oprev[cb] = O[cb];
      } else if (write_o) {
        const int64_t tok = (x0 + xl) * rec::kC + lc;
        if (tok < T) {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const bf16x4 y = {(bf16_t)O[cb][0], (bf16_t)O[cb][1], (bf16_t)O[cb][2],
                              (bf16_t)O[cb][3]};
            *(bf16x4*)(o + rowoff(xl, lc) + col0 + wl + 16 * cb + 4 * lg) = y;
          }
        }
      }
    }
    __syncthreads();  // tile xl + 1 is in LDS; the slot of tile xl - 1 may be refilled
    slot = slot == kRing - 1 ? 0 : slot + 1;
  }

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

template <int DVW, int CPW, bool GATE>
hipError_t launch_state_t(const ChunkArgs& a, const unsigned char* recs, const float* s_in,
                          float* s_next, int64_t x0, int64_t nseg) {
  const int64_t nblk = a.B * a.H * (rec::kDV / DVW);
  if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((kda_state_kernel<DVW, CPW, GATE>), dim3((unsigned)nblk),
                     dim3(64 * (DVW / CPW + kLoaders)), 0, (hipStream_t)a.stream, recs,
                     (const bf16_t*)a.v, s_in, s_next, (bf16_t*)a.o, (const bf16_t*)a.gate,
                     a.norm_w, a.eps, a.T, a.H, a.B * a.H, x0, nseg);
  return hipGetLastError();
}

// Columns per workgroup: a head's whole dv row when the gated norm is fused
// (it needs the row), otherwise half of it when that is what fills the GPU.
int split_for(const ChunkArgs& a) {
  if (a.gate != nullptr) return 1;
  if (const char* e = getenv("KDA_CHUNK_SPLIT")) {
    const int s = atoi(e);
    if (s == 1 || s == 2) return s;
  }
  return (a.B * a.H < 256) ? 2 : 1;
}

// Tiles per segment: the records of one segment of all heads are written by
// the tile kernel and read back by the state kernel right after, so a segment
// is sized to stay resident in the 256 MB memory-side cache.
int64_t seg_tiles(int64_t BH, int64_t nchunks) {
  int64_t seg = 0;
  if (const char* e = getenv("KDA_SEG_TILES")) seg = atoll(e);
  if (seg <= 0) {
    constexpr int64_t kTarget = int64_t(128) << 20;
    seg = kTarget / (BH * (int64_t)rec::kBytes);
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
  // records of one segment, then a carried state for when s_out is absent
  return (size_t)(BH * seg * rec::kBytes) + (size_t)(BH * rec::kDK * rec::kDV * 4);
}

hipError_t launch_chunk_mfma(const ChunkArgs& a) {
  if (!chunk_mfma_supports(a.dk, a.dv, a.io_bf16)) return hipErrorNotSupported;
  const int64_t BH = a.B * a.H, nch = (a.T + rec::kC - 1) / rec::kC;
  const int64_t seg = seg_tiles(BH, nch);
  unsigned char* recs = (unsigned char*)a.workspace;
  float* carry = a.s_out != nullptr ? a.s_out : (float*)(recs + BH * seg * rec::kBytes);
  const int split = split_for(a);
  for (int64_t x0 = 0; x0 < nch; x0 += seg) {
    const int64_t n = (nch - x0) < seg ? (nch - x0) : seg;
    hipError_t e = launch_chunk_tiles(a, recs, x0, n);
    if (e != hipSuccess) return e;
    const float* s_in = (x0 == 0) ? a.s0 : carry;
    float* s_next = (x0 + n >= nch) ? a.s_out : carry;
    if (a.gate != nullptr)
      e = launch_state_t<128, 32, true>(a, recs, s_in, s_next, x0, n);
    else if (split == 2)
      e = launch_state_t<64, 32, false>(a, recs, s_in, s_next, x0, n);
    else
      e = launch_state_t<128, 32, false>(a, recs, s_in, s_next, x0, n);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kda
