// C ABI of the KDA layer core: host-side argument validation and dispatch.
//
// Every check runs before any HIP call, so a rejected call launches nothing
// and touches no output.  The entry points and their contracts are declared
// and documented in include/kda.h.
#include "kda.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "kda_check.h"
#include "kda_launch.h"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 60;

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool aligned(const void* p, uintptr_t bytes) {
  return p == nullptr || (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0;
}

struct Span {
  const void* p;
  int64_t bytes;
};

bool overlap(Span a, Span b) {
  if (a.p == nullptr || b.p == nullptr || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

// a * b * c * d without overflow past kMaxElems; returns -1 on overflow.
int64_t prod(int64_t a, int64_t b, int64_t c = 1, int64_t d = 1) {
  int64_t r = 1;
  for (int64_t x : {a, b, c, d}) {
    if (x <= 0) return -1;
    if (r > kMaxElems / x) return -1;
    r *= x;
  }
  return r;
}

// Input-check mode: the check kernels over a call's inputs (kda_check.hip).
kda_status run_checks(const kda::CheckItem* items, int n, void* stream) {
  bool bad = false;
  if (kda::check_inputs(items, n, stream, &bad) != hipSuccess) return KDA_ERR_LAUNCH;
  return bad ? KDA_ERR_INPUT_RANGE : KDA_OK;
}

// The raw q and k norms the matrix-core path of the normalising entry points supports.
constexpr float kRawNormLo = 0.0625f, kRawNormHi = 128.f;

bool force_token_bwd() {
  const char* e = getenv("KDA_BWD_TOKEN");
  return e != nullptr && e[0] == '1';
}

bool force_valu() {
  const char* e = getenv("KDA_FORCE_VALU");
  return e != nullptr && e[0] == '1';
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL_POINTER: return "KDA_ERR_NULL_POINTER: a required pointer is NULL";
    case KDA_ERR_BAD_SHAPE: return "KDA_ERR_BAD_SHAPE: a size is < 1 or the tensor is too large";
    case KDA_ERR_UNSUPPORTED_DIM: return "KDA_ERR_UNSUPPORTED_DIM: dk and dv must be 16, 32, 64 or 128";
    case KDA_ERR_BAD_DTYPE: return "KDA_ERR_BAD_DTYPE: io dtype must be KDA_F32 or KDA_BF16";
    case KDA_ERR_MISALIGNED: return "KDA_ERR_MISALIGNED: a pointer lacks the alignment its argument requires";
    case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS: an output overlaps an input";
    case KDA_ERR_BAD_ARGUMENT: return "KDA_ERR_BAD_ARGUMENT: eps or scale is not finite, or eps < 0";
    case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
    case KDA_ERR_WORKSPACE:
      return "KDA_ERR_WORKSPACE: the workspace is NULL, smaller than "
             "kda_chunk_fwd_workspace_size() or not 256-byte aligned (kda_chunk_fwd_noalloc: "
             "the fixed scratch cannot hold one pair of records per head)";
    case KDA_ERR_INPUT_RANGE:
      return "KDA_ERR_INPUT_RANGE: an input is not finite, a log-decay g lies outside [-5, 0], "
             "or a raw q or k norm lies outside its supported range (KDA_CHECK_INPUTS=1)";
  }
  return "KDA_ERR_UNKNOWN";
}

int kda_version(void) { return 200; }

const char* kda_chunk_fwd_kernel(int dk, int dv, kda_dtype io) {
  if ((io != KDA_F32 && io != KDA_BF16) || !dim_ok(dk) || !dim_ok(dv)) return nullptr;
  if (!force_valu() && kda::chunk_mfma_supports(dk, dv, io == KDA_BF16)) return "kda_chunk_mfma";
  return "kda_chunk_valu";
}

size_t kda_chunk_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int dk, int dv,
                                    kda_dtype io) {
  if ((io != KDA_F32 && io != KDA_BF16) || !dim_ok(dk) || !dim_ok(dv)) return 0;
  if (prod(B, T, H, dk) < 0 || prod(B, H, dk, dv) < 0) return 0;
  if (force_valu() || !kda::chunk_mfma_supports(dk, dv, io == KDA_BF16)) return 0;
  return kda::chunk_mfma_workspace(B, T, H);
}

size_t kda_recurrent_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int dk, int dv) {
  if (dk != 128 || dv != 128 || prod(B, T, H, dk) < 0) return 0;
  // At most 2^40 token-heads (far beyond any device), so that every size term
  // below (under 2^17 bytes per token-head) stays within int64.
  if (prod(B, T, H, 1) > (int64_t(1) << 40)) return 0;
  const int64_t n = kda::bwd_workspace_floats(B, T, H);
  if (n <= 0 || n >= kMaxElems) return 0;
  // the larger of the two paths' needs (the path depends on the io dtype and alignment)
  const int64_t c = kda::bwd_chunk_workspace_bytes(B, T, H);
  return (size_t)(4 * n > c ? 4 * n : c);
}

}  // extern "C"

namespace {

// kda_recurrent_bwd and kda_recurrent_bwd_ckpt: ckpt is NULL for the former.
kda_status recurrent_bwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* s0, const void* dout,
                         const float* ds_final, void* dq, void* dk_out, void* dv_out, float* dg,
                         float* dbeta, float* ds0, int64_t B, int64_t T, int64_t H, int dk, int dv,
                         float scale, kda_dtype io, void* workspace, size_t workspace_bytes,
                         const float* ckpt, bool with_ckpt, void* stream) {
  if (!q || !k || !v || !g || !beta || !dout || !dq || !dk_out || !dv_out || !dg || !dbeta)
    return KDA_ERR_NULL_POINTER;
  if (with_ckpt && ckpt == nullptr) return KDA_ERR_NULL_POINTER;
  if (io != KDA_F32 && io != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (with_ckpt && io != KDA_BF16) return KDA_ERR_BAD_DTYPE;  // the chunkwise pass only
  if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED_DIM;
  if (dk != 128 || dv != 128) return KDA_ERR_UNSUPPORTED_DIM;
  const int64_t nqk = prod(B, T, H, dk), nb = prod(B, T, H), ns = prod(B, H, dk, dv);
  if (nqk < 0 || nb < 0 || ns < 0 || B * H > 0x7fffffffLL) return KDA_ERR_BAD_SHAPE;
  if (!isfinite(scale)) return KDA_ERR_BAD_ARGUMENT;
  const size_t need = kda_recurrent_bwd_workspace_size(B, T, H, dk, dv);
  if (need == 0) return KDA_ERR_BAD_SHAPE;
  if (workspace == nullptr || workspace_bytes < need) return KDA_ERR_WORKSPACE;
  const uintptr_t ea = (io == KDA_BF16) ? 2 : 4;
  for (const void* p : {q, k, v, dout, (const void*)dq, (const void*)dk_out, (const void*)dv_out})
    if (!aligned(p, ea)) return KDA_ERR_MISALIGNED;
  for (const void* p : {(const void*)g, (const void*)beta, (const void*)dg, (const void*)dbeta})
    if (!aligned(p, 4)) return KDA_ERR_MISALIGNED;
  for (const void* p : {(const void*)s0, (const void*)ds_final, (const void*)ds0,
                        (const void*)workspace, (const void*)ckpt})
    if (!aligned(p, 16)) return KDA_ERR_MISALIGNED;
  // bfloat16 with 16-byte aligned token tensors: the chunkwise matrix-core pass;
  // otherwise (and with KDA_BWD_TOKEN=1) the token-serial vector kernel
  bool tok_aligned = true;
  for (const void* p : {q, k, v, dout, (const void*)g, (const void*)dq, (const void*)dk_out,
                        (const void*)dv_out, (const void*)dg})
    tok_aligned = tok_aligned && aligned(p, 16);
  if (with_ckpt && !tok_aligned) return KDA_ERR_MISALIGNED;
  const bool chunk = with_ckpt || (io == KDA_BF16 && !force_token_bwd() && tok_aligned);

  const int64_t es = (io == KDA_BF16) ? 2 : 4;
  const int64_t nck = with_ckpt ? B * (T / 64) * H * dk * dv : 0;
  const Span in[] = {{q, nqk * es}, {k, nqk * es}, {v, nqk * es}, {g, nqk * 4}, {beta, nb * 4},
                     {s0, ns * 4}, {dout, nqk * es}, {ds_final, ns * 4},
                     {nck > 0 ? ckpt : nullptr, nck * 4}};
  const Span out[] = {{dq, nqk * es}, {dk_out, nqk * es}, {dv_out, nqk * es}, {dg, nqk * 4},
                      {dbeta, nb * 4}, {ds0, ns * 4}, {workspace, (int64_t)need}};
  for (int i = 0; i < 7; ++i) {
    for (const Span& x : in)
      if (overlap(out[i], x)) return KDA_ERR_ALIAS;
    for (int j = i + 1; j < 7; ++j)
      if (overlap(out[i], out[j])) return KDA_ERR_ALIAS;
  }

  kda::BwdArgs a{q, k, v, g, beta, s0, dout, ds_final, dq, dk_out, dv_out, dg, dbeta, ds0,
                 B, T, H, scale, io == KDA_BF16, (float*)workspace, stream};
  a.ckpt = with_ckpt ? ckpt : nullptr;
  const hipError_t err = chunk ? kda::launch_bwd_chunk(a) : kda::launch_recurrent_bwd(a);
  return err == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

kda_status kda_recurrent_bwd(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const float* s0, const void* dout,
                             const float* ds_final, void* dq, void* dk_out, void* dv_out,
                             float* dg, float* dbeta, float* ds0, int64_t B, int64_t T,
                             int64_t H, int dk, int dv, float scale, kda_dtype io,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return recurrent_bwd(q, k, v, g, beta, s0, dout, ds_final, dq, dk_out, dv_out, dg, dbeta, ds0,
                       B, T, H, dk, dv, scale, io, workspace, workspace_bytes, nullptr, false,
                       stream);
}

kda_status kda_recurrent_bwd_ckpt(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, const float* s0, const void* dout,
                                  const float* ds_final, const float* ckpt, void* dq,
                                  void* dk_out, void* dv_out, float* dg, float* dbeta,
                                  float* ds0, int64_t B, int64_t T, int64_t H, int dk, int dv,
                                  float scale, kda_dtype io, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return recurrent_bwd(q, k, v, g, beta, s0, dout, ds_final, dq, dk_out, dv_out, dg, dbeta, ds0,
                       B, T, H, dk, dv, scale, io, workspace, workspace_bytes, ckpt, true, stream);
}

int64_t kda_chunk_fwd_launches(int64_t B, int64_t T, int64_t H, int dk, int dv, kda_dtype io) {
  if ((io != KDA_F32 && io != KDA_BF16) || !dim_ok(dk) || !dim_ok(dv)) return 0;
  if (prod(B, T, H, dk) < 0 || prod(B, H, dk, dv) < 0) return 0;
  if (force_valu() || !kda::chunk_mfma_supports(dk, dv, io == KDA_BF16)) return 1;
  return kda::chunk_mfma_launches(B, T, H);
}

}  // extern "C"

namespace {

// kda_chunk_fwd with optional state checkpoints (ckpt NULL: none) and packed
// sequences (cu non-NULL: B sequences in `total` token rows, T the longest).
kda_status chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                     const float* beta, const float* s0, void* o, float* s_out, const void* gate,
                     const float* norm_w, float eps, int64_t B, int64_t T, int64_t H, int dk,
                     int dv, float scale, kda_dtype io, void* workspace, size_t workspace_bytes,
                     float* ckpt, int64_t ckpt_every, const int32_t* cu, int64_t total,
                     const void* ga, void* stream, bool small_ws = false) {
  // ga: the log-decay logits a (g = -5 sigmoid(a)) in place of g; beta then holds logits,
  // and q, k are L2-normalised in the kernels.  small_ws: the workspace may be smaller
  // than kda_chunk_fwd_workspace_size() (at least chunk_mfma_workspace_min()); the
  // matrix-core path then runs shorter segments.
  if (!q || !k || !v || (!g && !ga) || !beta) return KDA_ERR_NULL_POINTER;
  if (!o && !s_out) return KDA_ERR_NULL_POINTER;
  if (io != KDA_F32 && io != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED_DIM;
  const int64_t rows = cu != nullptr ? total : prod(B, T);  // token rows of q, k, v, g, beta, o
  if (rows < 1 || prod(B, T) < 0) return KDA_ERR_BAD_SHAPE;
  const int64_t nqk = prod(rows, H, dk), nv = prod(rows, H, dv), nb = prod(rows, H);
  const int64_t ns = prod(B, H, dk, dv);
  if (nqk < 0 || nv < 0 || nb < 0 || ns < 0) return KDA_ERR_BAD_SHAPE;
  if (B * H > 0x7fffffffLL) return KDA_ERR_BAD_SHAPE;  // one workgroup per (b, h)
  if (!isfinite(scale) || !isfinite(eps) || eps < 0.f) return KDA_ERR_BAD_ARGUMENT;
  // Tiles are moved with 16-byte accesses; beta, states and the norm weight
  // are read element by element.
  for (const void* p : {(const void*)q, (const void*)k, (const void*)v, (const void*)g,
                        (const void*)o, (const void*)gate, ga})
    if (!aligned(p, 16)) return KDA_ERR_MISALIGNED;
  for (const void* p : {(const void*)beta, (const void*)s0, (const void*)s_out,
                        (const void*)norm_w})
    if (!aligned(p, 4)) return KDA_ERR_MISALIGNED;

  const int64_t es = (io == KDA_BF16) ? 2 : 4;
  // the decay input: float32 g, or its logits in the io dtype
  const Span sg = ga != nullptr ? Span{ga, nqk * es} : Span{g, nqk * 4};
  const Span sq{q, nqk * es}, sk{k, nqk * es}, sv{v, nv * es}, sb{beta, nb * 4};
  const Span ss0{s0, ns * 4}, so{o, nv * es}, sso{s_out, ns * 4}, sgt{gate, nv * es};
  const Span sw{norm_w, (int64_t)dv * 4}, scu{cu, (B + 1) * 4};
  for (Span in : {sq, sk, sv, sg, sb, ss0, sgt, sw, sso, scu})
    if (overlap(so, in)) return KDA_ERR_ALIAS;
  for (Span in : {sq, sk, sv, sg, sb, sgt, sw, scu})
    if (overlap(sso, in)) return KDA_ERR_ALIAS;
  if (overlap(sso, ss0) && (const void*)s_out != (const void*)s0) return KDA_ERR_ALIAS;
  if (ckpt != nullptr) {
    const int64_t nck = T / ckpt_every;
    const Span sck{ckpt, nck > 0 ? prod(B, nck, H, dk) * dv * 4 : 0};
    if (nck > 0 && prod(B, nck, H, dk) < 0) return KDA_ERR_BAD_SHAPE;
    for (Span in : {sq, sk, sv, sg, sb, ss0, so, sso, sgt, sw, scu})
      if (overlap(sck, in)) return KDA_ERR_ALIAS;
  }

  const bool mfma = !force_valu() && kda::chunk_mfma_supports(dk, dv, io == KDA_BF16);
  if (mfma) {
    size_t need = kda::chunk_mfma_workspace(B, T, H);
    if (small_ws) {
      if (workspace_bytes < kda::chunk_mfma_workspace_min(B, H)) return KDA_ERR_WORKSPACE;
      need = workspace_bytes < need ? workspace_bytes : need;
    }
    if (workspace == nullptr || workspace_bytes < need || !aligned(workspace, 256))
      return KDA_ERR_WORKSPACE;
    const Span sws{workspace, (int64_t)need};
    for (Span in : {sq, sk, sv, sg, sb, ss0, so, sso, sgt, sw, scu})
      if (overlap(sws, in)) return KDA_ERR_ALIAS;
    if (ckpt != nullptr && overlap(sws, Span{ckpt, prod(B, T / ckpt_every, H, dk) * dv * 4}))
      return KDA_ERR_ALIAS;
  }

  if (kda::check_mode_on()) {
    using namespace kda;
    const int fk = io == KDA_BF16 ? kCheckFiniteBF16 : kCheckFiniteF32;
    // raw q and k on the matrix-core path: their norms must suit its float16 operands
    const bool norms = ga != nullptr && mfma;
    const CheckItem qk = norms ? CheckItem{q, rows * H, kCheckRowNormBF16, dk, kRawNormLo, kRawNormHi}
                               : CheckItem{q, nqk, fk, 0, 0.f, 0.f};
    CheckItem kk = qk;
    kk.p = k;
    const CheckItem it[] = {
        qk, kk, {v, nv, fk, 0, 0.f, 0.f},
        ga != nullptr ? CheckItem{ga, nqk, fk, 0, 0.f, 0.f}
                      : CheckItem{g, nqk, kCheckRangeF32, 0, -5.f, 0.f},
        {beta, nb, kCheckFiniteF32, 0, 0.f, 0.f}, {s0, ns, kCheckFiniteF32, 0, 0.f, 0.f},
        {gate, nv, fk, 0, 0.f, 0.f}, {norm_w, dv, kCheckFiniteF32, 0, 0.f, 0.f}};
    const kda_status st = run_checks(it, 8, stream);
    if (st != KDA_OK) return st;
  }

  kda::ChunkArgs a{q, k, v, g, beta, s0, o, s_out, gate, norm_w, eps,
                   B, T, H, dk, dv, scale, io == KDA_BF16, workspace, stream};
  if (ckpt != nullptr && T >= ckpt_every) {
    a.ckpt = ckpt;
    a.ckpt_every = ckpt_every;
  }
  a.cu = cu;
  a.total = rows;
  if (small_ws) a.ws_bytes = (int64_t)workspace_bytes;
  if (ga != nullptr) {
    a.g = nullptr;
    a.ga = ga;
  }
  const hipError_t err = mfma ? kda::launch_chunk_mfma(a) : kda::launch_chunk_valu(a);
  return err == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace

namespace kda {

// kda_chunk_fwd on a workspace that may be smaller than the default one (the
// library's fixed scratch of kda_chunk_fwd_noalloc).
kda_status chunk_fwd_fixed_scratch(const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, const float* s0, void* o, float* s_out,
                                   const void* gate, const float* norm_w, float eps, int64_t B,
                                   int64_t T, int64_t H, int dk, int dv, float scale,
                                   kda_dtype io, void* scratch, size_t scratch_bytes,
                                   void* stream) {
  return chunk_fwd(q, k, v, g, beta, s0, o, s_out, gate, norm_w, eps, B, T, H, dk, dv, scale, io,
                   scratch, scratch_bytes, nullptr, 0, nullptr, 0, nullptr, stream, true);
}

}  // namespace kda

namespace {

// Packed sequences: the checks of the varlen entry points, then chunk_fwd.
kda_status varlen_fwd(const void* q, const void* k, const void* v, const float* g,
                      const float* beta, const int32_t* cu_seqlens, int64_t N, int64_t total,
                      int64_t max_len, const float* s0, void* o, float* s_out, const void* gate,
                      const float* norm_w, float eps, int64_t H, int dk, int dv, float scale,
                      kda_dtype io, void* workspace, size_t workspace_bytes, float* ckpt,
                      int64_t ckpt_every, const void* ga, void* stream) {
  if (cu_seqlens == nullptr) return KDA_ERR_NULL_POINTER;
  if (N < 1 || total < 1 || max_len < 1) return KDA_ERR_BAD_SHAPE;
  if (!aligned(cu_seqlens, 4)) return KDA_ERR_MISALIGNED;
  if (ckpt != nullptr) {
    if (ckpt_every <= 0 || ckpt_every % 32 != 0) return KDA_ERR_BAD_SHAPE;
    if (!aligned(ckpt, 4)) return KDA_ERR_MISALIGNED;
  }
  return chunk_fwd(q, k, v, g, beta, s0, o, s_out, gate, norm_w, eps, N, max_len, H, dk, dv,
                   scale, io, workspace, workspace_bytes, ckpt, ckpt_every, cu_seqlens, total,
                   ga, stream);
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* s0, void* o, float* s_out,
                         const void* gate, const float* norm_w, float eps, int64_t B, int64_t T,
                         int64_t H, int dk, int dv, float scale, kda_dtype io, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return chunk_fwd(q, k, v, g, beta, s0, o, s_out, gate, norm_w, eps, B, T, H, dk, dv, scale, io,
                   workspace, workspace_bytes, nullptr, 0, nullptr, 0, nullptr, stream);
}

kda_status kda_chunk_fwd_prologue(const void* q, const void* k, const void* v, const void* a,
                                  const float* b, const float* s0, void* o, float* s_out,
                                  const void* gate, const float* norm_w, float eps, int64_t B,
                                  int64_t T, int64_t H, int dk, int dv, float scale,
                                  kda_dtype io, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (a == nullptr) return KDA_ERR_NULL_POINTER;
  return chunk_fwd(q, k, v, nullptr, b, s0, o, s_out, gate, norm_w, eps, B, T, H, dk, dv, scale,
                   io, workspace, workspace_bytes, nullptr, 0, nullptr, 0, a, stream);
}

kda_status kda_chunk_fwd_checkpoints(const void* q, const void* k, const void* v,
                                     const float* g, const float* beta, const float* s0,
                                     void* o, float* s_out, const void* gate,
                                     const float* norm_w, float eps, int64_t B, int64_t T,
                                     int64_t H, int dk, int dv, float scale, kda_dtype io,
                                     void* workspace, size_t workspace_bytes, float* ckpt,
                                     int64_t ckpt_every, void* stream) {
  if (ckpt == nullptr) return KDA_ERR_NULL_POINTER;
  if (ckpt_every <= 0 || ckpt_every % 32 != 0) return KDA_ERR_BAD_SHAPE;
  if (!aligned(ckpt, 4)) return KDA_ERR_MISALIGNED;
  return chunk_fwd(q, k, v, g, beta, s0, o, s_out, gate, norm_w, eps, B, T, H, dk, dv, scale, io,
                   workspace, workspace_bytes, ckpt, ckpt_every, nullptr, 0, nullptr, stream);
}

kda_status kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const int32_t* cu_seqlens, int64_t N,
                                int64_t total, int64_t max_len, const float* s0, void* o,
                                float* s_out, const void* gate, const float* norm_w, float eps,
                                int64_t H, int dk, int dv, float scale, kda_dtype io,
                                void* workspace, size_t workspace_bytes, float* ckpt,
                                int64_t ckpt_every, void* stream) {
  return varlen_fwd(q, k, v, g, beta, cu_seqlens, N, total, max_len, s0, o, s_out, gate, norm_w,
                    eps, H, dk, dv, scale, io, workspace, workspace_bytes, ckpt, ckpt_every,
                    nullptr, stream);
}

kda_status kda_chunk_fwd_varlen_prologue(const void* q, const void* k, const void* v,
                                         const void* a, const float* b,
                                         const int32_t* cu_seqlens, int64_t N, int64_t total,
                                         int64_t max_len, const float* s0, void* o,
                                         float* s_out, const void* gate, const float* norm_w,
                                         float eps, int64_t H, int dk, int dv, float scale,
                                         kda_dtype io, void* workspace, size_t workspace_bytes,
                                         float* ckpt, int64_t ckpt_every, void* stream) {
  if (a == nullptr) return KDA_ERR_NULL_POINTER;
  return varlen_fwd(q, k, v, nullptr, b, cu_seqlens, N, total, max_len, s0, o, s_out, gate,
                    norm_w, eps, H, dk, dv, scale, io, workspace, workspace_bytes, ckpt,
                    ckpt_every, a, stream);
}

}  // extern "C"

namespace {

// Input-check mode for the decode entry points (float32 arithmetic: every
// input finite, g in [-5, 0]).
kda_status check_decode(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* state, const void* gate,
                        const float* norm_w, int64_t nqk, int64_t nv, int64_t nb, int64_t ns,
                        int dv, kda_dtype io, const void* ga, void* stream) {
  using namespace kda;
  const int fk = io == KDA_BF16 ? kCheckFiniteBF16 : kCheckFiniteF32;
  const CheckItem it[] = {
      {q, nqk, fk, 0, 0.f, 0.f}, {k, nqk, fk, 0, 0.f, 0.f}, {v, nv, fk, 0, 0.f, 0.f},
      ga != nullptr ? CheckItem{ga, nqk, fk, 0, 0.f, 0.f}
                    : CheckItem{g, nqk, kCheckRangeF32, 0, -5.f, 0.f},
      {beta, nb, kCheckFiniteF32, 0, 0.f, 0.f}, {state, ns, kCheckFiniteF32, 0, 0.f, 0.f},
      {gate, nv, fk, 0, 0.f, 0.f}, {norm_w, dv, kCheckFiniteF32, 0, 0.f, 0.f}};
  return run_checks(it, 8, stream);
}

// kda_decode_step, with the prologue (q, k normalised, gates from their logits)
// when ga is non-NULL.
kda_status decode_step(const void* q, const void* k, const void* v, const float* g,
                       const float* beta, float* state, void* o, const void* gate,
                       const float* norm_w, float eps, int64_t B, int64_t H, int dk, int dv,
                       float scale, kda_dtype io, const void* ga, void* stream) {
  if (!q || !k || !v || (!g && !ga) || !beta || !state || !o) return KDA_ERR_NULL_POINTER;
  if (io != KDA_F32 && io != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED_DIM;
  const int64_t nqk = prod(B, H, dk), nv = prod(B, H, dv), nb = prod(B, H);
  const int64_t ns = prod(B, H, dk, dv);
  if (nqk < 0 || nv < 0 || nb < 0 || ns < 0) return KDA_ERR_BAD_SHAPE;
  if (nb > 0x7fffffffLL) return KDA_ERR_BAD_SHAPE;
  if (!isfinite(scale) || !isfinite(eps) || eps < 0.f) return KDA_ERR_BAD_ARGUMENT;
  // The state is streamed with 16-byte accesses; the per-token vectors are
  // read element by element.
  const uintptr_t ea = (io == KDA_BF16) ? 2 : 4;
  if (!aligned(state, 16)) return KDA_ERR_MISALIGNED;
  for (const void* p : {q, k, v, (const void*)o, gate, ga})
    if (!aligned(p, ea)) return KDA_ERR_MISALIGNED;
  for (const void* p : {(const void*)g, (const void*)beta, (const void*)norm_w})
    if (!aligned(p, 4)) return KDA_ERR_MISALIGNED;

  const int64_t es = (io == KDA_BF16) ? 2 : 4;
  const Span sg = ga != nullptr ? Span{ga, nqk * es} : Span{g, nqk * 4};
  const Span sq{q, nqk * es}, sk{k, nqk * es}, sv{v, nv * es}, sb{beta, nb * 4};
  const Span sst{state, ns * 4}, so{o, nv * es}, sgt{gate, nv * es}, sw{norm_w, (int64_t)dv * 4};
  for (Span in : {sq, sk, sv, sg, sb, sst, sgt, sw})
    if (overlap(so, in)) return KDA_ERR_ALIAS;
  for (Span in : {sq, sk, sv, sg, sb, sgt, sw})
    if (overlap(sst, in)) return KDA_ERR_ALIAS;

  if (kda::check_mode_on()) {
    const kda_status st = check_decode(q, k, v, g, beta, state, gate, norm_w, nqk, nv, nb, ns,
                                       dv, io, ga, stream);
    if (st != KDA_OK) return st;
  }

  kda::DecodeArgs a{q, k, v, g, beta, state, o, gate, norm_w, eps,
                    B, H, dk, dv, scale, io == KDA_BF16, stream};
  a.ga = ga;
  return kda::launch_decode(a) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

kda_status kda_decode_step(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, float* state, void* o, const void* gate,
                           const float* norm_w, float eps, int64_t B, int64_t H, int dk, int dv,
                           float scale, kda_dtype io, void* stream) {
  return decode_step(q, k, v, g, beta, state, o, gate, norm_w, eps, B, H, dk, dv, scale, io,
                     nullptr, stream);
}

kda_status kda_decode_step_prologue(const void* q, const void* k, const void* v,
                                    const void* a, const float* b, float* state, void* o,
                                    const void* gate, const float* norm_w, float eps, int64_t B,
                                    int64_t H, int dk, int dv, float scale, kda_dtype io,
                                    void* stream) {
  if (a == nullptr) return KDA_ERR_NULL_POINTER;
  return decode_step(q, k, v, nullptr, b, state, o, gate, norm_w, eps, B, H, dk, dv, scale, io,
                     a, stream);
}

}  // extern "C"

namespace {

// kda_decode_multi, with the prologue (q, k normalised, gates from their
// logits) when ga is non-NULL.
kda_status decode_multi(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, float* state, const int32_t* n_commit, void* o,
                        const void* gate, const float* norm_w, float eps, int64_t B, int64_t K,
                        int64_t H, int dk, int dv, float scale, kda_dtype io, const void* ga,
                        void* stream) {
  if (!q || !k || !v || (!g && !ga) || !beta || !state) return KDA_ERR_NULL_POINTER;
  if (io != KDA_F32 && io != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED_DIM;
  const int64_t nqk = prod(B, K, H, dk), nv = prod(B, K, H, dv), nb = prod(B, K, H);
  const int64_t ns = prod(B, H, dk, dv);
  if (nqk < 0 || nv < 0 || nb < 0 || ns < 0) return KDA_ERR_BAD_SHAPE;
  if (B * H > 0x7fffffffLL || K > 0x7fffffffLL) return KDA_ERR_BAD_SHAPE;
  if (!isfinite(scale) || !isfinite(eps) || eps < 0.f) return KDA_ERR_BAD_ARGUMENT;
  const uintptr_t ea = (io == KDA_BF16) ? 2 : 4;
  if (!aligned(state, 16)) return KDA_ERR_MISALIGNED;
  for (const void* p : {q, k, v, (const void*)o, gate, ga})
    if (!aligned(p, ea)) return KDA_ERR_MISALIGNED;
  for (const void* p : {(const void*)g, (const void*)beta, (const void*)norm_w,
                        (const void*)n_commit})
    if (!aligned(p, 4)) return KDA_ERR_MISALIGNED;

  const int64_t es = (io == KDA_BF16) ? 2 : 4;
  const Span sg = ga != nullptr ? Span{ga, nqk * es} : Span{g, nqk * 4};
  const Span sq{q, nqk * es}, sk{k, nqk * es}, sv{v, nv * es}, sb{beta, nb * 4};
  const Span sst{state, ns * 4}, so{o, nv * es}, sgt{gate, nv * es}, sw{norm_w, (int64_t)dv * 4};
  const Span sn{n_commit, B * 4};
  for (Span in : {sq, sk, sv, sg, sb, sst, sgt, sw, sn})
    if (overlap(so, in)) return KDA_ERR_ALIAS;
  for (Span in : {sq, sk, sv, sg, sb, sgt, sw, sn})
    if (overlap(sst, in)) return KDA_ERR_ALIAS;

  if (kda::check_mode_on()) {
    const kda_status st = check_decode(q, k, v, g, beta, state, gate, norm_w, nqk, nv, nb, ns,
                                       dv, io, ga, stream);
    if (st != KDA_OK) return st;
  }

  kda::DecodeArgs a{q, k, v, g, beta, state, o, gate, norm_w, eps,
                    B, H, dk, dv, scale, io == KDA_BF16, stream};
  a.K = K;
  a.n_commit = n_commit;
  a.ga = ga;
  return kda::launch_decode(a) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

kda_status kda_decode_multi(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, float* state, const int32_t* n_commit, void* o,
                            const void* gate, const float* norm_w, float eps, int64_t B,
                            int64_t K, int64_t H, int dk, int dv, float scale, kda_dtype io,
                            void* stream) {
  return decode_multi(q, k, v, g, beta, state, n_commit, o, gate, norm_w, eps, B, K, H, dk, dv,
                      scale, io, nullptr, stream);
}

kda_status kda_decode_multi_prologue(const void* q, const void* k, const void* v, const void* a,
                                     const float* b, float* state, const int32_t* n_commit,
                                     void* o, const void* gate, const float* norm_w, float eps,
                                     int64_t B, int64_t K, int64_t H, int dk, int dv, float scale,
                                     kda_dtype io, void* stream) {
  if (a == nullptr) return KDA_ERR_NULL_POINTER;
  return decode_multi(q, k, v, nullptr, b, state, n_commit, o, gate, norm_w, eps, B, K, H, dk,
                      dv, scale, io, a, stream);
}


kda_status kda_gate_rmsnorm(const void* x, const void* gate, const float* norm_w, void* y,
                            int64_t rows, int dv, float eps, kda_dtype io, void* stream) {
  if (!x || !gate || !y) return KDA_ERR_NULL_POINTER;
  if (io != KDA_F32 && io != KDA_BF16) return KDA_ERR_BAD_DTYPE;
  if (!dim_ok(dv)) return KDA_ERR_UNSUPPORTED_DIM;
  const int64_t n = prod(rows, dv);
  if (n < 0) return KDA_ERR_BAD_SHAPE;
  if (!isfinite(eps) || eps < 0.f) return KDA_ERR_BAD_ARGUMENT;
  for (const void* p : {x, gate, (const void*)norm_w, (const void*)y})
    if (!aligned(p, 16)) return KDA_ERR_MISALIGNED;
  const int64_t es = (io == KDA_BF16) ? 2 : 4;
  const Span sx{x, n * es}, sgt{gate, n * es}, sy{y, n * es}, sw{norm_w, (int64_t)dv * 4};
  if (overlap(sy, sgt) || overlap(sy, sw)) return KDA_ERR_ALIAS;
  if (overlap(sy, sx) && x != y) return KDA_ERR_ALIAS;
  kda::NormArgs a{x, gate, norm_w, y, rows, dv, eps, io == KDA_BF16, stream};
  return kda::launch_gate_rmsnorm(a) == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // extern "C"
