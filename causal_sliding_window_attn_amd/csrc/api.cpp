// C ABI of libswattn.so (declared in include/swattn.h): argument validation, workspace sizing and
// kernel launch on the caller's stream.  Every check runs before the first HIP call, so a bad
// call fails identically with or without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/swattn.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return SWATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_ptr(const void* p, const char* name, bool nullable = false) {
  if (!p) return nullable ? SWATTN_OK : fail(SWATTN_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(SWATTN_EINVAL, "%s is not 16-byte aligned", name);
  return SWATTN_OK;
}

int check_dims(const char* what, int B, int H, int T, const char* tname, int D, int window) {
  if (B < 1) return fail(SWATTN_EINVAL, "%s: B = %d must be >= 1", what, B);
  if (H < 1) return fail(SWATTN_EINVAL, "%s: H = %d must be >= 1", what, H);
  if (T < 1) return fail(SWATTN_EINVAL, "%s: %s = %d must be >= 1", what, tname, T);
  if (window < 1) return fail(SWATTN_EINVAL, "%s: window = %d must be >= 1", what, window);
  if (D != 64 && D != 128)
    return fail(SWATTN_EUNSUPPORTED, "%s: head dim D = %d is not supported (64 or 128)", what, D);
  // launch grids: B and H are grid dimensions of the decode (<= 65535 each); the tiled kernels
  // launch (T / 128 + 1) * B * H workgroups on one 31-bit grid dimension
  if (B > 65535 || H > 65535)
    return fail(SWATTN_EINVAL, "%s: B = %d and H = %d must be <= 65535", what, B, H);
  if ((int64_t)(T / 128 + 1) * B * H >= ((int64_t)1 << 31))
    return fail(SWATTN_EINVAL, "%s: (%s/128 + 1) * B * H exceeds 2^31", what, tname);
  return SWATTN_OK;
}

#define TRY(x)                       \
  do {                               \
    int rc_ = (x);                   \
    if (rc_ != SWATTN_OK) return rc_; \
  } while (0)

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SWATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

float scale_log2_for(int D) { return (float)(1.4426950408889634 / sqrt((double)D)); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int decode_chunks(int Lcap) { return (Lcap + swattn::kDecodeChunk - 1) / swattn::kDecodeChunk; }

// The split decode launches one workgroup per (head, chunk, sequence) with the chunk index on the
// grid's y dimension, at most 65535.
int check_decode_cap(const char* what, int Lcap) {
  if (decode_chunks(Lcap) > 65535)
    return fail(SWATTN_EINVAL, "%s: Lcap = %d exceeds %d rows", what, Lcap,
                65535 * swattn::kDecodeChunk);
  return SWATTN_OK;
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return SWATTN_ABI_VERSION; }

const char* attn_last_error(void) { return g_err; }

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int T,
             int D, int window, int dtype, void* stream) {
  TRY(check_dims("attn_fwd", B, H, T, "T", D, window));
  if (dtype != SWATTN_BF16 && dtype != SWATTN_F32)
    return fail(SWATTN_EUNSUPPORTED, "attn_fwd: dtype %d is not supported", dtype);
  // the fp32 kernel launches one workgroup per 32 queries of each (sequence, head)
  if (dtype == SWATTN_F32 && (int64_t)(T / 32 + 1) * B * H >= ((int64_t)1 << 31))
    return fail(SWATTN_EINVAL, "attn_fwd: (T/32 + 1) * B * H exceeds 2^31 for fp32");
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(k, "k"));
  TRY(check_ptr(v, "v"));
  TRY(check_ptr(o, "o"));
  TRY(check_ptr(lse, "lse", true));
  swattn::FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.lens = nullptr;
  a.q_bstride = a.kv_bstride = (int64_t)T * H * D;
  a.row_stride = H * D;
  a.H = H;
  a.BH = B * H;
  a.D = D;
  a.T = T;
  a.kv_len = T;
  a.window = window;
  a.lse_T = T;
  a.scale_log2 = scale_log2_for(D);
  (void)hipGetLastError();
  return hip_status(swattn::launch_fwd(a, dtype == SWATTN_F32, static_cast<hipStream_t>(stream)),
                    "attn_fwd launch");
}

size_t attn_bwd_workspace_bytes(int B, int H, int T, int D) {
  if (B < 1 || H < 1 || T < 1 || (D != 64 && D != 128)) return 0;
  // Delta, then LSE in base 2, then the packed-sequence dK/dV pass's job queue counter and plan
  return 2 * align256((size_t)B * H * T * sizeof(float)) + 256 +
         align256((size_t)swattn::kDkdvPlanMax * sizeof(int));
}

}  // extern "C"

namespace {

enum BwdPass { kBoth, kDq, kDkdv };

int bwd_common(const char* what, BwdPass pass, const void* q, const void* k, const void* v,
               const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
               int B, int H, int T, int D, int window, int dtype, void* ws, size_t ws_bytes,
               void* stream, const float* rq = nullptr, const float* rk = nullptr) {
  TRY(check_dims(what, B, H, T, "T", D, window));
  if (dtype != SWATTN_BF16)
    return fail(SWATTN_EUNSUPPORTED, "%s: only bf16 (dtype 0) is implemented, got %d", what, dtype);
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(k, "k"));
  TRY(check_ptr(v, "v"));
  if (pass != kDkdv) TRY(check_ptr(o, "o"));
  TRY(check_ptr(lse, "lse"));
  TRY(check_ptr(dout, "dout"));
  if (pass != kDkdv) TRY(check_ptr(dq, "dq"));
  if (pass != kDq) {
    TRY(check_ptr(dk, "dk"));
    TRY(check_ptr(dv, "dv"));
  }
  const size_t need = attn_bwd_workspace_bytes(B, H, T, D);
  if (!ws) return fail(SWATTN_EWORKSPACE, "%s: workspace is NULL (%zu bytes needed)", what, need);
  if (!aligned16(ws)) return fail(SWATTN_EINVAL, "%s: workspace is not 16-byte aligned", what);
  if (ws_bytes < need)
    return fail(SWATTN_EWORKSPACE, "%s: workspace of %zu bytes < %zu needed", what, ws_bytes, need);
  swattn::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  const size_t rows_bytes = align256((size_t)B * H * T * sizeof(float));
  a.delta = static_cast<float*>(ws);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(ws) + rows_bytes);
  a.qctr = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + 2 * rows_bytes);
  a.bstride = (int64_t)T * H * D;
  a.row_stride = H * D;
  a.H = H;
  a.BH = B * H;
  a.D = D;
  a.T = T;
  a.window = window;
  a.rq = rq;
  a.rk = rk;
  a.scale = (float)(1.0 / sqrt((double)D));
  a.scale_log2 = scale_log2_for(D);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (pass != kDkdv) {
    const int rc = hip_status(swattn::launch_bwd_dq(a, s), what);
    if (rc != SWATTN_OK) return rc;
  }
  if (pass != kDq) return hip_status(swattn::launch_bwd_dkdv(a, s), what);
  return ok();
}

}  // namespace

extern "C" {

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int B, int H, int T, int D, int window,
             int dtype, void* ws, size_t ws_bytes, void* stream) {
  return bwd_common("attn_bwd", kBoth, q, k, v, o, lse, dout, dq, dk, dv, B, H, T, D, window, dtype,
                    ws, ws_bytes, stream);
}

int attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dout, void* dq, int B, int H, int T, int D, int window, int dtype,
                void* ws, size_t ws_bytes, void* stream) {
  return bwd_common("attn_bwd_dq", kDq, q, k, v, o, lse, dout, dq, nullptr, nullptr, B, H, T, D,
                    window, dtype, ws, ws_bytes, stream);
}

int attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                  void* dk, void* dv, int B, int H, int T, int D, int window, int dtype, void* ws,
                  size_t ws_bytes, void* stream) {
  return bwd_common("attn_bwd_dkdv", kDkdv, q, k, v, nullptr, lse, dout, nullptr, dk, dv, B, H, T,
                    D, window, dtype, ws, ws_bytes, stream);
}

int attn_prefill(const void* q, const void* kcache, const void* vcache, const int* lens, void* o,
                 float* lse, int B, int H, int Tq, int Lcap, int D, int window, void* stream) {
  TRY(check_dims("attn_prefill", B, H, Tq, "Tq", D, window));
  if (Lcap < 1) return fail(SWATTN_EINVAL, "attn_prefill: Lcap = %d must be >= 1", Lcap);
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(kcache, "kcache"));
  TRY(check_ptr(vcache, "vcache"));
  if (!lens) return fail(SWATTN_EINVAL, "lens is NULL");
  if (reinterpret_cast<uintptr_t>(lens) & 3u) return fail(SWATTN_EINVAL, "lens is not 4-byte aligned");
  TRY(check_ptr(o, "o"));
  TRY(check_ptr(lse, "lse", true));
  swattn::FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(kcache);
  a.v = static_cast<const uint16_t*>(vcache);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.lens = lens;
  a.q_bstride = (int64_t)Tq * H * D;
  a.kv_bstride = (int64_t)Lcap * H * D;
  a.row_stride = H * D;
  a.H = H;
  a.BH = B * H;
  a.D = D;
  a.T = Tq;
  a.kv_len = Tq < Lcap ? Tq : Lcap;
  a.window = window;
  a.lse_T = Tq;
  a.scale_log2 = scale_log2_for(D);
  (void)hipGetLastError();
  return hip_status(swattn::launch_fwd(a, false, static_cast<hipStream_t>(stream)),
                    "attn_prefill launch");
}

int attn_kv_append(void* kcache, void* vcache, const void* knew, const void* vnew, const int* pos,
                   int B, int H, int Lcap, int D, void* stream) {
  TRY(check_dims("attn_kv_append", B, H, Lcap, "Lcap", D, 1));
  TRY(check_ptr(kcache, "kcache"));
  TRY(check_ptr(vcache, "vcache"));
  TRY(check_ptr(knew, "knew"));
  TRY(check_ptr(vnew, "vnew"));
  if (!pos) return fail(SWATTN_EINVAL, "pos is NULL");
  if (reinterpret_cast<uintptr_t>(pos) & 3u) return fail(SWATTN_EINVAL, "pos is not 4-byte aligned");
  swattn::AppendArgs a{};
  a.kc = static_cast<uint16_t*>(kcache);
  a.vc = static_cast<uint16_t*>(vcache);
  a.kn = static_cast<const uint16_t*>(knew);
  a.vn = static_cast<const uint16_t*>(vnew);
  a.pos = pos;
  a.B = B;
  a.H = H;
  a.D = D;
  a.Lcap = Lcap;
  (void)hipGetLastError();
  return hip_status(swattn::launch_append(a, static_cast<hipStream_t>(stream)),
                    "attn_kv_append launch");
}

size_t attn_decode_workspace_bytes(int B, int H, int Lcap, int D) {
  if (B < 1 || H < 1 || Lcap < 1 || (D != 64 && D != 128)) return 0;
  const size_t slots = (size_t)B * H * decode_chunks(Lcap);
  return align256(slots * D * sizeof(float)) + align256(slots * 2 * sizeof(float));
}

int attn_decode_launches(int B, int H, int Lcap, int D, int window) {
  TRY(check_dims("attn_decode_launches", B, H, Lcap, "Lcap", D, window));
  TRY(check_decode_cap("attn_decode_launches", Lcap));
  ok();
  return swattn::decode_uses_fused(B, H, Lcap, window) ? 1 : 2;
}

int attn_decode(const void* q, const void* kcache, const void* vcache, const int* lens, void* o,
                float* lse, int B, int H, int Lcap, int D, int window, void* ws, size_t ws_bytes,
                void* stream) {
  TRY(check_dims("attn_decode", B, H, Lcap, "Lcap", D, window));
  TRY(check_decode_cap("attn_decode", Lcap));
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(kcache, "kcache"));
  TRY(check_ptr(vcache, "vcache"));
  if (!lens) return fail(SWATTN_EINVAL, "lens is NULL");
  if (reinterpret_cast<uintptr_t>(lens) & 3u) return fail(SWATTN_EINVAL, "lens is not 4-byte aligned");
  TRY(check_ptr(o, "o"));
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(SWATTN_EINVAL, "lse is not 4-byte aligned");
  const size_t need = attn_decode_workspace_bytes(B, H, Lcap, D);
  if (!ws) return fail(SWATTN_EWORKSPACE, "attn_decode: workspace is NULL (%zu bytes needed)", need);
  if (!aligned16(ws)) return fail(SWATTN_EINVAL, "attn_decode: workspace is not 16-byte aligned");
  if (ws_bytes < need)
    return fail(SWATTN_EWORKSPACE, "attn_decode: workspace of %zu bytes < %zu needed", ws_bytes,
                need);
  const int nc_max = decode_chunks(Lcap);
  const size_t slots = (size_t)B * H * nc_max;
  swattn::DecArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kc = static_cast<const uint16_t*>(kcache);
  a.vc = static_cast<const uint16_t*>(vcache);
  a.lens = lens;
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.ws_o = static_cast<float*>(ws);
  a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(slots * D * sizeof(float)));
  a.B = B;
  a.H = H;
  a.D = D;
  a.Lcap = Lcap;
  a.window = window;
  a.nc_max = nc_max;
  a.scale_log2 = scale_log2_for(D);
  (void)hipGetLastError();
  return hip_status(swattn::launch_decode(a, static_cast<hipStream_t>(stream)),
                    "attn_decode launch");
}

int attn_decode_step(const void* q, const void* knew, const void* vnew, void* kcache, void* vcache,
                     const int* pos, void* o, float* lse, int B, int H, int Lcap, int D,
                     int window, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_dims("attn_decode_step", B, H, Lcap, "Lcap", D, window));
  TRY(check_decode_cap("attn_decode_step", Lcap));
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(knew, "knew"));
  TRY(check_ptr(vnew, "vnew"));
  TRY(check_ptr(kcache, "kcache"));
  TRY(check_ptr(vcache, "vcache"));
  if (!pos) return fail(SWATTN_EINVAL, "pos is NULL");
  if (reinterpret_cast<uintptr_t>(pos) & 3u) return fail(SWATTN_EINVAL, "pos is not 4-byte aligned");
  TRY(check_ptr(o, "o"));
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(SWATTN_EINVAL, "lse is not 4-byte aligned");
  const size_t need = attn_decode_workspace_bytes(B, H, Lcap, D);
  if (!ws)
    return fail(SWATTN_EWORKSPACE, "attn_decode_step: workspace is NULL (%zu bytes needed)", need);
  if (!aligned16(ws))
    return fail(SWATTN_EINVAL, "attn_decode_step: workspace is not 16-byte aligned");
  if (ws_bytes < need)
    return fail(SWATTN_EWORKSPACE, "attn_decode_step: workspace of %zu bytes < %zu needed",
                ws_bytes, need);
  const int nc_max = decode_chunks(Lcap);
  const size_t slots = (size_t)B * H * nc_max;
  swattn::DecArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kc = static_cast<const uint16_t*>(kcache);
  a.vc = static_cast<const uint16_t*>(vcache);
  a.pos = pos;
  a.kn = static_cast<const uint16_t*>(knew);
  a.vn = static_cast<const uint16_t*>(vnew);
  a.kcw = static_cast<uint16_t*>(kcache);
  a.vcw = static_cast<uint16_t*>(vcache);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.ws_o = static_cast<float*>(ws);
  a.ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + align256(slots * D * sizeof(float)));
  a.B = B;
  a.H = H;
  a.D = D;
  a.Lcap = Lcap;
  a.window = window;
  a.nc_max = nc_max;
  a.scale_log2 = scale_log2_for(D);
  (void)hipGetLastError();
  return hip_status(swattn::launch_decode(a, static_cast<hipStream_t>(stream)),
                    "attn_decode_step launch");
}

int attn_decode_step_noalloc(const void* q, const void* knew, const void* vnew, void* kcache,
                             void* vcache, const int* pos, void* o, float* lse, int B, int H,
                             int Lcap, int D, int window, void* stream) {
  const char* what = "attn_decode_step_noalloc";
  TRY(check_dims(what, B, H, Lcap, "Lcap", D, window));
  TRY(check_decode_cap(what, Lcap));
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(knew, "knew"));
  TRY(check_ptr(vnew, "vnew"));
  TRY(check_ptr(kcache, "kcache"));
  TRY(check_ptr(vcache, "vcache"));
  if (!pos) return fail(SWATTN_EINVAL, "pos is NULL");
  if (reinterpret_cast<uintptr_t>(pos) & 3u) return fail(SWATTN_EINVAL, "pos is not 4-byte aligned");
  TRY(check_ptr(o, "o"));
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(SWATTN_EINVAL, "lse is not 4-byte aligned");
  // only the split schedule keeps partial results; the one-launch schedule needs no scratch
  const bool split = !swattn::decode_uses_fused(B, H, Lcap, window);
  const int nc_max = decode_chunks(Lcap);
  const size_t slots = (size_t)B * H * nc_max;
  const size_t need = split ? attn_decode_workspace_bytes(B, H, Lcap, D) : 0;
  if (need > swattn::kNoAllocScratchBytes)
    return fail(SWATTN_EWORKSPACE,
                "%s: these sizes take the split schedule, whose partial results need %zu bytes, "
                "more than the %zu-byte static scratch (use attn_decode_step with a workspace)",
                what, need, swattn::kNoAllocScratchBytes);
  void* ws = nullptr;
  (void)hipGetLastError();
  if (split) TRY(hip_status(swattn::decode_noalloc_scratch(&ws), "attn_decode_step_noalloc scratch"));
  swattn::DecArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kc = static_cast<const uint16_t*>(kcache);
  a.vc = static_cast<const uint16_t*>(vcache);
  a.pos = pos;
  a.kn = static_cast<const uint16_t*>(knew);
  a.vn = static_cast<const uint16_t*>(vnew);
  a.kcw = static_cast<uint16_t*>(kcache);
  a.vcw = static_cast<uint16_t*>(vcache);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.ws_o = static_cast<float*>(ws);
  a.ws_ml = split ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                             align256(slots * D * sizeof(float)))
                  : nullptr;
  a.B = B;
  a.H = H;
  a.D = D;
  a.Lcap = Lcap;
  a.window = window;
  a.nc_max = nc_max;
  a.scale_log2 = scale_log2_for(D);
  return hip_status(swattn::launch_decode(a, static_cast<hipStream_t>(stream)),
                    "attn_decode_step_noalloc launch");
}

// Packed sequences (documents): shared argument checks of attn_fwd_varlen / attn_bwd_varlen.
static int check_varlen(const char* what, const int* cu, int nseq, int total, int max_seqlen,
                        int H, int D, int window) {
  TRY(check_dims(what, nseq, H, max_seqlen, "max_seqlen", D, window));
  if (total < 1) return fail(SWATTN_EINVAL, "%s: total = %d must be >= 1", what, total);
  if (max_seqlen > total)
    return fail(SWATTN_EINVAL, "%s: max_seqlen = %d exceeds total = %d", what, max_seqlen, total);
  if (!cu) return fail(SWATTN_EINVAL, "%s: cu_seqlens is NULL", what);
  if (reinterpret_cast<uintptr_t>(cu) & 3u)
    return fail(SWATTN_EINVAL, "%s: cu_seqlens is not 4-byte aligned", what);
  return SWATTN_OK;
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens, int nseq, int total, int max_seqlen, int H, int D,
                    int window, void* stream) {
  TRY(check_varlen("attn_fwd_varlen", cu_seqlens, nseq, total, max_seqlen, H, D, window));
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(k, "k"));
  TRY(check_ptr(v, "v"));
  TRY(check_ptr(o, "o"));
  TRY(check_ptr(lse, "lse", true));
  swattn::FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.cu = cu_seqlens;
  a.total = total;
  a.row_stride = H * D;
  a.H = H;
  a.BH = nseq * H;
  a.D = D;
  a.T = max_seqlen;
  a.kv_len = max_seqlen;
  a.window = window;
  a.scale_log2 = scale_log2_for(D);
  (void)hipGetLastError();
  return hip_status(swattn::launch_fwd(a, false, static_cast<hipStream_t>(stream)),
                    "attn_fwd_varlen launch");
}

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, const int* cu_seqlens,
                    int nseq, int total, int max_seqlen, int H, int D, int window, void* ws,
                    size_t ws_bytes, void* stream) {
  const char* what = "attn_bwd_varlen";
  TRY(check_varlen(what, cu_seqlens, nseq, total, max_seqlen, H, D, window));
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(k, "k"));
  TRY(check_ptr(v, "v"));
  TRY(check_ptr(o, "o"));
  TRY(check_ptr(lse, "lse"));
  TRY(check_ptr(dout, "dout"));
  TRY(check_ptr(dq, "dq"));
  TRY(check_ptr(dk, "dk"));
  TRY(check_ptr(dv, "dv"));
  const size_t need = attn_bwd_workspace_bytes(1, H, total, D);
  if (!ws) return fail(SWATTN_EWORKSPACE, "%s: workspace is NULL (%zu bytes needed)", what, need);
  if (!aligned16(ws)) return fail(SWATTN_EINVAL, "%s: workspace is not 16-byte aligned", what);
  if (ws_bytes < need)
    return fail(SWATTN_EWORKSPACE, "%s: workspace of %zu bytes < %zu needed", what, ws_bytes, need);
  swattn::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  const size_t rows_bytes = align256((size_t)H * total * sizeof(float));
  a.delta = static_cast<float*>(ws);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(ws) + rows_bytes);
  a.qctr = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + 2 * rows_bytes);
  a.plan = swattn::dkdv_plan_fits(nseq, total, max_seqlen)
               ? reinterpret_cast<int*>(static_cast<char*>(ws) + 2 * rows_bytes + 256)
               : nullptr;
  a.cu = cu_seqlens;
  a.total = total;
  a.row_stride = H * D;
  a.H = H;
  a.BH = nseq * H;
  a.D = D;
  a.T = max_seqlen;
  a.window = window;
  a.scale = (float)(1.0 / sqrt((double)D));
  a.scale_log2 = scale_log2_for(D);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int rc = hip_status(swattn::launch_bwd_dq(a, s), what);
  if (rc != SWATTN_OK) return rc;
  return hip_status(swattn::launch_bwd_dkdv(a, s), what);
}

int attn_fwd_qknorm(const void* q, const void* k, const void* v, void* qn, void* kn, float* rq,
                    float* rk, void* o, float* lse, int B, int H, int T, int D, int window,
                    float eps, void* stream) {
  TRY(check_dims("attn_fwd_qknorm", B, H, T, "T", D, window));
  if (!(eps >= 0.f) || !isfinite(eps))
    return fail(SWATTN_EINVAL, "attn_fwd_qknorm: eps = %g must be finite and >= 0", (double)eps);
  TRY(check_ptr(q, "q"));
  TRY(check_ptr(k, "k"));
  TRY(check_ptr(v, "v"));
  TRY(check_ptr(qn, "qn"));
  TRY(check_ptr(kn, "kn"));
  TRY(check_ptr(rq, "rq"));
  TRY(check_ptr(rk, "rk"));
  TRY(check_ptr(o, "o"));
  TRY(check_ptr(lse, "lse", true));
  // k through the normalisation pass; q is normalised inside the forward's prologue
  swattn::NormArgs na{};
  na.q = nullptr;
  na.k = static_cast<const uint16_t*>(k);
  na.kn = static_cast<uint16_t*>(kn);
  na.rk = rk;
  na.B = B;
  na.T = T;
  na.H = H;
  na.D = D;
  na.eps = eps;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  TRY(hip_status(swattn::launch_qk_rmsnorm(na, s), "attn_fwd_qknorm norm launch"));
  swattn::FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.qn = static_cast<uint16_t*>(qn);
  a.rq = rq;
  a.eps = eps;
  a.k = static_cast<const uint16_t*>(kn);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.q_bstride = a.kv_bstride = (int64_t)T * H * D;
  a.row_stride = H * D;
  a.H = H;
  a.BH = B * H;
  a.D = D;
  a.T = T;
  a.kv_len = T;
  a.window = window;
  a.lse_T = T;
  a.scale_log2 = scale_log2_for(D);
  return hip_status(swattn::launch_fwd(a, false, s), "attn_fwd_qknorm launch");
}

int attn_bwd_qknorm(const void* qn, const void* kn, const void* v, const void* o, const float* lse,
                    const void* dout, const float* rq, const float* rk, void* dq, void* dk,
                    void* dv, int B, int H, int T, int D, int window, void* ws, size_t ws_bytes,
                    void* stream) {
  if (!rq) return fail(SWATTN_EINVAL, "attn_bwd_qknorm: rq is NULL");
  if (!rk) return fail(SWATTN_EINVAL, "attn_bwd_qknorm: rk is NULL");
  if (!aligned16(rq) || !aligned16(rk))
    return fail(SWATTN_EINVAL, "attn_bwd_qknorm: rq / rk are not 16-byte aligned");
  return bwd_common("attn_bwd_qknorm", kBoth, qn, kn, v, o, lse, dout, dq, dk, dv, B, H, T, D,
                    window, SWATTN_BF16, ws, ws_bytes, stream, rq, rk);
}

}  // extern "C"
