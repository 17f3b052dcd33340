// Internal host-side launch interface between the C ABI (api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swattn {

// Forward / prefill.  Pointers are bf16 (uint16_t) or fp32 (reinterpreted by the fp32 kernel).
struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;          // [BH, lse_T] or null
  const int* lens;     // per-batch valid length (prefill) or null (training: every row valid)
  const int* cu;       // packed sequences: sequence b is rows cu[b] .. cu[b + 1] - 1 of
                       // [total, H, D] (lse [H, total]), or null
  int total;           // packed sequences: rows in q / k / v / o
  int64_t q_bstride;   // elements between batches of q / o
  int64_t kv_bstride;  // elements between batches of k / v
  int row_stride;      // elements between consecutive tokens (H * D)
  int H, BH, D;
  int T;               // query rows per batch
  int kv_len;          // keys per batch (training: T; prefill: min(Tq, Lcap), lens clamp)
  int window;          // >= 1
  int lse_T;
  int n_qtiles;        // filled by the launcher
  float scale_log2;    // log2(e) / sqrt(D)
  // QK-norm forward (dense training only): q holds the raw rows; each row is RMS-normalised in
  // registers, the bf16 result written to qn ([B, T, H, D]) and 1 / rms to rq ([B, H, T]).
  uint16_t* qn;        // null: q is used as given
  float* rq;
  float eps;
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;  // [BH, T]
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;      // [BH, T] workspace: Delta_i = dO_i . O_i (written by the dQ pass)
  float* lse2;       // [BH, T] workspace: LSE_i * log2(e) (written by the dQ pass)
  unsigned* qctr;    // workspace: packed sequences' dK/dV job queue counter
  int* plan;         // workspace: packed sequences' dK/dV job plan (built by the dQ pass), or
                     // null (the dK/dV pass then runs one workgroup per unit)
  const int* cu;     // packed sequences (rows cu[b] .. cu[b + 1] - 1 of [total, H, D]; lse,
                     // Delta and LSE * log2(e) as [H, total]), or null; T is then the longest
  int total;         // packed sequences: rows in q / k / v / o / dO
  const float* rq;   // QK-norm backward: 1 / rms of each q row [BH, T] (q holds the normalised
  const float* rk;   // rows), and of each k row; dq, dk are then taken back through the norm
  int64_t bstride;   // T * H * D
  int row_stride;    // H * D
  int H, BH, D, T, window;
  int n_tiles;       // filled by the launcher
  int paired;        // filled by the launcher: full-causal training schedule (tile pairs)
  float scale;       // 1 / sqrt(D)
  float scale_log2;  // log2(e) / sqrt(D)
};

struct DecArgs {
  const uint16_t* q;   // [B, H, D]
  const uint16_t* kc;  // [B, Lcap, H, D]
  const uint16_t* vc;
  const int* lens;     // decode: cached tokens including the new one
  const int* pos;      // decode step (append + decode): the new row's index, or null
  const uint16_t* kn;  // decode step: the new row's key / value [B, H, D]
  const uint16_t* vn;
  uint16_t* kcw;       // decode step: the caches, written at row pos
  uint16_t* vcw;
  uint16_t* o;         // [B, H, D]
  float* lse;          // [B, H] or null
  float* ws_o;         // [B*H, nc_max, D]
  float* ws_ml;        // [B*H, nc_max, 2]
  int B, H, D, Lcap, window, nc_max;
  float scale_log2;
};

// Parameter-free RMS normalisation of the q and k rows ([B, T, H, D] bf16).
struct NormArgs {
  const uint16_t* q;  // null: k only
  const uint16_t* k;
  uint16_t* qn;  // q / rms(q), bf16
  uint16_t* kn;
  float* rq;     // 1 / rms per row, [B, H, T]
  float* rk;
  int B, T, H, D;
  float eps;
};

struct AppendArgs {
  uint16_t* kc;
  uint16_t* vc;
  const uint16_t* kn;
  const uint16_t* vn;
  const int* pos;
  int B, H, D, Lcap;
};

constexpr int kDecodeChunk = 64;  // keys per split of the decode

// Decode schedule: one workgroup of 8 waves per (sequence, head), its chunks merged in LDS, in one
// launch; or one wave per (head, chunk, sequence) and a merge kernel.  Measured on MI355X (H = 15,
// D = 128, ragged and full-length caches of 512 to 16384 rows): with at most 2048 visible rows the
// one-launch schedule is at most 30% slower at 1-4 sequences over full caches and up to 25% faster
// over ragged ones; over longer caches the split schedule is 1.1-4.3x faster below 128 (sequence,
// head) pairs (one workgroup per pair leaves most CUs idle there), and 7-12% slower from 240 up.
constexpr int kDecodeFusedMinPairs = 128;
constexpr int kDecodeFusedMaxRows = 2048;
inline bool decode_uses_fused(int B, int H, int Lcap, int window) {
  const int visible = window < Lcap ? window : Lcap;
  return (long long)B * H >= kDecodeFusedMinPairs || visible <= kDecodeFusedMaxRows;
}

// Packed sequences' dK/dV job plan: for every 128-key level kt (key tile kt of a sequence), the
// sequences long enough to have that tile, in sequence order.  Laid out as C[0 .. levels] (C[kt]:
// entries before level kt), then the entries (sequence indices).  Used only when it surely fits
// kDkdvPlanMax ints (the dK/dV workgroups hold it in LDS) and there are at most kDkdvPlanSeqs
// sequences (the dQ pass builds it in LDS).
constexpr int kDkdvPlanMax = 6144;
constexpr int kDkdvPlanSeqs = 8192;
inline bool dkdv_plan_fits(long long nseq, long long total, long long max_seqlen) {
  const long long levels = (max_seqlen + 127) / 128;
  long long entries = nseq * levels;  // at most: every nonempty sequence adds one per 128 rows
  const long long by_rows = total / 128 + (nseq < total ? nseq : total);
  if (by_rows < entries) entries = by_rows;
  return nseq <= kDkdvPlanSeqs && levels + 1 + entries <= kDkdvPlanMax;
}

// Static scratch of the allocation-free decode step (attn_decode_step_noalloc): the split
// schedule's partial results, in a file-scope device array of decode.hip (one copy per GPU, held
// until the process ends).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
// Device address of this GPU's copy of the scratch array (the current device's), looked up with
// hipGetSymbolAddress on the first call on each device and kept.
hipError_t decode_noalloc_scratch(void** ptr);

// Compute units of the current device (looked up once per device).
int device_compute_units();

// Whether the full-causal tile-pair schedule (every workgroup the same work) fills whole rounds of
// `slots` resident workgroups closely enough.  When the last round is mostly empty (d26: 1664 pairs
// on 512 forward slots, 3.25 rounds), single query tiles taken longest first pack it better.
inline bool pairs_fill_rounds(unsigned pairs, unsigned slots) {
  if (slots == 0 || pairs <= slots) return true;
  const unsigned long long cap = (unsigned long long)((pairs + slots - 1) / slots) * slots;
  return (cap - pairs) * 16 <= cap;  // at most 1/16 of the last round's slots idle
}

hipError_t launch_fwd(const FwdArgs& a, bool f32, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t s);
hipError_t launch_decode(const DecArgs& a, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_qk_rmsnorm(const NormArgs& a, hipStream_t s);

}  // namespace swattn
