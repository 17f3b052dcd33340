/*
 * swattn.h -- C ABI of libswattn.so: exact softmax causal self-attention with an optional sliding
 * window, for AMD Instinct MI355X (gfx950).
 *
 * What the operations are
 *   The training attention with a per-layer window: "nanochat: GPT-2-grade LLM for <<$100" post
 *   (web3.cnoyu.life, the "Jan29" entry), list of the largest improvements, item 1 -- attention
 *   kernels whose window_size keyword lets layers alternate short and long attention patterns.
 *   The KV-cache Engine with its prefill and decode phases: walkthrough "A fully hand-made copy of
 *   ChatGPT for $100 and 8,000 lines of code" (followin.io), section "Pretraining", closing
 *   paragraph; nanochat launch post (web3.ouchyi.army), feature list.
 *   Shapes of the d20 layer (1280 channels = 10 heads x 128; 32 x 2048 tokens per GPU): same
 *   walkthrough, section "Pretraining".
 *
 * Definition (the pages give no formula; this is the textbook one, with the window read as
 * counting the query's own key):
 *   query i sees key j iff 0 <= j <= i and i - j < w;  any w >= T is full causal attention.
 *   s_ij = q_i . k_j / sqrt(D);  LSE_i = ln sum_j exp(s_ij);  P_ij = exp(s_ij - LSE_i);
 *   O_i = sum_j P_ij v_j.   Backward (no gradient into LSE):
 *   dV_j = sum_i P_ij dO_i;  dS_ij = P_ij (dO_i.v_j - dO_i.O_i);
 *   dQ_i = sum_j dS_ij k_j / sqrt(D);  dK_j = sum_i dS_ij q_i / sqrt(D).
 *
 * Conventions shared by every entry point
 *   Layout:    activations [B, T, H, D] row-major, D fastest (what a fused QKV projection yields);
 *              KV cache [B, Lcap, H, D]; LSE [B, H, T] float32 (natural log).
 *   Types:     bf16 storage with fp32 accumulation; the forward also accepts fp32 (SWATTN_F32).
 *   Pointers:  device memory owned by the caller; the library allocates nothing and keeps no state
 *              besides the thread-local error text and the static scratch array of
 *              attn_decode_step_noalloc.  Tensor and workspace pointers must be 16-byte aligned;
 *              int32 length / position arrays and the decode's lse need 4 bytes.
 *   Streams:   `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue and return; the
 *              caller keeps every buffer alive until the stream has passed the kernels.
 *   Errors:    every check below runs on the host before any HIP call.  A failing call returns a
 *              negative status, launches nothing and sets attn_last_error() (thread-local text,
 *              valid until the next call on that thread).  Faults inside kernels surface at the
 *              caller's next synchronisation.  No entry point throws.
 *   Window:    window >= 1; any window >= the sequence length means full causal attention.
 *   Head dim:  D in {64, 128}.
 *   Threads:   entry points are re-entrant; concurrent calls may share nothing they write (calls
 *              of attn_decode_step_noalloc on one GPU share its scratch, see there).
 */
#ifndef SWATTN_H
#define SWATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWATTN_ABI_VERSION 6  /* 2: attn_decode_step; 3: *_varlen; 4: *_qknorm;
                                 5: attn_decode_launches; 6: attn_decode_step_noalloc */

typedef enum { SWATTN_BF16 = 0, SWATTN_F32 = 1 } swattn_dtype;

enum {
  SWATTN_OK = 0,
  SWATTN_EINVAL = -1,       /* null pointer, size < 1, window < 1, misaligned pointer          */
  SWATTN_EUNSUPPORTED = -2, /* D not 64/128, or a dtype the entry point does not implement      */
  SWATTN_EWORKSPACE = -3,   /* workspace pointer null or smaller than the *_workspace_bytes size */
  SWATTN_EHIP = -4          /* the HIP runtime refused the launch (message in attn_last_error)  */
};

/* ABI version of the loaded library (SWATTN_ABI_VERSION at build time). */
int attn_abi_version(void);

/* Text of the last failure on the calling thread ("" after a successful call). */
const char* attn_last_error(void);

/*
 * Training forward (the "Jan29" post's attention kernel with window_size).
 *   q, k, v  [B, T, H, D] in `dtype` (read).        o [B, T, H, D] in `dtype` (written).
 *   lse      [B, H, T] float32 (written), may be NULL when no backward will follow.
 *   window   keys visible to each query, counting itself (>= T: full causal).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int T,
             int D, int window, int dtype, void* stream);

/* Bytes of device workspace attn_bwd needs: per row, Delta_i = dO_i . O_i and LSE_i * log2(e)
 * (float32 each), written by the dQ pass and read by the dK/dV pass, and a fixed 24.25 KiB for the
 * packed-sequence dK/dV pass's job queue and plan. */
size_t attn_bwd_workspace_bytes(int B, int H, int T, int D);

/*
 * Training backward, split into a dQ pass and a dK/dV pass that both recompute P from LSE.
 *   q, k, v, o, dout [B, T, H, D] bf16 (read); lse [B, H, T] float32 from attn_fwd (read).
 *   dq, dk, dv [B, T, H, D] bf16 (written, fully overwritten; no accumulation into them).
 *   ws / ws_bytes: caller-owned device scratch of at least attn_bwd_workspace_bytes(); its
 *   contents on entry do not matter.  dtype must be SWATTN_BF16 (fp32 returns -2).
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int B, int H, int T, int D, int window,
             int dtype, void* ws, size_t ws_bytes, void* stream);

/*
 * The two passes of attn_bwd, for callers that schedule or time them separately.  attn_bwd is
 * exactly attn_bwd_dq followed by attn_bwd_dkdv on the same stream with the same arguments.
 *   attn_bwd_dq:   writes Delta_i = dO_i . O_i and LSE_i * log2(e) into ws, and dq.
 *   attn_bwd_dkdv: reads both from ws as left there by attn_bwd_dq for the same (q, k, v, o, lse,
 *                  dout, shapes, window) and writes dk, dv.  Called without that, results are
 *                  undefined (but every access stays inside the buffers).
 * Arguments, layouts, validation and status codes are those of attn_bwd.
 */
int attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dout, void* dq, int B, int H, int T, int D, int window, int dtype,
                void* ws, size_t ws_bytes, void* stream);
int attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                  void* dk, void* dv, int B, int H, int T, int D, int window, int dtype, void* ws,
                  size_t ws_bytes, void* stream);

/*
 * Engine prefill over a KV cache (walkthrough, section "Pretraining", Engine paragraph).
 *   q       [B, Tq, H, D] bf16: prompt b's queries at positions 0..L_b-1 (read).
 *   kcache, vcache [B, Lcap, H, D] bf16: prompt b's keys/values already in rows 0..L_b-1 (read).
 *   lens    device int32 [B]: prompt lengths L_b; values are clamped to [0, min(Tq, Lcap)].
 *   o       [B, Tq, H, D] bf16: rows t < L_b written; rows t >= L_b left untouched.
 *   lse     [B, H, Tq] float32 or NULL; same rows written.
 *   window  keys visible to each query, counting itself (>= L_b: full causal).
 */
int attn_prefill(const void* q, const void* kcache, const void* vcache, const int* lens, void* o,
                 float* lse, int B, int H, int Tq, int Lcap, int D, int window, void* stream);

/*
 * Engine KV-cache append: kcache[b, pos[b], h, :] = knew[b, h, :] (same for v).
 *   knew, vnew [B, H, D] bf16 (read); pos device int32 [B]; rows with pos[b] outside [0, Lcap)
 *   are skipped (nothing is written for them).
 */
int attn_kv_append(void* kcache, void* vcache, const void* knew, const void* vnew, const int* pos,
                   int B, int H, int Lcap, int D, void* stream);

/* Bytes of device workspace attn_decode needs (split-K partial results, float32; only the
 * two-kernel schedule writes it, but every call checks its size). */
size_t attn_decode_workspace_bytes(int B, int H, int Lcap, int D);

/* Kernel launches that attn_decode and attn_decode_step make for these sizes: 1 (split-K inside a
 * workgroup per (sequence, head), merged in LDS) or 2 (split across workgroups into the workspace,
 * then a merge kernel).  Negative status for invalid sizes, as attn_decode. */
int attn_decode_launches(int B, int H, int Lcap, int D, int window);

/*
 * Engine decode: one new query per sequence attends to its cache (split-K over the cache length,
 * then a log-sum-exp merge of the partial results).  One launch, with the split inside a
 * workgroup per (sequence, head); two (split across workgroups, then a merge kernel) when fewer
 * than 128 (sequence, head) pairs each see more than 2048 rows (min(window, Lcap) > 2048).
 *   q      [B, H, D] bf16 (read); kcache, vcache [B, Lcap, H, D] bf16 (read).
 *   lens   device int32 [B]: cached tokens including the new one (append first, then decode);
 *          the query sits at position L_b - 1.  Values are clamped to [0, Lcap]; L_b = 0 gives
 *          o = 0 and lse = -inf.
 *   o      [B, H, D] bf16 (written);  lse [B, H] float32 or NULL.
 *   window keys visible to the query, counting itself.
 *   ws / ws_bytes: caller-owned device scratch of at least attn_decode_workspace_bytes().
 *   Lcap <= 65535 * 64 (the split schedule puts the 64-row chunk index on a grid dimension).
 */
int attn_decode(const void* q, const void* kcache, const void* vcache, const int* lens, void* o,
                float* lse, int B, int H, int Lcap, int D, int window, void* ws, size_t ws_bytes,
                void* stream);

/*
 * One Engine decode step, KV append and decode together: for each sequence b with
 * 0 <= pos[b] < Lcap, writes knew[b] / vnew[b] to cache row pos[b], then the query (at position
 * pos[b]) attends to rows max(0, pos[b] - window + 1) .. pos[b] of the updated cache.  The same
 * operation as attn_kv_append(pos) followed by attn_decode(lens = pos + 1), in one launch (two
 * when fewer than 128 (sequence, head) pairs each see more than 2048 rows, min(window, Lcap) >
 * 2048); no launch reads a cache row written in the same launch.  It makes
 * no host synchronisation and issues no memset, so a model's whole decode step (one call per
 * layer) can be captured in one HIP graph and replayed per generated token.
 * (Operation: walkthrough, section "Pretraining", Engine paragraph -- the decode phase over the
 * KV cache.)
 *   q, knew, vnew [B, H, D] bf16 (read); kcache, vcache [B, Lcap, H, D] bf16 (row pos[b] written).
 *   pos    device int32 [B]: cached tokens before this step.  A sequence with pos[b] outside
 *          [0, Lcap) is not written and gets o = 0, lse = -inf.
 *   o      [B, H, D] bf16 (written);  lse [B, H] float32 or NULL.
 *   window keys visible to the query, counting itself.
 *   ws / ws_bytes: caller-owned device scratch of at least attn_decode_workspace_bytes().
 * Errors as attn_decode.
 */
int attn_decode_step(const void* q, const void* knew, const void* vnew, void* kcache, void* vcache,
                     const int* pos, void* o, float* lse, int B, int H, int Lcap, int D,
                     int window, void* ws, size_t ws_bytes, void* stream);

/*
 * attn_decode_step without a workspace argument, for callers that cannot allocate device memory:
 * code being captured into a HIP graph, tight serving loops, harnesses that forbid hipMalloc.
 * Same operation, arguments (minus ws / ws_bytes), kernels and results as attn_decode_step; it
 * calls no hipMalloc / hipFree and allocates nothing.  The split schedule's partial results go
 * to a static device array of 32 MiB inside the library (one per GPU, kept until the process
 * ends; its address is looked up once per device, on the first call made with that device
 * current).  Sizes whose split schedule would need more than 32 MiB (attn_decode_workspace_bytes
 * above 32 MiB when attn_decode_launches returns 2) return SWATTN_EWORKSPACE; the one-launch
 * schedule needs no scratch at any size.  All calls on one GPU share that array: calls that may
 * run at the same time on one GPU (different streams, different host threads) race on it and
 * must be ordered by the caller.  Errors otherwise as attn_decode_step.
 */
int attn_decode_step_noalloc(const void* q, const void* knew, const void* vnew, void* kcache,
                             void* vcache, const int* pos, void* o, float* lse, int B, int H,
                             int Lcap, int D, int window, void* stream);

/*
 * Packed variable-length sequences (documents), for training and packed prefill.  A row of
 * training data holds several documents separated by the beginning-of-sequence token (walkthrough,
 * section "Midtraining": that token separates documents); here each document is one sequence and
 * attends only to itself:
 *   sequence s occupies rows cu_seqlens[s] .. cu_seqlens[s + 1] - 1 of q, k, v, o, dout, dq, dk,
 *   dv, each [total, H, D] bf16; query i of s sees key j of s iff 0 <= i - j < window (positions
 *   counted from the sequence's first row).  No key of another sequence is ever visible.
 *   lse    [H, total] float32 (natural log); optional (NULL) in the forward, read by the backward.
 *   cu_seqlens  device int32 [nseq + 1]: non-decreasing offsets, cu_seqlens[0] = 0 and
 *          cu_seqlens[nseq] = total.  Values are clamped to [0, total] on the device, so no value
 *          makes a kernel leave the buffers; an empty sequence is skipped.
 *   max_seqlen  host int >= the longest sequence (it sizes the launch; rows of a longer sequence
 *          past max_seqlen are not computed).  1 <= max_seqlen <= total.
 *   ws / ws_bytes (backward): at least attn_bwd_workspace_bytes(1, H, total, D).
 * bf16 only.  Each sequence gives, bit for bit, what attn_fwd / attn_bwd give for it alone
 * (B = 1, T = its length).  Errors as attn_fwd / attn_bwd.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens, int nseq, int total, int max_seqlen, int H, int D,
                    int window, void* stream);
int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, const int* cu_seqlens,
                    int nseq, int total, int max_seqlen, int H, int D, int window, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * QK-norm: attention over parameter-free RMS-normalised queries and keys (the model's RMS norms
 * carry no trainable parameters: walkthrough, section "Pretraining", the paragraph on the
 * optimisers).  Per row (one token of one head): r = 1 / sqrt(mean_d x_d^2 + eps), x_hat = x r.
 *   attn_fwd_qknorm: writes qn = bf16(q r_q), kn = bf16(k r_k) ([B, T, H, D]) and rq, rk (r per
 *     row, float32 [B, H, T]), then runs attn_fwd on (qn, kn, v): o, lse as attn_fwd.
 *     eps >= 0 and finite.  Two launches: the normalisation of k, then the attention, which
 *     normalises q in its prologue (same arithmetic, same order: rq, qn as the pass on k gives
 *     rk, kn for an equal row).
 *   attn_bwd_qknorm: the backward of the whole map (q, k, v) -> o, given the forward's qn, kn, rq,
 *     rk, o, lse: dq, dk are gradients with respect to the raw q and k (the norm's backward,
 *     dx = r (dx_hat - x_hat (dx_hat . x_hat) / D), runs inside the passes' epilogues), dv as
 *     attn_bwd.  Workspace as attn_bwd.
 * bf16 only; errors as attn_fwd / attn_bwd.
 */
int attn_fwd_qknorm(const void* q, const void* k, const void* v, void* qn, void* kn, float* rq,
                    float* rk, void* o, float* lse, int B, int H, int T, int D, int window,
                    float eps, void* stream);
int attn_bwd_qknorm(const void* qn, const void* kn, const void* v, const void* o, const float* lse,
                    const void* dout, const float* rq, const float* rk, void* dq, void* dk,
                    void* dv, int B, int H, int T, int D, int window, void* ws, size_t ws_bytes,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWATTN_H */
