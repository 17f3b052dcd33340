// Forward attention (training forward and Engine prefill) for gfx950.
//
// Operation: exact softmax causal attention with a per-layer sliding window -- the attention
// kernel with a window_size keyword credited in the "nanochat: GPT-2-grade LLM for <<$100" post
// (web3.cnoyu.life, "Jan29" entry), list of the largest improvements, item 1; the same kernel
// serves the Engine's prefill phase (followin.io walkthrough, section "Pretraining", Engine
// paragraph).  Query i sees key j iff j <= i and i - j < w; scale 1/sqrt(D).
//
// Design (bf16): one workgroup = NW waves x 32 queries of one (batch, head), two workgroups per CU.
// Each wave keeps its queries' Q in registers as MFMA B fragments and computes S^T = K Q^T per
// 64-key tile, so a lane owns one query column: the row max / row sum of the online softmax are
// lane-local plus one v_permlane32_swap.  O^T = V^T P^T reuses the S^T accumulators directly as the
// B operand (P split into bf16 hi + lo, two MFMAs on one V fragment); the V^T fragments come from
// the row-major V tile through ds_read_b64_tr_b16.  K/V tiles stream global -> LDS with
// buffer_load ... lds into a two-stage ring, one tile ahead of the compute (one barrier per tile).
// Tiles outside [q0 - w + 1, q_end] are never loaded; per wave, tiles wholly outside the window
// are skipped, and only tiles crossing the diagonal or the window edge run the masked loop.  O is
// rescaled lazily, only when a row maximum grows by more than 2^8.  Under the full causal mask
// (training) a workgroup owns a pair of query tiles of equal total work (pair_job).  VARLEN:
// packed documents (walkthrough, section "Midtraining"), each attending only to itself; a
// workgroup reads its document's offset and length from cu and runs the same job on that slice.
// QNORM: the QK-norm forward (the model's parameter-free RMS norm on q and k: walkthrough,
// section "Pretraining", the paragraph on the optimisers); q arrives raw and each lane
// normalises its half of a query row in the prologue, writing the bf16 row and 1 / rms out at
// the job's end.
#include <atomic>

#include "common.h"
#include "launch.h"

namespace swattn {

constexpr int kFwdBC = 64;  // keys per tile
#ifndef FWD_NW
#define FWD_NW 4  // waves (x 32 queries) per workgroup
#endif
#ifndef FWD_NS
#define FWD_NS 2  // K/V ring stages
#endif

// Streams one 64-key tile of K and of V into LDS (row-major, swizzled) by DMA.
template <int D, int NW>
__device__ __forceinline__ void fwd_issue_tile(const RowDma<D, NW, kFwdBC>& dma,
                                               const uint16_t* kb, const uint16_t* vb, int rs,
                                               int kt, int L, uint16_t* sK, uint16_t* sV,
                                               int wave, int lane) {
  const int64_t row0 = (int64_t)kt * kFwdBC * rs;
  const int nvalid = L - kt * kFwdBC;
  dma.issue(kb + row0, nvalid, sK, wave, lane);
  dma.issue(vb + row0, nvalid, sV, wave, lane);
}

// Per-wave state of the forward that lives across key tiles.
template <int D>
struct FwdState {
  f32x16 oacc[D / 32];
  float m_use, l_run;
};

// Softmax bookkeeping of one key tile held in two 32-key S^T accumulator blocks: mask (boundary
// tiles only), row max over the whole tile, and the lazy rescale of O -- all before any of the
// tile's probabilities reach O.
template <int D, bool MASK>
__device__ __forceinline__ void fwd_tile_max(f32x16& s0, f32x16& s1, int k_lo, int qi, int w,
                                             int half, float sl2, FwdState<D>& S) {
  constexpr int MB = D / 32;
  constexpr float kRescale = 8.f;  // lazy rescaling threshold (log2 units)
  float mraw = -INFINITY;
  // key j is visible to query i iff 0 <= i - j < w, i.e. (unsigned)(i - j) < w
  const int d0 = qi - k_lo - 4 * half;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (MASK) {
      const int off = 8 * (r >> 2) + (r & 3);
      s0[r] = (unsigned)(d0 - off) < (unsigned)w ? s0[r] : -INFINITY;
      s1[r] = (unsigned)(d0 - 32 - off) < (unsigned)w ? s1[r] : -INFINITY;
    }
    // med3(a, b, largest float) = max(a, b) as one instruction whose result the compiler knows to be
    // canonical, so the fmaxf chain below needs no canonicalising moves of the MFMA outputs
    mraw = fmaxf(mraw, __builtin_amdgcn_fmed3f(s0[r], s1[r], 3.4028235e38f));
  }
  const float m_tile = max_with_partner(mraw) * sl2;
  // rescale O only when some row max has grown past the threshold (exact either way)
  if (__builtin_amdgcn_ballot_w64(m_tile > S.m_use + kRescale) != 0) {
    const float m_new = fmaxf(S.m_use, m_tile);
    // a row with no visible key yet keeps m = -inf (and O = 0, l = 0): avoid exp2(-inf + inf)
    const float alpha = (m_new == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(S.m_use - m_new);
    S.l_run *= alpha;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) S.oacc[m][r] *= alpha;
    S.m_use = m_new;
  }
}

template <int D>
__device__ __forceinline__ void fwd_block_exp(f32x16& s, float sl2, FwdState<D>& S, uint4 (&ph)[2],
                                              uint4 (&pl)[2]) {
  const float m_eff = (S.m_use == -INFINITY) ? 0.f : S.m_use;
  float lsum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float e = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -m_eff));
    s[r] = e;
    lsum += e;
  }
  S.l_run += lsum;
  // P as bf16 hi + lo: the output is stored in bf16, whose rounding alone costs up to half an
  // ulp, so P must not add 2^-9 relative on top
  pack_frag_split(s, 0, ph[0], pl[0]);
  pack_frag_split(s, 1, ph[1], pl[1]);
}

// O^T += V^T P^T for one 32-key block: the hi MFMAs of all D / 32 accumulators, then the lo
// ones, so that no two consecutive MFMAs update the same accumulator (each keeps its hi-then-lo
// order; 0.5-2.5% off the forward and the prefill, bit-identical).
template <int D>
__device__ __forceinline__ void fwd_block_pv(const uint16_t* sV, const LdsOffsets<D>& lo, int nb,
                                             const uint4 (&ph)[2], const uint4 (&pl)[2],
                                             FwdState<D>& S) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    uint4 a[D / 32];
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
      a[m] = tr_frag_o<D>(sV, lo, nb * 32 + 16 * u, m);
      S.oacc[m] = mfma32(a[m], ph[u], S.oacc[m]);
    }
#pragma unroll
    for (int m = 0; m < D / 32; ++m) S.oacc[m] = mfma32(a[m], pl[u], S.oacc[m]);
  }
}

// S^T of one key tile (two 32-key blocks) and its softmax bookkeeping.  Only this part differs
// between boundary and interior tiles.
template <int D, bool MASK>
__device__ __forceinline__ void fwd_tile_s(const uint16_t* __restrict__ sK, int k_lo, int qi,
                                           int w, float sl2, const uint4 (&qf)[D / 16],
                                           const LdsOffsets<D>& lo, FwdState<D>& S, f32x16& s0,
                                           f32x16& s1, int lane) {
  constexpr int DK = D / 16;
  s0 = zero16();
  s1 = zero16();
#pragma unroll
  for (int t = 0; t < DK; ++t) {
    s0 = mfma32(rc_frag<D>(sK, lo, 0, t), qf[t], s0);
    s1 = mfma32(rc_frag<D>(sK, lo, 1, t), qf[t], s1);
  }
  sched_mfma_chain<2 * DK, 1, 8>();
  fwd_tile_max<D, MASK>(s0, s1, k_lo, qi, w, lane >> 5, sl2, S);
}

// Probabilities and O update of one key tile, shared by boundary and interior tiles (one copy of
// the code keeps O in the same registers on both paths): block 0's PV MFMAs run under block 1's
// exponentials (interleave pinned with sched_group_barrier) before block 1's PV.
template <int D>
__device__ __forceinline__ void fwd_tile_pv(const uint16_t* __restrict__ sV, float sl2,
                                            const LdsOffsets<D>& lo, FwdState<D>& S, f32x16& s0,
                                            f32x16& s1) {
  uint4 ph0[2], pl0[2], ph1[2], pl1[2];
  fwd_block_exp<D>(s0, sl2, S, ph0, pl0);
  // { PV of block 0 } || { exponentials and packing of block 1 }
  fwd_block_pv<D>(sV, lo, 0, ph0, pl0, S);
  fwd_block_exp<D>(s1, sl2, S, ph1, pl1);
#pragma unroll
  for (int t = 0; t < 2 * D / 32; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read (transposed pair)
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA hi, lo
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // VALU
  }
  fwd_block_pv<D>(sV, lo, 1, ph1, pl1, S);
}

// One key tile: issue the DMA of the next tile into `nxt`, then consume `cur`.  Within one call the
// two stages are distinct buffers, which the __restrict__ qualifiers state; that lets the compiler
// see that the LDS reads of `cur` do not depend on the DMA writes to `nxt` still in flight.  MASK
// tiles may cross the diagonal or the window edge for some wave; a wave skips a tile it cannot see.
template <int D, int NW, bool MASK>
__device__ __forceinline__ void fwd_step(const uint16_t* __restrict__ cur,
                                         uint16_t* __restrict__ nxt, bool issue_next, int kt_next,
                                         const uint16_t* kb, const uint16_t* vb, int rs, int L,
                                         int kt, int qa, int qi, int w, float sl2,
                                         const uint4 (&qf)[D / 16], const LdsOffsets<D>& lo,
                                         const RowDma<D, NW, kFwdBC>& dma, FwdState<D>& S,
                                         int wave, int lane) {
  constexpr int BC = kFwdBC, TILE = BC * D;
  static_assert(BC == 64, "two 32-key blocks per tile");
  if (issue_next)
    fwd_issue_tile<D, NW>(dma, kb, vb, rs, kt_next, L, nxt, nxt + TILE, wave, lane);
  const int k_lo = kt * BC;
  if (MASK) {
    const int k_hi = k_lo + BC - 1, qz = qa + 31;
    if ((qa >= L) || (k_lo > qz) || (qa - k_hi >= w)) return;
  } else {
    if (qa >= L) return;
  }
  f32x16 s0, s1;
  fwd_tile_s<D, MASK>(cur, k_lo, qi, w, sl2, qf, lo, S, s0, s1, lane);
  fwd_tile_pv<D>(cur + TILE, sl2, lo, S, s0, s1);
}

// One key tile through the NS-stage ring: wait for tile kt (stage st), refill the stage freed one
// tile ago with tile kt + NS - 1, consume tile kt.
template <int D, int NW, int NS, bool MASK>
__device__ __forceinline__ void fwd_ring_tile(int kt, int kt_end, int st, uint16_t* smem,
                                              const uint16_t* kb, const uint16_t* vb, int rs,
                                              int L, int qa, int qi, int w, float sl2,
                                              const uint4 (&qf)[D / 16], const LdsOffsets<D>& lo,
                                              const RowDma<D, NW, kFwdBC>& dma, FwdState<D>& S,
                                              int wave, int lane) {
  constexpr int TILE = kFwdBC * D;
  constexpr int LOADS = 2 * (kFwdBC * D / 512) / NW;  // DMA instructions per wave per tile
  // tile kt has landed once at most the younger tiles' DMA (up to NS - 2 of them) is in flight
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  const int younger = min(NS - 2, kt_end - kt);
  if constexpr (NS == 4) {
    if (younger >= 2) wait_vmcnt<2 * LOADS>();
    else if (younger >= 1) wait_vmcnt<LOADS>();
    else wait_vmcnt<0>();
  } else if constexpr (NS == 3) {
    if (younger >= 1) wait_vmcnt<LOADS>();
    else wait_vmcnt<0>();
  } else {
    wait_vmcnt<0>();
  }
  lds_barrier();  // ... for every wave (no drain of younger DMA); every wave is done with the
                  // stage refilled next
  const int nx = (st + NS - 1) % NS;
  fwd_step<D, NW, MASK>(smem + st * 2 * TILE, smem + nx * 2 * TILE, kt + NS - 1 <= kt_end,
                        kt + NS - 1, kb, vb, rs, L, kt, qa, qi, w, sl2, qf, lo, dma, S, wave, lane);
}

// Key tiles kt0 .. kt1 - 1 through the NS-stage ring (stage `st` holds tile kt0 on entry).  With
// two stages the loop takes two tiles per trip, so that each stage's LDS base is a compile-time
// constant and every operand read is the lane's offset plus an immediate.
template <int D, int NW, int NS, bool MASK>
__device__ __forceinline__ void fwd_run(int kt0, int kt1, int kt_end, int& st, uint16_t* smem,
                                        const uint16_t* kb, const uint16_t* vb, int rs, int L,
                                        int qa, int qi, int w, float sl2,
                                        const uint4 (&qf)[D / 16], const LdsOffsets<D>& lo,
                                        const RowDma<D, NW, kFwdBC>& dma, FwdState<D>& S,
                                        int wave, int lane) {
  int kt = kt0;
  if constexpr (NS == 2) {
    if (st == 1 && kt < kt1) {
      fwd_ring_tile<D, NW, NS, MASK>(kt, kt_end, 1, smem, kb, vb, rs, L, qa, qi, w, sl2, qf, lo,
                                     dma, S, wave, lane);
      ++kt;
      st = 0;
    }
    for (; kt + 1 < kt1; kt += 2) {
      fwd_ring_tile<D, NW, NS, MASK>(kt, kt_end, 0, smem, kb, vb, rs, L, qa, qi, w, sl2, qf, lo,
                                     dma, S, wave, lane);
      fwd_ring_tile<D, NW, NS, MASK>(kt + 1, kt_end, 1, smem, kb, vb, rs, L, qa, qi, w, sl2, qf,
                                     lo, dma, S, wave, lane);
    }
    if (kt < kt1) {
      fwd_ring_tile<D, NW, NS, MASK>(kt, kt_end, 0, smem, kb, vb, rs, L, qa, qi, w, sl2, qf, lo,
                                     dma, S, wave, lane);
      st = 1;
    }
  } else {
    for (; kt < kt1; ++kt) {
      fwd_ring_tile<D, NW, NS, MASK>(kt, kt_end, st, smem, kb, vb, rs, L, qa, qi, w, sl2, qf, lo,
                                     dma, S, wave, lane);
      st = (st + 1) % NS;
    }
  }
}

// QK-norm: RMS-normalises the lane's query row in registers and returns r = 1 / sqrt(mean x^2 +
// eps).  The lane holds the row's 8-column chunks 2 t + half (t < D / 16), its partner lane
// (lane ^ 32) the others.  The sum of squares runs per chunk, then over chunk pairs (c, c ^ 1),
// (c, c ^ 2), ...: the order of the normalisation pass (norm.hip), so that r and the bf16 row come
// out bit for bit as that pass gives them.
template <int D>
__device__ __forceinline__ float qnorm_regs(uint4 (&qf)[D / 16], float eps) {
  constexpr int DK = D / 16;
  float x[DK][8], v[DK];
#pragma unroll
  for (int t = 0; t < DK; ++t) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&qf[t]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[t][2 * e] = bf16_lo(w[e]);
      x[t][2 * e + 1] = bf16_hi(w[e]);
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[t][e], x[t][e], ss);
    v[t] = ss + __shfl_xor(ss, 32);  // chunks 2 t and 2 t + 1
  }
#pragma unroll
  for (int off = 1; off < DK; off <<= 1)
#pragma unroll
    for (int t = 0; t < DK; t += 2 * off) v[t] = v[t] + v[t + off];
  const float r = 1.f / sqrtf(v[0] / (float)D + eps);
#pragma unroll
  for (int t = 0; t < DK; ++t) {
    qf[t].x = pack_bf16x2(x[t][0] * r, x[t][1] * r);
    qf[t].y = pack_bf16x2(x[t][2] * r, x[t][3] * r);
    qf[t].z = pack_bf16x2(x[t][4] * r, x[t][5] * r);
    qf[t].w = pack_bf16x2(x[t][6] * r, x[t][7] * r);
  }
  return r;
}

// One job: query tile qt (NW waves x 32 queries) of head bh, NS-stage K/V ring (prefetch NS - 1
// tiles ahead).  Returns with every wave past its last read of the ring.  QNORM: the QK-norm
// forward; q holds raw rows, normalised in the prologue and written to qn / rq at the end.
template <int D, int NW, int NS, bool VARLEN, bool QNORM>
__device__ __forceinline__ void fwd_job(const FwdArgs& p, int bh, int qt, uint16_t* smem,
                                        int wave, int lane) {
  constexpr int BR = 32 * NW;
  constexpr int BC = kFwdBC;
  constexpr int DK = D / 16;  // MFMA k-steps over D
  constexpr int MB = D / 32;  // 32-row blocks of O^T
  constexpr int TILE = BC * D;
  const int half = lane >> 5, l32 = lane & 31;
  const int b = bh / p.H, h = bh % p.H;

  int L = p.kv_len;
  int64_t q_row0 = (int64_t)b * p.q_bstride, kv_row0 = (int64_t)b * p.kv_bstride;
  int64_t lse0 = (int64_t)bh * p.lse_T;
  if constexpr (VARLEN) {  // packed sequences; offsets clamped so any cu stays inside the buffers
    const int off = min(max(p.cu[b], 0), p.total);
    L = min(min(max(p.cu[b + 1], off), p.total) - off, p.kv_len);
    q_row0 = kv_row0 = (int64_t)off * p.row_stride;
    lse0 = (int64_t)h * p.total + off;
  } else if (p.lens) {
    L = min(max(p.lens[b], 0), p.kv_len);
  }
  const int q0 = qt * BR;
  if (q0 >= L) return;
  const int w = min(p.window, L);
  const int kstart = max(0, q0 - w + 1);
  const int qend = min(q0 + BR, L);
  const int kt_begin = kstart / BC, kt_end = (qend - 1) / BC;

  const uint16_t* qb = p.q + q_row0 + h * D;
  const uint16_t* kb = p.k + kv_row0 + h * D;
  const uint16_t* vb = p.v + kv_row0 + h * D;
  const int rs = p.row_stride;

  const int qa = q0 + 32 * wave;  // this wave's first query
  const int qi = qa + l32;        // this lane's query
  const bool qvalid = qi < L;

  uint4 qf[DK];  // rows past L load row L - 1 (in bounds) and are zeroed
  const int64_t qoff = (int64_t)min(qi, L - 1) * rs + 8 * half;
#pragma unroll
  for (int t = 0; t < DK; ++t) qf[t] = ldg16(qb + qoff + 16 * t);
  if (!QNORM && !qvalid)  // QK-norm: after the normalisation, below
#pragma unroll
    for (int t = 0; t < DK; ++t) qf[t] = make_uint4(0, 0, 0, 0);

  FwdState<D> S;
#pragma unroll
  for (int m = 0; m < MB; ++m) S.oacc[m] = zero16();
  S.m_use = -INFINITY;
  S.l_run = 0.f;

  const LdsOffsets<D> lo(lane);
  const RowDma<D, NW, BC> dma(rs, wave, lane);
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (kt_begin + i <= kt_end)
      fwd_issue_tile<D, NW>(dma, kb, vb, rs, kt_begin + i, L, smem + i * 2 * TILE,
                            smem + i * 2 * TILE + TILE, wave, lane);
  float qr = 0.f;
  if constexpr (QNORM) {  // under the first tiles' DMA
    qr = qnorm_regs<D>(qf, p.eps);
    if (!qvalid)
#pragma unroll
      for (int t = 0; t < DK; ++t) qf[t] = make_uint4(0, 0, 0, 0);
  }
  // Tiles that every wave of the workgroup sees whole (k_hi <= q0 and q0 + BR - 1 - k_lo < w) run
  // without the mask; the window-edge tiles before them and the diagonal tiles after them run with
  // it.  Three loops rather than a per-tile branch keep O in one set of registers.
  const int xw = q0 + BR - 1 - w;
  const int in_lo = max(kt_begin, xw < 0 ? 0 : xw / BC + 1);
  const int in_hi = min(kt_end + 1, (q0 + 1) / BC);  // exclusive
  int st = 0;  // stage of the next tile
  if (in_lo < in_hi) {
    fwd_run<D, NW, NS, true>(kt_begin, in_lo, kt_end, st, smem, kb, vb, rs, L, qa, qi, w,
                             p.scale_log2, qf, lo, dma, S, wave, lane);
    fwd_run<D, NW, NS, false>(in_lo, in_hi, kt_end, st, smem, kb, vb, rs, L, qa, qi, w,
                              p.scale_log2, qf, lo, dma, S, wave, lane);
    fwd_run<D, NW, NS, true>(in_hi, kt_end + 1, kt_end, st, smem, kb, vb, rs, L, qa, qi, w,
                             p.scale_log2, qf, lo, dma, S, wave, lane);
  } else {
    fwd_run<D, NW, NS, true>(kt_begin, kt_end + 1, kt_end, st, smem, kb, vb, rs, L, qa, qi, w,
                             p.scale_log2, qf, lo, dma, S, wave, lane);
  }

  const float l_tot = sum_with_partner(S.l_run);
  if (!qvalid) return;
  const float inv = 1.f / l_tot;
  uint16_t* ob = p.o + q_row0 + h * D + (int64_t)qi * rs;
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint2 st;
      st.x = pack_bf16x2(S.oacc[m][4 * j + 0] * inv, S.oacc[m][4 * j + 1] * inv);
      st.y = pack_bf16x2(S.oacc[m][4 * j + 2] * inv, S.oacc[m][4 * j + 3] * inv);
      *reinterpret_cast<uint2*>(ob + m * 32 + 8 * j + 4 * half) = st;
    }
  if (p.lse && half == 0) p.lse[lse0 + qi] = (S.m_use + __log2f(l_tot)) * kLn2;
  if constexpr (QNORM) {  // the normalised row, as the MFMAs used it, and its r
    uint16_t* qnb = p.qn + q_row0 + h * D + (int64_t)qi * rs + 8 * half;
#pragma unroll
    for (int t = 0; t < DK; ++t) *reinterpret_cast<uint4*>(qnb + 16 * t) = qf[t];
    if (half == 0) p.rq[(int64_t)bh * p.T + qi] = qr;
  }
}

// PAIRED (full-causal training forward): workgroup = head + query-tile pair (j, n - 1 - j), the
// short tile first, so that a head's workgroups start on the same K/V tiles together (pair_job).
// Otherwise (prefill, sliding window): workgroup = one query tile, longest tiles first.
template <int D, int NW, int NS, bool PAIRED, bool VARLEN, bool QNORM>
__global__ __launch_bounds__(64 * NW, (NW >= 8 ? 1 : 2)) void fwd_bf16_kernel(FwdArgs p) {
  static_assert((kFwdBC * D / 512) % NW == 0, "every wave issues the same number of DMA loads");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * 2 * kFwdBC * D];  // [stage][K|V]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = blockIdx.x;
  if (PAIRED) {
    const PairJob jb = pair_job(bid, p.BH, (p.n_qtiles + 1) / 2);
    const int qt1 = p.n_qtiles - 1 - jb.j;
    const int njobs = qt1 != jb.j ? 2 : 1;
#pragma unroll 1
    for (int jx = 0; jx < njobs; ++jx) {  // one copy of the job's code for both tiles
      if (jx) __syncthreads();  // every wave is done with the ring before the next job refills it
      fwd_job<D, NW, NS, false, QNORM>(p, jb.bh, jx ? qt1 : jb.j, smem, wave, lane);
    }
  } else {
    fwd_job<D, NW, NS, VARLEN, QNORM>(p, bid % p.BH, p.n_qtiles - 1 - bid / p.BH, smem, wave,
                                      lane);
  }
}

// ---------------------------------------------------------------------------------------------
// fp32 forward (fp32 in, fp32 out, fp32 MFMA v_mfma_f32_32x32x2f32).  Each MFMA k-step carries one
// value per lane half, so V is read row-major straight from LDS and P^T feeds the PV product one
// accumulator slot at a time without rounding.  One workgroup owns 32 queries of one head; its
// four waves take the query tile's 32-key tiles in turn (tile kt_begin + wave + 4 i), each with
// its own LDS area, loads for its next tile in flight under the current one and its own online
// softmax, and merge their (max, sum, O) through LDS at the end.  Small problems (the fp32 case
// is used at sizes like T = 128) so spread a query tile's keys over four waves instead of
// walking them in one.
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdArgs p) {
  constexpr int NW = 4, BC = 32, MB = D / 32;
  constexpr int SK = D + 1;                      // padded K row stride (floats) against bank conflicts
  constexpr int WAREA = BC * SK + BC * D;        // one wave's K and V tiles (floats)
  constexpr int LPW = BC * D / 4 / 64;           // float4 loads per lane per tile and tensor
  static_assert(MB * 16 * 64 + 128 <= WAREA, "the merge data fits a wave's tile area");
  __shared__ __attribute__((aligned(16))) float smem[NW * WAREA];

  const float* qg = reinterpret_cast<const float*>(p.q);
  const float* kg = reinterpret_cast<const float*>(p.k);
  const float* vg = reinterpret_cast<const float*>(p.v);
  float* og = reinterpret_cast<float*>(p.o);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int bid = blockIdx.x;
  const int qt = p.n_qtiles - 1 - bid / p.BH;
  const int bh = bid % p.BH;
  const int b = bh / p.H, h = bh % p.H;
  int L = p.kv_len;
  if (p.lens) L = min(max(p.lens[b], 0), p.kv_len);
  const int q0 = qt * 32;
  if (q0 >= L) return;
  const int w = min(p.window, L);
  const int kstart = max(0, q0 - w + 1);
  const int qend = min(q0 + 32, L);
  const int kt_begin = kstart / BC, kt_end = (qend - 1) / BC;
  const float* qb = qg + (int64_t)b * p.q_bstride + h * D;
  const float* kb = kg + (int64_t)b * p.kv_bstride + h * D;
  const float* vb = vg + (int64_t)b * p.kv_bstride + h * D;
  const int rs = p.row_stride;
  const int qi = q0 + l32;
  const bool qvalid = qi < L;
  float* sK = smem + wave * WAREA;
  float* sV = sK + BC * SK;

  float qf[D / 2];
#pragma unroll
  for (int t = 0; t < D / 2; ++t) qf[t] = qvalid ? qb[(int64_t)qi * rs + 2 * t + half] : 0.f;
  f32x16 oacc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) oacc[m] = zero16();
  float m_run = -INFINITY, l_run = 0.f;

  // this wave's tiles; rows past L load as zero (and are masked: they lie past every valid query)
  float4 kr[LPW], vr[LPW];
  auto load = [&](int kt) {
#pragma unroll
    for (int it = 0; it < LPW; ++it) {
      const int idx = lane + 64 * it;
      const int r = idx / (D / 4), c4 = idx % (D / 4);
      const int j = kt * BC + r;
      kr[it] = vr[it] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < L) {
        kr[it] = *reinterpret_cast<const float4*>(kb + (int64_t)j * rs + 4 * c4);
        vr[it] = *reinterpret_cast<const float4*>(vb + (int64_t)j * rs + 4 * c4);
      }
    }
  };
  int kt = kt_begin + wave;
  if (kt <= kt_end) load(kt);
  for (; kt <= kt_end; kt += NW) {
    // this wave's previous tile is fully read before its area is rewritten
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int it = 0; it < LPW; ++it) {
      const int idx = lane + 64 * it;
      const int r = idx / (D / 4), c4 = idx % (D / 4);
      float* dk = sK + r * SK + 4 * c4;  // padded rows: four scalar stores
      dk[0] = kr[it].x;
      dk[1] = kr[it].y;
      dk[2] = kr[it].z;
      dk[3] = kr[it].w;
      *reinterpret_cast<float4*>(sV + r * D + 4 * c4) = vr[it];
    }
    if (kt + NW <= kt_end) load(kt + NW);  // next tile's loads in flight under this one
    // the tile's stores land before any lane of the wave reads them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int k_lo = kt * BC;

    f32x16 s = zero16();
#pragma unroll
    for (int t = 0; t < D / 2; ++t) s = mfma32_f32(sK[l32 * SK + 2 * t + half], qf[t], s);
    float mloc = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k_lo + 8 * (r >> 2) + 4 * half + (r & 3);
      float x = s[r] * p.scale_log2;
      if (key > qi || qi - key >= w) x = -INFINITY;
      s[r] = x;
      mloc = fmaxf(mloc, x);
    }
    const float m_new = fmaxf(m_run, max_with_partner(mloc));
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = exp2f(s[r] - m_use);
      lsum += s[r];
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[m][r] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * half + (r & 3);
        oacc[m] = mfma32_f32(sV[key * D + m * 32 + l32], s[r], oacc[m]);
      }
    }
  }

  // merge: every wave leaves (max, sum, O) in its own area; wave 0 combines them.  A wave with no
  // tile leaves max = -inf, sum = 0, O = 0, which the merge weighs by 0.
  const float l_w = sum_with_partner(l_run);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  float* mo = sK;
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) mo[(m * 16 + r) * 64 + lane] = oacc[m][r];
  mo[MB * 16 * 64 + lane] = m_run;
  mo[MB * 16 * 64 + 64 + lane] = l_w;
  __syncthreads();
  if (wave != 0 || !qvalid) return;
  float mw[NW], mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    mw[v] = smem[v * WAREA + MB * 16 * 64 + lane];
    mx = fmaxf(mx, mw[v]);
  }
  float wt[NW], l_tot = 0.f;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    wt[v] = (mw[v] == -INFINITY) ? 0.f : exp2f(mw[v] - mx);
    l_tot += wt[v] * smem[v * WAREA + MB * 16 * 64 + 64 + lane];
  }
  const float inv = 1.f / l_tot;
  float* ob = og + (int64_t)b * p.q_bstride + h * D + (int64_t)qi * rs;
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float o4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int v = 0; v < NW; ++v) acc += wt[v] * smem[v * WAREA + (m * 16 + 4 * j + i) * 64 + lane];
        o4[i] = acc * inv;
      }
      *reinterpret_cast<float4*>(ob + m * 32 + 8 * j + 4 * half) =
          make_float4(o4[0], o4[1], o4[2], o4[3]);
    }
  if (p.lse && half == 0) p.lse[(int64_t)bh * p.lse_T + qi] = (mx + log2f(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------------------------
int device_compute_units() {
  static std::atomic<int> cache[64];  // per device, 0 until looked up
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
  if (dev < 64 && n > 0) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int D, int NW, int NS>
static hipError_t launch_bf16(const FwdArgs& a, hipStream_t s) {
  FwdArgs p = a;
  p.n_qtiles = (p.T + 32 * NW - 1) / (32 * NW);
  // tile pairs carry equal work only when every query sees all earlier keys
  const unsigned grid = (unsigned)p.n_qtiles * (unsigned)p.BH;
  const unsigned pairs = (unsigned)(p.n_qtiles + 1) / 2 * (unsigned)p.BH;
  const bool paired = p.cu == nullptr && p.lens == nullptr && p.window >= p.T &&
                      p.kv_len == p.T && pairs_fill_rounds(pairs, 2u * device_compute_units());
  const dim3 block(64 * NW);
  if (p.cu)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, NS, false, true, false>), dim3(grid), block, 0, s,
                       p);
  else if (p.qn && paired)  // QK-norm (dense training only)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, NS, true, false, true>), dim3(pairs), block, 0, s,
                       p);
  else if (p.qn)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, NS, false, false, true>), dim3(grid), block, 0, s,
                       p);
  else if (paired)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, NS, true, false, false>), dim3(pairs), block, 0, s,
                       p);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, NS, false, false, false>), dim3(grid), block, 0, s,
                       p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_f32(const FwdArgs& a, hipStream_t s) {
  FwdArgs p = a;
  p.n_qtiles = (p.T + 31) / 32;  // 32 queries per workgroup
  const unsigned grid = (unsigned)p.n_qtiles * (unsigned)p.BH;
  hipLaunchKernelGGL((fwd_f32_kernel<D>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Launches too small to give every CU a workgroup of FWD_NW waves (short sequences, few heads) take
// one wave per workgroup instead: four times the workgroups, each walking only its own 32 queries'
// key tiles.
hipError_t launch_fwd(const FwdArgs& a, bool f32, hipStream_t s) {
  if (f32) return a.D == 64 ? launch_f32<64>(a, s) : launch_f32<128>(a, s);
  const long long wide = (long long)((a.T + 32 * FWD_NW - 1) / (32 * FWD_NW)) * a.BH;
  if (wide < device_compute_units())
    return a.D == 64 ? launch_bf16<64, 1, FWD_NS>(a, s) : launch_bf16<128, 1, FWD_NS>(a, s);
  return a.D == 64 ? launch_bf16<64, FWD_NW, FWD_NS>(a, s) : launch_bf16<128, FWD_NW, FWD_NS>(a, s);
}

}  // namespace swattn
