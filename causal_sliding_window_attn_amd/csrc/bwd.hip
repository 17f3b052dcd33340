// Backward attention for gfx950, split into a dQ pass and a dK/dV pass that both recompute the
// probabilities from the forward's LSE (no atomics, one owner per output tile, deterministic).
//
// Operation: the gradient of the windowed causal attention of the "nanochat: GPT-2-grade LLM for
// <<$100" post (web3.cnoyu.life, "Jan29" entry), list of the largest improvements, item 1, used
// in training (followin.io walkthrough, section "Pretraining": forward/backward over 32 x 2048
// tokens per GPU).  With P_ij = exp(s_ij - LSE_i) and no gradient into LSE:
//   Delta_i = dO_i . O_i,  dS_ij = P_ij (dO_i . v_j - Delta_i),
//   dQ_i = sum_j dS_ij k_j / sqrt(D),  dK_j = sum_i dS_ij q_i / sqrt(D),  dV_j = sum_i P_ij dO_i.
//
// dQ pass: a workgroup owns NW x 32 queries (Q, dO in registers as B fragments, lane = query as in
// the forward), computes Delta and LSE * log2(e) for them first and writes both to the workspace,
// then walks the in-window key tiles: S^T = K Q^T, dP^T = V dO^T, dS^T, and dQ^T += K^T dS^T.
// dK/dV pass: a workgroup owns 128 keys and walks the query tiles that can see them, last tile
// first; half of its waves compute S = Q K^T and P, the other half, one tile behind,
// dP = dO V^T, dS, dV^T += dO^T P and dK^T += Q^T dS, taking P through LDS (lane = key in both).
// Under the full causal mask both passes give each workgroup a pair of tiles of equal total work
// (pair_job).  Tiles stream global -> LDS by DMA (the dQ pass through buffer_load ... lds, the dK/dV
// pass through global_load_lds), one tile ahead with one barrier per tile: a two-stage K/V ring in
// the dQ pass, a three-stage Q/dO ring in the dK/dV pass (the dS waves still read the tile
// before).  Every transposed operand (K^T, Q^T, dO^T) comes straight from the row-major tile
// through ds_read_b64_tr_b16.  On dense launches the dK/dV pass runs on a persistent grid whose
// workgroups chain their jobs through one tile stream (bwd_dkdv_chain_kernel).
//
// Modes (template flags; the dense instantiation is unchanged by them):
//   VARLEN  packed documents (rows cu[s] .. cu[s+1] - 1 of [total, H, D], each attending only to
//           itself -- walkthrough, section "Midtraining": documents separated by the
//           beginning-of-sequence token): a workgroup reads its document's offset and length and
//           runs the dense job on that slice;
//   QKN     q and k are RMS-normalised rows (norm.hip); the epilogues take dQ and dK back through
//           the parameter-free norm before storing (store_through_rmsnorm).
#include "common.h"
#include "launch.h"

namespace swattn {

constexpr int kBwdBC = 64;  // keys per tile in the dQ pass
constexpr int kBwdBQ = 64;  // queries per tile in the dK/dV pass

// Rows of head h of sequence b: dense [B, T, H, D] (statistics [B, H, T]) or packed sequences
// ([total, H, D] rows cu[b] .. cu[b + 1] - 1, statistics [H, total]); packed offsets are clamped
// so that any cu stays inside the buffers.
struct BwdRows {
  int T;         // rows of the sequence
  int64_t base;  // element offset of its row 0 at head h
  int64_t stat;  // index of its row 0 in lse, Delta and LSE * log2(e)
};

// A row's MFMA fragments (the lane holds its 8-column chunks 2 t + half in f[t], the partner lane
// lane ^ 32 the others) rearranged into the accumulator's element order (columns 8 c + 4 half ..
// + 3 of every chunk c, as y[c / 4][c % 4]): per fragment, one v_permlane32_swap for each dword
// pair hands the partner the four columns it lacks and takes the four this lane lacks.
template <int D>
__device__ __forceinline__ void frag_to_acc_order(const uint4 (&f)[D / 16],
                                                  uint2 (&y)[D / 32][4]) {
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const auto a = __builtin_amdgcn_permlane32_swap(f[t].x, f[t].z, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(f[t].y, f[t].w, false, false);
    const int m = t / 2, j = 2 * (t % 2);
    y[m][j] = make_uint2(a[0], b[0]);      // chunk 2 t
    y[m][j + 1] = make_uint2(a[1], b[1]);  // chunk 2 t + 1
  }
}

// QK-norm backward, fused into a pass's epilogue.  With y = x / rms(x) the normalised row (the
// attention's input, in the accumulator's element order), g = acc * sc the gradient with respect
// to y and r = 1 / rms(x):  dx = r (g - y (g . y) / D).  A lane and its partner (lane ^ 32) hold
// the two halves of the row.
template <int D>
__device__ __forceinline__ void store_through_rmsnorm(const f32x16 (&acc)[D / 32], float sc,
                                                      const uint2 (&y)[D / 32][4], float r,
                                                      uint16_t* out, int half) {
  constexpr int MB = D / 32;
  float dot = 0.f;
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dot = fmaf(acc[m][4 * j + 0] * sc, bf16_lo(y[m][j].x), dot);
      dot = fmaf(acc[m][4 * j + 1] * sc, bf16_hi(y[m][j].x), dot);
      dot = fmaf(acc[m][4 * j + 2] * sc, bf16_lo(y[m][j].y), dot);
      dot = fmaf(acc[m][4 * j + 3] * sc, bf16_hi(y[m][j].y), dot);
    }
  const float c = sum_with_partner(dot) / (float)D;
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint2 st;
      st.x = pack_bf16x2(r * (acc[m][4 * j + 0] * sc - bf16_lo(y[m][j].x) * c),
                         r * (acc[m][4 * j + 1] * sc - bf16_hi(y[m][j].x) * c));
      st.y = pack_bf16x2(r * (acc[m][4 * j + 2] * sc - bf16_lo(y[m][j].y) * c),
                         r * (acc[m][4 * j + 3] * sc - bf16_hi(y[m][j].y) * c));
      *reinterpret_cast<uint2*>(out + m * 32 + 8 * j + 4 * half) = st;
    }
}

template <bool VARLEN>
__device__ __forceinline__ BwdRows bwd_rows(const BwdArgs& p, int b, int h, int D) {
  BwdRows r;
  if constexpr (VARLEN) {
    const int off = min(max(p.cu[b], 0), p.total);
    r.T = min(min(max(p.cu[b + 1], off), p.total) - off, p.T);
    r.base = (int64_t)off * p.row_stride + h * D;
    r.stat = (int64_t)h * p.total + off;
  } else {
    r.T = p.T;
    r.base = (int64_t)b * p.bstride + h * D;
    r.stat = (int64_t)(b * p.H + h) * p.T;
  }
  return r;
}

// ------------------------------------------------------------------------------------------ dQ
// dS^T = P^T (dP^T - Delta) for one 32-key block, in place in the S^T accumulator; `dp` already
// holds dP^T - Delta (its MFMA chain starts from -Delta).
template <bool MASK>
__device__ __forceinline__ void dq_ds(f32x16& s, const f32x16& dp, int d0, int w, float sl2,
                                      float lse2) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float pr = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -lse2));
    if (MASK) {
      // key j is visible to query i iff (unsigned)(i - j) < w
      const unsigned dist = (unsigned)(d0 - (8 * (r >> 2) + (r & 3)));
      pr = dist < (unsigned)w ? pr : 0.f;
    }
    s[r] = pr * dp[r];
  }
}

// One key tile.  Only the probabilities depend on `mask` (a wave-uniform branch around them), so
// the MFMA code and dQ's registers are the same for boundary and interior tiles.
template <int D>
__device__ __forceinline__ void dq_tile(const uint16_t* __restrict__ sK,
                                        const uint16_t* __restrict__ sV, bool mask, int k_lo,
                                        int qi, int w, float sl2, float lse2, const f32x16& ndelta,
                                        const uint4 (&qf)[D / 16], const uint4 (&df)[D / 16],
                                        const LdsOffsets<D>& lo, f32x16 (&dqacc)[D / 32],
                                        int lane) {
  constexpr int BC = kBwdBC, DK = D / 16, MB = D / 32, NB = BC / 32;
  const int half = lane >> 5;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    // the dP^T chain takes -Delta (the lane's query) as its first C operand: no subtraction later
    f32x16 s = zero16(), dp = ndelta;
#pragma unroll
    for (int t = 0; t < DK; ++t) {
      s = mfma32(rc_frag<D>(sK, lo, nb, t), qf[t], s);
      dp = mfma32(rc_frag<D>(sV, lo, nb, t), df[t], dp);
    }
    sched_mfma_chain<2 * DK, 1, 8>();
    const int d0 = qi - (k_lo + nb * 32) - 4 * half;
    if (mask)
      dq_ds<true>(s, dp, d0, w, sl2, lse2);
    else
      dq_ds<false>(s, dp, d0, w, sl2, lse2);
    const uint4 dsf[2] = {pack_frag(s, 0), pack_frag(s, 1)};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int m = 0; m < MB; ++m)
        dqacc[m] = mfma32(tr_frag_o<D>(sK, lo, nb * 32 + 16 * u, m), dsf[u], dqacc[m]);
    sched_mfma_chain<2 * MB, 2, 4>();
  }
}

// Streams key tile kt of K and of V into one ring stage.
template <int D, int NW>
__device__ __forceinline__ void dq_issue(const RowDma<D, NW, kBwdBC>& dma, const uint16_t* kb,
                                         const uint16_t* vb, int rs, int T, int kt,
                                         uint16_t* stage, int wave, int lane) {
  const int64_t row0 = (int64_t)kt * kBwdBC * rs;
  dma.issue(kb + row0, T - kt * kBwdBC, stage, wave, lane);
  dma.issue(vb + row0, T - kt * kBwdBC, stage + kBwdBC * D, wave, lane);
}

template <int D, int NW>
__device__ __forceinline__ void dq_step(const uint16_t* __restrict__ cur,
                                        uint16_t* __restrict__ nxt, bool issue_next,
                                        const RowDma<D, NW, kBwdBC>& dma, const uint16_t* kb,
                                        const uint16_t* vb, int rs, int T, int kt, int qa, int qi,
                                        int w, float sl2, float lse2, const f32x16& ndelta,
                                        const uint4 (&qf)[D / 16], const uint4 (&df)[D / 16],
                                        const LdsOffsets<D>& lo, f32x16 (&dqacc)[D / 32],
                                        int wave, int lane) {
  constexpr int BC = kBwdBC, TILE = BC * D;
  if (issue_next) dq_issue<D, NW>(dma, kb, vb, rs, T, kt + 1, nxt, wave, lane);
  const int k_lo = kt * BC, k_hi = k_lo + BC - 1, qz = qa + 31;
  if ((qa >= T) || (k_lo > qz) || (qa - k_hi >= w)) return;
  const bool mask = !(k_hi <= qa && qz - k_lo < w);
  dq_tile<D>(cur, cur + TILE, mask, k_lo, qi, w, sl2, lse2, ndelta, qf, df, lo, dqacc, lane);
}

// One job: query tile qt (NW waves x 32 queries) of head bh.  Returns with every wave past its
// last read of the two-stage ring.
template <int D, int NW, bool VARLEN, bool QKN>
__device__ __forceinline__ void dq_job(const BwdArgs& p, int bh, int qt, uint16_t* smem, int wave,
                                       int lane) {
  constexpr int BR = 32 * NW, BC = kBwdBC;
  constexpr int DK = D / 16, MB = D / 32, TILE = BC * D;
  const int half = lane >> 5, l32 = lane & 31;
  const int b = bh / p.H, h = bh % p.H;
  const BwdRows rw = bwd_rows<VARLEN>(p, b, h, D);
  const int T = rw.T;
  const int q0 = qt * BR;
  if (q0 >= T) return;
  const int w = min(p.window, T);
  const int kstart = max(0, q0 - w + 1);
  const int qend = min(q0 + BR, T);
  const int kt_begin = kstart / BC, kt_end = (qend - 1) / BC;

  const int64_t base = rw.base;
  const int rs = p.row_stride;
  const uint16_t* kb = p.k + base;
  const uint16_t* vb = p.v + base;

  const RowDma<D, NW, BC> dma(rs, wave, lane);
  dq_issue<D, NW>(dma, kb, vb, rs, T, kt_begin, smem, wave, lane);

  const int qa = q0 + 32 * wave;
  const int qi = qa + l32;
  const bool qvalid = qi < T;

  // rows past T load row T - 1 (in bounds) and are zeroed below
  uint4 qf[DK], df[DK], of[DK];
  const int qc = min(qi, T - 1);
  const int64_t roff = base + (int64_t)qc * rs + 8 * half;
#pragma unroll
  for (int t = 0; t < DK; ++t) {
    qf[t] = ldg16(p.q + roff + 16 * t);
    df[t] = ldg16(p.dout + roff + 16 * t);
    of[t] = ldg16(p.o + roff + 16 * t);
  }
  const float lse_raw = p.lse[rw.stat + qc];
  const float rq = QKN ? p.rq[rw.stat + qc] : 0.f;  // QK-norm: 1 / rms of the raw row
  float dsum = 0.f;
#pragma unroll
  for (int t = 0; t < DK; ++t) {
    const uint32_t* dw = reinterpret_cast<const uint32_t*>(&df[t]);
    const uint32_t* ow = reinterpret_cast<const uint32_t*>(&of[t]);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dsum += bf16_lo(dw[e]) * bf16_lo(ow[e]) + bf16_hi(dw[e]) * bf16_hi(ow[e]);
  }
  if (!qvalid) {
#pragma unroll
    for (int t = 0; t < DK; ++t) {
      qf[t] = make_uint4(0, 0, 0, 0);
      df[t] = make_uint4(0, 0, 0, 0);
    }
    dsum = 0.f;
  }
  const float delta = sum_with_partner(dsum);
  if (qvalid && half == 0) {
    p.delta[rw.stat + qi] = delta;
    p.lse2[rw.stat + qi] = lse_raw * kLog2e;  // the dK/dV pass reads LSE in base 2
  }
  const float lse2 = qvalid ? lse_raw * kLog2e : 0.f;
  f32x16 ndelta;
#pragma unroll
  for (int r = 0; r < 16; ++r) ndelta[r] = -delta;

  f32x16 dqacc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) dqacc[m] = zero16();

  const LdsOffsets<D> lo(lane);
  // two tiles per trip, so that each stage's LDS base is a compile-time constant and every
  // operand read is the lane's offset plus an immediate
  uint16_t* stage0 = smem;
  uint16_t* stage1 = smem + 2 * TILE;
  int kt = kt_begin;
  for (; kt < kt_end; kt += 2) {
    wait_vmcnt<0>();
    __syncthreads();
    dq_step<D, NW>(stage0, stage1, true, dma, kb, vb, rs, T, kt, qa, qi, w, p.scale_log2, lse2, ndelta,
                   qf, df, lo, dqacc, wave, lane);
    wait_vmcnt<0>();
    __syncthreads();
    dq_step<D, NW>(stage1, stage0, kt + 1 < kt_end, dma, kb, vb, rs, T, kt + 1, qa, qi, w,
                   p.scale_log2, lse2, ndelta, qf, df, lo, dqacc, wave, lane);
  }
  if (kt == kt_end) {
    wait_vmcnt<0>();
    __syncthreads();
    dq_step<D, NW>(stage0, stage1, false, dma, kb, vb, rs, T, kt, qa, qi, w, p.scale_log2, lse2, ndelta,
                   qf, df, lo, dqacc, wave, lane);
  }

  if (!qvalid) return;
  const float sc = p.scale;
  uint16_t* out = p.dq + base + (int64_t)qi * rs;
  if constexpr (QKN) {  // dq with respect to the raw rows; qf holds the normalised ones
    uint2 y[MB][4];
    frag_to_acc_order<D>(qf, y);
    store_through_rmsnorm<D>(dqacc, sc, y, rq, out, half);
    return;
  }
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint2 st;
      st.x = pack_bf16x2(dqacc[m][4 * j + 0] * sc, dqacc[m][4 * j + 1] * sc);
      st.y = pack_bf16x2(dqacc[m][4 * j + 2] * sc, dqacc[m][4 * j + 3] * sc);
      *reinterpret_cast<uint2*>(out + m * 32 + 8 * j + 4 * half) = st;
    }
}

// Packed sequences: the dK/dV pass's job plan (layout in launch.h) and its queue counter, set by
// workgroup 0 of the dQ pass before its own job.  Level kt lists the sequences with more than kt
// 128-key tiles, in sequence order: wave 0 walks the levels, 64 sequences per step, and a ballot
// gives each its place.  `nd` is LDS for one int per sequence.
template <int D>
__device__ void dkdv_build_plan(const BwdArgs& p, int* nd) {
  const int nseq = p.BH / p.H, levels = (p.T + 127) / 128;
  for (int d = threadIdx.x; d < nseq; d += blockDim.x)
    nd[d] = (bwd_rows<true>(p, d, 0, D).T + 127) / 128;
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int run = 0;
    // entries beyond the capacity (possible only when cu's ranges overlap, which the host's
    // bound does not foresee) are dropped, and the offsets clamped, so that no read or write of
    // the plan leaves it
    const int cap = kDkdvPlanMax - levels - 1;
    for (int kt = 0; kt < levels; ++kt) {
      if (lane == 0) p.plan[kt] = min(run, cap);
      for (int c0 = 0; c0 < nseq; c0 += 64) {
        const int d = c0 + lane;
        const bool in = d < nseq && nd[d] > kt;
        const uint64_t m = __ballot(in);
        const int pos = run + __popcll(m & ((1ull << lane) - 1));
        if (in && pos < cap) p.plan[levels + 1 + pos] = d;
        run += __popcll(m);
      }
    }
    if (lane == 0) {
      p.plan[levels] = min(run, cap);
      *p.qctr = 0u;
    }
  }
  __syncthreads();  // the caller reuses the LDS
}

// Full-causal training pass (p.paired): workgroup = head + query-tile pair (j, n - 1 - j), short
// tile first (pair_job).  Otherwise: workgroup = one query tile, longest tiles first.
template <int D, int NW, bool VARLEN, bool QKN>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dq_kernel(BwdArgs p) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * 2 * kBwdBC * D];  // [stage][K|V]
  const int tid = threadIdx.x;
  if (VARLEN && p.plan && blockIdx.x == 0)  // the dK/dV pass's job plan, before this job
    dkdv_build_plan<D>(p, reinterpret_cast<int*>(smem));
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = blockIdx.x;
  int bh, qt0, qt1, njobs;
  if (p.paired) {
    const PairJob jb = pair_job(bid, p.BH, (p.n_tiles + 1) / 2);
    bh = jb.bh;
    qt0 = jb.j;
    qt1 = p.n_tiles - 1 - jb.j;
    njobs = qt1 != qt0 ? 2 : 1;
  } else {
    bh = bid % p.BH;
    qt0 = qt1 = p.n_tiles - 1 - bid / p.BH;
    njobs = 1;
  }
#pragma unroll 1
  for (int jx = 0; jx < njobs; ++jx) {
    if (jx) __syncthreads();  // every wave is done with the ring before the next job refills it
    dq_job<D, NW, VARLEN, QKN>(p, bh, jx ? qt1 : qt0, smem, wave, lane);
  }
}

// ---------------------------------------------------------------------------------------- dK/dV
// Eight waves own 128 keys: waves 0-3 ("P waves") compute S = Q K^T and P for key block w;
// waves 4-7 ("dS waves") compute dP = dO V^T for the same key block and accumulate both
// dV^T += dO^T P and dK^T += Q^T dS.  The dS waves run one query tile behind: in iteration i the
// P waves handle tile i and leave its P (bf16, register order) in one of two LDS buffers, while the
// dS waves handle tile i - 1 with the P left there in iteration i - 1.  A three-stage Q/dO ring
// keeps tiles i + 1 (in flight), i and i - 1 resident, so one barrier per tile suffices.  The split
// of the work gives the P waves the exponentials and 8 MFMAs per 32-query block and the dS waves
// 24 MFMAs and little VALU work, so the two waves sharing a SIMD lean on different units (with
// dV on the P waves, 16 MFMAs each, the pass was 4-5% slower).
constexpr int kDkdvWaves = 8;
constexpr int kDkdvStages = 3;
// The P waves (0-3) alone issue the ring's DMA: the dS waves finish each tile last, and taking the
// DMA issue off them shortens every tile (1.6-3% of the pass, measured in one process)
constexpr int kDkdvDmaWaves = 4;

template <int D>
struct DkdvStage {
  static constexpr int TILE = kBwdBQ * D;
  static constexpr int ELEMS = 2 * TILE + 2 * kBwdBQ * 2;  // Q | dO | LSE | Delta, uint16 units
  static constexpr int PELEMS = 4 * kBwdBQ * 32;           // bf16 P of 4 key blocks x 64 queries
};

template <int D, int NW>
__device__ __forceinline__ void dkdv_issue(const RowDmaFlat<D, NW, kBwdBQ>& dma, const uint16_t* qb,
                                           const uint16_t* db, const float* lseb,
                                           const float* delb, int rs, int qt, int T,
                                           uint16_t* stage, int wave, int lane) {
  constexpr int BQ = kBwdBQ, TILE = DkdvStage<D>::TILE;
  if (wave >= NW) return;  // only waves 0 .. NW - 1 issue
  const int64_t row0 = (int64_t)qt * BQ * rs;
  dma.issue(qb + row0, T - qt * BQ, stage, wave, lane);
  dma.issue(db + row0, T - qt * BQ, stage + TILE, wave, lane);
  static_assert(BQ == 64, "one 4-byte DMA per lane covers the 64 rows' LSE / Delta");
  if (wave == NW - 1) {
    const int j = min(qt * BQ + lane, T - 1);
    float* sl = reinterpret_cast<float*>(stage + 2 * TILE);
    g2lds4(lseb + j, sl);
    g2lds4(delb + j, sl + BQ);
  }
}

// P = exp2(S * scale * log2(e) - LSE * log2(e)) for one 32-query block (lane = key kj,
// accumulator r = query row); sL holds the rows' LSE already in base 2.
template <bool MASK>
__device__ __forceinline__ void dkdv_probs(f32x16& acc, const float* sL, int qb2, int qt, int kj,
                                           int T, int w, float sl2, int half) {
  constexpr int BQ = kBwdBQ;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ql0 = 32 * qb2 + 8 * j + 4 * half;
    const float4 l4 = *reinterpret_cast<const float4*>(sL + ql0);
    const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * j + i;
      float pr = __builtin_amdgcn_exp2f(fmaf(acc[r], sl2, -lv[i]));
      if (MASK) {
        // query i sees key j iff (unsigned)(i - j) < w; rows past T hold a clamped copy: drop them
        const int qg = qt * BQ + ql0 + i;
        pr = (((unsigned)(qg - kj) < (unsigned)w) & (qg < T)) ? pr : 0.f;
      }
      acc[r] = pr;
    }
  }
}

__device__ __forceinline__ bool dkdv_block_live(int qt, int qb2, int ka, int T, int w) {
  const int qs = qt * kBwdBQ + 32 * qb2, qz = qs + 31, kz = ka + 31;
  return !(ka >= T || qz < ka || qs - kz >= w || qs >= T);
}

// P waves, one query tile: S and P (to sP, bf16).
template <int D>
__device__ __forceinline__ void dkdv_pwave(const uint16_t* __restrict__ cur,
                                           uint16_t* __restrict__ sP, int qt, int ka, int kj,
                                           int T, int w, float sl2, const uint4 (&kf)[D / 16],
                                           const LdsOffsets<D>& lo, int lane) {
  constexpr int BQ = kBwdBQ, DK = D / 16, TILE = DkdvStage<D>::TILE;
  const int half = lane >> 5;
  const uint16_t* sQ = cur;
  const float* sL = reinterpret_cast<const float*>(cur + 2 * TILE);
#pragma unroll
  for (int qb2 = 0; qb2 < BQ / 32; ++qb2) {
    if (!dkdv_block_live(qt, qb2, ka, T, w)) continue;
    f32x16 acc = zero16();
#pragma unroll
    for (int t = 0; t < DK; ++t) acc = mfma32(rc_frag<D>(sQ, lo, qb2, t), kf[t], acc);
    sched_mfma_chain<DK, 1, DK>();
    const int qs = qt * BQ + 32 * qb2, qz = qs + 31, kz = ka + 31;
    if (qs >= kz && qz - ka < w && qz < T)
      dkdv_probs<false>(acc, sL, qb2, qt, kj, T, w, sl2, half);
    else
      dkdv_probs<true>(acc, sL, qb2, qt, kj, T, w, sl2, half);
    const uint4 pf0 = pack_frag(acc, 0), pf1 = pack_frag(acc, 1);
    uint4* dst = reinterpret_cast<uint4*>(sP) + qb2 * 2 * 64;
    dst[lane] = pf0;
    dst[64 + lane] = pf1;
    __builtin_amdgcn_sched_barrier(0);
  }
}

// dS waves, one query tile: dP, dS = P (dP - Delta) with P from sP, dV^T += dO^T P and
// dK^T += Q^T dS.
template <int D>
__device__ __forceinline__ void dkdv_swave(const uint16_t* __restrict__ cur,
                                           const uint16_t* __restrict__ sP, int qt, int ka, int T,
                                           int w, const uint4 (&vf)[D / 16],
                                           f32x16 (&dkacc)[D / 32], f32x16 (&dvacc)[D / 32],
                                           const LdsOffsets<D>& lo, int lane) {
  constexpr int BQ = kBwdBQ, DK = D / 16, MB = D / 32, TILE = DkdvStage<D>::TILE;
  const int half = lane >> 5;
  const uint16_t* sQ = cur;
  const uint16_t* sO = cur + TILE;
  const float* sDl = reinterpret_cast<const float*>(cur + 2 * TILE) + BQ;
#pragma unroll
  for (int qb2 = 0; qb2 < BQ / 32; ++qb2) {
    if (!dkdv_block_live(qt, qb2, ka, T, w)) continue;
    // the accumulator starts at the rows' Delta (the broadcast reads land in its own row order)
    // and vf holds -V, so the chain leaves Delta - dP and dS = P * that carries a sign that the
    // final scale of dK removes
    f32x16 dp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 d4 = *reinterpret_cast<const float4*>(sDl + 32 * qb2 + 8 * j + 4 * half);
      dp[4 * j + 0] = d4.x;
      dp[4 * j + 1] = d4.y;
      dp[4 * j + 2] = d4.z;
      dp[4 * j + 3] = d4.w;
    }
#pragma unroll
    for (int t = 0; t < DK; ++t) dp = mfma32(rc_frag<D>(sO, lo, qb2, t), vf[t], dp);
    sched_mfma_chain<DK, 1, DK>();
    const uint4* src = reinterpret_cast<const uint4*>(sP) + qb2 * 2 * 64;
    const uint4 pw[2] = {src[lane], src[64 + lane]};
    const uint32_t* pu = reinterpret_cast<const uint32_t*>(pw);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t word = pu[r >> 1];  // P slot r is bf16 element r of the packed pair
      const float pr = (r & 1) ? bf16_hi(word) : bf16_lo(word);
      dp[r] = pr * dp[r];
    }
    const uint4 df0 = pack_frag(dp, 0), df1 = pack_frag(dp, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      dvacc[m] = mfma32(tr_frag_o<D>(sO, lo, 32 * qb2, m), pw[0], dvacc[m]);
      dvacc[m] = mfma32(tr_frag_o<D>(sO, lo, 32 * qb2 + 16, m), pw[1], dvacc[m]);
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      dkacc[m] = mfma32(tr_frag_o<D>(sQ, lo, 32 * qb2, m), df0, dkacc[m]);
      dkacc[m] = mfma32(tr_frag_o<D>(sQ, lo, 32 * qb2 + 16, m), df1, dkacc[m]);
    }
    sched_mfma_chain<4 * MB, 2, 4>();
  }
}

// One iteration: DMA of tile qt_next (of a sequence of T_next rows) into `nxt`, then a P wave on `curp` (tile qt_p) or a dS wave
// on `curs` (tile qt_s, the P waves' tile of the previous iteration).  The __restrict__ qualifiers
// state that, within one iteration, the three stages and the two P buffers are distinct, so LDS
// reads need not wait for the DMA.
template <int D, int NW, bool PW>
__device__ __forceinline__ void dkdv_step(const uint16_t* __restrict__ curp,
                                          const uint16_t* __restrict__ curs,
                                          uint16_t* __restrict__ nxt, uint16_t* __restrict__ pw,
                                          const uint16_t* __restrict__ pr, bool issue_next,
                                          bool on, const uint16_t* qb, const uint16_t* db,
                                          const float* lseb, const float* delb, int rs, int qt_p,
                                          int qt_s, int qt_next, int T_next, int ka, int kj, int T,
                                          int w, float sl2, const uint4 (&frag)[D / 16],
                                          f32x16 (&acc)[D / 32], f32x16 (&acc2)[D / 32],
                                          const LdsOffsets<D>& lo,
                                          const RowDmaFlat<D, kDkdvDmaWaves, kBwdBQ>& dma, int wave,
                                          int lane) {
  if (issue_next)
    dkdv_issue<D, kDkdvDmaWaves>(dma, qb, db, lseb, delb, rs, qt_next, T_next, nxt, wave, lane);
  if (!on) return;
  if (PW)
    dkdv_pwave<D>(curp, pw, qt_p, ka, kj, T, w, sl2, frag, lo, lane);
  else
    dkdv_swave<D>(curs, pr, qt_s, ka, T, w, frag, acc, acc2, lo, lane);
}

// The tile loop of one role over query tiles qt_hi down to qt_lo (stage 0 holds tile qt_hi on
// entry).  Both roles pass the same barriers in the same order; each role gets its own copy of the
// loop so that its accumulators stay in one set of registers.  Iteration i: P waves on tile
// qt_hi - i (stage i % 3), dS waves on tile qt_hi - i + 1.
template <int D, int NW, bool PW>
__device__ __forceinline__ void dkdv_loop(uint16_t* smem, uint16_t* myP, int qt_lo, int qt_hi,
                                          const uint16_t* qb, const uint16_t* db,
                                          const float* lseb, const float* delb, int rs, int ka,
                                          int kj, int T, int w, float sl2,
                                          const uint4 (&frag)[D / 16], f32x16 (&acc)[D / 32],
                                          f32x16 (&acc2)[D / 32], const LdsOffsets<D>& lo,
                                          const RowDmaFlat<D, kDkdvDmaWaves, kBwdBQ>& dma, int wave,
                                          int lane) {
  constexpr int SE = DkdvStage<D>::ELEMS, PE = DkdvStage<D>::PELEMS;
  const int n = qt_hi - qt_lo + 1;
  int s0 = 0, s1 = 2 * SE, s2 = SE;  // element offsets of stages i % 3, (i - 1) % 3, (i + 1) % 3
  for (int i = 0; i <= n; ++i) {
    // tile i (the only DMA in flight) has landed: the P waves issued it and wait for it; then an
    // LDS-only barrier (no release fence: nothing here hands data through global memory)
    if (PW) wait_vmcnt<0>();
    lds_barrier();  // ... for all waves; P of tile i - 1 is complete; stage (i + 1) % 3 is free
    const int pb = (i & 1) * PE;
    const int qt = qt_hi - i;
    dkdv_step<D, NW, PW>(smem + s0, smem + s1, smem + s2, myP + pb, myP + (PE - pb), i + 1 < n,
                         PW ? (i < n) : (i >= 1), qb, db, lseb, delb, rs, qt, qt + 1, qt - 1, T,
                         ka, kj, T, w, sl2, frag, acc, acc2, lo, dma, wave, lane);
    const int t = s1;  // rotate: the stage just read one behind becomes the next DMA target
    s1 = s0;
    s0 = s2;
    s2 = t;
  }
}

// One job: key tile kt (128 keys) of head bh, walking the query tiles that see it from the last
// one down.  Returns with every wave past its last read of the ring and the P buffers.
template <int D, bool VARLEN, bool QKN>
__device__ __forceinline__ void dkdv_job(const BwdArgs& p, int bh, int kt, uint16_t* smem,
                                         uint16_t* sPbuf, int wave, int lane) {
  constexpr int NW = kDkdvWaves, BK = 128, BQ = kBwdBQ;
  constexpr int DK = D / 16, MB = D / 32, PE = DkdvStage<D>::PELEMS;
  const int half = lane >> 5, l32 = lane & 31;
  const bool pwave = wave < 4;
  const int kblk = wave & 3;

  const int b = bh / p.H, h = bh % p.H;
  const BwdRows rw = bwd_rows<VARLEN>(p, b, h, D);
  const int T = rw.T;
  const int k0 = kt * BK;
  if (k0 >= T) return;
  const int w = min(p.window, T);
  const int q_last = min(T, k0 + BK - 1 + w) - 1;
  const int qt_lo = k0 / BQ, qt_hi = q_last / BQ;

  const int64_t base = rw.base;
  const int rs = p.row_stride;
  const uint16_t* qb = p.q + base;
  const uint16_t* db = p.dout + base;
  const float* lseb = p.lse2 + rw.stat;  // LSE * log2(e), from the dQ pass
  const float* delb = p.delta + rw.stat;

  const RowDmaFlat<D, kDkdvDmaWaves, BQ> dma(rs, wave, lane);  // used by the issuing waves only
  dkdv_issue<D, kDkdvDmaWaves>(dma, qb, db, lseb, delb, rs, qt_hi, T, smem, wave, lane);

  const int ka = k0 + 32 * kblk;
  const int kj = ka + l32;
  const bool kvalid = kj < T;
  // P waves hold K (B operand of S = Q K^T), dS waves hold V (B operand of dP = dO V^T)
  const uint16_t* fsrc = pwave ? p.k : p.v;
  uint4 frag[DK];
  const int64_t foff = base + (int64_t)min(kj, T - 1) * rs + 8 * half;
#pragma unroll
  for (int t = 0; t < DK; ++t) frag[t] = ldg16(fsrc + foff + 16 * t);
  // QK-norm: 1 / rms of the raw k row, for dk's epilogue in the dS waves
  const float rk = QKN && !pwave ? p.rk[rw.stat + min(kj, T - 1)] : 0.f;
  if (!kvalid)
#pragma unroll
    for (int t = 0; t < DK; ++t) frag[t] = make_uint4(0, 0, 0, 0);
  if (!pwave)  // -V: the dS waves' dP chain accumulates onto Delta
#pragma unroll
    for (int t = 0; t < DK; ++t) {
      frag[t].x ^= 0x80008000u;
      frag[t].y ^= 0x80008000u;
      frag[t].z ^= 0x80008000u;
      frag[t].w ^= 0x80008000u;
    }
  f32x16 acc[MB], acc2[MB];  // dS waves: dK^T, dV^T
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = acc2[m] = zero16();

  const LdsOffsets<D> lo(lane);
  uint16_t* myP = sPbuf + kblk * (PE / 4);  // this key block's part of each P buffer
  if (pwave)
    dkdv_loop<D, NW, true>(smem, myP, qt_lo, qt_hi, qb, db, lseb, delb, rs, ka, kj, T, w,
                           p.scale_log2, frag, acc, acc2, lo, dma, wave, lane);
  else
    dkdv_loop<D, NW, false>(smem, myP, qt_lo, qt_hi, qb, db, lseb, delb, rs, ka, kj, T, w,
                            p.scale_log2, frag, acc, acc2, lo, dma, wave, lane);

  // QK-norm: the normalised k rows sit in the P waves' fragments; they reach the dS waves through
  // the ring's LDS (free once every wave is past the loop), rows padded by 16 bytes.
  uint2 ky[QKN ? MB : 1][4];
  if constexpr (QKN) {
    constexpr int XS = D + 8;
    static_assert(NW * 16 * XS <= kDkdvStages * DkdvStage<D>::ELEMS, "k rows fit the ring");
    uint16_t* xrow = smem + (kblk * 32 + l32) * XS;
    __syncthreads();
    if (pwave)
#pragma unroll
      for (int t = 0; t < DK; ++t) *reinterpret_cast<uint4*>(xrow + 16 * t + 8 * half) = frag[t];
    __syncthreads();
    if (!pwave)
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          ky[m][j] = *reinterpret_cast<const uint2*>(xrow + m * 32 + 8 * j + 4 * half);
  }

  if (!kvalid || pwave) return;
  {
    uint16_t* out = p.dv + base + (int64_t)kj * rs;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint2 a;
        a.x = pack_bf16x2(acc2[m][4 * j + 0], acc2[m][4 * j + 1]);
        a.y = pack_bf16x2(acc2[m][4 * j + 2], acc2[m][4 * j + 3]);
        *reinterpret_cast<uint2*>(out + m * 32 + 8 * j + 4 * half) = a;
      }
  }
  const float sc = -p.scale;  // the dS waves accumulated -dK^T
  uint16_t* out = p.dk + base + (int64_t)kj * rs;
  if constexpr (QKN) {  // dk with respect to the raw rows
    store_through_rmsnorm<D>(acc, sc, ky, rk, out, half);
    return;
  }
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint2 a;
      a.x = pack_bf16x2(acc[m][4 * j + 0] * sc, acc[m][4 * j + 1] * sc);
      a.y = pack_bf16x2(acc[m][4 * j + 2] * sc, acc[m][4 * j + 3] * sc);
      *reinterpret_cast<uint2*>(out + m * 32 + 8 * j + 4 * half) = a;
    }
}

// One workgroup per unit (QK-norm launches, and packed launches whose job plan would not fit):
// full-causal training pass
// (p.paired): workgroup = head + key-tile pair (n - 1 - j, j), the short tile (fewest queries)
// first, so that a head's workgroups start on the same query tiles together (pair_job).
// Otherwise: workgroup = one key tile, those seeing the most queries first.
template <int D, bool VARLEN, bool QKN>
__global__ __launch_bounds__(64 * kDkdvWaves, 1) void bwd_dkdv_kernel(BwdArgs p) {
  constexpr int SE = DkdvStage<D>::ELEMS, PE = DkdvStage<D>::PELEMS;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[kDkdvStages * SE];
  __shared__ __attribute__((aligned(16))) uint16_t sPbuf[2 * PE];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bid = blockIdx.x;
  int bh, kt0, kt1, njobs;
  if (p.paired) {
    const PairJob jb = pair_job(bid, p.BH, (p.n_tiles + 1) / 2);
    bh = jb.bh;
    kt0 = p.n_tiles - 1 - jb.j;
    kt1 = jb.j;
    njobs = kt1 != kt0 ? 2 : 1;
  } else {
    bh = bid % p.BH;
    kt0 = kt1 = bid / p.BH;
    njobs = 1;
  }
#pragma unroll 1
  for (int jx = 0; jx < njobs; ++jx) {
    if (jx) __syncthreads();  // every wave is done with the ring and P before the next job
    dkdv_job<D, VARLEN, QKN>(p, bh, jx ? kt1 : kt0, smem, sPbuf, wave, lane);
  }
}

// ------------------------------------------------------------------------ dK/dV, chained jobs
// Dense and packed-sequence launches (not QK-norm) run the dK/dV pass on a persistent grid, one
// workgroup per CU (a workgroup fills a CU: 8 waves at up to 256 VGPRs, 132 KB of LDS).  Each
// walks a list of jobs whose query tiles form one stream through the ring and the P buffers, so
// the P waves start a job's first tile while the dS waves finish the previous job's last one: no
// pipeline fill or drain and no start-up per job.  The P waves load the next job's K right after
// their last tile of the current one; the dS waves load the next job's V and then store dK and dV
// right after theirs.
//
// Units: paired (full causal), unit u is the tile pair pair_job(u) (key tiles n - 1 - j, then j);
// otherwise unit u is key tile u / BH of head u % BH (of sequence u % BH / H when packed; tiles
// past that sequence's end are empty).
//   dense: workgroup w takes units w, w + G, w + 2G, ... (G workgroups; every unit carries about
//     the same work);
//   packed: jobs differ widely in work (and most units lie past their sequence's end), so the live
//     jobs are handed out one at a time from a queue, longest first: the dQ pass leaves a plan
//     listing, per 128-key level, the sequences long enough for it; queue index i maps through
//     the plan (held in LDS) to a job; workgroup w's first job is index w, the others come from
//     an atomic counter in the workspace.  Wave 0 takes the jobs and publishes them two ahead in
//     an LDS ring that both roles read, each entry behind at least one barrier.
struct DkdvJob {
  int bh, kt;
  int T;             // rows of the sequence
  int qt_hi, qt_lo;  // the query tiles that see key tile kt, walked from qt_hi down
  int64_t base;      // element offset of the sequence's row 0 at the head
  int64_t stat;      // index of its row 0 in LSE * log2(e) and Delta
};

constexpr int kDkdvRing = 8;  // published jobs in LDS

// Key tile kt of head bh; false if it lies past the end of the head's sequence.
template <int D, bool VARLEN>
__device__ __forceinline__ bool dkdv_make_job(const BwdArgs& p, int bh, int kt, DkdvJob& jb) {
  const BwdRows rw = bwd_rows<VARLEN>(p, bh / p.H, bh % p.H, D);
  const int k0 = kt * 128;
  if (k0 >= rw.T) return false;
  const int w = min(p.window, rw.T);
  jb.bh = bh;
  jb.kt = kt;
  jb.T = rw.T;
  jb.qt_lo = k0 / kBwdBQ;
  jb.qt_hi = (min(rw.T, k0 + 127 + w) - 1) / kBwdBQ;
  jb.base = rw.base;
  jb.stat = rw.stat;
  return true;
}

// Dense jobs: job s (0 or 1) of unit u.  kDkdvLive: jb set; kDkdvEmpty: no such job; kDkdvEnd: u is
// past the last unit.
enum { kDkdvEnd, kDkdvEmpty, kDkdvLive };
template <int D>
__device__ __forceinline__ int dkdv_unit_job(const BwdArgs& p, int u, int s, DkdvJob& jb) {
  const int n = p.n_tiles;
  int bh, kt;
  if (p.paired) {
    const int npair = (n + 1) / 2;
    if (u >= p.BH * npair) return kDkdvEnd;
    const PairJob pj = pair_job(u, p.BH, npair);
    const int kt0 = n - 1 - pj.j;
    if (s == 1 && pj.j == kt0) return kDkdvEmpty;
    bh = pj.bh;
    kt = s ? pj.j : kt0;
  } else {
    if (u >= n * p.BH) return kDkdvEnd;
    if (s != 0) return kDkdvEmpty;
    bh = u % p.BH;
    kt = u / p.BH;
  }
  return dkdv_make_job<D, false>(p, bh, kt, jb) ? kDkdvLive : kDkdvEmpty;
}

// The job source of one workgroup.  Dense: a cursor over its units.  Packed: the queue (wave 0
// only) and the LDS ring.
struct DkdvSource {
  int u, s;       // dense: unit and job within it of the last job taken
  unsigned pend;  // packed, wave 0 lane 0: the queue index taken for the next job to publish
  int taken;      // packed: jobs published so far
};

// Packed: unit (kt * BH + bh) of queue index `idx` under the plan in LDS, or -1 past the last job.
// Index order: level by level (longest jobs first), sequences in order, heads innermost.
__device__ __forceinline__ int dkdv_plan_unit(const BwdArgs& p, const int* plan, int levels,
                                              int idx) {
  if (idx >= p.H * plan[levels]) return -1;
  int lo = 0, hi = levels - 1;  // the last level whose first index is <= idx (it is not empty)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.H * plan[mid] <= idx) lo = mid;
    else hi = mid - 1;
  }
  const int r = idx - p.H * plan[lo];
  const int seq = plan[levels + 1 + plan[lo] + r / p.H];
  return lo * p.BH + seq * p.H + r % p.H;
}

// Packed: publishes the workgroup's next job (wave 0 writes the ring).  The workgroup's first job
// is queue index blockIdx.x; the others come from the counter, each taken one publication before
// it is used, so that the atomic's latency passes under a job.
__device__ __forceinline__ void dkdv_publish(const BwdArgs& p, DkdvSource& src, const int* plan,
                                             int levels, int* ring, int wave, int lane) {
  if (wave == 0) {
    const int idx = src.taken == 0
                        ? (int)blockIdx.x
                        : (int)(gridDim.x + __builtin_amdgcn_readfirstlane(src.pend));
    unsigned nx = 0;
    if (lane == 0) nx = atomicAdd(p.qctr, 1u);
    src.pend = nx;
    const int u = dkdv_plan_unit(p, plan, levels, idx);
    if (lane == 0) ring[src.taken % kDkdvRing] = u;
  }
  ++src.taken;
}

// Packed: the job of published entry k; false at the end of the list.
template <int D>
__device__ __forceinline__ bool dkdv_ring_job(const BwdArgs& p, const int* ring, int k,
                                              DkdvJob& jb) {
  const int u = __builtin_amdgcn_readfirstlane(ring[k % kDkdvRing]);
  if (u < 0) return false;
  dkdv_make_job<D, true>(p, u % p.BH, u / p.BH, jb);  // live by the plan's construction
  return true;
}

// Dense: the job after the cursor's (the cursor moves to it); false past the last.
template <int D>
__device__ __forceinline__ bool dkdv_dense_next(const BwdArgs& p, DkdvSource& c, DkdvJob& jb) {
  while (true) {
    if (c.s == 0) {
      c.s = 1;
    } else {
      c.s = 0;
      c.u += gridDim.x;
    }
    const int r = dkdv_unit_job<D>(p, c.u, c.s, jb);
    if (r != kDkdvEmpty) return r == kDkdvLive;
  }
}

// The B fragments of a job: K for the P waves, -V for the dS waves (rows past T zero).
template <int D, bool PW>
__device__ __forceinline__ void dkdv_load_frag(const BwdArgs& p, const DkdvJob& jb, int kblk,
                                               int lane, uint4 (&frag)[D / 16]) {
  const int half = lane >> 5, l32 = lane & 31;
  const int kj = jb.kt * 128 + 32 * kblk + l32;
  const uint16_t* src = (PW ? p.k : p.v) + jb.base + (int64_t)min(kj, jb.T - 1) * p.row_stride +
                        8 * half;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) frag[t] = ldg16(src + 16 * t);
  if (kj >= jb.T)
#pragma unroll
    for (int t = 0; t < D / 16; ++t) frag[t] = make_uint4(0, 0, 0, 0);
  if (!PW)
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      frag[t].x ^= 0x80008000u;
      frag[t].y ^= 0x80008000u;
      frag[t].z ^= 0x80008000u;
      frag[t].w ^= 0x80008000u;
    }
}

// dS waves: dV and dK of a finished job (the waves accumulated dV^T and -dK^T).
template <int D>
__device__ __forceinline__ void dkdv_store(const BwdArgs& p, const DkdvJob& jb, int kblk,
                                           int lane, const f32x16 (&dkacc)[D / 32],
                                           const f32x16 (&dvacc)[D / 32]) {
  const int half = lane >> 5, l32 = lane & 31;
  const int kj = jb.kt * 128 + 32 * kblk + l32;
  if (kj >= jb.T) return;
  const int64_t row = jb.base + (int64_t)kj * p.row_stride + 4 * half;
  const float sc = -p.scale;
#pragma unroll
  for (int m = 0; m < D / 32; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint2 v, k;
      v.x = pack_bf16x2(dvacc[m][4 * j + 0], dvacc[m][4 * j + 1]);
      v.y = pack_bf16x2(dvacc[m][4 * j + 2], dvacc[m][4 * j + 3]);
      k.x = pack_bf16x2(dkacc[m][4 * j + 0] * sc, dkacc[m][4 * j + 1] * sc);
      k.y = pack_bf16x2(dkacc[m][4 * j + 2] * sc, dkacc[m][4 * j + 3] * sc);
      *reinterpret_cast<uint2*>(p.dv + row + m * 32 + 8 * j) = v;
      *reinterpret_cast<uint2*>(p.dk + row + m * 32 + 8 * j) = k;
    }
}

// Rows of a job's sequence at its head: Q, dO and LSE * log2(e), Delta.
struct DkdvRows {
  const uint16_t *q, *dout;
  const float *lse2, *delta;
};
__device__ __forceinline__ DkdvRows dkdv_rows(const BwdArgs& p, const DkdvJob& jb) {
  return {p.q + jb.base, p.dout + jb.base, p.lse2 + jb.stat, p.delta + jb.stat};
}

// One role's walk over the workgroup's jobs.  Global iteration g runs the P waves on stream tile
// g and the dS waves on tile g - 1, one barrier each (tiles + 1 in all for both roles, plus one
// before the walk when packed): the P waves idle in the last iteration, the dS waves in the
// first.  Within a job the tile loop is the single-job loop's; between jobs the P waves load the
// next K, the dS waves store dK and dV and load the next -V.  A workgroup without a job passes no
// further barrier, in both roles.
template <int D, bool VARLEN, bool PW>
__device__ __forceinline__ void dkdv_chain(const BwdArgs& p, uint16_t* smem, uint16_t* myP,
                                           int* ring, int* plan, int kblk, int wave, int lane) {
  constexpr int BQ = kBwdBQ, MB = D / 32;
  constexpr int SE = DkdvStage<D>::ELEMS, PE = DkdvStage<D>::PELEMS;
  const int l32 = lane & 31;
  const int rs = p.row_stride;
  const LdsOffsets<D> lo(lane);
  const RowDmaFlat<D, kDkdvDmaWaves, BQ> dma(rs, wave, lane);
  DkdvSource src{(int)blockIdx.x, 0, 0u, 0};
  DkdvJob J, N;
  bool hasN;
  const int levels = p.n_tiles;
  if constexpr (VARLEN) {
    // the plan into LDS, then jobs 0 and 1 published before the walk
    const int nplan = min(levels + 1 + p.plan[levels], kDkdvPlanMax);
    for (int i = threadIdx.x; i < nplan; i += blockDim.x) plan[i] = p.plan[i];
    __syncthreads();
    dkdv_publish(p, src, plan, levels, ring, wave, lane);
    dkdv_publish(p, src, plan, levels, ring, wave, lane);
    __syncthreads();
    if (!dkdv_ring_job<D>(p, ring, 0, J)) return;
    N = J;
    hasN = dkdv_ring_job<D>(p, ring, 1, N);
  } else {
    const int r = dkdv_unit_job<D>(p, src.u, 0, J);
    if (r != kDkdvLive) return;  // the launch has no more workgroups than units
    N = J;
    hasN = dkdv_dense_next<D>(p, src, N);
  }
  int k = 0;  // the job in hand (packed: its ring entry)
  uint4 frag[D / 16];
  dkdv_load_frag<D, PW>(p, J, kblk, lane, frag);
  f32x16 acc[MB], acc2[MB];  // dS waves: dK^T, dV^T
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = acc2[m] = zero16();

  int g = 0, s0 = 0, s1 = 2 * SE, s2 = SE;  // stages g % 3, (g - 1) % 3, (g + 1) % 3
  auto rotate = [&] {  // the stage just read one behind becomes the next DMA target
    const int t = s1;
    s1 = s0;
    s0 = s2;
    s2 = t;
    ++g;
  };
  if (PW) {
    const DkdvRows rj = dkdv_rows(p, J);
    dkdv_issue<D, kDkdvDmaWaves>(dma, rj.q, rj.dout, rj.lse2, rj.delta, rs, J.qt_hi, J.T, smem,
                                 wave, lane);
  } else {
    lds_barrier();  // iteration 0: the P waves' first tile
    rotate();
  }
#pragma unroll 1
  while (true) {
    // packed: wave 0 publishes job k + 2 before job k's tiles (their barriers order the write
    // before any read of it: job k + 1's, at the earliest)
    if (VARLEN && PW) dkdv_publish(p, src, plan, levels, ring, wave, lane);
    const DkdvRows rj = dkdv_rows(p, J);
    const int ka = J.kt * 128 + 32 * kblk, n = J.qt_hi - J.qt_lo + 1;
    const int TJ = VARLEN ? J.T : p.T, TN = VARLEN ? N.T : p.T;  // dense: every job has T rows
    const int w = min(p.window, TJ);
#pragma unroll 1
    for (int i = 0; i < n; ++i) {
      // tile g (the only DMA in flight) has landed: the P waves issued it and wait for it; then
      // an LDS-only barrier for all waves: P of tile g - 1 is complete, stage (g + 1) % 3 is free
      if (PW) wait_vmcnt<0>();
      lds_barrier();
      const int pb = (g & 1) * PE, qt = J.qt_hi - i;
      const bool last = i == n - 1;  // the next stream tile is the next job's first
      const DkdvRows rx = last && hasN ? dkdv_rows(p, N) : rj;
      dkdv_step<D, kDkdvWaves, PW>(smem + s0, smem + s1, smem + s2, myP + pb, myP + (PE - pb),
                                   PW && (!last || hasN), true, rx.q, rx.dout, rx.lse2, rx.delta,
                                   rs, qt, qt, last ? N.qt_hi : qt - 1, last ? TN : TJ, ka,
                                   ka + l32, TJ, w, p.scale_log2, frag, acc, acc2, lo, dma, wave,
                                   lane);
      rotate();
    }
    // the next job's fragments are loaded before this job's dK / dV stores are issued: a wait
    // for the loads then need not wait for the stores (vector memory counts them in order)
    if (hasN) dkdv_load_frag<D, PW>(p, N, kblk, lane, frag);
    if (!PW) {
      dkdv_store<D>(p, J, kblk, lane, acc, acc2);
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[m] = acc2[m] = zero16();
    }
    if (!hasN) break;
    J = N;
    ++k;
    if constexpr (VARLEN) hasN = dkdv_ring_job<D>(p, ring, k + 1, N);
    else hasN = dkdv_dense_next<D>(p, src, N);
  }
  if (PW) {  // the last iteration: the dS waves' last tile
    wait_vmcnt<0>();
    lds_barrier();
  }
}

template <int D, bool VARLEN>
__global__ __launch_bounds__(64 * kDkdvWaves, 1) void bwd_dkdv_chain_kernel(BwdArgs p) {
  constexpr int SE = DkdvStage<D>::ELEMS, PE = DkdvStage<D>::PELEMS;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[kDkdvStages * SE];
  __shared__ __attribute__((aligned(16))) uint16_t sPbuf[2 * PE];
  __shared__ int ring[VARLEN ? kDkdvRing : 1];       // packed: the workgroup's published jobs
  __shared__ int plan[VARLEN ? kDkdvPlanMax : 1];    // packed: the job plan
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kblk = wave & 3;
  uint16_t* myP = sPbuf + kblk * (PE / 4);  // this key block's part of each P buffer
  if (wave < 4)
    dkdv_chain<D, VARLEN, true>(p, smem, myP, ring, plan, kblk, wave, lane);
  else
    dkdv_chain<D, VARLEN, false>(p, smem, myP, ring, plan, kblk, wave, lane);
}

// ------------------------------------------------------------------------------------- launchers
template <int D, int NW>
static hipError_t launch_dq_d(const BwdArgs& a, hipStream_t s) {
  BwdArgs p = a;
  p.n_tiles = (p.T + 32 * NW - 1) / (32 * NW);
  // tile pairs carry equal work under the full causal mask over equal-length sequences; they are
  // used when they fill whole rounds of the two-per-CU slots (else single tiles, longest first)
  p.paired = (p.cu == nullptr && p.window >= p.T &&
              pairs_fill_rounds((unsigned)(p.n_tiles + 1) / 2 * (unsigned)p.BH,
                                2u * (unsigned)device_compute_units()))
                 ? 1
                 : 0;
  const unsigned per_head = p.paired ? (unsigned)(p.n_tiles + 1) / 2 : (unsigned)p.n_tiles;
  const unsigned grid = per_head * (unsigned)p.BH;
  if (p.cu)
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW, true, false>), dim3(grid), dim3(64 * NW), 0, s, p);
  else if (p.rq)
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW, false, true>), dim3(grid), dim3(64 * NW), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW, false, false>), dim3(grid), dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_dkdv_d(const BwdArgs& a, hipStream_t s) {
  BwdArgs p = a;
  p.n_tiles = (p.T + 127) / 128;  // 128 keys per job
  // tile pairs carry equal work under the full causal mask over equal-length sequences
  p.paired = (p.cu == nullptr && p.window >= p.T) ? 1 : 0;
  const unsigned per_head = p.paired ? (unsigned)(p.n_tiles + 1) / 2 : (unsigned)p.n_tiles;
  const unsigned grid = per_head * (unsigned)p.BH;
  if (p.rk) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, true>), dim3(grid), dim3(64 * kDkdvWaves), 0, s,
                       p);
    return hipGetLastError();
  }
  if (p.cu && !p.plan) {  // packed, with more sequences or jobs than a plan holds
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, false>), dim3(grid), dim3(64 * kDkdvWaves), 0, s,
                       p);
    return hipGetLastError();
  }
  // persistent: one workgroup per CU, each chaining its share of the units (packed: of the jobs
  // of the plan; workgroups beyond the number of jobs leave at once)
  const unsigned cus = (unsigned)device_compute_units();
  const unsigned pgrid = cus > 0 && cus < grid ? cus : grid;
  if (p.cu)
    hipLaunchKernelGGL((bwd_dkdv_chain_kernel<D, true>), dim3(pgrid), dim3(64 * kDkdvWaves), 0, s,
                       p);
  else
    hipLaunchKernelGGL((bwd_dkdv_chain_kernel<D, false>), dim3(pgrid), dim3(64 * kDkdvWaves), 0, s,
                       p);
  return hipGetLastError();
}

// As in the forward: launches with fewer 4-wave workgroups than CUs take one wave per workgroup.
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t s) {
  const long long wide = (long long)((a.T + 127) / 128) * a.BH;
  if (wide < device_compute_units())
    return a.D == 64 ? launch_dq_d<64, 1>(a, s) : launch_dq_d<128, 1>(a, s);
  return a.D == 64 ? launch_dq_d<64, 4>(a, s) : launch_dq_d<128, 4>(a, s);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t s) {
  return a.D == 64 ? launch_dkdv_d<64>(a, s) : launch_dkdv_d<128>(a, s);
}

}  // namespace swattn
