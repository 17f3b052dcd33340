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
// the forward), computes Delta for them first and writes it to the workspace, then walks the
// in-window key tiles: S^T = K Q^T, dP^T = V dO^T, dS^T, and dQ^T += K^T dS^T.
// dK/dV pass: a workgroup owns 128 keys and walks the query tiles that can see them; half of its
// waves compute S = Q K^T, P and dV^T += dO^T P, the other half dP = dO V^T, dS and dK^T += Q^T dS,
// exchanging P through LDS (lane = key in both).
// Both passes stream their tiles global -> LDS with global_load_lds into a two-stage ring (one
// tile ahead, one barrier per tile) and take every transposed operand (K^T, Q^T, dO^T) straight
// from the row-major tile with ds_read_b64_tr_b16.
#include "common.h"
#include "launch.h"

namespace swattn {

constexpr int kBwdBC = 64;  // keys per tile in the dQ pass
constexpr int kBwdBQ = 64;  // queries per tile in the dK/dV pass

// ------------------------------------------------------------------------------------------ dQ
template <int D, bool MASK>
__device__ __forceinline__ void dq_tile(const uint16_t* __restrict__ sK,
                                        const uint16_t* __restrict__ sV, int k_lo, int qi, int w,
                                        float sl2, float lse2, float delta,
                                        const uint4 (&qf)[D / 16], const uint4 (&df)[D / 16],
                                        const LdsOffsets<D>& lo, f32x16 (&dqacc)[D / 32],
                                        int lane) {
  constexpr int BC = kBwdBC, DK = D / 16, MB = D / 32, NB = BC / 32;
  const int half = lane >> 5;
#pragma unroll 1
  for (int nb = 0; nb < NB; ++nb) {
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int t = 0; t < DK; ++t) {
      s = mfma32(rc_frag<D>(sK, lo, nb, t), qf[t], s);
      dp = mfma32(rc_frag<D>(sV, lo, nb, t), df[t], dp);
    }
    // key j is visible to query i iff (unsigned)(i - j) < w
    const int d0 = qi - (k_lo + nb * 32) - 4 * half;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pr = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -lse2));
      if (MASK) {
        const unsigned dist = (unsigned)(d0 - (8 * (r >> 2) + (r & 3)));
        pr = dist < (unsigned)w ? pr : 0.f;
      }
      s[r] = pr * (dp[r] - delta);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint4 dsf = pack_frag(s, u);
#pragma unroll
      for (int m = 0; m < MB; ++m)
        dqacc[m] = mfma32(tr_frag_o<D>(sK, lo, nb * 32 + 16 * u, m), dsf, dqacc[m]);
    }
  }
}

template <int D, int NW>
__device__ __forceinline__ void dq_step(const uint16_t* __restrict__ cur,
                                        uint16_t* __restrict__ nxt, bool issue_next,
                                        const uint16_t* kb, const uint16_t* vb, int rs, int T,
                                        int kt, int qa, int qi, int w, float sl2, float lse2,
                                        float delta, const uint4 (&qf)[D / 16],
                                        const uint4 (&df)[D / 16], const LdsOffsets<D>& lo,
                                        f32x16 (&dqacc)[D / 32], int wave, int lane) {
  constexpr int BC = kBwdBC, TILE = BC * D;
  if (issue_next) {
    issue_rows<D, NW, BC>(kb, rs, (kt + 1) * BC, T - 1, nxt, wave, lane);
    issue_rows<D, NW, BC>(vb, rs, (kt + 1) * BC, T - 1, nxt + TILE, wave, lane);
  }
  const int k_lo = kt * BC, k_hi = k_lo + BC - 1, qz = qa + 31;
  if ((qa >= T) || (k_lo > qz) || (qa - k_hi >= w)) return;
  if (k_hi <= qa && qz - k_lo < w)
    dq_tile<D, false>(cur, cur + TILE, k_lo, qi, w, sl2, lse2, delta, qf, df, lo, dqacc, lane);
  else
    dq_tile<D, true>(cur, cur + TILE, k_lo, qi, w, sl2, lse2, delta, qf, df, lo, dqacc, lane);
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dq_kernel(BwdArgs p) {
  constexpr int BR = 32 * NW, BC = kBwdBC;
  constexpr int DK = D / 16, MB = D / 32, TILE = BC * D;

  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * 2 * TILE];  // [stage][K|V]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int bid = blockIdx.x;
  const int qt = p.n_tiles - 1 - bid / p.BH;
  const int bh = bid % p.BH;
  const int b = bh / p.H, h = bh % p.H;
  const int T = p.T;
  const int q0 = qt * BR;
  const int w = min(p.window, T);
  const int kstart = max(0, q0 - w + 1);
  const int qend = min(q0 + BR, T);
  const int kt_begin = kstart / BC, kt_end = (qend - 1) / BC;

  const int64_t base = (int64_t)b * p.bstride + h * D;
  const int rs = p.row_stride;
  const uint16_t* kb = p.k + base;
  const uint16_t* vb = p.v + base;

  issue_rows<D, NW, BC>(kb, rs, kt_begin * BC, T - 1, smem, wave, lane);
  issue_rows<D, NW, BC>(vb, rs, kt_begin * BC, T - 1, smem + TILE, wave, lane);

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
  const float lse_raw = p.lse[(int64_t)bh * T + qc];
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
  if (qvalid && half == 0) p.delta[(int64_t)bh * T + qi] = delta;
  const float lse2 = qvalid ? lse_raw * kLog2e : 0.f;

  f32x16 dqacc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) dqacc[m] = zero16();

  const LdsOffsets<D> lo(lane);
  uint16_t* stage0 = smem;
  uint16_t* stage1 = smem + 2 * TILE;
  for (int kt = kt_begin; kt <= kt_end; ++kt) {
    wait_vmcnt<0>();
    __syncthreads();
    const bool even = ((kt - kt_begin) & 1) == 0;
    dq_step<D, NW>(even ? stage0 : stage1, even ? stage1 : stage0, kt < kt_end, kb, vb, rs, T, kt,
                   qa, qi, w, p.scale_log2, lse2, delta, qf, df, lo, dqacc, wave, lane);
  }

  if (!qvalid) return;
  const float sc = p.scale;
  uint16_t* out = p.dq + base + (int64_t)qi * rs;
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

// ---------------------------------------------------------------------------------------- dK/dV
// Eight waves own 128 keys: waves 0-3 ("P waves") compute S = Q K^T and P for key block w and
// accumulate dV^T += dO^T P; waves 4-7 ("dS waves") compute dP = dO V^T for the same key block and
// accumulate dK^T += Q^T dS.  P passes from one to the other through LDS in register order (fp32),
// so each wave carries one operand fragment set and one accumulator set -- two waves per SIMD --
// and the MFMA work per phase is balanced: {S | dP}, barrier, {dV | dS, dK}.
constexpr int kDkdvWaves = 8;

template <int D>
struct DkdvStage {
  static constexpr int TILE = kBwdBQ * D;
  static constexpr int ELEMS = 2 * TILE + 2 * kBwdBQ * 2;  // Q | dO | LSE | Delta, uint16 units
};

template <int D, int NW>
__device__ __forceinline__ void dkdv_issue(const uint16_t* qb, const uint16_t* db,
                                           const float* lseb, const float* delb, int rs, int qt,
                                           int T, uint16_t* stage, int wave, int lane) {
  constexpr int BQ = kBwdBQ, TILE = DkdvStage<D>::TILE;
  issue_rows<D, NW, BQ>(qb, rs, qt * BQ, T - 1, stage, wave, lane);
  issue_rows<D, NW, BQ>(db, rs, qt * BQ, T - 1, stage + TILE, wave, lane);
  static_assert(BQ == 64, "one 4-byte DMA per lane covers the 64 rows' LSE / Delta");
  if (wave == NW - 1) {
    const int j = min(qt * BQ + lane, T - 1);
    float* sl = reinterpret_cast<float*>(stage + 2 * TILE);
    g2lds4(lseb + j, sl);
    g2lds4(delb + j, sl + BQ);
  }
}

// P = exp2(S * scale - LSE) for one 32-query block (lane = key kj, accumulator r = query row).
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
      float pr = __builtin_amdgcn_exp2f(fmaf(acc[r], sl2, -lv[i] * kLog2e));
      if (MASK) {
        // query i sees key j iff (unsigned)(i - j) < w; rows past T hold a clamped copy: drop them
        const int qg = qt * BQ + ql0 + i;
        pr = ((unsigned)(qg - kj) < (unsigned)w) & (qg < T) ? pr : 0.f;
      }
      acc[r] = pr;
    }
  }
}

// Phase 1 of one query tile.  P waves: S, P (written to sP); dS waves: dP (kept in registers).
template <int D>
__device__ __forceinline__ void dkdv_phase1(const uint16_t* __restrict__ cur,
                                            float* __restrict__ sP, bool pwave, int qt, int ka,
                                            int kj, int T, int w, float sl2,
                                            const uint4 (&frag)[D / 16], f32x16 (&dp)[2],
                                            const LdsOffsets<D>& lo, int lane) {
  constexpr int BQ = kBwdBQ, DK = D / 16, TILE = DkdvStage<D>::TILE;
  const int half = lane >> 5, l32 = lane & 31;
  const uint16_t* src = pwave ? cur : cur + TILE;  // Q rows for S, dO rows for dP
  const float* sL = reinterpret_cast<const float*>(cur + 2 * TILE);
#pragma unroll
  for (int qb2 = 0; qb2 < BQ / 32; ++qb2) {
    const int qs = qt * BQ + 32 * qb2, qz = qs + 31, kz = ka + 31;
    if (ka >= T || qz < ka || qs - kz >= w || qs >= T) continue;
    f32x16 acc = zero16();
#pragma unroll
    for (int t = 0; t < DK; ++t) acc = mfma32(rc_frag<D>(src, lo, qb2, t), frag[t], acc);
    if (!pwave) {
      dp[qb2] = acc;
      continue;
    }
    if (qs >= kz && qz - ka < w && qz < T)
      dkdv_probs<false>(acc, sL, qb2, qt, kj, T, w, sl2, half);
    else
      dkdv_probs<true>(acc, sL, qb2, qt, kj, T, w, sl2, half);
    float4* dst = reinterpret_cast<float4*>(sP) + qb2 * 4 * 64;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dst[j * 64 + lane] = make_float4(acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]);
  }
}

// Phase 2.  P waves: dV^T += dO^T P; dS waves: dS = P (dP - Delta), dK^T += Q^T dS.
template <int D>
__device__ __forceinline__ void dkdv_phase2(const uint16_t* __restrict__ cur,
                                            const float* __restrict__ sP, bool pwave, int qt,
                                            int ka, int T, int w, const f32x16 (&dp)[2],
                                            f32x16 (&acc)[D / 32], const LdsOffsets<D>& lo,
                                            int lane) {
  constexpr int BQ = kBwdBQ, MB = D / 32, TILE = DkdvStage<D>::TILE;
  const int half = lane >> 5;
  const uint16_t* sQ = cur;
  const uint16_t* sO = cur + TILE;
  const float* sDl = reinterpret_cast<const float*>(cur + 2 * TILE) + BQ;
#pragma unroll
  for (int qb2 = 0; qb2 < BQ / 32; ++qb2) {
    const int qs = qt * BQ + 32 * qb2, qz = qs + 31, kz = ka + 31;
    if (ka >= T || qz < ka || qs - kz >= w || qs >= T) continue;
    const float4* src = reinterpret_cast<const float4*>(sP) + qb2 * 4 * 64;
    f32x16 x;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v4 = src[j * 64 + lane];
      x[4 * j] = v4.x;
      x[4 * j + 1] = v4.y;
      x[4 * j + 2] = v4.z;
      x[4 * j + 3] = v4.w;
    }
    if (!pwave) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 d4 = *reinterpret_cast<const float4*>(sDl + 32 * qb2 + 8 * j + 4 * half);
        x[4 * j] *= dp[qb2][4 * j] - d4.x;
        x[4 * j + 1] *= dp[qb2][4 * j + 1] - d4.y;
        x[4 * j + 2] *= dp[qb2][4 * j + 2] - d4.z;
        x[4 * j + 3] *= dp[qb2][4 * j + 3] - d4.w;
      }
    }
    const uint16_t* tsrc = pwave ? sO : sQ;  // dO^T for dV, Q^T for dK
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint4 f = pack_frag(x, u);
#pragma unroll
      for (int m = 0; m < MB; ++m)
        acc[m] = mfma32(tr_frag_o<D>(tsrc, lo, 32 * qb2 + 16 * u, m), f, acc[m]);
    }
  }
}

// One query tile: issue the next tile's DMA into `nxt`, phase 1, LDS hand-off of P, phase 2.  The
// __restrict__ qualifiers state that, within one tile, the stage being read, the stage being
// filled and the P exchange buffer are distinct, so the LDS reads need not wait for the DMA.
template <int D, int NW>
__device__ __forceinline__ void dkdv_step(const uint16_t* __restrict__ cur,
                                          uint16_t* __restrict__ nxt, float* __restrict__ sP,
                                          bool issue_next, const uint16_t* qb, const uint16_t* db,
                                          const float* lseb, const float* delb, int rs, int qt,
                                          int ka, int kj, int T, int w, float sl2, bool pwave,
                                          const uint4 (&frag)[D / 16], f32x16 (&dp)[2],
                                          f32x16 (&acc)[D / 32], const LdsOffsets<D>& lo,
                                          int wave, int lane) {
  if (issue_next) dkdv_issue<D, NW>(qb, db, lseb, delb, rs, qt + 1, T, nxt, wave, lane);
  dkdv_phase1<D>(cur, sP, pwave, qt, ka, kj, T, w, sl2, frag, dp, lo, lane);
  lds_barrier();  // P of this tile is in LDS
  dkdv_phase2<D>(cur, sP, pwave, qt, ka, T, w, dp, acc, lo, lane);
}

template <int D>
__global__ __launch_bounds__(64 * kDkdvWaves, 1) void bwd_dkdv_kernel(BwdArgs p) {
  constexpr int NW = kDkdvWaves, BK = 128, BQ = kBwdBQ;
  constexpr int DK = D / 16, MB = D / 32, SE = DkdvStage<D>::ELEMS;
  constexpr int PELEMS = 4 * BQ * 32;  // fp32 P of 4 key blocks x 64 queries

  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * SE];
  __shared__ __attribute__((aligned(16))) float sPall[PELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const bool pwave = wave < 4;
  const int kblk = wave & 3;
  float* sP = sPall + kblk * BQ * 32;

  const int bid = blockIdx.x;
  const int kt = bid / p.BH;  // key tiles nearest the start see the most queries: first
  const int bh = bid % p.BH;
  const int b = bh / p.H, h = bh % p.H;
  const int T = p.T;
  const int k0 = kt * BK;
  const int w = min(p.window, T);
  const int q_last = min(T, k0 + BK - 1 + w) - 1;
  const int qt_begin = k0 / BQ, qt_end = q_last / BQ;

  const int64_t base = (int64_t)b * p.bstride + h * D;
  const int rs = p.row_stride;
  const uint16_t* qb = p.q + base;
  const uint16_t* db = p.dout + base;
  const float* lseb = p.lse + (int64_t)bh * T;
  const float* delb = p.delta + (int64_t)bh * T;

  dkdv_issue<D, NW>(qb, db, lseb, delb, rs, qt_begin, T, smem, wave, lane);

  const int ka = k0 + 32 * kblk;
  const int kj = ka + l32;
  const bool kvalid = kj < T;
  // P waves hold K (B operand of S = Q K^T), dS waves hold V (B operand of dP = dO V^T)
  const uint16_t* fsrc = pwave ? p.k : p.v;
  uint4 frag[DK];
  const int64_t foff = base + (int64_t)min(kj, T - 1) * rs + 8 * half;
#pragma unroll
  for (int t = 0; t < DK; ++t) frag[t] = ldg16(fsrc + foff + 16 * t);
  if (!kvalid)
#pragma unroll
    for (int t = 0; t < DK; ++t) frag[t] = make_uint4(0, 0, 0, 0);
  f32x16 acc[MB];  // dV^T (P waves) or dK^T (dS waves)
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = zero16();
  f32x16 dp[2];

  const LdsOffsets<D> lo(lane);
  uint16_t* stage0 = smem;
  uint16_t* stage1 = smem + SE;
  for (int qt = qt_begin; qt <= qt_end; ++qt) {
    wait_vmcnt<0>();
    __syncthreads();  // stage qt landed for all waves; previous tile's phase 2 is finished
    const bool even = ((qt - qt_begin) & 1) == 0;
    dkdv_step<D, NW>(even ? stage0 : stage1, even ? stage1 : stage0, sP, qt < qt_end, qb, db,
                     lseb, delb, rs, qt, ka, kj, T, w, p.scale_log2, pwave, frag, dp, acc, lo,
                     wave, lane);
  }

  if (!kvalid) return;
  const float sc = pwave ? 1.f : p.scale;
  uint16_t* out = (pwave ? p.dv : p.dk) + base + (int64_t)kj * rs;
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

// ------------------------------------------------------------------------------------- launchers
template <int D>
static hipError_t launch_dq_d(const BwdArgs& a, hipStream_t s) {
  constexpr int NW = 4;
  BwdArgs p = a;
  p.n_tiles = (p.T + 32 * NW - 1) / (32 * NW);
  const unsigned grid = (unsigned)p.n_tiles * (unsigned)p.BH;
  hipLaunchKernelGGL((bwd_dq_kernel<D, NW>), dim3(grid), dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_dkdv_d(const BwdArgs& a, hipStream_t s) {
  BwdArgs p = a;
  p.n_tiles = (p.T + 127) / 128;  // 128 keys per workgroup
  const unsigned grid = (unsigned)p.n_tiles * (unsigned)p.BH;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3(grid), dim3(64 * kDkdvWaves), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t s) {
  return a.D == 64 ? launch_dq_d<64>(a, s) : launch_dq_d<128>(a, s);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t s) {
  return a.D == 64 ? launch_dkdv_d<64>(a, s) : launch_dkdv_d<128>(a, s);
}

}  // namespace swattn
