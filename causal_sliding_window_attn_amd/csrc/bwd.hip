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
// dK/dV pass: a workgroup owns NW x 32 keys (K, V in registers, lane = key) and walks the query
// tiles that can see them: S = Q K^T, dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS.
// Both passes stream their tiles global -> LDS with global_load_lds into a two-stage ring (one
// tile ahead, one barrier per tile) and take every transposed operand (K^T, Q^T, dO^T) straight
// from the row-major tile with ds_read_b64_tr_b16.
#include "common.h"
#include "launch.h"

namespace swattn {

constexpr int kBwdBC = 64;  // keys per tile in the dQ pass
constexpr int kBwdBQ = 64;  // queries per tile in the dK/dV pass

// ------------------------------------------------------------------------------------------ dQ
template <int D, int NW>
__device__ __forceinline__ void dq_step(const uint16_t* __restrict__ cur,
                                        uint16_t* __restrict__ nxt, bool issue_next,
                                        const uint16_t* kb, const uint16_t* vb, int rs, int T,
                                        int kt, int qa, int qi, int w, float sl2, float lse2,
                                        float delta, const uint4 (&qf)[D / 16],
                                        const uint4 (&df)[D / 16], f32x16 (&dqacc)[D / 32],
                                        int wave, int lane) {
  constexpr int BC = kBwdBC, DK = D / 16, MB = D / 32, NB = BC / 32, TILE = BC * D;
  const int half = lane >> 5, l32 = lane & 31;
  if (issue_next) {
    issue_rows<D, NW, BC>(kb, rs, (kt + 1) * BC, T - 1, nxt, wave, lane);
    issue_rows<D, NW, BC>(vb, rs, (kt + 1) * BC, T - 1, nxt + TILE, wave, lane);
  }
  const uint16_t* sK = cur;
  const uint16_t* sV = cur + TILE;
  const int k_lo = kt * BC, k_hi = k_lo + BC - 1, qz = qa + 31;
  if ((qa >= T) || (k_lo > qz) || (qa - k_hi >= w)) return;
  const bool need_mask = !(k_hi <= qa && qz - k_lo < w);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f32x16 s = zero16(), dp = zero16();
    const int row = nb * 32 + l32;
#pragma unroll
    for (int t = 0; t < DK; ++t) {
      s = mfma32(row_chunk<D>(sK, row, 2 * t + half), qf[t], s);
      dp = mfma32(row_chunk<D>(sV, row, 2 * t + half), df[t], dp);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pr = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -lse2));
      if (need_mask) {
        const int key = k_lo + nb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (key > qi || qi - key >= w) pr = 0.f;
      }
      s[r] = pr * (dp[r] - delta);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint4 dsf = pack_frag(s, u);
#pragma unroll
      for (int m = 0; m < MB; ++m)
        dqacc[m] = mfma32(tr_frag<D>(sK, nb * 32 + 16 * u, m, lane), dsf, dqacc[m]);
    }
  }
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dq_kernel(BwdArgs p) {
  constexpr int BR = 32 * NW, BC = kBwdBC;
  constexpr int DK = D / 16, MB = D / 32, TILE = BC * D;

  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * 2 * TILE];  // [stage][K|V]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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

  uint4 qf[DK], df[DK];
  float dsum = 0.f;
#pragma unroll
  for (int t = 0; t < DK; ++t) {
    const int64_t off = base + (int64_t)qi * rs + 16 * t + 8 * half;
    if (qvalid) {
      qf[t] = ldg16(p.q + off);
      df[t] = ldg16(p.dout + off);
      const uint4 ov = ldg16(p.o + off);
      const uint32_t* dw = reinterpret_cast<const uint32_t*>(&df[t]);
      const uint32_t* ow = reinterpret_cast<const uint32_t*>(&ov);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dsum += bf16_lo(dw[e]) * bf16_lo(ow[e]) + bf16_hi(dw[e]) * bf16_hi(ow[e]);
    } else {
      qf[t] = make_uint4(0, 0, 0, 0);
      df[t] = make_uint4(0, 0, 0, 0);
    }
  }
  const float delta = sum_with_partner(dsum);
  if (qvalid && half == 0) p.delta[(int64_t)bh * T + qi] = delta;
  const float lse2 = qvalid ? p.lse[(int64_t)bh * T + qi] * kLog2e : 0.f;

  f32x16 dqacc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) dqacc[m] = zero16();

  uint16_t* stage0 = smem;
  uint16_t* stage1 = smem + 2 * TILE;
  for (int kt = kt_begin; kt <= kt_end; ++kt) {
    wait_vmcnt<0>();
    __syncthreads();
    const bool even = ((kt - kt_begin) & 1) == 0;
    dq_step<D, NW>(even ? stage0 : stage1, even ? stage1 : stage0, kt < kt_end, kb, vb, rs, T, kt,
                   qa, qi, w, p.scale_log2, lse2, delta, qf, df, dqacc, wave, lane);
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
// One query tile's stage: Q rows, dO rows (row-major, swizzled), then LSE and Delta of the rows.
template <int D>
struct DkdvStage {
  static constexpr int TILE = kBwdBQ * D;
  static constexpr int ELEMS = 2 * TILE + 2 * kBwdBQ * 2;  // in uint16 units
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

template <int D, int NW>
__device__ __forceinline__ void dkdv_step(const uint16_t* __restrict__ cur,
                                          uint16_t* __restrict__ nxt, bool issue_next,
                                          const uint16_t* qb, const uint16_t* db,
                                          const float* lseb, const float* delb, int rs, int T,
                                          int qt, int ka, int kj, int w, float sl2,
                                          const uint4 (&kf)[D / 16], const uint4 (&vf)[D / 16],
                                          f32x16 (&dkacc)[D / 32], f32x16 (&dvacc)[D / 32],
                                          int wave, int lane) {
  constexpr int BQ = kBwdBQ, DK = D / 16, MB = D / 32, QB = BQ / 32, TILE = DkdvStage<D>::TILE;
  const int half = lane >> 5, l32 = lane & 31;
  if (issue_next) dkdv_issue<D, NW>(qb, db, lseb, delb, rs, qt + 1, T, nxt, wave, lane);
  const uint16_t* sQ = cur;
  const uint16_t* sO = cur + TILE;
  const float* sL = reinterpret_cast<const float*>(cur + 2 * TILE);
  const float* sDl = sL + BQ;
#pragma unroll
  for (int qb2 = 0; qb2 < QB; ++qb2) {
    const int qs = qt * BQ + 32 * qb2, qz = qs + 31, kz = ka + 31;
    if (ka >= T || qz < ka || qs - kz >= w || qs >= T) continue;
    const bool need_mask = !(qs >= kz && qz - ka < w && qz < T);
    f32x16 s = zero16(), dp = zero16();
    const int row = 32 * qb2 + l32;
#pragma unroll
    for (int t = 0; t < DK; ++t) {
      s = mfma32(row_chunk<D>(sQ, row, 2 * t + half), kf[t], s);
      dp = mfma32(row_chunk<D>(sO, row, 2 * t + half), vf[t], dp);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ql0 = 32 * qb2 + 8 * j + 4 * half;
      const float4 l4 = *reinterpret_cast<const float4*>(sL + ql0);
      const float4 d4 = *reinterpret_cast<const float4*>(sDl + ql0);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
      const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * j + i;
        float pr = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -lv[i] * kLog2e));
        if (need_mask) {
          const int qg = qt * BQ + ql0 + i;
          if (kj > qg || qg - kj >= w || qg >= T) pr = 0.f;
        }
        s[r] = pr;
        dp[r] = pr * (dp[r] - dv[i]);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint4 pf = pack_frag(s, u);
      const uint4 dsf = pack_frag(dp, u);
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        dvacc[m] = mfma32(tr_frag<D>(sO, 32 * qb2 + 16 * u, m, lane), pf, dvacc[m]);
        dkacc[m] = mfma32(tr_frag<D>(sQ, 32 * qb2 + 16 * u, m, lane), dsf, dkacc[m]);
      }
    }
  }
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 1) void bwd_dkdv_kernel(BwdArgs p) {
  constexpr int BK = 32 * NW, BQ = kBwdBQ;
  constexpr int DK = D / 16, MB = D / 32, SE = DkdvStage<D>::ELEMS;

  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * SE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
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

  const int ka = k0 + 32 * wave;
  const int kj = ka + l32;
  const bool kvalid = kj < T;
  uint4 kf[DK], vf[DK];
#pragma unroll
  for (int t = 0; t < DK; ++t) {
    const int64_t off = base + (int64_t)kj * rs + 16 * t + 8 * half;
    kf[t] = kvalid ? ldg16(p.k + off) : make_uint4(0, 0, 0, 0);
    vf[t] = kvalid ? ldg16(p.v + off) : make_uint4(0, 0, 0, 0);
  }
  f32x16 dkacc[MB], dvacc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    dkacc[m] = zero16();
    dvacc[m] = zero16();
  }

  uint16_t* stage0 = smem;
  uint16_t* stage1 = smem + SE;
  for (int qt = qt_begin; qt <= qt_end; ++qt) {
    wait_vmcnt<0>();
    __syncthreads();
    const bool even = ((qt - qt_begin) & 1) == 0;
    dkdv_step<D, NW>(even ? stage0 : stage1, even ? stage1 : stage0, qt < qt_end, qb, db, lseb,
                     delb, rs, T, qt, ka, kj, w, p.scale_log2, kf, vf, dkacc, dvacc, wave, lane);
  }

  if (!kvalid) return;
  const float sc = p.scale;
  uint16_t* dko = p.dk + base + (int64_t)kj * rs;
  uint16_t* dvo = p.dv + base + (int64_t)kj * rs;
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint2 a, c;
      a.x = pack_bf16x2(dkacc[m][4 * j + 0] * sc, dkacc[m][4 * j + 1] * sc);
      a.y = pack_bf16x2(dkacc[m][4 * j + 2] * sc, dkacc[m][4 * j + 3] * sc);
      c.x = pack_bf16x2(dvacc[m][4 * j + 0], dvacc[m][4 * j + 1]);
      c.y = pack_bf16x2(dvacc[m][4 * j + 2], dvacc[m][4 * j + 3]);
      *reinterpret_cast<uint2*>(dko + m * 32 + 8 * j + 4 * half) = a;
      *reinterpret_cast<uint2*>(dvo + m * 32 + 8 * j + 4 * half) = c;
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
  constexpr int NW = 4;
  BwdArgs p = a;
  p.n_tiles = (p.T + 32 * NW - 1) / (32 * NW);
  const unsigned grid = (unsigned)p.n_tiles * (unsigned)p.BH;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW>), dim3(grid), dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t s) {
  return a.D == 64 ? launch_dq_d<64>(a, s) : launch_dq_d<128>(a, s);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t s) {
  return a.D == 64 ? launch_dkdv_d<64>(a, s) : launch_dkdv_d<128>(a, s);
}

}  // namespace swattn
