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
// in-window key tiles: S^T = K Q^T, dP^T = V dO^T, dS^T, and dQ^T += K^T dS^T with K^T stored
// transposed in LDS.
// dK/dV pass: a workgroup owns NW x 32 keys (K, V in registers, lane = key) and walks the query
// tiles that can see them: S = Q K^T, dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS with
// dO^T and Q^T stored transposed in LDS.
#include "common.h"
#include "launch.h"

namespace swattn {

constexpr int kBwdBC = 64;  // keys per tile in the dQ pass
constexpr int kBwdBQ = 64;  // queries per tile in the dK/dV pass

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_dq_kernel(BwdArgs p) {
  constexpr int BR = 32 * NW, BC = kBwdBC, NT = 64 * NW;
  constexpr int DK = D / 16, MB = D / 32, NB = BC / 32;
  constexpr int GROUPS = (BC / 4) * (D / 8);
  constexpr int ITEMS = (GROUPS + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) uint16_t sK[BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t sKt[D * BC];
  __shared__ __attribute__((aligned(16))) uint16_t sV[BC * D];

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
  const uint16_t* qb = p.q + base;
  const uint16_t* kb = p.k + base;
  const uint16_t* vb = p.v + base;

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
  const float sl2 = p.scale_log2;

  f32x16 dqacc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) dqacc[m] = zero16();

  uint4 kr[ITEMS][4], vr[ITEMS][4];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int idx = tid + it * NT;
      if (idx < GROUPS) {
        const int g = idx / (D / 8), c = idx % (D / 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = kt * BC + 4 * g + i;
          if (j < T) {
            kr[it][i] = ldg16(kb + (int64_t)j * rs + 8 * c);
            vr[it][i] = ldg16(vb + (int64_t)j * rs + 8 * c);
          } else {
            kr[it][i] = make_uint4(0, 0, 0, 0);
            vr[it][i] = make_uint4(0, 0, 0, 0);
          }
        }
      }
    }
  };

  load_tile(kt_begin);
  for (int kt = kt_begin; kt <= kt_end; ++kt) {
    if (kt != kt_begin) __syncthreads();
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int idx = tid + it * NT;
      if (idx < GROUPS) {
        const int g = idx / (D / 8), c = idx % (D / 8);
        store_group<D, BC, true, true>(sK, sKt, g, c, kr[it]);
        store_group<D, BC, true, false>(sV, nullptr, g, c, vr[it]);
      }
    }
    __syncthreads();
    if (kt < kt_end) load_tile(kt + 1);

    const int k_lo = kt * BC, k_hi = k_lo + BC - 1, qz = qa + 31;
    if ((qa >= T) || (k_lo > qz) || (qa - k_hi >= w)) continue;
    const bool need_mask = !(k_hi <= qa && qz - k_lo < w);

    f32x16 s[NB], dp[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      s[nb] = zero16();
      dp[nb] = zero16();
      const int row = nb * 32 + l32;
#pragma unroll
      for (int t = 0; t < DK; ++t) {
        const int off = normal_off<D>(row, 2 * t + half);
        s[nb] = mfma32(*reinterpret_cast<const uint4*>(sK + off), qf[t], s[nb]);
        dp[nb] = mfma32(*reinterpret_cast<const uint4*>(sV + off), df[t], dp[nb]);
      }
    }
    uint4 dsf[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = __builtin_amdgcn_exp2f(s[nb][r] * sl2 - lse2);
        if (need_mask) {
          const int key = k_lo + nb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key > qi || qi - key >= w) pr = 0.f;
        }
        s[nb][r] = pr * (dp[nb][r] - delta);
      }
      dsf[nb][0] = pack_frag(s[nb], 0);
      dsf[nb][1] = pack_frag(s[nb], 1);
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int d = m * 32 + l32;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint4 a =
              *reinterpret_cast<const uint4*>(sKt + trans_off<BC>(d, 2 * (2 * nb + u) + half));
          dqacc[m] = mfma32(a, dsf[nb][u], dqacc[m]);
        }
    }
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

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_dkdv_kernel(BwdArgs p) {
  constexpr int BK = 32 * NW, BQ = kBwdBQ, NT = 64 * NW;
  constexpr int DK = D / 16, MB = D / 32, QB = BQ / 32;
  constexpr int GROUPS = (BQ / 4) * (D / 8);
  constexpr int ITEMS = (GROUPS + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) uint16_t sQ[BQ * D];
  __shared__ __attribute__((aligned(16))) uint16_t sQt[D * BQ];
  __shared__ __attribute__((aligned(16))) uint16_t sO[BQ * D];   // dO, row-major
  __shared__ __attribute__((aligned(16))) uint16_t sOt[D * BQ];  // dO, transposed
  __shared__ float sL[BQ];
  __shared__ float sDl[BQ];

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
  const float sl2 = p.scale_log2;

  uint4 qr[ITEMS][4], dr[ITEMS][4];
  float lr = 0.f, dl = 0.f;
  auto load_tile = [&](int qt) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int idx = tid + it * NT;
      if (idx < GROUPS) {
        const int g = idx / (D / 8), c = idx % (D / 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = qt * BQ + 4 * g + i;
          if (j < T) {
            qr[it][i] = ldg16(qb + (int64_t)j * rs + 8 * c);
            dr[it][i] = ldg16(db + (int64_t)j * rs + 8 * c);
          } else {
            qr[it][i] = make_uint4(0, 0, 0, 0);
            dr[it][i] = make_uint4(0, 0, 0, 0);
          }
        }
      }
    }
    if (tid < BQ) {
      const int j = qt * BQ + tid;
      lr = j < T ? lseb[j] * kLog2e : INFINITY;  // +inf makes P = 0 for rows past T
      dl = j < T ? delb[j] : 0.f;
    }
  };

  load_tile(qt_begin);
  for (int qt = qt_begin; qt <= qt_end; ++qt) {
    if (qt != qt_begin) __syncthreads();
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int idx = tid + it * NT;
      if (idx < GROUPS) {
        const int g = idx / (D / 8), c = idx % (D / 8);
        store_group<D, BQ, true, true>(sQ, sQt, g, c, qr[it]);
        store_group<D, BQ, true, true>(sO, sOt, g, c, dr[it]);
      }
    }
    if (tid < BQ) {
      sL[tid] = lr;
      sDl[tid] = dl;
    }
    __syncthreads();
    if (qt < qt_end) load_tile(qt + 1);

#pragma unroll
    for (int qb2 = 0; qb2 < QB; ++qb2) {
      const int qs = qt * BQ + 32 * qb2, qz = qs + 31, kz = ka + 31;
      if (ka >= T || qz < ka || qs - kz >= w) continue;
      const bool need_mask = !(qs >= kz && qz - ka < w && qz < T);
      f32x16 s = zero16(), dp = zero16();
      const int row = 32 * qb2 + l32;
#pragma unroll
      for (int t = 0; t < DK; ++t) {
        const int off = normal_off<D>(row, 2 * t + half);
        s = mfma32(*reinterpret_cast<const uint4*>(sQ + off), kf[t], s);
        dp = mfma32(*reinterpret_cast<const uint4*>(sO + off), vf[t], dp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = 32 * qb2 + 8 * (r >> 2) + 4 * half + (r & 3);
        float pr = __builtin_amdgcn_exp2f(s[r] * sl2 - sL[ql]);
        if (need_mask) {
          const int qg = qt * BQ + ql;
          if (kj > qg || qg - kj >= w) pr = 0.f;
        }
        s[r] = pr;
        dp[r] = pr * (dp[r] - sDl[ql]);
      }
      uint4 pf[2], dsf[2];
      pf[0] = pack_frag(s, 0);
      pf[1] = pack_frag(s, 1);
      dsf[0] = pack_frag(dp, 0);
      dsf[1] = pack_frag(dp, 1);
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const int d = m * 32 + l32;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int off = trans_off<BQ>(d, 2 * (2 * qb2 + u) + half);
          dvacc[m] = mfma32(*reinterpret_cast<const uint4*>(sOt + off), pf[u], dvacc[m]);
          dkacc[m] = mfma32(*reinterpret_cast<const uint4*>(sQt + off), dsf[u], dkacc[m]);
        }
      }
    }
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
