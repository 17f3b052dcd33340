// Engine decode and KV-cache append for gfx950.
//
// Operation: the Engine's decode phase over its KV cache (followin.io walkthrough, section
// "Pretraining", Engine paragraph; nanochat launch post, feature list): each sequence's one new
// query attends to cache rows max(0, p - w + 1) .. p with p = L - 1, where L counts the cached
// tokens including the new one.
//
// Design: decode is a matrix-vector product per (sequence, head) -- about one flop per byte of
// cache -- so it is HBM-bound and uses VALU dot products, not MFMA.  The visible key range is
// split into 64-key chunks; a wave issues all of one chunk's K and V loads (16-byte, D/8 lanes per
// key row) before using any of them and reduces q.k over the row's lanes with DPP.  Two schedules:
//   one workgroup per (sequence, head), chunks dealt to its 8 waves, partial results merged in
//   LDS (decode_fused_kernel, one launch, no workspace) -- the usual case;
//   few pairs over long caches (decode_uses_fused): one wave per (head, chunk, sequence) writes
//   its chunk's (max, sum, unnormalised output) to the workspace and a second kernel merges the
//   chunks.
// Both merge with the log-sum-exp rule and write O (bf16) and LSE.
//
// Decode step (STEP): the same kernels also append the step's new key / value row at pos[b] and
// attend over rows .. pos[b].  The chunk ending at the new row takes that row's key / value from
// the new-row inputs instead of the cache, and one wave copies the row into the cache after its
// own loads, so no launch reads a cache row written in the same launch.
#include <mutex>

#include "common.h"
#include "launch.h"

namespace swattn {

// Scratch of the allocation-free decode step.  In host code `scratch` names a host-side stand-in,
// not device memory: only the address that hipGetSymbolAddress returns for the current device is
// ever passed to a kernel.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of N lanes (N in {8, 16}); every lane of the group receives the sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N == 16) {
    x += dpp_f<0x128>(x);  // row_ror:8
    x += dpp_f<0x124>(x);  // row_ror:4
    x += dpp_f<0x122>(x);  // row_ror:2
    x += dpp_f<0x121>(x);  // row_ror:1
  } else {
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 1);
  }
  return x;
}

// Cache rows the query of sequence b sees the end of: a decode clamps lens to [0, Lcap]; a decode
// step appends at pos (valid in [0, Lcap)) and sees pos + 1 rows, or none for an invalid pos.
template <bool STEP>
__device__ __forceinline__ int dec_len(const DecArgs& p, int b) {
  if (STEP) {
    const int ps = p.pos[b];
    return (ps >= 0 && ps < p.Lcap) ? ps + 1 : 0;
  }
  return min(max(p.lens[b], 0), p.Lcap);
}

// K and V rows of the decode step's last 64-key chunk, which ends at the new row L - 1: that row's
// key / value come from the new-row inputs; rows past ce re-read row ce - 1 (masked later).
template <int D>
__device__ __forceinline__ void dec_load_chunk(const DecArgs& p, const uint16_t* kb,
                                               const uint16_t* vb, int64_t rowstride, int b, int h,
                                               int cs, int ce, int L, int kq, int dc,
                                               uint4 (&kr)[kDecodeChunk / (64 / (D / 8))],
                                               uint4 (&vr)[kDecodeChunk / (64 / (D / 8))]) {
  constexpr int KPI = 64 / (D / 8), NL = kDecodeChunk / KPI;
  const int64_t nrow = ((int64_t)b * p.H + h) * D + 8 * dc;
#pragma unroll
  for (int r = 0; r < NL; ++r) {
    const int j = min(cs + r * KPI + kq, ce - 1);
    const uint16_t* ks = kb + j * rowstride;
    const uint16_t* vs = vb + j * rowstride;
    if (j == L - 1) {
      ks = p.kn + nrow;
      vs = p.vn + nrow;
    }
    kr[r] = ldg16_stream(ks);
    vr[r] = ldg16_stream(vs);
  }
}

// Decode step: the new row of head h of sequence b (16 bytes per lane over lanes 0 .. D / 8 - 1)
// is loaded when a kernel starts, without waiting, and written to cache row L - 1 after the
// kernel's own loads, so the copy adds no wait to the attention.
template <int D>
struct NewRow {
  uint4 k, v;
  bool mine;
  __device__ __forceinline__ void load(const DecArgs& p, int b, int h, int lane, bool owner) {
    mine = owner && lane < D / 8;
    if (mine) {
      const int64_t src = ((int64_t)b * p.H + h) * D + 8 * lane;
      k = ldg16(p.kn + src);
      v = ldg16(p.vn + src);
    }
  }
  __device__ __forceinline__ void store(const DecArgs& p, int b, int h, int L, int lane) const {
    if (!mine) return;
    const int64_t dst = (((int64_t)b * p.Lcap + (L - 1)) * p.H + h) * D + 8 * lane;
    *reinterpret_cast<uint4*>(p.kcw + dst) = k;
    *reinterpret_cast<uint4*>(p.vcw + dst) = v;
  }
};

template <int D, bool STEP>
__global__ __launch_bounds__(64) void decode_split_kernel(DecArgs p) {
  constexpr int LPK = D / 8;      // lanes per key row (16 bytes each)
  constexpr int KPI = 64 / LPK;   // key rows per load instruction
  constexpr int C = kDecodeChunk;
  constexpr int NL = C / KPI;     // loads per lane per tensor

  const int h = blockIdx.x, c = blockIdx.y, b = blockIdx.z;  // heads fastest: adjacent bytes
  const int L = dec_len<STEP>(p, b);
  if (L == 0) return;
  const int nvis = min(p.window, L);
  const int j0 = L - nvis;
  const int nc = (nvis + C - 1) / C;
  if (c >= nc) return;
  const int cs = j0 + c * C;
  const int ce = min(cs + C, L);

  const int lane = threadIdx.x;
  const int kq = lane / LPK, dc = lane % LPK;
  const int64_t rowstride = (int64_t)p.H * D;
  const uint16_t* kb = p.kc + ((int64_t)b * p.Lcap) * rowstride + h * D + 8 * dc;
  const uint16_t* vb = p.vc + ((int64_t)b * p.Lcap) * rowstride + h * D + 8 * dc;

  NewRow<D> nr;
  if (STEP) nr.load(p, b, h, lane, c == nc - 1);
  uint4 kr[NL], vr[NL];
  if (STEP && c == nc - 1) {  // the chunk ending at the new row
    dec_load_chunk<D>(p, kb, vb, rowstride, b, h, cs, ce, L, kq, dc, kr, vr);
  } else {
#pragma unroll
    for (int r = 0; r < NL; ++r) {
      const int j = cs + r * KPI + kq;
      if (j < ce) {
        kr[r] = ldg16_stream(kb + j * rowstride);
        vr[r] = ldg16_stream(vb + j * rowstride);
      } else {
        kr[r] = make_uint4(0, 0, 0, 0);
        vr[r] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  float qv[8];
  {
    const uint4 qq = ldg16(p.q + ((int64_t)b * p.H + h) * D + 8 * dc);
    const uint32_t* qw = reinterpret_cast<const uint32_t*>(&qq);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[2 * e] = bf16_lo(qw[e]) * p.scale_log2;
      qv[2 * e + 1] = bf16_hi(qw[e]) * p.scale_log2;
    }
  }

  float sc[NL];
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < NL; ++r) {
    const uint32_t* kw = reinterpret_cast<const uint32_t*>(&kr[r]);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(qv[2 * e], bf16_lo(kw[e]), acc);
      acc = fmaf(qv[2 * e + 1], bf16_hi(kw[e]), acc);
    }
    acc = group_sum<LPK>(acc);
    const int j = cs + r * KPI + kq;
    sc[r] = (j < ce) ? acc : -INFINITY;
    mx = fmaxf(mx, sc[r]);
  }
  // chunk max over all key rows (groups of LPK lanes differ in kq)
#pragma unroll
  for (int off = LPK; off < 32; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  mx = max_with_partner(mx);

  float lsum = 0.f;
  float ov[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ov[e] = 0.f;
#pragma unroll
  for (int r = 0; r < NL; ++r) {
    const float pr = __builtin_amdgcn_exp2f(sc[r] - mx);
    lsum += pr;
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(&vr[r]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ov[2 * e] = fmaf(pr, bf16_lo(vw[e]), ov[2 * e]);
      ov[2 * e + 1] = fmaf(pr, bf16_hi(vw[e]), ov[2 * e + 1]);
    }
  }
  if (STEP) nr.store(p, b, h, L, lane);
  // reduce over the key-row groups: lanes with equal dc
#pragma unroll
  for (int off = LPK; off < 32; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] += __shfl_xor(ov[e], off);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) ov[e] = sum_with_partner(ov[e]);
  // lsum: each group of LPK lanes holds the same partial (one per kq); count it once per group
  lsum = (dc == 0) ? lsum : 0.f;
  for (int off = 1; off < 32; off <<= 1) lsum += __shfl_xor(lsum, off);
  lsum = sum_with_partner(lsum);

  const int64_t slot = ((int64_t)b * p.H + h) * p.nc_max + c;
  if (kq == 0) {
    float4* dst = reinterpret_cast<float4*>(p.ws_o + slot * D + 8 * dc);
    dst[0] = make_float4(ov[0], ov[1], ov[2], ov[3]);
    dst[1] = make_float4(ov[4], ov[5], ov[6], ov[7]);
  }
  if (lane == 0) {
    p.ws_ml[2 * slot] = mx;
    p.ws_ml[2 * slot + 1] = lsum;
  }
}

// Merge of the split schedule, one workgroup per (sequence, head).  A long cache leaves hundreds
// of partial results per pair, so the threads share them out: D / 4 threads cover one chunk's
// features (a float4 each) and the workgroup's rows of threads take every R-th chunk, with the
// rows' sums meeting in LDS.
constexpr int kCombineThreads = 256;

template <int D, bool STEP>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecArgs p) {
  constexpr int F4 = D / 4;                // threads per chunk row
  constexpr int R = kCombineThreads / F4;  // chunk rows
  constexpr int NWV = kCombineThreads / 64;
  __shared__ float s_max[NWV];
  __shared__ float4 s_o[R][F4];
  __shared__ float s_l[R];
  const int bh = blockIdx.x;
  const int b = bh / p.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = dec_len<STEP>(p, b);
  uint16_t* ob = p.o + (int64_t)bh * D;
  if (L == 0) {
    if (tid < D) ob[tid] = 0;
    if (p.lse && tid == 0) p.lse[bh] = -INFINITY;
    return;
  }
  const int nvis = min(p.window, L);
  const int nc = (nvis + kDecodeChunk - 1) / kDecodeChunk;
  const int64_t slot0 = (int64_t)bh * p.nc_max;
  // M: the largest chunk maximum (every chunk holds a visible key, so M is finite)
  float m = -INFINITY;
  for (int c = tid; c < nc; c += kCombineThreads) m = fmaxf(m, p.ws_ml[2 * (slot0 + c)]);
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
  m = max_with_partner(m);
  if (lane == 0) s_max[wave] = m;
  __syncthreads();
  float M = s_max[0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) M = fmaxf(M, s_max[w]);
  // this thread's four features summed over its row's chunks, each weighted by 2^(m_c - M)
  const int f = tid % F4, row = tid / F4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float ls = 0.f;
#pragma unroll 4  // four chunks' loads in flight per thread (8-13% faster over 16384 rows)
  for (int c = row; c < nc; c += R) {
    const float2 ml = *reinterpret_cast<const float2*>(p.ws_ml + 2 * (slot0 + c));
    const float wgt = __builtin_amdgcn_exp2f(ml.x - M);
    ls = fmaf(ml.y, wgt, ls);
    const float4 o4 = *reinterpret_cast<const float4*>(p.ws_o + (slot0 + c) * D + 4 * f);
    acc.x = fmaf(o4.x, wgt, acc.x);
    acc.y = fmaf(o4.y, wgt, acc.y);
    acc.z = fmaf(o4.z, wgt, acc.z);
    acc.w = fmaf(o4.w, wgt, acc.w);
  }
  s_o[row][f] = acc;
  if (f == 0) s_l[row] = ls;
  __syncthreads();
  if (tid >= F4) return;
  float4 a = s_o[0][tid];
  float Ls = s_l[0];
#pragma unroll
  for (int r = 1; r < R; ++r) {
    const float4 o4 = s_o[r][tid];
    a.x += o4.x;
    a.y += o4.y;
    a.z += o4.z;
    a.w += o4.w;
    Ls += s_l[r];
  }
  const float inv = 1.f / Ls;
  uint2 st;
  st.x = pack_bf16x2(a.x * inv, a.y * inv);
  st.y = pack_bf16x2(a.z * inv, a.w * inv);
  *reinterpret_cast<uint2*>(ob + 4 * tid) = st;
  if (p.lse && tid == 0) p.lse[bh] = (M + __log2f(Ls)) * kLn2;
}

// One workgroup of NW waves per (sequence, head): the visible key range is split into 64-key chunks
// dealt round-robin to the waves (split-K inside the workgroup); each wave keeps a running online
// softmax over its chunks, and the NW partial results are merged in LDS with the log-sum-exp rule.
// Used when there are enough (sequence, head) pairs to fill the GPU; no workspace is touched.
template <int D, int NW, bool STEP>
__global__ __launch_bounds__(64 * NW) void decode_fused_kernel(DecArgs p) {
  constexpr int LPK = D / 8, KPI = 64 / LPK, C = kDecodeChunk, NL = C / KPI;
  __shared__ float s_o[NW][D];
  __shared__ float s_ml[NW][2];

  const int bh = blockIdx.x;  // consecutive workgroups: consecutive heads, adjacent bytes
  const int b = bh / p.H, h = bh % p.H;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int L = dec_len<STEP>(p, b);
  uint16_t* ob = p.o + (int64_t)bh * D;
  if (L == 0) {
    for (int d = threadIdx.x; d < D; d += 64 * NW) ob[d] = 0;
    if (p.lse && threadIdx.x == 0) p.lse[bh] = -INFINITY;
    return;
  }
  const int nvis = min(p.window, L);
  const int j0 = L - nvis;
  const int nc = (nvis + C - 1) / C;

  const int kq = lane / LPK, dc = lane % LPK;
  const int64_t rowstride = (int64_t)p.H * D;
  const uint16_t* kb = p.kc + ((int64_t)b * p.Lcap) * rowstride + h * D + 8 * dc;
  const uint16_t* vb = p.vc + ((int64_t)b * p.Lcap) * rowstride + h * D + 8 * dc;
  float qv[8];
  {
    const uint4 qq = ldg16(p.q + (int64_t)bh * D + 8 * dc);
    const uint32_t* qw = reinterpret_cast<const uint32_t*>(&qq);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[2 * e] = bf16_lo(qw[e]) * p.scale_log2;
      qv[2 * e + 1] = bf16_hi(qw[e]) * p.scale_log2;
    }
  }
  NewRow<D> nr;
  if (STEP) nr.load(p, b, h, lane, wave == NW - 1);
  float m_run = -INFINITY, l_run = 0.f;  // l_run: this lane's key rows only
  float ov[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ov[e] = 0.f;

  for (int c = wave; c < nc; c += NW) {
    const int cs = j0 + c * C;
    const int ce = min(cs + C, L);
    uint4 kr[NL], vr[NL];
    if (STEP && c == nc - 1) {  // the chunk ending at the new row
      dec_load_chunk<D>(p, kb, vb, rowstride, b, h, cs, ce, L, kq, dc, kr, vr);
    } else {
#pragma unroll
      for (int r = 0; r < NL; ++r) {
        const int j = min(cs + r * KPI + kq, ce - 1);  // rows past the chunk re-read a valid row
        kr[r] = ldg16_stream(kb + j * rowstride);
        vr[r] = ldg16_stream(vb + j * rowstride);
      }
    }
    float sc[NL];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < NL; ++r) {
      const uint32_t* kw = reinterpret_cast<const uint32_t*>(&kr[r]);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(qv[2 * e], bf16_lo(kw[e]), acc);
        acc = fmaf(qv[2 * e + 1], bf16_hi(kw[e]), acc);
      }
      acc = group_sum<LPK>(acc);
      sc[r] = (cs + r * KPI + kq < ce) ? acc : -INFINITY;
      mx = fmaxf(mx, sc[r]);
    }
#pragma unroll
    for (int off = LPK; off < 32; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    mx = max_with_partner(mx);
    const float m_new = fmaxf(m_run, mx);  // finite: every chunk holds a visible key
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int r = 0; r < NL; ++r) {
      const float pr = __builtin_amdgcn_exp2f(sc[r] - m_new);
      l_run += pr;
      const uint32_t* vw = reinterpret_cast<const uint32_t*>(&vr[r]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ov[2 * e] = fmaf(pr, bf16_lo(vw[e]), ov[2 * e]);
        ov[2 * e + 1] = fmaf(pr, bf16_hi(vw[e]), ov[2 * e + 1]);
      }
    }
  }
  if (STEP) nr.store(p, b, h, L, lane);
  // this wave's partial: sum over the key-row groups (lanes with equal dc)
#pragma unroll
  for (int off = LPK; off < 32; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] += __shfl_xor(ov[e], off);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) ov[e] = sum_with_partner(ov[e]);
  float lsum = (dc == 0) ? l_run : 0.f;
  for (int off = 1; off < 32; off <<= 1) lsum += __shfl_xor(lsum, off);
  lsum = sum_with_partner(lsum);
  if (kq == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s_o[wave][8 * dc + e] = ov[e];
  }
  if (lane == 0) {
    s_ml[wave][0] = m_run;  // -inf for a wave that got no chunk
    s_ml[wave][1] = lsum;
  }
  __syncthreads();
  if (wave != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, s_ml[w][0]);
  float wt[NW], Ls = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    wt[w] = (s_ml[w][0] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_ml[w][0] - M);
    Ls = fmaf(s_ml[w][1], wt[w], Ls);
  }
  const float inv = 1.f / Ls;
  for (int d = lane; d < D; d += 64) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) a = fmaf(s_o[w][d], wt[w], a);
    ob[d] = __builtin_bit_cast(uint16_t, (__bf16)(a * inv));
  }
  if (p.lse && lane == 0) p.lse[bh] = (M + __log2f(Ls)) * kLn2;
}

__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs p) {
  const int chunks = p.D / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)p.B * p.H * chunks) return;
  const int c = (int)(idx % chunks);
  const int bh = (int)(idx / chunks);
  const int b = bh / p.H, h = bh % p.H;
  const int pos = p.pos[b];
  if (pos < 0 || pos >= p.Lcap) return;
  const int64_t dst = (((int64_t)b * p.Lcap + pos) * p.H + h) * p.D + 8 * c;
  const int64_t src = (int64_t)bh * p.D + 8 * c;
  *reinterpret_cast<uint4*>(p.kc + dst) = ldg16(p.kn + src);
  *reinterpret_cast<uint4*>(p.vc + dst) = ldg16(p.vn + src);
}

template <int D, bool STEP>
static hipError_t launch_decode_d(const DecArgs& a, hipStream_t s) {
  if (decode_uses_fused(a.B, a.H, a.Lcap, a.window)) {
    hipLaunchKernelGGL((decode_fused_kernel<D, 8, STEP>), dim3(a.B * a.H), dim3(512), 0, s, a);
    return hipGetLastError();
  }
  const int vis_max = a.window < a.Lcap ? a.window : a.Lcap;
  const int nc = (vis_max + kDecodeChunk - 1) / kDecodeChunk;
  hipLaunchKernelGGL((decode_split_kernel<D, STEP>), dim3(a.H, nc, a.B), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D, STEP>), dim3(a.B * a.H), dim3(kCombineThreads), 0,
                     s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecArgs& a, hipStream_t s) {
  if (a.pos)
    return a.D == 64 ? launch_decode_d<64, true>(a, s) : launch_decode_d<128, true>(a, s);
  return a.D == 64 ? launch_decode_d<64, false>(a, s) : launch_decode_d<128, false>(a, s);
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.H * (a.D / 8);
  const unsigned grid = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(kv_append_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace swattn
