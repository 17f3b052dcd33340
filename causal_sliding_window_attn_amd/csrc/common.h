// Device-side building blocks shared by the attention kernels (gfx950 / CDNA4, wave64).
//
// MFMA fragment conventions used everywhere (v_mfma_f32_32x32x16_bf16):
//   A operand (32 x 16): lane l holds row (l % 32) and 8 consecutive k-slots of half (l / 32).
//   B operand (16 x 32): lane l holds column (l % 32) and the same 8 k-slots of half (l / 32).
//   C (32 x 32, fp32):   lane l holds column (l % 32); accumulator r holds row
//                        8 * (r / 4) + 4 * (l / 32) + (r % 4).
// The hardware sums over (half, slot); which logical k a slot stands for is our choice, as long
// as A and B agree.  We exploit that twice: contraction over D uses slot s of half h = element
// 8h + s of a 16-wide chunk, and contraction over the sequence reuses the C layout of a previous
// product directly as the B operand (slot s of half h = row 8 * (s / 4) + 4h + (s % 4) of a
// 16-row step), with the other operand's LDS copy laid out in the same permuted order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Round-to-nearest-even fp32 -> bf16 pair (hardware v_cvt_pk_bf16_f32), packed in 32 bits.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Eight fp32 values (accumulator slots 8u .. 8u+7) -> one bf16x8 B-operand fragment.
__device__ __forceinline__ uint4 pack_frag(const f32x16& acc, int u) {
  uint4 r;
  r.x = pack_bf16x2(acc[8 * u + 0], acc[8 * u + 1]);
  r.y = pack_bf16x2(acc[8 * u + 2], acc[8 * u + 3]);
  r.z = pack_bf16x2(acc[8 * u + 4], acc[8 * u + 5]);
  r.w = pack_bf16x2(acc[8 * u + 6], acc[8 * u + 7]);
  return r;
}

// Eight fp32 values -> two bf16x8 fragments hi + lo with hi = x truncated to bf16 (one v_perm per
// pair) and lo = bf16(x - hi): x - hi is exact in fp32, so hi + lo carries x to about 2^-16
// relative (one bf16 alone keeps only 2^-9).
__device__ __forceinline__ void pack_frag_split(const f32x16& acc, int u, uint4& hi, uint4& lo) {
  uint32_t* h = reinterpret_cast<uint32_t*>(&hi);
  uint32_t* l = reinterpret_cast<uint32_t*>(&lo);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = acc[8 * u + 2 * e], b = acc[8 * u + 2 * e + 1];
    const uint32_t ab = __float_as_uint(a), bb = __float_as_uint(b);
    h[e] = __builtin_amdgcn_perm(bb, ab, 0x07060302u);  // upper halves of a (low) and b (high)
    l[e] = pack_bf16x2(a - __uint_as_float(ab & 0xffff0000u), b - __uint_as_float(bb & 0xffff0000u));
  }
}

// v_permlane32_swap(x, x) returns {x of lanes 0-31 | x of lane l-32, x of lane l+32 | x of lanes
// 32-63}: each lane sees its own value in one slot and lane (l ^ 32)'s in the other.
__device__ __forceinline__ float max_with_partner(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}

__device__ __forceinline__ float sum_with_partner(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// A 16-byte load of data that is read once and never again by the same launch (the KV cache in a
// decode): nontemporal, so that it streams through the caches without displacing reused lines.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16_stream(const uint16_t* p) {
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

// ---------------------------------------------------------------------------------------------
// Direct global -> LDS tile streaming (buffer_load_dwordx4 ... lds, global_load_lds_dwordx4) and
// transposed LDS reads (ds_read_b64_tr_b16), with the lane semantics measured on gfx950:
//   16-byte LDS DMA (either form): lane l's 16 bytes land at (wave-uniform LDS base) + 16 * l.
//   ds_read_tr16_b64: within each group of 16 lanes, lane i receives in slot j element (i % 4) of
//   the 8-byte row addressed by lane 4 * j + i / 4 of that group.
// ---------------------------------------------------------------------------------------------
#define SWATTN_AS3 __attribute__((address_space(3)))
#define SWATTN_AS1 __attribute__((address_space(1)))
typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void g2lds16(const uint16_t* gsrc, uint16_t* lds_base) {
  __builtin_amdgcn_global_load_lds((const SWATTN_AS1 void*)gsrc, (SWATTN_AS3 void*)lds_base, 16, 0,
                                   0);
}

__device__ __forceinline__ void g2lds4(const float* gsrc, float* lds_base) {
  __builtin_amdgcn_global_load_lds((const SWATTN_AS1 void*)gsrc, (SWATTN_AS3 void*)lds_base, 4, 0,
                                   0);
}

__device__ __forceinline__ uint2 lds_tr16(const uint16_t* p) {
  v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SWATTN_AS3 v4i16*)p);
  return __builtin_bit_cast(uint2, r);
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt / lgkmcnt left open).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS-only hand-off between waves: waits for this wave's LDS accesses, then
// s_barrier.  Unlike __syncthreads it carries no release fence, so it does not drain LDS DMA still
// in flight to another stage.  The "memory" clobber keeps the compiler from moving memory
// operations across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Physical 16-byte chunk of logical chunk c in row r of a row-major [rows][D] bf16 tile.  One
// swizzle serves both ways a tile is read:
//   row reads (ds_read_b128, 32 consecutive rows, one chunk each): the XOR term is a bijection over
//   every 16 rows (D = 128) or over the 8 rows of one 256-byte bank parity (D = 64);
//   transposed reads (ds_read_b64_tr_b16, 4 consecutive rows x 64 bytes per 32 lanes): the 4 rows
//   land in 4 different 64-byte bank segments.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  return D == 128 ? (c ^ (4 * (r & 3) + ((r >> 2) & 3)))
                  : (c ^ (4 * ((r >> 1) & 1) + ((r >> 2) & 3)));
}

// Word 3 of a raw buffer resource on gfx950: 32-bit data format, byte offsets, and loads at or past
// num_records bytes return zero.
constexpr int kRawBufferWord3 = 0x00020000;

// Plan for streaming ROWS consecutive rows of a [*, rs]-strided bf16 tensor into a row-major
// swizzled LDS tile with buffer_load_dwordx4 ... lds, NW waves sharing the work (one 1 KB
// instruction per wave each).  Each lane's byte offset inside a tile is the same for every tile, so
// the offsets are computed once; a tile then costs a scalar resource (its first row and its valid
// byte count) and no vector arithmetic.  Rows at or past `nvalid` fall outside the resource's range
// and land as zeros; every load stays inside the valid rows, whatever the row stride (>= D).
template <int D, int NW, int ROWS>
struct RowDma {
  static constexpr int CPR = D / 8;     // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;  // rows per load instruction
  static constexpr int INSTS = ROWS / RPI;
  static constexpr int PER = INSTS / NW;  // instructions per wave
  static_assert(INSTS % NW == 0, "every wave issues the same number of loads");
  uint32_t voff[PER];  // this lane's byte offset inside the tile, per load of the wave
  uint32_t rs2;        // row stride in bytes
  __device__ __forceinline__ RowDma(int rs, int wave, int lane) : rs2(2u * (uint32_t)rs) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int r = (wave + k * NW) * RPI + lane / CPR;
      voff[k] = (uint32_t)r * rs2 + 16u * (uint32_t)swz<D>(r, lane % CPR);
    }
  }
  // Tile whose first row is `tile_row0` (pointer to that row's features of this head); rows at or
  // past nvalid read as zero.
  __device__ __forceinline__ void issue(const uint16_t* tile_row0, int nvalid, uint16_t* lds,
                                        int wave, int lane) const {
    (void)lane;
#if defined(__HIP_DEVICE_COMPILE__)  // the buffer resource type exists in the device pass only
    // the tile's base and size are wave-uniform; readfirstlane states it, so the resource lives
    // in scalar registers and each load is a single instruction
    const uint64_t a = reinterpret_cast<uint64_t>(tile_row0);
    const uint64_t au = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const int rows = min(max(nvalid, 0), ROWS);
    const int nrec = __builtin_amdgcn_readfirstlane((int)((uint32_t)rows * rs2));
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(au), (short)0, nrec, kRawBufferWord3);
#pragma unroll
    for (int k = 0; k < PER; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (SWATTN_AS3 void*)(lds + (wave + k * NW) * 512),
                                               16, voff[k], 0, 0, 0);
#else
    (void)tile_row0, (void)nvalid, (void)lds, (void)wave;
#endif
  }
};

// The same plan with global_load_lds and 64-bit per-lane addresses (one add per load per tile).
// Rows past `nvalid` re-read the last valid row: callers mask them, and no load leaves the tensor.
// The dK/dV pass keeps this form: with the buffer form its ring measured 2-4% slower, while the
// forward and the dQ pass gained 3-6% from it.
template <int D, int NW, int ROWS>
struct RowDmaFlat {
  static constexpr int CPR = D / 8;     // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;  // rows per load instruction
  static constexpr int INSTS = ROWS / RPI;
  static constexpr int PER = INSTS / NW;  // instructions per wave
  static_assert(INSTS % NW == 0, "every wave issues the same number of loads");
  // a wave's successive loads are NW * RPI rows apart, a multiple of 16, so the swizzle term is
  // the same for all of them: one per-lane offset plus a uniform stride
  static_assert((NW * RPI) % 16 == 0, "swizzle period");
  uint32_t off0;  // this lane's byte offset inside the tile for the wave's first load
  int rs2;
  __device__ __forceinline__ RowDmaFlat(int rs, int wave, int lane) : rs2(2 * rs) {
    const int r = wave * RPI + lane / CPR;
    off0 = (uint32_t)(r * rs2 + 16 * swz<D>(r, lane % CPR));
  }
  // Tile whose first row is `tile_row0` (pointer to that row's features of this head); rows
  // past nvalid re-read row nvalid - 1.
  __device__ __forceinline__ void issue(const uint16_t* tile_row0, int nvalid, uint16_t* lds,
                                        int wave, int lane) const {
    const char* b = reinterpret_cast<const char*>(tile_row0);
    if (nvalid >= ROWS) {
      // opaque copy: keeps the compiler from hoisting one 64-bit address per load out of the
      // caller's loop, which costs more registers than the one add per load it saves
      uint32_t o = off0;
      asm volatile("" : "+v"(o));
#pragma unroll
      for (int k = 0; k < PER; ++k)
        g2lds16(reinterpret_cast<const uint16_t*>(b + (int64_t)(k * NW * RPI) * rs2 + o),
                lds + (wave + k * NW) * 512);
    } else {
      // the partial tile (at most one per sequence): an opaque copy of the row count keeps its
      // clamped addresses from being computed speculatively on every full tile as well
      int last = nvalid - 1;
      asm volatile("" : "+s"(last));
      const int cp = lane % CPR;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int r = (wave + k * NW) * RPI + lane / CPR;
        const uint32_t rc = (uint32_t)min(r, last);
        g2lds16(reinterpret_cast<const uint16_t*>(b + rc * (uint32_t)rs2 + 16 * swz<D>(r, cp)),
                lds + (wave + k * NW) * 512);
      }
    }
  }
};

// Per-lane LDS byte offsets of the two kinds of MFMA operand reads from a row-major swizzled tile,
// computed once per kernel.  A read's address is (tile base) + (this per-lane offset) + (a
// compile-time row offset), i.e. one VGPR add plus an immediate:
//   rc[t]:     the 16-byte chunk (2t + half) of row (l % 32) -- an A or B fragment over D for
//              k-step t; add 32 * D * 2 bytes per 32-row block;
//   tr[mb][e]: the two ds_read_b64_tr_b16 reads that assemble an A fragment of the transposed tile
//              (feature rows 32 mb .. +32, 16 sequence rows): slot s of lane (d, half) receives
//              sequence row 8 (s / 4) + 4 half + (s % 4); add row0 * D * 2 bytes for the 16-row
//              step starting at row0.
template <int D>
struct LdsOffsets {
  uint32_t rc[D / 16];     // byte offsets
  uint32_t tr[D / 32][2];  // byte offsets
  __device__ __forceinline__ explicit LdsOffsets(int lane) {
    const int l32 = lane & 31, half = lane >> 5;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) rc[t] = 2 * (l32 * D + 8 * swz<D>(l32, 2 * t + half));
    const int g = lane >> 4, j = (lane >> 2) & 3, c = lane & 3, h = g >> 1;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
      const int d = 32 * mb + 16 * (g & 1) + 4 * c;
      const int r1 = 4 * h + j, r2 = r1 + 8;
      tr[mb][0] = 2 * (r1 * D + 8 * swz<D>(r1, d >> 3) + (d & 7));
      tr[mb][1] = 2 * (r2 * D + 8 * swz<D>(r2, d >> 3) + (d & 7));
    }
  }
};

// Byte address arithmetic on an LDS tile: the per-lane offset is one VGPR add onto the (scalar)
// tile base, and block offsets that are compile-time constants fold into the instruction.
__device__ __forceinline__ const char* lds_at(const uint16_t* tile, uint32_t lane_off,
                                              int const_bytes) {
  return reinterpret_cast<const char*>(tile) + lane_off + const_bytes;
}

template <int D>
__device__ __forceinline__ uint4 rc_frag(const uint16_t* tile, const LdsOffsets<D>& o, int blk32,
                                         int t) {
  return *reinterpret_cast<const uint4*>(lds_at(tile, o.rc[t], blk32 * 32 * D * 2));
}

template <int D>
__device__ __forceinline__ uint4 tr_frag_o(const uint16_t* tile, const LdsOffsets<D>& o, int row0,
                                           int mb) {
  const uint2 lo = lds_tr16(reinterpret_cast<const uint16_t*>(lds_at(tile, o.tr[mb][0], row0 * D * 2)));
  const uint2 hi = lds_tr16(reinterpret_cast<const uint16_t*>(lds_at(tile, o.tr[mb][1], row0 * D * 2)));
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Scheduling pin for a chain of N MFMAs that each take R LDS reads (written just above the call):
// the reads of the first A MFMAs issue first, then each MFMA is followed by the reads of the MFMA
// A places later, so LDS latency hides under A MFMAs instead of stalling each one.  The
// sched_barrier stops later code from being mixed into the pattern.
template <int N, int R, int A>
__device__ __forceinline__ void sched_mfma_chain() {
  static_assert(A >= 1 && A <= N, "lookahead");
  __builtin_amdgcn_sched_group_barrier(0x100, R * A, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if (i + A < N) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup schedule for full-causal training passes, where the work of tile t of a head grows
// (or shrinks) linearly with t: workgroup g owns the tile pair (j, n - 1 - j) of one head, so all
// workgroups carry equal work and the launch ends without a tail.  Workgroups are handed to the
// chip's 8 XCDs round-robin by index; the index -> (head, j) map gives each XCD a contiguous run of
// heads with j fastest, so a head's workgroups run at the same time on one XCD and share its L2.
constexpr int kXcds = 8;

struct PairJob {
  int bh;   // head (batch * H + h)
  int j;    // pair index: tiles j and n - 1 - j
};

__device__ __forceinline__ PairJob pair_job(int bid, int BH, int npair) {
  const int G = BH * npair;
  const int x = bid % kXcds, n = bid / kXcds;
  const int q = G / kXcds, r = G % kXcds;
  const int lin = x * q + min(x, r) + n;  // XCD x owns [x q + min(x, r), +q + (x < r))
  PairJob jb;
  jb.bh = lin / npair;
  jb.j = lin % npair;
  return jb;
}

}  // namespace swattn
