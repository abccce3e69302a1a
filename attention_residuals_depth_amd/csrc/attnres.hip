// libattnres: Attention Residuals forward and backward for gfx950 (MI355X).
//
// The operator mixes a token's depth sources with softmax weights of the
// sub-layer pseudo-query against each RMS-normalised source and returns the
// weighted sum of the raw sources (formula box of the architecture figure in
// "Kimi K3 模型结构（10）：RL 与服务中的状态管理").  The Attention Residuals section
// of "Kimi K3 on Fireworks: Fast RL at frontier scale" fuses normalisation and
// weighted sum so that nothing per-source is materialised; here that means:
//
//   forward   one kernel, one HBM pass over the sources, one workgroup per
//             token; each thread keeps a fixed D-slice of all N source rows
//             in registers, forms its partial sum of squares and w.x,
//             reduces them across the wave with DPP and across waves through
//             a few LDS words, computes rstd/softmax redundantly in every
//             thread, and writes the fp32-accumulated weighted sum from the
//             same registers.  The same kernel serves training batches and
//             single decoding steps.
//   backward  one kernel re-reads each source row once (plus dout), forms
//             da_i = g.x_i and w.x_i with the same kind of fixed reduction
//             tree, then writes (or accumulates into) dsources from the
//             registers and accumulates this workgroup's dw partial row; a
//             second small kernel sums the fixed number of partial rows in
//             index order (deterministic, no atomics).
//
// Determinism and batch invariance (the determinism section of the Fireworks
// report fixes reduction orders so results do not depend on the batch): the
// per-token reduction tree depends only on (N, D), never on T or the grid, so
// a token's outputs are bitwise the same whatever batch it sits in.
//
// No MFMA: the work is a batched GEMV ([T*N x D] . [D]) bound by HBM bandwidth.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <mutex>

#include "attnres.h"

namespace {

constexpr int kWave = 64;
constexpr int kMaxWaves = 16;  // 1024 threads

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

// Round-to-nearest-even fp32 -> bf16 pair (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Unpack the eight bf16 values of a 16-byte vector.
__device__ __forceinline__ void unpack8(const uint4& q, float (&f)[8]) {
  f[0] = bf_lo(q.x); f[1] = bf_hi(q.x);
  f[2] = bf_lo(q.y); f[3] = bf_hi(q.y);
  f[4] = bf_lo(q.z); f[5] = bf_hi(q.z);
  f[6] = bf_lo(q.w); f[7] = bf_hi(q.w);
}

__device__ __forceinline__ uint4 pack8(const float (&d)[8]) {
  uint4 o;
  o.x = pack_bf16x2(d[0], d[1]);
  o.y = pack_bf16x2(d[2], d[3]);
  o.z = pack_bf16x2(d[4], d[5]);
  o.w = pack_bf16x2(d[6], d[7]);
  return o;
}

// acc + a.b over the four bf16 pairs of two 16-byte vectors, with the pair
// products formed exactly and added in fp32 (v_dot2_f32_bf16 on gfx950).
__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), acc, false);
  return acc;
}

// ---------------------------------------------------------------------------
// Buffer access
// ---------------------------------------------------------------------------
// Every row is addressed through a raw buffer descriptor built in scalar
// registers (base = the row, size = the row's bytes); a lane supplies only a
// 32-bit byte offset.  The hardware range check turns loads past the row end
// into zeros and drops such stores, which masks the row tail for free.
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Cache policy of the streaming accesses (sources, dout, out, dsources): each
// byte is touched once per call, so loads and stores carry the nontemporal
// hint (aux bit 1, "nt"); small reused data (w, dw rows) uses the default.
#ifndef ATTNRES_STREAM_LOAD_AUX
#define ATTNRES_STREAM_LOAD_AUX 2
#endif
#ifndef ATTNRES_STREAM_STORE_AUX
#define ATTNRES_STREAM_STORE_AUX 2
#endif
constexpr int kAuxDefault = 0;
constexpr int kAuxStreamLoad = ATTNRES_STREAM_LOAD_AUX;
constexpr int kAuxStreamStore = ATTNRES_STREAM_STORE_AUX;

template <int AUX = kAuxDefault>
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}

template <int AUX = kAuxDefault>
__device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, AUX);
}

// ---------------------------------------------------------------------------
// Fixed-order reductions
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_masked(float v) {
  // lanes outside ROW_MASK receive 0.0f, the identity of the sum below
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes of a wave, complete in lane 63.  Butterfly within each
// 16-lane row (xor 1, xor 2, half-row mirror, row mirror: every lane of a row
// ends with the same bits because fp32 addition commutes), then the row sums
// R0..R3 are combined with the row broadcasts as (R3 + R2) + (R1 + R0).
// Pure VALU/DPP, fixed order.
__device__ __forceinline__ float wave_sum_lane63(float v) {
  v += dpp_f<0xB1>(v);             // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);             // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);            // row_half_mirror
  v += dpp_f<0x140>(v);            // row_mirror
  v += dpp_masked<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_masked<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// This lane's index in its wave, recomputed (two VALU ops) instead of kept live.
__device__ __forceinline__ int lane_id() {
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// This wave's index in the workgroup, in a scalar register.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave); }

// Workgroup-wide sums of K (<= 64) per-thread values, returned wave-uniform.
// Each wave reduces its values, lane 63 stores them in red[k][wave], one
// barrier, then lane k adds the kMaxWaves slots of red[k] in slot order (slots
// of absent waves hold zeros, written once at kernel start) and the K totals
// are broadcast from lane k with v_readlane.  `red` is double-buffered by the
// caller (alternating tokens), which makes one barrier per token enough: a
// wave can only overwrite a buffer after passing the next token's barrier,
// which every wave reaches only after it finished reading that buffer.
template <int K>
__device__ __forceinline__ void block_sums(float (&v)[K], float (*red)[kMaxWaves]) {
  static_assert(K <= kWave, "one lane per value");
  const int lane = lane_id(), wave = wave_id();
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = wave_sum_lane63(v[k]);
  if (lane == kWave - 1) {
#pragma unroll
    for (int k = 0; k < K; ++k) red[k][wave] = v[k];
  }
  __syncthreads();
  float s = 0.f;
  if (lane < K) {
    const float4* r4 = reinterpret_cast<const float4*>(red[lane]);
    float4 q[kMaxWaves / 4];
#pragma unroll
    for (int j = 0; j < kMaxWaves / 4; ++j) q[j] = r4[j];
#pragma unroll
    for (int j = 0; j < kMaxWaves / 4; ++j) {
      s += q[j].x;
      s += q[j].y;
      s += q[j].z;
      s += q[j].w;
    }
  }
  const int sb = __builtin_bit_cast(int, s);
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(sb, k));
}

// Zero both reduction buffers once, before the first token.
template <int K>
__device__ __forceinline__ void clear_red(float (*red)[K][kMaxWaves]) {
  float* p = &red[0][0][0];
  for (int j = threadIdx.x; j < 2 * K * kMaxWaves; j += blockDim.x) p[j] = 0.f;
  __syncthreads();
}

// For a single token: zero only the slots of absent waves in buffer 0.  No
// barrier: no wave writes those slots, and the barrier inside block_sums
// orders these stores before the slots are read.
template <int K>
__device__ __forceinline__ void clear_absent(float (*red)[K][kMaxWaves]) {
  const int present = (int)blockDim.x / kWave;
  const int absent = kMaxWaves - present;
  for (int j = threadIdx.x; j < K * absent; j += blockDim.x) red[0][j / absent][present + j % absent] = 0.f;
}

// Hide a register's contents from the optimiser so values derived from it
// (unpacked floats) are recomputed after a barrier instead of being kept live
// across it: holding 8 unpacked floats per packed vector would double the
// register footprint of a row group.
__device__ __forceinline__ void opaque(uint4& q) {
  u32x4_t v = __builtin_bit_cast(u32x4_t, q);
  asm volatile("" : "+v"(v));  // one 128-bit operand: the register tuple stays whole
  q = __builtin_bit_cast(uint4, v);
}

// Keep the scheduler from moving instructions across this point: prefetch
// loads must stay where they are issued, before the next token's work, or the
// in-order wait counts would make a token wait for loads issued after it.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Order this wave's LDS accesses across its lanes: everything before the
// call (release) happens before everything after it (acquire) for every lane
// of the wave.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Move a wave-uniform value into a scalar register (frees a VGPR per value).
__device__ __forceinline__ float uniform(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// ---------------------------------------------------------------------------
// Row-group slices
// ---------------------------------------------------------------------------
// Thread j of a workgroup owns the 16-byte vectors j + k*blockDim.x (k < VPT)
// of every row of the token: eight consecutive channels per vector, so one
// wave-wide load covers 1 KiB of a row.  off[k] is that vector's byte offset
// within a bf16 row (past the row end for tail threads: the buffer range
// check then reads zeros and drops stores).  w and the running dw of the
// backward pass live in LDS slots private to the thread (slot j + k*blockDim.x
// holds 8 floats), so they need no barrier and leave the register file to the
// row group.
// When the row's D/8 vectors do not fill VPT * blockDim.x slots, whole waves
// can own no vector k at all (D = 7168 with 256 threads x 4 vectors: waves 2
// and 3 have no fourth vector); bit k of `live` (wave-uniform, in a scalar
// register) says whether any lane of this wave owns a vector k inside the
// row, so the arithmetic on a dead vector is skipped with a scalar branch.
// Its loads are still issued (size-checked to zeros), which keeps the number
// of outstanding loads, and so the compiler's wait counts, the same in every
// wave.
template <int VPT>
struct Slice {
  uint32_t off[VPT];  // byte offset in a bf16 row
  int slot[VPT];      // private LDS slot (8 floats)
  uint32_t live;      // bit k: this wave owns some vector k inside the row
  __device__ __forceinline__ Slice(int tid, int nthreads, int32_t D) {
    const int first = __builtin_amdgcn_readfirstlane(tid) & ~(kWave - 1);  // this wave's first thread
    live = 0;
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      slot[k] = tid + k * nthreads;
      off[k] = (uint32_t)slot[k] * 16u;
      if (first + k * nthreads < D / 8) live |= 1u << k;
    }
  }
  __device__ __forceinline__ bool has(int k) const { return k == 0 || ((live >> k) & 1u) != 0; }
};

__device__ __forceinline__ void load8(const float4* p, int slot, float (&f)[8]) {
  const float4 a = p[2 * slot], b = p[2 * slot + 1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

__device__ __forceinline__ void store8(float4* p, int slot, const float (&f)[8]) {
  p[2 * slot] = make_float4(f[0], f[1], f[2], f[3]);
  p[2 * slot + 1] = make_float4(f[4], f[5], f[6], f[7]);
}

// The thread's slice of w (fp32, 8 values per vector; zeros past the row
// end), requested into registers so that the row loads can be issued right
// behind it, then parked in the thread's LDS slots.
template <int VPT>
__device__ __forceinline__ void load_w(uint4 (&wv)[VPT][2], const float* __restrict__ w, int32_t D,
                                       const Slice<VPT>& sl) {
  const __amdgpu_buffer_rsrc_t r = rsrc(w, (uint32_t)D * 4u);
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    wv[k][0] = bload(r, 2u * sl.off[k]);
    wv[k][1] = bload(r, 2u * sl.off[k] + 16u);
  }
}

template <int VPT>
__device__ __forceinline__ void store_w(const uint4 (&wv)[VPT][2], float4* wl, const Slice<VPT>& sl) {
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    wl[2 * sl.slot[k]] = __builtin_bit_cast(float4, wv[k][0]);
    wl[2 * sl.slot[k] + 1] = __builtin_bit_cast(float4, wv[k][1]);
  }
}

// Per-source rows: row (i, t) starts at p[i] + t*pitch (elements, pitch >= D).
// Stacked [N][T][D] sources use p[i] = src + i*T*D and pitch D; separately
// allocated sources pass their own bases and pitch D; sources interleaved by
// token ([T][N][D]) use p[i] = base + i*D and pitch N*D.  Passed by value
// (kernel arguments).
struct SrcRows {
  const uint16_t* p[ATTNRES_MAX_SOURCES];
  int64_t pitch;
};
// Source gradients: bf16 or fp32 rows (the backward's MODE says which), row
// (i, t) at p[i] + t*pitch elements of that type.
struct DstRows {
  void* p[ATTNRES_MAX_SOURCES];
  int64_t pitch;
};

// Backward gradient modes: bit 0 accumulate into the existing gradients,
// bit 1 fp32 gradients (else bf16).  Same values as ATTNRES_GRAD_* in the
// header.
constexpr int kGradAccumulate = 1;
constexpr int kGradF32 = 2;

template <bool F32>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t grad_row(const DstRows& d, int i, int64_t t, int32_t D) {
  if constexpr (F32)
    return rsrc(static_cast<float*>(d.p[i]) + t * d.pitch, (uint32_t)D * 4u);
  else
    return rsrc(static_cast<uint16_t*>(d.p[i]) + t * d.pitch, (uint32_t)D * 2u);
}

// Old gradients of sources [I0, I1) for vector k: bf16 rows give one 16-byte
// vector per slice vector, fp32 rows two.
template <bool F32, int I0, int I1, int VPT, int OW>
__device__ __forceinline__ void load_grads(uint4 (&o)[I1 - I0][OW], const DstRows& d, int64_t t, int32_t D,
                                           const Slice<VPT>& sl, int k) {
#pragma unroll
  for (int i = I0; i < I1; ++i) {
    const __amdgpu_buffer_rsrc_t r = grad_row<F32>(d, i, t, D);
    if constexpr (F32) {
      // a lane's 32 bytes are split over two instructions with a 32-byte lane
      // stride: default policy, so the second half finds the line in L2
      o[i - I0][0] = bload(r, 2u * sl.off[k]);
      o[i - I0][1] = bload(r, 2u * sl.off[k] + 16u);
    } else {
      o[i - I0][0] = bload<kAuxStreamLoad>(r, sl.off[k]);
    }
  }
}

// This thread's slice of token t's N source rows; each row's descriptor is
// built in scalar registers.  With valid == false the descriptors have size 0:
// every lane reads zeros and no memory is touched, but the instructions are
// still issued.  Keeping the number of loads independent of the path lets the
// compiler's wait counts stay exact (only the oldest outstanding loads are
// waited for).
template <int N, int VPT, typename Rows>
__device__ __forceinline__ void load_rows(uint4 (&x)[N][VPT], const Rows& rows, int64_t t, int32_t D,
                                          const Slice<VPT>& sl, bool valid = true) {
  const int64_t tt = valid ? t : 0;
  const uint32_t bytes = valid ? (uint32_t)D * 2u : 0u;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const __amdgpu_buffer_rsrc_t r = rsrc(rows.p[i] + tt * rows.pitch, bytes);
#pragma unroll
    for (int k = 0; k < VPT; ++k) x[i][k] = bload<kAuxStreamLoad>(r, sl.off[k]);
  }
}

template <int VPT>
__device__ __forceinline__ void load_row(uint4 (&g)[VPT], const uint16_t* __restrict__ p, int64_t t, int32_t D,
                                         const Slice<VPT>& sl, bool valid = true) {
  const int64_t tt = valid ? t : 0;
  const __amdgpu_buffer_rsrc_t r = rsrc(p + tt * D, valid ? (uint32_t)D * 2u : 0u);
#pragma unroll
  for (int k = 0; k < VPT; ++k) g[k] = bload<kAuxStreamLoad>(r, sl.off[k]);
}

// Token t's saved softmax weight and rstd, lane i holding source i (lanes >= N
// read zeros).  Loaded with the row group, so they complete in the same order.
template <int N>
__device__ __forceinline__ void load_saved(float& a, float& r, const float* __restrict__ alpha,
                                           const float* __restrict__ rstd, int64_t t, bool valid = true) {
  const int lane = lane_id();
  const int64_t tt = valid ? t : 0;
  const uint32_t bytes = valid ? (uint32_t)N * 4u : 0u;
  a = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(alpha + tt * N, bytes), lane * 4, 0, 0));
  r = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(rstd + tt * N, bytes), lane * 4, 0, 0));
}

__device__ __forceinline__ float lane_value(float v, int i) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), i));
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
struct FwdCtx {
  int32_t D;
  float eps;
  float inv_d;
  uint16_t* out;
  float* rstd_out;
  float* alpha_out;
  const float4* wl;
  float (*red)[kMaxWaves];  // red[buf * 2N + k][wave]
  int tid;
};

// Forward of token t whose row group is already in x: partial sums, workgroup
// reduction, softmax, weighted sum, stores.  Issues no loads of its own.
// SCORED: the first N-1 sources arrive with their rstd and this sub-layer's
// score already formed (block-batched scores); lane i of (rgv, zgv) holds
// source i's.  Only the last source -- the current block's partial sum -- is
// reduced here.  Without SCORED every source is reduced (the code is the
// plain forward's).
template <int N, int VPT, bool SCORED = false>
__device__ __forceinline__ void fwd_token(uint4 (&x)[N][VPT], int64_t t, int& buf, const FwdCtx& c,
                                          const Slice<VPT>& sl, float zgv = 0.f, float rgv = 0.f) {
  constexpr int NR = SCORED ? 1 : N;  // sources reduced here: the last NR
  constexpr int I0 = N - NR;
  // partial sum of squares (first NR) and w.x (last NR)
  float part[2 * NR];
#pragma unroll
  for (int i = 0; i < 2 * NR; ++i) part[i] = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if (!sl.has(k)) continue;  // wave-uniform: no lane of this wave owns a vector k
    float wr[8];
    load8(c.wl, sl.slot[k], wr);
#pragma unroll
    for (int ii = 0; ii < NR; ++ii) {
      const int i = I0 + ii;
      float f[8];
      unpack8(x[i][k], f);
      part[ii] = dot8_bf16(x[i][k], x[i][k], part[ii]);
#pragma unroll
      for (int e = 0; e < 8; ++e) part[NR + ii] = fmaf(wr[e], f[e], part[NR + ii]);
    }
  }
  block_sums<2 * NR>(part, c.red + buf * 2 * N);
  buf ^= 1;
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int k = 0; k < VPT; ++k) opaque(x[i][k]);

  // rstd, scores, softmax over the sources (fp32, max-subtracted).  Every
  // lane of every wave evaluates these N-value formulas, so their cost is paid
  // once per wave (7 waves per token at D = 7168).  The hardware reciprocal
  // square root (v_rsq_f32, 1 ulp), the hardware exp2 on the scaled argument
  // and one division for the N weights keep the forward off the VALU limit:
  // with the correctly rounded sqrt, expf and N divisions the kernel ran 3-5%
  // slower on MI355X.  The errors stay at the 1e-6 level relative, far inside
  // the weights' 1e-5 absolute tolerance.
  float r[N], a[N];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i < I0) {  // given (SCORED only)
      r[i] = uniform(lane_value(rgv, i));
      a[i] = uniform(lane_value(zgv, i));
    } else {
      r[i] = uniform(__builtin_amdgcn_rsqf(part[i - I0] * c.inv_d + c.eps));
      a[i] = r[i] * part[NR + i - I0];  // z_i
    }
    m = fmaxf(m, a[i]);
  }
  float den = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    a[i] = __expf(a[i] - m);
    den += a[i];
  }
  const float inv_den = 1.0f / den;
#pragma unroll
  for (int i = 0; i < N; ++i) a[i] = uniform(a[i] * inv_den);

  // weighted sum of the raw sources
  const __amdgpu_buffer_rsrc_t ro = rsrc(c.out + t * c.D, (uint32_t)c.D * 2u);
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if (!sl.has(k)) continue;  // a dead vector's store would be dropped anyway
    float acc[8];
    {
      float f[8];
      unpack8(x[0][k], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = a[0] * f[e];
    }
#pragma unroll
    for (int i = 1; i < N; ++i) {
      float f[8];
      unpack8(x[i][k], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(a[i], f[e], acc[e]);
    }
    bstore<kAuxStreamStore>(ro, sl.off[k], pack8(acc));
  }
  if (c.rstd_out != nullptr && c.tid < N) {  // the decode call may skip the saved state
    float rv = r[0], av = a[0];
#pragma unroll
    for (int i = 1; i < N; ++i) {
      rv = c.tid == i ? r[i] : rv;
      av = c.tid == i ? a[i] : av;
    }
    c.rstd_out[t * N + c.tid] = rv;
    c.alpha_out[t * N + c.tid] = av;
  }
}

// One workgroup per token: workgroup b handles token t0 + xcd_chunked(b).  The
// hardware dispatcher starts the next token as soon as a workgroup retires, two
// workgroups share a CU, and the tokens in flight at any moment are
// neighbours, so the rows the chip reads are close together in every source.
// This beat a persistent kernel with a two-token software pipeline per
// workgroup at every T on MI355X (T = 32768, N = 9: 5.79 vs 5.39 TB/s; T = 1:
// 6.9 vs 7.8 us kernel time).  The w slice is requested first and the row
// group right behind it, so both latencies overlap; w then goes to the
// thread's LDS slots while the rows arrive.
// VPT = 4 (512 < D <= 8192: 256 threads at D = 7168 -- 224 are needed for its
// 896 vectors, rounded up to four waves, of which waves 2 and 3 own only three
// vectors and skip the fourth; 190 VGPRs at N = 9, two waves per SIMD) or 2
// (larger D: up to 1024 threads, 113 VGPRs; and D <= 512).  At D = 7168
// four vectors per thread measured 3-5% faster than two at T = 2K-8K, the same
// at T >= 16K, and 0.4 us slower for one token (fewer waves share its work);
// one vector per thread (896 threads) was 12-20% slower.
//
// UPDATE: the last source is the current block's partial sum after adding
// the previous sub-layer's output (architecture figure of "Kimi K3
// 模型结构（10）"): src.p[N-1] holds the partial sum before the update and
// `delta` the output to add.  Each thread adds its slice in fp32 and rounds
// to bf16 once (for two bf16 operands the fp32 sum is exact whenever the
// rounding can depend on it, so this is the correctly rounded sum), writes
// the new partial sum to partial_out and uses it as the last source.  This
// folds the separate elementwise update (read p and y, write p) into the
// read the operator makes anyway: one row fewer read per token.  In place
// (partial_out == src.p[N-1]) is fine: a thread rewrites only the slice it
// has already read.
//
// SCORED: the first N-1 sources' rstd and scores come from the block-batched
// scores (zg, rg: [T][N-1] fp32, lane i of each wave loads source i's with the
// row group); only the last source is reduced here.
constexpr int kFwdPlain = 0;
constexpr int kFwdUpdate = 1;
constexpr int kFwdScored = 2;

// The token of workgroup b in a launch of n one-token workgroups.  The
// dispatcher deals the workgroups of a launch to the 8 XCDs in turn
// (workgroup b runs on XCD b mod 8), so with t = b consecutive tokens land on
// different XCDs.  Here, in groups of 8C tokens, XCD x takes the C consecutive
// tokens x*C .. x*C + C-1 of each group (the last, partial group keeps t = b).
// On MI355X the forward read 13% faster at T = 131072 with C = 16 (5.53 ->
// 6.25 TB/s; 6% at T = 16384 and 32768, equal at T = 1024), C = 32 within 1%
// of that; each token's arithmetic is unchanged, so its results are the same
// bits.  Only where two or more workgroups share a CU (D <= 8192): with one
// workgroup of 768-1024 threads per CU (D = 12288, 16384) the same mapping
// read 2% and 12% slower.  The block sums and the merged forward use it too
// (2-3% and 1% at D = 7168); the backward kernels measured no gain from it
// (the one-token backward's workgroup-to-token stride, the split backward's
// spans with all slices on one XCD: 10-15% slower).
constexpr int64_t kXcdCount = 8;
constexpr int64_t kXcdChunk = 16;
__device__ __forceinline__ int64_t xcd_chunked(int64_t b, int64_t n) {
  constexpr int64_t G = kXcdCount * kXcdChunk;
  if (b >= n / G * G) return b;
  const int64_t r = b % G;
  return b - r + (r % kXcdCount) * kXcdChunk + r / kXcdCount;
}

template <int N, int VPT, int VARIANT>
__global__ void __launch_bounds__(VPT >= 4 ? 256 : 1024) fwd_kernel(SrcRows src, const uint16_t* __restrict__ delta,
                                                   uint16_t* partial_out, const float* __restrict__ zg,
                                                   const float* __restrict__ rg, const float* __restrict__ w,
                                                   float eps, int64_t t0, int32_t D, uint16_t* __restrict__ out,
                                                   float* __restrict__ rstd_out, float* __restrict__ alpha_out) {
  constexpr bool UPDATE = VARIANT == kFwdUpdate;
  constexpr bool SCORED = VARIANT == kFwdScored;
  static_assert(!SCORED || N >= 2, "the scored forward has given sources and the partial sum");
  __shared__ __attribute__((aligned(16))) float red[2][2 * N][kMaxWaves];
  extern __shared__ float4 dyn_lds[];
  FwdCtx c;
  c.D = D;
  c.eps = eps;
  c.inv_d = 1.0f / (float)D;
  c.out = out;
  c.rstd_out = rstd_out;
  c.alpha_out = alpha_out;
  c.wl = dyn_lds;
  c.red = &red[0][0];
  c.tid = threadIdx.x;
  const Slice<VPT> sl(c.tid, blockDim.x, D);
  // the host launches one workgroup per token; VPT = 4 <=> 512 < D <= 8192
  const int64_t t = t0 + (VPT >= 4 ? xcd_chunked(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x);

  uint4 wv[VPT][2];
  load_w<VPT>(wv, w, D, sl);
  sched_fence();
  uint4 x[N][VPT];
  uint4 yv[UPDATE ? VPT : 1];
  load_rows<N, VPT>(x, src, t, D, sl);
  if constexpr (UPDATE) load_row<VPT>(yv, delta, t, D, sl);
  float zgv = 0.f, rgv = 0.f;
  if constexpr (SCORED) {  // lane i: source i's given score and rstd (lanes >= N-1 read zeros)
    const int lane = lane_id();
    constexpr uint32_t gb = (uint32_t)(N - 1) * 4u;
    zgv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(zg + t * (N - 1), gb), lane * 4, 0, 0));
    rgv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(rg + t * (N - 1), gb), lane * 4, 0, 0));
  }
  sched_fence();
  if constexpr (UPDATE) {
    const __amdgpu_buffer_rsrc_t rp = rsrc(partial_out + t * src.pitch, (uint32_t)D * 2u);  // the sources' layout
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      if (!sl.has(k)) continue;
      float a[8], b[8];
      unpack8(x[N - 1][k], a);
      unpack8(yv[k], b);
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] += b[e];
      x[N - 1][k] = pack8(a);
      bstore<kAuxStreamStore>(rp, sl.off[k], x[N - 1][k]);
    }
  }
  store_w<VPT>(wv, dyn_lds, sl);
  clear_absent<2 * N>(red);
  int buf = 0;
  fwd_token<N, VPT, SCORED>(x, t, buf, c, sl, zgv, rgv);
}

// ---------------------------------------------------------------------------
// Block-batched scores (MFMA)
// ---------------------------------------------------------------------------
// Every 12 layers form one AttnRes block, and the embedding and the completed
// block sums are the same sources before every alpha of the block, while each
// sub-layer has its own pseudo-query (architecture figure of "Kimi K3
// 模型结构（10）：RL 与服务中的状态管理").  For those n sources the RMS
// statistic is shared by the block's L sub-layers, and the L scores of a row
// are one row of a skinny product [T*n x D] . [D x L]: the only dense
// contraction on this path, so it runs on the matrix cores.
//
// The pseudo-queries are fp32; each is split exactly into three bf16 parts
// (hi = bf16(w), mid = bf16(w - hi), lo = w - hi - mid: 8 + 8 + 8 significand
// bits cover fp32's 24), so the bf16 MFMA forms every product w_d x_d exactly
// and sums in fp32 -- the same precision as the forward's fp32 dots.  Each
// run of 16 k-steps accumulates into a fresh fp32 accumulator that is then
// added to an fp64 running sum, which keeps the rounding error of a score at
// a few fp32 ulps (below).
//
// Layout: workgroup = 4 waves x 64 rows (tokens t of one source); wave rows
// are four 16-row MFMA tiles; per k-step of 32 channels lane l holds 8
// channels of row l % 16 (A) and of query column l % 16 (B), both at channel
// 32 s + 8 (l / 16), and after the loop rows 4 (l / 16) + j, column l % 16
// of the 16 x 16 result (v_mfma_f32_16x16x32_bf16; lane layout verified on
// the device).  Wp: the three parts of the queries, zero past L and D, in
// the B operand's lane order: [k-step][part][column tile][lane] x 8 bf16.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

#ifndef ATTNRES_BS_TILES
#define ATTNRES_BS_TILES 4
#endif
#ifndef ATTNRES_BS_PREFETCH
#define ATTNRES_BS_PREFETCH 0
#endif
constexpr int kBsWaves = 4;
constexpr int kBsTiles = ATTNRES_BS_TILES;        // 16-row tiles per wave
constexpr int kBsWaveRows = kBsTiles * 16;        // 64
constexpr int kBsRows = kBsWaves * kBsWaveRows;   // 256 tokens per workgroup
constexpr int kBsChunk = 4;                       // k-steps per fresh accumulator (even: see the loop)
// A operand staged through LDS (the default): a wave's global loads read 8
// rows x 128 bytes each -- whole lines -- into registers, the wave writes
// them to its own LDS slots, and the MFMA operands (16 rows x 16 bytes per
// lane group) are read back from there.  Loaded straight into the operand
// layout, each load instruction touches 16 rows x 64 bytes: half lines.
#ifndef ATTNRES_BS_LDS
#define ATTNRES_BS_LDS 1
#endif
// the staged loads consume whole lines, so they carry the streaming hint
// (0.85 against 0.91 ms with the default policy at T = 32768, n = 8, L = 24)
#ifndef ATTNRES_BS_LDS_AUX
#define ATTNRES_BS_LDS_AUX 2
#endif
// two waves per SIMD (<= 256 registers) keep a second wave's loads in flight
// while one computes
#ifndef ATTNRES_BS_WAVES_PER_EU
#define ATTNRES_BS_WAVES_PER_EU __attribute__((amdgpu_waves_per_eu(2)))
#endif
constexpr int kBsStageSteps = 2;                        // k-steps per stage: 64 channels, 128 bytes per row
constexpr int kBsStageLoads = kBsWaveRows * 8 / kWave;  // 16-byte loads per lane per stage (8 rows per load)
constexpr int kBsLdsPitch = 9;                          // uint4 slots per staged row: 8 + 1 to spread the banks

__global__ void __launch_bounds__(256) split_queries_kernel(const float* __restrict__ W, int32_t L, int32_t D,
                                                            int32_t Lpad, int32_t Dpad, uint16_t* __restrict__ Wp) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)Lpad * Dpad;
  if (idx >= total) return;
  const int l = (int)(idx / Dpad), d = (int)(idx % Dpad);
  const float w = (l < L && d < D) ? W[(int64_t)l * D + d] : 0.f;
  const __bf16 hi = (__bf16)w;  // round to nearest even
  const float r1 = w - (float)hi;  // exact
  const __bf16 mid = (__bf16)r1;
  const __bf16 lo = (__bf16)(r1 - (float)mid);  // exact: at most 8 significant bits remain
  // stored in the lane order of the MFMA B operand: for k-step s, part p and
  // column tile c, lane 16 q + r holds column 16 c + r, channels 32 s + 8 q ..
  // 32 s + 8 q + 7, so one wave-wide load of a B operand reads 1 KiB
  // contiguous (with [p][l][d] rows it touched 16 rows x 64 bytes, and the
  // kernel ran 1.37 ms instead of 1.05-1.09 ms at T = 32768, n = 8, L = 24)
  const int s = d / 32, q = (d % 32) / 8, e = d % 8, c = l / 16, r = l % 16;
  const int64_t ctl = Lpad / 16;
  const int64_t base = ((int64_t)s * 3 * ctl + c) * kWave + q * 16 + r;
  Wp[base * 8 + e] = __builtin_bit_cast(uint16_t, hi);
  Wp[(base + ctl * kWave) * 8 + e] = __builtin_bit_cast(uint16_t, mid);
  Wp[(base + 2 * ctl * kWave) * 8 + e] = __builtin_bit_cast(uint16_t, lo);
}

// Loads of one k-step without the LDS stage (ATTNRES_BS_LDS = 0): this lane's
// 16 bytes of each of its four rows (A) and of each query part of each column
// tile (B).
template <int CT>
__device__ __forceinline__ void bs_load(uint4 (&a)[kBsTiles], uint4 (&b)[CT][3], __amdgpu_buffer_rsrc_t ra,
                                        __amdgpu_buffer_rsrc_t rb, const uint32_t (&roff)[kBsTiles], int s, int q,
                                        int r, int32_t D, int32_t Lpad) {
  const int ch = 32 * s + 8 * q;  // this lane's first channel
  const uint32_t kb = (uint32_t)ch * 2u;
  // default policy here: a k-step reads 64 of a row's 128-byte line, and the L2
  // keeps the line for the next k-step; with the streaming hint it was often
  // gone by then and fetched again (1.67x the algorithmic bytes, 1.50 against
  // 1.37 ms at T = 32768, n = 8, L = 24)
#pragma unroll
  for (int m = 0; m < kBsTiles; ++m) a[m] = bload(ra, ch < D ? roff[m] + kb : 0xFFFFFFF0u);
  // the parts in the B operand's lane order (split_queries_kernel); column
  // tiles past Lpad (CT > Lpad / 16) read whatever follows, or zeros past the
  // end, and their scores are never stored
  const int ctl = Lpad / 16;
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int p = 0; p < 3; ++p)
      b[c][p] = bload(rb, (uint32_t)((((s * 3 + p) * ctl + c) * kWave + q * 16 + r) * 16));
}

// The B operands of one k-step (the A operands come from LDS).
template <int CT>
__device__ __forceinline__ void bs_load_b(uint4 (&b)[CT][3], __amdgpu_buffer_rsrc_t rb, int s, int q, int r,
                                          int32_t Lpad) {
  const int ctl = Lpad / 16;
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int p = 0; p < 3; ++p)
      b[c][p] = bload(rb, (uint32_t)((((s * 3 + p) * ctl + c) * kWave + q * 16 + r) * 16));
}

// One k-step: squares of the rows (exact products, fp32 sums) and the three
// query parts into the chunk accumulators.  With SEP the hi part has an
// accumulator of its own: the lo and mid products are 2^-8 and 2^-16 of the
// hi ones, so the roundings of their accumulator are negligible, and the hi
// accumulator takes one rounding per k-step instead of three.
template <int CT, bool SEP>
__device__ __forceinline__ void bs_step(const uint4 (&a)[kBsTiles], const uint4 (&b)[CT][3],
                                        f32x4_t (&acc)[kBsTiles][CT], f32x4_t (&acch)[kBsTiles][CT],
                                        float (&ss)[kBsTiles]) {
#pragma unroll
  for (int m = 0; m < kBsTiles; ++m) {
    ss[m] += dot8_bf16(a[m], a[m], 0.f);
    const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a[m]);
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      acc[m][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, b[c][2]), acc[m][c], 0, 0, 0);
      acc[m][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, b[c][1]), acc[m][c], 0, 0, 0);
      if constexpr (SEP)
        acch[m][c] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, b[c][0]), acch[m][c], 0, 0, 0);
      else
        acc[m][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, b[c][0]), acc[m][c], 0, 0, 0);
    }
  }
}

// Accuracy: the scores of a peaked softmax reach |z| ~ 150, where one ulp of
// relative error in z moves a weight by ~4e-6.  So the chunk sums (4 k-steps
// each, fp32 MFMA accumulation, the hi query part in its own accumulator
// where the registers allow: L <= 32) are added into fp64 running sums, the
// rstd comes from a double-precision reciprocal square root of the fp32 sum
// of squares, and z = rstd * dot is formed in fp64 and rounded once.  With
// chunks of 16 k-steps and one accumulator the scores of a peaked block were
// off by up to ~5e-5 (a few ulps), enough to move a weight by 1e-5.
template <int CT, bool AHEAD>  // query column tiles: L <= 16 * CT; AHEAD: see the stage loop
__device__ __forceinline__ void block_scores_body(const SrcRows& src, int64_t T, int32_t D, float eps, int32_t n,
                                                  const uint16_t* __restrict__ Wp, int32_t L, int32_t Lpad,
                                                  int32_t Dpad, int64_t wg_per_source, float* __restrict__ rstd_out,
                                                  float* __restrict__ z_out) {
  const int wave = wave_id(), lane = lane_id();
  const int r = lane & 15, q = lane >> 4;
  // workgroup b runs on XCD b % 8 (round-robin dispatch): the n workgroups of
  // one token group share b % 8 and follow each other, so that XCD's L2 can
  // merge their 4-byte score stores, which interleave at a stride of n floats
  // ([L][T][n]), before the lines go to memory; the grid has whole rounds
  // of 8 token groups, and groups past the last one return at once
  const int64_t bx = blockIdx.x, kx = bx / 8;
  const int i = (int)(kx % n);
  const int64_t tg = bx % 8 + 8 * (kx / n);
  if (tg >= wg_per_source) return;
  const int64_t tw = tg * kBsRows + wave * kBsWaveRows;  // wave's first token
  if (tw >= T) return;  // no barrier in this kernel
  const int64_t rows = T - tw < kBsWaveRows ? T - tw : kBsWaveRows;
  const int64_t pitch_b = src.pitch * 2;
  // one descriptor over the wave's rows of source i: lanes of rows past T
  // (offset >= the size) read zeros
  const __amdgpu_buffer_rsrc_t ra = rsrc(src.p[i] + tw * src.pitch, (uint32_t)((rows - 1) * pitch_b + (int64_t)D * 2));
  const __amdgpu_buffer_rsrc_t rb = rsrc(Wp, (uint32_t)(3u * (uint32_t)Lpad * (uint32_t)Dpad * 2u));
  uint32_t roff[kBsTiles];
#pragma unroll
  for (int m = 0; m < kBsTiles; ++m) roff[m] = (uint32_t)((16 * m + r) * pitch_b);
  constexpr bool SEP = CT <= 2;
  f32x4_t acc[kBsTiles][CT], acch[kBsTiles][CT];
  double run[kBsTiles][CT][4];
  float ss_acc[kBsTiles];
  double ss_run[kBsTiles];
#pragma unroll
  for (int m = 0; m < kBsTiles; ++m) {
    ss_run[m] = 0.0;
    ss_acc[m] = 0.f;
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      acc[m][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acch[m][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) run[m][c][j] = 0.0;
    }
  }
  auto fold = [&]() {  // chunk sums into the fp64 running sums
#pragma unroll
    for (int m = 0; m < kBsTiles; ++m) {
      ss_run[m] += (double)ss_acc[m];
      ss_acc[m] = 0.f;
#pragma unroll
      for (int c = 0; c < CT; ++c) {
#pragma unroll
        for (int j = 0; j < 4; ++j) run[m][c][j] += SEP ? (double)acch[m][c][j] + (double)acc[m][c][j] : (double)acc[m][c][j];
        acc[m][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acch[m][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  // The LDS-staged loop is the default: 0.81 against 0.99-1.02 ms for the
  // operands loaded straight into registers at T = 32768, n = 8, L = 24 (and
  // 0.71 against 0.94-0.98 at L = 16).  Of the direct loops, one register set
  // per k-step, loaded right before its matrix ops, measured 3% faster than
  // two sets alternating (the loads of step s + 1 in flight while step s runs,
  // ATTNRES_BS_PREFETCH = 1), whose extra registers cost more than the
  // overlap gained; the other waves of the CU cover the load latency.
  const int S = Dpad / 32;
#if ATTNRES_BS_LDS
  // this wave's slots: row j of the wave at [j * kBsLdsPitch, + 8); only this
  // wave touches them, so wave-level ordering suffices (no workgroup barrier)
  __shared__ uint4 stage_lds[kBsWaves][kBsWaveRows * kBsLdsPitch];
  uint4* const my = stage_lds[wave];
  // load k of a stage reads row 8 k + lane / 8 of the wave, bytes
  // 16 (lane % 8) .. + 15 of the stage's 128 (channels 64 g + 8 (lane % 8) ..)
  const int srow = lane >> 3, scol = lane & 7;
  const uint32_t sbase = (uint32_t)(srow * pitch_b + scol * 16);
  const int G = (S + kBsStageSteps - 1) / kBsStageSteps;
  uint4 stg[kBsStageLoads];
  auto stage_load = [&](int g) {
    const bool in = 64 * g + 8 * scol < D;
#pragma unroll
    for (int k = 0; k < kBsStageLoads; ++k)
      stg[k] = bload<ATTNRES_BS_LDS_AUX>(ra, in ? sbase + (uint32_t)(8 * k * pitch_b) + (uint32_t)(128 * g) : 0xFFFFFFF0u);
  };
  stage_load(0);
  for (int g = 0; g < G; ++g) {
    wave_sync();  // every lane's reads of the previous stage are done
#pragma unroll
    for (int k = 0; k < kBsStageLoads; ++k) my[(8 * k + srow) * kBsLdsPitch + scol] = stg[k];
    wave_sync();  // the stage is in LDS for every lane
    // AHEAD: the B operands of both k-steps go out before the next stage's
    // loads; the wait counts are in order, so the k-steps then wait for their
    // own loads only and the stage loads have both k-steps to arrive (0.81
    // against 0.84-0.87 ms at T = 32768, n = 8, L = 24).  Otherwise (the
    // four-tile kernel, where the extra registers cost more: 1.42 against
    // 1.30 ms at L = 48) they go out behind the first k-step's B operands.
    uint4 b[AHEAD ? kBsStageSteps : 1][CT][3];
    if constexpr (AHEAD) {
#pragma unroll
      for (int j = 0; j < kBsStageSteps; ++j)
        if (g * kBsStageSteps + j < S) bs_load_b<CT>(b[j], rb, g * kBsStageSteps + j, q, r, Lpad);
      if (g + 1 < G) stage_load(g + 1);
    }
#pragma unroll
    for (int j = 0; j < kBsStageSteps; ++j) {
      const int s = g * kBsStageSteps + j;
      if (s >= S) break;
      uint4 a[kBsTiles];
      if constexpr (!AHEAD) {
        bs_load_b<CT>(b[0], rb, s, q, r, Lpad);
        if (j == 0 && g + 1 < G) stage_load(g + 1);
      }
      const uint4(&bj)[CT][3] = b[AHEAD ? j : 0];
#pragma unroll
      for (int m = 0; m < kBsTiles; ++m) a[m] = my[(16 * m + r) * kBsLdsPitch + 4 * j + q];  // channels 32 s + 8 q ..
      bs_step<CT, SEP>(a, bj, acc, acch, ss_acc);
      if (s % kBsChunk == kBsChunk - 1 || s + 1 >= S) fold();
    }
  }
#elif !ATTNRES_BS_PREFETCH
  for (int s = 0; s < S; ++s) {
    uint4 a[kBsTiles], b[CT][3];
    bs_load<CT>(a, b, ra, rb, roff, s, q, r, D, Lpad);
    bs_step<CT, SEP>(a, b, acc, acch, ss_acc);
    if (s % kBsChunk == kBsChunk - 1 || s + 1 >= S) fold();
  }
#else
  uint4 a0[kBsTiles], a1[kBsTiles], b0[CT][3], b1[CT][3];
  bs_load<CT>(a0, b0, ra, rb, roff, 0, q, r, D, Lpad);
  for (int s = 0; s < S; s += 2) {
    if (s + 1 < S) bs_load<CT>(a1, b1, ra, rb, roff, s + 1, q, r, D, Lpad);
    sched_fence();
    bs_step<CT, SEP>(a0, b0, acc, acch, ss_acc);  // s is even: a chunk never ends here except at the last step
    if (s + 1 >= S) fold();
    if (s + 1 >= S) break;
    if (s + 2 < S) bs_load<CT>(a0, b0, ra, rb, roff, s + 2, q, r, D, Lpad);
    sched_fence();
    bs_step<CT, SEP>(a1, b1, acc, acch, ss_acc);
    if ((s + 1) % kBsChunk == kBsChunk - 1 || s + 2 >= S) fold();
  }
#endif
  const double inv_d = 1.0 / (double)D;
#pragma unroll
  for (int m = 0; m < kBsTiles; ++m) {
    // row 16 m + r: its four k groups sit in lanes r, r + 16, r + 32, r + 48
    double ss = ss_run[m];
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const double rs = __builtin_amdgcn_rsq(ss * inv_d + (double)eps);
    if (q == 0 && 16 * m + r < rows) rstd_out[(tw + 16 * m + r) * n + i] = (float)rs;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * m + 4 * q + j;          // this lane's result row
      const double rr = __shfl(rs, row - 16 * m);  // that row's rstd (lane row - 16 m holds it)
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const int col = 16 * c + r;
        if (col < L && row < rows) z_out[((int64_t)col * T + tw + row) * n + i] = (float)(rr * run[m][c][j]);
      }
    }
  }
}

// Up to 32 queries (one or two column tiles) at two waves per SIMD.
template <int CT>
__global__ void __launch_bounds__(256) ATTNRES_BS_WAVES_PER_EU
    block_scores_kernel(SrcRows src, int64_t T, int32_t D, float eps, int32_t n, const uint16_t* __restrict__ Wp,
                        int32_t L, int32_t Lpad, int32_t Dpad, int64_t wg_per_source, float* __restrict__ rstd_out,
                        float* __restrict__ z_out) {
  block_scores_body<CT, true>(src, T, D, eps, n, Wp, L, Lpad, Dpad, wg_per_source, rstd_out, z_out);
}

// Four column tiles (33-64 queries): held to 256 registers they spill, so
// this one runs at whatever occupancy its registers allow.
__global__ void __launch_bounds__(256)
    block_scores_kernel_wide(SrcRows src, int64_t T, int32_t D, float eps, int32_t n, const uint16_t* __restrict__ Wp,
                             int32_t L, int32_t Lpad, int32_t Dpad, int64_t wg_per_source, float* __restrict__ rstd_out,
                             float* __restrict__ z_out) {
  block_scores_body<4, false>(src, T, D, eps, n, Wp, L, Lpad, Dpad, wg_per_source, rstd_out, z_out);
}

// ---------------------------------------------------------------------------
// Block-batched shared sums
// ---------------------------------------------------------------------------
// The weighted sum is linear in the sources, and within a block only the
// last source -- the current partial sum -- changes from one sub-layer to the
// next (architecture figure of "Kimi K3 模型结构（10）：RL 与服务中的状态管理").
// So the part of sub-layer l's weighted sum that the n shared sources
// contribute is formed for all L sub-layers of the block in one pass over
// those sources, from the block-batched scores, up to the softmax normaliser
// (which also depends on the partial sum's score):
//     m_l = max_i z[l][t][i],   U[l][t] = sum_i exp(z[l][t][i] - m_l) x_i[t]   (fp32)
// Each sub-layer's forward (fwd_merged_kernel) then reads its U row and the
// partial sum instead of all N source rows.
//
// One workgroup per token, the shared rows in registers as in the forward
// (thread j owns vectors j + k*blockDim.x).  The first L threads form one
// sub-layer's n weights each into LDS while the rows arrive; then each thread
// unpacks one vector of every shared row and runs the L weighted sums over it
// (8n fp32 FMAs and 32 bytes of fp32 stores per sub-layer, 24 in the 24-bit
// format below: 4.16 against 5.13 ms for the same block).  The weights are
// read from LDS at a wave-uniform address (a broadcast).  One vector per
// thread up to D = 8192 (896 threads at D = 7168, 87 VGPRs at n = 8), two
// above: 2-3% faster than four or two per thread at D = 7168 on MI355X.
// Without the weighted sums (timing only) the same loads and stores took
// 4.44 ms against 5.2-5.3 ms at T = 32768, n = 8, L = 24: the arithmetic is
// only partly hidden behind the stores.
//
// The shared sums' 24-bit element format (ATTNRES_U_F24): an fp32 value
// rounded to nearest even at bit 8 of its bit pattern (16 significant bits,
// the fp32 exponent range), stored as the upper three bytes, little-endian,
// three bytes per element.  Four elements take three dwords:
//     dw0 = e0 | e1 << 24,  dw1 = e1 >> 8 | e2 << 16,  dw2 = e2 >> 16 | e3 << 8
// with e_k the 24-bit codes.  Rounding the bit pattern is the round-to-nearest
// of the value on a 16-bit significand (a carry into the exponent is the
// correct result; finite values near the fp32 maximum round to infinity).
typedef unsigned int u32x3_t __attribute__((ext_vector_type(3)));

__device__ __forceinline__ uint32_t rne24(float v) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  return (b + 0x7Fu + ((b >> 8) & 1u)) & 0xFFFFFF00u;
}

// four rounded values (low bytes zero) -> three dwords
__device__ __forceinline__ void pack24(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3, uint32_t* d) {
  d[0] = (r0 >> 8) | (r1 << 16);
  d[1] = (r1 >> 16) | (r2 << 8);
  d[2] = (r2 >> 24) | r3;
}

__device__ __forceinline__ float4 unpack24(const u32x3_t& d) {
  return make_float4(__builtin_bit_cast(float, d.x << 8),
                     __builtin_bit_cast(float, __builtin_amdgcn_alignbyte(d.y, d.x, 3) << 8),
                     __builtin_bit_cast(float, __builtin_amdgcn_alignbyte(d.z, d.y, 2) << 8),
                     __builtin_bit_cast(float, d.z & 0xFFFFFF00u));
}

template <int NS, int VPT, bool F24>
__global__ void __launch_bounds__(1024) block_sums_kernel(SrcRows src, const float* __restrict__ z,
                                                                         int32_t L, int64_t T, int32_t D, int64_t t0,
                                                                         void* __restrict__ U, int64_t u_lstride,
                                                                         int64_t u_pitch) {
  constexpr uint32_t EB = F24 ? 3 : 4;  // bytes per element of U
  constexpr int NS4 = (NS + 3) / 4;
  __shared__ float4 ew[ATTNRES_MAX_QUERIES][NS4];
  __shared__ float4 stage[kMaxWaves * 2 * kWave];  // 2 KiB per wave
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const Slice<VPT> sl(tid, blockDim.x, D);
  // one workgroup per token; VPT = 1 <=> D <= 8192 (2-3% faster than t = b at D = 7168)
  const int64_t t = t0 + (VPT == 1 ? xcd_chunked(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x);
  float zz[NS];
  if (tid < L) {  // requested first: the weights can form while the rows are in flight
    const float* zt = z + ((int64_t)tid * T + t) * NS;
#pragma unroll
    for (int i = 0; i < NS; ++i) zz[i] = zt[i];
  }
  sched_fence();
  uint4 x[NS][VPT];
  load_rows<NS, VPT>(x, src, t, D, sl);
  sched_fence();
  if (tid < L) {
    float m = zz[0];
#pragma unroll
    for (int i = 1; i < NS; ++i) m = fmaxf(m, zz[i]);
    float e[4 * NS4];
#pragma unroll
    for (int i = 0; i < 4 * NS4; ++i) e[i] = i < NS ? __expf(zz[i] - m) : 0.f;
#pragma unroll
    for (int q = 0; q < NS4; ++q) ew[tid][q] = make_float4(e[4 * q], e[4 * q + 1], e[4 * q + 2], e[4 * q + 3]);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    if (!sl.has(k)) continue;  // wave-uniform: no lane of this wave owns a vector k
    float f[NS][8];
#pragma unroll
    for (int i = 0; i < NS; ++i) unpack8(x[i][k], f[i]);
    const uint32_t wbase = 2u * sl.off[k] - 32u * (uint32_t)lane;  // the wave's first vector k, fp32 bytes
    for (int l = 0; l < L; ++l) {
      float e[4 * NS4];
#pragma unroll
      for (int q = 0; q < NS4; ++q) {
        const float4 v = ew[l][q];
        e[4 * q] = v.x; e[4 * q + 1] = v.y; e[4 * q + 2] = v.z; e[4 * q + 3] = v.w;
      }
      float acc[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = e[0] * f[0][c];
#pragma unroll
      for (int i = 1; i < NS; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(e[i], f[i][c], acc[c]);
      // the wave's 64 x 32 bytes pass through its LDS stage so that each store
      // writes one contiguous KiB (lane j: bytes [16 j, 16 j + 16) and
      // [1024 + 16 j, ...) of the wave's 2 KiB); the wave barriers order the
      // stage's writes before other lanes' reads, and those reads before the
      // next sub-layer's writes.  Two half-vector streaming stores per lane
      // ran at 2.7 TB/s, the same with the default policy at 3.1, staged at
      // 4.9 with the streaming hint and 1.5-3% faster again with the default
      // policy (T = 8192 and 32768, n = 8, L = 24, both element formats).
      // (24-bit elements: 24 bytes per lane, 1536 per wave, stored as two
      // runs of 768 bytes, 12 bytes per lane; 3D is a multiple of 12, so a
      // lane's 12 bytes are wholly inside the row or wholly past its end)
      const __amdgpu_buffer_rsrc_t ru =
          rsrc(static_cast<uint8_t*>(U) + ((int64_t)l * u_lstride + t * u_pitch) * EB, (uint32_t)D * EB);
      float4* st = stage + wave * (2 * kWave);
      if constexpr (F24) {
        uint32_t* s32 = reinterpret_cast<uint32_t*>(st);
        uint32_t d[6];
        pack24(rne24(acc[0]), rne24(acc[1]), rne24(acc[2]), rne24(acc[3]), d);
        pack24(rne24(acc[4]), rne24(acc[5]), rne24(acc[6]), rne24(acc[7]), d + 3);
        uint2* s64 = reinterpret_cast<uint2*>(s32 + 6 * lane);
        s64[0] = make_uint2(d[0], d[1]);
        s64[1] = make_uint2(d[2], d[3]);
        s64[2] = make_uint2(d[4], d[5]);
        wave_sync();
        u32x3_t lo, hi;
        lo.x = s32[3 * lane]; lo.y = s32[3 * lane + 1]; lo.z = s32[3 * lane + 2];
        hi.x = s32[3 * kWave + 3 * lane]; hi.y = s32[3 * kWave + 3 * lane + 1]; hi.z = s32[3 * kWave + 3 * lane + 2];
        wave_sync();
        const uint32_t wb24 = (sl.off[k] >> 4) * 24u - 24u * (uint32_t)lane;  // the wave's first vector, bytes
        __builtin_amdgcn_raw_buffer_store_b96(lo, ru, wb24 + 12u * (uint32_t)lane, 0, kAuxDefault);
        __builtin_amdgcn_raw_buffer_store_b96(hi, ru, wb24 + 768u + 12u * (uint32_t)lane, 0, kAuxDefault);
      } else {
        st[2 * lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        st[2 * lane + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        wave_sync();
        const float4 lo = st[lane], hi = st[kWave + lane];
        wave_sync();
        bstore(ru, wbase + 16u * (uint32_t)lane, __builtin_bit_cast(uint4, lo));
        bstore(ru, wbase + 1024u + 16u * (uint32_t)lane, __builtin_bit_cast(uint4, hi));
      }
    }
  }
}

// Forward of one sub-layer from its block-batched shared sum U (above) and the
// current partial sum p, the last of its N sources.  p is normalised and
// scored here with w; the given rstd and scores of the N-1 shared sources
// arrive as in the scored forward (lane i of each wave loads source i's), and
// the softmax over all N scores is that forward's sequence.  Then, with m the
// largest given score and M the largest of all N,
//     out = exp(m - M) / den * U + alpha_p * p
// since exp(m - M) exp(z_i - m) = exp(z_i - M): the plain weighted sum, from
// one fp32 row and one bf16 row instead of N bf16 rows.
// Thread j owns the channel quads j + k*blockDim.x (k < kMergedQuads): 16
// contiguous bytes of U and of w and 8 of p and out per quad, so every load
// and store instruction of a wave covers one contiguous run (1 KiB of U,
// 512 bytes of p).  Eight-channel vectors, whose 32 bytes of U take two
// loads with a 32-byte lane stride, ran 11% slower (5.57 against 6.20 TB/s at
// T = 32768, D = 7168); 256 threads (7 quads each) beat 448 (4) and 896 (2).
// The partial sum's dots are therefore summed in another order than in the
// scored forward: its rstd and score, and so alpha, agree with that forward's
// to within fp32 rounding, not bit for bit.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kMergedQuads = 7;

__device__ __forceinline__ void unpack4(const u32x2_t& q, float (&f)[4]) {
  f[0] = __builtin_bit_cast(float, q.x << 16);
  f[1] = __builtin_bit_cast(float, q.x & 0xFFFF0000u);
  f[2] = __builtin_bit_cast(float, q.y << 16);
  f[3] = __builtin_bit_cast(float, q.y & 0xFFFF0000u);
}

//
// UPDATE: the partial sum is first advanced by the previous sub-layer's output
// y (delta), as the fused update of the plain forward does: each thread adds
// its quads in fp32, rounds once to bf16 (the correctly rounded sum of two
// bf16 values), stores the new partial sum to partial_out (row pitch p_pitch;
// may be p itself: a thread rewrites only the quads it has already read) and
// continues with it.
template <int N, bool UPDATE, bool F24>
__global__ void __launch_bounds__(1024) fwd_merged_kernel(
    const void* __restrict__ U, int64_t u_pitch, const uint16_t* p, int64_t p_pitch,
    const uint16_t* __restrict__ delta, uint16_t* partial_out, const float* __restrict__ zg,
    const float* __restrict__ rg, const float* __restrict__ w, float eps, int64_t t0, int32_t D,
    uint16_t* __restrict__ out, float* __restrict__ rstd_out, float* __restrict__ alpha_out) {
  static_assert(N >= 2, "the shared sources and the partial sum");
  constexpr int Q = kMergedQuads;
  __shared__ __attribute__((aligned(16))) float red[1][2][kMaxWaves];
  const int tid = threadIdx.x;
  // one workgroup per token (1% faster than t = b at D = 7168; up to D = 8192)
  const int64_t t = t0 + (D <= 8192 ? xcd_chunked(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x);
  const int V4 = D / 4;
  const __amdgpu_buffer_rsrc_t rw = rsrc(w, (uint32_t)D * 4u);
  constexpr uint32_t EB = F24 ? 3 : 4;  // bytes per element of U
  const __amdgpu_buffer_rsrc_t ru = rsrc(static_cast<const uint8_t*>(U) + t * u_pitch * EB, (uint32_t)D * EB);
  const __amdgpu_buffer_rsrc_t rp = rsrc(p + t * p_pitch, (uint32_t)D * 2u);
  uint4 wq[Q];
  u32x4_t uq[F24 ? 1 : Q];
  u32x3_t uq3[F24 ? Q : 1];
  u32x2_t pq[Q];
  uint32_t o16[Q];  // the quad's byte offset in an fp32 row (past the row end: reads zeros, stores dropped)
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    const int q = tid + k * (int)blockDim.x;
    o16[k] = q < V4 ? (uint32_t)q * 16u : 0xFFFFFFF0u;
    wq[k] = bload(rw, o16[k]);
  }
  sched_fence();
#pragma unroll
  for (int k = 0; k < Q; ++k) pq[k] = __builtin_amdgcn_raw_buffer_load_b64(rp, o16[k] / 2u, 0, kAuxStreamLoad);
  u32x2_t yq[UPDATE ? Q : 1];
  if constexpr (UPDATE) {
    const __amdgpu_buffer_rsrc_t ry = rsrc(delta + t * D, (uint32_t)D * 2u);
#pragma unroll
    for (int k = 0; k < Q; ++k) yq[k] = __builtin_amdgcn_raw_buffer_load_b64(ry, o16[k] / 2u, 0, kAuxStreamLoad);
  }
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    if constexpr (F24)  // 12 bytes per quad; past the row end (o16 = 0xFFFFFFF0): zeros
      uq3[k] = __builtin_amdgcn_raw_buffer_load_b96(ru, o16[k] == 0xFFFFFFF0u ? o16[k] : o16[k] / 4u * 3u, 0,
                                                    kAuxStreamLoad);
    else
      uq[k] = __builtin_amdgcn_raw_buffer_load_b128(ru, o16[k], 0, kAuxStreamLoad);
  }
  float zgv, rgv;
  {  // lane i: shared source i's given score and rstd (lanes >= N-1 read zeros)
    const int lane = lane_id();
    constexpr uint32_t gb = (uint32_t)(N - 1) * 4u;
    zgv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(zg + t * (N - 1), gb), lane * 4, 0, 0));
    rgv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(rg + t * (N - 1), gb), lane * 4, 0, 0));
  }
  sched_fence();
  if constexpr (UPDATE) {
    const __amdgpu_buffer_rsrc_t rq = rsrc(partial_out + t * p_pitch, (uint32_t)D * 2u);
#pragma unroll
    for (int k = 0; k < Q; ++k) {
      float a[4], b[4];
      unpack4(pq[k], a);
      unpack4(yq[k], b);
      const float s8[8] = {a[0] + b[0], a[1] + b[1], a[2] + b[2], a[3] + b[3], 0.f, 0.f, 0.f, 0.f};
      const uint4 pk = pack8(s8);
      pq[k].x = pk.x;
      pq[k].y = pk.y;
      __builtin_amdgcn_raw_buffer_store_b64(pq[k], rq, o16[k] / 2u, 0, kAuxStreamStore);
    }
  }
  clear_absent<2>(red);
  // the partial sum's sum of squares and w.p
  float part[2] = {0.f, 0.f};
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    const float4 wv = __builtin_bit_cast(float4, wq[k]);
    float f[4];
    unpack4(pq[k], f);
    part[0] = fmaf(f[0], f[0], part[0]);
    part[0] = fmaf(f[1], f[1], part[0]);
    part[0] = fmaf(f[2], f[2], part[0]);
    part[0] = fmaf(f[3], f[3], part[0]);
    part[1] = fmaf(wv.x, f[0], part[1]);
    part[1] = fmaf(wv.y, f[1], part[1]);
    part[1] = fmaf(wv.z, f[2], part[1]);
    part[1] = fmaf(wv.w, f[3], part[1]);
  }
  block_sums<2>(part, red[0]);

  // rstd, scores and softmax: the scored forward's sequence
  float r[N], a[N];
  float m = -INFINITY, ms = -INFINITY;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i < N - 1) {
      r[i] = uniform(lane_value(rgv, i));
      a[i] = uniform(lane_value(zgv, i));
      ms = fmaxf(ms, a[i]);
    } else {
      r[i] = uniform(__builtin_amdgcn_rsqf(part[0] * (1.0f / (float)D) + eps));
      a[i] = r[i] * part[1];
    }
    m = fmaxf(m, a[i]);
  }
  float den = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    a[i] = __expf(a[i] - m);
    den += a[i];
  }
  const float inv_den = 1.0f / den;
#pragma unroll
  for (int i = 0; i < N; ++i) a[i] = uniform(a[i] * inv_den);
  const float cs = uniform(__expf(ms - m) * inv_den);

  const __amdgpu_buffer_rsrc_t ro = rsrc(out + t * D, (uint32_t)D * 2u);
#pragma unroll
  for (int k = 0; k < Q; ++k) {
    float4 u;
    if constexpr (F24)
      u = unpack24(uq3[k]);
    else
      u = __builtin_bit_cast(float4, uq[k]);
    float f[4];
    unpack4(pq[k], f);
    const float acc[8] = {fmaf(a[N - 1], f[0], cs * u.x), fmaf(a[N - 1], f[1], cs * u.y),
                          fmaf(a[N - 1], f[2], cs * u.z), fmaf(a[N - 1], f[3], cs * u.w), 0.f, 0.f, 0.f, 0.f};
    const uint4 pk = pack8(acc);
    u32x2_t o;
    o.x = pk.x;
    o.y = pk.y;
    __builtin_amdgcn_raw_buffer_store_b64(o, ro, o16[k] / 2u, 0, kAuxStreamStore);
  }
  if (tid < N) {
    float rv = r[0], av = a[0];
#pragma unroll
    for (int i = 1; i < N; ++i) {
      rv = tid == i ? r[i] : rv;
      av = tid == i ? a[i] : av;
    }
    rstd_out[t * N + tid] = rv;
    alpha_out[t * N + tid] = av;
  }
}

// ---------------------------------------------------------------------------
// Backward: dsources and dw partial rows
// ---------------------------------------------------------------------------
// The launch has exactly P = min(T, 256) workgroups.  Workgroup c handles the
// tokens c, c + P, c + 2P, ... and sums their dw contributions in token order
// into partial row ws[c][:]; the split depends only on T, so dw does not
// depend on how many workgroups are resident at once.  Interleaving the tokens
// keeps the workgroups on neighbouring rows of each source at any moment
// (contiguous per-workgroup ranges measured 2-7% slower on MI355X: the HBM
// accesses of 256 separate streams per source are less local).

// Softmax backward, dz_i = alpha_i (da_i - s) with s = sum_j alpha_j da_j
// (da_i = g.x_i), evaluated without cancellation.  When one source holds
// nearly all the weight, s agrees with that source's da_i to within its
// fp32 rounding, and da_i - s formed directly loses the whole difference
// (alpha_m = 1 - 1e-10: the difference is 1e-10 of da_m, below an ulp) --
// and with it that source's dz, which carries as much of dw as the other
// sources' together.  With m the source of the largest weight (the first
// such), e_j = da_j - da_m and s' = sum_j alpha_j e_j, the same quantity is
// e_i - s' (the weights sum to 1), where no term cancels a much larger one.
// The da_i are the token's totals, the same in every lane.
// The weights are non-negative, so their bit patterns order like their
// values: the search for m runs on the scalar unit (the weights and the
// totals are wave-uniform), carrying da_m along instead of indexing by m.
template <int N>
__device__ __forceinline__ void softmax_bwd(const float (&al)[N], const float (&da)[N], float (&dz)[N]) {
  uint32_t best = __builtin_bit_cast(uint32_t, al[0]);
  float dam = da[0];
#pragma unroll
  for (int i = 1; i < N; ++i) {
    const uint32_t b = __builtin_bit_cast(uint32_t, al[i]);
    const bool gt = b > best;  // strictly: the first of equal weights stays m
    best = gt ? b : best;
    dam = gt ? da[i] : dam;
  }
  float e[N], sp = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    e[i] = da[i] - dam;
    sp = fmaf(al[i], e[i], sp);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) dz[i] = al[i] * (e[i] - sp);
}

struct BwdCtx {
  int64_t T;
  int32_t D;
  float inv_d;
  DstRows dsrc;
  const float4* wl;
  float4* dwl;
  float (*red)[kMaxWaves];
  float4* stage;  // written fp32 gradients, one vector per thread: 2 KiB per wave
};

// Backward of token t whose sources and dout are already in x and g:
// g.x_i and w.x_i, workgroup reduction, softmax backward, dsources stores and
// this workgroup's running dw (LDS).  Issues no loads of the row group.
// MODE (kGradAccumulate | kGradF32): with accumulation the old gradients are
// requested once the partial sums are formed (in flight during the reduction
// but not live during the first pass; below, how many and when) and the new
// gradient is added to them in fp32 before the single rounding (bf16) or
// store (fp32).
template <int N, int VPT, int MODE>
__device__ __forceinline__ void bwd_token(uint4 (&x)[N][VPT], uint4 (&g)[VPT], float sa, float sr, int64_t t,
                                          int& buf, const BwdCtx& c, const Slice<VPT>& sl) {
  constexpr bool ACC = (MODE & kGradAccumulate) != 0;
  constexpr bool F32 = (MODE & kGradF32) != 0;
  constexpr int OW = F32 ? 2 : 1;  // 16-byte vectors of old gradient per slice vector
  // Accumulation with one vector per thread: the old gradients of the first H
  // sources are requested before the reduction (all of them for bf16, half
  // for fp32, whose old rows take twice the registers) and the other R when
  // the stores reach source H.
  constexpr int H = F32 ? (N + 1) / 2 : N;
  constexpr int R = N - H;
  // Accumulation with two vectors per thread (D > 8192): two vectors of old
  // gradients next to two of sources exceed the 128 VGPRs of a 1024-thread
  // workgroup, so the old gradients roll through a window of W items instead:
  // W are requested before the reduction, and each one the stores consume is
  // replaced by the request for the item W later (item j = k*N + i: slice
  // vector k of source i).  Measured on MI355X at D = 12288 / 16384: bf16
  // 3.55 -> 5.15 TB/s, fp32 4.5 -> 4.6 TB/s; with one vector per thread the
  // loads above (all early for bf16, half early for fp32) stay faster.
  constexpr bool ROLL = ACC && VPT > 1;
  constexpr int W = F32 ? 3 : 4;
  // request the old gradient of item j into dst
  auto load_item = [&](uint4 (&dst)[OW], int j) {
    const __amdgpu_buffer_rsrc_t r = grad_row<F32>(c.dsrc, j % N, t, c.D);
    if constexpr (F32) {
      dst[0] = bload(r, 2u * sl.off[j / N]);
      dst[OW - 1] = bload(r, 2u * sl.off[j / N] + 16u);
    } else {
      dst[0] = bload<kAuxStreamLoad>(r, sl.off[j / N]);
    }
  };

  // partial g.x_i (first N) and w.x_i (last N)
  float part[2 * N];
#pragma unroll
  for (int i = 0; i < 2 * N; ++i) part[i] = 0.f;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    float wr[8];
    load8(c.wl, sl.slot[k], wr);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      float f[8];
      unpack8(x[i][k], f);
      part[i] = dot8_bf16(g[k], x[i][k], part[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) part[N + i] = fmaf(wr[e], f[e], part[N + i]);
    }
  }
  static_assert(ROLL || !ACC || VPT == 1, "two vectors per thread accumulate through the window");
  uint4 old[(ACC && !ROLL) ? H : 1][OW];
  uint4 win[ROLL ? W : 1][OW];
  if constexpr (ACC) {
    sched_fence();
    if constexpr (ROLL) {
#pragma unroll
      for (int j = 0; j < W && j < VPT * N; ++j) load_item(win[j], j);
    } else {
      load_grads<F32, 0, H>(old, c.dsrc, t, c.D, sl, 0);
    }
    sched_fence();
  }
  block_sums<2 * N>(part, c.red + buf * 2 * N);
  buf ^= 1;
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    opaque(g[k]);
#pragma unroll
    for (int i = 0; i < N; ++i) opaque(x[i][k]);
  }

  // softmax backward: dz_i = alpha_i (da_i - sum_j alpha_j da_j), da_i = part[i]
  float al[N], c1[N], kx[N], da[N], dzv[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    al[i] = lane_value(sa, i);
    da[i] = part[i];
  }
  softmax_bwd<N>(al, da, dzv);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float rs = lane_value(sr, i);
    const float dz = dzv[i];
    const float z = rs * part[N + i];
    // dx_id = alpha_i g_d + c1 (w_d - kx x_id): c1 = dz rstd, kx = z rstd / D.
    // The bracket is formed first, so no intermediate carries rstd^2 (with
    // eps = 0 and a row of rms ~1e-15, dz rstd^2 alone would overflow fp32
    // while dx itself is representable).
    c1[i] = uniform(dz * rs);           // coefficient of the bracket in dx and of x_id in dw
    kx[i] = uniform(z * rs * c.inv_d);  // coefficient of x_id inside the bracket
    al[i] = uniform(al[i]);
  }

#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    float gf[8], wr[8], dwr[8];
    unpack8(g[k], gf);
    load8(c.wl, sl.slot[k], wr);
    load8(c.dwl, sl.slot[k], dwr);
    uint4 rest[(ACC && F32 && R > 0 && !ROLL) ? R : 1][OW];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if constexpr (ACC && F32 && R > 0 && !ROLL) {
        if (i == H) {
          sched_fence();
          load_grads<true, H, N>(rest, c.dsrc, t, c.D, sl, k);
          sched_fence();
        }
      }
      float f[8], d[8];
      unpack8(x[i][k], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        d[e] = fmaf(c1[i], fmaf(-kx[i], f[e], wr[e]), al[i] * gf[e]);
        dwr[e] = fmaf(c1[i], f[e], dwr[e]);
      }
      if constexpr (ACC) {
        float o[8];
        if constexpr (ROLL) {
          const int j = k * N + i;
          if constexpr (F32) {
            const uint4& a = win[j % W][0];
            const uint4& b = win[j % W][OW - 1];
            o[0] = __builtin_bit_cast(float, a.x); o[1] = __builtin_bit_cast(float, a.y);
            o[2] = __builtin_bit_cast(float, a.z); o[3] = __builtin_bit_cast(float, a.w);
            o[4] = __builtin_bit_cast(float, b.x); o[5] = __builtin_bit_cast(float, b.y);
            o[6] = __builtin_bit_cast(float, b.z); o[7] = __builtin_bit_cast(float, b.w);
          } else {
            unpack8(win[j % W][0], o);
          }
          if (j + W < VPT * N) {
            // fenced, or the scheduler hoists every later request to the top
            // and the window is gone
            sched_fence();
            load_item(win[j % W], j + W);
            sched_fence();
          }
        } else if constexpr (F32) {
          const uint4& a = i < H ? old[i < H ? i : 0][0] : rest[i < H ? 0 : i - H][0];
          const uint4& b = i < H ? old[i < H ? i : 0][1] : rest[i < H ? 0 : i - H][1];
          o[0] = __builtin_bit_cast(float, a.x); o[1] = __builtin_bit_cast(float, a.y);
          o[2] = __builtin_bit_cast(float, a.z); o[3] = __builtin_bit_cast(float, a.w);
          o[4] = __builtin_bit_cast(float, b.x); o[5] = __builtin_bit_cast(float, b.y);
          o[6] = __builtin_bit_cast(float, b.z); o[7] = __builtin_bit_cast(float, b.w);
        } else {
          unpack8(old[i][0], o);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) d[e] = o[e] + d[e];
      }
      const __amdgpu_buffer_rsrc_t rd = grad_row<F32>(c.dsrc, i, t, c.D);
      if constexpr (F32 && !ACC && VPT == 1) {
        // written fp32 gradients: the wave's 64 x 32 bytes pass through its
        // LDS stage so that each store instruction writes one contiguous KiB
        // (lane l: bytes [16 l, 16 l + 16) and [1024 + 16 l, ...) of the
        // wave's 2 KiB) and can carry the streaming hint; 4-5% faster on
        // MI355X than two half-vector stores merged in L2 (bitwise the same
        // values).  The accumulating variant keeps the plain stores: its
        // registers are full and the stage cost it 1-2%.
        // The exchange is between lanes of one wave, so a wave barrier (with
        // wavefront-scope fences) orders the stage's writes before the reads
        // of other lanes' data, and the reads before the next source's writes.
        const int lane = lane_id();
        float4* st = c.stage + wave_id() * (2 * kWave);
        st[2 * lane] = make_float4(d[0], d[1], d[2], d[3]);
        st[2 * lane + 1] = make_float4(d[4], d[5], d[6], d[7]);
        wave_sync();
        const float4 lo = st[lane], hi = st[kWave + lane];
        wave_sync();
        const uint32_t wbase = 2u * sl.off[k] - 32u * (uint32_t)lane;  // the wave's first vector, fp32 bytes
        bstore<kAuxStreamStore>(rd, wbase + 16u * (uint32_t)lane, __builtin_bit_cast(uint4, lo));
        bstore<kAuxStreamStore>(rd, wbase + 1024u + 16u * (uint32_t)lane, __builtin_bit_cast(uint4, hi));
      } else if constexpr (F32) {
        // two 16-byte halves per lane, 32 bytes apart between lanes: default
        // policy, so L2 merges the halves into whole lines before they go out
        bstore(rd, 2u * sl.off[k], make_uint4(__builtin_bit_cast(uint32_t, d[0]),
                                                               __builtin_bit_cast(uint32_t, d[1]),
                                                               __builtin_bit_cast(uint32_t, d[2]),
                                                               __builtin_bit_cast(uint32_t, d[3])));
        bstore(rd, 2u * sl.off[k] + 16u, make_uint4(__builtin_bit_cast(uint32_t, d[4]),
                                                                     __builtin_bit_cast(uint32_t, d[5]),
                                                                     __builtin_bit_cast(uint32_t, d[6]),
                                                                     __builtin_bit_cast(uint32_t, d[7])));
      } else {
        bstore<kAuxStreamStore>(rd, sl.off[k], pack8(d));
      }
    }
    store8(c.dwl, sl.slot[k], dwr);
  }
}

// Publish this workgroup's dw partial row (the sum over its tokens).
template <int VPT>
__device__ __forceinline__ void publish_dw(float* __restrict__ ws, int64_t ch, int32_t D, const float4* dwl,
                                           const Slice<VPT>& sl) {
  const __amdgpu_buffer_rsrc_t rw = rsrc(ws + ch * D, (uint32_t)D * 4u);
#pragma unroll
  for (int k = 0; k < VPT; ++k) {
    bstore(rw, 2u * sl.off[k], __builtin_bit_cast(uint4, dwl[2 * sl.slot[k]]));
    bstore(rw, 2u * sl.off[k] + 16u, __builtin_bit_cast(uint4, dwl[2 * sl.slot[k] + 1]));
  }
}

// With PIPE, two register sets A and B alternate: while the workgroup works
// on the token in one set, the next token's loads are in flight in the other,
// and a set is refilled with the workgroup's token two steps ahead as soon as
// its token is done.  Loads past the last token use size-0 descriptors and
// scheduling fences keep each prefetch where it is issued, so the in-order
// wait counts only ever wait for the oldest row group.  When accumulating
// (no prefetch) the old gradients are loaded during the reduction.  Dynamic LDS
// holds w and the workgroup's running dw, in the thread's private slots, and
// for written fp32 gradients a 2 KiB output stage per wave.
template <int N, int VPT, bool PIPE, int MODE>
__global__ void __launch_bounds__(1024) bwd_kernel(const uint16_t* __restrict__ dout, SrcRows src,
                                                   const float* __restrict__ w, const float* __restrict__ rstd,
                                                   const float* __restrict__ alpha, int64_t T, int32_t D, int32_t P,
                                                   DstRows dsrc, float* __restrict__ ws) {
  static_assert(!(PIPE && (MODE & kGradAccumulate)), "the accumulating variants do not prefetch");
  __shared__ __attribute__((aligned(16))) float red[2][2 * N][kMaxWaves];
  extern __shared__ float4 dyn_lds[];
  BwdCtx c;
  c.T = T;
  c.D = D;
  c.inv_d = 1.0f / (float)D;
  c.dsrc = dsrc;
  c.wl = dyn_lds;
  c.dwl = dyn_lds + 2 * VPT * (int)blockDim.x;
  c.stage = dyn_lds + 4 * VPT * (int)blockDim.x;  // after w and dw (used only by the written fp32 gradients)
  c.red = &red[0][0];
  const int tid = threadIdx.x;
  const Slice<VPT> sl(tid, blockDim.x, D);
  const int64_t ch = blockIdx.x;  // host launches exactly P <= T workgroups

  // w first, then (with PIPE) the first token's rows right behind it, so the
  // set-up below overlaps their latency
  uint4 wv[VPT][2];
  load_w<VPT>(wv, w, D, sl);
  sched_fence();
  uint4 xa[PIPE ? N : 1][VPT], xb[PIPE ? N : 1][VPT], ga[VPT], gb[VPT];
  float saa = 0.f, sra = 0.f, sab = 0.f, srb = 0.f;
  if constexpr (PIPE) {
    load_row<VPT>(ga, dout, ch, D, sl);
    load_rows<N, VPT>(xa, src, ch, D, sl);
    load_saved<N>(saa, sra, alpha, rstd, ch);
    sched_fence();
  }
  store_w<VPT>(wv, dyn_lds, sl);
  const float zero8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < VPT; ++k) store8(c.dwl, sl.slot[k], zero8);
  clear_red<2 * N>(red);

  int buf = 0;
  if constexpr (PIPE) {
    int64_t t = ch;
    load_row<VPT>(gb, dout, t + P, D, sl, t + P < T);
    load_rows<N, VPT>(xb, src, t + P, D, sl, t + P < T);
    load_saved<N>(sab, srb, alpha, rstd, t + P, t + P < T);
    sched_fence();
    while (true) {
      bwd_token<N, VPT, MODE>(xa, ga, saa, sra, t, buf, c, sl);
      sched_fence();
      load_row<VPT>(ga, dout, t + 2 * P, D, sl, t + 2 * P < T);
      load_rows<N, VPT>(xa, src, t + 2 * P, D, sl, t + 2 * P < T);
      load_saved<N>(saa, sra, alpha, rstd, t + 2 * P, t + 2 * P < T);
      sched_fence();
      t += P;
      if (t >= T) break;
      bwd_token<N, VPT, MODE>(xb, gb, sab, srb, t, buf, c, sl);
      sched_fence();
      load_row<VPT>(gb, dout, t + 2 * P, D, sl, t + 2 * P < T);
      load_rows<N, VPT>(xb, src, t + 2 * P, D, sl, t + 2 * P < T);
      load_saved<N>(sab, srb, alpha, rstd, t + 2 * P, t + 2 * P < T);
      sched_fence();
      t += P;
      if (t >= T) break;
    }
  } else {
    for (int64_t t = ch; t < T; t += P) {
      uint4 x[N][VPT], g[VPT];
      float sa, sr;
      load_row<VPT>(g, dout, t, D, sl);
      load_rows<N, VPT>(x, src, t, D, sl);
      load_saved<N>(sa, sr, alpha, rstd, t);
      bwd_token<N, VPT, MODE>(x, g, sa, sr, t, buf, c, sl);
    }
  }
  publish_dw<VPT>(ws, ch, D, c.dwl, sl);
}

// ---------------------------------------------------------------------------
// dw stage 2: dw[d] = sum_{p<P} ws[p][d], fixed order
// ---------------------------------------------------------------------------
// A workgroup of kReduceThreads threads covers kReduceCols consecutive float4
// columns (256 B of each partial row); thread (c, g) = (tid % kReduceCols, tid / kReduceCols) sums rows
// g, g + kReduceGroups, g + 2*kReduceGroups, ... in increasing order (all loads
// issued first), then thread group g = 0 adds the kReduceGroups group sums in
// group order.  Requires P <= kReduceGroups * kReduceRows.
constexpr int kReduceCols = 16;
constexpr int kReduceGroups = 16;
constexpr int kReduceThreads = kReduceCols * kReduceGroups;
constexpr int kReduceRows = ATTNRES_DW_PARTIALS / kReduceGroups;

__global__ void __launch_bounds__(kReduceThreads) dw_reduce_kernel(const float4* __restrict__ ws, int32_t P,
                                                                    int32_t D4, float4* __restrict__ dw) {
  __shared__ float4 part[kReduceGroups][kReduceCols];
  const int cl = threadIdx.x % kReduceCols;
  const int g = threadIdx.x / kReduceCols;
  const int c = blockIdx.x * kReduceCols + cl;  // float4 column
  const bool col_ok = c < D4;
  float4 v[kReduceRows];
#pragma unroll
  for (int j = 0; j < kReduceRows; ++j) {
    const int p = g + j * kReduceGroups;
    v[j] = (col_ok && p < P) ? ws[(int64_t)p * D4 + c] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 s = v[0];
#pragma unroll
  for (int j = 1; j < kReduceRows; ++j) {
    s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w;
  }
  part[g][cl] = s;
  __syncthreads();
  if (g == 0 && col_ok) {
    float4 t = part[0][cl];
#pragma unroll
    for (int r = 1; r < kReduceGroups; ++r) {
      const float4 u = part[r][cl];
      t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
    }
    dw[c] = t;
  }
}

// ---------------------------------------------------------------------------
// Backward with tokens split over workgroups (where ATTNRES_BWD_SPLIT(N, D))
// ---------------------------------------------------------------------------
// Each token's D channels are cut into K slices of 128 16-byte vectors, and a
// workgroup takes one slice of ATTNRES_SPLIT_TOKENS consecutive tokens side
// by side (4 x 128 threads, one vector per thread): workgroup b = span * K +
// slice.  Measured on MI355X, the memory system moves the backward's 19 row
// streams faster when each token is spread over K short-lived workgroups than
// when one workgroup walks whole tokens (5.4-5.8 vs 5.1-5.4 TB/s over
// 32K-256K tokens at N = 9, D = 7168), and 512-thread workgroups (two per CU
// at this kernel's register use) beat 1024-thread ones, whose tails leave
// the CU idle, and workgroups that walk two or four such spans in turn.
// With fewer sources a token carries less work per exchange: at T = 32768
// the one-token backward was faster for N <= 7 at D = 2048-7168 (up to 1.5x
// at N = 1) and at D = 8192 for every N, the split one for N >= 8 up to
// D = 7168 and for every N at D = 1024 (1.3-1.7x); ATTNRES_BWD_SPLIT in the
// header encodes that choice, which depends on (N, D) alone.
//
// The per-token sums g.x_i and w.x_i then span K workgroups.  Each member
// publishes its slice's 2N partial sums as 64-bit {tag, value} words in a
// ring indexed by token (tag = token + 1; the ring is zeroed by the host
// before the launch), agent-scope relaxed atomics, and reads the other
// members' words, spinning with a bound.  Members are consecutive workgroups,
// dispatched together, and walk their rounds in step.  Should a word not
// arrive within the bound (a member not resident, e.g. the device shared with
// other work), the waiting workgroup recomputes that member's partial sums
// from HBM with the same per-slice reduction tree, so the result does not
// depend on which route was taken.  The totals are the K partials added in
// member order: every token's reduction tree depends only on (N, D), as in
// the other kernels.
//
// dw: the workgroup sums its tokens' contributions to its slice in side
// order and writes one partial row slice per span.  The spans run in chunks
// of ATTNRES_SPLIT_CHUNK_SPANS (one launch each), and after each chunk
// dw_fold_kernel adds the chunk's partial rows into at most 256 fold rows;
// dw_reduce_kernel sums those in index order.  The order depends on T alone
// and no atomics touch dw.  A chunk's partial rows (235 MB at D = 7168) stay
// in the 256 MB Infinity Cache until the fold reads them: measured on MI355X
// at N = 9, one launch over all spans was 3% slower at T = 128K-256K, when
// the partial rows of the whole batch (0.9-1.9 GB) went to HBM and back, and
// chunks of 12K or 16K spans lost the gain again.
constexpr int kSpSliceVectors = 128;                        // vectors (threads) per slice
constexpr int kSpSide = ATTNRES_SPLIT_TOKENS;               // tokens side by side
constexpr int kSpThreads = kSpSliceVectors * kSpSide;       // 512
constexpr int kSpRing = ATTNRES_SPLIT_RING;                 // exchange ring, tokens
constexpr int kSpMaxSlices = ATTNRES_SPLIT_MAX_D / 8 / kSpSliceVectors;  // 8
constexpr uint32_t kSpSpin = ATTNRES_SPLIT_SPIN_DEFAULT;    // polls before a word is recomputed
constexpr int kSpFirstPollSleep = 48;                       // s_sleep units (64 cycles) before the first poll
constexpr int64_t kSpChunk = ATTNRES_SPLIT_CHUNK_SPANS;     // spans per launch and fold
static_assert(kSpRing % kSpSide == 0, "ring of whole spans");

// The poll bound the next split-backward launches use (attnres_set_split_spin).
std::atomic<uint32_t> g_split_spin{kSpSpin};

struct SplitArgs {
  const uint16_t* dout;
  SrcRows src;
  const float* w;
  const float* rstd;
  const float* alpha;
  int64_t T;
  int32_t D;
  int32_t K;  // slices per row
  DstRows dsrc;
  uint64_t* ring;   // [kSpRing][K][2N] words
  float* partial;   // [ATTNRES_SPLIT_PARTIAL_ROWS(T)][D]: one row per span of the chunk
  int64_t s0;       // first token span of this launch
  int64_t p0;       // the span whose dw partial row is partial[0] (first span of the chunk)
  uint32_t spin;    // polls before a member's word is recomputed
};

// This thread's partial g.x_i and w.x_i over its vector of source i: v_dot2
// on the bf16 pairs, fp32 FMAs for w (the plain backward's per-thread
// arithmetic).  Used by both routes to a member's partial sums, so they agree
// bit for bit.
__device__ __forceinline__ void split_partial(float& gx, float& wx, const uint4& x, const uint4& g,
                                              const float (&wr)[8]) {
  float f[8];
  unpack8(x, f);
  gx = dot8_bf16(g, x, 0.f);
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) a = fmaf(wr[e], f[e], a);
  wx = a;
}

template <int N>
__device__ __forceinline__ void split_partials(float (&part)[2 * N], const uint4 (&x)[N], const uint4& g,
                                               const float (&wr)[8]) {
#pragma unroll
  for (int i = 0; i < N; ++i) split_partial(part[i], part[N + i], x[i], g, wr);
}

// Wave sums of part[], complete in lane 63, into red[side][half][j].
template <int N>
__device__ __forceinline__ void split_wave_sums(float (&part)[2 * N], float (*red)[2][2 * N], int side, int half) {
#pragma unroll
  for (int j = 0; j < 2 * N; ++j) part[j] = wave_sum_lane63(part[j]);
  if (lane_id() == kWave - 1) {
#pragma unroll
    for (int j = 0; j < 2 * N; ++j) red[side][half][j] = part[j];
  }
}

template <int N, int MODE>
__global__ void __launch_bounds__(kSpThreads) bwd_split_kernel(SplitArgs a) {
  constexpr bool ACC = (MODE & kGradAccumulate) != 0;
  constexpr bool F32 = (MODE & kGradF32) != 0;
  constexpr int OW = F32 ? 2 : 1;
  constexpr int H = F32 ? (N + 1) / 2 : N;  // accumulating: old gradients of the first H sources early
  __shared__ float red[kSpSide][2][2 * N];                                  // per-wave sums
  __shared__ float words[kSpSide][kSpMaxSlices][2 * N];                     // the K members' partials
  __shared__ float tot[kSpSide][2 * N];
  __shared__ int redo[kSpSide][kSpMaxSlices];                               // members to recompute
  __shared__ int any_redo;
  __shared__ __attribute__((aligned(16))) float4 dws[kSpSide][kSpSliceVectors][2];

  const int tid = threadIdx.x;
  // a side is two whole waves: its index is wave-uniform, and saying so keeps
  // every token address (and the buffer descriptors made from it) scalar
  const int side = __builtin_amdgcn_readfirstlane(tid / kSpSliceVectors);
  const int tl = tid % kSpSliceVectors;
  const int half = __builtin_amdgcn_readfirstlane(tl / kWave);  // wave within the side
  const int K = a.K;
  const int64_t span = a.s0 + blockIdx.x / K;
  const int k = (int)(blockIdx.x % K);
  const int32_t D = a.D;
  const int V = D / 8;
  const int v = k * kSpSliceVectors + tl;
  const uint32_t off = v < V ? (uint32_t)v * 16u : 0xFFFFFFF0u;  // past the row: zeros, stores dropped

  // this thread's 8 elements of w (the slice is read by every side: L2 hits)
  float wr[8];
  {
    const __amdgpu_buffer_rsrc_t rw = rsrc(a.w, (uint32_t)D * 4u);
    const uint4 w0 = bload(rw, 2u * off), w1 = bload(rw, 2u * off + 16u);
    wr[0] = __builtin_bit_cast(float, w0.x); wr[1] = __builtin_bit_cast(float, w0.y);
    wr[2] = __builtin_bit_cast(float, w0.z); wr[3] = __builtin_bit_cast(float, w0.w);
    wr[4] = __builtin_bit_cast(float, w1.x); wr[5] = __builtin_bit_cast(float, w1.y);
    wr[6] = __builtin_bit_cast(float, w1.z); wr[7] = __builtin_bit_cast(float, w1.w);
  }

  const int64_t t = span * kSpSide + side;
  const bool valid = t < a.T;  // uniform over the side's two waves
  const int64_t tt = valid ? t : 0;
  const uint32_t row_bytes = valid ? (uint32_t)D * 2u : 0u;

  // this side's rows, dout, and the saved alpha / rstd (lane i: source i) of its token
  uint4 g = bload<kAuxStreamLoad>(rsrc(a.dout + tt * D, row_bytes), off);
  uint4 x[N];
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = bload<kAuxStreamLoad>(rsrc(a.src.p[i] + tt * a.src.pitch, row_bytes), off);
  float sa, sr;
  load_saved<N>(sa, sr, a.alpha, a.rstd, t, valid);
  sched_fence();
  if (tid < kSpSide * kSpMaxSlices) redo[tid / kSpMaxSlices][tid % kSpMaxSlices] = 0;
  if (tid == 0) any_redo = 0;

  // this member's partial sums of its slice
  float part[2 * N];
  split_partials<N>(part, x, g, wr);
  split_wave_sums<N>(part, red, side, half);
  __syncthreads();
  uint64_t* ring = a.ring + (t % kSpRing) * (int64_t)K * (2 * N);
  const uint32_t tag = (uint32_t)t + 1u;
  const bool alone = K == 1;  // one slice per row (D <= 1024): no other member to wait for
  if (valid && tl < 2 * N) {
    const float p = red[side][0][tl] + red[side][1][tl];
    if (alone) {
      words[side][0][tl] = p;  // the value the ring would carry
    } else {
      const uint64_t word = ((uint64_t)tag << 32) | __builtin_bit_cast(uint32_t, p);
      __hip_atomic_store(ring + k * (2 * N) + tl, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // the K members' words, member by member (this one's included).  The
  // members start within about a microsecond of each other, so the first poll
  // waits ~3000 cycles: polling at once mostly reads words not yet written,
  // and those device-coherent reads compete with the row traffic (measured on
  // MI355X at N = 9, D = 7168: 2-3% faster at T = 4K-128K than polling at
  // once; longer waits were slower again).
  if (valid && !alone) {
    if (a.spin > 0) __builtin_amdgcn_s_sleep(kSpFirstPollSleep);
    for (int q = tl; q < K * 2 * N; q += kSpSliceVectors) {
      uint64_t word = 0;
      bool got = false;
      for (uint32_t n = 0; n < a.spin; ++n) {
        word = __hip_atomic_load(ring + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(word >> 32) == tag) {
          got = true;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      words[side][q / (2 * N)][q % (2 * N)] = __builtin_bit_cast(float, (uint32_t)word);
      if (!got) {
        redo[side][q / (2 * N)] = 1;
        any_redo = 1;
      }
    }
  }
  __syncthreads();
  if (any_redo) {
    // recompute the missing members' partial sums from HBM, with the
    // member's own per-thread arithmetic and wave tree: every side runs the
    // loop (its barriers are workgroup-wide), only sides missing member m load
    for (int m = 0; m < K; ++m) {
      const bool mine = redo[side][m] != 0;
      float pm[2 * N];
      if (mine) {  // source by source: one row of member m in registers at a time
        const int vm = m * kSpSliceVectors + tl;
        const uint32_t om = vm < V ? (uint32_t)vm * 16u : 0xFFFFFFF0u;
        const __amdgpu_buffer_rsrc_t rw = rsrc(a.w, (uint32_t)D * 4u);
        const uint4 wa = bload(rw, 2u * om), wb = bload(rw, 2u * om + 16u);
        const float wm[8] = {__builtin_bit_cast(float, wa.x), __builtin_bit_cast(float, wa.y),
                             __builtin_bit_cast(float, wa.z), __builtin_bit_cast(float, wa.w),
                             __builtin_bit_cast(float, wb.x), __builtin_bit_cast(float, wb.y),
                             __builtin_bit_cast(float, wb.z), __builtin_bit_cast(float, wb.w)};
        const uint4 gm = bload(rsrc(a.dout + tt * D, row_bytes), om);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const uint4 xm = bload(rsrc(a.src.p[i] + tt * a.src.pitch, row_bytes), om);
          split_partial(pm[i], pm[N + i], xm, gm, wm);
        }
        split_wave_sums<N>(pm, red, side, half);
      }
      __syncthreads();
      if (mine && tl < 2 * N) words[side][m][tl] = red[side][0][tl] + red[side][1][tl];
      __syncthreads();
    }
    // this route is rare: the side's own rows are loaded again instead of
    // being held in registers across the recomputation
    g = bload<kAuxStreamLoad>(rsrc(a.dout + tt * D, row_bytes), off);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = bload<kAuxStreamLoad>(rsrc(a.src.p[i] + tt * a.src.pitch, row_bytes), off);
  }
  // the token's totals: the K partials in member order
  if (tl < 2 * N) {
    float s = 0.f;
    for (int m = 0; m < K; ++m) s += words[side][m][tl];
    tot[side][tl] = valid ? s : 0.f;
  }
  __syncthreads();

  // accumulating: old gradients of the first H sources (the rest after the
  // first H are stored, in the registers those sources free)
  uint4 old[ACC ? H : 1][OW];
  if constexpr (ACC) {
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const __amdgpu_buffer_rsrc_t r = grad_row<F32>(a.dsrc, i, tt, valid ? D : 0);
      if constexpr (F32) {
        old[i][0] = bload(r, 2u * off);
        old[i][OW - 1] = bload(r, 2u * off + 16u);
      } else {
        old[i][0] = bload<kAuxStreamLoad>(r, off);
      }
    }
  }

  // softmax backward (every lane evaluates the N-value formulas, as the other kernels)
  // (the side's two waves hold the same token: these values are wave-uniform)
  float al[N], c1[N], kx[N], da[N], dzv[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    al[i] = lane_value(sa, i);
    da[i] = uniform(tot[side][i]);
  }
  softmax_bwd<N>(al, da, dzv);
  const float inv_d = 1.0f / (float)D;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float rs = lane_value(sr, i);
    const float dz = dzv[i];
    const float z = rs * uniform(tot[side][N + i]);
    // dx_id = alpha_i g_d + c1 (w_d - kx x_id): the bracket is formed first, so
    // no intermediate carries rstd^2 (see the plain backward)
    c1[i] = uniform(dz * rs);           // coefficient of the bracket in dx and of x_id in dw
    kx[i] = uniform(z * rs * inv_d);    // coefficient of x_id inside the bracket
    al[i] = uniform(al[i]);
  }

  // dsources and this token's dw contribution (none from a token past T)
  float gf[8], dwr[8];
  unpack8(g, gf);
#pragma unroll
  for (int e = 0; e < 8; ++e) dwr[e] = 0.f;
  uint4 rest[(ACC && H < N) ? N - H : 1][OW];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if constexpr (ACC && H < N) {
      if (i == H) {
        sched_fence();
#pragma unroll
        for (int j = H; j < N; ++j) {
          const __amdgpu_buffer_rsrc_t r = grad_row<F32>(a.dsrc, j, tt, valid ? D : 0);
          rest[j - H][0] = bload(r, 2u * off);
          rest[j - H][OW - 1] = bload(r, 2u * off + 16u);
        }
        sched_fence();
      }
    }
    float f[8], d[8];
    unpack8(x[i], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      d[e] = fmaf(c1[i], fmaf(-kx[i], f[e], wr[e]), al[i] * gf[e]);
      dwr[e] = valid ? fmaf(c1[i], f[e], dwr[e]) : dwr[e];
    }
    if constexpr (ACC) {
      float o[8];
      if constexpr (F32) {
        const uint4& p0 = i < H ? old[i < H ? i : 0][0] : rest[i < H ? 0 : i - H][0];
        const uint4& p1 = i < H ? old[i < H ? i : 0][OW - 1] : rest[i < H ? 0 : i - H][OW - 1];
        o[0] = __builtin_bit_cast(float, p0.x); o[1] = __builtin_bit_cast(float, p0.y);
        o[2] = __builtin_bit_cast(float, p0.z); o[3] = __builtin_bit_cast(float, p0.w);
        o[4] = __builtin_bit_cast(float, p1.x); o[5] = __builtin_bit_cast(float, p1.y);
        o[6] = __builtin_bit_cast(float, p1.z); o[7] = __builtin_bit_cast(float, p1.w);
      } else {
        unpack8(old[i][0], o);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) d[e] = o[e] + d[e];
    }
    if (valid) {
      const __amdgpu_buffer_rsrc_t rd = grad_row<F32>(a.dsrc, i, t, D);
      if constexpr (F32 && !ACC) {
        // written fp32 gradients: the wave's 64 x 32 bytes pass through an LDS
        // stage (the wave's part of dws, free until the dw sums) so that each
        // store writes one contiguous KiB with the streaming hint, as in the
        // one-token backward; wave barriers order the lanes' exchange
        const int lane = lane_id();
        float4* st = &dws[side][kWave * half][0];
        st[2 * lane] = make_float4(d[0], d[1], d[2], d[3]);
        st[2 * lane + 1] = make_float4(d[4], d[5], d[6], d[7]);
        wave_sync();
        const float4 lo = st[lane], hi = st[kWave + lane];
        wave_sync();
        // the wave's first vector in fp32 bytes; lanes past the row store past D * 4: dropped
        const uint32_t wbase = (uint32_t)(k * kSpSliceVectors + kWave * half) * 32u;
        bstore<kAuxStreamStore>(rd, wbase + 16u * (uint32_t)lane, __builtin_bit_cast(uint4, lo));
        bstore<kAuxStreamStore>(rd, wbase + 1024u + 16u * (uint32_t)lane, __builtin_bit_cast(uint4, hi));
      } else if constexpr (F32) {
        bstore(rd, 2u * off, make_uint4(__builtin_bit_cast(uint32_t, d[0]), __builtin_bit_cast(uint32_t, d[1]),
                                        __builtin_bit_cast(uint32_t, d[2]), __builtin_bit_cast(uint32_t, d[3])));
        bstore(rd, 2u * off + 16u, make_uint4(__builtin_bit_cast(uint32_t, d[4]), __builtin_bit_cast(uint32_t, d[5]),
                                              __builtin_bit_cast(uint32_t, d[6]), __builtin_bit_cast(uint32_t, d[7])));
      } else {
        bstore<kAuxStreamStore>(rd, off, pack8(d));
      }
    }
  }
  // dw: this slice's sum over the workgroup's tokens, in side order (each
  // lane writes only its own slots, which its wave's last stage reads, if any,
  // have passed: the wave barrier after them)
  dws[side][tl][0] = make_float4(dwr[0], dwr[1], dwr[2], dwr[3]);
  dws[side][tl][1] = make_float4(dwr[4], dwr[5], dwr[6], dwr[7]);
  __syncthreads();
  if (side == 0) {
    float4 s0 = dws[0][tl][0], s1 = dws[0][tl][1];
#pragma unroll
    for (int q = 1; q < kSpSide; ++q) {
      const float4 u0 = dws[q][tl][0], u1 = dws[q][tl][1];
      s0.x += u0.x; s0.y += u0.y; s0.z += u0.z; s0.w += u0.w;
      s1.x += u1.x; s1.y += u1.y; s1.z += u1.z; s1.w += u1.w;
    }
    const __amdgpu_buffer_rsrc_t rp = rsrc(a.partial + (span - a.p0) * D, (uint32_t)D * 4u);
    bstore(rp, 2u * off, __builtin_bit_cast(uint4, s0));
    bstore(rp, 2u * off + 16u, __builtin_bit_cast(uint4, s1));
  }
}

// dw stage 2a: fold row b (of P = min(spans, ATTNRES_DW_PARTIALS)) sums the
// partial rows of the spans s = b (mod P), in increasing s.  One launch
// covers the spans [c0, c0 + n) of one chunk, whose partial rows sit at
// partial[s - c0]; the first chunk writes the fold rows, later chunks add to
// them, so the order over all spans is fixed by T alone.  At any moment the
// workgroups read neighbouring rows; thread c owns float4 column c of its
// column block.
constexpr int kFoldCols = 256;  // float4 columns per workgroup
__global__ void __launch_bounds__(kFoldCols) dw_fold_kernel(const float4* __restrict__ partial, int64_t c0, int64_t n,
                                                            int32_t P, int32_t D4, int first,
                                                            float4* __restrict__ fold) {
  const int c = blockIdx.y * kFoldCols + threadIdx.x;
  if (c >= D4) return;
  const int b = blockIdx.x;
  float4 s = first ? make_float4(0.f, 0.f, 0.f, 0.f) : fold[(int64_t)b * D4 + c];
  const int64_t end = c0 + n;
  int64_t sp = c0 + ((b - c0 % P) % P + P) % P;  // the chunk's first span that is b (mod P)
  for (; sp + 3 * (int64_t)P < end; sp += 4 * (int64_t)P) {  // four loads in flight, added in span order
    const float4 u0 = partial[(sp - c0) * D4 + c], u1 = partial[(sp + P - c0) * D4 + c];
    const float4 u2 = partial[(sp + 2 * P - c0) * D4 + c], u3 = partial[(sp + 3 * P - c0) * D4 + c];
    s.x += u0.x; s.y += u0.y; s.z += u0.z; s.w += u0.w;
    s.x += u1.x; s.y += u1.y; s.z += u1.z; s.w += u1.w;
    s.x += u2.x; s.y += u2.y; s.z += u2.z; s.w += u2.w;
    s.x += u3.x; s.y += u3.y; s.z += u3.z; s.w += u3.w;
  }
  for (; sp < end; sp += P) {
    const float4 u = partial[(sp - c0) * D4 + c];
    s.x += u.x; s.y += u.y; s.z += u.z; s.w += u.w;
  }
  fold[(int64_t)b * D4 + c] = s;
}

__global__ void zero_kernel(float4* __restrict__ p, int32_t n4) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
struct LaunchShape {
  bool pipe;    // backward: prefetch the next token's rows into a second register set
  int vpt;      // 16-byte vectors per thread per row
  int threads;  // workgroup size
  size_t lds;   // dynamic LDS bytes per forward workgroup (backward: twice this)
};

// forward: four vectors per thread for 512 < D <= 8192 (256 threads at
// D = 7168: ceil(896 / 4) = 224 rounded up to whole waves), two above (at
// most 1024 threads) and at D <= 512
constexpr int kFwdVptMaxV4 = 1024;      // largest D/8 taking four vectors per thread
constexpr int kFwdVptMaxV2Small = 64;   // D/8 up to this takes two

LaunchShape make_shape(int32_t D, int vpt, bool pipe) {
  const int V = D / 8;
  LaunchShape s;
  s.pipe = pipe;
  s.vpt = vpt;
  const int need = (V + vpt - 1) / vpt;
  s.threads = ((need + kWave - 1) / kWave) * kWave;
  s.lds = (size_t)vpt * (size_t)s.threads * 32;
  return s;
}

// Both shapes depend only on D, so the per-token reduction trees never change
// with T or with the call: every forward call gives bitwise the same
// per-token results, and so does every backward call (with or without
// accumulation, stacked or per source).
// Forward: four vectors per thread for 512 < D <= 8192, else two; blockDim =
// D/(8*VPT) rounded up to whole waves.
// At D <= 512 four vectors per thread leave most lanes of the token's single
// wave idle and a 190-VGPR wave per token; two vectors measured 1.3-1.4x
// faster there (T = 65536, N = 3 and 9), while at D = 1024-2048 the shapes
// were within a few percent of each other.
LaunchShape fwd_shape(int32_t D) {
  const int V = D / 8;
  return make_shape(D, V <= kFwdVptMaxV2Small ? 2 : V <= kFwdVptMaxV4 ? 4 : 2, false);
}

// Backward: D <= 8192 takes one vector per thread (896 threads, 14 waves at
// D = 7168) with a two-token prefetch; measured 1-2% faster on MI355X than
// two vectors per thread with 7 waves.  Larger D takes two vectors per thread
// (up to 1024 threads) without prefetch.
LaunchShape bwd_shape(int32_t D) {
  const int V = D / 8;
  return V <= 1024 ? make_shape(D, 1, true) : make_shape(D, 2, false);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// The bytes a buffer argument covers: `rows` rows of `row_bytes` bytes, one
// every `pitch` bytes, from `lo` (a dense buffer is one row).
struct Range {
  uintptr_t lo;
  uint64_t rows, row_bytes, pitch;
};

Range range_of(const void* p, size_t bytes) { return Range{reinterpret_cast<uintptr_t>(p), 1, bytes, bytes}; }

Range rows_of(const void* p, int64_t rows, int64_t row_bytes, int64_t pitch_bytes) {
  return Range{reinterpret_cast<uintptr_t>(p), (uint64_t)rows, (uint64_t)row_bytes, (uint64_t)pitch_bytes};
}

uintptr_t range_end(const Range& a) { return a.lo + (a.rows - 1) * a.pitch + a.row_bytes; }

// Do two argument ranges share a byte?  Exact for dense buffers and for two
// row sets with the same pitch (their rows are compared modulo the pitch, so
// sources interleaved by token do not collide); conservative otherwise (any
// overlap of the spans counts).
bool overlap(const Range& a, const Range& b) {
  if (a.rows == 0 || a.row_bytes == 0 || b.rows == 0 || b.row_bytes == 0) return false;
  if (!(a.lo < range_end(b) && b.lo < range_end(a))) return false;
  if (a.rows > 1 && b.rows > 1 && a.pitch == b.pitch && a.row_bytes <= a.pitch && b.row_bytes <= a.pitch) {
    const uint64_t P = a.pitch;
    const uint64_t d = b.lo >= a.lo ? (b.lo - a.lo) % P : (P - (a.lo - b.lo) % P) % P;
    return d < a.row_bytes || d + b.row_bytes > P;  // b's row segment against a's, modulo the pitch
  }
  return true;
}

// A source pitch (elements between consecutive tokens' rows) must keep rows
// 16-byte aligned, not shorten them, and keep every offset well inside int64.
bool pitch_ok(int64_t pitch, int64_t T, int32_t D) {
  return pitch >= D && pitch % 8 == 0 && (T == 0 || pitch <= (INT64_C(1) << 41) / T);
}

bool sizes_ok(int32_t N, int64_t T, int32_t D) {
  if (N < 1 || N > ATTNRES_MAX_SOURCES) return false;
  if (T < 0) return false;
  if (D < 8 || D > ATTNRES_MAX_D || (D % 8) != 0) return false;
  // keep every byte offset well inside int64
  if (T > (INT64_C(1) << 40) / ((int64_t)N * D)) return false;
  return true;
}

// Resident workgroups of `fn` on the current device (occupancy x CUs).  The
// launches call it to validate their shape before enqueueing (a kernel that
// cannot be resident at that block size and LDS is refused with an error
// instead of failing at dispatch); grids are set by T and P, never by this
// count.  The answer is cached per (device, kernel, shape): the two runtime
// queries cost more host time than a small launch itself.
struct OccupancyEntry {
  const void* fn;
  int dev, threads;
  size_t lds;
  int64_t blocks;
};
constexpr int kOccupancySlots = 256;
std::mutex g_occupancy_mu;
OccupancyEntry g_occupancy[kOccupancySlots];
int g_occupancy_used = 0;

hipError_t resident_blocks(const void* fn, int threads, size_t lds, int64_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lock(g_occupancy_mu);
    for (int i = 0; i < g_occupancy_used; ++i) {
      const OccupancyEntry& o = g_occupancy[i];
      if (o.fn == fn && o.dev == dev && o.threads == threads && o.lds == lds) {
        *out = o.blocks;
        return hipSuccess;
      }
    }
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  *out = (int64_t)per_cu * cus;
  std::lock_guard<std::mutex> lock(g_occupancy_mu);
  if (g_occupancy_used < kOccupancySlots) g_occupancy[g_occupancy_used++] = OccupancyEntry{fn, dev, threads, lds, *out};
  return hipSuccess;
}

struct FwdArgs {
  SrcRows src;
  const uint16_t* delta;  // update: output added to the partial sum (src.p[N-1])
  uint16_t* partial_out;  // update: the new partial sum
  const float* zg;        // scored: given scores of the first N-1 sources, [T][N-1]
  const float* rg;        // scored: their rstd, [T][N-1]
  const float* w;
  float eps;
  int64_t T;
  int32_t D;
  uint16_t* out;
  float* rstd;
  float* alpha;
};

struct BwdArgs {
  const uint16_t* dout;
  SrcRows src;
  const float* w;
  const float* rstd;
  const float* alpha;
  int64_t T;
  int32_t D;
  int32_t P;
  DstRows dsrc;
  float* ws;
};

// One workgroup per token.  The dispatch packet counts work-items in 32 bits,
// so very large T (possible only for tiny D) is split over several launches.
template <int N, int VPT, int VARIANT>
hipError_t run_fwd_vpt(const LaunchShape& s, hipStream_t st, const FwdArgs& a) {
  const void* fn = reinterpret_cast<const void*>(&fwd_kernel<N, VPT, VARIANT>);
  int64_t res = 0;
  hipError_t e = resident_blocks(fn, s.threads, s.lds, &res);  // validates the launch shape
  if (e != hipSuccess) return e;
  const int64_t per_launch = (int64_t)(UINT32_MAX / (uint32_t)s.threads);
  for (int64_t t0 = 0; t0 < a.T; t0 += per_launch) {
    const int64_t n = a.T - t0 < per_launch ? a.T - t0 : per_launch;
    hipLaunchKernelGGL((fwd_kernel<N, VPT, VARIANT>), dim3((unsigned)n), dim3((unsigned)s.threads), s.lds, st, a.src,
                       a.delta, a.partial_out, a.zg, a.rg, a.w, a.eps, t0, a.D, a.out, a.rstd, a.alpha);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int N, int VARIANT>
hipError_t run_fwd_n(const LaunchShape& s, hipStream_t st, const FwdArgs& a) {
  return s.vpt == 4 ? run_fwd_vpt<N, 4, VARIANT>(s, st, a) : run_fwd_vpt<N, 2, VARIANT>(s, st, a);
}

template <int N>
hipError_t run_fwd_variant(int variant, const LaunchShape& s, hipStream_t st, const FwdArgs& a) {
  if (variant == kFwdUpdate) return run_fwd_n<N, kFwdUpdate>(s, st, a);
  if constexpr (N >= 2) {
    if (variant == kFwdScored) return run_fwd_n<N, kFwdScored>(s, st, a);
  }
  if (variant == kFwdPlain) return run_fwd_n<N, kFwdPlain>(s, st, a);
  return hipErrorInvalidValue;
}

template <int N, int VPT, bool PIPE, int MODE>
hipError_t launch_bwd_n(const LaunchShape& s, hipStream_t st, const BwdArgs& a) {
  const void* fn = reinterpret_cast<const void*>(&bwd_kernel<N, VPT, PIPE, MODE>);
  int64_t res = 0;
  // w and the running dw (thread-private slots), plus, for written fp32
  // gradients with one vector per thread, a 2 KiB output stage per wave
  const size_t lds = 2 * s.lds + ((MODE == kGradF32 && VPT == 1) ? (size_t)s.threads * 32 : 0);
  hipError_t e = resident_blocks(fn, s.threads, lds, &res);  // validates the launch shape
  if (e != hipSuccess) return e;
  // one workgroup per dw partial row (P = min(T, ATTNRES_DW_PARTIALS))
  hipLaunchKernelGGL((bwd_kernel<N, VPT, PIPE, MODE>), dim3((unsigned)a.P), dim3((unsigned)s.threads),
                     lds, st, a.dout, a.src, a.w, a.rstd, a.alpha, a.T, a.D, a.P, a.dsrc, a.ws);
  return hipGetLastError();
}

template <int N, int VPT>
hipError_t run_bwd_vpt(const LaunchShape& s, int mode, hipStream_t st, const BwdArgs& a) {
  // with one vector per thread the overwriting modes prefetch the next token;
  // the accumulating ones keep the old gradients instead of a second row group
  constexpr bool P = VPT == 1;
  switch (mode) {
    case 0: return launch_bwd_n<N, VPT, P, 0>(s, st, a);
    case kGradAccumulate: return launch_bwd_n<N, VPT, false, kGradAccumulate>(s, st, a);
    case kGradF32: return launch_bwd_n<N, VPT, P, kGradF32>(s, st, a);
    case kGradF32 | kGradAccumulate: return launch_bwd_n<N, VPT, false, kGradF32 | kGradAccumulate>(s, st, a);
    default: return hipErrorInvalidValue;
  }
}

template <int N>
hipError_t run_bwd_n(const LaunchShape& s, int mode, hipStream_t st, const BwdArgs& a) {
  return s.vpt == 1 ? run_bwd_vpt<N, 1>(s, mode, st, a) : run_bwd_vpt<N, 2>(s, mode, st, a);
}

hipError_t run_fwd(int32_t N, const LaunchShape& s, int variant, hipStream_t st, const FwdArgs& a) {
  switch (N) {
    case 1: return run_fwd_variant<1>(variant, s, st, a);
    case 2: return run_fwd_variant<2>(variant, s, st, a);
    case 3: return run_fwd_variant<3>(variant, s, st, a);
    case 4: return run_fwd_variant<4>(variant, s, st, a);
    case 5: return run_fwd_variant<5>(variant, s, st, a);
    case 6: return run_fwd_variant<6>(variant, s, st, a);
    case 7: return run_fwd_variant<7>(variant, s, st, a);
    case 8: return run_fwd_variant<8>(variant, s, st, a);
    case 9: return run_fwd_variant<9>(variant, s, st, a);
    default: return hipErrorInvalidValue;
  }
}

template <int N, int MODE>
hipError_t launch_split_n(hipStream_t st, SplitArgs a, int64_t groups) {
  const void* fn = reinterpret_cast<const void*>(&bwd_split_kernel<N, MODE>);
  int64_t res = 0;
  hipError_t e = resident_blocks(fn, kSpThreads, 0, &res);  // validates the launch shape
  if (e != hipSuccess) return e;
  // the dispatch packet counts work-items in 32 bits
  const int64_t per_launch = (int64_t)(UINT32_MAX / kSpThreads) / a.K;
  const int64_t first = a.s0;
  for (int64_t g0 = 0; g0 < groups; g0 += per_launch) {
    const int64_t n = groups - g0 < per_launch ? groups - g0 : per_launch;
    a.s0 = first + g0;
    hipLaunchKernelGGL((bwd_split_kernel<N, MODE>), dim3((unsigned)(n * a.K)), dim3(kSpThreads), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int N>
hipError_t run_split_n(int mode, hipStream_t st, const SplitArgs& a, int64_t groups) {
  switch (mode) {
    case 0: return launch_split_n<N, 0>(st, a, groups);
    case kGradAccumulate: return launch_split_n<N, kGradAccumulate>(st, a, groups);
    case kGradF32: return launch_split_n<N, kGradF32>(st, a, groups);
    case kGradF32 | kGradAccumulate: return launch_split_n<N, kGradF32 | kGradAccumulate>(st, a, groups);
    default: return hipErrorInvalidValue;
  }
}

hipError_t run_split(int32_t N, int mode, hipStream_t st, const SplitArgs& a, int64_t groups) {
  switch (N) {
    case 1: return run_split_n<1>(mode, st, a, groups);
    case 2: return run_split_n<2>(mode, st, a, groups);
    case 3: return run_split_n<3>(mode, st, a, groups);
    case 4: return run_split_n<4>(mode, st, a, groups);
    case 5: return run_split_n<5>(mode, st, a, groups);
    case 6: return run_split_n<6>(mode, st, a, groups);
    case 7: return run_split_n<7>(mode, st, a, groups);
    case 8: return run_split_n<8>(mode, st, a, groups);
    case 9: return run_split_n<9>(mode, st, a, groups);
    default: return hipErrorInvalidValue;
  }
}

hipError_t run_bwd(int32_t N, const LaunchShape& s, int mode, hipStream_t st, const BwdArgs& a) {
  switch (N) {
    case 1: return run_bwd_n<1>(s, mode, st, a);
    case 2: return run_bwd_n<2>(s, mode, st, a);
    case 3: return run_bwd_n<3>(s, mode, st, a);
    case 4: return run_bwd_n<4>(s, mode, st, a);
    case 5: return run_bwd_n<5>(s, mode, st, a);
    case 6: return run_bwd_n<6>(s, mode, st, a);
    case 7: return run_bwd_n<7>(s, mode, st, a);
    case 8: return run_bwd_n<8>(s, mode, st, a);
    case 9: return run_bwd_n<9>(s, mode, st, a);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
// Host-side validation and launch, shared by the stacked and per-source calls
// ---------------------------------------------------------------------------
// srcs: N source rows (with an update, srcs[N-1] is the partial sum before
// it).  allow_no_state: rstd and alpha may both be NULL (decoding calls).
// delta / partial_out: the update's addend and result, or both NULL.
// zg / rg: the scored forward's given scores and rstd of the first N-1
// sources ([T][N-1] fp32), or both NULL.
attnres_status fwd_impl(const uint16_t* const* srcs, int64_t pitch, const float* w, float eps, int32_t N, int64_t T,
                        int32_t D, uint16_t* out, float* rstd, float* alpha, bool allow_no_state,
                        const uint16_t* delta, uint16_t* partial_out, void* stream, const float* zg = nullptr,
                        const float* rg = nullptr) {
  const size_t nTD = (size_t)T * (size_t)D, nTN = (size_t)T * (size_t)N;
  const bool update = delta != nullptr || partial_out != nullptr;
  const bool scored = zg != nullptr || rg != nullptr;
  if (update && (delta == nullptr || partial_out == nullptr)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (scored && (zg == nullptr || rg == nullptr || update || N < 2)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (!aligned(zg, 4) || !aligned(rg, 4)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (!pitch_ok(pitch, T, D)) return ATTNRES_ERR_INVALID_ARGUMENT;
  Range ins[ATTNRES_MAX_SOURCES + 4];
  SrcRows rows{};
  rows.pitch = pitch;
  for (int i = 0; i < N; ++i) {
    if (srcs[i] == nullptr || !aligned(srcs[i], 16)) return ATTNRES_ERR_INVALID_ARGUMENT;
    rows.p[i] = srcs[i];
    ins[i] = rows_of(srcs[i], T, (int64_t)D * 2, pitch * 2);
  }
  ins[N] = range_of(w, (size_t)D * 4);
  ins[N + 1] = range_of(delta, update ? nTD * 2 : 0);
  const size_t nTG = scored ? (size_t)T * (size_t)(N - 1) * 4 : 0;
  ins[N + 2] = range_of(zg, nTG);
  ins[N + 3] = range_of(rg, nTG);
  if (!aligned(delta, 16) || !aligned(partial_out, 16)) return ATTNRES_ERR_INVALID_ARGUMENT;
  // rstd and alpha are written together or (decoding calls only) not at all
  const bool save = rstd != nullptr || alpha != nullptr;
  if (out == nullptr || (save && (rstd == nullptr || alpha == nullptr))) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (!save && !allow_no_state) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (!aligned(out, 16) || !aligned(rstd, 4) || !aligned(alpha, 4)) return ATTNRES_ERR_INVALID_ARGUMENT;
  const Range outs[4] = {range_of(out, nTD * 2), range_of(rstd, save ? nTN * 4 : 0),
                         range_of(alpha, save ? nTN * 4 : 0),
                         rows_of(partial_out, update ? T : 0, (int64_t)D * 2, pitch * 2)};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b <= N + 3; ++b) {
      // the partial sum may be updated in place: exactly its own buffer
      const bool in_place = a == 3 && b == N - 1 && partial_out == srcs[N - 1];
      if (!in_place && overlap(outs[a], ins[b])) return ATTNRES_ERR_INVALID_ARGUMENT;
    }
    for (int b = a + 1; b < 4; ++b)
      if (overlap(outs[a], outs[b])) return ATTNRES_ERR_INVALID_ARGUMENT;
  }
  const LaunchShape s = fwd_shape(D);
  const FwdArgs args{rows, delta, partial_out, zg, rg, w, eps, T, D, out, rstd, alpha};
  const int variant = update ? kFwdUpdate : scored ? kFwdScored : kFwdPlain;
  const hipError_t e = run_fwd(N, s, variant, reinterpret_cast<hipStream_t>(stream), args);
  return e == hipSuccess ? ATTNRES_OK : ATTNRES_ERR_HIP;
}

// Block-batched scores: validate, split the queries into the workspace, run
// the MFMA kernel.
attnres_status block_scores_impl(const uint16_t* const* srcs, int64_t pitch, const float* W, int32_t L, float eps,
                                 int32_t n, int64_t T, int32_t D, float* rstd, float* z, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!sizes_ok(n, T, D)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (L < 1 || L > ATTNRES_MAX_QUERIES) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (!(eps >= 0.0f) || !__builtin_isfinite(eps)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (W == nullptr || !aligned(W, 16)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (T == 0) return ATTNRES_OK;
  if (srcs == nullptr || rstd == nullptr || z == nullptr) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (!aligned(rstd, 4) || !aligned(z, 4)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (!pitch_ok(pitch, T, D)) return ATTNRES_ERR_INVALID_ARGUMENT;
  // the wave descriptors span 64 rows: keep them inside 32-bit byte offsets
  if (pitch > (INT64_C(1) << 24)) return ATTNRES_ERR_INVALID_ARGUMENT;
  const size_t need = ATTNRES_BLOCK_SCORES_WORKSPACE_BYTES(L, D);
  if (workspace == nullptr || workspace_bytes < need) return ATTNRES_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return ATTNRES_ERR_INVALID_ARGUMENT;
  const int64_t wg_per_source = (T + kBsRows - 1) / kBsRows;
  const int64_t bs_groups = (wg_per_source + 7) / 8 * 8;  // token groups in whole rounds of the 8 XCDs
  if (bs_groups * n > (int64_t)UINT32_MAX / 256) return ATTNRES_ERR_INVALID_ARGUMENT;
  Range ins[ATTNRES_MAX_SOURCES + 1];
  SrcRows rows{};
  rows.pitch = pitch;
  for (int i = 0; i < n; ++i) {
    if (srcs[i] == nullptr || !aligned(srcs[i], 16)) return ATTNRES_ERR_INVALID_ARGUMENT;
    rows.p[i] = srcs[i];
    ins[i] = rows_of(srcs[i], T, (int64_t)D * 2, pitch * 2);
  }
  ins[n] = range_of(W, (size_t)L * (size_t)D * 4);
  const Range outs[3] = {range_of(rstd, (size_t)T * (size_t)n * 4), range_of(z, (size_t)L * (size_t)T * (size_t)n * 4),
                         range_of(workspace, need)};
  for (int a = 0; a < 3; ++a) {
    for (int b = 0; b <= n; ++b)
      if (overlap(outs[a], ins[b])) return ATTNRES_ERR_INVALID_ARGUMENT;
    for (int b = a + 1; b < 3; ++b)
      if (overlap(outs[a], outs[b])) return ATTNRES_ERR_INVALID_ARGUMENT;
  }
  const int32_t Lpad = (L + 15) / 16 * 16, Dpad = (D + 31) / 32 * 32;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint16_t* Wp = reinterpret_cast<uint16_t*>(workspace);
  const int64_t total = (int64_t)Lpad * Dpad;
  hipLaunchKernelGGL(split_queries_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, W, L, D, Lpad, Dpad,
                     Wp);
  if (hipGetLastError() != hipSuccess) return ATTNRES_ERR_HIP;
  const dim3 grid((unsigned)(bs_groups * n)), block(kBsWaves * kWave);
  if (Lpad <= 16)
    hipLaunchKernelGGL(block_scores_kernel<1>, grid, block, 0, st, rows, T, D, eps, n, Wp, L, Lpad, Dpad,
                       wg_per_source, rstd, z);
  else if (Lpad <= 32)
    hipLaunchKernelGGL(block_scores_kernel<2>, grid, block, 0, st, rows, T, D, eps, n, Wp, L, Lpad, Dpad,
                       wg_per_source, rstd, z);
  else
    hipLaunchKernelGGL(block_scores_kernel_wide, grid, block, 0, st, rows, T, D, eps, n, Wp, L, Lpad, Dpad,
                       wg_per_source, rstd, z);
  return hipGetLastError() == hipSuccess ? ATTNRES_OK : ATTNRES_ERR_HIP;
}

// One workgroup per token for the block sums and the merged forward; the
// dispatch packet counts work-items in 32 bits, so very large T is split over
// several launches.
int threads_for(int32_t D, int vpt) { return ((D / 8 + vpt - 1) / vpt + kWave - 1) / kWave * kWave; }

template <int NS, int VPT, bool F24>
hipError_t run_sums_vpt(hipStream_t st, const SrcRows& rows, const float* z, int32_t L, int64_t T, int32_t D, void* U,
                        int64_t ls, int64_t tp) {
  const int threads = threads_for(D, VPT);
  int64_t res = 0;
  hipError_t e = resident_blocks(reinterpret_cast<const void*>(&block_sums_kernel<NS, VPT, F24>), threads, 0, &res);
  if (e != hipSuccess) return e;  // validates the launch shape
  const int64_t per_launch = (int64_t)(UINT32_MAX / (uint32_t)threads);
  for (int64_t t0 = 0; t0 < T; t0 += per_launch) {
    const int64_t n = T - t0 < per_launch ? T - t0 : per_launch;
    hipLaunchKernelGGL((block_sums_kernel<NS, VPT, F24>), dim3((unsigned)n), dim3((unsigned)threads), 0, st, rows, z,
                       L, T, D, t0, U, ls, tp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int NS>
hipError_t run_sums_n(int vpt, bool f24, hipStream_t st, const SrcRows& rows, const float* z, int32_t L, int64_t T,
                      int32_t D, void* U, int64_t ls, int64_t tp) {
  if (f24)
    return vpt == 1 ? run_sums_vpt<NS, 1, true>(st, rows, z, L, T, D, U, ls, tp)
                    : run_sums_vpt<NS, 2, true>(st, rows, z, L, T, D, U, ls, tp);
  return vpt == 1 ? run_sums_vpt<NS, 1, false>(st, rows, z, L, T, D, U, ls, tp)
                  : run_sums_vpt<NS, 2, false>(st, rows, z, L, T, D, U, ls, tp);
}

// The sums' vectors per thread: one while a token's vectors fit 1024 threads.
int sums_vpt(int32_t D) { return D / 8 <= 1024 ? 1 : 2; }

attnres_status block_sums_impl(const uint16_t* const* srcs, int64_t pitch, const float* z, int32_t L, int32_t n,
                               int64_t T, int32_t D, void* U, int64_t ls, int64_t tp, int32_t u_format, void* stream) {
  if (!sizes_ok(n, T, D)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (L < 1 || L > ATTNRES_MAX_QUERIES) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (T == 0) return ATTNRES_OK;
  if (srcs == nullptr || z == nullptr || U == nullptr) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (u_format != ATTNRES_U_F32 && u_format != ATTNRES_U_F24) return ATTNRES_ERR_INVALID_ARGUMENT;
  const bool f24 = u_format == ATTNRES_U_F24;
  if (!aligned(z, 4) || !aligned(U, f24 ? 4 : 16)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (!pitch_ok(pitch, T, D)) return ATTNRES_ERR_INVALID_ARGUMENT;
  // U rows start on 16-byte (fp32) or 4-byte (24-bit: 12-byte multiples from
  // a 4-byte aligned base) boundaries and never overlap: sub-layer-major
  // (tp >= D, ls past the last token's row) or token-major (ls >= D, tp past
  // the last sub-layer's row); every offset stays far inside int64.
  if (ls < D || tp < D || ls % 4 != 0 || tp % 4 != 0) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (ls > (INT64_C(1) << 40) || tp > (INT64_C(1) << 40) / T) return ATTNRES_ERR_INVALID_ARGUMENT;
  const bool l_major = ls >= (T - 1) * tp + D, t_major = tp >= (int64_t)(L - 1) * ls + D;
  if (!l_major && !t_major) return ATTNRES_ERR_INVALID_ARGUMENT;
  Range ins[ATTNRES_MAX_SOURCES + 1];
  SrcRows rows{};
  rows.pitch = pitch;
  for (int i = 0; i < n; ++i) {
    if (srcs[i] == nullptr || !aligned(srcs[i], 16)) return ATTNRES_ERR_INVALID_ARGUMENT;
    rows.p[i] = srcs[i];
    ins[i] = rows_of(srcs[i], T, (int64_t)D * 2, pitch * 2);
  }
  ins[n] = range_of(z, (size_t)L * (size_t)T * (size_t)n * 4);
  const Range out = range_of(U, (size_t)((int64_t)(L - 1) * ls + (T - 1) * tp + D) * (f24 ? 3 : 4));
  for (int b = 0; b <= n; ++b)
    if (overlap(out, ins[b])) return ATTNRES_ERR_INVALID_ARGUMENT;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int vpt = sums_vpt(D);
  hipError_t e;
  switch (n) {
    case 1: e = run_sums_n<1>(vpt, f24, st, rows, z, L, T, D, U, ls, tp); break;
    case 2: e = run_sums_n<2>(vpt, f24, st, rows, z, L, T, D, U, ls, tp); break;
    case 3: e = run_sums_n<3>(vpt, f24, st, rows, z, L, T, D, U, ls, tp); break;
    case 4: e = run_sums_n<4>(vpt, f24, st, rows, z, L, T, D, U, ls, tp); break;
    case 5: e = run_sums_n<5>(vpt, f24, st, rows, z, L, T, D, U, ls, tp); break;
    case 6: e = run_sums_n<6>(vpt, f24, st, rows, z, L, T, D, U, ls, tp); break;
    case 7: e = run_sums_n<7>(vpt, f24, st, rows, z, L, T, D, U, ls, tp); break;
    case 8: e = run_sums_n<8>(vpt, f24, st, rows, z, L, T, D, U, ls, tp); break;
    case 9: e = run_sums_n<9>(vpt, f24, st, rows, z, L, T, D, U, ls, tp); break;
    default: return ATTNRES_ERR_INVALID_ARGUMENT;
  }
  return e == hipSuccess ? ATTNRES_OK : ATTNRES_ERR_HIP;
}

struct MergedArgs {
  const void* U;
  int64_t u_pitch;
  int32_t u_format;
  const uint16_t* p;
  int64_t p_pitch;
  const uint16_t* delta;  // with partial_out: the fused partial-sum update, else both NULL
  uint16_t* partial_out;
  const float* zg;
  const float* rg;
  const float* w;
  float eps;
  int64_t T;
  int32_t D;
  uint16_t* out;
  float* rstd;
  float* alpha;
};

// kMergedQuads channel quads per thread, whole waves: 256 threads at D = 7168,
// 640 at D = 16384.
template <int N, bool UPDATE, bool F24>
hipError_t run_merged_nu(hipStream_t st, const MergedArgs& a) {
  const int threads = ((a.D / 4 + kMergedQuads - 1) / kMergedQuads + kWave - 1) / kWave * kWave;
  int64_t res = 0;
  hipError_t e =
      resident_blocks(reinterpret_cast<const void*>(&fwd_merged_kernel<N, UPDATE, F24>), threads, 0, &res);
  if (e != hipSuccess) return e;  // validates the launch shape
  const int64_t per_launch = (int64_t)(UINT32_MAX / (uint32_t)threads);
  for (int64_t t0 = 0; t0 < a.T; t0 += per_launch) {
    const int64_t n = a.T - t0 < per_launch ? a.T - t0 : per_launch;
    hipLaunchKernelGGL((fwd_merged_kernel<N, UPDATE, F24>), dim3((unsigned)n), dim3((unsigned)threads), 0, st, a.U,
                       a.u_pitch, a.p, a.p_pitch, a.delta, a.partial_out, a.zg, a.rg, a.w, a.eps, t0, a.D, a.out,
                       a.rstd, a.alpha);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int N>
hipError_t run_merged_n(hipStream_t st, const MergedArgs& a) {
  if (a.u_format == ATTNRES_U_F24)
    return a.delta != nullptr ? run_merged_nu<N, true, true>(st, a) : run_merged_nu<N, false, true>(st, a);
  return a.delta != nullptr ? run_merged_nu<N, true, false>(st, a) : run_merged_nu<N, false, false>(st, a);
}

attnres_status fwd_merged_impl(const MergedArgs& a, int32_t N, void* stream) {
  const size_t nTD = (size_t)a.T * (size_t)a.D, nTN = (size_t)a.T * (size_t)N, nTG = (size_t)a.T * (size_t)(N - 1);
  if (a.U == nullptr || a.p == nullptr || a.zg == nullptr || a.rg == nullptr) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (a.out == nullptr || a.rstd == nullptr || a.alpha == nullptr) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (a.u_format != ATTNRES_U_F32 && a.u_format != ATTNRES_U_F24) return ATTNRES_ERR_INVALID_ARGUMENT;
  const int64_t eb = a.u_format == ATTNRES_U_F24 ? 3 : 4;  // bytes per element of U
  if (!aligned(a.U, eb == 4 ? 16 : 4) || !aligned(a.p, 16) || !aligned(a.out, 16)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (!aligned(a.zg, 4) || !aligned(a.rg, 4) || !aligned(a.rstd, 4) || !aligned(a.alpha, 4))
    return ATTNRES_ERR_INVALID_ARGUMENT;
  if (!pitch_ok(a.p_pitch, a.T, a.D)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (a.u_pitch < a.D || a.u_pitch % 4 != 0 || a.u_pitch > (INT64_C(1) << 40) / a.T) return ATTNRES_ERR_INVALID_ARGUMENT;
  const bool update = a.delta != nullptr || a.partial_out != nullptr;
  if (update && (a.delta == nullptr || a.partial_out == nullptr)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (!aligned(a.delta, 16) || !aligned(a.partial_out, 16)) return ATTNRES_ERR_INVALID_ARGUMENT;
  const Range ins[6] = {rows_of(a.U, a.T, (int64_t)a.D * eb, a.u_pitch * eb), rows_of(a.p, a.T, (int64_t)a.D * 2, a.p_pitch * 2),
                        range_of(a.zg, nTG * 4), range_of(a.rg, nTG * 4), range_of(a.w, (size_t)a.D * 4),
                        range_of(a.delta, update ? nTD * 2 : 0)};
  const Range outs[4] = {range_of(a.out, nTD * 2), range_of(a.rstd, nTN * 4), range_of(a.alpha, nTN * 4),
                         rows_of(a.partial_out, update ? a.T : 0, (int64_t)a.D * 2, a.p_pitch * 2)};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j) {
      // the partial sum may be updated in place: exactly its own rows
      const bool in_place = i == 3 && j == 1 && a.partial_out == a.p;
      if (!in_place && overlap(outs[i], ins[j])) return ATTNRES_ERR_INVALID_ARGUMENT;
    }
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return ATTNRES_ERR_INVALID_ARGUMENT;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  switch (N) {
    case 2: e = run_merged_n<2>(st, a); break;
    case 3: e = run_merged_n<3>(st, a); break;
    case 4: e = run_merged_n<4>(st, a); break;
    case 5: e = run_merged_n<5>(st, a); break;
    case 6: e = run_merged_n<6>(st, a); break;
    case 7: e = run_merged_n<7>(st, a); break;
    case 8: e = run_merged_n<8>(st, a); break;
    case 9: e = run_merged_n<9>(st, a); break;
    default: return ATTNRES_ERR_INVALID_ARGUMENT;
  }
  return e == hipSuccess ? ATTNRES_OK : ATTNRES_ERR_HIP;
}

attnres_status fwd_common_checks(const float* w, float eps, int32_t N, int64_t T, int32_t D) {
  if (!sizes_ok(N, T, D)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (!(eps >= 0.0f) || !__builtin_isfinite(eps)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (w == nullptr || !aligned(w, 16)) return ATTNRES_ERR_INVALID_ARGUMENT;
  return ATTNRES_OK;
}

attnres_status bwd_zero_dw(float* dw, int32_t D, void* stream) {
  const int n4 = D / 4;
  hipLaunchKernelGGL(zero_kernel, dim3((n4 + 255) / 256), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<float4*>(dw), n4);
  return hipGetLastError() == hipSuccess ? ATTNRES_OK : ATTNRES_ERR_HIP;
}

attnres_status bwd_common_checks(const float* w, int32_t N, int64_t T, int32_t D, float* dw) {
  if (!sizes_ok(N, T, D)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (w == nullptr || dw == nullptr || !aligned(w, 16) || !aligned(dw, 16)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (overlap(range_of(dw, (size_t)D * 4), range_of(w, (size_t)D * 4))) return ATTNRES_ERR_INVALID_ARGUMENT;
  return ATTNRES_OK;
}

// split: the split-token backward (where ATTNRES_BWD_SPLIT(N, D)) with the
// workspace layout [fold rows][ring][partial rows]; otherwise the
// one-token-per-workgroup backward with its ATTNRES_DW_PARTIALS rows.
attnres_status bwd_impl(const uint16_t* dout, const uint16_t* const* srcs, int64_t src_pitch, const float* w,
                        const float* rstd, const float* alpha, int32_t N, int64_t T, int32_t D,
                        void* const* dsrcs, int64_t dsrc_pitch, int mode, float* dw, void* workspace,
                        size_t workspace_bytes, void* stream, bool split = true) {
  split = split && ATTNRES_BWD_SPLIT(N, D);
  const int64_t gsize = (mode & kGradF32) ? 4 : 2;  // bytes per gradient element
  if (dout == nullptr || rstd == nullptr || alpha == nullptr) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (!aligned(dout, 16) || !aligned(rstd, 4) || !aligned(alpha, 4)) return ATTNRES_ERR_INVALID_ARGUMENT;
  const size_t nTD = (size_t)T * (size_t)D, nTN = (size_t)T * (size_t)N;
  Range ins[ATTNRES_MAX_SOURCES + 4];
  int nin = 0;
  if (!pitch_ok(src_pitch, T, D) || !pitch_ok(dsrc_pitch, T, D)) return ATTNRES_ERR_INVALID_ARGUMENT;
  SrcRows rows{};
  DstRows drows{};
  rows.pitch = src_pitch;
  drows.pitch = dsrc_pitch;
  for (int i = 0; i < N; ++i) {
    if (srcs[i] == nullptr || !aligned(srcs[i], 16)) return ATTNRES_ERR_INVALID_ARGUMENT;
    if (dsrcs[i] == nullptr || !aligned(dsrcs[i], 16)) return ATTNRES_ERR_INVALID_ARGUMENT;
    rows.p[i] = srcs[i];
    drows.p[i] = dsrcs[i];
    ins[nin++] = rows_of(srcs[i], T, (int64_t)D * 2, src_pitch * 2);
  }
  ins[nin++] = range_of(dout, nTD * 2);
  ins[nin++] = range_of(w, (size_t)D * 4);
  ins[nin++] = range_of(rstd, nTN * 4);
  ins[nin++] = range_of(alpha, nTN * 4);
  const size_t need = split ? ATTNRES_BWD_WORKSPACE_BYTES(T, N, D) : (size_t)ATTNRES_DW_PARTIALS * (size_t)D * 4;
  if (workspace == nullptr || workspace_bytes < need) return ATTNRES_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return ATTNRES_ERR_INVALID_ARGUMENT;
  Range outs[ATTNRES_MAX_SOURCES + 2];
  int nout = 0;
  for (int i = 0; i < N; ++i) outs[nout++] = rows_of(dsrcs[i], T, (int64_t)D * gsize, dsrc_pitch * gsize);
  outs[nout++] = range_of(dw, (size_t)D * 4);
  outs[nout++] = range_of(workspace, need);
  for (int a = 0; a < nout; ++a) {
    for (int b = 0; b < nin; ++b)
      if (overlap(outs[a], ins[b])) return ATTNRES_ERR_INVALID_ARGUMENT;
    for (int b = a + 1; b < nout; ++b)
      if (overlap(outs[a], outs[b])) return ATTNRES_ERR_INVALID_ARGUMENT;
  }
  float* ws = reinterpret_cast<float*>(workspace);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int D4 = D / 4;
  int32_t P = 0;            // rows dw_reduce_kernel sums
  const float* reduce_rows = ws;  // where they are
  if (split) {
    const int K = (D / 8 + kSpSliceVectors - 1) / kSpSliceVectors;
    const int64_t groups = (T + kSpSide - 1) / kSpSide;  // token spans
    uint64_t* ring = reinterpret_cast<uint64_t*>(ws + (size_t)ATTNRES_DW_PARTIALS * D);
    const size_t ring_words = (size_t)kSpRing * K * 2 * N;
    float* partial = reinterpret_cast<float*>(ring + ring_words);
    // tags are token + 1: a zeroed ring holds no valid word.  Token t uses
    // slot t mod kSpRing, so a batch of fewer tokens clears only its slots.
    // With one slice per row (K = 1) the ring is not used.
    const int64_t slots = T < kSpRing ? T : kSpRing;
    const int ring4 = (int)((size_t)slots * K * 2 * N / 2);
    if (K > 1) {
      hipLaunchKernelGGL(zero_kernel, dim3((ring4 + 255) / 256), dim3(256), 0, st, reinterpret_cast<float4*>(ring),
                         ring4);
      if (hipGetLastError() != hipSuccess) return ATTNRES_ERR_HIP;
    }
    // chunks of spans, each folded into the P rows dw_reduce_kernel sums
    P = (int32_t)(groups < ATTNRES_DW_PARTIALS ? groups : ATTNRES_DW_PARTIALS);
    const uint32_t spin = g_split_spin.load(std::memory_order_relaxed);
    for (int64_t c0 = 0; c0 < groups; c0 += kSpChunk) {
      const int64_t n = groups - c0 < kSpChunk ? groups - c0 : kSpChunk;
      const SplitArgs sa{dout, rows, w, rstd, alpha, T, D, K, drows, ring, partial, c0, c0, spin};
      if (run_split(N, mode, st, sa, n) != hipSuccess) return ATTNRES_ERR_HIP;
      if (groups <= ATTNRES_DW_PARTIALS) {
        // one span per fold row: the fold would add each partial row to +0,
        // which returns it unchanged (a partial row holds no -0: its sums
        // start from +0), so the final sum reads the partial rows directly
        reduce_rows = partial;
        break;
      }
      hipLaunchKernelGGL(dw_fold_kernel, dim3((unsigned)P, (unsigned)((D4 + kFoldCols - 1) / kFoldCols)),
                         dim3(kFoldCols), 0, st, reinterpret_cast<const float4*>(partial), c0, n, P, D4,
                         c0 == 0 ? 1 : 0, reinterpret_cast<float4*>(ws));
      if (hipGetLastError() != hipSuccess) return ATTNRES_ERR_HIP;
    }
  } else {
    const LaunchShape s = bwd_shape(D);
    P = (int32_t)(T < ATTNRES_DW_PARTIALS ? T : ATTNRES_DW_PARTIALS);
    const BwdArgs args{dout, rows, w, rstd, alpha, T, D, P, drows, ws};
    if (run_bwd(N, s, mode, st, args) != hipSuccess) return ATTNRES_ERR_HIP;
  }
  hipLaunchKernelGGL(dw_reduce_kernel, dim3((D4 + kReduceCols - 1) / kReduceCols), dim3(kReduceThreads), 0, st,
                     reinterpret_cast<const float4*>(reduce_rows), P, D4, reinterpret_cast<float4*>(dw));
  return hipGetLastError() == hipSuccess ? ATTNRES_OK : ATTNRES_ERR_HIP;
}

}  // namespace

// ---------------------------------------------------------------------------
// Entry point without allocation: dw partial rows in a static device array
// ---------------------------------------------------------------------------
// The backward's only scratch is its dw partial rows (ATTNRES_DW_PARTIALS rows
// of D fp32).  attnres_bwd_noalloc keeps them in this file-scope array instead
// of a caller workspace: 256 x 8192 x 4 B = 8 MiB per device, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory, so the kernels receive the device address that hipGetSymbolAddress
// returns for the current device (each device has its own copy at its own
// address), looked up once per device and cached.
static __device__ __align__(256) float scratch[ATTNRES_DW_PARTIALS * ATTNRES_NOALLOC_MAX_D];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (nullptr if the runtime refuses).
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" attnres_status attnres_fwd(const uint16_t* src, const float* w, float eps, int32_t N, int64_t T,
                                      int32_t D, uint16_t* out, float* rstd, float* alpha, void* stream) {
  const attnres_status st = fwd_common_checks(w, eps, N, T, D);
  if (st != ATTNRES_OK) return st;
  if (T == 0) return ATTNRES_OK;
  if (src == nullptr) return ATTNRES_ERR_INVALID_ARGUMENT;
  const uint16_t* srcs[ATTNRES_MAX_SOURCES];
  for (int i = 0; i < N; ++i) srcs[i] = src + (size_t)i * (size_t)T * (size_t)D;
  return fwd_impl(srcs, D, w, eps, N, T, D, out, rstd, alpha, false, nullptr, nullptr, stream);
}

extern "C" attnres_status attnres_fwd_sources(const uint16_t* const* srcs, int64_t src_pitch, const float* w,
                                              float eps, int32_t N, int64_t T, int32_t D, uint16_t* out,
                                              float* rstd, float* alpha, void* stream) {
  const attnres_status st = fwd_common_checks(w, eps, N, T, D);
  if (st != ATTNRES_OK) return st;
  if (T == 0) return ATTNRES_OK;
  if (srcs == nullptr) return ATTNRES_ERR_INVALID_ARGUMENT;
  return fwd_impl(srcs, src_pitch, w, eps, N, T, D, out, rstd, alpha, false, nullptr, nullptr, stream);
}

extern "C" attnres_status attnres_fwd_decode(const uint16_t* const* srcs, int64_t src_pitch, const float* w,
                                             float eps, int32_t N, int64_t T, int32_t D, uint16_t* out, float* rstd,
                                             float* alpha, void* stream) {
  const attnres_status st = fwd_common_checks(w, eps, N, T, D);
  if (st != ATTNRES_OK) return st;
  if (T == 0) return ATTNRES_OK;
  if (srcs == nullptr) return ATTNRES_ERR_INVALID_ARGUMENT;
  return fwd_impl(srcs, src_pitch, w, eps, N, T, D, out, rstd, alpha, true, nullptr, nullptr, stream);
}

extern "C" attnres_status attnres_fwd_update(const uint16_t* const* srcs, int64_t src_pitch,
                                             const uint16_t* partial, const uint16_t* delta, const float* w,
                                             float eps, int32_t N, int64_t T, int32_t D, uint16_t* partial_out,
                                             uint16_t* out, float* rstd, float* alpha, void* stream) {
  const attnres_status st = fwd_common_checks(w, eps, N, T, D);
  if (st != ATTNRES_OK) return st;
  if (T == 0) return ATTNRES_OK;
  if ((N > 1 && srcs == nullptr) || partial == nullptr || delta == nullptr || partial_out == nullptr)
    return ATTNRES_ERR_INVALID_ARGUMENT;
  const uint16_t* all[ATTNRES_MAX_SOURCES];
  for (int i = 0; i + 1 < N; ++i) all[i] = srcs[i];
  all[N - 1] = partial;
  return fwd_impl(all, src_pitch, w, eps, N, T, D, out, rstd, alpha, true, delta, partial_out, stream);
}

extern "C" attnres_status attnres_block_scores(const uint16_t* const* srcs, int64_t src_pitch, const float* W,
                                               int32_t L, float eps, int32_t n, int64_t T, int32_t D, float* rstd,
                                               float* z, void* workspace, size_t workspace_bytes, void* stream) {
  return block_scores_impl(srcs, src_pitch, W, L, eps, n, T, D, rstd, z, workspace, workspace_bytes, stream);
}

extern "C" attnres_status attnres_fwd_scored(const uint16_t* const* srcs, int64_t src_pitch, const float* z_given,
                                             const float* rstd_given, const float* w, float eps, int32_t N, int64_t T,
                                             int32_t D, uint16_t* out, float* rstd, float* alpha, void* stream) {
  const attnres_status st = fwd_common_checks(w, eps, N, T, D);
  if (st != ATTNRES_OK) return st;
  if (N < 2) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (T == 0) return ATTNRES_OK;
  if (srcs == nullptr || z_given == nullptr || rstd_given == nullptr) return ATTNRES_ERR_INVALID_ARGUMENT;
  return fwd_impl(srcs, src_pitch, w, eps, N, T, D, out, rstd, alpha, false, nullptr, nullptr, stream, z_given,
                  rstd_given);
}

extern "C" attnres_status attnres_block_sums(const uint16_t* const* srcs, int64_t src_pitch, const float* z,
                                             int32_t L, int32_t n, int64_t T, int32_t D, void* U, int64_t u_lstride,
                                             int64_t u_pitch, int32_t u_format, void* stream) {
  return block_sums_impl(srcs, src_pitch, z, L, n, T, D, U, u_lstride, u_pitch, u_format, stream);
}

extern "C" attnres_status attnres_fwd_merged(const void* U, int64_t u_pitch, int32_t u_format,
                                             const uint16_t* partial, int64_t partial_pitch,
                                             const uint16_t* delta, uint16_t* partial_out,
                                             const float* z_given, const float* rstd_given, const float* w, float eps,
                                             int32_t N, int64_t T, int32_t D, uint16_t* out, float* rstd,
                                             float* alpha, void* stream) {
  const attnres_status st = fwd_common_checks(w, eps, N, T, D);
  if (st != ATTNRES_OK) return st;
  if (N < 2) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (T == 0) return ATTNRES_OK;
  const MergedArgs a{U,   u_pitch, u_format, partial, partial_pitch, delta, partial_out, z_given, rstd_given, w,
                     eps, T,       D,        out,     rstd,          alpha};
  return fwd_merged_impl(a, N, stream);
}

extern "C" attnres_status attnres_bwd(const uint16_t* dout, const uint16_t* src, const float* w, const float* rstd,
                                      const float* alpha, int32_t N, int64_t T, int32_t D, uint16_t* dsrc, float* dw,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  const attnres_status st = bwd_common_checks(w, N, T, D, dw);
  if (st != ATTNRES_OK) return st;
  if (T == 0) return bwd_zero_dw(dw, D, stream);
  if (src == nullptr || dsrc == nullptr) return ATTNRES_ERR_INVALID_ARGUMENT;
  const uint16_t* srcs[ATTNRES_MAX_SOURCES];
  uint16_t* dsrcs[ATTNRES_MAX_SOURCES];
  for (int i = 0; i < N; ++i) {
    srcs[i] = src + (size_t)i * (size_t)T * (size_t)D;
    dsrcs[i] = dsrc + (size_t)i * (size_t)T * (size_t)D;
  }
  return bwd_impl(dout, srcs, D, w, rstd, alpha, N, T, D, reinterpret_cast<void* const*>(dsrcs), D, 0, dw, workspace,
                  workspace_bytes, stream);
}

extern "C" attnres_status attnres_bwd_sources(const uint16_t* dout, const uint16_t* const* srcs, int64_t src_pitch,
                                              const float* w, const float* rstd, const float* alpha, int32_t N,
                                              int64_t T, int32_t D, void* const* dsrcs, int64_t dsrc_pitch,
                                              int32_t grad_mode, float* dw, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  const attnres_status st = bwd_common_checks(w, N, T, D, dw);
  if (st != ATTNRES_OK) return st;
  if (grad_mode < 0 || grad_mode > (kGradAccumulate | kGradF32)) return ATTNRES_ERR_INVALID_ARGUMENT;
  if (T == 0) return bwd_zero_dw(dw, D, stream);
  if (srcs == nullptr || dsrcs == nullptr) return ATTNRES_ERR_INVALID_ARGUMENT;
  return bwd_impl(dout, srcs, src_pitch, w, rstd, alpha, N, T, D, dsrcs, dsrc_pitch, grad_mode, dw, workspace,
                  workspace_bytes, stream);
}

extern "C" attnres_status attnres_bwd_noalloc(const uint16_t* dout, const uint16_t* src, const float* w,
                                              const float* rstd, const float* alpha, int32_t N, int64_t T, int32_t D,
                                              uint16_t* dsrc, float* dw, void* stream) {
  const attnres_status st = bwd_common_checks(w, N, T, D, dw);
  if (st != ATTNRES_OK) return st;
  if (D > ATTNRES_NOALLOC_MAX_D) return ATTNRES_ERR_WORKSPACE;  // the static partial rows hold D <= 8192
  if (T == 0) return bwd_zero_dw(dw, D, stream);
  if (src == nullptr || dsrc == nullptr) return ATTNRES_ERR_INVALID_ARGUMENT;
  void* ws = scratch_address();
  if (ws == nullptr) return ATTNRES_ERR_HIP;
  const uint16_t* srcs[ATTNRES_MAX_SOURCES];
  uint16_t* dsrcs[ATTNRES_MAX_SOURCES];
  for (int i = 0; i < N; ++i) {
    srcs[i] = src + (size_t)i * (size_t)T * (size_t)D;
    dsrcs[i] = dsrc + (size_t)i * (size_t)T * (size_t)D;
  }
  return bwd_impl(dout, srcs, D, w, rstd, alpha, N, T, D, reinterpret_cast<void* const*>(dsrcs), D, 0, dw, ws,
                  (size_t)ATTNRES_DW_PARTIALS * (size_t)D * 4, stream, /*split=*/false);
}

// ---------------------------------------------------------------------------
// Poll bound of the split backward's exchange
// ---------------------------------------------------------------------------
extern "C" uint32_t attnres_set_split_spin(uint32_t polls) {
  return g_split_spin.exchange(polls, std::memory_order_relaxed);
}
