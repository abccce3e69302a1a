// libattnres_probes: HBM bandwidth ceilings on gfx950 (MI355X), measured with
// access patterns and no arithmetic.  Not part of the operator; the benchmark
// times these next to it.  Declarations and contracts: attnres_probes.h.
//
// Streaming accesses use raw buffer loads/stores with the nontemporal hint
// (aux bit 1), as the operator's kernels do, so the two are compared under
// the same cache policy.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "attnres_probes.h"

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kChunkThreads = 256;                   // one 4 KiB chunk per workgroup
constexpr uint32_t kChunkBytes = kChunkThreads * 16;
constexpr int kNt = 2;                               // nontemporal
constexpr int kMaxN = 9;
constexpr int kPersistent = 256;                     // backward pattern: workgroups, as the operator's dw rows

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4_t ld(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNt);
}

__device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kNt);
}

// The chunk of workgroup b: bytes [b * 4 KiB, min(bytes, (b + 1) * 4 KiB)).
__device__ __forceinline__ uint32_t chunk_len(uint64_t bytes) {
  const uint64_t base = (uint64_t)blockIdx.x * kChunkBytes;
  const uint64_t left = bytes - base;
  return left < kChunkBytes ? (uint32_t)left : kChunkBytes;
}

__global__ void __launch_bounds__(kChunkThreads) read_kernel(const uint8_t* __restrict__ src, uint64_t bytes,
                                                             uint32_t key, uint32_t* __restrict__ sink) {
  const __amdgpu_buffer_rsrc_t r = rsrc(src + (uint64_t)blockIdx.x * kChunkBytes, chunk_len(bytes));
  const u32x4_t v = ld(r, threadIdx.x * 16u);
  const uint32_t x = v.x ^ v.y ^ v.z ^ v.w;
  if (x == key) sink[0] = x;  // data-dependent, so the load cannot be dropped
}

__global__ void __launch_bounds__(kChunkThreads) write_kernel(uint8_t* __restrict__ dst, uint64_t bytes) {
  const __amdgpu_buffer_rsrc_t r = rsrc(dst + (uint64_t)blockIdx.x * kChunkBytes, chunk_len(bytes));
  st(r, threadIdx.x * 16u, u32x4_t{0u, 0u, 0u, 0u});
}

__global__ void __launch_bounds__(kChunkThreads) copy_kernel(const uint8_t* __restrict__ src,
                                                             uint8_t* __restrict__ dst, uint64_t bytes) {
  const uint32_t len = chunk_len(bytes);
  const uint64_t base = (uint64_t)blockIdx.x * kChunkBytes;
  const u32x4_t v = ld(rsrc(src + base, len), threadIdx.x * 16u);
  st(rsrc(dst + base, len), threadIdx.x * 16u, v);
}

struct Rows {
  const uint16_t* p[kMaxN];
};
struct WRows {
  uint16_t* p[kMaxN];
};

// Forward pattern: one workgroup per token reads the token's row of each of
// the N row sets (four 16-byte vectors per thread, all loads issued before any
// use) and writes its row of out.  Tokens are dealt to workgroups as the
// operator's forward deals them: workgroup b runs on XCD b mod 8, and in
// groups of 128 tokens XCD x takes the 16 consecutive tokens 16x .. 16x + 15
// (the last, partial group keeps token = b; the operator does this for
// 512 < D <= 8192, where this probe's four vectors per thread apply).
__device__ __forceinline__ int64_t xcd_token(int64_t b, int64_t n) {
  constexpr int64_t C = 16, G = 8 * C;
  if (b >= n / G * G) return b;
  const int64_t r = b % G;
  return b - r + (r % 8) * C + r / 8;
}

__global__ void __launch_bounds__(256) fwd_pattern_kernel(Rows src, int32_t N, int32_t D,
                                                          uint16_t* __restrict__ out) {
  const int64_t t = xcd_token(blockIdx.x, gridDim.x);
  const uint32_t bytes = (uint32_t)D * 2u;
  u32x4_t x[kMaxN][4];
#pragma unroll
  for (int i = 0; i < kMaxN; ++i) {
    if (i < N) {  // N is uniform: a scalar branch
      const __amdgpu_buffer_rsrc_t r = rsrc(src.p[i] + t * D, bytes);
#pragma unroll
      for (int k = 0; k < 4; ++k) x[i][k] = ld(r, (threadIdx.x + k * blockDim.x) * 16u);
    }
  }
  const __amdgpu_buffer_rsrc_t ro = rsrc(out + t * D, bytes);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    u32x4_t acc = x[0][k];
#pragma unroll
    for (int i = 1; i < kMaxN; ++i)
      if (i < N) acc |= x[i][k];
    st(ro, (threadIdx.x + k * blockDim.x) * 16u, acc);
  }
}

// Backward pattern: 256 persistent workgroups, one 16-byte vector per thread,
// workgroup c taking tokens c, c + 256, ...; two register sets alternate so
// the next token's loads are in flight while the current one is stored (the
// operator's two-token prefetch).  Loads past the last token use size-0
// descriptors (every lane reads zeros, no memory is touched).
struct Set {
  u32x4_t x[kMaxN];
  u32x4_t g;
};

__device__ __forceinline__ void load_set(Set& s, const Rows& src, const uint16_t* dout, int32_t N, int64_t t,
                                         int64_t T, int32_t D) {
  const bool valid = t < T;
  const int64_t tt = valid ? t : 0;
  const uint32_t bytes = valid ? (uint32_t)D * 2u : 0u;
  const uint32_t off = threadIdx.x * 16u;
  s.g = ld(rsrc(dout + tt * D, bytes), off);
#pragma unroll
  for (int i = 0; i < kMaxN; ++i)
    if (i < N) s.x[i] = ld(rsrc(src.p[i] + tt * D, bytes), off);
}

__device__ __forceinline__ void store_set(const Set& s, const WRows& dst, int32_t N, int64_t t, int32_t D) {
  const uint32_t off = threadIdx.x * 16u;
#pragma unroll
  for (int i = 0; i < kMaxN; ++i)
    if (i < N) st(rsrc(dst.p[i] + t * D, (uint32_t)D * 2u), off, s.x[i] | s.g);
}

__global__ void __launch_bounds__(1024) bwd_pattern_kernel(Rows src, const uint16_t* __restrict__ dout, WRows dst,
                                                           int32_t N, int64_t T, int32_t D, int32_t P) {
  Set a, b;
  int64_t t = blockIdx.x;
  load_set(a, src, dout, N, t, T, D);
  load_set(b, src, dout, N, t + P, T, D);
  while (true) {
    store_set(a, dst, N, t, D);
    load_set(a, src, dout, N, t + 2 * P, T, D);
    t += P;
    if (t >= T) break;
    store_set(b, dst, N, t, D);
    load_set(b, src, dout, N, t + 2 * P, T, D);
    t += P;
    if (t >= T) break;
  }
}


// Split backward pattern: a workgroup of 4 x 128 threads takes one
// 1024-channel slice (128 16-byte vectors) of 4 consecutive tokens side by
// side (workgroup b = span * K + slice, K = ceil(D / 1024)); each thread reads
// its vector of dout and of the N source rows of its token, writes its vector
// of the N gradient rows, and side 0 writes the span's fp32 partial row slice
// (2 x 16 bytes per thread) into `partial`, whose rows are reused every
// kSplitChunk spans as the operator's chunked workspace is.  No exchange and
// no arithmetic beyond an OR.
constexpr int kSplitSide = 4;
constexpr int kSplitSlice = 128;
constexpr int64_t kSplitChunk = 8192;

__global__ void __launch_bounds__(kSplitSide * kSplitSlice) split_bwd_pattern_kernel(Rows src,
                                                                                     const uint16_t* __restrict__ dout,
                                                                                     WRows dst, int32_t N, int64_t T,
                                                                                     int32_t D, int32_t K,
                                                                                     float* __restrict__ partial) {
  const int side = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kSplitSlice);
  const int tl = (int)threadIdx.x % kSplitSlice;
  const int64_t span = blockIdx.x / K;
  const int k = (int)(blockIdx.x % K);
  const int v = k * kSplitSlice + tl;
  const uint32_t off = v < D / 8 ? (uint32_t)v * 16u : 0xFFFFFFF0u;  // past the row: zeros, stores dropped
  const int64_t t = span * kSplitSide + side;
  const bool valid = t < T;
  const int64_t tt = valid ? t : 0;
  const uint32_t bytes = valid ? (uint32_t)D * 2u : 0u;
  const u32x4_t g = ld(rsrc(dout + tt * D, bytes), off);
  u32x4_t x[kMaxN];
#pragma unroll
  for (int i = 0; i < kMaxN; ++i)
    if (i < N) x[i] = ld(rsrc(src.p[i] + tt * D, bytes), off);
#pragma unroll
  for (int i = 0; i < kMaxN; ++i)
    if (i < N) st(rsrc(dst.p[i] + tt * D, bytes), off, x[i] | g);
  if (side == 0) {
    const __amdgpu_buffer_rsrc_t rp = rsrc(partial + (span % kSplitChunk) * D, (uint32_t)D * 4u);
    __builtin_amdgcn_raw_buffer_store_b128(g, rp, 2u * off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(g, rp, 2u * off + 16u, 0, 0);
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launched() { return hipGetLastError() == hipSuccess ? 0 : 3; }

int threads_for(int32_t D, int vpt) {
  const int need = (D / 8 + vpt - 1) / vpt;
  return ((need + kWave - 1) / kWave) * kWave;
}

bool pattern_sizes_ok(int32_t N, int64_t T, int32_t D) {
  return N >= 1 && N <= kMaxN && T >= 0 && D >= 8 && D <= 8192 && D % 8 == 0 &&
         T <= (INT64_C(1) << 40) / ((int64_t)N * D) && T < (INT64_C(1) << 31);
}

}  // namespace

extern "C" int attnres_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (src == nullptr || sink == nullptr || !aligned16(src) || bytes % 16 != 0) return 1;
  if (bytes == 0) return 0;
  const uint64_t chunks = (bytes + kChunkBytes - 1) / kChunkBytes;
  if (chunks > (uint64_t)UINT32_MAX / kChunkThreads) return 1;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)chunks), dim3(kChunkThreads), 0, (hipStream_t)stream,
                     (const uint8_t*)src, (uint64_t)bytes, 0x9E3779B9u, sink);
  return launched();
}

extern "C" int attnres_probe_write(void* dst, size_t bytes, void* stream) {
  if (dst == nullptr || !aligned16(dst) || bytes % 16 != 0) return 1;
  if (bytes == 0) return 0;
  const uint64_t chunks = (bytes + kChunkBytes - 1) / kChunkBytes;
  if (chunks > (uint64_t)UINT32_MAX / kChunkThreads) return 1;
  hipLaunchKernelGGL(write_kernel, dim3((unsigned)chunks), dim3(kChunkThreads), 0, (hipStream_t)stream,
                     (uint8_t*)dst, (uint64_t)bytes);
  return launched();
}

extern "C" int attnres_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (src == nullptr || dst == nullptr || !aligned16(src) || !aligned16(dst) || bytes % 16 != 0) return 1;
  const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
  if (bytes > 0 && s < d + bytes && d < s + bytes) return 1;  // must be disjoint
  if (bytes == 0) return 0;
  const uint64_t chunks = (bytes + kChunkBytes - 1) / kChunkBytes;
  if (chunks > (uint64_t)UINT32_MAX / kChunkThreads) return 1;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)chunks), dim3(kChunkThreads), 0, (hipStream_t)stream,
                     (const uint8_t*)src, (uint8_t*)dst, (uint64_t)bytes);
  return launched();
}

extern "C" int attnres_probe_fwd_pattern(const uint16_t* const* srcs, int32_t N, int64_t T, int32_t D, uint16_t* out,
                                         void* stream) {
  if (!pattern_sizes_ok(N, T, D) || srcs == nullptr) return 1;
  if (T == 0) return 0;
  Rows r{};
  for (int i = 0; i < N; ++i) {
    if (srcs[i] == nullptr || !aligned16(srcs[i])) return 1;
    r.p[i] = srcs[i];
  }
  if (out == nullptr || !aligned16(out)) return 1;
  hipLaunchKernelGGL(fwd_pattern_kernel, dim3((unsigned)T), dim3(threads_for(D, 4)), 0, (hipStream_t)stream, r, N, D,
                     out);
  return launched();
}

extern "C" int attnres_probe_bwd_pattern(const uint16_t* const* srcs, const uint16_t* dout, int32_t N, int64_t T,
                                         int32_t D, uint16_t* const* dsrcs, void* stream) {
  if (!pattern_sizes_ok(N, T, D) || srcs == nullptr || dsrcs == nullptr) return 1;
  if (T == 0) return 0;
  if (dout == nullptr || !aligned16(dout)) return 1;
  Rows r{};
  WRows w{};
  for (int i = 0; i < N; ++i) {
    if (srcs[i] == nullptr || !aligned16(srcs[i]) || dsrcs[i] == nullptr || !aligned16(dsrcs[i])) return 1;
    r.p[i] = srcs[i];
    w.p[i] = dsrcs[i];
  }
  const int P = T < kPersistent ? (int)T : kPersistent;
  hipLaunchKernelGGL(bwd_pattern_kernel, dim3((unsigned)P), dim3(threads_for(D, 1)), 0, (hipStream_t)stream, r, dout,
                     w, N, T, D, P);
  return launched();
}

extern "C" int attnres_probe_split_bwd_pattern(const uint16_t* const* srcs, const uint16_t* dout, int32_t N, int64_t T,
                                               int32_t D, uint16_t* const* dsrcs, float* partial, void* stream) {
  if (!pattern_sizes_ok(N, T, D) || srcs == nullptr || dsrcs == nullptr) return 1;
  if (T == 0) return 0;
  if (dout == nullptr || !aligned16(dout) || partial == nullptr || !aligned16(partial)) return 1;
  Rows r{};
  WRows w{};
  for (int i = 0; i < N; ++i) {
    if (srcs[i] == nullptr || !aligned16(srcs[i]) || dsrcs[i] == nullptr || !aligned16(dsrcs[i])) return 1;
    r.p[i] = srcs[i];
    w.p[i] = dsrcs[i];
  }
  const int K = (D / 8 + kSplitSlice - 1) / kSplitSlice;
  const int64_t spans = (T + kSplitSide - 1) / kSplitSide;
  if (spans * K > (int64_t)UINT32_MAX / (kSplitSide * kSplitSlice)) return 1;
  hipLaunchKernelGGL(split_bwd_pattern_kernel, dim3((unsigned)(spans * K)), dim3(kSplitSide * kSplitSlice), 0,
                     (hipStream_t)stream, r, dout, w, N, T, D, K, partial);
  return launched();
}
