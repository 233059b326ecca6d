// Per-tensor FP8-E4M3 and INT8 quantisation of bf16 tensors.
//
// One scale per tensor from the tensor's own maximum magnitude, chosen so no
// value overflows, with a clip at the format maximum ("Deploying 2:4 Sparsity
// with FP8 on Hopper", pipeline step 3, step 6 and "Troubleshooting quick
// hits").  E4M3: s = fp32(amax / 448) (1 when amax is 0), q = e4m3_rne(clamp(x / s)).
// INT8 (the page's W8A8 recipe, symmetric): s = fp32(amax / 127) (1 when amax
// is 0), q = clamp(rne(x / s), -127, 127).  The kernels are templates on the
// code type; the reduction is shared.
//
// amax is order-independent and exact: it is taken on the integer keys
// (bits & 0x7FFF), which order finite bf16 magnitudes exactly.
//   small tensors (<= kFusedMax values): one launch; every workgroup takes
//                   amax over the whole tensor (at most 256 KB, from L2) and
//                   casts its own slice of kFusedSlice values, so the cast is
//                   spread over the CUs while the reduction needs no second
//                   launch (a launch costs ~2 us).  2K-value slices (twice the
//                   workgroups of 4K ones, each reading X for the maximum)
//                   measured best: up-projection quantise + GEMM at m = 16 11.8
//                   against 12.0 us (1K: 11.9; 16K on 1024 threads: 13.4);
//   larger tensors: kernel 1 writes one partial maximum per workgroup into the
//                   workspace; kernel 2 re-reduces those partials in every
//                   workgroup (a few KB from L2), stores the scale from
//                   workgroup 0 and casts.  No atomics, no memset, no host sync.
#include "sp24_common.hpp"
#include "sp24_fp8.hpp"
#include "sp24_internal.hpp"

namespace sp24 {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxPartials = 1024;
constexpr int kFusedThreads = 512;
constexpr int64_t kFusedMax = 131072;  // values
constexpr int kFusedSlice = 2048;      // values cast per workgroup (4 per thread)

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Block-wide maximum; every thread receives the result.
template <int NT>
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* sh) {
  v = wave_max(v);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) r = max(r, sh[i]);
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void amax_partial_kernel(const uint16_t* __restrict__ x,
                                                                int64_t count,
                                                                uint32_t* __restrict__ partial) {
  __shared__ uint32_t sh[kThreads / kWave];
  const int64_t nvec = count / 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  uint32_t m = 0;
  int64_t i = t0;
  for (; i + 3 * stride < nvec; i += 4 * stride) {  // four loads in flight
    const u32x4 a = xv[i], b = xv[i + stride], c = xv[i + 2 * stride], d = xv[i + 3 * stride];
    m = max(m, max(max(key_max8(a), key_max8(b)), max(key_max8(c), key_max8(d))));
  }
  for (; i < nvec; i += stride) m = max(m, key_max8(*(xv + i)));
  for (int64_t j = nvec * 8 + t0; j < count; j += stride) m = max(m, (uint32_t)(x[j] & 0x7FFFu));
  m = block_max<kThreads>(m, sh);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void cast_kernel(const uint16_t* __restrict__ x, int64_t count,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ scale,
                                                        const uint32_t* __restrict__ partial,
                                                        int npartial) {
  __shared__ uint32_t sh[kThreads / kWave];
  QDiv s;
  if (partial != nullptr) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < npartial; i += kThreads) m = max(m, partial[i]);
    m = block_max<kThreads>(m, sh);
    s = qdiv<DT>(m);
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale = s.s;
  } else {
    s = qdiv_static(*scale);
  }
  const int64_t nvec = count / 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  u32x2* qv = reinterpret_cast<u32x2*>(q);
  int64_t i = t0;
  for (; i + 3 * stride < nvec; i += 4 * stride) {  // four loads in flight
    const u32x4 a = xv[i], b = xv[i + stride], c = xv[i + 2 * stride], d = xv[i + 3 * stride];
    qv[i] = qcast8<DT>(a, s);
    qv[i + stride] = qcast8<DT>(b, s);
    qv[i + 2 * stride] = qcast8<DT>(c, s);
    qv[i + 3 * stride] = qcast8<DT>(d, s);
  }
  for (; i < nvec; i += stride) qv[i] = qcast8<DT>(*(xv + i), s);
  for (int64_t j = nvec * 8 + t0; j < count; j += stride) q[j] = qcast1<DT>(x[j], s);
}

// Small tensors in one launch: workgroup b takes amax over the whole tensor,
// then casts values [b * kFusedSlice, (b + 1) * kFusedSlice).
template <int DT>
__global__ __launch_bounds__(kFusedThreads) void fused_quant_kernel(const uint16_t* __restrict__ x,
                                                                    int64_t count,
                                                                    uint8_t* __restrict__ q,
                                                                    float* __restrict__ scale,
                                                                    int dynamic) {
  __shared__ uint32_t sh[kFusedThreads / kWave];
  const int nvec = (int)(count / 8);
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  QDiv s;
  if (dynamic) {
    uint32_t m = 0;
    int i = threadIdx.x;
    for (; i + 7 * kFusedThreads < nvec; i += 8 * kFusedThreads) {  // eight loads in flight
      u32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = xv[i + j * kFusedThreads];
#pragma unroll
      for (int j = 0; j < 8; ++j) m = max(m, key_max8(v[j]));
    }
    for (; i + 3 * kFusedThreads < nvec; i += 4 * kFusedThreads) {  // four loads in flight
      const u32x4 a = xv[i], b = xv[i + kFusedThreads], c = xv[i + 2 * kFusedThreads],
                  d = xv[i + 3 * kFusedThreads];
      m = max(m, max(max(key_max8(a), key_max8(b)), max(key_max8(c), key_max8(d))));
    }
    for (; i < nvec; i += kFusedThreads) m = max(m, key_max8(xv[i]));
    const int tail = nvec * 8 + threadIdx.x;
    if (tail < count) m = max(m, (uint32_t)(x[tail] & 0x7FFFu));
    m = block_max<kFusedThreads>(m, sh);
    s = qdiv<DT>(m);
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale = s.s;
  } else {
    s = qdiv_static(*scale);
  }
  const int v0 = blockIdx.x * (kFusedSlice / 8);
  const int v1 = min(nvec, v0 + kFusedSlice / 8);
  u32x2* qv = reinterpret_cast<u32x2*>(q);
  for (int i = v0 + threadIdx.x; i < v1; i += kFusedThreads) qv[i] = qcast8<DT>(xv[i], s);
  const int tail = nvec * 8 + threadIdx.x;  // the last workgroup casts the 0..7 trailing values
  if (blockIdx.x == gridDim.x - 1 && tail < count) q[tail] = qcast1<DT>(x[tail], s);
}

// Per-row (per-token) scales: X [m, k] (k % 8 == 0), row r with s_r = fp32(amax_r /
// 448) (1 for a zero row).  Workgroup (c, b) takes the maximum over the whole of rows
// b, b + gridDim.y, ... and casts chunk c (chunk_vecs 8-value vectors) of each: a
// few rows are cast by many workgroups (with the IEEE division per value one CU per
// row took ~2 us for 14336 values), each reading its rows' maximum from
// L2.  A row of up to kRowRegVecs * kThreads vectors cast by one workgroup stays in
// registers from the maximum to the cast (one pass over global memory).
constexpr int kRowRegVecs = 4;
constexpr int kRowMinChunkVecs = 64;  // vectors a workgroup casts at least when a row is split

template <int DT>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(const uint16_t* __restrict__ x, int64_t m,
                                                              int64_t k, uint8_t* __restrict__ q,
                                                              float* __restrict__ scales, int64_t chunk_vecs) {
  __shared__ uint32_t sh[kThreads / kWave];
  const int64_t nvec = k / 8;
  const bool whole = chunk_vecs >= nvec;  // one workgroup per row (gridDim.x == 1)
  const bool in_regs = whole && nvec <= (int64_t)kRowRegVecs * kThreads;
  const int64_t c0 = (int64_t)blockIdx.x * chunk_vecs, c1 = min(nvec, c0 + chunk_vecs);
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y) {
    const u32x4* xv = reinterpret_cast<const u32x4*>(x + r * k);
    u32x2* qv = reinterpret_cast<u32x2*>(q + r * k);
    u32x4 v[kRowRegVecs];
    uint32_t mk = 0;
    if (in_regs) {
#pragma unroll
      for (int j = 0; j < kRowRegVecs; ++j) {
        const int64_t i = threadIdx.x + (int64_t)j * kThreads;
        v[j] = i < nvec ? xv[i] : u32x4{0u, 0u, 0u, 0u};
        mk = max(mk, key_max8(v[j]));
      }
    } else {
      int64_t i = threadIdx.x;
      for (; i + 3 * kThreads < nvec; i += 4 * kThreads) {  // four loads in flight
        const u32x4 a = xv[i], b = xv[i + kThreads], c = xv[i + 2 * kThreads], d = xv[i + 3 * kThreads];
        mk = max(mk, max(max(key_max8(a), key_max8(b)), max(key_max8(c), key_max8(d))));
      }
      for (; i < nvec; i += kThreads) mk = max(mk, key_max8(xv[i]));
    }
    const QDiv s = qdiv<DT>(block_max<kThreads>(mk, sh));
    if (blockIdx.x == 0 && threadIdx.x == 0) scales[r] = s.s;
    if (in_regs) {
#pragma unroll
      for (int j = 0; j < kRowRegVecs; ++j) {
        const int64_t i = threadIdx.x + (int64_t)j * kThreads;
        if (i < nvec) qv[i] = qcast8<DT>(v[j], s);
      }
    } else {
      for (int64_t i = c0 + threadIdx.x; i < c1; i += kThreads) qv[i] = qcast8<DT>(xv[i], s);
    }
  }
}

// Per-group scales: each group of `group` consecutive values of a row of X [m, k]
// (k % group == 0, group % 8 == 0) gets s = fp32(amax_group / 448) (1 for a zero
// group) and its codes as the per-tensor quantiser would give the group alone --
// the per-channel or per-group scales the research-roadmap page ("La Densite
// Dynamique et les Noyaux Non Structures", quantisation under extreme sparsity)
// recommends.  A segment of S lanes (S a power of two up to 64 that divides the
// group's vector count, group / 8) takes one group: each lane V = group / 8 / S
// vectors, the maximum over the segment by shuffles, then the cast.  Up to
// kGroupRegVecs vectors per lane stay in registers between the two.
constexpr int kGroupRegVecs = 4;

template <int DT>
__global__ __launch_bounds__(kThreads) void quant_groups_kernel(const uint16_t* __restrict__ x, int64_t ngroups,
                                                                int64_t group, int seg, uint8_t* __restrict__ q,
                                                                float* __restrict__ scales) {
  const int64_t vpg = group / 8;     // 8-value vectors per group
  const int per = (int)(vpg / seg);  // vectors per lane
  const int lseg = threadIdx.x % seg;
  const int64_t segs = (int64_t)gridDim.x * (kThreads / seg);
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  u32x2* qv = reinterpret_cast<u32x2*>(q);
  for (int64_t g = (int64_t)blockIdx.x * (kThreads / seg) + threadIdx.x / seg; g < ngroups; g += segs) {
    const int64_t base = g * vpg + lseg;  // vector j of this lane: base + j * seg
    u32x4 v[kGroupRegVecs];
    uint32_t mk = 0;
    if (per <= kGroupRegVecs) {
#pragma unroll
      for (int j = 0; j < kGroupRegVecs; ++j)
        if (j < per) {
          v[j] = xv[base + (int64_t)j * seg];
          mk = max(mk, key_max8(v[j]));
        }
    } else {
      for (int j = 0; j < per; ++j) mk = max(mk, key_max8(xv[base + (int64_t)j * seg]));
    }
    for (int off = 1; off < seg; off <<= 1) mk = max(mk, (uint32_t)__shfl_xor((int)mk, off, 64));
    const QDiv s = qdiv<DT>(mk);
    if (lseg == 0) scales[g] = s.s;
    if (per <= kGroupRegVecs) {
#pragma unroll
      for (int j = 0; j < kGroupRegVecs; ++j)
        if (j < per) qv[base + (int64_t)j * seg] = qcast8<DT>(v[j], s);
    } else {
      for (int j = 0; j < per; ++j) qv[base + (int64_t)j * seg] = qcast8<DT>(xv[base + (int64_t)j * seg], s);
    }
  }
}

// Workgroups of the maximum pass: one 8-value vector per thread up to
// kMaxPartials workgroups (each thread's loads are all in flight at once)
int n_partials(int64_t count) {
  int64_t g = (count / 8 + kThreads - 1) / kThreads;
  if (g > kMaxPartials) g = kMaxPartials;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

size_t quant_workspace_bytes(int64_t count) {
  if (count <= kFusedMax) return 0;
  return (size_t)n_partials(count) * sizeof(uint32_t);
}

namespace {

template <int DT>
hipError_t launch_quant_rows_dt(const uint16_t* x, int64_t m, int64_t k, uint8_t* q, float* scales,
                                hipStream_t s) {
  // rows over grid.y; each row's cast split over grid.x so that few rows still fill
  // about 256 workgroups (chunks of at least kRowMinChunkVecs vectors)
  const int64_t rows = m < 65535 ? m : 65535, nvec = k / 8;
  int64_t splits = 256 / rows;
  const int64_t most = nvec / kRowMinChunkVecs;
  if (splits > most) splits = most;
  if (splits < 1) splits = 1;
  const int64_t chunk = (nvec + splits - 1) / splits;
  splits = (nvec + chunk - 1) / chunk;
  hipLaunchKernelGGL(quant_rows_kernel<DT>, dim3((int)splits, (int)rows), dim3(kThreads), 0, s, x, m, k, q, scales,
                     chunk);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_quant_dt(const uint16_t* x, int64_t count, uint8_t* q, float* scale, int mode, void* ws,
                           hipStream_t s) {
  const bool dynamic = mode == SP24_SCALE_DYNAMIC;
  if (count <= kFusedMax) {
    const int blocks = (int)((count + kFusedSlice - 1) / kFusedSlice);
    hipLaunchKernelGGL(fused_quant_kernel<DT>, dim3(blocks), dim3(kFusedThreads), 0, s, x, count, q, scale,
                       dynamic ? 1 : 0);
    return hipGetLastError();
  }
  // one vector per thread up to 2048 workgroups: the cast is spread over as many CUs
  // as there are vectors
  int64_t cast_blocks = (count / 8 + kThreads - 1) / kThreads;
  if (cast_blocks > 256 * 8) cast_blocks = 256 * 8;
  if (cast_blocks < 1) cast_blocks = 1;
  if (!dynamic) {
    hipLaunchKernelGGL(cast_kernel<DT>, dim3((int)cast_blocks), dim3(kThreads), 0, s, x, count, q,
                       scale, (const uint32_t*)nullptr, 0);
    return hipGetLastError();
  }
  const int np = n_partials(count);
  uint32_t* partial = static_cast<uint32_t*>(ws);
  hipLaunchKernelGGL(amax_partial_kernel, dim3(np), dim3(kThreads), 0, s, x, count, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cast_kernel<DT>, dim3((int)cast_blocks), dim3(kThreads), 0, s, x, count, q, scale,
                     (const uint32_t*)partial, np);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_rows(int dtype, const uint16_t* x, int64_t m, int64_t k, uint8_t* q, float* scales,
                             hipStream_t s) {
  return dtype == SP24_INT8 ? launch_quant_rows_dt<SP24_INT8>(x, m, k, q, scales, s)
                            : launch_quant_rows_dt<SP24_FP8_E4M3>(x, m, k, q, scales, s);
}

hipError_t launch_quant_groups(const uint16_t* x, int64_t rows, int64_t cols, int64_t group, uint8_t* q,
                               float* scales, hipStream_t s) {
  const int64_t vpg = group / 8, ngroups = rows * (cols / group);
  int seg = 1;
  while (seg < 64 && vpg % (2 * seg) == 0) seg *= 2;  // segments never straddle a wave
  int64_t blocks = (ngroups + kThreads / seg - 1) / (kThreads / seg);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(quant_groups_kernel<SP24_FP8_E4M3>, dim3((int)blocks), dim3(kThreads), 0, s, x, ngroups, group,
                     seg, q, scales);
  return hipGetLastError();
}

hipError_t launch_quant(int dtype, const uint16_t* x, int64_t count, uint8_t* q, float* scale, int mode,
                        void* ws, hipStream_t s) {
  return dtype == SP24_INT8 ? launch_quant_dt<SP24_INT8>(x, count, q, scale, mode, ws, s)
                            : launch_quant_dt<SP24_FP8_E4M3>(x, count, q, scale, mode, ws, s);
}

}  // namespace sp24
