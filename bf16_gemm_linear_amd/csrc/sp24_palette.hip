// Lossless BF16 exponent-palette weights and their GEMM ("Unweight: Compresion
// Lossless de Pesos de LLM para Inferencia en GPU H100", architecture and
// execution pipelines).
//
// Format.  The 8 exponent bits are the redundant part of a BF16 weight; sign
// and mantissa are kept as one byte.  One palette per tensor holds its 16 most
// common exponents (by count, ties to the smaller exponent; unused entries
// 0xFF, the Inf/NaN exponent, which no finite weight has).  A row whose
// exponents are all in the palette is stored as sign+mantissa bytes plus one
// 4-bit palette index per element (element 8g + t, t < 4, at bits [8t, 8t+4)
// of word g, element 8g + 4 + t at bits [8t+4, 8t+8)); any other row is stored
// verbatim.  Both kinds are compact, in ascending row order, with their row
// numbers, so the GEMM never branches per element.
//
// Storage order.  The arrays of each kind are cut into blocks of 16 rows (the
// last block padded; padding is read, never stored) and K into chunks of 512
// (the last chunk T*128 values when K % 512 != 0).  Inside a (block, chunk)
// tile the 16-byte pieces are ordered [piece j][lane group q][row r16], lane
// group q holding K [32Tq, 32T(q+1)) of the chunk, which is exactly the order
// in which the GEMM's lanes (lane = 16q + r16) consume them: every 64-lane
// load reads 1 KB of consecutive memory, whole cache lines.
//
// Encoding (load time, three passes over W): an exponent histogram, the palette
// with the exponent -> index table, a per-row verdict, a scan that gives every
// row its slot, and the pack.  No host synchronisation inside a call; the
// caller reads the two row counts between sp24_palette_analyze and
// sp24_palette_pack to size the outputs.
//
// GEMM.  For few tokens (m <= 16, the page's "direct palette" pipeline) a
// kernel streams the encoded rows and rebuilds BF16 in registers right before
// the matrix instructions, so BF16 weights never exist in memory: 1.5 bytes
// per weight instead of 2 for paletted rows.  For more tokens the page's "full
// decode" pipeline is used: the weight is rebuilt into the workspace and the
// dense BF16 GEMM runs on it.
#include "sp24_common.hpp"
#include "sp24_internal.hpp"

namespace sp24 {
namespace {

constexpr int kPalThreads = 256;
constexpr uint32_t kUnused = 0xFFu;

__device__ __forceinline__ uint32_t exp_of(uint32_t h) { return (h >> 7) & 0xFFu; }

// Byte offset, in the storage order of an array with b32 bytes per 32 values
// of a row (sign+mantissa 32, index words 16, verbatim bf16 64), of value kel
// of compact row p.
__device__ __forceinline__ int64_t tile_offset(int64_t p, int64_t kel, int64_t k, int b32) {
  const int64_t b = p >> 4, r16 = p & 15;
  const int64_t c = kel >> 9, kk = kel & 511;
  const int64_t units = k >> 7, full = units >> 2;
  const int64_t t = c < full ? 4 : units - 4 * full;       // units of this chunk
  const int64_t span = 32 * t;                              // values per lane group
  const int64_t q = kk / span, o = (kk - q * span) * b32 / 32;  // byte offset in the lane group's range
  return b * 16 * (k / 32 * b32) + c * 256 * b32 + 16 * (64 * (o >> 4) + 16 * q + r16) + (o & 15);
}

// ---------------------------------------------------------------- analysis

__global__ __launch_bounds__(kPalThreads) void pal_zero_kernel(uint32_t* __restrict__ p, int count) {
  for (int i = threadIdx.x; i < count; i += kPalThreads) p[i] = 0u;
}

// Exponent histogram: per-workgroup counts in LDS, then added to the global table.
__global__ __launch_bounds__(kPalThreads) void pal_hist_kernel(const uint16_t* __restrict__ w, int64_t count,
                                                               uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[256];
  h[threadIdx.x] = 0u;
  __syncthreads();
  const int64_t nvec = count / 8;
  const int64_t stride = (int64_t)gridDim.x * kPalThreads;
  const u32x4* wv = reinterpret_cast<const u32x4*>(w);
  for (int64_t i = (int64_t)blockIdx.x * kPalThreads + threadIdx.x; i < nvec; i += stride) {
    const u32x4 v = wv[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      atomicAdd(&h[exp_of(v[j] & 0xFFFFu)], 1u);
      atomicAdd(&h[exp_of(v[j] >> 16)], 1u);
    }
  }
  __syncthreads();
  if (h[threadIdx.x] != 0u) atomicAdd(&hist[threadIdx.x], h[threadIdx.x]);
}

// Palette = exponents ranked by (count descending, exponent ascending), the
// first 16 that occur; lut[e] = its palette index or 0xFF.
__global__ __launch_bounds__(256) void pal_select_kernel(const uint32_t* __restrict__ hist,
                                                         uint8_t* __restrict__ palette,
                                                         uint8_t* __restrict__ lut) {
  __shared__ uint32_t c[256];
  const int e = threadIdx.x;
  c[e] = hist[e];
  if (e < 16) palette[e] = (uint8_t)kUnused;
  __syncthreads();
  const uint32_t mine = c[e];
  int rank = 0;
  for (int j = 0; j < 256; ++j) rank += (c[j] > mine || (c[j] == mine && j < e)) ? 1 : 0;
  const bool in = mine > 0u && rank < 16;
  lut[e] = in ? (uint8_t)rank : (uint8_t)kUnused;
  __syncthreads();  // every unused entry is written before the used ones
  if (in) palette[rank] = (uint8_t)e;
}

// verdict[r] = 1 when row r has an exponent outside the palette.
__global__ __launch_bounds__(kPalThreads) void pal_classify_kernel(const uint16_t* __restrict__ w, int64_t n,
                                                                   int64_t k, const uint8_t* __restrict__ lut_g,
                                                                   uint32_t* __restrict__ verdict) {
  __shared__ uint8_t lut[256];
  __shared__ uint32_t any;
  lut[threadIdx.x] = lut_g[threadIdx.x];
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    if (threadIdx.x == 0) any = 0u;
    __syncthreads();
    const u32x4* row = reinterpret_cast<const u32x4*>(w + r * k);
    uint32_t miss = 0u;
    for (int64_t i = threadIdx.x; i < k / 8; i += kPalThreads) {
      const u32x4 v = row[i];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        miss |= (uint32_t)(lut[exp_of(v[j] & 0xFFFFu)] == kUnused) | (uint32_t)(lut[exp_of(v[j] >> 16)] == kUnused);
    }
    if (miss) any = 1u;  // benign race: every writer stores 1
    __syncthreads();
    if (threadIdx.x == 0) verdict[r] = any;
    __syncthreads();
  }
}

// Slots in row order: paletted row -> its index p (>= 0), verbatim row -> -(v + 1).
__global__ __launch_bounds__(1024) void pal_scan_kernel(const uint32_t* __restrict__ verdict, int64_t n,
                                                        int32_t* __restrict__ slot, int32_t* __restrict__ counts) {
  __shared__ int32_t part[1024];
  __shared__ int32_t base_v;
  if (threadIdx.x == 0) base_v = 0;
  __syncthreads();
  for (int64_t r0 = 0; r0 < n; r0 += 1024) {
    const int64_t r = r0 + threadIdx.x;
    const int32_t v = r < n ? (int32_t)verdict[r] : 0;
    part[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan of the verbatim flags
      const int32_t add = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += add;
      __syncthreads();
    }
    const int32_t before = base_v + part[threadIdx.x] - v;  // verbatim rows before r
    if (r < n) slot[r] = v ? -(before + 1) : (int32_t)(r - before);
    __syncthreads();
    if (threadIdx.x == 1023) base_v += part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    counts[0] = (int32_t)(n - base_v);
    counts[1] = base_v;
  }
}

// ---------------------------------------------------------------- pack / rebuild

// Pack every row into its slot (slots outside [0, n_pal) / [0, n_verb) are skipped).
__global__ __launch_bounds__(kPalThreads) void pal_pack_kernel(
    const uint16_t* __restrict__ w, int64_t n, int64_t k, const uint8_t* __restrict__ palette,
    const int32_t* __restrict__ slot, int64_t n_pal, int64_t n_verb, uint8_t* __restrict__ sm,
    uint32_t* __restrict__ ix, int32_t* __restrict__ pal_rows, uint16_t* __restrict__ verb,
    int32_t* __restrict__ verb_rows) {
  __shared__ uint8_t lut[256];
  lut[threadIdx.x] = (uint8_t)kUnused;
  __syncthreads();
  if (threadIdx.x < 16 && palette[threadIdx.x] != kUnused) lut[palette[threadIdx.x]] = (uint8_t)threadIdx.x;
  __syncthreads();
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    const int32_t s = slot[r];
    const u32x4* row = reinterpret_cast<const u32x4*>(w + r * k);
    if (s >= 0 && s < n_pal) {
      if (threadIdx.x == 0) pal_rows[s] = (int32_t)r;
      for (int64_t i = threadIdx.x; i < k / 8; i += kPalThreads) {
        const u32x4 v = row[i];
        uint32_t b[2] = {0u, 0u}, word = 0u;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const uint32_t h = (v[t >> 1] >> (16 * (t & 1))) & 0xFFFFu;
          const uint32_t byte = ((h >> 8) & 0x80u) | (h & 0x7Fu);
          b[t >> 2] |= byte << (8 * (t & 3));
          const uint32_t idx = lut[exp_of(h)] & 15u;  // rows in this slot kind are all in the palette
          word |= idx << (t < 4 ? 8 * t : 8 * (t - 4) + 4);
        }
        *reinterpret_cast<u32x2*>(sm + tile_offset(s, 8 * i, k, 32)) = u32x2{b[0], b[1]};
        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(ix) + tile_offset(s, 8 * i, k, 16)) = word;
      }
    } else if (s < 0 && -(int64_t)s - 1 < n_verb) {
      const int64_t v = -(int64_t)s - 1;
      if (threadIdx.x == 0) verb_rows[v] = (int32_t)r;
      uint8_t* vb = reinterpret_cast<uint8_t*>(verb);
      for (int64_t i = threadIdx.x; i < k / 8; i += kPalThreads)
        *reinterpret_cast<u32x4*>(vb + tile_offset(v, 8 * i, k, 64)) = row[i];
    }
  }
}

// Exponents of 4 palette indices (one per byte, 0..15) from the 16-byte
// palette t0..t3: two byte permutes pick from entries 0..7 and 8..15, bit 3
// of each index selects between them.
__device__ __forceinline__ uint32_t lut4(uint32_t s, uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3) {
  const uint32_t sel = s & 0x07070707u;
  const uint32_t lo = __builtin_amdgcn_perm(t1, t0, sel);
  const uint32_t hi = __builtin_amdgcn_perm(t3, t2, sel);
  const uint32_t m = ((s >> 3) & 0x01010101u) * 0xFFu;
  return (hi & m) | (lo & ~m);
}

// 8 BF16 (as 4 words, element 2j in the low half of word j) from 8
// sign+mantissa bytes and one index word.
__device__ __forceinline__ i32x4 rebuild8(u32x2 smv, uint32_t word, uint32_t t0, uint32_t t1, uint32_t t2,
                                          uint32_t t3) {
  const uint32_t e_lo = lut4(word & 0x0F0F0F0Fu, t0, t1, t2, t3);         // elements 0..3
  const uint32_t e_hi = lut4((word >> 4) & 0x0F0F0F0Fu, t0, t1, t2, t3);  // elements 4..7
  // per element: high byte = sign | exponent >> 1, low byte = exponent bit 0 << 7 | mantissa
  const uint32_t h0 = (smv[0] & 0x80808080u) | ((e_lo >> 1) & 0x7F7F7F7Fu);
  const uint32_t l0 = ((e_lo << 7) & 0x80808080u) | (smv[0] & 0x7F7F7F7Fu);
  const uint32_t h1 = (smv[1] & 0x80808080u) | ((e_hi >> 1) & 0x7F7F7F7Fu);
  const uint32_t l1 = ((e_hi << 7) & 0x80808080u) | (smv[1] & 0x7F7F7F7Fu);
  return i32x4{(int)__builtin_amdgcn_perm(h0, l0, 0x05010400u), (int)__builtin_amdgcn_perm(h0, l0, 0x07030602u),
               (int)__builtin_amdgcn_perm(h1, l1, 0x05010400u), (int)__builtin_amdgcn_perm(h1, l1, 0x07030602u)};
}

__device__ __forceinline__ void load_palette(const uint8_t* palette, uint32_t& t0, uint32_t& t1, uint32_t& t2,
                                             uint32_t& t3) {
  const u32x4 p = *reinterpret_cast<const u32x4*>(palette);
  t0 = p[0];
  t1 = p[1];
  t2 = p[2];
  t3 = p[3];
}

// Rebuild W [n, k]: paletted rows first (blocks [0, n_pal)), then verbatim rows.
__global__ __launch_bounds__(kPalThreads) void pal_decode_kernel(
    const uint8_t* __restrict__ palette, int64_t n_pal, const uint8_t* __restrict__ sm,
    const uint32_t* __restrict__ ix, const int32_t* __restrict__ pal_rows, int64_t n_verb,
    const uint16_t* __restrict__ verb, const int32_t* __restrict__ verb_rows, int64_t n, int64_t k,
    uint16_t* __restrict__ w) {
  uint32_t t0, t1, t2, t3;
  load_palette(palette, t0, t1, t2, t3);
  for (int64_t b = blockIdx.x; b < n_pal + n_verb; b += gridDim.x) {
    if (b < n_pal) {
      const int64_t r = pal_rows[b];
      if (r < 0 || r >= n) continue;
      const uint8_t* ixb = reinterpret_cast<const uint8_t*>(ix);
      i32x4* dst = reinterpret_cast<i32x4*>(w + r * k);
      for (int64_t i = threadIdx.x; i < k / 8; i += kPalThreads)
        dst[i] = rebuild8(*reinterpret_cast<const u32x2*>(sm + tile_offset(b, 8 * i, k, 32)),
                          *reinterpret_cast<const uint32_t*>(ixb + tile_offset(b, 8 * i, k, 16)), t0, t1, t2, t3);
    } else {
      const int64_t v = b - n_pal;
      const int64_t r = verb_rows[v];
      if (r < 0 || r >= n) continue;
      const uint8_t* vb = reinterpret_cast<const uint8_t*>(verb);
      u32x4* dst = reinterpret_cast<u32x4*>(w + r * k);
      for (int64_t i = threadIdx.x; i < k / 8; i += kPalThreads)
        dst[i] = *reinterpret_cast<const u32x4*>(vb + tile_offset(v, 8 * i, k, 64));
    }
  }
}

// ---------------------------------------------------------------- GEMM, m <= 16

// Each workgroup owns RB 16-row blocks of one kind (the first workgroups the
// paletted rows, the rest the verbatim rows) and all m <= 16 tokens; its NW
// waves share K in chunks of T units of 128 values, and a wave's X registers
// serve its RB row blocks.  Within a chunk, lane group q = lane / 16 takes the
// contiguous K range [kb + 32Tq, +32T) of row lane % 16 (one tile of the
// storage order: load j of the wave reads bytes [16 (64 j + lane), +16) of the
// tile) and instruction j uses its values [8j, 8j + 8); the X operand (token
// lane % 16) uses the same map, so the sum over K is the product's.  The
// accumulator (v_mfma_f32_16x16x32_bf16) is a tile of Y^T: lane l, register
// j <-> row 4(l/16) + j, token l % 16.
template <bool VERB, int T, int RB, bool XL>
struct PalChunk {
  // per lane and row block: paletted: 32T sign+mantissa bytes (2T vectors) and
  // 4T index words (T vectors); verbatim: 32T bf16 (4T vectors); X: 32T bf16
  // (4T vectors), unless X sits in LDS (XL)
  static constexpr int WV = VERB ? 4 * T : 2 * T;
  i32x4 wv[RB][WV];
  i32x4 iv[RB][VERB ? 1 : T];
  i32x4 xv[XL ? 1 : 4 * T];
};

// The encoded rows are read once per call: their loads carry the non-temporal hint
// (up-projection at m = 1: 18.0 against 19.6 us, down 24.7 against 28.4 us).
template <bool VERB, int T, int RB, bool XL>
__device__ __forceinline__ void pal_load(PalChunk<VERB, T, RB, XL>& c, const uint8_t* __restrict__ wbase,
                                         const uint8_t* __restrict__ ixbase, const uint16_t* __restrict__ x,
                                         int blk0, int last_blk, int chunk, int lane, int token, int kq, int M,
                                         int K) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t blk = min(blk0 + rb, last_blk);  // past the last block: reread it, never stored
    if constexpr (VERB) {  // 64 bytes per 32 values: tile of 16 rows x 512 values = 16 KB
      const uint8_t* p = wbase + blk * 32 * K + (int64_t)chunk * 16384 + 16 * lane;
#pragma unroll
      for (int j = 0; j < 4 * T; ++j) c.wv[rb][j] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p + 1024 * j));
    } else {               // sign+mantissa: 32 bytes per 32 values; indices: 16 bytes per 32 values
      const uint8_t* p = wbase + blk * 16 * K + (int64_t)chunk * 8192 + 16 * lane;
#pragma unroll
      for (int j = 0; j < 2 * T; ++j) c.wv[rb][j] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p + 1024 * j));
      const uint8_t* q = ixbase + blk * 8 * K + (int64_t)chunk * 4096 + 16 * lane;
#pragma unroll
      for (int j = 0; j < T; ++j) c.iv[rb][j] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(q + 1024 * j));
    }
  }
  if constexpr (!XL) {
    if (token < M) {
      const uint16_t* xr = x + (int64_t)token * K + kq;
#pragma unroll
      for (int j = 0; j < 4 * T; ++j) c.xv[j] = *reinterpret_cast<const i32x4*>(xr + 8 * j);
    } else {
#pragma unroll
      for (int j = 0; j < 4 * T; ++j) c.xv[j] = i32x4{0, 0, 0, 0};
    }
  }
}

// X in LDS (XL): row t of X at byte t * xstride; lanes of tokens >= M use zeros.
template <bool VERB, int T, int RB, bool XL>
__device__ __forceinline__ void pal_mma(f32x4 (&acc)[RB], const PalChunk<VERB, T, RB, XL>& c, uint32_t t0, uint32_t t1,
                                        uint32_t t2, uint32_t t3, const uint8_t* xl, int kq, int token, int M) {
#pragma unroll
  for (int j = 0; j < 4 * T; ++j) {  // instruction j: values [8j, 8j + 8) of the lane's range
    i32x4 xb;
    if constexpr (XL) {
      xb = i32x4{0, 0, 0, 0};
      if (token < M) xb = *reinterpret_cast<const i32x4*>(xl + 2 * (kq + 8 * j));
    } else {
      xb = c.xv[j];
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      i32x4 a;
      if constexpr (VERB) {
        a = c.wv[rb][j];
      } else {
        const i32x4 s = c.wv[rb][j >> 1];
        const u32x2 smv = (j & 1) ? u32x2{(uint32_t)s[2], (uint32_t)s[3]} : u32x2{(uint32_t)s[0], (uint32_t)s[1]};
        a = rebuild8(smv, (uint32_t)c.iv[rb][j >> 2][j & 3], t0, t1, t2, t3);
      }
      acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, xb),
                                                        acc[rb], 0, 0, 0);
    }
  }
}

template <bool VERB, int T, int RB, bool XL>
__device__ __forceinline__ void pal_chunk(f32x4 (&acc)[RB], const uint8_t* wbase, const uint8_t* ixbase,
                                          const uint16_t* x, const uint8_t* xl, int blk0, int last_blk, int chunk,
                                          int lane, int token, int M, int K, uint32_t t0, uint32_t t1, uint32_t t2,
                                          uint32_t t3) {
  PalChunk<VERB, T, RB, XL> c;
  const int kq = chunk * 512 + 32 * T * (lane >> 4);
  pal_load<VERB, T, RB, XL>(c, wbase, ixbase, x, blk0, last_blk, chunk, lane, token, kq, M, K);
  pal_mma<VERB, T, RB, XL>(acc, c, t0, t1, t2, t3, xl, kq, token, M);
}

template <bool VERB, int NW, int RB, bool XL>
__device__ __forceinline__ void pal_rows_tile(f32x4 (&acc)[RB], const uint8_t* wbase, const uint8_t* ixbase,
                                              const uint16_t* x, const uint8_t* xl, int blk0, int last_blk, int token,
                                              int wave, int lane, int M, int K, uint32_t t0, uint32_t t1,
                                              uint32_t t2, uint32_t t3) {
  const int units = K / 128, full = units / 4, tail = units % 4;
  int c = wave;
  if constexpr (XL) {
    // X comes from LDS, so the registers hold two chunks of W: both loads in flight
    for (; c + NW < full; c += 2 * NW) {
      PalChunk<VERB, 4, RB, XL> a, b;
      const int ka = c * 512 + 128 * (lane >> 4), kb = ka + NW * 512;
      pal_load<VERB, 4, RB, XL>(a, wbase, ixbase, x, blk0, last_blk, c, lane, token, ka, M, K);
      pal_load<VERB, 4, RB, XL>(b, wbase, ixbase, x, blk0, last_blk, c + NW, lane, token, kb, M, K);
      pal_mma<VERB, 4, RB, XL>(acc, a, t0, t1, t2, t3, xl, ka, token, M);
      pal_mma<VERB, 4, RB, XL>(acc, b, t0, t1, t2, t3, xl, kb, token, M);
    }
  }
  // otherwise one chunk's loads in flight per wave; the waves of the CU's
  // workgroups keep the memory system busy
  for (; c < full; c += NW)
    pal_chunk<VERB, 4, RB, XL>(acc, wbase, ixbase, x, xl, blk0, last_blk, c, lane, token, M, K, t0, t1, t2, t3);
  if (tail != 0 && wave == full % NW) {
    if (tail == 1)
      pal_chunk<VERB, 1, RB, XL>(acc, wbase, ixbase, x, xl, blk0, last_blk, full, lane, token, M, K, t0, t1, t2, t3);
    else if (tail == 2)
      pal_chunk<VERB, 2, RB, XL>(acc, wbase, ixbase, x, xl, blk0, last_blk, full, lane, token, M, K, t0, t1, t2, t3);
    else
      pal_chunk<VERB, 3, RB, XL>(acc, wbase, ixbase, x, xl, blk0, last_blk, full, lane, token, M, K, t0, t1, t2, t3);
  }
}

template <int NW, int RB, bool XL>
__global__ __launch_bounds__(NW * 64) void pal_gemm_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ palette, int n_pal, const uint8_t* __restrict__ sm,
    const uint32_t* __restrict__ ix, const int32_t* __restrict__ pal_rows, int n_verb,
    const uint16_t* __restrict__ verb, const int32_t* __restrict__ verb_rows, uint16_t* __restrict__ y, int M, int N,
    int K) {
  __shared__ float red[NW * RB * 256];
  extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];  // XL: X [M, K] bf16, rows xstride apart
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gp = (n_pal + 16 * RB - 1) / (16 * RB);     // workgroups of paletted rows
  const bool verb_blk = (int)blockIdx.x >= gp;          // uniform per workgroup
  const int count = verb_blk ? n_verb : n_pal;          // rows past count: padding or reread, never stored
  const int blk0 = ((int)blockIdx.x - (verb_blk ? gp : 0)) * RB;
  const int last_blk = (count + 15) / 16 - 1;
  const int token = lane & 15;
  uint32_t t0, t1, t2, t3;
  load_palette(palette, t0, t1, t2, t3);
  const int xstride = 2 * K + 64;  // bytes: consecutive tokens' rows start 16 banks apart
  if constexpr (XL) {
    const int vecs = K / 8;  // 16-byte vectors per row
    for (int i = threadIdx.x; i < M * vecs; i += NW * 64) {
      const int t = i / vecs, v = i - t * vecs;
      *reinterpret_cast<i32x4*>(xlds + t * xstride + 16 * v) =
          *reinterpret_cast<const i32x4*>(x + (int64_t)t * K + 8 * v);
    }
    __syncthreads();
  }
  const uint8_t* xl = xlds + (token < M ? token : 0) * xstride;

  f32x4 acc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (verb_blk)
    pal_rows_tile<true, NW, RB, XL>(acc, reinterpret_cast<const uint8_t*>(verb), nullptr, x, xl, blk0, last_blk,
                                    token, wave, lane, M, K, t0, t1, t2, t3);
  else
    pal_rows_tile<false, NW, RB, XL>(acc, sm, reinterpret_cast<const uint8_t*>(ix), x, xl, blk0, last_blk, token,
                                     wave, lane, M, K, t0, t1, t2, t3);

#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[(wave * RB + rb) * 256 + j * 64 + lane] = acc[rb][j];
  __syncthreads();
  // output o = (rb * 16 + token) * 16 + row-in-block: waves summed in a fixed order
  const int32_t* rows = verb_blk ? verb_rows : pal_rows;
  for (int o = threadIdx.x; o < RB * 256; o += NW * 64) {
    const int rl = o & 15, tk = (o >> 4) & 15, rb = o >> 8;
    const int src = rb * 256 + (rl & 3) * 64 + (rl >> 2) * 16 + tk;  // register rl % 4 of lane 16 (rl / 4) + tk
    float s = 0.f;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) s += red[wv * RB * 256 + src];
    const int ri = (blk0 + rb) * 16 + rl;
    if (ri < count && tk < M) {
      const int n = rows[ri];
      if (n >= 0 && n < N) y[(int64_t)tk * N + n] = (uint16_t)f32_to_bf16_rne(s);
    }
  }
}

int grid_rows(int64_t rows) { return (int)(rows < 65536 ? (rows > 0 ? rows : 1) : 65536); }

}  // namespace

size_t palette_analyze_ws_bytes(int64_t n) { return 256 * 4 + 256 + ((size_t)n * 4 + 15) / 16 * 16; }

hipError_t launch_palette_analyze(const uint16_t* w, int64_t n, int64_t k, uint8_t* palette, int32_t* slot,
                                  int32_t* counts, void* ws, hipStream_t s) {
  uint8_t* b = static_cast<uint8_t*>(ws);
  uint32_t* hist = reinterpret_cast<uint32_t*>(b);
  uint8_t* lut = b + 1024;
  uint32_t* verdict = reinterpret_cast<uint32_t*>(b + 1280);
  hipLaunchKernelGGL(pal_zero_kernel, dim3(1), dim3(kPalThreads), 0, s, hist, 256);
  const int64_t nvec = n * k / 8;
  int64_t blocks = (nvec + kPalThreads * 8 - 1) / (kPalThreads * 8);
  blocks = blocks < 1 ? 1 : (blocks > 2048 ? 2048 : blocks);
  hipLaunchKernelGGL(pal_hist_kernel, dim3((int)blocks), dim3(kPalThreads), 0, s, w, n * k, hist);
  hipLaunchKernelGGL(pal_select_kernel, dim3(1), dim3(256), 0, s, hist, palette, lut);
  hipLaunchKernelGGL(pal_classify_kernel, dim3(grid_rows(n)), dim3(kPalThreads), 0, s, w, n, k, lut, verdict);
  hipLaunchKernelGGL(pal_scan_kernel, dim3(1), dim3(1024), 0, s, verdict, n, slot, counts);
  return hipGetLastError();
}

hipError_t launch_palette_pack(const uint16_t* w, int64_t n, int64_t k, const uint8_t* palette, const int32_t* slot,
                               int64_t n_pal, int64_t n_verb, uint8_t* sm, uint32_t* ix, int32_t* pal_rows,
                               uint16_t* verb, int32_t* verb_rows, hipStream_t s) {
  hipLaunchKernelGGL(pal_pack_kernel, dim3(grid_rows(n)), dim3(kPalThreads), 0, s, w, n, k, palette, slot, n_pal,
                     n_verb, sm, ix, pal_rows, verb, verb_rows);
  return hipGetLastError();
}

hipError_t launch_palette_decode(const PaletteArgs& p, int64_t n, int64_t k, uint16_t* w, hipStream_t s) {
  hipLaunchKernelGGL(pal_decode_kernel, dim3(grid_rows(p.n_pal + p.n_verb)), dim3(kPalThreads), 0, s, p.palette,
                     p.n_pal, p.sm, p.ix, p.pal_rows, p.n_verb, p.verb, p.verb_rows, n, k, w);
  return hipGetLastError();
}

template <int RB, bool XL>
hipError_t launch_pal_gemm(const uint16_t* x, const PaletteArgs& p, uint16_t* y, int m, int n, int k, hipStream_t s) {
  const int64_t blocks = (p.n_pal + 16 * RB - 1) / (16 * RB) + (p.n_verb + 16 * RB - 1) / (16 * RB);
  const size_t lds = XL ? (size_t)m * (2 * k + 64) : 0;
  hipLaunchKernelGGL((pal_gemm_kernel<kPaletteWaves, RB, XL>), dim3((int)blocks), dim3(kPaletteWaves * 64), lds, s,
                     x, p.palette, (int)p.n_pal, p.sm, p.ix, p.pal_rows, (int)p.n_verb, p.verb, p.verb_rows, y, m, n,
                     k);
  return hipGetLastError();
}

hipError_t launch_palette_gemm_small(const uint16_t* x, const PaletteArgs& p, uint16_t* y, int m, int n, int k,
                                     hipStream_t s) {
  // one token with a short enough X: X once per workgroup into LDS, and the registers
  // free for two chunks of W in flight (measured faster at m = 1, slower at m = 4);
  // more tokens: more row blocks share a wave's X registers (X is re-read from L2 per
  // workgroup)
  if (m <= kPaletteXlMaxM && (int64_t)m * (2 * k + 64) <= kPaletteXLdsBytes)
    return launch_pal_gemm<1, true>(x, p, y, m, n, k, s);
  return m <= kPaletteRb1MaxM ? launch_pal_gemm<1, false>(x, p, y, m, n, k, s)
                              : launch_pal_gemm<kPaletteRbWide, false>(x, p, y, m, n, k, s);
}

}  // namespace sp24
