// Device-side building blocks shared by the libdflash kernels (gfx950 only).
//
// Matrix-core fragments.  Every dense contraction in this library is cut into
// 16 x 16 output tiles and 32-wide k-chunks.  A fragment is the 8 consecutive
// k-elements one lane contributes to one k-chunk: lane l serves row (or column)
// l % 16 and k-elements 8*(l/16) .. 8*(l/16)+7 of the chunk.  Both operands of
// a product use the same lane -> k assignment, so the contraction is exact for
// any order in which the hardware walks k inside a chunk.
//   bf16: one v_mfma_f32_16x16x32_bf16 per chunk (fragment = 16 bytes).
//   fp32: eight v_mfma_f32_16x16x4_f32 per chunk; product j takes element j of
//         every lane's fragment (fragment = 32 bytes).
// The accumulator of a 16 x 16 tile holds, in lane l, column l % 16 and rows
// 4*(l/16) .. 4*(l/16)+3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct bf16_t {
  uint16_t bits;
};

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// scalar conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (NaN stays NaN), by gfx950's
// conversion instruction (v_cvt_pk_bf16_f32) rather than integer bit arithmetic.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// silu(g) * u = g / (1 + e^-g) * u with the exponential and the reciprocal from
// the transcendental unit (v_exp_f32 on g * -log2(e), v_rcp_f32): a few fp32
// ulps in all, far below the bf16 rounding of the product that follows.  Very
// negative g gives -0 (e^-g overflows to +inf), +inf gives +inf, NaN stays NaN.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896341f)) * u;
}

template <typename T> struct Storage;
template <> struct Storage<float> {
  __device__ __forceinline__ static float load(const float *p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float *p, size_t i, float v) { p[i] = v; }
  // value after rounding to the storage type
  __device__ __forceinline__ static float round(float v) { return v; }
};
template <> struct Storage<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t *p, size_t i) { return bf16_to_f32(p[i].bits); }
  __device__ __forceinline__ static void store(bf16_t *p, size_t i, float v) { p[i].bits = f32_to_bf16(v); }
  __device__ __forceinline__ static float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

// ---------------------------------------------------------------------------
// fragments
// ---------------------------------------------------------------------------
template <typename T> struct Frag;

template <> struct Frag<bf16_t> {
  uint4 v;  // 8 bf16
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void load(const bf16_t *p) { v = *reinterpret_cast<const uint4 *>(p); }
  // A weight fragment that one pass reads once: a non-temporal load (the `nt`
  // hint).  Streaming reads of HBM measured 6.8-7.1 TB/s with it and 6.0-6.2
  // TB/s without, on every grid shape tried.
  __device__ __forceinline__ void load_stream(const bf16_t *p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    v = make_uint4(t[0], t[1], t[2], t[3]);
  }
  __device__ __forceinline__ void store(bf16_t *p) const { *reinterpret_cast<uint4 *>(p) = v; }
  // element e as float (e in 0..7)
  __device__ __forceinline__ float get(int e) const {
    uint32_t w = (e < 2) ? v.x : (e < 4) ? v.y : (e < 6) ? v.z : v.w;
    return bf16_to_f32(static_cast<uint16_t>((e & 1) ? (w >> 16) : (w & 0xffffu)));
  }
  // pack 8 floats (rounded to bf16)
  __device__ __forceinline__ void set(const float *f) {
    v.x = f32_to_bf16(f[0]) | (static_cast<uint32_t>(f32_to_bf16(f[1])) << 16);
    v.y = f32_to_bf16(f[2]) | (static_cast<uint32_t>(f32_to_bf16(f[3])) << 16);
    v.z = f32_to_bf16(f[4]) | (static_cast<uint32_t>(f32_to_bf16(f[5])) << 16);
    v.w = f32_to_bf16(f[6]) | (static_cast<uint32_t>(f32_to_bf16(f[7])) << 16);
  }
};

typedef float f32x8 __attribute__((ext_vector_type(8)));
template <> struct Frag<float> {
  f32x8 v;
  __device__ __forceinline__ void zero() { v = f32x8{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ void load(const float *p) { v = *reinterpret_cast<const f32x8 *>(p); }
  __device__ __forceinline__ void load_stream(const float *p) {
    v = __builtin_nontemporal_load(reinterpret_cast<const f32x8 *>(p));
  }
  __device__ __forceinline__ void store(float *p) const { *reinterpret_cast<f32x8 *>(p) = v; }
  __device__ __forceinline__ float get(int e) const { return v[e]; }
  __device__ __forceinline__ void set(const float *f) { v = f32x8{f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]}; }
};

// acc += A_chunk * B_chunk for one 16 x 16 tile and one 32-wide k-chunk.
__device__ __forceinline__ f32x4 mma(f32x4 acc, const Frag<bf16_t> &a, const Frag<bf16_t> &b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v), __builtin_bit_cast(bf16x8, b.v),
                                                 acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x4 acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
  return acc;
}

// Four consecutive elements (group q4) of a row as floats, and the reverse
// (rounded to the storage type).
__device__ __forceinline__ float4 load4(const float *p, int q4) { return reinterpret_cast<const float4 *>(p)[q4]; }
__device__ __forceinline__ float4 load4(const bf16_t *p, int q4) {
  const uint2 u = reinterpret_cast<const uint2 *>(p)[q4];
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ void store4(float *p, int q4, float4 v) { reinterpret_cast<float4 *>(p)[q4] = v; }
__device__ __forceinline__ void store4(bf16_t *p, int q4, float4 v) {
  uint2 u;
  u.x = f32_to_bf16(v.x) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16);
  u.y = f32_to_bf16(v.z) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16);
  reinterpret_cast<uint2 *>(p)[q4] = u;
}

// acc += A * B for one 32 x 32 tile and a 16-wide k-chunk (v_mfma_f32_32x32x16_bf16):
// lane l supplies row (or column) l % 32 and k-elements 8*(l/32) .. +7, and holds
// column l % 32, rows 8*(i/4) + 4*(l/32) + i%4 of the result in element i.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mma32(f32x16 acc, const Frag<bf16_t> &a, const Frag<bf16_t> &b) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v), __builtin_bit_cast(bf16x8, b.v),
                                                 acc, 0, 0, 0);
}

// LDS-direct load: each lane's 16 bytes at gsrc land at LDS byte offset
// lds_off + 16 * lane (lds_off wave-uniform).  Issued through inline assembly
// so that the compiler does not treat later LDS reads as waiting on it (it
// would wait for every such load in flight, not just the ones those reads
// need); the caller waits with an explicit vmcnt.  Being invisible to the
// compiler's counters, such loads can only make its own waits stricter.
__device__ __forceinline__ unsigned lds_offset(const void *p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) void *)p;
}
// M0 carries the LDS base.  An SALU write of M0 needs one wait state before an
// LDS-DMA load reads it (a hazard the compiler cannot see inside asm), and M0
// is a reserved register the compiler may hold a value in, so it is saved and
// restored around the load.
__device__ __forceinline__ void lds_dma16(const void *gsrc, unsigned lds_off) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_off), "v"(gsrc)
      : "memory");
}

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (gfx9 encoding: vmcnt split over bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their no-wait maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) & 3) << 14 | 0x7 << 4 | 0xF << 8; }

__device__ __forceinline__ float f4get(const f32x4 &v, int i) {
  return i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3];
}

// Workgroup barrier ordering LDS accesses only.  Global loads and stores in
// flight stay in flight (a full __syncthreads would drain them when the wave
// has stored to global memory), so prefetched weights survive the barrier.
// Only for barriers that protect LDS data.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// RoPE angle pos * inv_freq with inv_freq = theta^(-2i/d): the angle in turns
// (pos * inv_freq / 2 pi) and its reduction to [-1/2, 1/2] in double, then the
// hardware sine and cosine of the reduced turn (v_sin_f32 / v_cos_f32, which
// take their argument in turns; max abs error 1.3e-7 on this range, measured,
// against 7e-8 for the library sincosf).
// A library sincosf here made the RoPE epilogues of the many-rows GEMMs ~5 us
// per 256 x 256 tile slower.
__device__ __forceinline__ void rope_cs_inv(int pos, double inv_freq, float *c, float *s) {
  const double t = static_cast<double>(pos) * inv_freq * 0.15915494309189535;
  const float f = static_cast<float>(t - rint(t));
  *s = __builtin_amdgcn_sinf(f);
  *c = __builtin_amdgcn_cosf(f);
}

__device__ __forceinline__ double rope_inv_freq(int i, int d, double log2_theta) {
  return exp2(-2.0 * static_cast<double>(i) / static_cast<double>(d) * log2_theta);
}

}  // namespace dflash
