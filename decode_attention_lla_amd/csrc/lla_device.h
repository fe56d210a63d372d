// Device-side helpers shared by the LLA kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lla {

// Storage tags. bf16 values are carried as raw 16-bit patterns. row(r): bytes of a latent row.
struct F32 {
  using T = float;
  static constexpr int kBytes = 4;
  static constexpr int row(int r) { return 4 * r; }
};
struct BF16 {
  using T = uint16_t;
  static constexpr int kBytes = 2;
  static constexpr int row(int r) { return 2 * r; }
};
// Low-bit latent rows: r OCP FP8 E4M3 codes, zero padding, the row's float32 scale in the last 4
// bytes, rounded up to 16 bytes. Only latent caches use it; the other arrays of such a call are bf16.
struct Q8 {
  static constexpr int kBytes = 1;
  static constexpr int row(int r) { return (r + 4 + 15) / 16 * 16; }
};
// The same rows with symmetric int8 codes (scale max|z| / 127).
struct I8 {
  static constexpr int kBytes = 1;
  static constexpr int row(int r) { return Q8::row(r); }
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// A value the caller knows to be the same in every lane (e.g. loaded from a wave-uniform address
// through a generic pointer, which the compiler must assume may differ per lane), moved to a
// scalar register so that what derives from it (loop bounds, buffer descriptors) stays scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16-byte LDS DMA of each lane's bytes at base + voffset + soffset into lds + 16 * lane, through a
// raw buffer descriptor of `bytes` bytes (stride 0, 32-bit data format word). A lane whose offset
// falls past `bytes` gets zeros. The lane offset and the wave-uniform offset stay separate
// operands, so the lane offset's register is never rewritten while a transfer may read it.
__device__ __forceinline__ void buffer_lds16(const void* base, int bytes, __attribute__((address_space(3))) void* lds,
                                             uint32_t voffset, uint32_t soffset) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, voffset, soffset, 0, 0);
}

// Workgroup barrier for LDS hand-offs: this wave's LDS accesses have completed (lgkmcnt(0)), then
// every wave arrives. Unlike __syncthreads() it neither waits for this wave's global loads still in
// flight into registers nor for global_load_lds transfers into other buffers (a workgroup-scope
// release fence counts those as pending LDS writes and waits for all of them). The memory clobbers
// keep the compiler from moving memory accesses across it.
// A value the compiler must treat as unknown (and as new at every evaluation), for LDS offsets:
// it keeps the compiler from deriving the addresses of one ring stage from another's (which loses
// the information that tells the stage read from the stages still being filled, so that it waits
// for every outstanding transfer) and from hoisting every stage's addresses out of a loop.
__device__ __forceinline__ int opaque(int v) {
  __asm__ volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// float32 -> bf16 bits, round to nearest, ties to even; NaN stays NaN (gfx950's v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));

// two float32 -> packed bf16 bits (a in the low half), round to nearest even, one instruction
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{a, b}, bf16x2_v));
}

template <class S>
__device__ __forceinline__ float ld(const void* base, size_t i);
template <>
__device__ __forceinline__ float ld<F32>(const void* base, size_t i) {
  return static_cast<const float*>(base)[i];
}
template <>
__device__ __forceinline__ float ld<BF16>(const void* base, size_t i) {
  return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[i]) << 16);
}

template <class S>
__device__ __forceinline__ void st(void* base, size_t i, float v);
template <>
__device__ __forceinline__ void st<F32>(void* base, size_t i, float v) {
  static_cast<float*>(base)[i] = v;
}
template <>
__device__ __forceinline__ void st<BF16>(void* base, size_t i, float v) {
  static_cast<uint16_t*>(base)[i] = f32_to_bf16(v);
}

// Element e of a register fragment holding E storage values as raw 16-byte words.
template <class S>
__device__ __forceinline__ float frag_elem(const uint4* f, int e);
template <>
__device__ __forceinline__ float frag_elem<F32>(const uint4* f, int e) {
  const uint4 w = f[e >> 2];
  const uint32_t x = (e & 3) == 0 ? w.x : (e & 3) == 1 ? w.y : (e & 3) == 2 ? w.z : w.w;
  return __uint_as_float(x);
}
template <>
__device__ __forceinline__ float frag_elem<BF16>(const uint4* f, int e) {
  const uint4 w = f[e >> 3];
  const int k = (e & 7) >> 1;
  const uint32_t x = k == 0 ? w.x : k == 1 ? w.y : k == 2 ? w.z : w.w;
  return (e & 1) ? bf16_hi(x) : bf16_lo(x);
}

template <>
__device__ __forceinline__ float frag_elem<Q8>(const uint4* f, int e) {
  const uint4 w = f[e >> 4];
  const int k = (e & 15) >> 2;
  const uint32_t x = k == 0 ? w.x : k == 1 ? w.y : k == 2 ? w.z : w.w;
  // hardware E4M3 -> f32 of byte e % 4 (the byte select must be a literal)
  switch (e & 3) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(x), 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(x), 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(x), 2);
    default: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(x), 3);
  }
}
// The float32 scale of a low-bit row held as V 16-byte words.
template <>
__device__ __forceinline__ float frag_elem<I8>(const uint4* f, int e) {
  const uint4 w = f[e >> 4];
  const int k = (e & 15) >> 2;
  const uint32_t x = k == 0 ? w.x : k == 1 ? w.y : k == 2 ? w.z : w.w;
  return static_cast<float>(static_cast<int8_t>(x >> (8 * (e & 3))));  // sign-extending byte extract
}

__device__ __forceinline__ float q8_row_scale(const uint4* f, int V) { return __uint_as_float(f[V - 1].w); }

// 16-byte load of data that is read exactly once, for loads whose 64 lanes cover whole cache
// lines (one instruction reads 1 KiB contiguous): a non-temporal hint keeps the stream from
// displacing reused data. Partial-line patterns must use ordinary loads, which let the next
// instruction hit the same lines.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// W 32-bit words (1..4) at byte offset voff of a raw buffer, returned in the low words of a uint4
// (the rest zero). An offset at or past the descriptor's size reads zeros. AUX is the cache policy
// (2: non-temporal, for data read once by loads that cover whole lines).
template <int W, int AUX>
__device__ __forceinline__ uint4 buffer_words(__amdgpu_buffer_rsrc_t rs, uint32_t voff) {
  static_assert(W >= 1 && W <= 4, "1 to 4 words");
  if constexpr (W == 4) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, AUX);
    return make_uint4(v[0], v[1], v[2], v[3]);
  } else if constexpr (W == 3) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b96(rs, voff, 0, AUX);
    return make_uint4(v[0], v[1], v[2], 0u);
  } else if constexpr (W == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, 0, AUX);
    return make_uint4(v[0], v[1], 0u, 0u);
  } else {
    return make_uint4(__builtin_amdgcn_raw_buffer_load_b32(rs, voff, 0, AUX), 0u, 0u, 0u);
  }
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const u32x4_t t = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Max and sum over lanes l, l^16, l^32, l^48 (the four 16-lane groups of a wave) with the gfx950
// lane-swap instructions: VALU only, no LDS round trip. Each swap hands every lane its partner's
// value in one of the two results and its own value in the other.
__device__ __forceinline__ float max_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Rotate the pair (x0, x1) of channel pair i at position pos (float64 angle and trigonometry).
__device__ __forceinline__ void rotate_pair(float x0, float x1, int i, int d, double pos,
                                            double base, float* y0, float* y1) {
  const double theta = pow(base, -2.0 * i / d);
  double s, c;
  sincos(pos * theta, &s, &c);
  *y0 = static_cast<float>(x0 * c - x1 * s);
  *y1 = static_cast<float>(x0 * s + x1 * c);
}

// Sum over aligned groups of N lanes (N a power of two, 1..64), VALU only: a butterfly whose
// partner steps are DPP quad permutes (lane ^ 1, lane ^ 2), the half-row and row mirrors (which
// pair each 4- and 8-lane group with its neighbour) and the two lane swaps. Every step adds two
// values, so all lanes of a group end with the same bits.
template <int DPP>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), DPP, 0xf, 0xf, false));
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "power of two up to the wave");
  if constexpr (N >= 2) v += dpp_f32<0xb1>(v);   // quad_perm(1, 0, 3, 2)
  if constexpr (N >= 4) v += dpp_f32<0x4e>(v);   // quad_perm(2, 3, 0, 1)
  if constexpr (N >= 8) v += dpp_f32<0x141>(v);  // row_half_mirror
  if constexpr (N >= 16) v += dpp_f32<0x140>(v); // row_mirror
  if constexpr (N >= 32) {
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  }
  if constexpr (N >= 64) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  }
  return v;
}

}  // namespace lla
