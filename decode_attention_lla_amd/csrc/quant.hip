// Low-bit latent rows (LLA_BF16_Q8, LLA_BF16_I8): bf16 latent rows quantised to OCP FP8 E4M3 or
// symmetric int8 codes with one float32 scale per row, written into a low-bit cache.
//
// Method context: O'Neill & Reid, "Looped Latent Attention", arXiv 2607.15456. Section 8
// ("Compositionality") notes that quantisation acts on a different tensor dimension than the loop
// codec and can be stacked on it; Appendix C evaluates an 8-bit codec. The row format is stated at
// LLA_BF16_Q8 in lla.h: s = max|z| / 448, code_j = e4m3(z_j / s), both divisions in float32 and
// rounded to nearest even (gfx950's v_cvt_pk_fp8_f32 rounds to nearest even in the OCP E4M3
// format), codes at bytes [0, r), zero padding, s in the last 4 bytes of a 16-byte-aligned row.
// LLA_BF16_I8: s = max|z| / 127, code_j = round(z_j / s) with halves to even (v_rndne_f32) as a
// two's-complement byte, the division in float32; same layout.
#include <hip/hip_runtime.h>

#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace {

constexpr int kThreads = 256;

// One thread per source row (b, h, c): per-head source [B][H][C][r] (LLA-2D: H = 1). Grid y is
// the axis: the K rows (pk) and the V rows (pv) of one call share a launch.
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(QuantParams pk, QuantParams pv) {
  const bool v = blockIdx.y != 0;
  QuantParams p;  // field by field, so each stays a scalar
  p.src = v ? pv.src : pk.src;
  p.dst = v ? pv.dst : pk.dst;
  p.pos = v ? pv.pos : pk.pos;
  p.B = v ? pv.B : pk.B;
  p.C = v ? pv.C : pk.C;
  p.H = v ? pv.H : pk.H;
  p.r = v ? pv.r : pk.r;
  p.n_max = v ? pv.n_max : pk.n_max;
  p.int8 = v ? pv.int8 : pk.int8;
  const long row = static_cast<long>(blockIdx.x) * kThreads + threadIdx.x;
  const long rows = static_cast<long>(p.B) * p.H * p.C;
  if (row >= rows) return;
  const int c = static_cast<int>(row % p.C);
  const long bh = row / p.C;
  const int h = static_cast<int>(bh % p.H);
  const int b = static_cast<int>(bh / p.H);
  const int slot = p.pos[b] + c;
  if (slot < 0 || slot >= p.n_max) return;

  const uint16_t* src = static_cast<const uint16_t*>(p.src) + row * p.r;
  float amax = 0.f;
  for (int j = 0; j < p.r; ++j) amax = fmaxf(amax, fabsf(__uint_as_float(uint32_t(src[j]) << 16)));
  const float s = amax / (p.int8 ? 127.0f : 448.0f);

  const int row_bytes = Q8::row(p.r);
  uint4* dst = reinterpret_cast<uint4*>(static_cast<char*>(p.dst) +
                                        ((static_cast<size_t>(b) * p.H + h) * p.n_max + slot) * row_bytes);
  const int chunks = row_bytes / 16;
  for (int k = 0; k < chunks; ++k) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 16 * k + 4 * q + e;
        v[e] = (j < p.r && s > 0.f) ? __uint_as_float(uint32_t(src[j]) << 16) / s : 0.f;
      }
      if (p.int8) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c = fminf(fmaxf(__builtin_rintf(v[e]), -127.f), 127.f);  // |v| <= 127 already
          word |= (static_cast<uint32_t>(static_cast<int32_t>(c)) & 0xffu) << (8 * e);
        }
        w[q] = word;
      } else {
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);  // bytes 0, 1
        word = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], word, true);     // bytes 2, 3
        w[q] = static_cast<uint32_t>(word);
      }
    }
    if (k == chunks - 1) w[3] = __float_as_uint(s);  // codes never reach the last word
    dst[k] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

// pk and pv: the K and V rows of one call (the same B, C, H, n_max and positions)
hipError_t launch_quantize(const QuantParams& pk, const QuantParams& pv, hipStream_t stream) {
  const long rows = static_cast<long>(pk.B) * pk.H * pk.C;
  const unsigned blocks = static_cast<unsigned>((rows + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(quantize_rows_kernel, dim3(blocks, 2), dim3(kThreads), 0, stream, pk, pv);
  return hipGetLastError();
}

}  // namespace lla
