// Reconstruct-then-attend comparator: rebuild loop t's K and V of every cached token, then attend.
//
// Method: O'Neill & Reid, "Looped Latent Attention", arXiv 2607.15456. Section 7 ("Per-head LLA
// versus LLA-2D at inference") measures the absorbed read against a decoder that rebuilds the
// cached tokens' K/V (Eq. 3: x_hat_t = W_t z + mu_t, column form) and then runs ordinary
// attention over them. This file is that comparator on MI355X: an MFMA kernel writes the rebuilt
// K_t and V_t of the visible tokens as bf16 rows into the workspace, and the streaming decode
// kernel then attends over them with identity factors (with W = I the absorbed read is plain
// softmax attention over explicit K/V).
#include <hip/hip_runtime.h>

#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4_t mfma16(uint4 a, uint4 b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int kTokWave = 32;               // tokens per wave: two 16-token MFMA blocks
constexpr int kWaves = 4;
constexpr int kTokWG = kTokWave * kWaves;  // tokens per workgroup
constexpr int kMaxR = 256;

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// X^T = W_t (D x r) . Z^T (r x tokens) for one (b, h) and a 128-token tile, stored as bf16 rows
// X[token][D] (+ mu_t). A operand: rows of W_t[h] (k = latent entry), staged in LDS with rows
// padded by 16 bytes so the 16 rows of a ds_read_b128 fall on distinct banks for every r that is
// a multiple of 32. B operand: each lane's 16 bytes of a latent row, straight from HBM. C: lane
// (token j, group g) holds rows 4g .. 4g+3 of X^T, i.e. 4 consecutive channels of token j.
template <int D>
__global__ __launch_bounds__(256) void reconstruct_kernel(ReconParams p) {
  __shared__ __attribute__((aligned(16))) char w_s[D * (kMaxR * 2 + 16)];
  const int r = p.r;
  const int RS = r * 2 + 16;
  const int bh = blockIdx.y;
  const int h = bh % p.H;
  const int b = bh / p.H;
  int nb = p.seq_lens != nullptr ? uniform(p.seq_lens[b]) : p.n_max;
  nb = min(max(nb, 0), p.n_max);
  const int tok0 = blockIdx.x * kTokWG;
  if (tok0 >= nb) return;  // workgroup-uniform, before any barrier

  const uint16_t* W = static_cast<const uint16_t*>(p.W) + (static_cast<size_t>(p.t) * p.H + h) * D * r;
  const int cpr = r / 8;  // 16-byte chunks per W row
  for (int idx = threadIdx.x; idx < D * cpr; idx += 256) {
    const int row = idx / cpr;
    const int c = idx - row * cpr;
    *reinterpret_cast<uint4*>(w_s + row * RS + c * 16) =
        *reinterpret_cast<const uint4*>(W + static_cast<size_t>(row) * r + c * 8);
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int wtok = tok0 + wave * kTokWave;
  const uint16_t* Z = static_cast<const uint16_t*>(p.z) + static_cast<size_t>(bh) * p.n_max * r;

  floatx4_t acc[D / 16][2];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    acc[db][0] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    acc[db][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
  for (int ks = 0; ks < r / 32; ++ks) {
    uint4 bz[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int tok = wtok + 16 * tb + col;
      bz[tb] = tok < nb ? *reinterpret_cast<const uint4*>(Z + static_cast<size_t>(tok) * r + 32 * ks + 8 * g)
                        : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const uint4 a = *reinterpret_cast<const uint4*>(w_s + (16 * db + col) * RS + (32 * ks + 8 * g) * 2);
      acc[db][0] = mfma16(a, bz[0], acc[db][0]);
      acc[db][1] = mfma16(a, bz[1], acc[db][1]);
    }
  }

  // per-head mu [H][T*d] at (h, t*d)
  const uint16_t* mu = p.mu != nullptr
                           ? static_cast<const uint16_t*>(p.mu) + (static_cast<size_t>(h) * p.T + p.t) * D
                           : nullptr;
  uint16_t* X = static_cast<uint16_t*>(p.x) + static_cast<size_t>(bh) * p.n_max * D;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int tok = wtok + 16 * tb + col;
    if (tok >= nb) continue;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = 16 * db + 4 * g + e;
        v[e] = acc[db][tb][e] + (mu != nullptr ? __uint_as_float(uint32_t(mu[ch]) << 16) : 0.f);
      }
      *reinterpret_cast<uint2*>(X + static_cast<size_t>(tok) * D + 16 * db + 4 * g) =
          make_uint2(f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3]));
    }
  }
}

// Identity factors [H][D][D] (bf16 1.0 on the diagonal) for the attention over explicit K/V.
__global__ void identity_kernel(uint16_t* w, int D) {
  const int i = blockIdx.x % D;  // row within a head; blockIdx.x = h * D + i
  for (int j = threadIdx.x; j < D; j += blockDim.x)
    w[static_cast<size_t>(blockIdx.x) * D + j] = (i == j) ? uint16_t(0x3F80) : uint16_t(0);
}

struct ReconWs {
  void* k;
  void* v;
  void* ident;
  float* partials;
  size_t partial_bytes;
};

ReconWs carve(const lla_desc& desc, int B, void* ws, size_t ws_bytes) {
  const size_t kv = align256(static_cast<size_t>(B) * desc.H * desc.n_max * desc.d_head * 2);
  const size_t id = align256(static_cast<size_t>(desc.H) * desc.d_head * desc.d_head * 2);
  char* base = static_cast<char*>(ws);
  ReconWs w{};
  w.k = base;
  w.v = base + kv;
  w.ident = base + 2 * kv;
  w.partials = reinterpret_cast<float*>(base + 2 * kv + id);
  w.partial_bytes = ws_bytes > 2 * kv + id ? ws_bytes - 2 * kv - id : 0;
  return w;
}

lla_desc attend_desc(const lla_desc& desc) {
  lla_desc a = desc;  // plain attention over explicit K/V: r = d, identity factors, one loop
  a.r_k = desc.d_head;
  a.r_v = desc.d_head;
  a.T = 1;
  return a;
}

}  // namespace

bool reconstruct_supported(const lla_desc& desc) {
  return desc.variant == LLA_PER_HEAD && desc.dtype == LLA_BF16 &&
         (desc.d_head == 64 || desc.d_head == 128) && desc.r_k % 32 == 0 && desc.r_v % 32 == 0 &&
         desc.r_k <= kMaxR && desc.r_v <= kMaxR;
}

void reconstruct_plan(const lla_desc& desc, int B, int* splits, int* chunk) {
  valu_plan(attend_desc(desc), B, splits, chunk);
}

size_t reconstruct_workspace_bytes(const lla_desc& desc, int B) {
  const size_t kv = align256(static_cast<size_t>(B) * desc.H * desc.n_max * desc.d_head * 2);
  const size_t id = align256(static_cast<size_t>(desc.H) * desc.d_head * desc.d_head * 2);
  int s, c;
  reconstruct_plan(desc, B, &s, &c);
  return 2 * kv + id + valu_workspace_bytes(attend_desc(desc), B, s);
}

hipError_t launch_decode_reconstruct(const DecodeParams& p, const lla_desc& desc, hipStream_t stream) {
  if (!reconstruct_supported(desc)) return hipErrorNotSupported;
  if (reconstruct_workspace_bytes(desc, p.B) > p.ws_bytes) return hipErrorInvalidValue;
  const ReconWs w = carve(desc, p.B, p.ws, p.ws_bytes);
  const int D = p.d;
  const dim3 grid((p.n_max + kTokWG - 1) / kTokWG, p.B * p.H);
  ReconParams rp{};
  rp.seq_lens = p.seq_lens;
  rp.H = p.H;
  rp.T = p.T;
  rp.t = p.t;
  rp.n_max = p.n_max;
  for (int axis = 0; axis < 2; ++axis) {
    rp.z = axis == 0 ? p.zk : p.zv;
    rp.W = axis == 0 ? p.Wk : p.Wv;
    rp.mu = axis == 0 ? p.mu_k : p.mu_v;
    rp.x = axis == 0 ? w.k : w.v;
    rp.r = axis == 0 ? p.r_k : p.r_v;
    if (D == 128)
      hipLaunchKernelGGL(reconstruct_kernel<128>, grid, dim3(256), 0, stream, rp);
    else
      hipLaunchKernelGGL(reconstruct_kernel<64>, grid, dim3(256), 0, stream, rp);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(identity_kernel, dim3(p.H * D), dim3(64), 0, stream,
                     static_cast<uint16_t*>(w.ident), D);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  DecodeParams a = p;
  a.zk = w.k;
  a.zv = w.v;
  a.Wk = w.ident;
  a.Wv = w.ident;
  a.mu_k = nullptr;
  a.mu_v = nullptr;
  a.r_k = D;
  a.r_v = D;
  a.T = 1;
  a.t = 0;
  a.ws = w.partials;
  a.ws_bytes = w.partial_bytes;
  reconstruct_plan(desc, p.B, &a.splits, &a.chunk);
  return launch_decode(a, LLA_BF16, stream);
}

}  // namespace lla
