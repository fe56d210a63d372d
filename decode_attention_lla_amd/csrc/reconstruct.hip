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

#include <algorithm>
#include <utility>

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
constexpr int kTokWG = kTokWave * kWaves;  // tokens per tile
constexpr int kMaxR = 256;
constexpr int kTargetWG = 3072;            // about four rounds of three workgroups per CU

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// X^T = W_t (D x R) . Z^T (R x tokens) for one (b, h), stored as bf16 rows X[token][D] (+ mu_t).
// A workgroup (one-dimensional grid: (b * H + h) * slots + slot) stages W_t[h] in LDS once and
// then walks 128-token tiles (tile = slot, slot + slots, ...), so the factor is read once per
// workgroup rather than per tile; neighbouring workgroups take neighbouring tiles of one head.
// A operand: rows of W_t[h] (k = latent entry) from LDS, rows padded by 16 bytes so the 16 rows of
// a ds_read_b128 fall on distinct banks (R is a multiple of 32). B operand: each lane's 16 bytes
// of a latent row, all R/32 k-steps issued before the first product, through a buffer descriptor
// that ends at the sequence's last token (rows past it read zeros). C: lane (token j, group g)
// holds channels 16*db + 4g .. +3 of token j; a row swap between lane groups g and g^1 of two
// neighbouring blocks turns that into 8 consecutive channels, one 16-byte store per lane. The rows
// are written non-temporally: the attention reads them back only after every row is written.
template <int D, int R>
__global__ __launch_bounds__(256, 3) void reconstruct_kernel(ReconParams p, int slots) {
  constexpr int KS = R / 32;
  constexpr int RS = R * 2 + 16;
  __shared__ __attribute__((aligned(16))) char w_s[D * RS];
  const int bh = blockIdx.x / slots;
  const int slot = blockIdx.x - bh * slots;
  const int h = bh % p.H;
  const int b = bh / p.H;
  int nb = p.seq_lens != nullptr ? uniform(p.seq_lens[b]) : p.n_max;
  nb = min(max(nb, 0), p.n_max);
  const int ntiles = (nb + kTokWG - 1) / kTokWG;
  if (slot >= ntiles) return;  // workgroup-uniform, before any barrier

  const uint16_t* W = static_cast<const uint16_t*>(p.W) + (static_cast<size_t>(p.t) * p.H + h) * D * R;
  constexpr int cpr = R / 8;  // 16-byte chunks per W row
  for (int idx = threadIdx.x; idx < D * cpr; idx += 256) {
    const int row = idx / cpr;
    const int c = idx - row * cpr;
    *reinterpret_cast<uint4*>(w_s + row * RS + c * 16) =
        *reinterpret_cast<const uint4*>(W + static_cast<size_t>(row) * R + c * 8);
  }

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int g = lane >> 4;
  // per-head mu [H][T*d] at (h, t*d): this lane's channels 16*db + 4g .. +3 as bf16 pairs
  uint2 mu_r[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
    mu_r[db] = p.mu != nullptr
                   ? *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.mu) +
                                                     (static_cast<size_t>(h) * p.T + p.t) * D + 16 * db + 4 * g)
                   : make_uint2(0u, 0u);
  const __amdgpu_buffer_rsrc_t zr =
      buffer_rsrc(static_cast<const uint16_t*>(p.z) + static_cast<size_t>(bh) * p.n_max * R,
                  static_cast<uint32_t>(nb) * R * 2);
  uint16_t* X = static_cast<uint16_t*>(p.x) + static_cast<size_t>(bh) * p.n_max * D;
  __syncthreads();

  for (int tile = slot; tile < ntiles; tile += slots) {
    const int wtok = tile * kTokWG + wave * kTokWave;
    uint4 bz[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        bz[ks][tb] = buffer_words<4, 0>(
            zr, static_cast<uint32_t>((wtok + 16 * tb + col) * R + 32 * ks + 8 * g) * 2u);
    floatx4_t acc[D / 16][2];
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      acc[db][0] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      acc[db][1] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const uint4 a = *reinterpret_cast<const uint4*>(w_s + (16 * db + col) * RS + (32 * ks + 8 * g) * 2);
        acc[db][0] = mfma16(a, bz[ks][0], acc[db][0]);
        acc[db][1] = mfma16(a, bz[ks][1], acc[db][1]);
      }
    }
    // issue order: every latent load, then the W fragments two ahead of the products using them
    // (left to itself the scheduler reads all fragments first, and the registers spill)
    __builtin_amdgcn_sched_group_barrier(0x020, 2 * KS, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < KS * (D / 16) - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int tok = wtok + 16 * tb + col;
#pragma unroll
      for (int dp = 0; dp < D / 32; ++dp) {
        uint32_t w[2][2];  // [block 2dp, 2dp+1][channel pair]
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const floatx4_t& a = acc[2 * dp + k][tb];
          const uint2 m = mu_r[2 * dp + k];
          w[k][0] = f32x2_to_bf16x2(a[0] + bf16_lo(m.x), a[1] + bf16_hi(m.x));
          w[k][1] = f32x2_to_bf16x2(a[2] + bf16_lo(m.y), a[3] + bf16_hi(m.y));
        }
        // lane groups 1 and 3 trade their block-2dp words for groups 0 and 2's block-2dp+1 words
        const auto s0 = __builtin_amdgcn_permlane16_swap(w[0][0], w[1][0], false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(w[0][1], w[1][1], false, false);
        const int ch = 32 * dp + 16 * (g & 1) + 8 * (g >> 1);
        if (tok < nb)
          __builtin_nontemporal_store(u32x4_t{s0[0], s1[0], s0[1], s1[1]},
                                      reinterpret_cast<u32x4_t*>(X + static_cast<size_t>(tok) * D + ch));
      }
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

typedef void (*ReconFn)(ReconParams, int);

template <int D, int... Rs>
ReconFn recon_pick(int r, std::integer_sequence<int, Rs...>) {
  ReconFn f = nullptr;
  ((r == 32 * (Rs + 1) ? (f = reconstruct_kernel<D, 32 * (Rs + 1)>, 0) : 0), ...);
  return f;
}

// ranks 32, 64, ..., 256 for d_head 64 and 128
ReconFn recon_fn(int D, int r) {
  constexpr auto ranks = std::make_integer_sequence<int, kMaxR / 32>{};
  return D == 128 ? recon_pick<128>(r, ranks) : D == 64 ? recon_pick<64>(r, ranks) : nullptr;
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

void reconstruct_plan(const lla_desc& desc, int B, int* splits, int* chunk, int* wg_waves) {
  valu_plan(attend_desc(desc), B, splits, chunk, wg_waves);
}

size_t reconstruct_workspace_bytes(const lla_desc& desc, int B) {
  const size_t kv = align256(static_cast<size_t>(B) * desc.H * desc.n_max * desc.d_head * 2);
  const size_t id = align256(static_cast<size_t>(desc.H) * desc.d_head * desc.d_head * 2);
  int s, c, nw;
  reconstruct_plan(desc, B, &s, &c, &nw);  // the plan the call runs
  return 2 * kv + id + valu_workspace_bytes(attend_desc(desc), B, s);
}

hipError_t launch_decode_reconstruct(const DecodeParams& p, const lla_desc& desc, hipStream_t stream) {
  if (!reconstruct_supported(desc)) return hipErrorNotSupported;
  if (reconstruct_workspace_bytes(desc, p.B) > p.ws_bytes) return hipErrorInvalidValue;
  const ReconWs w = carve(desc, p.B, p.ws, p.ws_bytes);
  const int D = p.d;
  const int tiles = (p.n_max + kTokWG - 1) / kTokWG;
  const int per_seq = (kTargetWG + p.B * p.H - 1) / (p.B * p.H);
  const int slots = std::max(1, std::min(tiles, per_seq));
  const dim3 grid(static_cast<unsigned>(p.B * p.H * slots));
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
    const auto fn = recon_fn(D, rp.r);
    if (fn == nullptr) return hipErrorNotSupported;
    hipLaunchKernelGGL(fn, grid, dim3(256), 0, stream, rp, slots);
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
  reconstruct_plan(desc, p.B, &a.splits, &a.chunk, &a.wg_waves);
  return launch_decode(a, LLA_BF16, stream);
}

}  // namespace lla
