// C ABI of the LLA latent-cache library: host-side validation, planning and dispatch.
// Declarations and the contract of every function are in include/lla.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "lla.h"
#include "lla_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Null is allowed for optional pointers; any non-null device pointer must be 16-byte aligned.
bool opt_ok(const void* p) { return p == nullptr || aligned16(p); }
bool req_ok(const void* p) { return p != nullptr && aligned16(p); }

bool desc_ok(const lla_desc* d) {
  if (d == nullptr) return false;
  if (d->variant != LLA_PER_HEAD && d->variant != LLA_2D) return false;
  if (d->dtype != LLA_F32 && d->dtype != LLA_BF16 && d->dtype != LLA_BF16_Q8 && d->dtype != LLA_BF16_I8)
    return false;
  if (d->H <= 0 || d->T <= 0 || d->r_k <= 0 || d->r_v <= 0 || d->n_max <= 0) return false;
  if (d->H > 65535) return false;  // heads index a launch dimension of at most 65535
  if (d->d_head <= 0 || d->d_head > 256 || (d->d_head % 8) != 0) return false;
  if (!(d->scale >= 0.f) || std::isinf(d->scale)) return false;
  // H * n_max rows of the wider axis stay under 2 GiB: flattened per-sequence indices and the
  // 32-bit byte offsets of the buffer loads never wrap
  const int64_t row = static_cast<int64_t>(lla_latent_row_bytes(d->dtype, d->r_k > d->r_v ? d->r_k : d->r_v));
  const int64_t per_seq = static_cast<int64_t>(d->H) * d->n_max * row;
  if (per_seq >= (int64_t(1) << 31)) return false;
  return true;
}

float scale_log2(const lla_desc* d) {
  const float s = d->scale > 0.f ? d->scale : 1.0f / std::sqrt(static_cast<float>(d->d_head));
  return s * 1.4426950408889634f;
}

lla_status from_hip(hipError_t e) {
  if (e == hipSuccess) return LLA_OK;
  if (e == hipErrorNotSupported) return LLA_ERR_UNSUPPORTED;
  if (e == hipErrorInvalidValue) return LLA_ERR_WORKSPACE;  // a launcher refused an unfitting plan
  return LLA_ERR_HIP;
}

// Argument checks shared by the two decode entry points.
lla_status decode_args_ok(const lla_desc* desc, int32_t B, int32_t t, const void* q,
                          const void* zk, const void* zv, const int32_t* lens, const void* Wk,
                          const void* Wv, const void* mu_k, const void* mu_v, const void* k_self,
                          const void* v_self, const void* out, const float* lse, const void* ws) {
  if (!desc_ok(desc) || B <= 0 || t < 0 || t >= desc->T) return LLA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(B) * desc->H >= (int64_t(1) << 31) / 64) return LLA_ERR_INVALID_ARG;
  if (!req_ok(q) || !req_ok(zk) || !req_ok(zv) || !req_ok(Wk) || !req_ok(Wv) || !req_ok(out))
    return LLA_ERR_INVALID_ARG;
  if (!opt_ok(lens) || !opt_ok(mu_k) || !opt_ok(mu_v) || !opt_ok(k_self) || !opt_ok(v_self) ||
      !opt_ok(lse) || !opt_ok(ws))
    return LLA_ERR_INVALID_ARG;
  if ((k_self == nullptr) != (v_self == nullptr)) return LLA_ERR_INVALID_ARG;
  return LLA_OK;
}

lla::DecodeParams decode_params(const lla_desc* desc, int32_t B, int32_t t, const void* q,
                                const void* zk, const void* zv, const int32_t* lens,
                                const void* Wk, const void* Wv, const void* mu_k,
                                const void* mu_v, const void* k_self, const void* v_self,
                                void* out, float* lse, void* ws, size_t ws_bytes) {
  lla::DecodeParams p{};
  p.q = q;
  p.zk = zk;
  p.zv = zv;
  p.seq_lens = lens;
  p.Wk = Wk;
  p.Wv = Wv;
  p.mu_k = mu_k;
  p.mu_v = mu_v;
  p.k_self = k_self;
  p.v_self = v_self;
  p.out = out;
  p.lse = lse;
  p.ws = static_cast<float*>(ws);
  p.B = B;
  p.H = desc->H;
  p.d = desc->d_head;
  p.T = desc->T;
  p.t = t;
  p.n_max = desc->n_max;
  p.r_k = desc->r_k;
  p.r_v = desc->r_v;
  p.rows_per_seq = 1;
  p.causal = 0;
  p.variant = desc->variant;
  p.scale_log2 = scale_log2(desc);
  p.ws_bytes = ws == nullptr ? 0 : ws_bytes;
  return p;
}


// Row counts the calls accept: B (times C for prefill) times H below 2^31 / 64. The workspace
// queries return 0 beyond them (the calls themselves refuse such sizes), which also keeps every
// product below in range.
bool rows_ok(const lla_desc* desc, int64_t rows) {
  return rows > 0 && rows * desc->H < (int64_t(1) << 31) / 64;
}

// Scratch of lla_attend_decode_noalloc: the split partials (and, on the LLA-2D MFMA read, the
// absorbed queries) of one call live here instead of a caller-given workspace. Every GPU the
// library runs on holds its own copy for the life of the process. In host code `scratch` names a
// host-side stand-in, never the device memory: kernels receive the address that
// hipGetSymbolAddress returns for the current device (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[LLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on `dev`, which must be the current device. Looked up once per
// device; no allocation happens here (the array is part of the loaded code object).
hipError_t noalloc_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255u) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int32_t lla_abi_version(void) { return LLA_ABI_VERSION; }

const char* lla_status_string(lla_status s) {
  switch (s) {
    case LLA_OK: return "ok";
    case LLA_ERR_INVALID_ARG: return "invalid argument";
    case LLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case LLA_ERR_WORKSPACE: return "workspace too small";
    case LLA_ERR_HIP: return "HIP launch error";
    case LLA_ERR_SCRATCH_LIMIT:
      return "call needs more scratch than the library's static buffer holds (LLA_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

size_t lla_latent_row_bytes(int32_t dtype, int32_t r) {
  if (r <= 0) return 0;
  switch (dtype) {
    case LLA_F32: return 4 * static_cast<size_t>(r);
    case LLA_BF16: return 2 * static_cast<size_t>(r);
    case LLA_BF16_Q8:
    case LLA_BF16_I8: return (static_cast<size_t>(r) + 4 + 15) / 16 * 16;
  }
  return 0;
}

lla_status lla_quantize_latents(const lla_desc* desc, int32_t B, int32_t C, const void* zk_src,
                                const void* zv_src, const int32_t* pos, void* zk, void* zv,
                                void* stream) {
  if (!desc_ok(desc) || (desc->dtype != LLA_BF16_Q8 && desc->dtype != LLA_BF16_I8) || B <= 0 ||
      C <= 0 || C > desc->n_max)
    return LLA_ERR_INVALID_ARG;
  if (desc->r_k > 512 || desc->r_v > 512) return LLA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(B) * C * desc->H >= (int64_t(1) << 31)) return LLA_ERR_INVALID_ARG;
  if (!req_ok(zk_src) || !req_ok(zv_src) || !req_ok(pos) || !req_ok(zk) || !req_ok(zv))
    return LLA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  lla::QuantParams p{};
  p.int8 = desc->dtype == LLA_BF16_I8;
  p.pos = pos;
  p.B = B;
  p.C = C;
  p.H = desc->variant == LLA_PER_HEAD ? desc->H : 1;
  p.n_max = desc->n_max;
  lla::QuantParams pv = p;
  p.src = zk_src;
  p.dst = zk;
  p.r = desc->r_k;
  pv.src = zv_src;
  pv.dst = zv;
  pv.r = desc->r_v;
  return from_hip(lla::launch_quantize(p, pv, s));
}

size_t lla_workspace_bytes(const lla_desc* desc, int32_t B, int32_t C) {
  if (!desc_ok(desc) || B <= 0 || C <= 0 || !rows_ok(desc, static_cast<int64_t>(B) * C)) return 0;
  const size_t pre = lla::prefill_workspace_bytes(*desc, B, C);
  if (C > 1) return pre;
  const size_t dec = lla::decode_workspace_bytes(*desc, B);  // decode and one-row prefill
  return dec > pre ? dec : pre;
}

lla_status lla_encode(const lla_desc* desc, int32_t B, int32_t C, const void* xk, const void* xv,
                      const void* Ek, const void* Ev, const void* mu_k, const void* mu_v,
                      const int32_t* pos, void* zk, void* zv, void* stream) {
  if (!desc_ok(desc) || B <= 0 || C <= 0) return LLA_ERR_INVALID_ARG;
  // the encode kernels count tokens (B * C) in 32-bit integers and launch grids from that count
  if (static_cast<int64_t>(B) * C >= (int64_t(1) << 31)) return LLA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(B) * C * desc->T * desc->H * desc->d_head >= (int64_t(1) << 40))
    return LLA_ERR_INVALID_ARG;
  if (C > desc->n_max) return LLA_ERR_INVALID_ARG;
  if (!req_ok(xk) || !req_ok(xv) || !req_ok(Ek) || !req_ok(Ev) || !req_ok(pos) || !req_ok(zk) ||
      !req_ok(zv) || !opt_ok(mu_k) || !opt_ok(mu_v))
    return LLA_ERR_INVALID_ARG;
  if (!lla::encode_supported(desc->dtype, desc->r_k) || !lla::encode_supported(desc->dtype, desc->r_v))
    return LLA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  lla::EncodeParams p{};
  p.B = B;
  p.C = C;
  p.T = desc->T;
  p.n_max = desc->n_max;
  p.pos = pos;
  if (desc->variant == LLA_PER_HEAD) {
    p.H = desc->H;
    p.d = desc->d_head;
  } else {  // LLA-2D: the (loop, head, channel) stack of one token is T runs of H*d values
    p.H = 1;
    p.d = desc->H * desc->d_head;
  }
  lla::EncodeParams pv = p;
  p.x = xk;
  p.E = Ek;
  p.mu = mu_k;
  p.z = zk;
  p.r = desc->r_k;
  pv.x = xv;
  pv.E = Ev;
  pv.mu = mu_v;
  pv.z = zv;
  pv.r = desc->r_v;
  return from_hip(lla::launch_encode_kv(p, pv, desc->dtype, s));
}


lla_status lla_attend_decode(const lla_desc* desc, int32_t B, int32_t t, const void* q,
                             const void* zk, const void* zv, const int32_t* seq_lens,
                             const void* Wk, const void* Wv, const void* mu_k, const void* mu_v,
                             const void* k_self, const void* v_self, void* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream) {
  const lla_status st = decode_args_ok(desc, B, t, q, zk, zv, seq_lens, Wk, Wv, mu_k, mu_v,
                                       k_self, v_self, out, lse, ws);
  if (st != LLA_OK) return st;
  if (!lla::decode_supported(desc->variant, desc->dtype, desc->r_k, desc->r_v, desc->d_head))
    return LLA_ERR_UNSUPPORTED;
  const size_t need = lla::decode_workspace_bytes(*desc, B);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return LLA_ERR_WORKSPACE;

  lla::DecodeParams p = decode_params(desc, B, t, q, zk, zv, seq_lens, Wk, Wv, mu_k, mu_v, k_self,
                                      v_self, out, lse, ws, ws_bytes);
  lla::decode_plan(*desc, B, &p.splits, &p.chunk, &p.wg_waves);
  return from_hip(lla::launch_decode(p, desc->dtype, static_cast<hipStream_t>(stream)));
}

lla_status lla_attend_decode_noalloc(const lla_desc* desc, int32_t B, int32_t t, const void* q,
                                     const void* zk, const void* zv, const int32_t* seq_lens,
                                     const void* Wk, const void* Wv, const void* mu_k,
                                     const void* mu_v, const void* k_self, const void* v_self,
                                     void* out, float* lse, void* stream) {
  const lla_status st = decode_args_ok(desc, B, t, q, zk, zv, seq_lens, Wk, Wv, mu_k, mu_v,
                                       k_self, v_self, out, lse, nullptr);
  if (st != LLA_OK) return st;
  if (!lla::decode_supported(desc->variant, desc->dtype, desc->r_k, desc->r_v, desc->d_head))
    return LLA_ERR_UNSUPPORTED;
  const size_t need = lla::decode_workspace_bytes(*desc, B);
  if (need > LLA_NOALLOC_SCRATCH_BYTES) return LLA_ERR_SCRATCH_LIMIT;
  // the scratch used is the one of the device the kernels run on: the stream's, which must be
  // the current device (the array's address is looked up with that device current)
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LLA_ERR_HIP;
  if (s != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return LLA_ERR_HIP;
    if (sdev != dev) return LLA_ERR_INVALID_ARG;
  }
  void* ws = nullptr;
  if (need > 0 && noalloc_scratch(dev, &ws) != hipSuccess) return LLA_ERR_HIP;
  lla::DecodeParams p = decode_params(desc, B, t, q, zk, zv, seq_lens, Wk, Wv, mu_k, mu_v, k_self,
                                      v_self, out, lse, ws, need > 0 ? LLA_NOALLOC_SCRATCH_BYTES : 0);
  lla::decode_plan(*desc, B, &p.splits, &p.chunk, &p.wg_waves);
  return from_hip(lla::launch_decode(p, desc->dtype, s));
}

lla_status lla_rope_write(const lla_desc* desc, int32_t B, int32_t C, int32_t d_rope, float base,
                          const void* k_in, const int32_t* pos, void* k_rope, void* stream) {
  if (!desc_ok(desc) || desc->dtype != LLA_BF16 || B <= 0 || C <= 0 || C > desc->n_max)
    return LLA_ERR_INVALID_ARG;
  if (d_rope <= 0 || d_rope > 256 || (d_rope % 2) != 0 || !(base >= 0.f) || std::isinf(base))
    return LLA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(B) * desc->n_max * d_rope >= (int64_t(1) << 40)) return LLA_ERR_INVALID_ARG;
  if (!req_ok(k_in) || !req_ok(pos) || !req_ok(k_rope)) return LLA_ERR_INVALID_ARG;
  lla::RopeWriteParams p{};
  p.k_in = k_in;
  p.pos = pos;
  p.k_rope = k_rope;
  p.B = B;
  p.C = C;
  p.n_max = desc->n_max;
  p.d_r = d_rope;
  p.base = base > 0.f ? base : 10000.0;
  return from_hip(lla::launch_rope_write(p, static_cast<hipStream_t>(stream)));
}

size_t lla_rope_workspace_bytes(const lla_desc* desc, int32_t B) {
  if (!desc_ok(desc) || B <= 0 || !rows_ok(desc, B)) return 0;
  return lla::rope_workspace_bytes(*desc, B);
}

lla_status lla_attend_decode_rope(const lla_desc* desc, int32_t B, int32_t t, const void* q,
                                  const void* q_rope, const void* zk, const void* zv,
                                  const void* k_rope, int32_t d_rope, float base,
                                  const int32_t* seq_lens, const void* Wk, const void* Wv,
                                  const void* mu_k, const void* mu_v, const void* k_self,
                                  const void* v_self, const void* k_rope_self, void* out,
                                  float* lse, void* ws, size_t ws_bytes, void* stream) {
  const lla_status st = decode_args_ok(desc, B, t, q, zk, zv, seq_lens, Wk, Wv, mu_k, mu_v,
                                       k_self, v_self, out, lse, ws);
  if (st != LLA_OK) return st;
  if (!req_ok(q_rope) || !req_ok(k_rope) || !opt_ok(k_rope_self)) return LLA_ERR_INVALID_ARG;
  if ((k_self == nullptr) != (k_rope_self == nullptr)) return LLA_ERR_INVALID_ARG;
  if (!(base >= 0.f) || std::isinf(base)) return LLA_ERR_INVALID_ARG;
  if (!lla::rope_supported(*desc, d_rope)) return LLA_ERR_UNSUPPORTED;
  const size_t need = lla::rope_workspace_bytes(*desc, B);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return LLA_ERR_WORKSPACE;
  lla::DecodeParams p = decode_params(desc, B, t, q, zk, zv, seq_lens, Wk, Wv, mu_k, mu_v, k_self,
                                      v_self, out, lse, ws, ws_bytes);
  // the concatenated (content, rotary) key is d_head + d_rope wide
  const float sc = desc->scale > 0.f ? desc->scale
                                     : 1.0f / std::sqrt(static_cast<float>(desc->d_head + d_rope));
  p.scale_log2 = sc * 1.4426950408889634f;
  lla::rope_plan(*desc, B, &p.splits, &p.chunk, &p.wg_waves, &p.wg_heads);
  p.q_rope = q_rope;
  p.k_rope = k_rope;
  p.k_rope_self = k_rope_self;
  p.d_rope = d_rope;
  p.rope_base = base > 0.f ? base : 10000.0;
  return from_hip(lla::launch_decode_rope(p, desc->dtype, static_cast<hipStream_t>(stream)));
}

size_t lla_reconstruct_workspace_bytes(const lla_desc* desc, int32_t B) {
  if (!desc_ok(desc) || B <= 0 || !rows_ok(desc, B)) return 0;
  return lla::reconstruct_workspace_bytes(*desc, B);
}

lla_status lla_attend_decode_reconstruct(const lla_desc* desc, int32_t B, int32_t t,
                                         const void* q, const void* zk, const void* zv,
                                         const int32_t* seq_lens, const void* Wk, const void* Wv,
                                         const void* mu_k, const void* mu_v, const void* k_self,
                                         const void* v_self, void* out, float* lse, void* ws,
                                         size_t ws_bytes, void* stream) {
  const lla_status st = decode_args_ok(desc, B, t, q, zk, zv, seq_lens, Wk, Wv, mu_k, mu_v,
                                       k_self, v_self, out, lse, ws);
  if (st != LLA_OK) return st;
  if (!lla::reconstruct_supported(*desc)) return LLA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(B) * desc->H * desc->n_max * desc->d_head >= (int64_t(1) << 40))
    return LLA_ERR_INVALID_ARG;
  const size_t need = lla::reconstruct_workspace_bytes(*desc, B);
  if (ws == nullptr || ws_bytes < need) return LLA_ERR_WORKSPACE;
  lla::DecodeParams p = decode_params(desc, B, t, q, zk, zv, seq_lens, Wk, Wv, mu_k, mu_v, k_self,
                                      v_self, out, lse, ws, ws_bytes);
  return from_hip(lla::launch_decode_reconstruct(p, *desc, static_cast<hipStream_t>(stream)));
}

size_t lla_gather_workspace_bytes(const lla_desc* desc, int32_t B, int32_t budget) {
  if (!desc_ok(desc) || B <= 0 || budget <= 0 || !rows_ok(desc, B)) return 0;
  if (static_cast<int64_t>(B) * budget >= (int64_t(1) << 31)) return 0;  // as the call
  return lla::gather_workspace_bytes(*desc, B, budget);
}

lla_status lla_attend_decode_gather(const lla_desc* desc, int32_t B, int32_t t, const void* q,
                                    const void* zk, const void* zv, const int32_t* slots,
                                    int32_t budget, const int32_t* counts, const void* Wk,
                                    const void* Wv, const void* mu_k, const void* mu_v,
                                    const void* k_self, const void* v_self, void* out, float* lse,
                                    void* ws, size_t ws_bytes, void* stream) {
  const lla_status st = decode_args_ok(desc, B, t, q, zk, zv, counts, Wk, Wv, mu_k, mu_v, k_self,
                                       v_self, out, lse, ws);
  if (st != LLA_OK) return st;
  if (!req_ok(slots) || budget <= 0) return LLA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(B) * budget >= (int64_t(1) << 31)) return LLA_ERR_INVALID_ARG;
  if (!lla::valu_supported(desc->variant, desc->dtype, desc->r_k, desc->r_v))
    return LLA_ERR_UNSUPPORTED;
  const size_t need = lla::gather_workspace_bytes(*desc, B, budget);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return LLA_ERR_WORKSPACE;

  lla::DecodeParams p = decode_params(desc, B, t, q, zk, zv, counts, Wk, Wv, mu_k, mu_v, k_self,
                                      v_self, out, lse, ws, ws_bytes);
  p.slots = slots;
  p.budget = budget;
  lla::gather_plan(*desc, B, budget, &p.splits, &p.chunk);
  return from_hip(lla::launch_decode_gather(p, desc->dtype, static_cast<hipStream_t>(stream)));
}


lla_status lla_attend_prefill(const lla_desc* desc, int32_t B, int32_t C, int32_t t,
                              const void* q, const void* zk, const void* zv,
                              const int32_t* ctx_lens, const void* Wk, const void* Wv,
                              const void* mu_k, const void* mu_v, void* out, void* ws,
                              size_t ws_bytes, void* stream) {
  if (!desc_ok(desc) || B <= 0 || C <= 0 || t < 0 || t >= desc->T) return LLA_ERR_INVALID_ARG;
  if (C > desc->n_max) return LLA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(B) * C * desc->H >= (int64_t(1) << 31) / 64) return LLA_ERR_INVALID_ARG;
  if (!req_ok(q) || !req_ok(zk) || !req_ok(zv) || !req_ok(ctx_lens) || !req_ok(Wk) ||
      !req_ok(Wv) || !req_ok(out))
    return LLA_ERR_INVALID_ARG;
  if (!opt_ok(mu_k) || !opt_ok(mu_v) || !opt_ok(ws)) return LLA_ERR_INVALID_ARG;
  if (!lla::prefill_supported(desc->variant, desc->dtype, desc->r_k, desc->r_v))
    return LLA_ERR_UNSUPPORTED;
  const size_t need = lla::prefill_workspace_bytes(*desc, B, C);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return LLA_ERR_WORKSPACE;

  lla::PrefillParams p{};
  p.q = q;
  p.zk = zk;
  p.zv = zv;
  p.ctx_lens = ctx_lens;
  p.Wk = Wk;
  p.Wv = Wv;
  p.mu_k = mu_k;
  p.mu_v = mu_v;
  p.out = out;
  p.ws = ws;
  p.B = B;
  p.C = C;
  p.H = desc->H;
  p.d = desc->d_head;
  p.T = desc->T;
  p.t = t;
  p.n_max = desc->n_max;
  p.r_k = desc->r_k;
  p.r_v = desc->r_v;
  p.variant = desc->variant;
  p.scale_log2 = scale_log2(desc);
  p.ws_bytes = ws == nullptr ? 0 : ws_bytes;
  lla::prefill_plan(*desc, B, C, &p.splits, &p.chunk, &p.wg_waves);
  return from_hip(lla::launch_prefill(p, desc->dtype, static_cast<hipStream_t>(stream)));
}

lla_status lla_attend_prefill_rope(const lla_desc* desc, int32_t B, int32_t C, int32_t t,
                                   const void* q, const void* q_rope, const void* zk,
                                   const void* zv, const void* k_rope, int32_t d_rope, float base,
                                   const int32_t* ctx_lens, const void* Wk, const void* Wv,
                                   const void* mu_k, const void* mu_v, void* out, void* ws,
                                   size_t ws_bytes, void* stream) {
  if (!desc_ok(desc) || B <= 0 || C <= 0 || t < 0 || t >= desc->T) return LLA_ERR_INVALID_ARG;
  if (C > desc->n_max) return LLA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(B) * C * desc->H >= (int64_t(1) << 31) / 64) return LLA_ERR_INVALID_ARG;
  if (!req_ok(q) || !req_ok(q_rope) || !req_ok(zk) || !req_ok(zv) || !req_ok(k_rope) ||
      !req_ok(ctx_lens) || !req_ok(Wk) || !req_ok(Wv) || !req_ok(out))
    return LLA_ERR_INVALID_ARG;
  if (!opt_ok(mu_k) || !opt_ok(mu_v) || !opt_ok(ws)) return LLA_ERR_INVALID_ARG;
  if (!(base >= 0.f) || std::isinf(base)) return LLA_ERR_INVALID_ARG;
  if (!lla::prefill_rope_supported(*desc, d_rope)) return LLA_ERR_UNSUPPORTED;
  const size_t need = lla::prefill_workspace_bytes(*desc, B, C);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return LLA_ERR_WORKSPACE;

  lla::PrefillParams p{};
  p.q = q;
  p.zk = zk;
  p.zv = zv;
  p.ctx_lens = ctx_lens;
  p.Wk = Wk;
  p.Wv = Wv;
  p.mu_k = mu_k;
  p.mu_v = mu_v;
  p.out = out;
  p.ws = ws;
  p.B = B;
  p.C = C;
  p.H = desc->H;
  p.d = desc->d_head;
  p.T = desc->T;
  p.t = t;
  p.n_max = desc->n_max;
  p.r_k = desc->r_k;
  p.r_v = desc->r_v;
  p.variant = desc->variant;
  // the concatenated (content, rotary) key is d_head + d_rope wide
  const float sc = desc->scale > 0.f ? desc->scale
                                     : 1.0f / std::sqrt(static_cast<float>(desc->d_head + d_rope));
  p.scale_log2 = sc * 1.4426950408889634f;
  p.ws_bytes = ws == nullptr ? 0 : ws_bytes;
  p.q_rope = q_rope;
  p.k_rope = k_rope;
  p.d_rope = d_rope;
  p.rope_base = base > 0.f ? base : 10000.0;
  lla::prefill_plan(*desc, B, C, &p.splits, &p.chunk, &p.wg_waves);
  return from_hip(lla::launch_prefill(p, desc->dtype, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
