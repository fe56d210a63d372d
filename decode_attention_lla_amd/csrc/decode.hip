// Absorbed latent decode attention (per-head LLA, and LLA-2D on the VALU path).
//
// Method: O'Neill & Reid, "Looped Latent Attention", arXiv 2607.15456. Section 3, Eq. 3 rebuilds
// loop t as k_t = W^K_t z^K + mu^K_t (column form). Section 7 ("Per-head LLA versus LLA-2D at
// inference") notes that the score is bilinear, so q . k_t = (W^K_t^T q) . z^K + q . mu^K_t, and
// that sum_i p_i W^V_t z^V_i = W^V_t sum_i p_i z^V_i. The kernels below therefore
//   1. form q~ = scale*log2(e) * W^K_t^T q and beta = scale*log2(e) * q . mu^K_t once per (b, h);
//   2. stream the bf16/fp32 latents of one (b, h, token range) from HBM, one token per LPT lanes,
//      computing base-2 scores q~ . z^K_i + beta with a per-lane online softmax;
//   3. accumulate sum_i 2^(s_i - m) z^V_i in r_v-wide fp32 registers (latent space);
//   4. merge lanes, then either write a split partial (m, l, a) or finish: merge the optional
//      self token, apply W^V_t once, add l * mu^V_t, normalise and store o and lse.
// The reconstructed K/V of cached tokens are never formed.
#include <type_traits>

#include "lla_device.h"
#include "lla_internal.h"

namespace lla {
namespace {

// Largest growth of the running maximum tolerated before rescaling (base-2 units). Weights are
// at most 2^kLazy = 256 relative to the stored maximum, which float32 sums absorb without loss of
// range; skipping most rescales keeps the branch rare.
constexpr float kLazy = 8.0f;

// First latent row of sequence `seq` (head h): per-head cache [B][H][n_max][r], 2D [B][n_max][r].
__device__ __forceinline__ size_t latent_row(const DecodeParams& p, int seq, int h) {
  return p.variant == LLA_2D ? static_cast<size_t>(seq) * p.n_max
                             : (static_cast<size_t>(seq) * p.H + h) * p.n_max;
}

// Listed slots of a gather-indexed row, clamped to [0, budget].
__device__ __forceinline__ int gather_keys(const DecodeParams& p, int row) {
  const int n = p.seq_lens != nullptr ? uniform(p.seq_lens[row]) : p.budget;
  return min(max(n, 0), p.budget);
}

// Keys visible to query row `row` (see DecodeParams), clamped to [0, n_max].
__device__ __forceinline__ int row_keys(const DecodeParams& p, int row) {
  const int seq = row / p.rows_per_seq;
  int n = p.seq_lens != nullptr ? uniform(p.seq_lens[seq]) : p.n_max;
  if (p.causal) n += row - seq * p.rows_per_seq + 1;
  return min(max(n, 0), p.n_max);
}

// Offset of mu_t restricted to head h: per-head [H][T*d] at (h, t*d); 2D [T*H*d] at t*H*d + h*d.
__device__ __forceinline__ size_t mu_offset(const DecodeParams& p, int h) {
  return p.variant == LLA_2D ? (static_cast<size_t>(p.t) * p.H + h) * p.d
                             : (static_cast<size_t>(h) * p.T + p.t) * p.d;
}

// W_t restricted to head h: per-head [T][H][d][r] at (t, h); 2D [T][H*d][r] at rows t*H*d + h*d.
// Both are element offset (t*H + h)*d*r.
__device__ __forceinline__ size_t w_offset(const DecodeParams& p, int h, int r) {
  return (static_cast<size_t>(p.t) * p.H + h) * p.d * r;
}

// Finish one (b, h): merge the latent part (M, l, a[] in LDS, base-2, relative to M) with the
// optional self token, apply W^V_t once, add mu^V_t, normalise, store. Runs on one wave.
template <class S>
__device__ void finish_unit(const DecodeParams& p, int b, int h, float M, float l,
                            const float* a_s, const float* q_s, int lane) {
  const size_t bh = static_cast<size_t>(b) * p.H + h;
  float s_self = kNegInf;
  if (p.k_self != nullptr) {
    float part = 0.f;
    for (int j = lane; j < p.d; j += 64) part += q_s[j] * ld<S>(p.k_self, bh * p.d + j);
    s_self = wave_sum(part) * p.scale_log2;
    if (p.sr_self != nullptr) s_self += p.sr_self[bh];  // the self token's rotary score
  }
  const float M2 = fmaxf(M, s_self);
  const float f_lat = (M == kNegInf) ? 0.f : fast_exp2(M - M2);
  const float p_self = (s_self == kNegInf) ? 0.f : fast_exp2(s_self - M2);
  const float den = l * f_lat + p_self;
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  const size_t woff = w_offset(p, h, p.r_v);
  const size_t moff = mu_offset(p, h);
  for (int j = lane; j < p.d; j += 64) {
    float o = 0.f;
    const size_t row = woff + static_cast<size_t>(j) * p.r_v;
    for (int r = 0; r < p.r_v; ++r) o += ld<S>(p.Wv, row + r) * a_s[r];
    if (p.mu_v != nullptr) o += l * ld<S>(p.mu_v, moff + j);
    o *= f_lat;
    if (p.v_self != nullptr) o += p_self * ld<S>(p.v_self, bh * p.d + j);
    st<S>(p.out, bh * p.d + j, o * inv);
  }
  if (p.lse != nullptr && lane == 0)
    p.lse[bh] = den > 0.f ? (M2 + fast_log2(den)) * kLn2 : kNegInf;
}

// One wave per (b, h, split). LPT lanes share a token; each holds EK = RK/LPT K elements and
// EV = RV/LPT V elements. U tiles of 64/LPT tokens are loaded before any is consumed. With G the
// split ranges over the row's slot list instead of its first N latents: each token's slot is read
// first, and a slot outside [0, n_max) counts as masked. S is the storage of q, W, mu, the self
// token and out; LS that of the latent rows (S itself, or Q8 low-bit rows read whole by one lane:
// the K row scale multiplies the score, the V row scale the token's weight). With R each token's
// score also gets its precomputed base-2 rotary score p.sr[bh][slot] (decoupled RoPE branch).
// A lane's S-byte row slice (whole words, S <= 32) of the row at byte offset row of a raw buffer,
// for lane sub of the LPT lanes that share the row. Up to 16 bytes: one load at S*sub. Longer
// slices are split: the first 16 bytes at 16*sub (into f[0]), the rest at 16*LPT + (S-16)*sub
// (into f[1]), so each of the two load instructions reads every row as one run without gaps.
template <int S, int AUX, int LPT>
__device__ __forceinline__ void load_slice(__amdgpu_buffer_rsrc_t rs, uint32_t row, int sub, uint4* f) {
  if constexpr (S <= 16) {
    f[0] = buffer_words<S / 4, AUX>(rs, row + S * sub);
  } else {
    f[0] = buffer_words<4, AUX>(rs, row + 16 * sub);
    f[1] = buffer_words<(S - 16) / 4, AUX>(rs, row + 16 * LPT + (S - 16) * sub);
  }
}
// The latent entry that element e of lane sub's slice holds (E elements per slice, E16 of them in
// the first 16 bytes; SPLIT: the slice is split as load_slice splits slices over 16 bytes).
template <bool SPLIT, int E, int E16, int LPT>
__device__ __forceinline__ int slice_entry(int sub, int e) {
  if constexpr (SPLIT) return e < E16 ? sub * E16 + e : LPT * E16 + sub * (E - E16) + (e - E16);
  return sub * E + e;
}

template <class S, class LS, int RK, int RV, int LPT, int U, bool G, bool R = false>
__global__ __launch_bounds__(64) void decode_partial_kernel(DecodeParams p) {
  constexpr bool kQ8 = std::is_same<LS, Q8>::value || std::is_same<LS, I8>::value;  // low-bit rows
  constexpr int RKB = LS::row(RK);  // bytes per latent row
  constexpr int RVB = LS::row(RV);
  // A lane's slice of a row: RK / LPT elements, or for low-bit rows RKB / LPT byte slots (codes,
  // then the row's zero padding and, in the last lane of the token's group, its float32 scale).
  constexpr int EK = kQ8 ? RKB / LPT : RK / LPT;
  constexpr int EV = kQ8 ? RVB / LPT : RV / LPT;
  constexpr int TPW = 64 / LPT;
  constexpr int SK = EK * LS::kBytes;  // bytes of a lane's slice of a K row
  constexpr int SV = EV * LS::kBytes;
  // Buffer loads of whole-word slices of at most 32 bytes (one load of up to 16 bytes, a second
  // for the rest): the LPT lanes of a token then read its row as one run, and each load
  // instruction covers 64 / LPT consecutive rows without gaps (one load per slice) or leaves only
  // the second load's bytes for the next instruction; the contiguous read streams past the caches
  // (non-temporal). Low-bit slices stay within one load.
  constexpr bool kOne = SK % 4 == 0 && SV % 4 == 0 && SK <= 32 && SV <= 32 && (!kQ8 || (SK <= 16 && SV <= 16));
  constexpr int VK = kOne ? (SK + 15) / 16 : SK / 16;
  constexpr int VV = kOne ? (SV + 15) / 16 : SV / 16;
  static_assert(kQ8 ? (EK * LPT == RKB && EV * LPT == RVB) : (EK * LPT == RK && EV * LPT == RV),
                "rows must split evenly over lanes");
  static_assert(kOne || (VK * 16 == SK && VV * 16 == SV), "16-byte fragments");
  static_assert(!kQ8 || kOne || LPT == 1, "a low-bit row is one lane's, or one load per lane");
  constexpr int E16 = 16 / LS::kBytes;                // elements in a slice's first 16 bytes
  constexpr bool kSplitK = kOne && SK > 16;          // slices read by two loads (load_slice)
  constexpr bool kSplitV = kOne && SV > 16;
  static_assert(!kQ8 || !(kSplitK || kSplitV), "low-bit slices are one load");

  __shared__ float q_s[256];
  __shared__ float qt_s[RK];
  __shared__ float a_s[RV];

  const int lane = threadIdx.x;
  const int unit = blockIdx.x;
  const int split = unit % p.splits;
  const int bh = unit / p.splits;
  const int h = bh % p.H;
  const int b = bh / p.H;

  const int nb = G ? gather_keys(p, b) : row_keys(p, b);
  const int tb = uniform(split * p.chunk);
  const int te = uniform(min(nb, tb + p.chunk));

  // One-load rows stream two register batches ahead. The gather read first stages its split's
  // slot list in LDS (when it fits), so finding a row costs an LDS read rather than a memory round
  // trip in front of every batch; longer splits take the one-batch loop below.
  static_assert(!(G && R), "the rotary scores are read for contiguous rows only");
  constexpr int kSlotCap = 2048;
  __shared__ __attribute__((aligned(16))) int32_t slot_s[G ? kSlotCap : 4];
  const int32_t* srow = G ? p.slots + static_cast<size_t>(b) * p.budget : nullptr;
  const bool piped = kOne && (!G || te - tb <= kSlotCap);
  // every 16-byte load of the list is issued here (positions past the split read as zeros) and
  // written to LDS after the query absorption below, whose own loads then overlap the list's
  const int nsl = G && kOne && piped ? (max(te - tb, 0) + 255) / 256 : 0;  // 256 positions per load
  uint4 sl[G && kOne ? kSlotCap / 256 : 1];
  if constexpr (G && kOne) {
    const __amdgpu_buffer_rsrc_t rl = buffer_rsrc(srow + tb, static_cast<uint32_t>(max(te - tb, 0)) * 4);
#pragma unroll
    for (int k = 0; k < kSlotCap / 256; ++k)
      if (k < nsl) sl[k] = buffer_words<4, 0>(rl, static_cast<uint32_t>(k * 64 + lane) * 16);
  }

  // --- 1. query absorption ------------------------------------------------------------------
  const size_t qoff = static_cast<size_t>(bh) * p.d;
  for (int j = lane; j < p.d; j += 64) q_s[j] = ld<S>(p.q, qoff + j);
  __syncthreads();
  const size_t wk = w_offset(p, h, RK);
  for (int r = lane; r < RK; r += 64) {
    float acc = 0.f;
    for (int j = 0; j < p.d; ++j) acc += ld<S>(p.Wk, wk + static_cast<size_t>(j) * RK + r) * q_s[j];
    qt_s[r] = acc * p.scale_log2;
  }
  float beta = 0.f;
  if (p.mu_k != nullptr) {
    const size_t moff = mu_offset(p, h);
    float part = 0.f;
    for (int j = lane; j < p.d; j += 64) part += q_s[j] * ld<S>(p.mu_k, moff + j);
    beta = wave_sum(part) * p.scale_log2;
  }
  if constexpr (G && kOne) {
#pragma unroll
    for (int k = 0; k < kSlotCap / 256; ++k)
      if (k < nsl) *reinterpret_cast<uint4*>(&slot_s[(k * 64 + lane) * 4]) = sl[k];
  }
  __syncthreads();  // the slot list is visible to every lane from here

  const int sub = lane % LPT;
  const int grp = lane / LPT;
  float qt[EK];
#pragma unroll
  for (int e = 0; e < EK; ++e) {
    const int c = slice_entry<kSplitK, EK, E16, LPT>(sub, e);  // low-bit slots past the codes take a zero query weight
    qt[e] = (!kQ8 || c < RK) ? qt_s[min(c, RK - 1)] : 0.f;
  }
  // low-bit slices: the bytes of each of this lane's words that hold codes (padding and the scale
  // must never be converted as codes: a scale byte can be an E4M3 NaN pattern)
  uint32_t kmask[4], vmask[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int nk = min(max(RK - (sub * EK + 4 * k), 0), 4);
    const int nv = min(max(RV - (sub * EV + 4 * k), 0), 4);
    kmask[k] = nk == 4 ? 0xffffffffu : (1u << (8 * nk)) - 1u;
    vmask[k] = nv == 4 ? 0xffffffffu : (1u << (8 * nv)) - 1u;
  }

  // --- 2-3. latent stream with online softmax -------------------------------------------------
  const size_t lrow = latent_row(p, b / p.rows_per_seq, h);
  const char* zkp = static_cast<const char*>(p.zk) + lrow * RKB + sub * SK;
  const char* zvp = static_cast<const char*>(p.zv) + lrow * RVB + sub * SV;
  // kOne: buffer descriptors over the rows this wave may read (the gather read: all n_max slots;
  // the contiguous read: its split [tb, te)); an offset at the end reads zeros
  const int row0 = G ? 0 : tb;
  const uint32_t nrows = static_cast<uint32_t>(uniform(G ? p.n_max : max(te - tb, 0)));
  const __amdgpu_buffer_rsrc_t rsk = buffer_rsrc(static_cast<const char*>(p.zk) + (lrow + row0) * RKB, nrows * RKB);
  const __amdgpu_buffer_rsrc_t rsv = buffer_rsrc(static_cast<const char*>(p.zv) + (lrow + row0) * RVB, nrows * RVB);
  // non-temporal: rows are read once. For the gather read this pays when listed slots run in
  // order (a sink + window list: 248 -> 229 us at the capacity shape); a random list of 48-byte
  // rows reads ~5% slower than with ordinary loads.
  constexpr int kAux = 2;
  constexpr bool kPipe = kOne && !G;  // the contiguous buffer-load read (always two batches ahead)
  // Rotary scores (R). With at most 4 lanes per token the pipelined path loads them once per batch:
  // lane `sub` of a group loads tile sub + LPT*k's score (one load covers 64 consecutive tokens)
  // and each tile's score is broadcast inside the group (DPP) when the tile is consumed.
  constexpr bool kSrB = kPipe && LPT <= 4;
  constexpr int NSR = kSrB ? (U + LPT - 1) / LPT : U;  // score registers per batch
  const __amdgpu_buffer_rsrc_t rss =
      buffer_rsrc(R ? p.sr + static_cast<size_t>(bh) * p.sr_stride + row0 : nullptr, R ? nrows * 4 : 0);

  float m = kNegInf;
  float l = 0.f;
  float acc[EV];
#pragma unroll
  for (int e = 0; e < EV; ++e) acc[e] = 0.f;

  // fold one batch of U tiles (ok: token inside the split and valid) into (m, l, acc)
  auto consume = [&](uint4 (&kr)[U][VK], uint4 (&vr)[U][VV], const bool (&ok)[U], const float (&srv)[NSR]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float sk = 1.f, sv = 1.f;  // low-bit row scales
      if constexpr (kQ8 && kOne) {
        // the scale is the last word of the group's last lane; a zero-padded group sum gives it
        // to every lane of the group exactly. Then the non-code bytes are cleared.
        constexpr int WK = SK / 4 - 1, WV = SV / 4 - 1;
        const uint32_t kw = WK == 0 ? kr[u][0].x : WK == 1 ? kr[u][0].y : WK == 2 ? kr[u][0].z : kr[u][0].w;
        const uint32_t vw = WV == 0 ? vr[u][0].x : WV == 1 ? vr[u][0].y : WV == 2 ? vr[u][0].z : vr[u][0].w;
        sk = group_sum<LPT>(sub == LPT - 1 ? __uint_as_float(kw) : 0.f);
        sv = group_sum<LPT>(sub == LPT - 1 ? __uint_as_float(vw) : 0.f);
        kr[u][0] = make_uint4(kr[u][0].x & kmask[0], kr[u][0].y & kmask[1], kr[u][0].z & kmask[2],
                              kr[u][0].w & kmask[3]);
        vr[u][0] = make_uint4(vr[u][0].x & vmask[0], vr[u][0].y & vmask[1], vr[u][0].z & vmask[2],
                              vr[u][0].w & vmask[3]);
      } else if constexpr (kQ8) {
        // the last 16 bytes of a low-bit row hold padding the arithmetic never reads; without
        // this the compiler narrows their load and a row takes three partial loads, not two
        asm("" : "+v"(kr[u][VK - 1].x), "+v"(kr[u][VK - 1].y), "+v"(kr[u][VK - 1].z));
        asm("" : "+v"(vr[u][VV - 1].x), "+v"(vr[u][VV - 1].y), "+v"(vr[u][VV - 1].z));
        sk = q8_row_scale(kr[u], VK);
        sv = q8_row_scale(vr[u], VV);
      }
      float sc = 0.f;
#pragma unroll
      for (int e = 0; e < EK; ++e)
        if (!kQ8 || kOne || e < RK) sc += qt[e] * frag_elem<LS>(kr[u], e);
      sc = group_sum<LPT>(sc);
      if (kQ8) sc *= sk;
      sc += beta;
      if constexpr (R) {
        if constexpr (kSrB && LPT == 2) {
          sc += u % 2 == 0 ? dpp_f32<0xa0>(srv[u / 2]) : dpp_f32<0xf5>(srv[u / 2]);  // quad_perm(0,0,2,2) / (1,1,3,3)
        } else if constexpr (kSrB && LPT == 4) {
          const float x = srv[u / 4];  // quad_perm(s,s,s,s), s = u % 4 (a constant once unrolled)
          sc += u % 4 == 0 ? dpp_f32<0x00>(x) : u % 4 == 1 ? dpp_f32<0x55>(x) : u % 4 == 2 ? dpp_f32<0xaa>(x) : dpp_f32<0xff>(x);
        } else {
          sc += srv[u];
        }
      }
      if (ok[u]) {
        if (sc > m + kLazy) {
          const float c = fast_exp2(m - sc);
          l *= c;
#pragma unroll
          for (int e = 0; e < EV; ++e) acc[e] *= c;
          m = sc;
        }
        const float pr = fast_exp2(sc - m);
        l += pr;
        const float pv = kQ8 ? pr * sv : pr;
#pragma unroll
        for (int e = 0; e < EV; ++e)
          if (!kQ8 || kOne || e < RV) acc[e] += pv * frag_elem<LS>(vr[u], e);
      }
    }
  };

  if (piped) {
   if constexpr (kOne) {
    // Two register batches in turn, the next batch's loads issued before the current one is
    // consumed, so a wave always has a batch in flight. Rows past the split (or, gathered, with
    // a slot outside the cache) read as zeros through the descriptor bound (no memory access)
    // and are masked; a batch wholly past the split costs only its masked arithmetic.
    auto issue = [&](int t0, uint4 (&kr)[U][VK], uint4 (&vr)[U][VV], float (&srv)[NSR]) {
#pragma unroll
      for (int k = 0; k < NSR; ++k) {
        if constexpr (R) {
          const int tile = kSrB ? sub + LPT * k : k;
          const int tok = t0 + tile * TPW + grp;
          const uint32_t rr = tile < U ? static_cast<uint32_t>(min(tok, te) - row0) : nrows;
          srv[k] = __uint_as_float(buffer_words<1, kAux>(rss, rr * 4).x);
        } else {
          srv[k] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int tok = t0 + u * TPW + grp;
        uint32_t rr;
        if constexpr (G) {
          const int s = tok < te ? slot_s[min(tok - tb, kSlotCap - 1)] : -1;
          rr = static_cast<unsigned>(s) < static_cast<unsigned>(p.n_max) ? static_cast<uint32_t>(s) : nrows;
        } else {
          rr = static_cast<uint32_t>(min(tok, te) - row0);
        }
        load_slice<SK, kAux, LPT>(rsk, rr * RKB, sub, kr[u]);
        load_slice<SV, kAux, LPT>(rsv, rr * RVB, sub, vr[u]);
      }
    };
    auto mask = [&](int t0, bool (&ok)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int tok = t0 + u * TPW + grp;
        ok[u] = tok < te;
        if constexpr (G)
          ok[u] = ok[u] && static_cast<unsigned>(slot_s[min(tok - tb, kSlotCap - 1)]) < static_cast<unsigned>(p.n_max);
      }
    };
    constexpr int kStep = TPW * U;
    uint4 ka[U][VK], va[U][VV], kb[U][VK], vb[U][VV];
    float sa[NSR], sb[NSR];
    bool ok[U];
    if (tb < te) issue(tb, ka, va, sa);
    for (int t0 = tb; t0 < te; t0 += 2 * kStep) {
      issue(t0 + kStep, kb, vb, sb);
      mask(t0, ok);
      consume(ka, va, ok, sa);
      // no early exit here: with one exit at the bottom the compiler's wait before the loop top
      // leaves the batch just issued in flight (an exit here made it drain every load)
      issue(t0 + 2 * kStep, ka, va, sa);
      mask(t0 + kStep, ok);
      consume(kb, vb, ok, sb);
    }
   }
  } else if constexpr (!kPipe) {  // the contiguous one-load read always takes the loop above
    for (int t0 = tb; t0 < te; t0 += TPW * U) {
      uint4 kr[U][VK];
      uint4 vr[U][VV];
      bool ok[U];
      int slot[U];
      float srv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int tok = t0 + u * TPW + grp;
        ok[u] = tok < te;
        slot[u] = tok;
        if (G) {
          slot[u] = ok[u] ? srow[tok] : 0;
          ok[u] = ok[u] && static_cast<unsigned>(slot[u]) < static_cast<unsigned>(p.n_max);
        }
        if constexpr (R && kOne) {
          srv[u] = __uint_as_float(buffer_words<1, kAux>(rss, (ok[u] ? static_cast<uint32_t>(slot[u] - row0) : nrows) * 4).x);
        } else {
          srv[u] = (R && ok[u]) ? p.sr[static_cast<size_t>(bh) * p.sr_stride + slot[u]] : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if constexpr (kOne) {
          const uint32_t rr = ok[u] ? static_cast<uint32_t>(slot[u] - row0) : nrows;
          load_slice<SK, kAux, LPT>(rsk, rr * RKB, sub, kr[u]);
          load_slice<SV, kAux, LPT>(rsv, rr * RVB, sub, vr[u]);
        } else if (ok[u]) {
          const uint4* kp = reinterpret_cast<const uint4*>(zkp + static_cast<size_t>(slot[u]) * RKB);
          const uint4* vp = reinterpret_cast<const uint4*>(zvp + static_cast<size_t>(slot[u]) * RVB);
#pragma unroll
          for (int i = 0; i < VK; ++i) kr[u][i] = kp[i];
#pragma unroll
          for (int i = 0; i < VV; ++i) vr[u][i] = vp[i];
        } else {
#pragma unroll
          for (int i = 0; i < VK; ++i) kr[u][i] = make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < VV; ++i) vr[u][i] = make_uint4(0, 0, 0, 0);
        }
      }
      consume(kr, vr, ok, srv);
    }
  }

  // --- 4. merge lanes ---------------------------------------------------------------------------
  const float M = wave_max(m);
  const float f = (m == kNegInf) ? 0.f : fast_exp2(m - M);
  l *= f;
#pragma unroll
  for (int e = 0; e < EV; ++e) acc[e] *= f;
#pragma unroll
  for (int o = LPT; o < 64; o <<= 1) {
    l += __shfl_xor(l, o, 64);
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
  }

  if (p.splits > 1) {
    float* w = p.ws + (static_cast<size_t>(bh) * p.splits + split) * (2 + RV);
    if (lane == 0) {
      w[0] = M;
      w[1] = l;
    }
    if (lane < LPT) {
#pragma unroll
      for (int e = 0; e < EV; ++e)
        if (!kQ8 || lane * EV + e < RV) w[2 + slice_entry<kSplitV, EV, E16, LPT>(lane, e)] = acc[e];
    }
    return;
  }
  if (lane < LPT) {
#pragma unroll
    for (int e = 0; e < EV; ++e)
      if (!kQ8 || lane * EV + e < RV) a_s[slice_entry<kSplitV, EV, E16, LPT>(lane, e)] = acc[e];
  }
  __syncthreads();
  finish_unit<S>(p, b, h, M, l, a_s, q_s, lane);
}

// Log-sum-exp merge of the S split partials of one (b, h), then the same finish. 256 threads:
// the split maximum and weighted sum are block reductions, each thread merges one latent entry
// across every split (loads coalesced over entries), and wave 0 runs the finish. (With one wave
// per (b, h), a long context at B = 1 -- 16 units, 256 splits -- left the merge latency-bound.)
constexpr int kCombineThreads = 256;

template <class S>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecodeParams p) {
  __shared__ float q_s[256];
  __shared__ float a_s[512];
  __shared__ float f_s[256];
  __shared__ float red[kCombineThreads / 64];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int bh = blockIdx.x;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int S_ = p.splits;  // <= 256 (valu_plan)
  const int stride = 2 + p.r_v;
  const float* w = p.ws + static_cast<size_t>(bh) * S_ * stride;

  float mloc = kNegInf;
  for (int s = tid; s < S_; s += kCombineThreads) mloc = fmaxf(mloc, w[static_cast<size_t>(s) * stride]);
  mloc = wave_max(mloc);
  if (lane == 0) red[wave] = mloc;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int i = 1; i < kCombineThreads / 64; ++i) M = fmaxf(M, red[i]);
  __syncthreads();  // red is reused below
  float lloc = 0.f;
  for (int s = tid; s < S_; s += kCombineThreads) {
    const float ms = w[static_cast<size_t>(s) * stride];
    const float fs = (ms == kNegInf) ? 0.f : fast_exp2(ms - M);
    f_s[s] = fs;
    lloc += fs * w[static_cast<size_t>(s) * stride + 1];
  }
  lloc = wave_sum(lloc);
  if (lane == 0) red[wave] = lloc;
  for (int j = tid; j < p.d; j += kCombineThreads) q_s[j] = ld<S>(p.q, static_cast<size_t>(bh) * p.d + j);
  __syncthreads();
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < kCombineThreads / 64; ++i) l += red[i];
  for (int r = tid; r < p.r_v; r += kCombineThreads) {
    float a = 0.f;
#pragma unroll 8
    for (int s = 0; s < S_; ++s) a += f_s[s] * w[static_cast<size_t>(s) * stride + 2 + r];
    a_s[r] = a;
  }
  __syncthreads();
  if (wave == 0) finish_unit<S>(p, b, h, M, l, a_s, q_s, lane);
}

using PartialFn = void (*)(DecodeParams);

template <class S, int RK, int RV, int LPT, int U>
PartialFn partial_fn() {
  return decode_partial_kernel<S, S, RK, RV, LPT, U, false>;
}
template <class S, int RK, int RV, int LPT, int U>
PartialFn gather_fn() {
  return decode_partial_kernel<S, S, RK, RV, LPT, U, true>;
}
template <class S, int RK, int RV, int LPT, int U>
PartialFn rope_fn() {
  return decode_partial_kernel<S, S, RK, RV, LPT, U, false, true>;
}
template <class LS, int RK, int RV, int LPT, int U>
PartialFn q8_fn() {
  return decode_partial_kernel<BF16, LS, RK, RV, LPT, U, false>;
}
template <class LS, int RK, int RV, int LPT, int U>
PartialFn q8_gather_fn() {
  return decode_partial_kernel<BF16, LS, RK, RV, LPT, U, true>;
}

struct Entry {
  int dtype, r_k, r_v;
  PartialFn fn;   // contiguous read
  PartialFn gfn;  // gather-indexed read
  PartialFn rfn;  // contiguous read with rotary scores (bf16 pairs only)
};

// Compiled (dtype, r_k, r_v) -> (lanes per token, tiles in flight). Lanes per token are chosen so
// that a lane's slice of a row is one load of at most 16 bytes wherever the rank allows it.
const Entry kTable[] = {
    {LLA_BF16, 8, 8, partial_fn<BF16, 8, 8, 1, 4>(), gather_fn<BF16, 8, 8, 1, 4>(),
     rope_fn<BF16, 8, 8, 1, 4>()},
    {LLA_BF16, 16, 16, partial_fn<BF16, 16, 16, 2, 4>(), gather_fn<BF16, 16, 16, 2, 4>(),
     rope_fn<BF16, 16, 16, 2, 4>()},
    {LLA_BF16, 24, 24, partial_fn<BF16, 24, 24, 4, 8>(), gather_fn<BF16, 24, 24, 4, 8>(),
     rope_fn<BF16, 24, 24, 4, 8>()},
    {LLA_BF16, 32, 32, partial_fn<BF16, 32, 32, 4, 8>(), gather_fn<BF16, 32, 32, 4, 8>(),
     rope_fn<BF16, 32, 32, 4, 8>()},
    {LLA_BF16, 64, 64, partial_fn<BF16, 64, 64, 8, 8>(), gather_fn<BF16, 64, 64, 8, 8>(),
     rope_fn<BF16, 64, 64, 8, 8>()},
    {LLA_BF16, 96, 96, partial_fn<BF16, 96, 96, 16, 8>(), gather_fn<BF16, 96, 96, 16, 8>(),
     rope_fn<BF16, 96, 96, 16, 8>()},
    {LLA_BF16, 128, 128, partial_fn<BF16, 128, 128, 16, 8>(), gather_fn<BF16, 128, 128, 16, 8>(),
     rope_fn<BF16, 128, 128, 16, 8>()},
    {LLA_BF16, 96, 160, partial_fn<BF16, 96, 160, 16, 8>(), gather_fn<BF16, 96, 160, 16, 8>(),
     rope_fn<BF16, 96, 160, 16, 8>()},
    {LLA_BF16, 256, 256, partial_fn<BF16, 256, 256, 32, 8>(), gather_fn<BF16, 256, 256, 32, 8>(),
     rope_fn<BF16, 256, 256, 32, 8>()},
    {LLA_F32, 8, 8, partial_fn<F32, 8, 8, 2, 4>(), gather_fn<F32, 8, 8, 2, 4>(), nullptr},
    {LLA_F32, 16, 16, partial_fn<F32, 16, 16, 4, 4>(), gather_fn<F32, 16, 16, 4, 4>(), nullptr},
    {LLA_F32, 24, 24, partial_fn<F32, 24, 24, 8, 4>(), gather_fn<F32, 24, 24, 8, 4>(), nullptr},
    {LLA_F32, 32, 32, partial_fn<F32, 32, 32, 8, 4>(), gather_fn<F32, 32, 32, 8, 4>(), nullptr},
    {LLA_F32, 64, 64, partial_fn<F32, 64, 64, 16, 4>(), gather_fn<F32, 64, 64, 16, 4>(), nullptr},
    {LLA_F32, 96, 96, partial_fn<F32, 96, 96, 32, 4>(), gather_fn<F32, 96, 96, 32, 4>(), nullptr},
    {LLA_F32, 128, 128, partial_fn<F32, 128, 128, 32, 4>(), gather_fn<F32, 128, 128, 32, 4>(), nullptr},
    {LLA_F32, 96, 160, partial_fn<F32, 96, 160, 8, 1>(), gather_fn<F32, 96, 160, 8, 1>(), nullptr},
    {LLA_F32, 256, 256, partial_fn<F32, 256, 256, 64, 4>(), gather_fn<F32, 256, 256, 64, 4>(), nullptr},
    {LLA_BF16_Q8, 8, 8, q8_fn<Q8, 8, 8, 1, 4>(), q8_gather_fn<Q8, 8, 8, 1, 4>(), nullptr},
    {LLA_BF16_Q8, 16, 16, q8_fn<Q8, 16, 16, 2, 4>(), q8_gather_fn<Q8, 16, 16, 2, 4>(), nullptr},
    {LLA_BF16_Q8, 24, 24, q8_fn<Q8, 24, 24, 2, 4>(), q8_gather_fn<Q8, 24, 24, 2, 4>(), nullptr},
    {LLA_BF16_Q8, 32, 32, q8_fn<Q8, 32, 32, 4, 8>(), q8_gather_fn<Q8, 32, 32, 4, 8>(), nullptr},
    {LLA_BF16_I8, 8, 8, q8_fn<I8, 8, 8, 1, 4>(), q8_gather_fn<I8, 8, 8, 1, 4>(), nullptr},
    {LLA_BF16_I8, 16, 16, q8_fn<I8, 16, 16, 2, 4>(), q8_gather_fn<I8, 16, 16, 2, 4>(), nullptr},
    {LLA_BF16_I8, 24, 24, q8_fn<I8, 24, 24, 2, 4>(), q8_gather_fn<I8, 24, 24, 2, 4>(), nullptr},
    {LLA_BF16_I8, 32, 32, q8_fn<I8, 32, 32, 4, 8>(), q8_gather_fn<I8, 32, 32, 4, 8>(), nullptr},
};

const Entry* find(int dtype, int r_k, int r_v) {
  for (const Entry& e : kTable)
    if (e.dtype == dtype && e.r_k == r_k && e.r_v == r_v) return &e;
  return nullptr;
}

}  // namespace

bool valu_supported(int variant, int dtype, int r_k, int r_v) {
  if (variant != LLA_PER_HEAD && variant != LLA_2D) return false;
  return find(dtype, r_k, r_v) != nullptr;
}

bool decode_supported(int variant, int dtype, int r_k, int r_v, int d_head) {
  return valu_supported(variant, dtype, r_k, r_v) ||
         (variant == LLA_2D && decode2d_mfma_supported(dtype, r_k, r_v, d_head));
}

bool decode_uses_mfma2d(const lla_desc& desc) {
  return desc.variant == LLA_2D && decode2d_mfma_supported(desc.dtype, desc.r_k, desc.r_v, desc.d_head);
}

void valu_plan(const lla_desc& desc, int B, int* splits, int* chunk) {
  // Few (row, head) units are split so the launch is about 2048 waves: one round for any of these
  // kernels (all fit 8 waves per CU), each wave keeping two batches of rows in flight. More waves
  // than fit at once leave a last, partly filled round that streams at a fraction of the bandwidth
  // (4096 waves at 12 per CU: 410 us for the 262k-token read). No split shorter than 256 tokens.
  const long units = static_cast<long>(B) * desc.H;
  const int target_waves = 2048;
  int s = static_cast<int>((target_waves + units - 1) / units);
  const int max_by_len = desc.n_max / 256 > 0 ? desc.n_max / 256 : 1;
  if (s > max_by_len) s = max_by_len;
  if (s > 256) s = 256;  // long contexts at small B*H: up to 256 splits fill the chip
  if (s < 1) s = 1;
  // tokens per split, a multiple of 128 so every tile but the last is full
  int c = (desc.n_max + s - 1) / s;
  c = (c + 127) / 128 * 128;
  s = (desc.n_max + c - 1) / c;
  *splits = s;
  *chunk = c;
}

void decode_plan(const lla_desc& desc, int B, int* splits, int* chunk) {
  if (decode_uses_mfma2d(desc))
    decode2d_plan(desc, B, splits, chunk);
  else
    valu_plan(desc, B, splits, chunk);
}

size_t decode_workspace_bytes(const lla_desc& desc, int B) {
  int s, c;
  decode_plan(desc, B, &s, &c);
  if (decode_uses_mfma2d(desc)) return decode2d_workspace_bytes(desc, B, s);
  return valu_workspace_bytes(desc, B, s);
}

size_t valu_workspace_bytes(const lla_desc& desc, int rows, int splits) {
  if (splits <= 1) return 0;
  return static_cast<size_t>(rows) * desc.H * splits * (2 + desc.r_v) * sizeof(float);
}

namespace {

// Streaming partial kernel (contiguous or gather-indexed), then the split combine when S > 1.
hipError_t launch_valu(const DecodeParams& p, int dtype, PartialFn fn, hipStream_t stream) {
  if (p.splits > 1 &&
      static_cast<size_t>(p.B) * p.H * p.splits * (2 + p.r_v) * sizeof(float) > p.ws_bytes)
    return hipErrorInvalidValue;  // the plan does not fit the workspace: never launch
  const unsigned units = static_cast<unsigned>(p.B) * p.H * p.splits;
  hipLaunchKernelGGL(fn, dim3(units), dim3(64), 0, stream, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.splits <= 1) return err;
  if (dtype == LLA_BF16 || dtype == LLA_BF16_Q8 || dtype == LLA_BF16_I8)
    hipLaunchKernelGGL(decode_combine_kernel<BF16>, dim3(p.B * p.H), dim3(kCombineThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_combine_kernel<F32>, dim3(p.B * p.H), dim3(kCombineThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int dtype, hipStream_t stream) {
  // LLA-2D decode rows (one query per sequence) take the MFMA path when it is compiled
  if (p.variant == LLA_2D && p.rows_per_seq == 1 && !p.causal &&
      decode2d_mfma_supported(dtype, p.r_k, p.r_v, p.d))
    return launch_decode2d(p, stream);
  const Entry* e = find(dtype, p.r_k, p.r_v);
  if (e == nullptr) return hipErrorNotSupported;
  return launch_valu(p, dtype, e->fn, stream);
}

void gather_plan(const lla_desc& desc, int B, int budget, int* splits, int* chunk) {
  lla_desc g = desc;
  g.n_max = budget;  // splits range over list positions
  valu_plan(g, B, splits, chunk);
  // at most 2048 positions per split where 256 splits allow it: such a split's slot list is staged
  // in LDS by the kernel (a longer split is read without that staging)
  if (*chunk > 2048 && *splits < 256) {
    int s = (budget + 2047) / 2048;
    if (s > 256) s = 256;
    int c = (budget + s - 1) / s;
    c = (c + 127) / 128 * 128;
    *splits = (budget + c - 1) / c;
    *chunk = c;
  }
}

size_t gather_workspace_bytes(const lla_desc& desc, int B, int budget) {
  int s, c;
  gather_plan(desc, B, budget, &s, &c);
  return valu_workspace_bytes(desc, B, s);
}

bool rope_supported(const lla_desc& desc, int d_rope) {
  const Entry* e = find(desc.dtype, desc.r_k, desc.r_v);
  return desc.dtype == LLA_BF16 && e != nullptr && e->rfn != nullptr &&
         (d_rope == 32 || d_rope == 64 || d_rope == 128) &&
         static_cast<long>(desc.H) * d_rope * 4 <= 64 * 1024;
}

namespace {
size_t align256(size_t n) { return (n + 255) / 256 * 256; }
}  // namespace

int rope_sr_stride(int n_max) { return (n_max + 3) / 4 * 4; }

size_t rope_workspace_bytes(const lla_desc& desc, int B) {
  int s, c;
  decode_plan(desc, B, &s, &c);
  // LLA-2D on MFMA: the branch is fused into the read (q~ rows widened by up to 128 entries)
  if (decode_uses_mfma2d(desc)) return decode2d_workspace_bytes(desc, B, s, 128);
  // streaming read: the rotary scores of every (row, head, slot) and of the self token first
  return align256(static_cast<size_t>(B) * desc.H * rope_sr_stride(desc.n_max) * 4) +
         align256(static_cast<size_t>(B) * desc.H * 4) + valu_workspace_bytes(desc, B, s);
}

hipError_t launch_decode_rope(const DecodeParams& p, const RopeScoreParams& rp0, int dtype,
                              hipStream_t stream) {
  const bool mfma2d = p.variant == LLA_2D && decode2d_mfma_supported(dtype, p.r_k, p.r_v, p.d);
  if (mfma2d) {  // rotary keys as extra MFMA k-steps of the read: no score pre-pass
    DecodeParams q = p;
    q.q_rope = rp0.q_rope;
    q.k_rope = rp0.k_rope;
    q.k_rope_self = rp0.k_rope_self;
    q.d_rope = rp0.d_r;
    q.rope_base = rp0.base;
    return launch_decode2d(q, stream);
  }
  const Entry* e = find(dtype, p.r_k, p.r_v);
  if (e == nullptr || e->rfn == nullptr) return hipErrorNotSupported;
  const int stride = rope_sr_stride(p.n_max);
  const size_t a = align256(static_cast<size_t>(p.B) * p.H * stride * 4);
  const size_t b = align256(static_cast<size_t>(p.B) * p.H * 4);
  if (a + b > p.ws_bytes) return hipErrorInvalidValue;
  char* base = reinterpret_cast<char*>(p.ws);
  RopeScoreParams rp = rp0;
  rp.sr = reinterpret_cast<float*>(base);
  rp.sr_self = reinterpret_cast<float*>(base + a);
  rp.sr_stride = stride;
  hipError_t err = launch_rope_scores(rp, stream);
  if (err != hipSuccess) return err;
  DecodeParams q = p;
  q.sr = rp.sr;
  q.sr_self = rp.k_rope_self != nullptr ? rp.sr_self : nullptr;
  q.sr_stride = stride;
  q.ws = reinterpret_cast<float*>(base + a + b);
  q.ws_bytes = p.ws_bytes - a - b;
  return launch_valu(q, dtype, e->rfn, stream);
}

hipError_t launch_decode_gather(const DecodeParams& p, int dtype, hipStream_t stream) {
  const Entry* e = find(dtype, p.r_k, p.r_v);
  if (e == nullptr) return hipErrorNotSupported;
  if (p.slots == nullptr || p.budget <= 0 || p.rows_per_seq != 1 || p.causal)
    return hipErrorInvalidValue;
  return launch_valu(p, dtype, e->gfn, stream);
}

}  // namespace lla
