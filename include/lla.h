/*
 * lla.h - C ABI of the MI355X (gfx950) Looped Latent Attention (LLA) latent-cache library.
 *
 * Method: O'Neill & Reid, "Looped Latent Attention: Cross-Loop KV Compression for Looped
 * Transformers" (arXiv 2607.15456). A looped (weight-tied) transformer writes T per-loop K/V
 * vectors per token, layer and head. LLA stores one low-rank latent per (token, head, axis)
 * instead, encoded once the token's last loop has run (Section 3, Eqs. 1-2), and rebuilds the
 * loop-t K/V only when attention reads them (Eq. 3). This library performs that read in absorbed
 * form (Section 7, "Per-head LLA versus LLA-2D at inference"): the K up-projection is moved to the
 * query, and the V up-projection is applied once to the probability-weighted sum of latents.
 *
 * Conventions shared by every entry point
 *   - Column-vector form of the paper's row form: E = W_down^T with shape [r][T*d_head], and
 *     W_t = W_up,t with shape [d_head][r]. So z = E (x - mu) and x_hat_t = W_t z + mu_t.
 *   - Loops are numbered t = 0 .. T-1 (the paper counts 1 .. T).
 *   - Every array is dense, row-major and innermost-last, as written next to each argument.
 *   - Storage dtype: desc->dtype (LLA_F32 or LLA_BF16) applies to every floating-point array
 *     argument except `lse`, which is always float32. LLA_BF16_Q8 and LLA_BF16_I8 mean bf16 for
 *     every array except the latent cache (zk, zv), whose rows are low-bit (see
 *     lla_latent_row_bytes). Accumulation is always float32. Stored
 *     results are rounded to nearest-even once.
 *   - Pointers marked [device] are HIP device addresses (or managed memory). Device pointers must
 *     be 16-byte aligned. Pointers marked [host] are ordinary host memory.
 *   - Ownership: the caller allocates and frees every buffer, including the workspace. The
 *     library keeps no state between calls, allocates nothing, and never synchronises. Functions
 *     are re-entrant.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the default stream). All work is
 *     enqueued on it in order. Calls return as soon as the work is enqueued.
 *   - Errors: arguments are checked on the host before anything is enqueued. A failed check
 *     returns a non-zero status and enqueues nothing. A failed kernel launch returns
 *     LLA_ERR_HIP. Faults inside kernels surface at the caller's next synchronisation (HIP
 *     semantics). Device-resident integer arrays (seq_lens, pos, ctx_lens) cannot be checked on
 *     the host; their handling is stated per function and never reads or writes outside the
 *     buffers described by desc.
 */
#ifndef LLA_H_
#define LLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LLA_ABI_VERSION 2

typedef enum {
  LLA_OK = 0,
  LLA_ERR_INVALID_ARG = 1, /* a null required pointer, bad size, t >= T, misaligned pointer */
  LLA_ERR_UNSUPPORTED = 2, /* a (variant, dtype, d_head, r_k, r_v) combination not compiled in */
  LLA_ERR_WORKSPACE = 3,   /* ws_bytes smaller than lla_workspace_bytes() */
  LLA_ERR_HIP = 4,         /* the HIP runtime refused a launch */
  LLA_ERR_SCRATCH_LIMIT = 5 /* lla_attend_decode_noalloc: the call needs more than
                               LLA_NOALLOC_SCRATCH_BYTES of scratch */
} lla_status;

/* Size of the library's static per-device scratch buffer (lla_attend_decode_noalloc). */
#define LLA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* LLA_BF16_Q8: the precision axis stacked on the loop axis (Section 8, "Compositionality";
 * Appendix C evaluates an 8-bit codec). Each cached latent row of r values is stored as r OCP FP8
 * E4M3 codes followed by one float32 scale: s = max|z| / 448 and code_j = e4m3(z_j / s), both
 * divisions in float32 and rounded to nearest even (a zero row has s = 0 and zero codes). The
 * row is padded to a multiple of 16 bytes: codes at bytes [0, r), zeros, s in the last 4 bytes.
 * Rows are written by lla_quantize_latents and read by lla_attend_decode, lla_attend_decode_gather
 * and lla_attend_prefill on the streaming kernels, and by the LLA-2D MFMA decode (codes converted to
 * bf16 exactly on the way to the MFMA, the K scale applied to each score, the V scale to each
 * weight; no rotary branch with low-bit rows); lla_encode returns LLA_ERR_UNSUPPORTED for
 * it (encode with a bf16 descriptor, then quantise).
 *
 * LLA_BF16_I8: the same rows with symmetric integer codes (the pages' 8-bit codec is not specified
 * further; both common 8-bit forms are offered): s = max|z| / 127 and code_j = round(z_j / s) with
 * halves to even, a two's-complement int8 in [-127, 127], both divisions in float32; same layout
 * (codes at bytes [0, r), zeros, s in the last 4 bytes of a 16-byte-aligned row). Uniform steps
 * of s across the row instead of E4M3's 3-bit mantissa: finer near the row maximum, coarser near
 * zero. */
typedef enum { LLA_F32 = 0, LLA_BF16 = 1, LLA_BF16_Q8 = 2, LLA_BF16_I8 = 3 } lla_dtype;

/* LLA_PER_HEAD: one latent per (token, head, axis); Section 3, Eqs. 2-3.
 * LLA_2D:       one latent per (token, axis) that rebuilds every head; Section 3, "The LLA-2D
 *               variant". Its encoder input is the whole T*H*d_head stack, ordered (loop, head,
 *               channel), so loop t's W^K_t is one [H*d_head][r_k] block whose rows h*d_head ..
 *               (h+1)*d_head-1 rebuild head h. */
typedef enum { LLA_PER_HEAD = 0, LLA_2D = 1 } lla_variant;

typedef struct {
  int32_t variant; /* lla_variant */
  int32_t dtype;   /* lla_dtype */
  int32_t H;       /* heads, 1 .. 65535 */
  int32_t d_head;  /* channels per head, multiple of 8, <= 256 */
  int32_t T;       /* loops (recurrence steps) */
  int32_t r_k;     /* K latent rank */
  int32_t r_v;     /* V latent rank (the paper uses r_v > r_k; any compiled pair is allowed) */
  int32_t n_max;   /* latent slots per sequence in the cache; H * n_max rows of the wider axis
                      (lla_latent_row_bytes each) must stay under 2 GiB */
  float scale;     /* softmax scale; 0 means 1/sqrt(d_head) */
} lla_desc;

/* Bytes of one cached latent row of r values for a storage dtype: 4r (LLA_F32), 2r (LLA_BF16),
 * r + 4 rounded up to a multiple of 16 (LLA_BF16_Q8, LLA_BF16_I8). 0 for an unknown dtype or
 * r <= 0. The cache
 * is [B][H][n_max][row] per head and [B][n_max][row] for LLA-2D, rows of this many bytes. */
size_t lla_latent_row_bytes(int32_t dtype, int32_t r);

/* Write C latent rows per sequence (and head) into a low-bit cache (desc->dtype == LLA_BF16_Q8 or
 * LLA_BF16_I8), quantising each row as described at that dtype.
 *
 *   zk_src, zv_src [device] bf16 rows: per-head [B][H][C][r], 2D [B][C][r] (for instance the
 *                  output of lla_encode with a bf16 descriptor, n_max = C and pos = 0).
 *   pos     [device] int32 [B]: row c of sequence b goes to slot pos[b] + c; a slot outside
 *           [0, n_max) is not written (no fault).
 *   zk, zv  [device] the low-bit caches. Only the C slots per sequence (and head) are written.
 * Any r_k, r_v in 1 .. 512. */
lla_status lla_quantize_latents(const lla_desc* desc, int32_t B, int32_t C, const void* zk_src,
                                const void* zv_src, const int32_t* pos, void* zk, void* zv,
                                void* stream);

/* Compiled (r_k, r_v) pairs.
 *   Streaming (VALU) kernels, every variant and storage type:
 *       (8,8) (16,16) (24,24) (32,32) (64,64) (96,96) (128,128) (96,160) (256,256)
 *   LLA-2D decode, bf16, d_head <= 128, on MFMA:              (64,64) (128,128) (256,256)
 *   Chunked prefill, bf16, d_head a multiple of 32, on MFMA:  (64,64) (128,128) (256,256)
 *                                                              (64,128) (128,256)
 *   Encode: any r <= 512 (bf16 on MFMA, fp32 on the VALU).
 *   Low-bit latents (LLA_BF16_Q8, LLA_BF16_I8), decode, gather decode and prefill, both
 *   variants on the streaming kernels:                        (8,8) (16,16) (24,24) (32,32)
 *                                                              (96,96)
 *   Low-bit LLA-2D decode on MFMA, d_head <= 128:              (64,64) (128,128) (256,256)
 * A decode or prefill call with a pair that none of these covers returns LLA_ERR_UNSUPPORTED. */

/* Bytes of device workspace that lla_attend_prefill with a chunk of C rows needs for this
 * descriptor and batch; with C == 1 the larger of that and what lla_attend_decode needs, so one
 * size serves a decode call and a one-row prefill chunk. May be 0. Returns 0 as well for an
 * invalid descriptor (the call itself then reports the error). */
size_t lla_workspace_bytes(const lla_desc* desc, int32_t B, int32_t C);

/* Encode C finished tokens per sequence into the latent cache (Section 3, Eq. 2, applied after
 * loop T; Eq. 1 fixes the loop-major stack x = [x_1; ...; x_T]).
 *
 *   xk, xv  [device] [B][C][T][H][d_head]  per-loop K and V of the tokens being written.
 *   Ek, Ev  [device] per-head [H][r][T*d_head]; 2D [r][T*H*d_head] (stack order loop, head,
 *                    channel).
 *   mu_k, mu_v [device] per-head [H][T*d_head]; 2D [T*H*d_head]; either may be NULL (mu = 0).
 *   pos     [device] int32 [B]: token c of sequence b is written to slot pos[b] + c.
 *   zk, zv  [device] the cache: per-head [B][H][n_max][r]; 2D [B][n_max][r]. Only the C slots
 *                    per sequence (and head) are written.
 * z = E (x - mu) is accumulated in float32 and rounded once to the storage dtype. A slot
 * pos[b] + c outside [0, n_max) is not written (no fault). */
lla_status lla_encode(const lla_desc* desc, int32_t B, int32_t C,
                      const void* xk, const void* xv, const void* Ek, const void* Ev,
                      const void* mu_k, const void* mu_v, const int32_t* pos,
                      void* zk, void* zv, void* stream);

/* Decode-time attention of one new token per sequence at loop t over the latent cache.
 *
 * Mathematically, for each (b, h): rebuild k_i = W^K_t z^K_i + mu^K_t and v_i = W^V_t z^V_i +
 * mu^V_t for the cached tokens i < N_b (Eq. 3), append the token's own uncompressed loop-t
 * (k_self, v_self) if given, and return softmax(scale * K q) V and its log-sum-exp. It is
 * computed in absorbed form (Section 7): q~ = W^K_t^T q and beta = q . mu^K_t once per (b, h);
 * scores scale * (q~ . z^K_i + beta) streamed over the latents with an online softmax; the weights
 * applied to z^V in latent space; one W^V_t projection at the end, with mu^V_t entering through
 * the total latent weight. The K/V of cached tokens are never formed.
 *
 *   t        loop index, 0 <= t < T.
 *   q        [device] [B][H][d_head].
 *   zk, zv   [device] cache as in lla_encode.
 *   seq_lens [device] int32 [B] or NULL (all n_max). N_b is clamped to [0, n_max].
 *   Wk, Wv   [device] per-head [T][H][d_head][r]; 2D [T][H*d_head][r].
 *   mu_k, mu_v [device] as in lla_encode, or NULL.
 *   k_self, v_self [device] [B][H][d_head], both given or both NULL.
 *   out      [device] [B][H][d_head].
 *   lse      [device] float32 [B][H] (natural log) or NULL.
 *   ws       [device] workspace of at least lla_workspace_bytes(desc, B, 1) bytes (NULL if 0).
 * An empty key set (N_b = 0 and no self token) gives out = 0 and lse = -inf. */
lla_status lla_attend_decode(const lla_desc* desc, int32_t B, int32_t t, const void* q,
                             const void* zk, const void* zv, const int32_t* seq_lens,
                             const void* Wk, const void* Wv, const void* mu_k, const void* mu_v,
                             const void* k_self, const void* v_self, void* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream);

/* lla_attend_decode for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments (minus ws, ws_bytes), same
 * arithmetic and same kernels as lla_attend_decode, so the results are identical to a
 * lla_attend_decode call with a fresh workspace. The split partials (and the LLA-2D MFMA read's
 * absorbed queries) go to a static device array of LLA_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends; nothing is allocated or freed, by this
 * call or any routine it calls.
 *   - A call whose plan needs more than LLA_NOALLOC_SCRATCH_BYTES returns LLA_ERR_SCRATCH_LIMIT and
 *     enqueues nothing; what a plan needs is at most lla_workspace_bytes(desc, B, 1).
 *   - The scratch of a GPU is shared by every call on it and keeps the last call's contents. Calls
 *     that may overlap on one GPU (different streams without ordering, other host threads) race on
 *     it and give wrong results; serialise them (one stream, or events).
 *   - `stream` must belong to the current device (NULL: the current device's default stream);
 *     otherwise LLA_ERR_INVALID_ARG. */
lla_status lla_attend_decode_noalloc(const lla_desc* desc, int32_t B, int32_t t, const void* q,
                                     const void* zk, const void* zv, const int32_t* seq_lens,
                                     const void* Wk, const void* Wv, const void* mu_k,
                                     const void* mu_v, const void* k_self, const void* v_self,
                                     void* out, float* lse, void* stream);

/* Decoupled rotary branch (Section 7, "Per-head LLA versus LLA-2D at inference": RoPE cannot be
 * absorbed, so the latent path carries the NoPE content and a small explicit rotary branch, shared
 * across recurrence steps for a token, carries position, MLA-style). One rotary key of width d_rope
 * is cached per token, shared by every head and loop: k_rope [device] bf16 [B][n_max][d_rope],
 * stored already rotated at its slot position. Rotation (Su et al., 2021, RoFormer): channel
 * pairs (2i, 2i+1) at position p turn by p * base^(-2i/d_rope), evaluated in float64; base 0
 * means 10000. Positions are slot indices.
 *
 * lla_rope_write: rotate and store C rotary keys per sequence, k_in [device] bf16 [B][C][d_rope],
 * row c of sequence b at slot pos[b] + c (a slot outside [0, n_max) is not written). desc->dtype
 * must be LLA_BF16; d_rope even, <= 256. */
lla_status lla_rope_write(const lla_desc* desc, int32_t B, int32_t C, int32_t d_rope, float base,
                          const void* k_in, const int32_t* pos, void* k_rope, void* stream);

/* Bytes of device workspace that lla_attend_decode_rope needs: the split partials of its plan (and
 * on the LLA-2D MFMA read the absorbed queries). May be 0 (then ws may be NULL); 0 as well for an
 * invalid descriptor. */
size_t lla_rope_workspace_bytes(const lla_desc* desc, int32_t B);

/* lla_attend_decode with the rotary branch: key i of row b is [k_i ; k_rope[b][i]] (k_i rebuilt
 * content key, Eq. 3, absorbed as in lla_attend_decode), the query is [q ; rope(q_rope, N_b)] (the
 * decoding token sits at position N_b), the optional self key is [k_self ; rope(k_rope_self, N_b)],
 * values are the content values. The scale defaults (desc->scale == 0) to 1/sqrt(d_head + d_rope),
 * the width of the concatenated key.
 *   q_rope [device] bf16 [B][H][d_rope], unrotated; k_rope_self [device] bf16 [B][d_rope], given
 *   exactly when k_self is; ws at least lla_rope_workspace_bytes(desc, B) bytes (NULL if 0).
 * The rotary scores are formed inside the read: each token's rotary key is read beside its latent
 * rows and dotted with the head's rotated rotary query (LLA-2D on MFMA: extra contraction steps of
 * the read). All heads of a sequence read the same rotary keys: on the streaming read, workgroups
 * of 8 heads load each rotary row once and share it (when H >= 8 groups well), and when B is a
 * multiple of 8 a sequence's workgroups run on one XCD, so the keys come from HBM about once per
 * sequence.
 * LLA_BF16, d_rope 32, 64 or 128, the streaming bf16 (r_k, r_v) pairs (both variants) or the
 * LLA-2D MFMA pairs; otherwise LLA_ERR_UNSUPPORTED. */
lla_status lla_attend_decode_rope(const lla_desc* desc, int32_t B, int32_t t, const void* q,
                                  const void* q_rope, const void* zk, const void* zv,
                                  const void* k_rope, int32_t d_rope, float base,
                                  const int32_t* seq_lens, const void* Wk, const void* Wv,
                                  const void* mu_k, const void* mu_v, const void* k_self,
                                  const void* v_self, const void* k_rope_self, void* out,
                                  float* lse, void* ws, size_t ws_bytes, void* stream);

/* lla_attend_prefill with the rotary branch: row j of sequence b sits at position ctx_lens[b] + j
 * and attends latents 0 .. ctx_lens[b] + j, key i being [k_i ; k_rope[b][i]] and the row's query
 * [q ; rope(q_rope, ctx_lens[b] + j)]; the chunk's rotary keys must already be in k_rope (written
 * by lla_rope_write at slots ctx_lens[b] .. + C - 1, like its latents by lla_encode). Scale as in
 * lla_attend_decode_rope (default 1/sqrt(d_head + d_rope)).
 *   q_rope [device] bf16 [B][C][H][d_rope], unrotated; k_rope as above; ws at least
 *   lla_workspace_bytes(desc, B, C).
 * LLA_BF16 only. The chunked-prefill MFMA (r_k, r_v) pairs (d_head a multiple of 32) take d_rope 64
 * or 128 on the MFMA path; the other streaming bf16 pairs (both variants) take d_rope 32, 64 or 128
 * on the streaming path (each chunk row a query with its own key count and position, the rotary
 * scores formed in the read); otherwise LLA_ERR_UNSUPPORTED. */
lla_status lla_attend_prefill_rope(const lla_desc* desc, int32_t B, int32_t C, int32_t t,
                                   const void* q, const void* q_rope, const void* zk,
                                   const void* zv, const void* k_rope, int32_t d_rope, float base,
                                   const int32_t* ctx_lens, const void* Wk, const void* Wv,
                                   const void* mu_k, const void* mu_v, void* out, void* ws,
                                   size_t ws_bytes, void* stream);

/* Bytes of device workspace that lla_attend_decode_reconstruct needs for B sequences: the rebuilt
 * K and V of every slot ([B][H][n_max][d_head] bf16 each), identity factors and split partials.
 * 0 for an invalid descriptor. */
size_t lla_reconstruct_workspace_bytes(const lla_desc* desc, int32_t B);

/* Reconstruct-then-attend comparator of lla_attend_decode (Section 7, "Per-head LLA versus LLA-2D
 * at inference": the absorbed read is measured against this decoder). It rebuilds loop t's
 * k_i = W^K_t z^K_i + mu^K_t and v_i = W^V_t z^V_i + mu^V_t (Eq. 3) of every visible cached token
 * into the workspace as bf16 rows, then runs plain softmax attention over them (plus the optional
 * self token). Same arguments and result as lla_attend_decode up to rounding (the rebuilt K/V are
 * rounded to bf16 once). Per-head LLA, bf16 storage, d_head 64 or 128, r_k and r_v multiples of 32
 * up to 256; otherwise LLA_ERR_UNSUPPORTED. ws: at least lla_reconstruct_workspace_bytes(desc, B). */
lla_status lla_attend_decode_reconstruct(const lla_desc* desc, int32_t B, int32_t t,
                                         const void* q, const void* zk, const void* zv,
                                         const int32_t* seq_lens, const void* Wk, const void* Wv,
                                         const void* mu_k, const void* mu_v, const void* k_self,
                                         const void* v_self, void* out, float* lse, void* ws,
                                         size_t ws_bytes, void* stream);

/* Bytes of device workspace that lla_attend_decode_gather needs for B rows of `budget` listed
 * slots. May be 0; 0 as well for an invalid descriptor or size. */
size_t lla_gather_workspace_bytes(const lla_desc* desc, int32_t B, int32_t budget);

/* Decode-time attention over a listed subset of the cached latents: token eviction composed with
 * LLA (Section 7, "Memory, capacity and latency", and Appendix C, where a StreamingLLM/H2O-style
 * policy keeps attention sinks plus a recent window). Same arithmetic as lla_attend_decode, with
 * row b's key set given by a slot list instead of the first N_b slots.
 *
 *   slots   [device] int32 [B][budget]: row b attends the cached latents at slots[b][0 ..
 *           counts[b]-1], in any order. A slot outside [0, n_max) is skipped (never read); a slot
 *           listed twice is two keys.
 *   budget  list capacity per row, >= 1.
 *   counts  [device] int32 [B] or NULL (all budget); clamped to [0, budget].
 *   ws      [device] at least lla_gather_workspace_bytes(desc, B, budget) bytes (NULL if 0).
 *   Other arguments as in lla_attend_decode. Both variants run on the streaming kernels, so the
 *   compiled (r_k, r_v) pairs are the streaming ones. An empty key set (no listed slot in range and
 *   no self token) gives out = 0 and lse = -inf. */
lla_status lla_attend_decode_gather(const lla_desc* desc, int32_t B, int32_t t, const void* q,
                                    const void* zk, const void* zv, const int32_t* slots,
                                    int32_t budget, const int32_t* counts, const void* Wk,
                                    const void* Wv, const void* mu_k, const void* mu_v,
                                    const void* k_self, const void* v_self, void* out, float* lse,
                                    void* ws, size_t ws_bytes, void* stream);

/* Chunked-prefill attention at loop t: C query rows per sequence over the latent cache, causal.
 *
 * The chunk's own latents must already be in slots ctx_lens[b] .. ctx_lens[b]+C-1 (written by
 * lla_encode: the two-pass order of the paper's cached decoder, Appendix A, "Decoding and
 * caching"). Row j sits at position ctx_lens[b] + j and attends latents 0 .. ctx_lens[b] + j,
 * inclusive. Same absorbed arithmetic as lla_attend_decode, without a self token.
 *
 *   q   [device] [B][C][H][d_head];  out [device] [B][C][H][d_head].
 *   ctx_lens [device] int32 [B]; a row whose position is outside [0, n_max) attends the clamped
 *            range 0 .. min(position, n_max-1), and an empty range gives 0.
 *   ws  [device] at least lla_workspace_bytes(desc, B, C) bytes.
 *   Other arguments as in lla_attend_decode. */
lla_status lla_attend_prefill(const lla_desc* desc, int32_t B, int32_t C, int32_t t,
                              const void* q, const void* zk, const void* zv,
                              const int32_t* ctx_lens, const void* Wk, const void* Wv,
                              const void* mu_k, const void* mu_v, void* out,
                              void* ws, size_t ws_bytes, void* stream);

/* Static, human-readable name of a status code. */
const char* lla_status_string(lla_status s);

/* LLA_ABI_VERSION of the built library. */
int32_t lla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LLA_H_ */
