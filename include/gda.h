/* gda.h - C ABI of libgda: the Grouped Differential (Latent) Attention forward on
 * AMD Instinct MI355X (gfx950).
 *
 * Operation (Motif 3 technical-report walk-through, paper.rainbus.top, step 2
 * "GDLA forward", equation D_t; head split of the Motif-2-12.7B overview,
 * section 2.2, and the Motif 3 release post, architecture paragraph):
 *
 *   signal heads i < S and noise heads j < N attend over the same expanded KV
 *   heads h < Hkv, each path with its own softmax attention
 *       H_x[t] = sum_{s visible from t} softmax_s(q_x[t] . k[s] / sqrt(dqk)) v[s]
 *   signal head i reads KV head floor(i*Hkv/S), noise head j reads KV head
 *   floor(j*Hkv/N); noise head j is repeated onto signal heads g*j .. g*j+g-1
 *   (g = S/N), and
 *       out[t,i,:] = gate[t,i,:] * (H_S[t,i,:] - lambda[t,i] * H_N[t,floor(i/g),:]).
 *   Key s is visible from query t iff s <= t and (window == 0 or t-s <= window-1).
 *   lambda and gate are values in (0,1) (the sigmoid that produces them is
 *   upstream of this call). W^O is not applied.
 *
 * Conventions shared by every entry point:
 *   - All tensors are dense, row-major, innermost dimension contiguous, device
 *     memory, 16-byte aligned, of the element type `dtype` (all share it).
 *   - Ownership: the caller owns every buffer. The library allocates no device
 *     memory at run time and keeps no mutable global state beyond a thread-local
 *     diagnostic string and, for gda_decode_latent_noalloc only, one static
 *     device array per GPU (below) with its looked-up address; calls are
 *     thread-safe. `out` must not alias an input.
 *   - Asynchrony: a call enqueues its kernels on `stream` (a hipStream_t; NULL
 *     is the default stream) and returns without synchronizing.
 *   - Errors: arguments are validated on the host before any HIP call; a
 *     rejected call launches nothing and returns GDA_ERROR_INVALID_ARGUMENT or
 *     GDA_ERROR_UNSUPPORTED. A HIP failure (including "no device") returns
 *     GDA_ERROR_HIP. Nothing is thrown or aborted across the ABI.
 *   - Offsets are 64-bit: a tensor may hold more than 2^31 elements.
 *   - Results are bitwise reproducible run to run for identical inputs.
 */
#ifndef GDA_H
#define GDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDA_SUCCESS = 0,
  GDA_ERROR_INVALID_ARGUMENT = 1, /* null or misaligned pointer, size < 1, window < 0,
                                     head counts that do not divide, unknown dtype         */
  GDA_ERROR_UNSUPPORTED = 2,      /* valid but not compiled: (dqk, dv) for bf16, or a form
                                     offered for bf16 only (training, latent decode)        */
  GDA_ERROR_HIP = 3               /* a HIP runtime or launch failure                       */
} gda_status;

typedef enum { GDA_BF16 = 0, GDA_F32 = 1 } gda_dtype;

/* Prefill (every query position of each sequence).
 *   q_sig   [B, L, S,   dqk]      signal queries
 *   q_noise [B, L, N,   dqk]      noise queries
 *   k       [B, L, Hkv, dqk]      expanded keys (post-RoPE)
 *   v       [B, L, Hkv, dv ]      expanded values
 *   lambda  [B, L, S]             per-token, per-signal-head noise coefficient
 *   gate    [B, L, S,   dv ]      output gate values
 *   out     [B, L, S,   dv ]      written: gate * (H_S - lambda * Repeat_g(H_N))
 * Requirements: all sizes >= 1; S % N == 0; S % Hkv == 0; N % Hkv == 0 or
 * Hkv % N == 0; window >= 0 (0 = full causal, W >= 1 = keys t-W+1 .. t).
 * GDA_BF16 needs (dqk, dv) in {(64,64), (128,128), (192,128)} (returns
 * GDA_ERROR_UNSUPPORTED otherwise) and takes every head layout the requirements
 * allow. GDA_F32 takes any sizes and layout.
 * Accumulation is fp32 in both dtypes; bf16 outputs are rounded to nearest even. */
gda_status gda_fwd(const void* q_sig, const void* q_noise, const void* k, const void* v,
                   const void* lambda, const void* gate, void* out,
                   int B, int L, int S, int N, int Hkv, int dqk, int dv,
                   int window, gda_dtype dtype, void* stream);

/* Decode: one new query token per sequence, attending over a KV cache that
 * already holds that token's K/V at position cache_lens[b]-1.
 *   q_sig   [B, S,   dqk]
 *   q_noise [B, N,   dqk]
 *   k_cache [B, Lmax, Hkv, dqk]
 *   v_cache [B, Lmax, Hkv, dv ]
 *   cache_lens  device int32 [B] (4-byte aligned), or NULL for "every sequence holds Lmax tokens".
 *               A length above Lmax is clamped to Lmax; a length below 1 yields
 *               an all-zero output row (there is no key to attend to).
 *   lambda  [B, S]
 *   gate    [B, S, dv]
 *   out     [B, S, dv]
 * Same requirements as gda_fwd, plus Lmax >= 1. GDA_BF16 needs the same
 * (dqk, dv) set and takes every valid head layout. */
gda_status gda_decode(const void* q_sig, const void* q_noise, const void* k_cache,
                      const void* v_cache, const int32_t* cache_lens, const void* lambda,
                      const void* gate, void* out,
                      int B, int Lmax, int S, int N, int Hkv, int dqk, int dv,
                      int window, gda_dtype dtype, void* stream);

/* Call options of the _ex entry points (fused neighbours of the attention core).
 *   softmax_scale: 0 = 1/sqrt(dqk) (the plain calls); > 0 = scores are q.k times
 *     this value (for example a long-context mscale folded in); negative, NaN or
 *     infinite values are rejected.
 *   flags: GDA_LAMBDA_LOGITS - lambda holds logits; the kernels apply the
 *     sigmoid 1/(1+exp(-x)) that makes lambda a per-token value in (0,1) (the
 *     Motif 3 walk-through, novelty point one); GDA_GATE_LOGITS - the gate holds
 *     logits, likewise (step 2's sigmoid gate G_t). Other bits are rejected.
 * The sigmoid is computed in fp32 from the stored value. */
typedef struct {
  float softmax_scale;
  uint32_t flags;
} gda_options;

enum { GDA_LAMBDA_LOGITS = 1u, GDA_GATE_LOGITS = 2u };

/* gda_fwd / gda_decode with options; opts == NULL is the plain call. Everything
 * else (arguments, layouts, ownership, errors) as for the plain calls; invalid
 * options return GDA_ERROR_INVALID_ARGUMENT. */
gda_status gda_fwd_ex(const void* q_sig, const void* q_noise, const void* k, const void* v,
                      const void* lambda, const void* gate, void* out,
                      int B, int L, int S, int N, int Hkv, int dqk, int dv,
                      int window, gda_dtype dtype, const gda_options* opts, void* stream);

gda_status gda_decode_ex(const void* q_sig, const void* q_noise, const void* k_cache,
                         const void* v_cache, const int32_t* cache_lens, const void* lambda,
                         const void* gate, void* out,
                         int B, int Lmax, int S, int N, int Hkv, int dqk, int dv,
                         int window, gda_dtype dtype, const gda_options* opts, void* stream);

/* Prefill over packed sequences with a query offset (packed documents, and the
 * chunk-with-halo form of a sequence-sharded sliding-window layer: the Motif 3
 * walk-through's step 5 exchanges one halo of the window's keys per rank).
 *   q_sig   [Tq, S, dqk], q_noise [Tq, N, dqk], lambda [Tq, S], gate [Tq, S, dv],
 *   out     [Tq, S, dv]    the queries of all sequences, packed
 *   k       [Tk, Hkv, dqk], v [Tk, Hkv, dv]   the keys of all sequences, packed
 *   cu_seqlens_q, cu_seqlens_k: device int32 [nseq+1], nondecreasing from 0;
 *     sequence i owns query rows cu_seqlens_q[i] .. cu_seqlens_q[i+1]-1 and key
 *     rows cu_seqlens_k[i] .. cu_seqlens_k[i+1]-1 (Lq_i and Lk_i rows; Tq and Tk
 *     are the last entries).
 *   max_seqlen_q >= every Lq_i (sizes the grid).
 * Local query t of sequence i sits at key position Lk_i - Lq_i + t (its queries are
 * its last Lq_i positions) and sees keys s <= that position (and, with a window,
 * within W of it). Lq_i = Lk_i is a packed document; Lk_i = Lq_i + W - 1 is a
 * chunk whose previous W-1 keys came as a halo. A query at a negative position
 * (Lk_i < Lq_i) sees no key and gets zeros. The cu_seqlens contents are not
 * validated (device memory): values outside the tensors are undefined behaviour.
 * Everything else as gda_fwd_ex (head maps, dtypes, options, support). */
gda_status gda_fwd_varlen(const void* q_sig, const void* q_noise, const void* k, const void* v,
                          const void* lambda, const void* gate, void* out,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                          int max_seqlen_q, int S, int N, int Hkv, int dqk, int dv, int window,
                          gda_dtype dtype, const gda_options* opts, void* stream);

/* Decode over the latent KV cache (GDLA's inference form; Motif 3 walk-through,
 * step 2 "GDLA forward" and novelty point one: the cache holds the KV latent and
 * the decoupled rotary key, MLA-sized, and W^KV_b expands the latent into the KV
 * heads that signal and noise queries share).
 *   q_sig   [B, S, Dn+Dr]   signal queries: Dn non-rotary dims, then Dr rotary dims
 *   q_noise [B, N, Dn+Dr]
 *   c_kv    [B, Lmax, Dc]   KV latent per cached token (after its RMSNorm)
 *   k_rope  [B, Lmax, Dr]   decoupled rotary key per cached token (all heads)
 *   w_kv_b  [Hkv, Dn+dv, Dc] up-projection of KV head h: rows 0..Dn-1 give the
 *                           key's non-rotary part, rows Dn..Dn+dv-1 the value
 *   cache_lens, lambda [B,S], gate [B,S,dv], out [B,S,dv], window: as gda_decode.
 * Head h's key at token s is [w_kv_b[h][0:Dn] c_s ; k_rope_s], its value
 * w_kv_b[h][Dn:Dn+dv] c_s; then exactly the gda_decode operation (scale
 * 1/sqrt(Dn+Dr) unless opts gives one). Nothing is expanded in memory: the
 * kernels attend in the latent space and up-project the result.
 * workspace: device memory of at least gda_decode_latent_workspace_bytes(...)
 * bytes, 16-byte aligned, owned by the caller and not read across calls; calls
 * that share a workspace must be ordered (same stream).
 * Supported: GDA_BF16, (Dn, Dr, Dc, dv) = (128, 64, 512, 128), S + N <= 128, at
 * most 15 signal heads per noise head and 16 query heads per KV head
 * (GDA_ERROR_UNSUPPORTED otherwise); a workspace that is too small or missing
 * returns GDA_ERROR_INVALID_ARGUMENT. */
size_t gda_decode_latent_workspace_bytes(int B, int Lmax, int S, int N, int window);

gda_status gda_decode_latent(const void* q_sig, const void* q_noise, const void* c_kv,
                             const void* k_rope, const void* w_kv_b, const int32_t* cache_lens,
                             const void* lambda, const void* gate, void* out,
                             int B, int Lmax, int S, int N, int Hkv, int Dn, int Dr, int Dc,
                             int dv, int window, gda_dtype dtype, const gda_options* opts,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free latent-cache decode, for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): gda_decode_latent with the same arguments
 * minus the workspace, which is a static device array of
 * GDA_DECODE_LATENT_SCRATCH_BYTES bytes built into the library (each GPU the
 * library runs on holds its own copy from load until the process ends). Calls
 * whose gda_decode_latent_workspace_bytes(...) exceeds that size return
 * GDA_ERROR_INVALID_ARGUMENT and launch nothing. The call allocates nothing and
 * needs no zeroed memory (every scratch byte it reads it wrote earlier in the
 * same call). Every call on one GPU uses that GPU's one array: calls that may
 * overlap in time on one GPU (different streams, or threads without ordering)
 * race and must be serialised by the caller; calls on one stream are ordered. */
#define GDA_DECODE_LATENT_SCRATCH_BYTES ((size_t)64 << 20)

gda_status gda_decode_latent_noalloc(const void* q_sig, const void* q_noise, const void* c_kv,
                                     const void* k_rope, const void* w_kv_b,
                                     const int32_t* cache_lens, const void* lambda,
                                     const void* gate, void* out, int B, int Lmax, int S, int N,
                                     int Hkv, int Dn, int Dr, int Dc, int dv, int window,
                                     gda_dtype dtype, const gda_options* opts, void* stream);

/* Training: the forward that also keeps what the backward needs, and the
 * backward (the pages' setting is training: the Motif 3 walk-through trains the
 * GDLA layers, steps 4 and 5). bf16 only.
 *
 * gda_fwd_train: gda_fwd_ex (same tensors, options, support) that also writes
 *   h_sig   [B, L, S, dv] bf16   each signal head's normalised attention output H_S
 *   h_noise [B, L, N, dv] bf16   each noise head's normalised attention output H_N
 *   lse     [B, S+N, L]   float  each attention row's log-sum-exp of its scaled
 *                                scores, natural log (heads 0..S-1 signal, then noise)
 * h_sig and h_noise 16-byte aligned, lse 4-byte aligned. fp32 returns
 * GDA_ERROR_UNSUPPORTED. */
gda_status gda_fwd_train(const void* q_sig, const void* q_noise, const void* k, const void* v,
                         const void* lambda, const void* gate, void* out, void* h_sig,
                         void* h_noise, float* lse, int B, int L, int S, int N, int Hkv,
                         int dqk, int dv, int window, gda_dtype dtype, const gda_options* opts,
                         void* stream);

/* Workspace bytes gda_bwd needs (each path's dO and every row's delta), or 0 for
 * sizes below 1. */
size_t gda_bwd_workspace_bytes(int B, int L, int S, int N, int dv);

/* gda_bwd: gradients of sum(d_out (.) out) for the forward gda_fwd_train ran, from
 * the same inputs, options and window, and its h_sig, h_noise and lse.
 *   d_out [B,L,S,dv]; outputs (all bf16, written, not accumulated):
 *   dq_sig [B,L,S,dqk], dq_noise [B,L,N,dqk], dk [B,L,Hkv,dqk], dv_out [B,L,Hkv,dv],
 *   dlambda [B,L,S], dgate [B,L,S,dv]; with GDA_LAMBDA_LOGITS / GDA_GATE_LOGITS the
 *   gradients are with respect to the logits.
 * workspace: device memory of at least gda_bwd_workspace_bytes(B, L, S, N, dv)
 * bytes, 256-byte aligned, owned by the caller, not read across calls. Tensors
 * 16-byte aligned (lse 4-byte). Supported as gda_fwd_train; fp32 returns
 * GDA_ERROR_UNSUPPORTED. Outputs are written once each (no atomics), so results
 * are deterministic. */
gda_status gda_bwd(const void* q_sig, const void* q_noise, const void* k, const void* v,
                   const void* lambda, const void* gate, const void* h_sig, const void* h_noise,
                   const float* lse, const void* d_out, void* dq_sig, void* dq_noise, void* dk,
                   void* dv_out, void* dlambda, void* dgate, int B, int L, int S, int N, int Hkv,
                   int dqk, int dv, int window, gda_dtype dtype, const gda_options* opts,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Training over packed sequences (sequences and positions as gda_fwd_varlen; the
 * chunk-with-halo form trains a sequence-sharded sliding-window layer).
 * gda_fwd_train_varlen: gda_fwd_varlen plus h_sig [Tq,S,dv], h_noise [Tq,N,dv] and
 *   lse [S+N, Tq] (total_q = Tq, the last cu_seqlens_q entry). A query at a
 *   negative position gets zero path outputs and lse -inf.
 * gda_bwd_varlen: gda_bwd over the packed tensors (gradients shaped like them:
 *   dq_sig [Tq,S,dqk], dq_noise [Tq,N,dqk], dk [Tk,Hkv,dqk], dv_out [Tk,Hkv,dv],
 *   dlambda [Tq,S], dgate [Tq,S,dv]); max_seqlen_k >= every sequence's key count.
 *   Workspace: gda_bwd_workspace_bytes(1, total_q, S, N, dv) bytes. Keys no query
 *   sees get zero gradients. Other rules as gda_bwd. */
gda_status gda_fwd_train_varlen(const void* q_sig, const void* q_noise, const void* k,
                                const void* v, const void* lambda, const void* gate, void* out,
                                void* h_sig, void* h_noise, float* lse,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int nseq, int max_seqlen_q, int total_q, int S, int N, int Hkv,
                                int dqk, int dv, int window, gda_dtype dtype,
                                const gda_options* opts, void* stream);

gda_status gda_bwd_varlen(const void* q_sig, const void* q_noise, const void* k, const void* v,
                          const void* lambda, const void* gate, const void* h_sig,
                          const void* h_noise, const float* lse, const void* d_out,
                          void* dq_sig, void* dq_noise, void* dk, void* dv_out, void* dlambda,
                          void* dgate, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          int nseq, int max_seqlen_q, int max_seqlen_k, int total_q, int S,
                          int N, int Hkv, int dqk, int dv, int window, gda_dtype dtype,
                          const gda_options* opts, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Static, never-NULL description of a status code. */
const char* gda_status_string(gda_status s);

/* Static text of the last validation or HIP error seen on the calling thread
 * ("" if none). Meant for diagnostics; not needed to use the library. */
const char* gda_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
