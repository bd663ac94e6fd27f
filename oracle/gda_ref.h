/* gda_ref.h - fp64 CPU oracle for the Grouped Differential (Latent) Attention core.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the bench's
 * CPU-baseline leg may load this library. The product path (libgda) neither
 * includes this header nor links this code, and this code includes nothing
 * from the product path.
 *
 * The operation is the one the Motif 3 technical-report walk-through
 * (paper.rainbus.top, step 2 "GDLA forward", equation D_t) writes out: signal
 * and noise query heads attend over the same expanded KV heads, each path with
 * its own softmax attention; the noise output is repeated g times by group;
 * D = H_S - lambda (.) Repeat_g(H_N); a sigmoid gate G multiplies D elementwise.
 *
 * All inputs are read at their stored values (bf16 bit patterns or float32,
 * widened exactly to double); every sum, exponential and quotient is in double.
 */
#ifndef GDA_REF_H
#define GDA_REF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { GDA_REF_BF16 = 0, GDA_REF_F32 = 1 };

/* Prefill. Layouts (row-major, innermost contiguous):
 *   q_sig [B,L,S,dqk], q_noise [B,L,N,dqk], k [B,L,Hkv,dqk], v [B,L,Hkv,dv],
 *   lambda [B,L,S], gate [B,L,S,dv]; all of storage type `dtype`.
 * rows: NULL for every (b,t) (out is [B,L,S,dv]), else n_rows flat indices
 *   r = b*L + t (out is [n_rows,S,dv]).
 * Returns 0, or a negative value for arguments it cannot take. */
int gda_ref_fwd(const void* q_sig, const void* q_noise, const void* k, const void* v,
                const void* lambda, const void* gate, double* out,
                int64_t B, int64_t L, int64_t S, int64_t N, int64_t Hkv,
                int64_t dqk, int64_t dv, int64_t window, int dtype,
                const int64_t* rows, int64_t n_rows);

/* Decode: one query token per sequence at position len_b - 1 over a cache that
 * already holds that token's K/V.
 *   q_sig [B,S,dqk], q_noise [B,N,dqk], k_cache [B,Lmax,Hkv,dqk],
 *   v_cache [B,Lmax,Hkv,dv], lambda [B,S], gate [B,S,dv]; cache_lens host
 *   int32 [B] or NULL (= Lmax). A length above Lmax is clamped to Lmax; a
 *   length below 1 gives an all-zero output row. out is [B,S,dv]. */
int gda_ref_decode(const void* q_sig, const void* q_noise, const void* k_cache,
                   const void* v_cache, const int32_t* cache_lens, const void* lambda,
                   const void* gate, double* out,
                   int64_t B, int64_t Lmax, int64_t S, int64_t N, int64_t Hkv,
                   int64_t dqk, int64_t dv, int64_t window, int dtype);

/* Options of the _ex forms (0 and 0 give the plain forms above):
 *   softmax_scale > 0 replaces 1/sqrt(dqk); 0 keeps it; negative or NaN is rejected;
 *   flags: lambda and/or gate hold logits, turned into values by 1/(1+exp(-x)). */
enum { GDA_REF_LAMBDA_LOGITS = 1, GDA_REF_GATE_LOGITS = 2 };

int gda_ref_fwd_ex(const void* q_sig, const void* q_noise, const void* k, const void* v,
                   const void* lambda, const void* gate, double* out,
                   int64_t B, int64_t L, int64_t S, int64_t N, int64_t Hkv,
                   int64_t dqk, int64_t dv, int64_t window, int dtype,
                   const int64_t* rows, int64_t n_rows, double softmax_scale, int flags);

int gda_ref_decode_ex(const void* q_sig, const void* q_noise, const void* k_cache,
                      const void* v_cache, const int32_t* cache_lens, const void* lambda,
                      const void* gate, double* out,
                      int64_t B, int64_t Lmax, int64_t S, int64_t N, int64_t Hkv,
                      int64_t dqk, int64_t dv, int64_t window, int dtype,
                      double softmax_scale, int flags);

/* Packed sequences with a query offset. Sequence i has query rows cu_q[i] ..
 * cu_q[i+1]-1 and key rows cu_k[i] .. cu_k[i+1]-1 of the packed tensors
 * q_sig [Tq,S,dqk], q_noise [Tq,N,dqk], k [Tk,Hkv,dqk], v [Tk,Hkv,dv], lambda [Tq,S],
 * gate [Tq,S,dv]; out is [Tq,S,dv]. Local query t of a sequence with Lq queries and
 * Lk keys sits at key position Lk - Lq + t; a query at a negative position gives
 * zeros. cu_q and cu_k are host arrays of nseq+1 nondecreasing values from 0. */
int gda_ref_fwd_varlen(const void* q_sig, const void* q_noise, const void* k, const void* v,
                       const void* lambda, const void* gate, double* out,
                       const int32_t* cu_q, const int32_t* cu_k, int64_t nseq,
                       int64_t S, int64_t N, int64_t Hkv, int64_t dqk, int64_t dv,
                       int64_t window, int dtype, double softmax_scale, int flags);

/* Latent-cache decode: the cache holds per token the KV latent c (Dc values) and
 * the decoupled rotary key (Dr values, shared by all heads); w_kv_b [Hkv, Dn+dv, Dc]
 * expands c into head h's key [W[h][0:Dn] c ; k_rope] and value W[h][Dn:Dn+dv] c.
 *   q_sig [B,S,Dn+Dr], q_noise [B,N,Dn+Dr], c_kv [B,Lmax,Dc], k_rope [B,Lmax,Dr],
 *   lambda [B,S], gate [B,S,dv], cache_lens as in gda_ref_decode; out [B,S,dv].
 * The expansion is computed in double, then the decode definition applies. */
int gda_ref_decode_latent(const void* q_sig, const void* q_noise, const void* c_kv,
                          const void* k_rope, const void* w_kv_b, const int32_t* cache_lens,
                          const void* lambda, const void* gate, double* out,
                          int64_t B, int64_t Lmax, int64_t S, int64_t N, int64_t Hkv,
                          int64_t Dn, int64_t Dr, int64_t Dc, int64_t dv, int64_t window,
                          int dtype, double softmax_scale, int flags);

/* Training form of the forward: out as gda_ref_fwd_ex, plus what the backward
 * takes from the forward:
 *   h_sig [B,L,S,dv], h_noise [B,L,N,dv]: each path's normalised attention output;
 *   lse [B,S+N,L]: log(sum_s exp(z_s)) of each attention row's scaled scores z
 *   (natural log; heads 0..S-1 are the signal heads, S..S+N-1 the noise heads). */
int gda_ref_fwd_train(const void* q_sig, const void* q_noise, const void* k, const void* v,
                      const void* lambda, const void* gate, double* out, double* h_sig,
                      double* h_noise, double* lse,
                      int64_t B, int64_t L, int64_t S, int64_t N, int64_t Hkv,
                      int64_t dqk, int64_t dv, int64_t window, int dtype,
                      double softmax_scale, int flags);

/* Backward of the prefill: the gradients of sum(d_out (.) out) with respect to
 * q_sig, q_noise, k, v, lambda and gate (with the logit flags, with respect to the
 * logits). d_out [B,L,S,dv] is of storage type dtype; every gradient is double.
 * q_rows: NULL for every (b,t), else n_q_rows flat query rows b*L+t; the query-side
 *   gradients are then dq_sig [n_q_rows,S,dqk], dq_noise [n_q_rows,N,dqk],
 *   dlambda [n_q_rows,S], dgate [n_q_rows,S,dv] (else [B,L,...]).
 * k_rows: likewise for the key side: dk [n_k_rows,Hkv,dqk], dv_out [n_k_rows,Hkv,dv]. */
int gda_ref_bwd(const void* q_sig, const void* q_noise, const void* k, const void* v,
                const void* lambda, const void* gate, const void* d_out, double* dq_sig,
                double* dq_noise, double* dk, double* dv_out, double* dlambda, double* dgate,
                int64_t B, int64_t L, int64_t S, int64_t N, int64_t Hkv,
                int64_t dqk, int64_t dv, int64_t window, int dtype,
                double softmax_scale, int flags,
                const int64_t* q_rows, int64_t n_q_rows, const int64_t* k_rows,
                int64_t n_k_rows);

/* Packed-sequence forms of the two above (sequences as in gda_ref_fwd_varlen):
 * gda_ref_fwd_train_varlen: out [Tq,S,dv], h_sig [Tq,S,dv], h_noise [Tq,N,dv] and
 *   lse [S+N, Tq]; gda_ref_bwd_varlen: d_out [Tq,S,dv] -> dq_sig [Tq,S,dqk],
 *   dq_noise [Tq,N,dqk], dk [Tk,Hkv,dqk], dv_out [Tk,Hkv,dv], dlambda [Tq,S],
 *   dgate [Tq,S,dv]. A query at a negative position has no visible key: its path
 *   outputs are zero, its lse is -inf, and it contributes no gradient to K or V. */
int gda_ref_fwd_train_varlen(const void* q_sig, const void* q_noise, const void* k,
                             const void* v, const void* lambda, const void* gate, double* out,
                             double* h_sig, double* h_noise, double* lse,
                             const int32_t* cu_q, const int32_t* cu_k, int64_t nseq,
                             int64_t S, int64_t N, int64_t Hkv, int64_t dqk, int64_t dv,
                             int64_t window, int dtype, double softmax_scale, int flags);

int gda_ref_bwd_varlen(const void* q_sig, const void* q_noise, const void* k, const void* v,
                       const void* lambda, const void* gate, const void* d_out,
                       double* dq_sig, double* dq_noise, double* dk, double* dv_out,
                       double* dlambda, double* dgate, const int32_t* cu_q,
                       const int32_t* cu_k, int64_t nseq, int64_t S, int64_t N, int64_t Hkv,
                       int64_t dqk, int64_t dv, int64_t window, int dtype,
                       double softmax_scale, int flags);

/* Threads an OpenMP parallel region of this library starts with (for timing reports). */
int gda_ref_threads(void);

#ifdef __cplusplus
}
#endif
#endif
