/* gda_ref.c - fp64 CPU oracle for the Grouped Differential (Latent) Attention core.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * bench's CPU-baseline leg, never by the product path. Shares no code with it.
 *
 * It is the definition written out, in the order the Motif 3 technical-report
 * walk-through (paper.rainbus.top, step 2 "GDLA forward") states it:
 *   1. signal and noise query paths share the expanded KV heads and each
 *      computes its own softmax attention over the visible keys;
 *   2. the noise output is repeated g = S/N times by group;
 *   3. D_t = H_S,t - lambda_t (.) Repeat_g(H_N,t)      (equation D_t);
 *   4. the sigmoid gate G_t multiplies D_t elementwise (before W^O).
 * Readings taken where the pages are silent (each listed in the design notes):
 *   - softmax scale 1/sqrt(dqk), dqk the contraction length;
 *   - signal head i reads KV head floor(i*Hkv/S), noise head j reads KV head
 *     floor(j*Hkv/N), and noise head j serves signal heads g*j .. g*j+g-1
 *     (block order of "repeated g times by group");
 *   - lambda is one value per (token, signal head), broadcast over dv; lambda
 *     and gate arrive as values in (0,1) (the sigmoid is upstream), or, when the
 *     caller says so, as logits that the sigmoid 1/(1+exp(-x)) turns into those
 *     values here (the walk-through's sigmoid gate G_t and sigmoid-bounded
 *     per-token lambda, novelty point one);
 *   - an explicit softmax scale replaces 1/sqrt(dqk) when the caller gives one;
 *   - key s is visible from query t iff s <= t and, for a window W >= 1,
 *     t - s <= W - 1 (W keys including the query's own); W = 0 is full causal;
 *   - decode attends from position len-1 of a cache that already holds it.
 * Built with -ffp-contract=off so no fused multiply-add changes a rounding.
 */
#include "gda_ref.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  const void* k;
  const void* v;
  int64_t Lk, Hkv, dqk, dv;
  int dtype;
  int mutant;
  double scale;  /* softmax scale given by the caller, or 0 for 1/sqrt(dqk) */
  int flags;     /* GDA_REF_LAMBDA_LOGITS | GDA_REF_GATE_LOGITS */
} kv_view;

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Stored value -> double. bf16 is the upper half of a float32, so the
 * widening is exact. */
static double rd(const void* base, int64_t i, int dtype) {
  if (dtype == GDA_REF_F32) return (double)((const float*)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int64_t k_index(const kv_view* kv, int64_t b, int64_t s, int64_t h, int64_t d) {
  if (kv->mutant == GDA_REF_MUT_K_TRANSPOSED)
    return ((b * kv->Hkv + h) * kv->Lk + s) * kv->dqk + d;
  return ((b * kv->Lk + s) * kv->Hkv + h) * kv->dqk + d;
}

static int64_t v_index(const kv_view* kv, int64_t b, int64_t s, int64_t h, int64_t e) {
  return ((b * kv->Lk + s) * kv->Hkv + h) * kv->dv + e;
}

/* Visible keys of query position t: [lo, hi]. */
static void visible_range(int64_t t, int64_t W, int64_t Lk, int mutant, int64_t* lo,
                          int64_t* hi) {
  int64_t h = t, l;
  if (mutant == GDA_REF_MUT_NO_CAUSAL) h = Lk - 1;
  if (W == 0)
    l = 0;
  else if (mutant == GDA_REF_MUT_WINDOW_OBO)
    l = t - W;
  else
    l = t - W + 1;
  if (l < 0) l = 0;
  if (mutant == GDA_REF_MUT_SKIP_FIRST_KEY && l == 0) l = 1;
  *lo = l;
  *hi = h;
}

/* One path's attention for one query row over KV head h of batch row b:
 *   z_s = scale * sum_d q[d] k[b,s,h,d]           for s in [lo, hi]
 *   w_s = exp(z_s - max_s z_s),  l = sum_s w_s
 *   H[e] = (sum_s w_s v[b,s,h,e]) / l
 * z is scratch of at least hi-lo+1 doubles. */
static void attend(const void* q, int64_t q_off, const kv_view* kv, int64_t b, int64_t h,
                   int64_t lo, int64_t hi, double scale, double* z, double* H) {
  for (int64_t e = 0; e < kv->dv; ++e) H[e] = 0.0;
  if (hi < lo) return;
  double m = -INFINITY;
  for (int64_t s = lo; s <= hi; ++s) {
    double acc = 0.0;
    for (int64_t d = 0; d < kv->dqk; ++d)
      acc += rd(q, q_off + d, kv->dtype) * rd(kv->k, k_index(kv, b, s, h, d), kv->dtype);
    z[s - lo] = scale * acc;
    if (z[s - lo] > m) m = z[s - lo];
  }
  double l = 0.0;
  for (int64_t s = lo; s <= hi; ++s) {
    z[s - lo] = exp(z[s - lo] - m);
    l += z[s - lo];
  }
  for (int64_t s = lo; s <= hi; ++s)
    for (int64_t e = 0; e < kv->dv; ++e)
      H[e] += z[s - lo] * rd(kv->v, v_index(kv, b, s, h, e), kv->dtype);
  if (kv->mutant != GDA_REF_MUT_NO_NORMALIZE)
    for (int64_t e = 0; e < kv->dv; ++e) H[e] /= l;
}

/* Every output of one query row: out[i][e] for signal heads i, dv channels e. */
static void gda_row(const void* q_sig, int64_t qs_off, const void* q_noise, int64_t qn_off,
                    const void* lambda, int64_t lam_off, const void* gate, int64_t gate_off,
                    const kv_view* kv, int64_t b, int64_t t, int64_t S, int64_t N,
                    int64_t window, double* z, double* Hn, double* Hs, double* out) {
  const int64_t Hkv = kv->Hkv, dqk = kv->dqk, dv = kv->dv;
  const int mut = kv->mutant;
  const int64_t g = S / N;
  const double scale = kv->scale > 0.0
                           ? kv->scale
                           : 1.0 / sqrt((double)(mut == GDA_REF_MUT_SCALE_DV ? dv : dqk));
  int64_t lo, hi;
  visible_range(t, window, kv->Lk, mut, &lo, &hi);

  /* Noise path: noise head j on KV head floor(j*Hkv/N). */
  for (int64_t j = 0; j < N; ++j)
    attend(q_noise, qn_off + j * dqk, kv, b, (j * Hkv) / N, lo, hi, scale, z, Hn + j * dv);

  /* Signal path, then D = H_S - lambda * Repeat_g(H_N), then the gate. */
  for (int64_t i = 0; i < S; ++i) {
    const int64_t kvs = (mut == GDA_REF_MUT_KV_INTERLEAVE) ? i % Hkv : (i * Hkv) / S;
    attend(q_sig, qs_off + i * dqk, kv, b, kvs, lo, hi, scale, z, Hs);
    const int64_t j = (mut == GDA_REF_MUT_TILED_REPEAT) ? i % N : i / g;
    double lam = rd(lambda, lam_off + (mut == GDA_REF_MUT_LAMBDA_BY_GROUP ? j : i), kv->dtype);
    if (kv->flags & GDA_REF_LAMBDA_LOGITS) lam = sigmoid(lam);
    for (int64_t e = 0; e < dv; ++e) {
      double D;
      if (mut == GDA_REF_MUT_DROP_LAMBDA)
        D = Hs[e];
      else if (mut == GDA_REF_MUT_PLUS_LAMBDA)
        D = Hs[e] + lam * Hn[j * dv + e];
      else
        D = Hs[e] - lam * Hn[j * dv + e];
      double G = rd(gate, gate_off + i * dv + e, kv->dtype);
      if (kv->flags & GDA_REF_GATE_LOGITS) G = sigmoid(G);
      out[i * dv + e] = (mut == GDA_REF_MUT_NO_GATE) ? D : G * D;
    }
  }
}

static int check_common(int64_t B, int64_t L, int64_t S, int64_t N, int64_t Hkv, int64_t dqk,
                        int64_t dv, int64_t window, int dtype) {
  if (B < 1 || L < 1 || S < 1 || N < 1 || Hkv < 1 || dqk < 1 || dv < 1) return -1;
  if (S % N != 0 || S % Hkv != 0) return -2;
  if (N % Hkv != 0 && Hkv % N != 0) return -3;
  if (window < 0) return -4;
  if (dtype != GDA_REF_BF16 && dtype != GDA_REF_F32) return -5;
  return 0;
}

int gda_ref_fwd(const void* q_sig, const void* q_noise, const void* k, const void* v,
                const void* lambda, const void* gate, double* out, int64_t B, int64_t L,
                int64_t S, int64_t N, int64_t Hkv, int64_t dqk, int64_t dv, int64_t window,
                int dtype, const int64_t* rows, int64_t n_rows, int mutant) {
  return gda_ref_fwd_ex(q_sig, q_noise, k, v, lambda, gate, out, B, L, S, N, Hkv, dqk, dv,
                        window, dtype, rows, n_rows, 0.0, 0, mutant);
}

int gda_ref_fwd_ex(const void* q_sig, const void* q_noise, const void* k, const void* v,
                   const void* lambda, const void* gate, double* out, int64_t B, int64_t L,
                   int64_t S, int64_t N, int64_t Hkv, int64_t dqk, int64_t dv, int64_t window,
                   int dtype, const int64_t* rows, int64_t n_rows, double softmax_scale,
                   int flags, int mutant) {
  int rc = check_common(B, L, S, N, Hkv, dqk, dv, window, dtype);
  if (rc) return rc;
  if (!q_sig || !q_noise || !k || !v || !lambda || !gate || !out) return -6;
  if (!(softmax_scale >= 0.0) || (flags & ~(GDA_REF_LAMBDA_LOGITS | GDA_REF_GATE_LOGITS)))
    return -9;
  const kv_view kv = {k, v, L, Hkv, dqk, dv, dtype, mutant, softmax_scale, flags};
  const int64_t total = rows ? n_rows : B * L;
  for (int64_t r = 0; r < total; ++r) {
    const int64_t flat = rows ? rows[r] : r;
    if (flat < 0 || flat >= B * L) return -7;
  }
  int failed = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)L);
    double* Hn = (double*)malloc(sizeof(double) * (size_t)(N * dv));
    double* Hs = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!z || !Hn || !Hs) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < total; ++r) {
        const int64_t flat = rows ? rows[r] : r;
        const int64_t b = flat / L, t = flat % L;
        gda_row(q_sig, flat * S * dqk, q_noise, flat * N * dqk, lambda, flat * S, gate,
                flat * S * dv, &kv, b, t, S, N, window, z, Hn, Hs, out + r * S * dv);
      }
    }
    free(z);
    free(Hn);
    free(Hs);
  }
  return failed ? -8 : 0;
}

int gda_ref_decode(const void* q_sig, const void* q_noise, const void* k_cache,
                   const void* v_cache, const int32_t* cache_lens, const void* lambda,
                   const void* gate, double* out, int64_t B, int64_t Lmax, int64_t S,
                   int64_t N, int64_t Hkv, int64_t dqk, int64_t dv, int64_t window, int dtype,
                   int mutant) {
  return gda_ref_decode_ex(q_sig, q_noise, k_cache, v_cache, cache_lens, lambda, gate, out, B,
                           Lmax, S, N, Hkv, dqk, dv, window, dtype, 0.0, 0, mutant);
}

int gda_ref_decode_ex(const void* q_sig, const void* q_noise, const void* k_cache,
                      const void* v_cache, const int32_t* cache_lens, const void* lambda,
                      const void* gate, double* out, int64_t B, int64_t Lmax, int64_t S,
                      int64_t N, int64_t Hkv, int64_t dqk, int64_t dv, int64_t window,
                      int dtype, double softmax_scale, int flags, int mutant) {
  int rc = check_common(B, Lmax, S, N, Hkv, dqk, dv, window, dtype);
  if (rc) return rc;
  if (!q_sig || !q_noise || !k_cache || !v_cache || !lambda || !gate || !out) return -6;
  if (!(softmax_scale >= 0.0) || (flags & ~(GDA_REF_LAMBDA_LOGITS | GDA_REF_GATE_LOGITS)))
    return -9;
  const kv_view kv = {k_cache, v_cache, Lmax, Hkv, dqk, dv, dtype, mutant, softmax_scale, flags};
  int failed = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)Lmax);
    double* Hn = (double*)malloc(sizeof(double) * (size_t)(N * dv));
    double* Hs = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!z || !Hn || !Hs) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t b = 0; b < B; ++b) {
        int64_t len = cache_lens ? (int64_t)cache_lens[b] : Lmax;
        if (len > Lmax) len = Lmax;
        double* o = out + b * S * dv;
        if (len < 1) {
          for (int64_t x = 0; x < S * dv; ++x) o[x] = 0.0;
          continue;
        }
        int64_t p = len - 1;
        if (mutant == GDA_REF_MUT_DECODE_POS) p = len < Lmax ? len : Lmax - 1;
        gda_row(q_sig, b * S * dqk, q_noise, b * N * dqk, lambda, b * S, gate, b * S * dv, &kv,
                b, p, S, N, window, z, Hn, Hs, o);
      }
    }
    free(z);
    free(Hn);
    free(Hs);
  }
  return failed ? -8 : 0;
}

/* ---- Packed sequences with a query offset -----------------------------------------
 * Sequence i owns query rows cu_q[i] .. cu_q[i+1]-1 and key rows cu_k[i] ..
 * cu_k[i+1]-1 of the packed tensors (Lq_i and Lk_i rows). Its queries are the last
 * Lq_i positions of its keys: local query t sits at key position (Lk_i - Lq_i) + t,
 * and sees the keys s <= that position (and within the window). Packed documents
 * are the case Lq_i = Lk_i; a sliding-window layer's halo exchange (walk-through
 * step 5: one halo exchange of the window's keys) is the case Lk_i = Lq_i + W - 1.
 * A query at a negative position sees no key and gives zeros. */
static const void* offset_ptr(const void* base, int64_t elems, int dtype) {
  return (const char*)base + elems * (dtype == GDA_REF_F32 ? 4 : 2);
}

int gda_ref_fwd_varlen(const void* q_sig, const void* q_noise, const void* k, const void* v,
                       const void* lambda, const void* gate, double* out,
                       const int32_t* cu_q, const int32_t* cu_k, int64_t nseq, int64_t S,
                       int64_t N, int64_t Hkv, int64_t dqk, int64_t dv, int64_t window,
                       int dtype, double softmax_scale, int flags) {
  int rc = check_common(1, 1, S, N, Hkv, dqk, dv, window, dtype);
  if (rc) return rc;
  if (nseq < 1 || !cu_q || !cu_k) return -1;
  if (!q_sig || !q_noise || !k || !v || !lambda || !gate || !out) return -6;
  if (!(softmax_scale >= 0.0) || (flags & ~(GDA_REF_LAMBDA_LOGITS | GDA_REF_GATE_LOGITS)))
    return -9;
  if (cu_q[0] != 0 || cu_k[0] != 0) return -10;
  int64_t maxk = 1;
  for (int64_t i = 0; i < nseq; ++i) {
    if (cu_q[i + 1] < cu_q[i] || cu_k[i + 1] < cu_k[i]) return -10;
    if (cu_k[i + 1] - cu_k[i] > maxk) maxk = cu_k[i + 1] - cu_k[i];
  }
  const int64_t Tq = cu_q[nseq];
  int failed = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)maxk);
    double* Hn = (double*)malloc(sizeof(double) * (size_t)(N * dv));
    double* Hs = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!z || !Hn || !Hs) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < Tq; ++r) {
        int64_t i = 0;
        while (cu_q[i + 1] <= r) ++i;  /* the sequence of query row r */
        const int64_t Lq = cu_q[i + 1] - cu_q[i], Lk = cu_k[i + 1] - cu_k[i];
        const int64_t pos = (Lk - Lq) + (r - cu_q[i]);
        const kv_view kv = {offset_ptr(k, (int64_t)cu_k[i] * Hkv * dqk, dtype),
                            offset_ptr(v, (int64_t)cu_k[i] * Hkv * dv, dtype),
                            Lk, Hkv, dqk, dv, dtype, GDA_REF_EXACT, softmax_scale, flags};
        gda_row(q_sig, r * S * dqk, q_noise, r * N * dqk, lambda, r * S, gate, r * S * dv, &kv,
                0, pos, S, N, window, z, Hn, Hs, out + r * S * dv);
      }
    }
    free(z);
    free(Hn);
    free(Hs);
  }
  return failed ? -8 : 0;
}

/* ---- Latent-cache decode --------------------------------------------------------
 * The cache holds, per token, the KV latent c (Dc values, after its RMSNorm) and
 * the decoupled rotary key (Dr values, shared by every head); W^KV_b expands the
 * latent into the KV heads (walk-through step 2: c_KV in R^512 -> RMSNorm -> W^KV_b
 * -> 16 KV heads; novelty point one: both query paths share the up-projected KV
 * and the broadcast rotary key, so the cache is MLA-sized). Written out plainly:
 *   key of head h at s   = [ W[h][0:Dn] c_s ; k_rope_s ]      (Dn + Dr values)
 *   value of head h at s = W[h][Dn:Dn+dv] c_s                 (dv values)
 * each computed in double, then the decode of gda_ref_decode_ex over those keys
 * and values (same head maps, window, lambda, gate, options). */
static void expand_head(const void* c_kv, const void* w, int64_t b, int64_t h, int64_t lo,
                        int64_t hi, int64_t Lmax, int64_t Dn, int64_t Dc, int64_t dv, int dtype,
                        int mutant, double* Kh, double* Vh) {
  const int64_t rows = Dn + dv;
  for (int64_t s = lo; s <= hi; ++s) {
    const int64_t c0 = (b * Lmax + s) * Dc;
    for (int64_t r = 0; r < rows; ++r) {
      int64_t wr = r;
      if (mutant == GDA_REF_MUT_LATENT_V_ROWS && r >= Dn) wr = r - Dn; /* value from key rows */
      double acc = 0.0;
      for (int64_t c = 0; c < Dc; ++c) {
        const int64_t wi = (mutant == GDA_REF_MUT_LATENT_W_T) ? (h * Dc + c) * rows + wr
                                                               : (h * rows + wr) * Dc + c;
        acc += rd(w, wi, dtype) * rd(c_kv, c0 + c, dtype);
      }
      if (r < Dn)
        Kh[(s - lo) * Dn + r] = acc;
      else
        Vh[(s - lo) * dv + (r - Dn)] = acc;
    }
  }
}

/* Attention of one query head over the expanded keys/values of its KV head. */
static void attend_latent(const void* q, int64_t q_off, const void* k_rope, int64_t b,
                          int64_t lo, int64_t hi, int64_t Lmax, int64_t Dn, int64_t Dr,
                          int64_t dv, int dtype, int mutant, double scale, const double* Kh,
                          const double* Vh, double* z, double* H) {
  for (int64_t e = 0; e < dv; ++e) H[e] = 0.0;
  double m = -INFINITY;
  for (int64_t s = lo; s <= hi; ++s) {
    double acc = 0.0;
    for (int64_t d = 0; d < Dn; ++d) acc += rd(q, q_off + d, dtype) * Kh[(s - lo) * Dn + d];
    if (mutant != GDA_REF_MUT_LATENT_NO_ROPE)
      for (int64_t r = 0; r < Dr; ++r)
        acc += rd(q, q_off + Dn + r, dtype) * rd(k_rope, (b * Lmax + s) * Dr + r, dtype);
    z[s - lo] = scale * acc;
    if (z[s - lo] > m) m = z[s - lo];
  }
  double l = 0.0;
  for (int64_t s = lo; s <= hi; ++s) {
    z[s - lo] = exp(z[s - lo] - m);
    l += z[s - lo];
  }
  for (int64_t s = lo; s <= hi; ++s)
    for (int64_t e = 0; e < dv; ++e) H[e] += z[s - lo] * Vh[(s - lo) * dv + e];
  for (int64_t e = 0; e < dv; ++e) H[e] /= l;
}

int gda_ref_decode_latent(const void* q_sig, const void* q_noise, const void* c_kv,
                          const void* k_rope, const void* w_kv_b, const int32_t* cache_lens,
                          const void* lambda, const void* gate, double* out, int64_t B,
                          int64_t Lmax, int64_t S, int64_t N, int64_t Hkv, int64_t Dn,
                          int64_t Dr, int64_t Dc, int64_t dv, int64_t window, int dtype,
                          double softmax_scale, int flags, int mutant) {
  int rc = check_common(B, Lmax, S, N, Hkv, Dn + Dr, dv, window, dtype);
  if (rc) return rc;
  if (Dn < 1 || Dr < 0 || Dc < 1) return -1;
  if (!q_sig || !q_noise || !c_kv || (Dr > 0 && !k_rope) || !w_kv_b || !lambda || !gate || !out)
    return -6;
  if (!(softmax_scale >= 0.0) || (flags & ~(GDA_REF_LAMBDA_LOGITS | GDA_REF_GATE_LOGITS)))
    return -9;
  const int64_t dqk = Dn + Dr, g = S / N;
  const double scale = softmax_scale > 0.0 ? softmax_scale : 1.0 / sqrt((double)dqk);
  /* Per-head outputs of every sequence, then the combine. */
  double* Hs = (double*)calloc((size_t)(B * S * dv), sizeof(double));
  double* Hn = (double*)calloc((size_t)(B * N * dv), sizeof(double));
  if (!Hs || !Hn) {
    free(Hs);
    free(Hn);
    return -8;
  }
  int failed = 0;
#pragma omp parallel
  {
    double* Kh = (double*)malloc(sizeof(double) * (size_t)(Lmax * Dn));
    double* Vh = (double*)malloc(sizeof(double) * (size_t)(Lmax * dv));
    double* z = (double*)malloc(sizeof(double) * (size_t)Lmax);
    if (!Kh || !Vh || !z) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t bh = 0; bh < B * Hkv; ++bh) {
        const int64_t b = bh / Hkv, h = bh % Hkv;
        int64_t len = cache_lens ? (int64_t)cache_lens[b] : Lmax;
        if (len > Lmax) len = Lmax;
        if (len < 1) continue;
        const int64_t pos = len - 1;
        const int64_t lo = window ? (pos - window + 1 > 0 ? pos - window + 1 : 0) : 0;
        expand_head(c_kv, w_kv_b, b, h, lo, pos, Lmax, Dn, Dc, dv, dtype, mutant, Kh, Vh);
        for (int64_t j = 0; j < N; ++j)
          if ((j * Hkv) / N == h)
            attend_latent(q_noise, (b * N + j) * dqk, k_rope, b, lo, pos, Lmax, Dn, Dr, dv,
                          dtype, mutant, scale, Kh, Vh, z, Hn + (b * N + j) * dv);
        for (int64_t i = 0; i < S; ++i)
          if ((i * Hkv) / S == h)
            attend_latent(q_sig, (b * S + i) * dqk, k_rope, b, lo, pos, Lmax, Dn, Dr, dv,
                          dtype, mutant, scale, Kh, Vh, z, Hs + (b * S + i) * dv);
      }
    }
    free(Kh);
    free(Vh);
    free(z);
  }
  for (int64_t b = 0; b < B && !failed; ++b) {
    int64_t len = cache_lens ? (int64_t)cache_lens[b] : Lmax;
    double* o = out + b * S * dv;
    for (int64_t i = 0; i < S; ++i) {
      double lam = rd(lambda, b * S + i, dtype);
      if (flags & GDA_REF_LAMBDA_LOGITS) lam = sigmoid(lam);
      for (int64_t e = 0; e < dv; ++e) {
        if (len < 1) {
          o[i * dv + e] = 0.0;
          continue;
        }
        double G = rd(gate, (b * S + i) * dv + e, dtype);
        if (flags & GDA_REF_GATE_LOGITS) G = sigmoid(G);
        o[i * dv + e] = G * (Hs[(b * S + i) * dv + e] - lam * Hn[(b * N + i / g) * dv + e]);
      }
    }
  }
  free(Hs);
  free(Hn);
  return failed ? -8 : 0;
}

int gda_ref_threads(void) { return omp_get_max_threads(); }
