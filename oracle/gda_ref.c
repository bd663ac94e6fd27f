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
 * Readings taken where the pages are silent:
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
  return ((b * kv->Lk + s) * kv->Hkv + h) * kv->dqk + d;
}

static int64_t v_index(const kv_view* kv, int64_t b, int64_t s, int64_t h, int64_t e) {
  return ((b * kv->Lk + s) * kv->Hkv + h) * kv->dv + e;
}

/* Visible keys of query position t: [lo, hi]. */
static void visible_range(int64_t t, int64_t W, int64_t* lo, int64_t* hi) {
  int64_t l = W == 0 ? 0 : t - W + 1;
  if (l < 0) l = 0;
  *lo = l;
  *hi = t;
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
  for (int64_t e = 0; e < kv->dv; ++e) H[e] /= l;
}

/* Every output of one query row: out[i][e] for signal heads i, dv channels e. */
static void gda_row(const void* q_sig, int64_t qs_off, const void* q_noise, int64_t qn_off,
                    const void* lambda, int64_t lam_off, const void* gate, int64_t gate_off,
                    const kv_view* kv, int64_t b, int64_t t, int64_t S, int64_t N,
                    int64_t window, double* z, double* Hn, double* Hs, double* out) {
  const int64_t Hkv = kv->Hkv, dqk = kv->dqk, dv = kv->dv;
  const int64_t g = S / N;
  const double scale = kv->scale > 0.0 ? kv->scale : 1.0 / sqrt((double)dqk);
  int64_t lo, hi;
  visible_range(t, window, &lo, &hi);

  /* Noise path: noise head j on KV head floor(j*Hkv/N). */
  for (int64_t j = 0; j < N; ++j)
    attend(q_noise, qn_off + j * dqk, kv, b, (j * Hkv) / N, lo, hi, scale, z, Hn + j * dv);

  /* Signal path, then D = H_S - lambda * Repeat_g(H_N), then the gate. */
  for (int64_t i = 0; i < S; ++i) {
    const int64_t kvs = (i * Hkv) / S;
    attend(q_sig, qs_off + i * dqk, kv, b, kvs, lo, hi, scale, z, Hs);
    const int64_t j = i / g;
    double lam = rd(lambda, lam_off + i, kv->dtype);
    if (kv->flags & GDA_REF_LAMBDA_LOGITS) lam = sigmoid(lam);
    for (int64_t e = 0; e < dv; ++e) {
      const double D = Hs[e] - lam * Hn[j * dv + e];
      double G = rd(gate, gate_off + i * dv + e, kv->dtype);
      if (kv->flags & GDA_REF_GATE_LOGITS) G = sigmoid(G);
      out[i * dv + e] = G * D;
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
                int dtype, const int64_t* rows, int64_t n_rows) {
  return gda_ref_fwd_ex(q_sig, q_noise, k, v, lambda, gate, out, B, L, S, N, Hkv, dqk, dv,
                        window, dtype, rows, n_rows, 0.0, 0);
}

int gda_ref_fwd_ex(const void* q_sig, const void* q_noise, const void* k, const void* v,
                   const void* lambda, const void* gate, double* out, int64_t B, int64_t L,
                   int64_t S, int64_t N, int64_t Hkv, int64_t dqk, int64_t dv, int64_t window,
                   int dtype, const int64_t* rows, int64_t n_rows, double softmax_scale,
                   int flags) {
  int rc = check_common(B, L, S, N, Hkv, dqk, dv, window, dtype);
  if (rc) return rc;
  if (!q_sig || !q_noise || !k || !v || !lambda || !gate || !out) return -6;
  if (!(softmax_scale >= 0.0) || (flags & ~(GDA_REF_LAMBDA_LOGITS | GDA_REF_GATE_LOGITS)))
    return -9;
  const kv_view kv = {k, v, L, Hkv, dqk, dv, dtype, softmax_scale, flags};
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
                   int64_t N, int64_t Hkv, int64_t dqk, int64_t dv, int64_t window,
                   int dtype) {
  return gda_ref_decode_ex(q_sig, q_noise, k_cache, v_cache, cache_lens, lambda, gate, out, B,
                           Lmax, S, N, Hkv, dqk, dv, window, dtype, 0.0, 0);
}

int gda_ref_decode_ex(const void* q_sig, const void* q_noise, const void* k_cache,
                      const void* v_cache, const int32_t* cache_lens, const void* lambda,
                      const void* gate, double* out, int64_t B, int64_t Lmax, int64_t S,
                      int64_t N, int64_t Hkv, int64_t dqk, int64_t dv, int64_t window,
                      int dtype, double softmax_scale, int flags) {
  int rc = check_common(B, Lmax, S, N, Hkv, dqk, dv, window, dtype);
  if (rc) return rc;
  if (!q_sig || !q_noise || !k_cache || !v_cache || !lambda || !gate || !out) return -6;
  if (!(softmax_scale >= 0.0) || (flags & ~(GDA_REF_LAMBDA_LOGITS | GDA_REF_GATE_LOGITS)))
    return -9;
  const kv_view kv = {k_cache, v_cache, Lmax, Hkv, dqk, dv, dtype, softmax_scale, flags};
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
        const int64_t p = len - 1;
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
                            Lk, Hkv, dqk, dv, dtype, softmax_scale, flags};
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
                        double* Kh, double* Vh) {
  const int64_t rows = Dn + dv;
  for (int64_t s = lo; s <= hi; ++s) {
    const int64_t c0 = (b * Lmax + s) * Dc;
    for (int64_t r = 0; r < rows; ++r) {
      double acc = 0.0;
      for (int64_t c = 0; c < Dc; ++c)
        acc += rd(w, (h * rows + r) * Dc + c, dtype) * rd(c_kv, c0 + c, dtype);
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
                          int64_t dv, int dtype, double scale, const double* Kh,
                          const double* Vh, double* z, double* H) {
  for (int64_t e = 0; e < dv; ++e) H[e] = 0.0;
  double m = -INFINITY;
  for (int64_t s = lo; s <= hi; ++s) {
    double acc = 0.0;
    for (int64_t d = 0; d < Dn; ++d) acc += rd(q, q_off + d, dtype) * Kh[(s - lo) * Dn + d];
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
                          double softmax_scale, int flags) {
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
        expand_head(c_kv, w_kv_b, b, h, lo, pos, Lmax, Dn, Dc, dv, dtype, Kh, Vh);
        for (int64_t j = 0; j < N; ++j)
          if ((j * Hkv) / N == h)
            attend_latent(q_noise, (b * N + j) * dqk, k_rope, b, lo, pos, Lmax, Dn, Dr, dv,
                          dtype, scale, Kh, Vh, z, Hn + (b * N + j) * dv);
        for (int64_t i = 0; i < S; ++i)
          if ((i * Hkv) / S == h)
            attend_latent(q_sig, (b * S + i) * dqk, k_rope, b, lo, pos, Lmax, Dn, Dr, dv,
                          dtype, scale, Kh, Vh, z, Hs + (b * S + i) * dv);
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

/* ---- Training form of the forward, and the backward ----------------------------
 * The backward is the chain rule taken through the forward definition above, its
 * steps in reverse order:
 *   out = G (.) D with D = H_S - lambda Repeat_g(H_N):
 *     dG = d_out (.) D                       (times G(1-G) when the gate is a logit)
 *     dD = d_out (.) G
 *     dlambda_i = -sum_e dD_i,e H_N,j(i),e    (times lambda(1-lambda) for a logit)
 *     dH_S,i = dD_i,   dH_N,j = -sum over the group's signal heads of lambda_i dD_i
 *   every attention row (query t of head h over KV head kv(h)), with the
 *   normalised weights P_s = exp(z_s - lse) of its scaled scores z:
 *     dP_s = dH . v_s,   delta = sum_s P_s dP_s,   dz_s = P_s (dP_s - delta)
 *     dq_t = scale sum_s dz_s k_s,   dk_s += scale dz_s q_t,   dv_s += P_s dH
 */

static double score(const void* q, int64_t q_off, const kv_view* kv, int64_t b, int64_t h,
                    int64_t s, double scale) {
  double acc = 0.0;
  for (int64_t d = 0; d < kv->dqk; ++d)
    acc += rd(q, q_off + d, kv->dtype) * rd(kv->k, k_index(kv, b, s, h, d), kv->dtype);
  return scale * acc;
}

/* Scaled scores of one query row over keys lo..hi into z; returns their
 * log-sum-exp (natural log), -inf when no key is visible. */
static double row_lse(const void* q, int64_t q_off, const kv_view* kv, int64_t b, int64_t h,
                      int64_t lo, int64_t hi, double scale, double* z) {
  if (hi < lo) return -INFINITY;
  double m = -INFINITY;
  for (int64_t s = lo; s <= hi; ++s) {
    z[s - lo] = score(q, q_off, kv, b, h, s, scale);
    if (z[s - lo] > m) m = z[s - lo];
  }
  double l = 0.0;
  for (int64_t s = lo; s <= hi; ++s) l += exp(z[s - lo] - m);
  return m + log(l);
}

static double softmax_scale_of(const kv_view* kv) {
  return kv->scale > 0.0 ? kv->scale : 1.0 / sqrt((double)kv->dqk);
}

/* Head h of a row (0..S-1 signal, S..S+N-1 noise): its query offset and KV head. */
static void head_of(int64_t h, int64_t flat, int64_t S, int64_t N, int64_t Hkv, int64_t dqk,
                    const void* q_sig, const void* q_noise, const void** q, int64_t* q_off,
                    int64_t* kvh) {
  if (h < S) {
    *q = q_sig;
    *q_off = (flat * S + h) * dqk;
    *kvh = (h * Hkv) / S;
  } else {
    *q = q_noise;
    *q_off = (flat * N + (h - S)) * dqk;
    *kvh = ((h - S) * Hkv) / N;
  }
}

int gda_ref_fwd_train(const void* q_sig, const void* q_noise, const void* k, const void* v,
                      const void* lambda, const void* gate, double* out, double* h_sig,
                      double* h_noise, double* lse, int64_t B, int64_t L, int64_t S,
                      int64_t N, int64_t Hkv, int64_t dqk, int64_t dv, int64_t window,
                      int dtype, double softmax_scale, int flags) {
  int rc = gda_ref_fwd_ex(q_sig, q_noise, k, v, lambda, gate, out, B, L, S, N, Hkv, dqk, dv,
                          window, dtype, NULL, 0, softmax_scale, flags);
  if (rc) return rc;
  if (!h_sig || !h_noise || !lse) return -6;
  const kv_view kv = {k, v, L, Hkv, dqk, dv, dtype, softmax_scale, flags};
  const double scale = softmax_scale_of(&kv);
  const int64_t HT = S + N;
  int failed = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)L);
    if (!z) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t flat = 0; flat < B * L; ++flat) {
        const int64_t b = flat / L, t = flat % L;
        int64_t lo, hi;
        visible_range(t, window, &lo, &hi);
        for (int64_t h = 0; h < HT; ++h) {
          const void* q;
          int64_t q_off, kvh;
          head_of(h, flat, S, N, Hkv, dqk, q_sig, q_noise, &q, &q_off, &kvh);
          const double ls = row_lse(q, q_off, &kv, b, kvh, lo, hi, scale, z);
          lse[(b * HT + h) * L + t] = ls;
          double* H = h < S ? h_sig + (flat * S + h) * dv : h_noise + (flat * N + h - S) * dv;
          for (int64_t e = 0; e < dv; ++e) H[e] = 0.0;
          for (int64_t s2 = lo; s2 <= hi; ++s2) {
            const double P = exp(z[s2 - lo] - ls);
            for (int64_t e = 0; e < dv; ++e)
              H[e] += P * rd(v, v_index(&kv, b, s2, kvh, e), dtype);
          }
        }
      }
    }
    free(z);
  }
  return failed ? -8 : 0;
}

int gda_ref_bwd(const void* q_sig, const void* q_noise, const void* k, const void* v,
                const void* lambda, const void* gate, const void* d_out, double* dq_sig,
                double* dq_noise, double* dk, double* dv_out, double* dlambda, double* dgate,
                int64_t B, int64_t L, int64_t S, int64_t N, int64_t Hkv, int64_t dqk,
                int64_t dv, int64_t window, int dtype, double softmax_scale, int flags,
                const int64_t* q_rows, int64_t n_q_rows, const int64_t* k_rows,
                int64_t n_k_rows) {
  int rc = check_common(B, L, S, N, Hkv, dqk, dv, window, dtype);
  if (rc) return rc;
  if (!q_sig || !q_noise || !k || !v || !lambda || !gate || !d_out || !dq_sig || !dq_noise ||
      !dk || !dv_out || !dlambda || !dgate)
    return -6;
  if (!(softmax_scale >= 0.0) || (flags & ~(GDA_REF_LAMBDA_LOGITS | GDA_REF_GATE_LOGITS)))
    return -9;
  const int64_t BL = B * L, HT = S + N, g = S / N;
  const int64_t nq = q_rows ? n_q_rows : BL, nk = k_rows ? n_k_rows : BL;
  for (int64_t r = 0; r < nq; ++r)
    if (q_rows && (q_rows[r] < 0 || q_rows[r] >= BL)) return -7;
  for (int64_t r = 0; r < nk; ++r)
    if (k_rows && (k_rows[r] < 0 || k_rows[r] >= BL)) return -7;
  const kv_view kv = {k, v, L, Hkv, dqk, dv, dtype, softmax_scale, flags};
  const double scale = softmax_scale_of(&kv);

  /* Query rows whose forward quantities are needed: the query-side outputs, and
   * every query that sees one of the key-side rows. */
  int64_t* slot = (int64_t*)malloc(sizeof(int64_t) * (size_t)BL);
  if (!slot) return -8;
  for (int64_t i = 0; i < BL; ++i) slot[i] = -1;
  for (int64_t r = 0; r < nq; ++r) slot[q_rows ? q_rows[r] : r] = 0;
  for (int64_t r = 0; r < nk; ++r) {
    const int64_t flat = k_rows ? k_rows[r] : r, b = flat / L, s = flat % L;
    const int64_t t_hi = window ? (s + window - 1 < L - 1 ? s + window - 1 : L - 1) : L - 1;
    for (int64_t t = s; t <= t_hi; ++t) slot[b * L + t] = 0;
  }
  int64_t nrow = 0;
  for (int64_t i = 0; i < BL; ++i)
    if (slot[i] == 0) slot[i] = nrow++;
  int64_t* row_flat = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nrow ? nrow : 1));
  double* dH = (double*)malloc(sizeof(double) * (size_t)((nrow ? nrow : 1) * HT * dv));
  double* row_lse_v = (double*)malloc(sizeof(double) * (size_t)((nrow ? nrow : 1) * HT));
  double* delta = (double*)malloc(sizeof(double) * (size_t)((nrow ? nrow : 1) * HT));
  /* query-side output position of each needed row (-1: not an output row) */
  int64_t* q_out = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nrow ? nrow : 1));
  if (!row_flat || !dH || !row_lse_v || !delta || !q_out) {
    free(slot);
    free(row_flat);
    free(dH);
    free(row_lse_v);
    free(delta);
    free(q_out);
    return -8;
  }
  for (int64_t i = 0; i < BL; ++i)
    if (slot[i] >= 0) row_flat[slot[i]] = i;
  for (int64_t r = 0; r < nrow; ++r) q_out[r] = -1;
  for (int64_t r = 0; r < nq; ++r) q_out[slot[q_rows ? q_rows[r] : r]] = r;

  int failed = 0;
  /* 1. Per needed row: every head's forward (lse, H), then the combine and gate
   *    backward (dG, dlambda, dH), then delta = sum_s P_s dP_s for every head. */
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)L);
    double* H = (double*)malloc(sizeof(double) * (size_t)(HT * dv));
    double* lam = (double*)malloc(sizeof(double) * (size_t)S);
    if (!z || !H || !lam) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < nrow; ++r) {
        const int64_t flat = row_flat[r], b = flat / L, t = flat % L;
        int64_t lo, hi;
        visible_range(t, window, &lo, &hi);
        for (int64_t h = 0; h < HT; ++h) {
          const void* q;
          int64_t q_off, kvh;
          head_of(h, flat, S, N, Hkv, dqk, q_sig, q_noise, &q, &q_off, &kvh);
          const double ls = row_lse(q, q_off, &kv, b, kvh, lo, hi, scale, z);
          row_lse_v[r * HT + h] = ls;
          for (int64_t e = 0; e < dv; ++e) H[h * dv + e] = 0.0;
          for (int64_t s2 = lo; s2 <= hi; ++s2) {
            const double P = exp(z[s2 - lo] - ls);
            for (int64_t e = 0; e < dv; ++e)
              H[h * dv + e] += P * rd(v, v_index(&kv, b, s2, kvh, e), dtype);
          }
        }
        double* dHr = dH + r * HT * dv;
        for (int64_t i = 0; i < S; ++i) {
          const int64_t j = i / g;
          double lm = rd(lambda, flat * S + i, dtype);
          if (flags & GDA_REF_LAMBDA_LOGITS) lm = sigmoid(lm);
          lam[i] = lm;
          double dlam = 0.0;
          for (int64_t e = 0; e < dv; ++e) {
            const double D = H[i * dv + e] - lm * H[(S + j) * dv + e];
            const double gi = rd(gate, (flat * S + i) * dv + e, dtype);
            const double G = (flags & GDA_REF_GATE_LOGITS) ? sigmoid(gi) : gi;
            const double dO = rd(d_out, (flat * S + i) * dv + e, dtype);
            double dG = dO * D;
            if (flags & GDA_REF_GATE_LOGITS) dG *= G * (1.0 - G);
            const double dD = dO * G;
            dHr[i * dv + e] = dD;
            dlam -= dD * H[(S + j) * dv + e];
            if (q_out[r] >= 0) dgate[(q_out[r] * S + i) * dv + e] = dG;
          }
          if (flags & GDA_REF_LAMBDA_LOGITS) dlam *= lm * (1.0 - lm);
          if (q_out[r] >= 0) dlambda[q_out[r] * S + i] = dlam;
        }
        for (int64_t j = 0; j < N; ++j)
          for (int64_t e = 0; e < dv; ++e) {
            double acc = 0.0;
            for (int64_t i = g * j; i < g * j + g; ++i) acc -= lam[i] * dHr[i * dv + e];
            dHr[(S + j) * dv + e] = acc;
          }
        for (int64_t h = 0; h < HT; ++h) {
          const void* q;
          int64_t q_off, kvh;
          head_of(h, flat, S, N, Hkv, dqk, q_sig, q_noise, &q, &q_off, &kvh);
          double dl = 0.0;
          for (int64_t s2 = lo; s2 <= hi; ++s2) {
            const double P = exp(score(q, q_off, &kv, b, kvh, s2, scale) - row_lse_v[r * HT + h]);
            double dP = 0.0;
            for (int64_t e = 0; e < dv; ++e)
              dP += dHr[h * dv + e] * rd(v, v_index(&kv, b, s2, kvh, e), dtype);
            dl += P * dP;
          }
          delta[r * HT + h] = dl;
        }
      }
    }
    free(z);
    free(H);
    free(lam);
  }

  /* 2. Query side: dq_t = scale sum_s dz_s k_s for every head. */
  if (!failed) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t rq = 0; rq < nq; ++rq) {
      const int64_t flat = q_rows ? q_rows[rq] : rq, b = flat / L, t = flat % L;
      const int64_t r = slot[flat];
      int64_t lo, hi;
      visible_range(t, window, &lo, &hi);
      for (int64_t h = 0; h < HT; ++h) {
        const void* q;
        int64_t q_off, kvh;
        head_of(h, flat, S, N, Hkv, dqk, q_sig, q_noise, &q, &q_off, &kvh);
        double* dq = h < S ? dq_sig + (rq * S + h) * dqk : dq_noise + (rq * N + h - S) * dqk;
        for (int64_t d = 0; d < dqk; ++d) dq[d] = 0.0;
        for (int64_t s2 = lo; s2 <= hi; ++s2) {
          const double P = exp(score(q, q_off, &kv, b, kvh, s2, scale) - row_lse_v[r * HT + h]);
          double dP = 0.0;
          for (int64_t e = 0; e < dv; ++e)
            dP += dH[(r * HT + h) * dv + e] * rd(v, v_index(&kv, b, s2, kvh, e), dtype);
          const double dz = P * (dP - delta[r * HT + h]);
          for (int64_t d = 0; d < dqk; ++d)
            dq[d] += scale * dz * rd(k, k_index(&kv, b, s2, kvh, d), dtype);
        }
      }
    }

    /* 3. Key side: dk_s = scale sum_t dz_ts q_t, dv_s = sum_t P_ts dH_t over every
     *    query t that sees key s and every head on the KV head. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t rk = 0; rk < nk; ++rk) {
      const int64_t flat = k_rows ? k_rows[rk] : rk, b = flat / L, s2 = flat % L;
      for (int64_t x = 0; x < Hkv * dqk; ++x) dk[rk * Hkv * dqk + x] = 0.0;
      for (int64_t x = 0; x < Hkv * dv; ++x) dv_out[rk * Hkv * dv + x] = 0.0;
      const int64_t t_hi = window ? (s2 + window - 1 < L - 1 ? s2 + window - 1 : L - 1) : L - 1;
      for (int64_t t = s2; t <= t_hi; ++t) {
        int64_t lo, hi;
        visible_range(t, window, &lo, &hi);
        if (s2 < lo || s2 > hi) continue;
        const int64_t qflat = b * L + t, r = slot[qflat];
        for (int64_t h = 0; h < HT; ++h) {
          const void* q;
          int64_t q_off, kvh;
          head_of(h, qflat, S, N, Hkv, dqk, q_sig, q_noise, &q, &q_off, &kvh);
          const double P = exp(score(q, q_off, &kv, b, kvh, s2, scale) - row_lse_v[r * HT + h]);
          double dP = 0.0;
          for (int64_t e = 0; e < dv; ++e)
            dP += dH[(r * HT + h) * dv + e] * rd(v, v_index(&kv, b, s2, kvh, e), dtype);
          const double dz = P * (dP - delta[r * HT + h]);
          for (int64_t d = 0; d < dqk; ++d)
            dk[(rk * Hkv + kvh) * dqk + d] += scale * dz * rd(q, q_off + d, dtype);
          for (int64_t e = 0; e < dv; ++e)
            dv_out[(rk * Hkv + kvh) * dv + e] += P * dH[(r * HT + h) * dv + e];
        }
      }
    }
  }
  free(slot);
  free(row_flat);
  free(dH);
  free(row_lse_v);
  free(delta);
  free(q_out);
  return failed ? -8 : 0;
}

/* ---- Packed sequences: training form of the forward, and the backward ------------
 * The same steps over packed sequences with a query offset: sequence i owns query
 * rows cu_q[i] .. cu_q[i+1]-1 and key rows cu_k[i] .. cu_k[i+1]-1; its local query t
 * sits at key position Lk - Lq + t (a negative position sees no key). */

static int check_cu(const int32_t* cu_q, const int32_t* cu_k, int64_t nseq, int64_t* maxk) {
  if (nseq < 1 || !cu_q || !cu_k) return -1;
  if (cu_q[0] != 0 || cu_k[0] != 0) return -10;
  *maxk = 1;
  for (int64_t i = 0; i < nseq; ++i) {
    if (cu_q[i + 1] < cu_q[i] || cu_k[i + 1] < cu_k[i]) return -10;
    if (cu_k[i + 1] - cu_k[i] > *maxk) *maxk = cu_k[i + 1] - cu_k[i];
  }
  return 0;
}

/* The sequence of packed row r under offsets cu (nseq+1 entries). */
static int64_t seq_of(const int32_t* cu, int64_t r) {
  int64_t i = 0;
  while (cu[i + 1] <= r) ++i;
  return i;
}

/* K/V view of sequence i: its key 0 at packed key row cu_k[i]. */
static kv_view seq_view(const void* k, const void* v, const int32_t* cu_k, int64_t i,
                        int64_t Hkv, int64_t dqk, int64_t dv, int dtype,
                        double softmax_scale, int flags) {
  const kv_view kv = {offset_ptr(k, (int64_t)cu_k[i] * Hkv * dqk, dtype),
                      offset_ptr(v, (int64_t)cu_k[i] * Hkv * dv, dtype),
                      cu_k[i + 1] - cu_k[i], Hkv, dqk, dv, dtype, softmax_scale, flags};
  return kv;
}

int gda_ref_fwd_train_varlen(const void* q_sig, const void* q_noise, const void* k,
                             const void* v, const void* lambda, const void* gate, double* out,
                             double* h_sig, double* h_noise, double* lse, const int32_t* cu_q,
                             const int32_t* cu_k, int64_t nseq, int64_t S, int64_t N,
                             int64_t Hkv, int64_t dqk, int64_t dv, int64_t window, int dtype,
                             double softmax_scale, int flags) {
  int rc = gda_ref_fwd_varlen(q_sig, q_noise, k, v, lambda, gate, out, cu_q, cu_k, nseq, S, N,
                              Hkv, dqk, dv, window, dtype, softmax_scale, flags);
  if (rc) return rc;
  if (!h_sig || !h_noise || !lse) return -6;
  int64_t maxk;
  if ((rc = check_cu(cu_q, cu_k, nseq, &maxk))) return rc;
  const int64_t Tq = cu_q[nseq], HT = S + N;
  int failed = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)maxk);
    if (!z) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < Tq; ++r) {
        const int64_t i = seq_of(cu_q, r);
        const kv_view kv = seq_view(k, v, cu_k, i, Hkv, dqk, dv, dtype, softmax_scale,
                                    flags);
        const double scale = softmax_scale_of(&kv);
        const int64_t pos = (kv.Lk - (cu_q[i + 1] - cu_q[i])) + (r - cu_q[i]);
        int64_t lo, hi;
        visible_range(pos, window, &lo, &hi);
        for (int64_t h = 0; h < HT; ++h) {
          const void* q;
          int64_t q_off, kvh;
          head_of(h, r, S, N, Hkv, dqk, q_sig, q_noise, &q, &q_off, &kvh);
          const double ls = row_lse(q, q_off, &kv, 0, kvh, lo, hi, scale, z);
          lse[h * Tq + r] = ls;
          double* H = h < S ? h_sig + (r * S + h) * dv : h_noise + (r * N + h - S) * dv;
          for (int64_t e = 0; e < dv; ++e) H[e] = 0.0;
          for (int64_t s2 = lo; s2 <= hi; ++s2) {
            const double P = exp(z[s2 - lo] - ls);
            for (int64_t e = 0; e < dv; ++e)
              H[e] += P * rd(kv.v, v_index(&kv, 0, s2, kvh, e), dtype);
          }
        }
      }
    }
    free(z);
  }
  return failed ? -8 : 0;
}

int gda_ref_bwd_varlen(const void* q_sig, const void* q_noise, const void* k, const void* v,
                       const void* lambda, const void* gate, const void* d_out, double* dq_sig,
                       double* dq_noise, double* dk, double* dv_out, double* dlambda,
                       double* dgate, const int32_t* cu_q, const int32_t* cu_k, int64_t nseq,
                       int64_t S, int64_t N, int64_t Hkv, int64_t dqk, int64_t dv,
                       int64_t window, int dtype, double softmax_scale, int flags) {
  int rc = check_common(1, 1, S, N, Hkv, dqk, dv, window, dtype);
  if (rc) return rc;
  if (!q_sig || !q_noise || !k || !v || !lambda || !gate || !d_out || !dq_sig || !dq_noise ||
      !dk || !dv_out || !dlambda || !dgate)
    return -6;
  if (!(softmax_scale >= 0.0) || (flags & ~(GDA_REF_LAMBDA_LOGITS | GDA_REF_GATE_LOGITS)))
    return -9;
  int64_t maxk;
  if ((rc = check_cu(cu_q, cu_k, nseq, &maxk))) return rc;
  const int64_t Tq = cu_q[nseq], Tk = cu_k[nseq], HT = S + N, g = S / N;
  const size_t n1 = (size_t)(Tq ? Tq : 1);
  double* dH = (double*)malloc(sizeof(double) * n1 * (size_t)(HT * dv));
  double* lse = (double*)malloc(sizeof(double) * n1 * (size_t)HT);
  double* delta = (double*)malloc(sizeof(double) * n1 * (size_t)HT);
  if (!dH || !lse || !delta) {
    free(dH);
    free(lse);
    free(delta);
    return -8;
  }
  int failed = 0;
  /* 1. Per query row: every head's forward, the combine and gate backward, delta. */
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)maxk);
    double* H = (double*)malloc(sizeof(double) * (size_t)(HT * dv));
    double* lam = (double*)malloc(sizeof(double) * (size_t)S);
    if (!z || !H || !lam) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < Tq; ++r) {
        const int64_t i = seq_of(cu_q, r);
        const kv_view kv = seq_view(k, v, cu_k, i, Hkv, dqk, dv, dtype, softmax_scale,
                                    flags);
        const double scale = softmax_scale_of(&kv);
        const int64_t pos = (kv.Lk - (cu_q[i + 1] - cu_q[i])) + (r - cu_q[i]);
        int64_t lo, hi;
        visible_range(pos, window, &lo, &hi);
        for (int64_t h = 0; h < HT; ++h) {
          const void* q;
          int64_t q_off, kvh;
          head_of(h, r, S, N, Hkv, dqk, q_sig, q_noise, &q, &q_off, &kvh);
          const double ls = row_lse(q, q_off, &kv, 0, kvh, lo, hi, scale, z);
          lse[r * HT + h] = ls;
          for (int64_t e = 0; e < dv; ++e) H[h * dv + e] = 0.0;
          for (int64_t s2 = lo; s2 <= hi; ++s2) {
            const double P = exp(z[s2 - lo] - ls);
            for (int64_t e = 0; e < dv; ++e)
              H[h * dv + e] += P * rd(kv.v, v_index(&kv, 0, s2, kvh, e), dtype);
          }
        }
        double* dHr = dH + r * HT * dv;
        for (int64_t i2 = 0; i2 < S; ++i2) {
          const int64_t j = i2 / g;
          double lm = rd(lambda, r * S + i2, dtype);
          if (flags & GDA_REF_LAMBDA_LOGITS) lm = sigmoid(lm);
          lam[i2] = lm;
          double dlam = 0.0;
          for (int64_t e = 0; e < dv; ++e) {
            const double D = H[i2 * dv + e] - lm * H[(S + j) * dv + e];
            const double gi = rd(gate, (r * S + i2) * dv + e, dtype);
            const double G = (flags & GDA_REF_GATE_LOGITS) ? sigmoid(gi) : gi;
            const double dO = rd(d_out, (r * S + i2) * dv + e, dtype);
            double dG = dO * D;
            if (flags & GDA_REF_GATE_LOGITS) dG *= G * (1.0 - G);
            const double dD = dO * G;
            dHr[i2 * dv + e] = dD;
            dlam -= dD * H[(S + j) * dv + e];
            dgate[(r * S + i2) * dv + e] = dG;
          }
          if (flags & GDA_REF_LAMBDA_LOGITS) dlam *= lm * (1.0 - lm);
          dlambda[r * S + i2] = dlam;
        }
        for (int64_t j = 0; j < N; ++j)
          for (int64_t e = 0; e < dv; ++e) {
            double acc = 0.0;
            for (int64_t i2 = g * j; i2 < g * j + g; ++i2) acc -= lam[i2] * dHr[i2 * dv + e];
            dHr[(S + j) * dv + e] = acc;
          }
        for (int64_t h = 0; h < HT; ++h) {
          const void* q;
          int64_t q_off, kvh;
          head_of(h, r, S, N, Hkv, dqk, q_sig, q_noise, &q, &q_off, &kvh);
          double dl = 0.0;
          for (int64_t s2 = lo; s2 <= hi; ++s2) {
            const double P = exp(score(q, q_off, &kv, 0, kvh, s2, scale) - lse[r * HT + h]);
            double dP = 0.0;
            for (int64_t e = 0; e < dv; ++e)
              dP += dHr[h * dv + e] * rd(kv.v, v_index(&kv, 0, s2, kvh, e), dtype);
            dl += P * dP;
          }
          delta[r * HT + h] = dl;
        }
      }
    }
    free(z);
    free(H);
    free(lam);
  }
  if (!failed) {
    /* 2. Query side. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < Tq; ++r) {
      const int64_t i = seq_of(cu_q, r);
      const kv_view kv = seq_view(k, v, cu_k, i, Hkv, dqk, dv, dtype, softmax_scale,
                                  flags);
      const double scale = softmax_scale_of(&kv);
      const int64_t pos = (kv.Lk - (cu_q[i + 1] - cu_q[i])) + (r - cu_q[i]);
      int64_t lo, hi;
      visible_range(pos, window, &lo, &hi);
      for (int64_t h = 0; h < HT; ++h) {
        const void* q;
        int64_t q_off, kvh;
        head_of(h, r, S, N, Hkv, dqk, q_sig, q_noise, &q, &q_off, &kvh);
        double* dq = h < S ? dq_sig + (r * S + h) * dqk : dq_noise + (r * N + h - S) * dqk;
        for (int64_t d = 0; d < dqk; ++d) dq[d] = 0.0;
        for (int64_t s2 = lo; s2 <= hi; ++s2) {
          const double P = exp(score(q, q_off, &kv, 0, kvh, s2, scale) - lse[r * HT + h]);
          double dP = 0.0;
          for (int64_t e = 0; e < dv; ++e)
            dP += dH[(r * HT + h) * dv + e] * rd(kv.v, v_index(&kv, 0, s2, kvh, e), dtype);
          const double dz = P * (dP - delta[r * HT + h]);
          for (int64_t d = 0; d < dqk; ++d)
            dq[d] += scale * dz * rd(kv.k, k_index(&kv, 0, s2, kvh, d), dtype);
        }
      }
    }
    /* 3. Key side: every query of the key's sequence that sees it. */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t kr = 0; kr < Tk; ++kr) {
      const int64_t i = seq_of(cu_k, kr);
      const kv_view kv = seq_view(k, v, cu_k, i, Hkv, dqk, dv, dtype, softmax_scale,
                                  flags);
      const double scale = softmax_scale_of(&kv);
      const int64_t s2 = kr - cu_k[i], Lq = cu_q[i + 1] - cu_q[i], qoff = kv.Lk - Lq;
      for (int64_t x = 0; x < Hkv * dqk; ++x) dk[kr * Hkv * dqk + x] = 0.0;
      for (int64_t x = 0; x < Hkv * dv; ++x) dv_out[kr * Hkv * dv + x] = 0.0;
      for (int64_t t = 0; t < Lq; ++t) {
        int64_t lo, hi;
        visible_range(qoff + t, window, &lo, &hi);
        if (s2 < lo || s2 > hi) continue;
        const int64_t r = cu_q[i] + t;
        for (int64_t h = 0; h < HT; ++h) {
          const void* q;
          int64_t q_off, kvh;
          head_of(h, r, S, N, Hkv, dqk, q_sig, q_noise, &q, &q_off, &kvh);
          const double P = exp(score(q, q_off, &kv, 0, kvh, s2, scale) - lse[r * HT + h]);
          double dP = 0.0;
          for (int64_t e = 0; e < dv; ++e)
            dP += dH[(r * HT + h) * dv + e] * rd(kv.v, v_index(&kv, 0, s2, kvh, e), dtype);
          const double dz = P * (dP - delta[r * HT + h]);
          for (int64_t d = 0; d < dqk; ++d)
            dk[(kr * Hkv + kvh) * dqk + d] += scale * dz * rd(q, q_off + d, dtype);
          for (int64_t e = 0; e < dv; ++e)
            dv_out[(kr * Hkv + kvh) * dv + e] += P * dH[(r * HT + h) * dv + e];
        }
      }
    }
  }
  free(dH);
  free(lse);
  free(delta);
  return failed ? -8 : 0;
}

int gda_ref_threads(void) { return omp_get_max_threads(); }
