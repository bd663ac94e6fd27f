// gda_api.cpp - host side of libgda: argument validation, head grouping, dispatch.
//
// Every argument is checked before the first HIP call, so a rejected call
// launches nothing and does not touch the device. No device memory is
// allocated and nothing is synchronised: kernels are enqueued on the caller's
// stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>

#include "../../include/gda.h"
#include "gda_kernels.hpp"

namespace {

thread_local char g_last_error[256] = "";

gda_status fail(gda_status st, const char* msg) {
  std::snprintf(g_last_error, sizeof g_last_error, "%s", msg);
  return st;
}

// Heads of one batch row grouped into units (the head maps of the Motif 3
// walk-through's GDLA forward, step 2, as read here: signal head i reads KV head
// floor(i*Hkv/S), noise head j reads KV head floor(j*Hkv/N), noise head j
// serves signal heads g*j .. g*j+g-1, g = S/N):
//  * Hkv >= N: unit j = noise head j, its g signal heads and KV heads
//    j*R .. j*R+R-1 (R = Hkv/N); phase p attends KV head j*R+p with the
//    NS = S/Hkv signal heads reading it, and phase 0 also with noise head j;
//  * N > Hkv: unit h = KV head h with its NS = S/Hkv signal heads and
//    NN = N/Hkv noise heads (one phase).
gda::UnitPlan make_plan(int S, int N, int Hkv) {
  gda::UnitPlan p;
  p.NS = S / Hkv;
  if (Hkv >= N) {
    p.units = N;
    p.NN = 1;
    p.R = Hkv / N;
  } else {
    p.units = Hkv;
    p.NN = N / Hkv;
    p.R = 1;
  }
  return p;
}

gda_status validate_common(int B, int L, int S, int N, int Hkv, int dqk, int dv, int window,
                           gda_dtype dtype) {
  if (B < 1 || L < 1 || S < 1 || N < 1 || Hkv < 1 || dqk < 1 || dv < 1)
    return fail(GDA_ERROR_INVALID_ARGUMENT, "every size must be >= 1");
  if (window < 0) return fail(GDA_ERROR_INVALID_ARGUMENT, "window must be >= 0");
  if (S % N != 0) return fail(GDA_ERROR_INVALID_ARGUMENT, "S must be a multiple of N");
  if (S % Hkv != 0) return fail(GDA_ERROR_INVALID_ARGUMENT, "S must be a multiple of Hkv");
  if (N % Hkv != 0 && Hkv % N != 0)
    return fail(GDA_ERROR_INVALID_ARGUMENT, "one of N, Hkv must divide the other");
  if (dtype != GDA_BF16 && dtype != GDA_F32)
    return fail(GDA_ERROR_INVALID_ARGUMENT, "unknown dtype");
  return GDA_SUCCESS;
}

gda_status check_bf16_dims(int dqk, int dv) {
  const bool ok = (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
  if (!ok) return fail(GDA_ERROR_UNSUPPORTED, "bf16 needs (dqk, dv) in {(64,64), (128,128), (192,128)}");
  return GDA_SUCCESS;
}

bool aligned(const void* p, uintptr_t bytes) { return ((uintptr_t)p & (bytes - 1)) == 0; }

gda_status check_alignment(const void* a, const void* b, const void* c, const void* d,
                           const void* e, const void* f, const void* g) {
  for (const void* p : {a, b, c, d, e, f, g})
    if (!aligned(p, 16)) return fail(GDA_ERROR_INVALID_ARGUMENT, "tensors must be 16-byte aligned");
  return GDA_SUCCESS;
}

// Options of the _ex calls -> softmax scale and kernel flags; NULL is the plain call.
gda_status apply_options(const gda_options* opts, int dqk, float* scale, float* scale_log2,
                         int* flags) {
  double sc = 1.0 / std::sqrt((double)dqk);
  uint32_t fl = 0;
  if (opts) {
    if (!(opts->softmax_scale >= 0.0f) || !std::isfinite(opts->softmax_scale))
      return fail(GDA_ERROR_INVALID_ARGUMENT, "softmax_scale must be 0 or a finite positive value");
    if (opts->flags & ~(uint32_t)(GDA_LAMBDA_LOGITS | GDA_GATE_LOGITS))
      return fail(GDA_ERROR_INVALID_ARGUMENT, "unknown option flags");
    if (opts->softmax_scale > 0.0f) sc = (double)opts->softmax_scale;
    fl = opts->flags;
  }
  *scale = (float)sc;
  *scale_log2 = (float)(1.4426950408889634 * sc);
  *flags = (int)fl;
  return GDA_SUCCESS;
}

gda_status from_hip(hipError_t e) {
  if (e == hipSuccess) {
    g_last_error[0] = '\0';
    return GDA_SUCCESS;
  }
  if (e == (hipError_t)-1) return fail(GDA_ERROR_UNSUPPORTED, "no compiled kernel instance");
  return fail(GDA_ERROR_HIP, hipGetErrorString(e));
}

// A device must exist before launching; hipGetDeviceCount is the first HIP call
// of a valid request.
gda_status require_device() {
  int n = 0;
  const hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n < 1) return fail(GDA_ERROR_HIP, "no HIP device available");
  return GDA_SUCCESS;
}

}  // namespace

extern "C" {

gda_status gda_fwd(const void* q_sig, const void* q_noise, const void* k, const void* v,
                   const void* lambda, const void* gate, void* out, int B, int L, int S, int N,
                   int Hkv, int dqk, int dv, int window, gda_dtype dtype, void* stream) {
  return gda_fwd_ex(q_sig, q_noise, k, v, lambda, gate, out, B, L, S, N, Hkv, dqk, dv, window,
                    dtype, nullptr, stream);
}

gda_status gda_fwd_ex(const void* q_sig, const void* q_noise, const void* k, const void* v,
                      const void* lambda, const void* gate, void* out, int B, int L, int S,
                      int N, int Hkv, int dqk, int dv, int window, gda_dtype dtype,
                      const gda_options* opts, void* stream) {
  if (!q_sig || !q_noise || !k || !v || !lambda || !gate || !out)
    return fail(GDA_ERROR_INVALID_ARGUMENT, "null tensor pointer");
  gda_status st = check_alignment(q_sig, q_noise, k, v, lambda, gate, out);
  if (st != GDA_SUCCESS) return st;
  st = validate_common(B, L, S, N, Hkv, dqk, dv, window, dtype);
  if (st != GDA_SUCCESS) return st;
  gda::FwdArgs a;
  a.q_sig = q_sig;
  a.q_noise = q_noise;
  a.k = k;
  a.v = v;
  a.lam = lambda;
  a.gate = gate;
  a.out = out;
  a.cu_q = nullptr;
  a.cu_k = nullptr;
  a.B = B;
  a.L = L;
  a.S = S;
  a.N = N;
  a.Hkv = Hkv;
  a.dqk = dqk;
  a.dv = dv;
  a.window = window;
  a.plan = make_plan(S, N, Hkv);
  if ((st = apply_options(opts, dqk, &a.scale, &a.scale_log2, &a.flags)) != GDA_SUCCESS)
    return st;
  if (dtype == GDA_BF16) {
    if ((st = check_bf16_dims(dqk, dv)) != GDA_SUCCESS) return st;
    if (!gda::fwd_bf16_supported(dqk, dv, a.plan))
      return fail(GDA_ERROR_UNSUPPORTED, "bf16 prefill: (dqk, dv) not compiled");
  }
  if ((st = require_device()) != GDA_SUCCESS) return st;
  const hipStream_t s = (hipStream_t)stream;
  return from_hip(dtype == GDA_BF16 ? gda::launch_fwd_bf16(a, s) : gda::launch_fwd_f32(a, s));
}

gda_status gda_decode(const void* q_sig, const void* q_noise, const void* k_cache,
                      const void* v_cache, const int32_t* cache_lens, const void* lambda,
                      const void* gate, void* out, int B, int Lmax, int S, int N, int Hkv,
                      int dqk, int dv, int window, gda_dtype dtype, void* stream) {
  return gda_decode_ex(q_sig, q_noise, k_cache, v_cache, cache_lens, lambda, gate, out, B, Lmax,
                       S, N, Hkv, dqk, dv, window, dtype, nullptr, stream);
}

gda_status gda_decode_ex(const void* q_sig, const void* q_noise, const void* k_cache,
                         const void* v_cache, const int32_t* cache_lens, const void* lambda,
                         const void* gate, void* out, int B, int Lmax, int S, int N, int Hkv,
                         int dqk, int dv, int window, gda_dtype dtype, const gda_options* opts,
                         void* stream) {
  if (!q_sig || !q_noise || !k_cache || !v_cache || !lambda || !gate || !out)
    return fail(GDA_ERROR_INVALID_ARGUMENT, "null tensor pointer");
  gda_status st = check_alignment(q_sig, q_noise, k_cache, v_cache, lambda, gate, out);
  if (st != GDA_SUCCESS) return st;
  if (!aligned(cache_lens, 4)) return fail(GDA_ERROR_INVALID_ARGUMENT, "cache_lens must be 4-byte aligned");
  st = validate_common(B, Lmax, S, N, Hkv, dqk, dv, window, dtype);
  if (st != GDA_SUCCESS) return st;
  gda::DecodeArgs a;
  a.q_sig = q_sig;
  a.q_noise = q_noise;
  a.k = k_cache;
  a.v = v_cache;
  a.lens = cache_lens;
  a.lam = lambda;
  a.gate = gate;
  a.out = out;
  a.B = B;
  a.Lmax = Lmax;
  a.S = S;
  a.N = N;
  a.Hkv = Hkv;
  a.dqk = dqk;
  a.dv = dv;
  a.window = window;
  a.plan = make_plan(S, N, Hkv);
  if ((st = apply_options(opts, dqk, &a.scale, &a.scale_log2, &a.flags)) != GDA_SUCCESS)
    return st;
  if (dtype == GDA_BF16) {
    if ((st = check_bf16_dims(dqk, dv)) != GDA_SUCCESS) return st;
    if (!gda::decode_bf16_supported(dqk, dv, a.plan))
      return fail(GDA_ERROR_UNSUPPORTED, "bf16 decode: (dqk, dv) not compiled");
  }
  if ((st = require_device()) != GDA_SUCCESS) return st;
  const hipStream_t s = (hipStream_t)stream;
  return from_hip(dtype == GDA_BF16 ? gda::launch_decode_bf16(a, s) : gda::launch_decode_f32(a, s));
}

gda_status gda_fwd_varlen(const void* q_sig, const void* q_noise, const void* k, const void* v,
                          const void* lambda, const void* gate, void* out,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                          int max_seqlen_q, int S, int N, int Hkv, int dqk, int dv, int window,
                          gda_dtype dtype, const gda_options* opts, void* stream) {
  if (!q_sig || !q_noise || !k || !v || !lambda || !gate || !out || !cu_seqlens_q ||
      !cu_seqlens_k)
    return fail(GDA_ERROR_INVALID_ARGUMENT, "null pointer");
  gda_status st = check_alignment(q_sig, q_noise, k, v, lambda, gate, out);
  if (st != GDA_SUCCESS) return st;
  if (!aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return fail(GDA_ERROR_INVALID_ARGUMENT, "cu_seqlens must be 4-byte aligned");
  st = validate_common(nseq, max_seqlen_q, S, N, Hkv, dqk, dv, window, dtype);
  if (st != GDA_SUCCESS) return st;
  gda::FwdArgs a;
  a.q_sig = q_sig;
  a.q_noise = q_noise;
  a.k = k;
  a.v = v;
  a.lam = lambda;
  a.gate = gate;
  a.out = out;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.B = nseq;
  a.L = max_seqlen_q;
  a.S = S;
  a.N = N;
  a.Hkv = Hkv;
  a.dqk = dqk;
  a.dv = dv;
  a.window = window;
  a.plan = make_plan(S, N, Hkv);
  if ((st = apply_options(opts, dqk, &a.scale, &a.scale_log2, &a.flags)) != GDA_SUCCESS)
    return st;
  if (dtype == GDA_BF16) {
    if ((st = check_bf16_dims(dqk, dv)) != GDA_SUCCESS) return st;
    if (!gda::fwd_bf16_supported(dqk, dv, a.plan))
      return fail(GDA_ERROR_UNSUPPORTED, "bf16 prefill: (dqk, dv) not compiled");
  }
  if ((st = require_device()) != GDA_SUCCESS) return st;
  const hipStream_t s = (hipStream_t)stream;
  return from_hip(dtype == GDA_BF16 ? gda::launch_fwd_bf16(a, s) : gda::launch_fwd_f32(a, s));
}

gda_status gda_fwd_train(const void* q_sig, const void* q_noise, const void* k, const void* v,
                         const void* lambda, const void* gate, void* out, void* h_sig,
                         void* h_noise, float* lse, int B, int L, int S, int N, int Hkv,
                         int dqk, int dv, int window, gda_dtype dtype, const gda_options* opts,
                         void* stream) {
  if (!q_sig || !q_noise || !k || !v || !lambda || !gate || !out || !h_sig || !h_noise || !lse)
    return fail(GDA_ERROR_INVALID_ARGUMENT, "null tensor pointer");
  gda_status st = check_alignment(q_sig, q_noise, k, v, lambda, gate, out);
  if (st != GDA_SUCCESS) return st;
  if (!aligned(h_sig, 16) || !aligned(h_noise, 16) || !aligned(lse, 4))
    return fail(GDA_ERROR_INVALID_ARGUMENT, "tensors must be 16-byte aligned (lse 4-byte)");
  st = validate_common(B, L, S, N, Hkv, dqk, dv, window, dtype);
  if (st != GDA_SUCCESS) return st;
  if (dtype != GDA_BF16) return fail(GDA_ERROR_UNSUPPORTED, "the training form is bf16 only");
  if ((st = check_bf16_dims(dqk, dv)) != GDA_SUCCESS) return st;
  gda::FwdArgs a;
  a.q_sig = q_sig;
  a.q_noise = q_noise;
  a.k = k;
  a.v = v;
  a.lam = lambda;
  a.gate = gate;
  a.out = out;
  a.cu_q = nullptr;
  a.cu_k = nullptr;
  a.B = B;
  a.L = L;
  a.S = S;
  a.N = N;
  a.Hkv = Hkv;
  a.dqk = dqk;
  a.dv = dv;
  a.window = window;
  a.plan = make_plan(S, N, Hkv);
  a.h_sig = h_sig;
  a.h_noise = h_noise;
  a.lse = lse;
  a.lse_b = (int64_t)(S + N) * L;  // lse [B, S+N, L]
  a.lse_q = 0;
  a.lse_h = L;
  if ((st = apply_options(opts, dqk, &a.scale, &a.scale_log2, &a.flags)) != GDA_SUCCESS)
    return st;
  if (!gda::fwd_bf16_supported(dqk, dv, a.plan))
    return fail(GDA_ERROR_UNSUPPORTED, "bf16 prefill: (dqk, dv) not compiled");
  if ((st = require_device()) != GDA_SUCCESS) return st;
  return from_hip(gda::launch_fwd_bf16(a, (hipStream_t)stream));
}

gda_status gda_fwd_train_varlen(const void* q_sig, const void* q_noise, const void* k,
                                const void* v, const void* lambda, const void* gate, void* out,
                                void* h_sig, void* h_noise, float* lse,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int nseq, int max_seqlen_q, int total_q, int S, int N, int Hkv,
                                int dqk, int dv, int window, gda_dtype dtype,
                                const gda_options* opts, void* stream) {
  if (!q_sig || !q_noise || !k || !v || !lambda || !gate || !out || !h_sig || !h_noise ||
      !lse || !cu_seqlens_q || !cu_seqlens_k)
    return fail(GDA_ERROR_INVALID_ARGUMENT, "null pointer");
  gda_status st = check_alignment(q_sig, q_noise, k, v, lambda, gate, out);
  if (st != GDA_SUCCESS) return st;
  if (!aligned(h_sig, 16) || !aligned(h_noise, 16) || !aligned(lse, 4) ||
      !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return fail(GDA_ERROR_INVALID_ARGUMENT,
                "h_sig, h_noise 16-byte, lse and cu_seqlens 4-byte aligned");
  st = validate_common(nseq, max_seqlen_q, S, N, Hkv, dqk, dv, window, dtype);
  if (st != GDA_SUCCESS) return st;
  if (total_q < 1) return fail(GDA_ERROR_INVALID_ARGUMENT, "total_q must be >= 1");
  if (dtype != GDA_BF16) return fail(GDA_ERROR_UNSUPPORTED, "the training form is bf16 only");
  if ((st = check_bf16_dims(dqk, dv)) != GDA_SUCCESS) return st;
  gda::FwdArgs a;
  a.q_sig = q_sig;
  a.q_noise = q_noise;
  a.k = k;
  a.v = v;
  a.lam = lambda;
  a.gate = gate;
  a.out = out;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.B = nseq;
  a.L = max_seqlen_q;
  a.S = S;
  a.N = N;
  a.Hkv = Hkv;
  a.dqk = dqk;
  a.dv = dv;
  a.window = window;
  a.plan = make_plan(S, N, Hkv);
  a.h_sig = h_sig;
  a.h_noise = h_noise;
  a.lse = lse;
  a.lse_b = 0;  // lse [S+N, total_q]
  a.lse_q = 1;
  a.lse_h = total_q;
  if ((st = apply_options(opts, dqk, &a.scale, &a.scale_log2, &a.flags)) != GDA_SUCCESS)
    return st;
  if (!gda::fwd_bf16_supported(dqk, dv, a.plan))
    return fail(GDA_ERROR_UNSUPPORTED, "bf16 prefill: (dqk, dv) not compiled");
  if ((st = require_device()) != GDA_SUCCESS) return st;
  return from_hip(gda::launch_fwd_bf16(a, (hipStream_t)stream));
}

size_t gda_bwd_workspace_bytes(int B, int L, int S, int N, int dv) {
  if (B < 1 || L < 1 || S < 1 || N < 1 || dv < 1) return 0;
  return gda::bwd_workspace_bytes(B, L, S, N, dv);
}

gda_status gda_bwd(const void* q_sig, const void* q_noise, const void* k, const void* v,
                   const void* lambda, const void* gate, const void* h_sig, const void* h_noise,
                   const float* lse, const void* d_out, void* dq_sig, void* dq_noise, void* dk,
                   void* dv_out, void* dlambda, void* dgate, int B, int L, int S, int N, int Hkv,
                   int dqk, int dv, int window, gda_dtype dtype, const gda_options* opts,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!q_sig || !q_noise || !k || !v || !lambda || !gate || !h_sig || !h_noise || !lse ||
      !d_out || !dq_sig || !dq_noise || !dk || !dv_out || !dlambda || !dgate || !workspace)
    return fail(GDA_ERROR_INVALID_ARGUMENT, "null pointer");
  gda_status st = check_alignment(q_sig, q_noise, k, v, lambda, gate, h_sig);
  if (st != GDA_SUCCESS) return st;
  if ((st = check_alignment(h_noise, d_out, dq_sig, dq_noise, dk, dv_out, dgate)) != GDA_SUCCESS)
    return st;
  if (!aligned(dlambda, 16) || !aligned(workspace, 256) || !aligned(lse, 4))
    return fail(GDA_ERROR_INVALID_ARGUMENT,
                "dlambda must be 16-byte, workspace 256-byte, lse 4-byte aligned");
  st = validate_common(B, L, S, N, Hkv, dqk, dv, window, dtype);
  if (st != GDA_SUCCESS) return st;
  if (workspace_bytes < gda::bwd_workspace_bytes(B, L, S, N, dv))
    return fail(GDA_ERROR_INVALID_ARGUMENT, "workspace smaller than gda_bwd_workspace_bytes");
  gda::BwdArgs a;
  a.q_sig = q_sig;
  a.q_noise = q_noise;
  a.k = k;
  a.v = v;
  a.lam = lambda;
  a.gate = gate;
  a.h_sig = h_sig;
  a.h_noise = h_noise;
  a.lse = lse;
  a.d_out = d_out;
  a.dq_sig = dq_sig;
  a.dq_noise = dq_noise;
  a.dk = dk;
  a.dv_out = dv_out;
  a.dlam = dlambda;
  a.dgate = dgate;
  a.workspace = workspace;
  a.B = B;
  a.L = L;
  a.S = S;
  a.N = N;
  a.Hkv = Hkv;
  a.dqk = dqk;
  a.dv = dv;
  a.window = window;
  a.Lk_max = L;
  a.rows = (int64_t)B * L;
  a.lse_b = (int64_t)(S + N) * L;  // lse and delta [B, S+N, L]
  a.lse_q = 0;
  a.lse_h = L;
  if ((st = apply_options(opts, dqk, &a.scale, &a.scale_log2, &a.flags)) != GDA_SUCCESS)
    return st;
  if (dtype != GDA_BF16) return fail(GDA_ERROR_UNSUPPORTED, "the backward is bf16 only");
  if ((st = check_bf16_dims(dqk, dv)) != GDA_SUCCESS) return st;
  if ((st = require_device()) != GDA_SUCCESS) return st;
  return from_hip(gda::launch_bwd_bf16(a, (hipStream_t)stream));
}

gda_status gda_bwd_varlen(const void* q_sig, const void* q_noise, const void* k, const void* v,
                          const void* lambda, const void* gate, const void* h_sig,
                          const void* h_noise, const float* lse, const void* d_out,
                          void* dq_sig, void* dq_noise, void* dk, void* dv_out, void* dlambda,
                          void* dgate, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          int nseq, int max_seqlen_q, int max_seqlen_k, int total_q, int S,
                          int N, int Hkv, int dqk, int dv, int window, gda_dtype dtype,
                          const gda_options* opts, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (!q_sig || !q_noise || !k || !v || !lambda || !gate || !h_sig || !h_noise || !lse ||
      !d_out || !dq_sig || !dq_noise || !dk || !dv_out || !dlambda || !dgate || !workspace ||
      !cu_seqlens_q || !cu_seqlens_k)
    return fail(GDA_ERROR_INVALID_ARGUMENT, "null pointer");
  gda_status st = check_alignment(q_sig, q_noise, k, v, lambda, gate, h_sig);
  if (st != GDA_SUCCESS) return st;
  if ((st = check_alignment(h_noise, d_out, dq_sig, dq_noise, dk, dv_out, dgate)) != GDA_SUCCESS)
    return st;
  if (!aligned(dlambda, 16) || !aligned(workspace, 256) || !aligned(lse, 4) ||
      !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return fail(GDA_ERROR_INVALID_ARGUMENT,
                "dlambda must be 16-byte, workspace 256-byte, lse and cu_seqlens 4-byte aligned");
  st = validate_common(nseq, max_seqlen_q, S, N, Hkv, dqk, dv, window, dtype);
  if (st != GDA_SUCCESS) return st;
  if (max_seqlen_k < 1 || total_q < 1)
    return fail(GDA_ERROR_INVALID_ARGUMENT, "max_seqlen_k and total_q must be >= 1");
  if (workspace_bytes < gda::bwd_workspace_bytes(1, total_q, S, N, dv))
    return fail(GDA_ERROR_INVALID_ARGUMENT,
                "workspace smaller than gda_bwd_workspace_bytes(1, total_q, ...)");
  gda::BwdArgs a;
  a.q_sig = q_sig;
  a.q_noise = q_noise;
  a.k = k;
  a.v = v;
  a.lam = lambda;
  a.gate = gate;
  a.h_sig = h_sig;
  a.h_noise = h_noise;
  a.lse = lse;
  a.d_out = d_out;
  a.dq_sig = dq_sig;
  a.dq_noise = dq_noise;
  a.dk = dk;
  a.dv_out = dv_out;
  a.dlam = dlambda;
  a.dgate = dgate;
  a.workspace = workspace;
  a.B = nseq;
  a.L = max_seqlen_q;
  a.S = S;
  a.N = N;
  a.Hkv = Hkv;
  a.dqk = dqk;
  a.dv = dv;
  a.window = window;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.Lk_max = max_seqlen_k;
  a.rows = total_q;
  a.lse_b = 0;  // lse and delta [S+N, total_q]
  a.lse_q = 1;
  a.lse_h = total_q;
  if ((st = apply_options(opts, dqk, &a.scale, &a.scale_log2, &a.flags)) != GDA_SUCCESS)
    return st;
  if (dtype != GDA_BF16) return fail(GDA_ERROR_UNSUPPORTED, "the backward is bf16 only");
  if ((st = check_bf16_dims(dqk, dv)) != GDA_SUCCESS) return st;
  if ((st = require_device()) != GDA_SUCCESS) return st;
  return from_hip(gda::launch_bwd_bf16(a, (hipStream_t)stream));
}

size_t gda_decode_latent_workspace_bytes(int B, int Lmax, int S, int N, int window) {
  if (B < 1 || Lmax < 1 || S < 1 || N < 1 || window < 0) return 0;
  return gda::latent_workspace_bytes(B, Lmax, S, N, window);
}

}  // extern "C"

namespace {

// Validation and argument packing shared by the two latent-decode entry points.
gda_status latent_prepare(const void* q_sig, const void* q_noise, const void* c_kv,
                          const void* k_rope, const void* w_kv_b, const int32_t* cache_lens,
                          const void* lambda, const void* gate, void* out, int B, int Lmax,
                          int S, int N, int Hkv, int Dn, int Dr, int Dc, int dv, int window,
                          gda_dtype dtype, const gda_options* opts, gda::LatentArgs* a) {
  if (!q_sig || !q_noise || !c_kv || !k_rope || !w_kv_b || !lambda || !gate || !out)
    return fail(GDA_ERROR_INVALID_ARGUMENT, "null tensor pointer");
  gda_status st = check_alignment(q_sig, q_noise, c_kv, k_rope, w_kv_b, lambda, gate);
  if (st != GDA_SUCCESS) return st;
  if (!aligned(out, 16)) return fail(GDA_ERROR_INVALID_ARGUMENT, "tensors must be 16-byte aligned");
  if (!aligned(cache_lens, 4)) return fail(GDA_ERROR_INVALID_ARGUMENT, "cache_lens must be 4-byte aligned");
  if (Dn < 1 || Dr < 0 || Dc < 1)
    return fail(GDA_ERROR_INVALID_ARGUMENT, "every size must be >= 1 (Dr >= 0)");
  st = validate_common(B, Lmax, S, N, Hkv, Dn + Dr, dv, window, dtype);
  if (st != GDA_SUCCESS) return st;
  a->q_sig = q_sig;
  a->q_noise = q_noise;
  a->c_kv = c_kv;
  a->k_rope = k_rope;
  a->w_kv_b = w_kv_b;
  a->lens = cache_lens;
  a->lam = lambda;
  a->gate = gate;
  a->out = out;
  a->workspace = nullptr;
  a->B = B;
  a->Lmax = Lmax;
  a->S = S;
  a->N = N;
  a->Hkv = Hkv;
  a->window = window;
  float scale = 0.f;
  if ((st = apply_options(opts, Dn + Dr, &scale, &a->scale_log2, &a->flags)) != GDA_SUCCESS)
    return st;
  if (dtype != GDA_BF16) return fail(GDA_ERROR_UNSUPPORTED, "latent decode: bf16 only");
  if (!gda::latent_supported(Dn, Dr, Dc, dv, S, N, Hkv))
    return fail(GDA_ERROR_UNSUPPORTED,
                "latent decode: needs (Dn,Dr,Dc,dv) = (128,64,512,128), S+N <= 128, "
                "g <= 15 and <= 16 query heads per KV head");
  return GDA_SUCCESS;
}

}  // namespace

extern "C" {

gda_status gda_decode_latent(const void* q_sig, const void* q_noise, const void* c_kv,
                             const void* k_rope, const void* w_kv_b, const int32_t* cache_lens,
                             const void* lambda, const void* gate, void* out, int B, int Lmax,
                             int S, int N, int Hkv, int Dn, int Dr, int Dc, int dv, int window,
                             gda_dtype dtype, const gda_options* opts, void* workspace,
                             size_t workspace_bytes, void* stream) {
  gda::LatentArgs a;
  gda_status st = latent_prepare(q_sig, q_noise, c_kv, k_rope, w_kv_b, cache_lens, lambda, gate,
                                 out, B, Lmax, S, N, Hkv, Dn, Dr, Dc, dv, window, dtype, opts, &a);
  if (st != GDA_SUCCESS) return st;
  if (!workspace || !aligned(workspace, 16))
    return fail(GDA_ERROR_INVALID_ARGUMENT, "latent decode: workspace missing or misaligned");
  if (workspace_bytes < gda::latent_workspace_bytes(B, Lmax, S, N, window))
    return fail(GDA_ERROR_INVALID_ARGUMENT, "latent decode: workspace too small");
  a.workspace = workspace;
  if ((st = require_device()) != GDA_SUCCESS) return st;
  return from_hip(gda::launch_decode_latent(a, (hipStream_t)stream));
}

gda_status gda_decode_latent_noalloc(const void* q_sig, const void* q_noise, const void* c_kv,
                                     const void* k_rope, const void* w_kv_b,
                                     const int32_t* cache_lens, const void* lambda,
                                     const void* gate, void* out, int B, int Lmax, int S, int N,
                                     int Hkv, int Dn, int Dr, int Dc, int dv, int window,
                                     gda_dtype dtype, const gda_options* opts, void* stream) {
  gda::LatentArgs a;
  gda_status st = latent_prepare(q_sig, q_noise, c_kv, k_rope, w_kv_b, cache_lens, lambda, gate,
                                 out, B, Lmax, S, N, Hkv, Dn, Dr, Dc, dv, window, dtype, opts, &a);
  if (st != GDA_SUCCESS) return st;
  if (gda::latent_workspace_bytes(B, Lmax, S, N, window) > GDA_DECODE_LATENT_SCRATCH_BYTES)
    return fail(GDA_ERROR_INVALID_ARGUMENT,
                "latent decode (no allocation): these sizes need more scratch than the "
                "static GDA_DECODE_LATENT_SCRATCH_BYTES; use gda_decode_latent with a workspace");
  if ((st = require_device()) != GDA_SUCCESS) return st;
  void* scratch = nullptr;
  const hipError_t e = gda::latent_scratch(&scratch);
  if (e != hipSuccess) return from_hip(e);
  a.workspace = scratch;
  return from_hip(gda::launch_decode_latent(a, (hipStream_t)stream));
}

const char* gda_status_string(gda_status s) {
  switch (s) {
    case GDA_SUCCESS:
      return "GDA_SUCCESS";
    case GDA_ERROR_INVALID_ARGUMENT:
      return "GDA_ERROR_INVALID_ARGUMENT";
    case GDA_ERROR_UNSUPPORTED:
      return "GDA_ERROR_UNSUPPORTED";
    case GDA_ERROR_HIP:
      return "GDA_ERROR_HIP";
  }
  return "GDA_UNKNOWN_STATUS";
}

const char* gda_last_error(void) { return g_last_error; }

}  // extern "C"
