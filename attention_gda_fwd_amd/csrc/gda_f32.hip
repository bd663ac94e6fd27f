// gda_f32.hip - fp32 instance of the GDA/GDLA attention core (prefill and decode).
//
// Same operation as the bf16 kernels (Motif 3 technical-report walk-through,
// step 2 "GDLA forward", equation D_t, then the sigmoid gate), for fp32
// tensors. It exists for fp32 callers and for checking the method at full fp32
// precision; it is a plain VALU kernel (fp32 FMA, fp32 softmax, no bf16
// rounding anywhere), not the tuned path. Any head layout the API accepts
// works here.
//
// One thread computes 16 output channels of one (query row, signal head): it
// streams the visible keys twice, once with the signal query and once with the
// noise query of its group, each with an online softmax, and combines them.
#include "gda_device.hpp"
#include "gda_kernels.hpp"

namespace gda {
namespace {

constexpr int NT = 256;
constexpr int DCH = 16;  // output channels per thread

// softmax(q . k_s * scale) weighted sum of v_s[d0 .. d0+DCH) over keys [lo, hi].
__device__ void attend_row_f32(const float* __restrict__ q, const float* __restrict__ kbase,
                               const float* __restrict__ vbase, int64_t kstride,
                               int64_t vstride, int lo, int hi, int dqk, int d0, int nd,
                               float scale, float (&acc)[DCH], float& l) {
  float m = -INFINITY;
  l = 0.f;
#pragma unroll
  for (int e = 0; e < DCH; ++e) acc[e] = 0.f;
  for (int s = lo; s <= hi; ++s) {
    const float* kr = kbase + s * kstride;
    float dot = 0.f;
    for (int d = 0; d < dqk; ++d) dot = fmaf(q[d], kr[d], dot);
    const float z = dot * scale;
    if (z > m) {
      const float alpha = expf(m - z);  // exp(-inf) = 0 on the first key
      l *= alpha;
#pragma unroll
      for (int e = 0; e < DCH; ++e) acc[e] *= alpha;
      m = z;
    }
    const float p = expf(z - m);
    l += p;
    const float* vr = vbase + s * vstride + d0;
#pragma unroll
    for (int e = 0; e < DCH; ++e)
      if (e < nd) acc[e] = fmaf(p, vr[e], acc[e]);
  }
}

struct F32Row {
  const float* qs;    // signal query row of head i
  const float* qn;    // noise query row of head grp(i)
  const float* kbase; // key 0 of the signal head's KV head
  const float* vbase;
  const float* knb;   // key 0 of the noise head's KV head
  const float* vnb;
};

__device__ void combine_f32(const F32Row& r, int64_t kstride, int64_t vstride, int lo, int hi,
                            int dqk, int d0, int nd, float scale, float lam,
                            const float* __restrict__ gate, float* __restrict__ out) {
  float hs[DCH], hn[DCH], ls, ln;
  attend_row_f32(r.qs, r.kbase, r.vbase, kstride, vstride, lo, hi, dqk, d0, nd, scale, hs, ls);
  attend_row_f32(r.qn, r.knb, r.vnb, kstride, vstride, lo, hi, dqk, d0, nd, scale, hn, ln);
  const float is = 1.f / ls, in = 1.f / ln;
#pragma unroll
  for (int e = 0; e < DCH; ++e)
    if (e < nd) out[d0 + e] = gate[d0 + e] * (hs[e] * is - lam * (hn[e] * in));
}

__global__ void __launch_bounds__(NT)
fwd_f32_kernel(const float* __restrict__ q_sig, const float* __restrict__ q_noise,
               const float* __restrict__ kg, const float* __restrict__ vg,
               const float* __restrict__ lam, const float* __restrict__ gate,
               float* __restrict__ out, int B, int L, int S, int N, int Hkv, int dqk, int dv,
               int window, float scale) {
  const int nchunk = (dv + DCH - 1) / DCH;
  const int64_t total = (int64_t)B * L * S * nchunk;
  const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (gid >= total) return;
  const int ch = (int)(gid % nchunk);
  const int i = (int)((gid / nchunk) % S);
  const int64_t row = gid / ((int64_t)nchunk * S);  // b*L + t
  const int b = (int)(row / L), t = (int)(row % L);
  const int g = S / N;
  const int j = i / g;
  const int hs = (int)(((int64_t)i * Hkv) / S), hn = (int)(((int64_t)j * Hkv) / N);
  const int lo = window ? max(0, t - window + 1) : 0;
  const int64_t kstride = (int64_t)Hkv * dqk, vstride = (int64_t)Hkv * dv;
  F32Row r;
  r.qs = q_sig + (row * S + i) * dqk;
  r.qn = q_noise + (row * N + j) * dqk;
  r.kbase = kg + (int64_t)b * L * kstride + (int64_t)hs * dqk;
  r.vbase = vg + (int64_t)b * L * vstride + (int64_t)hs * dv;
  r.knb = kg + (int64_t)b * L * kstride + (int64_t)hn * dqk;
  r.vnb = vg + (int64_t)b * L * vstride + (int64_t)hn * dv;
  const int d0 = ch * DCH;
  combine_f32(r, kstride, vstride, lo, t, dqk, d0, min(DCH, dv - d0), scale, lam[row * S + i],
              gate + (row * S + i) * dv, out + (row * S + i) * dv);
}

__global__ void __launch_bounds__(NT)
decode_f32_kernel(const float* __restrict__ q_sig, const float* __restrict__ q_noise,
                  const float* __restrict__ kg, const float* __restrict__ vg,
                  const int32_t* __restrict__ lens, const float* __restrict__ lam,
                  const float* __restrict__ gate, float* __restrict__ out, int B, int Lmax,
                  int S, int N, int Hkv, int dqk, int dv, int window, float scale) {
  const int nchunk = (dv + DCH - 1) / DCH;
  const int64_t total = (int64_t)B * S * nchunk;
  const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (gid >= total) return;
  const int ch = (int)(gid % nchunk);
  const int i = (int)((gid / nchunk) % S);
  const int b = (int)(gid / ((int64_t)nchunk * S));
  const int d0 = ch * DCH, nd = min(DCH, dv - d0);
  float* o = out + ((int64_t)b * S + i) * dv;
  int len = lens ? lens[b] : Lmax;
  if (len > Lmax) len = Lmax;
  if (len < 1) {
    for (int e = 0; e < nd; ++e) o[d0 + e] = 0.f;
    return;
  }
  const int pos = len - 1;
  const int g = S / N;
  const int j = i / g;
  const int hs = (int)(((int64_t)i * Hkv) / S), hn = (int)(((int64_t)j * Hkv) / N);
  const int lo = window ? max(0, pos - window + 1) : 0;
  const int64_t kstride = (int64_t)Hkv * dqk, vstride = (int64_t)Hkv * dv;
  F32Row r;
  r.qs = q_sig + ((int64_t)b * S + i) * dqk;
  r.qn = q_noise + ((int64_t)b * N + j) * dqk;
  r.kbase = kg + (int64_t)b * Lmax * kstride + (int64_t)hs * dqk;
  r.vbase = vg + (int64_t)b * Lmax * vstride + (int64_t)hs * dv;
  r.knb = kg + (int64_t)b * Lmax * kstride + (int64_t)hn * dqk;
  r.vnb = vg + (int64_t)b * Lmax * vstride + (int64_t)hn * dv;
  combine_f32(r, kstride, vstride, lo, pos, dqk, d0, nd, scale, lam[(int64_t)b * S + i],
              gate + ((int64_t)b * S + i) * dv, o);
}

int64_t blocks_for(int64_t threads) { return (threads + NT - 1) / NT; }

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  const int64_t nblk = blocks_for((int64_t)a.B * a.L * a.S * ((a.dv + DCH - 1) / DCH));
  if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fwd_f32_kernel, dim3((unsigned)nblk), dim3(NT), 0, stream,
                     (const float*)a.q_sig, (const float*)a.q_noise, (const float*)a.k,
                     (const float*)a.v, (const float*)a.lam, (const float*)a.gate,
                     (float*)a.out, a.B, a.L, a.S, a.N, a.Hkv, a.dqk, a.dv, a.window, a.scale);
  return hipGetLastError();
}

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream) {
  const int64_t nblk = blocks_for((int64_t)a.B * a.S * ((a.dv + DCH - 1) / DCH));
  if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(decode_f32_kernel, dim3((unsigned)nblk), dim3(NT), 0, stream,
                     (const float*)a.q_sig, (const float*)a.q_noise, (const float*)a.k,
                     (const float*)a.v, a.lens, (const float*)a.lam, (const float*)a.gate,
                     (float*)a.out, a.B, a.Lmax, a.S, a.N, a.Hkv, a.dqk, a.dv, a.window,
                     a.scale);
  return hipGetLastError();
}

}  // namespace gda
