// gda_f32.hip - fp32 instance of the GDA/GDLA attention core (prefill and decode).
//
// Same operation as the bf16 kernels (Motif 3 technical-report walk-through,
// step 2 "GDLA forward", equation D_t, then the sigmoid gate), for fp32
// tensors, with no bf16 rounding anywhere: scores, softmax weights P and
// accumulators are all fp32.
//
// Prefill at head sizes (64,64), (128,128), (192,128): fwd_f32_mfma_kernel, on
// the fp32 matrix cores (v_mfma_f32_16x16x4_f32). A workgroup takes 16 query
// rows of one batch row and one noise head j with its g = S/N signal heads;
// wave 0 computes noise head j, every other wave one signal head, each a whole
// head in registers:
//   S^T = K Q^T (A = a 16-key tile, B = the wave's 16 query rows), so lane l
//   holds the scores of keys 4(l/16)..+3 of query row l%16; an online softmax
//   per row (the row's four lane groups combine with lane swaps); then
//   O^T += V^T P^T, whose B operand is P^T exactly as S^T left it in the
//   lanes, provided the k index of step s is key 4(l/16)+s (the A operand,
//   V^T, is loaded in that key order).
// The noise head's normalised output goes through LDS in the accumulator
// layout, so each signal wave reads back exactly its own lanes' rows and
// channels, then applies lambda and the gate and stores.
//
// Any other head size: fwd_f32_kernel, a plain VALU kernel (one thread per 16
// output channels of one (row, signal head)). Decode uses the VALU form too.
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
                            const float* __restrict__ gate, float* __restrict__ out, int flags) {
  if (flags & kLambdaLogits) lam = sigmoid_f32(lam);
  float hs[DCH], hn[DCH], ls, ln;
  attend_row_f32(r.qs, r.kbase, r.vbase, kstride, vstride, lo, hi, dqk, d0, nd, scale, hs, ls);
  attend_row_f32(r.qn, r.knb, r.vnb, kstride, vstride, lo, hi, dqk, d0, nd, scale, hn, ln);
  // A query at a negative position (packed sequences) has no visible key: zeros.
  const float is = ls > 0.f ? 1.f / ls : 0.f, in = ln > 0.f ? 1.f / ln : 0.f;
#pragma unroll
  for (int e = 0; e < DCH; ++e)
    if (e < nd) {
      const float gv = (flags & kGateLogits) ? sigmoid_f32(gate[d0 + e]) : gate[d0 + e];
      out[d0 + e] = gv * (hs[e] * is - lam * (hn[e] * in));
    }
}

__global__ void __launch_bounds__(NT)
fwd_f32_kernel(const float* __restrict__ q_sig, const float* __restrict__ q_noise,
               const float* __restrict__ kg, const float* __restrict__ vg,
               const float* __restrict__ lam, const float* __restrict__ gate,
               float* __restrict__ out, const int32_t* __restrict__ cu_q,
               const int32_t* __restrict__ cu_k, int B, int L, int S, int N, int Hkv, int dqk,
               int dv, int window, float scale, int flags) {
  const int nchunk = (dv + DCH - 1) / DCH;
  const int64_t total = (int64_t)B * L * S * nchunk;
  const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (gid >= total) return;
  const int ch = (int)(gid % nchunk);
  const int i = (int)((gid / nchunk) % S);
  const int64_t bt = gid / ((int64_t)nchunk * S);  // b*L + t
  const int b = (int)(bt / L), t = (int)(bt % L);
  // Sequence b (a batch row, or packed sequence b with its query offset).
  int64_t qbase = (int64_t)b * L, kbase = (int64_t)b * L;
  int Lq = L, Lk = L;
  if (cu_q) {
    qbase = cu_q[b];
    Lq = cu_q[b + 1] - cu_q[b];
    kbase = cu_k[b];
    Lk = cu_k[b + 1] - cu_k[b];
    if (t >= Lq) return;
  }
  const int64_t row = qbase + t;
  const int pos = Lk - Lq + t;  // key position of the query
  const int g = S / N;
  const int j = i / g;
  const int hs = (int)(((int64_t)i * Hkv) / S), hn = (int)(((int64_t)j * Hkv) / N);
  const int lo = window ? max(0, pos - window + 1) : 0;
  const int64_t kstride = (int64_t)Hkv * dqk, vstride = (int64_t)Hkv * dv;
  F32Row r;
  r.qs = q_sig + (row * S + i) * dqk;
  r.qn = q_noise + (row * N + j) * dqk;
  r.kbase = kg + kbase * kstride + (int64_t)hs * dqk;
  r.vbase = vg + kbase * vstride + (int64_t)hs * dv;
  r.knb = kg + kbase * kstride + (int64_t)hn * dqk;
  r.vnb = vg + kbase * vstride + (int64_t)hn * dv;
  const int d0 = ch * DCH;
  combine_f32(r, kstride, vstride, lo, pos, dqk, d0, min(DCH, dv - d0), scale, lam[row * S + i],
              gate + (row * S + i) * dv, out + (row * S + i) * dv, flags);
}

__global__ void __launch_bounds__(NT)
decode_f32_kernel(const float* __restrict__ q_sig, const float* __restrict__ q_noise,
                  const float* __restrict__ kg, const float* __restrict__ vg,
                  const int32_t* __restrict__ lens, const float* __restrict__ lam,
                  const float* __restrict__ gate, float* __restrict__ out, int B, int Lmax,
                  int S, int N, int Hkv, int dqk, int dv, int window, float scale, int flags) {
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
              gate + ((int64_t)b * S + i) * dv, o, flags);
}

// ---- fp32 MFMA prefill ---------------------------------------------------------

constexpr int MF_MAX_WAVES = 8;  // wave 0: noise head; waves 1..7: signal heads

__device__ __forceinline__ floatx4 mfma_16x16x4(float a, float b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// One head over 16 query rows: o[c] = normalised softmax(q k^T * scale) v, in
// the accumulator layout (lane l: row row0 + l%16, channels 16c + 4(l/16) .. +3).
// q points at query 0 of this head (row stride qstride floats), kb / vb at key 0
// of its KV head (key strides kstride / vstride); the sequence has Lq queries and
// Lk keys, query t at key position Lk - Lq + t. Rows >= Lq are computed on clamped
// (valid) addresses and never stored by the caller; a query at a negative position
// sees no key and gets zeros.
template <int DQK, int DV>
__device__ void head_f32(const float* __restrict__ q, int64_t qstride,
                         const float* __restrict__ kb, const float* __restrict__ vb,
                         int64_t kstride, int64_t vstride, int row0, int Lq, int Lk,
                         int window, float scale_log2, floatx4 (&o)[DV / 16]) {
  constexpr int QB = DQK / 16, VC = DV / 16;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int qoff = Lk - Lq;
  const int row = qoff + row0 + lr;  // the lane's query position
  const int L = Lk;
  // Dimension block sb of lane group lq is dims 16sb + 4lq .. +3; MFMA step
  // 4sb + e takes component e, for Q and K alike (the dot product's terms are
  // permuted the same way on both sides).
  float4 qv[QB];
  {
    const float* qr = q + (int64_t)min(row0 + lr, Lq - 1) * qstride + 4 * lq;
#pragma unroll
    for (int sb = 0; sb < QB; ++sb) qv[sb] = *(const float4*)(qr + 16 * sb);
  }
#pragma unroll
  for (int c = 0; c < VC; ++c) o[c] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;
  const int last = qoff + min(row0 + 15, Lq - 1);
  const int first = window ? max(0, qoff + row0 - window + 1) : 0;
  for (int key0 = first & ~15; key0 <= last; key0 += 16) {
    float4 kv[QB];
    {
      const float* kr = kb + (int64_t)min(key0 + lr, L - 1) * kstride + 4 * lq;
#pragma unroll
      for (int sb = 0; sb < QB; ++sb) kv[sb] = *(const float4*)(kr + 16 * sb);
    }
    float vv[4][VC];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const float* vr = vb + (int64_t)min(key0 + 4 * lq + st, L - 1) * vstride + lr;
#pragma unroll
      for (int c = 0; c < VC; ++c) vv[st][c] = vr[16 * c];
    }
    floatx4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sb = 0; sb < QB; ++sb) {
      sc = mfma_16x16x4(kv[sb].x, qv[sb].x, sc);
      sc = mfma_16x16x4(kv[sb].y, qv[sb].y, sc);
      sc = mfma_16x16x4(kv[sb].z, qv[sb].z, sc);
      sc = mfma_16x16x4(kv[sb].w, qv[sb].w, sc);
    }
    float z[4];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + 4 * lq + r;
      const bool vis = key <= row && (window == 0 || row - key < window);
      z[r] = vis ? sc[r] * scale_log2 : -INFINITY;
      mt = fmaxf(mt, z[r]);
    }
    mt = col_max4(mt);
    const float mn = fmaxf(m, mt);
    float p[4];
    float alpha = 1.f;
    if (mn == -INFINITY) {  // no key of this row visible yet
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = 0.f;
    } else {
      alpha = fast_exp2(m - mn);  // 0 when m is still -inf
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = fast_exp2(z[r] - mn);
    }
    lsum = lsum * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    m = mn;
#pragma unroll
    for (int c = 0; c < VC; ++c) {
      floatx4 acc = o[c] * alpha;
#pragma unroll
      for (int st = 0; st < 4; ++st) acc = mfma_16x16x4(vv[st][c], p[st], acc);
      o[c] = acc;
    }
  }
  const float tot = col_sum4(lsum);
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int c = 0; c < VC; ++c) o[c] = o[c] * inv;
}

template <int DQK, int DV>
__global__ void __launch_bounds__(64 * MF_MAX_WAVES)
fwd_f32_mfma_kernel(const float* __restrict__ q_sig, const float* __restrict__ q_noise,
                    const float* __restrict__ kg, const float* __restrict__ vg,
                    const float* __restrict__ lam, const float* __restrict__ gate,
                    float* __restrict__ out, const int32_t* __restrict__ cu_q,
                    const int32_t* __restrict__ cu_k, int B, int L, int S, int N, int Hkv,
                    int window, float scale_log2, int flags) {
  constexpr int VC = DV / 16;
  __shared__ floatx4 sHN[VC][64];
  const int ntiles = (L + 15) / 16;
  // Longest (latest) query tiles first.
  const int bid = blockIdx.x;
  const int j = bid % N;
  const int b = (bid / N) % B;
  const int tile = ntiles - 1 - bid / (N * B);
  const int row0 = tile * 16;
  // Sequence b (a batch row, or packed sequence b with its query offset).
  int64_t qbase = (int64_t)b * L, kbase = (int64_t)b * L;
  int Lq = L, Lk = L;
  if (cu_q) {
    qbase = cu_q[b];
    Lq = cu_q[b + 1] - cu_q[b];
    kbase = cu_k[b];
    Lk = cu_k[b + 1] - cu_k[b];
    if (row0 >= Lq) return;  // the whole workgroup
  }
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int lane = threadIdx.x & 63, lr = lane & 15, lq = lane >> 4;
  const int g = S / N;
  const int64_t kstride = (int64_t)Hkv * DQK, vstride = (int64_t)Hkv * DV;
  const float* kb0 = kg + kbase * kstride;
  const float* vb0 = vg + kbase * vstride;
  floatx4 o[VC];
  int i = -1;
  if (wave == 0) {
    const int hk = (int)(((int64_t)j * Hkv) / N);
    head_f32<DQK, DV>(q_noise + (qbase * N + j) * DQK, (int64_t)N * DQK,
                      kb0 + (int64_t)hk * DQK, vb0 + (int64_t)hk * DV, kstride, vstride, row0, Lq,
                      Lk, window, scale_log2, o);
#pragma unroll
    for (int c = 0; c < VC; ++c) sHN[c][lane] = o[c];
  } else {
    i = j * g + wave - 1;
    if (i < (j + 1) * g) {
      const int hk = (int)(((int64_t)i * Hkv) / S);
      head_f32<DQK, DV>(q_sig + (qbase * S + i) * DQK, (int64_t)S * DQK,
                        kb0 + (int64_t)hk * DQK, vb0 + (int64_t)hk * DV, kstride, vstride, row0,
                        Lq, Lk, window, scale_log2, o);
    }
  }
  __syncthreads();
  if (wave == 0) return;
  const int row = row0 + lr;
  for (; i < (j + 1) * g; i += nw - 1) {
    if (i != j * g + wave - 1) {  // heads beyond the first pass
      const int hk = (int)(((int64_t)i * Hkv) / S);
      head_f32<DQK, DV>(q_sig + (qbase * S + i) * DQK, (int64_t)S * DQK,
                        kb0 + (int64_t)hk * DQK, vb0 + (int64_t)hk * DV, kstride, vstride, row0,
                        Lq, Lk, window, scale_log2, o);
    }
    if (row < Lq) {
      const int64_t ri = (qbase + row) * S + i;
      const float li = (flags & kLambdaLogits) ? sigmoid_f32(lam[ri]) : lam[ri];
      const bool glog = (flags & kGateLogits) != 0;
      const float* gr = gate + ri * DV + 4 * lq;
      float* orow = out + ri * DV + 4 * lq;
#pragma unroll
      for (int c = 0; c < VC; ++c) {
        const floatx4 hn = sHN[c][lane];
        float4 gt = *(const float4*)(gr + 16 * c);
        if (glog) {
          gt.x = sigmoid_f32(gt.x);
          gt.y = sigmoid_f32(gt.y);
          gt.z = sigmoid_f32(gt.z);
          gt.w = sigmoid_f32(gt.w);
        }
        float4 y;
        y.x = gt.x * (o[c][0] - li * hn[0]);
        y.y = gt.y * (o[c][1] - li * hn[1]);
        y.z = gt.z * (o[c][2] - li * hn[2]);
        y.w = gt.w * (o[c][3] - li * hn[3]);
        *(float4*)(orow + 16 * c) = y;
      }
    }
  }
}

template <int DQK, int DV>
hipError_t launch_f32_mfma(const FwdArgs& a, hipStream_t stream) {
  const int g = a.S / a.N;
  const int nw = 1 + min(g, MF_MAX_WAVES - 1);
  const int64_t nblk = (int64_t)((a.L + 15) / 16) * a.B * a.N;
  if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_f32_mfma_kernel<DQK, DV>), dim3((unsigned)nblk), dim3(64 * nw), 0,
                     stream, (const float*)a.q_sig, (const float*)a.q_noise, (const float*)a.k,
                     (const float*)a.v, (const float*)a.lam, (const float*)a.gate,
                     (float*)a.out, a.cu_q, a.cu_k, a.B, a.L, a.S, a.N, a.Hkv, a.window,
                     a.scale_log2, a.flags);
  return hipGetLastError();
}

int64_t blocks_for(int64_t threads) { return (threads + NT - 1) / NT; }

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  if (a.dqk == 64 && a.dv == 64) return launch_f32_mfma<64, 64>(a, stream);
  if (a.dqk == 128 && a.dv == 128) return launch_f32_mfma<128, 128>(a, stream);
  if (a.dqk == 192 && a.dv == 128) return launch_f32_mfma<192, 128>(a, stream);
  const int64_t nblk = blocks_for((int64_t)a.B * a.L * a.S * ((a.dv + DCH - 1) / DCH));
  if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fwd_f32_kernel, dim3((unsigned)nblk), dim3(NT), 0, stream,
                     (const float*)a.q_sig, (const float*)a.q_noise, (const float*)a.k,
                     (const float*)a.v, (const float*)a.lam, (const float*)a.gate,
                     (float*)a.out, a.cu_q, a.cu_k, a.B, a.L, a.S, a.N, a.Hkv, a.dqk, a.dv,
                     a.window, a.scale, a.flags);
  return hipGetLastError();
}

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream) {
  const int64_t nblk = blocks_for((int64_t)a.B * a.S * ((a.dv + DCH - 1) / DCH));
  if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(decode_f32_kernel, dim3((unsigned)nblk), dim3(NT), 0, stream,
                     (const float*)a.q_sig, (const float*)a.q_noise, (const float*)a.k,
                     (const float*)a.v, a.lens, (const float*)a.lam, (const float*)a.gate,
                     (float*)a.out, a.B, a.Lmax, a.S, a.N, a.Hkv, a.dqk, a.dv, a.window,
                     a.scale, a.flags);
  return hipGetLastError();
}

}  // namespace gda
