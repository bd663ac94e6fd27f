// gda_fwd_bf16.hip - bf16 prefill kernel of the GDA/GDLA attention core (gfx950).
//
// Computes, for every query t of every sequence, the output the Motif 3
// technical-report walk-through (paper.rainbus.top, step 2 "GDLA forward",
// equation D_t) defines: each signal and noise head's softmax attention over
// the KV head it shares, the noise output repeated over its g signal heads,
// D = H_S - lambda * Repeat_g(H_N), and the gate product G * D.
//
// Work decomposition (MI355X-first; the pages give no kernel design):
//  * a workgroup owns (batch row b, unit u, tile of 64 queries); a unit is the
//    set of KV heads, signal heads and noise heads that the fused epilogue
//    needs together, so the noise output never leaves registers;
//  * 4 waves, each owning 16 queries for ALL heads of the current phase: every
//    K/V tile staged in LDS is read once per wave and used by every head;
//  * scores are computed transposed, S^T = K . Q^T (16x16x32 bf16 MFMA, fp32
//    accumulation), so a lane owns one query column: the online softmax row
//    max/sum is in-lane plus two permlane swaps;
//  * P^T in the accumulator layout is already the B operand of O^T = V^T . P^T;
//    V stays row-major in LDS and its transposed A operand comes from
//    ds_read_b64_tr_b16;
//  * lambda and the gate are applied to the fp32 accumulators in registers and
//    the result is rounded to bf16 once.
#include "gda_device.hpp"
#include "gda_kernels.hpp"

namespace gda {
namespace {

constexpr int BM = 64;  // queries per workgroup: 4 waves x 16
constexpr int BN = 64;  // keys per LDS tile
constexpr int NT = 256;

template <int DQK, int DV>
struct FwdTile {
  static constexpr int KS = DQK / 32;  // MFMA k-steps of Q.K
  static constexpr int DB = DV / 16;   // 16-wide blocks of the output channels
  // Row pads: K rows 16 B longer so the 16 rows of one ds_read_b128 fall on
  // distinct banks; V rows 32 B longer for the 16 rows of one transposed read.
  static constexpr int KROW = DQK + 8;
  static constexpr int VROW = DV + 16;
  static constexpr int KCH = DQK / 8;  // 16-byte chunks per K row
  static constexpr int VCH = DV / 8;
};

struct FwdCtx {
  const uint16_t* kg;
  const uint16_t* vg;
  int L, Hkv, window;
  int b;
  int q_lo, q_hi;  // the workgroup's query rows [q_lo, q_hi]
  int w_lo, w_hi;  // this wave's query rows (empty when w_lo > w_hi)
  int t;           // this lane's query row (may be >= L: then unused)
  int col, g4, tid;
  float c;  // log2(e)/sqrt(dqk)
};

// Stage keys [k0, k0+BN) of KV head kvh into LDS (rows past L are zero).
template <int DQK, int DV>
__device__ __forceinline__ void load_kv_tile(const FwdCtx& x, int kvh, int k0, uint16_t* sK,
                                             uint16_t* sV) {
  using T = FwdTile<DQK, DV>;
#pragma unroll
  for (int i = 0; i < (BN * T::KCH) / NT; ++i) {
    const int c = x.tid + i * NT;
    const int key = c / T::KCH, ch = c % T::KCH;
    const int ka = k0 + key;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (ka < x.L) val = ldg16(x.kg + (((int64_t)x.b * x.L + ka) * x.Hkv + kvh) * DQK + ch * 8);
    *(u32x4*)(sK + key * T::KROW + ch * 8) = val;
  }
#pragma unroll
  for (int i = 0; i < (BN * T::VCH) / NT; ++i) {
    const int c = x.tid + i * NT;
    const int key = c / T::VCH, ch = c % T::VCH;
    const int ka = k0 + key;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (ka < x.L) val = ldg16(x.vg + (((int64_t)x.b * x.L + ka) * x.Hkv + kvh) * DV + ch * 8);
    *(u32x4*)(sV + key * T::VROW + ch * 8) = val;
  }
}

// Lazy rescaling threshold (log2 units): a column's reference max is only
// raised when a score exceeds it by more than this, so P <= 2^8 and the
// accumulators are rarely rescaled. O/l does not depend on the reference.
constexpr float kRescaleTau = 8.f;
constexpr float kNoMax = -1e30f;  // finite "no key seen yet" reference

// One phase: NH query heads (row pointers qp, already at this lane's query row)
// attend over KV head kvh. On return o[h] holds the unnormalised O^T tile and
// lsum[h] the full softmax denominator of this lane's query.
template <int DQK, int DV, int NH>
__device__ __forceinline__ void attend(const FwdCtx& x, const uint16_t* const (&qp)[NH], int kvh,
                                       uint16_t* sK, uint16_t* sV,
                                       floatx4 (&o)[NH][DV / 16], float (&lsum)[NH]) {
  using T = FwdTile<DQK, DV>;
  bf16x8 qf[NH][T::KS];
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks)
      qf[h][ks] = __builtin_bit_cast(bf16x8, ldg16(qp[h] + ks * 32 + 8 * x.g4));

  float mref[NH];  // per column reference max, in log2 units (score * c)
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    mref[h] = kNoMax;
    lsum[h] = 0.f;
#pragma unroll
    for (int db = 0; db < T::DB; ++db) o[h][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const int W = x.window;
  const int k_lo = W ? max(0, x.q_lo - W + 1) : 0;
  const int kt0 = k_lo / BN, kt1 = x.q_hi / BN;
  const bool wave_active = x.w_lo <= x.w_hi;
  const int wk_lo = W ? max(0, x.w_lo - W + 1) : 0;

  for (int kt = kt0; kt <= kt1; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();
    load_kv_tile<DQK, DV>(x, kvh, k0, sK, sV);
    __syncthreads();
#pragma unroll 1
    for (int cc = 0; cc < BN / 32; ++cc) {
      const int c0 = k0 + 32 * cc;  // first key of this 32-key chunk
      if (!wave_active || c0 > x.w_hi || c0 + 31 < wk_lo) continue;
      const bool need_mask = (c0 + 31 > x.w_lo) || (W && c0 < x.w_hi - W + 1);

      // S^T = K . Q^T for 2 key blocks of 16.
      floatx4 s[NH][2];
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        s[h][0] = floatx4{0.f, 0.f, 0.f, 0.f};
        s[h][1] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a =
              *(const bf16x8*)(sK + (32 * cc + 16 * kb + x.col) * T::KROW + ks * 32 + 8 * x.g4);
#pragma unroll
          for (int h = 0; h < NH; ++h) s[h][kb] = mfma_16x16x32(a, qf[h][ks], s[h][kb]);
        }
      }

      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = c0 + 16 * kb + 4 * x.g4 + r;
            const bool vis = key <= x.t && (!W || x.t - key < W);
            if (!vis)
#pragma unroll
              for (int h = 0; h < NH; ++h) s[h][kb][r] = -INFINITY;
          }
      }

      // Online softmax per head; P^T packed to bf16 as the PV B operand.
      bf16x8 pb[NH];
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        float mx = fmaxf(fmaxf(fmaxf(s[h][0][0], s[h][0][1]), fmaxf(s[h][0][2], s[h][0][3])),
                         fmaxf(fmaxf(s[h][1][0], s[h][1][1]), fmaxf(s[h][1][2], s[h][1][3])));
        const bool grow = mx * x.c > mref[h] + kRescaleTau;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float cm = col_max4(mx) * x.c;  // -inf if the column saw no key here
          const float mnew = fmaxf(mref[h], cm);
          const float alpha = fast_exp2(mref[h] - mnew);
          mref[h] = mnew;
          lsum[h] *= alpha;
#pragma unroll
          for (int db = 0; db < T::DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[h][db][r] *= alpha;
        }
        const float nm = -mref[h];
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(fmaf(s[h][kb][r], x.c, nm));
            ps += p;
            pb[h][4 * kb + r] = (__bf16)p;
          }
        lsum[h] += ps;
      }

      // O^T += V^T . P^T over this chunk's 32 keys.
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
        const uint16_t* va =
            sV + (32 * cc + 4 * x.g4 + (x.col >> 2)) * T::VROW + 16 * db + 4 * (x.col & 3);
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)va);
        const shortx4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(va + 16 * T::VROW));
        typedef __attribute__((__vector_size__(8 * sizeof(short)))) short shortx8;
        const shortx8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x8 a = __builtin_bit_cast(bf16x8, a8);
#pragma unroll
        for (int h = 0; h < NH; ++h) o[h][db] = mfma_16x16x32(a, pb[h], o[h][db]);
      }
    }
  }

#pragma unroll
  for (int h = 0; h < NH; ++h) lsum[h] = col_sum4(lsum[h]);
}

// out[t, i, :] = gate * (hs - lam * hn) for one signal head, this lane's 4*DB channels.
template <int DV>
__device__ __forceinline__ void store_head(const uint16_t* lam, const uint16_t* gate,
                                           uint16_t* out, int64_t row, int S, int i, int g4,
                                           const floatx4 (&hs)[DV / 16], float inv_s,
                                           const float (&hn)[DV / 16][4]) {
  const float lm = bf16_to_f32(lam[row * S + i]);
  const int64_t base = (row * S + i) * DV + 4 * g4;
#pragma unroll
  for (int db = 0; db < DV / 16; ++db) {
    const u32x2 gw = ldg8(gate + base + 16 * db);
    const float d0 = hs[db][0] * inv_s - lm * hn[db][0];
    const float d1 = hs[db][1] * inv_s - lm * hn[db][1];
    const float d2 = hs[db][2] * inv_s - lm * hn[db][2];
    const float d3 = hs[db][3] * inv_s - lm * hn[db][3];
    u32x2 ow;
    ow[0] = pack_bf16x2(bf16_lo(gw[0]) * d0, bf16_hi(gw[0]) * d1);
    ow[1] = pack_bf16x2(bf16_lo(gw[1]) * d2, bf16_hi(gw[1]) * d3);
    *(u32x2*)(out + base + 16 * db) = ow;
  }
}

template <int DQK, int DV, int NS, int NN, int R>
__global__ void __launch_bounds__(NT, 1)
fwd_bf16_kernel(const uint16_t* __restrict__ q_sig, const uint16_t* __restrict__ q_noise,
                const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
                const uint16_t* __restrict__ lam, const uint16_t* __restrict__ gate,
                uint16_t* __restrict__ out, int B, int L, int S, int N, int Hkv, int window,
                int units, int nqt, int heavy_first, float c) {
  using T = FwdTile<DQK, DV>;
  constexpr int DB = T::DB;
  static_assert(R == 1 || NN == 1, "several phases only with one noise head per unit");
  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * T::KROW];
  __shared__ __attribute__((aligned(16))) uint16_t sV[BN * T::VROW];

  FwdCtx x;
  x.kg = kg;
  x.vg = vg;
  x.L = L;
  x.Hkv = Hkv;
  x.window = window;
  x.tid = threadIdx.x;
  const int wave = x.tid >> 6, lane = x.tid & 63;
  x.col = lane & 15;
  x.g4 = lane >> 4;
  x.c = c;
  const int per = B * units;
  const int slot = blockIdx.x / per;
  const int qt = heavy_first ? nqt - 1 - slot : slot;
  const int bu = blockIdx.x - slot * per;
  const int b = bu / units, u = bu - (bu / units) * units;
  x.b = b;
  x.q_lo = qt * BM;
  x.q_hi = min(x.q_lo + BM, L) - 1;
  x.w_lo = x.q_lo + wave * 16;
  x.w_hi = min(x.w_lo + 15, L - 1);
  x.t = x.w_lo + x.col;
  const bool t_ok = x.t < L;
  const int64_t row = (int64_t)b * L + min(x.t, L - 1);
  const int sig0 = u * (R * NS);  // first signal head of the unit

  float hn[DB][4];
  {
    constexpr int NH = NS + NN;
    const uint16_t* qp[NH];
#pragma unroll
    for (int s = 0; s < NS; ++s) qp[s] = q_sig + (row * S + sig0 + s) * DQK;
#pragma unroll
    for (int n = 0; n < NN; ++n) qp[NS + n] = q_noise + (row * N + u * NN + n) * DQK;
    floatx4 o[NH][DB];
    float l[NH];
    attend<DQK, DV, NH>(x, qp, u * R, sK, sV, o, l);
    constexpr int g = NS / NN;  // signal heads per noise head within the phase
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int n = s / g;
      const float inv_n = 1.f / l[NS + n];
      float hns[DB][4];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) hns[db][r] = o[NS + n][db][r] * inv_n;
      if (t_ok) store_head<DV>(lam, gate, out, row, S, sig0 + s, x.g4, o[s], 1.f / l[s], hns);
    }
    if (R > 1) {
      const float inv_n = 1.f / l[NS];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) hn[db][r] = o[NS][db][r] * inv_n;
    }
  }
#pragma unroll 1
  for (int ph = 1; ph < R; ++ph) {
    const uint16_t* qp[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) qp[s] = q_sig + (row * S + sig0 + ph * NS + s) * DQK;
    floatx4 o[NS][DB];
    float l[NS];
    attend<DQK, DV, NS>(x, qp, u * R + ph, sK, sV, o, l);
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if (t_ok) store_head<DV>(lam, gate, out, row, S, sig0 + ph * NS + s, x.g4, o[s], 1.f / l[s], hn);
  }
}

template <int DQK, int DV, int NS, int NN, int R>
hipError_t launch_inst(const FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.L + BM - 1) / BM;
  const int64_t grid = (int64_t)nqt * a.B * a.plan.units;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int heavy_first = a.window == 0 ? 1 : 0;
  hipLaunchKernelGGL((fwd_bf16_kernel<DQK, DV, NS, NN, R>), dim3((unsigned)grid), dim3(NT), 0,
                     stream, (const uint16_t*)a.q_sig, (const uint16_t*)a.q_noise,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.lam,
                     (const uint16_t*)a.gate, (uint16_t*)a.out, a.B, a.L, a.S, a.N, a.Hkv,
                     a.window, a.plan.units, nqt, heavy_first, a.scale_log2);
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t dispatch_layout(const FwdArgs& a, hipStream_t stream) {
  const UnitPlan& p = a.plan;
  if (p.NN != 1) return (hipError_t)-1;
  if (p.R == 1) {
    if (p.NS == 1) return launch_inst<DQK, DV, 1, 1, 1>(a, stream);
    if (p.NS == 2) return launch_inst<DQK, DV, 2, 1, 1>(a, stream);
    if (p.NS == 4) return launch_inst<DQK, DV, 4, 1, 1>(a, stream);
  } else if (p.R == 2) {
    if (p.NS == 1) return launch_inst<DQK, DV, 1, 1, 2>(a, stream);
    if (p.NS == 2) return launch_inst<DQK, DV, 2, 1, 2>(a, stream);
  }
  return (hipError_t)-1;
}

}  // namespace

bool fwd_bf16_supported(int dqk, int dv, const UnitPlan& p) {
  const bool dims = (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
  if (!dims || p.NN != 1) return false;
  if (p.R == 1) return p.NS == 1 || p.NS == 2 || p.NS == 4;
  if (p.R == 2) return p.NS == 1 || p.NS == 2;
  return false;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.dqk == 64 && a.dv == 64) return dispatch_layout<64, 64>(a, stream);
  if (a.dqk == 128 && a.dv == 128) return dispatch_layout<128, 128>(a, stream);
  if (a.dqk == 192 && a.dv == 128) return dispatch_layout<192, 128>(a, stream);
  return (hipError_t)-1;
}

}  // namespace gda
