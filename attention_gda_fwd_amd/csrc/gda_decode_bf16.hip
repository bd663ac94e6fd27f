// gda_decode_bf16.hip - bf16 split-KV decode kernel of the GDA/GDLA attention core (gfx950).
//
// One new query token per sequence attends over a KV cache that already holds
// it (the overview page's inference notes enable a KV cache; the Motif 3
// walk-through, novelty point one, notes GDLA's cache is MLA-sized because both
// query paths share the KV heads). The output is the D_t of the Motif 3
// walk-through (step 2) times the gate, as in prefill.
//
// Work decomposition: one workgroup per (sequence b, unit u). Its 4 waves split
// the visible key range into contiguous slices; each wave streams its slice
// straight from HBM (K fragments go global -> VGPR -> MFMA A operand; V rows go
// through a wave-private LDS tile and come back transposed with
// ds_read_b64_tr_b16), keeping a partial (max, sum, O^T) per query head. All
// query heads of the unit are the 16 columns of one 16x16 MFMA tile (unused
// columns are zero queries), so each K/V byte is read once for all of them.
// The partials are merged through LDS and the lambda/gate epilogue writes
// coalesced rows.
#include "gda_device.hpp"
#include "gda_kernels.hpp"

namespace gda {
namespace {

constexpr int NW = 4;           // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int CK = 32;          // keys per chunk
constexpr float kNoMax = -1e30f;

template <int DQK, int DV>
struct DecTile {
  static constexpr int KS = DQK / 32;
  static constexpr int DB = DV / 16;
  static constexpr int VROW = DV + 16;   // padded row of the V staging tile
  static constexpr int VCH = DV / 8;     // 16-byte chunks per V row
  static constexpr int STAGE = CK * VROW;            // elements per wave stage
  // merge area per wave: m[16], l[16], O^T[DV][16]
  static constexpr int MERGE_FLOATS = 32 + DV * 16;
  static constexpr int STAGE_BYTES = NW * STAGE * 2;
  static constexpr int MERGE_BYTES = NW * MERGE_FLOATS * 4;
  static constexpr int SHARED_BYTES = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
};

// Normalised output of column h, channel d, from the waves' partials in LDS:
// m* = max_w m_w, H = sum_w 2^(m_w - m*) O_w / sum_w 2^(m_w - m*) l_w.
template <int MERGE_FLOATS>
__device__ __forceinline__ float merged_impl(const float* merge, int h, int d) {
  float ms = kNoMax;
#pragma unroll
  for (int w = 0; w < NW; ++w) ms = fmaxf(ms, merge[w * MERGE_FLOATS + h]);
  float ls = 0.f, acc = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float* m2 = merge + w * MERGE_FLOATS;
    const float e = fast_exp2(m2[h] - ms);
    ls += e * m2[16 + h];
    acc += e * m2[32 + d * 16 + h];
  }
  return acc / ls;
}

// 4 waves per SIMD (<= 128 VGPRs) so that 4 workgroups share a CU and a
// B x units = 1024-workgroup grid is resident at once on 256 CUs.
template <int DQK, int DV>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4, 4)))
decode_bf16_kernel(const uint16_t* __restrict__ q_sig, const uint16_t* __restrict__ q_noise,
                   const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
                   const int32_t* __restrict__ lens, const uint16_t* __restrict__ lam,
                   const uint16_t* __restrict__ gate, uint16_t* __restrict__ out, int Lmax,
                   int S, int N, int Hkv, int window, int units, int NS, int NN, int R, float c) {
  using T = DecTile<DQK, DV>;
  constexpr int DB = T::DB;
  __shared__ __attribute__((aligned(16))) unsigned char smem[T::SHARED_BYTES];
  __shared__ float sHN[DV];  // the unit's noise output, kept across phases when R > 1

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, g4 = lane >> 4;
  const int b = blockIdx.x / units, u = blockIdx.x - (blockIdx.x / units) * units;
  const int sig0 = u * R * NS;

  int len = lens ? lens[b] : Lmax;
  if (len > Lmax) len = Lmax;
  if (len < 1) {  // no visible key: the output row is zero
    for (int idx = tid; idx < R * NS * DV; idx += NT)
      out[((int64_t)b * S + sig0 + idx / DV) * DV + idx % DV] = 0;
    return;
  }
  const int pos = len - 1;
  const int lo = window ? max(0, pos - window + 1) : 0;
  const int nch = (pos - lo + CK) / CK;
  const int ch0 = (int)(((int64_t)wave * nch) / NW), ch1 = (int)(((int64_t)(wave + 1) * nch) / NW);

  uint16_t* stage = (uint16_t*)smem + wave * T::STAGE;
  float* merge = (float*)smem;
  auto merged = [](const float* mg, int h, int d) { return merged_impl<T::MERGE_FLOATS>(mg, h, d); };

#pragma unroll 1
  for (int ph = 0; ph < R; ++ph) {
    const int nh = ph == 0 ? NS + NN : NS;  // query heads (MFMA columns) of this phase
    const int kvh = u * R + ph;
    // Q^T B operand: column col is head col of the phase (zero if unused).
    bf16x8 qf[T::KS];
    {
      const uint16_t* qp = nullptr;
      if (col < NS)
        qp = q_sig + ((int64_t)b * S + sig0 + ph * NS + col) * DQK;
      else if (col < nh)
        qp = q_noise + ((int64_t)b * N + u * NN + (col - NS)) * DQK;
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (qp) w = ldg16(qp + ks * 32 + 8 * g4);
        qf[ks] = __builtin_bit_cast(bf16x8, w);
      }
    }
    const int64_t kbase = ((int64_t)b * Lmax * Hkv + kvh) * DQK;  // key s at kbase + s*Hkv*DQK
    const int64_t vbase = ((int64_t)b * Lmax * Hkv + kvh) * DV;
    const int64_t kstride = (int64_t)Hkv * DQK, vstride = (int64_t)Hkv * DV;

    float mref = kNoMax, lsum = 0.f;
    floatx4 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = floatx4{0.f, 0.f, 0.f, 0.f};

#pragma unroll 1
    for (int ch = ch0; ch < ch1; ++ch) {
      const int s0 = lo + ch * CK;
      // V rows of the chunk -> wave-private LDS tile (rows past pos are zero).
      u32x4 vv[(CK * T::VCH) / 64];
#pragma unroll
      for (int i = 0; i < (CK * T::VCH) / 64; ++i) {
        const int cidx = lane + 64 * i;
        const int key = cidx / T::VCH, cc = cidx % T::VCH;
        const int ka = s0 + key;
        vv[i] = u32x4{0u, 0u, 0u, 0u};
        if (ka <= pos) vv[i] = ldg16(vg + vbase + ka * vstride + cc * 8);
      }
      // S^T = K . Q^T, K fragments straight from global memory.
      floatx4 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = min(s0 + 16 * kb + col, pos);
        const uint16_t* kp = kg + kbase + key * kstride + 8 * g4;
        bf16x8 a[T::KS];
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) a[ks] = __builtin_bit_cast(bf16x8, ldg16(kp + ks * 32));
        s[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) s[kb] = mfma_16x16x32(a[ks], qf[ks], s[kb]);
      }
#pragma unroll
      for (int i = 0; i < (CK * T::VCH) / 64; ++i) {
        const int cidx = lane + 64 * i;
        const int key = cidx / T::VCH, cc = cidx % T::VCH;
        *(u32x4*)(stage + key * T::VROW + cc * 8) = vv[i];
      }
      if (s0 + CK - 1 > pos) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (s0 + 16 * kb + 4 * g4 + r > pos) s[kb][r] = -INFINITY;
      }
      // Online softmax of each column (query head), lazily rescaled.
      float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                       fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
      if (__builtin_amdgcn_ballot_w64(mx * c > mref + 8.f)) {
        const float mnew = fmaxf(mref, col_max4(mx) * c);
        const float alpha = fast_exp2(mref - mnew);
        mref = mnew;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[db][r] *= alpha;
      }
      bf16x8 pb;
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(fmaf(s[kb][r], c, -mref));
          ps += p;
          pb[4 * kb + r] = (__bf16)p;
        }
      lsum += ps;
      // O^T += V^T . P^T
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* va = stage + (4 * g4 + (col >> 2)) * T::VROW + 16 * db + 4 * (col & 3);
        const shortx4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)va);
        const shortx4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(va + 16 * T::VROW));
        typedef __attribute__((__vector_size__(8 * sizeof(short)))) short shortx8;
        const shortx8 a8 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        o[db] = mfma_16x16x32(__builtin_bit_cast(bf16x8, a8), pb, o[db]);
      }
    }
    lsum = col_sum4(lsum);

    // Merge the waves' partials: m* = max m_w, l* = sum 2^(m_w - m*) l_w, same for O.
    __syncthreads();  // every wave is done with its V stage (the merge area aliases it)
    float* mw = merge + wave * T::MERGE_FLOATS;
    if (g4 == 0) {
      mw[col] = mref;
      mw[16 + col] = lsum;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) mw[32 + (16 * db + 4 * g4 + r) * 16 + col] = o[db][r];
    __syncthreads();
    // out = gate * (H_S - lambda * Repeat_g(H_N)) for this phase's signal heads;
    // each thread merges the two columns it needs.
    const int g = S / N;
    for (int idx = tid; idx < NS * DV; idx += NT) {
      const int sl = idx / DV, d = idx - (idx / DV) * DV;
      const int i = sig0 + ph * NS + sl;
      const int nl = i / g - u * NN;  // noise head of signal i, local to the unit
      const float hs = merged(merge, sl, d);
      float hn;
      if (ph == 0) {
        hn = merged(merge, NS + nl, d);
        if (R > 1 && sl == 0) sHN[d] = hn;  // one noise head per unit when R > 1
      } else {
        hn = sHN[d];
      }
      const int64_t o_idx = ((int64_t)b * S + i) * DV + d;
      const float lm = bf16_to_f32(lam[(int64_t)b * S + i]);
      const float gv = bf16_to_f32(gate[o_idx]);
      out[o_idx] = f32_to_bf16(gv * (hs - lm * hn));
    }
    __syncthreads();  // sH / stage reuse by the next phase
  }
}

template <int DQK, int DV>
hipError_t launch_dec(const DecodeArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.B * a.plan.units;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_bf16_kernel<DQK, DV>), dim3((unsigned)grid), dim3(NT), 0, stream,
                     (const uint16_t*)a.q_sig, (const uint16_t*)a.q_noise, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, a.lens, (const uint16_t*)a.lam,
                     (const uint16_t*)a.gate, (uint16_t*)a.out, a.Lmax, a.S, a.N, a.Hkv,
                     a.window, a.plan.units, a.plan.NS, a.plan.NN, a.plan.R, a.scale_log2);
  return hipGetLastError();
}

}  // namespace

bool decode_bf16_supported(int dqk, int dv, const UnitPlan& p) {
  const bool dims = (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
  return dims && p.NS + p.NN <= 16 && p.NN <= 16;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  if (a.dqk == 64 && a.dv == 64) return launch_dec<64, 64>(a, stream);
  if (a.dqk == 128 && a.dv == 128) return launch_dec<128, 128>(a, stream);
  if (a.dqk == 192 && a.dv == 128) return launch_dec<192, 128>(a, stream);
  return (hipError_t)-1;
}

}  // namespace gda
