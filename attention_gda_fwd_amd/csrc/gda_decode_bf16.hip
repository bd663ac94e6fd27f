// gda_decode_bf16.hip - bf16 split-KV decode kernels of the GDA/GDLA attention core (gfx950).
//
// One new query token per sequence attends over a KV cache that already holds
// it (the overview page's inference notes enable a KV cache; the Motif 3
// walk-through, novelty point one, notes GDLA's cache is MLA-sized because both
// query paths share the KV heads). The output is the D_t of the Motif 3
// walk-through (step 2) times the gate, as in prefill.
//
// Work decomposition (both kernels): one workgroup per (sequence b, unit u).
// Its 4 waves split the visible key range into contiguous slices of 32-key
// chunks, keeping a partial (max, sum, O^T) per query head. All query heads of
// the unit are the 16 columns of one 16x16 MFMA tile (unused columns are zero
// queries), so each K/V byte is read once for all of them. The partials are
// merged through LDS and the lambda/gate epilogue writes coalesced rows.
//
// Two ways to move the cache, chosen by the span of visible keys:
//  * long spans (decode_stream_kernel): each wave copies its chunks HBM -> LDS
//    with nontemporal global_load_lds_dwordx4, double-buffered in its own LDS
//    region (no VGPR staging, no barriers in the loop: each wave waits only for
//    its own older chunk). Every copy instruction covers whole 128-byte lines
//    (a line read in halves by two nontemporal loads can be fetched twice), and
//    the K rows are stored with their 16-byte pieces XOR-swizzled by row so that
//    MFMA fragment reads are bank-conflict free. One workgroup per CU (the
//    double-buffered chunks take the LDS), so grids larger than the CU count run
//    in rounds; worth it only when each wave streams many chunks;
//  * short spans (decode_bf16_kernel): K fragments go global -> VGPR -> MFMA A
//    operand, V rows through a wave-private LDS tile; small enough that four
//    workgroups share a CU and a 1024-workgroup grid is resident at once, which
//    is what a latency-bound short span needs.
#include "gda_device.hpp"
#include "gda_kernels.hpp"

namespace gda {
namespace {

constexpr int NW = 4;           // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int CK = 32;          // keys per chunk
constexpr float kNoMax = -1e30f;

// Which heads a decode workgroup computes. A unit (as the prefill groups heads:
// with Hkv >= N, noise head u and the R = Hkv/N KV heads u*R .. of its signal
// heads; with N > Hkv, KV head u with its NS = S/Hkv signal and NN = N/Hkv
// noise heads) normally fits the 16 columns of one MFMA tile. When it does not,
// it is split into K sub-units, each recomputing the noise head(s) it needs:
//   mode 0: the whole unit (K = 1);
//   mode 1: (R > 1) sub-unit k takes signal heads k*c .. of each phase's NS,
//           with the unit's noise head;
//   mode 2: (R = 1, g < 16) sub-unit k takes noise heads k*m .. k*m+m-1 of the
//           unit with their m*g signal heads;
//   mode 3: (R = 1, g >= 16) sub-unit k takes one noise head of the unit and a
//           chunk of c of its g signal heads.
// Phase p of a sub-unit attends KV head kv0 + p with signal heads
// (kv0+p)*NS + off .. +ns-1 and, in phase 0, noise heads nb .. nb+nn-1.
struct DecMap {
  int nsub;  // sub-units per sequence
  int K;     // sub-units per unit
  int mode;
  int c, m;  // chunk sizes of modes 1 and 3, and of mode 2
  int g, NS, NN, R;
};

struct SubHeads {
  int kv0, nb, nn, off, ns;
};

__device__ __forceinline__ SubHeads sub_heads(const DecMap& d, int v) {
  const int u = v / d.K, k = v - (v / d.K) * d.K;
  SubHeads h;
  h.kv0 = u * d.R;
  switch (d.mode) {
    case 1:
      h.nb = u; h.nn = 1; h.off = k * d.c; h.ns = min(d.c, d.NS - h.off);
      break;
    case 2:
      h.nb = u * d.NN + k * d.m; h.nn = d.m; h.off = k * d.m * d.g; h.ns = d.m * d.g;
      break;
    case 3: {
      const int kc_n = (d.g + d.c - 1) / d.c;
      const int j = k / kc_n, kc = k - (k / kc_n) * kc_n;
      h.nb = u * d.NN + j; h.nn = 1; h.off = j * d.g + kc * d.c; h.ns = min(d.c, d.g - kc * d.c);
      break;
    }
    default:
      h.nb = u * d.NN; h.nn = d.NN; h.off = 0; h.ns = d.NS;
  }
  return h;
}

template <int DQK, int DV>
struct DecTile {
  static constexpr int KS = DQK / 32;
  static constexpr int DB = DV / 16;
  static constexpr int VCH = DV / 8;     // 16-byte chunks per V row
  static constexpr int VPAIR = VCH / 2;  // 32-byte chunk pairs per V row
  static constexpr int VRPB = 512 / DV;  // V rows per 1 KB copy block
  static constexpr int VB = DV / 16;     // 1 KB copy blocks per 32-row V chunk
  static constexpr int STAGE = CK * DV;  // elements per wave stage (one V chunk)
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
// B x units = 1024-workgroup grid is resident at once on 256 CUs. The V chunk
// goes HBM -> LDS with direct copies (no registers), so the K fragments, the
// queries and the accumulators fit the 128 registers without spilling.
template <int DQK, int DV>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4, 4)))
decode_bf16_kernel(const uint16_t* __restrict__ q_sig, const uint16_t* __restrict__ q_noise,
                   const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
                   const int32_t* __restrict__ lens, const uint16_t* __restrict__ lam,
                   const uint16_t* __restrict__ gate, uint16_t* __restrict__ out, int Lmax,
                   int S, int N, int Hkv, int window, DecMap dm, float c, int flags) {
  using T = DecTile<DQK, DV>;
  constexpr int DB = T::DB;
  __shared__ __attribute__((aligned(16))) unsigned char smem[T::SHARED_BYTES];
  __shared__ float sHN[DV];  // the unit's noise output, kept across phases when R > 1

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, g4 = lane >> 4;
  const int b = blockIdx.x / dm.nsub, v = blockIdx.x - (blockIdx.x / dm.nsub) * dm.nsub;
  const SubHeads sh = sub_heads(dm, v);
  const int NS = dm.NS, R = dm.R, ns = sh.ns;

  int len = lens ? lens[b] : Lmax;
  if (len > Lmax) len = Lmax;
  if (len < 1) {  // no visible key: the output rows are zero
    for (int idx = tid; idx < R * ns * DV; idx += NT) {
      const int ph = idx / (ns * DV), rem = idx - ph * (ns * DV);
      out[((int64_t)b * S + (sh.kv0 + ph) * NS + sh.off + rem / DV) * DV + rem % DV] = 0;
    }
    return;
  }
  const int pos = len - 1;
  const int lo = window ? max(0, pos - window + 1) : 0;
  const int nch = (pos - lo + CK) / CK;
  const int ch0 = (int)(((int64_t)wave * nch) / NW), ch1 = (int)(((int64_t)(wave + 1) * nch) / NW);

  const uint16_t* stage = (const uint16_t*)smem + wave * T::STAGE;
  const uint32_t stage_lds = (uint32_t)(uintptr_t)(const lds_void*)stage;
  float* merge = (float*)smem;
  auto merged = [](const float* mg, int h, int d) { return merged_impl<T::MERGE_FLOATS>(mg, h, d); };

  // The epilogue's first lambda and gate values (phase 0, two per thread), loaded
  // now so that their latency hides behind the key loop: with short spans the
  // loop is one chunk per wave, and a second round trip to memory after it would
  // be a large part of the kernel.
  // Packed two bf16 per register: value k in bits 16k .. 16k+15.
  uint32_t lam_pre = 0, gate_pre = 0;
  {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int idx = tid + k * NT;
      if (idx < ns * DV) {
        const int i = sh.kv0 * NS + sh.off + idx / DV;
        lam_pre |= (uint32_t)lam[(int64_t)b * S + i] << (16 * k);
        gate_pre |= (uint32_t)gate[((int64_t)b * S + i) * DV + idx % DV] << (16 * k);
      }
    }
  }

#pragma unroll 1
  for (int ph = 0; ph < R; ++ph) {
    const int nh = ph == 0 ? ns + sh.nn : ns;  // query heads (MFMA columns) of this phase
    const int kvh = sh.kv0 + ph;
    const int sig0 = kvh * NS + sh.off;       // this phase's first signal head
    // Q^T B operand: column col is head col of the phase (zero if unused). Each
    // load takes a wave-uniform base and a 32-bit lane offset, so no 64-bit
    // per-lane address stays live.
    bf16x8 qf[T::KS];
    {
      const uint16_t* qs_row = q_sig + ((int64_t)b * S + sig0) * DQK;
      const uint16_t* qn_row = q_noise + ((int64_t)b * N + sh.nb) * DQK;
      const bool is_sig = col < ns, is_noise = !is_sig && col < nh;
      const uint32_t off = (uint32_t)((is_sig ? col : col - ns) * DQK + 8 * g4);
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (is_sig) w = ldg16(qs_row + off + ks * 32);
        if (is_noise) w = ldg16(qn_row + off + ks * 32);
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
      // V rows of the chunk -> this wave's LDS stage, direct copies in 1 KB blocks
      // of VRPB rows with 32-byte chunk pairs XOR-swizzled by row (the prefill's V
      // layout). Rows past pos read row pos: finite data whose weights are 0.
      {
        const int nrows = min(CK, pos - s0 + 1);
        const char* vb = (const char*)(vg + vbase + (int64_t)s0 * vstride);
#pragma unroll
        for (int j = 0; j < T::VB; ++j) {
          const int r = T::VRPB * j + lane / T::VCH;
          const int cch = (lane % T::VCH) ^ ((r % T::VPAIR) << 1);
          dma16_lds(vb, (uint32_t)min(r, nrows - 1) * (uint32_t)(vstride * 2) + 16u * (uint32_t)cch,
                    stage_lds + 1024u * (uint32_t)j);
        }
      }
      // S^T = K . Q^T, K fragments straight from global memory (a wave-uniform
      // chunk base plus a 32-bit lane offset).
      floatx4 s[2];
      const uint16_t* kchunk = kg + kbase + (int64_t)s0 * kstride;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t kr = (uint32_t)min(16 * kb + col, pos - s0);
        const uint32_t koff = kr * (uint32_t)kstride + 8u * (uint32_t)g4;
        bf16x8 a[T::KS];
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks)
          a[ks] = __builtin_bit_cast(bf16x8, ldg16(kchunk + koff + ks * 32));
        s[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) s[kb] = mfma_16x16x32(a[ks], qf[ks], s[kb]);
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
      // O^T += V^T . P^T, V^T from transposed reads of the swizzled V rows, once
      // this wave's copies of the chunk have landed.
      wait_vmcnt<0>();
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        shortx4 half[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int r = 16 * hf + 4 * g4 + (col >> 2);
          const int chunk = 2 * db + ((col & 3) >> 1);
          const uint16_t* va =
              stage + r * DV + ((chunk ^ ((r % T::VPAIR) << 1)) << 3) + 4 * (col & 1);
          half[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)va);
        }
        typedef __attribute__((__vector_size__(8 * sizeof(short)))) short shortx8;
        const shortx8 a8 = {half[0][0], half[0][1], half[0][2], half[0][3],
                            half[1][0], half[1][1], half[1][2], half[1][3]};
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
    for (int idx = tid; idx < ns * DV; idx += NT) {
      const int sl = idx / DV, d = idx - (idx / DV) * DV;
      const int i = sig0 + sl;
      const int nl = i / g - sh.nb;  // noise head of signal i, local to the sub-unit
      const float hs = merged(merge, sl, d);
      float hn;
      if (ph == 0) {
        hn = merged(merge, ns + nl, d);
        if (R > 1 && sl == 0) sHN[d] = hn;  // one noise head per sub-unit when R > 1
      } else {
        hn = sHN[d];
      }
      const int64_t o_idx = ((int64_t)b * S + i) * DV + d;
      const int k = (idx - tid) / NT;  // this thread's k-th value of the phase
      const bool pre = ph == 0 && k < 2;
      float lm = pre ? (k == 0 ? bf16_lo(lam_pre) : bf16_hi(lam_pre))
                     : bf16_to_f32(lam[(int64_t)b * S + i]);
      float gv = pre ? (k == 0 ? bf16_lo(gate_pre) : bf16_hi(gate_pre))
                     : bf16_to_f32(gate[o_idx]);
      if (flags & kLambdaLogits) lm = sigmoid_f32(lm);
      if (flags & kGateLogits) gv = sigmoid_f32(gv);
      out[o_idx] = f32_to_bf16(gv * (hs - lm * hn));
    }
    __syncthreads();  // sH / stage reuse by the next phase
  }
}

// ---- long spans: K/V chunks streamed HBM -> LDS ---------------------------------

template <int DQK, int DV>
struct StreamTile {
  static constexpr int KS = DQK / 32;
  static constexpr int DB = DV / 16;
  static constexpr int PR = DQK / 8;      // 16-byte pieces per K row
  static constexpr int KB = DQK / 16;     // 1 KB copy blocks per 32-row K chunk
  static constexpr int VB = DV / 16;      // 1 KB copy blocks per 32-row V chunk
  static constexpr int VCH = DV / 8;      // 16-byte chunks per V row
  static constexpr int VPAIR = VCH / 2;   // 32-byte chunk pairs per V row
  static constexpr int VRPB = 512 / DV;   // V rows per 1 KB block
  static constexpr int STAGE = (KB + VB) * 1024;  // bytes: K chunk, then V chunk
  static constexpr int WAVE_BYTES = 2 * STAGE;    // two stages per wave
  static constexpr int MERGE_FLOATS = 32 + DV * 16;
  static constexpr int SHARED_BYTES =
      NW * WAVE_BYTES > NW * MERGE_FLOATS * 4 ? NW * WAVE_BYTES : NW * MERGE_FLOATS * 4;
  static_assert(KB + VB < 64, "one chunk's copies fit the vmcnt counter");
};

// Slot of 16-byte piece c of K row r inside its row: c ^ kswz(r). For the 16 rows
// of one fragment read (fixed c) the slots fall on 16 distinct 16-byte bank
// groups: with 24 or 8 pieces per row, odd rows start half a bank row later and
// (r >> 1) & 7 spreads the 8 row pairs; with 16 pieces per row, r & 15 does it
// alone. The XOR stays inside the piece's aligned group of 8 (16), so the slots
// of a row are a permutation of its pieces.
template <int PR>
__device__ __forceinline__ int kswz(int r) {
  return PR == 16 ? (r & 15) : ((r >> 1) & 7);
}

// Per-lane byte offsets (from the chunk's first row) of the copy blocks: block j
// of the K chunk fills stage slots 64j .. 64j+63 (row P / PR, slot P % PR); block j
// of the V chunk fills VRPB rows, 32-byte chunk pairs XOR-swizzled by row (as the
// prefill stores V). Rows at or past nrows read row nrows-1 instead (finite data,
// masked or multiplied by zero).
template <class T>
__device__ __forceinline__ void copy_offsets(int lane, int nrows, uint32_t kstride,
                                             uint32_t vstride, uint32_t (&ko)[T::KB],
                                             uint32_t (&vo)[T::VB]) {
#pragma unroll
  for (int j = 0; j < T::KB; ++j) {
    const int P = 64 * j + lane;
    const int r = P / T::PR, slot = P - (P / T::PR) * T::PR;
    const int c = slot ^ kswz<T::PR>(r);
    ko[j] = (uint32_t)min(r, nrows - 1) * kstride + 16u * (uint32_t)c;
  }
#pragma unroll
  for (int j = 0; j < T::VB; ++j) {
    const int r = T::VRPB * j + lane / T::VCH;
    const int cch = (lane % T::VCH) ^ ((r % T::VPAIR) << 1);
    vo[j] = (uint32_t)min(r, nrows - 1) * vstride + 16u * (uint32_t)cch;
  }
}

template <int DQK, int DV>
__global__ void __launch_bounds__(NT, 1)
decode_stream_kernel(const uint16_t* __restrict__ q_sig, const uint16_t* __restrict__ q_noise,
                     const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
                     const int32_t* __restrict__ lens, const uint16_t* __restrict__ lam,
                     const uint16_t* __restrict__ gate, uint16_t* __restrict__ out, int Lmax,
                     int S, int N, int Hkv, int window, DecMap dm, float c, int flags) {
  using T = StreamTile<DQK, DV>;
  constexpr int DB = T::DB;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[T::SHARED_BYTES];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, g4 = lane >> 4;
  const int b = blockIdx.x / dm.nsub, v = blockIdx.x - (blockIdx.x / dm.nsub) * dm.nsub;
  const SubHeads sh = sub_heads(dm, v);
  const int NS = dm.NS, R = dm.R, ns = sh.ns;

  int len = lens ? lens[b] : Lmax;
  if (len > Lmax) len = Lmax;
  if (len < 1) {  // no visible key: the output rows are zero
    for (int idx = tid; idx < R * ns * DV; idx += NT) {
      const int ph = idx / (ns * DV), rem = idx - ph * (ns * DV);
      out[((int64_t)b * S + (sh.kv0 + ph) * NS + sh.off + rem / DV) * DV + rem % DV] = 0;
    }
    return;
  }
  const int pos = len - 1;
  const int lo = window ? max(0, pos - window + 1) : 0;
  const int nch = (pos - lo + CK) / CK;
  const int ch0 = (int)(((int64_t)wave * nch) / NW), ch1 = (int)(((int64_t)(wave + 1) * nch) / NW);

  const unsigned char* wmem = smem + wave * T::WAVE_BYTES;
  const uint32_t wlds = (uint32_t)(uintptr_t)(const lds_void*)wmem;
  float* merge = (float*)smem;
  const uint32_t kstride = (uint32_t)Hkv * DQK * 2, vstride = (uint32_t)Hkv * DV * 2;
  uint32_t ko[T::KB], vo[T::VB];
  copy_offsets<T>(lane, CK, kstride, vstride, ko, vo);
  float hn_keep = 0.f;  // this thread's noise channel, kept across phases when R > 1

#pragma unroll 1
  for (int ph = 0; ph < R; ++ph) {
    const int nh = ph == 0 ? ns + sh.nn : ns;
    const int kvh = sh.kv0 + ph;
    const int sig0 = kvh * NS + sh.off;
    bf16x8 qf[T::KS];
    {
      const uint16_t* qp = nullptr;
      if (col < ns)
        qp = q_sig + ((int64_t)b * S + sig0 + col) * DQK;
      else if (col < nh)
        qp = q_noise + ((int64_t)b * N + sh.nb + (col - ns)) * DQK;
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (qp) w = ldg16(qp + ks * 32 + 8 * g4);
        qf[ks] = __builtin_bit_cast(bf16x8, w);
      }
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) settle(qf[ks]);  // before any copy is issued
    }
    const char* kcol = (const char*)(kg + ((int64_t)b * Lmax * Hkv + kvh) * DQK);  // key 0
    const char* vcol = (const char*)(vg + ((int64_t)b * Lmax * Hkv + kvh) * DV);

    // Copies of chunk ch into stage st of this wave.
    auto issue = [&](int ch, int st) {
      const int s0 = lo + ch * CK;
      const char* kb = kcol + (int64_t)s0 * kstride;
      const char* vb = vcol + (int64_t)s0 * vstride;
      const uint32_t lk = wlds + (uint32_t)(st * T::STAGE), lv = lk + T::KB * 1024;
      if (s0 + CK - 1 <= pos) {
#pragma unroll
        for (int j = 0; j < T::KB; ++j) dma16_lds_nt(kb, ko[j], lk + 1024u * j);
#pragma unroll
        for (int j = 0; j < T::VB; ++j) dma16_lds_nt(vb, vo[j], lv + 1024u * j);
      } else {  // the chunk runs past the last key: rows clamped to it
        uint32_t k2[T::KB], v2[T::VB];
        copy_offsets<T>(lane, pos - s0 + 1, kstride, vstride, k2, v2);
#pragma unroll
        for (int j = 0; j < T::KB; ++j) dma16_lds_nt(kb, k2[j], lk + 1024u * j);
#pragma unroll
        for (int j = 0; j < T::VB; ++j) dma16_lds_nt(vb, v2[j], lv + 1024u * j);
      }
    };

    float mref = kNoMax, lsum = 0.f;
    floatx4 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = floatx4{0.f, 0.f, 0.f, 0.f};

    if (ch0 < ch1) issue(ch0, 0);
#pragma unroll 1
    for (int ch = ch0; ch < ch1; ++ch) {
      const int st = (ch - ch0) & 1;
      if (ch + 1 < ch1) {
        issue(ch + 1, st ^ 1);  // that stage was consumed by the previous chunk
        wait_vmcnt<T::KB + T::VB>();
      } else {
        wait_vmcnt<0>();
      }
      const unsigned char* sK = wmem + st * T::STAGE;
      const uint16_t* sV = (const uint16_t*)(sK + T::KB * 1024);
      const int s0 = lo + ch * CK;
      // S^T = K . Q^T; K fragment (16 keys x 32 dims) from the swizzled rows.
      floatx4 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int r = 16 * kb + col;
        s[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
          const int slot = (4 * ks + g4) ^ kswz<T::PR>(r);
          const bf16x8 a = *(const bf16x8*)(sK + (r * T::PR + slot) * 16);
          s[kb] = mfma_16x16x32(a, qf[ks], s[kb]);
        }
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
      // O^T += V^T . P^T, V^T from transposed reads of the swizzled V rows.
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        shortx4 half[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int r = 16 * hf + 4 * g4 + (col >> 2);
          const int chunk = 2 * db + ((col & 3) >> 1);
          const uint16_t* va = sV + r * DV + ((chunk ^ ((r % T::VPAIR) << 1)) << 3) + 4 * (col & 1);
          half[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)va);
        }
        typedef __attribute__((__vector_size__(8 * sizeof(short)))) short shortx8;
        const shortx8 a8 = {half[0][0], half[0][1], half[0][2], half[0][3],
                            half[1][0], half[1][1], half[1][2], half[1][3]};
        o[db] = mfma_16x16x32(__builtin_bit_cast(bf16x8, a8), pb, o[db]);
      }
    }
    lsum = col_sum4(lsum);

    // Merge the waves' partials (the merge area overlays the stages).
    __syncthreads();
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
    const int g = S / N;
    for (int idx = tid; idx < ns * DV; idx += NT) {
      const int sl = idx / DV, d = idx - (idx / DV) * DV;
      const int i = sig0 + sl;
      const int nl = i / g - sh.nb;
      const float hs = merged_impl<T::MERGE_FLOATS>(merge, sl, d);
      float hn;
      if (ph == 0) {
        hn = merged_impl<T::MERGE_FLOATS>(merge, ns + nl, d);
        hn_keep = hn;  // R > 1 means one noise head per sub-unit: the same for every sl
      } else {
        hn = hn_keep;  // this thread's d is the same in every phase (NT % DV == 0)
      }
      const int64_t o_idx = ((int64_t)b * S + i) * DV + d;
      float lm = bf16_to_f32(lam[(int64_t)b * S + i]);
      float gv = bf16_to_f32(gate[o_idx]);
      if (flags & kLambdaLogits) lm = sigmoid_f32(lm);
      if (flags & kGateLogits) gv = sigmoid_f32(gv);
      out[o_idx] = f32_to_bf16(gv * (hs - lm * hn));
    }
    __syncthreads();  // the next phase's copies overwrite the merge area
  }
}

// Visible keys per sequence above which the streaming kernel is used.
constexpr int kStreamMinSpan = 2048;

// Sub-units of a head layout: the whole unit when its query heads fit the 16
// MFMA columns, else the split described at DecMap.
DecMap make_decmap(const DecodeArgs& a) {
  const UnitPlan& p = a.plan;
  DecMap d;
  d.g = a.S / a.N;
  d.NS = p.NS;
  d.NN = p.NN;
  d.R = p.R;
  d.c = d.m = 1;
  if (p.NS + p.NN <= 16) {
    d.mode = 0;
    d.K = 1;
  } else if (p.R > 1) {  // one noise head per unit
    d.mode = 1;
    d.c = 15;
    d.K = (p.NS + 14) / 15;
  } else if (d.g < 16) {
    d.mode = 2;
    d.m = 1;
    for (int m = p.NN; m > 1; --m)
      if (p.NN % m == 0 && m * (d.g + 1) <= 16) {
        d.m = m;
        break;
      }
    d.K = p.NN / d.m;
  } else {
    d.mode = 3;
    d.c = 15;
    d.K = p.NN * ((d.g + 14) / 15);
  }
  d.nsub = p.units * d.K;
  return d;
}

template <int DQK, int DV>
hipError_t launch_stream(const DecodeArgs& a, hipStream_t stream) {
  static_assert(NT % DV == 0, "a thread keeps one output channel across phases");
  const DecMap dm = make_decmap(a);
  const int64_t grid = (int64_t)a.B * dm.nsub;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_stream_kernel<DQK, DV>), dim3((unsigned)grid), dim3(NT), 0, stream,
                     (const uint16_t*)a.q_sig, (const uint16_t*)a.q_noise, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, a.lens, (const uint16_t*)a.lam,
                     (const uint16_t*)a.gate, (uint16_t*)a.out, a.Lmax, a.S, a.N, a.Hkv,
                     a.window, dm, a.scale_log2, a.flags);
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t launch_dec(const DecodeArgs& a, hipStream_t stream) {
  const DecMap dm = make_decmap(a);
  const int64_t grid = (int64_t)a.B * dm.nsub;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_bf16_kernel<DQK, DV>), dim3((unsigned)grid), dim3(NT), 0, stream,
                     (const uint16_t*)a.q_sig, (const uint16_t*)a.q_noise, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, a.lens, (const uint16_t*)a.lam,
                     (const uint16_t*)a.gate, (uint16_t*)a.out, a.Lmax, a.S, a.N, a.Hkv,
                     a.window, dm, a.scale_log2, a.flags);
  return hipGetLastError();
}

}  // namespace

bool decode_bf16_supported(int dqk, int dv, const UnitPlan&) {
  // Every valid head layout maps onto sub-units (DecMap); only head sizes are compiled.
  return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  const int span = a.window > 0 && a.window < a.Lmax ? a.window : a.Lmax;
  const bool streamed = span >= kStreamMinSpan;
  if (a.dqk == 64 && a.dv == 64)
    return streamed ? launch_stream<64, 64>(a, stream) : launch_dec<64, 64>(a, stream);
  if (a.dqk == 128 && a.dv == 128)
    return streamed ? launch_stream<128, 128>(a, stream) : launch_dec<128, 128>(a, stream);
  if (a.dqk == 192 && a.dv == 128)
    return streamed ? launch_stream<192, 128>(a, stream) : launch_dec<192, 128>(a, stream);
  return (hipError_t)-1;
}

}  // namespace gda
