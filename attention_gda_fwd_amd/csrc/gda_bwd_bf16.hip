// gda_bwd_bf16.hip - backward of the GDA/GDLA prefill, bf16 inputs, fp32 accumulation.
//
// The chain rule through out = G (.) (H_S - lambda Repeat_g(H_N)) (the combine
// and gate of the Motif 3 walk-through's GDLA forward, equation D_t), then
// through each path's softmax attention:
//   dG = d_out (.) D,  dD = d_out (.) G,  dlambda_i = -dD_i . H_N,j(i)
//   dO_S,i = dD_i,     dO_N,j = -sum over the group's signal heads lambda_i dD_i
//   per attention row: P = exp(z - lse), dP = dO . v, delta = dO . H,
//   dS = P (dP - delta), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO
// Three kernels:
//   bwd_prep_kernel  elementwise: dG, dlambda, each path's dO (bf16) and every
//                    row's delta; one wave per (token, noise group);
//   bwd_dq_kernel    one workgroup per (sequence, 64 queries, two query heads of
//                    one KV head): that KV head's K/V tiles stream through LDS
//                    while each wave keeps its 16 queries' Q^T, dO^T and dQ^T of
//                    both heads in registers (every K/V fragment read serves two
//                    heads); scores transposed (S^T = K Q^T) as in the forward;
//   bwd_dkdv_kernel  one workgroup per (sequence, KV head, 64 keys): the Q and
//                    dO tiles of every query head on that KV head stream through
//                    LDS while each wave keeps its 16 keys' K, V and the dK^T,
//                    dV^T accumulators in registers; scores S = Q K^T so that P
//                    and dS are directly the B operands of dV^T = dO^T P and
//                    dK^T = Q^T dS.
// A batch and packed sequences with a query offset (a sequence's queries are its
// last Lq key positions) take the same kernels; keys no query sees get zeros.
// No atomics: every output row is written by exactly one workgroup.
#include "gda_device.hpp"
#include "gda_kernels.hpp"

namespace gda {
namespace {

constexpr int kBwdThreads = 256;  // 4 waves
// 16-key column tiles per dK/dV wave. Two tiles halve the LDS reads per matrix
// instruction but need about 330 registers, so one wave per SIMD: measured
// 22.0 ms against 15.1-15.5 ms for one tile on the Motif-3 full-layer backward.
constexpr int kDkvTiles = 1;

// Store 16-row accumulator tiles (lane (g, c) holds rows 16t + 4g + r of column c)
// as one bf16 row per column: tile pairs are regrouped across lanes l and l^16
// so each lane stores 8 consecutive values (16 bytes).
template <int NTILE>
__device__ __forceinline__ void store_col_row(uint16_t* row, int g4, const floatx4 (&acc)[NTILE],
                                              float mul) {
  static_assert(NTILE % 2 == 0, "tiles come in pairs");
  uint16_t* dst = row + 16 * (g4 & 1) + 8 * (g4 >> 1);
#pragma unroll
  for (int p = 0; p < NTILE / 2; ++p) {
    float e[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // vdst's odd rows trade places with vsrc's even rows.
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[2 * p][r] * mul),
                                                       __float_as_uint(acc[2 * p + 1][r] * mul),
                                                       false, false);
      e[r] = __uint_as_float(sw[0]);
      e[4 + r] = __uint_as_float(sw[1]);
    }
    u32x4 ow;
#pragma unroll
    for (int w = 0; w < 4; ++w) ow[w] = pack_bf16x2(e[2 * w], e[2 * w + 1]);
    *(u32x4*)(dst + 32 * p) = ow;
  }
}

// A operand [16 rows x 32] of an MFMA taken transposed from a row-major LDS tile
// T[32][cols] (row stride in bytes): lane (g, i) receives T[16h + 4g + r][m0 + i]
// in element 4h + r. Its K order matches a B operand built from two accumulator
// tiles (element 4h + r = row 4g + r of tile h).
__device__ __forceinline__ bf16x8 tr_operand(const unsigned char* tile, int stride, int m0,
                                             int g4, int col) {
  shortx4 half[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const unsigned char* a =
        tile + (16 * h + 4 * g4 + (col >> 2)) * stride + (m0 + 4 * (col & 3)) * 2;
    half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)a);
  }
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short shortx8;
  const shortx8 a8 = {half[0][0], half[0][1], half[0][2], half[0][3],
                      half[1][0], half[1][1], half[1][2], half[1][3]};
  return __builtin_bit_cast(bf16x8, a8);
}

// Row operand: lane (g, c) reads T[r0 + c][32 ks + 8g .. +7].
__device__ __forceinline__ bf16x8 row_operand(const unsigned char* tile, int stride, int r0,
                                              int ks, int g4, int col) {
  return *(const bf16x8*)(tile + (r0 + col) * stride + (32 * ks + 8 * g4) * 2);
}

// ---------------------------------------------------------------------------------
// Elementwise part. One wave per (token row, noise group j). The wave takes the
// group's g signal heads HP = 64 / (DV / 8) at a time: lane l works on head slot
// l / (DV / 8) and the 8 channels 8 (l % (DV / 8)) .. +7 of it, so every load and
// store moves 16 bytes per lane and whole rows per wave; a head's dot products
// reduce over its DV / 8 lanes, and the noise head's dO sums the slots at the end.
template <int DV>
__device__ __forceinline__ float group_sum(float x) {  // over the DV / 8 lanes of a slot
#pragma unroll
  for (int o = DV / 16; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int DV>
__global__ void __launch_bounds__(kBwdThreads)
bwd_prep_kernel(const uint16_t* __restrict__ d_out, const uint16_t* __restrict__ gate,
                const uint16_t* __restrict__ lam, const uint16_t* __restrict__ h_sig,
                const uint16_t* __restrict__ h_noise, uint16_t* __restrict__ dgate,
                uint16_t* __restrict__ dlam, uint16_t* __restrict__ do_sig,
                uint16_t* __restrict__ do_noise, float* __restrict__ delta, int64_t items,
                int Lrow, int64_t dl_b, int64_t dl_h, int S, int N, int flags) {
  constexpr int LPH = DV / 8;    // lanes per head
  constexpr int HP = 64 / LPH;   // head slots per wave
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * (kBwdThreads / 64) + (threadIdx.x >> 6);
  if (item >= items) return;
  const int64_t row = item / N;
  const int j = (int)(item - row * N);
  // delta of head hd for token row at delta[b * dl_b + hd * dl_h + t], with b, t
  // the row's (sequence, position) for a batch of Lrow-row sequences (packed
  // sequences pass Lrow = all rows: b = 0, t = row).
  const int64_t b = row / Lrow;
  const int t = (int)(row - b * Lrow);
  const int g = S / N;
  const int slot = lane / LPH, c8 = lane - (lane / LPH) * LPH;
  const u32x4 hnw = ldg16(h_noise + (row * N + j) * DV + 8 * c8);
  float hn[8], dn[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    hn[2 * w] = bf16_lo(hnw[w]);
    hn[2 * w + 1] = bf16_hi(hnw[w]);
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) dn[c] = 0.f;
  for (int p0 = 0; p0 < g; p0 += HP) {
    const int ii = p0 + slot;
    const bool on = ii < g;  // uniform over a slot's lanes
    const int i = j * g + (on ? ii : 0);
    const int64_t base = (row * S + i) * DV + 8 * c8;
    float lm = bf16_to_f32(lam[row * S + i]);
    if (flags & kLambdaLogits) lm = sigmoid_f32(lm);
    const u32x4 hsw = ldg16(h_sig + base), gw = ldg16(gate + base), ow = ldg16(d_out + base);
    float pl = 0.f, pd = 0.f;
    u32x4 dgw, ddw;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float dg2[2], dd2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 2 * w + h;
        const float hs = h ? bf16_hi(hsw[w]) : bf16_lo(hsw[w]);
        float G = h ? bf16_hi(gw[w]) : bf16_lo(gw[w]);
        if (flags & kGateLogits) G = sigmoid_f32(G);
        const float dO = h ? bf16_hi(ow[w]) : bf16_lo(ow[w]);
        const float D = hs - lm * hn[c];
        float dG = dO * D;
        if (flags & kGateLogits) dG *= G * (1.f - G);
        const float dD = dO * G;
        dg2[h] = dG;
        dd2[h] = dD;
        const float dDb = bf16_to_f32(f32_to_bf16(dD));
        pl += dD * hn[c];
        pd += dDb * hs;  // delta from the dO the matrix kernels use
        if (on) dn[c] -= lm * dD;
      }
      dgw[w] = pack_bf16x2(dg2[0], dg2[1]);
      ddw[w] = pack_bf16x2(dd2[0], dd2[1]);
    }
    pl = group_sum<DV>(pl);
    pd = group_sum<DV>(pd);
    if (on) {
      *(u32x4*)(dgate + base) = dgw;
      *(u32x4*)(do_sig + base) = ddw;
      if (c8 == 0) {
        float dl = -pl;
        if (flags & kLambdaLogits) dl *= lm * (1.f - lm);
        dlam[row * S + i] = f32_to_bf16(dl);
        delta[b * dl_b + i * dl_h + t] = pd;
      }
    }
  }
  // The noise head's dO: the sum over the slots (lanes c8, c8 + LPH, ...).
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int o = LPH; o < 64; o <<= 1) dn[c] += __shfl_xor(dn[c], o);
  if (slot == 0) {
    u32x4 dnw;
    float pn = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dnw[w] = pack_bf16x2(dn[2 * w], dn[2 * w + 1]);
      pn += bf16_lo(dnw[w]) * hn[2 * w] + bf16_hi(dnw[w]) * hn[2 * w + 1];
    }
    *(u32x4*)(do_noise + (row * N + j) * DV + 8 * c8) = dnw;
    pn = group_sum<DV>(pn);
    if (lane == 0) delta[b * dl_b + (S + j) * dl_h + t] = pn;
  }
}

// One query head's view: its Q and dO rows, and its KV head.
struct HeadRef {
  const uint16_t* q;   // row t at q + t * qstride
  const uint16_t* dO;  // row t at dO + t * ostride
  int64_t qstride, ostride;
  int kvh;
};

// qbase: the sequence's first query row.
__device__ __forceinline__ HeadRef head_ref(int hd, int64_t qbase, int S, int N, int Hkv,
                                            int DQK, int DV, const uint16_t* q_sig,
                                            const uint16_t* q_noise, const uint16_t* do_sig,
                                            const uint16_t* do_noise) {
  HeadRef r;
  if (hd < S) {
    r.q = q_sig + (qbase * S + hd) * DQK;
    r.dO = do_sig + (qbase * S + hd) * DV;
    r.qstride = (int64_t)S * DQK;
    r.ostride = (int64_t)S * DV;
    r.kvh = (hd * Hkv) / S;
  } else {
    const int j = hd - S;
    r.q = q_noise + (qbase * N + j) * DQK;
    r.dO = do_noise + (qbase * N + j) * DV;
    r.qstride = (int64_t)N * DQK;
    r.ostride = (int64_t)N * DV;
    r.kvh = (j * Hkv) / N;
  }
  return r;
}

// Sequence b: Lq queries from packed row qbase, Lk keys from packed row kbase, its
// local query t at key position qoff + t (packed sequences), or rows b*L .. of both
// (a batch). Its lse and delta entries for head hd and local query t sit at
// lbase + hd * lh + t.
struct SeqRef {
  int64_t qbase, kbase, lbase;
  int Lq, Lk, qoff;
};

__device__ __forceinline__ SeqRef seq_ref(const int32_t* cu_q, const int32_t* cu_k, int b,
                                          int L, int64_t lse_b, int lse_q) {
  SeqRef r;
  if (cu_q) {
    r.qbase = cu_q[b];
    r.Lq = cu_q[b + 1] - cu_q[b];
    r.kbase = cu_k[b];
    r.Lk = cu_k[b + 1] - cu_k[b];
  } else {
    r.qbase = r.kbase = (int64_t)b * L;
    r.Lq = r.Lk = L;
  }
  r.qoff = r.Lk - r.Lq;
  r.lbase = lse_b * b + lse_q * r.qbase;
  return r;
}

// ---------------------------------------------------------------------------------
// dQ. LDS tile of 32 keys: K rows then V rows, each row padded by 16 bytes,
// each region rounded up to whole 1 KB copy blocks. The tiles arrive by direct
// global -> LDS copies: copy block i of a region is the region's bytes
// 1024 i .. 1024 i + 1023, and each lane fetches the row piece that lands at its
// 16 bytes (pad and slack slots fetch row 0's first piece).
template <int DQK, int DV>
struct DqShape {
  static constexpr int KS = DQK / 32, VS = DV / 32, DT = DQK / 16;
  static constexpr int KROW = DQK * 2 + 16, VROW = DV * 2 + 16;
  static constexpr int KBLK = (32 * KROW + 1023) / 1024, VBLK = (32 * VROW + 1023) / 1024;
  static constexpr int V_OFF = KBLK * 1024;
  static constexpr int TILE = (KBLK + VBLK) * 1024;
};

// Issue this wave's copy blocks (wave, wave + 4, ...) of a region of 32 rows:
// source rows row0 + r (r clamped to rows_ok - 1), row r at src + r * gstride bytes.
template <int ROWB, int STRIDE, int NBLK>
__device__ __forceinline__ void copy_rows(const void* src, uint32_t gstride, int rows_ok,
                                          uint32_t lds, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < (NBLK + 3) / 4; ++i) {
    const int blk = wave + 4 * i;
    if (blk < NBLK) {
      const int o = blk * 1024 + 16 * lane;
      int r = o / STRIDE, c = o - (o / STRIDE) * STRIDE;
      if (c >= ROWB || r >= 32) r = 0, c = 0;
      r = min(r, rows_ok - 1);
      dma16_lds(src, (uint32_t)r * gstride + (uint32_t)c, lds + 1024u * blk);
    }
  }
}

// The query heads on KV head h: signal heads h*S/Hkv .. (S/Hkv of them), then
// noise heads ceil(h*N/Hkv) .. ceil((h+1)*N/Hkv) - 1. Entry i of that list:
__device__ __forceinline__ int kv_head_member(int h, int i, int S, int N, int Hkv) {
  const int n_sig = S / Hkv;
  return i < n_sig ? h * n_sig + i : S + (h * N + Hkv - 1) / Hkv + (i - n_sig);
}

__device__ __forceinline__ int kv_head_count(int h, int S, int N, int Hkv) {
  return S / Hkv + ((h + 1) * N + Hkv - 1) / Hkv - (h * N + Hkv - 1) / Hkv;
}

// NH query heads of one KV head per wave (1 or 2): the K/V fragments read from
// LDS serve every head of the wave. Workgroup: (query tile slot, sequence, KV
// head, head group); with NH = 2 group p takes list entries 2p, 2p+1; with
// NH = 1 the workgroup takes the last entry when the list is odd.
template <int DQK, int DV, int NH>
__global__ void __launch_bounds__(kBwdThreads, 2)
bwd_dq_kernel(const uint16_t* __restrict__ q_sig, const uint16_t* __restrict__ q_noise,
              const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
              const float* __restrict__ lse, const uint16_t* __restrict__ do_sig,
              const uint16_t* __restrict__ do_noise, const float* __restrict__ delta,
              uint16_t* __restrict__ dq_sig, uint16_t* __restrict__ dq_noise,
              const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int B, int L,
              int S, int N, int Hkv, int window, int nqt, int groups, int heavy_first,
              int64_t lse_b, int lse_q, int64_t lse_h, float c2, float scale) {
  using C = DqShape<DQK, DV>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * C::TILE];
  const int HT = S + N;
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, g4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per = B * Hkv * groups;
  const int slot = blockIdx.x / per;
  const int qt = heavy_first ? nqt - 1 - slot : slot;
  int rem = blockIdx.x - slot * per;
  const int b = rem / (Hkv * groups);
  rem -= b * (Hkv * groups);
  const int h = rem / groups, grp = rem - (rem / groups) * groups;
  const SeqRef sq = seq_ref(cu_q, cu_k, b, L, lse_b, lse_q);
  const int q0 = qt * 64;  // this tile's first query of the sequence
  if (q0 >= sq.Lq) return;  // past the sequence (whole workgroup, before any barrier)
  const int nh_kv = kv_head_count(h, S, N, Hkv);
  int first;
  if (NH == 2) {
    if (2 * grp + 1 >= nh_kv) return;  // whole workgroup, before any barrier
    first = 2 * grp;
  } else {
    if ((nh_kv & 1) == 0) return;
    first = nh_kv - 1;
  }
  int hd[NH];
  HeadRef hr[NH];
#pragma unroll
  for (int u = 0; u < NH; ++u) {
    hd[u] = kv_head_member(h, first + u, S, N, Hkv);
    hr[u] = head_ref(hd[u], sq.qbase, S, N, Hkv, DQK, DV, q_sig, q_noise, do_sig, do_noise);
  }
  const int t0w = q0 + 16 * wave;
  const int t = t0w + col;  // this lane's query (local)
  const bool t_ok = t < sq.Lq;
  const int tq = min(t, sq.Lq - 1);
  const int pos = sq.qoff + t;  // its key position

  bf16x8 qT[NH][C::KS], doT[NH][C::VS];
  float lse2[NH], dl[NH];
  floatx4 dqT[NH][C::DT];
#pragma unroll
  for (int u = 0; u < NH; ++u) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qT[u][ks] =
          __builtin_bit_cast(bf16x8, ldg16(hr[u].q + tq * hr[u].qstride + 32 * ks + 8 * g4));
#pragma unroll
    for (int kv = 0; kv < C::VS; ++kv)
      doT[u][kv] =
          __builtin_bit_cast(bf16x8, ldg16(hr[u].dO + tq * hr[u].ostride + 32 * kv + 8 * g4));
    lse2[u] = lse[sq.lbase + hd[u] * lse_h + tq] * kLog2e;
    dl[u] = delta[sq.lbase + hd[u] * lse_h + tq];
#pragma unroll
    for (int d = 0; d < C::DT; ++d) dqT[u][d] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // Keys visible to the tile's queries (key positions qoff + q0 ..); none when every
  // query sits at a negative position.
  const int k_lo = window ? max(0, sq.qoff + q0 - window + 1) : 0;
  const int k_hi = sq.qoff + min(q0 + 63, sq.Lq - 1);
  const int kt0 = k_lo / 32, kt1 = k_hi >= 0 ? k_hi / 32 : kt0 - 1;
  const uint16_t* kbase = kg + (sq.kbase * Hkv + h) * DQK;
  const uint16_t* vbase = vg + (sq.kbase * Hkv + h) * DV;
  const int64_t kstride = (int64_t)Hkv * DQK, vstride = (int64_t)Hkv * DV;

  const uint32_t smem_lds = (uint32_t)(uintptr_t)(const lds_void*)smem;
  auto issue = [&](int kt, int buf) {
    const int rows_ok = min(32, sq.Lk - kt * 32);  // >= 1: kt * 32 <= k_hi <= Lk - 1
    const uint32_t base = smem_lds + (uint32_t)(buf * C::TILE);
    copy_rows<DQK * 2, C::KROW, C::KBLK>(kbase + (int64_t)kt * 32 * kstride,
                                         (uint32_t)(kstride * 2), rows_ok, base, wave, lane);
    copy_rows<DV * 2, C::VROW, C::VBLK>(vbase + (int64_t)kt * 32 * vstride,
                                        (uint32_t)(vstride * 2), rows_ok, base + C::V_OFF, wave,
                                        lane);
  };

  if (kt0 <= kt1) issue(kt0, 0);
  for (int kt = kt0; kt <= kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of tile kt have landed
    __syncthreads();                // ... and every wave's; tile kt-1 is consumed
    if (kt + 1 <= kt1) issue(kt + 1, buf ^ 1);
    const unsigned char* Kl = smem + buf * C::TILE;
    const unsigned char* Vl = Kl + C::V_OFF;
    const int k0 = kt * 32;
    // Is any key of this tile visible to a query of this wave? (wave-uniform)
    const int p0 = sq.qoff + t0w;  // the wave's first query position
    const bool live = k0 <= p0 + 15 && (!window || k0 + 31 >= p0 - window + 1);
    if (live) {
      // One 16-key half at a time: its scores and dP are dead once its dS is packed.
      bf16x8 dsb[NH];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        floatx4 sT[NH], dpT[NH];
#pragma unroll
        for (int u = 0; u < NH; ++u) {
          sT[u] = floatx4{0.f, 0.f, 0.f, 0.f};
          dpT[u] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const bf16x8 a = row_operand(Kl, C::KROW, 16 * kb, ks, g4, col);
#pragma unroll
          for (int u = 0; u < NH; ++u) sT[u] = mfma_16x16x32(a, qT[u][ks], sT[u]);
        }
#pragma unroll
        for (int kv = 0; kv < C::VS; ++kv) {
          const bf16x8 a = row_operand(Vl, C::VROW, 16 * kb, kv, g4, col);
#pragma unroll
          for (int u = 0; u < NH; ++u) dpT[u] = mfma_16x16x32(a, doT[u][kv], dpT[u]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + 16 * kb + 4 * g4 + r;
          const bool vis = t_ok && key <= pos && (!window || pos - key < window);
#pragma unroll
          for (int u = 0; u < NH; ++u) {
            const float p = vis ? fast_exp2(fmaf(sT[u][r], c2, -lse2[u])) : 0.f;
            dsb[u][4 * kb + r] = (__bf16)(p * (dpT[u][r] - dl[u]));
          }
        }
      }
#pragma unroll
      for (int d = 0; d < C::DT; ++d) {
        const bf16x8 a = tr_operand(Kl, C::KROW, 16 * d, g4, col);
#pragma unroll
        for (int u = 0; u < NH; ++u) dqT[u][d] = mfma_16x16x32(a, dsb[u], dqT[u][d]);
      }
    }
  }
  if (t_ok) {
#pragma unroll
    for (int u = 0; u < NH; ++u) {
      uint16_t* dst = hd[u] < S ? dq_sig + ((sq.qbase + t) * S + hd[u]) * DQK
                                : dq_noise + ((sq.qbase + t) * N + hd[u] - S) * DQK;
      store_col_row<C::DT>(dst, g4, dqT[u], scale);
    }
  }
}

// ---------------------------------------------------------------------------------
// dK, dV. LDS tile of 32 queries of one head: Q rows, dO rows (each padded by 16
// bytes), then the rows' lse (log2 units) and delta.
template <int DQK, int DV>
struct DkvShape {
  static constexpr int KS = DQK / 32, VS = DV / 32, DT = DQK / 16, VT = DV / 16;
  static constexpr int QROW = DQK * 2 + 16, OROW = DV * 2 + 16;
  static constexpr int QBLK = (32 * QROW + 1023) / 1024, OBLK = (32 * OROW + 1023) / 1024;
  static constexpr int O_OFF = QBLK * 1024;
  static constexpr int L_OFF = (QBLK + OBLK) * 1024;
  static constexpr int D_OFF = L_OFF + 32 * 4;
  static constexpr int TILE = D_OFF + 32 * 4;
};

// KT 16-key column tiles per wave (64*KT keys per workgroup): every Q/dO
// fragment read from LDS serves KT tiles.
template <int DQK, int DV, int KT>
__global__ void __launch_bounds__(kBwdThreads, KT == 1 ? 2 : 1)
bwd_dkdv_kernel(const uint16_t* __restrict__ q_sig, const uint16_t* __restrict__ q_noise,
                const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
                const float* __restrict__ lse, const uint16_t* __restrict__ do_sig,
                const uint16_t* __restrict__ do_noise, const float* __restrict__ delta,
                uint16_t* __restrict__ dk, uint16_t* __restrict__ dvo,
                const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int B, int L,
                int S, int N, int Hkv, int window, int64_t lse_b, int lse_q, int64_t lse_h,
                float c2, float scale) {
  using C = DkvShape<DQK, DV>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * C::TILE];
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, g4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int per = B * Hkv;
  const int kt = blockIdx.x / per;  // key tiles in order: the first ones see the most queries
  const int rem = blockIdx.x - kt * per;
  const int b = rem / Hkv, h = rem - (rem / Hkv) * Hkv;
  const SeqRef sq = seq_ref(cu_q, cu_k, b, L, lse_b, lse_q);
  if (kt * 64 * KT >= sq.Lk) return;  // past the sequence's keys (whole workgroup)
  const int k0w = kt * 64 * KT + 16 * KT * wave;  // this wave's first key (local)
  int s[KT];  // this lane's key in each column tile
  bf16x8 kT[KT][C::KS], vT[KT][C::VS];
  floatx4 dkT[KT][C::DT], dvT[KT][C::VT];
#pragma unroll
  for (int kc = 0; kc < KT; ++kc) {
    s[kc] = k0w + 16 * kc + col;
    const int sk = min(s[kc], sq.Lk - 1);
    const uint16_t* kr = kg + ((sq.kbase + sk) * Hkv + h) * DQK;
    const uint16_t* vr = vg + ((sq.kbase + sk) * Hkv + h) * DV;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      kT[kc][ks] = __builtin_bit_cast(bf16x8, ldg16(kr + 32 * ks + 8 * g4));
#pragma unroll
    for (int kv = 0; kv < C::VS; ++kv)
      vT[kc][kv] = __builtin_bit_cast(bf16x8, ldg16(vr + 32 * kv + 8 * g4));
#pragma unroll
    for (int d = 0; d < C::DT; ++d) dkT[kc][d] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < C::VT; ++d) dvT[kc][d] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  // Wait for K and V here, once (a first use inside the item loop would put the
  // wait there, where it drains the copies in flight every item).
#pragma unroll
  for (int kc = 0; kc < KT; ++kc) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) settle(kT[kc][ks]);
#pragma unroll
    for (int kv = 0; kv < C::VS; ++kv) settle(vT[kc][kv]);
  }

  const int nh = kv_head_count(h, S, N, Hkv);
  // Local queries that see one of the tile's keys (query t sits at position qoff + t);
  // none, and zero gradients, when that range is empty.
  const int q_lo = max(0, kt * 64 * KT - sq.qoff);
  const int q_hi = window ? min(sq.Lq - 1, kt * 64 * KT + 64 * KT - 1 + window - 1 - sq.qoff)
                          : sq.Lq - 1;
  const int qb0 = q_lo / 32, nqb = q_hi >= q_lo ? q_hi / 32 - qb0 + 1 : 0;
  const int n_items = nh * nqb;

  // Q and dO rows arrive by direct global -> LDS copies; the 32 rows' lse (log2
  // units) and delta by plain loads of threads 0..63, written after the compute.
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(const lds_void*)smem;
  float stg_s = 0.f;
  auto head_of_item = [&](int it) -> int { return kv_head_member(h, it / nqb, S, N, Hkv); };
  auto issue = [&](int it, int buf) {
    const int hd = head_of_item(it);
    const int qb = qb0 + (it - (it / nqb) * nqb);
    const HeadRef hr = head_ref(hd, sq.qbase, S, N, Hkv, DQK, DV, q_sig, q_noise, do_sig,
                                do_noise);
    const int rows_ok = min(32, sq.Lq - qb * 32);  // >= 1: qb * 32 <= q_hi
    const uint32_t base = smem_lds + (uint32_t)(buf * C::TILE);
    copy_rows<DQK * 2, C::QROW, C::QBLK>(hr.q + (int64_t)qb * 32 * hr.qstride,
                                         (uint32_t)(hr.qstride * 2), rows_ok, base, wave, lane);
    copy_rows<DV * 2, C::OROW, C::OBLK>(hr.dO + (int64_t)qb * 32 * hr.ostride,
                                        (uint32_t)(hr.ostride * 2), rows_ok, base + C::O_OFF,
                                        wave, lane);
    if (tid < 64) {
      const int q = min(qb * 32 + (tid & 31), sq.Lq - 1);
      const int64_t at = sq.lbase + hd * lse_h + q;
      stg_s = tid < 32 ? lse[at] * kLog2e : delta[at];
    }
  };
  auto store_scalars = [&](int buf) {
    if (tid < 64) *(float*)(smem + buf * C::TILE + C::L_OFF + 4 * tid) = stg_s;
  };

  if (n_items > 0) {
    issue(0, 0);
    store_scalars(0);
  }
  for (int it = 0; it < n_items; ++it) {
    const int buf = it & 1;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of item it have landed
    __syncthreads();                // ... and every wave's; item it-1 is consumed
    if (it + 1 < n_items) issue(it + 1, buf ^ 1);
    const unsigned char* Ql = smem + buf * C::TILE;
    const unsigned char* Ol = Ql + C::O_OFF;
    const float* sL = (const float*)(Ql + C::L_OFF);
    const float* sD = (const float*)(Ql + C::D_OFF);
    const int q0 = (qb0 + (it - (it / nqb) * nqb)) * 32;
    const int p0 = sq.qoff + q0;  // the block's first query position
    const bool live = k0w <= p0 + 31 && (!window || p0 <= k0w + 16 * KT - 2 + window);
    if (live) {
      floatx4 sc[KT][2], dp[KT][2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
        for (int kc = 0; kc < KT; ++kc) {
          sc[kc][qt] = floatx4{0.f, 0.f, 0.f, 0.f};
          dp[kc][qt] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const bf16x8 a = row_operand(Ql, C::QROW, 16 * qt, ks, g4, col);
#pragma unroll
          for (int kc = 0; kc < KT; ++kc) sc[kc][qt] = mfma_16x16x32(a, kT[kc][ks], sc[kc][qt]);
        }
#pragma unroll
        for (int kv = 0; kv < C::VS; ++kv) {
          const bf16x8 a = row_operand(Ol, C::OROW, 16 * qt, kv, g4, col);
#pragma unroll
          for (int kc = 0; kc < KT; ++kc) dp[kc][qt] = mfma_16x16x32(a, vT[kc][kv], dp[kc][qt]);
        }
      }
      // Schedule (dqk <= 128; at dqk = 192 the compiler's own order measured faster):
      // Q and dO row fragments six reads ahead of the products that use them.
      if constexpr (DQK <= 128) {
        constexpr int NR = 2 * (C::KS + C::VS), AHEAD = 6;
        __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, KT, 0);
          if (i + AHEAD < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      bf16x8 pb[KT], dsb[KT];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qi = 16 * qt + 4 * g4 + r;
          const int q = q0 + qi;
          const float l2 = sL[qi], dl = sD[qi];
#pragma unroll
          for (int kc = 0; kc < KT; ++kc) {
            const int qp = sq.qoff + q;  // the query's key position
            const bool vis = s[kc] < sq.Lk && q < sq.Lq && s[kc] <= qp &&
                             (!window || qp - s[kc] < window);
            const float p = vis ? fast_exp2(fmaf(sc[kc][qt][r], c2, -l2)) : 0.f;
            pb[kc][4 * qt + r] = (__bf16)p;
            dsb[kc][4 * qt + r] = (__bf16)(p * (dp[kc][qt][r] - dl));
          }
        }
#pragma unroll
      for (int d = 0; d < C::VT; ++d) {
        const bf16x8 a = tr_operand(Ol, C::OROW, 16 * d, g4, col);
#pragma unroll
        for (int kc = 0; kc < KT; ++kc) dvT[kc][d] = mfma_16x16x32(a, pb[kc], dvT[kc][d]);
      }
#pragma unroll
      for (int d = 0; d < C::DT; ++d) {
        const bf16x8 a = tr_operand(Ql, C::QROW, 16 * d, g4, col);
#pragma unroll
        for (int kc = 0; kc < KT; ++kc) dkT[kc][d] = mfma_16x16x32(a, dsb[kc], dkT[kc][d]);
      }
      // Schedule (dqk <= 128): transposed dO / Q fragment pairs four ahead of their
      // products.
      if constexpr (DQK <= 128) {
        constexpr int NT = C::VT + C::DT, AHEAD2 = 4;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD2, 1);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, KT, 1);
          if (i + AHEAD2 < NT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
      }
    }
    if (it + 1 < n_items) store_scalars(buf ^ 1);
  }
#pragma unroll
  for (int kc = 0; kc < KT; ++kc)
    if (s[kc] < sq.Lk) {
      store_col_row<C::DT>(dk + ((sq.kbase + s[kc]) * Hkv + h) * DQK, g4, dkT[kc], scale);
      store_col_row<C::VT>(dvo + ((sq.kbase + s[kc]) * Hkv + h) * DV, g4, dvT[kc], 1.f);
    }
}

template <int DQK, int DV>
hipError_t launch_bwd_dims(const BwdArgs& a, hipStream_t stream) {
  // a.B sequences of at most a.L queries and a.Lk_max keys (a batch: a.Lk_max = a.L).
  const int64_t items = (int64_t)a.rows * a.N;
  const int64_t prep_blocks = (items + 3) / 4;
  const int nqt = (a.L + 63) / 64;
  const int64_t dq_blocks = (int64_t)nqt * a.B * a.Hkv;  // per head group
  const int64_t dkv_blocks =
      (int64_t)((a.Lk_max + 64 * kDkvTiles - 1) / (64 * kDkvTiles)) * a.B * a.Hkv;
  const int HT = a.S + a.N;
  if (prep_blocks > 0x7fffffff || dq_blocks * (HT / a.Hkv + 2) > 0x7fffffff ||
      dkv_blocks > 0x7fffffff)
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_prep_kernel<DV>), dim3((unsigned)prep_blocks), dim3(kBwdThreads), 0,
                     stream, (const uint16_t*)a.d_out, (const uint16_t*)a.gate,
                     (const uint16_t*)a.lam, (const uint16_t*)a.h_sig,
                     (const uint16_t*)a.h_noise, (uint16_t*)a.dgate, (uint16_t*)a.dlam,
                     a.do_sig, a.do_noise, a.delta, items, a.cu_q ? a.rows : a.L,
                     a.cu_q ? (int64_t)0 : (int64_t)HT * a.L, a.lse_h, a.S, a.N, a.flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int heavy_first = a.window == 0 ? 1 : 0;
  // Heads per KV head: the most any KV head has (noise heads may sit on some only).
  int nh_max = 0, any_odd = 0;
  for (int h = 0; h < a.Hkv; ++h) {
    const int n = a.S / a.Hkv + ((h + 1) * a.N + a.Hkv - 1) / a.Hkv - (h * a.N + a.Hkv - 1) / a.Hkv;
    nh_max = n > nh_max ? n : nh_max;
    any_odd |= n & 1;
  }
  const int pairs = nh_max / 2;
  if (pairs > 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<DQK, DV, 2>), dim3((unsigned)(dq_blocks * pairs)),
                       dim3(kBwdThreads), 0, stream, (const uint16_t*)a.q_sig,
                       (const uint16_t*)a.q_noise, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       a.lse, a.do_sig, a.do_noise, a.delta, (uint16_t*)a.dq_sig,
                       (uint16_t*)a.dq_noise, a.cu_q, a.cu_k, a.B, a.L, a.S, a.N, a.Hkv,
                       a.window, nqt, pairs, heavy_first, a.lse_b, a.lse_q, a.lse_h,
                       a.scale_log2, a.scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (any_odd) {
    hipLaunchKernelGGL((bwd_dq_kernel<DQK, DV, 1>), dim3((unsigned)dq_blocks), dim3(kBwdThreads),
                       0, stream, (const uint16_t*)a.q_sig, (const uint16_t*)a.q_noise,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, a.lse, a.do_sig, a.do_noise,
                       a.delta, (uint16_t*)a.dq_sig, (uint16_t*)a.dq_noise, a.cu_q, a.cu_k, a.B,
                       a.L, a.S, a.N, a.Hkv, a.window, nqt, 1, heavy_first, a.lse_b, a.lse_q,
                       a.lse_h, a.scale_log2, a.scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((bwd_dkdv_kernel<DQK, DV, kDkvTiles>), dim3((unsigned)dkv_blocks),
                     dim3(kBwdThreads), 0, stream, (const uint16_t*)a.q_sig,
                     (const uint16_t*)a.q_noise, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     a.lse, a.do_sig, a.do_noise, a.delta, (uint16_t*)a.dk,
                     (uint16_t*)a.dv_out, a.cu_q, a.cu_k, a.B, a.L, a.S, a.N, a.Hkv, a.window,
                     a.lse_b, a.lse_q, a.lse_h, a.scale_log2, a.scale);
  return hipGetLastError();
}

}  // namespace

bool bwd_bf16_supported(int dqk, int dv) {
  return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
}

size_t bwd_workspace_bytes(int B, int L, int S, int N, int dv) {
  const size_t rows = (size_t)B * L;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return up(rows * S * dv * 2) + up(rows * N * dv * 2) + up(rows * (S + N) * 4);
}

hipError_t launch_bwd_bf16(BwdArgs a, hipStream_t stream) {
  const size_t rows = (size_t)a.rows;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  unsigned char* w = (unsigned char*)a.workspace;
  a.do_sig = (uint16_t*)w;
  w += up(rows * a.S * a.dv * 2);
  a.do_noise = (uint16_t*)w;
  w += up(rows * a.N * a.dv * 2);
  a.delta = (float*)w;
  if (a.dqk == 64 && a.dv == 64) return launch_bwd_dims<64, 64>(a, stream);
  if (a.dqk == 128 && a.dv == 128) return launch_bwd_dims<128, 128>(a, stream);
  if (a.dqk == 192 && a.dv == 128) return launch_bwd_dims<192, 128>(a, stream);
  return (hipError_t)-1;
}

}  // namespace gda
