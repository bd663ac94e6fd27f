// gda_latent_bf16.hip - decode over the latent KV cache (GDLA's inference form), bf16, gfx950.
//
// The cache holds, per token, the KV latent c (Dc = 512 values, after its
// RMSNorm) and the decoupled rotary key (Dr = 64 values, shared by every head);
// W^KV_b [Hkv, Dn+dv, Dc] expands the latent into KV head h's key
// [W_k[h] c ; k_rope] and value W_v[h] c (Motif 3 walk-through, step 2: c_KV in
// R^512 -> RMSNorm -> W^KV_b -> 16 KV heads; novelty point one: both query paths
// share the up-projected KV and the broadcast rotary key, so the cache is the
// size of MLA's). The output is the same D_t times the gate as the other paths.
//
// Nothing is expanded. The key term q_nope . (W_k[h] c) is (W_k[h]^T q_nope) . c,
// and the value sum sum_s p_s W_v[h] c_s is W_v[h] (sum_s p_s c_s), so:
//  1. latent_absorb_kernel: q~ = [W_k[h]^T q_nope ; q_rope] (Dc + Dr values) for
//     every query head, rounded to bf16, into the workspace;
//  2. latent_attend_kernel: every query head of a sequence attends over the same
//     latent keys [c ; k_rope] with the latent c as the value (a multi-query
//     attention of all S + N heads); split-KV over workgroups, each writing
//     partial (max, sum, o) per head to the workspace;
//  3. latent_merge_kernel: merges the splits, up-projects o with W_v[h] (fp32),
//     and applies lambda and the gate.
// Reading 1152 B per cached token instead of Hkv * (dqk + dv) * 2 = 10240 B.
#include <mutex>

#include "../../include/gda.h"
#include "gda_device.hpp"
#include "gda_kernels.hpp"

// The workspace of the allocation-free entry point: a file-scope device array
// (each GPU holds its own copy). Host code must never pass its name to a kernel
// or a copy: the name is a host-side stand-in; latent_scratch() gives the
// device address.
static __device__ __align__(256) unsigned char scratch[GDA_DECODE_LATENT_SCRATCH_BYTES];

namespace gda {
namespace {

constexpr int LDN = 128, LDR = 64, LDC = 512, LDV = 128;  // compiled head sizes
constexpr int LQW = LDC + LDR;    // absorbed query width (576)
constexpr int LCK = 32;           // keys per chunk
constexpr int LNSTAGE = 3;        // chunk ring depth
constexpr int LC_BYTES = LCK * LDC * 2;                   // latent rows of a chunk (32 KB)
constexpr int LR_BYTES = LCK * LDR * 2;                   // rotary rows of a chunk (4 KB)
constexpr int LSTAGE = LC_BYTES + LR_BYTES;               // 36 KB
constexpr int LBLK = LSTAGE / 1024;                       // 1 KB copy blocks per chunk (36)
constexpr int LPART = 4 + LDC;    // floats per (split, head) partial: m, l, 2 pad, o[Dc]
constexpr int LMAX_WAVES = 8;     // up to 128 query heads (16 per wave)
constexpr float kLNoMax = -1e30f; // finite "no key seen yet" reference

// Slot of 16-byte piece p of latent row r: p ^ lswz(r). For the 16 rows of an
// MFMA fragment read (fixed p) the slots fall on 16 distinct bank groups, and
// for the transposed V^T reads (4 consecutive rows, a 32-byte piece pair each)
// the pairs stay adjacent and on distinct banks. The XOR stays inside the
// piece's aligned group of 16, so a row's slots are a permutation of its pieces.
__device__ __forceinline__ int lswz(int r) { return 2 * (r & 7) + ((r >> 3) & 1); }
// Rotary rows (8 pieces of 16 bytes): the same rule as 128-byte K rows.
__device__ __forceinline__ int rswz(int r) { return (r >> 1) & 7; }

// Heads of KV head h: signal i when floor(i*Hkv/S) == h, noise j when floor(j*Hkv/N) == h.
// Column of a head in the workspace: signal i -> i, noise j -> S + j.

// ---- 1. absorb ----------------------------------------------------------------
constexpr int ABS_SEQ = 4;  // sequences per absorb workgroup (the weight slice is loaded once)

// One workgroup per (KV head h, ABS_SEQ sequences). Thread t owns latent columns
// 8(t%64) .. +7 and key dims 32(t/64) .. +31 of W_k[h], loaded once with 32
// independent 16-byte loads; for each sequence and group of 4 heads the four dim
// quarters are summed through LDS.
__global__ void __launch_bounds__(256)
latent_absorb_kernel(const uint16_t* __restrict__ q_sig, const uint16_t* __restrict__ q_noise,
                     const uint16_t* __restrict__ w_kv_b, uint16_t* __restrict__ qa, int B,
                     int S, int N, int Hkv, int XP) {
  constexpr int MAXH = 16, HG = 4;
  __shared__ float sq[MAXH][LDN];
  __shared__ float sred[4][HG][LDC];
  __shared__ int scol[MAXH];
  __shared__ int snh;
  const int h = blockIdx.x % Hkv, b0 = (blockIdx.x / Hkv) * ABS_SEQ;
  const int tid = threadIdx.x;
  if (tid == 0) {
    int n = 0;
    for (int i = 0; i < S && n < MAXH; ++i)
      if ((int)(((int64_t)i * Hkv) / S) == h) scol[n++] = i;
    for (int j = 0; j < N && n < MAXH; ++j)
      if ((int)(((int64_t)j * Hkv) / N) == h) scol[n++] = S + j;
    snh = n;
  }
  const int cg = tid & 63, dq = tid >> 6;
  const uint16_t* w = w_kv_b + ((int64_t)h * (LDN + LDV) + 32 * dq) * LDC + 8 * cg;
  u32x4 wr[32];
#pragma unroll
  for (int d = 0; d < 32; ++d) wr[d] = ldg16(w + (int64_t)d * LDC);
  __syncthreads();
  const int nh = snh;
  for (int b = b0; b < min(B, b0 + ABS_SEQ); ++b) {
    for (int idx = tid; idx < nh * LDN; idx += 256) {
      const int x = idx / LDN, d = idx - (idx / LDN) * LDN;
      const int col = scol[x];
      const uint16_t* q = col < S ? q_sig + ((int64_t)b * S + col) * (LDN + LDR)
                                  : q_noise + ((int64_t)b * N + (col - S)) * (LDN + LDR);
      sq[x][d] = bf16_to_f32(q[d]);
    }
    __syncthreads();
    for (int h0 = 0; h0 < nh; h0 += HG) {
      float acc[HG][8];
#pragma unroll
      for (int x = 0; x < HG; ++x)
#pragma unroll
        for (int u = 0; u < 8; ++u) acc[x][u] = 0.f;
#pragma unroll
      for (int d = 0; d < 32; ++d) {
#pragma unroll
        for (int x = 0; x < HG; ++x) {
          const float qv = sq[min(h0 + x, nh - 1)][32 * dq + d];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            acc[x][2 * u] = fmaf(qv, bf16_lo(wr[d][u]), acc[x][2 * u]);
            acc[x][2 * u + 1] = fmaf(qv, bf16_hi(wr[d][u]), acc[x][2 * u + 1]);
          }
        }
      }
#pragma unroll
      for (int x = 0; x < HG; ++x)
#pragma unroll
        for (int u = 0; u < 8; ++u) sred[dq][x][8 * cg + u] = acc[x][u];
      __syncthreads();
      for (int idx = tid; idx < HG * LDC; idx += 256) {
        const int x = idx / LDC, cidx = idx - (idx / LDC) * LDC;
        if (h0 + x < nh) {
          const float v =
              (sred[0][x][cidx] + sred[1][x][cidx]) + (sred[2][x][cidx] + sred[3][x][cidx]);
          qa[((int64_t)b * XP + scol[h0 + x]) * LQW + cidx] = f32_to_bf16(v);
        }
      }
      __syncthreads();
    }
    // The rotary part of each query is copied as it is.
    for (int idx = tid; idx < nh * LDR; idx += 256) {
      const int x = idx / LDR, r = idx - (idx / LDR) * LDR;
      const int col = scol[x];
      const uint16_t* q = col < S ? q_sig + ((int64_t)b * S + col) * (LDN + LDR)
                                  : q_noise + ((int64_t)b * N + (col - S)) * (LDN + LDR);
      qa[((int64_t)b * XP + col) * LQW + LDC + r] = q[LDN + r];
    }
    // Padding columns (S + N .. XP-1) are zero queries; the workgroups of KV head 0 clear them.
    if (h == 0)
      for (int idx = tid; idx < (XP - S - N) * LQW; idx += 256)
        qa[((int64_t)b * XP + S + N) * LQW + idx] = 0;
  }
}

// ---- 2. attend ----------------------------------------------------------------
// Wait until at most n (a wave's copy blocks per chunk: 36 dealt over 1..8 waves)
// vector-memory operations are outstanding.
__device__ __forceinline__ void wait_own_blocks(int n) {
  switch (n) {
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 18: wait_vmcnt<18>(); break;
    case 36: wait_vmcnt<36>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// One workgroup per (sequence b, split k); wave w owns query-head columns
// 16w .. 16w+15. Chunk j's 36 copy blocks (32 latent rows, 4 rotary blocks of 8
// rows) are dealt round-robin to the waves.
__global__ void __launch_bounds__(64 * LMAX_WAVES, 1)
latent_attend_kernel(const uint16_t* __restrict__ qa, const uint16_t* __restrict__ c_kv,
                     const uint16_t* __restrict__ k_rope, const int32_t* __restrict__ lens,
                     float* __restrict__ part, int Lmax, int window, int nsplit, int XP,
                     float c) {
  __shared__ __attribute__((aligned(1024))) unsigned char ring[LNSTAGE * LSTAGE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, nw = blockDim.x >> 6;
  const int col = lane & 15, g4 = lane >> 4;
  const int b = blockIdx.x / nsplit, k = blockIdx.x - (blockIdx.x / nsplit) * nsplit;
  float* pw = part + (((int64_t)b * nsplit + k) * XP + 16 * wave) * LPART;

  int len = lens ? lens[b] : Lmax;
  if (len > Lmax) len = Lmax;
  const int pos = len - 1;
  const int lo = window ? max(0, pos - window + 1) : 0;
  const int nch = len >= 1 ? (pos - lo + LCK) / LCK : 0;
  const int c0 = (int)(((int64_t)k * nch) / nsplit), c1 = (int)(((int64_t)(k + 1) * nch) / nsplit);

  // Absorbed queries of this wave's 16 heads as MFMA B operands (Q~^T).
  bf16x8 qf[LQW / 32];
  {
    const uint16_t* qp = qa + ((int64_t)b * XP + 16 * wave + col) * LQW + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < LQW / 32; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ldg16(qp + 32 * ks));
#pragma unroll
    for (int ks = 0; ks < LQW / 32; ++ks) settle(qf[ks]);  // before any copy is issued
  }
  float mref = kLNoMax, lsum = 0.f;
  floatx4 o[LDC / 16];
#pragma unroll
  for (int db = 0; db < LDC / 16; ++db) o[db] = floatx4{0.f, 0.f, 0.f, 0.f};

  const uint32_t ring_lds = (uint32_t)(uintptr_t)(const lds_void*)ring;
  const char* cbase = (const char*)(c_kv + (int64_t)b * Lmax * LDC);
  const char* rbase = (const char*)(k_rope + (int64_t)b * Lmax * LDR);
  // Copies of this wave's blocks of chunk j into stage st; rows past pos read row pos.
  auto issue = [&](int j, int st) {
    const int s0 = lo + j * LCK;
    const int last = pos - s0;  // rows 0 .. last are visible
    const uint32_t dst = ring_lds + (uint32_t)(st * LSTAGE);
    for (int blk = wave; blk < LBLK; blk += nw) {
      if (blk < LCK) {  // latent row blk: 64 pieces, piece lane ^ lswz(row) into slot lane
        const int r = min(blk, last);
        const uint32_t voff = (uint32_t)r * (LDC * 2) + 16u * (uint32_t)(lane ^ lswz(blk));
        dma16_lds_nt(cbase + (int64_t)s0 * (LDC * 2), voff, dst + 1024u * blk);
      } else {  // rotary rows 8q .. 8q+7, 8 pieces each
        const int q = blk - LCK;
        const int rr = 8 * q + (lane >> 3);
        const int r = min(rr, last);
        const uint32_t voff = (uint32_t)r * (LDR * 2) + 16u * (uint32_t)((lane & 7) ^ rswz(rr));
        dma16_lds_nt(rbase + (int64_t)s0 * (LDR * 2), voff, dst + 1024u * blk);
      }
    }
  };
  // Blocks this wave issues per chunk (the same for every chunk).
  const int nmine = (LBLK - wave + nw - 1) / nw;

  // Per-lane parts of the fragment addresses (see the reads below).
  int kbase, ktab[4], rtab[LDR / 32], vbase, vtab[8];
  {
    const int f = lswz(col);  // rows col and col+16
    kbase = col * (LDC * 2) + 16 * (g4 ^ (f & 3));
#pragma unroll
    for (int t = 0; t < 4; ++t) ktab[t] = 64 * (t ^ (f >> 2));
#pragma unroll
    for (int ks = 0; ks < LDR / 32; ++ks) rtab[ks] = col * (LDR * 2) + ((((4 * ks + g4) ^ rswz(col))) << 4);
    const int rv = 4 * g4 + (col >> 2);  // rows rv and rv+16
    const int fv = lswz(rv);
    vbase = rv * (LDC * 2) + 16 * (((col & 3) >> 1) ^ (fv & 1)) + 8 * (col & 1);
#pragma unroll
    for (int t = 0; t < 8; ++t) vtab[t] = 32 * (t ^ (rv & 7));
  }
  if (c0 < c1) issue(c0, 0);
  if (c0 + 1 < c1) issue(c0 + 1, 1);
#pragma unroll 1
  for (int j = c0; j < c1; ++j) {
    const int st = (j - c0) % LNSTAGE;
    // This wave's copies of chunk j have landed once only chunk j+1's may be outstanding.
    if (j + 1 < c1)
      wait_own_blocks(nmine);
    else
      wait_vmcnt<0>();
    __syncthreads();  // every wave's copies of chunk j landed; chunk j-1's stage is free
    if (j + 2 < c1) issue(j + 2, (j + 2 - c0) % LNSTAGE);
    const unsigned char* sC = ring + st * LSTAGE;
    const unsigned char* sR = sC + LC_BYTES;
    const int s0 = lo + j * LCK;
    // S^T = [c ; k_rope] . Q~^T (16 keys x 32 dims per MFMA). Piece 4ks+g4 of row
    // r sits at slot 4(ks ^ (f>>2)) + (g4 ^ (f&3)), f = lswz(r) (the same for r and
    // r+16): a per-lane base, a 4-entry per-lane table and an immediate.
    floatx4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < LDC / 32; ++ks) {
        const bf16x8 a = *(const bf16x8*)(sC + kbase + kb * (16 * LDC * 2) + 256 * (ks >> 2) +
                                          ktab[ks & 3]);
        s[kb] = mfma_16x16x32(a, qf[ks], s[kb]);
      }
#pragma unroll
      for (int ks = 0; ks < LDR / 32; ++ks) {
        const bf16x8 a = *(const bf16x8*)(sR + kb * (16 * LDR * 2) + rtab[ks]);
        s[kb] = mfma_16x16x32(a, qf[LDC / 32 + ks], s[kb]);
      }
    }
    if (s0 + LCK - 1 > pos) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (s0 + 16 * kb + 4 * g4 + r > pos) s[kb][r] = -INFINITY;
    }
    // Online softmax per column (query head), lazily rescaled.
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    if (__builtin_amdgcn_ballot_w64(mx * c > mref + 8.f)) {
      const float mnew = fmaxf(mref, col_max4(mx) * c);
      const float alpha = fast_exp2(mref - mnew);
      mref = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < LDC / 16; ++db)
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
    // O^T (latent dims x heads) += C^T . P^T, C^T from transposed reads.
    // Piece 2db+u of row r sits at slot 2((db&~7) + ((db&7) ^ (r&7))) + (u ^ (f&1)).
#pragma unroll
    for (int db = 0; db < LDC / 16; ++db) {
      shortx4 half[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const unsigned char* va = sC + vbase + hf * (16 * LDC * 2) + 256 * (db >> 3) + vtab[db & 7];
        half[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)va);
      }
      typedef __attribute__((__vector_size__(8 * sizeof(short)))) short shortx8;
      const shortx8 a8 = {half[0][0], half[0][1], half[0][2], half[0][3],
                          half[1][0], half[1][1], half[1][2], half[1][3]};
      o[db] = mfma_16x16x32(__builtin_bit_cast(bf16x8, a8), pb, o[db]);
    }
  }
  lsum = col_sum4(lsum);
  // Partials of this wave's 16 heads: m (log2 units), l, o[Dc] (unnormalised).
  float* ph = pw + col * LPART;
  if (g4 == 0) {
    ph[0] = mref;
    ph[1] = lsum;
  }
#pragma unroll
  for (int db = 0; db < LDC / 16; ++db)
    *(floatx4*)(ph + 4 + 16 * db + 4 * g4) = o[db];
}

// ---- 3. merge, up-project, epilogue ------------------------------------------------
// One workgroup per (sequence b, noise head j): heads = noise j and its g signal
// heads g*j .. g*j+g-1. Each head's o is merged over the splits (fp32, in LDS),
// then H[e] = W_v[h] o (fp32, one dot product per thread), then
// out = gate * (H_S - lambda * H_N).
__global__ void __launch_bounds__(256)
latent_merge_kernel(const float* __restrict__ part, const uint16_t* __restrict__ w_kv_b,
                    const int32_t* __restrict__ lens, const uint16_t* __restrict__ lam,
                    const uint16_t* __restrict__ gate, uint16_t* __restrict__ out, int Lmax,
                    int S, int N, int Hkv, int nsplit, int XP, int flags) {
  constexpr int MAXG = 15;
  __shared__ float so[MAXG + 1][LDC];   // merged o: [0] noise, [1 + t] signal g*j + t
  __shared__ float sH[MAXG + 1][LDV];   // up-projected outputs
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = blockIdx.x / N, j = blockIdx.x - (blockIdx.x / N) * N;
  const int g = S / N;
  const int nh = 1 + g;
  int len = lens ? lens[b] : Lmax;
  if (len > Lmax) len = Lmax;
  if (len < 1) {
    for (int idx = tid; idx < g * LDV; idx += 256)
      out[((int64_t)b * S + g * j + idx / LDV) * LDV + idx % LDV] = 0;
    return;
  }
  // Merge: thread t owns latent dims t and t+256 of every head.
  for (int x = 0; x < nh; ++x) {
    const int col = x == 0 ? S + j : g * j + (x - 1);
    const float* p0 = part + ((int64_t)b * nsplit * XP + col) * LPART;
    float M = -INFINITY;
    for (int k = 0; k < nsplit; ++k) M = fmaxf(M, p0[(int64_t)k * XP * LPART]);
    float L = 0.f, a0 = 0.f, a1 = 0.f;
    for (int k = 0; k < nsplit; ++k) {
      const float* pk = p0 + (int64_t)k * XP * LPART;
      const float wk = fast_exp2(pk[0] - M);
      L += wk * pk[1];
      a0 += wk * pk[4 + tid];
      a1 += wk * pk[4 + tid + 256];
    }
    so[x][tid] = a0 / L;
    so[x][tid + 256] = a1 / L;
  }
  __syncthreads();
  // Up-projection: thread-owned dot products H[x][e] = W_v[h(x)] row e . o_x (fp32),
  // 16-byte weight loads, o from LDS (the same address across a wave: a broadcast).
  for (int idx = tid; idx < nh * LDV; idx += 256) {
    const int x = idx / LDV, e = idx - (idx / LDV) * LDV;
    const int col = x == 0 ? S + j : g * j + (x - 1);
    const int h = x == 0 ? (int)(((int64_t)j * Hkv) / N) : (int)(((int64_t)col * Hkv) / S);
    const uint16_t* wv = w_kv_b + ((int64_t)h * (LDN + LDV) + LDN + e) * LDC;
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll 16
    for (int c8 = 0; c8 < LDC / 8; ++c8) {
      const u32x4 w = ldg16(wv + 8 * c8);
      const float* ov = &so[x][8 * c8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc0 = fmaf(bf16_lo(w[u]), ov[2 * u], acc0);
        acc1 = fmaf(bf16_hi(w[u]), ov[2 * u + 1], acc1);
      }
    }
    sH[x][e] = acc0 + acc1;
  }
  __syncthreads();
  for (int idx = tid; idx < g * LDV; idx += 256) {
    const int t = idx / LDV, e = idx - (idx / LDV) * LDV;
    const int i = g * j + t;
    float lm = bf16_to_f32(lam[(int64_t)b * S + i]);
    if (flags & kLambdaLogits) lm = sigmoid_f32(lm);
    const int64_t o_idx = ((int64_t)b * S + i) * LDV + e;
    float gv = bf16_to_f32(gate[o_idx]);
    if (flags & kGateLogits) gv = sigmoid_f32(gv);
    out[o_idx] = f32_to_bf16(gv * (sH[1 + t][e] - lm * sH[0][e]));
  }
}

// Splits per sequence: enough workgroups for the CUs, at least 4 chunks each.
int latent_nsplit(int B, int Lmax, int window) {
  const int span = window > 0 && window < Lmax ? window : Lmax;
  const int nch = (span + LCK - 1) / LCK;
  int ns = (512 + B - 1) / B;
  ns = min(ns, max(1, nch / 4));
  return max(1, min(ns, 64));
}

}  // namespace

bool latent_supported(int Dn, int Dr, int Dc, int dv, int S, int N, int Hkv) {
  if (Dn != LDN || Dr != LDR || Dc != LDC || dv != LDV) return false;
  if (S + N > 16 * LMAX_WAVES) return false;
  if (S / N > 15) return false;
  // The absorb kernel takes at most 16 query heads per KV head.
  int worst = 0;
  for (int h = 0; h < Hkv; ++h) {
    int n = 0;
    for (int i = 0; i < S; ++i) n += (int)(((int64_t)i * Hkv) / S) == h;
    for (int j = 0; j < N; ++j) n += (int)(((int64_t)j * Hkv) / N) == h;
    worst = max(worst, n);
  }
  return worst <= 16;
}

size_t latent_workspace_bytes(int B, int Lmax, int S, int N, int window) {
  const int XP = ((S + N + 15) / 16) * 16;
  const int ns = latent_nsplit(B, Lmax, window);
  const size_t qa = (size_t)B * XP * LQW * 2;
  const size_t qa_pad = (qa + 255) & ~(size_t)255;
  return qa_pad + (size_t)B * ns * XP * LPART * 4;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t latent_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_latent(const LatentArgs& a, hipStream_t stream) {
  const int XP = ((a.S + a.N + 15) / 16) * 16;
  const int ns = latent_nsplit(a.B, a.Lmax, a.window);
  const size_t qa_bytes = ((size_t)a.B * XP * LQW * 2 + 255) & ~(size_t)255;
  uint16_t* qa = (uint16_t*)a.workspace;
  float* part = (float*)((char*)a.workspace + qa_bytes);
  const int64_t g1 = (int64_t)((a.B + ABS_SEQ - 1) / ABS_SEQ) * a.Hkv;
  const int64_t g2 = (int64_t)a.B * ns, g3 = (int64_t)a.B * a.N;
  if (g1 > 0x7fffffff || g2 > 0x7fffffff || g3 > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(latent_absorb_kernel, dim3((unsigned)g1), dim3(256), 0, stream,
                     (const uint16_t*)a.q_sig, (const uint16_t*)a.q_noise,
                     (const uint16_t*)a.w_kv_b, qa, a.B, a.S, a.N, a.Hkv, XP);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(latent_attend_kernel, dim3((unsigned)g2), dim3(64 * (XP / 16)), 0, stream,
                     (const uint16_t*)qa, (const uint16_t*)a.c_kv, (const uint16_t*)a.k_rope,
                     a.lens, part, a.Lmax, a.window, ns, XP, a.scale_log2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(latent_merge_kernel, dim3((unsigned)g3), dim3(256), 0, stream,
                     (const float*)part, (const uint16_t*)a.w_kv_b, a.lens,
                     (const uint16_t*)a.lam, (const uint16_t*)a.gate, (uint16_t*)a.out, a.Lmax,
                     a.S, a.N, a.Hkv, ns, XP, a.flags);
  return hipGetLastError();
}

}  // namespace gda
