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
//  1. latent_absorb2_kernel: q~ = [W_k[h]^T q_nope ; q_rope] (Dc + Dr values) for
//     every query head, on the matrix cores, rounded to bf16, into the workspace;
//  2. latent_attend2_kernel (up to 80 query heads; latent_attend_kernel above
//     that): every query head of a sequence attends over the same latent keys
//     [c ; k_rope] with the latent c as the value (a multi-query attention of all
//     S + N heads); split-KV over workgroups, each writing partial (max, sum, o)
//     per head to the workspace;
//  3. latent_merge_kernel: merges the splits, up-projects o with W_v[h] (matrix
//     cores, several sequences per workgroup), and applies lambda and the gate.
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

// Slot of 16-byte piece p of latent row r: p ^ lswz(r), a function of r % 16 (so
// rows r and r + 16 of a chunk share it). Over the 16 rows of an MFMA fragment
// read (fixed p) lswz takes all 16 values, and over each aligned run of 8 rows
// its low three bits take all 8: the read is free of bank conflicts whether the
// LDS serves 16 lanes of 16 bytes per cycle or 8. For the transposed V^T reads
// (a 32-byte piece pair per row; pair index ^ lswz(r) / 2) lswz / 2 takes 8
// distinct values over each aligned 8 rows and 4 over each aligned 4. The XOR
// stays inside the piece's aligned group of 16, so a row's slots are a
// permutation of its pieces and the piece pairs stay adjacent.
__device__ __forceinline__ int lswz(int r) {
  return 2 * (r & 3) + ((r >> 2) & 1) + 8 * (((r >> 2) ^ (r >> 3)) & 1);
}
// Rotary rows (8 pieces of 16 bytes, two rows per 256 bytes): slot p ^ rswz(r),
// distinct over each aligned 8 rows and, with the row's half of 256 bytes, over 16.
__device__ __forceinline__ int rswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Heads of KV head h: signal i when floor(i*Hkv/S) == h, noise j when floor(j*Hkv/N) == h.
// Column of a head in the workspace: signal i -> i, noise j -> S + j.

// ---- 1. absorb on the matrix cores ---------------------------------------------
// Per KV head h the absorbed queries are one small GEMM: Q~^T[c][col] =
// sum_d W_k[h][d][c] q_nope[col][d] over the query columns col that read h. One
// workgroup per (h, block of AB_COLS columns) stages W_k[h] (128 rows of 1 KB)
// in LDS with direct copies, 32-byte chunk pairs XOR-swizzled by row (pair ^=
// row % 8), so that the W_k^T operand (16 latent dims x 32 rows) comes from
// conflict-free transposed reads; each wave takes 16 columns, holds their q_nope
// as the B operand (4 k-steps) and walks the 32 tiles of 16 latent dims, rounding
// each fp32 result to bf16 once. The rotary part of each query is copied, and
// padding columns are cleared by the workgroups of h = 0.
constexpr int AB_COLS = 64;  // query columns per workgroup (16 per wave)

__global__ void __launch_bounds__(256)
latent_absorb2_kernel(const uint16_t* __restrict__ q_sig, const uint16_t* __restrict__ q_noise,
                      const uint16_t* __restrict__ w_kv_b, uint16_t* __restrict__ qa, int B,
                      int S, int N, int Hkv, int XP) {
  __shared__ __attribute__((aligned(1024))) uint16_t sW[LDN * LDC];  // 128 KB
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g4 = lane >> 4;
  // Query heads of KV head h: signal heads h*NS .. +NS-1, then noise heads
  // ceil(h*N/Hkv) .. ceil((h+1)*N/Hkv)-1.
  const int NS = S / Hkv;
  const int nblk = (int)(((int64_t)B * (NS + (N + Hkv - 1) / Hkv) + AB_COLS - 1) / AB_COLS);
  const int h = blockIdx.x / nblk, blk = blockIdx.x - (blockIdx.x / nblk) * nblk;
  const int n0 = (int)(((int64_t)h * N + Hkv - 1) / Hkv);
  const int n1 = (int)(((int64_t)(h + 1) * N + Hkv - 1) / Hkv);
  const int nkv = NS + (n1 - n0);          // query heads on h
  const int ncols = B * nkv;               // (sequence, head) columns of h
  if (blk * AB_COLS >= ncols) return;

  // W_k[h] -> LDS: row d is 1 KB (64 pieces of 16 bytes), piece p stored at slot
  // p ^ ((d & 7) << 1); wave w copies rows w, w+4, ...
  {
    const char* wk = (const char*)(w_kv_b + (int64_t)h * (LDN + LDV) * LDC);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const lds_void*)sW;
    for (int d = wave; d < LDN; d += 4)
      dma16_lds(wk + (int64_t)d * LDC * 2, 16u * (uint32_t)(lane ^ ((d & 7) << 1)),
                lds0 + 1024u * (uint32_t)d);
  }
  // This wave's 16 columns: q_nope as the B operand (k-step ks: dims 32ks + 8 g4 ..).
  const int c0 = blk * AB_COLS + 16 * wave + col;  // this lane's column
  const bool live = c0 < ncols;
  const int cb = live ? c0 / nkv : 0, cx = live ? c0 - (c0 / nkv) * nkv : 0;
  const int head = cx < NS ? h * NS + cx : S + n0 + (cx - NS);
  const uint16_t* q = cx < NS ? q_sig + ((int64_t)cb * S + h * NS + cx) * (LDN + LDR)
                              : q_noise + ((int64_t)cb * N + n0 + (cx - NS)) * (LDN + LDR);
  bf16x8 qb[LDN / 32];
#pragma unroll
  for (int ks = 0; ks < LDN / 32; ++ks) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (live) w = ldg16(q + 32 * ks + 8 * g4);
    qb[ks] = __builtin_bit_cast(bf16x8, w);
  }
  // The rotary part: lanes with g4 < 2 copy 32 of their column's 64 values each.
  if (live && g4 < 2) {
    const uint16_t* src = q + LDN + 32 * g4;
    uint16_t* dst = qa + ((int64_t)cb * XP + head) * LQW + LDC + 32 * g4;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)(dst + 8 * i) = ldg16(src + 8 * i);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // W_k[h] is in LDS
  uint16_t* dst = qa + ((int64_t)cb * XP + head) * LQW + 4 * g4;
#pragma unroll 4
  for (int ct = 0; ct < LDC / 16; ++ct) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < LDN / 32; ++ks) {
      shortx4 half[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        // rows 32 ks + 8 g4 + 4 hf .. +3: lane (col, g4) gets W_k^T[16 ct + col][k]
        // for k = 8 g4 .. 8 g4 + 7 in order, the k order of the q_nope operand
        const int r = 32 * ks + 8 * g4 + 4 * hf + (col >> 2);
        const int chunk = 2 * ct + ((col & 3) >> 1);
        const uint16_t* va = sW + r * LDC + ((chunk ^ ((r & 7) << 1)) << 3) + 4 * (col & 1);
        half[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)va);
      }
      typedef __attribute__((__vector_size__(8 * sizeof(short)))) short shortx8;
      const shortx8 a8 = {half[0][0], half[0][1], half[0][2], half[0][3],
                          half[1][0], half[1][1], half[1][2], half[1][3]};
      acc = mfma_16x16x32(__builtin_bit_cast(bf16x8, a8), qb[ks], acc);
    }
    // lane (col, g4) holds latent dims 16 ct + 4 g4 .. +3 of its column
    if (live) *(u32x2*)(dst + 16 * ct) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  }
  // Padding columns S+N .. XP-1 are zero queries (cleared by the workgroups of h = 0).
  if (h == 0 && XP > S + N)
    for (int64_t idx = (int64_t)blk * 256 + tid; idx < (int64_t)B * (XP - S - N) * LQW;
         idx += (int64_t)nblk * 256) {
      const int64_t bb = idx / ((XP - S - N) * LQW), rem = idx - bb * ((XP - S - N) * LQW);
      qa[(bb * XP + S + N) * LQW + rem] = 0;
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
    for (int t = 0; t < 8; ++t) vtab[t] = 32 * (t ^ (fv >> 1));
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

// ---- 2'. attend, 8 waves in two roles (up to 5 head tiles) -------------------------
// The kernel above gives each wave 16 heads over the whole chunk, so every wave
// reads all 36 KB of the chunk from LDS and 5 head tiles load one SIMD twice.
// Here the work of a 32-key chunk is split by role:
//  * score waves (wave s < (HT+1)/2): head tiles 2s and 2s+1 (the last score wave
//    of an odd HT takes one): their absorbed queries for all 18 k-steps sit in
//    registers; the wave computes the tiles' complete S^T for both 16-key halves
//    of the chunk, each K fragment read serving both tiles, keeps their online
//    softmax (running reference and sum) and writes their P^T operands and
//    rescale factors;
//  * the other waves (and the one-tile score wave) accumulate O^T for runs of the
//    32 tiles of 16 latent dims and every head tile, sized so that the matrix
//    work per SIMD is even.
// The K fragment reads (the largest LDS stream: 36 KB per score wave and chunk)
// are what the score products wait on, so fewer score waves each serving two
// tiles halve them.
// One workgroup barrier per chunk: in step j the score waves take chunk j's
// scores and softmax while the other waves add chunk j-1's P.V (P^T and the
// rescale factors are double-buffered). The ring holds four chunks: j-1 and j are
// read in step j, j+1 is in flight, and j+2 goes into the stage of chunk j-2 right
// after the barrier, two steps before it is needed.
constexpr int A2_WAVES = 8;
constexpr int A2_KSTEPS = (LDC + LDR) / 32;       // 18 k-steps of the scores
constexpr int A2_NSTAGE = 4;                      // chunk ring depth
constexpr int A2_AH = 8;                          // K fragment reads in flight (score waves)
constexpr int A2_MAX_HT = 5;

template <int HT>
struct Attend2Smem {
  unsigned char ring[A2_NSTAGE * LSTAGE];          // latent + rotary rows of 4 chunks
  bf16x8 pt[2][HT][64];                             // P^T operands [step parity][tile][lane]
  float alpha[2][HT][16];                           // rescale factors, per head column
  int rescaled[2][HT];                              // tile t raised its reference
};
static_assert(sizeof(Attend2Smem<A2_MAX_HT>) <= 160 * 1024, "LDS of one workgroup per CU");

// First 16-dim O^T tile of wave w (the counts are the ND of its role). Five
// head tiles: waves 0 and 1 score two tiles each and take no dims, wave 2
// scores one and takes 2 dims, waves 4 and 5 take 3 and waves 3, 6, 7 take 8:
// 80-87 matrix instructions per SIMD and chunk (wave w runs on SIMD w % 4).
// Fewer head tiles: waves 4-7 take 8 dims each, the others none.
template <int HT>
__device__ __forceinline__ int a2_first_dim_tile(int w) {
  if constexpr (HT == A2_MAX_HT) return w == 3 ? 2 : w == 4 ? 10 : w == 5 ? 13 : w >= 6 ? 8 * (w - 4) : 0;
  return w >= 4 ? 8 * (w - 4) : 0;
}

// One wave's whole loop: NTS head tiles scored (0: none), ND dim tiles of O^T.
template <int HT, int NTS, int ND>
__device__ __forceinline__ void attend2_wave(Attend2Smem<HT>& sm, const uint16_t* __restrict__ qa,
                                             const char* cbase, const char* rbase,
                                             float* __restrict__ pw, int b, int wave, int lane,
                                             int lo, int pos, int c0, int c1, float c) {
  constexpr int XP = 16 * HT;
  constexpr int NQ = NTS > 0 ? NTS : 1;
  const int col = lane & 15, g4 = lane >> 4;
  const int d0 = a2_first_dim_tile<HT>(wave);
  const int t0 = 2 * wave;  // first head tile of a score wave

  // Score waves: their head tiles' absorbed queries, every k-step, as MFMA B
  // operands (Q~^T: 32 dims x 16 heads).
  bf16x8 qf[NQ][A2_KSTEPS];
  if constexpr (NTS > 0) {
#pragma unroll
    for (int u = 0; u < NTS; ++u) {
      const uint16_t* qp = qa + ((int64_t)b * XP + 16 * (t0 + u) + col) * LQW + 8 * g4;
#pragma unroll
      for (int ks = 0; ks < A2_KSTEPS; ++ks)
        qf[u][ks] = __builtin_bit_cast(bf16x8, ldg16(qp + 32 * ks));
    }
#pragma unroll
    for (int u = 0; u < NTS; ++u)
#pragma unroll
      for (int ks = 0; ks < A2_KSTEPS; ++ks) settle(qf[u][ks]);  // before any copy is issued
  }
  // O^T: dims 16 (d0 + dt) + (4 g4 .. +3), head 16 t + col.
  floatx4 o[ND > 0 ? ND : 1][HT];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int t = 0; t < HT; ++t) o[dt][t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float mref[NQ], lsum[NQ];  // the scored tiles' softmax state
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    mref[u] = kLNoMax;
    lsum[u] = 0.f;
  }

  const uint32_t ring_lds = (uint32_t)(uintptr_t)(const lds_void*)sm.ring;
  auto issue = [&](int j) {
    const int s0 = lo + j * LCK;
    const int last = pos - s0;
    const uint32_t dst = ring_lds + (uint32_t)(((j - c0) & (A2_NSTAGE - 1)) * LSTAGE);
    for (int blk = wave; blk < LBLK; blk += A2_WAVES) {
      if (blk < LCK) {
        const int r = min(blk, last);
        const uint32_t voff = (uint32_t)r * (LDC * 2) + 16u * (uint32_t)(lane ^ lswz(blk));
        dma16_lds_nt(cbase + (int64_t)s0 * (LDC * 2), voff, dst + 1024u * blk);
      } else {
        const int q = blk - LCK;
        const int rr = 8 * q + (lane >> 3);
        const int r = min(rr, last);
        const uint32_t voff = (uint32_t)r * (LDR * 2) + 16u * (uint32_t)((lane & 7) ^ rswz(rr));
        dma16_lds_nt(rbase + (int64_t)s0 * (LDR * 2), voff, dst + 1024u * blk);
      }
    }
  };
  const int nmine = (LBLK - wave + A2_WAVES - 1) / A2_WAVES;

  // Per-lane parts of the fragment addresses (the layout of the kernel above):
  // K fragment of key half kh, k-step ks: row 16 kh + col; V^T fragment of dim
  // tile d0 + dt: vofs[dt] within each 16-row half of the chunk.
  int kbase, ktab[4], rtab[LDR / 32], vofs[ND > 0 ? ND : 1];
  {
    const int f = lswz(col);
    kbase = col * (LDC * 2) + 16 * (g4 ^ (f & 3));
#pragma unroll
    for (int t = 0; t < 4; ++t) ktab[t] = 64 * (t ^ (f >> 2));
#pragma unroll
    for (int ks = 0; ks < LDR / 32; ++ks) rtab[ks] = col * (LDR * 2) + ((((4 * ks + g4) ^ rswz(col))) << 4);
    const int rv = 4 * g4 + (col >> 2);
    const int fv = lswz(rv);
    const int vbase = rv * (LDC * 2) + 16 * (((col & 3) >> 1) ^ (fv & 1)) + 8 * (col & 1);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      const int db = d0 + dt;
      vofs[dt] = vbase + 256 * (db >> 3) + 32 * ((db & 7) ^ (fv >> 1));
    }
  }
  auto stage_of = [&](int j) { return sm.ring + ((j - c0) & (A2_NSTAGE - 1)) * LSTAGE; };

  // Chunk j's scores of the wave's head tiles (both key halves, all k-steps) and
  // their softmax step: running reference and sum, the P^T operand and the
  // rescale flag and factors, into the buffers of step parity j & 1.
  auto scores_softmax = [&](int j) {
    const unsigned char* sC = stage_of(j);
    const unsigned char* sR = sC + LC_BYTES;
    floatx4 sk[NQ][2];
#pragma unroll
    for (int u = 0; u < NQ; ++u) sk[u][0] = sk[u][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < A2_KSTEPS; ++ks) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        bf16x8 a;
        if (ks < LDC / 32)
          a = *(const bf16x8*)(sC + kbase + kh * (16 * LDC * 2) + 256 * (ks >> 2) + ktab[ks & 3]);
        else
          a = *(const bf16x8*)(sR + kh * (16 * LDR * 2) + rtab[ks - LDC / 32]);
#pragma unroll
        for (int u = 0; u < NTS; ++u) sk[u][kh] = mfma_16x16x32(a, qf[u][ks], sk[u][kh]);
      }
    }
    // Schedule: the first A2_AH fragment reads, then each fragment's products
    // followed by the read A2_AH fragments ahead, so the LDS latency hides behind
    // the products (left to itself the compiler keeps one or two reads in flight).
    __builtin_amdgcn_sched_group_barrier(0x100, A2_AH, 0);
#pragma unroll
    for (int i = 0; i < 2 * A2_KSTEPS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, NTS, 0);
      if (i + A2_AH < 2 * A2_KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    const int s0 = lo + j * LCK;
    const int par = j & 1;
#pragma unroll
    for (int u = 0; u < NTS; ++u) {
      floatx4 (&s)[2] = sk[u];
      const int tt = t0 + u;
      if (s0 + LCK - 1 > pos) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (s0 + 16 * h + 4 * g4 + r > pos) s[h][r] = -INFINITY;
      }
      const float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                             fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
      int resc = 0;
      if (__builtin_amdgcn_ballot_w64(mx * c > mref[u] + 8.f)) {
        const float mnew = fmaxf(mref[u], col_max4(mx) * c);
        const float alpha = fast_exp2(mref[u] - mnew);
        mref[u] = mnew;
        lsum[u] *= alpha;
        if (g4 == 0) sm.alpha[par][tt][col] = alpha;
        resc = 1;
      }
      if (lane == 0) sm.rescaled[par][tt] = resc;
      bf16x8 pb;
      float ps = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(fmaf(s[h][r], c, -mref[u]));
          ps += p;
          pb[4 * h + r] = (__bf16)p;
        }
      lsum[u] += ps;
      sm.pt[par][tt][lane] = pb;
    }
  };

  // O^T (this wave's dim tiles) += C^T . P^T of chunk j, every head tile, after
  // the rescale chunk j's softmax asked for.
  auto pv = [&](int j) {
    const unsigned char* sC = stage_of(j);
    const int par = j & 1;
#pragma unroll
    for (int t = 0; t < HT; ++t) {
      if (__builtin_amdgcn_readfirstlane(sm.rescaled[par][t])) {
        const float al = sm.alpha[par][t][col];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[dt][t][r] *= al;
      }
    }
    bf16x8 pbt[HT];
#pragma unroll
    for (int t = 0; t < HT; ++t) pbt[t] = sm.pt[par][t][lane];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      shortx4 half[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const unsigned char* va = sC + vofs[dt] + hf * (16 * LDC * 2);
        half[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)va);
      }
      typedef __attribute__((__vector_size__(8 * sizeof(short)))) short shortx8;
      const shortx8 a8 = {half[0][0], half[0][1], half[0][2], half[0][3],
                          half[1][0], half[1][1], half[1][2], half[1][3]};
      const bf16x8 a = __builtin_bit_cast(bf16x8, a8);
#pragma unroll
      for (int t = 0; t < HT; ++t) o[dt][t] = mfma_16x16x32(a, pbt[t], o[dt][t]);
    }
  };

  if (c0 < c1) issue(c0);
  if (c0 + 1 < c1) issue(c0 + 1);
#pragma unroll 1
  for (int j = c0; j <= c1; ++j) {
    if (j < c1) {  // chunk j landed (chunk j+1's copies may still be in flight)
      if (j + 1 < c1)
        wait_own_blocks(nmine);
      else
        wait_vmcnt<0>();
    }
    // Chunk j landed; P^T of chunk j-1 written; chunk j-2's stage and the
    // step-parity buffers of chunk j no longer read.
    __syncthreads();
    if (j + 2 < c1) issue(j + 2);
    if constexpr (NTS > 0) {
      if (j < c1) scores_softmax(j);
    }
    if constexpr (ND > 0) {
      if (j > c0) pv(j - 1);
    }
  }
  // Partials: m (log2 units) and l of each head from its score wave, o[Dc]
  // (unnormalised) from every wave's dim tiles.
#pragma unroll
  for (int u = 0; u < NTS; ++u) {
    const float l = col_sum4(lsum[u]);
    float* ph = pw + (16 * (t0 + u) + col) * LPART;
    if (g4 == 0) {
      ph[0] = mref[u];
      ph[1] = l;
    }
  }
#pragma unroll
  for (int t = 0; t < HT; ++t) {
    float* ph = pw + (16 * t + col) * LPART + 4;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) *(floatx4*)(ph + 16 * (d0 + dt) + 4 * g4) = o[dt][t];
  }
}

template <int HT>
__global__ void __launch_bounds__(64 * A2_WAVES, 1)
latent_attend2_kernel(const uint16_t* __restrict__ qa, const uint16_t* __restrict__ c_kv,
                      const uint16_t* __restrict__ k_rope, const int32_t* __restrict__ lens,
                      float* __restrict__ part, int Lmax, int window, int nsplit, float c) {
  constexpr int XP = 16 * HT;
  __shared__ __attribute__((aligned(1024))) Attend2Smem<HT> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x / nsplit, k = blockIdx.x - (blockIdx.x / nsplit) * nsplit;
  float* pw = part + ((int64_t)b * nsplit + k) * XP * LPART;

  int len = lens ? lens[b] : Lmax;
  if (len > Lmax) len = Lmax;
  const int pos = len - 1;
  const int lo = window ? max(0, pos - window + 1) : 0;
  const int nch = len >= 1 ? (pos - lo + LCK) / LCK : 0;
  const int c0 = (int)(((int64_t)k * nch) / nsplit), c1 = (int)(((int64_t)(k + 1) * nch) / nsplit);
  const char* cbase = (const char*)(c_kv + (int64_t)b * Lmax * LDC);
  const char* rbase = (const char*)(k_rope + (int64_t)b * Lmax * LDR);
  // Wave-uniform role dispatch (a2_first_dim_tile gives the dims); every path
  // runs the same barrier sequence.
#define GDA_A2_WAVE(NTS, ND) \
  attend2_wave<HT, NTS, ND>(sm, qa, cbase, rbase, pw, b, wave, lane, lo, pos, c0, c1, c)
  if constexpr (HT == A2_MAX_HT) {
    if (wave < 2)
      GDA_A2_WAVE(2, 0);
    else if (wave == 2)
      GDA_A2_WAVE(1, 2);
    else if (wave == 4 || wave == 5)
      GDA_A2_WAVE(0, 3);
    else
      GDA_A2_WAVE(0, 8);
  } else {
    if (wave < HT / 2)
      GDA_A2_WAVE(2, 0);
    else if ((HT & 1) && wave == HT / 2)
      GDA_A2_WAVE(1, 0);
    else if (wave >= 4)
      GDA_A2_WAVE(0, 8);
    else
      GDA_A2_WAVE(0, 0);
  }
#undef GDA_A2_WAVE
}

// ---- 3. merge, up-project, epilogue ------------------------------------------------
// One workgroup per (noise head j, SB = 16 / (1 + g) consecutive sequences): heads =
// noise j and its g signal heads g*j .. g*j+g-1 of each of the SB sequences, at most
// 16 (column x: sequence x / nh of the group, its head x % nh, 0 the noise head).
// Each head's o is merged over the splits (fp32, in LDS), then H = W_v[h] o on the
// matrix cores: for each KV head h the group's heads use, H^T [128 x 16] +=
// W_v[h] [128 x 512] . O [512 x 16] with O's columns of the heads on h (the others
// zero), O split into bf16 high and low parts (two products with fp32
// accumulation, so the bf16 weights meet o at about fp32 precision). Wave w owns
// W_v rows 32 w .. 32 w + 31, read straight from global memory as A operands (the
// first KV head's fragments prefetched before the merge) and used for all SB
// sequences. Then out = gate * (H_S - lambda * H_N).
__global__ void __launch_bounds__(256)
latent_merge_kernel(const float* __restrict__ part, const uint16_t* __restrict__ w_kv_b,
                    const int32_t* __restrict__ lens, const uint16_t* __restrict__ lam,
                    const uint16_t* __restrict__ gate, uint16_t* __restrict__ out, int B,
                    int Lmax, int S, int N, int Hkv, int nsplit, int XP, int flags) {
  constexpr int MAXH = 16;  // heads of a workgroup (MFMA columns)
  constexpr int KST = LDC / 32;  // k-steps of the up-projection
  __shared__ __attribute__((aligned(16))) float so[MAXH][LDC];  // merged o per column
  __shared__ float sH[MAXH][LDV];                                // up-projected outputs
  __shared__ float sml[MAXH * 64][2];  // (m, l) of each (column, split), then (weight, l)
  __shared__ float sinvl[MAXH];
  __shared__ int slen[MAXH];  // each column's sequence length (0: empty or past B)
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, g4 = lane >> 4;
  const int g = S / N;
  const int nh = 1 + g;
  const int SB = MAXH / nh;  // sequences per workgroup
  const int j = blockIdx.x % N, b0 = (blockIdx.x / N) * SB;
  const int ncol = nh * SB;
  auto kv_of = [&](int x) {
    return x == 0 ? (int)(((int64_t)j * Hkv) / N) : (int)(((int64_t)(g * j + x - 1) * Hkv) / S);
  };
  if (tid < MAXH) {
    const int bb = b0 + tid / nh;
    int len = 0;
    if (tid < ncol && bb < B) {
      len = lens ? lens[bb] : Lmax;
      len = len > Lmax ? Lmax : len;
    }
    slen[tid] = len > 0 ? len : 0;
  }
  // This wave's W_v rows of KV head h as A operands: row 32 wave + 16 mt + col,
  // latent dims 32 ks + 8 g4 .. +7.
  auto w_frag = [&](int h, int mt, int ks) {
    const int row = 32 * wave + 16 * mt + col;
    return __builtin_bit_cast(
        bf16x8, ldg16(w_kv_b + ((int64_t)h * (LDN + LDV) + LDN + row) * LDC + 32 * ks + 8 * g4));
  };
  const int h0 = kv_of(0);
  bf16x8 wpre[2][KST];  // the first KV head's fragments, in flight during the merge
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) wpre[mt][ks] = w_frag(h0, mt, ks);
  __syncthreads();  // slen
  // Merge. First every (column, split) reference and sum into LDS in one round
  // trip, then each column's split weights 2^(m_k - max m) and 1/L, then thread t
  // sums latent dims t and t+256 of every column over the splits (all loads
  // independent of each other). Columns of empty sequences get o = 0.
  auto col_part = [&](int x) {
    const int hx = x % nh, bb = b0 + x / nh;
    const int hc = hx == 0 ? S + j : g * j + (hx - 1);
    return part + ((int64_t)bb * nsplit * XP + hc) * LPART;
  };
  for (int idx = tid; idx < ncol * nsplit; idx += 256) {
    const int x = idx / nsplit, k = idx - (idx / nsplit) * nsplit;
    float m = 0.f, l = 0.f;
    if (slen[x] > 0) {
      const float* pk = col_part(x) + (int64_t)k * XP * LPART;
      m = pk[0];
      l = pk[1];
    }
    sml[idx][0] = m;
    sml[idx][1] = l;
  }
  __syncthreads();
  if (tid < ncol) {  // per column: the split weights (in place of m) and 1/L
    if (slen[tid] > 0) {
      float M = -INFINITY;
      for (int k = 0; k < nsplit; ++k) M = fmaxf(M, sml[tid * nsplit + k][0]);
      float L = 0.f;
      for (int k = 0; k < nsplit; ++k) {
        const float wk = fast_exp2(sml[tid * nsplit + k][0] - M);
        sml[tid * nsplit + k][0] = wk;
        L += wk * sml[tid * nsplit + k][1];
      }
      sinvl[tid] = 1.f / L;
    } else {
      sinvl[tid] = 0.f;
    }
  }
  __syncthreads();
  for (int x = 0; x < ncol; ++x) {
    float a0 = 0.f, a1 = 0.f;
    if (slen[x] > 0) {  // uniform
      const float* p0 = col_part(x) + 4;
#pragma unroll 4
      for (int k = 0; k < nsplit; ++k) {
        const float* pk = p0 + (int64_t)k * XP * LPART;
        const float wk = sml[x * nsplit + k][0];
        a0 = fmaf(wk, pk[tid], a0);
        a1 = fmaf(wk, pk[tid + 256], a1);
      }
    }
    so[x][tid] = a0 * sinvl[x];
    so[x][tid + 256] = a1 * sinvl[x];
  }
  __syncthreads();
  // Up-projection: column col of the B operand is column col of the group (zero
  // unless it is one of the group's heads on KV head h).
  floatx4 acc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
  for (int x = 0; x < nh; ++x) {
    const int h = kv_of(x);
    bool seen = false;  // each KV head once (wave-uniform)
    for (int y = 0; y < x; ++y) seen |= kv_of(y) == h;
    if (seen) continue;
    const bool mine = col < ncol && kv_of(col % nh) == h;
    const bool pre = h == h0;
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) {
      const floatx4 v0 = *(const floatx4*)&so[col][32 * ks + 8 * g4];
      const floatx4 v1 = *(const floatx4*)&so[col][32 * ks + 8 * g4 + 4];
      bf16x8 bh, bl;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = mine ? (i < 4 ? v0[i] : v1[i - 4]) : 0.f;
        const __bf16 hi = (__bf16)v;
        bh[i] = hi;
        bl[i] = (__bf16)(v - (float)hi);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 a = pre ? wpre[mt][ks] : w_frag(h, mt, ks);
        acc[mt] = mfma_16x16x32(a, bh, acc[mt]);
        acc[mt] = mfma_16x16x32(a, bl, acc[mt]);
      }
    }
  }
  if (col < ncol) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sH[col][32 * wave + 16 * mt + 4 * g4 + r] = acc[mt][r];
  }
  __syncthreads();
  for (int idx = tid; idx < SB * g * LDV; idx += 256) {
    const int sb = idx / (g * LDV), rem = idx - sb * (g * LDV);
    const int t = rem / LDV, e = rem - (rem / LDV) * LDV;
    const int bb = b0 + sb;
    if (bb >= B) continue;
    const int i = g * j + t;
    const int64_t o_idx = ((int64_t)bb * S + i) * LDV + e;
    if (slen[sb * nh] == 0) {  // an empty cache gives zeros
      out[o_idx] = 0;
      continue;
    }
    float lm = bf16_to_f32(lam[(int64_t)bb * S + i]);
    if (flags & kLambdaLogits) lm = sigmoid_f32(lm);
    float gv = bf16_to_f32(gate[o_idx]);
    if (flags & kGateLogits) gv = sigmoid_f32(gv);
    out[o_idx] = f32_to_bf16(gv * (sH[sb * nh + 1 + t][e] - lm * sH[sb * nh][e]));
  }
}

// Splits per sequence: enough workgroups for the CUs (the eight-wave kernel
// fills a CU with one workgroup, the other with one of up to 8 waves).
int latent_nsplit(int B, int Lmax, int window, int XP) {
  const int span = window > 0 && window < Lmax ? window : Lmax;
  const int nch = (span + LCK - 1) / LCK;
  const int target = XP / 16 <= A2_MAX_HT ? 256 : 512;
  int ns = (target + B - 1) / B;
  // Long spans keep at least four chunks per split (the pipeline's fill and the
  // partials amortise over them); short spans (a window) split down to one chunk,
  // or a W = 128 decode of 64 sequences would run on 64 workgroups.
  ns = min(ns, max(1, nch < 16 ? nch : nch / 4));
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
  const int ns = latent_nsplit(B, Lmax, window, XP);
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
  const int ns = latent_nsplit(a.B, a.Lmax, a.window, XP);
  const size_t qa_bytes = ((size_t)a.B * XP * LQW * 2 + 255) & ~(size_t)255;
  uint16_t* qa = (uint16_t*)a.workspace;
  float* part = (float*)((char*)a.workspace + qa_bytes);
  const int sb = 16 / (1 + a.S / a.N);  // sequences per merge workgroup
  const int64_t g2 = (int64_t)a.B * ns, g3 = (int64_t)((a.B + sb - 1) / sb) * a.N;
  if (g2 > 0x7fffffff || g3 > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int nkv_max = a.S / a.Hkv + (a.N + a.Hkv - 1) / a.Hkv;
  const int64_t g1b = (int64_t)a.Hkv * (((int64_t)a.B * nkv_max + AB_COLS - 1) / AB_COLS);
  if (g1b > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(latent_absorb2_kernel, dim3((unsigned)g1b), dim3(256), 0, stream,
                     (const uint16_t*)a.q_sig, (const uint16_t*)a.q_noise,
                     (const uint16_t*)a.w_kv_b, qa, a.B, a.S, a.N, a.Hkv, XP);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint16_t* ckv = (const uint16_t*)a.c_kv;
  const uint16_t* kr = (const uint16_t*)a.k_rope;
  switch (XP / 16) {
#define GDA_ATTEND2(HT)                                                                          \
  case HT:                                                                                       \
    hipLaunchKernelGGL(latent_attend2_kernel<HT>, dim3((unsigned)g2), dim3(64 * A2_WAVES), 0,    \
                       stream, (const uint16_t*)qa, ckv, kr, a.lens, part, a.Lmax, a.window, ns, \
                       a.scale_log2);                                                            \
    break;
    GDA_ATTEND2(1)
    GDA_ATTEND2(2)
    GDA_ATTEND2(3)
    GDA_ATTEND2(4)
    GDA_ATTEND2(5)
#undef GDA_ATTEND2
    default:
      hipLaunchKernelGGL(latent_attend_kernel, dim3((unsigned)g2), dim3(64 * (XP / 16)), 0,
                         stream, (const uint16_t*)qa, ckv, kr, a.lens, part, a.Lmax, a.window, ns,
                         XP, a.scale_log2);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(latent_merge_kernel, dim3((unsigned)g3), dim3(256), 0, stream,
                     (const float*)part, (const uint16_t*)a.w_kv_b, a.lens,
                     (const uint16_t*)a.lam, (const uint16_t*)a.gate, (uint16_t*)a.out, a.B,
                     a.Lmax, a.S, a.N, a.Hkv, ns, XP, a.flags);
  return hipGetLastError();
}

}  // namespace gda
