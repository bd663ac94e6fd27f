// gda_fwd_bf16.hip - bf16 prefill kernel of the GDA/GDLA attention core (gfx950).
//
// Computes, for every query t of every sequence, the output the Motif 3
// technical-report walk-through (paper.rainbus.top, step 2 "GDLA forward",
// equation D_t) defines: each signal and noise head's softmax attention over
// the KV head it shares, the noise output repeated over its g signal heads,
// D = H_S - lambda * Repeat_g(H_N), and the gate product G * D.
//
// Work decomposition (MI355X-first; the pages give no kernel design):
//  * a workgroup owns (batch row b, sub-unit v, tile of 64 queries); a sub-unit
//    is one noise head with a chunk of the signal heads it serves (on the noise
//    head's KV head and, in layouts with more KV heads than noise heads, one
//    other KV head), so the noise output never goes to HBM. Layouts whose
//    groups are too large for one workgroup split into several sub-units, each
//    recomputing the noise head (SubMap below);
//  * 8 waves: wave w owns the 16 queries of group w%4; waves 0-3 ("A") compute
//    the noise head and the first signal heads, waves 4-7 ("B") the other
//    signal heads. Each SIMD then runs one A and one B wave over the same
//    queries (2 waves per SIMD, each under 256 registers), so one wave's
//    softmax overlaps the other's MFMAs, and the noise output goes from A to B
//    through LDS once per tile of queries;
//  * K/V tiles stream HBM -> LDS with global_load_lds_dwordx4 (no VGPRs), double
//    buffered: the next tile is in flight while the current one is consumed.
//    K is stored fragment-major (each 1 KB block is exactly one MFMA A operand
//    of 16 keys x 32 dims, read back with one conflict-free ds_read_b128); V is
//    row-major with its 32-byte chunk pairs XOR-swizzled by row (pair ^= r % 8)
//    so that the 4 rows each 16-lane group of a transposed read
//    (ds_read_b64_tr_b16) touches, and the 8 rows of each half wave, fall on
//    distinct banks;
//  * scores are computed transposed, S^T = K . Q^T (16x16x32 bf16 MFMA, fp32
//    accumulation), so a lane owns one query column: the online-softmax row
//    max/sum is in-lane plus two permlane swaps, and P^T in the accumulator
//    layout is already the B operand of O^T = V^T . P^T;
//  * lambda and the gate are applied to the fp32 accumulators in registers and
//    the result is rounded to bf16 once.
#include "gda_device.hpp"
#include "gda_kernels.hpp"

namespace gda {
namespace {

constexpr float kRescaleTau = 8.f;  // lazy rescale threshold, log2 units
constexpr float kNoMax = -1e30f;    // finite "no key seen yet" reference


// ASIG signal heads + the noise head run in the A waves, BSIG signal heads in the
// B waves; with TWO_KV the B heads read a second KV head (ASIG may then be 0:
// the A waves compute only the noise head the B heads need).
//
// NQG query groups of 16 make a workgroup's query tile (BM = 16*NQG); BN keys
// make an LDS tile. (NQG, BN) = (4, 64) fills a CU with one workgroup; (2, 32)
// uses under 80 KB of LDS and 4 waves, so two workgroups share a CU and one's
// memory phases overlap the other's compute.
template <int DQK_, int DV_, int ASIG_, int BSIG_, bool TWO_KV_, int NQG_, int BN_>
struct Cfg {
  static constexpr int DQK = DQK_, DV = DV_, ASIG = ASIG_, BSIG = BSIG_;
  static constexpr bool TWO_KV = TWO_KV_;
  static constexpr int NQG = NQG_;                  // query groups of 16 per workgroup
  static constexpr int BM = 16 * NQG;               // queries per workgroup
  static constexpr int NA = ASIG + 1;              // heads of an A wave
  static constexpr int NB = BSIG;                  // heads of a B wave
  static constexpr int USIG = ASIG + BSIG;         // signal heads of a unit
  static constexpr int NW = NQG * (NB > 0 ? 2 : 1); // waves per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int BN = BN_;                    // keys per LDS tile
  static constexpr int KS = DQK / 32;               // MFMA k-steps of Q.K
  static constexpr int DB = DV / 16;                // 16-channel blocks of the output
  static constexpr int KBLK = (BN / 16) * KS;       // 1 KB fragment blocks of a K tile
  static constexpr int VBLK = (BN * DV * 2) / 1024; // 1 KB blocks of a V tile
  static constexpr int NKV = TWO_KV ? 2 : 1;
  static constexpr int TBLK = NKV * (KBLK + VBLK);  // 1 KB blocks per tile (all KV heads)
  static constexpr int K_ELEMS = BN * DQK;
  static constexpr int V_ELEMS = BN * DV;
  static constexpr int KV_ELEMS = K_ELEMS + V_ELEMS;  // one KV head's tile: K then V
  static constexpr int STAGE_ELEMS = NKV * KV_ELEMS;
  static constexpr int VCH = DV / 8;                // 16-byte chunks per V row
  static constexpr int VPAIR = VCH / 2;             // 32-byte chunk pairs per V row
  static constexpr int VRPB = 512 / DV;             // V rows per 1 KB block
  // Short workgroups (two per CU) issue their epilogue loads right after the
  // key loop and release the B waves before the A waves' stores; long ones
  // (one per CU) run their measured-faster order: A stores, then B.
  static constexpr bool kEarlyEpilogue = NQG == 2;
  // Per-tile copy bases (issue_block_fast) where a tile is one 32-key chunk (its
  // copies' scalar arithmetic is then a larger share of the tile): the short
  // one-KV-head workgroups and the 64-query two-KV-head ones. In the short
  // two-KV-head and the 64-key shapes the extra live values spill registers.
  static constexpr bool kTileBase = NQG == 2 ? !TWO_KV : (TWO_KV && BN == 32);
  static_assert(BN == 32 || BN == 64, "an LDS tile is one or two 32-key chunks");
  static_assert(TBLK % NW == 0, "every wave issues the same number of tile blocks");
  static_assert(KBLK % NW == 0 && VBLK % NW == 0, "runs of NW blocks never mix K and V");
};

// Which heads a workgroup computes. Noise head n serves signal heads
// g*n .. g*n+g-1 and reads KV head kv_noise(n) = floor(n*Hkv/N); signal head i
// reads KV head floor(i/NS) (NS = S/Hkv). Sub-unit v of a batch row (v < nsub):
//   n = v / (PK*P), r = v % (PK*P), pk = first_p + r / P, q = r % P;
//   one KV head (TWO_KV false): the A and B heads are chunk q (ASIG+BSIG heads)
//     of the g signal heads, all on kv_noise(n);
//   two KV heads: the A heads are chunk q (ASIG heads) of the signal heads on
//     kv_noise(n), the B heads chunk q (BSIG heads) of those on kv_noise(n)+pk.
// The noise head's training outputs are written by the sub-unit with r == 0 of
// the launch that owns them (own_noise), so each is written exactly once.
struct SubMap {
  int nsub;       // sub-units per batch row
  int P;          // signal-head chunks per (noise head, KV head)
  int PK;         // other KV heads per noise head in this launch (1 with one KV head)
  int first_p;    // offset of the first other KV head from kv_noise(n)
  int g;          // S / N
  int NS;         // S / Hkv
  int own_noise;  // this launch writes the noise heads' training outputs
};

struct Ctx {
  const uint16_t* kg;  // this sequence's key 0
  const uint16_t* vg;  // this sequence's value 0
  int L, Hkv, window;  // L: this sequence's keys
  int kvA, kvB;
  // Query positions in key coordinates (a sequence's Lq queries are its last Lq
  // key positions: local query t sits at position L - Lq + t).
  int q_lo, q_hi;  // the workgroup's queries
  int w_lo, w_hi;  // this wave's queries (empty when w_lo > w_hi)
  int t;           // this lane's query (past the last for padding lanes)
  int lane, col, g4, wave;
  float c;  // log2(e)/sqrt(dqk)
};

// Issue one 1 KB direct-to-LDS block of a tile (keys k0 .. k0+BN-1) into the
// ring stage at LDS byte address stage_lds. Rows past the sequence's last key
// read that key (finite data; those keys are masked).
template <class C>
__device__ __forceinline__ void issue_block(const Ctx& x, int blk, int k0, uint32_t stage_lds) {
  constexpr int per = C::KBLK + C::VBLK;
  const int kvi = (C::TWO_KV && blk >= per) ? 1 : 0;
  const int bi = blk - kvi * per;
  const int kvh = kvi ? x.kvB : x.kvA;
  const uint32_t kv_lds = stage_lds + 2u * (uint32_t)(kvi * C::KV_ELEMS);
  // The per-lane part of every address is a 32-bit byte offset from a
  // wave-uniform base row (clamped so the base never passes row L-1).
  if (bi < C::KBLK) {
    const int kb = bi / C::KS, ks = bi - (bi / C::KS) * C::KS;
    const uint32_t stride = (uint32_t)x.Hkv * C::DQK * 2;
    const int row0 = min(k0 + 16 * kb, x.L - 1);
    const int rel = min(x.lane & 15, x.L - 1 - row0);
    const char* base = (const char*)x.kg +
                       (((int64_t)row0 * x.Hkv + kvh) * C::DQK + 32 * ks) * 2;
    dma16_lds(base, (uint32_t)rel * stride + 16u * (uint32_t)(x.lane >> 4), kv_lds + 1024u * bi);
  } else {
    const int vi = bi - C::KBLK;
    const int lr = x.lane / C::VCH;            // row within the block
    const int r = C::VRPB * vi + lr;           // row within the tile
    const int cch = (x.lane % C::VCH) ^ ((r % C::VPAIR) << 1);
    const uint32_t stride = (uint32_t)x.Hkv * C::DV * 2;
    const int row0 = min(k0 + C::VRPB * vi, x.L - 1);
    const int rel = min(lr, x.L - 1 - row0);
    const char* base = (const char*)x.vg + ((int64_t)row0 * x.Hkv + kvh) * C::DV * 2;
    dma16_lds(base, (uint32_t)rel * stride + 16u * (uint32_t)cch,
              kv_lds + 2u * C::K_ELEMS + 1024u * vi);
  }
}

// Every wave issues its share of the tile's 1 KB blocks into ring stage DST.
template <class C>
__device__ __forceinline__ void issue_tile(const Ctx& x, int k0, uint32_t ring_lds, int dst) {
  const uint32_t stage_lds = ring_lds + 2u * (uint32_t)(dst * C::STAGE_ELEMS);
#pragma unroll
  for (int i = 0; i < C::TBLK / C::NW; ++i) issue_block<C>(x, x.wave + i * C::NW, k0, stage_lds);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}

// Block i of this wave's share of a tile (key k0, ending inside the sequence)
// into ring stage DST. Blocks are dealt round-robin (block wave + i*NW); with
// the tile sizes used here every multiple of NW starts a run of blocks of one
// kind (K or V of one KV head), so the kind is known at compile time and only
// the index within the kind depends on the wave.
template <class C, int DST>
__device__ __forceinline__ void issue_block_fast(const Ctx& x, uint32_t ring_lds, int k0, int i) {
  constexpr int per = C::KBLK + C::VBLK;
  const int first = i * C::NW;  // compile-time after unrolling
  const int kvi = (C::TWO_KV && first >= per) ? 1 : 0;
  const int fb = first - kvi * per;
  const int kvh = kvi ? x.kvB : x.kvA;
  const uint32_t st_off = 2u * (uint32_t)((DST * C::NKV + kvi) * C::KV_ELEMS);
  // With kTileBase: one 64-bit base per tile and kind (the tile's first key row,
  // shared by every block of that kind, so it is computed once per tile), plus the
  // block's offset from it, which depends only on the wave and the block (the same
  // on every tile) and joins the lane's 32-bit offset; full 64-bit address
  // arithmetic per block costs about 13 scalar instructions per copy.
  if (fb < C::KBLK) {
    const int bi = fb + x.wave;
    const int kb = bi / C::KS, ks = bi - (bi / C::KS) * C::KS;
    const uint32_t lane_off =
        (uint32_t)(x.lane & 15) * (uint32_t)(x.Hkv * C::DQK * 2) + 16u * (uint32_t)(x.lane >> 4);
    if constexpr (C::kTileBase) {
      const char* g = (const char*)x.kg + (int64_t)k0 * (x.Hkv * C::DQK * 2);
      const uint32_t boff = (uint32_t)(((16 * kb) * x.Hkv + kvh) * C::DQK + 32 * ks) * 2u;
      dma16_lds(g, boff + lane_off, ring_lds + st_off + 1024u * (uint32_t)bi);
    } else {
      const char* g = (const char*)x.kg +
                      (((int64_t)(k0 + 16 * kb) * x.Hkv + kvh) * C::DQK + 32 * ks) * 2;
      dma16_lds(g, lane_off, ring_lds + st_off + 1024u * (uint32_t)bi);
    }
  } else {
    const int vi = fb - C::KBLK + x.wave;
    const int lr = x.lane / C::VCH;
    const int r = C::VRPB * vi + lr;
    const int cch = (x.lane % C::VCH) ^ ((r % C::VPAIR) << 1);
    const uint32_t lane_off = (uint32_t)lr * (uint32_t)(x.Hkv * C::DV * 2) + 16u * (uint32_t)cch;
    if constexpr (C::kTileBase) {
      const char* g = (const char*)x.vg + (int64_t)k0 * (x.Hkv * C::DV * 2);
      const uint32_t boff = (uint32_t)((C::VRPB * vi) * x.Hkv + kvh) * (uint32_t)(C::DV * 2);
      dma16_lds(g, boff + lane_off, ring_lds + st_off + 2u * C::K_ELEMS + 1024u * (uint32_t)vi);
    } else {
      const char* g =
          (const char*)x.vg + ((int64_t)(k0 + C::VRPB * vi) * x.Hkv + kvh) * C::DV * 2;
      dma16_lds(g, lane_off, ring_lds + st_off + 2u * C::K_ELEMS + 1024u * (uint32_t)vi);
    }
  }
}

template <class C, int DST>
__device__ __forceinline__ void issue_tile_fast(const Ctx& x, uint32_t ring_lds, int k0, int i0,
                                                int i1) {
#pragma unroll
  for (int i = 0; i < C::TBLK / C::NW; ++i)
    if (i >= i0 && i < i1) issue_block_fast<C, DST>(x, ring_lds, k0, i);
}

__device__ __forceinline__ void wait_loads_and_sync() {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's direct-to-LDS loads have landed
  __syncthreads();                // ... and every other wave's
}

// Per-wave online-softmax state for NH heads.
template <class C, int NH>
struct State {
  bf16x8 q[NH][C::KS];
  floatx4 o[NH][C::DB];
  float mref[NH];  // per column reference max (log2 units)
  float lsum[NH];  // per lane partial softmax denominator
};

// Is any key of chunk c0 .. c0+31 visible to a query of this wave? (wave-uniform)
__device__ __forceinline__ bool chunk_live(const Ctx& x, int c0) {
  const int W = x.window;
  const int wk_lo = W ? max(0, x.w_lo - W + 1) : 0;
  return x.w_lo <= x.w_hi && c0 <= x.w_hi && c0 + 31 >= wk_lo;
}

// S^T = K . Q^T for chunk cc of the LDS tile (keys 32 cc .. +31), first NACT heads.
template <class C, int NH, int NACT>
__device__ __forceinline__ void chunk_qk(const Ctx& x, const State<C, NH>& st, const uint16_t* sK,
                                         int cc, floatx4 (&s)[NH][2]) {
#pragma unroll
  for (int h = 0; h < NACT; ++h) {
    s[h][0] = floatx4{0.f, 0.f, 0.f, 0.f};
    s[h][1] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 a =
          *(const bf16x8*)(sK + (((2 * cc + kb) * C::KS + ks) << 9) + 8 * x.lane);
#pragma unroll
      for (int h = 0; h < NACT; ++h) s[h][kb] = mfma_16x16x32(a, st.q[h][ks], s[h][kb]);
    }
  }
  // Schedule: the first AH K fragment reads, then each fragment's MFMAs followed
  // by the read of the fragment AH steps ahead, so LDS latency hides behind MFMAs
  // instead of stalling them. AH = 2 for a three-head wave (more do not fit in
  // its registers), 4 for a wave of two heads or fewer.
  constexpr int AH = NACT <= 2 ? 4 : 2;
  __builtin_amdgcn_sched_group_barrier(0x100, AH, 0);
#pragma unroll
  for (int i = 0; i < 2 * C::KS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, NACT, 0);
    if (i + AH < 2 * C::KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// Mask chunk c0 .. c0+31, update the lazy online-softmax state and return
// P = 2^(S c - mref) as bf16 (first NACT heads).
template <class C, int NH, int NACT>
__device__ __forceinline__ void chunk_softmax(const Ctx& x, State<C, NH>& st, floatx4 (&s)[NH][2],
                                              int c0, bf16x8 (&pb)[NH]) {
  const int W = x.window;
  const bool need_mask = (c0 + 31 > x.w_lo) || (W && c0 < x.w_hi - W + 1);
  if (need_mask) {
    // Selects, not branches: a per-element branch here compiles to a divergent
    // exec-mask sequence per score, on every chunk that crosses the diagonal or
    // the window edge (two of the five chunks of a W = 128 window).
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = c0 + 16 * kb + 4 * x.g4 + r;
        const bool vis = key <= x.t && (!W || x.t - key < W);
#pragma unroll
        for (int h = 0; h < NACT; ++h) s[h][kb][r] = vis ? s[h][kb][r] : -INFINITY;
      }
  }
#pragma unroll
  for (int h = 0; h < NACT; ++h) {
    const float mx =
        fmaxf(fmaxf(fmaxf(s[h][0][0], s[h][0][1]), fmaxf(s[h][0][2], s[h][0][3])),
              fmaxf(fmaxf(s[h][1][0], s[h][1][1]), fmaxf(s[h][1][2], s[h][1][3])));
    if (__builtin_amdgcn_ballot_w64(mx * x.c > st.mref[h] + kRescaleTau)) {
      const float mnew = fmaxf(st.mref[h], col_max4(mx) * x.c);
      const float alpha = fast_exp2(st.mref[h] - mnew);
      st.mref[h] = mnew;
      st.lsum[h] *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) st.o[h][db][r] *= alpha;
    }
    const float nm = -st.mref[h];
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(fmaf(s[h][kb][r], x.c, nm));
        ps += p;
        pb[h][4 * kb + r] = (__bf16)p;
      }
    st.lsum[h] += ps;
  }
}

// O^T += V^T . P^T over chunk cc of the LDS tile; V^T from transposed LDS reads.
template <class C, int NH, int NACT>
__device__ __forceinline__ void chunk_pv(const Ctx& x, State<C, NH>& st, const uint16_t* sV,
                                         int cc, const bf16x8 (&pb)[NH]) {
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    shortx4 half[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int r = 32 * cc + 16 * hf + 4 * x.g4 + (x.col >> 2);
      const int chunk = 2 * db + ((x.col & 3) >> 1);
      const uint16_t* va =
          sV + r * C::DV + ((chunk ^ ((r % C::VPAIR) << 1)) << 3) + 4 * (x.col & 1);
      half[hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)va);
    }
    typedef __attribute__((__vector_size__(8 * sizeof(short)))) short shortx8;
    const shortx8 a8 = {half[0][0], half[0][1], half[0][2], half[0][3],
                        half[1][0], half[1][1], half[1][2], half[1][3]};
    const bf16x8 a = __builtin_bit_cast(bf16x8, a8);
#pragma unroll
    for (int h = 0; h < NACT; ++h) st.o[h][db] = mfma_16x16x32(a, pb[h], st.o[h][db]);
  }
  // Schedule: V^T pairs for two channel blocks ahead of the MFMAs that use them.
  constexpr int AV = NACT <= 2 ? 3 : 2;  // V^T channel blocks in flight
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * AV, 1);
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    __builtin_amdgcn_sched_group_barrier(0x008, NACT, 1);
    if (db + AV < C::DB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
  }
}

// One 32-key chunk (keys c0 .. c0+31, chunk cc of the LDS tile), first NACT heads.
template <class C, int NH, int NACT>
__device__ __forceinline__ void consume_chunk(const Ctx& x, State<C, NH>& st, const uint16_t* sK,
                                              const uint16_t* sV, int c0, int cc) {
  if (!chunk_live(x, c0)) return;
  floatx4 s[NH][2];
  bf16x8 pb[NH];
  // The score products run at raised wave priority: of the two waves sharing a
  // SIMD, the one that reaches its matrix phase first keeps the matrix core while
  // the other is in its softmax, which moves the two out of phase.
  __builtin_amdgcn_s_setprio(1);
  chunk_qk<C, NH, NACT>(x, st, sK, cc, s);
  __builtin_amdgcn_s_setprio(0);
  chunk_softmax<C, NH, NACT>(x, st, s, c0, pb);
  chunk_pv<C, NH, NACT>(x, st, sV, cc, pb);
}

// Consume the tile (keys k0 .. k0+BN-1) held in LDS stage STAGE. The wave's
// copies of the next tile (key dma_k0 >= 0, into the other stage) go out between
// a 64-key tile's two chunks: right after the barrier every wave starts its score
// products at once, and the copies' address arithmetic then delays them
// (issued before the first chunk: 1.6% slower; half before, half between: 2.4%).
// A one-chunk tile issues them before its chunk, to give them the whole chunk.
template <class C, int NH, int STAGE>
__device__ __forceinline__ void consume_tile(const Ctx& x, State<C, NH>& st, const uint16_t* sK,
                                             const uint16_t* sV, int k0, uint32_t ring_lds,
                                             int dma_k0) {
  constexpr int DST = 1 - STAGE;
  constexpr int NI = C::TBLK / C::NW;
  constexpr int H1 = C::BN == 64 ? 0 : NI;
  if (dma_k0 >= 0) issue_tile_fast<C, DST>(x, ring_lds, dma_k0, 0, H1);
  consume_chunk<C, NH, NH>(x, st, sK, sV, k0, 0);
  if constexpr (C::BN == 64) {
    if (dma_k0 >= 0) issue_tile_fast<C, DST>(x, ring_lds, dma_k0, H1, NI);
    consume_chunk<C, NH, NH>(x, st, sK, sV, k0 + 32, 1);
  }
}

// The epilogue of one signal head: out[t, i, :] = gate * (hs/l_s - lam * hn).
// In the accumulator layout a lane holds 4 channels of each 16-channel block, so
// a store would move 8 bytes per lane and 32 contiguous bytes per query row.
// Block pairs (2p, 2p+1) are first regrouped across lanes l and l^16 (one
// permlane16 swap per value; both lanes hold the same query): lane group g
// then holds the 8 consecutive channels 32p + 16(g&1) + 8(g>>1) .. +7, so each
// gate load and output store moves 16 bytes per lane and 64 contiguous bytes
// per query row.
template <int DV>
struct HeadIn {
  u32x4 gate[DV / 32];  // this lane's 8-channel gate pieces
  // lambda's bf16 bits: widened where it is used, so that the load's wait sits there
  // and not right after the load is issued.
  uint32_t lam_bits;
};

__device__ __forceinline__ int64_t head_base(int64_t row, int S, int i, int g4, int DV) {
  return (row * S + i) * DV + 16 * (g4 & 1) + 8 * (g4 >> 1);
}

// Issue the gate and lambda loads of one head (row is always a valid row).
template <int DV>
__device__ __forceinline__ void load_head_in(const uint16_t* lam, const uint16_t* gate,
                                             int64_t row, int S, int i, int g4, HeadIn<DV>& in) {
  const int64_t base = head_base(row, S, i, g4, DV);
#pragma unroll
  for (int p = 0; p < DV / 32; ++p) in.gate[p] = ldg16(gate + base + 32 * p);
  in.lam_bits = lam[row * S + i];
}

// The output values of one signal head, rounded to bf16 and regrouped for 16-byte
// stores (pair p goes to out + head_base + 32 p).
template <int DV>
__device__ __forceinline__ void pack_head(const floatx4 (&hs)[DV / 16], float inv_s,
                                          const floatx4 (&hn)[DV / 16], const HeadIn<DV>& in,
                                          int flags, u32x4 (&ow)[DV / 32]) {
  constexpr int NP = DV / 32;
  static_assert(DV % 32 == 0, "channel blocks come in pairs");
  const float lraw = __uint_as_float(in.lam_bits << 16);
  const float lm = (flags & kLambdaLogits) ? sigmoid_f32(lraw) : lraw;
  float e[NP][8];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float a = hs[2 * p][r] * inv_s - lm * hn[2 * p][r];
      const float b = hs[2 * p + 1][r] * inv_s - lm * hn[2 * p + 1][r];
      // vdst's odd rows trade places with vsrc's even rows.
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b),
                                                       false, false);
      e[p][r] = __uint_as_float(sw[0]);
      e[p][4 + r] = __uint_as_float(sw[1]);
    }
  const bool logits = (flags & kGateLogits) != 0;
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float glo = bf16_lo(in.gate[p][w]), ghi = bf16_hi(in.gate[p][w]);
      if (logits) {
        glo = sigmoid_f32(glo);
        ghi = sigmoid_f32(ghi);
      }
      ow[p][w] = pack_bf16x2(glo * e[p][2 * w], ghi * e[p][2 * w + 1]);
    }
}

template <int DV>
__device__ __forceinline__ void store_head(uint16_t* out, int64_t row, int S, int i, int g4,
                                           const floatx4 (&hs)[DV / 16], float inv_s,
                                           const floatx4 (&hn)[DV / 16], const HeadIn<DV>& in,
                                           int flags) {
  u32x4 ow[DV / 32];
  pack_head<DV>(hs, inv_s, hn, in, flags, ow);
  const int64_t base = head_base(row, S, i, g4, DV);
#pragma unroll
  for (int p = 0; p < DV / 32; ++p) *(u32x4*)(out + base + 32 * p) = ow[p];
}

// Training form: one path's normalised output h * inv (bf16, regrouped like
// store_head) and its row's log-sum-exp in natural-log units (-inf for a row
// with no visible key). The four lane groups of a query column hold the same
// value and all store it.
template <int DV>
__device__ __forceinline__ void store_train_head(uint16_t* h_out, float* lse_out, int g4,
                                                 const floatx4 (&h)[DV / 16], float inv,
                                                 float mref, float lsum) {
  constexpr int NP = DV / 32;
  uint16_t* dst = h_out + 16 * (g4 & 1) + 8 * (g4 >> 1);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    float e[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(h[2 * p][r] * inv),
                                                       __float_as_uint(h[2 * p + 1][r] * inv),
                                                       false, false);
      e[r] = __uint_as_float(sw[0]);
      e[4 + r] = __uint_as_float(sw[1]);
    }
    u32x4 ow;
#pragma unroll
    for (int w = 0; w < 4; ++w) ow[w] = pack_bf16x2(e[2 * w], e[2 * w + 1]);
    *(u32x4*)(dst + 32 * p) = ow;
  }
  *lse_out = lsum > 0.f ? (mref + log2f(lsum)) * kLn2 : -INFINITY;
}

// The main loop of one wave group. Both groups run the same barrier sequence.
template <class C, int NH, int PARITY>
__device__ __forceinline__ void run_tiles(const Ctx& x, State<C, NH>& st,
                                          const uint16_t* const (&qrow)[NH], uint32_t ring_lds,
                                          uint16_t* (&sk)[2][2], uint16_t* (&sv)[2][2]) {
#pragma unroll
  for (int h = 0; h < NH; ++h) {
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      st.q[h][ks] = __builtin_bit_cast(bf16x8, ldg16(qrow[h] + ks * 32 + 8 * x.g4));
    st.mref[h] = kNoMax;
    st.lsum[h] = 0.f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) st.o[h][db] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const int W = x.window;
  const int k_lo = W ? max(0, x.q_lo - W + 1) : 0;
  const int kt0 = k_lo / C::BN, kt1 = x.q_hi / C::BN;
  constexpr int kv = (C::TWO_KV && PARITY == 1) ? 1 : 0;  // the B waves (PARITY 1) read the second KV head
  // The next tile's copies: spread over this tile when it ends inside the
  // sequence, else issued at once with row clamping.
  auto next_job = [&](int knext, int dst) -> int {
    if (knext > kt1 * C::BN) return -1;
    if (knext + C::BN <= x.L) return knext;
    issue_tile<C>(x, knext, ring_lds, dst);
    return -1;
  };
  for (int kt = kt0; kt <= kt1; kt += 2) {
    wait_loads_and_sync();
    consume_tile<C, NH, 0>(x, st, sk[0][kv], sv[0][kv], kt * C::BN, ring_lds,
                                   next_job((kt + 1) * C::BN, 1));
    if (kt + 1 > kt1) break;
    wait_loads_and_sync();
    consume_tile<C, NH, 1>(x, st, sk[1][kv], sv[1][kv], (kt + 1) * C::BN, ring_lds,
                                   next_job((kt + 2) * C::BN, 0));
  }
#pragma unroll
  for (int h = 0; h < NH; ++h) st.lsum[h] = col_sum4(st.lsum[h]);
}

// A 4-wave workgroup is meant to share its CU with a second one (2 waves per
// SIMD, so at most 256 registers per wave).
// With TRAIN the kernel also writes what the backward takes from the forward:
// each path's normalised output h_sig [rows,S,dv] and h_noise [rows,N,dv], and
// each attention row's log-sum-exp at lse[lse_b * b + lse_q * qbase + hd * lse_h + t]
// for head hd and local query t: [B,S+N,L] for a batch (lse_b = (S+N) L, lse_q = 0,
// lse_h = L), [S+N,Tq] for packed sequences (lse_b = 0, lse_q = 1, lse_h = Tq).

template <class C, bool TRAIN>
__global__ void __launch_bounds__(C::NT, C::NW == 4 ? 2 : 1)
fwd_bf16_kernel(const uint16_t* __restrict__ q_sig, const uint16_t* __restrict__ q_noise,
                const uint16_t* __restrict__ kg, const uint16_t* __restrict__ vg,
                const uint16_t* __restrict__ lam, const uint16_t* __restrict__ gate,
                uint16_t* __restrict__ out, const int32_t* __restrict__ cu_q,
                const int32_t* __restrict__ cu_k, int B, int L, int S, int N, int Hkv,
                int window, SubMap sm, int nqt, int heavy_first, float c, int flags,
                uint16_t* __restrict__ h_sig, uint16_t* __restrict__ h_noise,
                float* __restrict__ lse, int64_t lse_b, int lse_q, int64_t lse_h) {
  // K/V ring: two stages, each the tiles of the sub-unit's KV heads.
  __shared__ __attribute__((aligned(16))) uint16_t ring[2 * C::STAGE_ELEMS];
  // Normalised noise output handed from the A waves to the B waves.
  __shared__ __attribute__((aligned(16))) float sHN[C::NB > 0 ? C::NQG * C::DB * 4 * 64 : 4];

  Ctx x;
  x.Hkv = Hkv;
  x.window = window;
  const int tid = threadIdx.x;
  x.wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  x.lane = tid & 63;
  x.col = x.lane & 15;
  x.g4 = x.lane >> 4;
  x.c = c;
  const bool group_b = x.wave >= C::NQG;
  const int qg = x.wave % C::NQG;
  const int per = B * sm.nsub;
  const int slot = blockIdx.x / per;
  const int qt = heavy_first ? nqt - 1 - slot : slot;
  const int bu = blockIdx.x - slot * per;
  const int b = bu / sm.nsub, v = bu - (bu / sm.nsub) * sm.nsub;
  // This sub-unit's heads (SubMap): noise head n, the A signal heads from sigA,
  // the B signal heads from sigB.
  const int pp = sm.PK * sm.P;
  const int n = v / pp, r_ = v - (v / pp) * pp;
  const int pk = sm.first_p + r_ / sm.P, q_ = r_ - (r_ / sm.P) * sm.P;
  const int kv_n = (int)(((int64_t)n * Hkv) / N);
  const int sigA = C::TWO_KV ? n * sm.g + q_ * C::ASIG : n * sm.g + q_ * C::USIG;
  const int sigB = C::TWO_KV ? n * sm.g + pk * sm.NS + q_ * C::BSIG : sigA + C::ASIG;
  const bool noise_owner = sm.own_noise && r_ == 0;
  // Sequence b: Lq queries from packed row qbase, Lk keys from packed row kbase
  // (packed sequences), or rows b*L .. b*L+L-1 of both (a batch).
  int64_t qbase, kbase;
  int Lq, Lk;
  if (cu_q) {
    qbase = cu_q[b];
    Lq = cu_q[b + 1] - cu_q[b];
    kbase = cu_k[b];
    Lk = cu_k[b + 1] - cu_k[b];
  } else {
    qbase = kbase = (int64_t)b * L;
    Lq = Lk = L;
  }
  const int ql = qt * C::BM;  // this tile's first query of the sequence
  if (ql >= Lq) return;        // past the sequence (the whole workgroup)
  const int qoff = Lk - Lq;
  x.L = Lk;
  x.kg = kg + kbase * Hkv * C::DQK;
  x.vg = vg + kbase * Hkv * C::DV;
  x.kvA = kv_n;
  x.kvB = C::TWO_KV ? kv_n + pk : kv_n;
  x.q_lo = qoff + ql;
  x.q_hi = qoff + min(ql + C::BM, Lq) - 1;
  const int64_t lbase = lse_b * b + lse_q * qbase;  // this sequence's lse origin
  const int64_t lstride = lse_h;
  if (x.q_hi < 0) {  // every query before the first key (or no key): zeros
    const int nq = min(ql + C::BM, Lq) - ql;
    for (int idx = threadIdx.x; idx < nq * C::USIG * C::DV; idx += C::NT) {
      const int r = idx / (C::USIG * C::DV), rem = idx - r * (C::USIG * C::DV);
      const int hh = rem / C::DV, e = rem - hh * C::DV;
      const int hd = hh < C::ASIG ? sigA + hh : sigB + (hh - C::ASIG);
      out[((qbase + ql + r) * S + hd) * C::DV + e] = 0;
      if constexpr (TRAIN) h_sig[((qbase + ql + r) * S + hd) * C::DV + e] = 0;
    }
    if constexpr (TRAIN) {
      if (noise_owner)
        for (int idx = threadIdx.x; idx < nq * C::DV; idx += C::NT) {
          const int r = idx / C::DV, e = idx - r * C::DV;
          h_noise[((qbase + ql + r) * N + n) * C::DV + e] = 0;
        }
      for (int idx = threadIdx.x; idx < nq * (C::USIG + 1); idx += C::NT) {
        const int r = idx / (C::USIG + 1), hh = idx - r * (C::USIG + 1);
        if (hh == C::USIG && !noise_owner) continue;
        const int hd = hh < C::ASIG ? sigA + hh : hh < C::USIG ? sigB + (hh - C::ASIG) : S + n;
        lse[lbase + hd * lstride + ql + r] = -INFINITY;
      }
    }
    return;
  }
  x.w_lo = x.q_lo + qg * 16;
  x.w_hi = min(x.w_lo + 15, x.q_hi);
  x.t = x.w_lo + x.col;
  const int tl = x.t - qoff;  // the lane's query, local to the sequence
  const bool t_ok = tl < Lq;
  const int64_t row = qbase + min(tl, Lq - 1);

  uint16_t* sk[2][2];
  uint16_t* sv[2][2];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      sk[st][kv] = ring + (st * C::NKV + (C::TWO_KV ? kv : 0)) * C::KV_ELEMS;
      sv[st][kv] = sk[st][kv] + C::K_ELEMS;
    }
  const uint32_t ring_lds = lds_addr(ring);
  // The first tile is in flight before the Q loads.
  {
    const int k_lo = window ? max(0, x.q_lo - window + 1) : 0;
    const int kf = (k_lo / C::BN) * C::BN;
    if (kf + C::BN <= Lk)
      issue_tile_fast<C, 0>(x, ring_lds, kf, 0, C::TBLK / C::NW);
    else
      issue_tile<C>(x, kf, ring_lds, 0);
  }

  if (!group_b) {
    constexpr int NH = C::NA;  // [A signal heads][noise]
    constexpr int NZ = C::ASIG;  // index of the noise head in the state
    State<C, NH> st;
    const uint16_t* qrow[NH];
#pragma unroll
    for (int s = 0; s < C::ASIG; ++s) qrow[s] = q_sig + (row * S + sigA + s) * C::DQK;
    qrow[NZ] = q_noise + (row * N + n) * C::DQK;
    run_tiles<C, NH, 0>(x, st, qrow, ring_lds, sk, sv);
    HeadIn<C::DV> in[C::ASIG > 0 ? C::ASIG : 1];
    if constexpr (C::kEarlyEpilogue) {
#pragma unroll
      for (int s = 0; s < C::ASIG; ++s)
        load_head_in<C::DV>(lam, gate, row, S, sigA + s, x.g4, in[s]);
    }
    // A query at a negative position has no visible key: its sums stay 0 and it
    // gives zeros.
    const float inv_n = st.lsum[NZ] > 0.f ? 1.f / st.lsum[NZ] : 0.f;
    floatx4 hn[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) hn[db][r] = st.o[NZ][db][r] * inv_n;
    if (C::NB > 0) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        *(floatx4*)(sHN + ((qg * C::DB + db) * 64 + x.lane) * 4) = hn[db];
      if constexpr (C::kEarlyEpilogue) __syncthreads();  // release the B waves first
    }
    if constexpr (!C::kEarlyEpilogue) {
#pragma unroll
      for (int s = 0; s < C::ASIG; ++s)
        load_head_in<C::DV>(lam, gate, row, S, sigA + s, x.g4, in[s]);
    }
    if (t_ok) {
#pragma unroll
      for (int s = 0; s < C::ASIG; ++s)
        store_head<C::DV>(out, row, S, sigA + s, x.g4, st.o[s],
                          st.lsum[s] > 0.f ? 1.f / st.lsum[s] : 0.f, hn, in[s], flags);
      if constexpr (TRAIN) {
        if (noise_owner)
          store_train_head<C::DV>(h_noise + (row * N + n) * C::DV,
                                  lse + lbase + (int64_t)(S + n) * lstride + tl, x.g4,
                                  st.o[NZ], inv_n, st.mref[NZ], st.lsum[NZ]);
#pragma unroll
        for (int s = 0; s < C::ASIG; ++s)
          store_train_head<C::DV>(h_sig + (row * S + sigA + s) * C::DV,
                                  lse + lbase + (int64_t)(sigA + s) * lstride + tl, x.g4, st.o[s],
                                  st.lsum[s] > 0.f ? 1.f / st.lsum[s] : 0.f, st.mref[s],
                                  st.lsum[s]);
      }
    }
    if constexpr (!C::kEarlyEpilogue) {
      if (C::NB > 0) __syncthreads();
    }
  } else if (C::NB > 0) {
    constexpr int NH = C::NB > 0 ? C::NB : 1;  // [B signal heads]
    State<C, NH> st;
    const uint16_t* qrow[NH];
#pragma unroll
    for (int s = 0; s < C::BSIG; ++s) qrow[s] = q_sig + (row * S + sigB + s) * C::DQK;
    run_tiles<C, NH, 1>(x, st, qrow, ring_lds, sk, sv);
    HeadIn<C::DV> in[NH];
    if constexpr (C::kEarlyEpilogue) {  // in flight while waiting for the A waves
#pragma unroll
      for (int s = 0; s < C::BSIG; ++s)
        load_head_in<C::DV>(lam, gate, row, S, sigB + s, x.g4, in[s]);
    }
    __syncthreads();  // the A waves' noise output is in LDS
    floatx4 hn[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
      hn[db] = *(const floatx4*)(sHN + ((qg * C::DB + db) * 64 + x.lane) * 4);
    if constexpr (!C::kEarlyEpilogue) {
#pragma unroll
      for (int s = 0; s < C::BSIG; ++s)
        load_head_in<C::DV>(lam, gate, row, S, sigB + s, x.g4, in[s]);
    }
    if (t_ok) {
#pragma unroll
      for (int s = 0; s < C::BSIG; ++s)
        store_head<C::DV>(out, row, S, sigB + s, x.g4, st.o[s],
                          st.lsum[s] > 0.f ? 1.f / st.lsum[s] : 0.f, hn, in[s], flags);
      if constexpr (TRAIN) {
#pragma unroll
        for (int s = 0; s < C::BSIG; ++s)
          store_train_head<C::DV>(h_sig + (row * S + sigB + s) * C::DV,
                                  lse + lbase + (int64_t)(sigB + s) * lstride + tl,
                                  x.g4, st.o[s],
                                  st.lsum[s] > 0.f ? 1.f / st.lsum[s] : 0.f, st.mref[s],
                                  st.lsum[s]);
      }
    }
  }
}

// Largest chunk of signal heads (at most MAXC) that divides n.
inline int chunk_of(int n, int maxc) {
  for (int c = maxc; c > 1; --c)
    if (n % c == 0) return c;
  return 1;
}

template <class C>
hipError_t launch_inst(const FwdArgs& a, const SubMap& sm, hipStream_t stream) {
  // Packed sequences: B sequences of at most L queries each.
  const int nqt = (a.L + C::BM - 1) / C::BM;
  const int64_t grid = (int64_t)nqt * a.B * sm.nsub;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int heavy_first = a.window == 0 ? 1 : 0;
  if (a.h_sig)
    hipLaunchKernelGGL((fwd_bf16_kernel<C, true>), dim3((unsigned)grid), dim3(C::NT), 0, stream,
                       (const uint16_t*)a.q_sig, (const uint16_t*)a.q_noise,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.lam,
                       (const uint16_t*)a.gate, (uint16_t*)a.out, a.cu_q, a.cu_k, a.B, a.L,
                       a.S, a.N, a.Hkv, a.window, sm, nqt, heavy_first,
                       a.scale_log2, a.flags, (uint16_t*)a.h_sig, (uint16_t*)a.h_noise,
                       a.lse, a.lse_b, a.lse_q, a.lse_h);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<C, false>), dim3((unsigned)grid), dim3(C::NT), 0,
                       stream, (const uint16_t*)a.q_sig, (const uint16_t*)a.q_noise,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.lam,
                       (const uint16_t*)a.gate, (uint16_t*)a.out, a.cu_q, a.cu_k, a.B, a.L,
                       a.S, a.N, a.Hkv, a.window, sm, nqt, heavy_first,
                       a.scale_log2, a.flags, (uint16_t*)a.h_sig, (uint16_t*)a.h_noise,
                       a.lse, a.lse_b, a.lse_q, a.lse_h);
  return hipGetLastError();
}

// Sub-unit launches of a head layout (g = S/N, NS = S/Hkv), for a (query
// groups, key tile) shape:
//  * N >= Hkv: every signal head of noise head n reads kv_noise(n); one launch,
//    each sub-unit the noise head and a chunk of c <= 4 of its g signal heads
//    (c = g, one sub-unit per noise head, in the workloads' layouts);
//  * N < Hkv (R = Hkv/N KV heads per noise head, NS signal heads on each): a
//    launch of sub-units pairing a chunk of the signal heads on kv_noise(n)
//    (with the noise head, A waves) with the same chunk of those on the next
//    KV head (B waves); for R > 2 a second launch whose A waves compute only the
//    noise head, the B waves a chunk of the signal heads on each further KV head.
template <int DQK, int DV, int NQG, int BN>
hipError_t dispatch_layout(const FwdArgs& a, hipStream_t stream) {
  const int g = a.S / a.N, NS = a.S / a.Hkv;
  if (a.N >= a.Hkv) {
    const int c = chunk_of(g, 4);
    const SubMap sm{a.N * (g / c), g / c, 1, 0, g, NS, 1};
    switch (c) {
      case 1: return launch_inst<Cfg<DQK, DV, 1, 0, false, NQG, BN>>(a, sm, stream);
      case 2: return launch_inst<Cfg<DQK, DV, 1, 1, false, NQG, BN>>(a, sm, stream);
      case 3: return launch_inst<Cfg<DQK, DV, 1, 2, false, NQG, BN>>(a, sm, stream);
      default: return launch_inst<Cfg<DQK, DV, 2, 2, false, NQG, BN>>(a, sm, stream);
    }
  }
  // Two KV heads' tiles per stage. With dqk = 192 only 32-key tiles fit, and
  // those split evenly over 4 waves, not 8. With dqk = 128, 32-key tiles too:
  // the 64-key form needs all 256 registers and runs 8% slower.
  constexpr int NQG2 = DQK > 128 ? 2 : NQG;
  constexpr int BN2 = DQK >= 128 ? 32 : BN;
  const int R = a.Hkv / a.N;
  const int c = chunk_of(NS, 2);
  const SubMap paired{a.N * (NS / c), NS / c, 1, 1, g, NS, 1};
  hipError_t e = c == 2 ? launch_inst<Cfg<DQK, DV, 2, 2, true, NQG2, BN2>>(a, paired, stream)
                        : launch_inst<Cfg<DQK, DV, 1, 1, true, NQG2, BN2>>(a, paired, stream);
  if (e != hipSuccess || R <= 2) return e;
  const SubMap extra{a.N * (R - 2) * (NS / c), NS / c, R - 2, 2, g, NS, 0};
  return c == 2 ? launch_inst<Cfg<DQK, DV, 0, 2, true, NQG2, BN2>>(a, extra, stream)
                : launch_inst<Cfg<DQK, DV, 0, 1, true, NQG2, BN2>>(a, extra, stream);
}

// Causal full attention: 64-query tiles over 64-key tiles, one workgroup per
// CU. Sliding window: each query tile only touches ~W keys, so the workgroup is
// short and its memory phases dominate; 32-query tiles over 32-key tiles let
// two workgroups share a CU.
template <int DQK, int DV>
hipError_t dispatch_shape(const FwdArgs& a, hipStream_t stream) {
  if (a.window > 0) return dispatch_layout<DQK, DV, 2, 32>(a, stream);
  return dispatch_layout<DQK, DV, 4, 64>(a, stream);
}

}  // namespace

bool fwd_bf16_supported(int dqk, int dv, const UnitPlan&) {
  // Every head layout the host accepts (S % N == 0, S % Hkv == 0, one of N, Hkv
  // dividing the other) maps onto sub-units; only the head sizes are compiled.
  return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.dqk == 64 && a.dv == 64) return dispatch_shape<64, 64>(a, stream);
  if (a.dqk == 128 && a.dv == 128) return dispatch_shape<128, 128>(a, stream);
  if (a.dqk == 192 && a.dv == 128) return dispatch_shape<192, 128>(a, stream);
  return (hipError_t)-1;
}

}  // namespace gda
