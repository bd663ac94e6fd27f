// gda_kernels.hpp - launch interface between the libgda host API and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gda {

// How the heads of one batch row are grouped into units (see gda_api.cpp):
// a unit is R KV heads u*R .. u*R+R-1; phase p of the unit attends over KV head
// u*R+p with NS signal heads (and, in phase 0, NN noise heads).
struct UnitPlan {
  int units;  // units per batch row
  int NS;     // signal heads per phase
  int NN;     // noise heads (all in phase 0)
  int R;      // phases (KV heads) per unit
};

struct FwdArgs {
  const void* q_sig;
  const void* q_noise;
  const void* k;
  const void* v;
  const void* lam;
  const void* gate;
  void* out;
  // Packed sequences (both NULL for a batch): B sequences, sequence i owning query
  // rows cu_q[i] .. cu_q[i+1]-1 and key rows cu_k[i] .. cu_k[i+1]-1 (device arrays);
  // L is then the longest query count.
  const int32_t* cu_q;
  const int32_t* cu_k;
  int B, L, S, N, Hkv, dqk, dv, window;
  UnitPlan plan;
  float scale_log2;  // log2(e) * softmax scale
  float scale;       // softmax scale (1 / sqrt(dqk) unless the caller gives one)
  int flags;         // GDA_LAMBDA_LOGITS | GDA_GATE_LOGITS
  // Training form (all NULL otherwise): per-path outputs h_sig [rows,S,dv],
  // h_noise [rows,N,dv] and row log-sum-exps, head hd of local query t of
  // sequence b at lse[lse_b * b + lse_q * (b's first query row) + hd * lse_h + t]:
  // [B,S+N,L] for a batch, [S+N,Tq] for packed sequences.
  void* h_sig = nullptr;
  void* h_noise = nullptr;
  float* lse = nullptr;
  int64_t lse_b = 0, lse_h = 0;
  int lse_q = 0;
};

struct DecodeArgs {
  const void* q_sig;
  const void* q_noise;
  const void* k;
  const void* v;
  const int32_t* lens;
  const void* lam;
  const void* gate;
  void* out;
  int B, Lmax, S, N, Hkv, dqk, dv, window;
  UnitPlan plan;
  float scale_log2;
  float scale;
  int flags;
};

struct LatentArgs {
  const void* q_sig;   // [B, S, Dn+Dr]
  const void* q_noise; // [B, N, Dn+Dr]
  const void* c_kv;    // [B, Lmax, Dc]
  const void* k_rope;  // [B, Lmax, Dr]
  const void* w_kv_b;  // [Hkv, Dn+dv, Dc]
  const int32_t* lens;
  const void* lam;
  const void* gate;
  void* out;
  void* workspace;
  int B, Lmax, S, N, Hkv, window;
  float scale_log2;
  int flags;
};

// Backward of the prefill (bf16): inputs, the training-form forward outputs,
// d_out, the gradients, and a workspace of bwd_workspace_bytes.
struct BwdArgs {
  const void* q_sig;
  const void* q_noise;
  const void* k;
  const void* v;
  const void* lam;
  const void* gate;
  const void* h_sig;    // [B,L,S,dv]
  const void* h_noise;  // [B,L,N,dv]
  const float* lse;     // [B,S+N,L], natural log
  const void* d_out;    // [B,L,S,dv]
  void* dq_sig;
  void* dq_noise;
  void* dk;
  void* dv_out;
  void* dlam;
  void* dgate;
  void* workspace;
  int B, L, S, N, Hkv, dqk, dv, window;
  float scale_log2;
  float scale;
  int flags;
  // Packed sequences (both NULL for a batch): B sequences, sequence i owning query
  // rows cu_q[i] .. cu_q[i+1]-1 and key rows cu_k[i] .. cu_k[i+1]-1; L is then the
  // longest query count and Lk_max the longest key count (a batch: Lk_max = L).
  const int32_t* cu_q = nullptr;
  const int32_t* cu_k = nullptr;
  int Lk_max = 0;
  int64_t rows = 0;  // query rows in all (B * L for a batch)
  // lse (and delta) of head hd, local query t of sequence b at
  // lse_b * b + lse_q * (b's first query row) + hd * lse_h + t
  int64_t lse_b = 0, lse_h = 0;
  int lse_q = 0;
  // carved from the workspace by the launcher
  uint16_t* do_sig = nullptr;    // [B,L,S,dv]
  uint16_t* do_noise = nullptr;  // [B,L,N,dv]
  float* delta = nullptr;        // [B,S+N,L]
};

// Each returns hipSuccess or the launch error; -1 cast to hipError_t means no
// compiled instance matches (the host API checks support first).
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream);

bool fwd_bf16_supported(int dqk, int dv, const UnitPlan& plan);
hipError_t launch_decode_latent(const LatentArgs& a, hipStream_t stream);
// Address of this GPU's static latent-decode scratch (looked up once per device,
// with that device current), for the allocation-free entry point.
hipError_t latent_scratch(void** ptr);
bool latent_supported(int Dn, int Dr, int Dc, int dv, int S, int N, int Hkv);
size_t latent_workspace_bytes(int B, int Lmax, int S, int N, int window);
bool decode_bf16_supported(int dqk, int dv, const UnitPlan& plan);
bool bwd_bf16_supported(int dqk, int dv);
size_t bwd_workspace_bytes(int B, int L, int S, int N, int dv);
hipError_t launch_bwd_bf16(BwdArgs a, hipStream_t stream);

}  // namespace gda
