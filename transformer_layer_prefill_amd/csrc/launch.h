// Host-side launchers of the prefill kernels (internal to the library).
// Every launcher enqueues on the given stream and returns the launch status;
// argument validation has already happened in the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tlp {

enum class Act { F32 = 0, BF16 = 1 };

// ---- RMSNorm over rows ------------------------------------------------------
// out[r][:] = gain * x[r][:] / sqrt(mean(x[r]^2) + eps) for r < rows.
// x_f32 selects the input type (fp32 residual stream or activation type);
// res_copy (nullable) receives x as fp32, the layer's residual stream.
hipError_t launch_rmsnorm(Act act, const void* x, bool x_f32, int ldx, float* res_copy,
                          const void* gain, void* out, bool out_f32, int rows, int H,
                          float eps, hipStream_t s);

// ---- projection GEMM: C[m][n] = sum_k A[m][k] * W[n][k] ---------------------
// Store: out = A W^T (act type).  Resid: out = resid + A W^T.  SwiGLU: out[:, j] =
// silu(gate_j) * up_j with gate rows [0, N) and up rows [N, 2N) of W.
// AtomicAdd: fp32 out += A W^T with atomic adds (bf16 only; may split K).
enum class Epi { Store = 0, Resid = 1, SwiGLU = 2, AtomicAdd = 3 };
struct GemmCall {
  Act act;             // A, W (dense) and Store/SwiGLU outputs use this type
  const void* A;       // [M][K], row stride lda
  int lda;
  const void* W;       // dense [Nw][K] (act type) or 1-bit sign words u32 [Nw][K/32]
  const void* Wscale;  // 1-bit: fp16 [Nw][K/128]; dense: nullptr
  int M, N, K;         // N = output columns (SwiGLU: the intermediate size I)
  Epi epi;
  void* out;           // Store/SwiGLU: act [M][ldo]; Resid: fp32 or act (out_f32)
  int ldo;
  bool out_f32;
  const float* resid;  // Resid: fp32 [M][ldr] added to the product (may alias out)
  int ldr;
  float* res_out;      // Resid, optional: fp32 copy of the sum, row stride ldr (may alias resid)
};
hipError_t launch_gemm(const GemmCall& c, hipStream_t s);

// ---- QK-norm + RoPE + KV-cache store -----------------------------------------
// Per token t (absolute position start + t): optional per-head RMSNorm of Q and K
// heads, rotate-half RoPE of Q (in place inside qkv) and K, then K (roped) and V
// (raw) into cache slot start + t of every kv head of this layer.
hipError_t launch_qk_rope_store(Act act, void* qkv, int M, int qkv_ld, const void* q_gain,
                                const void* k_gain, bool qk_norm, float eps,
                                const float* rope_cos, const float* rope_sin, void* k_layer,
                                void* v_layer, int max_seq, int start, int nq, int nkv,
                                int head_dim, hipStream_t s);

// ---- causal GQA attention ---------------------------------------------------
// out[t][h*hd + d] for query rows t < M (roped Q at q + t*q_ld + h*hd) against
// the cache slots [0, start + t] of kv head h / (nq / nkv).
hipError_t launch_attention(Act act, const void* q, int q_ld, const void* k_layer,
                            const void* v_layer, void* out, int out_ld, int M, int start,
                            int nq, int nkv, int head_dim, int max_seq, hipStream_t s);

// ---- last-token head --------------------------------------------------------
// logits[v] = sum_k W[v][k] * xn[k] with xn fp32 [H] and W [V][H] in act type.
hipError_t launch_lm_head(Act act, const float* xn, const void* W, float* logits, int V, int H,
                          hipStream_t s);

// Copy rows of the fp32 residual stream back to the activation type.
hipError_t launch_store_rows(Act act, const float* src, void* dst, int rows, int H,
                             hipStream_t s);

}  // namespace tlp
