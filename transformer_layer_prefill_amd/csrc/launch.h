// Host-side launchers of the prefill kernels (internal to the library).
// Every launcher enqueues on the given stream and returns the launch status;
// argument validation has already happened in the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tlp {

enum class Act { F32 = 0, BF16 = 1 };

// ---- residual assembly + RMSNorm over rows -----------------------------------
// Row r: sum = x[r] + sum_p part[p][r]; optionally res_out[r] = sum (fp32),
// act_out[r] = sum (activation type), norm_out[r] = gain * sum / sqrt(mean(sum^2) + eps).
struct RowArgs {
  const void* x;        // [rows][ldx], fp32 (x_f32) or activation type
  int x_f32, ldx;
  const float* part;    // [n_part][rows][H] split-K partial sums (nullable when n_part == 0)
  int n_part;
  size_t part_stride;   // elements between partial slices
  float* res_out;       // nullable, [rows][H]
  void* act_out;        // nullable, [rows][ld_act] activation type
  int ld_act;
  const void* gain;     // nullable (no norm), [H] activation type
  void* norm_out;       // [rows][H], fp32 (norm_f32) or activation type
  int norm_f32;
  int rows, H;
  float eps;
};
hipError_t launch_rownorm(Act act, const RowArgs& a, hipStream_t s);

// ---- projection GEMM: C[m][n] = sum_k A[m][k] * W[n][k] ---------------------
// Store: out = A W^T (act type).  Resid: out = resid + A W^T.  SwiGLU: out[:, j] =
// silu(gate_j) * up_j with gate rows [0, N) and up rows [N, 2N) of W.
// Partial: K is split into `splits` slices; slice s writes its fp32 product to
// part + s * part_stride (row stride ldo) for a later row pass to sum (bf16 only).
// StoreF32: out = A W^T as fp32 [M][ldo] in one pass (no K split).
enum class Epi { Store = 0, Resid = 1, SwiGLU = 2, Partial = 4, StoreF32 = 5 };
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
  size_t part_stride;  // Partial: elements between K-slice outputs (out is fp32)
  int* splits_out;     // Partial, optional: receives the number of K slices written
};
hipError_t launch_gemm(const GemmCall& c, hipStream_t s);

// K slices the Partial epilogue uses for an M x N x K bf16 product (1 if not split).
int gemm_partial_splits(int M, int N, int K);
// True when an M x N x K bf16 Store product runs in one pass on tiles that
// fill the GPU (128-row stream tiles, or 256x192 tiles that alone make a
// wave of blocks): such a product is better stored directly as bf16 rows
// than split into fp32 slices.
bool gemm_store_direct(int M, int N, int K, bool sign1);

// ---- skinny-M projection (decode steps, verify rows) -----------------------
// For M <= kSkinnyMaxM rows of bf16 A [M][lda] and bf16 W [N][K] (Wscale null)
// or 1-bit W (sign words u32 [N][K/32], fp16 scales Wscale [N][K/128], K % 128
// == 0): K is cut into `splits` slices and slice s writes its fp32 product
// A W^T to out + s * part_stride (row stride ldo); every slice is written, also
// an empty one (zeros).  skinny_splits picks the slice count for an N x K weight.
// (One row with dense weights runs on the vector ALUs, more rows or 1-bit
// weights on MFMAs; the slices are the same.)
constexpr int kSkinnyMaxM = 32;
constexpr int kSkinnyMaxSplits = 8;
int skinny_splits(int N, int K, bool sign1);
hipError_t launch_gemm_skinny(const void* A, int lda, const void* W, const void* Wscale, int M,
                              int N, int K, float* out, int ldo, size_t part_stride, int splits,
                              hipStream_t s);
// One bf16 row A [K] as stored, dense weights, normalised inside the
// projection: the input is RMSNorm(A) * gain (gain [K], eps), by the row
// pass's formula (only the order of the sum of squares differs) rounded to
// bf16, so no separate norm pass is needed.
// Slices and outputs are those of launch_gemm_skinny with M = 1.
// gemv_norm_ok says whether a shape's K slices are short enough to be staged
// in LDS.
bool gemv_norm_ok(int N, int K, int splits);
hipError_t launch_gemv_norm(const void* A, const void* gain, float eps, const void* W, int N, int K,
                            float* out, size_t part_stride, int splits, hipStream_t s);
// act[m][i] (bf16) = silu(g) * u with g, u the sums over `splits` fp32 slices of
// the [M][2I] gate/up product (gate columns [0, I), up columns [I, 2I)).
hipError_t launch_swiglu_finish(const float* part, int splits, size_t part_stride, int M, int I,
                                void* act, hipStream_t s);

// ---- QK-norm + RoPE + KV-cache store -----------------------------------------
// Per token t (absolute position start + t): optional per-head RMSNorm of Q and K
// heads, rotate-half RoPE of Q (written into qkv) and K, then K (roped) and V
// (raw) into cache slot start + t of every kv head of this layer.  The input row
// is qkv itself (n_part == 0) or the sum of n_part fp32 split-K slices of
// row stride qkv_ld, part_stride elements apart.
// kv16: the caches hold IEEE fp16 (bf16 activations only).
hipError_t launch_qk_rope_store(Act act, bool kv16, void* qkv, int M, int qkv_ld, const float* part,
                                int n_part, size_t part_stride, const void* q_gain,
                                const void* k_gain, bool qk_norm, float eps,
                                const float* rope_cos, const float* rope_sin, void* k_layer,
                                void* v_layer, int max_seq, int start, int nq, int nkv,
                                int head_dim, hipStream_t s);

// ---- causal GQA attention ---------------------------------------------------
// out[t][h*hd + d] for query rows t < M (roped Q at q + t*q_ld + h*hd) against
// the cache slots [0, start + t] of kv head h / (nq / nkv).
// When the (tile, head) grid alone would leave CUs idle (short micro-batches
// over long caches) and split_ws holds attention_split_floats(M, start + M, ..)
// floats, the keys are cut into ranges whose partial results (max, weight sum,
// unnormalised output) a second pass merges.
constexpr int kAttnMaxSplits = 64;
int attention_kv_splits(int M, int kv_len, int nq, int nkv);
size_t attention_split_floats(int M, int kv_len, int nq, int nkv, int head_dim);
hipError_t launch_attention(Act act, bool kv16, const void* q, int q_ld, const void* k_layer,
                            const void* v_layer, void* out, int out_ld, int M, int start,
                            int nq, int nkv, int head_dim, int max_seq, float* split_ws,
                            size_t split_ws_floats, hipStream_t s);

// ---- last-token head --------------------------------------------------------
// logits[v] = sum_k W[v][k] * xn[k] with xn fp32 [H] and W [V][H] in act type.
hipError_t launch_lm_head(Act act, const float* xn, const void* W, float* logits, int V, int H,
                          hipStream_t s);

// ---- greedy token choice ------------------------------------------------------
// out[r] = the lowest index v < vocab with logits[r * ld + v] maximal.
hipError_t launch_argmax_rows(const float* logits, int rows, int vocab, size_t ld, int32_t* out,
                              hipStream_t s);


}  // namespace tlp
