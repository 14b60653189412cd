// Token choice on the GPU (oxibonsai-kernels metal_prefill.rs: the greedy
// branch of encode_full_forward_prefill's tail, which dispatches an argmax
// over the logits and returns one u32 token id instead of the logits, and
// the per-position argmax of encode_full_forward_prefill_verify's tail).
// That page does not show the argmax kernel's body; here ties go to the
// lowest index.
#include <climits>

#include "common.h"
#include "launch.h"

namespace tlp {

// One block per row.  Each thread scans its strided share in increasing
// index order keeping the first maximum; the block then reduces (value,
// index) pairs preferring the larger value, then the smaller index.  NaN
// never compares greater, so it is never chosen; a row without any entry
// above -inf yields index 0.
__global__ __launch_bounds__(1024) void argmax_rows_kernel(const float* __restrict__ logits,
                                                           int vocab, size_t ld,
                                                           int32_t* __restrict__ out) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const float* row = logits + static_cast<size_t>(blockIdx.x) * ld;
  float best = -INFINITY;
  int idx = INT_MAX;
  auto take = [&](float x, int v) {
    if (x > best) {
      best = x;
      idx = v;
    }
  };
  // A thread visits its indices in increasing order (so its first maximum
  // is the lowest index), four 16-byte loads in flight at a time.
  int done = 0;
  if ((ld & 3) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0) {
    const float4* row4 = reinterpret_cast<const float4*>(row);
    const int n4 = vocab >> 2, bd = blockDim.x;
    for (int base = threadIdx.x; base < n4; base += 4 * bd) {
      float4 q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (base + u * bd < n4) q[u] = row4[base + u * bd];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + u * bd;
        if (i < n4) {
          take(q[u].x, 4 * i);
          take(q[u].y, 4 * i + 1);
          take(q[u].z, 4 * i + 2);
          take(q[u].w, 4 * i + 3);
        }
      }
    }
    done = n4 << 2;
  }
  for (int v = done + threadIdx.x; v < vocab; v += blockDim.x) take(row[v], v);
  auto better = [](float a, int ia, float b, int ib) { return b > a || (b == a && ib < ia); };
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ob = __shfl_xor(best, off, 64);
    const int oi = __shfl_xor(idx, off, 64);
    if (better(best, idx, ob, oi)) {
      best = ob;
      idx = oi;
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = idx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = sv[0];
    int i = si[0];
    for (int w = 1; w < nw; ++w)
      if (better(b, i, sv[w], si[w])) {
        b = sv[w];
        i = si[w];
      }
    out[blockIdx.x] = i == INT_MAX ? 0 : i;
  }
}

hipError_t launch_argmax_rows(const float* logits, int rows, int vocab, size_t ld, int32_t* out,
                              hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  argmax_rows_kernel<<<rows, 1024, 0, s>>>(logits, vocab, ld, out);
  return hipGetLastError();
}

}  // namespace tlp
