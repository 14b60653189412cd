// Projection GEMMs of the layer: C[m][n] = sum_k A[m][k] * W[n][k] over all
// tokens of a micro-batch (oxibonsai-kernels metal_prefill.rs,
// encode_layer_prefill steps 2, 4, 6 and 7: the QKV GEMM, the output
// projection with residual, the fused gate+up+SwiGLU GEMM and the down
// projection with residual).  Both operands are K-contiguous, tokens are rows.
//
// bf16 path: CDNA4 v_mfma_f32_32x32x16_bf16, fp32 accumulation, LDS-staged
// double-buffered tiles with register prefetch, XCD-aware tile order.
// 1-bit path: the same kernel with the weight tile expanded from packed sign
// bits and an fp16 group scale into bf16 while it is staged into LDS.
// fp32 path: a plain LDS-tiled FMA kernel (small correctness shapes).
#include "common.h"
#include "launch.h"

namespace tlp {

struct GemmArgs {
  const uint16_t* A;
  const void* W;
  const uint16_t* Wscale;  // fp16 bit patterns
  void* out;
  const float* resid;
  float* res_out;
  int lda, ldo, ldr;
  int M, N, K;
  int m_tiles, n_tiles;
  int up_row;  // SwiGLU: row offset of the up half (= N)
};

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Tile t of the grid, remapped so that each XCD (blocks b, b+8, ...) works
// through a contiguous run of tiles: the M-tiles that share one weight tile
// then meet in the same L2.
__device__ __forceinline__ int xcd_tile(int b, int nb) {
  if ((nb & 7) != 0) return b;
  return (b & 7) * (nb >> 3) + (b >> 3);
}

template <int BM, int BN, int WM, int WN, int EPI, bool SIGN1, bool OUT_F32>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int BK = 64;
  constexpr int LD = BK + 8;  // padded LDS row (elements): 144 B, conflict-free b128 reads
  constexpr int T = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int A_PER = BM * BK / 8 / T;  // 16-byte chunks per thread
  constexpr int B_PER = BN * BK / 8 / T;
  constexpr int S_PER = BN * 2 / T;       // 1-bit: (row, 32-column word) pairs per thread
  static_assert(A_PER >= 1 && BM * BK / 8 % T == 0, "A tile split");
  static_assert(SIGN1 ? (S_PER >= 1 && BN * 2 % T == 0) : (B_PER >= 1 && BN * BK / 8 % T == 0),
                "B tile split");
  static_assert(EPI != 2 || FN % 2 == 0, "SwiGLU pairs gate and up fragments");

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LD];

  const int t = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = t % g.m_tiles, nt = t / g.m_tiles;
  const int m0 = mt * BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // weight row of LDS tile row r (SwiGLU interleaves gate and up halves per wave)
  auto b_row = [&](int r, bool& ok) -> int {
    if constexpr (EPI == 2) {
      const int w = r / TN, rr = r % TN;
      const int jj = nt * (BN / 2) + w * (TN / 2) + rr % (TN / 2);
      ok = jj < g.N;
      return rr >= TN / 2 ? g.up_row + jj : jj;
    } else {
      const int n = nt * BN + r;
      ok = n < g.N;
      return n;
    }
  };

  uint4 a_reg[A_PER];
  uint4 b_reg[SIGN1 ? 1 : B_PER];
  uint32_t s_word[SIGN1 ? S_PER : 1];
  uint16_t s_scale[SIGN1 ? S_PER : 1];

  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * T;
      const int r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
      const int m = m0 + r, k = k0 + kc;
      a_reg[i] = (m < g.M && k < g.K)
                     ? *reinterpret_cast<const uint4*>(g.A + static_cast<size_t>(m) * g.lda + k)
                     : make_uint4(0, 0, 0, 0);
    }
    if constexpr (!SIGN1) {
      const uint16_t* W = static_cast<const uint16_t*>(g.W);
#pragma unroll
      for (int i = 0; i < B_PER; ++i) {
        const int c = tid + i * T;
        const int r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
        bool ok;
        const int n = b_row(r, ok);
        const int k = k0 + kc;
        b_reg[i] = (ok && k < g.K)
                       ? *reinterpret_cast<const uint4*>(W + static_cast<size_t>(n) * g.K + k)
                       : make_uint4(0, 0, 0, 0);
      }
    } else {
      const uint32_t* Wb = static_cast<const uint32_t*>(g.W);
#pragma unroll
      for (int i = 0; i < S_PER; ++i) {
        const int c = tid + i * T;
        const int r = c >> 1, wd = c & 1;
        bool ok;
        const int n = b_row(r, ok);
        const int k = k0 + wd * 32;
        ok = ok && k < g.K;
        s_word[i] = ok ? Wb[static_cast<size_t>(n) * (g.K >> 5) + (k >> 5)] : 0u;
        s_scale[i] = ok ? g.Wscale[static_cast<size_t>(n) * (g.K >> 7) + (k >> 7)] : 0;
      }
    }
  };

  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * T;
      const int r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
      *reinterpret_cast<uint4*>(&As[buf][r * LD + kc]) = a_reg[i];
    }
    if constexpr (!SIGN1) {
#pragma unroll
      for (int i = 0; i < B_PER; ++i) {
        const int c = tid + i * T;
        const int r = c / (BK / 8), kc = (c % (BK / 8)) * 8;
        *reinterpret_cast<uint4*>(&Bs[buf][r * LD + kc]) = b_reg[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < S_PER; ++i) {
        const int c = tid + i * T;
        const int r = c >> 1, wd = c & 1;
        // +scale for a set bit, -scale for a clear one, as bf16 bit patterns
        const uint32_t pos = f32_to_bf16(f16_to_f32(s_scale[i]));
        const uint32_t neg = pos | 0x8000u;
        const uint32_t w = s_word[i];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t b0 = (w >> (q * 8 + 2 * e)) & 1u;
            const uint32_t b1 = (w >> (q * 8 + 2 * e + 1)) & 1u;
            h[e] = (b0 ? pos : neg) | ((b1 ? pos : neg) << 16);
          }
          *reinterpret_cast<uint4*>(&Bs[buf][r * LD + wd * 32 + q * 8]) =
              make_uint4(h[0], h[1], h[2], h[3]);
        }
      }
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (g.K + BK - 1) / BK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();

  const int lr = lane & 31, lh = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tiles((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(
            &As[buf][(wm * TM + i * 32 + lr) * LD + kk * 16 + lh * 8]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(
            &Bs[buf][(wn * TN + j * 32 + lr) * LD + kk * 16 + lh * 8]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tiles(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: lane owns column (lane & 31) and rows
  // 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * TM + i * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
      if (m >= g.M) continue;
      if constexpr (EPI == 2) {
        uint16_t* o = static_cast<uint16_t*>(g.out) + static_cast<size_t>(m) * g.ldo;
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
          const int n = nt * (BN / 2) + wn * (TN / 2) + j * 32 + lr;
          if (n < g.N) {
            const float gate = acc[i][j][r], up = acc[i][j + FN / 2][r];
            o[n] = f32_to_bf16(silu_f32(gate) * up);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int n = nt * BN + wn * TN + j * 32 + lr;
          if (n >= g.N) continue;
          float v = acc[i][j][r];
          if constexpr (EPI == 1) {
            v += g.resid[static_cast<size_t>(m) * g.ldr + n];
            if (g.res_out) g.res_out[static_cast<size_t>(m) * g.ldr + n] = v;
          }
          if constexpr (OUT_F32)
            static_cast<float*>(g.out)[static_cast<size_t>(m) * g.ldo + n] = v;
          else
            static_cast<uint16_t*>(g.out)[static_cast<size_t>(m) * g.ldo + n] = f32_to_bf16(v);
        }
      }
    }
  }
}

// ---- fp32 FMA kernel --------------------------------------------------------
// 64x64 tile, 256 threads; thread (tx, ty) owns rows ty*4..+4 and columns
// {2tx, 2tx+1, 32+2tx, 33+2tx}, so the SwiGLU epilogue finds gate column c
// and its up partner c+32 in the same thread.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const float* A = reinterpret_cast<const float*>(g.A);
  const float* W = static_cast<const float*>(g.W);
  const int mt = blockIdx.x % g.m_tiles, nt = blockIdx.x / g.m_tiles;
  const int m0 = mt * BM;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += BK) {
    for (int c = tid; c < BM * BK; c += 256) {
      const int r = c / BK, k = c % BK;
      const int m = m0 + r;
      As[k][r] = (m < g.M && k0 + k < g.K) ? A[static_cast<size_t>(m) * g.lda + k0 + k] : 0.f;
      int n;
      bool ok;
      if (EPI == 2) {
        const int jj = nt * (BN / 2) + (r & 31);
        ok = jj < g.N;
        n = r >= 32 ? g.up_row + jj : jj;
      } else {
        n = nt * BN + r;
        ok = n < g.N;
      }
      Bs[k][r] = (ok && k0 + k < g.K) ? W[static_cast<size_t>(n) * g.K + k0 + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
      b[0] = Bs[k][2 * tx];
      b[1] = Bs[k][2 * tx + 1];
      b[2] = Bs[k][32 + 2 * tx];
      b[3] = Bs[k][33 + 2 * tx];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const int cols[4] = {2 * tx, 2 * tx + 1, 32 + 2 * tx, 33 + 2 * tx};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
    if (EPI == 2) {
      float* o = static_cast<float*>(g.out) + static_cast<size_t>(m) * g.ldo;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = nt * (BN / 2) + cols[j];
        if (n < g.N) o[n] = silu_f32(acc[i][j]) * acc[i][j + 2];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = nt * BN + cols[j];
        if (n >= g.N) continue;
        float v = acc[i][j];
        if (EPI == 1) {
          v += g.resid[static_cast<size_t>(m) * g.ldr + n];
          if (g.res_out) g.res_out[static_cast<size_t>(m) * g.ldr + n] = v;
        }
        static_cast<float*>(g.out)[static_cast<size_t>(m) * g.ldo + n] = v;
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI, bool SIGN1, bool OUT_F32>
static hipError_t run_bf16(GemmArgs g, hipStream_t s) {
  const int cols = EPI == 2 ? BN / 2 : BN;
  g.m_tiles = (g.M + BM - 1) / BM;
  g.n_tiles = (g.N + cols - 1) / cols;
  const int blocks = g.m_tiles * g.n_tiles;
  gemm_bf16_kernel<BM, BN, WM, WN, EPI, SIGN1, OUT_F32><<<blocks, WM * WN * 64, 0, s>>>(g);
  return hipGetLastError();
}

template <int EPI, bool SIGN1, bool OUT_F32>
static hipError_t pick_bf16(GemmArgs g, hipStream_t s) {
  return run_bf16<128, 128, 2, 2, EPI, SIGN1, OUT_F32>(g, s);
}

template <bool SIGN1>
static hipError_t dispatch_bf16(const GemmCall& c, GemmArgs g, hipStream_t s) {
  switch (c.epi) {
    case Epi::Store: return pick_bf16<0, SIGN1, false>(g, s);
    case Epi::SwiGLU: return pick_bf16<2, SIGN1, false>(g, s);
    case Epi::Resid:
      return c.out_f32 ? pick_bf16<1, SIGN1, true>(g, s) : pick_bf16<1, SIGN1, false>(g, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(const GemmCall& c, hipStream_t s) {
  if (c.M <= 0 || c.N <= 0) return hipSuccess;
  GemmArgs g{};
  g.A = static_cast<const uint16_t*>(c.A);
  g.W = c.W;
  g.Wscale = static_cast<const uint16_t*>(c.Wscale);
  g.out = c.out;
  g.resid = c.resid;
  g.res_out = c.res_out;
  g.lda = c.lda;
  g.ldo = c.ldo;
  g.ldr = c.ldr;
  g.M = c.M;
  g.N = c.N;
  g.K = c.K;
  g.up_row = c.N;
  if (c.act == Act::F32) {
    const int cols = c.epi == Epi::SwiGLU ? 32 : 64;
    g.m_tiles = (c.M + 63) / 64;
    g.n_tiles = (c.N + cols - 1) / cols;
    const int blocks = g.m_tiles * g.n_tiles;
    switch (c.epi) {
      case Epi::Store: gemm_f32_kernel<0><<<blocks, 256, 0, s>>>(g); break;
      case Epi::Resid: gemm_f32_kernel<1><<<blocks, 256, 0, s>>>(g); break;
      case Epi::SwiGLU: gemm_f32_kernel<2><<<blocks, 256, 0, s>>>(g); break;
    }
    return hipGetLastError();
  }
  return c.Wscale ? dispatch_bf16<true>(c, g, s) : dispatch_bf16<false>(c, g, s);
}

}  // namespace tlp
