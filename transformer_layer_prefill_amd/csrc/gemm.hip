// Projection GEMMs of the layer: C[m][n] = sum_k A[m][k] * W[n][k] over all
// tokens of a micro-batch (oxibonsai-kernels metal_prefill.rs,
// encode_layer_prefill steps 2, 4, 6 and 7: the QKV GEMM, the output
// projection with residual, the fused gate+up+SwiGLU GEMM and the down
// projection with residual).  Both operands are K-contiguous, tokens are rows.
//
// bf16 path: CDNA4 bf16 MFMAs with fp32 accumulation; tiles copied global ->
// LDS by DMA into a double buffer (register-staged when K is not a multiple
// of 64), XCD-aware tile order.
// 1-bit path: the same direct-to-LDS kernels; the threads expand each weight
// tile from packed sign bits and an fp16 group scale into bf16 in LDS.
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
  int splits, k_split;  // split-K: number of K slices and K per slice (multiple of 64)
  size_t part_stride;   // Partial epilogue: elements between K-slice outputs
  int* splits_out;      // host-side only: receives the K slice count
  int up_row;  // SwiGLU: row offset of the up half (= N)
  uint32_t a_bytes, w_bytes;   // buffer-copy kernels: bytes readable from A and from W
};

// v if ok, else zero.  Done per component: a select between two uint4
// aggregates compiles to a round trip through scratch memory.
__device__ __forceinline__ uint4 keep_if(uint4 v, bool ok) {
  const uint32_t m = ok ? 0xffffffffu : 0u;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

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

// Epilogue shared by the bf16 kernels.  32x32 accumulator layout: lane owns
// column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4 for r = 0..15.
template <int FM, int FN, int TM, int TN, int BN, int EPI, bool OUT_F32>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, f32x16_t (&acc)[FM][FN], int m0,
                                              int nt, int wm, int wn, int lr, int lh, int split) {
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
          if constexpr (EPI == 4) {
            static_cast<float*>(g.out)[split * g.part_stride + static_cast<size_t>(m) * g.ldo + n] = v;
            continue;
          }
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

template <int BM, int BN, int WM, int WN, int EPI, bool OUT_F32>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int BK = 64;
  constexpr int LD = BK + 8;  // padded LDS row (elements): 144 B, conflict-free b128 reads
  constexpr int T = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int A_PER = BM * BK / 8 / T;  // 16-byte chunks per thread
  constexpr int B_PER = BN * BK / 8 / T;
  static_assert(A_PER >= 1 && BM * BK / 8 % T == 0, "A tile split");
  static_assert(B_PER >= 1 && BN * BK / 8 % T == 0, "B tile split");
  static_assert(EPI != 2 || FN % 2 == 0, "SwiGLU pairs gate and up fragments");

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LD];

  // work item -> (split, M-tile, N-tile); the K slices of one tile and the
  // M-tiles of one weight tile stay on one XCD
  const int wi = xcd_tile(blockIdx.x, gridDim.x);
  const int split = wi % g.splits, t = wi / g.splits;
  const int mt = t % g.m_tiles, nt = t / g.m_tiles;
  const int m0 = mt * BM;
  const int k_begin = split * g.k_split;
  const int k_end = min(g.K, k_begin + g.k_split);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lh = lane >> 5;

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

  // Chunk i of a thread is tile row tid/8 + i*T/8 at column (tid%8)*8.  Rows
  // outside the matrix and columns past the K slice read a clamped in-bounds
  // address and are zeroed, so the loads never branch.
  const int kc = (tid & 7) * 8;
  const int r0 = tid >> 3;
  const uint16_t* Wd = static_cast<const uint16_t*>(g.W);

  uint4 a_reg[A_PER];
  uint4 b_reg[B_PER];

  // Validity of the chunks in flight; applied when they are written to LDS so
  // the wait for the global loads falls after the MFMAs of the current tile.
  bool a_ok[A_PER], b_ok[B_PER];

  auto load_tiles = [&](int k0) __attribute__((always_inline)) {
    const bool k_ok = k0 + kc < k_end;
    const int col = k_ok ? k0 + kc : 0;   // invalid chunks read column 0 of their row
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int m = m0 + r0 + i * (T / 8);
      a_ok[i] = m < g.M && k_ok;
      a_reg[i] = *reinterpret_cast<const uint4*>(
          g.A + static_cast<size_t>(m < g.M ? m : g.M - 1) * g.lda + col);
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      bool ok;
      const int n = b_row(r0 + i * (T / 8), ok);
      b_ok[i] = ok && k_ok;
      b_reg[i] = *reinterpret_cast<const uint4*>(
          Wd + static_cast<size_t>(ok ? n : 0) * g.K + col);
    }
  };

  auto store_tiles = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int r = r0 + i * (T / 8);
      *reinterpret_cast<uint4*>(&As[buf][r * LD + kc]) = keep_if(a_reg[i], a_ok[i]);
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int r = r0 + i * (T / 8);
      *reinterpret_cast<uint4*>(&Bs[buf][r * LD + kc]) = keep_if(b_reg[i], b_ok[i]);
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Fragment registers are double-buffered across the four 16-wide k-steps of
  // a tile, so the LDS reads of step kk+1 are in flight during step kk's MFMAs.
  bf16x8_t af0[FM], bf0[FN], af1[FM], bf1[FN];
#define TLP_LOAD_FRAGS(AF, BF, BUF, KK)                                                  \
  _Pragma("unroll") for (int i = 0; i < FM; ++i) AF[i] =                                 \
      *reinterpret_cast<const bf16x8_t*>(&As[BUF][(wm * TM + i * 32 + lr) * LD + (KK) * 16 + lh * 8]); \
  _Pragma("unroll") for (int j = 0; j < FN; ++j) BF[j] =                                 \
      *reinterpret_cast<const bf16x8_t*>(&Bs[BUF][(wn * TN + j * 32 + lr) * LD + (KK) * 16 + lh * 8]);
#define TLP_MMA(AF, BF)                                                                  \
  _Pragma("unroll") for (int i = 0; i < FM; ++i)                                         \
  _Pragma("unroll") for (int j = 0; j < FN; ++j)                                         \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AF[i], BF[j], acc[i][j], 0, 0, 0);

  const int nk = (k_end - k_begin + BK - 1) / BK;
  load_tiles(k_begin);
  store_tiles(0);
  __syncthreads();
  TLP_LOAD_FRAGS(af0, bf0, 0, 0)

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) load_tiles(k_begin + (kt + 1) * BK);
    TLP_LOAD_FRAGS(af1, bf1, buf, 1)
    TLP_MMA(af0, bf0)
    TLP_LOAD_FRAGS(af0, bf0, buf, 2)
    TLP_MMA(af1, bf1)
    TLP_LOAD_FRAGS(af1, bf1, buf, 3)
    TLP_MMA(af0, bf0)
    // the next tile goes into the other buffer, whose last reads (k-step 3 of
    // the previous tile) completed before the previous barrier
    if (more) store_tiles(buf ^ 1);
    __syncthreads();
    if (more) { TLP_LOAD_FRAGS(af0, bf0, buf ^ 1, 0) }
    TLP_MMA(af1, bf1)
  }
#undef TLP_LOAD_FRAGS
#undef TLP_MMA

  gemm_epilogue<FM, FN, TM, TN, BN, EPI, OUT_F32>(g, acc, m0, nt, wm, wn, lr, lh, split);
}

// ---- bf16 kernel with direct global->LDS loads ------------------------------
// Dense weights with K a multiple of 64.  Tiles are 64 wide in K (one full
// 128-byte line per row, which streams much faster than half lines) and are
// copied global -> LDS by global_load_lds_dwordx4 into a double buffer, so
// there is no register staging.  Each DMA instruction writes 1 KB (8 rows of
// 128 B) contiguously; lane l of it fetches the 16-byte chunk
// (l%8) ^ swz(row) of row l/8, which stores chunk c of row r at slot
// c ^ swz(r): any 8 consecutive rows, and any 16 rows taken as 8 pairs, read
// at one chunk hit distinct banks.  Rows past M or N are clamped to a valid
// row; their products land in discarded outputs.
__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// Chunk swizzle of the 16x16x32 kernel's tiles.  A 16-byte LDS read is served
// sixteen lanes per cycle, lanes 8h..8h+7 together with 32+8h..32+8h+7; in the
// 16x16x32 operand layout those two sets read chunks q and q^2 of the same
// eight rows, where the 32x32x16 layout reads q and q^1.  Rows of one parity
// (one half of the 64 banks) therefore need swizzles that stay distinct under
// ^2 within each group of eight rows and are all distinct within sixteen:
// {0, 1, 4, 5} for rows 0-7 of a parity, {2, 3, 6, 7} for rows 8-15.
__device__ __forceinline__ int swz16(int r) { return ((r >> 1) & 1) | (r & 4) | ((r >> 2) & 2); }

template <int BM, int BN, int WM, int WN, int EPI, bool OUT_F32, bool SIGN1>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_dma_kernel(GemmArgs g) {
  constexpr int BK = 64;
  constexpr int ROWB = BK * 2;          // 128 bytes
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_PW = A_BYTES / 1024 / NW, B_PW = B_BYTES / 1024 / NW;  // DMA blocks per wave
  static_assert(A_PW * NW * 1024 == A_BYTES && B_PW * NW * 1024 == B_BYTES, "DMA split");
  static_assert(EPI != 2 || FN % 2 == 0, "SwiGLU pairs gate and up fragments");
  constexpr int S_ITEMS = 2 * BN;       // 1-bit: (row, 32-column word) pairs per tile
  static_assert(!SIGN1 || (S_ITEMS <= NW * 64 && S_ITEMS % 64 == 0), "1-bit items");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int wi = xcd_tile(blockIdx.x, gridDim.x);
  const int split = wi % g.splits, t = wi / g.splits;
  const int mt = t % g.m_tiles, nt = t / g.m_tiles;
  const int m0 = mt * BM;
  const int k_begin = split * g.k_split;
  const int k_end = min(g.K, k_begin + g.k_split);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lh = lane >> 5;
  const uint16_t* W = static_cast<const uint16_t*>(g.W);
  // weight row of B-tile row r (SwiGLU: each wavefront column holds TN/2 gate
  // rows then the TN/2 up rows of the same output columns); rows past N are
  // clamped, their products land in discarded outputs
  auto b_row = [&](int r) -> int {
    if constexpr (EPI == 2) {
      const int w = r / TN, rr = r % TN;
      const int jj = min(nt * (BN / 2) + w * (TN / 2) + rr % (TN / 2), g.N - 1);
      return rr >= TN / 2 ? g.up_row + jj : jj;
    } else {
      return min(nt * BN + r, g.N - 1);
    }
  };

  // global source rows of this lane's DMA chunks (fixed over the K loop)
  const int drow = lane >> 3, dslot = lane & 7;
  const uint16_t* a_src[A_PW];
  const uint16_t* b_src[SIGN1 ? 1 : B_PW];
#pragma unroll
  for (int j = 0; j < A_PW; ++j) {
    const int row = (wave * A_PW + j) * 8 + drow;
    const int m = min(m0 + row, g.M - 1);
    a_src[j] = g.A + static_cast<size_t>(m) * g.lda + (dslot ^ swz8(row)) * 8;
  }
  if constexpr (!SIGN1) {
#pragma unroll
    for (int j = 0; j < B_PW; ++j) {
      const int row = (wave * B_PW + j) * 8 + drow;
      b_src[j] = W + static_cast<size_t>(b_row(row)) * g.K + (dslot ^ swz8(row)) * 8;
    }
  }
  // 1-bit weights: thread i < 2*BN owns (B-tile row i/2, 32-column word i%2),
  // loads its sign word and group scale two tiles ahead and expands them into
  // bf16 +-scale in the stage the barrier has freed, once this wavefront's
  // MFMAs of the iteration are issued (the next barrier publishes it);
  // ownership is wavefront-uniform
  const bool s_own = SIGN1 && tid < S_ITEMS;
  const int s_row = min(tid >> 1, BN - 1), s_wd = tid & 1;
  const uint32_t* s_wsrc = nullptr;
  const uint16_t* s_ssrc = nullptr;
  if constexpr (SIGN1) {
    const size_t wr = static_cast<size_t>(b_row(s_row));
    s_wsrc = static_cast<const uint32_t*>(g.W) + wr * (g.K >> 5) + s_wd;
    s_ssrc = g.Wscale + wr * (g.K >> 7);
  }
  const int s_off = A_BYTES + s_row * ROWB, s_sw = swz8(s_row);
  auto load_s = [&](int kt, uint32_t& word, uint32_t& scale) __attribute__((always_inline)) {
    const int k0 = k_begin + kt * BK;
    word = s_wsrc[k0 >> 5];
    scale = s_ssrc[k0 >> 7];
  };
  auto store_s = [&](int kt, uint32_t word, uint32_t scale) __attribute__((always_inline)) {
    char* st = smem + (kt & 1) * STAGE + s_off;
    const uint32_t sbf = f32_to_bf16(f16_to_f32(static_cast<uint16_t>(scale)));
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(st + (((4 * s_wd + q) ^ s_sw) << 4)) =
          sign1_expand8((word >> (8 * q)) & 0xffu, sbf);
  };

  auto issue = [&](int kt) __attribute__((always_inline)) {
    const int k0 = k_begin + kt * BK;
    char* st = smem + (kt & 1) * STAGE;
#pragma unroll
    for (int j = 0; j < A_PW; ++j) dma16(a_src[j] + k0, st + (wave * A_PW + j) * 1024);
    if constexpr (!SIGN1) {
#pragma unroll
      for (int j = 0; j < B_PW; ++j) dma16(b_src[j] + k0, st + A_BYTES + (wave * B_PW + j) * 1024);
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment byte offsets inside a stage: row * 128 + swizzled chunk; the
  // fragment rows are 32-aligned, so swz(row) = swz(lr)
  const int sw = swz8(lr);
  const int a_off = (wm * TM + lr) * ROWB, b_off = A_BYTES + (wn * TN + lr) * ROWB;
  int ch[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) ch[kk] = ((kk * 2 + lh) ^ sw) << 4;
  bf16x8_t af0[FM], bf0[FN], af1[FM], bf1[FN];
#define TLP_FRAGS(AF, BF, ST, C)                                                             \
  _Pragma("unroll") for (int i = 0; i < FM; ++i) AF[i] =                                     \
      *reinterpret_cast<const bf16x8_t*>((ST) + a_off + i * 32 * ROWB + (C));                \
  _Pragma("unroll") for (int j = 0; j < FN; ++j) BF[j] =                                     \
      *reinterpret_cast<const bf16x8_t*>((ST) + b_off + j * 32 * ROWB + (C));
#define TLP_MMA(AF, BF)                                                                      \
  _Pragma("unroll") for (int i = 0; i < FM; ++i)                                             \
  _Pragma("unroll") for (int j = 0; j < FN; ++j)                                             \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AF[i], BF[j], acc[i][j], 0, 0, 0);

  // Schedule per 64-wide tile kt (four 16-wide k-steps, fragments of step s+1
  // read during the MFMAs of step s): after the MFMAs of step 2 are issued,
  // wait for tile kt+1, barrier (every wave has read all of tile kt), refill
  // tile kt's stage with tile kt+2, read step 0 of tile kt+1, then step 3's MFMAs.
  const int nk = (k_end - k_begin) / BK;
  uint32_t s_word = 0, s_scale = 0;   // 1-bit: tile kt+2's item, in flight during tile kt
  if constexpr (SIGN1) {
    // tiles 0 and 1 are expanded before the first barrier
    uint32_t w0 = 0, c0 = 0, w1 = 0, c1 = 0;
    issue(0);
    if (s_own) load_s(0, w0, c0);
    if (nk > 1) {
      issue(1);
      if (s_own) load_s(1, w1, c1);
    }
    __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);
    if (s_own) {
      store_s(0, w0, c0);
      if (nk > 1) store_s(1, w1, c1);
      if (nk > 2) load_s(2, s_word, s_scale);
    }
  } else {
    issue(0);
    if (nk > 1) issue(1);
    if (nk > 1) __builtin_amdgcn_s_waitcnt(VmWait<A_PW + B_PW>::imm);
    else __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);
  }
  lds_barrier();
  TLP_FRAGS(af0, bf0, smem, ch[0])
  // drain every scalar load too: a scalar load still pending at the loop
  // entry would force full LDS waits inside the loop
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt/expcnt untouched

  int kt = 0;
  for (; kt + 1 < nk; ++kt) {
    const char* st = smem + (kt & 1) * STAGE;
    TLP_FRAGS(af1, bf1, st, ch[1])
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA(af0, bf0)
    __builtin_amdgcn_sched_barrier(0);
    TLP_FRAGS(af0, bf0, st, ch[2])
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA(af1, bf1)
    __builtin_amdgcn_sched_barrier(0);
    TLP_FRAGS(af1, bf1, st, ch[3])
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA(af0, bf0)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);   // tile kt+1 (and tile kt+2's 1-bit item)
    lds_barrier();
    if (kt + 2 < nk) issue(kt + 2);
    const char* st1 = smem + ((kt + 1) & 1) * STAGE;
    TLP_FRAGS(af0, bf0, st1, ch[0])
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA(af1, bf1)
    __builtin_amdgcn_sched_barrier(0);
    // 1-bit: tile kt+2's weights into that stage, after this step's MFMAs
    // are issued (the next iteration's barrier publishes them)
    if constexpr (SIGN1) {
      if (s_own && kt + 2 < nk) {
        store_s(kt + 2, s_word, s_scale);
        if (kt + 3 < nk) load_s(kt + 3, s_word, s_scale);
      }
    }
  }
  {
    const char* st = smem + (kt & 1) * STAGE;
    TLP_FRAGS(af1, bf1, st, ch[1])
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA(af0, bf0)
    TLP_FRAGS(af0, bf0, st, ch[2])
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA(af1, bf1)
    TLP_FRAGS(af1, bf1, st, ch[3])
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA(af0, bf0)
    TLP_MMA(af1, bf1)
  }
#undef TLP_FRAGS
#undef TLP_MMA

  gemm_epilogue<FM, FN, TM, TN, BN, EPI, OUT_F32>(g, acc, m0, nt, wm, wn, lr, lh, split);
}

// ---- gate/up + SwiGLU with 112- or 96-column output tiles ----------------------
// A block covers 256 token rows and COLS output columns, i.e. 2*COLS weight
// rows: each of the two wavefront columns holds COLS/2 gate and COLS/2 up rows
// interleaved eight by eight.  A 512-token micro-batch makes 2 x (I / COLS)
// blocks: 256 (one per CU) for I = 14336 with 112 columns and for I = 12288
// with 96, where 256x256 tiles make 224 and 192 and leave CUs idle.  Eight
// wavefronts of 64 rows x 2*COLS/2 weight rows use v_mfma_f32_16x16x32_bf16
// (4 x COLS/16 fragments of 16x16); K tiles of 64 are read from LDS with the
// same row swizzle as the 256x256 kernel.  In the 16x16 result layout lane l
// holds column l % 16 of its fragment, so the gate value of an output column
// sits eight lanes away from its up value.
//
// Dense weights: both tiles are copied global -> LDS with global_load_lds_dwordx4
// into a double buffer.  1-bit weights: the activation tile is copied the same
// way; thread i < 4*COLS owns (weight row i/2, 32-column word i%2) of the tile,
// loads its sign word and group scale two tiles ahead into registers and,
// once the barrier has freed a stage and this wavefront's MFMAs of the second
// k-step are issued, expands them into bf16 +-scale in that stage (K % 128 ==
// 0: a 64-wide tile lies inside one scale group).  The barrier of the next
// iteration publishes the expanded tile before its reads.
template <int COLS>
__device__ __forceinline__ int swiglu_b_row(const GemmArgs& g, int nt, int rr) {
  const int wn = rr / COLS, q = rr % COLS;
  const int idx = min(nt * COLS + wn * (COLS / 2) + 8 * (q / 16) + (q & 7), g.N - 1);
  return (q & 8) ? g.up_row + idx : idx;
}

template <int COLS, bool SIGN1>
__global__ __launch_bounds__(512) void gemm_swiglu_kernel(GemmArgs g) {
  constexpr int BM = 256, BR = 2 * COLS, BK = 64, ROWB = 128;
  constexpr int FM = 4, FN = COLS / 16;                     // 16x16 fragments per wavefront
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BR * ROWB;   // 32 KB + 28 or 24 KB
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_PW = 4;                                   // DMA blocks per wavefront
  constexpr int B_BLK = B_BYTES / 1024;                     // 28 or 24
  constexpr int B_PW = (B_BLK + 7) / 8;                     // 4 (wavefront 7 copies no B) or 3
  constexpr int S_ITEMS = 2 * BR;                           // 1-bit: (row, word) pairs per tile
  static_assert(COLS % 16 == 0 && S_ITEMS <= 512 && S_ITEMS % 64 == 0, "tile shape");
  typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int wi = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = wi % g.m_tiles, nt = wi / g.m_tiles;
  const int m0 = mt * BM;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, lq = lane >> 4;

  const int drow = lane >> 3, dslot = lane & 7;
  const uint16_t* a_src[A_PW];
#pragma unroll
  for (int j = 0; j < A_PW; ++j) {
    const int row = (wave * A_PW + j) * 8 + drow;
    a_src[j] = g.A + static_cast<size_t>(min(m0 + row, g.M - 1)) * g.lda + (dslot ^ swz16(row)) * 8;
  }
  const uint16_t* b_src[SIGN1 ? 1 : B_PW];
  const bool has_b = wave * B_PW < B_BLK;   // wavefront-uniform
  if constexpr (!SIGN1) {
    const uint16_t* W = static_cast<const uint16_t*>(g.W);
#pragma unroll
    for (int j = 0; j < B_PW; ++j) {
      const int rr = min((wave * B_PW + j) * 8 + drow, BR - 1);
      b_src[j] = W + static_cast<size_t>(swiglu_b_row<COLS>(g, nt, rr)) * g.K + (dslot ^ swz16(rr)) * 8;
    }
  }
  // 1-bit: this thread's (row, word) item; S_ITEMS is a multiple of 64, so
  // ownership is wavefront-uniform.  A 16-byte LDS write is served eight
  // consecutive lanes per cycle over one 128-byte bank line, so each eight
  // lanes must write eight different chunk slots: a wavefront's 64 lanes take
  // the two words of its 32 rows with lane bits (3, 1, 4, 2, 5) as row bits
  // 0-4 and lane bit 0 as the word.  Lanes 8k..8k+7 then hold both words of
  // rows r, r+2, r+8 and r+10, whose swizzles differ in bits 0 and 1 while
  // the word flips bit 2 of the chunk: eight different slots.
  static_assert(!SIGN1 || BR % 32 == 0, "whole wavefronts of items");
  const bool s_own = SIGN1 && tid < S_ITEMS;
  const int s_l = tid & 63;
  const int s_row = min((tid >> 6) * 32 + (((s_l >> 3) & 1) | (s_l & 2) | ((s_l >> 2) & 4) |
                                           ((s_l << 1) & 8) | ((s_l >> 1) & 16)),
                        BR - 1);
  const int s_wd = s_l & 1;
  const uint32_t* s_wsrc = nullptr;
  const uint16_t* s_ssrc = nullptr;
  if constexpr (SIGN1) {
    const size_t wr = static_cast<size_t>(swiglu_b_row<COLS>(g, nt, s_row));
    s_wsrc = static_cast<const uint32_t*>(g.W) + wr * (g.K >> 5) + s_wd;
    s_ssrc = g.Wscale + wr * (g.K >> 7);
  }
  const int s_off = A_BYTES + s_row * ROWB;
  const int s_sw = swz16(s_row);

  auto issue = [&](int kt) __attribute__((always_inline)) {
    const int k0 = kt * BK;
    char* st = smem + (kt & 1) * STAGE;
#pragma unroll
    for (int j = 0; j < A_PW; ++j) dma16(a_src[j] + k0, st + (wave * A_PW + j) * 1024);
    if constexpr (!SIGN1) {
      if (has_b) {
#pragma unroll
        for (int j = 0; j < B_PW; ++j)
          dma16(b_src[j] + k0, st + A_BYTES + (wave * B_PW + j) * 1024);
      }
    }
  };
  auto load_s = [&](int kt, uint32_t& word, uint32_t& scale) __attribute__((always_inline)) {
    const int k0 = kt * BK;
    word = s_wsrc[k0 >> 5];
    scale = s_ssrc[k0 >> 7];
  };
  // expand this thread's word of tile kt into its stage: columns 32*s_wd ..
  // +32 of row s_row are the four 16-byte chunks 4*s_wd + q
  auto store_s = [&](int kt, uint32_t word, uint32_t scale) __attribute__((always_inline)) {
    char* st = smem + (kt & 1) * STAGE + s_off;
    const uint32_t sbf = f32_to_bf16(f16_to_f32(static_cast<uint16_t>(scale)));
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(st + (((4 * s_wd + q) ^ s_sw) << 4)) =
          sign1_expand8((word >> (8 * q)) & 0xffu, sbf);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment rows are 16-aligned, so every row this lane reads has swz16(l16)
  const int sw = swz16(l16);
  const int a_off = (wm * 64 + l16) * ROWB, b_off = A_BYTES + (wn * COLS + l16) * ROWB;
  const int ch0 = ((0 * 4 + lq) ^ sw) << 4, ch1 = ((1 * 4 + lq) ^ sw) << 4;
  bf16x8_t af0[FM], bf0[FN], af1[FM], bf1[FN];
#define TLP_FRAGS16(AF, BF, ST, C)                                                           \
  _Pragma("unroll") for (int i = 0; i < FM; ++i) AF[i] =                                     \
      *reinterpret_cast<const bf16x8_t*>((ST) + a_off + i * 16 * ROWB + (C));                \
  _Pragma("unroll") for (int j = 0; j < FN; ++j) BF[j] =                                     \
      *reinterpret_cast<const bf16x8_t*>((ST) + b_off + j * 16 * ROWB + (C));
#define TLP_MMA16(AF, BF)                                                                    \
  _Pragma("unroll") for (int i = 0; i < FM; ++i)                                             \
  _Pragma("unroll") for (int j = 0; j < FN; ++j)                                             \
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(AF[i], BF[j], acc[i][j], 0, 0, 0);

  // per 64-wide tile: two 32-wide k-steps; fragments of step 1 are read
  // during the MFMAs of step 0, and the barrier + refill of the stage sit
  // between the two MFMA groups
  const int nk = g.K / BK;
  uint32_t s_word = 0, s_scale = 0;   // 1-bit: tile kt+2's item, in flight during tile kt
  if constexpr (SIGN1) {
    // tiles 0 and 1 are expanded before the first barrier
    uint32_t w0 = 0, c0 = 0, w1 = 0, c1 = 0;
    issue(0);
    if (s_own) load_s(0, w0, c0);
    if (nk > 1) {
      issue(1);
      if (s_own) load_s(1, w1, c1);
    }
    __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);
    if (s_own) {
      store_s(0, w0, c0);
      if (nk > 1) store_s(1, w1, c1);
      if (nk > 2) load_s(2, s_word, s_scale);
    }
  } else {
    issue(0);
    if (nk > 1) issue(1);
    if (nk > 1) {
      if (has_b) __builtin_amdgcn_s_waitcnt(VmWait<A_PW + B_PW>::imm);
      else __builtin_amdgcn_s_waitcnt(VmWait<A_PW>::imm);
    } else {
      __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);
    }
  }
  lds_barrier();
  TLP_FRAGS16(af0, bf0, smem, ch0)
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only

  int kt = 0;
  for (; kt + 1 < nk; ++kt) {
    const char* st = smem + (kt & 1) * STAGE;
    TLP_FRAGS16(af1, bf1, st, ch1)
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA16(af0, bf0)
    __builtin_amdgcn_sched_barrier(0);
    // tile kt+1 (its copy, and for 1-bit the item of tile kt+2) has landed
    __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);
    lds_barrier();
    // every read of tile kt is done: its stage takes tile kt+2
    if (kt + 2 < nk) issue(kt + 2);
    const char* st1 = smem + ((kt + 1) & 1) * STAGE;
    TLP_FRAGS16(af0, bf0, st1, ch0)
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA16(af1, bf1)
    __builtin_amdgcn_sched_barrier(0);
    // 1-bit: tile kt+2's weights into that stage, after this step's MFMAs
    // are issued (the next iteration's barrier publishes them)
    if constexpr (SIGN1) {
      if (s_own && kt + 2 < nk) {
        store_s(kt + 2, s_word, s_scale);
        if (kt + 3 < nk) load_s(kt + 3, s_word, s_scale);
      }
    }
  }
  {
    const char* st = smem + (kt & 1) * STAGE;
    TLP_FRAGS16(af1, bf1, st, ch1)
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA16(af0, bf0)
    TLP_MMA16(af1, bf1)
  }
#undef TLP_FRAGS16
#undef TLP_MMA16

  // epilogue: lane l holds column l16 of each fragment and rows 4*lq + r;
  // columns 0-7 are gate, 8-15 the up values of the same output columns.
  // Both halves of each 16-lane row finish outputs (each SiLU is evaluated
  // once, by the lane that stores it).
  uint16_t* out = static_cast<uint16_t*>(g.out);
  const bool lo = l16 < 8;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        // rows 2q and 2q+1 of the lane's four: the low half of each 16-lane
        // row finishes row 2q (its gate, the up value from eight lanes on),
        // the high half row 2q+1 (its up value, the gate from eight lanes
        // back); one rotate by eight brings each the missing value
        const float a0 = acc[i][j][2 * q], a1 = acc[i][j][2 * q + 1];
        const float send = lo ? a1 : a0;
        const float got = __builtin_bit_cast(
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), 0x128, 0xf, 0xf, false));
        const float gate = lo ? a0 : got, up = lo ? got : a1;
        const int m = m0 + wm * 64 + i * 16 + 4 * lq + 2 * q + (lo ? 0 : 1);
        const int idx = nt * COLS + wn * (COLS / 2) + 8 * j + (l16 & 7);
        if (m < g.M && idx < g.N)
          out[static_cast<size_t>(m) * g.ldo + idx] = f32_to_bf16(silu_f32(gate) * up);
      }
}

// ---- gate/up + SwiGLU, two wavefront groups half a tile apart (dense) --------
// The block, wavefront tiles, LDS swizzle and SwiGLU epilogue are those of
// gemm_swiglu_kernel (COLS output columns: 112 or 96).  What differs is
// when the copies are issued and how far ahead.  A copy instruction holds up
// the wavefront that issues it until the CU's load path accepts it (about 16
// cycles per KB), so copies issued in a burst before a run of MFMAs stall
// those MFMAs.  Here the eight wavefronts form two groups, waves 0-3 (token
// rows 0-127) and 4-7 (rows 128-255), one wavefront of each per SIMD, that run
// half a K tile apart; each phase ends in a workgroup barrier:
//   phase 2kt    group 0 copies the activation tile of tile kt+1 into the
//                stage freed by phase 2kt-1, then reads its fragments of tile
//                kt from LDS; group 1 runs the MFMAs of tile kt-1 with the
//                weight tile of tile kt+2 copied between them (one copy
//                instruction every four MFMAs of the second k-step) into the
//                ring stage of tile kt-1;
//   phase 2kt+1  group 0 runs the MFMAs of tile kt; group 1 reads tile kt.
// So the MFMA pipe of each SIMD is fed by one group while the other reads.
// The activation tiles (read from L2) sit in two stages; the weight tiles,
// streamed from HBM, in a ring of three, so each weight copy has two tiles
// of time to land.  Every wavefront waits for its copies of tile kt+1 before
// the barrier that ends phase 2kt+1.  Copies past the last tile re-copy the
// last tile into a stage nobody reads any more (a branch around them would
// split the scheduled MFMA block); all copies are waited for before the
// epilogue.
template <int N> struct IntC { static constexpr int value = N; };

template <int COLS>
__global__ __launch_bounds__(512) void gemm_swiglu_pp_kernel(GemmArgs g) {
  constexpr int BM = 256, BR = 2 * COLS, BK = 64, ROWB = 128;
  constexpr int FM = 4, FN = COLS / 16;
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BR * ROWB;
  constexpr int A_PW = A_BYTES / 1024 / 4;
  constexpr int B_PW = B_BYTES / 1024 / 4;
  constexpr int B_BASE = 2 * A_BYTES;   // weight ring of three stages after the two activation stages
  static_assert(COLS % 16 == 0 && B_BYTES % 4096 == 0 && 4 * B_PW <= FM * FN, "tile shape");
  typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
  __shared__ __attribute__((aligned(1024))) char smem[2 * A_BYTES + 3 * B_BYTES];

  const int wi = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = wi % g.m_tiles, nt = wi / g.m_tiles;
  const int m0 = mt * BM;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, cw = wave & 3;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, lq = lane >> 4;
  const int nk = g.K / BK;

  const int drow = lane >> 3, dslot = lane & 7;
  constexpr int C_PW = A_PW > B_PW ? A_PW : B_PW;
  uint32_t c_src[C_PW];
#pragma unroll
  for (int j = 0; j < C_PW; ++j) {
    if (grp == 0) {
      const int row = (cw * A_PW + j) * 8 + drow;
      c_src[j] = (static_cast<uint32_t>(min(m0 + row, g.M - 1)) * g.lda + (dslot ^ swz16(row)) * 8) * 2;
    } else {
      const int rr = min((cw * B_PW + j) * 8 + drow, BR - 1);
      c_src[j] = (static_cast<uint32_t>(swiglu_b_row<COLS>(g, nt, rr)) * g.K + (dslot ^ swz16(rr)) * 8) * 2;
    }
  }
  const i32x4_t c_rsrc = grp == 0 ? buffer_rsrc(g.A, g.a_bytes) : buffer_rsrc(g.W, g.w_bytes);
  auto kbyte = [&](int kt) { return __builtin_amdgcn_readfirstlane(kt * BK * 2); };
  // group 0: activation tile kt into stage kt & 1; group 1: weight tile kt into ring slot kt % 3
  auto a_copy = [&](int kt, int j) __attribute__((always_inline)) {
    dma16_buf(c_rsrc, c_src[j], kbyte(kt), smem + (kt & 1) * A_BYTES + (cw * A_PW + j) * 1024);
  };
  auto b_copy = [&](int kt, int slot, int j) __attribute__((always_inline)) {
    dma16_buf(c_rsrc, c_src[j], kbyte(kt), smem + B_BASE + slot * B_BYTES + (cw * B_PW + j) * 1024);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int sw = swz16(l16);
  const int a_off = (wm * 64 + l16) * ROWB, b_off = (wn * COLS + l16) * ROWB;
  const int ch0 = ((0 * 4 + lq) ^ sw) << 4, ch1 = ((1 * 4 + lq) ^ sw) << 4;
  bf16x8_t af[2][FM], bf[2][FN];
  auto read_frags = [&](const char* ast, const char* bst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      af[0][i] = *reinterpret_cast<const bf16x8_t*>(ast + a_off + i * 16 * ROWB + ch0);
      af[1][i] = *reinterpret_cast<const bf16x8_t*>(ast + a_off + i * 16 * ROWB + ch1);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      bf[0][j] = *reinterpret_cast<const bf16x8_t*>(bst + b_off + j * 16 * ROWB + ch0);
      bf[1][j] = *reinterpret_cast<const bf16x8_t*>(bst + b_off + j * 16 * ROWB + ch1);
    }
  };
  auto mfma_step = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks][i], bf[ks][j], acc[i][j], 0, 0, 0);
  };
  auto mfma_copy = [&](int ktc, int slot) __attribute__((always_inline)) {
    mfma_step(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < B_PW; ++j) b_copy(ktc, slot, j);
    mfma_step(1);
#pragma unroll
    for (int j = 0; j < B_PW; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - 4 * B_PW, 0);
  };
  auto bar = []() __attribute__((always_inline)) { asm volatile("s_barrier" ::: "memory"); };

  // prologue: activation tiles 0-1 and weight tiles 0-2 in flight (clamped to
  // the last tile); wait for tile 0
  if (grp == 0) {
#pragma unroll
    for (int j = 0; j < A_PW; ++j) a_copy(0, j);
#pragma unroll
    for (int j = 0; j < A_PW; ++j) a_copy(min(1, nk - 1), j);
    __builtin_amdgcn_s_waitcnt(VmWait<A_PW>::imm);
  } else {
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
      for (int j = 0; j < B_PW; ++j) b_copy(min(s, nk - 1), s, j);
    __builtin_amdgcn_s_waitcnt(VmWait<2 * B_PW>::imm);
  }
  lds_barrier();

  if (grp == 0) {
    int slot = 0;
    auto step = [&](int kt, auto par) __attribute__((always_inline)) {
      constexpr int P = decltype(par)::value;
      if (kt >= 1 && kt + 1 < nk) {
#pragma unroll
        for (int j = 0; j < A_PW; ++j) a_copy(kt + 1, j);
      }
      read_frags(smem + P * A_BYTES, smem + B_BASE + slot * B_BYTES);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      mfma_step(0);
      mfma_step(1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);   // this wavefront's copies of tile kt+1
      bar();
      __builtin_amdgcn_sched_barrier(0);
      slot = slot == 2 ? 0 : slot + 1;
    };
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      step(kt, IntC<0>{});
      step(kt + 1, IntC<1>{});
    }
    if (kt < nk) step(kt, IntC<0>{});
  } else {
    lds_barrier();
    int slot = 0;
    auto step = [&](int kt, auto par) __attribute__((always_inline)) {
      constexpr int P = decltype(par)::value;
      read_frags(smem + P * A_BYTES, smem + B_BASE + slot * B_BYTES);
      // this wavefront's weight copies of tile kt+1 (those of tile kt+2 may stay in flight)
      __builtin_amdgcn_s_waitcnt(VmWait<B_PW>::imm);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // tile kt's ring slot is free: weights of tile kt+3 go there
      mfma_copy(min(kt + 3, nk - 1), slot);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < nk) bar();
      __builtin_amdgcn_sched_barrier(0);
      slot = slot == 2 ? 0 : slot + 1;
    };
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      step(kt, IntC<0>{});
      step(kt + 1, IntC<1>{});
    }
    if (kt < nk) step(kt, IntC<0>{});
  }
  __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);   // no copy may land after the block ends

  uint16_t* out = static_cast<uint16_t*>(g.out);
  const bool lo = l16 < 8;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float a0 = acc[i][j][2 * q], a1 = acc[i][j][2 * q + 1];
        const float send = lo ? a1 : a0;
        const float got = __builtin_bit_cast(
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, send), 0x128, 0xf, 0xf, false));
        const float gate = lo ? a0 : got, up = lo ? got : a1;
        const int m = m0 + wm * 64 + i * 16 + 4 * lq + 2 * q + (lo ? 0 : 1);
        const int idx = nt * COLS + wn * (COLS / 2) + 8 * j + (l16 & 7);
        if (m < g.M && idx < g.N)
          out[static_cast<size_t>(m) * g.ldo + idx] = f32_to_bf16(silu_f32(gate) * up);
      }
}

// ---- dense projections, two wavefront groups half a tile apart ---------------
// For 128- and 192-wide weight tiles (a 256-wide tile's accumulators and
// fragments of a whole K tile do not fit in the registers of two wavefronts
// per SIMD).  The tiles (256 token rows x BN weight rows, 64-wide K tiles, eight
// wavefronts of 32x32x16 MFMAs), swizzle, K slices and epilogues of
// gemm_bf16_dma_kernel with the copy schedule of gemm_swiglu_pp_kernel:
// waves 0-3 (token rows 0-127) copy activation tiles at the start of their
// read phases, waves 4-7 (rows 128-255) copy weight tiles between the MFMAs of
// the second half of their tile.  The activation and weight tiles sit in rings
// of SA and SB stages (two or three each, as the LDS allows): activation tile
// kt+SA-1 goes into the stage of tile kt-1 when group 0 starts tile kt,
// weight tile kt+SB into the stage of tile kt once group 1 has read it, so a
// copy has up to two tiles of time to land before it is read.  Past the last
// tile the copies repeat the last tile into a stage nobody reads any more (a
// branch around them would split the scheduled MFMA block); each group waits
// for its copies of tile kt+1 before the barrier that ends tile kt, and for
// all of them before the epilogue.
template <int BN, int WM, int WN, int EPI, bool OUT_F32, int SA = 2, int SB = 2>
__global__ __launch_bounds__(WM* WN * 64) void gemm_pp_dma_kernel(GemmArgs g) {
  constexpr int BM = 256, BK = 64, ROWB = BK * 2;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  constexpr int B_BASE = SA * A_BYTES;
  constexpr int A_PW = A_BYTES / 1024 / 4, B_PW = B_BYTES / 1024 / 4;
  constexpr int HALF = 2 * FM * FN;
  static_assert(WM * WN == 8 && TM * 2 * (WM / 2) == BM, "waves 0-3 cover token rows 0-127");
  static_assert(B_BYTES % 4096 == 0 && B_PW <= HALF, "copy split");
  static_assert(SA >= 2 && SA <= 3 && SB >= 2 && SB <= 3, "ring depth");
  static_assert(EPI != 2 || FN % 2 == 0, "SwiGLU pairs gate and up fragments");
  __shared__ __attribute__((aligned(1024))) char smem[SA * A_BYTES + SB * B_BYTES];

  const int wi = xcd_tile(blockIdx.x, gridDim.x);
  const int split = wi % g.splits, t = wi / g.splits;
  const int mt = t % g.m_tiles, nt = t / g.m_tiles;
  const int m0 = mt * BM;
  const int k_begin = split * g.k_split;
  const int k_end = min(g.K, k_begin + g.k_split);
  const int nk = (k_end - k_begin) / BK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, cw = wave & 3;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lh = lane >> 5;
  auto b_row = [&](int r) -> int {
    if constexpr (EPI == 2) {
      const int w = r / TN, rr = r % TN;
      const int jj = min(nt * (BN / 2) + w * (TN / 2) + rr % (TN / 2), g.N - 1);
      return rr >= TN / 2 ? g.up_row + jj : jj;
    } else {
      return min(nt * BN + r, g.N - 1);
    }
  };

  const int drow = lane >> 3, dslot = lane & 7;
  constexpr int C_PW = A_PW > B_PW ? A_PW : B_PW;
  uint32_t c_src[C_PW];
#pragma unroll
  for (int j = 0; j < C_PW; ++j) {
    if (grp == 0) {
      const int row = (cw * A_PW + j) * 8 + drow;
      c_src[j] = (static_cast<uint32_t>(min(m0 + row, g.M - 1)) * g.lda + (dslot ^ swz8(row)) * 8) * 2;
    } else {
      const int row = min((cw * B_PW + j) * 8 + drow, BN - 1);
      c_src[j] = (static_cast<uint32_t>(b_row(row)) * g.K + (dslot ^ swz8(row)) * 8) * 2;
    }
  }
  const i32x4_t c_rsrc = grp == 0 ? buffer_rsrc(g.A, g.a_bytes) : buffer_rsrc(g.W, g.w_bytes);
  auto kbyte = [&](int kt) { return __builtin_amdgcn_readfirstlane((k_begin + min(kt, nk - 1) * BK) * 2); };
  auto a_copy = [&](int kt, int slot, int j) __attribute__((always_inline)) {
    dma16_buf(c_rsrc, c_src[j], kbyte(kt), smem + slot * A_BYTES + (cw * A_PW + j) * 1024);
  };
  auto b_copy = [&](int kt, int slot, int j) __attribute__((always_inline)) {
    dma16_buf(c_rsrc, c_src[j], kbyte(kt), smem + B_BASE + slot * B_BYTES + (cw * B_PW + j) * 1024);
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int sw = swz8(lr);
  const int a_off = (wm * TM + lr) * ROWB, b_off = (wn * TN + lr) * ROWB;
  bf16x8_t af[4][FM], bf[4][FN];
  auto read_frags = [&](const char* ast, const char* bst) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = ((kk * 2 + lh) ^ sw) << 4;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[kk][i] = *reinterpret_cast<const bf16x8_t*>(ast + a_off + i * 32 * ROWB + ch);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bf[kk][j] = *reinterpret_cast<const bf16x8_t*>(bst + b_off + j * 32 * ROWB + ch);
    }
  };
  auto mfma_steps = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = k0; kk < k0 + 2; ++kk)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk][i], bf[kk][j], acc[i][j], 0, 0, 0);
  };
  auto mfma_copy = [&](int ktc, int slot) __attribute__((always_inline)) {
    mfma_steps(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < B_PW; ++j) b_copy(ktc, slot, j);
    mfma_steps(2);
    constexpr int EVERY = HALF / B_PW;
#pragma unroll
    for (int j = 0; j < B_PW; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, EVERY, 0);
    }
    if constexpr (HALF - EVERY * B_PW > 0)
      __builtin_amdgcn_sched_group_barrier(0x008, HALF - EVERY * B_PW, 0);
  };
  auto bar = []() __attribute__((always_inline)) { asm volatile("s_barrier" ::: "memory"); };

  // prologue: activation tiles 0 .. SA-2 and weight tiles 0 .. SB-1 in flight
  // (clamped to the last tile); wait for tile 0
  if (grp == 0) {
#pragma unroll
    for (int s = 0; s < SA - 1; ++s)
#pragma unroll
      for (int j = 0; j < A_PW; ++j) a_copy(s, s, j);
    __builtin_amdgcn_s_waitcnt(VmWait<(SA - 2) * A_PW>::imm);
  } else {
#pragma unroll
    for (int s = 0; s < SB; ++s)
#pragma unroll
      for (int j = 0; j < B_PW; ++j) b_copy(s, s, j);
    __builtin_amdgcn_s_waitcnt(VmWait<(SB - 1) * B_PW>::imm);
  }
  lds_barrier();

  int sa = 0, sb = 0;   // ring stages of tile kt
  if (grp == 0) {
    for (int kt = 0; kt < nk; ++kt) {
      // activations of tile kt+SA-1 into the stage of tile kt-1
      const int fa = sa == 0 ? SA - 1 : sa - 1;
#pragma unroll
      for (int j = 0; j < A_PW; ++j) a_copy(kt + SA - 1, fa, j);
      read_frags(smem + sa * A_BYTES, smem + B_BASE + sb * B_BYTES);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      mfma_steps(0);
      mfma_steps(2);
      __builtin_amdgcn_sched_barrier(0);
      // this wavefront's copies of tile kt+1
      __builtin_amdgcn_s_waitcnt(VmWait<(SA - 2) * A_PW>::imm);
      bar();
      __builtin_amdgcn_sched_barrier(0);
      sa = sa == SA - 1 ? 0 : sa + 1;
      sb = sb == SB - 1 ? 0 : sb + 1;
    }
  } else {
    lds_barrier();
    for (int kt = 0; kt < nk; ++kt) {
      read_frags(smem + sa * A_BYTES, smem + B_BASE + sb * B_BYTES);
      // this wavefront's weight copies of tile kt+1
      __builtin_amdgcn_s_waitcnt(VmWait<(SB - 2) * B_PW>::imm);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // tile kt's weight stage is free: weights of tile kt+SB go there
      mfma_copy(kt + SB, sb);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < nk) bar();
      __builtin_amdgcn_sched_barrier(0);
      sa = sa == SA - 1 ? 0 : sa + 1;
      sb = sb == SB - 1 ? 0 : sb + 1;
    }
  }
  __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);   // no copy may land after the block ends

  gemm_epilogue<FM, FN, TM, TN, BN, EPI, OUT_F32>(g, acc, m0, nt, wm, wn, lr, lh, split);
}

// ---- dense 256x256 projections: each wavefront's copies spread over its MFMAs --
// The tiles, swizzle, K slices, fragment double-buffering and epilogues of
// gemm_bf16_dma_kernel at BM = BN = 256, where a whole K tile of fragments does
// not fit beside the accumulators and the two-group schedule of
// gemm_pp_dma_kernel is not possible.  Instead of issuing its share of the
// next-but-one tile's copies in one burst after the barrier (a copy
// instruction holds its wavefront until the load path accepts it, so a burst
// stalls the MFMAs behind it), every wavefront issues them one at a time
// between the MFMAs of the k-step that follows the barrier.  Copies use
// buffer-resource loads: wavefront w copies activation blocks A_PW*w .. and
// weight blocks B_PW*w .. (1 KB = 8 rows of 128 bytes; lane l fetches chunk
// (l & 7) ^ swz8(row) of row l >> 3).  Past the last tile the copies repeat
// the last tile into the stage nobody reads any more (a branch around them
// would split the scheduled MFMA group); all copies are waited for before the
// epilogue.
template <int BN, int WM, int WN, int EPI, bool OUT_F32>
__global__ __launch_bounds__(WM* WN * 64) void gemm_dma_spread_kernel(GemmArgs g) {
  constexpr int BM = 256, BK = 64, ROWB = 128, NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_PW = A_BYTES / 1024 / NW, B_PW = B_BYTES / 1024 / NW;   // copies per wavefront
  constexpr int CPW = A_PW + B_PW;
  static_assert(A_PW * NW * 1024 == A_BYTES && B_PW * NW * 1024 == B_BYTES, "copy split");
  static_assert((FM * FN) % CPW == 0, "copies spread evenly over a k-step's MFMAs");
  static_assert(EPI != 2 || FN % 2 == 0, "SwiGLU pairs gate and up fragments");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int wi = xcd_tile(blockIdx.x, gridDim.x);
  const int split = wi % g.splits, t = wi / g.splits;
  const int mt = t % g.m_tiles, nt = t / g.m_tiles;
  const int m0 = mt * BM;
  const int k_begin = split * g.k_split;
  const int k_end = min(g.K, k_begin + g.k_split);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lh = lane >> 5;
  // weight row of B-tile row r (SwiGLU: each wavefront column holds TN/2 gate
  // rows then the TN/2 up rows of the same output columns); rows past N are
  // clamped, their products land in discarded outputs
  auto b_row = [&](int r) -> int {
    if constexpr (EPI == 2) {
      const int w = r / TN, rr = r % TN;
      const int jj = min(nt * (BN / 2) + w * (TN / 2) + rr % (TN / 2), g.N - 1);
      return rr >= TN / 2 ? g.up_row + jj : jj;
    } else {
      return min(nt * BN + r, g.N - 1);
    }
  };
  const int drow = lane >> 3, dslot = lane & 7;
  uint32_t c_src[CPW];   // copy j < A_PW is an activation copy
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    if (j < A_PW) {
      const int row = (A_PW * wave + j) * 8 + drow;
      c_src[j] = (static_cast<uint32_t>(min(m0 + row, g.M - 1)) * g.lda + (dslot ^ swz8(row)) * 8) * 2;
    } else {
      const int row = (B_PW * wave + j - A_PW) * 8 + drow;
      c_src[j] = (static_cast<uint32_t>(b_row(row)) * g.K + (dslot ^ swz8(row)) * 8) * 2;
    }
  }
  const i32x4_t a_rsrc = buffer_rsrc(g.A, g.a_bytes);
  const i32x4_t b_rsrc = buffer_rsrc(g.W, g.w_bytes);
  auto kbyte = [&](int kt) { return __builtin_amdgcn_readfirstlane((k_begin + kt * BK) * 2); };
  auto copy = [&](int kt, int j) __attribute__((always_inline)) {
    char* st = smem + (kt & 1) * STAGE;
    if (j < A_PW) dma16_buf(a_rsrc, c_src[j], kbyte(kt), st + (A_PW * wave + j) * 1024);
    else dma16_buf(b_rsrc, c_src[j], kbyte(kt), st + A_BYTES + (B_PW * wave + j - A_PW) * 1024);
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // fragment rows are 32-aligned, so swz8(row) = swz8(lr)
  const int sw = swz8(lr);
  const int a_off = (wm * TM + lr) * ROWB, b_off = A_BYTES + (wn * TN + lr) * ROWB;
  int ch[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) ch[kk] = ((kk * 2 + lh) ^ sw) << 4;
  bf16x8_t af0[FM], bf0[FN], af1[FM], bf1[FN];
#define TLP_FRAGS(AF, BF, ST, C)                                                             \
  _Pragma("unroll") for (int i = 0; i < FM; ++i) AF[i] =                                     \
      *reinterpret_cast<const bf16x8_t*>((ST) + a_off + i * 32 * ROWB + (C));                \
  _Pragma("unroll") for (int j = 0; j < FN; ++j) BF[j] =                                     \
      *reinterpret_cast<const bf16x8_t*>((ST) + b_off + j * 32 * ROWB + (C));
#define TLP_MMA(AF, BF)                                                                      \
  _Pragma("unroll") for (int i = 0; i < FM; ++i)                                             \
  _Pragma("unroll") for (int j = 0; j < FN; ++j)                                             \
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AF[i], BF[j], acc[i][j], 0, 0, 0);

  const int nk = (k_end - k_begin) / BK;
#pragma unroll
  for (int j = 0; j < CPW; ++j) copy(0, j);
  if (nk > 1) {
#pragma unroll
    for (int j = 0; j < CPW; ++j) copy(1, j);
    __builtin_amdgcn_s_waitcnt(VmWait<CPW>::imm);
  } else {
    __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);
  }
  lds_barrier();
  TLP_FRAGS(af0, bf0, smem, ch[0])
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only

  // per 64-wide tile kt: four 16-wide k-steps, fragments of step s+1 read
  // during the MFMAs of step s; after step 2's MFMAs wait for tile kt+1,
  // barrier (every wavefront has read all of tile kt), then step 3's MFMAs
  // with the copies of tile kt+2 into tile kt's stage between them
  int kt = 0;
  for (; kt + 1 < nk; ++kt) {
    const char* st = smem + (kt & 1) * STAGE;
    TLP_FRAGS(af1, bf1, st, ch[1])
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA(af0, bf0)
    __builtin_amdgcn_sched_barrier(0);
    TLP_FRAGS(af0, bf0, st, ch[2])
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA(af1, bf1)
    __builtin_amdgcn_sched_barrier(0);
    TLP_FRAGS(af1, bf1, st, ch[3])
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA(af0, bf0)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);   // this wavefront's copies of tile kt+1
    lds_barrier();
    const char* st1 = smem + ((kt + 1) & 1) * STAGE;
    TLP_FRAGS(af0, bf0, st1, ch[0])
#pragma unroll
    for (int j = 0; j < CPW; ++j) copy(min(kt + 2, nk - 1), j);
    TLP_MMA(af1, bf1)
    // masks: 0x100 LDS read, 0x8 MFMA, 0x20 vector memory read
    __builtin_amdgcn_sched_group_barrier(0x100, FM + FN, 0);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, (FM * FN) / CPW, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  {
    const char* st = smem + (kt & 1) * STAGE;
    TLP_FRAGS(af1, bf1, st, ch[1])
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA(af0, bf0)
    TLP_FRAGS(af0, bf0, st, ch[2])
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA(af1, bf1)
    TLP_FRAGS(af1, bf1, st, ch[3])
    __builtin_amdgcn_sched_barrier(0);
    TLP_MMA(af0, bf0)
    TLP_MMA(af1, bf1)
  }
#undef TLP_FRAGS
#undef TLP_MMA
  __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);   // no copy may land after the block ends
  gemm_epilogue<FM, FN, TM, TN, BN, EPI, OUT_F32>(g, acc, m0, nt, wm, wn, lr, lh, split);
}

// ---- projections of few token rows: 128-row tiles over the whole of K -------
// For a bf16 product whose 128-row tiles fill the CUs without splitting K
// (the QKV projection of a 512-token micro-batch: 4 x 64 tiles of 128x96).
// A block owns 128 token rows x BN weight rows over all of K, so it writes
// finished bf16 rows and no fp32 partial slices go through memory (the row
// pass that follows reads 2 bytes per element instead of the 4 x 4 of four
// slices).  Such a tile needs more operand bytes per flop than the big tiles,
// so the kernel is built to stream them: NS stages of 64-wide K tiles in a
// ring, refilled by global->LDS buffer copies NS tiles ahead, and the four
// wavefronts (4x1 or 2x2 of 32x32x16 MFMA fragments) read a whole tile's
// fragments into registers while the MFMAs of the previous tile run.
// Scheduling pattern: copy j (of C) follows MFMAs ((j+1)*N)/C - (j*N)/C of a
// run of N (masks: 0x8 MFMA, 0x20 vector memory read).
template <int J, int N, int C>
struct SpreadCopies {
  static __device__ __forceinline__ void place() {
    constexpr int m = ((J + 1) * N) / C - (J * N) / C;
    if constexpr (m > 0) __builtin_amdgcn_sched_group_barrier(0x008, m, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    SpreadCopies<J + 1, N, C>::place();
  }
};
template <int N, int C>
struct SpreadCopies<C, N, C> {
  static __device__ __forceinline__ void place() {}
};

template <int BN, int WM, int WN, int EPI, bool OUT_F32, int NS>
__global__ __launch_bounds__(256) void gemm_stream_kernel(GemmArgs g) {
  constexpr int BM = 128, BK = 64, ROWB = 128;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int A_PW = A_BYTES / 1024 / 4, B_PW = B_BYTES / 1024 / 4;
  constexpr int CPW = A_PW + B_PW;
  static_assert(WM * WN == 4 && FM * 32 == TM && FN * 32 == TN, "four wavefronts of 32x32 fragments");
  static_assert(A_PW * 4096 == A_BYTES && B_PW * 4096 == B_BYTES, "copy split");
  static_assert((NS - 2) * CPW <= 63 && NS >= 3, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];

  const int wi = xcd_tile(blockIdx.x, gridDim.x);
  const int mt = wi % g.m_tiles, nt = wi / g.m_tiles;
  const int m0 = mt * BM;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lh = lane >> 5;
  const int nk = g.K / BK;

  // copy j < A_PW: activation block A_PW*wave + j; else weight block
  // B_PW*wave + j - A_PW (1 KB = 8 rows of 128 bytes; lane l fetches chunk
  // (l & 7) ^ swz8(row) of row l >> 3; rows past M or N re-fetch the last one)
  const int drow = lane >> 3, dslot = lane & 7;
  uint32_t c_src[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    if (j < A_PW) {
      const int row = (A_PW * wave + j) * 8 + drow;
      c_src[j] = (static_cast<uint32_t>(min(m0 + row, g.M - 1)) * g.lda + (dslot ^ swz8(row)) * 8) * 2;
    } else {
      const int row = (B_PW * wave + j - A_PW) * 8 + drow;
      c_src[j] = (static_cast<uint32_t>(min(nt * BN + row, g.N - 1)) * g.K + (dslot ^ swz8(row)) * 8) * 2;
    }
  }
  const i32x4_t a_rsrc = buffer_rsrc(g.A, g.a_bytes);
  const i32x4_t b_rsrc = buffer_rsrc(g.W, g.w_bytes);
  // tile kt (clamped to the last one) into ring stage `slot`
  auto copy = [&](int kt, int slot, int j) __attribute__((always_inline)) {
    const int kb = __builtin_amdgcn_readfirstlane(min(kt, nk - 1) * BK * 2);
    char* st = smem + slot * STAGE;
    if (j < A_PW) dma16_buf(a_rsrc, c_src[j], kb, st + (A_PW * wave + j) * 1024);
    else dma16_buf(b_rsrc, c_src[j], kb, st + A_BYTES + (B_PW * wave + j - A_PW) * 1024);
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int sw = swz8(lr);
  const int a_off = (wm * TM + lr) * ROWB, b_off = A_BYTES + (wn * TN + lr) * ROWB;
  int ch[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) ch[kk] = ((kk * 2 + lh) ^ sw) << 4;
  // all four k-steps of a tile's fragments, double-buffered across tiles
  bf16x8_t ax[4][FM], bx[4][FN], ay[4][FM], by[4][FN];
  auto frags = [&](bf16x8_t (&AF)[4][FM], bf16x8_t (&BF)[4][FN], const char* st) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
        AF[kk][i] = *reinterpret_cast<const bf16x8_t*>(st + a_off + i * 32 * ROWB + ch[kk]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        BF[kk][j] = *reinterpret_cast<const bf16x8_t*>(st + b_off + j * 32 * ROWB + ch[kk]);
    }
  };
  auto mma = [&](bf16x8_t (&AF)[4][FM], bf16x8_t (&BF)[4][FN]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(AF[kk][i], BF[kk][j], acc[i][j], 0, 0, 0);
  };

  // prologue: tiles 0 .. NS-1 in flight; tiles 0 and 1 landed; everyone holds
  // tile 0 in registers before its stage is refilled
#pragma unroll
  for (int t = 0; t < NS; ++t)
#pragma unroll
    for (int j = 0; j < CPW; ++j) copy(t, t, j);
  __builtin_amdgcn_s_waitcnt(VmWait<(NS - 2) * CPW>::imm);
  lds_barrier();
  frags(ax, bx, smem);
  lds_barrier();

  // step kt: fragments of tile kt are in registers; read those of tile kt+1,
  // run tile kt's MFMAs with the copies of tile kt+NS into tile kt's stage
  // between them; wait for this wavefront's copies of tile kt+2, then the
  // barrier (all reads of tile kt+1 done, every copy of tile kt+2 landed)
  int slot = 0;   // ring stage of tile kt
  auto step = [&](int kt, bf16x8_t (&AC)[4][FM], bf16x8_t (&BC)[4][FN], bf16x8_t (&AN)[4][FM],
                  bf16x8_t (&BN_)[4][FN]) __attribute__((always_inline)) {
    const int next = slot == NS - 1 ? 0 : slot + 1;
    frags(AN, BN_, smem + next * STAGE);
#pragma unroll
    for (int j = 0; j < CPW; ++j) copy(kt + NS, slot, j);
    mma(AC, BC);
    // masks: 0x100 LDS read, 0x8 MFMA, 0x20 vector memory read
    __builtin_amdgcn_sched_group_barrier(0x100, 4 * (FM + FN), 0);
    SpreadCopies<0, 4 * FM * FN, CPW>::place();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(VmWait<(NS - 2) * CPW>::imm);
    lds_barrier();
    slot = next;
  };
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, ax, bx, ay, by);
    step(kt + 1, ay, by, ax, bx);
  }
  if (kt < nk) step(kt, ax, bx, ay, by);
  __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);   // no copy may land after the block ends

  gemm_epilogue<FM, FN, TM, TN, BN, EPI, OUT_F32>(g, acc, m0, nt, wm, wn, lr, lh, 0);
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

// Byte extents the buffer-copy kernels address (their descriptors hold 32-bit
// sizes); false when a matrix is 4 GiB or larger.
static bool buffer_extents(GemmArgs& g, size_t w_rows) {
  const size_t a = (static_cast<size_t>(g.M - 1) * g.lda + g.K) * 2;
  const size_t w = w_rows * static_cast<size_t>(g.K) * 2;
  if (a > 0xffffffffu || w > 0xffffffffu) return false;
  g.a_bytes = static_cast<uint32_t>(a);
  g.w_bytes = static_cast<uint32_t>(w);
  return true;
}

template <int BM, int BN, int WM, int WN, int EPI, bool SIGN1, bool OUT_F32>
static hipError_t run_bf16(GemmArgs g, int splits, hipStream_t s) {
  const int cols = EPI == 2 ? BN / 2 : BN;
  g.m_tiles = (g.M + BM - 1) / BM;
  g.n_tiles = (g.N + cols - 1) / cols;
  // the direct-to-LDS kernels need whole 64-wide K tiles (1-bit weights
  // always have them: K % 128 == 0)
  const bool dma = g.K % 64 == 0;
  const int kt_w = 64;
  const int k_tiles = (g.K + kt_w - 1) / kt_w;
  if (splits > k_tiles) splits = k_tiles;
  if (splits < 1) splits = 1;
  const int per = (k_tiles + splits - 1) / splits;   // K tiles per slice
  g.k_split = per * kt_w;
  g.splits = (k_tiles + per - 1) / per;
  const int blocks = g.m_tiles * g.n_tiles * g.splits;
  if (g.splits_out) *g.splits_out = g.splits;
  if (dma) {
    if constexpr (!SIGN1 && BM == 256 && BN == 256) {
      if (buffer_extents(g, EPI == 2 ? static_cast<size_t>(2) * g.N : static_cast<size_t>(g.N))) {
        gemm_dma_spread_kernel<BN, WM, WN, EPI, OUT_F32><<<blocks, WM * WN * 64, 0, s>>>(g);
        return hipGetLastError();
      }
    }
    gemm_bf16_dma_kernel<BM, BN, WM, WN, EPI, OUT_F32, SIGN1><<<blocks, WM * WN * 64, 0, s>>>(g);
    return hipGetLastError();
  }
  if constexpr (SIGN1) {
    return hipErrorInvalidValue;   // 1-bit weights always have K % 128 == 0
  } else {
    gemm_bf16_kernel<BM, BN, WM, WN, EPI, OUT_F32><<<blocks, WM * WN * 64, 0, s>>>(g);
    return hipGetLastError();
  }
}

// Tile shape per call.  Large weight matrices take 256x256 tiles; shapes with
// too few such tiles to fill the 256 CUs fall back to 128x128.  The Partial
// epilogue (output projection and down projection, summed later by the row
// pass that consumes the residual stream) splits K until the grid has about
// one work item per CU, at most 8 slices.
constexpr int kCUs = 256;
constexpr int kMaxSplits = 8;

static int big_tiles(int M, int N) { return ((M + 255) / 256) * ((N + 255) / 256); }

// Split-K plan of the Partial epilogue: tile width (256 or 128 columns, 256
// rows either way) and slice count, about one work item per CU.  The next row
// pass reads every slice once, so 256x128 tiles with half as many slices are
// used where that pays: the output and down projections at the 8B shape (4
// slices of 256x128 instead of 8 of 256x256).
struct PartialPlan {
  int bn, splits;
};
// (the narrow tiles exist for the direct-to-LDS kernel only: K % 64 == 0)
static PartialPlan partial_plan(int M, int N, int K, bool narrow_ok) {
  const int k_tiles = (K + 63) / 64;
  auto clamp = [&](int sp) { return sp < 1 ? 1 : (sp > k_tiles ? k_tiles : sp); };
  // 192-column tiles when they split N exactly into a grid that, with its
  // slices (one, if the tiles alone make a wave: 2048 tokens of the 8B QKV),
  // fills the CUs better than 256-column tiles
  if (narrow_ok && N % 192 == 0) {
    const int t192 = ((M + 255) / 256) * (N / 192);
    const int sp192 = kCUs / t192;
    const int sp256 = kCUs / big_tiles(M, N);
    if (sp192 >= 1 && t192 * sp192 > big_tiles(M, N) * sp256)
      return {192, clamp(sp192 > kMaxSplits ? kMaxSplits : sp192)};
  }
  const int narrow = ((M + 255) / 256) * ((N + 127) / 128);
  int splits = kCUs / narrow;
  // (measured: with fewer than 4 slices the narrow grid under-fills the GPU;
  // at K = 14336 of the 8B down projection 4 slices of 256x128 tiles beat 8
  // of 256x256 by the slices the next row pass no longer reads)
  if (narrow_ok && splits >= 4)
    return {128, clamp(splits > kMaxSplits ? kMaxSplits : splits)};
  splits = kCUs / big_tiles(M, N);   // the grid stays within one wave of work items
  if (splits > kMaxSplits) splits = kMaxSplits;
  return {256, clamp(splits)};
}

// the slice count run_bf16 ends up with (whole 64-wide K tiles per slice)
static int slices_of(int K, int splits) {
  const int k_tiles = (K + 63) / 64;
  const int per = (k_tiles + splits - 1) / splits;
  return (k_tiles + per - 1) / per;
}

int gemm_partial_splits(int M, int N, int K) {
  // an upper bound over both plans (workspace sizing)
  const int a = slices_of(K, partial_plan(M, N, K, true).splits);
  const int b = slices_of(K, partial_plan(M, N, K, false).splits);
  return a > b ? a : b;
}

// Partial epilogue with 256x128 or 256x192 tiles: the direct-to-LDS kernel only.
template <int BN, bool OUT_F32, bool SIGN1>
static hipError_t run_partial_narrow(GemmArgs g, int splits, hipStream_t s) {
  g.m_tiles = (g.M + 255) / 256;
  g.n_tiles = (g.N + BN - 1) / BN;
  const int k_tiles = g.K / 64;
  if (splits > k_tiles) splits = k_tiles;
  const int per = (k_tiles + splits - 1) / splits;
  g.k_split = per * 64;
  g.splits = (k_tiles + per - 1) / per;
  if (g.splits_out) *g.splits_out = g.splits;
  const int blocks = g.m_tiles * g.n_tiles * g.splits;
  if constexpr (!SIGN1) {
    if (buffer_extents(g, static_cast<size_t>(g.N))) {
      // (rings measured at the 8B shape: a third weight stage helps both
      // widths; a third activation stage fits, and helps, only beside 128)
      if constexpr (BN == 192)
        gemm_pp_dma_kernel<192, 4, 2, 4, OUT_F32, 2, 3><<<blocks, 512, 0, s>>>(g);
      else
        gemm_pp_dma_kernel<128, 4, 2, 4, OUT_F32, 3, 3><<<blocks, 512, 0, s>>>(g);
      return hipGetLastError();
    }
  }
  if constexpr (BN == 192)   // 4 x 2 wavefronts of 64 x 96
    gemm_bf16_dma_kernel<256, 192, 4, 2, 4, OUT_F32, SIGN1><<<blocks, 512, 0, s>>>(g);
  else
    gemm_bf16_dma_kernel<256, 128, 2, 4, 4, OUT_F32, SIGN1><<<blocks, 512, 0, s>>>(g);
  return hipGetLastError();
}

// SwiGLU with K % 64 == 0 (always so for 1-bit weights): output columns per
// block, 128 (256x256 tiles), 112 or 96, whichever needs the fewest waves of
// 256 blocks times the work per block (COLS/128 of a 256x256 tile); ties keep
// the wider tile.  At 512 tokens: 112 for I = 14336, 96 for I = 12288.
static int swiglu_cols(const GemmArgs& g) {
  if (g.K % 64) return 128;
  const long mt = (g.M + 255) / 256;
  int best = 128;
  long best_cost = 0;
  for (int c : {128, 112, 96}) {
    const long tiles = mt * ((g.N + c - 1) / c);
    const long cost = ((tiles + kCUs - 1) / kCUs) * c;
    if (c == 128 || cost < best_cost) {
      best = c;
      best_cost = cost;
    }
  }
  return best;
}

template <int COLS, bool SIGN1>
static hipError_t run_swiglu_narrow(GemmArgs g, hipStream_t s) {
  g.m_tiles = (g.M + 255) / 256;
  g.n_tiles = (g.N + COLS - 1) / COLS;
  g.splits = 1;
  g.k_split = g.K;
  if (!SIGN1 && buffer_extents(g, static_cast<size_t>(2) * g.N))
    gemm_swiglu_pp_kernel<COLS><<<g.m_tiles * g.n_tiles, 512, 0, s>>>(g);
  else
    gemm_swiglu_kernel<COLS, SIGN1><<<g.m_tiles * g.n_tiles, 512, 0, s>>>(g);
  return hipGetLastError();
}

// 128-row stream tiles: 96 columns when N splits into them and 64-column
// tiles would need more than one block per CU, else 64 columns.
static bool stream_w96(int M, int N) {
  const long mt = (M + 127) / 128;
  return N % 96 == 0 && mt * (N / 96) <= kCUs && mt * ((N + 63) / 64) > kCUs;
}
static long stream_blocks(int M, int N) {
  const long mt = (M + 127) / 128;
  return mt * (stream_w96(M, N) ? N / 96 : (N + 63) / 64);
}
// A bf16 product takes the stream kernel when its 256x256 tiles would leave
// a quarter of the CUs idle and its 128-row tiles fill more than half of
// them in a single pass.
static bool stream_fits(int M, int N, int K) {
  if (K % 64 != 0 || M <= 0 || big_tiles(M, N) >= kCUs * 3 / 4) return false;
  const long b = stream_blocks(M, N);
  return b > kCUs / 2 && b <= kCUs;
}

// A bf16 Store product also runs in one pass on the two-group kernel's
// 256x192 tiles when those alone fill the GPU (the split plan for the
// product has a single slice: QKV at 2048 tokens).
static bool store_pp192(int M, int N, int K) {
  if (K % 64 != 0) return false;
  const PartialPlan p = partial_plan(M, N, K, true);
  return p.bn == 192 && p.splits == 1;
}

bool gemm_store_direct(int M, int N, int K, bool sign1) {
  return !sign1 && (store_pp192(M, N, K) || stream_fits(M, N, K));
}

template <int EPI, bool SIGN1, bool OUT_F32>
static hipError_t pick_bf16(GemmArgs g, hipStream_t s) {
  if constexpr (EPI == 2 && !OUT_F32) {
    const int cols = swiglu_cols(g);
    if (cols == 112) return run_swiglu_narrow<112, SIGN1>(g, s);
    if (cols == 96) return run_swiglu_narrow<96, SIGN1>(g, s);
  }
  const int cols_big = EPI == 2 ? 128 : 256;
  const long tiles_big = static_cast<long>((g.M + 255) / 256) * ((g.N + cols_big - 1) / cols_big);
  if (EPI == 4) {
    const PartialPlan p = partial_plan(g.M, g.N, g.K, g.K % 64 == 0);
    if (p.bn == 128) return run_partial_narrow<128, OUT_F32, SIGN1>(g, p.splits, s);
    if (p.bn == 192) return run_partial_narrow<192, OUT_F32, SIGN1>(g, p.splits, s);
    return run_bf16<256, 256, 2, 4, EPI, SIGN1, OUT_F32>(g, p.splits, s);
  }
  if constexpr (EPI == 0 && !SIGN1) {
    if (store_pp192(g.M, g.N, g.K) && buffer_extents(g, static_cast<size_t>(g.N))) {
      g.m_tiles = (g.M + 255) / 256;
      g.n_tiles = g.N / 192;
      g.splits = 1;
      g.k_split = g.K;
      gemm_pp_dma_kernel<192, 4, 2, EPI, OUT_F32, 2, 3><<<g.m_tiles * g.n_tiles, 512, 0, s>>>(g);
      return hipGetLastError();
    }
  }
  if (tiles_big >= kCUs * 3 / 4) return run_bf16<256, 256, 2, 4, EPI, SIGN1, OUT_F32>(g, 1, s);
  if constexpr (EPI == 0 && !SIGN1) {
    if (stream_fits(g.M, g.N, g.K) && buffer_extents(g, static_cast<size_t>(g.N))) {
      g.m_tiles = (g.M + 127) / 128;
      g.splits = 1;
      g.k_split = g.K;
      if (stream_w96(g.M, g.N)) {
        g.n_tiles = g.N / 96;
        gemm_stream_kernel<96, 4, 1, EPI, OUT_F32, 5><<<g.m_tiles * g.n_tiles, 256, 0, s>>>(g);
      } else {
        g.n_tiles = (g.N + 63) / 64;
        gemm_stream_kernel<64, 2, 2, EPI, OUT_F32, 5><<<g.m_tiles * g.n_tiles, 256, 0, s>>>(g);
      }
      return hipGetLastError();
    }
  }
  return run_bf16<128, 128, 2, 2, EPI, SIGN1, OUT_F32>(g, 1, s);
}

// fp32 output in one pass: the slice writer with a single slice
template <bool SIGN1>
static hipError_t pick_store_f32(GemmArgs g, hipStream_t s) {
  const long tiles_big = static_cast<long>((g.M + 255) / 256) * ((g.N + 255) / 256);
  if (tiles_big >= kCUs * 3 / 4) return run_bf16<256, 256, 2, 4, 4, SIGN1, true>(g, 1, s);
  return run_bf16<128, 128, 2, 2, 4, SIGN1, true>(g, 1, s);
}

template <bool SIGN1>
static hipError_t dispatch_bf16(const GemmCall& c, GemmArgs g, hipStream_t s) {
  switch (c.epi) {
    case Epi::StoreF32: return pick_store_f32<SIGN1>(g, s);
    case Epi::Store: return pick_bf16<0, SIGN1, false>(g, s);
    case Epi::SwiGLU: return pick_bf16<2, SIGN1, false>(g, s);
    case Epi::Partial: return pick_bf16<4, SIGN1, true>(g, s);
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
  g.part_stride = c.part_stride;
  g.splits_out = c.splits_out;
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
      case Epi::Store:
      case Epi::StoreF32: gemm_f32_kernel<0><<<blocks, 256, 0, s>>>(g); break;
      case Epi::Resid: gemm_f32_kernel<1><<<blocks, 256, 0, s>>>(g); break;
      case Epi::SwiGLU: gemm_f32_kernel<2><<<blocks, 256, 0, s>>>(g); break;
      case Epi::Partial: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  return c.Wscale ? dispatch_bf16<true>(c, g, s) : dispatch_bf16<false>(c, g, s);
}

}  // namespace tlp
