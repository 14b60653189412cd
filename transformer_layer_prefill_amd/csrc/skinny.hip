// Projections of short micro-batches (M <= 32 token rows): the decode steps
// of a token-by-token forward (oxibonsai-kernels metal_full_layer.rs, the
// per-token layer: the same projections applied to one hidden row) and the
// rows of a speculative verify batch.  At these sizes a projection reads each
// weight once and does little arithmetic per byte, so it is bound by HBM
// bandwidth; the 256x256 prefill tiles would waste almost all of their MFMA
// work on padding rows.
//
// Every wavefront multiplies 32 weight rows by all M activation rows,
// zero-padded to the 32 columns of v_mfma_f32_32x32x16_bf16, over one slice
// of K.  In the fragment layout (1-bit weights, K tails) the weight rows
// stream from HBM straight into registers: lane (row r, half h) loads the
// 16-byte chunks 2s + h of the row's 128-byte lines, so the two lanes of a
// row consume whole lines over four instructions (dense weights are loaded
// as whole lines per instruction, below).  The products are
// written as fp32 split-K slices that the following row kernel sums (or the
// SwiGLU finish below, for the fused gate/up weight).
//
// One activation row (a decode step) with 1-bit weights: its address is the
// same for every lane, so each 128-wide chunk of it is fetched with scalar
// loads (read-only, through the constant address space) instead of one 16-byte
// vector load per k-step, and each lane selects its 8 columns.  Every lane then
// holds real activations (only output column 0 is stored; other columns of the
// product are discarded).
//
// Several activation rows (2..32): the four wavefronts of a block take four
// consecutive 32-row weight groups of the same K slice, so they share the
// activations: each 128-wide chunk of the rows is loaded once per block (one
// 16-byte piece per thread and 16 rows) into a double-buffered LDS tile, rows
// padded to 272 bytes so the 16 rows a read touches hit distinct banks, with
// one barrier per chunk.  Their dense weights are loaded as whole lines (8
// rows x 128 bytes per load instruction) and rewritten into MFMA fragments
// through a private LDS tile per wavefront (one 16-byte write and one read per
// lane and k-step), bit-identical to loading the fragments directly.
//
// 1-bit weights: lane (row r, half h) loads the row's 128 sign bits and fp16
// group scale of each 128-wide K chunk (16 + 2 bytes instead of 256) and
// expands the 8 bits of each k-step into bf16 +-scale in registers; slices
// are whole 128-wide groups.
//
// One activation row with dense weights takes a kernel of its own (below):
// plain dot products on the vector ALUs, with loads that read whole 128-byte
// lines; as the QKV projection of a decode step it also computes the
// attention norm of its row itself.
//
// Whole-line weight loads (the one-row kernel, and dense weights with shared
// rows) read each line once, in one instruction, so they are non-temporal:
// they stream past the caches instead of evicting what the other kernels of
// the step (the KV cache, the activations, the split-K slices) still use
// (gate/up at the 8B decode shape 43 -> 39 µs).  The fragment-layout loads
// (1-bit weights, K tails) stay ordinary: each of their instructions reads a
// part of each line it touches and the following instructions read the rest
// from cache, which a non-temporal load does not keep (with non-temporal
// fragment loads the 16-row LM head of the verify tail went from 203 to 315 µs).
#include "common.h"
#include "launch.h"

namespace tlp {

struct SkinnyArgs {
  const uint16_t* A;     // [M][lda] bf16
  const void* W;         // dense: [N][K] bf16; 1-bit: sign words u32 [N][K/32]
  const uint16_t* Wscale;   // 1-bit: fp16 [N][K/128]
  float* out;            // slice s at out + s * part_stride, [M][ldo] fp32
  size_t part_stride;
  int lda, ldo;
  int M, N, K;
  int splits, k_split;   // k_split: a multiple of 64
  int groups;            // ceil(N / 32)
  // one-row kernel normalising its input row itself (launch_gemv_norm)
  const uint16_t* gain;  // RMSNorm gain [K]
  float eps;
};

__device__ __forceinline__ bf16x8_t ld16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ bf16x8_t zero16() { return __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0)); }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const u32x4_t const_u32x4;

// 16 bytes of weights, loaded non-temporally (the one-row kernel)
__device__ __forceinline__ uint4 ldw16(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(static_cast<const u32x4_t*>(p)));
}

// activation rows: one row through scalar loads, or 2..32 rows shared by the
// block through LDS (the K tails past the last 128-wide chunk load per lane)
enum SkinnyRows { kRowsOne = 1, kRowsShared = 2 };

template <bool SIGN1, int ROWS>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(SkinnyArgs g) {
  constexpr int STEPS = 8;   // 16-wide k-steps per buffer (128 of K)
  constexpr bool SHARED = ROWS == kRowsShared;   // else one row (kRowsOne)
  constexpr int AST = 17;    // LDS row stride of the shared activations, in 16-byte pieces
  __shared__ uint4 alds[SHARED ? 2 * 32 * AST : 1];
  // dense weights with shared rows: each wavefront's 32 rows x 128 of K pass
  // through a private 8 KB LDS tile (whole-line loads in, MFMA fragments out)
  constexpr bool LINES = SHARED && !SIGN1;
  __shared__ uint4 wlds[LINES ? 4 * 32 * 16 : 1];
  const int lane = threadIdx.x & 63;
  // wavefront-uniform (readfirstlane lets the compiler see it): K ranges and
  // the one-row activation addresses are scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int split, grp;
  if constexpr (SHARED) {
    // block = 4 consecutive groups of one slice; every wavefront takes part in
    // the loads and barriers, one past the last group stores nothing
    const int gblocks = (g.groups + 3) / 4;
    split = blockIdx.x / gblocks;
    grp = (blockIdx.x % gblocks) * 4 + wave;
  } else {
    const int item = blockIdx.x * 4 + wave;
    if (item >= g.groups * g.splits) return;   // whole wavefronts
    split = item % g.splits;
    grp = item / g.splits;
  }
  const int lr = lane & 31, lh = lane >> 5;
  const int n = grp * 32 + lr;
  const size_t nr = static_cast<size_t>(n < g.N ? n : g.N - 1);
  const uint16_t* wrow = static_cast<const uint16_t*>(g.W) + nr * g.K + 8 * lh;
  const uint32_t* brow = static_cast<const uint32_t*>(g.W) + nr * (g.K >> 5);   // 1-bit
  const uint16_t* srow = g.Wscale + nr * (g.K >> 7);                              // 1-bit
  // whole-line loads (LINES): lane (rr, c8) loads 16 bytes at column 8*c8 of
  // each 64-wide half of the chunk, of rows rr, rr+8, rr+16, rr+24 of the group
  const int rr = lane >> 3, c8 = lane & 7;
  const uint16_t* lrow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int nq = grp * 32 + 8 * q + rr;
    lrow[q] = static_cast<const uint16_t*>(g.W) + static_cast<size_t>(nq < g.N ? nq : g.N - 1) * g.K + 8 * c8;
  }
  // LDS tile: row r's 16-byte piece p at r*256 + (p ^ lsw(r))*16; the swizzle
  // keeps the 16 lanes of each write (two rows, 8 pieces) and of each fragment
  // read (16 rows, one piece) on distinct bank quads
  auto lsw = [](int r) { return ((r & 1) << 3) | ((r >> 1) & 7); };
  char* wtile = reinterpret_cast<char*>(wlds) + (LINES ? wave * 8192 : 0);
  const bool a_ok = lr < g.M;
  const uint16_t* arow = g.A + static_cast<size_t>(a_ok ? lr : 0) * g.lda + 8 * lh;
  const int k_begin = split * g.k_split;
  const int k_end = min(g.K, k_begin + g.k_split);

  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  if constexpr (SHARED) {
    for (int i = threadIdx.x; i < 2 * 32 * AST; i += 256) alds[i] = make_uint4(0, 0, 0, 0);
  }

  // Two register buffers of STEPS k-steps: the loads of the next 128 of K are
  // issued before the MFMAs of the current ones.
  // (1-bit: wv[0] holds the chunk's four sign words, wv[1] its scale)
  bf16x8_t w0[STEPS], a0[STEPS], w1[STEPS], a1[STEPS];
  auto load_w = [&](bf16x8_t (&wv)[STEPS], int k) __attribute__((always_inline)) {
    if constexpr (SIGN1) {
      wv[0] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(brow + (k >> 5)));
      wv[1] = __builtin_bit_cast(bf16x8_t, make_uint4(srow[k >> 7], 0, 0, 0));
    } else if constexpr (LINES) {
      // wv[2q + h]: row rr + 8q, columns k + 64h + 8*c8 .. +8 (non-temporal:
      // whole lines, each read once)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h) wv[2 * q + h] = __builtin_bit_cast(bf16x8_t, ldw16(lrow[q] + k + 64 * h));
    } else {
#pragma unroll
      for (int j = 0; j < STEPS; ++j) wv[j] = ld16(wrow + k + 16 * j);
    }
  };
  // LINES: rewrite the chunk as MFMA fragments (wv[j] = row lr, columns
  // 16j + 8*lh .. +8) through this wavefront's tile; a wavefront's LDS
  // accesses run in order, so the next chunk's writes cannot pass these reads
  auto relayout = [&](bf16x8_t (&wv)[STEPS]) __attribute__((always_inline)) {
    if constexpr (LINES) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = 8 * q + rr;
          *reinterpret_cast<bf16x8_t*>(wtile + r * 256 + (((8 * h + c8) ^ lsw(r)) << 4)) = wv[2 * q + h];
        }
#pragma unroll
      for (int j = 0; j < STEPS; ++j)
        wv[j] = *reinterpret_cast<const bf16x8_t*>(wtile + lr * 256 + (((2 * j + lh) ^ lsw(lr)) << 4));
    }
  };
  // (activations first: a wait for them leaves the weight loads in flight)
  auto load = [&](bf16x8_t (&wv)[STEPS], bf16x8_t (&av)[STEPS], int k) __attribute__((always_inline)) {
    if constexpr (SHARED) {
      // this thread's pieces of the chunk: rows t/16 and 16 + t/16, columns
      // k + 8*(t%16) .. +8 (raw bits in av[0], av[1])
      const int pr = threadIdx.x >> 4, pc = threadIdx.x & 15;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (pr + 16 * h < g.M)
          av[h] = ld16(g.A + static_cast<size_t>(pr + 16 * h) * g.lda + k + 8 * pc);
    } else {
      // one row: columns k .. k+127 as 16 uniform 16-byte pieces
      const const_u32x4* ap = (const const_u32x4*)(g.A + k);
      u32x4_t piece[2 * STEPS];
#pragma unroll
      for (int q = 0; q < 2 * STEPS; ++q) piece[q] = ap[q];
#pragma unroll
      for (int j = 0; j < STEPS; ++j)
        av[j] = __builtin_bit_cast(bf16x8_t, lh ? piece[2 * j + 1] : piece[2 * j]);
    }
    load_w(wv, k);
  };
  // shared rows: put this thread's pieces of the chunk into LDS buffer b,
  // barrier, then read this lane's 8 fragments (row lr, columns 16j + 8h)
  auto share = [&](bf16x8_t (&av)[STEPS], int b) __attribute__((always_inline)) {
    if constexpr (SHARED) {
      const int pr = threadIdx.x >> 4, pc = threadIdx.x & 15;
      uint4* t = alds + b * 32 * AST;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (pr + 16 * h < g.M) t[(pr + 16 * h) * AST + pc] = __builtin_bit_cast(uint4, av[h]);
      lds_barrier();
#pragma unroll
      for (int j = 0; j < STEPS; ++j) av[j] = __builtin_bit_cast(bf16x8_t, t[lr * AST + 2 * j + lh]);
    }
  };
  auto mma = [&](const bf16x8_t (&wv)[STEPS], const bf16x8_t (&av)[STEPS]) __attribute__((always_inline)) {
    if constexpr (SIGN1) {
      // k-step j covers columns 16j + 8h .. +8: word j/2, bits (j%2)*16 + 8h
      const uint4 q = __builtin_bit_cast(uint4, wv[0]);
      const uint32_t words[4] = {q.x, q.y, q.z, q.w};
      const uint32_t sbf =
          f32_to_bf16(static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(
              __builtin_bit_cast(uint4, wv[1]).x))));
#pragma unroll
      for (int j = 0; j < STEPS; ++j) {
        const uint32_t bits8 = (words[j >> 1] >> ((j & 1) * 16 + 8 * lh)) & 0xffu;
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, sign1_expand8(bits8, sbf)), av[j], acc, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < STEPS; ++j)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv[j], av[j], acc, 0, 0, 0);
    }
  };
  constexpr int KB = 16 * STEPS;
  int k = k_begin;
  if constexpr (SHARED) __syncthreads();   // the zeroed tile
  // (shared rows: chunk c goes through LDS buffer c % 2; the barrier in share()
  // also orders the reuse of a buffer two chunks later)
  if (k + KB <= k_end) {
    load(w0, a0, k);
    k += KB;
    for (;;) {
      if (k + KB > k_end) { share(a0, 0); relayout(w0); mma(w0, a0); break; }
      load(w1, a1, k);
      k += KB;
      share(a0, 0);
      relayout(w0);
      mma(w0, a0);
      if (k + KB > k_end) { share(a1, 1); relayout(w1); mma(w1, a1); break; }
      load(w0, a0, k);
      k += KB;
      share(a1, 1);
      relayout(w1);
      mma(w1, a1);
    }
  }
  // (1-bit slices are whole 128-wide chunks: nothing is left here)
  if constexpr (!SIGN1) {
  for (; k + 64 <= k_end; k += 64) {
    bf16x8_t wv[4], av[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wv[j] = ld16(wrow + k + 16 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) av[j] = a_ok ? ld16(arow + k + 16 * j) : zero16();
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv[j], av[j], acc, 0, 0, 0);
  }
  // remaining 16-wide steps; a half step past K (K % 16 == 8) reads zeros
  for (; k < k_end; k += 16) {
    const bool ok = k + 8 * lh < k_end;
    const bf16x8_t wv = ok ? ld16(wrow + k) : zero16();
    const bf16x8_t av = ok && a_ok ? ld16(arow + k) : zero16();
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv, av, acc, 0, 0, 0);
  }
  }

  // lane holds output column m = lr and weight rows grp*32 + 8*(r/4) + 4*lh + r%4
  if (!a_ok || grp >= g.groups) return;
  float* orow = g.out + split * g.part_stride + static_cast<size_t>(lr) * g.ldo;
  const bool vec = ((g.ldo | g.part_stride) & 3) == 0;   // float4-aligned rows
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int n0 = grp * 32 + 8 * q + 4 * lh;
    if (vec && n0 + 3 < g.N) {
      *reinterpret_cast<float4*>(orow + n0) =
          make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n0 + i < g.N) orow[n0 + i] = acc[4 * q + i];
    }
  }
}

// One activation row, dense weights: a dot product per weight row on the
// vector ALUs (v_dot2 multiplies bf16 pairs and adds them into fp32).  Lane
// (r = lane / 8, c = lane % 8) reads bytes 16c .. 16c+15 of a 64-wide K
// segment of row r of each of the wavefront's four 8-row sets, so one load
// instruction covers 8 rows x 128 contiguous bytes (the MFMA fragment layout
// above covers 32 rows x 32 bytes per instruction, which streams from HBM
// more slowly: gate/up at the 8B decode shape 46 -> 43 µs with this layout).
// Each lane keeps the activations of its 8 columns and one partial sum per row
// set; the 8 lanes of a row add theirs at the end.  B segments of K form one
// batch of loads, and the next batch is in flight while one is summed.  Work
// items, K slices and outputs are those of gemm_skinny_kernel.  With a
// normalised input (kGemvNorm: a decode step's QKV projection) each
// wavefront first reduces the whole row itself and writes its K slice of
// RMSNorm(row) * gain into LDS, so the step needs no separate norm pass.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// input of the one-row kernel: the row as stored, or RMSNorm(row) * gain
enum GemvIn { kGemvRow = 0, kGemvNorm = 1 };
constexpr int kGemvMaxSlice = 4096;   // longest K slice a normalised input stages in LDS

__device__ __forceinline__ float dot8(const uint4 w, const uint4 x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, x.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, x.w), acc, false);
  return acc;
}

template <int B, int IN>
__global__ __launch_bounds__(256) void gemv_bf16_kernel(SkinnyArgs g) {
  constexpr int SEG = 64;
  // normalised input: this wavefront's K slice of the row, built in LDS
  __shared__ uint4 xlds[IN == kGemvRow ? 1 : 4 * kGemvMaxSlice / 8];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x * 4 + wave;
  if (item >= g.groups * g.splits) return;   // whole wavefronts
  const int split = item % g.splits, grp = item / g.splits;
  const int rr = lane >> 3, c = lane & 7;
  const uint16_t* W = static_cast<const uint16_t*>(g.W);
  const uint16_t* wrow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int n = grp * 32 + 8 * q + rr;
    wrow[q] = W + static_cast<size_t>(n < g.N ? n : g.N - 1) * g.K + 8 * c;
  }
  const int k_begin = split * g.k_split;
  const int k_end = min(g.K, k_begin + g.k_split);
  // the input row from memory (kGemvRow) or from this wavefront's LDS slice
  // (indexed from k_begin); either way lane c reads columns 8c .. 8c+7 of a segment
  const uint16_t* xrow = g.A + 8 * c;
  uint16_t* const xw = reinterpret_cast<uint16_t*>(xlds) + (IN == kGemvRow ? 0 : wave * kGemvMaxSlice);
  auto xload = [&](int k) __attribute__((always_inline)) -> uint4 {
    if constexpr (IN == kGemvRow) return *reinterpret_cast<const uint4*>(xrow + k);
    else return *reinterpret_cast<const uint4*>(xw + (k - k_begin) + 8 * c);
  };
  // (the first batch's weight loads are issued before this, so the weight
  // stream starts with the kernel)
  auto prologue = [&]() __attribute__((always_inline)) {
    if constexpr (IN == kGemvNorm) {
      // RMSNorm of the whole row, then gain * (x * inv) rounded as the row pass does
      float ss = 0.f;
#pragma unroll 8
      for (int k = 8 * lane; k < g.K; k += 512) {
        const uint4 u = *reinterpret_cast<const uint4*>(g.A + k);
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = __uint_as_float(w4[i] << 16), hi = __uint_as_float(w4[i] & 0xffff0000u);
          ss += lo * lo + hi * hi;
        }
      }
      ss = wave_sum(ss);
      const float inv = rsqrtf(ss / static_cast<float>(g.K) + g.eps);
#pragma unroll 4
      for (int k = k_begin + 8 * lane; k < k_end; k += 512) {
        const uint4 u = *reinterpret_cast<const uint4*>(g.A + k);
        const uint4 gg = *reinterpret_cast<const uint4*>(g.gain + k);
        const uint32_t xv[4] = {u.x, u.y, u.z, u.w}, gv[4] = {gg.x, gg.y, gg.z, gg.w};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = __uint_as_float(xv[i] << 16), x1 = __uint_as_float(xv[i] & 0xffff0000u);
          const float g0 = __uint_as_float(gv[i] << 16), g1 = __uint_as_float(gv[i] & 0xffff0000u);
          o[i] = pack_bf16x2(g0 * (x0 * inv), g1 * (x1 * inv));
        }
        *reinterpret_cast<uint4*>(xw + (k - k_begin)) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    // (a wavefront's LDS accesses run in order: its reads below see these writes)
  };

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  uint4 wa[B][4], xa[B], wb[B][4], xb[B];
  auto load_x = [&](uint4 (&x)[B], int k) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < B; ++s) x[s] = xload(k + SEG * s);
  };
  auto load_w = [&](uint4 (&w)[B][4], int k) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < B; ++s)
#pragma unroll
      for (int q = 0; q < 4; ++q) w[s][q] = ldw16(wrow[q] + k + SEG * s);
  };
  auto load = [&](uint4 (&w)[B][4], uint4 (&x)[B], int k) __attribute__((always_inline)) {
    load_x(x, k);
    load_w(w, k);
  };
  auto sum = [&](const uint4 (&w)[B][4], const uint4 (&x)[B]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < B; ++s)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = dot8(w[s][q], x[s], acc[q]);
  };
  constexpr int KB = B * SEG;
  int k = k_begin;
  const bool batches = k + KB <= k_end;
  if (batches) load_w(wa, k);
  if constexpr (IN != kGemvRow) prologue();
  if (batches) {
    load_x(xa, k);
    k += KB;
    for (;;) {
      if (k + KB > k_end) { sum(wa, xa); break; }
      load(wb, xb, k);
      k += KB;
      sum(wa, xa);
      if (k + KB > k_end) { sum(wb, xb); break; }
      load(wa, xa, k);
      k += KB;
      sum(wb, xb);
    }
  }
  // remaining segments; columns past the slice's end (K % 64 != 0) read as zeros
  for (; k < k_end; k += SEG) {
    const bool ok = k + 8 * c < k_end;
    const uint4 z = make_uint4(0, 0, 0, 0);
    const uint4 x = ok ? xload(k) : z;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = dot8(ok ? ldw16(wrow[q] + k) : z, x, acc[q]);
  }
  // the 8 lanes of a row hold its partial sums over disjoint columns
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int off = 4; off > 0; off >>= 1) acc[q] += __shfl_xor(acc[q], off, 8);
  // lane c < 4 of row r stores row set c: weight row grp*32 + 8c + r (an
  // empty slice stores zeros)
  float v = acc[0];
#pragma unroll
  for (int q = 1; q < 4; ++q) v = c == q ? acc[q] : v;
  const int n = grp * 32 + 8 * c + rr;
  if (c < 4 && n < g.N) g.out[split * g.part_stride + n] = v;
}

// K slice length of a split into `splits` slices: whole 256-wide main-loop
// iterations when K allows (the last slice may be shorter, or empty)
static int skinny_k_split(int K, int splits, bool sign1) {
  const int gran = K >= 256 * splits ? 256 : (sign1 ? 128 : 64);
  return ((K + splits - 1) / splits + gran - 1) / gran * gran;
}

int skinny_splits(int N, int K, bool sign1) {
  const int groups = (N + 31) / 32;
  // ~8 wavefronts per CU; 1-bit weights have 16x fewer bytes per wavefront in
  // flight, so they take as many slices as the row passes accept
  int splits = (2048 + groups - 1) / groups;
  if (sign1) splits = kSkinnyMaxSplits;
  if (splits > kSkinnyMaxSplits) splits = kSkinnyMaxSplits;
  const int max_by_k = K / (sign1 ? 128 : 256);  // slices of at least 256 (1-bit: 128)
  if (splits > max_by_k) splits = max_by_k;
  return splits < 1 ? 1 : splits;
}

hipError_t launch_gemm_skinny(const void* A, int lda, const void* W, const void* Wscale, int M,
                              int N, int K, float* out, int ldo, size_t part_stride, int splits,
                              hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (M > kSkinnyMaxM || splits < 1 || (K & 7) || (lda & 7)) return hipErrorInvalidValue;
  const bool sign1 = Wscale != nullptr;
  if (sign1 && (K & 127)) return hipErrorInvalidValue;
  SkinnyArgs g{};
  g.A = static_cast<const uint16_t*>(A);
  g.W = W;
  g.Wscale = static_cast<const uint16_t*>(Wscale);
  g.out = out;
  g.part_stride = part_stride;
  g.lda = lda;
  g.ldo = ldo;
  g.M = M;
  g.N = N;
  g.K = K;
  g.splits = splits;
  // slices of whole 256-wide main-loop iterations when K allows (the last
  // slice may be shorter, or empty: it then writes zeros)
  g.k_split = skinny_k_split(K, splits, sign1);
  g.groups = (N + 31) / 32;
  const int waves = g.groups * splits;
  const unsigned blocks = (waves + 3) / 4;
  if (M == 1) {
    if (sign1) gemm_skinny_kernel<true, kRowsOne><<<blocks, 256, 0, s>>>(g);
    else gemv_bf16_kernel<2, kGemvRow><<<blocks, 256, 0, s>>>(g);
  } else {
    const unsigned sblocks = static_cast<unsigned>((g.groups + 3) / 4 * splits);
    if (sign1) gemm_skinny_kernel<true, kRowsShared><<<sblocks, 256, 0, s>>>(g);
    else gemm_skinny_kernel<false, kRowsShared><<<sblocks, 256, 0, s>>>(g);
  }
  return hipGetLastError();
}

bool gemv_norm_ok(int N, int K, int splits) {
  return N > 0 && K > 0 && K % 8 == 0 && splits >= 1 && skinny_k_split(K, splits, false) <= kGemvMaxSlice;
}

hipError_t launch_gemv_norm(const void* A, const void* gain, float eps, const void* W, int N, int K,
                            float* out, size_t part_stride, int splits, hipStream_t s) {
  if (!gemv_norm_ok(N, K, splits)) return hipErrorInvalidValue;
  SkinnyArgs g{};
  g.A = static_cast<const uint16_t*>(A);
  g.W = W;
  g.out = out;
  g.part_stride = part_stride;
  g.lda = K;
  g.ldo = N;
  g.M = 1;
  g.N = N;
  g.K = K;
  g.splits = splits;
  g.k_split = skinny_k_split(K, splits, false);
  g.groups = (N + 31) / 32;
  g.gain = static_cast<const uint16_t*>(gain);
  g.eps = eps;
  gemv_bf16_kernel<2, kGemvNorm><<<(g.groups * splits + 3) / 4, 256, 0, s>>>(g);
  return hipGetLastError();
}

// act[m][i] = silu(gate) * up with gate = sum_s part_s[m][i] and up =
// sum_s part_s[m][I + i] (the fused [gate ; up] weight's slices).
__global__ __launch_bounds__(256) void swiglu_finish_kernel(const float* __restrict__ part,
                                                            int splits, size_t part_stride,
                                                            int M, int I,
                                                            uint16_t* __restrict__ act) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<size_t>(M) * I) return;
  const int m = static_cast<int>(idx / I), i = static_cast<int>(idx % I);
  const float* p = part + static_cast<size_t>(m) * 2 * I + i;
  float gsum = 0.f, usum = 0.f;
  for (int sl = 0; sl < splits; ++sl) {
    gsum += p[sl * part_stride];
    usum += p[sl * part_stride + I];
  }
  act[idx] = f32_to_bf16(silu_f32(gsum) * usum);
}

hipError_t launch_swiglu_finish(const float* part, int splits, size_t part_stride, int M, int I,
                                void* act, hipStream_t s) {
  if (M <= 0 || I <= 0) return hipSuccess;
  const size_t n = static_cast<size_t>(M) * I;
  swiglu_finish_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
      part, splits, part_stride, M, I, static_cast<uint16_t*>(act));
  return hipGetLastError();
}

}  // namespace tlp
