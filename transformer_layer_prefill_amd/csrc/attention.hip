// Causal grouped-query attention over the KV cache for every query row of a
// micro-batch at once (oxibonsai-kernels metal_prefill.rs, encode_layer_prefill
// step 3e: scores q.K/sqrt(hd) over seq_len = pos + 1 keys, softmax, weighted
// sum of V; query head h reads kv head h / heads_per_group).  That page runs it
// one query position at a time with a materialised score row; here it is one
// flash-style kernel with an online softmax and no score buffer.
//
// bf16 kernel (gfx950 MFMA; with an fp16 cache the same kernel runs
// v_mfma_f32_32x32x16_f16 on fp16 K, V, Q and P).  A block owns one kv head and a tile of query
// tokens; its four or eight wavefronts are (query head of the group, 32-token
// slice) pairs that share every K/V block staged in LDS, so K/V are read once
// per group and tile.  Per 64-key block a wavefront computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (lane = query, 32 key scores per lane), runs the
// online softmax in fp32 with exp2, and accumulates O^T = V^T P^T, taking P
// straight from the score registers and V^T from transposing LDS reads.
//
// Short micro-batches over short histories (a grid of at most half as many
// blocks as CUs) take a two-key-group form: a block holds half as many query
// heads, and its wavefronts form two groups that run the same queries over
// alternate key blocks, each with its own K/V ring; at the end the second
// group passes its running max, weight sum and unnormalised output through
// LDS and the first merges them.  Twice the blocks, half the longest chain of
// key blocks.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace tlp {

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  int q_ld, out_ld;
  int M, start, nq, nkv, max_seq;
  int group;      // nq / nkv
  int hpb;        // query heads per block (min(group, 4))
  int waves;      // wavefronts per block (4 or 8): waves / hpb 32-token slices
  int tiles;      // token tiles
  float scale_log2;  // log2(e) / sqrt(hd)
  // split-KV form: the keys of every (tile, head quad) are cut into kv_splits
  // ranges whose unnormalised partial results go to po [split][M][nq][hd] and
  // pml [split][M][nq][2] = (running max in log2 units, weight sum)
  int kv_splits;
  float* po;
  float* pml;
};

// K and V blocks of 64 keys are copied global -> LDS with DMA into rings of
// three K and two V slots: while block kb's softmax runs on the VALUs, the
// MFMAs already compute block kb+1's scores, and the copies of K(kb+2) and
// V(kb+1) are in flight.  Eight wavefronts (one block per CU) use four K and
// four V slots and meet at a barrier every second key block, the copies of
// the next pair of blocks in flight meanwhile.
// Rows are stored as 16-byte chunks, chunk c of key row r at slot c ^ swz(r).
// The LDS has 64 banks (256 bytes per cycle): a b128 read is served 16 lanes
// at a time, a transposing b64 read 32 lanes at a time.  With RPL = 256 /
// row bytes key rows per bank line, K uses (r / RPL) % chunks so the 16 rows
// of a b128 step cover all banks once, and V uses 4 * ((r / RPL) % (chunks /
// 4)) so the four rows x 64 bytes of a transposing step do.  Key rows past
// the last visible key are clamped to it (finite data that the mask gives a
// zero weight), so unwritten cache slots never reach the products.
// MFMA operands of the bf16 cache, or of the fp16 cache (Q converted to fp16
// when loaded, P rounded to fp16).
template <bool KV16> struct AttnOps;
template <> struct AttnOps<false> {
  typedef bf16x8_t V8;
  static __device__ __forceinline__ f32x16_t mma(V8 a, V8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ __bf16 cvt(float x) { return static_cast<__bf16>(x); }
  static __device__ __forceinline__ float sum2(uint32_t pair, float acc) { return dot2_bf16_sum(pair, acc); }
};
template <> struct AttnOps<true> {
  typedef f16x8_t V8;
  static __device__ __forceinline__ f32x16_t mma(V8 a, V8 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ _Float16 cvt(float x) { return static_cast<_Float16>(x); }
  static __device__ __forceinline__ float sum2(uint32_t pair, float acc) { return dot2_f16_sum(pair, acc); }
};


// Global -> LDS copy of 16 bytes per lane (lane l writes lds + 16 l) issued
// from an asm block.  The compiler's wait insertion cannot tell which ring
// slot a copy writes, so a copy it tracks makes it drain every LDS read and
// every copy before the next LDS read; the kernel orders its copies and
// reads itself (its own vmcnt waits and barriers), so these are left
// untracked.  `lds` must be wavefront-uniform (it goes to M0).
__device__ __forceinline__ void dma16_untracked(const void* src, void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0), "v"(src)
               : "memory", "m0");
}

template <int HD, int NW, bool SPLIT, bool KV16, bool KSPLIT = false>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_fwd_bf16_kernel(AttnArgs a) {
  typedef AttnOps<KV16> Ops;
  typedef typename Ops::V8 V8;
  constexpr int KB = 64;                 // keys per block
  constexpr int ROWB = HD * 2;           // bytes per key row
  constexpr int CH = ROWB / 16;          // 16-byte chunks per row
  constexpr int RPI = 1024 / ROWB;       // rows per DMA instruction
  constexpr int TILE = KB * ROWB;        // bytes of one K (or V) block
  constexpr int GW = KSPLIT ? NW / 2 : NW;   // wavefronts per key group
  constexpr int PW = TILE / 1024 / GW;   // DMA instructions per wave per K (or V) block
  constexpr int KS = HD / 16;            // k-steps of the QK^T contraction
  constexpr int DB = HD / 32;            // 32-wide blocks of the head dimension
  constexpr int RPL = 256 / ROWB;        // key rows per LDS bank line
  auto swz_k = [](int r) { return (r / RPL) & (CH - 1); };
  auto swz_v = [](int r) { return ((r / RPL) & (CH / 4 - 1)) * 4; };
  // Eight wavefronts (one block per CU) meet at a barrier every second key
  // block, with four K and four V ring slots, so the copies of a pair of
  // blocks are issued a whole pair ahead.
  constexpr bool PAIR = NW == 8 && !KSPLIT && !SPLIT;
  constexpr int SK = PAIR ? 4 : KSPLIT ? 2 : 3, SV = PAIR ? 4 : 2;   // ring slots (per key group)
  constexpr int RING = (SK + SV) * TILE;
  __shared__ __attribute__((aligned(1024))) char smem[(KSPLIT ? 2 : 1) * RING];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases stay scalar
  // key group (two groups take alternate key blocks of the same queries) and
  // wavefront within it
  const int kg = KSPLIT ? wave / GW : 0, wq = KSPLIT ? wave % GW : wave;
  char* const kring = smem + kg * RING;
  char* const vring = kring + SK * TILE;
  const int lr = lane & 31, lh = lane >> 5;
  const int hpb = a.hpb;
  const int tsub = GW / hpb;           // 32-token slices per block
  const int bt = 32 * tsub;            // tokens per block
  // Work item w = (kv head j, head quad, tile[, key range]), tile fastest
  // (after the key range) and longest rows first.  Blocks are dealt
  // round-robin to the eight XCDs, so block b is given item
  // (b % 8) * (nb / 8) + b / 8: each XCD then works through a contiguous range
  // of items, i.e. the tiles of one kv head, whose K/V blocks its L2 serves to
  // all of them.
  const int nb = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
  const int w_all = (nb & 7) ? b : (b & 7) * (nb >> 3) + (b >> 3);
  const int n_split = SPLIT ? a.kv_splits : 1;
  const int split = w_all % n_split, w = w_all / n_split;
  const int tile = a.tiles - 1 - w % a.tiles;
  const int quads = a.group / hpb;
  const int jq = w / a.tiles;
  const int j = jq / quads, quad = jq % quads;
  const int h = j * a.group + quad * hpb + wq % hpb;
  const int t0w = tile * bt + (wq / hpb) * 32;        // first query token of this wave
  const int t = t0w + lr;                             // this lane's query token
  const bool q_ok = t < a.M;
  const int pos = a.start + t;
  const int pos_lo = a.start + t0w;                   // every key <= pos_lo is visible to the wave

  // Q^T fragments (B operand): lane holds Q[t][ks*16 + lh*8 .. +8]
  V8 qf[KS];
  {
    const uint16_t* qrow = a.q + static_cast<size_t>(q_ok ? t : 0) * a.q_ld + h * HD;
    const uint32_t keep = q_ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 u = *reinterpret_cast<const uint4*>(qrow + ks * 16 + lh * 8);
      u = make_uint4(u.x & keep, u.y & keep, u.z & keep, u.w & keep);
      if constexpr (KV16) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          qf[ks][e] = static_cast<_Float16>(bf16_to_f32(static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)))));
      } else {
        qf[ks] = __builtin_bit_cast(bf16x8_t, u);
      }
    }
  }

  const int last_tok = min(a.M, (tile + 1) * bt) - 1;
  const int kv_end = a.start + last_tok + 1;          // keys this block may need
  const int nkb = (kv_end + KB - 1) / KB;
  // key blocks [kb_lo, kb_hi) of this block (all of them unless split)
  const int per = (nkb + n_split - 1) / n_split;
  const int kb_lo = split * per;
  const int kb_hi = min(nkb, kb_lo + per);
  // step i of this wavefront's key group works on key block kb_lo + kg + KSTEP*i;
  // with two groups the second one's last step may be the block past the
  // last, whose keys are all masked
  constexpr int KSTEP = KSPLIT ? 2 : 1;
  const int n_steps = (kb_hi - kb_lo + KSTEP - 1) / KSTEP;
  auto kb_of = [&](int i) { return kb_lo + kg + KSTEP * i; };
  const uint16_t* kbase = a.k + static_cast<size_t>(j) * a.max_seq * HD;
  const uint16_t* vbase = a.v + static_cast<size_t>(j) * a.max_seq * HD;

  // DMA: instruction q covers key rows q*RPI .. +RPI; lane -> (row, slot).
  // Row `row` of block kb is key kb*KB + row; only a block that reaches past
  // kv_end needs its keys clamped.
  const int d_row = lane / CH, d_slot = lane % CH;
  // byte offsets of this lane's DMA chunks inside a block (the block base is
  // uniform, so each copy is a scalar base plus a 32-bit vector offset)
  uint32_t k_off[PW], v_off[PW];
#pragma unroll
  for (int jj = 0; jj < PW; ++jj) {
    const int row = (wq * PW + jj) * RPI + d_row;
    k_off[jj] = row * ROWB + (d_slot ^ swz_k(row)) * 16;
    v_off[jj] = row * ROWB + (d_slot ^ swz_v(row)) * 16;
  }
  const int full_blocks = kv_end / KB;
  auto issue = [&](int i, bool is_v) __attribute__((always_inline)) {
    const int kb = kb_of(i);
    char* st = is_v ? vring + (i % SV) * TILE : kring + (i % SK) * TILE;
    const uint16_t* base = is_v ? vbase : kbase;
    if (kb < full_blocks) {
      const char* blk = reinterpret_cast<const char*>(base) + static_cast<size_t>(kb) * TILE;
#pragma unroll
      for (int jj = 0; jj < PW; ++jj)
        dma16_untracked(blk + (is_v ? v_off[jj] : k_off[jj]), st + (wq * PW + jj) * 1024);
    } else {
#pragma unroll
      for (int jj = 0; jj < PW; ++jj) {
        const int q = wq * PW + jj;
        const int row = q * RPI + d_row;
        const int key = min(kb * KB + row, kv_end - 1);
        const int sw = is_v ? swz_v(row) : swz_k(row);
        dma16_untracked(base + static_cast<size_t>(key) * HD + (d_slot ^ sw) * 8, st + q * 1024);
      }
    }
  };

  // S^T of block kb for two 32-key halves: lane (query lr) gets keys
  // 8*(r/4) + 4*lh + r%4 of each half
  auto scores = [&](int i, f32x16_t (&sc)[2]) __attribute__((always_inline)) {
    const char* Kt = kring + (i % SK) * TILE;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[hb][r] = 0.f;
      const int krow = hb * 32 + lr;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const V8 kf = *reinterpret_cast<const V8*>(
            Kt + krow * ROWB + (((ks * 2 + lh) ^ swz_k(krow)) << 4));
        sc[hb] = Ops::mma(kf, qf[ks], sc[hb]);
      }
    }
  };

  f32x16_t o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
  // Running maximum in the log2 domain (scores times log2(e)/sqrt(hd)).  It
  // is only raised when a block's maximum exceeds it by more than 8, so the
  // weights exp2(s - m_run) stay below 256 and the rescale of o and l is
  // skipped for most blocks; o / l is the same for any such reference value.
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale_log2;

  // V^T transposing reads: lane group g = lane/16 covers head dims
  // (g%2)*16 .. +16 of a 32-wide block for key half lh = g/2; source lane
  // s = lane%16 points at key row (base + s/4), dims 4*(s%4) .. +4.
  const int tr_key = (lane & 15) >> 2;                       // + key base
  const int tr_dim = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;  // + 32*db

  if (SPLIT && kb_lo >= kb_hi) {   // an empty key range: a neutral partial result
    if (q_ok) {
      const size_t pr = (static_cast<size_t>(split) * a.M + t) * a.nq + h;
      for (int d = lh; d < HD; d += 2) a.po[pr * HD + d] = 0.f;
      if (lh == 0) {
        a.pml[pr * 2] = -INFINITY;
        a.pml[pr * 2 + 1] = 0.f;
      }
    }
    return;
  }

  // prologue: K(lo), V(lo), K(lo+1) in flight; scores of block lo once K(lo)
  // landed.  Paired: K(0..2) and V(0..1), everything landed.
  issue(0, false);
  issue(0, true);
  if constexpr (PAIR) {
    if (n_steps > 1) {
      issue(1, false);
      issue(1, true);
    }
    if (n_steps > 2) issue(2, false);
    __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);
  } else if (n_steps > 1) {
    issue(1, false);
    __builtin_amdgcn_s_waitcnt(VmWait<2 * PW>::imm);
  } else {
    __builtin_amdgcn_s_waitcnt(VmWait<PW>::imm);
  }
  lds_barrier();
  // One key block: softmax of block kb from its scores s, with the scores of
  // block kb+1 computed into s_next on the way.  The loop alternates the two
  // score arrays so that no registers are copied between blocks.
  auto step = [&](int i, f32x16_t (&s)[2], f32x16_t (&s_next)[2], bool sync) __attribute__((always_inline)) {
    const int key0 = kb_of(i) * KB;
    if constexpr (PAIR) {
      // at an even step: this wave's copies of V(i), V(i+1), K(i+1), K(i+2)
      // landed, then everyone's; the slots of steps i-2 and i-1 are free
      if (sync) {
        __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);
        lds_barrier();
        if (i + 2 < n_steps) issue(i + 2, true);
        if (i + 3 < n_steps) {
          issue(i + 3, true);
          issue(i + 3, false);
        }
        if (i + 4 < n_steps) issue(i + 4, false);
      }
    } else {
      __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);   // this wave's copies of V(i), K(i+1)
      lds_barrier();   // everyone's; the V and K slots of step i-1 are free
      if (i + 1 < n_steps) issue(i + 1, true);
      if (i + 2 < n_steps) issue(i + 2, false);
    }
    // the causal mask only cuts blocks that reach past the wave's first query
    if (key0 + KB - 1 > pos_lo) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + hb * 32 + (r >> 2) * 8 + lh * 4 + (r & 3);
          s[hb][r] = key <= pos ? s[hb][r] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[hb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_blk = mx * c;   // finite in block 0: key 0 is visible to every row
    if (__ballot(m_blk > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, m_blk);
      // In the split form a lane whose query lies before the range's first
      // key has seen no key yet (m_run = m_blk = -inf) while another lane of
      // the wavefront raised the ballot: exp2(-inf - -inf) would be NaN, and
      // its o and l (still zero) need no rescale.
      const float alpha = (SPLIT || KSPLIT) && m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
    }
    // The next block's scores go to the MFMAs while this block's weights are
    // computed on the VALUs.  A wavefront issues in order, so the two streams
    // are interleaved by hand: each group below issues one K fragment read
    // for AK products ahead, one score MFMA and EX weights, and the
    // scheduling fences keep the groups in that order (the compiler places
    // the LDS waits).  The last iteration recomputes its own block, whose K
    // slot is still intact.
    const char* Kt = kring + (min(i + 1, n_steps - 1) % SK) * TILE;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s_next[hb][r] = 0.f;
    // product i: key half hb = i % 2 (two independent chains), k-step i / 2
    auto kread = [&](int i) __attribute__((always_inline)) {
      const int krow = (i % 2) * 32 + lr;
      return *reinterpret_cast<const V8*>(Kt + krow * ROWB +
                                          ((((i / 2) * 2 + lh) ^ swz_k(krow)) << 4));
    };
    constexpr int NQK = 2 * KS, AK = 4, EX = 32 / NQK;
    V8 kf[AK + 1];
#pragma unroll
    for (int i = 0; i < AK; ++i) kf[i] = kread(i);
    // (a key range of the split form may hide every key from a row so far)
    const float neg_m = (SPLIT || KSPLIT) && m_run == -INFINITY ? 0.f : -m_run;
    V8 pf[4];   // B operand of step 2*hb + half: slots (lh, e) <- r = 8*half + e
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      if (i + AK < NQK) kf[(i + AK) % (AK + 1)] = kread(i + AK);
      s_next[i % 2] = Ops::mma(kf[i % (AK + 1)], qf[i / 2], s_next[i % 2]);
#pragma unroll
      for (int e = i * EX; e < (i + 1) * EX; ++e) {
        const int hb = e / 16, r = e % 16;
        pf[hb * 2 + (r >> 3)][r & 7] = Ops::cvt(fast_exp2(fmaf(s[hb][r], c, neg_m)));
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // O^T += V^T P^T.  Slot (lh, e) of step (hb, half) is key
    // hb*32 + half*16 + 8*(e/4) + 4*lh + e%4, matching the score layout above;
    // each run of four consecutive keys is one transposing read.  Product j
    // takes head-dim block j % DB (independent chains) and step j / DB; its
    // V^T fragment is read AV products ahead.
    const char* Vt = vring + (i % SV) * TILE;
    auto vread = [&](int jj) __attribute__((always_inline)) {
      const int dim = (jj % DB) * 32 + tr_dim, st = jj / DB;
      const int r0 = (st >> 1) * 32 + (st & 1) * 16 + lh * 4 + tr_key, r1 = r0 + 8;
      const uint2 lo = lds_read_tr16(Vt + r0 * ROWB + (((dim >> 3) ^ swz_v(r0)) << 4) +
                                     (dim & 7) * 2);
      const uint2 hi = lds_read_tr16(Vt + r1 * ROWB + (((dim >> 3) ^ swz_v(r1)) << 4) +
                                     (dim & 7) * 2);
      return __builtin_bit_cast(V8, make_uint4(lo.x, lo.y, hi.x, hi.y));
    };
    constexpr int NPV = 4 * DB, AV = 2;
    V8 vf[AV + 1];
#pragma unroll
    for (int jj = 0; jj < AV; ++jj) vf[jj] = vread(jj);
    // the row sum takes the same bf16 weights the products use, two per dot2
    float psum0 = 0.f, psum1 = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 u = __builtin_bit_cast(uint4, pf[q]);
      psum0 = Ops::sum2(u.x, psum0);
      psum1 = Ops::sum2(u.y, psum1);
      psum0 = Ops::sum2(u.z, psum0);
      psum1 = Ops::sum2(u.w, psum1);
    }
    l_run += psum0 + psum1;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jj = 0; jj < NPV; ++jj) {
      if (jj + AV < NPV) vf[(jj + AV) % (AV + 1)] = vread(jj + AV);
      o[jj % DB] = Ops::mma(vf[jj % (AV + 1)], pf[jj / DB], o[jj % DB]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  f32x16_t sa[2], sb[2];
  scores(0, sa);
  int i = 0;
  for (; i + 1 < n_steps; i += 2) {
    step(i, sa, sb, true);
    step(i + 1, sb, sa, !PAIR);
  }
  if (i < n_steps) step(i, sa, sb, true);
  __builtin_amdgcn_s_waitcnt(VmWait<0>::imm);   // (every copy has landed: the last steps issue none)

  float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if constexpr (KSPLIT) {
    // Group 1 hands its reference max, weight sum and unnormalised output to
    // group 0, which rescales both to the larger max and adds them.  Group 0
    // always holds key 0, visible to every row, so its max is finite; a row
    // that saw no key of group 1's blocks has max -inf there and weight 0.
    float4* xo = reinterpret_cast<float4*>(smem);   // [DB*4][GW*64 lanes] float4
    float* xm = reinterpret_cast<float*>(smem) + DB * 16 * GW * 64;
    const int me = wq * 64 + lane;
    lds_barrier();   // every wavefront is done with the rings
    if (kg == 1) {
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          xo[(d * 4 + r4) * GW * 64 + me] = make_float4(o[d][r4 * 4 + 0], o[d][r4 * 4 + 1],
                                                        o[d][r4 * 4 + 2], o[d][r4 * 4 + 3]);
      xm[me] = m_run;
      xm[GW * 64 + me] = l_tot;
    }
    lds_barrier();
    if (kg == 1) return;
    const float m1 = xm[me], l1 = xm[GW * 64 + me];
    const float mm = fmaxf(m_run, m1);
    const float f0 = fast_exp2(m_run - mm), f1 = fast_exp2(m1 - mm);
    l_tot = l_tot * f0 + l1 * f1;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 v = xo[(d * 4 + r4) * GW * 64 + me];
        o[d][r4 * 4 + 0] = o[d][r4 * 4 + 0] * f0 + v.x * f1;
        o[d][r4 * 4 + 1] = o[d][r4 * 4 + 1] * f0 + v.y * f1;
        o[d][r4 * 4 + 2] = o[d][r4 * 4 + 2] * f0 + v.z * f1;
        o[d][r4 * 4 + 3] = o[d][r4 * 4 + 3] * f0 + v.w * f1;
      }
  }
  if (!q_ok) return;
  if constexpr (SPLIT) {
    const size_t pr = (static_cast<size_t>(split) * a.M + t) * a.nq + h;
    float* prow = a.po + pr * HD;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dd = d * 32 + r4 * 8 + lh * 4;
        *reinterpret_cast<float4*>(prow + dd) = make_float4(
            o[d][r4 * 4 + 0], o[d][r4 * 4 + 1], o[d][r4 * 4 + 2], o[d][r4 * 4 + 3]);
      }
    if (lh == 0) {
      a.pml[pr * 2] = m_run;
      a.pml[pr * 2 + 1] = l_tot;
    }
    return;
  }
  const float inv = 1.0f / l_tot;
  uint16_t* orow = a.out + static_cast<size_t>(t) * a.out_ld + h * HD;
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dd = d * 32 + r4 * 8 + lh * 4;
      uint2 w;
      w.x = pack_bf16x2(o[d][r4 * 4 + 0] * inv, o[d][r4 * 4 + 1] * inv);
      w.y = pack_bf16x2(o[d][r4 * 4 + 2] * inv, o[d][r4 * 4 + 3] * inv);
      *reinterpret_cast<uint2*>(orow + dd) = w;
    }
}

// Merge of the split-KV partial results for few (query row, head) pairs
// (decode steps): one block per pair; threads take key ranges for the max and
// the weights (block reductions), then (head dim, range group) pairs for the
// weighted sum, so the loads of different ranges are in flight together.
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_block_kernel(
    const float* __restrict__ po, const float* __restrict__ pml, int n_split, int M, int nq,
    uint16_t* __restrict__ out, int out_ld) {
  constexpr int G = 256 / HD;   // range groups of the weighted sum
  __shared__ float wgt[kAttnMaxSplits];
  __shared__ float red[4];
  __shared__ float acc_g[256];
  const int pair = blockIdx.x, tid = threadIdx.x;
  const size_t row = static_cast<size_t>(pair);
  const size_t sstride = static_cast<size_t>(M) * nq;
  float mv = -INFINITY;
  for (int sp = tid; sp < n_split; sp += 256) mv = fmaxf(mv, pml[(sp * sstride + row) * 2]);
  mv = wave_max(mv);
  if ((tid & 63) == 0) red[tid >> 6] = mv;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float lv = 0.f;
  for (int sp = tid; sp < n_split; sp += 256) {
    const float w = fast_exp2(pml[(sp * sstride + row) * 2] - m);
    wgt[sp] = w;
    lv += pml[(sp * sstride + row) * 2 + 1] * w;
  }
  const float l = block_sum<4>(lv, red);   // its barriers also publish wgt[]
  const int d = tid % HD, grp = tid / HD;
  float acc = 0.f;
#pragma unroll 8
  for (int sp = grp; sp < n_split; sp += G) acc += po[(sp * sstride + row) * HD + d] * wgt[sp];
  acc_g[tid] = acc;
  __syncthreads();
  if (tid < HD) {
    float o = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < G; ++g2) o += acc_g[g2 * HD + tid];
    out[static_cast<size_t>(pair / nq) * out_ld + (pair % nq) * HD + tid] = f32_to_bf16(o / l);
  }
}

// Merge of at most kCombineRegRanges key ranges for many (query row, head)
// pairs (prefill micro-batches over long histories): half a wavefront per
// pair, HD / 32 head dims per lane.  Every lane reads the few (max, weight
// sum) pairs itself (the half-wavefront's addresses coincide), so the merge
// needs no cross-lane reduction: with M the largest running max,
// o = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), summed over s in order.
constexpr int kCombineRegRanges = 8;
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_reg_kernel(const float* __restrict__ po,
                                                              const float* __restrict__ pml,
                                                              int n_split, int M, int nq,
                                                              uint16_t* __restrict__ out, int out_ld) {
  constexpr int DPL = HD / 32;   // head dims per lane (4 or 2)
  typedef float fv __attribute__((ext_vector_type(DPL)));
  const int pair = blockIdx.x * 8 + (threadIdx.x >> 5);   // (row, head), head fastest
  if (pair >= M * nq) return;                             // whole half-wavefronts
  const int l32 = threadIdx.x & 31;
  const size_t row = static_cast<size_t>(pair);
  const size_t sstride = static_cast<size_t>(M) * nq;
  float ms[kCombineRegRanges], ls[kCombineRegRanges];
  float m = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kCombineRegRanges; ++sp)
    if (sp < n_split) {
      const float2 v = *reinterpret_cast<const float2*>(pml + (sp * sstride + row) * 2);
      ms[sp] = v.x;
      ls[sp] = v.y;
      m = fmaxf(m, v.x);
    }
  float l = 0.f;
  fv acc = {};
#pragma unroll
  for (int sp = 0; sp < kCombineRegRanges; ++sp)
    if (sp < n_split) {
      const float w = fast_exp2(ms[sp] - m);
      l += ls[sp] * w;
      acc += *reinterpret_cast<const fv*>(po + (sp * sstride + row) * HD + l32 * DPL) * w;
    }
  const float inv = 1.0f / l;
  uint16_t* dst = out + static_cast<size_t>(pair / nq) * out_ld + (pair % nq) * HD + l32 * DPL;
  if constexpr (DPL == 4) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv),
                                                pack_bf16x2(acc[2] * inv, acc[3] * inv));
  } else {
    *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  }
}

// Merge of the split-KV partial results for many (query row, head) pairs
// (prefill micro-batches): one wavefront per pair, four per block.  With M the largest running max,
// o = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).  Lanes take key ranges
// for the max and the weight sum (wavefront reductions), then head dims
// (HD / 64 per lane) for the weighted sum of the range outputs, whose loads
// are independent of each other.
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ po,
                                                          const float* __restrict__ pml,
                                                          int n_split, int M, int nq,
                                                          uint16_t* __restrict__ out, int out_ld) {
  constexpr int DPL = HD / 64;   // head dims per lane
  __shared__ float wgt_s[4][kAttnMaxSplits];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int pair = blockIdx.x * 4 + wv;           // (row, head), head fastest
  if (pair >= M * nq) return;                     // whole wavefronts
  const size_t row = static_cast<size_t>(pair);   // (t * nq + h) inside one split
  const size_t sstride = static_cast<size_t>(M) * nq;
  float* wgt = wgt_s[wv];
  float mv = -INFINITY;
  for (int sp = lane; sp < n_split; sp += 64) mv = fmaxf(mv, pml[(sp * sstride + row) * 2]);
  const float m = wave_max(mv);
  float lv = 0.f;
  for (int sp = lane; sp < n_split; sp += 64) {
    const float w = fast_exp2(pml[(sp * sstride + row) * 2] - m);
    wgt[sp] = w;
    lv += pml[(sp * sstride + row) * 2 + 1] * w;
  }
  const float l = wave_sum(lv);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // this wavefront's LDS writes of wgt[] are done
  __builtin_amdgcn_wave_barrier();
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int sp = 0; sp < n_split; ++sp) {
    const float w = wgt[sp];
    const float* src = po + (sp * sstride + row) * HD + lane * DPL;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] += src[e] * w;
  }
  const float inv = 1.0f / l;
  uint16_t* dst = out + static_cast<size_t>(pair / nq) * out_ld + (pair % nq) * HD + lane * DPL;
#pragma unroll
  for (int e = 0; e < DPL; ++e) dst[e] = f32_to_bf16(acc[e] * inv);
}

// fp32 kernel: one block per (query token, query head); keys in chunks of
// 256 with an online softmax in fp32 using expf.
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* __restrict__ q, int q_ld,
                                                       const float* __restrict__ k_layer,
                                                       const float* __restrict__ v_layer,
                                                       float* __restrict__ out, int out_ld,
                                                       int start, int nq, int nkv, int hd,
                                                       int max_seq, float scale) {
  __shared__ float qs[128];
  __shared__ float p[256];
  __shared__ float red[4];
  const int t = blockIdx.x, h = blockIdx.y;
  const int j = h / (nq / nkv);
  const int n_keys = start + t + 1;
  const int tid = threadIdx.x;
  if (tid < hd) qs[tid] = q[static_cast<size_t>(t) * q_ld + h * hd + tid];
  __syncthreads();
  const float* kb = k_layer + static_cast<size_t>(j) * max_seq * hd;
  const float* vb = v_layer + static_cast<size_t>(j) * max_seq * hd;
  float m_run = -INFINITY, l_run = 0.f, acc = 0.f;
  for (int base = 0; base < n_keys; base += 256) {
    const int u = base + tid;
    float s = -INFINITY;
    if (u < n_keys) {
      const float* kr = kb + static_cast<size_t>(u) * hd;
      float d = 0.f;
      for (int e = 0; e < hd; ++e) d = fmaf(qs[e], kr[e], d);
      s = d * scale;
    }
    // block max
    float mx = wave_max(s);
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const float m_new = fmaxf(m_run, mx);
    const float pe = u < n_keys ? expf(s - m_new) : 0.f;
    p[tid] = pe;
    const float bs = block_sum<4>(pe, red);   // its barriers also publish p[]
    const float alpha = expf(m_run - m_new);
    l_run = l_run * alpha + bs;
    if (tid < hd) {
      float a2 = acc * alpha;
      const int cnt = min(256, n_keys - base);
      for (int uu = 0; uu < cnt; ++uu) a2 = fmaf(p[uu], vb[static_cast<size_t>(base + uu) * hd + tid], a2);
      acc = a2;
    }
    m_run = m_new;
    __syncthreads();
  }
  if (tid < hd) out[static_cast<size_t>(t) * out_ld + h * hd + tid] = acc / l_run;
}

// Blocks of the attention grid: (tiles, kv heads x head quads, waves) for M rows.
struct AttnGrid {
  int hpb, quads, waves, tiles, blocks;
};
static AttnGrid attn_grid(int M, int nq, int nkv) {
  AttnGrid g{};
  const int group = nq / nkv;
  g.hpb = group < 4 ? group : 4;
  g.quads = group / g.hpb;
  // Eight wavefronts per block (one block per CU, K/V copied into LDS once per
  // CU) when that still gives every CU a block; four (two blocks per CU)
  // otherwise.
  const int tiles8 = (M + 32 * (8 / g.hpb) - 1) / (32 * (8 / g.hpb));
  g.waves = tiles8 * nkv * g.quads >= 256 ? 8 : 4;
  const int bt = 32 * (g.waves / g.hpb);
  g.tiles = (M + bt - 1) / bt;
  g.blocks = g.tiles * nkv * g.quads;
  return g;
}

int attention_kv_splits(int M, int kv_len, int nq, int nkv) {
  const AttnGrid g = attn_grid(M, nq, nkv);
  if (g.waves != 4 || g.blocks >= 256) return 1;   // the grid already fills the GPU
  if (kv_len < 2 * M) return 1;   // keys mostly on the causal diagonal: ranges unbalanced
  const int nkb = (kv_len + 63) / 64;
  // The two-key-group form keeps its partial results in LDS; while the keys
  // are few it beats the ranges and their merge pass through memory (Llama-3
  // shape, 512 tokens from position 512: 24 against 33 µs; from 1536: 39
  // against 43; from 3584 the ranges win, 59 against 70).
  if (g.hpb % 2 == 0 && 2 * g.blocks >= 192 && 2 * g.blocks <= 256 && nkb <= 32) return 1;
  int ns = (512 + g.blocks - 1) / g.blocks;        // about 512 blocks in all
  if (ns > kAttnMaxSplits) ns = kAttnMaxSplits;
  if (ns > nkb / 4) ns = nkb / 4;                  // at least 4 key blocks per range
  return ns < 2 ? 1 : ns;
}

size_t attention_split_floats(int M, int kv_len, int nq, int nkv, int head_dim) {
  const int ns = attention_kv_splits(M, kv_len, nq, nkv);
  return ns < 2 ? 0 : static_cast<size_t>(ns) * M * nq * (head_dim + 2);
}

hipError_t launch_attention(Act act, bool kv16, const void* q, int q_ld, const void* k_layer,
                            const void* v_layer, void* out, int out_ld, int M, int start,
                            int nq, int nkv, int head_dim, int max_seq, float* split_ws,
                            size_t split_ws_floats, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (act == Act::F32) {
    dim3 grid(M, nq);
    attn_f32_kernel<<<grid, 256, 0, s>>>(
        static_cast<const float*>(q), q_ld, static_cast<const float*>(k_layer),
        static_cast<const float*>(v_layer), static_cast<float*>(out), out_ld, start, nq, nkv,
        head_dim, max_seq, 1.0f / sqrtf(static_cast<float>(head_dim)));
    return hipGetLastError();
  }
  const AttnGrid gr = attn_grid(M, nq, nkv);
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_layer);
  a.v = static_cast<const uint16_t*>(v_layer);
  a.out = static_cast<uint16_t*>(out);
  a.q_ld = q_ld;
  a.out_ld = out_ld;
  a.M = M;
  a.start = start;
  a.nq = nq;
  a.nkv = nkv;
  a.max_seq = max_seq;
  a.group = nq / nkv;
  a.hpb = gr.hpb;
  a.waves = gr.waves;
  a.tiles = gr.tiles;
  a.scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(head_dim));
  a.kv_splits = 1;
  const int ns = attention_kv_splits(M, start + M, nq, nkv);
  if (ns > 1 && split_ws &&
      static_cast<size_t>(ns) * M * nq * (head_dim + 2) <= split_ws_floats) {
    // split-KV form: partial results per key range, then one merge pass
    a.kv_splits = ns;
    a.po = split_ws;
    a.pml = split_ws + static_cast<size_t>(ns) * M * nq * head_dim;
    dim3 grid(gr.blocks * ns);
    if (kv16) {
      if (head_dim == 128) attn_fwd_bf16_kernel<128, 4, true, true><<<grid, 256, 0, s>>>(a);
      else attn_fwd_bf16_kernel<64, 4, true, true><<<grid, 256, 0, s>>>(a);
    } else {
      if (head_dim == 128) attn_fwd_bf16_kernel<128, 4, true, false><<<grid, 256, 0, s>>>(a);
      else attn_fwd_bf16_kernel<64, 4, true, false><<<grid, 256, 0, s>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int pairs = M * nq;
    if (pairs < 1024) {   // few pairs: a whole block per pair
      if (head_dim == 128)
        attn_combine_block_kernel<128><<<pairs, 256, 0, s>>>(a.po, a.pml, ns, M, nq, a.out, out_ld);
      else
        attn_combine_block_kernel<64><<<pairs, 256, 0, s>>>(a.po, a.pml, ns, M, nq, a.out, out_ld);
    } else if (ns <= kCombineRegRanges) {   // few ranges: half a wavefront per pair
      const int cblocks = (pairs + 7) / 8;
      if (head_dim == 128)
        attn_combine_reg_kernel<128><<<cblocks, 256, 0, s>>>(a.po, a.pml, ns, M, nq, a.out, out_ld);
      else
        attn_combine_reg_kernel<64><<<cblocks, 256, 0, s>>>(a.po, a.pml, ns, M, nq, a.out, out_ld);
    } else {
      const int cblocks = (pairs + 3) / 4;
      if (head_dim == 128)
        attn_combine_kernel<128><<<cblocks, 256, 0, s>>>(a.po, a.pml, ns, M, nq, a.out, out_ld);
      else
        attn_combine_kernel<64><<<cblocks, 256, 0, s>>>(a.po, a.pml, ns, M, nq, a.out, out_ld);
    }
    return hipGetLastError();
  }
  // A grid that leaves at least half of the CUs idle (short micro-batches
  // over short histories) takes the two-key-group form: each block holds half
  // as many query heads in two wavefront groups that split the key blocks, so
  // there are twice the blocks and the longest chain of key blocks is halved.
  const bool ksplit = gr.waves == 4 && gr.blocks * 2 <= 256 && gr.hpb % 2 == 0;
  if (ksplit) a.hpb = gr.hpb / 2;
  dim3 grid(ksplit ? gr.blocks * 2 : gr.blocks);
#define TLP_ATTN(HD_, KV_)                                                                  \
  if (ksplit) attn_fwd_bf16_kernel<HD_, 4, false, KV_, true><<<grid, 256, 0, s>>>(a);       \
  else if (a.waves == 8) attn_fwd_bf16_kernel<HD_, 8, false, KV_><<<grid, 512, 0, s>>>(a);  \
  else attn_fwd_bf16_kernel<HD_, 4, false, KV_><<<grid, 256, 0, s>>>(a);
  if (head_dim == 128) {
    if (kv16) { TLP_ATTN(128, true) } else { TLP_ATTN(128, false) }
  } else {
    if (kv16) { TLP_ATTN(64, true) } else { TLP_ATTN(64, false) }
  }
#undef TLP_ATTN
  return hipGetLastError();
}

}  // namespace tlp
