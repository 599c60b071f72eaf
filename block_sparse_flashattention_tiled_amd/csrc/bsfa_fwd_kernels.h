// Block-sparse FlashAttention prefill forward kernel for gfx950 (MI355X).
//
// Operation: "Block Sparse Flash Attention" (paperpeel.com/paper/2512.07011).
// FlashAttention-2's tiled online softmax (App. B.2 steps (1)-(6)) with one
// gate per score tile (Sec. 4.1, 4.4): after S_ij = Q_i K_j^T / sqrt(d) is
// formed, its maximum over visible entries is compared with the threshold of
// (head, query block); an off-diagonal tile below it is skipped before any of
// its V rows is requested, and contributes nothing to the running max, sum
// or output.  Diagonal tiles always pass (Sec. 4.1); causal tiles above the
// diagonal are never visited (App. B.2).
//
// Tiles are B_M query rows by B_N keys (both 64 or 128).  The diagonal tiles of
// query block i - the ones that bypass the gate - are the key blocks whose
// positions overlap the query block's: j = i for square tiles, and for
// B_M != B_N every j with j B_N < (i+1) B_M and (j+1) B_N > i B_M.
//
// One kernel runs two query units per workgroup on one K/V stream: two query
// heads of a KV group on one query block, or two neighbouring query blocks of
// one head (an odd group's last head, multi-head attention, bidirectional
// attention with an odd group); every shape is served that way.
//
// Mapping onto CDNA4:
//  * 2 B_M/32 waves per workgroup, B_M/32 per unit; wave w of a unit owns its
//    query rows [32w, 32w+32); two waves share each SIMD;
//  * both contractions run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//    Scores are formed transposed, S^T = K Q^T, so that each lane ends up
//    holding one query row: its row statistics stay in-lane and the score
//    registers, exponentiated and rounded to bf16, are directly the B operand
//    of O^T = V^T P^T (both operands use the same k-slot order);
//  * Q lives in registers for the whole key loop (B.2 step (1));
//  * K goes straight from memory into LDS (buffer loads with an LDS
//    destination), two K tiles in turn: K_{j+2} is requested into K_j's tile
//    right after the barrier that follows S_j, and published by the same
//    barrier one step later;
//  * V_j is requested only after tile j passed its gate, straight into LDS;
//    its loads overlap the softmax of the tile.  The A operand of
//    O^T = V^T P^T needs V transposed: it is read with ds_read_b64_tr_b16,
//    whose 16-lane groups return a 4x16 block transposed.  The V tile is
//    XOR-swizzled so those reads are bank-conflict free;
//  * the tile maximum is reduced in-lane, across the wave with shuffles and
//    across waves through LDS; the skip decision is read back into a scalar
//    register so the branch is uniform for the workgroup;
//  * the running output is rescaled lazily: only when a row maximum grows by
//    more than 2^4 (exact: O and l always refer to the same reference max),
//    and l sums the bf16-rounded P~ that multiplies V;
//  * barriers wait for LDS instructions only, so direct-to-LDS loads stay in
//    flight across them: a wave waits for its own before the barrier that
//    publishes the tile.  The second barrier of a step is taken only when some
//    unit keeps a tile of it;
//  * the softmax and P.V run in two halves of the step's keys,
//    and after the second barrier the two units take the second half in
//    opposite orders, so that one wave's P.V overlaps the other wave's
//    exponentials on the same SIMD;
//  * workgroups are ordered heaviest query block first (causal) and, when the
//    grid allows, remapped for the XCDs' L2s: head pairs so that the query
//    heads of one KV group run back to back on the same XCD; block pairs so
//    that each XCD runs whole query heads, their block pairs back to back.
//    Either way the workgroups resident on an XCD share K_j/V_j in its L2.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "bsfa_internal.h"

namespace bsfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D, int BM, int BN>
struct Cfg {
  static constexpr int KC = D / 16;          // 16-wide d chunks of the QK^T contraction
  static constexpr int KB = BN / 32;         // 32-key sub-blocks of a tile
  static constexpr int PC = BN / 16;         // 16-key chunks of the P.V contraction
  static constexpr int DB = D / 32;          // 32-wide d sub-blocks of the output
  static constexpr int CPR = D / 8;          // 16-byte chunks per K / V row
  // diagonal tiles of a query block when both sides divide N: B_M / B_N for
  // tall tiles, else one (a query block lies inside one key block)
  static constexpr int ND = BM > BN ? BM / BN : 1;
};

// Diagonal key blocks of query block i: [first, last], the key blocks whose
// positions overlap the query block's (m_kv = key blocks of the sequence).
template <int BM, int BN>
__device__ __forceinline__ int diag_first(int i) {
  return (i * BM) / BN;
}
template <int BM, int BN>
__device__ __forceinline__ int diag_last(int i, int m_kv) {
  return min(((i + 1) * BM - 1) / BN, m_kv - 1);
}

// 16-byte chunk position of logical chunk cc of V row `row`: XOR with a
// function of the row so that the transposing reads (4 rows x 4 chunks per
// 32 lanes) hit 64 distinct banks.
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

// Cross-lane reductions in the VALU (no LDS round trip).  Lanes l and l ^ 32
// hold the two halves of one score row; v_permlane32_swap exchanges lanes 32-63
// of its first operand with lanes 0-31 of its second, v_permlane16_swap the odd
// 16-lane rows of the first with the even rows of the second.  Applied to a
// value and a copy of it, the first result holds the lower lanes (rows) twice
// and the second the upper ones.  The swaps are written in inline asm: through
// the builtins the compiler folds a maximum of the two results into the first
// one alone.  Each asm block makes the copy itself and waits the two cycles a
// VALU write needs before a permlane instruction reads the register.
__device__ __forceinline__ void swap_halves(float x, float& lo, float& hi) {
  unsigned a = __builtin_bit_cast(unsigned, x), b;
  asm volatile("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "=&v"(b));
  lo = __builtin_bit_cast(float, a);
  hi = __builtin_bit_cast(float, b);
}
__device__ __forceinline__ void swap_rows(float x, float& even, float& odd) {
  unsigned a = __builtin_bit_cast(unsigned, x), b;
  asm volatile("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "=&v"(b));
  even = __builtin_bit_cast(float, a);
  odd = __builtin_bit_cast(float, b);
}
// Maximum that propagates NaN (IEEE maximum, v_maximum3_f32 on gfx950): unlike
// fmaxf it needs no canonicalisation of operands that come from MFMA, DPP or
// LDS, and a NaN score makes the tile maximum NaN, as a plain max does.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max / sum over lanes l and l ^ 32
__device__ __forceinline__ float max_halves(float x) {
  float a, b;
  swap_halves(x, a, b);
  return vmax(a, b);
}
__device__ __forceinline__ float sum_halves(float x) {
  float a, b;
  swap_halves(x, a, b);
  return a + b;
}
// Maximum over the wave of a value that already agrees between lanes l and
// l ^ 32: within each 16-lane row by DPP (lane ^ 1, lane ^ 2, rotations by 4
// and 8), then across rows by v_permlane16_swap.
__device__ __forceinline__ float wave_max_sym(float x) {
  x = vmax(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false)));
  x = vmax(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false)));
  x = vmax(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false)));
  x = vmax(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false)));
  float e, o;
  swap_rows(x, e, o);
  return vmax(e, o);
}

// Gate of one query unit for tile j (a5).  Threshold gate (the pages'
// method, "Block Sparse Flash Attention" Sec. 4.1 and 4.4): an off-diagonal
// tile is skipped iff s_max < tau, strictly.  Gap gate (the comparison
// reference of BLASST and of SpargeAttention's in-kernel P.V skip, Sec. 3
// "Related Work": a tile far below the running maximum): skipped iff
// s_max < M - tau, where M is the largest s_max among the unit's tiles kept so
// far.  Both compare in the scaled-score domain; NaN compares false (kept).
__device__ __forceinline__ int gate_skip(int gap, bool off_diag, float tms, float tau, float& mrun) {
  const float ref = gap ? mrun - tau : tau;
  const int skip = (off_diag && tms < ref) ? 1 : 0;
  if (!skip) mrun = fmaxf(mrun, tms);
  return skip;
}

// (a9) one lane's share of an output row O = O_acc / l: four runs of four
// consecutive columns per 32-column block, fp32, or rounded to bf16 (nearest
// even) when the caller asked for a bf16 output.
template <int DB>
__device__ __forceinline__ void store_out_row(const FwdParams& p, size_t row, const f32x16 (&o)[DB], float inv,
                                              int hh) {
  constexpr int D = DB * 32;
  if (p.out_bf16) {
    uint16_t* ob = p.out_bf16 + row * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x2 lo = {o[db][4 * g4 + 0] * inv, o[db][4 * g4 + 1] * inv};
        const f32x2 hi = {o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv};
        uint2 val;
        val.x = __builtin_bit_cast(unsigned, __builtin_convertvector(lo, bf16x2));
        val.y = __builtin_bit_cast(unsigned, __builtin_convertvector(hi, bf16x2));
        *reinterpret_cast<uint2*>(ob + db * 32 + 8 * g4 + 4 * hh) = val;
      }
    return;
  }
  float* og = p.out + row * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      float4 val;
      val.x = o[db][4 * g4 + 0] * inv;
      val.y = o[db][4 * g4 + 1] * inv;
      val.z = o[db][4 * g4 + 2] * inv;
      val.w = o[db][4 * g4 + 3] * inv;
      *reinterpret_cast<float4*>(og + db * 32 + 8 * g4 + 4 * hh) = val;
    }
}

// Sequences whose length N is not a multiple of the tile: the last query and
// key blocks are partial, and positions >= N do not exist (masked, not padded).
// Loads of rows past the end read the last row instead, so that every load
// stays inside the tensor; mask_tail sets the scores of query rows >=
// rows_left and of keys >= keys_left (both relative to the tile) to -inf, so
// the values read there never reach a maximum, a sum or an output.
template <int NKB>
__device__ __forceinline__ void mask_tail(f32x16 (&s)[NKB], int qloc, int hh, int rows_left, int keys_left) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // -inf added (arithmetically, no compare masks) iff the row or the key
      // lies past the end
      const int key = kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
      const unsigned pen = (unsigned)(((rows_left - 1 - qloc) | (keys_left - 1 - key)) >> 31) & 0xFF800000u;
      s[kb][r] += __builtin_bit_cast(float, pen);
    }
}

// Causal masking inside a diagonal tile: key `key` of the tile (position
// j B_N + key) is hidden from query row qloc (position i B_M + qloc) iff
// key > qloc + off, off = i B_M - j B_N.
template <int NKB>
__device__ __forceinline__ void mask_causal(f32x16 (&s)[NKB], int qloc, int hh, int off) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (key > qloc + off) s[kb][r] = -INFINITY;
    }
}

// The same mask by integer arithmetic, for code where the compare masks of
// mask_causal would cost registers: -inf is added to the score of a hidden
// key, 0 to a visible one (exact for finite scores).
template <int NKB>
__device__ __forceinline__ void mask_causal_alu(f32x16 (&s)[NKB], int qloc, int hh, int off) {
  const int lim = qloc + off - 4 * hh;  // hidden iff kb*32 + 8(r/4) + r%4 > lim
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kc = kb * 32 + 8 * (r >> 2) + (r & 3);
      const unsigned pen = (unsigned)((lim - kc) >> 31) & 0xFF800000u;  // -inf iff kc > lim, else +0
      s[kb][r] += __builtin_bit_cast(float, pen);
    }
}

// ---------------------------------------------------------------------------
// The kernel: one workgroup of 2*B_M/32 waves runs two query units that read
// the same K/V stream - two query heads of one KV group on the same query
// block, or two neighbouring query blocks of one head.  Two waves share each
// SIMD; every wave keeps its 32 rows of Q in registers, and
// K_j is loaded once for both units, straight into LDS, two steps ahead into
// one of two K tiles.  Each unit keeps its own gate,
// statistics and output; V_j is requested when at least one unit keeps tile j
// and a unit that skipped the tile neither reads it nor updates anything.
// ---------------------------------------------------------------------------
template <int D, int BM, int BN>
struct PairCfg {
  using C = Cfg<D, BM, BN>;
  static constexpr int NWU = BM / 32;               // waves per unit
  static constexpr int NW = 2 * NWU;                // waves per workgroup
  static constexpr int NT = NW * 64;                // threads per workgroup
};

// 16 bytes per lane from a buffer (base, size in bytes; lane and scalar byte
// offsets) straight into LDS at dst + 16 * lane.
__device__ __forceinline__ void buffer_load_lds16(const void* base, int bytes, char* dst, int voff, int soff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

// The XCD (one of the eight compute dies) the wave runs on: bits 3:0 of the
// XCC_ID hardware register (register 20).
__device__ __forceinline__ int xcd_id() { return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 7; }

// Next work item of a persistent launch over n items.  Queue x holds the
// items L < n with L % 8 == x in increasing order - the share of the static
// grid that would run on XCD x, heaviest first.  A workgroup takes from the
// front of its own XCD's queue and, once that is empty, from the back of the
// others in turn, where their lightest items are, so that what moves between
// XCDs at the end is short.  work[x] packs the items taken from queue x's
// front (high 32 bits) and back (low 32 bits); one 64-bit atomic add both
// claims a position and reads how many were claimed before it, so a claim is
// valid exactly when the claims before it (from either end) leave an item,
// and the valid claims cover the queue once.  Returns -1 once every queue is
// empty; counts only grow, so an empty queue stays empty.
__device__ __forceinline__ int next_item(unsigned long long* work, int n, int xcd) {
  for (int t = 0; t < 8; ++t) {
    const int x = (xcd + t) & 7;
    const int nq = (n - x + 7) >> 3;
    if (nq <= 0) continue;
    const unsigned long long old = atomicAdd(work + x, t == 0 ? (1ull << 32) : 1ull);
    const int front = (int)(old >> 32), back = (int)(old & 0xffffffffu);
    if (front + back < nq) return (t == 0 ? front : nq - 1 - back) * 8 + x;
  }
  return -1;
}

// Chunk swizzle of a dense K tile in LDS (2D bytes per row): logical 16-byte
// chunk cc of row `row` sits at position cc ^ k_swz(row), so that 16
// consecutive rows read at one logical chunk hit distinct banks.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}

// Workgroup barrier over the LDS accesses of LDS instructions (lgkmcnt):
// direct-to-LDS loads stay in flight across it.  The memory clobber keeps the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier_keep_dma() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait until this wave's vector-memory operations, direct-to-LDS loads
// included, have completed (vmcnt(0); the LDS and export counters untouched).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// S^T = K Q^T with this wave's Q fragments in registers and K from a dense,
// swizzled tile.  The MFMAs go in pairs (chunk c, key blocks 2h and 2h + 1),
// each pair's two K fragments requested two pairs ahead of their use, so that
// the LDS latency runs under four MFMAs instead of stalling the next one.
template <int D, int BM, int BN, int NKB, int NKC>
__device__ __forceinline__ void qk_tile_swz(f32x16 (&s)[NKB], const char* ks, int l32, int hh,
                                            const bf16x8 (&qf)[NKC]) {
  using C = Cfg<D, BM, BN>;
  static_assert(NKB == C::KB && NKC == C::KC, "fragment sizes");
  static_assert(C::KB % 2 == 0 && C::KC * C::KB >= 4, "pairs of key blocks, at least two pairs");
  // Chunk 2c + hh of row l32 (rows kb*32 + l32 share the swizzle x) sits at
  // byte l32 2D + ((2c + hh) ^ x) 16 = bx ^ 32c: the row, the bit of hh and
  // the bits of c occupy disjoint address bits.  bx is made opaque so that
  // the addresses are formed at each use rather than held in registers.
  const int x = k_swz<D>(l32);
  int bx = l32 * (2 * D) + ((hh ^ (x & 1)) << 4) + ((x & ~1) << 4);
  asm volatile("" : "+v"(bx));
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) s[kb] = f32x16{};
  constexpr int NP = C::KC * C::KB / 2;  // MFMA pairs
  auto frag = [&](int q, int e) __attribute__((always_inline)) {
    const int c = q / (C::KB / 2), h = q % (C::KB / 2);
    return *reinterpret_cast<const bf16x8*>(ks + (bx ^ (c << 5)) + (2 * h + e) * 32 * 2 * D);
  };
  bf16x8 a0 = frag(0, 0), a1 = frag(0, 1), b0 = frag(1, 0), b1 = frag(1, 1);
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    bf16x8 n0, n1;
    if (q + 2 < NP) {
      n0 = frag(q + 2, 0);
      n1 = frag(q + 2, 1);
    }
    const int c = q / (C::KB / 2), h = q % (C::KB / 2);
    s[2 * h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[c], s[2 * h], 0, 0, 0);
    s[2 * h + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[c], s[2 * h + 1], 0, 0, 0);
    a0 = b0;
    a1 = b1;
    if (q + 2 < NP) {
      b0 = n0;
      b1 = n1;
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the reads two pairs ahead first
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);    // then this pair's MFMAs
    __builtin_amdgcn_sched_barrier(0);
  }
}

// HEADPAIR: units are query heads 2hp, 2hp+1 of a KV group (same query block);
// otherwise (bidirectional only) query blocks 2ip, 2ip+1 of one head.
template <int D, int BM, int BN, bool CAUSAL, bool DIAG_OUT, bool MAXONLY, bool HEADPAIR, bool RAGGED>
__global__ void __launch_bounds__(BM * 4) __attribute__((amdgpu_waves_per_eu(2, 2)))
    bsfa_fwd_pair_kernel(const FwdParams p) {
  // Key tiles per step: 128 x 64 tiles are processed two per 128-key step, so
  // the barriers and the MFMA sequence are those of 128 x 128 tiles, while each
  // 64-key tile keeps its own gate, V request, softmax and P.V.
  constexpr int SUB = (BM == 128 && BN == 64) ? 2 : 1;
  constexpr int KN = SUB * BN;  // keys per step
  using C = Cfg<D, BM, KN>;
  using P2 = PairCfg<D, BM, KN>;
  constexpr int KBS = C::KB / SUB;      // 32-key sub-blocks per key tile
  constexpr int PCS = C::PC / SUB;      // 16-key P.V chunks per key tile
  static_assert(C::ND == 1, "the causal diagonal fills one step");
  // K (two buffers) and V tiles in LDS: dense rows of 2D bytes with swizzled
  // 16-byte chunks, filled by direct-to-LDS loads of 1 KB per instruction
  constexpr int TILE_BYTES = KN * D * 2;
  constexpr int DMA = TILE_BYTES / (P2::NW * 1024);  // load instructions per wave and tile
  static_assert(DMA * P2::NW * 1024 == TILE_BYTES, "tile loads split evenly over the waves");
  static_assert(SUB == 1 || BN % (64 / C::CPR) == 0, "a load instruction stays inside one key tile");
  __shared__ __attribute__((aligned(16))) char k_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char k_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char v_lds[TILE_BYTES];
  __shared__ float red[2][2][P2::NWU][SUB];  // [step parity][unit][wave][key tile]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int u = w / P2::NWU;   // unit of this wave
  const int wu = w % P2::NWU;  // wave inside the unit
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- work item (a1): workgroup -> (b, KV group, two units) --------------
  const int per_group = HEADPAIR ? p.pair_hn / 2 : p.pair_hn;  // workgroups per KV group and block (pair)
  int L = blockIdx.x;
  const int n_pairs = (p.M + 1) / 2;  // block pairs per query head
  int lp = 0;                         // block pairs: pair index in launch order
  if (HEADPAIR) {
    if (p.remap) {
      const int x = L & 7;
      const int pp = L >> 3;
      L = ((pp / per_group) * 8 + x) * per_group + (pp % per_group);
    }
  } else if (p.remap) {
    // each XCD runs whole query heads, one after the other, their block pairs
    // back to back: the workgroups resident on an XCD stream one head's K/V
    const int x = L & 7;
    const int r = L >> 3;
    lp = r % n_pairs;
    L = (r / n_pairs) * 8 + x;
  } else {
    lp = L / (p.B * p.Hkv * per_group);
  }
  const int hin = L % per_group;
  L /= per_group;
  const int g = L % p.Hkv;
  L /= p.Hkv;
  const int b = L % p.B;
  L /= p.B;
  int hq_u[2], i_u[2];
  if (HEADPAIR) {
    const int i = CAUSAL ? (p.M - 1 - L) : L;  // causal: heaviest query blocks first
    hq_u[0] = g * p.G + p.pair_h0 + 2 * hin;
    hq_u[1] = hq_u[0] + 1;
    i_u[0] = i_u[1] = i;
  } else {
    const int ip = CAUSAL ? (n_pairs - 1 - lp) : lp;  // causal: heaviest block pairs first
    hq_u[0] = hq_u[1] = g * p.G + p.pair_h0 + hin;
    i_u[0] = 2 * ip;
    i_u[1] = 2 * ip + 1;
  }
  const int hq = hq_u[u];
  const int i = i_u[u];
  // Per-sequence length, clamped to [0, N]: query blocks past it exit before
  // the first barrier.  A block pair whose second block lies past the end
  // (per-sequence lengths, or an odd number of query blocks) keeps that unit
  // running through the barriers; it writes nothing
  const int n_seq = (RAGGED && p.seq_lens) ? min(max(p.seq_lens[b], 0), p.N) : p.N;
  const int m_seq = RAGGED ? (n_seq + BM - 1) / BM : p.M;
  const int mkv_seq = RAGGED ? (n_seq + BN - 1) / BN : p.Mkv;
  if (RAGGED && i_u[0] >= m_seq) return;  // both units past the end (i_u[0] <= i_u[1])
  const bool live = !RAGGED || i < m_seq;
  const size_t q_head = (size_t)(b * p.Hq + hq) * p.N;
  const size_t kv_head = (size_t)(b * p.Hkv + g) * p.N;
  const int qloc = 32 * wu + l32;
  const int qrow = i * BM + qloc;
  const int v_row = 4 * hh + ((lane & 15) >> 2);
  const int v_col = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int v_half = (lane & 1) * 8;

  // ---- (a2) Q: this wave's 32 rows stay in registers as MFMA B fragments ------
  // (a row past the end of the sequence reads the last row; it is masked)
  bf16x8 qf[C::KC];
  {
    const int qr = RAGGED ? min(qrow, n_seq - 1) : qrow;
    const bf16x8* qsrc = reinterpret_cast<const bf16x8*>(p.q) + (q_head + qr) * (D / 8) + hh;
#pragma unroll
    for (int c = 0; c < C::KC; ++c) qf[c] = qsrc[2 * c];
  }
  const u32x4* kg = reinterpret_cast<const u32x4*>(p.k) + kv_head * C::CPR;
  const u32x4* vg = reinterpret_cast<const u32x4*>(p.v) + kv_head * C::CPR;

  float tau_u[2];
#pragma unroll
  for (int uu = 0; uu < 2; ++uu)
    tau_u[uu] = MAXONLY ? INFINITY : p.thresholds[hq_u[uu] * p.T_len + min(i_u[uu], p.T_len - 1)];
  const float c2 = p.scale_log2;
  // diagonal key blocks of each unit.  Under causal masking a head pair shares
  // its query block; in a block pair the second unit's diagonal comes later,
  // and tiles past the first unit's diagonal do not exist for it
  int jd0_u[2], jd1_u[2];
#pragma unroll
  for (int uu = 0; uu < 2; ++uu) {
    jd0_u[uu] = diag_first<BM, BN>(i_u[uu]);
    jd1_u[uu] = diag_last<BM, BN>(i_u[uu], mkv_seq);
  }
  const int jend = CAUSAL ? jd1_u[1] : mkv_seq - 1;  // last computed key tile (of either unit)
  const int send = jend / SUB;                        // last step
  const size_t diag_row = ((size_t)(b * p.Hq + hq) * p.M + i) * p.Mkv;

  f32x16 o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  float lb_run = 0.f;
  float mrun_u[2] = {-INFINITY, -INFINITY};  // per unit: largest s_max of its kept tiles (gap gate)
  int nskip = 0;

  // Direct-to-LDS load of the K or V tile of the step whose first key is row0:
  // instruction n of wave w fills the 1 KB of chunks (w DMA + n) 64 .. + 63,
  // lane l the chunk at position l of them, with the logical chunk that the
  // swizzle puts there.  tmask: the step's key tiles to load.  Buffer loads:
  // the head's K or V is the buffer (its range is the head's own rows), the
  // tile's first row a scalar offset, the chunk a 32-bit lane offset.
  const int ws = __builtin_amdgcn_readfirstlane(w);
  auto dma_tile = [&](char* dst, const u32x4* head, int row0, bool is_k, int tmask) {
    // with tails, the lane offsets are formed here at each call rather than
    // kept across the loop (registers)
    int ln = lane;
    if constexpr (RAGGED) asm volatile("" : "+v"(ln));
#pragma unroll
    for (int n = 0; n < DMA; ++n) {
      const int chunk0 = (ws * DMA + n) * 64;
      if (SUB > 1 && !((tmask >> ((chunk0 / C::CPR) / BN)) & 1)) continue;
      const int slot = chunk0 + ln;
      const int row = slot / C::CPR;
      const int cc = (slot % C::CPR) ^ (is_k ? k_swz<D>(row) : v_swz<D>(row));
      const int rrow = RAGGED ? min(row, n_seq - 1 - row0) : row;  // rows past the end read the last row
      buffer_load_lds16(head, p.N * D * 2, dst + chunk0 * 16, (rrow * C::CPR + cc) * 16, row0 * (C::CPR * 16));
    }
  };
  // K_js lives in buffer (js + par) & 1, so that the last step reads k_lds0
  // and every buffer choice is known at compile time
  const int par = send & 1;
  if (par) dma_tile(k_lds1, kg, 0, true, (1 << SUB) - 1);
  else dma_tile(k_lds0, kg, 0, true, (1 << SUB) - 1);
  wait_vmem();
  lds_barrier_keep_dma();  // K_0 visible
  // K_1 (published by barrier (b) of step 0)
  if (send >= 1) {
    if (par) dma_tile(k_lds0, kg, KN, true, (1 << SUB) - 1);
    else dma_tile(k_lds1, kg, KN, true, (1 << SUB) - 1);
  }

  // Barriers per step.  (b) follows S_js and each wave's wait for its own
  // K_{js+1} loads: the tile maxima and K_{js+1} are complete, every wave is
  // done with K_js (whose tile then receives K_{js+2}) and, by program order,
  // with the previous step's P.V, so V_js may be loaded into LDS.  (c) follows
  // each wave's wait for its V_js loads and publishes them; it is taken only
  // when some unit keeps a tile of the step (the same decision in every wave),
  // so a step that both units skip has one barrier.  The tile maxima are
  // exchanged through one of two slots by step parity, so a wave that runs
  // ahead into the next step never overwrites maxima another wave still reads.

  // One step: key tiles SUB*js .. SUB*js + SUB - 1.  DIAGC is true only for the
  // causal diagonal step, the last visited, so the masking of keys after the
  // query is compiled into those steps and not evaluated (or predicated) on
  // every other step.
  auto step = [&](const int js, auto DIAGC, auto KBUF) {
    constexpr bool DIAG_TILE = decltype(DIAGC)::value;
    char* const k_cur = decltype(KBUF)::value ? k_lds1 : k_lds0;  // K_js
    // ---- (a4) S^T = K Q^T over the step's keys -------------------------------
    f32x16 s[C::KB];
    qk_tile_swz<D, BM, KN>(s, k_cur, l32, hh, qf);
    if constexpr (CAUSAL && DIAG_TILE) {
      mask_causal(s, qloc, hh, i * BM - js * KN);
    } else if constexpr (CAUSAL && !HEADPAIR && decltype(KBUF)::value == 1) {
      // causal block pair: the first unit's diagonal may fall one step before
      // the last (the step before the last always reads buffer 1)
      if (js == send - 1 && js >= jd0_u[0] / SUB) mask_causal_alu(s, qloc, hh, i * BM - js * KN);
    }
    if constexpr (RAGGED) {
      const int rows_left = n_seq - i * BM, keys_left = n_seq - js * KN;
      if (rows_left < BM || keys_left < KN) mask_tail(s, qloc, hh, rows_left, keys_left);
    }
    // ---- (a5) tile maxima of both units and their gates ---------------------
    float rm_t[SUB];  // this lane's row maximum over each key tile of the step
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
      float rm0 = -INFINITY, rm1 = -INFINITY;
#pragma unroll
      for (int kb = t * KBS; kb < (t + 1) * KBS; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          rm0 = vmax(rm0, s[kb][r]);
          rm1 = vmax(rm1, s[kb][r + 1]);
        }
      float rm = vmax(rm0, rm1);
      rm = max_halves(rm);
      rm_t[t] = rm;
      float wm;
      if (!DIAG_OUT && !MAXONLY && p.gate == 0) {
        // threshold gate, no tile maxima written: the gate needs only whether
        // some row's scaled maximum is not below tau (rounding of the positive
        // scale is monotone, so this is the decision the tile maximum gives,
        // NaN included).  Each wave publishes its vote as +inf or -inf.
        const bool keep = !(rm * p.scale < (u ? tau_u[1] : tau_u[0]));
        wm = __builtin_amdgcn_ballot_w64(keep) ? INFINITY : -INFINITY;
      } else {
        wm = wave_max_sym(rm);
      }
      if (lane == 0) red[decltype(KBUF)::value][u][wu][t] = wm;
    }
    wait_vmem();             // this wave's loads of K_{js+1} have landed
    lds_barrier_keep_dma();  // (b): maxima and K_{js+1} complete; every wave is done with S_js and
                             // with P.V of the previous step
    // K_{js+2} -> K_js's tile, published by barrier (b) of the next step
    if (!(CAUSAL && DIAG_TILE) && js + 2 <= send) dma_tile(k_cur, kg, (js + 2) * KN, true, (1 << SUB) - 1);
    // gates in increasing key-tile order (the gap gate's running maximum)
    int skip_of[2][SUB];
    bool ex_of[2][SUB];
#pragma unroll
    for (int uu = 0; uu < 2; ++uu)
#pragma unroll
      for (int t = 0; t < SUB; ++t) {
        const int j = js * SUB + t;
        // the last step may hold a tile past the end; under causal masking a
        // tile past the unit's diagonal is not computed for it
        const bool exists = (SUB == 1 || j < mkv_seq) && (!CAUSAL || HEADPAIR || j <= jd1_u[uu]);
        ex_of[uu][t] = exists;
        float tm = red[decltype(KBUF)::value][uu][0][t];
#pragma unroll
        for (int ww = 1; ww < P2::NWU; ++ww) tm = vmax(tm, red[decltype(KBUF)::value][uu][ww][t]);
        const float tms = tm * p.scale;
        const bool on_diag = j >= jd0_u[uu] && j <= jd1_u[uu];
        skip_of[uu][t] = (MAXONLY || !exists) ? 1 : gate_skip(p.gate, !on_diag, tms, tau_u[uu], mrun_u[uu]);
        if (DIAG_OUT && exists && uu == u && wu == 0 && lane == 0 && live) {
          if (p.tile_state) p.tile_state[diag_row + j] = on_diag ? 3 : (skip_of[uu][t] ? 2 : 1);
          if (p.tile_max) p.tile_max[diag_row + j] = tms;
        }
      }
    // kmask: key tiles this unit keeps; vmask: key tiles some unit keeps
    int km = 0, vm = 0, ns = 0;
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
      const int mine = u ? skip_of[1][t] : skip_of[0][t];
      km |= (mine ? 0 : 1) << t;
      vm |= ((skip_of[0][t] & skip_of[1][t]) ? 0 : 1) << t;
      ns += (mine && (u ? ex_of[1][t] : ex_of[0][t])) ? 1 : 0;
    }
    const int kmask = __builtin_amdgcn_readfirstlane(km);
    const int vmask = __builtin_amdgcn_readfirstlane(vm);
    nskip += ns;  // (a6)
    // ---- (a8) V of the step's key tiles that some unit keeps -> LDS -----------
    if (vmask) dma_tile(v_lds, vg, js * KN, false, vmask);
    bf16x8 pf[C::PC];
    // ---- (a7) online softmax over the kept key tiles, in two halves of the
    // step's keys ----------------------------------------------------------
    // O and l refer to the reference max m_run; it is raised (and O, l
    // rescaled) only when a row maximum exceeds it by more than 2^4, so
    // P~ <= 16.  The output is normalised by the sum of the same bf16-rounded
    // P~ that multiplies V, so the weights of a row normalise exactly; lse
    // uses the fp32 sum.
    // l sums the fp32 values, lb the bf16 ones over four independent chains,
    // in the same order as bsfa_fwd_pipe_kernel (the two give identical bits)
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float rs0 = 0.f, rs1 = 0.f;
    float rb[4] = {0.f, 0.f, 0.f, 0.f};
    auto softmax_half = [&](int h) {
#pragma unroll
      for (int kb = h * (C::KB / 2); kb < (h + 1) * (C::KB / 2); ++kb) {
        if (SUB > 1 && !((kmask >> (kb / KBS)) & 1)) continue;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int r = 0; r < 8; r += 2) {
            f32x2 pr;
            pr[0] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hf + r], c2, -m_run));
            pr[1] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hf + r + 1], c2, -m_run));
            const bf16x2 pb = __builtin_convertvector(pr, bf16x2);
            rs0 += pr[0];
            rs1 += pr[1];
            rb[(r >> 1) & 3] = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, rb[(r >> 1) & 3], false);
            pf[2 * kb + hf][r] = pb[0];
            pf[2 * kb + hf][r + 1] = pb[1];
          }
      }
    };
    // ---- (a8) P.V over one half of the step's keys ------------------------
    auto pv_half = [&](int h) {
#pragma unroll
      for (int kc = h * (C::PC / 2); kc < (h + 1) * (C::PC / 2); ++kc) {
        if (SUB > 1 && !((kmask >> (kc / PCS)) & 1)) continue;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const int row = 16 * kc + v_row;
          const int chunk = (4 * db + v_col) ^ v_swz<D>(row);
          const char* base = v_lds + row * (2 * D) + chunk * 16 + v_half;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * 2 * D));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kc], o[db], 0, 0, 0);
        }
      }
    };
    if (kmask) {
      float rm = -INFINITY;
#pragma unroll
      for (int t = 0; t < SUB; ++t)
        if (SUB == 1 || ((kmask >> t) & 1)) rm = vmax(rm, rm_t[t]);
      const float m_tile = rm * c2;
      const bool grow = m_tile > m_run + 4.f;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? m_tile : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        lb_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
        m_run = m_new;
      }
      softmax_half(0);
    }
    if (vmask) {
      wait_vmem();             // this wave's loads of V_js have landed
      lds_barrier_keep_dma();  // (c): V of the step's kept tiles complete
    }
    // The two units take the second half in opposite orders, so that one
    // wave's P.V of the first half runs against the other wave's exponentials
    // on the same SIMD (waves w and w + NWU share a SIMD).
    if (kmask) {
      const bool pv_first = __builtin_amdgcn_readfirstlane(u) == 0;
      if (pv_first) pv_half(0);
      softmax_half(1);
      if (!pv_first) pv_half(0);
      pv_half(1);
      l_run += rs0 + rs1;
      lb_run += (rb[0] + rb[1]) + (rb[2] + rb[3]);
    }
  };
  // Steps before the last in pairs (K in buffers 0, 1; a leading odd step in
  // buffer 1); the last step, the causal diagonal, reads buffer 0.
  using KB0 = std::integral_constant<int, 0>;
  using KB1 = std::integral_constant<int, 1>;
  for (int js = -par; js < send; js += 2) {
    if (js >= 0) step(js, std::false_type{}, KB0{});
    step(js + 1, std::false_type{}, KB1{});
  }
  step(send, std::integral_constant<bool, CAUSAL>{}, KB0{});

  const int utid = wu * 64 + lane;  // thread index inside the unit
  constexpr int UNT = P2::NWU * 64;
  const int jlast = CAUSAL ? jd1_u[u] : jend;  // this unit's last computed key tile
  if (MAXONLY) {
    if ((CAUSAL || RAGGED) && live)
      for (int jj = jlast + 1 + utid; jj < p.Mkv; jj += UNT) p.tile_max[diag_row + jj] = __builtin_nanf("");
    return;
  }
  // ---- (a9) epilogue -------------------------------------------------------
  const float l_tot = sum_halves(l_run);
  const float inv = 1.f / sum_halves(lb_run);
  if (!RAGGED || qrow < n_seq) {
    store_out_row(p, q_head + qrow, o, inv, hh);
    if (p.lse && hh == 0) p.lse[q_head + qrow] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
  }
  if (p.skip_counts && utid == 0 && live) p.skip_counts[(size_t)(b * p.Hq + hq) * p.M + i] = nskip;
  if (DIAG_OUT && (CAUSAL || RAGGED) && live) {
    for (int jj = jlast + 1 + utid; jj < p.Mkv; jj += UNT) {
      if (p.tile_state) p.tile_state[diag_row + jj] = 0;
      if (p.tile_max) p.tile_max[diag_row + jj] = __builtin_nanf("");
    }
  }
}

}  // namespace bsfa
// the software-pipelined kernel for aligned 128 x 128 tiles at d = 128 (it
// uses the helpers above)
#include "bsfa_fwd_pipe.h"
namespace bsfa {

// Query heads h0 .. h0 + hn - 1 of every KV group: in pairs of heads
// (HEADPAIR, hn even) or in pairs of neighbouring query blocks (with M odd
// the last pair's second block lies past the end: tail-handling instances
// only).
template <int D, int BM, int BN, bool CAUSAL, bool DIAG_OUT, bool MAXONLY, bool HEADPAIR, bool RAGGED>
static int launch_pair(FwdParams p, hipStream_t stream, int h0, int hn) {
  p.pair_h0 = h0;
  p.pair_hn = hn;
  const int per_group = HEADPAIR ? hn / 2 : hn;
  const size_t grid_n = (size_t)p.B * p.Hkv * per_group * (HEADPAIR ? p.M : (p.M + 1) / 2);
  p.remap = (HEADPAIR ? grid_n % (8 * (size_t)per_group) : ((size_t)p.B * p.Hkv * per_group) % 8) == 0 ? 1 : 0;
  const dim3 grid((unsigned)grid_n);
  const dim3 block(BM * 4);
  if constexpr (D == 128 && BM == 128 && BN == 128 && !MAXONLY) {
    // 128 x 128 tiles at d = 128, every pairing, with or without tails: the
    // software-pipelined kernel (one barrier per step), persistent - one
    // workgroup per compute unit taking the static grid's workgroups as work
    // items from per-XCD queues
    if (grid_n > (size_t)INT32_MAX) return 3;
    int n_cu = 0;
    p.work = pipe_work_slot(stream, &n_cu);
    if (!p.work || n_cu <= 0) return 5;
    p.n_items = (int)grid_n;
    const dim3 pgrid((unsigned)(grid_n < (size_t)n_cu ? grid_n : (size_t)n_cu));
    hipLaunchKernelGGL((bsfa_fwd_pipe_kernel<CAUSAL, DIAG_OUT, HEADPAIR, RAGGED>), pgrid, block, 0, stream, p);
  } else {
    hipLaunchKernelGGL((bsfa_fwd_pair_kernel<D, BM, BN, CAUSAL, DIAG_OUT, MAXONLY, HEADPAIR, RAGGED>), grid, block, 0,
                       stream, p);
  }
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// Two units per workgroup on one K/V stream: query-head pairs when the GQA
// group size is even; otherwise neighbouring query blocks of one head (all
// heads under bidirectional attention; under causal masking the group's last
// head, whose other heads run in head pairs in a launch of their own).
template <int D, int BM, int BN, bool CAUSAL, bool DIAG_OUT, bool MAXONLY, bool RAGGED>
static int launch_units_r(const FwdParams& p, hipStream_t s) {
  if (p.G % 2 == 0) return launch_pair<D, BM, BN, CAUSAL, DIAG_OUT, MAXONLY, true, RAGGED>(p, s, 0, p.G);
  // block pairs for heads h0 .. h0 + hn - 1; an odd number of query blocks
  // leaves the last pair's second block past the end, which the tail-handling
  // instances treat as a unit that writes nothing
  auto block_pairs = [&](int h0, int hn) {
    if (p.M % 2 == 0) return launch_pair<D, BM, BN, CAUSAL, DIAG_OUT, MAXONLY, false, RAGGED>(p, s, h0, hn);
    return launch_pair<D, BM, BN, CAUSAL, DIAG_OUT, MAXONLY, false, true>(p, s, h0, hn);
  };
  if (!CAUSAL) return block_pairs(0, p.G);
  if (p.G > 1) {
    const int st = launch_pair<D, BM, BN, CAUSAL, DIAG_OUT, MAXONLY, true, RAGGED>(p, s, 0, p.G - 1);
    if (st) return st;
  }
  return block_pairs(p.G - 1, 1);
}

// A sequence length that is not a multiple of both tile sides, or
// per-sequence lengths, select the kernels compiled with the tail handling;
// aligned lengths run without it.
template <int D, int BM, int BN, bool CAUSAL, bool DIAG_OUT, bool MAXONLY>
static int launch_units(const FwdParams& p, hipStream_t s) {
  if (p.N % BM || p.N % BN || p.seq_lens) return launch_units_r<D, BM, BN, CAUSAL, DIAG_OUT, MAXONLY, true>(p, s);
  return launch_units_r<D, BM, BN, CAUSAL, DIAG_OUT, MAXONLY, false>(p, s);
}

// mode: 0 = forward, 1 = forward with per-tile diagnostics, 2 = tile maxima only
template <int D, int BM, int BN>
static int launch_mode(const FwdParams& p, int causal, int mode, hipStream_t s) {
  if (causal) {
    if (mode == 2) return launch_units<D, BM, BN, true, true, true>(p, s);
    return mode ? launch_units<D, BM, BN, true, true, false>(p, s) : launch_units<D, BM, BN, true, false, false>(p, s);
  }
  if (mode == 2) return launch_units<D, BM, BN, false, true, true>(p, s);
  return mode ? launch_units<D, BM, BN, false, true, false>(p, s) : launch_units<D, BM, BN, false, false, false>(p, s);
}

// Both head dimensions for one tile shape (one translation unit per shape).
template <int BM, int BN>
static int launch_tile(const FwdParams& p, int head_dim, int causal, int mode, hipStream_t s) {
  if (head_dim == 128) return launch_mode<128, BM, BN>(p, causal, mode, s);
  if (head_dim == 64) return launch_mode<64, BM, BN>(p, causal, mode, s);
  return 3;
}

}  // namespace bsfa
