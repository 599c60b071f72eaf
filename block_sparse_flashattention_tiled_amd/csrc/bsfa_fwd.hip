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
// Mapping onto CDNA4:
//  * one workgroup per (batch, query head, query block); BLK/32 waves, wave w
//    owns query rows [32w, 32w+32) of the block;
//  * both contractions run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//    Scores are formed transposed, S^T = K Q^T, so that each lane ends up
//    holding one query row: its row statistics stay in-lane and the score
//    registers, rounded to bf16, are directly the B operand of O^T = V^T P^T;
//  * Q lives in registers for the whole key loop (B.2 step (1));
//  * K_j and V_j are staged through LDS (XOR-swizzled, bank-conflict free for
//    the access patterns used); V_j is stored transposed so that the A
//    operand of O^T = V^T P^T is one 16-byte LDS read;
//  * the tile maximum is reduced in-lane, across the wave with shuffles and
//    across waves through LDS; the skip decision is read back into a scalar
//    register so the branch is uniform for the workgroup.  The V_j loads are
//    issued only on the kept path;
//  * workgroups are ordered heaviest query block first (causal) and, when the
//    grid allows, remapped so that the query heads of one KV group land on
//    the same XCD at the same time and share K_j/V_j in that XCD's L2.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bsfa_internal.h"

namespace bsfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int D, int BLK>
struct Cfg {
  static constexpr int NW = BLK / 32;    // waves per workgroup
  static constexpr int NT = NW * 64;     // threads per workgroup
  static constexpr int KC = D / 16;      // 16-wide d chunks of the QK^T contraction
  static constexpr int KB = BLK / 32;    // 32-key sub-blocks of a tile
  static constexpr int PC = BLK / 16;    // 16-key chunks of the P.V contraction
  static constexpr int DB = D / 32;      // 32-wide d sub-blocks of the output
  static constexpr int CPR_K = D / 8;    // 16-byte chunks per K row (row = key)
  static constexpr int CPR_V = BLK / 8;  // 16-byte chunks per transposed V row (row = d)
  static constexpr int LD = D / 16;      // 16-byte global loads per thread per tile
  // XOR-swizzle shift of the transposed V tile, chosen so that both the
  // transposing 2-byte writes and the 16-byte operand reads are conflict free
  static constexpr int VSH = (D == 128 && BLK == 64) ? 2 : 3;
};

// Position of 16-byte chunk `chunk` of row `row` in a tile with `cpr` chunks
// per row.  A 256-byte line spans all 64 LDS banks; the chunk's position in
// its line is XORed with a function of the line index.
__device__ __forceinline__ int swz(int row, int chunk, int cpr, int sh) {
  const int lin = row * cpr + chunk;
  const int line = lin >> 4;
  const int f = (line ^ (line >> sh)) & 15;
  return (line << 4) | ((lin & 15) ^ f);
}

// MAXONLY: calibration pass - only the tile maxima of every computed tile are
// produced (no gate, no V, no output); used to build threshold tables.
template <int D, int BLK, bool CAUSAL, bool DIAG_OUT, bool MAXONLY>
__global__ void __launch_bounds__(BLK * 2) bsfa_fwd_kernel(const FwdParams p) {
  using C = Cfg<D, BLK>;
  constexpr int KSH = 30;  // K tile: XOR with the line index only
  __shared__ uint4 k_lds[BLK * D / 8];
  __shared__ uint4 v_lds[BLK * D / 8];
  __shared__ float red[C::NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- work item (a1): workgroup -> (b, query head, query block) ----------
  int L = blockIdx.x;
  if (p.remap) {
    // consecutive workgroups go to consecutive XCDs; regroup so that one XCD
    // runs the G query heads of a KV group on the same query block together
    const int x = L & 7;
    const int pp = L >> 3;
    L = ((pp / p.G) * 8 + x) * p.G + (pp % p.G);
  }
  const int hin = L % p.G;
  L /= p.G;
  const int g = L % p.Hkv;
  L /= p.Hkv;
  const int b = L % p.B;
  L /= p.B;
  const int i = CAUSAL ? (p.M - 1 - L) : L;  // causal: heaviest query blocks first
  const int hq = g * p.G + hin;

  const size_t q_head = (size_t)(b * p.Hq + hq) * p.N;
  const size_t kv_head = (size_t)(b * p.Hkv + g) * p.N;
  const int qloc = 32 * w + l32;  // this lane's query row inside the block
  const int qrow = i * BLK + qloc;

  // ---- (a2) Q_i stays in registers: B operand of S^T = K Q^T --------------
  // lane (l32, hh) holds query qloc, d = 16c + 8hh .. 16c + 8hh + 7
  bf16x8 qf[C::KC];
  {
    const uint4* qg = reinterpret_cast<const uint4*>(p.q) + (q_head + qrow) * C::CPR_K;
#pragma unroll
    for (int c = 0; c < C::KC; ++c) qf[c] = __builtin_bit_cast(bf16x8, qg[2 * c + hh]);
  }
  const uint4* kg = reinterpret_cast<const uint4*>(p.k) + kv_head * C::CPR_K;
  const uint4* vg = reinterpret_cast<const uint4*>(p.v) + kv_head * C::CPR_K;

  // threshold of (head, query block); blocks past the table reuse the last entry
  const float tau = MAXONLY ? INFINITY : p.thresholds[hq * p.T_len + min(i, p.T_len - 1)];
  const float c2 = p.scale_log2;

  f32x16 o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;  // running max, in units of scale*log2(e)
  float l_run = 0.f;        // running sum over this lane's half of the keys
  int nskip = 0;
  const int jend = CAUSAL ? i : p.M - 1;

  for (int j = 0; j <= jend; ++j) {
    // ---- (a3) stream K_j into LDS (skipped tiles included) ----------------
    uint4 st[C::LD];
#pragma unroll
    for (int it = 0; it < C::LD; ++it) {
      const int c = tid + C::NT * it;
      st[it] = kg[(size_t)(j * BLK + c / C::CPR_K) * C::CPR_K + (c % C::CPR_K)];
    }
    __syncthreads();  // every wave is done with the previous K_j / V_j
#pragma unroll
    for (int it = 0; it < C::LD; ++it) {
      const int c = tid + C::NT * it;
      k_lds[swz(c / C::CPR_K, c % C::CPR_K, C::CPR_K, KSH)] = st[it];
    }
    __syncthreads();

    // ---- (a4) S^T = K_j Q_i^T on MFMA --------------------------------------
    // s[kb][r] = raw score of query qloc and key kb*32 + 8(r/4) + 4hh + r%4
    f32x16 s[C::KB];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < C::KC; ++c) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, k_lds[swz(kb * 32 + l32, 2 * c + hh, C::CPR_K, KSH)]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[kb], 0, 0, 0);
      }
    }
    const bool diag = (j == i);
    if (CAUSAL && diag) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key > qloc) s[kb][r] = -INFINITY;
        }
    }

    // ---- (a5) tile maximum and gate -----------------------------------------
    float rm = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) rm = fmaxf(rm, s[kb][r]);
    rm = fmaxf(rm, __shfl_xor(rm, 32));  // full row max of query qloc
    float wm = rm;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) wm = fmaxf(wm, __shfl_xor(wm, off));
    if (lane == 0) red[w] = wm;
    __syncthreads();
    float tm = red[0];
#pragma unroll
    for (int ww = 1; ww < C::NW; ++ww) tm = fmaxf(tm, red[ww]);
    const float tms = tm * p.scale;  // s_max in the scaled-score domain
    int skip = (!diag && tms < tau) ? 1 : 0;
    skip = __builtin_amdgcn_readfirstlane(skip);
    if (DIAG_OUT && tid == 0) {
      const size_t t = ((size_t)(b * p.Hq + hq) * p.M + i) * p.M + j;
      if (p.tile_state) p.tile_state[t] = diag ? 3 : (skip ? 2 : 1);
      if (p.tile_max) p.tile_max[t] = tms;
    }
    if (MAXONLY) continue;
    if (skip) {  // (a6): no V load, no exp, no statistics update
      ++nskip;
      continue;
    }

    // ---- (a8) request V_j only now ------------------------------------------
#pragma unroll
    for (int it = 0; it < C::LD; ++it) {
      const int c = tid + C::NT * it;
      st[it] = vg[(size_t)(j * BLK + c / C::CPR_K) * C::CPR_K + (c % C::CPR_K)];
    }

    // ---- (a7) online softmax update while V_j is in flight ------------------
    const float m_new = fmaxf(m_run, rm * c2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float rs = 0.f;
    bf16x8 pf[C::PC];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r = 0; r < 8; r += 2) {
          f32x2 pr;
          pr[0] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hf + r], c2, -m_new));
          pr[1] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hf + r + 1], c2, -m_new));
          rs += pr[0] + pr[1];
          const bf16x2 pb = __builtin_convertvector(pr, bf16x2);
          pf[2 * kb + hf][r] = pb[0];
          pf[2 * kb + hf][r + 1] = pb[1];
        }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] *= alpha;

    // transposed V tile: row d, key slot chosen so that the 8 keys one lane
    // feeds to a 16-deep MFMA step are contiguous
    unsigned short* v16 = reinterpret_cast<unsigned short*>(v_lds);
#pragma unroll
    for (int it = 0; it < C::LD; ++it) {
      const int c = tid + C::NT * it;
      const int key = c / C::CPR_K;
      const int cd = c % C::CPR_K;
      const int q16 = key & 15;
      const int chunk = 2 * (key >> 4) + ((q16 >> 2) & 1);
      const int slot = (q16 & 3) + 4 * (q16 >> 3);
      const unsigned short* e8 = reinterpret_cast<const unsigned short*>(&st[it]);
#pragma unroll
      for (int e = 0; e < 8; ++e) v16[swz(8 * cd + e, chunk, C::CPR_V, C::VSH) * 8 + slot] = e8[e];
    }
    __syncthreads();

    // ---- (a8) O^T += V_j^T P~^T on MFMA -----------------------------------
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int kc = 0; kc < C::PC; ++kc) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, v_lds[swz(db * 32 + l32, 2 * kc + hh, C::CPR_V, C::VSH)]);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kc], o[db], 0, 0, 0);
      }
  }

  if (MAXONLY) {
    if (CAUSAL) {
      const size_t row = ((size_t)(b * p.Hq + hq) * p.M + i) * p.M;
      for (int jj = i + 1 + tid; jj < p.M; jj += C::NT) p.tile_max[row + jj] = __builtin_nanf("");
    }
    return;
  }
  // ---- (a9) epilogue: O_i = O_acc / l, lse, skip count -------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  float* og = p.out + (q_head + qrow) * D;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      float4 val;
      val.x = o[db][4 * g4 + 0] * inv;
      val.y = o[db][4 * g4 + 1] * inv;
      val.z = o[db][4 * g4 + 2] * inv;
      val.w = o[db][4 * g4 + 3] * inv;
      *reinterpret_cast<float4*>(og + db * 32 + 8 * g4 + 4 * hh) = val;
    }
  if (p.lse && hh == 0) p.lse[q_head + qrow] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
  if (p.skip_counts && tid == 0) p.skip_counts[(size_t)(b * p.Hq + hq) * p.M + i] = nskip;
  if (DIAG_OUT && CAUSAL) {
    const size_t row = ((size_t)(b * p.Hq + hq) * p.M + i) * p.M;
    for (int jj = i + 1 + tid; jj < p.M; jj += C::NT) {
      if (p.tile_state) p.tile_state[row + jj] = 0;
      if (p.tile_max) p.tile_max[row + jj] = __builtin_nanf("");
    }
  }
}

template <int D, int BLK, bool CAUSAL, bool DIAG_OUT, bool MAXONLY>
static int launch_one(const FwdParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((size_t)p.B * p.Hq * p.M));
  const dim3 block(BLK * 2);
  hipLaunchKernelGGL((bsfa_fwd_kernel<D, BLK, CAUSAL, DIAG_OUT, MAXONLY>), grid, block, 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// mode: 0 = forward, 1 = forward with per-tile diagnostics, 2 = tile maxima only
template <int D, int BLK>
static int launch_mode(const FwdParams& p, int causal, int mode, hipStream_t s) {
  if (causal) {
    if (mode == 2) return launch_one<D, BLK, true, true, true>(p, s);
    return mode ? launch_one<D, BLK, true, true, false>(p, s) : launch_one<D, BLK, true, false, false>(p, s);
  }
  if (mode == 2) return launch_one<D, BLK, false, true, true>(p, s);
  return mode ? launch_one<D, BLK, false, true, false>(p, s) : launch_one<D, BLK, false, false, false>(p, s);
}

int launch_fwd(const FwdParams& p, int head_dim, int block, int causal, int mode, hipStream_t stream) {
  if (head_dim == 128 && block == 128) return launch_mode<128, 128>(p, causal, mode, stream);
  if (head_dim == 128 && block == 64) return launch_mode<128, 64>(p, causal, mode, stream);
  if (head_dim == 64 && block == 128) return launch_mode<64, 128>(p, causal, mode, stream);
  if (head_dim == 64 && block == 64) return launch_mode<64, 64>(p, causal, mode, stream);
  return 3;
}

}  // namespace bsfa
