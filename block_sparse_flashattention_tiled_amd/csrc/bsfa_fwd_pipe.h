// Software-pipelined forward kernel for aligned 128 x 128 tiles at d = 128:
// the route of every benchmarked layer (query-head pairs, causal or not, and
// bidirectional block pairs).
//
// Operation: "Block Sparse Flash Attention" (paperpeel.com/paper/2512.07011),
// the same as bsfa_fwd_pair_kernel: FlashAttention-2's tiled online softmax
// (App. B.2 steps (1)-(6)) with one gate per score tile (Sec. 4.1, 4.4) -
// an off-diagonal tile whose maximum scaled score is below the threshold of
// its (head, query block) is skipped before any of its V rows is requested
// and takes no part in the running max, sum or output; diagonal tiles always
// pass; causal tiles above the diagonal are never visited.
//
// What differs from bsfa_fwd_pair_kernel is the step.  P~V runs one step
// behind the gate, which leaves one barrier per step instead of two:
//   phase A of step j:  S_j = K_j Q^T (MFMA), its row maxima and this wave's
//                       gate vote, then the step's barrier;
//   phase B of step j:  K_{j+2} and (when a unit keeps tile j) V_j requested,
//                       P~_{j-1} V_{j-1} (MFMA), then the softmax of S_j.
// The barrier of step j publishes the votes of S_j, K_{j+1} and V_{j-1}, and
// frees the K tile of S_j and the V tile of P~V_{j-2}: V_j has a whole step
// to land instead of the exponentials of one tile, and a step whose tile both
// units skip and whose predecessor they skipped is QK^T and one barrier.
// Two K and two V tiles live in LDS, chosen by step parity at compile time.
//
// The lazy rescale of the running output moves with P~V: when a kept tile
// raises a row's reference maximum, O is rescaled right after P~V_{j-1} has
// been accumulated (still against the old reference) and before P~V_j joins
// it in the next step; l and the bf16 sum are rescaled at once.
//
// S_j is formed by the same MFMA chains and its maxima by the same reductions
// as in bsfa_fwd_pair_kernel, so the tile maxima (and every gate decision) are
// bit-identical to those of the tile-maximum pass.
//
// The launch is persistent: one workgroup per compute unit, each taking work
// items (the workgroups of bsfa_fwd_pair_kernel's grid) from per-XCD queues in
// device memory.  The eight XCDs run at clocks of their own; a static grid
// gives each an eighth of the work and ends with the slowest, while the queues
// let an XCD that has emptied its own share take items from the others.
#pragma once

namespace bsfa {

template <bool CAUSAL, bool DIAG_OUT, bool HEADPAIR, bool RAGGED>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
    bsfa_fwd_pipe_kernel(const FwdParams p) {
  constexpr int D = 128, BM = 128, BN = 128;
  using C = Cfg<D, BM, BN>;
  using P2 = PairCfg<D, BM, BN>;
  constexpr int TILE_BYTES = BN * D * 2;
  constexpr int DMA = TILE_BYTES / (P2::NW * 1024);  // load instructions per wave and tile
  static_assert(DMA * P2::NW * 1024 == TILE_BYTES, "tile loads split evenly over the waves");
  __shared__ __attribute__((aligned(16))) char k_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char k_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char v_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char v_lds1[TILE_BYTES];
  __shared__ float red[2][2][P2::NWU];  // [step parity][unit][wave]
  __shared__ int item_sh[2];            // the work item of this and of the next iteration

  const int xcd = xcd_id();
  // This item's Q rows (MFMA B fragments), and whether the previous item's
  // last step already fetched this item's index (pf_idx) and requested its Q
  // rows and first two K tiles (pf_loads): the next item's prologue runs under
  // the last step of the current one.
  bf16x8 qf[C::KC];
  int pf_idx = 0, pf_loads = 0;

  // Persistent: one workgroup per compute unit takes work items - the
  // workgroups of the static grid - from its XCD's queue until it is empty,
  // then from the other XCDs' queues (next_item), so that XCDs running at
  // different clocks finish together.
  for (int iter = 0;; ++iter) {
    // Lane-derived values are formed anew for each item, where they are used,
    // rather than kept in registers across the items (the thread index and the
    // queue inputs are opaque to the compiler from one item to the next).
    int tid = threadIdx.x;
    int xcd_it = xcd;
    using KernargPtr = const __attribute__((address_space(4))) FwdParams*;
    KernargPtr pk = (KernargPtr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+v"(tid), "+s"(xcd_it), "+s"(pk));
    const FwdParams& p = *(const FwdParams*)pk;  // the arguments, read afresh for each item
    const int n_it = p.n_items;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
    const int u = w / P2::NWU;   // unit of this wave
    const int wu = w % P2::NWU;  // wave inside the unit
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    if (!pf_idx) {
      if (tid == 0) item_sh[iter & 1] = next_item(p.work, n_it, xcd_it);
    }
    if (pf_loads) wait_vmem();  // this wave's prefetched Q rows and K_0, K_1
    // also orders the previous item's last LDS reads (and its last loads into
    // LDS, waited before its last barrier) before this item's loads; with the
    // prologue prefetched, publishes K_0 and K_1
    lds_barrier_keep_dma();
    int L = __builtin_amdgcn_readfirstlane(item_sh[iter & 1]);  // uniform: the loop exit is too
    if (L < 0) break;
    const bool prefetched = pf_loads;
    pf_idx = pf_loads = 0;

    // ---- work item (a1): item -> (b, KV group, two units); the same mapping as
    // bsfa_fwd_pair_kernel's workgroups -----------------------------------------
    struct Item {
      int b, g, hq0, hq1, i0, i1;  // batch, KV group, the two units' query heads and blocks
    };
    auto decode = [&](int Li) __attribute__((always_inline)) {
      const int per_group = HEADPAIR ? p.pair_hn / 2 : p.pair_hn;
      const int n_pairs = (p.M + 1) / 2;
      int lp = 0;
      if (HEADPAIR) {
        if (p.remap) {
          const int x = Li & 7;
          const int pp = Li >> 3;
          Li = ((pp / per_group) * 8 + x) * per_group + (pp % per_group);
        }
      } else if (p.remap) {
        const int x = Li & 7;
        const int r = Li >> 3;
        lp = r % n_pairs;
        Li = (r / n_pairs) * 8 + x;
      } else {
        lp = Li / (p.B * p.Hkv * per_group);
      }
      Item it;
      const int hin = Li % per_group;
      Li /= per_group;
      it.g = Li % p.Hkv;
      Li /= p.Hkv;
      it.b = Li % p.B;
      Li /= p.B;
      if (HEADPAIR) {
        const int ib = CAUSAL ? (p.M - 1 - Li) : Li;  // causal: heaviest query blocks first
        it.hq0 = it.g * p.G + p.pair_h0 + 2 * hin;
        it.hq1 = it.hq0 + 1;
        it.i0 = it.i1 = ib;
      } else {
        const int ip = CAUSAL ? (n_pairs - 1 - lp) : lp;  // causal: heaviest block pairs first
        it.hq0 = it.hq1 = it.g * p.G + p.pair_h0 + hin;
        it.i0 = 2 * ip;
        it.i1 = 2 * ip + 1;
      }
      return it;
    };
    // an item's sequence length, key blocks and last step (one key tile per
    // step): the causal diagonal of a head pair, the later diagonal of a causal
    // block pair (the second unit's, or the first's when the second lies past
    // the end), the last key tile otherwise
    auto seq_of = [&](const Item& it) __attribute__((always_inline)) {
      return (RAGGED && p.seq_lens) ? min(max(p.seq_lens[it.b], 0), p.N) : p.N;
    };
    auto last_step = [&](const Item& it, int nseq) __attribute__((always_inline)) {
      const int mkv = RAGGED ? (nseq + BN - 1) / BN : p.Mkv;
      return CAUSAL ? (HEADPAIR ? it.i0 : min(it.i1, mkv - 1)) : mkv - 1;
    };
    const Item cur = decode(L);
    const int b = cur.b, g = cur.g;
    const int hq_u[2] = {cur.hq0, cur.hq1};
    const int i_u[2] = {cur.i0, cur.i1};
    const int hq = hq_u[u];
    const int i = i_u[u];
    // Tails (RAGGED: a length that is not a multiple of 128, per-sequence
    // lengths clamped to [0, N], or block pairs over an odd number of query
    // blocks): the last query and key blocks are partial and positions past the
    // end do not exist.  An item whose units both lie past the end is done at
    // once (the workgroup takes its next item); a block pair whose second block
    // lies past the end keeps that unit in the barriers (its rows masked, its
    // decisions unused) and writes nothing for it.
    const int n_seq = seq_of(cur);
    const int mkv_seq = RAGGED ? (n_seq + BN - 1) / BN : p.Mkv;
    if (RAGGED && i_u[0] * BM >= n_seq) continue;  // i_u[0] <= i_u[1]
    const bool live = !RAGGED || i * BM < n_seq;
    const size_t q_head = (size_t)(b * p.Hq + hq) * p.N;
    const size_t kv_head = (size_t)(b * p.Hkv + g) * p.N;
    const int qloc = 32 * wu + l32;
    const int qrow = i * BM + qloc;
    // P~V A-fragment reads (ds_read_b64_tr_b16): lane l reads V row
    // 16 kc + v_row, 16-byte chunk (4 db + v_col) ^ v_swz(row), half v_half.
    // v_swz(16 kc + v_row) = (v_row & 3) << 2, so the byte offset is
    // 4096 kc + (vb ^ (db << 6)) with vb below: the row, the chunk's low bits
    // and the half occupy bits disjoint from db's
    const int v_row = 4 * hh + ((lane & 15) >> 2);
    const int v_col = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    int vb = v_row * (2 * D) + (((v_row & 3) << 2) << 4) + (v_col << 4) + (lane & 1) * 8;
    asm volatile("" : "+v"(vb));

    // ---- (a2) Q: this wave's 32 rows stay in registers as MFMA B fragments ------
    // (a row past the end reads the last row; its scores are masked)
    auto load_q = [&](int b_, int hq_, int i_, int nseq) __attribute__((always_inline)) {
      const int qr = RAGGED ? min(i_ * BM + qloc, nseq - 1) : i_ * BM + qloc;
      const bf16x8* qsrc = reinterpret_cast<const bf16x8*>(p.q) + ((size_t)(b_ * p.Hq + hq_) * p.N + qr) * (D / 8) + hh;
      #pragma unroll
      for (int c = 0; c < C::KC; ++c) qf[c] = qsrc[2 * c];
    };
    if (!prefetched) load_q(b, hq, i, n_seq);
    const u32x4* kg = reinterpret_cast<const u32x4*>(p.k) + kv_head * C::CPR;
    const u32x4* vg = reinterpret_cast<const u32x4*>(p.v) + kv_head * C::CPR;

    float tau_u[2];
    #pragma unroll
    for (int uu = 0; uu < 2; ++uu) tau_u[uu] = p.thresholds[hq_u[uu] * p.T_len + min(i_u[uu], p.T_len - 1)];
    const float c2 = p.scale_log2;
    // Arguments read inside the step loop, held in registers: every barrier is
    // a compiler memory barrier, after which a read through p would be issued
    // again (a scalar load and its wait on the critical path of each step).
    const float scale = p.scale;
    const int gate = p.gate;
    const int kv_bytes = p.N * D * 2;  // one head's K or V: the range of its buffer loads
    uint8_t* const tile_state = p.tile_state;
    float* const tile_max = p.tile_max;
    // square tiles: the diagonal of query block i is key block i
    const int send = last_step(cur, n_seq);
    const size_t diag_row = ((size_t)(b * p.Hq + hq) * p.M + i) * p.Mkv;

    f32x16 o[C::DB];
    #pragma unroll
    for (int db = 0; db < C::DB; ++db) o[db] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;
    float lb_run = 0.f;
    float mrun_u[2] = {-INFINITY, -INFINITY};  // per unit: largest s_max of its kept tiles (gap gate)
    int nskip = 0;
    bf16x8 pprev[C::PC];  // P~ of the previous step (bf16), waiting for its P.V
    int kept_prev = 0;    // this unit kept the previous step's tile (uniform)

    // Direct-to-LDS load of the K or V tile whose first key is row0 (the same
    // layout and swizzles as bsfa_fwd_pair_kernel): instruction n of wave w fills
    // the 1 KB of 16-byte slots 64 (4 w + n) .. + 63, i.e. rows 4 (4 w + n) .. + 3;
    // lane l takes row r = 4 (4 w + n) + l / 16 and slot l % 16, holding logical
    // chunk (l % 16) ^ swz(r).  Since r % 16 = 4 n + l / 16, the K chunk is
    // ((l % 16) ^ (l / 16)) ^ 4 n and the V chunk (l % 16) ^ 4 ((l / 16) % 4):
    // the lane offset is one per-lane base (XOR n << 6 for K), and the rest,
    // 1 KB per instruction and the tile's first row, is a scalar offset.
    static_assert(D == 128 && DMA == 4, "lane offsets below assume 16 chunks per row and 4 loads per wave");
    int k_lane = (lane >> 4) * 256 + (((lane & 15) ^ (lane >> 4)) << 4);
    int v_lane = (lane >> 4) * 256 + (((lane & 15) ^ ((lane >> 4) << 2)) << 4);
    asm volatile("" : "+v"(k_lane), "+v"(v_lane));
    auto dma_tile = [&](char* dst, const u32x4* head, int row0, bool is_k) __attribute__((always_inline)) {
      #pragma unroll
      for (int n = 0; n < DMA; ++n) {
        const int chunk0 = (w * DMA + n) * 64;
        const int voff = is_k ? (k_lane ^ (n << 6)) : v_lane;
        buffer_load_lds16(head, kv_bytes, dst + chunk0 * 16, voff, row0 * (C::CPR * 16) + chunk0 * 16);
      }
    };
    // The tile that crosses the end of the sequence: lane offsets formed per
    // lane, rows past the end reading the last row (every load stays inside
    // the head); its scores past the end are masked.
    auto dma_tile_tail = [&](char* dst, const u32x4* head, int row0, bool is_k, int nseq)
                             __attribute__((always_inline)) {
      const int last = nseq - 1 - row0;
      #pragma unroll
      for (int n = 0; n < DMA; ++n) {
        const int chunk0 = (w * DMA + n) * 64;
        const int row = 4 * (w * DMA + n) + (lane >> 4);
        const int cc = (lane & 15) ^ (is_k ? k_swz<D>(row) : v_swz<D>(row));
        buffer_load_lds16(head, kv_bytes, dst + chunk0 * 16, (min(row, last) * C::CPR + cc) * 16,
                          row0 * (C::CPR * 16));
      }
    };
    auto dma_key_tile_n = [&](char* dst, const u32x4* head, int t, bool is_k, int nseq) __attribute__((always_inline)) {
      if (RAGGED && (t + 1) * BN > nseq) dma_tile_tail(dst, head, t * BN, is_k, nseq);
      else dma_tile(dst, head, t * BN, is_k);
    };
    auto dma_key_tile = [&](char* dst, const u32x4* head, int t, bool is_k) __attribute__((always_inline)) {
      dma_key_tile_n(dst, head, t, is_k, n_seq);
    };
    // Tile js (K and V alike) lives in buffer (js + par) & 1, so that the last
    // step reads buffer 0 and every buffer choice is known at compile time.
    const int par = send & 1;
    if (!prefetched) {
      if (par) dma_key_tile(k_lds1, kg, 0, true);
      else dma_key_tile(k_lds0, kg, 0, true);
      wait_vmem();
      lds_barrier_keep_dma();  // K_0 visible
      if (send >= 1) {         // K_1, published by the barrier of step 0
        if (par) dma_key_tile(k_lds0, kg, 1, true);
        else dma_key_tile(k_lds1, kg, 1, true);
      }
    }
    // The next item's prologue, from the last step once its K tile is read:
    // its index (fetched before the step's barrier), its Q rows into qf (dead
    // after this item's last QK^T) and its K_0 and K_1 into the two K tiles
    // (both free after the last step's barrier).  An item past the end loads
    // nothing.
    auto prefetch_next = [&]() __attribute__((always_inline)) {
      const int Ln = __builtin_amdgcn_readfirstlane(item_sh[(iter + 1) & 1]);
      pf_idx = 1;
      if (Ln < 0) return;
      const Item nx = decode(Ln);
      const int nseq = seq_of(nx);
      if (RAGGED && nx.i0 * BM >= nseq) return;
      load_q(nx.b, u ? nx.hq1 : nx.hq0, u ? nx.i1 : nx.i0, nseq);
      const int nsend = last_step(nx, nseq);
      const u32x4* kgn = reinterpret_cast<const u32x4*>(p.k) + (size_t)(nx.b * p.Hkv + nx.g) * p.N * C::CPR;
      dma_key_tile_n((nsend & 1) ? k_lds1 : k_lds0, kgn, 0, true, nseq);
      if (nsend >= 1) dma_key_tile_n((nsend & 1) ? k_lds0 : k_lds1, kgn, 1, true, nseq);
      pf_loads = 1;
    };

    // P~V against the V tile vt.  v_frag: the A fragment (V^T, 32 d x 16
    // keys) of column block db and 16-key chunk kc, by two transposing LDS
    // reads.  pv_all: every chunk's four MFMAs, each fragment of chunk kc + 1
    // requested right after the MFMA that consumed the same registers for chunk
    // kc, so that it has four MFMAs to land.
    auto v_frag = [&](const char* vt, int kc, int db) __attribute__((always_inline)) {
      const char* base = vt + kc * 16 * (2 * D) + (vb ^ (db << 6));
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * 2 * D));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto pv_all = [&](const char* vt) __attribute__((always_inline)) {
      bf16x8 a[C::DB];
      #pragma unroll
      for (int db = 0; db < C::DB; ++db) a[db] = v_frag(vt, 0, db);
      #pragma unroll
      for (int kc = 0; kc < C::PC; ++kc) {
        #pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[db], pprev[kc], o[db], 0, 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (kc + 1 < C::PC) {
            a[db] = v_frag(vt, kc + 1, db);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    auto step = [&](const int js, auto DIAGC, auto KBUF, auto DIAG0C, auto LASTC) __attribute__((always_inline)) {
      constexpr bool DIAG_TILE = decltype(DIAGC)::value;
      constexpr bool LAST = decltype(LASTC)::value;
      constexpr int kb_cur = decltype(KBUF)::value;
      char* const k_cur = kb_cur ? k_lds1 : k_lds0;       // K_js
      char* const v_cur = kb_cur ? v_lds1 : v_lds0;       // V_js (loaded in this step)
      const char* const v_prev = kb_cur ? v_lds0 : v_lds1;  // V_{js-1} (published by this step's barrier)
      // ---- phase A: (a4) S^T = K Q^T ----------------------------------------
      // (last step: the next item's index is claimed first, its latency under
      // the MFMAs, and published by the step's barrier)
      int nxt = -1;
      if constexpr (LAST) {
        if (tid == 0) nxt = next_item(p.work, n_it, xcd_it);
      }
      f32x16 s[C::KB];
      qk_tile_swz<D, BM, BN>(s, k_cur, l32, hh, qf);
      if constexpr (CAUSAL && DIAG_TILE) mask_causal(s, qloc, hh, i * BM - js * BN);
      if constexpr (decltype(DIAG0C)::value) {
        // causal block pair: the first unit's diagonal, the step before the
        // last (peeled, buffer 1); the second unit sees the whole tile
        if (u == 0) mask_causal_alu(s, qloc, hh, i * BM - js * BN);
      }
      if constexpr (RAGGED) {
        const int rows_left = n_seq - i * BM, keys_left = n_seq - js * BN;
        if (rows_left < BM || keys_left < BN) mask_tail(s, qloc, hh, rows_left, keys_left);
      }
      // ---- (a5) row maxima and this wave's vote or maximum --------------------
      float rm0 = -INFINITY, rm1 = -INFINITY;
      #pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
        #pragma unroll
        for (int r = 0; r < 16; r += 2) {
          rm0 = vmax(rm0, s[kb][r]);
          rm1 = vmax(rm1, s[kb][r + 1]);
        }
      float rm = vmax(rm0, rm1);
      rm = max_halves(rm);
      float wm;
      if (!DIAG_OUT && gate == 0) {
        // threshold gate without tile maxima written: each wave votes +inf if
        // some row's scaled maximum is not below tau (rounding of the positive
        // scale is monotone: the decision the tile maximum gives, NaN included)
        const bool keep = !(rm * scale < (u ? tau_u[1] : tau_u[0]));
        wm = __builtin_amdgcn_ballot_w64(keep) ? INFINITY : -INFINITY;
      } else {
        wm = wave_max_sym(rm);
      }
      if (lane == 0) red[kb_cur][u][wu] = wm;
      if constexpr (LAST) {
        if (tid == 0) item_sh[(iter + 1) & 1] = nxt;
      }
      wait_vmem();             // this wave's loads of K_{js+1} and V_{js-1} have landed
      lds_barrier_keep_dma();  // votes of S_js, K_{js+1} and V_{js-1} complete; K_js and V_{js-2} free
      // ---- phase B ------------------------------------------------------------
      if (!(CAUSAL && DIAG_TILE) && js + 2 <= send) dma_key_tile(k_cur, kg, js + 2, true);
      if constexpr (LAST) prefetch_next();
      int skip_of[2];
      bool exists_u[2];
      #pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        float tm = red[kb_cur][uu][0];
        #pragma unroll
        for (int ww = 1; ww < P2::NWU; ++ww) tm = vmax(tm, red[kb_cur][uu][ww]);
        const float tms = tm * scale;
        const bool on_diag = js == i_u[uu];
        // in a causal block pair the first unit has no tile past its diagonal
        exists_u[uu] = !CAUSAL || HEADPAIR || js <= i_u[uu];
        skip_of[uu] = exists_u[uu] ? gate_skip(gate, !on_diag, tms, tau_u[uu], mrun_u[uu]) : 1;
        if (DIAG_OUT && exists_u[uu] && uu == u && wu == 0 && lane == 0 && live) {
          if (tile_state) tile_state[diag_row + js] = on_diag ? 3 : (skip_of[uu] ? 2 : 1);
          if (tile_max) tile_max[diag_row + js] = tms;
        }
      }
      const int mine = u ? skip_of[1] : skip_of[0];
      const int kmask = __builtin_amdgcn_readfirstlane(mine ? 0 : 1);
      const int vmask = __builtin_amdgcn_readfirstlane((skip_of[0] & skip_of[1]) ? 0 : 1);
      nskip += (mine && (u ? exists_u[1] : exists_u[0])) ? 1 : 0;  // (a6)
      // ---- (a8) V_js -> LDS when some unit keeps the tile -----------------------
      if (vmask) dma_key_tile(v_cur, vg, js, false);
      // ---- (a7) reference maximum of the kept tile ------------------------------
      float alpha = 1.f;
      int rescale = 0;
      if (kmask) {
        const float m_tile = rm * c2;
        const bool grow = m_tile > m_run + 4.f;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float m_new = grow ? m_tile : m_run;
          alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= alpha;
          lb_run *= alpha;
          m_run = m_new;
          rescale = 1;
        }
      }
      // ---- (a8) P~V of the previous kept step, with (a7) the softmax of this one --
      // P~ = exp2(S c2 - m) rounded to bf16; l sums the fp32 values, lb the bf16
      // ones (the weights that multiply V), over four independent chains
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      float rs0 = 0.f, rs1 = 0.f;
      float rb[4] = {0.f, 0.f, 0.f, 0.f};
      // P~_js replaces P~_{js-1}, whose MFMAs are issued first
      auto softmax_chunk = [&](int kc) __attribute__((always_inline)) {
        const int kb = kc / 2, hf = kc % 2;
        #pragma unroll
        for (int r = 0; r < 8; r += 2) {
          f32x2 pr;
          pr[0] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hf + r], c2, -m_run));
          pr[1] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hf + r + 1], c2, -m_run));
          const bf16x2 pb = __builtin_convertvector(pr, bf16x2);
          rs0 += pr[0];
          rs1 += pr[1];
          rb[(r >> 1) & 3] = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, rb[(r >> 1) & 3], false);
          pprev[kc][r] = pb[0];
          pprev[kc][r + 1] = pb[1];
        }
      };
      if (kept_prev) pv_all(v_prev);
      if (kmask) {
        #pragma unroll
        for (int kc = 0; kc < C::PC; ++kc) softmax_chunk(kc);
      }
      if (rescale) {
        // after P~V_{js-1}, which is still relative to the old reference
        #pragma unroll
        for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
      }
      if (kmask) {
        l_run += rs0 + rs1;
        lb_run += (rb[0] + rb[1]) + (rb[2] + rb[3]);
      }
      kept_prev = kmask;
      return vmask;
    };
    using KB0 = std::integral_constant<int, 0>;
    using KB1 = std::integral_constant<int, 1>;
    // A causal block pair whose second unit is live has the first unit's
    // diagonal one step before the last: that step is peeled as well.
    const bool peel0 = CAUSAL && !HEADPAIR && send == i_u[0] + 1;
    const int lend = peel0 ? send - 1 : send;  // steps [0, lend) in the loop
    for (int js = -par; js < lend; js += 2) {
      if (js >= 0) step(js, std::false_type{}, KB0{}, std::false_type{}, std::false_type{});
      if (!(CAUSAL && !HEADPAIR) || js + 1 < lend)
        step(js + 1, std::false_type{}, KB1{}, std::false_type{}, std::false_type{});
    }
    if constexpr (CAUSAL && !HEADPAIR) {
      if (peel0) step(send - 1, std::false_type{}, KB1{}, std::true_type{}, std::false_type{});
    }
    const int v_last = step(send, std::integral_constant<bool, CAUSAL>{}, KB0{}, std::false_type{}, std::true_type{});
    // ---- drain: P~V of the last step (V_send in buffer 0) --------------------------
    if (v_last) {
      wait_vmem();
      lds_barrier_keep_dma();
      if (kept_prev) pv_all(v_lds0);
    }

    // ---- (a9) epilogue -------------------------------------------------------
    const int utid = wu * 64 + lane;
    constexpr int UNT = P2::NWU * 64;
    const float l_tot = sum_halves(l_run);
    const float inv = 1.f / sum_halves(lb_run);
    if (!RAGGED || qrow < n_seq) {
      store_out_row(p, q_head + qrow, o, inv, hh);
      if (p.lse && hh == 0) p.lse[q_head + qrow] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
    }
    if (p.skip_counts && utid == 0 && live) p.skip_counts[(size_t)(b * p.Hq + hq) * p.M + i] = nskip;
    if (DIAG_OUT && (CAUSAL || RAGGED) && live) {
      const int jlast = CAUSAL ? min(i, mkv_seq - 1) : mkv_seq - 1;  // this unit's last computed key tile
      for (int jj = jlast + 1 + utid; jj < p.Mkv; jj += UNT) {
        if (p.tile_state) p.tile_state[diag_row + jj] = 0;
        if (p.tile_max) p.tile_max[diag_row + jj] = __builtin_nanf("");
      }
    }
  }  // work items
}

}  // namespace bsfa
