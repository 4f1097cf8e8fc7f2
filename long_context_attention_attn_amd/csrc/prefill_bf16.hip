// prefill_bf16.hip -- lightning-attention prefill, bf16 storage, MFMA, fp32 state (gfx950).
//
// The method ("MiniMax-01 technical report digest", futurefh.com, section 1): causal linear
// attention split into an intra-block part computed with the left product ((Q K^T) masked) V
// and an inter-block part computed with the right product Q (K^T V), the latter carried by a
// running d x d state so that no cumulative sum over the sequence is needed.  With a constant
// per-head decay lambda, for block i of b rows (rows j = 0..b-1, KV_{-1} = initial state):
//
//   O_i  = ((Q_i K_i^T) * M) V_i  +  diag(lambda^(j+1)) Q_i KV_{i-1},
//          M[j][j'] = lambda^(j-j') if j' <= j, else exactly 0 (a select, not a product)
//   KV_i = lambda^b KV_{i-1}  +  K_i^T diag(lambda^(b-1-j)) V_i
//
// which is exact algebra for o_t = sum_{s<=t} lambda^(t-s) (q_t . k_s) v_s.
//
// Work decomposition (one fused pass: one HBM read of q/k/v, one write of out):
//   * one workgroup per (sequence, head, 32-column slice of the value dimension).  Value
//     columns are independent: KV[:, c] and O[:, c] depend on V[:, c] only.  The D/32 slices
//     of one head read the same Q and K blocks, so the workgroup index is mapped so that they
//     land on the same XCD (workgroups are dealt to the 8 XCDs round-robin) and share its L2.
//   * 8 waves, two per SIMD, in two specialised roles that run side by side on each SIMD so
//     that one wave's VALU work overlaps the other's MFMA and LDS traffic:
//       - output wave r (r = 0..3) owns output rows 16r..16r+15 of each block: S^T = K Q^T on
//         its r+1 causal tiles, decay mask in registers, O^T = lambda^(j+1) KV^T Q^T + V^T P^T
//         (the S^T accumulator layout is exactly the B-operand layout of P, so P never leaves
//         registers), and the store;
//       - state wave r owns a band of rows of the fp32 state, kept in MFMA accumulators for
//         the whole sequence: KV = lambda^b KV + K^T diag(lambda^(b-1-j)) V, reading K and the
//         decayed copy diag(lambda^(b-1-j)) V token-major through ds_read_b64_tr_b16 (LDS
//         transpose reads), then publishes a bf16 copy of its rows for the next block's inter
//         product.  Bands are dealt unevenly so that each SIMD's pair of waves carries about
//         the same MFMA work.  The decayed V copy is written once per block by the output
//         waves (each scales the 16 V rows it loads), so no state wave scales operands.
//     Every role is a template instance, so trip counts are static and code between
//     barriers is straight-line.
//   * q/k/v blocks go straight from HBM into LDS (buffer_load ... lds), two blocks ahead of
//     the one being computed, in a three-stage ring with explicit waits; one barrier per
//     block.  Buffer range checking zero-fills rows past the end of a sequence and drops
//     stores past it, so there are no branches around memory operations.  Output waves 0-2
//     issue the Q and V loads, each state wave its K rows, and the last state wave also pulls
//     each block's lines into L2 two blocks before their loads (sparse loads into a scratch
//     area of LDS), so those loads hit L2.
//
// Variants of the same scan, used by the sequence-split prefill and by the backward pass:
// a reversed scan (template REV: local token t is physical token n-1-t of the sequence, for the
// anti-causal gradients), an initial state that counts as already containing token -1's decay
// (weight lambda^t at local token t, final state times lambda), a transposed initial state, and
// a state-only instance (template SO: no Q loads, no outputs) that returns each chain's final
// state.
//
// MFMA used: v_mfma_f32_16x16x32_bf16.  Lane l (g = l/16, c = l%16) holds A[c][k in K(g)],
// B[k in K(g)][c] and C[4g+i][c], i = 0..3; any k-assignment K(g) shared by A and B gives
// the same product, which lets every operand be read in whatever k-order is cheapest.
#include "la_internal.h"

#include "bf16_tiles.h"
#include "seg_lookup.h"

namespace {

constexpr int BLK = 64;   // tokens per block
constexpr int NST = 3;    // pipeline stages (blocks resident in LDS)

template <int D>
struct Cfg : RowCfg<D> {
  using RowCfg<D>::ROWB;
  using RowCfg<D>::VROWB;
  // A stage holds everything one block needs: its Q, K and V rows (DMA targets), the bf16 copy
  // of the state it starts from and its decayed V rows.  Every LDS address in the block loop is
  // then a per-block base (one per lane pattern) plus an immediate below 64 KiB.
  static constexpr int Q_OFF = 0;                          // byte offsets inside a stage
  static constexpr int K_OFF = BLK * ROWB;
  static constexpr int V_OFF = 2 * BLK * ROWB;
  static constexpr int KVX = CV * ROWB;                    // bf16 state copy [CV][D]
  static constexpr int KVX_OFF = V_OFF + BLK * VROWB;
  static constexpr int LV = BLK * VROWB;                   // decayed V copy, [BLK][CV]
  static constexpr int LV_OFF = KVX_OFF + KVX;
  static constexpr int STAGE = LV_OFF + LV;
  static constexpr int PF_OFF = NST * STAGE;               // 1 KiB sink of the L2 prefetches
  static constexpr int SMEM = PF_OFF + 1024;
  static_assert(STAGE < 65536, "stage offsets must fit the LDS instruction offset");
};

// LDS offset of the incoming state of a segment in the sequence-split form (see
// IncomingState in seg_lookup.h): after the powers table in the last stage.
template <int D>
constexpr int SIN_OFF() { return (NST - 1) * Cfg<D>::STAGE + 1024; }

// State rows owned by state wave R (in 16-row tiles) and its first row.  Output wave r does
// r+1 score tiles, so the low bands are larger: each SIMD's pair then does about the same
// number of MFMAs.
template <int D, int R>
struct Band {
  static constexpr int T128[4] = {3, 3, 1, 1};
  static constexpr int T64[4] = {2, 1, 1, 0};
  static constexpr int tiles(int r) { return D == 128 ? T128[r] : T64[r]; }
  static constexpr int first(int r) { return r == 0 ? 0 : first(r - 1) + 16 * tiles(r - 1); }
  static constexpr int RT = tiles(R);
  static constexpr int DK0 = first(R);
};

// L2 prefetch of a share of the block's rows of q, k and the full v rows, two blocks before
// their DMA (farther ahead, the 4 MB L2 of an XCD evicts prefetched lines before their use,
// measured): one 16-byte read per 128-byte line, written to a scratch area of LDS that nothing
// reads.  Slice s takes rows (64 / (D/32)) s onwards: 16 rows of two lines at D = 128 (four
// slices), 32 rows of one line at D = 64 (two slices; lanes 32..63 repeat lanes 0..31), so the
// slices of a head together cover all 64 rows once and the later DMAs of every slice hit L2
// instead of waiting on HBM.
template <int D, bool REV>
__device__ __forceinline__ uint32_t prefetch_offset(int slice, int lane, uint32_t rowbytes) {
  if constexpr (D == 128)
    return lane_base<REV>(16 * slice + ((lane >> 1) & 15), (uint32_t)(lane & 1) * 128u, rowbytes);
  else
    return lane_base<REV>(32 * slice + (lane & 31), 0u, rowbytes);
}
template <bool SO, bool REV>
__device__ __forceinline__ void prefetch_l2(const Chain &c, const Span &s, uint32_t off,
                                            uint32_t sink) {
  const uint32_t o = at<REV>(s, off);
  if constexpr (SO)
    dma16_same2(rsrc(c.k + s.off, s.bytes), rsrc(c.v + s.off, s.bytes), o, sink);
  else
    dma16_same3(rsrc(c.q + s.off, s.bytes), rsrc(c.k + s.off, s.bytes), rsrc(c.v + s.off, s.bytes),
                o, sink);
}
// prefetch instructions per block (no Q when only the state is computed)
template <bool SO>
constexpr int pf_dma() { return SO ? 2 : 3; }
constexpr int PF_AHEAD = 2; // blocks between a block's prefetch and its DMA

// ------------------------------------------------------------------------------------------
// Output wave r: rows 16r..16r+15 of every block.  The loading duties are dealt against the
// score work (wave r does r+1 score tiles): wave 0 loads Q rows 0..15 and V rows 0..31, wave 1
// Q rows 16..31 and 48..63 and V rows 32..47, wave 2 Q rows 32..47 and V rows 48..63, wave 3
// (four score tiles) nothing.  Once its V rows of the next block have landed, a wave writes them
// decayed, lambda^(b-1-j) V[j], to that block's stage, where the state waves consume it (so no
// state wave scales operands).
// ------------------------------------------------------------------------------------------
template <int D, int R, bool SO, bool REV>
__device__ __forceinline__ void output_wave(const Chain &c, char *smem, const float *pw,
                                            int lane) {
  using C = Cfg<D>;
  constexpr int NT = R + 1;         // causal score tiles
  constexpr int NS = (NT + 1) / 2;  // 32-token k-steps of the intra product
  // 16-row groups of V this wave loads and decays: [VG0, VG0 + NVG).
  constexpr int VG0 = R == 0 ? 0 : R == 1 ? 2 : 3;
  constexpr int NVG = R == 0 ? 2 : R == 3 ? 0 : 1;
  // DMA instructions this wave issues per block (Q rows, none when only the state is computed,
  // then its V groups) and output stores per block.
  constexpr int QDMA = SO ? 0 : R == 1 ? 2 * C::QK_DMA : R < 3 ? C::QK_DMA : 0;
  constexpr int DMA = QDMA + NVG;
  constexpr int STORES = SO ? 0 : 2;
  const int l16 = lane & 15, g = lane >> 4;
  const int jrow = 16 * R + l16;  // this lane's output row inside a block
  const uint32_t smem_lds = lds_addr(smem);

  // Decay weights lambda^(jrow - j'), j' = 16 t + 4 g + i; only the diagonal tile t = R has
  // entries above the diagonal (j' > jrow), which are selected away.
  float maskw[NT][4];
  bool keep[4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jp = 16 * t + 4 * g + i;
      maskw[t][i] = jp <= jrow ? pw[jrow - jp] : 0.f;
      if (t == R) keep[i] = jp <= jrow;
    }
  const float inter_scale = pw[jrow + 1];
  // Block 0 applies the initial state; weighted lambda^j instead when it counts as inclusive.
  const float inter_first = c.incl ? pw[jrow] : inter_scale;
  const int trow = 4 * g + (l16 >> 2), tcol = 4 * (l16 & 3);
  const uint32_t rowbytes = c.rowbytes;
  // Lane offsets of this wave's DMA copies (Q row groups R and, for wave 1, 3; V row groups) and
  // of its output stores.
  uint32_t qoff[2][C::QK_DMA];
  rows_offsets<D, REV>(R, lane, rowbytes, qoff[0]);
  rows_offsets<D, REV>(3, lane, rowbytes, qoff[1]);
  uint32_t voff[NVG > 0 ? NVG : 1];
#pragma unroll
  for (int m = 0; m < NVG; ++m)
    voff[m] = lane_base<REV>(16 * (VG0 + m) + lane / 4,
                             16u * ((lane % 4) ^ vswf(16 * (VG0 + m) + lane / 4)), rowbytes) -
              (REV ? 0u : 1024u * m);  // forward: copy m adds m KiB back (rows >= 16 m)
  const uint32_t ooff = lane_base<REV>(jrow, 8u * g, rowbytes);
  const char *vslice = c.v + 2 * c.c0;
  // This wave's share of the decayed V copy: lane bytes 16 (lane % 4) .. +15 of V rows
  // 16 m + lane / 4, m in its groups, with their decay lambda^(b-1-row) (full and last block).
  const int b_last = c.b_last;
  float lv_full[NVG > 0 ? NVG : 1], lv_last[NVG > 0 ? NVG : 1];
#pragma unroll
  for (int m = 0; m < NVG; ++m) {
    const int vrow = 16 * (VG0 + m) + lane / 4;
    lv_full[m] = pw[BLK - 1 - vrow];
    lv_last[m] = vrow < b_last ? pw[b_last - 1 - vrow] : 0.f;
  }

  // Lane parts of this wave's LDS addresses; each block adds its stage offset once per pattern
  // (kept opaque to the compiler) and every access adds an immediate.  Rows 16 x + l16 of a
  // swizzled [rows][D] tile share the pattern of row l16 (the swizzle depends on row mod 8 and
  // bit 2); V rows 16 x + trow share that of row trow.
  uint32_t kpat[C::KSTEPS], vpat[2];
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks) kpat[ks] = (uint32_t)swz<D>(l16, 32 * ks + 8 * g);
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) vpat[ct] = (uint32_t)vswz(trow, 16 * ct + tcol);
  const uint32_t dpat = (uint32_t)((16 * VG0 + lane / 4) * C::VROWB + 16 * (lane % 4));

  // Blocks whose DMA is issued next (wi) and whose outputs are stored next (ws).
  Walk wi = walk_from<BLK, REV>(c, 0), ws = walk_from<BLK, REV>(c, 0);
  auto issue = [&](uint32_t st_off) {
    const uint32_t st = smem_lds + st_off;
    const Span sp = span_at<REV>(c, wi);
    advance<REV>(c, wi);
    if constexpr (!SO && R < 3)
      dma_rows<D, REV>(c.q, sp, qoff[0], st + C::Q_OFF + 16 * R * C::ROWB);
    if constexpr (!SO && R == 1) dma_rows<D, REV>(c.q, sp, qoff[1], st + C::Q_OFF + 48 * C::ROWB);
    const uint32_t vl = st + C::V_OFF + 16 * VG0 * C::VROWB;  // 1 KiB per 16-row group
    if constexpr (NVG == 2) {
      if constexpr (REV)
        dma16x2(rsrc(vslice + sp.off, sp.bytes), at<REV>(sp, voff[0]), at<REV>(sp, voff[1]), vl,
                vl + 1024);
      else
        dma_kib2(rsrc(vslice + sp.off, sp.bytes), voff[0], voff[1], vl);
    } else if constexpr (NVG == 1) {
      dma16(rsrc(vslice + sp.off, sp.bytes), at<REV>(sp, voff[0]), vl);
    }
  };
  // Decayed copy of this wave's V rows of block blk (landed in the stage at st_off) into the same
  // stage.  All reads are issued before any write, so the LDS round trips overlap.
  auto decay_v = [&](int blk, uint32_t st_off) {
    if constexpr (NVG > 0) {
      const bool last = blk == c.nb - 1;
      uint32_t db = dpat + st_off;
      asm volatile("" : "+v"(db));
      bf16x8 x[NVG];
#pragma unroll
      for (int m = 0; m < NVG; ++m)
        x[m] = *(const bf16x8 *)(smem + db + (C::V_OFF + 16 * m * C::VROWB));
#pragma unroll
      for (int m = 0; m < NVG; ++m)
        *(bf16x8 *)(smem + db + (C::LV_OFF + 16 * m * C::VROWB)) =
            scale8(x[m], last ? lv_last[m] : lv_full[m]);
    }
  };
  static_assert(NST == 3, "stage rotation and wait counts are written for three stages");
  // Stage offsets of blocks i (cur), i + 1 (nxt) and i + 2 (prv: the stage read in step i - 1).
  uint32_t s_cur = 0, s_nxt = C::STAGE, s_prv = 2 * C::STAGE;
  issue(0);
  issue(C::STAGE);
  if constexpr (DMA > 0) wait_vm<(NST - 2) * DMA>();  // own block-0 rows landed
  decay_v(0, 0);
  lds_barrier();  // block 0 and its decayed V visible to all waves

  for (int i = 0; i < c.nb; ++i) {
    issue(s_prv);  // block i + 2, into the stage read in step i - 1
    if constexpr (!SO) {
      uint32_t kb[C::KSTEPS], vb[2];
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        kb[ks] = kpat[ks] + s_cur;
        asm volatile("" : "+v"(kb[ks]));
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        vb[ct] = vpat[ct] + s_cur;
        asm volatile("" : "+v"(vb[ct]));
      }

      // Q operand (B of S^T and of the inter product): Q[jrow][32 ks + 8 g + 0..7].
      bf16x8 qop[C::KSTEPS];
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks)
        qop[ks] = *(const bf16x8 *)(smem + kb[ks] + (C::Q_OFF + 16 * R * C::ROWB));

      // S^T[16t + 4g + i][jrow] = P[jrow][16t + 4g + i] before masking.
      f32x4 sacc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          sacc[t] = mfma(*(const bf16x8 *)(smem + kb[ks] + (C::K_OFF + 16 * t * C::ROWB)),
                         qop[ks], sacc[t]);

      // Inter part: O^T[16ct + 4g + i][jrow] = sum_dk KV[dk][16ct + 4g + i] Q[jrow][dk].
      f32x4 o[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          o[ct] = mfma(*(const bf16x8 *)(smem + kb[ks] + (C::KVX_OFF + 16 * ct * C::ROWB)),
                       qop[ks], o[ct]);

      // V operands of the causal k-steps: lane (g, c) = V[32s + {4g+e, 16+4g+e}][16ct + c].
      bf16x8 vop[NS][2];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const bf16x4 lo = tr_read(smem + vb[ct] + (C::V_OFF + 32 * s * C::VROWB));
          const bf16x4 hi = tr_read(smem + vb[ct] + (C::V_OFF + (32 * s + 16) * C::VROWB));
          vop[s][ct] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }

      // Decay/causal mask in registers, then P in bf16 (tiles past the diagonal are zero).
      bf16x4 p[2 * NS];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4 m = sacc[t] * f32x4{maskw[t][0], maskw[t][1], maskw[t][2], maskw[t][3]};
        if (t == R) {
#pragma unroll
          for (int e = 0; e < 4; ++e) m[e] = keep[e] ? m[e] : 0.f;
        }
        p[t] = to_bf16x4(m);
      }
      if constexpr (NT % 2) p[NT] = bf16x4{(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};

      // O^T = lambda^(j+1) * inter + V^T P^T.
      const float isc = i == 0 ? inter_first : inter_scale;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) o[ct] *= isc;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 pop = __builtin_shufflevector(p[2 * s], p[2 * s + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) o[ct] = mfma(vop[s][ct], pop, o[ct]);
      }

      // Store: lane holds O[jrow][c0 + 16ct + 4g + 0..3]; rows past the end are dropped.
      {
        const Span sp = span_at<REV>(c, ws);
        const auto ro = rsrc(c.out + sp.off, sp.bytes);
        const uint32_t off = at<REV>(sp, ooff);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, to_bf16x4(o[ct])), ro,
                                                off + 32u * ct, 0, 0);
      }
    }  // !SO

    advance<REV>(c, ws);
    // Own rows of block i+1 landed: its DMA was issued in step i-1 (or the prologue); since
    // then this wave issued that step's stores (none in the prologue), this step's DMA and
    // stores.  Counting one step's stores only waits for step i-1's stores too, which were
    // issued a step ago.
    if constexpr (DMA > 0) wait_vm<DMA + STORES>();
    decay_v(i + 1, s_nxt);
    lds_barrier();
    const uint32_t so = s_cur;
    s_cur = s_nxt;
    s_nxt = s_prv;
    s_prv = so;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // DMAs in flight target this LDS
}

// ------------------------------------------------------------------------------------------
// State wave r: its band of the fp32 state.  Issues the DMA of K rows 16r..16r+15; the lightest
// state wave (r = 3) also issues the L2 prefetches.
// ------------------------------------------------------------------------------------------
template <int D, int R, bool SO, bool REV, bool SPLIT>
__device__ __forceinline__ void state_wave(const Chain &c, char *smem, const float *pw,
                                           const float *s0, float *fs, size_t sbase, int lane) {
  using C = Cfg<D>;
  using Bd = Band<D, R>;
  constexpr int RT = Bd::RT;
  constexpr int DK0 = Bd::DK0;
  constexpr bool PF = R == 3;
  constexpr int PF_DMA = pf_dma<SO>();
  constexpr int DMA = C::QK_DMA + (PF ? PF_DMA : 0);
  // Operations issued after a block's K DMA until the wait for it: the NST-2 later issues, plus,
  // with prefetches (issued after the K DMA of the same block), that block's own prefetches.
  constexpr int WAIT = (NST - 2) * DMA + (PF ? PF_DMA : 0);
  const int l16 = lane & 15, g = lane >> 4;
  const uint32_t smem_lds = lds_addr(smem);

  // kv[rt][ct][i] = KV[DK0 + 16 rt + 4 g + i][c0 + 16 ct + l16].
  f32x4 kv[RT > 0 ? RT : 1][2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dk = DK0 + 16 * rt + 4 * g + i, dv = c.c0 + 16 * ct + l16;
        if constexpr (SPLIT)  // the incoming state of the segment, formed in the prologue
          kv[rt][ct][i] = ((const float *)(smem + SIN_OFF<D>()))[dk * CV + 16 * ct + l16];
        else
          kv[rt][ct][i] =
              s0 ? s0[sbase + (c.s0t ? (size_t)dv * D + dk : (size_t)dk * D + dv)] : 0.f;
      }
  const int trow = 4 * g + (l16 >> 2), tcol = 4 * (l16 & 3);
  // Lane parts of the LDS addresses (see the output waves): state copy rows 16 ct + l16, K rows
  // 16 x + trow (transpose reads), decayed V rows 16 x + trow.
  uint32_t xpat[RT > 0 ? RT : 1], kpat[RT > 0 ? RT : 1], vpat[2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    xpat[rt] = (uint32_t)swz<D>(l16, DK0 + 16 * rt + 4 * g);
    kpat[rt] = (uint32_t)swz<D>(trow, DK0 + 16 * rt + tcol);
  }
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) vpat[ct] = (uint32_t)vswz(trow, 16 * ct + tcol);
  // bf16 copy of the state into the stage at st_off, for the inter product of its block
  auto write_kvx = [&](uint32_t st_off) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      uint32_t xb = xpat[rt] + st_off;
      asm volatile("" : "+v"(xb));
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        *(bf16x4 *)(smem + xb + (C::KVX_OFF + 16 * ct * C::ROWB)) = to_bf16x4(kv[rt][ct]);
    }
  };
  write_kvx(0);

  // lambda^b for full blocks and for the last block, which may be partial (b_last rows).
  const int b_last = c.b_last;
  const float lb_full = pw[BLK], lb_last = pw[b_last];
  // Block 0 decays the initial state by lambda^(b0 - 1) when it counts as inclusive.
  const int b0 = c.nb == 1 ? b_last : BLK;
  const float lb_first = c.incl ? pw[b0 - 1] : pw[b0];
  // Scale of the final state: lambda for an inclusive initial state (read now: the powers
  // table is overwritten by the pipeline's DMAs).
  const float fsc = c.incl && c.nb > 0 ? pw[1] : 1.f;

  uint32_t koff[C::QK_DMA];
  rows_offsets<D, REV>(R, lane, c.rowbytes, koff);
  const uint32_t pfoff = prefetch_offset<D, REV>(c.slice, lane, c.rowbytes);
  // Blocks whose K rows (wk) and L2 prefetch (wp) are issued next.
  Walk wk = walk_from<BLK, REV>(c, 0), wp = walk_from<BLK, REV>(c, PF_AHEAD);
  auto issue = [&](uint32_t st_off) {
    const uint32_t st = smem_lds + st_off;
    dma_rows<D, REV>(c.k, span_at<REV>(c, wk), koff, st + C::K_OFF + 16 * R * C::ROWB);
    advance<REV>(c, wk);
    // after the DMA, so that waiting for this DMA never waits for a prefetch (counters are
    // in order)
    if constexpr (PF) {
      prefetch_l2<SO, REV>(c, span_at<REV>(c, wp), pfoff, smem_lds + C::PF_OFF);
      advance<REV>(c, wp);
    }
  };
  if constexpr (PF) {
    // Blocks NST-1 .. PF_AHEAD-1 are not covered by the prefetches of the first issues.
    for (int blk = NST - 1; blk < PF_AHEAD; ++blk)
      prefetch_l2<SO, REV>(c, span_at<REV>(c, walk_from<BLK, REV>(c, blk)), pfoff,
                           smem_lds + C::PF_OFF);
  }
  static_assert(NST == 3, "stage rotation is written for three stages");
  uint32_t s_cur = 0, s_nxt = C::STAGE, s_prv = 2 * C::STAGE;
  issue(0);
  issue(C::STAGE);
  wait_vm_barrier<WAIT>();

  for (int i = 0; i < c.nb; ++i) {
    // A wave with a band issues its copies once its MFMAs are queued (they overlap them);
    // the copies of block i + 2 only need to land by the end of step i + 1.
    if constexpr (RT == 0) issue(s_prv);
    if constexpr (RT > 0) {
      uint32_t kb[RT], vb[2];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        kb[rt] = kpat[rt] + s_cur;
        asm volatile("" : "+v"(kb[rt]));
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        vb[ct] = vpat[ct] + s_cur;
        asm volatile("" : "+v"(vb[ct]));
      }
      const float lb = i == 0 ? lb_first : i == c.nb - 1 ? lb_last : lb_full;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) kv[rt][ct] *= lb;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 vop[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {  // lambda^(b-1-j) V[j]
          const bf16x4 lo = tr_read(smem + vb[ct] + (C::LV_OFF + 32 * s * C::VROWB));
          const bf16x4 hi = tr_read(smem + vb[ct] + (C::LV_OFF + (32 * s + 16) * C::VROWB));
          vop[ct] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const bf16x4 lo = tr_read(smem + kb[rt] + (C::K_OFF + 32 * s * C::ROWB));
          const bf16x4 hi = tr_read(smem + kb[rt] + (C::K_OFF + (32 * s + 16) * C::ROWB));
          const bf16x8 kop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) kv[rt][ct] = mfma(kop, vop[ct], kv[rt][ct]);
        }
      }
      issue(s_prv);  // block i + 2
      write_kvx(s_nxt);
    }
    // Block i+1's K rows landed: since their DMA this wave issued only the later issues.
    wait_vm_barrier<WAIT>();
    const uint32_t so = s_cur;
    s_cur = s_nxt;
    s_nxt = s_prv;
    s_prv = so;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (fs) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dk = DK0 + 16 * rt + 4 * g + i, dv = c.c0 + 16 * ct + l16;
          fs[sbase + (size_t)dk * D + dv] = kv[rt][ct][i] * fsc;
        }
  }
}

// Sequence-split form (SPLIT): one workgroup per segment slot of la_prefill_split's segment
// numbering (seg_lookup.h); the workgroup finds its segment and forms its incoming state itself,
// in the prologue, from the states the segment-state pass left for the earlier segments of its
// sequence: S_in(j) = lambda^L S_in(j-1) + L(j-1), S_in(0) = the sequence's initial state (or
// zero), L = the segment length, in fp32 with the rounding of the separate combine pass
// (seg_decay, one fmaf per step).  The slice's S_in (D x 32 fp32) goes through LDS to the state
// waves: it sits in the last stage after the powers table (SIN_OFF), which the first copy into
// that stage (block 2, after the prologue barrier) overwrites.
// flags: bit 1 inclusive initial state (only for sequences s with incl_v[s] != 0 when incl_v is
// given), bit 2 transposed initial state.  SO: compute only the
// final state (q and out are not touched).  REV: reversed (anti-causal) scan.
template <int D, bool SO, bool REV, bool SPLIT>
__global__ __launch_bounds__(NTHR, 1) void prefill_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ decay, const int32_t *__restrict__ cu,
    const float *__restrict__ s0, __bf16 *__restrict__ out, float *__restrict__ fs, int64_t T,
    int S, int H, int flags, const int32_t *__restrict__ incl_v, int64_t seg_len,
    const float *__restrict__ seg_states, int nslot, int sub) {
  using C = Cfg<D>;
  constexpr int NS = D / CV;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
  // lambda^m, m = 0..BLK: lives in the last stage until that stage's first DMA, which every
  // wave issues only after it has copied the powers it needs into registers.
  float *const pw = (float *)(smem + (NST - 1) * C::STAGE);

  int chain, slice;
  xcd_chain_slice(blockIdx.x, (SPLIT ? nslot : S) * H * NS, NS, chain, slice);
  const int seq = chain / H, h = chain % H;
  Chain c;
  int64_t tok0, tok1;
  SegPos sp{};
  if constexpr (SPLIT) {
    sp = find_segment(cu, T, S, seg_len, seq);  // the same in every wave
    if (sp.seq < 0) return;                     // an unused slot: the whole workgroup
    tok0 = sp.tok0;
    tok1 = sp.tok1;
  } else {
    tok0 = cu ? (int64_t)cu[seq] : 0;
    tok1 = cu ? (int64_t)cu[seq + 1] : T;
  }
  const int64_t first = (tok0 * H + h) * D;  // element offset of (tok0, h, 0)
  c.q = (const char *)(q + first);
  c.k = (const char *)(k + first);
  c.v = (const char *)(v + first);
  c.n = tok1 > tok0 ? tok1 - tok0 : 0;
  c.nb = (int)((c.n + BLK - 1) / BLK);
  c.b_last = c.nb > 0 ? (int)(c.n - (int64_t)(c.nb - 1) * BLK) : BLK;
  c.rowbytes = (uint32_t)H * D * 2;
  c.full_bytes = (uint32_t)BLK * c.rowbytes;
  c.last_bytes = (uint32_t)c.b_last * c.rowbytes;
  c.full_last = (uint32_t)(BLK - 1) * c.rowbytes;
  c.last_last = (uint32_t)(c.b_last - 1) * c.rowbytes;
  c.c0 = slice * CV;
  c.slice = slice;
  c.out = (char *)(out + first + c.c0);
  c.incl = (flags & 2) && (incl_v == nullptr || incl_v[seq] != 0);
  c.s0t = flags & 4;

  const int tid = threadIdx.x;
  const float lam = decay[h];
  // The split form's incoming-state loads go out first, in flight during the LDS zeroing and
  // the powers table.
  IncomingState<D, CV, NTHR> incoming;
  if constexpr (SPLIT) incoming.issue(s0, seg_states, sp, sub, H, h, c.c0, tid);
  // Zero the stages once: rows a partial block does not load then hold zeros or finite values
  // of earlier blocks, never stale bits from another kernel.
  for (int off = 16 * tid; off < NST * C::STAGE; off += 16 * NTHR)
    *(u32x4 *)(smem + off) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  if (tid <= BLK) pw[tid] = seg_decay(lam, tid);  // lambda^tid in fp64 (0^0 = 1), then fp32
  size_t sbase = ((size_t)seq * H + h) * (size_t)D * D;
  if constexpr (SPLIT) {
    // S_in lies past the powers table, in the zeroed stages: it needs no barrier of its own
    incoming.finish((float *)(smem + SIN_OFF<D>()), seg_states, sp, sub, H, h, c.c0,
                    seg_decay(lam, seg_len / sub), tid);
    // the final state is the sequence's, written by its last segment only
    sbase = ((size_t)sp.seq * H + h) * (size_t)D * D;
    if (sp.j != sp.count - 1) fs = nullptr;
  }
  __syncthreads();  // the powers, S_in and the zeroed stages visible before any copy or read
  const int lane = tid & 63;
  switch (tid >> 6) {
    case 0: output_wave<D, 0, SO, REV>(c, smem, pw, lane); break;
    case 1: output_wave<D, 1, SO, REV>(c, smem, pw, lane); break;
    case 2: output_wave<D, 2, SO, REV>(c, smem, pw, lane); break;
    case 3: output_wave<D, 3, SO, REV>(c, smem, pw, lane); break;
    case 4: state_wave<D, 0, SO, REV, SPLIT>(c, smem, pw, s0, fs, sbase, lane); break;
    case 5: state_wave<D, 1, SO, REV, SPLIT>(c, smem, pw, s0, fs, sbase, lane); break;
    case 6: state_wave<D, 2, SO, REV, SPLIT>(c, smem, pw, s0, fs, sbase, lane); break;
    default: state_wave<D, 3, SO, REV, SPLIT>(c, smem, pw, s0, fs, sbase, lane); break;
  }
}

template <int D, bool SO, bool REV>
hipError_t launch(const LaPrefillArgs &a, hipStream_t stream) {
  const int NS = D / CV;
  const long long grid = (long long)a.S * a.H * NS;
  if (grid <= 0) return hipSuccess;
  const int flags = (a.init_inclusive ? 2 : 0) | (a.init_transposed ? 4 : 0);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, SO, REV, false>), dim3((unsigned)grid), dim3(NTHR), 0, stream,
                     (const __bf16 *)a.q, (const __bf16 *)a.k, (const __bf16 *)a.v, a.decay,
                     a.cu_seqlens, a.initial_state, (__bf16 *)a.out, a.final_state, a.T, a.S,
                     a.H, flags, a.seq_incl, (int64_t)0, nullptr, 0, 1);
  return hipGetLastError();
}

}  // namespace

hipError_t la_launch_prefill_bf16(const LaPrefillArgs &a, hipStream_t stream) {
  if (a.state_only && a.reverse)
    return a.D == 128 ? launch<128, true, true>(a, stream) : launch<64, true, true>(a, stream);
  if (a.state_only)
    return a.D == 128 ? launch<128, true, false>(a, stream) : launch<64, true, false>(a, stream);
  if (a.reverse)
    return a.D == 128 ? launch<128, false, true>(a, stream) : launch<64, false, true>(a, stream);
  return a.D == 128 ? launch<128, false, false>(a, stream) : launch<64, false, false>(a, stream);
}

hipError_t la_launch_prefill_split_bf16(const LaPrefillArgs &a, int64_t seg_len,
                                        const float *seg_states, int32_t nslot, int32_t sub,
                                        hipStream_t stream) {
  if (sub < 1 || seg_len % sub != 0) return hipErrorInvalidValue;
  const int NS = a.D / CV;
  const long long grid = (long long)nslot * a.H * NS;
  if (grid <= 0) return hipSuccess;
  if (a.D == 128)
    hipLaunchKernelGGL((prefill_bf16_kernel<128, false, false, true>), dim3((unsigned)grid),
                       dim3(NTHR), 0, stream, (const __bf16 *)a.q, (const __bf16 *)a.k,
                       (const __bf16 *)a.v, a.decay, a.cu_seqlens, a.initial_state,
                       (__bf16 *)a.out, a.final_state, a.T, a.S, a.H, 0, nullptr, seg_len,
                       seg_states, nslot, sub);
  else
    hipLaunchKernelGGL((prefill_bf16_kernel<64, false, false, true>), dim3((unsigned)grid),
                       dim3(NTHR), 0, stream, (const __bf16 *)a.q, (const __bf16 *)a.k,
                       (const __bf16 *)a.v, a.decay, a.cu_seqlens, a.initial_state,
                       (__bf16 *)a.out, a.final_state, a.T, a.S, a.H, 0, nullptr, seg_len,
                       seg_states, nslot, sub);
  return hipGetLastError();
}
