// prefill_bf16_b128.hip -- lightning-attention prefill with 128-token blocks, bf16 storage,
// MFMA, fp32 state (gfx950).
//
// The block algorithm of prefill_bf16.hip (intra-block left product ((Q K^T) masked) V, inter-block
// right product Q KV through a running d x d state: "MiniMax-01 technical report digest",
// futurefh.com, section 1) with blocks of B = 128 tokens instead of 64.  The split into blocks is
// exact algebra for any B, so the result differs from the 64-token kernel only in rounding.  For
// block i of b rows (KV_{-1} = the initial state):
//
//   O_i  = ((Q_i K_i^T) * M) V_i + diag(lambda^(j+1)) Q_i KV_{i-1},
//          M[j][j'] = lambda^(j-j') for j' <= j, else exactly 0 (a select)
//   KV_i = lambda^b KV_{i-1} + K_i^T diag(lambda^(b-1-j)) V_i
//
// A longer block halves the serial block steps of a chain, and with them the per-step barrier,
// the waits for copies and the bf16 state copy, at the price of a larger intra-block product
// (4 B d + 4 d^2 FLOP per token-head).  Modes as in prefill_bf16.hip, for the backward's scans:
// a reversed scan (REV: local token t is physical token n-1-t), an initial state that counts as
// inclusive (weight lambda^t at local token t, final state times lambda; optionally only for
// flagged sequences) and a transposed one; and the sequence-split form (SPLIT).  No state-only
// form (prefill_bf16.hip has it).
//
// Work decomposition: as in prefill_bf16.hip, one workgroup of 8 waves per (sequence, head,
// 32-column slice of the value dimension), workgroups mapped so that the slices of a head share an
// XCD.  A block has eight 16-row groups:
//   * output wave w (w = 0..3) owns groups w and 7 - w (9 causal score tiles in all, the same for
//     every w): S^T = K Q^T, the decay mask in registers, O^T = lambda^(j+1) KV^T Q^T + V^T P^T
//     for both groups (the K tiles and the state copy are read once for both), and the stores.  It
//     copies its own Q rows;
//   * state wave r holds rows 32r..32r+31 (d = 128; 16r..16r+15 at d = 64) of the fp32 state
//     slice in MFMA accumulators for the whole sequence, KV = lambda^b KV + K^T (Lambda V) over
//     the block's 128 tokens, and publishes a bf16 copy of its rows.  It copies K and V rows
//     32r..32r+31 and writes those V rows decayed, lambda^(b-1-j) V[j], for the state product.
//     (Measured: with the V copies and the decay in the output waves instead, which carry the
//     critical path, the kernel is 0.4-0.9% slower.)
// LDS: a two-stage ring, each stage holding a block's K and V rows, the bf16 state copy the block
// starts from and its decayed V rows (56 KiB at d = 128), plus one Q buffer.  Only the output wave
// that owns a Q row copies and reads it, so each output wave copies its next block's Q rows as
// soon as it has read the current ones into registers, with no barrier.  K and V of block i + 1
// are copied during step i into the stage block i - 1 used; the last state wave pulls block i + 2
// into L2 during step i, so those copies hit L2.  One barrier per block.
#include "la_internal.h"
#include "bf16_tiles.h"
#include "seg_lookup.h"

namespace {

constexpr int BLK = 128;  // tokens per block
constexpr int NST = 2;    // stages of the K/V ring
constexpr int NG = BLK / 16;  // 16-row groups per block

template <int D>
struct Cfg : RowCfg<D> {
  using RowCfg<D>::ROWB;
  using RowCfg<D>::VROWB;
  // byte offsets inside a stage
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = BLK * ROWB;
  static constexpr int KVX_OFF = V_OFF + BLK * VROWB;  // bf16 state copy [CV][D]
  static constexpr int LV_OFF = KVX_OFF + CV * ROWB;   // decayed V rows [BLK][CV]
  static constexpr int STAGE = LV_OFF + BLK * VROWB;
  static constexpr int Q_OFF = NST * STAGE;            // the Q buffer [BLK][D]
  static constexpr int PF_OFF = Q_OFF + BLK * ROWB;    // 1 KiB sink of the L2 prefetches
  static constexpr int SMEM = PF_OFF + 1024;
  static_assert(STAGE < 65536 && BLK * ROWB < 65536,
                "stage and Q offsets must fit the LDS instruction offset");
};

// Sequence-split form (SPLIT): one workgroup per segment slot of la_prefill_split's segment
// numbering (seg_lookup.h), which finds its segment and forms its incoming state in the
// prologue from the states the segment-state pass left (IncomingState).  The slice's
// incoming state (D x 32 fp32) reaches the state waves through LDS, after the powers table in
// stage 1, which the first copies into that stage (step 0, after the prologue barrier) overwrite.
template <int D>
constexpr int SIN_OFF() { return Cfg<D>::STAGE + 1024; }

// State rows of state wave r: 16-row tiles [TILES r, TILES (r + 1)).
template <int D>
constexpr int state_tiles() { return D / 64; }

// L2 prefetch of the slice's share of a block's q, k and full v rows: one 16-byte read per
// 128-byte line into a sink in LDS that nothing reads.  d = 128: four slices of 32 rows of two
// lines; d = 64: two slices of 64 rows of one line.
template <int D, bool REV>
__device__ __forceinline__ uint32_t prefetch_offset(int slice, int lane, uint32_t rowbytes) {
  if constexpr (D == 128)
    return lane_base<REV>(32 * slice + (lane >> 1), (uint32_t)(lane & 1) * 128u, rowbytes);
  else
    return lane_base<REV>(64 * slice + lane, 0u, rowbytes);
}

// ------------------------------------------------------------------------------------------
// Output wave W: row groups GA = W and GB = 7 - W of every block.
// ------------------------------------------------------------------------------------------
template <int D, int W, bool REV>
__device__ __forceinline__ void output_wave(const Chain &c, char *smem, const float *pw,
                                            int lane) {
  using C = Cfg<D>;
  constexpr int GA = W, GB = NG - 1 - W;
  constexpr int NTA = GA + 1, NTB = GB + 1;            // causal score tiles of each group
  constexpr int NSA = (NTA + 1) / 2, NSB = (NTB + 1) / 2;  // 32-token k-steps of the intra product
  constexpr int STORES = 4;                           // two groups x two 16-column tiles
  const int l16 = lane & 15, g = lane >> 4;
  const int jA = 16 * GA + l16, jB = 16 * GB + l16;  // the lane's output rows inside a block
  const uint32_t smem_lds = lds_addr(smem);
  const uint32_t rowbytes = c.rowbytes;

  // Decay weights lambda^(j - j'), j' = 16 t + 4 g + i; the diagonal tile (t = G) has entries
  // above the diagonal, which are selected away.
  float mA[NTA][4], mB[NTB][4];
  bool keepA[4], keepB[4];
#pragma unroll
  for (int t = 0; t < NTB; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jp = 16 * t + 4 * g + i;
      mB[t][i] = jp <= jB ? pw[jB - jp] : 0.f;
      if (t == GB) keepB[i] = jp <= jB;
      if (t < NTA) {
        mA[t][i] = jp <= jA ? pw[jA - jp] : 0.f;
        if (t == GA) keepA[i] = jp <= jA;
      }
    }
  const float iscA = pw[jA + 1], iscB = pw[jB + 1];
  // Block 0 applies the initial state; weighted lambda^j instead when it counts as inclusive.
  const float iscA0 = c.incl ? pw[jA] : iscA, iscB0 = c.incl ? pw[jB] : iscB;

  // Lane offsets of the Q copies of both groups and of the stores.
  uint32_t qoffA[C::QK_DMA], qoffB[C::QK_DMA];
  rows_offsets<D, REV>(GA, lane, rowbytes, qoffA);
  rows_offsets<D, REV>(GB, lane, rowbytes, qoffB);
  const uint32_t ooffA = lane_base<REV>(jA, 8u * g, rowbytes);
  const uint32_t ooffB = lane_base<REV>(jB, 8u * g, rowbytes);
  const uint32_t qA_lds = smem_lds + C::Q_OFF + 16 * GA * C::ROWB;
  const uint32_t qB_lds = smem_lds + C::Q_OFF + 16 * GB * C::ROWB;

  // Lane parts of the LDS read addresses: rows 16 x + l16 of a swizzled [rows][D] tile share the
  // pattern of row l16; V rows 16 x + trow share that of row trow.
  const int trow = 4 * g + (l16 >> 2), tcol = 4 * (l16 & 3);
  uint32_t kpat[C::KSTEPS], vpat[2];
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks) kpat[ks] = (uint32_t)swz<D>(l16, 32 * ks + 8 * g);
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) vpat[ct] = (uint32_t)vswz(trow, 16 * ct + tcol);

  Walk wq = walk_from<BLK, REV>(c, 0), ws = walk_from<BLK, REV>(c, 0);
  // Q rows of the next block into the Q buffer.
  auto issue_q = [&]() {
    const Span sp = span_at<REV>(c, wq);
    advance<REV>(c, wq);
    dma_rows<D, REV>(c.q, sp, qoffA, qA_lds);
    dma_rows<D, REV>(c.q, sp, qoffB, qB_lds);
  };
  issue_q();
  wait_vm<0>();
  lds_barrier();  // block 0, its decayed V and the initial state copy visible to all waves

  uint32_t s_cur = 0, s_nxt = C::STAGE;
  for (int i = 0; i < c.nb; ++i) {
    // Own Q rows of block i landed: since their copy this wave issued only the previous
    // block's stores.
    wait_vm<STORES>();
    bf16x8 qa[C::KSTEPS], qb[C::KSTEPS];
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      qa[ks] = *(const bf16x8 *)(smem + ((qA_lds - smem_lds) + kpat[ks]));
      qb[ks] = *(const bf16x8 *)(smem + ((qB_lds - smem_lds) + kpat[ks]));
    }
    // The Q rows are in registers before their buffer is overwritten with the next block's.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue_q();

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

    // Scores: sX[t][i] = S^T[16 t + 4 g + i][jX] before masking; every K tile read once.
    f32x4 sA[NTA], sB[NTB];
#pragma unroll
    for (int t = 0; t < NTB; ++t) {
      sB[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (t < NTA) sA[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
      for (int t = 0; t < NTB; ++t) {
        const bf16x8 kt = *(const bf16x8 *)(smem + kb[ks] + (C::K_OFF + 16 * t * C::ROWB));
        sB[t] = mfma(kt, qb[ks], sB[t]);
        if (t < NTA) sA[t] = mfma(kt, qa[ks], sA[t]);
      }

    // Inter part: O^T[16 ct + 4 g + i][jX] = sum_dk KV[dk][16 ct + 4 g + i] Q[jX][dk].
    f32x4 oA[2], oB[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) oA[ct] = oB[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const bf16x8 kv = *(const bf16x8 *)(smem + kb[ks] + (C::KVX_OFF + 16 * ct * C::ROWB));
        oA[ct] = mfma(kv, qa[ks], oA[ct]);
        oB[ct] = mfma(kv, qb[ks], oB[ct]);
      }

    // V operands of the causal k-steps: lane (g, c) = V[32 s + {4 g + e, 16 + 4 g + e}][16 ct + c].
    bf16x8 vop[NSB][2];
#pragma unroll
    for (int s = 0; s < NSB; ++s)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const bf16x4 lo = tr_read(smem + vb[ct] + (C::V_OFF + 32 * s * C::VROWB));
        const bf16x4 hi = tr_read(smem + vb[ct] + (C::V_OFF + (32 * s + 16) * C::VROWB));
        vop[s][ct] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }

    // Decay/causal mask in registers, then P in bf16 (a padding tile past the diagonal is zero).
    bf16x4 pA[2 * NSA], pB[2 * NSB];
#pragma unroll
    for (int t = 0; t < NTB; ++t) {
      f32x4 m = sB[t] * f32x4{mB[t][0], mB[t][1], mB[t][2], mB[t][3]};
      if (t == GB) {
#pragma unroll
        for (int e = 0; e < 4; ++e) m[e] = keepB[e] ? m[e] : 0.f;
      }
      pB[t] = to_bf16x4(m);
    }
    if constexpr (NTB % 2) pB[NTB] = bf16x4{(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
#pragma unroll
    for (int t = 0; t < NTA; ++t) {
      f32x4 m = sA[t] * f32x4{mA[t][0], mA[t][1], mA[t][2], mA[t][3]};
      if (t == GA) {
#pragma unroll
        for (int e = 0; e < 4; ++e) m[e] = keepA[e] ? m[e] : 0.f;
      }
      pA[t] = to_bf16x4(m);
    }
    if constexpr (NTA % 2) pA[NTA] = bf16x4{(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};

    // O^T = lambda^(j+1) * inter + V^T P^T.
    const float ia = i == 0 ? iscA0 : iscA, ib = i == 0 ? iscB0 : iscB;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      oA[ct] *= ia;
      oB[ct] *= ib;
    }
#pragma unroll
    for (int s = 0; s < NSB; ++s) {
      const bf16x8 popB = __builtin_shufflevector(pB[2 * s], pB[2 * s + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) oB[ct] = mfma(vop[s][ct], popB, oB[ct]);
      if (s < NSA) {
        const bf16x8 popA =
            __builtin_shufflevector(pA[2 * s], pA[2 * s + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) oA[ct] = mfma(vop[s][ct], popA, oA[ct]);
      }
    }

    // Store: lane holds O[jX][c0 + 16 ct + 4 g + 0..3]; rows past the end are dropped.
    {
      const Span sp = span_at<REV>(c, ws);
      const auto ro = rsrc(c.out + sp.off, sp.bytes);
      const uint32_t oa = at<REV>(sp, ooffA), ob = at<REV>(sp, ooffB);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, to_bf16x4(oA[ct])), ro,
                                              oa + 32u * ct, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, to_bf16x4(oB[ct])), ro,
                                              ob + 32u * ct, 0, 0);
      }
    }
    advance<REV>(c, ws);
    lds_barrier();
    const uint32_t so = s_cur;
    s_cur = s_nxt;
    s_nxt = so;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // copies in flight target this LDS
}

// ------------------------------------------------------------------------------------------
// State wave R: state rows [16 RT R, 16 RT (R + 1)) of the slice.  Copies K rows
// [BLK/4 R, BLK/4 (R + 1)); the last state wave also issues the L2 prefetches.
// ------------------------------------------------------------------------------------------
template <int D, int R, bool REV, bool SPLIT>
__device__ __forceinline__ void state_wave(const Chain &c, char *smem, const float *pw,
                                           const float *s0, float *fs, size_t sbase, int lane) {
  using C = Cfg<D>;
  constexpr int RT = state_tiles<D>();
  constexpr int DK0 = 16 * RT * R;
  constexpr bool PF = R == 3;
  constexpr int PF_DMA = 3;
  const int l16 = lane & 15, g = lane >> 4;
  const uint32_t smem_lds = lds_addr(smem);

  // kv[rt][ct][i] = KV[DK0 + 16 rt + 4 g + i][c0 + 16 ct + l16].
  f32x4 kv[RT][2];
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
  uint32_t xpat[RT], kpat[RT], vpat[2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    xpat[rt] = (uint32_t)swz<D>(l16, DK0 + 16 * rt + 4 * g);
    kpat[rt] = (uint32_t)swz<D>(trow, DK0 + 16 * rt + tcol);
  }
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) vpat[ct] = (uint32_t)vswz(trow, 16 * ct + tcol);
  // bf16 copy of the state rows into the stage at st_off, for the inter product of its block
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

  // lambda^b for the first, full and last blocks (read now: the stage holding the powers is
  // overwritten by the first copies of step 0).
  const int b_last = c.b_last;
  const int b0 = c.nb == 1 ? b_last : BLK;
  // Block 0 decays the initial state by lambda^(b0 - 1) when it counts as inclusive.
  const float lb_full = pw[BLK], lb_last = pw[b_last], lb_first = c.incl ? pw[b0 - 1] : pw[b0];
  // Final state scale: lambda for an inclusive initial state (read now, before the stage holding
  // the powers is overwritten).
  const float fsc = c.incl && c.nb > 0 ? pw[1] : 1.f;

  // K rows [BLK/4 R, BLK/4 (R + 1)) as NG/4 16-row groups.
  constexpr int KG = NG / 4;
  uint32_t koff[KG][C::QK_DMA];
#pragma unroll
  for (int x = 0; x < KG; ++x) rows_offsets<D, REV>(KG * R + x, lane, c.rowbytes, koff[x]);
  const uint32_t pfoff = prefetch_offset<D, REV>(c.slice, lane, c.rowbytes);
  Walk wk = walk_from<BLK, REV>(c, 0), wp = walk_from<BLK, REV>(c, 1);
  auto issue_k = [&](uint32_t st_off) {
    const Span sp = span_at<REV>(c, wk);
    advance<REV>(c, wk);
#pragma unroll
    for (int x = 0; x < KG; ++x)
      dma_rows<D, REV>(c.k, sp, koff[x], smem_lds + st_off + C::K_OFF +
                                               16 * (KG * R + x) * C::ROWB);
  };
  // Pull the block after the next one into L2 (issued after the K copies, so that waiting for
  // them never waits for a prefetch: counters are in order).
  auto prefetch = [&]() {
    if constexpr (PF) {
      const Span sp = span_at<REV>(c, wp);
      advance<REV>(c, wp);
      dma16_same3(rsrc(c.q + sp.off, sp.bytes), rsrc(c.k + sp.off, sp.bytes),
                  rsrc(c.v + sp.off, sp.bytes), at<REV>(sp, pfoff), smem_lds + C::PF_OFF);
    }
  };
  // V rows 32R..32R+31 (two 1 KiB copies) and their decayed copy lambda^(b-1-j) V[j], which the
  // state product reads.
  const int vr0 = 32 * R + lane / 4, vr1 = vr0 + 16;
  const uint32_t voff0 = lane_base<REV>(vr0, 16u * ((lane % 4) ^ vswf(vr0)), c.rowbytes);
  // forward: the second copy's instruction offset adds 1 KiB back (rows >= 16)
  const uint32_t voff1 =
      lane_base<REV>(vr1, 16u * ((lane % 4) ^ vswf(vr1)), c.rowbytes) - (REV ? 0u : 1024u);
  const float lv0_full = pw[BLK - 1 - vr0], lv1_full = pw[BLK - 1 - vr1];
  const float lv0_last = vr0 < b_last ? pw[b_last - 1 - vr0] : 0.f;
  const float lv1_last = vr1 < b_last ? pw[b_last - 1 - vr1] : 0.f;
  const uint32_t dpat = (uint32_t)(vr0 * C::VROWB + 16 * (lane % 4));
  const char *vslice = c.v + 2 * c.c0;
  Walk wv = walk_from<BLK, REV>(c, 0);
  auto issue_v = [&](uint32_t st_off) {
    const Span sp = span_at<REV>(c, wv);
    advance<REV>(c, wv);
    const uint32_t lds = smem_lds + st_off + C::V_OFF + 32 * R * C::VROWB;
    if constexpr (REV)
      dma16x2(rsrc(vslice + sp.off, sp.bytes), at<REV>(sp, voff0), at<REV>(sp, voff1), lds,
              lds + 1024);
    else
      dma_kib2(rsrc(vslice + sp.off, sp.bytes), voff0, voff1, lds);
  };
  // The decayed copy of the rows of block blk (landed in the stage at st_off), in that stage.
  auto decay_v = [&](int blk, uint32_t st_off) {
    const bool last = blk == c.nb - 1;
    uint32_t d = dpat + st_off;
    asm volatile("" : "+v"(d));
    const bf16x8 x0 = *(const bf16x8 *)(smem + d + C::V_OFF);
    const bf16x8 x1 = *(const bf16x8 *)(smem + d + C::V_OFF + 16 * C::VROWB);
    *(bf16x8 *)(smem + d + C::LV_OFF) = scale8(x0, last ? lv0_last : lv0_full);
    *(bf16x8 *)(smem + d + C::LV_OFF + 16 * C::VROWB) = scale8(x1, last ? lv1_last : lv1_full);
  };
  issue_k(0);
  issue_v(0);
  prefetch();  // block 1
  wait_vm<PF ? PF_DMA : 0>();
  decay_v(0, 0);
  wait_vm_barrier<PF ? PF_DMA : 0>();

  uint32_t s_cur = 0, s_nxt = C::STAGE;
  for (int i = 0; i < c.nb; ++i) {
    issue_k(s_nxt);  // block i + 1, into the stage block i - 1 used
    issue_v(s_nxt);
    prefetch();      // block i + 2
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
    for (int s = 0; s < BLK / 32; ++s) {
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
    write_kvx(s_nxt);
    // Own K and V rows of block i + 1 landed (only the prefetch was issued after them).
    wait_vm<PF ? PF_DMA : 0>();
    decay_v(i + 1, s_nxt);
    wait_vm_barrier<PF ? PF_DMA : 0>();
    const uint32_t so = s_cur;
    s_cur = s_nxt;
    s_nxt = so;
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

template <int D, bool REV, bool SPLIT>
__global__ __launch_bounds__(NTHR, 1) void prefill_bf16_b128_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ decay, const int32_t *__restrict__ cu,
    const float *__restrict__ s0, __bf16 *__restrict__ out, float *__restrict__ fs, int64_t T,
    int S, int H, int flags, const int32_t *__restrict__ incl_v, int64_t seg_len,
    const float *__restrict__ seg_states, int nslot, int sub) {
  using C = Cfg<D>;
  constexpr int NS = D / CV;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
  // lambda^m, m = 0..BLK: lives in stage 1 until its first copy (step 0), which every wave issues
  // only after it has copied the powers it needs into registers (before the prologue barrier).
  float *const pw = (float *)(smem + C::STAGE);

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
  // flags bit 1: inclusive initial state (only for sequences s with incl_v[s] != 0 when incl_v
  // is given); bit 2: transposed initial state
  c.incl = (flags & 2) && (incl_v == nullptr || incl_v[seq] != 0);
  c.s0t = flags & 4;

  const int tid = threadIdx.x;
  const float lam = decay[h];
  // The split form's incoming-state loads go out first, in flight during the LDS zeroing and
  // the powers table.
  IncomingState<D, CV, NTHR> incoming;
  if constexpr (SPLIT) incoming.issue(s0, seg_states, sp, sub, H, h, c.c0, tid);
  // Zero the stages and the Q buffer once: rows a partial block does not load then hold zeros
  // or finite values of earlier blocks, never stale bits of another kernel.
  for (int off = 16 * tid; off < C::PF_OFF; off += 16 * NTHR)
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
    case 0: output_wave<D, 0, REV>(c, smem, pw, lane); break;
    case 1: output_wave<D, 1, REV>(c, smem, pw, lane); break;
    case 2: output_wave<D, 2, REV>(c, smem, pw, lane); break;
    case 3: output_wave<D, 3, REV>(c, smem, pw, lane); break;
    case 4: state_wave<D, 0, REV, SPLIT>(c, smem, pw, s0, fs, sbase, lane); break;
    case 5: state_wave<D, 1, REV, SPLIT>(c, smem, pw, s0, fs, sbase, lane); break;
    case 6: state_wave<D, 2, REV, SPLIT>(c, smem, pw, s0, fs, sbase, lane); break;
    default: state_wave<D, 3, REV, SPLIT>(c, smem, pw, s0, fs, sbase, lane); break;
  }
}

template <int D, bool REV>
hipError_t launch(const LaPrefillArgs &a, hipStream_t stream) {
  const int NS = D / CV;
  const long long grid = (long long)a.S * a.H * NS;
  if (grid <= 0) return hipSuccess;
  const int flags = (a.init_inclusive ? 2 : 0) | (a.init_transposed ? 4 : 0);
  hipLaunchKernelGGL((prefill_bf16_b128_kernel<D, REV, false>), dim3((unsigned)grid), dim3(NTHR),
                     0, stream, (const __bf16 *)a.q, (const __bf16 *)a.k, (const __bf16 *)a.v,
                     a.decay, a.cu_seqlens, a.initial_state, (__bf16 *)a.out, a.final_state,
                     a.T, a.S, a.H, flags, a.seq_incl, (int64_t)0, nullptr, 0, 1);
  return hipGetLastError();
}

template <int D>
hipError_t launch_split(const LaPrefillArgs &a, int64_t seg_len, const float *seg_states,
                        int32_t nslot, int32_t sub, hipStream_t stream) {
  const int NS = D / CV;
  const long long grid = (long long)nslot * a.H * NS;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_bf16_b128_kernel<D, false, true>), dim3((unsigned)grid),
                     dim3(NTHR), 0, stream, (const __bf16 *)a.q, (const __bf16 *)a.k,
                     (const __bf16 *)a.v, a.decay, a.cu_seqlens, a.initial_state,
                     (__bf16 *)a.out, a.final_state, a.T, a.S, a.H, 0, nullptr, seg_len,
                     seg_states, nslot, sub);
  return hipGetLastError();
}

}  // namespace

hipError_t la_launch_prefill_bf16_b128(const LaPrefillArgs &a, hipStream_t stream) {
  if (a.state_only) return hipErrorInvalidValue;  // not built for this kernel
  if (a.reverse)
    return a.D == 128 ? launch<128, true>(a, stream) : launch<64, true>(a, stream);
  return a.D == 128 ? launch<128, false>(a, stream) : launch<64, false>(a, stream);
}

hipError_t la_launch_prefill_split_bf16_b128(const LaPrefillArgs &a, int64_t seg_len,
                                             const float *seg_states, int32_t nslot,
                                             int32_t sub, hipStream_t stream) {
  if (seg_len % BLK != 0) return hipErrorInvalidValue;  // segments of whole 128-token blocks
  if (sub < 1 || seg_len % sub != 0) return hipErrorInvalidValue;
  return a.D == 128 ? launch_split<128>(a, seg_len, seg_states, nslot, sub, stream)
                    : launch_split<64>(a, seg_len, seg_states, nslot, sub, stream);
}
