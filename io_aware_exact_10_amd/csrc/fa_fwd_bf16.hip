// Forward pass, bf16 in/out, fp32 accumulation, gfx950 MFMA.
//
// Method: exact softmax attention with the online softmax, tile by tile
// ("FlashAttention: exact attention made fast by counting memory traffic",
// "The method"; "FlashAttention and IO-aware exact attention", "Core ideas":
// online softmax, tiling and fusion, one log-sum-exp per row). Only O and the
// row log-sum-exp are written; the N x N scores stay in registers.
//
// Work decomposition: one workgroup per (query tile, batch, head), or with a
// causal mask over a dense batch per pair of query tiles of one (batch, head)
// whose visible key ranges add up to the same length; each wave owns 32
// query rows (4 waves, 128 rows, or 8 waves, 256 rows, for long sequences;
// 32 and 64 rows on request), and query tiles run in parallel over the
// sequence ("Core ideas": parallelism over the sequence dimension). The
// workgroup streams 64-key tiles of K and V through LDS,
// double-buffered: tile t+1 is copied global -> LDS asynchronously (no
// registers) while tile t is computed.
//
// Per wave and key tile (two 32-key sub-blocks):
//   S^T = K Q^T     A = K rows from LDS, B = Q fragment held in registers.
//                   The C layout puts one query per lane (n = lane % 32) and
//                   16 keys per lane, so the row max and row sum are
//                   lane-local plus one exchange with lane ^ 32.
//   online softmax  p = 2^(c*s - m) with c = |scale| * log2(e) folded into
//                   one FMA. The reference max m is raised only when some row
//                   of the wave exceeds it by more than 8 (in log2 units);
//                   then acc and l are multiplied by 2^(m_old - m_new). Any
//                   reference max gives the same O = acc / l; this one keeps
//                   p <= 2^8 and skips almost every rescale.
//   O^T += V^T P^T  B = P^T straight from the S^T registers (rounded to
//                   bf16), A = V^T read from the row-major V tile with LDS
//                   transpose reads, in the key order P^T occupies.
// The loops wait on LDS latency (about 40-50 cycles per read) rather than on
// LDS bandwidth, so operand reads are issued early: the K reads of the S
// products run three ahead of them, and the first V^T blocks of each P.V
// product are read before the exponentials it waits for.
// Epilogue: O = acc / l, LSE = ln 2 * (m + log2 l).
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

constexpr int kFwdBC = 64;       // keys per LDS tile
constexpr int kMaskBlock = 128;  // block-sparse mask granularity

// Workgroup shape: NW waves of 32 query rows each, NBUF K/V tiles in LDS
// (NBUF - 1 copies in flight while one tile is computed). Four waves by
// default; for long sequences (thresholds at the launch below) eight waves,
// so 256 queries share every K/V tile copied into LDS.
// Double buffering in both: a third buffer was measured slower. Block-sparse
// keeps at most four waves so a workgroup's queries stay inside one 128-row
// mask block. One and two waves (32 and 64 rows) exist for callers that
// choose the tile height, e.g. to measure K/V traffic against it: every
// workgroup reads the K/V tiles its rows see, so that traffic scales as
// 1 / rows per workgroup.
template <int D, int MASK, int NW_, int NBUF_>
struct FwdShape {
  static constexpr int NW = NW_;
  static constexpr int NBUF = NBUF_;
  static constexpr int BR = 32 * NW;
  static constexpr int THREADS = 64 * NW;
};

template <int D, int NBUF>
struct alignas(16) FwdSmem {
  uint8_t k[NBUF][kFwdBC * D * 2];   // swizzled row-major K tiles
  uint8_t v[NBUF][kFwdBC * D * 2];   // swizzled row-major V tiles
};

constexpr float kRescaleThreshold = 8.0f;   // log2 units
// Unmasked tiles: the K fragment reads of a tile's S products run this many
// reads ahead of the products (the compiler's own order keeps them one ahead).
// Same-box timings: 0.5-3 % faster than one ahead; two and five ahead measured
// in between.
#ifndef FA_FWD_KDIST
#define FA_FWD_KDIST 3
#endif

template <int D, int MASK, int NW_, int NBUF>
__global__ __launch_bounds__((FwdShape<D, MASK, NW_, NBUF>::THREADS))
__attribute__((amdgpu_waves_per_eu(D == 128 || NW_ == 8 ? 2 : (MASK != 1 ? 4 : 3))))
void fwd_bf16_kernel(AttnParams p, uint32_t nqt, uint32_t total, uint32_t pairs) {
  __shared__ FwdSmem<D, NBUF> sm;
  constexpr int NW = NW_;
  constexpr int kFwdBR = FwdShape<D, MASK, NW_, NBUF>::BR;
  constexpr int TPB = kMaskBlock / kFwdBC;                 // key tiles per mask block
  constexpr int NDT = D / 32;                              // 32-row blocks of O^T
  // V^T column blocks of a sub-block read ahead of its P.V products: half of
  // them at d = 128 (all would not fit the registers); at d = 64 all of them
  // in the causal four-wave shape only. The other d = 64 shapes keep a
  // 128-register budget instead: four waves per SIMD (two eight-wave or four
  // four-wave workgroups per CU) hide more latency than the read-ahead does.
  // Same-box timings: d = 128 forward 2-12 % faster with the read-ahead; at
  // d = 64 without a mask or with a block mask, four waves per SIMD are 5-6 %
  // faster than three with the read-ahead, causal 7 % slower (it spills).
  constexpr int NPRE = D == 128 ? NDT / 2 : (NW_ == 8 || MASK != 1 ? 0 : NDT);

  // The wave index is the same in every lane; reading it into a scalar makes
  // everything derived from it (row ranges, tile classes, loop bounds, LDS
  // copy destinations) scalar, so the tile loops branch on scalars instead of
  // exec masks.
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Work items: one query tile of one (batch, head). Causal, dense batches
  // (pairs = 1, chosen at launch): a workgroup takes two, query tiles j and
  // nqs - 1 - j of one sequence and head (nqs = that sequence's query tiles),
  // longest first, so every workgroup sees about nqs + 1 key tiles and no
  // short tiles are left for the end of the grid (causal_pair_tile).
  // Otherwise one item per workgroup, causal longest first.
  // Head-major order: each XCD's contiguous share of the grid covers whole
  // heads of every sequence, so ragged packed batches spread evenly over the
  // XCDs and the query heads of one K/V group share an L2.
  constexpr int kItems = MASK == 1 ? 2 : 1;
  const bool paired = MASK == 1 && pairs != 0;
  const uint32_t G = work_item(p.rev, total);
  const uint32_t npair = paired ? (nqt + 1) / 2 : nqt;   // workgroups per (batch, head)
  const uint32_t bh = G / npair, j = G - bh * npair;
  const int hq = (int)bh / p.B, bat = (int)bh - hq * p.B;
  const SeqView sq = seq_view(p, bat);
  const uint32_t nqs = (uint32_t)((sq.nq + kFwdBR - 1) / kFwdBR);
  for (int it = 0; it < kItems; ++it) {
  int qt = (int)j;
  if (MASK == 1) {
    qt = paired ? causal_pair_tile(j, it, (int)nqs, true) : (it == 0 ? (int)(nqt - 1 - j) : -1);
    if (qt < 0) break;
  }
  const int q0 = qt * kFwdBR;
  if (q0 >= sq.nq) break;                      // past this sequence's queries (packed batches)
  // The lane index is taken per item behind an opaque copy, so lane-derived
  // values are not hoisted out of the item loop and held across both items.
  // (Not in the one-wave shape, which has registers to spare: there the copy
  // leads the compiler to an invalid comparison against the LDS aperture.)
  int lane = threadIdx.x & 63;
  if (NW > 1) asm volatile("" : "+v"(lane));
  const int h = lane >> 5, r = lane & 31;
  const int Nq = sq.nq, Nk = sq.nk;
  const int off = Nk - Nq;                     // causal: key j visible to query i iff j <= i + off
  // Uniform quotient, read into a scalar so the K/V head pointers stay scalar.
  const int hk = __builtin_amdgcn_readfirstlane(hq / (p.H / p.Hkv));
  const uint16_t* __restrict__ Qh = (const uint16_t*)p.q + sq.qb + hq * p.q_hs;
  const uint16_t* __restrict__ Kh = (const uint16_t*)p.k + sq.kb + hk * p.k_hs;
  const uint16_t* __restrict__ Vh = (const uint16_t*)p.v + sq.kb + hk * p.k_hs;
  const int64_t q_rs = p.q_rs;
  const int qw0 = q0 + w * 32;
  const int qi = qw0 + r;

  const int nkt = (Nk + kFwdBC - 1) / kFwdBC;
  int kend = nkt;
  if (MASK == 1) {
    const int last = q0 + kFwdBR - 1 + off;    // last key any row of the tile sees
    kend = last < 0 ? 0 : min(nkt, last / kFwdBC + 1);
  }
  MaskScan ms;
  // Mask row of the 128-row block holding this tile (query tiles of at most
  // 128 rows never straddle two).
  if (MASK == 2) ms.init(p.block_mask + (size_t)(q0 / kMaskBlock) * p.nblk, 1, p.nblk);
  auto next_tile = [&](int kt) -> int {
    if (MASK != 2 || kt >= kend) return kt < kend ? kt : kend;
    const int blk = kt / TPB;
    const int nb = ms.next(blk);
    if (nb >= p.nblk) return kend;
    const int t = nb == blk ? kt : nb * TPB;
    return t < kend ? t : kend;
  };
  TileLoader<D, kFwdBC, NW> ld;
  ld.init(w, lane, (int)(p.k_rs * 2));
  auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
    ld.load(sm.k[buf], Kh, kt * kFwdBC, Nk);
    ld.load(sm.v[buf], Vh, kt * kFwdBC, Nk);
  };
  const int kbase_l = row_frag_base<D>(lane);
  const int vbase0_l = col_frag_base<D>(lane, 0), vbase1_l = col_frag_base<D>(lane, 1);

  int kt = next_tile(0);
  if (kt < kend) issue(kt, 0);

  // Q fragment: B operand of S^T = K Q^T (lane: query qi, 8 consecutive d).
  u32x4 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < Nq) x = *(const u32x4*)(Qh + qi * q_rs + ks * 16 + h * 8);
    qf[ks] = x ^ p.qflip;
  }

  f32x16 acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = zero16();
  float m_run = -INFINITY;   // reference max of c*s (exp2 domain), per query
  float l_run = 0.f;         // this lane's partial running sum (its 16-key half)
  const float c = p.c;

  // One key tile in stages over its two 32-key sub-blocks, ordered so the
  // MFMA pipe and the VALU have independent work side by side:
  //   S0 | S1 with the masking and row max of S0 | max of S1, rescale
  //   decision | exp of S0 | PV0 with exp of S1 | PV1.
  // Operand fragments of a sub-block are read from LDS as a batch before its
  // products. NM selects the masked variant (diagonal and tail tiles only).
  auto tile = [&](int buf, int kt, auto nm) {
    constexpr bool NM = decltype(nm)::value;
    const int k0 = kt * kFwdBC;
    // Lane addresses of this tile's fragments relative to the start of the
    // shared block: the buffer offset (a multiple of 8 KiB) has no bits in
    // the XORed chunk field, so base + offset can be XORed directly. The
    // opaque copies make the compiler recompute the XORed addresses here
    // rather than keep all of them live across the loop.
    const uint8_t* sbase = (const uint8_t*)&sm;
    int kbase = kbase_l + (int)(sm.k[buf] - sbase);
    int vbase0 = vbase0_l + (int)(sm.v[buf] - sbase), vbase1 = vbase1_l + (int)(sm.v[buf] - sbase);
    asm volatile("" : "+v"(kbase), "+v"(vbase0), "+v"(vbase1));
    // Unmasked tiles are visible to every row, so both sub-blocks are live.
    const bool live1 = !NM || !(MASK == 1 && k0 + 32 > qw0 + 31 + off);

    f32x16 s0 = zero16(), s1 = zero16();
    if (!NM && FA_FWD_KDIST > 0) {
      // Unmasked: K fragment reads run KDIST ahead of the products.
      constexpr int KS = D / 16, KD = FA_FWD_KDIST;
      u32x4 ka[KS], kb2[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ka[ks] = row_frag(sbase, kbase, ks);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kb2[ks] = row_frag(sbase + 32 * 2 * D, kbase, ks);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s0 = mfma_32x32x16(ka[ks], qf[ks], s0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s1 = mfma_32x32x16(kb2[ks], qf[ks], s1);
      __builtin_amdgcn_sched_group_barrier(0x100, KD, 0);
#pragma unroll
      for (int j = 0; j < 2 * KS - KD; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, KD, 0);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      u32x4 kf[D / 16];
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) kf[ks] = row_frag(sbase, kbase, ks);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) s0 = mfma_32x32x16(kf[ks], qf[ks], s0);
      __builtin_amdgcn_sched_barrier(0);
      if (live1) {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) kf[ks] = row_frag(sbase + 32 * 2 * D, kbase, ks);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) s1 = mfma_32x32x16(kf[ks], qf[ks], s1);
      }
    }
    // The V^T fragments of the first NPRE column blocks of a sub-block are
    // read ahead (vpre), so their LDS latency hides behind the vector work.
    auto vread = [&](int kb, u32x4 (&vp)[NPRE > 0 ? NPRE : 1][2]) {
#pragma unroll
      for (int dt = 0; dt < NPRE; ++dt)
#pragma unroll
        for (int st = 0; st < 2; ++st) vp[dt][st] = col_frag(sbase + (kb * 32 + st * 16) * 2 * D, vbase0, vbase1, dt);
    };
    u32x4 vpre[NPRE > 0 ? NPRE : 1][2];
    if (NPRE > 0) vread(0, vpre);
    // Masked entries of a sub-block's scores to -inf; visible scores stay
    // raw, so they take the same arithmetic as in an unmasked tile (c >= 0:
    // the scale's sign is folded into Q). Masked entries are kept out of the
    // products with c explicitly, since c may be 0.
    auto apply_mask = [&](f32x16& sv, int kb, bool live) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
        const bool vis = live && key < Nk && (MASK != 1 || key <= qi + off);
        sv[i] = vis ? sv[i] : -INFINITY;
      }
    };
    float mx0 = -INFINITY, mx1 = -INFINITY;
    if (NM) apply_mask(s0, 0, true);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx0 = fmaxf(mx0, s0[i]);
    __builtin_amdgcn_sched_barrier(0);
    if (NM) apply_mask(s1, 1, live1);
    if (live1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) mx1 = fmaxf(mx1, s1[i]);
    }
    float mx = fmaxf(mx0, mx1);
    mx = xor32_max(mx);
    if (NM) mx = mx == -INFINITY ? mx : mx * c;   // c = 0 (zero scale): -inf * 0 would be NaN
    else mx *= c;
    // Raise the reference max only when some row of the wave outgrows it.
    if (__ballot(mx > m_run + kRescaleThreshold)) {
      const float m_new = fmaxf(m_run, mx);
      // 0 on a row's first update; 1 for a row that has seen no key yet
      // (-inf on both sides) while others in the wave raise theirs.
      const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    // p = 2^(t - m) packed to bf16 as the P^T B operand (k-steps st = 0, 1);
    // the fp32 row sum uses the unrounded p.
    auto expo = [&](const f32x16& sv, u32x4 pb[2]) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float t = sv[8 * st + e];
          x[e] = NM && t == -INFINITY ? 0.f : fast_exp2(__builtin_fmaf(t, c, -m_use));
          l_run += x[e];
        }
        pb[st] = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                       pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
      }
    };
    auto pv = [&](int kb, const u32x4 pb[2], const u32x4 (&vp)[NPRE > 0 ? NPRE : 1][2]) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        u32x4 vf[2];
#pragma unroll
        for (int st = 0; st < 2; ++st)
          vf[st] = dt < NPRE ? vp[dt < NPRE ? dt : 0][st] : col_frag(sbase + (kb * 32 + st * 16) * 2 * D, vbase0, vbase1, dt);
#pragma unroll
        for (int st = 0; st < 2; ++st) acc[dt] = mfma_32x32x16(vf[st], pb[st], acc[dt]);
      }
    };
    u32x4 pb0[2], pb1[2];
    expo(s0, pb0);
    __builtin_amdgcn_sched_barrier(0);
    if (live1) {
      pv(0, pb0, vpre);
      if (NPRE > 0) vread(1, vpre);
      expo(s1, pb1);
      __builtin_amdgcn_sched_barrier(0);
      pv(1, pb1, vpre);
    } else {
      pv(0, pb0, vpre);
    }
  };
  // Tile classes for this wave: 0 unmasked, 1 masked (diagonal or tail),
  // 2 wholly past the wave's diagonal (nothing to compute).
  auto cls = [&](int kt) {
    const int k0 = kt * kFwdBC;
    if (MASK == 1 && k0 > qw0 + 31 + off) return 2;
    return ((k0 + kFwdBC > Nk) || (MASK == 1 && k0 + kFwdBC - 1 > qw0 + off)) ? 1 : 0;
  };

  // NBUF - 1 tiles are issued ahead. At the top of an iteration tile kt is
  // complete in buffer `buf`; the tile NBUF - 1 ahead goes into the buffer
  // computed in the previous iteration (free after that iteration's barrier).
  constexpr int kPerTile = 2 * TileLoader<D, kFwdBC, NW>::PER;   // this wave's copies per K+V tile
  int ahead[NBUF > 2 ? NBUF - 2 : 1];          // tiles issued after kt, in order
#pragma unroll
  for (int j = 0; j + 2 < NBUF; ++j) {
    const int prev = j == 0 ? kt : ahead[j - 1];
    ahead[j] = prev < kend ? next_tile(prev + 1) : kend;
    if (ahead[j] < kend) issue(ahead[j], j + 1);
  }
  auto wait_next = [&](int last_issued) {      // the oldest outstanding tile is complete
    if (NBUF > 2 && last_issued < kend)
      wait_vmem_n<(NBUF > 2 ? kPerTile * (NBUF - 2) : 0)>();
    else
      wait_vmem();
    __syncthreads();
  };
  wait_next(NBUF > 2 ? ahead[NBUF > 2 ? NBUF - 3 : 0] : kend);
  int buf = 0;
  auto step = [&](auto nm, bool work) {
    const int last = NBUF > 2 ? ahead[NBUF > 2 ? NBUF - 3 : 0] : kt;
    const int ktn = last < kend ? next_tile(last + 1) : kend;   // NBUF - 1 tiles after kt
    if (ktn < kend) issue(ktn, (buf + NBUF - 1) % NBUF);
    if (work) tile(buf, kt, nm);
    wait_next(ktn);
    buf = (buf + 1) % NBUF;
    if (NBUF > 2) {
      kt = ahead[0];
#pragma unroll
      for (int j = 0; j + 3 < NBUF; ++j) ahead[j] = ahead[j + 1];
      ahead[NBUF > 2 ? NBUF - 3 : 0] = ktn;
    } else {
      kt = ktn;
    }
  };
  // Each class runs in a loop of its own (runs of equal tiles), so the
  // accumulators stay in place instead of being moved where the variants of
  // the tile code would join. Every wave takes one barrier per tile.
  while (kt < kend) {
    while (kt < kend && cls(kt) == 0) step(std::false_type{}, true);
    while (kt < kend && cls(kt) == 1) step(std::true_type{}, true);
    while (kt < kend && cls(kt) == 2) step(std::false_type{}, false);
  }

  // Epilogue: combine the two lane halves' partial sums, normalise, store.
  // Where registers are tightest the lane index is taken afresh here, so
  // that no lane-derived address is held across the tile loops (it would be
  // spilled to scratch memory); in the other shapes that choice makes the
  // register allocation spill elsewhere, so the item's index is kept. (mbcnt
  // counts the active lanes below this one: every lane is active here, all
  // control flow before this point being uniform across the wave.)
  const int lane_e = D == 64 || (MASK == 1 && NW == 8) ? (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) : lane;
  const int he = lane_e >> 5, qe = qw0 + (lane_e & 31);
  const float lt = xor32_sum(l_run);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (qe < Nq) {
    uint16_t* __restrict__ Orow = (uint16_t*)p.o + sq.qb + hq * p.q_hs + qe * q_rs;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = dt * 32 + 8 * g + 4 * he;
        u32x2 val = {pack_bf16x2(acc[dt][4 * g] * inv, acc[dt][4 * g + 1] * inv),
                     pack_bf16x2(acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv)};
        *(u32x2*)(Orow + dd) = val;
      }
    if (he == 0) p.lse[sq.lb + hq * p.l_hs + qe] = lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -INFINITY;
  }
  }
}

// Query length from which the eight-wave (256-row) shape is used, from
// interleaved timings of both shapes at B * N = 32K tokens, H = 16:
//   causal, d = 128: from 8K (1-2 % faster at 8K, 2-4 % from 16K; 5 % slower at 4K
//   with one tile per workgroup, within +-3 % at 4K with causal work pairs);
//   causal, d = 64: never (5-10 % slower at 32K);
//   no mask, d = 128: from 4K (2 % at 4K, 5-6 % from 8K); no mask, d = 64: from 2K (4-6 %).
#ifndef FA_FWD_LONG_N
#define FA_FWD_LONG_N 8192
#endif
#ifndef FA_FWD_LONG_N_FULL
#define FA_FWD_LONG_N_FULL 4096
#endif
#ifndef FA_FWD_LONG_N_FULL64
#define FA_FWD_LONG_N_FULL64 2048
#endif
#ifndef FA_FWD_LONG_NBUF
#define FA_FWD_LONG_NBUF 2
#endif

template <int D, int MASK, int NW, int NBUF>
static int launch_fwd_s(const AttnParams& p, hipStream_t stream) {
  using S = FwdShape<D, MASK, NW, NBUF>;
  const uint32_t nqt = (uint32_t)((p.Nq + S::BR - 1) / S::BR);
  // Causal pairs for dense batches only: in packed batches the sequences'
  // lengths already differ, and one item per workgroup keeps twice as many
  // workgroups of one head (and K/V group) on an XCD at once, which its L2
  // serves better (same-box timings on 16 packed sequences of 512-4096
  // tokens: pairs 2-4 % slower and 40-60 % more HBM traffic).
  uint32_t pairs = MASK == 1 && p.cu_q == nullptr ? 1u : 0u;
  const uint32_t per_bh = pairs ? (nqt + 1) / 2 : nqt;   // workgroups per (batch, head)
  const uint32_t total = per_bh * (uint32_t)p.B * (uint32_t)p.H;
  AttnParams pp = p;
  void* args[] = {&pp, (void*)&nqt, (void*)&total, (void*)&pairs};
  return (int)hipLaunchKernel((const void*)&fwd_bf16_kernel<D, MASK, NW, NBUF>, dim3(total), dim3(S::THREADS),
                              args, 0, stream);
}

template <int D, int MASK>
static int launch_fwd_t(const AttnParams& p, int block_rows, hipStream_t stream) {
  switch (block_rows) {
    case 32: return launch_fwd_s<D, MASK, 1, 2>(p, stream);
    case 64: return launch_fwd_s<D, MASK, 2, 2>(p, stream);
    case 128: return launch_fwd_s<D, MASK, 4, 2>(p, stream);
    case 256:
      if constexpr (MASK != 2) return launch_fwd_s<D, MASK, 8, FA_FWD_LONG_NBUF>(p, stream);
      return (int)hipErrorInvalidValue;
    default: break;
  }
  if constexpr (MASK == 0) {
    if (p.Nq >= (D == 128 ? FA_FWD_LONG_N_FULL : FA_FWD_LONG_N_FULL64))
      return launch_fwd_s<D, MASK, 8, FA_FWD_LONG_NBUF>(p, stream);
  }
  if constexpr (MASK == 1 && D == 128) {
    if (p.Nq >= FA_FWD_LONG_N) return launch_fwd_s<D, MASK, 8, FA_FWD_LONG_NBUF>(p, stream);
  }
  return launch_fwd_s<D, MASK, 4, 2>(p, stream);
}

int launch_fwd_bf16(const AttnParams& p, int mask_kind, hipStream_t stream, int block_rows) {
  if (p.d == 64) {
    if (mask_kind == 0) return launch_fwd_t<64, 0>(p, block_rows, stream);
    if (mask_kind == 1) return launch_fwd_t<64, 1>(p, block_rows, stream);
    return launch_fwd_t<64, 2>(p, block_rows, stream);
  }
  if (mask_kind == 0) return launch_fwd_t<128, 0>(p, block_rows, stream);
  if (mask_kind == 1) return launch_fwd_t<128, 1>(p, block_rows, stream);
  return launch_fwd_t<128, 2>(p, block_rows, stream);
}

}  // namespace fa
