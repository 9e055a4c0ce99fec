// Backward pass, bf16 in/out, fp32 accumulation, gfx950 MFMA.
//
// The probabilities are recomputed tile by tile from Q, K and the forward's
// row log-sum-exp instead of being stored ("FlashAttention: exact attention
// made fast by counting memory traffic", "The method"; "FlashAttention and
// IO-aware exact attention", "Core ideas": backward by recomputation). The
// gradient formulas are the derivative of the forward definition (no page
// prints them):
//   P = exp(scale*QK^T - LSE)   dV = P^T dO   dP = dO V^T
//   D = rowsum(dO * O)          dS = P * (dP - D)
//   dQ = scale * dS K           dK = scale * dS^T Q
//
// Three kernels, in stream order:
//   bwd_rowterm   D_i = sum_k dO_ik O_ik (a streaming pass over O and dO),
//                 stored negated, and -LSE_i log2(e) (-inf for an empty row),
//                 so that the loops form P = 2^(c s - LSE log2 e) with one
//                 FMA and start the dP accumulator at -D (dP - D comes out
//                 of the product).
//   bwd_dkdv      one workgroup per 128-key tile (32 keys per wave), looping
//                 over the visible 64-query tiles: K and V stay in registers
//                 as MFMA B operands; each Q and dO tile is copied once,
//                 global -> LDS, into a swizzled row-major tile that serves
//                 both as a row operand (S = Q K^T, dP = dO V^T) and, through
//                 LDS transpose reads, as a column operand (dV^T = dO^T P,
//                 dK^T = Q^T dS); dK^T and dV^T accumulate in registers and
//                 are written once. At d = 128 an eight-wave variant runs
//                 two waves per SIMD: wave pairs split each query tile, V is
//                 read from LDS, and the pairs' partial sums are added once.
//   bwd_dq        one workgroup per 128-query tile (32 queries per wave),
//                 looping over the visible 64-key tiles: Q and dO stay in
//                 registers; K and V tiles stream through LDS the same way
//                 (K read along rows for S^T and down columns for
//                 dQ^T = K^T dS^T); dQ^T accumulates in registers and is
//                 written once. dQ is thus accumulated separately from dK/dV
//                 and without atomics, so results are deterministic.
// In both loop kernels the scores are formed so that the C layout puts the
// index of the *accumulated* output (a key for dK/dV, a query for dQ) on the
// lane, which lets P and dS feed the next product as B operands directly.
// Both loop kernels double-buffer their LDS tiles: tile t+1 is copied while
// tile t is computed. Under a causal mask over a dense batch each workgroup
// of either kernel takes two tiles of one sequence and head, j and n - 1 - j,
// one after the other, so every workgroup does the same work
// (causal_pair_tile).
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

constexpr int kThreads = 256;
constexpr int kMaskBlk = 128;

// d = 128 dK/dV: the eight-wave kernel (two waves per SIMD, K and V in LDS)
// when 1, the four-wave kernel (K and V in registers, one wave per SIMD)
// when 0.
#ifndef FA_DKDV8
#define FA_DKDV8 1
#endif

// Column-operand fragments read from LDS ahead of the vector work that
// precedes their products (one 32-column block per sub-block; more did not
// help or did not fit the registers). Same-box timings: dK/dV and dQ 0-2 %
// faster, results bitwise unchanged.
constexpr int kDqPre = 1;     // K^T blocks, dQ kernel
constexpr int kDkvPre = 1;    // dO^T and Q^T blocks, four-wave dK/dV kernel at d = 64


// ---------------------------------------------------------------------------
// row term D = rowsum(dO * O), fp32 accumulation
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_rowterm_bf16_kernel(AttnParams p) {
  constexpr int DC = D / 8;
  const size_t rows = (size_t)p.rt_rows;
  const size_t gt = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t row = gt / DC;
  const int col = (int)(gt % DC);
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)((const uint16_t*)p.o + row * D + col * 8);
    const u32x4 b = *(const u32x4*)((const uint16_t*)p.dO + row * D + col * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc += __uint_as_float(a[j] << 16) * __uint_as_float(b[j] << 16);
      acc += __uint_as_float(a[j] & 0xffff0000u) * __uint_as_float(b[j] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int off = DC / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && col == 0) {
    const size_t inner = (size_t)p.rt_inner;
    const size_t idx = (row % inner) * (size_t)p.rt_hs + row / inner;
    const float l = p.lse[idx];
    p.dterm[idx] = -acc;
    p.lse2[idx] = l == -INFINITY ? -INFINITY : -l * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per 128-key tile
// ---------------------------------------------------------------------------
constexpr int kDkvBK = 128;   // keys per workgroup
constexpr int kDkvBQ = 64;    // queries per LDS tile

template <int D>
struct alignas(16) DkvSmem {
  uint8_t q[2][kDkvBQ * D * 2];    // swizzled row-major Q tiles (sign-adjusted on read)
  uint8_t dO[2][kDkvBQ * D * 2];   // swizzled row-major dO tiles
  float lse[2][kDkvBQ];     // -LSE log2(e) of the tile's queries
  float dterm[2][kDkvBQ];   // -D of the tile's queries
};

// d = 128 keeps K, V fragments and the dK^T, dV^T accumulators (192 VGPRs)
// resident, so it runs one wave per SIMD; d = 64 fits two.
template <int D, int MASK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : 2)))
void bwd_dkdv_bf16_kernel(AttnParams p, uint32_t nkt, uint32_t total, uint32_t pairs) {
  __shared__ DkvSmem<D> sm;
  constexpr int NDT = D / 32;
  constexpr int NPRE = D == 64 ? kDkvPre : 0;
  constexpr int QPB = kMaskBlk / kDkvBQ;               // query tiles per mask block

  // The wave index is the same in every lane; reading it into a scalar makes
  // everything derived from it (row ranges, tile classes, loop bounds, LDS
  // copy destinations) scalar, so the tile loops branch on scalars instead of
  // exec masks.
  const int lane0 = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Work items: one key tile of one (batch, K/V head), or under a causal mask
  // the pair of key tiles j and nks - 1 - j of one sequence and head, whose
  // visible query ranges add up to the same length (causal_pair_tile).
  constexpr int kItems = MASK == 1 ? 2 : 1;
  const uint32_t L = work_item(p.rev, total);
  const bool paired = MASK == 1 && pairs != 0;
  const uint32_t npair = paired ? (nkt + 1) / 2 : nkt;   // workgroups per (batch, K/V head)
  const uint32_t bh = L / npair, pj = L - bh * npair;      // (K/V head, batch), head-major as in the forward kernel
  const int hk = (int)bh / p.B, bat = (int)bh - hk * p.B;
  const SeqView sq = seq_view(p, bat);
  const int nks = (sq.nk + kDkvBK - 1) / kDkvBK;
  for (int item = 0; item < kItems; ++item) {
  const int kt = paired ? causal_pair_tile(pj, item, nks, false) : (item == 0 ? (int)pj : -1);
  if (MASK == 1 && kt < 0) break;
  const int k0 = kt * kDkvBK;
  if (k0 >= sq.nk) break;                      // past this sequence's keys (packed batches)
  // Lane index behind an opaque copy per item (causal pairs): lane-derived
  // values are not hoisted out of the item loop and held across both items.
  int lane = lane0;
  if (kItems > 1) {
    lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
  }
  const int h = lane >> 5, r = lane & 31;
  const int Nq = sq.nq, Nk = sq.nk;
  const int off = Nk - Nq;                     // causal: key j visible to query i iff j <= i + off
  const int G = p.H / p.Hkv;                   // query heads sharing this K/V head
  const int kw0 = k0 + 32 * w;
  const int kj = kw0 + r;
  const uint16_t* __restrict__ Kh = (const uint16_t*)p.k + sq.kb + hk * p.k_hs;
  const uint16_t* __restrict__ Vh = (const uint16_t*)p.v + sq.kb + hk * p.k_hs;
  const int64_t k_rs = p.k_rs;
  // Query head hk * G + j: its Q / dO rows and its LSE / row-term entries.
  const uint16_t* __restrict__ Qg = (const uint16_t*)p.q + sq.qb + (int64_t)hk * G * p.q_hs;
  const uint16_t* __restrict__ dOg = (const uint16_t*)p.dO + sq.qb + (int64_t)hk * G * p.q_hs;
  const float* __restrict__ lseg = p.lse2 + sq.lb + (int64_t)hk * G * p.l_hs;
  const float* __restrict__ dtg = p.dterm + sq.lb + (int64_t)hk * G * p.l_hs;

  const int nqt = (Nq + kDkvBQ - 1) / kDkvBQ;
  int qbeg = 0;
  if (MASK == 1) {
    const int first = k0 - off;                // first query that sees key k0
    qbeg = first <= 0 ? 0 : min(nqt, first / kDkvBQ);
  }
  MaskScan ms;
  if (MASK == 2) ms.init(p.block_mask + kt, p.nblk, p.nblk);   // column kt of the mask
  // The loop runs over the visible query tiles `it` of query head j = 0, then
  // those of head 1, ... (the visible tiles are the same in every head).
  auto next_in_head = [&](int it) -> int {
    if (MASK != 2 || it >= nqt) return it < nqt ? it : nqt;
    const int blk = it / QPB;
    const int nb = ms.next(blk);
    if (nb >= p.nblk) return nqt;
    const int t = nb == blk ? it : nb * QPB;
    return t < nqt ? t : nqt;
  };
  TileLoader<D, kDkvBQ, 4> ld;
  ld.init(w, lane, (int)(p.q_rs * 2));
  auto issue = [&](int it, int j, int buf) {
    const int q0 = it * kDkvBQ;
    ld.load(sm.q[buf], Qg + j * p.q_hs, q0, Nq);
    ld.load(sm.dO[buf], dOg + j * p.q_hs, q0, Nq);
    if (w < 2) {   // one dword per lane: 64 row statistics per tile
      const int q = min(q0 + lane, Nq - 1);
      const float* src = (w == 0 ? lseg : dtg) + j * p.l_hs;
      float* dst = w == 0 ? sm.lse[buf] : sm.dterm[buf];
      copy_to_lds<false>(src, q * 4, dst);
    }
  };

  int it = next_in_head(qbeg), j = 0;
  if (it < nqt) issue(it, j, 0);

  u32x4 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (kj < Nk) {
      a = *(const u32x4*)(Kh + kj * k_rs + ks * 16 + h * 8);
      b = *(const u32x4*)(Vh + kj * k_rs + ks * 16 + h * 8);
    }
    kf[ks] = a ^ p.qflip;   // S = |scale| Q (sign(scale) K)^T: the sign of scale rides on K here
    vf[ks] = b;
  }
  // Complete these loads here: the compiler would otherwise wait for them at
  // their first use inside the tile loop, in every iteration, and that wait
  // (vmcnt) would also wait for the next tile's copies in flight.
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+v"(kf[ks]), "+v"(vf[ks]));

  f32x16 dkT[NDT], dvT[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) {
    dkT[i] = zero16();
    dvT[i] = zero16();
  }
  const float c = p.c;
  const int rbase_l = row_frag_base<D>(lane);
  const int cbase0_l = col_frag_base<D>(lane, 0), cbase1_l = col_frag_base<D>(lane, 1);

  // One 64-query tile in stages over its two 32-query sub-blocks, ordered
  // so the MFMA pipe and the VALU have independent work side by side:
  //   S0, dP0 | S1, dP1 with P0, dS0 | dV, dK of block 0 with P1, dS1 |
  //   dV, dK of block 1.
  // NM selects the masked variant (diagonal and tail tiles only); in the
  // unmasked one both sub-blocks are live and the stages are straight-line.
  auto tile = [&](int buf, int q0, auto nm) {
    constexpr bool NM = decltype(nm)::value;
    // Per-tile lane addresses relative to the shared block (see the
    // forward kernel): one XOR per fragment, opaque so they are not all
    // kept live across the loop.
    const uint8_t* sbase = (const uint8_t*)&sm;
    const int oq = (int)(sm.q[buf] - sbase), oo = (int)(sm.dO[buf] - sbase);
    int qr = rbase_l + oq, orow = rbase_l + oo;
    int qc0 = cbase0_l + oq, qc1 = cbase1_l + oq, oc0 = cbase0_l + oo, oc1 = cbase1_l + oo;
    asm volatile("" : "+v"(qr), "+v"(orow), "+v"(qc0), "+v"(qc1), "+v"(oc0), "+v"(oc1));
    bool live[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) live[mb] = !NM || !(MASK == 1 && q0 + 32 * mb + 31 + off < kw0);

    // S and dP of sub-block mb; the sub-block's -LSE log2(e) values are read
    // from LDS between the two products, so the read latency hides behind the
    // dP products instead of stalling the exponentials.
    auto sdp = [&](int mb, f32x16& sv, f32x16& dpv, float nlv[16]) {
      sv = zero16();
      // dP - D: the accumulator starts at -D of each query row.
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 nd = *(const float4*)&sm.dterm[buf][mb * 32 + 8 * g + 4 * h];
        dpv[4 * g] = nd.x;
        dpv[4 * g + 1] = nd.y;
        dpv[4 * g + 2] = nd.z;
        dpv[4 * g + 3] = nd.w;
      }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        sv = mfma_32x32x16(row_frag(sbase + mb * 32 * 2 * D, qr, ks), kf[ks], sv);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 l4 = *(const float4*)&sm.lse[buf][mb * 32 + 8 * g + 4 * h];
        nlv[4 * g] = l4.x;
        nlv[4 * g + 1] = l4.y;
        nlv[4 * g + 2] = l4.z;
        nlv[4 * g + 3] = l4.w;
      }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        dpv = mfma_32x32x16(row_frag(sbase + mb * 32 * 2 * D, orow, ks), vf[ks], dpv);
    };
    // P = 2^(c s - LSE log2 e) and dS = P (dP - D), packed as B operands.
    auto pds = [&](int mb, const f32x16& sv, const f32x16& dpv, const float nlv[16], u32x4 pb[2], u32x4 db[2]) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float pv[8], dv[8];
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          const int g = 2 * st + g2;
          const int ql = mb * 32 + 8 * g + 4 * h;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * g + e;
            float pp = fast_exp2(__builtin_fmaf(sv[i], c, nlv[i]));
            if (NM) {
              const int q = q0 + ql + e;
              if (q >= Nq || (MASK == 1 && kj > q + off)) pp = 0.f;
            }
            pv[4 * g2 + e] = pp;
            dv[4 * g2 + e] = pp * dpv[i];
          }
        }
        pb[st] = u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                       pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
        db[st] = u32x4{pack_bf16x2(dv[0], dv[1]), pack_bf16x2(dv[2], dv[3]),
                       pack_bf16x2(dv[4], dv[5]), pack_bf16x2(dv[6], dv[7])};
      }
    };
    // dO^T and Q^T fragments of the first NPRE column blocks of a sub-block
    // are read ahead of its P and dS (opre, qpre), so their LDS latency hides
    // behind the vector work.
    u32x4 opre[NPRE > 0 ? NPRE : 1][2], qpre[NPRE > 0 ? NPRE : 1][2];
    auto cread = [&](int mb) {
#pragma unroll
      for (int dt = 0; dt < NPRE; ++dt)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const uint8_t* rowp = sbase + (mb * 32 + st * 16) * 2 * D;
          opre[dt][st] = col_frag(rowp, oc0, oc1, dt);
          qpre[dt][st] = col_frag(rowp, qc0, qc1, dt);
        }
    };
    auto dkdv = [&](int mb, const u32x4 pb[2], const u32x4 db[2], bool pre) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const uint8_t* rowp = sbase + (mb * 32 + st * 16) * 2 * D;
          const bool hp = pre && dt < NPRE;
          const int dp = dt < NPRE ? dt : 0;
          dvT[dt] = mfma_32x32x16(hp ? opre[dp][st] : col_frag(rowp, oc0, oc1, dt), pb[st], dvT[dt]);
          dkT[dt] = mfma_32x32x16(hp ? qpre[dp][st] : col_frag(rowp, qc0, qc1, dt), db[st], dkT[dt]);
        }
    };

    f32x16 s0, dp0, s1, dp1;
    float nl0[16], nl1[16];
    u32x4 pb0[2], db0[2], pb1[2], db1[2];
    if (!NM) {
      sdp(0, s0, dp0, nl0);
      __builtin_amdgcn_sched_barrier(0);
      sdp(1, s1, dp1, nl1);
      cread(0);
      pds(0, s0, dp0, nl0, pb0, db0);
      __builtin_amdgcn_sched_barrier(0);
      dkdv(0, pb0, db0, true);
      cread(1);
      pds(1, s1, dp1, nl1, pb1, db1);
      __builtin_amdgcn_sched_barrier(0);
      dkdv(1, pb1, db1, true);
    } else {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if (!live[mb]) continue;
        sdp(mb, s0, dp0, nl0);
        pds(mb, s0, dp0, nl0, pb0, db0);
        dkdv(mb, pb0, db0, false);
      }
    }
  };
  auto needm = [&](int it) {
    const int q0 = it * kDkvBQ;
    return (MASK == 1 && q0 + off < kw0 + 31) || q0 + kDkvBQ > Nq;
  };
  int buf = 0;
  // One pipelined step: issue the copies of the next tile, compute this one.
  auto step = [&](auto nm) {
    int itn = next_in_head(it + 1), jn = j;
    if (itn >= nqt && j + 1 < G) {   // on to the next query head of the group
      itn = next_in_head(qbeg);
      jn = j + 1;
    }
    if (itn < nqt) issue(itn, jn, buf ^ 1);
    tile(buf, it * kDkvBQ, nm);
    wait_vmem();
    __syncthreads();
    buf ^= 1;
    it = itn;
    j = jn;
  };

  wait_vmem();
  __syncthreads();
  // Masked and unmasked tiles come in runs (the diagonal band, then the
  // interior, then the ragged tail); each run has a loop of its own, so
  // the accumulators stay in place instead of being moved where the two
  // variants of the tile code would join.
  while (it < nqt) {
    while (it < nqt && needm(it)) step(std::true_type{});
    while (it < nqt && !needm(it)) step(std::false_type{});
  }

  if (kj < Nk) {
    const float sk = p.scale;   // dK = scale dS^T Q (Q unmodified; the sign of scale only entered S via kf)
    uint16_t* __restrict__ dKrow = (uint16_t*)p.dk + sq.kb + hk * p.k_hs + kj * k_rs;
    uint16_t* __restrict__ dVrow = (uint16_t*)p.dv + sq.kb + hk * p.k_hs + kj * k_rs;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = dt * 32 + 8 * g + 4 * h;
        u32x2 a = {pack_bf16x2(dkT[dt][4 * g] * sk, dkT[dt][4 * g + 1] * sk),
                   pack_bf16x2(dkT[dt][4 * g + 2] * sk, dkT[dt][4 * g + 3] * sk)};
        u32x2 b = {pack_bf16x2(dvT[dt][4 * g], dvT[dt][4 * g + 1]),
                   pack_bf16x2(dvT[dt][4 * g + 2], dvT[dt][4 * g + 3])};
        *(u32x2*)(dKrow + dd) = a;
        *(u32x2*)(dVrow + dd) = b;
      }
  }
  }
}

// ---------------------------------------------------------------------------
// dK, dV at d = 128 with two waves per SIMD: one workgroup of eight waves per
// 128-key tile. Waves w and w + 4 own the same 32 keys and take the two
// 32-query halves of every 64-query tile. Each wave keeps its keys' K
// fragment in registers (the B operand of S = Q K^T); the workgroup's V rows
// are copied to LDS once and read as the B operand of dP = dO V^T. A wave
// then holds its dK^T, dV^T accumulators, the K fragment and one half-tile
// of scores, and two waves fit on each SIMD (the four-wave kernel above keeps
// K and V in registers, has both halves' scores live and runs one). The two
// partial accumulators of a key group are summed through LDS at the end, so
// the keys' gradients are written once.
// ---------------------------------------------------------------------------
constexpr int kDkv8Q = 64;       // queries per LDS tile (two halves of 32)
constexpr int kDkv8Threads = 512;

struct alignas(16) Dkv8Smem {
  uint8_t v[kDkvBK * 128 * 2];       // the workgroup's V rows, swizzled row-major
  uint8_t q[2][kDkv8Q * 128 * 2];    // Q tiles
  uint8_t dO[2][kDkv8Q * 128 * 2];   // dO tiles
  float lse[2][kDkv8Q];              // -LSE log2(e) of the tile's queries
  float dterm[2][kDkv8Q];            // -D of the tile's queries
};
static_assert(sizeof(Dkv8Smem) <= 160 * 1024, "LDS per workgroup");
// the final exchange of partial accumulators (dK, then dV) reuses the first
// 64 KiB
static_assert(4 * 4 * 16 * 64 * sizeof(float) <= 2 * kDkvBK * 128 * 2, "exchange area");

template <int MASK>
__global__ __launch_bounds__(kDkv8Threads) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dkdv8_bf16_kernel(AttnParams p, uint32_t nkt, uint32_t total, uint32_t pairs) {
  constexpr int D = 128;
  constexpr int NDT = D / 32;
  constexpr int QPB = kMaskBlk / kDkv8Q;               // query tiles per mask block
  __shared__ Dkv8Smem sm;

  const int lane0 = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = w & 3, half = w >> 2;                  // key group, query half
  // Work items as in the four-wave kernel: one key tile, or a causal pair.
  constexpr int kItems = MASK == 1 ? 2 : 1;
  const uint32_t L = work_item(p.rev, total);
  const bool paired = MASK == 1 && pairs != 0;
  const uint32_t npair = paired ? (nkt + 1) / 2 : nkt;   // workgroups per (batch, K/V head)
  const uint32_t bh = L / npair, pj = L - bh * npair;      // (K/V head, batch), head-major
  const int hk = (int)bh / p.B, bat = (int)bh - hk * p.B;
  const SeqView sq = seq_view(p, bat);
  const int nks = (sq.nk + kDkvBK - 1) / kDkvBK;
  for (int item = 0; item < kItems; ++item) {
  const int kt = paired ? causal_pair_tile(pj, item, nks, false) : (item == 0 ? (int)pj : -1);
  if (MASK == 1 && kt < 0) break;
  const int k0 = kt * kDkvBK;
  if (k0 >= sq.nk) break;
  int lane = lane0;
  if (kItems > 1) {
    lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
  }
  const int h = lane >> 5, r = lane & 31;
  const int Nq = sq.nq, Nk = sq.nk;
  const int off = Nk - Nq;
  const int G = p.H / p.Hkv;
  const int kw0 = k0 + 32 * kg;
  const int kj = kw0 + r;
  const uint16_t* __restrict__ Kh = (const uint16_t*)p.k + sq.kb + hk * p.k_hs;
  const uint16_t* __restrict__ Vh = (const uint16_t*)p.v + sq.kb + hk * p.k_hs;
  const uint16_t* __restrict__ Qg = (const uint16_t*)p.q + sq.qb + (int64_t)hk * G * p.q_hs;
  const uint16_t* __restrict__ dOg = (const uint16_t*)p.dO + sq.qb + (int64_t)hk * G * p.q_hs;
  const float* __restrict__ lseg = p.lse2 + sq.lb + (int64_t)hk * G * p.l_hs;
  const float* __restrict__ dtg = p.dterm + sq.lb + (int64_t)hk * G * p.l_hs;

  const int nqt = (Nq + kDkv8Q - 1) / kDkv8Q;
  int qbeg = 0;
  if (MASK == 1) {
    const int first = k0 - off;                         // first query that sees key k0
    qbeg = first <= 0 ? 0 : min(nqt, first / kDkv8Q);
  }
  MaskScan ms;
  if (MASK == 2) ms.init(p.block_mask + kt, p.nblk, p.nblk);
  auto next_in_head = [&](int it) -> int {
    if (MASK != 2 || it >= nqt) return it < nqt ? it : nqt;
    const int blk = it / QPB;
    const int nb = ms.next(blk);
    if (nb >= p.nblk) return nqt;
    const int t = nb == blk ? it : nb * QPB;
    return t < nqt ? t : nqt;
  };
  TileLoader<D, kDkv8Q, 8> ld;
  ld.init(w, lane, (int)(p.q_rs * 2));
  auto issue = [&](int it, int j, int buf) {
    const int q0 = it * kDkv8Q;
    ld.load(sm.q[buf], Qg + j * p.q_hs, q0, Nq);
    ld.load(sm.dO[buf], dOg + j * p.q_hs, q0, Nq);
    if (w < 2) {   // one dword per lane: the tile's 64 row statistics
      const int q = min(q0 + lane, Nq - 1);
      copy_to_lds<false>((w == 0 ? lseg : dtg) + j * p.l_hs, q * 4, w == 0 ? sm.lse[buf] : sm.dterm[buf]);
    }
  };
  {
    // the workgroup's V rows; rows past Nk repeat row Nk - 1, and their
    // gradients are never written
    TileLoader<D, kDkvBK, 8> vl;
    vl.init(w, lane, (int)(p.k_rs * 2));
    vl.load(sm.v, Vh, k0, Nk);
  }
  u32x4 kf[D / 16];   // this lane's key: the B operand of S = Q K^T
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u};
    if (kj < Nk) a = *(const u32x4*)(Kh + kj * p.k_rs + ks * 16 + h * 8);
    kf[ks] = a;
  }
  // Complete these loads here: the compiler would otherwise wait for them at
  // their first use inside the tile loop, in every iteration, and that wait
  // (vmcnt) would also wait for the next tile's copies in flight.
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+v"(kf[ks]));
  int it = next_in_head(qbeg), j = 0;
  if (it < nqt) issue(it, j, 0);

  f32x16 dkT[NDT], dvT[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) {
    dkT[i] = zero16();
    dvT[i] = zero16();
  }
  // P = 2^(c s - LSE log2 e) with s = q . k and c = scale log2(e) (signed:
  // no max is taken here, so a negative scale needs no operand flip).
  const float c = p.scale * kLog2e;
  const int rbase_l = row_frag_base<D>(lane);
  const int cbase0_l = col_frag_base<D>(lane, 0), cbase1_l = col_frag_base<D>(lane, 1);
  const uint8_t* sbase = (const uint8_t*)&sm;
  const int hrow = half * 32 * 2 * D, krow = kg * 32 * 2 * D;   // this half's query rows, this group's key rows

  auto tile = [&](int buf, int q0, auto nm) {
    constexpr bool NM = decltype(nm)::value;
    const int qh0 = q0 + 32 * half;                      // this wave's first query
    if (NM && (qh0 >= Nq || (MASK == 1 && qh0 + 31 + off < kw0))) return;   // nothing visible
    const int oq = (int)(sm.q[buf] - sbase), oo = (int)(sm.dO[buf] - sbase), ov = (int)(sm.v - sbase);
    int qr = rbase_l + oq + hrow, orow = rbase_l + oo + hrow, vr = rbase_l + ov + krow;
    int qc0 = cbase0_l + oq, qc1 = cbase1_l + oq, oc0 = cbase0_l + oo, oc1 = cbase1_l + oo;
    asm volatile("" : "+v"(qr), "+v"(orow), "+v"(vr));
    asm volatile("" : "+v"(qc0), "+v"(qc1), "+v"(oc0), "+v"(oc1));
    f32x16 sv = zero16(), dpv;
    // dP - D: the accumulator starts at -D of each query row
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 nd = *(const float4*)&sm.dterm[buf][half * 32 + 8 * g + 4 * h];
      dpv[4 * g] = nd.x;
      dpv[4 * g + 1] = nd.y;
      dpv[4 * g + 2] = nd.z;
      dpv[4 * g + 3] = nd.w;
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) sv = mfma_32x32x16(row_frag(sbase, qr, ks), kf[ks], sv);
    float nlv[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 l4 = *(const float4*)&sm.lse[buf][half * 32 + 8 * g + 4 * h];
      nlv[4 * g] = l4.x;
      nlv[4 * g + 1] = l4.y;
      nlv[4 * g + 2] = l4.z;
      nlv[4 * g + 3] = l4.w;
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) dpv = mfma_32x32x16(row_frag(sbase, orow, ks), row_frag(sbase, vr, ks), dpv);
    // Column block 0's dO^T fragments are read ahead of P and dS (all the
    // registers allow).
    u32x4 opre[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) opre[st] = col_frag(sbase + hrow + st * 16 * 2 * D, oc0, oc1, 0);
    u32x4 pb[2], db[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      float pv[8], dv[8];
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const int g = 2 * st + g2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g + e;
          float pp = fast_exp2(__builtin_fmaf(sv[i], c, nlv[i]));
          if (NM) {
            const int q = qh0 + 8 * g + 4 * h + e;
            if (q >= Nq || (MASK == 1 && kj > q + off)) pp = 0.f;
          }
          pv[4 * g2 + e] = pp;
          dv[4 * g2 + e] = pp * dpv[i];
        }
      }
      pb[st] = u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                     pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
      db[st] = u32x4{pack_bf16x2(dv[0], dv[1]), pack_bf16x2(dv[2], dv[3]),
                     pack_bf16x2(dv[4], dv[5]), pack_bf16x2(dv[6], dv[7])};
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint8_t* rowp = sbase + hrow + st * 16 * 2 * D;
        dvT[dt] = mfma_32x32x16(dt == 0 ? opre[st] : col_frag(rowp, oc0, oc1, dt), pb[st], dvT[dt]);
        dkT[dt] = mfma_32x32x16(col_frag(rowp, qc0, qc1, dt), db[st], dkT[dt]);
      }
  };
  // masked: some (query, key) pair of this wave's half-tile is not visible,
  // or the half-tile reaches past the last query
  auto needm = [&](int it) {
    const int qh0 = it * kDkv8Q + 32 * half;
    return (MASK == 1 && qh0 + off < kw0 + 31) || qh0 + 32 > Nq;
  };
  int buf = 0;
  auto step = [&](auto nm) {
    int itn = next_in_head(it + 1), jn = j;
    if (itn >= nqt && j + 1 < G) {   // on to the next query head of the group
      itn = next_in_head(qbeg);
      jn = j + 1;
    }
    if (itn < nqt) issue(itn, jn, buf ^ 1);
    tile(buf, it * kDkv8Q, nm);
    wait_vmem();
    __syncthreads();
    buf ^= 1;
    it = itn;
    j = jn;
  };

  wait_vmem();
  __syncthreads();
  while (it < nqt) {
    while (it < nqt && needm(it)) step(std::true_type{});
    while (it < nqt && !needm(it)) step(std::false_type{});
  }

  // Sum the two halves' partial accumulators of each key group, dK first,
  // then dV: the second half writes its fp32 partials to LDS (the tiles are
  // no longer read: the loop ended with a barrier), the first adds them and
  // writes the result.
  float* xch = (float*)&sm;                              // [kg][dt][i][lane]
  uint16_t* __restrict__ dKrow = (uint16_t*)p.dk + sq.kb + hk * p.k_hs + kj * p.k_rs;
  uint16_t* __restrict__ dVrow = (uint16_t*)p.dv + sq.kb + hk * p.k_hs + kj * p.k_rs;
  auto exchange = [&](f32x16 (&acc)[NDT], uint16_t* __restrict__ out, float mul) {
    __syncthreads();
    if (half == 1) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) xch[((kg * NDT + dt) * 16 + i) * 64 + lane] = acc[dt][i];
    }
    __syncthreads();
    if (half == 0 && kj < Nk) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        float a[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) a[i] = (acc[dt][i] + xch[((kg * NDT + dt) * 16 + i) * 64 + lane]) * mul;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(u32x2*)(out + dt * 32 + 8 * g + 4 * h) =
              u32x2{pack_bf16x2(a[4 * g], a[4 * g + 1]), pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
      }
    }
  };
  exchange(dkT, dKrow, p.scale);   // dK = scale dS^T Q
  exchange(dvT, dVrow, 1.0f);
  // The next item's copies overwrite the exchange area: wait until every
  // wave has read its partials.
  if (kItems > 1) __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per 128-query tile
// ---------------------------------------------------------------------------
constexpr int kDqBQ = 128;   // queries per workgroup
constexpr int kDqBK = 64;    // keys per LDS tile

template <int D>
struct alignas(16) DqSmem {
  uint8_t k[2][kDqBK * D * 2];   // swizzled row-major K tiles
  uint8_t v[2][kDqBK * D * 2];   // swizzled row-major V tiles
};

// d = 64 fits three waves per SIMD (<= 168 VGPRs, 32 KiB LDS per workgroup);
// d = 128 two, except with the block-sparse mask scanner, which needs the
// registers of one wave per SIMD to stay free of spills.
template <int D, int MASK>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(D == 128 ? (MASK == 2 ? 1 : 2) : 3)))
void bwd_dq_bf16_kernel(AttnParams p, uint32_t nqt, uint32_t total, uint32_t pairs) {
  __shared__ DqSmem<D> sm;
  constexpr int NDT = D / 32;
  constexpr int NPRE = kDqPre;
  constexpr int TPB = kMaskBlk / kDqBK;

  // The wave index is the same in every lane; reading it into a scalar makes
  // everything derived from it (row ranges, tile classes, loop bounds, LDS
  // copy destinations) scalar, so the tile loops branch on scalars instead of
  // exec masks.
  const int lane0 = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Work items as in the forward kernel: one query tile of one (batch, head),
  // or under a causal mask the pair of query tiles j and nqs - 1 - j.
  constexpr int kItems = MASK == 1 ? 2 : 1;
  const uint32_t L = work_item(p.rev, total);
  const bool paired = MASK == 1 && pairs != 0;
  const uint32_t npair = paired ? (nqt + 1) / 2 : nqt;   // workgroups per (batch, head)
  const uint32_t bh = L / npair, pj = L - bh * npair;
  const int hq = (int)bh / p.B, bat = (int)bh - hq * p.B;   // head-major, as in the forward kernel
  const SeqView sq = seq_view(p, bat);
  const int nqs = (sq.nq + kDqBQ - 1) / kDqBQ;
  for (int item = 0; item < kItems; ++item) {
  int qt = (int)pj;
  if (MASK == 1) {
    qt = paired ? causal_pair_tile(pj, item, nqs, true) : (item == 0 ? (int)(nqt - 1 - pj) : -1);
    if (qt < 0) break;
  }
  const int q0 = qt * kDqBQ;
  if (q0 >= sq.nq) break;                      // past this sequence's queries (packed batches)
  // Lane index behind an opaque copy per item (causal pairs): lane-derived
  // values are not hoisted out of the item loop and held across both items.
  int lane = lane0;
  if (kItems > 1) {
    lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
  }
  const int h = lane >> 5, r = lane & 31;
  const int Nq = sq.nq, Nk = sq.nk;
  const int off = Nk - Nq;                     // causal: key j visible to query i iff j <= i + off
  const int hk = kItems > 1 ? __builtin_amdgcn_readfirstlane(hq / (p.H / p.Hkv)) : hq / (p.H / p.Hkv);
  const int qw0 = q0 + 32 * w;
  const int qi = qw0 + r;
  const int64_t q_rs = p.q_rs;
  const uint16_t* __restrict__ Qh = (const uint16_t*)p.q + sq.qb + hq * p.q_hs;
  const uint16_t* __restrict__ dOh = (const uint16_t*)p.dO + sq.qb + hq * p.q_hs;
  const uint16_t* __restrict__ Kh = (const uint16_t*)p.k + sq.kb + hk * p.k_hs;
  const uint16_t* __restrict__ Vh = (const uint16_t*)p.v + sq.kb + hk * p.k_hs;

  const int nkt = (Nk + kDqBK - 1) / kDqBK;
  int kend = nkt;
  if (MASK == 1) {
    const int last = q0 + kDqBQ - 1 + off;     // last key any row of the tile sees
    kend = last < 0 ? 0 : min(nkt, last / kDqBK + 1);
  }
  MaskScan ms;
  if (MASK == 2) ms.init(p.block_mask + (size_t)qt * p.nblk, 1, p.nblk);
  auto next_tile = [&](int kt) -> int {
    if (MASK != 2 || kt >= kend) return kt < kend ? kt : kend;
    const int blk = kt / TPB;
    const int nb = ms.next(blk);
    if (nb >= p.nblk) return kend;
    const int t = nb == blk ? kt : nb * TPB;
    return t < kend ? t : kend;
  };
  TileLoader<D, kDqBK, 4> ld;
  ld.init(w, lane, (int)(p.k_rs * 2));
  auto issue = [&](int kt, int buf) {
    ld.load_recompute(sm.k[buf], Kh, kt * kDqBK, Nk);
    ld.load(sm.v[buf], Vh, kt * kDqBK, Nk);
  };

  int kt = next_tile(0);
  if (kt < kend) issue(kt, 0);

  u32x4 qf[D / 16], of[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (qi < Nq) {
      a = *(const u32x4*)(Qh + qi * q_rs + ks * 16 + h * 8);
      b = *(const u32x4*)(dOh + qi * q_rs + ks * 16 + h * 8);
    }
    qf[ks] = a ^ p.qflip;
    of[ks] = b;
  }
  float nl = -INFINITY, ndt = 0.f;   // -LSE log2(e) and -D of this lane's query
  if (qi < Nq) {
    const int64_t li = sq.lb + hq * p.l_hs + qi;
    nl = p.lse2[li];
    ndt = p.dterm[li];
  }
  // Complete these loads before the tile loop (see the dK/dV kernel).
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+v"(qf[ks]), "+v"(of[ks]));
  asm volatile("" : "+v"(nl), "+v"(ndt));

  f32x16 dqT[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) dqT[i] = zero16();
  const float c = p.c;
  const int rbase_l = row_frag_base<D>(lane);
  const int cbase0_l = col_frag_base<D>(lane, 0), cbase1_l = col_frag_base<D>(lane, 1);

  // One 64-key tile in stages over its two 32-key sub-blocks (as in the
  // dK/dV kernel): S0, dP0 | S1, dP1 with dS0 | dQ += K^T dS of block 0
  // with dS1 | of block 1. NM selects the masked variant.
  auto tile = [&](int buf, int kt, auto nm) {
    constexpr bool NM = decltype(nm)::value;
    const int k0 = kt * kDqBK;
    const uint8_t* sbase = (const uint8_t*)&sm;
    const int ok = (int)(sm.k[buf] - sbase), ov = (int)(sm.v[buf] - sbase);
    int kr = rbase_l + ok, vr = rbase_l + ov, kc0 = cbase0_l + ok, kc1 = cbase1_l + ok;
    asm volatile("" : "+v"(kr), "+v"(vr), "+v"(kc0), "+v"(kc1));
    bool live[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) live[kb] = !NM || !(MASK == 1 && k0 + kb * 32 > qw0 + 31 + off);

    auto sdp = [&](int kb, f32x16& sv, f32x16& dpv) {
      sv = zero16();
      dpv = zero16();
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        sv = mfma_32x32x16(row_frag(sbase + kb * 32 * 2 * D, kr, ks), qf[ks], sv);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        dpv = mfma_32x32x16(row_frag(sbase + kb * 32 * 2 * D, vr, ks), of[ks], dpv);
    };
    auto ds = [&](int kb, const f32x16& sv, const f32x16& dpv, u32x4 db[2]) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * st + e;
          float pp = fast_exp2(__builtin_fmaf(sv[i], c, nl));
          if (NM) {
            const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
            if (key >= Nk || (MASK == 1 && key > qi + off)) pp = 0.f;
          }
          y[e] = pp * (dpv[i] + ndt);
        }
        db[st] = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                       pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
      }
    };
    // K^T fragments of the first NPRE column blocks of a sub-block are read
    // ahead of its dS (kpre), so their LDS latency hides behind the vector work.
    u32x4 kpre[NPRE > 0 ? NPRE : 1][2];
    auto kread = [&](int kb) {
#pragma unroll
      for (int dt = 0; dt < NPRE; ++dt)
#pragma unroll
        for (int st = 0; st < 2; ++st) kpre[dt][st] = col_frag(sbase + (kb * 32 + st * 16) * 2 * D, kc0, kc1, dt);
    };
    auto dqacc = [&](int kb, const u32x4 db[2], bool pre) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u32x4 kfr = pre && dt < NPRE ? kpre[dt < NPRE ? dt : 0][st]
                                             : col_frag(sbase + (kb * 32 + st * 16) * 2 * D, kc0, kc1, dt);
          dqT[dt] = mfma_32x32x16(kfr, db[st], dqT[dt]);
        }
    };

    f32x16 s0, dp0, s1, dp1;
    u32x4 db0[2], db1[2];
    if (!NM) {
      sdp(0, s0, dp0);
      __builtin_amdgcn_sched_barrier(0);
      sdp(1, s1, dp1);
      kread(0);
      ds(0, s0, dp0, db0);
      __builtin_amdgcn_sched_barrier(0);
      dqacc(0, db0, true);
      kread(1);
      ds(1, s1, dp1, db1);
      __builtin_amdgcn_sched_barrier(0);
      dqacc(1, db1, true);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!live[kb]) continue;
        sdp(kb, s0, dp0);
        ds(kb, s0, dp0, db0);
        dqacc(kb, db0, false);
      }
    }
  };
  // Tile classes for this wave: 0 unmasked, 1 masked (diagonal or tail),
  // 2 wholly past the wave's diagonal (nothing to compute).
  auto cls = [&](int kt) {
    const int k0 = kt * kDqBK;
    if (MASK == 1 && k0 > qw0 + 31 + off) return 2;
    return ((k0 + kDqBK > Nk) || (MASK == 1 && k0 + kDqBK - 1 > qw0 + off)) ? 1 : 0;
  };
  int buf = 0;
  // One pipelined step: issue the copies of the next tile, compute this one.
  auto step = [&](auto nm, bool work) {
    const int ktn = next_tile(kt + 1);
    if (ktn < kend) issue(ktn, buf ^ 1);
    if (work) tile(buf, kt, nm);
    wait_vmem();
    __syncthreads();
    buf ^= 1;
    kt = ktn;
  };

  wait_vmem();
  __syncthreads();
  // Each class runs in a loop of its own (runs of equal tiles), so the
  // accumulators stay in place instead of being moved where the variants of
  // the tile code would join. Every wave takes one barrier per tile.
  while (kt < kend) {
    while (kt < kend && cls(kt) == 0) step(std::false_type{}, true);
    while (kt < kend && cls(kt) == 1) step(std::true_type{}, true);
    while (kt < kend && cls(kt) == 2) step(std::false_type{}, false);
  }

  if (qi < Nq) {
    const float sc = p.scale;   // dQ = scale dS K (K unmodified; the sign of scale only entered S via qf)
    int qe = qi;                // opaque: the row offset is recomputed here, not kept live across the loop
    asm volatile("" : "+v"(qe));
    uint16_t* __restrict__ dQrow = (uint16_t*)p.dq + sq.qb + hq * p.q_hs + qe * q_rs;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = dt * 32 + 8 * g + 4 * h;
        u32x2 a = {pack_bf16x2(dqT[dt][4 * g] * sc, dqT[dt][4 * g + 1] * sc),
                   pack_bf16x2(dqT[dt][4 * g + 2] * sc, dqT[dt][4 * g + 3] * sc)};
        *(u32x2*)(dQrow + dd) = a;
      }
  }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int D, int MASK>
static int launch_bwd_t(const AttnParams& p, int steps, hipStream_t stream) {
  AttnParams pp = p;
  // Causal pairs for dense batches only, as in the forward launcher.
  uint32_t pairs = MASK == 1 && p.cu_q == nullptr ? 1u : 0u;
  if (steps & kBwdRowterm) {
    const size_t threads = (size_t)p.rt_rows * (D / 8);
    const uint32_t grid = (uint32_t)((threads + kThreads - 1) / kThreads);
    void* args[] = {&pp};
    hipError_t e = hipLaunchKernel((const void*)&bwd_rowterm_bf16_kernel<D>, dim3(grid), dim3(kThreads),
                                   args, 0, stream);
    if (e != hipSuccess) return (int)e;
  }
  if (steps & kBwdDkdv) {
    uint32_t nkt = (uint32_t)((p.Nk + kDkvBK - 1) / kDkvBK);
    uint32_t total = (pairs ? (nkt + 1) / 2 : nkt) * (uint32_t)p.B * (uint32_t)p.Hkv;
    void* args[] = {&pp, &nkt, &total, &pairs};
    hipError_t e;
    if (D == 128 && FA_DKDV8)
      e = hipLaunchKernel((const void*)&bwd_dkdv8_bf16_kernel<MASK>, dim3(total), dim3(kDkv8Threads), args, 0, stream);
    else
      e = hipLaunchKernel((const void*)&bwd_dkdv_bf16_kernel<D, MASK>, dim3(total), dim3(kThreads), args, 0, stream);
    if (e != hipSuccess) return (int)e;
  }
  if (steps & kBwdDq) {
    uint32_t nqt = (uint32_t)((p.Nq + kDqBQ - 1) / kDqBQ);
    uint32_t total = (pairs ? (nqt + 1) / 2 : nqt) * (uint32_t)p.B * (uint32_t)p.H;
    void* args[] = {&pp, &nqt, &total, &pairs};
    hipError_t e = hipLaunchKernel((const void*)&bwd_dq_bf16_kernel<D, MASK>, dim3(total), dim3(kThreads),
                                   args, 0, stream);
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

int launch_bwd_bf16(const AttnParams& p, int mask_kind, int steps, hipStream_t stream) {
  if (p.d == 64) {
    if (mask_kind == 0) return launch_bwd_t<64, 0>(p, steps, stream);
    if (mask_kind == 1) return launch_bwd_t<64, 1>(p, steps, stream);
    return launch_bwd_t<64, 2>(p, steps, stream);
  }
  if (mask_kind == 0) return launch_bwd_t<128, 0>(p, steps, stream);
  if (mask_kind == 1) return launch_bwd_t<128, 1>(p, steps, stream);
  return launch_bwd_t<128, 2>(p, steps, stream);
}

}  // namespace fa
