// Split-key forward for few queries per sequence against long key sequences
// (decoding), bf16 in/out, fp32 accumulation, gfx950 MFMA.
//
// With one to a few queries per sequence the query-tile grid of the main
// forward kernel has too few workgroups to keep the chip busy, and every
// query head would stream its K/V head again. Here one workgroup owns one
// (K/V head, sequence, key range): the queries of all H / Hkv query heads
// that read that K/V head are stacked as the rows of the workgroup (row
// g * nq + i is query i of query head hk * G + g), so each K/V tile is read
// from memory once for the whole group, and the key range of a sequence is
// split over several workgroups. Each workgroup writes its range's partial
// result, normalised over that range (O_s, LSE_s) in fp32; a second kernel
// merges the ranges with the block-combine rule ("Flash Attention —
// Revolutionizing Transformer Efficiency Through Memory-Aware Algorithms",
// "Mathematical Correctness": a row's exponential sum is the sum over blocks
// of each block's sum scaled by exp(block max - overall max)):
//   LSE = max_s LSE_s + ln sum_s exp(LSE_s - max_s LSE_s)
//   O   = sum_s exp(LSE_s - LSE) O_s.
// Within a range the arithmetic is that of the main forward kernel: K/V
// tiles stream through LDS (copied global -> LDS asynchronously, NBUF
// buffers deep), S^T = K Q^T and O^T += V^T P^T on MFMA with the online
// softmax in between.
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

constexpr float kSkRescale = 8.0f;      // lazy rescale threshold, log2 units

// Tile shape and pipeline depth per head dimension: BC keys per LDS tile,
// NBUF tiles in flight or in use per workgroup. Measured on the decoding
// shape (one query per sequence, 1K-8K keys, 8 K/V heads): 32-key tiles at
// d = 128 and 64-key tiles at d = 64, double-buffered, are the fastest;
// deeper pipelines gain nothing there.
#ifndef FA_SK_BC128
#define FA_SK_BC128 32
#endif
#ifndef FA_SK_NBUF128
#define FA_SK_NBUF128 2
#endif
#ifndef FA_SK_BC64
#define FA_SK_BC64 64
#endif
#ifndef FA_SK_NBUF64
#define FA_SK_NBUF64 2
#endif

template <int D, int NBUF, int BC>
struct alignas(16) SkSmem {
  uint8_t k[NBUF][BC * D * 2];
  uint8_t v[NBUF][BC * D * 2];
};

template <int D, int NW, int MASK, int NBUF, int BC>
__global__ __launch_bounds__(64 * NW) void splitkv_bf16_kernel(AttnParams p, uint32_t total) {
  __shared__ SkSmem<D, NBUF, BC> sm;
  constexpr int NDT = D / 32;
  constexpr int KB = BC / 32;                 // 32-key sub-blocks per tile
  using Loader = TileLoader<D, BC, NW>;
  constexpr int kPerTile = 2 * Loader::PER;   // this wave's copy instructions per K+V tile

  // The wave index is the same in every lane; reading it into a scalar makes
  // everything derived from it (row ranges, tile classes, loop bounds, LDS
  // copy destinations) scalar, so the tile loops branch on scalars instead of
  // exec masks.
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, r = lane & 31;
  const int S = p.splits;
  const uint32_t L = work_item(p.rev, total);
  const uint32_t bh = L / (uint32_t)S;
  const int sp = (int)(L - bh * (uint32_t)S);
  const int hk = (int)bh / p.B, bat = (int)bh - hk * p.B;   // head-major, as in the forward kernel
  const SeqView sq = seq_view(p, bat);
  const int Nq = sq.nq, Nk = sq.nk;
  const int G = p.H / p.Hkv;
  const int rows = G * Nq;
  if (rows == 0) return;                        // no queries in this sequence: nothing to write
  const int off = Nk - Nq;                      // causal: key j visible to query i iff j <= i + off

  // Key tiles of this range: every range holds `per` tiles (sized from the
  // longest sequence), so a shorter sequence has fewer ranges and every
  // workgroup has at most the same work; ranges past the sequence's keys
  // have nothing to do (the merge reads only the ranges that exist).
  const int nkt = (Nk + BC - 1) / BC;
  const int per = ((p.Nk + BC - 1) / BC + S - 1) / S;
  const int kt0 = sp * per, kt1 = min(nkt, kt0 + per);
  if (kt0 >= nkt) return;

  // This lane's stacked row.
  const int rho = 32 * w + r;
  const bool live_row = rho < rows;
  const int g = live_row ? rho / Nq : 0;
  const int qi = live_row ? rho - g * Nq : 0;
  const int hq = hk * G + g;
  const int lim = MASK == 1 ? qi + off : Nk - 1;   // last key this row sees (may be negative)

  const uint16_t* __restrict__ Kh = (const uint16_t*)p.k + sq.kb + hk * p.k_hs;
  const uint16_t* __restrict__ Vh = (const uint16_t*)p.v + sq.kb + hk * p.k_hs;
  Loader ld;
  ld.init(w, lane, (int)(p.k_rs * 2));
  auto issue = [&](int kt, int buf) {
    ld.load(sm.k[buf], Kh, kt * BC, Nk);
    ld.load(sm.v[buf], Vh, kt * BC, Nk);
  };
#pragma unroll
  for (int b = 0; b < NBUF - 1; ++b)
    if (kt0 + b < kt1) issue(kt0 + b, b);

  u32x4 qf[D / 16];
  {
    const uint16_t* __restrict__ Qrow = (const uint16_t*)p.q + sq.qb + (int64_t)qi * p.q_rs + hq * p.q_hs;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (live_row) x = *(const u32x4*)(Qrow + ks * 16 + h * 8);
      qf[ks] = x ^ p.qflip;
    }
  }

  f32x16 acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = zero16();
  float m_run = -INFINITY;   // reference max of c*s (exp2 domain), per row
  float l_run = 0.f;         // this lane's partial running sum (its 16-key half)
  const float c = p.c;
  const int kbase_l = row_frag_base<D>(lane);
  const int vbase0_l = col_frag_base<D>(lane, 0), vbase1_l = col_frag_base<D>(lane, 1);

  // One key tile: S^T for both 32-key sub-blocks, masking (tail and causal
  // tiles only), lazy rescale, exp, O^T += V^T P^T.
  auto tile = [&](int buf, int kt, auto nm) {
    constexpr bool NM = decltype(nm)::value;
    const int k0 = kt * BC;
    const uint8_t* sbase = (const uint8_t*)&sm;
    int kbase = kbase_l + (int)(sm.k[buf] - sbase);
    int vbase0 = vbase0_l + (int)(sm.v[buf] - sbase), vbase1 = vbase1_l + (int)(sm.v[buf] - sbase);
    asm volatile("" : "+v"(kbase), "+v"(vbase0), "+v"(vbase1));
    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      u32x4 kf[D / 16];
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) kf[ks] = row_frag(sbase + kb * 32 * 2 * D, kbase, ks);
      s[kb] = zero16();
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) s[kb] = mfma_32x32x16(kf[ks], qf[ks], s[kb]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float t = s[kb][i] * c;
        if (NM) {
          const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
          if (key >= Nk || key > lim) t = -INFINITY;
        }
        s[kb][i] = t;
        mx = fmaxf(mx, t);
      }
    mx = xor32_max(mx);
    if (__ballot(mx > m_run + kSkRescale)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      u32x4 pb[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          x[e] = fast_exp2(s[kb][8 * st + e] - m_use);
          l_run += x[e];
        }
        pb[st] = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                       pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        u32x4 vf[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) vf[st] = col_frag(sbase + (kb * 32 + st * 16) * 2 * D, vbase0, vbase1, dt);
#pragma unroll
        for (int st = 0; st < 2; ++st) acc[dt] = mfma_32x32x16(vf[st], pb[st], acc[dt]);
      }
    }
  };

  int buf = 0;
  int kt = kt0;
  auto step = [&](auto nm) {
    // Tile kt was issued NBUF - 1 tiles ago; later tiles may stay in flight.
    if (kt + NBUF - 2 < kt1 && NBUF > 2)
      wait_vmem_n<(NBUF > 2 ? kPerTile * (NBUF - 2) : 0)>();
    else
      wait_vmem();
    __syncthreads();
    const int ktn = kt + NBUF - 1;
    if (ktn < kt1) issue(ktn, (buf + NBUF - 1) % NBUF);
    tile(buf, kt, nm);
    buf = (buf + 1) % NBUF;
    ++kt;
  };
  // Unmasked tiles come first, masked ones (the causal end, the ragged tail)
  // last: one loop each, so the accumulators stay in place.
  auto needm = [&](int t) { return (t * BC + BC > Nk) || (MASK == 1 && t * BC + BC - 1 > off); };
  while (kt < kt1 && !needm(kt)) step(std::false_type{});
  while (kt < kt1) step(std::true_type{});

  // Partial result of this key range, normalised over the range.
  const float lt = xor32_sum(l_run);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (live_row) {
    const int64_t tok = sq.lb + qi;
    float* __restrict__ Op = p.part_o + (((int64_t)sp * p.Tq + tok) * p.H + hq) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int dd = dt * 32 + 8 * gg + 4 * h;
        *(float4*)(Op + dd) = float4{acc[dt][4 * gg] * inv, acc[dt][4 * gg + 1] * inv, acc[dt][4 * gg + 2] * inv,
                                     acc[dt][4 * gg + 3] * inv};
      }
    if (h == 0)
      p.part_lse[((int64_t)sp * p.H + hq) * p.Tq + tok] = lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -INFINITY;
  }
}

// Merge: one wave per (sequence, query, head); lane j holds D / 64 columns.
template <int D, int BC>
__global__ __launch_bounds__(256) void splitkv_combine_kernel(AttnParams p, uint32_t waves) {
  constexpr int CPL = D / 64;   // columns per lane
  const uint32_t wv = blockIdx.x * 4u + (threadIdx.x >> 6);
  if (wv >= waves) return;
  const int lane = threadIdx.x & 63;
  const int hq = (int)(wv % (uint32_t)p.H);
  const uint32_t rest = wv / (uint32_t)p.H;
  const int qi = (int)(rest % (uint32_t)p.Nq);
  const int bat = (int)(rest / (uint32_t)p.Nq);
  const SeqView sq = seq_view(p, bat);
  if (qi >= sq.nq) return;
  const int64_t tok = sq.lb + qi;
  // Ranges of this sequence (as laid out by the split kernel).
  const int per = ((p.Nk + BC - 1) / BC + p.splits - 1) / p.splits;
  const int S = (((sq.nk + BC - 1) / BC) + per - 1) / per;
  // Range s's LSE sits in lane s % 64 (two per lane: at most 128 ranges);
  // the max and the weight sum are wave reductions.
  const float* __restrict__ lp = p.part_lse + (int64_t)hq * p.Tq + tok;
  const int64_t lstride = (int64_t)p.H * p.Tq;
  const float l0 = lane < S ? lp[lane * lstride] : -INFINITY;
  const float l1 = lane + 64 < S ? lp[(lane + 64) * lstride] : -INFINITY;
  float m = fmaxf(l0, l1);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const float w0 = m == -INFINITY ? 0.f : fast_exp2((l0 - m) * kLog2e);   // 0 for an empty range
  const float w1 = m == -INFINITY ? 0.f : fast_exp2((l1 - m) * kLog2e);
  float tot = w0 + w1;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tot += __shfl_xor(tot, o);
  float acc[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) acc[j] = 0.f;
  const float* __restrict__ op = p.part_o + (tok * p.H + hq) * D + lane * CPL;
  const int64_t ostride = (int64_t)p.Tq * p.H * D;
#pragma unroll 4
  for (int s = 0; s < S; ++s) {
    const float wgt = __shfl(s < 64 ? w0 : w1, s & 63);
#pragma unroll
    for (int j = 0; j < CPL; ++j) acc[j] += wgt * op[s * ostride + j];
  }
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;
  uint16_t* __restrict__ Orow = (uint16_t*)p.o + tok * p.q_rs + hq * p.q_hs + lane * CPL;
  if (CPL == 2)
    *(uint32_t*)Orow = pack_bf16x2(acc[0] * inv, acc[CPL - 1] * inv);
  else
    Orow[0] = (uint16_t)(pack_bf16x2(acc[0] * inv, 0.f) & 0xffffu);
  if (lane == 0) p.lse[hq * p.l_hs + tok] = m == -INFINITY ? -INFINITY : m + logf(tot);
}

template <int D, int NW, int MASK>
static int launch_splitkv_t(const AttnParams& p, hipStream_t stream) {
  constexpr int NBUF = D == 128 ? FA_SK_NBUF128 : FA_SK_NBUF64;
  constexpr int BC = D == 128 ? FA_SK_BC128 : FA_SK_BC64;
  const uint32_t total = (uint32_t)p.B * (uint32_t)p.Hkv * (uint32_t)p.splits;
  AttnParams pp = p;
  uint32_t tt = total;
  void* args[] = {&pp, &tt};
  hipError_t e = hipLaunchKernel((const void*)&splitkv_bf16_kernel<D, NW, MASK, NBUF, BC>, dim3(total), dim3(64 * NW),
                                 args, 0, stream);
  if (e != hipSuccess) return (int)e;
  uint32_t waves = (uint32_t)p.B * (uint32_t)p.Nq * (uint32_t)p.H;
  void* cargs[] = {&pp, &waves};
  e = hipLaunchKernel((const void*)&splitkv_combine_kernel<D, BC>, dim3((waves + 3) / 4), dim3(256), cargs, 0, stream);
  return (int)e;
}

template <int D, int MASK>
static int launch_splitkv_d(const AttnParams& p, hipStream_t stream) {
  const int rows = (p.H / p.Hkv) * p.Nq;
  if (rows <= 32) return launch_splitkv_t<D, 1, MASK>(p, stream);
  if (rows <= 64) return launch_splitkv_t<D, 2, MASK>(p, stream);
  return launch_splitkv_t<D, 4, MASK>(p, stream);
}

int launch_splitkv_bf16(const AttnParams& p, int mask_kind, hipStream_t stream) {
  if (p.d == 64) return mask_kind == 1 ? launch_splitkv_d<64, 1>(p, stream) : launch_splitkv_d<64, 0>(p, stream);
  return mask_kind == 1 ? launch_splitkv_d<128, 1>(p, stream) : launch_splitkv_d<128, 0>(p, stream);
}

}  // namespace fa
