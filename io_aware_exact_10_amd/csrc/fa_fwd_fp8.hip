// Forward pass with FP8 (OCP E4M3) Q, K and V: bf16 O, fp32 LSE, fp32
// accumulation, on the gfx950 32x32x64 f8f6f4 MFMA (twice the bf16 rate).
//
// The method is the one of the bf16 forward kernel: exact softmax attention
// with the online softmax, tile by tile ("FlashAttention: exact attention made
// fast by counting memory traffic", "The method"; "FlashAttention and
// IO-aware exact attention", "Core ideas"); low-precision inputs are the
// variant "Flash Attention — Revolutionizing Transformer Efficiency Through
// Memory-Aware Algorithms", "Flash Attention 3 (2024)" lists (FP8 support).
// The operands hold E4M3 codes with one float descale factor per tensor:
// Q = q_descale * Q8 and so on. The scores are exact products of the codes
// accumulated in fp32; P is rounded to E4M3 for the P.V product (its row
// sum uses the unrounded fp32 P, as in the bf16 kernel).
//
// Operand layouts (v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales, for
// lane l, h = l / 32, r = l % 32): A holds row r and contraction slots
// 32 h .. 32 h + 31 (one byte each), B column r and the same slots; C as
// in the bf16 product.
//   S^T = K Q^T  A = 32 K rows x 64 d bytes from LDS, B = Q in registers.
//   O^T += V^T P^T  A = 32 rows of V^T (d) x 64 keys, B = P^T from the S^T
//                registers. For B the lane needs keys 32 h .. 32 h + 31 of
//                the tile in order; the C layout of S^T gives it LDS rows
//                32 kb + 8 a + 4 h + b (a, b < 4, kb < 2). The K tile is
//                therefore copied into LDS with its rows permuted: LDS row
//                32 kb + 8 a + 4 h + b holds key 32 h + 16 kb + 4 a + b, so
//                register i of sub-block kb is key 32 h + 16 kb + i, and the
//                lane's 32 P values are exactly its 32 contraction slots.
// V is taken transposed, V^T [d, keys] (leading dimension ldv bytes), so the
// A operand of the second product is two 16-byte reads along an LDS row.
#include <type_traits>

#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_f8_32x32x64(i32x8 a, i32x8 b, f32x16 c) {
  // cbsz = blgp = 0: both operands E4M3; E8M0 scale 127 = 1.0 for both.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Four floats -> four E4M3 codes in order (round to nearest even). The first
// conversion writes the low half of the word and keeps the high half of its
// "old" operand, which the second conversion then overwrites, so any value
// serves as that operand: a's own bits let the compiler convert in place
// instead of first zeroing a register.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

constexpr int kF8BC = 64;          // keys per tile
constexpr float kF8Rescale = 8.0f; // lazy rescale threshold (log2 units): keeps P <= 256 < 448

// Key held by LDS row r of a K tile (the permutation above).
__device__ __forceinline__ int f8_key_of_row(int r) {
  return 32 * ((r >> 2) & 1) + 16 * (r >> 5) + 4 * ((r >> 3) & 3) + (r & 3);
}
// 16-byte chunk swizzles: conflict-free 16-byte reads of one chunk from 16
// consecutive rows (K rows of D bytes; V^T rows of 64 bytes).
template <int D>
__device__ __forceinline__ int f8_swz_k(int r) {
  return D == 128 ? (r >> 1) & 7 : (r >> 2) & 3;
}
__device__ __forceinline__ int f8_swz_v(int r) { return (r >> 2) & 3; }

template <int D>
struct alignas(16) F8Smem {
  uint8_t k[2][kF8BC * D];   // K tiles, rows permuted, D bytes per row
  uint8_t v[2][D * kF8BC];   // V^T tiles, one 64-byte row per d
};

// NW waves of 32 queries each per workgroup; three waves per SIMD fit the
// register budget.
template <int D, int MASK, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(3)))
void fwd_fp8_kernel(AttnParams p, uint32_t nqt, uint32_t total, uint32_t pairs) {
  constexpr int kF8NW = NW;
  constexpr int kF8BR = 32 * NW;        // queries per workgroup
  __shared__ F8Smem<D> sm;
  constexpr int NDT = D / 32;            // 32-row blocks of O^T
  // V^T blocks read ahead of the vector work: two (all at d = 64); all four
  // at d = 128 would not fit the registers. Same-box timings: 0-7 % faster.
  constexpr int NPRE = NDT < 2 ? NDT : 2;
  constexpr int NKS = D / 64;            // 64-byte contraction steps of S^T
  constexpr int PK = kF8BC * D / 1024;   // 1 KiB pieces per K (and per V^T) tile
  constexpr int PER = PK / kF8NW;        // pieces per wave
  static_assert(PK % kF8NW == 0, "pieces per wave");

  // The wave index is the same in every lane; reading it into a scalar makes
  // everything derived from it (row ranges, tile classes, loop bounds, LDS
  // copy destinations) scalar, so the tile loops branch on scalars instead of
  // exec masks.
  const int lane0 = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Work items: one query tile of one (batch, head); under a causal mask
  // either the longest tiles first, one per workgroup, or (pairs = 1, chosen
  // at launch) as in the bf16 forward the pair of query tiles j and
  // nqt - 1 - j, whose visible key ranges add up to the same length
  // (causal_pair_tile).
  constexpr int kItems = MASK == 1 ? 2 : 1;
  const bool paired = MASK == 1 && pairs != 0;
  const uint32_t L = work_item(p.rev, total);
  const uint32_t npair = paired ? (nqt + 1) / 2 : nqt;   // workgroups per (batch, head)
  const uint32_t bh = L / npair, pj = L - bh * npair;
  const int hq = (int)bh / p.B, bat = (int)bh - hq * p.B;   // head-major
  for (int item = 0; item < kItems; ++item) {
  int qt = (int)pj;
  if (MASK == 1) {
    qt = paired ? causal_pair_tile(pj, item, (int)nqt, true) : (item == 0 ? (int)(nqt - 1 - pj) : -1);
    if (qt < 0) break;
  }
  const int q0 = qt * kF8BR;
  // Lane index behind an opaque copy per item (causal pairs): lane-derived
  // values are not hoisted out of the item loop and held across both items.
  int lane = lane0;
  if (kItems > 1) {
    lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
  }
  const int h = lane >> 5, r = lane & 31;
  const int N = p.N, ldv = p.ldv;
  const int64_t head = (int64_t)bat * p.H + hq;
  const uint8_t* __restrict__ Qh = (const uint8_t*)p.q + head * N * D;
  const uint8_t* __restrict__ Kh = (const uint8_t*)p.k + head * N * D;
  const uint8_t* __restrict__ Vt = (const uint8_t*)p.v + head * D * ldv;
  const int qw0 = q0 + 32 * w;
  const int qi = qw0 + r;

  const int nkt = (N + kF8BC - 1) / kF8BC;
  const int kend = MASK == 1 ? min(nkt, (q0 + kF8BR - 1) / kF8BC + 1) : nkt;

  // Tile copies, global -> LDS: lane l fills bytes [16 l, 16 l + 16) of
  // piece P. The per-lane source offsets are recomputed at each copy from an
  // opaque copy of the lane id (cheap integer work) rather than kept live
  // across the loop.
  auto issue = [&](int kt, int buf) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int k0 = kt * kF8BC;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int P = w + i * kF8NW;
      const int kr = (P * 1024 + 16 * ln) / D;
      const int kc = (ln % (D / 16)) ^ f8_swz_k<D>(kr);
      const int key = min(k0 + f8_key_of_row(kr), N - 1);   // rows past N: a real row, masked
      copy_to_lds(Kh, key * D + 16 * kc, sm.k[buf] + P * 1024);
      const int vr = 16 * P + (ln >> 2);
      const int vc = (ln & 3) ^ f8_swz_v(vr);
      const int col = min(k0 + 16 * vc, ldv - 16);            // chunks past ldv: keys >= N, zeroed
      copy_to_lds(Vt, vr * ldv + col, sm.v[buf] + P * 1024);
    }
  };

  int kt = 0;
  if (kt < kend) issue(kt, 0);

  // Q fragment: B operand of S^T (lane: query qi, 32 consecutive d bytes).
  i32x8 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
    if (qi < N) {
      const uint8_t* src = Qh + (int64_t)qi * D + 64 * ks + 32 * h;
      x0 = *(const u32x4*)src;
      x1 = *(const u32x4*)(src + 16);
    }
    const u32x4 f = {p.qflip, p.qflip, p.qflip, p.qflip};
    x0 ^= f;
    x1 ^= f;
    qf[ks] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  }

  f32x16 acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = zero16();
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.c;

  auto lds_frag = [](const uint8_t* row, int c0, int c1) -> i32x8 {
    const u32x4 a = *(const u32x4*)(row + 16 * c0), b = *(const u32x4*)(row + 16 * c1);
    return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
  };

  auto tile = [&](int buf, int kt, auto nm) {
    constexpr bool NM = decltype(nm)::value;
    const int k0 = kt * kF8BC;
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int row = 32 * kb + r;
      const uint8_t* rp = sm.k[buf] + row * D;
      const int sw = f8_swz_k<D>(row);
      s[kb] = zero16();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int c0 = 4 * ks + 2 * h;
        s[kb] = mfma_f8_32x32x64(lds_frag(rp, c0 ^ sw, (c0 + 1) ^ sw), qf[ks], s[kb]);
      }
    }
    // The V^T fragments of the first NPRE column blocks are read here, ahead
    // of the vector work, so their LDS latency is hidden behind it.
    i32x8 vpre[NPRE > 0 ? NPRE : 1];
#pragma unroll
    for (int dt = 0; dt < NPRE; ++dt) {
      const int row = 32 * dt + r;
      const int sw = f8_swz_v(row);
      vpre[dt] = lds_frag(sm.v[buf] + row * kF8BC, (2 * h) ^ sw, (2 * h + 1) ^ sw);
    }
    __builtin_amdgcn_sched_barrier(0);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // Masked tiles move to the exp2 domain here (masked keys -inf);
        // unmasked ones keep raw scores and fold c into the exp2 argument.
        float t = s[kb][i];
        if (NM) {
          const int key = k0 + 32 * h + 16 * kb + i;
          t = (key >= N || (MASK == 1 && key > qi)) ? -INFINITY : t * c;
          s[kb][i] = t;
        }
        mx = fmaxf(mx, t);
      }
    mx = xor32_max(mx);
    if (!NM) mx *= c;
    if (__ballot(mx > m_run + kF8Rescale)) {
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
    i32x8 pb;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = NM ? fast_exp2(s[kb][4 * g + e] - m_use) : fast_exp2(__builtin_fmaf(s[kb][4 * g + e], c, -m_use));
          l_run += x[e];
        }
        pb[4 * kb + g] = (int)pack_fp8x4(x[0], x[1], x[2], x[3]);
      }
    __builtin_amdgcn_sched_barrier(0);
    // Keys past N in the last tile: their V^T bytes may be anything
    // (padding), so they are zeroed before the product (P is already 0).
    uint32_t vmask[8];
    if (NM) {
      const int valid = N - (k0 + 32 * h);
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const int nv = valid - 4 * wd;
        vmask[wd] = nv >= 4 ? 0xffffffffu : (nv <= 0 ? 0u : (1u << (8 * nv)) - 1u);
      }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int row = 32 * dt + r;
      const int sw = f8_swz_v(row);
      i32x8 vf = dt < NPRE ? vpre[dt < NPRE ? dt : 0] : lds_frag(sm.v[buf] + row * kF8BC, (2 * h) ^ sw, (2 * h + 1) ^ sw);
      if (NM) {
#pragma unroll
        for (int wd = 0; wd < 8; ++wd) vf[wd] = (int)((uint32_t)vf[wd] & vmask[wd]);
      }
      acc[dt] = mfma_f8_32x32x64(vf, pb, acc[dt]);
    }
  };
  // Tile classes for this wave: 0 unmasked, 1 masked (diagonal or tail),
  // 2 wholly past the wave's diagonal. Each class runs in a loop of its own
  // so the accumulators stay in place (no moves where the variants would
  // join); every wave takes one barrier per tile.
  auto cls = [&](int kt) {
    const int k0 = kt * kF8BC;
    if (MASK == 1 && k0 > qw0 + 31) return 2;
    return ((k0 + kF8BC > N) || (MASK == 1 && k0 + kF8BC - 1 > qw0)) ? 1 : 0;
  };
  int buf = 0;
  auto step = [&](auto nm, bool work) {
    const int ktn = kt + 1;
    if (ktn < kend) issue(ktn, buf ^ 1);
    if (work) tile(buf, kt, nm);
    wait_vmem();
    __syncthreads();
    buf ^= 1;
    kt = ktn;
  };

  wait_vmem();
  __syncthreads();
  while (kt < kend) {
    while (kt < kend && cls(kt) == 0) step(std::false_type{}, true);
    while (kt < kend && cls(kt) == 1) step(std::true_type{}, true);
    while (kt < kend && cls(kt) == 2) step(std::false_type{}, false);
  }

  const float lt = xor32_sum(l_run);
  const float inv = lt > 0.f ? p.vscale / lt : 0.f;
  if (qi < N) {
    uint16_t* __restrict__ Orow = (uint16_t*)p.o + (head * N + qi) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = dt * 32 + 8 * g + 4 * h;
        u32x2 val = {pack_bf16x2(acc[dt][4 * g] * inv, acc[dt][4 * g + 1] * inv),
                     pack_bf16x2(acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv)};
        *(u32x2*)(Orow + dd) = val;
      }
    if (h == 0) p.lse[head * N + qi] = lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -INFINITY;
  }
  }
}

// Causal pairs up to this many query tiles per sequence (16K queries).
// Same-box timings against longest-first single tiles: 4K queries 8-13 %
// faster, 8K 5 %, 16K 1-4 %; 32K 2-4 % slower.
#ifndef FA_FP8_PAIR_MAX_NQT
#define FA_FP8_PAIR_MAX_NQT 128
#endif

template <int D, int MASK, int NW>
static int launch_fwd_fp8_s(const AttnParams& p, hipStream_t stream) {
  const uint32_t nqt = (uint32_t)((p.N + 32 * NW - 1) / (32 * NW));
  uint32_t pairs = MASK == 1 && nqt <= FA_FP8_PAIR_MAX_NQT ? 1u : 0u;
  const uint32_t total = (pairs ? (nqt + 1) / 2 : nqt) * (uint32_t)p.B * (uint32_t)p.H;
  AttnParams pp = p;
  void* args[] = {&pp, (void*)&nqt, (void*)&total, (void*)&pairs};
  return (int)hipLaunchKernel((const void*)&fwd_fp8_kernel<D, MASK, NW>, dim3(total), dim3(64 * NW), args, 0,
                              stream);
}

// Four waves per workgroup at every length: eight (256 queries sharing each
// K/V tile) measured 6 % slower at 32K queries, unlike the bf16 kernel.
template <int D, int MASK>
static int launch_fwd_fp8_t(const AttnParams& p, hipStream_t stream) {
  return launch_fwd_fp8_s<D, MASK, 4>(p, stream);
}

int launch_fwd_fp8(const AttnParams& p, int mask_kind, hipStream_t stream) {
  if (p.d == 64) return mask_kind == 1 ? launch_fwd_fp8_t<64, 1>(p, stream) : launch_fwd_fp8_t<64, 0>(p, stream);
  return mask_kind == 1 ? launch_fwd_fp8_t<128, 1>(p, stream) : launch_fwd_fp8_t<128, 0>(p, stream);
}

}  // namespace fa
