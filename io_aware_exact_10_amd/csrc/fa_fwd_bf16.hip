// Forward pass, bf16 in/out, fp32 accumulation, gfx950 MFMA.
//
// Method: exact softmax attention with the online softmax, tile by tile
// ("FlashAttention: exact attention made fast by counting memory traffic",
// "The method"; "FlashAttention and IO-aware exact attention", "Core ideas":
// online softmax, tiling and fusion, one log-sum-exp per row). Only O and the
// row log-sum-exp are written; the N x N scores stay in registers.
//
// Work decomposition: one 256-thread workgroup per (query tile of 128 rows,
// batch, head); each of the 4 waves owns 32 query rows, and the query tile
// is parallel over the sequence ("Core ideas": parallelism over the sequence
// dimension). The workgroup streams 64-key tiles of K and V through LDS,
// double-buffered: global loads of tile t+1 are issued into registers before
// tile t is computed and stored to the other LDS buffer afterwards.
//
// Per wave and key tile (two 32-key sub-blocks):
//   S^T = K Q^T     A = K rows from LDS, B = Q fragment held in registers.
//                   The C layout puts one query per lane (n = lane % 32) and
//                   16 keys per lane, so the row max and row sum are
//                   lane-local plus one exchange with lane ^ 32.
//   online softmax  m' = max(m, c * rowmax), alpha = 2^(m - m'),
//                   p = 2^(c*s - m'), l = alpha*l + rowsum p, acc *= alpha,
//                   with c = |scale| * log2(e) folded into one FMA.
//   O^T += V^T P^T  B = P^T straight from the S^T registers (rounded to
//                   bf16), A = V^T read from a transposed LDS copy whose key
//                   order matches the contraction slots P^T occupies.
// Epilogue: O = acc / l, LSE = ln 2 * (m + log2 l).
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

constexpr int kFwdBR = 128;      // queries per workgroup
constexpr int kFwdBC = 64;       // keys per LDS tile
constexpr int kFwdThreads = 256;
constexpr int kMaskBlock = 128;  // block-sparse mask granularity

template <int D>
struct alignas(16) FwdSmem {
  static constexpr int KS = D + 8;        // K row stride in bf16 (pad: conflict-free b128 reads)
  static constexpr int VS = kFwdBC + 8;   // V^T row stride in bf16
  uint16_t k[2][kFwdBC * KS];
  uint16_t vt[2][D * VS];
};

// Key position inside the transposed V tile. Within each group of 16 keys the
// second and third quads swap, so the 8 keys that lane half h holds in its
// P^T registers (keys 4h..4h+3 and 8+4h..8+4h+3) are contiguous at 8h.
__device__ __forceinline__ int vt_quad_pos(int kq) {
  const int q4 = kq & 3;
  return (kq & ~3) + (q4 == 1 ? 2 : (q4 == 2 ? 1 : q4));
}

template <int D, int MASK>
__global__ __launch_bounds__(kFwdThreads) void fwd_bf16_kernel(AttnParams p, uint32_t nqt, uint32_t total) {
  __shared__ FwdSmem<D> sm;
  constexpr int KS = FwdSmem<D>::KS;
  constexpr int VS = FwdSmem<D>::VS;
  constexpr int DC = D / 8;                                // 16-byte chunks per row
  constexpr int KCH = kFwdBC * DC / kFwdThreads;           // K chunks per thread
  constexpr int VUNITS = (kFwdBC / 4) * DC;                // 4-key x 8-column transpose units
  constexpr int TPB = kMaskBlock / kFwdBC;                 // key tiles per mask block
  constexpr int NDT = D / 32;                              // 32-row blocks of O^T
  static_assert(KCH >= 1 && VUNITS <= kFwdThreads, "tile shape");

  const int N = p.N;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, r = lane & 31;

  const uint32_t L = xcd_remap(blockIdx.x, total);
  const uint32_t bh = L / nqt;
  uint32_t qt = L - bh * nqt;
  if (MASK == 1) qt = nqt - 1 - qt;            // causal: longest rows first
  const int q0 = (int)qt * kFwdBR;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Qh = (const uint16_t*)p.q + hoff;
  const uint16_t* __restrict__ Kh = (const uint16_t*)p.k + hoff;
  const uint16_t* __restrict__ Vh = (const uint16_t*)p.v + hoff;
  const int qw0 = q0 + w * 32;
  const int qi = qw0 + r;

  // Q fragment: B operand of S^T = K Q^T (lane: query qi, 8 consecutive d).
  u32x4 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qi < N) x = *(const u32x4*)(Qh + (size_t)qi * D + ks * 16 + h * 8);
    qf[ks] = x ^ p.qflip;
  }

  const int nkt = (N + kFwdBC - 1) / kFwdBC;
  int kend = nkt;
  if (MASK == 1) kend = min(nkt, (q0 + kFwdBR + kFwdBC - 1) / kFwdBC);
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

  u32x4 kreg[KCH];
  u32x4 vreg[4];
  auto gload = [&](int kt) {
    const int k0 = kt * kFwdBC;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * kFwdThreads;
      const int row = c / DC, col = c % DC;
      const int key = k0 + row;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < N) x = *(const u32x4*)(Kh + (size_t)key * D + col * 8);
      kreg[i] = x;
    }
    if (tid < VUNITS) {
      const int dc = tid % DC, kq = tid / DC;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = k0 + kq * 4 + j;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key < N) x = *(const u32x4*)(Vh + (size_t)key * D + dc * 8);
        vreg[j] = x;
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * kFwdThreads;
      const int row = c / DC, col = c % DC;
      *(u32x4*)&sm.k[buf][row * KS + col * 8] = kreg[i];
    }
    if (tid < VUNITS) {
      const int dc = tid % DC, kq = tid / DC;
      const int pos = vt_quad_pos(kq) * 4;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint32_t a0 = vreg[0][jj], a1 = vreg[1][jj], a2 = vreg[2][jj], a3 = vreg[3][jj];
        u32x2 lo = {lo_halves(a0, a1), lo_halves(a2, a3)};
        u32x2 hi = {hi_halves(a0, a1), hi_halves(a2, a3)};
        *(u32x2*)&sm.vt[buf][(dc * 8 + 2 * jj) * VS + pos] = lo;
        *(u32x2*)&sm.vt[buf][(dc * 8 + 2 * jj + 1) * VS + pos] = hi;
      }
    }
  };

  f32x16 acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = zero16();
  float m_run = -INFINITY;   // running max of c*s (exp2 domain), per query
  float l_run = 0.f;         // this lane's partial running sum (its 16-key half)
  const float c = p.c;

  auto compute = [&](int buf, int kt) {
    const int k0 = kt * kFwdBC;
    if (MASK == 1 && k0 > qw0 + 31) return;      // whole tile above this wave's diagonal
    const bool need_mask = (k0 + kFwdBC > N) || (MASK == 1 && k0 + kFwdBC - 1 > qw0);
    bool live[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) live[kb] = !(MASK == 1 && k0 + kb * 32 > qw0 + 31);

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero16();
      if (live[kb]) {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const u32x4 a = *(const u32x4*)&sm.k[buf][(kb * 32 + r) * KS + ks * 16 + h * 8];
          s[kb] = mfma_32x32x16(a, qf[ks], s[kb]);
        }
      }
    }

    float m_new, m_use;
    float pv[2][16];
    if (!need_mask) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      m_new = fmaxf(m_run, mx * c);
      m_use = m_new == -INFINITY ? 0.f : m_new;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) pv[kb][i] = fast_exp2(__builtin_fmaf(s[kb][i], c, -m_use));
    } else {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
          const bool vis = live[kb] && key < N && (MASK != 1 || key <= qi);
          const float t = vis ? s[kb][i] * c : -INFINITY;
          pv[kb][i] = t;
          mx = fmaxf(mx, t);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      m_new = fmaxf(m_run, mx);
      m_use = m_new == -INFINITY ? 0.f : m_new;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) pv[kb][i] = fast_exp2(pv[kb][i] - m_use);
    }
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) rs += pv[kb][i];
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;

    // P^T as the B operand: registers 8s..8s+7 of sub-block kb form k-step s.
    u32x4 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const float* x = &pv[kb][8 * st];
        pb[kb][st] = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                           pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
      }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!live[kb]) continue;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u32x4 a = *(const u32x4*)&sm.vt[buf][(dt * 32 + r) * VS + kb * 32 + st * 16 + h * 8];
          acc[dt] = mfma_32x32x16(a, pb[kb][st], acc[dt]);
        }
      }
  };

  int kt = next_tile(0);
  if (kt < kend) {
    gload(kt);
    sstore(0);
  }
  __syncthreads();
  int buf = 0;
  while (kt < kend) {
    const int ktn = next_tile(kt + 1);
    const bool more = ktn < kend;
    if (more) gload(ktn);
    compute(buf, kt);
    if (more) sstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    kt = ktn;
  }

  // Epilogue: combine the two lane halves' partial sums, normalise, store.
  const float lt = l_run + __shfl_xor(l_run, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (qi < N) {
    uint16_t* __restrict__ Orow = (uint16_t*)p.o + hoff + (size_t)qi * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = dt * 32 + 8 * g + 4 * h;
        u32x2 val = {pack_bf16x2(acc[dt][4 * g] * inv, acc[dt][4 * g + 1] * inv),
                     pack_bf16x2(acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv)};
        *(u32x2*)(Orow + dd) = val;
      }
    if (h == 0) p.lse[(size_t)bh * N + qi] = lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -INFINITY;
  }
}

template <int D, int MASK>
static int launch_fwd_t(const AttnParams& p, hipStream_t stream) {
  const uint32_t nqt = (uint32_t)((p.N + kFwdBR - 1) / kFwdBR);
  const uint32_t total = nqt * (uint32_t)p.B * (uint32_t)p.H;
  AttnParams pp = p;
  void* args[] = {&pp, (void*)&nqt, (void*)&total};
  return (int)hipLaunchKernel((const void*)&fwd_bf16_kernel<D, MASK>, dim3(total), dim3(kFwdThreads),
                              args, 0, stream);
}

int launch_fwd_bf16(const AttnParams& p, int mask_kind, hipStream_t stream) {
  if (p.d == 64) {
    if (mask_kind == 0) return launch_fwd_t<64, 0>(p, stream);
    if (mask_kind == 1) return launch_fwd_t<64, 1>(p, stream);
    return launch_fwd_t<64, 2>(p, stream);
  }
  if (mask_kind == 0) return launch_fwd_t<128, 0>(p, stream);
  if (mask_kind == 1) return launch_fwd_t<128, 1>(p, stream);
  return launch_fwd_t<128, 2>(p, stream);
}

}  // namespace fa
