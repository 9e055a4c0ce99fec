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
//   bwd_rowterm   D_i = sum_k dO_ik O_ik (a streaming pass over O and dO).
//   bwd_dkdv      one workgroup per 128-key tile (32 keys per wave), looping
//                 over the visible 64-query tiles: K and V stay in registers
//                 as MFMA B operands, Q and dO tiles stream through LDS in
//                 row-major and transposed copies; dK^T and dV^T accumulate
//                 in registers and are written once.
//   bwd_dq        one workgroup per 128-query tile (32 queries per wave),
//                 looping over the visible 64-key tiles: Q and dO stay in
//                 registers, K (row-major and transposed) and V stream
//                 through LDS; dQ^T accumulates in registers and is written
//                 once. dQ is thus accumulated separately from dK/dV and
//                 without atomics, so results are deterministic.
// In both loop kernels the scores are formed so that the C layout puts the
// index of the *accumulated* output (a key for dK/dV, a query for dQ) on the
// lane, which lets P and dS feed the next product as B operands directly.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

constexpr int kThreads = 256;
constexpr int kMaskBlk = 128;

// Same key/query position swap as the forward's V^T tile: within each group
// of 16, quads 1 and 2 trade places so the 8 contraction slots of lane half h
// are contiguous at offset 8h.
__device__ __forceinline__ int quad_pos(int kq) {
  const int q4 = kq & 3;
  return (kq & ~3) + (q4 == 1 ? 2 : (q4 == 2 ? 1 : q4));
}

// Stores a 4-row x 8-column bf16 block (x[j] = row j, 8 columns) transposed:
// column c of the block goes to t[(col0 + c) * ts + pos .. + 3].
__device__ __forceinline__ void store_quad_transposed(uint16_t* t, int ts, int col0, int pos, const u32x4 x[4]) {
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const uint32_t a0 = x[0][jj], a1 = x[1][jj], a2 = x[2][jj], a3 = x[3][jj];
    u32x2 lo = {lo_halves(a0, a1), lo_halves(a2, a3)};
    u32x2 hi = {hi_halves(a0, a1), hi_halves(a2, a3)};
    *(u32x2*)&t[(col0 + 2 * jj) * ts + pos] = lo;
    *(u32x2*)&t[(col0 + 2 * jj + 1) * ts + pos] = hi;
  }
}

// ---------------------------------------------------------------------------
// row term D = rowsum(dO * O), fp32 accumulation
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_rowterm_bf16_kernel(AttnParams p, size_t rows) {
  constexpr int DC = D / 8;
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
  if (row < rows && col == 0) p.dterm[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per 128-key tile
// ---------------------------------------------------------------------------
constexpr int kDkvBK = 128;   // keys per workgroup
constexpr int kDkvBQ = 64;    // queries per LDS tile

template <int D>
struct alignas(16) DkvSmem {
  static constexpr int RS = D + 8;
  static constexpr int TS = kDkvBQ + 8;
  uint16_t q[2][kDkvBQ * RS];
  uint16_t dO[2][kDkvBQ * RS];
  uint16_t qt[2][D * TS];
  uint16_t dOt[2][D * TS];
  float lse2[2][kDkvBQ];
  float dterm[2][kDkvBQ];
};

template <int D, int MASK>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_bf16_kernel(AttnParams p, uint32_t nkt, uint32_t total) {
  __shared__ DkvSmem<D> sm;
  constexpr int RS = DkvSmem<D>::RS;
  constexpr int TS = DkvSmem<D>::TS;
  constexpr int DC = D / 8;
  constexpr int UNITS = (kDkvBQ / 4) * DC;             // 4-row x 8-col units per tensor
  constexpr int UPT = (2 * UNITS) / kThreads;          // units per thread (Q and dO together)
  constexpr int NDT = D / 32;
  constexpr int QPB = kMaskBlk / kDkvBQ;               // query tiles per mask block
  static_assert(UPT >= 1 && (2 * UNITS) % kThreads == 0, "tile shape");

  const int N = p.N;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, r = lane & 31;
  const uint32_t L = xcd_remap(blockIdx.x, total);
  const uint32_t bh = L / nkt;
  const int kt = (int)(L - bh * nkt);
  const int k0 = kt * kDkvBK;
  const int kw0 = k0 + 32 * w;
  const int kj = kw0 + r;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Qh = (const uint16_t*)p.q + hoff;
  const uint16_t* __restrict__ Kh = (const uint16_t*)p.k + hoff;
  const uint16_t* __restrict__ Vh = (const uint16_t*)p.v + hoff;
  const uint16_t* __restrict__ dOh = (const uint16_t*)p.dO + hoff;
  const float* __restrict__ lseh = p.lse + (size_t)bh * N;
  const float* __restrict__ dth = p.dterm + (size_t)bh * N;

  u32x4 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (kj < N) {
      a = *(const u32x4*)(Kh + (size_t)kj * D + ks * 16 + h * 8);
      b = *(const u32x4*)(Vh + (size_t)kj * D + ks * 16 + h * 8);
    }
    kf[ks] = a;
    vf[ks] = b;
  }

  const int nqt = (N + kDkvBQ - 1) / kDkvBQ;
  const int qbeg = MASK == 1 ? k0 / kDkvBQ : 0;
  MaskScan ms;
  if (MASK == 2) ms.init(p.block_mask + kt, p.nblk, p.nblk);   // column kt of the mask
  auto next_tile = [&](int it) -> int {
    if (MASK != 2 || it >= nqt) return it < nqt ? it : nqt;
    const int blk = it / QPB;
    const int nb = ms.next(blk);
    if (nb >= p.nblk) return nqt;
    const int t = nb == blk ? it : nb * QPB;
    return t < nqt ? t : nqt;
  };

  u32x4 reg[UPT][4];
  float lreg = 0.f, dreg = 0.f;
  auto gload = [&](int it) {
    const int q0 = it * kDkvBQ;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = tid + u * kThreads;
      const int which = unit / UNITS, uu = unit % UNITS;
      const int dc = uu % DC, kq = uu / DC;
      const uint16_t* src = which == 0 ? Qh : dOh;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int q = q0 + kq * 4 + j;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (q < N) x = *(const u32x4*)(src + (size_t)q * D + dc * 8);
        reg[u][j] = x;
      }
    }
    if (tid < kDkvBQ) {
      const int q = q0 + tid;
      float l2 = INFINITY, dv = 0.f;   // rows past N: P = 2^-inf = 0
      if (q < N) {
        const float l = lseh[q];
        l2 = l == -INFINITY ? INFINITY : l * kLog2e;
        dv = dth[q];
      }
      lreg = l2;
      dreg = dv;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = tid + u * kThreads;
      const int which = unit / UNITS, uu = unit % UNITS;
      const int dc = uu % DC, kq = uu / DC;
      u32x4 x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = which == 0 ? (reg[u][j] ^ p.qflip) : reg[u][j];
      uint16_t* rm = which == 0 ? sm.q[buf] : sm.dO[buf];
      uint16_t* tr = which == 0 ? sm.qt[buf] : sm.dOt[buf];
#pragma unroll
      for (int j = 0; j < 4; ++j) *(u32x4*)&rm[(kq * 4 + j) * RS + dc * 8] = x[j];
      store_quad_transposed(tr, TS, dc * 8, quad_pos(kq) * 4, x);
    }
    if (tid < kDkvBQ) {
      sm.lse2[buf][tid] = lreg;
      sm.dterm[buf][tid] = dreg;
    }
  };

  f32x16 dkT[NDT], dvT[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) {
    dkT[i] = zero16();
    dvT[i] = zero16();
  }
  const float c = p.c;

  auto compute = [&](int buf, int it) {
    const int q0 = it * kDkvBQ;
    bool live[2], needm[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int qb0 = q0 + 32 * mb;
      live[mb] = !(MASK == 1 && qb0 + 31 < kw0);
      needm[mb] = MASK == 1 && qb0 < kw0 + 31;
    }
    if (!live[0] && !live[1]) return;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = zero16();
      dp[mb] = zero16();
      if (!live[mb]) continue;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 aq = *(const u32x4*)&sm.q[buf][(mb * 32 + r) * RS + ks * 16 + h * 8];
        s[mb] = mfma_32x32x16(aq, kf[ks], s[mb]);
      }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 ao = *(const u32x4*)&sm.dO[buf][(mb * 32 + r) * RS + ks * 16 + h * 8];
        dp[mb] = mfma_32x32x16(ao, vf[ks], dp[mb]);
      }
    }
    u32x4 pb[2][2], db[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float pv[16], dv[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ql = mb * 32 + 8 * g + 4 * h;
        const float4 l4 = *(const float4*)&sm.lse2[buf][ql];
        const float4 d4 = *(const float4*)&sm.dterm[buf][ql];
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g + e;
          float pp = fast_exp2(__builtin_fmaf(s[mb][i], c, -lv[e]));
          if (needm[mb] && kj > q0 + ql + e) pp = 0.f;
          if (!live[mb]) pp = 0.f;
          pv[i] = pp;
          dv[i] = pp * (dp[mb][i] - dd[e]);
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const float* x = &pv[8 * st];
        const float* y = &dv[8 * st];
        pb[mb][st] = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                           pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
        db[mb][st] = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                           pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
      }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if (!live[mb]) continue;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int off = (dt * 32 + r) * TS + mb * 32 + st * 16 + h * 8;
          const u32x4 ao = *(const u32x4*)&sm.dOt[buf][off];
          dvT[dt] = mfma_32x32x16(ao, pb[mb][st], dvT[dt]);
          const u32x4 aq = *(const u32x4*)&sm.qt[buf][off];
          dkT[dt] = mfma_32x32x16(aq, db[mb][st], dkT[dt]);
        }
      }
  };

  int it = next_tile(qbeg);
  if (it < nqt) {
    gload(it);
    sstore(0);
  }
  __syncthreads();
  int buf = 0;
  while (it < nqt) {
    const int itn = next_tile(it + 1);
    const bool more = itn < nqt;
    if (more) gload(itn);
    compute(buf, it);
    if (more) sstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    it = itn;
  }

  if (kj < N) {
    const float ks = fabsf(p.scale);
    uint16_t* __restrict__ dKrow = (uint16_t*)p.dk + hoff + (size_t)kj * D;
    uint16_t* __restrict__ dVrow = (uint16_t*)p.dv + hoff + (size_t)kj * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = dt * 32 + 8 * g + 4 * h;
        u32x2 a = {pack_bf16x2(dkT[dt][4 * g] * ks, dkT[dt][4 * g + 1] * ks),
                   pack_bf16x2(dkT[dt][4 * g + 2] * ks, dkT[dt][4 * g + 3] * ks)};
        u32x2 b = {pack_bf16x2(dvT[dt][4 * g], dvT[dt][4 * g + 1]),
                   pack_bf16x2(dvT[dt][4 * g + 2], dvT[dt][4 * g + 3])};
        *(u32x2*)(dKrow + dd) = a;
        *(u32x2*)(dVrow + dd) = b;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per 128-query tile
// ---------------------------------------------------------------------------
constexpr int kDqBQ = 128;   // queries per workgroup
constexpr int kDqBK = 64;    // keys per LDS tile

template <int D>
struct alignas(16) DqSmem {
  static constexpr int RS = D + 8;
  static constexpr int TS = kDqBK + 8;
  uint16_t k[2][kDqBK * RS];
  uint16_t v[2][kDqBK * RS];
  uint16_t kt[2][D * TS];
};

template <int D, int MASK>
__global__ __launch_bounds__(kThreads) void bwd_dq_bf16_kernel(AttnParams p, uint32_t nqt, uint32_t total) {
  __shared__ DqSmem<D> sm;
  constexpr int RS = DqSmem<D>::RS;
  constexpr int TS = DqSmem<D>::TS;
  constexpr int DC = D / 8;
  constexpr int KUNITS = (kDqBK / 4) * DC;             // 4-key x 8-col units of K
  constexpr int VCH = kDqBK * DC / kThreads;           // 16-byte V chunks per thread
  constexpr int NDT = D / 32;
  constexpr int TPB = kMaskBlk / kDqBK;
  static_assert(KUNITS <= kThreads && VCH >= 1, "tile shape");

  const int N = p.N;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, r = lane & 31;
  const uint32_t L = xcd_remap(blockIdx.x, total);
  const uint32_t bh = L / nqt;
  uint32_t qt = L - bh * nqt;
  if (MASK == 1) qt = nqt - 1 - qt;
  const int q0 = (int)qt * kDqBQ;
  const int qw0 = q0 + 32 * w;
  const int qi = qw0 + r;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Qh = (const uint16_t*)p.q + hoff;
  const uint16_t* __restrict__ Kh = (const uint16_t*)p.k + hoff;
  const uint16_t* __restrict__ Vh = (const uint16_t*)p.v + hoff;
  const uint16_t* __restrict__ dOh = (const uint16_t*)p.dO + hoff;

  u32x4 qf[D / 16], of[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (qi < N) {
      a = *(const u32x4*)(Qh + (size_t)qi * D + ks * 16 + h * 8);
      b = *(const u32x4*)(dOh + (size_t)qi * D + ks * 16 + h * 8);
    }
    qf[ks] = a ^ p.qflip;
    of[ks] = b;
  }
  float lse2 = INFINITY, dti = 0.f;
  if (qi < N) {
    const float l = p.lse[(size_t)bh * N + qi];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
    dti = p.dterm[(size_t)bh * N + qi];
  }

  const int nkt = (N + kDqBK - 1) / kDqBK;
  int kend = nkt;
  if (MASK == 1) kend = min(nkt, (q0 + kDqBQ + kDqBK - 1) / kDqBK);
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

  u32x4 kreg[4], vreg[VCH];
  auto gload = [&](int kt) {
    const int k0 = kt * kDqBK;
    if (tid < KUNITS) {
      const int dc = tid % DC, kq = tid / DC;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = k0 + kq * 4 + j;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key < N) x = *(const u32x4*)(Kh + (size_t)key * D + dc * 8);
        kreg[j] = x;
      }
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int cidx = tid + i * kThreads;
      const int row = cidx / DC, col = cidx % DC;
      const int key = k0 + row;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < N) x = *(const u32x4*)(Vh + (size_t)key * D + col * 8);
      vreg[i] = x;
    }
  };
  auto sstore = [&](int buf) {
    if (tid < KUNITS) {
      const int dc = tid % DC, kq = tid / DC;
#pragma unroll
      for (int j = 0; j < 4; ++j) *(u32x4*)&sm.k[buf][(kq * 4 + j) * RS + dc * 8] = kreg[j];
      store_quad_transposed(sm.kt[buf], TS, dc * 8, quad_pos(kq) * 4, kreg);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int cidx = tid + i * kThreads;
      const int row = cidx / DC, col = cidx % DC;
      *(u32x4*)&sm.v[buf][row * RS + col * 8] = vreg[i];
    }
  };

  f32x16 dqT[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) dqT[i] = zero16();
  const float c = p.c;

  auto compute = [&](int buf, int kt) {
    const int k0 = kt * kDqBK;
    if (MASK == 1 && k0 > qw0 + 31) return;
    const bool need_mask = (k0 + kDqBK > N) || (MASK == 1 && k0 + kDqBK - 1 > qw0);
    bool live[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) live[kb] = !(MASK == 1 && k0 + kb * 32 > qw0 + 31);
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero16();
      dp[kb] = zero16();
      if (!live[kb]) continue;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 a = *(const u32x4*)&sm.k[buf][(kb * 32 + r) * RS + ks * 16 + h * 8];
        s[kb] = mfma_32x32x16(a, qf[ks], s[kb]);
      }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 a = *(const u32x4*)&sm.v[buf][(kb * 32 + r) * RS + ks * 16 + h * 8];
        dp[kb] = mfma_32x32x16(a, of[ks], dp[kb]);
      }
    }
    u32x4 db[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float dv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pp = fast_exp2(__builtin_fmaf(s[kb][i], c, -lse2));
        if (need_mask) {
          const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
          if (!live[kb] || key >= N || (MASK == 1 && key > qi)) pp = 0.f;
        }
        dv[i] = pp * (dp[kb][i] - dti);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const float* y = &dv[8 * st];
        db[kb][st] = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                           pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
      }
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!live[kb]) continue;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u32x4 a = *(const u32x4*)&sm.kt[buf][(dt * 32 + r) * TS + kb * 32 + st * 16 + h * 8];
          dqT[dt] = mfma_32x32x16(a, db[kb][st], dqT[dt]);
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

  if (qi < N) {
    const float sc = p.scale;
    uint16_t* __restrict__ dQrow = (uint16_t*)p.dq + hoff + (size_t)qi * D;
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

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int D, int MASK>
static int launch_bwd_t(const AttnParams& p, hipStream_t stream) {
  AttnParams pp = p;
  const size_t rows = (size_t)p.B * p.H * p.N;
  {
    const size_t threads = rows * (D / 8);
    const uint32_t grid = (uint32_t)((threads + kThreads - 1) / kThreads);
    size_t rr = rows;
    void* args[] = {&pp, &rr};
    hipError_t e = hipLaunchKernel((const void*)&bwd_rowterm_bf16_kernel<D>, dim3(grid), dim3(kThreads),
                                   args, 0, stream);
    if (e != hipSuccess) return (int)e;
  }
  {
    uint32_t nkt = (uint32_t)((p.N + kDkvBK - 1) / kDkvBK);
    uint32_t total = nkt * (uint32_t)p.B * (uint32_t)p.H;
    void* args[] = {&pp, &nkt, &total};
    hipError_t e = hipLaunchKernel((const void*)&bwd_dkdv_bf16_kernel<D, MASK>, dim3(total), dim3(kThreads),
                                   args, 0, stream);
    if (e != hipSuccess) return (int)e;
  }
  {
    uint32_t nqt = (uint32_t)((p.N + kDqBQ - 1) / kDqBQ);
    uint32_t total = nqt * (uint32_t)p.B * (uint32_t)p.H;
    void* args[] = {&pp, &nqt, &total};
    hipError_t e = hipLaunchKernel((const void*)&bwd_dq_bf16_kernel<D, MASK>, dim3(total), dim3(kThreads),
                                   args, 0, stream);
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

int launch_bwd_bf16(const AttnParams& p, int mask_kind, hipStream_t stream) {
  if (p.d == 64) {
    if (mask_kind == 0) return launch_bwd_t<64, 0>(p, stream);
    if (mask_kind == 1) return launch_bwd_t<64, 1>(p, stream);
    return launch_bwd_t<64, 2>(p, stream);
  }
  if (mask_kind == 0) return launch_bwd_t<128, 0>(p, stream);
  if (mask_kind == 1) return launch_bwd_t<128, 1>(p, stream);
  return launch_bwd_t<128, 2>(p, stream);
}

}  // namespace fa
