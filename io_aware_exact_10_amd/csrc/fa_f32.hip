// fp32 path: the same tiled, online-softmax algorithm as the bf16 kernels,
// computed on the vector ALUs in fp32 throughout (the bf16 matrix cores do not
// take fp32 operands at full precision). It serves fp32 inputs; it is not
// the throughput path.
//
// Forward ("FlashAttention: exact attention made fast by counting memory
// traffic", "The method"; "FlashAttention and IO-aware exact attention",
// "Core ideas": online softmax, tiling and fusion, recomputation): a group of
// D/32 lanes owns one query row, each lane a 32-wide slice of d; 32-key
// tiles of K and V are staged in LDS; the running max, running sum and
// unnormalised output are updated per tile. Backward: the row term, then one
// kernel per gradient family that recomputes P from Q, K and the saved
// log-sum-exp (dK/dV grouped by key, dQ grouped by query). Gradient formulas
// are those of the bf16 backward.
#include "fa_common.h"
#include "fa_kernels.h"

namespace fa {

constexpr int kF32Threads = 256;
constexpr int kF32BK = 32;   // rows per LDS tile

template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ bool block_visible(const AttnParams& p, int qrow, int krow) {
  return p.block_mask[(size_t)(qrow / 128) * p.nblk + krow / 128] != 0;
}

// Cooperative load of `rows` x D floats starting at row r0 into LDS (zero past N).
template <int D>
__device__ __forceinline__ void load_rows_f32(float (*dst)[D], const float* src, int r0, int N) {
  constexpr int V4 = kF32BK * D / 4;
  for (int i = threadIdx.x; i < V4; i += kF32Threads) {
    const int row = i / (D / 4), c4 = i % (D / 4);
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r0 + row < N) x = *(const float4*)(src + (size_t)(r0 + row) * D + c4 * 4);
    *(float4*)&dst[row][c4 * 4] = x;
  }
}

template <int D, int MASK>
__global__ __launch_bounds__(kF32Threads) void fwd_f32_kernel(AttnParams p, uint32_t nqt, uint32_t total) {
  constexpr int G = D / 32;
  constexpr int ROWS = kF32Threads / G;
  __shared__ float ks[kF32BK][D];
  __shared__ float vs[kF32BK][D];
  const int N = p.N;
  const int tid = threadIdx.x, sl = tid % G;
  const uint32_t L = work_item(p.rev, total);
  const uint32_t bh = L / nqt;
  const int q0 = (int)(L - bh * nqt) * ROWS;
  const int qi = q0 + tid / G;
  const size_t hoff = (size_t)bh * N * D;
  const float* Q = (const float*)p.q + hoff;
  const float* K = (const float*)p.k + hoff;
  const float* V = (const float*)p.v + hoff;
  const float c = p.scale * kLog2e;

  float q[32], acc[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    q[e] = qi < N ? Q[(size_t)qi * D + sl * 32 + e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  int kend = N;
  if (MASK == 1) kend = min(N, q0 + ROWS);
  for (int k0 = 0; k0 < kend; k0 += kF32BK) {
    if (MASK == 2 && !block_visible(p, q0, k0)) continue;
    __syncthreads();
    load_rows_f32<D>(ks, K, k0, N);
    load_rows_f32<D>(vs, V, k0, N);
    __syncthreads();
    float t[kF32BK];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32BK; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) dot = __builtin_fmaf(q[e], ks[j][sl * 32 + e], dot);
      dot = group_sum<G>(dot);
      const int key = k0 + j;
      const bool vis = key < N && (MASK != 1 || key <= qi);
      t[j] = vis ? dot * c : -INFINITY;
      mx = fmaxf(mx, t[j]);
    }
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kF32BK; ++j) {
      const float pj = fast_exp2(t[j] - m_use);
      rs += pj;
#pragma unroll
      for (int e = 0; e < 32; ++e) acc[e] = __builtin_fmaf(pj, vs[j][sl * 32 + e], acc[e]);
    }
    l = l * alpha + rs;
  }
  if (qi < N) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    float* O = (float*)p.o + hoff + (size_t)qi * D + sl * 32;
#pragma unroll
    for (int e = 0; e < 32; e += 4) *(float4*)&O[e] = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
    if (sl == 0) p.lse[(size_t)bh * N + qi] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D>
__global__ __launch_bounds__(kF32Threads) void bwd_rowterm_f32_kernel(AttnParams p, size_t rows) {
  constexpr int G = D / 32;
  const size_t gt = (size_t)blockIdx.x * kF32Threads + threadIdx.x;
  const size_t row = gt / G;
  const int sl = (int)(gt % G);
  float acc = 0.f;
  if (row < rows) {
    const float* o = (const float*)p.o + row * D + sl * 32;
    const float* g = (const float*)p.dO + row * D + sl * 32;
#pragma unroll
    for (int e = 0; e < 32; ++e) acc = __builtin_fmaf(o[e], g[e], acc);
  }
  acc = group_sum<G>(acc);
  if (row < rows && sl == 0) p.dterm[row] = acc;
}

template <int D, int MASK>
__global__ __launch_bounds__(kF32Threads) void bwd_dkdv_f32_kernel(AttnParams p, uint32_t nkt, uint32_t total) {
  constexpr int G = D / 32;
  constexpr int ROWS = kF32Threads / G;
  __shared__ float qs[kF32BK][D];
  __shared__ float gs[kF32BK][D];
  __shared__ float l2s[kF32BK], dts[kF32BK];
  const int N = p.N;
  const int tid = threadIdx.x, sl = tid % G;
  const uint32_t L = work_item(p.rev, total);
  const uint32_t bh = L / nkt;
  const int k0 = (int)(L - bh * nkt) * ROWS;
  const int kj = k0 + tid / G;
  const size_t hoff = (size_t)bh * N * D;
  const float* Q = (const float*)p.q + hoff;
  const float* K = (const float*)p.k + hoff;
  const float* V = (const float*)p.v + hoff;
  const float* GO = (const float*)p.dO + hoff;
  const float* lse = p.lse + (size_t)bh * N;
  const float* dterm = p.dterm + (size_t)bh * N;
  const float c = p.scale * kLog2e;

  float k[32], v[32], dk[32], dv[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    k[e] = kj < N ? K[(size_t)kj * D + sl * 32 + e] : 0.f;
    v[e] = kj < N ? V[(size_t)kj * D + sl * 32 + e] : 0.f;
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  const int qbeg = MASK == 1 ? (k0 / kF32BK) * kF32BK : 0;
  for (int q0 = qbeg; q0 < N; q0 += kF32BK) {
    if (MASK == 2 && !block_visible(p, q0, k0)) continue;
    __syncthreads();
    load_rows_f32<D>(qs, Q, q0, N);
    load_rows_f32<D>(gs, GO, q0, N);
    if (threadIdx.x < kF32BK) {
      const int q = q0 + threadIdx.x;
      float l2 = INFINITY, dd = 0.f;
      if (q < N) {
        l2 = lse[q] == -INFINITY ? INFINITY : lse[q] * kLog2e;
        dd = dterm[q];
      }
      l2s[threadIdx.x] = l2;
      dts[threadIdx.x] = dd;
    }
    __syncthreads();
    for (int j = 0; j < kF32BK; ++j) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        s = __builtin_fmaf(qs[j][sl * 32 + e], k[e], s);
        dp = __builtin_fmaf(gs[j][sl * 32 + e], v[e], dp);
      }
      s = group_sum<G>(s);
      dp = group_sum<G>(dp);
      float pj = fast_exp2(s * c - l2s[j]);
      if (MASK == 1 && kj > q0 + j) pj = 0.f;
      const float ds = pj * (dp - dts[j]);
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        dv[e] = __builtin_fmaf(pj, gs[j][sl * 32 + e], dv[e]);
        dk[e] = __builtin_fmaf(ds, qs[j][sl * 32 + e], dk[e]);
      }
    }
  }
  if (kj < N) {
    float* dK = (float*)p.dk + hoff + (size_t)kj * D + sl * 32;
    float* dV = (float*)p.dv + hoff + (size_t)kj * D + sl * 32;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      dK[e] = dk[e] * p.scale;
      dV[e] = dv[e];
    }
  }
}

template <int D, int MASK>
__global__ __launch_bounds__(kF32Threads) void bwd_dq_f32_kernel(AttnParams p, uint32_t nqt, uint32_t total) {
  constexpr int G = D / 32;
  constexpr int ROWS = kF32Threads / G;
  __shared__ float ks[kF32BK][D];
  __shared__ float vs[kF32BK][D];
  const int N = p.N;
  const int tid = threadIdx.x, sl = tid % G;
  const uint32_t L = work_item(p.rev, total);
  const uint32_t bh = L / nqt;
  const int q0 = (int)(L - bh * nqt) * ROWS;
  const int qi = q0 + tid / G;
  const size_t hoff = (size_t)bh * N * D;
  const float* Q = (const float*)p.q + hoff;
  const float* K = (const float*)p.k + hoff;
  const float* V = (const float*)p.v + hoff;
  const float* GO = (const float*)p.dO + hoff;
  const float c = p.scale * kLog2e;

  float q[32], g[32], dq[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    q[e] = qi < N ? Q[(size_t)qi * D + sl * 32 + e] : 0.f;
    g[e] = qi < N ? GO[(size_t)qi * D + sl * 32 + e] : 0.f;
    dq[e] = 0.f;
  }
  float l2 = INFINITY, dd = 0.f;
  if (qi < N) {
    const float l = p.lse[(size_t)bh * N + qi];
    l2 = l == -INFINITY ? INFINITY : l * kLog2e;
    dd = p.dterm[(size_t)bh * N + qi];
  }
  int kend = N;
  if (MASK == 1) kend = min(N, q0 + ROWS);
  for (int k0 = 0; k0 < kend; k0 += kF32BK) {
    if (MASK == 2 && !block_visible(p, q0, k0)) continue;
    __syncthreads();
    load_rows_f32<D>(ks, K, k0, N);
    load_rows_f32<D>(vs, V, k0, N);
    __syncthreads();
    for (int j = 0; j < kF32BK; ++j) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        s = __builtin_fmaf(q[e], ks[j][sl * 32 + e], s);
        dp = __builtin_fmaf(g[e], vs[j][sl * 32 + e], dp);
      }
      s = group_sum<G>(s);
      dp = group_sum<G>(dp);
      const int key = k0 + j;
      float pj = fast_exp2(s * c - l2);
      if (key >= N || (MASK == 1 && key > qi)) pj = 0.f;
      const float ds = pj * (dp - dd);
#pragma unroll
      for (int e = 0; e < 32; ++e) dq[e] = __builtin_fmaf(ds, ks[j][sl * 32 + e], dq[e]);
    }
  }
  if (qi < N) {
    float* dQ = (float*)p.dq + hoff + (size_t)qi * D + sl * 32;
#pragma unroll
    for (int e = 0; e < 32; ++e) dQ[e] = dq[e] * p.scale;
  }
}

template <int D, int MASK>
static int launch_fwd_f32_t(const AttnParams& p, hipStream_t stream) {
  constexpr int ROWS = kF32Threads / (D / 32);
  AttnParams pp = p;
  uint32_t nqt = (uint32_t)((p.N + ROWS - 1) / ROWS);
  uint32_t total = nqt * (uint32_t)p.B * (uint32_t)p.H;
  void* args[] = {&pp, &nqt, &total};
  return (int)hipLaunchKernel((const void*)&fwd_f32_kernel<D, MASK>, dim3(total), dim3(kF32Threads), args, 0, stream);
}

template <int D, int MASK>
static int launch_bwd_f32_t(const AttnParams& p, int steps, hipStream_t stream) {
  constexpr int ROWS = kF32Threads / (D / 32);
  AttnParams pp = p;
  if (steps & kBwdRowterm) {
    size_t rows = (size_t)p.B * p.H * p.N;
    const uint32_t grid = (uint32_t)((rows * (D / 32) + kF32Threads - 1) / kF32Threads);
    void* args[] = {&pp, &rows};
    hipError_t e = hipLaunchKernel((const void*)&bwd_rowterm_f32_kernel<D>, dim3(grid), dim3(kF32Threads), args, 0, stream);
    if (e != hipSuccess) return (int)e;
  }
  uint32_t nt = (uint32_t)((p.N + ROWS - 1) / ROWS);
  uint32_t total = nt * (uint32_t)p.B * (uint32_t)p.H;
  if (steps & kBwdDkdv) {
    void* args[] = {&pp, &nt, &total};
    hipError_t e = hipLaunchKernel((const void*)&bwd_dkdv_f32_kernel<D, MASK>, dim3(total), dim3(kF32Threads), args, 0, stream);
    if (e != hipSuccess) return (int)e;
  }
  if (steps & kBwdDq) {
    void* args[] = {&pp, &nt, &total};
    hipError_t e = hipLaunchKernel((const void*)&bwd_dq_f32_kernel<D, MASK>, dim3(total), dim3(kF32Threads), args, 0, stream);
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

int launch_fwd_f32(const AttnParams& p, int mask_kind, hipStream_t stream) {
  if (p.d == 64) {
    if (mask_kind == 0) return launch_fwd_f32_t<64, 0>(p, stream);
    if (mask_kind == 1) return launch_fwd_f32_t<64, 1>(p, stream);
    return launch_fwd_f32_t<64, 2>(p, stream);
  }
  if (mask_kind == 0) return launch_fwd_f32_t<128, 0>(p, stream);
  if (mask_kind == 1) return launch_fwd_f32_t<128, 1>(p, stream);
  return launch_fwd_f32_t<128, 2>(p, stream);
}

int launch_bwd_f32(const AttnParams& p, int mask_kind, int steps, hipStream_t stream) {
  if (p.d == 64) {
    if (mask_kind == 0) return launch_bwd_f32_t<64, 0>(p, steps, stream);
    if (mask_kind == 1) return launch_bwd_f32_t<64, 1>(p, steps, stream);
    return launch_bwd_f32_t<64, 2>(p, steps, stream);
  }
  if (mask_kind == 0) return launch_bwd_f32_t<128, 0>(p, steps, stream);
  if (mask_kind == 1) return launch_bwd_f32_t<128, 1>(p, steps, stream);
  return launch_bwd_f32_t<128, 2>(p, steps, stream);
}

}  // namespace fa
