// Shared device helpers for the gfx950 attention kernels.
//
// MFMA conventions (v_mfma_f32_32x32x16_bf16, D = A x B + C, A 32x16,
// B 16x32, C 32x32, wave64). For lane l, with h = l / 32 and r = l % 32:
//   A: the lane holds row m = r and 8 contraction slots;
//   B: the lane holds column n = r and the same 8 contraction slots;
//   C: register i holds element (m = 8*(i/4) + 4*h + i%4, n = r).
// Only these facts are used: A and B enumerate contraction slots the same
// way, so any permutation of the contraction index applied to both operands
// gives the same product. The kernels exploit this to feed the C layout of one
// product straight into the B operand of the next.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Two floats -> two bf16 (round to nearest even) packed low|high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// Low and high bf16 halves of two dwords, interleaved: {a.lo, b.lo} / {a.hi, b.hi}.
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup id -> logical tile id so that consecutive logical tiles (the query
// tiles of one head) run on the same XCD and share its L2. Hardware hands out
// workgroup ids round-robin over the 8 XCDs; this maps XCD x to the contiguous
// logical range [x*q + min(x, r), ...) where total = 8q + r.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t wg, uint32_t total) {
  const uint32_t q = total >> 3, r = total & 7u;
  const uint32_t x = wg & 7u, s = wg >> 3;
  return x * q + (x < r ? x : r) + s;
}

// Block-sparse mask scanner: finds visible 128-blocks along one row (or one
// column, with a stride) of the block mask, 64 entries per ballot.
struct MaskScan {
  const uint8_t* base;  // first entry of the row/column
  int stride;           // elements between consecutive entries
  int count;            // entries along the row/column
  int wbase;            // first block index covered by `win`
  uint64_t win;         // bit i set <=> block wbase + i is kept

  __device__ __forceinline__ void init(const uint8_t* b, int s, int n) {
    base = b; stride = s; count = n; wbase = -64; win = 0;
  }
  __device__ __forceinline__ void load(int blk) {
    wbase = blk & ~63;
    const int idx = wbase + (int)(threadIdx.x & 63);
    const uint8_t mv = idx < count ? base[(size_t)idx * stride] : (uint8_t)0;
    win = __ballot(mv != 0);
  }
  // First kept block >= blk, or `count` if none.
  __device__ __forceinline__ int next(int blk) {
    while (blk < count) {
      if (blk < wbase || blk >= wbase + 64) load(blk);
      const uint64_t bits = win >> (blk - wbase);
      if (bits) return blk + __builtin_ctzll(bits);
      blk = wbase + 64;
    }
    return count;
  }
};

}  // namespace fa
