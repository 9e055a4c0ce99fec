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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
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

// Two floats -> two bf16 (round to nearest even) packed low|high: a single
// two-source v_cvt_pk_bf16_f32.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }


// ---------------------------------------------------------------------------
// LDS tiles: dense row-major [rows][D] bf16, 16-byte chunk c of row r stored
// at chunk position c ^ swz<D>(r). The swizzle keeps two access patterns
// free of bank conflicts on the 64-bank LDS: 16-byte reads of one chunk from
// 16 consecutive rows (MFMA operands taken along a row), and 8-byte
// transpose reads (ds_read_b64_tr_b16) of 4 consecutive rows x 64 bytes
// (MFMA operands taken down a column).
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 64 || D == 128, "head dim");
  return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// Byte offset of element (r, col) of a swizzled tile; col is a multiple of 4.
template <int D>
__device__ __forceinline__ int tile_off(int r, int col) {
  return r * (D * 2) + ((((col >> 3) ^ swz<D>(r))) << 4) + ((col & 7) << 1);
}

// One global->LDS copy instruction (16 bytes per lane, or 4 with DW4 =
// false): lane i's bytes go to LDS byte address lds + 16 i (4 i). Written out
// so the compiler does not track the copy: it would otherwise wait for it
// (or coarsen every LDS wait) before each later LDS read, though every
// kernel orders its copies and reads itself (wait_vmem() and a barrier
// before any wave reads a buffer a copy writes). The instruction has no
// register result; M0 holds the LDS address, and one wait state separates
// the M0 write from the copy.
template <bool DW4 = true>
__device__ __forceinline__ void copy_to_lds(const void* gbase, int voff, const void* lds) {
  // Both bases are the same in every lane (the callers pass workgroup- or
  // wave-uniform values); readfirstlane states it where the compiler cannot
  // prove it, so they go to scalar registers as the instruction requires.
  const uint64_t gb = (uint64_t)(uintptr_t)gbase;
  const uint32_t glo = __builtin_amdgcn_readfirstlane((uint32_t)gb);
  const uint32_t ghi = __builtin_amdgcn_readfirstlane((uint32_t)(gb >> 32));
  gbase = (const void*)(((uint64_t)ghi << 32) | glo);
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  if (DW4)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(gbase), "s"(m)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(gbase), "s"(m)
                 : "memory", "m0");
}

// Asynchronous copy of rows [r0, r0 + ROWS) of an N-row bf16 matrix with D
// columns and a row stride of rsb bytes into a swizzled LDS tile, straight
// from global memory to LDS (no registers). Each wave instruction fills one
// contiguous KiB: lane i writes bytes [16 i, 16 i + 16), so lane i fetches
// the global chunk that belongs there. The byte offset of that chunk from the
// tile's first row does not depend on the tile, so it is computed once per
// lane (offs); a full tile is then one uniform base pointer plus offs[i] per
// instruction. Rows past N (only in the last tile) read row N - 1: finite
// data the callers mask or ignore.
// Completion: s_waitcnt vmcnt(0) then a workgroup barrier.
template <int D, int ROWS, int NWAVES>
struct TileLoader {
  static constexpr int RPK = 1024 / (2 * D);   // rows per KiB
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int NK = ROWS / RPK;        // KiB pieces per tile
  static constexpr int PER = NK / NWAVES;      // pieces per wave
  static_assert(NK % NWAVES == 0, "tile pieces per wave");
  int offs[PER];                               // bytes from the tile's first row
  int wave, lane_, rsb;

  __device__ __forceinline__ static int row_of(int w, int lane, int i) {
    return (w + i * NWAVES) * RPK + lane / CPR;
  }
  __device__ __forceinline__ static int chunk_of(int w, int lane, int i) {
    return (lane % CPR) ^ swz<D>(row_of(w, lane, i));
  }
  __device__ __forceinline__ void init(int w, int lane, int row_bytes) {
    wave = w;
    lane_ = lane;
    rsb = row_bytes;
#pragma unroll
    for (int i = 0; i < PER; ++i) offs[i] = row_of(w, lane, i) * rsb + (chunk_of(w, lane, i) << 4);
  }
  // Same as load() with the offsets recomputed at the call (no registers kept
  // live across the loop), for kernels short of VGPRs.
  __device__ __forceinline__ void load_recompute(uint8_t* tile, const uint16_t* __restrict__ X, int r0, int N) {
    int l = lane_;
    asm volatile("" : "+v"(l));
#pragma unroll
    for (int i = 0; i < PER; ++i) offs[i] = row_of(wave, l, i) * rsb + (chunk_of(wave, l, i) << 4);
    load(tile, X, r0, N);
  }
  __device__ __forceinline__ void load(uint8_t* tile, const uint16_t* __restrict__ X, int r0, int N) const {
    const uint8_t* base = (const uint8_t*)X + (int64_t)r0 * rsb;
    if (r0 + ROWS <= N) {
#pragma unroll
      for (int i = 0; i < PER; ++i) copy_to_lds(base, offs[i], tile + (wave + i * NWAVES) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        int o = offs[i];
        if (r0 + row_of(wave, lane_, i) >= N) o = (N - 1 - r0) * rsb + (chunk_of(wave, lane_, i) << 4);
        copy_to_lds(base, o, tile + (wave + i * NWAVES) * 1024);
      }
    }
  }
};

// Max and sum over the lane pair (l, l ^ 32), the two halves of one query
// row in the S^T layouts: v_permlane32_swap exchanges the two 32-lane halves
// in the VALU (no LDS round trip, unlike a shuffle). Given two copies of x,
// one result holds the low half in both halves and the other the high half,
// so the max (sum) of the two is the pair's max (sum) in every lane.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N of this wave's vector memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Cheap fragment addressing for swizzled tiles. The swizzle only XORs the
// chunk field (bits 4..7 of the byte offset within a 2D-byte row), so for
// rows row0 = multiple of 16 and column blocks col0 = 32 dt:
//   tile_off(row0 + r, 16 ks + 8 h) = row0 * 2D + (row_base ^ 32 ks)
//   tile_off(row0 + 8 sel + rl, 32 dt + c) = row0 * 2D + (col_base[sel] ^ 64 dt)
// with per-lane bases that do not change inside the kernel. One XOR per
// fragment (none for ks = 0 / dt = 0); row0 * 2D is a constant offset.
template <int D>
__device__ __forceinline__ int row_frag_base(int lane) {
  return tile_off<D>(lane & 31, 8 * (lane >> 5));
}
template <int D>
__device__ __forceinline__ int col_frag_base(int lane, int sel) {
  const int g = lane >> 4, jj = (lane >> 2) & 3, q = lane & 3;
  return tile_off<D>(8 * sel + 4 * (g >> 1) + jj, 16 * (g & 1) + 4 * q);
}
// Row operand (lane: row row0 + lane % 32, elements [16 ks + 8 h, +8)).
__device__ __forceinline__ u32x4 row_frag(const uint8_t* tile_row0, int base, int ks) {
  return *(const u32x4*)(tile_row0 + (base ^ (32 * ks)));
}
// Column operand (the tile transposed): lane (m = l % 32, h = l / 32) gets
// column m of the block at the 8 rows {4h..4h+3, 8+4h..8+4h+3}, the
// contraction slots a B operand built from an MFMA C layout occupies. Two
// transpose reads: within each 16-lane group, lane i receives element i % 4
// of the 8-byte chunks addressed by lanes 4 j + i / 4 (j = 0..3), so lane s
// of group g addresses row 8 sel + 4 (g / 2) + (s % 16) / 4, columns
// 16 (g % 2) + 4 (s % 4) (col_frag_base).
__device__ __forceinline__ u32x4 col_frag(const uint8_t* tile_row0, int base0, int base1, int dt) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile_row0 + (base0 ^ (64 * dt))));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile_row0 + (base1 ^ (64 * dt))));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

// Workgroup id -> logical tile id so that consecutive logical tiles (the query
// tiles of one head) run on the same XCD and share its L2. Hardware hands out
// workgroup ids round-robin over the 8 XCDs; this maps XCD x to the contiguous
// logical range [x*q + min(x, r), ...) where total = 8q + r.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t wg, uint32_t total) {
  const uint32_t q = total >> 3, r = total & 7u;
  const uint32_t x = wg & 7u, s = wg >> 3;
  return x * q + (x < r ? x : r) + s;
}

// Logical work item of this workgroup: the XCD-aware order, or that order
// reversed (rev = 1, a debug switch: every workgroup computes the same
// result in any order, so a difference between the two orders exposes a race).
__device__ __forceinline__ uint32_t work_item(uint32_t rev, uint32_t total) {
  const uint32_t L = xcd_remap(blockIdx.x, total);
  return rev ? total - 1u - L : L;
}

// Causal work pairs. Under a causal mask the work of a tile grows (query
// tiles) or shrinks (key tiles) linearly along the sequence, so tiles j and
// n - 1 - j of one sequence and head together cost about the same for every
// j. A workgroup takes pair j: item 0 is the longer tile (the higher index
// when long_high, else the lower), item 1 the shorter. Returns the tile
// index, or -1 where the pair has no such item (j past the pairs of an n-tile
// sequence, or the middle tile of an odd n, which has no partner).
__device__ __forceinline__ int causal_pair_tile(uint32_t j, int item, int n, bool long_high) {
  if ((int)j >= (n + 1) / 2) return -1;
  const int lo = (int)j, hi = n - 1 - (int)j;
  if (item == 1 && lo == hi) return -1;
  return (item == 0) == long_high ? hi : lo;
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
