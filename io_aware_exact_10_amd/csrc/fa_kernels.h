// Launch parameters and launcher entry points shared by the C ABI layer and
// the kernel translation units. Host-visible, no torch types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const void* dO;
  void* dq;
  void* dk;
  void* dv;
  float* dterm;             // backward row term D [B, H, N] (workspace)
  const uint8_t* block_mask;
  int B, H, N, d;
  int nblk;                 // ceil(N / 128): block-mask entries per side
  float scale;              // as given (any sign)
  float c;                  // |scale| * log2(e): scores -> exp2 domain
  uint32_t qflip;           // 0x80008000 when scale < 0: bf16 sign flip of Q pairs
};

// Each returns a hipError_t value (0 on success).
// The backward is three launches: the row term, then dK/dV and dQ (these two
// depend only on the row term).
enum BwdStep { kBwdRowterm = 1, kBwdDkdv = 2, kBwdDq = 4, kBwdAll = 7 };

int launch_fwd_bf16(const AttnParams& p, int mask_kind, hipStream_t stream);
int launch_bwd_bf16(const AttnParams& p, int mask_kind, int steps, hipStream_t stream);
int launch_fwd_f32(const AttnParams& p, int mask_kind, hipStream_t stream);
int launch_bwd_f32(const AttnParams& p, int mask_kind, int steps, hipStream_t stream);

}  // namespace fa
