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
  float* dterm;             // backward row term (workspace, layout of lse; bf16 path: -D)
  float* lse2;              // bf16 backward: -LSE * log2(e) (workspace, layout of lse; -inf for empty rows)
  const uint8_t* block_mask;
  int B, H, N, d;
  int nblk;                 // ceil(N / 128): block-mask entries per side
  float scale;              // as given (any sign)
  float c;                  // |scale| * log2(e): scores -> exp2 domain
  uint32_t qflip;           // 0x80008000 when scale < 0: bf16 sign flip of Q pairs
  uint32_t rev;             // 1: workgroups take their work items in reverse order (debug switch)

  // Shapes and strides of the bf16 kernels. Dense [B, H, N, d]: Hkv = H,
  // Nq = Nk = N, cu_q = cu_k = null. Packed batches: sequence b owns tokens
  // [cu_q[b], cu_q[b+1]) of Q and [cu_k[b], cu_k[b+1]) of K, lengths clamped
  // to [0, Nq] / [0, Nk] and offsets to [0, Tq] / [0, Tk].
  int Hkv;                  // key/value heads; query head h reads K/V head h / (H / Hkv)
  int Nq, Nk;               // query / key lengths (maxima when packed)
  int Tq, Tk;               // total tokens when packed
  const int* cu_q;          // [B + 1] token offsets (device) or null
  const int* cu_k;
  int64_t q_rs, q_hs, q_bs; // element strides of q, o, dO, dq: row, head, batch (dense only)
  int64_t k_rs, k_hs, k_bs; // element strides of k, v, dk, dv
  int64_t l_hs, l_bs;       // lse and row term: head, batch (dense only); rows are contiguous
  // Row term: O and dO are rt_rows contiguous rows of d elements; row r
  // goes to entry (r % rt_inner) * rt_hs + r / rt_inner of the row term
  // (dense: rt_inner = 1, the identity; packed: r = token * H + head).
  int64_t rt_rows, rt_inner, rt_hs;
  // Split-key forward: key ranges per sequence and the per-range partial
  // results (fp32 O [splits, Tq, H, d], LSE [splits, H, Tq]; workspace).
  int splits;
  float* part_o;
  float* part_lse;
  // FP8 forward: V is given transposed, [B, H, d, ldv] bytes; O is scaled
  // by vscale (the V descale factor).
  int ldv;
  float vscale;
};

// Per-sequence view used by the kernels: lengths and the element offsets of
// head 0's first row (q side, k side) and of its first LSE entry.
struct SeqView {
  int nq, nk;
  int64_t qb, kb, lb;
};

__device__ __forceinline__ SeqView seq_view(const AttnParams& p, int b) {
  SeqView s;
  if (p.cu_q) {
    int q0 = p.cu_q[b], q1 = p.cu_q[b + 1], k0 = p.cu_k[b], k1 = p.cu_k[b + 1];
    q0 = q0 < 0 ? 0 : (q0 > p.Tq ? p.Tq : q0);
    q1 = q1 < q0 ? q0 : (q1 > p.Tq ? p.Tq : q1);
    k0 = k0 < 0 ? 0 : (k0 > p.Tk ? p.Tk : k0);
    k1 = k1 < k0 ? k0 : (k1 > p.Tk ? p.Tk : k1);
    s.nq = q1 - q0 < p.Nq ? q1 - q0 : p.Nq;
    s.nk = k1 - k0 < p.Nk ? k1 - k0 : p.Nk;
    s.qb = (int64_t)q0 * p.q_rs;
    s.kb = (int64_t)k0 * p.k_rs;
    s.lb = q0;
  } else {
    s.nq = p.Nq;
    s.nk = p.Nk;
    s.qb = (int64_t)b * p.q_bs;
    s.kb = (int64_t)b * p.k_bs;
    s.lb = (int64_t)b * p.l_bs;
  }
  return s;
}

// Fills the shape and stride fields for dense [B, H, N, d] tensors
// (Hkv = H, Nq = Nk = N) from B, H, N, d.
void set_dense_layout(AttnParams& p);

// Each returns a hipError_t value (0 on success).
// The backward is three launches: the row term, then dK/dV and dQ (these two
// depend only on the row term).
enum BwdStep { kBwdRowterm = 1, kBwdDkdv = 2, kBwdDq = 4, kBwdAll = 7 };

// block_rows: query rows per workgroup, 32, 64, 128 or 256 (not 256 with the
// block-sparse mask); 0 picks by shape.
int launch_fwd_bf16(const AttnParams& p, int mask_kind, hipStream_t stream, int block_rows = 0);
int launch_bwd_bf16(const AttnParams& p, int mask_kind, int steps, hipStream_t stream);
int launch_fwd_f32(const AttnParams& p, int mask_kind, hipStream_t stream);
// FP8 (E4M3) forward, dense layout, bf16 O.
int launch_fwd_fp8(const AttnParams& p, int mask_kind, hipStream_t stream);
// Split-key forward of a packed batch (partial ranges, then the merge).
int launch_splitkv_bf16(const AttnParams& p, int mask_kind, hipStream_t stream);
int launch_bwd_f32(const AttnParams& p, int mask_kind, int steps, hipStream_t stream);

}  // namespace fa
