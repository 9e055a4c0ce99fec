// C ABI of libfa.so: host-side argument validation and kernel dispatch.
// Every check runs before anything is enqueued, so an invalid call returns a
// negative status and leaves all outputs untouched. No HIP API is called on
// an error path. The declarations and their contract live in include/fa.h.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "fa.h"
#include "fa_kernels.h"

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;   // per tensor; offsets are 64-bit inside

// Debug switch (fa_debug_reverse_order): launches made while it is set take
// their workgroups' work items in reverse order.
std::atomic<int> g_reverse_order{0};

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// [a, a+na) and [b, b+nb) overlap?
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int check_common(int B, int H, int N, int d, float scale, int mask_kind, const uint8_t* block_mask,
                 int dtype, int64_t* elems) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  const int64_t e = (int64_t)B * H * N;
  if (e > kMaxElems / 128) return FA_ERR_SHAPE;
  if ((int64_t)B * H * (((int64_t)N + 63) / 64) >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return FA_ERR_ARG;
  if (mask_kind != FA_MASK_NONE && mask_kind != FA_MASK_CAUSAL && mask_kind != FA_MASK_BLOCK_SPARSE)
    return FA_ERR_MASK;
  if (mask_kind == FA_MASK_BLOCK_SPARSE && block_mask == nullptr) return FA_ERR_MASK;
  *elems = e * d;
  return FA_OK;
}

fa::AttnParams make_params(int B, int H, int N, int d, float scale, int mask_kind,
                           const uint8_t* block_mask) {
  fa::AttnParams p = {};
  p.B = B;
  p.H = H;
  p.N = N;
  p.d = d;
  p.nblk = (N + 127) / 128;
  p.scale = scale;
  p.c = fabsf(scale) * 1.4426950408889634f;
  p.qflip = scale < 0.f ? 0x80008000u : 0u;
  p.rev = g_reverse_order.load() ? 1u : 0u;
  p.block_mask = mask_kind == FA_MASK_BLOCK_SPARSE ? block_mask : nullptr;
  fa::set_dense_layout(p);
  return p;
}

}  // namespace

namespace fa {

void set_dense_layout(AttnParams& p) {
  const int64_t d = p.d, N = p.N, H = p.H;
  p.Hkv = p.H;
  p.Nq = p.Nk = p.N;
  p.Tq = p.Tk = 0;
  p.cu_q = p.cu_k = nullptr;
  p.q_rs = p.k_rs = d;
  p.q_hs = p.k_hs = N * d;
  p.q_bs = p.k_bs = H * N * d;
  p.l_hs = N;
  p.l_bs = H * N;
  p.rt_rows = (int64_t)p.B * H * N;
  p.rt_inner = 1;
  p.rt_hs = 0;
}

}  // namespace fa

extern "C" {

int fa_debug_reverse_order(int on) {
  return g_reverse_order.exchange(on ? 1 : 0);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape (B, H, N must be >= 1 and the sizes must fit)";
    case FA_ERR_UNSUPPORTED:
      return "unsupported configuration (d must be 64 or 128; dtype as the entry point allows; split-key: "
             "(H / Hkv) * max_seqlen_q <= 128; tile height 0, 32, 64, 128 or 256, at most 128 with a block-sparse mask)";
    case FA_ERR_MASK: return "invalid mask (unknown mask_kind, or block_mask NULL for block-sparse)";
    case FA_ERR_WORKSPACE: return "workspace NULL or smaller than fa_bwd_workspace_bytes()";
    case FA_ERR_ALIGN: return "misaligned pointer (tensors 16-byte, lse 4-byte aligned)";
    case FA_ERR_HIP: return "HIP kernel launch failed";
    case FA_ERR_ARG: return "invalid argument (non-finite scale or overlapping output)";
    case FA_ERR_SCRATCH:
      return "fa_bwd_noalloc: B * H * N exceeds FA_BWD_NOALLOC_MAX_ROWS (use fa_bwd with a workspace)";
    default: return "unknown status";
  }
}

// Backward workspace: two float arrays of one entry per query row, each
// rounded up to 256 bytes: the row term, then the scaled LSE.
static size_t row_array_bytes(size_t rows) { return (rows * sizeof(float) + 255) & ~(size_t)255; }

size_t fa_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  return 2 * row_array_bytes((size_t)B * (size_t)H * (size_t)N);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale,
           int mask_kind, const uint8_t* block_mask, int dtype, hipStream_t stream) {
  return fa_fwd_tiled(q, k, v, o, lse, B, H, N, d, scale, mask_kind, block_mask, dtype, 0, stream);
}

int fa_fwd_tiled(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, float scale,
                 int mask_kind, const uint8_t* block_mask, int dtype, int block_rows, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int64_t elems = 0;
  int st = check_common(B, H, N, d, scale, mask_kind, block_mask, dtype, &elems);
  if (st != FA_OK) return st;
  if (block_rows != 0) {
    const bool known = block_rows == 32 || block_rows == 64 || block_rows == 128 || block_rows == 256;
    if (!known || dtype != FA_BF16 || (mask_kind == FA_MASK_BLOCK_SPARSE && block_rows > 128))
      return FA_ERR_UNSUPPORTED;
  }
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  const size_t tb = (size_t)elems * (dtype == FA_BF16 ? 2 : 4);
  const size_t lb = (size_t)B * H * N * sizeof(float);
  if (overlap(o, tb, q, tb) || overlap(o, tb, k, tb) || overlap(o, tb, v, tb) || overlap(o, tb, lse, lb) ||
      overlap(lse, lb, q, tb) || overlap(lse, lb, k, tb) || overlap(lse, lb, v, tb))
    return FA_ERR_ARG;
  fa::AttnParams p = make_params(B, H, N, d, scale, mask_kind, block_mask);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  const int e = dtype == FA_BF16 ? fa::launch_fwd_bf16(p, mask_kind, stream, block_rows)
                                 : fa::launch_fwd_f32(p, mask_kind, stream);
  return e == 0 ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"

namespace {

// Validation shared by fa_bwd and its three steps. Pointers a step does not
// use are passed as `unused` and skipped; every used pointer must be non-NULL
// and aligned, and no output may overlap an input or another output.
const char kUnusedTag = 0;
const void* const unused = &kUnusedTag;

int bwd_prepare(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, const void* dq, const void* dk, const void* dv,
                int B, int H, int N, int d, float scale, int mask_kind, const uint8_t* block_mask,
                int dtype, const void* workspace, size_t workspace_bytes, fa::AttnParams* out,
                bool builtin_scratch = false) {
  // builtin_scratch: the workspace is the library's own scratch array (no
  // caller pointer to check); the caller of this function sets dterm / lse2.
  if (builtin_scratch) {
    workspace = unused;
    workspace_bytes = 0;
  }
  const void* tens[8] = {q, k, v, o, dO, dq, dk, dv};
  for (const void* t : tens)
    if (!t) return FA_ERR_NULL;
  if (!lse) return FA_ERR_NULL;
  int64_t elems = 0;
  int st = check_common(B, H, N, d, scale, mask_kind, block_mask, dtype, &elems);
  if (st != FA_OK) return st;
  const size_t need = fa_bwd_workspace_bytes(B, H, N, d);
  if (!builtin_scratch && (!workspace || workspace_bytes < need)) return FA_ERR_WORKSPACE;
  for (const void* t : tens)
    if (t != unused && !aligned(t, 16)) return FA_ERR_ALIGN;
  if ((const void*)lse != unused && !aligned(lse, 4)) return FA_ERR_ALIGN;
  if (!builtin_scratch && !aligned(workspace, 16)) return FA_ERR_ALIGN;
  const size_t tb = (size_t)elems * (dtype == FA_BF16 ? 2 : 4);
  const size_t lb = (size_t)B * H * N * sizeof(float);
  const void* ins[6] = {q, k, v, o, dO, lse};
  const size_t insz[6] = {tb, tb, tb, tb, tb, lb};
  const void* outs[4] = {dq, dk, dv, workspace};
  const size_t outsz[4] = {tb, tb, tb, need};
  for (int i = 0; i < 4; ++i) {
    if (outs[i] == unused) continue;
    for (int j = 0; j < 6; ++j)
      if (ins[j] != unused && overlap(outs[i], outsz[i], ins[j], insz[j])) return FA_ERR_ARG;
    for (int j = i + 1; j < 4; ++j)
      if (outs[j] != unused && overlap(outs[i], outsz[i], outs[j], outsz[j])) return FA_ERR_ARG;
  }
  fa::AttnParams p = make_params(B, H, N, d, scale, mask_kind, block_mask);
  auto take = [](const void* x) -> const void* { return x == unused ? nullptr : x; };
  p.q = take(q);
  p.k = take(k);
  p.v = take(v);
  p.o = const_cast<void*>(take(o));
  p.lse = const_cast<float*>((const float*)take(lse));
  p.dO = take(dO);
  p.dq = const_cast<void*>(take(dq));
  p.dk = const_cast<void*>(take(dk));
  p.dv = const_cast<void*>(take(dv));
  if (!builtin_scratch) {
    p.dterm = (float*)const_cast<void*>(workspace);
    p.lse2 = (float*)((uint8_t*)const_cast<void*>(workspace) + row_array_bytes((size_t)B * H * N));
  }
  *out = p;
  return FA_OK;
}

int bwd_launch(const fa::AttnParams& p, int mask_kind, int dtype, int steps, hipStream_t stream) {
  const int e = dtype == FA_BF16 ? fa::launch_bwd_bf16(p, mask_kind, steps, stream)
                                 : fa::launch_bwd_f32(p, mask_kind, steps, stream);
  return e == 0 ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dO, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale,
           int mask_kind, const uint8_t* block_mask, int dtype,
           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fa::AttnParams p;
  const int st = bwd_prepare(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, mask_kind, block_mask,
                             dtype, workspace, workspace_bytes, &p);
  return st != FA_OK ? st : bwd_launch(p, mask_kind, dtype, fa::kBwdAll, stream);
}

int fa_bwd_rowterm(const void* o, const void* dO, const float* lse, int B, int H, int N, int d, int dtype,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fa::AttnParams p;
  const int st = bwd_prepare(unused, unused, unused, o, lse, dO, unused, unused, unused,
                             B, H, N, d, 1.0f, FA_MASK_NONE, nullptr, dtype, workspace, workspace_bytes, &p);
  return st != FA_OK ? st : bwd_launch(p, FA_MASK_NONE, dtype, fa::kBwdRowterm, stream);
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dO,
                void* dk, void* dv, int B, int H, int N, int d, float scale,
                int mask_kind, const uint8_t* block_mask, int dtype,
                const void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fa::AttnParams p;
  const int st = bwd_prepare(q, k, v, unused, lse, dO, unused, dk, dv, B, H, N, d, scale, mask_kind, block_mask,
                             dtype, workspace, workspace_bytes, &p);
  return st != FA_OK ? st : bwd_launch(p, mask_kind, dtype, fa::kBwdDkdv, stream);
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dO,
              void* dq, int B, int H, int N, int d, float scale,
              int mask_kind, const uint8_t* block_mask, int dtype,
              const void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fa::AttnParams p;
  const int st = bwd_prepare(q, k, v, unused, lse, dO, dq, unused, unused, B, H, N, d, scale, mask_kind, block_mask,
                             dtype, workspace, workspace_bytes, &p);
  return st != FA_OK ? st : bwd_launch(p, mask_kind, dtype, fa::kBwdDq, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// allocation-free backward: the workspace lives in a library-owned array
// ---------------------------------------------------------------------------
// The row term and the rescaled LSE of up to FA_BWD_NOALLOC_MAX_ROWS query
// rows (two float arrays, each a multiple of 256 bytes). The code object
// holds one copy per GPU it is loaded on, for the life of the process. In
// host code `scratch` names a host-side stand-in, never the device memory:
// only the per-device address from hipGetSymbolAddress is passed on.
namespace {
constexpr size_t kScratchRows = (size_t)FA_BWD_NOALLOC_MAX_ROWS;
constexpr size_t kScratchBytes = 2 * kScratchRows * sizeof(float);
static_assert(kScratchRows * sizeof(float) % 256 == 0, "each array a multiple of 256 bytes");
}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];   // device address of `scratch`, per device ordinal

// Address of this GPU's scratch array, looked up on the device's first call
// with that device current. Concurrent first calls look it up twice and store
// the same value.
int scratch_on_current_device(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  void* a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (a == nullptr) {
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || a == nullptr) return FA_ERR_HIP;
    g_scratch_addr[dev].store(a, std::memory_order_release);
  }
  *out = (uint8_t*)a;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dO, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale,
                   int mask_kind, const uint8_t* block_mask, int dtype, hipStream_t stream) {
  // The row limit first: a problem past it is rejected whatever else is wrong.
  const size_t rows = (size_t)(B > 0 ? B : 0) * (size_t)(H > 0 ? H : 0) * (size_t)(N > 0 ? N : 0);
  if (rows > kScratchRows) return FA_ERR_SCRATCH;
  fa::AttnParams p;
  int st = bwd_prepare(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, scale, mask_kind, block_mask, dtype,
                       nullptr, 0, &p, /*builtin_scratch=*/true);
  if (st != FA_OK) return st;
  uint8_t* base = nullptr;
  st = scratch_on_current_device(&base);
  if (st != FA_OK) return st;
  // Same split as fa_bwd's workspace: the row term, then the rescaled LSE.
  // The row-term kernel writes both for every row before the other two
  // kernels (later on the same stream) read them, so the previous call's
  // contents never reach a result and nothing needs clearing.
  p.dterm = (float*)base;
  p.lse2 = (float*)(base + row_array_bytes(rows));
  return bwd_launch(p, mask_kind, dtype, fa::kBwdAll, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// packed variable-length batches with shared K/V heads (bf16)
// ---------------------------------------------------------------------------
namespace {

constexpr int kMaxHeads = 1 << 16;   // keeps a 64-row tile's byte offsets in 32 bits

int varlen_check(int B, int H, int Hkv, int max_q, int max_k, int total_q, int total_k, int d, float scale,
                 int mask_kind, int dtype) {
  if (B < 1 || H < 1 || Hkv < 1 || max_q < 1 || max_k < 1 || total_q < 1 || total_k < 1) return FA_ERR_SHAPE;
  if (H > kMaxHeads || H % Hkv != 0) return FA_ERR_SHAPE;
  if ((int64_t)total_q * H > kMaxElems / 128 || (int64_t)total_k * Hkv > kMaxElems / 128) return FA_ERR_SHAPE;
  if ((int64_t)B * H * (((int64_t)max_q + 63) / 64) >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  if ((int64_t)B * Hkv * (((int64_t)max_k + 63) / 64) >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return FA_ERR_ARG;
  if (mask_kind == FA_MASK_BLOCK_SPARSE) return FA_ERR_MASK;
  if (mask_kind != FA_MASK_NONE && mask_kind != FA_MASK_CAUSAL) return FA_ERR_MASK;
  return FA_OK;
}

fa::AttnParams varlen_params(const int* cu_q, const int* cu_k, int B, int H, int Hkv, int max_q, int max_k,
                             int total_q, int total_k, int d, float scale) {
  fa::AttnParams p = {};
  p.B = B;
  p.H = H;
  p.N = max_q;
  p.d = d;
  p.scale = scale;
  p.c = fabsf(scale) * 1.4426950408889634f;
  p.qflip = scale < 0.f ? 0x80008000u : 0u;
  p.rev = g_reverse_order.load() ? 1u : 0u;
  p.Hkv = Hkv;
  p.Nq = max_q;
  p.Nk = max_k;
  p.Tq = total_q;
  p.Tk = total_k;
  p.cu_q = cu_q;
  p.cu_k = cu_k;
  p.q_rs = (int64_t)H * d;
  p.q_hs = d;
  p.k_rs = (int64_t)Hkv * d;
  p.k_hs = d;
  p.l_hs = total_q;
  p.rt_rows = (int64_t)total_q * H;
  p.rt_inner = H;
  p.rt_hs = total_q;
  return p;
}

}  // namespace

extern "C" {

size_t fa_bwd_varlen_workspace_bytes(int total_q, int H, int d) {
  if (total_q < 1 || H < 1 || (d != 64 && d != 128)) return 0;
  return 2 * row_array_bytes((size_t)total_q * (size_t)H);
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k,
                  int B, int H, int Hkv, int max_seqlen_q, int max_seqlen_k,
                  int total_q, int total_k, int d, float scale, int mask_kind,
                  int dtype, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
  int st = varlen_check(B, H, Hkv, max_seqlen_q, max_seqlen_k, total_q, total_k, d, scale, mask_kind, dtype);
  if (st != FA_OK) return st;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return FA_ERR_ALIGN;
  const size_t qb = (size_t)total_q * H * d * 2, kb = (size_t)total_k * Hkv * d * 2;
  const size_t lb = (size_t)total_q * H * sizeof(float), cb = (size_t)(B + 1) * sizeof(int);
  const void* ins[5] = {q, k, v, cu_seqlens_q, cu_seqlens_k};
  const size_t insz[5] = {qb, kb, kb, cb, cb};
  for (int j = 0; j < 5; ++j)
    if (overlap(o, qb, ins[j], insz[j]) || overlap(lse, lb, ins[j], insz[j])) return FA_ERR_ARG;
  if (overlap(o, qb, lse, lb)) return FA_ERR_ARG;
  fa::AttnParams p = varlen_params(cu_seqlens_q, cu_seqlens_k, B, H, Hkv, max_seqlen_q, max_seqlen_k, total_q,
                                   total_k, d, scale);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  return fa::launch_fwd_bf16(p, mask_kind, stream) == 0 ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dO, void* dq, void* dk, void* dv,
                  const int* cu_seqlens_q, const int* cu_seqlens_k,
                  int B, int H, int Hkv, int max_seqlen_q, int max_seqlen_k,
                  int total_q, int total_k, int d, float scale, int mask_kind, int dtype,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !cu_seqlens_q || !cu_seqlens_k)
    return FA_ERR_NULL;
  int st = varlen_check(B, H, Hkv, max_seqlen_q, max_seqlen_k, total_q, total_k, d, scale, mask_kind, dtype);
  if (st != FA_OK) return st;
  const size_t need = fa_bwd_varlen_workspace_bytes(total_q, H, d);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  const void* tens[8] = {q, k, v, o, dO, dq, dk, dv};
  for (const void* t : tens)
    if (!aligned(t, 16)) return FA_ERR_ALIGN;
  if (!aligned(lse, 4) || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4) || !aligned(workspace, 16))
    return FA_ERR_ALIGN;
  const size_t qb = (size_t)total_q * H * d * 2, kb = (size_t)total_k * Hkv * d * 2;
  const size_t lb = (size_t)total_q * H * sizeof(float), cb = (size_t)(B + 1) * sizeof(int);
  const void* ins[8] = {q, k, v, o, dO, lse, cu_seqlens_q, cu_seqlens_k};
  const size_t insz[8] = {qb, kb, kb, qb, qb, lb, cb, cb};
  const void* outs[4] = {dq, dk, dv, workspace};
  const size_t outsz[4] = {qb, kb, kb, need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 8; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return FA_ERR_ARG;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return FA_ERR_ARG;
  }
  fa::AttnParams p = varlen_params(cu_seqlens_q, cu_seqlens_k, B, H, Hkv, max_seqlen_q, max_seqlen_k, total_q,
                                   total_k, d, scale);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = const_cast<void*>(o);
  p.lse = const_cast<float*>(lse);
  p.dO = dO;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dterm = (float*)workspace;
  p.lse2 = (float*)((uint8_t*)workspace + row_array_bytes((size_t)total_q * H));
  return fa::launch_bwd_bf16(p, mask_kind, fa::kBwdAll, stream) == 0 ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// split-key forward of packed batches with few queries per sequence (bf16)
// ---------------------------------------------------------------------------
namespace {

constexpr int kMaxSplits = 128;
constexpr int kMaxSplitRows = 128;   // (H / Hkv) * max_seqlen_q: query rows of one workgroup

size_t splitkv_o_bytes(int total_q, int H, int d, int splits) {
  return ((size_t)splits * (size_t)total_q * (size_t)H * (size_t)d * sizeof(float) + 255) & ~(size_t)255;
}

}  // namespace

extern "C" {

int fa_splitkv_splits(int B, int Hkv, int max_seqlen_k, int num_splits) {
  if (B < 1 || Hkv < 1 || max_seqlen_k < 1) return FA_ERR_SHAPE;
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_ARG;
  if (num_splits > 0) return num_splits;
  // Every range has the same number of keys, sized from the longest
  // sequence (shorter sequences use fewer ranges): about 8192 ranges if every
  // sequence were that long (some 32 per compute unit, so the ragged last
  // ranges even out), and at least 256 keys per range where there are keys
  // enough.
  const int64_t groups = (int64_t)B * Hkv;
  int64_t s = (8192 + groups - 1) / groups;
  const int64_t cap = ((int64_t)max_seqlen_k + 255) / 256;
  if (s > cap) s = cap;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : (int)s;
}

size_t fa_splitkv_workspace_bytes(int total_q, int H, int d, int splits) {
  if (total_q < 1 || H < 1 || (d != 64 && d != 128) || splits < 1 || splits > kMaxSplits) return 0;
  const size_t lse = ((size_t)splits * (size_t)H * (size_t)total_q * sizeof(float) + 255) & ~(size_t)255;
  return splitkv_o_bytes(total_q, H, d, splits) + lse;
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   const int* cu_seqlens_q, const int* cu_seqlens_k,
                   int B, int H, int Hkv, int max_seqlen_q, int max_seqlen_k,
                   int total_q, int total_k, int d, float scale, int mask_kind, int dtype, int num_splits,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
  int st = varlen_check(B, H, Hkv, max_seqlen_q, max_seqlen_k, total_q, total_k, d, scale, mask_kind, dtype);
  if (st != FA_OK) return st;
  if ((int64_t)(H / Hkv) * max_seqlen_q > kMaxSplitRows) return FA_ERR_UNSUPPORTED;
  const int splits = fa_splitkv_splits(B, Hkv, max_seqlen_k, num_splits);
  if (splits < 0) return splits;
  if ((int64_t)B * Hkv * splits >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  const size_t need = fa_splitkv_workspace_bytes(total_q, H, d, splits);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4) || !aligned(workspace, 16))
    return FA_ERR_ALIGN;
  const size_t qb = (size_t)total_q * H * d * 2, kb = (size_t)total_k * Hkv * d * 2;
  const size_t lb = (size_t)total_q * H * sizeof(float), cb = (size_t)(B + 1) * sizeof(int);
  const void* ins[5] = {q, k, v, cu_seqlens_q, cu_seqlens_k};
  const size_t insz[5] = {qb, kb, kb, cb, cb};
  const void* outs[3] = {o, lse, workspace};
  const size_t outsz[3] = {qb, lb, need};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return FA_ERR_ARG;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return FA_ERR_ARG;
  }
  fa::AttnParams p = varlen_params(cu_seqlens_q, cu_seqlens_k, B, H, Hkv, max_seqlen_q, max_seqlen_k, total_q,
                                   total_k, d, scale);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.splits = splits;
  p.part_o = (float*)workspace;
  p.part_lse = (float*)((uint8_t*)workspace + splitkv_o_bytes(total_q, H, d, splits));
  return fa::launch_splitkv_bf16(p, mask_kind, stream) == 0 ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// FP8 (E4M3) forward, dense layout
// ---------------------------------------------------------------------------
extern "C" {

int fa_fwd_fp8(const void* q, const void* k, const void* v_t, void* o, float* lse,
               int B, int H, int N, int d, int ldv, float scale,
               float q_descale, float k_descale, float v_descale, int mask_kind, hipStream_t stream) {
  if (!q || !k || !v_t || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if ((int64_t)B * H * N > kMaxElems / 128) return FA_ERR_SHAPE;
  if ((int64_t)B * H * (((int64_t)N + 127) / 128) >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  if (ldv < N || ldv % 16 != 0 || (int64_t)ldv * 128 >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!isfinite(scale) || !isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale)) return FA_ERR_ARG;
  const float sk = scale * q_descale * k_descale;
  if (!isfinite(sk)) return FA_ERR_ARG;
  if (mask_kind != FA_MASK_NONE && mask_kind != FA_MASK_CAUSAL) return FA_ERR_MASK;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v_t, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA_ERR_ALIGN;
  const size_t heads = (size_t)B * H;
  const size_t qb = heads * N * d, vb = heads * d * (size_t)ldv, ob = heads * N * d * 2, lb = heads * N * 4;
  const void* ins[3] = {q, k, v_t};
  const size_t insz[3] = {qb, qb, vb};
  for (int j = 0; j < 3; ++j)
    if (overlap(o, ob, ins[j], insz[j]) || overlap(lse, lb, ins[j], insz[j])) return FA_ERR_ARG;
  if (overlap(o, ob, lse, lb)) return FA_ERR_ARG;
  fa::AttnParams p = {};
  p.B = B;
  p.H = H;
  p.N = N;
  p.d = d;
  p.scale = scale;
  p.c = fabsf(sk) * 1.4426950408889634f;
  p.qflip = sk < 0.f ? 0x80808080u : 0u;   // E4M3 sign bit of every Q byte
  p.rev = g_reverse_order.load() ? 1u : 0u;
  p.ldv = ldv;
  p.vscale = v_descale;
  p.q = q;
  p.k = k;
  p.v = v_t;
  p.o = o;
  p.lse = lse;
  return fa::launch_fwd_fp8(p, mask_kind, stream) == 0 ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
